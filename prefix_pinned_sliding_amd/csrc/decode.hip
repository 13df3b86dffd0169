// Split-KV decode attention over the pinned prefix and the window (K2) and the
// cross-split log-sum-exp merge (K3).
//
// [PS] 03: the query at t sees [1, P] and [max(P + 1, t - W + 1), t]. After the token at
// p = n - 1 is appended, the cache holds exactly that set: the prefix slots in use and the
// window's ring slots, which are contiguous modulo W from the window's head slot (the
// whole ring once it is full; see SeqView). [PS] 06 skips every block of the evicted
// middle; here the middle is never in memory, so the walk covers two slot ranges (the ring
// one wrapping at most once) and nothing else, and the only partially covered tile is the
// last one of a split (masked per key). Softmax order does not matter, so a full ring is
// walked from slot 0 rather than in age order.
//
// Work split: one workgroup (4 waves) per (kv head, split, sequence); grid x holds
// (split, head) pairs with the head fastest, grid y the sequences in the order array.
// Consecutive workgroups go to the eight XCDs in turn, so with H_kv = 8 each
// XCD takes one head of every split and the XCDs get equal work whatever the split count
// (with the split fastest, an even count put every sequence's first, full split on half of
// them). A split is a contiguous run of `split_tokens` entries of the concatenated
// [prefix | ring] list.
// Within a wave, LPK lanes share one key (each holds D / LPK of its elements, 16-byte
// loads), so a wave covers 64 / LPK keys per load; the G query heads of the kv head
// reuse every K/V element loaded. Logits are reduced over the LPK lanes with DPP, the
// softmax reference max is kept per wave (rescaling only when a tile max exceeds it by
// more than 2^8), and partial sums are combined across lane groups and waves once per
// split. K3 then merges the splits of each (sequence, query head).
#include "psa_internal.h"
#include "rope_round.h"

namespace psa {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;   // log2-domain headroom before a rescale

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem;
template <> struct Elem<PSA_BF16> { using T = uint16_t; };
template <> struct Elem<PSA_F32> { using T = float; };

__device__ __forceinline__ double to_f64(uint16_t b) {
    return (double)__uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ double to_f64(float f) { return (double)f; }

// Unpack one 16-byte chunk into floats.
__device__ __forceinline__ void unpack(const u32x4& w, float* f, uint16_t*) {
    f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xFFFF0000u);
    f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xFFFF0000u);
    f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xFFFF0000u);
    f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack(const u32x4& w, float* f, float*) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

// float32 -> bfloat16 bits, nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t out_as(float x, uint16_t*) { return f32_to_bf16(x); }
__device__ __forceinline__ uint16_t key_as(double x, uint16_t*) { return f64_to_bf16_bits(x); }
__device__ __forceinline__ float key_as(double x, float*) { return (float)x; }
__device__ __forceinline__ float out_as(float x, float*) { return x; }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                              0xF, 0xF, false));
}

// Sum over the LPK consecutive lanes that share a key (result in all of them).
template <int LPK>
__device__ __forceinline__ float key_sum(float x) {
    x += dpp<0xB1>(x);                               // quad_perm [1,0,3,2]
    if constexpr (LPK >= 4) x += dpp<0x4E>(x);       // quad_perm [2,3,0,1]
    if constexpr (LPK >= 8) x += dpp<0x141>(x);      // row_half_mirror
    if constexpr (LPK >= 16) x += dpp<0x140>(x);     // row_mirror
    return x;
}

// Max over the whole wave of a value replicated within each LPK-lane group.
template <int LPK>
__device__ __forceinline__ float wave_max(float x) {
    if constexpr (LPK < 8) x = fmaxf(x, dpp<0x124>(x));    // row_ror:4
    if constexpr (LPK < 16) x = fmaxf(x, dpp<0x128>(x));   // row_ror:8
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// Sum within a 16-lane row over the lane groups that hold the same elements.
template <int LPK>
__device__ __forceinline__ float row_group_sum(float x) {
    if constexpr (LPK < 8) x += dpp<0x124>(x);      // row_ror:4
    if constexpr (LPK < 16) x += dpp<0x128>(x);     // row_ror:8
    return x;
}

#ifndef PSA_DECODE_ROUNDS
#define PSA_DECODE_ROUNDS 2      // key rounds (of 64 / LPK keys) per wave per iteration
#endif
#ifndef PSA_DECODE_LPK_G2
#define PSA_DECODE_LPK_G2 8      // lanes per key when a KV head serves one or two query heads
#endif
#ifndef PSA_DECODE_RING
#define PSA_DECODE_RING 2        // K/V tiles per wave in the register ring (one in flight per
#endif                           // tile computed)

template <int DT, int D, int LPK, int U>
struct KVTile {
    static constexpr int CPL = (D / (16 / (int)sizeof(typename Elem<DT>::T))) / LPK;
    u32x4 k[U][CPL], v[U][CPL];
};

// With k_new != nullptr the launch first appends one token per sequence (k_new, v_new:
// [B][H_kv][D], as append_kernel with one token) and then decodes it: the state is the one
// after the append (n = len + 1). The new token's slot (the ring slot of the entry the
// append evicts, or prefix slot n - 1) is one logical entry of exactly one split; that
// split's workgroup writes the head's new key and value before it reads anything, and no
// other workgroup reads the slot. (Once the ring is full it is read from slot 0, so the
// new entry can sit in any split, not only the last.)
template <int DT, int D, int G, int LPK, bool PAGED>
__global__ __launch_bounds__(kBlock) void decode_partial_kernel(DevCache c,
                                                                const typename Elem<DT>::T* q,
                                                                int split_tokens,
                                                                const int32_t* __restrict__ len_cur,
                                                                const typename Elem<DT>::T* k_new,
                                                                const typename Elem<DT>::T* v_new,
                                                                int32_t* __restrict__ len_next) {
    using T = typename Elem<DT>::T;
    constexpr int EPC = 16 / (int)sizeof(T);    // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                // chunks per row
    constexpr int CPL = CPR / LPK;              // chunks per lane
    constexpr int EPL = CPL * EPC;              // elements per lane
    constexpr int KPW = 64 / LPK;               // keys per wave per load round
    constexpr int U = PSA_DECODE_ROUNDS;
    constexpr int STEP = kWaves * KPW * U;      // keys per workgroup iteration
    constexpr int ROWS = 4;                     // 16-lane rows per wave
    static_assert(CPL >= 1 && CPR % LPK == 0, "lane layout");
    using Tile = KVTile<DT, D, LPK, U>;

    const int h = blockIdx.x % c.Hkv, split = blockIdx.x / c.Hkv, b = c.order[blockIdx.y];
    const bool fused = k_new != nullptr;
    const int n = len_cur[b] + (fused ? 1 : 0);
    const SeqView sv = seq_view(c, b, n);
    const int n_pre = sv.n_pre, n_win = sv.n_win, ring_head = sv.head;
    const int Tb = n_pre + n_win;
    const int ns = split_count(n_pre, n_win, split_tokens, c.pe_mode);
    if (split >= ns) return;
    int i0, i1;
    int qpos = n - 1;                 // position the query is rotated at
    if (c.pe_mode == PSA_PE_RESET) {
        // prefix splits first, then window splits; prefix keys see the query at its
        // renumbered position n_pre + n_win - 1 (the newest window entry's)
        const int ns_pre = (n_pre + split_tokens - 1) / split_tokens;
        if (split < ns_pre) {
            i0 = split * split_tokens;
            i1 = min(n_pre, i0 + split_tokens);
            if (n_win > 0) qpos = n_pre + n_win - 1;
        } else {
            i0 = n_pre + (split - ns_pre) * split_tokens;
            i1 = min(Tb, i0 + split_tokens);
        }
    } else {
        i0 = split * split_tokens;
        i1 = min(Tb, i0 + split_tokens);
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPK, grp = lane / LPK;

    __shared__ float q_s[G][D];
    __shared__ float red_o[kWaves][ROWS][G][D];
    __shared__ float red_l[kWaves][ROWS][G];
    __shared__ float red_m[kWaves][G];

    // Prefix rows: the sequence's own slots, or its shared-prefix pool entry; ring rows
    // follow the own prefix slots.
    const size_t head_off = ((size_t)b * c.Hkv + h) * (size_t)c.S * D;
    const int pid = c.pid[b];
    const size_t pre_off = pid >= 0 ? ((size_t)pid * c.Hkv + h) * (size_t)c.shared_max * D : head_off;
    const T* Kp = (const T*)(pid >= 0 ? c.pool_k : c.k) + pre_off;
    const T* Vp = (const T*)(pid >= 0 ? c.pool_v : c.v) + pre_off;
    const T* Kr = (const T*)c.k + head_off + (size_t)c.Pmax * D;
    const T* Vr = (const T*)c.v + head_off + (size_t)c.Pmax * D;

    // Paged: the sequence's block table, read once into LDS.
    __shared__ int32_t tab_s[PAGED ? kMaxBlockTable : 1];
    if constexpr (PAGED) {
        for (int j = tid; j < c.NBT; j += kBlock) tab_s[j] = c.btab[(size_t)b * c.NBT + j];
        __syncthreads();
    }

    // Logical entry i -> physical row: the prefix rows, then the window's ring rows from
    // ring_head on, wrapping once. Attention does not depend on the order of its keys, so
    // a full ring is read from slot 0. Paged, logical slot s of the sequence is row
    // s mod Bs of block tab_s[s / Bs] (prefix rows of a shared prefix stay in the pool).
    auto load = [&](Tile& t, int base_i) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = min(base_i + u * KPW + grp, i1 - 1);
            const bool pre = i < n_pre;
            const int rr = i - n_pre + ring_head;
            const int ring_row = rr >= c.W ? rr - c.W : rr;
            const u32x4* kp;
            const u32x4* vp;
            if constexpr (PAGED) {
                const int slot = pre ? i : c.Pmax + ring_row;
                const bool pool = pre && pid >= 0;
                const size_t row = pool ? (size_t)i * D
                                        : block_rowidx(tab_s[slot >> c.bshift], h, slot & (c.Bs - 1),
                                                       c.Bs, c.n_blocks) * D;
                kp = reinterpret_cast<const u32x4*>((pool ? Kp : (const T*)c.k) + row);
                vp = reinterpret_cast<const u32x4*>((pool ? Vp : (const T*)c.v) + row);
            } else {
                const size_t row = (size_t)(pre ? i : ring_row) * D;
                kp = reinterpret_cast<const u32x4*>((pre ? Kp : Kr) + row);
                vp = reinterpret_cast<const u32x4*>((pre ? Vp : Vr) + row);
            }
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                t.k[u][cc] = __builtin_nontemporal_load(kp + cc * LPK + sub);
                t.v[u][cc] = __builtin_nontemporal_load(vp + cc * LPK + sub);
            }
        }
    };

    int owner = -1, i_new = 0;   // split holding the new token's entry (fused launch)
    if (fused) {
        const int p = n - 1, Pb = c.pre[b];
        i_new = p;                                         // prefix slot p
        if (p >= Pb) {
            const int r = (p - Pb) % c.W;                  // its ring slot
            i_new = n_pre + (r - ring_head + c.W) % c.W;
        }
        if (c.pe_mode == PSA_PE_RESET) {
            const int ns_pre = (n_pre + split_tokens - 1) / split_tokens;
            owner = i_new < n_pre ? i_new / split_tokens : ns_pre + (i_new - n_pre) / split_tokens;
        } else {
            owner = i_new / split_tokens;
        }
    }
    // The owner appends this head's new token (position n - 1) as append_kernel does, on
    // the last wave (the query set-up below runs on the first ones), then makes the stores
    // visible to the workgroup's loads: a fence, and a barrier before any load that may
    // reach the new entry. When the ring's first loads (entries [i0, i0 + R * STEP), any
    // past i1 read as i1 - 1) cannot reach it, those loads go out first and the barrier
    // after the query set-up serves; otherwise the append and a barrier come first.
    auto append_new = [&](bool barrier) {
        constexpr int H = D / 2;
        const int t = tid - (kBlock - H);
        if (t >= 0) {
            const size_t src = ((size_t)b * c.Hkv + h) * D;
            const T kx = k_new[src + t], ky = k_new[src + t + H];
            const T vx = v_new[src + t], vy = v_new[src + t + H];
            const double theta = c.inv_freq[t];
            const int slot = token_slot(c, b, 0, 1, n - 1, h == 0 && t == 0, len_next);
            if (slot >= 0) {
                double sn, cs, xr, yr;
                angle_sincos(n - 1, theta, &sn, &cs);
                rotate_with(to_f64(kx), to_f64(ky), sn, cs, &xr, &yr);
                const size_t dst = kv_rowidx(c, b, h, slot) * D;
                T* K = (T*)c.k;
                T* V = (T*)c.v;
                K[dst + t] = key_as(xr, (T*)nullptr);
                K[dst + t + H] = key_as(yr, (T*)nullptr);
                V[dst + t] = vx;
                V[dst + t + H] = vy;
            }
            __threadfence_block();
        }
        if (barrier) __syncthreads();
    };
    constexpr int R = PSA_DECODE_RING;
    const bool append_first = split == owner && i_new < i0 + R * STEP;
    if (append_first) append_new(true);

    // The ring's first K/V loads go out before the query set-up so that latency overlaps.
    const int base_i = i0 + wave * KPW * U;
    Tile ring[R];
#pragma unroll
    for (int r = 0; r < R; ++r) load(ring[r], base_i + r * STEP);
    if (split == owner && !append_first) append_new(false);   // barrier: after the query set-up

    {
        const int p = qpos;
        const float sc = c.scale * kLog2e;
        for (int idx = tid; idx < G * (D / 2); idx += kBlock) {
            const int g = idx / (D / 2), i = idx % (D / 2);
            const T* qp = q + ((size_t)b * c.Hq + h * G + g) * D;
            float xr, yr;
            rotate_query((float)to_f64(qp[i]), (float)to_f64(qp[i + D / 2]), p, c.inv_freq[i], sc,
                         &xr, &yr);
            q_s[g][i] = xr;
            q_s[g][i + D / 2] = yr;
        }
    }
    __syncthreads();

    float qr[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < EPC; ++e) qr[g][cc * EPC + e] = q_s[g][(cc * LPK + sub) * EPC + e];

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    // One tile of the wave's keys: logits, running max, then the value accumulation.
    auto consume = [&](const Tile& cur, const int cur_i) {
        float s[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = cur_i + u * KPW + grp < i1;
            float kf[EPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) unpack(cur.k[u][cc], kf + cc * EPC, (T*)nullptr);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d += qr[g][e] * kf[e];
                d = key_sum<LPK>(d);
                s[u][g] = ok ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mt = s[0][g];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][g]);
            mt = wave_max<LPK>(mt);
            if (mt > m[g] + kRescaleSlack) {          // wave-uniform
                const float f = __builtin_amdgcn_exp2f(m[g] - mt);
                l[g] *= f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] *= f;
                m[g] = mt;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) unpack(cur.v[u][cc], vf + cc * EPC, (T*)nullptr);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pr = __builtin_amdgcn_exp2f(s[u][g] - m[g]);
                l[g] += pr;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] += pr * vf[e];
            }
        }
    };
    // Register ring of R tiles, unrolled so that no tile is copied: each tile is consumed
    // and then reloaded R iterations ahead, so the compiler waits only for the tile about
    // to be used (a rotation by copies would wait for every load in flight). Loads past i1
    // repeat entry i1 - 1 and are never consumed.
    int cur_i = base_i;
    while (cur_i < i1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (cur_i < i1) consume(ring[r], cur_i);
            load(ring[r], cur_i + R * STEP);
            cur_i += STEP;
        }
    }

    // Combine: lane groups in a row share m, so sum them; rows and waves go through LDS.
    const int row = lane >> 4;
    const bool row_leader = (lane & 15) < LPK;      // first group of each row
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float lg = row_group_sum<LPK>(l[g]);
        if ((lane & 15) == 0) red_l[wave][row][g] = lg;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float a = row_group_sum<LPK>(acc[g][cc * EPC + e]);
                if (row_leader) red_o[wave][row][g][(cc * LPK + sub) * EPC + e] = a;
            }
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) red_m[wave][g] = m[g];
    }
    __syncthreads();

    for (int idx = tid; idx < G * D; idx += kBlock) {
        const int g = idx / D, d = idx % D;
        float M = red_m[0][g];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][g]);
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(red_m[w][g] - M);   // 0 for an idle wave
            float ow = 0.f, lw = 0.f;
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                ow += red_o[w][r][g][d];
                lw += red_l[w][r][g];
            }
            o += f * ow;
            L += f * lw;
        }
        const size_t hq = (size_t)b * c.Hq + h * G + g;
        const size_t part = hq * c.max_splits + split;
        c.part_o[part * D + d] = o;
        if (d == 0) {
            c.part_ml[part * 2 + 0] = M;
            c.part_ml[part * 2 + 1] = L;
        }
    }
}

// Merge the splits of one (sequence, query head): M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum O_s 2^(m_s - M) / L, rounded once to the output dtype; lse = (M + log2 L) ln 2.
template <int DT, int D>
__global__ __launch_bounds__(D) void merge_kernel(DevCache c, typename Elem<DT>::T* out,
                                                  float* lse, int split_tokens,
                                                  const int32_t* __restrict__ len_cur) {
    using T = typename Elem<DT>::T;
    const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int n = len_cur[b];
    const SeqView sv = seq_view(c, b, n);
    const int ns = split_count(sv.n_pre, sv.n_win, split_tokens, c.pe_mode);
    const size_t base = ((size_t)b * c.Hq + hq) * c.max_splits;
    const float* ml = c.part_ml + base * 2;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float f = __builtin_amdgcn_exp2f(ml[2 * s] - M);
        L += ml[2 * s + 1] * f;
        o += c.part_o[(base + s) * D + d] * f;
    }
    out[((size_t)b * c.Hq + hq) * D + d] = out_as(o / L, (T*)nullptr);
    if (lse != nullptr && d == 0) lse[(size_t)b * c.Hq + hq] = (M + __log2f(L)) * kLn2;
}

template <int DT, int D, int G>
hipError_t launch_partial_g(const DevCache& c, const void* q, int split_tokens, int grid_splits,
                            int cur, const void* k_new, const void* v_new, hipStream_t s) {
    using T = typename Elem<DT>::T;
    // Lanes per key: enough that q and the accumulators of G heads fit in registers,
    // never more than the 16-byte chunks in a row.
    constexpr int CPR = D / (16 / (int)sizeof(typename Elem<DT>::T));
    constexpr int PREF = G <= 2 ? PSA_DECODE_LPK_G2 : (G == 4 ? 8 : 16);
    constexpr int LPK = PREF < CPR ? PREF : CPR;
    const dim3 grid(c.Hkv * grid_splits, c.B);
    if (c.Bs > 0)
        hipLaunchKernelGGL((decode_partial_kernel<DT, D, G, LPK, true>), grid, dim3(kBlock), 0, s, c,
                           (const T*)q, split_tokens, c.len[cur], (const T*)k_new, (const T*)v_new,
                           c.len[cur ^ 1]);
    else
        hipLaunchKernelGGL((decode_partial_kernel<DT, D, G, LPK, false>), grid, dim3(kBlock), 0, s, c,
                           (const T*)q, split_tokens, c.len[cur], (const T*)k_new, (const T*)v_new,
                           c.len[cur ^ 1]);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_partial_d(const DevCache& c, const void* q, int split_tokens, int grid_splits,
                            int cur, const void* k_new, const void* v_new, hipStream_t s) {
    switch (c.Hq / c.Hkv) {
        case 1: return launch_partial_g<DT, D, 1>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s);
        case 2: return launch_partial_g<DT, D, 2>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s);
        case 4: return launch_partial_g<DT, D, 4>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s);
        default: return launch_partial_g<DT, D, 8>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s);
    }
}


template <int DT, int D, int G>
int wgs_per_cu_g() {
    constexpr int CPR = D / (16 / (int)sizeof(typename Elem<DT>::T));
    constexpr int PREF = G <= 2 ? PSA_DECODE_LPK_G2 : (G == 4 ? 8 : 16);
    constexpr int LPK = PREF < CPR ? PREF : CPR;
    static int cached = 0;
    if (cached == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, reinterpret_cast<const void*>(&decode_partial_kernel<DT, D, G, LPK, false>), kBlock,
                0) != hipSuccess || n < 1)
            n = 1;
        cached = n;
    }
    return cached;
}

template <int DT, int D>
int wgs_per_cu_d(int G) {
    switch (G) {
        case 1: return wgs_per_cu_g<DT, D, 1>();
        case 2: return wgs_per_cu_g<DT, D, 2>();
        case 4: return wgs_per_cu_g<DT, D, 4>();
        default: return wgs_per_cu_g<DT, D, 8>();
    }
}

}  // namespace

hipError_t launch_decode_partial(const DevCache& c, const void* q, int split_tokens,
                                 int grid_splits, int cur, const void* k_new, const void* v_new,
                                 hipStream_t s) {
    if (c.dtype == PSA_BF16)
        return c.D == 128 ? launch_partial_d<PSA_BF16, 128>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s)
                          : launch_partial_d<PSA_BF16, 64>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s);
    return c.D == 128 ? launch_partial_d<PSA_F32, 128>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s)
                      : launch_partial_d<PSA_F32, 64>(c, q, split_tokens, grid_splits, cur, k_new, v_new, s);
}

int decode_resident_wgs(const DevCache& c) {
    const int G = c.Hq / c.Hkv;
    const int per_cu = c.dtype == PSA_BF16
                           ? (c.D == 128 ? wgs_per_cu_d<PSA_BF16, 128>(G) : wgs_per_cu_d<PSA_BF16, 64>(G))
                           : (c.D == 128 ? wgs_per_cu_d<PSA_F32, 128>(G) : wgs_per_cu_d<PSA_F32, 64>(G));
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 1;
    return per_cu * cus;
}

hipError_t launch_merge(const DevCache& c, void* out, float* lse, int split_tokens, int cur,
                        hipStream_t s) {
    const dim3 grid(c.Hq, c.B);
#define PSA_MERGE(DT, DD)                                                                     \
    hipLaunchKernelGGL((merge_kernel<DT, DD>), grid, dim3(DD), 0, s, c,                       \
                       (typename Elem<DT>::T*)out, lse, split_tokens, c.len[cur])
    if (c.dtype == PSA_BF16) {
        if (c.D == 128) PSA_MERGE(PSA_BF16, 128); else PSA_MERGE(PSA_BF16, 64);
    } else {
        if (c.D == 128) PSA_MERGE(PSA_F32, 128); else PSA_MERGE(PSA_F32, 64);
    }
#undef PSA_MERGE
    return hipGetLastError();
}

}  // namespace psa
