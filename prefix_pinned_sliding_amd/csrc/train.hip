// Attention forward and backward over the prefix-window mask for training, on MFMA.
//
// [PS] 08: the trainer back-propagates long traces chunk by chunk, or only through the last
// window with a few windows of lead context; either way the attention it differentiates is
// the generator's: key row j is visible to query row i iff j <= i and (j < P or
// j >= i - W + 1), rows [0, P) being the pinned prefix and later rows consecutive
// positions. Queries and keys arrive rotated, so this is masked attention in row space.
//
// Forward: out and lse (natural log) per (row, query head), on the prefill kernel's tile
// step and schedule (S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16, 256 rows =
// 256 / G positions x G heads per 8-wave workgroup, 64-key tiles, skipped / unmasked /
// masked tiles, two wave groups half a tile apart, three LDS buffers).
// Backward, three kernels:
//   rowdot  Di = sum_d dO * O per (row, head) (float32);
//   dkdv    one 8-wave workgroup per 128-key tile; each wave keeps its 16 keys' K and V in
//           registers and walks the query tiles that see the tile: S = Q K^T, dP = dO V^T,
//           P = exp(S - lse), dS = P (dP - Di), dV += P^T dO, dK += dS^T Q;
//   dq      one workgroup per 128-row query tile walking its visible key tiles:
//           S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.
// P and dS enter the second products as bf16, accumulation is float32 throughout.
#include "mfma_tile.h"
#include "psa_internal.h"

namespace psa {
namespace {



constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr int kBN = 64;      // keys per tile
constexpr int kRows = 128;   // query rows per dq workgroup
constexpr int kBR = 64;      // query rows per dkdv step

struct TrainArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    uint16_t *out, *dq, *dk, *dv;
    float* lse;              // [B][T][Hq] natural log
    float* di;               // [B][T][Hq] workspace: sum_d dO * O
    const int32_t* pre;      // [B] prefix rows
    const int32_t* len;      // [B] valid rows
    int B, T, Hq, Hkv, W;
    float scale;
};

// XCD-aware order: workgroup L runs on XCD L % 8; consecutive logical tiles (those of one
// (sequence, KV head)) go to one XCD so the operands they share stay in its L2.
__device__ __forceinline__ int xcd_logical(int total) {
    const int per_xcd = (total + 7) / 8;
    const int L = blockIdx.x;
    return (L % 8) * per_xcd + L / 8;
}

// The two key ranges of query rows [r_lo, r_hi]: prefix [0, min(P, r_hi + 1)) and band
// [max(P, r_lo - W + 1), r_hi + 1). walk() steps (seg, t0) through them in 64-key tiles.
struct KeyWalk {
    int hi0, lo1, hi1;
    __device__ bool next(int& seg, int& t0) const {
        t0 += kBN;
        if (seg == 0 && t0 >= hi0) {
            seg = 1;
            t0 = lo1;
        }
        return seg == 0 || t0 < hi1;
    }
};

// ---------------------------------------------------------------------------------------
// Forward: the chunked-prefill kernel's schedule on row-space tiles. 8 waves, 256 rows per
// workgroup in two groups of 4 waves running half a tile apart (group A passes the tile's
// barrier after its PV products, group B after its QK^T products), three LDS buffers (tile
// N + 1 is written into tile N - 2's), the next tile's K/V loaded into registers while the
// current one is computed. Queries are used unscaled; tile_step applies scale * log2(e) to
// the products in float32.
constexpr int kFwdWaves = 8;
constexpr int kFwdBlock = 64 * kFwdWaves;
constexpr int kFwdRows = 32 * kFwdWaves;

// This thread's share of key rows t0 .. t0 + 63 (rows past `last` repeat row `last`) of
// K and V into registers, in stage_tile's order.
template <int D>
__device__ __forceinline__ void fetch_rows(const TrainArgs& a, size_t kv0, int t0, int last,
                                           int tid, u32x4* kreg, u32x4* vreg) {
    constexpr int CPR = D / 8;
    constexpr int KLD = (kTileKeys * CPR) / kFwdBlock;
#pragma unroll
    for (int rr = 0; rr < KLD; ++rr) {
        const int ci = tid + kFwdBlock * rr;
        const int kk = min(ci / CPR, last), col = ci % CPR;
        const size_t off = (kv0 + (size_t)(t0 + kk) * a.Hkv) * D + col * 8;
        kreg[rr] = *reinterpret_cast<const u32x4*>(a.k + off);
        vreg[rr] = *reinterpret_cast<const u32x4*>(a.v + off);
    }
}

template <int D, int G>
__global__ __launch_bounds__(kFwdBlock, 1) void train_fwd_kernel(TrainArgs a, int n_qtiles) {
    constexpr int BQ = kFwdRows / G;
    constexpr int KS = D / 32, DB = D / 16;
    constexpr int VSTR = D + kVPad;
    constexpr int KLD = (kTileKeys * (D / 8)) / kFwdBlock;
    __shared__ __attribute__((aligned(16))) uint16_t k_s[3][kTileKeys * D];
    __shared__ __attribute__((aligned(16))) uint16_t v_s[3][kTileKeys * VSTR];

    const int total = n_qtiles * a.Hkv * a.B;
    const int logical = xcd_logical(total);
    if (logical >= total) return;
    // query tiles of one (sequence, KV head) go out last first: rows in the first window see
    // fewer keys, so the longest tiles start first and the short ones fill the end
    const int qt = n_qtiles - 1 - logical % n_qtiles;
    const int bh = logical / n_qtiles;
    const int h = bh % a.Hkv, b = bh / a.Hkv;
    const int len = a.len[b], P = a.pre[b], W = a.W;
    const int c0 = qt * BQ;
    if (c0 >= len) return;
    const int p_lo = c0, p_hi = min(c0 + BQ, len) - 1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const float sc = a.scale * kLog2e, inv_sc = 1.f / sc;

    int row_pos[2];
    bf16x8 qop[2][KS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * wave + 16 * rb + l16;
        row_pos[rb] = c0 + r / G;
        const int cl = min(row_pos[rb], len - 1);
        const size_t off = (((size_t)b * a.T + cl) * a.Hq + h * G + r % G) * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[rb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.q + off + ks * 32));
    }
    SoftmaxRows<DB> st;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        st.m[rb] = kNeg;
        st.mb[rb] = 0.f;
        st.l[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db) st.o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const KeyWalk wk{min(P, p_hi + 1), max(P, p_lo - W + 1), p_hi + 1};
    const size_t kv0 = (size_t)b * a.T * a.Hkv + h;   // row j at (kv0 + j * Hkv) * D
    auto seg_hi = [&](int sg) { return sg == 0 ? wk.hi0 : wk.hi1; };
    // every wave runs the same walk, so all pass the same number of barriers
    const bool grp_b = __builtin_amdgcn_readfirstlane(wave) >= kFwdWaves / 2;
    u32x4 kreg[KLD], vreg[KLD];
    int seg = 0, t0 = -kTileKeys;
    if (wk.next(seg, t0)) {
        int ct0 = t0, chi = seg_hi(seg), cur = 0;
        fetch_rows<D>(a, kv0, t0, min(t0 + kTileKeys, chi) - 1 - t0, tid, kreg, vreg);
        stage_tile<D, kTileKeys, kFwdBlock, VSTR>(k_s[0], v_s[0], tid, kreg, vreg);
        bool have = wk.next(seg, t0);
        if (have) fetch_rows<D>(a, kv0, t0, min(t0 + kTileKeys, seg_hi(seg)) - 1 - t0, tid, kreg, vreg);
        __syncthreads();
#pragma unroll 1
        while (true) {
            const int nt0 = t0, nhi = seg_hi(seg);
            const int nxt = cur == 2 ? 0 : cur + 1;
            bool have_next = false;
            if (have) {
                stage_tile<D, kTileKeys, kFwdBlock, VSTR>(k_s[nxt], v_s[nxt], tid, kreg, vreg);
                have_next = wk.next(seg, t0);
                if (have_next)
                    fetch_rows<D>(a, kv0, t0, min(t0 + kTileKeys, seg_hi(seg)) - 1 - t0, tid, kreg, vreg);
            }
            const int t1 = min(ct0 + kTileKeys, chi);
            const bool full = (ct0 + kTileKeys == t1) && (t1 - 1 <= p_lo) &&
                              (t1 - 1 < P || ct0 >= p_hi - W + 1);
            tile_step<D>(st, qop, k_s[cur], v_s[cur], row_pos, ct0, t1, P, W, l16, lg, !full, grp_b,
                         sc, inv_sc);
            if (!grp_b) __syncthreads();
            if (!have) break;
            ct0 = nt0;
            chi = nhi;
            have = have_next;
            cur = nxt;
        }
    }

#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float l = st.l[rb][0];
        const int r = 32 * wave + 16 * rb + l16;
        if (row_pos[rb] >= len) continue;
        const size_t row = ((size_t)b * a.T + row_pos[rb]) * a.Hq + h * G + r % G;
        const float inv = 1.f / l;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x2 w;
            w[0] = pack_bf16(st.o[rb][db][0] * inv, st.o[rb][db][1] * inv);
            w[1] = pack_bf16(st.o[rb][db][2] * inv, st.o[rb][db][3] * inv);
            *reinterpret_cast<u32x2*>(a.out + row * D + db * 16 + 4 * lg) = w;
        }
        if (lg == 0) a.lse[row] = (st.m[rb] + __log2f(l)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------------
// Di = sum_d dO * O per (sequence, row, query head): D / 8 lanes per row, each with one
// 16-byte chunk of dO and of O, so a wave's loads cover whole consecutive rows; the partial
// sums are added across the row's lanes. Each lane group takes kRowdotRows rows, a block
// apart, with all their loads issued first.
constexpr int kRowdotRows = 4;
template <int D>
__global__ __launch_bounds__(kBlock) void train_rowdot_kernel(TrainArgs a) {
    constexpr int LPR = D / 8;                       // lanes per row
    constexpr int RPB = kBlock / LPR;                // rows per block and pass
    static_assert(LPR == 8 || LPR == 16, "head dims 64 and 128");
    const size_t rows = (size_t)a.B * a.T * a.Hq;
    const int chunk = threadIdx.x % LPR;
    const size_t idx0 = (size_t)blockIdx.x * (RPB * kRowdotRows) + threadIdx.x / LPR;
    bool ok[kRowdotRows];
    u32x4 x[kRowdotRows], y[kRowdotRows];
#pragma unroll
    for (int r = 0; r < kRowdotRows; ++r) {
        const size_t idx = idx0 + (size_t)r * RPB;
        ok[r] = idx < rows;
        if (ok[r]) {
            const int i = (int)((idx / a.Hq) % a.T);
            const int b = (int)(idx / ((size_t)a.Hq * a.T));
            ok[r] = i < a.len[b];
        }
        if (ok[r]) {
            x[r] = reinterpret_cast<const u32x4*>(a.dout + idx * D)[chunk];
            y[r] = reinterpret_cast<const u32x4*>(a.o + idx * D)[chunk];
        }
    }
#pragma unroll
    for (int r = 0; r < kRowdotRows; ++r) {
        // A bf16 value is the high half of the float32 with the same bits, so each 32-bit
        // word holding two bf16 values gives its floats by a shift and a mask.
        float acc = 0.f;
        if (ok[r]) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t xe = x[r][e], ye = y[r][e];
                acc += __uint_as_float(xe << 16) * __uint_as_float(ye << 16);
                acc += __uint_as_float(xe & 0xffff0000u) * __uint_as_float(ye & 0xffff0000u);
            }
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m);
        if (ok[r] && chunk == 0) a.di[idx0 + (size_t)r * RPB] = acc;
    }
}


// One wave-wide direct load into LDS: lane l's 16 bytes at `g` land at LDS byte address
// lds + 16 l (global_load_lds_dwordx4, LDS base in M0). The compiler does not see this
// load: the caller waits for it with lds_dma_wait (loads complete in issue order) and
// publishes the data with a barrier.
__device__ __forceinline__ void lds_dma16(uint32_t lds, const void* g) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory", "m0");
}
// At most N vector-memory loads in flight. The builtin (not inline assembly) lets the
// compiler's own wait placement see it: after lds_dma_wait<0>() it knows every earlier load
// has landed on every path, and adds no waits for them later in the loop (such waits would
// also wait for the next step's direct loads, which it cannot see).
template <int N>
__device__ __forceinline__ void lds_dma_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------------------
// dK, dV: one workgroup per (sequence, KV head, kDkBN-key tile). Wave w owns keys
// k0 + 16 w .. k0 + 16 w + 15. A query step is kBR rows = kBR / G positions x G heads.
constexpr int kDkWaves = 8;                 // dK/dV workgroup: 16 keys per wave
constexpr int kDkBlock = 64 * kDkWaves;
constexpr int kDkBN = 16 * kDkWaves;        // keys per dK/dV workgroup
template <int D, int G>
__global__ __launch_bounds__(kDkBlock, 1) void train_dkdv_kernel(TrainArgs a, int n_ktiles) {
    constexpr int BP = kBR / G;                 // positions per query step
    constexpr int KS = D / 32, DB = D / 16, RB = kBR / 16, RS = kBR / 32;
    // Q and dO tiles: two buffers, each the Q tile then the dO tile (one base address serves
    // both, the dO reads at a fixed offset); unpadded rows with chunk_swz, filled by direct
    // loads
    constexpr int TB = kBR * D * 2;             // bytes of one tile
    __shared__ __attribute__((aligned(1024))) uint16_t qg_s[2][2 * kBR * D];
    __shared__ __attribute__((aligned(16))) float lse_s[2][kBR];
    __shared__ __attribute__((aligned(16))) float di_s[2][kBR];

    const int total = n_ktiles * a.Hkv * a.B;
    const int logical = xcd_logical(total);
    if (logical >= total) return;
    int kt = logical % n_ktiles, bh = logical / n_ktiles;
    // When every XCD holds whole (sequence, KV head) ranges, take them key tile by key
    // tile across its pairs: the prefix tiles, which every query row sees, start first on
    // all pairs.
    {
        const int nbh = a.Hkv * a.B;
        if (nbh % 8 == 0) {
            const int per = nbh / 8;                       // pairs per XCD
            const int x = logical / (per * n_ktiles);      // this XCD's range
            const int j = logical % (per * n_ktiles);      // place in its dispatch order
            kt = j / per;
            bh = x * per + j % per;
        }
    }
    const int h = bh % a.Hkv, b = bh / a.Hkv;
    const int len = a.len[b], P = a.pre[b], W = a.W;
    const int k0 = kt * kDkBN;
    if (k0 >= len) return;
    const int k1 = min(k0 + kDkBN, len);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const float sc = a.scale * kLog2e;

    // this lane's key (B-operand column) and its K, V chunks
    const int key = k0 + 16 * wave + l16;
    bf16x8 kop[KS], vop[KS];
    {
        const size_t off = (((size_t)b * a.T + min(key, k1 - 1)) * a.Hkv + h) * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kop[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.k + off + ks * 32));
            vop[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.v + off + ks * 32));
        }
    }
    f32x4 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // query positions that see some key of the tile
    const int i_end = k0 < P ? len : min(len, k1 - 1 + W);
    const size_t row0 = (size_t)b * a.T * a.Hq + h * G;   // (row0 + i * Hq + g) * D
    auto row_off = [&](int i0, int r) { return (row0 + (size_t)(i0 + r / G) * a.Hq + r % G) * D; };
    // Step i0's Q and dO rows go straight from memory into buffer `buf` (each wave issues
    // its share; the loads are waited for at the top of that step), its lse and D rows
    // into registers; both one step ahead of the products.
    const uint32_t q_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)(&qg_s[0][0]));
    const uint32_t g_lds = q_lds + TB;
    float lse_r = 0.f, di_r = 0.f;
    constexpr int CPR = D / 8, RPL = 64 / CPR, NPW = kBR / RPL / kDkWaves;
    static_assert(NPW * RPL * kDkWaves == kBR, "tile rows per wave");
    // row r of a step (position r / G, head r % G) starts ((r / G) Hq + r % G) D elements
    // after the step's first row; its chunks land swizzled by r. This lane's rows of a full
    // step, once: r = (NPW wave + x) RPL + lane / CPR.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto lane_off = [&](int r, int src) {
        return (uint32_t)(((src / G) * a.Hq + src % G) * D + ((lane % CPR) ^ chunk_swz<D>(r)) * 8);
    };
    uint32_t loff[NPW];
#pragma unroll
    for (int x = 0; x < NPW; ++x) {
        const int r = (wave_u * NPW + x) * RPL + lane / CPR;
        loff[x] = lane_off(r, r);
    }
    auto issue = [&](int i0, int buf) {
        const int last = (min(i0 + BP, len) - i0) * G - 1;
        const size_t base = (row0 + (size_t)i0 * a.Hq) * D;
        const uint16_t* qb = a.q + base;
        const uint16_t* gb = a.dout + base;
        if (last >= kBR - 1) {
#pragma unroll
            for (int x = 0; x < NPW; ++x) {
                const uint32_t o = (uint32_t)(buf * 2 * TB + (wave_u * NPW + x) * 1024);
                lds_dma16(q_lds + o, qb + loff[x]);
                lds_dma16(g_lds + o, gb + loff[x]);
            }
        } else {
            // a short last step: rows past `last` repeat row `last`
#pragma unroll
            for (int x = 0; x < NPW; ++x) {
                const int r = (wave_u * NPW + x) * RPL + lane / CPR;
                const uint32_t e = lane_off(r, min(r, last));
                const uint32_t o = (uint32_t)(buf * 2 * TB + (wave_u * NPW + x) * 1024);
                lds_dma16(q_lds + o, qb + e);
                lds_dma16(g_lds + o, gb + e);
            }
        }
        if (tid < kBR) {
            const size_t ri = row_off(i0, min(tid, last)) / D;
            lse_r = a.lse[ri];   // scaled when stored: a use here would wait for every load
            di_r = a.di[ri];
        }
    };
    // this lane's chunk swizzles: row reads (rows = l16 mod 16) and transposing reads
    // (rows = 4 lg + l16 / 4 mod 16)
    const int swz_row = chunk_swz<D>(l16), swz_tr = chunk_swz<D>(4 * lg + l16 / 4);
    if (k0 < i_end) issue(k0, 0);
    int buf = 0;
#pragma unroll 1
    for (int i0 = k0; i0 < i_end; i0 += BP, buf ^= 1) {
        const int i1 = min(i0 + BP, len);             // positions [i0, i1)
        const int last = (i1 - i0) * G - 1;            // last valid row of the step
        const bool full = (i1 - i0 == BP) && (k1 - k0 == kDkBN) && (k1 - 1 <= i0) &&
                          (k1 - 1 < P || k0 >= (i1 - 1) - W + 1);
        lds_dma_wait<0>();
        if (tid < kBR) {
            lse_s[buf][tid] = lse_r * kLog2e;
            di_s[buf][tid] = di_r;
        }
        // step i0's tiles are in place, and every wave is done with the other buffer
        __syncthreads();
        if (i0 + BP < i_end) issue(i0 + BP, buf ^ 1);
        const uint16_t* qt = qg_s[buf];
        const uint16_t* gt = qt + kBR * D;

        // S = Q K^T and dP = dO V^T for this wave's 16 keys; lane: rows 16 rb + 4 lg + i.
        // Product pairs in k-step-major order (8 independent accumulators per k-step); each
        // pair's Q and dO operands are read two pairs ahead, through a ring of three.
        constexpr int NRD = RB * KS, NPV = RS * DB;
        f32x4 s[RB], dp[RB];
        bf16x8 qa[3], ga[3];
        auto rd_row = [&](int it) {
            const int ks = it / RB, rb = it % RB;
            const int e = (rb * 16 + l16) * D + ((ks * 4 + lg) ^ swz_row) * 8;
            qa[it % 3] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + e));
            ga[it % 3] = as_bf16x8(*reinterpret_cast<const u32x4*>(gt + e));
        };
        rd_row(0);
        rd_row(1);
#pragma unroll
        for (int it = 0; it < NRD; ++it) {
            const int ks = it / RB, rb = it % RB;
            if (it + 2 < NRD) rd_row(it + 2);
            const f32x4 s0 = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[rb];
            const f32x4 d0 = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : dp[rb];
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[it % 3], kop[ks], s0, 0, 0, 0);
            dp[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[it % 3], vop[ks], d0, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // transposed dO and Q operands of the second products (pair it: rows 32 (it / DB)..,
        // d-block it % DB), read two pairs ahead through a ring of three; the first two go
        // out before the softmax
        bf16x8 gb[3], qb[3];
        auto rd_tr = [&](int it) {
            const int rs = it / DB, db = it % DB;
            const int e = (32 * rs + 4 * lg + l16 / 4) * D +
                          ((db * 2 + (l16 % 4) / 2) ^ swz_tr) * 8 + (l16 & 1) * 4;
            gb[it % 3] = lds_read_tr2(gt + e, gt + e + 16 * D);
            qb[it % 3] = lds_read_tr2(qt + e, qt + e + 16 * D);
        };
        rd_tr(0);
        rd_tr(1);
        // P and dS as A operands of the row contraction (k = rows, order of vt_col). The
        // products of rows 0-31 (rs = 0) are issued with the P and dS values of rows 32-63
        // computed between them (scheduling barriers fix the order), so the wave's VALU work
        // runs while the matrix core is busy.
        static_assert(RS == 2 && RB == 4, "two 32-row halves per step");
        bf16x8 pa[RS], sa[RS];
        float4 lsq[RB], dsq[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            lsq[rb] = *reinterpret_cast<const float4*>(&lse_s[buf][rb * 16 + 4 * lg]);
            dsq[rb] = *reinterpret_cast<const float4*>(&di_s[buf][rb * 16 + 4 * lg]);
        }
        if (!full) {
            // invisible products to -inf (then P = exp2(-inf) = 0): row r of the step is at
            // position i0 + r / G; this lane's key is seen by positions [key, key + W - 1]
            // (every later one for a prefix key), by valid rows only
            const int d0 = i0 - key;
            const unsigned span = key < P ? 0x7fffffffu : (unsigned)(W - 1);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rb * 16 + 4 * lg + i;
                    const bool vis = r <= last && key < k1 && (unsigned)(d0 + r / G) <= span;
                    s[rb][i] = vis ? s[rb][i] : -INFINITY;
                }
        }
        auto pds = [&](int rb, int i) {   // P and dS of row 16 rb + 4 lg + i
            const float ls = i == 0 ? lsq[rb].x : (i == 1 ? lsq[rb].y : (i == 2 ? lsq[rb].z : lsq[rb].w));
            const float ds = i == 0 ? dsq[rb].x : (i == 1 ? dsq[rb].y : (i == 2 ? dsq[rb].z : dsq[rb].w));
            const float p = __builtin_amdgcn_exp2f(s[rb][i] * sc - ls);
            const float d = p * (dp[rb][i] - ds);
            pa[rb / 2][(rb & 1) * 4 + i] = (__bf16)p;
            sa[rb / 2][(rb & 1) * 4 + i] = (__bf16)d;
        };
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pds(rb, i);
        __builtin_amdgcn_sched_barrier(0);
        // dV += P^T dO, dK += dS^T Q (scaled at the end)
        constexpr int PER = 8 / DB;   // values of rows 32-63 per d-block of rows 0-31
        static_assert(PER * DB == 8, "d-blocks per step");
#pragma unroll
        for (int it = 0; it < NPV; ++it) {
            const int rs = it / DB, db = it % DB;
            if (it + 2 < NPV) rd_tr(it + 2);
            dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[rs], gb[it % 3], dv[db], 0, 0, 0);
            dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa[rs], qb[it % 3], dk[db], 0, 0, 0);
            if (rs == 0) {
#pragma unroll
                for (int x = db * PER; x < (db + 1) * PER; ++x) pds(2 + x / 4, x % 4);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // lane holds keys 16 w + 4 lg + i, dims 16 db + l16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = k0 + 16 * wave + 4 * lg + i;
        if (j >= k1) continue;
        const size_t row = (((size_t)b * a.T + j) * a.Hkv + h) * D + l16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            a.dk[row + db * 16] = __builtin_bit_cast(uint16_t, (__bf16)(dk[db][i] * a.scale));
            a.dv[row + db * 16] = __builtin_bit_cast(uint16_t, (__bf16)dv[db][i]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// dQ: one workgroup per (sequence, KV head, 128-row query tile), walking its key tiles.
template <int D, int G>
__global__ __launch_bounds__(kBlock, 2) void train_dq_kernel(TrainArgs a, int n_qtiles) {
    constexpr int BQ = kRows / G;
    constexpr int KS = D / 32, DB = D / 16, KB = kBN / 16, PVS = kBN / 32;
    // K and V tiles: two buffers, each the K tile then the V tile (one base address serves
    // both); unpadded rows with chunk_swz, filled by direct loads
    constexpr int TB = kBN * D * 2;             // bytes of one tile
    __shared__ __attribute__((aligned(1024))) uint16_t kv_s[2][2 * kBN * D];

    const int total = n_qtiles * a.Hkv * a.B;
    const int logical = xcd_logical(total);
    if (logical >= total) return;
    // query tiles of one (sequence, KV head) go out last first: rows in the first window see
    // fewer keys, so the longest tiles start first and the short ones fill the end
    const int qt = n_qtiles - 1 - logical % n_qtiles;
    const int bh = logical / n_qtiles;
    const int h = bh % a.Hkv, b = bh / a.Hkv;
    const int len = a.len[b], P = a.pre[b], W = a.W;
    const int c0 = qt * BQ;
    if (c0 >= len) return;
    const int p_lo = c0, p_hi = min(c0 + BQ, len) - 1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const float sc = a.scale * kLog2e;

    int row_pos[2];
    size_t row_idx[2];
    bf16x8 qop[2][KS], gop[2][KS];
    float lse2[2], di[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * wave + 16 * rb + l16;
        row_pos[rb] = c0 + r / G;
        const int cl = min(row_pos[rb], len - 1);
        row_idx[rb] = ((size_t)b * a.T + cl) * a.Hq + h * G + r % G;
        const size_t off = row_idx[rb] * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qop[rb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.q + off + ks * 32));
            gop[rb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.dout + off + ks * 32));
        }
        lse2[rb] = a.lse[row_idx[rb]] * kLog2e;
        di[rb] = a.di[row_idx[rb]];
    }
    f32x4 acc[2][DB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

    const KeyWalk wk{min(P, p_hi + 1), max(P, p_lo - W + 1), p_hi + 1};
    const size_t kv0 = (size_t)b * a.T * a.Hkv + h;
    // The next key tile's K and V rows go straight from memory into the other buffer
    // while this one is used (each wave issues its share; waited for at the top of the tile).
    const uint32_t k_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)(&kv_s[0][0]));
    const uint32_t v_lds = k_lds + TB;
    constexpr int CPR = D / 8, RPL = 64 / CPR, NPW = kBN / RPL / kWaves;
    static_assert(NPW * RPL * kWaves == kBN, "tile rows per wave");
    // key row r of a tile starts r Hkv D elements after the tile's first row; its chunks land
    // swizzled by r. This lane's rows of a full tile, once: r = (NPW wave + x) RPL + lane / CPR.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto lane_off = [&](int r, int src) {
        return (uint32_t)(src * a.Hkv * D + ((lane % CPR) ^ chunk_swz<D>(r)) * 8);
    };
    uint32_t loff[NPW];
#pragma unroll
    for (int x = 0; x < NPW; ++x) {
        const int r = (wave_u * NPW + x) * RPL + lane / CPR;
        loff[x] = lane_off(r, r);
    }
    auto issue = [&](int sg, int s0, int buf) {
        const int last = min(s0 + kBN, sg == 0 ? wk.hi0 : wk.hi1) - 1 - s0;
        const size_t base = (kv0 + (size_t)s0 * a.Hkv) * D;
        const uint16_t* kb_ = a.k + base;
        const uint16_t* vb_ = a.v + base;
        if (last >= kBN - 1) {
#pragma unroll
            for (int x = 0; x < NPW; ++x) {
                const uint32_t o = (uint32_t)(buf * 2 * TB + (wave_u * NPW + x) * 1024);
                lds_dma16(k_lds + o, kb_ + loff[x]);
                lds_dma16(v_lds + o, vb_ + loff[x]);
            }
        } else {
            // a partial tile: rows past `last` repeat row `last`
#pragma unroll
            for (int x = 0; x < NPW; ++x) {
                const int r = (wave_u * NPW + x) * RPL + lane / CPR;
                const uint32_t e = lane_off(r, min(r, last));
                const uint32_t o = (uint32_t)(buf * 2 * TB + (wave_u * NPW + x) * 1024);
                lds_dma16(k_lds + o, kb_ + e);
                lds_dma16(v_lds + o, vb_ + e);
            }
        }
    };
    // this lane's chunk swizzles: row reads (rows = l16 mod 16) and transposing reads
    // (rows = 4 lg + l16 / 4 mod 16)
    const int swz_row = chunk_swz<D>(l16), swz_tr = chunk_swz<D>(4 * lg + l16 / 4);
    int seg = 0, t0 = -kBN, buf = 0;
    bool have = wk.next(seg, t0);
    if (have) issue(seg, t0, 0);
#pragma unroll 1
    while (have) {
        const int t1 = min(t0 + kBN, seg == 0 ? wk.hi0 : wk.hi1);
        const bool full = (t0 + kBN == t1) && (t1 - 1 <= p_lo) && (t1 - 1 < P || t0 >= p_hi - W + 1);
        const int ct0 = t0;
        lds_dma_wait<0>();
        // this tile is in place, and every wave is done with the other buffer
        __syncthreads();
        have = wk.next(seg, t0);
        if (have) issue(seg, t0, buf ^ 1);
        const uint16_t* kt = kv_s[buf];
        const uint16_t* vt = kt + kBN * D;
        buf ^= 1;

        // S^T = K Q^T, dP^T = V dO^T; lane: keys 16 kb + 4 lg + i, row l16. Each step's K
        // and V operands (four products) are read one step ahead.
        constexpr int NRD = KB * KS, NDQ = DB * PVS;
        f32x4 s[2][KB], dp[2][KB];
        bf16x8 ka[2], va[2];
        auto rd_row = [&](int it) {
            const int kb = it / KS, ks = it % KS;
            const int e = (kb * 16 + l16) * D + ((ks * 4 + lg) ^ swz_row) * 8;
            ka[it % 2] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + e));
            va[it % 2] = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + e));
        };
        rd_row(0);
#pragma unroll
        for (int it = 0; it < NRD; ++it) {
            const int kb = it / KS, ks = it % KS;
            if (it + 1 < NRD) rd_row(it + 1);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const f32x4 s0 = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[rb][kb];
                const f32x4 d0 = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : dp[rb][kb];
                s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[it % 2], qop[rb][ks], s0, 0, 0, 0);
                dp[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[it % 2], gop[rb][ks], d0, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // dS^T as B operands (k = keys in vt_col order)
        if (!full) {
            // invisible products to -inf (then P = exp2(-inf) = 0): key jb + c (c = 16 kb + i)
            // is visible iff c <= hi and c is not in the gap [pe, pe + gap) between the prefix
            // and the window
            const int jb = ct0 + 4 * lg;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int p = row_pos[rb];
                const int hi = min(p, t1 - 1) - jb, pe = P - jb;
                const unsigned gap = (unsigned)max(p - W + 1 - P, 0);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int cc = kb * 16 + i;
                        const bool vis = cc <= hi && (unsigned)(cc - pe) >= gap;
                        s[rb][kb][i] = vis ? s[rb][kb][i] : -INFINITY;
                    }
            }
        }
        bf16x8 sb[2][PVS];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(s[rb][kb][i] * sc - lse2[rb]);
                    sb[rb][kb / 2][(kb & 1) * 4 + i] = (__bf16)(p * (dp[rb][kb][i] - di[rb]));
                }
        __builtin_amdgcn_sched_barrier(0);
        // dQ^T += K^T dS^T; the transposed K operands (pair it: d-block it / PVS, keys
        // 32 (it % PVS)..) are read two pairs ahead, through a ring of three
        bf16x8 kb3[3];
        auto rd_tr = [&](int it) {
            const int db = it / PVS, ps = it % PVS;
            const int e = (32 * ps + 4 * lg + l16 / 4) * D +
                          ((db * 2 + (l16 % 4) / 2) ^ swz_tr) * 8 + (l16 & 1) * 4;
            kb3[it % 3] = lds_read_tr2(kt + e, kt + e + 16 * D);
        };
        rd_tr(0);
        rd_tr(1);
#pragma unroll
        for (int it = 0; it < NDQ; ++it) {
            const int db = it / PVS, ps = it % PVS;
            if (it + 2 < NDQ) rd_tr(it + 2);
            acc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb3[it % 3], sb[0][ps], acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb3[it % 3], sb[1][ps], acc[1][db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        if (row_pos[rb] >= len) continue;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x2 w;
            w[0] = pack_bf16(acc[rb][db][0] * a.scale, acc[rb][db][1] * a.scale);
            w[1] = pack_bf16(acc[rb][db][2] * a.scale, acc[rb][db][3] * a.scale);
            *reinterpret_cast<u32x2*>(a.dq + row_idx[rb] * D + db * 16 + 4 * lg) = w;
        }
    }
}

template <int D, int G>
hipError_t launch_train_g(const TrainArgs& a, bool backward, hipStream_t s) {
    if (!backward) {
        constexpr int BF = kFwdRows / G;
        const int f_tiles = (a.T + BF - 1) / BF;
        const int f_total = f_tiles * a.Hkv * a.B;
        hipLaunchKernelGGL((train_fwd_kernel<D, G>), dim3(((f_total + 7) / 8) * 8), dim3(kFwdBlock),
                           0, s, a, f_tiles);
        return hipGetLastError();
    }
    constexpr int BQ = kRows / G;
    const int n_qtiles = (a.T + BQ - 1) / BQ;
    const int q_total = n_qtiles * a.Hkv * a.B;
    const int q_grid = ((q_total + 7) / 8) * 8;
    const size_t rows = (size_t)a.B * a.T * a.Hq;
    constexpr int rows_per_block = kBlock / (D / 8) * kRowdotRows;
    hipLaunchKernelGGL((train_rowdot_kernel<D>),
                       dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)), dim3(kBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_ktiles = (a.T + kDkBN - 1) / kDkBN;
    const int k_total = n_ktiles * a.Hkv * a.B;
    hipLaunchKernelGGL((train_dkdv_kernel<D, G>), dim3(((k_total + 7) / 8) * 8), dim3(kDkBlock), 0,
                       s, a, n_ktiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((train_dq_kernel<D, G>), dim3(q_grid), dim3(kBlock), 0, s, a, n_qtiles);
    return hipGetLastError();
}

template <int D>
hipError_t launch_train_d(const TrainArgs& a, int G, bool backward, hipStream_t s) {
    switch (G) {
        case 1: return launch_train_g<D, 1>(a, backward, s);
        case 2: return launch_train_g<D, 2>(a, backward, s);
        case 4: return launch_train_g<D, 4>(a, backward, s);
        default: return launch_train_g<D, 8>(a, backward, s);
    }
}

}  // namespace

hipError_t launch_train(const TrainLaunch& t, hipStream_t s) {
    TrainArgs a;
    a.q = (const uint16_t*)t.q;
    a.k = (const uint16_t*)t.k;
    a.v = (const uint16_t*)t.v;
    a.o = (const uint16_t*)t.out;
    a.dout = (const uint16_t*)t.dout;
    a.out = (uint16_t*)t.out;
    a.dq = (uint16_t*)t.dq;
    a.dk = (uint16_t*)t.dk;
    a.dv = (uint16_t*)t.dv;
    a.lse = t.lse;
    a.di = t.di;
    a.pre = t.pre;
    a.len = t.len;
    a.B = t.B;
    a.T = t.T;
    a.Hq = t.Hq;
    a.Hkv = t.Hkv;
    a.W = t.W;
    a.scale = t.scale;
    const int G = t.Hq / t.Hkv;
    return t.D == 128 ? launch_train_d<128>(a, G, t.backward, s)
                      : launch_train_d<64>(a, G, t.backward, s);
}

}  // namespace psa
