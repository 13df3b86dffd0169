// Chunked-prefill attention on MFMA (K4) and the staging of a chunk's rotated keys.
//
// A chunk of C new tokens at positions n .. n + C - 1 of a sequence: query row c (at
// p = n + c) attends to A(p) ([PS] 03): the pinned prefix, the window [p - w + 1, p] and
// so the chunk's own tokens up to p (w: the sequence's window length). Keys come from three
// ranges, walked in tiles of BN = 64 positions:
//   prefix   the cache's prefix slots [0, min(n, npin)),
//   old ring positions [max(wb, p_lo - w + 1), n) in the ring (slot (j - P_b) mod W), with
//            wb the oldest window position before the chunk,
//   chunk    positions [n, p_hi] from the staged rotated keys and the input values,
// where [p_lo, p_hi] are the positions of the workgroup's rows. A tile is skipped when no
// row sees any of its keys, computed without masks when every row sees every key, and
// masked element by element otherwise ([PS] 06: whole tiles in the evicted middle are never
// loaded, partially covered tiles are masked).
//
// Per workgroup: 8 waves, 256 rows = (256 / G) positions x G query heads of one KV head, so
// every K/V tile in LDS serves all G heads. Each wave owns 32 rows (two 16-row blocks).
// Both products run on v_mfma_f32_16x16x32_bf16 in transposed form: S^T = K Q^T (K from
// LDS as the A operand, Q^T held in registers as B) and O^T = V^T P^T (V^T from LDS, P^T
// from registers). In S^T's accumulator layout each lane holds one row (query) and four
// keys, which is exactly the B-operand layout P^T needs, so probabilities never leave
// registers; row maxima need one cross-lane exchange per tile, row sums come from an MFMA
// against ones. K and V are staged row-major; V^T operands are read with transposing LDS
// loads. Softmax runs on exp2 with the scale folded into the queries (rotated and scaled
// as each workgroup loads them); the running max is raised only when a tile exceeds it by
// more than 2^8.
//
// Schedule: the waves form two groups of four, one wave of each on every SIMD. Group A
// passes the tile's barrier after its PV products, group B right after its QK^T products,
// so the groups run half a tile apart and one wave's softmax overlaps the other's matrix
// products. Tiles go through three LDS buffers (tile N + 1 is written into tile N - 2's,
// which both groups have left by then), with one barrier per tile; the next tile's K/V
// are loaded into registers while the current one is computed.
#include "psa_internal.h"
#include "mfma_tile.h"
#include "rope_round.h"

namespace psa {
namespace {


constexpr int kPfWaves = 8;              // attention workgroup: two groups of 4 waves
constexpr int kPfBlock = 64 * kPfWaves;
constexpr int kRows = 32 * kPfWaves;     // rows (position x head) per workgroup
constexpr int kBN = kTileKeys;           // keys per tile
constexpr int kNBuf = 3;                 // LDS tile buffers

// Stage a chunk's keys: rotated at their absolute positions and rounded once (the bytes the
// cache will hold). One block per (token j, sequence b0 + blockIdx.y); its threads take the
// token's (group of kStageHeads KV heads, rotation pair) items, and each computes its
// pair's sin/cos once for the group. (Queries are rotated by the attention kernel as it
// loads them.)
constexpr int kStageHeads = 4;

template <int D>
__global__ __launch_bounds__(1024) void stage_chunk_kernel(DevCache c, const uint16_t* k, int chunk,
                                                           int b0,
                                                           const int32_t* __restrict__ len_cur) {
    constexpr int H = D / 2;
    const int j = blockIdx.x, b = b0 + blockIdx.y;
    const int heads = c.Hkv;
    const int groups = (heads + kStageHeads - 1) / kStageHeads;
    const size_t row0 = ((size_t)b * chunk + j) * c.Hkv;   // key row of head 0
    const int p = len_cur[b] + j;
    uint16_t* ko = (uint16_t*)c.stage_k;
    for (int t = threadIdx.x; t < groups * H; t += blockDim.x) {
        const int grp = t / H, i = t % H;
        const int h0 = grp * kStageHeads;
        // Every input element of the group is loaded before anything is stored: the staging
        // buffer could alias the input as far as the compiler knows, so loads issued after a
        // store would each wait for it. A group past the last head repeats it and stores
        // nothing.
        double xs[kStageHeads], ys[kStageHeads];
        size_t offs[kStageHeads];
#pragma unroll
        for (int u = 0; u < kStageHeads; ++u) {
            const int hh = min(h0 + u, heads - 1);
            offs[u] = (row0 + hh) * D;
            xs[u] = bf16_bits_to_f64(k[offs[u] + i]);
            ys[u] = bf16_bits_to_f64(k[offs[u] + i + H]);
        }
        double sn, cs;
        angle_sincos(p, c.inv_freq[i], &sn, &cs);
#pragma unroll
        for (int u = 0; u < kStageHeads; ++u) {
            if (h0 + u >= heads) break;
            double xr, yr;
            rotate_with(xs[u], ys[u], sn, cs, &xr, &yr);
            ko[offs[u] + i] = f64_to_bf16_bits(xr);
            ko[offs[u] + i + H] = f64_to_bf16_bits(yr);
        }
    }
}

// MFMA B operands of one 16-row block from a query row of the chunk: this lane's dims
// 32 ks + 8 lg + j, rotated at position p (dim i < D / 2 pairs with i + D / 2, which the same
// lane holds in k-step ks + KS / 2), multiplied by `sc` and rounded to bf16. `qrow` points
// at the row's element 8 lg. fetch_query issues the row's 16-byte loads, rotate_query_ops
// turns them into operands; load_query does both at once.
template <int D>
__device__ __forceinline__ void fetch_query(u32x4 (&raw)[D / 32], const uint16_t* qrow) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) raw[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 32);
}

template <int D>
__device__ __forceinline__ void rotate_query_ops(bf16x8 (&qo)[D / 32], const u32x4 (&raw)[D / 32],
                                                 int p, const double* inv_freq, int lg, float sc) {
    constexpr int KS = D / 32, HS = KS / 2;
#pragma unroll
    for (int ks = 0; ks < HS; ++ks) {
        const u32x4 xw = raw[ks];
        const u32x4 yw = raw[ks + HS];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t xb = (j & 1) ? (xw[j / 2] & 0xFFFF0000u) : (xw[j / 2] << 16);
            const uint32_t yb = (j & 1) ? (yw[j / 2] & 0xFFFF0000u) : (yw[j / 2] << 16);
            float xr, yr;
            rotate_query_bf16(__uint_as_float(xb), __uint_as_float(yb), p, inv_freq[ks * 32 + 8 * lg + j],
                              sc, &xr, &yr);
            qo[ks][j] = (__bf16)xr;
            qo[ks + HS][j] = (__bf16)yr;
        }
    }
}

template <int D>
__device__ __forceinline__ void load_query(bf16x8 (&qo)[D / 32], const uint16_t* qrow, int p,
                                           const double* inv_freq, int lg, float sc) {
    u32x4 raw[D / 32];
    fetch_query<D>(raw, qrow);
    rotate_query_ops<D>(qo, raw, p, inv_freq, lg, sc);
}

// The key ranges of a workgroup, in walk order: 0 = prefix in the cache, 1 = prefix
// tokens inside the chunk (n < P), 2 = still-visible ring (n > P), 3 = window tokens of
// the chunk. Prefix keys (ranges 0, 1) all come before window keys (2, 3). `win_lo` is
// the first row's window start; walk_next steps to the next tile [t0, t1) some row sees.
struct Walk {
    int hi0, lo1, hi1, lo2, hi2, lo3, hi3, P, win_lo;
    __device__ int lo(int seg) const {
        return seg == 1 ? lo1 : (seg == 2 ? lo2 : (seg == 3 ? lo3 : 0));
    }
    __device__ int hi(int seg) const {
        return seg == 0 ? hi0 : (seg == 1 ? hi1 : (seg == 2 ? hi2 : hi3));
    }
};

// Ranges 0, 1 and 3 are walked upwards from their start. Range 2 is walked downwards from
// its end (the chunk's first position, the same for every workgroup of a sequence and KV
// head) in tiles aligned to that end, so those workgroups, whose ring ranges differ only
// in where they start, read each ring tile at about the same time and one L2 fill serves
// them all; the partial tile is the lowest one.
template <int BN>
__device__ __forceinline__ bool walk_next(const Walk& w, int& seg, int& t0, int& t1) {
    if (seg == 2) {
        if (t0 > w.lo2) {
            t1 = t0;
            t0 = max(t1 - BN, w.lo2);
            return true;
        }
        seg = 3;
        t0 = w.lo3 - BN;
    }
    t0 += BN;
    while (seg < 4) {
        const int hi = w.hi(seg);
        if (t0 >= hi) {
            ++seg;
            if (seg == 2) {
                if (w.hi2 > w.lo2) {
                    t1 = w.hi2;
                    t0 = max(t1 - BN, w.lo2);
                    return true;
                }
                seg = 3;   // no ring keys
            }
            if (seg < 4) t0 = w.lo(seg);
            continue;
        }
        t1 = min(t0 + BN, hi);
        // no row sees any key: all past the prefix and older than the first row's window
        if (t0 >= w.P && t1 - 1 < w.win_lo) {
            t0 += BN;
            continue;
        }
        return true;
    }
    return false;
}

// Where the K and V rows of position j live for key range `seg`.
struct TileSrc {
    const uint16_t *k_cache, *v_cache, *k_chunk, *v_chunk;
    const uint16_t *k_prefix, *v_prefix;   // own prefix slots or the shared-prefix entry
    size_t chunk_row0;   // b * chunk
    int n, P, W, Pmax, Hkv, h;             // P: P_b (ring origin), W: ring slots
    const int32_t* tab;                    // paged: the sequence's block table (LDS)
    int Bs, bshift, nblk;
    bool pool_prefix;                      // prefix rows come from the shared-prefix pool
};

// This thread's share of a tile into registers: KLD 16-byte chunks of K rows (lanes along
// a row), and a block of 4 keys x 8 dims of V (lanes along the keys). Positions past t1
// read the last valid row (masked later). Each tile gets one base pointer per operand;
// rows are 32-bit offsets from it: consecutive rows for the prefix and the chunk, the ring
// slot (reduced modulo W once per tile, then one wrap) for the window.
template <int D, int BN, int NT, bool PAGED>
__device__ __forceinline__ void fetch_tile(const TileSrc& s, int seg, int t0, int t1, int tid,
                                           u32x4* kreg, u32x4* vreg) {
    constexpr int CPR = D / 8;
    constexpr int KLD = (BN * CPR) / NT;
    const int last = t1 - 1 - t0;
    if (PAGED && (seg == 2 || (seg == 0 && !s.pool_prefix))) {
        // paged cache rows: logical slot -> row of its physical block, row by row
        const int ring0 = seg == 2 ? (t0 - s.P) % s.W : 0;
#pragma unroll
        for (int rr = 0; rr < KLD; ++rr) {
            const int ci = tid + NT * rr;
            const int kk = min(ci / CPR, last), col = ci % CPR;
            int slot = t0 + kk;
            if (seg == 2) {
                const int r = ring0 + kk;
                slot = s.Pmax + (r >= s.W ? r - s.W : r);
            }
            const size_t e = block_rowidx(s.tab[slot >> s.bshift], s.h, slot & (s.Bs - 1), s.Bs,
                                          s.nblk) * D + col * 8;
            kreg[rr] = *reinterpret_cast<const u32x4*>(s.k_cache + e);
            vreg[rr] = *reinterpret_cast<const u32x4*>(s.v_cache + e);
        }
        return;
    }
    const uint16_t* kb;
    const uint16_t* vb;
    int stride, ring0 = 0;
    if (seg == 1 || seg == 3) {
        const size_t o = ((s.chunk_row0 + (size_t)(t0 - s.n)) * s.Hkv + s.h) * D;
        kb = s.k_chunk + o;
        vb = s.v_chunk + o;
        stride = s.Hkv * D;
    } else if (seg == 2) {
        kb = s.k_cache + (size_t)s.Pmax * D;
        vb = s.v_cache + (size_t)s.Pmax * D;
        stride = D;
        ring0 = (t0 - s.P) % s.W;
    } else {
        kb = s.k_prefix + (size_t)t0 * D;
        vb = s.v_prefix + (size_t)t0 * D;
        stride = D;
    }
    auto row = [&](int off) -> int {   // row index relative to the tile's base pointer
        if (seg != 2) return off;
        const int r = ring0 + off;
        return s.W >= BN ? (r >= s.W ? r - s.W : r) : r % s.W;
    };
#pragma unroll
    for (int rr = 0; rr < KLD; ++rr) {
        const int ci = tid + NT * rr;
        const int kk = ci / CPR, col = ci % CPR;
        const uint32_t e = __umul24((uint32_t)row(min(kk, last)), (uint32_t)stride) + col * 8;
        kreg[rr] = *reinterpret_cast<const u32x4*>(kb + e);
        vreg[rr] = *reinterpret_cast<const u32x4*>(vb + e);
    }
}


template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kPfBlock, 1) void prefill_kernel(DevCache c, const uint16_t* __restrict__ q_in,
                                                              const uint16_t* __restrict__ v_in,
                                                              uint16_t* __restrict__ out,
                                                              float* __restrict__ lse, int chunk,
                                                              int n_qtiles,
                                                              const int32_t* __restrict__ len_cur) {
    constexpr int BQ = kRows / G;         // positions per workgroup
    constexpr int KS = D / 32;            // k-steps of S^T = K Q^T
    constexpr int DB = D / 16;            // d-blocks of O^T
    constexpr int KB = kBN / 16;          // key blocks per tile
    constexpr int PVS = kBN / 32;         // k-steps of O^T = V^T P^T
    constexpr int VSTR = D + kVPad;
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int KLD = (kBN * CPR) / kPfBlock;

    __shared__ __attribute__((aligned(16))) uint16_t k_s[kNBuf][kBN * D];
    __shared__ __attribute__((aligned(16))) uint16_t v_s[kNBuf][kBN * VSTR];

    // XCD-aware tile order: workgroup L runs on XCD L % 8; give each XCD a contiguous run
    // of logical tiles so all query tiles of one (sequence, KV head) share that XCD's L2.
    const int total = n_qtiles * c.Hkv * c.B;
    const int per_xcd = (total + 7) / 8;
    const int L = blockIdx.x;
    const int logical = (L % 8) * per_xcd + L / 8;
    if (logical >= total) return;
    const int qt = logical % n_qtiles;
    const int bh = logical / n_qtiles;
    const int h = bh % c.Hkv;
    const int b = bh / c.Hkv;

    const int n = len_cur[b];
    const int P = c.npin[b];      // pinned entries: positions below it are prefix keys
    const int W = c.wlen[b];      // this sequence's window length
    const SeqView sv = seq_view(c, b, n);
    const int c0 = qt * BQ;
    const int p_lo = n + c0;
    const int p_hi = n + min(c0 + BQ, chunk) - 1;   // last valid row position

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    // rows of this lane: r = 32 * wave + 16 * rb + l16, position p = n + c0 + r / G
    int row_pos[2];
    size_t q_off[2];
    bf16x8 qop[2][KS];
    // Queries are rotated here, at the row's position, and scaled by scale * log2(e) so the
    // softmax runs on exp2. RESET: prefix tiles come first and see the query rotated at its
    // renumbered position, its index in the list [prefix, window] after the append
    // (p inside the prefix, else P + min(w_b, p + 1 - wfloor) - 1); the operands are
    // rotated again at p once the walk leaves the prefix.
    // The query rows' loads go out first; they are rotated after the first key tile's loads
    // have been issued, so that the rotation overlaps those loads.
    bool q_prefix = c.pe_mode == PSA_PE_RESET;
    const float q_sc = c.scale * kLog2e;
    int q_pos[2];
    u32x4 q_raw[2][KS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * wave + 16 * rb + l16;
        const int cl = min(c0 + r / G, chunk - 1);
        const int g = r % G;
        row_pos[rb] = n + c0 + r / G;
        q_off[rb] = (((size_t)b * chunk + cl) * c.Hq + h * G + g) * D + 8 * lg;
        const int p = n + cl;
        q_pos[rb] = q_prefix && p >= c.pre[b] ? c.pre[b] + min(c.wlen[b], p + 1 - c.wfloor[b]) - 1 : p;
        fetch_query<D>(q_raw[rb], q_in + q_off[rb]);
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

    const size_t head_off = ((size_t)b * c.Hkv + h) * (size_t)c.S * D;

    // Key ranges in position space (see Walk). Prefix slot i counts as position i: the
    // prefix keys come first (i < npin) and every window position is >= npin. Promoted
    // entries (prefix slots P_b .. npin - 1) are older than every chunk row, so visible.
    const int nA = sv.n_pre;
    const int hi1 = min(P, p_hi + 1);                  // chunk prefix: [n, hi1) when n < P
    const int lo2 = max(sv.wb, p_lo - W + 1);          // ring: [lo2, n), empty when n <= wb
    const int lo3 = max(n, P);                         // chunk window: [lo3, p_hi]
    const Walk wk{nA, n, hi1, lo2, n, lo3, p_hi + 1, P, p_lo - W + 1};
    const int pid = c.pid[b];
    const size_t pre_off = pid >= 0 ? ((size_t)pid * c.Hkv + h) * (size_t)c.shared_max * D : head_off;
    // Paged: the sequence's block table in LDS; cache rows are addressed from the pool base.
    __shared__ int32_t tab_s[PAGED ? kMaxBlockTable : 1];
    if constexpr (PAGED) {
        for (int j = tid; j < c.NBT; j += kPfBlock) tab_s[j] = c.btab[(size_t)b * c.NBT + j];
        __syncthreads();
    }
    const size_t cache_off = PAGED ? 0 : head_off;
    const TileSrc src{(const uint16_t*)c.k + cache_off, (const uint16_t*)c.v + cache_off,
                      (const uint16_t*)c.stage_k, v_in,
                      (const uint16_t*)(pid >= 0 ? c.pool_k : c.k) + pre_off,
                      (const uint16_t*)(pid >= 0 ? c.pool_v : c.v) + pre_off,
                      (size_t)b * chunk, n, c.pre[b], c.W, c.Pmax, c.Hkv, h,
                      tab_s, c.Bs, c.bshift, c.n_blocks, pid >= 0};

    u32x4 kreg[KLD], vreg[KLD];
    int seg = 0, t0 = -kBN, t1 = 0;
    // Two groups of waves, A (waves 0 .. kPfWaves/2 - 1) and B (the rest), each SIMD holding
    // one wave of each. A passes the tile's barrier after its PV products, B after its QK^T
    // products, so on every SIMD one wave's softmax overlaps the other wave's products.
    // Three LDS buffers: tile N + 1 is written (by every wave, after barrier N - 1) into the
    // buffer of tile N - 2, which both groups have finished reading by then. The walk is the
    // same for every wave of the workgroup, so all waves pass the same number of barriers:
    // one before the loop and one per tile.
    const bool grp_b = __builtin_amdgcn_readfirstlane(wave) >= kPfWaves / 2;
    if (walk_next<kBN>(wk, seg, t0, t1)) {
        int cseg = seg, ct0 = t0, ct1 = t1, cur = 0;
        fetch_tile<D, kBN, kPfBlock, PAGED>(src, seg, t0, t1, tid, kreg, vreg);
        stage_tile<D, kBN, kPfBlock, VSTR>(k_s[0], v_s[0], tid, kreg, vreg);
        bool have = walk_next<kBN>(wk, seg, t0, t1);
        if (have) fetch_tile<D, kBN, kPfBlock, PAGED>(src, seg, t0, t1, tid, kreg, vreg);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            rotate_query_ops<D>(qop[rb], q_raw[rb], q_pos[rb], c.inv_freq, lg, q_sc);
        __syncthreads();
#pragma unroll 1
        while (true) {
            const int nseg = seg, nt0 = t0, nt1 = t1;
            const int nxt = cur == 2 ? 0 : cur + 1;
            bool have_next = false;
            if (have) {
                stage_tile<D, kBN, kPfBlock, VSTR>(k_s[nxt], v_s[nxt], tid, kreg, vreg);
                have_next = walk_next<kBN>(wk, seg, t0, t1);
                if (have_next) fetch_tile<D, kBN, kPfBlock, PAGED>(src, seg, t0, t1, tid, kreg, vreg);
            }
            if (q_prefix && cseg >= 2) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    load_query<D>(qop[rb], q_in + q_off[rb], n + min(row_pos[rb] - n, chunk - 1),
                                  c.inv_freq, lg, q_sc);
                q_prefix = false;
            }
            const bool full = (ct0 + kBN == ct1) && (ct1 - 1 <= p_lo) &&
                              (ct1 - 1 < P || ct0 >= p_hi - W + 1);
            tile_step_pinned<D>(st, qop, k_s[cur], v_s[cur], row_pos, ct0, ct1, P, W, l16, lg,
                                !full, grp_b, __any(st.mb[0] != 0.f || st.mb[1] != 0.f));
            if (!grp_b) __syncthreads();
            if (!have) break;
            cseg = nseg;
            ct0 = nt0;
            ct1 = nt1;
            have = have_next;
            cur = nxt;
        }
    }

    // ---- normalise and write -------------------------------------------------------------
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float l = st.l[rb][0];
        const int r = 32 * wave + 16 * rb + l16;
        const int cl = c0 + r / G;
        if (cl >= chunk) continue;
        const int hq = h * G + r % G;
        const float inv = 1.f / l;
        uint16_t* orow = out + (((size_t)b * chunk + cl) * c.Hq + hq) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x2 w;
            const __bf16 e0 = (__bf16)(st.o[rb][db][0] * inv), e1 = (__bf16)(st.o[rb][db][1] * inv);
            const __bf16 e2 = (__bf16)(st.o[rb][db][2] * inv), e3 = (__bf16)(st.o[rb][db][3] * inv);
            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
            *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * lg) = w;
        }
        if (lse != nullptr && lg == 0)
            lse[((size_t)b * chunk + cl) * c.Hq + hq] = (st.mb[rb] + __log2f(l)) * kLn2;
    }
}

template <int D, int G>
hipError_t launch_g(const DevCache& c, const void* q, const void* v, void* out, float* lse,
                    int chunk, int cur, hipStream_t s) {
    constexpr int BQ = kRows / G;
    const int n_qtiles = (chunk + BQ - 1) / BQ;
    const int total = n_qtiles * c.Hkv * c.B;
    const int grid = ((total + 7) / 8) * 8;
    if (c.Bs > 0)
        hipLaunchKernelGGL((prefill_kernel<D, G, true>), dim3(grid), dim3(kPfBlock), 0, s, c,
                           (const uint16_t*)q, (const uint16_t*)v, (uint16_t*)out, lse, chunk,
                           n_qtiles, c.len[cur]);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, false>), dim3(grid), dim3(kPfBlock), 0, s, c,
                           (const uint16_t*)q, (const uint16_t*)v, (uint16_t*)out, lse, chunk,
                           n_qtiles, c.len[cur]);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DevCache& c, const void* q, const void* v, void* out, float* lse,
                    int chunk, int cur, hipStream_t s) {
    switch (c.Hq / c.Hkv) {
        case 1: return launch_g<D, 1>(c, q, v, out, lse, chunk, cur, s);
        case 2: return launch_g<D, 2>(c, q, v, out, lse, chunk, cur, s);
        case 4: return launch_g<D, 4>(c, q, v, out, lse, chunk, cur, s);
        default: return launch_g<D, 8>(c, q, v, out, lse, chunk, cur, s);
    }
}

}  // namespace

hipError_t launch_prefill_stage(const DevCache& c, const void* k, int chunk, int cur, hipStream_t s) {
    const int items = (c.Hkv + kStageHeads - 1) / kStageHeads * (c.D / 2);
    const int threads = items >= 1024 ? 1024 : (items + 63) / 64 * 64;
    // grid: x = token, y = sequence (at most 65535 per launch)
    for (int b0 = 0; b0 < c.B; b0 += 65535) {
        const dim3 grid((unsigned)chunk, (unsigned)(c.B - b0 < 65535 ? c.B - b0 : 65535));
        if (c.D == 128)
            hipLaunchKernelGGL((stage_chunk_kernel<128>), grid, dim3(threads), 0, s, c,
                               (const uint16_t*)k, chunk, b0, c.len[cur]);
        else
            hipLaunchKernelGGL((stage_chunk_kernel<64>), grid, dim3(threads), 0, s, c,
                               (const uint16_t*)k, chunk, b0, c.len[cur]);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_prefill(const DevCache& c, const void* q, const void* v, void* out, float* lse,
                          int chunk, int cur, hipStream_t s) {
    return c.D == 128 ? launch_d<128>(c, q, v, out, lse, chunk, cur, s)
                      : launch_d<64>(c, q, v, out, lse, chunk, cur, s);
}

}  // namespace psa
