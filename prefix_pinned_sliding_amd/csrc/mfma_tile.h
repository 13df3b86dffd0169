// Register and LDS helpers shared by the MFMA attention kernels (prefill and training).
//
// Layout of v_mfma_f32_16x16x32_bf16 on a wave of 64 lanes, l16 = lane % 16, lg = lane / 16:
// operand A (16 x 32): lane holds row l16, k = 8 lg .. 8 lg + 7;
// operand B (32 x 16): lane holds column l16, k = 8 lg .. 8 lg + 7;
// result (16 x 16): lane holds rows 4 lg .. 4 lg + 3 of column l16.
// The k order inside one instruction is free as long as A and B use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNeg = -1.0e30f;        // initial running max (finite: -inf - kNeg = -inf)
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr float kRescaleSlack = 8.0f;

constexpr int kTileKeys = 64;           // keys per attention tile
// LDS row stride of V tiles (elements): V is read only with transposing 8-byte loads that
// take 4 rows x 32 bytes at once, and an 8-bank offset between rows (D + 16) keeps them
// apart. K tiles (and every tile read as 16-byte row operands) are unpadded and swizzled
// (chunk_swz).
constexpr int kVPad = 16;

// Unpadded LDS tiles: the 16-byte chunk c of row r is stored at chunk c ^ chunk_swz<D>(r).
// Measured on gfx950 with single-pattern probes: a 16-byte LDS read (ds_read_b128) is
// served in four groups of 16 lanes, each group the lanes that share lane bit 5 and the
// parity of lane bits 2..4; it runs at full rate (about 215 B/clk per CU) when the 16 lanes
// of each group hit 16 distinct 16-byte bank groups (address bits 4..7), and at half rate
// when two share one. A transposing 8-byte read (ds_read_b64_tr_b16) runs at its full rate
// (about 150 B/clk) when each half of the wave (lanes 0..31, 32..63) hits 32 distinct
// 8-byte slots of the 256-byte bank cycle. The row-operand reads (lane (l16, lg) of a
// 16-row block: row l16, chunk 4 ks + lg) and the transposing reads (rows 4 lg + l16 / 4,
// a chunk pair) both meet those conditions with c ^ 2 (r & 7) for 256-byte rows (D = 128)
// and c ^ (r & 6) for 128-byte rows (D = 64). Padded rows (stride D + 8) and the XOR with
// r & 15 put two lanes of a group on one bank group (half rate) for the row reads; r & 15
// also halves the transposing reads.
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
    static_assert(D == 64 || D == 128, "head dims 64 and 128");
    if constexpr (D == 128) return (2 * r) & 14;
    else return r & 6;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) {
    return __builtin_bit_cast(bf16x8, w);
}

// Max over lanes l, l^16, l^32, l^48 (the four lane groups holding one row).
__device__ __forceinline__ float row_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float row_sum4(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed MFMA operand from a row-major bf16 tile in LDS (ds_read_b64_tr_b16, gfx950).
// Within each 16-lane group the instruction takes the 16 lanes' 4-element reads as a 16 x 4
// tile T and hands lane i the elements T[i / 4 + 4 j][i % 4], j = 0..3. So if lane k of a
// group reads row r0 + k / 4 at column c0 + 4 (k % 4), lane i receives column c0 + i of
// rows r0 .. r0 + 3. Two reads (rows r0 .. r0 + 3 and r1 .. r1 + 3) fill the 8 k-values of
// one operand. `p0`, `p1`: this lane's addresses for the two reads (8-byte aligned).
__device__ __forceinline__ bf16x8 lds_read_tr2(const uint16_t* p0, const uint16_t* p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// Two bf16 values packed into one 32-bit word (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Registers -> LDS (consecutive lanes on consecutive 16-byte chunks of a row): K rows
// unpadded with their chunks swizzled (chunk_swz), V rows padded to VSTR; V^T operands
// are read back with transposing LDS loads.
template <int D, int BN, int NT, int VSTR>
__device__ __forceinline__ void stage_tile(uint16_t* k_s, uint16_t* v_s, int tid,
                                           const u32x4* kreg, const u32x4* vreg) {
    constexpr int CPR = D / 8;
    constexpr int KLD = (BN * CPR) / NT;
#pragma unroll
    for (int rr = 0; rr < KLD; ++rr) {
        const int ci = tid + NT * rr;
        const int kk = ci / CPR, col = ci % CPR;
        *reinterpret_cast<u32x4*>(k_s + kk * D + (col ^ chunk_swz<D>(kk)) * 8) = kreg[rr];
        *reinterpret_cast<u32x4*>(v_s + kk * VSTR + col * 8) = vreg[rr];
    }
}

// This lane's K operand offsets within a 16-row block (elements, from the block's first
// row): row l16, chunk 4 ks + lg, swizzled, for each k-step ks.
template <int D>
__device__ __forceinline__ void k_operand_offsets(int (&ko)[D / 32], int l16, int lg) {
    const int swz = chunk_swz<D>(l16);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) ko[ks] = l16 * D + ((4 * ks + lg) ^ swz) * 8;
}

// Online-softmax state of one lane's two row blocks. m: running maximum (log2 domain),
// kNeg until a row has seen a visible key; mb: the value the S accumulator starts from
// (m once set, else 0), so the products arrive already shifted and exp2 needs no
// subtraction; o: O^T accumulators; l: row sums, accumulated by an MFMA against an all-ones
// A operand (every element of l[rb] holds the row's sum of the bf16-rounded probabilities,
// the same values that weight V).
template <int DB>
struct SoftmaxRows {
    f32x4 o[2][DB];
    f32x4 l[2];
    float m[2], mb[2];
};

// The three phases of one 64-key tile for a wave's 32 rows. tile_qk: S^T = K Q^T - mb.
// tile_softmax: tile_max (the mask, edge tiles only, and the running-max update, rescaling
// O and l when it moves), then P^T = exp2(S^T) as bf16 B operands. tile_pv: l += 1 P^T and
// O^T += V^T P^T.
//
// `sc` converts products to the log2 domain: 1 when the queries were loaded already scaled
// by scale * log2(e) (prefill), scale * log2(e) otherwise (training). The accumulators
// then start at -mb / sc, and exp2 takes sc times the product.
template <int D>
__device__ __forceinline__ void tile_qk(f32x4 (&s)[2][kTileKeys / 16], const SoftmaxRows<D / 16>& st,
                                        const bf16x8 (&qop)[2][D / 32], const uint16_t* k_s,
                                        int l16, int lg, float inv_sc) {
    constexpr int KS = D / 32, KB = kTileKeys / 16;
    const float s0 = -st.mb[0] * inv_sc, s1 = -st.mb[1] * inv_sc;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        s[0][kb] = f32x4{s0, s0, s0, s0};
        s[1][kb] = f32x4{s1, s1, s1, s1};
    }
    // k-step outer: the 8 accumulators are independent within a step. A step's K operands
    // are read two steps ahead (a ring of three), so each read has two steps of products
    // to land in; scheduling barriers keep that order.
    int ko[KS];
    k_operand_offsets<D>(ko, l16, lg);
    bf16x8 ka[3][KB];
    auto kread = [&](int ks) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            ka[ks % 3][kb] = as_bf16x8(*reinterpret_cast<const u32x4*>(k_s + kb * 16 * D + ko[ks]));
    };
    kread(0);
    if (KS > 1) kread(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) kread(ks + 2);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % 3][kb], qop[0][ks], s[0][kb], 0, 0, 0);
            s[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % 3][kb], qop[1][ks], s[1][kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__device__ __forceinline__ bool tile_max(f32x4 (&s)[2][kTileKeys / 16],
                                         SoftmaxRows<D / 16>& st, const int (&row_pos)[2],
                                         int ct0, int t1, int P, int W, int lg, bool masked,
                                         float sc, float inv_sc) {
    constexpr int DB = D / 16, KB = kTileKeys / 16;
    // Masked logits become -inf: exp2(-inf) is 0 for any finite shift.
    float ml[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        if (masked) {
            // key j = jb + c (c = 16 kb + i) is visible iff c <= hi and c is not in the gap
            // [pe, pe + gap) between the prefix and the window
            const int p = row_pos[rb];
            int jb = ct0 + 4 * lg;
            asm volatile("" : "+v"(jb));   // keeps the mask's arithmetic inside this branch
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
        ml[rb] = fmaxf(s[rb][0][0], s[rb][0][1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = (kb == 0 ? 2 : 0); i < 4; i += 2)
                ml[rb] = __builtin_fmaxf(__builtin_fmaxf(ml[rb], s[rb][kb][i]), s[rb][kb][i + 1]);
    }
    // The running max of a row only moves when some lane's own max exceeds it by the slack
    // (or the row has none yet); test that with one ballot, do the cross-lane max only then.
    const bool moved = __any(ml[0] * sc + st.mb[0] > st.m[0] + kRescaleSlack ||
                             ml[1] * sc + st.mb[1] > st.m[1] + kRescaleSlack);
    if (moved) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float mt = row_max4(ml[rb]) * sc + st.mb[rb];   // absolute tile max
            const bool need = mt > st.m[rb] + kRescaleSlack;
            if (need) {
                const float f = __builtin_amdgcn_exp2f(st.m[rb] - mt);
                const float shift = (mt - st.mb[rb]) * inv_sc;
                st.m[rb] = mt;
                st.mb[rb] = mt;
                st.l[rb] *= f;
#pragma unroll
                for (int db = 0; db < DB; ++db) st.o[rb][db] *= f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) s[rb][kb] -= shift;
            }
        }
    }
    return moved;
}

// tile_max for a reference pinned at 0 (prefill, products already in the log2 domain).
// The values subtracted from the logits, mb, stay 0 for every row whose logits stay within
// +-kRefRange of 0: then exp2 of a product is at most 2^kRefRange, the row sums and outputs
// stay far inside float32, and no tile needs a rescale. m holds the trigger, mb + kRefRange
// once the row has seen a key (kNeg before). A row's first visible tile keeps mb = 0 if its
// maximum lies in [-kRefRange, kRefRange], else takes that maximum; a later tile moves mb
// (rescaling O and l) only past mb + kRefRange. Returns whether some row of the wave changed
// its reference (then exponentials taken against the old one are stale).
constexpr float kRefRange = 64.0f;

template <int D>
__device__ __forceinline__ bool tile_max_pinned(f32x4 (&s)[2][kTileKeys / 16],
                                                SoftmaxRows<D / 16>& st, const int (&row_pos)[2],
                                                int ct0, int t1, int P, int W, int lg, bool masked) {
    constexpr int DB = D / 16, KB = kTileKeys / 16;
    float ml[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        if (masked) {
            // key j = jb + c of this lane (c = 16 kb + i) is visible iff j < t1, j <= p and
            // j is not in the gap [P, p - W + 1) between the prefix and the window: in c,
            // c <= hi and (unsigned)(c - pe) >= gap
            const int p = row_pos[rb];
            int jb = ct0 + 4 * lg;
            asm volatile("" : "+v"(jb));   // keeps the mask's arithmetic inside this branch
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
        ml[rb] = fmaxf(s[rb][0][0], s[rb][0][1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = (kb == 0 ? 2 : 0); i < 4; i += 2)
                ml[rb] = __builtin_fmaxf(__builtin_fmaxf(ml[rb], s[rb][kb][i]), s[rb][kb][i + 1]);
    }
    if (!__any(ml[0] + st.mb[0] > st.m[0] || ml[1] + st.mb[1] > st.m[1])) return false;
    bool changed = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float mt = row_max4(ml[rb]) + st.mb[rb];   // absolute tile max of the row
        if (mt > st.m[rb]) {
            const bool first = st.m[rb] == kNeg;
            const float nb = first && mt <= kRefRange && mt >= -kRefRange ? 0.f : mt;
            if (nb != st.mb[rb]) {
                // on the row's first visible keys O and l are still zero: the factor is not
                // formed (for a maximum below -128 it would overflow, and 0 * inf is NaN)
                const float f = first ? 0.f : __builtin_amdgcn_exp2f(st.mb[rb] - nb);
                const float shift = nb - st.mb[rb];
                st.l[rb] *= f;
#pragma unroll
                for (int db = 0; db < DB; ++db) st.o[rb][db] *= f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) s[rb][kb] -= shift;
                st.mb[rb] = nb;
                changed = true;
            }
            st.m[rb] = nb + kRefRange;
        }
    }
    return __any(changed);
}

template <int D>
__device__ __forceinline__ void tile_softmax(bf16x8 (&pb)[2][kTileKeys / 32], f32x4 (&s)[2][kTileKeys / 16],
                                             SoftmaxRows<D / 16>& st, const int (&row_pos)[2],
                                             int ct0, int t1, int P, int W, int lg, bool masked,
                                             float sc, float inv_sc) {
    constexpr int PVS = kTileKeys / 32;
    tile_max<D>(s, st, row_pos, ct0, t1, P, W, lg, masked, sc, inv_sc);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ps = 0; ps < PVS; ++ps)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pb[rb][ps][i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][2 * ps][i] * sc);
                pb[rb][ps][4 + i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][2 * ps + 1][i] * sc);
            }
}

template <int D>
__device__ __forceinline__ void tile_pv(SoftmaxRows<D / 16>& st, const bf16x8 (&pb)[2][kTileKeys / 32],
                                        const uint16_t* v_s, int l16, int lg) {
    constexpr int DB = D / 16, PVS = kTileKeys / 32;
    constexpr int VSTR = D + kVPad;
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int ps = 0; ps < PVS; ++ps) {
        st.l[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[0][ps], st.l[0], 0, 0, 0);
        st.l[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[1][ps], st.l[1], 0, 0, 0);
    }
    // V^T operand (d = 16 db + l16; keys in the order of P^T's accumulator layout:
    // 32 ps + 4 lg + j, then 32 ps + 16 + 4 lg + j) by two transposing reads of V rows
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int ps = 0; ps < PVS; ++ps) {
            const uint16_t* v0 = v_s + (32 * ps + 4 * lg + l16 / 4) * VSTR + db * 16 + 4 * (l16 % 4);
            const bf16x8 a = lds_read_tr2(v0, v0 + 16 * VSTR);
            st.o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[0][ps], st.o[0][db], 0, 0, 0);
            st.o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[1][ps], st.o[1][db], 0, 0, 0);
        }
}

// P^T operands (bf16) of keys 32 h .. 32 h + 31 of the tile, from S^T.
__device__ __forceinline__ void tile_exp_half(bf16x8 (&pb)[2], const f32x4 (&s)[2][kTileKeys / 16],
                                              int h, float sc) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pb[rb][i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][2 * h][i] * sc);
            pb[rb][4 + i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][2 * h + 1][i] * sc);
        }
}

// S^T = K Q^T - mb as tile_qk computes it, keys 0-31 first, then keys 32-63 with the P^T
// operands of keys 0-31 (`pb0`, exponentials against the running max from before this
// tile) taken between those products. pb0 holds for the tile unless the tile is masked or
// moves the running max (tile_max); the caller recomputes it then.
template <int D, bool ZERO = false>
__device__ __forceinline__ void tile_qk_exp(f32x4 (&s)[2][kTileKeys / 16], bf16x8 (&pb0)[2],
                                            const SoftmaxRows<D / 16>& st,
                                            const bf16x8 (&qop)[2][D / 32], const uint16_t* k_s,
                                            int l16, int lg, float sc, float inv_sc) {
    constexpr int KS = D / 32, KB = kTileKeys / 16;
    static_assert(KB == 4 && 16 % KS == 0, "two halves of two 16-key blocks");
    // ZERO: every row of the wave has reference 0, so the accumulators start from the
    // products' inline constant 0 instead of 32 register moves
    const float s0 = ZERO ? 0.f : -st.mb[0] * inv_sc, s1 = ZERO ? 0.f : -st.mb[1] * inv_sc;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        s[0][kb] = f32x4{s0, s0, s0, s0};
        s[1][kb] = f32x4{s1, s1, s1, s1};
    }
    // steps (half h, k-step ks) in order; each reads the K operands of its two key blocks,
    // two steps ahead (a ring of three)
    constexpr int NS = 2 * KS;
    bf16x8 ka[3][2];
    int ko[KS];
    k_operand_offsets<D>(ko, l16, lg);
    auto kread = [&](int step, int j) -> bf16x8 {
        const int h = step / KS, ks = step % KS;
        return as_bf16x8(*reinterpret_cast<const u32x4*>(k_s + (2 * h + j) * 16 * D + ko[ks]));
    };
    ka[0][0] = kread(0, 0);
    ka[0][1] = kread(0, 1);
    ka[1][0] = kread(1, 0);
    ka[1][1] = kread(1, 1);
#pragma unroll
    for (int step = 0; step < NS; ++step) {
        const int h = step / KS, ks = step % KS;
        if (step + 2 < NS) {
            ka[(step + 2) % 3][0] = kread(step + 2, 0);
            ka[(step + 2) % 3][1] = kread(step + 2, 1);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kb = 2 * h + j;
            s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % 3][j], qop[0][ks], s[0][kb], 0, 0, 0);
            s[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % 3][j], qop[1][ks], s[1][kb], 0, 0, 0);
        }
        if (h == 1) {
            // 16 / KS of the 16 exponentials of keys 0-31 per step of the second half
            constexpr int PER = 16 / KS;
#pragma unroll
            for (int e = PER * ks; e < PER * (ks + 1); ++e) {
                const int rb = e / 8, i = e % 8;
                pb0[rb][i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][i / 4][i % 4] * sc);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // keeps the exponentials here: without it the compiler sinks them past the caller's
    // branch that may recompute them
    asm volatile("" : "+v"(pb0[0]), "+v"(pb0[1]));
}

// The products of one tile, 32 keys at a time, given the P^T operands of keys 0-31. The
// wave issues in order (scheduling barriers fix it): keys 0-31's products with one
// exponential of keys 32-63 (and their V^T reads) between consecutive products, so that
// VALU work runs while the matrix core is busy, then keys 32-63's products.
template <int D>
__device__ __forceinline__ void tile_exp_pv(SoftmaxRows<D / 16>& st, const f32x4 (&s)[2][kTileKeys / 16],
                                            const bf16x8 (&pb0)[2], const uint16_t* v_s, int l16,
                                            int lg, float sc) {
    constexpr int DB = D / 16, PVS = kTileKeys / 32;
    constexpr int VSTR = D + kVPad;
    static_assert(PVS == 2 && DB >= 4, "two 32-key steps per tile, at least 16 products each");
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    const uint16_t* vrow = v_s + (4 * lg + l16 / 4) * VSTR + 4 * (l16 % 4);
    bf16x8 va[2][DB];
    bf16x8 pb1[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[0][db] = lds_read_tr2(vrow + db * 16, vrow + 16 * VSTR + db * 16);
    __builtin_amdgcn_sched_barrier(0);
    st.l[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb0[0], st.l[0], 0, 0, 0);
    st.l[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb0[1], st.l[1], 0, 0, 0);
    // 16 exponentials of keys 32-63 over keys 0-31's 2 DB products
    constexpr int PER = 16 / DB;   // exponentials per db (two products)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        st.o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0][db], pb0[0], st.o[0][db], 0, 0, 0);
        st.o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0][db], pb0[1], st.o[1][db], 0, 0, 0);
#pragma unroll
        for (int e = db * PER; e < (db + 1) * PER; ++e) {
            const int rb = e / 8, i = e % 8;
            pb1[rb][i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][2 + i / 4][i % 4] * sc);
        }
        va[1][db] = lds_read_tr2(vrow + 32 * VSTR + db * 16, vrow + 48 * VSTR + db * 16);
        __builtin_amdgcn_sched_barrier(0);
    }
    st.l[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb1[0], st.l[0], 0, 0, 0);
    st.l[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb1[1], st.l[1], 0, 0, 0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        st.o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1][db], pb1[0], st.o[0][db], 0, 0, 0);
        st.o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1][db], pb1[1], st.o[1][db], 0, 0, 0);
    }
}

// One whole tile: the three phases in order, with an optional workgroup barrier between
// the products S^T and the softmax. With kSplitExp the tile runs 32 keys at a time: keys
// 0-31's exponentials are taken during keys 32-63's S^T products (tile_qk_exp) and keys
// 32-63's during keys 0-31's PV products (tile_exp_pv). It pays where the products arrive
// in the log2 domain (sc = 1): about 1.5% on the prefill kernel; the training forward pass
// ran 3% slower with it.
// The prefill's tile: products in the log2 domain (sc = 1) and the softmax reference pinned
// at 0 (tile_max_pinned). The accumulators always start from the products' inline constant
// 0, so keys 0-31's exponentials taken during the products are against reference 0; a wave
// with some row on another reference (`shifted`, wave-uniform) subtracts it afterwards and
// takes those exponentials again.
template <int D>
__device__ __forceinline__ void tile_step_pinned(SoftmaxRows<D / 16>& st, const bf16x8 (&qop)[2][D / 32],
                                                 const uint16_t* k_s, const uint16_t* v_s,
                                                 const int (&row_pos)[2], int ct0, int t1, int P,
                                                 int W, int l16, int lg, bool masked,
                                                 bool mid_barrier, bool shifted) {
    f32x4 s[2][kTileKeys / 16];
    bf16x8 pb0[2];
    tile_qk_exp<D, true>(s, pb0, st, qop, k_s, l16, lg, 1.f, 1.f);
    if (mid_barrier) __syncthreads();
    if (shifted) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kb = 0; kb < kTileKeys / 16; ++kb) s[rb][kb] -= st.mb[rb];
    }
    if (tile_max_pinned<D>(s, st, row_pos, ct0, t1, P, W, lg, masked) || masked || shifted)
        tile_exp_half(pb0, s, 0, 1.f);
    tile_exp_pv<D>(st, s, pb0, v_s, l16, lg, 1.f);
}

template <int D, bool kSplitExp = false>
__device__ __forceinline__ void tile_step(SoftmaxRows<D / 16>& st, const bf16x8 (&qop)[2][D / 32],
                                          const uint16_t* k_s, const uint16_t* v_s,
                                          const int (&row_pos)[2], int ct0, int t1, int P, int W,
                                          int l16, int lg, bool masked, bool mid_barrier,
                                          float sc, float inv_sc) {
    f32x4 s[2][kTileKeys / 16];
    if constexpr (kSplitExp) {
        bf16x8 pb0[2];
        tile_qk_exp<D>(s, pb0, st, qop, k_s, l16, lg, sc, inv_sc);
        if (mid_barrier) __syncthreads();
        if (tile_max<D>(s, st, row_pos, ct0, t1, P, W, lg, masked, sc, inv_sc) || masked)
            tile_exp_half(pb0, s, 0, sc);
        tile_exp_pv<D>(st, s, pb0, v_s, l16, lg, sc);
    } else {
        tile_qk<D>(s, st, qop, k_s, l16, lg, inv_sc);
        if (mid_barrier) __syncthreads();
        bf16x8 pb[2][kTileKeys / 32];
        tile_softmax<D>(pb, s, st, row_pos, ct0, t1, P, W, lg, masked, sc, inv_sc);
        tile_pv<D>(st, pb, v_s, l16, lg);
    }
}

}  // namespace
}  // namespace psa
