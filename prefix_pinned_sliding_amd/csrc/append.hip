// Ring append with rotary encoding at the absolute position (K1) and the fills used by
// cache creation and sequence reset.
//
// [PS] 03 generation loop: the prefix KV is kept for good, each new token joins the
// window, and the window drops its oldest token once it holds more than W.
// [PS] 05 Continue PE: positions keep counting up, so a key is rotated once, at its
// absolute position, and reused unchanged while it stays cached.
// [KV-Lean] 3.2: every slot carries the absolute position of the token it holds.
#include "psa_internal.h"
#include "rope_round.h"

namespace psa {
namespace {

constexpr int kBlock = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Storage element types: bf16 is kept as raw 16-bit patterns.
template <int DT> struct Elem;
template <> struct Elem<PSA_BF16> { using T = uint16_t; };
template <> struct Elem<PSA_F32> { using T = float; };

__device__ __forceinline__ double to_f64(uint16_t b) { return bf16_bits_to_f64(b); }
__device__ __forceinline__ double to_f64(float f) { return (double)f; }

__device__ __forceinline__ uint16_t store_as(double x, uint16_t*) { return f64_to_bf16_bits(x); }
__device__ __forceinline__ float store_as(double x, float*) { return (float)x; }

// Tags -1; lengths, prefix lengths and token counts 0; prefix entries -1 (own prefix);
// decode order the identity; block-table entries -1 (paged).
__global__ void init_kernel(int32_t* tags, size_t n_tags, int32_t* state, int n_zero,
                            int32_t* pid, int32_t* order, int B, int32_t* btab, size_t n_btab) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_tags) tags[i] = -1;
    if (i < (size_t)n_zero) state[i] = 0;
    if (i < (size_t)B) {
        pid[i] = -1;
        order[i] = (int32_t)i;
    }
    if (i < n_btab) btab[i] = -1;
}

// Paged: block-table entries chosen by the host's block allocator.
__global__ void table_update_kernel(int32_t* btab, TableUpdate u) {
    const int i = threadIdx.x;
    if (i < u.n) btab[u.idx[i]] = u.blk[i];
}

// A new sequence pins its first prefix_len tokens and uses the full window length W.
__global__ void seq_reset_kernel(DevCache c, int32_t* len_cur, int seq, int prefix_len, int len0,
                                 int prefix_id) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < c.S) c.tags[(size_t)seq * c.S + i] = -1;
    if (i < c.NBT) c.btab[(size_t)seq * c.NBT + i] = -1;   // paged: blocks go back to the pool
    if (i == 0) {
        len_cur[seq] = len0;
        c.pre[seq] = prefix_len;
        c.pid[seq] = prefix_id;
        c.npin[seq] = prefix_len;
        c.wfloor[seq] = prefix_len;
        c.wlen[seq] = c.W;
    }
}

// New window length and floor; the ring positions [lo, hi) leave the window (their slots
// are not reused by the new window, so their tags go back to -1).
__global__ void seq_window_kernel(DevCache c, int seq, int wlen, int wfloor, int lo, int hi) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int p = lo + i;
    if (p < hi) c.tags[(size_t)seq * c.S + c.Pmax + (p - c.pre[seq]) % c.W] = -1;
    if (i == 0) {
        c.wlen[seq] = wlen;
        c.wfloor[seq] = wfloor;
    }
}

// Promotion copies the stored bytes of window positions [wb, wb + count) from their ring
// slots to prefix slots npin, npin + 1, ...: keys are stored rotated at their absolute
// positions, which they keep. One thread per (token, KV head, 4-byte word of a row).
__global__ __launch_bounds__(kBlock) void promote_kernel(DevCache c, int seq, int wb, int count,
                                                         int npin, int row_words) {
    const size_t idx = (size_t)blockIdx.x * kBlock + threadIdx.x;
    const size_t total = (size_t)count * c.Hkv * row_words;
    if (idx >= total) return;
    const int w = (int)(idx % row_words);
    const size_t r = idx / row_words;
    const int h = (int)(r % c.Hkv);
    const int j = (int)(r / c.Hkv);
    const int p = wb + j;
    const int from = c.Pmax + (p - c.pre[seq]) % c.W;
    const int to = npin + j;
    const size_t rf = kv_rowidx(c, seq, h, from), rt = kv_rowidx(c, seq, h, to);
    uint32_t* K = (uint32_t*)c.k;
    uint32_t* V = (uint32_t*)c.v;
    K[rt * row_words + w] = K[rf * row_words + w];
    V[rt * row_words + w] = V[rf * row_words + w];
    if (h == 0 && w == 0) {
        c.tags[(size_t)seq * c.S + to] = p;
        c.tags[(size_t)seq * c.S + from] = -1;
    }
    if (idx == 0) {
        c.npin[seq] = npin + count;
        c.wfloor[seq] = wb + count;
    }
}

// One thread per (token j, KV head h, pair i) of a shared prefix: position p = j, stored
// exactly as psa_append stores a prefix token (rotated at p, rounded once).
template <int DT, int D>
__global__ __launch_bounds__(kBlock) void pool_load_kernel(DevCache c, int id, int len,
                                                           const typename Elem<DT>::T* k,
                                                           const typename Elem<DT>::T* v) {
    using T = typename Elem<DT>::T;
    constexpr int H = D / 2;
    const size_t idx = (size_t)blockIdx.x * kBlock + threadIdx.x;
    const size_t total = (size_t)len * c.Hkv * H;
    if (idx >= total) return;
    const int i = (int)(idx % H);
    const size_t r = idx / H;
    const int h = (int)(r % c.Hkv);
    const int j = (int)(r / c.Hkv);
    const size_t src = ((size_t)j * c.Hkv + h) * D;
    const size_t dst = (((size_t)id * c.Hkv + h) * c.shared_max + j) * D;
    double sn, cs, xr, yr;
    angle_sincos(j, c.inv_freq[i], &sn, &cs);
    rotate_with(to_f64(k[src + i]), to_f64(k[src + i + H]), sn, cs, &xr, &yr);
    T* K = (T*)c.pool_k;
    T* V = (T*)c.pool_v;
    K[dst + i] = store_as(xr, (T*)nullptr);
    K[dst + i + H] = store_as(yr, (T*)nullptr);
    V[dst + i] = v[src + i];
    V[dst + i + H] = v[src + i + H];
}

// One block per (token j, sequence b0 + blockIdx.y); its threads take the token's
// (KV head h, rotation pair i) items, at most one per thread when H_kv * D / 2 <= 1024.
// Each thread reads its inputs before its first store: a store could alias them as far as
// the compiler knows, so a load issued after one would wait for it.
template <int DT, int D>
__global__ __launch_bounds__(1024) void append_kernel(DevCache c, const typename Elem<DT>::T* k,
                                                      const typename Elem<DT>::T* v, int n_stride,
                                                      int n_uniform, int ragged, int k_rotated,
                                                      int b0, const int32_t* __restrict__ len_cur,
                                                      int32_t* __restrict__ len_next) {
    using T = typename Elem<DT>::T;
    constexpr int H = D / 2;
    const int j = blockIdx.x, b = b0 + blockIdx.y;
    const int items = c.Hkv * H;
    const size_t row0 = ((size_t)b * n_stride + j) * c.Hkv;   // input row of head 0
    const int nb = ragged ? c.nnew[b] : n_uniform;
    const int L0 = len_cur[b];
    for (int t = threadIdx.x; t < items; t += blockDim.x) {
        const int h = t / H, i = t % H;
        const size_t src = (row0 + h) * D;
        const T kx = k[src + i], ky = k[src + i + H];
        const T vx = v[src + i], vy = v[src + i + H];
        const double theta = c.inv_freq[i];
        const int slot = token_slot(c, b, j, nb, L0, t == 0, len_next);
        if (slot < 0) return;
        const size_t dst = kv_rowidx(c, b, h, slot) * D;
        T* K = (T*)c.k;
        T* V = (T*)c.v;
        if (k_rotated) {
            K[dst + i] = kx;
            K[dst + i + H] = ky;
        } else {
            double sn, cs, xr, yr;
            angle_sincos(L0 + j, theta, &sn, &cs);
            rotate_with(to_f64(kx), to_f64(ky), sn, cs, &xr, &yr);
            K[dst + i] = store_as(xr, (T*)nullptr);
            K[dst + i + H] = store_as(yr, (T*)nullptr);
        }
        V[dst + i] = vx;
        V[dst + i + H] = vy;
    }
}

// Append of keys that are already rotated and rounded (a prefill chunk's staged keys) and
// their values: the same slots, evictions and tags as append_kernel, moved 16 bytes at a
// time. One block per (token j, sequence b0 + blockIdx.y); its threads take the token's
// (KV head, 16-byte chunk) items.
template <int DT, int D>
__global__ __launch_bounds__(1024) void commit_kernel(DevCache c, const uint32_t* k,
                                                      const uint32_t* v, int n_stride, int b0,
                                                      const int32_t* __restrict__ len_cur,
                                                      int32_t* __restrict__ len_next) {
    using T = typename Elem<DT>::T;
    constexpr int CPR = D * (int)sizeof(T) / 16;      // 16-byte chunks per row
    const int j = blockIdx.x, b = b0 + blockIdx.y;
    const int items = c.Hkv * CPR;
    const size_t row0 = ((size_t)b * n_stride + j) * c.Hkv;
    const int L0 = len_cur[b];
    for (int t = threadIdx.x; t < items; t += blockDim.x) {
        const int h = t / CPR, ch = t % CPR;
        const size_t src = (row0 + h) * CPR + ch;
        const u32x4 kk = reinterpret_cast<const u32x4*>(k)[src];   // before any store
        const u32x4 vv = reinterpret_cast<const u32x4*>(v)[src];
        const int slot = token_slot(c, b, j, n_stride, L0, t == 0, len_next);
        if (slot < 0) return;
        const size_t dst = kv_rowidx(c, b, h, slot) * CPR + ch;
        reinterpret_cast<u32x4*>(c.k)[dst] = kk;
        reinterpret_cast<u32x4*>(c.v)[dst] = vv;
    }
}

inline unsigned blocks_for(size_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

}  // namespace

hipError_t launch_init(const DevCache& c, hipStream_t s) {
    const size_t n_tags = (size_t)c.B * c.S;
    const int n_zero = 4 * c.B;   // len[0], len[1], pre, nnew are contiguous; the rest is set
                                  // by the reset of each sequence
    const size_t n = n_tags > (size_t)n_zero ? n_tags : (size_t)n_zero;
    const size_t n_btab = (size_t)c.B * c.NBT;
    const size_t m = n > n_btab ? n : n_btab;
    hipLaunchKernelGGL(init_kernel, dim3(blocks_for(m)), dim3(kBlock), 0, s, c.tags, n_tags,
                       c.len[0], n_zero, c.pid, c.order, c.B, c.btab, n_btab);
    return hipGetLastError();
}

hipError_t launch_table_update(const DevCache& c, const TableUpdate& u, hipStream_t s) {
    if (u.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(table_update_kernel, dim3(1), dim3(kTableUpdates), 0, s, c.btab, u);
    return hipGetLastError();
}

hipError_t launch_order_update(const DevCache& c, const TableUpdate& u, hipStream_t s) {
    if (u.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(table_update_kernel, dim3(1), dim3(kTableUpdates), 0, s, c.order, u);
    return hipGetLastError();
}

hipError_t launch_seq_reset(const DevCache& c, int seq, int prefix_len, int len0, int pid, int cur,
                            hipStream_t s) {
    hipLaunchKernelGGL(seq_reset_kernel, dim3(blocks_for((size_t)c.S)), dim3(kBlock), 0, s, c,
                       c.len[cur], seq, prefix_len, len0, pid);
    return hipGetLastError();
}

hipError_t launch_seq_window(const DevCache& c, int seq, int wlen, int wfloor, int clr_lo,
                             int clr_hi, hipStream_t s) {
    const int n = clr_hi > clr_lo ? clr_hi - clr_lo : 1;
    hipLaunchKernelGGL(seq_window_kernel, dim3(blocks_for((size_t)n)), dim3(kBlock), 0, s, c, seq,
                       wlen, wfloor, clr_lo, clr_hi);
    return hipGetLastError();
}

hipError_t launch_promote(const DevCache& c, int seq, int wb, int count, int npin, hipStream_t s) {
    const int row_words = c.D * (c.dtype == PSA_BF16 ? 2 : 4) / 4;
    const size_t total = (size_t)count * c.Hkv * row_words;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(promote_kernel, dim3(blocks_for(total)), dim3(kBlock), 0, s, c, seq, wb,
                       count, npin, row_words);
    return hipGetLastError();
}

hipError_t launch_pool_load(const DevCache& c, int id, int len, const void* k, const void* v,
                            hipStream_t s) {
    const size_t total = (size_t)len * c.Hkv * (c.D / 2);
    if (total == 0) return hipSuccess;
    const dim3 grid(blocks_for(total));
#define PSA_POOL(DT, DD)                                                                   \
    hipLaunchKernelGGL((pool_load_kernel<DT, DD>), grid, dim3(kBlock), 0, s, c, id, len, \
                       (const typename Elem<DT>::T*)k, (const typename Elem<DT>::T*)v)
    if (c.dtype == PSA_BF16) {
        if (c.D == 128) PSA_POOL(PSA_BF16, 128); else PSA_POOL(PSA_BF16, 64);
    } else {
        if (c.D == 128) PSA_POOL(PSA_F32, 128); else PSA_POOL(PSA_F32, 64);
    }
#undef PSA_POOL
    return hipGetLastError();
}

hipError_t launch_append(const DevCache& c, const void* k, const void* v, int n_stride,
                         int n_uniform, int ragged, int k_rotated, int cur, hipStream_t s) {
    if (n_stride == 0) return hipSuccess;
    const bool commit = k_rotated && !ragged && n_uniform == n_stride &&
                        (((uintptr_t)k | (uintptr_t)v) & 15u) == 0;
    const int per_row = commit ? c.D * (c.dtype == PSA_BF16 ? 2 : 4) / 16 : c.D / 2;
    const int items = c.Hkv * per_row;
    const int threads = items >= 1024 ? 1024 : (items + 63) / 64 * 64;
    // grid: x = token, y = sequence (at most 65535 per launch)
    for (int b0 = 0; b0 < c.B; b0 += 65535) {
        const dim3 grid((unsigned)n_stride, (unsigned)(c.B - b0 < 65535 ? c.B - b0 : 65535));
        if (commit) {
#define PSA_COMMIT(DT, DD)                                                                   \
    hipLaunchKernelGGL((commit_kernel<DT, DD>), grid, dim3(threads), 0, s, c, (const uint32_t*)k, \
                       (const uint32_t*)v, n_stride, b0, c.len[cur], c.len[cur ^ 1])
            if (c.dtype == PSA_BF16) {
                if (c.D == 128) PSA_COMMIT(PSA_BF16, 128); else PSA_COMMIT(PSA_BF16, 64);
            } else {
                if (c.D == 128) PSA_COMMIT(PSA_F32, 128); else PSA_COMMIT(PSA_F32, 64);
            }
#undef PSA_COMMIT
        } else {
#define PSA_APPEND(DT, DD)                                                                     \
    hipLaunchKernelGGL((append_kernel<DT, DD>), grid, dim3(threads), 0, s, c,                  \
                       (const typename Elem<DT>::T*)k, (const typename Elem<DT>::T*)v, n_stride, \
                       n_uniform, ragged, k_rotated, b0, c.len[cur], c.len[cur ^ 1])
            if (c.dtype == PSA_BF16) {
                if (c.D == 128) PSA_APPEND(PSA_BF16, 128); else PSA_APPEND(PSA_BF16, 64);
            } else {
                if (c.D == 128) PSA_APPEND(PSA_F32, 128); else PSA_APPEND(PSA_F32, 64);
            }
#undef PSA_APPEND
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace psa
