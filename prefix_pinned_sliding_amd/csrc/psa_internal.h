// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/psa.h"

namespace psa {

constexpr int kSplitGranule = 128;   // decode split lengths are multiples of this
constexpr int kMaxGroup = 8;         // largest supported H_q / H_kv
constexpr int kMaxGridYZ = 65535;    // largest grid y / z dimension the launches use

// Device view of one cache: base pointers carved out of the caller's buffer.
struct DevCache {
    void* k;             // [B][Hkv][S][D] storage dtype, or paged [Hkv][n_blocks][Bs][D]
    void* v;             // same layout as k
    void* pool_k;        // [n_shared][Hkv][shared_max][D] shared prefixes
    void* pool_v;
    int32_t* tags;       // [B][S]
    int32_t* btab;       // paged: [B][NBT] physical block of each logical block, -1 if none
    int32_t* len[2];     // [B] history lengths; len[cur] is current, the other is written by append
    int32_t* pre;        // [B] prefix length P_b
    int32_t* nnew;       // [B] per-call token counts (ragged append)
    int32_t* pid;        // [B] shared-prefix entry of each sequence, -1 for its own prefix
    int32_t* npin;       // [B] pinned entries once the prefix is complete (P_b + promoted)
    int32_t* wfloor;     // [B] no window entry is older than this position
    int32_t* wlen;       // [B] the sequence's window length w_b (<= W)
    int32_t* order;      // [B] decode workgroup order: grid index y -> sequence (longest first)
    double* inv_freq;    // [D/2] theta_i
    float* part_o;       // [B][Hq][max_splits][D] unnormalised split outputs
    float* part_ml;      // [B][Hq][max_splits][2] split max (log2 domain) and sum
    void* stage_k;       // [B][max_chunk][Hkv][D] rotated prefill-chunk keys (stored bytes)
    // W: ring slots per (sequence, head), the largest window any sequence may use
    int32_t B, Hq, Hkv, D, Pmax, W, S, dtype, max_chunk, max_splits, n_shared, shared_max, pe_mode;
    int32_t Bs, bshift, NBT, n_blocks;   // paged: block size (0: contiguous), log2, S / Bs
    float scale;
};

// Row (kv_rowidx) and element offset (kv_row) of logical slot `slot` of (sequence b, KV
// head h) in K or V: contiguous [B][Hkv][S][D], or paged [Hkv][n_blocks][Bs][D] through
// the block table.
// Paged: row of row `off` (< Bs) of physical block `blk`, KV head h. The pool is head-major
// ([Hkv][n_blocks][Bs][D]), so a sequence's consecutive blocks are one contiguous run per
// head, which keeps its reads as long as in the contiguous layout.
__host__ __device__ inline size_t block_rowidx(int blk, int h, int off, int Bs, int nblk) {
    return ((size_t)h * nblk + blk) * Bs + off;
}
__device__ inline size_t kv_rowidx(const DevCache& c, int b, int h, int slot) {
    if (c.Bs == 0) return ((size_t)b * c.Hkv + h) * c.S + slot;
    const int blk = c.btab[b * c.NBT + (slot >> c.bshift)];
    return block_rowidx(blk, h, slot & (c.Bs - 1), c.Bs, c.n_blocks);
}
__device__ inline size_t kv_row(const DevCache& c, int b, int h, int slot) {
    return kv_rowidx(c, b, h, slot) * c.D;
}



struct Layout {
    size_t k, v, pool_k, pool_v, tags, btab, state, inv_freq, part_o, part_ml, stage_k, total;
    int32_t S, elem, max_splits, n_blocks;
};

constexpr int kMaxBlockTable = 1024;   // paged: largest S / block_size
constexpr int kTableUpdates = 120;     // block-table entries one update launch carries

bool compute_layout(const psa_cache_desc& d, Layout* L, const char** why);

// What sequence b holds when its history has n tokens. Positions p < P_b fill prefix slot
// p; every later position p sits in ring slot (p - P_b) mod W. The window is the position
// range [wb, n) with wb = max(wfloor, n - w_b): appends move it by the length rule alone,
// while a window change or a promotion raises wfloor. Promoted entries occupy prefix
// slots P_b .. npin - 1, and every window position is >= npin.
struct SeqView {
    int n_pre;   // prefix slots in use: min(n, npin)
    int wb;      // oldest window position
    int n_win;   // window entries, max(0, n - wb)
    int head;    // ring slot of the oldest window entry (0 when all W slots are live)
};

__host__ __device__ inline SeqView seq_view(int n, int P, int npin, int wfloor, int wlen, int W) {
    SeqView v;
    v.n_pre = n < npin ? n : npin;
    v.wb = n - wlen > wfloor ? n - wlen : wfloor;
    v.n_win = n > v.wb ? n - v.wb : 0;
    v.head = v.n_win == W ? 0 : (v.wb - P) % W;
    return v;
}

__device__ inline SeqView seq_view(const DevCache& c, int b, int n) {
    return seq_view(n, c.pre[b], c.npin[b], c.wfloor[b], c.wlen[b], c.W);
}

// Where token j of sequence b goes when the sequence appends nb tokens (nb from the
// launch). Token j has position p = len[b] + j. Slot: p < P_b -> prefix slot p; else ring
// slot P_max + (p - P_b) mod W. The window after the call is [wb', n') with
// wb' = max(wfloor, n' - w_b); a token older than wb' (dropped again within the call) is
// not written (slot -1), so the writer of each slot is unique. Window entries that the
// call drops and whose slots no new token takes (possible when w_b < W) get tag -1: token
// j clears the j-th of them (there are at most nb). Run by one thread of the token's block
// (`lead`), which also writes the tag and, for j = 0, the new length.
__device__ inline int token_slot(const DevCache& c, int b, int j, int nb, int L0,
                                          bool lead, int32_t* len_next) {
    if (lead && j == 0) len_next[b] = L0 + nb;
    if (j >= nb) return -1;
    const int p = L0 + j;
    const int P = c.pre[b];
    const int wf = c.wfloor[b], wl = c.wlen[b];
    const int n1 = L0 + nb;
    const int wb1 = max(wf, n1 - wl);                // window base after the call
    if (lead && wl < c.W) {
        const int e = max(wf, L0 - wl) + j;          // j-th entry leaving the window
        if (e < min(L0, wb1)) {
            const int d = (wb1 - e) % c.W;           // e's slot relative to wb1's, mod W
            const int rel = d == 0 ? 0 : c.W - d;
            if (rel >= n1 - wb1) c.tags[(size_t)b * c.S + c.Pmax + (e - P) % c.W] = -1;
        }
    }
    int slot;
    if (p < P) {
        slot = p;
    } else {
        if (p < wb1) return -1;                      // dropped within this call
        slot = c.Pmax + (p - P) % c.W;
    }
    if (lead) c.tags[(size_t)b * c.S + slot] = p;
    return slot;
}

// Kernel launchers (stream-ordered, asynchronous). They return the launch status.
hipError_t launch_init(const DevCache& c, hipStream_t s);
// Write n (<= kTableUpdates) block-table entries: btab[idx[i]] = blk[i].
struct TableUpdate {
    int32_t n;
    int32_t idx[kTableUpdates];
    int32_t blk[kTableUpdates];
};
hipError_t launch_table_update(const DevCache& c, const TableUpdate& u, hipStream_t s);
// The same for the decode order: order[idx[i]] = blk[i] (blk holds sequence indices).
hipError_t launch_order_update(const DevCache& c, const TableUpdate& u, hipStream_t s);
// Start a sequence: tags -1, length `len0`, prefix length `prefix_len`, prefix entry `pid`.
hipError_t launch_seq_reset(const DevCache& c, int seq, int prefix_len, int len0, int pid, int cur,
                            hipStream_t s);
// Set a sequence's window length and floor; clear the tags of ring positions [clr_lo, clr_hi).
hipError_t launch_seq_window(const DevCache& c, int seq, int wlen, int wfloor, int clr_lo,
                             int clr_hi, hipStream_t s);
// Move window positions [wb, wb + count) of sequence seq from their ring slots to prefix
// slots npin .. npin + count - 1, then npin += count and wfloor = wb + count.
hipError_t launch_promote(const DevCache& c, int seq, int wb, int count, int npin, hipStream_t s);
// Rotate and store `len` prefix tokens (k, v: [len][Hkv][D]) into pool entry `id`.
hipError_t launch_pool_load(const DevCache& c, int id, int len, const void* k, const void* v,
                            hipStream_t s);
// Append n tokens per sequence (n_uniform, or nnew[] on device when ragged != 0).
// k/v: [B][n_stride][Hkv][D]; k_rotated != 0 means k already holds rotated, rounded keys.
hipError_t launch_append(const DevCache& c, const void* k, const void* v, int n_stride,
                         int n_uniform, int ragged, int k_rotated, int cur, hipStream_t s);
// Decode partials over the state len[cur]; with k_new != nullptr, first append one token
// per sequence (k_new, v_new: [B][Hkv][D]) and decode over len[cur] + 1, writing the new
// lengths to len[cur ^ 1].
hipError_t launch_decode_partial(const DevCache& c, const void* q, int split_tokens,
                                 int grid_splits, int cur, const void* k_new, const void* v_new,
                                 hipStream_t s);
// Decode splits of a sequence with n_pre prefix and n_win window entries. CONTINUE cuts the
// concatenated list; RESET cuts the prefix and the window separately, so a split never
// mixes keys that need differently rotated queries.
__host__ __device__ inline int split_count(int n_pre, int n_win, int L, int pe_mode) {
    if (pe_mode == PSA_PE_RESET) return (n_pre + L - 1) / L + (n_win + L - 1) / L;
    return (n_pre + n_win + L - 1) / L;
}

// Workgroups of the decode kernel (for this cache's shape) that fit on the device at once.
int decode_resident_wgs(const DevCache& c);
hipError_t launch_merge(const DevCache& c, void* out, float* lse, int split_tokens, int cur,
                        hipStream_t s);
// Rotate a prefill chunk's keys into the staging buffer (the bytes the cache will hold),
// then attend: the attention kernel rotates and scales the queries itself (bf16 storage
// only).
hipError_t launch_prefill_stage(const DevCache& c, const void* k, int chunk, int cur, hipStream_t s);
hipError_t launch_prefill(const DevCache& c, const void* q, const void* v, void* out, float* lse,
                          int chunk, int cur, hipStream_t s);

// Training attention (row space): forward writes out and lse; backward reads q, k, v,
// out, lse, dout and writes dq, dk, dv (di: float32 workspace [B][T][Hq]).
struct TrainLaunch {
    const void *q, *k, *v, *dout;
    void *out, *dq, *dk, *dv;
    float *lse, *di;
    const int32_t *pre, *len;   // device [B]
    int B, T, Hq, Hkv, D, W;
    float scale;
    bool backward;
};
hipError_t launch_train(const TrainLaunch& t, hipStream_t s);

}  // namespace psa
