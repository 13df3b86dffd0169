// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/psa.h"

namespace psa {

constexpr int kSplitGranule = 128;   // decode split lengths are multiples of this
constexpr int kMaxGroup = 8;         // largest supported H_q / H_kv

// Device view of one cache: base pointers carved out of the caller's buffer.
struct DevCache {
    void* k;             // [B][Hkv][S][D] storage dtype
    void* v;             // [B][Hkv][S][D]
    void* pool_k;        // [n_shared][Hkv][shared_max][D] shared prefixes
    void* pool_v;
    int32_t* tags;       // [B][S]
    int32_t* len[2];     // [B] history lengths; len[cur] is current, the other is written by append
    int32_t* pre;        // [B] prefix length P_b
    int32_t* nnew;       // [B] per-call token counts (ragged append)
    int32_t* pid;        // [B] shared-prefix entry of each sequence, -1 for its own prefix
    double* inv_freq;    // [D/2] theta_i
    float* part_o;       // [B][Hq][max_splits][D] unnormalised split outputs
    float* part_ml;      // [B][Hq][max_splits][2] split max (log2 domain) and sum
    void* stage_k;       // [B][max_chunk][Hkv][D] rotated prefill-chunk keys (stored bytes)
    void* stage_q;       // [B][max_chunk][Hq][D] rotated, scaled prefill-chunk queries (bf16)
    void* stage_qp;      // same, rotated at the renumbered position for prefix keys (RESET)
    int32_t B, Hq, Hkv, D, Pmax, W, S, dtype, max_chunk, max_splits, n_shared, shared_max, pe_mode;
    float scale;
};

struct Layout {
    size_t k, v, pool_k, pool_v, tags, state, inv_freq, part_o, part_ml, stage_k, stage_q, stage_qp,
        total;
    int32_t S, elem, max_splits;
};

bool compute_layout(const psa_cache_desc& d, Layout* L, const char** why);

// Kernel launchers (stream-ordered, asynchronous). They return the launch status.
hipError_t launch_init(const DevCache& c, hipStream_t s);
// Start a sequence: tags -1, length `len0`, prefix length `prefix_len`, prefix entry `pid`.
hipError_t launch_seq_reset(const DevCache& c, int seq, int prefix_len, int len0, int pid, int cur,
                            hipStream_t s);
// Rotate and store `len` prefix tokens (k, v: [len][Hkv][D]) into pool entry `id`.
hipError_t launch_pool_load(const DevCache& c, int id, int len, const void* k, const void* v,
                            hipStream_t s);
// Append n tokens per sequence (n_uniform, or nnew[] on device when ragged != 0).
// k/v: [B][n_stride][Hkv][D]; k_rotated != 0 means k already holds rotated, rounded keys.
hipError_t launch_append(const DevCache& c, const void* k, const void* v, int n_stride,
                         int n_uniform, int ragged, int k_rotated, int cur, hipStream_t s);
hipError_t launch_decode_partial(const DevCache& c, const void* q, int split_tokens,
                                 int grid_splits, int cur, hipStream_t s);
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
// Rotate a prefill chunk's keys (stored bytes) and queries (scaled, bf16) into the staging
// buffers, then attend (bf16 storage only).
hipError_t launch_prefill_stage(const DevCache& c, const void* q, const void* k, int chunk,
                                int cur, hipStream_t s);
hipError_t launch_prefill(const DevCache& c, const void* v, void* out, float* lse, int chunk,
                          int cur, hipStream_t s);

}  // namespace psa
