/*
 * psa.h -- prefix-pinned sliding-window attention on AMD Instinct MI355X (gfx950).
 *
 * A bounded KV cache per sequence: a pinned prefix of P_b tokens that is never
 * evicted, plus a fixed-length window of the last W tokens with oldest-first
 * eviction; attention over exactly that set.
 *
 * Sources (cited by title and section):
 *   [PS]      "Prefix Sliding 3倍加速", PaperDaily explainer of the Prefix Sliding
 *             paper (longzhangge.com): 03 visible set A(t) and generation loop,
 *             04 cost, 05 Continue PE, 06 the two-level kernel filter.
 *   [KV-Lean] the pnsm.cn article on a Lean 4 verification of a sliding-window KV
 *             cache: 2.2-2.4 window list model and slot positions, 3.2 cells with
 *             positions, 3.3 step, 3.4 ring buffer read as a list, 5.1 not-full
 *             pitfalls, 6.3 export-and-compare checks.
 *   [PS] 14 (open questions: how coarse the pinned prefix should be, whether the window
 *             could change while generating) motivates psa_seq_set_window and
 *             psa_seq_promote.
 *
 * Conventions used by every call:
 *   - Positions are 0-based absolute token positions p (p = t - 1 for the pages'
 *     1-based t). A sequence's history length n counts every token appended so far.
 *   - The query at position p attends to key j iff j <= p and (j < P_b or
 *     j >= p - W + 1): the pinned prefix [1, P] and the window
 *     [max(P + 1, t - W + 1), t] of [PS] 03. A query inside the prefix (p < P_b)
 *     attends causally to [0, p]. W is the sequence's window length w_b (desc.window
 *     unless psa_seq_set_window changed it); after a window change or a promotion the
 *     attended set is the list model's cache (see those calls).
 *   - Keys are rotated (rotary position encoding, rotate-half pairing (i, i + D/2),
 *     theta_i = rope_base^(-2i/D)) at their absolute position once, when appended,
 *     and reused as stored ([PS] 05, "Continue PE"). The rotation is computed in
 *     float64 and rounded once (nearest, ties to even) to the storage dtype.
 *   - Grouped-query heads: query head hq reads KV head hq / (n_q_heads / n_kv_heads).
 *   - Tensors are dense, row-major, in the cache dtype unless stated otherwise.
 *   - Every device pointer is caller-owned device memory on the cache's device;
 *     the library never allocates or frees device memory. Host pointers are
 *     caller-owned host memory.
 *   - Calls taking a stream enqueue work on it and return without waiting, except
 *     psa_cache_create and psa_export, which wait for the stream. The caller
 *     serialises calls on one handle (a handle is not thread-safe). Calls on one
 *     cache must be issued on one stream (or ordered by the caller).
 *   - Errors: every argument and state error is detected on the host before any
 *     work is enqueued, and leaves the cache unchanged. PSA_ERR_HIP reports a
 *     failed HIP runtime call or launch; psa_last_error() gives the text.
 */
#ifndef PSA_H
#define PSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque host handle, owned by the library (psa_cache_create / psa_cache_destroy). */
typedef struct psa_cache psa_cache;

/* A hipStream_t passed as a plain pointer; NULL is the null stream. */
typedef void *psa_stream;

/* Status codes. */
enum {
    PSA_OK = 0,
    PSA_ERR_ARG = 1,      /* invalid argument: null pointer, unsupported shape or dtype, size */
    PSA_ERR_STATE = 2,    /* operation not valid in the cache's current state */
    PSA_ERR_OVERFLOW = 3, /* a sequence length would exceed INT32_MAX */
    PSA_ERR_HIP = 4       /* a HIP runtime call or kernel launch failed */
};

/* Storage / input dtype. */
enum { PSA_BF16 = 0, PSA_F32 = 1 };

/* Cache description. */
typedef struct {
    int32_t max_batch;   /* number of sequences B, 1 <= B <= 65535 */
    int32_t n_q_heads;   /* H_q >= 1, a multiple of n_kv_heads, H_q / H_kv in {1, 2, 4, 8} */
    int32_t n_kv_heads;  /* H_kv, 1 <= H_kv <= 65535 */
    int32_t head_dim;    /* D: 64 or 128 */
    int32_t prefix_max;  /* P_max >= 0: largest pinned-prefix length any sequence may use */
    int32_t window;      /* W >= 1: window length (the largest psa_seq_set_window accepts);
                            prefix_max + window <= 2^30, n_kv_heads * (ceil((max(prefix_max,
                            shared_prefix_max) + window) / 128) + 1) < 2^24, and W < 2^24
                            when max_chunk > 0 */
    int32_t dtype;       /* PSA_BF16 or PSA_F32 (storage, inputs and outputs) */
    int32_t max_chunk;   /* largest prefill chunk C (0: psa_prefill_attn unavailable);
                            C * n_kv_heads * head_dim < 2^32 */
    double rope_base;    /* > 0, e.g. 10000 */
    float scale;         /* softmax scale; 0 selects 1 / sqrt(head_dim) */
    int32_t n_shared_prefixes; /* >= 0: entries of the shared-prefix pool */
    int32_t shared_prefix_max; /* >= 0: longest prefix one pool entry holds */
    int32_t pe_mode;     /* PSA_PE_CONTINUE or PSA_PE_RESET */
    int32_t block_size;  /* 0: contiguous slots per sequence; else paged K/V (see psa_layout):
                            a power of two >= 16 that divides prefix_max and window, with
                            (prefix_max + window) / block_size <= 1024 */
    int32_t n_blocks;    /* paged only: physical blocks in the pool (0 selects
                            max_batch * (prefix_max + window) / block_size); else 0 */
} psa_cache_desc;

/* Position encoding of attended tokens ([PS] 05).
 * CONTINUE: every token keeps its absolute position (the method's choice).
 * RESET: the attended tokens are renumbered as one sequence, prefix first: prefix token j
 *   keeps j, window token j gets P_b + (j - base) with base the oldest window position,
 *   and the query the position of the newest window entry. Stored keys are the same in
 *   both modes (rotated at absolute positions); with rotary encoding only position
 *   differences matter, and renumbering changes only the query-to-prefix distances, so
 *   RESET rotates the query at its renumbered position for prefix keys and at its
 *   absolute position for window keys. */
enum { PSA_PE_CONTINUE = 0, PSA_PE_RESET = 1 };

/* Byte offsets of the regions the library carves out of the caller's device buffer.
 * Every sequence has S = prefix_max + window logical slots: slots [0, P_max) hold prefix
 * positions p < P_b at slot p (promoted entries follow at slots P_b, P_b + 1, ...);
 * slots [P_max, S) are the ring, position p >= P_b at slot P_max + (p - P_b) mod W.
 * K and V, contiguous (block_size 0): [B][H_kv][S][D], slot s of (b, h) at row
 * (b * H_kv + h) * S + s.
 * K and V, paged ([KV-Lean] 6.1: the logical cache read through a table of physical
 * blocks): [H_kv][n_blocks][block_size][D]; the block table [B][S / block_size] int32
 * (at btab_offset) maps logical block s / block_size of sequence b to a physical block,
 * -1 if none, and slot s of (b, h) is row (h * n_blocks + blk) * block_size + s % block_size.
 * (Head-major, so the blocks a sequence takes one after another form one contiguous run per
 * head.)
 * The library owns the table: a block is taken from the pool when a call first writes
 * one of its slots (append, prefill, promotion) and returned when the sequence is reset
 * or attached; a window that has filled its ring reuses its blocks. A sequence holds
 * ceil(pinned entries / block_size) prefix blocks (none when attached to a shared
 * prefix) plus the ring blocks its window positions have touched, at most
 * window / block_size.
 * tags: [B][S] int32, the absolute position held by each slot, -1 if it holds no cached
 * entry (never written, or its entry left the cache without being overwritten).
 * pool K and V: [n_shared_prefixes][H_kv][shared_prefix_max][D], position p of entry e
 * at row p (absent when n_shared_prefixes is 0). */
typedef struct {
    size_t k_offset;
    size_t v_offset;
    size_t pool_k_offset;
    size_t pool_v_offset;
    size_t tags_offset;
    size_t btab_offset;   /* paged: block table [B][S / block_size] int32 */
    size_t state_offset;  /* library-private per-sequence state */
    size_t work_offset;   /* library-private workspace */
    size_t total_bytes;   /* == psa_cache_bytes() */
    int32_t slots;        /* S */
    int32_t elem_bytes;   /* 2 (bf16) or 4 (f32) */
    int32_t block_size;   /* 0 (contiguous) or the block size */
    int32_t n_blocks;     /* paged: physical blocks in the pool */
    int32_t max_splits;   /* decode splits the workspace holds per (sequence, query head):
                             enough for max(prefix_max, shared_prefix_max) + window visible
                             entries at the shortest split (128 entries) */
} psa_layout;

/* Device bytes the caller must provide for a cache described by *desc (0 if *desc is
 * invalid; psa_last_error() then says why). Host only; enqueues nothing. Memory management
 * of the library: no passage of the pages defines it. */
size_t psa_cache_bytes(const psa_cache_desc *desc);

/* Fill *out with the layout of a cache described by *desc. Host only.
 * Returns PSA_ERR_ARG for a null pointer or an invalid description. (Library
 * infrastructure: defined by no passage of the pages.) */
int psa_cache_layout(const psa_cache_desc *desc, psa_layout *out);

/* Create a cache over caller-owned device memory dev_mem (>= psa_cache_bytes(desc)
 * bytes, 256-byte aligned) on the current HIP device (library infrastructure: defined by
 * no passage of the pages; the empty cache is [KV-Lean] 2.3's empty window list). Initialises every slot tag to
 * -1 and every sequence to "not started", then waits for `stream`.
 * On success *out receives a new handle; on error *out is left unchanged.
 * The memory stays owned by the caller and must outlive the handle. */
int psa_cache_create(const psa_cache_desc *desc, void *dev_mem, size_t bytes, psa_stream stream,
                     psa_cache **out);

/* Release the host handle (the device memory is the caller's). NULL is accepted.
 * (Library infrastructure: defined by no passage of the pages.) */
int psa_cache_destroy(psa_cache *cache);

/* Start (or restart) sequence `seq` with a pinned prefix of prefix_len tokens
 * (0 <= prefix_len <= prefix_max; 0 gives the plain sliding window). Its history
 * becomes empty and all its slot tags -1. The prefix is the first prefix_len tokens
 * appended afterwards ([PS] 03: the prefix KV is encoded once and never evicted). */
int psa_seq_reset(psa_cache *cache, int32_t seq, int32_t prefix_len, psa_stream stream);

/* Shared pinned prefixes ([KV-Lean] 6.1-6.2: a logical cache read through a table of
 * physical blocks; a prompt's prefix reused across requests is safe when its positions
 * are the same, which Continue PE guarantees: prefix tokens sit at positions 0 .. P-1
 * in every sequence). One pool entry holds the K/V of one prompt prefix; any number of
 * sequences (e.g. many sampled runs of one problem) read it instead of holding a copy.
 *
 * psa_prefix_load: write pool entry `prefix_id` with `len` tokens at positions 0 .. len-1
 * (0 <= len <= shared_prefix_max; keys rotated at their positions and rounded as in
 * psa_append). k, v: [len][H_kv][D]. Errors: PSA_ERR_ARG for an out-of-range id or
 * length; PSA_ERR_STATE while sequences are attached to the entry. */
int psa_prefix_load(psa_cache *cache, int32_t prefix_id, int32_t len, const void *k, const void *v,
                    psa_stream stream);

/* Start (or restart) sequence `seq` on pool entry `prefix_id`: its pinned prefix is that
 * entry (P_b = the entry's length) and its history already holds positions 0 .. P_b - 1;
 * the next append is position P_b. The sequence reads the prefix from the pool and never
 * writes it. psa_seq_reset detaches. Errors: PSA_ERR_STATE if the entry was never
 * loaded; PSA_ERR_ARG for an out-of-range id. */
int psa_seq_attach(psa_cache *cache, int32_t seq, int32_t prefix_id, psa_stream stream);

/* Window length and promotion of one sequence (host checks, then a small kernel on
 * `stream`). The sequence's cache follows a list model: a pinned list and a window list
 * (oldest first). An append puts the token into the pinned list while p < P_b, else at
 * the window's tail, dropping the window's oldest entries while it holds more than w_b.
 *
 * psa_seq_set_window: w_b = window (1 <= window <= desc.window) from now on; a window
 * holding more entries drops its oldest ones at once. Dropped entries never come back,
 * so after a growth the window refills with new tokens only. No K/V bytes move.
 * Errors: PSA_ERR_ARG for a window out of range; PSA_ERR_STATE if `seq` was never reset
 * (psa_seq_reset and psa_seq_attach restore w_b = desc.window). */
int psa_seq_set_window(psa_cache *cache, int32_t seq, int32_t window, psa_stream stream);

/* psa_seq_promote: move the `count` oldest window entries to the end of the pinned list,
 * where they stay for good (their keys keep the rotation of their absolute positions;
 * they are copied to the next free prefix slots). Errors: PSA_ERR_ARG if count is
 * negative, exceeds the window's entries, or the pinned list would exceed prefix_max;
 * PSA_ERR_STATE if `seq` was never reset, reads a shared prefix (psa_seq_attach), the
 * cache uses PSA_PE_RESET (renumbered positions are defined for [prefix, window] only),
 * or (paged) no free block is left for the prefix slots. */
int psa_seq_promote(psa_cache *cache, int32_t seq, int32_t count, psa_stream stream);

/* Paged caches: copy sequence `seq`'s block table (S / block_size entries, physical block
 * or -1) into table_host (may be NULL) and its length into *entries; *free_blocks (may be
 * NULL) receives the pool's unused blocks. Host only. Errors: PSA_ERR_ARG for a
 * contiguous cache or a NULL `entries`; PSA_ERR_STATE if `seq` is out of range. */
int psa_seq_blocks(const psa_cache *cache, int32_t seq, int32_t *table_host, int32_t *entries,
                   int32_t *free_blocks);

/* From the host mirror: the sequence's window length, its pinned entries (min(n, P_b)
 * plus promoted ones) and its window entries; any output may be NULL. Host only.
 * Errors: PSA_ERR_STATE if `seq` is out of range or was never reset. */
int psa_seq_window(const psa_cache *cache, int32_t seq, int32_t *window, int32_t *pinned,
                   int32_t *window_entries);

/* Append new tokens to every sequence ([PS] 03 generation loop; [KV-Lean] 2.2, 3.3:
 * append at the tail, evict the oldest once the window holds more than W).
 * k, v: [B][n_stride][H_kv][D]. Sequence b appends n_b tokens, rows 0 .. n_b - 1 of
 * its block, at positions len_b, len_b + 1, ...: n_b = n_new_host[b] if n_new_host is
 * not NULL (a host array of B entries), else n_uniform. 0 <= n_b <= n_stride.
 * A token at p < P_b goes to prefix slot p; otherwise to ring slot (p - P_b) mod W,
 * overwriting (evicting) position p - W; with w_b < W the window's oldest entries leave
 * by the length rule and their slots get tag -1. The key is stored rotated at p. A token
 * that a later token of the same call evicts is not written.
 * Errors: PSA_ERR_STATE if a sequence with n_b > 0 was never reset, or (paged) if the
 * pool has fewer free blocks than the call needs; PSA_ERR_OVERFLOW if
 * len_b + n_b > INT32_MAX. */
int psa_append(psa_cache *cache, const int32_t *n_new_host, int32_t n_uniform, const void *k,
               const void *v, int32_t n_stride, psa_stream stream);

/* Decode attention for every sequence ([PS] 03 visible set; [PS] 06: only prefix and
 * window blocks are read). The query of sequence b is the token at p = len_b - 1,
 * i.e. the one most recently appended; it sees the prefix and the window, itself
 * included. q, out: [B][H_q][D]; lse: [B][H_q] float32 natural-log log-sum-exp of the
 * scaled logits, or NULL. Errors: PSA_ERR_STATE if any sequence is empty, or if the split
 * plan needs more than psa_layout.max_splits splits (refused before any launch; the layout's
 * sizing rules it out). */
int psa_decode_attn(psa_cache *cache, const void *q, void *out, float *lse, psa_stream stream);

/* One step of the generation loop ([PS] 03: append the new token, then attend to the
 * prefix and the window) in one decode launch: the same result, cache contents and state
 * as psa_append(cache, NULL, 1, k, v, 1, stream) followed by psa_decode_attn(cache, q,
 * out, lse, stream). k, v: [B][H_kv][D] (one token per sequence, as psa_append with
 * n_stride = 1); q, out, lse as psa_decode_attn. Errors: PSA_ERR_ARG for a NULL k, v,
 * q or out; PSA_ERR_STATE if a sequence was never reset or (paged) the pool has no free
 * block for a token that needs one; PSA_ERR_OVERFLOW as psa_append. These leave the
 * cache unchanged. PSA_ERR_HIP: a failed decode launch leaves the cache unchanged (paged:
 * the blocks the token needed stay mapped); a failed merge launch leaves it advanced by the
 * step, with `out` and `lse` not written. */
int psa_decode_step(psa_cache *cache, const void *k, const void *v, const void *q, void *out,
                    float *lse, psa_stream stream);

/* Chunked prefill: every sequence takes `chunk` new tokens at positions
 * len_b .. len_b + chunk - 1; query row c (at p = len_b + c) attends to A(p + 1) of
 * [PS] 03: the prefix, the window of p and the chunk's own tokens up to p. The pages never
 * discuss chunks; the reading taken is that a chunk equals `chunk` consecutive decode
 * steps. Key tiles no row of a query block sees are never loaded, tiles every row sees
 * entirely run unmasked, and only partially covered tiles are masked per element ([PS] 06,
 * the block-level then token-level filter). Then the chunk is appended as by psa_append. 
 * q, out: [B][chunk][H_q][D]; k, v: [B][chunk][H_kv][D]; lse: [B][chunk][H_q] float32
 * or NULL. 1 <= chunk <= max_chunk. Errors: PSA_ERR_STATE if a sequence was never
 * reset or (paged) the pool has fewer free blocks than the chunk needs;
 * PSA_ERR_OVERFLOW as psa_append. */
int psa_prefill_attn(psa_cache *cache, int32_t chunk, const void *q, const void *k,
                     const void *v, void *out, float *lse, psa_stream stream);

/* Copy sequence `seq`'s logical cache to host memory ([KV-Lean] 3.4 ring read back
 * as a list; 6.3 export and compare against the list model): the pinned entries (from
 * the pool for an attached sequence), then the window oldest first; count = pinned +
 * window entries (min(len, P_b + W) unless the window length changed or entries were
 * promoted). k_host, v_host: [S][H_kv][D] (capacity S = max(prefix_max,
 * shared_prefix_max) + window entries), pos_host: [S] int32 absolute positions; any of
 * the three may be NULL. Waits for `stream`. */
int psa_export(psa_cache *cache, int32_t seq, void *k_host, void *v_host, int32_t *pos_host,
               int32_t *count, psa_stream stream);

/* Training attention over the same visible set ([PS] 08: chunked or truncated
 * back-propagation through long traces needs the gradient of the generator's attention).
 * Works on caller tensors, not on a cache. A segment of sequence b has len_b rows: rows
 * [0, P_b) are its pinned prefix, later rows consecutive positions (for truncated
 * back-propagation, the prompt followed by the last tokens of the trace). Key row j is
 * visible to query row i iff j <= i and (j < P_b or j >= i - W + 1), the set A(t) of
 * [PS] 03 in row indices. Queries and keys are passed already rotated at their positions
 * (the rotation and its transpose in the backward pass are the caller's), so the calls
 * compute out = softmax(scale * q k^T + mask) v and its gradients.
 * Tensors are bf16 and dense: q, out, dout, dq: [B][T][H_q][D]; k, v, dk, dv:
 * [B][T][H_kv][D]; lse: [B][T][H_q] float32, natural log. Rows >= len_b are neither read
 * nor written. prefix_host, len_host: host arrays of B entries (len_host NULL: all T);
 * 0 <= P_b, 1 <= len_b <= T. workspace: caller-owned device memory of
 * psa_train_workspace_bytes() bytes, 256-byte aligned. Errors: PSA_ERR_ARG for a null
 * pointer, unsupported shape, a length or prefix out of range, or a short workspace. */
typedef struct {
    int32_t batch;       /* B >= 1 */
    int32_t seq_len;     /* T >= 1: rows per sequence (tensor stride) */
    int32_t n_q_heads;   /* H_q, a multiple of n_kv_heads with H_q / H_kv in {1, 2, 4, 8} */
    int32_t n_kv_heads;  /* H_kv >= 1 */
    int32_t head_dim;    /* D: 64 or 128 */
    int32_t window;      /* W >= 1 */
    float scale;         /* softmax scale; 0 selects 1 / sqrt(head_dim) */
    int32_t reserved;    /* must be 0 */
} psa_train_desc;

/* Workspace bytes for psa_train_fwd / psa_train_bwd (0 for an invalid description). */
size_t psa_train_workspace_bytes(const psa_train_desc *desc);

/* Forward: writes out and lse. */
int psa_train_fwd(const psa_train_desc *desc, const int32_t *prefix_host,
                  const int32_t *len_host, const void *q, const void *k, const void *v,
                  void *out, float *lse, void *workspace, size_t workspace_bytes,
                  psa_stream stream);

/* Backward: given the forward's out and lse and dout = dL/dout, writes dq = dL/dq,
 * dk = dL/dk and dv = dL/dv (a KV head's gradient sums over the query heads that read
 * it). */
int psa_train_bwd(const psa_train_desc *desc, const int32_t *prefix_host,
                  const int32_t *len_host, const void *q, const void *k, const void *v,
                  const void *out, const float *lse, const void *dout, void *dq, void *dk,
                  void *dv, void *workspace, size_t workspace_bytes, psa_stream stream);

/* psa_train_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * kernels and results as psa_train_bwd, without the workspace argument. Its scratch (the
 * sequences' prefix and length table and the float32 row dots sum_d dout * out,
 * [B][T][H_q]) lives in a static device array of PSA_TRAIN_STATIC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends; the call itself
 * allocates and frees nothing. Every call on one GPU shares that GPU's array and leaves
 * its contents behind (nothing in it needs to start at zero: each call writes every entry
 * it reads), so calls that overlap in time on one GPU (other streams, other threads) race.
 * Errors: as psa_train_bwd; PSA_ERR_ARG when psa_train_workspace_bytes(desc) exceeds the
 * array (B * T * H_q above about 4.19 million rows), before anything is enqueued. */
#define PSA_TRAIN_STATIC_SCRATCH_BYTES (16u << 20)
int psa_train_bwd_noalloc(const psa_train_desc *desc, const int32_t *prefix_host,
                          const int32_t *len_host, const void *q, const void *k, const void *v,
                          const void *out, const float *lse, const void *dout, void *dq,
                          void *dk, void *dv, psa_stream stream);

/* History length of `seq` from the host mirror (-1 if seq is out of range or the
 * sequence was never reset). Host only. (Library infrastructure: defined by no passage of
 * the pages.) */
int64_t psa_seq_length(const psa_cache *cache, int32_t seq);

/* Visible entries per decode split (the work unit of one workgroup); 0 restores the
 * automatic choice. (A tuning knob of this library's split-KV decode: defined by no passage
 * of the pages.) Must be 0 or >= 128. Results are the same up to float32 rounding
 * order for any value. Host only. */
int psa_set_split_tokens(psa_cache *cache, int32_t tokens);

/* Kernel timing with HIP events recorded on the launch stream around each kernel.
 * enable != 0 starts recording (and clears earlier totals), 0 stops it. Each figure brackets
 * one launch, so it includes the launch's ramp-up and drain and the sum over a step's
 * kernels can exceed the step's own time. (Measurement infrastructure: defined by no
 * passage of the pages.) */
int psa_profile(psa_cache *cache, int32_t enable);

/* Kernel ids for psa_profile_read. */
enum {
    PSA_K_APPEND = 0,        /* ring append with RoPE */
    PSA_K_DECODE = 1,        /* split-KV decode partials */
    PSA_K_MERGE = 2,         /* cross-split log-sum-exp merge */
    PSA_K_PREFILL_STAGE = 3, /* rotate a prefill chunk's keys */
    PSA_K_PREFILL = 4,       /* chunked-prefill attention */
    PSA_K_COUNT = 5
};

/* Waits for the recorded events, then gives the summed duration in milliseconds and
 * the number of launches of kernel `kernel` since profiling was enabled. */
int psa_profile_read(psa_cache *cache, int32_t kernel, double *total_ms, int64_t *launches);

/* Static text of a status code. (Library infrastructure: defined by no passage of the
 * pages.) */
const char *psa_status_string(int status);

/* Text of the last error on this thread (empty if none). (Library infrastructure: defined
 * by no passage of the pages.) */
const char *psa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PSA_H */
