// C-ABI entry points of libpsa: argument and state validation, layout of the caller's
// device buffer, the host mirror of sequence lengths and prefix lengths, decode split
// planning, export of the logical cache view, and optional per-kernel event timing.
// All device work is done by the kernels in append.hip, decode.hip and prefill.hip.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "psa_internal.h"

#define PSA_API extern "C" __attribute__((visibility("default")))



namespace {

thread_local std::string g_err;

int fail(int status, const std::string& msg) {
    g_err = msg;
    return status;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct EventPair {
    int kernel;
    hipEvent_t start, stop;
};

}  // namespace

struct psa_cache {
    psa_cache_desc desc;
    psa::Layout L;
    psa::DevCache dev;
    int device;
    int cur;                       // which device length buffer is current
    std::vector<int64_t> len;      // host mirror of history lengths
    std::vector<int32_t> pre;      // host mirror of P_b; -1 = never reset
    std::vector<int32_t> pid;      // shared-prefix entry per sequence, -1 = own prefix
    std::vector<int32_t> npin;     // pinned entries once the prefix is complete
    std::vector<int32_t> wfloor;   // no window entry is older than this position
    std::vector<int32_t> wlen;     // window length per sequence
    std::vector<int32_t> pool_len; // tokens held by each pool entry, -1 = never loaded
    std::vector<int32_t> attached; // sequences attached to each pool entry
    std::vector<int32_t> btab;     // paged: host copy of the block table [B][NBT]
    std::vector<int32_t> free_blk; // paged: unused physical blocks (a stack)
    std::vector<int32_t> order;    // decode workgroup order on the device (grid y -> sequence)
    int32_t split_tokens;          // 0 = automatic
    int resident_wgs;              // decode workgroups resident at once (0 = not yet queried)
    bool profiling;
    std::vector<EventPair> pending;
    double total_ms[PSA_K_COUNT];
    int64_t launches[PSA_K_COUNT];
};

namespace psa {

bool compute_layout(const psa_cache_desc& d, Layout* L, const char** why) {
    auto bad = [&](const char* w) {
        *why = w;
        return false;
    };
    // The decode and merge launches put sequences on grid y: at most 65535. The decode
    // launch's grid x holds (split, KV head) pairs (checked below).
    if (d.max_batch < 1 || d.max_batch > kMaxGridYZ) return bad("max_batch must be in [1, 65535]");
    if (d.n_kv_heads < 1 || d.n_kv_heads > kMaxGridYZ) return bad("n_kv_heads must be in [1, 65535]");
    if (d.n_q_heads < 1 || d.n_q_heads % d.n_kv_heads != 0)
        return bad("n_q_heads must be a positive multiple of n_kv_heads");
    const int G = d.n_q_heads / d.n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return bad("n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (d.head_dim != 64 && d.head_dim != 128) return bad("head_dim must be 64 or 128");
    if (d.prefix_max < 0) return bad("prefix_max must be >= 0");
    if (d.window < 1) return bad("window must be >= 1");
    if (d.dtype != PSA_BF16 && d.dtype != PSA_F32) return bad("dtype must be PSA_BF16 or PSA_F32");
    if (d.max_chunk < 0) return bad("max_chunk must be >= 0");
    if (!(d.rope_base > 0.0) || !isfinite(d.rope_base)) return bad("rope_base must be finite and > 0");
    if (!(d.scale >= 0.f) || !isfinite(d.scale)) return bad("scale must be finite and >= 0");
    if (d.n_shared_prefixes < 0 || d.shared_prefix_max < 0)
        return bad("n_shared_prefixes and shared_prefix_max must be >= 0");
    if (d.n_shared_prefixes > 0 && d.shared_prefix_max < 1)
        return bad("shared_prefix_max must be >= 1 when the pool has entries");
    if ((int64_t)d.shared_prefix_max + d.window > (1 << 30)) return bad("shared_prefix_max too large");
    if (d.pe_mode != PSA_PE_CONTINUE && d.pe_mode != PSA_PE_RESET)
        return bad("pe_mode must be PSA_PE_CONTINUE or PSA_PE_RESET");
    const int64_t S = (int64_t)d.prefix_max + d.window;
    if (S > (1 << 30)) return bad("prefix_max + window too large");
    // Chunked prefill addresses a tile's K/V rows as 24-bit row x 24-bit stride products
    // with a 32-bit result (elements): ring rows (< W) times D, and chunk rows (< chunk)
    // times H_kv * D.
    if (d.max_chunk > 0) {
        if (d.window >= (1 << 24)) return bad("window must be < 2^24 when max_chunk > 0");
        if ((int64_t)d.max_chunk * d.n_kv_heads * d.head_dim >= ((int64_t)1 << 32))
            return bad("max_chunk * n_kv_heads * head_dim must be < 2^32");
    }
    int64_t n_blocks = 0;
    if (d.block_size != 0) {
        const int bs = d.block_size;
        if (bs < 16 || (bs & (bs - 1)) != 0) return bad("block_size must be 0 or a power of two >= 16");
        if (d.prefix_max % bs != 0 || d.window % bs != 0)
            return bad("block_size must divide prefix_max and window");
        if (S / bs > kMaxBlockTable) return bad("(prefix_max + window) / block_size must be <= 1024");
        if (d.n_blocks < 0) return bad("n_blocks must be >= 0");
        n_blocks = d.n_blocks > 0 ? d.n_blocks : (int64_t)d.max_batch * (S / bs);
        if (n_blocks > (1 << 30)) return bad("n_blocks too large");
    } else if (d.n_blocks != 0) {
        return bad("n_blocks must be 0 for a contiguous cache");
    }
    const size_t elem = d.dtype == PSA_BF16 ? 2 : 4;
    const size_t B = (size_t)d.max_batch, Hq = (size_t)d.n_q_heads, Hkv = (size_t)d.n_kv_heads;
    const size_t D = (size_t)d.head_dim;
    // A sequence sees at most max(prefix_max, shared_prefix_max) + window entries (an
    // attached sequence's prefix is its pool entry). Splits hold at least kSplitGranule
    // entries; RESET splits the prefix and the window separately: one more split at most.
    const int64_t seen = (int64_t)std::max(d.prefix_max, d.shared_prefix_max) + d.window;
    const int64_t max_splits = (seen + kSplitGranule - 1) / kSplitGranule + 1;
    if ((int64_t)d.n_kv_heads * max_splits >= (1 << 24))
        return bad("n_kv_heads * decode splits must be < 2^24 (splits: one per 128 entries of "
                   "max(prefix_max, shared_prefix_max) + window, plus one)");
    const size_t A = 256;
    size_t off = 0;
    const size_t kv_rows = d.block_size ? (size_t)n_blocks * Hkv * (size_t)d.block_size
                                        : B * Hkv * (size_t)S;
    L->k = off;        off = align_up(off + kv_rows * D * elem, A);
    L->v = off;        off = align_up(off + kv_rows * D * elem, A);
    const size_t pool = (size_t)d.n_shared_prefixes * Hkv * (size_t)d.shared_prefix_max * D * elem;
    L->pool_k = off;   off = align_up(off + pool, A);
    L->pool_v = off;   off = align_up(off + pool, A);
    L->tags = off;     off = align_up(off + B * (size_t)S * 4, A);
    L->btab = off;     off = align_up(off + (d.block_size ? B * (size_t)(S / d.block_size) * 4 : 0), A);
    L->state = off;    off = align_up(off + 9 * B * 4, A);
    L->inv_freq = off; off = align_up(off + D / 2 * 8, A);
    L->part_o = off;   off = align_up(off + B * Hq * (size_t)max_splits * D * 4, A);
    L->part_ml = off;  off = align_up(off + B * Hq * (size_t)max_splits * 2 * 4, A);
    L->stage_k = off;  off = align_up(off + B * (size_t)d.max_chunk * Hkv * D * elem, A);
    L->total = off;
    L->S = (int32_t)S;
    L->elem = (int32_t)elem;
    L->max_splits = (int32_t)max_splits;
    L->n_blocks = (int32_t)n_blocks;
    return true;
}

}  // namespace psa

namespace {

int hip_fail(hipError_t e, const char* what) {
    return fail(PSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Launch bracketed by timing events when profiling is on.
template <typename F>
int timed(psa_cache* c, int kernel, hipStream_t s, const char* what, F&& launch) {
    EventPair ev{kernel, nullptr, nullptr};
    auto drop = [&] {   // events of a launch that will not be read
        if (ev.start) hipEventDestroy(ev.start);
        if (ev.stop) hipEventDestroy(ev.stop);
    };
    if (c->profiling) {
        hipError_t e = hipEventCreate(&ev.start);
        if (e == hipSuccess) e = hipEventCreate(&ev.stop);
        if (e == hipSuccess) e = hipEventRecord(ev.start, s);
        if (e != hipSuccess) {
            drop();
            return hip_fail(e, "profiling event");
        }
    }
    const hipError_t e = launch();
    if (e != hipSuccess) {
        drop();
        return hip_fail(e, what);
    }
    if (c->profiling) {
        const hipError_t e2 = hipEventRecord(ev.stop, s);
        if (e2 != hipSuccess) {
            drop();
            return hip_fail(e2, "profiling event");
        }
        c->pending.push_back(ev);
    }
    return PSA_OK;
}

// What sequence b holds now (the same function the kernels evaluate from device state).
psa::SeqView view_of(const psa_cache* c, int b) {
    return psa::seq_view((int)c->len[b], c->pre[b], c->npin[b], c->wfloor[b], c->wlen[b],
                         c->desc.window);
}

// Visible entries of sequence b: its prefix entries plus its window entries.
int64_t visible_count(const psa_cache* c, int b) {
    const psa::SeqView v = view_of(c, b);
    return (int64_t)v.n_pre + v.n_win;
}

// Automatic split length. Cut a sequence of `ref` visible entries into ns pieces with ns
// chosen so the grid is about two rounds of the workgroups that fit on the device at once
// (measured: longer splits amortise each workgroup's set-up and final reduction, and
// whole rounds avoid a ragged tail). ref is the longest sequence when there are at least
// as many (sequence, KV head) pairs as resident workgroups: then every pair is one piece
// and splitting long sequences would only add uneven pieces. With fewer pairs the batch
// must be split for parallelism, and ref is the mean length, so that the pieces of a
// ragged batch add up to about two rounds instead of leaving short sequences' workgroups
// underfilled; then the length is raised, if needed, to the shortest that keeps the grid
// within two full rounds. Never shorter than kSplitGranule entries.
int auto_split_tokens(psa_cache* c) {
    int64_t longest = 1, sum = 0;
    for (int b = 0; b < c->desc.max_batch; ++b) {
        const int64_t t = visible_count(c, b);
        sum += t;
        if (t > longest) longest = t;
    }
    if (c->resident_wgs == 0) c->resident_wgs = psa::decode_resident_wgs(c->dev);
    const int64_t pairs = (int64_t)c->desc.max_batch * c->desc.n_kv_heads;
    const int64_t mean = (sum + c->desc.max_batch - 1) / c->desc.max_batch;
    const bool few_pairs = pairs < c->resident_wgs && mean > 0;
    const int64_t ref = few_pairs ? mean : longest;
    int64_t ns = (2 * (int64_t)c->resident_wgs) / pairs;
    if (ns < 1) ns = 1;
    int64_t L = (ref + ns - 1) / ns;
    if (L < psa::kSplitGranule) L = psa::kSplitGranule;
    if (few_pairs) {
        // Each sequence's last split is partial, so pieces of the mean length add up to
        // more than two rounds (half a workgroup per sequence on average). Lengthen the
        // splits to the shortest that keeps the grid within two full rounds (the count
        // only falls as L grows, so a bisection finds it). With Reset PE the prefix forms
        // splits of its own, usually far shorter than L: they fill the gaps between the
        // window splits and are not counted (counting them would push L up to where the
        // window splits alone take more than two rounds).
        const int64_t budget = 2 * (int64_t)c->resident_wgs;
        const bool reset = c->desc.pe_mode == PSA_PE_RESET;
        auto wgs = [&](int64_t len) {
            int64_t n = 0;
            for (int b = 0; b < c->desc.max_batch; ++b) {
                const psa::SeqView v = view_of(c, b);
                n += reset ? (v.n_win + len - 1) / len
                           : psa::split_count(v.n_pre, v.n_win, (int)len, c->desc.pe_mode);
            }
            return n * c->desc.n_kv_heads;
        };
        if (wgs(L) > budget) {
            int64_t lo = L, hi = longest > L ? longest : L;   // wgs(hi) is the fewest
            if (wgs(hi) <= budget) {
                while (lo + 1 < hi) {
                    const int64_t mid = (lo + hi) / 2;
                    if (wgs(mid) <= budget) hi = mid; else lo = mid;
                }
                L = hi;
            }
        }
    }
    return (int)L;
}

bool valid_seq(const psa_cache* c, int32_t seq) { return seq >= 0 && seq < c->desc.max_batch; }

// Split length and the largest split count over the batch for a decode of the current host
// state. Every split's partial result has a slot in the workspace ([B][Hq][max_splits]);
// a plan that needs more is refused before anything is enqueued (the layout sizes
// max_splits for the longest visible list at the smallest split length, so this holds
// unless the sizing is wrong).
int plan_decode(psa_cache* c, int* split_len, int* grid_splits) {
    const int L = c->split_tokens > 0 ? c->split_tokens : auto_split_tokens(c);
    int64_t max_ns = 1;
    for (int b = 0; b < c->desc.max_batch; ++b) {
        const psa::SeqView v = view_of(c, b);
        const int64_t ns = psa::split_count(v.n_pre, v.n_win, L, c->desc.pe_mode);
        if (ns > max_ns) max_ns = ns;
    }
    if (max_ns > c->L.max_splits)
        return fail(PSA_ERR_STATE, "decode needs " + std::to_string(max_ns) + " splits, the workspace holds " +
                                       std::to_string(c->L.max_splits));
    *split_len = L;
    *grid_splits = (int)max_ns;
    return PSA_OK;
}

// Decode workgroups go out sequence by sequence in the device order array (grid y); with
// sequences of different lengths, the longest first, so the short ones fill the end of
// the launch instead of a long one running alone. Sequences are ranked by visible entries
// in units of kSplitGranule (ties in index order), so steady decoding, which adds one
// entry at a time, rarely changes the order; the entries that change are written by one
// small launch per kTableUpdates of them.
int update_decode_order(psa_cache* c, hipStream_t s) {
    const int B = c->desc.max_batch;
    std::vector<int64_t> key(B);
    for (int b = 0; b < B; ++b) key[b] = visible_count(c, b) / psa::kSplitGranule;
    std::vector<int32_t> want(B);
    for (int b = 0; b < B; ++b) want[b] = b;
    std::stable_sort(want.begin(), want.end(), [&](int32_t x, int32_t y) { return key[x] > key[y]; });
    psa::TableUpdate u;
    u.n = 0;
    for (int z = 0; z < B; ++z) {
        if (want[z] == c->order[z]) continue;
        u.idx[u.n] = z;
        u.blk[u.n] = want[z];
        if (++u.n == psa::kTableUpdates) {
            const hipError_t e = psa::launch_order_update(c->dev, u, s);
            if (e != hipSuccess) return hip_fail(e, "decode order update");
            u.n = 0;
        }
    }
    if (u.n > 0) {
        const hipError_t e = psa::launch_order_update(c->dev, u, s);
        if (e != hipSuccess) return hip_fail(e, "decode order update");
    }
    c->order = want;
    return PSA_OK;
}

// ---- paged caches: the host's block allocator -------------------------------------------
// Logical block j of sequence b covers slots [j * Bs, (j + 1) * Bs); the device table gets
// an entry when a call is about to write one of those slots for the first time.

// Logical blocks written when sequence b appends positions [n0, n1): prefix slots for
// p < P_b, ring slots (p - P_b) mod W otherwise (every ring block once n1 - n0 >= W; tokens
// dropped again within the call are counted too, which only maps a block early).
void blocks_of_positions(const psa_cache* c, int b, int64_t n0, int64_t n1, std::vector<int>& out) {
    const int Bs = c->dev.Bs, W = c->dev.W, Pmax = c->dev.Pmax;
    const int64_t P = c->pre[b];
    const int64_t pe = n1 < P ? n1 : P;
    for (int64_t p = n0; p < pe; p = (p / Bs + 1) * Bs) out.push_back((int)(p / Bs));
    const int64_t lo = n0 > P ? n0 : P;
    if (n1 <= lo) return;
    const int64_t count = n1 - lo;
    if (count >= W) {
        for (int j = Pmax / Bs; j < c->dev.NBT; ++j) out.push_back(j);
        return;
    }
    const int64_t r0 = (lo - P) % W;
    for (int64_t t = 0; t < count;) {
        const int64_t r = (r0 + t) % W;
        out.push_back((int)((Pmax + r) / Bs));
        t += Bs - r % Bs;
    }
}

// Give every listed logical block of sequence b that has no physical block one from the
// pool and write the new table entries on the stream. Nothing changes when the pool is
// short (PSA_ERR_STATE).
int map_blocks(psa_cache* c, int b, std::vector<int>& want, int64_t* taken, hipStream_t s,
               psa::TableUpdate* u) {
    int32_t* row = c->btab.data() + (size_t)b * c->dev.NBT;
    int64_t need = 0;
    for (int j : want)
        if (row[j] < 0) {
            row[j] = -2;   // counted once
            ++need;
        }
    if (*taken + need > (int64_t)c->free_blk.size()) {
        for (int j : want)
            if (row[j] == -2) row[j] = -1;
        return fail(PSA_ERR_STATE, "block pool exhausted: " + std::to_string(c->free_blk.size() - *taken) +
                                       " free blocks, the call needs more");
    }
    for (int j : want) {
        if (row[j] != -2) continue;
        row[j] = c->free_blk[c->free_blk.size() - 1 - *taken];
        *taken += 1;
        u->idx[u->n] = b * c->dev.NBT + j;
        u->blk[u->n] = row[j];
        if (++u->n == psa::kTableUpdates) {
            const hipError_t e = psa::launch_table_update(c->dev, *u, s);
            u->n = 0;
            if (e != hipSuccess) return hip_fail(e, "block table update");
        }
    }
    return PSA_OK;
}

// Map the blocks every sequence writes when it appends n[b] tokens (all sequences or none).
int map_append(psa_cache* c, const int32_t* n_host, int32_t n_uniform, hipStream_t s) {
    if (c->dev.Bs == 0) return PSA_OK;
    const int B = c->desc.max_batch;
    // first pass: check without changing anything
    int64_t total_new = 0;
    std::vector<int> want;
    for (int b = 0; b < B; ++b) {
        const int32_t nb = n_host ? n_host[b] : n_uniform;
        if (nb <= 0) continue;
        want.clear();
        blocks_of_positions(c, b, c->len[b], c->len[b] + nb, want);
        const int32_t* row = c->btab.data() + (size_t)b * c->dev.NBT;
        std::vector<char> seen(c->dev.NBT, 0);
        for (int j : want)
            if (row[j] < 0 && !seen[j]) {
                seen[j] = 1;
                ++total_new;
            }
    }
    if (total_new > (int64_t)c->free_blk.size())
        return fail(PSA_ERR_STATE, "block pool exhausted: " + std::to_string(c->free_blk.size()) +
                                       " free blocks, the call needs " + std::to_string(total_new));
    psa::TableUpdate u;
    u.n = 0;
    int64_t taken = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t nb = n_host ? n_host[b] : n_uniform;
        if (nb <= 0) continue;
        want.clear();
        blocks_of_positions(c, b, c->len[b], c->len[b] + nb, want);
        const int rc = map_blocks(c, b, want, &taken, s, &u);
        if (rc != PSA_OK) return rc;
    }
    c->free_blk.resize(c->free_blk.size() - taken);
    if (u.n > 0) {
        const hipError_t e = psa::launch_table_update(c->dev, u, s);
        if (e != hipSuccess) return hip_fail(e, "block table update");
    }
    return PSA_OK;
}

// Return sequence b's blocks to the pool (the device entries are cleared by the reset).
void release_blocks(psa_cache* c, int b) {
    if (c->dev.Bs == 0) return;
    int32_t* row = c->btab.data() + (size_t)b * c->dev.NBT;
    for (int j = 0; j < c->dev.NBT; ++j)
        if (row[j] >= 0) {
            c->free_blk.push_back(row[j]);
            row[j] = -1;
        }
}

}  // namespace

PSA_API size_t psa_cache_bytes(const psa_cache_desc* desc) {
    if (desc == nullptr) {
        fail(PSA_ERR_ARG, "desc is NULL");
        return 0;
    }
    psa::Layout L;
    const char* why = nullptr;
    if (!psa::compute_layout(*desc, &L, &why)) {
        fail(PSA_ERR_ARG, why);
        return 0;
    }
    return L.total;
}

PSA_API int psa_cache_layout(const psa_cache_desc* desc, psa_layout* out) {
    if (desc == nullptr || out == nullptr) return fail(PSA_ERR_ARG, "NULL argument");
    psa::Layout L;
    const char* why = nullptr;
    if (!psa::compute_layout(*desc, &L, &why)) return fail(PSA_ERR_ARG, why);
    out->k_offset = L.k;
    out->v_offset = L.v;
    out->pool_k_offset = L.pool_k;
    out->pool_v_offset = L.pool_v;
    out->tags_offset = L.tags;
    out->state_offset = L.state;
    out->work_offset = L.inv_freq;
    out->total_bytes = L.total;
    out->slots = L.S;
    out->elem_bytes = L.elem;
    out->btab_offset = L.btab;
    out->block_size = desc->block_size;
    out->n_blocks = L.n_blocks;
    out->max_splits = L.max_splits;
    return PSA_OK;
}

PSA_API int psa_cache_create(const psa_cache_desc* desc, void* dev_mem, size_t bytes,
                             psa_stream stream, psa_cache** out) {
    if (desc == nullptr || out == nullptr) return fail(PSA_ERR_ARG, "NULL argument");
    psa::Layout L;
    const char* why = nullptr;
    if (!psa::compute_layout(*desc, &L, &why)) return fail(PSA_ERR_ARG, why);
    if (dev_mem == nullptr) return fail(PSA_ERR_ARG, "dev_mem is NULL");
    if (((uintptr_t)dev_mem & 255u) != 0) return fail(PSA_ERR_ARG, "dev_mem must be 256-byte aligned");
    if (bytes < L.total)
        return fail(PSA_ERR_ARG, "buffer too small: need " + std::to_string(L.total) + " bytes");

    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");

    psa_cache* c = new psa_cache();
    c->desc = *desc;
    c->L = L;
    c->device = device;
    c->cur = 0;
    c->len.assign(desc->max_batch, 0);
    c->pre.assign(desc->max_batch, -1);
    c->pid.assign(desc->max_batch, -1);
    c->npin.assign(desc->max_batch, 0);
    c->wfloor.assign(desc->max_batch, 0);
    c->wlen.assign(desc->max_batch, desc->window);
    c->pool_len.assign(desc->n_shared_prefixes, -1);
    c->attached.assign(desc->n_shared_prefixes, 0);
    c->split_tokens = 0;
    c->resident_wgs = 0;
    c->order.resize(desc->max_batch);
    for (int b = 0; b < desc->max_batch; ++b) c->order[b] = b;   // init_kernel's order
    c->profiling = false;
    for (int i = 0; i < PSA_K_COUNT; ++i) {
        c->total_ms[i] = 0.0;
        c->launches[i] = 0;
    }
    char* base = (char*)dev_mem;
    psa::DevCache& d = c->dev;
    d.k = base + L.k;
    d.v = base + L.v;
    d.pool_k = base + L.pool_k;
    d.pool_v = base + L.pool_v;
    d.tags = (int32_t*)(base + L.tags);
    d.btab = (int32_t*)(base + L.btab);
    int32_t* st = (int32_t*)(base + L.state);
    d.len[0] = st;
    d.len[1] = st + desc->max_batch;
    d.pre = st + 2 * desc->max_batch;
    d.nnew = st + 3 * desc->max_batch;
    d.pid = st + 4 * desc->max_batch;
    d.npin = st + 5 * desc->max_batch;
    d.wfloor = st + 6 * desc->max_batch;
    d.wlen = st + 7 * desc->max_batch;
    d.order = st + 8 * desc->max_batch;
    d.inv_freq = (double*)(base + L.inv_freq);
    d.part_o = (float*)(base + L.part_o);
    d.part_ml = (float*)(base + L.part_ml);
    d.stage_k = base + L.stage_k;
    d.B = desc->max_batch;
    d.Hq = desc->n_q_heads;
    d.Hkv = desc->n_kv_heads;
    d.D = desc->head_dim;
    d.Pmax = desc->prefix_max;
    d.W = desc->window;
    d.S = L.S;
    d.dtype = desc->dtype;
    d.max_chunk = desc->max_chunk;
    d.max_splits = L.max_splits;
    d.n_shared = desc->n_shared_prefixes;
    d.shared_max = desc->shared_prefix_max;
    d.pe_mode = desc->pe_mode;
    d.Bs = desc->block_size;
    d.bshift = 0;
    while (d.Bs > 0 && (1 << d.bshift) < d.Bs) ++d.bshift;
    d.NBT = d.Bs > 0 ? L.S / d.Bs : 0;
    d.n_blocks = L.n_blocks;
    if (d.Bs > 0) {
        c->btab.assign((size_t)desc->max_batch * d.NBT, -1);
        c->free_blk.reserve(L.n_blocks);
        for (int32_t i = L.n_blocks - 1; i >= 0; --i) c->free_blk.push_back(i);
    }
    d.scale = desc->scale > 0.f ? desc->scale : (float)(1.0 / sqrt((double)desc->head_dim));

    // theta_i = base^(-2i/D) in float64 on the host.
    std::vector<double> theta(desc->head_dim / 2);
    for (int i = 0; i < desc->head_dim / 2; ++i)
        theta[i] = pow(desc->rope_base, (-2.0 * (double)i) / (double)desc->head_dim);
    hipStream_t s = (hipStream_t)stream;
    e = hipMemcpyAsync(d.inv_freq, theta.data(), theta.size() * sizeof(double),
                       hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = psa::launch_init(d, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "cache initialisation");
    }
    *out = c;
    return PSA_OK;
}

PSA_API int psa_cache_destroy(psa_cache* c) {
    if (c == nullptr) return PSA_OK;
    for (auto& ev : c->pending) {
        hipEventDestroy(ev.start);
        hipEventDestroy(ev.stop);
    }
    delete c;
    return PSA_OK;
}

namespace {

void detach(psa_cache* c, int32_t seq) {
    if (c->pid[seq] >= 0) c->attached[c->pid[seq]] -= 1;
    c->pid[seq] = -1;
}

// Host mirror of a (re)started sequence with pinned prefix length P (the device side is
// written by seq_reset_kernel).
void start(psa_cache* c, int32_t seq, int32_t P, int64_t len) {
    c->len[seq] = len;
    c->pre[seq] = P;
    c->npin[seq] = P;
    c->wfloor[seq] = P;
    c->wlen[seq] = c->desc.window;
}

}  // namespace

PSA_API int psa_seq_reset(psa_cache* c, int32_t seq, int32_t prefix_len, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    if (prefix_len < 0 || prefix_len > c->desc.prefix_max)
        return fail(PSA_ERR_ARG, "prefix_len must be in [0, prefix_max]");
    const hipError_t e =
        psa::launch_seq_reset(c->dev, seq, prefix_len, 0, -1, c->cur, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sequence reset");
    detach(c, seq);
    release_blocks(c, seq);
    start(c, seq, prefix_len, 0);
    return PSA_OK;
}

PSA_API int psa_prefix_load(psa_cache* c, int32_t prefix_id, int32_t len, const void* k,
                            const void* v, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (prefix_id < 0 || prefix_id >= c->desc.n_shared_prefixes)
        return fail(PSA_ERR_ARG, "prefix_id out of range");
    if (len < 0 || len > c->desc.shared_prefix_max)
        return fail(PSA_ERR_ARG, "len must be in [0, shared_prefix_max]");
    if (len > 0 && (k == nullptr || v == nullptr)) return fail(PSA_ERR_ARG, "k or v is NULL");
    if (c->attached[prefix_id] > 0)
        return fail(PSA_ERR_STATE, "pool entry has attached sequences");
    const hipError_t e = psa::launch_pool_load(c->dev, prefix_id, len, k, v, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prefix load");
    c->pool_len[prefix_id] = len;
    return PSA_OK;
}

PSA_API int psa_seq_attach(psa_cache* c, int32_t seq, int32_t prefix_id, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    if (prefix_id < 0 || prefix_id >= c->desc.n_shared_prefixes)
        return fail(PSA_ERR_ARG, "prefix_id out of range");
    const int32_t P = c->pool_len[prefix_id];
    if (P < 0) return fail(PSA_ERR_STATE, "pool entry was never loaded");
    const hipError_t e =
        psa::launch_seq_reset(c->dev, seq, P, P, prefix_id, c->cur, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sequence attach");
    detach(c, seq);
    release_blocks(c, seq);
    c->pid[seq] = prefix_id;
    c->attached[prefix_id] += 1;
    start(c, seq, P, P);
    return PSA_OK;
}

PSA_API int psa_seq_set_window(psa_cache* c, int32_t seq, int32_t window, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    if (c->pre[seq] < 0) return fail(PSA_ERR_STATE, "sequence was never reset");
    if (window < 1 || window > c->desc.window)
        return fail(PSA_ERR_ARG, "window must be in [1, desc.window]");
    const psa::SeqView v = view_of(c, seq);
    const int64_t n = c->len[seq];
    // entries beyond the new length leave now: the window becomes [wb', n)
    const int64_t wb1 = n - window > v.wb ? n - window : v.wb;
    const int lo = v.wb, hi = (int)(wb1 < n ? wb1 : n);
    const hipError_t e = psa::launch_seq_window(c->dev, seq, window, (int)wb1, lo, hi > lo ? hi : lo,
                                                (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "window change");
    c->wfloor[seq] = (int32_t)wb1;
    c->wlen[seq] = window;
    return PSA_OK;
}

PSA_API int psa_seq_promote(psa_cache* c, int32_t seq, int32_t count, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    if (c->pre[seq] < 0) return fail(PSA_ERR_STATE, "sequence was never reset");
    if (c->pid[seq] >= 0) return fail(PSA_ERR_STATE, "sequence reads a shared prefix");
    if (c->desc.pe_mode != PSA_PE_CONTINUE)
        return fail(PSA_ERR_STATE, "promotion needs PSA_PE_CONTINUE");
    const psa::SeqView v = view_of(c, seq);
    if (count < 0 || count > v.n_win) return fail(PSA_ERR_ARG, "count must be in [0, window entries]");
    if ((int64_t)c->npin[seq] + count > c->desc.prefix_max)
        return fail(PSA_ERR_ARG, "pinned entries would exceed prefix_max");
    if (count == 0) return PSA_OK;
    if (c->dev.Bs > 0) {   // the prefix slots npin .. npin + count - 1 need blocks
        std::vector<int> want;
        for (int64_t sl = c->npin[seq]; sl < (int64_t)c->npin[seq] + count; sl = (sl / c->dev.Bs + 1) * c->dev.Bs)
            want.push_back((int)(sl / c->dev.Bs));
        psa::TableUpdate u;
        u.n = 0;
        int64_t taken = 0;
        const int rc = map_blocks(c, seq, want, &taken, (hipStream_t)stream, &u);
        if (rc != PSA_OK) return rc;
        c->free_blk.resize(c->free_blk.size() - taken);
        const hipError_t eu = psa::launch_table_update(c->dev, u, (hipStream_t)stream);
        if (eu != hipSuccess) return hip_fail(eu, "block table update");
    }
    const hipError_t e =
        psa::launch_promote(c->dev, seq, v.wb, count, c->npin[seq], (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "promotion");
    c->npin[seq] += count;
    c->wfloor[seq] = v.wb + count;
    return PSA_OK;
}

PSA_API int psa_seq_window(const psa_cache* c, int32_t seq, int32_t* window, int32_t* pinned,
                           int32_t* window_entries) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    if (c->pre[seq] < 0) return fail(PSA_ERR_STATE, "sequence was never reset");
    const psa::SeqView v = view_of(c, seq);
    if (window) *window = c->wlen[seq];
    if (pinned) *pinned = v.n_pre;
    if (window_entries) *window_entries = v.n_win;
    return PSA_OK;
}

PSA_API int psa_append(psa_cache* c, const int32_t* n_new_host, int32_t n_uniform, const void* k,
                       const void* v, int32_t n_stride, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (n_stride < 0) return fail(PSA_ERR_ARG, "n_stride must be >= 0");
    const int B = c->desc.max_batch;
    bool any = false;
    for (int b = 0; b < B; ++b) {
        const int32_t nb = n_new_host ? n_new_host[b] : n_uniform;
        if (nb < 0 || nb > n_stride) return fail(PSA_ERR_ARG, "token count outside [0, n_stride]");
        if (nb == 0) continue;
        any = true;
        if (c->pre[b] < 0) return fail(PSA_ERR_STATE, "append to a sequence that was never reset");
        if (c->len[b] + nb > INT32_MAX) return fail(PSA_ERR_OVERFLOW, "sequence length overflow");
    }
    if (!any) return PSA_OK;
    if (k == nullptr || v == nullptr) return fail(PSA_ERR_ARG, "k or v is NULL");
    hipStream_t s = (hipStream_t)stream;
    const int mrc = map_append(c, n_new_host, n_uniform, s);
    if (mrc != PSA_OK) return mrc;
    if (n_new_host != nullptr) {
        const hipError_t e = hipMemcpyAsync(c->dev.nnew, n_new_host, (size_t)B * sizeof(int32_t),
                                            hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "token-count upload");
    }
    const int cur = c->cur;
    const int rc = timed(c, PSA_K_APPEND, s, "append", [&] {
        return psa::launch_append(c->dev, k, v, n_stride, n_uniform, n_new_host != nullptr, 0, cur, s);
    });
    if (rc != PSA_OK) return rc;
    c->cur ^= 1;
    for (int b = 0; b < B; ++b) c->len[b] += n_new_host ? n_new_host[b] : n_uniform;
    return PSA_OK;
}

PSA_API int psa_decode_attn(psa_cache* c, const void* q, void* out, float* lse, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (q == nullptr || out == nullptr) return fail(PSA_ERR_ARG, "q or out is NULL");
    const int B = c->desc.max_batch;
    for (int b = 0; b < B; ++b) {
        if (c->pre[b] < 0) return fail(PSA_ERR_STATE, "decode on a sequence that was never reset");
        if (c->len[b] < 1) return fail(PSA_ERR_STATE, "decode on an empty sequence");
    }
    int L = 0, max_ns = 0;
    const int prc = plan_decode(c, &L, &max_ns);
    if (prc != PSA_OK) return prc;
    hipStream_t s = (hipStream_t)stream;
    const int orc = update_decode_order(c, s);
    if (orc != PSA_OK) return orc;
    const int cur = c->cur;
    int rc = timed(c, PSA_K_DECODE, s, "decode partial", [&] {
        return psa::launch_decode_partial(c->dev, q, L, max_ns, cur, nullptr, nullptr, s);
    });
    if (rc != PSA_OK) return rc;
    return timed(c, PSA_K_MERGE, s, "split merge",
                 [&] { return psa::launch_merge(c->dev, out, lse, L, cur, s); });
}

PSA_API int psa_decode_step(psa_cache* c, const void* k, const void* v, const void* q, void* out,
                            float* lse, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (k == nullptr || v == nullptr || q == nullptr || out == nullptr)
        return fail(PSA_ERR_ARG, "k, v, q or out is NULL");
    const int B = c->desc.max_batch;
    for (int b = 0; b < B; ++b) {
        if (c->pre[b] < 0) return fail(PSA_ERR_STATE, "decode step on a sequence that was never reset");
        if (c->len[b] + 1 > INT32_MAX) return fail(PSA_ERR_OVERFLOW, "sequence length overflow");
    }
    hipStream_t s = (hipStream_t)stream;
    // Split planning and the decode order see the state after the append, as
    // psa_decode_attn would; the host lengths keep it only if every launch succeeds.
    auto undo = [&] {
        for (int b = 0; b < B; ++b) c->len[b] -= 1;
    };
    for (int b = 0; b < B; ++b) c->len[b] += 1;
    int L = 0, max_ns = 0;
    const int prc = plan_decode(c, &L, &max_ns);
    if (prc != PSA_OK) {
        undo();
        return prc;
    }
    for (int b = 0; b < B; ++b) c->len[b] -= 1;
    const int mrc = map_append(c, nullptr, 1, s);
    if (mrc != PSA_OK) return mrc;
    for (int b = 0; b < B; ++b) c->len[b] += 1;
    int rc = update_decode_order(c, s);
    const int cur = c->cur;
    if (rc == PSA_OK)
        rc = timed(c, PSA_K_DECODE, s, "decode step", [&] {
            return psa::launch_decode_partial(c->dev, q, L, max_ns, cur, k, v, s);
        });
    if (rc != PSA_OK) {
        undo();
        return rc;
    }
    // The decode launch appended the token on the device: the step has happened.
    c->cur ^= 1;
    return timed(c, PSA_K_MERGE, s, "split merge",
                 [&] { return psa::launch_merge(c->dev, out, lse, L, cur ^ 1, s); });
}

PSA_API int psa_prefill_attn(psa_cache* c, int32_t chunk, const void* q, const void* k,
                             const void* v, void* out, float* lse, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (c->desc.max_chunk < 1) return fail(PSA_ERR_ARG, "cache was created with max_chunk = 0");
    if (chunk < 1 || chunk > c->desc.max_chunk) return fail(PSA_ERR_ARG, "chunk must be in [1, max_chunk]");
    if (c->desc.dtype != PSA_BF16) return fail(PSA_ERR_ARG, "chunked prefill needs bf16 storage");
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return fail(PSA_ERR_ARG, "q, k, v or out is NULL");
    const int B = c->desc.max_batch;
    for (int b = 0; b < B; ++b) {
        if (c->pre[b] < 0) return fail(PSA_ERR_STATE, "prefill on a sequence that was never reset");
        if (c->len[b] + chunk > INT32_MAX) return fail(PSA_ERR_OVERFLOW, "sequence length overflow");
    }
    hipStream_t s = (hipStream_t)stream;
    const int mrc = map_append(c, nullptr, chunk, s);
    if (mrc != PSA_OK) return mrc;
    const int cur = c->cur;
    int rc = timed(c, PSA_K_PREFILL_STAGE, s, "prefill stage",
                   [&] { return psa::launch_prefill_stage(c->dev, k, chunk, cur, s); });
    if (rc != PSA_OK) return rc;
    rc = timed(c, PSA_K_PREFILL, s, "prefill attention",
               [&] { return psa::launch_prefill(c->dev, q, v, out, lse, chunk, cur, s); });
    if (rc != PSA_OK) return rc;
    rc = timed(c, PSA_K_APPEND, s, "prefill commit", [&] {
        return psa::launch_append(c->dev, c->dev.stage_k, v, chunk, chunk, 0, 1, cur, s);
    });
    if (rc != PSA_OK) return rc;
    c->cur ^= 1;
    for (int b = 0; b < B; ++b) c->len[b] += chunk;
    return PSA_OK;
}

PSA_API int psa_export(psa_cache* c, int32_t seq, void* k_host, void* v_host, int32_t* pos_host,
                       int32_t* count, psa_stream stream) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (count == nullptr) return fail(PSA_ERR_ARG, "count is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    if (c->pre[seq] < 0) return fail(PSA_ERR_STATE, "export of a sequence that was never reset");
    const psa::DevCache& d = c->dev;
    const psa::SeqView sv = view_of(c, seq);
    const int64_t W = d.W;
    const int64_t n_pre = sv.n_pre;
    const int64_t cnt = visible_count(c, seq);
    const int64_t head = (sv.wb - c->pre[seq]) % W;  // ring slot holding the oldest entry
    const size_t elem = (size_t)c->L.elem, D = (size_t)d.D, S = (size_t)d.S, Hkv = (size_t)d.Hkv;
    const size_t row = D * elem;
    const size_t seq_bytes = Hkv * S * row;
    hipStream_t s = (hipStream_t)stream;
    std::vector<char> kbuf, vbuf;
    std::vector<int32_t> tags(S);
    hipError_t e = hipSuccess;
    // Contiguous: the sequence's [H_kv][S][D] region. Paged: the rows of each mapped block,
    // head by head, into the same [H_kv][S][D] arrangement.
    const bool paged = d.Bs > 0;
    const size_t blk_rows_bytes = paged ? (size_t)d.Bs * row : 0;
    const int32_t* brow = paged ? c->btab.data() + (size_t)seq * d.NBT : nullptr;
    auto fetch = [&](std::vector<char>& buf, const void* dev) {
        buf.resize(seq_bytes);
        if (!paged)
            return hipMemcpyAsync(buf.data(), (const char*)dev + (size_t)seq * seq_bytes, seq_bytes,
                                  hipMemcpyDeviceToHost, s);
        hipError_t r = hipSuccess;
        for (int j = 0; j < d.NBT && r == hipSuccess; ++j)
            for (size_t h = 0; h < Hkv && brow[j] >= 0 && r == hipSuccess; ++h)
                r = hipMemcpyAsync(buf.data() + (h * S + (size_t)j * d.Bs) * row,
                                   (const char*)dev +
                                       psa::block_rowidx(brow[j], (int)h, 0, d.Bs, d.n_blocks) * row,
                                   blk_rows_bytes, hipMemcpyDeviceToHost, s);
        return r;
    };
    if (k_host) e = fetch(kbuf, d.k);
    if (e == hipSuccess && v_host) e = fetch(vbuf, d.v);
    if (e == hipSuccess)
        e = hipMemcpyAsync(tags.data(), d.tags + (size_t)seq * S, S * sizeof(int32_t),
                           hipMemcpyDeviceToHost, s);
    // An attached sequence's prefix rows live in its pool entry (positions 0 .. P_b - 1).
    const int32_t pid = c->pid[seq];
    const size_t SP = (size_t)d.shared_max;
    std::vector<char> pk, pv;
    if (pid >= 0 && n_pre > 0) {
        const size_t pool_bytes = Hkv * SP * row, at = (size_t)pid * pool_bytes;
        if (e == hipSuccess && k_host) {
            pk.resize(pool_bytes);
            e = hipMemcpyAsync(pk.data(), (const char*)d.pool_k + at, pool_bytes,
                               hipMemcpyDeviceToHost, s);
        }
        if (e == hipSuccess && v_host) {
            pv.resize(pool_bytes);
            e = hipMemcpyAsync(pv.data(), (const char*)d.pool_v + at, pool_bytes,
                               hipMemcpyDeviceToHost, s);
        }
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "export copy");
    // Logical order: prefix slots, then the ring from the oldest entry ([KV-Lean] 3.4).
    for (int64_t i = 0; i < cnt; ++i) {
        const bool pool_row = pid >= 0 && i < n_pre;
        const size_t slot = i < n_pre ? (size_t)i : (size_t)(d.Pmax + (head + (i - n_pre)) % W);
        if (pos_host) pos_host[i] = pool_row ? (int32_t)i : tags[slot];
        for (size_t h = 0; h < Hkv; ++h) {
            const size_t to = ((size_t)i * Hkv + h) * row;
            if (pool_row) {
                const size_t from = (h * SP + (size_t)i) * row;
                if (k_host) memcpy((char*)k_host + to, pk.data() + from, row);
                if (v_host) memcpy((char*)v_host + to, pv.data() + from, row);
            } else {
                const size_t from = (h * S + slot) * row;
                if (k_host) memcpy((char*)k_host + to, kbuf.data() + from, row);
                if (v_host) memcpy((char*)v_host + to, vbuf.data() + from, row);
            }
        }
    }
    *count = (int32_t)cnt;
    return PSA_OK;
}

PSA_API int psa_seq_blocks(const psa_cache* c, int32_t seq, int32_t* table_host, int32_t* entries,
                           int32_t* free_blocks) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (c->dev.Bs == 0) return fail(PSA_ERR_ARG, "the cache is not paged");
    if (entries == nullptr) return fail(PSA_ERR_ARG, "entries is NULL");
    if (!valid_seq(c, seq)) return fail(PSA_ERR_STATE, "sequence index out of range");
    const int32_t* row = c->btab.data() + (size_t)seq * c->dev.NBT;
    if (table_host) memcpy(table_host, row, (size_t)c->dev.NBT * sizeof(int32_t));
    *entries = c->dev.NBT;
    if (free_blocks) *free_blocks = (int32_t)c->free_blk.size();
    return PSA_OK;
}

PSA_API int64_t psa_seq_length(const psa_cache* c, int32_t seq) {
    if (c == nullptr || !valid_seq(c, seq) || c->pre[seq] < 0) return -1;
    return c->len[seq];
}

PSA_API int psa_set_split_tokens(psa_cache* c, int32_t tokens) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    if (tokens != 0 && tokens < psa::kSplitGranule)
        return fail(PSA_ERR_ARG, "split tokens must be 0 (automatic) or at least 128");
    c->split_tokens = tokens;
    return PSA_OK;
}

PSA_API int psa_profile(psa_cache* c, int32_t enable) {
    if (c == nullptr) return fail(PSA_ERR_ARG, "cache is NULL");
    for (auto& ev : c->pending) {
        hipEventSynchronize(ev.stop);
        hipEventDestroy(ev.start);
        hipEventDestroy(ev.stop);
    }
    c->pending.clear();
    if (enable) {
        for (int i = 0; i < PSA_K_COUNT; ++i) {
            c->total_ms[i] = 0.0;
            c->launches[i] = 0;
        }
    }
    c->profiling = enable != 0;
    return PSA_OK;
}

PSA_API int psa_profile_read(psa_cache* c, int32_t kernel, double* total_ms, int64_t* launches) {
    if (c == nullptr || total_ms == nullptr || launches == nullptr)
        return fail(PSA_ERR_ARG, "NULL argument");
    if (kernel < 0 || kernel >= PSA_K_COUNT) return fail(PSA_ERR_ARG, "unknown kernel id");
    for (auto& ev : c->pending) {
        hipError_t e = hipEventSynchronize(ev.stop);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev.start, ev.stop);
        hipEventDestroy(ev.start);
        hipEventDestroy(ev.stop);
        if (e != hipSuccess) {
            c->pending.clear();
            return hip_fail(e, "profiling event");
        }
        c->total_ms[ev.kernel] += ms;
        c->launches[ev.kernel] += 1;
    }
    c->pending.clear();
    *total_ms = c->total_ms[kernel];
    *launches = c->launches[kernel];
    return PSA_OK;
}

namespace {

struct TrainWs {
    size_t info, di, total;
};

bool train_check(const psa_train_desc* d, TrainWs* ws, const char** why) {
    auto bad = [&](const char* w) {
        *why = w;
        return false;
    };
    if (d == nullptr) return bad("desc is NULL");
    if (d->batch < 1 || d->seq_len < 1) return bad("batch and seq_len must be >= 1");
    if (d->n_kv_heads < 1 || d->n_q_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
        return bad("n_q_heads must be a positive multiple of n_kv_heads");
    const int G = d->n_q_heads / d->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return bad("n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (d->head_dim != 64 && d->head_dim != 128) return bad("head_dim must be 64 or 128");
    if (d->window < 1) return bad("window must be >= 1");
    if (!(d->scale >= 0.f) || !isfinite(d->scale)) return bad("scale must be finite and >= 0");
    if (d->reserved != 0) return bad("reserved must be 0");
    const size_t rows = (size_t)d->batch * d->seq_len * d->n_q_heads;
    if ((size_t)d->batch * d->seq_len > (size_t)1 << 31) return bad("batch * seq_len too large");
    ws->info = 0;
    ws->di = align_up(2 * (size_t)d->batch * 4, 256);
    ws->total = align_up(ws->di + rows * 4, 256);
    return true;
}

int train_run(const psa_train_desc* d, const int32_t* prefix_host, const int32_t* len_host,
              const void* q, const void* k, const void* v, const void* out_in, void* out,
              float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
              size_t ws_bytes, psa_stream stream, bool backward) {
    TrainWs ws;
    const char* why = nullptr;
    if (!train_check(d, &ws, &why)) return fail(PSA_ERR_ARG, why);
    if (prefix_host == nullptr) return fail(PSA_ERR_ARG, "prefix_host is NULL");
    if (workspace == nullptr || ws_bytes < ws.total)
        return fail(PSA_ERR_ARG, "workspace missing or smaller than psa_train_workspace_bytes()");
    if (((uintptr_t)workspace & 255u) != 0) return fail(PSA_ERR_ARG, "workspace must be 256-byte aligned");
    const int B = d->batch;
    std::vector<int32_t> info(2 * (size_t)B);
    for (int b = 0; b < B; ++b) {
        const int32_t n = len_host ? len_host[b] : d->seq_len;
        if (n < 1 || n > d->seq_len) return fail(PSA_ERR_ARG, "len must be in [1, seq_len]");
        if (prefix_host[b] < 0) return fail(PSA_ERR_ARG, "prefix lengths must be >= 0");
        info[b] = prefix_host[b];
        info[B + b] = n;
    }
    hipStream_t s = (hipStream_t)stream;
    char* w = (char*)workspace;
    hipError_t e = hipMemcpyAsync(w + ws.info, info.data(), info.size() * sizeof(int32_t),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "sequence-info upload");
    psa::TrainLaunch t;
    t.q = q;
    t.k = k;
    t.v = v;
    t.dout = dout;
    t.out = backward ? const_cast<void*>(out_in) : out;
    t.dq = dq;
    t.dk = dk;
    t.dv = dv;
    t.lse = lse;
    t.di = (float*)(w + ws.di);
    t.pre = (const int32_t*)(w + ws.info);
    t.len = t.pre + B;
    t.B = B;
    t.T = d->seq_len;
    t.Hq = d->n_q_heads;
    t.Hkv = d->n_kv_heads;
    t.D = d->head_dim;
    t.W = d->window;
    t.scale = d->scale > 0.f ? d->scale : (float)(1.0 / sqrt((double)d->head_dim));
    t.backward = backward;
    e = psa::launch_train(t, s);
    if (e != hipSuccess) return hip_fail(e, backward ? "training backward" : "training forward");
    return PSA_OK;
}

}  // namespace

PSA_API size_t psa_train_workspace_bytes(const psa_train_desc* desc) {
    TrainWs ws;
    const char* why = nullptr;
    if (!train_check(desc, &ws, &why)) {
        fail(PSA_ERR_ARG, why);
        return 0;
    }
    return ws.total;
}

PSA_API int psa_train_fwd(const psa_train_desc* desc, const int32_t* prefix_host,
                          const int32_t* len_host, const void* q, const void* k, const void* v,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          psa_stream stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr)
        return fail(PSA_ERR_ARG, "q, k, v, out or lse is NULL");
    return train_run(desc, prefix_host, len_host, q, k, v, nullptr, out, lse, nullptr, nullptr,
                     nullptr, nullptr, workspace, workspace_bytes, stream, false);
}

PSA_API int psa_train_bwd(const psa_train_desc* desc, const int32_t* prefix_host,
                          const int32_t* len_host, const void* q, const void* k, const void* v,
                          const void* out, const float* lse, const void* dout, void* dq, void* dk,
                          void* dv, void* workspace, size_t workspace_bytes, psa_stream stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr ||
        dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return fail(PSA_ERR_ARG, "an input or output pointer is NULL");
    return train_run(desc, prefix_host, len_host, q, k, v, out, nullptr, const_cast<float*>(lse),
                     dout, dq, dk, dv, workspace, workspace_bytes, stream, true);
}

// ---- psa_train_bwd_noalloc: the backward pass with its scratch in a static device array --
// For callers that cannot allocate device memory. The array's name is a host-side stand-in
// in host code: its device address is taken once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to kernels.

namespace {

constexpr size_t kStaticScratchBytes = (size_t)PSA_TRAIN_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch` (resolved on first use).
int scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(PSA_ERR_ARG, "device index beyond the static scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr || ((uintptr_t)p & 255u) != 0)
            return fail(PSA_ERR_HIP, "static scratch has no 256-byte aligned device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PSA_OK;
}

}  // namespace

PSA_API int psa_train_bwd_noalloc(const psa_train_desc* desc, const int32_t* prefix_host,
                                  const int32_t* len_host, const void* q, const void* k,
                                  const void* v, const void* out, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv,
                                  psa_stream stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr ||
        dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return fail(PSA_ERR_ARG, "an input or output pointer is NULL");
    TrainWs ws;
    const char* why = nullptr;
    if (!train_check(desc, &ws, &why)) return fail(PSA_ERR_ARG, why);
    if (ws.total > kStaticScratchBytes)
        return fail(PSA_ERR_ARG, "the backward pass needs " + std::to_string(ws.total) +
                                     " bytes of scratch; the static scratch holds " +
                                     std::to_string(kStaticScratchBytes));
    void* w = nullptr;
    const int rc = scratch_of_current_device(&w);
    if (rc != PSA_OK) return rc;
    return train_run(desc, prefix_host, len_host, q, k, v, out, nullptr, const_cast<float*>(lse),
                     dout, dq, dk, dv, w, kStaticScratchBytes, stream, true);
}

PSA_API const char* psa_status_string(int status) {
    switch (status) {
        case PSA_OK: return "ok";
        case PSA_ERR_ARG: return "invalid argument";
        case PSA_ERR_STATE: return "invalid state";
        case PSA_ERR_OVERFLOW: return "sequence length overflow";
        case PSA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

PSA_API const char* psa_last_error(void) { return g_err.c_str(); }
