// api.cpp -- the C ABI declared in include/kvcache.h: pool descriptors,
// argument validation, workspace sizing and kernel dispatch. Host code only;
// every computation on the hot path runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <set>
#include <utility>

#include "internal.h"
#include "window.h"

using namespace kvc;

struct kv_pool {
    kv_pool_desc desc;
    char *base;
    size_t bytes;
    size_t off[9];  // region offsets (SIZE_MAX if absent)
    size_t len[9];  // region sizes
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kNone = (size_t)-1;
// Largest batch, kv-head count and work units per sequence: launch grids put
// them in the y or z dimension (at most 65535 workgroups).
constexpr int kMaxGridYZ = 65535;
// Largest grid of the read probe (its workgroups are a measurement knob).
constexpr int kMaxGridX = 65535;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool desc_ok(const kv_pool_desc *d) {
    if (!d) return false;
    if (d->num_blocks < 1 || d->block_size != KV_BLOCK_TOKENS || d->num_kv_heads < 1) return false;
    if (d->num_kv_heads > kMaxGridYZ) return false;
    if (d->head_dim != 64 && d->head_dim != 128) return false;
    if (d->dtype != KV_F32 && d->dtype != KV_BF16 && d->dtype != KV_INT4) return false;
    if (d->dtype == KV_INT4 && d->max_seqs < 1) return false;
    if (d->dtype != KV_INT4 && d->max_seqs < 0) return false;
    return true;
}

// Region sizes of a descriptor (0 = region absent).
void region_sizes(const kv_pool_desc *d, size_t len[9]) {
    for (int i = 0; i < 9; ++i) len[i] = 0;
    const size_t tok = (size_t)d->num_blocks * KV_BLOCK_TOKENS * d->num_kv_heads;  // token rows
    if (d->dtype == KV_INT4) {
        len[KV_REGION_KQ] = tok * d->head_dim / 2;
        len[KV_REGION_VQ] = tok * d->head_dim / 2;
        len[KV_REGION_KS] = (size_t)d->num_blocks * d->num_kv_heads * d->head_dim * 2;
        len[KV_REGION_KM] = len[KV_REGION_KS];
        len[KV_REGION_VS] = tok * 2;
        len[KV_REGION_VM] = tok * 2;
        len[KV_REGION_KTAIL] = (size_t)d->max_seqs * d->num_kv_heads * KV_BLOCK_TOKENS * d->head_dim * 2;
    } else {
        const size_t es = d->dtype == KV_F32 ? 4 : 2;
        len[KV_REGION_K] = tok * d->head_dim * es;
        len[KV_REGION_V] = len[KV_REGION_K];
    }
}

size_t layout(const kv_pool_desc *d, size_t off[9], size_t len[9]) {
    region_sizes(d, len);
    size_t at = 0;
    for (int i = 0; i < 9; ++i) {
        if (len[i] == 0) {
            off[i] = kNone;
            continue;
        }
        off[i] = at;
        at = align_up(at + len[i]);
    }
    return at;
}

PoolPtrs pool_ptrs(const kv_pool *p) {
    auto at = [&](int r) -> char * { return p->off[r] == kNone ? nullptr : p->base + p->off[r]; };
    PoolPtrs q;
    q.k = at(KV_REGION_K);
    q.v = at(KV_REGION_V);
    q.kq = reinterpret_cast<uint8_t *>(at(KV_REGION_KQ));
    q.vq = reinterpret_cast<uint8_t *>(at(KV_REGION_VQ));
    q.ks = reinterpret_cast<uint16_t *>(at(KV_REGION_KS));
    q.km = reinterpret_cast<uint16_t *>(at(KV_REGION_KM));
    q.vs = reinterpret_cast<uint16_t *>(at(KV_REGION_VS));
    q.vm = reinterpret_cast<uint16_t *>(at(KV_REGION_VM));
    q.ktail = reinterpret_cast<uint16_t *>(at(KV_REGION_KTAIL));
    q.q4_span = 0;
    if (p->desc.dtype == KV_INT4) {
        const size_t span = p->off[KV_REGION_VM] + p->len[KV_REGION_VM] - p->off[KV_REGION_KQ];
        if (span <= UINT32_MAX) q.q4_span = (uint32_t)span;
    }
    return q;
}

kv_status hip_status(hipError_t e) { return e == hipSuccess ? KV_OK : KV_ERR_HIP; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Table widths whose token count (max_blocks * 16) the kernels can hold in 32
// bits.
bool max_blocks_ok(int32_t max_blocks) { return max_blocks >= 1 && max_blocks <= INT32_MAX / KV_BLOCK_TOKENS; }

// Attention launch geometry for a call.
struct AttnGeom {
    int kernel;        // 1 VALU, 2 MFMA
    int ncols;         // query columns per kv head
    int ctiles;        // 16-column tiles per kv head
    int ctw;           // column tiles per work unit
    int units;         // work units per sequence
    int slot_cols;     // balanced: rows of one workspace slot
    int schedule;      // KV_SCHED_SPLIT or KV_SCHED_BALANCED
    int split_blocks;
    int max_splits;
    int n_wg;          // balanced: persistent grid
    size_t ws_bytes;   // total workspace
    size_t off_ml;     // offset of the (m, l) partials
    size_t off_prefix; // balanced: offset of the block prefix sums
};

// Largest batch of the balanced schedule (its block prefix sums live in LDS).
constexpr int kMaxBalancedBatch = 8192;
// Balanced schedule: tiles' worth of time a (sequence, unit) pair costs on
// top of its tiles: its start (block ids, query, the first tile's latency,
// the partial or output it writes). Fitted on MI355X to the 8B-shaped
// layers: per-workgroup times showed workgroups that start a second pair
// ending 2-3 us after those with one at the earlier weights (1 for bf16, 5
// for INT4); the kernels measured best at 2 (bf16, 16 query tokens 159 ->
// 156 us, one token level) and 7 (INT4, three waves per SIMD: 51.4 -> 50.5
// us; 52.4 at 4). (A fused INT4 append costs about 2 more tiles, but it is
// not charged: the schedule of the decode step must equal that of the
// separate attention call, so that both give the same bits.) The INT4 kernel
// with more than four query columns (two waves per SIMD) keeps 5: 7 made it
// 1 % slower at 4 query tokens.
constexpr int kSegCost = 2;
constexpr int kSegCostQ4 = 7;
constexpr int kSegCostQ4Cols = 5;
constexpr int kMaxPairCost = kSegCostQ4;

kv_status attn_geom(const kv_pool *pool, int32_t batch, int32_t n_h, int32_t q_len, int32_t max_ctx,
                    const kv_attn_opts *opts, AttnGeom *g) {
    if (batch < 0 || n_h < 1 || max_ctx < 0 || q_len < 1) return KV_ERR_INVALID_ARG;
    if (batch > kMaxGridYZ) return KV_ERR_UNSUPPORTED;
    const int n_kv = pool->desc.num_kv_heads;
    const int dtype = pool->desc.dtype;
    if (n_h % n_kv) return KV_ERR_INVALID_ARG;
    const int group = n_h / n_kv;
    if (opts && (opts->kernel < 0 || opts->kernel > 2 || opts->schedule < 0 || opts->schedule > 2 ||
                 opts->window < 0 || opts->split_blocks < 0))
        return KV_ERR_INVALID_ARG;
    // MFMA kernels: bf16 pools (head_dim 64, 128) and INT4 pools (head_dim 128)
    const bool mfma_ok = dtype == KV_BF16 || (dtype == KV_INT4 && pool->desc.head_dim == 128);
    int kernel = opts ? opts->kernel : 0;
    if (kernel == 2 && !mfma_ok) return KV_ERR_UNSUPPORTED;
    if (kernel == 0) kernel = mfma_ok ? 2 : 1;
    // the VALU kernel serves one query token and groups of up to 16 heads; the
    // MFMA kernels tile any number of query columns (group * q_len) by 16
    if (kernel == 1 && (q_len > 1 || group > kMaxGroup)) return KV_ERR_UNSUPPORTED;
    if ((int64_t)group * q_len > INT32_MAX - 15) return KV_ERR_UNSUPPORTED;
    g->ncols = group * q_len;
    g->ctiles = (g->ncols + 15) / 16;
    // the bf16 MFMA kernels take two column tiles per unit when there are
    // several: each K/V tile is then read once per two column tiles. The
    // balanced schedule takes up to 8 per unit (wide units: a workgroup of
    // up to 4 waves sharing each K/V tile through LDS)
    int sb = opts ? opts->split_blocks : 0;
    int sched = opts ? opts->schedule : 0;
    if (sched == KV_SCHED_AUTO)
        sched = (kernel == 2 && sb == 0 && batch <= kMaxBalancedBatch) ? KV_SCHED_BALANCED : KV_SCHED_SPLIT;
    if (sched == KV_SCHED_BALANCED && (kernel != 2 || batch > kMaxBalancedBatch)) return KV_ERR_UNSUPPORTED;
    const bool bf16_mfma = kernel == 2 && dtype == KV_BF16;
    g->ctw = (bf16_mfma && g->ctiles > 1) ? 2 : 1;
    if (bf16_mfma && sched == KV_SCHED_BALANCED && g->ctiles > 2) g->ctw = g->ctiles > 4 ? 8 : 4;
    const int cgroups = (g->ctiles + g->ctw - 1) / g->ctw;
    if ((int64_t)n_kv * cgroups > kMaxGridYZ) return KV_ERR_UNSUPPORTED;
    g->units = kernel == 2 ? n_kv * cgroups : n_kv;
    g->slot_cols = std::min(16 * g->ctw, g->ncols);
    const int window = opts ? opts->window : 0;
    int nblk = (max_ctx + KV_BLOCK_TOKENS - 1) / KV_BLOCK_TOKENS;
    if (window > 0) {
        // the union of the query tokens' windows spans window + q_len - 1 tokens
        const int wb = (window + q_len - 1 + KV_BLOCK_TOKENS - 1) / KV_BLOCK_TOKENS + 1;
        if (wb < nblk) nblk = wb;
    }
    if (nblk < 1) nblk = 1;
    const size_t D = pool->desc.head_dim;
    g->kernel = kernel;
    g->schedule = sched;
    g->n_wg = 0;
    g->off_prefix = 0;
    if (sched == KV_SCHED_BALANCED) {
        // every attended block of every sequence is one tile; a sequence
        // longer than max_ctx does not fit the promise and reads as bad. The
        // kernels keep the schedule's per-unit prefix sums in 32 bits.
        if ((int64_t)batch * (nblk + kMaxPairCost) > INT32_MAX) return KV_ERR_UNSUPPORTED;
        g->split_blocks = nblk;
        g->max_splits = 1;
        const bool wide = g->ctw > 2 || (g->ctw == 2 && dtype == KV_BF16 && D == 128);  // as launch_attention
        const bool q4_one_score = dtype == KV_INT4 && g->ncols <= 4;  // as launch_attention
        g->n_wg = wide ? wide_grid((int)D, g->ctw, batch, nblk) : balanced_grid(dtype, (int)D, batch, nblk, q4_one_score);
        const size_t rows = (size_t)g->n_wg * 2 * g->slot_cols;
        g->off_ml = align_up(rows * D * sizeof(float));
        g->off_prefix = g->off_ml + align_up(rows * 2 * sizeof(float));
        g->ws_bytes = g->off_prefix + align_up(((size_t)batch + 1) * sizeof(int32_t));
        return KV_OK;
    }
    if (sb == 0) {
        // Aim for about 16 workgroups per compute unit (256 CUs) over the
        // grid when the (sequence, kv head) pairs alone cannot provide them;
        // never split below 8 blocks (the merge then costs more than it saves).
        const long pairs = (long)batch * g->units;
        const long target = 256L * 16;
        long want = pairs > 0 ? (target + pairs - 1) / pairs : 1;
        if (want < 1) want = 1;
        sb = (int)((nblk + want - 1) / want);
        if (sb < 8) sb = 8;
    }
    if (sb > nblk) sb = nblk;
    g->split_blocks = sb;
    g->max_splits = (nblk + sb - 1) / sb;
    if (g->max_splits <= 1) {
        g->ws_bytes = 0;
        g->off_ml = 0;
    } else {
        const size_t rows = (size_t)batch * q_len * n_h * g->max_splits;
        g->off_ml = align_up(rows * D * sizeof(float));
        g->ws_bytes = g->off_ml + align_up(rows * 2 * sizeof(float));
    }
    return KV_OK;
}


// Geometry of paged_decode_attention_shared: the schedule, blocks per work
// item (split schedule), the prefix group record the kernels get by value,
// and the workspace.
struct SharedGeom {
    int split_blocks, max_splits, ncols, ctiles, units;
    int schedule;      // KV_SCHED_SPLIT or KV_SCHED_BALANCED
    int n_wg;          // balanced: persistent grid
    size_t ws_bytes, off_ml;
    size_t off_plan;   // balanced: the plan's prefix sums (int32)
};

kv_status shared_geom(const kv_pool *pool, int32_t batch, int32_t n_h, int32_t max_ctx,
                      const kv_prefix_groups *groups, const kv_attn_opts *opts, SharedGeom *g, PrefixArgs *pa) {
    if (batch < 0 || n_h < 1 || max_ctx < 0 || !groups) return KV_ERR_INVALID_ARG;
    if (batch > kMaxGridYZ) return KV_ERR_UNSUPPORTED;
    const int n_kv = pool->desc.num_kv_heads;
    if (n_h % n_kv) return KV_ERR_INVALID_ARG;
    if (opts && (opts->kernel < 0 || opts->kernel > 2 || opts->schedule < 0 || opts->schedule > 2 ||
                 opts->window < 0 || opts->split_blocks < 0))
        return KV_ERR_INVALID_ARG;
    if (pool->desc.dtype != KV_BF16) return KV_ERR_UNSUPPORTED;
    if (opts && (opts->kernel == 1 || opts->window > 0)) return KV_ERR_UNSUPPORTED;
    const int ng = groups->n_groups;
    if (ng < 0 || ng > KV_MAX_PREFIX_GROUPS) return KV_ERR_INVALID_ARG;
    if (ng > 0 && (!groups->group_start || !groups->prefix_blocks)) return KV_ERR_INVALID_ARG;
    const int group = n_h / n_kv;
    int nblk = (max_ctx + KV_BLOCK_TOKENS - 1) / KV_BLOCK_TOKENS;
    if (nblk < 1) nblk = 1;
    pa->n_groups = ng;
    int max_members = 0, max_prefix = 0;
    long prefix_tiles = 0, member_prefix = 0;  // shared tile loads; prefix blocks summed over members
    int64_t n_pseg = 0;                          // balanced: prefix segments (group, kv head, column tile)
    for (int i = 0; i < ng; ++i) {
        const int a = groups->group_start[i], b = groups->group_start[i + 1], P = groups->prefix_blocks[i];
        if (a < 0 || b < a || b > batch || (i > 0 && a < groups->group_start[i - 1]) || P < 0 || P > nblk)
            return KV_ERR_INVALID_ARG;
        pa->start[i] = a;
        pa->blocks[i] = P;
        max_members = std::max(max_members, b - a);
        max_prefix = std::max(max_prefix, P);
        member_prefix += (long)P * (b - a);
        const long ct = ((long)(b - a) * group + 15) / 16;
        prefix_tiles += (long)P * ct;
        if (P > 0) n_pseg += (int64_t)n_kv * ct;
    }
    if (ng > 0) pa->start[ng] = groups->group_start[ng];
    g->ncols = group;
    g->ctiles = (group + 15) / 16;
    g->units = n_kv * g->ctiles;
    const size_t D = pool->desc.head_dim;
    // Balanced schedule (the default): every tile numbered, equal contiguous
    // shares of one persistent grid; its tile numbers are 32-bit
    const int64_t bal_tiles = (int64_t)n_kv * prefix_tiles + (int64_t)g->units * batch * nblk;
    const bool bal_ok = batch <= kMaxBalancedBatch && bal_tiles <= INT32_MAX;
    int sched = opts ? opts->schedule : 0;
    if (sched == KV_SCHED_AUTO)
        sched = ((opts ? opts->split_blocks : 0) == 0 && bal_ok) ? KV_SCHED_BALANCED : KV_SCHED_SPLIT;
    if (sched == KV_SCHED_BALANCED && !bal_ok) return KV_ERR_UNSUPPORTED;
    g->schedule = sched;
    g->n_wg = 0;
    g->off_plan = 0;
    if (sched == KV_SCHED_BALANCED) {
        g->split_blocks = nblk;  // the longest segment: sizes the staged block ids
        g->max_splits = 1;
        g->n_wg = shared_balanced_grid((int)D, shared_balanced_lds(ng, batch, nblk));
        // slots of 16 rows: two per workgroup, then one per segment
        const size_t rows = ((size_t)2 * g->n_wg + (size_t)n_pseg + (size_t)batch * g->units) * 16;
        g->off_ml = align_up(rows * D * sizeof(float));
        g->off_plan = g->off_ml + align_up(rows * 2 * sizeof(float));
        g->ws_bytes = g->off_plan + align_up(((size_t)2 * (ng + 1) + batch + 1) * sizeof(int32_t));
        return KV_OK;
    }
    pa->ctiles_p = std::max(1, (max_members * group + 15) / 16);
    pa->units_p = n_kv * pa->ctiles_p;
    int sb = opts ? opts->split_blocks : 0;
    if (sb == 0) {
        // about 4.5 work items per resident workgroup: fewer, longer items
        // leave a larger last round idle, more and shorter ones pay the
        // per-item start (block ids, first tile) more often (measured on the
        // long shared-prefix workload: 32 blocks per item, 4.5 rounds, beat
        // 18 to 86 blocks)
        const long tiles = (long)n_kv * (prefix_tiles + g->ctiles * ((long)batch * nblk - member_prefix));
        const long target = (long)balanced_grid(KV_BF16, (int)pool->desc.head_dim, batch, nblk) * 9 / 2;
        sb = (int)std::max(16L, (tiles + target - 1) / target);
    }
    if (sb > nblk) sb = nblk;
    g->split_blocks = sb;
    pa->max_chunks = std::max(1, (max_prefix + sb - 1) / sb);
    pa->suffix_splits = (nblk + sb - 1) / sb;
    g->max_splits = pa->max_chunks + pa->suffix_splits;
    // one flat grid over the prefix and suffix work items
    const int64_t items = (int64_t)ng * pa->units_p * pa->max_chunks + (int64_t)batch * g->units * pa->suffix_splits;
    if (items > INT32_MAX) return KV_ERR_UNSUPPORTED;
    const size_t rows = (size_t)batch * n_h * g->max_splits;
    g->off_ml = align_up(rows * D * sizeof(float));
    g->ws_bytes = g->off_ml + align_up(rows * 2 * sizeof(float));
    return KV_OK;
}

}  // namespace

extern "C" {

const char *kv_status_string(kv_status s) {
    switch (s) {
        case KV_OK: return "ok";
        case KV_ERR_INVALID_ARG: return "invalid argument";
        case KV_ERR_UNSUPPORTED: return "unsupported configuration";
        case KV_ERR_WORKSPACE: return "workspace missing or too small";
        case KV_ERR_HIP: return "HIP launch or runtime error";
        case KV_ERR_TABLE: return "block table or length out of range";
        default: return "unknown status";
    }
}

int32_t kv_abi_version(void) { return KV_ABI_VERSION; }

size_t kv_pool_required_bytes(const kv_pool_desc *desc) {
    if (!desc_ok(desc)) return 0;
    size_t off[9], len[9];
    return layout(desc, off, len);
}

kv_status kv_pool_create(const kv_pool_desc *desc, void *device_mem, size_t bytes, kv_pool_t *out) {
    if (!out) return KV_ERR_INVALID_ARG;
    *out = nullptr;
    if (!desc_ok(desc)) {
        if (desc && desc->block_size == KV_BLOCK_TOKENS && desc->num_blocks >= 1 && desc->num_kv_heads >= 1 &&
            desc->head_dim > 0 && desc->head_dim != 64 && desc->head_dim != 128)
            return KV_ERR_UNSUPPORTED;
        return KV_ERR_INVALID_ARG;
    }
    if (!device_mem || ((uintptr_t)device_mem % kAlign) != 0) return KV_ERR_INVALID_ARG;
    kv_pool *p = new (std::nothrow) kv_pool;
    if (!p) return KV_ERR_INVALID_ARG;
    p->desc = *desc;
    p->base = static_cast<char *>(device_mem);
    const size_t need = layout(desc, p->off, p->len);
    if (bytes < need) {
        delete p;
        return KV_ERR_INVALID_ARG;
    }
    p->bytes = bytes;
    *out = p;
    return KV_OK;
}

kv_status kv_pool_destroy(kv_pool_t pool) {
    if (!pool) return KV_ERR_INVALID_ARG;
    delete pool;
    return KV_OK;
}

kv_status kv_pool_region(kv_pool_t pool, int32_t region, size_t *offset, size_t *bytes) {
    if (!pool || region < 0 || region > 8 || !offset || !bytes) return KV_ERR_INVALID_ARG;
    if (pool->off[region] == kNone) return KV_ERR_INVALID_ARG;
    *offset = pool->off[region];
    *bytes = pool->len[region];
    return KV_OK;
}

kv_status kv_pool_get_desc(kv_pool_t pool, kv_pool_desc *desc) {
    if (!pool || !desc) return KV_ERR_INVALID_ARG;
    *desc = pool->desc;
    return KV_OK;
}

kv_status kv_append_tokens(kv_pool_t pool, const void *k_new, const void *v_new, const int32_t *block_tables,
                           int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                           int32_t n_new, void *stream) {
    if (!pool || batch < 0 || !max_blocks_ok(max_blocks) || n_new < 1) return KV_ERR_INVALID_ARG;
    if (batch > kMaxGridYZ) return KV_ERR_UNSUPPORTED;
    if (batch == 0) return KV_OK;
    if (!k_new || !v_new || !block_tables || !seq_lens) return KV_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return KV_ERR_INVALID_ARG;
    AppendParams a;
    a.pool = pool_ptrs(pool);
    a.k_new = k_new;
    a.v_new = v_new;
    a.tables = block_tables;
    a.seq_lens = seq_lens;
    a.seq_slots = pool->desc.dtype == KV_INT4 ? seq_slots : nullptr;
    a.max_blocks = max_blocks;
    a.batch = batch;
    a.n_kv = pool->desc.num_kv_heads;
    a.head_dim = pool->desc.head_dim;
    a.num_blocks = pool->desc.num_blocks;
    a.max_seqs = pool->desc.max_seqs;
    a.n_new = n_new;
    return hip_status(launch_append(pool->desc.dtype, a, static_cast<hipStream_t>(stream)));
}

kv_status kv_append(kv_pool_t pool, const void *k_new, const void *v_new, const int32_t *block_tables,
                    int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                    void *stream) {
    return kv_append_tokens(pool, k_new, v_new, block_tables, max_blocks, seq_lens, seq_slots, batch, 1, stream);
}

size_t paged_multi_token_attention_workspace_bytes(kv_pool_t pool, int32_t batch, int32_t num_q_heads,
                                                   int32_t q_len, int32_t max_ctx, const kv_attn_opts *opts) {
    AttnGeom g;
    if (!pool || attn_geom(pool, batch, num_q_heads, q_len, max_ctx, opts, &g) != KV_OK) return (size_t)-1;
    return g.ws_bytes;
}

size_t paged_decode_attention_workspace_bytes(kv_pool_t pool, int32_t batch, int32_t num_q_heads, int32_t max_ctx,
                                              const kv_attn_opts *opts) {
    return paged_multi_token_attention_workspace_bytes(pool, batch, num_q_heads, 1, max_ctx, opts);
}

}  // extern "C"

namespace {

// Attention over ctx_lens[b] + ctx_add tokens. With k_new / v_new (a decode
// step: the q_len = ctx_add new tokens are appended first), the append is
// fused into the attention kernel on the bf16 MFMA path and runs as its own
// kernel before attention otherwise.
kv_status attention_impl(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads, int32_t q_len, float scale,
                         const int32_t *block_tables, int32_t max_blocks, const int32_t *ctx_lens,
                         const int32_t *seq_slots, int32_t batch, int32_t max_ctx, void *workspace, size_t ws_bytes,
                         const kv_attn_opts *opts, void *stream, int32_t ctx_add, const void *k_new,
                         const void *v_new) {
    if (!pool || batch < 0 || num_q_heads < 1 || !max_blocks_ok(max_blocks) || max_ctx < 0 || q_len < 1)
        return KV_ERR_INVALID_ARG;
    if (max_ctx > max_blocks * KV_BLOCK_TOKENS) return KV_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return KV_ERR_INVALID_ARG;
    AttnGeom g;
    const kv_status gs = attn_geom(pool, batch, num_q_heads, q_len, max_ctx, opts, &g);
    if (gs != KV_OK) return gs;
    if (batch == 0) return KV_OK;
    if (!q || !out || !block_tables || !ctx_lens) return KV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out)) return KV_ERR_INVALID_ARG;
    if (k_new && (!v_new || !aligned16(k_new) || !aligned16(v_new))) return KV_ERR_INVALID_ARG;
    if (g.ws_bytes > 0 && (!workspace || ws_bytes < g.ws_bytes || !aligned16(workspace))) return KV_ERR_WORKSPACE;

    const int dtype = pool->desc.dtype;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the append runs inside the attention kernel on the MFMA path: bf16
    // pools for any q_len (every unit takes the new rows from k_new / v_new),
    // INT4 pools for one new token per sequence when a kv head is one work
    // unit. With several units per kv head (more than 16 query heads per kv
    // head) only the first codes the token while the others read the same
    // last block, so the append kernel runs first instead.
    const bool fused = k_new && g.kernel == 2 &&
                       (dtype == KV_BF16 || (dtype == KV_INT4 && q_len == 1 && g.ctiles == 1));
    if (k_new && !fused) {
        const kv_status st = kv_append_tokens(pool, k_new, v_new, block_tables, max_blocks, ctx_lens, seq_slots,
                                              batch, ctx_add, stream);
        if (st != KV_OK) return st;
    }
    AttnParams a;
    a.ctx_add = ctx_add;
    a.k_new = fused ? k_new : nullptr;
    a.v_new = fused ? v_new : nullptr;
    a.pool = pool_ptrs(pool);
    a.q = q;
    a.out = out;
    a.tables = block_tables;
    a.ctx_lens = ctx_lens;
    a.seq_slots = dtype == KV_INT4 ? seq_slots : nullptr;
    char *ws = static_cast<char *>(workspace);
    a.ws_o = g.ws_bytes ? reinterpret_cast<float *>(ws) : nullptr;
    a.ws_ml = g.ws_bytes ? reinterpret_cast<float *>(ws + g.off_ml) : nullptr;
    a.ws_prefix = g.off_prefix ? reinterpret_cast<int32_t *>(ws + g.off_prefix) : nullptr;
    a.max_blocks = max_blocks;
    a.batch = batch;
    a.n_h = num_q_heads;
    a.n_kv = pool->desc.num_kv_heads;
    a.group = num_q_heads / a.n_kv;
    a.head_dim = pool->desc.head_dim;
    a.num_blocks = pool->desc.num_blocks;
    a.max_seqs = pool->desc.max_seqs;
    a.split_blocks = g.split_blocks;
    a.max_splits = g.max_splits;
    a.window = opts ? opts->window : 0;
    a.q_len = q_len;
    a.ncols = g.ncols;
    a.ctiles = g.ctiles;
    a.ctw = g.ctw;
    a.units = g.units;
    a.slot_cols = g.slot_cols;
    a.schedule = g.schedule;
    a.n_wg = g.n_wg;
    const bool balanced = g.schedule == KV_SCHED_BALANCED;
    a.seg_cost = !balanced ? 0 : dtype != KV_INT4 ? kSegCost : g.ncols <= 4 ? kSegCostQ4 : kSegCostQ4Cols;
    a.pace = balanced ? 1 : 0;
    a.xcd_shares = balanced && dtype == KV_INT4 ? 1 : 0;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)

    void *const *ev = opts ? opts->events : nullptr;
    auto evt = [&](int i) { return ev ? static_cast<hipEvent_t>(ev[i]) : nullptr; };
    hipError_t e = launch_attention(dtype, g.kernel, a, s, evt(0), evt(1));
    if (e != hipSuccess) return KV_ERR_HIP;
    e = launch_merge(a, s, evt(2));
    if (e != hipSuccess) return KV_ERR_HIP;
    return KV_OK;
}

}  // namespace

extern "C" {

kv_status paged_multi_token_attention(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads, int32_t q_len,
                                      float scale, const int32_t *block_tables, int32_t max_blocks,
                                      const int32_t *ctx_lens, const int32_t *seq_slots, int32_t batch,
                                      int32_t max_ctx, void *workspace, size_t ws_bytes, const kv_attn_opts *opts,
                                      void *stream) {
    return attention_impl(pool, q, out, num_q_heads, q_len, scale, block_tables, max_blocks, ctx_lens, seq_slots,
                          batch, max_ctx, workspace, ws_bytes, opts, stream, 0, nullptr, nullptr);
}

kv_status kv_decode_step(kv_pool_t pool, const void *k_new, const void *v_new, const void *q, float *out,
                         int32_t num_q_heads, int32_t q_len, float scale, const int32_t *block_tables,
                         int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                         int32_t max_ctx, void *workspace, size_t ws_bytes, const kv_attn_opts *opts, void *stream) {
    if (batch > 0 && (!k_new || !v_new)) return KV_ERR_INVALID_ARG;
    return attention_impl(pool, q, out, num_q_heads, q_len, scale, block_tables, max_blocks, seq_lens, seq_slots,
                          batch, max_ctx, workspace, ws_bytes, opts, stream, q_len, k_new, v_new);
}


kv_status kv_decode_step_noalloc(kv_pool_t pool, const void *k_new, const void *v_new, const void *q, float *out,
                                 int32_t num_q_heads, int32_t q_len, float scale, const int32_t *block_tables,
                                 int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                                 int32_t max_ctx, const kv_attn_opts *opts, void *stream) {
    if (!pool) return KV_ERR_INVALID_ARG;
    const size_t need = paged_multi_token_attention_workspace_bytes(pool, batch, num_q_heads, q_len, max_ctx, opts);
    if (need == (size_t)-1)  // a geometry the library refuses: the full call reports why, before any launch
        return kv_decode_step(pool, k_new, v_new, q, out, num_q_heads, q_len, scale, block_tables, max_blocks,
                              seq_lens, seq_slots, batch, max_ctx, nullptr, 0, opts, stream);
    if (need > kNoallocScratchBytes) return KV_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0 && batch > 0) {
        ws = noalloc_scratch();
        if (!ws) return KV_ERR_HIP;
    }
    return kv_decode_step(pool, k_new, v_new, q, out, num_q_heads, q_len, scale, block_tables, max_blocks, seq_lens,
                          seq_slots, batch, max_ctx, ws, ws ? kNoallocScratchBytes : 0, opts, stream);
}

kv_status paged_decode_attention(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads, float scale,
                                 const int32_t *block_tables, int32_t max_blocks, const int32_t *ctx_lens,
                                 const int32_t *seq_slots, int32_t batch, int32_t max_ctx, void *workspace,
                                 size_t ws_bytes, const kv_attn_opts *opts, void *stream) {
    return paged_multi_token_attention(pool, q, out, num_q_heads, 1, scale, block_tables, max_blocks, ctx_lens,
                                       seq_slots, batch, max_ctx, workspace, ws_bytes, opts, stream);
}

size_t paged_decode_attention_shared_workspace_bytes(kv_pool_t pool, int32_t batch, int32_t num_q_heads,
                                                     int32_t max_ctx, const kv_prefix_groups *groups,
                                                     const kv_attn_opts *opts) {
    SharedGeom g;
    PrefixArgs pa;
    if (!pool || shared_geom(pool, batch, num_q_heads, max_ctx, groups, opts, &g, &pa) != KV_OK) return (size_t)-1;
    return g.ws_bytes;
}

kv_status paged_decode_attention_shared(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads,
                                        float scale, const int32_t *block_tables, int32_t max_blocks,
                                        const int32_t *ctx_lens, int32_t batch, int32_t max_ctx,
                                        const kv_prefix_groups *groups, void *workspace, size_t ws_bytes,
                                        const kv_attn_opts *opts, void *stream) {
    if (!pool || batch < 0 || num_q_heads < 1 || !max_blocks_ok(max_blocks) || max_ctx < 0)
        return KV_ERR_INVALID_ARG;
    if (max_ctx > max_blocks * KV_BLOCK_TOKENS) return KV_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return KV_ERR_INVALID_ARG;
    SharedGeom g;
    PrefixArgs pa;
    const kv_status gs = shared_geom(pool, batch, num_q_heads, max_ctx, groups, opts, &g, &pa);
    if (gs != KV_OK) return gs;
    if (batch == 0) return KV_OK;
    if (!q || !out || !block_tables || !ctx_lens) return KV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out)) return KV_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < g.ws_bytes || !aligned16(workspace)) return KV_ERR_WORKSPACE;
    AttnParams a{};
    a.ctx_add = 0;
    a.k_new = a.v_new = nullptr;
    a.pool = pool_ptrs(pool);
    a.q = q;
    a.out = out;
    a.tables = block_tables;
    a.ctx_lens = ctx_lens;
    a.seq_slots = nullptr;
    char *ws = static_cast<char *>(workspace);
    a.ws_o = reinterpret_cast<float *>(ws);
    a.ws_ml = reinterpret_cast<float *>(ws + g.off_ml);
    a.ws_prefix = g.off_plan ? reinterpret_cast<int32_t *>(ws + g.off_plan) : nullptr;
    a.max_blocks = max_blocks;
    a.batch = batch;
    a.n_h = num_q_heads;
    a.n_kv = pool->desc.num_kv_heads;
    a.group = num_q_heads / a.n_kv;
    a.head_dim = pool->desc.head_dim;
    a.num_blocks = pool->desc.num_blocks;
    a.max_seqs = pool->desc.max_seqs;
    a.split_blocks = g.split_blocks;
    a.max_splits = g.max_splits;
    a.window = 0;
    a.q_len = 1;
    a.ncols = g.ncols;
    a.ctiles = g.ctiles;
    a.ctw = 1;
    a.units = g.units;
    a.slot_cols = g.ncols < 16 ? g.ncols : 16;
    a.schedule = g.schedule;
    a.n_wg = g.n_wg;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    void *const *ev = opts ? opts->events : nullptr;
    auto evt = [&](int i) { return ev ? static_cast<hipEvent_t>(ev[i]) : nullptr; };
    return hip_status(launch_attention_shared(a, pa, static_cast<hipStream_t>(stream), evt(0), evt(1), evt(2)));
}

kv_status kv_quantize_int4(kv_pool_t dst, kv_pool_t src, const int32_t *block_tables, int32_t max_blocks,
                           const int32_t *lens, const int32_t *seq_slots, int32_t batch, void *stream) {
    if (!dst || !src || batch < 0 || !max_blocks_ok(max_blocks)) return KV_ERR_INVALID_ARG;
    if (batch > kMaxGridYZ) return KV_ERR_UNSUPPORTED;
    if (dst->desc.dtype != KV_INT4 || src->desc.dtype != KV_BF16) return KV_ERR_INVALID_ARG;
    if (dst->desc.num_blocks != src->desc.num_blocks || dst->desc.num_kv_heads != src->desc.num_kv_heads ||
        dst->desc.head_dim != src->desc.head_dim)
        return KV_ERR_INVALID_ARG;
    if (batch == 0) return KV_OK;
    if (!block_tables || !lens) return KV_ERR_INVALID_ARG;
    QuantParams a;
    a.dst = pool_ptrs(dst);
    a.src = pool_ptrs(src);
    a.tables = block_tables;
    a.lens = lens;
    a.seq_slots = seq_slots;
    a.max_blocks = max_blocks;
    a.batch = batch;
    a.n_kv = dst->desc.num_kv_heads;
    a.head_dim = dst->desc.head_dim;
    a.num_blocks = dst->desc.num_blocks;
    a.max_seqs = dst->desc.max_seqs;
    return hip_status(launch_quantize_int4(a, static_cast<hipStream_t>(stream)));
}

kv_status rope_rerotate(kv_pool_t pool, const int32_t *chunk_blocks, int32_t first_slot, int32_t num_tokens,
                        int32_t delta, float base, int32_t style, void *stream) {
    if (!pool || first_slot < 0 || num_tokens < 0 || (style != 0 && style != 1)) return KV_ERR_INVALID_ARG;
    if ((int64_t)first_slot + num_tokens > INT32_MAX) return KV_ERR_INVALID_ARG;
    if (!(base > 0.0f) || !std::isfinite(base)) return KV_ERR_INVALID_ARG;
    if (pool->desc.dtype == KV_INT4) return KV_ERR_UNSUPPORTED;
    if (num_tokens == 0) return KV_OK;
    if (!chunk_blocks) return KV_ERR_INVALID_ARG;
    RopeParams a;
    a.k = pool_ptrs(pool).k;
    a.chunk_blocks = chunk_blocks;
    a.first_slot = first_slot;
    a.num_tokens = num_tokens;
    a.n_kv = pool->desc.num_kv_heads;
    a.head_dim = pool->desc.head_dim;
    a.num_blocks = pool->desc.num_blocks;
    a.style = style;
    // angles in fp64: pair i turns by delta * base^(-2i / head_dim)
    for (int i = 0; i < 64; ++i) {
        a.cos_t[i] = 1.0f;
        a.sin_t[i] = 0.0f;
    }
    for (int i = 0; i < a.head_dim / 2; ++i) {
        const double theta = std::pow((double)base, -(2.0 * i) / a.head_dim);
        const double phi = (double)delta * theta;
        a.cos_t[i] = (float)std::cos(phi);
        a.sin_t[i] = (float)std::sin(phi);
    }
    return hip_status(launch_rope(pool->desc.dtype, a, static_cast<hipStream_t>(stream)));
}

static CopyParams copy_params(const kv_pool *pool) {
    CopyParams c;
    c.nreg = 0;
    c.per_block = 0;
    const int order[6] = {KV_REGION_K, KV_REGION_V, KV_REGION_KQ, KV_REGION_KS, KV_REGION_KM, KV_REGION_VQ};
    const int order4[6] = {KV_REGION_KQ, KV_REGION_KS, KV_REGION_KM, KV_REGION_VQ, KV_REGION_VS, KV_REGION_VM};
    const int *ord = pool->desc.dtype == KV_INT4 ? order4 : order;
    for (int i = 0; i < 6; ++i) {
        const int r = ord[i];
        if (pool->off[r] == kNone) continue;
        const size_t per = pool->len[r] / (size_t)pool->desc.num_blocks;  // a multiple of 16
        c.region[c.nreg] = pool->base + pool->off[r];
        c.chunks[c.nreg] = (uint32_t)(per / 16);
        c.per_block += (uint32_t)(per / 16);
        ++c.nreg;
    }
    c.num_blocks = pool->desc.num_blocks;
    return c;
}

size_t kv_block_bytes(kv_pool_t pool) {
    if (!pool) return 0;
    return (size_t)copy_params(pool).per_block * 16;
}

kv_status kv_layer_window(const int32_t *windows, int32_t n_windows, int32_t layer, int32_t *window_out) {
    if (!windows || !window_out || n_windows <= 0 || layer < 0) return KV_ERR_INVALID_ARG;
    const int32_t w = windows[layer % n_windows];
    if (w <= 0) return KV_ERR_INVALID_ARG;
    *window_out = w;
    return KV_OK;
}

kv_status kv_window_released_blocks(const int32_t *seq_lens, int32_t batch, int32_t window, int32_t *released,
                                    void *stream) {
    if (batch < 0 || window < 0) return KV_ERR_INVALID_ARG;
    if (batch == 0) return KV_OK;
    if (!seq_lens || !released) return KV_ERR_INVALID_ARG;
    return hip_status(launch_window_released(seq_lens, batch, window, released, static_cast<hipStream_t>(stream)));
}

kv_status kv_copy_blocks(kv_pool_t pool, const int32_t *src_blocks, const int32_t *dst_blocks, int32_t n,
                         void *stream) {
    if (!pool || n < 0) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    if (!src_blocks || !dst_blocks) return KV_ERR_INVALID_ARG;
    CopyParams c = copy_params(pool);
    c.src = src_blocks;
    c.dst = dst_blocks;
    c.buffer = nullptr;
    c.n = n;
    c.mode = 0;
    return hip_status(launch_copy_blocks(c, static_cast<hipStream_t>(stream)));
}

kv_status kv_gather_blocks(kv_pool_t pool, const int32_t *blocks, int32_t n, void *buffer, size_t bytes,
                           void *stream) {
    if (!pool || n < 0) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    CopyParams c = copy_params(pool);
    if (!blocks || !buffer || !aligned16(buffer) || bytes < (size_t)n * c.per_block * 16) return KV_ERR_INVALID_ARG;
    c.src = blocks;
    c.dst = nullptr;
    c.buffer = static_cast<char *>(buffer);
    c.n = n;
    c.mode = 1;
    return hip_status(launch_copy_blocks(c, static_cast<hipStream_t>(stream)));
}

kv_status kv_scatter_blocks(kv_pool_t pool, const int32_t *blocks, int32_t n, const void *buffer, size_t bytes,
                            void *stream) {
    if (!pool || n < 0) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    CopyParams c = copy_params(pool);
    if (!blocks || !buffer || !aligned16(buffer) || bytes < (size_t)n * c.per_block * 16) return KV_ERR_INVALID_ARG;
    c.src = nullptr;
    c.dst = blocks;
    c.buffer = const_cast<char *>(static_cast<const char *>(buffer));
    c.n = n;
    c.mode = 2;
    return hip_status(launch_copy_blocks(c, static_cast<hipStream_t>(stream)));
}

kv_status kv_token_deviation(kv_pool_t pool, const int32_t *block_tables, int32_t max_blocks, int32_t batch,
                             const int32_t *row_seq, const int32_t *row_pos, int32_t n_rows, const void *k_re,
                             const void *v_re, double *deviation, void *stream) {
    if (!pool || !max_blocks_ok(max_blocks) || batch < 0 || n_rows < 0) return KV_ERR_INVALID_ARG;
    if (pool->desc.dtype == KV_INT4) return KV_ERR_UNSUPPORTED;
    if (n_rows == 0) return KV_OK;
    if (!block_tables || !row_seq || !row_pos || !k_re || !v_re || !deviation) return KV_ERR_INVALID_ARG;
    if (!aligned16(k_re) || !aligned16(v_re)) return KV_ERR_INVALID_ARG;
    const PoolPtrs pp = pool_ptrs(pool);
    DeviationParams a;
    a.k = pp.k;
    a.v = pp.v;
    a.tables = block_tables;
    a.row_seq = row_seq;
    a.row_pos = row_pos;
    a.k_re = k_re;
    a.v_re = v_re;
    a.out = deviation;
    a.max_blocks = max_blocks;
    a.batch = batch;
    a.n_kv = pool->desc.num_kv_heads;
    a.head_dim = pool->desc.head_dim;
    a.num_blocks = pool->desc.num_blocks;
    a.n_rows = n_rows;
    const int es = pool->desc.dtype == KV_F32 ? 4 : 2;
    const int chunks = a.n_kv * a.head_dim * es / 16;
    int lanes = 64;
    while (lanes > 1 && lanes / 2 >= chunks) lanes /= 2;
    a.lanes = lanes;
    return hip_status(launch_deviation(pool->desc.dtype, a, static_cast<hipStream_t>(stream)));
}

kv_status kv_topk_select(const double *values, const int32_t *seg_offsets, const int32_t *seg_k, int32_t n_seg,
                         int32_t *selected, void *stream) {
    if (n_seg < 0) return KV_ERR_INVALID_ARG;
    if (n_seg == 0) return KV_OK;
    if (!values || !seg_offsets || !seg_k || !selected) return KV_ERR_INVALID_ARG;
    TopkParams t;
    t.values = values;
    t.offsets = seg_offsets;
    t.ks = seg_k;
    t.selected = selected;
    t.n_seg = n_seg;
    return hip_status(launch_topk(t, static_cast<hipStream_t>(stream)));
}

double kv_recompute_ratio(double load_time, double token_time, int32_t num_tokens, double floor_ratio) {
    double r = (num_tokens > 0 && token_time > 0.0) ? load_time / ((double)num_tokens * token_time) : 1.0;
    if (!(r >= floor_ratio)) r = floor_ratio;  // also a NaN ratio
    if (r > 1.0) r = 1.0;
    return r;
}

int32_t kv_recompute_count(double ratio, int32_t num_tokens) {
    if (num_tokens <= 0 || !(ratio > 0.0)) return 0;
    const double c = std::ceil(ratio * (double)num_tokens);
    return c >= (double)num_tokens ? num_tokens : (int32_t)c;
}

kv_status kv_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *sink, void *stream) {
    if (!buf || !sink || !aligned16(buf) || bytes % 4096 != 0 || workgroups < 0 || workgroups > kMaxGridX)
        return KV_ERR_INVALID_ARG;
    if (bytes / 4096 > INT32_MAX) return KV_ERR_UNSUPPORTED;  // piece indices stay far from 2^32
    return hip_status(launch_read_probe(buf, bytes, workgroups ? workgroups : 2048, sink,
                                        static_cast<hipStream_t>(stream)));
}

kv_status kv_validate_tables(const kv_pool_desc *desc, const int32_t *block_tables, int32_t max_blocks,
                             const int32_t *lens, int32_t batch, int32_t appending, int32_t *bad_row) {
    if (bad_row) *bad_row = -1;
    if (!desc_ok(desc) || batch < 0 || !max_blocks_ok(max_blocks)) return KV_ERR_INVALID_ARG;
    if (batch > 0 && (!block_tables || !lens)) return KV_ERR_INVALID_ARG;
    std::set<std::pair<int, int>> slots;
    for (int b = 0; b < batch; ++b) {
        const long n = (long)lens[b] + (appending ? 1 : 0);
        bool ok = lens[b] >= 0 && n <= (long)max_blocks * KV_BLOCK_TOKENS;
        const int nb = ok ? (int)((n + KV_BLOCK_TOKENS - 1) / KV_BLOCK_TOKENS) : 0;
        for (int j = 0; ok && j < nb; ++j) {
            const int32_t p = block_tables[(size_t)b * max_blocks + j];
            if (p < 0 || p >= desc->num_blocks) ok = false;
        }
        if (ok && appending) {
            const int32_t p = block_tables[(size_t)b * max_blocks + lens[b] / KV_BLOCK_TOKENS];
            ok = slots.insert({p, lens[b] % KV_BLOCK_TOKENS}).second;
        }
        if (!ok) {
            if (bad_row) *bad_row = b;
            return KV_ERR_TABLE;
        }
    }
    return KV_OK;
}

}  // extern "C"
