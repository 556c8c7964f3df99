// internal.h -- parameter records shared by the host API (api.cpp) and the
// kernel launchers (*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvcache.h"

namespace kvc {

constexpr int kBlock = KV_BLOCK_TOKENS;  // tokens per physical block
constexpr int kMaxGroup = 16;            // largest query group (n_h / n_kv)

// Device pointers of every region of a pool (null where the dtype has none).
struct PoolPtrs {
    void *k, *v;                 // f32 / bf16
    uint8_t *kq, *vq;            // int4 codes
    uint16_t *ks, *km, *vs, *vm; // fp16 scale / min
    uint16_t *ktail;             // bf16 K tail
    uint32_t q4_span;            // INT4: bytes from kq to the end of vm when below 4 GiB, else 0
};

// Everything a kernel needs about one attention call. Passed by value.
struct AttnParams {
    PoolPtrs pool;
    const void *q;
    float *out;
    const int32_t *tables;
    const int32_t *ctx_lens;
    const int32_t *seq_slots;
    float *ws_o;   // [batch][n_h][max_splits][head_dim]
    float *ws_ml;  // [batch][n_h][max_splits][2]  (running max in log2 units, sum)
    int32_t max_blocks, batch, n_h, n_kv, group, head_dim, num_blocks, max_seqs;
    int32_t split_blocks, max_splits, window;
    int32_t q_len;     // query tokens per sequence (1: decode)
    int32_t ncols;     // query columns per kv head: group * q_len
    int32_t ctiles;    // 16-column tiles per kv head
    int32_t ctw;       // column tiles per work unit (MFMA kernels: 2 on the bf16 path when ctiles > 1, else 1;
                       // balanced bf16 with more than 2 tiles: 4 or 8, one workgroup of ctw / 2 waves)
    int32_t units;     // work units per sequence: n_kv * ceil(ctiles / ctw)
    int32_t slot_cols; // balanced: columns of one workspace slot, min(16 * ctw, ncols)
    int32_t schedule;  // KV_SCHED_SPLIT or KV_SCHED_BALANCED
    int32_t n_wg;      // balanced: persistent grid size
    int32_t seg_cost;  // balanced: schedule positions a (sequence, unit) pair takes beyond its tiles
    int32_t pace;      // balanced INT4: waves set their issue priority from their progress (1) or not (0)
    int32_t xcd_shares;  // balanced: shares numbered XCD by XCD (XcdShares: INT4 pools) (1) or not (Shares) (0)
    int32_t *ws_prefix;  // balanced: [batch + 1] schedule positions per unit before each sequence
    float scale_log2;  // scale * log2(e): scores are kept in log2 units
    // Decode step: the attended length of sequence b is ctx_lens[b] + ctx_add
    // (ctx_lens then holds the lengths before the step's append). With
    // k_new / v_new set ([batch][ctx_add][n_kv][head_dim]; MFMA path: bf16
    // pools, or INT4 pools with ctx_add 1) the append is fused: bf16 tiles
    // take the new tokens' rows from there and the first column tile of each
    // kv head writes them into the pool; on INT4 the segment that ends with a
    // sequence's last block codes the new token into the pool first.
    int32_t ctx_add;
    const void *k_new, *v_new;
};

// Length after adding `add` tokens to a length L read from device metadata,
// summed in 64 bits (a corrupt L near INT32_MAX must not wrap); -1 when L is
// negative or the sum leaves int32.
__host__ __device__ inline int length_after(int L, int add) {
    if (L < 0) return -1;
    const long long n = (long long)L + add;
    return n > 2147483647LL ? -1 : (int)n;
}

// Whether n_new tokens appended at positions L0 .. L0 + n_new - 1 fit a table
// of max_blocks blocks (64-bit sum).
__host__ __device__ inline bool append_fits(int L0, int n_new, int max_blocks) {
    return L0 >= 0 && (long long)L0 + n_new <= (long long)max_blocks * kBlock;
}

// Positions [0, total) of a balanced schedule over n workgroups, as evenly
// as whole positions allow: q = total / n each, and one more for the
// total % n workgroups dispatched first (no share is left empty while others
// hold one position above the average; a SIMD issues to its oldest wave
// first). Share i is workgroup i.
struct Shares {
    long q;
    int r;
    __host__ __device__ inline long start(int w) const { return (long)w * q + (w < r ? w : r); }
    // the share that holds position p (0 <= p < total)
    __host__ __device__ inline int wg_of(long p) const {
        const long big = (long)r * (q + 1);
        return p < big ? (int)(p / (q + 1)) : r + (int)((p - big) / q);
    }
    __host__ __device__ inline int share_of(int i) const { return i; }
};
__host__ __device__ inline Shares shares_of(long total, int n) {
    Shares sh;
    sh.q = total / n;
    sh.r = (int)(total - sh.q * n);
    return sh;
}

// The same split with the shares numbered XCD by XCD, for the INT4 decode
// kernels. Workgroup i of a launch runs on XCD i mod 8, and each of the 8
// XCDs has an L2 of its own. When every share holds a position (q > 0), XCD x
// holds the consecutive shares first(x) ... first(x + 1) - 1, share
// first(x) + k being workgroup 8 k + x, and the total % n longer shares are
// still the workgroups dispatched first. Pairs next to each other in the
// schedule (the kv heads of one sequence, whose INT4 V scale and min rows
// share cache lines) thus run on one XCD at the same time, and each XCD's run
// of positions differs from the others' by at most one position beyond q
// times its workgroup count. With fewer positions than workgroups (q = 0) it
// is Shares' numbering, so the shares that hold a position are always the
// first ones: a pair's pieces sit in consecutive shares, which the merges
// rely on. (The bf16 kernels read no cache line twice; there this numbering
// measured no faster.)
struct XcdShares {
    long q;
    bool xcd;       // q > 0
    int n, q8, r8;  // XCD x holds q8 + (x < r8) workgroups
    int a, b;       // total % n = 8 a + b: XCD x has a + (x < b) longer shares
    __host__ __device__ inline int first(int x) const { return x * q8 + (x < r8 ? x : r8); }
    __host__ __device__ inline int longer(int x) const { return a + (x < b ? 1 : 0); }
    // first position of XCD x's run
    __host__ __device__ inline long xcd_start(int x) const { return (long)first(x) * q + (long)a * x + (x < b ? x : b); }
    // the share workgroup i works on
    __host__ __device__ inline int share_of(int i) const { return xcd ? first(i & 7) + (i >> 3) : i; }
    __host__ __device__ inline long start(int w) const {
        if (!xcd) {
            const int r = 8 * a + b;
            return w < r ? w : r;  // q = 0
        }
        if (w >= n) return xcd_start(8);
        const int big = r8 * (q8 + 1);
        const int x = w < big ? w / (q8 + 1) : r8 + (w - big) / q8;
        const int k = w - first(x);
        return xcd_start(x) + (long)k * q + (k < longer(x) ? k : longer(x));
    }
    // the share that holds position p (0 <= p < total)
    __host__ __device__ inline int wg_of(long p) const {
        if (!xcd) return (int)p;  // q = 0: share p holds position p
        int x = 0;
        long s0 = 0, s1 = (long)(q8 + (r8 > 0 ? 1 : 0)) * q + longer(0);  // XCD x's run is [s0, s1)
        while (x < 7 && s1 <= p) {
            ++x;
            s0 = s1;
            s1 += (long)(q8 + (x < r8 ? 1 : 0)) * q + longer(x);
        }
        const long off = p - s0;
        const int e = longer(x);
        const long big = (long)e * (q + 1);
        return first(x) + (off < big ? (int)(off / (q + 1)) : e + (int)((off - big) / q));
    }
};
__host__ __device__ inline XcdShares xcd_shares_of(long total, int n) {
    XcdShares sh;
    sh.q = total / n;
    const int r = (int)(total - sh.q * n);
    sh.xcd = sh.q > 0;
    sh.n = n;
    sh.q8 = n >> 3;
    sh.r8 = n & 7;
    sh.a = r >> 3;
    sh.b = r & 7;
    return sh;
}

// Attended length of sequence b (negative: invalid).
__host__ __device__ inline int ctx_of(const AttnParams &p, int b) {
    const int L = p.ctx_lens[b];
    return p.ctx_add == 0 ? L : length_after(L, p.ctx_add);
}

struct AppendParams {
    PoolPtrs pool;
    const void *k_new, *v_new;  // [batch][n_new][n_kv][head_dim]
    const int32_t *tables, *seq_lens, *seq_slots;
    int32_t max_blocks, batch, n_kv, head_dim, num_blocks, max_seqs;
    int32_t n_new;  // tokens appended per sequence, at positions seq_lens[b] ..
};

struct QuantParams {
    PoolPtrs dst, src;
    const int32_t *tables, *lens, *seq_slots;
    int32_t max_blocks, batch, n_kv, head_dim, num_blocks, max_seqs;
};

struct RopeParams {
    void *k;
    const int32_t *chunk_blocks;
    int32_t first_slot, num_tokens, n_kv, head_dim, num_blocks, style;
    float cos_t[64], sin_t[64];  // per pair i < head_dim / 2
};

// Whole-block copies between per-block regions and a packed buffer.
struct CopyParams {
    char *region[6];       // per-block regions, in packed order
    uint32_t chunks[6];    // 16-byte chunks per block of each region
    int32_t nreg;
    uint32_t per_block;    // 16-byte chunks of one packed block
    const int32_t *src, *dst;  // block lists (mode 0: src -> dst; 1: src -> buffer; 2: buffer -> dst)
    char *buffer;
    int32_t n, num_blocks, mode;
};

struct DeviationParams {
    const void *k, *v;            // pool K / V (f32 or bf16)
    const int32_t *tables, *row_seq, *row_pos;
    const void *k_re, *v_re;      // [n_rows][n_kv][head_dim], pool dtype
    double *out;                  // [n_rows]
    int32_t max_blocks, batch, n_kv, head_dim, num_blocks, n_rows;
    int32_t lanes;                // lanes per token: 64, or a smaller power of two
};

struct TopkParams {
    const double *values;
    const int32_t *offsets, *ks;  // [n_seg + 1], [n_seg]
    int32_t *selected;            // segment s writes at offsets[s] ..
    int32_t n_seg;
};

// Groups of sequences whose tables share a prefix of physical blocks
// (paged_decode_attention_shared). Passed by value beside AttnParams.
// Group i is sequences start[i] .. start[i+1]-1; their first blocks[i]
// logical blocks name the same physical blocks. Split schedule: work items
// of the shared kernel are first the prefix items (group, unit, chunk), then
// the suffix items (sequence, unit, split); partial slots of a row: the
// group's prefix chunks first, then the sequence's suffix splits. Balanced
// schedule: only n_groups, start and blocks are used (the kernel plans the
// rest itself).
struct PrefixArgs {
    int32_t n_groups;
    int32_t units_p;      // prefix units per group: n_kv * column tiles of the largest group
    int32_t ctiles_p;     // column tiles of a prefix unit
    int32_t max_chunks;   // prefix chunks of the longest prefix
    int32_t suffix_splits;// suffix splits of the longest sequence
    int32_t start[KV_MAX_PREFIX_GROUPS + 1];
    int32_t blocks[KV_MAX_PREFIX_GROUPS];
};

// Kernel launchers (defined in the .hip files). Each returns the launch status.
hipError_t launch_deviation(int dtype, const DeviationParams &p, hipStream_t s);
hipError_t launch_topk(const TopkParams &p, hipStream_t s);
hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t s);
hipError_t launch_append(int dtype, const AppendParams &p, hipStream_t s);
// e0 / e1 (may be null): events recorded at the start / end of the attention
// kernel; e_end: at the end of the merge (recorded on the stream when no merge
// kernel runs).
hipError_t launch_attention(int dtype, int kernel, const AttnParams &p, hipStream_t s, hipEvent_t e0 = nullptr,
                            hipEvent_t e1 = nullptr);
hipError_t launch_merge(const AttnParams &p, hipStream_t s, hipEvent_t e_end = nullptr);
// Shared-prefix decode attention: one kernel over prefix and suffix items,
// then the merge of every row's partials (events as for launch_attention).
hipError_t launch_attention_shared(const AttnParams &p, const PrefixArgs &g, hipStream_t s, hipEvent_t e0,
                                   hipEvent_t e1, hipEvent_t e_end);
// Persistent grid of the balanced schedule: resident workgroups per device
// (q4_one_score: the INT4 kernel with at most four query columns, which runs
// three waves per SIMD; the others run two).
int balanced_grid(int dtype, int head_dim, int batch, int max_blocks, bool q4_one_score = false);
// The same for wide units (bf16; units of ctw = 4 or 8 column tiles, or 2 at
// head_dim 128).
int wide_grid(int head_dim, int ctw, int batch, int max_blocks);
// The balanced shared-prefix kernel: its dynamic LDS (max_blocks: the longest
// segment in blocks) and its persistent grid for that LDS.
size_t shared_balanced_lds(int n_groups, int batch, int max_blocks);
int shared_balanced_grid(int head_dim, size_t lds);
hipError_t launch_quantize_int4(const QuantParams &p, hipStream_t s);
hipError_t launch_rope(int dtype, const RopeParams &p, hipStream_t s);
hipError_t launch_read_probe(const void *buf, size_t bytes, int workgroups, uint32_t *sink, hipStream_t s);
// kv_decode_step_noalloc's workspace: a device array of kNoallocScratchBytes
// (noalloc.hip). Its address on the current device, looked up there on the
// first call (null if the lookup fails); allocates nothing.
constexpr size_t kNoallocScratchBytes = (size_t)KV_NOALLOC_SCRATCH_BYTES;
void *noalloc_scratch();

// The attended block range of one sequence, shared by the split kernels and
// the merge kernels so that both agree on the number of splits. With q_len
// query tokens, query i attends tokens [lo_i, hi_i) with hi_i = n - q_len +
// i + 1 (causal among the new tokens) and lo_i = max(0, hi_i - window) for a
// window, else 0; [lo, hi) is their union, [all_lo, all_hi) their common part.
struct SeqRange {
    int n;              // attended length (after validation)
    int lo, hi;         // union of the query tokens' ranges [lo, hi)
    int all_lo, all_hi; // tokens every query token attends
    int blk_lo;         // first attended block
    int nblk;           // attended blocks
    int nsplit;         // splits (>= 1)
    bool bad;           // length outside [0, max_blocks * 16], or more splits than
                        // the grid and workspace were sized for (ctx above max_ctx)
};

__host__ __device__ inline SeqRange seq_range(int n, int max_blocks, int window, int split_blocks,
                                              int max_splits, int q_len) {
    SeqRange r;
    r.bad = n < 0 || (long long)n > (long long)max_blocks * kBlock;
    auto lo_of = [&](int m) {
        const int first_hi = m - q_len + 1;  // range end of query token 0
        return window > 0 ? (first_hi - window > 0 ? first_hi - window : 0) : 0;
    };
    if (!r.bad) {
        const int nb = (n + kBlock - 1) / kBlock - lo_of(n) / kBlock;
        r.bad = nb > (long)split_blocks * max_splits;
    }
    if (r.bad) n = 0;
    r.n = n;
    r.hi = n;
    r.lo = n > 0 ? lo_of(n) : 0;
    if (r.lo > r.hi) r.lo = r.hi;
    r.all_hi = n - q_len + 1;
    r.all_lo = window > 0 ? (n - window > 0 ? n - window : 0) : 0;
    r.blk_lo = r.lo / kBlock;
    int blk_hi = (n + kBlock - 1) / kBlock;
    r.nblk = blk_hi - r.blk_lo;
    if (r.nblk < 0) r.nblk = 0;
    r.nsplit = r.nblk == 0 ? 1 : (r.nblk + split_blocks - 1) / split_blocks;
    return r;
}

}  // namespace kvc
