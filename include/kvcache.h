/*
 * kvcache.h -- C ABI of a paged KV-cache decode library for AMD Instinct
 * MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [KVSYS] "KV 캐시 시스템 (KV Cache System)" (TensorRT-LLM KV cache, Korean
 *           wiki rendering): "MQA / GQA", "데이터 타입", "제한된 어텐션 윈도우 크기".
 *   [VLLM]  "LLM 서빙과 KV Cache, vLLM": "KV Cache", "PagedAttention".
 *   [CORE]  "KV Cache는 왜 LLM 서빙의 핵심인가": "KV Cache: O(T²)를 O(T)로"
 *           (decode-step listing), "메모리 공식과 GQA의 동기",
 *           "KVQuant: 마지막 4배" (quantizer equation).
 *   [BLEND] "Research Paper Review : CACHE BLEND": "Background" (full KV reuse
 *           and RoPE re-rotation of a precomputed chunk), "Methods" (KV
 *           deviation, selective recompute), "System Design" (recompute
 *           ratio).
 *
 * Conventions for every call:
 *   - Device pointers point to memory the caller owns (allocated with
 *     hipMalloc or any allocator on the same device). The library never
 *     allocates or frees device memory and never synchronizes.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Work is enqueued asynchronously on it; the caller synchronizes.
 *   - Calls return a kv_status synchronously. Arguments the host can check
 *     (null pointers, sizes, shapes, dtype combinations, workspace size) are
 *     checked before anything is launched; on error nothing is launched.
 *     A failed launch returns KV_ERR_HIP.
 *   - Device-resident metadata (block tables, lengths, slots) is not read by
 *     the host. Kernels bounds-check it: a block id outside [0, num_blocks)
 *     or a length outside [0, max_blocks * 16] never causes an out-of-range
 *     access; attention then writes NaN to the affected sequence's output
 *     and append/quantize/rotate skip the affected rows.
 *     kv_validate_tables checks host copies of the same arrays.
 *   - Table widths: max_blocks lies in [1, INT32_MAX / 16] (so max_blocks * 16
 *     tokens fit in 32 bits); other values are KV_ERR_INVALID_ARG.
 *   - Launch-grid limits: batch, num_kv_heads and the attention's work units
 *     per sequence (num_kv_heads * ceil(query columns / 16)) are at most
 *     65535; a call above them returns KV_ERR_UNSUPPORTED (a descriptor with
 *     more kv heads is KV_ERR_INVALID_ARG).
 */
#ifndef KVCACHE_H
#define KVCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_ABI_VERSION 1
/* Tokens per physical block [VLLM, "PagedAttention": fixed-size blocks]. */
#define KV_BLOCK_TOKENS 16
/* Largest number of prefix groups in one paged_decode_attention_shared call. */
#define KV_MAX_PREFIX_GROUPS 256

typedef int32_t kv_status;
enum {
    KV_OK = 0,
    KV_ERR_INVALID_ARG = -1, /* null pointer, bad size or shape             */
    KV_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim 96) */
    KV_ERR_WORKSPACE = -3,   /* workspace missing or too small              */
    KV_ERR_HIP = -4,         /* a HIP launch or runtime call failed         */
    KV_ERR_TABLE = -5        /* kv_validate_tables found a bad entry        */
};

/* Element type of the cache [KVSYS, "데이터 타입": the cache dtype]. */
typedef enum {
    KV_F32 = 0,  /* K, V, q, new tokens in fp32                                   */
    KV_BF16 = 1, /* K, V, q, new tokens in bf16                                   */
    KV_INT4 = 2  /* KVQuant INT4 storage; q and new tokens are bf16 [CORE, KVQuant] */
} kv_dtype;

/* Pool descriptor. A pool is num_blocks physical blocks of 16 tokens for
 * num_kv_heads kv heads of head_dim channels ([VLLM, "PagedAttention"]: a
 * block holds a fixed number of tokens and may sit anywhere in the pool;
 * [KVSYS, "MQA / GQA"]: blocks hold the state of one query group per kv head). */
typedef struct {
    int32_t num_blocks;   /* >= 1                                              */
    int32_t block_size;   /* must be 16                                        */
    int32_t num_kv_heads; /* >= 1                                              */
    int32_t head_dim;     /* 64 or 128                                         */
    int32_t max_seqs;     /* KV_INT4: rows of the bf16 K tail (>= 1); else 0   */
    int32_t dtype;        /* kv_dtype                                          */
} kv_pool_desc;

/* Opaque host-side handle: the descriptor, the bound device base pointer and
 * region offsets. It owns no device memory. */
typedef struct kv_pool *kv_pool_t;

/* Regions of a pool's device memory. Layouts (row-major, element (p,h,t,c)
 * of a K or V region at ((p * n_kv + h) * 16 + t) * head_dim + c):
 *   KV_F32 / KV_BF16 pools:
 *     K, V        elem [num_blocks][n_kv][16][head_dim]
 *   KV_INT4 pools:
 *     KQ, VQ      uint8 [num_blocks][n_kv][16][head_dim/2]; byte c/2 of a
 *                 token row holds channel c (even) in bits 0-3 and channel
 *                 c+1 in bits 4-7
 *     KS, KM      fp16 [num_blocks][n_kv][head_dim]   K scale, min per channel
 *     VS, VM      fp16 [num_blocks][n_kv][16]         V scale, min per token
 *     KTAIL       bf16 [max_seqs][n_kv][16][head_dim] K rows of each sequence's
 *                 block that is not yet full
 * Every region starts on a 256-byte boundary. */
enum {
    KV_REGION_K = 0,
    KV_REGION_V = 1,
    KV_REGION_KQ = 2,
    KV_REGION_KS = 3,
    KV_REGION_KM = 4,
    KV_REGION_VQ = 5,
    KV_REGION_VS = 6,
    KV_REGION_VM = 7,
    KV_REGION_KTAIL = 8
};

/* How the attended tiles are spread over workgroups. */
enum {
    KV_SCHED_AUTO = 0,     /* balanced for the MFMA kernel, fixed splits otherwise */
    KV_SCHED_SPLIT = 1,    /* one workgroup per (split of split_blocks blocks, kv
                              head, sequence), then a merge of the splits         */
    KV_SCHED_BALANCED = 2  /* a persistent grid; every workgroup takes an equal
                              share of all (sequence, kv head, block) tiles, then
                              a merge of the cut pairs (MFMA kernel only)          */
};

/* Options of paged_decode_attention; pass NULL for the defaults (all zero). */
typedef struct {
    int32_t split_blocks; /* KV_SCHED_SPLIT: blocks per split; 0 = chosen by the
                             library. A nonzero value selects KV_SCHED_SPLIT
                             when schedule is KV_SCHED_AUTO.                      */
    int32_t kernel;       /* 0 = chosen by the library, 1 = VALU dot products,
                             2 = MFMA tiles (bf16 pools)                          */
    int32_t window;       /* > 0: attend only the last `window` tokens of each
                             sequence [KVSYS, "제한된 어텐션 윈도우 크기"]; 0 = all  */
    int32_t schedule;     /* KV_SCHED_*                                           */
    void *events[3];      /* optional hipEvent_t handles, for timing: [0] and
                             [1] take the start and end time of the attention
                             kernel (recorded by its own dispatch), [2] the end
                             of the merge kernel (or a plain record on the
                             stream when no merge runs); NULL entries are
                             skipped                                             */
} kv_attn_opts;

/* Human-readable name of a status code (static storage). */
const char *kv_status_string(kv_status s);

/* KV_ABI_VERSION of the library that was loaded. */
int32_t kv_abi_version(void);

/* Device bytes a pool with this descriptor needs (regions laid out back to
 * back, each 256-byte aligned). 0 if the descriptor is invalid. For KV_F32 /
 * KV_BF16 the K and V regions hold exactly 2 * num_blocks * 16 * n_kv *
 * head_dim * elem_bytes bytes ([CORE, "메모리 공식과 GQA의 동기"]: M_KV =
 * 2 L T (d_h n_kv) b for one layer and T = 16 num_blocks). */
size_t kv_pool_required_bytes(const kv_pool_desc *desc);

/* Bind a descriptor to caller-owned device memory of at least
 * kv_pool_required_bytes(desc) bytes, 256-byte aligned. Launches nothing and
 * does not touch the memory. *out receives a handle to free with
 * kv_pool_destroy. */
kv_status kv_pool_create(const kv_pool_desc *desc, void *device_mem, size_t bytes, kv_pool_t *out);

/* Free the host-side handle (the device memory stays the caller's). */
kv_status kv_pool_destroy(kv_pool_t pool);

/* Byte offset (from device_mem) and size of one region; KV_ERR_INVALID_ARG if
 * the pool's dtype has no such region. */
kv_status kv_pool_region(kv_pool_t pool, int32_t region, size_t *offset, size_t *bytes);

/* Descriptor the pool was created with. */
kv_status kv_pool_get_desc(kv_pool_t pool, kv_pool_desc *desc);

/* Append one new token per sequence
 * [CORE, "KV Cache: O(T²)를 O(T)로": K_{1:t} = [K_{1:t-1}; k_t], same for V].
 *   k_new, v_new  device [batch][n_kv][head_dim], the pool's element type
 *                 (bf16 for KV_INT4 pools)
 *   block_tables  device int32 [batch][max_blocks]: physical block of each
 *                 logical 16-token block of each sequence [VLLM, PagedAttention]
 *   seq_lens      device int32 [batch]: length BEFORE the append; the token
 *                 goes to block block_tables[b][L/16], slot L % 16, and that
 *                 table entry must already name a block
 *   seq_slots     KV_INT4 only: device int32 [batch] row of the K tail that
 *                 belongs to each sequence; NULL means row b. Ignored otherwise.
 * KV_INT4 pools: V is coded per token at once; K goes to the tail row L % 16;
 * when that row is the 16th, the whole block's K is coded per channel into
 * the block (KQ/KS/KM). Two sequences must not write the same slot. */
kv_status kv_append(kv_pool_t pool, const void *k_new, const void *v_new,
                    const int32_t *block_tables, int32_t max_blocks, const int32_t *seq_lens,
                    const int32_t *seq_slots, int32_t batch, void *stream);

/* kv_append for n_new tokens per sequence at once (a chunk of a prompt, or
 * speculated tokens to verify): token t of sequence b (t < n_new) goes to
 * position seq_lens[b] + t, exactly as n_new kv_append calls in order would
 * place and code it. k_new, v_new: device [batch][n_new][n_kv][head_dim]; the
 * table entries of every position written must exist. A sequence whose
 * positions would pass max_blocks * 16 is skipped. kv_append is this call
 * with n_new = 1. */
kv_status kv_append_tokens(kv_pool_t pool, const void *k_new, const void *v_new, const int32_t *block_tables,
                           int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                           int32_t n_new, void *stream);

/* Bytes of workspace paged_decode_attention needs for these sizes and
 * options (0 is a valid answer: then workspace may be NULL). max_ctx is an
 * upper bound of every ctx_lens[b]. Returns (size_t)-1 on invalid input. */
size_t paged_decode_attention_workspace_bytes(kv_pool_t pool, int32_t batch, int32_t num_q_heads,
                                              int32_t max_ctx, const kv_attn_opts *opts);

/* Single-token decode attention over the paged cache
 * [CORE, "KV Cache: O(T²)를 O(T)로": attn_t = softmax(q_t K_{1:t}^T * scale) V_{1:t}],
 * with K, V gathered through each sequence's block table [VLLM, PagedAttention]
 * and query head h reading kv head h / (num_q_heads / n_kv) [KVSYS, MQA / GQA].
 *   q             device [batch][num_q_heads][head_dim], pool element type
 *                 (bf16 for KV_INT4)
 *   out           device fp32 [batch][num_q_heads][head_dim]
 *   num_q_heads   multiple of n_kv (num_q_heads / n_kv <= 16 for the VALU kernel)
 *   scale         softmax scale (1/sqrt(head_dim) for the usual model)
 *   ctx_lens      device int32 [batch]: tokens to attend (the cache length
 *                 after this step's append); 0 gives an output of 0
 *   seq_slots     KV_INT4: K tail row of each sequence (NULL = row b)
 *   max_ctx       host upper bound of ctx_lens (sizes the grid/workspace); a
 *                 sequence whose ctx_lens exceeds it may get a NaN output
 *   workspace     device buffer of at least ws_bytes >=
 *                 paged_decode_attention_workspace_bytes(...) bytes
 * KV_INT4 pools are dequantized on the fly: full blocks from their codes,
 * the K of a sequence's partial last block from its bf16 tail row.
 * num_q_heads / n_kv may exceed 16 only with the MFMA kernel. */
kv_status paged_decode_attention(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads,
                                 float scale, const int32_t *block_tables, int32_t max_blocks,
                                 const int32_t *ctx_lens, const int32_t *seq_slots, int32_t batch,
                                 int32_t max_ctx, void *workspace, size_t ws_bytes,
                                 const kv_attn_opts *opts, void *stream);

/* Groups of sequences whose block tables share a prefix: several sequences'
 * tables may name the same physical blocks [VLLM, "PagedAttention": blocks
 * shared between sequences; KVSYS, "부분 재사용": a request reusing the
 * blocks of a matching prefix]. Host arrays, read during the call only:
 *   group_start    [n_groups + 1], non-decreasing, group_start[n_groups] <=
 *                  batch; group i is sequences group_start[i] ..
 *                  group_start[i+1] - 1
 *   prefix_blocks  [n_groups], >= 0: the first prefix_blocks[i] entries of
 *                  every member's block table name the same physical blocks
 *                  (the kernels read them from the group's first member)
 * Sequences outside every group have no shared prefix. */
typedef struct {
    int32_t n_groups; /* 0 .. KV_MAX_PREFIX_GROUPS */
    const int32_t *group_start;
    const int32_t *prefix_blocks;
} kv_prefix_groups;

/* Bytes of workspace paged_decode_attention_shared needs ((size_t)-1 on
 * invalid input). */
size_t paged_decode_attention_shared_workspace_bytes(kv_pool_t pool, int32_t batch, int32_t num_q_heads,
                                                     int32_t max_ctx, const kv_prefix_groups *groups,
                                                     const kv_attn_opts *opts);

/* paged_decode_attention for a batch whose sequences share block-table
 * prefixes (`groups`): the same result within rounding, with each shared
 * (block, kv head) tile read once for its whole group - the group's query
 * rows are the columns of one tile product - instead of once per member.
 * A member attends its whole shared prefix and then its own blocks; a member
 * whose ctx_lens is below its prefix (prefix_blocks * 16 tokens) gets NaN.
 * bf16 pools only (MFMA kernel; opts->kernel 0 or 2), no window
 * (opts->window 0). Schedules: KV_SCHED_BALANCED (the default: every prefix
 * tile of every group and every own tile of every sequence is numbered, and
 * each workgroup of a persistent grid takes an equal contiguous share; up to
 * 8192 sequences) or KV_SCHED_SPLIT (work items of opts->split_blocks prefix
 * or own blocks, 0 = chosen by the library; a nonzero split_blocks selects it
 * under KV_SCHED_AUTO). Other arguments as for paged_decode_attention.
 * Errors: KV_ERR_UNSUPPORTED for other pools or options, KV_ERR_INVALID_ARG
 * for malformed groups. */
kv_status paged_decode_attention_shared(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads,
                                        float scale, const int32_t *block_tables, int32_t max_blocks,
                                        const int32_t *ctx_lens, int32_t batch, int32_t max_ctx,
                                        const kv_prefix_groups *groups, void *workspace, size_t ws_bytes,
                                        const kv_attn_opts *opts, void *stream);

/* Bytes of workspace paged_multi_token_attention needs ((size_t)-1 on invalid
 * input). */
size_t paged_multi_token_attention_workspace_bytes(kv_pool_t pool, int32_t batch, int32_t num_q_heads,
                                                   int32_t q_len, int32_t max_ctx, const kv_attn_opts *opts);

/* Attention of q_len new tokens per sequence over the paged cache, causal
 * among themselves (verifying speculated tokens, or a chunk of a prompt):
 * the cache already holds the new tokens (appended like any other), ctx_lens[b]
 * tokens in all, and query token i < q_len sits at position P = ctx_lens[b] -
 * q_len + i and attends tokens 0..P [CORE, "KV Cache: O(T²)를 O(T)로": each
 * token attends to the cache up to itself], or the last `window` of them
 * ([KVSYS, "제한된 어텐션 윈도우 크기"]). A query token with no token to
 * attend to (P < 0) outputs 0.
 *   q    device [batch][q_len][num_q_heads][head_dim] (bf16)
 *   out  device fp32 [batch][q_len][num_q_heads][head_dim]
 * The other arguments are those of paged_decode_attention, which is this call
 * with q_len = 1. MFMA kernels only (bf16 pools, INT4 pools with head_dim
 * 128); each kv head's group * q_len query rows are processed in tiles of 16. */
kv_status paged_multi_token_attention(kv_pool_t pool, const void *q, float *out, int32_t num_q_heads, int32_t q_len,
                                      float scale, const int32_t *block_tables, int32_t max_blocks,
                                      const int32_t *ctx_lens, const int32_t *seq_slots, int32_t batch,
                                      int32_t max_ctx, void *workspace, size_t ws_bytes, const kv_attn_opts *opts,
                                      void *stream);

/* One whole decode step [CORE, "KV Cache: O(T²)를 O(T)로", decode-step
 * listing: append the new k, v, then attend over the cache including them]:
 * the same result as kv_append_tokens(k_new, v_new, seq_lens, n_new = q_len)
 * followed by paged_multi_token_attention over seq_lens[b] + q_len tokens
 * (q_len = 1: paged_decode_attention), bit for bit, in pool contents and
 * output.
 *   k_new, v_new  device [batch][q_len][num_kv_heads][head_dim], pool dtype
 *                 (bf16 for INT4 pools), 16-byte aligned
 *   seq_lens      device int32 [batch], lengths BEFORE the append
 *   max_ctx       largest seq_lens[b] + q_len; the workspace is
 *                 paged_multi_token_attention_workspace_bytes(pool, batch,
 *                 num_q_heads, q_len, max_ctx, opts)
 * The other arguments are those of paged_multi_token_attention. With the
 * MFMA kernel the append is fused into the attention kernel (one kernel
 * fewer per step): on bf16 pools tiles take the new rows from k_new / v_new
 * and write them into the pool; on INT4 pools with q_len 1 the workgroup
 * that reads a sequence's last block codes the new token into the pool
 * first when each kv head has at most 16 query columns. Other pools, INT4
 * with q_len > 1 and INT4 with more than 16 query heads per kv head launch
 * the append kernel first.
 * seq_lens must not change between the two (same stream order). A sequence
 * whose length is out of range or above max_ctx gets NaN and may be left
 * unappended. */
kv_status kv_decode_step(kv_pool_t pool, const void *k_new, const void *v_new, const void *q, float *out,
                         int32_t num_q_heads, int32_t q_len, float scale, const int32_t *block_tables,
                         int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                         int32_t max_ctx, void *workspace, size_t ws_bytes, const kv_attn_opts *opts, void *stream);

/* Bytes of the device array kv_decode_step_noalloc uses as its workspace
 * (64 MiB; every device the library runs on holds one until the process
 * ends). It covers the one-token decode step on bf16 and INT4 pools at any
 * batch the balanced schedule takes (its workspace depends on the device's
 * persistent grid, 16 rows per slot and the batch's prefix sums: at most
 * about 51 MB on a 256-CU device). */
#define KV_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kv_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same call without workspace arguments. Its workspace is a file-scope
 * device array of KV_NOALLOC_SCRATCH_BYTES bytes, looked up on the calling
 * thread's current device on the first call there (the stream's device must
 * be current). Calls no hipMalloc, hipFree or other allocating routine.
 * Returns KV_ERR_WORKSPACE when the call's workspace
 * (paged_multi_token_attention_workspace_bytes) exceeds the array, and
 * KV_ERR_HIP if the array's address cannot be found. Every call on one device
 * shares that device's array and nothing in it has to start at zero (each
 * call writes what it reads), but calls that overlap on one device (two
 * streams, or two threads) race on it: order them. Outputs and pool contents
 * are those of kv_decode_step, bit for bit. */
kv_status kv_decode_step_noalloc(kv_pool_t pool, const void *k_new, const void *v_new, const void *q, float *out,
                                 int32_t num_q_heads, int32_t q_len, float scale, const int32_t *block_tables,
                                 int32_t max_blocks, const int32_t *seq_lens, const int32_t *seq_slots, int32_t batch,
                                 int32_t max_ctx, const kv_attn_opts *opts, void *stream);

/* Bulk KVQuant INT4 coding of bf16 pool contents [CORE, "KVQuant: 마지막 4배"]:
 * code = clamp(round((x - min) / s), 0, 15) with s = (max - min) / 15, s and min
 * stored in fp16 and the codes computed from the stored values (fp32
 * arithmetic, rounding half away from zero; a group whose fp16 s is 0 gets
 * codes 0). K groups: (block, kv head, channel) over the block's 16 tokens;
 * V groups: (token, kv head) over head_dim channels.
 * For each sequence b with lens[b] tokens in src (through block_tables, which
 * address both pools): full blocks get K and V codes; a partial last block
 * gets V codes for its tokens and its K rows copied to the K tail row
 * seq_slots[b] (NULL = b). dst: KV_INT4 pool; src: KV_BF16 pool with the same
 * num_blocks, num_kv_heads and head_dim. Nothing else in dst is written. */
kv_status kv_quantize_int4(kv_pool_t dst, kv_pool_t src, const int32_t *block_tables,
                           int32_t max_blocks, const int32_t *lens, const int32_t *seq_slots,
                           int32_t batch, void *stream);

/* RoPE re-rotation of a reused chunk's keys in place [BLEND, "Background":
 * keys precomputed as if the chunk started at position 0 are moved to the
 * real start by one extra rotation by delta = real start - 0].
 *   chunk_blocks  device int32: physical ids of the chunk's blocks in
 *                 logical order
 *   first_slot    logical position of the chunk's first token within that
 *                 block list (0 when the chunk starts a block)
 *   num_tokens    tokens in the chunk
 *   delta         rotation offset in positions (may be negative)
 *   base          RoPE base (10000 for LLaMA); pair i turns by delta * base^(-2i/head_dim)
 *   style         0: pairs (2i, 2i+1); 1: pairs (i, i + head_dim/2)
 * Angles and cos/sin are computed on the host in fp64 and rounded to fp32;
 * each pair (x, y) becomes (x c - y s, x s + y c) in fp32 without fused
 * multiply-add, rounded to the pool type. Every kv head is rotated; V is not
 * touched. KV_F32 and KV_BF16 pools only (rotate before coding to INT4). */
kv_status rope_rerotate(kv_pool_t pool, const int32_t *chunk_blocks, int32_t first_slot,
                        int32_t num_tokens, int32_t delta, float base, int32_t style, void *stream);

/* Bytes of one block in packed form: its slice of every per-block region in
 * region order (K, V for fp32/bf16 pools; KQ, KS, KM, VQ, VS, VM for INT4).
 * The INT4 K tail belongs to a sequence, not to a block, and is not part of
 * a packed block. 0 for a NULL pool. */
size_t kv_block_bytes(kv_pool_t pool);

/* Window of a layer [KVSYS, "어텐션 윈도우 크기": the maximum attention window
 * is given per layer as a list, repeated when it is shorter than the number
 * of layers]: *window_out = windows[layer % n_windows], to be passed as
 * kv_attn_opts.window for that layer.
 *   windows     host int32 [n_windows], each > 0 (tokens)
 *   layer       0-based layer index
 * Host only; touches no device. KV_ERR_INVALID_ARG for a NULL pointer,
 * n_windows <= 0, layer < 0 or a chosen entry <= 0. */
kv_status kv_layer_window(const int32_t *windows, int32_t n_windows, int32_t layer, int32_t *window_out);

/* Blocks that have left a limited attention window [KVSYS, "제한된 어텐션
 * 윈도우 크기": blocks outside the window are released for reuse].
 * released[b] = the number of leading table entries of sequence b that no
 * later query can attend. A later query sits at position >= seq_lens[b] and
 * attends the last `window` tokens up to and including itself, so every
 * token before seq_lens[b] + 1 - window is dead, and the count is
 * floor(max(0, seq_lens[b] + 1 - window) / 16). window 0 (all tokens)
 * releases nothing; a negative length gives -1. The caller frees those
 * blocks; the pool and the tables are not touched.
 *   seq_lens    device int32 [batch]: tokens now held by each sequence
 *   released    device int32 [batch], written
 * Asynchronous on `stream`. KV_ERR_INVALID_ARG for batch < 0, window < 0,
 * or a NULL array when batch > 0. */
kv_status kv_window_released_blocks(const int32_t *seq_lens, int32_t batch, int32_t window, int32_t *released,
                                    void *stream);

/* Copy whole blocks inside a pool [KVSYS, "부분 재사용": a partially matching
 * block is copied before a request that reuses it writes into it]:
 * block dst_blocks[i] <- block src_blocks[i] in every per-block region, i < n.
 *   src_blocks, dst_blocks  device int32 [n]; the two lists must be disjoint
 *                           and dst ids distinct (else the result depends on
 *                           the order of writes). Out-of-range ids skip the
 *                           pair. */
kv_status kv_copy_blocks(kv_pool_t pool, const int32_t *src_blocks, const int32_t *dst_blocks, int32_t n,
                         void *stream);

/* Offload [KVSYS, "호스트 메모리로의 오프로딩": blocks are copied to host
 * memory and copied back before reuse]: pack blocks[0..n) into `buffer`,
 * block i at byte i * kv_block_bytes(pool). `buffer` is device memory or
 * pinned host memory mapped for the device (hipHostMalloc), of at least
 * n * kv_block_bytes(pool) bytes (`bytes`), 16-byte aligned. Out-of-range ids
 * leave their slot of the buffer unwritten. */
kv_status kv_gather_blocks(kv_pool_t pool, const int32_t *blocks, int32_t n, void *buffer, size_t bytes,
                           void *stream);

/* Restore: unpack `buffer` (the layout kv_gather_blocks writes) into
 * blocks[0..n); ids must be distinct. */
kv_status kv_scatter_blocks(kv_pool_t pool, const int32_t *blocks, int32_t n, const void *buffer, size_t bytes,
                            void *stream);

/* KV deviation [BLEND, "Methods"]: for row i, the squared L2 distance between
 * the recomputed K/V of one token and the cached K/V of the same token,
 * summed over every kv head and channel of both K and V:
 *   deviation[i] = sum_h,c (k_re[i][h][c] - K[tok][h][c])^2
 *                        + (v_re[i][h][c] - V[tok][h][c])^2,
 * where tok is position row_pos[i] of sequence row_seq[i], found through
 * block_tables[row_seq[i]] (the distance ranks tokens the way the L2 norm
 * does). Computed in fp64 from exact differences; only the summation order
 * differs from a sequential sum.
 *   block_tables  device int32 [batch][max_blocks]
 *   row_seq, row_pos  device int32 [n_rows]
 *   k_re, v_re    device [n_rows][num_kv_heads][head_dim] of the pool dtype,
 *                 16-byte aligned
 *   deviation     device fp64 [n_rows]
 * A row whose sequence, position or block id is out of range gets -inf (it is
 * never selected ahead of a valid row). KV_F32 and KV_BF16 pools only. */
kv_status kv_token_deviation(kv_pool_t pool, const int32_t *block_tables, int32_t max_blocks, int32_t batch,
                             const int32_t *row_seq, const int32_t *row_pos, int32_t n_rows, const void *k_re,
                             const void *v_re, double *deviation, void *stream);

/* Selective recompute [BLEND, "Methods"]: the tokens of largest deviation are
 * recomputed. For each segment s, values[seg_offsets[s] .. seg_offsets[s+1])
 * (device fp64), write the indices (relative to the segment) of its
 * min(seg_k[s], length) largest values, in ascending order, to
 * selected[seg_offsets[s] ..]; equal values are taken lowest index first.
 * Values must not be NaN (a NaN's rank is unspecified); -0 equals +0.
 *   seg_offsets  device int32 [n_seg + 1], non-decreasing (a segment with a
 *                negative length is skipped); seg_k device int32 [n_seg]
 *   selected     device int32, at least seg_offsets[n_seg] entries; entries
 *                past a segment's count are left unwritten. */
kv_status kv_topk_select(const double *values, const int32_t *seg_offsets, const int32_t *seg_k, int32_t n_seg,
                         int32_t *selected, void *stream);

/* [BLEND, "System Design"]: recompute ratio = max(floor_ratio, the ratio at
 * which recomputing the chosen tokens of a layer takes as long as loading the
 * next layer's KV), capped at 1. load_time: time to load one layer's KV;
 * token_time: time to recompute one token of one layer (same unit). The pages
 * put the floor at 15 % (floor_ratio 0.15). Host only. */
double kv_recompute_ratio(double load_time, double token_time, int32_t num_tokens, double floor_ratio);

/* Tokens to recompute: ceil(ratio * num_tokens) in fp64, within
 * [0, num_tokens]. Host only. */
int32_t kv_recompute_count(double ratio, int32_t num_tokens);

/* Host-side check of HOST copies of the metadata a decode step would use:
 * every block the first lens[b] tokens (after the append when `appending`
 * is nonzero, i.e. lens[b] + 1 tokens) need is in [0, num_blocks), lens are
 * non-negative and fit max_blocks * 16, and no two sequences append into the
 * same (block, slot). KV_OK, or KV_ERR_TABLE with *bad_row set to the first
 * offending sequence (bad_row may be NULL). */
kv_status kv_validate_tables(const kv_pool_desc *desc, const int32_t *block_tables, int32_t max_blocks,
                             const int32_t *lens, int32_t batch, int32_t appending, int32_t *bad_row);

/* Measurement: the device's read ceiling for the kernels above. Reads the
 * `bytes` bytes at `buf` (device memory, 16-byte aligned, `bytes` a multiple
 * of 4096) once, in the pattern the attention kernels read a (block, kv head)
 * tile of a bf16 pool at head_dim 128: one wave per 4 KiB piece, four 16-byte
 * non-temporal loads per lane, two pieces in flight, over `workgroups`
 * workgroups of four waves (1 .. 65535; 0 = 2048). Nothing is written except
 * that the XOR of all words read is stored to *sink (device uint32) when it
 * equals 0x9e3779b9. Bytes read / the call's duration is the ceiling. */
kv_status kv_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVCACHE_H */
