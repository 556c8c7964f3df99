/*
 * kvoracle.c -- the oracle: a plain, slow CPU statement of what the paged
 * KV-cache hot path computes.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The product library
 * never links, calls or imports it, and it shares no code, header, table or
 * helper with the product. The only thing the two sides have in common is the
 * documented memory layout of the pool, which this file restates on its own.
 *
 * Sources (cited by page title and section; see the legend):
 *   [KVSYS]  "KV 캐시 시스템 (KV Cache System)" (data-sketchers.com wiki page on
 *            TensorRT-LLM's KV cache): sections "MQA / GQA",
 *            "제한된 어텐션 윈도우 크기", "어텐션 윈도우 크기".
 *   [VLLM]   "LLM 서빙과 KV Cache, vLLM" (velog.io/@cjkangme): sections
 *            "KV Cache", "KV Cache의 크기 계산 (naive)", "PagedAttention".
 *   [CORE]   "KV Cache는 왜 LLM 서빙의 핵심인가" (iq-universe.github.io):
 *            section "KV Cache: O(T²)를 O(T)로" (the decode-step listing),
 *            "메모리 공식과 GQA의 동기" (the M_KV formula and its GQA form),
 *            "KVQuant: 마지막 4배" (the INT4 quantizer equation).
 *   [BLEND]  "Research Paper Review : CACHE BLEND" (seokmin-hardstudy.tistory.com):
 *            section "Background" (full KV reuse with RoPE re-rotation).
 *
 * Readings of points the pages leave open (each one is also listed with the
 * other readings of the build):
 *   R1 scale is a caller-supplied factor, 1/sqrt(d_h) in every workload.
 *   R2 a decode step attends to the cache after the append, so the caller
 *      passes ctx_len = length before append + 1.
 *   R3 query head h reads kv head h / (n_h / n_kv) (contiguous groups).
 *   R4 INT4 is asymmetric: code = clamp(round((x - min) / s), 0, 15) with
 *      s = (max - min) / 15, rounding half away from zero, computed in fp32
 *      from the STORED fp16 s and min; a group whose fp16 s is 0 has all
 *      codes 0. A zero min or max of either sign is taken as +0. The clamp
 *      binds when fp16 rounding moves s or min: a subnormal fp16 s rounded
 *      down, a min rounded up, or an fp16 min of -inf (quotient +inf: 15).
 *      A quotient that is not a number (fp16 s and min both infinite) codes
 *      as 0.
 *   R5 K groups are (block, kv head, channel) over the block's 16 tokens;
 *      V groups are (token, kv head) over the d_h channels. The K of a block
 *      that is not yet full stays in bf16 in a per-sequence tail.
 *   R6 nibble packing: byte c/2 of a token row holds channel c (even c) in
 *      its low nibble and channel c+1 in its high nibble.
 *   R7 RoPE pairs are (2i, 2i+1) for style 0 and (i, i + d_h/2) for style 1;
 *      frequency theta_i = base^(-2i/d_h); angles and cos/sin in fp64, then
 *      cos/sin rounded to fp32; the rotation itself is fp32 multiply and
 *      add/subtract without fused multiply-add, then rounded to the pool type.
 *
 * Pool layout (shared by both sides as a documented format, written here
 * independently): one (block, kv head) tile is 16 token rows of d_h elements,
 * element (p, h, t, c) at ((p * n_kv + h) * 16 + t) * d_h + c.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math; x86-64
 * SSE arithmetic is IEEE single/double with round-to-nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLOCK 16

/* element types the oracle reads */
enum { O_F32 = 0, O_BF16 = 1, O_F64 = 3 };

/* ------------------------------------------------------------------ */
/* scalar conversions, written from the IEEE-754 definitions           */
/* ------------------------------------------------------------------ */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a float to the nearest bf16 (ties to even) and return its bits.
 * Done in double: snap |x| to the grid of 8 significant bits (quantum
 * 2^(e-7), floored at the subnormal quantum 2^-133), then take the top 16
 * bits of the (exactly representable) result. */
uint16_t kvo_f32_to_bf16(float x)
{
    if (isnan(x)) return 0x7fc0;
    double a = fabs((double)x);
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    /* midpoint between the largest bf16 (2 - 2^-7) * 2^127 and 2^128 */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7f80;
    int e;
    frexp(a, &e);
    int ex = e - 1;
    if (ex < -126) ex = -126;
    double q = ldexp(1.0, ex - 7);
    double r = rint(a / q) * q;
    float rf = (float)r; /* exact: r lies on the bf16 grid */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return sign | (uint16_t)(u >> 16);
}

/* Round a float to the nearest IEEE binary16 (ties to even), return bits. */
uint16_t kvo_f32_to_f16(float x)
{
    if (isnan(x)) return 0x7e00;
    double a = fabs((double)x);
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (a >= 65520.0) return sign | 0x7c00; /* midpoint of 65504 and 2^16 */
    int e;
    frexp(a, &e);
    int ex = e - 1;
    if (ex < -14) ex = -14; /* subnormal halves share the quantum 2^-24 */
    double q = ldexp(1.0, ex - 10);
    double r = rint(a / q) * q;
    if (r == 0.0) return sign;
    frexp(r, &e);
    ex = e - 1;
    if (ex < -14) return sign | (uint16_t)(r / ldexp(1.0, -24));
    uint16_t E = (uint16_t)(ex + 15);
    uint16_t M = (uint16_t)((r / ldexp(1.0, ex) - 1.0) * 1024.0);
    return sign | (uint16_t)(E << 10) | M;
}

float kvo_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int E = (h >> 10) & 0x1f;
    int M = h & 0x3ff;
    double v;
    if (E == 0)
        v = ldexp((double)M, -24);
    else if (E == 31)
        v = M ? NAN : INFINITY;
    else
        v = ldexp(1.0 + M / 1024.0, E - 15);
    return (float)(sign ? -v : v);
}

static double load_elem(int dtype, const void *base, size_t i)
{
    if (dtype == O_F32) return ((const float *)base)[i];
    if (dtype == O_BF16) return bf16_bits_to_float(((const uint16_t *)base)[i]);
    return ((const double *)base)[i];
}

static size_t row_index(int n_kv, int d, int p, int h, int t)
{
    return (((size_t)p * n_kv + h) * BLOCK + t) * (size_t)d;
}

/* ------------------------------------------------------------------ */
/* memory formula                                                      */
/* ------------------------------------------------------------------ */

/* [CORE, "메모리 공식과 GQA의 동기"]: bytes of KV cache for one request,
 * M_KV = 2 * L * T * d_cache * b, with d_cache = d_h * n_kv in the GQA form
 * (d_cache = model width for MHA, i.e. n_kv = n_h). The leading 2 counts K
 * and V; b is bytes per element (0.5 for INT4 without metadata). */
double kvo_kv_bytes(double layers, double tokens, double d_h, double n_kv, double b)
{
    return 2.0 * layers * tokens * (d_h * n_kv) * b;
}

/* ------------------------------------------------------------------ */
/* kv_append                                                           */
/* ------------------------------------------------------------------ */

/* [CORE, "KV Cache: O(T²)를 O(T)로", decode-step listing]: the new k_t, v_t
 * are appended after K_{1:t-1}, V_{1:t-1}. [VLLM, "PagedAttention"]: the
 * cache is split into fixed-size token blocks that need not be contiguous,
 * so logical token L of sequence b lives in physical block
 * tables[b][L / 16], slot L % 16.
 * k_new, v_new: [batch][n_kv][d] elements of elem_bytes bytes each.
 * seq_lens[b] is the length before the append (the slot written). */
void kvo_append(int elem_bytes, int n_kv, int d, void *K, void *V,
                const void *k_new, const void *v_new,
                const int32_t *tables, int max_blocks,
                const int32_t *seq_lens, int batch)
{
    for (int b = 0; b < batch; ++b) {
        int L = seq_lens[b];
        int p = tables[(size_t)b * max_blocks + L / BLOCK];
        int t = L % BLOCK;
        for (int h = 0; h < n_kv; ++h) {
            size_t dst = row_index(n_kv, d, p, h, t) * elem_bytes;
            size_t src = ((size_t)b * n_kv + h) * d * elem_bytes;
            memcpy((char *)K + dst, (const char *)k_new + src, (size_t)d * elem_bytes);
            memcpy((char *)V + dst, (const char *)v_new + src, (size_t)d * elem_bytes);
        }
    }
}

/* ------------------------------------------------------------------ */
/* decode attention                                                    */
/* ------------------------------------------------------------------ */

/* [CORE, "KV Cache: O(T²)를 O(T)로", decode-step listing]:
 *   attn_t = softmax(q_t . K_{1:t}^T * scale) . V_{1:t}
 * with K, V gathered token by token through the block table
 * ([VLLM, "PagedAttention"]), and query head h reading the K/V of its group
 * kv = h / (n_h / n_kv) ([KVSYS, "MQA / GQA"]; [CORE, "메모리 공식과 GQA의
 * 동기"]). window > 0 restricts attention to the last `window` tokens
 * ([KVSYS, "제한된 어텐션 윈도우 크기"]); window = 0 attends to all.
 * Everything is accumulated in fp64. ctx_lens[b] = 0 gives an output of 0.
 * q: [batch][n_h][d] (q_dtype), out: [batch][n_h][d] doubles.
 * Returns 0, or -1 if n_h is not a multiple of n_kv. */
int kvo_attention(int kv_dtype, const void *K, const void *V,
                  int q_dtype, const void *q,
                  const int32_t *tables, int max_blocks,
                  const int32_t *ctx_lens, int batch,
                  int n_h, int n_kv, int d, double scale, int window,
                  double *out)
{
    if (n_kv <= 0 || n_h % n_kv) return -1;
    int g = n_h / n_kv;
    long total = (long)batch * n_h;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < total; ++bh) {
        int b = (int)(bh / n_h), h = (int)(bh % n_h);
        int kvh = h / g;
        int n = ctx_lens[b];
        int start = (window > 0 && n > window) ? n - window : 0;
        double *o = out + ((size_t)b * n_h + h) * d;
        if (n - start <= 0) {
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            continue;
        }
        int cnt = n - start;
        double *w = (double *)malloc(sizeof(double) * (size_t)cnt);
        size_t *row = (size_t *)malloc(sizeof(size_t) * (size_t)cnt);
        size_t qoff = ((size_t)b * n_h + h) * d;
        /* scores */
        double m = -INFINITY;
        for (int j = start; j < n; ++j) {
            int p = tables[(size_t)b * max_blocks + j / BLOCK];
            size_t r = row_index(n_kv, d, p, kvh, j % BLOCK);
            double dot = 0.0;
            for (int c = 0; c < d; ++c)
                dot += load_elem(q_dtype, q, qoff + c) * load_elem(kv_dtype, K, r + c);
            double s = scale * dot;
            w[j - start] = s;
            row[j - start] = r;
            if (s > m) m = s;
        }
        /* softmax weights */
        double l = 0.0;
        for (int i = 0; i < cnt; ++i) {
            w[i] = exp(w[i] - m);
            l += w[i];
        }
        /* weighted sum of values */
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int i = 0; i < cnt; ++i) acc += w[i] * load_elem(kv_dtype, V, row[i] + c);
            o[c] = acc / l;
        }
        free(w);
        free(row);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* INT4 KVQuant                                                        */
/* ------------------------------------------------------------------ */

/* [CORE, "KVQuant: 마지막 4배"]: s = (max - min) / (2^b - 1) with b = 4, and
 * an integer code per value; readings R4 (asymmetric, fp32 spec) and R6. One
 * group of n fp32 values x[i * xs]; codes[i * cs] receives one code per byte
 * (unpacked); *s16, *m16 receive the fp16 bits of the stored scale and min. */
static void q4_group(const float *x, int n, size_t xs, uint8_t *codes, size_t cs,
                     uint16_t *s16, uint16_t *m16)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        float v = x[i * xs];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    if (mn == 0.0f) mn = 0.0f; /* a zero min or max of either sign is +0 */
    if (mx == 0.0f) mx = 0.0f;
    float s32 = (mx - mn) / 15.0f;
    *s16 = kvo_f32_to_f16(s32);
    *m16 = kvo_f32_to_f16(mn);
    float sf = kvo_f16_to_f32(*s16), mf = kvo_f16_to_f32(*m16);
    for (int i = 0; i < n; ++i) {
        int c = 0;
        if (sf != 0.0f) {
            float v = (x[i * xs] - mf) / sf;
            /* a quotient that is not a number (an infinite fp16 scale over an
             * infinite difference, when the min and the range both overflow
             * fp16) codes as 0, like a group whose scale is 0 */
            if (isnan(v) || v <= 0.0f)
                c = 0;
            else if (v >= 15.0f)
                c = 15;
            else
                c = (int)roundf(v); /* half away from zero */
        }
        codes[i * cs] = (uint8_t)c;
    }
}

/* Quantize one group given as bf16 bits; exported for the pins. codes are
 * returned unpacked, one per byte. */
void kvo_q4_group_bf16(const uint16_t *xb, int n, uint8_t *codes, uint16_t *s16, uint16_t *m16)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)n);
    for (int i = 0; i < n; ++i) x[i] = bf16_bits_to_float(xb[i]);
    q4_group(x, n, 1, codes, 1, s16, m16);
    free(x);
}

/* Same for fp32 inputs (exercises fp16 rounding of the min and scale). */
void kvo_q4_group_f32(const float *x, int n, uint8_t *codes, uint16_t *s16, uint16_t *m16)
{
    q4_group(x, n, 1, codes, 1, s16, m16);
}

static void set_nibble(uint8_t *row, int c, int code)
{
    if (c & 1)
        row[c / 2] = (uint8_t)((row[c / 2] & 0x0f) | (code << 4));
    else
        row[c / 2] = (uint8_t)((row[c / 2] & 0xf0) | code);
}

static int get_nibble(const uint8_t *row, int c)
{
    return (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 0x0f);
}

/* INT4 pool image, as separate arrays:
 *   kq  uint8  [nb][n_kv][16][d/2]   K codes
 *   ks, km fp16 [nb][n_kv][d]        K scale / min per channel
 *   vq  uint8  [nb][n_kv][16][d/2]   V codes
 *   vs, vm fp16 [nb][n_kv][16]       V scale / min per token
 *   kt  bf16   [max_seqs][n_kv][16][d]  K of each sequence's unfilled block */
typedef struct {
    uint8_t *kq;
    uint16_t *ks, *km;
    uint8_t *vq;
    uint16_t *vs, *vm;
    uint16_t *kt;
} q4pool;

/* K of one full block, per channel over its 16 tokens (R5). k holds the 16
 * token rows of d fp32 values. */
static void q4_block_k(const q4pool *P, int n_kv, int d, int p, int h, const float *k)
{
    uint8_t codes[BLOCK];
    for (int c = 0; c < d; ++c) {
        size_t pc = ((size_t)p * n_kv + h) * d + c;
        q4_group(k + c, BLOCK, (size_t)d, codes, 1, &P->ks[pc], &P->km[pc]);
        for (int t = 0; t < BLOCK; ++t)
            set_nibble(P->kq + row_index(n_kv, d, p, h, t) / 2, c, codes[t]);
    }
}

/* V of one token, per token over its d channels (R5). */
static void q4_token_v(const q4pool *P, int n_kv, int d, int p, int h, int t, const float *v)
{
    uint8_t codes[256];
    size_t pt = ((size_t)p * n_kv + h) * BLOCK + t;
    q4_group(v, d, 1, codes, 1, &P->vs[pt], &P->vm[pt]);
    for (int c = 0; c < d; ++c) set_nibble(P->vq + row_index(n_kv, d, p, h, t) / 2, c, codes[c]);
}

/* Bulk conversion of bf16 pool contents to the INT4 image. For sequence b
 * with lens[b] tokens: every full block gets K codes per channel and V codes
 * per token; the trailing partial block gets V codes per token for its
 * tokens, and its K rows are copied (bf16) to the tail of slot
 * slots[b] (slots == NULL: slot b). Nothing else is written. */
void kvo_q4_quantize_pool(const uint16_t *Kb, const uint16_t *Vb, int n_kv, int d,
                          const int32_t *tables, int max_blocks, const int32_t *lens,
                          const int32_t *slots, int batch,
                          uint8_t *kq, uint16_t *ks, uint16_t *km,
                          uint8_t *vq, uint16_t *vs, uint16_t *vm, uint16_t *kt)
{
    q4pool P = {kq, ks, km, vq, vs, vm, kt};
    float *kbuf = (float *)malloc(sizeof(float) * BLOCK * (size_t)d);
    float *vbuf = (float *)malloc(sizeof(float) * (size_t)d);
    for (int b = 0; b < batch; ++b) {
        int n = lens[b];
        int slot = slots ? slots[b] : b;
        for (int j = 0; j * BLOCK < n; ++j) {
            int p = tables[(size_t)b * max_blocks + j];
            int r = n - j * BLOCK < BLOCK ? n - j * BLOCK : BLOCK;
            for (int h = 0; h < n_kv; ++h) {
                for (int t = 0; t < r; ++t) {
                    size_t row = row_index(n_kv, d, p, h, t);
                    for (int c = 0; c < d; ++c) vbuf[c] = bf16_bits_to_float(Vb[row + c]);
                    q4_token_v(&P, n_kv, d, p, h, t, vbuf);
                }
                if (r == BLOCK) {
                    for (int t = 0; t < BLOCK; ++t)
                        for (int c = 0; c < d; ++c)
                            kbuf[t * d + c] = bf16_bits_to_float(Kb[row_index(n_kv, d, p, h, t) + c]);
                    q4_block_k(&P, n_kv, d, p, h, kbuf);
                } else {
                    for (int t = 0; t < r; ++t)
                        memcpy(kt + row_index(n_kv, d, slot, h, t), Kb + row_index(n_kv, d, p, h, t),
                               sizeof(uint16_t) * (size_t)d);
                }
            }
        }
    }
    free(kbuf);
    free(vbuf);
}

/* Append of one bf16 token per sequence to an INT4 image (R5): V is coded
 * per token at once; K goes to the tail row L % 16 of the sequence's slot;
 * when that row is the 16th, the whole tail block is coded per channel into
 * physical block tables[b][L / 16]. */
void kvo_q4_append(const uint16_t *k_new, const uint16_t *v_new, int n_kv, int d,
                   const int32_t *tables, int max_blocks, const int32_t *seq_lens,
                   const int32_t *slots, int batch,
                   uint8_t *kq, uint16_t *ks, uint16_t *km,
                   uint8_t *vq, uint16_t *vs, uint16_t *vm, uint16_t *kt)
{
    q4pool P = {kq, ks, km, vq, vs, vm, kt};
    float *kbuf = (float *)malloc(sizeof(float) * BLOCK * (size_t)d);
    float *vbuf = (float *)malloc(sizeof(float) * (size_t)d);
    for (int b = 0; b < batch; ++b) {
        int L = seq_lens[b];
        int slot = slots ? slots[b] : b;
        int p = tables[(size_t)b * max_blocks + L / BLOCK];
        int t = L % BLOCK;
        for (int h = 0; h < n_kv; ++h) {
            size_t src = ((size_t)b * n_kv + h) * d;
            for (int c = 0; c < d; ++c) vbuf[c] = bf16_bits_to_float(v_new[src + c]);
            q4_token_v(&P, n_kv, d, p, h, t, vbuf);
            memcpy(kt + row_index(n_kv, d, slot, h, t), k_new + src, sizeof(uint16_t) * (size_t)d);
            if (t == BLOCK - 1) {
                for (int tt = 0; tt < BLOCK; ++tt)
                    for (int c = 0; c < d; ++c)
                        kbuf[tt * d + c] = bf16_bits_to_float(kt[row_index(n_kv, d, slot, h, tt) + c]);
                q4_block_k(&P, n_kv, d, p, h, kbuf);
            }
        }
    }
    free(kbuf);
    free(vbuf);
}

/* Dequantize what attention reads, x = min + code * scale in fp64, into
 * fp64 pool images Kd, Vd [nb][n_kv][16][d], for the first ctx_lens[b]
 * tokens of every sequence: full blocks from the codes, the K of a partial
 * last block from the bf16 tail. Other entries of Kd, Vd are not written. */
void kvo_q4_dequant(int n_kv, int d, const int32_t *tables, int max_blocks,
                    const int32_t *ctx_lens, const int32_t *slots, int batch,
                    const uint8_t *kq, const uint16_t *ks, const uint16_t *km,
                    const uint8_t *vq, const uint16_t *vs, const uint16_t *vm,
                    const uint16_t *kt, double *Kd, double *Vd)
{
    for (int b = 0; b < batch; ++b) {
        int n = ctx_lens[b];
        int slot = slots ? slots[b] : b;
        for (int j = 0; j < n; ++j) {
            int blk = j / BLOCK, t = j % BLOCK;
            int p = tables[(size_t)b * max_blocks + blk];
            int full = (blk + 1) * BLOCK <= n;
            for (int h = 0; h < n_kv; ++h) {
                size_t row = row_index(n_kv, d, p, h, t);
                size_t pt = ((size_t)p * n_kv + h) * BLOCK + t;
                double vsc = kvo_f16_to_f32(vs[pt]), vmn = kvo_f16_to_f32(vm[pt]);
                for (int c = 0; c < d; ++c) {
                    Vd[row + c] = vmn + (double)get_nibble(vq + row / 2, c) * vsc;
                    if (full) {
                        size_t pc = ((size_t)p * n_kv + h) * d + c;
                        Kd[row + c] = (double)kvo_f16_to_f32(km[pc]) +
                                      (double)get_nibble(kq + row / 2, c) * (double)kvo_f16_to_f32(ks[pc]);
                    } else {
                        Kd[row + c] = bf16_bits_to_float(kt[row_index(n_kv, d, slot, h, t) + c]);
                    }
                }
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* RoPE re-rotation of a reused chunk                                  */
/* ------------------------------------------------------------------ */

static void pair_channels(int d, int style, int i, int *c0, int *c1)
{
    if (style == 0) {
        *c0 = 2 * i;
        *c1 = 2 * i + 1;
    } else {
        *c0 = i;
        *c1 = i + d / 2;
    }
}

/* [BLEND, "Background"]: a chunk's keys, computed as if the chunk started at
 * position 0, are moved to their real start by one extra rotation by
 * delta = real start - 0; values and queries are not touched. Reading R7 fixes
 * the pair convention, frequencies and precision. The chunk's tokens are
 * logical positions first_slot .. first_slot + num_tokens - 1 of the block
 * list chunk_blocks (physical ids in logical order); every kv head rotates.
 * dtype: O_F32 or O_BF16 pool, rotated in place. */
void kvo_rope_rerotate(int dtype, int n_kv, int d, void *K, const int32_t *chunk_blocks,
                       int first_slot, int num_tokens, int delta, double base, int style)
{
    int half = d / 2;
    float *cs = (float *)malloc(sizeof(float) * (size_t)half);
    float *sn = (float *)malloc(sizeof(float) * (size_t)half);
    for (int i = 0; i < half; ++i) {
        double theta = pow(base, -(2.0 * i) / d);
        double phi = (double)delta * theta;
        cs[i] = (float)cos(phi);
        sn[i] = (float)sin(phi);
    }
    for (int k = 0; k < num_tokens; ++k) {
        int pos = first_slot + k;
        int p = chunk_blocks[pos / BLOCK];
        for (int h = 0; h < n_kv; ++h) {
            size_t row = row_index(n_kv, d, p, h, pos % BLOCK);
            for (int i = 0; i < half; ++i) {
                int c0, c1;
                pair_channels(d, style, i, &c0, &c1);
                float x = (float)load_elem(dtype, K, row + c0);
                float y = (float)load_elem(dtype, K, row + c1);
                float xc = x * cs[i], ys = y * sn[i];
                float xs = x * sn[i], yc = y * cs[i];
                float nx = xc - ys, ny = xs + yc;
                if (dtype == O_F32) {
                    ((float *)K)[row + c0] = nx;
                    ((float *)K)[row + c1] = ny;
                } else {
                    ((uint16_t *)K)[row + c0] = kvo_f32_to_bf16(nx);
                    ((uint16_t *)K)[row + c1] = kvo_f32_to_bf16(ny);
                }
            }
        }
    }
    free(cs);
    free(sn);
}

/* The same rotation applied to one vector in fp64 throughout (for the
 * relative-position pins): x <- R(delta) x. */
void kvo_rope_rotate_f64(double *x, int d, double delta, double base, int style)
{
    for (int i = 0; i < d / 2; ++i) {
        int c0, c1;
        pair_channels(d, style, i, &c0, &c1);
        double phi = delta * pow(base, -(2.0 * i) / d);
        double a = x[c0], b = x[c1];
        x[c0] = a * cos(phi) - b * sin(phi);
        x[c1] = a * sin(phi) + b * cos(phi);
    }
}

/* ------------------------------------------------------------------ */
/* threads used by kvo_attention                                       */
/* ------------------------------------------------------------------ */

void kvo_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int kvo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* block copies: copy-on-reuse and offload / restore                   */
/* ------------------------------------------------------------------ */

/* [KVSYS, "부분 재사용"]: a partially matching block may be copied before a
 * request that reuses it writes into it; [KVSYS, "호스트 메모리로의
 * 오프로딩"]: blocks are copied to host memory and copied back to the GPU
 * before reuse. A block of a pool is its slice of every per-block region;
 * region r holds block_bytes[r] bytes per block, block p at p * block_bytes[r].
 * The packed form of one block is the concatenation of its slices in region
 * order. */

/* dst block dst[i] <- src block src[i] in every region (lists disjoint). */
void kvo_copy_blocks(int nreg, uint8_t **regions, const size_t *block_bytes, const int32_t *src,
                     const int32_t *dst, int n)
{
    for (int i = 0; i < n; ++i)
        for (int r = 0; r < nreg; ++r)
            memcpy(regions[r] + (size_t)dst[i] * block_bytes[r], regions[r] + (size_t)src[i] * block_bytes[r],
                   block_bytes[r]);
}

/* buffer <- packed blocks[0..n) ; packed block i at offset i * sum(block_bytes). */
void kvo_gather_blocks(int nreg, uint8_t **regions, const size_t *block_bytes, const int32_t *blocks, int n,
                       uint8_t *buffer)
{
    size_t per = 0;
    for (int r = 0; r < nreg; ++r) per += block_bytes[r];
    for (int i = 0; i < n; ++i) {
        size_t off = (size_t)i * per;
        for (int r = 0; r < nreg; ++r) {
            memcpy(buffer + off, regions[r] + (size_t)blocks[i] * block_bytes[r], block_bytes[r]);
            off += block_bytes[r];
        }
    }
}

/* blocks[0..n) <- packed buffer (the inverse of kvo_gather_blocks). */
void kvo_scatter_blocks(int nreg, uint8_t **regions, const size_t *block_bytes, const int32_t *blocks, int n,
                        const uint8_t *buffer)
{
    size_t per = 0;
    for (int r = 0; r < nreg; ++r) per += block_bytes[r];
    for (int i = 0; i < n; ++i) {
        size_t off = (size_t)i * per;
        for (int r = 0; r < nreg; ++r) {
            memcpy(regions[r] + (size_t)blocks[i] * block_bytes[r], buffer + off, block_bytes[r]);
            off += block_bytes[r];
        }
    }
}

/* ------------------------------------------------------------------ */
/* several query tokens per sequence (speculative verification,        */
/* chunked prefill)                                                    */
/* ------------------------------------------------------------------ */

/* The decode step of [CORE, "KV Cache: O(T²)를 O(T)로"] for q_len new tokens
 * at once: the cache already holds them, ctx_lens[b] tokens in all, and query
 * token i (i < q_len) sits at position P = ctx - q_len + i and attends to
 * tokens 0..P (causal among the new tokens), or to the last `window` of them
 * ([KVSYS, "제한된 어텐션 윈도우 크기"]). A query with no token (P < 0)
 * outputs 0. q, out: [batch][q_len][n_h][d]. Returns 0, or -1 for bad heads. */
int kvo_attention_multi(int kv_dtype, const void *K, const void *V, int q_dtype, const void *q,
                        const int32_t *tables, int max_blocks, const int32_t *ctx_lens, int batch, int q_len,
                        int n_h, int n_kv, int d, double scale, int window, double *out)
{
    if (n_kv <= 0 || n_h % n_kv || q_len < 1) return -1;
    int g = n_h / n_kv;
    long total = (long)batch * q_len * n_h;
#pragma omp parallel for schedule(dynamic, 1)
    for (long idx = 0; idx < total; ++idx) {
        int h = (int)(idx % n_h);
        int i = (int)((idx / n_h) % q_len);
        int b = (int)(idx / ((long)n_h * q_len));
        int kvh = h / g;
        int hi = ctx_lens[b] - q_len + i + 1; /* tokens 0 .. hi-1 */
        int lo = (window > 0 && hi > window) ? hi - window : 0;
        double *o = out + (size_t)idx * d;
        if (hi - lo <= 0) {
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            continue;
        }
        int cnt = hi - lo;
        double *w = (double *)malloc(sizeof(double) * (size_t)cnt);
        size_t *row = (size_t *)malloc(sizeof(size_t) * (size_t)cnt);
        size_t qoff = (size_t)idx * d;
        double m = -INFINITY;
        for (int j = lo; j < hi; ++j) {
            int p = tables[(size_t)b * max_blocks + j / BLOCK];
            size_t r = row_index(n_kv, d, p, kvh, j % BLOCK);
            double dot = 0.0;
            for (int c = 0; c < d; ++c)
                dot += load_elem(q_dtype, q, qoff + c) * load_elem(kv_dtype, K, r + c);
            w[j - lo] = scale * dot;
            row[j - lo] = r;
            if (w[j - lo] > m) m = w[j - lo];
        }
        double l = 0.0;
        for (int k = 0; k < cnt; ++k) {
            w[k] = exp(w[k] - m);
            l += w[k];
        }
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int k = 0; k < cnt; ++k) acc += w[k] * load_elem(kv_dtype, V, row[k] + c);
            o[c] = acc / l;
        }
        free(w);
        free(row);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* CacheBlend token selection                                          */
/* ------------------------------------------------------------------ */

/* [BLEND, "Methods"]: a token's KV deviation is how far its precomputed K/V
 * lie from the recomputed ones; tokens with the largest deviation are
 * recomputed. Reading: the deviation of a token is the squared L2 distance
 * over all kv heads and channels, sum (K_re - K_pre)^2 + (V_re - V_pre)^2.
 * Row i of k_re / v_re ([n_rows][n_kv][d], pool dtype) is the recomputed KV of
 * the token at position row_pos[i] of sequence row_seq[i], whose cached KV is
 * found through that sequence's block table. fp64. */
void kvo_deviation(int dtype, int n_kv, int d, const void *K, const void *V, const int32_t *tables, int max_blocks,
                   const int32_t *row_seq, const int32_t *row_pos, int n_rows, const void *k_re, const void *v_re,
                   double *dev)
{
    for (int i = 0; i < n_rows; ++i) {
        int pos = row_pos[i];
        int p = tables[(size_t)row_seq[i] * max_blocks + pos / BLOCK];
        double acc = 0.0;
        for (int h = 0; h < n_kv; ++h) {
            size_t row = row_index(n_kv, d, p, h, pos % BLOCK);
            size_t rr = ((size_t)i * n_kv + h) * d;
            for (int c = 0; c < d; ++c) {
                double dk = load_elem(dtype, k_re, rr + c) - load_elem(dtype, K, row + c);
                double dv = load_elem(dtype, v_re, rr + c) - load_elem(dtype, V, row + c);
                acc += dk * dk + dv * dv;
            }
        }
        dev[i] = acc;
    }
}

/* [BLEND, "Methods"]: keep the k rows of largest deviation; equal values go
 * to the lower row first. The chosen rows are returned in ascending order
 * (row ids; with a candidate list the caller maps them through it).
 * Plainly: sort (value, row) pairs by value descending, row ascending, keep
 * the first k, then sort those rows ascending. -0 and +0 compare equal. */
typedef struct {
    double v;
    int32_t i;
} kvo_vi;

static int kvo_vi_rank(const void *pa, const void *pb)
{
    const kvo_vi *a = (const kvo_vi *)pa, *b = (const kvo_vi *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

static int kvo_i32_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

void kvo_topk(const double *values, int n, int k, int32_t *out)
{
    if (k > n) k = n;
    if (k <= 0) return;
    kvo_vi *all = (kvo_vi *)malloc(sizeof(kvo_vi) * (size_t)n);
    for (int i = 0; i < n; ++i) {
        all[i].v = values[i];
        all[i].i = i;
    }
    qsort(all, (size_t)n, sizeof(kvo_vi), kvo_vi_rank);
    for (int r = 0; r < k; ++r) out[r] = all[r].i;
    qsort(out, (size_t)k, sizeof(int32_t), kvo_i32_asc);
    free(all);
}

/* [BLEND, "System Design"]: recompute ratio = max(15 %, the ratio at which
 * recomputing the selected tokens takes as long as loading the next layer's
 * KV). With load_time the time to load one layer's KV and token_time the time
 * to recompute one token of one layer, that ratio is load_time /
 * (num_tokens * token_time); the result is also capped at 1. */
double kvo_recompute_ratio(double load_time, double token_time, int num_tokens, double floor_ratio)
{
    double r = (num_tokens > 0 && token_time > 0.0) ? load_time / ((double)num_tokens * token_time) : 1.0;
    if (r < floor_ratio) r = floor_ratio;
    if (r > 1.0) r = 1.0;
    return r;
}

/* Tokens to recompute out of num_tokens at a ratio: the smallest whole count
 * not below ratio * num_tokens (fp64), within [0, num_tokens]. */
int kvo_recompute_count(double ratio, int num_tokens)
{
    double c = ceil(ratio * (double)num_tokens);
    if (c < 0.0) c = 0.0;
    if (c > (double)num_tokens) c = (double)num_tokens;
    return (int)c;
}

/* [KVSYS, "어텐션 윈도우 크기"]: the maximum attention window is given per
 * layer as a list, and a list shorter than the number of layers is repeated
 * as often as needed. Layer `layer` (0-based) gets the entry that the list,
 * written out again and again, holds at that place. */
int kvo_layer_window(const int *windows, int n_windows, int layer)
{
    int i, pos = 0;
    if (n_windows <= 0 || layer < 0) return -1;
    for (;;) {  /* walk the repeated list up to the layer */
        for (i = 0; i < n_windows; ++i, ++pos)
            if (pos == layer) return windows[i];
    }
}

/* [KVSYS, "제한된 어텐션 윈도우 크기"]: blocks outside a layer's limited
 * attention window are released for reuse. A sequence holding L tokens gets
 * its next query at position L, and that query attends the last `window`
 * tokens up to and including itself (a window of 0 attends every token);
 * every later query starts later still. A block is released once its last
 * token lies before the first position the next query attends: count the
 * leading blocks for which that holds. A negative length gives -1. */
void kvo_window_released(const int *lens, int batch, int window, int *out)
{
    int b;
    for (b = 0; b < batch; ++b) {
        const long long L = lens[b];
        long long first = 0, n = 0;  /* first attended position, released blocks */
        if (L < 0) {
            out[b] = -1;
            continue;
        }
        if (window > 0 && L + 1 - window > 0) first = L + 1 - window;
        while (n * 16 + 15 < first) ++n;  /* block n ends before the window */
        out[b] = (int)n;
    }
}
