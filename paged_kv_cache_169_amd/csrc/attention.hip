// attention.hip -- split-context paged decode attention for gfx950.
//
// Computes, for every sequence b and query head h,
//   out[b][h] = softmax(q[b][h] . K_b^T * scale) . V_b
// over the first ctx_lens[b] tokens (or the last `window` of them)
// ["KV Cache는 왜 LLM 서빙의 핵심인가", section "KV Cache: O(T²)를 O(T)로",
// decode-step listing; "KV 캐시 시스템 (KV Cache System)", section
// "제한된 어텐션 윈도우 크기" for the window], where K_b, V_b are gathered
// block by block through the sequence's block table ["LLM 서빙과 KV Cache,
// vLLM", section "PagedAttention"] and query head h reads kv head
// h / (n_h / n_kv) ["KV 캐시 시스템", section "MQA / GQA"].
//
// Decomposition: one wave64 workgroup per (context split, kv head, sequence).
// It streams its split's (block, kv head) tiles once and serves all g = n_h /
// n_kv query heads of the group from each tile, keeping an online softmax
// (running max m and sum l, in log2 units: scores are pre-multiplied by
// scale * log2 e so exp becomes the hardware exp2). A sequence with one split
// writes its output directly; otherwise each split writes (o, m, l) to the
// workspace and attn_merge_kernel combines them:
//   M = max_s m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
//
// Two inner kernels:
//  * attn_valu_kernel (fp32, bf16, INT4): VALU dot products. Lane l takes
//    token l/4 of a block and a quarter of its channels for q.K (two xor
//    shuffles finish each dot product); for p.V lane l owns head_dim/64
//    channels and walks the block's tokens, the weights broadcast through LDS.
//  * attn_mfma_bf16_kernel (bf16): the block's scores for the whole query
//    group are one 16x16 MFMA tile, S^T[token][head] = K_tile . Q^T (heads
//    padded to 16), and the value update is O^T[channel][head] +=
//    V_tile^T . P^T with 16x16x16 MFMAs. P is split into bf16 hi + lo parts
//    so the weights keep ~16 bits (a single bf16 would cost up to 2^-9
//    relative error per weight). The QK output layout (lane = head + 16 *
//    token-quad) is exactly the B-operand layout the PV product needs, so P
//    never leaves registers.
#include "device.h"
#include "internal.h"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum { KIND_F32 = 0, KIND_BF16 = 1, KIND_INT4 = 2 };

struct SplitWork {
    SeqRange r;
    int j0, j1;  // blocks [j0, j1) of this split
};

__device__ __forceinline__ bool split_work(const AttnParams &p, int b, int split, SplitWork &w) {
    w.r = seq_range(p.ctx_lens[b], p.max_blocks, p.window, p.split_blocks, p.max_splits);
    if (split >= w.r.nsplit) return false;
    w.j0 = w.r.blk_lo + split * p.split_blocks;
    w.j1 = min(w.r.blk_lo + w.r.nblk, w.j0 + p.split_blocks);
    return true;
}

// Final store of one lane's run of `n` consecutive channels of one head.
__device__ __forceinline__ void store_result(const AttnParams &p, int b, int head, int split, int nsplit,
                                             int ch0, const float *o, int n, float m, float l, bool bad,
                                             bool write_ml) {
    const float nan = __uint_as_float(0x7fc00000u);
    if (nsplit == 1) {
        float *dst = p.out + ((size_t)b * p.n_h + head) * p.head_dim + ch0;
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        for (int c = 0; c < n; ++c) dst[c] = bad ? nan : o[c] * inv;
    } else {
        const size_t base = ((size_t)b * p.n_h + head) * p.max_splits + split;
        float *dst = p.ws_o + base * p.head_dim + ch0;
        for (int c = 0; c < n; ++c) dst[c] = bad ? nan : o[c];
        if (write_ml) {
            p.ws_ml[base * 2] = m;
            p.ws_ml[base * 2 + 1] = bad ? nan : l;
        }
    }
}

// ---------------------------------------------------------------------------
// VALU kernel
// ---------------------------------------------------------------------------

template <int KIND, int D>
__device__ __forceinline__ void load_q_quarter(const AttnParams &p, int b, int head, int qt, float *qf) {
    constexpr int CQ = D / 4;
    if (KIND == KIND_F32) {
        const float4 *src = reinterpret_cast<const float4 *>(
            reinterpret_cast<const float *>(p.q) + ((size_t)b * p.n_h + head) * D + qt * CQ);
#pragma unroll
        for (int i = 0; i < CQ / 4; ++i) {
            const float4 v = src[i];
            qf[4 * i] = v.x;
            qf[4 * i + 1] = v.y;
            qf[4 * i + 2] = v.z;
            qf[4 * i + 3] = v.w;
        }
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.q) + ((size_t)b * p.n_h + head) * D + qt * CQ);
#pragma unroll
        for (int i = 0; i < CQ / 8; ++i) {
            const uint4 v = src[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qf[8 * i + 2 * k] = bf16_lo(w[k]);
                qf[8 * i + 2 * k + 1] = bf16_hi(w[k]);
            }
        }
    }
}

// Key row of token t, channels [qt*CQ, qt*CQ + CQ), widened to fp32.
template <int KIND, int D>
__device__ __forceinline__ void load_key_quarter(const AttnParams &p, int pid, int kvh, int t, int qt, bool full,
                                                 int slot, float *kf) {
    constexpr int CQ = D / 4;
    const size_t tile = (size_t)pid * p.n_kv + kvh;
    if (KIND == KIND_F32) {
        const float4 *src =
            reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p.pool.k) + (tile * kBlock + t) * D + qt * CQ);
#pragma unroll
        for (int i = 0; i < CQ / 4; ++i) {
            const float4 v = src[i];
            kf[4 * i] = v.x;
            kf[4 * i + 1] = v.y;
            kf[4 * i + 2] = v.z;
            kf[4 * i + 3] = v.w;
        }
    } else if (KIND == KIND_BF16 || !full) {
        // bf16 pool, or the bf16 tail row of an INT4 sequence's partial block
        const uint16_t *row = KIND == KIND_BF16
                                  ? reinterpret_cast<const uint16_t *>(p.pool.k) + (tile * kBlock + t) * D
                                  : p.pool.ktail + (((size_t)slot * p.n_kv + kvh) * kBlock + t) * D;
        const uint4 *src = reinterpret_cast<const uint4 *>(row + qt * CQ);
#pragma unroll
        for (int i = 0; i < CQ / 8; ++i) {
            const uint4 v = src[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                kf[8 * i + 2 * k] = bf16_lo(w[k]);
                kf[8 * i + 2 * k + 1] = bf16_hi(w[k]);
            }
        }
    } else {
        // INT4 full block: x = min_c + code * scale_c, per channel
        const uint8_t *codes = p.pool.kq + (tile * kBlock + t) * (D / 2) + qt * (CQ / 2);
        const uint16_t *sc = p.pool.ks + tile * D + qt * CQ;
        const uint16_t *mn = p.pool.km + tile * D + qt * CQ;
#pragma unroll
        for (int i = 0; i < CQ / 8; ++i) {
            const uint32_t cw = reinterpret_cast<const uint32_t *>(codes)[i];  // 8 codes
            const uint4 sv = reinterpret_cast<const uint4 *>(sc)[i];
            const uint4 mv = reinterpret_cast<const uint4 *>(mn)[i];
            const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w}, m4[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float code = (float)((cw >> (4 * k)) & 15u);
                const uint16_t sb = (uint16_t)(s4[k / 2] >> (16 * (k & 1)));
                const uint16_t mb = (uint16_t)(m4[k / 2] >> (16 * (k & 1)));
                kf[8 * i + k] = f16_bits_to_f(mb) + code * f16_bits_to_f(sb);
            }
        }
    }
}

// This lane's CV = D/64 value channels of token t.
template <int KIND, int D>
__device__ __forceinline__ void load_value(const AttnParams &p, int pid, int kvh, int t, int lane, float *vv) {
    constexpr int CV = D / 64;
    const size_t tile = (size_t)pid * p.n_kv + kvh;
    const size_t row = tile * kBlock + t;
    if (KIND == KIND_F32) {
        const float *src = reinterpret_cast<const float *>(p.pool.v) + row * D + lane * CV;
#pragma unroll
        for (int c = 0; c < CV; ++c) vv[c] = src[c];
    } else if (KIND == KIND_BF16) {
        if (CV == 2) {
            const uint32_t w = reinterpret_cast<const uint32_t *>(p.pool.v)[row * (D / 2) + lane];
            vv[0] = bf16_lo(w);
            vv[CV - 1] = bf16_hi(w);
        } else {
            vv[0] = bf16_to_f(reinterpret_cast<const uint16_t *>(p.pool.v)[row * D + lane]);
        }
    } else {
        const float s = f16_bits_to_f(p.pool.vs[row]), m = f16_bits_to_f(p.pool.vm[row]);
        const uint8_t *codes = p.pool.vq + row * (D / 2);
        if (CV == 2) {
            const uint32_t byte = codes[lane];
            vv[0] = m + (float)(byte & 15u) * s;
            vv[CV - 1] = m + (float)(byte >> 4) * s;
        } else {
            const uint32_t byte = codes[lane >> 1];
            vv[0] = m + (float)((byte >> (4 * (lane & 1))) & 15u) * s;
        }
    }
}

template <int KIND, int D, int GMAX>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnParams p) {
    constexpr int CQ = D / 4;   // key channels per lane
    constexpr int CV = D / 64;  // value channels per lane
    __shared__ float pl[GMAX][kBlock];
    const int lane = threadIdx.x, t = lane >> 2, qt = lane & 3;
    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    SplitWork w;
    if (!split_work(p, b, split, w)) return;
    const int g = p.group;
    int slot = 0;
    bool bad = w.r.bad;
    if (KIND == KIND_INT4) {
        slot = p.seq_slots ? p.seq_slots[b] : b;
        if (slot < 0 || slot >= p.max_seqs) {
            bad = true;
            slot = 0;
        }
    }

    float qf[GMAX][CQ];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h < g) {
            load_q_quarter<KIND, D>(p, b, kvh * g + h, qt, qf[h]);
        } else {
#pragma unroll
            for (int c = 0; c < CQ; ++c) qf[h][c] = 0.0f;
        }
    }
    float m_run[GMAX], l_run[GMAX], acc[GMAX][CV];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < CV; ++c) acc[h][c] = 0.0f;
    }

    for (int j = w.j0; j < w.j1; ++j) {
        int pid = p.tables[(size_t)b * p.max_blocks + j];
        if (pid < 0 || pid >= p.num_blocks) {
            bad = true;
            pid = 0;
        }
        const int tok0 = j * kBlock;
        const int tlo = max(w.r.lo - tok0, 0), thi = min(w.r.hi - tok0, kBlock);
        const bool full = tok0 + kBlock <= w.r.n;
        float kf[CQ];
        load_key_quarter<KIND, D>(p, pid, kvh, t, qt, full, slot, kf);
        const bool valid = t >= tlo && t < thi;
        float s[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            float a = 0.0f;
#pragma unroll
            for (int c = 0; c < CQ; ++c) a = fmaf(qf[h][c], kf[c], a);
            a += __shfl_xor(a, 1);
            a += __shfl_xor(a, 2);
            s[h] = valid ? a * p.scale_log2 : -INFINITY;
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            float mb = s[h];
            mb = fmaxf(mb, __shfl_xor(mb, 4));
            mb = fmaxf(mb, __shfl_xor(mb, 8));
            mb = fmaxf(mb, __shfl_xor(mb, 16));
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float mn = fmaxf(m_run[h], mb);
            const float alpha = exp2f(m_run[h] - mn);
            const float pe = exp2f(s[h] - mn);
            l_run[h] = l_run[h] * alpha + pe;
#pragma unroll
            for (int c = 0; c < CV; ++c) acc[h][c] *= alpha;
            m_run[h] = mn;
            if (qt == 0) pl[h][t] = pe;
        }
        __syncthreads();
        for (int tt = tlo; tt < thi; ++tt) {
            float vv[CV];
            load_value<KIND, D>(p, pid, kvh, tt, lane, vv);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                const float pw = pl[h][tt];
#pragma unroll
                for (int c = 0; c < CV; ++c) acc[h][c] = fmaf(pw, vv[c], acc[h][c]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        float l = l_run[h];
        l += __shfl_xor(l, 4);
        l += __shfl_xor(l, 8);
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (h < g) store_result(p, b, kvh * g + h, split, w.r.nsplit, lane * CV, acc[h], CV, m_run[h], l, bad,
                                lane == 0);
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16 pools)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack_bf16x2(uint32_t lo, uint32_t hi) { return (lo & 0xffffu) | (hi << 16); }

template <int D>
__global__ __launch_bounds__(64) void attn_mfma_bf16_kernel(AttnParams p) {
    constexpr int KS = D / 32;  // k-steps of S^T = K . Q^T (16x16x32)
    constexpr int MS = D / 16;  // channel tiles of O^T (16x16x16)
    constexpr int VC = D / 16;  // value channels per lane per token row
    const int lane = threadIdx.x, n16 = lane & 15, G = lane >> 4;
    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    SplitWork w;
    if (!split_work(p, b, split, w)) return;
    const int g = p.group;
    bool bad = w.r.bad;

    // Q^T as B operand: lane (G, n16) holds channels s*32 + 8G .. +8 of head n16.
    bf16x8_t qB[KS];
    const int head = kvh * g + n16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n16 < g)
            v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.q) +
                                                 ((size_t)b * p.n_h + head) * D + s * 32 + 8 * G);
        qB[s] = __builtin_bit_cast(bf16x8_t, v);
    }
    f32x4_t o[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) o[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    const uint16_t *Kb = reinterpret_cast<const uint16_t *>(p.pool.k);
    const uint16_t *Vb = reinterpret_cast<const uint16_t *>(p.pool.v);
    for (int j = w.j0; j < w.j1; ++j) {
        int pid = p.tables[(size_t)b * p.max_blocks + j];
        if (pid < 0 || pid >= p.num_blocks) {
            bad = true;
            pid = 0;
        }
        const size_t tile = ((size_t)pid * p.n_kv + kvh) * kBlock * D;
        // K as A operand: lane (G, n16) holds token n16, channels s*32 + 8G .. +8
        bf16x8_t kA[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kA[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Kb + tile + n16 * D + s * 32 + 8 * G));
        // V rows 4G + i, channels n16*VC .. +VC
        uint32_t vr[4][VC / 2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t *src = Vb + tile + (4 * G + i) * D + n16 * VC;
            if (VC == 8) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src);
                vr[i][0] = v.x;
                vr[i][1] = v.y;
                vr[i][VC / 2 - 2] = v.z;
                vr[i][VC / 2 - 1] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
                vr[i][0] = v.x;
                vr[i][VC / 2 - 1] = v.y;
            }
        }
        f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[s], qB[s], sc, 0, 0, 0);

        const int tok0 = j * kBlock;
        const int tlo = max(w.r.lo - tok0, 0), thi = min(w.r.hi - tok0, kBlock);
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tt = 4 * G + r;
            sv[r] = (tt >= tlo && tt < thi) ? sc[r] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - mn);
        m_run = mn;
        float pr[4];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = exp2f(sv[r] - mn);
            psum += pr[r];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int m = 0; m < MS; ++m) o[m] *= alpha;
        // P^T as B operand (hi and lo bf16 parts)
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hi[r] = f_to_bf16(pr[r]);
            lo[r] = f_to_bf16(pr[r] - bf16_to_f((uint16_t)hi[r]));
        }
        const bf16x4_t pHi = __builtin_bit_cast(bf16x4_t, make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
        const bf16x4_t pLo = __builtin_bit_cast(bf16x4_t, make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])));
        // rows of slots outside [tlo, thi) may hold anything (even NaN): zero them
        if (tlo > 0 || thi < kBlock) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 4 * G + i;
                if (tt < tlo || tt >= thi) {
#pragma unroll
                    for (int k = 0; k < VC / 2; ++k) vr[i][k] = 0u;
                }
            }
        }
        // V^T as A operand for channel tile m: lane (G, n16) holds channel
        // n16*VC + m of tokens 4G .. 4G+3.
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int wi = m >> 1, sh = (m & 1) * 16;
            const uint32_t e0 = vr[0][wi] >> sh, e1 = vr[1][wi] >> sh, e2 = vr[2][wi] >> sh, e3 = vr[3][wi] >> sh;
            const bf16x4_t a = __builtin_bit_cast(bf16x4_t, make_uint2(pack_bf16x2(e0, e1), pack_bf16x2(e2, e3)));
            o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pHi, o[m], 0, 0, 0);
            o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pLo, o[m], 0, 0, 0);
        }
    }

    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (n16 < g) {
        // lane (G, n16) holds channel (4G + r) * VC + m in o[m][r]: a contiguous
        // run of 4 * VC channels starting at 4G * VC
        float res[4 * VC];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int m = 0; m < MS; ++m) res[r * VC + m] = o[m][r];
        store_result(p, b, head, split, w.r.nsplit, 4 * G * VC, res, 4 * VC, m_run, l, bad, G == 0);
    }
}

// ---------------------------------------------------------------------------
// merge of split partials
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(64) void attn_merge_kernel(AttnParams p) {
    const int head = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const SeqRange r = seq_range(p.ctx_lens[b], p.max_blocks, p.window, p.split_blocks, p.max_splits);
    if (r.nsplit <= 1) return;
    const size_t base = ((size_t)b * p.n_h + head) * p.max_splits;
    const float *ml = p.ws_ml + base * 2;
    float M = -INFINITY;
    for (int s = 0; s < r.nsplit; ++s) M = fmaxf(M, ml[2 * s]);
    const int D = p.head_dim;
    const int cv = D / 64;
    float acc[2] = {0.0f, 0.0f};
    float L = 0.0f;
    for (int s = 0; s < r.nsplit; ++s) {
        const float wgt = exp2f(ml[2 * s] - M);
        L += wgt * ml[2 * s + 1];
        const float *o = p.ws_o + (base + s) * D + lane * cv;
        for (int c = 0; c < cv; ++c) acc[c] = fmaf(wgt, o[c], acc[c]);
    }
    float *dst = p.out + ((size_t)b * p.n_h + head) * D + lane * cv;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int c = 0; c < cv; ++c) dst[c] = acc[c] * inv;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int KIND, int D>
static hipError_t launch_valu_d(const AttnParams &p, dim3 grid, hipStream_t s) {
    const int g = p.group;
    if (g <= 1)
        hipLaunchKernelGGL((attn_valu_kernel<KIND, D, 1>), grid, dim3(64), 0, s, p);
    else if (g <= 2)
        hipLaunchKernelGGL((attn_valu_kernel<KIND, D, 2>), grid, dim3(64), 0, s, p);
    else if (g <= 4)
        hipLaunchKernelGGL((attn_valu_kernel<KIND, D, 4>), grid, dim3(64), 0, s, p);
    else if (g <= 8)
        hipLaunchKernelGGL((attn_valu_kernel<KIND, D, 8>), grid, dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL((attn_valu_kernel<KIND, D, 16>), grid, dim3(64), 0, s, p);
    return hipGetLastError();
}

template <int KIND>
static hipError_t launch_valu(const AttnParams &p, dim3 grid, hipStream_t s) {
    return p.head_dim == 64 ? launch_valu_d<KIND, 64>(p, grid, s) : launch_valu_d<KIND, 128>(p, grid, s);
}

hipError_t launch_attention(int dtype, int kernel, const AttnParams &p, hipStream_t s) {
    const dim3 grid(p.max_splits, p.n_kv, p.batch);
    if (p.batch == 0) return hipSuccess;
    if (dtype == KV_F32) return launch_valu<KIND_F32>(p, grid, s);
    if (dtype == KV_INT4) return launch_valu<KIND_INT4>(p, grid, s);
    if (kernel == 2) {
        if (p.head_dim == 64)
            hipLaunchKernelGGL(attn_mfma_bf16_kernel<64>, grid, dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL(attn_mfma_bf16_kernel<128>, grid, dim3(64), 0, s, p);
        return hipGetLastError();
    }
    return launch_valu<KIND_BF16>(p, grid, s);
}

hipError_t launch_merge(const AttnParams &p, hipStream_t s) {
    if (p.batch == 0 || p.max_splits <= 1) return hipSuccess;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(p.n_h, p.batch), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
