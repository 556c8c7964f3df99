// attention.hip -- paged decode attention for gfx950 (one or several query
// tokens per sequence).
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
// Work units. The query columns of a kv head are its g = n_h / n_kv query
// heads times the q_len query tokens, in 16-column tiles; a work unit is a
// kv head and one column tile (two on the bf16 MFMA path when there are
// several, four or eight in the wide units of attn_mfma_wide_kernel). A
// workgroup is one wave64 (two or four for wide units, which share each tile
// through LDS). It streams the unit's (block, kv head) tiles once and serves
// all its columns from each tile, keeping an online
// softmax (running max m and sum l, in log2 units: scores are pre-multiplied
// by scale * log2 e so exp becomes the hardware exp2; the max moves lazily,
// see kLazyLog2).
//
// Schedules (which workgroup takes which tiles):
//  * fixed splits (attn_mfma_kernel, attn_valu_kernel): grid (split, unit,
//    sequence), split_blocks blocks per split; attn_merge_kernel combines the
//    splits' (o, m, l): M = max_s m_s, out = sum_s 2^(m_s - M) o_s /
//    sum_s 2^(m_s - M) l_s.
//  * balanced (attn_mfma_balanced_kernel, the default): a persistent grid of
//    two waves per SIMD; every workgroup takes an equal share of all tiles of
//    the call; pairs cut between workgroups are merged by
//    attn_merge_balanced_rows_kernel / attn_merge_balanced_unit_kernel.
//  * shared prefixes (attn_mfma_shared_balanced_kernel, attn_mfma_shared_kernel):
//    a group's shared blocks are read once with the members' queries as the
//    columns.
//
// Tile engines:
//  * attn_valu_kernel (fp32, bf16, INT4): VALU dot products. Lane l takes
//    token l/4 of a block and a quarter of its channels for q.K (two xor
//    shuffles finish each dot product); for p.V lane l owns head_dim/64
//    channels and walks the block's tokens, the weights broadcast through LDS.
//  * mfma_block (bf16): the block's scores for a column tile are one 16x16
//    MFMA tile, S^T[token][column] = K_tile . Q^T, and the value update is
//    O^T[channel][column] += V_tile^T . P^T. P is split into bf16 hi + lo
//    parts so the weights keep ~16 bits (a single bf16 would cost up to 2^-9
//    relative error per weight); both parts go into one 16x16x32 MFMA per
//    channel tile, the tile's 4 tokens repeated along k against hi then lo.
//    The QK output layout (lane = column + 16 * token-quad) is exactly the
//    B-operand layout the PV product needs, so P never leaves registers.
//  * q4_block (INT4): the same products on the codes, with the scales and
//    minimums folded into the query and weight operands (see q4_block); with
//    at most four query columns the softmax runs on one score per lane
//    (q4_softmax_pv_one).
#include "device.h"
#include <hip/hip_ext.h>

#include <climits>

#include "internal.h"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// K/V tiles are read once per call: non-temporal loads keep them from
// displacing reusable lines in L2 and the Infinity Cache (measured: +12 %
// bandwidth on the 70B-shaped decode layer, +15 % on the 8B-shaped one).
__device__ __forceinline__ u32x4_t stream_load16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}
__device__ __forceinline__ u32x2_t stream_load8(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
}

// Pointers into global memory with the address space spelled out. A pointer
// chosen per lane between two buffers otherwise falls back to a flat
// (generic) load, which also counts against the LDS counter: every LDS wait
// in the softmax would then wait for the tile prefetch as well.
typedef const __attribute__((address_space(1))) uint16_t gu16_t;
typedef const __attribute__((address_space(1))) u32x4_t gu32x4_t;
typedef const __attribute__((address_space(1))) u32x2_t gu32x2_t;
__device__ __forceinline__ gu16_t *global_u16(const void *p) { return (gu16_t *)(p); }
__device__ __forceinline__ u32x4_t stream_load16(gu16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<gu32x4_t *>(p));
}
__device__ __forceinline__ u32x2_t stream_load8(gu16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<gu32x2_t *>(p));
}

enum { KIND_F32 = 0, KIND_BF16 = 1, KIND_INT4 = 2 };

// 2^x with the hardware instruction alone. Every argument here is a
// difference from a reference maximum (at most kLazyLog2, or -inf for a
// masked slot), so a result below the normal range, which the instruction
// flushes to 0, is a weight no fp32 softmax sum can register anyway.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy rescaling of the MFMA paths' online softmax: a column's reference
// maximum m moves only when a tile's score exceeds it by more than kLazyLog2
// (log2 units), so weights 2^(s - m) stay below 2^kLazyLog2 and the
// accumulators are rescaled a few times per segment instead of at every new
// maximum. (m, l, o) stay consistent for any m, so the merge is unchanged.
constexpr float kLazyLog2 = 8.0f;

// A value every lane of the wave reads from the same address, moved to a
// scalar register: the loads these come from are vector loads (the kernels
// also write global memory), and whatever is derived from them - block
// ranges, loop counters, tile addresses - would otherwise stay in vector
// registers and cost vector instructions on every tile.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The balanced schedule's split: shares numbered XCD by XCD on INT4 pools
// (XcdShares), in workgroup order otherwise (Shares).
template <bool XCD>
__device__ __forceinline__ auto split_of(long total, int n) {
    if constexpr (XCD)
        return xcd_shares_of(total, n);
    else
        return shares_of(total, n);
}

// Orders one wave's LDS accesses for its other lanes, for workgroups of a
// single wave: the LDS executes a wave's instructions in issue order, so no
// barrier or wait is needed, only that the compiler keeps the order.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Max / sum over lanes l, l^16, l^32, l^48: the four lanes that hold one
// column in the 16x16 MFMA layouts. gfx950's lane-swap instructions do both
// butterfly steps inside the VALU (no LDS round trip); every lane of the
// four ends with the same bits (each step adds the same two operands in the
// same order on both lanes of a pair).
// Larger of two floats by the hardware maximum alone. fmaxf also quiets
// signalling NaNs first (an extra instruction per operand that the compiler
// cannot prove canonical, e.g. a lane-swap result); no arithmetic produces
// one, and a quiet NaN operand gives the other operand either way.
__device__ __forceinline__ float max_raw(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float col_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max_raw(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Cross-lane moves inside each row of 16 lanes (DPP). A row's four banks are
// lanes 0-3, 4-7, 8-11, 12-15 of it.
enum { kDppRowShl = 0x100, kDppRowShr = 0x110, kDppRowRor = 0x120 };
// src moved by CTRL into the lanes of the banks in BANK; other lanes keep old.
template <int CTRL, int BANK>
__device__ __forceinline__ float dpp_f(float old, float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xf, BANK, false));
}
// x combined with x as moved by a DPP control that every lane of every row
// takes part in, in one instruction (the DPP move as a source modifier: no
// copy of x, no separate move). The s_nop gives the two wait states a DPP
// read needs after a vector write of its source.
#define KVC_DPP_OP(name, op, ctrl)                                                              \
    __device__ __forceinline__ float name(float x) {                                           \
        float r;                                                                               \
        asm("s_nop 1\n\t" op "_dpp %0, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x)); \
        return r;                                                                              \
    }
KVC_DPP_OP(dpp_max_ror4, "v_max_f32", "row_ror:4")
KVC_DPP_OP(dpp_max_ror8, "v_max_f32", "row_ror:8")
KVC_DPP_OP(dpp_add_ror4, "v_add_f32", "row_ror:4")
KVC_DPP_OP(dpp_add_ror8, "v_add_f32", "row_ror:8")
KVC_DPP_OP(dpp_add_xor1, "v_add_f32", "quad_perm:[1,0,3,2]")
KVC_DPP_OP(dpp_add_xor2, "v_add_f32", "quad_perm:[2,3,0,1]")
#undef KVC_DPP_OP
// Max / sum over lanes l, l^4, l^8, l^12 (the four banks of a row).
__device__ __forceinline__ float bank_max(float x) { return dpp_max_ror8(dpp_max_ror4(x)); }
__device__ __forceinline__ float bank_sum(float x) { return dpp_add_ror8(dpp_add_ror4(x)); }
// Sum over the 16 lanes of a row, in every lane of it.
__device__ __forceinline__ float row_sum(float x) { return bank_sum(dpp_add_xor2(dpp_add_xor1(x))); }

struct SplitWork {
    SeqRange r;
    int j0, j1;  // blocks [j0, j1) of this split
};

__device__ __forceinline__ bool split_work(const AttnParams &p, int b, int split, SplitWork &w) {
    w.r = seq_range(uniform(ctx_of(p, b)), p.max_blocks, p.window, p.split_blocks, p.max_splits, p.q_len);
    if (split >= w.r.nsplit) return false;
    w.j0 = w.r.blk_lo + split * p.split_blocks;
    w.j1 = min(w.r.blk_lo + w.r.nblk, w.j0 + p.split_blocks);
    return true;
}

// Final store of one lane's run of `n` consecutive channels of output row
// `row` ((sequence * q_len + query token) * n_h + head).
__device__ __forceinline__ void store_result(const AttnParams &p, size_t row, int split, int nsplit,
                                             int ch0, const float *o, int n, float m, float l, bool bad,
                                             bool write_ml) {
    const float nan = __uint_as_float(0x7fc00000u);
    if (nsplit == 1) {
        float *dst = p.out + row * p.head_dim + ch0;
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        for (int c = 0; c < n; ++c) dst[c] = bad ? nan : o[c] * inv;
    } else {
        const size_t base = row * p.max_splits + split;
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
            const float alpha = mn == m_run[h] ? 1.0f : fast_exp2(m_run[h] - mn);
            const float pe = fast_exp2(s[h] - mn);
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
        if (h < g)
            store_result(p, (size_t)b * p.n_h + kvh * g + h, split, w.r.nsplit, lane * CV, acc[h], CV, m_run[h], l,
                         bad, lane == 0);
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16 pools)
// ---------------------------------------------------------------------------

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
// (hardware conversion)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// One (block, kv head) tile in MFMA operand layout.
template <int D>
struct MfmaTile {
    bf16x8_t k[D / 32];          // A operand of S^T = K . Q^T: token n16, channels s*32 + 8G .. +8
    uint32_t v[4][D / 32];       // rows 4G + i, channels n16 * (D/16) .. + D/16 (bf16 pairs)
};

// Tile of block j. Rows of positions in [L0, L0 + n_new) come from the step's
// k_new / v_new instead of the pool (fused append); newpos = L0 - 16 j is
// uniform, and >= 16 when the block holds no new token.
// KEEP: ordinary (cached) loads instead of non-temporal ones. A template
// argument, not a run-time flag: a select between the two loads of one
// address is merged into one load without the non-temporal hint.
template <int D, bool KEEP = false>
__device__ __forceinline__ void fetch_tile(const AttnParams &p, int pid, int kvh, int n16, int G, MfmaTile<D> &T,
                                           int b = 0, int newpos = kBlock) {
    constexpr int KS = D / 32, VC = D / 16;
    gu16_t *tile = global_u16(p.pool.k) + ((size_t)pid * p.n_kv + kvh) * kBlock * D;
    gu16_t *vt = global_u16(p.pool.v) + ((size_t)pid * p.n_kv + kvh) * kBlock * D;
    gu16_t *krow = tile + n16 * D;
    gu16_t *vrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vrow[i] = vt + (4 * G + i) * D;
    if (newpos < kBlock) {
        auto fresh = [&](const void *base, int slot) {
            return global_u16(base) + (((size_t)b * p.ctx_add + (slot - newpos)) * p.n_kv + kvh) * D;
        };
        if (n16 >= newpos && n16 < newpos + p.ctx_add) krow = fresh(p.k_new, n16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = 4 * G + i;
            if (slot >= newpos && slot < newpos + p.ctx_add) vrow[i] = fresh(p.v_new, slot);
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        gu16_t *src = krow + s * 32 + 8 * G;
        T.k[s] = __builtin_bit_cast(bf16x8_t, KEEP ? *reinterpret_cast<gu32x4_t *>(src) : stream_load16(src));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gu16_t *src = vrow[i] + n16 * VC;
        if constexpr (VC == 8) {
            const u32x4_t v = KEEP ? *reinterpret_cast<gu32x4_t *>(src) : stream_load16(src);
            T.v[i][0] = v[0];
            T.v[i][1] = v[1];
            T.v[i][2] = v[2];
            T.v[i][3] = v[3];
        } else {
            const u32x2_t v = KEEP ? *reinterpret_cast<gu32x2_t *>(src) : stream_load8(src);
            T.v[i][0] = v[0];
            T.v[i][1] = v[1];
        }
    }
}

// Fused append: write the new tokens' K and V rows that fall in block j
// (slots [max(newpos, 0), min(newpos + n_new, hi_slot))) into the pool tile.
template <int D>
__device__ __forceinline__ void store_new_rows(const AttnParams &p, int b, int kvh, int pid, int newpos, int lane) {
    constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
    const int first = max(newpos, 0), last = min(newpos + p.ctx_add, kBlock);
    const int rows = last - first;
    for (int idx = lane; idx < 2 * rows * CPR; idx += 64) {
        const int which = idx / (rows * CPR), rem = idx - which * rows * CPR;
        const int slot = first + rem / CPR, c = rem % CPR;
        const uint4 *src = reinterpret_cast<const uint4 *>(which ? p.v_new : p.k_new) +
                           (((size_t)b * p.ctx_add + (slot - newpos)) * p.n_kv + kvh) * CPR + c;
        uint4 *dst = reinterpret_cast<uint4 *>(which ? p.pool.v : p.pool.k) +
                     (((size_t)pid * p.n_kv + kvh) * kBlock + slot) * CPR + c;
        *dst = *src;
    }
}

// Online-softmax state of one lane: head n16, the lane's 4 token rows.
template <int D>
struct MfmaState {
    f32x4_t o[D / 16];
    float m, l;
    float bv;  // INT4: numerator term common to every channel (this lane's part)
};

// The query column a lane serves: c = ct * 16 + n16 of kv head kvh's g * q_len
// columns is query token i = c / g of head kvh * g + c % g; it attends tokens
// [lo, hi). Padded columns (c >= ncols) get a query of 0 and the common range.
struct Column {
    bool valid;
    size_t row;  // output / query row ((b * q_len + i) * n_h + head)
    int lo, hi;
};

__device__ __forceinline__ Column column_of(const AttnParams &p, int b, int kvh, int ct, int n16, const SeqRange &r) {
    Column c;
    const int ci = ct * 16 + n16;
    c.valid = ci < p.ncols;
    const int i = c.valid ? ci / p.group : p.q_len - 1, hq = c.valid ? ci % p.group : 0;
    c.row = ((size_t)b * p.q_len + i) * p.n_h + kvh * p.group + hq;
    c.hi = r.n - p.q_len + i + 1;
    c.lo = p.window > 0 ? max(c.hi - p.window, 0) : 0;
    return c;
}

// Score masking of one block: token position tok0 + 4G + r is valid for the
// lane's column if it lies in [col.lo, col.hi). Blocks inside the range every
// column attends skip the test (uniform branch).
__device__ __forceinline__ bool needs_mask(int tok0, const SeqRange &r) {
    return tok0 < r.all_lo || tok0 + kBlock > r.all_hi;
}

template <int D>
__device__ __forceinline__ void mfma_block(const AttnParams &p, const MfmaTile<D> &T, const bf16x8_t (&qB)[D / 32],
                                           int tok0, int tlo, int thi, bool mask, const Column &col, int G,
                                           MfmaState<D> &st) {
    constexpr int KS = D / 32, MS = D / 16, VC = D / 16;
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[s], qB[s], sc, 0, 0, 0);
    const bool partial = tlo > 0 || thi < kBlock;  // uniform: slots outside [tlo, thi) hold no token
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tp = tok0 + 4 * G + r;
        bool ok = true;
        if (mask) ok = (tp >= col.lo) & (tp < col.hi);  // mask is uniform
        sv[r] = ok ? sc[r] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[r]);
    }
    // A column's maximum exceeds its reference by more than the slack
    // exactly when one of its lanes' maxima does: the test needs no
    // reduction, and the column maxima are formed only when it passes.
    if (__any(mx > st.m + kLazyLog2)) {
        // some column's maximum moved past its reference by more than the
        // slack: move every column's reference to its maximum and rescale
        const float cm = col_max(mx);
        const float mn = fmaxf(st.m, cm);
        const float alpha = mn == st.m ? 1.0f : fast_exp2(st.m - mn);  // unchanged (even -inf): 1
        st.l *= alpha;
#pragma unroll
        for (int m = 0; m < MS; ++m) st.o[m] *= alpha;
        st.m = mn;
    }
    // a column that has seen no token yet (max -inf) gets weights 0, not NaN
    const float mref = st.m == -INFINITY ? 0.0f : st.m;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pr[r] = fast_exp2(sv[r] - mref);
        st.l += pr[r];
    }
    // P^T as B operand, split into bf16 hi and lo parts (the lo part rounds
    // the exact fp32 remainder)
    const uint32_t h01 = cvt_pk_bf16(pr[0], pr[1]), h23 = cvt_pk_bf16(pr[2], pr[3]);
    const uint32_t l01 = cvt_pk_bf16(pr[0] - __uint_as_float(h01 << 16), pr[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = cvt_pk_bf16(pr[2] - __uint_as_float(h23 << 16), pr[3] - __uint_as_float(h23 & 0xffff0000u));
    // hi and lo parts side by side along k: one 16x16x32 product per channel
    // tile takes both (k = 8G + i: hi of token 4G + i for i < 4, lo of token
    // 4G + i - 4 after)
    const bf16x8_t pB = __builtin_bit_cast(bf16x8_t, make_uint4(h01, h23, l01, l23));
    uint32_t vr[4][VC / 2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < VC / 2; ++k) vr[i][k] = T.v[i][k];
    if (partial) {
        // slots outside [tlo, thi) may hold anything (even NaN): zero their rows
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
        // the 16-bit half m & 1 of word m >> 1 of tokens (0, 1) and (2, 3)
        const int wi = m >> 1;
        const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t a01 = __builtin_amdgcn_perm(vr[1][wi], vr[0][wi], sel);
        const uint32_t a23 = __builtin_amdgcn_perm(vr[3][wi], vr[2][wi], sel);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a01, a23, a01, a23));
        st.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pB, st.o[m], 0, 0, 0);
    }
}

// The same for the CT column tiles one wave holds, on one tile, side by side
// (CT > 1): the score products of every column tile first (each in two
// MFMA chains), one lazy-rescale test for all of them, and each V operand
// formed once for the CT value products. Independent work between the
// dependent steps of each column tile, and fewer instructions: 8B shape, 16
// query tokens 178 -> 166 us, 32 tokens 287 -> 256 us (wide units, which
// also keep the sequence search in scalar registers).
// The mask test is read into a scalar register: one branch per tile rather
// than lane masking around every score.
template <int D, int CT>
__device__ __forceinline__ void mfma_block_ct(const AttnParams &p, const MfmaTile<D> &T,
                                              const bf16x8_t (&qB)[CT][D / 32], int tok0, int tlo, int thi, bool mask,
                                              const Column *col, int G, MfmaState<D> *st) {
    constexpr int KS = D / 32, MS = D / 16, VC = D / 16;
    static_assert(KS % 2 == 0, "two score chains of KS / 2 products");
    f32x4_t sc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[s], qB[c][s], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[s + 1], qB[c][s + 1], s1, 0, 0, 0);
        }
        sc[c] = s0 + s1;
    }
    const bool partial = tlo > 0 || thi < kBlock;  // uniform
    float sv[CT][4], mx[CT];
    if (__builtin_amdgcn_readfirstlane((int)mask)) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            mx[c] = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tp = tok0 + 4 * G + r;
                const bool ok = (tp >= col[c].lo) & (tp < col[c].hi);
                sv[c][r] = ok ? sc[c][r] * p.scale_log2 : -INFINITY;
                mx[c] = fmaxf(mx[c], sv[c][r]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            mx[c] = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sv[c][r] = sc[c][r] * p.scale_log2;
                mx[c] = fmaxf(mx[c], sv[c][r]);
            }
        }
    }
    bool grow = false;
#pragma unroll
    for (int c = 0; c < CT; ++c) grow |= mx[c] > st[c].m + kLazyLog2;
    if (__any(grow)) {  // as in mfma_block, for every column tile at once
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const float mn = fmaxf(st[c].m, col_max(mx[c]));
            const float alpha = mn == st[c].m ? 1.0f : fast_exp2(st[c].m - mn);
            st[c].l *= alpha;
#pragma unroll
            for (int m = 0; m < MS; ++m) st[c].o[m] *= alpha;
            st[c].m = mn;
        }
    }
    bf16x8_t pB[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const float mref = st[c].m == -INFINITY ? 0.0f : st[c].m;
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = fast_exp2(sv[c][r] - mref);
            st[c].l += pr[r];
        }
        const uint32_t h01 = cvt_pk_bf16(pr[0], pr[1]), h23 = cvt_pk_bf16(pr[2], pr[3]);
        const uint32_t l01 = cvt_pk_bf16(pr[0] - __uint_as_float(h01 << 16), pr[1] - __uint_as_float(h01 & 0xffff0000u));
        const uint32_t l23 = cvt_pk_bf16(pr[2] - __uint_as_float(h23 << 16), pr[3] - __uint_as_float(h23 & 0xffff0000u));
        pB[c] = __builtin_bit_cast(bf16x8_t, make_uint4(h01, h23, l01, l23));
    }
    uint32_t vr[4][VC / 2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < VC / 2; ++k) vr[i][k] = T.v[i][k];
    if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = 4 * G + i;
            if (tt < tlo || tt >= thi) {
#pragma unroll
                for (int k = 0; k < VC / 2; ++k) vr[i][k] = 0u;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const int wi = m >> 1;
        const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t a01 = __builtin_amdgcn_perm(vr[1][wi], vr[0][wi], sel);
        const uint32_t a23 = __builtin_amdgcn_perm(vr[3][wi], vr[2][wi], sel);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a01, a23, a01, a23));
#pragma unroll
        for (int c = 0; c < CT; ++c) st[c].o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pB[c], st[c].o[m], 0, 0, 0);
    }
}

// Block ids [j0, j1) of one sequence's table row (at most kSidsWindow of
// them), staged in LDS before a piece's tile loop. A segment longer than that
// runs as several pieces that carry the softmax state (run_pieces), so a
// workgroup's dynamic LDS holds at most kSidsWindow ids however long its
// segments are.
constexpr int kSidsWindow = 256;
constexpr int kSidsPerLane = kSidsWindow / 64;
struct BlockIds {
    int *sids;
    const int32_t *row;  // the sequence's table row
    int j0;
    int last;  // the table's entry for block j1 - 1, as read (unchecked; uniform)
    __device__ __forceinline__ int id(int j) const { return __builtin_amdgcn_readfirstlane(sids[j - j0]); }
};

// For the one-wave workgroups of the decode kernels: the LDS executes a
// wave's accesses in issue order, so the staging needs no barrier (a
// workgroup barrier's fence would also wait for the wave's earlier global
// stores and loads, e.g. the previous segment's results). All of the piece's
// table loads go out before any is used: one memory round trip, however
// many ids. CHECK: an id outside [0, num_blocks) is staged as 0 and sets bad
// (the ids are then checked once here rather than per tile); otherwise ids
// are staged as read.
template <bool CHECK>
__device__ __forceinline__ BlockIds stage_ids(const AttnParams &p, int b, int j0, int j1, int lane, int *sids,
                                              bool &bad) {
    BlockIds ids;
    ids.sids = sids;
    ids.row = p.tables + (size_t)b * p.max_blocks;
    ids.j0 = j0;
    const int n = j1 - j0;  // 1 .. kSidsWindow
    int v[kSidsPerLane];
#pragma unroll
    for (int k = 0; k < kSidsPerLane; ++k) {
        const int i = lane + 64 * k;
        v[k] = i < n ? ids.row[j0 + i] : 0;
    }
    ids.last = 0;
#pragma unroll
    for (int k = 0; k < kSidsPerLane; ++k)
        if (k == (n - 1) >> 6) ids.last = __builtin_amdgcn_readlane(v[k], (n - 1) & 63);
    wave_lds_sync();  // this wave's earlier reads of sids come first
    bool wrong = false;
#pragma unroll
    for (int k = 0; k < kSidsPerLane; ++k) {
        const int i = lane + 64 * k;
        if (i < n) {
            int id = v[k];
            if constexpr (CHECK) {
                const bool ok = id >= 0 && id < p.num_blocks;
                wrong |= !ok;
                id = ok ? id : 0;
            }
            sids[i] = id;
        }
    }
    if (CHECK && __any(wrong)) bad = true;
    wave_lds_sync();
    return ids;
}
__device__ __forceinline__ BlockIds stage_block_ids(const AttnParams &p, int b, int j0, int j1, int lane,
                                                    int *sids) {
    bool unused = false;
    return stage_ids<false>(p, b, j0, j1, lane, sids, unused);
}
__device__ __forceinline__ BlockIds stage_checked_block_ids(const AttnParams &p, int b, int j0, int j1, int lane,
                                                            int *sids, bool &bad) {
    return stage_ids<true>(p, b, j0, j1, lane, sids, bad);
}

// Runs seg(c0, c1, init) over [j0, j1) in pieces of at most kSidsWindow
// blocks; init is true for the first piece only (it resets the softmax
// state, the others continue it). An empty range still makes one call.
// Pacing of the persistent balanced kernels. The two waves that share a SIMD
// get equal shares, but issue goes to the older wave first, so one of them
// used to finish long before the other (INT4, 8B shape: 40 vs 51 us on
// average), which then ran alone and slower. Each wave instead sets its own
// priority from its progress through its share (s_setprio: priority is
// compared before age): 3 in the first half, 2 up to 80 %, 1 up to 95 %, 0
// after. A wave that falls behind its partner is issued first until it
// catches up, so the pair ends within a few percent of a share of each
// other. The state is only values: block j of a piece sits at share
// position base + j, and the band ends th1..th3 are fixed per workgroup
// (share 0: no pacing). Kept in registers: a pacing state in memory made
// every tile wait for the next tile's loads.
struct Pace {
    int base, th1, th2, th3;
};

__device__ __forceinline__ Pace pace_for(long share) {
    Pace pc;
    const int sh = (int)share;
    pc.base = 0;
    pc.th1 = sh > 0 ? sh / 2 : INT_MAX;
    pc.th2 = sh > 0 ? (int)((long)sh * 4 / 5) : INT_MAX;
    pc.th3 = sh > 0 ? (int)((long)sh * 19 / 20) : INT_MAX;
    return pc;
}

// Priority of the band holding share position pos (uniform).
__device__ __forceinline__ void pace_set(const Pace &pc, int pos) {
    if (pc.th1 == INT_MAX) return;
    if (pos >= pc.th3)
        __builtin_amdgcn_s_setprio(0);
    else if (pos >= pc.th2)
        __builtin_amdgcn_s_setprio(1);
    else if (pos >= pc.th1)
        __builtin_amdgcn_s_setprio(2);
    else
        __builtin_amdgcn_s_setprio(3);
}

// After block j of a piece: the band changes when the next position reaches
// one of its ends.
__device__ __forceinline__ void pace_tick(const Pace &pc, int j) {
    const int pos = pc.base + j + 1;
    if (pos == pc.th1 || pos == pc.th2 || pos == pc.th3) pace_set(pc, pos);
}

template <class Seg>
__device__ __forceinline__ void run_pieces(int j0, int j1, Seg seg) {
    for (int c0 = j0;; c0 += kSidsWindow) {
        const int c1 = min(j1, c0 + kSidsWindow);
        seg(c0, c1, c0 == j0);
        if (c1 >= j1) break;
    }
}

// One lane's run of the online softmax over blocks [j0, j1) of sequence b,
// kv head kvh (at most kSidsWindow blocks; init: start a new state, else
// continue st), for CT column tiles at once (col[c], st[c]): each K/V tile is
// loaded once and multiplied with every column tile's queries. On return
// st[c].l is still the lane's partial sum (the caller adds the 4 token
// quads).
//
// Every tile iteration issues the same vector-memory loads and nothing else:
// the piece's block ids are staged in LDS before the loop and the fused
// append's rows are written before it, so the waits inside the loop cover
// exactly the tile's own loads.
template <int D, int CT, bool KEEP = false>
__device__ __forceinline__ void bf16_segment_ct(const AttnParams &p, int b, int kvh, const Column *col,
                                                const SeqRange &r, int j0, int j1, int lane, MfmaState<D> *st,
                                                bool &bad, bool write_new, int *sids, bool init,
                                                Pace pace = Pace{0, INT_MAX, INT_MAX, INT_MAX}) {
    constexpr int KS = D / 32, MS = D / 16;
    const int n16 = lane & 15, G = lane >> 4;
    // Q^T as B operand: lane (G, n16) holds channels s*32 + 8G .. +8 of its column.
    bf16x8_t qB[CT][KS];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col[c].valid)
                v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.q) + col[c].row * D + s * 32 +
                                                     8 * G);
            qB[c][s] = __builtin_bit_cast(bf16x8_t, v);
        }
    if (init) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
            for (int m = 0; m < MS; ++m) st[c].o[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            st[c].m = -INFINITY;
            st[c].l = 0.0f;
            st[c].bv = 0.0f;
        }
    }
    if (j0 >= j1) return;

    const BlockIds ids = stage_block_ids(p, b, j0, j1, lane, sids);
    auto pid_of = [&](int j) {
        int pid = ids.id(j);
        if (pid < 0 || pid >= p.num_blocks) {
            bad = true;
            pid = 0;
        }
        return pid;
    };
    // fused append: positions from L0 on are the step's new tokens; their rows
    // go into the pool now (nothing in this kernel reads those slots)
    const int L0 = p.k_new ? r.n - p.ctx_add : INT_MAX;
    if (write_new && L0 != INT_MAX) {
        for (int j = max(j0, L0 / kBlock); j < j1; ++j) {
            const int id = ids.id(j);
            if (id >= 0 && id < p.num_blocks) store_new_rows<D>(p, b, kvh, id, L0 - j * kBlock, lane);
        }
    }
    auto fetch = [&](int j, MfmaTile<D> &T) {
        const int newpos = L0 == INT_MAX ? kBlock : min(L0 - j * kBlock, kBlock);  // may be negative
        fetch_tile<D, KEEP>(p, pid_of(j), kvh, n16, G, T, b, newpos);
    };
    auto compute = [&](const MfmaTile<D> &T, int j) {
        const int tok0 = j * kBlock;
        const int tlo = max(r.lo - tok0, 0), thi = min(r.hi - tok0, kBlock);
        // one column tile after the other: the side-by-side form of the wide
        // units (mfma_block_ct) measured no faster on this single-wave path
        // (5 query tokens 121 vs 123 us)
#pragma unroll
        for (int c = 0; c < CT; ++c) mfma_block<D>(p, T, qB[c], tok0, tlo, thi, needs_mask(tok0, r), col[c], G, st[c]);
    };
    // No software prefetch: each tile is loaded and then used. The waves that
    // share a SIMD cover each other's compute; a deeper prefetch puts more
    // bytes in flight and measured slower (6.8 vs 6.0-6.4 TB/s in a probe of
    // this tile pattern with per-tile work).
    for (int j = j0; j < j1; ++j) {
        MfmaTile<D> T;
        fetch(j, T);
        compute(T, j);
        pace_tick(pace, j);
    }
}

template <int D>
__device__ __forceinline__ void bf16_segment(const AttnParams &p, int b, int kvh, const Column &col,
                                             const SeqRange &r, int j0, int j1, int lane, MfmaState<D> &st,
                                             bool &bad, bool write_new, int *sids, bool init) {
    bf16_segment_ct<D, 1>(p, b, kvh, &col, r, j0, j1, lane, &st, bad, write_new, sids, init);
}

// lane (G, n16) holds channel (4G + r) * (D/16) + m of head n16 in o[m][r]:
// a contiguous run of D/4 channels starting at G * D/4.
template <int D>
__device__ __forceinline__ void mfma_gather_run(const MfmaState<D> &st, float bv, float (&res)[D / 4]) {
    constexpr int MS = D / 16, VC = D / 16;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int m = 0; m < MS; ++m) res[r * VC + m] = st.o[m][r] + bv;
}


// ---------------------------------------------------------------------------
// INT4 path (head_dim 128) of the MFMA kernels
//
// Full blocks: s_t = sum_c code_tc * (q_c * scale_c) + sum_c q_c * min_c.
// q_c * scale_c is exact in fp32 (8-bit by 11-bit significands) and enters
// the B operand as bf16 hi + lo; codes enter the A operand as exact bf16
// integers; the min term is a per-head correction added to the scores.
// A sequence's partial last block takes its K from the bf16 tail row with
// plain q. Values: sum_t p_t (min_t + scale_t * code_tc) = sum_t P'_t *
// code_tc + sum_t p_t * min_t with P'_t = p_t * scale_t (bf16 hi + lo in
// the B operand) and the exact codes in the A operand; the second sum is a
// per-head numerator term kept beside o.
// Lane (G, n16) covers channels 32G .. 32G+31 in the score product and
// value channels 8 n16 .. 8 n16 + 7 in the value product.
// ---------------------------------------------------------------------------


typedef const __attribute__((address_space(1))) uint8_t gu8_t;
typedef const __attribute__((address_space(1))) uint32_t gu32_t;
typedef const __attribute__((address_space(1))) uint2 gu2_t;
__device__ __forceinline__ gu8_t *global_u8(const void *p) { return (gu8_t *)(p); }

struct Q4Tile {
    uint4 kc;        // K codes of token n16, channels 32G .. 32G+31 (score A operand)
    uint4 ks, km;    // fp16 K scales / mins of channels 8 n16 .. 8 n16 + 7
    uint32_t vc[4];  // V codes of tokens 4G+i, channels 8 n16 .. 8 n16 + 7
    uint2 vs, vm;    // fp16 V scales / mins of tokens 4G .. 4G+3
};

// All of a block's loads, whether or not the block is full (a partial block
// takes its K from the tail row, and its pool K bytes go unused): the same
// loads on every path keep the compiler's waits to the tile being used.
// Buffer resource over `bytes` bytes from base (scalar registers), for raw
// buffer loads: the tile base stays scalar, the lane offset is a 32-bit
// vector operand, and reads past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
enum { kLoadStream = 2 };  // cache policy of a raw buffer load: non-temporal

// none: issue the same loads with empty descriptors (they read nothing from
// memory and return 0), for the prefetch slot past a segment's last tile.
__device__ __forceinline__ void q4_fetch(const AttnParams &p, int pid, int kvh, int n16, int G, Q4Tile &T,
                                         bool none) {
    const size_t tile = (size_t)pid * p.n_kv + kvh;
    const int on = none ? 0 : 1;
    const auto kq = tile_rsrc(p.pool.kq + tile * (kBlock * 64), on * kBlock * 64);
    const auto vq = tile_rsrc(p.pool.vq + tile * (kBlock * 64), on * kBlock * 64);
    const auto ks = tile_rsrc(p.pool.ks + tile * 128, on * 256);
    const auto km = tile_rsrc(p.pool.km + tile * 128, on * 256);
    const auto vs = tile_rsrc(p.pool.vs + tile * kBlock, on * kBlock * 2);
    const auto vm = tile_rsrc(p.pool.vm + tile * kBlock, on * kBlock * 2);
    T.kc = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kq, n16 * 64 + 16 * G, 0, kLoadStream));
    T.ks = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ks, 16 * n16, 0, kLoadStream));
    T.km = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(km, 16 * n16, 0, kLoadStream));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        T.vc[i] = __builtin_amdgcn_raw_buffer_load_b32(vq, (4 * G + i) * 64 + 4 * n16, 0, kLoadStream);
    const u32x2_t s = __builtin_amdgcn_raw_buffer_load_b64(vs, 8 * G, 0, kLoadStream);
    const u32x2_t m = __builtin_amdgcn_raw_buffer_load_b64(vm, 8 * G, 0, kLoadStream);
    T.vs = make_uint2(s[0], s[1]);
    T.vm = make_uint2(m[0], m[1]);
}

// The same loads when the pool's INT4 arrays, from the K codes to the end
// of the V minimums, span less than 4 GiB: one buffer descriptor over that
// span for the whole segment, and each tile reached through 32-bit scalar
// offsets (a handful of scalar instructions per tile instead of six
// descriptors built from 64-bit addresses).
struct Q4Flat {
    __amdgpu_buffer_rsrc_t rsrc, none;  // the span, and an empty descriptor (reads return 0)
    uint32_t vq, ks, km, vs, vm;        // byte offsets of the other arrays from the K codes
};
__device__ __forceinline__ Q4Flat q4_flat(const AttnParams &p) {
    const char *kq = reinterpret_cast<const char *>(p.pool.kq);
    auto off = [&](const void *a) { return (uint32_t)(reinterpret_cast<const char *>(a) - kq); };
    Q4Flat f;
    f.rsrc = tile_rsrc(p.pool.kq, (int)p.pool.q4_span);
    f.none = tile_rsrc(p.pool.kq, 0);
    f.vq = off(p.pool.vq);
    f.ks = off(p.pool.ks);
    f.km = off(p.pool.km);
    f.vs = off(p.pool.vs);
    f.vm = off(p.pool.vm);
    return f;
}
__device__ __forceinline__ void q4_fetch_flat(const Q4Flat &f, uint32_t tile, int n16, int G, Q4Tile &T,
                                              bool none) {
    const uint32_t codes = tile * (kBlock * 64), kpar = tile * 256, vpar = tile * (kBlock * 2);
    const auto rs = none ? f.none : f.rsrc;
    T.kc = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, n16 * 64 + 16 * G, codes, kLoadStream));
    T.ks = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * n16, f.ks + kpar, kLoadStream));
    T.km = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * n16, f.km + kpar, kLoadStream));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        T.vc[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (4 * G + i) * 64 + 4 * n16, f.vq + codes, kLoadStream);
    const u32x2_t s = __builtin_amdgcn_raw_buffer_load_b64(rs, 8 * G, f.vs + vpar, kLoadStream);
    const u32x2_t m = __builtin_amdgcn_raw_buffer_load_b64(rs, 8 * G, f.vm + vpar, kLoadStream);
    T.vs = make_uint2(s[0], s[1]);
    T.vm = make_uint2(m[0], m[1]);
}


// 8 codes of one dword (channel 2k in the low nibble of byte k) as exact bf16,
// in the order channels 0, 2, 4, 6, 1, 3, 5, 7 (even channels from the low
// nibbles, odd ones from the high nibbles: no byte permutes). The score
// product's B operand (q4_block) takes its channels in the same order.
// A byte c < 16 read as an OCP E4M3 value is exactly c * 2^-9 (a subnormal
// for c < 8, exponent field 1 for 8 <= c < 16), so the hardware fp8 -> bf16
// conversion with scale 2^9 gives c itself, two codes per instruction.
__device__ __forceinline__ bf16x8_t q4_codes_bf16(uint32_t w) {
    const uint32_t ev = w & 0x0f0f0f0fu, od = (w >> 4) & 0x0f0f0f0fu;  // codes of channels 0,2,4,6 / 1,3,5,7
    const bf16x2_t d0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 512.0f, false);  // channels 0, 2
    const bf16x2_t d1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 512.0f, true);   // 4, 6
    const bf16x2_t d2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 512.0f, false);  // 1, 3
    const bf16x2_t d3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 512.0f, true);   // 5, 7
    return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, d0), __builtin_bit_cast(uint32_t, d1),
                                                   __builtin_bit_cast(uint32_t, d2), __builtin_bit_cast(uint32_t, d3)));
}

__device__ __forceinline__ float f16_lo(uint32_t w) { return f16_bits_to_f((uint16_t)w); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16_bits_to_f((uint16_t)(w >> 16)); }

// Per-workgroup LDS of the INT4 path: the score product's B operand (query
// times per-channel K scale, bf16 hi and lo parts) of the 16 columns, and the
// per-column partial sums of query times K min. Rows are padded to 17 chunks
// of 8 channels (272 bytes) so that the reads of 8 consecutive lanes, one row
// each, fall in distinct banks.
struct Q4Lds {
    uint4 b[2][16][17];   // [hi / lo][column][channel chunk]
    float corr[16];       // [column]: the column's sum over channels of q times K min
};

// Query of the columns this lane computes products for: column 4 pi + G,
// channels 8 n16 .. 8 n16 + 7, pass pi < npass (fp32, bf16-exact; 0 for
// padded columns).
template <int NP>
struct Q4Query {
    float q[NP][8];
    int npass;
    float nz;  // -0.0, hidden from the compiler: fma(q, s, nz) would otherwise become a plain multiply
};

// Masking of an INT4 tile some of whose slots are outside the attended
// range (partial block, window, causal columns), in place: their scores sv
// become -inf, and their V scale and min (vs, vm), which may be anything
// there, 0, so that their zero weights contribute exactly 0.
__device__ __forceinline__ void q4_mask(int tok0, int tlo, int thi, const Column &col, int G, float (&sv)[4],
                                        uint2 &vs, uint2 &vm) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tt = 4 * G + r, tp = tok0 + tt;
        const bool ok = (tt >= tlo) & (tt < thi) & (tp >= col.lo) & (tp < col.hi);
        sv[r] = ok ? sv[r] : -INFINITY;
        const uint32_t keep = ok ? 0xffffffffu : 0u, half = (r & 1) ? 0xffff0000u : 0x0000ffffu;
        const uint32_t clear = ~half | keep;  // all ones, or the slot's half cleared
        if (r < 2) {
            vs.x &= clear;
            vm.x &= clear;
        } else {
            vs.y &= clear;
            vm.y &= clear;
        }
    }
}

// Online softmax and value update of one INT4 tile, given its scores sv and
// V scales / mins vs, vm (fp16 pairs; masked slots have score -inf and zero
// parameters). Full and masked tiles share this code (only their inputs
// differ), so the accumulators are updated in place.
// Values: sum_t p_t (min_t + scale_t * code_tc) = sum_t P'_t * code_tc +
// sum_t p_t * min_t with P'_t = p_t * scale_t (bf16 hi + lo in the B
// operand) and the exact codes in the A operand; the second sum is a
// per-column numerator term kept beside o.
__device__ __forceinline__ void q4_softmax_pv(const AttnParams &p, const Q4Tile &T, const float (&sv)[4], uint2 vs,
                                              uint2 vm, MfmaState<128> &st) {
    const float mx = max_raw(max3_raw(sv[0], sv[1], sv[2]), sv[3]);
    if (__any(mx > st.m + kLazyLog2)) {  // lazy rescale, as in mfma_block
        const float mn = fmaxf(st.m, col_max(mx));
        const float alpha = mn == st.m ? 1.0f : fast_exp2(st.m - mn);  // unchanged (even -inf): 1
        st.l *= alpha;
        st.bv *= alpha;
#pragma unroll
        for (int m = 0; m < 8; ++m) st.o[m] *= alpha;
        st.m = mn;
    }
    const uint32_t vsw[2] = {vs.x, vs.y}, vmw[2] = {vm.x, vm.y};
    const float mref = st.m == -INFINITY ? 0.0f : st.m;  // no token seen yet: weights 0
    float pv[4];
    float bv = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float pr = fast_exp2(sv[r] - mref);  // 0 for masked slots
        st.l += pr;
        const float vsc = (r & 1) ? f16_hi(vsw[r >> 1]) : f16_lo(vsw[r >> 1]);
        const float vmn = (r & 1) ? f16_hi(vmw[r >> 1]) : f16_lo(vmw[r >> 1]);
        pv[r] = pr * vsc;
        bv = fmaf(pr, vmn, bv);
    }
    st.bv += bv;
    const uint32_t h01 = cvt_pk_bf16(pv[0], pv[1]), h23 = cvt_pk_bf16(pv[2], pv[3]);
    const uint32_t l01 = cvt_pk_bf16(pv[0] - __uint_as_float(h01 << 16), pv[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = cvt_pk_bf16(pv[2] - __uint_as_float(h23 << 16), pv[3] - __uint_as_float(h23 & 0xffff0000u));
    const bf16x4_t pHi = __builtin_bit_cast(bf16x4_t, make_uint2(h01, h23));
    const bf16x4_t pLo = __builtin_bit_cast(bf16x4_t, make_uint2(l01, l23));
    // A operand of channel tile m: the exact codes of tokens 4G .. 4G+3 at
    // channel 8 n16 + m. Bytes of tokens (0,1) and (2,3) are interleaved so
    // that after splitting nibbles each 16-bit half holds one channel of both
    // tokens, which the fp8 conversion turns into a bf16 pair (see
    // q4_codes_bf16 for why that conversion is exact).
    uint32_t a01[8], a23[8];
    auto spread = [](uint32_t x, uint32_t(&dst)[8], int c0) {
        const uint32_t e = x & 0x0f0f0f0fu, o = (x >> 4) & 0x0f0f0f0fu;
        dst[c0 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(e, 512.0f, false));
        dst[c0 + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(e, 512.0f, true));
        dst[c0 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(o, 512.0f, false));
        dst[c0 + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(o, 512.0f, true));
    };
    spread(__builtin_amdgcn_perm(T.vc[1], T.vc[0], 0x05010400u), a01, 0);  // channels 0-3
    spread(__builtin_amdgcn_perm(T.vc[1], T.vc[0], 0x07030602u), a01, 4);  // channels 4-7
    spread(__builtin_amdgcn_perm(T.vc[3], T.vc[2], 0x05010400u), a23, 0);
    spread(__builtin_amdgcn_perm(T.vc[3], T.vc[2], 0x07030602u), a23, 4);
    // masked slots: P' is 0 there and the codes are finite, so nothing leaks
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        // two 16x16x16 products: one 16x16x32 would need the A operand twice
        // (register copies, and this path is bound by vector instructions)
        const bf16x4_t a = __builtin_bit_cast(bf16x4_t, make_uint2(a01[m], a23[m]));
        st.o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pHi, st.o[m], 0, 0, 0);
        st.o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pLo, st.o[m], 0, 0, 0);
    }
}

// The INT4 tile's softmax and value update for at most four query columns,
// one score per lane. Only columns 0-3 of the 16-column score product are
// real, so lane (G, n16) of the product holds four real scores when n16 < 4
// and none otherwise. Moving them inside each 16-lane row gives lane
// (G, n16) the score of token 4G + n16/4 and column n16 % 4 (from register
// n16/4 of lane n16 % 4), so each exponential and weight is formed once. The
// state (m, l, bv) is per lane for that column; l and bv are summed over the
// banks and G at the end (q4_state_sum). The weights P' go back to the value
// product's B layout (lane (G, c < 4) takes those of lane (G, 4i + c)), as
// bf16 hi + lo parts. sc: raw products before corr (this lane's column's
// min term); ok: the slot is attended (the caller's mask); vs, vm: the
// lane's token's V scale and min words and their half (vsh = 0 or 16).
__device__ __forceinline__ void q4_softmax_pv_one(const AttnParams &p, const Q4Tile &T, float s, bool ok,
                                                  uint32_t vsw, uint32_t vmw, int vsh, MfmaState<128> &st) {
    if (__any(s > st.m + kLazyLog2)) {  // lazy rescale, as in mfma_block
        const float mn = fmaxf(st.m, col_max(bank_max(s)));
        const float alpha = mn == st.m ? 1.0f : fast_exp2(st.m - mn);  // unchanged (even -inf): 1
        st.l *= alpha;
        st.bv *= alpha;
#pragma unroll
        for (int m = 0; m < 8; ++m) st.o[m] *= alpha;
        st.m = mn;
    }
    const float mref = st.m == -INFINITY ? 0.0f : st.m;  // no token seen yet: weight 0
    const float pr = fast_exp2(s - mref);                 // 0 for a masked slot
    st.l += pr;
    // a masked slot's V parameters may be anything: 0 there
    const float vsc = ok ? f16_bits_to_f((uint16_t)(vsw >> vsh)) : 0.0f;
    const float vmn = ok ? f16_bits_to_f((uint16_t)(vmw >> vsh)) : 0.0f;
    const float pv = pr * vsc;
    st.bv = fmaf(pr, vmn, st.bv);
    // bf16 hi (low half) and lo (high half) of this lane's weight
    const uint32_t h = cvt_pk_bf16(pv, 0.0f);
    const uint32_t hl = cvt_pk_bf16(pv, pv - __uint_as_float(h << 16));
    // lane (G, c) of each row gathers tokens 4G + i from lanes (G, 4i + c)
    const float hf = __uint_as_float(hl);
    const uint32_t t0 = hl;
    const uint32_t t1 = __float_as_uint(__int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(hf), kDppRowShl + 4, 0xf, 0xf, true)));
    const uint32_t t2 = __float_as_uint(__int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(hf), kDppRowShl + 8, 0xf, 0xf, true)));
    const uint32_t t3 = __float_as_uint(__int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(hf), kDppRowShl + 12, 0xf, 0xf, true)));
    const bf16x4_t pHi = __builtin_bit_cast(
        bf16x4_t, make_uint2(__builtin_amdgcn_perm(t1, t0, 0x05040100u), __builtin_amdgcn_perm(t3, t2, 0x05040100u)));
    const bf16x4_t pLo = __builtin_bit_cast(
        bf16x4_t, make_uint2(__builtin_amdgcn_perm(t1, t0, 0x07060302u), __builtin_amdgcn_perm(t3, t2, 0x07060302u)));
    // the value product, as in q4_softmax_pv
    uint32_t a01[8], a23[8];
    auto spread = [](uint32_t x, uint32_t(&dst)[8], int c0) {
        const uint32_t e = x & 0x0f0f0f0fu, o = (x >> 4) & 0x0f0f0f0fu;
        dst[c0 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(e, 512.0f, false));
        dst[c0 + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(e, 512.0f, true));
        dst[c0 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(o, 512.0f, false));
        dst[c0 + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(o, 512.0f, true));
    };
    spread(__builtin_amdgcn_perm(T.vc[1], T.vc[0], 0x05010400u), a01, 0);
    spread(__builtin_amdgcn_perm(T.vc[1], T.vc[0], 0x07030602u), a01, 4);
    spread(__builtin_amdgcn_perm(T.vc[3], T.vc[2], 0x05010400u), a23, 0);
    spread(__builtin_amdgcn_perm(T.vc[3], T.vc[2], 0x07030602u), a23, 4);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const bf16x4_t a = __builtin_bit_cast(bf16x4_t, make_uint2(a01[m], a23[m]));
        st.o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pHi, st.o[m], 0, 0, 0);
        st.o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pLo, st.o[m], 0, 0, 0);
    }
}

// Row sums of an MFMA state at the end of a unit: over the four lanes that
// hold a column (G), and for the INT4 path with at most four columns (one
// score per lane, Q4 == 1) also over a row's four banks.
template <int Q4>
__device__ __forceinline__ float q4_state_sum(float x) {
    if constexpr (Q4 == 1) x = bank_sum(x);
    return col_sum(x);
}

// One (block, kv head) tile. Scores of a full block: s_t = sum_c code_tc *
// (q_c * kscale_c) + sum_c q_c * kmin_c. The products are formed once per
// (column, channel) by the lane that owns them (column 4 pi + G, channels
// 8 n16 ..) and exchanged through LDS into the MFMA B layout; the min term is
// summed per column the same way. A partial last block takes bf16 K from the
// tail row (global, 16 x 128 per sequence and kv head) with plain q.
// masked (uniform): some slot of the tile lies outside a column's range
// (partial block, window, causal columns); every other tile is a full block.
template <int NP>
__device__ __forceinline__ void q4_block(const AttnParams &p, const Q4Tile &T, const Q4Query<NP> &Q, bool masked,
                                         bool full, gu16_t *tail_row, int tok0, int tlo, int thi,
                                         const Column &col, int n16, int G, Q4Lds &L, MfmaState<128> &st) {
    // NP == 1: col is the Column of query column n16 % 4 (one score per lane)
    const int ccol = NP == 1 ? (n16 & 3) : n16;  // the column whose min term this lane adds
    wave_lds_sync();  // the previous tile's reads of L come first (one-wave workgroup)
    const uint32_t sw[4] = {T.ks.x, T.ks.y, T.ks.z, T.ks.w}, mw[4] = {T.km.x, T.km.y, T.km.z, T.km.w};
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
        if (pi >= Q.npass) break;
        const int c = 4 * pi + G;
        uint32_t hi[4], lo[4];
        if (full) {
            float cp = 0.0f, pr[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float q0 = Q.q[pi][2 * k], q1 = Q.q[pi][2 * k + 1];
                // exact products (an fma with -0 added: one mixed-precision
                // instruction per product, fp16 operand widened inside it)
                pr[2 * k] = fmaf(q0, f16_lo(sw[k]), Q.nz);
                pr[2 * k + 1] = fmaf(q1, f16_hi(sw[k]), Q.nz);
                cp = fmaf(q0, f16_lo(mw[k]), cp);
                cp = fmaf(q1, f16_hi(mw[k]), cp);
            }
            // channel order of q4_codes_bf16: pairs (0, 2), (4, 6), (1, 3), (5, 7)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int c0 = (k & 1) * 4 + (k >> 1);  // 0, 4, 1, 5
                const float p0 = pr[c0], p1 = pr[c0 + 2];
                hi[k] = cvt_pk_bf16(p0, p1);
                lo[k] = cvt_pk_bf16(p0 - __uint_as_float(hi[k] << 16), p1 - __uint_as_float(hi[k] & 0xffff0000u));
            }
            L.b[1][c][n16] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            cp = row_sum(cp);  // row G of the wave holds column c's 16 channel chunks
            if (n16 == 0) L.corr[c] = cp;
        } else {  // the tail row's bf16 K in natural channel order
#pragma unroll
            for (int k = 0; k < 4; ++k) hi[k] = cvt_pk_bf16(Q.q[pi][2 * k], Q.q[pi][2 * k + 1]);  // exact
        }
        L.b[0][c][n16] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
    wave_lds_sync();
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
    float corr = 0.0f;
    if (full) {
        corr = L.corr[ccol];
        const uint32_t kcw[4] = {T.kc.x, T.kc.y, T.kc.z, T.kc.w};
        f32x4_t sl = {0.0f, 0.0f, 0.0f, 0.0f};  // hi and lo parts in two chains: half the dependent latency
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8_t a = q4_codes_bf16(kcw[s]);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, L.b[0][n16][4 * G + s]), sc, 0, 0, 0);
            sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, L.b[1][n16][4 * G + s]), sl, 0, 0, 0);
        }
        sc += sl;
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8_t kt = __builtin_bit_cast(bf16x8_t, stream_load16(tail_row + 8 * s));
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, __builtin_bit_cast(bf16x8_t, L.b[0][n16][4 * G + s]), sc, 0, 0, 0);
        }
    }
    if constexpr (NP == 1) {
        // lane (G, n16): token 4G + n16 / 4, column n16 % 4
        float raw = dpp_f<kDppRowShr + 4, 0x2>(sc[0], sc[1]);  // bank 1 takes register 1 of bank 0, ...
        raw = dpp_f<kDppRowShr + 8, 0x4>(raw, sc[2]);
        raw = dpp_f<kDppRowShr + 12, 0x8>(raw, sc[3]);
        float s = (raw + corr) * p.scale_log2;  // log2 units
        bool ok = true;
        if (masked) {  // only the rare masked tiles test positions
            const int tt = 4 * G + (n16 >> 2), tp = tok0 + tt;
            ok = (tt >= tlo) & (tt < thi) & (tp >= col.lo) & (tp < col.hi);
            s = ok ? s : -INFINITY;
        }
        const bool hiword = n16 & 8;
        q4_softmax_pv_one(p, T, s, ok, hiword ? T.vs.y : T.vs.x, hiword ? T.vm.y : T.vm.x, (n16 & 4) * 4, st);
    } else {
        float sv[4];  // scores in log2 units
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = (sc[r] + corr) * p.scale_log2;
        uint2 vs = T.vs, vm = T.vm;
        if (masked) q4_mask(tok0, tlo, thi, col, G, sv, vs, vm);  // only the rare masked tiles test positions
        q4_softmax_pv(p, T, sv, vs, vm, st);
    }
}

// Fused append of a decode step with one new token per sequence, INT4 pool
// (head_dim 128): the same coding as the append kernel. The token's V row
// is coded per token; its K row goes to slot t of the sequence's bf16 tail,
// and when it is the block's 16th token the block's K is coded per channel
// from the tail rows. pid: the block that receives the token.
__device__ __forceinline__ void q4_append_token(const AttnParams &p, int b, int kvh, int slot, int pid, int t,
                                                int lane) {
    constexpr int hd = 64;  // 32-bit words of a 128-channel bf16 row
    const size_t src = ((size_t)b * p.n_kv + kvh) * hd;
    const uint32_t vw = reinterpret_cast<const uint32_t *>(p.v_new)[src + lane];
    const uint32_t kw = reinterpret_cast<const uint32_t *>(p.k_new)[src + lane];
    const size_t tile = (size_t)pid * p.n_kv + kvh, row = tile * kBlock + t;
    code_v_row(vw, true, p.pool.vq + row * hd, p.pool.vs + row, p.pool.vm + row, lane);
    uint32_t *tail = reinterpret_cast<uint32_t *>(p.pool.ktail) + ((size_t)slot * p.n_kv + kvh) * kBlock * hd;
    tail[t * hd + lane] = kw;
    if (t == kBlock - 1) {
        uint32_t w[kBlock];
#pragma unroll
        for (int tt = 0; tt < kBlock - 1; ++tt) w[tt] = tail[tt * hd + lane];
        w[kBlock - 1] = kw;
        code_k_block(w, true, p.pool.kq + tile * kBlock * hd, p.pool.ks + tile * 128, p.pool.km + tile * 128, lane,
                     hd);
    }
}

// Blocks [j0, j1) (at most kSidsWindow) of sequence b, kv head kvh, column
// tile ct; init: start a new state, else continue st. FLAT: tiles addressed
// as in q4_fetch_flat (the launch checks the pool's span).
template <int D, int NP, bool FLAT>
__device__ __forceinline__ void q4_segment(const AttnParams &p, int b, int kvh, int ct, const Column &col,
                                           const SeqRange &r, int j0, int j1, int lane, MfmaState<D> &st, bool &bad,
                                           int *sids, bool init, Pace pace = Pace{0, INT_MAX, INT_MAX, INT_MAX}) {
    static_assert(D == 128, "INT4 MFMA path is built for head_dim 128");
    const int n16 = lane & 15, G = lane >> 4;
    // The segment's first global loads (the sequence's tail slot, the query,
    // the block ids) go out together and are waited on once, in the id
    // staging: values loaded here are used only after it.
    const int slot_v = p.seq_slots ? p.seq_slots[b] : b;  // the same value in every lane
    auto take_slot = [&]() {
        int s = uniform(slot_v);
        if (s < 0 || s >= p.max_seqs) {
            bad = true;
            s = -1;
        }
        return s;
    };
    // query of the product layout: column 4 pi + G of this column tile,
    // channels 8 n16 .. 8 n16 + 7
    Q4Query<NP> Q;
    Q.npass = min((min(p.ncols - ct * 16, 16) + 3) / 4, NP);
    Q.nz = -0.0f;
    asm("" : "+v"(Q.nz));
    uint4 qraw[NP];
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
        const Column cq = column_of(p, b, kvh, ct, 4 * pi + G, r);
        qraw[pi] = make_uint4(0, 0, 0, 0);
        if (pi < Q.npass && cq.valid)
            qraw[pi] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.q) + cq.row * 128 + 8 * n16);
    }
    if (init) {
#pragma unroll
        for (int m = 0; m < 8; ++m) st.o[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        st.m = -INFINITY;
        st.l = 0.0f;
        st.bv = 0.0f;
    }
    if (j0 >= j1) {
        take_slot();
        return;
    }
    __shared__ Q4Lds L;
    wave_lds_sync();  // this wave's reads of L in the previous segment come first (one-wave workgroup)
    // columns past the passes are never written: zero B rows (padded columns)
    for (int i = lane; i < (16 - 4 * Q.npass) * 17; i += 64) {
        const int c = 4 * Q.npass + i / 17, k = i % 17;
        L.b[0][c][k] = make_uint4(0, 0, 0, 0);
        L.b[1][c][k] = make_uint4(0, 0, 0, 0);
        if (k == 0) L.corr[c] = 0.0f;
    }
    // every staged id is a valid block (bad ones were replaced by 0)
    const BlockIds ids = stage_checked_block_ids(p, b, j0, j1, lane, sids, bad);
    int slot = take_slot();
    const bool slot_bad = slot < 0;
    slot = slot_bad ? 0 : slot;
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
        const uint32_t w[4] = {qraw[pi].x, qraw[pi].y, qraw[pi].z, qraw[pi].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            Q.q[pi][2 * k] = bf16_lo(w[k]);
            Q.q[pi][2 * k + 1] = bf16_hi(w[k]);
        }
    }
    auto is_full = [&](int j) { return (j + 1) * kBlock <= r.n; };
    gu16_t *tail_row = global_u16(p.pool.ktail) + (((size_t)slot * p.n_kv + kvh) * kBlock + n16) * 128 + 32 * G;
    // blocks [jA, jB) lie inside every column's range (needs_mask is false
    // there); a partial or last block never does
    const int jA = (r.all_lo + kBlock - 1) / kBlock, jB = r.all_hi > 0 ? r.all_hi / kBlock : 0;
    // the column whose scores this lane masks: n16 % 4 with one score per lane
    const Column colq = NP == 1 ? column_of(p, b, kvh, ct, n16 & 3, r) : col;
    auto step = [&](const Q4Tile &T, int j) {
        const int tok0 = j * kBlock;
        const bool masked = j < jA || j >= jB;
        const int tlo = max(r.lo - tok0, 0), thi = min(r.hi - tok0, kBlock);
        q4_block<NP>(p, T, Q, masked, !masked || is_full(j), tail_row, tok0, tlo, thi, colq, n16, G, L, st);
        pace_tick(pace, j);
    };
    // Fused append (decode step, one new token at position r.n - 1): the
    // segment that ends with the sequence's last block codes the token into
    // the pool, as the append kernel would: unless the sequence's length or
    // tail slot is invalid, or its block id for the token. The first tile's
    // loads are issued before that work (unless the first tile is the last
    // block), and every load of the last block's tile waits for the coded
    // token's stores.
    const bool append = p.k_new && ct == 0 && j1 == r.blk_lo + r.nblk && !r.bad && !slot_bad;
    bool appended = false;
    const Q4Flat flat = FLAT ? q4_flat(p) : Q4Flat{};
    // The loop issues the same loads every iteration (so the compiler's waits
    // cover exactly the tile in use); past the end they go through empty
    // descriptors, which read nothing.
    auto fetch = [&](int j, Q4Tile &T) {
        const bool past = j >= j1;
        const int jc = past ? j1 - 1 : j;
        if (appended && jc == j1 - 1) __builtin_amdgcn_s_waitcnt(0);
        if constexpr (FLAT)
            q4_fetch_flat(flat, (uint32_t)(ids.id(jc) * p.n_kv + kvh), n16, G, T, past);
        else
            q4_fetch(p, ids.id(jc), kvh, n16, G, T, past);
    };
    Q4Tile A, B;
    if (!append || j0 < j1 - 1) fetch(j0, A);
    if (append) {
        const int pid = ids.last;  // the table's entry as read (a bad one is staged as 0)
        if (pid >= 0 && pid < p.num_blocks) q4_append_token(p, b, kvh, slot, pid, (r.n - 1) % kBlock, lane);
        appended = true;
        if (j0 == j1 - 1) fetch(j0, A);
    }
    // one tile in flight ahead of the one in use
    for (int j = j0; j < j1; j += 2) {
        fetch(j + 1, B);
        step(A, j);
        if (j + 1 >= j1) break;
        fetch(j + 2, A);
        step(B, j + 1);
    }
}

// Column tiles ct0 .. ct0 + CT - 1 of kv head kvh (col[c], st[c]; CT > 1 on
// the bf16 path only). Only the unit holding column tile 0 stores the fused
// append's rows, so that each new row is written once. KEEP: ordinary loads
// (the launch sets it when a kv head's columns take several units, each
// reading every K/V tile: the tiles then stay in the caches for the other
// units, which read them about the same time; 8B shape, 16 query tokens:
// 286 -> 256 us; with one unit per kv head they cost 4 %). FLAT: INT4 tiles
// addressed through one descriptor (q4_fetch_flat).
template <int D, int Q4, int CT, bool KEEP, bool FLAT>
__device__ __forceinline__ void run_segment(const AttnParams &p, int b, int kvh, int ct0, const Column *col,
                                            const SeqRange &r, int j0, int j1, int lane, MfmaState<D> *st, bool &bad,
                                            int *sids, Pace pace = Pace{0, INT_MAX, INT_MAX, INT_MAX}) {
    if constexpr (Q4 > 0) {
        static_assert(CT == 1, "the INT4 path takes one column tile per unit");
        run_pieces(j0, j1, [&](int c0, int c1, bool init) {
            static_assert(!KEEP, "the INT4 path streams its tiles");
            q4_segment<D, Q4, FLAT>(p, b, kvh, ct0, col[0], r, c0, c1, lane, st[0], bad, sids, init, pace);
        });
    } else {
        run_pieces(j0, j1, [&](int c0, int c1, bool init) {
            bf16_segment_ct<D, CT, KEEP>(p, b, kvh, col, r, c0, c1, lane, st, bad, ct0 == 0, sids, init, pace);
        });
    }
}

// Fixed-split schedule: grid (max_splits, n_kv, batch).
// Two resident waves per SIMD: the register budget the kernels are written to
// (no spills; the INT4 path would otherwise take 1 wave per SIMD).
#define KV_MFMA_WAVES __attribute__((amdgpu_waves_per_eu(2)))

// Work unit u of a sequence: kv head u / groups, column tiles CT * (u % groups)
// .. + CT - 1 (groups = units / n_kv).
template <int D, int Q4, int CT, bool KEEP = false, bool FLAT = false>
__global__ __launch_bounds__(64) KV_MFMA_WAVES void attn_mfma_kernel(AttnParams p) {
    extern __shared__ int sids[];  // [min(split_blocks, kSidsWindow)] staged block ids
    const int lane = threadIdx.x, n16 = lane & 15, G = lane >> 4;
    const int split = blockIdx.x, unit = blockIdx.y, b = blockIdx.z;
    const int cgroups = p.units / p.n_kv;
    const int kvh = unit / cgroups, ct0 = (unit % cgroups) * CT;
    SplitWork w;
    if (!split_work(p, b, split, w)) return;
    bool bad = w.r.bad;
    Column col[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) col[c] = column_of(p, b, kvh, ct0 + c, n16, w.r);
    MfmaState<D> st[CT];
    run_segment<D, Q4, CT, KEEP, FLAT>(p, b, kvh, ct0, col, w.r, w.j0, w.j1, lane, st, bad, sids);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const float l = q4_state_sum<Q4>(st[c].l), bv = q4_state_sum<Q4>(st[c].bv);
        if (col[c].valid) {
            float res[D / 4];
            mfma_gather_run<D>(st[c], bv, res);
            store_result(p, col[c].row, split, w.r.nsplit, G * (D / 4), res, D / 4, st[c].m, l, bad, G == 0);
        }
    }
}

// Balanced schedule. The attended (sequence, unit, block) tiles are laid out
// in sequence-major, unit, block order on a cost axis where every (sequence,
// unit) pair also takes seg_cost positions after its tiles: the start of a
// segment (its block ids, query and first tile) costs about that many tiles
// of time. Workgroup w of the persistent grid takes the positions of its
// share (Shares: total / grid each, one more for the first total % grid) and
// works the tiles among them.
// A workgroup walks its range one pair at a time; a pair whose tiles all
// fall in its range writes the output directly. Otherwise the piece leaves a
// partial in slot 0 of the workgroup's two workspace slots when the pair
// started before the range (only a workgroup's first piece can), else in
// slot 1 (the pair goes on past the range: only its last piece can);
// attn_merge_balanced_rows_kernel (or _unit_kernel) combines them.
// Workgroup 0 also stores the prefix sums for the merge.
// Dynamic LDS of the balanced kernels: the prefix sums [batch + 1]; for
// batches of at most kCtxInLds sequences their attended lengths [batch]
// (read once by the prefix pass: a segment then takes its sequence's length
// from LDS, not from a global load that would wait behind the previous
// segment's result stores); then the staged block ids.
constexpr int kCtxInLds = 512;
__host__ __device__ inline int balanced_lds_ints(int batch, int max_ids) {
    return batch + 1 + (batch <= kCtxInLds ? batch : 0) + (max_ids < kSidsWindow ? max_ids : kSidsWindow);
}
struct BalancedLds {
    int *pre, *ctx, *sids;  // ctx: null for larger batches
};
__device__ __forceinline__ BalancedLds balanced_lds(const AttnParams &p, int *base) {
    BalancedLds l;
    l.pre = base;
    l.ctx = p.batch <= kCtxInLds ? base + p.batch + 1 : nullptr;
    l.sids = base + p.batch + 1 + (p.batch <= kCtxInLds ? p.batch : 0);
    return l;
}
// Attended length of sequence b in a balanced kernel.
__device__ __forceinline__ int balanced_ctx(const AttnParams &p, const BalancedLds &l, int b) {
    return l.ctx ? l.ctx[b] : ctx_of(p, b);
}

__device__ __forceinline__ int balanced_prefix(const AttnParams &p, const BalancedLds &l, int lane) {
    // pre[b] = positions of sequences < b per unit (attended blocks plus
    // seg_cost for a sequence with any), in LDS; returns pre[batch]
    int *pre = l.pre;
    int carry = 0;
    if (lane == 0) pre[0] = 0;
    for (int base = 0; base < p.batch; base += 64) {
        const int b = base + lane;
        int nb = 0;
        if (b < p.batch) {
            const int ctx = ctx_of(p, b);
            if (l.ctx) l.ctx[b] = ctx;
            const SeqRange r = seq_range(ctx, p.max_blocks, p.window, p.split_blocks, p.max_splits, p.q_len);
            nb = r.nblk > 0 ? r.nblk + p.seg_cost : 0;
        }
        // inclusive wave scan
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int x = __shfl_up(nb, o);
            if (lane >= o) nb += x;
        }
        if (b < p.batch) pre[b + 1] = carry + nb;
        carry += __shfl(nb, 63);
    }
    __syncthreads();
    return carry;
}

// Largest i < n with mult * v[i] <= t, for v in LDS, non-decreasing, with
// mult * v[0] <= t. The whole wave searches: each round tests 64 evenly
// spaced candidates at once (one LDS read per lane and a ballot) and narrows
// the range 64-fold, so up to 64 entries take one round and up to 4096 two,
// instead of a chain of log2(n) dependent LDS reads (about 1.3 us at the start
// of the INT4 8B-shaped kernel). The result is uniform.
__device__ __forceinline__ int last_le(const int *v, int n, long mult, long t, int lane) {
    int lo = 0;
    for (;;) {
        const int step = n <= 64 ? 1 : (n + 63) >> 6;
        const bool in = lane * step < n;
        const int x = in ? v[lo + lane * step] : 0;
        const unsigned long long le = __ballot(in && (long)x * mult <= t);
        const int k = __popcll(le) - 1;  // candidates 0 .. k pass (lane 0 always)
        lo += k * step;
        if (step == 1) return uniform(lo);
        n = min(step, n - k * step);
    }
}
// The sequence holding share position t of a balanced kernel.
__device__ __forceinline__ int sequence_at(const int *pre, int batch, int units, long t, int lane) {
    return last_le(pre, batch, units, t, lane);
}

// Work unit of share position t inside the pair run starting at pair0 (span
// positions per unit): in 32 bits when the sequence's positions fit them.
__device__ __forceinline__ int unit_at(long t, long pair0, int span, int units) {
    if ((long)units * span <= INT_MAX) return (int)(t - pair0) / span;
    return (int)((t - pair0) / span);
}

// The INT4 kernel with one score per lane (at most four query columns) runs
// three waves per SIMD (168 registers; the few spilled ones are stored and
// reloaded once per segment, outside the tile loop): its waves are bound by
// the dependency chains inside a tile, which the third wave covers (8B shape
// 55 -> 52 us, the merge of the larger grid 4.9 -> 5.8 us). The others stay at two.
#define KV_BALANCED_WAVES(Q4) __attribute__((amdgpu_waves_per_eu((Q4) == 1 ? 3 : 2)))
constexpr int kBalancedWavesQ4One = 3;

template <int D, int Q4, int CT, bool KEEP = false, bool FLAT = false>
__global__ __launch_bounds__(64) KV_BALANCED_WAVES(Q4) void attn_mfma_balanced_kernel(AttnParams p) {
    extern __shared__ int lds_ints[];  // BalancedLds
    const BalancedLds bl = balanced_lds(p, lds_ints);
    int *pre = bl.pre, *sids = bl.sids;
    const int lane = threadIdx.x, n16 = lane & 15, G = lane >> 4;
    // The INT4 path is bound by vector instructions: there the sequence
    // search and everything derived from it are moved to scalar registers.
    // The bf16 path keeps them in vector registers (measured faster: the
    // scalar form runs out of scalar registers there).
    const int npos = Q4 ? uniform(balanced_prefix(p, bl, lane)) : balanced_prefix(p, bl, lane);
    if (blockIdx.x == 0)
        for (int i = lane; i <= p.batch; i += 64) p.ws_prefix[i] = pre[i];
    const long total = (long)npos * p.units;
    const auto sh = split_of<Q4 != 0>(total, p.n_wg);
    const int wg = sh.share_of(blockIdx.x);
    const long s = sh.start(wg);
    const long e = sh.start(wg + 1);
    // paced on INT4 pools only (measured: INT4 60 vs 62-63.5 us on the 8B
    // shape; the bf16 kernels unchanged, and without it they keep fewer
    // registers)
    Pace pace = pace_for(Q4 && p.pace ? e - s : 0);
    pace_set(pace, 0);
    for (long t = s; t < e;) {
        auto pre_s = [&](int i) { return Q4 ? uniform(pre[i]) : pre[i]; };
        const int b = sequence_at(pre, p.batch, p.units, t, lane);
        const int pb = pre_s(b);
        const int ctx = balanced_ctx(p, bl, b);
        const int span = pre_s(b + 1) - pb;  // nb + seg_cost positions per unit
        const int nb = span - p.seg_cost;
        const long pair0 = (long)pb * p.units;
        const int unit = unit_at(t, pair0, span, p.units);
        const long pair_t = pair0 + (long)unit * span;  // position of the pair's first tile
        const int jr = (int)(t - pair_t);
        if (jr >= nb) {  // in the pair's start cost: go on at the next pair
            t = pair_t + span;
            continue;
        }
        const int cgroups = p.units / p.n_kv;
        const int kvh = unit / cgroups, ct0 = (unit % cgroups) * CT;
        const long seg_end = min(e, pair_t + nb);
        const int cnt = (int)(seg_end - t);
        const SeqRange r = seq_range(Q4 ? uniform(ctx) : ctx, p.max_blocks, p.window, p.split_blocks, p.max_splits,
                                     p.q_len);
        bool bad = r.bad;
        Column col[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) col[c] = column_of(p, b, kvh, ct0 + c, n16, r);
        MfmaState<D> st[CT];
        // block j of this piece sits at share position (t - s) + j - (blk_lo + jr)
        pace.base = (int)(t - s) - (r.blk_lo + jr);
        pace_set(pace, (int)(t - s));
        run_segment<D, Q4, CT, KEEP, FLAT>(p, b, kvh, ct0, col, r, r.blk_lo + jr, r.blk_lo + jr + cnt, lane, st, bad,
                                           sids, pace);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const float l = q4_state_sum<Q4>(st[c].l), bv = q4_state_sum<Q4>(st[c].bv);
            if (col[c].valid) {
                const float nan = __uint_as_float(0x7fc00000u);
                // a bad sequence's row is NaN: the NaN enters through the
                // term every output value adds (no select per value)
                float res[D / 4];
                mfma_gather_run<D>(st[c], bad ? nan : bv, res);
                if (jr == 0 && cnt == nb) {
                    float *dst = p.out + col[c].row * D + G * (D / 4);
                    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
                    for (int k = 0; k < D / 4; ++k) dst[k] = res[k] * inv;
                } else {
                    // slot row: column tile c of the unit at 16 c + n16
                    const int slot = jr > 0 ? 0 : 1;
                    const size_t row = ((size_t)wg * 2 + slot) * p.slot_cols + c * 16 + n16;
                    float *dst = p.ws_o + row * D + G * (D / 4);
#pragma unroll
                    for (int k = 0; k < D / 4; ++k) dst[k] = res[k];
                    if (G == 0) {
                        p.ws_ml[row * 2] = st[c].m;
                        p.ws_ml[row * 2 + 1] = bad ? nan : l;
                    }
                }
            }
        }
        t = seg_end;
    }
}

// ---------------------------------------------------------------------------
// wide work units (bf16, many query columns per kv head)
//
// A unit of CT W column tiles is one workgroup of W waves (CT column tiles
// per wave, as in bf16_segment_ct): the waves load each (block, kv head) K/V
// tile once, together, into LDS and each reads it back in the MFMA operand
// layout. So a K/V tile leaves HBM once per CT W column tiles.
// Three LDS tile buffers: the next two tiles' global loads are in flight
// while the current one is used, and one barrier per tile orders them.
// ---------------------------------------------------------------------------

// One K/V tile in LDS: 16 rows of D bf16 for K, then for V, in 16-byte
// slots. Slot column c of row r sits at position c ^ (r % SPR) of the row, so
// that the 16 lanes of one operand read (16 rows of one column, or 16
// columns of one row) fall on distinct banks.
template <int D>
struct TileLds {
    static constexpr int SPR = D * 2 / 16;          // slots per row
    static constexpr int SLOTS = 2 * kBlock * SPR;  // K rows, then V rows
    u32x4_t slot[SLOTS];
    __device__ __forceinline__ static int at(int which, int row, int col) {
        return (which * kBlock + row) * SPR + (col ^ (row % SPR));
    }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Column tiles per wave of the wide kernels (units of 4 or 8 column tiles).
// One per wave (4 or 8 waves, no spilled registers) measured slower than two
// (the K/V operands read from LDS serve both): 8B shape, 16 query tokens 218
// vs 203 us, 32 tokens 384 vs 326 us.
constexpr int kWideCT = 2;
// K/V tile buffers in LDS per wide unit (two tiles in flight).
constexpr int kWideBufs = 3;

// Wait until at most N of this wave's vector-memory operations are
// outstanding (N < 16; the LDS and export counters are not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt field of s_waitcnt");
    __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier of the wide tile loop. Each wave has already waited for
// its own tile loads (wait_vm); here it waits for its LDS reads (so no wave
// refills a buffer another is still reading) and meets the others. Unlike
// __syncthreads() it carries no memory fence: a workgroup fence waits for
// every outstanding global-to-LDS load, which would drain the second tile in
// flight. The scheduling barriers keep the compiler from moving instructions
// across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited on
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// Issues this wave's share of one tile's loads straight into LDS
// (global_load_lds, 16 bytes per lane): instruction q of the tile fills slots
// [64 q, 64 q + 64), wave w issues q = w, w + W, ... Rows of the step's new
// tokens (slots from newpos on) come from k_new / v_new. Complete after the
// wave's vector-memory counter reaches 0.
// Slots of a K/V tile in LDS that wave `wave` of a wide unit loads: slot
// q * 64 + lane for q = wave, wave + W, ...; the first TS slots are K, the
// rest V. Byte offset of each of this lane's slots within its (block, kv
// head) K or V tile; they do not change from tile to tile.
template <int D, int W>
struct WideSlots {
    static constexpr int SPR = TileLds<D>::SPR, NI = TileLds<D>::SLOTS / 64, TS = kBlock * SPR,
                         NQ = (NI + W - 1) / W;  // a wave's slot groups (waves past NI - 1 have none)
    static_assert(TS % 64 == 0, "a wave's 64 slots lie in the K or in the V tile");
    uint32_t off[NQ];  // row * D * 2 + 16-byte column * 16
    int wave;          // uniform
};

template <int D, int W>
__device__ __forceinline__ WideSlots<D, W> wide_slots(int wave, int lane) {
    using S = WideSlots<D, W>;
    S w;
    w.wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int k = 0; k < S::NQ; ++k) {
        const uint32_t rem = (uint32_t)((w.wave + k * W) * 64 % S::TS) + (uint32_t)lane;
        const uint32_t row = rem / S::SPR, col = (rem % S::SPR) ^ (row % S::SPR);
        w.off[k] = (row * D + col * 8) * 2;
    }
    return w;
}

// Issue the global-to-LDS loads of this wave's slots of one (block pid, kv
// head) K/V tile into t. The XOR swizzle of TileLds is applied on the global
// side. Decode step with the append fused: rows of the step's new tokens
// (slots from newpos on) come from k_new / v_new. Complete after the wave's
// vector-memory counter reaches 0.
template <int D, int W>
__device__ __forceinline__ void wide_issue(const AttnParams &p, int pid, int kvh, int b, int newpos,
                                           const WideSlots<D, W> &S, TileLds<D> &t) {
    using WS = WideSlots<D, W>;
    typedef const __attribute__((address_space(1))) char gchar_t;
    // the tile's base (uniform), and each lane's fixed offset within it
    const size_t tile = ((size_t)pid * p.n_kv + kvh) * kBlock * D * 2;
    gchar_t *kt = (gchar_t *)(p.pool.k) + tile, *vt = (gchar_t *)(p.pool.v) + tile;
    // only a tile that holds new tokens tests rows (newpos is uniform: in a
    // scalar register the test is a branch, not an exec mask)
    newpos = __builtin_amdgcn_readfirstlane(newpos);
    const bool fresh = newpos < kBlock && newpos + p.ctx_add > 0;
    if (!fresh) {
        // the common case: uniform base plus a 32-bit lane offset, the form
        // with the base in scalar registers (no per-lane address arithmetic)
#pragma unroll
        for (int k = 0; k < WS::NQ; ++k) {
            const int q = S.wave + k * W;
            if (WS::NI % W != 0 && q >= WS::NI) break;  // uniform
            gchar_t *src = (q * 64 >= WS::TS ? vt : kt) + S.off[k];  // uniform base: K or V
            __builtin_amdgcn_global_load_lds(src, (lds_void_t *)&t.slot[q * 64], 16, 0, kLoadStream);
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < WS::NQ; ++k) {
        const int q = S.wave + k * W;
        if (WS::NI % W != 0 && q >= WS::NI) break;  // uniform
        const bool v = q * 64 >= WS::TS;  // uniform: K or V
        gchar_t *src = (v ? vt : kt) + S.off[k];
        const int row = (int)(S.off[k] / (D * 2));
        if (row >= newpos && row < newpos + p.ctx_add)
            src = (gchar_t *)(v ? p.v_new : p.k_new) +
                  (((size_t)b * p.ctx_add + (row - newpos)) * p.n_kv + kvh) * D * 2 + S.off[k] % (D * 2);
        __builtin_amdgcn_global_load_lds(src, (lds_void_t *)&t.slot[q * 64], 16, 0, kLoadStream);
    }
}

// The MFMA operands of a tile in LDS (layout of MfmaTile).
template <int D>
__device__ __forceinline__ void wide_operands(const TileLds<D> &t, int n16, int G, MfmaTile<D> &T) {
    constexpr int KS = D / 32, VC = D / 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) T.k[s] = __builtin_bit_cast(bf16x8_t, t.slot[TileLds<D>::at(0, n16, 4 * s + G)]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * G + i;
        if constexpr (VC == 8) {
            const u32x4_t v = t.slot[TileLds<D>::at(1, r, n16)];
            T.v[i][0] = v[0];
            T.v[i][1] = v[1];
            T.v[i][2] = v[2];
            T.v[i][3] = v[3];
        } else {  // 8 bytes: half n16 & 1 of slot n16 / 2
            const u32x2_t v = *reinterpret_cast<const u32x2_t *>(
                reinterpret_cast<const uint8_t *>(&t.slot[TileLds<D>::at(1, r, n16 >> 1)]) + (n16 & 1) * 8);
            T.v[i][0] = v[0];
            T.v[i][1] = v[1];
        }
    }
}

// Blocks [j0, j1) (at most kSidsWindow) of sequence b, kv head kvh for this
// wave's CT column tiles (col, st; init: start a new state). Every wave of
// the workgroup calls it with the same blocks.
template <int D, int W, int CT>
__device__ __forceinline__ void wide_segment(const AttnParams &p, int b, int kvh, const Column *col,
                                             const SeqRange &r, int j0, int j1, int tid, MfmaState<D> *st, bool &bad,
                                             bool write_new, int *sids, TileLds<D> (&tl)[kWideBufs], bool init) {
    constexpr int KS = D / 32, MS = D / 16;
    const int lane = tid & 63, n16 = lane & 15, G = lane >> 4;
    bf16x8_t qB[CT][KS];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col[c].valid)
                v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.q) + col[c].row * D + s * 32 +
                                                     8 * G);
            qB[c][s] = __builtin_bit_cast(bf16x8_t, v);
        }
    if (init) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
            for (int m = 0; m < MS; ++m) st[c].o[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            st[c].m = -INFINITY;
            st[c].l = 0.0f;
            st[c].bv = 0.0f;
        }
    }
    if (j0 >= j1) return;
    // block ids of the piece, staged by the whole workgroup
    const int32_t *row_ids = p.tables + (size_t)b * p.max_blocks;
    __syncthreads();  // earlier reads of sids and of the tile buffers are done
    for (int i = tid; i < j1 - j0; i += 64 * W) sids[i] = row_ids[j0 + i];
    __syncthreads();
    auto pid_of = [&](int j) {
        int pid = __builtin_amdgcn_readfirstlane(sids[j - j0]);
        if (pid < 0 || pid >= p.num_blocks) {
            bad = true;
            pid = 0;
        }
        return pid;
    };
    const int L0 = p.k_new ? r.n - p.ctx_add : INT_MAX;
    if (write_new && tid < 64 && L0 != INT_MAX) {
        for (int j = max(j0, L0 / kBlock); j < j1; ++j) {
            const int id = __builtin_amdgcn_readfirstlane(sids[j - j0]);
            if (id >= 0 && id < p.num_blocks) store_new_rows<D>(p, b, kvh, id, L0 - j * kBlock, lane);
        }
    }
    auto newpos_of = [&](int j) { return L0 == INT_MAX ? kBlock : min(L0 - j * kBlock, kBlock); };
    const WideSlots<D, W> slots = wide_slots<D, W>(tid >> 6, lane);
    // Three tile buffers, two tiles in flight: tile j is used while tiles j + 1
    // and j + 2 load. Each wave issues kAhead loads per tile (when the waves
    // share the slot groups evenly), so waiting until at most kAhead of its
    // loads are outstanding means all but the newest tile have landed; with
    // an uneven share every wait is a full one.
    using WS = WideSlots<D, W>;
    constexpr int kAhead = WS::NI % W == 0 ? WS::NQ : 0;
    wide_issue<D, W>(p, pid_of(j0), kvh, b, newpos_of(j0), slots, tl[0]);
    if (j0 + 1 < j1) {
        wide_issue<D, W>(p, pid_of(j0 + 1), kvh, b, newpos_of(j0 + 1), slots, tl[1]);
        wait_vm<kAhead>();  // tile j0 is in LDS
    } else {
        wait_vm<0>();
    }
    lds_barrier();
    // one step per buffer, unrolled, so that every LDS address is a
    // constant offset from a per-lane base
    auto step = [&](int j, const TileLds<D> &use, TileLds<D> &fill) {
        // tile j + 2 goes into the buffer tile j - 1 used (every wave passed
        // the barrier after using it)
        if (j + 2 < j1) wide_issue<D, W>(p, pid_of(j + 2), kvh, b, newpos_of(j + 2), slots, fill);
        MfmaTile<D> T;
        wide_operands<D>(use, n16, G, T);
        const int tok0 = j * kBlock;
        const int tlo = max(r.lo - tok0, 0), thi = min(r.hi - tok0, kBlock);
        mfma_block_ct<D, CT>(p, T, qB, tok0, tlo, thi, needs_mask(tok0, r), col, G, st);
        if (j + 2 < j1)
            wait_vm<kAhead>();  // tile j + 1 has landed
        else
            wait_vm<0>();
        lds_barrier();
    };
    static_assert(kWideBufs == 3, "the loop below cycles through three buffers");
    for (int j = j0; j < j1; j += 3) {
        step(j, tl[0], tl[2]);
        if (j + 1 >= j1) break;
        step(j + 1, tl[1], tl[0]);
        if (j + 2 >= j1) break;
        step(j + 2, tl[2], tl[1]);
    }
}

// Balanced schedule over wide units: as attn_mfma_balanced_kernel, with one
// workgroup of W waves per share; wave w takes column tiles CT w .. CT w +
// CT - 1 of the unit. Partial slots hold the unit's 16 CT W columns (row
// 16 c + n16 for the unit's column tile c).
template <int D, int W, int CT>
__global__ __launch_bounds__(64 * W) KV_MFMA_WAVES void attn_mfma_wide_kernel(AttnParams p) {
    extern __shared__ int lds_ints[];  // BalancedLds
    const BalancedLds bl = balanced_lds(p, lds_ints);
    int *pre = bl.pre, *sids = bl.sids;
    __shared__ TileLds<D> tl[kWideBufs];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n16 = lane & 15, G = lane >> 4;
    // every wave computes the same sums (identical LDS writes); the sequence
    // search and what derives from it are kept in scalar registers, so the
    // tile loop's bounds and masks are uniform branches
    const int npos = uniform(balanced_prefix(p, bl, lane));
    if (blockIdx.x == 0 && wave == 0)
        for (int i = lane; i <= p.batch; i += 64) p.ws_prefix[i] = pre[i];
    const long total = (long)npos * p.units;
    const Shares sh = shares_of(total, p.n_wg);
    const int wg = sh.share_of(blockIdx.x);
    const long s = sh.start(wg);
    const long e = sh.start(wg + 1);
    for (long t = s; t < e;) {
        const int b = sequence_at(pre, p.batch, p.units, t, lane);
        const int pb = uniform(pre[b]);
        const int span = uniform(pre[b + 1]) - pb;
        const int nb = span - p.seg_cost;
        const long pair0 = (long)pb * p.units;
        const int unit = unit_at(t, pair0, span, p.units);
        const long pair_t = pair0 + (long)unit * span;
        const int jr = (int)(t - pair_t);
        if (jr >= nb) {
            t = pair_t + span;
            continue;
        }
        const int cgroups = p.units / p.n_kv;
        const int kvh = unit / cgroups, cu = (unit % cgroups) * p.ctw;  // first column tile of the unit
        const long seg_end = min(e, pair_t + nb);
        const int cnt = (int)(seg_end - t);
        const SeqRange r =
            seq_range(uniform(balanced_ctx(p, bl, b)), p.max_blocks, p.window, p.split_blocks, p.max_splits, p.q_len);
        bool bad = r.bad;
        Column col[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) col[c] = column_of(p, b, kvh, cu + CT * wave + c, n16, r);
        MfmaState<D> st[CT];
        run_pieces(r.blk_lo + jr, r.blk_lo + jr + cnt, [&](int c0, int c1, bool init) {
            wide_segment<D, W, CT>(p, b, kvh, col, r, c0, c1, tid, st, bad, cu == 0, sids, tl, init);
        });
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const float l = col_sum(st[c].l), bv = col_sum(st[c].bv);
            if (col[c].valid) {
                const float nan = __uint_as_float(0x7fc00000u);
                float res[D / 4];
                mfma_gather_run<D>(st[c], bad ? nan : bv, res);  // NaN row for a bad sequence, as above
                if (jr == 0 && cnt == nb) {
                    float *dst = p.out + col[c].row * D + G * (D / 4);
                    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
                    for (int k = 0; k < D / 4; ++k) dst[k] = res[k] * inv;
                } else {
                    const int slot = jr > 0 ? 0 : 1;
                    const size_t row = ((size_t)wg * 2 + slot) * p.slot_cols + (CT * wave + c) * 16 + n16;
                    float *dst = p.ws_o + row * D + G * (D / 4);
#pragma unroll
                    for (int k = 0; k < D / 4; ++k) dst[k] = res[k];
                    if (G == 0) {
                        p.ws_ml[row * 2] = st[c].m;
                        p.ws_ml[row * 2 + 1] = bad ? nan : l;
                    }
                }
            }
        }
        t = seg_end;
    }
}

// ---------------------------------------------------------------------------
// shared-prefix decode attention (bf16 MFMA path)
//
// Sequences of a prefix group name the same physical blocks for their first
// blocks[i] logical blocks. A prefix work item streams a chunk of those
// shared tiles once for the whole group: its columns are the group members'
// query rows (member k, head hq -> column k * group + hq), so one tile
// product serves every member. Suffix work items are the ordinary split work
// on each sequence's own blocks after its prefix. Every row that has a prefix
// keeps its results as partials (slots: the group's prefix chunks first, then
// the sequence's suffix splits) and attn_merge_shared_kernel combines them.
// ---------------------------------------------------------------------------

// Group holding sequence b, or -1.
__device__ __forceinline__ int prefix_group_of(const PrefixArgs &g, int b) {
    if (g.n_groups == 0 || b < g.start[0]) return -1;
    int lo = 0, hi = g.n_groups - 1;  // largest i with start[i] <= b
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (g.start[mid] <= b)
            lo = mid;
        else
            hi = mid - 1;
    }
    return b < g.start[lo + 1] ? lo : -1;
}

// Slots of one row: prefix chunks and suffix splits of sequence b with n
// attended tokens and P shared blocks (bad: the length is out of range or
// shorter than the prefix).
struct SharedRow {
    int nchunk, nsplit, blk_hi;
    bool bad;
};
__device__ __forceinline__ SharedRow shared_row(const AttnParams &p, int n, int P) {
    SharedRow w;
    w.bad = n < 0 || n > p.max_blocks * kBlock || n < P * kBlock;
    w.blk_hi = w.bad ? P : (n + kBlock - 1) / kBlock;
    w.nchunk = (P + p.split_blocks - 1) / p.split_blocks;
    w.nsplit = (w.blk_hi - P + p.split_blocks - 1) / p.split_blocks;
    return w;
}

// Partial (o, m, l) of one column into slot `slot` of row `row`.
template <int D>
__device__ __forceinline__ void store_partial(const AttnParams &p, size_t row, int slot, int G, const float *res,
                                              float m, float l, bool bad) {
    const float nan = __uint_as_float(0x7fc00000u);
    const size_t base = row * p.max_splits + slot;
    float *dst = p.ws_o + base * D + G * (D / 4);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) dst[c] = bad ? nan : res[c];
    if (G == 0) {
        p.ws_ml[base * 2] = m;
        p.ws_ml[base * 2 + 1] = bad ? nan : l;
    }
}

template <int D>
__global__ __launch_bounds__(64) KV_MFMA_WAVES void attn_mfma_shared_kernel(AttnParams p, PrefixArgs g) {
    extern __shared__ int sids[];  // [min(split_blocks, kSidsWindow)] staged block ids
    const int lane = threadIdx.x, n16 = lane & 15, G = lane >> 4;
    const int n_pref = g.n_groups * g.units_p * g.max_chunks;
    const int item = blockIdx.x;
    MfmaState<D> st;
    if (item < n_pref) {
        // prefix chunk c of group gi, kv head kvh, column tile ct
        const int gi = item / (g.units_p * g.max_chunks), rem = item % (g.units_p * g.max_chunks);
        const int unit = rem / g.max_chunks, c = rem % g.max_chunks;
        const int kvh = unit / g.ctiles_p, ct = unit % g.ctiles_p;
        const int first = g.start[gi], members = g.start[gi + 1] - first, P = g.blocks[gi];
        const int j0 = c * p.split_blocks, j1 = min(P, j0 + p.split_blocks);
        if (members <= 0 || j0 >= j1 || ct * 16 >= members * p.group) return;
        const int ci = ct * 16 + n16, k = ci / p.group, hq = ci % p.group;
        Column col;
        col.valid = k < members;
        col.row = (size_t)(first + (col.valid ? k : 0)) * p.n_h + kvh * p.group + hq;
        col.lo = 0;
        col.hi = P * kBlock;
        const SharedRow w = shared_row(p, col.valid ? ctx_of(p, first + k) : P * kBlock, P);
        SeqRange r;  // the prefix: P full blocks, attended whole by every member
        r.n = r.hi = r.all_hi = P * kBlock;
        r.lo = r.all_lo = 0;
        r.blk_lo = 0;
        r.nblk = P;
        r.nsplit = w.nchunk;
        r.bad = false;
        bool bad = false;  // a bad block id in the shared table
        run_pieces(j0, j1, [&](int c0, int c1, bool init) {
            bf16_segment<D>(p, first, kvh, col, r, c0, c1, lane, st, bad, false, sids, init);
        });
        const float l = col_sum(st.l);
        if (col.valid) {
            float res[D / 4];
            mfma_gather_run<D>(st, 0.0f, res);
            store_partial<D>(p, col.row, c, G, res, st.m, l, bad || w.bad);
        }
        return;
    }
    // suffix split `split` of sequence b, kv head kvh, column tile ct
    const int it = item - n_pref;
    const int b = it / (p.units * g.suffix_splits), rem = it % (p.units * g.suffix_splits);
    const int unit = rem / g.suffix_splits, split = rem % g.suffix_splits;
    const int kvh = unit / p.ctiles, ct = unit % p.ctiles;
    const int gi = prefix_group_of(g, b);
    const int P = gi < 0 ? 0 : g.blocks[gi];
    const int n = uniform(ctx_of(p, b));
    const SharedRow w = shared_row(p, n, P);
    SeqRange r;
    r.n = r.hi = r.all_hi = w.bad ? 0 : n;
    r.lo = r.all_lo = 0;
    r.blk_lo = 0;
    r.nblk = w.blk_hi;
    r.nsplit = w.nsplit;
    r.bad = w.bad;
    const Column col = column_of(p, b, kvh, ct, n16, r);
    if (split >= w.nsplit) {
        // no suffix block here; a sequence with neither prefix nor blocks
        // (length 0, or out of range) still gets its output
        if (split == 0 && P == 0 && col.valid) {
            const float v = w.bad ? __uint_as_float(0x7fc00000u) : 0.0f;
            float *dst = p.out + col.row * D + G * (D / 4);
#pragma unroll
            for (int c = 0; c < D / 4; ++c) dst[c] = v;
        }
        return;
    }
    const int j0 = P + split * p.split_blocks, j1 = min(w.blk_hi, j0 + p.split_blocks);
    bool bad = w.bad;
    run_pieces(j0, j1, [&](int c0, int c1, bool init) {
        bf16_segment<D>(p, b, kvh, col, r, c0, c1, lane, st, bad, false, sids, init);
    });
    const float l = col_sum(st.l);
    if (col.valid) {
        float res[D / 4];
        mfma_gather_run<D>(st, 0.0f, res);
        if (P == 0 && w.nsplit == 1) {  // the row's only part: the output itself
            const float nan = __uint_as_float(0x7fc00000u);
            float *dst = p.out + col.row * D + G * (D / 4);
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int c = 0; c < D / 4; ++c) dst[c] = bad ? nan : res[c] * inv;
        } else {
            store_partial<D>(p, col.row, w.nchunk + split, G, res, st.m, l, bad);
        }
    }
}

// ---------------------------------------------------------------------------
// shared-prefix decode attention, balanced schedule
//
// Every tile of the call is numbered: the prefix tiles first (group, its
// units, block), then the suffix tiles (sequence, unit, block of its own
// part). Workgroup w of the persistent grid takes its share (Shares) and
// walks it one segment (a group's unit over its prefix, or a sequence's unit
// over its own blocks) at a time, as the balanced schedule does. A piece (a
// segment's part inside one workgroup) leaves its partials in the segment's
// own slot when the piece is the whole segment, else in the workgroup's slot
// 0 (the piece starts the workgroup's range) or slot 1 (it ends it); a
// sequence without a prefix whose suffix is one whole piece writes its output
// directly. Workspace rows (16 columns each): the workgroups' slots
// [n_wg][2], then one slot per segment (prefix segments, then suffix
// segments [batch][units]). Workgroup 0 stores the plan's prefix sums for the
// merge.
// ---------------------------------------------------------------------------

// Prefix sums of the call's tiles, in LDS: prefix tiles and prefix segments
// before group i, own blocks before sequence b (per unit).
struct SharedPlan {
    int *gtile, *gseg, *stile;
    int ng;
};

// Column tiles of group i's prefix units (0: no prefix or no member).
__device__ __forceinline__ int group_ctiles(const AttnParams &p, const PrefixArgs &g, int i) {
    const int m = g.start[i + 1] - g.start[i], P = g.blocks[i];
    return (m > 0 && P > 0) ? (m * p.group + 15) / 16 : 0;
}

// Own (suffix) blocks of sequence b and its prefix blocks; bad as in
// shared_row.
__device__ __forceinline__ int own_blocks(const AttnParams &p, const PrefixArgs &g, int b, int *P_out,
                                          bool *bad_out) {
    const int gi = prefix_group_of(g, b);
    const int P = gi < 0 ? 0 : g.blocks[gi];
    const SharedRow w = shared_row(p, ctx_of(p, b), P);
    *P_out = P;
    *bad_out = w.bad;
    return w.bad ? 0 : w.blk_hi - P;
}

// Inclusive scan over the wave.
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

__device__ __forceinline__ void shared_plan(const AttnParams &p, const PrefixArgs &g, const SharedPlan &pl,
                                            int lane) {
    if (lane == 0) {
        pl.gtile[0] = 0;
        pl.gseg[0] = 0;
        pl.stile[0] = 0;
    }
    int ct = 0, cs = 0;
    for (int base = 0; base < pl.ng; base += 64) {
        const int i = base + lane;
        int segs = 0, tiles = 0;
        if (i < pl.ng) {
            segs = p.n_kv * group_ctiles(p, g, i);
            tiles = segs * g.blocks[i];
        }
        segs = wave_scan(segs, lane);
        tiles = wave_scan(tiles, lane);
        if (i < pl.ng) {
            pl.gseg[i + 1] = cs + segs;
            pl.gtile[i + 1] = ct + tiles;
        }
        cs += __shfl(segs, 63);
        ct += __shfl(tiles, 63);
    }
    int cb = 0;
    for (int base = 0; base < p.batch; base += 64) {
        const int b = base + lane;
        int nb = 0;
        if (b < p.batch) {
            int P;
            bool bad;
            nb = own_blocks(p, g, b, &P, &bad);
        }
        nb = wave_scan(nb, lane);
        if (b < p.batch) pl.stile[b + 1] = cb + nb;
        cb += __shfl(nb, 63);
    }
    __syncthreads();
}

// Workspace row of a piece's partial: the segment's own slot, or slot 0 / 1
// of workgroup w, for segment tiles [a, a + len) and a range share `per`.
__device__ __forceinline__ size_t shared_piece_row(const AttnParams &p, long a, int len, const Shares &sh, int w,
                                                   int seg, int n16) {
    const long lo = max(a, sh.start(w)), hi = min(a + len, sh.start(w + 1));
    size_t slot;
    if (lo == a && hi == a + len)
        slot = (size_t)2 * p.n_wg + seg;
    else
        slot = (size_t)w * 2 + (lo == sh.start(w) ? 0 : 1);
    return slot * 16 + n16;
}

template <int D>
__device__ __forceinline__ void store_piece(const AttnParams &p, size_t row, int G, const float *res, float m,
                                            float l, bool bad) {
    const float nan = __uint_as_float(0x7fc00000u);
    float *dst = p.ws_o + row * D + G * (D / 4);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) dst[c] = bad ? nan : res[c];
    if (G == 0) {
        p.ws_ml[row * 2] = m;
        p.ws_ml[row * 2 + 1] = bad ? nan : l;
    }
}

template <int D>
__global__ __launch_bounds__(64) KV_MFMA_WAVES void attn_mfma_shared_balanced_kernel(AttnParams p, PrefixArgs g) {
    extern __shared__ int lds[];  // plan [ng + 1][2] + [batch + 1], then the staged block ids
    SharedPlan pl;
    pl.ng = g.n_groups;
    pl.gtile = lds;
    pl.gseg = lds + pl.ng + 1;
    pl.stile = lds + 2 * (pl.ng + 1);
    int *sids = pl.stile + p.batch + 1;
    const int lane = threadIdx.x, n16 = lane & 15, G = lane >> 4;
    shared_plan(p, g, pl, lane);
    if (blockIdx.x == 0) {
        for (int i = lane; i < 2 * (pl.ng + 1) + p.batch + 1; i += 64) p.ws_prefix[i] = lds[i];
    }
    const long tp = pl.gtile[pl.ng];  // prefix tiles
    const long total = tp + (long)pl.stile[p.batch] * p.units;
    const Shares sh = shares_of(total, p.n_wg);
    const int wg = sh.share_of(blockIdx.x);
    const long s = sh.start(wg);
    const long e = sh.start(wg + 1);
    for (long t = s; t < e;) {
        MfmaState<D> st;
        long seg_end;
        if (t < tp) {
            // prefix segment: group gi, unit (kvh, ct) over its P shared blocks
            const int gi = last_le(pl.gtile, pl.ng + 1, 1, t, lane);
            const int P = g.blocks[gi], first = g.start[gi], members = g.start[gi + 1] - first;
            const int cti = group_ctiles(p, g, gi);
            const long a0 = pl.gtile[gi];
            const int unit = (int)((t - a0) / P), jr = (int)(t - a0 - (long)unit * P);
            const long a = a0 + (long)unit * P;
            seg_end = min(e, a + P);
            const int kvh = unit / cti, ct = unit % cti;
            const int ci = ct * 16 + n16, k = ci / p.group, hq = ci % p.group;
            Column col;
            col.valid = k < members;
            col.row = (size_t)(first + (col.valid ? k : 0)) * p.n_h + kvh * p.group + hq;
            col.lo = 0;
            col.hi = P * kBlock;
            const SharedRow w = shared_row(p, col.valid ? ctx_of(p, first + k) : P * kBlock, P);
            SeqRange r;  // the prefix: P full blocks, attended whole by every member
            r.n = r.hi = r.all_hi = P * kBlock;
            r.lo = r.all_lo = 0;
            r.blk_lo = 0;
            r.nblk = P;
            r.nsplit = 1;
            r.bad = false;
            bool bad = false;  // a bad block id in the shared table
            run_pieces(jr, jr + (int)(seg_end - t), [&](int c0, int c1, bool init) {
                bf16_segment<D>(p, first, kvh, col, r, c0, c1, lane, st, bad, false, sids, init);
            });
            const float l = col_sum(st.l);
            if (col.valid) {
                float res[D / 4];
                mfma_gather_run<D>(st, 0.0f, res);
                const size_t row = shared_piece_row(p, a, P, sh, wg, pl.gseg[gi] + unit, n16);
                store_piece<D>(p, row, G, res, st.m, l, bad || w.bad);
            }
        } else {
            // suffix segment: sequence b, unit (kvh, ct) over its own blocks
            const long u = t - tp;
            const int b = last_le(pl.stile, p.batch + 1, p.units, u, lane);
            const int nb = pl.stile[b + 1] - pl.stile[b];
            const long a0 = (long)pl.stile[b] * p.units;
            const int unit = (int)((u - a0) / nb), jr = (int)(u - a0 - (long)unit * nb);
            const long a = tp + a0 + (long)unit * nb;
            seg_end = min(e, a + nb);
            const int kvh = unit / p.ctiles, ct = unit % p.ctiles;
            int P;
            bool bad;
            own_blocks(p, g, b, &P, &bad);
            const int n = uniform(ctx_of(p, b));
            SeqRange r;
            r.n = r.hi = r.all_hi = n;
            r.lo = r.all_lo = 0;
            r.blk_lo = 0;
            r.nblk = P + nb;
            r.nsplit = 1;
            r.bad = false;
            const Column col = column_of(p, b, kvh, ct, n16, r);
            run_pieces(P + jr, P + jr + (int)(seg_end - t), [&](int c0, int c1, bool init) {
                bf16_segment<D>(p, b, kvh, col, r, c0, c1, lane, st, bad, false, sids, init);
            });
            const float l = col_sum(st.l);
            if (col.valid) {
                float res[D / 4];
                mfma_gather_run<D>(st, 0.0f, res);
                if (P == 0 && jr == 0 && seg_end - t == nb) {  // the row's only part: the output itself
                    const float nan = __uint_as_float(0x7fc00000u);
                    float *dst = p.out + col.row * D + G * (D / 4);
                    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
                    for (int c = 0; c < D / 4; ++c) dst[c] = bad ? nan : res[c] * inv;
                } else {
                    const int seg = pl.gseg[pl.ng] + b * p.units + unit;
                    store_piece<D>(p, shared_piece_row(p, a, nb, sh, wg, seg, n16), G, res, st.m, l, bad);
                }
            }
        }
        t = seg_end;
    }
}

// ---------------------------------------------------------------------------
// merge of split partials
// ---------------------------------------------------------------------------

// Combines n partials (o, m, l) of one output row into dst (this lane's cv
// channels): out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M the
// largest m_i. row_of(i) is the workspace row of partial i. Partials 64 at a
// time: lane i reads the (m, l) of partial base + i, so a chunk's maxima and
// sums take one round trip and a wave reduction. The value rows are read NB
// at a time (NB = 4 for a short chunk, else 16), the first batch issued with
// the (m, l) loads (the rows do not depend on the weights), so a row with few
// partials costs one round trip; their weights are read from the lanes that
// hold them. A NaN l (bad sequence or table) makes the row NaN; a row no
// partial saw a token for gets 0.
template <int NB, class RowOf>
__device__ __forceinline__ void merge_batch(const AttnParams &p, int base, int i0, int cnt, RowOf row_of, int lane,
                                            int cv, float (&o)[NB][2]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const int i = min(i0 + k, cnt - 1);  // past the end: row re-read, weight 0
        const float *src = p.ws_o + row_of(base + i) * p.head_dim + lane * cv;
#pragma unroll
        for (int c = 0; c < 2; ++c) o[k][c] = c < cv ? src[c] : 0.0f;
    }
}

template <int NB, class RowOf>
__device__ __forceinline__ void merge_chunk(const AttnParams &p, int base, int cnt, RowOf row_of, int lane, int cv,
                                            float &M, float &L, float (&acc)[2]) {
    const int w = base + lane;
    float m = -INFINITY, l = 0.0f;
    if (w < base + cnt) {
        const size_t row = row_of(w);
        m = p.ws_ml[row * 2];
        l = p.ws_ml[row * 2 + 1];
    }
    float o[NB][2];
    merge_batch<NB>(p, base, 0, cnt, row_of, lane, cv, o);
    const float Mn = fmaxf(M, wave_max(m));
    if (Mn == -INFINITY) return;  // no partial has seen a token yet
    const float a = fast_exp2(M - Mn);  // 0 while M is -inf
    L *= a;
    acc[0] *= a;
    acc[1] *= a;
    M = Mn;
    const float wgt = w < base + cnt ? fast_exp2(m - M) : 0.0f;
    L += wave_sum(wgt * l);
    for (int i0 = 0; i0 < cnt; i0 += NB) {
        if (i0 > 0) merge_batch<NB>(p, base, i0, cnt, row_of, lane, cv, o);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const float wi = i0 + k < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), i0 + k))
                                          : 0.0f;
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[c] = fmaf(wi, o[k][c], acc[c]);
        }
    }
}

template <class RowOf>
__device__ __forceinline__ void merge_partials(const AttnParams &p, int n, RowOf row_of, int lane, int cv,
                                               float *dst) {
    float M = -INFINITY, L = 0.0f;
    float acc[2] = {0.0f, 0.0f};
    for (int base = 0; base < n; base += 64) {
        const int cnt = min(64, n - base);
        if (cnt <= 4)
            merge_chunk<4>(p, base, cnt, row_of, lane, cv, M, L, acc);
        else
            merge_chunk<16>(p, base, cnt, row_of, lane, cv, M, L, acc);
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int c = 0; c < cv; ++c) dst[c] = acc[c] * inv;
}

// Grid (n_h * q_len, batch): one wave per output row (query token, head).
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnParams p) {
    const int b = blockIdx.y, lane = threadIdx.x;
    const size_t row = (size_t)b * p.q_len * p.n_h + blockIdx.x;
    const SeqRange r = seq_range(ctx_of(p, b), p.max_blocks, p.window, p.split_blocks, p.max_splits, p.q_len);
    if (r.nsplit <= 1) return;
    const size_t base = row * p.max_splits;
    const int cv = p.head_dim / 64;
    merge_partials(p, r.nsplit, [&](int s) { return base + s; }, lane, cv, p.out + row * p.head_dim + lane * cv);
}

// Merge for the balanced schedule with one workgroup of four waves per
// (sequence, unit) pair, the waves taking the unit's output rows (query
// token, head) in turn; each row combines the partials of the workgroups
// whose tile ranges cut the pair, and gets 0 (NaN for a bad sequence) when
// the sequence has no attended block.
template <bool XCD>
__global__ __launch_bounds__(256) void attn_merge_balanced_unit_kernel(AttnParams p) {
    const int unit = blockIdx.x, b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwaves = 4;
    const int D = p.head_dim, cv = D / 64;
    const int cgroups = p.units / p.n_kv, ucols = 16 * p.ctw;  // column groups per kv head, columns per unit
    const int kvh = unit / cgroups, ci0 = (unit % cgroups) * ucols;
    const int rows = min(ucols, p.ncols - ci0);
    auto dst_of = [&](int r) {  // output of the unit's row r (query column ci0 + r)
        const int ci = ci0 + r, qi = ci / p.group, head = kvh * p.group + ci % p.group;
        return p.out + ((size_t)b * p.q_len + qi) * p.n_h * D + (size_t)head * D + lane * cv;
    };
    const int span = p.ws_prefix[b + 1] - p.ws_prefix[b];  // nb + seg_cost, or 0
    const int nb = span > 0 ? span - p.seg_cost : 0;
    if (nb == 0) {
        const SeqRange r = seq_range(ctx_of(p, b), p.max_blocks, p.window, p.split_blocks, p.max_splits, p.q_len);
        const float v = r.bad ? __uint_as_float(0x7fc00000u) : 0.0f;
        for (int row = wave; row < rows; row += nwaves) {
            float *dst = dst_of(row);
            for (int c = 0; c < cv; ++c) dst[c] = v;
        }
        return;
    }
    const long total = (long)p.ws_prefix[p.batch] * p.units;
    const auto sh = split_of<XCD>(total, p.n_wg);
    const long start = (long)p.ws_prefix[b] * p.units + (long)unit * span;
    const long end = start + nb;
    const int w0 = sh.wg_of(start), w1 = sh.wg_of(end - 1);
    if (w0 == w1) return;  // complete inside one workgroup: already written
    for (int row = wave; row < rows; row += nwaves) {
        // workspace row of the partial that workgroup w holds for this pair:
        // the first piece goes on past its range (slot 1), the others started
        // before theirs (slot 0)
        auto ws_row = [&](int w) {
            const int slot = w == w0 ? 1 : 0;
            return ((size_t)w * 2 + slot) * p.slot_cols + row;
        };
        merge_partials(p, w1 - w0 + 1, [&](int i) { return ws_row(w0 + i); }, lane, cv, dst_of(row));
    }
}


// The same merge with one workgroup per group of rows of a (sequence, unit)
// pair, each thread one 8-channel chunk of one row, so the pair's pieces are
// found once per group and every thread's loads (the pieces' m, l and o) go
// out together. out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M
// the largest m_i, as in merge_partials: a NaN l or o makes the row NaN, and
// a row no piece saw a token for gets 0. Grid (units * groups, batch); a
// group is blockDim / (D / 8) rows, and a unit's slot_cols rows take groups
// of them.
template <bool XCD>
__global__ __launch_bounds__(256) void attn_merge_balanced_rows_kernel(AttnParams p) {
    const int D = p.head_dim, chunks = D / 8, rpg = (int)blockDim.x / chunks;  // chunks per row, rows per group
    const int cgroups = p.units / p.n_kv, ucols = 16 * p.ctw;      // column groups per kv head, columns per unit
    const int groups = (p.slot_cols + rpg - 1) / rpg;              // as the launch: slot_cols = min(ucols, ncols)
    const int unit = blockIdx.x / groups, b = blockIdx.y;
    const int row = (blockIdx.x % groups) * rpg + (int)threadIdx.x / chunks, ch = (int)threadIdx.x % chunks;
    const int kvh = unit / cgroups, ci0 = (unit % cgroups) * ucols;
    const int rows = min(ucols, p.ncols - ci0);
    if (row >= rows) return;
    const int ci = ci0 + row, qi = ci / p.group, head = kvh * p.group + ci % p.group;
    float4 *dst = reinterpret_cast<float4 *>(p.out + (((size_t)b * p.q_len + qi) * p.n_h + head) * D + ch * 8);
    const int span = p.ws_prefix[b + 1] - p.ws_prefix[b];  // nb + seg_cost, or 0
    const int nb = span > 0 ? span - p.seg_cost : 0;
    if (nb == 0) {
        const SeqRange r = seq_range(ctx_of(p, b), p.max_blocks, p.window, p.split_blocks, p.max_splits, p.q_len);
        const float v = r.bad ? __uint_as_float(0x7fc00000u) : 0.0f;
        dst[0] = make_float4(v, v, v, v);
        dst[1] = make_float4(v, v, v, v);
        return;
    }
    const long total = (long)p.ws_prefix[p.batch] * p.units;
    const auto sh = split_of<XCD>(total, p.n_wg);
    const long start = (long)p.ws_prefix[b] * p.units + (long)unit * span;
    const long end = start + nb;
    const int w0 = sh.wg_of(start), w1 = sh.wg_of(end - 1);
    if (w0 == w1) return;  // complete inside one workgroup: already written
    const int n = w1 - w0 + 1;
    // workspace row of piece i: the first piece goes on past its range (slot
    // 1 of its workgroup), the others started before theirs (slot 0)
    auto ws_row = [&](int i) { return ((size_t)(w0 + i) * 2 + (i == 0 ? 1 : 0)) * p.slot_cols + row; };
    constexpr int NB = 4;  // pieces whose loads go out together
    float L = 0.0f;
    float4 acc[2] = {make_float4(0.0f, 0.0f, 0.0f, 0.0f), make_float4(0.0f, 0.0f, 0.0f, 0.0f)};
    if (n <= 2 * NB) {
        // up to 8 pieces (the usual count): every load of every piece goes
        // out at once, one memory round trip instead of one per 4 pieces in
        // each of the two passes below. The same operations in the same
        // order as those passes, so the same bits.
        constexpr int NB2 = 2 * NB;
        const int used = (n + NB - 1) / NB * NB;  // the passes below touch whole groups of 4
        float m[NB2], l[NB2];
        float4 o[NB2][2];
#pragma unroll
        for (int k = 0; k < NB2; ++k) {
            const size_t r = ws_row(min(k, n - 1));  // past the end: a repeat, weight 0
            m[k] = p.ws_ml[r * 2];
            l[k] = p.ws_ml[r * 2 + 1];
            const float4 *src = reinterpret_cast<const float4 *>(p.ws_o + r * D + ch * 8);
            o[k][0] = src[0];
            o[k][1] = src[1];
        }
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NB2; ++k)
            if (k < used) M = fmaxf(M, m[k]);
        if (M != -INFINITY) {
#pragma unroll
            for (int k = 0; k < NB2; ++k) {
                if (k >= used) break;
                const float w = k < n ? fast_exp2(m[k] - M) : 0.0f;
                L = fmaf(w, l[k], L);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    acc[h].x = fmaf(w, o[k][h].x, acc[h].x);
                    acc[h].y = fmaf(w, o[k][h].y, acc[h].y);
                    acc[h].z = fmaf(w, o[k][h].z, acc[h].z);
                    acc[h].w = fmaf(w, o[k][h].w, acc[h].w);
                }
            }
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            dst[h] = make_float4(acc[h].x * inv, acc[h].y * inv, acc[h].z * inv, acc[h].w * inv);
        return;
    }
    float M = -INFINITY;
    for (int i0 = 0; i0 < n; i0 += NB) {
        float m[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) m[k] = p.ws_ml[ws_row(min(i0 + k, n - 1)) * 2];  // past the end: a repeat
#pragma unroll
        for (int k = 0; k < NB; ++k) M = fmaxf(M, m[k]);
    }
    if (M != -INFINITY) {
        for (int i0 = 0; i0 < n; i0 += NB) {
            float m[NB], l[NB];
            float4 o[NB][2];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const size_t r = ws_row(min(i0 + k, n - 1));  // past the end: re-read, weight 0
                m[k] = p.ws_ml[r * 2];
                l[k] = p.ws_ml[r * 2 + 1];
                const float4 *src = reinterpret_cast<const float4 *>(p.ws_o + r * D + ch * 8);
                o[k][0] = src[0];
                o[k][1] = src[1];
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float w = i0 + k < n ? fast_exp2(m[k] - M) : 0.0f;
                L = fmaf(w, l[k], L);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    acc[h].x = fmaf(w, o[k][h].x, acc[h].x);
                    acc[h].y = fmaf(w, o[k][h].y, acc[h].y);
                    acc[h].z = fmaf(w, o[k][h].z, acc[h].z);
                    acc[h].w = fmaf(w, o[k][h].w, acc[h].w);
                }
            }
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) dst[h] = make_float4(acc[h].x * inv, acc[h].y * inv, acc[h].z * inv, acc[h].w * inv);
}

// Merge of the shared-prefix call: one wave per (sequence, head) row with
// more than one part (a prefix, or several suffix splits).
__global__ __launch_bounds__(64) void attn_merge_shared_kernel(AttnParams p, PrefixArgs g) {
    const int b = blockIdx.y, lane = threadIdx.x;
    const size_t row = (size_t)b * p.n_h + blockIdx.x;
    const int gi = prefix_group_of(g, b);
    const int P = gi < 0 ? 0 : g.blocks[gi];
    const SharedRow w = shared_row(p, ctx_of(p, b), P);
    const int total = (P > 0 ? w.nchunk : 0) + w.nsplit;
    if (P == 0 && total <= 1) return;  // written by the attention kernel
    const int cv = p.head_dim / 64;
    float *dst = p.out + row * p.head_dim + lane * cv;
    if (w.bad) {
        for (int c = 0; c < cv; ++c) dst[c] = __uint_as_float(0x7fc00000u);
        return;
    }
    const size_t base = row * p.max_splits;
    merge_partials(p, total, [&](int s) { return base + s; }, lane, cv, dst);
}

// Merge of the balanced shared-prefix call: one wave per (sequence, head)
// row. Finds the pieces of the row's prefix segment and of its own (suffix)
// segment from the plan the attention kernel stored, and combines their
// partials; a sequence that is bad or shorter than its prefix gets NaN, one
// with no token 0.
__global__ __launch_bounds__(64) void attn_merge_shared_balanced_kernel(AttnParams p, PrefixArgs g) {
    const int b = blockIdx.y, lane = threadIdx.x, head = blockIdx.x;
    const int ng = g.n_groups;
    const int *gtile = p.ws_prefix, *gseg = gtile + ng + 1, *stile = gseg + ng + 1;
    const size_t row = (size_t)b * p.n_h + head;
    const int cv = p.head_dim / 64;
    float *dst = p.out + row * p.head_dim + lane * cv;
    const int kvh = head / p.group, hq = head % p.group;
    int P;
    bool bad;
    const int nb = own_blocks(p, g, b, &P, &bad);
    if (bad || (P == 0 && nb == 0)) {
        const float v = bad ? __uint_as_float(0x7fc00000u) : 0.0f;
        for (int c = 0; c < cv; ++c) dst[c] = v;
        return;
    }
    const long tp = gtile[ng];
    const long total = tp + (long)stile[p.batch] * p.units;
    const Shares sh = shares_of(total, p.n_wg);
    // prefix segment of the row: group gi, column k * group + hq
    long pa = 0;
    int pseg = 0, pw0 = 0, npre = 0, pn16 = 0;
    if (P > 0) {
        const int gi = prefix_group_of(g, b);
        const int ci = (b - g.start[gi]) * p.group + hq, cti = group_ctiles(p, g, gi);
        const int unit = kvh * cti + ci / 16;
        pn16 = ci % 16;
        pa = gtile[gi] + (long)unit * P;
        pseg = gseg[gi] + unit;
        pw0 = sh.wg_of(pa);
        npre = sh.wg_of(pa + P - 1) - pw0 + 1;
    }
    // own segment of the row
    const int unit = kvh * p.ctiles + hq / 16, sn16 = hq % 16;
    const long sa = tp + (long)stile[b] * p.units + (long)unit * nb;
    const int sseg = gseg[ng] + b * p.units + unit;
    const int sw0 = nb > 0 ? sh.wg_of(sa) : 0;
    const int nsuf = nb > 0 ? sh.wg_of(sa + nb - 1) - sw0 + 1 : 0;
    if (P == 0 && nsuf == 1) return;  // written by the attention kernel
    merge_partials(p, npre + nsuf, [&](int i) {
        return i < npre ? shared_piece_row(p, pa, P, sh, pw0 + i, pseg, pn16)
                        : shared_piece_row(p, sa, nb, sh, sw0 + i - npre, sseg, sn16);
    }, lane, cv, dst);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Every launch goes through hipExtLaunchKernelGGL so that optional timing
// events are recorded by the kernel's own dispatch (start and end of the
// kernel), not by separate queue packets between kernels.
template <int KIND, int D>
static hipError_t launch_valu_d(const AttnParams &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int g = p.group;
    if (g <= 1)
        hipExtLaunchKernelGGL((attn_valu_kernel<KIND, D, 1>), grid, dim3(64), 0, s, e0, e1, 0, p);
    else if (g <= 2)
        hipExtLaunchKernelGGL((attn_valu_kernel<KIND, D, 2>), grid, dim3(64), 0, s, e0, e1, 0, p);
    else if (g <= 4)
        hipExtLaunchKernelGGL((attn_valu_kernel<KIND, D, 4>), grid, dim3(64), 0, s, e0, e1, 0, p);
    else if (g <= 8)
        hipExtLaunchKernelGGL((attn_valu_kernel<KIND, D, 8>), grid, dim3(64), 0, s, e0, e1, 0, p);
    else
        hipExtLaunchKernelGGL((attn_valu_kernel<KIND, D, 16>), grid, dim3(64), 0, s, e0, e1, 0, p);
    return hipGetLastError();
}

template <int KIND>
static hipError_t launch_valu(const AttnParams &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    return p.head_dim == 64 ? launch_valu_d<KIND, 64>(p, grid, s, e0, e1) : launch_valu_d<KIND, 128>(p, grid, s, e0, e1);
}

hipError_t launch_attention(int dtype, int kernel, const AttnParams &p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid(p.max_splits, kernel == 2 ? p.units : p.n_kv, p.batch);
    if (p.batch == 0) return hipSuccess;
    if (kernel == 2) {
        const bool q4 = dtype == KV_INT4;
        const bool keep = p.units > p.n_kv;  // several units per kv head: cached loads
        const bool flat = p.pool.q4_span > 0;  // INT4 arrays within 4 GiB: one descriptor
        if (p.schedule == KV_SCHED_BALANCED) {
            const uint32_t lds = (uint32_t)(balanced_lds_ints(p.batch, p.split_blocks) * sizeof(int));
            const dim3 bg(p.n_wg);
            if (!q4 && p.ctw == 2 && p.head_dim == 128) {
                // two column tiles: two waves share each tile through LDS,
                // one column tile each (the next tiles' loads fly while this
                // one is used; one wave with both column tiles has no
                // register room for that). 8B shape, 5 query tokens: 135.6
                // -> 124.6 us; 8: 146 -> 139 us.
                hipExtLaunchKernelGGL((attn_mfma_wide_kernel<128, 2, 1>), bg, dim3(128), lds, s, e0, e1, 0, p);
            } else if (!q4 && p.ctw > 2) {  // wide units: ctw / kWideCT waves per workgroup
                constexpr int C = kWideCT, W4 = 4 / C, W8 = 8 / C;
                if (p.head_dim == 64 && p.ctw == 4)
                    hipExtLaunchKernelGGL((attn_mfma_wide_kernel<64, W4, C>), bg, dim3(64 * W4), lds, s, e0, e1, 0, p);
                else if (p.head_dim == 64)
                    hipExtLaunchKernelGGL((attn_mfma_wide_kernel<64, W8, C>), bg, dim3(64 * W8), lds, s, e0, e1, 0, p);
                else if (p.ctw == 4)
                    hipExtLaunchKernelGGL((attn_mfma_wide_kernel<128, W4, C>), bg, dim3(64 * W4), lds, s, e0, e1, 0, p);
                else
                    hipExtLaunchKernelGGL((attn_mfma_wide_kernel<128, W8, C>), bg, dim3(64 * W8), lds, s, e0, e1, 0, p);
            } else if (q4 && p.ncols <= 4 && flat)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 1, 1, false, true>), bg, dim3(64), lds, s, e0, e1,
                                      0, p);
            else if (q4 && flat)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 4, 1, false, true>), bg, dim3(64), lds, s, e0, e1,
                                      0, p);
            else if (q4 && p.ncols <= 4)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 1, 1>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else if (q4)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 4, 1>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.head_dim == 64 && p.ctw == 2 && keep)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<64, 0, 2, true>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.head_dim == 64 && p.ctw == 2)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<64, 0, 2>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.head_dim == 64)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<64, 0, 1>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.ctw == 2 && keep)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 0, 2, true>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.ctw == 2)
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 0, 2>), bg, dim3(64), lds, s, e0, e1, 0, p);
            else
                hipExtLaunchKernelGGL((attn_mfma_balanced_kernel<128, 0, 1>), bg, dim3(64), lds, s, e0, e1, 0, p);
        } else {
            const uint32_t lds = (uint32_t)(min(p.split_blocks, kSidsWindow) * sizeof(int));
            if (q4 && p.ncols <= 4 && flat)
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 1, 1, false, true>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (q4 && flat)
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 4, 1, false, true>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (q4 && p.ncols <= 4)
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 1, 1>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (q4)
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 4, 1>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.head_dim == 64 && p.ctw == 2 && keep)
                hipExtLaunchKernelGGL((attn_mfma_kernel<64, 0, 2, true>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.head_dim == 64 && p.ctw == 2)
                hipExtLaunchKernelGGL((attn_mfma_kernel<64, 0, 2>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.head_dim == 64)
                hipExtLaunchKernelGGL((attn_mfma_kernel<64, 0, 1>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.ctw == 2 && keep)
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 0, 2, true>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else if (p.ctw == 2)
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 0, 2>), grid, dim3(64), lds, s, e0, e1, 0, p);
            else
                hipExtLaunchKernelGGL((attn_mfma_kernel<128, 0, 1>), grid, dim3(64), lds, s, e0, e1, 0, p);
        }
        return hipGetLastError();
    }
    if (dtype == KV_F32) return launch_valu<KIND_F32>(p, grid, s, e0, e1);
    if (dtype == KV_INT4) return launch_valu<KIND_INT4>(p, grid, s, e0, e1);
    return launch_valu<KIND_BF16>(p, grid, s, e0, e1);
}

int balanced_grid(int dtype, int head_dim, int batch, int max_blocks, bool q4_one_score) {
    // compute units x resident workgroups per compute unit; 256 x 2 when the
    // runtime cannot tell (no device: only the size of a workspace is asked)
    int dev = 0, cus = 0, per_cu = 0;
    const size_t lds = (size_t)balanced_lds_ints(batch, max_blocks) * sizeof(int);
    const int waves = dtype == KV_INT4 && q4_one_score ? kBalancedWavesQ4One : 2;  // per SIMD
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256 * waves;
    hipError_t e;
    if (dtype == KV_INT4 && q4_one_score)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_balanced_kernel<128, 1, 1, false, true>, 64,
                                                         lds);
    else if (dtype == KV_INT4)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_balanced_kernel<128, 4, 1>, 64, lds);
    else if (head_dim == 64)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_balanced_kernel<64, 0, 2>, 64, lds);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_balanced_kernel<128, 0, 2>, 64, lds);
    if (e != hipSuccess || per_cu <= 0) per_cu = 2;
    // bf16: at most two waves per SIMD: with more, more tile bytes are in
    // flight and the 8B- and 70B-shaped decode layers measured slower (109
    // vs 104 us at three waves on the 8B shape)
    if (per_cu > 4 * waves) per_cu = 4 * waves;
    return cus * per_cu;
}

int wide_grid(int head_dim, int ctw, int batch, int max_blocks) {
    constexpr int C = kWideCT, W4 = 4 / C, W8 = 8 / C;
    const int waves = ctw == 2 ? 2 : ctw / C;  // two column tiles: two waves of one
    int dev = 0, cus = 0, per_cu = 0;
    const size_t lds = (size_t)balanced_lds_ints(batch, max_blocks) * sizeof(int);
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 1024 / ctw;
    hipError_t e;
    if (ctw == 2)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_wide_kernel<128, 2, 1>, 128, lds);
    else if (head_dim == 64)
        e = ctw == 4 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_wide_kernel<64, W4, C>, 64 * W4, lds)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_wide_kernel<64, W8, C>, 64 * W8, lds);
    else
        e = ctw == 4
                ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_wide_kernel<128, W4, C>, 64 * W4, lds)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_wide_kernel<128, W8, C>, 64 * W8, lds);
    if (e != hipSuccess || per_cu <= 0) per_cu = 1;
    if (per_cu > std::max(8 / waves, 1)) per_cu = std::max(8 / waves, 1);  // two waves per SIMD, as balanced_grid
    return cus * per_cu;
}

size_t shared_balanced_lds(int n_groups, int batch, int max_blocks) {
    return (size_t)(2 * (n_groups + 1) + batch + 1 + std::min(max_blocks, kSidsWindow)) * sizeof(int);
}

int shared_balanced_grid(int head_dim, size_t lds) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256 * 2;
    const hipError_t e =
        head_dim == 64
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_shared_balanced_kernel<64>, 64, lds)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_shared_balanced_kernel<128>, 64, lds);
    if (e != hipSuccess || per_cu <= 0) per_cu = 2;
    if (per_cu > 8) per_cu = 8;  // two waves per SIMD, as balanced_grid
    return cus * per_cu;
}

// One four-wave workgroup per unit for units of 5-16 rows when there are at
// least 2048 units (the 70B-shaped merge 4.2 us, 4.6 with row groups);
// otherwise row groups (one wave per row before them: 8B shape 5.4 -> 5.1
// us, 4 query tokens 10.9 -> 7.3, 16 query tokens 25 -> 14).
constexpr int kMergeUnitRows = 5, kMergeUnitMin = 2048;

hipError_t launch_merge(const AttnParams &p, hipStream_t s, hipEvent_t e_end) {
    const bool none = p.batch == 0 || (p.schedule != KV_SCHED_BALANCED && p.max_splits <= 1);
    if (none) return e_end ? hipEventRecord(e_end, s) : hipSuccess;
    if (p.schedule == KV_SCHED_BALANCED && p.slot_cols >= kMergeUnitRows && p.slot_cols <= 16 &&
        (long)p.batch * p.units >= kMergeUnitMin) {
        if (p.xcd_shares)
            hipExtLaunchKernelGGL(attn_merge_balanced_unit_kernel<true>, dim3(p.units, p.batch), dim3(256), 0, s,
                                  nullptr, e_end, 0, p);
        else
            hipExtLaunchKernelGGL(attn_merge_balanced_unit_kernel<false>, dim3(p.units, p.batch), dim3(256), 0, s,
                                  nullptr, e_end, 0, p);
    } else if (p.schedule == KV_SCHED_BALANCED) {
        // whole waves, up to 256 threads: 16 rows of 128 channels, 32 of 64
        const int chunks = p.head_dim / 8;
        const int threads = std::min(256, (p.slot_cols * chunks + 63) / 64 * 64), rpg = threads / chunks;
        const int groups = (p.slot_cols + rpg - 1) / rpg;
        if (p.xcd_shares)
            hipExtLaunchKernelGGL(attn_merge_balanced_rows_kernel<true>, dim3(p.units * groups, p.batch),
                                  dim3(threads), 0, s, nullptr, e_end, 0, p);
        else
            hipExtLaunchKernelGGL(attn_merge_balanced_rows_kernel<false>, dim3(p.units * groups, p.batch),
                                  dim3(threads), 0, s, nullptr, e_end, 0, p);
    } else
        hipExtLaunchKernelGGL(attn_merge_kernel, dim3(p.n_h * p.q_len, p.batch), dim3(64), 0, s, nullptr, e_end, 0,
                              p);
    return hipGetLastError();
}


hipError_t launch_attention_shared(const AttnParams &p, const PrefixArgs &g, hipStream_t s, hipEvent_t e0,
                                   hipEvent_t e1, hipEvent_t e_end) {
    if (p.batch == 0) return e_end ? hipEventRecord(e_end, s) : hipSuccess;
    if (p.schedule == KV_SCHED_BALANCED) {
        const uint32_t lds = (uint32_t)shared_balanced_lds(g.n_groups, p.batch, p.split_blocks);
        if (p.head_dim == 64)
            hipExtLaunchKernelGGL((attn_mfma_shared_balanced_kernel<64>), dim3(p.n_wg), dim3(64), lds, s, e0, e1, 0,
                                  p, g);
        else
            hipExtLaunchKernelGGL((attn_mfma_shared_balanced_kernel<128>), dim3(p.n_wg), dim3(64), lds, s, e0, e1, 0,
                                  p, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipExtLaunchKernelGGL(attn_merge_shared_balanced_kernel, dim3(p.n_h, p.batch), dim3(64), 0, s, nullptr, e_end,
                              0, p, g);
        return hipGetLastError();
    }
    const long items = (long)g.n_groups * g.units_p * g.max_chunks + (long)p.batch * p.units * g.suffix_splits;
    const uint32_t lds = (uint32_t)(min(p.split_blocks, kSidsWindow) * sizeof(int));
    if (p.head_dim == 64)
        hipExtLaunchKernelGGL((attn_mfma_shared_kernel<64>), dim3((uint32_t)items), dim3(64), lds, s, e0, e1, 0, p, g);
    else
        hipExtLaunchKernelGGL((attn_mfma_shared_kernel<128>), dim3((uint32_t)items), dim3(64), lds, s, e0, e1, 0, p,
                              g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL(attn_merge_shared_kernel, dim3(p.n_h, p.batch), dim3(64), 0, s, nullptr, e_end, 0, p, g);
    return hipGetLastError();
}

}  // namespace kvc
