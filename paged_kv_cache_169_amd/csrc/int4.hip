// int4.hip -- KVQuant INT4 coding: append to an INT4 pool and bulk coding of
// bf16 pool contents.
//
// Quantizer ["KV Cache는 왜 LLM 서빙의 핵심인가", section "KVQuant: 마지막 4배"]:
// s = (max - min) / 15 per group, one 4-bit code per value. K is grouped per
// channel (over the 16 tokens of a block), V per token (over the head_dim
// channels). Codes are clamp(round((x - min) / s), 0, 15) computed in fp32 from
// the stored fp16 s and min, rounding half away from zero.
//
// Lane mapping (one wave64 per (sequence, kv head) or (sequence, block, kv
// head)): lane l owns channel pair (2l, 2l+1), i.e. one 32-bit word of a bf16
// row and one byte of a code row; for head_dim 64 lanes 32..63 idle. A V row's
// min/max is a wave reduction; a K block's per-channel min/max stays in the
// lane (its 16 tokens are 16 loads of the same word).
//
// Built with -ffp-contract=off: the codes must match a plain fp32 evaluation.
#include "device.h"
#include "internal.h"

namespace kvc {

// Append to an INT4 pool. Grid (n_kv, batch), one wave each; the wave takes
// the sequence's n_new tokens in order. The K rows of the block being filled
// live in LDS (seeded from the sequence's tail row and kept in the tail too),
// so a block completed in the middle of the chunk is coded from LDS.
__global__ __launch_bounds__(64) void append_int4_kernel(AppendParams p) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int D = p.head_dim, hd = D / 2;
    const bool act = lane < hd;
    __shared__ uint32_t rows[kBlock][64];  // K rows of the open block, one word per lane
    const int L0 = p.seq_lens[b];
    if (!append_fits(L0, p.n_new, p.max_blocks)) return;
    const int slot = p.seq_slots ? p.seq_slots[b] : b;
    if (slot < 0 || slot >= p.max_seqs) return;
    uint32_t *tail = reinterpret_cast<uint32_t *>(p.pool.ktail) + ((size_t)slot * p.n_kv + h) * kBlock * hd;
    // the rows already in the open block are needed only if this call
    // completes it; they are loaded together (independent loads)
    const int t0 = L0 % kBlock;
    if (t0 > 0 && t0 + p.n_new >= kBlock) {
        uint32_t w[kBlock - 1];
#pragma unroll
        for (int tt = 0; tt < kBlock - 1; ++tt) w[tt] = (act && tt < t0) ? tail[(size_t)tt * hd + lane] : 0u;
#pragma unroll
        for (int tt = 0; tt < kBlock - 1; ++tt)
            if (tt < t0) rows[tt][lane] = w[tt];
    }
    __syncthreads();
    for (int k = 0; k < p.n_new; ++k) {
        const int L = L0 + k;
        const int pid = p.tables[(size_t)b * p.max_blocks + L / kBlock];
        if (pid < 0 || pid >= p.num_blocks) return;
        const int t = L % kBlock;
        const size_t src = (((size_t)b * p.n_new + k) * p.n_kv + h) * hd;  // in words
        const uint32_t vw = act ? reinterpret_cast<const uint32_t *>(p.v_new)[src + lane] : 0u;
        const uint32_t kw = act ? reinterpret_cast<const uint32_t *>(p.k_new)[src + lane] : 0u;

        const size_t tile = (size_t)pid * p.n_kv + h;   // (block, head) tile index
        const size_t row = tile * kBlock + t;            // token row index
        code_v_row(vw, act, p.pool.vq + row * hd, p.pool.vs + row, p.pool.vm + row, lane);

        if (act) tail[(size_t)t * hd + lane] = kw;
        rows[t][lane] = kw;
        __syncthreads();
        if (t == kBlock - 1) {
            uint32_t w[kBlock];
#pragma unroll
            for (int tt = 0; tt < kBlock; ++tt) w[tt] = rows[tt][lane];
            code_k_block(w, act, p.pool.kq + tile * kBlock * hd, p.pool.ks + tile * D, p.pool.km + tile * D, lane, hd);
        }
        __syncthreads();
    }
}

// Bulk coding. Grid (max_blocks, n_kv, batch), one wave per (block, head, seq).
// DPP move inside each 16-lane row (every source lane is in the row).
template <int CTRL>
__device__ __forceinline__ float row_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
enum { kQuadXor1 = 0xb1, kQuadXor2 = 0x4e, kRowHalfMirror = 0x141, kRowMirror = 0x140 };

// Min and max over each aligned group of `lanes` lanes (8 or 16) of a row,
// in registers: pairs, quads, then the half-row mirror (lane i with 7 - i)
// joins the two quads of a half row and the row mirror (i with 15 - i) its
// two halves. (fminf / fmaxf ignore NaN; the order does not matter.)
__device__ __forceinline__ void row_group_min_max(float &mn, float &mx, int lanes) {
    mn = fminf(mn, row_dpp<kQuadXor1>(mn));
    mx = fmaxf(mx, row_dpp<kQuadXor1>(mx));
    mn = fminf(mn, row_dpp<kQuadXor2>(mn));
    mx = fmaxf(mx, row_dpp<kQuadXor2>(mx));
    mn = fminf(mn, row_dpp<kRowHalfMirror>(mn));
    mx = fmaxf(mx, row_dpp<kRowHalfMirror>(mx));
    if (lanes == 16) {
        mn = fminf(mn, row_dpp<kRowMirror>(mn));
        mx = fmaxf(mx, row_dpp<kRowMirror>(mx));
    }
}

__global__ __launch_bounds__(64) void quantize_int4_kernel(QuantParams p) {
    const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int D = p.head_dim, hd = D / 2;
    const bool act = lane < hd;
    const int n = p.lens[b];
    if (n < 0 || n > p.max_blocks * kBlock || j * kBlock >= n) return;
    const int pid = p.tables[(size_t)b * p.max_blocks + j];
    if (pid < 0 || pid >= p.num_blocks) return;
    const int r = min(kBlock, n - j * kBlock);
    const size_t tile = (size_t)pid * p.n_kv + h;
    const uint32_t *ks = reinterpret_cast<const uint32_t *>(p.src.k) + tile * kBlock * hd;
    const uint32_t *vs = reinterpret_cast<const uint32_t *>(p.src.v) + tile * kBlock * hd;
    // Every row of the block is loaded before any is coded (one round trip).
    // V rows are coded several at a time: lpt = head_dim / 8 lanes per row,
    // 8 channels each, so a row's min / max is a reduction over lpt lanes
    // and 64 / lpt rows go through each pass (4 passes at head_dim 128).
    const int lpt = D / 8, rows_per = 64 / lpt, gi = lane / lpt, cc = lane % lpt;
    uint4 vrow[4];
    uint32_t w[kBlock];
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
        const int t = ps * rows_per + gi;
        vrow[ps] = ps * rows_per < kBlock && t < r
                       ? reinterpret_cast<const uint4 *>(vs + (size_t)t * hd)[cc]
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kBlock; ++t) w[t] = act && t < r ? ks[(size_t)t * hd + lane] : 0u;
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
        if (ps * rows_per >= kBlock) break;
        const int t = ps * rows_per + gi;
        const uint32_t x[4] = {vrow[ps].x, vrow[ps].y, vrow[ps].z, vrow[ps].w};
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mn = fminf(mn, fminf(bf16_lo(x[k]), bf16_hi(x[k])));
            mx = fmaxf(mx, fmaxf(bf16_lo(x[k]), bf16_hi(x[k])));
        }
        row_group_min_max(mn, mx, lpt);
        if (t >= r) continue;
        const Q4Params q = q4_params(mn, mx);
        uint32_t code[4];
        q4_code_pairs<4>(x, q, q, code);
        const uint32_t packed = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        const size_t row = tile * kBlock + t;
        reinterpret_cast<uint32_t *>(p.dst.vq + row * hd)[cc] = packed;
        if (cc == 0) {
            p.dst.vs[row] = q.s16;
            p.dst.vm[row] = q.m16;
        }
    }
    if (r == kBlock) {
        // per-channel K coding, lane = channel pair; the code bytes go through
        // LDS so that each lane stores 16 contiguous bytes of the code tile
        __shared__ uint8_t kc[kBlock * 64];
        float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int t = 0; t < kBlock; ++t) {
            mn0 = fminf(mn0, bf16_lo(w[t]));
            mx0 = fmaxf(mx0, bf16_lo(w[t]));
            mn1 = fminf(mn1, bf16_hi(w[t]));
            mx1 = fmaxf(mx1, bf16_hi(w[t]));
        }
        const Q4Params q0 = q4_params(mn0, mx0), q1 = q4_params(mn1, mx1);
        if (act) {
            // four rows at a time: one near-tie branch per 8 values, and few
            // values live at once
#pragma unroll
            for (int t0 = 0; t0 < kBlock; t0 += 4) {
                const uint32_t wg[4] = {w[t0], w[t0 + 1], w[t0 + 2], w[t0 + 3]};
                uint32_t code[4];
                q4_code_pairs<4>(wg, q0, q1, code);
#pragma unroll
                for (int t = 0; t < 4; ++t) kc[(t0 + t) * hd + lane] = (uint8_t)code[t];
            }
            reinterpret_cast<uint32_t *>(p.dst.ks + tile * D)[lane] = (uint32_t)q0.s16 | ((uint32_t)q1.s16 << 16);
            reinterpret_cast<uint32_t *>(p.dst.km + tile * D)[lane] = (uint32_t)q0.m16 | ((uint32_t)q1.m16 << 16);
        }
        __syncthreads();
        if (lane < hd)  // the tile's 16 * hd code bytes, 16 per lane
            reinterpret_cast<uint4 *>(p.dst.kq + tile * kBlock * hd)[lane] = reinterpret_cast<const uint4 *>(kc)[lane];
    } else {
        const int slot = p.seq_slots ? p.seq_slots[b] : b;
        if (slot < 0 || slot >= p.max_seqs || !act) return;
        uint32_t *tail = reinterpret_cast<uint32_t *>(p.dst.ktail) + ((size_t)slot * p.n_kv + h) * kBlock * hd;
#pragma unroll
        for (int t = 0; t < kBlock; ++t) {
            if (t >= r) break;
            tail[(size_t)t * hd + lane] = w[t];
        }
    }
}

hipError_t launch_append_int4(const AppendParams &p, hipStream_t s) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(append_int4_kernel, dim3(p.n_kv, p.batch), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_quantize_int4(const QuantParams &p, hipStream_t s) {
    if (p.batch == 0 || p.max_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_int4_kernel, dim3(p.max_blocks, p.n_kv, p.batch), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
