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
    if (L0 < 0 || L0 + p.n_new > p.max_blocks * kBlock) return;
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
    for (int t = 0; t < r; ++t) {
        const uint32_t vw = act ? vs[(size_t)t * hd + lane] : 0u;
        const size_t row = tile * kBlock + t;
        code_v_row(vw, act, p.dst.vq + row * hd, p.dst.vs + row, p.dst.vm + row, lane);
    }
    if (r == kBlock) {
        uint32_t w[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) w[t] = act ? ks[(size_t)t * hd + lane] : 0u;
        code_k_block(w, act, p.dst.kq + tile * kBlock * hd, p.dst.ks + tile * D, p.dst.km + tile * D, lane, hd);
    } else {
        const int slot = p.seq_slots ? p.seq_slots[b] : b;
        if (slot < 0 || slot >= p.max_seqs || !act) return;
        uint32_t *tail = reinterpret_cast<uint32_t *>(p.dst.ktail) + ((size_t)slot * p.n_kv + h) * kBlock * hd;
        for (int t = 0; t < r; ++t) tail[(size_t)t * hd + lane] = ks[(size_t)t * hd + lane];
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
