// rope.hip -- RoPE re-rotation of a reused chunk's keys, in place.
//
// Full KV reuse ["Research Paper Review : CACHE BLEND", section "Background"]:
// a chunk's K/V are computed as if the chunk began at position 0; because RoPE
// encodes only relative position, its keys are moved to the real start by a
// single extra rotation by delta = real start - 0. Values (and queries) are
// left alone.
//
// Pair i of a key turns by delta * base^(-2i/head_dim). The host computes the
// angles and cos/sin in fp64 and passes fp32 cos/sin per pair in the kernel
// arguments; each pair (x, y) becomes (x c - y s, x s + y c) with separately
// rounded fp32 products (no fused multiply-add; file built with
// -ffp-contract=off), rounded to the pool type.
//
// Work: one thread per (token, kv head, group of 4 pairs): a pure streaming
// kernel (read and write each key element once).
#include "device.h"
#include "internal.h"

namespace kvc {

__device__ __forceinline__ void rotate(float x, float y, float c, float s, float &nx, float &ny) {
    nx = __fsub_rn(__fmul_rn(x, c), __fmul_rn(y, s));
    ny = __fadd_rn(__fmul_rn(x, s), __fmul_rn(y, c));
}

template <bool BF16>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
    const int D = p.head_dim;
    const int groups = D / 8;  // groups of 4 pairs per row
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)p.num_tokens * p.n_kv * groups;
    if (i >= total) return;
    const int gq = (int)(i % groups);
    long r = i / groups;
    const int h = (int)(r % p.n_kv);
    const int k = (int)(r / p.n_kv);
    const int pos = p.first_slot + k;
    const int pid = p.chunk_blocks[pos / kBlock];
    if (pid < 0 || pid >= p.num_blocks) return;
    const size_t row = (((size_t)pid * p.n_kv + h) * kBlock + pos % kBlock) * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int pi = 4 * gq + e;
        const int c0 = p.style == 0 ? 2 * pi : pi;
        const int c1 = p.style == 0 ? 2 * pi + 1 : pi + D / 2;
        const float c = p.cos_t[pi], s = p.sin_t[pi];
        float nx, ny;
        if (BF16) {
            uint16_t *kr = reinterpret_cast<uint16_t *>(p.k) + row;
            rotate(bf16_to_f(kr[c0]), bf16_to_f(kr[c1]), c, s, nx, ny);
            kr[c0] = f_to_bf16(nx);
            kr[c1] = f_to_bf16(ny);
        } else {
            float *kr = reinterpret_cast<float *>(p.k) + row;
            rotate(kr[c0], kr[c1], c, s, nx, ny);
            kr[c0] = nx;
            kr[c1] = ny;
        }
    }
}

hipError_t launch_rope(int dtype, const RopeParams &p, hipStream_t s) {
    const long total = (long)p.num_tokens * p.n_kv * (p.head_dim / 8);
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const unsigned blocks = (unsigned)((total + threads - 1) / threads);
    if (dtype == KV_BF16)
        hipLaunchKernelGGL(rope_kernel<true>, dim3(blocks), dim3(threads), 0, s, p);
    else
        hipLaunchKernelGGL(rope_kernel<false>, dim3(blocks), dim3(threads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
