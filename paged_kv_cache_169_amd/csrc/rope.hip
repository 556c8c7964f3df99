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
// Work: one thread per (token, kv head, group of 4 pairs), one workgroup
// per (block, kv head) tile: a pure streaming kernel (read and write each key
// element once).
#include "device.h"
#include "internal.h"

namespace kvc {

__device__ __forceinline__ void rotate(float x, float y, float c, float s, float &nx, float &ny) {
    nx = __fsub_rn(__fmul_rn(x, c), __fmul_rn(y, s));
    ny = __fadd_rn(__fmul_rn(x, s), __fmul_rn(y, c));
}

// bf16 pool: pairs 4gq .. 4gq+3 of one row. Style 0 takes them from one
// 16-byte chunk (channels 8gq .. 8gq+7), style 1 from two 8-byte chunks
// (channels 4gq .. 4gq+3 and head_dim/2 + 4gq ..).
__device__ __forceinline__ void rope_bf16_group(const RopeParams &p, uint16_t *row, int gq) {
    const int D = p.head_dim;
    if (p.style == 0) {
        uint4 *ptr = reinterpret_cast<uint4 *>(row + 8 * gq);
        const uint4 v = *ptr;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pi = 4 * gq + e;
            float nx, ny;
            rotate(bf16_lo(w[e]), bf16_hi(w[e]), p.cos_t[pi], p.sin_t[pi], nx, ny);
            o[e] = (uint32_t)f_to_bf16(nx) | ((uint32_t)f_to_bf16(ny) << 16);
        }
        *ptr = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
        uint2 *px = reinterpret_cast<uint2 *>(row + 4 * gq);
        uint2 *py = reinterpret_cast<uint2 *>(row + D / 2 + 4 * gq);
        const uint2 vx = *px, vy = *py;
        const uint32_t wx[2] = {vx.x, vx.y}, wy[2] = {vy.x, vy.y};
        uint32_t ox[2], oy[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float x0, y0, x1, y1;
            const int p0 = 4 * gq + 2 * h, p1 = p0 + 1;
            rotate(bf16_lo(wx[h]), bf16_lo(wy[h]), p.cos_t[p0], p.sin_t[p0], x0, y0);
            rotate(bf16_hi(wx[h]), bf16_hi(wy[h]), p.cos_t[p1], p.sin_t[p1], x1, y1);
            ox[h] = (uint32_t)f_to_bf16(x0) | ((uint32_t)f_to_bf16(x1) << 16);
            oy[h] = (uint32_t)f_to_bf16(y0) | ((uint32_t)f_to_bf16(y1) << 16);
        }
        *px = make_uint2(ox[0], ox[1]);
        *py = make_uint2(oy[0], oy[1]);
    }
}

// One workgroup per (chunk block, kv head): thread (slot t, group gq) of
// the block's 16 x head_dim / 8 groups, so consecutive threads touch
// consecutive bytes of the (block, kv head) tile.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
    const int D = p.head_dim;
    const int groups = D / 8;  // groups of 4 pairs per row
    const int kb = p.first_slot / kBlock + (int)blockIdx.x, h = blockIdx.y;
    const int t = (int)threadIdx.x / groups, gq = (int)threadIdx.x % groups;
    const int pos = kb * kBlock + t;  // position in the block list
    if (pos < p.first_slot || pos >= p.first_slot + p.num_tokens) return;
    const int pid = p.chunk_blocks[kb];
    if (pid < 0 || pid >= p.num_blocks) return;
    const size_t row = (((size_t)pid * p.n_kv + h) * kBlock + t) * D;
    if (BF16) {
        rope_bf16_group(p, reinterpret_cast<uint16_t *>(p.k) + row, gq);
        return;
    }
    float *kr = reinterpret_cast<float *>(p.k) + row;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int pi = 4 * gq + e;
        const int c0 = p.style == 0 ? 2 * pi : pi;
        const int c1 = p.style == 0 ? 2 * pi + 1 : pi + D / 2;
        float nx, ny;
        rotate(kr[c0], kr[c1], p.cos_t[pi], p.sin_t[pi], nx, ny);
        kr[c0] = nx;
        kr[c1] = ny;
    }
}

hipError_t launch_rope(int dtype, const RopeParams &p, hipStream_t s) {
    if (p.num_tokens <= 0) return hipSuccess;
    const int first = p.first_slot / kBlock, last = (p.first_slot + p.num_tokens - 1) / kBlock;
    const dim3 grid((unsigned)(last - first + 1), (unsigned)p.n_kv);
    const dim3 block((unsigned)(kBlock * (p.head_dim / 8)));
    if (dtype == KV_BF16)
        hipLaunchKernelGGL(rope_kernel<true>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(rope_kernel<false>, grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
