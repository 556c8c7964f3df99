// copy.hip -- whole-block copies: inside a pool (copy before a reusing request
// writes into a shared block, "KV 캐시 시스템 (KV Cache System)", section
// "부분 재사용") and between a pool and a packed buffer in device or pinned
// host memory (offload and restore, section "호스트 메모리로의 오프로딩").
//
// A block's packed form is its slice of every per-block region in region
// order. One thread moves one 16-byte chunk; consecutive threads take
// consecutive chunks of a block, so both sides are coalesced. A pure streaming
// kernel: every byte is read once and written once.
#include "internal.h"

namespace kvc {

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)p.n * p.per_block;
    if (i >= total) return;
    const int k = (int)(i / p.per_block);
    uint32_t c = (uint32_t)(i % p.per_block);  // chunk within the packed block
    int r = 0;
    while (r < p.nreg - 1 && c >= p.chunks[r]) {
        c -= p.chunks[r];
        ++r;
    }
    const size_t in_region = (size_t)c * 16;
    if (p.mode == 2) {  // buffer -> block
        const int d = p.dst[k];
        if (d < 0 || d >= p.num_blocks) return;
        const uint4 v = reinterpret_cast<const uint4 *>(p.buffer)[i];
        *reinterpret_cast<uint4 *>(p.region[r] + (size_t)d * p.chunks[r] * 16 + in_region) = v;
        return;
    }
    const int sblk = p.src[k];
    if (sblk < 0 || sblk >= p.num_blocks) return;
    const uint4 v = *reinterpret_cast<const uint4 *>(p.region[r] + (size_t)sblk * p.chunks[r] * 16 + in_region);
    if (p.mode == 1) {  // block -> buffer
        reinterpret_cast<uint4 *>(p.buffer)[i] = v;
    } else {            // block -> block
        const int d = p.dst[k];
        if (d < 0 || d >= p.num_blocks) return;
        *reinterpret_cast<uint4 *>(p.region[r] + (size_t)d * p.chunks[r] * 16 + in_region) = v;
    }
}

hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t s) {
    const long total = (long)p.n * p.per_block;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
