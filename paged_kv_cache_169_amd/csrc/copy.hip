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

typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk

// One workgroup per listed block: region by region, 256 threads move the
// region's 16-byte chunks, four loads in flight per thread before the
// stores; all index arithmetic in 32 bits within a block. Loads and stores
// are non-temporal: no byte is touched twice, so none is kept in the caches.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
    const int k = blockIdx.x;
    const int sblk = p.mode == 2 ? 0 : p.src[k];
    const int dblk = p.mode == 1 ? 0 : p.dst[k];
    if (p.mode != 2 && (sblk < 0 || sblk >= p.num_blocks)) return;
    if (p.mode != 1 && (dblk < 0 || dblk >= p.num_blocks)) return;
    const chunk_t *buf_in = reinterpret_cast<const chunk_t *>(p.buffer) + (size_t)k * p.per_block;
    chunk_t *buf_out = reinterpret_cast<chunk_t *>(p.buffer) + (size_t)k * p.per_block;
    uint32_t packed = 0;  // chunks of the packed block before region r
    for (int r = 0; r < p.nreg; ++r) {
        const uint32_t n = p.chunks[r];
        const chunk_t *src = p.mode == 2 ? buf_in + packed
                                          : reinterpret_cast<const chunk_t *>(p.region[r]) + (size_t)sblk * n;
        chunk_t *dst = p.mode == 1 ? buf_out + packed : reinterpret_cast<chunk_t *>(p.region[r]) + (size_t)dblk * n;
        for (uint32_t c0 = threadIdx.x; c0 < n; c0 += 4 * blockDim.x) {
            chunk_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t c = c0 + u * blockDim.x;
                if (c < n) v[u] = __builtin_nontemporal_load(src + c);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t c = c0 + u * blockDim.x;
                if (c < n) __builtin_nontemporal_store(v[u], dst + c);
            }
        }
        packed += n;
    }
}

hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t s) {
    if (p.n <= 0 || p.per_block == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)p.n), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
