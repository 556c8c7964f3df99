// append.hip -- kv_append for fp32 / bf16 pools.
//
// One decode step appends one token per sequence: k_t, v_t go after
// K_{1:t-1}, V_{1:t-1} ["KV Cache는 왜 LLM 서빙의 핵심인가", section
// "KV Cache: O(T²)를 O(T)로", decode-step listing], i.e. into physical block
// tables[b][L / 16], slot L % 16 of the block pool ["LLM 서빙과 KV Cache, vLLM",
// section "PagedAttention"].
//
// Work: 2 * batch * n_new * n_kv rows of head_dim elements, moved in 16-byte
// chunks, one chunk per thread; consecutive threads take consecutive chunks of
// a row, so both the read of k_new/v_new and the write into the tile are
// coalesced. Token t of sequence b goes to position seq_lens[b] + t.
#include "internal.h"

namespace kvc {

template <int ES>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int cpr = p.head_dim * ES / 16;  // 16-byte chunks per row
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)p.batch * p.n_new * p.n_kv * 2 * cpr;
    if (i >= total) return;
    const int c = (int)(i % cpr);
    long r = i / cpr;
    const int which = (int)(r % 2);  // 0: K, 1: V
    r /= 2;
    const int h = (int)(r % p.n_kv);
    r /= p.n_kv;
    const int t_new = (int)(r % p.n_new);
    const int b = (int)(r / p.n_new);
    const int L0 = p.seq_lens[b];
    if (!append_fits(L0, p.n_new, p.max_blocks)) return;  // the chunk must fit the table
    const int L = L0 + t_new;
    const int pid = p.tables[(size_t)b * p.max_blocks + L / kBlock];
    if (pid < 0 || pid >= p.num_blocks) return;
    const int t = L % kBlock;
    const size_t row_bytes = (size_t)p.head_dim * ES;
    const char *src = (const char *)(which ? p.v_new : p.k_new) + (((size_t)b * p.n_new + t_new) * p.n_kv + h) * row_bytes;
    char *dst = (char *)(which ? p.pool.v : p.pool.k) + (((size_t)pid * p.n_kv + h) * kBlock + t) * row_bytes;
    reinterpret_cast<uint4 *>(dst)[c] = reinterpret_cast<const uint4 *>(src)[c];
}

hipError_t launch_append_int4(const AppendParams &p, hipStream_t s);

hipError_t launch_append(int dtype, const AppendParams &p, hipStream_t s) {
    if (dtype == KV_INT4) return launch_append_int4(p, s);
    const int es = dtype == KV_F32 ? 4 : 2;
    const long total = (long)p.batch * p.n_new * p.n_kv * 2 * (p.head_dim * es / 16);
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const unsigned blocks = (unsigned)((total + threads - 1) / threads);
    if (es == 4)
        hipLaunchKernelGGL(append_kernel<4>, dim3(blocks), dim3(threads), 0, s, p);
    else
        hipLaunchKernelGGL(append_kernel<2>, dim3(blocks), dim3(threads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
