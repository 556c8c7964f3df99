// window.hip -- the blocks a limited attention window has left behind ("KV
// 캐시 시스템 (KV Cache System)", section "제한된 어텐션 윈도우 크기": blocks
// outside the window are released for reuse): one thread per sequence reads
// its length and writes how many leading table entries no later query can
// attend (window_released in internal.h).
#include "window.h"

namespace kvc {

__global__ __launch_bounds__(256) void window_released_kernel(const int32_t *lens, int batch, int window,
                                                              int32_t *out) {
    const int b = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (b < batch) out[b] = window_released(lens[b], window);
}

hipError_t launch_window_released(const int32_t *lens, int batch, int window, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(window_released_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, lens, batch, window, out);
    return hipGetLastError();
}

}  // namespace kvc
