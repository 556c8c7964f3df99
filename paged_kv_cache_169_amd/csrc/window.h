// window.h -- the blocks a limited attention window has left behind ("KV 캐시
// 시스템 (KV Cache System)", section "제한된 어텐션 윈도우 크기"): the
// per-sequence count (host and device) and the launcher of window.hip.
#pragma once

#include "internal.h"

namespace kvc {

// Leading blocks of a sequence of L tokens that no later query can attend
// under a window of `window` tokens (0: all tokens): a later query at
// position >= L attends positions >= L + 1 - window. -1 for a negative L.
__host__ __device__ inline int window_released(int L, int window) {
    if (L < 0) return -1;
    if (window <= 0) return 0;
    const long long dead = (long long)L + 1 - window;  // tokens before the window
    return dead > 0 ? (int)(dead / kBlock) : 0;
}

hipError_t launch_window_released(const int32_t *lens, int batch, int window, int32_t *out, hipStream_t s);

}  // namespace kvc
