// hostcheck_stubs.cpp -- stand-ins for the kernel launchers of the HIP
// library, for a host-only build of api.cpp under the address and
// undefined-behaviour sanitizers (tests/test_sanitizers.py). Every launcher
// aborts: the argument checks the host tests drive must return before any
// launch. The grid helpers return what the library returns when no device
// is present.
#include <cstdio>
#include <cstdlib>

#include "internal.h"
#include "window.h"

namespace kvc {

[[noreturn]] static void reached(const char *what) {
    std::fprintf(stderr, "host-check build: %s reached a kernel launch\n", what);
    std::abort();
}

hipError_t launch_deviation(int, const DeviationParams &, hipStream_t) { reached("launch_deviation"); }
hipError_t launch_topk(const TopkParams &, hipStream_t) { reached("launch_topk"); }
hipError_t launch_copy_blocks(const CopyParams &, hipStream_t) { reached("launch_copy_blocks"); }
hipError_t launch_window_released(const int32_t *, int, int, int32_t *, hipStream_t) {
    reached("launch_window_released");
}
hipError_t launch_append(int, const AppendParams &, hipStream_t) { reached("launch_append"); }
hipError_t launch_attention(int, int, const AttnParams &, hipStream_t, hipEvent_t, hipEvent_t) {
    reached("launch_attention");
}
hipError_t launch_merge(const AttnParams &, hipStream_t, hipEvent_t) { reached("launch_merge"); }
hipError_t launch_attention_shared(const AttnParams &, const PrefixArgs &, hipStream_t, hipEvent_t, hipEvent_t,
                                   hipEvent_t) {
    reached("launch_attention_shared");
}
hipError_t launch_quantize_int4(const QuantParams &, hipStream_t) { reached("launch_quantize_int4"); }
hipError_t launch_rope(int, const RopeParams &, hipStream_t) { reached("launch_rope"); }
hipError_t launch_read_probe(const void *, size_t, int, uint32_t *, hipStream_t) { reached("launch_read_probe"); }

void *noalloc_scratch() { reached("noalloc_scratch"); }

int balanced_grid(int dtype, int, int, int, bool q4_one_score) { return 256 * (dtype == KV_INT4 && q4_one_score ? 3 : 2); }
int wide_grid(int, int ctw, int, int) { return 1024 / ctw; }
size_t shared_balanced_lds(int n_groups, int batch, int max_blocks) {
    return (size_t)(2 * (n_groups + 1) + batch + 1 + (max_blocks < 256 ? max_blocks : 256)) * sizeof(int);
}
int shared_balanced_grid(int, size_t) { return 256 * 2; }

}  // namespace kvc
