// blend.hip -- token selection for selective recompute of a reused chunk.
//
// ["Research Paper Review : CACHE BLEND", section "Methods"]: a token whose
// precomputed KV differs most from its recomputed KV (its KV deviation) is the
// one that needs the cross-chunk attention it missed, and only the tokens of
// largest deviation are recomputed; the candidate set is wide at the first
// layer and narrowed at deeper ones. Two kernels:
//
//   deviation_kernel: squared L2 distance between recomputed rows and the
//     cached rows of the same tokens (all kv heads, K and V), accumulated in
//     fp64. A streaming kernel: it reads 4 * n_kv * head_dim elements per
//     token once. A group of L lanes (L = 64, or the power of two that covers
//     a token's 16-byte chunks when that is smaller) takes one token; the
//     differences of two pool-type values are exact in fp64, the squares are
//     summed with fma and reduced by xor shuffles inside the group.
//
//   topk_kernel: per segment, the k largest values, equal values taken in
//     increasing index order, written as ascending indices. One 1024-thread
//     workgroup per segment does an MSD radix select over order-preserving
//     64-bit keys (8 passes of 8 bits, leaving early once the remaining
//     count equals the matching count), then one ordered pass that takes
//     every key above the threshold prefix and the first k_rem keys equal to
//     it, with wave ballots for the in-order ranks. A segment of up to 16384
//     values is read once into registers (16 keys per thread, all loads in
//     flight together); longer ones are re-read (from L2) in every pass.
#include "internal.h"

namespace kvc {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_lo_d(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi_d(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

template <int ES>
__device__ __forceinline__ double chunk_dev(u32x4_t a, u32x4_t b, double acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (ES == 2) {
            const double d0 = bf16_lo_d(a[e]) - bf16_lo_d(b[e]);
            const double d1 = bf16_hi_d(a[e]) - bf16_hi_d(b[e]);
            acc = fma(d0, d0, acc);
            acc = fma(d1, d1, acc);
        } else {
            const double d0 = (double)__uint_as_float(a[e]) - (double)__uint_as_float(b[e]);
            acc = fma(d0, d0, acc);
        }
    }
    return acc;
}

template <int ES>
__global__ __launch_bounds__(256) void deviation_kernel(DeviationParams p) {
    const int cph = p.head_dim * ES / 16;  // 16-byte chunks per head row
    const int cpt = p.n_kv * cph;          // per token
    const int L = p.lanes;                 // lanes per token (power of two)
    const int lane = threadIdx.x & 63;
    const int sub = lane & (L - 1);
    const long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) / L;
    // rows of a group are uniform; a row past the end still joins the shuffles
    const bool live = row < p.n_rows;
    bool ok = false;
    int pid = 0, t = 0;
    if (live) {
        const int s = p.row_seq[row], pos = p.row_pos[row];
        if (s >= 0 && s < p.batch && pos >= 0 && pos < p.max_blocks * kBlock) {
            pid = p.tables[(size_t)s * p.max_blocks + pos / kBlock];
            t = pos % kBlock;
            ok = pid >= 0 && pid < p.num_blocks;
        }
    }
    double acc = 0.0;
    if (ok) {
        const u32x4_t *kr = reinterpret_cast<const u32x4_t *>(p.k_re) + (size_t)row * cpt;
        const u32x4_t *vr = reinterpret_cast<const u32x4_t *>(p.v_re) + (size_t)row * cpt;
        const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(p.k);
        const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(p.v);
        for (int c = sub; c < cpt; c += L) {
            const int h = c / cph, part = c - h * cph;
            const size_t pc = (((size_t)pid * p.n_kv + h) * kBlock + t) * cph + part;
            const u32x4_t a = __builtin_nontemporal_load(kr + c);
            const u32x4_t b = __builtin_nontemporal_load(kp + pc);
            const u32x4_t x = __builtin_nontemporal_load(vr + c);
            const u32x4_t y = __builtin_nontemporal_load(vp + pc);
            acc = chunk_dev<ES>(a, b, acc);
            acc = chunk_dev<ES>(x, y, acc);
        }
    }
    for (int off = L >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (live && sub == 0) p.out[row] = ok ? acc : -INFINITY;
}

hipError_t launch_deviation(int dtype, const DeviationParams &p, hipStream_t s) {
    if (p.n_rows == 0) return hipSuccess;
    const int threads = 256;
    const long lanes = (long)p.n_rows * p.lanes;
    const unsigned blocks = (unsigned)((lanes + threads - 1) / threads);
    if (dtype == KV_BF16)
        hipLaunchKernelGGL(deviation_kernel<2>, dim3(blocks), dim3(threads), 0, s, p);
    else
        hipLaunchKernelGGL(deviation_kernel<4>, dim3(blocks), dim3(threads), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k selection
// ---------------------------------------------------------------------------

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkRegKeys = 16;     // keys per thread held in registers: segments up to 16384

// Order-preserving key: larger value, larger key; both zeros map to +0's key.
__device__ __forceinline__ uint64_t order_key(double x) {
    uint64_t b = (uint64_t)__double_as_longlong(x == 0.0 ? 0.0 : x);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Histogram add for one wave: the lanes that share the first active lane's
// digit are counted with a single atomic (early passes put most keys in one
// or two bins, where per-lane atomics on one address serialize).
__device__ __forceinline__ void hist_add(int *hist, int digit, bool active) {
    const uint64_t act = __ballot(active);
    if (act == 0) return;
    const int first = __ffsll((long long)act) - 1;  // uniform
    const int d0 = __builtin_amdgcn_readlane(digit, first);
    const uint64_t same = __ballot(active && digit == d0);
    const int lane = threadIdx.x & 63;
    if (lane == first) atomicAdd(&hist[d0], __popcll(same));
    else if (active && digit != d0) atomicAdd(&hist[digit], 1);
}

// Exclusive prefix counts of two flags over the workgroup in thread order:
// returns this thread's ranks and the workgroup totals.
__device__ __forceinline__ void block_rank2(bool fa, bool fb, int2 *wave_tot, int &ra, int &rb, int &ta, int &tb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t ba = __ballot(fa), bb = __ballot(fb);
    const uint64_t below = (1ull << lane) - 1ull;
    if (lane == 0) wave_tot[w] = make_int2(__popcll(ba), __popcll(bb));
    __syncthreads();
    ra = __popcll(ba & below);
    rb = __popcll(bb & below);
    ta = tb = 0;
    for (int i = 0; i < kTopkWaves; ++i) {
        const int2 v = wave_tot[i];
        ra += i < w ? v.x : 0;
        rb += i < w ? v.y : 0;
        ta += v.x;
        tb += v.y;
    }
    __syncthreads();  // wave_tot is reused by the next call
}

struct TopkShared {
    int hist[256];
    int2 wave_tot[kTopkWaves];
    int sel_digit, sel_gt, sel_eq;
};

// Select the k largest of n keys (0 < k < n) and write their indices in
// ascending order. key_of(j) is this thread's key of index j * 1024 + tid
// (called only for indices below n). MAXJ > 0: the chunk loops run over
// j < MAXJ, unrolled, so that key_of may read a register array; MAXJ == 0:
// j < ceil(n / 1024).
template <int MAXJ, class KeyFn>
__device__ __forceinline__ void topk_segment(int n, int k, KeyFn key_of, int32_t *out, TopkShared &sh) {
    const int tid = threadIdx.x;
    const int chunks = MAXJ > 0 ? MAXJ : (n + kTopkThreads - 1) / kTopkThreads;
    uint64_t prefix = 0, mask = 0;
    int k_rem = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
        if (tid < 256) sh.hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < chunks; ++j) {
            if (j * kTopkThreads < n) {  // uniform
                const int i = j * kTopkThreads + tid;
                uint64_t key = 0;
                bool m = false;
                if (i < n) {
                    key = key_of(j);
                    m = ((key ^ prefix) & mask) == 0;
                }
                hist_add(sh.hist, (int)((key >> shift) & 255), m);
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 4l..4l+3; count of larger digits from the top
            int c[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = sh.hist[4 * tid + q];
                tot += c[q];
            }
            int suf = tot;  // inclusive suffix sum of the lane totals
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_down(suf, off, 64);
                if (tid + off < 64) suf += v;
            }
            int gt = suf - tot;  // keys with a larger digit than this lane's bins
#pragma unroll
            for (int q = 3; q >= 0; --q) {
                if (gt < k_rem && gt + c[q] >= k_rem) {
                    sh.sel_digit = 4 * tid + q;
                    sh.sel_gt = gt;
                    sh.sel_eq = c[q];
                }
                gt += c[q];
            }
        }
        __syncthreads();
        prefix |= (uint64_t)sh.sel_digit << shift;
        mask |= (uint64_t)255 << shift;
        k_rem -= sh.sel_gt;
        const int eq = sh.sel_eq;
        __syncthreads();
        if (eq == k_rem) break;  // every key with this prefix is taken
    }

    // ordered pass: every key above the prefix, and the first k_rem keys equal
    // to it; a selected key's slot is (keys above before it) + min(keys equal
    // before it, k_rem)
    int above_seen = 0, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < chunks; ++j) {
        if (j * kTopkThreads < n) {  // uniform
            const int i = j * kTopkThreads + tid;
            bool above = false, equal = false;
            if (i < n) {
                const uint64_t key = key_of(j) & mask;
                above = key > prefix;
                equal = key == prefix;
            }
            int ra, re, ta, te;
            block_rank2(above, equal, sh.wave_tot, ra, re, ta, te);
            const int eq_before = eq_seen + re;
            const bool sel = above || (equal && eq_before < k_rem);
            if (sel) out[above_seen + ra + min(eq_before, k_rem)] = i;
            above_seen += ta;
            eq_seen += te;
        }
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
    __shared__ TopkShared sh;
    const int s = blockIdx.x, tid = threadIdx.x;
    const int begin = p.offsets[s], end = p.offsets[s + 1];
    const int n = end - begin;
    if (n <= 0) return;
    const int k = min(max(p.ks[s], 0), n);
    if (k == 0) return;
    const double *vals = p.values + begin;
    int32_t *out = p.selected + begin;
    if (k == n) {
        for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
        return;
    }
    if (n <= kTopkRegKeys * kTopkThreads) {
        // every key in registers: all loads issued at once, passes touch no memory
        uint64_t kr[kTopkRegKeys];
#pragma unroll
        for (int j = 0; j < kTopkRegKeys; ++j) {
            const int i = j * kTopkThreads + tid;
            kr[j] = i < n ? order_key(vals[i]) : 0;
        }
        topk_segment<kTopkRegKeys>(n, k, [&](int j) { return kr[j]; }, out, sh);
    } else {
        topk_segment<0>(n, k, [&](int j) { return order_key(vals[j * kTopkThreads + tid]); }, out, sh);
    }
}

hipError_t launch_topk(const TopkParams &p, hipStream_t s) {
    if (p.n_seg == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(p.n_seg), dim3(kTopkThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
