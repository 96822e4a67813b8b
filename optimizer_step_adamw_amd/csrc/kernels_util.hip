// kernels_util.hip -- gradient non-finite check and bf16 + int16 remainder
// split / reconstruct.
#include "device_common.h"

namespace optim {
namespace {

// ---------------------------------------------------------------- finite check
// [LTN] analysis: found_inf marks a NaN or +-Inf anywhere in the gradients.
template <int GK>
__global__ __launch_bounds__(kThreads) void finite_kernel(StepArgs a) {
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const bool vec = T.vec_ok && (start % 8 == 0);
        bool bad = false;
        for (int64_t rel = threadIdx.x * 8; rel < len; rel += kThreads * 8) {
            const int64_t e = start + rel;
            if constexpr (GK == G_F32) {
                const uint32_t *g = static_cast<const uint32_t *>(T.g);
                if (vec && rel + 8 <= len) {
                    const uint4 *q = reinterpret_cast<const uint4 *>(g + e);
                    const uint4 x = q[0], y = q[1];
                    const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) bad |= (w[i] & 0x7F800000u) == 0x7F800000u;
                } else {
                    const int64_t n = len - rel < 8 ? len - rel : 8;
                    for (int64_t j = 0; j < n; ++j) bad |= (g[e + j] & 0x7F800000u) == 0x7F800000u;
                }
            } else {
                const uint16_t *g = static_cast<const uint16_t *>(T.g);
                if (vec && rel + 8 <= len) {
                    uint32_t w[8];
                    ldh<8>(g, e, w);
#pragma unroll
                    for (int i = 0; i < 8; ++i) bad |= (w[i] & 0x7F80u) == 0x7F80u;
                } else {
                    const int64_t n = len - rel < 8 ? len - rel : 8;
                    for (int64_t j = 0; j < n; ++j) bad |= (g[e + j] & 0x7F80u) == 0x7F80u;
                }
            }
        }
        if (bad) *a.found_inf = 1.0f;
    });
}

// ---------------------------------------------------------------- remainder utils
__global__ __launch_bounds__(kThreads) void split_kernel(const float *x, uint16_t *b, int16_t *r,
                                                         int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        uint32_t bb, rr;
        rem_split(x[i], bb, rr);
        b[i] = (uint16_t)bb;
        r[i] = (int16_t)(uint16_t)rr;
    }
}

__global__ __launch_bounds__(kThreads) void reconstruct_kernel(const uint16_t *b,
                                                               const int16_t *r, float *x,
                                                               int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        x[i] = rem_reconstruct(b[i], (uint16_t)r[i]);
}

int flat_grid(int64_t n) {
    int64_t g = (n + kThreads - 1) / kThreads;
    return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_check_finite(const StepArgs &args, int gk, hipStream_t s) {
    // a read-only scan streams best with ~8192 elements per workgroup
    StepArgs a = args;
    a.units_per_wg = (int32_t)(a.tile >= kFiniteCheckElems ? 1 : kFiniteCheckElems / a.tile);
    if (gk == G_F32)
        LAUNCH_PERSISTENT((finite_kernel<G_F32>), a, s);
    else
        LAUNCH_PERSISTENT((finite_kernel<G_BF16>), a, s);
    return hipGetLastError();
}


hipError_t launch_remainder_split(const float *x, uint16_t *b, int16_t *r, int64_t n,
                                  hipStream_t s) {
    hipLaunchKernelGGL(split_kernel, dim3(flat_grid(n)), dim3(kThreads), 0, s, x, b, r, n);
    return hipGetLastError();
}

hipError_t launch_remainder_reconstruct(const uint16_t *b, const int16_t *r, float *x,
                                        int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(reconstruct_kernel, dim3(flat_grid(n)), dim3(kThreads), 0, s, b, r, x, n);
    return hipGetLastError();
}

}  // namespace optim
