// numerics_check.hip -- device checks of the step library's own numeric
// helpers, for the test suite (not part of the C ABI of liboptim_step.so).
// Built with the step library's floating-point flags (no contraction, IEEE
// fp32 division, denormals kept) and its device header, so the function
// checked is the one the step kernels inline.
#include "device_common.h"

namespace {

// optim::recip_rn (Markstein's corrected hardware reciprocal inside
// [2^-126, 2^126], IEEE division elsewhere) against the IEEE quotient 1/a,
// for the 2^24 bit patterns whose top byte is `top`.  Only a > 0 is checked:
// the blockwise step takes the reciprocal of a positive block maximum.
__global__ __launch_bounds__(256) void recip_check_kernel(uint32_t top, unsigned long long *mismatches,
                                                          unsigned long long *fast_path) {
    const uint32_t bits = (top << 24) | (blockIdx.x * 256u + threadIdx.x);
    const float a = __uint_as_float(bits);
    if (!(a > 0.0f)) return;
    const float want = 1.0f / a;
    const float got = optim::recip_rn(a);
    if (__float_as_uint(want) != __float_as_uint(got)) atomicAdd(mismatches, 1ull);
    if (a >= 0x1p-126f && a <= 0x1p126f && threadIdx.x == 0) atomicAdd(fast_path, 256ull);
}

}  // namespace

extern "C" {
// Runs the check for top bytes [top_begin, top_end) (each a grid of 2^24
// threads); mismatches and fast_path are device counters the caller zeroes.
int check_recip_rn(uint32_t top_begin, uint32_t top_end, unsigned long long *mismatches,
                   unsigned long long *fast_path, void *stream) {
    if (top_end > 256 || top_begin > top_end) return -1;
    for (uint32_t t = top_begin; t < top_end; ++t)
        hipLaunchKernelGGL(recip_check_kernel, dim3(65536), dim3(256), 0, static_cast<hipStream_t>(stream), t,
                           mismatches, fast_path);
    return (int)hipGetLastError();
}
}
