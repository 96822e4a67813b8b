// kernels_util.hip -- gradient non-finite check and bf16 + int16 remainder
// split / reconstruct.
#include "device_common.h"

namespace optim {
namespace {

// ---------------------------------------------------------------- finite check
// [LTN] analysis: found_inf marks a NaN or +-Inf anywhere in the gradients.
// A read-only scan: each workgroup takes kFiniteCheckElems elements (several
// consecutive units, merged into one walk where they are contiguous; packs
// of small tensors member by member).
// Measured on MI355X: bf16 gradients stream best with 8 groups of 4 per lane
// in flight (7.4 TB/s), fp32 with one group at a time (7.0 TB/s).
// NORM: the same pass also sums the squares of the (scaled) gradients into
// partials[workgroup]: per lane in fp32 (Acc = float), then across lanes and
// workgroups in fp64.  A loss-scaled gradient can be finite and still have
// an fp32 square of +inf (|G| above ~1.8e19): if any lane's fp32 sum
// overflows without the lane having met a NaN / Inf, the workgroup walks its
// range again summing exact fp64 squares (Acc = double), so finite gradients
// always give a finite norm and are clipped; only a NaN / Inf element, which
// sets found_inf, makes the norm non-finite.  (Squares in fp64 on every
// pass measured 13% slower on the 1.1B bf16 list: 373 against 330 us.)

// This lane's N gradient elements of T (a TensorDesc or a pack's PackMember)
// from element e (N = 1, or whole groups of 4 in the step layout).
template <int GK, bool NORM, int N, class Acc, class D>
__device__ __forceinline__ bool scan_elems(const D &T, int64_t e, Acc &acc) {
    bool bad = false;
    float x[N];
    if constexpr (GK == G_F32) {
        ldf<N>(static_cast<const float *>(T.g), e, x);
#pragma unroll
        for (int i = 0; i < N; ++i) bad |= (__float_as_uint(x[i]) & 0x7F800000u) == 0x7F800000u;
    } else {
        uint32_t w[N];
        ldh<N>(static_cast<const uint16_t *>(T.g), e, w);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            bad |= (w[i] & 0x7F80u) == 0x7F80u;
            x[i] = bf16_to_f32(w[i]);
        }
    }
    if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if constexpr (sizeof(Acc) == 8)
                acc = __builtin_fma((double)x[i], (double)x[i], acc);
            else
                acc += x[i] * x[i];
        }
    }
    return bad;
}

template <int GK, bool NORM, class Acc>
__device__ __forceinline__ bool scan_grads(const TensorDesc &T, int64_t start, int64_t len, Acc &acc) {
    // (the rare fp64 pass takes one group at a time: it must not raise the
    // kernel's register count)
    constexpr int G = (GK == G_F32 || sizeof(Acc) == 8) ? 1 : 8;
    bool bad = false;
    lane_walk<G>(start, len, T.vec_ok, [&](auto n, int64_t e) {
        bad |= scan_elems<GK, NORM, decltype(n)::value>(T, e, acc);
    });
    return bad;
}

// The workgroup's whole range; true if this lane met a NaN / Inf.
template <int GK, bool NORM, class Acc>
__device__ __forceinline__ bool scan_workgroup(const StepArgs &a, PackLds &PL, Acc &acc) {
    bool bad = false;
    int tensor = -1;
    int64_t start = 0, len = 0;
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t s, int64_t l) {
        if (sp.tensor == kPackTensor) {  // small tensors laid end to end
            const PackDesc P = a.packs[sp.elem_begin];
            pack_fill(a, P, PL);
            for (int32_t v0 = (int32_t)threadIdx.x * kVec; v0 < P.len; v0 += 2 * (int32_t)kSub) {
                const PackSlots<2> sl = pack_slots<2>(PL, P, v0);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const PackMember &T = PL.td[sl.j[q]];
                    if (sl.n[q] == kVec && T.vec_ok) {
                        bad |= scan_elems<GK, NORM, kVec>(T, sl.e[q], acc);
                    } else {
                        for (int j = 0; j < sl.n[q]; ++j) bad |= scan_elems<GK, NORM, 1>(T, sl.e[q] + j, acc);
                    }
                }
            }
            __syncthreads();  // PL is refilled for the next pack
            return;
        }
        if (sp.tensor == tensor && s == start + len) {
            len += l;
            return;
        }
        if (len > 0) bad |= scan_grads<GK, NORM>(a.tensors[tensor], start, len, acc);
        tensor = sp.tensor;
        start = s;
        len = l;
    });
    if (len > 0) bad |= scan_grads<GK, NORM>(a.tensors[tensor], start, len, acc);
    return bad;
}

template <int GK, bool NORM>
__global__ __launch_bounds__(kThreads) void finite_kernel(StepArgs a) {
    __shared__ PackLds PL;
    float acc32 = 0.0f;
    const bool bad = scan_workgroup<GK, NORM>(a, PL, acc32);
    if (bad) *a.found_inf = 1.0f;
    if constexpr (NORM) {
        double acc = (double)acc32;
        // a finite-gradient overflow of the fp32 sums: again in fp64
        if (__syncthreads_or(!bad && !(acc32 <= 3.4028234663852886e38f))) {
            acc = 0.0;
            scan_workgroup<GK, NORM>(a, PL, acc);
        }
        __shared__ double red[kThreads / 64];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t = 0.0;
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) t += red[w];
            a.partials[blockIdx.x] = t;
        }
    }
}

// The partial sums are added in a fixed order in two stages: workgroup w of
// stage 1 sums partials [w*kNormChunk, (w+1)*kNormChunk) (16 independent
// loads per lane) into partials2[w]; one workgroup then sums partials2 and
// derives
//   norm = sqrt(sum G^2) * s                 (the norm of the unscaled G s)
//   clip = s * min(1, max_norm / (norm + 1e-6))
// with s = *inv_scale (1 if absent).  No clipping when max_norm <= 0 or is
// +inf, or when the norm is not finite (found_inf is set and the step that
// reads clip is skipped).
constexpr int kNormPerLane = 16;
constexpr int64_t kNormChunk = (int64_t)kThreads * kNormPerLane;

__device__ __forceinline__ double block_sum(double x, double *red) {
    red[threadIdx.x] = x;
    __syncthreads();
    for (int st = kThreads / 2; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
        __syncthreads();
    }
    return red[0];
}

__global__ __launch_bounds__(kThreads) void norm_stage1_kernel(const double *partials, int64_t n,
                                                                double *partials2) {
    __shared__ double red[kThreads];
    const int64_t base = (int64_t)blockIdx.x * kNormChunk + threadIdx.x;
    double v[kNormPerLane];
#pragma unroll
    for (int j = 0; j < kNormPerLane; ++j) {
        const int64_t i = base + (int64_t)j * kThreads;
        v[j] = i < n ? partials[i] : 0.0;
    }
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kNormPerLane; ++j) acc += v[j];
    const double t = block_sum(acc, red);
    if (threadIdx.x == 0) partials2[blockIdx.x] = t;
}

__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(const double *partials2, int64_t n2,
                                                                  const float *inv_scale, double max_norm,
                                                                  float *norm_out, float *clip_out) {
    __shared__ double red[kThreads];
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < n2; i += kThreads) acc += partials2[i];
    const double total = block_sum(acc, red);
    if (threadIdx.x == 0) {
        const double s = inv_scale ? (double)*inv_scale : 1.0;
        const double norm = sqrt(total) * fabs(s);
        double coef = 1.0;
        if (max_norm > 0.0 && isfinite(max_norm) && isfinite(norm)) {
            const double c = max_norm / (norm + 1e-6);
            coef = c < 1.0 ? c : 1.0;
        }
        if (norm_out) *norm_out = (float)norm;
        *clip_out = (float)(s * coef);
    }
}

// Dynamic loss scale: backoff on a non-finite step (count reset), growth
// after `interval` clean steps (kept only if finite); each product in double,
// rounded once to the stored float.  inv_scale, if given, becomes 1/scale.
__global__ void scaler_kernel(float *scale, float *inv_scale, int32_t *tracker, const float *found_inf,
                              double growth, double backoff, int32_t interval) {
    if (threadIdx.x != 0) return;
    float S = *scale;
    int32_t k = *tracker;
    if (*found_inf != 0.0f) {
        S = (float)((double)S * backoff);
        k = 0;
    } else if (++k >= interval) {
        const float grown = (float)((double)S * growth);
        if (isfinite(grown)) S = grown;
        k = 0;
    }
    *scale = S;
    *tracker = k;
    if (inv_scale) *inv_scale = (float)(1.0 / (double)S);
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

// Without a persistent grid, a finite-check / norm workgroup takes
// kFiniteCheckElems consecutive elements (that many / tile units).
static int32_t finite_units_per_wg(int64_t tile) {
    return (int32_t)(tile >= kFiniteCheckElems ? 1 : kFiniteCheckElems / tile);
}

int64_t finite_pass_grid(int64_t nunits, int64_t tile, int32_t grid_request) {
    const int64_t units = nunits > 0 ? nunits : 1;
    if (grid_request > 0) return grid_request < units ? grid_request : units;
    const int64_t upw = finite_units_per_wg(tile);
    return (units + upw - 1) / upw;
}

int64_t norm_partials(int64_t nunits, int64_t tile, int32_t grid_request) {
    const int64_t g = finite_pass_grid(nunits, tile, grid_request);
    return g + (g + kNormChunk - 1) / kNormChunk;
}

hipError_t launch_check_finite(const StepArgs &args, int gk, hipStream_t s) {
    StepArgs a = args;
    a.units_per_wg = finite_units_per_wg(a.tile);
    if (gk == G_F32)
        LAUNCH_PERSISTENT((finite_kernel<G_F32, false>), a, s);
    else
        LAUNCH_PERSISTENT((finite_kernel<G_BF16, false>), a, s);
    return hipGetLastError();
}

hipError_t launch_grad_norm(const StepArgs &args, int gk, const float *inv_scale, double max_norm,
                            float *norm_out, float *clip_out, hipStream_t s) {
    StepArgs a = args;
    a.units_per_wg = finite_units_per_wg(a.tile);
    const int64_t grid = finite_pass_grid(a.nunits, a.tile, a.grid_request);
    const int64_t grid1 = (grid + kNormChunk - 1) / kNormChunk;
    if (grid + grid1 > a.npartials || grid != persistent_grid(0, a)) return hipErrorInvalidValue;
    if (gk == G_F32)
        LAUNCH_PERSISTENT((finite_kernel<G_F32, true>), a, s);
    else
        LAUNCH_PERSISTENT((finite_kernel<G_BF16, true>), a, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    double *partials2 = a.partials + grid;
    LAUNCH_TRACED(norm_stage1_kernel, (unsigned)grid1, kThreads, s, a.partials, grid, partials2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    LAUNCH_TRACED(norm_finalize_kernel, 1, kThreads, s, partials2, grid1, inv_scale, max_norm,
                       norm_out, clip_out);
    return hipGetLastError();
}

hipError_t launch_scaler_update(float *scale, float *inv_scale, int32_t *tracker, const float *found_inf,
                                double growth, double backoff, int32_t interval, hipStream_t s) {
    hipLaunchKernelGGL(scaler_kernel, dim3(1), dim3(64), 0, s, scale, inv_scale, tracker, found_inf, growth,
                       backoff, interval);
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
