// kernels_adam.hip -- AdamW and AdEMAMix step kernels (fp32 or bf16+remainder params,
// fp32 or bf16 grads).
#include "device_common.h"

namespace optim {
namespace {

// EARLY: a workgroup whose unit is one whole, aligned tile (one group of
// loads per lane) issues the unit's loads before the per-step prologue, so
// their latency overlaps the scalar loads and fp64 arithmetic.  Measured on
// MI355X: 5-10% faster up to ~2 resident waves of workgroups (8M elements:
// AdamW 41.9 -> 39.1 us, AdEMAMix 54.3 -> 51.4 us), 1-6% slower from 12M
// elements on, where the early loads of new workgroups crowd the stores of
// the finishing ones -- so the launcher chooses by size.
template <int PK, int GK, bool ADE, bool EARLY>
__global__ __launch_bounds__(kThreads) void adam_kernel(StepArgs a) {
    __shared__ Scalars S;
    constexpr int N = kAdamGroups * kVec;
    // (an empty plan still launches one workgroup, which has no unit)
    if (EARLY && a.unit0 + (int64_t)blockIdx.x < a.nunits) {
        const int64_t u = a.unit0 + blockIdx.x;
        int si = span_of(a, u);
        while (a.spans[si + 1].unit_begin <= u) ++si;
        const SpanDesc sp = a.spans[si];
        const int64_t off = (u - sp.unit_begin) * a.tile;
        const TensorDesc &T = a.tensors[sp.tensor];
        const int64_t start = sp.elem_begin + off;
        if (sp.len - off >= a.tile && T.vec_ok && start % kVec == 0) {
            const int64_t e = start + threadIdx.x * kVec;
            AdamRegs<N> r;
            adam_load<PK, GK, ADE, N>(T, e, 1.0f, r);
            step_begin(a, S);
            const StepCommit commit{a, S};
            if (S.skip) return;
            const AdamK k = adam_consts(S);
#pragma unroll
            for (int i = 0; i < N; ++i) r.g[i] = r.g[i] * k.inv_scale;  // g * 1 * s == g * s
            adam_math<ADE, N>(r, k, uniform(S.lrwd[T.group]));
            adam_store<PK, ADE, N>(T, e, r);
            return;
        }
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        adam_unit<PK, GK, ADE>(T, start, len, k, uniform(S.lrwd[T.group]));
    });
}

// Up to this many units (2048 elements each) the early-load form is used.
constexpr int64_t kEarlyLoadUnits = 4096;

}  // namespace

template <bool ADE, int PK, int GK>
static void launch_adam_g(const StepArgs &a, hipStream_t s) {
    // the early form needs one whole tile of one group per lane per
    // workgroup: the default grid over 2048-element units
    const bool early = a.grid_request == 0 && a.units_per_wg == 1 && a.tile == (int64_t)kAdamGroups * kSub &&
                       a.nunits <= kEarlyLoadUnits;
    if (early)
        LAUNCH_PERSISTENT((adam_kernel<PK, GK, ADE, true>), a, s);
    else
        LAUNCH_PERSISTENT((adam_kernel<PK, GK, ADE, false>), a, s);
}

template <bool ADE, int PK>
static void launch_adam_pk(const StepArgs &a, int gk, hipStream_t s) {
    if (gk == G_F32)
        launch_adam_g<ADE, PK, G_F32>(a, s);
    else
        launch_adam_g<ADE, PK, G_BF16>(a, s);
}

template <bool ADE>
static hipError_t launch_adam_t(const StepArgs &a, int pk, int gk, hipStream_t s) {
    switch (pk) {
    case P_F32: launch_adam_pk<ADE, P_F32>(a, gk, s); break;
    case P_BF16R: launch_adam_pk<ADE, P_BF16R>(a, gk, s); break;
    case P_MBF16: launch_adam_pk<ADE, P_MBF16>(a, gk, s); break;
    default: launch_adam_pk<ADE, P_MF16>(a, gk, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_adamw(const StepArgs &a, int pk, int gk, hipStream_t s) {
    return launch_adam_t<false>(a, pk, gk, s);
}

hipError_t launch_ademamix(const StepArgs &a, int pk, int gk, hipStream_t s) {
    return launch_adam_t<true>(a, pk, gk, s);
}

}  // namespace optim
