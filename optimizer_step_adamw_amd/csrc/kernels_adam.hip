// kernels_adam.hip -- AdamW and AdEMAMix step kernels (fp32 or bf16+remainder params,
// fp32 or bf16 grads).
#include "device_common.h"

namespace optim {
namespace {

template <int PK, int GK, bool ADE>
__global__ __launch_bounds__(kThreads) void adam_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        adam_unit<PK, GK, ADE>(T, start, len, k, uniform(S.decay[T.group]));
    });
}

}  // namespace

template <bool ADE, int PK>
static void launch_adam_pk(const StepArgs &a, int gk, hipStream_t s) {
    if (gk == G_F32)
        LAUNCH_PERSISTENT((adam_kernel<PK, G_F32, ADE>), a, s);
    else
        LAUNCH_PERSISTENT((adam_kernel<PK, G_BF16, ADE>), a, s);
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
