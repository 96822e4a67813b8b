// kernels_adam.hip -- AdamW and AdEMAMix step kernels (fp32 or bf16+remainder params,
// fp32 or bf16 grads).
#include "device_common.h"

namespace optim {
namespace {

// The tensor descriptor a unit works with: a copy in scalar registers
// (uniform_desc: the unit's stores issue back to back) for bf16 + remainder
// params, and for fp32 masters with a 16-bit model copy in the early-load
// form; otherwise a reference into the plan's table, which the compiler
// re-reads after each array's stores and waits for them first.  Measured on
// MI355X in one process on the same arrays, table reference against
// register copy: bf16 + remainder 2^28 elements 1174.7 / 1163.6 us, the
// Llama-1.1B list 5352 / 5223 us, with interleaved moments 1228.9 / 1136.6
// and 5484 / 4830 us; fp32 master + bf16 copy 4096^2 (early form) 82.6 /
// 80.7 us, 2^28 1288.5 / 1355.1 us; fp32 4096^2 78.4 / 82.1 us, fp32 2^28
// 1252.5 / 1283.2 us (with interleaved moments 1224.3 / 1253.7 us) -- the
// fp32 steps stream faster with their stores spaced out by those waits.
template <int PK, int EG>
constexpr bool kDescInRegs = PK == P_BF16R || (EG > 0 && (PK == P_MBF16 || PK == P_MF16));

template <int PK, int EG, class F>
__device__ __forceinline__ void with_desc(const TensorDesc &T, F &&f) {
    if constexpr (kDescInRegs<PK, EG>) f(uniform_desc(T));
    else f(T);
}

// EG > 0 (early form): a workgroup whose unit is one whole, aligned tile of
// EG groups per lane (EG * 1024 elements) issues all of the unit's loads
// before the per-step prologue, so their latency overlaps the scalar loads
// and fp64 arithmetic.  Plans up to ~2 resident waves of workgroups take it
// (see kEarlyLoadUnits): 2048-element units of 2 groups for lists up to
// 2^20 elements, 4096-element units of 4 groups above that up to 2^24.
// Measured on MI355X with two state sets alternating (nothing cached),
// against 2048-element units of two groups without early loads: AdamW 2^22
// elements 22.5 -> 20.9 us, 2^23 42.1 -> 40.6 us, 2^24 80.8 -> 79.3 us;
// AdEMAMix 28.8 -> 26.3, 54.9 -> 51.9, 104.2 -> 103.6 us.  From 2^25
// elements on early loads of new workgroups crowd the stores of the
// finishing ones (2^26: AdamW 311.7 -> 317.5 us; re-timed in one process
// on the same arrays, early loads on 2048- / 4096-element units against
// none: fp32 2^26 320.9 / 309.9 against 304.7 us, 2^28 1305.9 / 1275.0
// against 1235.8 us, bf16 + remainder 2^28 1264.0 / 1234.1 against 1143.6
// us, the 1.1B-element bf16 + remainder list 5179 / 5301 against 5070 us),
// so larger plans take 2048-element units of 2 groups without them
// (EG = 0).  The plan picks the unit size by its element count and the
// launcher the form by the units.
//
// MI: the plan's interleaved moment layout (moment_at).
template <int PK, int GK, bool ADE, int EG, bool MI>
__global__ __launch_bounds__(kThreads) void adam_kernel(StepArgs a) {
    __shared__ Scalars S;
    constexpr int G = EG > 0 ? EG : kAdamGroups;
    constexpr int N = G * kVec;
    // (an empty plan still launches one workgroup, which has no unit)
    if (EG > 0 && a.unit0 + (int64_t)blockIdx.x < a.nunits) {
        const int64_t u = a.unit0 + blockIdx.x;
        int si = span_of(a, u);
        while (a.spans[si + 1].unit_begin <= u) ++si;
        const SpanDesc sp = a.spans[si];
        const int64_t off = (u - sp.unit_begin) * a.tile;
        const TensorDesc &Tt = a.tensors[sp.tensor];
        const int64_t start = sp.elem_begin + off;
        if (sp.len - off >= a.tile && Tt.vec_ok && start % kVec == 0) {
            with_desc<PK, EG>(Tt, [&](const TensorDesc &T) {
                const int64_t e = start + threadIdx.x * kVec;
                AdamRegs<N> r;
                adam_load<PK, GK, ADE, N, MI>(T, e, 1.0f, r);
                step_begin(a, S);
                const StepCommit commit{a, S};
                if (S.skip) return;
                const AdamK k = adam_consts(S);
#pragma unroll
                for (int i = 0; i < N; ++i) r.g[i] = r.g[i] * k.inv_scale;  // g * 1 * s == g * s
                adam_math<ADE, N>(r, k, uniform(S.lrwd[T.group]));
                adam_store<PK, ADE, N, MI>(T, e, r);
            });
            return;
        }
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        with_desc<PK, EG>(a.tensors[sp.tensor], [&](const TensorDesc &T) {
            adam_unit<PK, GK, ADE, G, MI>(T, start, len, k, uniform(S.lrwd[T.group]));
        });
    });
}

// Up to this many units the early-load form is used.
constexpr int64_t kEarlyLoadUnits = 4096;

// Packs of small tensors (the plan's units from pack_unit0 on; see
// PackDesc), G groups of 4 elements per lane and pass.  On the default grid
// a workgroup takes one pack and, when the pack fits one pass (always: a
// pack holds at most kPackElems = G * 1024 elements), copies its tables to
// LDS and issues the lanes' loads before the per-step prologue, as the early
// form above; otherwise (persistent grid) it walks its packs after the
// prologue.  Measured on MI355X, 2^24 AdamW elements as 65536 tensors of
// 256 (four state sets in turn): one workgroup per tensor 285.7 us; packs
// of 16 tensors (4096-element units) in the step kernel itself 115.7 us;
// in kernels of their own, with the member descriptors in LDS and the loads
// before the prologue, 89.6 us with 4096-element packs and 84.5 us with
// 2048-element packs (see kPackElems).
template <int PK, int GK, bool ADE, int G>
__global__ __launch_bounds__(kThreads) void adam_pack_kernel(StepArgs a) {
    __shared__ Scalars S;
    __shared__ PackLds PL;
    if (a.grid_request == 0 && a.units_per_wg == 1 && a.unit0 + (int64_t)blockIdx.x < a.nunits) {
        const PackDesc P = a.packs[a.unit0 + blockIdx.x - a.pack_unit0];
        if (P.len <= G * kSub) {
            pack_fill(a, P, PL);
            const int32_t v0 = (int32_t)threadIdx.x * kVec;
            const bool mine = v0 < P.len;
            PackSlots<G> sl;
            AdamRegs<kVec> r[G];
            if (mine) {
                sl = pack_slots<G>(PL, P, v0);
                adam_pack_load<PK, GK, ADE, G>(PL, sl, 1.0f, r);
            }
            step_begin(a, S);
            const StepCommit commit{a, S};
            if (S.skip) return;
            const AdamK k = adam_consts(S);
            if (mine) adam_pack_finish<PK, GK, ADE, G>(PL, sl, S, k, k.inv_scale, r);  // g * 1 * s == g * s
            return;
        }
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t, int64_t) { adam_pack_unit<PK, GK, ADE, G>(a, sp, PL, S, k); });
}

}  // namespace

// MI: the plan's interleaved moment layout (pack members are one moment
// block each, so the pack kernel needs no variant)
template <bool ADE, int PK, int GK, bool MI>
static void launch_adam_mi(const StepArgs &args, hipStream_t s) {
    // units of single tensors [unit0, pack_unit0), then the packs
    StepArgs a = args;
    const bool packs = a.pack_unit0 < a.nunits;
    if (packs) {
        a.nunits = a.pack_unit0;
        a.commit = 0;  // the pack launch publishes the step
    }
    if (!packs || a.nunits > a.unit0) {
        // the early form needs one whole tile of its groups per lane per
        // workgroup: the default grid over 2048- or 4096-element units
        const bool early = a.grid_request == 0 && a.units_per_wg == 1 && a.nunits - a.unit0 <= kEarlyLoadUnits;
        if (early && a.tile == (int64_t)kAdamGroups * kSub)
            LAUNCH_PERSISTENT((adam_kernel<PK, GK, ADE, kAdamGroups, MI>), a, s);
        else if (early && a.tile == (int64_t)kAdamGroupsEarly * kSub)
            LAUNCH_PERSISTENT((adam_kernel<PK, GK, ADE, kAdamGroupsEarly, MI>), a, s);
        else
            LAUNCH_PERSISTENT((adam_kernel<PK, GK, ADE, 0, MI>), a, s);
    }
    if (packs) {
        StepArgs b = args;
        b.unit0 = args.pack_unit0;
        static_assert(kPackElems == (int64_t)kAdamGroups * kSub, "a pack is one pass of the pack kernel");
        LAUNCH_PERSISTENT((adam_pack_kernel<PK, GK, ADE, kAdamGroups>), b, s);
    }
}

template <bool ADE, int PK, int GK>
static void launch_adam_g(const StepArgs &a, hipStream_t s) {
    if (a.interleaved)
        launch_adam_mi<ADE, PK, GK, true>(a, s);
    else
        launch_adam_mi<ADE, PK, GK, false>(a, s);
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
