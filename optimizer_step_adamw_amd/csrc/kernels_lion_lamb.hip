// kernels_lion_lamb.hip -- Lion and LAMB step kernels (fp32 or bf16+remainder
// params, fp32 or bf16 grads), in the streaming layout of the AdamW kernels.
#include "device_common.h"

namespace optim {
namespace {

// ---------------------------------------------------------------- Lion
// [BNB] PR review: Lion applies decoupled decay to the parameter before its
// sign update.  Per element (Chen et al., arXiv:2302.06675), fp32, no
// contraction:
//   c = b1 m + c1 g;  p <- p (1 - lr wd) - lr sign(c);  m <- b2 m + c2 g
template <int N>
__device__ __forceinline__ void lion_math(float (&p)[N], const float (&g)[N], float (&m)[N], const AdamK &k,
                                          float lw) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float c = k.b1 * m[i] + k.c1 * g[i];
        const float s = c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f);
        p[i] = decayed(p[i], lw, k.lr * s);
        m[i] = k.b2 * m[i] + k.c2 * g[i];
    }
}

template <int PK, int GK, int N, class D>
__device__ __forceinline__ void lion_elems(const D &T, int64_t e, const AdamK &k, float lw) {
    float p[N], g[N], m[N];
    load_p<PK, N>(T, e, p);
    load_g<GK, N>(T.g, e, k.inv_scale, g);
    ldf<N>(T.m, e, m);
    lion_math<N>(p, g, m, k, lw);
    store_p<PK, N>(T, e, p);
    stf<N>(T.m, e, m);
}

// A lane's G groups of a pack (as adam_pack_load / adam_pack_finish).
template <int G>
struct LionRegs {
    float p[G][kVec], g[G][kVec], m[G][kVec];
};

template <int PK, int GK, int G>
__device__ __forceinline__ void lion_pack_load(const PackLds &L, const PackSlots<G> &sl, float gscale,
                                               LionRegs<G> &r) {
    if (!sl.whole) return;
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const PackMember &T = L.td[sl.j[q]];
        load_p<PK, kVec>(T, sl.e[q], r.p[q]);
        load_g<GK, kVec>(T.g, sl.e[q], gscale, r.g[q]);
        ldf<kVec>(T.m, sl.e[q], r.m[q]);
    }
}

template <int PK, int GK, int G>
__device__ __forceinline__ void lion_pack_finish(const PackLds &L, const PackSlots<G> &sl, const Scalars &S,
                                                 const AdamK &k, float rs, LionRegs<G> &r) {
    if (sl.whole) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int i = 0; i < kVec; ++i) r.g[q][i] = r.g[q][i] * rs;
            lion_math<kVec>(r.p[q], r.g[q], r.m[q], k, S.lrwd[L.td[sl.j[q]].group]);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const PackMember &T = L.td[sl.j[q]];
            store_p<PK, kVec>(T, sl.e[q], r.p[q]);
            stf<kVec>(T.m, sl.e[q], r.m[q]);
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
        if (sl.n[q] == 0) continue;
        const PackMember &T = L.td[sl.j[q]];
        const float lw = S.lrwd[T.group];
        if (sl.n[q] == kVec && T.vec_ok)
            lion_elems<PK, GK, kVec>(T, sl.e[q], k, lw);
        else
            for (int i = 0; i < sl.n[q]; ++i) lion_elems<PK, GK, 1>(T, sl.e[q] + i, k, lw);
    }
}

// EG > 0: the early-load form of the AdamW kernel (a whole unit of EG groups
// per lane loaded before the per-step prologue), for plans of at most
// kLionEarlyUnits units; the plan's unit size (2048 or 4096 elements) fixes
// EG.
template <int PK, int GK, int EG>
__global__ __launch_bounds__(kThreads) void lion_kernel(StepArgs a) {
    __shared__ Scalars S;
    constexpr int G = EG > 0 ? EG : kAdamGroups;
    constexpr int N = G * kVec;
    if (EG > 0 && a.unit0 + (int64_t)blockIdx.x < a.nunits) {
        const int64_t u = a.unit0 + blockIdx.x;
        int si = span_of(a, u);
        while (a.spans[si + 1].unit_begin <= u) ++si;
        const SpanDesc sp = a.spans[si];
        const int64_t off = (u - sp.unit_begin) * a.tile;
        const TensorDesc &T = a.tensors[sp.tensor];
        const int64_t start = sp.elem_begin + off;
        if (sp.len - off >= a.tile && T.vec_ok && start % kVec == 0) {
            const int64_t e = start + threadIdx.x * kVec;
            float p[N], g[N], m[N];
            load_p<PK, N>(T, e, p);
            load_g<GK, N>(T.g, e, 1.0f, g);
            ldf<N>(T.m, e, m);
            step_begin(a, S);
            const StepCommit commit{a, S};
            if (S.skip) return;
            const AdamK k = adam_consts(S);
#pragma unroll
            for (int i = 0; i < N; ++i) g[i] = g[i] * k.inv_scale;  // g * 1 * s == g * s
            lion_math<N>(p, g, m, k, uniform(S.lrwd[T.group]));
            store_p<PK, N>(T, e, p);
            stf<N>(T.m, e, m);
            return;
        }
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float lw = uniform(S.lrwd[T.group]);
        lane_walk<G>(start, len, T.vec_ok, [&](auto n, int64_t e) {
            lion_elems<PK, GK, decltype(n)::value>(T, e, k, lw);
        });
    });
}

constexpr int64_t kLionEarlyUnits = 4096;

// Packs of small tensors (as adam_pack_kernel).
template <int PK, int GK, int G>
__global__ __launch_bounds__(kThreads) void lion_pack_kernel(StepArgs a) {
    __shared__ Scalars S;
    __shared__ PackLds PL;
    if (a.grid_request == 0 && a.units_per_wg == 1 && a.unit0 + (int64_t)blockIdx.x < a.nunits) {
        const PackDesc P = a.packs[a.unit0 + blockIdx.x - a.pack_unit0];
        if (P.len <= G * kSub) {
            pack_fill(a, P, PL);
            const int32_t v0 = (int32_t)threadIdx.x * kVec;
            const bool mine = v0 < P.len;
            PackSlots<G> sl;
            LionRegs<G> r;
            if (mine) {
                sl = pack_slots<G>(PL, P, v0);
                lion_pack_load<PK, GK, G>(PL, sl, 1.0f, r);
            }
            step_begin(a, S);
            const StepCommit commit{a, S};
            if (S.skip) return;
            const AdamK k = adam_consts(S);
            if (mine) lion_pack_finish<PK, GK, G>(PL, sl, S, k, k.inv_scale, r);  // g * 1 * s == g * s
            return;
        }
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t, int64_t) {
        const PackDesc P = a.packs[sp.elem_begin];
        pack_fill(a, P, PL);
        for (int32_t v0 = (int32_t)threadIdx.x * kVec; v0 < P.len; v0 += G * (int32_t)kSub) {
            const PackSlots<G> sl = pack_slots<G>(PL, P, v0);
            LionRegs<G> r;
            lion_pack_load<PK, GK, G>(PL, sl, k.inv_scale, r);
            lion_pack_finish<PK, GK, G>(PL, sl, S, k, 1.0f, r);
        }
        __syncthreads();  // PL is refilled for the next pack
    });
}

// ---------------------------------------------------------------- LAMB
// You et al., arXiv:1904.00962, Algorithm 2, with Adam's direction as in the
// AdamW kernel ([BNB] PR description: LAMB shares the Adam kernels):
//   r = (m/bc1) / (sqrt(v)/sqrt(bc2) + eps),  u = r + wd p,
//   p <- p - lr (|p|/|u|) u   per tensor.
// Three kernels: moments + per-unit sums of p^2 and u^2 (from the previous
// p) -> per-tensor factor lr |p|/|u| (fixed-order fp64 sums) -> update,
// which recomputes u from the stored m, v and the untouched p with the same
// fp32 operations.
// groups of 4 elements per lane both passes load at once: a whole
// 4096-element unit (measured on MI355X, 4096^2: 113.4 us per step against
// 115.4 with two groups at a time)
constexpr int kLambGroups = 4;

__device__ __forceinline__ float lamb_u(float p, float m, float v, const AdamK &k, float wd) {
    const float h = sqrtf(v) * k.isb2 + k.eps;
    return (m * k.ibc1) / h + wd * p;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// KEEP: p, m and v, which the update pass reads again, go through ordinary
// accesses in both passes (kept in the Infinity Cache) and the update walks
// backwards.
template <int PK, int GK, bool KEEP>
__global__ __launch_bounds__(kThreads) void lamb_moments_kernel(StepArgs a) {
    constexpr int RL = KEEP ? kStridedKeep : kStrided;  // re-read by the update
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    __shared__ double red[2][kThreads / 64];
    for_units(a, [&](int64_t u, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float wd = uniform((float)a.prep.group_wd[T.group]);
        float sp2 = 0.0f, su2 = 0.0f;
        lane_walk<kLambGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
            constexpr int N = decltype(n)::value;
            float p[N], g[N], m[N], v[N];
            load_p<PK, N, RL>(T, e, p);
            load_g<GK, N>(T.g, e, k.inv_scale, g);
            ldf<N>(T.m, e, m);
            ldf<N>(T.v, e, v);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                m[i] = k.b1 * m[i] + k.c1 * g[i];
                v[i] = k.b2 * v[i] + k.c2 * (g[i] * g[i]);
                const float uu = lamb_u(p[i], m[i], v[i], k, wd);
                sp2 += p[i] * p[i];
                su2 += uu * uu;
            }
            stf<N, RL>(T.m, e, m);
            stf<N, RL>(T.v, e, v);
        });
        sp2 = wave_sum(sp2);
        su2 = wave_sum(su2);
        if ((threadIdx.x & 63) == 0) {
            red[0][threadIdx.x >> 6] = (double)sp2;
            red[1][threadIdx.x >> 6] = (double)su2;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double tp = 0.0, tu = 0.0;
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) {
                tp += red[0][w];
                tu += red[1][w];
            }
            a.partials[2 * u] = tp;
            a.partials[2 * u + 1] = tu;
        }
        __syncthreads();
    });
}

__global__ __launch_bounds__(kThreads) void lamb_trust_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    __shared__ double red[2][kThreads];
    for (int b = blockIdx.x; b < a.nblocks; b += gridDim.x) {
        const int si = a.blockspan[b];
        const int64_t u0 = a.spans[si].unit_begin, u1 = a.spans[si + 1].unit_begin;
        red[0][threadIdx.x] = lane_sum(a.partials, 2, u0, u1);
        red[1][threadIdx.x] = lane_sum(a.partials + 1, 2, u0, u1);
        __syncthreads();
        for (int st = kThreads / 2; st > 0; st >>= 1) {
            if ((int)threadIdx.x < st) {
                red[0][threadIdx.x] += red[0][threadIdx.x + st];
                red[1][threadIdx.x] += red[1][threadIdx.x + st];
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            const double pn = red[0][0], un = red[1][0];
            const double trust = (pn > 0.0 && un > 0.0) ? sqrt(pn) / sqrt(un) : 1.0;
            a.blockfac[b] = (float)(S.lr64 * trust);
        }
        __syncthreads();
    }
}

template <int PK, int GK, bool KEEP>
__global__ __launch_bounds__(kThreads) void lamb_update_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    constexpr int RL = KEEP ? kStridedKeep : kStrided;
    const AdamK k = adam_consts(S);
    for_units<KEEP>(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float wd = uniform((float)a.prep.group_wd[T.group]);
        const float f = a.blockfac[sp.block];
        lane_walk<kLambGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
            constexpr int N = decltype(n)::value;
            float p[N], m[N], v[N];
            load_p<PK, N, RL>(T, e, p);
            ldf<N, RL>(T.m, e, m);
            ldf<N, RL>(T.v, e, v);
#pragma unroll
            for (int i = 0; i < N; ++i) p[i] = p[i] - f * lamb_u(p[i], m[i], v[i], k, wd);
            store_p<PK, N>(T, e, p);
        });
    });
}

}  // namespace

template <int PK, int GK>
static void launch_lion_t(const StepArgs &args, hipStream_t s) {
    // units of single tensors [unit0, pack_unit0), then the packs
    StepArgs a = args;
    const bool packs = a.pack_unit0 < a.nunits;
    if (packs) {
        a.nunits = a.pack_unit0;
        a.commit = 0;  // the pack launch publishes the step
    }
    if (!packs || a.nunits > a.unit0) {
        const bool early = a.grid_request == 0 && a.units_per_wg == 1 && a.nunits - a.unit0 <= kLionEarlyUnits;
        if (early && a.tile == (int64_t)kAdamGroups * kSub)
            LAUNCH_PERSISTENT((lion_kernel<PK, GK, kAdamGroups>), a, s);
        else if (early && a.tile == (int64_t)kAdamGroupsEarly * kSub)
            LAUNCH_PERSISTENT((lion_kernel<PK, GK, kAdamGroupsEarly>), a, s);
        else
            LAUNCH_PERSISTENT((lion_kernel<PK, GK, 0>), a, s);
    }
    if (packs) {
        StepArgs b = args;
        b.unit0 = args.pack_unit0;
        static_assert(kPackElems == (int64_t)kAdamGroups * kSub, "a pack is one pass of the pack kernel");
        LAUNCH_PERSISTENT((lion_pack_kernel<PK, GK, kAdamGroups>), b, s);
    }
}

hipError_t launch_lion(const StepArgs &a, int pk, int gk, hipStream_t s) {
    if (pk == P_F32 && gk == G_F32)
        launch_lion_t<P_F32, G_F32>(a, s);
    else if (pk == P_F32 && gk == G_BF16)
        launch_lion_t<P_F32, G_BF16>(a, s);
    else if (pk == P_BF16R && gk == G_F32)
        launch_lion_t<P_BF16R, G_F32>(a, s);
    else
        launch_lion_t<P_BF16R, G_BF16>(a, s);
    return hipGetLastError();
}

template <int PK, int GK, bool KEEP>
hipError_t launch_lamb_t(const StepArgs &args, hipStream_t s) {
    // the moments and ratios read the step's inputs; the update publishes it
    StepArgs a = args;
    a.commit = 0;
    LAUNCH_PERSISTENT((lamb_moments_kernel<PK, GK, KEEP>), a, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.nblocks > 0) {
        const int fg = a.nblocks < 2048 ? a.nblocks : 2048;
        LAUNCH_TRACED(lamb_trust_kernel, fg, kThreads, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    a.commit = 1;
    LAUNCH_PERSISTENT((lamb_update_kernel<PK, GK, KEEP>), a, s);
    return hipGetLastError();
}

template <int PK, int GK>
hipError_t launch_lamb_keep(const StepArgs &a, hipStream_t s) {
    // p, m, v (12 bytes an element) are read again by the update; measured:
    // 4096x4096 (201 MB re-read) 6% faster kept, 4096x8192 no faster
    return keep_for_second_pass(a, 12, int64_t(256) << 20) ? launch_lamb_t<PK, GK, true>(a, s)
                                                            : launch_lamb_t<PK, GK, false>(a, s);
}

hipError_t launch_lamb(const StepArgs &a, int pk, int gk, hipStream_t s) {
    if (pk == P_F32 && gk == G_F32) return launch_lamb_keep<P_F32, G_F32>(a, s);
    if (pk == P_F32 && gk == G_BF16) return launch_lamb_keep<P_F32, G_BF16>(a, s);
    if (pk == P_BF16R && gk == G_F32) return launch_lamb_keep<P_BF16R, G_F32>(a, s);
    return launch_lamb_keep<P_BF16R, G_BF16>(a, s);
}

}  // namespace optim
