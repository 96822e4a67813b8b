// kernels_mini.hip -- Adam-mini step kernels: per-unit block sums of g^2,
// per-block finalize, elementwise update.
#include "device_common.h"

namespace optim {
namespace {

// ---------------------------------------------------------------- Adam-mini
// [MINI] AdamWMini.step, q/k and "other" branches: one v per block of the
// flattened gradient, updated with the block mean of g^2.  Three kernels:
// per-unit partial sums of g^2 -> per-block finalize (fixed-order fp64 sum,
// v update, step factor) -> elementwise m/p update.
//
// The three run once per segment of the list (whole tensors holding at most
// a bounded number of gradient bytes, 384 MiB by default), not once over the
// whole list.  The sum pass reads g with ordinary loads, so much of a
// segment's g is still in the 256 MB Infinity Cache when its update pass
// reads it again right after; the update then takes mostly p, m (and v)
// from HBM.  Measured on MI355X for one 180 MB-gradient tensor after
// non-temporal traffic: the ordinary-load sum costs what a non-temporal one
// does (28.8 vs 27.6 us) and the update drops from 150.5 to 124.6 us; on the
// Llama-7B-shaped list the step drops from 28.1 to 25.8 ms.
constexpr int32_t kMiniSumUnitsPerWg = 2;
// groups of 4 elements per lane the block sums and the update load at once:
// a whole 4096-element unit (measured on MI355X, segmented 7B list: 25.0 ms
// per step against 25.4 with two groups at a time; again in one process on
// the same arrays, the update with two groups at a time: 24.92 against
// 25.27 ms)
constexpr int kMiniGroups = 4;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Block sums of one unit: partials[u] = sum of g^2 over the unit (fp32 per
// lane, fp64 across the wavefronts).  g stays in the Infinity Cache for the
// update pass that follows (ordinary loads).  Called by every thread.
template <int GK>
__device__ __forceinline__ void mini_sums_unit(const StepArgs &a, float s, int64_t u, const SpanDesc &sp,
                                               int64_t start, int64_t len, double *red) {
    constexpr int LAY = kStridedKeep;
    if (sp.block < 0) return;  // full-v tensor: no shared block
    const TensorDesc &T = a.tensors[sp.tensor];
    float acc = 0.0f;
    lane_walk<kMiniGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
        constexpr int N = decltype(n)::value;
        float g[N];
        load_g<GK, N, LAY>(T.g, e, s, g);
#pragma unroll
        for (int i = 0; i < N; ++i) acc += g[i] * g[i];
    });
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (double)acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) t += red[w];
        a.partials[u] = t;
    }
    __syncthreads();
}

// Early form (default grid): when both of a workgroup's units are whole,
// aligned 4096-element units of shared-v blocks, their gradients are
// loaded before the per-step prologue (unscaled; the scale is applied after
// it, g * s as in load_g) and the two sums share one reduction round.
template <int GK>
__global__ __launch_bounds__(kThreads) void mini_sumsq_kernel(StepArgs a) {
    constexpr int P = kMiniSumUnitsPerWg;
    constexpr int N = kMiniGroups * kVec;
    __shared__ Scalars S;
    __shared__ double red[P][kThreads / 64];
    if (a.grid_request == 0 && a.units_per_wg == P && a.tile == (int64_t)kMiniGroups * kSub) {
        const int64_t u0 = a.unit0 + (int64_t)blockIdx.x * P;
        bool whole = u0 + P <= a.nunits;
        const TensorDesc *T[P];
        int64_t e[P];
        if (whole) {
            int si = span_of(a, u0);
#pragma unroll
            for (int q = 0; q < P; ++q) {
                while (a.spans[si + 1].unit_begin <= u0 + q) ++si;
                const SpanDesc sp = a.spans[si];
                const int64_t off = (u0 + q - sp.unit_begin) * a.tile;
                T[q] = &a.tensors[sp.tensor];
                e[q] = sp.elem_begin + off;
                whole = whole && sp.block >= 0 && sp.len - off >= a.tile && T[q]->vec_ok && e[q] % kVec == 0;
                e[q] += threadIdx.x * kVec;
            }
        }
        if (whole) {
            float g[P][N];
#pragma unroll
            for (int q = 0; q < P; ++q) load_g<GK, N, kStridedKeep>(T[q]->g, e[q], 1.0f, g[q]);
            step_begin(a, S);
            const StepCommit commit{a, S};
            if (S.skip) return;
            const float s = S.inv_scale;
            float acc[P];
#pragma unroll
            for (int q = 0; q < P; ++q) {
                acc[q] = 0.0f;
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    const float x = g[q][i] * s;  // g * 1 * s == g * s
                    acc[q] += x * x;
                }
                acc[q] = wave_sum(acc[q]);
                if ((threadIdx.x & 63) == 0) red[q][threadIdx.x >> 6] = (double)acc[q];
            }
            __syncthreads();
            if (threadIdx.x < P) {
                double t = 0.0;
#pragma unroll
                for (int w = 0; w < kThreads / 64; ++w) t += red[threadIdx.x][w];
                a.partials[u0 + threadIdx.x] = t;
            }
            return;
        }
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const float s = S.inv_scale;
    for_units(a, [&](int64_t u, const SpanDesc &sp, int64_t start, int64_t len) {
        mini_sums_unit<GK>(a, s, u, sp, start, len, red[0]);
    });
}

// Per block b of [block0, nblocks): V_b <- beta2 V_b + (1 - beta2) mean(g^2)
// (fixed-order fp64 sum of the unit partials: per lane, then across each
// wave, then over the four waves), step factor lr/bc1 / h_b.  The first
// block's partial sums, and in thread 0 the chain block -> span -> tensor ->
// V_b, are loaded before the per-step prologue (if the step turns out
// skipped they are not used).
__global__ __launch_bounds__(kThreads) void mini_finalize_kernel(StepArgs a) {
    __shared__ Scalars S;
    static_assert(kThreads == 256, "the cross-wave sum below adds four waves");
    __shared__ double red[kThreads / 64];
    int b = a.block0 + blockIdx.x;
    const auto block_sum = [&](int blk) {
        const int si = a.blockspan[blk];
        return lane_sum(a.partials, 1, a.spans[si].unit_begin, a.spans[si + 1].unit_begin);
    };
    struct BlockV {
        float *v;
        float old;
        int64_t len;
    };
    const auto block_v = [&](int blk) {
        const SpanDesc sp = a.spans[a.blockspan[blk]];
        const TensorDesc &T = a.tensors[sp.tensor];
        float *v = T.v + sp.elem_begin / T.block_len;
        return BlockV{v, *v, sp.len};
    };
    double part = 0.0;
    BlockV bv{nullptr, 0.0f, 1};
    if (b < a.nblocks) {
        part = block_sum(b);
        if (threadIdx.x == 0) bv = block_v(b);
    }
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    for (bool first = true; b < a.nblocks; b += gridDim.x, first = false) {
        double x = first ? part : block_sum(b);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
        __syncthreads();
        if (threadIdx.x == 0) {
            if (!first) bv = block_v(b);
            const double mean = ((red[0] + red[1]) + (red[2] + red[3])) / (double)bv.len;
            const double V = S.beta2_64 * (double)bv.old + S.c2_64 * mean;
            *bv.v = (float)V;
            const double h = sqrt(V) * S.inv_sqrt_bc2_64 + S.eps64;
            a.blockfac[b] = (float)(S.step_size64 / h);
        }
        __syncthreads();
    }
}

template <int PK, int GK, int N>
__device__ __forceinline__ void mini_elems(const TensorDesc &T, int64_t e, const AdamK &k,
                                           float lw, float f) {
    float p[N], g[N], m[N];
    load_p<PK, N>(T, e, p);
    load_g<GK, N>(T.g, e, k.inv_scale, g);
    ldf<N>(T.m, e, m);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        m[i] = k.b1 * m[i] + k.c1 * g[i];
        p[i] = decayed(p[i], lw, f * m[i]);
    }
    store_p<PK, N>(T, e, p);
    stf<N>(T.m, e, m);
}

// Update of one unit: full-v tensors as AdamW, shared-v blocks with their
// block's factor.
template <int PK, int GK>
__device__ __forceinline__ void mini_update_unit(const StepArgs &a, const Scalars &S, const AdamK &k,
                                                 const SpanDesc &sp, int64_t start, int64_t len) {
    const TensorDesc &T = a.tensors[sp.tensor];
    const float lw = uniform(S.lrwd[T.group]);
    if (sp.block < 0) {
        adam_unit<PK, GK, false, kMiniGroups>(T, start, len, k, lw);
        return;
    }
    const float f = a.blockfac[sp.block];
    lane_walk<kMiniGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
        mini_elems<PK, GK, decltype(n)::value>(T, e, k, lw, f);
    });
}

// The update walks its units backwards, meeting first the g lines the block
// sums read last.  Timed in one process on the same arrays (7B list) this
// is no faster than the forward walk (24.88 against 24.86 ms per step): how
// much of a segment's g the Infinity Cache still holds does not depend on
// the order here.
template <int PK, int GK>
__global__ __launch_bounds__(kThreads) void mini_update_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units<true>(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        mini_update_unit<PK, GK>(a, S, k, sp, start, len);
    });
}

}  // namespace

template <int PK, int GK>
static void launch_mini_update(const StepArgs &a, hipStream_t s) {
    LAUNCH_PERSISTENT((mini_update_kernel<PK, GK>), a, s);
}

static hipError_t launch_mini_update_kind(const StepArgs &a, int pk, int gk, hipStream_t s) {
    if (pk == P_F32 && gk == G_F32)
        launch_mini_update<P_F32, G_F32>(a, s);
    else if (pk == P_F32 && gk == G_BF16)
        launch_mini_update<P_F32, G_BF16>(a, s);
    else if (pk == P_BF16R && gk == G_F32)
        launch_mini_update<P_BF16R, G_F32>(a, s);
    else
        launch_mini_update<P_BF16R, G_BF16>(a, s);
    return hipGetLastError();
}

// Per segment: block sums, finalize, update.  Measured on MI355X (7B list):
// one launch holding a segment's update and the next segment's block sums
// (its workgroups after the update's) took 25.06 ms per step against 24.68
// ms for separate launches -- the next segment's g, streamed into the
// Infinity Cache during the update, evicts the current segment's.
hipError_t launch_adam_mini(const StepArgs &args, int pk, int gk, const MiniSegment *segs, int32_t nsegs,
                            hipStream_t s) {
    // every launch reads the step's inputs; the last update publishes it
    StepArgs a = args;
    a.commit = 0;
    if (nsegs == 0) {  // empty plan: one workgroup commits
        a.unit0 = a.nunits = 0;
        a.commit = 1;
        return launch_mini_update_kind(a, pk, gk, s);
    }
    for (int32_t i = 0; i < nsegs; ++i) {
        const MiniSegment &sg = segs[i];
        a.unit0 = sg.unit_begin;
        a.nunits = sg.unit_end;
        if (sg.block_end > sg.block_begin) {
            // the read-only sum pass streams better with 2 consecutive units
            // per workgroup (measured on MI355X, segmented 7B list: 25.5 ms
            // per step against 26.0 with 1, 25.8 with 4, 26.3 with 8 or 16;
            // in one process on the same arrays, with the early form, 24.88
            // against 25.31 ms with 4)
            if (a.grid_request == 0) a.units_per_wg = kMiniSumUnitsPerWg;
            if (gk == G_F32)
                LAUNCH_PERSISTENT((mini_sumsq_kernel<G_F32>), a, s);
            else
                LAUNCH_PERSISTENT((mini_sumsq_kernel<G_BF16>), a, s);
            a.units_per_wg = args.units_per_wg;
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            a.block0 = sg.block_begin;
            a.nblocks = sg.block_end;
            const int nb = sg.block_end - sg.block_begin;
            LAUNCH_TRACED(mini_finalize_kernel, nb < 2048 ? nb : 2048, kThreads, s, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        a.commit = i == nsegs - 1 ? 1 : 0;
        const hipError_t e = launch_mini_update_kind(a, pk, gk, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace optim
