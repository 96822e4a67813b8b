// kernels.hip -- gfx950 kernels of the fused, multi-tensor AdamW-family
// optimizer step.
//
// The step is elementwise and HBM-bound (a few flops per byte), so there is
// no matrix-core work here.  Every step kernel is a persistent grid: each
// workgroup owns a contiguous range of work units (kTile elements of one
// span) and walks it with 128-bit loads and stores, 8 consecutive elements
// per lane.  Per-step scalars come from the Scalars record the prep kernel
// writes at the start of the step (uniform loads).
//
// Sources (web pages, by title and section):
//  [BNB]  "Fix decoupled weight decay ordering in the CUDA Adam/AdEMAMix
//         kernels" (bitsandbytes PR #2040): decay before the update
//         (Loshchilov & Hutter Algorithm 2 order); AdEMAMix; blockwise 8-bit.
//  [AO]   "4 bit Adam should support non constant lr" (pytorch/ao #730):
//         device-resident lr, cosine schedule, 4-bit states.
//  [MINI] "Adam-mini <> DTensor" (Adam-mini #14): AdamWMini.step.
//  [LTN]  "FusedAdam & PyTorch Lightning AMP" (Lightning #15501): in-step
//         unscale and found_inf skip.
//  [TE]   "Support store_param_remainders feature from Apex in TE Fused
//         Adam" (TransformerEngine PR #1408): bf16 + int16 remainder.
//
// Build flags: -ffp-contract=off (every multiply and add below rounds on
// its own, as written), IEEE division and sqrt, fp32 denormals kept.
#include "plan.h"

#include <math.h>

namespace optim {
namespace {

constexpr double kPi = 3.141592653589793;

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// [TE] description: the fp32 master is rebuilt from the bf16 param b and the
// int16 remainder r.  Encoding: r = low half of the master's bits; b = high
// half + carry (bit 15 of r), so the carry is undone before concatenating.
__device__ __forceinline__ float rem_reconstruct(uint32_t b, uint32_t r) {
    const uint32_t c = (r >> 15) & 1u;
    return __uint_as_float((((b - c) & 0xFFFFu) << 16) | (r & 0xFFFFu));
}

__device__ __forceinline__ void rem_split(float x, uint32_t &b, uint32_t &r) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t lo = u & 0xFFFFu;
    b = ((u >> 16) + (lo >> 15)) & 0xFFFFu;
    r = lo;
}

// ---------------------------------------------------------------- loads
// Every tensor lives in HBM: accesses go through global-address-space
// pointers so they compile to global_load/store (not flat) instructions.
// N = 8: two 128-bit accesses (fp32) or one (16-bit); N = 1: one element.
#define GMEM __attribute__((address_space(1)))
typedef float __attribute__((ext_vector_type(4))) f32x4;
typedef uint32_t __attribute__((ext_vector_type(4))) u32x4;
typedef uint32_t __attribute__((ext_vector_type(2))) u32x2;

template <class T>
__device__ __forceinline__ GMEM T *gp(T *p) { return (GMEM T *)p; }
template <class T>
__device__ __forceinline__ const GMEM T *gp(const T *p) { return (const GMEM T *)p; }

#ifndef OPTIM_NT
#define OPTIM_NT 0  // 1: nontemporal 128-bit loads and stores
#endif
template <class V>
__device__ __forceinline__ V vload(const GMEM V *q) {
#if OPTIM_NT
    return __builtin_nontemporal_load(q);
#else
    return *q;
#endif
}
template <class V>
__device__ __forceinline__ void vstore(GMEM V *q, V x) {
#if OPTIM_NT
    __builtin_nontemporal_store(x, q);
#else
    *q = x;
#endif
}

template <int N>
__device__ __forceinline__ void ldf(const float *a, int64_t e, float (&x)[N]) {
    if constexpr (N == 8) {
        const GMEM f32x4 *q = (const GMEM f32x4 *)gp(a + e);
        const f32x4 u = vload(q), w = vload(q + 1);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
    } else if constexpr (N == 4) {
        const f32x4 u = *(const GMEM f32x4 *)gp(a + e);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    } else {
        const GMEM float *q = gp(a);
#pragma unroll
        for (int k = 0; k < N; ++k) x[k] = q[e + k];
    }
}

template <int N>
__device__ __forceinline__ void stf(float *a, int64_t e, const float (&x)[N]) {
    if constexpr (N == 8) {
        GMEM f32x4 *q = (GMEM f32x4 *)gp(a + e);
        vstore(q, f32x4{x[0], x[1], x[2], x[3]});
        vstore(q + 1, f32x4{x[4], x[5], x[6], x[7]});
    } else if constexpr (N == 4) {
        *(GMEM f32x4 *)gp(a + e) = f32x4{x[0], x[1], x[2], x[3]};
    } else {
        GMEM float *q = gp(a);
#pragma unroll
        for (int k = 0; k < N; ++k) q[e + k] = x[k];
    }
}

template <int N>
__device__ __forceinline__ void ldh(const uint16_t *a, int64_t e, uint32_t (&x)[N]) {
    if constexpr (N == 8) {
        const u32x4 u = vload((const GMEM u32x4 *)gp(a + e));
        x[0] = u.x & 0xFFFFu; x[1] = u.x >> 16; x[2] = u.y & 0xFFFFu; x[3] = u.y >> 16;
        x[4] = u.z & 0xFFFFu; x[5] = u.z >> 16; x[6] = u.w & 0xFFFFu; x[7] = u.w >> 16;
    } else if constexpr (N == 4) {
        const u32x2 u = *(const GMEM u32x2 *)gp(a + e);
        x[0] = u.x & 0xFFFFu; x[1] = u.x >> 16; x[2] = u.y & 0xFFFFu; x[3] = u.y >> 16;
    } else {
        const GMEM uint16_t *q = gp(a);
#pragma unroll
        for (int k = 0; k < N; ++k) x[k] = q[e + k];
    }
}

template <int N>
__device__ __forceinline__ void sth(uint16_t *a, int64_t e, const uint32_t (&x)[N]) {
    if constexpr (N == 8) {
        vstore((GMEM u32x4 *)gp(a + e),
               u32x4{(x[0] & 0xFFFFu) | (x[1] << 16), (x[2] & 0xFFFFu) | (x[3] << 16),
                     (x[4] & 0xFFFFu) | (x[5] << 16), (x[6] & 0xFFFFu) | (x[7] << 16)});
    } else if constexpr (N == 4) {
        *(GMEM u32x2 *)gp(a + e) = u32x2{(x[0] & 0xFFFFu) | (x[1] << 16), (x[2] & 0xFFFFu) | (x[3] << 16)};
    } else {
        GMEM uint16_t *q = gp(a);
#pragma unroll
        for (int k = 0; k < N; ++k) q[e + k] = (uint16_t)x[k];
    }
}

template <int PK, int N>
__device__ __forceinline__ void load_p(const TensorDesc &T, int64_t e, float (&p)[N]) {
    if constexpr (PK == P_F32) {
        ldf<N>(static_cast<const float *>(T.p), e, p);
    } else {
        uint32_t b[N], r[N];
        ldh<N>(static_cast<const uint16_t *>(T.p), e, b);
        ldh<N>(T.rem, e, r);
#pragma unroll
        for (int k = 0; k < N; ++k) p[k] = rem_reconstruct(b[k], r[k]);
    }
}

template <int PK, int N>
__device__ __forceinline__ void store_p(const TensorDesc &T, int64_t e, const float (&p)[N]) {
    if constexpr (PK == P_F32) {
        stf<N>(static_cast<float *>(T.p), e, p);
    } else {
        uint32_t b[N], r[N];
#pragma unroll
        for (int k = 0; k < N; ++k) rem_split(p[k], b[k], r[k]);
        sth<N>(static_cast<uint16_t *>(T.p), e, b);
        sth<N>(T.rem, e, r);
    }
}

// Gradient load with the AMP unscale applied exactly once ([LTN] analysis).
template <int GK, int N>
__device__ __forceinline__ void load_g(const void *g, int64_t e, float s, float (&x)[N]) {
    if constexpr (GK == G_F32) {
        ldf<N>(static_cast<const float *>(g), e, x);
    } else {
        uint32_t b[N];
        ldh<N>(static_cast<const uint16_t *>(g), e, b);
#pragma unroll
        for (int k = 0; k < N; ++k) x[k] = bf16_to_f32(b[k]);
    }
#pragma unroll
    for (int k = 0; k < N; ++k) x[k] = x[k] * s;
}

// ---------------------------------------------------------------- traversal
// Calls body(u, span, first element, element count) for every unit u this
// workgroup owns.  All arguments are uniform across the workgroup.
// OPTIM_TRAVERSAL 1 (default): grid-stride -- workgroup b takes units b,
// b+G, b+2G, ..., so the resident workgroups sweep one contiguous window of
// each array at a time (DRAM pages stay local).  0: one contiguous range of
// units per workgroup.
#ifndef OPTIM_TRAVERSAL
#define OPTIM_TRAVERSAL 1
#endif
__device__ __forceinline__ int span_of(const StepArgs &a, int64_t u) {
    int lo = 0, hi = a.nspans;  // spans[nspans].unit_begin == nunits > u
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.spans[mid].unit_begin <= u) lo = mid; else hi = mid;
    }
    return lo;
}

template <class Body>
__device__ __forceinline__ void for_units(const StepArgs &a, Body &&body) {
    const int64_t G = gridDim.x, b = blockIdx.x;
#if OPTIM_TRAVERSAL == 0
    int64_t u = a.nunits * b / G;
    const int64_t u1 = a.nunits * (b + 1) / G, stride = 1;
#else
    int64_t u = b;
    const int64_t u1 = a.nunits, stride = G;
#endif
    if (u >= u1) return;
    int s = span_of(a, u);
    for (; u < u1; u += stride) {
        while (a.spans[s + 1].unit_begin <= u) ++s;
        const SpanDesc sp = a.spans[s];
        const int64_t off = (u - sp.unit_begin) * kTile;
        const int64_t len = sp.len - off < kTile ? sp.len - off : kTile;
        body(u, sp, sp.elem_begin + off, len);
    }
}

// ---------------------------------------------------------------- per-step scalars
// Bias corrections and step sizes in fp64, rounded once to fp32: in fp32,
// 1 - beta2^t cancels badly at small t, and fast power/divide intrinsics put
// a kernel micro-units off the closed form ([BNB] PR body).  beta^t is taken
// by repeated squaring (t is an integer; a few ulp of fp64 at most).  The lr
// is read from a device scalar (or computed from the device iteration
// counter for the cosine schedule), never passed from the host per step
// ([AO]).
__device__ __forceinline__ double ipow(double b, int32_t t) {
    double r = 1.0;
    for (; t > 0; t >>= 1) {
        if (t & 1) r *= b;
        b *= b;
    }
    return r;
}

// Thread 0 derives the step's scalars into LDS; the caller then reads them
// back as wave-uniform values.
__device__ __forceinline__ void step_begin(const StepArgs &a, Scalars &S) {
    const PrepArgs &p = a.prep;
    if (threadIdx.x == 0) {
        float lr;
        int32_t k = 0;
        if (p.sched == 1) {
            k = *p.iter_dev;
            const int32_t kk = k < 0 ? 0 : (k < p.K ? k : p.K);
            const double x = (double)kk / (double)p.K;
            lr = (float)(p.lr_min + (p.lr_max - p.lr_min) * 0.5 * (1.0 + cos(kPi * x)));
        } else {
            lr = *p.lr_dev;
        }
        const int skip = (p.found_inf != nullptr) && (*p.found_inf != 0.0f);
        const int32_t t = *p.step_dev + 1;
        const double bc1 = 1.0 - ipow(p.beta1, t);
        const double bc2 = 1.0 - ipow(p.beta2, t);
        const double lr64 = (double)lr;
        const double rs2 = 1.0 / sqrt(bc2);
        S.skip = skip;
        S.t = t;
        S.k = k;
        S.lr = lr;
        S.step_size = (float)(lr64 / bc1);
        S.inv_sqrt_bc2 = (float)rs2;
        S.inv_bc1 = (float)(1.0 / bc1);
        S.b1 = (float)p.beta1;
        S.c1 = (float)(1.0 - p.beta1);
        S.b2 = (float)p.beta2;
        S.c2 = (float)(1.0 - p.beta2);
        S.b3 = (float)p.beta3;
        S.c3 = (float)(1.0 - p.beta3);
        S.alpha = (float)p.alpha;
        S.eps = (float)p.eps;
        S.inv_scale = p.inv_scale ? *p.inv_scale : 1.0f;
        S.lr64 = lr64;
        S.step_size64 = lr64 / bc1;
        S.inv_sqrt_bc2_64 = rs2;
        S.eps64 = p.eps;
        S.beta2_64 = p.beta2;
        S.c2_64 = 1.0 - p.beta2;
    }
    __syncthreads();
    if ((int)threadIdx.x < p.ngroups)
        S.decay[threadIdx.x] = (float)(1.0 - S.lr64 * p.group_wd[threadIdx.x]);
    __syncthreads();
}

// Commit: every workgroup read the step counter, lr and iteration in its
// prologue, before it arrives here; the last workgroup to arrive publishes
// t (unless the step was skipped), the scheduled lr and k + 1, and rearms the
// counters.  Arrivals go through kSubCounters counters on separate lines and
// then one top counter, so no single address takes every workgroup's atomic.
// Ordering: the only requirement is that every prologue load has returned
// before its workgroup arrives, so a workgroup-scope fence (a wait on
// outstanding memory operations) precedes a relaxed device-scope RMW.  An
// acquire/release RMW at device scope would instead write back and
// invalidate the XCD's L2 in every workgroup.
__device__ __forceinline__ uint32_t arrive(uint32_t *c) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void step_end(const StepArgs &a, const Scalars &S) {
    if (!a.commit || threadIdx.x != 0) return;
    const uint32_t G = gridDim.x, b = blockIdx.x;
    const uint32_t nsub = G < (uint32_t)kSubCounters ? G : (uint32_t)kSubCounters;
    const uint32_t j = b % nsub;
    const uint32_t members = G / nsub + (j < G % nsub ? 1u : 0u);
    uint32_t *sub = a.done + (1 + j) * kCounterStride;
    if (arrive(sub) != members - 1) return;
    __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (arrive(a.done) != nsub - 1) return;
    __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const PrepArgs &p = a.prep;
    if (p.sched == 1) {
        *p.lr_dev = S.lr;
        *p.iter_dev = S.k + 1;
    }
    if (!S.skip) *p.step_dev = S.t;
}

// Runs the commit on every exit path of a step kernel (skipped steps too).
struct StepCommit {
    const StepArgs &a;
    const Scalars &S;
    __device__ ~StepCommit() { step_end(a, S); }
};

__device__ __forceinline__ float uniform(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// ---------------------------------------------------------------- AdamW / AdEMAMix
struct AdamK {
    float b1, c1, b2, c2, b3, c3, alpha, eps, ss, isb2, ibc1, lr, inv_scale;
};

__device__ __forceinline__ AdamK adam_consts(const Scalars &S) {
    AdamK k;
    k.b1 = uniform(S.b1); k.c1 = uniform(S.c1); k.b2 = uniform(S.b2); k.c2 = uniform(S.c2);
    k.b3 = uniform(S.b3); k.c3 = uniform(S.c3); k.alpha = uniform(S.alpha);
    k.eps = uniform(S.eps); k.ss = uniform(S.step_size); k.isb2 = uniform(S.inv_sqrt_bc2);
    k.ibc1 = uniform(S.inv_bc1); k.lr = uniform(S.lr); k.inv_scale = uniform(S.inv_scale);
    return k;
}

// [BNB] PR description / [MINI] AdamWMini full-v branch, per element:
//   m <- b1 m + c1 g;  v <- b2 v + c2 g^2;  h = sqrt(v)/sqrt(bc2) + eps
//   p <- p (1 - lr wd) - (lr/bc1) m / h          (decay from the old p)
// AdEMAMix adds m2 <- b3 m2 + c3 g and uses lr (m/bc1 + alpha m2) / h.
template <int PK, int GK, bool ADE, int N>
__device__ __forceinline__ void adam_elems(const TensorDesc &T, int64_t e, const AdamK &k,
                                           float decay) {
    float p[N], g[N], m[N], v[N], m2[N];
    load_p<PK, N>(T, e, p);
    load_g<GK, N>(T.g, e, k.inv_scale, g);
    ldf<N>(T.m, e, m);
    ldf<N>(T.v, e, v);
    if constexpr (ADE) ldf<N>(T.m2, e, m2);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        m[i] = k.b1 * m[i] + k.c1 * g[i];
        v[i] = k.b2 * v[i] + k.c2 * (g[i] * g[i]);
        const float h = sqrtf(v[i]) * k.isb2 + k.eps;
        if constexpr (ADE) {
            m2[i] = k.b3 * m2[i] + k.c3 * g[i];
            p[i] = p[i] * decay - k.lr * ((m[i] * k.ibc1 + k.alpha * m2[i]) / h);
        } else {
            p[i] = p[i] * decay - k.ss * (m[i] / h);
        }
    }
    store_p<PK, N>(T, e, p);
    stf<N>(T.m, e, m);
    stf<N>(T.v, e, v);
    if constexpr (ADE) stf<N>(T.m2, e, m2);
}

template <int PK, int GK, bool ADE>
__device__ __forceinline__ void adam_unit(const TensorDesc &T, int64_t start, int64_t len,
                                          const AdamK &k, float decay) {
    const bool vec = T.vec_ok && (start % 8 == 0);
    for (int64_t rel = threadIdx.x * 8; rel < len; rel += kThreads * 8) {
        const int64_t e = start + rel;
        if (vec && rel + 8 <= len) {
            adam_elems<PK, GK, ADE, 8>(T, e, k, decay);
        } else {
            const int64_t n = len - rel < 8 ? len - rel : 8;
            for (int64_t j = 0; j < n; ++j) adam_elems<PK, GK, ADE, 1>(T, e + j, k, decay);
        }
    }
}

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

// ---------------------------------------------------------------- Adam-mini
// [MINI] AdamWMini.step, q/k and "other" branches: one v per block of the
// flattened gradient, updated with the block mean of g^2.  Three kernels:
// per-unit partial sums of g^2 -> per-block finalize (fixed-order fp64 sum,
// v update, step factor) -> elementwise m/p update.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int GK>
__global__ __launch_bounds__(kThreads) void mini_sumsq_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const float s = S.inv_scale;
    __shared__ double red[kThreads / 64];
    for_units(a, [&](int64_t u, const SpanDesc &sp, int64_t start, int64_t len) {
        if (sp.block < 0) return;  // full-v tensor: no shared block
        const TensorDesc &T = a.tensors[sp.tensor];
        const bool vec = T.vec_ok && (start % 8 == 0);
        float acc = 0.0f;
        for (int64_t rel = threadIdx.x * 8; rel < len; rel += kThreads * 8) {
            const int64_t e = start + rel;
            if (vec && rel + 8 <= len) {
                float g[8];
                load_g<GK, 8>(T.g, e, s, g);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc += g[i] * g[i];
            } else {
                const int64_t n = len - rel < 8 ? len - rel : 8;
                for (int64_t j = 0; j < n; ++j) {
                    float g[1];
                    load_g<GK, 1>(T.g, e + j, s, g);
                    acc += g[0] * g[0];
                }
            }
        }
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
    });
}

__global__ __launch_bounds__(kThreads) void mini_finalize_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    __shared__ double red[kThreads];
    for (int b = blockIdx.x; b < a.nblocks; b += gridDim.x) {
        const int si = a.blockspan[b];
        const SpanDesc sp = a.spans[si];
        const int64_t u0 = sp.unit_begin, u1 = a.spans[si + 1].unit_begin;
        double acc = 0.0;
        for (int64_t u = u0 + threadIdx.x; u < u1; u += kThreads) acc += a.partials[u];
        red[threadIdx.x] = acc;
        __syncthreads();
        for (int st = kThreads / 2; st > 0; st >>= 1) {
            if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            const TensorDesc &T = a.tensors[sp.tensor];
            const int64_t j = sp.elem_begin / T.block_len;
            const double mean = red[0] / (double)sp.len;
            const double V = S.beta2_64 * (double)T.v[j] + S.c2_64 * mean;
            T.v[j] = (float)V;
            const double h = sqrt(V) * S.inv_sqrt_bc2_64 + S.eps64;
            a.blockfac[b] = (float)(S.step_size64 / h);
        }
        __syncthreads();
    }
}

template <int PK, int GK, int N>
__device__ __forceinline__ void mini_elems(const TensorDesc &T, int64_t e, const AdamK &k,
                                           float decay, float f) {
    float p[N], g[N], m[N];
    load_p<PK, N>(T, e, p);
    load_g<GK, N>(T.g, e, k.inv_scale, g);
    ldf<N>(T.m, e, m);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        m[i] = k.b1 * m[i] + k.c1 * g[i];
        p[i] = p[i] * decay - f * m[i];
    }
    store_p<PK, N>(T, e, p);
    stf<N>(T.m, e, m);
}

template <int PK, int GK>
__global__ __launch_bounds__(kThreads) void mini_update_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float decay = uniform(S.decay[T.group]);
        if (sp.block < 0) {
            adam_unit<PK, GK, false>(T, start, len, k, decay);
            return;
        }
        const float f = a.blockfac[sp.block];
        const bool vec = T.vec_ok && (start % 8 == 0);
        for (int64_t rel = threadIdx.x * 8; rel < len; rel += kThreads * 8) {
            const int64_t e = start + rel;
            if (vec && rel + 8 <= len) {
                mini_elems<PK, GK, 8>(T, e, k, decay, f);
            } else {
                const int64_t n = len - rel < 8 ? len - rel : 8;
                for (int64_t j = 0; j < n; ++j) mini_elems<PK, GK, 1>(T, e + j, k, decay, f);
            }
        }
    });
}

// ---------------------------------------------------------------- blockwise
// [BNB]: 2-state blockwise 8-bit AdamW with the Algorithm 2 decay order;
// [AO]: 4-bit states.  One quantization block = L consecutive lanes of one
// wavefront (L = block / E, E elements per lane), so the block absmax is a
// butterfly max over L lanes.  Code tables live in LDS.
template <int C>
__device__ __forceinline__ int code_search(const float *T, float a) {
    // largest j with T[j] <= a (T[0] = 0 acts as the floor)
    int lo = 0;
#pragma unroll
    for (int s = C >> 1; s > 0; s >>= 1)
        if (T[lo + s] <= a) lo += s;
    return lo;
}

template <int GK, int BITS>
__global__ __launch_bounds__(kThreads) void blockwise_kernel(StepArgs a) {
    constexpr int E = BITS == 8 ? 4 : 8;  // elements per lane per row
    constexpr int MBM = BITS - 1;         // magnitude bits of the signed m map
    constexpr int CM = 1 << MBM, CV = 1 << BITS;
    constexpr uint32_t CMASK = (1u << BITS) - 1u;
    __shared__ float sMm[CM], sTm[CM], sMv[CV], sTv[CV];
    {
        const float *cb = a.codebook;
        const int om = BITS == 8 ? kCb8SignedVals : kCb4SignedVals;
        const int otm = BITS == 8 ? kCb8SignedThr : kCb4SignedThr;
        const int ov = BITS == 8 ? kCb8UnsVals : kCb4UnsVals;
        const int otv = BITS == 8 ? kCb8UnsThr : kCb4UnsThr;
        for (int i = threadIdx.x; i < CM; i += kThreads) { sMm[i] = cb[om + i]; sTm[i] = cb[otm + i]; }
        for (int i = threadIdx.x; i < CV; i += kThreads) { sMv[i] = cb[ov + i]; sTv[i] = cb[otv + i]; }
    }
    __syncthreads();
    __shared__ Scalars S;
    step_begin(a, S);
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    const int L = a.block / E;  // lanes per quantization block (power of 2, <= 64)
    const int lane = threadIdx.x & 63;
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float decay = uniform(S.decay[T.group]);
        float *P = static_cast<float *>(T.p);
        const int rows = (int)((len + kThreads * E - 1) / (kThreads * E));
        for (int row = 0; row < rows; ++row) {
            const int64_t rel = (int64_t)row * kThreads * E + threadIdx.x * E;
            const int nv = len - rel >= E ? E : (len - rel > 0 ? (int)(len - rel) : 0);
            const int64_t e = start + rel;           // multiple of E
            const int64_t blk = e / a.block;
            const bool full = T.vec_ok && nv == E;
            float p[E], g[E];
            uint32_t cm = 0, cv = 0;
            float Am = 0.0f, Av = 0.0f;
            if (nv > 0) { Am = T.am[blk]; Av = T.av[blk]; }
            if (full) {
                ldf<E>(P, e, p);
                load_g<GK, E>(T.g, e, k.inv_scale, g);
                cm = *reinterpret_cast<const uint32_t *>(T.qm + (e * BITS) / 8);
                cv = *reinterpret_cast<const uint32_t *>(T.qv + (e * BITS) / 8);
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    p[j] = 0.0f; g[j] = 0.0f;
                    if (j < nv) {
                        float pj[1], gj[1];
                        ldf<1>(P, e + j, pj);
                        load_g<GK, 1>(T.g, e + j, k.inv_scale, gj);
                        p[j] = pj[0]; g[j] = gj[0];
                        const int64_t bit = (e + j) * BITS;
                        cm |= (uint32_t)((T.qm[bit >> 3] >> (bit & 7)) & CMASK) << (j * BITS);
                        cv |= (uint32_t)((T.qv[bit >> 3] >> (bit & 7)) & CMASK) << (j * BITS);
                    }
                }
            }
            // dequantize, update the fp32 states (no contraction), update p
            float mn[E], vn[E];
            float mx_m = 0.0f, mx_v = 0.0f;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const uint32_t c = (cm >> (j * BITS)) & CMASK;
                const float mag = sMm[c & (CM - 1)] * Am;
                const float mt = ((c >> MBM) & 1u) ? -mag : mag;
                const float vt = sMv[(cv >> (j * BITS)) & CMASK] * Av;
                mn[j] = k.b1 * mt + k.c1 * g[j];
                vn[j] = k.b2 * vt + k.c2 * (g[j] * g[j]);
                const float h = sqrtf(vn[j]) * k.isb2 + k.eps;
                p[j] = p[j] * decay - k.ss * (mn[j] / h);
                if (j < nv) {
                    mx_m = fmaxf(mx_m, fabsf(mn[j]));
                    mx_v = fmaxf(mx_v, vn[j]);
                }
            }
            for (int o = L >> 1; o > 0; o >>= 1) {
                mx_m = fmaxf(mx_m, __shfl_xor(mx_m, o));
                mx_v = fmaxf(mx_v, __shfl_xor(mx_v, o));
            }
            const float rm = mx_m > 0.0f ? 1.0f / mx_m : 0.0f;
            const float rv = mx_v > 0.0f ? 1.0f / mx_v : 0.0f;
            uint32_t om = 0, ov = 0;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                uint32_t im = 0, iv = 0;
                if (mx_m > 0.0f) {
                    im = (uint32_t)code_search<CM>(sTm, fabsf(mn[j]) * rm);
                    if (mn[j] < 0.0f && im > 0) im |= 1u << MBM;
                }
                if (mx_v > 0.0f) iv = (uint32_t)code_search<CV>(sTv, vn[j] * rv);
                om |= im << (j * BITS);
                ov |= iv << (j * BITS);
            }
            if (full) {
                stf<E>(P, e, p);
                *reinterpret_cast<uint32_t *>(T.qm + (e * BITS) / 8) = om;
                *reinterpret_cast<uint32_t *>(T.qv + (e * BITS) / 8) = ov;
            } else if (nv > 0) {
                for (int j = 0; j < nv; ++j) {
                    float pj[1] = {p[j]};
                    stf<1>(P, e + j, pj);
                }
                // whole bytes only: this lane owns bytes [e*BITS/8, (e+nv)*BITS/8)
                const int nbytes = (nv * BITS + 7) / 8;
                for (int q = 0; q < nbytes; ++q) {
                    uint32_t bm = (om >> (8 * q)) & 0xFFu, bv = (ov >> (8 * q)) & 0xFFu;
                    T.qm[(e * BITS) / 8 + q] = (uint8_t)bm;
                    T.qv[(e * BITS) / 8 + q] = (uint8_t)bv;
                }
            }
            if (nv > 0 && (lane & (L - 1)) == 0) {
                T.am[blk] = mx_m;
                T.av[blk] = mx_v;
            }
        }
    });
}

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

// Persistent grid: as many workgroups as fit on the device at once (so no
// workgroup starts late and owns a tail), never more than there are units.
// A positive request overrides the occupancy query.
template <class K>
int persistent_grid(K kernel, const StepArgs &a) {
    const int64_t units = a.nunits > 0 ? a.nunits : 1;
    if (a.grid_request > 0) return (int)(a.grid_request < units ? a.grid_request : units);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int64_t g = (int64_t)per_cu * (a.cus > 0 ? a.cus : 1);
    return (int)(g < units ? g : units);
}

}  // namespace

// ---------------------------------------------------------------- launchers
#define LAUNCH_PERSISTENT(K, a, s)                                                     \
    hipLaunchKernelGGL(K, dim3(persistent_grid(K, a)), dim3(kThreads), 0, s, a)

template <bool ADE>
static hipError_t launch_adam_t(const StepArgs &a, int pk, int gk, hipStream_t s) {
    if (pk == P_F32 && gk == G_F32)
        LAUNCH_PERSISTENT((adam_kernel<P_F32, G_F32, ADE>), a, s);
    else if (pk == P_F32 && gk == G_BF16)
        LAUNCH_PERSISTENT((adam_kernel<P_F32, G_BF16, ADE>), a, s);
    else if (pk == P_BF16R && gk == G_F32)
        LAUNCH_PERSISTENT((adam_kernel<P_BF16R, G_F32, ADE>), a, s);
    else
        LAUNCH_PERSISTENT((adam_kernel<P_BF16R, G_BF16, ADE>), a, s);
    return hipGetLastError();
}

hipError_t launch_adamw(const StepArgs &a, int pk, int gk, hipStream_t s) {
    return launch_adam_t<false>(a, pk, gk, s);
}

hipError_t launch_ademamix(const StepArgs &a, int pk, int gk, hipStream_t s) {
    return launch_adam_t<true>(a, pk, gk, s);
}

hipError_t launch_adam_mini(const StepArgs &args, int pk, int gk, hipStream_t s) {
    // block sums and finalize read the step's inputs; the update publishes it
    StepArgs a = args;
    a.commit = 0;
    if (gk == G_F32)
        LAUNCH_PERSISTENT((mini_sumsq_kernel<G_F32>), a, s);
    else
        LAUNCH_PERSISTENT((mini_sumsq_kernel<G_BF16>), a, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.nblocks > 0) {
        const int fg = a.nblocks < 2048 ? a.nblocks : 2048;
        hipLaunchKernelGGL(mini_finalize_kernel, dim3(fg), dim3(kThreads), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    a.commit = 1;
    if (pk == P_F32 && gk == G_F32)
        LAUNCH_PERSISTENT((mini_update_kernel<P_F32, G_F32>), a, s);
    else if (pk == P_F32 && gk == G_BF16)
        LAUNCH_PERSISTENT((mini_update_kernel<P_F32, G_BF16>), a, s);
    else if (pk == P_BF16R && gk == G_F32)
        LAUNCH_PERSISTENT((mini_update_kernel<P_BF16R, G_F32>), a, s);
    else
        LAUNCH_PERSISTENT((mini_update_kernel<P_BF16R, G_BF16>), a, s);
    return hipGetLastError();
}

hipError_t launch_blockwise(const StepArgs &a, int gk, hipStream_t s) {
    if (a.bits == 8 && gk == G_F32)
        LAUNCH_PERSISTENT((blockwise_kernel<G_F32, 8>), a, s);
    else if (a.bits == 8)
        LAUNCH_PERSISTENT((blockwise_kernel<G_BF16, 8>), a, s);
    else if (gk == G_F32)
        LAUNCH_PERSISTENT((blockwise_kernel<G_F32, 4>), a, s);
    else
        LAUNCH_PERSISTENT((blockwise_kernel<G_BF16, 4>), a, s);
    return hipGetLastError();
}

hipError_t launch_check_finite(const StepArgs &a, int gk, hipStream_t s) {
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
