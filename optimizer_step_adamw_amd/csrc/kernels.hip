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
// N = 8: two 128-bit accesses (fp32) or one (16-bit); N = 1: one element.
template <int N>
__device__ __forceinline__ void ldf(const float *a, int64_t e, float (&x)[N]) {
    if constexpr (N == 8) {
        const float4 *q = reinterpret_cast<const float4 *>(a + e);
        const float4 u = q[0], w = q[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
    } else if constexpr (N == 4) {
        const float4 u = *reinterpret_cast<const float4 *>(a + e);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) x[k] = a[e + k];
    }
}

template <int N>
__device__ __forceinline__ void stf(float *a, int64_t e, const float (&x)[N]) {
    if constexpr (N == 8) {
        float4 *q = reinterpret_cast<float4 *>(a + e);
        q[0] = make_float4(x[0], x[1], x[2], x[3]);
        q[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else if constexpr (N == 4) {
        *reinterpret_cast<float4 *>(a + e) = make_float4(x[0], x[1], x[2], x[3]);
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) a[e + k] = x[k];
    }
}

template <int N>
__device__ __forceinline__ void ldh(const uint16_t *a, int64_t e, uint32_t (&x)[N]) {
    if constexpr (N == 8) {
        const uint4 u = *reinterpret_cast<const uint4 *>(a + e);
        x[0] = u.x & 0xFFFFu; x[1] = u.x >> 16; x[2] = u.y & 0xFFFFu; x[3] = u.y >> 16;
        x[4] = u.z & 0xFFFFu; x[5] = u.z >> 16; x[6] = u.w & 0xFFFFu; x[7] = u.w >> 16;
    } else if constexpr (N == 4) {
        const uint2 u = *reinterpret_cast<const uint2 *>(a + e);
        x[0] = u.x & 0xFFFFu; x[1] = u.x >> 16; x[2] = u.y & 0xFFFFu; x[3] = u.y >> 16;
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) x[k] = a[e + k];
    }
}

template <int N>
__device__ __forceinline__ void sth(uint16_t *a, int64_t e, const uint32_t (&x)[N]) {
    if constexpr (N == 8) {
        uint4 u;
        u.x = (x[0] & 0xFFFFu) | (x[1] << 16);
        u.y = (x[2] & 0xFFFFu) | (x[3] << 16);
        u.z = (x[4] & 0xFFFFu) | (x[5] << 16);
        u.w = (x[6] & 0xFFFFu) | (x[7] << 16);
        *reinterpret_cast<uint4 *>(a + e) = u;
    } else if constexpr (N == 4) {
        uint2 u;
        u.x = (x[0] & 0xFFFFu) | (x[1] << 16);
        u.y = (x[2] & 0xFFFFu) | (x[3] << 16);
        *reinterpret_cast<uint2 *>(a + e) = u;
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) a[e + k] = (uint16_t)x[k];
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
template <class Body>
__device__ __forceinline__ void for_units(const StepArgs &a, Body &&body) {
    const int64_t G = gridDim.x, b = blockIdx.x;
    int64_t u = a.nunits * b / G;
    const int64_t u1 = a.nunits * (b + 1) / G;
    if (u >= u1) return;
    int lo = 0, hi = a.nspans;  // spans[nspans].unit_begin == nunits > u
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.spans[mid].unit_begin <= u) lo = mid; else hi = mid;
    }
    int s = lo;
    for (; u < u1; ++u) {
        while (a.spans[s + 1].unit_begin <= u) ++s;
        const SpanDesc sp = a.spans[s];
        const int64_t off = (u - sp.unit_begin) * kTile;
        const int64_t len = sp.len - off < kTile ? sp.len - off : kTile;
        body(u, sp, sp.elem_begin + off, len);
    }
}

// ---------------------------------------------------------------- AdamW / AdEMAMix
struct AdamK {
    float b1, c1, b2, c2, b3, c3, alpha, eps, ss, isb2, ibc1, lr, inv_scale;
};

__device__ __forceinline__ AdamK adam_consts(const Scalars &S) {
    AdamK k;
    k.b1 = S.b1; k.c1 = S.c1; k.b2 = S.b2; k.c2 = S.c2; k.b3 = S.b3; k.c3 = S.c3;
    k.alpha = S.alpha; k.eps = S.eps; k.ss = S.step_size; k.isb2 = S.inv_sqrt_bc2;
    k.ibc1 = S.inv_bc1; k.lr = S.lr; k.inv_scale = S.inv_scale;
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
    const Scalars &S = *a.sc;
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        adam_unit<PK, GK, ADE>(T, start, len, k, S.decay[T.group]);
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
    const Scalars &S = *a.sc;
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
    const Scalars &S = *a.sc;
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
    const Scalars &S = *a.sc;
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float decay = S.decay[T.group];
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
    const Scalars &S = *a.sc;
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    const int L = a.block / E;  // lanes per quantization block (power of 2, <= 64)
    const int lane = threadIdx.x & 63;
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float decay = S.decay[T.group];
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

// ---------------------------------------------------------------- prep
// Per-step scalars in fp64, rounded once to fp32.  Bias corrections are not
// evaluated in fp32: 1 - beta2^t cancels badly there at small t, and fast
// power/divide intrinsics put a kernel microns off the closed form ([BNB] PR
// body).  The lr is read from (or, with a schedule, written to) a device
// scalar, never passed from the host per step ([AO]).
__global__ void prep_kernel(PrepArgs a) {
    __shared__ float s_lr;
    if (threadIdx.x == 0) {
        float lr;
        int32_t k = 0;
        if (a.sched == 1) {
            k = *a.iter_dev;
            const int32_t kk = k < 0 ? 0 : (k < a.K ? k : a.K);
            const double x = (double)kk / (double)a.K;
            lr = (float)(a.lr_min + (a.lr_max - a.lr_min) * 0.5 * (1.0 + cos(kPi * x)));
        } else {
            lr = *a.lr_dev;
        }
        const int skip = (a.found_inf != nullptr) && (*a.found_inf != 0.0f);
        const int32_t t = *a.step_dev + 1;
        const double bc1 = 1.0 - pow(a.beta1, (double)t);
        const double bc2 = 1.0 - pow(a.beta2, (double)t);
        const double lr64 = (double)lr;
        Scalars *sc = a.sc;
        sc->skip = skip;
        sc->t = t;
        sc->lr = lr;
        sc->step_size = (float)(lr64 / bc1);
        sc->inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
        sc->inv_bc1 = (float)(1.0 / bc1);
        sc->b1 = (float)a.beta1;
        sc->c1 = (float)(1.0 - a.beta1);
        sc->b2 = (float)a.beta2;
        sc->c2 = (float)(1.0 - a.beta2);
        sc->b3 = (float)a.beta3;
        sc->c3 = (float)(1.0 - a.beta3);
        sc->alpha = (float)a.alpha;
        sc->eps = (float)a.eps;
        sc->inv_scale = a.inv_scale ? *a.inv_scale : 1.0f;
        sc->lr64 = lr64;
        sc->step_size64 = lr64 / bc1;
        sc->inv_sqrt_bc2_64 = 1.0 / sqrt(bc2);
        sc->eps64 = a.eps;
        sc->beta2_64 = a.beta2;
        sc->c2_64 = 1.0 - a.beta2;
        s_lr = lr;
        if (a.sched == 1) {
            *a.lr_dev = lr;
            *a.iter_dev = k + 1;
        }
        if (!skip) *a.step_dev = t;
    }
    __syncthreads();
    if ((int)threadIdx.x < a.ngroups)
        a.sc->decay[threadIdx.x] = (float)(1.0 - (double)s_lr * a.group_wd[threadIdx.x]);
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
    if (a.grid_request > 0) return a.grid_request < a.nunits ? a.grid_request : (int)a.nunits;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int64_t g = (int64_t)per_cu * (a.cus > 0 ? a.cus : 1);
    return (int)(g < a.nunits ? g : (a.nunits > 0 ? a.nunits : 1));
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_prep(const PrepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(kMaxGroups), 0, s, a);
    return hipGetLastError();
}

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

hipError_t launch_adam_mini(const StepArgs &a, int pk, int gk, hipStream_t s) {
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
