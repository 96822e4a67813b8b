// kernels_scaled.hip -- AdamW with 16-bit moments and a per-tensor scale
// ([TE] review thread: a scaled low-precision optimizer state, its fp32
// value being stored * scale and a new state being value * rscale copied into
// the low-precision tensor).  The update itself is the AdamW one, in fp32,
// from the decoded moments.
//
// bf16 moments keep scale 1 (bf16 has fp32's range), so the step is one
// pass: p, g, m, v read; p, m, v written; the last workgroup sets each
// tensor's scales to 1.
//
// fp16 moments: the new scale is max|x| / 65504 over the tensor's new
// moments, known only once every element is updated, so two passes:
//   pass 1  m, v from the stored ones, p update; each wave's max |m| and
//           |v| go by atomic max on their fp32 bits (non-negative floats
//           order as their bit patterns) into one of kAmaxSlots words of
//           the tensor, so no one address takes every wave's atomic;
//   pass 2  the new scales from the slots; m, v recomputed from the stored
//           (not yet overwritten) moments with the same fp32 operations and
//           stored as rne16(fl32(x * rscale)); the last workgroup writes the
//           new scales, clears the slots and publishes the step.
// Traffic per element (fp32 p and g): bf16 20 B; fp16 pass 1 reads p, g, m,
// v and writes p (16 B), pass 2 reads g, m, v and writes m, v (12 B).
#include "device_common.h"

namespace optim {
namespace {

template <int SK>
__device__ __forceinline__ float h16_to_f32(uint32_t b) {
    if constexpr (SK == S_F16) return __half2float(__ushort_as_half((unsigned short)b));
    else return __uint_as_float(b << 16);
}

// x rounded to fp32 and kept there: the scaled moment is an fp32 value
// copied into 16 bits (two roundings).  Without the empty asm the compiler
// fuses the multiply and the fp16 conversion into one mixed-precision FMA
// (v_fma_mixlo_f16), which rounds once and differs at fp16 ties.
__device__ __forceinline__ float in_f32(float x) {
    asm("" : "+v"(x));
    return x;
}

// The moments of this step from the stored ones, as fp32 (no contraction).
template <int SK, int N, int LAY = kStrided>
__device__ __forceinline__ void scaled_moments(const TensorDesc &T, int64_t e, const AdamK &k, float sm, float sv,
                                               const float (&g)[N], float (&m)[N], float (&v)[N]) {
    uint32_t qm[N], qv[N];
    ldh<N, LAY>(reinterpret_cast<const uint16_t *>(T.m), e, qm);
    ldh<N, LAY>(reinterpret_cast<const uint16_t *>(T.v), e, qv);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float mt = h16_to_f32<SK>(qm[i]) * sm;
        const float vt = h16_to_f32<SK>(qv[i]) * sv;
        m[i] = k.b1 * mt + k.c1 * g[i];
        v[i] = k.b2 * vt + k.c2 * (g[i] * g[i]);
    }
}

template <int N>
__device__ __forceinline__ void adamw_update(float (&p)[N], const float (&m)[N], const float (&v)[N],
                                             const AdamK &k, float lw) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float h = sqrtf(v[i]) * k.isb2 + k.eps;
        p[i] = decayed(p[i], lw, k.ss * (m[i] / h));
    }
}

__device__ __forceinline__ uint32_t *amax_slot(const StepArgs &a, int b, int which, int slot) {
    return reinterpret_cast<uint32_t *>(a.blockfac) +
           ((int64_t)(2 * b + which) * kAmaxSlots + slot) * kCounterStride;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// fp16 scale from a maximum: fl32(max / 65504) (the quotient in fp64,
// rounded once), 1 for an all-zero tensor.
__device__ __forceinline__ float f16_scale(float amax) {
    return amax > 0.0f ? (float)((double)amax / 65504.0) : 1.0f;
}

// Maxima of tensor block b over its slots: lanes 0..15 read the m slots,
// lanes 16..31 the v slots.  Pass 1 ended before this kernel started (stream
// order, caches invalidated at launch), so plain loads see every atomic.
__device__ __forceinline__ void slots_max(const StepArgs &a, int b, float &am, float &av) {
    const int l = threadIdx.x & 63;
    uint32_t x = 0;
    if (l < 2 * kAmaxSlots) x = *gp(amax_slot(a, b, l / kAmaxSlots, l % kAmaxSlots));
#pragma unroll
    for (int o = kAmaxSlots / 2; o > 0; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)x, o);
        x = x > y ? x : y;
    }
    am = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)x, 0));
    av = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)x, kAmaxSlots));
}

// End of a committing kernel: the last workgroup to arrive runs epi with
// all of its threads, then publishes the step.  Every workgroup's loads of
// the old scales were consumed before its barrier, so epi may overwrite them.
template <class Epi>
__device__ __forceinline__ void commit_last(const StepArgs &a, const Scalars &S, Epi epi) {
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) last = last_arrival(a);
    __syncthreads();
    if (!last) return;
    epi();
    if (threadIdx.x == 0) publish_step(a, S);
}

template <int PK, int GK>
__global__ __launch_bounds__(kThreads) void scaled_bf16_kernel(StepArgs a) {
    __shared__ Scalars S;
    step_begin(a, S);
    if (!S.skip) {
        const AdamK k = adam_consts(S);
        for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
            // the descriptor in scalar registers, so p, m and v are stored
            // back to back (measured on MI355X, 4096^2 fp32 p / g, in one
            // process on the same arrays: 62.4 -> 61.3 us against a
            // reference into the plan's table, see uniform_desc)
            const TensorDesc T = uniform_desc(a.tensors[sp.tensor]);
            const float lw = uniform(S.lrwd[T.group]);
            const float sm = uniform(*T.scale_m), sv = uniform(*T.scale_v);
            lane_walk<kAdamGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
                constexpr int N = decltype(n)::value;
                float p[N], g[N], m[N], v[N];
                load_p<PK, N>(T, e, p);
                load_g<GK, N>(T.g, e, k.inv_scale, g);
                scaled_moments<S_BF16, N>(T, e, k, sm, sv, g, m, v);
                adamw_update<N>(p, m, v, k, lw);
                uint32_t qm[N], qv[N];
#pragma unroll
                for (int i = 0; i < N; ++i) {  // scale 1: x * 1 is x
                    qm[i] = f32_to_bf16_rne(m[i]);
                    qv[i] = f32_to_bf16_rne(v[i]);
                }
                store_p<PK, N>(T, e, p);
                sth<N>(reinterpret_cast<uint16_t *>(T.m), e, qm);
                sth<N>(reinterpret_cast<uint16_t *>(T.v), e, qv);
            });
        });
    }
    commit_last(a, S, [&] {
        if (S.skip) return;
        for (int b = threadIdx.x; b < a.nblocks; b += kThreads) {
            const TensorDesc &T = a.tensors[a.spans[a.blockspan[b]].tensor];
            *T.scale_m = 1.0f;
            *T.scale_v = 1.0f;
        }
    });
}

// KEEP: g, m and v, which pass 2 reads again, go through ordinary accesses
// in both passes (kept in the Infinity Cache) and pass 2 walks backwards.
template <int PK, int GK, bool KEEP>
__global__ __launch_bounds__(kThreads) void scaled_f16_pass1_kernel(StepArgs a) {
    constexpr int RL = KEEP ? kStridedKeep : kStrided;  // re-read by pass 2
    __shared__ Scalars S;
    step_begin(a, S);
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    const int slot = (int)((blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) % kAmaxSlots);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const float lw = uniform(S.lrwd[T.group]);
        const float sm = uniform(*T.scale_m), sv = uniform(*T.scale_v);
        float mx = 0.0f, vx = 0.0f;
        lane_walk<kAdamGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
            constexpr int N = decltype(n)::value;
            float p[N], g[N], m[N], v[N];
            load_p<PK, N>(T, e, p);
            load_g<GK, N, RL>(T.g, e, k.inv_scale, g);
            scaled_moments<S_F16, N, RL>(T, e, k, sm, sv, g, m, v);
            adamw_update<N>(p, m, v, k, lw);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                mx = fmaxf(mx, fabsf(m[i]));
                vx = fmaxf(vx, fabsf(v[i]));
            }
            store_p<PK, N>(T, e, p);
        });
        mx = wave_max(mx);
        vx = wave_max(vx);
        if ((threadIdx.x & 63) == 0) {
            if (mx > 0.0f)
                __hip_atomic_fetch_max(amax_slot(a, sp.block, 0, slot), __float_as_uint(mx), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            if (vx > 0.0f)
                __hip_atomic_fetch_max(amax_slot(a, sp.block, 1, slot), __float_as_uint(vx), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    });
}

template <int GK, bool KEEP>
__global__ __launch_bounds__(kThreads) void scaled_f16_pass2_kernel(StepArgs a) {
    constexpr int RL = KEEP ? kStridedKeep : kStrided;
    __shared__ Scalars S;
    step_begin(a, S);
    if (!S.skip) {
        const AdamK k = adam_consts(S);
        for_units<KEEP>(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
            const TensorDesc &T = a.tensors[sp.tensor];
            const float sm = uniform(*T.scale_m), sv = uniform(*T.scale_v);
            float am, av;
            slots_max(a, sp.block, am, av);
            // rscale = fl32(1 / scale'), the quotient in fp64 rounded once
            const float rm = (float)(1.0 / (double)f16_scale(am));
            const float rv = (float)(1.0 / (double)f16_scale(av));
            lane_walk<kAdamGroups>(start, len, T.vec_ok, [&](auto n, int64_t e) {
                constexpr int N = decltype(n)::value;
                float g[N], m[N], v[N];
                load_g<GK, N, RL>(T.g, e, k.inv_scale, g);
                scaled_moments<S_F16, N, RL>(T, e, k, sm, sv, g, m, v);
                uint32_t qm[N], qv[N];
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    qm[i] = f32_to_f16_rne(in_f32(m[i] * rm));
                    qv[i] = f32_to_f16_rne(in_f32(v[i] * rv));
                }
                sth<N>(reinterpret_cast<uint16_t *>(T.m), e, qm);
                sth<N>(reinterpret_cast<uint16_t *>(T.v), e, qv);
            });
        });
    }
    commit_last(a, S, [&] {
        if (S.skip) return;  // pass 1 was skipped too: the slots are still 0
        for (int b = threadIdx.x; b < a.nblocks; b += kThreads) {
            uint32_t mm = 0, mv = 0;
            for (int j = 0; j < kAmaxSlots; ++j) {
                uint32_t *pm = amax_slot(a, b, 0, j), *pv = amax_slot(a, b, 1, j);
                const uint32_t xm = __hip_atomic_load(pm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t xv = __hip_atomic_load(pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                mm = mm > xm ? mm : xm;
                mv = mv > xv ? mv : xv;
                __hip_atomic_store(pm, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pv, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const TensorDesc &T = a.tensors[a.spans[a.blockspan[b]].tensor];
            *T.scale_m = f16_scale(__uint_as_float(mm));
            *T.scale_v = f16_scale(__uint_as_float(mv));
        }
    });
}

template <int PK, int GK, bool KEEP>
hipError_t launch_f16_t(const StepArgs &a, hipStream_t s) {
    LAUNCH_PERSISTENT((scaled_f16_pass1_kernel<PK, GK, KEEP>), a, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    LAUNCH_PERSISTENT((scaled_f16_pass2_kernel<GK, KEEP>), a, s);
    return hipGetLastError();
}

template <int PK, int GK>
hipError_t launch_scaled_t(const StepArgs &args, int sk, hipStream_t s) {
    StepArgs a = args;
    a.commit = 1;
    if (sk == S_BF16) {
        LAUNCH_PERSISTENT((scaled_bf16_kernel<PK, GK>), a, s);
        return hipGetLastError();
    }
    // g, m, v (gradient bytes + 4) are read again by pass 2; measured with
    // fp32 grads: 9-11% faster kept up to 32M elements (256 MB re-read), 3%
    // at 64M (512 MB)
    return keep_for_second_pass(a, (GK == G_F32 ? 4 : 2) + 4, int64_t(512) << 20)
               ? launch_f16_t<PK, GK, true>(a, s)
               : launch_f16_t<PK, GK, false>(a, s);
}

}  // namespace

hipError_t launch_adamw_scaled(const StepArgs &a, int pk, int gk, int sk, hipStream_t s) {
    if (pk == P_F32 && gk == G_F32) return launch_scaled_t<P_F32, G_F32>(a, sk, s);
    if (pk == P_F32 && gk == G_BF16) return launch_scaled_t<P_F32, G_BF16>(a, sk, s);
    if (pk == P_BF16R && gk == G_F32) return launch_scaled_t<P_BF16R, G_F32>(a, sk, s);
    if (pk == P_BF16R && gk == G_BF16) return launch_scaled_t<P_BF16R, G_BF16>(a, sk, s);
    return hipErrorInvalidValue;
}

}  // namespace optim
