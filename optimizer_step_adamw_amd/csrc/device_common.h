// device_common.h -- device-side building blocks shared by the gfx950
// kernels of the fused, multi-tensor AdamW-family optimizer step: storage
// formats, global-memory accesses, unit traversal, the per-step scalar
// prologue and commit, and the AdamW/AdEMAMix element update.
//
// The step is elementwise and HBM-bound (a few flops per byte), so there is
// no matrix-core work.  A step kernel processes work units (`tile`
// consecutive elements of one span) with non-temporal 128-bit (fp32) or
// 64-bit (16-bit) loads and stores, each instruction of a wave covering one
// contiguous run; by default one workgroup per unit.  Every workgroup
// derives the step's scalars in its prologue and the last one to finish
// publishes the new step counter.
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
// Build flags: -ffp-contract=off (every multiply and add rounds on its own,
// as written), IEEE division and sqrt, fp32 denormals kept.
#pragma once

#include "plan.h"

#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
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
//
// Two register layouts for a lane's N elements:
//  kStrided (step kernels): N = 4V elements in V groups of 4 consecutive
//    elements, group j at e + j*kSub, with lane t's e = unit start + 4t.
//    One instruction of a wave then covers one contiguous 1 KiB (fp32) or
//    512 B (16-bit) run, and the accesses are non-temporal: streamed data is
//    touched once per step, and on MI355X non-temporal loads plus stores of
//    whole contiguous runs sustain ~13% more bandwidth on the AdamW access
//    pattern than ordinary ones (measured 5.99 vs 5.29 TB/s for 4 reads and
//    3 writes per element), while non-temporal stores of half-filled lines
//    (8 adjacent fp32 per lane) lose write combining and fall far below.
//  kRun (blockwise quantizer rows): N consecutive elements from e, ordinary
//    loads and stores; the per-block DPP reductions want each lane's
//    elements adjacent.
//  kStridedKeep: kStrided's addresses with ordinary accesses, for arrays a
//    second pass of the same step reads again (LAMB, fp16 scaled moments):
//    ordinary accesses in both passes leave them in the Infinity Cache, and
//    the second pass, walking the units backwards, meets the most recent
//    ones first (measured on MI355X: LAMB and fp16-moment steps 6-11% faster
//    up to a few hundred MB re-read; slower past that, so the launchers
//    choose by size).
// N = 1 is one element, ordinary access, in either layout.
#define GMEM __attribute__((address_space(1)))
typedef float __attribute__((ext_vector_type(4))) f32x4;
typedef uint32_t __attribute__((ext_vector_type(4))) u32x4;
typedef uint32_t __attribute__((ext_vector_type(2))) u32x2;

constexpr int kVec = 4;                             // elements per lane per group
constexpr int64_t kSub = (int64_t)kVec * kThreads;  // elements per workgroup per group
enum Layout { kStrided = 0, kRun = 1, kStridedKeep = 2 };
// groups of 4 elements per lane the AdamW / AdEMAMix / Adam-mini update
// loads before computing (one 1 KiB run per array per wave and group)
constexpr int kAdamGroups = 2;
// the same for the early-load AdamW / AdEMAMix kernel on 4096-element units
// (lists of more than 2^20 and at most 2^24 elements)
constexpr int kAdamGroupsEarly = 4;

template <class T>
__device__ __forceinline__ GMEM T *gp(T *p) { return (GMEM T *)p; }
template <class T>
__device__ __forceinline__ const GMEM T *gp(const T *p) { return (const GMEM T *)p; }

template <int LAY, class V>
__device__ __forceinline__ V vload(const GMEM V *q) {
    if constexpr (LAY == kStrided) return __builtin_nontemporal_load(q);
    else return *q;
}
template <int LAY, class V>
__device__ __forceinline__ void vstore(GMEM V *q, V x) {
    if constexpr (LAY == kStrided) __builtin_nontemporal_store(x, q);
    else *q = x;
}
// element offset of group j of a lane's elements
template <int LAY>
__device__ __forceinline__ constexpr int64_t group_off(int j) {
    return LAY == kRun ? (int64_t)j * kVec : j * kSub;
}

// gs: the distance between a lane's groups in the strided layouts (kSub,
// or more in an interleaved moment array).
template <int N, int LAY = kStrided>
__device__ __forceinline__ void ldf(const float *a, int64_t e, float (&x)[N], int64_t gs = kSub) {
    if constexpr (N == 1) {
        x[0] = gp(a)[e];
    } else {
        static_assert(N % kVec == 0, "groups of 4");
#pragma unroll
        for (int j = 0; j < N / kVec; ++j) {
            const f32x4 u = vload<LAY>((const GMEM f32x4 *)gp(a + e + (LAY == kRun ? group_off<LAY>(j) : j * gs)));
            x[4 * j] = u.x; x[4 * j + 1] = u.y; x[4 * j + 2] = u.z; x[4 * j + 3] = u.w;
        }
    }
}

template <int N, int LAY = kStrided>
__device__ __forceinline__ void stf(float *a, int64_t e, const float (&x)[N], int64_t gs = kSub) {
    if constexpr (N == 1) {
        gp(a)[e] = x[0];
    } else {
        static_assert(N % kVec == 0, "groups of 4");
#pragma unroll
        for (int j = 0; j < N / kVec; ++j)
            vstore<LAY>((GMEM f32x4 *)gp(a + e + (LAY == kRun ? group_off<LAY>(j) : j * gs)),
                        f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]});
    }
}

// 16-bit arrays (bf16 params and grads, int16 remainders): values are
// returned zero-extended in 32-bit registers.
template <int N, int LAY = kStrided>
__device__ __forceinline__ void ldh(const uint16_t *a, int64_t e, uint32_t (&x)[N]) {
    if constexpr (N == 1) {
        x[0] = gp(a)[e];
    } else if constexpr (LAY == kRun && N == 8) {
        const u32x4 u = vload<LAY>((const GMEM u32x4 *)gp(a + e));
        x[0] = u.x & 0xFFFFu; x[1] = u.x >> 16; x[2] = u.y & 0xFFFFu; x[3] = u.y >> 16;
        x[4] = u.z & 0xFFFFu; x[5] = u.z >> 16; x[6] = u.w & 0xFFFFu; x[7] = u.w >> 16;
    } else {
        static_assert(N % kVec == 0, "groups of 4");
#pragma unroll
        for (int j = 0; j < N / kVec; ++j) {
            const u32x2 u = vload<LAY>((const GMEM u32x2 *)gp(a + e + group_off<LAY>(j)));
            x[4 * j] = u.x & 0xFFFFu; x[4 * j + 1] = u.x >> 16;
            x[4 * j + 2] = u.y & 0xFFFFu; x[4 * j + 3] = u.y >> 16;
        }
    }
}

template <int N, int LAY = kStrided>
__device__ __forceinline__ void sth(uint16_t *a, int64_t e, const uint32_t (&x)[N]) {
    if constexpr (N == 1) {
        gp(a)[e] = (uint16_t)x[0];
    } else {
        static_assert(N % kVec == 0, "groups of 4");
#pragma unroll
        for (int j = 0; j < N / kVec; ++j)
            vstore<LAY>((GMEM u32x2 *)gp(a + e + group_off<LAY>(j)),
                        u32x2{(x[4 * j] & 0xFFFFu) | (x[4 * j + 1] << 16),
                              (x[4 * j + 2] & 0xFFFFu) | (x[4 * j + 3] << 16)});
    }
}

// fp32 -> bf16 pattern, round to nearest even ([TE] review: the model copy
// of an fp32 master is the master rounded to the model dtype); NaN stays a
// quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> fp16 pattern: the hardware conversion, round to nearest even
// (the default mode), fp16 denormals kept.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float x) {
    return (uint32_t)__half_as_ushort(__float2half_rn(x));
}

// Parameters: fp32 (P_F32); bf16 + int16 remainder rebuilding the fp32
// master (P_BF16R); or an fp32 master with a bf16 / fp16 model copy in p
// (P_MBF16 / P_MF16), rewritten from the updated master.
// (D: a TensorDesc, or a pack's PackMember record.)
template <int PK, int N, int LAY = kStrided, class D>
__device__ __forceinline__ void load_p(const D &T, int64_t e, float (&p)[N]) {
    if constexpr (PK == P_F32) {
        ldf<N, LAY>(static_cast<const float *>(T.p), e, p);
    } else if constexpr (PK == P_BF16R) {
        uint32_t b[N], r[N];
        ldh<N, LAY>(static_cast<const uint16_t *>(T.p), e, b);
        ldh<N, LAY>(T.rem, e, r);
#pragma unroll
        for (int k = 0; k < N; ++k) p[k] = rem_reconstruct(b[k], r[k]);
    } else {
        ldf<N, LAY>(T.master, e, p);
    }
}

template <int PK, int N, class D>
__device__ __forceinline__ void store_p(const D &T, int64_t e, const float (&p)[N]) {
    if constexpr (PK == P_F32) {
        stf<N>(static_cast<float *>(T.p), e, p);
    } else if constexpr (PK == P_BF16R) {
        uint32_t b[N], r[N];
#pragma unroll
        for (int k = 0; k < N; ++k) rem_split(p[k], b[k], r[k]);
        sth<N>(static_cast<uint16_t *>(T.p), e, b);
        sth<N>(T.rem, e, r);
    } else {
        stf<N>(T.master, e, p);
        uint32_t c[N];
#pragma unroll
        for (int k = 0; k < N; ++k) c[k] = PK == P_MBF16 ? f32_to_bf16_rne(p[k]) : f32_to_f16_rne(p[k]);
        sth<N>(static_cast<uint16_t *>(T.p), e, c);
    }
}

// fl32(1/a), correctly rounded, for a > 0.  Inside [2^-126, 2^126] (normal a
// with a normal reciprocal) Markstein's correction of the hardware
// reciprocal -- y = rcp(a), e = fma(-a, y, 1), y + e y as one fma (P.
// Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Dev. 34(1), 1990) -- gives the IEEE
// quotient for every such a on gfx950 (a GPU test checks all 2^32 inputs);
// elsewhere (denormal a, or a denormal quotient) the IEEE division.  Three
// VALU instructions instead of the division's ten.
__device__ __forceinline__ float recip_rn(float a) {
    if (a >= 0x1p-126f && a <= 0x1p126f) {
        const float y = __builtin_amdgcn_rcpf(a);
        return __builtin_fmaf(__builtin_fmaf(-a, y, 1.0f), y, y);
    }
    return 1.0f / a;
}

// Gradient load with the AMP unscale applied exactly once ([LTN] analysis).
template <int GK, int N, int LAY = kStrided>
__device__ __forceinline__ void load_g(const void *g, int64_t e, float s, float (&x)[N]) {
    if constexpr (GK == G_F32) {
        ldf<N, LAY>(static_cast<const float *>(g), e, x);
    } else {
        uint32_t b[N];
        ldh<N, LAY>(static_cast<const uint16_t *>(g), e, b);
#pragma unroll
        for (int k = 0; k < N; ++k) x[k] = bf16_to_f32(b[k]);
    }
#pragma unroll
    for (int k = 0; k < N; ++k) x[k] = x[k] * s;
}

// ---------------------------------------------------------------- traversal
// Calls body(u, span, first element, element count) for every unit u this
// workgroup owns.  All arguments are uniform across the workgroup.
// A launch covers units [unit0, nunits).
// Default grid: workgroup b owns units_per_wg consecutive units (usually
// one), and the hardware dispatcher keeps the resident workgroups on one
// narrow, advancing window of every array.  Persistent grid: workgroup b
// takes units b, b + G, b + 2G, ..., so its resident workgroups also sweep
// one window at a time (measured faster on MI355X than one contiguous range
// per workgroup, whose ~1500 separate streams lose DRAM page locality).
__device__ __forceinline__ int span_of(const StepArgs &a, int64_t u) {
    int lo = 0, hi = a.nspans;  // spans[nspans].unit_begin == nunits > u
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.spans[mid].unit_begin <= u) lo = mid; else hi = mid;
    }
    return lo;
}

// REV: the default grid walks the units backwards (workgroup b takes the
// units of workgroup G-1-b), for a second pass that should meet the lines
// its first pass touched last.
template <bool REV = false, class Body>
__device__ __forceinline__ void for_units(const StepArgs &a, Body &&body) {
    int64_t u, u1, stride;
    if (a.grid_request > 0) {
        u = a.unit0 + blockIdx.x;
        u1 = a.nunits;
        stride = gridDim.x;
    } else {
        const int64_t wb = REV ? (int64_t)gridDim.x - 1 - blockIdx.x : (int64_t)blockIdx.x;
        u = a.unit0 + wb * a.units_per_wg;
        u1 = u + a.units_per_wg < a.nunits ? u + a.units_per_wg : a.nunits;
        stride = 1;
    }
    if (u >= u1) return;
    int s = span_of(a, u);
    for (; u < u1; u += stride) {
        while (a.spans[s + 1].unit_begin <= u) ++s;
        const SpanDesc sp = a.spans[s];
        const int64_t off = (u - sp.unit_begin) * a.tile;
        const int64_t len = sp.len - off < a.tile ? sp.len - off : a.tile;
        body(u, sp, sp.elem_begin + off, len);
    }
}

// Visits this lane's elements of the unit [start, start + len) in the
// kStrided layout: lane t owns the groups of 4 at start + 4t + q*kSub.
// body(Int<N>{}, e) handles N elements from e; full groups go G at a time
// (all their loads issue before any use), then one at a time, and a ragged
// end (or a unit whose pointers are not 16-byte aligned) element by element.
template <int N>
struct Int {
    static constexpr int value = N;
};

template <int G, class Body>
__device__ __forceinline__ void lane_walk(int64_t start, int64_t len, bool vec_ok, Body &&body) {
    int64_t rel = threadIdx.x * kVec;
    if (vec_ok && start % kVec == 0) {
        if constexpr (G > 1)
            for (; rel + (G - 1) * kSub + kVec <= len; rel += G * kSub) body(Int<kVec * G>{}, start + rel);
        for (; rel + kVec <= len; rel += kSub) body(Int<kVec>{}, start + rel);
    }
    for (; rel < len; rel += kSub) {
        const int64_t n = len - rel < kVec ? len - rel : kVec;
        for (int64_t j = 0; j < n; ++j) body(Int<1>{}, start + rel + j);
    }
}

// ---------------------------------------------------------------- packs
// A pack span (tensor == kPackTensor) holds several small tensors end to end
// (see PackDesc).  A workgroup copies the pack's offsets and its members'
// PackMember records into LDS (one contiguous copy), then lane t takes the
// pack's groups of 4 elements at 4t + q kSub, as in a unit of one tensor,
// and finds the member holding each group by a binary search of the
// offsets (every member starts at a multiple of 4, so a group never crosses
// two members).  Member records are then read from LDS.
struct PackLds {
    PackMember td[kMaxPackTensors];
    int32_t off[kMaxPackTensors + 1];
};

// Copies pack P's tables into L; ends with a barrier.
__device__ __forceinline__ void pack_fill(const StepArgs &a, const PackDesc &P, PackLds &L) {
    constexpr int kWords = (int)(sizeof(PackMember) / 4);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.pack_td + P.td_base);
    uint32_t *dst = reinterpret_cast<uint32_t *>(L.td);
    for (int i = threadIdx.x; i < P.k * kWords; i += kThreads) dst[i] = src[i];
    for (int i = threadIdx.x; i <= P.k; i += kThreads) L.off[i] = a.pack_off[P.off_base + i];
    __syncthreads();
}

// This lane's G groups from pack element v0 on (v0 + q kSub): member j[q],
// first element e[q] of that member, count n[q] (1..4; 0 past the pack's
// end); whole: every group is 4 elements of a member whose arrays are
// 16-byte aligned.
template <int G>
struct PackSlots {
    int32_t j[G];
    int32_t e[G];
    int32_t n[G];
    bool whole;
};

template <int G>
__device__ __forceinline__ PackSlots<G> pack_slots(const PackLds &L, const PackDesc &P, int32_t v0) {
    PackSlots<G> sl;
    sl.whole = true;
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const int32_t v = v0 + q * (int32_t)kSub;
        int lo = 0, hi = P.k;  // off[lo] <= v < off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (L.off[mid] <= v) lo = mid; else hi = mid;
        }
        sl.j[q] = lo;
        sl.e[q] = v - L.off[lo];
        const int64_t left = v < P.len ? L.td[lo].numel - sl.e[q] : 0;
        sl.n[q] = left < kVec ? (int32_t)left : kVec;
        sl.whole = sl.whole && sl.n[q] == kVec && L.td[lo].vec_ok;
    }
    return sl;
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
        S.lrwd[threadIdx.x] = (float)(S.lr64 * p.group_wd[threadIdx.x]);
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

// Called by thread 0 of every workgroup; true in the last one to arrive
// (the counters are rearmed by then).
__device__ __forceinline__ bool last_arrival(const StepArgs &a) {
    const uint32_t G = gridDim.x, b = blockIdx.x;
    const uint32_t nsub = G < (uint32_t)kSubCounters ? G : (uint32_t)kSubCounters;
    const uint32_t j = b % nsub;
    const uint32_t members = G / nsub + (j < G % nsub ? 1u : 0u);
    uint32_t *sub = a.done + (1 + j) * kCounterStride;
    if (arrive(sub) != members - 1) return false;
    __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (arrive(a.done) != nsub - 1) return false;
    __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

__device__ __forceinline__ void publish_step(const StepArgs &a, const Scalars &S) {
    const PrepArgs &p = a.prep;
    if (p.sched == 1) {
        *p.lr_dev = S.lr;
        *p.iter_dev = S.k + 1;
    }
    if (!S.skip) *p.step_dev = S.t;
}

__device__ __forceinline__ void step_end(const StepArgs &a, const Scalars &S) {
    if (!a.commit || threadIdx.x != 0) return;
    if (last_arrival(a)) publish_step(a, S);
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

// A 64-bit pointer that is the same in every lane, moved to scalar registers.
// readfirstlane returns int: each half goes back through uint32_t, so a low
// half with bit 31 set is not sign-extended into the high half.
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t v = (uint64_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (T *)((hi << 32) | lo);
}

// The descriptor of the tensor a workgroup works on, copied into scalar
// registers.  Through a reference into the plan's table, the compiler must
// assume that the step's own stores may have changed the table, and reloads
// each array's pointer after the previous array's stores, waiting for all of
// them to complete (s_waitcnt vmcnt(0)) before the next array's stores can
// go out; a register copy lets every store of a unit issue back to back.
__device__ __forceinline__ TensorDesc uniform_desc(const TensorDesc &src) {
    TensorDesc T = src;
    T.p = uniform_ptr(T.p);
    T.g = uniform_ptr(T.g);
    T.m = uniform_ptr(T.m);
    T.v = uniform_ptr(T.v);
    T.m2 = uniform_ptr(T.m2);
    T.rem = uniform_ptr(T.rem);
    T.master = uniform_ptr(T.master);
    T.group = __builtin_amdgcn_readfirstlane(T.group);
    T.vec_ok = __builtin_amdgcn_readfirstlane(T.vec_ok);
    return T;
}

// ---------------------------------------------------------------- partial sums
// Sum of x[i * stride] over i in [i0, i1), this lane taking i0 + lane,
// i0 + lane + kThreads, ...: eight independent accumulators, combined in a
// fixed order -- deterministic.  Loads go out 32 at a time (a whole-matrix
// Adam-mini block has up to ~11,000 unit partials, 43 a lane), each
// accumulator still adding its elements in ascending order, so the sum is
// the same as with 8 at a time.
__device__ __forceinline__ double lane_sum(const double *x, int64_t stride, int64_t i0, int64_t i1) {
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    int64_t i = i0 + threadIdx.x;
    for (; i + 31 * kThreads < i1; i += 32 * kThreads) {
        double y[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) y[j] = x[(i + j * kThreads) * stride];
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[j & 7] += y[j];
    }
    for (; i + 7 * kThreads < i1; i += 8 * kThreads) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += x[(i + j * kThreads) * stride];
    }
    for (; i < i1; i += kThreads) acc[0] += x[i * stride];
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
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
// A lane's N elements of every array of the update.
template <int N>
struct AdamRegs {
    float p[N], g[N], m[N], v[N], m2[N];
};

// Where element e's moments sit.  Separate arrays (MI false): m[e], v[e],
// m2[e].  Interleaved (MI, the plan's moment layout): one array per tensor
// in blocks of kMomentBlock elements, block b holding m, then v (then m2)
// of elements [b kMomentBlock, (b + 1) kMomentBlock); the descriptor's v and
// m2 point kMomentBlock and 2 kMomentBlock floats past m, so every moment of
// e sits at the same index e + X (e - e mod kMomentBlock), X the number of
// moments after m, and a lane's groups (kSub = kMomentBlock elements apart)
// are (X + 1) kSub apart.  A pack member (at most kMomentBlock elements, one
// block) needs no remapping.
template <bool MI, bool ADE>
__device__ __forceinline__ int64_t moment_at(int64_t e) {
    if constexpr (MI) return e + (ADE ? 2 : 1) * (e & ~(kMomentBlock - 1));
    else return e;
}
template <bool MI, bool ADE>
constexpr int64_t moment_gs() { return MI ? (ADE ? 3 : 2) * kSub : kSub; }
// v and m2 of the interleaved layout taken from m, so the compiler sees
// that the moments of a group are one run (one address for m and v)
template <bool MI, class D>
__device__ __forceinline__ float *moment_v(const D &T) { return MI ? T.m + kMomentBlock : T.v; }
template <bool MI, class D>
__device__ __forceinline__ float *moment_m2(const D &T) { return MI ? T.m + 2 * kMomentBlock : T.m2; }
static_assert(kSub == kMomentBlock, "a lane's groups step whole moment blocks");

// Loads; the gradient is multiplied by gscale (1 to defer the unscale).
template <int PK, int GK, bool ADE, int N, bool MI = false, class D>
__device__ __forceinline__ void adam_load(const D &T, int64_t e, float gscale, AdamRegs<N> &r) {
    load_p<PK, N>(T, e, r.p);
    load_g<GK, N>(T.g, e, gscale, r.g);
    const int64_t i = moment_at<MI, ADE>(e), gs = moment_gs<MI, ADE>();
    ldf<N>(T.m, i, r.m, gs);
    ldf<N>(moment_v<MI>(T), i, r.v, gs);
    if constexpr (ADE) ldf<N>(moment_m2<MI>(T), i, r.m2, gs);
}

// Decoupled decay and update with one rounding at the parameter's scale:
// p - fma(lw, p, d), lw = fl32(lr wd), d the update term (the fused inner
// term also keeps the register footprint of the bf16-remainder kernels at
// that of a plain multiply by a factor).  Multiplying by
// fl32(1 - lr wd) instead carries that factor's rounding (up to 2^-25
// relative, the same sign every step) into every step: over 100 steps a
// parameter decaying toward zero drifts by several times the fp32 rounding
// of its own value (measured: 1.4e-4 against 4.1e-5 relerr_tau, lr 3e-4).
__device__ __forceinline__ float decayed(float p, float lw, float d) { return p - __builtin_fmaf(lw, p, d); }

template <bool ADE, int N>
__device__ __forceinline__ void adam_math(AdamRegs<N> &r, const AdamK &k, float lw) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r.m[i] = k.b1 * r.m[i] + k.c1 * r.g[i];
        r.v[i] = k.b2 * r.v[i] + k.c2 * (r.g[i] * r.g[i]);
        const float h = sqrtf(r.v[i]) * k.isb2 + k.eps;
        if constexpr (ADE) {
            r.m2[i] = k.b3 * r.m2[i] + k.c3 * r.g[i];
            r.p[i] = decayed(r.p[i], lw, k.lr * ((r.m[i] * k.ibc1 + k.alpha * r.m2[i]) / h));
        } else {
            r.p[i] = decayed(r.p[i], lw, k.ss * (r.m[i] / h));
        }
    }
}

template <int PK, bool ADE, int N, bool MI = false, class D>
__device__ __forceinline__ void adam_store(const D &T, int64_t e, const AdamRegs<N> &r) {
    store_p<PK, N>(T, e, r.p);
    const int64_t i = moment_at<MI, ADE>(e), gs = moment_gs<MI, ADE>();
    stf<N>(T.m, i, r.m, gs);
    stf<N>(moment_v<MI>(T), i, r.v, gs);
    if constexpr (ADE) stf<N>(moment_m2<MI>(T), i, r.m2, gs);
}

template <int PK, int GK, bool ADE, int N, bool MI = false, class D>
__device__ __forceinline__ void adam_elems(const D &T, int64_t e, const AdamK &k, float lw) {
    AdamRegs<N> r;
    adam_load<PK, GK, ADE, N, MI>(T, e, k.inv_scale, r);
    adam_math<ADE, N>(r, k, lw);
    adam_store<PK, ADE, N, MI>(T, e, r);
}

// AdamW / AdEMAMix over a lane's G groups of a pack.  Whole slots: all
// loads (adam_pack_load, gradient times gscale) issue before the
// arithmetic and the stores (adam_pack_finish, which applies the remaining
// gradient scale rs); otherwise adam_pack_finish goes group by group,
// element by element where a group is partial.
template <int PK, int GK, bool ADE, int G>
__device__ __forceinline__ void adam_pack_load(const PackLds &L, const PackSlots<G> &sl, float gscale,
                                               AdamRegs<kVec> (&r)[G]) {
    if (!sl.whole) return;
#pragma unroll
    for (int q = 0; q < G; ++q) adam_load<PK, GK, ADE, kVec>(L.td[sl.j[q]], sl.e[q], gscale, r[q]);
}

template <int PK, int GK, bool ADE, int G>
__device__ __forceinline__ void adam_pack_finish(const PackLds &L, const PackSlots<G> &sl, const Scalars &S,
                                                 const AdamK &k, float rs, AdamRegs<kVec> (&r)[G]) {
    if (sl.whole) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int i = 0; i < kVec; ++i) r[q].g[i] = r[q].g[i] * rs;
            adam_math<ADE, kVec>(r[q], k, S.lrwd[L.td[sl.j[q]].group]);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) adam_store<PK, ADE, kVec>(L.td[sl.j[q]], sl.e[q], r[q]);
        return;
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
        if (sl.n[q] == 0) continue;
        const PackMember &T = L.td[sl.j[q]];
        const float lw = S.lrwd[T.group];
        if (sl.n[q] == kVec && T.vec_ok)
            adam_elems<PK, GK, ADE, kVec>(T, sl.e[q], k, lw);
        else
            for (int i = 0; i < sl.n[q]; ++i) adam_elems<PK, GK, ADE, 1>(T, sl.e[q] + i, k, lw);
    }
}

// A whole pack after the prologue: G groups per lane at a time.
template <int PK, int GK, bool ADE, int G>
__device__ __forceinline__ void adam_pack_unit(const StepArgs &a, const SpanDesc &sp, PackLds &L, const Scalars &S,
                                               const AdamK &k) {
    const PackDesc P = a.packs[sp.elem_begin];
    pack_fill(a, P, L);
    for (int32_t v0 = (int32_t)threadIdx.x * kVec; v0 < P.len; v0 += G * (int32_t)kSub) {
        const PackSlots<G> sl = pack_slots<G>(L, P, v0);
        AdamRegs<kVec> r[G];
        adam_pack_load<PK, GK, ADE, G>(L, sl, k.inv_scale, r);
        adam_pack_finish<PK, GK, ADE, G>(L, sl, S, k, 1.0f, r);
    }
    __syncthreads();  // L is refilled for the next pack
}

template <int PK, int GK, bool ADE, int G = kAdamGroups, bool MI = false>
__device__ __forceinline__ void adam_unit(const TensorDesc &T, int64_t start, int64_t len,
                                          const AdamK &k, float lw) {
    lane_walk<G>(start, len, T.vec_ok, [&](auto n, int64_t e) {
        adam_elems<PK, GK, ADE, decltype(n)::value, MI>(T, e, k, lw);
    });
}

// Grid: ceil(units / units_per_wg) workgroups, unless the plan asked for a
// persistent grid of grid_request workgroups (never more than there are
// units).  At least one workgroup: the commit must run for an empty plan.
template <class K>
int persistent_grid(K, const StepArgs &a) {
    const int64_t units = a.nunits > a.unit0 ? a.nunits - a.unit0 : 1;
    int64_t g;
    if (a.grid_request > 0)
        g = a.grid_request < units ? a.grid_request : units;
    else
        g = (units + a.units_per_wg - 1) / a.units_per_wg;
    return (int)(g < INT32_MAX ? g : INT32_MAX);
}

// Whether a two-pass step keeps the arrays its second pass reads again in
// the Infinity Cache (kStridedKeep accesses in both passes, the second pass
// walking backwards): only on the default grid and while those bytes stay
// under `limit`; past it, ordinary accesses stream slower than non-temporal
// ones.  The limits are measured per step on MI355X.
inline bool keep_for_second_pass(const StepArgs &a, int64_t reread_bytes_per_elem, int64_t limit) {
    return a.grid_request == 0 && (a.nunits - a.unit0) * a.tile * reread_bytes_per_elem <= limit;
}

// Launch of kernel K over `grid` workgroups of `block` lanes; under a plan
// trace the kernel's own start and end stamp the trace's next event pair.
#define LAUNCH_TRACED(K, grid, block, s, ...)                                                      \
    do {                                                                                           \
        TraceRec *tr_ = trace_slot(#K, (int64_t)(grid));                                           \
        if (tr_)                                                                                   \
            hipExtLaunchKernelGGL(K, dim3(grid), dim3(block), 0, s, tr_->start, tr_->stop, 0, __VA_ARGS__); \
        else                                                                                       \
            hipLaunchKernelGGL(K, dim3(grid), dim3(block), 0, s, __VA_ARGS__);                    \
    } while (0)

#define LAUNCH_PERSISTENT(K, a, s) LAUNCH_TRACED(K, persistent_grid(K, a), kThreads, s, a)

}  // namespace
}  // namespace optim
