// kernels_blockwise.hip -- blockwise 8-bit / 4-bit state step and the
// quantize / dequantize helpers that share its device code.
//
// [BNB]: the 2-state branch of the blockwise 8-bit kernel, with the
// Algorithm 2 decay order; [AO]: 4-bit optimizer states.  Each lane owns 8
// consecutive elements per row of 2048; one quantization block is L = block/8
// consecutive lanes of one wavefront, so the block absmax is a max over an
// aligned lane group (DPP row operations, then one swizzle / readlane step).
// The maps -- values, thresholds and the bucket table of the code search --
// live in LDS.  This step issues far more VALU and LDS work per byte than the
// elementwise steps, so every per-element instruction counts here.
#include "device_common.h"

namespace optim {
namespace {

constexpr int kQE = 8;  // elements per lane per row
constexpr int64_t kQRow = (int64_t)kThreads * kQE;

template <int MB>
struct LdsMap {
    float vals[1 << MB];
    float thr[(1 << MB) + 4];  // thr[2^MB] = +inf ends the search
    uint8_t lut[kLutBuckets];
};

template <int MB>
__device__ __forceinline__ void load_map(LdsMap<MB> &dst, const QuantMap &src) {
    for (int i = threadIdx.x; i < (1 << MB); i += kThreads) dst.vals[i] = src.vals[i];
    for (int i = threadIdx.x; i <= (1 << MB); i += kThreads) dst.thr[i] = src.thr[i];
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src.lut);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(dst.lut);
    for (int i = threadIdx.x; i < kLutBuckets / 16; i += kThreads) d4[i] = s4[i];
}

// Largest j with thr[j] <= a (a >= 0).  The bucket of a (exponent and top
// mantissa bits, clamped to the table) gives the index of the bucket's
// smallest value; the bucket holds at most one threshold, so one comparison
// finishes.  Below 2^-26 every a maps to 0 (bucket 0 holds index 0 and
// thr[1] > 2^-26).
template <int MB>
__device__ __forceinline__ uint32_t code_index(const LdsMap<MB> &M, float a) {
    int32_t b = (int32_t)(__float_as_uint(a) >> (23 - kLutMantBits)) - (kLutBaseExp << kLutMantBits);
    b = b < 0 ? 0 : (b < kLutBuckets ? b : kLutBuckets - 1);
    const uint32_t c = M.lut[b];
    return c + (M.thr[c + 1] <= a ? 1u : 0u);
}

template <int CTRL>
__device__ __forceinline__ float max_dpp(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false);
    return fmaxf(x, __int_as_float(y));
}

// Max over each aligned group of L lanes (L a power of two, <= 64); every
// lane of a group receives its group's max.  Needs all 64 lanes active.
__device__ __forceinline__ float group_max(float x, int L) {
    if (L >= 2) x = max_dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if (L >= 4) x = max_dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if (L >= 8) x = max_dpp<0x141>(x);  // row_half_mirror
    if (L >= 16) x = max_dpp<0x140>(x); // row_mirror
    if (L >= 32)                        // lanes i <-> i ^ 16 within 32
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
    if (L >= 64)
        x = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)));
    return x;
}

// Codes of this lane's 8 elements (element j in bits [j*BITS, (j+1)*BITS));
// the block is this lane's group of L lanes.  A = max|x| over the block,
// r = fl32(1/A) (IEEE division), a = fl32(|x| r); signed maps put the sign
// above the magnitude bits, sign 0 for index 0; A = 0 gives all-zero codes.
// Elements outside the tensor must hold 0.
template <int BITS, bool SIGNED>
__device__ __forceinline__ uint64_t quantize_lane(const float (&x)[kQE], int L,
                                                  const LdsMap<SIGNED ? BITS - 1 : BITS> &M, float &A) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    float mx = fabsf(x[0]);
#pragma unroll
    for (int j = 1; j < kQE; ++j) mx = fmaxf(mx, fabsf(x[j]));
    mx = group_max(mx, L);
    A = mx;
    const float r = mx > 0.0f ? 1.0f / mx : 0.0f;
    uint64_t out = 0;
#pragma unroll
    for (int j = 0; j < kQE; ++j) {
        uint32_t c = code_index<MB>(M, fabsf(x[j]) * r);
        if (SIGNED) c |= (x[j] < 0.0f && c > 0) ? (1u << MB) : 0u;
        out |= (uint64_t)c << (j * BITS);
    }
    return out;
}

// x = fl32(+-vals[idx] * A)
template <int BITS, bool SIGNED>
__device__ __forceinline__ void dequantize_lane(uint64_t codes, float A,
                                                const LdsMap<SIGNED ? BITS - 1 : BITS> &M, float (&x)[kQE]) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
#pragma unroll
    for (int j = 0; j < kQE; ++j) {
        const uint32_t c = (uint32_t)(codes >> (j * BITS)) & ((1u << BITS) - 1u);
        const float mag = M.vals[c & ((1u << MB) - 1u)] * A;
        x[j] = (SIGNED && ((c >> MB) & 1u)) ? -mag : mag;
    }
}

// Packed codes of elements [e, e + 8) (e a multiple of 8, so this lane owns
// whole bytes).  Full: one 8-byte (8-bit) or 4-byte (4-bit) access.
template <int BITS>
__device__ __forceinline__ uint64_t load_codes_full(const uint8_t *q, int64_t e) {
    const int64_t byte0 = e * BITS / 8;
    if constexpr (BITS == 8) {
        const u32x2 w = *(const GMEM u32x2 *)gp(q + byte0);
        return (uint64_t)w.x | ((uint64_t)w.y << 32);
    } else {
        return *(const GMEM uint32_t *)gp(q + byte0);
    }
}

template <int BITS>
__device__ __forceinline__ void store_codes_full(uint8_t *q, int64_t e, uint64_t c) {
    const int64_t byte0 = e * BITS / 8;
    if constexpr (BITS == 8)
        *(GMEM u32x2 *)gp(q + byte0) = u32x2{(uint32_t)c, (uint32_t)(c >> 32)};
    else
        *(GMEM uint32_t *)gp(q + byte0) = (uint32_t)c;
}

// Tail: nv < 8 valid elements, byte by byte; a half byte beyond the tensor
// reads as 0 and is written as 0.
template <int BITS>
__device__ __forceinline__ uint64_t load_codes_part(const uint8_t *q, int64_t e, int nv) {
    const int64_t byte0 = e * BITS / 8;
    uint64_t out = 0;
    const int nbytes = (nv * BITS + 7) / 8;
    for (int b = 0; b < nbytes; ++b) out |= (uint64_t)gp(q)[byte0 + b] << (8 * b);
    return nv * BITS < 64 ? out & ((1ull << (nv * BITS)) - 1ull) : out;
}

template <int BITS>
__device__ __forceinline__ void store_codes_part(uint8_t *q, int64_t e, int nv, uint64_t c) {
    const int64_t byte0 = e * BITS / 8;
    const int nbytes = (nv * BITS + 7) / 8;
    for (int b = 0; b < nbytes; ++b) gp(q)[byte0 + b] = (uint8_t)(c >> (8 * b));
}

struct BlockCtx {
    const TensorDesc *T;
    int L, lane, block;
    float decay;
};

// One row of 2048 elements: this lane's 8 elements start at element e.
// FULL: the whole row is inside the tensor and every pointer is aligned.
template <int GK, int BITS, bool FULL>
__device__ __forceinline__ void blockwise_row(const BlockCtx &c, const AdamK &k, int64_t e, int nv,
                                              const LdsMap<BITS - 1> &Mm, const LdsMap<BITS> &Mv) {
    const TensorDesc &T = *c.T;
    float *P = static_cast<float *>(T.p);
    const int64_t blk = e / c.block;
    float p[kQE], g[kQE], am = 0.0f, av = 0.0f;
    uint64_t cm = 0, cv = 0;
    if (FULL || nv > 0) {
        am = gp(T.am)[blk];
        av = gp(T.av)[blk];
    }
    if (FULL) {
        ldf<kQE, kRun>(P, e, p);
        load_g<GK, kQE, kRun>(T.g, e, k.inv_scale, g);
        cm = load_codes_full<BITS>(T.qm, e);
        cv = load_codes_full<BITS>(T.qv, e);
    } else {
#pragma unroll
        for (int j = 0; j < kQE; ++j) {
            float pj[1] = {0.0f}, gj[1] = {0.0f};
            if (j < nv) {
                ldf<1>(P, e + j, pj);
                load_g<GK, 1>(T.g, e + j, k.inv_scale, gj);
            }
            p[j] = pj[0];
            g[j] = gj[0];
        }
        if (nv > 0) {
            cm = load_codes_part<BITS>(T.qm, e, nv);
            cv = load_codes_part<BITS>(T.qv, e, nv);
        }
    }
    float mt[kQE], vt[kQE];
    dequantize_lane<BITS, true>(cm, am, Mm, mt);
    dequantize_lane<BITS, false>(cv, av, Mv, vt);
    // fp32 state recipe, every product and sum rounded on its own; outside
    // the tensor g = 0 and the codes are 0, so the new states are 0 there
    float mn[kQE], vn[kQE];
#pragma unroll
    for (int j = 0; j < kQE; ++j) {
        mn[j] = k.b1 * mt[j] + k.c1 * g[j];
        vn[j] = k.b2 * vt[j] + k.c2 * (g[j] * g[j]);
        // parameter update: hardware sqrt / reciprocal (1 ulp each)
        const float h = __builtin_amdgcn_sqrtf(vn[j]) * k.isb2 + k.eps;
        p[j] = p[j] * c.decay - k.ss * (mn[j] * __builtin_amdgcn_rcpf(h));
    }
    float am2, av2;
    const uint64_t om = quantize_lane<BITS, true>(mn, c.L, Mm, am2);
    const uint64_t ov = quantize_lane<BITS, false>(vn, c.L, Mv, av2);
    if (FULL) {
        stf<kQE, kRun>(P, e, p);
        store_codes_full<BITS>(T.qm, e, om);
        store_codes_full<BITS>(T.qv, e, ov);
    } else if (nv > 0) {
        for (int j = 0; j < nv; ++j) {
            const float pj[1] = {p[j]};
            stf<1>(P, e + j, pj);
        }
        store_codes_part<BITS>(T.qm, e, nv, om);
        store_codes_part<BITS>(T.qv, e, nv, ov);
    }
    if ((FULL || nv > 0) && (c.lane & (c.L - 1)) == 0) {
        gp(T.am)[blk] = am2;
        gp(T.av)[blk] = av2;
    }
}

template <int GK, int BITS>
__global__ __launch_bounds__(kThreads) void blockwise_kernel(StepArgs a) {
    __shared__ LdsMap<BITS - 1> Mm;
    __shared__ LdsMap<BITS> Mv;
    load_map(Mm, BITS == 8 ? a.codebook->m8 : a.codebook->m4);
    load_map(Mv, BITS == 8 ? a.codebook->v8 : a.codebook->v4);
    __shared__ Scalars S;
    step_begin(a, S);  // its barriers also publish the maps
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len) {
        BlockCtx c;
        c.T = &a.tensors[sp.tensor];
        c.L = a.block / kQE;
        c.lane = threadIdx.x & 63;
        c.block = a.block;
        c.decay = uniform(S.decay[c.T->group]);
        const bool aligned = c.T->vec_ok;
        for (int64_t r0 = 0; r0 < len; r0 += kQRow) {
            const int64_t rel = r0 + threadIdx.x * kQE;
            const int64_t e = start + rel;  // a multiple of 8
            if (aligned && r0 + kQRow <= len) {
                blockwise_row<GK, BITS, true>(c, k, e, kQE, Mm, Mv);
            } else {
                const int nv = len - rel >= kQE ? kQE : (len - rel > 0 ? (int)(len - rel) : 0);
                blockwise_row<GK, BITS, false>(c, k, e, nv, Mm, Mv);
            }
        }
    });
}

// Blockwise quantize / dequantize of a plain fp32 array with the same code
// path as the step (state import and export).  Rows of 2048 elements,
// grid-stride; the loop trip count is uniform per workgroup.
template <int BITS, bool SIGNED>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const Codebook *cb, int block, const float *x,
                                                           int64_t n, bool vec, uint8_t *codes, float *absmax) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    __shared__ LdsMap<MB> M;
    load_map(M, BITS == 8 ? (SIGNED ? cb->m8 : cb->v8) : (SIGNED ? cb->m4 : cb->v4));
    __syncthreads();
    const int L = block / kQE;
    const int64_t nrows = (n + kQRow - 1) / kQRow;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t e = row * kQRow + threadIdx.x * kQE;
        const int nv = n - e >= kQE ? kQE : (n - e > 0 ? (int)(n - e) : 0);
        const bool full = vec && nv == kQE;
        float v[kQE];
        if (full) {
            ldf<kQE, kRun>(x, e, v);
        } else {
#pragma unroll
            for (int j = 0; j < kQE; ++j) {
                float vj[1] = {0.0f};
                if (j < nv) ldf<1>(x, e + j, vj);
                v[j] = vj[0];
            }
        }
        float A;
        const uint64_t c = quantize_lane<BITS, SIGNED>(v, L, M, A);
        if (full)
            store_codes_full<BITS>(codes, e, c);
        else if (nv > 0)
            store_codes_part<BITS>(codes, e, nv, c);
        if (nv > 0 && (threadIdx.x & (L - 1)) == 0) gp(absmax)[e / block] = A;
    }
}

template <int BITS, bool SIGNED>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const Codebook *cb, int block, const uint8_t *codes,
                                                             const float *absmax, int64_t n, bool vec, float *x) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    __shared__ LdsMap<MB> M;
    load_map(M, BITS == 8 ? (SIGNED ? cb->m8 : cb->v8) : (SIGNED ? cb->m4 : cb->v4));
    __syncthreads();
    const int64_t nrows = (n + kQRow - 1) / kQRow;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t e = row * kQRow + threadIdx.x * kQE;
        const int nv = n - e >= kQE ? kQE : (n - e > 0 ? (int)(n - e) : 0);
        if (nv == 0) continue;
        const bool full = vec && nv == kQE;
        float v[kQE];
        const uint64_t c = full ? load_codes_full<BITS>(codes, e) : load_codes_part<BITS>(codes, e, nv);
        dequantize_lane<BITS, SIGNED>(c, gp(absmax)[e / block], M, v);
        if (full) {
            stf<kQE, kRun>(x, e, v);
        } else {
            for (int j = 0; j < nv; ++j) {
                const float vj[1] = {v[j]};
                stf<1>(x, e + j, vj);
            }
        }
    }
}

}  // namespace

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

hipError_t launch_quantize(const Codebook *cb, int bits, int block, int is_signed, const float *x,
                           int64_t n, uint8_t *codes, float *absmax, hipStream_t s) {
    const int64_t rows = (n + kQRow - 1) / kQRow;
    const int grid = (int)(rows < 16384 ? (rows > 0 ? rows : 1) : 16384);
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 8 == 0);
    if (bits == 8 && is_signed)
        hipLaunchKernelGGL((quantize_kernel<8, true>), dim3(grid), dim3(kThreads), 0, s, cb, block, x, n, vec, codes, absmax);
    else if (bits == 8)
        hipLaunchKernelGGL((quantize_kernel<8, false>), dim3(grid), dim3(kThreads), 0, s, cb, block, x, n, vec, codes, absmax);
    else if (is_signed)
        hipLaunchKernelGGL((quantize_kernel<4, true>), dim3(grid), dim3(kThreads), 0, s, cb, block, x, n, vec, codes, absmax);
    else
        hipLaunchKernelGGL((quantize_kernel<4, false>), dim3(grid), dim3(kThreads), 0, s, cb, block, x, n, vec, codes, absmax);
    return hipGetLastError();
}

hipError_t launch_dequantize(const Codebook *cb, int bits, int block, int is_signed, const uint8_t *codes,
                             const float *absmax, int64_t n, float *x, hipStream_t s) {
    const int64_t rows = (n + kQRow - 1) / kQRow;
    const int grid = (int)(rows < 16384 ? (rows > 0 ? rows : 1) : 16384);
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 8 == 0);
    if (bits == 8 && is_signed)
        hipLaunchKernelGGL((dequantize_kernel<8, true>), dim3(grid), dim3(kThreads), 0, s, cb, block, codes, absmax, n, vec, x);
    else if (bits == 8)
        hipLaunchKernelGGL((dequantize_kernel<8, false>), dim3(grid), dim3(kThreads), 0, s, cb, block, codes, absmax, n, vec, x);
    else if (is_signed)
        hipLaunchKernelGGL((dequantize_kernel<4, true>), dim3(grid), dim3(kThreads), 0, s, cb, block, codes, absmax, n, vec, x);
    else
        hipLaunchKernelGGL((dequantize_kernel<4, false>), dim3(grid), dim3(kThreads), 0, s, cb, block, codes, absmax, n, vec, x);
    return hipGetLastError();
}

}  // namespace optim
