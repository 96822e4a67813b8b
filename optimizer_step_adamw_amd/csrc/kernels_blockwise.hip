// kernels_blockwise.hip -- blockwise 8-bit / 4-bit state step and the quantize /
// dequantize helpers that share its device code.
#include "device_common.h"

namespace optim {
namespace {

// ---------------------------------------------------------------- blockwise
// [BNB]: 2-state blockwise 8-bit AdamW with the Algorithm 2 decay order;
// [AO]: 4-bit states.  One quantization block = L consecutive lanes of one
// wavefront (L = block / E, E elements per lane), so the block absmax is a
// butterfly max over L lanes.  The maps (values, thresholds, bucket table)
// live in LDS.
template <int MB>
struct LdsMap {
    float vals[1 << MB];
    float thr[1 << MB];
    uint8_t lut[kLutBuckets];
};

template <int MB>
__device__ __forceinline__ void load_map(LdsMap<MB> &dst, const QuantMap &src) {
    for (int i = threadIdx.x; i < (1 << MB); i += kThreads) {
        dst.vals[i] = src.vals[i];
        dst.thr[i] = src.thr[i];
    }
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src.lut);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(dst.lut);
    for (int i = threadIdx.x; i < kLutBuckets / 16; i += kThreads) d4[i] = s4[i];
}

// Largest j with thr[j] <= a, for a >= 0 (a below 2^-26 is below thr[1]).
template <int MB>
__device__ __forceinline__ uint32_t code_index(const LdsMap<MB> &M, float a) {
    const int32_t bucket =
        (int32_t)(__float_as_uint(a) >> (23 - kLutMantBits)) - (kLutBaseExp << kLutMantBits);
    if (bucket < 0) return 0;
    uint32_t c = M.lut[bucket < kLutBuckets ? bucket : kLutBuckets - 1];
    if (c + 1 < (1u << MB) && M.thr[c + 1] <= a) ++c;
    return c;
}

// Codes of this lane's E elements (element j in bits [j*BITS, (j+1)*BITS));
// the block is this lane's group of L lanes.  A = max|x| over the block,
// r = fl32(1/A) (IEEE division), a = fl32(|x| r); signed maps put the sign
// above the magnitude bits, sign 0 for index 0; A = 0 gives all-zero codes.
// Elements j >= nv must hold 0.
template <int BITS, bool SIGNED, int E>
__device__ __forceinline__ uint32_t quantize_lane(const float (&x)[E], int L,
                                                  const LdsMap<SIGNED ? BITS - 1 : BITS> &M, float &A) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j) mx = fmaxf(mx, fabsf(x[j]));
    for (int o = L >> 1; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    A = mx;
    if (!(mx > 0.0f)) return 0u;
    const float r = 1.0f / mx;
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        uint32_t c = code_index<MB>(M, fabsf(x[j]) * r);
        if (SIGNED && x[j] < 0.0f && c > 0) c |= 1u << MB;
        out |= c << (j * BITS);
    }
    return out;
}

// x = fl32(+-vals[idx] * A)
template <int BITS, bool SIGNED, int E>
__device__ __forceinline__ void dequantize_lane(uint32_t codes, float A,
                                                const LdsMap<SIGNED ? BITS - 1 : BITS> &M, float (&x)[E]) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint32_t c = (codes >> (j * BITS)) & MASK;
        const float mag = M.vals[c & ((1u << MB) - 1u)] * A;
        x[j] = (SIGNED && ((c >> MB) & 1u)) ? -mag : mag;
    }
}

// Packed codes of elements [e, e + E) (e a multiple of E, so this lane owns
// whole bytes); the nv < E tail is read and written byte by byte.
template <int BITS, int E>
__device__ __forceinline__ uint32_t load_codes(const uint8_t *q, int64_t e, int nv, bool full) {
    const int64_t byte0 = e * BITS / 8;
    if (full) return *(const GMEM uint32_t *)gp(q + byte0);
    uint32_t out = 0;
    const int nbytes = (nv * BITS + 7) / 8;
    for (int b = 0; b < nbytes; ++b) out |= (uint32_t)gp(q)[byte0 + b] << (8 * b);
    if (nv * BITS < 32) out &= (1u << (nv * BITS)) - 1u;  // drop a foreign half byte
    return out;
}

template <int BITS, int E>
__device__ __forceinline__ void store_codes(uint8_t *q, int64_t e, int nv, bool full, uint32_t c) {
    const int64_t byte0 = e * BITS / 8;
    if (full) {
        *(GMEM uint32_t *)gp(q + byte0) = c;
        return;
    }
    const int nbytes = (nv * BITS + 7) / 8;
    for (int b = 0; b < nbytes; ++b) gp(q)[byte0 + b] = (uint8_t)(c >> (8 * b));
}

template <int GK, int BITS>
__global__ __launch_bounds__(kThreads) void blockwise_kernel(StepArgs a) {
    constexpr int E = BITS == 8 ? 4 : 8;  // elements per lane per row
    __shared__ LdsMap<BITS - 1> Mm;
    __shared__ LdsMap<BITS> Mv;
    load_map(Mm, BITS == 8 ? a.codebook->m8 : a.codebook->m4);
    load_map(Mv, BITS == 8 ? a.codebook->v8 : a.codebook->v4);
    __shared__ Scalars S;
    step_begin(a, S);  // its barriers also publish the maps
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
            const int64_t e = start + rel;  // a multiple of E
            const int64_t blk = e / a.block;
            const bool full = T.vec_ok && nv == E;
            float p[E], g[E];
            float Am = 0.0f, Av = 0.0f;
            if (nv > 0) {
                Am = gp(T.am)[blk];
                Av = gp(T.av)[blk];
            }
            if (full) {
                ldf<E>(P, e, p);
                load_g<GK, E>(T.g, e, k.inv_scale, g);
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    float pj[1] = {0.0f}, gj[1] = {0.0f};
                    if (j < nv) {
                        ldf<1>(P, e + j, pj);
                        load_g<GK, 1>(T.g, e + j, k.inv_scale, gj);
                    }
                    p[j] = pj[0];
                    g[j] = gj[0];
                }
            }
            const uint32_t cm = nv > 0 ? load_codes<BITS, E>(T.qm, e, nv, full) : 0u;
            const uint32_t cv = nv > 0 ? load_codes<BITS, E>(T.qv, e, nv, full) : 0u;
            float mt[E], vt[E];
            dequantize_lane<BITS, true, E>(cm, Am, Mm, mt);
            dequantize_lane<BITS, false, E>(cv, Av, Mv, vt);
            // fp32 state recipe, every product and sum rounded on its own
            float mn[E], vn[E];
#pragma unroll
            for (int j = 0; j < E; ++j) {
                mn[j] = j < nv ? k.b1 * mt[j] + k.c1 * g[j] : 0.0f;
                vn[j] = j < nv ? k.b2 * vt[j] + k.c2 * (g[j] * g[j]) : 0.0f;
                // parameter update: hardware sqrt / reciprocal (1 ulp each)
                const float h = __builtin_amdgcn_sqrtf(vn[j]) * k.isb2 + k.eps;
                p[j] = p[j] * decay - k.ss * (mn[j] * __builtin_amdgcn_rcpf(h));
            }
            float Am2, Av2;
            const uint32_t om = quantize_lane<BITS, true, E>(mn, L, Mm, Am2);
            const uint32_t ov = quantize_lane<BITS, false, E>(vn, L, Mv, Av2);
            if (full) {
                stf<E>(P, e, p);
            } else {
                for (int j = 0; j < nv; ++j) {
                    const float pj[1] = {p[j]};
                    stf<1>(P, e + j, pj);
                }
            }
            if (nv > 0) {
                store_codes<BITS, E>(T.qm, e, nv, full, om);
                store_codes<BITS, E>(T.qv, e, nv, full, ov);
                if ((lane & (L - 1)) == 0) {
                    gp(T.am)[blk] = Am2;
                    gp(T.av)[blk] = Av2;
                }
            }
        }
    });
}

// Blockwise quantize / dequantize of a plain fp32 array with the same code
// path as the step (state import and export).  Rows of kThreads * E
// elements, grid-stride; the loop trip count is uniform per workgroup.
template <int BITS, bool SIGNED>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const Codebook *cb, int block, const float *x,
                                                           int64_t n, bool vec, uint8_t *codes, float *absmax) {
    constexpr int E = BITS == 8 ? 4 : 8;
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    __shared__ LdsMap<MB> M;
    load_map(M, BITS == 8 ? (SIGNED ? cb->m8 : cb->v8) : (SIGNED ? cb->m4 : cb->v4));
    __syncthreads();
    const int L = block / E;
    const int64_t rowlen = (int64_t)kThreads * E, nrows = (n + rowlen - 1) / rowlen;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t e = row * rowlen + threadIdx.x * E;
        const int nv = n - e >= E ? E : (n - e > 0 ? (int)(n - e) : 0);
        const bool full = vec && nv == E;
        float v[E];
        if (full) {
            ldf<E>(x, e, v);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                float vj[1] = {0.0f};
                if (j < nv) ldf<1>(x, e + j, vj);
                v[j] = vj[0];
            }
        }
        float A;
        const uint32_t c = quantize_lane<BITS, SIGNED, E>(v, L, M, A);
        if (nv > 0) {
            store_codes<BITS, E>(codes, e, nv, full, c);
            if ((threadIdx.x & (L - 1)) == 0) gp(absmax)[e / block] = A;
        }
    }
}

template <int BITS, bool SIGNED>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const Codebook *cb, int block, const uint8_t *codes,
                                                             const float *absmax, int64_t n, bool vec, float *x) {
    constexpr int E = BITS == 8 ? 4 : 8;
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    __shared__ LdsMap<MB> M;
    load_map(M, BITS == 8 ? (SIGNED ? cb->m8 : cb->v8) : (SIGNED ? cb->m4 : cb->v4));
    __syncthreads();
    const int64_t rowlen = (int64_t)kThreads * E, nrows = (n + rowlen - 1) / rowlen;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t e = row * rowlen + threadIdx.x * E;
        const int nv = n - e >= E ? E : (n - e > 0 ? (int)(n - e) : 0);
        if (nv == 0) continue;
        const bool full = vec && nv == E;
        float v[E];
        dequantize_lane<BITS, SIGNED, E>(load_codes<BITS, E>(codes, e, nv, full), gp(absmax)[e / block], M, v);
        if (full) {
            stf<E>(x, e, v);
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
    const int E = bits == 8 ? 4 : 8;
    const int64_t rows = (n + (int64_t)kThreads * E - 1) / ((int64_t)kThreads * E);
    const int grid = (int)(rows < 16384 ? (rows > 0 ? rows : 1) : 16384);
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 4 == 0);
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
    const int E = bits == 8 ? 4 : 8;
    const int64_t rows = (n + (int64_t)kThreads * E - 1) / ((int64_t)kThreads * E);
    const int grid = (int)(rows < 16384 ? (rows > 0 ? rows : 1) : 16384);
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 4 == 0);
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
