// kernels_blockwise.hip -- blockwise 8-bit / 4-bit state step and the
// quantize / dequantize helpers that share its device code.
//
// [BNB]: the 2-state branch of the blockwise 8-bit kernel, with the
// Algorithm 2 decay order; [AO]: 4-bit optimizer states.  Each lane owns E
// consecutive elements per row of 256*E; one quantization block is
// L = block/E consecutive lanes of one wavefront, so the block absmax is a
// max over an aligned lane group (DPP row operations, then one swizzle /
// readlane step).  E = 4 wherever a block fits in one wave (block <= 256):
// a wave instruction then covers one contiguous run and the accesses are
// non-temporal, as in the elementwise steps.  E = 8 (ordinary accesses) for
// 4-bit blocks of 512.  The maps -- values, thresholds and the bucket table
// of the code search -- live in LDS.  This step issues far more VALU and LDS
// work per byte than the elementwise steps, so every per-element
// instruction counts here.
#include "device_common.h"

#include <type_traits>

namespace optim {
namespace {

// lanes per block <= 64 (one wave): E = 4 up to block 256, else 8
__host__ __device__ constexpr int lane_elems(int block) { return block <= 256 ? 4 : 8; }
template <int E>
constexpr int row_layout() { return E == 4 ? kStrided : kRun; }

// vals: the 2^MB magnitudes, then their negations, so a signed code (sign
// bit above the MB magnitude bits) indexes its signed value directly.
template <int MB>
struct LdsMap {
    float vals[2 << MB];
    float thr[(1 << MB) + 4];  // thr[2^MB] = +inf ends the search
    uint8_t lut[kLutBuckets];
};

template <int MB>
__device__ __forceinline__ void load_map(LdsMap<MB> &dst, const QuantMap &src) {
    for (int i = threadIdx.x; i < (2 << MB); i += kThreads)
        dst.vals[i] = i < (1 << MB) ? src.vals[i] : -src.vals[i - (1 << MB)];
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
    const int32_t b = __builtin_elementwise_min(
        __builtin_elementwise_max((int32_t)(__float_as_uint(a) >> (23 - kLutMantBits)) -
                                      (kLutBaseExp << kLutMantBits), 0),
        kLutBuckets - 1);
    const uint32_t c = M.lut[b];
    return c + (M.thr[c + 1] <= a ? 1u : 0u);
}

// Lane-group max on the bit patterns of non-negative, NaN-free floats,
// whose unsigned order is their numeric order (no canonicalisation of
// exchanged values, and the exchange folds into the max instruction).
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t x) {
    const uint32_t y = __builtin_amdgcn_update_dpp(0u, x, CTRL, 0xF, 0xF, false);
    return x > y ? x : y;
}

// Max over each aligned group of L lanes (L a power of two, <= 64); every
// lane of a group receives its group's max.  Needs all 64 lanes active.
template <int L>
__device__ __forceinline__ uint32_t group_max(uint32_t x) {
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lane group");
    if constexpr (L >= 2) x = max_dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (L >= 4) x = max_dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (L >= 8) x = max_dpp<0x141>(x);  // row_half_mirror
    if constexpr (L >= 16) x = max_dpp<0x140>(x); // row_mirror
    // Swapping a register with itself across rows: permlane16_swap pairs lane
    // i with i ^ 16, permlane32_swap pairs i with i ^ 32 (VALU, no LDS).
    if constexpr (L >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        x = r[0] > r[1] ? r[0] : r[1];
    }
    if constexpr (L >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        x = r[0] > r[1] ? r[0] : r[1];
    }
    return x;
}

// Codes of this lane's E elements (element j in bits [j*BITS, (j+1)*BITS));
// the block is this lane's group of L lanes.  A = max|x| over the block,
// r = fl32(1/A) (IEEE division), a = fl32(|x| r); signed maps put the sign
// above the magnitude bits, sign 0 for index 0; A = 0 gives all-zero codes.
// Elements outside the tensor must hold 0.
template <int BITS, bool SIGNED, int E, int L>
__device__ __forceinline__ uint64_t quantize_lane(const float (&x)[E],
                                                  const LdsMap<SIGNED ? BITS - 1 : BITS> &M, float &A) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    // max|x| of the lane, NaN ignored as the threshold rule ignores it (an
    // all-NaN lane counts as 0), then of the block
    float lm = fabsf(x[0]);
#pragma unroll
    for (int j = 1; j < E; ++j) lm = fmaxf(lm, fabsf(x[j]));
    const float mx = __uint_as_float(group_max<L>(lm == lm ? __float_as_uint(lm) : 0u));
    A = mx;
    const float r = mx > 0.0f ? recip_rn(mx) : 0.0f;
    uint64_t out = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        uint32_t c = code_index<MB>(M, fabsf(x[j]) * r);
        if (SIGNED) c |= (x[j] < 0.0f && c > 0) ? (1u << MB) : 0u;
        out |= (uint64_t)c << (j * BITS);
    }
    return out;
}

// x = fl32(+-vals[idx] * A): the table holds the signed value of a signed
// code, and (-v) * A = -(v * A) exactly.
template <int BITS, bool SIGNED, int E>
__device__ __forceinline__ void dequantize_lane(uint64_t codes, float A,
                                                const LdsMap<SIGNED ? BITS - 1 : BITS> &M, float (&x)[E]) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint32_t c = (uint32_t)(codes >> (j * BITS)) & ((1u << BITS) - 1u);
        x[j] = M.vals[c] * A;
    }
}

// Packed codes of elements [e, e + E) (e a multiple of E, so this lane owns
// whole bytes).  Full: one access of E*BITS bits (64, 32 or 16).  A 16-bit
// run per lane (4-bit codes, E = 4) makes 128-byte wave accesses, which
// measured faster with ordinary than with non-temporal loads and stores on
// MI355X (4-bit step -4%); 32-bit runs keep the row's access kind.
template <int BITS, int E>
constexpr int code_layout() { return E * BITS >= 32 ? row_layout<E>() : kRun; }

template <int BITS, int E>
__device__ __forceinline__ uint64_t load_codes_full(const uint8_t *q, int64_t e) {
    constexpr int LAY = code_layout<BITS, E>();
    const int64_t byte0 = e * BITS / 8;
    if constexpr (E * BITS == 64) {
        const u32x2 w = vload<LAY>((const GMEM u32x2 *)gp(q + byte0));
        return (uint64_t)w.x | ((uint64_t)w.y << 32);
    } else if constexpr (E * BITS == 32) {
        return vload<LAY>((const GMEM uint32_t *)gp(q + byte0));
    } else {
        static_assert(E * BITS == 16, "code run");
        return vload<LAY>((const GMEM uint16_t *)gp(q + byte0));
    }
}

template <int BITS, int E>
__device__ __forceinline__ void store_codes_full(uint8_t *q, int64_t e, uint64_t c) {
    constexpr int LAY = code_layout<BITS, E>();
    const int64_t byte0 = e * BITS / 8;
    if constexpr (E * BITS == 64)
        vstore<LAY>((GMEM u32x2 *)gp(q + byte0), u32x2{(uint32_t)c, (uint32_t)(c >> 32)});
    else if constexpr (E * BITS == 32)
        vstore<LAY>((GMEM uint32_t *)gp(q + byte0), (uint32_t)c);
    else
        vstore<LAY>((GMEM uint16_t *)gp(q + byte0), (uint16_t)c);
}

// Tail: nv < E valid elements, byte by byte; a half byte beyond the tensor
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

// Interleaved layout: element j's m and v codes are one field of 2*BITS
// bits (m in the low BITS), fields in element order; a lane's E elements
// are E*BITS/4 bytes.  split / join convert to and from the per-state
// packing above (element j in bits [j*BITS, (j+1)*BITS) of cm and cv).
template <int BITS, int E>
__device__ __forceinline__ void split_il(uint64_t raw, uint64_t &cm, uint64_t &cv) {
    constexpr uint64_t mask = (1ull << BITS) - 1ull;
    cm = 0;
    cv = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint64_t f = raw >> (j * 2 * BITS);
        cm |= (f & mask) << (j * BITS);
        cv |= ((f >> BITS) & mask) << (j * BITS);
    }
}

template <int BITS, int E>
__device__ __forceinline__ uint64_t join_il(uint64_t cm, uint64_t cv) {
    constexpr uint64_t mask = (1ull << BITS) - 1ull;
    uint64_t raw = 0;
#pragma unroll
    for (int j = 0; j < E; ++j)
        raw |= (((cm >> (j * BITS)) & mask) | (((cv >> (j * BITS)) & mask) << BITS)) << (j * 2 * BITS);
    return raw;
}

// Whole lanes: one 32- or 64-bit access of the lane's fields, in the row's
// access kind.
template <int BITS, int E>
__device__ __forceinline__ uint64_t load_il_full(const uint8_t *q, int64_t e) {
    constexpr int NB = E * BITS / 4;
    constexpr int LAY = row_layout<E>();
    const int64_t byte0 = e * BITS / 4;
    if constexpr (NB == 8) {
        const u32x2 w = vload<LAY>((const GMEM u32x2 *)gp(q + byte0));
        return (uint64_t)w.x | ((uint64_t)w.y << 32);
    } else {
        static_assert(NB == 4, "interleaved run");
        return vload<LAY>((const GMEM uint32_t *)gp(q + byte0));
    }
}

template <int BITS, int E>
__device__ __forceinline__ void store_il_full(uint8_t *q, int64_t e, uint64_t raw) {
    constexpr int NB = E * BITS / 4;
    constexpr int LAY = row_layout<E>();
    const int64_t byte0 = e * BITS / 4;
    if constexpr (NB == 8)
        vstore<LAY>((GMEM u32x2 *)gp(q + byte0), u32x2{(uint32_t)raw, (uint32_t)(raw >> 32)});
    else
        vstore<LAY>((GMEM uint32_t *)gp(q + byte0), (uint32_t)raw);
}

// Tail: the fields of nv < E valid elements, byte by byte (a field is whole
// bytes: 2 for 8-bit codes, 1 for 4-bit).
template <int BITS>
__device__ __forceinline__ uint64_t load_il_part(const uint8_t *q, int64_t e, int nv) {
    const int64_t byte0 = e * BITS / 4;
    uint64_t out = 0;
    for (int b = 0; b < nv * BITS / 4; ++b) out |= (uint64_t)gp(q)[byte0 + b] << (8 * b);
    return out;
}

template <int BITS>
__device__ __forceinline__ void store_il_part(uint8_t *q, int64_t e, int nv, uint64_t raw) {
    const int64_t byte0 = e * BITS / 4;
    for (int b = 0; b < nv * BITS / 4; ++b) gp(q)[byte0 + b] = (uint8_t)(raw >> (8 * b));
}

// One unit's arrays, offset to the unit's first element (a multiple of the
// tile, hence of the quantization block and of 8 elements) and kept in scalar
// registers: the tensor descriptor is read once per unit, not once per row.
struct UnitPtrs {
    float *p;
    const void *g;
    uint8_t *qm, *qv, *qm2;
    float *am, *av, *am2;
    float lw;  // fl32(lr wd)
    int lane;
};

// IL: interleaved layout, qm / am hold both states (qv, av unused).
template <int GK, int BITS, int BLOCK, bool ADE, bool IL>
__device__ __forceinline__ UnitPtrs unit_ptrs(const TensorDesc &T, int64_t start, float lw) {
    UnitPtrs u;
    u.p = uniform_ptr(static_cast<float *>(T.p) + start);
    u.g = uniform_ptr(static_cast<const char *>(T.g) + start * (GK == G_F32 ? 4 : 2));
    if (IL) {
        u.qm = uniform_ptr(T.qm + start * BITS / 4);
        u.am = uniform_ptr(T.am + 2 * (start / BLOCK));
        u.qv = nullptr;
        u.av = nullptr;
    } else {
        u.qm = uniform_ptr(T.qm + start * BITS / 8);
        u.qv = uniform_ptr(T.qv + start * BITS / 8);
        u.am = uniform_ptr(T.am + start / BLOCK);
        u.av = uniform_ptr(T.av + start / BLOCK);
    }
    if (ADE) {
        u.qm2 = uniform_ptr(T.qm2 + start * BITS / 8);
        u.am2 = uniform_ptr(T.am2 + start / BLOCK);
    }
    u.lw = lw;
    u.lane = threadIdx.x & 63;
    return u;
}

// One row of 256*E elements, this lane's E elements from element e of the
// unit: its inputs, loaded ahead of the row's arithmetic.
template <int E>
struct RowIn {
    float p[E], g[E];
    uint64_t cm, cv, cm2;
    float am, av, am2;
};

// FULL: the whole row is inside the tensor and every pointer is aligned;
// otherwise nv (0..E) of the lane's elements are valid and the rest read 0.
template <int GK, int BITS, int BLOCK, bool ADE, bool FULL, bool IL>
__device__ __forceinline__ void load_row(const UnitPtrs &u, const AdamK &k, uint32_t e, int nv,
                                         RowIn<lane_elems(BLOCK)> &in) {
    constexpr int E = lane_elems(BLOCK);
    constexpr int LAY = row_layout<E>();
    const uint32_t blk = e / BLOCK;
    in.am = in.av = in.am2 = 0.0f;
    in.cm = in.cv = in.cm2 = 0;
    if (FULL || nv > 0) {
        if constexpr (IL) {
            const u32x2 w = gp(reinterpret_cast<const u32x2 *>(u.am))[blk];
            in.am = __uint_as_float(w.x);
            in.av = __uint_as_float(w.y);
        } else {
            in.am = gp(u.am)[blk];
            in.av = gp(u.av)[blk];
            if (ADE) in.am2 = gp(u.am2)[blk];
        }
    }
    if (FULL) {
        ldf<E, LAY>(u.p, e, in.p);
        load_g<GK, E, LAY>(u.g, e, k.inv_scale, in.g);
        if constexpr (IL) {
            split_il<BITS, E>(load_il_full<BITS, E>(u.qm, e), in.cm, in.cv);
        } else {
            in.cm = load_codes_full<BITS, E>(u.qm, e);
            in.cv = load_codes_full<BITS, E>(u.qv, e);
            if (ADE) in.cm2 = load_codes_full<BITS, E>(u.qm2, e);
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            float pj[1] = {0.0f}, gj[1] = {0.0f};
            if (j < nv) {
                ldf<1>(u.p, e + j, pj);
                load_g<GK, 1>(u.g, e + j, k.inv_scale, gj);
            }
            in.p[j] = pj[0];
            in.g[j] = gj[0];
        }
        if (nv > 0) {
            if constexpr (IL) {
                split_il<BITS, E>(load_il_part<BITS>(u.qm, e, nv), in.cm, in.cv);
            } else {
                in.cm = load_codes_part<BITS>(u.qm, e, nv);
                in.cv = load_codes_part<BITS>(u.qv, e, nv);
                if (ADE) in.cm2 = load_codes_part<BITS>(u.qm2, e, nv);
            }
        }
    }
}

// ADE: AdEMAMix's third state m2 (signed map) and update
// p <- p (1 - lr wd) - lr (m/bc1 + alpha m2) / h.
template <int GK, int BITS, int BLOCK, bool ADE, bool FULL, bool IL>
__device__ __forceinline__ void step_row(const UnitPtrs &u, const AdamK &k, uint32_t e, int nv,
                                         RowIn<lane_elems(BLOCK)> &in, const LdsMap<BITS - 1> &Mm,
                                         const LdsMap<BITS> &Mv) {
    constexpr int E = lane_elems(BLOCK), L = BLOCK / E;
    constexpr int LAY = row_layout<E>();
    float mt[E], vt[E], m2t[E];
    dequantize_lane<BITS, true, E>(in.cm, in.am, Mm, mt);
    dequantize_lane<BITS, false, E>(in.cv, in.av, Mv, vt);
    if (ADE) dequantize_lane<BITS, true, E>(in.cm2, in.am2, Mm, m2t);
    // fp32 state recipe, every product and sum rounded on its own; outside
    // the tensor g = 0 and the codes are 0, so the new states are 0 there
    float mn[E], vn[E], m2n[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        mn[j] = k.b1 * mt[j] + k.c1 * in.g[j];
        vn[j] = k.b2 * vt[j] + k.c2 * (in.g[j] * in.g[j]);
        // parameter update: hardware sqrt / reciprocal (1 ulp each)
        const float h = __builtin_amdgcn_sqrtf(vn[j]) * k.isb2 + k.eps;
        if (ADE) {
            m2n[j] = k.b3 * m2t[j] + k.c3 * in.g[j];
            in.p[j] = decayed(in.p[j], u.lw, k.lr * ((mn[j] * k.ibc1 + k.alpha * m2n[j]) * __builtin_amdgcn_rcpf(h)));
        } else {
            in.p[j] = decayed(in.p[j], u.lw, k.ss * (mn[j] * __builtin_amdgcn_rcpf(h)));
        }
    }
    float am2, av2, am22 = 0.0f;
    const uint64_t om = quantize_lane<BITS, true, E, L>(mn, Mm, am2);
    const uint64_t ov = quantize_lane<BITS, false, E, L>(vn, Mv, av2);
    uint64_t om2 = 0;
    if (ADE) om2 = quantize_lane<BITS, true, E, L>(m2n, Mm, am22);
    if (FULL) {
        stf<E, LAY>(u.p, e, in.p);
        if constexpr (IL) {
            store_il_full<BITS, E>(u.qm, e, join_il<BITS, E>(om, ov));
        } else {
            store_codes_full<BITS, E>(u.qm, e, om);
            store_codes_full<BITS, E>(u.qv, e, ov);
            if (ADE) store_codes_full<BITS, E>(u.qm2, e, om2);
        }
    } else if (nv > 0) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float pj[1] = {in.p[j]};
            if (j < nv) stf<1>(u.p, e + j, pj);
        }
        if constexpr (IL) {
            store_il_part<BITS>(u.qm, e, nv, join_il<BITS, E>(om, ov));
        } else {
            store_codes_part<BITS>(u.qm, e, nv, om);
            store_codes_part<BITS>(u.qv, e, nv, ov);
            if (ADE) store_codes_part<BITS>(u.qm2, e, nv, om2);
        }
    }
    // every lane of a block holds the block's absmax: all of them store it
    // (one line per wave instruction, no branch around the store)
    if (FULL || nv > 0) {
        const uint32_t blk = e / BLOCK;
        if constexpr (IL) {
            gp(reinterpret_cast<u32x2 *>(u.am))[blk] = u32x2{__float_as_uint(am2), __float_as_uint(av2)};
        } else {
            gp(u.am)[blk] = am2;
            gp(u.av)[blk] = av2;
            if (ADE) gp(u.am2)[blk] = am22;
        }
    }
}

template <int GK, int BITS, int BLOCK, bool ADE, bool IL>
__global__ __launch_bounds__(kThreads) void blockwise_kernel(StepArgs a) {
    static_assert(!(ADE && IL), "the interleaved layout holds two states");
    constexpr int E = lane_elems(BLOCK);
    constexpr uint32_t kRow = (uint32_t)kThreads * E;
    __shared__ LdsMap<BITS - 1> Mm;
    __shared__ LdsMap<BITS> Mv;
    load_map(Mm, BITS == 8 ? a.codebook->m8 : a.codebook->m4);
    load_map(Mv, BITS == 8 ? a.codebook->v8 : a.codebook->v4);
    __shared__ Scalars S;
    step_begin(a, S);  // its barriers also publish the maps
    const StepCommit commit{a, S};
    if (S.skip) return;
    const AdamK k = adam_consts(S);
    for_units(a, [&](int64_t, const SpanDesc &sp, int64_t start, int64_t len64) {
        const TensorDesc &T = a.tensors[sp.tensor];
        const UnitPtrs u = unit_ptrs<GK, BITS, BLOCK, ADE, IL>(T, start, uniform(S.lrwd[T.group]));
        const uint32_t len = (uint32_t)len64;  // <= tile <= 2^24
        const uint32_t lane0 = threadIdx.x * E;
        // full rows, software-pipelined: the loads of the next rows are in
        // flight while a row computes -- two rows ahead for the 2-state step
        // with 4 elements per lane (measured on MI355X: 4-bit -2%), one with
        // AdEMAMix's third state or 8 elements per lane, whose extra
        // registers would cost occupancy
        const uint32_t nfull = T.vec_ok ? len / kRow : 0;
        const auto load_at = [&](uint32_t r, RowIn<E> &in) {
            load_row<GK, BITS, BLOCK, ADE, true, IL>(u, k, lane0 + r * kRow, E, in);
        };
        const auto step_at = [&](uint32_t r, RowIn<E> &in) {
            step_row<GK, BITS, BLOCK, ADE, true, IL>(u, k, lane0 + r * kRow, E, in, Mm, Mv);
        };
        uint32_t r = 0;
        if (!ADE && E == 4 && nfull > 1) {
            RowIn<E> cur, nxt;
            load_at(0, cur);
            load_at(1, nxt);
            for (; r + 2 < nfull; ++r) {
                RowIn<E> nn;
                load_at(r + 2, nn);
                step_at(r, cur);
                cur = nxt;
                nxt = nn;
            }
            step_at(r, cur);
            step_at(r + 1, nxt);
        } else if (nfull > 0) {
            RowIn<E> cur;
            load_at(0, cur);
            for (; r + 1 < nfull; ++r) {
                RowIn<E> nxt;
                load_at(r + 1, nxt);
                step_at(r, cur);
                cur = nxt;
            }
            step_at(r, cur);
        }
        for (uint32_t r0 = nfull * kRow; r0 < len; r0 += kRow) {
            const uint32_t rel = r0 + lane0;
            const int nv = rel + E <= len ? E : (rel < len ? (int)(len - rel) : 0);
            RowIn<E> in;
            load_row<GK, BITS, BLOCK, ADE, false, IL>(u, k, rel, nv, in);
            step_row<GK, BITS, BLOCK, ADE, false, IL>(u, k, rel, nv, in, Mm, Mv);
        }
    });
}

// Blockwise quantize / dequantize of a plain fp32 array with the same code
// path as the step (state import and export).  Rows of 256*E elements,
// grid-stride; the loop trip count is uniform per workgroup.
template <int BITS, bool SIGNED, int BLOCK>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const Codebook *cb, const float *x, int64_t n, bool vec,
                                                           uint8_t *codes, float *absmax) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    constexpr int E = lane_elems(BLOCK), L = BLOCK / E;
    constexpr int LAY = row_layout<E>();
    constexpr int64_t kRow = (int64_t)kThreads * E;
    __shared__ LdsMap<MB> M;
    load_map(M, BITS == 8 ? (SIGNED ? cb->m8 : cb->v8) : (SIGNED ? cb->m4 : cb->v4));
    __syncthreads();
    const int64_t nrows = (n + kRow - 1) / kRow;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t e = row * kRow + threadIdx.x * E;
        const int nv = n - e >= E ? E : (n - e > 0 ? (int)(n - e) : 0);
        const bool full = vec && nv == E;
        float v[E];
        if (full) {
            ldf<E, LAY>(x, e, v);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                float vj[1] = {0.0f};
                if (j < nv) ldf<1>(x, e + j, vj);
                v[j] = vj[0];
            }
        }
        float A;
        const uint64_t c = quantize_lane<BITS, SIGNED, E, L>(v, M, A);
        if (full)
            store_codes_full<BITS, E>(codes, e, c);
        else if (nv > 0)
            store_codes_part<BITS>(codes, e, nv, c);
        if (nv > 0 && (threadIdx.x & (L - 1)) == 0) gp(absmax)[e / BLOCK] = A;
    }
}

template <int BITS, bool SIGNED, int BLOCK>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const Codebook *cb, const uint8_t *codes,
                                                             const float *absmax, int64_t n, bool vec, float *x) {
    constexpr int MB = SIGNED ? BITS - 1 : BITS;
    constexpr int E = lane_elems(BLOCK);
    constexpr int LAY = row_layout<E>();
    constexpr int64_t kRow = (int64_t)kThreads * E;
    __shared__ LdsMap<MB> M;
    load_map(M, BITS == 8 ? (SIGNED ? cb->m8 : cb->v8) : (SIGNED ? cb->m4 : cb->v4));
    __syncthreads();
    const int64_t nrows = (n + kRow - 1) / kRow;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t e = row * kRow + threadIdx.x * E;
        const int nv = n - e >= E ? E : (n - e > 0 ? (int)(n - e) : 0);
        if (nv == 0) continue;
        const bool full = vec && nv == E;
        float v[E];
        const uint64_t c = full ? load_codes_full<BITS, E>(codes, e) : load_codes_part<BITS>(codes, e, nv);
        dequantize_lane<BITS, SIGNED, E>(c, gp(absmax)[e / BLOCK], M, v);
        if (full) {
            stf<E, LAY>(x, e, v);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float vj[1] = {v[j]};
                if (j < nv) stf<1>(x, e + j, vj);
            }
        }
    }
}

// (bits, block) -> compile-time block size; the plan admits 8-bit blocks of
// 64, 128, 256 and 4-bit blocks of 128, 256, 512.
template <class F>
hipError_t with_block(int bits, int block, F &&f) {
    if (bits == 8) {
        if (block == 64) return f(std::integral_constant<int, 8>{}, std::integral_constant<int, 64>{});
        if (block == 128) return f(std::integral_constant<int, 8>{}, std::integral_constant<int, 128>{});
        if (block == 256) return f(std::integral_constant<int, 8>{}, std::integral_constant<int, 256>{});
    } else if (bits == 4) {
        if (block == 128) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 128>{});
        if (block == 256) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 256>{});
        if (block == 512) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 512>{});
    }
    return hipErrorInvalidValue;
}

int quant_grid(int64_t n, int E) {
    const int64_t rows = (n + (int64_t)kThreads * E - 1) / ((int64_t)kThreads * E);
    return (int)(rows < 16384 ? (rows > 0 ? rows : 1) : 16384);
}

}  // namespace

hipError_t launch_blockwise(const StepArgs &a, int gk, bool ademamix, hipStream_t s) {
    return with_block(a.bits, a.block, [&](auto bits, auto block) {
        constexpr int B = decltype(bits)::value, K = decltype(block)::value;
        const bool il = a.interleaved != 0;
        if (ademamix && il) return hipErrorInvalidValue;
        if (gk == G_F32 && !ademamix && il)
            LAUNCH_PERSISTENT((blockwise_kernel<G_F32, B, K, false, true>), a, s);
        else if (!ademamix && il)
            LAUNCH_PERSISTENT((blockwise_kernel<G_BF16, B, K, false, true>), a, s);
        else if (gk == G_F32 && !ademamix)
            LAUNCH_PERSISTENT((blockwise_kernel<G_F32, B, K, false, false>), a, s);
        else if (!ademamix)
            LAUNCH_PERSISTENT((blockwise_kernel<G_BF16, B, K, false, false>), a, s);
        else if (gk == G_F32)
            LAUNCH_PERSISTENT((blockwise_kernel<G_F32, B, K, true, false>), a, s);
        else
            LAUNCH_PERSISTENT((blockwise_kernel<G_BF16, B, K, true, false>), a, s);
        return hipGetLastError();
    });
}

hipError_t launch_quantize(const Codebook *cb, int bits, int block, int is_signed, const float *x,
                           int64_t n, uint8_t *codes, float *absmax, hipStream_t s) {
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 8 == 0);
    return with_block(bits, block, [&](auto b, auto k) {
        constexpr int B = decltype(b)::value, K = decltype(k)::value;
        const dim3 grid(quant_grid(n, lane_elems(K)));
        if (is_signed)
            hipLaunchKernelGGL((quantize_kernel<B, true, K>), grid, dim3(kThreads), 0, s, cb, x, n, vec, codes, absmax);
        else
            hipLaunchKernelGGL((quantize_kernel<B, false, K>), grid, dim3(kThreads), 0, s, cb, x, n, vec, codes, absmax);
        return hipGetLastError();
    });
}

hipError_t launch_dequantize(const Codebook *cb, int bits, int block, int is_signed, const uint8_t *codes,
                             const float *absmax, int64_t n, float *x, hipStream_t s) {
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)codes % 8 == 0);
    return with_block(bits, block, [&](auto b, auto k) {
        constexpr int B = decltype(b)::value, K = decltype(k)::value;
        const dim3 grid(quant_grid(n, lane_elems(K)));
        if (is_signed)
            hipLaunchKernelGGL((dequantize_kernel<B, true, K>), grid, dim3(kThreads), 0, s, cb, codes, absmax, n, vec, x);
        else
            hipLaunchKernelGGL((dequantize_kernel<B, false, K>), grid, dim3(kThreads), 0, s, cb, codes, absmax, n, vec, x);
        return hipGetLastError();
    });
}

}  // namespace optim
