// stream_probe.hip -- access-pattern ceilings for the optimizer step
// kernels on MI355X (gfx950).  Benchmark-only: not part of the C ABI of
// liboptim_step.so and never called by it.
//
// Each probe moves exactly the bytes of one step kernel, in that kernel's
// lane layout, unit size and access kind, and does no arithmetic: what it
// stores is a bit permutation of what it loaded (so no load can be
// dropped), without the per-step prologue, the commit or any math.  Its
// bandwidth is what the access pattern alone sustains on this part -- the
// ceiling the kernel's own bandwidth is compared against.
//
// Patterns (fp32 unless noted; R = read, W = written in place):
//  adamw      R p g m v,  W p m v     4 elements per lane per group, G groups
//                                     per lane, one workgroup per G*1024
//                                     elements, non-temporal accesses
//  ademamix   R p g m v m2, W p m v m2  as adamw
//  bf16r      R p r g (16-bit) m v, W p r (16-bit) m v   as adamw; or with
//             m and v in one array, in blocks of 1024 elements (m, then v)
//  mini       R p g m,  W p m         as adamw (the Adam-mini update's
//                                     HBM pattern when g comes from HBM)
//  blockwise  rows of 1024 elements, 4 per lane: R p g (16 B a lane),
//             codes qm qv (BITS*4 bits a lane), absmax am av (one float per
//             block, read by every lane of it); W p qm qv am av; 8 rows per
//             workgroup, R rows of loads in flight
//  read       R one fp32 or 16-bit stream, 8 groups of 4 per lane in flight,
//             32768 elements per workgroup (the non-finite check, the
//             block-sum pass)
//  write      W one fp32 stream (8 groups of 4 per lane; non-temporal or ordinary)
//  copy       R x, W y (ordinary accesses, 4 per lane, 1024 per workgroup)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef float __attribute__((ext_vector_type(4))) f32x4;
typedef uint32_t __attribute__((ext_vector_type(4))) u32x4;
typedef uint32_t __attribute__((ext_vector_type(2))) u32x2;
#define GMEM __attribute__((address_space(1)))

template <class V>
__device__ __forceinline__ V ntl(const V *p) { return __builtin_nontemporal_load((const GMEM V *)p); }
template <class V>
__device__ __forceinline__ void nts(V *p, V x) { __builtin_nontemporal_store(x, (GMEM V *)p); }

__device__ __forceinline__ u32x4 bits(f32x4 x) { return __builtin_bit_cast(u32x4, x); }
__device__ __forceinline__ f32x4 flt(u32x4 x) { return __builtin_bit_cast(f32x4, x); }

// lane t owns elements 4t..4t+3 of each group of 1024; group j at +j*1024.
// Accesses go array by array (all G groups of p, then of g, ...), in the
// order the step kernels issue them (one array's groups 4 KiB apart, back
// to back; measured on MI355X 1-2% faster than group by group).
template <int G, int NS>
__global__ __launch_bounds__(kThreads) void fp32_pattern(float *p, const float *g, float *m, float *v, float *m2) {
    const int64_t e = (int64_t)blockIdx.x * (G * 1024) + threadIdx.x * 4;
    u32x4 P[G], Gr[G], M[G], V[G], M2[G];
#pragma unroll
    for (int j = 0; j < G; ++j) P[j] = bits(ntl((const f32x4 *)(p + e + j * 1024)));
#pragma unroll
    for (int j = 0; j < G; ++j) Gr[j] = bits(ntl((const f32x4 *)(g + e + j * 1024)));
#pragma unroll
    for (int j = 0; j < G; ++j) M[j] = bits(ntl((const f32x4 *)(m + e + j * 1024)));
    if (NS >= 4) {
#pragma unroll
        for (int j = 0; j < G; ++j) V[j] = bits(ntl((const f32x4 *)(v + e + j * 1024)));
    }
    if (NS >= 5) {
#pragma unroll
        for (int j = 0; j < G; ++j) M2[j] = bits(ntl((const f32x4 *)(m2 + e + j * 1024)));
    }
#pragma unroll
    for (int j = 0; j < G; ++j) nts((f32x4 *)(p + e + j * 1024), flt(P[j] ^ Gr[j]));
    if (NS >= 4) {
#pragma unroll
        for (int j = 0; j < G; ++j) nts((f32x4 *)(m + e + j * 1024), flt(V[j]));
#pragma unroll
        for (int j = 0; j < G; ++j) nts((f32x4 *)(v + e + j * 1024), flt(M[j]));
    } else {
#pragma unroll
        for (int j = 0; j < G; ++j) nts((f32x4 *)(m + e + j * 1024), flt(M[j] ^ Gr[j]));
    }
    if (NS >= 5) {
#pragma unroll
        for (int j = 0; j < G; ++j) nts((f32x4 *)(m2 + e + j * 1024), flt(M2[j] ^ Gr[j]));
    }
}

// bf16 param + int16 remainder + bf16 grad (4 x 16 bits a lane per group) and fp32 m, v;
// IL: m and v interleaved in m, block b (1024 elements) holding m then v
template <int G, bool IL>
__global__ __launch_bounds__(kThreads) void bf16r_pattern(uint16_t *p, uint16_t *r, const uint16_t *g, float *mm,
                                                          float *vv) {
    const int64_t e = (int64_t)blockIdx.x * (G * 1024) + threadIdx.x * 4;
    // IL: element e's m at 2e - e mod 1024, its v 1024 further; a lane's
    // groups (1024 elements apart) are two blocks apart
    float *m = IL ? mm + (2 * e - (e & 1023)) : mm;
    float *v = IL ? m + 1024 : vv;
    const int64_t ms = IL ? 2048 : 1024;  // distance between a lane's groups in m and v
    const int64_t me = IL ? 0 : e;
    u32x2 P[G], R[G], Gr[G];
    u32x4 M[G], V[G];
    // array by array, as fp32_pattern
#pragma unroll
    for (int j = 0; j < G; ++j) P[j] = ntl((const u32x2 *)(p + e + j * 1024));
#pragma unroll
    for (int j = 0; j < G; ++j) R[j] = ntl((const u32x2 *)(r + e + j * 1024));
#pragma unroll
    for (int j = 0; j < G; ++j) Gr[j] = ntl((const u32x2 *)(g + e + j * 1024));
#pragma unroll
    for (int j = 0; j < G; ++j) M[j] = bits(ntl((const f32x4 *)(m + me + j * ms)));
#pragma unroll
    for (int j = 0; j < G; ++j) V[j] = bits(ntl((const f32x4 *)(v + me + j * ms)));
#pragma unroll
    for (int j = 0; j < G; ++j) nts((u32x2 *)(p + e + j * 1024), R[j] ^ Gr[j]);
#pragma unroll
    for (int j = 0; j < G; ++j) nts((u32x2 *)(r + e + j * 1024), P[j]);
#pragma unroll
    for (int j = 0; j < G; ++j) nts((f32x4 *)(m + me + j * ms), flt(V[j]));
#pragma unroll
    for (int j = 0; j < G; ++j) nts((f32x4 *)(v + me + j * ms), flt(M[j]));
}

// blockwise 2-state step, separate layout, 4 elements a lane per row of
// 1024; one workgroup per unit of ROWS rows (the step's unit: 4096 elements
// for 8-bit codes, 8192 for 4-bit); R rows in flight
template <int BITS, int BLOCK, int R, int ROWS>
__global__ __launch_bounds__(kThreads) void blockwise_pattern(float *p, const float *g, uint8_t *qm, uint8_t *qv,
                                                              float *am, float *av) {
    constexpr int kRows = ROWS;
    static_assert(kRows % R == 0, "whole batches of rows");
    const int64_t base = (int64_t)blockIdx.x * (kRows * 1024);
#pragma unroll
    for (int r0 = 0; r0 < kRows; r0 += R) {
        u32x4 P[R], Gr[R];
        uint32_t CM[R], CV[R];
        float AM[R], AV[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t e = base + (int64_t)(r0 + j) * 1024 + threadIdx.x * 4;
            P[j] = bits(ntl((const f32x4 *)(p + e)));
            Gr[j] = bits(ntl((const f32x4 *)(g + e)));
            if constexpr (BITS == 8) {
                CM[j] = ntl((const uint32_t *)(qm + e));
                CV[j] = ntl((const uint32_t *)(qv + e));
            } else {
                CM[j] = *(const GMEM uint16_t *)(qm + e / 2);
                CV[j] = *(const GMEM uint16_t *)(qv + e / 2);
            }
            AM[j] = *(const GMEM float *)(am + e / BLOCK);
            AV[j] = *(const GMEM float *)(av + e / BLOCK);
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t e = base + (int64_t)(r0 + j) * 1024 + threadIdx.x * 4;
            nts((f32x4 *)(p + e), flt(P[j] ^ Gr[j]));
            if constexpr (BITS == 8) {
                nts((uint32_t *)(qm + e), CV[j]);
                nts((uint32_t *)(qv + e), CM[j]);
            } else {
                *(GMEM uint16_t *)(qm + e / 2) = (uint16_t)CV[j];
                *(GMEM uint16_t *)(qv + e / 2) = (uint16_t)CM[j];
            }
            *(GMEM float *)(am + e / BLOCK) = AV[j];
            *(GMEM float *)(av + e / BLOCK) = AM[j];
        }
    }
}

// read-only: 8 groups of 4 per lane in flight, 32768 elements per workgroup;
// the OR of all words is stored once per workgroup so no load is dropped
template <int EB>
__global__ __launch_bounds__(kThreads) void read_pattern(const uint8_t *x, uint32_t *sink) {
    constexpr int64_t kPer = 32768;
    const int64_t e0 = (int64_t)blockIdx.x * kPer + threadIdx.x * 4;
    uint32_t acc = 0;
    for (int64_t s = 0; s < kPer; s += 8 * 1024) {
        if constexpr (EB == 4) {
            u32x4 w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = ntl((const u32x4 *)(x + 4 * (e0 + s + j * 1024)));
#pragma unroll
            for (int j = 0; j < 8; ++j) acc |= w[j].x | w[j].y | w[j].z | w[j].w;
        } else {
            u32x2 w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = ntl((const u32x2 *)(x + 2 * (e0 + s + j * 1024)));
#pragma unroll
            for (int j = 0; j < 8; ++j) acc |= w[j].x | w[j].y;
        }
    }
    if (acc == 0x12345678u) sink[blockIdx.x] = acc;  // practically never taken, not provable
}

// W one fp32 stream, 8 groups of 4 per lane (8192 elements per workgroup),
// non-temporal stores (as the step kernels store) or ordinary ones
template <bool NT>
__global__ __launch_bounds__(kThreads) void write_pattern(float *y) {
    const int64_t e0 = (int64_t)blockIdx.x * 8192 + threadIdx.x * 4;
    const float b = (float)blockIdx.x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const f32x4 x{b, b, b, (float)j};
        if (NT) nts((f32x4 *)(y + e0 + j * 1024), x);
        else *(GMEM f32x4 *)(y + e0 + j * 1024) = x;
    }
}

__global__ __launch_bounds__(kThreads) void copy_pattern(const float *x, float *y) {
    const int64_t e = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
    *(GMEM f32x4 *)(y + e) = *(const GMEM f32x4 *)(x + e);
}

int grid_of(int64_t n, int64_t per) { return (int)(n / per); }

}  // namespace

// Every probe takes arrays of n elements, n a multiple of its workgroup's
// elements (the caller checks: 32768 divides every size used here), and
// returns the launch's hipError_t.
extern "C" {

int probe_adamw(float *p, const float *g, float *m, float *v, int64_t n, int groups, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (groups == 4)
        hipLaunchKernelGGL((fp32_pattern<4, 4>), dim3(grid_of(n, 4096)), dim3(kThreads), 0, s, p, g, m, v, nullptr);
    else
        hipLaunchKernelGGL((fp32_pattern<2, 4>), dim3(grid_of(n, 2048)), dim3(kThreads), 0, s, p, g, m, v, nullptr);
    return (int)hipGetLastError();
}

int probe_ademamix(float *p, const float *g, float *m, float *v, float *m2, int64_t n, int groups, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (groups == 4)
        hipLaunchKernelGGL((fp32_pattern<4, 5>), dim3(grid_of(n, 4096)), dim3(kThreads), 0, s, p, g, m, v, m2);
    else
        hipLaunchKernelGGL((fp32_pattern<2, 5>), dim3(grid_of(n, 2048)), dim3(kThreads), 0, s, p, g, m, v, m2);
    return (int)hipGetLastError();
}

int probe_mini(float *p, const float *g, float *m, int64_t n, void *stream) {
    hipLaunchKernelGGL((fp32_pattern<4, 3>), dim3(grid_of(n, 4096)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), p, g, m, nullptr, nullptr);
    return (int)hipGetLastError();
}

// interleaved != 0: m holds 2n floats (m and v blocks), v is unused
int probe_bf16r(uint16_t *p, uint16_t *r, const uint16_t *g, float *m, float *v, int64_t n, int interleaved,
                void *stream) {
    if (n <= 0 || n % 2048 != 0) return -1;  // whole units only
    if (interleaved)
        hipLaunchKernelGGL((bf16r_pattern<2, true>), dim3(grid_of(n, 2048)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), p, r, g, m, v);
    else
        hipLaunchKernelGGL((bf16r_pattern<2, false>), dim3(grid_of(n, 2048)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), p, r, g, m, v);
    return (int)hipGetLastError();
}

int probe_blockwise(float *p, const float *g, uint8_t *qm, uint8_t *qv, float *am, float *av, int64_t n, int bits,
                    int unit_rows, int rows_in_flight, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n <= 0 || n % ((int64_t)unit_rows * 1024) != 0) return -1;  // whole units only
    const dim3 grid(grid_of(n, (int64_t)unit_rows * 1024));
    if (bits == 8 && unit_rows == 4 && rows_in_flight == 2)
        hipLaunchKernelGGL((blockwise_pattern<8, 256, 2, 4>), grid, dim3(kThreads), 0, s, p, g, qm, qv, am, av);
    else if (bits == 8 && unit_rows == 4 && rows_in_flight == 4)
        hipLaunchKernelGGL((blockwise_pattern<8, 256, 4, 4>), grid, dim3(kThreads), 0, s, p, g, qm, qv, am, av);
    else if (bits == 4 && unit_rows == 8 && rows_in_flight == 2)
        hipLaunchKernelGGL((blockwise_pattern<4, 128, 2, 8>), grid, dim3(kThreads), 0, s, p, g, qm, qv, am, av);
    else if (bits == 4 && unit_rows == 8 && rows_in_flight == 8)
        hipLaunchKernelGGL((blockwise_pattern<4, 128, 8, 8>), grid, dim3(kThreads), 0, s, p, g, qm, qv, am, av);
    else
        return -1;
    return (int)hipGetLastError();
}

int probe_read(const void *x, int64_t n, int elem_bytes, uint32_t *sink, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(grid_of(n, 32768));
    if (elem_bytes == 4)
        hipLaunchKernelGGL((read_pattern<4>), grid, dim3(kThreads), 0, s, static_cast<const uint8_t *>(x), sink);
    else
        hipLaunchKernelGGL((read_pattern<2>), grid, dim3(kThreads), 0, s, static_cast<const uint8_t *>(x), sink);
    return (int)hipGetLastError();
}

int probe_write(float *y, int64_t n, int nontemporal, void *stream) {
    if (n <= 0 || n % 8192 != 0) return -1;
    if (nontemporal)
        hipLaunchKernelGGL(write_pattern<true>, dim3(grid_of(n, 8192)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), y);
    else
        hipLaunchKernelGGL(write_pattern<false>, dim3(grid_of(n, 8192)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), y);
    return (int)hipGetLastError();
}

int probe_copy(const float *x, float *y, int64_t n, void *stream) {
    hipLaunchKernelGGL(copy_pattern, dim3(grid_of(n, 1024)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), x, y);
    return (int)hipGetLastError();
}

}  // extern "C"
