// plan.h -- device-visible plan tables shared by the C-ABI host layer
// (api.cpp) and the gfx950 kernels (kernels_*.hip).  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <deque>
#include <string>
#include <utility>
#include <vector>

namespace optim {

// Work decomposition: every tensor (Adam-mini: every shared-v block) is a
// "span"; a span is cut into units of `tile` consecutive elements (the last
// one ragged).  Units are numbered globally.  By default one workgroup runs
// per unit, so the hardware dispatcher keeps the resident workgroups on one
// narrow, advancing window of every array; a plan may instead ask for a
// persistent grid whose workgroups walk the units grid-stride.
constexpr int kThreads = 256;        // workgroup size (4 wavefronts of 64)
constexpr int64_t kDefaultTile = 2048;
// AdamW / AdEMAMix / Lion plans of more than 2^20 and at most 2^24 elements:
// units of 4096, which the step runs in its early-load form (see
// kernels_adam.hip)
constexpr int64_t kEarlyTile = 4096;
constexpr int64_t kEarlyTileMinElems = int64_t(1) << 20;
constexpr int64_t kEarlyTileMaxElems = int64_t(1) << 24;
constexpr int64_t kAdamMiniTile = 4096;   // also LAMB and the fp16 scaled-state step
// Adam-mini: gradient bytes per segment (a segment's g is read twice, the
// second time mostly from the 256 MB Infinity Cache).  Measured on MI355X,
// Llama-7B-shaped list: 28.1 ms per step in one pass over the list; with
// segments of 160 / 256 / 384 / 512 / 1024 MiB 27.3 / 26.5 / 25.8 / 26.0 /
// 26.8 ms (fewer, larger segments launch less often; past the cache's size
// less of g is found there).  With today's kernels, every size timed in one
// process on the same arrays: 256 / 320 / 384 / 448 / 512 MiB 25.18 /
// 24.95 / 24.88 / 24.99 / 25.06 ms.
constexpr int64_t kMiniSegmentBytes = (int64_t)384 << 20;
// blockwise units, measured best on MI355X over 2^28 elements (4096-16384,
// every size timed in one process on the same arrays, since where the
// driver places a fresh set of arrays moves the step by up to several
// percent): 8-bit separate layout 4096 (757 us against 766 at 8192),
// interleaved 8192 (729 against 751 at 4096), 4-bit 8192 either layout
// (632-634 against 678-684 at 4096 and 653-684 at 16384), AdEMAMix 8-bit
// 8192 (874 against 935 / 895), 4-bit 16384
constexpr int64_t blockwise_tile(bool ademamix, int bits, bool interleaved) {
    return ademamix ? (bits == 8 ? 8192 : 16384) : (bits == 8 && !interleaved) ? 4096 : 8192;
}
// read-only scans (finite check, gradient norm): elements per workgroup;
// measured on MI355X over a 1.1B bf16 gradient list: 8192 -> 5.3 TB/s,
// 32768 -> 6.2 (check) / 6.4 (check + norm), 65536 no better
constexpr int64_t kFiniteCheckElems = 32768;
constexpr int64_t kMinTile = 1024;   // one group of 4 elements per lane
constexpr int64_t kMinBlockwiseTile = 2048;  // one quantizer row: 256 lanes x 8 elements
// AdamW / AdEMAMix interleaved moment layout: blocks of this many elements
// (one group of 4 per lane of a workgroup), m then v (then m2) per block
constexpr int64_t kMomentBlock = 1024;
constexpr int kMaxGroups = 64;    // distinct weight-decay values per plan
constexpr int64_t kMaxNumel = int64_t(1) << 48;  // per tensor (byte sizes stay far from overflow)

// fp32; bf16 + int16 remainder; fp32 master + bf16 or fp16 model copy
enum ParamKind { P_F32 = 0, P_BF16R = 1, P_MBF16 = 2, P_MF16 = 3 };
enum GradKind { G_F32 = 0, G_BF16 = 1 };
// 16-bit scaled moments (same codes as the public state_dtype values)
enum StateKind { S_BF16 = 1, S_F16 = 2 };

struct TensorDesc {       // 152 bytes
    void *p;              // param (fp32 or bf16 patterns)
    const void *g;        // gradient
    float *m;             // first moment
    float *v;             // second moment (Adam-mini HEAD/SCALAR: per block)
    float *m2;            // AdEMAMix slow EMA
    uint16_t *rem;        // int16 remainder (as raw 16-bit patterns)
    uint8_t *qm, *qv;     // blockwise codes
    float *am, *av;       // blockwise absmax
    int64_t numel;
    int64_t block_len;    // Adam-mini shared-v block length (0 = full v)
    int32_t group;        // weight-decay group
    int32_t kind;         // Adam-mini partition
    int32_t vec_ok;       // every pointer 16-byte aligned
    int32_t pad_;
    uint8_t *qm2;         // blockwise AdEMAMix: codes of m2
    float *am2;           // blockwise AdEMAMix: absmax of m2
    float *master;        // fp32 master of a bf16 / fp16 model param (p)
    float *scale_m;       // 16-bit states: device scale of the stored m
    float *scale_v;       // 16-bit states: device scale of the stored v
};
static_assert(sizeof(TensorDesc) == 152, "TensorDesc layout");

// Packs (AdamW, AdEMAMix and Lion plans): a run of whole tensors of at most
// half a pack each (in list order, empty tensors left out), laid end to end
// as one unit of at most kPackElems elements (or the plan's unit, if
// smaller), each tensor's length rounded up to a multiple of 4.  A
// pack is one span whose tensor field is kPackTensor and whose elem_begin is
// the pack's index; its len is the rounded total.  Packs take the plan's
// last units, after every unit of a single tensor, and have kernels of
// their own (the step kernels of single tensors stay free of their registers
// and LDS).  Member j holds the pack's
// elements [off[j], off[j + 1]), off[j] = pack_off[off_base + j], off[0] = 0,
// off[k] = len; pack_td[td_base + j] is its PackMember record (the fields of
// its tensor descriptor the pack kernels read), so a workgroup loads a
// pack's tables with one contiguous copy into LDS.
constexpr int32_t kPackTensor = -2;
constexpr int32_t kMaxPackTensors = 64;  // members per pack (LDS: 64 descriptors, ~10 KB)
// Pack capacity: 2048 elements, two groups of 4 per lane.  A pack kernel's
// workgroup waits for its member tables before it can load, and per-lane
// member pointers cost registers (4-group packs: 143 VGPRs, 3 waves per
// SIMD; 2-group: 96, 5 waves), so smaller packs in more, leaner workgroups
// hide that wait better.  Measured on MI355X, 2^24 AdamW elements in one
// process on the same arrays (four state sets in turn), 4096- / 2048- /
// 1024-element packs: 65536 tensors of 256 89.6 / 84.5 / 84.5 us, 32768 of
// 512 87.7 / 83.1 / 82.8 us, 262144 of 64 98.5 / 88.4 / 90.6 us.
constexpr int64_t kPackElems = 2048;
// A pack member as the pack kernels see it: its arrays, length, weight-decay
// group and alignment (72 bytes, against 152 for the full TensorDesc; the
// tables are read from HBM once per step, so their size is traffic).
struct PackMember {
    void *p;
    const void *g;
    float *m;
    float *v;
    float *m2;
    uint16_t *rem;
    float *master;
    int32_t numel;        // at most kPackElems / 2
    int32_t group;
    int32_t vec_ok;
    int32_t pad_;
};
static_assert(sizeof(PackMember) == 72, "PackMember layout");
struct PackDesc {         // 16 bytes
    int32_t td_base;      // index of member 0 in pack_td
    int32_t off_base;     // index of off[0] in pack_off
    int32_t k;            // members
    int32_t len;          // elements including the rounding
};
static_assert(sizeof(PackDesc) == 16, "PackDesc layout");

struct SpanDesc {         // 32 bytes
    int64_t unit_begin;   // first global unit number of this span
    int64_t elem_begin;   // first element, relative to the tensor
    int64_t len;          // elements in the span
    int32_t tensor;       // index into the tensor table
    int32_t block;        // Adam-mini global block number, -1 for full v
};
static_assert(sizeof(SpanDesc) == 32, "SpanDesc layout");

// Per-step scalars.  Every workgroup of a step kernel derives them in its
// prologue (fp64, rounded once to fp32) into LDS from the device lr, step
// counter, found_inf and inv_scale.
struct Scalars {
    int32_t skip;         // non-zero: found_inf was set, write nothing
    int32_t t;            // applied-step count including this step
    float lr;
    float step_size;      // fl32(lr / (1 - beta1^t))
    float inv_sqrt_bc2;   // fl32(1 / sqrt(1 - beta2^t))
    float inv_bc1;        // fl32(1 / (1 - beta1^t))
    float b1, c1;         // fl32(beta1), fl32(1 - beta1)
    float b2, c2;
    float b3, c3;         // AdEMAMix
    float alpha;
    float eps;
    float inv_scale;      // gradient multiplier (AMP unscale), 1 if none
    int32_t k;            // schedule iteration read by this step
    double lr64, step_size64, inv_sqrt_bc2_64, eps64, beta2_64, c2_64;
    float lrwd[kMaxGroups];   // fl32(lr * wd_group)
};

// Commit counters: one top counter and kSubCounters sub-counters, each on its
// own 128-byte line, so arrivals of different workgroups spread over lines.
constexpr int kSubCounters = 32;
constexpr int kCounterStride = 32;  // uint32 words between counters
constexpr size_t kCounterBytes = (1 + kSubCounters) * kCounterStride * sizeof(uint32_t);
// fp16 scaled moments: per tensor and moment, the running maximum |x| of
// the step as fp32 bits, kept in kAmaxSlots words on separate lines (a
// workgroup's atomic max goes to one of them); 0 between steps.
constexpr int kAmaxSlots = 16;
constexpr size_t kAmaxBytesPerBlock = 2 * kAmaxSlots * kCounterStride * sizeof(uint32_t);

// Workspace layout (byte offsets from the workspace base, 256-aligned).
// `counters` holds the arrival counters of the step kernels' commit.
struct Layout {
    size_t counters, group_wd, tensors, spans, codebook, partials, blockfac,
        blockspan, packs, pack_off, pack_td, total;
};

// Quantization maps.  A normalised magnitude a in [0, 1] maps to the largest
// j with thr[j] <= a.  The search starts from a bucket table indexed by a's
// exponent and top kLutMantBits mantissa bits over [2^-26, 2): lut[bucket]
// is the index of the bucket's smallest value, and table construction
// checks that no bucket holds more than one threshold, so one comparison
// finishes the search.  Every threshold of every map is above 2^-26.
constexpr int kLutMantBits = 8;
constexpr int kLutBaseExp = 127 - 26;  // biased exponent of 2^-26
constexpr int kLutBinades = 27;        // 2^-26 ... [1, 2)
constexpr int kLutBuckets = kLutBinades << kLutMantBits;

struct QuantMap {
    float vals[256];       // sorted magnitudes (first 2^mb used)
    float thr[260];        // thr[j] = fl32((vals[j-1] + vals[j]) / 2), thr[0] = 0,
                           // thr[2^mb...] = +inf (ends the search)
    uint8_t lut[kLutBuckets];
};

struct Codebook {          // signed map for m, unsigned map for v
    QuantMap m8, v8, m4, v4;
};

struct PrepArgs {
    const double *group_wd;
    int32_t ngroups;
    int32_t sched;        // OPTIM_SCHED_*
    float *lr_dev;
    const float *inv_scale;
    const float *found_inf;
    int32_t *step_dev;
    int32_t *iter_dev;
    double lr_max, lr_min;
    int32_t K;
    double beta1, beta2, beta3, alpha, eps;
};

struct StepArgs {
    PrepArgs prep;            // inputs of the per-step scalars
    uint32_t *done;           // arrival counters (workspace), 0 between steps
    int32_t commit;           // this kernel publishes step / lr / iteration
    const TensorDesc *tensors;
    const SpanDesc *spans;    // nspans + 1 entries (sentinel at the end)
    int32_t nspans;
    int64_t unit0;            // this launch covers units [unit0, nunits)
    int64_t nunits;
    int64_t tile;             // elements per unit
    double *partials;         // Adam-mini: one per unit; LAMB: two per unit;
                              // gradient norm: one per workgroup (+ stage 2)
    int64_t npartials;        // capacity of partials
    float *blockfac;          // per block: Adam-mini lr/bc1/h, LAMB lr*trust;
                              // fp16 scaled moments: the maxima slots
    const int32_t *blockspan; // span index of each block (Adam-mini shared-v
                              // block; LAMB or scaled-moment tensor)
    int32_t block0;           // Adam-mini finalize: blocks [block0, nblocks)
    int32_t nblocks;
    const Codebook *codebook;
    int32_t bits, block;
    int32_t interleaved;      // blockwise 2-state: m and v codes (and absmax)
                              // side by side in qm (absmax_m); AdamW /
                              // AdEMAMix: the moments of a tensor in one
                              // array, in blocks of kMomentBlock elements
    float *found_inf;         // finite check output
    int32_t cus;              // compute units of the device
    const PackDesc *packs;    // packs of small tensors (elementwise plans)
    const int32_t *pack_off;
    const PackMember *pack_td;
    int64_t pack_unit0;       // units [pack_unit0, nunits) of the plan are packs
    int32_t grid_request;     // persistent workgroups (0 = see units_per_wg)
    int32_t units_per_wg;     // without a persistent grid: consecutive units
                              // per workgroup (set by the launcher)
};

// Kernel trace of a plan (optim_plan_trace): while one of a traced plan's
// entry points runs, g_trace points at its trace and every launch takes the
// next start / stop event pair, which the kernel's dispatch stamps itself
// (hipExtLaunchKernel); nothing is added to the stream.
struct TraceRec {
    const char *name;  // the launch site's kernel expression (a literal)
    int64_t grid;      // workgroups
    hipEvent_t start, stop;
};
struct Trace {
    std::vector<TraceRec> recs;  // capacity: one pair per launch
    size_t used = 0;
    int64_t dropped = 0;         // launches after the trace was full
    std::deque<std::pair<const char *, std::string>> names;  // cleaned names (stable addresses)
};
extern thread_local Trace *g_trace;
// The event pair for the next launch of `name` over `grid` workgroups, or
// nullptr (no trace, or the trace is full).
TraceRec *trace_slot(const char *name, int64_t grid);

// Launchers (kernels_*.hip).  Return the hipError_t of the launch.  Step
// launchers always start at least one workgroup (the commit must run even
// for an empty plan).
hipError_t launch_adamw(const StepArgs &a, int pk, int gk, hipStream_t s);
hipError_t launch_ademamix(const StepArgs &a, int pk, int gk, hipStream_t s);
// Adam-mini runs its three kernels segment by segment: a segment is a run of
// whole tensors (units [unit_begin, unit_end), shared-v blocks
// [block_begin, block_end)), either all with shared v and at most a bounded
// number of gradient bytes, or all with full v (no block sums).
struct MiniSegment {
    int64_t unit_begin, unit_end;
    int32_t block_begin, block_end;
};
hipError_t launch_adam_mini(const StepArgs &a, int pk, int gk, const MiniSegment *segs, int32_t nsegs,
                            hipStream_t s);
hipError_t launch_lion(const StepArgs &a, int pk, int gk, hipStream_t s);
// AdamW with 16-bit moments and per-tensor scales (sk: S_F16 / S_BF16)
hipError_t launch_adamw_scaled(const StepArgs &a, int pk, int gk, int sk, hipStream_t s);
hipError_t launch_lamb(const StepArgs &a, int pk, int gk, hipStream_t s);
hipError_t launch_blockwise(const StepArgs &a, int gk, bool ademamix, hipStream_t s);
hipError_t launch_check_finite(const StepArgs &a, int gk, hipStream_t s);
// Workgroups of the finite check / gradient norm pass for a plan.
int64_t finite_pass_grid(int64_t nunits, int64_t tile, int32_t grid_request);
// Partial sums the gradient norm pass needs (both reduction stages).
int64_t norm_partials(int64_t nunits, int64_t tile, int32_t grid_request);
hipError_t launch_grad_norm(const StepArgs &a, int gk, const float *inv_scale, double max_norm,
                            float *norm_out, float *clip_out, hipStream_t s);
hipError_t launch_scaler_update(float *scale, float *inv_scale, int32_t *tracker, const float *found_inf,
                                double growth, double backoff, int32_t interval, hipStream_t s);
hipError_t launch_quantize(const Codebook *cb, int bits, int block, int is_signed, const float *x,
                           int64_t n, uint8_t *codes, float *absmax, hipStream_t s);
hipError_t launch_dequantize(const Codebook *cb, int bits, int block, int is_signed, const uint8_t *codes,
                             const float *absmax, int64_t n, float *x, hipStream_t s);
hipError_t launch_remainder_split(const float *x, uint16_t *b, int16_t *r, int64_t n,
                                  hipStream_t s);
hipError_t launch_remainder_reconstruct(const uint16_t *b, const int16_t *r, float *x,
                                        int64_t n, hipStream_t s);

}  // namespace optim
