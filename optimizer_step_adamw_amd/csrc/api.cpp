// api.cpp -- C ABI of the fused AdamW-family optimizer step: validation,
// plan tables (tensor descriptors, unit spans, weight-decay groups,
// quantization tables), workspace layout and launches.  Declared in
// include/optim_step.h, which documents each entry point and its sources.
#include "optim_step.h"
#include "plan.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

using namespace optim;

namespace optim {
thread_local Trace *g_trace = nullptr;

TraceRec *trace_slot(const char *name, int64_t grid) {
    Trace *t = g_trace;
    if (!t) return nullptr;
    if (t->used >= t->recs.size()) {
        ++t->dropped;
        return nullptr;
    }
    TraceRec &r = t->recs[t->used++];
    r.name = name;
    r.grid = grid;
    return &r;
}
}  // namespace optim

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &msg) {
    g_err = msg;
    return code;
}

#define HIP_OK(expr)                                                                 \
    do {                                                                             \
        hipError_t e_ = (expr);                                                      \
        if (e_ != hipSuccess)                                                        \
            return fail(OPTIM_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------- codebook
// Dynamic map with mb magnitude bits (see optim_quant_codebook).
void dynamic_map(int mb, float *vals, float *thr) {
    std::vector<float> M;
    M.reserve(size_t(1) << mb);
    M.push_back(0.0f);
    for (int e = 0; e < mb; ++e) {
        const int nk = 1 << (mb - 1 - e);
        const double dec = std::pow(10.0, -(double)e);
        for (int k = 0; k < nk; ++k)
            M.push_back((float)(dec * (0.1 + 0.9 * (double)(k + 1) / (double)nk)));
    }
    std::sort(M.begin(), M.end());
    for (size_t j = 0; j < M.size(); ++j) {
        vals[j] = M[j];
        thr[j] = j == 0 ? 0.0f : (float)(((double)M[j - 1] + (double)M[j]) * 0.5);
    }
}

float bits_to_float(uint32_t u) {
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

// Largest j >= 1 with thr[j] <= a, else 0 (the threshold rule itself).
int threshold_index(const float *thr, int count, float a) {
    int idx = 0;
    for (int j = 1; j < count; ++j)
        if (thr[j] <= a) idx = j;
    return idx;
}

// Values, thresholds and the bucket table of one map.  Returns false if a
// bucket would hold two thresholds or a threshold lies below the table.
bool build_map(int mb, QuantMap &q) {
    std::memset(&q, 0, sizeof q);
    dynamic_map(mb, q.vals, q.thr);
    const int count = 1 << mb;
    for (int j = count; j < (int)(sizeof q.thr / sizeof q.thr[0]); ++j) q.thr[j] = INFINITY;
    const uint32_t shift = 23 - kLutMantBits;
    if (threshold_index(q.thr, count, bits_to_float(((uint32_t)kLutBaseExp << 23) - 1)) != 0) return false;
    for (int b = 0; b < kLutBuckets; ++b) {
        const uint32_t lo = (uint32_t)(b + (kLutBaseExp << kLutMantBits)) << shift;
        const uint32_t hi = lo + (1u << shift) - 1u;
        const int ilo = threshold_index(q.thr, count, bits_to_float(lo));
        const int ihi = threshold_index(q.thr, count, bits_to_float(hi));
        if (ihi - ilo > 1) return false;
        q.lut[b] = (uint8_t)ilo;
    }
    return true;
}

// ---------------------------------------------------------------- plan build
struct Built {
    std::vector<TensorDesc> tensors;
    std::vector<SpanDesc> spans;  // with sentinel
    std::vector<int32_t> blockspan;
    std::vector<double> group_wd;
    int64_t nunits = 0;
    int64_t tile = 0;
    int32_t grid = 0;        // requested persistent workgroups
    bool states16 = false;   // AdamW moments stored in 16 bits with scales
    int64_t npartials = 0;   // capacity of the partials region
    int32_t nblocks = 0;
    std::vector<MiniSegment> segs;  // Adam-mini launch segments
    bool interleaved = false;       // blockwise: interleaved state layout
    std::vector<PackDesc> packs;    // packs of small tensors
    std::vector<int32_t> pack_off;
    std::vector<PackMember> pack_td;
    int64_t pack_unit0 = 0;         // first pack unit (packs come last)
    Layout L{};
};

struct Range {
    uintptr_t lo, hi;
    bool written;
    int tensor;
    const char *what;
};

int check_hp_beta(double b, const char *name) {
    if (!(b >= 0.0 && b < 1.0))
        return fail(OPTIM_EINVAL, std::string("invalid ") + name + " (need 0 <= beta < 1)");
    return OPTIM_OK;
}

bool is_blockwise(int32_t algo) { return algo == OPTIM_ALGO_BLOCKWISE || algo == OPTIM_ALGO_BLOCKWISE_ADEMAMIX; }

int build(const optim_tensor_list *list, int32_t algo, const optim_plan_opts *opts, Built &B) {
    if (!list) return fail(OPTIM_EINVAL, "tensor list is NULL");
    if (algo < OPTIM_ALGO_ADAMW || algo > OPTIM_ALGO_LAMB)
        return fail(OPTIM_EINVAL, "unknown algorithm");
    const int n = list->n;
    if (n < 0) return fail(OPTIM_EINVAL, "negative tensor count");
    const int32_t pdt = list->param_dtype;
    if (pdt != OPTIM_F32 && pdt != OPTIM_BF16 && pdt != OPTIM_F16)
        return fail(OPTIM_EDTYPE, "param_dtype must be OPTIM_F32, OPTIM_BF16 or OPTIM_F16");
    if (list->grad_dtype != OPTIM_F32 && list->grad_dtype != OPTIM_BF16)
        return fail(OPTIM_EDTYPE, "grad_dtype must be OPTIM_F32 or OPTIM_BF16");
    const bool masterw = list->master != nullptr;
    if (masterw && pdt == OPTIM_F32) return fail(OPTIM_EINVAL, "master weights need a BF16 or F16 model param");
    if (pdt == OPTIM_F16 && !masterw) return fail(OPTIM_EUNSUPPORTED, "F16 params need fp32 master weights");
    if (masterw && algo != OPTIM_ALGO_ADAMW && algo != OPTIM_ALGO_ADEMAMIX)
        return fail(OPTIM_EUNSUPPORTED, "master weights are supported for AdamW and AdEMAMix");
    const bool bf16p = pdt == OPTIM_BF16 && !masterw;  // bf16 + remainder
    if (pdt != OPTIM_F32 && is_blockwise(algo))
        return fail(OPTIM_EUNSUPPORTED, "blockwise states take fp32 params only");
    int bits = 0, block = 0;
    if (is_blockwise(algo)) {
        if (!opts) return fail(OPTIM_EINVAL, "blockwise plans need opts (bits, block)");
        bits = opts->bits;
        block = opts->block;
        // a block is L = block/E lanes of one wavefront (E = 4 codes per lane
        // up to block 256, else 8), L a power of two in [16, 64]
        if (bits != 8 && bits != 4) return fail(OPTIM_EINVAL, "bits must be 8 or 4");
        const bool ok = bits == 8 ? (block == 64 || block == 128 || block == 256)
                                  : (block == 128 || block == 256 || block == 512);
        if (!ok)
            return fail(OPTIM_EINVAL, bits == 8 ? "8-bit block must be 64, 128 or 256"
                                                : "4-bit block must be 128, 256 or 512");
    }
    const int32_t layout = opts ? opts->state_layout : OPTIM_LAYOUT_SEPARATE;
    if (layout != OPTIM_LAYOUT_SEPARATE && layout != OPTIM_LAYOUT_INTERLEAVED)
        return fail(OPTIM_EINVAL, "unknown state_layout");
    const bool adam_like = algo == OPTIM_ALGO_ADAMW || algo == OPTIM_ALGO_ADEMAMIX;
    if (layout == OPTIM_LAYOUT_INTERLEAVED && algo != OPTIM_ALGO_BLOCKWISE && !adam_like)
        return fail(OPTIM_EUNSUPPORTED,
                    "the interleaved state layout is for AdamW, AdEMAMix and the 2-state blockwise step");
    // blockwise: m and v codes side by side; AdamW / AdEMAMix: the moments
    // of each tensor in one array, in blocks of kMomentBlock elements
    const bool il = layout == OPTIM_LAYOUT_INTERLEAVED && algo == OPTIM_ALGO_BLOCKWISE;
    const bool mom_il = layout == OPTIM_LAYOUT_INTERLEAVED && adam_like;
    B.interleaved = il || mom_il;
    if (opts && opts->grid < 0) return fail(OPTIM_EINVAL, "negative grid");
    B.grid = opts ? opts->grid : 0;
    if (opts && opts->tile < 0) return fail(OPTIM_EINVAL, "negative tile");
    if (opts && opts->segment_bytes < 0) return fail(OPTIM_EINVAL, "negative segment_bytes");
    const int64_t seg_cap = (opts && opts->segment_bytes > 0) ? opts->segment_bytes : kMiniSegmentBytes;
    bool seg_shared = false;
    int64_t seg_gbytes = 0;
    const int32_t sdt = opts ? opts->state_dtype : OPTIM_F32;
    if (sdt != OPTIM_F32 && sdt != OPTIM_F16 && sdt != OPTIM_BF16)
        return fail(OPTIM_EDTYPE, "state_dtype must be OPTIM_F32, OPTIM_F16 or OPTIM_BF16");
    const bool states16 = sdt != OPTIM_F32;
    if (states16 && algo != OPTIM_ALGO_ADAMW) return fail(OPTIM_EUNSUPPORTED, "16-bit states are for AdamW plans");
    if (states16 && masterw) return fail(OPTIM_EUNSUPPORTED, "16-bit states take fp32 or bf16 + remainder params");
    if (states16 && mom_il) return fail(OPTIM_EUNSUPPORTED, "the interleaved moment layout holds fp32 moments");
    if (n > 0 && states16 && (!list->scale_m || !list->scale_v))
        return fail(OPTIM_EINVAL, "16-bit states need scale_m and scale_v arrays");
    B.states16 = states16;
    // measured on MI355X: 2048 elements per workgroup (two groups of 4 per
    // lane, loaded at once) stream best for AdamW / AdEMAMix / Lion;
    // Adam-mini, LAMB and the two-pass fp16-state step prefer 4096 (per-unit
    // reductions), and the blockwise step amortises its LDS tables and
    // prologue over larger units
    const bool unit_sums = algo == OPTIM_ALGO_ADAM_MINI || algo == OPTIM_ALGO_LAMB || sdt == OPTIM_F16;
    // AdamW / AdEMAMix (fp32 moments) and Lion plans of (2^20, 2^24]
    // elements take the units of the early-load kernel form
    int64_t total = 0;  // elements, counted only up to past the bound
    if (n > 0 && list->numel)
        for (int i = 0; i < n && total <= kEarlyTileMaxElems; ++i)
            total += std::min<int64_t>(std::max<int64_t>(list->numel[i], 0), kMaxNumel);
    const bool early_units = (algo == OPTIM_ALGO_ADAMW || algo == OPTIM_ALGO_ADEMAMIX || algo == OPTIM_ALGO_LION) &&
                             !states16 &&
                             total > kEarlyTileMinElems && total <= kEarlyTileMaxElems;
    const int64_t tile = (opts && opts->tile > 0) ? opts->tile
                         : is_blockwise(algo) ? blockwise_tile(algo == OPTIM_ALGO_BLOCKWISE_ADEMAMIX, bits, il)
                         : unit_sums          ? kAdamMiniTile
                         : early_units        ? kEarlyTile
                                              : kDefaultTile;
    if (tile < kMinTile || tile > (1 << 24) || (tile & (tile - 1)))
        return fail(OPTIM_EINVAL, "tile must be a power of two in [1024, 2^24]");
    if (is_blockwise(algo) && tile < kMinBlockwiseTile)
        return fail(OPTIM_EINVAL, "blockwise tile must be at least 2048");
    B.tile = tile;
    if (n > 0 && (!list->numel || !list->param || !list->grad || !list->weight_decay))
        return fail(OPTIM_EINVAL, "numel, param, grad and weight_decay arrays are required");
    const bool need_mv = !is_blockwise(algo) && algo != OPTIM_ALGO_LION;
    if (n > 0 && need_mv && (!list->m || (!mom_il && !list->v)))
        return fail(OPTIM_EINVAL, mom_il ? "the m array is required" : "m and v arrays are required");
    if (n > 0 && algo == OPTIM_ALGO_LION && !list->m) return fail(OPTIM_EINVAL, "Lion needs the m array");
    if (n > 0 && algo == OPTIM_ALGO_ADEMAMIX && !mom_il && !list->m2)
        return fail(OPTIM_EINVAL, "AdEMAMix needs the m2 array");
    if (n > 0 && is_blockwise(algo) && (!list->qm || (!il && !list->qv) || !list->absmax_m || (!il && !list->absmax_v)))
        return fail(OPTIM_EINVAL, il ? "interleaved blockwise plans need qm and absmax_m"
                                     : "blockwise plans need qm, qv, absmax_m and absmax_v");
    if (n > 0 && algo == OPTIM_ALGO_BLOCKWISE_ADEMAMIX && (!list->qm2 || !list->absmax_m2))
        return fail(OPTIM_EINVAL, "blockwise AdEMAMix plans need qm2 and absmax_m2");
    if (n > 0 && algo == OPTIM_ALGO_ADAM_MINI && (!list->mini_kind || !list->head_numel))
        return fail(OPTIM_EINVAL, "Adam-mini needs mini_kind and head_numel arrays");
    if (n > 0 && bf16p && !list->remainder)
        return fail(OPTIM_EUNSUPPORTED, "bf16 params need int16 remainders (fp32 master)");

    const size_t psz = pdt == OPTIM_F32 ? 4 : 2, gsz = list->grad_dtype == OPTIM_BF16 ? 2 : 4;
    std::vector<Range> ranges;
    B.tensors.assign(n, TensorDesc{});
    B.spans.clear();
    B.blockspan.clear();
    B.group_wd.clear();
    B.nunits = 0;
    B.nblocks = 0;
    B.segs.clear();
    B.packs.clear();
    B.pack_off.clear();
    B.pack_td.clear();
    // Packs: AdamW / AdEMAMix (fp32 moments) and Lion plans lay runs of
    // tensors of at most half a pack end to end in shared units of up to
    // pack_cap elements, so a workgroup serves many small tensors (one
    // prologue, every lane busy) instead of one each.
    const bool packable = (algo == OPTIM_ALGO_ADAMW || algo == OPTIM_ALGO_ADEMAMIX || algo == OPTIM_ALGO_LION) &&
                          !states16;
    const int64_t pack_cap = std::min<int64_t>(tile, kPackElems);
    std::vector<int32_t> open_pack;  // members of the pack being filled
    int64_t open_len = 0;
    auto close_pack = [&]() {
        if (open_pack.empty()) return;
        if (open_pack.size() == 1) {  // a lone member: an ordinary span
            const int32_t t = open_pack[0];
            B.spans.push_back(SpanDesc{B.nunits, 0, B.tensors[t].numel, t, -1});
        } else {
            PackDesc P{(int32_t)B.pack_td.size(), (int32_t)B.pack_off.size(), (int32_t)open_pack.size(),
                       (int32_t)open_len};
            int32_t off = 0;
            for (int32_t t : open_pack) {
                const TensorDesc &T = B.tensors[t];
                B.pack_td.push_back(PackMember{T.p, T.g, T.m, T.v, T.m2, T.rem, T.master, (int32_t)T.numel, T.group,
                                               T.vec_ok, 0});
                B.pack_off.push_back(off);
                off += (int32_t)((B.tensors[t].numel + 3) / 4 * 4);
            }
            B.pack_off.push_back(off);
            B.packs.push_back(P);  // its span is laid after all single-tensor units
        }
        if (open_pack.size() == 1) B.nunits += 1;
        open_pack.clear();
        open_len = 0;
    };
    for (int i = 0; i < n; ++i) {
        const std::string ti = "tensor " + std::to_string(i) + ": ";
        TensorDesc &T = B.tensors[i];
        const int64_t numel = list->numel[i];
        if (numel < 0) return fail(OPTIM_EINVAL, ti + "negative numel");
        if (numel > kMaxNumel) return fail(OPTIM_EINVAL, ti + "numel above 2^48");
        const double wd = list->weight_decay[i];
        if (!(wd >= 0.0) || !std::isfinite(wd)) return fail(OPTIM_EINVAL, ti + "invalid weight_decay");
        auto git = std::find(B.group_wd.begin(), B.group_wd.end(), wd);
        if (git == B.group_wd.end()) {
            if ((int)B.group_wd.size() >= kMaxGroups)
                return fail(OPTIM_EUNSUPPORTED, "more than 64 distinct weight_decay values");
            B.group_wd.push_back(wd);
            git = B.group_wd.end() - 1;
        }
        T.group = (int32_t)(git - B.group_wd.begin());
        T.numel = numel;
        T.p = list->param[i];
        T.g = list->grad[i];
        if (numel > 0 && (!T.p || !T.g)) return fail(OPTIM_EINVAL, ti + "NULL param or grad");
        if (!aligned(T.p, psz) || !aligned(T.g, gsz)) return fail(OPTIM_EALIGN, ti + "param/grad misaligned");
        bool vec = aligned(T.p, 16) && aligned(T.g, 16);
        auto add = [&](const void *ptr, size_t bytes, bool written, const char *what) {
            if (ptr && bytes) ranges.push_back({(uintptr_t)ptr, (uintptr_t)ptr + bytes, written, i, what});
        };
        add(T.p, numel * psz, true, "param");
        add(T.g, numel * gsz, false, "grad");
        if (bf16p) {
            T.rem = static_cast<uint16_t *>(list->remainder[i]);
            if (numel > 0 && !T.rem) return fail(OPTIM_EINVAL, ti + "NULL remainder");
            if (!aligned(T.rem, 2)) return fail(OPTIM_EALIGN, ti + "remainder misaligned");
            vec = vec && aligned(T.rem, 16);
            add(T.rem, numel * 2, true, "remainder");
        } else if (list->remainder && list->remainder[i]) {
            return fail(OPTIM_EINVAL, ti + (masterw ? "remainder given with master weights"
                                                    : "remainder given for fp32 params"));
        }
        if (masterw) {
            T.master = list->master[i];
            if (numel > 0 && !T.master) return fail(OPTIM_EINVAL, ti + "NULL master");
            if (!aligned(T.master, 4)) return fail(OPTIM_EALIGN, ti + "master misaligned");
            vec = vec && aligned(T.master, 16);
            add(T.master, numel * 4, true, "master");
        }
        int32_t kind = OPTIM_MINI_FULL_V;
        int64_t vlen = numel;
        if (algo == OPTIM_ALGO_ADAM_MINI) {
            kind = list->mini_kind[i];
            if (kind == OPTIM_MINI_HEAD) {
                const int64_t h = list->head_numel[i];
                if (h <= 0 || numel % h != 0)
                    return fail(OPTIM_EINVAL, ti + "head_numel must be > 0 and divide numel");
                T.block_len = h;
                vlen = numel / h;
            } else if (kind == OPTIM_MINI_SCALAR) {
                T.block_len = numel;
                vlen = numel > 0 ? 1 : 0;
            } else if (kind == OPTIM_MINI_FULL_V) {
                T.block_len = 0;
            } else {
                return fail(OPTIM_EINVAL, ti + "unknown mini_kind");
            }
        }
        T.kind = kind;
        if (mom_il) {
            // m, v (, m2) of each block of kMomentBlock elements side by side
            // in m: K kMomentBlock floats per block, the last block whole
            const int K = algo == OPTIM_ALGO_ADEMAMIX ? 3 : 2;
            if ((list->v && list->v[i]) || (list->m2 && list->m2[i]))
                return fail(OPTIM_EINVAL, ti + "interleaved moments: v and m2 must be NULL (they live in m)");
            T.m = static_cast<float *>(list->m[i]);
            if (numel > 0 && !T.m) return fail(OPTIM_EINVAL, ti + "NULL m");
            if (!aligned(T.m, 4)) return fail(OPTIM_EALIGN, ti + "m misaligned");
            T.v = T.m ? T.m + kMomentBlock : nullptr;
            T.m2 = T.m && K == 3 ? T.m + 2 * kMomentBlock : nullptr;
            vec = vec && aligned(T.m, 16);
            add(T.m, (numel + kMomentBlock - 1) / kMomentBlock * K * kMomentBlock * 4, true, "m");
        } else if (need_mv) {
            T.m = static_cast<float *>(list->m[i]);
            T.v = static_cast<float *>(list->v[i]);
            if (numel > 0 && (!T.m || !T.v)) return fail(OPTIM_EINVAL, ti + "NULL m or v");
            const size_t ssz = states16 ? 2 : 4;  // bytes per stored moment
            if (!aligned(T.m, ssz) || !aligned(T.v, ssz)) return fail(OPTIM_EALIGN, ti + "m/v misaligned");
            vec = vec && aligned(T.m, 16) && (kind != OPTIM_MINI_FULL_V || aligned(T.v, 16));
            add(T.m, numel * ssz, true, "m");
            add(T.v, vlen * ssz, true, "v");
            if (states16) {
                T.scale_m = list->scale_m[i];
                T.scale_v = list->scale_v[i];
                if (numel > 0 && (!T.scale_m || !T.scale_v)) return fail(OPTIM_EINVAL, ti + "NULL state scale");
                if (!aligned(T.scale_m, 4) || !aligned(T.scale_v, 4))
                    return fail(OPTIM_EALIGN, ti + "state scale misaligned");
                add(T.scale_m, 4, true, "scale_m");
                add(T.scale_v, 4, true, "scale_v");
            }
        }
        if (algo == OPTIM_ALGO_LION) {
            T.m = static_cast<float *>(list->m[i]);
            if (numel > 0 && !T.m) return fail(OPTIM_EINVAL, ti + "NULL m");
            if (!aligned(T.m, 4)) return fail(OPTIM_EALIGN, ti + "m misaligned");
            vec = vec && aligned(T.m, 16);
            add(T.m, numel * 4, true, "m");
        }
        if (algo == OPTIM_ALGO_ADEMAMIX && !mom_il) {
            T.m2 = static_cast<float *>(list->m2[i]);
            if (numel > 0 && !T.m2) return fail(OPTIM_EINVAL, ti + "NULL m2");
            if (!aligned(T.m2, 4)) return fail(OPTIM_EALIGN, ti + "m2 misaligned");
            vec = vec && aligned(T.m2, 16);
            add(T.m2, numel * 4, true, "m2");
        }
        if (is_blockwise(algo) && il) {
            // m and v codes side by side in qm, (absmax m, absmax v) pairs in am
            if ((list->qv && list->qv[i]) || (list->absmax_v && list->absmax_v[i]))
                return fail(OPTIM_EINVAL, ti + "interleaved layout: qv and absmax_v must be NULL");
            T.qm = static_cast<uint8_t *>(list->qm[i]);
            T.am = list->absmax_m[i];
            if (numel > 0 && (!T.qm || !T.am)) return fail(OPTIM_EINVAL, ti + "NULL code or absmax buffer");
            if (!aligned(T.am, 8)) return fail(OPTIM_EALIGN, ti + "interleaved absmax must be 8-byte aligned");
            vec = vec && aligned(T.qm, 16);
            add(T.qm, numel * 2 * bits / 8, true, "qm");
            add(T.am, (numel + block - 1) / block * 8, true, "absmax_m");
        } else if (is_blockwise(algo)) {
            T.qm = static_cast<uint8_t *>(list->qm[i]);
            T.qv = static_cast<uint8_t *>(list->qv[i]);
            T.am = list->absmax_m[i];
            T.av = list->absmax_v[i];
            if (numel > 0 && (!T.qm || !T.qv || !T.am || !T.av))
                return fail(OPTIM_EINVAL, ti + "NULL code or absmax buffer");
            if (!aligned(T.am, 4) || !aligned(T.av, 4)) return fail(OPTIM_EALIGN, ti + "absmax misaligned");
            vec = vec && aligned(T.qm, 16) && aligned(T.qv, 16);
            const int64_t cbytes = (numel * bits + 7) / 8;
            const int64_t nblk = (numel + block - 1) / block;
            add(T.qm, cbytes, true, "qm");
            add(T.qv, cbytes, true, "qv");
            add(T.am, nblk * 4, true, "absmax_m");
            add(T.av, nblk * 4, true, "absmax_v");
            if (algo == OPTIM_ALGO_BLOCKWISE_ADEMAMIX) {
                T.qm2 = static_cast<uint8_t *>(list->qm2[i]);
                T.am2 = list->absmax_m2[i];
                if (numel > 0 && (!T.qm2 || !T.am2)) return fail(OPTIM_EINVAL, ti + "NULL qm2 or absmax_m2");
                if (!aligned(T.am2, 4)) return fail(OPTIM_EALIGN, ti + "absmax_m2 misaligned");
                vec = vec && aligned(T.qm2, 16);
                add(T.qm2, cbytes, true, "qm2");
                add(T.am2, nblk * 4, true, "absmax_m2");
            }
        }
        T.vec_ok = vec ? 1 : 0;
        if (numel == 0) continue;
        const int64_t units_before = B.nunits;
        const int32_t blocks_before = B.nblocks;
        // spans
        if (algo == OPTIM_ALGO_ADAM_MINI && kind != OPTIM_MINI_FULL_V) {
            for (int64_t s = 0; s < numel; s += T.block_len) {
                SpanDesc sp{B.nunits, s, T.block_len, i, B.nblocks};
                B.blockspan.push_back((int32_t)B.spans.size());
                B.spans.push_back(sp);
                B.nunits += (T.block_len + tile - 1) / tile;
                if (B.nblocks == INT32_MAX) return fail(OPTIM_EUNSUPPORTED, "too many blocks");
                ++B.nblocks;
            }
        } else if (algo == OPTIM_ALGO_LAMB || states16) {
            // one block per tensor: its trust ratio, or its state scales
            B.blockspan.push_back((int32_t)B.spans.size());
            B.spans.push_back(SpanDesc{B.nunits, 0, numel, i, B.nblocks});
            B.nunits += (numel + tile - 1) / tile;
            ++B.nblocks;
        } else if (packable && numel <= pack_cap / 2) {
            const int64_t r = (numel + 3) / 4 * 4;
            if (open_len + r > pack_cap || (int32_t)open_pack.size() >= kMaxPackTensors) close_pack();
            open_pack.push_back(i);
            open_len += r;
        } else {
            close_pack();
            B.spans.push_back(SpanDesc{B.nunits, 0, numel, i, -1});
            B.nunits += (numel + tile - 1) / tile;
        }
        // Adam-mini segments: runs of whole tensors, all with shared v and
        // at most seg_cap gradient bytes (a larger tensor alone), or all
        // with full v
        if (algo == OPTIM_ALGO_ADAM_MINI) {
            const bool shared = kind != OPTIM_MINI_FULL_V;
            const int64_t gb = numel * (int64_t)gsz;
            if (B.segs.empty() || shared != seg_shared || (shared && seg_gbytes + gb > seg_cap)) {
                B.segs.push_back(MiniSegment{units_before, B.nunits, blocks_before, B.nblocks});
                seg_shared = shared;
                seg_gbytes = gb;
            } else {
                B.segs.back().unit_end = B.nunits;
                B.segs.back().block_end = B.nblocks;
                seg_gbytes += gb;
            }
        }
    }
    close_pack();
    B.pack_unit0 = B.nunits;
    for (size_t k = 0; k < B.packs.size(); ++k) {
        B.spans.push_back(SpanDesc{B.nunits, (int64_t)k, B.packs[k].len, kPackTensor, -1});
        B.nunits += 1;
    }
    if (B.spans.size() >= (size_t)INT32_MAX || B.pack_off.size() >= (size_t)INT32_MAX)
        return fail(OPTIM_EUNSUPPORTED, "too many spans");
    B.spans.push_back(SpanDesc{B.nunits, 0, 0, -1, -1});  // sentinel

    // no written buffer may overlap any other buffer of the plan
    std::sort(ranges.begin(), ranges.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
    uintptr_t end_all = 0, end_w = 0;
    const Range *cov_all = nullptr, *cov_w = nullptr;
    for (const Range &r : ranges) {
        const Range *hit = nullptr;
        if (r.written && r.lo < end_all) hit = cov_all;
        else if (!r.written && r.lo < end_w) hit = cov_w;
        if (hit)
            return fail(OPTIM_EINVAL, "buffers overlap: tensor " + std::to_string(hit->tensor) + " " +
                                          hit->what + " and tensor " + std::to_string(r.tensor) + " " +
                                          r.what);
        if (r.hi > end_all) { end_all = r.hi; cov_all = &r; }
        if (r.written && r.hi > end_w) { end_w = r.hi; cov_w = &r; }
    }

    Layout &L = B.L;
    size_t off = 0;
    L.counters = off; off += align256(kCounterBytes);
    L.group_wd = off; off += align256(kMaxGroups * sizeof(double));
    L.tensors = off; off += align256(std::max<size_t>(1, B.tensors.size()) * sizeof(TensorDesc));
    L.spans = off; off += align256(B.spans.size() * sizeof(SpanDesc));
    L.codebook = off; off += is_blockwise(algo) ? align256(sizeof(Codebook)) : 0;
    L.blockspan = off; off += align256(std::max<size_t>(1, B.blockspan.size()) * sizeof(int32_t));
    L.packs = off; off += align256(B.packs.size() * sizeof(PackDesc));
    L.pack_off = off; off += align256(B.pack_off.size() * sizeof(int32_t));
    L.pack_td = off; off += align256(B.pack_td.size() * sizeof(PackMember));
    // partial sums: Adam-mini's block sums (one per unit) and the gradient
    // norm pass (one per workgroup) share the region; they never overlap in
    // stream order
    L.partials = off;
    // (LAMB: two per unit, sums of p^2 and u^2)
    B.npartials = std::max<int64_t>(algo == OPTIM_ALGO_ADAM_MINI ? B.nunits
                                    : algo == OPTIM_ALGO_LAMB    ? 2 * B.nunits
                                                                 : 0,
                                    norm_partials(B.nunits, B.tile, B.grid));
    off += align256(std::max<int64_t>(1, B.npartials) * sizeof(double));
    // per-block factors; 16-bit states: the maxima slots of each tensor
    // (zero in the uploaded image)
    L.blockfac = off;
    off += align256(B.states16 ? std::max<int32_t>(1, B.nblocks) * kAmaxBytesPerBlock
                               : std::max<int32_t>(1, 2 * B.nblocks) * sizeof(float));
    L.total = off;
    return OPTIM_OK;
}

}  // namespace

struct optim_plan {
    int32_t algo;
    int32_t pk, gk;
    int32_t bits, block;
    int32_t grid;  // requested persistent workgroups (0 = one per unit)
    int32_t cus;
    int32_t nspans, nblocks, ngroups;
    int64_t nunits;
    int64_t tile;
    int64_t npartials;
    int32_t state_dtype;
    char *ws;
    Layout L;
    std::vector<MiniSegment> segs;  // Adam-mini launch segments
    int32_t interleaved;            // blockwise: interleaved state layout
    int32_t sched;
    double lr_max, lr_min;
    int32_t K;
    int32_t *iter_dev;
    // plans on the static workspace: the device and the creation number
    // (0 for a plan on a caller's workspace)
    int32_t static_dev;
    uint64_t static_gen;
    Trace *trace;  // kernel trace (optim_plan_trace), or NULL
    int64_t pack_unit0;  // first pack unit
};

extern "C" {

const char *optim_last_error(void) { return g_err.c_str(); }

int optim_quant_codebook(int32_t bits, int32_t is_signed, float *values, float *thresholds) {
    if (bits != 8 && bits != 4) return fail(OPTIM_EINVAL, "bits must be 8 or 4");
    if (!values || !thresholds) return fail(OPTIM_EINVAL, "NULL output");
    dynamic_map(is_signed ? bits - 1 : bits, values, thresholds);
    return OPTIM_OK;
}

int optim_plan_workspace_size(const optim_tensor_list *list, int32_t algo,
                              const optim_plan_opts *opts, size_t *bytes) {
    if (!bytes) return fail(OPTIM_EINVAL, "bytes is NULL");
    Built B;
    const int rc = build(list, algo, opts, B);
    if (rc) return rc;
    *bytes = B.L.total;
    return OPTIM_OK;
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- static workspace
// The workspace of plans made by optim_plan_create_static, for callers that
// cannot allocate device memory.  One array per device (each device that
// loads the library holds its own copy at its own address until the process
// ends).  In host code `scratch` is only a stand-in for the symbol: its
// device address is looked up once per device with hipGetSymbolAddress and
// kept in g_scratch_ptr, and only that address is ever handed to the device.
__device__ __align__(256) unsigned char scratch[OPTIM_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
// creation number of the live static plan of each device; a plan made
// earlier on the same device has been overwritten and is refused
std::atomic<uint64_t> g_static_gen[kMaxDevices];

int scratch_of_device(int dev, void **ptr) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(OPTIM_EUNSUPPORTED, "static workspace: device index " + std::to_string(dev) + " above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        HIP_OK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || !aligned(p, 256)) return fail(OPTIM_EHIP, "static workspace: no 256-byte aligned device address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return OPTIM_OK;
}

// Refuses a static plan whose tables a later optim_plan_create_static on the
// same device has overwritten (its kernels would walk another plan's tables).
int check_live(const optim_plan *P, const char *fn) {
    if (P->static_gen && P->static_gen != g_static_gen[P->static_dev].load(std::memory_order_acquire))
        return fail(OPTIM_EINVAL, std::string(fn) +
                                      ": this static plan was superseded by a later optim_plan_create_static "
                                      "on its device (the static workspace holds one plan at a time)");
    return OPTIM_OK;
}

// ---------------------------------------------------------------- kernel trace
void free_trace(optim_plan *P) {
    if (!P->trace) return;
    for (TraceRec &r : P->trace->recs) {
        if (r.start) (void)hipEventDestroy(r.start);
        if (r.stop) (void)hipEventDestroy(r.stop);
    }
    delete P->trace;
    P->trace = nullptr;
}

// "(mini_update_kernel<PK, GK>)" -> "mini_update_kernel"; kept in the trace
// so the returned pointers live until the trace is freed.
const char *clean_name(Trace *t, const char *raw) {
    for (const auto &kv : t->names)
        if (kv.first == raw) return kv.second.c_str();
    std::string s(raw ? raw : "");
    s.erase(std::remove(s.begin(), s.end(), '('), s.end());
    const size_t lt = s.find('<');
    if (lt != std::string::npos) s.resize(lt);
    while (!s.empty() && (s.back() == ')' || s.back() == ' ')) s.pop_back();
    t->names.emplace_back(raw, s);
    return t->names.back().second.c_str();
}

// Points the launches of one entry point at its plan's trace.
struct TraceScope {
    explicit TraceScope(const optim_plan *P) { g_trace = P ? P->trace : nullptr; }
    ~TraceScope() { g_trace = nullptr; }
};

// Plan creation on a given workspace (the caller's, or the static one).
int create_on(const Built &B, const optim_tensor_list *list, int32_t algo, const optim_plan_opts *opts,
              void *workspace, hipStream_t s, int dev, optim_plan **out) {
    // host image of the table region [0, partials); with 16-bit states the
    // whole workspace, so the maxima slots start at zero
    std::vector<char> img(B.states16 ? B.L.total : B.L.partials, 0);
    std::memcpy(img.data() + B.L.group_wd, B.group_wd.data(), B.group_wd.size() * sizeof(double));
    std::memcpy(img.data() + B.L.tensors, B.tensors.data(), B.tensors.size() * sizeof(TensorDesc));
    std::memcpy(img.data() + B.L.spans, B.spans.data(), B.spans.size() * sizeof(SpanDesc));
    std::memcpy(img.data() + B.L.blockspan, B.blockspan.data(), B.blockspan.size() * sizeof(int32_t));
    std::memcpy(img.data() + B.L.packs, B.packs.data(), B.packs.size() * sizeof(PackDesc));
    std::memcpy(img.data() + B.L.pack_off, B.pack_off.data(), B.pack_off.size() * sizeof(int32_t));
    std::memcpy(img.data() + B.L.pack_td, B.pack_td.data(), B.pack_td.size() * sizeof(PackMember));
    if (is_blockwise(algo)) {
        Codebook *cb = reinterpret_cast<Codebook *>(img.data() + B.L.codebook);
        if (!build_map(7, cb->m8) || !build_map(8, cb->v8) || !build_map(3, cb->m4) || !build_map(4, cb->v4))
            return fail(OPTIM_EUNSUPPORTED, "quantization map does not fit the bucket table");
    }
    int cus = 0;
    HIP_OK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    HIP_OK(hipMemcpyAsync(workspace, img.data(), img.size(), hipMemcpyHostToDevice, s));
    HIP_OK(hipStreamSynchronize(s));

    optim_plan *P = new (std::nothrow) optim_plan{};
    if (!P) return fail(OPTIM_EINVAL, "out of host memory");
    P->algo = algo;
    P->pk = list->param_dtype == OPTIM_F32 ? P_F32
            : !list->master                 ? P_BF16R
            : list->param_dtype == OPTIM_BF16 ? P_MBF16
                                              : P_MF16;
    P->gk = list->grad_dtype == OPTIM_BF16 ? G_BF16 : G_F32;
    P->bits = opts ? opts->bits : 0;
    P->block = opts ? opts->block : 0;
    P->grid = opts ? opts->grid : 0;
    P->cus = cus;
    P->nspans = (int32_t)B.spans.size() - 1;
    P->nblocks = B.nblocks;
    P->ngroups = (int32_t)B.group_wd.size();
    P->nunits = B.nunits;
    P->tile = B.tile;
    P->npartials = B.npartials;
    P->state_dtype = opts ? opts->state_dtype : OPTIM_F32;
    P->ws = static_cast<char *>(workspace);
    P->L = B.L;
    P->segs = B.segs;
    P->interleaved = B.interleaved ? 1 : 0;
    P->sched = OPTIM_SCHED_NONE;
    P->static_dev = dev;
    P->static_gen = 0;
    P->pack_unit0 = B.pack_unit0;
    *out = P;
    return OPTIM_OK;
}

}  // namespace

extern "C" {

int optim_plan_create(const optim_tensor_list *list, int32_t algo, const optim_plan_opts *opts,
                      void *workspace, size_t workspace_bytes, void *stream, optim_plan **out) {
    if (!out) return fail(OPTIM_EINVAL, "out is NULL");
    *out = nullptr;
    Built B;
    int rc = build(list, algo, opts, B);
    if (rc) return rc;
    if (!workspace || !aligned(workspace, 256))
        return fail(OPTIM_EWORKSPACE, "workspace must be a 256-byte aligned device pointer");
    if (workspace_bytes < B.L.total)
        return fail(OPTIM_EWORKSPACE, "workspace too small: need " + std::to_string(B.L.total) +
                                          " bytes, got " + std::to_string(workspace_bytes));
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    return create_on(B, list, algo, opts, workspace, static_cast<hipStream_t>(stream), dev, out);
}

int optim_plan_create_static(const optim_tensor_list *list, int32_t algo, const optim_plan_opts *opts,
                             void *stream, optim_plan **out) {
    if (!out) return fail(OPTIM_EINVAL, "out is NULL");
    *out = nullptr;
    Built B;
    int rc = build(list, algo, opts, B);
    if (rc) return rc;
    if (B.L.total > (size_t)OPTIM_STATIC_WORKSPACE_BYTES)
        return fail(OPTIM_EWORKSPACE, "optim_plan_create_static: the plan needs " + std::to_string(B.L.total) +
                                          " bytes of workspace; the static workspace holds " +
                                          std::to_string((size_t)OPTIM_STATIC_WORKSPACE_BYTES) +
                                          " (use optim_plan_create with a caller workspace)");
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    void *ws = nullptr;
    if ((rc = scratch_of_device(dev, &ws))) return rc;
    // every earlier static plan of this device is superseded from here on,
    // also if this creation fails after overwriting part of the tables
    const uint64_t gen = g_static_gen[dev].fetch_add(1, std::memory_order_acq_rel) + 1;
    optim_plan *P = nullptr;
    if ((rc = create_on(B, list, algo, opts, ws, static_cast<hipStream_t>(stream), dev, &P))) return rc;
    P->static_gen = gen;
    *out = P;
    return OPTIM_OK;
}

int optim_plan_destroy(optim_plan *plan) {
    if (plan) free_trace(plan);
    delete plan;
    return OPTIM_OK;
}

int optim_plan_trace(optim_plan *plan, int32_t capacity) {
    if (!plan) return fail(OPTIM_EINVAL, "plan is NULL");
    if (capacity < 0) return fail(OPTIM_EINVAL, "negative trace capacity");
    free_trace(plan);
    if (capacity == 0) return OPTIM_OK;
    Trace *t = new (std::nothrow) Trace{};
    if (!t) return fail(OPTIM_EINVAL, "out of host memory");
    t->recs.reserve((size_t)capacity);
    for (int32_t i = 0; i < capacity; ++i) {
        TraceRec r{nullptr, 0, nullptr, nullptr};
        hipError_t e = hipEventCreate(&r.start);
        if (e == hipSuccess) {
            e = hipEventCreate(&r.stop);
            if (e != hipSuccess) (void)hipEventDestroy(r.start);
        }
        if (e != hipSuccess) {
            plan->trace = t;
            free_trace(plan);
            return fail(OPTIM_EHIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
        }
        t->recs.push_back(r);
    }
    plan->trace = t;
    return OPTIM_OK;
}

int optim_plan_trace_read(optim_plan *plan, optim_kernel_time *out, int32_t max, int32_t *count,
                          int64_t *dropped) {
    if (!plan || !count) return fail(OPTIM_EINVAL, "plan and count are required");
    if (max < 0 || (max > 0 && !out)) return fail(OPTIM_EINVAL, "need out[max], max >= 0");
    Trace *t = plan->trace;
    if (!t) return fail(OPTIM_EINVAL, "the plan has no trace (optim_plan_trace)");
    const size_t n = t->used;
    t->used = 0;
    const int64_t lost = t->dropped;
    t->dropped = 0;
    for (size_t i = 0; i < n; ++i) {
        const TraceRec &r = t->recs[i];
        HIP_OK(hipEventSynchronize(r.stop));
        float ms = 0.0f;
        HIP_OK(hipEventElapsedTime(&ms, r.start, r.stop));
        if ((int64_t)i < (int64_t)max) out[i] = optim_kernel_time{clean_name(t, r.name), r.grid, (double)ms};
    }
    *count = (int32_t)n;
    if (dropped) *dropped = lost;
    return OPTIM_OK;
}

int optim_plan_set_schedule(optim_plan *plan, int32_t kind, double lr_max, double lr_min, int32_t K,
                            int32_t *iter_dev) {
    if (!plan) return fail(OPTIM_EINVAL, "plan is NULL");
    if (kind == OPTIM_SCHED_NONE) {
        plan->sched = OPTIM_SCHED_NONE;
        plan->iter_dev = nullptr;
        return OPTIM_OK;
    }
    if (kind != OPTIM_SCHED_COSINE) return fail(OPTIM_EINVAL, "unknown schedule kind");
    if (!(lr_max >= 0.0) || !(lr_min >= 0.0) || !std::isfinite(lr_max) || !std::isfinite(lr_min))
        return fail(OPTIM_EINVAL, "invalid learning rate (need 0 <= lr, finite)");
    if (K <= 0) return fail(OPTIM_EINVAL, "schedule length K must be > 0");
    if (!iter_dev || !aligned(iter_dev, 4)) return fail(OPTIM_EINVAL, "iter_dev must be an aligned device int32");
    plan->sched = kind;
    plan->lr_max = lr_max;
    plan->lr_min = lr_min;
    plan->K = K;
    plan->iter_dev = iter_dev;
    return OPTIM_OK;
}

}  // extern "C"

namespace {

StepArgs step_args(optim_plan *P) {
    StepArgs a{};
    a.done = reinterpret_cast<uint32_t *>(P->ws + P->L.counters);
    a.commit = 1;
    a.tensors = reinterpret_cast<const TensorDesc *>(P->ws + P->L.tensors);
    a.spans = reinterpret_cast<const SpanDesc *>(P->ws + P->L.spans);
    a.nspans = P->nspans;
    a.nunits = P->nunits;
    a.tile = P->tile;
    a.partials = reinterpret_cast<double *>(P->ws + P->L.partials);
    a.npartials = P->npartials;
    a.blockfac = reinterpret_cast<float *>(P->ws + P->L.blockfac);
    a.blockspan = reinterpret_cast<const int32_t *>(P->ws + P->L.blockspan);
    a.packs = reinterpret_cast<const PackDesc *>(P->ws + P->L.packs);
    a.pack_off = reinterpret_cast<const int32_t *>(P->ws + P->L.pack_off);
    a.pack_td = reinterpret_cast<const PackMember *>(P->ws + P->L.pack_td);
    a.pack_unit0 = P->pack_unit0;
    a.nblocks = P->nblocks;
    a.codebook = reinterpret_cast<const Codebook *>(P->ws + P->L.codebook);
    a.bits = P->bits;
    a.block = P->block;
    a.interleaved = P->interleaved;
    a.cus = P->cus;
    a.grid_request = P->grid;
    a.units_per_wg = 1;
    return a;
}

// Validates the per-step device scalars and fills the inputs every step
// kernel derives its scalars from.
int step_inputs(optim_plan *P, double b1, double b2, double b3, double alpha, double eps, float *lr_dev,
                const float *inv_scale, const float *found_inf, int32_t *step_dev, StepArgs &a) {
    if (!lr_dev || !aligned(lr_dev, 4)) return fail(OPTIM_EINVAL, "lr_dev must be an aligned device float");
    if (!step_dev || !aligned(step_dev, 4)) return fail(OPTIM_EINVAL, "step_dev must be an aligned device int32");
    if (!aligned(inv_scale, 4) || !aligned(found_inf, 4)) return fail(OPTIM_EALIGN, "scalar pointer misaligned");
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(OPTIM_EINVAL, "invalid eps (need finite eps >= 0)");
    a = step_args(P);
    PrepArgs &p = a.prep;
    p.group_wd = reinterpret_cast<const double *>(P->ws + P->L.group_wd);
    p.ngroups = P->ngroups;
    p.sched = P->sched;
    p.lr_dev = lr_dev;
    p.inv_scale = inv_scale;
    p.found_inf = found_inf;
    p.step_dev = step_dev;
    p.iter_dev = P->iter_dev;
    p.lr_max = P->lr_max;
    p.lr_min = P->lr_min;
    p.K = P->K;
    p.beta1 = b1;
    p.beta2 = b2;
    p.beta3 = b3;
    p.alpha = alpha;
    p.eps = eps;
    return OPTIM_OK;
}

int check_plan(optim_plan *P, int32_t algo, const char *fn) {
    if (!P) return fail(OPTIM_EINVAL, std::string(fn) + ": plan is NULL");
    if (P->algo != algo) return fail(OPTIM_EINVAL, std::string(fn) + ": plan was built for another algorithm");
    return check_live(P, fn);
}

// the quantize / dequantize helpers take either blockwise plan
int check_blockwise_plan(optim_plan *P, const char *fn) {
    if (!P) return fail(OPTIM_EINVAL, std::string(fn) + ": plan is NULL");
    if (!is_blockwise(P->algo)) return fail(OPTIM_EINVAL, std::string(fn) + ": plan is not blockwise");
    return check_live(P, fn);
}

int check_ademamix_hp(const optim_ademamix_hp *hp) {
    if (!hp) return fail(OPTIM_EINVAL, "hyperparameters are NULL");
    int rc;
    if ((rc = check_hp_beta(hp->beta1, "beta1")) || (rc = check_hp_beta(hp->beta2, "beta2")) ||
        (rc = check_hp_beta(hp->beta3, "beta3")))
        return rc;
    if (!std::isfinite(hp->alpha) || hp->alpha < 0.0) return fail(OPTIM_EINVAL, "invalid alpha (need finite alpha >= 0)");
    return OPTIM_OK;
}

int check_adamw_hp(const optim_adamw_hp *hp) {
    if (!hp) return fail(OPTIM_EINVAL, "hyperparameters are NULL");
    int rc = check_hp_beta(hp->beta1, "beta1");
    if (rc) return rc;
    return check_hp_beta(hp->beta2, "beta2");
}

}  // namespace

extern "C" {

int optim_step_adamw(optim_plan *plan, const optim_adamw_hp *hp, float *lr_dev, const float *inv_scale_dev,
                     const float *found_inf_dev, int32_t *step_dev, void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_ADAMW, "optim_step_adamw");
    if (!rc) rc = check_adamw_hp(hp);
    if (rc) return rc;
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, 0.0, 0.0, hp->eps, lr_dev, inv_scale_dev, found_inf_dev,
                     step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    if (plan->state_dtype != OPTIM_F32)
        HIP_OK(launch_adamw_scaled(a, plan->pk, plan->gk, plan->state_dtype == OPTIM_F16 ? S_F16 : S_BF16,
                                   static_cast<hipStream_t>(stream)));
    else
        HIP_OK(launch_adamw(a, plan->pk, plan->gk, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_step_ademamix(optim_plan *plan, const optim_ademamix_hp *hp, float *lr_dev,
                        const float *inv_scale_dev, const float *found_inf_dev, int32_t *step_dev,
                        void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_ADEMAMIX, "optim_step_ademamix");
    if (!rc) rc = check_ademamix_hp(hp);
    if (rc) return rc;
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, hp->beta3, hp->alpha, hp->eps, lr_dev, inv_scale_dev,
                     found_inf_dev, step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    HIP_OK(launch_ademamix(a, plan->pk, plan->gk, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_step_adam_mini(optim_plan *plan, const optim_adamw_hp *hp, float *lr_dev, const float *inv_scale_dev,
                         const float *found_inf_dev, int32_t *step_dev, void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_ADAM_MINI, "optim_step_adam_mini");
    if (!rc) rc = check_adamw_hp(hp);
    if (rc) return rc;
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, 0.0, 0.0, hp->eps, lr_dev, inv_scale_dev, found_inf_dev,
                     step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    HIP_OK(launch_adam_mini(a, plan->pk, plan->gk, plan->segs.data(), (int32_t)plan->segs.size(),
                            static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_step_lion(optim_plan *plan, const optim_lion_hp *hp, float *lr_dev, const float *inv_scale_dev,
                    const float *found_inf_dev, int32_t *step_dev, void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_LION, "optim_step_lion");
    if (rc) return rc;
    if (!hp) return fail(OPTIM_EINVAL, "hyperparameters are NULL");
    if ((rc = check_hp_beta(hp->beta1, "beta1")) || (rc = check_hp_beta(hp->beta2, "beta2"))) return rc;
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, 0.0, 0.0, 0.0, lr_dev, inv_scale_dev, found_inf_dev, step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    HIP_OK(launch_lion(a, plan->pk, plan->gk, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_step_lamb(optim_plan *plan, const optim_adamw_hp *hp, float *lr_dev, const float *inv_scale_dev,
                    const float *found_inf_dev, int32_t *step_dev, void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_LAMB, "optim_step_lamb");
    if (!rc) rc = check_adamw_hp(hp);
    if (rc) return rc;
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, 0.0, 0.0, hp->eps, lr_dev, inv_scale_dev, found_inf_dev,
                     step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    HIP_OK(launch_lamb(a, plan->pk, plan->gk, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_step_8bit_blockwise(optim_plan *plan, const optim_adamw_hp *hp, int32_t bits, int32_t block,
                              float *lr_dev, const float *inv_scale_dev, const float *found_inf_dev,
                              int32_t *step_dev, void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_BLOCKWISE, "optim_step_8bit_blockwise");
    if (!rc) rc = check_adamw_hp(hp);
    if (rc) return rc;
    if (bits != plan->bits || block != plan->block)
        return fail(OPTIM_EINVAL, "bits/block differ from the plan's");
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, 0.0, 0.0, hp->eps, lr_dev, inv_scale_dev, found_inf_dev,
                     step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    HIP_OK(launch_blockwise(a, plan->gk, false, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_step_8bit_blockwise_ademamix(optim_plan *plan, const optim_ademamix_hp *hp, int32_t bits, int32_t block,
                                       float *lr_dev, const float *inv_scale_dev, const float *found_inf_dev,
                                       int32_t *step_dev, void *stream) {
    int rc = check_plan(plan, OPTIM_ALGO_BLOCKWISE_ADEMAMIX, "optim_step_8bit_blockwise_ademamix");
    if (!rc) rc = check_ademamix_hp(hp);
    if (rc) return rc;
    if (bits != plan->bits || block != plan->block)
        return fail(OPTIM_EINVAL, "bits/block differ from the plan's");
    StepArgs a;
    rc = step_inputs(plan, hp->beta1, hp->beta2, hp->beta3, hp->alpha, hp->eps, lr_dev, inv_scale_dev,
                     found_inf_dev, step_dev, a);
    if (rc) return rc;
    const TraceScope ts(plan);
    HIP_OK(launch_blockwise(a, plan->gk, true, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_check_finite(optim_plan *plan, float *found_inf_dev, void *stream) {
    if (!plan) return fail(OPTIM_EINVAL, "plan is NULL");
    if (int rc = check_live(plan, "optim_check_finite")) return rc;
    if (!found_inf_dev || !aligned(found_inf_dev, 4))
        return fail(OPTIM_EINVAL, "found_inf_dev must be an aligned device float");
    if (plan->nunits == 0) return OPTIM_OK;
    StepArgs a = step_args(plan);
    a.commit = 0;
    a.found_inf = found_inf_dev;
    const TraceScope ts(plan);
    HIP_OK(launch_check_finite(a, plan->gk, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_grad_norm(optim_plan *plan, const float *inv_scale_dev, double max_norm, float *found_inf_dev,
                    float *norm_dev, float *clip_inv_scale_dev, void *stream) {
    if (!plan) return fail(OPTIM_EINVAL, "plan is NULL");
    if (int rc = check_live(plan, "optim_grad_norm")) return rc;
    if (!found_inf_dev || !aligned(found_inf_dev, 4))
        return fail(OPTIM_EINVAL, "found_inf_dev must be an aligned device float");
    if (!clip_inv_scale_dev || !aligned(clip_inv_scale_dev, 4))
        return fail(OPTIM_EINVAL, "clip_inv_scale_dev must be an aligned device float");
    if (!aligned(inv_scale_dev, 4) || !aligned(norm_dev, 4)) return fail(OPTIM_EALIGN, "scalar pointer misaligned");
    if (std::isnan(max_norm)) return fail(OPTIM_EINVAL, "max_norm is NaN");
    StepArgs a = step_args(plan);
    a.commit = 0;
    a.found_inf = found_inf_dev;
    const TraceScope ts(plan);
    HIP_OK(launch_grad_norm(a, plan->gk, inv_scale_dev, max_norm, norm_dev, clip_inv_scale_dev,
                            static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_scaler_update(float *scale_dev, float *inv_scale_dev, int32_t *growth_tracker_dev,
                        const float *found_inf_dev, double growth_factor, double backoff_factor,
                        int32_t growth_interval, void *stream) {
    if (!scale_dev || !growth_tracker_dev || !found_inf_dev)
        return fail(OPTIM_EINVAL, "scale, growth tracker and found_inf are required");
    if (!aligned(scale_dev, 4) || !aligned(inv_scale_dev, 4) || !aligned(growth_tracker_dev, 4) ||
        !aligned(found_inf_dev, 4))
        return fail(OPTIM_EALIGN, "scalar pointer misaligned");
    if (!(growth_factor > 1.0) || !std::isfinite(growth_factor))
        return fail(OPTIM_EINVAL, "growth_factor must be finite and > 1");
    if (!(backoff_factor > 0.0 && backoff_factor < 1.0)) return fail(OPTIM_EINVAL, "backoff_factor must be in (0, 1)");
    if (growth_interval < 1) return fail(OPTIM_EINVAL, "growth_interval must be >= 1");
    HIP_OK(launch_scaler_update(scale_dev, inv_scale_dev, growth_tracker_dev, found_inf_dev, growth_factor,
                                backoff_factor, growth_interval, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_quantize_blockwise(optim_plan *plan, int32_t is_signed, const float *x_dev, int64_t n,
                             uint8_t *codes_dev, float *absmax_dev, void *stream) {
    int rc = check_blockwise_plan(plan, "optim_quantize_blockwise");
    if (rc) return rc;
    if (n < 0) return fail(OPTIM_EINVAL, "negative n");
    if (n == 0) return OPTIM_OK;
    if (!x_dev || !codes_dev || !absmax_dev) return fail(OPTIM_EINVAL, "NULL buffer");
    if (!aligned(x_dev, 4) || !aligned(absmax_dev, 4)) return fail(OPTIM_EALIGN, "buffer misaligned");
    HIP_OK(launch_quantize(reinterpret_cast<const Codebook *>(plan->ws + plan->L.codebook), plan->bits,
                           plan->block, is_signed ? 1 : 0, x_dev, n, codes_dev, absmax_dev,
                           static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_dequantize_blockwise(optim_plan *plan, int32_t is_signed, const uint8_t *codes_dev,
                               const float *absmax_dev, int64_t n, float *x_dev, void *stream) {
    int rc = check_blockwise_plan(plan, "optim_dequantize_blockwise");
    if (rc) return rc;
    if (n < 0) return fail(OPTIM_EINVAL, "negative n");
    if (n == 0) return OPTIM_OK;
    if (!x_dev || !codes_dev || !absmax_dev) return fail(OPTIM_EINVAL, "NULL buffer");
    if (!aligned(x_dev, 4) || !aligned(absmax_dev, 4)) return fail(OPTIM_EALIGN, "buffer misaligned");
    HIP_OK(launch_dequantize(reinterpret_cast<const Codebook *>(plan->ws + plan->L.codebook), plan->bits,
                             plan->block, is_signed ? 1 : 0, codes_dev, absmax_dev, n, x_dev,
                             static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_remainder_split(const float *master_dev, uint16_t *bf16_dev, int16_t *rem_dev, int64_t n,
                          void *stream) {
    if (n < 0) return fail(OPTIM_EINVAL, "negative n");
    if (n == 0) return OPTIM_OK;
    if (!master_dev || !bf16_dev || !rem_dev) return fail(OPTIM_EINVAL, "NULL buffer");
    if (!aligned(master_dev, 4) || !aligned(bf16_dev, 2) || !aligned(rem_dev, 2))
        return fail(OPTIM_EALIGN, "buffer misaligned");
    HIP_OK(launch_remainder_split(master_dev, bf16_dev, rem_dev, n, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

int optim_remainder_reconstruct(const uint16_t *bf16_dev, const int16_t *rem_dev, float *master_dev, int64_t n,
                                void *stream) {
    if (n < 0) return fail(OPTIM_EINVAL, "negative n");
    if (n == 0) return OPTIM_OK;
    if (!master_dev || !bf16_dev || !rem_dev) return fail(OPTIM_EINVAL, "NULL buffer");
    if (!aligned(master_dev, 4) || !aligned(bf16_dev, 2) || !aligned(rem_dev, 2))
        return fail(OPTIM_EALIGN, "buffer misaligned");
    HIP_OK(launch_remainder_reconstruct(bf16_dev, rem_dev, master_dev, n, static_cast<hipStream_t>(stream)));
    return OPTIM_OK;
}

}  // extern "C"
