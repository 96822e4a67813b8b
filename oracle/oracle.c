/*
 * oracle.c -- plain, slow, scalar CPU oracle for the fused AdamW-family
 * optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant generator with the HIP library; it is built with gcc, without
 * fast-math and without FP contraction.
 *
 * Arithmetic is IEEE double unless a function is marked "fp32-faithful", in
 * which case every single-precision operation the method prescribes is
 * emulated as one double operation followed by one rounding to float.  For a
 * single +, -, *, / or sqrt of two floats that double rounding is innocuous
 * (53 >= 2*24 + 2), so the result is the correctly rounded float.
 *
 * Sources (web pages; cited by title and section):
 *  [BNB]  "Fix decoupled weight decay ordering in the CUDA Adam/AdEMAMix
 *         kernels" (bitsandbytes PR #2040): PR description; review "Which
 *         ordering is correct"; second review (float64 referee, one-step
 *         algebra); PR body "Why the current tests do not catch it".
 *  [AO]   "4 bit Adam should support non constant lr" (pytorch/ao #730).
 *  [MINI] "Adam-mini <> DTensor" (Adam-mini issue #14): the AdamWMini class.
 *  [LTN]  "FusedAdam & PyTorch Lightning AMP" (Lightning issue #15501).
 *  [TE]   "Support store_param_remainders feature from Apex in TE Fused
 *         Adam" (TransformerEngine PR #1408): description.
 *  [LTN]  also for the loop around the step: scale, backward, the optional
 *         unscale_ that exists for gradient clipping, step, update.
 *
 * Parity pins: every function below is pinned by a CPU test against a closed
 * form, an invariant, a library routine (torch.optim.AdamW in float64) or an
 * exhaustive / brute-force check.  The multi-step fp32 trajectories have no
 * closed form; beyond those pins the oracle is the reference.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define F32(x) ((double)(float)(x)) /* one rounding to float, kept as double */

/* ------------------------------------------------------------------------ */
/* AdamW, decoupled decay in Loshchilov & Hutter Algorithm 2 order.
 * [BNB] PR description and review "Which ordering is correct": the decay and
 * the gradient-based update are both taken from the previous parameter,
 * p <- p*(1 - lr*wd) + step_size*update; torch.optim.AdamW shrinks the
 * parameter before the moment updates.  [MINI] AdamWMini (full-v branch):
 * h = sqrt(v)/sqrt(1 - beta2^t) + eps, stepsize = lr/(1 - beta1^t).
 * t is the 1-based count of applied steps including this one.            */
void oracle_adamw_step(int64_t n, double *p, double *m, double *v,
                       const double *g, double lr, double beta1, double beta2,
                       double eps, double wd, int64_t t)
{
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    double step_size = lr / bc1;
    double bc2_sqrt = sqrt(bc2);
    for (int64_t i = 0; i < n; ++i) {
        p[i] = p[i] * (1.0 - lr * wd);
        m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];
        v[i] = beta2 * v[i] + (1.0 - beta2) * g[i] * g[i];
        double h = sqrt(v[i]) / bc2_sqrt + eps;
        p[i] = p[i] - step_size * m[i] / h;
    }
}

/* TEST MUTANT -- not the method.  The "decay-after" ordering that [BNB]
 * removes: p <- (p - step_size*update)*(1 - lr*wd).  It exists only so the
 * tests can show that they discriminate between the two orderings.        */
void mutant_adamw_decay_after_step(int64_t n, double *p, double *m, double *v,
                                   const double *g, double lr, double beta1,
                                   double beta2, double eps, double wd,
                                   int64_t t)
{
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    for (int64_t i = 0; i < n; ++i) {
        m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];
        v[i] = beta2 * v[i] + (1.0 - beta2) * g[i] * g[i];
        double h = sqrt(v[i]) / sqrt(bc2) + eps;
        p[i] = (p[i] - (lr / bc1) * m[i] / h) * (1.0 - lr * wd);
    }
}

/* ------------------------------------------------------------------------ */
/* AdEMAMix.  [BNB] PR description: same decay ordering as AdamW; PR body
 * "Why the current tests do not catch it": on a fresh step AdEMAMix mixes in
 * alpha*(1-beta3)*g on top of AdamW's -lr*g/(|g|+eps), i.e. the slow EMA m2
 * carries no bias correction.  alpha and beta3 are constants (the pages
 * describe no warm-up schedule for them).                                 */
void oracle_ademamix_step(int64_t n, double *p, double *m1, double *m2,
                          double *nu, const double *g, double lr, double beta1,
                          double beta2, double beta3, double alpha, double eps,
                          double wd, int64_t t)
{
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    for (int64_t i = 0; i < n; ++i) {
        p[i] = p[i] * (1.0 - lr * wd);
        m1[i] = beta1 * m1[i] + (1.0 - beta1) * g[i];
        m2[i] = beta3 * m2[i] + (1.0 - beta3) * g[i];
        nu[i] = beta2 * nu[i] + (1.0 - beta2) * g[i] * g[i];
        double h = sqrt(nu[i]) / sqrt(bc2) + eps;
        p[i] = p[i] - lr * (m1[i] / bc1 + alpha * m2[i]) / h;
    }
}

/* ------------------------------------------------------------------------ */
/* Adam-mini, one tensor whose second moment is shared per block.
 * [MINI] AdamWMini: for q/k weights the gradient is viewed as rows of
 * head_numel = dim*dim/n_heads elements and each row keeps one vmean,
 * updated with the row mean of g*g; every other non-embedding tensor keeps a
 * single vmean updated with sum(g*g)/numel (block = whole tensor).  Decay
 * p*(1-lr*wd) comes first, m is an EMA of g, h = sqrt(vmean)/sqrt(bc2)+eps,
 * p <- p - lr*(m/bc1)/h.  The mean is summed in index order.
 * n must be a multiple of block; V holds n/block entries.                 */
void oracle_adam_mini_step(int64_t n, int64_t block, double *p, double *m,
                           double *V, const double *g, double lr, double beta1,
                           double beta2, double eps, double wd, int64_t t)
{
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    int64_t nb = n / block;
    for (int64_t j = 0; j < nb; ++j) {
        const double *gj = g + j * block;
        double s = 0.0;
        for (int64_t i = 0; i < block; ++i)
            s += gj[i] * gj[i];
        V[j] = beta2 * V[j] + (1.0 - beta2) * (s / (double)block);
        double h = sqrt(V[j]) / sqrt(bc2) + eps;
        for (int64_t i = j * block; i < (j + 1) * block; ++i) {
            p[i] = p[i] * (1.0 - lr * wd);
            m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];
            p[i] = p[i] - lr * (m[i] / bc1) / h;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* AMP: a step is skipped when any gradient element is NaN or +-Inf.
 * [LTN] analysis: the fused optimizer receives grad_scale and found_inf and
 * unscales / skips inside the step.  Returns 1 if any x[i] is not finite. */
int oracle_any_nonfinite(int64_t n, const double *x)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i]))
            return 1;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gradient clipping inside the fused step.  [LTN] analysis: unscale_ runs
 * before step only so that gradients can be clipped, and with a fused
 * optimizer that unscales inside its step an explicit unscale_ is applied a
 * second time.  Reading used here: clipping is folded into the step's
 * unscale factor.  The global L2 norm is taken over every gradient of the
 * step after unscaling, norm = sqrt(sum (G s)^2), summed in index order; the
 * clip coefficient is min(1, max_norm / (norm + 1e-6)) (the form of
 * torch.nn.utils.clip_grad_norm_), and 1 when max_norm <= 0 or is +inf, or
 * when the norm is not finite (the step is skipped then).                  */
double oracle_sumsq(int64_t n, const double *x)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += x[i] * x[i];
    return s;
}

double oracle_clip_coef(double norm, double max_norm)
{
    if (!(max_norm > 0.0) || isinf(max_norm) || !isfinite(norm))
        return 1.0;
    double c = max_norm / (norm + 1e-6);
    return c < 1.0 ? c : 1.0;
}

/* Dynamic loss scale, updated once per loop iteration after the step.
 * [LTN] shows scaler.update() closing the loop; the pages give no rule.
 * Reading used here (GradScaler's documented behaviour): a step with a
 * non-finite gradient multiplies the scale by backoff and resets the count
 * of clean steps; otherwise the count grows, and when it reaches interval
 * the scale is multiplied by growth (kept only if the product is finite)
 * and the count restarts.  The scale is stored as a float: each product is
 * taken in double and rounded once.                                         */
void oracle_scaler_update(float *scale, int32_t *tracker, int found_inf, double growth,
                          double backoff, int32_t interval)
{
    if (found_inf) {
        *scale = (float)((double)*scale * backoff);
        *tracker = 0;
        return;
    }
    int32_t k = *tracker + 1;
    if (k >= interval) {
        float grown = (float)((double)*scale * growth);
        if (isfinite(grown))
            *scale = grown;
        *tracker = 0;
    } else {
        *tracker = k;
    }
}

/* ------------------------------------------------------------------------ */
/* Cosine learning-rate schedule evaluated once per loop iteration k and kept
 * as a float scalar.  [AO]: the lr is recomputed every step from a schedule
 * (cosine in the benchmark the issue cites) and should stay a scalar tensor
 * updated in place.  The pages give no formula; this is plain cosine decay
 * from lr_max at k = 0 to lr_min at k = K, held at lr_min afterwards,
 * evaluated in double and rounded once to float.                          */
float oracle_cosine_lr(int64_t k, int64_t K, double lr_max, double lr_min)
{
    if (k > K)
        k = K;
    double x = (double)k / (double)K;
    double lr = lr_min + (lr_max - lr_min) * 0.5 * (1.0 + cos(M_PI * x));
    return (float)lr;
}

/* ------------------------------------------------------------------------ */
/* BF16 model parameter + int16 remainder.  [TE] description: store the
 * trailing 16 bits and rebuild the FP32 master from (BF16 param, remainder).
 * The page gives no encoding.  Reading used here, stated arithmetically on
 * the 32-bit pattern u of the master: r is the balanced residue of u modulo
 * 2^16, r in [-2^15, 2^15), and b = (u - r) / 2^16 modulo 2^16; hence
 * u = b*2^16 + r (mod 2^32).  b is the master rounded to the nearest bf16
 * pattern with ties away from zero.                                      */
void oracle_remainder_split(int64_t n, const uint32_t *u, uint16_t *b,
                            int16_t *r)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t x = (int64_t)u[i];
        int64_t res = ((x + 32768) % 65536) - 32768; /* in [-32768, 32767] */
        int64_t hi = ((x - res) % 4294967296LL + 4294967296LL) % 4294967296LL;
        b[i] = (uint16_t)(hi / 65536);
        r[i] = (int16_t)res;
    }
}

void oracle_remainder_reconstruct(int64_t n, const uint16_t *b,
                                  const int16_t *r, uint32_t *u)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t x = (int64_t)b[i] * 65536 + (int64_t)r[i];
        x = (x % 4294967296LL + 4294967296LL) % 4294967296LL;
        u[i] = (uint32_t)x;
    }
}

/* Exhaustive check over every 32-bit pattern: reconstruct(split(u)) == u.
 * Returns the number of patterns that fail (0 expected).                  */
int64_t oracle_remainder_exhaustive(void)
{
    int64_t bad = 0;
    uint32_t chunk[4096];
    uint16_t b[4096];
    int16_t r[4096];
    uint32_t back[4096];
    for (uint64_t base = 0; base < 4294967296ULL; base += 4096) {
        for (int i = 0; i < 4096; ++i)
            chunk[i] = (uint32_t)(base + (uint64_t)i);
        oracle_remainder_split(4096, chunk, b, r);
        oracle_remainder_reconstruct(4096, b, r, back);
        for (int i = 0; i < 4096; ++i)
            bad += (back[i] != chunk[i]);
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Dynamic quantization map for blockwise 8-bit / 4-bit optimizer states.
 * The pages name blockwise 8-bit 2-state kernels ([BNB]) and 4-bit states
 * ([AO]) but give no code values.  Definition used here, after the dynamic
 * (decimal exponent + linear fraction) map of Dettmers et al.,
 * arXiv:2110.02861, with b magnitude bits:
 *   M = sorted({0} U {10^-e * (0.1 + 0.9*(k+1)/2^(b-1-e)) :
 *                     e = 0..b-1, k = 0..2^(b-1-e)-1}),
 * each value evaluated as the double expression
 *   pow(10.0, -e) * (0.1 + 0.9 * (k + 1) / 2^(b-1-e))
 * and rounded once to float.  |M| = 2^b, M[0] = 0, M[2^b-1] = 1.
 * Writes the 2^b sorted magnitudes to M; returns the count.               */
int oracle_dynamic_map(int b, float *M)
{
    int cnt = 0;
    M[cnt++] = 0.0f;
    for (int e = 0; e < b; ++e) {
        int nk = 1 << (b - 1 - e);
        for (int k = 0; k < nk; ++k) {
            double val = pow(10.0, -(double)e) *
                         (0.1 + 0.9 * (double)(k + 1) / (double)nk);
            M[cnt++] = (float)val;
        }
    }
    /* insertion sort, ascending */
    for (int i = 1; i < cnt; ++i) {
        float key = M[i];
        int j = i - 1;
        while (j >= 0 && M[j] > key) {
            M[j + 1] = M[j];
            --j;
        }
        M[j + 1] = key;
    }
    return cnt;
}

/* Decision thresholds: T[j] = fl32((M[j-1] + M[j]) / 2) for j >= 1; T[0] is
 * unused (set to 0).  A normalised magnitude a maps to the largest j with
 * T[j] <= a (ties go to the larger code), or to 0.                        */
void oracle_thresholds(int count, const float *M, float *T)
{
    T[0] = 0.0f;
    for (int j = 1; j < count; ++j)
        T[j] = (float)(((double)M[j - 1] + (double)M[j]) / 2.0);
}

static int nearest_index(int count, const float *T, float a)
{
    int idx = 0;
    for (int j = 1; j < count; ++j)
        if (T[j] <= a)
            idx = j;
    return idx;
}

/* Quantize x blockwise (blocks of `block` consecutive elements from element
 * 0; the last block may be partial).  Per block: A = max|x| (stored as the
 * block's absmax), r = fl32(1/A), a = fl32(|x|*r), code index = threshold
 * rule.  Signed maps put the sign in bit b (b = magnitude bits) and use sign
 * 0 for index 0.  If A == 0 every code is 0.  One code per byte in `codes`
 * (4-bit packing is a separate step).                                     */
void oracle_quantize(int64_t n, int64_t block, int b, int is_signed,
                     const float *x, const float *T, uint8_t *codes,
                     float *absmax)
{
    int count = 1 << b;
    for (int64_t s = 0, blk = 0; s < n; s += block, ++blk) {
        int64_t e = s + block < n ? s + block : n;
        float A = 0.0f;
        for (int64_t i = s; i < e; ++i)
            if (fabsf(x[i]) > A)
                A = fabsf(x[i]);
        absmax[blk] = A;
        if (A == 0.0f) {
            for (int64_t i = s; i < e; ++i)
                codes[i] = 0;
            continue;
        }
        float r = (float)(1.0 / (double)A);
        for (int64_t i = s; i < e; ++i) {
            float a = (float)((double)fabsf(x[i]) * (double)r);
            int idx = nearest_index(count, T, a);
            int sign = (is_signed && x[i] < 0.0f && idx > 0) ? 1 : 0;
            codes[i] = (uint8_t)((sign << b) | idx);
        }
    }
}

/* Dequantize: x = fl32(+-M[idx] * A).                                     */
void oracle_dequantize(int64_t n, int64_t block, int b, int is_signed,
                       const uint8_t *codes, const float *M,
                       const float *absmax, float *x)
{
    for (int64_t i = 0; i < n; ++i) {
        int c = codes[i];
        int idx = is_signed ? (c & ((1 << b) - 1)) : c;
        double mag = (double)M[idx] * (double)absmax[i / block];
        x[i] = (float)((is_signed && (c >> b) & 1) ? -mag : mag);
    }
}

/* 4-bit packing: element 2i in the low nibble of byte i, 2i+1 in the high. */
void oracle_pack_nibbles(int64_t n, const uint8_t *codes, uint8_t *packed)
{
    for (int64_t i = 0; i < (n + 1) / 2; ++i) {
        uint8_t lo = codes[2 * i] & 15;
        uint8_t hi = (2 * i + 1 < n) ? (codes[2 * i + 1] & 15) : 0;
        packed[i] = (uint8_t)(lo | (hi << 4));
    }
}

void oracle_unpack_nibbles(int64_t n, const uint8_t *packed, uint8_t *codes)
{
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (i & 1) ? (packed[i / 2] >> 4) : (packed[i / 2] & 15);
}

/* ------------------------------------------------------------------------ */
/* Blockwise-quantized 2-state AdamW step.  [BNB] PR description: the
 * 2-state branch of the blockwise 8-bit kernel takes the same Algorithm 2
 * decay ordering; PR body: a fresh optimizer's zero state quantizes exactly
 * and the first update has the closed form -lr*g/(|g|+eps).
 * States: m with the signed map, v with the unsigned map; codes unpacked
 * (one per byte), absmax per block.  The state recipe is fp32-faithful:
 *   m = fl32(fl32(b1*m~) + fl32(c1*g)),  v = fl32(fl32(b2*v~) + fl32(c2*fl32(g*g)))
 * with b1 = fl32(beta1), c1 = fl32(1-beta1) (likewise for beta2) and m~, v~
 * the dequantized previous states.  The parameter update uses these fp32 m, v
 * in double, exactly as oracle_adamw_step does; then m and v are requantized.
 * g holds the float gradients (already unscaled).                          */
void oracle_blockwise_step(int64_t n, int64_t block, int bits, double *p,
                           const float *g, uint8_t *qm, uint8_t *qv, float *am,
                           float *av, double lr, double beta1, double beta2,
                           double eps, double wd, int64_t t, float *scratch_m,
                           float *scratch_v)
{
    int bm = bits - 1, bv = bits; /* magnitude bits: signed m, unsigned v */
    float Mm[256], Tm[256], Mv[256], Tv[256];
    oracle_dynamic_map(bm, Mm);
    oracle_thresholds(1 << bm, Mm, Tm);
    oracle_dynamic_map(bv, Mv);
    oracle_thresholds(1 << bv, Mv, Tv);

    double b1 = F32(beta1), c1 = F32(1.0 - beta1);
    double b2 = F32(beta2), c2 = F32(1.0 - beta2);
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);

    oracle_dequantize(n, block, bm, 1, qm, Mm, am, scratch_m);
    oracle_dequantize(n, block, bv, 0, qv, Mv, av, scratch_v);
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)g[i];
        double mi = F32(F32(b1 * (double)scratch_m[i]) + F32(c1 * gi));
        double vi = F32(F32(b2 * (double)scratch_v[i]) + F32(c2 * F32(gi * gi)));
        scratch_m[i] = (float)mi;
        scratch_v[i] = (float)vi;
        p[i] = p[i] * (1.0 - lr * wd);
        double h = sqrt(vi) / sqrt(bc2) + eps;
        p[i] = p[i] - (lr / bc1) * mi / h;
    }
    oracle_quantize(n, block, bm, 1, scratch_m, Tm, qm, am);
    oracle_quantize(n, block, bv, 0, scratch_v, Tv, qv, av);
}

/* ------------------------------------------------------------------------ */
/* Blockwise-quantized AdEMAMix (three states).  [BNB] PR description and the
 * review's confirmation of the 8-bit blockwise site: the 2-state blockwise
 * kernel has an AdEMAMix branch, which takes the same Algorithm 2 decay
 * order; PR body: on a fresh step AdEMAMix mixes in alpha*(1-beta3)*g.
 * States: m1 and m2 with the signed map, nu with the unsigned map, each with
 * its own absmax per block.  fp32-faithful state recipe as in
 * oracle_blockwise_step, with m2 = fl32(fl32(b3*m2~) + fl32(c3*g)),
 * b3 = fl32(beta3), c3 = fl32(1-beta3).  The parameter update uses the fp32
 * states in double: p <- p(1-lr wd) - lr (m1/bc1 + alpha m2)/h, m2 not
 * bias-corrected, as oracle_ademamix_step.  Then all three requantize.      */
void oracle_blockwise_ademamix_step(int64_t n, int64_t block, int bits, double *p,
                                    const float *g, uint8_t *qm, uint8_t *qm2, uint8_t *qv,
                                    float *am, float *am2, float *av, double lr, double beta1,
                                    double beta2, double beta3, double alpha, double eps,
                                    double wd, int64_t t, float *scratch_m, float *scratch_m2,
                                    float *scratch_v)
{
    int bm = bits - 1, bv = bits;
    float Mm[256], Tm[256], Mv[256], Tv[256];
    oracle_dynamic_map(bm, Mm);
    oracle_thresholds(1 << bm, Mm, Tm);
    oracle_dynamic_map(bv, Mv);
    oracle_thresholds(1 << bv, Mv, Tv);

    double b1 = F32(beta1), c1 = F32(1.0 - beta1);
    double b2 = F32(beta2), c2 = F32(1.0 - beta2);
    double b3 = F32(beta3), c3 = F32(1.0 - beta3);
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);

    oracle_dequantize(n, block, bm, 1, qm, Mm, am, scratch_m);
    oracle_dequantize(n, block, bm, 1, qm2, Mm, am2, scratch_m2);
    oracle_dequantize(n, block, bv, 0, qv, Mv, av, scratch_v);
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)g[i];
        double mi = F32(F32(b1 * (double)scratch_m[i]) + F32(c1 * gi));
        double m2i = F32(F32(b3 * (double)scratch_m2[i]) + F32(c3 * gi));
        double vi = F32(F32(b2 * (double)scratch_v[i]) + F32(c2 * F32(gi * gi)));
        scratch_m[i] = (float)mi;
        scratch_m2[i] = (float)m2i;
        scratch_v[i] = (float)vi;
        p[i] = p[i] * (1.0 - lr * wd);
        double h = sqrt(vi) / sqrt(bc2) + eps;
        p[i] = p[i] - lr * (mi / bc1 + alpha * m2i) / h;
    }
    oracle_quantize(n, block, bm, 1, scratch_m, Tm, qm, am);
    oracle_quantize(n, block, bm, 1, scratch_m2, Tm, qm2, am2);
    oracle_quantize(n, block, bv, 0, scratch_v, Tv, qv, av);
}

/* ------------------------------------------------------------------------ */
/* Lion.  [BNB] PR review on the 1-state kernels: Lion applies decoupled
 * decay to the parameter before its sign update (the ordering the PR
 * establishes for the 2-state kernels).  The pages give no formula; the
 * update is Lion's published one (Chen et al., arXiv:2302.06675):
 *   c = b1 m + c1 g;  p <- p (1 - lr wd) - lr sign(c);  m <- b2 m + c2 g
 * sign(0) = 0.  The sign is an integer decision taken from c, so c and the
 * state m follow the fp32 recipe of the kernel (fp32-faithful):
 *   c = fl32(fl32(b1 m) + fl32(c1 g)),  m = fl32(fl32(b2 m) + fl32(c2 g)),
 * with b1 = fl32(beta1), c1 = fl32(1 - beta1) (likewise beta2) and g the
 * float gradient; the parameter update is taken in double.                  */
void oracle_lion_step(int64_t n, double *p, float *m, const float *g, double lr, double beta1,
                      double beta2, double wd)
{
    double b1 = F32(beta1), c1 = F32(1.0 - beta1);
    double b2 = F32(beta2), c2 = F32(1.0 - beta2);
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)g[i];
        double c = F32(F32(b1 * (double)m[i]) + F32(c1 * gi));
        double sg = c > 0.0 ? 1.0 : (c < 0.0 ? -1.0 : 0.0);
        p[i] = p[i] * (1.0 - lr * wd);
        p[i] = p[i] - lr * sg;
        m[i] = (float)F32(F32(b2 * (double)m[i]) + F32(c2 * gi));
    }
}

/* ------------------------------------------------------------------------ */
/* LAMB, one tensor (the trust ratio is per tensor).  [BNB] PR description:
 * LAMB shares the Adam kernels and their decay ordering.  The pages give no
 * formula; the update is LAMB's published one (You et al., arXiv:1904.00962,
 * Algorithm 2), with Adam's direction in the form used above:
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
 *   r = (m/bc1) / (sqrt(v)/sqrt(bc2) + eps);  u = r + wd p
 *   p <- p - lr (|p| / |u|) u        (L2 norms over the tensor, previous p)
 * with the trust ratio |p|/|u| taken as 1 when either norm is 0.  Norms are
 * summed in index order.                                                     */
void oracle_lamb_step(int64_t n, double *p, double *m, double *v, const double *g, double lr,
                      double beta1, double beta2, double eps, double wd, int64_t t, double *u)
{
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    double pn = 0.0, un = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];
        v[i] = beta2 * v[i] + (1.0 - beta2) * g[i] * g[i];
        double r = (m[i] / bc1) / (sqrt(v[i]) / sqrt(bc2) + eps);
        u[i] = r + wd * p[i];
        pn += p[i] * p[i];
        un += u[i] * u[i];
    }
    double trust = (pn > 0.0 && un > 0.0) ? sqrt(pn) / sqrt(un) : 1.0;
    for (int64_t i = 0; i < n; ++i)
        p[i] = p[i] - lr * trust * u[i];
}

/* ------------------------------------------------------------------------ */
/* Low-precision model copy of an fp32 master.  [TE] page, review thread:
 * with master weights the model parameter is BF16 or FP16 and the FP32
 * master is kept beside it (the remainder feature applies to BF16 only);
 * after the step the model copy is the master rounded to the model dtype.
 * Rounding is to nearest, ties to even (the IEEE default), written here from
 * the bit patterns:
 *   bf16: keep the top 16 bits of the fp32 pattern, rounded on the low 16;
 *   fp16: 1 sign, 5 exponent (bias 15), 10 fraction bits; overflow to +-inf,
 *         gradual underflow to subnormals and zero.
 * NaN inputs map to a quiet NaN of the same sign.                          */
uint16_t oracle_f32_to_bf16_rne(uint32_t u)
{
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lo = u & 0xFFFFu, hi = u >> 16;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u; /* a carry into the exponent is the correct rounding */
    return (uint16_t)hi;
}

uint16_t oracle_f32_to_f16_rne(uint32_t u)
{
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ex = (u >> 23) & 0xFFu, fr = u & 0x007FFFFFu;
    if (ex == 0xFFu)
        return (uint16_t)(sign | 0x7C00u | (fr ? 0x0200u : 0u));
    /* value = 1.fr * 2^(ex-127) for normal fp32; fp32 subnormals are far
     * below the fp16 range and round to zero */
    if (ex == 0)
        return sign;
    int e = (int)ex - 127 + 15; /* fp16 biased exponent */
    uint32_t mant = fr | 0x00800000u; /* 24-bit significand */
    if (e >= 31)
        return (uint16_t)(sign | 0x7C00u);
    int shift; /* bits to drop from the 24-bit significand */
    uint32_t out_exp;
    if (e >= 1) {
        shift = 13;
        out_exp = (uint32_t)e;
    } else {
        shift = 14 - e; /* subnormal: the significand shifts further right */
        out_exp = 0;
        if (shift > 24)
            return sign;
    }
    uint32_t kept = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u)))
        kept += 1u;
    /* normal: kept holds the implicit bit at 2^10; subnormal: no implicit bit.
     * A carry out of the fraction moves into the exponent field naturally. */
    uint32_t bits = (out_exp ? ((out_exp << 10) + (kept - 0x400u)) : kept);
    if (bits >= 0x7C00u)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | bits);
}

void oracle_round_model_copy(int64_t n, int to_half, const uint32_t *master, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = to_half ? oracle_f32_to_f16_rne(master[i]) : oracle_f32_to_bf16_rne(master[i]);
}

/* ------------------------------------------------------------------------ */
/* AdamW with per-tensor scaled 16-bit moments.  [TE] review thread shows the
 * state scaling of the fused optimizer: a state kept in a low-precision
 * dtype with a per-tensor scale, the fp32 value being stored * scale, and a
 * new state written as (fp32 value * rscale) copied into the low-precision
 * tensor.  The page shows no rule for the scale; reading used here: fp16
 * states take scale = fl32(amax / 65504) over the tensor's new state (1 if
 * the state is all zero) and rscale = fl32(1 / scale), so the largest
 * magnitude lands on the top of the fp16 range; bf16 states keep scale 1
 * (bf16 has the range of fp32).  One tensor, fp32-faithful state recipe:
 *   m~ = fl32(h(qm) * sm), v~ = fl32(h(qv) * sv)      (h = 16-bit value)
 *   m = fl32(fl32(b1 m~) + fl32(c1 g)),  v = fl32(fl32(b2 v~) + fl32(c2 fl32(g g)))
 *   p <- p (1 - lr wd) - (lr/bc1) m / (sqrt(v)/sqrt(bc2) + eps)   (double)
 *   sm' = scale(max |m|), qm = rne16(fl32(m * fl32(1/sm'))), likewise v.
 * half = 1: fp16 states; 0: bf16 states.  qm, qv hold 16-bit patterns.    */
static double h16_to_double(uint16_t b, int half)
{
    if (!half) {
        uint32_t u = (uint32_t)b << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    int s = (b >> 15) & 1, e = (b >> 10) & 31, f = b & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 1024), e - 25);
    return s ? -v : v;
}

static uint16_t f32_to_16(float x, int half)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return half ? oracle_f32_to_f16_rne(u) : oracle_f32_to_bf16_rne(u);
}

void oracle_adamw_scaled_step(int64_t n, int half, double *p, uint16_t *qm, uint16_t *qv,
                              float *sm, float *sv, const float *g, double lr, double beta1,
                              double beta2, double eps, double wd, int64_t t, float *scratch_m,
                              float *scratch_v)
{
    double b1 = F32(beta1), c1 = F32(1.0 - beta1);
    double b2 = F32(beta2), c2 = F32(1.0 - beta2);
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    double am = 0.0, av = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)g[i];
        double mt = F32(h16_to_double(qm[i], half) * (double)*sm);
        double vt = F32(h16_to_double(qv[i], half) * (double)*sv);
        double mi = F32(F32(b1 * mt) + F32(c1 * gi));
        double vi = F32(F32(b2 * vt) + F32(c2 * F32(gi * gi)));
        scratch_m[i] = (float)mi;
        scratch_v[i] = (float)vi;
        if (fabs(mi) > am) am = fabs(mi);
        if (fabs(vi) > av) av = fabs(vi);
        p[i] = p[i] * (1.0 - lr * wd);
        double h = sqrt(vi) / sqrt(bc2) + eps;
        p[i] = p[i] - (lr / bc1) * mi / h;
    }
    float nsm = 1.0f, nsv = 1.0f;
    if (half) {
        if (am > 0.0) nsm = (float)(am / 65504.0);
        if (av > 0.0) nsv = (float)(av / 65504.0);
    }
    float rm = (float)(1.0 / (double)nsm), rv = (float)(1.0 / (double)nsv);
    for (int64_t i = 0; i < n; ++i) {
        qm[i] = f32_to_16((float)((double)scratch_m[i] * (double)rm), half);
        qv[i] = f32_to_16((float)((double)scratch_v[i] * (double)rv), half);
    }
    *sm = nsm;
    *sv = nsv;
}
