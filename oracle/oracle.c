/*
 * CPU oracle for INT8-QK / BF16-PV flash attention (forward only).
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The GPU library never
 * links, includes or calls it, and it shares no code, header or table with
 * the GPU path.
 *
 * It is a plain, slow, obviously correct statement of what the method
 * computes, following the pages' steps in order:
 *   1. mean of K over the valid keys                       (kmean)
 *   2. per-token symmetric int8 quantization of Q and K-mu  (quantize_rows)
 *   3. the centring term q.mu used to report the true LSE  (qmu)
 *   4. int8 scores into int32                              (scores_i32)
 *   5. dequantized logits + bias/mask, softmax, PV, LSE    (attn)
 *   6. exact two-way merge of partial softmaxes by LSE     (lse_merge)
 *   7. tile mask -> ascending key-tile list + count        (blockmask_to_index)
 * Everything from the logits on is computed in fp64 with a two-pass
 * (max, then exp-sum) softmax; nothing is blocked, fused or reordered.
 *
 * Sources (the web pages this method is described on):
 *  [FV]  FastVideo API docs, "minimax_h3_sparse_int8": the module description
 *        and the listing of sparse_sm89_attention (K mean over the valid
 *        tokens, per-token Q/K scales, K centring, tile-64 mask + validity
 *        vector, per-(head,channel) V scale, BF16 PV).
 *  [CK177] comfy-kitchen issue #177 "int8_attention: masked path costs ~1.8x
 *        unmasked, and a request for optional return_lse": per-key additive
 *        bias [1,1,1,K] in natural-log units; the core/skirt split merged
 *        exactly by LSE ("Question 2").
 *  [MK3] model-kernels issue #3 "[attention-int8] Multiple build issues and
 *        numerical accuracy problem": symmetric [-127,127] range, one scale
 *        per K row instead of independently rescaled tiles.
 *  [FLY] ROCm/FlyDSL PR #886 "Add optional forward LSE output": LSE is fp32
 *        [B,H,Sq], natural log, includes the softmax scale, -inf for fully
 *        masked rows; split-K combine from the combined max and denominator.
 *
 * Readings where the pages leave a step open (each is also a test):
 *  R1 the K mean is the exact sum over valid keys, rounded once to fp64,
 *     divided by n in fp64 and rounded to fp32; n = max(1, Sk), or
 *     max(1, sum vbs) when a validity vector is given (the pages clamp the
 *     valid count to 1; the same clamp gives an empty K the mean 0).  The exact sum is accumulated in
 *     __float128, which is exact for bf16/fp16 data whose bit span stays
 *     below 113 bits (always for fp16; bf16 within a 2^+-40 magnitude band).
 *  R2 quantizer: a = max|x|; rows with a < 127*FLT_MIN (the scale would be
 *     subnormal) become all-zero with scale 0; otherwise scale = fp32(a/127),
 *     inv = fp32(127/a), q = clamp(rint_half_even(fp32(x*inv)), -127, 127).
 *  R3 pad rows (j mod 64 >= vbs[j/64]) of Q and K quantize to 0 with scale 0
 *     and do not enter the mean.
 *  R4 only K is centred; x - mu is one fp32 subtraction.
 *  R5 bias is in natural-log units and is added after the softmax scale.
 *  R6 LSE is that of the uncentred scores: the centring shift
 *     -sm_scale*(q.mu) is added back as +sm_scale*qmu.
 *  R7 a fully excluded row gives O = 0 and LSE = -inf.
 *  R8 grouped-query attention: H query heads share Hkv K/V heads (H a
 *     multiple of Hkv), query head h reading K/V head h / (H/Hkv) (runs of
 *     consecutive query heads per K/V head); K mean, K codes and the V scale
 *     belong to the K/V head, and q.mu of a query row uses its K/V head's mean.
 *  R9 non-finite inputs: a row of Q or of K - mu holding a NaN or +-inf
 *     quantizes to codes 0 with scale NaN (its centring term is NaN too),
 *     and a K channel whose valid keys hold a NaN or +-inf has mean NaN, so
 *     every centred K row of that head is such a row. Scores with such a
 *     row are NaN.
 *
 * Parity pins (tests/test_oracle_*.py): hand-worked quantization examples
 * (tests/golden/), exact-rational means, brute-force integer scores, the
 * library SDPA/logsumexp in fp64 for no-quant attention, closed forms
 * (Sk = 1, Q = 0, constant bias, fully masked rows), shift invariance,
 * broadcast == expanded bias, sparse == dense with -inf bias, split + merge
 * == unsplit.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_BF16 = 1, OR_FP16 = 2, OR_FP32 = 3 };

/* ---- element decoding (exact) ------------------------------------------ */

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float fp16_to_float(uint16_t h) {
    int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);              /* subnormal / zero */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

static float load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == OR_BF16) return bf16_to_float(((const uint16_t*)base)[idx]);
    if (dtype == OR_FP16) return fp16_to_float(((const uint16_t*)base)[idx]);
    return ((const float*)base)[idx];
}

static int is_pad_row(const int32_t* vbs, int64_t j) {
    return vbs != NULL && (int32_t)(j % 64) >= vbs[j / 64];
}

/* ---- step 1: K mean [FV listing: sum over the sequence / sum(vbs).clamp_min(1)] ---- */

/* k: contiguous [B,H,S,D]; mean: [B,H,D] fp32. vbs may be NULL (then n = S). */
void oracle_kmean(const void* k, int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                  const int32_t* vbs, float* mean) {
    int64_t n = S;
    if (vbs) {
        n = 0;
        for (int64_t t = 0; t < (S + 63) / 64; ++t) n += vbs[t];
    }
    if (n < 1) n = 1;   /* reading R1: the count is clamped to 1, so an empty K has mean 0 */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t c = 0; c < D; ++c) {
            __float128 acc = 0;
            int finite = 1;
            for (int64_t j = 0; j < S; ++j) {
                if (is_pad_row(vbs, j)) continue;
                float x = load_elem(k, dtype, (bh * S + j) * D + c);
                if (!isfinite(x)) finite = 0;             /* reading R9 */
                acc += (__float128)x;
            }
            double sum = (double)acc;                 /* exact sum rounded once */
            mean[bh * D + c] = finite ? (float)(sum / (double)n) : NAN;
        }
}

/* ---- step 2: per-token symmetric int8 [FV description; MK3 symmetric range] ---- */

static void quantize_one_row(const float* x, int64_t D, int8_t* q, float* scale) {
    float a = 0.0f;
    for (int64_t c = 0; c < D; ++c) {
        if (!isfinite(x[c])) {                           /* reading R9 */
            for (int64_t d = 0; d < D; ++d) q[d] = 0;
            *scale = NAN;
            return;
        }
        float m = fabsf(x[c]);
        if (m > a) a = m;
    }
    if (a < 127.0f * FLT_MIN) {                          /* reading R2 */
        for (int64_t c = 0; c < D; ++c) q[c] = 0;
        *scale = 0.0f;
        return;
    }
    float s = a / 127.0f;
    float inv = 127.0f / a;
    for (int64_t c = 0; c < D; ++c) {
        float y = rintf(x[c] * inv);                      /* round half to even */
        if (y > 127.0f) y = 127.0f;
        if (y < -127.0f) y = -127.0f;
        q[c] = (int8_t)y;
    }
    *scale = s;
}

/* x: contiguous [B,H,S,D] (bf16/fp16/fp32); mean: [B,H,D] or NULL (no centring);
 * vbs: NULL or ceil(S/64) entries; q: [B,H,S,D] int8; scale: [B,H,S] fp32. */
void oracle_quantize_rows(const void* x, int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                          const float* mean, const int32_t* vbs, int8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < B * H * S; ++r) {
        int64_t bh = r / S, j = r % S;
        float* row = (float*)malloc(sizeof(float) * (size_t)D);
        if (is_pad_row(vbs, j)) {                         /* reading R3 */
            memset(q + r * D, 0, (size_t)D);
            scale[r] = 0.0f;
        } else {
            for (int64_t c = 0; c < D; ++c) {
                float v = load_elem(x, dtype, r * D + c);
                row[c] = mean ? v - mean[bh * D + c] : v;  /* reading R4: one fp32 subtraction */
            }
            quantize_one_row(row, D, q + r * D, scale + r);
        }
        free(row);
    }
}

/* ---- step 3: centring term qmu_i = sum_c q_ic * mu_c (fp64) [reading R6] ---- */

/* qx: [B,H,S,D]; mean: [B,Hkv,D], the K mean of the K/V head query head h
 * reads (h / (H/Hkv), reading R8); qmu: [B,H,S]. */
void oracle_qmu(const void* qx, int dtype, int64_t B, int64_t H, int64_t Hkv, int64_t S, int64_t D,
                const float* mean, const int32_t* vbs, double* qmu) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < B * H * S; ++r) {
        int64_t bh = r / S, j = r % S;
        int64_t kvh = (bh / H) * Hkv + (bh % H) / (H / Hkv);
        double acc = 0.0;
        if (!is_pad_row(vbs, j))
            for (int64_t c = 0; c < D; ++c) {
                float x = load_elem(qx, dtype, r * D + c);
                if (!isfinite(x)) { acc = NAN; break; }    /* reading R9 */
                acc += (double)x * (double)mean[kvh * D + c];
            }
        qmu[r] = acc;
    }
}

/* ---- step 4: int8 scores into int32 (exact) ---- */

/* q8: [Sq,D], k8: [Sk,D] for one head; s: [Sq,Sk]. */
void oracle_scores_i32(const int8_t* q8, const int8_t* k8, int64_t Sq, int64_t Sk, int64_t D,
                       int32_t* s) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < Sq; ++i)
        for (int64_t j = 0; j < Sk; ++j) {
            int32_t acc = 0;
            for (int64_t c = 0; c < D; ++c) acc += (int32_t)q8[i * D + c] * (int32_t)k8[j * D + c];
            s[i * Sk + j] = acc;
        }
}

/* ---- step 5: logits, softmax, PV, LSE ---- */

/*
 * One call of attention for the rows listed in `rows` (flat indices into
 * [B,H,Sq]; NULL = every row). Scores come either from the quantized
 * operands (q8 != NULL):
 *     s_ij = sm_scale * qs_i * ks_j * S32_ij + bias_ij
 * or, in the no-quant mode used to pin the softmax/PV/LSE steps, from raw
 * fp64 operands (q8 == NULL, qf/kf given):
 *     s_ij = sm_scale * sum_c Q_ic K_jc + bias_ij.
 * A key is excluded (s = -inf) when it lies outside every segment, when the
 * block mask drops its tile or it is a pad key of its tile, when its
 * bias is -inf, or (causal, self-attention: Sq = Sk) when j > i.
 *
 * Query head h reads K/V head h / (H/Hkv) (grouped-query attention; Hkv = H
 * is plain multi-head attention; reading R8).
 *
 * Layouts (all contiguous except the bias, which takes element strides so
 * that a [1,1,1,K] stride-0 broadcast and its [B,H,Q,K] expansion are both
 * expressible):
 *   q8 [B,H,Sq,D] int8, qs [B,H,Sq], k8 [B,Hkv,Sk,D] int8, ks [B,Hkv,Sk]
 *   qf [B,H,Sq,D] f64, kf [B,Hkv,Sk,D] f64 (no-quant mode)
 *   v  [B,Hkv,Sk,D] of v_dtype
 *   bias (nullable) of bias_dtype, element (b,h,i,j) at
 *        b*bsb + h*bsh + i*bsq + j*bsk
 *   mask (nullable) [B,H,Sq/64,Sk/64] uint8, vbs [Sk/64] (nullable)
 *   v_scale (nullable) [Hkv,D] fp32, the scale of the stored V head
 *   seg: nseg pairs (start, len); nseg = 0 means the whole [0, Sk)
 *   qmu (nullable) [B,H,Sq] fp64, added as sm_scale*qmu to the LSE
 *   o [nrows, D] f64, lse [nrows] f64 (row order of `rows`)
 */
void oracle_attn(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                 const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                 const double* qf, const double* kf,
                 const void* v, int v_dtype, float sm_scale,
                 const void* bias, int bias_dtype, int64_t bsb, int64_t bsh, int64_t bsq, int64_t bsk,
                 const uint8_t* mask, const int32_t* vbs,
                 const float* v_scale, int nseg, const int64_t* seg, const double* qmu, int causal,
                 const int64_t* rows, int64_t nrows, double* o, double* lse) {
    int64_t Tq = Sq / 64, Tk = Sk / 64;
    if (rows == NULL) nrows = B * H * Sq;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < nrows; ++n) {
        int64_t r = rows ? rows[n] : n;
        int64_t bh = r / Sq, i = r % Sq, b = bh / H, h = bh % H;
        int64_t hk = h / (H / Hkv), kvh = b * Hkv + hk;   /* the K/V head of query head h */
        double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
        double m = -INFINITY;
        for (int64_t j = 0; j < Sk; ++j) {
            int keep = (nseg == 0);
            for (int g = 0; g < nseg; ++g)
                if (j >= seg[2 * g] && j < seg[2 * g] + seg[2 * g + 1]) keep = 1;
            if (mask) {
                if (!mask[(bh * Tq + i / 64) * Tk + j / 64]) keep = 0;
                if (is_pad_row(vbs, j)) keep = 0;
            }
            if (causal && j > i) keep = 0;
            double sij = -INFINITY;
            if (keep) {
                double dot;
                if (q8) {
                    int32_t acc = 0;
                    for (int64_t c = 0; c < D; ++c)
                        acc += (int32_t)q8[r * D + c] * (int32_t)k8[(kvh * Sk + j) * D + c];
                    dot = (double)qs[r] * (double)ks[kvh * Sk + j] * (double)acc;
                } else {
                    dot = 0.0;
                    for (int64_t c = 0; c < D; ++c) dot += qf[r * D + c] * kf[(kvh * Sk + j) * D + c];
                }
                sij = (double)sm_scale * dot;
                if (bias) sij += (double)load_elem(bias, bias_dtype, b * bsb + h * bsh + i * bsq + j * bsk);
            }
            s[j] = sij;
            if (sij > m) m = sij;
        }
        double* orow = o + n * D;
        for (int64_t c = 0; c < D; ++c) orow[c] = 0.0;
        if (m == -INFINITY) {                               /* reading R7 */
            lse[n] = -INFINITY;
        } else {
            double l = 0.0;
            for (int64_t j = 0; j < Sk; ++j) {
                if (s[j] == -INFINITY) continue;
                double p = exp(s[j] - m);
                l += p;
                for (int64_t c = 0; c < D; ++c)
                    orow[c] += p * (double)load_elem(v, v_dtype, (kvh * Sk + j) * D + c);
            }
            for (int64_t c = 0; c < D; ++c) {
                orow[c] /= l;
                if (v_scale) orow[c] *= (double)v_scale[hk * D + c];
            }
            lse[n] = m + log(l) + (qmu ? (double)sm_scale * qmu[r] : 0.0);
        }
        free(s);
    }
}

/* ---- step 6: exact two-way merge by LSE [CK177 Question 2; FLY split-K combine] ---- */

/* oa, ob, o: [N, D] f64; la, lb, l: [N] f64. */
void oracle_lse_merge(const double* oa, const double* la, const double* ob, const double* lb,
                      int64_t N, int64_t D, double* o, double* l) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double m = la[n] > lb[n] ? la[n] : lb[n];
        if (m == -INFINITY) {
            for (int64_t c = 0; c < D; ++c) o[n * D + c] = 0.0;
            l[n] = -INFINITY;
            continue;
        }
        double wa = exp(la[n] - m), wb = exp(lb[n] - m);
        for (int64_t c = 0; c < D; ++c) o[n * D + c] = (wa * oa[n * D + c] + wb * ob[n * D + c]) / (wa + wb);
        l[n] = m + log(wa + wb);
    }
}

/* ---- step 7: tile mask -> index list [FV listing: map_to_index] ---- */

/* mask [R, Tk] uint8 (R = B*H*Tq rows); index [R, Tk] int32 (first count entries
 * hold the ascending key tiles, the rest are left untouched); count [R]. */
void oracle_blockmask_to_index(const uint8_t* mask, int64_t R, int64_t Tk, int32_t* index, int32_t* count) {
    for (int64_t r = 0; r < R; ++r) {
        int32_t c = 0;
        for (int64_t t = 0; t < Tk; ++t)
            if (mask[r * Tk + t]) index[r * Tk + c++] = (int32_t)t;
        count[r] = c;
    }
}
