/*
 * qfa — INT8-QK / BF16-PV flash attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libqfa.so. Every entry point takes plain pointers and sizes and
 * returns a status code. All tensor pointers are DEVICE pointers owned by the
 * caller; the library allocates no device memory, keeps no state besides a
 * thread-local error message, and never synchronises: kernels are enqueued on
 * the caller's HIP stream (`stream`, a hipStream_t; NULL is the default
 * stream) and results are ready once that stream has completed them.
 *
 * Errors: every argument check runs on the host before any launch, so a call
 * that returns an error has launched nothing and written nothing. A device
 * fault, if one happens, surfaces at the caller's next synchronisation.
 *
 * Logical layouts. A "[B,H,S,D] tensor with strides (sb, sh, ss)" holds
 * element (b,h,s,d) at base + b*sb + h*sh + s*ss + d, strides counted in
 * elements; the channel stride is always 1. This covers contiguous BHSD as
 * well as BSHD-backed views (sb = S*H*D, sh = D, ss = H*D). Quantized Q/K,
 * scales, means, LSE and index arrays are always contiguous.
 *
 * Method (sources are the web pages this operation is described on):
 *  - FastVideo API docs, "minimax_h3_sparse_int8" (module description and the
 *    sparse_sm89_attention listing): K mean over the valid tokens, K centring
 *    as a softmax-invariant shift, per-token int8 Q/K with fp32 scales, int8
 *    QK with fp32 accumulation, BF16 PV, a tile-64 block mask with a per-tile
 *    validity vector, one V scale per (head, channel) applied in the epilogue,
 *    quantized Q/K and the output contiguous BHSD, BSHD views accepted.
 *  - comfy-kitchen issue #177 (measurement table, observations, Question 2):
 *    an additive per-key bias [1,1,1,K] shared by heads and queries, and the
 *    core/skirt split whose partial softmaxes merge exactly through the LSE.
 *  - ROCm/FlyDSL PR #886 ("Public API", "Kernel implementation"): the LSE is
 *    fp32 [B,H,Sq], natural log, includes the softmax scale, is -inf for fully
 *    masked rows, is written once per row, and is requested by passing the
 *    output buffer (a caller-owned lse= out parameter).
 *  - model-kernels issue #3 (maintainer reply): symmetric [-127,127] codes;
 *    every score dequantized with its own row and key scales.
 */
#ifndef QFA_H
#define QFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QFA_OK 0
#define QFA_ERR_INVALID_ARG 1 /* a null/misaligned pointer, bad size, stride or combination */
#define QFA_ERR_UNSUPPORTED 2 /* valid request the library does not implement (e.g. D not in {64,128}) */
#define QFA_ERR_HIP 3         /* the HIP runtime rejected a launch */

/* Element types. */
#define QFA_BF16 1
#define QFA_FP16 2
#define QFA_FP32 3
#define QFA_BOOL 4 /* bytes, nonzero = true (a keep mask) */

#define QFA_MAX_SEGMENTS 4
#define QFA_MAX_SPLITS 64

/* Version of this ABI (major*100 + minor). */
int qfa_version(void);

/* Static description of a status code. */
const char* qfa_status_string(int status);

/* Detail of the last failed call made by this thread ("" if none). */
const char* qfa_last_error(void);

/*
 * qfa_quantize_workspace_bytes — device workspace qfa_quantize_qk needs for
 * the K mean (fp64 partial sums). H is K's head count (Hkv of a
 * grouped-query call). Writes the byte count to *bytes.
 */
int qfa_quantize_workspace_bytes(int64_t B, int64_t H, int64_t Sk, int64_t D, size_t* bytes);

/*
 * qfa_quantize_qk — K mean, K centring and per-token symmetric int8
 * quantization of Q and K (FastVideo "minimax_h3_sparse_int8": module
 * description and the K-mean / _quantize_qk steps of sparse_sm89_attention;
 * model-kernels issue #3: symmetric range).
 *
 * For every row x of Q, and of K - mu when center_k != 0:
 *   a = max_c |x_c|;
 *   a < 127*FLT_MIN  -> codes 0, scale 0;
 *   else scale = fp32(a / 127), inv = fp32(127 / a),
 *        code_c = clamp(round_half_even(fp32(x_c * inv)), -127, 127).
 * mu[b,g,c] = fp32( fp64( exact sum over valid keys of K[b,g,j,c] ) / n ),
 * n = Sk, or max(1, sum(vbs)) when vbs is given; K - mu is one fp32
 * subtraction. qmu[b,h,i] = sum_c Q[b,h,i,c]*mu[b,h/(H/Hkv),c] (fp32) lets
 * attn_fwd report the LSE of the uncentred scores.
 * Non-finite values (the pages do not treat them; this library's reading):
 * a row of Q, or of K - mu, holding a NaN or +-inf gets codes 0 and scale
 * NaN, and for Q a NaN qmu; a K channel whose valid keys hold a NaN or
 * +-inf gets a NaN mean, so every centred K row of that K/V head is such a
 * row. Pad rows (vbs) are never read. Scores involving a NaN scale are NaN,
 * and qfa_attn_fwd's output for a query row that attends such a score is
 * unspecified (no fault).
 *
 * H, Hkv:  heads of Q and of K. Hkv divides H; Hkv < H is grouped-query
 *          attention (ROCm/FlyDSL PR #886 tests and times "MHA and GQA"):
 *          query head h shares K/V head h / (H/Hkv) with the other query
 *          heads of its run. Hkv == H is multi-head attention.
 * q, k:    [B,H,Sq,D] / [B,Hkv,Sk,D] of `dtype` (QFA_BF16 or QFA_FP16),
 *          strides as above; base and row strides 16-byte aligned.
 * vbs:     nullable; int32[Sk/64] per-tile valid-token counts in [0,64]
 *          (requires Sq == Sk, a multiple of 64). Pad rows (j mod 64 >=
 *          vbs[j/64]) of Q and K get codes 0 and scale 0 and are left out of
 *          the mean.
 * center_k: 0 = no centring (kmean, qmu unused and may be NULL).
 * q8, k8:  int8 [B,H,Sq,D] / [B,Hkv,Sk,D] contiguous outputs.
 * qs, ks:  fp32 [B,H,Sq] / [B,Hkv,Sk] contiguous outputs.
 * kmean:   fp32 [B,Hkv,D] output (required when center_k).
 * qmu:     nullable fp32 [B,H,Sq] output (only when center_k).
 * workspace: device buffer of at least qfa_quantize_workspace_bytes(B,
 *          Hkv, Sk, D) bytes, 16-byte aligned (may be NULL when center_k == 0).
 * D must be 64 or 128.
 */
int qfa_quantize_qk(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int dtype,
                    const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                    const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                    const int32_t* vbs, int center_k,
                    int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean, float* qmu,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qfa_quantize_qk_noalloc — qfa_quantize_qk without the workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). The K-mean
 * partials go to a scratch array of 8 MiB that the library holds in static
 * device memory, one copy per GPU it runs on, until the process ends; the
 * call allocates nothing. Arguments, outputs and errors as qfa_quantize_qk;
 * in addition a centring call with B*Hkv above 4096 is rejected with
 * QFA_ERR_UNSUPPORTED before any launch. The calls of a process on one GPU
 * share its scratch, which keeps the last call's contents (nothing in it needs
 * clearing: a call reads only what it wrote): calls that overlap in time on
 * one GPU (different streams or threads) race; calls ordered on one stream do
 * not.
 */
int qfa_quantize_qk_noalloc(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int dtype,
                            const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                            const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                            const int32_t* vbs, int center_k,
                            int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean, float* qmu, void* stream);

/*
 * qfa_blockmask_to_index — tile mask to per-query-tile key-tile lists
 * (FastVideo "minimax_h3_sparse_int8", sparse_sm89_attention: map_to_index).
 *
 * mask:  uint8 [B,H,Tq,Tk] contiguous, nonzero = query tile attends key tile.
 * index: int32 [B,H,Tq,Tk] contiguous output; entries [0, count) of each row
 *        hold the attended key tiles in ascending order, the rest are left
 *        unwritten.
 * count: int32 [B,H,Tq] contiguous output.
 */
int qfa_blockmask_to_index(const uint8_t* mask, int64_t B, int64_t H, int64_t Tq, int64_t Tk,
                           int32_t* index, int32_t* count, void* stream);

/*
 * qfa_attn_fwd — attention forward on int8 Q/K codes and bf16/fp16 V
 * (FastVideo "minimax_h3_sparse_int8"; comfy-kitchen issue #177; FlyDSL
 * PR #886 for the LSE).
 *
 * For each row i of each (b,h) and each key j the call attends:
 *   s_ij = sm_scale * qs_i * ks_j * (q8_i . k8_j) + bias_j       (natural log)
 *   O_i  = v_scale[h,:] * sum_j softmax_j(s_ij) V_j
 *   LSE_i = log sum_j exp(s_ij) + sm_scale * qmu_i
 * The int8 dot is exact in int32; the softmax runs online in fp32 (log2
 * domain) with P rounded to V's type for the PV product (fp32 accumulation).
 * Key j is attended when it lies in one of the segments and, for block-sparse
 * calls, its tile is listed for the query's tile and j mod 64 < vbs[j/64];
 * a bias of -inf also excludes it. A row with no attended key gives O = 0 and
 * LSE = -inf.
 *
 * H, Hkv:  heads of Q and of K/V; Hkv divides H, and query head h reads K/V
 *           head h / (H/Hkv) (grouped-query attention when Hkv < H).
 * q8, qs:   int8 [B,H,Sq,D], fp32 [B,H,Sq] (from qfa_quantize_qk).
 * qmu:      nullable fp32 [B,H,Sq]; sm_scale*qmu is added to the LSE.
 * k_centered: nonzero when k8/ks were quantized from K - mu (center_k of
 *           qfa_quantize_qk). The LSE is then only right with the centring
 *           term, so lse != NULL with k_centered and qmu == NULL is rejected
 *           (QFA_ERR_INVALID_ARG), as is qmu != NULL without k_centered.
 * k8, ks:   int8 [B,Hkv,Sk,D], fp32 [B,Hkv,Sk].
 * v:        [B,Hkv,Sk,D] of v_dtype (QFA_BF16 or QFA_FP16), strides (v_sb,
 *           v_sh, v_ss); base and row strides 16-byte aligned; v_ss below
 *           2^24 elements (else QFA_ERR_UNSUPPORTED). Keys are processed in
 *           tiles of 64. V rows past the end of a segment, of block-sparse pad
 *           keys and past Sk are never read into the product (they may hold
 *           anything). Any other excluded key of a visited tile (before a
 *           segment's start, or excluded by a keep mask, a -inf bias or the
 *           causal diagonal) enters the PV product with weight zero, so its V
 *           row must be finite (0 * inf and 0 * NaN are NaN).
 * sm_scale: softmax scale (typically D^-0.5).
 * bias:     nullable additive per-key bias of bias_dtype (QFA_FP32, QFA_BF16
 *           or QFA_FP16), element (b,h,j) at bias + b*bias_sb + h*bias_sh + j;
 *           pass 0 for a broadcast batch/head stride. It is shared by every
 *           query row (a [B|1,H|1,1,K] tensor or a stride-0 expansion of one).
 *           With bias_dtype QFA_BOOL it is a keep mask of the same layout
 *           (one byte per key, nonzero attends; torch bool semantics): a
 *           masked key is excluded (-inf), so a row whose keys are all masked
 *           gets O = 0 and LSE = -inf. The mask is folded into the per-key
 *           terms and adds no per-score work.
 * bias_sq:  0 for the shared per-key form above. Nonzero: a materialised
 *           per-query bias or keep mask [B|1,H|1,Q,K] (comfy-kitchen issue
 *           #177 passes such masks to attn_mask): element (b,h,i,j) at
 *           bias + b*bias_sb + h*bias_sh + i*bias_sq + j, with bias_sq >= Sk;
 *           base and the three strides 16-byte aligned in bytes, 32*bias_sq
 *           elements below 2^31 bytes (else QFA_ERR_UNSUPPORTED). Values must
 *           be finite or -inf. Each lane loads its row's 64 values per key
 *           tile (the slow path: every score reads one bias value). The row
 *           padding past key Sk - 1 may hold anything (NaN included): it is
 *           read but never used; in the last row the read stops at the
 *           4-byte boundary after key Sk - 1. Not with unquantized Q/K
 *           (QFA_ERR_UNSUPPORTED).
 * index, count, vbs: block-sparse mode when index != NULL: int32 [B,H,T,T],
 *           int32 [B,H,T], int32 [T] (from qfa_blockmask_to_index; vbs may be
 *           NULL for full tiles), T = Sq/64 = Sk/64. Not combinable with bias.
 *           Each row's entries [0, count) must be strictly ascending key tiles
 *           in [0, T), as qfa_blockmask_to_index writes them (the kernel
 *           merges the lists of neighbouring query tiles); other lists give
 *           unspecified results, with every access still in bounds.
 * v_scale:  nullable fp32 [Hkv,D] per-(V head, channel) factor applied to O.
 * nseg, seg: host array of nseg (<= 4) (start, length) pairs of key ranges,
 *           ascending and disjoint; nseg = 0 means the whole [0, Sk).
 * causal:   nonzero: causal self-attention, row i attends keys j <= i only
 *           (the causal mode that ROCm/FlyDSL PR #886 tests and times,
 *           "Test Plan"; read as self-attention, key j <= row i). Needs Sq == Sk
 *           (else QFA_ERR_INVALID_ARG); combines with a bias or keep mask,
 *           v_scale and the LSE, not with segments or a block-sparse mask
 *           (QFA_ERR_UNSUPPORTED). The walk of each 128-row block stops at
 *           its last row's key, so about half the key tiles are read.
 * out:      [B,H,Sq,D] of out_dtype (QFA_BF16, QFA_FP16 or QFA_FP32), strides
 *           (o_sb, o_sh, o_ss); base and row strides 16-byte aligned.
 * lse:      nullable fp32 [B,H,Sq] contiguous output; non-NULL requests it.
 * D must be 64 or 128.
 */
int qfa_attn_fwd(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                 const int8_t* q8, const float* qs, const float* qmu,
                 const int8_t* k8, const float* ks, int k_centered,
                 const void* v, int v_dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                 float sm_scale,
                 const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                 const int32_t* index, const int32_t* count, const int32_t* vbs,
                 const float* v_scale, int nseg, const int64_t* seg, int causal,
                 void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                 float* lse, void* stream);

/*
 * qfa_qk_scores_i32 — the int32 scores S = Q8 K8^T exactly as the attention
 * kernel computes them (FastVideo "minimax_h3_sparse_int8": int8 QK with
 * integer accumulation), for checking them bit for bit. The call runs the
 * attention kernel's own tile copies, LDS layout and int8 MFMA path and
 * stores every score instead of taking the softmax.
 *
 * q8:  int8 [B,H,Sq,D] contiguous (from qfa_quantize_qk).
 * k8:  int8 [B,H,Sk,D] contiguous.
 * s32: int32 [B,H,Sq,Sk] contiguous output, S[b,h,i,j] = sum_c q8[b,h,i,c]*k8[b,h,j,c]
 *      (exact: |S| <= 128*127^2 < 2^31).
 * All three 16-byte aligned; D must be 64 or 128.
 */
int qfa_qk_scores_i32(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                      const int8_t* q8, const int8_t* k8, int32_t* s32, void* stream);

/*
 * qfa_attn_fwd_splitk — qfa_attn_fwd with each (128-row query block, head)
 * key walk cut into num_splits contiguous ranges run by separate blocks, then
 * combined (the split-K path and combine of ROCm/FlyDSL PR #886: "split-K
 * combine", the LSE taken from the combined max and denominator).
 *
 * Split k writes its normalised partial O_k and LSE L_k (fp32) to the
 * workspace; a combine kernel then writes, per row,
 *   m = max_k L_k,  w_k = exp(L_k - m),  O = sum_k w_k O_k / sum_k w_k,
 *   LSE = m + log(sum_k w_k)       (O = 0, LSE = -inf when every L_k = -inf)
 * to out/lse with the same layouts as qfa_attn_fwd. The result equals
 * qfa_attn_fwd's up to fp32 rounding. It fills the GPU when B*H*ceil(Sq/128)
 * is small against the number of CUs.
 *
 * Arguments as qfa_attn_fwd, plus:
 * num_splits: 1..QFA_MAX_SPLITS (1 is qfa_attn_fwd; see qfa_attn_splits_auto).
 *           Block-sparse calls (index != NULL) take only 1
 *           (QFA_ERR_UNSUPPORTED otherwise).
 * workspace: device buffer of at least qfa_attn_split_workspace_bytes(B, H,
 *           Sq, D, num_splits) bytes, 16-byte aligned, owned by the caller;
 *           the call overwrites it and leaves nothing in it that a later
 *           call reads (NULL allowed when num_splits == 1). Calls that run
 *           concurrently need separate workspaces.
 */
int qfa_attn_fwd_splitk(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                        const int8_t* q8, const float* qs, const float* qmu,
                        const int8_t* k8, const float* ks, int k_centered,
                        const void* v, int v_dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                        float sm_scale,
                        const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                        const int32_t* index, const int32_t* count, const int32_t* vbs,
                        const float* v_scale, int nseg, const int64_t* seg, int causal,
                        void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                        float* lse, int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qfa_attn_fwd_unquant — the same attention with Q K^T on the unquantized
 * bf16/fp16 Q and K (the BF16-QK ablation of FastVideo
 * "minimax_h3_sparse_int8": sparse_sm89_attention with int8_qk=False runs
 * the same kernel on the unquantized, uncentred Q and K).
 *
 *   s_ij = sm_scale * (q_i . k_j) + bias_j, products exact, accumulated in
 *   fp32 by the bf16/fp16 MFMA; softmax, PV, masks, LSE, GQA, causal and
 *   split-K as qfa_attn_fwd_splitk (the LSE needs no centring term).
 *
 * q:        [B,H,Sq,D] of dtype, strides (q_sb, q_sh, q_ss) in elements.
 * k:        [B,Hkv,Sk,D] of dtype, strides (k_sb, k_sh, k_ss); k_ss below
 *           2^24 (else QFA_ERR_UNSUPPORTED).
 * v:        [B,Hkv,Sk,D] of dtype (QFA_BF16 or QFA_FP16: one type for Q, K
 *           and V). Base pointers and row strides 16-byte aligned.
 * Every other argument as qfa_attn_fwd_splitk (num_splits 1 for none).
 */
int qfa_attn_fwd_unquant(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                         const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                         const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                         const void* v, int dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                         float sm_scale,
                         const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                         const int32_t* index, const int32_t* count, const int32_t* vbs,
                         const float* v_scale, int nseg, const int64_t* seg, int causal,
                         void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                         float* lse, int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qfa_attn_split_workspace_bytes — workspace qfa_attn_fwd_splitk needs:
 * num_splits * B*H*Sq * (D + 1) * 4 bytes (0 for one split). Writes *bytes.
 */
int qfa_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t Sq, int64_t D, int num_splits, size_t* bytes);

/*
 * qfa_attn_splits_auto — a split count for the current device (a power of
 * two up to 16; 1 when the unsplit grid already fills it): first enough
 * (query block, head, split) blocks for about one round of two per CU while
 * a split keeps at least 16 key tiles of the walk (causal calls: of the
 * average walk), then, for long non-causal walks, more splits while each
 * keeps at least 128 tiles, up to three rounds. Writes *num_splits.
 */
int qfa_attn_splits_auto(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int causal, int* num_splits);

/*
 * qfa_lse_merge — exact merge of two partial softmaxes over disjoint key sets
 * (comfy-kitchen issue #177, Question 2; FlyDSL PR #886, split-K combine):
 *   m = max(La, Lb); m = -inf -> O = 0, L = -inf;
 *   else wa = exp(La - m), wb = exp(Lb - m),
 *        O = (wa*Oa + wb*Ob) / (wa + wb), L = m + log(wa + wb).
 * Arithmetic is fp32.
 *
 * o_a, o_b, o: [B,H,S,D] of their dtypes (QFA_BF16, QFA_FP16, QFA_FP32) with
 *              their own strides; o may alias o_a or o_b exactly (same
 *              pointer, dtype and strides). Bases and row strides 16-byte
 *              aligned.
 * lse_a, lse_b: fp32 [B,H,S] contiguous. lse: nullable fp32 [B,H,S] output,
 *              may alias lse_a or lse_b.
 * D must be 64 or 128.
 */
int qfa_lse_merge(int64_t B, int64_t H, int64_t S, int64_t D,
                  const void* o_a, int a_dtype, int64_t a_sb, int64_t a_sh, int64_t a_ss, const float* lse_a,
                  const void* o_b, int b_dtype, int64_t b_sb, int64_t b_sh, int64_t b_ss, const float* lse_b,
                  void* o, int o_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss, float* lse,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QFA_H */
