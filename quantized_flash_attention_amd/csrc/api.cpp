// C ABI of libqfa.so: argument checking, dispatch and launches on the
// caller's stream. Every check runs before any launch, so a call that fails
// leaves device memory untouched. The declarations and their documentation
// are in include/qfa.h.
#include "../../include/qfa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "qfa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return QFA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dt) { return dt == QFA_FP32 ? 4 : 2; }

// A [B,H,S,D] tensor view: non-null, 16-byte aligned base, row strides whose
// byte size is a multiple of 16 (D is 64 or 128 here, so a row is a whole
// number of 16-byte chunks), non-negative strides.
int check_view(const char* name, const void* p, int dt, int64_t sb, int64_t sh, int64_t ss) {
  if (!p) return fail(QFA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(QFA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  if (sb < 0 || sh < 0 || ss < 0) return fail(QFA_ERR_INVALID_ARG, "%s has a negative stride", name);
  const int64_t eb = elem_bytes(dt);
  if ((sb * eb) % 16 || (sh * eb) % 16 || (ss * eb) % 16)
    return fail(QFA_ERR_INVALID_ARG, "%s strides (%lld,%lld,%lld) are not multiples of 16 bytes", name,
                (long long)sb, (long long)sh, (long long)ss);
  return QFA_OK;
}

int check_dims(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return fail(QFA_ERR_INVALID_ARG, "negative size");
  if (D != 64 && D != 128) return fail(QFA_ERR_UNSUPPORTED, "head dimension %lld (supported: 64, 128)", (long long)D);
  if (B * H > (1ll << 24) || Sq > (1ll << 30) || Sk > (1ll << 30))
    return fail(QFA_ERR_UNSUPPORTED, "sizes beyond the kernels' 32-bit tile indexing");
  return QFA_OK;
}

// Hkv K/V heads shared by runs of H / Hkv query heads
int check_kv_heads(int64_t H, int64_t Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv) {
    if (H == 0 && Hkv == 0) return QFA_OK;
    return fail(QFA_ERR_INVALID_ARG, "%lld query heads cannot share %lld K/V heads (Hkv must divide H)",
                (long long)H, (long long)Hkv);
  }
  return QFA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace qfa {

bool debug_enabled() {
  static const bool on = [] {
    const char* v = getenv("QFA_DEBUG");
    return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

void debug_log(const char* fmt, ...) {
  if (!debug_enabled()) return;
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "qfa: %s\n", line);
}

}  // namespace qfa

extern "C" {

int qfa_version(void) { return 400; }

const char* qfa_status_string(int status) {
  switch (status) {
    case QFA_OK: return "ok";
    case QFA_ERR_INVALID_ARG: return "invalid argument";
    case QFA_ERR_UNSUPPORTED: return "unsupported";
    case QFA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* qfa_last_error(void) { return g_err; }

int qfa_quantize_workspace_bytes(int64_t B, int64_t H, int64_t Sk, int64_t D, size_t* bytes) {
  if (!bytes) return fail(QFA_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 0 || H < 0 || Sk < 0 || D <= 0) return fail(QFA_ERR_INVALID_ARG, "negative size");
  *bytes = (size_t)qfa::quantize_workspace_size(B * H, Sk, D);
  return ok();
}

}  // extern "C"

namespace {

// Argument checks and launches of qfa_quantize_qk, on a workspace the caller (or the
// allocation-free entry point) provides.
int quantize_impl(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int dtype,
                  const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                  const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                  const int32_t* vbs, int center_k,
                  int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean, float* qmu,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_dims(B, H, Sq, Sk, D))) return st;
  if ((st = check_kv_heads(H, Hkv))) return st;
  if (dtype != QFA_BF16 && dtype != QFA_FP16)
    return fail(dtype == QFA_FP32 ? QFA_ERR_UNSUPPORTED : QFA_ERR_INVALID_ARG, "Q/K dtype %d (supported: bf16, fp16)", dtype);
  if (B * H == 0) return ok();  // nothing to read or write: empty tensors may have NULL data
  // 1-D grids of 256-thread blocks over at least 64 rows each stay within 2^32 threads
  if (B * H * Sq > (1ll << 30) || B * Hkv * Sk > (1ll << 30))
    return fail(QFA_ERR_UNSUPPORTED, "more than 2^30 rows of Q or K");
  if (Sq > 0) {
    if ((st = check_view("q", q, dtype, q_sb, q_sh, q_ss))) return st;
    if (!q8 || !qs) return fail(QFA_ERR_INVALID_ARG, "q8/qs output is NULL");
    if (!aligned16(q8) || !aligned16(qs)) return fail(QFA_ERR_INVALID_ARG, "q8/qs outputs must be 16-byte aligned");
  }
  if (Sk > 0) {
    if ((st = check_view("k", k, dtype, k_sb, k_sh, k_ss))) return st;
    if (!k8 || !ks) return fail(QFA_ERR_INVALID_ARG, "k8/ks output is NULL");
    if (!aligned16(k8) || !aligned16(ks)) return fail(QFA_ERR_INVALID_ARG, "k8/ks outputs must be 16-byte aligned");
  }
  if (vbs && (Sq != Sk || Sk % 64)) return fail(QFA_ERR_INVALID_ARG, "vbs requires Sq == Sk, a multiple of 64");
  if (center_k) {
    if (!kmean) return fail(QFA_ERR_INVALID_ARG, "kmean output is NULL with center_k");
    if (!aligned16(kmean) || (qmu && !aligned16(qmu))) return fail(QFA_ERR_INVALID_ARG, "kmean/qmu must be 16-byte aligned");
    const size_t need = (size_t)qfa::quantize_workspace_size(B * Hkv, Sk, D);
    if (need && (!workspace || workspace_bytes < need || !aligned16(workspace)))
      return fail(QFA_ERR_INVALID_ARG, "workspace needs %zu bytes (16-byte aligned), got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
  }
  qfa::QuantArgs a{};
  a.dtype = dtype;
  a.B = B; a.H = H; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.D = D;
  a.q = q; a.q_sb = q_sb; a.q_sh = q_sh; a.q_ss = q_ss;
  a.k = k; a.k_sb = k_sb; a.k_sh = k_sh; a.k_ss = k_ss;
  a.vbs = vbs;
  a.q8 = q8; a.qs = qs; a.qmu = center_k ? qmu : nullptr;
  a.k8 = k8; a.ks = ks;
  a.kmean = center_k ? kmean : nullptr;
  a.workspace = workspace;
  return hip_status(qfa::launch_quantize(a, (hipStream_t)stream), "quantize launch");
}

}  // namespace

extern "C" {

int qfa_quantize_qk(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int dtype,
                    const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                    const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                    const int32_t* vbs, int center_k,
                    int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean, float* qmu,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_impl(B, H, Hkv, Sq, Sk, D, dtype, q, q_sb, q_sh, q_ss, k, k_sb, k_sh, k_ss, vbs, center_k,
                       q8, qs, k8, ks, kmean, qmu, workspace, workspace_bytes, stream);
}

int qfa_quantize_qk_noalloc(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int dtype,
                            const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                            const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                            const int32_t* vbs, int center_k,
                            int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean, float* qmu, void* stream) {
  int st;
  if ((st = check_dims(B, H, Sq, Sk, D))) return st;
  if ((st = check_kv_heads(H, Hkv))) return st;
  void* ws = nullptr;
  size_t cap = 0;
  const int64_t need = center_k ? qfa::quantize_workspace_size(B * Hkv, Sk, D) : 0;
  if (need > 0) {
    if (B * Hkv > qfa::kMeanSlots)
      return fail(QFA_ERR_UNSUPPORTED, "qfa_quantize_qk_noalloc: the K-mean scratch holds %lld (batch, K/V head) "
                  "pairs, the call has %lld", (long long)qfa::kMeanSlots, (long long)(B * Hkv));
    if ((st = hip_status(qfa::noalloc_scratch(&ws, &cap), "scratch address"))) return st;
    if ((size_t)need > cap)
      return fail(QFA_ERR_UNSUPPORTED, "qfa_quantize_qk_noalloc: the call needs %lld bytes of scratch, %zu exist",
                  (long long)need, cap);
  }
  return quantize_impl(B, H, Hkv, Sq, Sk, D, dtype, q, q_sb, q_sh, q_ss, k, k_sb, k_sh, k_ss, vbs, center_k,
                       q8, qs, k8, ks, kmean, qmu, ws, cap, stream);
}

int qfa_blockmask_to_index(const uint8_t* mask, int64_t B, int64_t H, int64_t Tq, int64_t Tk,
                           int32_t* index, int32_t* count, void* stream) {
  if (B < 0 || H < 0 || Tq < 0 || Tk < 0) return fail(QFA_ERR_INVALID_ARG, "negative size");
  if (B * H * Tq * Tk == 0) {
    if (B * H * Tq > 0 && count) {
      return hip_status(qfa::launch_zero_words(count, B * H * Tq, (hipStream_t)stream), "count clear");
    }
    return ok();
  }
  if (!mask || !index || !count) return fail(QFA_ERR_INVALID_ARG, "mask/index/count is NULL");
  if (Tk > (1ll << 30)) return fail(QFA_ERR_UNSUPPORTED, "Tk too large");
  return hip_status(qfa::launch_blockmask_to_index(mask, B * H * Tq, Tk, index, count, (hipStream_t)stream),
                    "blockmask_to_index launch");
}

int qfa_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t Sq, int64_t D, int num_splits, size_t* bytes) {
  if (!bytes) return fail(QFA_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 0 || H < 0 || Sq < 0) return fail(QFA_ERR_INVALID_ARG, "negative size");
  if (D != 64 && D != 128) return fail(QFA_ERR_UNSUPPORTED, "head dimension %lld (supported: 64, 128)", (long long)D);
  if (num_splits < 1 || num_splits > QFA_MAX_SPLITS)
    return fail(QFA_ERR_INVALID_ARG, "num_splits %d (1..%d)", num_splits, QFA_MAX_SPLITS);
  // fp32 partial O [splits][B*H*Sq][D], then fp32 partial LSE [splits][B*H*Sq]
  *bytes = num_splits > 1 ? (size_t)num_splits * (size_t)(B * H * Sq) * (size_t)(D + 1) * 4u : 0;
  return ok();
}

int qfa_attn_splits_auto(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int causal, int* num_splits) {
  if (!num_splits) return fail(QFA_ERR_INVALID_ARG, "num_splits is NULL");
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return fail(QFA_ERR_INVALID_ARG, "negative size");
  int ncu = 0;
  int st;
  if ((st = hip_status(qfa::device_cu_count(&ncu), "device query"))) return st;
  // Powers of two only (odd counts measured slower). First fill about one
  // round of two blocks per CU while a split keeps >= 16 key tiles of the
  // (causal: average) walk; then, for long non-causal walks, keep halving
  // them while a split keeps >= 128 tiles, up to three rounds, so the last
  // round's tail is short (causal grids are already ordered longest walk
  // first, and splitting them measured no gain). Tuned on banded B1 H1..14
  // Sq1024..4096 Sk4096..33600 and causal S2048..32768 shapes.
  const int64_t blocks = (Sq + 127) / 128 * B * H;
  const int64_t walk = causal ? ((Sk + 63) / 64 + 1) / 2 : (Sk + 63) / 64;
  const int64_t slots = 2 * (int64_t)std::max(ncu, 1);
  int64_t n = 1;
  while (n < 16 && blocks * n * 100 < 85 * slots && walk / (2 * n) >= 8) n *= 2;
  while (!causal && n < 16 && blocks * n < 3 * slots && walk / n >= 128) n *= 2;
  *num_splits = (int)n;
  return ok();
}

namespace {
// Q/K operands of an attention call: int8 codes and scales, or (qf != NULL)
// the unquantized Q and K views in V's dtype
struct QKSrc {
  const int8_t* q8;
  const float* qs;
  const float* qmu;
  const int8_t* k8;
  const float* ks;
  int k_centered;       // k8/ks come from K - mu
  const void* qf;
  const void* kf;
  int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss;
};

int attn_fwd_impl(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, const QKSrc& qk,
                  const void* v, int v_dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                  float sm_scale,
                  const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                  const int32_t* index, const int32_t* count, const int32_t* vbs,
                  const float* v_scale, int nseg, const int64_t* seg, int causal,
                  void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                  float* lse, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_dims(B, H, Sq, Sk, D))) return st;
  if ((st = check_kv_heads(H, Hkv))) return st;
  if (v_dtype != QFA_BF16 && v_dtype != QFA_FP16)
    return fail(v_dtype == QFA_FP32 ? QFA_ERR_UNSUPPORTED : QFA_ERR_INVALID_ARG, "V dtype %d (supported: bf16, fp16)", v_dtype);
  if (B * H * Sq == 0) return ok();  // no output rows: empty tensors may have NULL data
  const bool unquant = qk.qf != nullptr;
  if (unquant) {
    if ((st = check_view("q", qk.qf, v_dtype, qk.q_sb, qk.q_sh, qk.q_ss))) return st;
  } else {
    if (!qk.q8 || !qk.qs) return fail(QFA_ERR_INVALID_ARG, "q8/qs is NULL");
    if (!aligned16(qk.q8)) return fail(QFA_ERR_INVALID_ARG, "q8 must be 16-byte aligned");
    // the LSE of centred codes needs the centring term sm_scale * q.mu
    if (lse && qk.k_centered && !qk.qmu)
      return fail(QFA_ERR_INVALID_ARG, "LSE requested on centred K codes without qmu (the centring term)");
    if (qk.qmu && !qk.k_centered) return fail(QFA_ERR_INVALID_ARG, "qmu given but K is not centred");
  }
  if (Sk > 0) {  // with no keys every row is fully masked and K/V are never read
    if (unquant) {
      if ((st = check_view("k", qk.kf, v_dtype, qk.k_sb, qk.k_sh, qk.k_ss))) return st;
      if (qk.k_ss >= (1ll << 24))
        return fail(QFA_ERR_UNSUPPORTED, "K sequence stride %lld elements (supported: below 2^24)",
                    (long long)qk.k_ss);
    } else {
      if (!qk.k8 || !qk.ks) return fail(QFA_ERR_INVALID_ARG, "k8/ks is NULL");
      if (!aligned16(qk.k8)) return fail(QFA_ERR_INVALID_ARG, "k8 must be 16-byte aligned");
    }
    if ((st = check_view("v", v, v_dtype, v_sb, v_sh, v_ss))) return st;
    // one 64-key tile of V then spans less than 2^31 bytes (32-bit copy ranges)
    if (v_ss >= (1ll << 24))
      return fail(QFA_ERR_UNSUPPORTED, "V sequence stride %lld elements (supported: below 2^24)", (long long)v_ss);
  }
  if (out_dtype != QFA_BF16 && out_dtype != QFA_FP16 && out_dtype != QFA_FP32)
    return fail(QFA_ERR_INVALID_ARG, "out dtype %d", out_dtype);
  if ((st = check_view("out", out, out_dtype, o_sb, o_sh, o_ss))) return st;
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY) return fail(QFA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (v_scale && !aligned16(v_scale)) return fail(QFA_ERR_INVALID_ARG, "v_scale must be 16-byte aligned");
  if (bias) {
    if (bias_dtype != QFA_FP32 && bias_dtype != QFA_BF16 && bias_dtype != QFA_FP16 && bias_dtype != QFA_BOOL)
      return fail(QFA_ERR_INVALID_ARG, "bias dtype %d", bias_dtype);
    if (bias_sb < 0 || bias_sh < 0 || bias_sq < 0) return fail(QFA_ERR_INVALID_ARG, "negative bias stride");
    if (index) return fail(QFA_ERR_INVALID_ARG, "bias and block-sparse mask are mutually exclusive");
    if (bias_sq != 0) {
      // materialised per-query bias: rows read 4 keys per 16-byte load
      const int64_t esz = bias_dtype == QFA_FP32 ? 4 : (bias_dtype == QFA_BOOL ? 1 : 2);
      if (unquant) return fail(QFA_ERR_UNSUPPORTED, "a per-query bias with unquantized Q/K");
      if ((reinterpret_cast<uintptr_t>(bias) % 16) || (bias_sb * esz) % 16 || (bias_sh * esz) % 16 ||
          (bias_sq * esz) % 16)
        return fail(QFA_ERR_INVALID_ARG, "a per-query bias needs a 16-byte aligned base and row strides");
      if (bias_sq < Sk) return fail(QFA_ERR_INVALID_ARG, "bias query stride %lld below Sk", (long long)bias_sq);
      if (32 * bias_sq * esz >= (1ll << 31))
        return fail(QFA_ERR_UNSUPPORTED, "bias query stride %lld elements (supported: 32 rows below 2^31 bytes)",
                    (long long)bias_sq);
    }
  }
  qfa::AttnArgs a{};
  if (index) {
    if (!count) return fail(QFA_ERR_INVALID_ARG, "block-sparse call without count");
    if (Sq != Sk || Sk % 64) return fail(QFA_ERR_INVALID_ARG, "block-sparse needs Sq == Sk, a multiple of 64");
    if (nseg != 0) return fail(QFA_ERR_INVALID_ARG, "segments are not combinable with a block-sparse mask");
  }
  if (causal) {
    if (Sq != Sk) return fail(QFA_ERR_INVALID_ARG, "causal attention needs Sq == Sk (got %lld, %lld)", (long long)Sq, (long long)Sk);
    if (index) return fail(QFA_ERR_UNSUPPORTED, "causal attention with a block-sparse mask");
    if (nseg != 0) return fail(QFA_ERR_UNSUPPORTED, "causal attention with key segments");
  }
  if (num_splits < 1 || num_splits > QFA_MAX_SPLITS)
    return fail(QFA_ERR_INVALID_ARG, "num_splits %d (1..%d)", num_splits, QFA_MAX_SPLITS);
  if (num_splits > 1 && index) return fail(QFA_ERR_UNSUPPORTED, "split-K with a block-sparse mask");
  // one 128-row block per (query tile, head, split); 256 threads per block
  // keep the launch within 2^32 threads
  if ((Sq + 127) / 128 * B * H * num_splits > (1ll << 24))
    return fail(QFA_ERR_UNSUPPORTED, "more than 2^24 blocks of 128 query rows");
  if (num_splits > 1) {
    size_t need = 0;
    qfa_attn_split_workspace_bytes(B, H, Sq, D, num_splits, &need);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
      return fail(QFA_ERR_INVALID_ARG, "split workspace needs %zu bytes (16-byte aligned), got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
  }
  if (nseg < 0 || nseg > QFA_MAX_SEGMENTS) return fail(QFA_ERR_INVALID_ARG, "nseg %d (0..4)", nseg);
  if (nseg > 0 && !seg) return fail(QFA_ERR_INVALID_ARG, "seg is NULL with nseg > 0");
  int64_t prev_end = 0;
  for (int g = 0; g < nseg; ++g) {
    const int64_t s0 = seg[2 * g], n = seg[2 * g + 1];
    if (s0 < 0 || n < 0 || s0 + n > Sk)
      return fail(QFA_ERR_INVALID_ARG, "segment %d [%lld, +%lld) outside [0, %lld)", g, (long long)s0, (long long)n, (long long)Sk);
    if (s0 < prev_end) return fail(QFA_ERR_INVALID_ARG, "segments must be ascending and disjoint");
    prev_end = s0 + n;
    a.seg_lo[g] = (int)s0;
    a.seg_hi[g] = (int)(s0 + n);
  }
  if (nseg == 0) {
    a.seg_lo[0] = 0;
    a.seg_hi[0] = (int)Sk;
    nseg = 1;
  }
  a.nseg = nseg;
  a.causal = causal ? 1 : 0;
  a.B = (int)B; a.H = (int)H; a.Hkv = (int)Hkv; a.Sq = (int)Sq; a.Sk = (int)Sk; a.D = (int)D;
  if (unquant) {
    a.qf = qk.qf; a.kf = qk.kf;
    a.q_sb = qk.q_sb; a.q_sh = qk.q_sh; a.q_ss = qk.q_ss; a.k_sb = qk.k_sb; a.k_sh = qk.k_sh; a.k_ss = qk.k_ss;
  } else {
    a.q8 = qk.q8; a.qs = qk.qs; a.qmu = qk.qmu; a.k8 = qk.k8; a.ks = qk.ks;
  }
  a.v = v; a.v_dtype = v_dtype; a.v_sb = v_sb; a.v_sh = v_sh; a.v_ss = v_ss;
  a.sm_scale = sm_scale;
  a.bias = bias; a.bias_dtype = bias_dtype; a.bias_sb = bias_sb; a.bias_sh = bias_sh; a.bias_sq = bias ? bias_sq : 0;
  a.index = index; a.count = count; a.vbs = index ? vbs : nullptr;
  a.v_scale = v_scale;
  a.out = out; a.out_dtype = out_dtype; a.o_sb = o_sb; a.o_sh = o_sh; a.o_ss = o_ss;
  a.lse = lse;
  a.nsplit = num_splits;
  if (num_splits > 1) {
    a.part_o = (float*)workspace;
    a.part_lse = a.part_o + (size_t)num_splits * (size_t)(B * H * Sq) * (size_t)D;
  }
  return hip_status(qfa::launch_attn_fwd(a, (hipStream_t)stream), "attn_fwd launch");
}
}  // namespace

int qfa_attn_fwd(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                 const int8_t* q8, const float* qs, const float* qmu,
                 const int8_t* k8, const float* ks, int k_centered,
                 const void* v, int v_dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                 float sm_scale,
                 const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                 const int32_t* index, const int32_t* count, const int32_t* vbs,
                 const float* v_scale, int nseg, const int64_t* seg, int causal,
                 void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                 float* lse, void* stream) {
  const QKSrc qk{q8, qs, qmu, k8, ks, k_centered, nullptr, nullptr, 0, 0, 0, 0, 0, 0};
  return attn_fwd_impl(B, H, Hkv, Sq, Sk, D, qk, v, v_dtype, v_sb, v_sh, v_ss, sm_scale,
                       bias, bias_dtype, bias_sb, bias_sh, bias_sq, index, count, vbs, v_scale, nseg, seg, causal,
                       out, out_dtype, o_sb, o_sh, o_ss, lse, 1, nullptr, 0, stream);
}

int qfa_attn_fwd_splitk(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                        const int8_t* q8, const float* qs, const float* qmu,
                        const int8_t* k8, const float* ks, int k_centered,
                        const void* v, int v_dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                        float sm_scale,
                        const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                        const int32_t* index, const int32_t* count, const int32_t* vbs,
                        const float* v_scale, int nseg, const int64_t* seg, int causal,
                        void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                        float* lse, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  const QKSrc qk{q8, qs, qmu, k8, ks, k_centered, nullptr, nullptr, 0, 0, 0, 0, 0, 0};
  return attn_fwd_impl(B, H, Hkv, Sq, Sk, D, qk, v, v_dtype, v_sb, v_sh, v_ss, sm_scale,
                       bias, bias_dtype, bias_sb, bias_sh, bias_sq, index, count, vbs, v_scale, nseg, seg, causal,
                       out, out_dtype, o_sb, o_sh, o_ss, lse, num_splits, workspace, workspace_bytes, stream);
}

int qfa_attn_fwd_unquant(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                         const void* q, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                         const void* k, int64_t k_sb, int64_t k_sh, int64_t k_ss,
                         const void* v, int dtype, int64_t v_sb, int64_t v_sh, int64_t v_ss,
                         float sm_scale,
                         const void* bias, int bias_dtype, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                         const int32_t* index, const int32_t* count, const int32_t* vbs,
                         const float* v_scale, int nseg, const int64_t* seg, int causal,
                         void* out, int out_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss,
                         float* lse, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  const QKSrc qk{nullptr, nullptr, nullptr, nullptr, nullptr, 0, q, k, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss};
  if (!q && B * H * Sq > 0) return fail(QFA_ERR_INVALID_ARG, "q is NULL");
  return attn_fwd_impl(B, H, Hkv, Sq, Sk, D, qk, v, dtype, v_sb, v_sh, v_ss, sm_scale,
                       bias, bias_dtype, bias_sb, bias_sh, bias_sq, index, count, vbs, v_scale, nseg, seg, causal,
                       out, out_dtype, o_sb, o_sh, o_ss, lse, num_splits, workspace, workspace_bytes, stream);
}

int qfa_qk_scores_i32(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                      const int8_t* q8, const int8_t* k8, int32_t* s32, void* stream) {
  int st;
  if ((st = check_dims(B, H, Sq, Sk, D))) return st;
  if (B * H * Sq == 0 || Sk == 0) return ok();  // no scores
  if (!q8 || !k8 || !s32) return fail(QFA_ERR_INVALID_ARG, "q8/k8/s32 is NULL");
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(s32))
    return fail(QFA_ERR_INVALID_ARG, "q8, k8 and s32 must be 16-byte aligned");
  if (B * H * Sq * Sk > (1ll << 40)) return fail(QFA_ERR_UNSUPPORTED, "score tensor too large");
  qfa::AttnArgs a{};
  a.B = (int)B; a.H = (int)H; a.Hkv = (int)H; a.Sq = (int)Sq; a.Sk = (int)Sk; a.D = (int)D;
  a.q8 = q8; a.k8 = k8;
  a.nseg = 1;
  a.seg_lo[0] = 0;
  a.seg_hi[0] = (int)Sk;
  a.out = s32;
  return hip_status(qfa::launch_qk_scores(a, (hipStream_t)stream), "qk_scores launch");
}

int qfa_lse_merge(int64_t B, int64_t H, int64_t S, int64_t D,
                  const void* o_a, int a_dtype, int64_t a_sb, int64_t a_sh, int64_t a_ss, const float* lse_a,
                  const void* o_b, int b_dtype, int64_t b_sb, int64_t b_sh, int64_t b_ss, const float* lse_b,
                  void* o, int o_dtype, int64_t o_sb, int64_t o_sh, int64_t o_ss, float* lse,
                  void* stream) {
  int st;
  if ((st = check_dims(B, H, S, S, D))) return st;
  for (int dt : {a_dtype, b_dtype, o_dtype})
    if (dt != QFA_BF16 && dt != QFA_FP16 && dt != QFA_FP32) return fail(QFA_ERR_INVALID_ARG, "dtype %d", dt);
  if (B * H * S == 0) return ok();
  if ((st = check_view("o_a", o_a, a_dtype, a_sb, a_sh, a_ss))) return st;
  if ((st = check_view("o_b", o_b, b_dtype, b_sb, b_sh, b_ss))) return st;
  if ((st = check_view("o", o, o_dtype, o_sb, o_sh, o_ss))) return st;
  if (!lse_a || !lse_b) return fail(QFA_ERR_INVALID_ARG, "lse_a/lse_b is NULL");
  auto same = [&](const void* p, int dt, int64_t sb, int64_t sh, int64_t ss) {
    return p == o && dt == o_dtype && sb == o_sb && sh == o_sh && ss == o_ss;
  };
  // o may alias an input only exactly (element-wise in place)
  if (o == o_a && !same(o_a, a_dtype, a_sb, a_sh, a_ss)) return fail(QFA_ERR_INVALID_ARG, "o aliases o_a with another layout");
  if (o == o_b && !same(o_b, b_dtype, b_sb, b_sh, b_ss)) return fail(QFA_ERR_INVALID_ARG, "o aliases o_b with another layout");
  qfa::MergeArgs m{B, H, S, D, o_a, a_dtype, a_sb, a_sh, a_ss, lse_a, o_b, b_dtype, b_sb, b_sh, b_ss, lse_b,
                   o, o_dtype, o_sb, o_sh, o_ss, lse};
  return hip_status(qfa::launch_lse_merge(m, (hipStream_t)stream), "lse_merge launch");
}

}  // extern "C"
