// C-ABI entry points of liblbq (declared in include/lbq.h): host-side
// validation, buffer layout, NF4 codebook and kernel dispatch.  Every argument
// check runs before anything is enqueued; nothing here synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "lbq.h"
#include "lbq_internal.h"

namespace {

thread_local std::string g_detail;

lbq_status fail(lbq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lbq_status fail(lbq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

lbq_status ok() {
  g_detail.clear();
  return LBQ_OK;
}

lbq_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(LBQ_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---- NF4 codebook ----------------------------------------------------------
// Standard normal quantile by bisection on Phi(x) = erfc(-x/sqrt 2)/2 in fp64,
// run until the bracket cannot shrink further.
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 2000; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    const double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (cdf < p) {
      lo = mid;
    } else {
      hi = mid;
    }
  }
  return 0.5 * (lo + hi);
}

// NF4 levels ("QLoRA技术在量化微调中的应用", section QLoRA技术原理: a 4-bit
// NormalFloat type for normally distributed weights).  Eight positive levels
// are the normal quantiles of 9 evenly spaced probabilities from delta down to
// 1/2 without the last; seven negative levels likewise from 8 points; plus an
// exact zero; all divided by the quantile at delta so the extremes are +-1.
lbq::Nf4Table make_nf4_table() {
  const double delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  std::vector<double> v;
  for (int i = 0; i < 8; ++i) v.push_back(normal_quantile(delta + (0.5 - delta) * i / 8.0));
  for (int i = 0; i < 7; ++i) v.push_back(-normal_quantile(delta + (0.5 - delta) * i / 7.0));
  v.push_back(0.0);
  std::sort(v.begin(), v.end());
  const double top = normal_quantile(delta);
  lbq::Nf4Table t;
  for (int i = 0; i < 16; ++i) t.c[i] = (float)(v[i] / top);
  return t;
}

const lbq::Nf4Table& nf4_table() {
  static const lbq::Nf4Table t = make_nf4_table();
  return t;
}

// ---- validation ------------------------------------------------------------
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

lbq_status check_desc(const lbq_desc* d) {
  if (d == nullptr) return fail(LBQ_E_NULL, "desc is NULL");
  if (d->format == LBQ_MINMAX) {
    if (d->bits != 4 && d->bits != 2) return fail(LBQ_E_FORMAT, "MINMAX bits must be 4 or 2 (got %d)", d->bits);
    if (d->group != 128 && d->group != 64) return fail(LBQ_E_FORMAT, "MINMAX group must be 64 or 128 (got %d)", d->group);
    if (d->double_quant != 0 || d->dq_block != 0) return fail(LBQ_E_FORMAT, "MINMAX takes no double quantization");
    if (d->meta != LBQ_META_F32 && d->meta != LBQ_META_COMPACT)
      return fail(LBQ_E_FORMAT, "MINMAX meta must be 0 (fp32 scale, byte zero point) or 1 (compact), got %d", d->meta);
    if (d->meta == LBQ_META_COMPACT && !((d->bits == 4 && d->group == 128) || (d->bits == 2 && d->group == 64)))
      return fail(LBQ_E_FORMAT, "compact metadata is defined for INT4 g128 and INT2 g64 only");
  } else if (d->format == LBQ_NF4) {
    if (d->meta != 0) return fail(LBQ_E_FORMAT, "NF4 takes meta = 0");
    if (d->bits != 4) return fail(LBQ_E_FORMAT, "NF4 bits must be 4 (got %d)", d->bits);
    if (d->group != 64) return fail(LBQ_E_FORMAT, "NF4 absmax block must be 64 (got %d)", d->group);
    if (d->double_quant < 0 || d->double_quant > 2)
      return fail(LBQ_E_FORMAT, "double_quant must be 0, 1 or 2 (with an offset), got %d", d->double_quant);
    if (d->dq_block != (d->double_quant ? 256 : 0)) return fail(LBQ_E_FORMAT, "dq_block must be 256 with double quantization and 0 otherwise");
  } else {
    return fail(LBQ_E_FORMAT, "unknown format %d (MINMAX=0, NF4=1)", d->format);
  }
  if (d->n < 1 || d->n > (int64_t(1) << 31) - 1) return fail(LBQ_E_SHAPE, "n must be in [1, 2^31) (got %lld)", (long long)d->n);
  if (d->k < 64 || d->k > (int64_t(1) << 24)) return fail(LBQ_E_SHAPE, "k must be in [64, 2^24] (got %lld)", (long long)d->k);
  if (d->k % 64 != 0 || d->k % d->group != 0) return fail(LBQ_E_SHAPE, "k (%lld) must be a multiple of 64 and of the group", (long long)d->k);
  if (d->n * d->k > (int64_t(1) << 40)) return fail(LBQ_E_SHAPE, "n*k too large");
  if (d->format == LBQ_MINMAX && d->meta == LBQ_META_COMPACT && (d->k / d->group) * d->bits % 8 != 0)
    return fail(LBQ_E_SHAPE, "compact metadata needs (k / group) * bits %% 8 == 0 (k %lld)", (long long)d->k);
  return LBQ_OK;
}

lbq::WKind kind_of(const lbq_desc* d) {
  if (d->format == LBQ_NF4)
    return d->double_quant == 2 ? lbq::WK_NF4DQO : (d->double_quant ? lbq::WK_NF4DQ : lbq::WK_NF4);
  if (d->meta == LBQ_META_COMPACT) return d->bits == 4 ? lbq::WK_I4G128C : lbq::WK_I2G64C;
  if (d->bits == 4) return d->group == 128 ? lbq::WK_I4G128 : lbq::WK_I4G64;
  return d->group == 64 ? lbq::WK_I2G64 : lbq::WK_I2G128;
}

// Serialized blob: "LBQ1", uint32 version, the descriptor, six uint64 byte
// counts, then the buffers at 16-byte boundaries.
constexpr char kBlobMagic[4] = {'L', 'B', 'Q', '1'};
constexpr uint32_t kBlobVersion = 1;
constexpr size_t kBlobHeader = 96;
static_assert(sizeof(lbq_desc) == 40, "blob layout assumes a 40-byte descriptor");

void sizes_of(const lbq_desc* d, lbq_sizes* s) {
  std::memset(s, 0, sizeof *s);
  s->packed = (size_t)(d->n * d->k * d->bits / 8);
  if (d->format == LBQ_MINMAX) {
    const int64_t ng = d->n * (d->k / d->group);
    if (d->meta == LBQ_META_COMPACT) {
      s->scales = (size_t)ng * 2;                 // fp16
      s->zeros = (size_t)(ng * d->bits / 8);      // packed like the codes
    } else {
      s->scales = (size_t)ng * sizeof(float);
      s->zeros = (size_t)ng;
    }
  } else {
    const int64_t nb = d->n * d->k / 64;
    if (d->double_quant) {
      s->absmax_q = (size_t)nb;
      // with an offset, one more fp32 after the per-run scales
      s->absmax_scale = (size_t)((nb + 255) / 256 + (d->double_quant == 2 ? 1 : 0)) * sizeof(float);
    } else {
      s->absmax = (size_t)nb * sizeof(float);
    }
  }
}

// Pointers of `q` that the format reads (or writes, for quantize).
lbq_status check_qtensor(const lbq_desc* d, const lbq_qtensor* q) {
  if (q == nullptr) return fail(LBQ_E_NULL, "qtensor is NULL");
  if (q->packed == nullptr) return fail(LBQ_E_NULL, "qtensor.packed is NULL");
  if (!aligned(q->packed, 16)) return fail(LBQ_E_ALIGN, "qtensor.packed must be 16-byte aligned");
  if (d->format == LBQ_MINMAX) {
    if (q->scales == nullptr || q->zeros == nullptr) return fail(LBQ_E_NULL, "MINMAX needs scales and zeros");
    if (!aligned(q->scales, d->meta == LBQ_META_COMPACT ? 2 : 4))
      return fail(LBQ_E_ALIGN, "scales must be 4-byte (fp32) or 2-byte (fp16) aligned");
  } else if (d->double_quant) {
    if (q->absmax_q == nullptr || q->absmax_scale == nullptr) return fail(LBQ_E_NULL, "NF4 with double quant needs absmax_q and absmax_scale");
    if (!aligned(q->absmax_scale, 4)) return fail(LBQ_E_ALIGN, "absmax_scale must be 4-byte aligned");
  } else {
    if (q->absmax == nullptr) return fail(LBQ_E_NULL, "NF4 needs absmax");
    if (!aligned(q->absmax, 4)) return fail(LBQ_E_ALIGN, "absmax must be 4-byte aligned");
  }
  return LBQ_OK;
}

lbq::WView view_of(const lbq_desc* d, const lbq_qtensor* q) {
  lbq::WView w;
  w.packed = static_cast<const uint8_t*>(q->packed);
  w.scales = static_cast<const float*>(q->scales);
  w.zeros = q->zeros;
  w.absmax = q->absmax;
  w.absmax_q = q->absmax_q;
  w.absmax_scale = q->absmax_scale;
  w.n = d->n;
  w.k = d->k;
  return w;
}

lbq_status check_fwd_common(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                            int64_t m, uint16_t* Y, int64_t ldy) {
  lbq_status st = check_desc(desc);
  if (st != LBQ_OK) return st;
  if ((st = check_qtensor(desc, q)) != LBQ_OK) return st;
  if (m < 0 || m > (int64_t(1) << 31) - 1) return fail(LBQ_E_SHAPE, "m must be in [0, 2^31) (got %lld)", (long long)m);
  if (m == 0) return LBQ_OK;
  // The GEMM addresses X and the weight with 32-bit byte offsets (plus one
  // tile of slack past the last row).
  if ((uint64_t)(m + 256) * (uint64_t)desc->k * 2 >= (uint64_t(1) << 32) ||
      (uint64_t)(desc->n + 256) * (uint64_t)desc->k >= (uint64_t(1) << 32))
    return fail(LBQ_E_SHAPE, "(m + 256) * k * 2 and (n + 256) * k must be below 2^32 (m %lld, n %lld, k %lld)",
                (long long)m, (long long)desc->n, (long long)desc->k);
  if (X == nullptr || Y == nullptr) return fail(LBQ_E_NULL, "X and Y must be non-NULL");
  if (!aligned(X, 16)) return fail(LBQ_E_ALIGN, "X must be 16-byte aligned");
  if (!aligned(Y, 2)) return fail(LBQ_E_ALIGN, "Y must be 2-byte aligned");
  if (q->out_rows == nullptr && ldy < desc->n) return fail(LBQ_E_SHAPE, "ldy (%lld) < n (%lld)", (long long)ldy, (long long)desc->n);
  if (ldy < 1) return fail(LBQ_E_SHAPE, "ldy must be >= 1");
  return LBQ_OK;
}

int32_t round_rank(int32_t r) { return (r + 31) / 32 * 32; }
int64_t round_rows(int64_t m) { return (m + 31) / 32 * 32; }

// Forward kernel choice: single-token decode streams the weight (GEMV);
// 2 <= m <= 64 uses the small-batch MFMA kernel (fp32 partials in `ws` when K
// is split); larger m the MFMA GEMM with the dequantized weight tile in LDS.
// The multi-row GEMV serves 2 <= m <= 4 while the m rows of x fit its LDS
// (gemvm_fits) -- except, at m >= 3, a weight large enough that the
// small-batch MFMA kernel runs it unsplit (its row tiles alone fill a fifth of
// that kernel's resident workgroups, with a short K range: n > 13056 and
// k <= 4096 for m = 3..4): there the MFMA
// kernel is faster (8B gate+up at m = 3 and 4: 29.7 -> 23.7 and 30.6 ->
// 23.6 us; q+k+v and o stay faster on the GEMV).  Decided per weight, so a
// grouped call serves each weight as the single-weight call does.
bool use_gemvm(const lbq_desc* d, int64_t m) {
  if (!lbq::gemvm_fits(kind_of(d), d->k, m)) return false;
  return m < 3 || !lbq::skinny_fills_unsplit(d->n, d->k, m);
}

// The GEMM's K-split partials (m > kSkinnyMaxM) for weights ns[0..count):
// the workspace when it holds them (16-byte aligned), else nullptr -- then
// nothing splits.  Only the small-batch kernel's partials are required.
float* gemm_part(const int64_t* ns, int count, int64_t k, int64_t m, void* ws, size_t ws_bytes) {
  const size_t need = lbq::gemm_fwd_workspace_bytes(ns, count, k, m);
  if (need == 0 || ws == nullptr || ws_bytes < need || !aligned(ws, 16)) return nullptr;
  return static_cast<float*>(ws);
}

hipError_t dispatch_fwd(const lbq_desc* desc, const lbq::WView& w, const uint16_t* X, int64_t m,
                        uint16_t* Y, int64_t ldy, const int32_t* out_rows,
                        const lbq::LoraEpi& lora, void* ws, size_t ws_bytes, hipStream_t s) {
  const lbq::WKind kind = kind_of(desc);
  if (m == 1) return lbq::launch_gemv1(kind, &w, &Y, &out_rows, 1, X, lora, nf4_table(), s);
  if (use_gemvm(desc, m)) return lbq::launch_gemvm(kind, &w, &Y, &ldy, &out_rows, 1, X, m, lora, nf4_table(), s);
  if (m <= lbq::kSkinnyMaxM)
    return lbq::launch_skinny(kind, w, X, m, Y, ldy, out_rows, static_cast<float*>(ws), lora,
                              nf4_table(), s);
  const int64_t n = desc->n;
  return lbq::launch_gemm_fwd(kind, w, X, m, Y, ldy, out_rows, lora, gemm_part(&n, 1, desc->k, m, ws, ws_bytes),
                              nf4_table(), s);
}

// Workspace of the forward: the small-batch kernel's partials (required) or,
// for m > kSkinnyMaxM, the GEMM's K-split partials (optional).
size_t fwd_workspace(const lbq_desc* desc, int64_t m, bool lora) {
  if (use_gemvm(desc, m)) return 0;
  if (m >= 2 && m <= lbq::kSkinnyMaxM) return lbq::skinny_workspace_bytes(desc->n, desc->k, m, lora);
  if (m > lbq::kSkinnyMaxM) {
    const int64_t n = desc->n;
    return lbq::gemm_fwd_workspace_bytes(&n, 1, desc->k, m);
  }
  return 0;
}

// Checks shared by the two input-gradient entries (m == 0 passes).
lbq_status check_bwd_common(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* dY,
                            int64_t m, uint16_t* dX, const char* who) {
  lbq_status st = check_desc(desc);
  if (st != LBQ_OK) return st;
  if ((st = check_qtensor(desc, q)) != LBQ_OK) return st;
  if (q->out_rows != nullptr) return fail(LBQ_E_UNSUPPORTED, "%s does not take out_rows", who);
  if (m < 0 || m > (int64_t(1) << 31) - 1) return fail(LBQ_E_SHAPE, "m must be in [0, 2^31)");
  if (m == 0) return LBQ_OK;
  if (dY == nullptr || dX == nullptr) return fail(LBQ_E_NULL, "dY and dX must be non-NULL");
  if (!aligned(dY, 16) || !aligned(dX, 16)) return fail(LBQ_E_ALIGN, "dY and dX must be 16-byte aligned");
  if (desc->n % 8 != 0) return fail(LBQ_E_SHAPE, "%s needs n %% 8 == 0 (got %lld)", who, (long long)desc->n);
  if ((uint64_t)(m + 256) * (uint64_t)desc->n * 2 >= (uint64_t(1) << 32) ||
      (uint64_t)(m + 256) * (uint64_t)desc->k * 2 >= (uint64_t(1) << 32) ||
      (uint64_t)(desc->n + 256) * (uint64_t)desc->k >= (uint64_t(1) << 32))
    return fail(LBQ_E_SHAPE, "(m + 256) * n * 2, (m + 256) * k * 2 and (n + 256) * k must be below 2^32 "
                "(m %lld, n %lld, k %lld)", (long long)m, (long long)desc->n, (long long)desc->k);
  return LBQ_OK;
}

}  // namespace

namespace lbq {

// Shared with the allocation-free forward (k_noalloc.hip): records the
// detail of a failure for lbq_last_error_detail().
lbq_status set_error(lbq_status s, const char* what) { return fail(s, "%s", what); }

lbq_status check_fwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X, int64_t m, uint16_t* Y,
                     int64_t ldy) {
  return check_fwd_common(desc, q, X, m, Y, ldy);
}

// The forward of lbq_linear_fwd once the arguments have passed check_fwd:
// the workspace check and the dispatch.
lbq_status linear_fwd_body(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X, int64_t m,
                           uint16_t* Y, int64_t ldy, void* workspace, size_t ws_bytes, void* stream,
                           const char* who) {
  if (m == 0) return ok();
  const size_t need = fwd_workspace(desc, m, false);
  if (m <= lbq::kSkinnyMaxM && need > 0) {  // the GEMM's partials are optional
    if (workspace == nullptr || ws_bytes < need)
      return fail(LBQ_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (!aligned(workspace, 16)) return fail(LBQ_E_ALIGN, "workspace must be 16-byte aligned");
  }
  const lbq::LoraEpi none{nullptr, nullptr, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lbq::WView w = view_of(desc, q);
  return hip_status(dispatch_fwd(desc, w, X, m, Y, ldy, q->out_rows, none, workspace, ws_bytes, s), who);
}

}  // namespace lbq

extern "C" {

lbq_status lbq_layout(const lbq_desc* desc, lbq_sizes* out) {
  lbq_status st = check_desc(desc);
  if (st != LBQ_OK) return st;
  if (out == nullptr) return fail(LBQ_E_NULL, "out is NULL");
  sizes_of(desc, out);
  return ok();
}

lbq_status lbq_quantize(const lbq_desc* desc, const float* W, const lbq_qtensor* q, void* stream) {
  lbq_status st = check_desc(desc);
  if (st != LBQ_OK) return st;
  if ((st = check_qtensor(desc, q)) != LBQ_OK) return st;
  if (W == nullptr) return fail(LBQ_E_NULL, "W is NULL");
  if (!aligned(W, 16)) return fail(LBQ_E_ALIGN, "W must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (desc->format == LBQ_MINMAX) {
    e = lbq::launch_quant_minmax(desc->bits, desc->group, desc->meta == LBQ_META_COMPACT, W,
                                 static_cast<uint8_t*>(q->packed), static_cast<float*>(q->scales), q->zeros,
                                 desc->n, desc->k, s);
  } else {
    e = lbq::launch_quant_nf4(desc->double_quant, W, static_cast<uint8_t*>(q->packed),
                              q->absmax, q->absmax_q, q->absmax_scale, desc->n, desc->k,
                              nf4_table(), s);
  }
  return hip_status(e, "lbq_quantize");
}

lbq_status lbq_dequant(const lbq_desc* desc, const lbq_qtensor* q, uint16_t* W_bf16, void* stream) {
  lbq_status st = check_desc(desc);
  if (st != LBQ_OK) return st;
  if ((st = check_qtensor(desc, q)) != LBQ_OK) return st;
  if (W_bf16 == nullptr) return fail(LBQ_E_NULL, "W_bf16 is NULL");
  if (!aligned(W_bf16, 16)) return fail(LBQ_E_ALIGN, "W_bf16 must be 16-byte aligned");
  return hip_status(lbq::launch_dequant(kind_of(desc), view_of(desc, q), W_bf16, nf4_table(),
                                        static_cast<hipStream_t>(stream)),
                    "lbq_dequant");
}

size_t lbq_linear_workspace_bytes(const lbq_desc* desc, int64_t m) {
  if (check_desc(desc) != LBQ_OK || m < 1) return 0;
  return fwd_workspace(desc, m, false);
}

lbq_status lbq_linear_fwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                          int64_t m, uint16_t* Y, int64_t ldy, void* workspace, size_t ws_bytes,
                          void* stream) {
  const lbq_status st = check_fwd_common(desc, q, X, m, Y, ldy);
  if (st != LBQ_OK) return st;
  return lbq::linear_fwd_body(desc, q, X, m, Y, ldy, workspace, ws_bytes, stream, "lbq_linear_fwd");
}

// A grouped call at 2 <= m <= 64 whose weights are all INT4 g128 or INT2 g64,
// with both formats present and neither served by the multi-row GEMV (the
// two row sets of channel-mixed linears that share X): one small-batch launch
// for both formats.
static bool skinny_mix_set(int32_t count, const lbq_desc* descs, int64_t m) {
  if (m < 2 || m > lbq::kSkinnyMaxM) return false;
  int ca = 0, cb = 0;
  for (int32_t i = 0; i < count; ++i) {
    const lbq::WKind kd = kind_of(&descs[i]);
    if (kd == lbq::WK_I4G128) ++ca;
    else if (kd == lbq::WK_I2G64) ++cb;
    else return false;
  }
  if (ca == 0 || cb == 0) return false;
  for (int32_t i = 0; i < count; ++i)
    if (use_gemvm(&descs[i], m)) return false;
  return true;
}

// A grouped call of INT4 g128 and INT2 g64 weights (both present) that all
// take the multi-row GEMV (2 <= m <= 4, rows short enough): one multi-row
// launch for both formats.
static bool gemvm_mix_set(int32_t count, const lbq_desc* descs, int64_t m) {
  if (m < 2 || m > lbq::kGemvmMaxM) return false;
  int ca = 0, cb = 0;
  for (int32_t i = 0; i < count; ++i) {
    const lbq::WKind kd = kind_of(&descs[i]);
    if (kd == lbq::WK_I4G128) ++ca;
    else if (kd == lbq::WK_I2G64) ++cb;
    else return false;
    if (!use_gemvm(&descs[i], m)) return false;
  }
  return ca > 0 && cb > 0;
}

// Weights of one kind in a grouped call run as one launch (one launch pair
// for the small-batch kernel when it splits K, and up to two GEMM launches
// when splitting the set fills the chip better), one kind after another on
// the stream; the workspace holds the partials of the largest kind group (of
// all the weights when the two channel-mix formats share one launch).
size_t lbq_linear_fwd_grouped_workspace_bytes(int32_t count, const lbq_desc* descs, int64_t m) {
  if (count < 1 || count > LBQ_MAX_GROUP || descs == nullptr) return 0;
  for (int32_t i = 0; i < count; ++i)
    if (check_desc(&descs[i]) != LBQ_OK || descs[i].k != descs[0].k) return 0;
  if (m > lbq::kSkinnyMaxM) {  // the GEMM's K-split partials, per kind group
    size_t need = 0;
    bool done[LBQ_MAX_GROUP] = {};
    for (int32_t i = 0; i < count; ++i) {
      if (done[i]) continue;
      int64_t ns[LBQ_MAX_GROUP];
      int c = 0;
      for (int32_t j = i; j < count; ++j)
        if (!done[j] && kind_of(&descs[j]) == kind_of(&descs[i])) {
          done[j] = true;
          ns[c++] = descs[j].n;
        }
      need = std::max(need, lbq::gemm_fwd_workspace_bytes(ns, c, descs[i].k, m));
    }
    return need;
  }
  if (m < 2) return 0;
  if (skinny_mix_set(count, descs, m)) {
    int64_t ns[LBQ_MAX_GROUP];
    for (int32_t i = 0; i < count; ++i) ns[i] = descs[i].n;
    return lbq::skinny_set_workspace_bytes(ns, count, descs[0].k, m);
  }
  size_t need = 0;
  bool done[LBQ_MAX_GROUP] = {};
  for (int32_t i = 0; i < count; ++i) {
    if (done[i]) continue;
    const lbq::WKind kind = kind_of(&descs[i]);
    if (use_gemvm(&descs[i], m)) continue;
    int64_t ns[LBQ_MAX_GROUP];
    int c = 0;
    for (int32_t j = i; j < count; ++j)
      if (!done[j] && kind_of(&descs[j]) == kind && !use_gemvm(&descs[j], m)) {
        done[j] = true;
        ns[c++] = descs[j].n;
      }
    need = std::max(need, lbq::skinny_set_workspace_bytes(ns, c, descs[i].k, m));
  }
  return need;
}

lbq_status lbq_linear_fwd_grouped(int32_t count, const lbq_desc* descs, const lbq_qtensor* qs,
                                  const uint16_t* X, int64_t m, uint16_t* const* Ys, const int64_t* ldys,
                                  void* workspace, size_t ws_bytes, void* stream) {
  if (count < 1 || count > LBQ_MAX_GROUP)
    return fail(LBQ_E_SHAPE, "count must be in [1, %d] (got %d)", LBQ_MAX_GROUP, count);
  if (descs == nullptr || qs == nullptr || Ys == nullptr || ldys == nullptr)
    return fail(LBQ_E_NULL, "descs, qs, Ys and ldys must be non-NULL");
  for (int32_t i = 0; i < count; ++i) {
    const lbq_status st = check_fwd_common(&descs[i], &qs[i], X, m, Ys[i], ldys[i]);
    if (st != LBQ_OK) return st;
    if (descs[i].k != descs[0].k)
      return fail(LBQ_E_SHAPE, "weight %d has k = %lld, weight 0 has %lld", i, (long long)descs[i].k,
                  (long long)descs[0].k);
  }
  if (m == 0) return ok();
  const size_t need = lbq_linear_fwd_grouped_workspace_bytes(count, descs, m);
  if (m <= lbq::kSkinnyMaxM && need > 0) {  // the GEMM's partials are optional
    if (workspace == nullptr || ws_bytes < need)
      return fail(LBQ_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (!aligned(workspace, 16)) return fail(LBQ_E_ALIGN, "workspace must be 16-byte aligned");
  }
  const lbq::LoraEpi none{nullptr, nullptr, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (m == 1 || skinny_mix_set(count, descs, m) || gemvm_mix_set(count, descs, m)) {
    // The INT4 g128 and INT2 g64 row sets of channel-mixed linears (and
    // nothing else): one launch for both formats (m = 1: the GEMV; 2 <= m <=
    // 4 with rows the multi-row GEMV takes: that kernel; else up to m = 64
    // the small-batch kernel and its reduce).
    lbq::WView ws[LBQ_MAX_GROUP];
    uint16_t* ys[LBQ_MAX_GROUP];
    int64_t lds[LBQ_MAX_GROUP];
    const int32_t* rows[LBQ_MAX_GROUP];
    int ca = 0, cb = 0;
    for (int pass = 0; pass < 2; ++pass)
      for (int32_t i = 0; i < count; ++i)
        if (kind_of(&descs[i]) == (pass == 0 ? lbq::WK_I4G128 : lbq::WK_I2G64)) {
          const int j = ca + cb;
          ws[j] = view_of(&descs[i], &qs[i]);
          ys[j] = Ys[i];
          lds[j] = ldys[i];
          rows[j] = qs[i].out_rows;
          (pass == 0 ? ca : cb)++;
        }
    if (ca > 0 && cb > 0 && ca + cb == count) {
      if (m == 1)
        return hip_status(lbq::launch_gemv1_mix(ws, ys, rows, ca, cb, X, nf4_table(), s), "lbq_linear_fwd_grouped");
      if (gemvm_mix_set(count, descs, m))
        return hip_status(lbq::launch_gemvm_mix(ws, ys, lds, rows, ca, cb, X, m, nf4_table(), s),
                          "lbq_linear_fwd_grouped");
      return hip_status(lbq::launch_skinny_mix(ws, ys, lds, rows, ca, cb, X, m, static_cast<float*>(workspace),
                                               nf4_table(), s),
                        "lbq_linear_fwd_grouped");
    }
  }
  // One launch per distinct (weight kind, kernel) pair, in order of first
  // appearance, with the kernel lbq_linear_fwd picks for each weight (all
  // weights share k).
  bool done[LBQ_MAX_GROUP] = {};
  for (int32_t i = 0; i < count && e == hipSuccess; ++i) {
    if (done[i]) continue;
    const lbq::WKind kind = kind_of(&descs[i]);
    const bool gemvm = use_gemvm(&descs[i], m);
    lbq::WView ws[LBQ_MAX_GROUP];
    uint16_t* ys[LBQ_MAX_GROUP];
    int64_t lds[LBQ_MAX_GROUP];
    const int32_t* rows[LBQ_MAX_GROUP];
    int c = 0;
    for (int32_t j = i; j < count; ++j) {
      if (done[j] || kind_of(&descs[j]) != kind || use_gemvm(&descs[j], m) != gemvm) continue;
      done[j] = true;
      ws[c] = view_of(&descs[j], &qs[j]);
      ys[c] = Ys[j];
      lds[c] = ldys[j];
      rows[c] = qs[j].out_rows;
      ++c;
    }
    if (m == 1) e = lbq::launch_gemv1(kind, ws, ys, rows, c, X, none, nf4_table(), s);
    else if (gemvm) e = lbq::launch_gemvm(kind, ws, ys, lds, rows, c, X, m, none, nf4_table(), s);
    else if (m <= lbq::kSkinnyMaxM)
      e = lbq::launch_skinny_set(kind, ws, ys, lds, rows, c, X, m, static_cast<float*>(workspace), nf4_table(), s);
    else {
      int64_t ns[LBQ_MAX_GROUP];
      for (int j = 0; j < c; ++j) ns[j] = ws[j].n;
      e = lbq::launch_gemm_fwd_set(kind, ws, ys, lds, rows, c, X, m,
                                   gemm_part(ns, c, descs[i].k, m, workspace, ws_bytes), nf4_table(), s);
    }
  }
  return hip_status(e, "lbq_linear_fwd_grouped");
}

lbq_status lbq_linear_bwd_dx(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* dY,
                             int64_t m, uint16_t* dX, void* stream) {
  lbq_status st = check_bwd_common(desc, q, dY, m, dX, "lbq_linear_bwd_dx");
  if (st != LBQ_OK || m == 0) return st == LBQ_OK ? ok() : st;
  const lbq::LoraDx none{nullptr, nullptr, 0, 0};
  return hip_status(lbq::launch_bwd_dx(kind_of(desc), view_of(desc, q), dY, m, dX, none, nf4_table(),
                                       static_cast<hipStream_t>(stream)),
                    "lbq_linear_bwd_dx");
}

lbq_status lbq_linear_bwd_dx_grouped(int32_t count, const lbq_desc* descs, const lbq_qtensor* qs,
                                     const uint16_t* const* dYs, int64_t m, uint16_t* dX, void* stream) {
  if (count < 1 || count > LBQ_MAX_GROUP)
    return fail(LBQ_E_SHAPE, "count must be in [1, %d] (got %d)", LBQ_MAX_GROUP, count);
  if (descs == nullptr || qs == nullptr || dYs == nullptr) return fail(LBQ_E_NULL, "descs, qs and dYs must be non-NULL");
  for (int32_t i = 0; i < count; ++i) {
    const lbq_status st = check_bwd_common(&descs[i], &qs[i], dYs[i], m, dX, "lbq_linear_bwd_dx_grouped");
    if (st != LBQ_OK) return st;
    if (descs[i].k != descs[0].k)
      return fail(LBQ_E_SHAPE, "weight %d has k = %lld, weight 0 has %lld", i, (long long)descs[i].k,
                  (long long)descs[0].k);
    if (kind_of(&descs[i]) != kind_of(&descs[0]))
      return fail(LBQ_E_UNSUPPORTED, "lbq_linear_bwd_dx_grouped takes weights of one format (weight %d differs)", i);
  }
  if (m == 0) return ok();
  lbq::WView ws[LBQ_MAX_GROUP];
  for (int32_t i = 0; i < count; ++i) ws[i] = view_of(&descs[i], &qs[i]);
  return hip_status(lbq::launch_bwd_dx_set(kind_of(&descs[0]), ws, dYs, count, m, dX, nf4_table(),
                                           static_cast<hipStream_t>(stream)),
                    "lbq_linear_bwd_dx_grouped");
}

// LoRA backward workspace (16-byte aligned pieces): Bt = B^T [rp][n] bf16,
// G = bf16(sigma dY B) [m][rp], T = bf16(sigma X A^T) [m][rp], then the fp32
// partial sums of the dA / dB reductions (reused by both).
static size_t align16(size_t b) { return (b + 15) / 16 * 16; }

// LoRA backward workspace: Bt [rp][n], G [m][rp], Gt and Tt [rp][mp] (bf16),
// then fp32 partial sums shared by the four reductions (they run in turn).
size_t lbq_lora_bwd_workspace_bytes(const lbq_desc* desc, int64_t m, int32_t r) {
  if (check_desc(desc) != LBQ_OK || m <= 0 || r < 1 || r > 64) return 0;
  const size_t rp = (size_t)round_rank(r);
  const size_t mp = (size_t)round_rows(m);
  // the two adapter products run together, then the two outer products
  const size_t part = std::max(lbq::lora_xa_part_bytes(m, desc->n, r) + lbq::lora_xa_part_bytes(m, desc->k, r),
                               lbq::lora_outer_part_bytes(m, desc->k, r) + lbq::lora_outer_part_bytes(m, desc->n, r));
  return align16(rp * (size_t)desc->n * 2) + align16((size_t)m * rp * 2) + 2 * align16(rp * mp * 2) + align16(part);
}

lbq_status lbq_lora_bwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                        const uint16_t* dY, int64_t m, const uint16_t* A, const uint16_t* B,
                        int32_t r, float sigma, uint16_t* dX, float* dA, float* dB,
                        void* workspace, size_t ws_bytes, void* stream) {
  lbq_status st = check_bwd_common(desc, q, dY, m, dX, "lbq_lora_bwd");
  if (st != LBQ_OK) return st;
  if (r < 1 || r > 64) return fail(LBQ_E_SHAPE, "LoRA rank r must be in [1, 64] (got %d)", r);
  if (A == nullptr || B == nullptr || dA == nullptr || dB == nullptr)
    return fail(LBQ_E_NULL, "A, B, dA and dB must be non-NULL");
  if (!std::isfinite(sigma)) return fail(LBQ_E_SHAPE, "sigma must be finite");
  if (!aligned(dA, 4) || !aligned(dB, 4)) return fail(LBQ_E_ALIGN, "dA and dB must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m == 0) {  // an empty batch has zero adapter gradients
    hipError_t e = lbq::launch_fill_zero_f32(dA, (int64_t)r * desc->k, s);
    if (e == hipSuccess) e = lbq::launch_fill_zero_f32(dB, desc->n * (int64_t)r, s);
    return hip_status(e, "lbq_lora_bwd (empty batch)");
  }
  if (X == nullptr) return fail(LBQ_E_NULL, "X must be non-NULL");
  if (!aligned(X, 16) || !aligned(A, 16)) return fail(LBQ_E_ALIGN, "X and A must be 16-byte aligned");
  if (!aligned(B, 2)) return fail(LBQ_E_ALIGN, "B must be 2-byte aligned");
  if (desc->n % 64 != 0) return fail(LBQ_E_SHAPE, "lbq_lora_bwd needs n %% 64 == 0 (got %lld)", (long long)desc->n);
  const size_t need = lbq_lora_bwd_workspace_bytes(desc, m, r);
  if (workspace == nullptr || ws_bytes < need) return fail(LBQ_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned(workspace, 16)) return fail(LBQ_E_ALIGN, "workspace must be 16-byte aligned");
  const int32_t rp = round_rank(r);
  const int64_t mp = round_rows(m);
  uint8_t* p = static_cast<uint8_t*>(workspace);
  uint16_t* Bt = reinterpret_cast<uint16_t*>(p);
  p += align16((size_t)rp * (size_t)desc->n * 2);
  uint16_t* G = reinterpret_cast<uint16_t*>(p);
  p += align16((size_t)m * rp * 2);
  uint16_t* Gt = reinterpret_cast<uint16_t*>(p);
  p += align16((size_t)rp * mp * 2);
  uint16_t* Tt = reinterpret_cast<uint16_t*>(p);
  p += align16((size_t)rp * mp * 2);
  float* part = reinterpret_cast<float*>(p);
  // G = bf16(sigma dY B) row-major for the input gradient and transposed for
  // dA; T = bf16(sigma X A^T) transposed for dB.
  hipError_t e = lbq::launch_transpose_b(B, desc->n, r, rp, Bt, s);
  if (e == hipSuccess) {
    const uint16_t* xs[2] = {dY, X};
    const int64_t ks[2] = {desc->n, desc->k};
    const uint16_t* as[2] = {Bt, A};
    uint16_t* trm[2] = {G, nullptr};
    uint16_t* ttr[2] = {Gt, Tt};
    e = lbq::launch_lora_xa_jobs(2, xs, ks, as, trm, ttr, m, r, rp, sigma, part, mp, s);
  }
  if (e != hipSuccess) return hip_status(e, "lbq_lora_bwd (adapter products)");
  const lbq::LoraDx lora{G, A, r, rp};
  e = lbq::launch_bwd_dx(kind_of(desc), view_of(desc, q), dY, m, dX, lora, nf4_table(), s);
  if (e != hipSuccess) return hip_status(e, "lbq_lora_bwd (input gradient)");
  {
    const uint16_t* pts[2] = {Gt, Tt};
    const uint16_t* qs2[2] = {X, dY};
    const int64_t cs[2] = {desc->k, desc->n};
    const bool tr[2] = {false, true};
    float* outs[2] = {dA, dB};
    e = lbq::launch_lora_outer_jobs(2, pts, qs2, cs, tr, outs, mp, r, m, part, s);
  }
  return hip_status(e, "lbq_lora_bwd (adapter gradients)");
}


// LoRA workspace: bf16 T = sigma X A^T [m][rp], then (16-byte aligned) fp32
// partial sums, first of T's product and then of the small-batch kernel when
// that kernel runs.
static size_t lora_t_bytes(int64_t m, int32_t r) {
  return ((size_t)m * (size_t)round_rank(r) * sizeof(uint16_t) + 15) / 16 * 16;
}

size_t lbq_lora_workspace_bytes(const lbq_desc* desc, int64_t m, int32_t r) {
  if (check_desc(desc) != LBQ_OK || m <= 0 || r < 1 || r > 64) return 0;
  return lora_t_bytes(m, r) + std::max(lbq::lora_xa_part_bytes(m, desc->k, r), fwd_workspace(desc, m, true));
}

lbq_status lbq_lora_fwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X, int64_t m,
                        const uint16_t* A, const uint16_t* B, int32_t r, float sigma, uint16_t* Y,
                        int64_t ldy, void* workspace, size_t ws_bytes, void* stream) {
  lbq_status st = check_fwd_common(desc, q, X, m, Y, ldy);
  if (st != LBQ_OK) return st;
  if (r < 1 || r > 64) return fail(LBQ_E_SHAPE, "LoRA rank r must be in [1, 64] (got %d)", r);
  if (m == 0) return ok();
  if (A == nullptr || B == nullptr) return fail(LBQ_E_NULL, "LoRA A and B must be non-NULL");
  if (!aligned(A, 16)) return fail(LBQ_E_ALIGN, "LoRA A must be 16-byte aligned");
  if (!aligned(B, 2)) return fail(LBQ_E_ALIGN, "LoRA B must be 2-byte aligned");
  if (!std::isfinite(sigma)) return fail(LBQ_E_SHAPE, "sigma must be finite");
  const size_t need = lbq_lora_workspace_bytes(desc, m, r);
  if (workspace == nullptr || ws_bytes < need) return fail(LBQ_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned(workspace, 16)) return fail(LBQ_E_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t rp = round_rank(r);
  uint16_t* T = static_cast<uint16_t*>(workspace);
  void* part = static_cast<uint8_t*>(workspace) + lora_t_bytes(m, r);
  hipError_t e = lbq::launch_lora_xa(X, m, desc->k, A, r, rp, sigma, static_cast<float*>(part), T, nullptr, m, s);
  if (e != hipSuccess) return hip_status(e, "lbq_lora_fwd (adapter product)");
  const lbq::LoraEpi lora{T, B, r, rp};
  const lbq::WView w = view_of(desc, q);
  return hip_status(dispatch_fwd(desc, w, X, m, Y, ldy, q->out_rows, lora, part, ws_bytes - lora_t_bytes(m, r), s),
                    "lbq_lora_fwd");
}

// ---- serialization --------------------------------------------------------

size_t lbq_serialized_bytes(const lbq_desc* desc) {
  if (check_desc(desc) != LBQ_OK) return 0;
  lbq_sizes z;
  sizes_of(desc, &z);
  return kBlobHeader + align16(z.packed) + align16(z.scales) + align16(z.zeros) + align16(z.absmax) +
         align16(z.absmax_q) + align16(z.absmax_scale);
}

lbq_status lbq_serialize(const lbq_desc* desc, const lbq_qtensor* q, void* blob, size_t blob_bytes,
                         void* stream) {
  lbq_status st = check_desc(desc);
  if (st != LBQ_OK) return st;
  if ((st = check_qtensor(desc, q)) != LBQ_OK) return st;
  if (blob == nullptr) return fail(LBQ_E_NULL, "blob is NULL");
  const size_t need = lbq_serialized_bytes(desc);
  if (blob_bytes < need) return fail(LBQ_E_SHAPE, "blob needs %zu bytes (got %zu)", need, blob_bytes);
  lbq_sizes z;
  sizes_of(desc, &z);
  uint8_t* b = static_cast<uint8_t*>(blob);
  std::memset(b, 0, need);
  std::memcpy(b, kBlobMagic, 4);
  const uint32_t version = kBlobVersion;
  std::memcpy(b + 4, &version, 4);
  std::memcpy(b + 8, desc, sizeof(lbq_desc));
  const uint64_t counts[6] = {z.packed, z.scales, z.zeros, z.absmax, z.absmax_q, z.absmax_scale};
  std::memcpy(b + 48, counts, sizeof(counts));
  const void* src[6] = {q->packed, q->scales, q->zeros, q->absmax, q->absmax_q, q->absmax_scale};
  hipStream_t s = static_cast<hipStream_t>(stream);
  size_t off = kBlobHeader;
  hipError_t e = hipSuccess;
  for (int i = 0; i < 6 && e == hipSuccess; ++i) {
    if (counts[i] > 0) e = hipMemcpyAsync(b + off, src[i], counts[i], hipMemcpyDeviceToHost, s);
    off += align16(counts[i]);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, "lbq_serialize");
}

lbq_status lbq_blob_desc(const void* blob, size_t blob_bytes, lbq_desc* desc) {
  if (blob == nullptr || desc == nullptr) return fail(LBQ_E_NULL, "blob and desc must be non-NULL");
  if (blob_bytes < kBlobHeader) return fail(LBQ_E_SHAPE, "blob shorter than its %zu-byte header", kBlobHeader);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  if (std::memcmp(b, kBlobMagic, 4) != 0) return fail(LBQ_E_FORMAT, "not an lbq blob (magic)");
  uint32_t version;
  std::memcpy(&version, b + 4, 4);
  if (version != kBlobVersion) return fail(LBQ_E_FORMAT, "blob version %u (this library reads %u)", version, kBlobVersion);
  lbq_desc d;
  std::memcpy(&d, b + 8, sizeof(lbq_desc));
  if (check_desc(&d) != LBQ_OK) {
    const std::string why = g_detail;
    return fail(LBQ_E_FORMAT, "blob descriptor invalid: %s", why.c_str());
  }
  lbq_sizes z;
  sizes_of(&d, &z);
  uint64_t counts[6];
  std::memcpy(counts, b + 48, sizeof(counts));
  const uint64_t want[6] = {z.packed, z.scales, z.zeros, z.absmax, z.absmax_q, z.absmax_scale};
  for (int i = 0; i < 6; ++i)
    if (counts[i] != want[i]) return fail(LBQ_E_FORMAT, "blob byte count %d is %llu, the descriptor needs %llu", i,
                                          (unsigned long long)counts[i], (unsigned long long)want[i]);
  const size_t need = lbq_serialized_bytes(&d);
  if (blob_bytes < need) return fail(LBQ_E_SHAPE, "blob holds %zu of its %zu bytes", blob_bytes, need);
  *desc = d;
  return ok();
}

lbq_status lbq_deserialize(const void* blob, size_t blob_bytes, const lbq_qtensor* q, void* stream) {
  lbq_desc d;
  lbq_status st = lbq_blob_desc(blob, blob_bytes, &d);
  if (st != LBQ_OK) return st;
  if ((st = check_qtensor(&d, q)) != LBQ_OK) return st;
  lbq_sizes z;
  sizes_of(&d, &z);
  const uint64_t counts[6] = {z.packed, z.scales, z.zeros, z.absmax, z.absmax_q, z.absmax_scale};
  void* dst[6] = {q->packed, q->scales, q->zeros, q->absmax, q->absmax_q, q->absmax_scale};
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  hipStream_t s = static_cast<hipStream_t>(stream);
  size_t off = kBlobHeader;
  hipError_t e = hipSuccess;
  for (int i = 0; i < 6 && e == hipSuccess; ++i) {
    if (counts[i] > 0) e = hipMemcpyAsync(dst[i], b + off, counts[i], hipMemcpyHostToDevice, s);
    off += align16(counts[i]);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, "lbq_deserialize");
}

void lbq_nf4_codebook(float out[16]) {
  const lbq::Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) out[i] = t.c[i];
}

const char* lbq_strerror(lbq_status s) {
  switch (s) {
    case LBQ_OK: return "ok";
    case LBQ_E_NULL: return "required pointer is NULL";
    case LBQ_E_SHAPE: return "shape out of range or inconsistent";
    case LBQ_E_FORMAT: return "unknown or unsupported quantization format";
    case LBQ_E_ALIGN: return "pointer or leading dimension misaligned";
    case LBQ_E_WORKSPACE: return "workspace missing or too small";
    case LBQ_E_UNSUPPORTED: return "request not supported by this library";
    case LBQ_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* lbq_last_error_detail(void) { return g_detail.c_str(); }

const char* lbq_version(void) { return "lbq 0.1.0 (gfx950)"; }

}  // extern "C"
