// Internal interface between the C-ABI layer (lbq_api.cpp) and the gfx950
// kernels.  Not installed; the public interface is include/lbq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbq {

enum Fmt : int { FMT_MINMAX = 0, FMT_NF4 = 1 };

// One quantized weight as the kernels see it (device pointers + shape).
// `scales` holds fp32 values, or fp16 bit patterns under compact metadata.
struct WView {
  const uint8_t* packed;
  const float* scales;
  const uint8_t* zeros;
  const float* absmax;
  const int8_t* absmax_q;
  const float* absmax_scale;
  int64_t n, k;
};

// The 16 NF4 levels, passed by value to every kernel that needs them.
struct Nf4Table {
  float c[16];
};

// LoRA epilogue operands: T = bf16(sigma * X A^T) [m][rp] (rp = r rounded up
// to a multiple of 32, zero padded) and B [n][r] bf16.  t == nullptr: none.
struct LoraEpi {
  const uint16_t* t;
  const uint16_t* b;
  int32_t r;
  int32_t rp;
};

// LoRA term of the input gradient: dX += G . A with G = bf16(sigma * dY . B)
// [m][rp] (zero past r) and A [r][k] bf16.  g == nullptr: none.
struct LoraDx {
  const uint16_t* g;
  const uint16_t* a;
  int32_t r;
  int32_t rp;
};

// Supported weight encodings (format, bits, group, double quant).
enum WKind : int {
  WK_I4G128 = 0,  // MinMax 4-bit, group 128
  WK_I4G64 = 1,   // MinMax 4-bit, group 64
  WK_I2G64 = 2,   // MinMax 2-bit, group 64
  WK_I2G128 = 3,  // MinMax 2-bit, group 128
  WK_NF4 = 4,     // NF4, block 64, fp32 absmax
  WK_NF4DQ = 5,   // NF4, block 64, int8 absmax + fp32 scale per 256 blocks
  WK_I4G128C = 6, // MinMax 4-bit, group 128, compact metadata (fp16 scale, packed zero)
  WK_I2G64C = 7,  // MinMax 2-bit, group 64, compact metadata
  WK_NF4DQO = 8,  // NF4, block 64, double quant with a per-tensor offset
};

// ---- launchers (each returns hipGetLastError() after the launch) ----------
// compact: fp16 scales and packed zero points (INT4 g128 and INT2 g64 only).
hipError_t launch_quant_minmax(int bits, int group, bool compact, const float* W, uint8_t* packed,
                               float* scales, uint8_t* zeros, int64_t n, int64_t k,
                               hipStream_t s);
// dq: 0 none, 1 double quantization, 2 double quantization with an offset.
hipError_t launch_quant_nf4(int dq, const float* W, uint8_t* packed, float* absmax,
                            int8_t* absmax_q, float* absmax_scale, int64_t n, int64_t k,
                            const Nf4Table& tab, hipStream_t s);
hipError_t launch_dequant(WKind kind, const WView& w, uint16_t* out, const Nf4Table& tab,
                          hipStream_t s);
// m == 1 decode GEMV over up to kGemvMaxGroup weights of one kind that share x
// and k (ws[i], ys[i], out_rows[i] per weight; the LoRA term only with count 1).
constexpr int kGemvMaxGroup = 8;
// m = 1, the two row sets of channel-mixed linears that share x in one launch:
// INT4 g128 weights ws[0, count_a), INT2 g64 weights ws[count_a, count_a +
// count_b) (same k); outputs equal those of the two per-format launches.
hipError_t launch_gemv1_mix(const WView* ws, uint16_t* const* ys, const int32_t* const* out_rows, int count_a,
                            int count_b, const uint16_t* X, const Nf4Table& tab, hipStream_t s);
hipError_t launch_gemv1(WKind kind, const WView* ws, uint16_t* const* ys, const int32_t* const* out_rows,
                        int count, const uint16_t* X, const LoraEpi& lora, const Nf4Table& tab,
                        hipStream_t s);
// 2 <= m <= kGemvmMaxM: the GEMV streaming of up to kGemvMaxGroup weights of
// one kind with every row of x staged in LDS (usable when gemvm_fits; the
// LoRA term only with count 1).
constexpr int64_t kGemvmMaxM = 4;
bool gemvm_fits(WKind kind, int64_t k, int64_t m);
hipError_t launch_gemvm(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                        const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m,
                        const LoraEpi& lora, const Nf4Table& tab, hipStream_t s);
// The INT4 g128 weights ws[0, count_a) and INT2 g64 weights ws[count_a,
// count_a + count_b) (same k, both fitting the multi-row GEMV at m) in one
// multi-row launch; outputs equal those of the two per-format launches.
hipError_t launch_gemvm_mix(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* out_rows,
                            int count_a, int count_b, const uint16_t* X, int64_t m, const Nf4Table& tab,
                            hipStream_t s);
// 2 <= m <= kSkinnyMaxM: MFMA with the weight streamed once; K split over
// skinny_splits() workgroups whose fp32 partials (workspace) are summed by a
// second kernel when more than one range is used or a LoRA term is added.
int skinny_splits(int64_t n, int64_t k, int64_t m);
int skinny_splits_tiles(int64_t tiles, int64_t k, int64_t m);
// True when the small-batch kernel runs an n x k weight at m unsplit because
// its row tiles alone fill the chip (then skinny_splits() == 1).
bool skinny_fills_unsplit(int64_t n, int64_t k, int64_t m);
// Weights of one kind that share X (count <= kGemvMaxGroup, same k): one
// launch over all their row tiles and, when K is split, one reduce launch.
// Workspace: skinny_set_workspace_bytes() bytes of fp32 partials.
size_t skinny_set_workspace_bytes(const int64_t* ns, int count, int64_t k, int64_t m);
hipError_t launch_skinny_set(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                             const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m, float* part,
                             const Nf4Table& tab, hipStream_t s);
// The INT4 g128 weights ws[0, count_a) and INT2 g64 weights ws[count_a,
// count_a + count_b) (same k) in one small-batch launch (plus one reduce),
// each weight with the K split it has alone: outputs equal the per-format
// launches'.  Workspace: skinny_set_workspace_bytes() over all the weights.
hipError_t launch_skinny_mix(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* out_rows,
                             int count_a, int count_b, const uint16_t* X, int64_t m, float* part, const Nf4Table& tab,
                             hipStream_t s);
size_t skinny_workspace_bytes(int64_t n, int64_t k, int64_t m, bool lora);
hipError_t launch_skinny(WKind kind, const WView& w, const uint16_t* X, int64_t m, uint16_t* Y,
                         int64_t ldy, const int32_t* out_rows, float* part, const LoraEpi& lora,
                         const Nf4Table& tab, hipStream_t s);
// m > kSkinnyMaxM: the MFMA GEMM.  With `part` (at least
// gemm_fwd_workspace_bytes() bytes, 16-byte aligned) a weight whose tiles
// fill at most half the chip splits K over several workgroups, whose fp32
// partials a second kernel sums; with part == nullptr nothing splits.
size_t gemm_fwd_workspace_bytes(const int64_t* ns, int count, int64_t k, int64_t m);
hipError_t launch_gemm_fwd(WKind kind, const WView& w, const uint16_t* X, int64_t m,
                           uint16_t* Y, int64_t ldy, const int32_t* out_rows,
                           const LoraEpi& lora, float* part, const Nf4Table& tab, hipStream_t s);
// m > kSkinnyMaxM over up to kGemvMaxGroup weights of one kind that share X
// (their column tiles side by side in one launch; each weight keeps the K
// split it has alone, so its outputs equal the single-weight call's).
hipError_t launch_gemm_fwd_set(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                               const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m,
                               float* part, const Nf4Table& tab, hipStream_t s);
hipError_t launch_bwd_dx(WKind kind, const WView& w, const uint16_t* dY, int64_t m,
                         uint16_t* dX, const LoraDx& lora, const Nf4Table& tab, hipStream_t s);
// Input gradient of several weights of one kind and k that share X, summed:
// dX = sum_i dys[i] . deq(ws[i]), 1 <= count <= kGemvMaxGroup.
hipError_t launch_bwd_dx_set(WKind kind, const WView* ws, const uint16_t* const* dys, int count, int64_t m,
                             uint16_t* dX, const Nf4Table& tab, hipStream_t s);
// Adapter products and gradients (k_lora.hip).
// Bt = B^T zero-padded to rp rows.
hipError_t launch_transpose_b(const uint16_t* B, int64_t n, int32_t r, int32_t rp, uint16_t* Bt,
                              hipStream_t s);
// T = bf16(sigma * X . A^T) (X [m][K], A [r][K]) into Trm [m][rp] and/or the
// transposed Ttr [rp][mp] (mp >= m, a multiple of 32), zero past r and past m;
// either output may be null.  `part` holds lora_xa_part_bytes(m, K, r) bytes.
size_t lora_xa_part_bytes(int64_t m, int64_t K, int32_t r);
hipError_t launch_lora_xa(const uint16_t* X, int64_t m, int64_t K, const uint16_t* A, int32_t r,
                          int32_t rp, float sigma, float* part, uint16_t* Trm, uint16_t* Ttr,
                          int64_t mp, hipStream_t s);
// out = sum over rows t < m of Pt[j][t] * Q[t][c] (Pt [rp][mp], zero past m;
// Q [m][C], C % 8 == 0), fp32 [r][C], or [C][r] with transpose.  `part`
// holds lora_outer_part_bytes(m, C, r) bytes.
// The same for count = 1 or 2 products in one launch pair, jobs[i] = (Xs[i],
// Ks[i], As[i]) -> (Trms[i], Ttrs[i]); `part` holds the sum of their
// lora_xa_part_bytes.
hipError_t launch_lora_xa_jobs(int count, const uint16_t* const* Xs, const int64_t* Ks, const uint16_t* const* As,
                               uint16_t* const* Trms, uint16_t* const* Ttrs, int64_t m, int32_t r, int32_t rp,
                               float sigma, float* part, int64_t mp, hipStream_t s);
size_t lora_outer_part_bytes(int64_t m, int64_t C, int32_t r);
hipError_t launch_lora_outer(const uint16_t* Pt, int64_t mp, int32_t r, const uint16_t* Q, int64_t m,
                             int64_t C, bool transpose, float* part, float* out, hipStream_t s);
// The same for count = 1 or 2 outer products in one launch pair; `part` holds
// the sum of their lora_outer_part_bytes.
hipError_t launch_lora_outer_jobs(int count, const uint16_t* const* Pts, const uint16_t* const* Qs,
                                  const int64_t* Cs, const bool* transposes, float* const* outs, int64_t mp,
                                  int32_t r, int64_t m, float* part, hipStream_t s);
hipError_t launch_fill_zero_f32(float* p, int64_t count, hipStream_t s);

// Largest m served by the small-batch MFMA kernel.
constexpr int64_t kSkinnyMaxM = 64;

}  // namespace lbq

// C-ABI helpers shared between lbq_api.cpp and the allocation-free forward
// (k_noalloc.hip); the types come from include/lbq.h.
#include "lbq.h"

namespace lbq {

// Records `what` as the detail of the calling thread's last failure; returns s.
lbq_status set_error(lbq_status s, const char* what);
// Argument checks of lbq_linear_fwd (everything but the workspace).
lbq_status check_fwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X, int64_t m, uint16_t* Y,
                     int64_t ldy);
// lbq_linear_fwd after check_fwd: workspace check and dispatch (`who` names
// the entry point in error details).
lbq_status linear_fwd_body(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X, int64_t m,
                           uint16_t* Y, int64_t ldy, void* workspace, size_t ws_bytes, void* stream,
                           const char* who);

}  // namespace lbq
