// Prefill / training-size forward (m > 4): Y = X . deq(W)^T (+ LoRA) on bf16
// MFMA (v_mfma_f32_16x16x32_bf16) with LDS-staged, double-buffered tiles.
//
// bitsandbytes FSDP-QLoRA guide, section 通过BitsAndBytesConfig配置: the packed
// weight is unpacked and dequantized to the bf16 compute dtype inside the
// kernel that does the matmul.  LoRA: same guide, step 4 (LoraConfig), and
// "QLoRA技术在量化微调中的应用", section QLoRA技术原理 (low-rank adapters on a
// frozen 4-bit base).
//
// Workgroup tile: BN rows of W (output columns) x BM rows of X, K-step 64.
// Per K-step each thread fetches 32 packed codes of one W row (16 bytes for
// 4-bit, 8 for 2-bit) and a few 16-byte chunks of X, dequantizes the codes in
// registers (one fp32 FMA per weight, hardware bf16 packing) and writes both
// into the idle half of a double-buffered LDS tile while the MFMAs consume the
// other half; one barrier per K-step.  The packed weight is therefore read
// from memory once per workgroup tile at a quarter (4-bit) or an eighth
// (2-bit) of its bf16 size, and dequantized exactly once per tile.
//
// MFMA operand A is the weight (rows n), B is X (rows m); a lane's four
// accumulators are four consecutive n of one m, so the epilogue writes 8
// contiguous bytes of a Y row.  Workgroups are renumbered so that each of the
// 8 XCDs (each with its own L2) receives a contiguous run of tiles, walked in
// groups of 2 X-row tiles so that concurrently running tiles share operands.
#include "lbq_device.h"

namespace lbq {

namespace {

constexpr int BK = 64;  // K per LDS stage: one tile row is 128 bytes


// 32 codes of one row -> 16 dwords of bf16 pairs (element 2i in the low half).
// MinMax: (q - z) * s evaluated as fma(q, s, -z*s); NF4: c[code] * a.
template <int KIND>
__device__ __forceinline__ void dequant32(const u32x4_t& raw, float s, float zs,
                                          const f32x2_t* __restrict__ pairlut, uint32_t out[16]) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_MINMAX && T::bits == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t ev = (raw[d] >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 of the dword
      const uint32_t od = raw[d] & 0x0F0F0F0Fu;         // elements 1,3,5,7
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float qe = (float)((ev >> (8 * i)) & 0xFFu);
        const float qo = (float)((od >> (8 * i)) & 0xFFu);
        out[4 * d + i] = cvt_pk_bf16(fmaf(qe, s, -zs), fmaf(qo, s, -zs));
      }
    }
  } else if constexpr (T::fmt == FMT_MINMAX) {
    // 2-bit: 32 codes in raw[0..1]; byte j of a dword holds elements 4j..4j+3, first in bits 7..6
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t c0 = (raw[d] >> 6) & 0x03030303u, c1 = (raw[d] >> 4) & 0x03030303u;
      const uint32_t c2 = (raw[d] >> 2) & 0x03030303u, c3 = raw[d] & 0x03030303u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float q0 = (float)((c0 >> (8 * j)) & 0xFFu), q1 = (float)((c1 >> (8 * j)) & 0xFFu);
        const float q2 = (float)((c2 >> (8 * j)) & 0xFFu), q3 = (float)((c3 >> (8 * j)) & 0xFFu);
        out[8 * d + 2 * j] = cvt_pk_bf16(fmaf(q0, s, -zs), fmaf(q1, s, -zs));
        out[8 * d + 2 * j + 1] = cvt_pk_bf16(fmaf(q2, s, -zs), fmaf(q3, s, -zs));
      }
    }
  } else {
    // NF4: byte -> (c[hi nibble], c[lo nibble]) from an LDS table, times the block absmax s
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2_t c = pairlut[(raw[d] >> (8 * i)) & 0xFFu];
        out[4 * d + i] = cvt_pk_bf16(c[0] * s, c[1] * s);
      }
  }
}

// LDS of one workgroup, declared by the kernel and handed to the tile code.
template <int BN, int BM>
struct GemmLds {
  uint16_t Ws[2][BN * BK];
  uint16_t Xs[2][BM * BK];
  f32x2_t pairlut[256];  // NF4 byte -> codebook pair
  float cbs[16];
};

// One BN x BM output tile (tx, ty) of Y = X . deq(W)^T (+ the LoRA slab).
template <int KIND, int BN, int BM, int WGN, int WGM, bool LORA>
__device__ __forceinline__ void gemm_fwd_tile(const WView& w, const uint16_t* __restrict__ X, int m,
                                              uint16_t* __restrict__ Y, int64_t ldy,
                                              const int32_t* __restrict__ out_rows,
                                              const LoraEpi& lora, const Nf4Table& tab, int tx, int ty,
                                              GemmLds<BN, BM>& lds) {
  using T = WKindTraits<KIND>;
  constexpr int NT = WGN * WGM * 64;
  constexpr int CPT = BN * BK / NT;  // codes of one W row a thread dequantizes per stage
  constexpr int NQ = CPT / 32;       // 32-code pieces per thread
  static_assert(CPT == 32 || CPT == 64, "a thread owns 32 or 64 codes of one W row per stage");
  constexpr int WN = BN / WGN, WM = BM / WGM;
  constexpr int TN = WN / 16, TM = WM / 16;
  constexpr int XCH = BM * BK / 8 / NT;  // 16-byte X chunks per thread per stage
  static_assert(XCH * NT * 8 == BM * BK, "X tile split");

  auto& Ws = lds.Ws;
  auto& Xs = lds.Xs;
  f32x2_t* const pairlut = lds.pairlut;
  float* const cbs = lds.cbs;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WGN, wm = wave / WGN;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t n0 = (int64_t)tx * BN;
  const int64_t m0 = (int64_t)ty * BM;
  const int64_t K = w.k;
  const int64_t KB = K * T::bits / 8;
  const bool vec_store = out_rows == nullptr && (ldy & 3) == 0 &&
                         (reinterpret_cast<uintptr_t>(Y) & 7) == 0;

  if constexpr (T::fmt == FMT_NF4) {
    // constant indices keep the kernel-argument table out of scratch memory
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tid == i) cbs[i] = tab.c[i];
    __syncthreads();
    for (int b = tid; b < 256; b += NT) pairlut[b] = (f32x2_t){cbs[b >> 4], cbs[b & 15]};
  }

  // W ownership: row n0 + wrow, codes [CPT*wpart, +CPT) of each stage.
  const int wrow = tid / (BK / CPT), wpart = tid % (BK / CPT);
  const int64_t wn_g = n0 + wrow;
  const bool wrow_ok = wn_g < w.n;  // rows past n read row 0 and are zeroed
  const uint8_t* wsrc = w.packed + (wrow_ok ? wn_g : 0) * KB;
  const int64_t gpr = K / T::group;  // groups (or absmax blocks) per row
  const int64_t grow = (wrow_ok ? wn_g : 0) * gpr;

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prefetch registers.  Code and X loads are unconditional from clamped
  // addresses (no branches, so they are all in flight at once).  Metadata is
  // loaded at the first stage of each group, or of each batch of 4 groups (a
  // branch that every lane takes alike); it stays raw here and is combined in
  // store_stage, one K-step later, so no wave waits on it.
  u32x4_t xr[XCH];
  u32x4_t wr[NQ];
  float md_s = 0.f;  // scale (MinMax), absmax or second-level scale (NF4)
  int md_i = 0;      // zero point (MinMax) or int8 absmax code (NF4 + DQ)
  // When every row's metadata starts 16-byte aligned (groups per row a
  // multiple of 4, aligned arrays), the entries of 4 consecutive groups are
  // loaded together once per 4 groups: one 16-byte load of scales or absmax
  // and one 4-byte load of zero points or absmax codes, instead of two small
  // loads per stage.  The stage picks its entry in store_stage.
  const float* const mf_arr = T::fmt == FMT_MINMAX ? w.scales : (T::dq ? nullptr : w.absmax);
  const uint8_t* const mb_arr =
      T::fmt == FMT_MINMAX ? w.zeros : (T::dq ? reinterpret_cast<const uint8_t*>(w.absmax_q) : nullptr);
  const bool md4 = (gpr & 3) == 0 && (reinterpret_cast<uintptr_t>(mf_arr) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(mb_arr) & 3) == 0;
  float mb0 = 0.f, mb1 = 0.f, mb2 = 0.f, mb3 = 0.f;  // scales / absmax of the batch
  uint32_t mb_b = 0;                                 // zero points / absmax codes of the batch
  int md_j = 0;  // entry of the loaded stage in the batch (the same in every lane)
  auto load_stage = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + NT * i;
      const int row = c >> 3, col = (c & 7) * 8;
      const int64_t mr = min(m0 + row, (int64_t)m - 1);
      xr[i] = *reinterpret_cast<const u32x4_t*>(X + mr * K + kt + col);
    }
    const int64_t kk = kt + CPT * wpart;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if constexpr (T::bits == 4) {
        wr[q] = *reinterpret_cast<const u32x4_t*>(wsrc + (kk + 32 * q) / 2);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(wsrc + (kk + 32 * q) / 4);
        wr[q] = u32x4_t{v.x, v.y, 0u, 0u};
      }
    }
    const int64_t gi = grow + kk / T::group;
    // Both forms fill the batch registers (the per-stage form as entry 0), so
    // the same variables are written either way.
    md_j = md4 ? (int)((kt / T::group) & 3) : 0;  // rows start at multiples of 4 entries
    if (md_j == 0 && kt % T::group == 0) {       // first stage of a batch or group (uniform)
      if (md4) {
        if constexpr (T::fmt != FMT_NF4 || !T::dq) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(mf_arr + gi);
          mb0 = v[0], mb1 = v[1], mb2 = v[2], mb3 = v[3];
        }
        if constexpr (T::fmt == FMT_MINMAX || T::dq) mb_b = *reinterpret_cast<const uint32_t*>(mb_arr + gi);
      } else {
        if constexpr (T::fmt != FMT_NF4 || !T::dq) {
          const float v = mf_arr[gi];
          mb0 = v, mb1 = v, mb2 = v, mb3 = v;
        }
        if constexpr (T::fmt == FMT_MINMAX || T::dq) mb_b = mb_arr[gi];
      }
      if constexpr (T::dq) md_s = w.absmax_scale[gi >> 8];  // a batch never straddles a 256-block one
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + NT * i;
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(&Xs[buf][0]) + swz(c >> 3, c & 7)) = xr[i];
    }
    {
      const float f01 = (md_j & 1) ? mb1 : mb0, f23 = (md_j & 1) ? mb3 : mb2;
      if constexpr (!T::dq) md_s = (md_j & 2) ? f23 : f01;
      if constexpr (T::fmt == FMT_MINMAX) md_i = (int)((mb_b >> (8 * md_j)) & 0xFFu);
      if constexpr (T::dq) md_i = (int)(int8_t)(uint8_t)((mb_b >> (8 * md_j)) & 0xFFu);
    }
    float ws_s, ws_zs = 0.f;
    if constexpr (T::fmt == FMT_MINMAX) {
      ws_s = md_s;
      ws_zs = (float)md_i * md_s;
    } else if constexpr (T::dq) {
      ws_s = (float)md_i * md_s;
    } else {
      ws_s = md_s;
    }
    if (!wrow_ok) ws_s = ws_zs = 0.f;  // rows past n contribute zeros
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      uint32_t d[16];
      dequant32<KIND>(wr[q], ws_s, ws_zs, pairlut, d);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(&Ws[buf][0]) +
                                    swz(wrow, (CPT / 8) * wpart + 4 * q + j)) =
            u32x4_t{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
    }
  };
  // Operand rows of this lane: W rows wn*WN + 16*a + li, X rows wm*WM + 16*b + li
  // (row & 7 == li & 7), chunk 4*(ks/32) + lg of each.
  const uint32_t a_base = swz(wn * WN + li, lg), a_base1 = swz(wn * WN + li, 4 + lg);
  const uint32_t b_base = swz(wm * WM + li, lg), b_base1 = swz(wm * WM + li, 4 + lg);
  auto compute = [&](int buf) {
    const char* wsb = reinterpret_cast<const char*>(&Ws[buf][0]);
    const char* xsb = reinterpret_cast<const char*>(&Xs[buf][0]);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      u32x4_t af[TN], bf[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a)
        af[a] = *reinterpret_cast<const u32x4_t*>(wsb + (ks ? a_base1 : a_base) + a * 16 * 128);
#pragma unroll
      for (int b = 0; b < TM; ++b)
        bf[b] = *reinterpret_cast<const u32x4_t*>(xsb + (ks ? b_base1 : b_base) + b * 16 * 128);
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma16x16x32(af[a], bf[b], acc[a][b]);
    }
  };

  if constexpr (T::fmt == FMT_NF4) __syncthreads();  // pair table visible
  load_stage(0);
  store_stage(0);
  if (BK < K) load_stage(BK);
  __syncthreads();
  int buf = 0;
  if constexpr (WGN * WGM == 8 && BM == 256) {
    // Two phases per stage, with a barrier between them: the first four waves
    // stage the next tile while the last four run their MFMAs, then the other
    // way round.  Waves w and w + 4 share a SIMD, so at any time one of them
    // feeds the matrix core (at raised priority) while the other does the
    // dequant and LDS writes.  (With 128-row X tiles a wave's MFMA phase is
    // no longer than its staging, and the extra barrier costs more than the
    // overlap gains.)
    const bool late = wave >= 4;
    auto stage = [&](int64_t t) {
      if (t + BK < K) {
        store_stage(buf ^ 1);
        if (t + 2 * BK < K) load_stage(t + 2 * BK);
      }
    };
    auto mfma_phase = [&]() {
      __builtin_amdgcn_s_setprio(1);
      compute(buf);
      __builtin_amdgcn_s_setprio(0);
    };
    for (int64_t kt = 0; kt < K; kt += BK) {
      if (late) mfma_phase();
      else stage(kt);
      __syncthreads();
      if (late) stage(kt);
      else mfma_phase();
      __syncthreads();
      buf ^= 1;
    }
  } else {
    for (int64_t kt = 0; kt < K; kt += BK) {
      if (kt + BK < K) {
        store_stage(buf ^ 1);
        if (kt + 2 * BK < K) load_stage(kt + 2 * BK);
      }
      compute(buf);
      __syncthreads();
      buf ^= 1;
    }
  }

  // LoRA slab: acc += B_lora[n][:] . T[m][:], r zero-padded to rp (multiple of 32).
  if constexpr (LORA) {
    for (int ks = 0; ks < lora.rp; ks += 32) {
      u32x4_t af[TN], bf[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int64_t n = n0 + wn * WN + 16 * a + li;
        uint32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c0 = ks + 8 * lg + 2 * j;
          uint32_t lo = 0, hi = 0;
          if (n < w.n && c0 < lora.r) lo = lora.b[n * lora.r + c0];
          if (n < w.n && c0 + 1 < lora.r) hi = lora.b[n * lora.r + c0 + 1];
          v[j] = lo | (hi << 16);
        }
        af[a] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const int64_t mr = m0 + wm * WM + 16 * b + li;
        bf[b] = (mr < m) ? *reinterpret_cast<const u32x4_t*>(lora.t + mr * lora.rp + ks + 8 * lg)
                         : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma16x16x32(af[a], bf[b], acc[a][b]);
    }
  }

  // Epilogue: lane holds D[n = base + 4*lg + i][m = base + li], i = 0..3.
  if (out_rows != nullptr) {
    // Scattered columns: the lane's 4*TN target columns are loaded together,
    // once (clamped indices; columns past n are never stored).
    int32_t col[TN][4];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + wn * WN + 16 * a + 4 * lg + i;
        col[a][i] = out_rows[n < w.n ? n : w.n - 1];
      }
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int64_t nb = n0 + wn * WN + 16 * a + 4 * lg;
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const int64_t mr = m0 + wm * WM + 16 * b + li;
        if (mr >= m) continue;
        uint16_t* yrow = Y + mr * ldy;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nb + i < w.n) yrow[col[a][i]] = (uint16_t)bf16_rne(acc[a][b][i]);
      }
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int64_t nb = n0 + wn * WN + 16 * a + 4 * lg;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int64_t mr = m0 + wm * WM + 16 * b + li;
      if (mr >= m) continue;
      uint16_t* yrow = Y + mr * ldy;
      if (vec_store && nb + 3 < w.n) {
        uint2 v;
        v.x = cvt_pk_bf16(acc[a][b][0], acc[a][b][1]);
        v.y = cvt_pk_bf16(acc[a][b][2], acc[a][b][3]);
        *reinterpret_cast<uint2*>(yrow + nb) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nb + i < w.n) yrow[nb + i] = (uint16_t)bf16_rne(acc[a][b][i]);
      }
    }
  }
}

template <int KIND, int BN, int BM, int WGN, int WGM, bool LORA>
__global__ __launch_bounds__(WGN* WGM * 64) void k_gemm_fwd(WView w, const uint16_t* __restrict__ X,
                                                          int m, uint16_t* __restrict__ Y,
                                                          int64_t ldy,
                                                          const int32_t* __restrict__ out_rows,
                                                          LoraEpi lora, Nf4Table tab) {
  const int nx = (int)((w.n + BN - 1) / BN), ny = (m + BM - 1) / BM;
  int tx, ty;
  tile_of(blockIdx.x, nx, ny, tx, ty);
  __shared__ __attribute__((aligned(16))) GemmLds<BN, BM> lds;
  gemm_fwd_tile<KIND, BN, BM, WGN, WGM, LORA>(w, X, m, Y, ldy, out_rows, lora, tab, tx, ty, lds);
}

// Several weights that share X: their column tiles are laid side by side
// (weight i owns tile columns [tile_end[i-1], tile_end[i])), so one launch
// covers them all and its last round of tiles is shared.
struct GemmSet {
  WView w[kGemvMaxGroup];
  uint16_t* y[kGemvMaxGroup];
  int64_t ldy[kGemvMaxGroup];
  const int32_t* out_rows[kGemvMaxGroup];
  int tile_end[kGemvMaxGroup];
  int count;
};

template <int KIND, int BN, int BM, int WGN, int WGM>
__global__ __launch_bounds__(WGN* WGM * 64) void k_gemm_fwd_set(GemmSet set, const uint16_t* __restrict__ X,
                                                              int m, Nf4Table tab) {
  int nx = set.tile_end[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count) nx = set.tile_end[i];
  int tx, ty;
  tile_of(blockIdx.x, nx, (m + BM - 1) / BM, tx, ty);
  int pi = 0, tbeg = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count && tx >= set.tile_end[i - 1]) { pi = i; tbeg = set.tile_end[i - 1]; }
  const LoraEpi none{nullptr, nullptr, 0, 0};
  __shared__ __attribute__((aligned(16))) GemmLds<BN, BM> lds;
  gemm_fwd_tile<KIND, BN, BM, WGN, WGM, false>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi],
                                               none, tab, tx - tbeg, ty, lds);
}

template <int KIND, int BN, int BM, int WGN, int WGM>
hipError_t launch_set_cfg(const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                          const int32_t* const* orows, int count, const uint16_t* X, int64_t m,
                          const Nf4Table& tab, hipStream_t s) {
  GemmSet set{};
  set.count = count;
  int64_t nx = 0;
  for (int i = 0; i < count; ++i) {
    nx += (ws[i].n + BN - 1) / BN;
    set.w[i] = ws[i];
    set.y[i] = ys[i];
    set.ldy[i] = ldys[i];
    set.out_rows[i] = orows[i];
    set.tile_end[i] = (int)nx;
  }
  const dim3 grid((unsigned)(nx * ((m + BM - 1) / BM))), block(WGN * WGM * 64);
  hipLaunchKernelGGL((k_gemm_fwd_set<KIND, BN, BM, WGN, WGM>), grid, block, 0, s, set, X, (int)m, tab);
  return hipGetLastError();
}

template <int KIND, int BN, int BM, int WGN, int WGM>
hipError_t launch_cfg(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                      const int32_t* out_rows, const LoraEpi& lora, const Nf4Table& tab,
                      hipStream_t s) {
  const int64_t tiles = ((w.n + BN - 1) / BN) * ((m + BM - 1) / BM);
  const dim3 grid((unsigned)tiles), block(WGN * WGM * 64);
  if (lora.t != nullptr) {
    hipLaunchKernelGGL((k_gemm_fwd<KIND, BN, BM, WGN, WGM, true>), grid, block, 0, s, w, X, (int)m,
                       Y, ldy, out_rows, lora, tab);
  } else {
    hipLaunchKernelGGL((k_gemm_fwd<KIND, BN, BM, WGN, WGM, false>), grid, block, 0, s, w, X, (int)m,
                       Y, ldy, out_rows, lora, tab);
  }
  return hipGetLastError();
}

// Fraction of the chip's 256 CUs kept busy by `tiles` one-per-CU workgroups.
double fill(int64_t tiles) {
  const int64_t waves = (tiles + 255) / 256;
  return (double)tiles / (double)(waves * 256);
}

// Tile shape with the best (chip fill x per-tile efficiency) for weights of
// n[0..count) rows: 0 = 256x256, 1 = 256x128, 2 = 128x128.  The per-tile
// factors are the measured throughput of each shape relative to 256x256 (8
// waves of 64x128) at full occupancy.
int pick_tile(const WView* ws, int count, int64_t m) {
  int64_t t0 = 0, t1 = 0, t2 = 0;
  for (int i = 0; i < count; ++i) {
    t0 += ((ws[i].n + 255) / 256) * ((m + 255) / 256);
    t1 += ((ws[i].n + 255) / 256) * ((m + 127) / 128);
    t2 += ((ws[i].n + 127) / 128) * ((m + 127) / 128);
  }
  const double e0 = fill(t0) * 1.00, e1 = fill(t1) * 0.78, e2 = fill(t2) * 0.74;
  if (e0 >= e1 && e0 >= e2) return 0;
  return e1 >= e2 ? 1 : 2;
}

template <int KIND>
struct GemmFwdLauncher {
  static hipError_t run(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                        const int32_t* out_rows, const LoraEpi& lora, const Nf4Table& tab,
                        hipStream_t s) {
    switch (pick_tile(&w, 1, m)) {
      case 0: return launch_cfg<KIND, 256, 256, 4, 2>(w, X, m, Y, ldy, out_rows, lora, tab, s);
      case 1: return launch_cfg<KIND, 256, 128, 4, 2>(w, X, m, Y, ldy, out_rows, lora, tab, s);
      default: return launch_cfg<KIND, 128, 128, 2, 2>(w, X, m, Y, ldy, out_rows, lora, tab, s);
    }
  }
};

// Time of one launch over weights ws[0..count), in 256x256-tile units at full
// efficiency: the work divided by the best (chip fill x per-tile factor).
double launch_cost(const WView* ws, int count, int64_t m) {
  int64_t t0 = 0, t1 = 0, t2 = 0;
  double work = 0.0;
  for (int i = 0; i < count; ++i) {
    t0 += ((ws[i].n + 255) / 256) * ((m + 255) / 256);
    t1 += ((ws[i].n + 255) / 256) * ((m + 127) / 128);
    t2 += ((ws[i].n + 127) / 128) * ((m + 127) / 128);
    work += (double)ws[i].n * (double)m / 65536.0;
  }
  const double e = fmax(fill(t0) * 1.00, fmax(fill(t1) * 0.78, fill(t2) * 0.74));
  return work / e;
}

// A set whose last round of tiles is partly empty under every tile shape can
// run faster as two launches, a prefix of the weights and the rest, each with
// its own tile shape: q (4096 rows) at m = 4096 fills one round of 256x256
// tiles exactly, and k + v (2048 rows) one round of 256x128 tiles.  Returns
// the prefix length, or 0 for one launch; a split must save over 5% (it pays
// a second launch).
int split_point(const WView* ws, int count, int64_t m) {
  int best = 0;
  double best_cost = 0.95 * launch_cost(ws, count, m);
  for (int j = 1; j < count; ++j) {
    const double c = launch_cost(ws, j, m) + launch_cost(ws + j, count - j, m);
    if (c < best_cost) {
      best = j;
      best_cost = c;
    }
  }
  return best;
}

template <int KIND>
hipError_t launch_set_tiles(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* orows,
                            int count, const uint16_t* X, int64_t m, const Nf4Table& tab, hipStream_t s) {
  switch (pick_tile(ws, count, m)) {
    case 0: return launch_set_cfg<KIND, 256, 256, 4, 2>(ws, ys, ldys, orows, count, X, m, tab, s);
    case 1: return launch_set_cfg<KIND, 256, 128, 4, 2>(ws, ys, ldys, orows, count, X, m, tab, s);
    default: return launch_set_cfg<KIND, 128, 128, 2, 2>(ws, ys, ldys, orows, count, X, m, tab, s);
  }
}

template <int KIND>
struct GemmFwdSetLauncher {
  static hipError_t run(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* orows,
                        int count, const uint16_t* X, int64_t m, const Nf4Table& tab, hipStream_t s) {
    const int j = split_point(ws, count, m);
    if (j == 0) return launch_set_tiles<KIND>(ws, ys, ldys, orows, count, X, m, tab, s);
    const hipError_t e = launch_set_tiles<KIND>(ws, ys, ldys, orows, j, X, m, tab, s);
    if (e != hipSuccess) return e;
    return launch_set_tiles<KIND>(ws + j, ys + j, ldys + j, orows + j, count - j, X, m, tab, s);
  }
};

}  // namespace

hipError_t launch_gemm_fwd_set(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                               const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m,
                               const Nf4Table& tab, hipStream_t s) {
  if (count < 1 || count > kGemvMaxGroup) return hipErrorInvalidValue;
  return dispatch_kind<GemmFwdSetLauncher>(kind, ws, ys, ldys, out_rows, count, X, m, tab, s);
}

hipError_t launch_gemm_fwd(WKind kind, const WView& w, const uint16_t* X, int64_t m,
                           uint16_t* Y, int64_t ldy, const int32_t* out_rows,
                           const LoraEpi& lora, const Nf4Table& tab, hipStream_t s) {
  return dispatch_kind<GemmFwdLauncher>(kind, w, X, m, Y, ldy, out_rows, lora, tab, s);
}

}  // namespace lbq
