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
// groups of 4 X-row tiles so that concurrently running tiles share operands.
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

// One BN x BM output tile (tx, ty) of Y = X . deq(W)^T (+ the LoRA slab),
// summed over K range [k_lo, k_hi) (multiples of 1024 codes, or k_hi = K).
// With `part` set the fp32 sums go to part[m][n] (a K-split partial; the
// LoRA slab belongs to the range that starts at 0), else bf16 to Y.
template <int KIND, int BN, int BM, int WGN, int WGM, bool LORA>
__device__ __forceinline__ void gemm_fwd_tile(const WView& w, const uint16_t* __restrict__ X, int m,
                                              uint16_t* __restrict__ Y, int64_t ldy,
                                              const int32_t* __restrict__ out_rows,
                                              const LoraEpi& lora, const Nf4Table& tab, int tx, int ty,
                                              GemmLds<BN, BM>& lds, int64_t k_lo, int64_t k_hi,
                                              float* __restrict__ part) {
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
  // (Compact metadata -- fp16 scales, packed zero points -- takes the
  // per-stage form.)
  const bool md4 = !T::compact && (gpr & 3) == 0 && (reinterpret_cast<uintptr_t>(mf_arr) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(mb_arr) & 3) == 0;
  const float dqoff = T::dqo ? nf4_dq_offset(w) : 0.f;
  float mb0 = 0.f, mb1 = 0.f, mb2 = 0.f, mb3 = 0.f;  // scales / absmax of the batch
  uint32_t mb_b = 0;                                 // zero points / absmax codes of the batch
  int md_j = 0;  // entry of the loaded stage in the batch (the same in every lane)
  int64_t md_gi = 0;  // metadata entry of the loaded stage (compact zero points)
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
        if constexpr (T::fmt == FMT_MINMAX) {
          // raw words (compact: fp16 bits and the packed zero byte), decoded
          // in store_stage so that no wave waits for them here
          const MetaRaw r = load_meta_raw<KIND>(w, gi);
          const float v = __uint_as_float(r.s);
          mb0 = v, mb1 = v, mb2 = v, mb3 = v;
          mb_b = r.z;
          md_gi = gi;
        } else {
          if constexpr (!T::dq) {
            const float v = mf_arr[gi];
            mb0 = v, mb1 = v, mb2 = v, mb3 = v;
          }
          if constexpr (T::dq) mb_b = mb_arr[gi];
        }
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
      if constexpr (T::compact) {
        md_s = f16_bits_to_f32(__float_as_uint(md_s));
        md_i = zero_from_byte<KIND>(mb_b, md_gi);
      } else if constexpr (T::fmt == FMT_MINMAX) {
        md_i = (int)((mb_b >> (8 * md_j)) & 0xFFu);
      }
      if constexpr (T::dq) md_i = (int)(int8_t)(uint8_t)((mb_b >> (8 * md_j)) & 0xFFu);
    }
    float ws_s, ws_zs = 0.f;
    if constexpr (T::fmt == FMT_MINMAX) {
      ws_s = md_s;
      ws_zs = (float)md_i * md_s;
    } else if constexpr (T::dq) {
      ws_s = (float)md_i * md_s;
      if constexpr (T::dqo) ws_s += dqoff;
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
  load_stage(k_lo);
  store_stage(0);
  if (k_lo + BK < k_hi) load_stage(k_lo + BK);
  __syncthreads();
  int buf = 0;
  if constexpr (WGN * WGM == 8 && BM == 256) {
    // Two phases per stage, with a barrier between them: the first four waves
    // stage the next tile while the last four run their MFMAs, then the other
    // way round.  Waves w and w + 4 share a SIMD, so at any time one of them
    // feeds the matrix core while the other does the dequant and LDS writes.
    // The staging wave runs at raised priority: its loads, table reads and
    // conversions are a chain of short instructions that would otherwise wait
    // behind the MFMA wave's issue slots, while the MFMAs queue up anyway
    // (8B NF4+DQ layer at m = 4096, against raising the MFMA wave: forward
    // +0.8-1.5%, input gradient +1%).  (With 128-row X tiles a wave's MFMA phase is
    // no longer than its staging, and the extra barrier costs more than the
    // overlap gains.)
    const bool late = wave >= 4;
    auto stage = [&](int64_t t) {
      __builtin_amdgcn_s_setprio(1);
      if (t + BK < k_hi) {
        store_stage(buf ^ 1);
        if (t + 2 * BK < k_hi) load_stage(t + 2 * BK);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    auto mfma_phase = [&]() { compute(buf); };
    for (int64_t kt = k_lo; kt < k_hi; kt += BK) {
      if (late) mfma_phase();
      else stage(kt);
      __syncthreads();
      if (late) stage(kt);
      else mfma_phase();
      __syncthreads();
      buf ^= 1;
    }
  } else {
    for (int64_t kt = k_lo; kt < k_hi; kt += BK) {
      if (kt + BK < k_hi) {
        store_stage(buf ^ 1);
        if (kt + 2 * BK < k_hi) load_stage(kt + 2 * BK);
      }
      compute(buf);
      __syncthreads();
      buf ^= 1;
    }
  }

  // LoRA slab: acc += B_lora[n][:] . T[m][:], r zero-padded to rp (multiple of 32).
  if constexpr (LORA) {
    for (int ks = 0; ks < (k_lo == 0 ? lora.rp : 0); ks += 32) {
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
  if (part != nullptr) {
    // fp32 partial sums, [m][n] (the reduce applies out_rows)
    const bool vec = (w.n & 3) == 0;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int64_t mr = m0 + wm * WM + 16 * b + li;
      if (mr >= m) continue;
      float* prow = part + mr * w.n;
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int64_t nb = n0 + wn * WN + 16 * a + 4 * lg;
        if (vec && nb + 3 < w.n) {
          *reinterpret_cast<f32x4_t*>(prow + nb) = acc[a][b];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < w.n) prow[nb + i] = acc[a][b][i];
        }
      }
    }
    return;
  }
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
  // Row tile b outer, column tile a inner: the TN stores that fill a row's
  // WN contiguous outputs (whole 128-byte lines for WN = 64) follow one
  // another, so each line is complete in L2 before it is written back.
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int64_t mr = m0 + wm * WM + 16 * b + li;
    if (mr >= m) continue;
    uint16_t* yrow = Y + mr * ldy;
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int64_t nb = n0 + wn * WN + 16 * a + 4 * lg;
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

// K split of an n x k weight at m (its outputs are the same whichever launch
// runs it): a weight whose 256x256 tiles fill at most half the chip runs its
// K in ks ranges -- ks up to 256 / tiles and at most 8.  Its tile time is
// that of the whole K whatever the tile count, so a split saves about
// (1 - 1/ks) of it against fp32 partials of ks * m * n * 8 bytes of traffic.
//  * In general ks is kept to k / 3200 (the partials at most about a quarter
//    of the tile time at 1 PFLOP/s and 5 TB/s), in ranges of whole 1024-code
//    blocks.
//  * For m <= 256 a weight that alone fills at most an eighth of the chip (32
//    tiles: q, k, v, o or down of an 8B layer, whose tile time does not
//    shrink with m there) may use ranges of 512 codes, k / 512 of them: its
//    partials are small.  A larger weight (gate or up) is left alone: its
//    set already fills the chip.
// Either way every range starts on a metadata batch of four groups (or four
// NF4 blocks).
__host__ __device__ inline int split_unit(int64_t n, int64_t m) {
  return m <= 256 && ((n + 255) / 256) * ((m + 255) / 256) <= 32 ? 512 : 1024;
}
int gemm_splits(int64_t n, int64_t k, int64_t m) {
  const int64_t t = ((n + 255) / 256) * ((m + 255) / 256);
  if (t > 128) return 1;
  int64_t ks = 256 / t;
  if (ks > 8) ks = 8;
  const int unit = split_unit(n, m);
  const int64_t kmax = unit == 512 ? k / 512 : k / 3200;
  if (ks > kmax) ks = kmax;
  if (ks < 2) return 1;
  const int64_t per = ((k + ks - 1) / ks + unit - 1) / unit * unit;
  return (int)((k + per - 1) / per);  // every range non-empty
}

// K range [lo, hi) of range `split` of ks (unit: split_unit of the weight).
__device__ __forceinline__ void split_range(int64_t k, int ks, int unit, int split, int64_t& lo, int64_t& hi) {
  const int64_t per = ((k + ks - 1) / ks + unit - 1) / unit * unit;
  lo = (int64_t)split * per;
  hi = lo + per < k ? lo + per : k;
}

template <int KIND, int BN, int BM, int WGN, int WGM, bool LORA, bool SPLIT>
__global__ __launch_bounds__(WGN* WGM * 64) void k_gemm_fwd(WView w, const uint16_t* __restrict__ X,
                                                          int m, uint16_t* __restrict__ Y,
                                                          int64_t ldy,
                                                          const int32_t* __restrict__ out_rows,
                                                          LoraEpi lora, Nf4Table tab, float* __restrict__ part,
                                                          int ks) {
  const int nx = (int)((w.n + BN - 1) / BN), ny = (m + BM - 1) / BM;
  int tx, ty;
  __shared__ __attribute__((aligned(16))) GemmLds<BN, BM> lds;
  if constexpr (!SPLIT) {
    tile_of(blockIdx.x, nx, ny, tx, ty);
    gemm_fwd_tile<KIND, BN, BM, WGN, WGM, LORA>(w, X, m, Y, ldy, out_rows, lora, tab, tx, ty, lds, 0, w.k,
                                                nullptr);
  } else {
    // workgroups [split * tiles, (split + 1) * tiles) run K range `split`
    const int tiles = nx * ny;
    const int split = (int)blockIdx.x / tiles;
    tile_of((int)blockIdx.x - split * tiles, nx, ny, tx, ty);
    int64_t lo, hi;
    split_range(w.k, ks, split_unit(w.n, m), split, lo, hi);
    gemm_fwd_tile<KIND, BN, BM, WGN, WGM, LORA>(w, X, m, Y, ldy, out_rows, lora, tab, tx, ty, lds, lo, hi,
                                                part + (int64_t)split * m * w.n);
  }
}

// Several weights that share X: their column tiles are laid side by side
// (weight i owns tile columns [tile_end[i-1], tile_end[i])), so one launch
// covers them all and its last round of tiles is shared.  With K splits
// (SPLIT), weight i owns workgroups [wg_end[i-1], wg_end[i]) = its tiles x
// ks[i] instead, and when ks[i] > 1 its partials [ks][m][n] start at part +
// part_off[i].
struct GemmSet {
  WView w[kGemvMaxGroup];
  uint16_t* y[kGemvMaxGroup];
  int64_t ldy[kGemvMaxGroup];
  const int32_t* out_rows[kGemvMaxGroup];
  int tile_end[kGemvMaxGroup];
  int wg_end[kGemvMaxGroup];
  int ks[kGemvMaxGroup];
  int64_t part_off[kGemvMaxGroup];
  int64_t quad_end[kGemvMaxGroup];  // prefix sums of ceil(n / 4) (the reduce's column quads)
  float* part;
  int count;
};

template <int KIND, int BN, int BM, int WGN, int WGM, bool SPLIT>
__global__ __launch_bounds__(WGN* WGM * 64) void k_gemm_fwd_set(GemmSet set, const uint16_t* __restrict__ X,
                                                              int m, Nf4Table tab) {
  const LoraEpi none{nullptr, nullptr, 0, 0};
  __shared__ __attribute__((aligned(16))) GemmLds<BN, BM> lds;
  const int ny = (m + BM - 1) / BM;
  int tx, ty;
  if constexpr (!SPLIT) {
    int nx = set.tile_end[0];
#pragma unroll
    for (int i = 1; i < kGemvMaxGroup; ++i)
      if (i < set.count) nx = set.tile_end[i];
    tile_of(blockIdx.x, nx, ny, tx, ty);
    int pi = 0, tbeg = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxGroup; ++i)
      if (i < set.count && tx >= set.tile_end[i - 1]) { pi = i; tbeg = set.tile_end[i - 1]; }
    gemm_fwd_tile<KIND, BN, BM, WGN, WGM, false>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi],
                                                 none, tab, tx - tbeg, ty, lds, 0, set.w[pi].k, nullptr);
  } else {
    const int b = blockIdx.x;
    int pi = 0, wbeg = 0;
#pragma unroll
    for (int i = 1; i < kGemvMaxGroup; ++i)
      if (i < set.count && b >= set.wg_end[i - 1]) { pi = i; wbeg = set.wg_end[i - 1]; }
    const int nx = (int)((set.w[pi].n + BN - 1) / BN);
    const int tiles = nx * ny, ks = set.ks[pi];
    const int split = (b - wbeg) / tiles;
    tile_of(b - wbeg - split * tiles, nx, ny, tx, ty);
    int64_t lo, hi;
    split_range(set.w[pi].k, ks, split_unit(set.w[pi].n, m), split, lo, hi);
    float* const p = ks == 1 ? nullptr : set.part + set.part_off[pi] + (int64_t)split * m * set.w[pi].n;
    gemm_fwd_tile<KIND, BN, BM, WGN, WGM, false>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi],
                                                 none, tab, tx, ty, lds, lo, hi, p);
  }
}

// Y[m][col(c)] = bf16(sum over the K ranges of the partials), for the weights
// of a set with ks > 1.  A thread takes 4 adjacent columns of one weight
// (weight i owns the quads [quad_end[i-1], quad_end[i]) of the column space,
// its n rounded up to a multiple of 4) in row mr = blockIdx.y; the ranges are
// added in order, 16-byte partial loads when n % 4 == 0, and an 8-byte store
// of the 4 bf16 results when Y is contiguous and aligned.
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmSet set, int m) {
  const int64_t mr = blockIdx.y;
  const int64_t qg = (int64_t)blockIdx.x * 256 + threadIdx.x;  // column quad
  int64_t nq = set.quad_end[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count) nq = set.quad_end[i];
  if (qg >= nq) return;
  int pi = 0;
  int64_t qbeg = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count && qg >= set.quad_end[i - 1]) { pi = i; qbeg = set.quad_end[i - 1]; }
  const int ks = set.ks[pi];
  if (ks == 1) return;  // written by the GEMM itself
  const int64_t n = set.w[pi].n, c = 4 * (qg - qbeg);
  const float* p = set.part + set.part_off[pi] + mr * n + c;
  const int64_t stride = (int64_t)m * n;
  const int nc = n - c < 4 ? (int)(n - c) : 4;
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if ((n & 3) == 0) {
    int sidx = 0;
    for (; sidx + 4 <= ks; sidx += 4) {
      f32x4_t t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = *reinterpret_cast<const f32x4_t*>(p + (sidx + j) * stride);
#pragma unroll
      for (int j = 0; j < 4; ++j) v += t[j];
    }
    for (; sidx < ks; ++sidx) v += *reinterpret_cast<const f32x4_t*>(p + sidx * stride);
  } else {
    for (int sidx = 0; sidx < ks; ++sidx)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < nc) v[e] += p[sidx * stride + e];
  }
  uint16_t* yrow = set.y[pi] + mr * set.ldy[pi];
  const int32_t* orow = set.out_rows[pi];
  if (orow == nullptr && nc == 4 && (set.ldy[pi] & 3) == 0 && (reinterpret_cast<uintptr_t>(set.y[pi]) & 7) == 0) {
    uint2 o;
    o.x = cvt_pk_bf16(v[0], v[1]);
    o.y = cvt_pk_bf16(v[2], v[3]);
    *reinterpret_cast<uint2*>(yrow + c) = o;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < nc) yrow[orow ? (int64_t)orow[c + e] : c + e] = (uint16_t)bf16_rne(v[e]);
  }
}

// The set's K splits and partial areas (ks[i] = 1 for every weight when
// `part` is null); returns whether any weight splits.
bool plan_splits(GemmSet& set, const WView* ws, int count, int64_t m, float* part) {
  int64_t off = 0, nq = 0;
  bool any = false;
  for (int i = 0; i < count; ++i) {
    const int ks = part == nullptr ? 1 : gemm_splits(ws[i].n, ws[i].k, m);
    set.ks[i] = ks;
    set.part_off[i] = off;
    if (ks > 1) {
      off += ((int64_t)ks * m * ws[i].n + 3) / 4 * 4;  // 16-byte aligned areas
      any = true;
    }
    nq += (ws[i].n + 3) / 4;
    set.quad_end[i] = nq;
  }
  set.part = part;
  return any;
}

template <int BN, int BM>
int64_t tiles_of(int64_t n, int64_t m) {
  return ((n + BN - 1) / BN) * ((m + BM - 1) / BM);
}

template <int KIND, int BN, int BM, int WGN, int WGM>
hipError_t launch_set_cfg(const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                          const int32_t* const* orows, int count, const uint16_t* X, int64_t m,
                          float* part, const Nf4Table& tab, hipStream_t s) {
  GemmSet set{};
  set.count = count;
  int64_t nx = 0, wgs = 0;
  const bool split = plan_splits(set, ws, count, m, part);
  for (int i = 0; i < count; ++i) {
    nx += (ws[i].n + BN - 1) / BN;
    wgs += tiles_of<BN, BM>(ws[i].n, m) * set.ks[i];
    set.w[i] = ws[i];
    set.y[i] = ys[i];
    set.ldy[i] = ldys[i];
    set.out_rows[i] = orows[i];
    set.tile_end[i] = (int)nx;
    set.wg_end[i] = (int)wgs;
  }
  const dim3 block(WGN * WGM * 64);
  if (!split) {
    hipLaunchKernelGGL((k_gemm_fwd_set<KIND, BN, BM, WGN, WGM, false>), dim3((unsigned)(nx * ((m + BM - 1) / BM))),
                       block, 0, s, set, X, (int)m, tab);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_fwd_set<KIND, BN, BM, WGN, WGM, true>), dim3((unsigned)wgs), block, 0, s, set, X,
                     (int)m, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((set.quad_end[count - 1] + 255) / 256), (unsigned)m), dim3(256),
                     0, s, set, (int)m);
  return hipGetLastError();
}

template <int KIND, int BN, int BM, int WGN, int WGM>
hipError_t launch_cfg(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                      const int32_t* out_rows, const LoraEpi& lora, float* part, const Nf4Table& tab,
                      hipStream_t s) {
  const int64_t tiles = tiles_of<BN, BM>(w.n, m);
  const int ks = part == nullptr ? 1 : gemm_splits(w.n, w.k, m);
  const dim3 block(WGN * WGM * 64);
  if (ks == 1) {
    if (lora.t != nullptr)
      hipLaunchKernelGGL((k_gemm_fwd<KIND, BN, BM, WGN, WGM, true, false>), dim3((unsigned)tiles), block, 0, s, w,
                         X, (int)m, Y, ldy, out_rows, lora, tab, nullptr, 1);
    else
      hipLaunchKernelGGL((k_gemm_fwd<KIND, BN, BM, WGN, WGM, false, false>), dim3((unsigned)tiles), block, 0, s, w,
                         X, (int)m, Y, ldy, out_rows, lora, tab, nullptr, 1);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(tiles * ks));
  if (lora.t != nullptr)
    hipLaunchKernelGGL((k_gemm_fwd<KIND, BN, BM, WGN, WGM, true, true>), grid, block, 0, s, w, X, (int)m, Y, ldy,
                       out_rows, lora, tab, part, ks);
  else
    hipLaunchKernelGGL((k_gemm_fwd<KIND, BN, BM, WGN, WGM, false, true>), grid, block, 0, s, w, X, (int)m, Y, ldy,
                       out_rows, lora, tab, part, ks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmSet set{};
  set.count = 1;
  set.w[0] = w;
  set.y[0] = Y;
  set.ldy[0] = ldy;
  set.out_rows[0] = out_rows;
  plan_splits(set, &w, 1, m, part);
  hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((set.quad_end[0] + 255) / 256), (unsigned)m), dim3(256), 0, s,
                     set, (int)m);
  return hipGetLastError();
}

// Fraction of the chip's 256 CUs kept busy by `wgs` one-per-CU workgroups.
double fill(int64_t wgs) {
  const int64_t waves = (wgs + 255) / 256;
  return (double)wgs / (double)(waves * 256);
}

// Workgroups of each tile shape (0 = 256x256, 1 = 256x128, 2 = 128x128) for
// weights ws[0..count), with their K splits when `split`.
void shape_wgs(const WView* ws, int count, int64_t m, bool split, int64_t t[3]) {
  t[0] = t[1] = t[2] = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t ks = split ? gemm_splits(ws[i].n, ws[i].k, m) : 1;
    t[0] += tiles_of<256, 256>(ws[i].n, m) * ks;
    t[1] += tiles_of<256, 128>(ws[i].n, m) * ks;
    t[2] += tiles_of<128, 128>(ws[i].n, m) * ks;
  }
}

// Tile shape with the best (chip fill x per-tile efficiency) for weights of
// n[0..count) rows: 0 = 256x256, 1 = 256x128, 2 = 128x128.  The per-tile
// factors are the measured throughput of each shape relative to 256x256 (8
// waves of 64x128) at full occupancy.
int pick_tile(const WView* ws, int count, int64_t m, bool split) {
  int64_t t[3];
  shape_wgs(ws, count, m, split, t);
  const double e0 = fill(t[0]) * 1.00, e1 = fill(t[1]) * 0.78, e2 = fill(t[2]) * 0.74;
  if (e0 >= e1 && e0 >= e2) return 0;
  return e1 >= e2 ? 1 : 2;
}

template <int KIND>
struct GemmFwdLauncher {
  static hipError_t run(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                        const int32_t* out_rows, const LoraEpi& lora, float* part, const Nf4Table& tab,
                        hipStream_t s) {
    switch (pick_tile(&w, 1, m, part != nullptr)) {
      case 0: return launch_cfg<KIND, 256, 256, 4, 2>(w, X, m, Y, ldy, out_rows, lora, part, tab, s);
      case 1: return launch_cfg<KIND, 256, 128, 4, 2>(w, X, m, Y, ldy, out_rows, lora, part, tab, s);
      default: return launch_cfg<KIND, 128, 128, 2, 2>(w, X, m, Y, ldy, out_rows, lora, part, tab, s);
    }
  }
};

// Time of one launch over weights ws[0..count), in 256x256-tile units at full
// efficiency: the work divided by the best (chip fill x per-tile factor).
double launch_cost(const WView* ws, int count, int64_t m, bool split) {
  int64_t t[3];
  shape_wgs(ws, count, m, split, t);
  double work = 0.0;
  for (int i = 0; i < count; ++i) work += (double)ws[i].n * (double)m / 65536.0;
  const double e = fmax(fill(t[0]) * 1.00, fmax(fill(t[1]) * 0.78, fill(t[2]) * 0.74));
  return work / e;
}

// A set whose last round of tiles is partly empty under every tile shape can
// run faster as two launches, a prefix of the weights and the rest, each with
// its own tile shape: q (4096 rows) at m = 4096 fills one round of 256x256
// tiles exactly, and k + v (2048 rows) one round of 256x128 tiles.  Returns
// the prefix length, or 0 for one launch; a split must save over 5% (it pays
// a second launch).
int split_point(const WView* ws, int count, int64_t m, bool split) {
  int best = 0;
  double best_cost = 0.95 * launch_cost(ws, count, m, split);
  for (int j = 1; j < count; ++j) {
    const double c = launch_cost(ws, j, m, split) + launch_cost(ws + j, count - j, m, split);
    if (c < best_cost) {
      best = j;
      best_cost = c;
    }
  }
  return best;
}

template <int KIND>
hipError_t launch_set_tiles(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* orows,
                            int count, const uint16_t* X, int64_t m, float* part, const Nf4Table& tab,
                            hipStream_t s) {
  switch (pick_tile(ws, count, m, part != nullptr)) {
    case 0: return launch_set_cfg<KIND, 256, 256, 4, 2>(ws, ys, ldys, orows, count, X, m, part, tab, s);
    case 1: return launch_set_cfg<KIND, 256, 128, 4, 2>(ws, ys, ldys, orows, count, X, m, part, tab, s);
    default: return launch_set_cfg<KIND, 128, 128, 2, 2>(ws, ys, ldys, orows, count, X, m, part, tab, s);
  }
}

// Rows [r0, r1) of a weight as a weight of its own (r0 a multiple of 256):
// every buffer starts r0 rows further on.  Not for the offset kind, whose
// offset entry is found from the weight's own row count.
template <int KIND>
WView row_view(const WView& w, int64_t r0, int64_t r1) {
  using T = WKindTraits<KIND>;
  static_assert(!T::dqo, "row views of the offset kind");
  WView v = w;
  v.n = r1 - r0;
  v.packed = w.packed + r0 * (w.k * T::bits / 8);
  if constexpr (T::fmt == FMT_MINMAX) {
    const int64_t g = r0 * (w.k / T::group);  // metadata entries before row r0 (a multiple of 4)
    v.scales = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(w.scales) + (T::compact ? 2 : 4) * g);
    v.zeros = w.zeros + (T::compact ? g * T::bits / 8 : g);
  } else {
    const int64_t b = r0 * (w.k / 64);  // absmax blocks before row r0 (a multiple of 256)
    if constexpr (T::dq) {
      v.absmax_q = w.absmax_q + b;
      v.absmax_scale = w.absmax_scale + b / 256;
    } else {
      v.absmax = w.absmax + b;
    }
  }
  return v;
}

// A set whose 256x256 tiles leave the last round partly empty can also be cut
// inside a weight, at the n-tile where whole rounds end: the prefix runs full
// rounds of 256x256 tiles, the rest its own launch with the shape that fills
// the chip best (8B gate + up at m = 2048: 896 tiles = 3 rounds + 128 tiles).
// Only sets that split K nowhere: every output is then the same sum as in the
// single-weight call, whatever the tile shape.  Returns false when the cut
// does not save over the best of one launch or a cut between weights.
template <int KIND>
bool row_cut(const WView* ws, int count, int64_t m, float* part, int j_weights, WView* wa, int& na, WView* wb,
             int& nb, int& jw, int64_t& r) {
  if constexpr (WKindTraits<KIND>::dqo) {
    return false;
  } else {
    int64_t t0 = 0;
    for (int i = 0; i < count; ++i) {
      if (part != nullptr && gemm_splits(ws[i].n, ws[i].k, m) > 1) return false;
      t0 += tiles_of<256, 256>(ws[i].n, m);
    }
    const int64_t ny = (m + 255) / 256;
    if (t0 <= 256 || t0 % 256 == 0) return false;
    int64_t left = (t0 / 256) * 256 / ny;  // n-tiles of the prefix
    for (jw = 0; jw < count; ++jw) {
      const int64_t nt = (ws[jw].n + 255) / 256;
      if (left < nt) break;
      left -= nt;
    }
    if (jw == count || left == 0) return false;  // the cut falls between weights
    r = left * 256;
    na = nb = 0;
    for (int i = 0; i < jw; ++i) wa[na++] = ws[i];
    wa[na++] = row_view<KIND>(ws[jw], 0, r);
    wb[nb++] = row_view<KIND>(ws[jw], r, ws[jw].n);
    for (int i = jw + 1; i < count; ++i) wb[nb++] = ws[i];
    const double cut = launch_cost(wa, na, m, false) + launch_cost(wb, nb, m, false);
    const double best = j_weights == 0 ? 0.95 * launch_cost(ws, count, m, false)
                                       : launch_cost(ws, j_weights, m, false) +
                                             launch_cost(ws + j_weights, count - j_weights, m, false);
    return cut < best;
  }
}

// The two launches of a divided set run one after the other on the stream
// and reuse the same partial area.
template <int KIND>
struct GemmFwdSetLauncher {
  static hipError_t run(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* orows,
                        int count, const uint16_t* X, int64_t m, float* part, const Nf4Table& tab, hipStream_t s) {
    const int j = split_point(ws, count, m, part != nullptr);
    {
      WView wa[kGemvMaxGroup], wb[kGemvMaxGroup];
      int na = 0, nb = 0, jw = 0;
      int64_t r = 0;
      if (row_cut<KIND>(ws, count, m, part, j, wa, na, wb, nb, jw, r)) {
        // outputs of the cut weight: its columns from r on (or its out_rows from r on)
        uint16_t* yb[kGemvMaxGroup];
        int64_t lb[kGemvMaxGroup];
        const int32_t* ob[kGemvMaxGroup];
        for (int i = jw; i < count; ++i) {
          const bool cut = i == jw;
          yb[i - jw] = cut && orows[i] == nullptr ? ys[i] + r : ys[i];
          ob[i - jw] = cut && orows[i] != nullptr ? orows[i] + r : orows[i];
          lb[i - jw] = ldys[i];
        }
        const hipError_t e = launch_set_tiles<KIND>(wa, ys, ldys, orows, na, X, m, nullptr, tab, s);
        if (e != hipSuccess) return e;
        return launch_set_tiles<KIND>(wb, yb, lb, ob, nb, X, m, nullptr, tab, s);
      }
    }
    if (j == 0) return launch_set_tiles<KIND>(ws, ys, ldys, orows, count, X, m, part, tab, s);
    const hipError_t e = launch_set_tiles<KIND>(ws, ys, ldys, orows, j, X, m, part, tab, s);
    if (e != hipSuccess) return e;
    return launch_set_tiles<KIND>(ws + j, ys + j, ldys + j, orows + j, count - j, X, m, part, tab, s);
  }
};

}  // namespace

size_t gemm_fwd_workspace_bytes(const int64_t* ns, int count, int64_t k, int64_t m) {
  size_t b = 0;
  for (int i = 0; i < count; ++i) {
    const int ks = gemm_splits(ns[i], k, m);
    if (ks > 1) b += (size_t)(((int64_t)ks * m * ns[i] + 3) / 4 * 4) * sizeof(float);
  }
  return b;
}

hipError_t launch_gemm_fwd_set(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                               const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m,
                               float* part, const Nf4Table& tab, hipStream_t s) {
  if (count < 1 || count > kGemvMaxGroup) return hipErrorInvalidValue;
  return dispatch_kind<GemmFwdSetLauncher>(kind, ws, ys, ldys, out_rows, count, X, m, part, tab, s);
}

hipError_t launch_gemm_fwd(WKind kind, const WView& w, const uint16_t* X, int64_t m,
                           uint16_t* Y, int64_t ldy, const int32_t* out_rows,
                           const LoraEpi& lora, float* part, const Nf4Table& tab, hipStream_t s) {
  return dispatch_kind<GemmFwdLauncher>(kind, w, X, m, Y, ldy, out_rows, lora, part, tab, s);
}

}  // namespace lbq
