// Single-token decode (m == 1): y = deq(W) . x as a streaming GEMV, the
// HBM-bound half of the frozen low-bit linear layer.
//
// The kernel that unpacks and dequantizes the weight to bf16 before the
// matmul: bitsandbytes FSDP-QLoRA guide, section 通过BitsAndBytesConfig配置.
// Weight formats: GreenBit.AI "只需单卡RTX 3090，低比特量化训练就能实现LLaMA-3
// 8B全参微调", section 模型量化 (MinMax INT4 g128 / INT2 g64) and
// "QLoRA技术在量化微调中的应用", section QLoRA技术原理 (NF4, double quantization).
//
// Structure.
//  * One launch serves up to kGemvMaxGroup weights that share x and K (q, k and v
//    of a layer, gate and up, or the INT4 and INT2 row sets of a mixed-precision
//    layer in separate launches per kind): the waves are dealt out per weight,
//    so a wave works on one weight for its whole life.
//  * x either comes from global memory with each step (4-bit MinMax: the
//    vector stays in L1/L2 and no barrier delays the first weight loads), or
//    is staged in LDS once per workgroup (2-bit MinMax, whose 16-byte chunk
//    needs 128 bytes of x, and NF4), unless the staged copy would not fit.
//    Either way it is arranged the way the dot products consume it (see
//    below), with the sum of x over every 16-byte weight chunk (MinMax).  NF4 builds a 256-entry byte -> pair of
//    bf16 levels table in LDS, 32 copies so each lane of a 32-lane half reads
//    its own bank.
//  * Work: a wave owns a run of groups of R consecutive rows; each step loads
//    CB 16-byte chunks of each of the R rows (lanes contiguous along K, 1 KiB
//    of a row per chunk index), and the loads of up to D steps (weights,
//    scales, zero points or block absmax) are in flight while earlier steps
//    are computed.
//  * MinMax: codes never become (q - z) * s per weight.  The low and high
//    nibbles (or 2-bit crumbs) of a weight dword are split into byte vectors
//    and v_perm_b32 lays two of them next to the byte 0x43, giving the bf16
//    numbers 128 + q (exact for q < 128) as a pair; v_dot2_f32_bf16 multiplies
//    the pair into x.  Per chunk (inside one group):
//        sum x (q - z) s = s * (sum x (128 + q) - (128 + z) sum x).
//    x is arranged in the same pair order, so the weight side costs about 1.4
//    VALU operations per code.
//  * NF4: each packed byte (two codes) indexes the table and the pair is dotted
//    with x; the block absmax scales the chunk sum.
#include "lbq_device.h"

#include <algorithm>

namespace lbq {

namespace {

constexpr int kThreads = 256;
constexpr int kLutCopies = 32;
constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1.0, 1.0)
constexpr uint32_t k43 = 0x43434343u;    // bf16 exponent byte of 128

// Bytes 0/1 (or 2/3) of `v`, each followed by 0x43: two bf16 numbers 128 + b.
__device__ __forceinline__ uint32_t pair01(uint32_t v) { return perm_b32(k43, v, 0x04010400u); }
__device__ __forceinline__ uint32_t pair23(uint32_t v) { return perm_b32(k43, v, 0x04030402u); }

template <int KIND>
struct Gemv1Traits {
  using T = WKindTraits<KIND>;
  static constexpr int CPC = 16 * 8 / T::bits;  // codes per 16-byte chunk
  static constexpr int XD = CPC / 2;            // x dwords per chunk
  static constexpr int XQ = XD / 4;             // 16-byte x quads per chunk
  static constexpr int GRP = T::fmt == FMT_MINMAX ? T::group : 64;
};

// x chunk (natural order, XD dwords) -> the order the weight pairs use.
template <int KIND>
__device__ __forceinline__ void arrange_x(const uint32_t* xn, uint32_t* xo) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int j = 0; j < Gemv1Traits<KIND>::XD; ++j) xo[j] = xn[j];
  } else if constexpr (T::bits == 4) {
    // weight dword d (codes 8d..8d+7): pairs (1,3) (5,7) (0,2) (4,6)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = xn[4 * d], b = xn[4 * d + 1], c = xn[4 * d + 2], e = xn[4 * d + 3];
      xo[4 * d + 0] = pair_hi(a, b);
      xo[4 * d + 1] = pair_hi(c, e);
      xo[4 * d + 2] = pair_lo(a, b);
      xo[4 * d + 3] = pair_lo(c, e);
    }
  } else {
    // weight dword d (codes 16d..16d+15), crumb t of byte j = code 4j + t:
    // pairs (3,7) (11,15) (2,6) (10,14) (1,5) (9,13) (0,4) (8,12)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t* v = xn + 8 * d;  // v[i] = (x_{2i}, x_{2i+1})
      xo[8 * d + 0] = pair_hi(v[1], v[3]);
      xo[8 * d + 1] = pair_hi(v[5], v[7]);
      xo[8 * d + 2] = pair_lo(v[1], v[3]);
      xo[8 * d + 3] = pair_lo(v[5], v[7]);
      xo[8 * d + 4] = pair_hi(v[0], v[2]);
      xo[8 * d + 5] = pair_hi(v[4], v[6]);
      xo[8 * d + 6] = pair_lo(v[0], v[2]);
      xo[8 * d + 7] = pair_lo(v[4], v[6]);
    }
  }
}

// Dot product of one 16-byte weight chunk with its arranged x (two chains).
template <int KIND>
__device__ __forceinline__ float chunk_dot(const u32x4_t& wq, const uint32_t* xa,
                                           const uint32_t* lut, int lane32) {
  using T = WKindTraits<KIND>;
  float p0 = 0.f, p1 = 0.f;
  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t byte = (wq[d] >> (8 * j)) & 0xFFu;
        const uint32_t e = lut[byte * kLutCopies + lane32];
        if (j & 1) p1 = dot2_bf16(e, xa[4 * d + j], p1);
        else p0 = dot2_bf16(e, xa[4 * d + j], p0);
      }
  } else if constexpr (T::bits == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = wq[d] & 0x0F0F0F0Fu;         // codes 1,3,5,7
      const uint32_t hi = (wq[d] >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6
      p0 = dot2_bf16(pair01(lo), xa[4 * d + 0], p0);
      p1 = dot2_bf16(pair23(lo), xa[4 * d + 1], p1);
      p0 = dot2_bf16(pair01(hi), xa[4 * d + 2], p0);
      p1 = dot2_bf16(pair23(hi), xa[4 * d + 3], p1);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t c3 = wq[d] & 0x03030303u;
      const uint32_t c2 = (wq[d] >> 2) & 0x03030303u;
      const uint32_t c1 = (wq[d] >> 4) & 0x03030303u;
      const uint32_t c0 = (wq[d] >> 6) & 0x03030303u;
      p0 = dot2_bf16(pair01(c3), xa[8 * d + 0], p0);
      p1 = dot2_bf16(pair23(c3), xa[8 * d + 1], p1);
      p0 = dot2_bf16(pair01(c2), xa[8 * d + 2], p0);
      p1 = dot2_bf16(pair23(c2), xa[8 * d + 3], p1);
      p0 = dot2_bf16(pair01(c1), xa[8 * d + 4], p0);
      p1 = dot2_bf16(pair23(c1), xa[8 * d + 5], p1);
      p0 = dot2_bf16(pair01(c0), xa[8 * d + 6], p0);
      p1 = dot2_bf16(pair23(c0), xa[8 * d + 7], p1);
    }
  }
  return p0 + p1;
}

template <int KIND, int R, int CB>
struct Step {
  u32x4_t wq[CB][R];
  uint32_t sc[CB][R];  // raw metadata as loaded (load_meta)
  uint32_t zq[CB][R];
  u32x4_t xv[CB][Gemv1Traits<KIND>::XQ];  // x of the chunk (global-x mode only)
};

// The weights of one launch.  Waves [wave_end[i-1], wave_end[i]) work on
// weight i, which has ngroups[i] groups of R rows.  Arrays of fields (not of
// structs) so that a wave finds its weight from one scalar load of wave_end.
struct Gemv1Set {
  WView w[kGemvMaxGroup];
  uint16_t* y[kGemvMaxGroup];
  int64_t ldy[kGemvMaxGroup];  // row stride of y (several x rows only)
  const int32_t* out_rows[kGemvMaxGroup];
  int wave_end[kGemvMaxGroup];
  int ngroups[kGemvMaxGroup];
  int count;
};

// x chunk `c` (natural order, from global or from the raw quads) -> arranged
// dwords and, for MinMax, the chunk's sum of x.
template <int KIND>
__device__ __forceinline__ float x_chunk(const u32x4_t* xv, uint32_t* xa) {
  using G = Gemv1Traits<KIND>;
  uint32_t xn[G::XD];
#pragma unroll
  for (int q = 0; q < G::XQ; ++q) {
    xn[4 * q] = xv[q][0]; xn[4 * q + 1] = xv[q][1]; xn[4 * q + 2] = xv[q][2]; xn[4 * q + 3] = xv[q][3];
  }
  float s0 = 0.f, s1 = 0.f;
  if constexpr (WKindTraits<KIND>::fmt == FMT_MINMAX) {
#pragma unroll
    for (int j = 0; j < G::XD; j += 2) {
      s0 = dot2_bf16(xn[j], kOnes, s0);
      s1 = dot2_bf16(xn[j + 1], kOnes, s1);
    }
  }
  arrange_x<KIND>(xn, xa);
  return s0 + s1;
}

// Metadata of entry gc of row `row` (gpr entries per row), as loaded: the
// raw scale word (MinMax fp32 or fp16 bits, NF4 absmax or second-level
// scale) and the raw zero-point / absmax-code byte.  Nothing is computed on
// the loaded values here: a use right after the load would make the wave wait
// for it at once and empty the prefetch ring; meta_scale / meta_zero decode
// them where the step is consumed.  The row offset is wave-uniform (a scalar
// offset), gc the lane's.
template <int KIND>
__device__ __forceinline__ void load_meta(__amdgpu_buffer_rsrc_t r_s, __amdgpu_buffer_rsrc_t r_z, int row, int gpr,
                                          int gc, uint32_t& sraw, uint32_t& zraw) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_MINMAX && T::compact) {
    // fp16 scales; zero points packed bits wide (rows hold whole bytes)
    sraw = __builtin_amdgcn_raw_buffer_load_b16(r_s, (uint32_t)gc * 2u, row * gpr * 2, 0);
    zraw = __builtin_amdgcn_raw_buffer_load_b8(r_z, (uint32_t)(gc * T::bits / 8), row * gpr * T::bits / 8, 0);
  } else if constexpr (T::fmt == FMT_MINMAX) {
    sraw = __builtin_amdgcn_raw_buffer_load_b32(r_s, (uint32_t)gc * 4u, row * gpr * 4, 0);
    zraw = __builtin_amdgcn_raw_buffer_load_b8(r_z, (uint32_t)gc, row * gpr, 0);
  } else if constexpr (T::dq) {
    zraw = __builtin_amdgcn_raw_buffer_load_b8(r_z, (uint32_t)gc, row * gpr, 0);
    sraw = __builtin_amdgcn_raw_buffer_load_b32(r_s, (uint32_t)((row * gpr + gc) >> 8) * 4u, 0, 0);
  } else {
    sraw = __builtin_amdgcn_raw_buffer_load_b32(r_s, (uint32_t)gc * 4u, row * gpr * 4, 0);
    zraw = 0;
  }
}
// The scale of a loaded entry: MinMax s, or the NF4 block absmax (decoded
// from the int8 code and second-level scale under double quantization).
template <int KIND>
__device__ __forceinline__ float meta_scale(uint32_t sraw, uint32_t zraw, float dqoff) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_MINMAX) {
    return scale_from_bits<KIND>(sraw);
  } else if constexpr (T::dq) {
    const float p = (float)(int)(int8_t)(uint8_t)zraw * __uint_as_float(sraw);
    return T::dqo ? p + dqoff : p;
  } else {
    return __uint_as_float(sraw);
  }
}
// The MinMax zero point of entry gc of a row (rows hold whole bytes of zero
// points, so the row's offset does not change the field's position).
template <int KIND>
__device__ __forceinline__ int meta_zero(uint32_t zraw, int gc) {
  return zero_from_byte<KIND>(zraw, gc);
}

// The work of one wave (and its share of the workgroup prologue): weight `w`,
// output `Y` / `out_rows`, row groups [g0, g1) of R rows; `total` == 0 for a
// wave without work (it still joins the prologue's barriers).
template <int KIND, int R, int CB, int D, bool XG>
__device__ __forceinline__ void gemv1_body(const WView& w, uint16_t* __restrict__ Y,
                                           const int32_t* __restrict__ out_rows, int g0, int g1,
                                           bool active, const uint16_t* __restrict__ X,
                                           const LoraEpi& lora, const Nf4Table& tab) {
  using T = WKindTraits<KIND>;
  using G = Gemv1Traits<KIND>;
  constexpr int CPC = G::CPC, XD = G::XD, XQ = G::XQ, GRP = G::GRP;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  const int KB = (int)(w.k * T::bits / 8);  // bytes per packed row (< 2^24)
  const int nchunk = KB / 16;               // 16-byte chunks per row
  const int gpr = (int)(w.k / GRP);         // metadata entries per row

  uint32_t* lut = smem;                                               // NF4 table
  uint32_t* xq = smem + (T::fmt == FMT_NF4 ? 256 * kLutCopies : 0);  // [XQ][nchunk] quads
  float* xsum = reinterpret_cast<float*>(xq + (size_t)XQ * 4 * nchunk);

  // ---- work: groups of R rows, steps of CB chunk indices per lane ------------
  const int cpl = (nchunk + 63) / 64;      // chunk indices per lane and row
  const int nsteps = (cpl + CB - 1) / CB;  // steps per group
  const int total = (active && g0 < g1) ? (g1 - g0) * nsteps : 0;
  const int lane32 = lane & 31;

  // Buffer loads: the row base is a wave-uniform scalar offset, the lane's
  // chunk a 32-bit vector offset (the boundary keeps (n + 256) * k < 2^32).
  const int64_t nmeta = w.n * gpr;
  const __amdgpu_buffer_rsrc_t r_w = make_rsrc(w.packed, w.n * KB);
  const __amdgpu_buffer_rsrc_t r_x = make_rsrc(X, w.k * 2);
  __amdgpu_buffer_rsrc_t r_s, r_z;
  meta_rsrc<KIND>(w, nmeta, r_s, r_z);
  const float dqoff = T::dqo ? nf4_dq_offset(w) : 0.f;
  auto load = [&](int s, Step<KIND, R, CB>& st) {
    const int g = g0 + s / nsteps, b = s % nsteps;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = min((b * CB + cb) * 64 + lane, nchunk - 1);  // clamped: always valid
      const int gc = (c * CPC) / GRP;  // metadata entry of the chunk within the row
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = (int)min((int64_t)g * R + r, w.n - 1);
        st.wq[cb][r] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_w, (uint32_t)c * 16u, row * KB, 2 /*nt*/));
        load_meta<KIND>(r_s, r_z, row, gpr, gc, st.sc[cb][r], st.zq[cb][r]);
      }
      if constexpr (XG) {
#pragma unroll
        for (int q = 0; q < XQ; ++q)
          st.xv[cb][q] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_x, (uint32_t)(c * CPC * 2 + 16 * q), 0, 0));
      }
    }
  };

  // The loads of the first D steps go out before the prologue, so their
  // latency overlaps it; afterwards each computed step's slot is refilled with
  // the step D ahead (a ring of D steps in registers).
  Step<KIND, R, CB> st[D];
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < total) load(i, st[i]);

  // ---- prologue: NF4 table; arranged x (and chunk sums) in LDS ---------------
  __shared__ float cbs[16];
  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tid == i) cbs[i] = tab.c[i];
    lds_barrier();
    for (int e = tid; e < 256 * kLutCopies; e += kThreads) {
      const int b = e / kLutCopies;
      lut[e] = (uint32_t)bf16_rne(cbs[b >> 4]) | ((uint32_t)bf16_rne(cbs[b & 15]) << 16);
    }
  }
  if constexpr (!XG) {
    for (int c = tid; c < nchunk; c += kThreads) {
      u32x4_t xv[XQ];
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(X + (int64_t)c * CPC);
#pragma unroll
      for (int q = 0; q < XQ; ++q) xv[q] = src[q];
      uint32_t xo[XD];
      const float sx = x_chunk<KIND>(xv, xo);
      if constexpr (T::fmt == FMT_MINMAX) xsum[c] = sx;
#pragma unroll
      for (int q = 0; q < XQ; ++q)
        reinterpret_cast<u32x4_t*>(xq)[(size_t)q * nchunk + c] =
            u32x4_t{xo[4 * q], xo[4 * q + 1], xo[4 * q + 2], xo[4 * q + 3]};
    }
  }
  if constexpr (!XG || T::fmt == FMT_NF4) lds_barrier();

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  auto compute = [&](int s, const Step<KIND, R, CB>& st) {
    const int g = g0 + s / nsteps, b = s % nsteps;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = (b * CB + cb) * 64 + lane;
      const bool cok = c < nchunk;
      uint32_t xa[XD];
      float xs;
      if constexpr (XG) {
        xs = x_chunk<KIND>(st.xv[cb], xa);
      } else {
        const int cc = cok ? c : 0;
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
          const u32x4_t v = reinterpret_cast<const u32x4_t*>(xq)[(size_t)q * nchunk + cc];
          xa[4 * q] = v[0]; xa[4 * q + 1] = v[1]; xa[4 * q + 2] = v[2]; xa[4 * q + 3] = v[3];
        }
        xs = (T::fmt == FMT_MINMAX) ? xsum[cc] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float p = chunk_dot<KIND>(st.wq[cb][r], xa, lut, lane32);
        const float sr = (cok && (int64_t)g * R + r < w.n) ? meta_scale<KIND>(st.sc[cb][r], st.zq[cb][r], dqoff) : 0.f;
        if constexpr (T::fmt == FMT_MINMAX) {
          const int z = meta_zero<KIND>(st.zq[cb][r], (c * CPC) / GRP);
          acc[r] = fmaf(sr, fmaf(-(float)(128 + z), xs, p), acc[r]);
        } else {
          acc[r] = fmaf(sr, p, acc[r]);
        }
      }
    }
    if (b == nsteps - 1) {  // group finished: LoRA term, wave reduction, store
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = (int64_t)g * R + r;
        if (lora.t != nullptr && lane < lora.r && row < w.n)
          acc[r] = fmaf(bf16_lo(lora.t[lane]), bf16_lo(lora.b[row * lora.r + lane]), acc[r]);
        const float v = wave_sum(acc[r]);
        if (lane == 0 && row < w.n) Y[out_rows ? (int64_t)out_rows[row] : row] = (uint16_t)bf16_rne(v);
        acc[r] = 0.f;
      }
    }
  };

  for (int s = 0; s < total; s += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (s + i >= total) break;
      compute(s + i, st[i]);
      if (s + i + D < total) load(s + i + D, st[i]);
    }
  }
}

// One weight (with an optional LoRA term): waves take gpw row groups each.
template <int KIND, int R, int CB, int D, bool XG>
__global__ __launch_bounds__(kThreads) void k_gemv1(WView w, const uint16_t* __restrict__ X,
                                                   uint16_t* __restrict__ Y,
                                                   const int32_t* __restrict__ out_rows,
                                                   LoraEpi lora, Nf4Table tab, int gpw) {
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ngroups = (int)((w.n + R - 1) / R);
  const int g0 = gw * gpw;
  gemv1_body<KIND, R, CB, D, XG>(w, Y, out_rows, g0, min(g0 + gpw, ngroups), true, X, lora, tab);
}

// Several weights sharing x: each wave finds its weight from the wave ranges.
template <int KIND, int R, int CB, int D, bool XG>
__global__ __launch_bounds__(kThreads) void k_gemv1_set(Gemv1Set set, const uint16_t* __restrict__ X,
                                                       Nf4Table tab, int gpw) {
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int pi = 0, wbeg = 0, wlast = set.wave_end[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count) {
      if (gw >= set.wave_end[i - 1]) { pi = i; wbeg = set.wave_end[i - 1]; }
      wlast = set.wave_end[i];
    }
  const int g0 = (gw - wbeg) * gpw;
  const LoraEpi none{nullptr, nullptr, 0, 0};
  gemv1_body<KIND, R, CB, D, XG>(set.w[pi], set.y[pi], set.out_rows[pi], g0, min(g0 + gpw, set.ngroups[pi]),
                                 gw < wlast, X, none, tab);
}

// Waves of set entries [lo, hi), whose wave ranges start at wave wbeg0.
template <int KIND, int R, int CB, int D, bool XG>
__device__ __forceinline__ void gemv1_set_part(const Gemv1Set& set, int lo, int hi, int wbeg0, int gw,
                                               const uint16_t* __restrict__ X, const Nf4Table& tab, int gpw) {
  int pi = lo, wbeg = wbeg0, wlast = set.wave_end[lo];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i > lo && i < hi) {
      if (gw >= set.wave_end[i - 1]) { pi = i; wbeg = set.wave_end[i - 1]; }
      wlast = set.wave_end[i];
    }
  const int g0 = (gw - wbeg) * gpw;
  const LoraEpi none{nullptr, nullptr, 0, 0};
  gemv1_body<KIND, R, CB, D, XG>(set.w[pi], set.y[pi], set.out_rows[pi], g0, min(g0 + gpw, set.ngroups[pi]),
                                 gw < wlast, X, none, tab);
}

template <int R_, int CB_, int D_, bool XG_>
struct G1Cfg {
  static constexpr int R = R_, CB = CB_, D = D_;
  static constexpr bool XG = XG_;
};

// The INT4 g128 and INT2 g64 row sets of channel-mixed linears that share x,
// in one launch: workgroups [0, wg_a) run set entries [0, first_b) (INT4),
// the rest entries [first_b, count) (INT2), whose wave ranges start at wave
// 4 * wg_a.  Each format keeps the launch shape and the per-wave work of its
// own launch, so the outputs are the same bits.
template <class CA, class CB2>
__global__ __launch_bounds__(kThreads) void k_gemv1_mix(Gemv1Set set, const uint16_t* __restrict__ X,
                                                       Nf4Table tab, int first_b, int wg_a, int gpw_a,
                                                       int gpw_b) {
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((int)blockIdx.x < wg_a)
    gemv1_set_part<WK_I4G128, CA::R, CA::CB, CA::D, CA::XG>(set, 0, first_b, 0, gw, X, tab, gpw_a);
  else
    gemv1_set_part<WK_I2G64, CB2::R, CB2::CB, CB2::D, CB2::XG>(set, first_b, set.count, (kThreads / 64) * wg_a,
                                                               gw, X, tab, gpw_b);
}

// ---------------------------------------------------------------------------
// Several x rows (2 <= m <= MV <= 4): the same streaming of the weight, with
// the arranged x of every row staged in LDS.  A chunk's codes become bf16
// pairs once and are dotted with each row's x; per row the sums run in the
// same order as the one-row kernel's, so each output row is bit for bit what
// the one-row kernel gives for that row of x.
// ---------------------------------------------------------------------------

// The pairs of one 16-byte weight chunk, in the order arrange_x lays out x.
template <int KIND>
__device__ __forceinline__ void chunk_pairs(const u32x4_t& wq, const uint32_t* lut, int lane32, uint32_t* wv) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[4 * d + j] = lut[((wq[d] >> (8 * j)) & 0xFFu) * kLutCopies + lane32];
  } else if constexpr (T::bits == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = wq[d] & 0x0F0F0F0Fu, hi = (wq[d] >> 4) & 0x0F0F0F0Fu;
      wv[4 * d + 0] = pair01(lo);
      wv[4 * d + 1] = pair23(lo);
      wv[4 * d + 2] = pair01(hi);
      wv[4 * d + 3] = pair23(hi);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t c3 = wq[d] & 0x03030303u, c2 = (wq[d] >> 2) & 0x03030303u;
      const uint32_t c1 = (wq[d] >> 4) & 0x03030303u, c0 = (wq[d] >> 6) & 0x03030303u;
      wv[8 * d + 0] = pair01(c3);
      wv[8 * d + 1] = pair23(c3);
      wv[8 * d + 2] = pair01(c2);
      wv[8 * d + 3] = pair23(c2);
      wv[8 * d + 4] = pair01(c1);
      wv[8 * d + 5] = pair23(c1);
      wv[8 * d + 6] = pair01(c0);
      wv[8 * d + 7] = pair23(c0);
    }
  }
}

// Same two alternating chains as chunk_dot.
template <int XD>
__device__ __forceinline__ float dot_pairs(const uint32_t* wv, const uint32_t* xa) {
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int i = 0; i < XD; ++i) {
    if (i & 1) p1 = dot2_bf16(wv[i], xa[i], p1);
    else p0 = dot2_bf16(wv[i], xa[i], p0);
  }
  return p0 + p1;
}

template <int KIND, int R, int CB, int D, int MV>
__device__ __forceinline__ void gemvm_body(const WView& w, uint16_t* __restrict__ Y, int64_t ldy,
                                           const int32_t* __restrict__ out_rows, int g0, int g1, bool active,
                                           const uint16_t* __restrict__ X, int m, const LoraEpi& lora,
                                           const Nf4Table& tab) {
  using T = WKindTraits<KIND>;
  using G = Gemv1Traits<KIND>;
  constexpr int CPC = G::CPC, XD = G::XD, XQ = G::XQ, GRP = G::GRP;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int KB = (int)(w.k * T::bits / 8);
  const int nchunk = KB / 16;
  const int gpr = (int)(w.k / GRP);
  uint32_t* lut = smem;
  uint32_t* xq = smem + (T::fmt == FMT_NF4 ? 256 * kLutCopies : 0);  // [MV][XQ][nchunk] quads
  float* xsum = reinterpret_cast<float*>(xq + (size_t)MV * XQ * 4 * nchunk);  // [MV][nchunk]
  const int cpl = (nchunk + 63) / 64;
  const int nsteps = (cpl + CB - 1) / CB;
  const int total = (active && g0 < g1) ? (g1 - g0) * nsteps : 0;
  const int lane32 = lane & 31;
  const int64_t nmeta = w.n * gpr;
  const __amdgpu_buffer_rsrc_t r_w = make_rsrc(w.packed, w.n * KB);
  __amdgpu_buffer_rsrc_t r_s, r_z;
  meta_rsrc<KIND>(w, nmeta, r_s, r_z);
  const float dqoff = T::dqo ? nf4_dq_offset(w) : 0.f;
  auto load = [&](int s, Step<KIND, R, CB>& st) {
    const int g = g0 + s / nsteps, b = s % nsteps;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = min((b * CB + cb) * 64 + lane, nchunk - 1);
      const int gc = (c * CPC) / GRP;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = (int)min((int64_t)g * R + r, w.n - 1);
        st.wq[cb][r] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_w, (uint32_t)c * 16u, row * KB, 2 /*nt*/));
        load_meta<KIND>(r_s, r_z, row, gpr, gc, st.sc[cb][r], st.zq[cb][r]);
      }
    }
  };
  Step<KIND, R, CB> st[D];
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < total) load(i, st[i]);

  // prologue: NF4 table; arranged x of every row (zeros past m) in LDS
  __shared__ float cbs[16];
  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tid == i) cbs[i] = tab.c[i];
    lds_barrier();
    for (int e = tid; e < 256 * kLutCopies; e += kThreads) {
      const int b = e / kLutCopies;
      lut[e] = (uint32_t)bf16_rne(cbs[b >> 4]) | ((uint32_t)bf16_rne(cbs[b & 15]) << 16);
    }
  }
  for (int e = tid; e < MV * nchunk; e += kThreads) {
    const int mv = e / nchunk, c = e % nchunk;
    u32x4_t xv[XQ];
    if (mv < m) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(X + (int64_t)mv * w.k + (int64_t)c * CPC);
#pragma unroll
      for (int q = 0; q < XQ; ++q) xv[q] = src[q];
    } else {
#pragma unroll
      for (int q = 0; q < XQ; ++q) xv[q] = u32x4_t{0u, 0u, 0u, 0u};
    }
    uint32_t xo[XD];
    const float sx = x_chunk<KIND>(xv, xo);
    if constexpr (T::fmt == FMT_MINMAX) xsum[mv * nchunk + c] = sx;
#pragma unroll
    for (int q = 0; q < XQ; ++q)
      reinterpret_cast<u32x4_t*>(xq)[((size_t)mv * XQ + q) * nchunk + c] =
          u32x4_t{xo[4 * q], xo[4 * q + 1], xo[4 * q + 2], xo[4 * q + 3]};
  }
  lds_barrier();

  float acc[R][MV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < MV; ++v) acc[r][v] = 0.f;

  auto compute = [&](int s, const Step<KIND, R, CB>& st) {
    const int g = g0 + s / nsteps, b = s % nsteps;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = (b * CB + cb) * 64 + lane;
      const bool cok = c < nchunk;
      const int cc = cok ? c : 0;
      uint32_t wv[R][XD];
#pragma unroll
      for (int r = 0; r < R; ++r) chunk_pairs<KIND>(st.wq[cb][r], lut, lane32, wv[r]);
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        uint32_t xa[XD];
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
          const u32x4_t t = reinterpret_cast<const u32x4_t*>(xq)[((size_t)v * XQ + q) * nchunk + cc];
          xa[4 * q] = t[0]; xa[4 * q + 1] = t[1]; xa[4 * q + 2] = t[2]; xa[4 * q + 3] = t[3];
        }
        const float xs = (T::fmt == FMT_MINMAX) ? xsum[v * nchunk + cc] : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float p = dot_pairs<XD>(wv[r], xa);
          const float sr = (cok && (int64_t)g * R + r < w.n) ? meta_scale<KIND>(st.sc[cb][r], st.zq[cb][r], dqoff) : 0.f;
          if constexpr (T::fmt == FMT_MINMAX) {
            const int z = meta_zero<KIND>(st.zq[cb][r], (c * CPC) / GRP);
            acc[r][v] = fmaf(sr, fmaf(-(float)(128 + z), xs, p), acc[r][v]);
          } else {
            acc[r][v] = fmaf(sr, p, acc[r][v]);
          }
        }
      }
    }
    if (b == nsteps - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = (int64_t)g * R + r;
#pragma unroll
        for (int v = 0; v < MV; ++v) {
          if (v >= m) break;
          if (lora.t != nullptr && lane < lora.r && row < w.n)
            acc[r][v] = fmaf(bf16_lo(lora.t[(int64_t)v * lora.rp + lane]), bf16_lo(lora.b[row * lora.r + lane]),
                             acc[r][v]);
          const float y = wave_sum(acc[r][v]);
          if (lane == 0 && row < w.n)
            Y[(int64_t)v * ldy + (out_rows ? (int64_t)out_rows[row] : row)] = (uint16_t)bf16_rne(y);
        }
#pragma unroll
        for (int v = 0; v < MV; ++v) acc[r][v] = 0.f;
      }
    }
  };

  for (int s = 0; s < total; s += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (s + i >= total) break;
      compute(s + i, st[i]);
      if (s + i + D < total) load(s + i + D, st[i]);
    }
  }
}

template <int KIND, int R, int CB, int D, int MV>
__global__ __launch_bounds__(kThreads) void k_gemvm(WView w, const uint16_t* __restrict__ X, int m,
                                                   uint16_t* __restrict__ Y, int64_t ldy,
                                                   const int32_t* __restrict__ out_rows, LoraEpi lora,
                                                   Nf4Table tab, int gpw) {
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ngroups = (int)((w.n + R - 1) / R);
  const int g0 = gw * gpw;
  gemvm_body<KIND, R, CB, D, MV>(w, Y, ldy, out_rows, g0, min(g0 + gpw, ngroups), true, X, m, lora, tab);
}

template <int KIND, int R, int CB, int D, int MV>
__global__ __launch_bounds__(kThreads) void k_gemvm_set(Gemv1Set set, const uint16_t* __restrict__ X, int m,
                                                       Nf4Table tab, int gpw) {
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int pi = 0, wbeg = 0, wlast = set.wave_end[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count) {
      if (gw >= set.wave_end[i - 1]) { pi = i; wbeg = set.wave_end[i - 1]; }
      wlast = set.wave_end[i];
    }
  const int g0 = (gw - wbeg) * gpw;
  const LoraEpi none{nullptr, nullptr, 0, 0};
  gemvm_body<KIND, R, CB, D, MV>(set.w[pi], set.y[pi], set.ldy[pi], set.out_rows[pi], g0,
                                 min(g0 + gpw, set.ngroups[pi]), gw < wlast, X, m, none, tab);
}

// Waves of set entries [lo, hi), whose wave ranges start at wave wbeg0.
template <int KIND, int R, int CB, int D, int MV>
__device__ __forceinline__ void gemvm_set_part(const Gemv1Set& set, int lo, int hi, int wbeg0, int gw,
                                               const uint16_t* __restrict__ X, int m, const Nf4Table& tab,
                                               int gpw) {
  int pi = lo, wbeg = wbeg0, wlast = set.wave_end[lo];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i > lo && i < hi) {
      if (gw >= set.wave_end[i - 1]) { pi = i; wbeg = set.wave_end[i - 1]; }
      wlast = set.wave_end[i];
    }
  const int g0 = (gw - wbeg) * gpw;
  const LoraEpi none{nullptr, nullptr, 0, 0};
  gemvm_body<KIND, R, CB, D, MV>(set.w[pi], set.y[pi], set.ldy[pi], set.out_rows[pi], g0,
                                 min(g0 + gpw, set.ngroups[pi]), gw < wlast, X, m, none, tab);
}

// The INT4 g128 and INT2 g64 row sets of channel-mixed linears that share X
// (2 <= m <= MV), in one launch: workgroups [0, wg_a) run set entries
// [0, first_b) (INT4), the rest entries [first_b, count) (INT2), whose wave
// ranges start at wave 4 * wg_a.  A workgroup stages x in its own format's
// order, and each format keeps the plan of its own launch, so the outputs
// are the bits of the two per-format launches.
template <int R, int CB, int D, int MV>
__global__ __launch_bounds__(kThreads) void k_gemvm_mix(Gemv1Set set, const uint16_t* __restrict__ X, int m,
                                                       Nf4Table tab, int first_b, int wg_a, int gpw_a, int gpw_b) {
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((int)blockIdx.x < wg_a)
    gemvm_set_part<WK_I4G128, R, CB, D, MV>(set, 0, first_b, 0, gw, X, m, tab, gpw_a);
  else
    gemvm_set_part<WK_I2G64, R, CB, D, MV>(set, first_b, set.count, (kThreads / 64) * wg_a, gw, X, m, tab, gpw_b);
}

// Dynamic LDS per workgroup: the NF4 table, plus the arranged x and chunk sums
// when x is staged.
template <int KIND>
size_t lds_bytes(int64_t k, bool xg) {
  using T = WKindTraits<KIND>;
  using G = Gemv1Traits<KIND>;
  const int64_t nchunk = k * T::bits / 8 / 16;
  size_t b = T::fmt == FMT_NF4 ? 256 * kLutCopies * 4 : 0;
  if (!xg) b += (size_t)nchunk * G::XD * 4 + (T::fmt == FMT_MINMAX ? (size_t)nchunk * 4 : 0);
  return b;
}

// Wave plan of `count` weights of one kind (entries [first, first + count) of
// `set`, wave ranges from wave `base`): groups of R rows, gpw groups per wave.
// Returns gpw; *wend = the end of the last wave range.
template <int KIND, int R, int CB>
int64_t plan_set(const WView* ws, uint16_t* const* ys, const int32_t* const* orows, int count, int spw,
                 int min_waves, Gemv1Set& set, int first, int64_t base, int64_t* wend_out) {
  using T = WKindTraits<KIND>;
  const int64_t nchunk = ws[0].k * T::bits / 8 / 16;
  const int64_t nsteps = ((nchunk + 63) / 64 + CB - 1) / CB;
  int64_t groups = 0;
  for (int i = 0; i < count; ++i) groups += (ws[i].n + R - 1) / R;
  int64_t waves = (groups * nsteps + spw - 1) / spw;
  waves = waves < min_waves ? min_waves : waves;
  waves = waves > groups ? groups : waves;
  const int64_t gpw = (groups + waves - 1) / waves;
  int64_t wend = base;
  for (int i = 0; i < count; ++i) {
    const int64_t ng = (ws[i].n + R - 1) / R;
    wend += (ng + gpw - 1) / gpw;
    set.w[first + i] = ws[i];
    set.y[first + i] = ys[i];
    set.out_rows[first + i] = orows[i];
    set.wave_end[first + i] = (int)wend;
    set.ngroups[first + i] = (int)ng;
  }
  *wend_out = wend;
  return gpw;
}

// spw: target steps per wave (each wave keeps up to D steps of loads in
// flight); the grid never has fewer than min_waves waves when there is that
// much work.  The row groups of all weights share one wave budget; each
// weight gets whole waves.
template <int KIND, int R, int CB, int D, bool XG>
hipError_t launch_set(const WView* ws, uint16_t* const* ys, const int32_t* const* orows, int count,
                      const uint16_t* X, const LoraEpi& lora, const Nf4Table& tab, hipStream_t s,
                      int spw, int min_waves = 1024) {
  Gemv1Set set{};
  set.count = count;
  int64_t wend = 0;
  const int64_t gpw = plan_set<KIND, R, CB>(ws, ys, orows, count, spw, min_waves, set, 0, 0, &wend);
  const dim3 grid((unsigned)((wend + 3) / 4));
  const size_t lds = lds_bytes<KIND>(ws[0].k, XG);
  if (count == 1)
    hipLaunchKernelGGL((k_gemv1<KIND, R, CB, D, XG>), grid, dim3(kThreads), lds, s, ws[0], X, ys[0], orows[0],
                       lora, tab, (int)gpw);
  else
    hipLaunchKernelGGL((k_gemv1_set<KIND, R, CB, D, XG>), grid, dim3(kThreads), lds, s, set, X, tab, (int)gpw);
  return hipGetLastError();
}

template <int KIND>
struct Gemv1Launcher {
  static hipError_t run(const WView* ws, uint16_t* const* ys, const int32_t* const* orows, int count,
                        const uint16_t* X, const LoraEpi& lora, const Nf4Table& tab, hipStream_t s) {
    using T = WKindTraits<KIND>;
    const int64_t k = ws[0].k;
    // Measured on the LLaMA-3-8B and 70B-shaped layers (all weights of one
    // launch together).  4-bit MinMax reads x from global memory and takes 2
    // chunks (32 B) of each row per step: 1 row per wave with 2 steps in
    // flight under 2048 rows in all (more waves), 2 rows with 2 steps up to
    // 8192 rows of length <= 8192; larger launches 1 step, with 4 rows from
    // 8192 rows up (each x load then serves four rows: the 70B-shaped INT4
    // layer 8.5% faster than with 2), else 2 (4 rows left the 8B down, 4096
    // rows of 14336, with one wave per SIMD: 10.0 -> 11.0 us).  NF4 stages x in
    // LDS, 2 chunks per step with 2 steps in flight.  2-bit MinMax (128 B of x
    // per 16-byte chunk) takes 4 rows per wave with 1 chunk per step and 1
    // step in flight, so each x read serves four rows of weights: x staged in
    // LDS (70B-shaped all-INT2 layer 7% faster than 2 rows with 2 chunks and
    // 2 steps, or, over 8192, 1 chunk and 4 steps; the compact layer 8%, the
    // Qwen-shaped layer 10%), or read from global memory when the staged copy
    // would not fit 64 KiB (Qwen-shaped down, k = 49152: the Qwen decode layer
    // 9-11% faster than with 2 rows).  The rows per wave, chunks per step and
    // steps in flight never change a row's sum: every lane adds its chunks
    // c, c + 64, ... in the same order.
    const bool fits = lds_bytes<KIND>(k, false) <= 65536;
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) rows += ws[i].n;
    if constexpr (T::fmt == FMT_MINMAX && T::bits == 4) {
      if (rows < 2048) return launch_set<KIND, 1, 2, 2, true>(ws, ys, orows, count, X, lora, tab, s, 1);
      if (rows <= 8192 && k <= 8192) return launch_set<KIND, 2, 2, 2, true>(ws, ys, orows, count, X, lora, tab, s, 1);
      if (rows >= 8192) return launch_set<KIND, 4, 2, 1, true>(ws, ys, orows, count, X, lora, tab, s, 1);
      return launch_set<KIND, 2, 2, 1, true>(ws, ys, orows, count, X, lora, tab, s, 1);
    } else if constexpr (T::fmt == FMT_MINMAX) {
      if (!fits) return launch_set<KIND, 4, 1, 1, true>(ws, ys, orows, count, X, lora, tab, s, 2);
      return launch_set<KIND, 4, 1, 1, false>(ws, ys, orows, count, X, lora, tab, s, k <= 8192 ? 1 : 2);
    } else {
      if (fits) return launch_set<KIND, 2, 2, 2, false>(ws, ys, orows, count, X, lora, tab, s, 4);
      return launch_set<KIND, 2, 2, 1, true>(ws, ys, orows, count, X, lora, tab, s, 4);
    }
  }
};

// The mixed launch: each format planned exactly as its own launch would be
// (Gemv1Launcher's choice of shape), INT4 waves first, rounded up to whole
// workgroups.
template <class CA, class CB2>
hipError_t launch_mix_cfg(const WView* ws, uint16_t* const* ys, const int32_t* const* orows, int count_a,
                          int count_b, const uint16_t* X, const Nf4Table& tab, hipStream_t s, int spw_a,
                          int spw_b) {
  Gemv1Set set{};
  set.count = count_a + count_b;
  int64_t wend_a = 0, wend_b = 0;
  const int64_t gpw_a = plan_set<WK_I4G128, CA::R, CA::CB>(ws, ys, orows, count_a, spw_a, 1024, set, 0, 0, &wend_a);
  const int64_t wg_a = (wend_a + 3) / 4;
  const int64_t gpw_b = plan_set<WK_I2G64, CB2::R, CB2::CB>(ws + count_a, ys + count_a, orows + count_a, count_b,
                                                           spw_b, 1024, set, count_a, 4 * wg_a, &wend_b);
  const int64_t k = ws[0].k;
  const size_t lds = std::max(lds_bytes<WK_I4G128>(k, CA::XG), lds_bytes<WK_I2G64>(k, CB2::XG));
  hipLaunchKernelGGL((k_gemv1_mix<CA, CB2>), dim3((unsigned)((wend_b + 3) / 4)), dim3(kThreads), lds, s, set, X,
                     tab, count_a, (int)wg_a, (int)gpw_a, (int)gpw_b);
  return hipGetLastError();
}

template <class CA>
hipError_t launch_mix_b(const WView* ws, uint16_t* const* ys, const int32_t* const* orows, int count_a,
                        int count_b, const uint16_t* X, const Nf4Table& tab, hipStream_t s) {
  const int64_t k = ws[0].k;
  if (lds_bytes<WK_I2G64>(k, false) > 65536)
    return launch_mix_cfg<CA, G1Cfg<4, 1, 1, true>>(ws, ys, orows, count_a, count_b, X, tab, s, 1, 2);
  return launch_mix_cfg<CA, G1Cfg<4, 1, 1, false>>(ws, ys, orows, count_a, count_b, X, tab, s, 1, k <= 8192 ? 1 : 2);
}

template <int KIND, int MV>
size_t lds_bytes_m(int64_t k) {
  using T = WKindTraits<KIND>;
  using G = Gemv1Traits<KIND>;
  const int64_t nchunk = k * T::bits / 8 / 16;
  return (T::fmt == FMT_NF4 ? 256 * kLutCopies * 4 : 0) +
         (size_t)MV * ((size_t)nchunk * G::XD * 4 + (T::fmt == FMT_MINMAX ? (size_t)nchunk * 4 : 0));
}

template <int KIND, int R, int CB, int D, int MV>
hipError_t launch_setm(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* orows,
                       int count, const uint16_t* X, int64_t m, const LoraEpi& lora, const Nf4Table& tab,
                       hipStream_t s, int spw, int min_waves = 1024) {
  using T = WKindTraits<KIND>;
  const int64_t nchunk = ws[0].k * T::bits / 8 / 16;
  const int64_t nsteps = ((nchunk + 63) / 64 + CB - 1) / CB;
  int64_t groups = 0;
  for (int i = 0; i < count; ++i) groups += (ws[i].n + R - 1) / R;
  int64_t waves = (groups * nsteps + spw - 1) / spw;
  waves = waves < min_waves ? min_waves : waves;
  waves = waves > groups ? groups : waves;
  const int64_t gpw = (groups + waves - 1) / waves;
  const size_t lds = lds_bytes_m<KIND, MV>(ws[0].k);
  if (count == 1) {
    const int64_t nw = ((ws[0].n + R - 1) / R + gpw - 1) / gpw;
    hipLaunchKernelGGL((k_gemvm<KIND, R, CB, D, MV>), dim3((unsigned)((nw + 3) / 4)), dim3(kThreads), lds, s, ws[0],
                       X, (int)m, ys[0], ldys[0], orows[0], lora, tab, (int)gpw);
    return hipGetLastError();
  }
  Gemv1Set set{};
  set.count = count;
  int64_t wend = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t ng = (ws[i].n + R - 1) / R;
    wend += (ng + gpw - 1) / gpw;
    set.w[i] = ws[i];
    set.y[i] = ys[i];
    set.ldy[i] = ldys[i];
    set.out_rows[i] = orows[i];
    set.wave_end[i] = (int)wend;
    set.ngroups[i] = (int)ng;
  }
  hipLaunchKernelGGL((k_gemvm_set<KIND, R, CB, D, MV>), dim3((unsigned)((wend + 3) / 4)), dim3(kThreads), lds, s, set,
                     X, (int)m, tab, (int)gpw);
  return hipGetLastError();
}

template <int KIND>
struct GemvmLauncher {
  static hipError_t run(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* orows,
                        int count, const uint16_t* X, int64_t m, const LoraEpi& lora, const Nf4Table& tab,
                        hipStream_t s) {
    if (m <= 2) return launch_setm<KIND, 2, 1, 2, 2>(ws, ys, ldys, orows, count, X, m, lora, tab, s, 2);
    return launch_setm<KIND, 2, 1, 2, 4>(ws, ys, ldys, orows, count, X, m, lora, tab, s, 2);
  }
};

// The mixed multi-row launch: each format planned as GemvmLauncher plans its
// own launch (2 rows per group, 1 chunk per step, 2 steps in flight, 2 steps
// per wave), INT4 waves first, rounded up to whole workgroups.
template <int MV>
hipError_t launch_gemvm_mix_mv(const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                               const int32_t* const* orows, int count_a, int count_b, const uint16_t* X, int64_t m,
                               const Nf4Table& tab, hipStream_t s) {
  Gemv1Set set{};
  set.count = count_a + count_b;
  int64_t wend_a = 0, wend_b = 0;
  const int64_t gpw_a = plan_set<WK_I4G128, 2, 1>(ws, ys, orows, count_a, 2, 1024, set, 0, 0, &wend_a);
  const int64_t wg_a = (wend_a + 3) / 4;
  const int64_t gpw_b = plan_set<WK_I2G64, 2, 1>(ws + count_a, ys + count_a, orows + count_a, count_b, 2, 1024, set,
                                                 count_a, 4 * wg_a, &wend_b);
  for (int i = 0; i < set.count; ++i) set.ldy[i] = ldys[i];
  const int64_t k = ws[0].k;
  const size_t lds = std::max(lds_bytes_m<WK_I4G128, MV>(k), lds_bytes_m<WK_I2G64, MV>(k));
  hipLaunchKernelGGL((k_gemvm_mix<2, 1, 2, MV>), dim3((unsigned)((wend_b + 3) / 4)), dim3(kThreads), lds, s, set, X,
                     (int)m, tab, count_a, (int)wg_a, (int)gpw_a, (int)gpw_b);
  return hipGetLastError();
}

}  // namespace

bool gemvm_fits(WKind kind, int64_t k, int64_t m) {
  if (m < 2 || m > kGemvmMaxM) return false;
  size_t b = 0;
  switch (kind) {
    case WK_I4G128: b = m <= 2 ? lds_bytes_m<WK_I4G128, 2>(k) : lds_bytes_m<WK_I4G128, 4>(k); break;
    case WK_I4G64: b = m <= 2 ? lds_bytes_m<WK_I4G64, 2>(k) : lds_bytes_m<WK_I4G64, 4>(k); break;
    case WK_I2G64: b = m <= 2 ? lds_bytes_m<WK_I2G64, 2>(k) : lds_bytes_m<WK_I2G64, 4>(k); break;
    case WK_I2G128: b = m <= 2 ? lds_bytes_m<WK_I2G128, 2>(k) : lds_bytes_m<WK_I2G128, 4>(k); break;
    case WK_NF4: b = m <= 2 ? lds_bytes_m<WK_NF4, 2>(k) : lds_bytes_m<WK_NF4, 4>(k); break;
    case WK_NF4DQ: b = m <= 2 ? lds_bytes_m<WK_NF4DQ, 2>(k) : lds_bytes_m<WK_NF4DQ, 4>(k); break;
    case WK_I4G128C: b = m <= 2 ? lds_bytes_m<WK_I4G128C, 2>(k) : lds_bytes_m<WK_I4G128C, 4>(k); break;
    case WK_I2G64C: b = m <= 2 ? lds_bytes_m<WK_I2G64C, 2>(k) : lds_bytes_m<WK_I2G64C, 4>(k); break;
    case WK_NF4DQO: b = m <= 2 ? lds_bytes_m<WK_NF4DQO, 2>(k) : lds_bytes_m<WK_NF4DQO, 4>(k); break;
  }
  return b <= 65536;
}

hipError_t launch_gemvm(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                        const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m,
                        const LoraEpi& lora, const Nf4Table& tab, hipStream_t s) {
  if (count < 1 || count > kGemvMaxGroup || !gemvm_fits(kind, ws[0].k, m)) return hipErrorInvalidValue;
  return dispatch_kind<GemvmLauncher>(kind, ws, ys, ldys, out_rows, count, X, m, lora, tab, s);
}

hipError_t launch_gemvm_mix(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* out_rows,
                            int count_a, int count_b, const uint16_t* X, int64_t m, const Nf4Table& tab,
                            hipStream_t s) {
  if (count_a < 1 || count_b < 1 || count_a + count_b > kGemvMaxGroup || !gemvm_fits(WK_I4G128, ws[0].k, m) ||
      !gemvm_fits(WK_I2G64, ws[0].k, m))
    return hipErrorInvalidValue;
  if (m <= 2) return launch_gemvm_mix_mv<2>(ws, ys, ldys, out_rows, count_a, count_b, X, m, tab, s);
  return launch_gemvm_mix_mv<4>(ws, ys, ldys, out_rows, count_a, count_b, X, m, tab, s);
}

hipError_t launch_gemv1_mix(const WView* ws, uint16_t* const* ys, const int32_t* const* out_rows, int count_a,
                            int count_b, const uint16_t* X, const Nf4Table& tab, hipStream_t s) {
  if (count_a < 1 || count_b < 1 || count_a + count_b > kGemvMaxGroup) return hipErrorInvalidValue;
  int64_t rows_a = 0;
  for (int i = 0; i < count_a; ++i) rows_a += ws[i].n;
  const int64_t k = ws[0].k;
  if (rows_a < 2048) return launch_mix_b<G1Cfg<1, 2, 2, true>>(ws, ys, out_rows, count_a, count_b, X, tab, s);
  if (rows_a <= 8192 && k <= 8192)
    return launch_mix_b<G1Cfg<2, 2, 2, true>>(ws, ys, out_rows, count_a, count_b, X, tab, s);
  // 4 rows per INT4 wave here at any row count: the INT2 row sets give the
  // launch waves enough (70B channel mix at m = 1: with 2 rows for the INT4
  // rows of down, 2048 of 28672, the layer ran 8% slower)
  return launch_mix_b<G1Cfg<4, 2, 1, true>>(ws, ys, out_rows, count_a, count_b, X, tab, s);
}

hipError_t launch_gemv1(WKind kind, const WView* ws, uint16_t* const* ys, const int32_t* const* out_rows,
                        int count, const uint16_t* X, const LoraEpi& lora, const Nf4Table& tab,
                        hipStream_t s) {
  if (count < 1 || count > kGemvMaxGroup) return hipErrorInvalidValue;
  return dispatch_kind<Gemv1Launcher>(kind, ws, ys, out_rows, count, X, lora, tab, s);
}

}  // namespace lbq
