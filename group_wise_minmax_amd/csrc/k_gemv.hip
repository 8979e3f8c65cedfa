// Decode-size forward (m <= 4): Y = X . deq(W)^T as a wavefront-reduction GEMV
// that streams the packed weight once from HBM.
//
// The frozen low-bit linear layer whose kernel unpacks and dequantizes the
// weight to bf16 before multiplying: bitsandbytes FSDP-QLoRA guide, section
// 通过BitsAndBytesConfig配置 (compute_dtype).  Weight formats: GreenBit.AI
// "只需单卡RTX 3090，低比特量化训练就能实现LLaMA-3 8B全参微调", section 模型量化
// (MinMax INT4 g128 / INT2 g64) and "QLoRA技术在量化微调中的应用", section
// QLoRA技术原理 (NF4, double quantization).
//
// Layout of the work: a wave owns R consecutive rows of W; each lane streams
// 16-byte chunks of those rows (lanes contiguous along K, so a wave reads 1 KiB
// of each row per step) and keeps R x MT fp32 partial sums, reduced across the
// wave at the end.  X chunks are read once per step and shared by the R rows.
//
// MinMax dequantization never forms (q - z) * s per weight.  A code q is
// turned into the bf16 number 128 + q by OR-ing it into the exponent pattern
// of 128 (exact for q < 128), two codes per dword, and multiplied into X with
// v_dot2_f32_bf16.  A 16-byte chunk lies inside one group, so per chunk
//     sum_k x_k (q_k - z) s = s * (sum_k x_k (128 + q_k) - (128 + z) sum_k x_k).
// The dot2 pairs take codes (k, k+4) (4-bit) or (k, k+8) (2-bit) from one
// dword; X is permuted into the same pairs with v_perm_b32.
//
// NF4 uses a 256-entry byte -> (bf16 c[hi nibble], bf16 c[lo nibble]) table in
// LDS, replicated 64 times so that lane l always reads bank l (conflict-free);
// the block absmax multiplies the per-chunk dot product.
#include "lbq_device.h"

namespace lbq {

namespace {

constexpr int kWaves = 4;
constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1.0, 1.0)

template <int KIND, int MT, int R>
__global__ __launch_bounds__(kWaves * 64) void k_gemv(WView w, const uint16_t* __restrict__ X,
                                                     int m, uint16_t* __restrict__ Y,
                                                     int64_t ldy,
                                                     const int32_t* __restrict__ out_rows,
                                                     LoraEpi lora, Nf4Table tab) {
  using T = WKindTraits<KIND>;
  constexpr int CPB = 8 / T::bits;     // codes per byte
  constexpr int CPC = 16 * CPB;        // codes per 16-byte chunk
  constexpr int XD = CPC / 2;          // X dwords (bf16 pairs) per chunk
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * kWaves + wave) * R;
  const int64_t KB = w.k * T::bits / 8;  // bytes per packed row

  extern __shared__ uint32_t lut[];  // NF4 only: [256 bytes][64 lanes]
  if constexpr (T::fmt == FMT_NF4) {
    for (int b = threadIdx.x; b < 256; b += kWaves * 64) {
      const uint32_t e = (uint32_t)bf16_rne(tab.c[b >> 4]) | ((uint32_t)bf16_rne(tab.c[b & 15]) << 16);
#pragma unroll 8
      for (int c = 0; c < 64; ++c) lut[b * 64 + c] = e;
    }
    __syncthreads();
  }

  bool rv[R];
  const uint8_t* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rv[r] = row0 + r < w.n;
    wrow[r] = w.packed + (rv[r] ? (row0 + r) : 0) * KB;
  }
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.f;

  for (int64_t kb = (int64_t)lane * 16; kb < KB; kb += 1024) {
    u32x4_t wc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (rv[r]) {
        wc[r] = *reinterpret_cast<const u32x4_t*>(wrow[r] + kb);
      } else {
        wc[r] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    const int64_t k0 = kb * CPB;
    uint32_t xd[MT][XD];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      if (mm < m) {
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(X + (int64_t)mm * w.k + k0);
#pragma unroll
        for (int j = 0; j < XD / 4; ++j) {
          const u32x4_t v = xp[j];
          xd[mm][4 * j + 0] = v[0];
          xd[mm][4 * j + 1] = v[1];
          xd[mm][4 * j + 2] = v[2];
          xd[mm][4 * j + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int j = 0; j < XD; ++j) xd[mm][j] = 0u;
      }
    }

    if constexpr (T::fmt == FMT_MINMAX) {
      // X permuted into the dot2 pairs of each weight dword, and its chunk sum.
      uint32_t xp[MT][XD];
      float xs[MT];
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        xs[mm] = 0.f;
#pragma unroll
        for (int j = 0; j < XD; ++j) xs[mm] = dot2_bf16(xd[mm][j], kOnes, xs[mm]);
        if constexpr (T::bits == 4) {
          // weight dword d holds codes 8d..8d+7; shift 4s pairs codes (e, e+4), e = s ^ 1
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int e = s ^ 1;
              const uint32_t a = xd[mm][4 * d + (e >> 1)], b = xd[mm][4 * d + (e >> 1) + 2];
              xp[mm][4 * d + s] = (e & 1) ? pair_hi(a, b) : pair_lo(a, b);
            }
        } else {
          // weight dword d holds codes 16d..16d+15; shift 2s pairs codes (e, e+8)
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int e = s < 4 ? 3 - s : 11 - s;
              const uint32_t a = xd[mm][8 * d + (e >> 1)], b = xd[mm][8 * d + (e >> 1) + 4];
              xp[mm][8 * d + s] = (e & 1) ? pair_hi(a, b) : pair_lo(a, b);
            }
        }
      }
      const int64_t gpr = w.k / T::group;  // groups per row
      const int64_t gk = k0 / T::group;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t gi = (rv[r] ? (row0 + r) : 0) * gpr + gk;
        const float s = w.scales[gi];
        const float off = (float)(128 + (int)w.zeros[gi]);
        float p[MT];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) p[mm] = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = wc[r][d];
          if constexpr (T::bits == 4) {
#pragma unroll
            for (int sh = 0; sh < 4; ++sh) {
              const uint32_t q2 = ((wd >> (4 * sh)) & 0x000F000Fu) | 0x43004300u;
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) p[mm] = dot2_bf16(q2, xp[mm][4 * d + sh], p[mm]);
            }
          } else {
#pragma unroll
            for (int sh = 0; sh < 8; ++sh) {
              const uint32_t q2 = ((wd >> (2 * sh)) & 0x00030003u) | 0x43004300u;
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) p[mm] = dot2_bf16(q2, xp[mm][8 * d + sh], p[mm]);
            }
          }
        }
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) acc[r][mm] = fmaf(s, fmaf(-off, xs[mm], p[mm]), acc[r][mm]);
      }
    } else {
      const int64_t bpr = w.k / 64;  // absmax blocks per row
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float a = nf4_block_scale<T::dq>(w, (rv[r] ? (row0 + r) : 0) * bpr + k0 / 64);
        float p[MT];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) p[mm] = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = wc[r][d];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t e = lut[((wd >> (8 * j)) & 0xFFu) * 64 + lane];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) p[mm] = dot2_bf16(e, xd[mm][4 * d + j], p[mm]);
          }
        }
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) acc[r][mm] = fmaf(a, p[mm], acc[r][mm]);
      }
    }
  }

  // LoRA branch: lane j < r adds T[mm][j] * B[row][j] before the reduction.
  if (lora.t != nullptr && lane < lora.r) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!rv[r]) continue;
      const float bv = bf16_lo(lora.b[(row0 + r) * lora.r + lane]);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        if (mm < m) acc[r][mm] = fmaf(bf16_lo(lora.t[(int64_t)mm * lora.rp + lane]), bv, acc[r][mm]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      float v = acc[r][mm];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      acc[r][mm] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!rv[r]) continue;
      const int64_t col = out_rows ? (int64_t)out_rows[row0 + r] : row0 + r;
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        if (mm < m) Y[(int64_t)mm * ldy + col] = (uint16_t)bf16_rne(acc[r][mm]);
      }
    }
  }
}

template <int KIND, int MT>
hipError_t run_mt(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                  const int32_t* out_rows, const LoraEpi& lora, const Nf4Table& tab,
                  hipStream_t s) {
  using T = WKindTraits<KIND>;
  const size_t lds = (T::fmt == FMT_NF4) ? 256 * 64 * sizeof(uint32_t) : 0;
  // Four rows per wave when there are enough rows to fill the chip, else one.
  if (w.n >= 4096) {
    constexpr int R = 4;
    const dim3 grid((unsigned)((w.n + kWaves * R - 1) / (kWaves * R)));
    hipLaunchKernelGGL((k_gemv<KIND, MT, R>), grid, dim3(kWaves * 64), lds, s, w, X, (int)m, Y,
                       ldy, out_rows, lora, tab);
  } else {
    constexpr int R = 1;
    const dim3 grid((unsigned)((w.n + kWaves * R - 1) / (kWaves * R)));
    hipLaunchKernelGGL((k_gemv<KIND, MT, R>), grid, dim3(kWaves * 64), lds, s, w, X, (int)m, Y,
                       ldy, out_rows, lora, tab);
  }
  return hipGetLastError();
}

template <int KIND>
struct GemvLauncher {
  static hipError_t run(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                        const int32_t* out_rows, const LoraEpi& lora, const Nf4Table& tab,
                        hipStream_t s) {
    if (m == 1) return run_mt<KIND, 1>(w, X, m, Y, ldy, out_rows, lora, tab, s);
    if (m == 2) return run_mt<KIND, 2>(w, X, m, Y, ldy, out_rows, lora, tab, s);
    return run_mt<KIND, 4>(w, X, m, Y, ldy, out_rows, lora, tab, s);
  }
};

}  // namespace

hipError_t launch_gemv(WKind kind, const WView& w, const uint16_t* X, int64_t m, uint16_t* Y,
                       int64_t ldy, const int32_t* out_rows, const LoraEpi& lora,
                       const Nf4Table& tab, hipStream_t s) {
  if (m < 1 || m > kGemvMaxM) return hipErrorInvalidValue;
  return dispatch_kind<GemvLauncher>(kind, w, X, m, Y, ldy, out_rows, lora, tab, s);
}

}  // namespace lbq
