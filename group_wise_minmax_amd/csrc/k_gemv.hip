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
// wave at the end.  Every load of a batch of U steps -- weight chunks, their
// group scales / zero points (or block absmax), and the X chunks -- is issued
// before any arithmetic, so a lane keeps U*R 16-byte weight loads in flight and
// never waits on a dependent metadata load.
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

template <int KIND, int MT, int R, int U>
__global__ __launch_bounds__(kWaves * 64) void k_gemv(WView w, const uint16_t* __restrict__ X,
                                                     int m, uint16_t* __restrict__ Y,
                                                     int64_t ldy,
                                                     const int32_t* __restrict__ out_rows,
                                                     LoraEpi lora, Nf4Table tab) {
  using T = WKindTraits<KIND>;
  constexpr int CPB = 8 / T::bits;  // codes per byte
  constexpr int CPC = 16 * CPB;     // codes per 16-byte chunk
  constexpr int XD = CPC / 2;       // X dwords (bf16 pairs) per chunk
  constexpr int GRP = T::fmt == FMT_MINMAX ? T::group : 64;  // metadata granularity
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * kWaves + wave) * R;
  const int64_t KB = w.k * T::bits / 8;  // bytes per packed row
  const int64_t gpr = w.k / GRP;         // metadata entries per row

  extern __shared__ uint32_t lut[];  // NF4 only: [256 bytes][64 lanes]
  __shared__ float cbs[16];
  if constexpr (T::fmt == FMT_NF4) {
    // constant indices keep the kernel-argument table out of scratch memory
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (threadIdx.x == i) cbs[i] = tab.c[i];
    __syncthreads();
    for (int b = threadIdx.x; b < 256; b += kWaves * 64) {
      const uint32_t e = (uint32_t)bf16_rne(cbs[b >> 4]) | ((uint32_t)bf16_rne(cbs[b & 15]) << 16);
#pragma unroll 8
      for (int c = 0; c < 64; ++c) lut[b * 64 + c] = e;
    }
    __syncthreads();
  }

  bool rv[R];
  int64_t rix[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rv[r] = row0 + r < w.n;
    rix[r] = rv[r] ? row0 + r : 0;
  }
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.f;

  for (int64_t kbase = 0; kbase < KB; kbase += 1024 * U) {
    // Addresses are clamped to valid memory and every load is unconditional
    // (no branches), so the compiler can keep them all in flight; invalid
    // rows / steps are zeroed through their scale at compute time.
    u32x4_t wc[U][R];
    float sc[U][R];   // scale (MinMax) or block absmax (NF4)
    int zq[U][R];     // zero point (MinMax)
    bool okk[U][R];
    uint32_t xd[U][MT][XD];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kb = kbase + 1024 * u + (int64_t)lane * 16;
      const bool kok = kb < KB;
      const int64_t kbc = kok ? kb : 0;
      const int64_t k0 = kbc * CPB;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        okk[u][r] = rv[r] && kok;
        wc[u][r] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(w.packed + rix[r] * KB + kbc));
        const int64_t gi = rix[r] * gpr + k0 / GRP;
        if constexpr (T::fmt == FMT_MINMAX) {
          sc[u][r] = w.scales[gi];
          zq[u][r] = w.zeros[gi];
        } else {
          sc[u][r] = nf4_block_scale<T::dq>(w, gi);
          zq[u][r] = 0;
        }
      }
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        const int mmc = mm < m ? mm : 0;
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(X + (int64_t)mmc * w.k + k0);
#pragma unroll
        for (int j = 0; j < XD / 4; ++j) {
          const u32x4_t v = xp[j];
          xd[u][mm][4 * j + 0] = v[0];
          xd[u][mm][4 * j + 1] = v[1];
          xd[u][mm][4 * j + 2] = v[2];
          xd[u][mm][4 * j + 3] = v[3];
        }
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (T::fmt == FMT_MINMAX) {
        // X permuted into the dot2 pairs of each weight dword, and its chunk sum.
        uint32_t xp[MT][XD];
        float xs[MT];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          float xs0 = 0.f, xs1 = 0.f;
#pragma unroll
          for (int j = 0; j < XD; j += 2) {
            xs0 = dot2_bf16(xd[u][mm][j], kOnes, xs0);
            xs1 = dot2_bf16(xd[u][mm][j + 1], kOnes, xs1);
          }
          xs[mm] = xs0 + xs1;
          if constexpr (T::bits == 4) {
            // weight dword d holds codes 8d..8d+7; shift 4s pairs codes (e, e+4), e = s ^ 1
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const int e = s ^ 1;
                const uint32_t a = xd[u][mm][4 * d + (e >> 1)], b = xd[u][mm][4 * d + (e >> 1) + 2];
                xp[mm][4 * d + s] = (e & 1) ? pair_hi(a, b) : pair_lo(a, b);
              }
          } else {
            // weight dword d holds codes 16d..16d+15; shift 2s pairs codes (e, e+8)
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
              for (int s = 0; s < 8; ++s) {
                const int e = s < 4 ? 3 - s : 11 - s;
                const uint32_t a = xd[u][mm][8 * d + (e >> 1)], b = xd[u][mm][8 * d + (e >> 1) + 4];
                xp[mm][8 * d + s] = (e & 1) ? pair_hi(a, b) : pair_lo(a, b);
              }
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float p0[MT], p1[MT];  // two chains per row for latency
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) p0[mm] = p1[mm] = 0.f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t wd = wc[u][r][d];
            if constexpr (T::bits == 4) {
#pragma unroll
              for (int sh = 0; sh < 4; ++sh) {
                const uint32_t q2 = ((wd >> (4 * sh)) & 0x000F000Fu) | 0x43004300u;
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                  if (sh & 1) p1[mm] = dot2_bf16(q2, xp[mm][4 * d + sh], p1[mm]);
                  else p0[mm] = dot2_bf16(q2, xp[mm][4 * d + sh], p0[mm]);
                }
              }
            } else {
#pragma unroll
              for (int sh = 0; sh < 8; ++sh) {
                const uint32_t q2 = ((wd >> (2 * sh)) & 0x00030003u) | 0x43004300u;
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                  if (sh & 1) p1[mm] = dot2_bf16(q2, xp[mm][8 * d + sh], p1[mm]);
                  else p0[mm] = dot2_bf16(q2, xp[mm][8 * d + sh], p0[mm]);
                }
              }
            }
          }
          const float sr = okk[u][r] ? sc[u][r] : 0.f;
          const float off = (float)(128 + zq[u][r]);
#pragma unroll
          for (int mm = 0; mm < MT; ++mm)
            acc[r][mm] = fmaf(sr, fmaf(-off, xs[mm], p0[mm] + p1[mm]), acc[r][mm]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float p0[MT], p1[MT];
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) p0[mm] = p1[mm] = 0.f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t wd = wc[u][r][d];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t e = lut[((wd >> (8 * j)) & 0xFFu) * 64 + lane];
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) {
                if (j & 1) p1[mm] = dot2_bf16(e, xd[u][mm][4 * d + j], p1[mm]);
                else p0[mm] = dot2_bf16(e, xd[u][mm][4 * d + j], p0[mm]);
              }
            }
          }
          const float sr = okk[u][r] ? sc[u][r] : 0.f;
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) acc[r][mm] = fmaf(sr, p0[mm] + p1[mm], acc[r][mm]);
        }
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
  constexpr int U = MT == 1 ? 2 : 1;
  // Four rows per wave when there are enough rows to fill the chip, else one.
  if (w.n >= 4096) {
    constexpr int R = 4;
    const dim3 grid((unsigned)((w.n + kWaves * R - 1) / (kWaves * R)));
    hipLaunchKernelGGL((k_gemv<KIND, MT, R, U>), grid, dim3(kWaves * 64), lds, s, w, X, (int)m, Y,
                       ldy, out_rows, lora, tab);
  } else {
    constexpr int R = 1;
    const dim3 grid((unsigned)((w.n + kWaves * R - 1) / (kWaves * R)));
    hipLaunchKernelGGL((k_gemv<KIND, MT, R, U>), grid, dim3(kWaves * 64), lds, s, w, X, (int)m, Y,
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
