// Input gradient through the frozen low-bit weight (dX = dY . deq(W)) on bf16
// MFMA, and the LoRA prologue T = sigma * X . A^T.
#include "lbq_device.h"

namespace lbq {

namespace {

// ---------------------------------------------------------------------------
// Input gradient dX = dY . deq(W) ("QLoRA技术在量化微调中的应用", section
// QLoRA技术原理: backpropagation through the frozen quantized weights).
// The reduction runs over n, while the packed weight is contiguous along k:
// each thread dequantizes 8 codes of 4 consecutive rows and writes them to LDS
// transposed (k-major, 4 n per 8-byte store), so MFMA operand A (rows k) reads
// 8 consecutive n with one 16-byte LDS load.  B is dY (rows m).
// ---------------------------------------------------------------------------
constexpr int BNR = 64;        // reduction (n) per stage
constexpr int LDN = BNR + 8;   // padded LDS row

template <int KIND, int BM, int BKO>
__global__ __launch_bounds__(256) void k_bwd_dx(WView w, const uint16_t* __restrict__ dY, int m,
                                               uint16_t* __restrict__ dX, Nf4Table tab) {
  using T = WKindTraits<KIND>;
  static_assert(BKO == 128, "16 chunks of 8 codes per row");
  constexpr int WK = BKO / 2, WM = BM / 2;
  constexpr int TK = WK / 16, TM = WM / 16;
  constexpr int DCH = BM * BNR / 8 / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Wt[BKO * LDN];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[BM * LDN];
  __shared__ float cb[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wk = wave & 1, wm = wave >> 1;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t k0 = (int64_t)blockIdx.x * BKO;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t K = w.k, N = w.n;
  const int64_t KB = K * T::bits / 8;

  if constexpr (T::fmt == FMT_NF4) {
    if (tid < 16) cb[tid] = tab.c[tid];
  }

  // W ownership: rows 4*(tid>>4) .. +3 of the stage, codes [8*(tid&15), +8) of the k tile.
  const int quad = tid >> 4, chunk = tid & 15;
  const int64_t kc = k0 + 8 * chunk;
  const bool kc_ok = kc < K;

  f32x4_t acc[TK][TM];
#pragma unroll
  for (int a = 0; a < TK; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t dr[DCH];
  uint32_t wr[4];
  auto load_stage = [&](int64_t nt) {
#pragma unroll
    for (int i = 0; i < DCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 8;
      const int64_t mr = m0 + row;
      dr[i] = (mr < m && nt + col < N)
                  ? *reinterpret_cast<const u32x4_t*>(dY + mr * N + nt + col)
                  : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = nt + 4 * quad + r;
      if (n < N && kc_ok) {
        if constexpr (T::bits == 4) {
          wr[r] = *reinterpret_cast<const uint32_t*>(w.packed + n * KB + kc / 2);
        } else {
          wr[r] = *reinterpret_cast<const uint16_t*>(w.packed + n * KB + kc / 4);
        }
      } else {
        wr[r] = 0u;
      }
    }
  };
  auto store_stage = [&](int64_t nt) {
#pragma unroll
    for (int i = 0; i < DCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&Ds[row * LDN + col]) = dr[i];
    }
    float v[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = nt + 4 * quad + r;
      if (n < N && kc_ok) {
        if constexpr (T::fmt == FMT_MINMAX) {
          const int64_t gi = n * (K / T::group) + kc / T::group;
          const float s = w.scales[gi];
          const int z = w.zeros[gi];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[r][j] = (float)(code_of<T::bits>(wr[r], j) - z) * s;
        } else {
          const float a = nf4_block_scale<T::dq>(w, n * (K / 64) + kc / 64);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[r][j] = cb[code_of<4>(wr[r], j)] * a;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[r][j] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint2 p;
      p.x = pack_bf16x2(v[0][j], v[1][j]);
      p.y = pack_bf16x2(v[2][j], v[3][j]);
      *reinterpret_cast<uint2*>(&Wt[(8 * chunk + j) * LDN + 4 * quad]) = p;
    }
  };

  __syncthreads();
  load_stage(0);
  for (int64_t nt = 0; nt < N; nt += BNR) {
    __syncthreads();
    store_stage(nt);
    __syncthreads();
    if (nt + BNR < N) load_stage(nt + BNR);
#pragma unroll
    for (int ks = 0; ks < BNR; ks += 32) {
      u32x4_t af[TK], bf[TM];
#pragma unroll
      for (int a = 0; a < TK; ++a)
        af[a] = *reinterpret_cast<const u32x4_t*>(&Wt[(wk * WK + 16 * a + li) * LDN + ks + 8 * lg]);
#pragma unroll
      for (int b = 0; b < TM; ++b)
        bf[b] = *reinterpret_cast<const u32x4_t*>(&Ds[(wm * WM + 16 * b + li) * LDN + ks + 8 * lg]);
#pragma unroll
      for (int a = 0; a < TK; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma16x16x32(af[a], bf[b], acc[a][b]);
    }
  }

#pragma unroll
  for (int a = 0; a < TK; ++a) {
    const int64_t kb = k0 + wk * WK + 16 * a + 4 * lg;
    if (kb >= K) continue;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int64_t mr = m0 + wm * WM + 16 * b + li;
      if (mr >= m) continue;
      uint2 v;
      v.x = pack_bf16x2(acc[a][b][0], acc[a][b][1]);
      v.y = pack_bf16x2(acc[a][b][2], acc[a][b][3]);
      *reinterpret_cast<uint2*>(dX + mr * K + kb) = v;
    }
  }
}

template <int KIND>
struct BwdLauncher {
  static hipError_t run(const WView& w, const uint16_t* dY, int64_t m, uint16_t* dX,
                        const Nf4Table& tab, hipStream_t s) {
    constexpr int BM = 128, BKO = 128;
    const dim3 grid((unsigned)((w.k + BKO - 1) / BKO), (unsigned)((m + BM - 1) / BM));
    hipLaunchKernelGGL((k_bwd_dx<KIND, BM, BKO>), grid, dim3(256), 0, s, w, dY, (int)m, dX, tab);
    return hipGetLastError();
  }
};

// ---------------------------------------------------------------------------
// LoRA prologue: T[m][j] = bf16(sigma * sum_k X[m][k] A[j][k]) for j < r, and 0
// for r <= j < rp.  A workgroup owns 16 rows of X; its four waves split the
// K-steps and reduce through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lora_t(const uint16_t* __restrict__ X, int m, int64_t K,
                                               const uint16_t* __restrict__ A, int r, int rp,
                                               float sigma, uint16_t* __restrict__ Tout) {
  __shared__ f32x4_t red[4][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int nt = rp / 16;
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t mr = m0 + li;
  const int64_t steps = K / 32;
  for (int64_t s = wave; s < steps; s += 4) {
    const int64_t k = 32 * s + 8 * lg;
    const u32x4_t a = (mr < m) ? *reinterpret_cast<const u32x4_t*>(X + mr * K + k)
                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nt) {
        const int j = 16 * t + li;
        const u32x4_t b = (j < r) ? *reinterpret_cast<const u32x4_t*>(A + (int64_t)j * K + k)
                                  : u32x4_t{0u, 0u, 0u, 0u};
        acc[t] = mfma16x16x32(a, b, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave == 0) {
    for (int t = 0; t < nt; ++t) {
      f32x4_t v = red[0][t][lane];
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const f32x4_t u = red[q][t][lane];
        v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
      }
      const int j = 16 * t + li;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + 4 * lg + i;
        if (row < m) Tout[row * rp + j] = (uint16_t)((j < r) ? bf16_rne(sigma * v[i]) : 0u);
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_dx(WKind kind, const WView& w, const uint16_t* dY, int64_t m,
                         uint16_t* dX, const Nf4Table& tab, hipStream_t s) {
  return dispatch_kind<BwdLauncher>(kind, w, dY, m, dX, tab, s);
}

hipError_t launch_lora_t(const uint16_t* X, int64_t m, int64_t k, const uint16_t* A, int32_t r,
                         int32_t rp, float sigma, uint16_t* T, hipStream_t s) {
  const dim3 grid((unsigned)((m + 15) / 16));
  hipLaunchKernelGGL(k_lora_t, grid, dim3(256), 0, s, X, (int)m, k, A, (int)r, (int)rp, sigma, T);
  return hipGetLastError();
}

}  // namespace lbq
