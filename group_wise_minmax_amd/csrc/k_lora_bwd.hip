// LoRA backward pieces ("QLoRA技术在量化微调中的应用", section QLoRA技术原理: the
// gradient passes through the frozen quantized weight into the low-rank
// adapters).  For Y = X . deq(W)^T + sigma * (X . A^T) . B^T and an output
// gradient dY:
//     G  = bf16(sigma * dY . B)          [m][rp]   (k_lora_t on dY and B^T)
//     dX = dY . deq(W) + G . A           (k_bwd_dx with its LoRA slab)
//     dA = G^T . X                       [r][k]    fp32
//     dB = (T^T . dY)^T, T = bf16(sigma * X . A^T)   [n][r]   fp32
// This file holds the transpose of B and the two reductions over m (dA, dB).
#include "lbq_device.h"

namespace lbq {

namespace {

// Bt[j][i] = B[i][j] for j < r, 0 for r <= j < rp  (B is [n][r], Bt is [rp][n]).
__global__ __launch_bounds__(256) void k_transpose_b(const uint16_t* __restrict__ B, int64_t n, int r,
                                                    int rp, uint16_t* __restrict__ Bt) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rp * n) return;
  const int j = (int)(idx / n);
  const int64_t i = idx % n;
  Bt[idx] = j < r ? B[i * r + j] : (uint16_t)0;
}

// part[s][j][c] = sum over the s-th range of rows t of P[t][j] * Q[t][c], for
// j < RB (P is [m][rp] bf16, zero past r) and c < C (Q is [m][C] bf16).  A
// thread owns two adjacent columns and RB x 2 fp32 accumulators; 64-row tiles
// of P are staged in LDS and read as broadcasts.
constexpr int OT = 64;  // rows of P per LDS tile

template <int RB>
__global__ __launch_bounds__(256) void k_lora_outer(const uint16_t* __restrict__ P, int rp,
                                                   const uint16_t* __restrict__ Q, int64_t m,
                                                   int64_t C, int rows_per_split,
                                                   float* __restrict__ part) {
  __shared__ uint32_t Ps[OT][RB / 2];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 512 + 2 * tid;
  const int64_t m_lo = (int64_t)blockIdx.y * rows_per_split;
  const int64_t m_hi = min(m_lo + rows_per_split, m);
  const bool cok = c0 < C;  // C is even, so c0 + 1 < C as well
  float acc[RB][2];
#pragma unroll
  for (int j = 0; j < RB; ++j) acc[j][0] = acc[j][1] = 0.f;

  for (int64_t mt = m_lo; mt < m_hi; mt += OT) {
    const int rows = (int)min((int64_t)OT, m_hi - mt);
    __syncthreads();
    for (int e = tid; e < OT * RB / 2; e += 256) {
      const int row = e / (RB / 2), col = e % (RB / 2);
      Ps[row][col] = row < rows ? reinterpret_cast<const uint32_t*>(P + (mt + row) * rp)[col] : 0u;
    }
    __syncthreads();
    for (int i = 0; i < rows; ++i) {
      const uint32_t q = cok ? *reinterpret_cast<const uint32_t*>(Q + (mt + i) * C + c0) : 0u;
      const float q0 = bf16_lo(q), q1 = bf16_hi(q);
#pragma unroll
      for (int jj = 0; jj < RB / 2; ++jj) {
        const uint32_t p = Ps[i][jj];
        const float p0 = bf16_lo(p), p1 = bf16_hi(p);
        acc[2 * jj][0] = fmaf(p0, q0, acc[2 * jj][0]);
        acc[2 * jj][1] = fmaf(p0, q1, acc[2 * jj][1]);
        acc[2 * jj + 1][0] = fmaf(p1, q0, acc[2 * jj + 1][0]);
        acc[2 * jj + 1][1] = fmaf(p1, q1, acc[2 * jj + 1][1]);
      }
    }
  }
  if (cok) {
    float* dst = part + (int64_t)blockIdx.y * RB * C;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      dst[(int64_t)j * C + c0] = acc[j][0];
      dst[(int64_t)j * C + c0 + 1] = acc[j][1];
    }
  }
}

// out = sum over s of part[s][j][c] for j < r: out[j][c] ([r][C]) or, with
// transpose, out[c][j] ([C][r]).  Fixed summation order (deterministic).
__global__ __launch_bounds__(256) void k_lora_outer_reduce(const float* __restrict__ part, int splits,
                                                          int RB, int r, int64_t C, bool transpose,
                                                          float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)r * C) return;
  const int j = (int)(idx / C);
  const int64_t c = idx % C;
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += part[((int64_t)s * RB + j) * C + c];
  if (transpose) out[c * r + j] = v;
  else out[(int64_t)j * C + c] = v;
}

__global__ __launch_bounds__(256) void k_fill_zero_f32(float* __restrict__ p, int64_t count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < count) p[idx] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero_f32(float* p, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, p, count);
  return hipGetLastError();
}

hipError_t launch_transpose_b(const uint16_t* B, int64_t n, int32_t r, int32_t rp, uint16_t* Bt,
                              hipStream_t s) {
  const int64_t total = (int64_t)rp * n;
  hipLaunchKernelGGL(k_transpose_b, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, B, n, (int)r,
                     (int)rp, Bt);
  return hipGetLastError();
}

int lora_outer_splits(int64_t m, int64_t C) {
  // about 256 workgroups, ranges of whole 64-row tiles
  const int64_t cblocks = (C + 511) / 512;
  int64_t sp = (256 + cblocks - 1) / cblocks;
  const int64_t tiles = (m + OT - 1) / OT;
  if (sp > tiles) sp = tiles;
  return (int)(sp < 1 ? 1 : sp);
}

size_t lora_outer_part_bytes(int64_t m, int64_t C, int32_t r) {
  const int rb = (r + 15) / 16 * 16;
  return (size_t)lora_outer_splits(m, C) * (size_t)rb * (size_t)C * sizeof(float);
}

hipError_t launch_lora_outer(const uint16_t* P, int32_t r, int32_t rp, const uint16_t* Q, int64_t m,
                             int64_t C, bool transpose, float* part, float* out, hipStream_t s) {
  const int sp = lora_outer_splits(m, C);
  const int64_t tiles = (m + OT - 1) / OT;
  const int rows_per_split = (int)(((tiles + sp - 1) / sp) * OT);
  const dim3 grid((unsigned)((C + 511) / 512), (unsigned)sp);
  const int rb = (r + 15) / 16 * 16;
  switch (rb) {
    case 16: hipLaunchKernelGGL(k_lora_outer<16>, grid, dim3(256), 0, s, P, (int)rp, Q, m, C, rows_per_split, part); break;
    case 32: hipLaunchKernelGGL(k_lora_outer<32>, grid, dim3(256), 0, s, P, (int)rp, Q, m, C, rows_per_split, part); break;
    case 48: hipLaunchKernelGGL(k_lora_outer<48>, grid, dim3(256), 0, s, P, (int)rp, Q, m, C, rows_per_split, part); break;
    default: hipLaunchKernelGGL(k_lora_outer<64>, grid, dim3(256), 0, s, P, (int)rp, Q, m, C, rows_per_split, part); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)r * C;
  hipLaunchKernelGGL(k_lora_outer_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, sp,
                     rb, (int)r, C, transpose, out);
  return hipGetLastError();
}

}  // namespace lbq
