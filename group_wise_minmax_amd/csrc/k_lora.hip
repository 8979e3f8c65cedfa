// Low-rank adapter pieces around the frozen quantized weight ("QLoRA技术在量化
// 微调中的应用", section QLoRA技术原理: the adapters are the only trained
// parameters and the gradient reaches them through the frozen 4-bit weight;
// the bitsandbytes FSDP-QLoRA guide, section 训练 FSDP-QLoRA, step 4 (配置
// LoRA): a LoraConfig with lora_alpha and rank r on every linear layer, so the
// adapter term is scaled by lora_alpha / r).  For
//     Y = X . deq(W)^T + sigma * (X . A^T) . B^T
// and an output gradient dY:
//     T  = bf16(sigma * X . A^T)   [m][r]   adapter product (forward and dB)
//     G  = bf16(sigma * dY . B)    [m][r]   adapter product of the gradient
//     dX = dY . deq(W) + G . A              (the input-gradient GEMM, k_bwd.hip)
//     dA = G^T . X                 [r][k]   fp32, a reduction over the m rows
//     dB = (T^T . dY)^T            [n][r]   fp32, likewise
// Both kinds of product are dense contractions and run on MFMA.  They read an
// m x k (or m x n) bf16 matrix once and are HBM bound; the rank r <= 64 only
// sets how many 16-wide MFMA tiles each step issues.
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

// ---------------------------------------------------------------------------
// Adapter product, partial sums: part[s][t][j] = sum over the s-th range of
// 32-wide K-steps of X[t][c] * A[j][c], for j < 16*NT.
//
// A workgroup owns 64 rows of X (four 16-row MFMA tiles, so every A fragment
// it loads feeds four MFMAs) and one K-range; its four waves take alternate
// K-steps and reduce through LDS.  Lane (li, lg) loads the 16-byte runs
// X[t0 + 16a + li][c + 8lg ..] and A[16jt + li][c + 8lg ..]: the MFMA's A
// operand is X and its B operand is A^T, so D[4lg + v][li] is the partial
// T[t0 + 16a + 4lg + v][16jt + li].  Rows of X past m and rows of A past r
// are read as zeros through the buffer resources' range checks.
// ---------------------------------------------------------------------------
constexpr int XA_ROWS = 64;

// One adapter product of a launch; a launch runs one or two of them (blockIdx.z
// picks the job, and blocks past a job's own split count return at once).
struct XaJob {
  const uint16_t* X;
  int64_t K;
  const uint16_t* A;
  int steps_per_split, splits;
  float* part;
};

template <int NT>
__global__ __launch_bounds__(256) void k_lora_xa(XaJob j0, XaJob j1, int m, int r) {
  const XaJob J = blockIdx.z ? j1 : j0;
  if ((int)blockIdx.y >= J.splits) return;
  const uint16_t* __restrict__ X = J.X;
  const int64_t K = J.K;
  const uint16_t* __restrict__ A = J.A;
  const int steps_per_split = J.steps_per_split;
  float* __restrict__ part = J.part;
  __shared__ f32x4_t red[3][4 * NT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * XA_ROWS;
  const int64_t steps = K / 32;
  const int64_t s_lo = (int64_t)blockIdx.y * steps_per_split;
  const int64_t s_hi = min(s_lo + steps_per_split, steps);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (int64_t)m * K * 2);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (int64_t)r * K * 2);
  uint32_t xo[4], ao[NT];
#pragma unroll
  for (int a = 0; a < 4; ++a) xo[a] = (uint32_t)(((t0 + 16 * a + li) * K + 8 * lg) * 2);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) ao[jt] = (uint32_t)(((16 * jt + li) * K + 8 * lg) * 2);

  f32x4_t acc[4][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) acc[a][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Wave w takes steps s_lo + w, s_lo + w + 4, ...; U steps' loads are issued
  // before their MFMAs.  The row offset is in the vector offset, so the range
  // check sees it; the column step goes in the scalar offset.
  constexpr int U = 2;
  for (int64_t s0 = s_lo + wave; s0 < s_hi; s0 += 4 * U) {
    u32x4_t xf[U][4], af[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = min(s0 + 4 * u, s_hi - 1);  // clamped; extra steps are skipped below
      const int so = (int)(s * 64);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        xf[u][a] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xo[a], so, 0));
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        af[u][jt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, ao[jt], so, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + 4 * u >= s_hi) break;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[a][jt] = mfma16x16x32(xf[u][a], af[u][jt], acc[a][jt]);
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) red[wave - 1][a * NT + jt][lane] = acc[a][jt];
  }
  __syncthreads();
  if (wave != 0) return;
  float* dst = part + (int64_t)blockIdx.y * m * (16 * NT);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      f32x4_t v = acc[a][jt];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const f32x4_t u = red[w][a * NT + jt][lane];
        v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 16 * a + 4 * lg + i;
        if (t < m) dst[t * (16 * NT) + 16 * jt + li] = v[i];
      }
    }
}

// Sum of part[s * stride + off] over s < splits, in order; four loads are in
// flight at a time.
__device__ __forceinline__ float sum_splits(const float* __restrict__ part, int splits, int64_t stride,
                                            int64_t off) {
  float v = 0.f;
  int s = 0;
  for (; s + 4 <= splits; s += 4) {
    const float p0 = part[(s + 0) * stride + off], p1 = part[(s + 1) * stride + off];
    const float p2 = part[(s + 2) * stride + off], p3 = part[(s + 3) * stride + off];
    v += p0; v += p1; v += p2; v += p3;
  }
  for (; s < splits; ++s) v += part[s * stride + off];
  return v;
}

// T = bf16(sigma * sum over s of part[s][t][j]) for t < m, j < r, 0 elsewhere:
// row-major [m][rp] into Trm and/or transposed [rp][mp] into Ttr (rows t in
// [m, mp) zero).  A workgroup finalizes 16 rows and transposes them in LDS.
// Fixed summation order.
constexpr int FIN_ROWS = 16;

struct FinJob {
  const float* part;
  int splits;
  uint16_t* Trm;
  uint16_t* Ttr;
};

__global__ __launch_bounds__(256) void k_lora_xa_finalize(FinJob j0, FinJob j1, int rb, int m, int r, int rp,
                                                         float sigma, int64_t mp) {
  const FinJob J = blockIdx.z ? j1 : j0;
  const float* __restrict__ part = J.part;
  const int splits = J.splits;
  uint16_t* __restrict__ Trm = J.Trm;
  uint16_t* __restrict__ Ttr = J.Ttr;
  __shared__ uint16_t tile[FIN_ROWS][64 + 2];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * FIN_ROWS;
  for (int e = tid; e < FIN_ROWS * rp; e += 256) {
    const int tt = e / rp, j = e % rp;
    const int64_t t = t0 + tt;
    uint16_t b = 0;
    if (t < m && j < r) b = (uint16_t)bf16_rne(sigma * sum_splits(part, splits, (int64_t)m * rb, t * rb + j));
    if (Trm != nullptr && t < m) Trm[t * rp + j] = b;
    tile[tt][j] = b;
  }
  if (Ttr == nullptr) return;
  __syncthreads();
  for (int e = tid; e < FIN_ROWS * rp; e += 256) {
    const int j = e / FIN_ROWS, tt = e % FIN_ROWS;
    const int64_t t = t0 + tt;
    if (t < mp) Ttr[(int64_t)j * mp + t] = tile[tt][j];
  }
}

// ---------------------------------------------------------------------------
// Outer product over the rows, partial sums: part[s][j][c] = sum over the s-th
// range of 32-row steps t of Pt[j][t] * Q[t][c], for j < 16*NT and c < C.
//
// The contraction runs down the rows of Q, so an MFMA B operand (eight
// contraction slots of one column per lane) is gathered in registers: lane
// (li, lg) loads the 8 x 8 block Q[t0 + 8lg + e][cb + 8li + 0..7], e = 0..7,
// with eight 16-byte loads, and MFMA i (i = 0..7) takes column cb + 8li + i
// of it, re-paired with v_perm.  The A operand is the 16-byte run
// Pt[16jt + li][t0 + 8lg ..] of the transposed adapter product, so
// D_i[4lg + v][li] is the partial for j = 16jt + 4lg + v and column
// cb + 8li + i.  A workgroup owns 128 columns and one row range; its four
// waves take alternate steps and reduce through LDS one j-tile at a time.
// Rows of Q past m read as zeros (buffer range check) and Pt is zero there;
// a 16-byte run that starts at or past column C feeds only columns that are
// never stored.
// ---------------------------------------------------------------------------
constexpr int OUT_COLS = 128;

// One outer product of a launch; a launch runs one or two of them (blockIdx.z
// picks the job; blocks past a job's columns or split count return at once).
struct OuterJob {
  const uint16_t* Pt;
  const uint16_t* Q;
  int64_t C;
  int steps_per_split, splits;
  float* part;
};

template <int NT>
__global__ __launch_bounds__(256) void k_lora_outer(OuterJob j0, OuterJob j1, int64_t mp, int m) {
  const OuterJob J = blockIdx.z ? j1 : j0;
  if ((int)blockIdx.y >= J.splits || (int64_t)blockIdx.x * OUT_COLS >= J.C) return;
  const uint16_t* __restrict__ Pt = J.Pt;
  const uint16_t* __restrict__ Q = J.Q;
  const int64_t C = J.C;
  const int steps_per_split = J.steps_per_split;
  float* __restrict__ part = J.part;
  __shared__ f32x4_t red[3][8][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t cb = (int64_t)blockIdx.x * OUT_COLS;
  const int64_t steps = (m + 31) / 32;
  const int64_t s_lo = (int64_t)blockIdx.y * steps_per_split;
  const int64_t s_hi = min(s_lo + steps_per_split, steps);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q, (int64_t)m * C * 2);
  const uint32_t qbase = (uint32_t)(((8 * lg) * C + cb + 8 * li) * 2);
  const uint32_t qrow = (uint32_t)(C * 2);
  const uint16_t* pbase = Pt + (int64_t)li * mp + 8 * lg;

  f32x4_t acc[NT][8];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[jt][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = NT <= 2 ? 2 : 1;  // steps in flight per wave, within the register budget
  for (int64_t s0 = s_lo + wave; s0 < s_hi; s0 += 4 * U) {
    u32x4_t qf[U][8], pf[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = min(s0 + 4 * u, s_hi - 1);
      const uint32_t vo = qbase + (uint32_t)(s * 32) * qrow;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qf[u][e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, vo + e * qrow, 0, 0));
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        pf[u][jt] = *reinterpret_cast<const u32x4_t*>(pbase + (int64_t)16 * jt * mp + s * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + 4 * u >= s_hi) break;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u32x4_t b;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          b[p] = (i & 1) ? pair_hi(qf[u][2 * p][i >> 1], qf[u][2 * p + 1][i >> 1])
                         : pair_lo(qf[u][2 * p][i >> 1], qf[u][2 * p + 1][i >> 1]);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[jt][i] = mfma16x16x32(pf[u][jt], b, acc[jt][i]);
      }
    }
  }

  const bool cok = cb + 8 * li < C;  // C % 8 == 0: a lane's 8 columns are all in or all out
  float* dst = part + (int64_t)blockIdx.y * (16 * NT) * C;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    if (jt > 0) __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave - 1][i][lane] = acc[jt][i];
    }
    __syncthreads();
    if (wave == 0) {
      f32x4_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = acc[jt][i];
#pragma unroll
        for (int w = 0; w < 3; ++w) {
          const f32x4_t u = red[w][i][lane];
          v[i][0] += u[0]; v[i][1] += u[1]; v[i][2] += u[2]; v[i][3] += u[3];
        }
      }
      if (cok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float* row = dst + (int64_t)(16 * jt + 4 * lg + q) * C + cb + 8 * li;
          *reinterpret_cast<f32x4_t*>(row) = f32x4_t{v[0][q], v[1][q], v[2][q], v[3][q]};
          *reinterpret_cast<f32x4_t*>(row + 4) = f32x4_t{v[4][q], v[5][q], v[6][q], v[7][q]};
        }
      }
    }
  }
}

// out = sum over s of part[s][j][c] for j < r: out[j][c] ([r][C]) or, with
// transpose, out[c][j] ([C][r]).  A workgroup reduces 16 columns; the
// transposed store goes through LDS so that it is row-contiguous.  Fixed
// summation order.
constexpr int RED_COLS = 16;

struct RedJob {
  const float* part;
  int splits;
  int64_t C;
  bool transpose;
  float* out;
};

__global__ __launch_bounds__(256) void k_lora_outer_reduce(RedJob j0, RedJob j1, int rb, int r) {
  const RedJob J = blockIdx.z ? j1 : j0;
  if ((int64_t)blockIdx.x * RED_COLS >= J.C) return;
  const float* __restrict__ part = J.part;
  const int splits = J.splits;
  const int64_t C = J.C;
  const bool transpose = J.transpose;
  float* __restrict__ out = J.out;
  __shared__ float tile[RED_COLS][64 + 1];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * RED_COLS;
  for (int e = tid; e < r * RED_COLS; e += 256) {
    const int j = e / RED_COLS, cc = e % RED_COLS;
    const int64_t c = c0 + cc;
    const float v = c < C ? sum_splits(part, splits, (int64_t)rb * C, (int64_t)j * C + c) : 0.f;
    if (!transpose) {
      if (c < C) out[(int64_t)j * C + c] = v;
    } else {
      tile[cc][j] = v;
    }
  }
  if (!transpose) return;
  __syncthreads();
  for (int e = tid; e < RED_COLS * r; e += 256) {
    const int cc = e / r, j = e % r;
    if (c0 + cc < C) out[(c0 + cc) * r + j] = tile[cc][j];
  }
}

__global__ __launch_bounds__(256) void k_fill_zero_f32(float* __restrict__ p, int64_t count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < count) p[idx] = 0.f;
}

int tiles_of(int32_t r) { return (r + 15) / 16; }

// K-ranges per 64-row block: about 512 workgroups, at least 8 steps each.
int xa_splits(int64_t m, int64_t K) {
  const int64_t blocks = (m + XA_ROWS - 1) / XA_ROWS;
  const int64_t steps = K / 32;
  int64_t sp = (512 + blocks - 1) / blocks;
  const int64_t cap = steps / 8;
  if (sp > cap) sp = cap;
  return (int)(sp < 1 ? 1 : sp);
}

// Row ranges per 128-column block: about 384 workgroups, at least 8 steps each.
int outer_splits(int64_t m, int64_t C) {
  const int64_t blocks = (C + OUT_COLS - 1) / OUT_COLS;
  const int64_t steps = (m + 31) / 32;
  int64_t sp = (384 + blocks - 1) / blocks;
  const int64_t cap = steps / 8;
  if (sp > cap) sp = cap;
  return (int)(sp < 1 ? 1 : sp);
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

size_t lora_xa_part_bytes(int64_t m, int64_t K, int32_t r) {
  return (size_t)xa_splits(m, K) * (size_t)m * (size_t)(16 * tiles_of(r)) * sizeof(float);
}

// One or two adapter products (count = 1 or 2; jobs[i] = X, K, A with its
// outputs), each with its own area of fp32 partials, in one product launch and
// one finalize launch.
hipError_t launch_lora_xa_jobs(int count, const uint16_t* const* Xs, const int64_t* Ks, const uint16_t* const* As,
                               uint16_t* const* Trms, uint16_t* const* Ttrs, int64_t m, int32_t r, int32_t rp,
                               float sigma, float* part, int64_t mp, hipStream_t s) {
  XaJob xj[2];
  FinJob fj[2];
  int sp_max = 0;
  float* p = part;
  for (int i = 0; i < count; ++i) {
    const int sp = xa_splits(m, Ks[i]);
    const int64_t steps = Ks[i] / 32;
    xj[i] = XaJob{Xs[i], Ks[i], As[i], (int)((steps + sp - 1) / sp), sp, p};
    fj[i] = FinJob{p, sp, Trms[i], Ttrs[i]};
    sp_max = sp > sp_max ? sp : sp_max;
    p += lora_xa_part_bytes(m, Ks[i], r) / sizeof(float);
  }
  if (count == 1) xj[1] = xj[0], fj[1] = fj[0];
  const dim3 grid((unsigned)((m + XA_ROWS - 1) / XA_ROWS), (unsigned)sp_max, (unsigned)count);
  const int nt = tiles_of(r);
  switch (nt) {
    case 1: hipLaunchKernelGGL(k_lora_xa<1>, grid, dim3(256), 0, s, xj[0], xj[1], (int)m, (int)r); break;
    case 2: hipLaunchKernelGGL(k_lora_xa<2>, grid, dim3(256), 0, s, xj[0], xj[1], (int)m, (int)r); break;
    case 3: hipLaunchKernelGGL(k_lora_xa<3>, grid, dim3(256), 0, s, xj[0], xj[1], (int)m, (int)r); break;
    default: hipLaunchKernelGGL(k_lora_xa<4>, grid, dim3(256), 0, s, xj[0], xj[1], (int)m, (int)r); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // every job with a transposed output covers mp rows, else m
  int64_t rows = m;
  for (int i = 0; i < count; ++i)
    if (Ttrs[i] != nullptr) rows = mp;
  hipLaunchKernelGGL(k_lora_xa_finalize, dim3((unsigned)((rows + FIN_ROWS - 1) / FIN_ROWS), 1, (unsigned)count),
                     dim3(256), 0, s, fj[0], fj[1], 16 * nt, (int)m, (int)r, (int)rp, sigma, mp);
  return hipGetLastError();
}

hipError_t launch_lora_xa(const uint16_t* X, int64_t m, int64_t K, const uint16_t* A, int32_t r,
                          int32_t rp, float sigma, float* part, uint16_t* Trm, uint16_t* Ttr,
                          int64_t mp, hipStream_t s) {
  return launch_lora_xa_jobs(1, &X, &K, &A, &Trm, &Ttr, m, r, rp, sigma, part, mp, s);
}

size_t lora_outer_part_bytes(int64_t m, int64_t C, int32_t r) {
  return (size_t)outer_splits(m, C) * (size_t)(16 * tiles_of(r)) * (size_t)C * sizeof(float);
}

// One or two outer products (count = 1 or 2), each with its own area of fp32
// partials, in one product launch and one reduce launch.
hipError_t launch_lora_outer_jobs(int count, const uint16_t* const* Pts, const uint16_t* const* Qs,
                                  const int64_t* Cs, const bool* transposes, float* const* outs, int64_t mp,
                                  int32_t r, int64_t m, float* part, hipStream_t s) {
  OuterJob oj[2];
  RedJob rj[2];
  int sp_max = 0;
  int64_t c_max = 0;
  float* p = part;
  for (int i = 0; i < count; ++i) {
    const int sp = outer_splits(m, Cs[i]);
    const int64_t steps = (m + 31) / 32;
    oj[i] = OuterJob{Pts[i], Qs[i], Cs[i], (int)((steps + sp - 1) / sp), sp, p};
    rj[i] = RedJob{p, sp, Cs[i], transposes[i], outs[i]};
    sp_max = sp > sp_max ? sp : sp_max;
    c_max = Cs[i] > c_max ? Cs[i] : c_max;
    p += lora_outer_part_bytes(m, Cs[i], r) / sizeof(float);
  }
  if (count == 1) oj[1] = oj[0], rj[1] = rj[0];
  const dim3 grid((unsigned)((c_max + OUT_COLS - 1) / OUT_COLS), (unsigned)sp_max, (unsigned)count);
  const int nt = tiles_of(r);
  switch (nt) {
    case 1: hipLaunchKernelGGL(k_lora_outer<1>, grid, dim3(256), 0, s, oj[0], oj[1], mp, (int)m); break;
    case 2: hipLaunchKernelGGL(k_lora_outer<2>, grid, dim3(256), 0, s, oj[0], oj[1], mp, (int)m); break;
    case 3: hipLaunchKernelGGL(k_lora_outer<3>, grid, dim3(256), 0, s, oj[0], oj[1], mp, (int)m); break;
    default: hipLaunchKernelGGL(k_lora_outer<4>, grid, dim3(256), 0, s, oj[0], oj[1], mp, (int)m); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lora_outer_reduce, dim3((unsigned)((c_max + RED_COLS - 1) / RED_COLS), 1, (unsigned)count),
                     dim3(256), 0, s, rj[0], rj[1], 16 * nt, (int)r);
  return hipGetLastError();
}

hipError_t launch_lora_outer(const uint16_t* Pt, int64_t mp, int32_t r, const uint16_t* Q, int64_t m,
                             int64_t C, bool transpose, float* part, float* out, hipStream_t s) {
  return launch_lora_outer_jobs(1, &Pt, &Q, &C, &transpose, &out, mp, r, m, part, s);
}

}  // namespace lbq
