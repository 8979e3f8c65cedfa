// Small-batch forward (2 <= m <= 64): Y = X . deq(W)^T on bf16 MFMA while the
// packed weight streams from HBM once.
//
// The kernel that unpacks and dequantizes the weight to bf16 before the
// matmul: bitsandbytes FSDP-QLoRA guide, section 通过BitsAndBytesConfig配置.
// Formats: GreenBit.AI "只需单卡RTX 3090，低比特量化训练就能实现LLaMA-3 8B全参微调",
// section 模型量化 (MinMax INT4 g128 / INT2 g64) and "QLoRA技术在量化微调中的应用",
// section QLoRA技术原理 (NF4, double quantization).
//
// Work split: a workgroup owns 64 rows of W (one 16-row MFMA tile per wave)
// and one of KS contiguous K ranges, walked in 256-code chunks.  Per chunk the
// workgroup stages the packed bytes of its 64 rows, the x rows (already in the
// k-slot order the weight fragments use) and the group metadata into one half
// of a double-buffered LDS area with coalesced 16-byte loads issued one chunk
// ahead; each lane then reads an A fragment (8 codes of one row) with one
// 4-byte LDS read.  With KS > 1 the ranges' fp32 partials are summed (with the
// LoRA term) by a second, deterministic kernel.
//  * MinMax: codes become the bf16 numbers 128 + q (v_perm_b32 next to byte
//    0x43; exact for q < 128) and the MFMA accumulates sum x (128 + q) per
//    group; a second MFMA with an all-ones A operand accumulates sum x in the
//    same layout, so at the end of each group
//        acc += s * (sum x (128 + q) - (128 + z) * sum x).
//    X is read in the matching k-slot order (permuted within 8-code groups).
//  * NF4: a packed byte (two codes) indexes a 256-entry table of bf16 level
//    pairs in LDS; the block absmax scales the per-block accumulator.
#include "lbq_device.h"

namespace lbq {

namespace {

constexpr int kThreads = 256;
constexpr int KC = 256;        // codes per chunk
constexpr int ROWS = 64;       // W rows per workgroup
constexpr int kLutCopies = 32;
constexpr uint32_t k43 = 0x43434343u;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

__device__ __forceinline__ uint32_t pr01(uint32_t v) { return perm_b32(k43, v, 0x04010400u); }
__device__ __forceinline__ uint32_t pr23(uint32_t v) { return perm_b32(k43, v, 0x04030402u); }

template <int KIND>
struct SkTraits {
  using T = WKindTraits<KIND>;
  static constexpr int RB = KC * T::bits / 8;   // packed bytes per row per chunk (128 / 64)
  static constexpr int RBP = RB + 16;           // padded LDS row: conflict-free A reads
  static constexpr int GRP = T::fmt == FMT_MINMAX ? T::group : 64;
  static constexpr int KSG = GRP / 32;          // k-steps per group / block
};

// A fragment (8 codes -> 4 dwords of bf16 pairs) for k-step t of row `row`
// and lane group lg from a staged chunk.  Its k-slot order matches the order
// in which x is stored (arrange8()).
template <int KIND>
__device__ __forceinline__ u32x4_t a_frag(const uint8_t* wl, int row, int lg, int t,
                                          const uint32_t* lut, int lane32) {
  using T = WKindTraits<KIND>;
  using S = SkTraits<KIND>;
  if constexpr (T::bits == 4) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(wl + row * S::RBP + 16 * t + 4 * lg);
    if constexpr (T::fmt == FMT_MINMAX) {
      const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
      return u32x4_t{pr01(lo), pr23(lo), pr01(hi), pr23(hi)};  // codes 1,3 5,7 0,2 4,6
    } else {
      return u32x4_t{lut[(w & 0xFFu) * kLutCopies + lane32], lut[((w >> 8) & 0xFFu) * kLutCopies + lane32],
                     lut[((w >> 16) & 0xFFu) * kLutCopies + lane32], lut[(w >> 24) * kLutCopies + lane32]};
    }
  } else {
    // 2-bit: one dword = 16 codes = k-steps 2T and 2T+1 of lane group lg
    const uint32_t w = *reinterpret_cast<const uint32_t*>(wl + row * S::RBP + 16 * (t >> 1) + 4 * lg);
    const uint32_t c3 = w & 0x03030303u, c2 = (w >> 2) & 0x03030303u;
    const uint32_t c1 = (w >> 4) & 0x03030303u, c0 = (w >> 6) & 0x03030303u;
    if ((t & 1) == 0) return u32x4_t{pr01(c3), pr01(c2), pr01(c1), pr01(c0)};  // 3,7 2,6 1,5 0,4
    return u32x4_t{pr23(c3), pr23(c2), pr23(c1), pr23(c0)};                   // 11,15 10,14 9,13 8,12
  }
}

// 8 consecutive x values (natural bf16 pairs) -> the k-slot order of a_frag.
template <int KIND>
__device__ __forceinline__ u32x4_t arrange8(const u32x4_t& v) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_NF4) {
    return v;
  } else if constexpr (T::bits == 4) {
    return u32x4_t{pair_hi(v[0], v[1]), pair_hi(v[2], v[3]), pair_lo(v[0], v[1]), pair_lo(v[2], v[3])};
  } else {
    return u32x4_t{pair_hi(v[1], v[3]), pair_lo(v[1], v[3]), pair_hi(v[0], v[2]), pair_lo(v[0], v[2])};
  }
}

// Element offset (within the chunk) of the 8 x values lane group lg feeds to k-step t.
template <int KIND>
__device__ __forceinline__ int x_off(int lg, int t) {
  if constexpr (WKindTraits<KIND>::bits == 4) return 32 * t + 8 * lg;
  return 64 * (t >> 1) + 16 * lg + 8 * (t & 1);
}

// Row tile `tile` (ROWS rows of W) over K range `split` of ks_count; with
// `part` set, the fp32 sums go to part[split][m][n], else bf16 to Y.
template <int KIND, int MB>
__device__ __forceinline__ void skinny_tile(const WView& w, const uint16_t* __restrict__ X, int m,
                                            uint16_t* __restrict__ Y, int64_t ldy,
                                            const int32_t* __restrict__ out_rows,
                                            float* __restrict__ part, int ks_count,
                                            const LoraEpi& lora, const Nf4Table& tab, int tile, int split) {
  using T = WKindTraits<KIND>;
  using S = SkTraits<KIND>;
  constexpr int RB = S::RB, RBP = S::RBP, KSG = S::KSG, GRP = S::GRP;
  constexpr int NG = KC / GRP;          // groups (blocks) per chunk
  constexpr int LDX = KC + 8;           // padded x row (bf16)
  constexpr int WCOL = RB / 16;         // 16-byte W columns per row
  constexpr int WLD = ROWS * WCOL / kThreads;   // W loads per thread per chunk
  constexpr int XLD = MB * 16 * (KC / 8) / kThreads;  // X loads per thread per chunk
  __shared__ __attribute__((aligned(16))) uint8_t Ws[2][ROWS * RBP];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][MB * 16 * LDX];
  __shared__ float2 meta[2][ROWS][NG];  // (scale, 128 + zero) or (absmax, 0)
  __shared__ uint32_t lut[T::fmt == FMT_NF4 ? 256 * kLutCopies : 1];
  __shared__ float cbs[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t n0 = (int64_t)tile * ROWS;
  const int64_t K = w.k;
  const int64_t KB = K * T::bits / 8;
  const int64_t gpr = K / GRP;
  const int nchunk = (int)((K + KC - 1) / KC);
  const int per = (nchunk + ks_count - 1) / ks_count;
  const int c_lo = split * per;
  const int c_hi = min(c_lo + per, nchunk);

  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tid == i) cbs[i] = tab.c[i];
    __syncthreads();
    for (int e = tid; e < 256 * kLutCopies; e += kThreads) {
      const int b = e / kLutCopies;
      lut[e] = (uint32_t)bf16_rne(cbs[b >> 4]) | ((uint32_t)bf16_rne(cbs[b & 15]) << 16);
    }
  }

  // ---- staging of one chunk: packed W rows, arranged X rows, group metadata --
  u32x4_t wr[WLD], xr[XLD];
  float2 mr;
  auto load = [&](int c) {
    const int64_t kc = (int64_t)c * KC;
    const int64_t kend = (K - kc) < KC ? (K - kc) : KC;  // codes in this chunk (multiple of 64)
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int e = tid + kThreads * i;
      const int row = e / WCOL, col = e % WCOL;
      const int64_t n = min(n0 + row, w.n - 1);
      const bool ok = col * 16 * 8 / T::bits < kend;
      const int64_t off = n * KB + kc * T::bits / 8 + (ok ? col * 16 : 0);
      wr[i] = *reinterpret_cast<const u32x4_t*>(w.packed + off);
      if (!ok) wr[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
      const int e = tid + kThreads * i;
      const int row = e / (KC / 8), col = e % (KC / 8);
      const int64_t mrow = min((int64_t)row, (int64_t)m - 1);
      const bool ok = col * 8 < kend;
      xr[i] = *reinterpret_cast<const u32x4_t*>(X + mrow * K + kc + (ok ? col * 8 : 0));
      if (!ok) xr[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
    {
      const int row = tid / 4, j = tid % 4;
      const int64_t n = min(n0 + row, w.n - 1);
      const bool ok = j < NG && (int64_t)j * GRP < kend;
      const int64_t gi = n * gpr + (ok ? (kc / GRP + j) : 0);
      if constexpr (T::fmt == FMT_MINMAX) {
        mr = make_float2(w.scales[gi], (float)(128 + (int)w.zeros[gi]));
      } else {
        mr = make_float2(nf4_block_scale<T::dq>(w, gi), 0.f);
      }
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int e = tid + kThreads * i;
      *reinterpret_cast<u32x4_t*>(&Ws[b][(e / WCOL) * RBP + (e % WCOL) * 16]) = wr[i];
    }
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
      const int e = tid + kThreads * i;
      *reinterpret_cast<u32x4_t*>(&Xs[b][(e / (KC / 8)) * LDX + (e % (KC / 8)) * 8]) = arrange8<KIND>(xr[i]);
    }
    if (tid / 4 < ROWS && tid % 4 < NG) meta[b][tid / 4][tid % 4] = mr;
  };

  f32x4_t acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t ones = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
  const int lane32 = lane & 31;
  const int trow = 16 * wave;  // this wave's 16-row tile

  auto compute = [&](int b, int c) {
    const int64_t kc = (int64_t)c * KC;
    const int64_t kend = (K - kc) < KC ? (K - kc) : KC;
    const uint8_t* wl = Ws[b];
    for (int gi = 0; gi < NG; ++gi) {
      if ((int64_t)gi * GRP >= kend) break;
      f32x4_t ag[MB], xs[MB];
#pragma unroll
      for (int q = 0; q < MB; ++q) ag[q] = xs[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < KSG; ++tt) {
        const int t = gi * KSG + tt;
        const u32x4_t af = a_frag<KIND>(wl, trow + li, lg, t, lut, lane32);
#pragma unroll
        for (int q = 0; q < MB; ++q) {
          const u32x4_t xf = *reinterpret_cast<const u32x4_t*>(&Xs[b][(16 * q + li) * LDX + x_off<KIND>(lg, t)]);
          if constexpr (T::fmt == FMT_MINMAX) xs[q] = mfma16x16x32(ones, xf, xs[q]);
          ag[q] = mfma16x16x32(af, xf, ag[q]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 md = meta[b][trow + 4 * lg + i][gi];
#pragma unroll
        for (int q = 0; q < MB; ++q) {
          if constexpr (T::fmt == FMT_MINMAX) {
            acc[q][i] = fmaf(md.x, fmaf(-md.y, xs[q][i], ag[q][i]), acc[q][i]);
          } else {
            acc[q][i] = fmaf(md.x, ag[q][i], acc[q][i]);
          }
        }
      }
    }
  };

  if (c_lo < c_hi) {
    load(c_lo);
    store(0);
    if (c_lo + 1 < c_hi) load(c_lo + 1);
    __syncthreads();
    int b = 0;
    for (int c = c_lo; c < c_hi; ++c) {
      if (c + 1 < c_hi) {
        store(b ^ 1);
        if (c + 2 < c_hi) load(c + 2);
      }
      compute(b, c);
      __syncthreads();
      b ^= 1;
    }
  }

  // lane holds D[n = n0 + trow + 4lg + i][m = 16q + li]
#pragma unroll
  for (int q = 0; q < MB; ++q) {
    const int mrow = 16 * q + li;
    if (mrow >= m) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + trow + 4 * lg + i;
      if (n >= w.n) continue;
      if (part != nullptr) {
        part[((int64_t)split * m + mrow) * w.n + n] = acc[q][i];
      } else {
        Y[(int64_t)mrow * ldy + (out_rows ? (int64_t)out_rows[n] : n)] = (uint16_t)bf16_rne(acc[q][i]);
      }
    }
  }
}

template <int KIND, int MB>
__global__ __launch_bounds__(kThreads) void k_skinny(WView w, const uint16_t* __restrict__ X, int m,
                                                    uint16_t* __restrict__ Y, int64_t ldy,
                                                    const int32_t* __restrict__ out_rows,
                                                    float* __restrict__ part, int ks_count,
                                                    LoraEpi lora, Nf4Table tab) {
  skinny_tile<KIND, MB>(w, X, m, Y, ldy, out_rows, part, ks_count, lora, tab, blockIdx.x, blockIdx.y);
}

// Several weights that share X in one launch.  Each keeps the K split it
// has alone (ks[i], so its outputs equal the single-weight call's): weight i
// owns workgroups [wg_end[i-1], wg_end[i]) = tiles x ks[i], and when
// ks[i] > 1 its partials [ks][m][n] start at part + part_off[i].
struct SkinnySet {
  WView w[kGemvMaxGroup];
  uint16_t* y[kGemvMaxGroup];
  int64_t ldy[kGemvMaxGroup];
  const int32_t* out_rows[kGemvMaxGroup];
  int64_t part_off[kGemvMaxGroup];
  int64_t col_end[kGemvMaxGroup];  // prefix sums of n (the reduce's column space)
  int wg_end[kGemvMaxGroup];
  int ks[kGemvMaxGroup];
  int count;
};

template <int KIND, int MB>
__global__ __launch_bounds__(kThreads) void k_skinny_set(SkinnySet set, const uint16_t* __restrict__ X, int m,
                                                        float* __restrict__ part, Nf4Table tab) {
  const int b = blockIdx.x;
  int pi = 0, wbeg = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count && b >= set.wg_end[i - 1]) { pi = i; wbeg = set.wg_end[i - 1]; }
  const int ks = set.ks[pi];
  const int tiles = (int)((set.w[pi].n + ROWS - 1) / ROWS);
  const int r = b - wbeg;
  const LoraEpi none{nullptr, nullptr, 0, 0};
  skinny_tile<KIND, MB>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi],
                        ks == 1 ? nullptr : part + set.part_off[pi], ks, none, tab, r % tiles, r / tiles);
}

// Y[m][col(n)] = bf16( sum over K ranges of part + LoRA term ).  Row mr =
// blockIdx.y; the partials are summed in range order, their loads issued
// eight at a time.
__global__ __launch_bounds__(256) void k_skinny_reduce(const float* __restrict__ part, int ks_count,
                                                      int m, int64_t n, uint16_t* __restrict__ Y,
                                                      int64_t ldy, const int32_t* __restrict__ out_rows,
                                                      LoraEpi lora) {
  const int64_t mr = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  const float* p = part + mr * n + c;
  const int64_t stride = (int64_t)m * n;
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= ks_count; s += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = p[(s + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += t[j];
  }
  for (; s < ks_count; ++s) v += p[s * stride];
  if (lora.t != nullptr) {
    for (int j = 0; j < lora.r; ++j)
      v = fmaf(bf16_lo(lora.t[mr * lora.rp + j]), bf16_lo(lora.b[c * lora.r + j]), v);
  }
  Y[mr * ldy + (out_rows ? (int64_t)out_rows[c] : c)] = (uint16_t)bf16_rne(v);
}

// The set form: columns of all weights side by side (weight i owns columns
// [col_end[i-1], col_end[i])), same summation order as k_skinny_reduce.
__global__ __launch_bounds__(256) void k_skinny_reduce_set(const float* __restrict__ part, int m, SkinnySet set) {
  const int64_t mr = blockIdx.y;
  const int64_t cg = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t ncol = set.col_end[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count) ncol = set.col_end[i];
  if (cg >= ncol) return;
  int pi = 0;
  int64_t cbeg = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count && cg >= set.col_end[i - 1]) { pi = i; cbeg = set.col_end[i - 1]; }
  const int ks_count = set.ks[pi];
  if (ks_count == 1) return;  // written by the main kernel
  const int64_t n = set.w[pi].n, c = cg - cbeg;
  const float* p = part + set.part_off[pi] + mr * n + c;
  const int64_t stride = (int64_t)m * n;
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= ks_count; s += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = p[(s + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += t[j];
  }
  for (; s < ks_count; ++s) v += p[s * stride];
  const int32_t* orow = set.out_rows[pi];
  set.y[pi][mr * set.ldy[pi] + (orow ? (int64_t)orow[c] : c)] = (uint16_t)bf16_rne(v);
}

template <int KIND, int MB>
hipError_t launch_set_mb(const SkinnySet& set, int64_t wgs, int64_t ncol, bool reduce, const uint16_t* X,
                         int64_t m, float* part, const Nf4Table& tab, hipStream_t s) {
  hipLaunchKernelGGL((k_skinny_set<KIND, MB>), dim3((unsigned)wgs), dim3(kThreads), 0, s, set, X, (int)m, part,
                     tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !reduce) return e;
  hipLaunchKernelGGL(k_skinny_reduce_set, dim3((unsigned)((ncol + 255) / 256), (unsigned)m), dim3(256), 0, s,
                     part, (int)m, set);
  return hipGetLastError();
}

template <int KIND>
struct SkinnySetLauncher {
  static hipError_t run(const SkinnySet& set, int64_t wgs, int64_t ncol, bool reduce, const uint16_t* X,
                        int64_t m, float* part, const Nf4Table& tab, hipStream_t s) {
    if (m <= 16) return launch_set_mb<KIND, 1>(set, wgs, ncol, reduce, X, m, part, tab, s);
    if (m <= 32) return launch_set_mb<KIND, 2>(set, wgs, ncol, reduce, X, m, part, tab, s);
    return launch_set_mb<KIND, 4>(set, wgs, ncol, reduce, X, m, part, tab, s);
  }
};

template <int KIND, int MB>
hipError_t launch_mb(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                     const int32_t* out_rows, float* part, int ks, const LoraEpi& lora,
                     const Nf4Table& tab, hipStream_t s) {
  const dim3 grid((unsigned)((w.n + ROWS - 1) / ROWS), (unsigned)ks);
  const bool direct = ks == 1 && lora.t == nullptr;
  hipLaunchKernelGGL((k_skinny<KIND, MB>), grid, dim3(kThreads), 0, s, w, X, (int)m, Y, ldy, out_rows,
                     direct ? nullptr : part, ks, lora, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || direct) return e;
  hipLaunchKernelGGL(k_skinny_reduce, dim3((unsigned)((w.n + 255) / 256), (unsigned)m), dim3(256), 0, s, part,
                     ks, (int)m, w.n, Y, ldy, out_rows, lora);
  return hipGetLastError();
}

template <int KIND>
struct SkinnyLauncher {
  static hipError_t run(const WView& w, const uint16_t* X, int64_t m, uint16_t* Y, int64_t ldy,
                        const int32_t* out_rows, float* part, int ks, const LoraEpi& lora,
                        const Nf4Table& tab, hipStream_t s) {
    if (m <= 16) return launch_mb<KIND, 1>(w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
    if (m <= 32) return launch_mb<KIND, 2>(w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
    return launch_mb<KIND, 4>(w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
  }
};

}  // namespace

int skinny_splits(int64_t n, int64_t k, int64_t m) {
  return skinny_splits_tiles((n + ROWS - 1) / ROWS, k, m);
}

int skinny_splits_tiles(int64_t tiles, int64_t k, int64_t m) {
  const int64_t nchunk = (k + KC - 1) / KC;
  // Aim at ~512 workgroups, but keep the fp32 partial traffic (ks * m * n * 8
  // bytes) below the packed weight (n * k / 2 bytes for 4-bit).  Measured on
  // the 8B layer: more splits lose to the shorter K ranges, a tighter cap
  // (a quarter of the weight) costs 3% at m = 16 and 15% at m = 32.
  int64_t ks = (512 + tiles - 1) / tiles;
  const int64_t cap = (k / 16) / (m < 1 ? 1 : m);
  if (ks > cap) ks = cap;
  if (ks > nchunk) ks = nchunk;
  if (ks < 1) ks = 1;
  return (int)ks;
}

size_t skinny_workspace_bytes(int64_t n, int64_t k, int64_t m, bool lora) {
  const int ks = skinny_splits(n, k, m);
  if (ks == 1 && !lora) return 0;
  return (size_t)ks * (size_t)m * (size_t)n * sizeof(float);
}

size_t skinny_set_workspace_bytes(const int64_t* ns, int count, int64_t k, int64_t m) {
  size_t b = 0;
  for (int i = 0; i < count; ++i) b += skinny_workspace_bytes(ns[i], k, m, false);
  return b;
}

hipError_t launch_skinny_set(WKind kind, const WView* ws, uint16_t* const* ys, const int64_t* ldys,
                             const int32_t* const* out_rows, int count, const uint16_t* X, int64_t m, float* part,
                             const Nf4Table& tab, hipStream_t s) {
  if (count < 1 || count > kGemvMaxGroup || m < 1 || m > kSkinnyMaxM) return hipErrorInvalidValue;
  SkinnySet set{};
  set.count = count;
  int64_t wgs = 0, ncol = 0, off = 0;
  bool reduce = false;
  for (int i = 0; i < count; ++i) {
    set.w[i] = ws[i];
    set.y[i] = ys[i];
    set.ldy[i] = ldys[i];
    set.out_rows[i] = out_rows[i];
    const int ks = skinny_splits(ws[i].n, ws[i].k, m);
    set.ks[i] = ks;
    wgs += (ws[i].n + ROWS - 1) / ROWS * ks;
    set.wg_end[i] = (int)wgs;
    ncol += ws[i].n;
    set.col_end[i] = ncol;
    set.part_off[i] = off;  // weight i's partials: [ks][m][n_i], when ks > 1
    if (ks > 1) {
      off += (int64_t)ks * m * ws[i].n;
      reduce = true;
    }
  }
  return dispatch_kind<SkinnySetLauncher>(kind, set, wgs, ncol, reduce, X, m, part, tab, s);
}

hipError_t launch_skinny(WKind kind, const WView& w, const uint16_t* X, int64_t m, uint16_t* Y,
                         int64_t ldy, const int32_t* out_rows, float* part, const LoraEpi& lora,
                         const Nf4Table& tab, hipStream_t s) {
  if (m < 1 || m > kSkinnyMaxM) return hipErrorInvalidValue;
  const int ks = skinny_splits(w.n, w.k, m);
  return dispatch_kind<SkinnyLauncher>(kind, w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
}

}  // namespace lbq
