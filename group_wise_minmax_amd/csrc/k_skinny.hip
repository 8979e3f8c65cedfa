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

// Codes per chunk of the MB x 16-row tiles: 256, or 128 for MB = 4, whose x
// tile would otherwise leave room for one workgroup per CU (90 KB of LDS;
// with 128-code chunks, 49 KB: three).  K splits are still counted in
// 256-code chunks.
template <int MB>
constexpr int kct_of() { return MB == 4 ? 128 : KC; }

template <int KIND, int KCT = KC>
struct SkTraits {
  using T = WKindTraits<KIND>;
  static constexpr int RB = KCT * T::bits / 8;  // packed bytes per row per chunk (128 / 64 at KCT = 256)
  static constexpr int RBP = RB + 16;           // padded LDS row: conflict-free A reads
  static constexpr int GRP = T::fmt == FMT_MINMAX ? T::group : 64;
};

// A fragment (8 codes -> 4 dwords of bf16 pairs) for k-step t of row `row`
// and lane group lg from a staged chunk.  Its k-slot order matches the order
// in which x is stored (arrange8()).
template <int KIND, int KCT>
__device__ __forceinline__ u32x4_t a_frag(const uint8_t* wl, int row, int lg, int t,
                                          const uint32_t* lut, int lane32) {
  using T = WKindTraits<KIND>;
  using S = SkTraits<KIND, KCT>;
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

// LDS of one workgroup, declared by the kernel and sized for the weight kinds
// its tiles may take: packed rows of pitch RBP_, NG_ metadata slots per row
// and chunk (one per 64 codes; groups of 128 use the first half), the NF4
// table (LUT entries) when a kind needs it.
template <int RBP_, int NG_, int MB, int LUT>
struct SkLds {
  uint8_t Ws[2][ROWS * RBP_];
  uint16_t Xs[2][MB * 16 * (kct_of<MB>() + 8)];
  float2 meta[2][ROWS][NG_];  // (scale, 128 + zero) or (absmax, 0)
  uint32_t lut[LUT];
  float cbs[16];
};
template <int KIND, int MB>
using SkLdsOf = SkLds<SkTraits<KIND, kct_of<MB>()>::RBP, KC / 64, MB,
                      WKindTraits<KIND>::fmt == FMT_NF4 ? 256 * kLutCopies : 1>;
// A workgroup of the INT4 g128 / INT2 g64 mix holds either kind's tile.
template <int MB>
using SkLdsMix = SkLds<SkTraits<WK_I4G128, kct_of<MB>()>::RBP, KC / 64, MB, 1>;

// Row tile `tile` (ROWS rows of W) over K range `split` of ks_count; with
// `part` set, the fp32 sums go to part[split][m][n], else bf16 to Y.
template <int KIND, int MB, typename LDS>
__device__ __forceinline__ void skinny_tile(const WView& w, const uint16_t* __restrict__ X, int m,
                                            uint16_t* __restrict__ Y, int64_t ldy,
                                            const int32_t* __restrict__ out_rows,
                                            float* __restrict__ part, int ks_count,
                                            const LoraEpi& lora, const Nf4Table& tab, int tile, int split,
                                            LDS& lds) {
  using T = WKindTraits<KIND>;
  constexpr int KCT = kct_of<MB>();     // codes per chunk
  using S = SkTraits<KIND, KCT>;
  constexpr int RB = S::RB, RBP = S::RBP, GRP = S::GRP;
  constexpr int NG = KCT / GRP;         // groups (blocks) per chunk
  constexpr int LDX = KCT + 8;          // padded x row (bf16)
  constexpr int WCOL = RB / 16;         // 16-byte W columns per row
  constexpr int WLDN = ROWS * WCOL;     // 16-byte W loads per chunk
  constexpr int WLD = (WLDN + kThreads - 1) / kThreads;  // per thread (the last partly idle)
  constexpr int XLD = MB * 16 * (KCT / 8) / kThreads;    // X loads per thread per chunk
  constexpr int KSW = KCT / 128;        // k-steps of 32 codes per wave and chunk
  static_assert(sizeof(lds.Ws[0]) >= ROWS * RBP && sizeof(lds.Xs[0]) == MB * 16 * LDX * 2, "tile LDS");
  static_assert(sizeof(lds.meta[0][0]) == 4 * sizeof(float2) && NG <= 4 && kThreads == 4 * ROWS, "tile LDS");
  static_assert(T::fmt != FMT_NF4 || sizeof(lds.lut) >= 256 * kLutCopies * 4, "tile LDS");
  auto& Ws = lds.Ws;
  auto& Xs = lds.Xs;
  auto& meta = lds.meta;
  uint32_t* const lut = lds.lut;
  float* const cbs = lds.cbs;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t n0 = (int64_t)tile * ROWS;
  const int64_t K = w.k;
  const int64_t KB = K * T::bits / 8;
  const int64_t gpr = K / GRP;
  // The split's range of 256-code chunks, then in chunks of KCT codes.
  const int nchunk = (int)((K + KC - 1) / KC);
  const int per = (nchunk + ks_count - 1) / ks_count;
  const int c_lo = split * per * (KC / KCT);
  const int c_hi = (int)min((int64_t)min(split * per + per, nchunk) * (KC / KCT), (K + KCT - 1) / KCT);
  float dqoff = 0.f;  // offset of double quantization with an offset
  if constexpr (T::dqo) dqoff = nf4_dq_offset(w);

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
  // Buffer loads with 32-bit lane offsets: the boundary keeps the packed
  // weight and X below 2^32 bytes.
  const __amdgpu_buffer_rsrc_t r_w = make_rsrc(w.packed, w.n * KB);
  const __amdgpu_buffer_rsrc_t r_x = make_rsrc(X, (int64_t)m * K * 2);
  __amdgpu_buffer_rsrc_t r_s, r_z;
  meta_rsrc<KIND>(w, w.n * gpr, r_s, r_z);
  u32x4_t wr[WLD], xr[XLD];
  MetaRaw mraw;      // this thread's metadata entry of the loaded chunk, as loaded
  int64_t mgi = 0;   // its entry index
  // Loop-invariant parts of this thread's load offsets (32-bit: the
  // boundary keeps the packed weight and X below 2^32 bytes): the clamped
  // packed row, x row and metadata row of each load.
  uint32_t wrow[WLD], xrow[XLD];
#pragma unroll
  for (int i = 0; i < WLD; ++i)
    wrow[i] = (uint32_t)min(n0 + min(tid + kThreads * i, WLDN - 1) / WCOL, w.n - 1) * (uint32_t)KB;
#pragma unroll
  for (int i = 0; i < XLD; ++i)
    xrow[i] = 2u * (uint32_t)min((tid + kThreads * i) / (KCT / 8), m - 1) * (uint32_t)K;
  const uint32_t mrow = (uint32_t)min(n0 + tid / 4, w.n - 1) * (uint32_t)gpr;
  auto load = [&](int c) {
    const uint32_t kc = (uint32_t)c * (uint32_t)KCT;
    const int kend = (int)min(K - (int64_t)kc, (int64_t)KCT);  // codes in this chunk (multiple of 64)
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int col = (tid + kThreads * i) % WCOL;
      // Past the chunk's end (a last, partial chunk) the load reads the
      // chunk's first bytes instead; the waves whose codes start at or past
      // kend skip the chunk, so those LDS bytes are never used.  (Zeroing
      // them here would make the wave wait for the load at once.)
      const uint32_t off = wrow[i] + kc * T::bits / 8 + (col * 16 * 8 / T::bits < kend ? col * 16u : 0u);
      wr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_w, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
      const int col = (tid + kThreads * i) % (KCT / 8);
      const uint32_t xo = xrow[i] + 2u * (kc + (col * 8 < kend ? col * 8u : 0u));  // as above
      xr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_x, xo, 0, 0));
    }
    {
      const int j = tid % 4;
      const bool ok = j < NG && j * GRP < kend;
      mgi = (int64_t)(mrow + (ok ? kc / GRP + j : 0u));
      mraw = load_meta_buf<KIND>(r_s, r_z, (uint32_t)mgi);  // decoded in store(), one chunk later
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int e = tid + kThreads * i;
      if (WLDN % kThreads == 0 || e < WLDN)  // (2-bit 128-code chunks: half the threads)
        *reinterpret_cast<u32x4_t*>(&Ws[b][(e / WCOL) * RBP + (e % WCOL) * 16]) = wr[i];
    }
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
      const int e = tid + kThreads * i;
      *reinterpret_cast<u32x4_t*>(&Xs[b][(e / (KCT / 8)) * LDX + (e % (KCT / 8)) * 8]) = arrange8<KIND>(xr[i]);
    }
    if (tid % 4 < NG) {
      const float sc = meta_raw_scale<KIND>(mraw, dqoff);
      meta[b][tid / 4][tid % 4] =
          make_float2(sc, T::fmt == FMT_MINMAX ? (float)(128 + meta_raw_zero<KIND>(mraw, mgi)) : 0.f);
    }
  };

  // Wave w takes k-steps KSW w .. KSW w + KSW - 1 of every chunk (codes
  // [KCT w / 4, KCT (w + 1) / 4)) for all ROWS rows: each x fragment it reads
  // feeds the 4 row tiles, and the sum of x (MinMax) is formed once for them.
  // The waves' sums are added in wave order at the end.
  f32x4_t acc[4][MB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < MB; ++q) acc[j][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t ones = u32x4_t{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
  const int lane32 = lane & 31;
  const int t0 = KSW * wave;               // this wave's first k-step in a chunk
  const int gw = (KCT / 4) * wave / GRP;   // the group (block) its codes belong to

  auto compute = [&](int b, int c) {
    const int64_t kc = (int64_t)c * KCT;
    const int64_t kend = (K - kc) < KCT ? (K - kc) : KCT;  // a multiple of 64
    if ((int64_t)(KCT / 4) * wave >= kend) return;
    const uint8_t* wl = Ws[b];
    f32x4_t ag[4][MB], xs[MB];
#pragma unroll
    for (int q = 0; q < MB; ++q) {
      xs[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) ag[j][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tt = 0; tt < KSW; ++tt) {
      const int t = t0 + tt;
      u32x4_t xf[MB];
#pragma unroll
      for (int q = 0; q < MB; ++q) {
        xf[q] = *reinterpret_cast<const u32x4_t*>(&Xs[b][(16 * q + li) * LDX + x_off<KIND>(lg, t)]);
        if constexpr (T::fmt == FMT_MINMAX) xs[q] = mfma16x16x32(ones, xf[q], xs[q]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t af = a_frag<KIND, KCT>(wl, 16 * j + li, lg, t, lut, lane32);
#pragma unroll
        for (int q = 0; q < MB; ++q) ag[j][q] = mfma16x16x32(af, xf[q], ag[j][q]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 md = meta[b][16 * j + 4 * lg + i][gw];
#pragma unroll
        for (int q = 0; q < MB; ++q) {
          if constexpr (T::fmt == FMT_MINMAX) {
            acc[j][q][i] = fmaf(md.x, fmaf(-md.y, xs[q][i], ag[j][q][i]), acc[j][q][i]);
          } else {
            acc[j][q][i] = fmaf(md.x, ag[j][q][i], acc[j][q][i]);
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

  // Sum of the four waves' accumulators through LDS (the x buffers are free
  // after the last barrier): red[w][j][q][i][lane] for RQ of the MB column
  // tiles at a time (all of them unless the x buffers are too small); wave w
  // then adds row tile j = w's values in wave order.
  constexpr int RQ1 = (int)(sizeof(lds.Xs) / (4 * 4 * 4 * 64 * sizeof(float)));
  constexpr int RQ = RQ1 < MB ? RQ1 : MB;
  static_assert(RQ >= 1 && MB % RQ == 0, "reduction LDS");
  float* const red = reinterpret_cast<float*>(&Xs[0][0]);
  f32x4_t sum[MB];
#pragma unroll
  for (int q0 = 0; q0 < MB; q0 += RQ) {
    if (q0 > 0) __syncthreads();  // the previous part has been read
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < RQ; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(((wave * 4 + j) * RQ + q) * 4 + i) * 64 + lane] = acc[j][q0 + q][i];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = red[(((0 * 4 + wave) * RQ + q) * 4 + i) * 64 + lane];
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) v += red[(((w2 * 4 + wave) * RQ + q) * 4 + i) * 64 + lane];
        sum[q0 + q][i] = v;
      }
  }

  // lane holds D[n = n0 + 16 wave + 4lg + i][m = 16q + li]
  const int trow = 16 * wave;
#pragma unroll
  for (int q = 0; q < MB; ++q) {
    const int mrow = 16 * q + li;
    if (mrow >= m) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + trow + 4 * lg + i;
      if (n >= w.n) continue;
      if (part != nullptr) {
        part[((int64_t)split * m + mrow) * w.n + n] = sum[q][i];
      } else {
        Y[(int64_t)mrow * ldy + (out_rows ? (int64_t)out_rows[n] : n)] = (uint16_t)bf16_rne(sum[q][i]);
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
  __shared__ __attribute__((aligned(16))) SkLdsOf<KIND, MB> lds;
  skinny_tile<KIND, MB>(w, X, m, Y, ldy, out_rows, part, ks_count, lora, tab, blockIdx.x, blockIdx.y, lds);
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
  __shared__ __attribute__((aligned(16))) SkLdsOf<KIND, MB> lds;
  skinny_tile<KIND, MB>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi],
                        ks == 1 ? nullptr : part + set.part_off[pi], ks, none, tab, r % tiles, r / tiles, lds);
}

// The INT4 g128 and INT2 g64 row sets of channel-mixed linears that share X
// in one launch: set entries [0, first_b) are INT4 g128, the rest INT2 g64.
// A workgroup's tile belongs to one weight and runs that weight's format;
// each weight keeps the K split it has alone, so the outputs equal those of
// the per-format launches bit for bit.
template <int MB>
__global__ __launch_bounds__(kThreads) void k_skinny_mix(SkinnySet set, const uint16_t* __restrict__ X, int m,
                                                        float* __restrict__ part, Nf4Table tab, int first_b) {
  const int b = blockIdx.x;
  int pi = 0, wbeg = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count && b >= set.wg_end[i - 1]) { pi = i; wbeg = set.wg_end[i - 1]; }
  const int ks = set.ks[pi];
  const int tiles = (int)((set.w[pi].n + ROWS - 1) / ROWS);
  const int r = b - wbeg;
  const LoraEpi none{nullptr, nullptr, 0, 0};
  float* const p = ks == 1 ? nullptr : part + set.part_off[pi];
  __shared__ __attribute__((aligned(16))) SkLdsMix<MB> lds;
  if (pi < first_b)
    skinny_tile<WK_I4G128, MB>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi], p, ks, none, tab,
                               r % tiles, r / tiles, lds);
  else
    skinny_tile<WK_I2G64, MB>(set.w[pi], X, m, set.y[pi], set.ldy[pi], set.out_rows[pi], p, ks, none, tab,
                              r % tiles, r / tiles, lds);
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
    if (m <= 48) return launch_set_mb<KIND, 3>(set, wgs, ncol, reduce, X, m, part, tab, s);
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
    if (m <= 48) return launch_mb<KIND, 3>(w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
    return launch_mb<KIND, 4>(w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
  }
};

// The set's per-weight tiles, K splits and partial-sum areas.
void plan_skinny_set(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* out_rows,
                     int count, int64_t m, SkinnySet& set, int64_t& wgs, int64_t& ncol, bool& reduce) {
  set = SkinnySet{};
  set.count = count;
  wgs = 0;
  ncol = 0;
  int64_t off = 0;
  reduce = false;
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
}

template <int MB>
hipError_t launch_mix_mb(const SkinnySet& set, int64_t wgs, int64_t ncol, bool reduce, const uint16_t* X, int64_t m,
                         float* part, const Nf4Table& tab, int first_b, hipStream_t s) {
  hipLaunchKernelGGL((k_skinny_mix<MB>), dim3((unsigned)wgs), dim3(kThreads), 0, s, set, X, (int)m, part, tab,
                     first_b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !reduce) return e;
  hipLaunchKernelGGL(k_skinny_reduce_set, dim3((unsigned)((ncol + 255) / 256), (unsigned)m), dim3(256), 0, s,
                     part, (int)m, set);
  return hipGetLastError();
}

}  // namespace

int skinny_splits(int64_t n, int64_t k, int64_t m) {
  return skinny_splits_tiles((n + ROWS - 1) / ROWS, k, m);
}

// Workgroups of the small-batch kernel resident at once on the chip for m
// (LDS-limited; the INT4 g128 tile, which the other 4- and 2-bit kinds match
// or undercut).
template <int MB>
constexpr int64_t skinny_slots() {
  return 256 * ((160 * 1024) / (int64_t)sizeof(SkLdsOf<WK_I4G128, MB>) > 0
                    ? (160 * 1024) / (int64_t)sizeof(SkLdsOf<WK_I4G128, MB>) : 1);
}

namespace {
bool fills_unsplit(int64_t tiles, int64_t nchunk, int64_t m) {
  const int mb = m <= 16 ? 1 : m <= 32 ? 2 : m <= 48 ? 3 : 4;
  const int64_t slots = mb == 1 ? skinny_slots<1>() : mb == 2 ? skinny_slots<2>() : mb == 3 ? skinny_slots<3>()
                                                                                           : skinny_slots<4>();
  return tiles * 5 >= slots && nchunk <= 16 * mb;
}
}  // namespace

bool skinny_fills_unsplit(int64_t n, int64_t k, int64_t m) {
  return fills_unsplit((n + ROWS - 1) / ROWS, (k + KC - 1) / KC, m);
}

int skinny_splits_tiles(int64_t tiles, int64_t k, int64_t m) {
  const int64_t nchunk = (k + KC - 1) / KC;
  // A weight whose row tiles alone fill a fifth of the resident workgroups,
  // with at most 16 chunks per 16-column tile of m, runs unsplit: no partial
  // sums and no reduce launch.  (Such weights come in sets -- gate and up --
  // that fill the chip together.  Measured: 8B gate+up at m = 16 31.1 ->
  // 25.7 us and at m = 48 56.1 -> 41.5 us; the 70B channel-mix layer at
  // m = 40 +8%, gate+up at m = 64 75.0 -> 55.5 us.  Longer K ranges -- the
  // 70B INT2 gate/up rows at m = 3 and 16 -- lost 4-7% unsplit.)  Other
  // weights aim at ~512 workgroups,
  // with the fp32 partial traffic (ks * m * n * 8 bytes) kept below the
  // packed weight (n * k / 2 bytes for 4-bit).  Measured on the 8B layer:
  // more splits lose to the shorter K ranges, a tighter cap (a quarter of the
  // weight) costs 3% at m = 16 and 15% at m = 32.
  if (fills_unsplit(tiles, nchunk, m)) return 1;
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
  SkinnySet set;
  int64_t wgs, ncol;
  bool reduce;
  plan_skinny_set(ws, ys, ldys, out_rows, count, m, set, wgs, ncol, reduce);
  return dispatch_kind<SkinnySetLauncher>(kind, set, wgs, ncol, reduce, X, m, part, tab, s);
}

hipError_t launch_skinny_mix(const WView* ws, uint16_t* const* ys, const int64_t* ldys, const int32_t* const* out_rows,
                             int count_a, int count_b, const uint16_t* X, int64_t m, float* part, const Nf4Table& tab,
                             hipStream_t s) {
  const int count = count_a + count_b;
  if (count_a < 1 || count_b < 1 || count > kGemvMaxGroup || m < 1 || m > kSkinnyMaxM) return hipErrorInvalidValue;
  SkinnySet set;
  int64_t wgs, ncol;
  bool reduce;
  plan_skinny_set(ws, ys, ldys, out_rows, count, m, set, wgs, ncol, reduce);
  if (m <= 16) return launch_mix_mb<1>(set, wgs, ncol, reduce, X, m, part, tab, count_a, s);
  if (m <= 32) return launch_mix_mb<2>(set, wgs, ncol, reduce, X, m, part, tab, count_a, s);
  if (m <= 48) return launch_mix_mb<3>(set, wgs, ncol, reduce, X, m, part, tab, count_a, s);
  return launch_mix_mb<4>(set, wgs, ncol, reduce, X, m, part, tab, count_a, s);
}

hipError_t launch_skinny(WKind kind, const WView& w, const uint16_t* X, int64_t m, uint16_t* Y,
                         int64_t ldy, const int32_t* out_rows, float* part, const LoraEpi& lora,
                         const Nf4Table& tab, hipStream_t s) {
  if (m < 1 || m > kSkinnyMaxM) return hipErrorInvalidValue;
  const int ks = skinny_splits(w.n, w.k, m);
  return dispatch_kind<SkinnyLauncher>(kind, w, X, m, Y, ldy, out_rows, part, ks, lora, tab, s);
}

}  // namespace lbq
