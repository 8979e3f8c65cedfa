// Quantize / pack and standalone dequantize kernels for gfx950.
//
// Bit-exactness: every fp32 step below is one IEEE binary32 operation rounded
// to nearest-even.  Contraction into FMA is switched off for this file (here
// and with -ffp-contract=off on its compile line), division is the correctly
// rounded v_div_scale/fmas/fixup sequence, and rne() is v_rndne_f32.
//
// Sources:
//   MinMax: GreenBit.AI, "只需单卡RTX 3090，低比特量化训练就能实现LLaMA-3 8B全参微调",
//           section 模型量化 -- group-wise MinMax, INT4 g128 / INT2 g64, RTN.
//   NF4 + double quantization: "QLoRA技术在量化微调中的应用", section
//           QLoRA技术原理 -- NF4 for normal weights; the absmax constants are
//           quantized a second time.
//   Packing: bitsandbytes FSDP-QLoRA guide, section 量化数据的存储 -- two codes
//           per byte, the even-indexed code in the high nibble.
#pragma clang fp contract(off)

#include "lbq_device.h"

#include <cmath>

namespace lbq {

namespace {

constexpr int kThreads = 256;

// 8 consecutive fp32 weights, read once: non-temporal loads (they stream past
// the caches, as the packed output does on the way out).
__device__ __forceinline__ void load8(const float* __restrict__ p, float w[8]) {
  const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + 1);
  w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
}

// ---------------------------------------------------------------------------
// MinMax.  One lane owns a chunk of 8 consecutive weights; the G/8 lanes of a
// group are adjacent in the wave and combine their min/max with xor shuffles.
// Chunks never straddle groups or rows (k % G == 0, G % 8 == 0).
// ---------------------------------------------------------------------------
// Compact metadata stores the scale as the smallest fp16 value >= s (round
// toward +inf, so Qmax * s still covers the group's range) and derives z and
// the codes from that stored value.  fp16 bits of that value for 0 < s,
// saturating at 65504; integer arithmetic only, normal and subnormal results.
__device__ __forceinline__ uint32_t f32_to_f16_up(float s) {
  if (s >= 65504.f) return 0x7BFFu;
  const uint32_t u = __float_as_uint(s);
  const int e = (int)(u >> 23);          // biased exponent (s > 0)
  const uint32_t mant = u & 0x7FFFFFu;
  if (e >= 113) {                        // s >= 2^-14: an fp16 normal
    uint32_t h = ((uint32_t)(e - 112) << 10) | (mant >> 13);
    if (mant & 0x1FFFu) h += 1;          // a carry moves into the exponent
    return h;
  }
  // fp16 subnormal: ceil(s / 2^-24) units of 2^-24
  const uint32_t M = e > 0 ? (mant | 0x800000u) : mant;
  const int shift = 126 - (e > 0 ? e : 1);  // s / 2^-24 = M / 2^shift, shift >= 14
  if (shift >= 32) return 1u;
  return (M >> shift) + ((M & ((1u << shift) - 1u)) ? 1u : 0u);
}

template <int BITS, int G, bool COMPACT>
__global__ __launch_bounds__(kThreads) void k_quant_minmax(const float* __restrict__ W,
                                                          uint8_t* __restrict__ packed,
                                                          float* __restrict__ scales,
                                                          uint8_t* __restrict__ zeros,
                                                          int64_t nchunks) {
  constexpr int QMAX = (1 << BITS) - 1;
  constexpr int LPG = G / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  // Whole waves iterate together so the shuffles below see converged waves.
  const int64_t bound = (nchunks + 63) & ~int64_t(63);
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < bound; c += stride) {
    const bool valid = c < nchunks;
    float w[8];
    if (valid) {
      load8(W + 8 * c, w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 0.f;
    }
    float mn = w[0], mx = w[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = fminf(mn, w[i]);
      mx = fmaxf(mx, w[i]);
    }
#pragma unroll
    for (int o = 1; o < LPG; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const float lo = fminf(0.f, mn);
    const float hi = fmaxf(0.f, mx);
    float s = (hi - lo) / (float)QMAX;
    if (s == 0.f) s = 1.f;
    uint32_t s16 = 0;
    if constexpr (COMPACT) {
      s16 = f32_to_f16_up(s);
      s = f16_bits_to_f32(s16);
    }
    int z = (int)__builtin_rintf(-lo / s);
    z = z < 0 ? 0 : (z > QMAX ? QMAX : z);
    // Compact zero points share a byte: 2 (4-bit) or 4 (2-bit) consecutive
    // groups, whose lanes lie in the same wave (a byte's groups never
    // straddle a row, and waves start at multiples of 64 chunks).
    uint32_t zbyte = 0;
    if constexpr (COMPACT && BITS == 4) {
      zbyte = ((uint32_t)z << 4) | (uint32_t)__shfl_xor(z, LPG);
    } else if constexpr (COMPACT) {
      zbyte = ((uint32_t)z << 6) | ((uint32_t)__shfl_xor(z, LPG) << 4) | ((uint32_t)__shfl_xor(z, 2 * LPG) << 2) |
              (uint32_t)__shfl_xor(z, 3 * LPG);
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int q = (int)__builtin_rintf(w[i] / s) + z;
      q = q < 0 ? 0 : (q > QMAX ? QMAX : q);
      if constexpr (BITS == 4) {
        word |= (uint32_t)q << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
      } else {
        word |= (uint32_t)q << (8 * (i >> 2) + 6 - 2 * (i & 3));
      }
    }
    if (valid) {
      if constexpr (BITS == 4) {
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(packed) + c);
      } else {
        __builtin_nontemporal_store((uint16_t)word, reinterpret_cast<uint16_t*>(packed) + c);
      }
      if ((c % LPG) == 0) {
        if constexpr (COMPACT) {
          reinterpret_cast<uint16_t*>(scales)[c / LPG] = (uint16_t)s16;
          if ((c % (LPG * 8 / BITS)) == 0) zeros[(c / LPG) * BITS / 8] = (uint8_t)zbyte;
        } else {
          scales[c / LPG] = s;
          zeros[c / LPG] = (uint8_t)z;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NF4.  A workgroup owns a run of 256 consecutive 64-blocks (16384 weights),
// which is exactly one double-quantization block: the 256 absmax values stay
// in LDS and the second-level int8 codes are produced in the same launch.
// Eight lanes share a 64-block (8 weights each); a workgroup of NT threads
// walks its run in 2048 / NT passes.  More threads per run give each CU more
// waves to hide the load, divide and table latencies behind; the launcher
// picks NT from the number of runs.
// ---------------------------------------------------------------------------
// Code of x = w / absmax (|x| <= 1): the number of midpoints strictly below
// x.  BUCKET: [-1, 1] cut into 64 equal buckets, each holding at most one
// midpoint, none within 1/1000 of a bucket width of an edge (the launcher
// checks the table); bucket b stores the midpoints below its lower edge and
// the one inside it, so a code is one LDS read and one compare.  The bucket
// coordinate (x + 1) * 32 is within 4e-6 of a bucket width of exact, so the
// bucket never changes the answer.  Otherwise a 4-probe binary search.
constexpr int kNf4Buckets = 64;

// Sum of the 256 values of `v` (LDS) over the binary tree of adjacent pairs:
// each level adds entries 2i and 2i+1.  Every thread of the workgroup calls it;
// the result is returned in every thread and v is overwritten.
__device__ __forceinline__ float lds_tree_sum256(float* v) {
  const int t = threadIdx.x;
  for (int width = 128; width >= 1; width >>= 1) {
    float x = 0.f;
    if (t < width) x = v[2 * t] + v[2 * t + 1];
    __syncthreads();
    if (t < width) v[t] = x;
    __syncthreads();
  }
  const float r = v[0];
  __syncthreads();
  return r;
}

// MODE 0: codes + fp32 absmax; 1: codes + double quantization of each run's
// 256 absmax; 2: codes + the adjacent-pair tree sum of each run's absmax into
// absmax_scale[run] (first pass of double quantization with an offset).
template <int MODE, bool BUCKET, int NT>
__global__ __launch_bounds__(NT) void k_quant_nf4(const float* __restrict__ W,
                                                       uint8_t* __restrict__ packed,
                                                       float* __restrict__ absmax,
                                                       int8_t* __restrict__ absmax_q,
                                                       float* __restrict__ absmax_scale,
                                                       int64_t nblocks, Nf4Table tab) {
  __shared__ float mids[16];
  __shared__ float2 bk[kNf4Buckets];  // (midpoint inside or +inf, midpoints below as int bits)
  __shared__ float am[256];
  __shared__ float red[NT / 64];
  const int t = threadIdx.x;
  if (t < 15) mids[t] = (tab.c[t] + tab.c[t + 1]) * 0.5f;
  __syncthreads();
  if (BUCKET && t < kNf4Buckets) {
    const float lo = -1.f + (float)t * (2.f / kNf4Buckets), hi = lo + 2.f / kNf4Buckets;
    int below = 0;
    float inside = __builtin_huge_valf();
    for (int j = 0; j < 15; ++j) {
      if (mids[j] < lo) ++below;
      else if (mids[j] < hi) inside = mids[j];
    }
    bk[t] = make_float2(inside, __int_as_float(below));
  }
  if (BUCKET) __syncthreads();

  const int64_t b0 = (int64_t)blockIdx.x * 256;
  const int nb_here = (int)((nblocks - b0) < 256 ? (nblocks - b0) : 256);

#pragma unroll
  for (int it = 0; it < 2048 / NT; ++it) {  // all loads of a lane in flight together
    const int lb = it * (NT / 8) + (t >> 3);
    const bool valid = lb < nb_here;
    const int64_t c = (b0 + lb) * 8 + (t & 7);
    float w[8];
    if (valid) {
      load8(W + 8 * c, w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 0.f;
    }
    float a = fabsf(w[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) a = fmaxf(a, fabsf(w[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int code = 7;
      if (a != 0.f) {
        const float x = w[i] / a;
        if constexpr (BUCKET) {
          // NaN lands in bucket 0 and compares false: code 0, as in the search
          const float u = fminf(fmaxf((x + 1.f) * (kNf4Buckets / 2), 0.f), (float)(kNf4Buckets - 1));
          const float2 e = bk[(int)u];
          code = __float_as_int(e.y) + (x > e.x ? 1 : 0);
        } else {
          // number of midpoints strictly below x (binary search, 4 probes)
          code = (x > mids[7]) ? 8 : 0;
          code += (x > mids[code + 3]) ? 4 : 0;
          code += (x > mids[code + 1]) ? 2 : 0;
          code += (x > mids[code]) ? 1 : 0;
        }
      }
      word |= (uint32_t)code << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
    }
    if (valid) {
      __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(packed) + c);
      if ((t & 7) == 0) {
        if constexpr (MODE != 0) {
          am[lb] = a;
        } else {
          absmax[b0 + lb] = a;
        }
      }
    } else if (MODE == 2 && (t & 7) == 0) {
      am[lb] = 0.f;  // zero padding of a partial run
    }
  }

  if constexpr (MODE == 2) {
    __syncthreads();
    const float sum = lds_tree_sum256(am);
    if (t == 0) absmax_scale[blockIdx.x] = sum;
  }
  if constexpr (MODE == 1) {
    __syncthreads();
    const float v = t < nb_here ? am[t] : 0.f;  // absmax >= 0: 0 is neutral
    float m = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i]);
    const float c2 = m / 127.f;
    if (t < nb_here) {
      int q2 = 0;
      if (c2 != 0.f) {
        q2 = (int)__builtin_rintf(v / c2);
        q2 = q2 < 0 ? 0 : (q2 > 127 ? 127 : q2);
      }
      absmax_q[b0 + t] = (int8_t)q2;
    }
    if (t == 0) absmax_scale[blockIdx.x] = c2;
  }
}

// ---------------------------------------------------------------------------
// Double quantization with an offset, passes 2 and 3.
// Pass 2 (one workgroup): the tree sum over the nr run sums (zero-padded to a
// power of two P) -- each thread folds an aligned run of P/256 leaves with a
// stack of complete subtrees, which adds exactly the adjacent pairs of the
// tree, then the 256 partial sums meet in LDS -- and the offset
// fp32(fp64(sum) / nb) into absmax_scale[nr].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_dqo_offset(float* __restrict__ absmax_scale, int64_t nr,
                                                         int64_t nb) {
  __shared__ float part[kThreads];
  const int t = threadIdx.x;
  int64_t P = 1;
  while (P < nr) P <<= 1;
  float r = 0.f;
  if (P <= kThreads) {
    r = t < nr ? absmax_scale[t] : 0.f;
  } else {
    const int64_t L = P / kThreads;  // leaves per thread, a power of two
    float stack[40];
    int top = 0;
    for (int64_t i = 0; i < L; ++i) {
      const int64_t idx = (int64_t)t * L + i;
      float v = idx < nr ? absmax_scale[idx] : 0.f;
      for (int64_t j = i; j & 1; j >>= 1) v = stack[--top] + v;  // close complete subtrees
      stack[top++] = v;
    }
    r = stack[0];
  }
  part[t] = r;
  __syncthreads();
  const float sum = lds_tree_sum256(part);
  if (t == 0) absmax_scale[nr] = (float)((double)sum / (double)nb);
}

// Pass 3: one workgroup per run of 256 blocks recomputes the blocks' absmax
// from W (as pass 1 does), subtracts the offset and writes the signed int8
// codes and the run's scale c2 = fl(max |a - off| / 127).
__global__ __launch_bounds__(kThreads) void k_dqo_codes(const float* __restrict__ W, int8_t* __restrict__ absmax_q,
                                                        float* __restrict__ absmax_scale, int64_t nblocks,
                                                        int64_t nr) {
  __shared__ float am[256];
  __shared__ float red[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * 256;
  const int nb_here = (int)((nblocks - b0) < 256 ? (nblocks - b0) : 256);
  const float off = absmax_scale[nr];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int lb = it * 32 + (t >> 3);
    const bool valid = lb < nb_here;
    const int64_t c = (b0 + lb) * 8 + (t & 7);
    float w[8];
    if (valid) {
      load8(W + 8 * c, w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 0.f;
    }
    float a = fabsf(w[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) a = fmaxf(a, fabsf(w[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    if (valid && (t & 7) == 0) am[lb] = a;
  }
  __syncthreads();
  const float d = t < nb_here ? am[t] - off : 0.f;
  float m = fabsf(d);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, red[i]);
  const float c2 = m / 127.f;
  if (t < nb_here) {
    int q2 = 0;
    if (c2 != 0.f) {
      q2 = (int)__builtin_rintf(d / c2);
      q2 = q2 < -127 ? -127 : (q2 > 127 ? 127 : q2);
    }
    absmax_q[b0 + t] = (int8_t)q2;
  }
  if (t == 0) absmax_scale[blockIdx.x] = c2;
}

// ---------------------------------------------------------------------------
// Dequantize to bf16: a lane handles chunks of 8 codes (one packed load, one
// 16-byte store), four chunks a grid stride apart per iteration so that four
// loads are in flight; every load and store instruction of a wave covers a
// contiguous run of memory.
// ---------------------------------------------------------------------------
template <int KIND>
__device__ __forceinline__ u32x4_t dequant8(const WView& w, int64_t c, const float* cb, float off) {
  using T = WKindTraits<KIND>;
  uint32_t word;
  if constexpr (T::bits == 4) {
    word = reinterpret_cast<const uint32_t*>(w.packed)[c];
  } else {
    word = reinterpret_cast<const uint16_t*>(w.packed)[c];
  }
  float v[8];
  if constexpr (T::fmt == FMT_MINMAX) {
    const int64_t g = c / (T::group / 8);
    const float s = minmax_scale<KIND>(w, g);
    const int z = minmax_zero<KIND>(w, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)(code_of<T::bits>(word, i) - z) * s;
  } else {
    const float a = nf4_block_scale<KIND>(w, c >> 3, off);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = cb[code_of<4>(word, i)] * a;
  }
  return u32x4_t{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]), cvt_pk_bf16(v[4], v[5]),
                 cvt_pk_bf16(v[6], v[7])};
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void k_dequant(WView w, uint16_t* __restrict__ out,
                                                     int64_t nchunks, Nf4Table tab) {
  using T = WKindTraits<KIND>;
  __shared__ float cb[16];
  if constexpr (T::fmt == FMT_NF4) {
    if (threadIdx.x < 16) cb[threadIdx.x] = tab.c[threadIdx.x];
    __syncthreads();
  }
  float off = 0.f;
  if constexpr (T::dqo) off = nf4_dq_offset(w);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; c + 3 * stride < nchunks; c += 4 * stride) {
    u32x4_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = dequant8<KIND>(w, c + p * stride, cb, off);
#pragma unroll
    for (int p = 0; p < 4; ++p) __builtin_nontemporal_store(o[p], dst + c + p * stride);
  }
  for (; c < nchunks; c += stride) dst[c] = dequant8<KIND>(w, c, cb, off);
}

int grid_for(int64_t nchunks) {
  int64_t g = (nchunks + kThreads - 1) / kThreads;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  return (int)g;
}

template <int KIND>
struct DequantLauncher {
  static hipError_t run(const WView& w, uint16_t* out, const Nf4Table& tab, hipStream_t s) {
    const int64_t nchunks = w.n * w.k / 8;
    hipLaunchKernelGGL((k_dequant<KIND>), dim3(grid_for((nchunks + 3) / 4)), dim3(kThreads), 0, s, w, out,
                       nchunks, tab);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_quant_minmax(int bits, int group, bool compact, const float* W, uint8_t* packed,
                               float* scales, uint8_t* zeros, int64_t n, int64_t k,
                               hipStream_t s) {
  const int64_t nchunks = n * k / 8;
  // whole waves per grid stride (the compact zero bytes combine lanes)
  const dim3 grid(grid_for(nchunks)), block(kThreads);
  if (bits == 4 && group == 128 && compact) {
    hipLaunchKernelGGL((k_quant_minmax<4, 128, true>), grid, block, 0, s, W, packed, scales, zeros, nchunks);
  } else if (bits == 2 && group == 64 && compact) {
    hipLaunchKernelGGL((k_quant_minmax<2, 64, true>), grid, block, 0, s, W, packed, scales, zeros, nchunks);
  } else if (compact) {
    return hipErrorInvalidValue;
  } else if (bits == 4 && group == 128) {
    hipLaunchKernelGGL((k_quant_minmax<4, 128, false>), grid, block, 0, s, W, packed, scales, zeros, nchunks);
  } else if (bits == 4 && group == 64) {
    hipLaunchKernelGGL((k_quant_minmax<4, 64, false>), grid, block, 0, s, W, packed, scales, zeros, nchunks);
  } else if (bits == 2 && group == 64) {
    hipLaunchKernelGGL((k_quant_minmax<2, 64, false>), grid, block, 0, s, W, packed, scales, zeros, nchunks);
  } else if (bits == 2 && group == 128) {
    hipLaunchKernelGGL((k_quant_minmax<2, 128, false>), grid, block, 0, s, W, packed, scales, zeros, nchunks);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_nf4(int dq, const float* W, uint8_t* packed, float* absmax,
                            int8_t* absmax_q, float* absmax_scale, int64_t n, int64_t k,
                            const Nf4Table& tab, hipStream_t s) {
  const int64_t nblocks = n * k / 64;
  const int64_t runs = (nblocks + 255) / 256;
  const dim3 grid((unsigned)runs), block(kThreads);
  // Up to one run per CU: 1024 threads a run, else 512 (measured on the 8B
  // shapes: 1024-row weights, 256 runs, 14.5 -> 8.2 us with 1024 threads;
  // 1024 and 3584 runs 3-4% faster with 512 threads than with 256, 5-9%
  // slower with 1024).
  const bool wide = runs <= 256;
  // The bucket lookup needs at most one midpoint per bucket, each clear of
  // the bucket edges (midpoints formed in fp32 as the kernel forms them).
  bool bucket = true;
  int per[kNf4Buckets] = {};
  for (int j = 0; j < 15 && bucket; ++j) {
    const float mid = (tab.c[j] + tab.c[j + 1]) * 0.5f;
    const double u = ((double)mid + 1.0) * (kNf4Buckets / 2);
    const double f = u - std::floor(u);
    if (!(u > 0.0 && u < kNf4Buckets) || f < 1e-3 || f > 1.0 - 1e-3 || ++per[(int)u] > 1) bucket = false;
  }
#define LBQ_NF4_LAUNCH_NT(MODE, NT)                                                              \
  do {                                                                                           \
    if (bucket)                                                                                  \
      hipLaunchKernelGGL((k_quant_nf4<MODE, true, NT>), grid, dim3(NT), 0, s, W, packed, absmax,  \
                         absmax_q, absmax_scale, nblocks, tab);                                 \
    else                                                                                         \
      hipLaunchKernelGGL((k_quant_nf4<MODE, false, NT>), grid, dim3(NT), 0, s, W, packed, absmax, \
                         absmax_q, absmax_scale, nblocks, tab);                                 \
  } while (0)
#define LBQ_NF4_LAUNCH(MODE)         \
  do {                               \
    if (wide)                        \
      LBQ_NF4_LAUNCH_NT(MODE, 1024); \
    else                             \
      LBQ_NF4_LAUNCH_NT(MODE, 512);  \
  } while (0)
  if (dq == 0) {
    LBQ_NF4_LAUNCH(0);
  } else if (dq == 1) {
    LBQ_NF4_LAUNCH(1);
  } else {
    // with an offset: codes and run sums, the offset, then the int8 codes
    LBQ_NF4_LAUNCH(2);
    const int64_t nr = (nblocks + 255) / 256;
    hipLaunchKernelGGL(k_dqo_offset, dim3(1), block, 0, s, absmax_scale, nr, nblocks);
    hipLaunchKernelGGL(k_dqo_codes, grid, block, 0, s, W, absmax_q, absmax_scale, nblocks, nr);
  }
#undef LBQ_NF4_LAUNCH
#undef LBQ_NF4_LAUNCH_NT
  return hipGetLastError();
}

hipError_t launch_dequant(WKind kind, const WView& w, uint16_t* out, const Nf4Table& tab,
                          hipStream_t s) {
  return dispatch_kind<DequantLauncher>(kind, w, out, tab, s);
}

}  // namespace lbq
