// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lbq_internal.h"

namespace lbq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest, ties to even (NaN is out of contract).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> one dword of two bf16 with the hardware RNE conversion
// (v_cvt_pk_bf16_f32); lo in bits 15..0.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Two fp32 -> one dword of two bf16 (lo in bits 15..0), software RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// v_perm_b32: bytes of {hi:lo} selected by `sel` (0..3 -> lo, 4..7 -> hi).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// (lo16(a), lo16(b)) and (hi16(a), hi16(b)) as bf16 pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// D(16x16, f32) += A(16x32) * B(32x16), bf16 operands.  Lane l holds
// A[l%16][kslot(l/16, 0..7)], B[kslot(l/16, 0..7)][l%16] and
// D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Sum over the 64 lanes of a wave, result in every lane: four DPP steps
// (xor 1, xor 2 within quads, half-row and row mirrors) and two cross-row
// exchanges.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Barrier that orders LDS accesses only: global loads issued before it stay
// in flight (a full __syncthreads() would wait for them as well).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Integer code of element i (0..7) from the packed bytes of a chunk of 8
// consecutive codes: 4-bit chunks are one dword (4 bytes), 2-bit chunks a
// 16-bit word.  Even element -> high nibble (4-bit); first element -> bits
// 7..6 (2-bit).
template <int BITS>
__device__ __forceinline__ int code_of(uint32_t word, int i) {
  if constexpr (BITS == 4) {
    return (word >> (8 * (i >> 1) + ((i & 1) ? 0 : 4))) & 0xF;
  } else {
    return (word >> (8 * (i >> 2) + 6 - 2 * (i & 3))) & 0x3;
  }
}

// LDS tiles of 64 bf16 (128 bytes) per row store the eight 16-byte chunks of
// row r at position c ^ (r & 7).  Byte offset of logical chunk c of row r.
// Measured on gfx950 this keeps MFMA operand reads (16 rows x 4 chunk columns,
// ds_read_b128) and whole-row or 8-byte column writes free of bank conflicts.
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t c) { return r * 128u + 16u * (c ^ (r & 7u)); }

// Raw buffer resource over `bytes` bytes at p; loads at or past `bytes`
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

// Tile index of workgroup `bid` among nx * ny tiles, XCD-aware and grouped.
__device__ __forceinline__ void tile_of(int bid, int nx, int ny, int& tx, int& ty) {
  const int total = nx * ny;
  // hardware round-robins workgroups over 8 XCDs: give XCD j the contiguous
  // logical range [j*per, (j+1)*per) (the remainder goes to the first XCDs)
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int start = xcd * per + (xcd < rem ? xcd : rem);
  int t = start + slot;
  if (slot >= per + (xcd < rem ? 1 : 0)) t = bid;  // cannot happen for grid == total
  constexpr int GM = 4;  // X-row tiles per group (measured: 2 -> 4 +1.5% on the 8B layer at m = 4096)
  const int group = t / (GM * nx);
  const int first = group * GM;
  const int gm = (ny - first) < GM ? (ny - first) : GM;
  const int r = t - group * GM * nx;
  ty = first + r % gm;
  tx = r / gm;
}

// compact: fp16 scales and zero points packed `bits` wide, like the codes.
// dqo: double quantization with a per-tensor offset (absmax_scale holds the
// per-256 scales and then the offset).
template <int K> struct WKindTraits;
template <> struct WKindTraits<WK_I4G128>  { static constexpr int fmt = FMT_MINMAX, bits = 4, group = 128; static constexpr bool dq = false, compact = false, dqo = false; };
template <> struct WKindTraits<WK_I4G64>   { static constexpr int fmt = FMT_MINMAX, bits = 4, group = 64;  static constexpr bool dq = false, compact = false, dqo = false; };
template <> struct WKindTraits<WK_I2G64>   { static constexpr int fmt = FMT_MINMAX, bits = 2, group = 64;  static constexpr bool dq = false, compact = false, dqo = false; };
template <> struct WKindTraits<WK_I2G128>  { static constexpr int fmt = FMT_MINMAX, bits = 2, group = 128; static constexpr bool dq = false, compact = false, dqo = false; };
template <> struct WKindTraits<WK_NF4>     { static constexpr int fmt = FMT_NF4,    bits = 4, group = 64;  static constexpr bool dq = false, compact = false, dqo = false; };
template <> struct WKindTraits<WK_NF4DQ>   { static constexpr int fmt = FMT_NF4,    bits = 4, group = 64;  static constexpr bool dq = true,  compact = false, dqo = false; };
template <> struct WKindTraits<WK_I4G128C> { static constexpr int fmt = FMT_MINMAX, bits = 4, group = 128; static constexpr bool dq = false, compact = true,  dqo = false; };
template <> struct WKindTraits<WK_I2G64C>  { static constexpr int fmt = FMT_MINMAX, bits = 2, group = 64;  static constexpr bool dq = false, compact = true,  dqo = false; };
template <> struct WKindTraits<WK_NF4DQO>  { static constexpr int fmt = FMT_NF4,    bits = 4, group = 64;  static constexpr bool dq = true,  compact = false, dqo = true; };

// fp16 bit pattern -> its exact fp32 value (normal and subnormal; no NaN/Inf
// in the contract).  One v_cvt_f32_f16: every fp16 value, subnormals
// included, is a normal fp32 number, and fp16 denormals are kept by the
// default floating-point mode, so the conversion is exact.
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Zero point of metadata entry gi from the zeros array: one byte per entry,
// or (compact) `bits`-wide fields packed like the codes, the first entry in
// the high bits; rows hold whole bytes, so entry gi sits in byte gi*bits/8.
template <int KIND>
__device__ __forceinline__ int zero_from_byte(uint32_t byte, int64_t gi) {
  using T = WKindTraits<KIND>;
  if constexpr (!T::compact) {
    return (int)(byte & 0xFFu);
  } else if constexpr (T::bits == 4) {
    return (int)((byte >> ((gi & 1) ? 0 : 4)) & 0xFu);
  } else {
    return (int)((byte >> (6 - 2 * (int)(gi & 3))) & 0x3u);
  }
}
// Byte offset in the zeros array of metadata entry gi.
template <int KIND>
__device__ __forceinline__ int64_t zero_byte_index(int64_t gi) {
  using T = WKindTraits<KIND>;
  if constexpr (T::compact) return gi * T::bits / 8;
  return gi;
}
// Byte offset in the scales array of metadata entry gi (fp32 or fp16).
template <int KIND>
__device__ __forceinline__ int64_t scale_byte_index(int64_t gi) {
  return gi * (WKindTraits<KIND>::compact ? 2 : 4);
}
// Scale value from the raw bits loaded at scale_byte_index (fp32, or fp16 in
// the low 16 bits).
template <int KIND>
__device__ __forceinline__ float scale_from_bits(uint32_t raw) {
  if constexpr (WKindTraits<KIND>::compact) return f16_bits_to_f32(raw & 0xFFFFu);
  return __uint_as_float(raw);
}
// MinMax scale and zero point of metadata entry gi (generic loads).
template <int KIND>
__device__ __forceinline__ float minmax_scale(const WView& w, int64_t gi) {
  if constexpr (WKindTraits<KIND>::compact)
    return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(w.scales)[gi]);
  return w.scales[gi];
}
template <int KIND>
__device__ __forceinline__ int minmax_zero(const WView& w, int64_t gi) {
  return zero_from_byte<KIND>(w.zeros[zero_byte_index<KIND>(gi)], gi);
}

// The metadata words of entry gi as loaded: the scale word (MinMax fp32 or
// fp16 bits, NF4 absmax or second-level scale) and the zero-point byte (the
// int8 absmax code under double quantization).  No arithmetic touches the
// loaded values, so a prefetch is not waited for where it is issued; decode
// them where they are used (meta_raw_scale, meta_raw_zero).
struct MetaRaw {
  uint32_t s, z;
};
template <int KIND>
__device__ __forceinline__ MetaRaw load_meta_raw(const WView& w, int64_t gi) {
  using T = WKindTraits<KIND>;
  MetaRaw r{0u, 0u};
  if constexpr (T::fmt == FMT_MINMAX && T::compact) {
    r.s = reinterpret_cast<const uint16_t*>(w.scales)[gi];
    r.z = w.zeros[gi * T::bits / 8];
  } else if constexpr (T::fmt == FMT_MINMAX) {
    r.s = __float_as_uint(w.scales[gi]);
    r.z = w.zeros[gi];
  } else if constexpr (T::dq) {
    r.s = __float_as_uint(w.absmax_scale[gi >> 8]);
    r.z = (uint8_t)w.absmax_q[gi];
  } else {
    r.s = __float_as_uint(w.absmax[gi]);
  }
  return r;
}
// Buffer resources over a weight's metadata arrays (scales / zero points, or
// the NF4 absmax data).
template <int KIND>
__device__ __forceinline__ void meta_rsrc(const WView& w, int64_t nmeta, __amdgpu_buffer_rsrc_t& r_s,
                                          __amdgpu_buffer_rsrc_t& r_z) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_MINMAX) {
    r_s = make_rsrc(w.scales, scale_byte_index<KIND>(nmeta));
    r_z = make_rsrc(w.zeros, zero_byte_index<KIND>(nmeta));
  } else if constexpr (T::dq) {
    r_s = make_rsrc(w.absmax_scale, ((nmeta + 255) >> 8) * 4);
    r_z = make_rsrc(w.absmax_q, nmeta);
  } else {
    r_s = make_rsrc(w.absmax, nmeta * 4);
    r_z = r_s;
  }
}

// The metadata words of entry gi through the buffer resources of
// meta_rsrc, as loaded (a 32-bit lane offset; nothing computed on the loaded
// values, see MetaRaw).
template <int KIND>
__device__ __forceinline__ MetaRaw load_meta_buf(__amdgpu_buffer_rsrc_t r_s, __amdgpu_buffer_rsrc_t r_z,
                                                 uint32_t gi) {
  using T = WKindTraits<KIND>;
  MetaRaw r{0u, 0u};
  if constexpr (T::fmt == FMT_MINMAX && T::compact) {
    r.s = __builtin_amdgcn_raw_buffer_load_b16(r_s, gi * 2u, 0, 0);
    r.z = __builtin_amdgcn_raw_buffer_load_b8(r_z, gi * (uint32_t)T::bits / 8u, 0, 0);
  } else if constexpr (T::fmt == FMT_MINMAX) {
    r.s = __builtin_amdgcn_raw_buffer_load_b32(r_s, gi * 4u, 0, 0);
    r.z = __builtin_amdgcn_raw_buffer_load_b8(r_z, gi, 0, 0);
  } else if constexpr (T::dq) {
    r.z = __builtin_amdgcn_raw_buffer_load_b8(r_z, gi, 0, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b32(r_s, (gi >> 8) * 4u, 0, 0);
  } else {
    r.s = __builtin_amdgcn_raw_buffer_load_b32(r_s, gi * 4u, 0, 0);
  }
  return r;
}
// Per-tensor offset of double quantization with an offset: the entry after
// the ceil(nb / 256) per-block scales.
__device__ __forceinline__ float nf4_dq_offset(const WView& w) {
  return w.absmax_scale[(w.n * w.k / 64 + 255) >> 8];
}

// Decoded scale (MinMax s or the NF4 block absmax) and MinMax zero point of
// a MetaRaw loaded for entry gi.
template <int KIND>
__device__ __forceinline__ float meta_raw_scale(const MetaRaw& r, float off) {
  using T = WKindTraits<KIND>;
  if constexpr (T::fmt == FMT_MINMAX) {
    return T::compact ? f16_bits_to_f32(r.s) : __uint_as_float(r.s);
  } else if constexpr (T::dq) {
    const float p = (float)(int)(int8_t)(uint8_t)r.z * __uint_as_float(r.s);
    return T::dqo ? p + off : p;
  } else {
    return __uint_as_float(r.s);
  }
}
template <int KIND>
__device__ __forceinline__ int meta_raw_zero(const MetaRaw& r, int64_t gi) {
  return zero_from_byte<KIND>(r.z, gi);
}

// Block absmax of NF4 block `blk`: fp32, fl(q2 * c2) under double quant, or
// fl(fl(q2 * c2) + off) with an offset (`off` from nf4_dq_offset).
template <int KIND>
__device__ __forceinline__ float nf4_block_scale(const WView& w, int64_t blk, float off) {
  using T = WKindTraits<KIND>;
  if constexpr (T::dqo) {
    const float p = (float)w.absmax_q[blk] * w.absmax_scale[blk >> 8];
    return p + off;
  } else if constexpr (T::dq) {
    return (float)w.absmax_q[blk] * w.absmax_scale[blk >> 8];
  } else {
    return w.absmax[blk];
  }
}

// Dispatch a functor templated on the weight kind.
template <template <int> class F, typename... Args>
hipError_t dispatch_kind(WKind kind, Args&&... args) {
  switch (kind) {
    case WK_I4G128: return F<WK_I4G128>::run(args...);
    case WK_I4G64: return F<WK_I4G64>::run(args...);
    case WK_I2G64: return F<WK_I2G64>::run(args...);
    case WK_I2G128: return F<WK_I2G128>::run(args...);
    case WK_NF4: return F<WK_NF4>::run(args...);
    case WK_NF4DQ: return F<WK_NF4DQ>::run(args...);
    case WK_I4G128C: return F<WK_I4G128C>::run(args...);
    case WK_I2G64C: return F<WK_I2G64C>::run(args...);
    case WK_NF4DQO: return F<WK_NF4DQO>::run(args...);
  }
  return hipErrorInvalidValue;
}

}  // namespace lbq
