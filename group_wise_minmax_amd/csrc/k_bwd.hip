// Input gradient through the frozen low-bit weight (dX = dY . deq(W)) on bf16
// MFMA, and the LoRA prologue T = sigma * X . A^T.
#include "lbq_device.h"

namespace lbq {

namespace {

// ---------------------------------------------------------------------------
// Input gradient dX = dY . deq(W) ("QLoRA技术在量化微调中的应用", section
// QLoRA技术原理: backpropagation through the frozen quantized weights).
//
// Workgroup tile: BKO columns of dX (k) x BM rows (m), reduction over n in
// stages of 64, WGK x WGM waves.  MFMA operand A is the dequantized weight
// transposed (rows k, 8 consecutive n per lane), B is dY (rows m), so each
// lane's accumulators are four consecutive k of one m and the epilogue writes
// 8 contiguous bytes of a dX row.
//
// The packed weight is contiguous along k, the reduction runs along n: per
// stage a thread dequantizes 8 codes (one k-chunk) of 4 consecutive rows n
// and writes, for each of its 8 k, the 4 values of the rows as one 8-byte LDS
// store into the k-major tile.  The n-quad is the lane's low 4 bits, which
// (with the row swizzle) keeps these column writes bank-conflict free.  The
// codes are loaded row-wise, though: 32 codes of one row (one 16- or 8-byte
// load, with that row's metadata), and four permlane swaps transpose the
// 4 x 4 dwords across the lanes that share the n-quad.  A stage so costs 3
// weight loads per thread rather than a code word, a scale and a zero point
// for each of 4 rows.  dY chunks are staged like X in the forward GEMM.  Both
// tiles are double-buffered (one barrier per stage, two with the 8-wave
// two-phase loop), and every global load goes through a buffer resource
// (reads past the end return zeros), so rows past n, m or k need no guards.
// ---------------------------------------------------------------------------
constexpr int BNR = 64;  // reduction (n) per stage = one 128-byte LDS row

// Lane rows are the four groups of 16 lanes.  gfx950's permlane swaps:
// swap32(a, b) exchanges lanes 32..63 of a with lanes 0..31 of b, swap16(a, b)
// the odd lane rows of a with the even lane rows of b.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
// 4 x 4 transpose over the lane rows: afterwards x_r in lane row j holds what
// x_j held in lane row r (same lane within the row).
__device__ __forceinline__ void transpose_rows4(uint32_t& x0, uint32_t& x1, uint32_t& x2, uint32_t& x3) {
  swap32(x0, x2);
  swap32(x1, x3);
  swap16(x0, x1);
  swap16(x2, x3);
}
// out[r] = v of lane row r (same lane within the row), in every lane row.
__device__ __forceinline__ void gather_rows4(float v, float out[4]) {
  uint32_t a = __float_as_uint(v), b = a;
  swap32(a, b);  // a: v0 v1 v0 v1, b: v2 v3 v2 v3 (by lane row)
  uint32_t a2 = a, b2 = b;
  swap16(a, a2);  // a: v0 everywhere, a2: v1
  swap16(b, b2);  // b: v2, b2: v3
  out[0] = __uint_as_float(a);
  out[1] = __uint_as_float(a2);
  out[2] = __uint_as_float(b);
  out[3] = __uint_as_float(b2);
}

// Weights of one kind and k whose input gradients add up (they share X):
// dX = sum_i dY_i . deq(W_i).  The reduction runs over their rows one weight
// after the other; weight i owns the 64-row stages [stage_end[i-1],
// stage_end[i]).  A single weight is a set of one.
struct BwdSet {
  WView w[kGemvMaxGroup];
  const uint16_t* dy[kGemvMaxGroup];
  int stage_end[kGemvMaxGroup];
  int count;
  int k_begin, k_cols;  // the launch's columns of dX: [k_begin, k_begin + k_cols)
};

// SET: the set may hold several weights (the weight of the stage about to be
// loaded is looked up at the top of each K step and bound when it changes);
// otherwise it holds one, bound once.
template <int KIND, int BKO, int BM, int WGK, int WGM, bool LORA, bool SET>
__global__ __launch_bounds__(WGK* WGM * 64) void k_bwd_dx(BwdSet set, int m, uint16_t* __restrict__ dX,
                                                        LoraDx lora, Nf4Table tab) {
  using T = WKindTraits<KIND>;
  constexpr int NT = WGK * WGM * 64;
  constexpr int WK = BKO / WGK, WM = BM / WGM;
  constexpr int TK = WK / 16, TM = WM / 16;
  constexpr int KCH = BKO / 8;                 // 8-code k-chunks per tile row
  static_assert(KCH * 16 == NT, "a thread owns one k-chunk of 4 rows n per stage");
  constexpr int DCH = BM * BNR / 8 / NT;       // 16-byte dY chunks per thread per stage
  static_assert(DCH * NT * 8 == BM * BNR, "dY tile split");

  __shared__ __attribute__((aligned(16))) uint16_t Wt[2][BKO * BNR];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[2][BM * BNR];
  __shared__ f32x2_t pairlut[T::fmt == FMT_NF4 ? 256 : 1];
  __shared__ float cbs[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wk = wave % WGK, wm = wave / WGK;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t K = set.w[0].k;
  const int nx = (set.k_cols + BKO - 1) / BKO, ny = (m + BM - 1) / BM;
  int tx, ty;
  tile_of(blockIdx.x, nx, ny, tx, ty);
  const int64_t k0 = set.k_begin + (int64_t)tx * BKO;
  const int64_t m0 = (int64_t)ty * BM;
  // the reduction: 64-row stages over all weights of the set
  int nstage = set.stage_end[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxGroup; ++i)
    if (i < set.count) nstage = set.stage_end[i];
  const int64_t N = (int64_t)nstage * BNR;
  const int64_t KB = K * T::bits / 8;
  const int64_t gpr = K / T::group;

  if constexpr (T::fmt == FMT_NF4) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (tid == i) cbs[i] = tab.c[i];
    __syncthreads();
    for (int b = tid; b < 256; b += NT) pairlut[b] = (f32x2_t){cbs[b >> 4], cbs[b & 15]};
  }

  // Buffer resources of the weight whose rows a stage reads, and that
  // weight's row count (the dY row stride).  They are (re)bound only in code
  // that every lane of the workgroup runs alike, before the stage's loads:
  // the loads themselves run under a branch on the wave index, and a value
  // changed inside that branch would be taken as varying per lane (every
  // buffer load would then loop over distinct resources).
  struct Bound {
    __amdgpu_buffer_rsrc_t w, d, s, z;
    int64_t n;
    int beg;    // first stage of the weight
    float off;  // offset of double quantization with an offset
  };
  auto bind = [&](int i) {
    const WView& w = set.w[i];
    Bound b;
    b.n = w.n;
    b.beg = i == 0 ? 0 : set.stage_end[i - 1];
    const int64_t nblk = b.n * gpr;
    b.w = make_rsrc(w.packed, b.n * KB);
    b.d = make_rsrc(set.dy[i], (int64_t)m * b.n * 2);
    b.off = 0.f;
    if constexpr (T::fmt == FMT_MINMAX) {
      b.s = make_rsrc(w.scales, scale_byte_index<KIND>(nblk));
      b.z = make_rsrc(w.zeros, zero_byte_index<KIND>(nblk));
    } else if constexpr (T::dq) {
      b.s = make_rsrc(w.absmax_scale, ((nblk + 255) >> 8) * 4);
      b.z = make_rsrc(w.absmax_q, nblk);
      if constexpr (T::dqo) b.off = nf4_dq_offset(w);
    } else {
      b.s = make_rsrc(w.absmax, nblk * 4);
      b.z = b.s;
    }
    return b;
  };
  Bound cur = bind(0);
  int cur_i = 0;
  // bind the weight of the stage starting at row vt of the set
  auto bind_for = [&](int64_t vt) {
    if constexpr (SET) {
      const int st = (int)(vt / BNR);
      int wi = 0;
#pragma unroll
      for (int i = 1; i < kGemvMaxGroup; ++i)
        if (i < set.count && st >= set.stage_end[i - 1]) wi = i;
      if (wi != cur_i) {
        cur_i = wi;
        cur = bind(wi);
      }
    }
  };

  // Weight ownership: rows 4*q .. 4*q+3 of each stage, codes [8*c, +8) of the
  // k tile, with q = lane & 15 and c = (NT/64 waves) x 4 chunks.  The loads
  // are row-wise: lane (q, lg) reads the 32 codes [32*wave, +32) of row
  // 4*q + lg and that row's metadata, and a transpose over the lane rows
  // (lanes q, q+16, q+32, q+48) hands each lane its chunk lg of the 4 rows.
  const int q = lane & 15, c = 4 * wave + lg;
  const int64_t kp = k0 + 32 * wave;
  const uint32_t w_voff = (uint32_t)((4 * q + lg) * KB + kp * T::bits / 8);
  const uint32_t g_voff = (uint32_t)((4 * q + lg) * gpr + kp / T::group);
  // dY chunks of this thread: chunk ci = tid + NT*i -> row ci >> 3, chunk ci & 7.
  const int64_t d_row = m0 + (tid >> 3), d_col = 8 * (tid & 7);
  char* const wt_base = reinterpret_cast<char*>(&Wt[0][0]);
  char* const ds_base = reinterpret_cast<char*>(&Ds[0][0]);
  constexpr uint32_t WT_BUF = BKO * BNR * 2, DS_BUF = BM * BNR * 2;

  f32x4_t acc[TK][TM];
#pragma unroll
  for (int a = 0; a < TK; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t dr[DCH];
  u32x4_t wraw;  // 32 codes of row 4q + lg (2-bit: dwords 0 and 1)
  float md_s;
  int md_i;
  float md_off = 0.f;  // the loaded stage's weight's offset (the binding may move on before the store)
  // loads of the stage starting at row vt of the set, from the bound weight
  auto load_stage = [&](int64_t vt) {
    const int st = (int)(vt / BNR);
    const Bound& b = cur;
    const __amdgpu_buffer_rsrc_t r_w = b.w, r_d = b.d, r_s = b.s, r_z = b.z;
    const int64_t Nw = b.n;
    const int64_t nt = (int64_t)(st - b.beg) * BNR;
    const uint32_t d_voff = (uint32_t)((d_row * Nw + d_col) * 2);
#pragma unroll
    for (int i = 0; i < DCH; ++i) {
      // chunk tid + NT*i: NT/8 rows further down per i
      const int so = (int)((NT / 8) * i * Nw * 2 + nt * 2);
      dr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_d, d_voff, so, 0));
    }
    const int so = (int)(nt * KB);
    if constexpr (T::bits == 4) {
      wraw = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_w, w_voff, so, 0));
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r_w, w_voff, so, 0);
      wraw = u32x4_t{v[0], v[1], 0u, 0u};
    }
    const int go = (int)(nt * gpr);
    if constexpr (T::fmt == FMT_MINMAX && T::compact) {
      // fp16 scale bits and the packed zero byte, as loaded (decoded in
      // store_stage: a use here would make the wave wait for the load)
      md_s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b16(r_s, g_voff * 2, go * 2, 0));
      md_i = __builtin_amdgcn_raw_buffer_load_b8(r_z, g_voff * T::bits / 8, go * T::bits / 8, 0);
    } else if constexpr (T::fmt == FMT_MINMAX) {
      md_s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_s, g_voff * 4, go * 4, 0));
      md_i = __builtin_amdgcn_raw_buffer_load_b8(r_z, g_voff, go, 0);
    } else if constexpr (T::dq) {
      md_i = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(r_z, g_voff, go, 0);
      md_s = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(r_s, ((g_voff + (uint32_t)go) >> 8) * 4, 0, 0));
      if constexpr (T::dqo) md_off = b.off;
    } else {
      md_s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_s, g_voff * 4, go * 4, 0));
    }
  };
  auto store_stage = [&](int buf) {
    char* ds = ds_base + buf * DS_BUF;
#pragma unroll
    for (int i = 0; i < DCH; ++i) {
      const int ci = tid + NT * i;
      *reinterpret_cast<u32x4_t*>(ds + swz(ci >> 3, ci & 7)) = dr[i];
    }
    // wr[r]: chunk lg (8 codes) of row 4q + r
    uint32_t wr[4];
    if constexpr (T::bits == 4) {
      wr[0] = wraw[0], wr[1] = wraw[1], wr[2] = wraw[2], wr[3] = wraw[3];
    } else {
      wr[0] = wraw[0] & 0xFFFFu, wr[1] = wraw[0] >> 16, wr[2] = wraw[1] & 0xFFFFu, wr[3] = wraw[1] >> 16;
    }
    transpose_rows4(wr[0], wr[1], wr[2], wr[3]);
    // scale (MinMax: and z*s; NF4: the block absmax) of row 4q + r
    float sc[4], zc[4];
    if constexpr (T::fmt == FMT_MINMAX) {
      float s_ = md_s;
      int z_ = md_i;
      if constexpr (T::compact) {
        // go is a multiple of 64 rows' entries, so entry go + g_voff has the
        // parity of g_voff within its zero byte
        s_ = f16_bits_to_f32(__float_as_uint(md_s));
        z_ = zero_from_byte<KIND>((uint32_t)md_i, g_voff);
      }
      gather_rows4(s_, sc);
      gather_rows4((float)z_ * s_, zc);
    } else {
      gather_rows4(T::dqo ? (float)md_i * md_s + md_off : (T::dq ? (float)md_i * md_s : md_s), sc);
    }
    // v[r][j]: row 4q + r, code j of the chunk
    float v[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (T::fmt == FMT_MINMAX) {
        const float s = sc[r], zs = zc[r];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[r][j] = fmaf((float)code_of<T::bits>(wr[r], j), s, -zs);
      } else {
        const float a = sc[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2_t cc = pairlut[(wr[r] >> (8 * j)) & 0xFFu];
          v[r][2 * j] = cc[0] * a;
          v[r][2 * j + 1] = cc[1] * a;
        }
      }
    }
    char* wt = wt_base + buf * WT_BUF;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint2 p;
      p.x = cvt_pk_bf16(v[0][j], v[1][j]);
      p.y = cvt_pk_bf16(v[2][j], v[3][j]);
      *reinterpret_cast<uint2*>(wt + swz(8 * c + j, q >> 1) + 8 * (q & 1)) = p;
    }
  };
  // Operand rows: Wt rows wk*WK + 16*a + li, Ds rows wm*WM + 16*b + li; chunk
  // 4*(ks/32) + lg of each.
  const uint32_t a_base = swz(wk * WK + li, lg), a_base1 = swz(wk * WK + li, 4 + lg);
  const uint32_t b_base = swz(wm * WM + li, lg), b_base1 = swz(wm * WM + li, 4 + lg);
  auto compute = [&](int buf) {
    const char* wt = wt_base + buf * WT_BUF;
    const char* ds = ds_base + buf * DS_BUF;
#pragma unroll
    for (int ks = 0; ks < BNR; ks += 32) {
      u32x4_t af[TK], bf[TM];
#pragma unroll
      for (int a = 0; a < TK; ++a)
        af[a] = *reinterpret_cast<const u32x4_t*>(wt + (ks ? a_base1 : a_base) + a * 16 * 128);
#pragma unroll
      for (int b = 0; b < TM; ++b)
        bf[b] = *reinterpret_cast<const u32x4_t*>(ds + (ks ? b_base1 : b_base) + b * 16 * 128);
#pragma unroll
      for (int a = 0; a < TK; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma16x16x32(af[a], bf[b], acc[a][b]);
    }
  };

  // n % 8 == 0, so the rows of a weight's last 64-wide stage past its n only
  // meet zero weights (buffer reads past the end) times finite dY values.
  if constexpr (T::fmt == FMT_NF4) __syncthreads();  // pair table visible
  load_stage(0);
  store_stage(0);
  if (BNR < N) {
    bind_for(BNR);
    load_stage(BNR);
  }
  __syncthreads();
  int buf = 0;
  if constexpr (WGK * WGM == 8) {
    // Two phases per stage, with a barrier between them: the first four waves
    // stage the next tile while the last four run their MFMAs, then the other
    // way round.  Waves w and w + 4 share a SIMD, so at any time one of them
    // feeds the matrix core while the other does the dequant and LDS writes.
    // The staging wave runs at raised priority: its loads, table reads and
    // conversions are a chain of short instructions that would otherwise wait
    // behind the MFMA wave's issue slots, while the MFMAs queue up anyway
    // (8B NF4+DQ layer at m = 4096, against raising the MFMA wave: forward
    // +0.8-1.5%, input gradient +1%).
    const bool late = wave >= 4;
    auto stage = [&](int64_t t) {
      __builtin_amdgcn_s_setprio(1);
      if (t + BNR < N) {
        store_stage(buf ^ 1);
        if (t + 2 * BNR < N) load_stage(t + 2 * BNR);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    auto mfma_phase = [&]() { compute(buf); };
    for (int64_t nt = 0; nt < N; nt += BNR) {
      if (nt + 2 * BNR < N) bind_for(nt + 2 * BNR);  // both wave groups load this stage
      if (late) mfma_phase();
      else stage(nt);
      __syncthreads();
      if (late) stage(nt);
      else mfma_phase();
      __syncthreads();
      buf ^= 1;
    }
  } else {
    for (int64_t nt = 0; nt < N; nt += BNR) {
      if (nt + BNR < N) {
        store_stage(buf ^ 1);
        if (nt + 2 * BNR < N) {
          bind_for(nt + 2 * BNR);
          load_stage(nt + 2 * BNR);
        }
      }
      compute(buf);
      __syncthreads();
      buf ^= 1;
    }
  }

  // LoRA slab: acc[k][m] += sum over j of A[j][k] * G[m][j], r zero-padded to rp.
  if constexpr (LORA) {
    for (int ks = 0; ks < lora.rp; ks += 32) {
      u32x4_t la[TK], lb[TM];
#pragma unroll
      for (int a = 0; a < TK; ++a) {
        const int64_t k = k0 + wk * WK + 16 * a + li;
        uint32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c0 = ks + 8 * lg + 2 * j;
          uint32_t lo = 0, hi = 0;
          if (k < K && c0 < lora.r) lo = lora.a[(int64_t)c0 * K + k];
          if (k < K && c0 + 1 < lora.r) hi = lora.a[(int64_t)(c0 + 1) * K + k];
          v[j] = lo | (hi << 16);
        }
        la[a] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const int64_t mr = m0 + wm * WM + 16 * b + li;
        lb[b] = (mr < m) ? *reinterpret_cast<const u32x4_t*>(lora.g + mr * lora.rp + ks + 8 * lg)
                         : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int a = 0; a < TK; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma16x16x32(la[a], lb[b], acc[a][b]);
    }
  }

  // Row tile b outer, column tile a inner: the TK stores that fill a row's
  // WK contiguous outputs (whole 128-byte lines) follow one another.
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int64_t mr = m0 + wm * WM + 16 * b + li;
    if (mr >= m) continue;
#pragma unroll
    for (int a = 0; a < TK; ++a) {
      const int64_t kb = k0 + wk * WK + 16 * a + 4 * lg;
      if (kb >= K) continue;
      uint2 v;
      v.x = cvt_pk_bf16(acc[a][b][0], acc[a][b][1]);
      v.y = cvt_pk_bf16(acc[a][b][2], acc[a][b][3]);
      *reinterpret_cast<uint2*>(dX + mr * K + kb) = v;
    }
  }
}

template <int KIND, int BKO, int BM, int WGK, int WGM>
hipError_t launch_bwd_cfg(const BwdSet& set, int64_t m, uint16_t* dX, const LoraDx& lora, const Nf4Table& tab,
                          hipStream_t s) {
  const int64_t tiles = ((set.k_cols + BKO - 1) / BKO) * ((m + BM - 1) / BM);
  if (lora.g != nullptr) {  // LoRA: single weights only
    hipLaunchKernelGGL((k_bwd_dx<KIND, BKO, BM, WGK, WGM, true, false>), dim3((unsigned)tiles),
                       dim3(WGK * WGM * 64), 0, s, set, (int)m, dX, lora, tab);
  } else if (set.count > 1) {
    hipLaunchKernelGGL((k_bwd_dx<KIND, BKO, BM, WGK, WGM, false, true>), dim3((unsigned)tiles),
                       dim3(WGK * WGM * 64), 0, s, set, (int)m, dX, lora, tab);
  } else {
    hipLaunchKernelGGL((k_bwd_dx<KIND, BKO, BM, WGK, WGM, false, false>), dim3((unsigned)tiles),
                       dim3(WGK * WGM * 64), 0, s, set, (int)m, dX, lora, tab);
  }
  return hipGetLastError();
}

double bwd_fill(int64_t tiles) {
  const int64_t waves = (tiles + 255) / 256;
  return (double)tiles / (double)(waves * 256);
}

template <int KIND>
struct BwdLauncher {
  static hipError_t run(const BwdSet& set, int64_t m, uint16_t* dX, const LoraDx& lora, const Nf4Table& tab,
                        hipStream_t s) {
    // 256 x 256 tiles (8 waves of 128 x 64) unless they leave most of the chip idle.
    const int64_t k = set.k_cols;
    const int64_t t256 = ((k + 255) / 256) * ((m + 255) / 256);
    const int64_t t128 = ((k + 127) / 128) * ((m + 127) / 128);
    // Several rounds of 256 x 256 tiles with a partly empty last one: the
    // columns that fill whole rounds in one launch, the rest in a second one
    // on 128 x 128 tiles (8B down at m = 4096: 896 tiles = 3.5 rounds become
    // 768 tiles and 512 small ones; the layer's input gradient +1-1.5%).
    // Each output's sum runs over n in the same order whatever the tile, so
    // the cut changes no bit.
    const int64_t ny = (m + 255) / 256;
    const int64_t kc = (t256 / 256) * 256 / ny * 256;  // columns of the whole rounds
    if (t256 > 256 && t256 % 256 != 0 && kc > 0 && kc < k) {
      BwdSet a = set, b = set;
      a.k_cols = (int)kc;
      b.k_begin = set.k_begin + (int)kc;
      b.k_cols = (int)(k - kc);
      const hipError_t e = launch_bwd_cfg<KIND, 256, 256, 2, 4>(a, m, dX, lora, tab, s);
      if (e != hipSuccess) return e;
      return launch_bwd_cfg<KIND, 128, 128, 2, 2>(b, m, dX, lora, tab, s);
    }
    if (bwd_fill(t256) >= 0.5 * bwd_fill(t128)) return launch_bwd_cfg<KIND, 256, 256, 2, 4>(set, m, dX, lora, tab, s);
    return launch_bwd_cfg<KIND, 128, 128, 2, 2>(set, m, dX, lora, tab, s);
  }
};

BwdSet make_bwd_set(const WView* ws, const uint16_t* const* dys, int count) {
  BwdSet set{};
  set.count = count;
  int end = 0;
  for (int i = 0; i < count; ++i) {
    set.w[i] = ws[i];
    set.dy[i] = dys[i];
    end += (int)((ws[i].n + BNR - 1) / BNR);
    set.stage_end[i] = end;
  }
  set.k_begin = 0;
  set.k_cols = (int)ws[0].k;
  return set;
}

}  // namespace

hipError_t launch_bwd_dx(WKind kind, const WView& w, const uint16_t* dY, int64_t m,
                         uint16_t* dX, const LoraDx& lora, const Nf4Table& tab, hipStream_t s) {
  return dispatch_kind<BwdLauncher>(kind, make_bwd_set(&w, &dY, 1), m, dX, lora, tab, s);
}

hipError_t launch_bwd_dx_set(WKind kind, const WView* ws, const uint16_t* const* dys, int count, int64_t m,
                             uint16_t* dX, const Nf4Table& tab, hipStream_t s) {
  if (count < 1 || count > kGemvMaxGroup) return hipErrorInvalidValue;
  for (int i = 1; i < count; ++i)
    if (ws[i].k != ws[0].k) return hipErrorInvalidValue;
  const LoraDx none{nullptr, nullptr, 0, 0};
  return dispatch_kind<BwdLauncher>(kind, make_bwd_set(ws, dys, count), m, dX, none, tab, s);
}


}  // namespace lbq
