/*
 * lbq -- group-wise low-bit weight quantization and the fused
 * dequantize-then-matmul of a frozen low-bit linear layer, for AMD MI355X
 * (gfx950).  Plain C ABI: pointers and sizes only, no framework types.
 *
 * Sources (cited by page title and section):
 *   [GB]  GreenBit.AI, "只需单卡RTX 3090，低比特量化训练就能实现LLaMA-3 8B全参微调",
 *         section 模型量化: classic group-wise MinMax quantizer, INT4 with
 *         group size 128 and INT2 with group size 64 as the base
 *         representations (chosen per layer or per channel), round-to-nearest.
 *   [BNB] bitsandbytes FSDP-QLoRA guide (walk-through of docs/source/fsdp_qlora.md),
 *         section 量化数据的存储: two 4-bit codes per byte, even-indexed code in
 *         the high nibble; packed bytes may be viewed as any dtype of equal
 *         width without changing them; section 通过BitsAndBytesConfig配置: the
 *         kernel unpacks and dequantizes weights to the compute dtype (bf16)
 *         before the matmul; step 2's parameter table: quant type nf4 or fp4
 *         (type-checked), double quantization of the absmax statistics;
 *         step 4: LoRA adapters (lora_alpha, r).
 *   [QL]  "QLoRA技术在量化微调中的应用", section QLoRA技术原理: NF4 for normally
 *         distributed weights; double quantization of the quantization
 *         constants; gradients are backpropagated through the frozen 4-bit
 *         model into low-rank adapters.
 *
 * Conventions shared by every entry point
 *   Ownership:  every buffer is device memory owned by the caller; the library
 *               never allocates or frees device memory and keeps no device
 *               state between calls.
 *   Execution:  every call that touches the device only enqueues kernels on
 *               `stream` (a hipStream_t passed as void*, NULL = the default
 *               stream) and returns without synchronizing.
 *   Errors:     argument, shape, format and alignment errors are detected on
 *               the host before anything is enqueued and returned as a status;
 *               a failed launch returns LBQ_E_HIP.  lbq_last_error_detail()
 *               gives a human-readable message for the last failure on the
 *               calling thread.  Inputs containing NaN or Inf are outside the
 *               contract.
 *   Layouts:    row-major.  W is n x k (out x in, like a linear layer's
 *               weight); X is m x k; Y is m x ldy; dY is m x n; dX is m x k.
 *               bf16 tensors are passed as uint16_t bit patterns.
 *   Alignment:  `packed`, W, X, dY, dX, LoRA A and the LoRA workspace must
 *               be 16-byte aligned; Y, LoRA B 2-byte aligned; scales (fp16
 *               scales 2-byte), absmax and absmax_scale 4-byte aligned.
 */
#ifndef LBQ_H
#define LBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LBQ_OK = 0,
  LBQ_E_NULL = 1,        /* a required pointer is NULL                       */
  LBQ_E_SHAPE = 2,       /* n, k, m, r, ldy out of range or inconsistent     */
  LBQ_E_FORMAT = 3,      /* unknown format / bits / group / dq settings      */
  LBQ_E_ALIGN = 4,       /* a pointer or leading dimension is misaligned     */
  LBQ_E_WORKSPACE = 5,   /* workspace missing or smaller than required       */
  LBQ_E_UNSUPPORTED = 6, /* valid request this library does not implement    */
  LBQ_E_HIP = 7          /* the HIP runtime reported an error                */
} lbq_status;

typedef enum {
  LBQ_MINMAX = 0, /* asymmetric group-wise MinMax RTN [GB]                   */
  LBQ_NF4 = 1     /* 4-bit NormalFloat, blockwise absmax, optional DQ [QL]   */
} lbq_format;

/* MinMax metadata layouts (lbq_desc.meta). */
typedef enum {
  LBQ_META_F32 = 0,     /* fp32 scale and one byte per zero point            */
  LBQ_META_COMPACT = 1  /* fp16 scale and the zero point packed bits wide    */
} lbq_meta;

/* Describes one quantized weight W[n][k].
 *   MINMAX: bits in {4, 2}, group in {64, 128}, k % group == 0;
 *           double_quant = 0, dq_block = 0; meta = LBQ_META_F32, or
 *           LBQ_META_COMPACT for INT4 g128 and INT2 g64 with
 *           (k / group) * bits % 8 == 0 (see lbq_quantize).
 *   NF4:    bits = 4, group = 64 (absmax block; blocks run row-major and never
 *           straddle rows because k % 64 == 0); meta = 0; double_quant 0
 *           (fp32 absmax), 1 (absmax double-quantized) or 2 (double-quantized
 *           with a per-tensor offset); dq_block = 256 with double
 *           quantization, else 0.
 * n >= 1, k >= 64. */
typedef struct {
  int32_t format;
  int32_t bits;
  int32_t group;
  int32_t double_quant;
  int32_t dq_block;
  int32_t meta;
  int64_t n;
  int64_t k;
} lbq_desc;

/* Device buffers of one quantized weight.  Which fields are used:
 *   packed        all formats  u8[n][k*bits/8]; 4-bit: byte i of a row holds
 *                              code 2i in bits 7..4 and code 2i+1 in bits 3..0
 *                              [BNB]; 2-bit: code 4i in bits 7..6, then 5..4,
 *                              3..2, 1..0.  Only the bytes matter: the caller
 *                              may hold them in any dtype of the same size.
 *   scales        MINMAX       f32[n][k/group]; compact: fp16 bit patterns
 *                              u16[n][k/group] (2-byte aligned)
 *   zeros         MINMAX       u8 [n][k/group]  (integer zero point 0..2^bits-1);
 *                              compact: u8[n][(k/group)*bits/8], the zero
 *                              points of a row packed like the codes (first
 *                              group in the high bits)
 *   absmax        NF4, DQ=0    f32[n*k/64]
 *   absmax_q      NF4, DQ=1    i8 [n*k/64]      (0..127); DQ=2: -127..127
 *   absmax_scale  NF4, DQ=1    f32[ceil(n*k/64/256)]; DQ=2: one more entry
 *                              at the end, the per-tensor offset
 *   out_rows      optional (forward only): int32[n]; row i of W writes output
 *                 column out_rows[i] of Y (channel-mix scatter [GB]).  NULL
 *                 means row i writes column i.  Entries must be distinct and
 *                 in [0, ldy); this is the caller's responsibility.
 * Unused fields are ignored. */
typedef struct {
  void* packed;
  void* scales;
  uint8_t* zeros;
  float* absmax;
  int8_t* absmax_q;
  float* absmax_scale;
  const int32_t* out_rows;
} lbq_qtensor;

/* Byte sizes of every buffer of a quantized weight (0 for unused ones). */
typedef struct {
  size_t packed;
  size_t scales;
  size_t zeros;
  size_t absmax;
  size_t absmax_q;
  size_t absmax_scale;
} lbq_sizes;

/* Host only, no device access.  Validates `desc` and returns the sizes of the
 * buffers lbq_quantize fills.  Errors: LBQ_E_NULL, LBQ_E_FORMAT, LBQ_E_SHAPE. */
lbq_status lbq_layout(const lbq_desc* desc, lbq_sizes* out);

/* Quantize fp32 W[n][k] (device) into the buffers of `q`.
 *   MINMAX [GB] 模型量化: per row and group of `group` consecutive weights:
 *     lo = min(0, min w), hi = max(0, max w); s = fl(fl(hi-lo)/(2^bits-1)),
 *     s := 1 if it is 0; z = clamp(rne(fl(-lo/s)), 0, 2^bits-1);
 *     q = clamp(rne(fl(w/s)) + z, 0, 2^bits-1); codes packed as above.
 *   NF4 [QL] QLoRA技术原理: per block of 64: a = max|w|; codes 7 if a == 0, else
 *     the number of fp32 codebook midpoints strictly below fl(w/a).  With
 *     double_quant = 1 the block absmax values are re-quantized in runs of
 *     256: c2 = fl(max/127), q2 = clamp(rne(fl(a/c2)), 0, 127) (0 if c2 == 0);
 *     the 4-bit codes always use the un-quantized a.
 *   MINMAX, compact metadata (an fp16 scale per group, the form GPTQ-style
 *     checkpoints store [GB] 模型量化): s32 as above; the stored scale s is
 *     the smallest fp16 value >= s32 (65504 at most), and z and q are formed
 *     with that s, so Qmax * s still spans the group's range.
 *   NF4, double_quant = 2 ([QL] 结论: double quantization re-quantizes the
 *     scale factor and the offset; [BNB] 源码纵深: `offset` is a field of the
 *     quantization state): off = fp32(fp64(S) / nb), S the sum of the nb
 *     absmax values over the binary tree of adjacent pairs in index order
 *     (zero-padded to a power of two, fp32 additions); per run of 256:
 *     d = fl(a - off), c2 = fl(max|d|/127), q2 = clamp(rne(fl(d/c2)), -127,
 *     127) (0 if c2 == 0); decoded as fl(fl(q2 * c2) + off).  Three launches.
 * Every fp32 step is one IEEE operation rounded to nearest-even (true
 * division, no contraction); results are bit-exact across runs.
 * Pure: it never inspects the old contents of the outputs. */
lbq_status lbq_quantize(const lbq_desc* desc, const float* W, const lbq_qtensor* q,
                        void* stream);

/* Dequantize to bf16 W_bf16[n][k] (device) [BNB] 通过BitsAndBytesConfig配置:
 *   MINMAX: bf16(fl((q - z) * s));  NF4: bf16(fl(c[code] * A)) with A the block
 *   absmax, fl(q2 * c2) under double quantization, or fl(fl(q2 * c2) + off)
 *   with an offset.  bf16 rounding is round-to-nearest-even; the result is
 *   bit-exact. */
lbq_status lbq_dequant(const lbq_desc* desc, const lbq_qtensor* q, uint16_t* W_bf16,
                       void* stream);

/* Workspace bytes lbq_linear_fwd takes for m rows (0 when none): for
 * 2 <= m <= 64 the small-batch kernel's partial sums (required); for m > 64
 * the partial sums of a GEMM that splits K (optional, see lbq_linear_fwd). */
size_t lbq_linear_workspace_bytes(const lbq_desc* desc, int64_t m);

/* Forward of the frozen low-bit linear layer, Y = X . deq(W)^T ([BNB]
 * 通过BitsAndBytesConfig配置: the kernel unpacks the stored 4-bit weight and
 * dequantizes it to the bf16 compute dtype for the matmul; [GB] 模型量化 for
 * the INT4 g128 / INT2 g64 MinMax weights the same call multiplies):
 *   Y[i][col(j)] = bf16( sum_k X[i][k] * w_hat[j][k] ),  col(j) = out_rows ?
 *   out_rows[j] : j, with w_hat the dequantized weight and fp32 accumulation.
 * X: bf16 [m][k] (device); Y: bf16 [m][ldy] (device), ldy >= n (or >
 * max(out_rows)); only the n addressed columns of each row are written.
 * m >= 0 (m == 0 is an empty batch: nothing is read or written);
 * (m + 256) * k * 2 and (n + 256) * k must be below 2^32 (LBQ_E_SHAPE
 * otherwise: the GEMM uses 32-bit byte offsets).  For m <= 64 `workspace`
 * must hold lbq_linear_workspace_bytes(desc, m) bytes, 16-byte aligned (may
 * be NULL when that is 0; LBQ_E_WORKSPACE / LBQ_E_ALIGN otherwise).  For
 * m > 64 it is optional: with that many bytes (16-byte aligned), a weight
 * whose 256x256 output tiles fill at most half the chip (for m <= 256 and
 * short K, at most an eighth) splits K over up to 8 workgroups and a second
 * kernel sums their fp32 partials in a fixed order;
 * with less (or NULL) the GEMM runs unsplit.  The two results agree within
 * fp32 rounding, not bit for bit.
 * m == 1 runs a GEMV that streams the packed weight once; 2 <= m <= 4 the
 * same streaming with every row of X staged in LDS (when the rows fit in 64
 * KiB: k up to 7680 for 4-bit MinMax, 7936 for 2-bit and 4096 for NF4 at
 * m = 3..4; 15360, 15872 and 8192 at m = 2), each output row bit for bit what
 * m == 1 gives for that row of X -- except at m = 3..4 for a weight of
 * n > 13056 rows and k <= 4096, which takes the next kernel (faster there);
 * otherwise, up to m = 64, a bf16-MFMA kernel that streams the weight
 * once with K split over workgroups; larger m a bf16-MFMA GEMM whose weight
 * tiles are dequantized once into LDS. */
lbq_status lbq_linear_fwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                          int64_t m, uint16_t* Y, int64_t ldy, void* workspace,
                          size_t ws_bytes, void* stream);

/* Scratch memory, per device, of lbq_linear_fwd_noalloc: 16 MiB. */
#define LBQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* For callers that cannot allocate device memory (work captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of lbq_linear_fwd, the same kernels and the same results bit for bit
 * (except as noted below for m > 64), with no workspace argument.  The only scratch memory the forward uses (the fp32
 * K-split partial sums of the small-batch kernel, 2 <= m <= 64, and of a
 * GEMM that splits K, m > 64) lives in an array of LBQ_NOALLOC_SCRATCH_BYTES
 * in the library's device image, one per device, held until the process
 * ends; the call allocates and frees nothing.  Arguments, layouts and errors
 * as lbq_linear_fwd; LBQ_E_WORKSPACE when a call with m <= 64 would need
 * more scratch than the array holds (no shape does: at most 16.75 MB).  For
 * m > 64 a GEMM whose partials do not fit the array runs unsplit, as
 * lbq_linear_fwd does without a workspace (then the results agree with
 * lbq_linear_fwd given its workspace within fp32 rounding, not bit for
 * bit).  The array's device address is looked up on the
 * first call on a device that needs it; that call uses the current device
 * (which must be the stream's).  Every call on a device shares that device's
 * array: calls that overlap on one device (two streams or two host threads)
 * race and must be serialized by the caller. */
lbq_status lbq_linear_fwd_noalloc(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                                  int64_t m, uint16_t* Y, int64_t ldy, void* stream);

/* Largest count accepted by lbq_linear_fwd_grouped. */
#define LBQ_MAX_GROUP 8

/* Workspace bytes lbq_linear_fwd_grouped takes for m rows (0 when none). */
size_t lbq_linear_fwd_grouped_workspace_bytes(int32_t count, const lbq_desc* descs, int64_t m);

/* Forward of several frozen linears that read the same input X (the q, k and
 * v projections of an attention block, gate and up of an MLP, or the INT4 and
 * INT2 row sets of a channel-mixed layer, [GB] 模型量化):
 *   Ys[i] = X . deq(W_i)^T   for 0 <= i < count, each as in lbq_linear_fwd.
 * descs, qs, Ys, ldys: host arrays of `count` entries (1 <= count <=
 * LBQ_MAX_GROUP); every weight has the same k.  Several weights may scatter
 * (out_rows) into disjoint columns of one Y.  Every weight is checked as in
 * lbq_linear_fwd before anything is enqueued.  The weights of one kind run
 * in a single launch of the kernel lbq_linear_fwd picks for that m (one
 * launch per distinct kind, in order of first appearance: a GEMV streaming all
 * of them, the small-batch kernel over all their row tiles, or a GEMM whose
 * column tiles cover all of them); the small-batch kernel adds one launch
 * that sums its K-split partials.  For m > 64 a kind's GEMM may instead run
 * as two launches, a prefix of its weights and the rest, each with its own
 * tile shape, when that fills the chip's rounds of tiles better (q with
 * 256x256 tiles and k+v with 256x128 at m = 4096); when no weight of the
 * kind splits K, the two launches may also divide one weight at a multiple
 * of 256 rows (gate + up at m = 2048: the rows that fill three whole rounds
 * of 256x256 tiles, then the rest).  For m <= 64 a set made
 * of INT4 g128 and INT2 g64 weights only (the channel-mixed layer's two row
 * sets) runs as one launch for both formats: the GEMV at m == 1, the
 * multi-row GEMV at 2 <= m <= 4 when every weight takes it, else the
 * small-batch kernel (and its reduce).  Each Ys[i] equals what lbq_linear_fwd
 * writes for weight i alone, bit for bit (given workspaces of the queried
 * sizes: each weight splits K as it does alone).  `workspace` takes
 * lbq_linear_fwd_grouped_workspace_bytes(count, descs, m) bytes (16-byte
 * aligned; 0 for m == 1 and the multi-row GEMV): required for m <= 64,
 * optional for m > 64 as in lbq_linear_fwd. */
lbq_status lbq_linear_fwd_grouped(int32_t count, const lbq_desc* descs, const lbq_qtensor* qs,
                                  const uint16_t* X, int64_t m, uint16_t* const* Ys,
                                  const int64_t* ldys, void* workspace, size_t ws_bytes,
                                  void* stream);

/* Input gradient through the frozen weight, dX = dY . deq(W) ([QL]
 * QLoRA技术原理: gradients pass through the frozen 4-bit model):
 *   dX[i][k] = bf16( sum_j dY[i][j] * w_hat[j][k] ), fp32 accumulation.
 * dY: bf16 [m][n]; dX: bf16 [m][k] (device), both 16-byte aligned; n % 8
 * == 0; (m + 256) * n * 2 and (n + 256) * k below 2^32 (LBQ_E_SHAPE
 * otherwise).  out_rows must be NULL (LBQ_E_UNSUPPORTED otherwise). */
lbq_status lbq_linear_bwd_dx(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* dY,
                             int64_t m, uint16_t* dX, void* stream);

/* Input gradient of several frozen linears that read the same X (q, k and v;
 * gate and up), summed as the chain rule gives it for a shared input ([QL]
 * QLoRA技术原理: the gradient passes through each frozen 4-bit weight):
 *   dX = bf16( sum_i dYs[i] . deq(W_i) ), one fp32 accumulation over the
 * rows of all the weights, weight 0's first.  descs, qs, dYs: host arrays of
 * `count` entries (1 <= count <= LBQ_MAX_GROUP); the weights share one
 * format (LBQ_E_UNSUPPORTED otherwise) and k; dYs[i]: bf16 [m][n_i] (device);
 * dX: bf16 [m][k].  Each weight and dYs[i] are checked as in
 * lbq_linear_bwd_dx before anything is enqueued.  One launch.  When every
 * n_i but the last is a multiple of 64, dX equals lbq_linear_bwd_dx of the
 * weights stacked along n (with the dY blocks side by side), bit for bit. */
lbq_status lbq_linear_bwd_dx_grouped(int32_t count, const lbq_desc* descs, const lbq_qtensor* qs,
                                     const uint16_t* const* dYs, int64_t m, uint16_t* dX, void* stream);

/* Workspace bytes lbq_lora_bwd needs for m rows and rank r (0 for m <= 0). */
size_t lbq_lora_bwd_workspace_bytes(const lbq_desc* desc, int64_t m, int32_t r);

/* Backward of lbq_lora_fwd for a frozen quantized weight ([QL]
 * QLoRA技术原理: the gradient flows through the frozen 4-bit weight into the
 * low-rank adapters, which are the only trained parameters):
 *   G  = sigma * dY . B                  [m][r], rounded once to bf16
 *   dX = dY . deq(W) + G . A             bf16 [m][k]
 *   dA = G^T . X                         fp32 [r][k]
 *   dB = sigma * dY^T . (X . A^T)        fp32 [n][r]  (X . A^T rounded once to
 *                                         bf16, as in the forward)
 * X: bf16 [m][k], dY: bf16 [m][n], A: bf16 [r][k], B: bf16 [n][r] (device);
 * X, A, dY, dX 16-byte aligned, dA, dB 4-byte aligned; 1 <= r <= 64;
 * n % 64 == 0; the size limits of lbq_linear_bwd_dx and lbq_linear_fwd apply.
 * m == 0 writes zeros to dA and dB and nothing else.  `workspace` must hold
 * lbq_lora_bwd_workspace_bytes(desc, m, r) bytes (16-byte aligned).  dA and dB
 * are summed in a fixed order (run-to-run identical). */
lbq_status lbq_lora_bwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                        const uint16_t* dY, int64_t m, const uint16_t* A, const uint16_t* B,
                        int32_t r, float sigma, uint16_t* dX, float* dA, float* dB,
                        void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes lbq_lora_fwd needs for m rows and rank r. */
size_t lbq_lora_workspace_bytes(const lbq_desc* desc, int64_t m, int32_t r);

/* Forward with a LoRA branch ([BNB] step 4; [QL] QLoRA技术原理):
 *   Y = X . deq(W)^T + sigma * (X . A^T) . B^T,  sigma = lora_alpha / r.
 * A: bf16 [r][k], B: bf16 [n][r] (device), 1 <= r <= 64.  The adapter
 * product T = sigma * X . A^T is formed in fp32 and rounded once to bf16
 * before it meets B.  Other arguments as lbq_linear_fwd; `workspace` must
 * hold lbq_lora_workspace_bytes(desc, m, r) bytes. */
lbq_status lbq_lora_fwd(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                        int64_t m, const uint16_t* A, const uint16_t* B, int32_t r,
                        float sigma, uint16_t* Y, int64_t ldy, void* workspace,
                        size_t ws_bytes, void* stream);

/* ---- Serialization ([BNB] 源码纵深: the state dict saves the 4-bit weight
 * together with its quantization-state fields so that the layer can be rebuilt
 * exactly; section 量化数据的存储: the packed bytes are plain bytes, whatever
 * dtype holds them).  A blob is little-endian host memory:
 *   bytes  0..3   the characters "LBQ1"
 *          4..7   uint32 version, 1
 *          8..47  the lbq_desc
 *         48..95  six uint64 byte counts, as lbq_layout reports them, of
 *                 packed, scales, zeros, absmax, absmax_q, absmax_scale
 *         96..    those six buffers in that order, each starting at a
 *                 multiple of 16 bytes (zero padding in between)
 * out_rows belongs to a use of the weight, not to the weight, and is not
 * stored. */

/* Host only.  Bytes of the blob for `desc` (0 if `desc` is invalid). */
size_t lbq_serialized_bytes(const lbq_desc* desc);

/* Copies the weight's buffers (device) into `blob` (host, at least
 * lbq_serialized_bytes(desc) bytes) on `stream` and waits for the copies:
 * unlike the other device calls it returns only when `blob` is complete.
 * Errors: those of lbq_layout, LBQ_E_NULL, LBQ_E_SHAPE (blob too small),
 * LBQ_E_HIP. */
lbq_status lbq_serialize(const lbq_desc* desc, const lbq_qtensor* q, void* blob, size_t blob_bytes,
                         void* stream);

/* Host only.  Validates a blob's header and byte counts and writes its
 * descriptor to *desc, so that the caller can size the device buffers with
 * lbq_layout.  LBQ_E_FORMAT for a wrong magic, version, descriptor or byte
 * count, LBQ_E_SHAPE for a blob shorter than its contents. */
lbq_status lbq_blob_desc(const void* blob, size_t blob_bytes, lbq_desc* desc);

/* Copies a blob into the device buffers `q` (sized by lbq_layout of the
 * blob's descriptor) on `stream` and waits for the copies.  The restored
 * weight dequantizes and multiplies bit for bit like the serialized one.
 * Errors: those of lbq_blob_desc, LBQ_E_NULL, LBQ_E_ALIGN, LBQ_E_HIP. */
lbq_status lbq_deserialize(const void* blob, size_t blob_bytes, const lbq_qtensor* q, void* stream);

/* Host only.  The library's NF4 codebook (16 fp32 levels, ascending, with
 * c[0] = -1, c[7] = 0, c[15] = 1), computed by the library from normal
 * quantiles at evenly spaced probabilities [QL]. */
void lbq_nf4_codebook(float out[16]);

/* Host only.  Static text for a status code. */
const char* lbq_strerror(lbq_status s);

/* Host only.  Detail of the last failure on the calling thread ("" if none). */
const char* lbq_last_error_detail(void);

/* Host only.  Library version string. */
const char* lbq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LBQ_H */
