/*
 * bqd.h -- C ABI of libbqd.so, the MI355X (gfx950) W4A8 single-token decode
 * GEMV library.
 *
 * The operation, from the page "Jetson Orin AGX INT4 推理优化实践：super 分支
 * 从 9 tok/s 到 24 tok/s", section "从 FP 线性层到 INT4 DP4A 的数学推导"
 * (FP linear layer -> INT4 DP4A derivation):
 *
 *     y_j = s^W_j * s^x * sum_i q^W_ji * q^x_i + b_j
 *
 * with per-row INT4 weight codes q^W in [-8, 7] and scale s^W_j, a per-token
 * INT8 activation q^x in [-127, 127] with s^x = max_i |x_i| / 127, and an
 * exact int32 accumulator.  Variants from the page "在香橙派上跑 Gemma4：vLLM
 * 适配昇腾 310B 的内核开发实录": one fp16 scale per 32 weights (section 3.1),
 * an int8-expanded lm_head with fp16 group scales against fp16 activations
 * (section 3.2), and the M-token verification of speculative decoding
 * (section 5).
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are HIP device pointers owned by the caller;
 *     (host) pointers are ordinary host memory.  The library never allocates,
 *     frees, or keeps a reference to caller memory after the call returns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *     work is enqueued on it; calls return after enqueue, never synchronise.
 *   - Return value: BQD_OK (0) or a negative BQD_ERR_* code.  Arguments are
 *     validated on the host before anything is enqueued; on error nothing is
 *     launched.  Faults inside a launched kernel surface at the caller's
 *     next synchronisation, as for any HIP kernel.
 *   - Layouts are row-major.  Packed INT4: eight codes per uint32, code 0 of
 *     the eight in the least-significant nibble (word = [w7 ... w0], the page
 *     "Jetson Orin AGX INT4 ..." section "DP4A 做了什么"), each nibble the
 *     two's-complement low four bits of the code.  Row j of an [N, K] matrix
 *     is K/8 consecutive words.
 *   - K must be a positive multiple of 32 and at most BQD_MAX_K, except for
 *     gemv_w4a8, linear_w4a8, quantize_act and gemm_w4a8_verify (impl 0),
 *     which take any K % 8 == 0 up to BQD_MAX_K_ANY: shapes outside the
 *     first range run a general kernel (4-byte weight words, the activation
 *     read from memory, r and lanes_per_row not used); N >= 0
 *     (N == 0 or M == 0 enqueue nothing).  Packed weights, int8 activations
 *     and fp32/fp16 activation inputs must be 16-byte aligned; every other
 *     array 4-byte aligned (2-byte for fp16 arrays).
 *   - Only gfx950 devices are accepted (BQD_ERR_DEVICE otherwise).
 */
#ifndef BQD_H
#define BQD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQD_ABI_VERSION 4

#define BQD_OK 0
#define BQD_ERR_NULL (-1)      /* a required pointer is NULL                 */
#define BQD_ERR_SHAPE (-2)     /* N/M < 0, K <= 0, K % 32 (or 8) != 0, count */
#define BQD_ERR_ALIGN (-3)     /* a pointer violates its alignment           */
#define BQD_ERR_BOUND (-4)     /* K > BQD_MAX_K or M > BQD_MAX_TOKENS        */
#define BQD_ERR_DTYPE (-5)     /* unknown dtype or scale kind                */
#define BQD_ERR_CONFIG (-6)    /* unsupported r / lanes_per_row              */
#define BQD_ERR_LAUNCH (-7)    /* the HIP runtime rejected a launch          */
#define BQD_ERR_DEVICE (-8)    /* no HIP device, or not a gfx950 device      */

/* Buffers of one launch: an output of a per-token entry point (y, acc,
 * qx_out, sx_out, h_out, ...) may overlap neither another output of the same
 * call nor anything that call reads (weights, scales, bias, x, qx, sx, h,
 * delta, gamma): every workgroup reads the inputs while other workgroups
 * already write, so such a call is refused with BQD_ERR_SHAPE and nothing
 * launched.  add_rmsnorm_quant's h_out / y_out, which may equal h or delta
 * (each element is read before it is written by the same thread), and the
 * persistent pass's chaining rules below are the stated exceptions. */

#define BQD_F32 0              /* activation dtype: IEEE binary32            */
#define BQD_F16 1              /* activation dtype: IEEE binary16            */

#define BQD_SCALE_ROW_F32 0    /* float[N]: one fp32 scale per output row    */
#define BQD_SCALE_GROUP32_F16 1 /* uint16[N, K/32]: fp16 scale per 32 codes  */

/* Largest reduction length.  The int32 argument of the page "Jetson Orin AGX
 * INT4 ..." section "INT32 accumulator 是否安全" bounds each product by
 * 8 * 127 = 1016 and so allows K up to floor((2^31 - 1) / 1016) = 2,113,665;
 * the kernels stage the whole activation in 64 KiB of LDS, which is the
 * tighter limit. */
#define BQD_MAX_K 65536
/* Largest K of the entry points with a general path: the int32 bound above,
 * rounded down to a multiple of 8. */
#define BQD_MAX_K_ANY 2113664
/* Largest token count of gemm_w4a8_verify. */
#define BQD_MAX_TOKENS 16

/* Version of this header's ABI (BQD_ABI_VERSION). */
int bqd_abi_version(void);

/* Static, human-readable text for a status code.  Never NULL. */
const char* bqd_status_string(int status);

/* Checks that the current HIP device is a gfx950 and caches its properties.
 * Idempotent; every entry point calls it for the current device. */
int bqd_init(void);

/* ---------------------------------------------------------------------- */
/* Load-time weight preparation (not on the per-token path).               */
/* ---------------------------------------------------------------------- */

/* Per-row INT4 ("Jetson Orin AGX INT4 ...", derivation section):
 *   sw[j] = max_i |W[j,i]| / 7                      (fp32, correctly rounded)
 *   code  = clip(round_half_even(W[j,i] / sw[j]), -8, 7)   (fp32 division;
 *           every code of an all-zero row is 0)
 * W (device) fp32 [N, K]; wq (device) uint32 [N, K/8] packed; sw (device)
 * float [N].  W must be finite. */
int quantize_weights_int4_rowwise(const float* W, int32_t N, int32_t K,
                                  uint32_t* wq, float* sw, void* stream);

/* Q4_0-style group-32 INT4 ("在香橙派上跑 Gemma4 ...", section 3.1): per block of
 * 32 weights s = fp16_rne(max|W_block| / 7), codes taken against the stored
 * fp16 value, clip to [-8, 7].  wq (device) uint32 [N, K/8]; s16 (device)
 * uint16 fp16 bit patterns [N, K/32]. */
int quantize_weights_int4_group32(const float* W, int32_t N, int32_t K,
                                  uint32_t* wq, uint16_t* s16, void* stream);

/* int8-expanded lm_head ("在香橙派上跑 Gemma4 ...", section 3.2): per block of 32
 * weights s = fp16_rne(max|W_block| / 31), codes clip(round(W / s), -32, 31)
 * stored one per byte.  w8 (device) int8 [N, K]; s16 (device) uint16 [N, K/32]. */
int quantize_weights_int8_group32(const float* W, int32_t N, int32_t K,
                                  int8_t* w8, uint16_t* s16, void* stream);

/* Host helpers: pack int8 codes in [-8, 7] (host, [N, K]) into words (host,
 * [N, K/8]) and back.  K % 8 == 0 is enough here.  Out-of-range codes give
 * BQD_ERR_SHAPE with nothing written. */
int pack_int4_rows_host(const int8_t* q, int32_t N, int32_t K, uint32_t* out);
int unpack_int4_rows_host(const uint32_t* w, int32_t N, int32_t K, int8_t* out);

/* ---------------------------------------------------------------------- */
/* Per-token hot path.                                                     */
/* ---------------------------------------------------------------------- */

/* Dynamic per-token INT8 activation quantisation ("Jetson Orin AGX INT4 ...",
 * derivation section), one token per row of x:
 *   sx[m] = max_i |x[m,i]| / 127                     (fp32, correctly rounded)
 *   qx[m,i] = clip(round_half_even(x[m,i] / sx[m]), -127, 127)  (fp32 division;
 *             all zero when sx[m] == 0)
 * x (device) [M, K] of x_dtype (BQD_F32 or BQD_F16; fp16 is widened exactly);
 * qx (device) int8 [M, K]; sx (device) float [M].  x must be finite. */
int quantize_act(const void* x, int32_t x_dtype, int32_t M, int32_t K,
                 int8_t* qx, float* sx, void* stream);

/* Producers of a linear's activation fused with its quantisation ("Jetson
 * Orin AGX INT4 ...", section "后续还能继续优化什么", items 1 and 2, which name
 * the residual add, RMSNorm and SwiGLU as the next kernel boundaries to
 * remove and the quantisation as the step to fold into the operator before
 * the linear).  The page does not define the operators; the textbook forms
 * are used.  One workgroup per token reads the token once and writes the
 * int8 codes and scale directly; they equal quantize_act of the fp32 values
 * the same call writes to y_out / h_out.  Every fp32 value that decides a
 * code comes from a fixed sequence of IEEE operations, so results are
 * reproducible bit for bit.  K (or I) % 32 == 0 and <= BQD_MAX_PROD_K
 * (BQD_ERR_BOUND otherwise); M >= 0 tokens, any number. */
#define BQD_MAX_PROD_K 32768

/* Residual add + RMSNorm + per-token quantisation, per token m:
 *   h1 = h + delta                        (fp32; delta may be NULL)
 *   r  = fp32(1 / sqrt(sum_i h1_i^2 / K + eps))   (sum, root and division in
 *        binary64; a token with a zero denominator normalises to 0)
 *   y_i = (h1_i * r) * gamma_i            (two fp32 products)
 *   sx[m], qx[m, :] of y as quantize_act.
 * h, delta (device) float [M, K]; gamma (device) float [K]; eps >= 0 finite
 * (BQD_ERR_SHAPE otherwise); h_out, y_out (device) float [M, K] or NULL
 * (may equal h or delta); qx (device) int8 [M, K] or NULL; sx (device)
 * float [M], required with qx.  16-byte alignment for the arrays, 4 for sx.
 * Inputs must be finite and r finite (eps > 0 guarantees it). */
int add_rmsnorm_quant(const float* h, const float* delta, const float* gamma, float eps,
                      float* h_out, float* y_out, int8_t* qx, float* sx, int32_t M, int32_t K,
                      void* stream);

/* The same residual add + RMSNorm + quantisation folded into the prologue
 * of the W4A8 linear that consumes it (one launch instead of two): every
 * workgroup computes h1 = h + delta, r and the codes of (h1 * r) * gamma
 * itself -- the operations of add_rmsnorm_quant, so the same codes -- then
 * runs the GEMV of gemv_w4a8 on them; workgroup 0 writes h1 to h_out.
 *   y[j] = sw[j] * s^x * acc[j] + bias[j]
 * h, delta (NULL allowed), gamma, h_out (NULL allowed): device float [K],
 * 16-byte aligned; no output may overlap h, delta, gamma or another output
 * (BQD_ERR_SHAPE: other workgroups read them while workgroup 0 writes).  qx_out int8 [K], sx_out
 * float [1], acc int32 [N]: optional outputs.  K % 32 == 0 and K <= 8192
 * (BQD_ERR_BOUND); eps >= 0 finite.  r, lanes_per_row as in gemv_w4a8. */
int linear_rmsnorm_w4a8(const uint32_t* wq, const float* sw, const float* bias, const float* h,
                        const float* delta, const float* gamma, float eps, float* h_out, float* y,
                        int8_t* qx_out, float* sx_out, int32_t* acc, int32_t N, int32_t K, int32_t r,
                        int32_t lanes_per_row, void* stream);

/* SwiGLU + per-token quantisation.  gu (device) float [M, 2I] holds each
 * token's fused gate/up output, gate g = gu[m, 0:I] then up u = gu[m, I:2I];
 *   h_i = (g_i / (1 + e^(-g_i))) * u_i   (fp32, correctly rounded division;
 *   e^x by Cody-Waite reduction and a degree-7 Taylor polynomial, each step
 *   one IEEE fp32 operation, argument clamped to [-104, 89])
 *   sx[m], qx[m, :] of h as quantize_act.
 * h_out (device) float [M, I], required: it receives h, which the
 * quantisation then reads (two kernels on the stream: the elementwise part
 * spread over the chip, then the codes).  qx (device) int8 [M, I] or NULL
 * (h only); sx (device) float [M], required with qx.  Inputs must be
 * finite. */
int swiglu_quant(const float* gu, float* h_out, int8_t* qx, float* sx, int32_t M, int32_t I,
                 void* stream);

/* W4A8 GEMV over per-row scales ("Jetson Orin AGX INT4 ...", derivation and
 * "o2-all 和 o4-all 为什么能加速" sections):
 *   acc[j] = sum_i q^W[j,i] * qx[i]            (exact int32)
 *   y[j]   = (sw[j] * sx[0]) * acc[j] + bias[j] (fp32; bias may be NULL)
 * wq (device) uint32 [N, K/8]; sw, bias (device) float [N]; qx (device) int8
 * [K] with codes in [-127, 127]; sx (device) float [1]; y (device) float [N];
 * acc (device) int32 [N] or NULL (written only when given).
 * r: output rows each lane group accumulates at once, reusing every staged
 * activation chunk r times (the pages' "o-r" kernels): 1, 2, 4 or 8;
 * lanes_per_row: lanes that split one row's reduction, 16, 32 or 64;
 * 0 for either picks it from N and K. */
int gemv_w4a8(const uint32_t* wq, const float* sw, const float* bias,
              const int8_t* qx, const float* sx, float* y, int32_t* acc,
              int32_t N, int32_t K, int32_t r, int32_t lanes_per_row, void* stream);

/* One decode linear in one launch: the activation quantisation of
 * quantize_act folded into the prologue of gemv_w4a8 (every workgroup
 * quantises x itself, bit-identically), so no int8 copy of x goes through
 * memory.  x (device) [K] of x_dtype.  qx_out (device int8 [K]) and sx_out
 * (device float [1]) are optional copies of the quantised activation written
 * by one workgroup; acc as in gemv_w4a8.  With r = lanes_per_row = 0, up to
 * 8192 rows and K <= 24576 run in 1024-thread workgroups of one wave per row
 * (same bits). */
int linear_w4a8(const uint32_t* wq, const float* sw, const float* bias,
                const void* x, int32_t x_dtype, float* y, int8_t* qx_out,
                float* sx_out, int32_t* acc, int32_t N, int32_t K, int32_t r,
                int32_t lanes_per_row, void* stream);

/* Group-32 W4A8 GEMV ("在香橙派上跑 Gemma4 ...", section 3.1 format with the
 * INT8 activation of "Jetson Orin AGX INT4 ..."):
 *   acc_g[j,g] = sum_{i in block g} q^W[j,i] * qx[i]            (exact int32)
 *   y[j] = sx[0] * sum_g fp32(s16[j,g]) * acc_g[j,g] + bias[j]   (fp32)
 * s16 (device) uint16 fp16 [N, K/32]; acc_g (device) int32 [N, K/32] or
 * NULL; other arguments as in gemv_w4a8. */
int gemv_w4a8_group32(const uint32_t* wq, const uint16_t* s16, const float* bias,
                      const int8_t* qx, const float* sx, float* y, int32_t* acc_g,
                      int32_t N, int32_t K, int32_t r, int32_t lanes_per_row,
                      void* stream);

/* linear_w4a8 for group-32 weights: quantise x in the prologue, then
 * gemv_w4a8_group32.  qx_out, sx_out, acc_g optional. */
int linear_w4a8_group32(const uint32_t* wq, const uint16_t* s16, const float* bias,
                        const void* x, int32_t x_dtype, float* y, int8_t* qx_out,
                        float* sx_out, int32_t* acc_g, int32_t N, int32_t K, int32_t r,
                        int32_t lanes_per_row, void* stream);

/* W8A16 lm_head ("在香橙派上跑 Gemma4 ...", section 3.2): int8 codes times fp16
 * group scales against fp16 activations, fp32 accumulation:
 *   y[j] = sum_g fp32(s16[j,g]) * sum_{i in block g} w8[j,i] * fp32(x16[i])
 * w8 (device) int8 [N, K] (codes in [-32, 31]); s16 (device) uint16 [N, K/32];
 * x16 (device) uint16 fp16 [K] (finite); y (device) float [N]. */
int gemv_w8a16_group32(const int8_t* w8, const uint16_t* s16, const uint16_t* x16,
                       float* y, int32_t N, int32_t K, int32_t r,
                       int32_t lanes_per_row, void* stream);

/* Packed 6-bit lm_head ("在香橙派上跑 Gemma4 ...", section 3.2: a Q6_K weight
 * stores 256 weights in 210 bytes -- 4-bit low and 2-bit high fields of each
 * code, an int8 scale per 16 weights, an fp16 scale per 256 -- and the page
 * expands it to int8 at load time because decoding the fields was vector-
 * instruction bound on its chip).  The quantiser and the layout are this
 * library's own.  Per row (K % 256 == 0), as separate arrays:
 *   ql [N, K/2] uint8: low nibble of u = q + 32 in byte i/2 (bits 0-3 for
 *      even i, 4-7 for odd i);
 *   qh [N, K/4] uint8: per 16 weights a little-endian uint32; weight 8k + e
 *      (k in {0, 1}, e in 0..7) puts bits 4-5 of u at bit
 *      2(e mod 4) + 8k + 16[e >= 4];
 *   sc [N, K/16] int8 sub-block scales; d [N, K/256] fp16 super-block scales.
 * Value of weight i: d * sc[i/16] * q_i, q in [-32, 31]. */

/* Load-time quantisation: per 16 weights t = max|w| / 31; per 256 weights
 * d = fp16_rne(max t / 127); sc = clip(round(t / d), 0, 127); codes
 * q = clip(round(w / (d * sc)), -32, 31) (fp32 divisions, round half to even;
 * a zero scale gives zero codes).  W (device) float [N, K], 16-byte aligned;
 * ql 8-, qh 4-, d 2-byte aligned.  K <= BQD_MAX_K. */
int quantize_weights_q6k(const float* W, int32_t N, int32_t K, uint8_t* ql, uint8_t* qh,
                         int8_t* sc, uint16_t* d, void* stream);

/* y[j] = sum over 16-weight sub-blocks s of fp32(d) * sc_s * sum_{i in s} q_i * x16[i]
 * (fp32 accumulation), the codes decoded from the packed fields in registers.
 * x16 (device) fp16 bits [K], 16-byte aligned; y (device) float [N]; ql and
 * qh 16-, sc 4-, d 2-byte aligned (true for row-major arrays from aligned
 * bases).  K <= 32768.  r, lanes_per_row as in gemv_w4a8, and lanes_per_row
 * may also be 8 (0 = 2 rows, 8 lanes). */
int gemv_q6k_f16(const uint8_t* ql, const uint8_t* qh, const int8_t* sc, const uint16_t* d,
                 const uint16_t* x16, float* y, int32_t N, int32_t K, int32_t r,
                 int32_t lanes_per_row, void* stream);

/* INT8-X (3,5,8): lossless INT8 weights ("定長無損 INT8 壓縮與 Triton 融合解碼",
 * sections 2.1-2.5) over the row-major flattened tensor of n weights:
 *   level 1 |v| <= 3: 3-bit two's complement code in the L1 stream;
 *   level 2 |v| <= 15: 5-bit code in the L2 stream; level 3: the byte in L3;
 *   B1: a bit per weight, 1 = not level 1; B2: a bit per non-level-1 weight
 *   in order, 1 = level 3; b1_blk[b] / b2_blk[b]: set bits of B1 / B2 before
 *   block b of BQD_INT8X_BLOCK weights (one extra entry holds the totals).
 * Bit streams are LSB-first (bit p = bit p % 32 of word p / 32). */
#define BQD_INT8X_BLOCK 512

/* Host: weights of each level, counts[3] = {n1, n2, n3}. */
int int8x_counts_host(const int8_t* q, int64_t n, int64_t* counts);

/* Host: byte sizes of the seven arrays {b1, b2, l1, l2, l3, b1_blk, b2_blk}
 * for n weights with the given level counts, the bit streams padded by
 * three words for the decoder's read windows. */
int int8x_stream_bytes_host(int64_t n, const int64_t* counts, int64_t* bytes);

/* Host: encode q (host int8, n weights) into host arrays of the sizes
 * above (zeroed here first).  Offline, once per tensor. */
int int8x_encode_host(const int8_t* q, int64_t n, uint32_t* b1, uint32_t* b2, uint32_t* l1,
                      uint32_t* l2, uint8_t* l3, int32_t* b1_blk, int32_t* b2_blk);

/* W8A8 GEMV over INT8-X weights [N, K] (K % BQD_INT8X_BLOCK == 0), decoded
 * in registers (the fused decode of section 2.4):
 *   acc[j] = sum_i q[j,i] * qx[i] (exact int32);  y[j] = (sw * sx[0]) * acc[j]
 * with one per-tensor weight scale sw (section 2.5: INT8 per-tensor).  The
 * seven arrays (device, 4-byte aligned) hold what int8x_encode_host wrote;
 * stream_bytes (host, [7]) their sizes from int8x_stream_bytes_host (reads
 * are clamped to them; the block sums must hold N*K/BQD_INT8X_BLOCK + 1
 * entries).  qx (device) int8 [K], 8-byte aligned; sx (device)
 * float [1]; y (device) float [N]; acc (device) int32 [N] or NULL.  rows =
 * rows per workgroup, 1, 2, 4 or 8, or 0 (4 from N = 8192 on, else 1).  N*K < 2^31 and each stream below
 * 2^26 words (BQD_ERR_BOUND otherwise). */
int gemv_int8x(const uint32_t* b1, const uint32_t* b2, const uint32_t* l1, const uint32_t* l2,
               const uint8_t* l3, const int32_t* b1_blk, const int32_t* b2_blk,
               const int64_t* stream_bytes, const int8_t* qx, const float* sx, float sw, float* y,
               int32_t* acc, int32_t N, int32_t K, int32_t rows, void* stream);

/* W4A16 comparison GEMV: the same packed per-row INT4 weights against an
 * fp16 activation, unpacked to fp16 and multiplied in floating point (the
 * route "Jetson Orin AGX INT4 ..." section "为什么 INT4 float 解包不快"
 * weighs against the integer dot; "在香橙派上跑 Gemma4 ..." section 3.1
 * dequantises to fp16 for fp16 MACs):
 *   y[j] = sw[j] * sum_i q^W[j,i] * x[i] + bias[j]   (fp32 accumulation)
 * wq (device) uint32 [N, K/8]; sw, bias (device) float [N] (bias may be
 * NULL); x16 (device) uint16 fp16 bit patterns [K], 16-byte aligned;
 * y (device) float [N].  K <= 32768.  r, lanes_per_row as in gemv_w4a8,
 * except that 0 picks 64 lanes and 2 rows per lane group when N >= 16384,
 * else 1. */
int gemv_w4a16(const uint32_t* wq, const float* sw, const float* bias, const uint16_t* x16, float* y,
               int32_t N, int32_t K, int32_t r, int32_t lanes_per_row, void* stream);

/* M-token verification ("在香橙派上跑 Gemma4 ...", section 5): one pass over the
 * weights serves M quantised tokens.
 *   acc[m,j] = sum_i q^W[j,i] * qx[m,i],  y[m,j] = (sw[j] * sx[m]) * acc[m,j] + bias[j]
 * qx (device) int8 [M, K]; sx (device) float [M]; y (device) float [M, N];
 * acc (device) int32 [M, N] or NULL.  1 <= M <= BQD_MAX_TOKENS.
 * impl: 1 integer dot-product kernel (v_dot4_i32_i8); 2 matrix-core
 * kernel (v_mfma_i32_16x16x64_i8, 16 token columns), every workgroup
 * staging all K of the tokens' codes; 3 the same matrix-core arithmetic in
 * balanced blocks: one block per workgroup, a range of 16-row tiles times a
 * K slice with about the same number of weights in each, only the slice's
 * codes staged.  When the K range is split, each slice's exact int32
 * partials go through the workspace and the slice that started a tile last
 * adds them and writes y (it waits only for slices that have already
 * started, so no wait depends on which workgroups are resident together).
 * 0 automatic: M = 1 runs gemv_w4a8's kernel; M >= 2 impl 3 when the
 * shape needs no workspace or the given one suffices, else impl 2.  Every
 * impl gives the same acc and y bits.
 * workspace (device, 256-byte aligned) of workspace_bytes bytes, or NULL /
 * 0: needed by impl 3 when gemm_w4a8_verify_workspace_bytes reports more
 * than 0 for the shape (impl 3 refuses a NULL one with BQD_ERR_NULL and a
 * smaller one with BQD_ERR_BOUND).  Zero-filled once by the caller; every
 * call leaves it zeroed again.  Calls that share a workspace must not
 * overlap in time. */
int gemm_w4a8_verify(const uint32_t* wq, const float* sw, const float* bias,
                     const int8_t* qx, const float* sx, float* y, int32_t* acc,
                     int32_t M, int32_t N, int32_t K, int32_t impl, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Bytes of workspace gemm_w4a8_verify's impl 3 needs for M tokens over
 * [N, K] on the current device: 0 when it splits no tile's K range (or for
 * invalid shapes, or without a gfx950 device). */
size_t gemm_w4a8_verify_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* One linear of a decoder layer, as handed to layer_w4a8_forward.  The
 * struct lives in host memory; its pointers are device pointers. */
typedef struct bqd_linear_w4a8 {
    const uint32_t* wq;    /* packed codes [N, K/8]                         */
    const void* scales;    /* float[N] or uint16 fp16 [N, K/32]             */
    const float* bias;     /* [N] or NULL                                   */
    int32_t N;
    int32_t K;
    int32_t scale_kind;    /* BQD_SCALE_ROW_F32 or BQD_SCALE_GROUP32_F16    */
    int32_t r;             /* as in gemv_w4a8; 0 = automatic                */
    int32_t lanes_per_row; /* as in gemv_w4a8; 0 = automatic                */
} bqd_linear_w4a8;

/* The linears of one decoder layer in order on one stream, each one launch
 * of linear_w4a8 / linear_w4a8_group32 (quantise x[i], GEMV into y[i]).
 * With q/k/v and gate/up rows concatenated at load time ("在香橙派上跑 Gemma4
 * ...", section 3.1) a layer is 4 linears and 4 launches.  lin (host) [n];
 * x (host) array of n device pointers to [K_i] activations of x_dtype;
 * y (host) array of n device pointers to float [N_i].  0 <= n <= 64.
 * y[i] may not overlap x[i] or linear i's weights, scales or bias; it may
 * be a later linear's x (the launches run in order on the stream). */
int layer_w4a8_forward(const bqd_linear_w4a8* lin, int32_t n, const void* const* x,
                       int32_t x_dtype, float* const* y, void* stream);

/* ---------------------------------------------------------------------- */
/* Persistent token pass                                                   */
/* ---------------------------------------------------------------------- */

/* Most linears one pass may hold (a Qwen2-7B-shaped decoder has 113). */
#define BQD_MAX_PASS_LINEARS 4096
/* Largest K of a linear in a pass: a workgroup keeps the fp32 activation
 * and its int8 codes in LDS (5 bytes per element of 160 KiB). */
#define BQD_MAX_PASS_K 24576

/* Bytes of the descriptors decode_pass_encode writes for n linears. */
size_t decode_pass_desc_bytes(int32_t n);

/* Validates n per-row linears (bqd_linear_w4a8 with BQD_SCALE_ROW_F32 and
 * r = lanes_per_row = 0: the pass chooses its own work split) with their
 * activation x[i] (device, [K_i] of x_dtype) and output y[i] (device float
 * [N_i], N_i > 0), and serialises them into desc_host (host,
 * decode_pass_desc_bytes(n) bytes) for the current device: the work split
 * is encoded for the grid the launch will use there, so a device must be
 * current (BQD_ERR_DEVICE otherwise).  *max_k receives the largest K,
 * *sync_bytes the size of the workspace decode_pass_w4a8 needs and *slots
 * the 16-byte chunks per lane of each pipeline step, which selects the
 * kernel instance: 4 when every linear is group-32 (small shares per
 * compute unit: a step's fixed work is on each link's critical path), else
 * 8.  The launch takes all three back unchanged.
 * K_i % 32 == 0 and K_i <= BQD_MAX_PASS_K (BQD_ERR_BOUND otherwise).
 * Where each activation comes from:
 *   - x[i] overlaps no output: it was written before the launch and is read
 *     with no wait;
 *   - x[i] lies inside the output y[k] of an earlier linear (k < i; a
 *     decoder's chain, "从 FP 线性层到 INT4 DP4A 的数学推导" of the Jetson
 *     Orin page: each linear's input derives from the previous output): it
 *     is read from the pass's own exchange once y[k]'s rows are written.
 *     x_dtype must then be BQD_F32 (BQD_ERR_DTYPE) and x[i] 4-byte aligned
 *     within y[k] (BQD_ERR_ALIGN).
 * Refused with BQD_ERR_SHAPE: x[i] overlapping y[k] for k >= i or two
 * outputs, or not contained in the one it overlaps; outputs overlapping
 * each other or any linear's weights, scales or bias.  (Workgroups run
 * ahead of each other wherever no data dependency holds them, so an output
 * is written exactly once and never over anything the pass reads.)  The
 * caller copies desc_host unchanged to 16-byte-aligned device memory
 * before decode_pass_w4a8 reads it. */
int decode_pass_encode(const bqd_linear_w4a8* lin, int32_t n, const void* const* x, int32_t x_dtype,
                       float* const* y, void* desc_host, size_t desc_bytes, int32_t* max_k,
                       size_t* sync_bytes, int32_t* slots);

/* One decode step over the n encoded linears in order, in one launch of one
 * workgroup per compute unit, all resident at once: for each linear, the activation quantisation of quantize_act and
 * the GEMV of gemv_w4a8 (same codes, same y bits as linear_w4a8).  A linear
 * whose activation is an earlier linear's output waits for exactly those
 * values: each output row read later in the pass is also stored into an
 * exchange in sync_dev, and the readers poll the words they need (one
 * device-scope store and one device-scope load per dependency, no counters
 * or fences).  Weights of the next linear are prefetched while waiting.
 * desc_dev (device) holds the encoded descriptors; max_k and slots are the
 * values decode_pass_encode reported (slots 4 or 8, else BQD_ERR_CONFIG;
 * descriptors encoded for the other instance set bit 1 in the kernel);
 * sync_dev (device, 256-byte aligned) is the
 * workspace of *sync_bytes bytes it reported, zero-filled once by the
 * caller (sync_bytes: that size, which bounds what the kernel may
 * touch; descriptors needing more are refused in the kernel with bit 1)
 * and then handed unchanged to every pass over the same descriptors (each pass leaves it ready for the next; zero it again
 * before using it with other descriptors).  Passes over one workspace must
 * not overlap in time.  An output row equal to the NaN bit pattern
 * 0xFFFFFFFF cannot be passed on (its exchange word would read as "not
 * written"); finite inputs never produce it.  spin_limit bounds each wait
 * (0 = default: 2^21 polling rounds, about 2 s); a wait that runs out sets bit 0 of
 * sync_dev[0] and proceeds with what it read, so the kernel always ends;
 * bit 1 is set (and nothing computed) when the descriptors were encoded
 * for another grid, another n or another slots.  The caller reads sync_dev[0] to check,
 * and clears it to reuse. */
int decode_pass_w4a8(const void* desc_dev, int32_t n, int32_t max_k, int32_t slots, uint32_t* sync_dev,
                     size_t sync_bytes, int32_t spin_limit, void* stream);

/* Largest workspace decode_pass_w4a8_static holds: 16 MiB of device memory
 * per GPU the library runs on (a 28-layer Qwen2-7B-shaped chained pass with
 * its lm_head needs about 11 MiB). */
#define BQD_STATIC_PASS_BYTES 16777216 /* 16 MiB */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the pass
 * of decode_pass_w4a8 with its workspace in a static device array the
 * library holds per GPU, instead of a caller's sync_dev.  sync_bytes is
 * the size decode_pass_encode reported (BQD_ERR_BOUND above
 * BQD_STATIC_PASS_BYTES; BQD_ERR_SHAPE if it is not a workspace size).
 * Each call first zero-fills that much of the array with a kernel on
 * `stream` (the array keeps the last call's contents, whatever descriptors
 * it ran), then runs the pass, then copies the pass's error word (bits as
 * in decode_pass_w4a8) to err_dev (device, one uint32).  Nothing is
 * allocated.  All calls on one GPU share its array: calls that overlap in
 * time on one GPU (other streams, other threads) race and give wrong
 * results, so callers serialise them.  Launch errors and argument checks as
 * in decode_pass_w4a8; BQD_ERR_LAUNCH also if the array's address could
 * not be found on this GPU. */
int decode_pass_w4a8_static(const void* desc_dev, int32_t n, int32_t max_k, int32_t slots, size_t sync_bytes,
                            int32_t spin_limit, uint32_t* err_dev, void* stream);

/* ---------------------------------------------------------------------- */
/* Measurement                                                             */
/* ---------------------------------------------------------------------- */

/* Streaming read of buf (device, bytes % 16 == 0, 16-byte aligned): the
 * reference kernel whose bandwidth is the measured read ceiling the GEMV
 * rooflines are compared with ("在香橙派上跑 Gemma4 ..." section 4.1 sets the
 * decode bound by the measured read bandwidth).  grid workgroups of 256
 * threads, unroll in {1, 4, 8} 16-byte loads in flight per thread; sink
 * (device) receives one uint32 per workgroup (an XOR of what it read). */
int read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, int32_t unroll, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BQD_H */
