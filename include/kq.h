/*
 * kq.h — C ABI of the KroQuant online activation quantizer for AMD gfx950
 * (MI350 / MI355X).
 *
 * What it computes.  For every token row t of a linear-layer input X[T][d] and
 * every 32-channel block b (channels 32b .. 32b+31), the block is multiplied by
 * its own invertible 32x32 transform T_b and the result is encoded as MXFP4:
 * 32 E2M1 codes sharing one E8M0 scale.
 *   - KroQuant abstract (arXiv 2607.21446): one learned Kronecker-structured
 *     invertible transform per 32-element activation block, applied online
 *     before W4A4 (MXFP4) quantization; its inverse is folded into the weights;
 *     per-channel scaling (SmoothQuant) is the cheap comparison transform.
 *   - KroQuant researchpod summary, method paragraph: T_b is the Kronecker
 *     product of five 2x2 unit-determinant LU-decomposed factors.
 *   - OCP Microscaling Formats (MX) v1.0: MXFP4 element and scale encodings.
 *
 * Conventions fixed by this library (the pages leave them open):
 *   factor   F = L*U, L = [[1,0],[l,1]], U = [[u,v],[0,1/u]]   (det F = 1)
 *   params   float32 [nb][5][3] = (l, u, v) for F1..F5 of each block
 *   T_b      = F1 (x) F2 (x) F3 (x) F4 (x) F5; F1 acts on bit 4 of the within-block
 *            index i (stride 16), F5 on bit 0 (stride 1)
 *   y_b      = T_b * x_b   (so a consumer's weights take W_b * T_b^-1)
 *   scale    e = clamp(floor(log2(max_i |y_i|)) - 2, -127, 127), byte S = e + 127;
 *            an all-zero block gives S = 0; a block holding NaN or Inf gives
 *            S = 0xFF and all-zero codes
 *   codes    |y_i| / 2^e rounded to the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}
 *            (midpoints to the even code, above 6 saturates to 6); bit 3 is the
 *            sign of y_i, so a negative value that rounds to zero encodes as 0x8
 *   layout   Q: uint8 [T][ldq], byte 16b + i/2 of row t holds channel 32b+i, even i
 *            in the low nibble; S: uint8 [T][lds], byte b of row t is the block's
 *            E8M0 scale; X and Q/S are row-major with the given row pitches
 *
 * Calling rules shared by every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronizes; each call enqueues work on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *     returns without waiting.
 *   - Arguments are checked on the host before any HIP call; a rejected call
 *     returns a negative kq_status and enqueues nothing.  KQ_ERR_HIP means a
 *     launch failed; kq_last_hip_error() gives the hipError_t (per thread).
 *     Nothing is printed and no exception crosses the ABI.
 *   - rows == 0 is a no-op that returns KQ_OK.  rows < 2^31; d must be a positive
 *     multiple of 32 and at most 2^27 (2^22 blocks); every row pitch must be below
 *     4 GiB.  x, q and their row pitches (in bytes) must be 16-byte aligned.
 *   - Factor parameters must be finite with u != 0; otherwise the output is
 *     unspecified (checking would cost a device pass).  Inputs are expected to be
 *     finite; the NaN/Inf scale rule above is best effort.
 *   - Calls are reentrant and thread-safe; the only global state is a per-device
 *     cache of the compute-unit count.
 */
#ifndef KQ_H
#define KQ_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KQ_OK = 0,
  KQ_ERR_NULL = -1,     /* a required pointer is NULL                       */
  KQ_ERR_SHAPE = -2,    /* rows negative or >= 2^31, d not a positive
                           multiple of 32 (or above 2^27), a pitch smaller
                           than the row or of 4 GiB and more                 */
  KQ_ERR_ALIGN = -3,    /* x, q (or a pitch in bytes) not 16-byte aligned   */
  KQ_ERR_DTYPE = -4,    /* unknown input dtype                              */
  KQ_ERR_FORMAT = -5,   /* unknown transform format, or one the variant
                           cannot consume                                    */
  KQ_ERR_VARIANT = -6,  /* unknown variant                                  */
  KQ_ERR_HIP = -7,      /* a HIP call failed                                */
  KQ_ERR_VALUE = -8     /* a scalar argument out of range (eps, a workspace
                           size)                                            */
} kq_status;

typedef enum { KQ_BF16 = 0, KQ_FP32 = 1 } kq_dtype;

/* Transform formats.  Element counts per block: PARAMS 15 floats, DENSE_F32
 * 1024 floats, DENSE_BF16X3 3 x 1024 bf16, FACTORS_2X2_F32 20 floats. */
typedef enum {
  KQ_T_PARAMS = 0,        /* float32 [nb][5][3] (l,u,v): the factors' parameters  */
  KQ_T_DENSE_F32 = 1,     /* float32 [nb][32][32]: T_b[i][j] row-major            */
  KQ_T_DENSE_BF16X3 = 2,  /* bf16 [3][nb][32][32]: hi, mid, lo with
                             hi + mid + lo == fp32(T_b) (each the bf16 rounding of
                             what the previous parts leave)                       */
  KQ_T_FACTORS_2X2_F32 = 3  /* float32 [nb][5][2][2]: F_k = L_k U_k =
                             [[u, v], [l u, l v + 1/u]] row-major; an expansion
                             output only (no quantize entry point reads it)       */
} kq_tfmt;

typedef enum {
  KQ_AUTO = 0,       /* BUTTERFLY for KQ_T_PARAMS, MFMA for KQ_T_DENSE_BF16X3     */
  KQ_BUTTERFLY = 1,  /* fp32 in-register factored transform; needs KQ_T_PARAMS   */
  KQ_MFMA = 2        /* per-block 32x32 bf16 matrix-core product with fp32
                        accumulation over the 3-way split T; needs
                        KQ_T_DENSE_BF16X3                                         */
} kq_variant;

/* Expand factor parameters into a transform format (the work the abstract
 * describes as folding the block structure into small GEMMs).
 *   params  device float32 [nb][5][3]
 *   nb      number of 32-channel blocks (>= 0; 0 is a no-op)
 *   tfmt    KQ_T_DENSE_F32, KQ_T_DENSE_BF16X3 or KQ_T_FACTORS_2X2_F32
 *           (KQ_T_PARAMS is rejected: it needs no expansion)
 *   t_out   device buffer of the format's size (see kq_tfmt)
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE (nb < 0), KQ_ERR_FORMAT, KQ_ERR_HIP. */
int kq_expand_factors(const float* params, int64_t nb, int tfmt, void* t_out, void* stream);

/* Transform each 32-channel block of every row and encode it as MXFP4.
 *   x       device [rows][ldx] of dtype (bf16 held as 16-bit words, or float32)
 *   rows    token rows (>= 0); d channels (multiple of 32); ldx row pitch in
 *           elements (>= d)
 *   t, tfmt the transform in one of the kq_tfmt formats, nb = d/32 blocks
 *   q       device uint8 [rows][ldq], ldq >= d/2 bytes
 *   s       device uint8 [rows][lds], lds >= d/32 bytes
 *   variant kq_variant
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_DTYPE, KQ_ERR_FORMAT,
 *         KQ_ERR_VARIANT, KQ_ERR_HIP. */
int kq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                const void* t, int tfmt, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                int variant, void* stream);

/* SmoothQuant baseline on the same memory skeleton: y[t][c] = x[t][c] * mult[c]
 * (mult = 1/s_c in float32, the per-channel smoothing the abstract compares
 * against), then the same MXFP4 encoding and layout as kq_quantize.
 *   mult    device float32 [d], 16-byte aligned (KQ_ERR_ALIGN otherwise)
 * Errors: as kq_quantize (KQ_ERR_FORMAT and KQ_ERR_VARIANT never occur). */
int sq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                const float* mult, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                void* stream);

/* Validation entry: kq_quantize from the same kernels, additionally writing the
 * float32 pre-quantization values y into y [rows][ldy] (ldy >= d elements, any
 * 4-byte-aligned pointer).  Slower; not for production use. */
int kq_transform_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       const void* t, int tfmt, uint8_t* q, int64_t ldq, uint8_t* s,
                       int64_t lds, int variant, float* y, int64_t ldy, void* stream);

/* Same for the SmoothQuant baseline. */
int sq_transform_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       const float* mult, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                       float* y, int64_t ldy, void* stream);

/* Weight side (KroQuant abstract: the inverse of each block transform is folded
 * into the weights, so a layer computes W' (T x) = W x).  For a weight matrix
 * W[N][d] of a linear layer y = W x, row r becomes w'_r = w_r T^-1 per 32-channel
 * block (w'_rb = T_b^-T w_rb as a column), and is encoded as MXFP4 along d with the
 * same scale rule, codes and layout as kq_quantize (blocks of 32 input channels).
 *   w       device [rows][ldw] of dtype; rows = N output channels; ldw in elements
 *   params  device float32 [d/32][5][3], the same factors the activations use
 *   q, s    as in kq_quantize
 * The transform runs in fp32 from the factors: diag(1/d_i), then the lower shears
 * by -u_k v_k, then the upper shears by -l_k (the mixed-product split of
 * F^-T = L^-T U^-T).  Usually run once per learned transform, not per token.
 * Errors: as sq_quantize. */
int kq_quantize_weights(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                        const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                        void* stream);

/* Validation entry of kq_quantize_weights: also writes the float32 W' (before
 * quantization) into y [rows][ldy] (ldy >= d elements, 4-byte aligned). */
int kq_weights_debug(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                     const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                     float* y, int64_t ldy, void* stream);

/* Fixed block-Hadamard comparison transform (KroQuant abstract: fixed Hadamard
 * rotations quantize well but are the costly alternative at large blocks): here
 * at the same 32-channel blocks, y_b = H x_b / sqrt(32) with the Sylvester matrix
 * H[i][j] = (-1)^popcount(i & j), then the same MXFP4 encoding and layout as
 * kq_quantize.  H / sqrt(32) is symmetric and orthogonal, so a layer's weights
 * take this same call.  Computed in fp32: five add/subtract stages, then one
 * multiply by fp32(1/sqrt(32)).
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_DTYPE, KQ_ERR_HIP. */
int hq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, uint8_t* q,
                int64_t ldq, uint8_t* s, int64_t lds, void* stream);

/* Validation entry of hq_quantize: also writes the float32 transformed values
 * into y [rows][ldy] (ldy >= d elements, 4-byte aligned). */
int hq_transform_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y, int64_t ldy,
                       void* stream);

/* Normalization fused ahead of the quantizer (KroQuant abstract: the
 * normalization layers between blocks are what force the transform to run online
 * at every step).  For every row t of the pre-normalization activations x:
 *   mu, var = mean and biased variance of x[t][0 .. d-1];  rstd = 1/sqrt(var + eps)
 *   h[t][c] = (x[t][c] - mu) * rstd * (1 + scale[g][c]) + shift[g][c],  g = t / rows_per_sample
 * (LayerNorm without affine parameters followed by the adaptive-norm modulation of
 * a DiT block), then y_b = T_b h_b and the MXFP4 encoding, as kq_quantize.  The
 * row is read from HBM once; nothing intermediate is written.
 *   shift, scale     device float32 [ceil(rows / rows_per_sample)][d], 16-byte
 *                    aligned; both NULL for a plain LayerNorm (one NULL alone is
 *                    KQ_ERR_NULL)
 *   rows_per_sample  rows (tokens) per modulation vector, >= 1
 *   eps              >= 0, finite (KQ_ERR_VALUE otherwise)
 *   params           device float32 [d/32][5][3] (KQ_T_PARAMS format)
 * d is at most 16384 here (a row's d/32 blocks, one per lane, must fit in one
 * workgroup of 512 lanes; KQ_ERR_SHAPE beyond).
 * Computed in fp32: the row mean from a sum reduction, then the variance from the
 * same reduction of the squared deviations (both in a fixed order, so the result
 * is deterministic); the modulation folded into the transform's diagonal plus a
 * constant T_b shift.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_DTYPE, KQ_ERR_VALUE, KQ_ERR_HIP. */
int kq_norm_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                     const float* shift, const float* scale, int64_t rows_per_sample, float eps,
                     const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                     void* stream);

/* Validation entry of kq_norm_quantize: also writes the float32 y (after the
 * transform, before quantization) into y [rows][ldy] (ldy >= d, 4-byte aligned). */
int kq_norm_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                  const float* shift, const float* scale, int64_t rows_per_sample, float eps,
                  const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y,
                  int64_t ldy, void* stream);

/* The W4A4 product that consumes the quantizer's outputs (KroQuant abstract:
 * W4A4 with MXFP4 activations; the transform's inverse sits in the weights):
 *   out[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k],   deq = E2M1(code) * 2^(S - 127)
 * A: activations as kq_quantize / kq_norm_quantize write them, qa uint8 [M][lda]
 *    codes (lda >= K/2 bytes) and sa uint8 [M][ldsa] E8M0 scales (ldsa >= K/32);
 * B: weights as kq_quantize_weights writes them, qb [N][ldb], sb [N][ldsb].
 * out: [M][ldo] (ldo >= N elements) of out_dtype KQ_FP32 or KQ_BF16 (round to
 * nearest even from the fp32 accumulation).  K: multiple of 32.  qa, qb and their
 * pitches 16-byte aligned; lda and ldb below 2^24 bytes (KQ_ERR_SHAPE otherwise).
 * Runs on the gfx950 scaled matrix cores
 * (fp4 x fp4 with per-32 E8M0 scales, fp32 accumulation); scale bytes 0xFF (NaN)
 * give unspecified results.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_DTYPE, KQ_ERR_HIP. */
int kq_mx_gemm(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
               const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
               int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* stream);

/* The W4A4 product with the quantizer in its prologue (KroQuant abstract: the
 * online transform feeds the W4A4 MXFP4 product):
 *   out[m][n] = sum_k deq(Q(T X))[m][k] * deq(B)[n][k]
 * X: bf16 [M][ldx] activations (dtype KQ_BF16; KQ_FP32 returns KQ_ERR_DTYPE),
 * ldx >= K elements, x and its row pitch 16-byte aligned; params: fp32
 * [K/32][5][3] factor parameters (l, u, v) as kq_quantize takes them (KQ_T_PARAMS);
 * B: the weights as kq_quantize_weights writes them (qb [N][ldb], sb [N][ldsb]); out
 * as kq_mx_gemm.  The activations' codes and scales are those kq_quantize computes,
 * bit for bit, and the product is kq_mx_gemm's: the result equals kq_mx_gemm on
 * kq_quantize's output exactly.  K: multiple of 32, at most 16384 (every block's
 * transform constants are held on chip).  The activation tile is quantized again
 * for every 256-column tile of out, so this pays only when N is small.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_DTYPE, KQ_ERR_HIP. */
int kq_mx_gemm_fused(const void* x, int dtype, int64_t ldx, const float* params,
                     const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                     int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* stream);

/* Bytes of device workspace that kq_mx_gemm_fused_ws uses for an M x N x K product
 * on the current device (written to *bytes; 0 when nothing is split, which is then
 * the same product as kq_mx_gemm_fused).  The fused product computes 128 x 256
 * output tiles, at most one workgroup per compute unit, and each tile quantizes its
 * activation rows over all of K, so with few tiles the quantization runs on few
 * compute units.  When twice the tiles (rounded up to a multiple of 8) fit on the
 * compute units and K has at least 6 steps of 256, each tile is computed as S
 * parts of K on S compute units of one XCD (each quantizing and multiplying its K
 * steps only), which meet through the workspace: S is the largest of 2, 4 and 8
 * such that S times the tiles (rounded up to 8) fit on the compute units and every
 * part has at least 3 K steps.  The workspace is 4096 bytes of flag words, then
 * S x 128 KiB of fp32 partial sums per tile; the parts' sums are added in part
 * order.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_HIP. */
int kq_mx_gemm_fused_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/* kq_mx_gemm_fused with a caller-owned device workspace (same arguments, and the
 * result up to the fp32 rounding of the parts' sums, within the product's bound):
 *   workspace        device memory, 256-byte aligned (KQ_ERR_ALIGN), of at least
 *                    kq_mx_gemm_fused_workspace_size bytes (KQ_ERR_VALUE); its first
 *                    4096 bytes are zero before the first call, and every call
 *                    leaves them zero.  NULL with workspace_bytes 0: no split, as
 *                    kq_mx_gemm_fused (NULL with other sizes: KQ_ERR_NULL).
 * Calls that share a workspace must not run at the same time (one stream, or
 * ordered streams).  The library allocates nothing.
 * Errors: as kq_mx_gemm_fused, and KQ_ERR_VALUE. */
int kq_mx_gemm_fused_ws(const void* x, int dtype, int64_t ldx, const float* params,
                        const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                        int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* workspace,
                        int64_t workspace_bytes, void* stream);

/* Bytes of device workspace that kq_mx_gemm_ws uses for an M x N x K product on
 * the current device (written to *bytes; 0 when nothing is split, which is then
 * the same product as kq_mx_gemm).  The product computes 256 x 256 output tiles, at
 * most one workgroup per compute unit.  When twice the tiles (rounded up to a
 * multiple of 8) fit on the compute units and K has at least 10 steps of 256,
 * each tile is computed as S parts of K on S compute units of one XCD, which meet
 * through the workspace: S is the largest of 2, 4 and 8 such that S times the
 * tiles (rounded up to 8) fit on the compute units and every part has at least 5
 * K steps.  The workspace is 4096 bytes of flag words, then S x 256 KiB of fp32
 * partial sums per tile (1024 x 3072 x 12288: 48 tiles, S = 4, 48 MiB, 0.54x the
 * unsplit time).  Each XCD's tiles, with all their parts, form one compact block of
 * the tile grid.  The parts' sums are added in part order, so the result does not
 * depend on the order in which they finish.  With more tiles the matrix cores are
 * already busy on most compute units and nothing is split.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_HIP. */
int kq_mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/* kq_mx_gemm with a caller-owned device workspace (same arguments and result):
 *   workspace        device memory, 256-byte aligned (KQ_ERR_ALIGN), of at least
 *                    kq_mx_gemm_workspace_size bytes (KQ_ERR_VALUE); its first 4096
 *                    bytes are zero before the first call, and every call leaves
 *                    them zero again.  NULL with workspace_bytes 0: no split, as
 *                    kq_mx_gemm (NULL with other sizes: KQ_ERR_NULL).
 * Calls that share a workspace must not run at the same time (one stream, or
 * ordered streams).  The library allocates nothing.
 * Errors: as kq_mx_gemm, and KQ_ERR_VALUE. */
int kq_mx_gemm_ws(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
                  const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                  int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* workspace,
                  int64_t workspace_bytes, void* stream);

/* kq_mx_gemm_ws without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid allocation): same arguments and errors as kq_mx_gemm, and it allocates
 * nothing.  The split tiles meet through the library's own static device array of
 * 4096 + 128 x 256 KiB bytes (32 MiB + 4 KiB), which every device the library
 * runs on holds until the process ends.  Its 128 slots of partial sums bound the
 * parts: the tiles are split as kq_mx_gemm_ws splits them when S x tiles <= 128,
 * else in the largest of 4 and 2 parts that fits (the same result up to the fp32
 * rounding of the parts' sums), else not at all.  The array's address is looked
 * up on a device's first call, which also clears its flag words with a kernel on
 * `stream`.  Every call on one device shares that device's array: calls that
 * overlap on one device (other streams, other threads) race and must not be made.
 * Errors: as kq_mx_gemm. */
int kq_mx_gemm_static(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
                      const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                      int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* stream);

/* Static text for a kq_status value (never NULL). */
const char* kq_status_string(int status);

/* hipError_t of this thread's last KQ_ERR_HIP (0 if none). */
int kq_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif
