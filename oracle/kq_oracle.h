/*
 * kq_oracle.h — plain, slow, fp64 CPU oracle of the KroQuant online activation
 * quantizer (Kronecker-factored 32x32 block transform followed by MXFP4).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include, link
 * or call this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the GPU kernels.
 *
 * Sources (the pages are abstracts; where they are silent the reading is stated):
 *  [ABS]  KroQuant: Kronecker-Structured Block Transforms for Efficient
 *         Post-Training Quantization of Diffusion Transformers, arXiv 2607.21446,
 *         abstract (arxivdaily page and paper-with-me page): one learned
 *         invertible Kronecker-structured transform per 32-element activation
 *         block; the inverse goes to the weights; fewer than half the parameters
 *         of per-channel scaling; W4A4 with MXFP4 activations; SmoothQuant
 *         per-channel scaling is the cheap comparison transform.
 *  [POD]  Same paper, researchpod summary, method paragraph: each 32x32 block is
 *         a Kronecker product of five 2x2 unit-determinant LU-decomposed matrices.
 *  [MX]   OCP Microscaling Formats (MX) v1.0: MXFP4 = 32 E2M1 elements sharing
 *         one E8M0 scale; scale exponent = floor(log2(amax)) - emax_elem with
 *         emax_elem = 2 for E2M1; element conversion rounds to nearest even and
 *         saturates to the largest magnitude (6).
 *  Fixed conventions (the pages leave them open):
 *   - factor  F = L*U, L = [[1,0],[l,1]], U = [[u,v],[0,1/u]]  (det F = 1)
 *   - T_b = kron(F1, kron(F2, kron(F3, kron(F4, F5)))): F1 acts on bit 4 of the
 *     within-block index, F5 on bit 0
 *   - y_b = T_b * x_b (column convention; weights would take W_b * T_b^-1)
 *   - all-zero block: exponent -127 (E8M0 byte 0x00); any NaN/Inf in the block's
 *     transformed values: E8M0 byte 0xFF and all codes 0
 *   - codes: bit 3 = sign of y (so a tiny negative value encodes as 0x8),
 *     bits 0..2 index {0, .5, 1, 1.5, 2, 3, 4, 6}
 *   - packing: Q[t][16b + i/2] holds channel 32b+i in the low nibble for even i,
 *     the high nibble for odd i; S[t][b] is the E8M0 byte
 *
 * Arrays are row-major; every pointer is host memory owned by the caller.
 * Functions return 0 on success and a negative value on a bad argument.
 */
#ifndef KQ_ORACLE_H
#define KQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OQ_BF16 = 0, OQ_FP32 = 1 };

/* 2x2 factor F = L*U from (l, u, v), row-major F[0..3]. [POD] */
void oq_factor(double l, double u, double v, double F[4]);

/* Inverse factor U^-1 * L^-1, row-major. [ABS] (the inverse goes to the weights) */
void oq_factor_inverse(double l, double u, double v, double Finv[4]);

/* Kronecker product C = A (ar x ac) (x) B (br x bc); C is (ar*br) x (ac*bc). */
void oq_kron(const double* A, int ar, int ac, const double* B, int br, int bc, double* C);

/* Dense T_b for every block: params [nb][5][3] fp32 (l,u,v) -> T [nb][32][32] fp64.
 * inverse != 0 builds kron of the factor inverses instead.  [POD] */
int oq_expand(const float* params, int64_t nb, int inverse, double* T);

/* Determinant of an n x n fp64 matrix by Gaussian elimination with partial pivoting. */
double oq_det(const double* A, int n);

/* Widen one input element to fp64 (exact): dtype OQ_BF16 reads uint16 bits, OQ_FP32 floats. */
double oq_load(const void* x, int dtype, int64_t idx);

/* y[t][32b+i] = sum_j T_b[i][j] x[t][32b+j] in fp64 (the plain definition). [ABS][POD]
 * x has row pitch ldx elements; y is [rows][d] fp64. */
int oq_transform_dense(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       const double* T, double* y);

/* Same transform applied factor by factor (F_k on index bit 5-k), fp64; a self-check. */
int oq_transform_factored(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                          const float* params, double* y);

/* MX scale exponent e of a block from its amax. [MX]
 * Returns e in [-127, 127] (amax = 0 -> -127) or 128 when amax is NaN/Inf. */
int oq_scale_exp(double amax);

/* E2M1 code (sign bit 3, magnitude bits 0..2) of value y in a block whose scale
 * exponent is e (|e| <= 127). [MX] */
int oq_e2m1_code(double y, int e);

/* Decoded signed value of a code at scale exponent e (for round trips). */
double oq_e2m1_value(int code, int e);

/* MXFP4-encode fp64 rows y[rows][d] (d % 32 == 0) into q [rows][ldq] bytes and
 * s [rows][lds] bytes. [MX] */
int oq_encode(const double* y, int64_t rows, int64_t d, uint8_t* q, int64_t ldq,
              uint8_t* s, int64_t lds);

/* The whole path: expand, transform (dense, fp64), MXFP4 encode.  y_out (optional,
 * [rows][d] fp64) receives the pre-quantization values.  nthreads <= 0 uses all cores. */
int oq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                double* y_out, int nthreads);

/* SmoothQuant baseline: y[t][c] = x[t][c] * mult[c] (mult = fp32 1/s_c), then MXFP4. [ABS] */
int oq_sq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                   const float* mult, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                   double* y_out, int nthreads);

/* Weight side: W'[r][32b+j] = sum_i W[r][32b+i] * Tinv_b[i][j], i.e. W' = W T^-1 with
 * T^-1 block-diagonal (the inverse folded into the weights, so that W' (T x) = W x).
 * [ABS]  w is [rows][ldw] of dtype; w_out [rows][d] fp64. */
int oq_weight_transform(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                        const float* params, double* w_out);

/* W' followed by the MXFP4 encoding along d (blocks of 32 input channels). */
int oq_quantize_weights(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                        const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                        double* w_out, int nthreads);

/* Fixed block-Hadamard comparison transform: y_b = H x_b / sqrt(32) with the
 * Sylvester matrix H[i][j] = (-1)^popcount(i & j) (symmetric, H H = 32 I, so the
 * weights take the same transform), then the MXFP4 encoding.  [ABS] (fixed
 * Hadamard transforms are the accurate but costly comparison point) */
int oq_hadamard_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                         uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, double* y_out,
                         int nthreads);

/* Normalization fused ahead of the quantizer ([ABS]: the normalization layers
 * between blocks are what force the transform to run online).  Per row t
 *   mu = mean_c x[t][c],  var = mean_c (x[t][c] - mu)^2,  rstd = 1 / sqrt(var + eps)
 *   h[t][c] = (x[t][c] - mu) * rstd * (1 + scale[g][c]) + shift[g][c],  g = t / rows_per_sample
 * (LayerNorm without affine parameters, then the adaptive-norm modulation of a DiT
 * block; scale/shift may be NULL for zero), then y_b = T_b h_b and MXFP4.
 * scale, shift: float32 [ceil(rows / rows_per_sample)][d].  h_out and y_out
 * (optional, fp64 [rows][d]) receive h and y. */
int oq_norm_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                     const float* shift, const float* scale, int64_t rows_per_sample, double eps,
                     const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                     double* h_out, double* y_out, int nthreads);

/* Decode MXFP4 rows back to values: out[t][c] = E2M1(code) * 2^(S - 127) with the
 * block's E8M0 byte S (0xFF, the NaN scale, decodes to NaN).  [MX] */
int oq_dequantize(const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds, int64_t rows,
                  int64_t d, double* out);

/* Parity accounting of candidate outputs against the oracle's fp64 values y_o.
 * Per block the tolerance is tol_coef * max|x_blk| (tol_mode 0, the fp32 rule) or
 * tol_coef * max|y_o_blk| (tol_mode 1, the block-relative bf16 rule).
 *  - scale byte equal: exact; else excused when some amax within tol of the
 *    oracle's amax yields the candidate's byte (the block's codes are then judged
 *    at the candidate's scale and the block counts 32 excused elements); else
 *    unexcused (the block counts 32 unexcused elements).
 *  - code equal: exact; else excused when some value within tol of y_o encodes to
 *    the candidate's code at the block's scale; else unexcused.
 * y_c (optional, fp32 [rows][ldy]) is the candidate's pre-quantization output:
 * when given, stats[5] counts elements with |y_c - y_o| > tol and stats[6] holds the
 * largest |y_c - y_o| / (tol / tol_coef).
 * stats (double[8]): 0 exact elements, 1 excused elements, 2 unexcused elements,
 *   3 excused scale blocks, 4 unexcused scale blocks, 5 pre-quant violations,
 *   6 max normalized pre-quant error, 7 first unexcused flat element index or -1. */
int oq_classify(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                const double* y_o, int tol_mode, double tol_coef,
                const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds,
                const float* y_c, int64_t ldy, double* stats);

#ifdef __cplusplus
}
#endif
#endif
