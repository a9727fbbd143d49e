/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear forward.
 *
 * Citations: [PMV] is the produtoramaxvision.com.br blog article on BitNet b1.58
 * (ternary quantisation, the BitLinear layer and Zero-GEMM).  [PMV s1] is its
 * section on why ternary weights carry 1.58 bits (AbsMean and AbsMax
 * equations), [PMV s2] the section on how BitLinear removes multiplications
 * (add/subtract/skip, INT32 accumulation, rescale by gamma_A * gamma / 127),
 * [PMV s3] the section on the memory wall (2-bit packing, 0.25 byte/weight),
 * [PMV s4] the section on how bitnet.cpp speeds up inference on CPUs (the
 * LUT figure and the Radix-3 packing of five weights per byte), [PMV s6] its
 * section on trade-offs and engineering challenges.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Array pointers are DEVICE pointers to contiguous row-major arrays that the
 *    caller allocates and owns.  The library allocates nothing and keeps no
 *    mutable global state; calls on different streams do not interact.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on it: no host synchronisation, results are ready
 *    when the stream reaches them.  Faults inside kernels surface at the
 *    caller's next synchronisation of that stream.
 *  - Every argument is checked on the host before anything is launched; a
 *    failed check returns a negative status and enqueues nothing.  A failed
 *    launch returns BITLINEAR_ERR_HIP.  Nothing throws or aborts.
 *  - Sizes: 1 <= M, N, K; N*K < 2^32; a packed matrix below 2 GiB
 *    (N * bitlinear_padded_k(K) / 4 < 2^31); M*N < 2^40; K <= 2^20.
 *  - Non-finite inputs (inf/nan in W or X) give unspecified results.
 *
 * Packed ternary weights (the format of `packed` outside the radix-3 calls)
 * -------------------------------------------------------------------------
 * Each weight is stored as a 2-bit code c = q + 1 in {0,1,2} (3 never occurs),
 * [PMV s3].  A row of K weights is padded to Kp = bitlinear_padded_k(K) (a
 * multiple of 64) with c = 1, i.e. zero weights, and encoded as Kp/16
 * little-endian uint32 words; bits [8b+2i, 8b+2i+1] of word j hold the code of
 * k = 16j + 4i + b.  So `(word >> 2i) & 0x03030303` is four int8 codes for
 * k = 16j+4i .. 16j+4i+3.
 *
 * Memory order (both formats): a row is a run of U 16-byte units (here four
 * words, U = Kp/64).  Rows are stored in blocks of 16 consecutive rows (the
 * last block holds N % 16 rows if that is not 0) and each block's units in
 * chunks of 4 consecutive units (the last chunk holds U % 4 units if that is
 * not 0); within a chunk, each row of the block in turn stores its units of
 * that chunk contiguously.  Unit u of row n is therefore at byte
 *     16*b*U*16 + c*R*64 + j*W*16 + (u%4)*16,
 * with b = n/16, j = n%16, c = u/4, R = min(16, N - 16b), W = min(4, U - 4c).
 * A full chunk (16 rows x 4 units) is one contiguous KiB, which the decode
 * kernel reads with one load instruction; a single row (N = 1) is stored
 * row-major.  The whole buffer is bitlinear_packed_bytes(N, K) = N*Kp/4 bytes
 * and carries no header: a forward must be given the N and K it was packed with.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define BITLINEAR_OK             0
#define BITLINEAR_ERR_NULL      -1 /* a required pointer is NULL                  */
#define BITLINEAR_ERR_SHAPE     -2 /* M, N, K or L out of the supported range      */
#define BITLINEAR_ERR_DTYPE     -3 /* unknown activation dtype                     */
#define BITLINEAR_ERR_ALIGN     -4 /* a pointer is not aligned as required         */
#define BITLINEAR_ERR_WORKSPACE -5 /* workspace missing or smaller than required   */
#define BITLINEAR_ERR_HIP       -6 /* a HIP call or kernel launch failed           */
#define BITLINEAR_ERR_ARG       -7 /* another argument (path selector) is invalid  */

/* ---- activation dtypes (Y is always float32) --------------------------- */
#define BITLINEAR_F32  0
#define BITLINEAR_BF16 1

/* ---- forward path selector (bitlinear_forward_ex) ----------------------- */
#define BITLINEAR_PATH_AUTO    0 /* decode for M <= bitlinear_max_decode_m(), else prefill */
#define BITLINEAR_PATH_DECODE  1 /* fused quantise + GEMV kernel (M <= bitlinear_max_decode_m()) */
#define BITLINEAR_PATH_PREFILL 2 /* activation quantiser + INT8-MFMA GEMM */

/* ---- sizes ------------------------------------------------------------- */

/* Kp: K rounded up to a multiple of 64 (the packed row length in weights). */
int64_t bitlinear_padded_k(int64_t K);

/* Bytes of a packed [N, K] ternary matrix: N * Kp / 4.  [PMV s3] */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Workspace bytes bitlinear_quantize_weights needs (a constant, < 128 KiB). */
size_t bitlinear_quantize_workspace_bytes(void);

/* Workspace bytes bitlinear_forward / _ex need for an M x K activation on the
 * prefill path: M*Kp int8 codes + M float32 scales + M int32 code sums, each
 * part 256-byte aligned.  The decode path needs none (it may be passed 0). */
size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t K);

/* Largest M the decode path accepts (16), and the largest M*(Kp+16) it
 * accepts (the codes of all tokens live in on-chip memory, each token row
 * padded by 16 bytes: 65536 bytes).  The decode path also needs M*N < 2^29. */
int bitlinear_max_decode_m(void);
int64_t bitlinear_max_decode_codes(void);

/* ---- a1 + a2: offline weight quantisation ------------------------------ */
/*
 * gamma = (1/(N*K)) * sum |W|                      [PMV s1, AbsMean equation]
 * q     = Round(Clip(W / (gamma + eps), -1, 1))    [PMV s1, RoundClip]
 * then packed 2 bits per weight                    [PMV s3]
 *
 * W:      device float32 [N, K] row-major, 16-byte aligned.
 * packed: device, bitlinear_packed_bytes(N, K) bytes, 16-byte aligned (output).
 * gamma:  device float32[1] (output).
 * workspace: device, >= bitlinear_quantize_workspace_bytes(), 16-byte aligned;
 *         scratch only, contents on entry do not matter.
 *
 * Arithmetic: the sum of |W| is formed exactly (per-exponent integer digits)
 * and rounded once to the nearest float64; gamma = float32(sum / (N*K)) with a
 * float64 division.  eps = 1e-5f; W / (gamma + eps) is an IEEE float32
 * division; Round is round-half-to-even.  Deterministic: the result does not
 * depend on launch shape or scheduling.
 */
int bitlinear_quantize_weights(const float* W, int64_t N, int64_t K,
                               uint32_t* packed, float* gamma,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---- a3: per-token AbsMax INT8 activation quantisation ------------------ */
/*
 * gamma_A[m] = max_k |X[m,k]|                                   [PMV s1, AbsMax]
 * Xq[m,k]    = Clip(Round(X[m,k] * (127 / (gamma_A[m] + eps))), -128, 127)
 * rowsum[m]  = sum_k Xq[m,k] (exact)
 *
 * X:       device [M, K] float32 or bfloat16 (x_dtype), aligned to its element
 *          size (rows of any length; 16-byte alignment of X together with
 *          K*sizeof % 16 == 0 selects 16-byte loads).
 * Xq:      device int8 [M, Kp] (output); columns K..Kp-1 are written as 0.
 *          16-byte aligned.
 * gamma_a: device float32 [M] (output).  rowsum: device int32 [M] (output).
 *
 * Arithmetic: float32; s = 127 / (gamma_A + 1e-5f) is one IEEE division per
 * token, each code is rint(X * s) (half to even) clipped to [-128, 127].
 */
int bitlinear_quantize_activations(const void* X, int x_dtype, int64_t M, int64_t K,
                                   int8_t* Xq, float* gamma_a, int32_t* rowsum,
                                   void* stream);

/* ---- a3..a6: the forward ------------------------------------------------ */
/*
 * Y[m,n] = (sum_k Xq[m,k] * q[n,k]) * gamma * gamma_A[m] / 127
 *          [PMV s2: add for +1, subtract for -1, skip for 0; INT32 accumulator;
 *           one rescale by gamma_A * gamma / 127]
 *
 * X:      device [M, K] float32 or bfloat16, aligned to its element size.
 * packed: device packed codes of an [N, K] ternary matrix, 16-byte aligned.
 * gamma:  device float32[1], the weight scale from bitlinear_quantize_weights.
 * Y:      device float32 [M, N] (output), 4-byte aligned.
 * workspace: device, >= bitlinear_forward_workspace_bytes(M, K) when the
 *         prefill path runs (M > bitlinear_max_decode_m() or
 *         M*(Kp+16) > bitlinear_max_decode_codes()),
 *         256-byte aligned; may be NULL/0 on the decode path.
 *
 * The INT32 accumulator is exact (|acc| <= 127 * K); Y is acc converted to
 * float32 times the float32 product gamma * gamma_A[m] / 127 (three float32
 * roundings in all, relative error < 2e-7).
 */
int bitlinear_forward(const void* X, int x_dtype, int64_t M, int64_t K,
                      const uint32_t* packed, int64_t N, const float* gamma,
                      float* Y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same as bitlinear_forward with two additions for tests and benchmarks:
 *   path:  BITLINEAR_PATH_AUTO / _DECODE / _PREFILL (forcing decode with M or
 *          M*(Kp+16) beyond its limits returns BITLINEAR_ERR_SHAPE);
 *   acc:   if not NULL, device int32 [M, N] receiving the exact accumulator
 *          sum_k Xq[m,k] * q[n,k] as well (Y is still written).
 */
int bitlinear_forward_ex(const void* X, int x_dtype, int64_t M, int64_t K,
                         const uint32_t* packed, int64_t N, const float* gamma,
                         float* Y, int32_t* acc, int path,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The contraction and rescale alone, from activation codes that are already
 * quantised (by bitlinear_quantize_activations, or by a producer kernel that
 * writes the same format):  Y = (Xq x q^T) * gamma * gamma_A / 127   [PMV s2]
 *
 * Xq:      device int8 [M, Kp], 16-byte aligned; columns K..Kp-1 must be 0.
 * gamma_a: device float32 [M].  rowsum: device int32 [M], the exact sum of
 *          each token's codes (the kernel forms sum c*x with c = q + 1 and
 *          subtracts it).
 * packed, gamma, Y, acc: as for bitlinear_forward_ex.  Runs the INT8-MFMA
 * GEMM for any M.
 */
int bitlinear_forward_quantized(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum,
                                int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                                const float* gamma, float* Y, int32_t* acc, void* stream);

/*
 * L independent decode forwards of one shape in one launch (the decode path's
 * batched form: e.g. several projections of one token batch, or the experts
 * of a layer).  Layer l reads X + l*M*K elements, packed + l*N*Kp/16 words,
 * gamma[l], and writes Y + l*M*N; all 16-byte aligned as above.
 * Requires M <= bitlinear_max_decode_m() and
 * M*(Kp+16) <= bitlinear_max_decode_codes().
 */
int bitlinear_forward_batched(int64_t L, const void* X, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, int64_t N, const float* gamma,
                              float* Y, void* stream);

/* ---- the BitNet FFN block: BitLinear up -> ReLU^2 -> BitLinear down ----- */
/*
 * For l = 0..L-1:
 *   H_l = BitLinear_up(X_l)            (packed_up: [F, D] ternary, gamma_up[l])
 *   A_l = ReLU^2(H_l) = max(H_l, 0)^2  [MBC: bit_layers.py gives ReLU^2 as BitNet's
 *                                       activation]
 *   Y_l = BitLinear_down(A_l)          (packed_down: [D_out, F], gamma_down[l]);
 *         A_l is quantised per token with AbsMax like any BitLinear input [PMV s1]
 * [MBC] is the shadowgraph.io page on a multimodal architecture around
 * bitnet.cpp.  Norms stay outside, in floating point [PMV s6: the trade-offs
 * section].  H is formed in float32 exactly as every output here
 * (fp32(acc) * fp32(fp32(gamma * gamma_A) / 127)) and A = fp32(r * r), r = max(H, 0).
 *
 * The up projection's epilogue applies ReLU^2, so the hidden layer is written
 * once as float32 and read once by the quantiser of the down projection's
 * input.  Decode path (both projections fit the decode kernel): three
 * launches for all L layers (up with the ReLU^2 epilogue, the quantiser over
 * all L * M hidden rows, down on those codes).  Prefill path: per layer,
 * quantise X, GEMM with the ReLU^2 epilogue, quantise A, GEMM.
 *
 * X: device [L, M, D] float32 or bfloat16.  packed_up: L matrices of F rows,
 * bitlinear_packed_bytes(F, D) bytes each, back to back; packed_down: L
 * matrices of D_out rows, bitlinear_packed_bytes(D_out, F) bytes each.
 * gamma_up, gamma_down: device float32 [L].  Y: device float32 [L, M, D_out].
 * hidden: NULL, or device float32 [L, M, F], 16-byte aligned, receiving A.
 * path: BITLINEAR_PATH_AUTO / _DECODE / _PREFILL as for bitlinear_forward_ex.
 * workspace: >= bitlinear_ffn_workspace_bytes(L, M, D, F), 256-byte aligned
 * (holds A when hidden is NULL, and the activation codes: one layer's on the
 * prefill path, all L layers' hidden rows on the decode path).
 */
size_t bitlinear_ffn_workspace_bytes(int64_t L, int64_t M, int64_t D, int64_t F);

int bitlinear_ffn_forward(int64_t L, const void* X, int x_dtype, int64_t M, int64_t D, int64_t F,
                          int64_t D_out, const uint32_t* packed_up, const float* gamma_up,
                          const uint32_t* packed_down, const float* gamma_down, float* Y,
                          float* hidden, int path, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- backward with the straight-through estimator ----------------------- */
/*
 * [PMV s2, its STE passage]: the quantiser's gradient is taken as the identity
 * inside the valid range.  With the forward Y = A_hat W_hat^T,
 * A_hat = (gamma_A / 127) A_q and W_hat = gamma W_q:
 *   dX = dY W_hat = gamma (dY W_q)                          [M, K]
 *   dW = (dY^T A_hat) * 1[|fp32(W / fp32(gamma + eps))| <= 1]  [N, K]
 * (the activation clip never binds; gamma, gamma_A are constants).  Training
 * precision: dY is bfloat16, A_hat = bf16(fp32(fp32(gamma_A/127) * A_q)) (round
 * half to even), products on bf16 matrix cores with float32 accumulation, so
 * results differ from exact sums by float32 accumulation rounding.
 */

/* Bytes of the range mask of an [N, K] weight matrix: N rows of
 * ceil(K / 32) 32-bit words. */
size_t bitlinear_ste_mask_bytes(int64_t N, int64_t K);

/* What the backward needs from W, formed once per weight update:
 * packedT: the codes of W^T for dX, i.e. the same ternary codes (same gamma,
 *   from bitlinear_quantize_weights on W) transposed, as a [K, N] matrix in the
 *   2-bit packed format of this file (bitlinear_packed_bytes(K, N) bytes),
 *   16-byte aligned;
 * mask: the range mask for dW, bit k % 32 of word k / 32 of row n set iff
 *   |fp32(W[n, k] / fp32(gamma + eps))| <= 1 (bits past K are 0),
 *   bitlinear_ste_mask_bytes(N, K) bytes, 4-byte aligned.
 * Either output may be NULL (not both).  W: device float32 [N, K];
 * gamma: device float32[1]. */
int bitlinear_pack_transposed(const float* W, int64_t N, int64_t K, const float* gamma,
                              uint32_t* packedT, uint32_t* mask, void* stream);

/* Workspace bytes of bitlinear_backward: padded and transposed bf16 copies of
 * dY and A_hat (about 2 M (2N + K) bytes; when N % 8 == 0 and dY and Xq are
 * 16-byte aligned only A_hat is formed there, untransposed). */
size_t bitlinear_backward_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * dY: device bfloat16 [M, N] (bit patterns), the gradient of Y.
 * packedT: from bitlinear_pack_transposed (needed for dX).
 * Xq, gamma_a: the forward's activation codes [M, Kp] and scales [M], as
 *   bitlinear_quantize_activations writes them (needed for dW).
 * mask: the range mask from bitlinear_pack_transposed (needed for dW).
 * dX: device float32 [M, K] or NULL;  dW: device float32 [N, K] or NULL
 *   (at least one).  workspace: >= bitlinear_backward_workspace_bytes(M, N, K),
 *   256-byte aligned.  Requires M*padded_k(N), N*M and K*M (M rounded up to 64)
 *   below 2^30.
 */
int bitlinear_backward(const uint16_t* dY, int64_t M, int64_t N, int64_t K,
                       const uint32_t* packedT, const float* gamma,
                       const int8_t* Xq, const float* gamma_a, const uint32_t* mask,
                       float* dX, float* dW, void* workspace, size_t workspace_bytes, void* stream);

/* ---- radix-3 weights: five per byte ------------------------------------ */
/*
 * The Radix-3 packing of [PMV s4] (the section on how bitnet.cpp speeds up CPU
 * inference): five ternary weights per byte since 3^5 = 243 <= 256, 1.60 bits
 * per weight, 20% fewer weight bytes than the 2-bit format for the
 * bandwidth-bound decode path.  The section's LUT figure indexes a group of
 * weights as a base-3 number of the offset digits c = q + 1.
 *
 * Format (this library's own; the article fixes only the count): a row of K
 * weights is padded with c = 1 to Kp3 = bitlinear_r3_padded_k(K), a multiple
 * of 80, and encoded as Kp3/5 bytes.  Byte 4j + b of a row (b = 0..3) holds
 * the five weights k = 20j + 4t + b, t = 0..4, as ceil(256 * v / 243) with
 * v = sum_t c_t * 3^(4 - t); 13 byte values never occur.  Rows are stored in
 * the interleaved memory order described at the top of this file, with
 * 16-byte units of 80 weights (U = Kp3/80).  The buffer carries no header.
 */

/* Kp3: K rounded up to a multiple of 80. */
int64_t bitlinear_r3_padded_k(int64_t K);

/* Bytes of a radix-3 packed [N, K] matrix: N * Kp3 / 5. */
size_t bitlinear_r3_packed_bytes(int64_t N, int64_t K);

/*
 * bitlinear_quantize_weights with the radix-3 format: the same gamma and the
 * same ternary codes (bit-identical), packed five per byte.
 * packed: device, bitlinear_r3_packed_bytes(N, K) bytes, 16-byte aligned.
 * Other arguments and the workspace as for bitlinear_quantize_weights.
 */
int bitlinear_quantize_weights_r3(const float* W, int64_t N, int64_t K,
                                  uint8_t* packed, float* gamma,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode forward(s) over radix-3 weights: for l = 0..L-1,
 *   Y_l = (Xq_l x q_l^T) * gamma[l] * gamma_A / 127              [PMV s2]
 * with the same fused kernel as the 2-bit decode path (token codes in on-chip
 * memory, weights streamed once).  Layer l reads X + l*M*K elements,
 * packed + l*bitlinear_r3_packed_bytes(N, K) bytes and gamma[l], and writes
 * Y + l*M*N (and acc + l*M*N when acc is not NULL: the exact INT32
 * accumulators).  Requires M <= bitlinear_max_decode_m(),
 * M*(Kp3+16) <= bitlinear_max_decode_codes() and M*N < 2^29;
 * packed 16-byte aligned, Y and acc 4-byte aligned.
 */
int bitlinear_forward_r3(int64_t L, const void* X, int x_dtype, int64_t M, int64_t K,
                         const uint8_t* packed, int64_t N, const float* gamma,
                         float* Y, int32_t* acc, void* stream);

/* ---- LUT contraction: the CPU prior art, kept as a comparison ---------- */
/*
 * [PMV s4] (the LUT-GEMM figure) contracts a block of four INT8 activations
 * with four ternary weights by reading one of 81 pre-computed sums, indexed by
 * the weights' base-3 pattern (index 0 = all -1, 40 = all 0, 80 = all +1).
 * These calls run that scheme on the GPU over the ordinary 2-bit weights: a
 * workgroup builds the 81-entry tables of its tokens in LDS for a slice of K
 * and every thread looks up, per packed byte (four weights), one entry per
 * token.  The accumulators are the exact INT32 sums of every other path.  It
 * is slower than the matrix-core decode GEMV and is not chosen by
 * bitlinear_forward; it exists to measure the two schemes side by side.
 */

/* Workspace of bitlinear_forward_lut: the codes, scales and code sums of
 * L*M tokens (as bitlinear_forward_workspace_bytes(L*M, K)); 0 on bad sizes. */
size_t bitlinear_lut_workspace_bytes(int64_t L, int64_t M, int64_t K);

/*
 * LUT forward(s) over 2-bit weights: for l = 0..L-1,
 *   Y_l = (Xq_l x q_l^T) * gamma[l] * gamma_A / 127              [PMV s2, s4]
 * Layer l reads X + l*M*K elements (dtype x_dtype), the packed matrix at
 * packed + l*bitlinear_packed_bytes(N, K) bytes and gamma[l], and writes
 * Y + l*M*N (and acc + l*M*N when acc is not NULL).  Two launches: the
 * per-token AbsMax quantiser over the L*M tokens, then the LUT kernel.
 * Requires 1 <= M <= bitlinear_max_decode_m(), 1 <= L <= 2^20,
 * L*ceil(N/256) < 2^31; packed 16-byte aligned, Y and acc 4-byte aligned,
 * workspace device memory of bitlinear_lut_workspace_bytes(L, M, K) bytes,
 * 256-byte aligned.
 * Errors: BITLINEAR_ERR_NULL, _SHAPE, _DTYPE, _ALIGN, _WORKSPACE, _HIP.
 */
int bitlinear_forward_lut(int64_t L, const void* X, int x_dtype, int64_t M, int64_t K,
                          const uint32_t* packed, int64_t N, const float* gamma,
                          float* Y, int32_t* acc, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- the forward without allocation ------------------------------------ */
/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation.  The same
 * forward as bitlinear_forward (same kernels, same results, bit for bit),
 * without a workspace argument: the prefill path's activation codes, scales
 * and code sums go to a scratch array that the library holds on every GPU it
 * runs on (BITLINEAR_NOALLOC_SCRATCH_BYTES of device memory per GPU, from the
 * moment the library's code is loaded on that GPU until the process ends).
 * The call itself allocates nothing.
 *
 * Limit: the prefill path (M > bitlinear_max_decode_m(), or rows too long for
 * the decode kernel) needs bitlinear_forward_workspace_bytes(M, K) <=
 * BITLINEAR_NOALLOC_SCRATCH_BYTES (80 MiB: e.g. 8192 tokens of K = 8192, or
 * 16384 tokens of K = 4096), else the call returns BITLINEAR_ERR_WORKSPACE and
 * enqueues nothing.  The decode path uses no scratch.
 *
 * Every call on one GPU shares that GPU's scratch array: calls that may
 * overlap on one GPU (different streams, or host threads without an order
 * between them) race and give wrong results; serialise them.  The array is
 * looked up once per GPU, on the first call that runs there.
 * Arguments, errors and the stream's role are as for bitlinear_forward.
 */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (80u * 1024u * 1024u)

int bitlinear_forward_noalloc(const void* X, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, int64_t N, const float* gamma,
                              float* Y, void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* bitlinear_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
