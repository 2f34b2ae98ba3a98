/*
 * gemm05.h -- dense GEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation is the plain matrix product
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N
 *
 * with 2*M*N*K floating-point operations, as stated by page "4.1 Tối ưu hiệu
 * năng toán tử GEMM trên CUDA" (§1.1, and the naive kernel of §3.1), by the
 * MUSA learning-center lesson m11-l5 (case 4, problem statement) and by page
 * "Operator & Runtime" (§5.2.1).  Batched GEMM for multi-head attention is
 * named in §1.2 of the first page.  For BF16 operands the products are
 * accumulated in FP32 and, for a BF16 output, the finished FP32 sum is rounded
 * once to BF16, round to nearest, ties to even ("Operator & Runtime", the
 * FFN projection at the start of the chapter, §5.2.2 and §5.4.3).
 *
 * Layout.  Every matrix is row-major.  lda, ldb, ldc are row strides counted
 * in ELEMENTS: A[i][k] is at A + i*lda + k, B[k][j] at B + k*ldb + j, C[i][j]
 * at C + i*ldc + j.  C is overwritten (alpha, beta and a bias are the
 * affine epilogue's, gemm_bf16_affine).
 *
 * Ownership.  The caller owns all device memory: A, B, C and, for
 * gemm_run, an optional workspace.  Each call validates its arguments on the
 * host, enqueues its kernel(s) on `stream` (a hipStream_t; NULL means the
 * null stream) and returns; completion is observed through the stream.  The
 * library never allocates, frees, copies or waits for device memory, and
 * keeps no state beyond a thread-safe cache of each device's architecture;
 * calls are thread-safe.  Three paths need scratch memory and run only when
 * the caller passes a workspace to gemm_run: K split over workgroups (the
 * small-M path and tiled bf16 outputs with too few tiles to fill the GPU;
 * FP32 partial sums and arrival counters) and the copy of operand rows that
 * are not 16-byte aligned into aligned rows (large bf16 products, and the
 * transposed and fused layouts whose kernels read 16-byte rows only).  The
 * named entry points (gemm_bf16, ...) take none: they run the same
 * arithmetic on the paths that need no scratch (whole K per workgroup;
 * operands read as they are), or return GEMM_ERR_UNSUPPORTED where only a
 * realigned copy could run the call.  The environment variable
 * GEMM_FORCE_KSPLIT=S (diagnostics and tests) forces a split of S slices on
 * gemm_run calls with a workspace that use 128x128 tiles (1 = none;
 * GEMM_ERR_UNSUPPORTED when S slices of at least 4 32-deep stages do not
 * fit K, or without a workspace); GEMM_DECODE_PAIR=0 makes the small-M path
 * combine its two workgroups per strip through counters and partial sums
 * instead of exchange slots (the same bits, either way).
 * No alignment is required; aligned operands (16-byte rows and pointers)
 * select the faster kernel variants.
 *
 * Edge semantics.  M == 0, N == 0 or batch == 0: nothing to do, GEMM_OK.
 * K == 0: C := 0 (the empty sum).  Results are deterministic: the same call
 * on the same inputs gives the same bits (no atomics on data, fixed
 * reduction order), and the small-M path splits K the same way for every M,
 * so a row's result does not depend on how many rows are in the call.
 *
 * Errors.  A negative status is returned and nothing is enqueued when the
 * arguments are invalid (GEMM_ERR_INVALID_ARG): a negative size or batch;
 * lda < K, ldb < N or ldc < N for a non-empty operand (for the transposed
 * layouts: ldat < M, ldbt < K); a NULL pointer for an
 * operand that is read or written; a c_type outside gemm_out_type; a negative
 * batch stride; batch > 1 with strideC < (M-1)*ldc + N (C entries would
 * overlap); or C's byte range overlapping A's or B's.  GEMM_ERR_UNSUPPORTED:
 * a kernel configuration forced through the GEMM_FORCE_CONFIG environment
 * variable cannot run this problem, or only a workspace path could and none
 * was passed.  GEMM_ERR_NO_DEVICE: no HIP device is current, or the current
 * one is not a gfx950.  GEMM_ERR_LAUNCH: the kernel launch failed
 * (hipGetLastError).  GEMM_ERR_WORKSPACE: gemm_run was passed a workspace
 * smaller than gemm_workspace_size reports for the call.
 */
#ifndef GEMM05_H
#define GEMM05_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,
    GEMM_ERR_UNSUPPORTED = -2,
    GEMM_ERR_LAUNCH = -3,
    GEMM_ERR_NO_DEVICE = -4,
    GEMM_ERR_WORKSPACE = -5
} gemm_status;

/* Output element type of the BF16 entry points. */
typedef enum {
    GEMM_OUT_BF16 = 0, /* C holds bf16 bit patterns (uint16_t), RNE of the FP32 sum */
    GEMM_OUT_F32 = 1,  /* C holds float, the FP32 sum */
    GEMM_OUT_E4M3 = 2  /* SwiGLU only: C holds E4M3FN codes (uint8_t) against a fixed
                          range (gemm_bf16_swiglu_e4m3) */
} gemm_out_type;

/* FP32 GEMM: A [M,K] float, B [K,N] float, C [M,N] float (FP32 products and
 * FP32 accumulation on the matrix cores). */
int gemm_sgemm(int64_t M, int64_t N, int64_t K,
               const float *A, int64_t lda,
               const float *B, int64_t ldb,
               float *C, int64_t ldc,
               void *stream);

/* BF16 GEMM with FP32 accumulation: A [M,K] and B [K,N] hold bf16 bit
 * patterns; C [M,N] is bf16 (c_type GEMM_OUT_BF16) or float (GEMM_OUT_F32).
 * M <= 16 uses the memory-bound small-M (decode) path; with a workspace
 * (gemm_run) its K split over workgroups. */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const uint16_t *A, int64_t lda,
              const uint16_t *B, int64_t ldb,
              void *C, int64_t ldc, int c_type,
              void *stream);

/* Batched BF16 GEMM: for b in [0, batch), entry b computes
 * C + b*strideC := (A + b*strideA) . (B + b*strideB), each as gemm_bf16.
 * Strides are in elements and >= 0; strideA or strideB of 0 broadcasts that
 * operand to every entry. */
int gemm_bf16_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                      const uint16_t *A, int64_t lda, int64_t strideA,
                      const uint16_t *B, int64_t ldb, int64_t strideB,
                      void *C, int64_t ldc, int64_t strideC, int c_type,
                      void *stream);

/* BF16 GEMM with B given transposed ("NT"): C [M,N] := A [M,K] . Bt^T, where
 * Bt [N,K] is row-major with row stride ldbt >= K, so B's element (k, n) is
 * Bt[n*ldbt + k].  This is the layout of a linear layer's weight ([out, in])
 * and of the keys in attention scores Q.K^T (the batched GEMM for multi-head
 * attention named in §1.2 of page "4.1 Tối ưu hiệu năng toán tử GEMM trên
 * CUDA"): no transposed copy of B is needed.  Everything else follows
 * gemm_bf16 / gemm_bf16_batched (strideBt is the batch stride of Bt), except
 * that M <= 16 with 16-byte aligned Bt rows runs a small-M kernel of its
 * own, and Bt rows that are not 16-byte aligned need a workspace
 * (gemm_run), into which they are first copied to aligned rows
 * (GEMM_ERR_UNSUPPORTED without one). */
int gemm_bf16_nt(int64_t M, int64_t N, int64_t K,
                 const uint16_t *A, int64_t lda,
                 const uint16_t *Bt, int64_t ldbt,
                 void *C, int64_t ldc, int c_type,
                 void *stream);
int gemm_bf16_nt_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda, int64_t strideA,
                         const uint16_t *Bt, int64_t ldbt, int64_t strideBt,
                         void *C, int64_t ldc, int64_t strideC, int c_type,
                         void *stream);

/* BF16 GEMM with A given transposed ("TN"): C [M,N] := At^T . B [K,N],
 * where At [K,M] is row-major with row stride ldat >= M, so A's element
 * (m, k) is At[k*ldat + m].  This is the layout of the activations X [K,M]
 * in a weight gradient X^T . dY, which would otherwise need a transposed
 * copy.  Everything else follows gemm_bf16 / gemm_bf16_batched (strideAt is
 * the batch stride of At), except that every size runs on the tiled
 * kernels, and At rows that are not 16-byte aligned, or M not a multiple
 * of 8, are first copied to aligned rows of ceil(M/8)*8 elements (zero
 * padded) in a workspace (gemm_run; GEMM_ERR_UNSUPPORTED without one). */
int gemm_bf16_tn(int64_t M, int64_t N, int64_t K,
                 const uint16_t *At, int64_t ldat,
                 const uint16_t *B, int64_t ldb,
                 void *C, int64_t ldc, int c_type,
                 void *stream);
int gemm_bf16_tn_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                         const uint16_t *At, int64_t ldat, int64_t strideAt,
                         const uint16_t *B, int64_t ldb, int64_t strideB,
                         void *C, int64_t ldc, int64_t strideC, int c_type,
                         void *stream);

/* ---- FP8 (E4M3FN) ---------------------------------------------------------
 *
 * Page "Operator & Runtime" (§5.4.3) quantizes to E4M3FN -- 1 sign, 4
 * exponent and 3 mantissa bits, largest finite value 448 -- with a factor
 * from the whole row's maximum (Example 5-7), and prefers quantizing the
 * input once, before the GEMM, to quantizing inside every output tile
 * (Example 5-8).  Codes are the OCP E4M3FN encoding (exponent bias 7, no
 * infinities, 0x7f/0xff NaN), which is what gfx950's fp8 matrix cores read.
 */

/* Per-row quantization of bf16 rows X [rows, cols] (row stride ldx) into
 * E4M3FN codes Q (row stride ldq, bytes) and dequantization factors
 * scale[rows] (float, 4-byte aligned): with amax the row's largest
 * magnitude, the code of x is the E4M3FN value nearest to the exact
 * quotient x * 448 / amax (ties to the even mantissa; Example 5-7), reached
 * through a binary32 quotient of x * 448 by amax whose code is that of the
 * correctly rounded division (a reciprocal and one residual step for amax
 * in [2^-126, 2^118], the division itself otherwise), and scale =
 * amax / 448 rounded to binary32.  A row of zeros gives zero codes
 * (signed) and factor 0.  Inputs are expected finite (a NaN element becomes
 * a NaN code).
 * GEMM_ERR_INVALID_ARG: negative sizes, ldx or ldq < cols, NULL or
 * unaligned pointers, or overlapping X, Q and scale. */
int gemm_fp8_quantize_rows(int64_t rows, int64_t cols,
                           const uint16_t *X, int64_t ldx,
                           uint8_t *Q, int64_t ldq, float *scale,
                           void *stream);

/* Per-column E4M3FN quantization of a weight stored [K, N] (the layout of
 * Example 5-8's FP8 weight): column j of W (bf16 bit patterns, K rows, row
 * stride ldw >= N elements) is quantized with its own factor exactly as
 * gemm_fp8_quantize_rows quantizes a row -- codes nearest to
 * W[k][j] * 448 / amax_j, scale[j] = amax_j / 448 -- and its codes are
 * written as row j of Qt [N, K] (row stride ldq >= K bytes), the Bt operand
 * of the FP8 products.  Caller-owned device memory, nothing else touched
 * (scale[] holds the column maxima until the call's last pass turns them
 * into factors); deterministic.  GEMM_ERR_INVALID_ARG: negative sizes, ldw < N or
 * ldq < K, NULL or unaligned pointers (W 2-byte, scale 4-byte), or
 * overlapping W, Qt and scale. */
int gemm_fp8_quantize_cols(int64_t K, int64_t N,
                           const uint16_t *W, int64_t ldw,
                           uint8_t *Qt, int64_t ldq, float *scale,
                           void *stream);

/* Scaled FP8 GEMM with B given transposed:
 *     C[i][j] = (sum_k dec(A[i][k]) * dec(Bt[j][k])) * scale_a[i] * scale_b[j]
 * A [M,K] and Bt [N,K] E4M3FN codes (row strides lda, ldbt >= K, bytes);
 * the products are exact in FP32 and summed in FP32; the sum is multiplied
 * by the row's factor, then the column's (NULL: factors of 1); C is bf16
 * (rounded once, to nearest even) or float by c_type.  Layout and errors as
 * gemm_bf16_nt, with: GEMM_ERR_INVALID_ARG for unaligned scale pointers or C
 * overlapping a scale vector; GEMM_ERR_UNSUPPORTED when Bt's rows are not
 * 16-byte aligned or A's rows not 4-byte aligned.  M <= 16 runs on a GEMV
 * kernel over the rows of Bt, larger M on the tiled kernels. */
int gemm_fp8_nt(int64_t M, int64_t N, int64_t K,
                const uint8_t *A, int64_t lda, const float *scale_a,
                const uint8_t *Bt, int64_t ldbt, const float *scale_b,
                void *C, int64_t ldc, int c_type,
                void *stream);

/* The scaled FP8 product with the input quantized inside the GEMM, the
 * alternative Example 5-8 ("Operator & Runtime" §5.4.3) weighs against
 * quantizing it first: X [M, K] bf16 rows (row stride ldx elements), Bt
 * [N, K] E4M3FN codes with factors scale_b (or NULL).  A first pass reads X
 * once for each row's largest magnitude (into the caller's workspace, M
 * floats after its first GEMM_WORKSPACE_COUNTER_BYTES) and writes the
 * row's factor amax/448 to
 * scale_x[M]; the product
 * then reads X as bf16 in every output tile (128 rows by 128 or 256
 * columns) and converts it to codes on the way into local memory, by the
 * rule of gemm_fp8_quantize_rows, so C equals gemm_fp8_nt on the codes
 * gemm_fp8_quantize_rows(X) gives, computed with 128x128 tiles and no K
 * split (bit for bit).  C bf16 or float by c_type.  Requires
 * K % 64 == 0 and 16-byte aligned rows of X and Bt (else
 * GEMM_ERR_UNSUPPORTED); workspace: at least GEMM_WORKSPACE_COUNTER_BYTES +
 * 4 M bytes, 256-byte aligned (else GEMM_ERR_WORKSPACE, or
 * GEMM_ERR_INVALID_ARG for the alignment); its counter region is left
 * untouched, so the same workspace serves gemm_run calls;
 * GEMM_ERR_INVALID_ARG for negative sizes, short strides, NULL or unaligned
 * pointers and overlapping buffers.  Nothing is allocated. */
int gemm_fp8_nt_quant_a(int64_t M, int64_t N, int64_t K,
                        const uint16_t *X, int64_t ldx, float *scale_x,
                        const uint8_t *Bt, int64_t ldbt, const float *scale_b,
                        void *C, int64_t ldc, int c_type,
                        void *workspace, uint64_t workspace_bytes,
                        void *stream);

/* The same for a batch of products (e.g. the experts of a mixture-of-
 * experts layer): entry b multiplies A + b*strideA by Bt + b*strideBt into
 * C + b*strideC (strides in elements; a stride of 0 broadcasts an operand).
 * An operand's factors follow its stride: a broadcast operand (stride 0, or
 * batch 1) has one vector (scale_a[M], scale_b[N]) for every entry, else
 * entry b's factors start at scale_a + b*M (scale_b + b*N).  Errors as
 * gemm_fp8_nt and gemm_bf16_batched. */
int gemm_fp8_nt_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                        const uint8_t *A, int64_t lda, int64_t strideA, const float *scale_a,
                        const uint8_t *Bt, int64_t ldbt, int64_t strideBt, const float *scale_b,
                        void *C, int64_t ldc, int64_t strideC, int c_type,
                        void *stream);

/* The scaled FP8 product (batched as gemm_fp8_nt_batched, batch >= 1) with
 * the affine epilogue of gemm_bf16_affine:
 *     C := alpha * D + bias[j] + beta * C,  D the dequantized sum above,
 * evaluated in FP32 and rounded once to C's type (C read only when
 * beta != 0; bias bf16 [N] or NULL, shared by the batch entries).  Layout
 * and errors as gemm_fp8_nt_batched and gemm_bf16_affine (output rows
 * 16-byte aligned and N % 8 == 0, else GEMM_ERR_UNSUPPORTED). */
int gemm_fp8_nt_affine(int64_t batch, int64_t M, int64_t N, int64_t K,
                       const uint8_t *A, int64_t lda, int64_t strideA, const float *scale_a,
                       const uint8_t *Bt, int64_t ldbt, int64_t strideBt, const float *scale_b,
                       float alpha, const uint16_t *bias, float beta,
                       void *C, int64_t ldc, int64_t strideC, int c_type,
                       void *stream);

/* ---- fused epilogues ------------------------------------------------------
 *
 * Page "Operator & Runtime" fuses the element-wise step after a projection
 * into the GEMM's output tile, so that the intermediate never travels to HBM
 * and back: an activation applied to the finished output tile (§5.4.2,
 * Y = SiLU(A.W)), and the SwiGLU product of the two projections that share
 * the input X (§5.3.1, Z = SiLU(X.W_g) (.) (X.W_u)).  §5.4.3 requires the
 * fused program to keep the rounding of the unfused one: each product is
 * accumulated in FP32 and rounded once to bf16 before the activation, and
 * every intermediate the unfused program would store as bf16 is rounded to
 * bf16.  SiLU(x) = x / (1 + e^-x), evaluated in FP32.
 *
 * Both calls take bf16 operands (bit patterns), write a bf16 result and
 * follow gemm_bf16 for layout, ownership, streams, determinism and errors,
 * with these additions.  GEMM_ERR_UNSUPPORTED: the output rows are not
 * 16-byte aligned (C or Z pointer and ldc/ldz), N is not a multiple of 8,
 * or no LDS-ring kernel can run the call (B rows not 16-byte aligned, or an
 * operand spanning 2 GiB or more, or A rows only 2-byte aligned without a
 * workspace).  With a workspace (gemm_run) A's rows, when not 16-byte
 * aligned, are first copied to aligned rows, at any size of the product.
 * K == 0 writes zeros (SiLU(0) = 0).
 */

/* C [M,N] := bf16(SiLU(bf16(A.B))): A [M,K], B [K,N] as in gemm_bf16. */
int gemm_bf16_silu(int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb,
                   uint16_t *C, int64_t ldc,
                   void *stream);

/* SwiGLU with a merged gate|up weight: X [M,K]; Wgu [K,2N] (ldw >= 2N)
 * holds W_g in columns 0..N-1 and W_u in columns N..2N-1.  With
 * g = bf16(X.W_g), u = bf16(X.W_u) and t = bf16(SiLU(g)), elementwise,
 * Z [M,N] := bf16(t * u). */
int gemm_bf16_swiglu(int64_t M, int64_t N, int64_t K,
                     const uint16_t *X, int64_t ldx,
                     const uint16_t *Wgu, int64_t ldw,
                     uint16_t *Z, int64_t ldz,
                     void *stream);

/* Batched forms (each entry as the single call, strides in elements as in
 * gemm_bf16_batched, 0 broadcasting an operand): e.g. the experts of a
 * mixture-of-experts FFN, each with its own tokens and weights. */
int gemm_bf16_silu_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                           const uint16_t *A, int64_t lda, int64_t strideA,
                           const uint16_t *B, int64_t ldb, int64_t strideB,
                           uint16_t *C, int64_t ldc, int64_t strideC,
                           void *stream);
int gemm_bf16_swiglu_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                             const uint16_t *X, int64_t ldx, int64_t strideX,
                             const uint16_t *Wgu, int64_t ldw, int64_t strideW,
                             uint16_t *Z, int64_t ldz, int64_t strideZ,
                             void *stream);

/* ---- the activation chain on stored operands -----------------------------
 *
 * "Operator & Runtime" §5.3.1, Example 5-4: with G = X.W_g and U = X.W_u
 * already stored (bf16 [M,N], e.g. by two separate projections), the chain
 * computes T = SiLU(G), Z = T (.) U and quantizes Z to one byte with a fixed
 * scale factor -- each step as its own pass over HBM, or fused so that the
 * intermediates are never written and read back (the page counts 156 MiB of
 * traffic for the three passes at [1024, 12288], 108 with the first two
 * fused, 60 with all three).  Element by element, as the fused epilogues:
 * t = bf16(SiLU(g)) in FP32, z = bf16(t * u), and the code of z as
 * gemm_bf16_swiglu_e4m3 forms it against the range amax; so a fused step
 * gives the same bits as the separate steps in sequence. */
typedef enum {
    GEMM_ACT_SILU = 0,        /* out = T [M,N] bf16 from in0 = G */
    GEMM_ACT_MUL = 1,         /* out = Z [M,N] bf16 from in0 = T, in1 = U */
    GEMM_ACT_SWIGLU = 2,      /* out = Z bf16 from in0 = G, in1 = U (SiLU and product fused) */
    GEMM_ACT_QUANT = 3,       /* out = E4M3FN codes [M,N] (uint8_t) of in0 = Z against amax */
    GEMM_ACT_SWIGLU_E4M3 = 4  /* out = the codes of Z from in0 = G, in1 = U (all three fused) */
} gemm_act_step;

/* One step of the chain: in0 and in1 (the latter read by the two-input steps
 * only, else ignored) bf16 bit patterns [M,N] with row strides ld0, ld1; out
 * [M,N] with row stride ldo, all strides in elements (bytes for codes); amax
 * read by the quantizing steps only (finite, > 0).  Device pointers; the
 * caller owns the memory; enqueued on `stream`.  Rows of whole 16-byte
 * chunks at 16-byte aligned starts (8-byte for codes) stream 16 bytes per
 * lane; any other shape or alignment runs element by element, with the same
 * results.  Deterministic.  Errors, nothing enqueued: GEMM_ERR_INVALID_ARG
 * for an unknown step, M or N < 0, a missing pointer, a stride below N, a
 * misaligned element, the output overlapping an input (no in-place form),
 * or a bad amax; M == 0 or N == 0 is a no-op. */
int gemm_act_chain(int step, int64_t M, int64_t N,
                   const uint16_t *in0, int64_t ld0,
                   const uint16_t *in1, int64_t ld1,
                   void *out, int64_t ldo, float amax,
                   void *stream);

/* SwiGLU with its output stored as one byte per element ("Operator &
 * Runtime" §5.3.1 carries Example 5-4 on: Z is quantized with one fixed
 * scale factor, and fusing the quantization too leaves the reads of the
 * operands and the write of the codes).  What is quantized is the bf16
 * output of gemm_bf16_swiglu, z = bf16(t * u), the value the unfused program
 * stores, so the codes equal gemm_act_chain's quantization of that output
 * bit for bit; Zq [M,N] (uint8_t, ldz and strideZ in bytes) receives the
 * E4M3FN code nearest to the binary32 quotient fl(z * 448 / amax) (ties to
 * the even mantissa; beyond +-448 saturating to +-448; NaN to 0x7f).  amax is the caller's fixed range:
 * the magnitude that maps to 448, so the codes dequantize by the factor
 * amax / 448; finite and > 0, else GEMM_ERR_INVALID_ARG.  Everything else
 * -- operands, ownership, streams, determinism, the other errors (16-byte
 * aligned Zq rows: pointer and ldz multiples of 16 bytes) -- as
 * gemm_bf16_swiglu and its batched form. */
int gemm_bf16_swiglu_e4m3(int64_t M, int64_t N, int64_t K,
                          const uint16_t *X, int64_t ldx,
                          const uint16_t *Wgu, int64_t ldw,
                          uint8_t *Zq, int64_t ldz, float amax,
                          void *stream);
int gemm_bf16_swiglu_e4m3_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                  const uint16_t *X, int64_t ldx, int64_t strideX,
                                  const uint16_t *Wgu, int64_t ldw, int64_t strideW,
                                  uint8_t *Zq, int64_t ldz, int64_t strideZ, float amax,
                                  void *stream);

/* ---- affine epilogue -------------------------------------------------------
 *
 * C := alpha * (A.B) + bias + beta * C, the scaling and accumulation of the
 * BLAS GEMM and the bias of a linear layer, applied to the finished output
 * tile like the activations above.  The pages fix no formula for it; the
 * reading here keeps the rounding rule of "Operator & Runtime" §5.4.3: the
 * product is accumulated in FP32 and
 *
 *     C[i][j] := round(fma(alpha, S[i][j], fma(beta, C_old[i][j], bias[j])))
 *
 * is evaluated in FP32 and rounded once to C's type (bf16 RNE, or float).
 * bias is a bf16 vector of N elements (bit patterns, any 2-byte alignment)
 * shared by every row and batch entry, or NULL for none.  C is read only
 * when beta != 0 (so with beta == 0 its old contents, NaN included, do not
 * matter), and A and B only when alpha != 0 and K > 0; otherwise the call
 * computes bias[j] + beta * C_old[i][j] element by element.
 *
 * Arguments follow gemm_bf16_batched (batch 1 for a single product), plus:
 * GEMM_ERR_INVALID_ARG when alpha or beta is not finite, bias is not 2-byte
 * aligned, or bias overlaps C; GEMM_ERR_UNSUPPORTED as for the fused
 * epilogues above (16-byte aligned rows of C, N % 8 == 0, B rows 16-byte
 * aligned) when a product is formed on the tiled kernels.  M <= 16 runs
 * the small-M kernels of gemm_bf16, whose final store applies the same
 * formula (there B may have any alignment).  With a workspace (gemm_run),
 * small outputs split K over workgroups as gemm_bf16 does (the workgroup
 * that completes a tile applies the epilogue, once).
 */
int gemm_bf16_affine(int64_t batch, int64_t M, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda, int64_t strideA,
                     const uint16_t *B, int64_t ldb, int64_t strideB,
                     float alpha, const uint16_t *bias, float beta,
                     void *C, int64_t ldc, int64_t strideC, int c_type,
                     void *stream);

/* The same with B given transposed as in gemm_bf16_nt: Bt [N,K] row-major
 * (ldbt >= K), the [out, in] weight of a linear layer, so that
 * C := alpha * (A . Bt^T) + bias + beta * C is the layer's output with its
 * bias and, with beta = 1, a residual add.  M <= 16 with 16-byte aligned Bt
 * rows runs the small-M transposed-B kernel, which applies the same
 * epilogue; other calls follow gemm_bf16_nt for the realignment of Bt
 * rows. */
int gemm_bf16_nt_affine(int64_t batch, int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda, int64_t strideA,
                        const uint16_t *Bt, int64_t ldbt, int64_t strideBt,
                        float alpha, const uint16_t *bias, float beta,
                        void *C, int64_t ldc, int64_t strideC, int c_type,
                        void *stream);

/* The same with A given transposed as in gemm_bf16_tn: At [K,M] row-major
 * (ldat >= M), so that with beta = 1 the call accumulates a weight gradient,
 * dW := dW + X^T . dY, in place (C in float keeps the accumulation in FP32).
 * Every size runs on the tiled kernels; At rows are realigned as in
 * gemm_bf16_tn. */
int gemm_bf16_tn_affine(int64_t batch, int64_t M, int64_t N, int64_t K,
                        const uint16_t *At, int64_t ldat, int64_t strideAt,
                        const uint16_t *B, int64_t ldb, int64_t strideB,
                        float alpha, const uint16_t *bias, float beta,
                        void *C, int64_t ldc, int64_t strideC, int c_type,
                        void *stream);

/* Bytes at the start of a gemm_run workspace that hold arrival counters and
 * exchange slots (zero between calls). */
#define GEMM_WORKSPACE_COUNTER_BYTES (1u << 20)

/* ---- one entry point for every operation, with a caller workspace --------
 *
 * gemm_run performs the call that the named entry point of `op` (a
 * gemm_op, below) would, with the same arguments and semantics, and may in
 * addition use `workspace`: device memory of `workspace_bytes` bytes on the
 * current device, owned by the caller, 256-byte aligned, holding at least
 * what gemm_workspace_size reports for the same call (GEMM_ERR_WORKSPACE
 * otherwise; NULL runs the call without scratch, exactly as the named entry
 * point).  Its first GEMM_WORKSPACE_COUNTER_BYTES (1 MiB) hold arrival
 * counters and exchange slots: they must be zero before a workspace is
 * first used (e.g. zero-filled at allocation) and every call leaves them
 * zero when it completes; the rest needs no initial value.
 * A workspace serves one call at a time: calls that may overlap in time
 * (on different streams) need different workspaces; calls on one stream
 * may share one.
 * Arguments: A, lda, strideA and B, ldb, strideB as the op's entry point
 * names them (A = At for the TN ops, B = Bt for the NT and FP8 ops, B = Wgu
 * for SwiGLU), batch 1 for GEMM_OP_SGEMM (the one op without a batched
 * form); c_type is ignored where the op fixes it (SGEMM: float;
 * SiLU: bf16; SwiGLU: bf16 unless c_type is GEMM_OUT_E4M3, which writes the
 * codes of gemm_bf16_swiglu_e4m3 with alpha as the range amax); alpha, bias
 * and beta are read by the affine ops only (and alpha by that SwiGLU form),
 * scale_a and scale_b by the FP8 ops only. */
int gemm_run(int op, int64_t batch, int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda, int64_t strideA,
             const void *B, int64_t ldb, int64_t strideB,
             void *C, int64_t ldc, int64_t strideC, int c_type,
             float alpha, const uint16_t *bias, float beta,
             const float *scale_a, const float *scale_b,
             void *workspace, uint64_t workspace_bytes,
             void *stream);

/* For callers that cannot allocate a workspace -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: gemm_run
 * with the library's own scratch memory in place of a caller workspace.
 * That memory is a file-scope device array of 16 MiB, one copy per GPU the
 * library runs on (kept until the process ends), shared by every
 * gemm_run_noalloc call on that GPU and keeping the last call's contents;
 * each call first clears the arrival counters it uses (a small fill kernel
 * on `stream`), then runs as gemm_run.  Calls that overlap in time on one
 * GPU (several streams or threads) race on it: the caller must order them.
 * A call whose plan needs more than 16 MiB (gemm_workspace_size) returns
 * GEMM_ERR_WORKSPACE and enqueues nothing.  Allocates nothing: no hipMalloc,
 * hipFree or allocating library call.  Arguments, results and the other
 * errors as gemm_run. */
int gemm_run_noalloc(int op, int64_t batch, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, int64_t strideA,
                     const void *B, int64_t ldb, int64_t strideB,
                     void *C, int64_t ldc, int64_t strideC, int c_type,
                     float alpha, const uint16_t *bias, float beta,
                     const float *scale_a, const float *scale_b,
                     void *stream);

/* Workspace bytes gemm_run needs for a call (0: none; host only, no GPU
 * work).  Arguments as gemm_plan_query; writes *bytes and returns the
 * validation status. */
int gemm_workspace_size(int op, int64_t batch, int64_t M, int64_t N, int64_t K,
                        uint64_t a_addr, int64_t lda, int64_t strideA,
                        uint64_t b_addr, int64_t ldb, int64_t strideB,
                        uint64_t c_addr, int64_t ldc, int64_t strideC,
                        int c_type, uint64_t *bytes);

/* Static, NUL-terminated description of a status code. */
const char *gemm_status_string(int status);

/* ---- host-only queries (no GPU work, usable without a device) ------------ */

/* Kernel families the selector chooses between. */
typedef enum {
    GEMM_FAMILY_NONE = 0,      /* nothing to launch (empty problem) */
    GEMM_FAMILY_ZERO = 1,      /* K == 0: fill C with zeros */
    GEMM_FAMILY_BF16_MFMA = 2, /* tiled bf16 MFMA kernel */
    GEMM_FAMILY_F32_MFMA = 3,  /* tiled f32 MFMA kernel */
    GEMM_FAMILY_DECODE = 4,    /* small-M bf16 path (M <= 16) */
    GEMM_FAMILY_GENERIC = 5    /* any shape/alignment, LDS-tiled vector ALU */
} gemm_family;

/* What a call would launch.  Filled by gemm_plan_query. */
typedef struct {
    int family;        /* gemm_family */
    int config_id;     /* index of the compiled kernel configuration */
    int tile_m, tile_n, tile_k;
    int threads;       /* per workgroup */
    int vec_a, vec_b;  /* bytes per global load of A and of B rows (16 for A
                          when its rows are realigned first) */
    int even;          /* 1 when no edge masking is compiled in */
    int variant;       /* tiled kernels: 0 fully general (register-staged copies),
                          1 aligned LDS-ring kernel, 2/3 masked LDS-ring kernel
                          copying A in 16-/4-byte pieces; the small-M
                          family: 1 for whole aligned column chunks, else 0;
                          other families: 0 */
    int64_t grid;      /* workgroups launched */
    int64_t lds_bytes; /* LDS per workgroup */
    double model_bytes;/* traffic model of "Operator & Runtime" §5.2.2 for the chosen tile */
    char name[48];     /* configuration name, as accepted by GEMM_FORCE_CONFIG */
    int64_t workspace_bytes; /* workspace the planned call needs (gemm_run):
                                the 1 MiB counter region plus the partial
                                sums of the split small-M path or of a
                                K-split tiled call and the realigned row
                                copies of A and Bt, each rounded up to 256
                                bytes; 0 when it needs none */
    int ksplit;        /* tiled bf16 calls: workgroups sharing each output
                          tile's K range (1: no split); grid counts them all */
    int streamk;       /* 1: the persistent stream-K schedule (grid = one
                          workgroup per CU, each walking an equal share of
                          the (tile, K stage) pairs) */
} gemm_plan;

/* Operation selector for gemm_plan_query. */
typedef enum {
    GEMM_OP_SGEMM = 0,       /* gemm_sgemm */
    GEMM_OP_BF16 = 1,        /* gemm_bf16, gemm_bf16_batched */
    GEMM_OP_BF16_SILU = 2,   /* gemm_bf16_silu(_batched) (c_type ignored) */
    GEMM_OP_BF16_SWIGLU = 3, /* gemm_bf16_swiglu(_batched) (b = Wgu; c_type GEMM_OUT_E4M3:
                                gemm_bf16_swiglu_e4m3(_batched), range in alpha) */
    GEMM_OP_BF16_NT = 4,     /* gemm_bf16_nt, gemm_bf16_nt_batched (b = Bt, ldb = ldbt) */
    GEMM_OP_FP8_NT = 5,      /* gemm_fp8_nt(_batched) (b = Bt; scales do not change the plan) */
    GEMM_OP_BF16_AFFINE = 6, /* gemm_bf16_affine with alpha = 1 (alpha, beta and bias do not change the
                                plan; alpha == 0 plans the element-wise pass of K == 0) */
    GEMM_OP_BF16_TN = 7,     /* gemm_bf16_tn, gemm_bf16_tn_batched (a = At, lda = ldat) */
    GEMM_OP_BF16_NT_AFFINE = 8, /* gemm_bf16_nt_affine with alpha = 1 (b = Bt, ldb = ldbt) */
    GEMM_OP_BF16_TN_AFFINE = 9, /* gemm_bf16_tn_affine with alpha = 1 (a = At, lda = ldat) */
    GEMM_OP_FP8_NT_AFFINE = 10  /* gemm_fp8_nt_affine with alpha = 1 (b = Bt, ldb = ldbt) */
} gemm_op;

/* Validate the arguments of a call and report the plan gemm_run launches
 * for it with a sufficient workspace, without touching the GPU.  Pointers
 * are passed as integers (their values only decide alignment and overlap).
 * Returns the status the call would return from validation (GEMM_OK,
 * GEMM_ERR_INVALID_ARG or GEMM_ERR_UNSUPPORTED); `out` may be NULL. */
int gemm_plan_query(int op, int64_t batch, int64_t M, int64_t N, int64_t K,
                    uint64_t a_addr, int64_t lda, int64_t strideA,
                    uint64_t b_addr, int64_t ldb, int64_t strideB,
                    uint64_t c_addr, int64_t ldc, int64_t strideC,
                    int c_type, gemm_plan *out);
/* The same, for a call with (with_workspace != 0) or without a workspace:
 * the named entry points run the plan without. */
int gemm_plan_query_ex(int with_workspace, int op, int64_t batch, int64_t M, int64_t N, int64_t K,
                       uint64_t a_addr, int64_t lda, int64_t strideA,
                       uint64_t b_addr, int64_t ldb, int64_t strideB,
                       uint64_t c_addr, int64_t ldc, int64_t strideC,
                       int c_type, gemm_plan *out);

/* Tile traffic model of "Operator & Runtime" §5.2.2 (Example 5-3): for an
 * m x n output tile with reduction slab k and element size e bytes (FP32
 * accumulator of 4 bytes), local memory S = e*m*k + e*k*n + 4*m*n bytes and
 * interface traffic V = e*M*K*ceil(N/n) + e*K*N*ceil(M/m) + e*M*N bytes. */
int64_t gemm_model_local_bytes(int64_t m, int64_t n, int64_t k, int64_t elem_bytes);
double gemm_model_traffic_bytes(int64_t M, int64_t N, int64_t K, int64_t m, int64_t n,
                                int64_t elem_bytes);

/* Traffic of quantizing a GEMM input per row, "Operator & Runtime" §5.4.3
 * Example 5-8: input A [M,K] of in_bytes per element quantized to q_bytes,
 * weights [K,N] of w_bytes, output [M,N] of out_bytes, m x n output tiles,
 * factors from each row's maximum.  Quantizing separately reads A once,
 * writes the codes and has each of the ceil(N/n) column blocks read the
 * codes; quantizing inside the GEMM reads A once for the factors and has
 * every column block read A again.  Both add ceil(M/m) reads of the weights
 * and one write of the output.  Writes the two byte counts (either pointer
 * may be NULL). */
void gemm_model_quant_traffic(int64_t M, int64_t N, int64_t K, int64_t m, int64_t n, int64_t in_bytes,
                              int64_t q_bytes, int64_t w_bytes, int64_t out_bytes, double *separate,
                              double *fused);

/* Traffic of one gemm_act_chain call of step `step` on [M,N] operands
 * ("Operator & Runtime" §5.3.1, Example 5-4): every input read once and the
 * output written once, bf16 2 bytes and codes 1 byte per element -- SiLU
 * 4MN, the product 6MN, SiLU and product fused 6MN, the quantization 3MN,
 * all three fused 5MN.  A program's traffic is the sum over its calls (the
 * page's 120, 72, 156, 108 and 60 MiB at [1024, 12288]).  0 for an unknown
 * step or negative sizes. */
double gemm_model_act_chain_bytes(int step, int64_t M, int64_t N);

/* The workgroup -> output-tile map used by the tiled kernels: workgroup id
 * `wg` of a launch covering `batch` x tiles_m x tiles_n tiles is assigned
 * (b, tm, tn).  Workgroups are dispatched round-robin over the chip's 8
 * accelerator complex dies (XCDs); the map gives each XCD a contiguous run
 * of tiles, ordered in column bands `group_m` tiles tall, so that the tiles
 * resident on one XCD share rows of A and columns of B in that die's L2.
 * group_m <= 0 gives the orders it is measured against (environment
 * GEMM_TILE_ORDER): 0 plain row-major order, -g column bands g tiles tall
 * without the per-XCD gathering.  The map is a bijection on
 * [0, batch*tiles_m*tiles_n).  Returns 0, or -1 for out-of-range arguments. */
int gemm_tile_map(int64_t wg, int64_t batch, int64_t tiles_m, int64_t tiles_n,
                  int64_t group_m, int64_t *b, int64_t *tm, int64_t *tn);

#ifdef __cplusplus
}
#endif

#endif /* GEMM05_H */
