// g5_kernels.hip -- gfx950 (CDNA4) kernels of the dense-GEMM library.
//
// Every kernel computes C[i][j] = sum_k A[i][k] B[k][j] for row-major
// operands (page "4.1 Tối ưu hiệu năng toán tử GEMM trên CUDA", §1.1; page
// "Operator & Runtime", §5.2.1).  The tiled kernels follow the structure that
// both pages build up -- an output tile per workgroup, K walked in slabs
// staged through on-chip memory, double buffered, accumulators kept in
// registers -- re-designed for the CDNA4 execution model:
//
//  * 64-lane waves; the inner product runs on the matrix cores
//    (v_mfma_f32_16x16x32_bf16 for bf16, v_mfma_f32_16x16x4_f32 for fp32).
//  * Each wave computes its sub-tile transposed, D = B^T A^T, so that a lane
//    ends up owning 4 consecutive columns of one row of C and can store them
//    with one 8-byte (bf16) or 16-byte (fp32) write.
//  * The bf16 B operand (N-contiguous in memory, needed K-contiguous per lane
//    by the matrix core) is read from LDS with the gfx950 transposing read
//    ds_read_b64_tr_b16; A (K-contiguous) is read with ds_read_b128.
//  * LDS layouts use XOR swizzles of 16-byte chunks so that the fragment
//    reads spread over the LDS banks (the padding/XOR remedies of page "4.1"
//    §8.5 and "Operator & Runtime" §5.2.3, with gfx950 constants).
//  * Out-of-range elements of A and B load as zero and only in-range
//    elements of C are written (page "4.1" §4.5; "Operator & Runtime" §5.4.2
//    masked last tile).  The FP32 sum of a bf16 output is rounded once, to
//    nearest even ("Operator & Runtime" §5.4.3).
#include <hip/hip_runtime.h>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

// ===================================================== bf16 tiled MFMA kernel
//
// Workgroup tile BM x BN, K slab 64, WGM x WGN waves each owning a
// (BM/WGM) x (BN/WGN) sub-tile as 16x16 MFMA blocks.  Two LDS buffers; the
// global loads of slab k+1 are issued before the MFMAs of slab k and written
// to the other buffer after them, with one barrier per slab (page "4.1" §9.4;
// MUSA lesson m11-l5 case 4 double buffering).
template <int BM, int BN, int WGM, int WGN, bool EVEN>
__global__ void __launch_bounds__(WGM *WGN * 64, 1) k_bf16_mfma(GemmArgs p)
{
    constexpr int T = WGM * WGN * 64;
    constexpr int BK = 64;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int A_CPR = BK / 8;            // 16-byte chunks per A slab row
    constexpr int B_CPR = BN / 8;            // chunks per B slab row
    constexpr int CA = BM * A_CPR / T;       // A chunks per thread
    constexpr int CB = BK * B_CPR / T;       // B chunks per thread
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole MFMA blocks");
    static_assert((BM * A_CPR) % T == 0 && (BK * B_CPR) % T == 0, "slab chunks must divide threads");
    static_assert(B_CPR % 8 == 0, "B slab rows must be whole swizzle groups");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (A_ELEMS + B_ELEMS)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, li = lane & 15;

    const TileCoord tc = tile_map(blockIdx.x, p.batch, p.tiles_m, p.tiles_n, p.group_m);
    const int64_t m0 = tc.tm * BM, n0 = tc.tn * BN;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint16_t *Ab = (const uint16_t *)p.A + tc.b * p.sA + m0 * lda;
    const uint16_t *Bb = (const uint16_t *)p.B + tc.b * p.sB + n0;

    // Per-thread chunk coordinates in the slabs.
    int a_row[CA], a_c[CA], b_row[CB], b_c[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int q = tid + T * i;
        a_row[i] = q / A_CPR;
        a_c[i] = q % A_CPR;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int q = tid + T * i;
        b_row[i] = q / B_CPR;
        b_c[i] = q % B_CPR;
    }

    u32x4 ra[CA], rb[CB];
    auto load_slab = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const uint16_t *row = Ab + (int64_t)a_row[i] * lda;
            if (EVEN) {
                ra[i] = *(const u32x4 *)(row + k0 + a_c[i] * 8);
            } else {
                ra[i] = load_chunk8_bf16(row, k0 + a_c[i] * 8, K, m0 + a_row[i] < M, p.align_a);
            }
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int64_t k = k0 + b_row[i];
            const uint16_t *row = Bb + k * ldb;
            if (EVEN) {
                rb[i] = *(const u32x4 *)(row + b_c[i] * 8);
            } else {
                rb[i] = load_chunk8_bf16(row, b_c[i] * 8, N - n0, k < K, p.align_b);
            }
        }
    };
    auto store_slab = [&](int buf) {
        uint16_t *As = smem + buf * (A_ELEMS + B_ELEMS);
        uint16_t *Bs = As + A_ELEMS;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            *(u32x4 *)(As + a_row[i] * BK + ((a_c[i] ^ swz_a(a_row[i])) * 8)) = ra[i];
#pragma unroll
        for (int i = 0; i < CB; ++i)
            *(u32x4 *)(Bs + b_row[i] * BN + ((b_c[i] ^ swz_b(b_row[i])) * 8)) = rb[i];
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = (int)((K + BK - 1) / BK);
    load_slab(0);
    store_slab(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_slab(kt + 1);
        const uint16_t *As = smem + cur * (A_ELEMS + B_ELEMS);
        const uint16_t *Bs = As + A_ELEMS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * TM + fm * 16 + li;
                const int c = ks * 4 + g;
                const u32x4 v = *(const u32x4 *)(As + row * BK + ((c ^ swz_a(row)) * 8));
                af[fm] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int k = ks * 32 + g * 8 + (li >> 2);
                const int ncol = wn * TN + fn * 16 + (li & 3) * 4;
                const int c = ncol >> 3, half = (ncol >> 2) & 1;
                const uint16_t *p0 = Bs + k * BN + ((c ^ swz_b(k)) * 8) + half * 4;
                const uint16_t *p1 = Bs + (k + 4) * BN + ((c ^ swz_b(k + 4)) * 8) + half * 4;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G5_LDS(i16x4, p0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G5_LDS(i16x4, p1));
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                bfr[fn] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], af[fm], acc[fn][fm], 0, 0, 0);
        }
        if (kt + 1 < KT) store_slab(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: lane (g, li) of block (fn, fm) holds C[m][n..n+3].
    void *Cb = (char *)p.C + tc.b * p.sC * (p.out_f32 ? 4 : 2);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t m = m0 + wm * TM + fm * 16 + li;
            const int64_t n = n0 + wn * TN + fn * 16 + g * 4;
            const bool full = EVEN || (m < M && n + 4 <= N);
            if (!EVEN && (m >= M || n >= N)) continue;
            store4(Cb, p.out_f32 != 0, p.ldc, m, n, acc[fn][fm], full, M, N, p.align_c);
        }
}

// ===================================================== fp32 tiled MFMA kernel
//
// Same structure with fp32 operands: K slab 32 floats, MFMA 16x16x4 f32.
// Within a 16-deep K step, the 4 MFMAs q = 0..3 use k = 4*g + q for lane
// group g, so one 16-byte LDS read of an A row feeds 4 MFMAs.  B rows are
// padded by 4 floats so the 4 lane groups (rows 4 apart) hit different banks.
template <int BM, int BN, int WGM, int WGN, bool EVEN>
__global__ void __launch_bounds__(WGM *WGN * 64, 2) k_f32_mfma(GemmArgs p)
{
    constexpr int T = WGM * WGN * 64;
    constexpr int BK = 32;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int A_CPR = BK / 4;            // 16-byte chunks per A slab row (8)
    constexpr int B_CPR = BN / 4;
    constexpr int BLD = BN + 4;              // padded B slab row, floats
    constexpr int CA = BM * A_CPR / T;
    constexpr int CB = BK * B_CPR / T;
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BLD;
    static_assert((BM * A_CPR) % T == 0 && (BK * B_CPR) % T == 0, "slab chunks must divide threads");
    __shared__ __attribute__((aligned(16))) float smem[2 * (A_ELEMS + B_ELEMS)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, li = lane & 15;

    const TileCoord tc = tile_map(blockIdx.x, p.batch, p.tiles_m, p.tiles_n, p.group_m);
    const int64_t m0 = tc.tm * BM, n0 = tc.tn * BN;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const float *Ab = (const float *)p.A + tc.b * p.sA + m0 * lda;
    const float *Bb = (const float *)p.B + tc.b * p.sB + n0;

    int a_row[CA], a_c[CA], b_row[CB], b_c[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int q = tid + T * i;
        a_row[i] = q / A_CPR;
        a_c[i] = q % A_CPR;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int q = tid + T * i;
        b_row[i] = q / B_CPR;
        b_c[i] = q % B_CPR;
    }

    u32x4 ra[CA], rb[CB];
    auto load_slab = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const float *row = Ab + (int64_t)a_row[i] * lda;
            if (EVEN) ra[i] = *(const u32x4 *)(row + k0 + a_c[i] * 4);
            else ra[i] = load_chunk4_f32(row, k0 + a_c[i] * 4, K, m0 + a_row[i] < M, p.align_a);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int64_t k = k0 + b_row[i];
            const float *row = Bb + k * ldb;
            if (EVEN) rb[i] = *(const u32x4 *)(row + b_c[i] * 4);
            else rb[i] = load_chunk4_f32(row, b_c[i] * 4, N - n0, k < K, p.align_b);
        }
    };
    auto store_slab = [&](int buf) {
        float *As = smem + buf * (A_ELEMS + B_ELEMS);
        float *Bs = As + A_ELEMS;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            *(u32x4 *)(As + a_row[i] * BK + ((a_c[i] ^ swz_a(a_row[i])) * 4)) = ra[i];
#pragma unroll
        for (int i = 0; i < CB; ++i) *(u32x4 *)(Bs + b_row[i] * BLD + b_c[i] * 4) = rb[i];
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = (int)((K + BK - 1) / BK);
    load_slab(0);
    store_slab(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_slab(kt + 1);
        const float *As = smem + cur * (A_ELEMS + B_ELEMS);
        const float *Bs = As + A_ELEMS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f32x4 af[FM];
            float bfr[FN][4];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * TM + fm * 16 + li;
                const int c = ks * 4 + g;
                af[fm] = *(const f32x4 *)(As + row * BK + ((c ^ swz_a(row)) * 4));
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    bfr[fn][q] = Bs[(ks * 16 + g * 4 + q) * BLD + wn * TN + fn * 16 + li];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
                        acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x4f32(bfr[fn][q], af[fm][q], acc[fn][fm], 0, 0, 0);
        }
        if (kt + 1 < KT) store_slab(cur ^ 1);
        __syncthreads();
    }

    float *Cb = (float *)p.C + tc.b * p.sC;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t m = m0 + wm * TM + fm * 16 + li;
            const int64_t n = n0 + wn * TN + fn * 16 + g * 4;
            if (!EVEN && (m >= M || n >= N)) continue;
            const bool full = EVEN || (m < M && n + 4 <= N);
            store4(Cb, true, p.ldc, m, n, acc[fn][fm], full, M, N, p.align_c);
        }
}

// FP32, all of K staged at once (K <= KMAX, whole tiles, 16-byte aligned
// rows).  A small problem gives each CU only a few slabs to multiply, so the
// double-buffered kernel above spends its time on one global-load latency per
// slab in sequence.  Here every thread issues the loads of every slab of its
// tile before the first is stored to LDS, so the tile waits for one latency,
// then multiplies all slabs from LDS with a single barrier.  Slab layout and
// fragment reads are those of k_f32_mfma.
template <int BM, int BN, int WGM, int WGN, int KMAX>
__global__ void __launch_bounds__(WGM *WGN * 64, 2) k_f32_wholek(GemmArgs p)
{
    constexpr int T = WGM * WGN * 64;
    constexpr int BK = 32;
    constexpr int NS = KMAX / BK;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int A_CPR = BK / 4;
    constexpr int B_CPR = BN / 4;
    constexpr int BLD = BN + 4;
    constexpr int CA = BM * A_CPR / T;
    constexpr int CB = BK * B_CPR / T;
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BLD;
    static_assert((BM * A_CPR) % T == 0 && (BK * B_CPR) % T == 0 && CA >= 1 && CB >= 1, "slab chunks must divide threads");
    __shared__ __attribute__((aligned(16))) float smem[NS * (A_ELEMS + B_ELEMS)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, li = lane & 15;
    const TileCoord tc = tile_map(blockIdx.x, p.batch, p.tiles_m, p.tiles_n, p.group_m);
    const int64_t m0 = tc.tm * BM, n0 = tc.tn * BN;
    const int64_t lda = p.lda, ldb = p.ldb;
    const float *Ab = (const float *)p.A + tc.b * p.sA + m0 * lda;
    const float *Bb = (const float *)p.B + tc.b * p.sB + n0;
    const int KT = (int)(p.K / BK);                  // 1 <= KT <= NS (host checked)

    u32x4 ra[NS][CA], rb[NS][CB];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s >= KT) break;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int q = tid + T * i, row = q / A_CPR, c = q % A_CPR;
            ra[s][i] = *(const u32x4 *)(Ab + (int64_t)row * lda + s * BK + c * 4);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int q = tid + T * i, k = q / B_CPR, c = q % B_CPR;
            rb[s][i] = *(const u32x4 *)(Bb + (int64_t)(s * BK + k) * ldb + c * 4);
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s >= KT) break;
        float *As = smem + s * (A_ELEMS + B_ELEMS);
        float *Bs = As + A_ELEMS;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int q = tid + T * i, row = q / A_CPR, c = q % A_CPR;
            *(u32x4 *)(As + row * BK + ((c ^ swz_a(row)) * 4)) = ra[s][i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int q = tid + T * i, k = q / B_CPR, c = q % B_CPR;
            *(u32x4 *)(Bs + k * BLD + c * 4) = rb[s][i];
        }
    }
    __syncthreads();

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < KT; ++kt) {
        const float *As = smem + kt * (A_ELEMS + B_ELEMS);
        const float *Bs = As + A_ELEMS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f32x4 af[FM];
            float bfr[FN][4];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * TM + fm * 16 + li;
                const int c = ks * 4 + g;
                af[fm] = *(const f32x4 *)(As + row * BK + ((c ^ swz_a(row)) * 4));
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) bfr[fn][q] = Bs[(ks * 16 + g * 4 + q) * BLD + wn * TN + fn * 16 + li];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
                        acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x4f32(bfr[fn][q], af[fm][q], acc[fn][fm], 0, 0, 0);
        }
    }

    float *Cb = (float *)p.C + tc.b * p.sC;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t m = m0 + wm * TM + fm * 16 + li;
            const int64_t n = n0 + wn * TN + fn * 16 + g * 4;
            store4(Cb, true, p.ldc, m, n, acc[fn][fm], true, p.M, p.N, p.align_c);
        }
}

// ========================================================= small-M (decode)
//
// C[M,N] = X[M,K] . W[K,N] for M <= 16 is bound by streaming W once from HBM
// (arithmetic intensity about M FLOP per byte; MUSA lesson m11-l5, case 2
// GEMV; "Operator & Runtime" §5.2.4 on splitting a single decode row's
// reduction to occupy the device).  Design:
//  * a workgroup owns 64 columns of W and all of K; its NW waves split K in a
//    fixed partition that does not depend on M, and their partial sums are
//    added in wave order through LDS (no atomics: bitwise reproducible and
//    independent of how many rows the call has; "Operator & Runtime" §5.2.4);
//  * lane (g, r) streams 8 rows x 8 bytes of W straight into registers --
//    each load instruction reads 4 rows x 128 contiguous bytes, marked
//    non-temporal (W is read once; measured 8% faster streaming) -- and a
//    4x8 transpose of 16-bit halves in registers turns them into the
//    K-contiguous operands of 4 matrix-core blocks, whose logical column r
//    maps to physical column 4r + b;
//  * X rows (zero beyond M) are the other MFMA operand; the 16-row MFMA
//    covers any M <= 16 at no extra memory traffic.
//
// GLU: SwiGLU epilogue -- the workgroup's 64 output columns take their gate
// sums from columns n of the merged weight [K, 2N] and their up sums from
// columns N + n, both accumulated in the same pass over K.
template <int NW, bool FAST, bool GLU>
__global__ void __launch_bounds__(NW * 64, 1) k_decode(GemmArgs p)
{
    constexpr int NC = 64;                   // output columns per workgroup
    constexpr int NB = GLU ? 2 : 1;          // column groups read per row: gate (and up)
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int64_t n0 = (int64_t)blockIdx.x * NC;
    const int64_t bidx = blockIdx.y;
    const uint16_t *X = (const uint16_t *)p.A + bidx * p.sA;
    const uint16_t *W = (const uint16_t *)p.B + bidx * p.sB;

    // Fixed partition of the 32-row K steps over the waves (independent of M).
    const int64_t steps = (K + 31) / 32, full = K / 32;
    const int64_t s_begin = steps * wave / NW, s_end = steps * (wave + 1) / NW;
    const int64_t s_full_end = s_end < full ? s_end : full;
    const int64_t ncol = n0 + 4 * li;        // first of this lane's 4 columns
    const bool m_ok = li < M;
    // This lane's X row (row 0 stands in for rows beyond M; zeroed below).
    const uint16_t *xr = X + (int64_t)(m_ok ? li : 0) * lda;
    const uint16_t *wcol = W + ncol;

    f32x4 acc[4 * NB];
#pragma unroll
    for (int b = 0; b < 4 * NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // W rows kb + j (j = 0..7) for this lane's 4 columns of group h (column
    // offset h * N in the merged weight), whole step in range.
    auto load_w = [&](int64_t s, u32x2 (*w)[8]) {
#pragma unroll
        for (int h = 0; h < NB; ++h) {
            const uint16_t *src = wcol + h * N + (s * 32 + g * 8) * ldb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (FAST) {
                    w[h][j] = __builtin_nontemporal_load((const u32x2 *)(src + j * ldb));
                } else {
                    uint32_t e[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) e[c] = (ncol + c < N) ? (uint32_t)src[j * ldb + c] : 0u;
                    w[h][j] = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
                }
            }
        }
    };
    auto load_x = [&](int64_t s) -> u32x4 {
        const int64_t kb = s * 32 + g * 8;
        u32x4 v = FAST ? *(const u32x4 *)(xr + kb) : load_chunk8_bf16(xr, kb, K, true, 2);
        if (!m_ok) v = u32x4{0u, 0u, 0u, 0u};
        return v;
    };
    // 4x8 transpose of 16-bit halves: block b takes column b of the 8 rows.
    auto mma = [&](const u32x2 (*w)[8], u32x4 xv) {
        const bf16x8 xf = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                u32x4 a;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = w[h][2 * q][b >> 1], hi = w[h][2 * q + 1][b >> 1];
                    a[q] = (b & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                acc[4 * h + b] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), xf, acc[4 * h + b], 0, 0, 0);
            }
    };

    // Whole steps, software pipelined: the next step's loads are issued
    // before the current step's transpose and MFMAs.
    if (s_begin < s_full_end) {
        u32x2 w0[NB][8], w1[NB][8];
        u32x4 x0 = load_x(s_begin), x1;
        load_w(s_begin, w0);
        int64_t s = s_begin;
        for (; s + 2 <= s_full_end; s += 2) {
            x1 = load_x(s + 1 < s_full_end ? s + 1 : s);
            load_w(s + 1 < s_full_end ? s + 1 : s, w1);
            mma(w0, x0);
            if (s + 1 < s_full_end) {
                if (s + 2 < s_full_end) {
                    x0 = load_x(s + 2);
                    load_w(s + 2, w0);
                }
                mma(w1, x1);
            }
        }
        if (s < s_full_end) mma(w0, x0);
    }
    // A partial last step (K % 32), rows beyond K read as zero.
    for (int64_t s = s_full_end > s_begin ? s_full_end : s_begin; s < s_end; ++s) {
        const int64_t kb = s * 32 + g * 8;
        u32x2 w[NB][8];
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t k = kb + j;
                uint32_t e[4] = {0u, 0u, 0u, 0u};
                if (k < K) {
                    const uint16_t *src = wcol + h * N + k * ldb;
#pragma unroll
                    for (int c = 0; c < 4; ++c) e[c] = (ncol + c < N) ? (uint32_t)src[c] : 0u;
                }
                w[h][j] = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            }
        u32x4 xv = load_chunk8_bf16(xr, kb, K, true, 2);
        if (!m_ok) xv = u32x4{0u, 0u, 0u, 0u};
        mma(w, xv);
    }

    // acc[4 h + b][q] of lane (g, li) is the partial C[li][n0 + 16 g + 4 q + b]
    // of column group h.  Each lane's 16 NB partials go to LDS at a stride
    // of 16 NB + 1 floats, so the 64 lanes of one write instruction fall on
    // 64 different banks.
    constexpr int RS = 16 * NB + 1;
    __shared__ float red[NW * 64 * RS];
    float *mine = red + (wave * 64 + lane) * RS;
    if (li < M) {                            // rows < M only (the others are zero X rows)
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b) mine[h * 16 + q * 4 + b] = acc[4 * h + b][q];
    }
    __syncthreads();
    // Entry e of the 64 M kept ones: g = e / (16 M), row m = (e / 16) % M,
    // v = e % 16 -> lane L = 16 g + m, column n0 + 16 g + v.
    const int Mi = (int)M;
    for (int e = tid; e < 64 * Mi; e += NW * 64) {
        const int g2 = e / (16 * Mi), r = e - g2 * 16 * Mi, m = r >> 4, v = r & 15;
        const int L = 16 * g2 + m;
        float sum[NB];
#pragma unroll
        for (int h = 0; h < NB; ++h) {
            sum[h] = 0.f;
            for (int w2 = 0; w2 < NW; ++w2) sum[h] += red[(w2 * 64 + L) * RS + h * 16 + v];
        }
        const int64_t n = n0 + 16 * g2 + v;
        if (n < N) {
            if constexpr (GLU) store_swiglu(p, bidx, m, n, sum[0], sum[1]);
            else store_out(p, bidx, m, n, sum[0]);
        }
    }
}

// ============================================= small-M path, K split over workgroups
//
// Streaming W from HBM is capped per CU, and at the same workgroup count it
// runs faster with 256-byte row pieces than with 128-byte ones (measured:
// 192 workgroups, 128-byte strips 4.4 TB/s, 256-byte strips with K halved
// 5.1 TB/s).  This kernel gives a workgroup 128 columns (256 bytes of each W
// row) and one of KS contiguous slices of the K steps, so N = 12288 becomes
// 96 strips x 2 slices.  Within the workgroup the NW waves split the slice
// and add their partial sums through LDS in wave order, as in k_decode.
//  * Lane (g, r) loads 16 bytes (8 columns) of 8 rows per 32-row step, each
//    load instruction covering 4 rows x 256 contiguous bytes; an 8x8
//    transpose of 16-bit halves in registers feeds 8 matrix-core blocks
//    whose logical column r is physical column 8r + c.
//  * Counter path (more than two members, or outputs that do not fit the
//    exchange slots): slices are combined without atomics on data: every
//    workgroup writes its partial sums to the workspace with device-scope
//    stores, waits until
//    they have completed, and then one thread adds 1 to the strip's counter
//    (device-scope atomic).  The workgroup that brings the counter to KS
//    reads the KS partials with device-scope loads and adds them in slice
//    order -- the same order whichever workgroup arrives last, so the result
//    is deterministic and, the partition being independent of M, the same
//    for every row count -- then writes C and resets the counter for the
//    next call.  Why no fence is needed: the partials are written and read
//    only by device-scope (sc1) atomic stores and loads, which gfx950 never
//    leaves dirty in, nor serves stale from, an XCD's private L2 -- they
//    complete at the device's coherence point; s_waitcnt(0) plus the
//    barrier make every store of the workgroup complete before the counter
//    atomic (performed at that same point) is issued; and the last
//    arriver's loads are issued only after it has read the atomic's
//    result.  A release/acquire pair would add an L2 write-back and an L2
//    invalidate, needed only for data moved by ordinary loads and stores;
//    with them the path measured twice as slow.
//  * W is read once: its loads are non-temporal.
//  * SwiGLU (p.epi == EPI_SWIGLU): a strip's gate columns (n0.. of the
//    merged weight [K, 2N]) and its up columns (N + n0..) are read by
//    separate workgroups, KS of each, which all publish their partial sums;
//    the last of the 2 KS adds the gate slices and the up slices, each in
//    slice order, and stores bf16(bf16(SiLU(g)) * u).
// Requires N % 128 == 0, K % 32 == 0, 16-byte aligned rows of X and W.
// DB: double-buffer the W rows of two steps in registers.
//  * Two members per strip (pair != NULL: two K slices, or SwiGLU's gate
//    and up workgroups with one slice each): no counter.  Each output has a
//    32-bit slot in pair[] (zero on entry; [batch][M][N]); a workgroup
//    exchanges its partial, stored as its bit pattern with every bit
//    flipped, into the slot (a device-scope atomic exchange).  The one that
//    gets a nonzero value back holds both partials and finishes the output
//    as the counter path would -- (0 + p0) + p1 in slice order, or SwiGLU
//    of (0 + g) and (0 + u) -- then puts the slot back to zero.  One atomic round trip per output instead of the
//    store-wait-count-reload sequence; the value read is the atomic's own
//    result, so no ordering beyond the atomic is needed.
template <int NW, bool DB>
__global__ void __launch_bounds__(NW * 64, 1) k_decode_sk(GemmArgs p, float *ws, unsigned *cnt, int KS, unsigned *pair)
{
    constexpr int NC = 128;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t M = p.M, K = p.K, lda = p.lda, ldb = p.ldb;
    const int64_t nstrip = p.tiles_n;
    const bool glu = p.epi == EPI_SWIGLU;
    const int nmem = glu ? 2 * KS : KS;      // workgroups per strip
    const int64_t group = (int64_t)blockIdx.x / KS, slice = (int64_t)blockIdx.x % KS;
    const int64_t strip = glu ? group >> 1 : group, half = glu ? group & 1 : 0;
    const int64_t n0 = strip * NC;
    const int64_t bidx = blockIdx.y;
    const uint16_t *X = (const uint16_t *)p.A + bidx * p.sA;
    const uint16_t *W = (const uint16_t *)p.B + bidx * p.sB;

    // Fixed partition of the 32-row steps: over slices, then over waves.
    const int64_t steps = K / 32;
    const int64_t sl0 = steps * slice / KS, sl1 = steps * (slice + 1) / KS;
    const int64_t s_begin = sl0 + (sl1 - sl0) * wave / NW, s_end = sl0 + (sl1 - sl0) * (wave + 1) / NW;
    const bool m_ok = li < M;
    const uint16_t *xr = X + (int64_t)(m_ok ? li : 0) * lda;
    const uint16_t *wcol = W + half * p.N + n0 + 8 * li;

    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_w = [&](int64_t s, u32x4 *w) {
        const uint16_t *src = wcol + (s * 32 + g * 8) * ldb;
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = __builtin_nontemporal_load((const u32x4 *)(src + j * ldb));
    };
    auto load_x = [&](int64_t s) -> u32x4 {
        u32x4 v = *(const u32x4 *)(xr + s * 32 + g * 8);
        if (!m_ok) v = u32x4{0u, 0u, 0u, 0u};
        return v;
    };
    // 8x8 transpose of 16-bit halves: block c takes column c of the 8 rows.
    auto mma = [&](const u32x4 *w, u32x4 xv) {
        const bf16x8 xf = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 a;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = w[2 * q][c >> 1], hi = w[2 * q + 1][c >> 1];
                a[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), xf, acc[c], 0, 0, 0);
        }
    };
    if (!DB) {
        for (int64_t s = s_begin; s < s_end; ++s) {
            u32x4 w[8];
            const u32x4 xv = load_x(s);
            load_w(s, w);
            mma(w, xv);
        }
    } else if (s_begin < s_end) {
        u32x4 w0[8], w1[8];
        u32x4 x0 = load_x(s_begin), x1;
        load_w(s_begin, w0);
        int64_t s = s_begin;
        for (; s + 2 <= s_end; s += 2) {
            x1 = load_x(s + 1);
            load_w(s + 1, w1);
            mma(w0, x0);
            if (s + 2 < s_end) {
                x0 = load_x(s + 2);
                load_w(s + 2, w0);
            }
            mma(w1, x1);
        }
        if (s < s_end) mma(w0, x0);
    }

    // acc[c][q] of lane (g, li) is the partial C[li][n0 + 32 g + 8 q + c].
    // Each lane's 32 partials go to LDS at a stride of 33 floats, so the 64
    // lanes of one write instruction fall on 64 different banks.
    constexpr int RS = 33;
    __shared__ float red[NW * 64 * RS];
    __shared__ unsigned arrived;
    float *mine = red + (wave * 64 + lane) * RS;
    // Only the lanes of rows < M hold partial sums that are stored; the
    // others (zero X rows) skip the LDS round trip.
    if (li < M) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 8; ++c) mine[q * 8 + c] = acc[c][q];
    }
    __syncthreads();
    float *part = ws + ((bidx * nstrip + strip) * nmem + half * KS + slice) * (16 * NC);
    const bool direct = KS == 1 && !glu;     // one workgroup per strip: no partial sums
    // Entry e of the 128 M kept ones: g = e / (32 M), row m = (e / 32) % M,
    // j = e % 32 = 8 q + c -> lane L = 16 g + m, column 32 g + j of the strip.
    const int Mi = (int)M;
    for (int e = tid; e < 128 * Mi; e += NW * 64) {
        const int g2 = e / (32 * Mi), r = e - g2 * 32 * Mi, m = r >> 5, j = r & 31;
        const int L = 16 * g2 + m;
        float sum = 0.f;
        for (int w2 = 0; w2 < NW; ++w2) sum += red[(w2 * 64 + L) * RS + j];
        const int n = 32 * g2 + j;
        if (direct) {
            store_out(p, bidx, m, n0 + n, sum);
        } else if (pair) {
            unsigned *slot = pair + (bidx * M + m) * p.N + n0 + n;
            unsigned mine = ~__float_as_uint(sum);
            if (mine == 0u) mine = 1u;           // (a NaN pattern no bf16 product produces)
            const unsigned other = __hip_atomic_exchange(slot, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (other != 0u) {
                const float o = __uint_as_float(~other);
                const bool first = (glu ? half : slice) == 0;   // this member's partial comes first
                const float p0 = first ? sum : o, p1 = first ? o : sum;
                if (glu) store_swiglu(p, bidx, m, n0 + n, 0.f + p0, 0.f + p1);
                else store_out(p, bidx, m, n0 + n, (0.f + p0) + p1);
                __hip_atomic_store(slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            __hip_atomic_store(part + m * NC + n, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (direct || pair) return;
    // Publish this slice; the last of the nmem workgroups of the strip sums.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    unsigned *c_strip = cnt + bidx * nstrip + strip;
    if (tid == 0) arrived = __hip_atomic_fetch_add(c_strip, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (unsigned)(nmem - 1)) return;
    const float *parts = ws + (bidx * nstrip + strip) * nmem * (16 * NC);
    for (int t = tid; t < Mi * NC; t += NW * 64) {
        const int m = t / NC, n = t % NC;
        float sum = 0.f;
        for (int k2 = 0; k2 < KS; ++k2)
            sum += __hip_atomic_load(parts + k2 * (16 * NC) + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (glu) {
            float up = 0.f;
            for (int k2 = KS; k2 < 2 * KS; ++k2)
                up += __hip_atomic_load(parts + k2 * (16 * NC) + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            store_swiglu(p, bidx, m, n0 + n, sum, up);
        } else {
            store_out(p, bidx, m, n0 + n, sum);
        }
    }
    if (tid == 0) __hip_atomic_store(c_strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_decode_split(const GemmArgs &a, float *ws, unsigned *cnt, int ks, unsigned *pair, hipStream_t s)
{
    if (pair && (a.epi == EPI_SWIGLU ? ks != 1 : ks != 2)) return hipErrorInvalidValue;
    // 16 waves, one 32-row step in registers at a time (two would spill at
    // 16 waves per CU; the waves themselves keep enough loads in flight).
    const int64_t groups = a.epi == EPI_SWIGLU ? 2 * a.tiles_n : a.tiles_n;
    hipLaunchKernelGGL((k_decode_sk<16, false>), dim3((unsigned)(groups * ks), (unsigned)a.batch), dim3(16 * 64), 0,
                       s, a, ws, cnt, ks, pair);
    return hipGetLastError();
}

// ============================================= small-M path, B given transposed
//
// C[M, N] = X[M, K] . Bt[N, K]^T for M <= 16: every output is a dot product
// along a contiguous row of Bt, the GEMV case of MUSA lesson m11-l5 (rows of
// the matrix reduced against one vector, here up to 16 vectors at once).
// A workgroup owns 16 rows of Bt (16 output columns); its NW waves split K
// into contiguous ranges, so each wave streams 16 row pieces of about
// K / NW elements, 64 bytes of each row per 32-deep step and the next 64
// bytes in the next step: every 128-byte line is read whole, by one wave,
// back to back.  The rows go straight from HBM into the matrix core as the
// 16-row operand (lane (g, r): row r, 8 consecutive K values; no transpose
// is needed), X rows as the other operand (rows past M are zero).  The
// waves' 16x16 partial sums are added in LDS in wave order: the K partition
// is independent of M, so a row's result does not depend on how many rows
// the call has.  A K remainder (K % 32) is a final step loaded element by
// element with zero fill.  RB blocks of 16 rows per workgroup share each X
// fragment (X is re-read once per block otherwise: as many bytes as Bt when
// M = 16).  Requires 16-byte aligned rows of Bt.
template <int NW, int RB>
__global__ void __launch_bounds__(NW * 64) k_decode_nt(GemmArgs p)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
    const int64_t bidx = blockIdx.y;
    const uint16_t *X = (const uint16_t *)p.A + bidx * p.sA;
    const uint16_t *Bt = (const uint16_t *)p.B + bidx * p.sB;
    const bool m_ok = li < M;
    bool n_ok[RB];
    const uint16_t *brow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        n_ok[r] = n0 + 16 * r + li < N;
        brow[r] = Bt + (n_ok[r] ? n0 + 16 * r + li : 0) * ldb;
    }
    const uint16_t *xrow = X + (m_ok ? li : 0) * lda;

    const int64_t whole = K / 32;                          // whole 32-deep steps
    const int64_t s_begin = whole * wave / NW, s_end = whole * (wave + 1) / NW;
    f32x4 acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_b = [&](int r, int64_t s) -> u32x4 {
        return n_ok[r] ? __builtin_nontemporal_load((const u32x4 *)(brow[r] + s * 32 + g * 8)) : u32x4{0u, 0u, 0u, 0u};
    };
    auto load_x = [&](int64_t s) -> u32x4 {
        return load_chunk8_bf16(xrow, s * 32 + g * 8, K, m_ok, p.align_a);
    };
    auto mma = [&](int r, u32x4 b, u32x4 x) {
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, x),
                                                         acc[r], 0, 0, 0);
    };
    // D steps of Bt in flight ahead of the matrix core.
    constexpr int D = RB == 1 ? 4 : 2;
    int64_t s = s_begin;
    for (; s + D <= s_end; s += D) {
        u32x4 b[D][RB], x[D];
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int r = 0; r < RB; ++r) b[j][r] = load_b(r, s + j);
#pragma unroll
        for (int j = 0; j < D; ++j) x[j] = load_x(s + j);
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int r = 0; r < RB; ++r) mma(r, b[j][r], x[j]);
    }
    for (; s < s_end; ++s) {
        const u32x4 x = load_x(s);
#pragma unroll
        for (int r = 0; r < RB; ++r) mma(r, load_b(r, s), x);
    }
    if (wave == NW - 1 && K % 32 != 0) {
        // the K remainder, zero-filled past K
        const u32x4 x = load_x(whole);
#pragma unroll
        for (int r = 0; r < RB; ++r) mma(r, load_chunk8_bf16(brow[r], whole * 32 + g * 8, K, n_ok[r], p.align_b), x);
    }

    // acc[r][q] of lane (g, li) is the partial sum for column
    // n0 + 16 r + 4 g + q, row li.
    __shared__ f32x4 red[NW][RB][64];
#pragma unroll
    for (int r = 0; r < RB; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (tid < 64 * RB) {
        const int r = tid >> 6, t = tid & 63;
        f32x4 sum = red[0][r][t];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) sum += red[w2][r][t];
        const int m = t & 15, gg = t >> 4;
        if (m < M) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + 16 * r + 4 * gg + q;
                if (n >= N) continue;
                store_out(p, bidx, m, n, sum[q]);
            }
        }
    }
}

// ===================================================== row realignment
//
// A bf16 operand whose rows are not 16-byte aligned can only be copied into
// LDS 4 bytes per lane, four times the copy instructions of the 16-byte
// copies (measured on 1000x12280x4100: 142 against 125 us for the same
// product with aligned rows).  For a large product the library first copies
// the rows into a buffer with a row length of lda2 elements (K rounded up to
// a multiple of 8; columns K..lda2-1 hold zeros) and multiplies from there.
// One thread per 16-byte chunk of the destination, grid-stride.
__global__ void __launch_bounds__(256) k_realign_rows(const uint16_t *A, int64_t lda, int64_t sA, int64_t batch,
                                                      int64_t M, int64_t K, int align, uint16_t *A2, int64_t lda2)
{
    const int64_t cpr = lda2 / 8;                      // chunks per row
    const int64_t total = batch * M * cpr;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
        const int64_t r = q / cpr, c = q % cpr;
        const int64_t b = r / M, m = r % M;
        const u32x4 v = load_chunk8_bf16(A + b * sA + m * lda, 8 * c, K, true, align);
        *(u32x4 *)(A2 + r * lda2 + 8 * c) = v;
    }
}

hipError_t launch_realign_rows(const uint16_t *A, int64_t lda, int64_t sA, int64_t batch, int64_t M, int64_t K,
                               int align, uint16_t *A2, int64_t lda2, hipStream_t s)
{
    const int64_t total = batch * M * (lda2 / 8);
    int64_t grid = (total + 255) / 256;
    if (grid > 4096) grid = 4096;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_realign_rows, dim3((unsigned)grid), dim3(256), 0, s, A, lda, sA, batch, M, K, align, A2, lda2);
    return hipGetLastError();
}

// ============================================================ generic path
//
// Any shape, stride and alignment: 16x16 output tile per workgroup, element
// loads staged through LDS, FP32 FMA on the vector ALU in k order.
template <typename TIn>
__device__ __forceinline__ float widen(TIn v);
template <>
__device__ __forceinline__ float widen<float>(float v) { return v; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

template <typename TIn>
__global__ void __launch_bounds__(256) k_generic(GemmArgs p)
{
    __shared__ float As[16][17], Bs[16][17];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const TileCoord tc = tile_map(blockIdx.x, p.batch, p.tiles_m, p.tiles_n, 1);
    const int64_t m = tc.tm * 16 + ty, n = tc.tn * 16 + tx;
    const TIn *A = (const TIn *)p.A + tc.b * p.sA;
    const TIn *B = (const TIn *)p.B + tc.b * p.sB;
    float acc = 0.f;
    for (int64_t k0 = 0; k0 < p.K; k0 += 16) {
        const int64_t ka = k0 + tx, kb = k0 + ty;
        As[ty][tx] = (m < p.M && ka < p.K) ? widen<TIn>(A[m * p.lda + ka]) : 0.f;
        Bs[ty][tx] = (kb < p.K && n < p.N) ? widen<TIn>(B[kb * p.ldb + n]) : 0.f;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) acc = __builtin_fmaf(As[ty][kk], Bs[kk][tx], acc);
        __syncthreads();
    }
    if (m < p.M && n < p.N) {
        if (p.out_f32) ((float *)p.C + tc.b * p.sC)[m * p.ldc + n] = acc;
        else ((uint16_t *)p.C + tc.b * p.sC)[m * p.ldc + n] = (uint16_t)bf16_rne(acc);
    }
}

// K == 0: C := 0 over batch x M x N (grid-stride).
// Rows whose starts are 16-byte aligned are written in 16-byte chunks,
// non-temporal (C is written once), with the columns past the last whole
// chunk element by element; other rows element by element.
__global__ void __launch_bounds__(256) k_zero(GemmArgs p)
{
    // (E4M3FN codes of SwiGLU: the output of zero sums is SiLU(0) * 0 = +0, code 0)
    const int esz = p.c_e4m3 ? 1 : p.out_f32 ? 4 : 2;
    const int64_t rows = p.batch * p.M;
    const int64_t stride = (int64_t)gridDim.x * 256, first = (int64_t)blockIdx.x * 256 + threadIdx.x;
    auto elem = [&](int64_t r, int64_t n) {
        const int64_t b = r / p.M, m = r % p.M;
        if (p.c_e4m3) ((uint8_t *)p.C + b * p.sC)[m * p.ldc + n] = 0;
        else if (p.out_f32) ((float *)p.C + b * p.sC)[m * p.ldc + n] = 0.f;
        else ((uint16_t *)p.C + b * p.sC)[m * p.ldc + n] = 0;
    };
    int64_t done_cols = 0;                              // columns written as chunks
    if (p.align_c >= 16) {
        const int64_t per = 16 / esz, cpr = p.N / per;
        done_cols = cpr * per;
        for (int64_t q = first; q < rows * cpr; q += stride) {
            const int64_t r = q / cpr, c = q % cpr;
            const int64_t b = r / p.M, m = r % p.M;
            char *dst = (char *)p.C + ((b * p.sC + m * p.ldc) * esz) + c * 16;
            __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, (u32x4 *)dst);
        }
    }
    const int64_t rest = p.N - done_cols;
    for (int64_t q = first; q < rows * rest; q += stride) elem(q / rest, done_cols + q % rest);
}

// ================================================================ launchers

// variant: 0 general (k_bf16_mfma), 1 ring kernel aligned, 2 ring kernel
// masked with 16-byte A rows, 3 ring kernel masked with 4-byte A copies.
// NSA, NSB: slots of the A and B rings of the ring kernels (NSA-2 and NSB-2
// slabs of copies in flight while one is consumed).
template <int BM, int BN, int WGM, int WGN, int DWGM, int DWGN, int NSA, int NSB>
static hipError_t launch_bf16(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(DWGM * DWGN * 64);
    if constexpr (BM == 128 && BN == 128) {
        // K split over workgroups (128x128 tiles only: the smallest partial tiles)
        if (a.ksplit > 1) return launch_ring<BM, BN, DWGM, DWGN, NSA, NSB, EPI_NONE, true, false>(a, variant, g, b8, s);
    }
    switch (variant) {
    case 1: hipLaunchKernelGGL((k_bf16_ms<BM, BN, DWGM, DWGN, NSA, NSB, 16, false>), g, b8, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_bf16_ms<BM, BN, DWGM, DWGN, NSA, NSB, 16, true>), g, b8, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_bf16_ms<BM, BN, DWGM, DWGN, NSA, NSB, 4, true>), g, b8, 0, s, a); break;
    default: hipLaunchKernelGGL((k_bf16_mfma<BM, BN, WGM, WGN, false>), g, dim3(WGM * WGN * 64), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_f32(const GemmArgs &a, bool even, int64_t grid, hipStream_t s)
{
    if (even) hipLaunchKernelGGL((k_f32_mfma<BM, BN, WGM, WGN, true>), dim3((unsigned)grid), dim3(WGM * WGN * 64), 0, s, a);
    else hipLaunchKernelGGL((k_f32_mfma<BM, BN, WGM, WGN, false>), dim3((unsigned)grid), dim3(WGM * WGN * 64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_config(int config_id, bool f32_inputs, const GemmArgs &a, int variant, int64_t grid,
                         hipStream_t s)
{
    switch (config_id) {
    case CFG_ZERO:
        hipLaunchKernelGGL(k_zero, dim3((unsigned)grid), dim3(256), 0, s, a);
        return hipGetLastError();
    case CFG_BF16_256x192:
    case CFG_BF16_128x128:
    case CFG_BF16_256x128:
    case CFG_BF16_256x256:
        if (a.fp8) return launch_ring_fp8(config_id, a, variant, grid, s);
        if (a.b_trans) return launch_ring_bt(config_id, a, variant, grid, s);
        if (a.a_trans) return launch_ring_at(config_id, a, variant, grid, s);
        break;
    default: break;
    }
    switch (config_id) {
    case CFG_BF16_256x192: return launch_bf16<256, 192, 2, 2, 2, 4, 4, 4>(a, variant, grid, s);
    case CFG_BF16_128x128: return launch_bf16<128, 128, 2, 2, 4, 2, 4, 4>(a, variant, grid, s);
    case CFG_BF16_256x128: return launch_bf16<256, 128, 2, 2, 4, 2, 4, 4>(a, variant, grid, s);
    case CFG_BF16_256x256: return launch_bf16<256, 256, 2, 2, 2, 4, 4, 4>(a, variant, grid, s);
    case CFG_F32_128x128: return launch_f32<128, 128, 2, 2>(a, variant == 1, grid, s);
    case CFG_F32_64x64: return launch_f32<64, 64, 2, 2>(a, variant == 1, grid, s);
    case CFG_F32_32x32_WK:
        // variant 1 only: whole tiles, K % 32 == 0, K <= 256, 16-byte aligned rows
        if (variant != 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_f32_wholek<32, 32, 2, 2, 256>), dim3((unsigned)grid), dim3(256), 0, s, a);
        return hipGetLastError();
    case CFG_DECODE_64:
        // variant 1: every column chunk in range, 8-byte aligned W rows and
        // 16-byte aligned X rows
        if (a.epi == EPI_SWIGLU) {
            // (8 waves: the gate and up rows of two steps in flight take
            // more registers than 4 waves per SIMD leave)
            if (variant == 1)
                hipLaunchKernelGGL((k_decode<8, true, true>), dim3((unsigned)grid, (unsigned)a.batch), dim3(8 * 64), 0, s,
                                   a);
            else
                hipLaunchKernelGGL((k_decode<8, false, true>), dim3((unsigned)grid, (unsigned)a.batch), dim3(8 * 64), 0, s,
                                   a);
        } else if (variant == 1) {
            hipLaunchKernelGGL((k_decode<16, true, false>), dim3((unsigned)grid, (unsigned)a.batch), dim3(16 * 64), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_decode<16, false, false>), dim3((unsigned)grid, (unsigned)a.batch), dim3(16 * 64), 0, s,
                               a);
        }
        return hipGetLastError();
    case CFG_DECODE_NT:
        if (a.fp8) return launch_decode_nt_f8(a, variant, grid, s);
        // variant 1: one 16-row block per workgroup (M = 1); 2: three, which
        // share each X fragment (for M = 16 the fragments would otherwise
        // cost as much traffic as Bt: 29.2 against 23.9 us at N = 12288)
        if (variant == 2)
            hipLaunchKernelGGL((k_decode_nt<8, 3>), dim3((unsigned)grid, (unsigned)a.batch), dim3(8 * 64), 0, s, a);
        else
            hipLaunchKernelGGL((k_decode_nt<8, 1>), dim3((unsigned)grid, (unsigned)a.batch), dim3(8 * 64), 0, s, a);
        return hipGetLastError();
    case CFG_GENERIC:
        if (f32_inputs) hipLaunchKernelGGL(k_generic<float>, dim3((unsigned)grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_generic<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
        return hipGetLastError();
    default: return hipErrorInvalidValue;
    }
}

}  // namespace g5
