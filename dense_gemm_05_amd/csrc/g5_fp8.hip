// g5_fp8.hip -- FP8 (E4M3FN) path: per-row quantization of bf16 rows and the
// launchers of the LDS-ring kernel on E4M3FN operands (page "Operator &
// Runtime" §5.4.3, Examples 5-7 and 5-8: quantize each row with a factor from
// the whole row's maximum, before the GEMM, then multiply the codes and
// dequantize the FP32 sums by the row and column factors).
#include <hip/hip_runtime.h>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

// One workgroup per row.  Pass 1 finds the row's largest magnitude (each
// thread over its 16-byte chunks, then across the wave by butterfly
// exchanges, then across the 4 waves in LDS: the tree reduction of the
// reduce page, "3.1 Tối ưu toán tử CUDA Reduce").  Pass 2 writes the codes:
// y = (x * 448) / amax in binary32 (one correctly rounded division), then
// the hardware conversion, which rounds to the nearest E4M3FN value, ties
// to even -- the code nearest to the exact quotient of Example 5-7 (see
// quot below).  The row's dequantization factor is amax / 448; a row of
// zeros gets zero codes and factor 0.  Rows of up to
// NCH * 2048 elements stay in registers between the passes; longer rows
// are read again in pass 2.
template <int NCH>
__global__ void __launch_bounds__(256) k_quant_rows_e4m3(const uint16_t *X, int64_t ldx, int64_t cols, int align_x,
                                                         uint8_t *Q, int64_t ldq, int align_q, float *scale)
{
    const int64_t r = blockIdx.x;
    const uint16_t *x = X + r * ldx;
    uint8_t *q = Q + r * ldq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool held = cols <= (int64_t)NCH * 2048;
    u32x4 v[NCH];
    float m = 0.0f;
    auto absmax8 = [](float m, const u32x4 &c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(c[i])), fabsf(bf16_hi(c[i]))));
        return m;
    };
    if (held) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int64_t c = (int64_t)tid * 8 + (int64_t)j * 2048;
            v[j] = c < cols ? load_chunk8_bf16(x, c, cols, true, align_x) : u32x4{0u, 0u, 0u, 0u};
            m = absmax8(m, v[j]);
        }
    } else {
        for (int64_t c = (int64_t)tid * 8; c < cols; c += 2048) m = absmax8(m, load_chunk8_bf16(x, c, cols, true, align_x));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float red[4];
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (tid == 0) scale[r] = amax / 448.0f;
    // y = x * 448 / amax with one rounding: x * 448 is exact in binary32 (a
    // bf16 significand times 7 * 64), and the division is correctly rounded.
    // A quotient that is exactly the midpoint of two E4M3FN values (at most
    // 5 significant bits) is then exact, and any other lies at least
    // ~2^-13 of its size away from every midpoint, far beyond the 2^-24 of
    // the rounding, so the conversion below (round to nearest even) picks
    // the code nearest to the exact quotient.  |x| <= amax keeps |y| <= 448
    // (the clamp only guards the conversion, which turns larger values into
    // NaN).  A row of zeros gives signed zeros.
    auto clamp448 = [](float y) { return y > 448.0f ? 448.0f : (y < -448.0f ? -448.0f : y); };
    auto quot = [&](float x) { return amax > 0.0f ? clamp448(__fdiv_rn(x * 448.0f, amax)) : x * 0.0f; };
    auto emit = [&](int64_t c, const u32x4 &cv) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float y0 = quot(bf16_lo(cv[2 * h])), y1 = quot(bf16_hi(cv[2 * h]));
            const float y2 = quot(bf16_lo(cv[2 * h + 1])), y3 = quot(bf16_hi(cv[2 * h + 1]));
            int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, packed, true);
            w[h] = (uint32_t)packed;
        }
        if (c + 8 <= cols && align_q >= 8) {
            u32x2 st = {w[0], w[1]};
            *(u32x2 *)(q + c) = st;
        } else {
            for (int i = 0; i < 8 && c + i < cols; ++i) q[c + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        }
    };
    if (held) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int64_t c = (int64_t)tid * 8 + (int64_t)j * 2048;
            if (c < cols) emit(c, v[j]);
        }
    } else {
        for (int64_t c = (int64_t)tid * 8; c < cols; c += 2048) emit(c, load_chunk8_bf16(x, c, cols, true, align_x));
    }
}

hipError_t launch_quant_rows_e4m3(const uint16_t *X, int64_t ldx, int64_t rows, int64_t cols, int align_x,
                                  uint8_t *Q, int64_t ldq, int align_q, float *scale, hipStream_t s)
{
    hipLaunchKernelGGL(k_quant_rows_e4m3<4>, dim3((unsigned)rows), dim3(256), 0, s, X, ldx, cols, align_x, Q, ldq,
                       align_q, scale);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_f8(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(WGM * WGN * 64);
    if constexpr (BM == 128 && BN == 128) {
        if (a.ksplit > 1) return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI_NONE, true, true, true>(a, variant, g, b8, s);
    }
    return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI_NONE, false, true, true>(a, variant, g, b8, s);
}

hipError_t launch_ring_fp8(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    switch (config_id) {
    case CFG_BF16_256x192: return launch_f8<256, 192, 2, 4>(a, variant, grid, s);
    case CFG_BF16_256x256: return launch_f8<256, 256, 2, 4>(a, variant, grid, s);
    case CFG_BF16_128x128: return launch_f8<128, 128, 4, 2>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

// Small M on E4M3FN operands: C[M, N] = (X[M, K] . Bt[N, K]^T) scaled by
// the factor of each row of X and of each row of Bt, for M <= 16.  As the
// bf16 transposed-B GEMV: a workgroup owns 16 x RB rows of Bt, its NW waves
// split K into contiguous ranges of 64-deep steps, and each lane loads 16
// bytes (16 K values) of a row per step, which feed two
// v_mfma_f32_16x16x32_fp8_fp8 (bytes 0-7, then 8-15: the same permutation
// of K for both operands).  A K remainder (K % 64) is a final step loaded
// element by element with zero fill.  The waves' partial sums are added in
// LDS in wave order (so a row's result does not depend on M), then scaled
// and rounded once.  Requires 16-byte aligned rows of Bt.
template <int NW, int RB>
__global__ void __launch_bounds__(NW * 64) k_decode_nt_f8(GemmArgs p)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
    const uint8_t *X = (const uint8_t *)p.A;
    const uint8_t *Bt = (const uint8_t *)p.B;
    const bool m_ok = li < M;
    bool n_ok[RB];
    const uint8_t *brow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        n_ok[r] = n0 + 16 * r + li < N;
        brow[r] = Bt + (n_ok[r] ? n0 + 16 * r + li : 0) * ldb;
    }
    const uint8_t *xrow = X + (m_ok ? li : 0) * lda;

    const int64_t whole = K / 64;                          // whole 64-deep steps
    const int64_t s_begin = whole * wave / NW, s_end = whole * (wave + 1) / NW;
    f32x4 acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_b = [&](int r, int64_t st) -> u32x4 {
        return n_ok[r] ? __builtin_nontemporal_load((const u32x4 *)(brow[r] + st * 64 + g * 16))
                       : u32x4{0u, 0u, 0u, 0u};
    };
    auto load_x = [&](int64_t st) -> u32x4 { return load_chunk16_u8(xrow, st * 64 + g * 16, K, m_ok, p.align_a); };
    auto mma = [&](int r, u32x4 b, u32x4 x) {
        const i64x2 b2 = __builtin_bit_cast(i64x2, b), x2 = __builtin_bit_cast(i64x2, x);
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(b2[0], x2[0], acc[r], 0, 0, 0);
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(b2[1], x2[1], acc[r], 0, 0, 0);
    };
    // D steps of Bt in flight ahead of the matrix core.
    constexpr int D = RB == 1 ? 4 : 2;
    int64_t st = s_begin;
    for (; st + D <= s_end; st += D) {
        u32x4 b[D][RB], x[D];
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int r = 0; r < RB; ++r) b[j][r] = load_b(r, st + j);
#pragma unroll
        for (int j = 0; j < D; ++j) x[j] = load_x(st + j);
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int r = 0; r < RB; ++r) mma(r, b[j][r], x[j]);
    }
    for (; st < s_end; ++st) {
        const u32x4 x = load_x(st);
#pragma unroll
        for (int r = 0; r < RB; ++r) mma(r, load_b(r, st), x);
    }
    if (wave == NW - 1 && K % 64 != 0) {
        const u32x4 x = load_x(whole);
#pragma unroll
        for (int r = 0; r < RB; ++r) mma(r, load_chunk16_u8(brow[r], whole * 64 + g * 16, K, n_ok[r], p.align_b), x);
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
            const float sa = p.scale_a ? p.scale_a[m] : 1.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + 16 * r + 4 * gg + q;
                if (n >= N) continue;
                const float sb = p.scale_b ? p.scale_b[n] : 1.0f;
                const float v = sum[q] * sa * sb;
                if (p.out_f32) ((float *)p.C)[m * p.ldc + n] = v;
                else ((uint16_t *)p.C)[m * p.ldc + n] = (uint16_t)bf16_rne(v);
            }
        }
    }
}

hipError_t launch_decode_nt_f8(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    if (variant == 2)
        hipLaunchKernelGGL((k_decode_nt_f8<8, 3>), dim3((unsigned)grid), dim3(8 * 64), 0, s, a);
    else
        hipLaunchKernelGGL((k_decode_nt_f8<8, 1>), dim3((unsigned)grid), dim3(8 * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace g5
