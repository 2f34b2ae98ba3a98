// g5_fp8.hip -- FP8 (E4M3FN) path: per-row quantization of bf16 rows and the
// launchers of the LDS-ring kernel on E4M3FN operands (page "Operator &
// Runtime" §5.4.3, Examples 5-7 and 5-8: quantize each row with a factor from
// the whole row's maximum, before the GEMM, then multiply the codes and
// dequantize the FP32 sums by the row and column factors).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

// Per-row quantization.  Pass 1 finds the row's largest magnitude: each
// lane over its 16-byte chunks (all of a held row's loads issued before the
// first is used), then across the wave by butterfly exchanges (the tree
// reduction of the reduce page, "3.1 Tối ưu toán tử CUDA Reduce", at wave
// scope: no LDS, no barrier; wave_row_amax does this for one wave per row,
// k_quant_rows_e4m3 also for several waves per row).  Pass 2 writes the
// codes: the quotient x * 448 / amax in binary32 (E4m3Quot), then the
// hardware conversion, which rounds to the nearest E4M3FN value, ties to
// even -- the code nearest to the exact quotient of Example 5-7.  The row's
// dequantization factor is amax / 448; a row of zeros gets zero codes and
// factor 0.  Rows of up to NCH * 512 elements stay in registers between the
// passes; longer rows are read again in pass 2.
template <int NCH>
__device__ __forceinline__ float wave_row_amax(const uint16_t *x, int64_t cols, int align_x, int lane, u32x4 (&v)[NCH],
                                               bool held)
{
    auto absmax8 = [](float m, const u32x4 &c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(c[i])), fabsf(bf16_hi(c[i]))));
        return m;
    };
    float m = 0.0f;
    if (held) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int64_t c = (int64_t)lane * 8 + (int64_t)j * 512;
            v[j] = c < cols ? load_chunk8_bf16(x, c, cols, true, align_x) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) m = absmax8(m, v[j]);
    } else {
        for (int64_t c = (int64_t)lane * 8; c < cols; c += 512) m = absmax8(m, load_chunk8_bf16(x, c, cols, true, align_x));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    return m;
}

// WPR waves per row (4 / WPR rows per workgroup of 4 waves): wave `part`
// of a row holds its chunks (512 columns each) part, part + WPR, ...; the
// row's maximum is the largest of its waves' (through LDS when WPR > 1: a
// maximum does not depend on the order, so the codes are those of one wave
// per row).  Several waves per row give a short matrix enough loads in
// flight: X [1024, 4096] is 1024 rows, 4 per CU at one wave each.
template <int NCH, int WPR>
__global__ void __launch_bounds__(256) k_quant_rows_e4m3(const uint16_t *X, int64_t ldx, int64_t rows, int64_t cols,
                                                         int align_x, uint8_t *Q, int64_t ldq, int align_q,
                                                         float *scale)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, part = wv % WPR;
    const int64_t r = (int64_t)blockIdx.x * (4 / WPR) + wv / WPR;
    const bool r_ok = r < rows;
    if (WPR == 1 && !r_ok) return;          // a whole wave; nothing below synchronises waves
    const uint16_t *x = X + (r_ok ? r : 0) * ldx;
    uint8_t *q = Q + (r_ok ? r : 0) * ldq;
    const bool held = cols <= (int64_t)NCH * 512 * WPR;
    u32x4 v[NCH];
    auto absmax8 = [](float m, const u32x4 &c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(c[i])), fabsf(bf16_hi(c[i]))));
        return m;
    };
    float amax = 0.0f;
    if (r_ok) {
        if (held) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int64_t c = (int64_t)lane * 8 + (int64_t)(j * WPR + part) * 512;
                v[j] = c < cols ? load_chunk8_bf16(x, c, cols, true, align_x) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) amax = absmax8(amax, v[j]);
        } else {
            for (int64_t c = (int64_t)lane * 8 + (int64_t)part * 512; c < cols; c += 512 * WPR)
                amax = absmax8(amax, load_chunk8_bf16(x, c, cols, true, align_x));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    }
    if constexpr (WPR > 1) {
        __shared__ float wmax[4];
        if (lane == 0) wmax[wv] = amax;
        __syncthreads();
        const int w0 = wv - part;
#pragma unroll
        for (int k = 0; k < WPR; ++k) amax = fmaxf(amax, wmax[w0 + k]);
    }
    if (!r_ok) return;
    if (lane == 0 && part == 0) scale[r] = amax / 448.0f;
    // amax is the same for the whole row, so is the choice of quotient
    const E4m3Quot qz(amax);
    auto emit = [&](auto fast, int64_t c, const u32x4 &cv) {
        constexpr bool F = decltype(fast)::value;
        const uint32_t w0 = qz.code4<F>(cv[0], cv[1]), w1 = qz.code4<F>(cv[2], cv[3]);
        if (c + 8 <= cols && align_q >= 8) {
            u32x2 st = {w0, w1};
            *(u32x2 *)(q + c) = st;
        } else {
            const uint32_t w[2] = {w0, w1};
            for (int i = 0; i < 8 && c + i < cols; ++i) q[c + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        }
    };
    auto pass2 = [&](auto fast) {
        if (held) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int64_t c = (int64_t)lane * 8 + (int64_t)(j * WPR + part) * 512;
                if (c < cols) emit(fast, c, v[j]);
            }
        } else {
            for (int64_t c = (int64_t)lane * 8 + (int64_t)part * 512; c < cols; c += 512 * WPR)
                emit(fast, c, load_chunk8_bf16(x, c, cols, true, align_x));
        }
    };
    if (qz.fast) pass2(std::true_type{});
    else pass2(std::false_type{});
}

hipError_t launch_quant_rows_e4m3(const uint16_t *X, int64_t ldx, int64_t rows, int64_t cols, int align_x,
                                  uint8_t *Q, int64_t ldq, int align_q, float *scale, hipStream_t s)
{
    // four waves per row while that leaves rows for at most 16 waves per CU
    if (rows <= 1024)
        hipLaunchKernelGGL((k_quant_rows_e4m3<2, 4>), dim3((unsigned)rows), dim3(256), 0, s, X, ldx, rows, cols,
                           align_x, Q, ldq, align_q, scale);
    else
        hipLaunchKernelGGL((k_quant_rows_e4m3<8, 1>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, X, ldx,
                           rows, cols, align_x, Q, ldq, align_q, scale);
    return hipGetLastError();
}

// Per-column quantization of a weight W [K, N] (bf16) into the rows of
// Qt [N, K]: column j gets the factor of its own largest magnitude and the
// codes of the row quantizer above (same quotient, same rounding), written
// transposed so that the FP8 products read them as Bt.  Three passes over a
// grid of workgroups (x, y), each owning 64 columns and the y-th of
// gridDim.y ranges of 64-row blocks (8 lanes cover 128 bytes of a row, 8
// columns each; 32 rows per step); the column maxima live in scale[] as
// float bit patterns until the last pass turns them into factors.
//  1. k_cols_amax: each workgroup's maxima over its rows (per lane, then
//     over the 32 lanes of a column chunk in LDS), merged into scale[] by an
//     atomic maximum on the bits (non-negative floats order like their bit
//     patterns; scale[] was zeroed first; fmaxf drops NaN, so none enters).
//  2. k_quant_cols_e4m3: per 64-row block of its range, every lane
//     quantizes 8 columns of 2 rows into an LDS tile laid out [column][k],
//     and the tile goes out as 64 rows of 64 code bytes.
//  3. k_cols_factor: scale[n] = amax / 448.
__global__ void __launch_bounds__(256) k_fill_u32(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__device__ __forceinline__ void cols_block_range(int64_t K, int64_t &b0, int64_t &b1)
{
    const int64_t blocks = (K + 63) / 64;
    b0 = blocks * blockIdx.y / gridDim.y;
    b1 = blocks * (blockIdx.y + 1) / gridDim.y;
}

__global__ void __launch_bounds__(256) k_cols_amax(const uint16_t *W, int64_t ldw, int64_t K, int64_t N, int align_w,
                                                   uint32_t *amax_bits)
{
    __shared__ float red[32][65];
    const int tid = threadIdx.x, cc = tid & 7, r0 = tid >> 3;
    const int64_t n0 = (int64_t)blockIdx.x * 64;
    const int64_t col = n0 + 8 * cc;
    int64_t b0, b1;
    cols_block_range(K, b0, b1);
    const int64_t kend = b1 * 64 < K ? b1 * 64 : K;
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t k = b0 * 64 + r0; k < kend; k += 32) {
        const u32x4 v = load_chunk8_bf16(W + k * ldw, col, N, true, align_w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[2 * i] = fmaxf(m[2 * i], fabsf(bf16_lo(v[i])));
            m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(bf16_hi(v[i])));
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[r0][8 * cc + i] = m[i];
    __syncthreads();
    if (tid < 64 && n0 + tid < N) {
        float a = 0.f;
        for (int r = 0; r < 32; ++r) a = fmaxf(a, red[r][tid]);
        if (a > 0.f)
            __hip_atomic_fetch_max(amax_bits + n0 + tid, __float_as_uint(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void __launch_bounds__(256) k_quant_cols_e4m3(const uint16_t *W, int64_t ldw, int64_t K, int64_t N,
                                                         int align_w, uint8_t *Qt, int64_t ldq, int align_q,
                                                         const float *amax_n)
{
    constexpr int TP = 68;                   // tile pitch (bytes): 64 codes + 4, rows on different banks
    __shared__ __attribute__((aligned(16))) uint8_t tile[64 * TP];
    const int tid = threadIdx.x, cc = tid & 7, r0 = tid >> 3;
    const int64_t n0 = (int64_t)blockIdx.x * 64;
    const int64_t col = n0 + 8 * cc;
    float amax[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) amax[i] = col + i < N ? amax_n[col + i] : 0.f;
    // codes by E4m3Quot, one per column (the quotient's form is chosen per
    // column)
    const E4m3Quot qz[8] = {E4m3Quot(amax[0]), E4m3Quot(amax[1]), E4m3Quot(amax[2]), E4m3Quot(amax[3]),
                            E4m3Quot(amax[4]), E4m3Quot(amax[5]), E4m3Quot(amax[6]), E4m3Quot(amax[7])};
    int64_t b0, b1;
    cols_block_range(K, b0, b1);
    for (int64_t kb = b0 * 64; kb < b1 * 64; kb += 64) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kr = r0 + 32 * h;
            const int64_t k = kb + kr;
            const u32x4 v = k < K ? load_chunk8_bf16(W + k * ldw, col, N, true, align_w) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tile[(8 * cc + 2 * i) * TP + kr] = (uint8_t)qz[2 * i].code1(bf16_lo(v[i]));
                tile[(8 * cc + 2 * i + 1) * TP + kr] = (uint8_t)qz[2 * i + 1].code1(bf16_hi(v[i]));
            }
        }
        __syncthreads();
        // lane t: 16 codes (k = kb + 16 (t % 4) ..) of column n0 + t / 4
        const int c = tid >> 2, part = (tid & 3) * 16;
        const int64_t n = n0 + c, k = kb + part;
        if (n < N && k < K) {
            uint8_t *dst = Qt + n * ldq + k;
            const uint8_t *src = tile + c * TP + part;
            if (k + 16 <= K && align_q >= 16) {
                const uint32_t *s4 = (const uint32_t *)src;
                *(u32x4 *)dst = u32x4{s4[0], s4[1], s4[2], s4[3]};
            } else {
                for (int i = 0; i < 16 && k + i < K; ++i) dst[i] = src[i];
            }
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256) k_cols_factor(float *scale, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) scale[i] = scale[i] / 448.0f;
}

hipError_t launch_quant_cols_e4m3(const uint16_t *W, int64_t ldw, int64_t K, int64_t N, int align_w, uint8_t *Qt,
                                  int64_t ldq, int align_q, float *scale, hipStream_t s)
{
    // enough workgroups for the 256 CUs: column strips times ranges of K
    const int64_t strips = (N + 63) / 64, blocks = (K + 63) / 64;
    int64_t ky = (1024 + strips - 1) / strips;
    if (ky > blocks) ky = blocks;
    if (ky > 64) ky = 64;
    if (ky < 1) ky = 1;
    const dim3 g((unsigned)strips, (unsigned)ky), g1((unsigned)((N + 255) / 256));
    hipLaunchKernelGGL(k_fill_u32, g1, dim3(256), 0, s, (uint32_t *)scale, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (K > 0) {
        hipLaunchKernelGGL(k_cols_amax, g, dim3(256), 0, s, W, ldw, K, N, align_w, (uint32_t *)scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_quant_cols_e4m3, g, dim3(256), 0, s, W, ldw, K, N, align_w, Qt, ldq, align_q,
                           (const float *)scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_cols_factor, g1, dim3(256), 0, s, scale, N);
    }
    return hipGetLastError();
}

// The largest magnitude of each bf16 row of X (pass 1 of the row quantizer,
// the same reduction) into amax[r], and its factor amax / 448 into scale[r].
__global__ void __launch_bounds__(256) k_row_amax(const uint16_t *X, int64_t ldx, int64_t rows, int64_t cols,
                                                  int align_x, float *amax_out, float *scale)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    u32x4 v[8];
    const float amax = wave_row_amax<8>(X + r * ldx, cols, align_x, lane, v, cols <= 8 * 512);
    if (lane == 0) {
        amax_out[r] = amax;
        scale[r] = amax / 448.0f;
    }
}

// The scaled FP8 product with A quantized on load (Example 5-8's fused
// alternative): ring tiles 128 rows tall whose A slab is read as bf16 and
// converted to codes in LDS (RingTile QA).  Masked edges; K % 64 == 0.
// Each A element is converted once per column tile, so wider tiles convert
// less per flop: 128x256 (8 waves 2x4, 112 KiB of LDS, one workgroup per
// CU) or 128x128 (8 waves 4x2, 80 KiB, two per CU: its registers are held
// to 128 so that both fit).
template <int BN, int WGM, int WGN, int MINW>
__global__ void __launch_bounds__(512, MINW) k_f8_qa(GemmArgs p)
{
    using R = RingTile<128, BN, WGM, WGN, 2, 4, 16, true, EPI_NONE, true, true, false, true>;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[R::LDS_BYTES / 2];
    const TileCoord tc = tile_map(blockIdx.x, p.batch, p.tiles_m, p.tiles_n, p.group_m);
    f32x4 acc[R::FN][R::FM];
    R::zero(acc);
    R::accumulate(p, smem, tc, 0, p.K, acc);
    R::store(p, smem, tc, acc);
}

hipError_t launch_fp8_quant_a(const GemmArgs &a, float *amax, int tile_n, int64_t grid, hipStream_t s)
{
    if (tile_n != 128 && tile_n != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_row_amax, dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, s, (const uint16_t *)a.A, a.lda, a.M,
                       a.K, a.align_a, amax, const_cast<float *>(a.scale_a));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmArgs b = a;
    b.amax_a = amax;
    if (tile_n == 256) hipLaunchKernelGGL((k_f8_qa<256, 2, 4, 2>), dim3((unsigned)grid), dim3(512), 0, s, b);
    else hipLaunchKernelGGL((k_f8_qa<128, 4, 2, 4>), dim3((unsigned)grid), dim3(512), 0, s, b);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int EPI>
static hipError_t launch_f8(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(WGM * WGN * 64);
    if constexpr (BM == 128 && BN == 128) {
        if (a.ksplit > 1) return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI, true, true, true>(a, variant, g, b8, s);
    }
    return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI, false, true, true>(a, variant, g, b8, s);
}

template <int EPI>
static hipError_t launch_f8_cfg(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    switch (config_id) {
    case CFG_BF16_256x192: return launch_f8<256, 192, 2, 4, EPI>(a, variant, grid, s);
    case CFG_BF16_256x256: return launch_f8<256, 256, 2, 4, EPI>(a, variant, grid, s);
    case CFG_BF16_128x128: return launch_f8<128, 128, 4, 2, EPI>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ring_fp8(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    return launch_f8_cfg<EPI_NONE>(config_id, a, variant, grid, s);
}

hipError_t launch_ring_fp8_affine(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    return launch_f8_cfg<EPI_AFFINE>(config_id, a, variant, grid, s);
}

// Small M on E4M3FN operands: C[M, N] = (X[M, K] . Bt[N, K]^T) scaled by
// the factor of each row of X and of each row of Bt, for M <= 16.  As the
// bf16 transposed-B GEMV: a workgroup owns 16 x RB rows of Bt, its NW waves
// split K into contiguous ranges of 64-deep steps, and each lane loads 16
// bytes (16 K values) of a row per step, which feed two
// v_mfma_f32_16x16x32_fp8_fp8 (bytes 0-7, then 8-15: the same permutation
// of K for both operands).  A K remainder (K % 64) is a final step loaded
// element by element with zero fill.  The waves' partial sums are added in
// LDS in wave order (so a row's result does not depend on M), then scaled,
// passed through the affine epilogue when the call has one, and rounded
// once.  Batch entries are the second grid dimension.  Requires 16-byte
// aligned rows of Bt.
template <int NW, int RB>
__global__ void __launch_bounds__(NW * 64) k_decode_nt_f8(GemmArgs p)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
    const int64_t bidx = blockIdx.y;
    const uint8_t *X = (const uint8_t *)p.A + bidx * p.sA;
    const uint8_t *Bt = (const uint8_t *)p.B + bidx * p.sB;
    const float *scale_a = p.scale_a ? p.scale_a + bidx * p.s_scale_a : nullptr;
    const float *scale_b = p.scale_b ? p.scale_b + bidx * p.s_scale_b : nullptr;
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
            const float sa = scale_a ? scale_a[m] : 1.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + 16 * r + 4 * gg + q;
                if (n >= N) continue;
                const float sb = scale_b ? scale_b[n] : 1.0f;
                store_out(p, bidx, m, n, sum[q] * sa * sb);
            }
        }
    }
}

hipError_t launch_decode_nt_f8(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    if (variant == 2)
        hipLaunchKernelGGL((k_decode_nt_f8<8, 3>), dim3((unsigned)grid, (unsigned)a.batch), dim3(8 * 64), 0, s, a);
    else
        hipLaunchKernelGGL((k_decode_nt_f8<8, 1>), dim3((unsigned)grid, (unsigned)a.batch), dim3(8 * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace g5
