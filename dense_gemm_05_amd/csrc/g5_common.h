// g5_common.h -- definitions shared by the host dispatcher and the gfx950
// kernels of the dense-GEMM library: the workgroup -> tile map, the kernel
// argument block and the table of compiled kernel configurations.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define G5_HD __host__ __device__
#else
#define G5_HD
#endif

namespace g5 {

// Workgroups of one launch are handed to the 8 XCDs of an MI355X in
// round-robin order (workgroup w runs on XCD w % 8).  Each XCD has a private
// L2, so the map below first gathers the ids that land on one XCD into a
// contiguous run of logical tile indices, then walks the tile grid in column
// bands `group_m` tiles tall, column by column.  Tiles resident on one XCD at
// the same time then share a few row panels of A and column panels of B.
// This is the block-order argument of page "4.1 Tối ưu hiệu năng toán tử GEMM
// trên CUDA" (§2.3: block order moves the L2 hit rate) and the block-id
// swizzle of MUSA lesson m11-l5 (case 4: changing rows every few blocks lets
// A and B panels both be reused), re-derived for an XCD-partitioned L2.
constexpr int kNumXcd = 8;

struct TileCoord {
    int64_t b, tm, tn;
};

// group_m <= 0 selects the orders the XCD-aware one is measured against:
// 0 plain row-major tile order (workgroup w takes tile w, rows of tiles one
// after another), -g column bands g tiles tall without the XCD regrouping.
G5_HD inline TileCoord tile_map(int64_t wg, int64_t batch, int64_t tiles_m, int64_t tiles_n,
                                int64_t group_m)
{
    const int64_t per_batch = tiles_m * tiles_n;
    TileCoord t;
    if (group_m == 0) {
        t.b = wg / per_batch;
        const int64_t r = wg - t.b * per_batch;
        t.tm = r / tiles_n;
        t.tn = r - t.tm * tiles_n;
        return t;
    }
    const int64_t total = batch * per_batch;
    const int64_t rounds = total / kNumXcd;
    int64_t L = wg;
    if (group_m > 0 && wg < rounds * kNumXcd) L = (wg % kNumXcd) * rounds + wg / kNumXcd;
    if (group_m < 0) group_m = -group_m;
    t.b = L / per_batch;
    const int64_t r = L - t.b * per_batch;
    const int64_t band_tiles = group_m * tiles_n;
    const int64_t band = r / band_tiles;
    const int64_t first_m = band * group_m;
    const int64_t rem_m = tiles_m - first_m;
    const int64_t h = rem_m < group_m ? rem_m : group_m;
    const int64_t rr = r - band * band_tiles;
    t.tm = first_m + rr % h;
    t.tn = rr / h;
    return t;
}

// Argument block shared by all tiled kernels (passed by value).
struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;      // batch strides in elements
    int64_t batch;
    int64_t tiles_m, tiles_n;
    int64_t group_m;
    int32_t align_a;         // 16, 8, 4 or 2: alignment of every row start of A
    int32_t align_b;
    int32_t align_c;
    int32_t out_f32;         // 1: C is float, 0: C is bf16 bits
    // K split over workgroups (LDS-ring kernels with ksplit > 1): workgroup
    // w computes slice w / (batch*tiles_m*tiles_n) of the 32-deep stages of
    // tile w % (batch*tiles_m*tiles_n), kt_per stages (the last slice also
    // the rest of K); FP32 partial tiles and per-tile arrival counters live
    // in ws_part and ws_cnt.
    int32_t ksplit;
    int32_t kt_per;
    int32_t b_trans;         // 1: B is given as Bt [N, K] (element (k, n) at B + n*ldb + k)
    int32_t fp8;             // 1: A and Bt hold E4M3FN codes (with b_trans)
    const float *scale_a;    // fp8: factor of each row of A (M floats) or NULL
    const float *scale_b;    // fp8: factor of each row of Bt (N floats) or NULL
    int64_t s_scale_a;       // fp8: batch strides of the factors (floats; 0: shared by every entry)
    int64_t s_scale_b;
    // fp8 with A quantized on load: A holds bf16 rows and amax_a each row's
    // largest magnitude (M floats); scale_a = amax_a / 448.
    const float *amax_a;
    float *ws_part;
    unsigned *ws_cnt;
    // EPI_AFFINE: C := alpha * (A.B) + bias[n] + beta * C (C read only when
    // beta != 0; bias bf16 [N] or NULL, its start `align_bias`-byte aligned).
    float alpha, beta;
    const uint16_t *bias;
    int32_t align_bias;
    int32_t affine;          // 1: the small-M kernels apply the affine epilogue
    int32_t a_trans;         // 1: A is given as At [K, M] (element (m, k) at A + k*lda + m)
    // Epilogue of the small-M kernels (an Epilogue value).  EPI_SWIGLU: B is
    // the merged gate|up weight [K, 2N] (gate columns [0, N), up columns
    // [N, 2N)) and C the N columns of bf16(bf16(SiLU(g)) * u).
    int32_t epi;
    // EPI_SWIGLU with c_e4m3 = 1: C holds one E4M3FN code per output (bytes,
    // ldc and sC in bytes), the code nearest to z * 448 / c_amax for the
    // bf16 output z = bf16(t * u) (c_amax: the caller's fixed range, finite
    // and > 0).
    int32_t c_e4m3 = 0;
    float c_amax = 0.f;
};

// Fused epilogues of the bf16 ring kernels.
enum Epilogue { EPI_NONE = 0, EPI_SILU = 1, EPI_SWIGLU = 2, EPI_AFFINE = 3 };

// Compiled configurations.  The selector picks one; GEMM_FORCE_CONFIG may
// name one explicitly.
enum ConfigId {
    CFG_NONE = 0,
    CFG_ZERO,
    CFG_BF16_256x192,      // general kernel: 4 waves (2x2); ring kernels: 8 waves (2x4, wave tile 128x48)
    CFG_BF16_128x128,      // 4 waves (2x2), wave tile 64x64
    CFG_BF16_256x128,      // 4 waves (2x2), wave tile 128x64
    CFG_BF16_256x256,      // general kernel: 4 waves (2x2); ring kernels: 8 waves (2x4, wave tile 128x64)
    CFG_F32_128x128,       // 4 waves (2x2), wave tile 64x64
    CFG_F32_64x64,         // 4 waves (2x2), wave tile 32x32
    CFG_F32_32x32_WK,      // 4 waves (2x2), wave tile 16x16, all of K (<= 256) staged at once
    CFG_DECODE_64,         // small M, 64 columns per workgroup, 16 waves, K split in-workgroup
    CFG_DECODE_SPLIT,      // small M, 128-column strips, K split over workgroups too
    CFG_DECODE_NT,         // small M, B given transposed: 16 rows of Bt per workgroup, K split over 8 waves
    CFG_GENERIC,
    CFG_COUNT
};

struct ConfigInfo {
    int id;
    int family;            // gemm_family
    int tile_m, tile_n, tile_k;
    int threads;
    int lds_bytes;
    const char *name;
};

}  // namespace g5
