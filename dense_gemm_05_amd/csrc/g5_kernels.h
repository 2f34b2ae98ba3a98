// g5_kernels.h -- launch entry of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "g5_common.h"

namespace g5 {

// Enqueue compiled configuration `config_id` on stream `s` with `grid`
// workgroups.  `variant` selects the kernel variant (tiled configs: 0 fully
// general, 1 aligned without edge masking, 2/3 masked ring kernel copying A in
// 16- or 4-byte pieces); the caller guarantees its preconditions.  Returns the
// launch status.
hipError_t launch_config(int config_id, bool f32_inputs, const GemmArgs &a, int variant, int64_t grid,
                         hipStream_t s);

// The bf16 ring kernels with B given transposed (a.b_trans): variants 1-3
// of the configs 256x192, 256x256, 256x128 and 128x128, the last also with
// K split (a.ksplit > 1).
hipError_t launch_ring_bt(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// The bf16 ring kernels with A given transposed (a.a_trans): variants 1 and
// 2 of the configs 256x192, 256x256 and 128x128, the last also with K split.
hipError_t launch_ring_at(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// The ring kernels on E4M3FN operands (a.fp8, a.b_trans): variants 1-3 of
// the configs 256x192, 256x256 and 128x128, the last also with K split.
hipError_t launch_ring_fp8(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// The same with the affine epilogue applied to the dequantized sums.
hipError_t launch_ring_fp8_affine(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// The FP8 product with A quantized on load: each bf16 row's largest
// magnitude into amax[M] (device scratch) and its factor into a.scale_a,
// then 128 x tile_n tiles (tile_n 128 or 256; grid of them) that convert A
// to codes in LDS.  a.A
// holds bf16 rows (16-byte aligned), a.B the Bt codes; K % 64 == 0.
hipError_t launch_fp8_quant_a(const GemmArgs &a, float *amax, int tile_n, int64_t grid, hipStream_t s);

// Small M (<= 16) on E4M3FN operands with B given transposed: variant 1
// one 16-row block of Bt per workgroup, 2 three (grid = blocks of Bt rows).
hipError_t launch_decode_nt_f8(const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// Per-row E4M3FN quantization of `rows` bf16 rows of `cols` elements (row
// strides ldx, ldq; align_x, align_q the byte alignments of the row starts)
// into codes Q and dequantization factors scale[rows].
hipError_t launch_quant_rows_e4m3(const uint16_t *X, int64_t ldx, int64_t rows, int64_t cols, int align_x,
                                  uint8_t *Q, int64_t ldq, int align_q, float *scale, hipStream_t s);

// Per-column E4M3FN quantization of W [K, N] (bf16, row stride ldw, rows
// `align_w`-byte aligned) into the rows of Qt [N, K] (row stride ldq, rows
// `align_q`-byte aligned) with the factors scale[N].
hipError_t launch_quant_cols_e4m3(const uint16_t *W, int64_t ldw, int64_t K, int64_t N, int align_w, uint8_t *Qt,
                                  int64_t ldq, int align_q, float *scale, hipStream_t s);

// The same for a bf16 product with a fused epilogue (EPI_SILU, EPI_SWIGLU
// or EPI_AFFINE; ring kernel variants 1-3 of the configs 256x192, 256x256
// and 128x128, the last also with K split for EPI_AFFINE, with a.tiles_n
// counting output tiles of tile_n / 2 columns for EPI_SWIGLU).
hipError_t launch_fused(int config_id, int epi, const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// The affine epilogue alone (K == 0 or alpha == 0): C := bias[n] + beta * C
// over a.batch x a.M x a.N, reading C only when a.beta != 0.
hipError_t launch_affine_no_product(const GemmArgs &a, int64_t grid, hipStream_t s);

// Copy batch x M rows of K bf16 elements (row stride lda, batch stride sA,
// rows `align`-byte aligned) into A2 with row stride lda2 (a multiple of 8,
// >= K) and batch stride M x lda2, zero-filling columns K..lda2-1.
hipError_t launch_realign_rows(const uint16_t *A, int64_t lda, int64_t sA, int64_t batch, int64_t M, int64_t K,
                               int align, uint16_t *A2, int64_t lda2, hipStream_t s);

// Small-M path with K split over `ks` workgroups per 128-column strip
// (a.tiles_n strips; 2 ks for a.epi == EPI_SWIGLU: ks on the gate columns,
// ks on the up columns): `ws` holds batch x strips x (ks or 2 ks) x 16 x 128
// floats of partial sums, `cnt` batch x strips counters that are zero on
// entry and left zero on exit.  With `pair` (ks == 2, or ks == 1 for
// SwiGLU: two members per strip): no partial sums or counters, but
// batch x M x N 32-bit exchange slots, zero on entry and left zero.
// Requires N % 128 == 0, K % 32 == 0, 16-byte aligned rows of X and W.
hipError_t launch_decode_split(const GemmArgs &a, float *ws, unsigned *cnt, int ks, unsigned *pair, hipStream_t s);

// The bf16 ring kernel on a persistent stream-K schedule (variants 1 and 2
// of the configs 256x256 and 256x192; `grid` workgroups, a multiple of 8):
// a.ws_part holds 2 x grid partial tiles of FP32, a.ws_cnt one counter per
// output tile (zero on entry, left zero).  Requires K % 32 == 0.
hipError_t launch_streamk(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s);

// The library's own scratch memory (gemm_run_noalloc): kScratchBytes of
// device memory per GPU, in a file-scope device array.  noalloc_scratch
// returns the current device's copy (its address looked up once per
// device); launch_clear_counters zeroes its first n arrival counters.
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_clear_counters(void *base, int64_t n, hipStream_t s);

// The activation chain on stored bf16 operands (g5_act.hip): steps of page
// "Operator & Runtime" §5.3.1, Example 5-4, each alone or fused.
enum ActStep {
    ACT_SILU = 0,         // in0 = G -> out = T = bf16(SiLU(g))
    ACT_MUL = 1,          // in0 = T, in1 = U -> out = Z = bf16(t * u)
    ACT_SWIGLU = 2,       // in0 = G, in1 = U -> out = Z (SiLU and product fused)
    ACT_QUANT = 3,        // in0 = Z -> out = E4M3FN codes against amax
    ACT_SWIGLU_E4M3 = 4   // in0 = G, in1 = U -> out = the codes of Z (all three fused)
};
struct ActArgs {
    const uint16_t *in0;
    const uint16_t *in1;     // NULL for the one-input steps
    void *out;               // bf16, or E4M3FN codes (bytes) for the quantizing steps
    int64_t M, N;
    int64_t ld0, ld1, ldo;   // row strides in elements
    float amax;              // the quantizing steps' range (> 0)
};
// vec: N % 8 == 0, 16-byte aligned input rows, 16-byte (bf16) or 8-byte
// (codes) aligned output rows and M * N / 8 < 2^32; contig additionally every
// ld == N.  Else one element per thread.
hipError_t launch_act_chain(int step, const ActArgs &a, bool vec, bool contig, hipStream_t s);

}  // namespace g5
