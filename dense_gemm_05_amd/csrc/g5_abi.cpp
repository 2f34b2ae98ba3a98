// g5_abi.cpp -- C entry points of the dense-GEMM library: argument
// validation, the tile-configuration selector and kernel dispatch.
//
// Validation and selection run on the host only and touch no GPU state, so
// they are usable (through gemm_plan_query) without a device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/gemm05.h"
#include "g5_common.h"
#include "g5_kernels.h"

namespace g5 {
namespace {

// ------------------------------------------------------------ config table
const ConfigInfo kConfigs[CFG_COUNT] = {
    {CFG_NONE, GEMM_FAMILY_NONE, 0, 0, 0, 0, 0, "none"},
    {CFG_ZERO, GEMM_FAMILY_ZERO, 0, 0, 0, 256, 0, "zero"},
    {CFG_BF16_256x192, GEMM_FAMILY_BF16_MFMA, 256, 192, 64, 256, 2 * (256 * 64 + 64 * 192) * 2, "bf16_256x192"},
    {CFG_BF16_128x128, GEMM_FAMILY_BF16_MFMA, 128, 128, 64, 256, 2 * (128 * 64 + 64 * 128) * 2, "bf16_128x128"},
    {CFG_BF16_256x128, GEMM_FAMILY_BF16_MFMA, 256, 128, 64, 256, 2 * (256 * 64 + 64 * 128) * 2, "bf16_256x128"},
    {CFG_BF16_256x256, GEMM_FAMILY_BF16_MFMA, 256, 256, 64, 256, 2 * (256 * 64 + 64 * 256) * 2, "bf16_256x256"},
    {CFG_F32_128x128, GEMM_FAMILY_F32_MFMA, 128, 128, 32, 256, 2 * (128 * 32 + 32 * 132) * 4, "f32_128x128"},
    {CFG_F32_64x64, GEMM_FAMILY_F32_MFMA, 64, 64, 32, 256, 2 * (64 * 32 + 32 * 68) * 4, "f32_64x64"},
    {CFG_F32_32x32_WK, GEMM_FAMILY_F32_MFMA, 32, 32, 256, 256, 8 * (32 * 32 + 32 * 36) * 4, "f32_32x32_wholek"},
    {CFG_DECODE_64, GEMM_FAMILY_DECODE, 16, 64, 32, 1024, 16 * 64 * 17 * 4, "decode_64"},
    {CFG_DECODE_SPLIT, GEMM_FAMILY_DECODE, 16, 128, 32, 1024, 16 * 64 * 33 * 4 + 4, "decode_splitk"},
    {CFG_DECODE_NT, GEMM_FAMILY_DECODE, 16, 16, 32, 512, 8 * 64 * 16, "decode_nt"},
    {CFG_GENERIC, GEMM_FAMILY_GENERIC, 16, 16, 16, 256, 2 * 16 * 17 * 4, "generic"},
};

// MI355X figures used by the selector's cost model.
constexpr int kNumCU = 256;
constexpr int64_t kLdsPerCU = 160 * 1024;
constexpr double kHbmBytesPerS = 8.0e12;
constexpr double kCopyBytesPerCUperS = 40.8e9;   // measured, LDS-ring kernels (see model_time)
constexpr double kBf16FlopsPerCUperS = 2.5166e15 / kNumCU;
constexpr double kF32FlopsPerCUperS = 157.3e12 / kNumCU;

struct Problem {
    int op;  // gemm_op
    int64_t batch, M, N, K;
    uint64_t a, b, c;
    int64_t lda, ldb, ldc, sA, sB, sC;
    int c_type;
    uint64_t scale_a = 0, scale_b = 0;   // fp8: dequantization factors (float), 0 = none
    // affine epilogue: C := alpha * (A.B) + bias[n] + beta * C
    float alpha = 1.0f, beta = 0.0f;
    uint64_t bias = 0;                   // bf16 [N], 0 = none
    // SwiGLU with c_type GEMM_OUT_E4M3: the fixed range that maps to 448
    float out_amax = 0.0f;
};

struct Plan {
    int config = CFG_NONE;
    bool even = false;       // no edge masking
    int variant = 0;         // kernel variant passed to launch_config
    int64_t grid = 0;
    int64_t tiles_m = 0, tiles_n = 0, group_m = 1;
    int align_a = 2, align_b = 2, align_c = 2;
    int ks = 1;              // K slices of the split small-M path
    int ksplit = 1;          // K slices of a tiled bf16 call (128x128 ring kernel)
    bool realign_a = false;  // copy A's rows to 16-byte aligned ones first
    int64_t lda2 = 0;        // row stride of that copy (elements)
    bool realign_b = false;  // the same for the rows of a transposed B (Bt [N, K])
    int64_t ldb2 = 0;
    bool streamk = false;    // tiled bf16 call on the persistent stream-K schedule (grid = kNumCU)
    double model_bytes = 0.0;
};

// K slices per strip of the split small-M path: enough workgroups for the
// 256 CUs (at most 8 slices, each at least 16 steps of 32 rows).
int decode_slices(int64_t strips, int64_t K)
{
    int64_t ks = 256 / (strips > 0 ? strips : 1);
    const int64_t by_k = K / (32 * 16);
    if (ks > by_k) ks = by_k;
    if (ks > 8) ks = 8;
    return ks < 1 ? 1 : (int)ks;
}

// E4M3FN operands (A and Bt codes with per-row factors).
bool is_fp8(const Problem &p) { return p.op == GEMM_OP_FP8_NT || p.op == GEMM_OP_FP8_NT_AFFINE; }
int elem_a(const Problem &p) { return p.op == GEMM_OP_SGEMM ? 4 : is_fp8(p) ? 1 : 2; }
// K per stage of the LDS-ring kernels: 64-byte slot rows of bf16 or fp8.
int stage_k(const Problem &p) { return is_fp8(p) ? 64 : 32; }
// Batch strides of the fp8 factors (floats): an operand shared by every
// batch entry (stride 0, or a single entry) shares its factors too; else
// entry b's factors follow entry b-1's (M of A's rows, N of Bt's).
int64_t scale_stride_a(const Problem &p) { return p.batch > 1 && p.sA != 0 ? p.M : 0; }
int64_t scale_stride_b(const Problem &p) { return p.batch > 1 && p.sB != 0 ? p.N : 0; }
// Fused epilogue of an operation (EPI_NONE for the plain products).
int epi_of(const Problem &p)
{
    return p.op == GEMM_OP_BF16_SILU     ? EPI_SILU
           : p.op == GEMM_OP_BF16_SWIGLU ? EPI_SWIGLU
           : p.op == GEMM_OP_BF16_AFFINE || p.op == GEMM_OP_BF16_NT_AFFINE || p.op == GEMM_OP_BF16_TN_AFFINE ||
                   p.op == GEMM_OP_FP8_NT_AFFINE
               ? EPI_AFFINE
               : EPI_NONE;
}
bool is_affine(const Problem &p) { return epi_of(p) == EPI_AFFINE; }
// The output type of the generic entry points: FP32 for SGEMM, bf16 for
// SiLU, bf16 or (when asked for) E4M3FN codes for SwiGLU, else the caller's.
int op_c_type(int op, int c_type)
{
    if (op == GEMM_OP_SGEMM) return GEMM_OUT_F32;
    if (op == GEMM_OP_BF16_SILU) return GEMM_OUT_BF16;
    if (op == GEMM_OP_BF16_SWIGLU) return c_type == GEMM_OUT_E4M3 ? GEMM_OUT_E4M3 : GEMM_OUT_BF16;
    return c_type;
}
// An affine call with no product to form (alpha == 0: A and B are not read).
bool no_product(const Problem &p) { return is_affine(p) && p.alpha == 0.0f; }
// B is given transposed, Bt [N, K].
bool b_trans(const Problem &p)
{
    return p.op == GEMM_OP_BF16_NT || is_fp8(p) || p.op == GEMM_OP_BF16_NT_AFFINE;
}
// A is given transposed, At [K, M].
bool a_trans(const Problem &p) { return p.op == GEMM_OP_BF16_TN || p.op == GEMM_OP_BF16_TN_AFFINE; }
// Rows and columns of the A operand as stored: [M, K] or At [K, M].
int64_t a_rows(const Problem &p) { return a_trans(p) ? p.K : p.M; }
int64_t a_cols(const Problem &p) { return a_trans(p) ? p.M : p.K; }
// Rows and columns of the B operand as stored: [K, N], Bt [N, K], or the
// merged gate|up weight [K, 2N] of SwiGLU.
int64_t b_rows(const Problem &p) { return b_trans(p) ? p.N : p.K; }
int64_t b_cols(const Problem &p) { return b_trans(p) ? p.K : p.op == GEMM_OP_BF16_SWIGLU ? 2 * p.N : p.N; }
// Calls only the LDS-ring kernels can run (variants 1-3) when they take a
// tiled config (the affine epilogue also runs in the small-M kernels).
bool ring_only(const Problem &p) { return epi_of(p) != EPI_NONE || b_trans(p) || a_trans(p); }
bool tiled(int config) { return kConfigs[config].family == GEMM_FAMILY_BF16_MFMA; }
// Output columns per tile of a tiled config (SwiGLU: half the B columns).
int64_t out_tile_n(const Problem &p, const ConfigInfo &c)
{
    return p.op == GEMM_OP_BF16_SWIGLU ? c.tile_n / 2 : c.tile_n;
}
int elem_c(const Problem &p)
{
    return p.c_type == GEMM_OUT_E4M3 ? 1 : (p.op == GEMM_OP_SGEMM || p.c_type == GEMM_OUT_F32) ? 4 : 2;
}

// Largest power of two <= 16 dividing the address of every row start of an
// operand (pointer, row stride and batch stride all in bytes).
int row_alignment(uint64_t ptr, int64_t ld, int64_t stride, int64_t batch, int esz)
{
    uint64_t bits = ptr | (uint64_t)(ld * esz);
    if (batch > 1) bits |= (uint64_t)(stride * esz);
    int a = 16;
    while (a > 1 && (bits % (uint64_t)a) != 0) a >>= 1;
    return a;
}

// [lo, hi) byte range touched by an operand with rows x cols elements.
struct Range {
    __int128 lo, hi;
};
Range extent(uint64_t ptr, int64_t batch, int64_t rows, int64_t cols, int64_t ld, int64_t stride, int esz)
{
    __int128 last = (__int128)(batch - 1) * stride + (__int128)(rows - 1) * ld + cols;
    return Range{(__int128)ptr, (__int128)ptr + last * esz};
}
bool overlap(const Range &x, const Range &y) { return x.lo < y.hi && y.lo < x.hi; }

int validate(const Problem &p)
{
    if (p.op != GEMM_OP_SGEMM && p.op != GEMM_OP_BF16 && p.op != GEMM_OP_BF16_SILU && p.op != GEMM_OP_BF16_SWIGLU &&
        p.op != GEMM_OP_BF16_NT && p.op != GEMM_OP_FP8_NT && p.op != GEMM_OP_BF16_AFFINE && p.op != GEMM_OP_BF16_TN &&
        p.op != GEMM_OP_BF16_NT_AFFINE && p.op != GEMM_OP_BF16_TN_AFFINE && p.op != GEMM_OP_FP8_NT_AFFINE)
        return GEMM_ERR_INVALID_ARG;
    if (p.batch < 0 || p.M < 0 || p.N < 0 || p.K < 0) return GEMM_ERR_INVALID_ARG;
    if ((p.op == GEMM_OP_BF16 || p.op == GEMM_OP_BF16_NT || is_fp8(p) || is_affine(p) ||
         p.op == GEMM_OP_BF16_TN) &&
        p.c_type != GEMM_OUT_BF16 && p.c_type != GEMM_OUT_F32)
        return GEMM_ERR_INVALID_ARG;
    if (is_fp8(p) && ((p.scale_a % 4) || (p.scale_b % 4))) return GEMM_ERR_INVALID_ARG;
    if (p.op == GEMM_OP_BF16_SILU && p.c_type != GEMM_OUT_BF16) return GEMM_ERR_INVALID_ARG;
    // SwiGLU writes bf16, or E4M3FN codes against a finite positive range
    if (p.op == GEMM_OP_BF16_SWIGLU && p.c_type != GEMM_OUT_BF16 &&
        (p.c_type != GEMM_OUT_E4M3 || !std::isfinite(p.out_amax) || !(p.out_amax > 0.0f)))
        return GEMM_ERR_INVALID_ARG;
    if (is_affine(p) && (!std::isfinite(p.alpha) || !std::isfinite(p.beta) || (p.bias % 2)))
        return GEMM_ERR_INVALID_ARG;
    if (p.sA < 0 || p.sB < 0 || p.sC < 0) return GEMM_ERR_INVALID_ARG;
    if (p.batch == 0 || p.M == 0 || p.N == 0) return GEMM_OK;  // nothing to do
    if (p.ldc < p.N || p.c == 0) return GEMM_ERR_INVALID_ARG;
    if (p.batch > 1 && (__int128)p.sC < (__int128)(p.M - 1) * p.ldc + p.N) return GEMM_ERR_INVALID_ARG;
    const Range rc = extent(p.c, p.batch, p.M, p.N, p.ldc, p.sC, elem_c(p));
    if (rc.hi > ((__int128)1 << 63)) return GEMM_ERR_INVALID_ARG;
    if (p.bias && overlap(rc, Range{(__int128)p.bias, (__int128)p.bias + 2 * (__int128)p.N})) return GEMM_ERR_INVALID_ARG;
    if (p.K == 0 || no_product(p)) return GEMM_OK;
    if (p.lda < a_cols(p) || p.ldb < b_cols(p) || p.a == 0 || p.b == 0) return GEMM_ERR_INVALID_ARG;
    const Range ra = extent(p.a, p.batch, a_rows(p), a_cols(p), p.lda, p.sA, elem_a(p));
    const Range rb = extent(p.b, p.batch, b_rows(p), b_cols(p), p.ldb, p.sB, elem_a(p));
    if (ra.hi > ((__int128)1 << 63) || rb.hi > ((__int128)1 << 63)) return GEMM_ERR_INVALID_ARG;
    if (overlap(rc, ra) || overlap(rc, rb)) return GEMM_ERR_INVALID_ARG;
    const __int128 na = (__int128)(p.batch - 1) * scale_stride_a(p) + p.M;
    const __int128 nb = (__int128)(p.batch - 1) * scale_stride_b(p) + p.N;
    if (p.scale_a && overlap(rc, Range{(__int128)p.scale_a, (__int128)p.scale_a + 4 * na})) return GEMM_ERR_INVALID_ARG;
    if (p.scale_b && overlap(rc, Range{(__int128)p.scale_b, (__int128)p.scale_b + 4 * nb})) return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Cost model of a tiled config (seconds), page "Operator & Runtime" §5.4.5
// (estimate first, then correct by measurement).  The interface traffic of
// §5.2.2 -- every tile reads its A row panel and B column panel and writes
// its C block -- is on gfx950 served mostly by the L2 and the Infinity Cache,
// and what it limits is each CU's copy path: a tile's operand bytes pass
// through one CU at the measured copy rate of the LDS-ring kernels (about
// 41 GB/s per CU: 3.77 MB per 256x192 tile of the FFN projection in a
// ~92 us main loop).  A CU that runs n tiles pays n times the slower of its
// matrix-core time and its copy time; the whole call is never faster than
// reading the operands and writing C once from HBM.  The result is divided
// by a relative efficiency measured per tile shape.
double model_time(const Problem &p, const ConfigInfo &c, double eff)
{
    const int64_t tm = cdiv(p.M, c.tile_m), tn = cdiv(p.N, out_tile_n(p, c));
    const int64_t tiles = p.batch * tm * tn;
    const int64_t per_cu = cdiv(tiles, (int64_t)kNumCU);
    // (E4M3 operands: the double-rate fp8 matrix instruction)
    const double rate = p.op == GEMM_OP_SGEMM ? kF32FlopsPerCUperS
                        : is_fp8(p)           ? 2.0 * kBf16FlopsPerCUperS
                                              : kBf16FlopsPerCUperS;
    const double kpad = (double)cdiv(p.K, c.tile_k) * c.tile_k;
    const double t_mfma = (2.0 * c.tile_m * c.tile_n * kpad) / rate;
    const double tile_bytes =
        (double)(c.tile_m + c.tile_n) * kpad * elem_a(p) + (double)c.tile_m * out_tile_n(p, c) * elem_c(p);
    const double t_copy = tile_bytes / kCopyBytesPerCUperS;
    const double t_tiles = (double)per_cu * (t_mfma > t_copy ? t_mfma : t_copy);
    const double once =
        (double)p.batch * ((double)elem_a(p) * (p.M * p.K + p.K * b_cols(p)) + (double)elem_c(p) * p.M * p.N);
    const double t_hbm = once / kHbmBytesPerS;
    return (t_tiles > t_hbm ? t_tiles : t_hbm) / eff;
}

// The same for the 128x128 ring kernel with K split into S slices: each
// tile's S workgroups run 1/S of the stages, each publishes its FP32 tile
// and the last reads the other S-1 back (both through the CU's copy path).
double model_time_split(const Problem &p, const ConfigInfo &c, int S, double eff)
{
    Problem q = p;
    q.K = cdiv(cdiv(p.K, stage_k(p)), S) * stage_k(p);
    q.batch = p.batch * S;
    const double combine = (double)S * c.tile_m * c.tile_n * 4 / kCopyBytesPerCUperS;
    return model_time(q, c, eff) + combine / eff;
}

int find_config_by_name(const char *name)
{
    for (int i = 0; i < CFG_COUNT; ++i)
        if (std::strcmp(kConfigs[i].name, name) == 0) return i;
    return -1;
}

// Configurations compiled with the fused epilogues (and with fp8 operands).
bool has_epilogues(int id) { return id == CFG_BF16_256x192 || id == CFG_BF16_256x256 || id == CFG_BF16_128x128; }

bool config_fits(const Problem &p, int id)
{
    const ConfigInfo &c = kConfigs[id];
    if (epi_of(p) != EPI_NONE && c.family == GEMM_FAMILY_DECODE) {   // the small-M kernels apply them too
        if (a_trans(p)) return false;
        if (b_trans(p)) return id == CFG_DECODE_NT && p.M <= 16 && p.batch <= 65535;   // (affine only)
        return (id == CFG_DECODE_64 || id == CFG_DECODE_SPLIT) && p.M <= 16 && p.batch <= 65535;
    }
    if (epi_of(p) != EPI_NONE) return has_epilogues(id);
    if (p.op == GEMM_OP_FP8_NT && id == CFG_DECODE_NT) return p.M <= 16 && p.batch <= 65535;   // k_decode_nt_f8
    if (p.op == GEMM_OP_FP8_NT) return has_epilogues(id);         // fp8 ring kernels: 256x192, 256x256, 128x128
    if (a_trans(p)) return has_epilogues(id);                       // transposed-A ring kernels: the same three
    if (b_trans(p)) return c.family == GEMM_FAMILY_BF16_MFMA;   // the ring kernels of every bf16 tile config
    switch (c.family) {
    case GEMM_FAMILY_BF16_MFMA: return p.op == GEMM_OP_BF16;
    case GEMM_FAMILY_F32_MFMA: return p.op == GEMM_OP_SGEMM;
    case GEMM_FAMILY_DECODE:
        if (id == CFG_DECODE_NT) return p.op == GEMM_OP_BF16_NT && p.M <= 16 && p.batch <= 65535;
        return p.op == GEMM_OP_BF16 && p.M <= 16 && p.batch <= 65535;
    case GEMM_FAMILY_GENERIC: return true;
    default: return false;
    }
}

void fill_grid(const Problem &p, Plan &pl, bool ws)
{
    const ConfigInfo &c = kConfigs[pl.config];
    switch (c.family) {
    case GEMM_FAMILY_ZERO: {
        const int64_t total = p.batch * p.M * p.N;
        int64_t g = cdiv(total, 256);
        if (g > 4096) g = 4096;
        pl.grid = g;
        break;
    }
    case GEMM_FAMILY_DECODE:
        pl.tiles_m = 1;
        // (decode_nt: three 16-row blocks per workgroup when M > 1)
        pl.tiles_n = cdiv(p.N, c.tile_n * (pl.config == CFG_DECODE_NT && p.M > 1 ? 3 : 1));
        pl.grid = pl.tiles_n;  // x; batch goes to grid y
        if (pl.config == CFG_DECODE_SPLIT) {
            // (SwiGLU: a strip's gate and up columns are read by separate workgroups)
            // (one slice, a direct store, without a workspace)
            const int64_t groups = pl.tiles_n * (p.op == GEMM_OP_BF16_SWIGLU ? 2 : 1);
            pl.ks = ws ? decode_slices(groups * p.batch, p.K) : 1;
            pl.grid = groups * pl.ks;
        }
        break;
    default:
        pl.tiles_m = cdiv(p.M, c.tile_m);
        pl.tiles_n = cdiv(p.N, out_tile_n(p, c));
        pl.grid = p.batch * pl.tiles_m * pl.tiles_n * pl.ksplit;
        break;
    }
    // Column bands as tall as the whole M extent when it is only a few tiles
    // (each XCD then owns whole column panels of B), else 8 tiles tall.
    pl.group_m = pl.tiles_m <= 8 ? (pl.tiles_m > 0 ? pl.tiles_m : 1) : 8;
    // diagnostic: the orders the map is measured against (GEMM_TILE_ORDER =
    // "rowmajor": tile w for workgroup w; "bands": the same column bands
    // without gathering each XCD's workgroups)
    if (const char *o = std::getenv("GEMM_TILE_ORDER")) {
        if (std::strcmp(o, "rowmajor") == 0) pl.group_m = 0;
        else if (std::strcmp(o, "bands") == 0) pl.group_m = -pl.group_m;
    }
    pl.model_bytes = (c.tile_m > 0 && p.K > 0)
                         ? p.batch * gemm_model_traffic_bytes(p.M, p.N, p.K, c.tile_m, c.tile_n, elem_a(p))
                         : 0.0;
}

// Tiled kernel variant for a config (see launch_config): the aligned ring
// kernel when the problem is whole tiles with 16-byte rows, the masked ring
// kernel when B rows are 16-byte and A rows at least 4-byte aligned and each
// operand's byte extent fits 31 bits (32-bit buffer offsets), else the fully
// general kernel.
int pick_variant(const Problem &p, const Plan &pl, bool *even)
{
    const ConfigInfo &c = kConfigs[pl.config];
    *even = false;
    if (pl.config == CFG_F32_32x32_WK) {     // all of K at once: whole tiles and slabs only
        *even = !(p.M % 32 || p.N % 32 || p.K % 32) && p.K <= 256 && pl.align_a >= 16 && pl.align_b >= 16 &&
                pl.align_c >= 16;
        return *even ? 1 : -1;
    }
    if (c.family == GEMM_FAMILY_F32_MFMA) {
        *even = !(p.M % c.tile_m || p.N % c.tile_n || p.K % c.tile_k) && pl.align_a >= 16 && pl.align_b >= 16 &&
                pl.align_c >= 16;
        return *even ? 1 : 0;
    }
    if (pl.config == CFG_DECODE_NT) {      // 16-byte loads of Bt rows; 3 row blocks per workgroup for M > 1
        *even = pl.align_b >= 16;
        return *even ? (p.M > 1 ? 2 : 1) : -1;
    }
    if (c.family == GEMM_FAMILY_DECODE) {
        *even = (p.N % c.tile_n == 0) && pl.align_b >= 8 && pl.align_a >= 16;
        if (pl.config == CFG_DECODE_SPLIT)     // 16-byte loads of whole steps only
            return (*even && pl.align_b >= 16 && p.K % 32 == 0) ? 1 : -1;
        return *even ? 1 : 0;
    }
    if (c.family != GEMM_FAMILY_BF16_MFMA) return 0;
    // (At: the masked copy reads the last row up to M rounded up to 8)
    const __int128 a_bytes = ((__int128)(a_rows(p) - 1) * p.lda + (a_trans(p) ? (p.M + 7) / 8 * 8 : p.K)) * 2;
    const __int128 b_bytes = ((__int128)(b_rows(p) - 1) * p.ldb + b_cols(p)) * 2;
    const bool fits = a_bytes < ((__int128)1 << 31) && b_bytes < ((__int128)1 << 31);
    // N % 8: every 16-byte chunk of B lies wholly inside or wholly past the
    // descriptor extent (no partially out-of-range copies).
    // (Bt's chunks run along K like A's: no condition on N.)
    if (!fits || pl.align_b < 16 || pl.align_a < 4 || (!b_trans(p) && p.N % 8 != 0)) return 0;
    // At is copied 16 bytes per lane in whole chunks: aligned rows, and M % 8
    // == 0 unless the rows are the padded copy.
    if (a_trans(p) && (pl.align_a < 16 || (p.M % 8 != 0 && !pl.realign_a))) return 0;
    const int ring_k = stage_k(p);
    const bool c_ok = pl.align_c >= (elem_c(p) == 4 ? 16 : 8);
    *even = !(p.M % c.tile_m || p.N % out_tile_n(p, c) || p.K % ring_k) && pl.align_a >= 16 && c_ok;
    if (*even) return 1;
    return pl.align_a >= 16 ? 2 : 3;
}

// A K split into S slices of whole 32-deep stages, each at least 4 stages,
// with partial tiles addressable by 32-bit buffer offsets per tile.
bool split_ok(const Problem &p, int S)
{
    const int64_t kt = p.K / stage_k(p);
    return S >= 2 && S <= 8 && kt >= 4 * S && p.batch * cdiv(p.M, 128) * cdiv(p.N, 128) * S <= ((int64_t)1 << 24);
}

// Stages per slice of a K split (the last slice also takes the rest of K).
int split_kt_per(const Problem &p, int S) { return (int)((p.K / stage_k(p)) / S); }

// Counters live in the first kCounterBytes of a workspace: a split call
// needs one per output tile (tiled kernels) or per strip (small-M path), or
// one exchange slot per output (small-M path with two slices).
constexpr size_t kCounterBytes = GEMM_WORKSPACE_COUNTER_BYTES;
constexpr int64_t kMaxCounters = (int64_t)(kCounterBytes / sizeof(unsigned));

// The plan of a call.  `ws`: a caller workspace will be passed, so the
// paths that need scratch memory (K split over workgroups, the split small-M
// path, realigned row copies) may be chosen; without one they are not.
// The persistent stream-K schedule runs plain bf16 products (A as [M, K], B
// as [K, N], no fused epilogue) on the 256x256 and 256x192 ring kernels with
// 16-byte rows (variants 1 and 2), whole 32-deep stages, a workspace and at
// most one counter per tile in its counter region.
bool streamk_ok(const Problem &p, const Plan &pl, bool ws)
{
    return ws && p.op == GEMM_OP_BF16 && (pl.config == CFG_BF16_256x256 || pl.config == CFG_BF16_256x192) &&
           (pl.variant == 1 || pl.variant == 2) && !pl.realign_a && p.K % 32 == 0 && p.K > 0 &&
           p.batch * pl.tiles_m * pl.tiles_n <= kMaxCounters;
}

// Returns GEMM_OK or GEMM_ERR_UNSUPPORTED.
int select_plan(const Problem &p, Plan &pl, bool ws)
{
    pl = Plan();
    if (p.batch == 0 || p.M == 0 || p.N == 0) {
        pl.config = CFG_NONE;
        return GEMM_OK;
    }
    const int ea = elem_a(p), ec = elem_c(p);
    pl.align_a = row_alignment(p.a, p.lda, p.sA, p.batch, ea);
    pl.align_b = row_alignment(p.b, p.ldb, p.sB, p.batch, ea);
    pl.align_c = row_alignment(p.c, p.ldc, p.sC, p.batch, ec);
    if (p.K == 0 || no_product(p)) {
        pl.config = CFG_ZERO;
        fill_grid(p, pl, ws);
        return GEMM_OK;
    }

    // The fused epilogues run in the LDS-staged store of the ring kernels:
    // 16-byte aligned output rows and whole 16-byte output chunks.
    if (epi_of(p) != EPI_NONE && (pl.align_c < 16 || p.N % 8 != 0)) return GEMM_ERR_UNSUPPORTED;
    const char *force = std::getenv("GEMM_FORCE_CONFIG");
    if (force && *force) {
        const int id = find_config_by_name(force);
        if (id < 0 || !config_fits(p, id) || kConfigs[id].family == GEMM_FAMILY_ZERO ||
            kConfigs[id].family == GEMM_FAMILY_NONE)
            return GEMM_ERR_UNSUPPORTED;
        pl.config = id;
    } else if (p.op == GEMM_OP_SGEMM && p.K <= 256 && cdiv(p.M, 64) * cdiv(p.N, 64) * p.batch < kNumCU &&
               [&] { Plan t = pl; t.config = CFG_F32_32x32_WK; bool ev; return pick_variant(p, t, &ev) == 1; }()) {
        // A small FP32 problem with few slabs: 32x32 tiles with all of K
        // staged at once (one load latency per tile instead of one per slab;
        // 256^3 measured 9.4 us with the double-buffered 64x64 kernel).
        pl.config = CFG_F32_32x32_WK;
    } else if ((p.op == GEMM_OP_BF16_NT || p.op == GEMM_OP_BF16_NT_AFFINE || is_fp8(p)) && p.M <= 16 &&
               p.batch <= 65535 && pl.align_b >= 16) {
        // Small M with B transposed: a GEMV over the contiguous rows of Bt.
        pl.config = CFG_DECODE_NT;
    } else if ((p.op == GEMM_OP_BF16 || p.op == GEMM_OP_BF16_AFFINE || p.op == GEMM_OP_BF16_SILU ||
                p.op == GEMM_OP_BF16_SWIGLU) &&
               p.M <= 16 && p.batch <= 65535) {
        // The split path (128-column strips, 256 bytes of each W row) when
        // its preconditions hold and it would use more than one slice, or
        // enough whole-K strips to occupy most CUs on their own (one slice:
        // no partial sums, no workspace); SwiGLU always combines its gate and
        // up workgroups, so it needs the workspace.  Else whole-K strips of
        // 64 columns.
        pl.config = CFG_DECODE_SPLIT;
        bool ev = false;
        const bool glu = p.op == GEMM_OP_BF16_SWIGLU;
        const int64_t strips = cdiv(p.N, 128) * p.batch;
        const int ks = ws ? decode_slices(strips * (glu ? 2 : 1), p.K) : 1;
        const bool split = glu ? ws : (ks >= 2 || strips >= kNumCU * 3 / 4);
        if (!split || pick_variant(p, pl, &ev) < 0 || strips > kMaxCounters) pl.config = CFG_DECODE_64;
    } else {
        // Candidates with their measured relative efficiency; the model
        // picks the fastest (page "Operator & Runtime" §5.4.5: feasibility,
        // then an estimate, then measurement).
        struct Cand {
            int id;
            double eff;
        };
        // 256x256 tiles move the fewest bytes per flop through the copy
        // path and LDS, and carry the same measured per-flop rate as 256x192
        // when the tile count fills whole waves: bf16 4096^3 116.6 us
        // against 164.9 us for 256x192 (352 tiles, 2 waves); the FFN shape
        // (192 tiles of 256x256, a 0.75 wave) 115.7 against 97.9 us.
        static const Cand bf16c[] = {{CFG_BF16_256x192, 1.0}, {CFG_BF16_256x256, 1.0}, {CFG_BF16_256x128, 0.95},
                                     {CFG_BF16_128x128, 0.85}};
        // With only a few 32-deep stages per tile, a tile's time is mostly
        // its first-load latency and its epilogue, which a second resident
        // workgroup per CU hides: the 128x128 ring kernel (64 KiB of LDS,
        // two per CU) measured 1.12x faster than 256x128 (96 KiB, one per
        // CU) on 32 x 1024x1024x128 with FP32 output.
        static const Cand bf16_short_k[] = {{CFG_BF16_256x192, 0.7}, {CFG_BF16_256x256, 0.65}, {CFG_BF16_256x128, 0.75},
                                            {CFG_BF16_128x128, 1.0}};
        static const Cand f32c[] = {{CFG_F32_128x128, 1.0}, {CFG_F32_64x64, 0.8}};
        // FP8 ring kernels (256x192, 256x256, 128x128): the 256x256 one runs
        // single-rate stages (its registers do not hold stage pairs) and is
        // half as fast; two co-resident 128x128 workgroups per CU beat the
        // model's copy rate (measured: 4096x1536x4096 39.2 against 51.6 us
        // for 256x192, 4096^3 90.3 against 105.7 us for 256x256, while the
        // FFN's one tile per CU stays on 256x192, 58.8 against 67.6 us).
        static const Cand fp8c[] = {{CFG_BF16_256x192, 1.0}, {CFG_BF16_256x256, 0.5}, {CFG_BF16_128x128, 1.4}};
        const bool bf16 = p.op != GEMM_OP_SGEMM;
        const Cand *cands = is_fp8(p) ? fp8c : bf16 ? (p.K <= 8 * 32 ? bf16_short_k : bf16c) : f32c;
        const int nc = is_fp8(p) ? 3 : bf16 ? 4 : 2;
        double best = 0.0;
        for (int i = 0; i < nc; ++i) {
            if (!config_fits(p, cands[i].id)) continue;
            Plan trial = pl;
            trial.config = cands[i].id;
            bool ev = false;
            const int var = pick_variant(p, trial, &ev);
            // measured relative speed of the kernel variants
            const double veff = var == 1 ? 1.0 : (var == 2 || var == 3) ? 0.85 : 0.3;
            const double t = model_time(p, kConfigs[cands[i].id], cands[i].eff * veff);
            if (pl.config == CFG_NONE || t < best) {
                best = t;
                pl.config = cands[i].id;
            }
        }
        // An output with fewer tiles than CUs: K split over workgroups of
        // 128x128 tiles when the model gives it the shortest time
        // (page "Operator & Runtime" §5.2.4 splits the reduction dimension
        // to occupy the device).
        if (ws && bf16 && (epi_of(p) == EPI_NONE || epi_of(p) == EPI_AFFINE) &&
            p.batch * cdiv(p.M, 128) * cdiv(p.N, 128) < kNumCU) {
            Plan t = pl;
            t.config = CFG_BF16_128x128;
            bool ev = false;
            int var = pick_variant(p, t, &ev);
            if (b_trans(p) && var == 0 && pl.align_b < 16) var = 2;   // Bt rows realigned below
            if (a_trans(p) && var == 0) var = 2;                          // At rows realigned below
            for (int S = 2; S <= 8 && var >= 1; ++S) {
                if (!split_ok(p, S)) continue;
                // (the 128x128 entry of the candidate table above)
                const double base = is_fp8(p) ? 1.4 : p.K <= 8 * 32 ? 1.0 : 0.85;
                const double eff = base * (var == 1 ? 1.0 : 0.85);
                const double tm = model_time_split(p, kConfigs[CFG_BF16_128x128], S, eff);
                if (tm < best) {
                    best = tm;
                    pl.config = CFG_BF16_128x128;
                    pl.ksplit = S;
                }
            }
        }
    }
    if (const char *fk = std::getenv("GEMM_FORCE_KSPLIT")) {
        // diagnostic: force the K split of the 128x128 ring kernel (1 = none)
        const int S = std::atoi(fk);
        if (S >= 1 && pl.config == CFG_BF16_128x128 && (epi_of(p) == EPI_NONE || epi_of(p) == EPI_AFFINE)) {
            if (S > 1 && (!ws || !split_ok(p, S) || p.batch * cdiv(p.M, 128) * cdiv(p.N, 128) > kMaxCounters))
                return GEMM_ERR_UNSUPPORTED;
            pl.ksplit = S;
        }
    }
    fill_grid(p, pl, ws);
    if (pl.grid <= 0 || pl.grid > (int64_t)1 << 24) return GEMM_ERR_UNSUPPORTED;
    // (a forced split path that would need partial sums without a workspace)
    if (pl.config == CFG_DECODE_SPLIT && !ws && p.op == GEMM_OP_BF16_SWIGLU) return GEMM_ERR_UNSUPPORTED;
    pl.variant = pick_variant(p, pl, &pl.even);
    if (pl.variant < 0) return GEMM_ERR_UNSUPPORTED;   // forced split path without its preconditions
    // A large bf16 product whose A rows are not 16-byte aligned: multiply
    // from a copy of A with aligned rows when that lets the ring kernel copy
    // A 16 bytes per lane (the copy costs 2 x M x K x 2 bytes of traffic,
    // small next to the product from 2^30 multiply-adds on).
    // The fused epilogues and a transposed B exist only in the ring kernels,
    // so such a call whose rows no ring variant takes is realigned at any
    // size: Bt's rows first, then A's.
    if (ws && kConfigs[pl.config].family == GEMM_FAMILY_BF16_MFMA && b_trans(p) && !is_fp8(p) &&
        pl.align_b < 16) {
        pl.realign_b = true;
        pl.ldb2 = (p.K + 7) / 8 * 8;
        pl.align_b = 16;
        Problem q = p;
        q.ldb = pl.ldb2;
        q.sB = p.N * pl.ldb2;
        pl.variant = pick_variant(q, pl, &pl.even);
    }
    if (ws && kConfigs[pl.config].family == GEMM_FAMILY_BF16_MFMA && !is_fp8(p) &&
        (pl.align_a < 16 || (a_trans(p) && p.M % 8 != 0)) &&
        ((double)p.batch * p.M * p.N * p.K >= (double)(1 << 30) || (ring_only(p) && pl.variant == 0))) {
        Problem q = p;
        if (pl.realign_b) {
            q.ldb = pl.ldb2;
            q.sB = p.N * pl.ldb2;
        }
        q.lda = (a_cols(p) + 7) / 8 * 8;
        q.sA = a_rows(p) * q.lda;
        Plan t = pl;
        t.align_a = 16;
        t.realign_a = true;
        bool ev = false;
        const int v = pick_variant(q, t, &ev);
        if (v == 1 || v == 2) {
            pl.realign_a = true;
            pl.lda2 = q.lda;
            pl.align_a = 16;
            pl.variant = v;
            pl.even = ev;
        }
    }
    // fused epilogues and a transposed B exist in the ring kernels only (variants 1-3)
    if (ring_only(p) && tiled(pl.config) && pl.variant == 0) return GEMM_ERR_UNSUPPORTED;
    if (const char *fs = std::getenv("GEMM_FORCE_STREAMK")) {
        // diagnostic: the persistent stream-K schedule for the chosen tile
        if (*fs == '1') {
            if (!streamk_ok(p, pl, ws)) return GEMM_ERR_UNSUPPORTED;
            pl.streamk = true;
            pl.ksplit = 1;
            const int64_t units = p.batch * pl.tiles_m * pl.tiles_n * (p.K / 32);
            pl.grid = units < kNumCU ? units : kNumCU;
        }
    }
    return GEMM_OK;
}

size_t realign_bytes(const Problem &p, const Plan &pl)
{
    return pl.realign_a ? (size_t)p.batch * a_rows(p) * pl.lda2 * 2 : 0;
}
size_t realign_b_bytes(const Problem &p, const Plan &pl)
{
    return pl.realign_b ? (size_t)p.batch * p.N * pl.ldb2 * 2 : 0;
}

// The split small-M path with one workgroup per strip stores C directly
// (no partial sums, no counters).
bool decode_split_direct(const Problem &p, const Plan &pl)
{
    return pl.config == CFG_DECODE_SPLIT && pl.ks == 1 && p.op != GEMM_OP_BF16_SWIGLU;
}

// Two workgroups per strip (two K slices, or SwiGLU's gate and up with one
// slice each) whose outputs fit the counter region as exchange slots (one
// 32-bit word per output, zero between calls): the split small-M path pairs
// their partial sums by atomic exchange instead of counters and a
// partial-sum buffer (the same sums, in the same order).
bool decode_split_pair(const Problem &p, const Plan &pl)
{
    const bool two = p.op == GEMM_OP_BF16_SWIGLU ? pl.ks == 1 : pl.ks == 2;
    if (const char *e = std::getenv("GEMM_DECODE_PAIR"))    // diagnostic: 0 = counters and partial sums
        if (std::strcmp(e, "0") == 0) return false;
    return pl.config == CFG_DECODE_SPLIT && two && (uint64_t)p.batch * p.M * p.N * 4 <= kCounterBytes;
}

// Partial sums of the split small-M path: one slot of 16 x 128 FP32 per
// (batch entry, strip, K slice); of a K-split tiled call: ksplit FP32 tiles
// per output tile.  The arrival counters (one per strip or tile) are in the
// workspace's counter region.
size_t partial_bytes(const Problem &p, const Plan &pl)
{
    if (pl.config == CFG_DECODE_SPLIT)
        return decode_split_direct(p, pl) || decode_split_pair(p, pl)
                   ? 0
                   : (size_t)p.batch * pl.tiles_n * pl.ks * (p.op == GEMM_OP_BF16_SWIGLU ? 2 : 1) * 16 * 128 *
                         sizeof(float);
    const ConfigInfo &c = kConfigs[pl.config];
    if (pl.streamk) return (size_t)2 * pl.grid * c.tile_m * c.tile_n * 4;
    return pl.ksplit > 1 ? (size_t)p.batch * pl.tiles_m * pl.tiles_n * pl.ksplit * c.tile_m * c.tile_n * 4 : 0;
}

// Workspace layout (byte offsets from its start, each region 256-byte
// aligned): [0, kCounterBytes) arrival counters, then the partial sums,
// then the realigned copy of A, then that of Bt.  A plan that needs none of
// them and no counters (or exchange slots) needs no workspace (0 bytes).
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
struct WsLayout {
    size_t part = 0, rows_a = 0, rows_b = 0, total = 0;
};
int64_t counters_used(const Problem &p, const Plan &pl);

WsLayout ws_layout(const Problem &p, const Plan &pl)
{
    WsLayout L;
    const size_t pb = partial_bytes(p, pl), ab = realign_bytes(p, pl), bb = realign_b_bytes(p, pl);
    if (pb == 0 && ab == 0 && bb == 0 && counters_used(p, pl) == 0) return L;
    L.part = kCounterBytes;
    L.rows_a = L.part + round256(pb);
    L.rows_b = L.rows_a + round256(ab);
    L.total = L.rows_b + round256(bb);
    return L;
}

void fill_public_plan(const Problem &p, const Plan &pl, gemm_plan *out)
{
    if (!out) return;
    std::memset(out, 0, sizeof *out);
    const ConfigInfo &c = kConfigs[pl.config];
    out->family = c.family;
    out->config_id = pl.config;
    out->tile_m = c.tile_m;
    out->tile_n = c.tile_n;
    out->tile_k = c.tile_k;
    out->threads = c.threads;
    out->vec_a = pl.align_a;
    out->vec_b = pl.align_b;
    out->even = pl.even ? 1 : 0;
    out->variant = pl.variant;
    out->grid = pl.grid * (c.family == GEMM_FAMILY_DECODE ? p.batch : 1);
    out->lds_bytes = c.lds_bytes;
    if (c.family == GEMM_FAMILY_BF16_MFMA && pl.variant >= 1 && pl.variant <= 3) {
        // LDS-ring kernels: 8 waves, 4 slots of a 32-deep K slab of A and B
        out->threads = 512;
        out->tile_k = 32;
        out->lds_bytes = 4 * (c.tile_m * 32 + 32 * c.tile_n) * 2;
    }
    out->model_bytes = pl.model_bytes;
    std::snprintf(out->name, sizeof out->name, "%s", c.name);
    out->workspace_bytes = (int64_t)ws_layout(p, pl).total;
    out->ksplit = pl.ksplit;
    out->streamk = pl.streamk ? 1 : 0;
}

// ------------------------------------------------------------ device check
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 gfx950, -1 another architecture (no usable device)

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_ERR_NO_DEVICE;
    if (dev >= 64) return GEMM_OK;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_NO_DEVICE;
        g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_dev_state[dev] == 1 ? GEMM_OK : GEMM_ERR_NO_DEVICE;
}

bool log_enabled()
{
    static int v = -1;
    if (v < 0) {
        const char *e = std::getenv("GEMM_LOG");
        v = (e && *e && *e != '0') ? 1 : 0;
    }
    return v == 1;
}

// Arrival counters, or exchange slots, a plan uses (32-bit words at the
// start of the workspace, zero between calls).
int64_t counters_used(const Problem &p, const Plan &pl)
{
    if (pl.config == CFG_DECODE_SPLIT)
        return decode_split_direct(p, pl) ? 0 : decode_split_pair(p, pl) ? p.batch * p.M * p.N : p.batch * pl.tiles_n;
    if (pl.ksplit > 1 || pl.streamk) return p.batch * pl.tiles_m * pl.tiles_n;
    return 0;
}

// The plan a call runs: with the workspace paths when the caller passes a
// workspace (which must then hold what the plan needs), else without.
int plan_for_call(const Problem &p, const void *ws, size_t ws_bytes, Plan &pl, WsLayout &L)
{
    int st = select_plan(p, pl, ws != nullptr);
    if (st != GEMM_OK) return st;
    L = ws_layout(p, pl);
    if (ws != nullptr && L.total > ws_bytes) return GEMM_ERR_WORKSPACE;
    if (ws != nullptr && ((uintptr_t)ws % 256) != 0) return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

// Validate, plan and enqueue one call.  `ws`: the caller's workspace (NULL:
// none); no memory is allocated, freed, copied or waited for here.
int run(const Problem &p, void *stream, void *ws = nullptr, size_t ws_bytes = 0)
{
    int st = validate(p);
    if (st != GEMM_OK) return st;
    Plan pl;
    WsLayout L;
    st = plan_for_call(p, ws, ws_bytes, pl, L);
    if (st != GEMM_OK) return st;
    if (pl.config == CFG_NONE) return GEMM_OK;
    st = check_device();
    if (st != GEMM_OK) return st;
    char *wsb = (char *)ws;
    unsigned *counters = (unsigned *)wsb;
    if (log_enabled())
        std::fprintf(stderr, "[gemm05] op=%d batch=%lld M=%lld N=%lld K=%lld -> %s variant=%d grid=%lld align=(%d,%d,%d)\n",
                     p.op, (long long)p.batch, (long long)p.M, (long long)p.N, (long long)p.K,
                     kConfigs[pl.config].name, pl.variant, (long long)pl.grid, pl.align_a, pl.align_b,
                     pl.align_c);
    GemmArgs a;
    a.A = (const void *)p.a;
    a.B = (const void *)p.b;
    a.C = (void *)p.c;
    a.M = p.M;
    a.N = p.N;
    a.K = p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.sA = p.sA;
    a.sB = p.sB;
    a.sC = p.sC;
    a.batch = p.batch;
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.group_m = pl.group_m;
    a.align_a = pl.align_a;
    a.align_b = pl.align_b;
    a.align_c = pl.align_c;
    a.out_f32 = elem_c(p) == 4 ? 1 : 0;
    a.ksplit = 1;
    a.kt_per = 0;
    a.b_trans = b_trans(p) ? 1 : 0;
    a.fp8 = is_fp8(p) ? 1 : 0;
    a.scale_a = (const float *)p.scale_a;
    a.scale_b = (const float *)p.scale_b;
    a.s_scale_a = scale_stride_a(p);
    a.s_scale_b = scale_stride_b(p);
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.bias = (const uint16_t *)p.bias;
    a.align_bias = row_alignment(p.bias, 0, 0, 1, 2);
    a.affine = is_affine(p) ? 1 : 0;
    a.a_trans = a_trans(p) ? 1 : 0;
    a.epi = epi_of(p);
    a.c_e4m3 = p.c_type == GEMM_OUT_E4M3 ? 1 : 0;
    a.c_amax = p.out_amax;
    if (pl.realign_b) {
        uint16_t *B2 = (uint16_t *)(wsb + L.rows_b);
        const hipError_t e = launch_realign_rows((const uint16_t *)p.b, p.ldb, p.sB, p.batch, p.N, p.K,
                                                 row_alignment(p.b, p.ldb, p.sB, p.batch, 2), B2, pl.ldb2,
                                                 (hipStream_t)stream);
        if (e != hipSuccess) return GEMM_ERR_LAUNCH;
        a.B = B2;
        a.ldb = pl.ldb2;
        a.sB = p.N * pl.ldb2;
        a.align_b = 16;
    }
    a.ws_part = nullptr;
    a.ws_cnt = nullptr;
    if (pl.ksplit > 1 || pl.streamk) {
        a.ksplit = pl.ksplit;
        a.kt_per = pl.ksplit > 1 ? split_kt_per(p, pl.ksplit) : 0;
        a.ws_part = (float *)(wsb + L.part);
        a.ws_cnt = counters;
    }
    if (pl.streamk) {
        const hipError_t e = launch_streamk(pl.config, a, pl.variant, pl.grid, (hipStream_t)stream);
        return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    if (pl.realign_a) {
        uint16_t *A2 = (uint16_t *)(wsb + L.rows_a);
        const hipError_t e = launch_realign_rows((const uint16_t *)p.a, p.lda, p.sA, p.batch, a_rows(p), a_cols(p),
                                                 row_alignment(p.a, p.lda, p.sA, p.batch, 2), A2, pl.lda2,
                                                 (hipStream_t)stream);
        if (e != hipSuccess) return GEMM_ERR_LAUNCH;
        a.A = A2;
        a.lda = pl.lda2;
        a.sA = a_rows(p) * pl.lda2;
        a.align_a = 16;
    }
    if (pl.config == CFG_DECODE_SPLIT) {
        const bool pair = decode_split_pair(p, pl);
        const hipError_t e = launch_decode_split(a, pair ? nullptr : (float *)(wsb + L.part), counters, pl.ks,
                                                 pair ? counters : nullptr, (hipStream_t)stream);
        return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    const hipError_t e =
        pl.config == CFG_ZERO ? (is_affine(p) ? launch_affine_no_product(a, pl.grid, (hipStream_t)stream)
                                                             : launch_config(pl.config, false, a, 0, pl.grid, (hipStream_t)stream))
        : epi_of(p) == EPI_NONE || !tiled(pl.config)
            ? launch_config(pl.config, p.op == GEMM_OP_SGEMM, a, pl.variant, pl.grid, (hipStream_t)stream)
                                : launch_fused(pl.config, epi_of(p), a, pl.variant, pl.grid, (hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace
}  // namespace g5

using g5::Problem;

extern "C" {

int gemm_sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
               float *C, int64_t ldc, void *stream)
{
    const Problem p{GEMM_OP_SGEMM, 1, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc, 0, 0, 0,
                    GEMM_OUT_F32};
    return g5::run(p, stream);
}

int gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
              void *C, int64_t ldc, int c_type, void *stream)
{
    const Problem p{GEMM_OP_BF16, 1, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc, 0, 0, 0,
                    c_type};
    return g5::run(p, stream);
}

int gemm_bf16_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                      int64_t strideA, const uint16_t *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                      int64_t strideC, int c_type, void *stream)
{
    const Problem p{GEMM_OP_BF16, batch, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc,
                    strideA, strideB, strideC, c_type};
    return g5::run(p, stream);
}

int gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *Bt, int64_t ldbt,
                 void *C, int64_t ldc, int c_type, void *stream)
{
    const Problem p{GEMM_OP_BF16_NT, 1, M, N, K, (uint64_t)A, (uint64_t)Bt, (uint64_t)C, lda, ldbt, ldc, 0, 0, 0,
                    c_type};
    return g5::run(p, stream);
}

int gemm_bf16_nt_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                         int64_t strideA, const uint16_t *Bt, int64_t ldbt, int64_t strideBt, void *C, int64_t ldc,
                         int64_t strideC, int c_type, void *stream)
{
    const Problem p{GEMM_OP_BF16_NT, batch, M, N, K, (uint64_t)A, (uint64_t)Bt, (uint64_t)C, lda, ldbt, ldc,
                    strideA, strideBt, strideC, c_type};
    return g5::run(p, stream);
}

int gemm_fp8_nt(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const float *scale_a,
                const uint8_t *Bt, int64_t ldbt, const float *scale_b, void *C, int64_t ldc, int c_type, void *stream)
{
    Problem p{GEMM_OP_FP8_NT, 1, M, N, K, (uint64_t)A, (uint64_t)Bt, (uint64_t)C, lda, ldbt, ldc, 0, 0, 0, c_type};
    p.scale_a = (uint64_t)scale_a;
    p.scale_b = (uint64_t)scale_b;
    return g5::run(p, stream);
}

int gemm_fp8_nt_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                        int64_t strideA, const float *scale_a, const uint8_t *Bt, int64_t ldbt, int64_t strideBt,
                        const float *scale_b, void *C, int64_t ldc, int64_t strideC, int c_type, void *stream)
{
    Problem p{GEMM_OP_FP8_NT, batch, M, N, K, (uint64_t)A, (uint64_t)Bt, (uint64_t)C, lda, ldbt, ldc, strideA,
              strideBt, strideC, c_type};
    p.scale_a = (uint64_t)scale_a;
    p.scale_b = (uint64_t)scale_b;
    return g5::run(p, stream);
}

int gemm_fp8_nt_affine(int64_t batch, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                       int64_t strideA, const float *scale_a, const uint8_t *Bt, int64_t ldbt, int64_t strideBt,
                       const float *scale_b, float alpha, const uint16_t *bias, float beta, void *C, int64_t ldc,
                       int64_t strideC, int c_type, void *stream)
{
    Problem p{GEMM_OP_FP8_NT_AFFINE, batch, M, N, K, (uint64_t)A, (uint64_t)Bt, (uint64_t)C, lda, ldbt, ldc, strideA,
              strideBt, strideC, c_type};
    p.scale_a = (uint64_t)scale_a;
    p.scale_b = (uint64_t)scale_b;
    p.alpha = alpha;
    p.beta = beta;
    p.bias = (uint64_t)bias;
    return g5::run(p, stream);
}

int gemm_fp8_nt_quant_a(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx, float *scale_x,
                        const uint8_t *Bt, int64_t ldbt, const float *scale_b, void *C, int64_t ldc, int c_type,
                        void *workspace, uint64_t workspace_bytes, void *stream)
{
    using g5::Range;
    if (M < 0 || N < 0 || K < 0 || M > 0x7fffffff) return GEMM_ERR_INVALID_ARG;
    if (c_type != GEMM_OUT_BF16 && c_type != GEMM_OUT_F32) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return GEMM_OK;
    if (!X || !Bt || !C || !scale_x || ldx < K || ldbt < K || ldc < N) return GEMM_ERR_INVALID_ARG;
    if (((uint64_t)scale_x % 4) || ((uint64_t)scale_b % 4) || ((uint64_t)X % 2)) return GEMM_ERR_INVALID_ARG;
    const int ec = c_type == GEMM_OUT_F32 ? 4 : 2;
    const Range rx = g5::extent((uint64_t)X, 1, M, K > 0 ? K : 1, ldx, 0, 2);
    const Range rb = g5::extent((uint64_t)Bt, 1, N, K > 0 ? K : 1, ldbt, 0, 1);
    const Range rc = g5::extent((uint64_t)C, 1, M, N, ldc, 0, ec);
    const Range rs{(__int128)(uint64_t)scale_x, (__int128)(uint64_t)scale_x + 4 * (__int128)M};
    // the row maxima go after the workspace's arrival counters, which other
    // calls sharing the workspace expect to find at zero
    const Range rw{(__int128)(uint64_t)workspace + (__int128)g5::kCounterBytes,
                   (__int128)(uint64_t)workspace + (__int128)g5::kCounterBytes + 4 * (__int128)M};
    if (g5::overlap(rc, rx) || g5::overlap(rc, rb) || g5::overlap(rc, rs) || g5::overlap(rs, rx) || g5::overlap(rs, rb))
        return GEMM_ERR_INVALID_ARG;
    if (scale_b && g5::overlap(rc, Range{(__int128)(uint64_t)scale_b, (__int128)(uint64_t)scale_b + 4 * (__int128)N}))
        return GEMM_ERR_INVALID_ARG;
    // whole 64-deep stages, 16-byte rows of X and Bt, 32-bit buffer offsets
    if (K == 0 || K % 64 != 0 || g5::row_alignment((uint64_t)X, ldx, 0, 1, 2) < 16 ||
        g5::row_alignment((uint64_t)Bt, ldbt, 0, 1, 1) < 16 || rx.hi - rx.lo >= ((__int128)1 << 31) ||
        rb.hi - rb.lo >= ((__int128)1 << 31))
        return GEMM_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < g5::kCounterBytes + 4 * (uint64_t)M) return GEMM_ERR_WORKSPACE;
    if (((uint64_t)workspace % 256) || g5::overlap(rw, rx) || g5::overlap(rw, rb) || g5::overlap(rw, rc) ||
        g5::overlap(rw, rs))
        return GEMM_ERR_INVALID_ARG;
    const int st = g5::check_device();
    if (st != GEMM_OK) return st;
    g5::GemmArgs a{};
    a.A = X;
    a.B = Bt;
    a.C = C;
    a.M = M;
    a.N = N;
    a.K = K;
    a.lda = ldx;
    a.ldb = ldbt;
    a.ldc = ldc;
    a.batch = 1;
    // Tile width: 256 columns convert each A element half as often as 128
    // (the conversion, not the MFMAs, bounds the loop), at one workgroup
    // per CU instead of two.  Per-CU costs measured with K = 4096 (both
    // scale with K alike): one 128x256 tile 72 us; two 128x128 tiles
    // sharing a CU 87 us, one alone 50 us.  The width with the smaller
    // estimate for the busiest CU is taken (e.g. 4096x1536: 256, one tile
    // per CU on 192 CUs; 1024x12288: 128, three tiles per CU against two
    // rounds of the wider ones).  GEMM_QA_TILE_N=128|256 forces one
    // (diagnostic).
    const int64_t tm = (M + 127) / 128;
    const int64_t k256 = (tm * ((N + 255) / 256) + g5::kNumCU - 1) / g5::kNumCU;
    const int64_t k128 = (tm * ((N + 127) / 128) + g5::kNumCU - 1) / g5::kNumCU;
    int tile_n = 72.0 * k256 < 87.0 * (k128 / 2) + 50.0 * (k128 % 2) ? 256 : 128;
    if (const char *f = std::getenv("GEMM_QA_TILE_N")) {
        if (std::strcmp(f, "128") == 0) tile_n = 128;
        else if (std::strcmp(f, "256") == 0) tile_n = 256;
    }
    a.tiles_m = tm;
    a.tiles_n = (N + tile_n - 1) / tile_n;
    a.group_m = a.tiles_m <= 8 ? a.tiles_m : 8;
    a.align_a = 16;
    a.align_b = 16;
    a.align_c = g5::row_alignment((uint64_t)C, ldc, 0, 1, ec);
    a.out_f32 = ec == 4 ? 1 : 0;
    a.ksplit = 1;
    a.b_trans = 1;
    a.fp8 = 1;
    a.scale_a = scale_x;
    a.scale_b = scale_b;
    a.alpha = 1.0f;
    const hipError_t e = g5::launch_fp8_quant_a(a, (float *)((char *)workspace + g5::kCounterBytes), tile_n,
                                                a.tiles_m * a.tiles_n, (hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_fp8_quantize_rows(int64_t rows, int64_t cols, const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq,
                           float *scale, void *stream)
{
    if (rows < 0 || cols < 0 || rows > 0x7fffffff) return GEMM_ERR_INVALID_ARG;
    if (rows == 0) return GEMM_OK;
    if (!scale || ((uint64_t)scale % 4)) return GEMM_ERR_INVALID_ARG;
    if (cols > 0 && (!X || !Q || ldx < cols || ldq < cols)) return GEMM_ERR_INVALID_ARG;
    const g5::Range rs{(__int128)(uint64_t)scale, (__int128)(uint64_t)scale + 4 * (__int128)rows};
    if (cols > 0) {
        const g5::Range rx = g5::extent((uint64_t)X, 1, rows, cols, ldx, 0, 2);
        const g5::Range rq = g5::extent((uint64_t)Q, 1, rows, cols, ldq, 0, 1);
        if (g5::overlap(rx, rq) || g5::overlap(rs, rx) || g5::overlap(rs, rq)) return GEMM_ERR_INVALID_ARG;
    }
    int st = g5::check_device();
    if (st != GEMM_OK) return st;
    const hipError_t e = g5::launch_quant_rows_e4m3(X, ldx, rows, cols, g5::row_alignment((uint64_t)X, ldx, 0, 1, 2),
                                                    Q, ldq, g5::row_alignment((uint64_t)Q, ldq, 0, 1, 1), scale,
                                                    (hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_act_chain(int step, int64_t M, int64_t N, const uint16_t *in0, int64_t ld0, const uint16_t *in1,
                   int64_t ld1, void *out, int64_t ldo, float amax, void *stream)
{
    if (step < GEMM_ACT_SILU || step > GEMM_ACT_SWIGLU_E4M3 || M < 0 || N < 0) return GEMM_ERR_INVALID_ARG;
    const bool two = step == GEMM_ACT_MUL || step == GEMM_ACT_SWIGLU || step == GEMM_ACT_SWIGLU_E4M3;
    const bool codes = step == GEMM_ACT_QUANT || step == GEMM_ACT_SWIGLU_E4M3;
    if (codes && !(std::isfinite(amax) && amax > 0.0f)) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return GEMM_OK;
    const int eo = codes ? 1 : 2;
    if (!in0 || !out || (two && !in1) || ld0 < N || ldo < N || (two && ld1 < N)) return GEMM_ERR_INVALID_ARG;
    if (((uint64_t)in0 % 2) || (two && ((uint64_t)in1 % 2)) || ((uint64_t)out % eo)) return GEMM_ERR_INVALID_ARG;
    const g5::Range r0 = g5::extent((uint64_t)in0, 1, M, N, ld0, 0, 2);
    const g5::Range ro = g5::extent((uint64_t)out, 1, M, N, ldo, 0, eo);
    if (r0.hi > ((__int128)1 << 63) || ro.hi > ((__int128)1 << 63) || g5::overlap(r0, ro)) return GEMM_ERR_INVALID_ARG;
    if (two) {
        const g5::Range r1 = g5::extent((uint64_t)in1, 1, M, N, ld1, 0, 2);
        if (r1.hi > ((__int128)1 << 63) || g5::overlap(r1, ro)) return GEMM_ERR_INVALID_ARG;
    }
    int st = g5::check_device();
    if (st != GEMM_OK) return st;
    // 16-byte chunks when every row holds whole chunks at aligned starts
    const bool vec = N % 8 == 0 && (__int128)M * (N / 8) < ((__int128)1 << 31) &&
                     g5::row_alignment((uint64_t)in0, ld0, 0, 1, 2) >= 16 &&
                     (!two || g5::row_alignment((uint64_t)in1, ld1, 0, 1, 2) >= 16) &&
                     g5::row_alignment((uint64_t)out, ldo, 0, 1, eo) >= 8 * eo;
    const bool contig = ld0 == N && ldo == N && (!two || ld1 == N);
    const g5::ActArgs a{in0, two ? in1 : nullptr, out, M, N, ld0, two ? ld1 : N, ldo, codes ? amax : 1.0f};
    const hipError_t e = g5::launch_act_chain(step, a, vec, contig, (hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_fp8_quantize_cols(int64_t K, int64_t N, const uint16_t *W, int64_t ldw, uint8_t *Qt, int64_t ldq,
                           float *scale, void *stream)
{
    if (K < 0 || N < 0 || N > ((int64_t)1 << 36)) return GEMM_ERR_INVALID_ARG;
    if (N == 0) return GEMM_OK;
    if (!scale || ((uint64_t)scale % 4)) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && (!W || !Qt || ((uint64_t)W % 2) || ldw < N || ldq < K)) return GEMM_ERR_INVALID_ARG;
    const g5::Range rs{(__int128)(uint64_t)scale, (__int128)(uint64_t)scale + 4 * (__int128)N};
    if (K > 0) {
        const g5::Range rw = g5::extent((uint64_t)W, 1, K, N, ldw, 0, 2);
        const g5::Range rq = g5::extent((uint64_t)Qt, 1, N, K, ldq, 0, 1);
        if (g5::overlap(rw, rq) || g5::overlap(rs, rw) || g5::overlap(rs, rq)) return GEMM_ERR_INVALID_ARG;
    }
    int st = g5::check_device();
    if (st != GEMM_OK) return st;
    const hipError_t e = g5::launch_quant_cols_e4m3(W, ldw, K, N, g5::row_alignment((uint64_t)W, ldw, 0, 1, 2), Qt, ldq,
                                                    g5::row_alignment((uint64_t)Qt, ldq, 0, 1, 1), scale,
                                                    (hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_bf16_silu(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                   uint16_t *C, int64_t ldc, void *stream)
{
    const Problem p{GEMM_OP_BF16_SILU, 1, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc, 0, 0, 0,
                    GEMM_OUT_BF16};
    return g5::run(p, stream);
}

int gemm_bf16_swiglu(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx, const uint16_t *Wgu,
                     int64_t ldw, uint16_t *Z, int64_t ldz, void *stream)
{
    const Problem p{GEMM_OP_BF16_SWIGLU, 1, M, N, K, (uint64_t)X, (uint64_t)Wgu, (uint64_t)Z, ldx, ldw, ldz, 0, 0,
                    0, GEMM_OUT_BF16};
    return g5::run(p, stream);
}

int gemm_bf16_swiglu_e4m3(int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx, const uint16_t *Wgu,
                          int64_t ldw, uint8_t *Zq, int64_t ldz, float amax, void *stream)
{
    Problem p{GEMM_OP_BF16_SWIGLU, 1, M, N, K, (uint64_t)X, (uint64_t)Wgu, (uint64_t)Zq, ldx, ldw, ldz, 0, 0,
              0, GEMM_OUT_E4M3};
    p.out_amax = amax;
    return g5::run(p, stream);
}

int gemm_bf16_silu_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                           int64_t strideA, const uint16_t *B, int64_t ldb, int64_t strideB, uint16_t *C, int64_t ldc,
                           int64_t strideC, void *stream)
{
    const Problem p{GEMM_OP_BF16_SILU, batch, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc,
                    strideA, strideB, strideC, GEMM_OUT_BF16};
    return g5::run(p, stream);
}

int gemm_bf16_swiglu_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                             int64_t strideX, const uint16_t *Wgu, int64_t ldw, int64_t strideW, uint16_t *Z,
                             int64_t ldz, int64_t strideZ, void *stream)
{
    const Problem p{GEMM_OP_BF16_SWIGLU, batch, M, N, K, (uint64_t)X, (uint64_t)Wgu, (uint64_t)Z, ldx, ldw, ldz,
                    strideX, strideW, strideZ, GEMM_OUT_BF16};
    return g5::run(p, stream);
}

int gemm_bf16_swiglu_e4m3_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *X, int64_t ldx,
                                  int64_t strideX, const uint16_t *Wgu, int64_t ldw, int64_t strideW, uint8_t *Zq,
                                  int64_t ldz, int64_t strideZ, float amax, void *stream)
{
    Problem p{GEMM_OP_BF16_SWIGLU, batch, M, N, K, (uint64_t)X, (uint64_t)Wgu, (uint64_t)Zq, ldx, ldw, ldz,
              strideX, strideW, strideZ, GEMM_OUT_E4M3};
    p.out_amax = amax;
    return g5::run(p, stream);
}

int gemm_bf16_tn(int64_t M, int64_t N, int64_t K, const uint16_t *At, int64_t ldat, const uint16_t *B, int64_t ldb,
                 void *C, int64_t ldc, int c_type, void *stream)
{
    const Problem p{GEMM_OP_BF16_TN, 1, M, N, K, (uint64_t)At, (uint64_t)B, (uint64_t)C, ldat, ldb, ldc, 0, 0, 0,
                    c_type};
    return g5::run(p, stream);
}

int gemm_bf16_tn_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *At, int64_t ldat,
                         int64_t strideAt, const uint16_t *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                         int64_t strideC, int c_type, void *stream)
{
    const Problem p{GEMM_OP_BF16_TN, batch, M, N, K, (uint64_t)At, (uint64_t)B, (uint64_t)C, ldat, ldb, ldc,
                    strideAt, strideB, strideC, c_type};
    return g5::run(p, stream);
}

int gemm_bf16_affine(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, int64_t strideA,
                     const uint16_t *B, int64_t ldb, int64_t strideB, float alpha, const uint16_t *bias, float beta,
                     void *C, int64_t ldc, int64_t strideC, int c_type, void *stream)
{
    Problem p{GEMM_OP_BF16_AFFINE, batch, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc,
              strideA, strideB, strideC, c_type};
    p.alpha = alpha;
    p.beta = beta;
    p.bias = (uint64_t)bias;
    return g5::run(p, stream);
}

int gemm_bf16_tn_affine(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *At, int64_t ldat,
                        int64_t strideAt, const uint16_t *B, int64_t ldb, int64_t strideB, float alpha,
                        const uint16_t *bias, float beta, void *C, int64_t ldc, int64_t strideC, int c_type,
                        void *stream)
{
    Problem p{GEMM_OP_BF16_TN_AFFINE, batch, M, N, K, (uint64_t)At, (uint64_t)B, (uint64_t)C, ldat, ldb, ldc,
              strideAt, strideB, strideC, c_type};
    p.alpha = alpha;
    p.beta = beta;
    p.bias = (uint64_t)bias;
    return g5::run(p, stream);
}

int gemm_bf16_nt_affine(int64_t batch, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                        int64_t strideA, const uint16_t *Bt, int64_t ldbt, int64_t strideBt, float alpha,
                        const uint16_t *bias, float beta, void *C, int64_t ldc, int64_t strideC, int c_type,
                        void *stream)
{
    Problem p{GEMM_OP_BF16_NT_AFFINE, batch, M, N, K, (uint64_t)A, (uint64_t)Bt, (uint64_t)C, lda, ldbt, ldc,
              strideA, strideBt, strideC, c_type};
    p.alpha = alpha;
    p.beta = beta;
    p.bias = (uint64_t)bias;
    return g5::run(p, stream);
}

const char *gemm_status_string(int status)
{
    switch (status) {
    case GEMM_OK: return "GEMM_OK: success";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG: invalid size, stride, pointer, output type or overlap";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: no compiled kernel configuration can run this call";
    case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: kernel launch failed";
    case GEMM_ERR_NO_DEVICE: return "GEMM_ERR_NO_DEVICE: no usable HIP device is current (none, or not gfx950)";
    case GEMM_ERR_WORKSPACE:
        return "GEMM_ERR_WORKSPACE: the workspace passed is smaller than the call needs (gemm_workspace_size)";
    default: return "unknown gemm status";
    }
}

static int plan_query_impl(int with_workspace, int op, int64_t batch, int64_t M, int64_t N, int64_t K,
                           uint64_t a_addr, int64_t lda, int64_t strideA, uint64_t b_addr, int64_t ldb,
                           int64_t strideB, uint64_t c_addr, int64_t ldc, int64_t strideC, int c_type,
                           gemm_plan *out)
{
    Problem p{op, batch, M, N, K, a_addr, b_addr, c_addr, lda, ldb, ldc, strideA, strideB, strideC,
              g5::op_c_type(op, c_type)};
    if (p.c_type == GEMM_OUT_E4M3) p.out_amax = 1.0f;   // (the range does not change the plan)
    int st = g5::validate(p);
    if (st != GEMM_OK) return st;
    g5::Plan pl;
    st = g5::select_plan(p, pl, with_workspace != 0);
    if (st != GEMM_OK) return st;
    g5::fill_public_plan(p, pl, out);
    return GEMM_OK;
}

int gemm_plan_query(int op, int64_t batch, int64_t M, int64_t N, int64_t K, uint64_t a_addr, int64_t lda,
                    int64_t strideA, uint64_t b_addr, int64_t ldb, int64_t strideB, uint64_t c_addr, int64_t ldc,
                    int64_t strideC, int c_type, gemm_plan *out)
{
    return plan_query_impl(1, op, batch, M, N, K, a_addr, lda, strideA, b_addr, ldb, strideB, c_addr, ldc, strideC,
                           c_type, out);
}

int gemm_plan_query_ex(int with_workspace, int op, int64_t batch, int64_t M, int64_t N, int64_t K, uint64_t a_addr,
                       int64_t lda, int64_t strideA, uint64_t b_addr, int64_t ldb, int64_t strideB, uint64_t c_addr,
                       int64_t ldc, int64_t strideC, int c_type, gemm_plan *out)
{
    return plan_query_impl(with_workspace, op, batch, M, N, K, a_addr, lda, strideA, b_addr, ldb, strideB, c_addr,
                           ldc, strideC, c_type, out);
}

int gemm_workspace_size(int op, int64_t batch, int64_t M, int64_t N, int64_t K, uint64_t a_addr, int64_t lda,
                        int64_t strideA, uint64_t b_addr, int64_t ldb, int64_t strideB, uint64_t c_addr, int64_t ldc,
                        int64_t strideC, int c_type, uint64_t *bytes)
{
    gemm_plan pl;
    const int st = plan_query_impl(1, op, batch, M, N, K, a_addr, lda, strideA, b_addr, ldb, strideB, c_addr, ldc,
                                   strideC, c_type, &pl);
    if (bytes) *bytes = st == GEMM_OK ? (uint64_t)pl.workspace_bytes : 0;
    return st;
}

static g5::Problem run_problem(int op, int64_t batch, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                               int64_t strideA, const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                               int64_t strideC, int c_type, float alpha, const uint16_t *bias, float beta,
                               const float *scale_a, const float *scale_b)
{
    Problem p{op, batch, M, N, K, (uint64_t)A, (uint64_t)B, (uint64_t)C, lda, ldb, ldc, strideA, strideB, strideC,
              g5::op_c_type(op, c_type)};
    if (p.c_type == GEMM_OUT_E4M3) p.out_amax = alpha;   // SwiGLU's fixed range
    if (op == GEMM_OP_FP8_NT || op == GEMM_OP_FP8_NT_AFFINE) {
        p.scale_a = (uint64_t)scale_a;
        p.scale_b = (uint64_t)scale_b;
    }
    if (op == GEMM_OP_BF16_AFFINE || op == GEMM_OP_BF16_NT_AFFINE || op == GEMM_OP_BF16_TN_AFFINE ||
        op == GEMM_OP_FP8_NT_AFFINE) {
        p.alpha = alpha;
        p.beta = beta;
        p.bias = (uint64_t)bias;
    }
    return p;
}

int gemm_run(int op, int64_t batch, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
             const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc, int64_t strideC, int c_type,
             float alpha, const uint16_t *bias, float beta, const float *scale_a, const float *scale_b,
             void *workspace, uint64_t workspace_bytes, void *stream)
{
    if (op < GEMM_OP_SGEMM || op > GEMM_OP_FP8_NT_AFFINE) return GEMM_ERR_INVALID_ARG;
    if (op == GEMM_OP_SGEMM && batch != 1) return GEMM_ERR_INVALID_ARG;
    const Problem p = run_problem(op, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, c_type, alpha,
                                  bias, beta, scale_a, scale_b);
    return g5::run(p, stream, workspace, (size_t)workspace_bytes);
}

int gemm_run_noalloc(int op, int64_t batch, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     int64_t strideA, const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                     int64_t strideC, int c_type, float alpha, const uint16_t *bias, float beta,
                     const float *scale_a, const float *scale_b, void *stream)
{
    if (op < GEMM_OP_SGEMM || op > GEMM_OP_FP8_NT_AFFINE) return GEMM_ERR_INVALID_ARG;
    if (op == GEMM_OP_SGEMM && batch != 1) return GEMM_ERR_INVALID_ARG;
    const Problem p = run_problem(op, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, c_type, alpha,
                                  bias, beta, scale_a, scale_b);
    int st = g5::validate(p);
    if (st != GEMM_OK) return st;
    g5::Plan pl;
    st = g5::select_plan(p, pl, true);
    if (st != GEMM_OK) return st;
    if (pl.config == g5::CFG_NONE) return GEMM_OK;
    if (g5::ws_layout(p, pl).total > g5::kScratchBytes) return GEMM_ERR_WORKSPACE;
    st = g5::check_device();
    if (st != GEMM_OK) return st;
    void *scratch = nullptr;
    if (g5::noalloc_scratch(&scratch) != hipSuccess) return GEMM_ERR_LAUNCH;
    // The scratch keeps the last call's contents: the arrival counters this
    // call uses are cleared first (every call leaves them zero, but a call
    // that overlapped another on this GPU may not have).
    if (g5::launch_clear_counters(scratch, g5::counters_used(p, pl), (hipStream_t)stream) != hipSuccess)
        return GEMM_ERR_LAUNCH;
    return g5::run(p, stream, scratch, g5::kScratchBytes);
}

int64_t gemm_model_local_bytes(int64_t m, int64_t n, int64_t k, int64_t elem_bytes)
{
    return elem_bytes * m * k + elem_bytes * k * n + 4 * m * n;
}

double gemm_model_traffic_bytes(int64_t M, int64_t N, int64_t K, int64_t m, int64_t n, int64_t elem_bytes)
{
    if (m <= 0 || n <= 0) return 0.0;
    const double e = (double)elem_bytes;
    return e * M * K * (double)((N + n - 1) / n) + e * K * N * (double)((M + m - 1) / m) + e * M * N;
}

void gemm_model_quant_traffic(int64_t M, int64_t N, int64_t K, int64_t m, int64_t n, int64_t in_bytes,
                              int64_t q_bytes, int64_t w_bytes, int64_t out_bytes, double *separate, double *fused)
{
    double sep = 0.0, fus = 0.0;
    if (m > 0 && n > 0 && M >= 0 && N >= 0 && K >= 0) {
        const double in = (double)in_bytes * M * K, q = (double)q_bytes * M * K;
        const double col_blocks = (double)((N + n - 1) / n), row_blocks = (double)((M + m - 1) / m);
        const double common = row_blocks * w_bytes * (double)K * N + (double)out_bytes * M * N;
        sep = in + q + col_blocks * q + common;     // read once, write the codes, each column block reads them
        fus = in + col_blocks * in + common;        // read once for the factors, each column block re-reads it
    }
    if (separate) *separate = sep;
    if (fused) *fused = fus;
}

double gemm_model_act_chain_bytes(int step, int64_t M, int64_t N)
{
    // bytes per element: the inputs read plus the output written
    static const int kPerElem[5] = {2 + 2, 2 + 2 + 2, 2 + 2 + 2, 2 + 1, 2 + 2 + 1};
    if (step < GEMM_ACT_SILU || step > GEMM_ACT_SWIGLU_E4M3 || M < 0 || N < 0) return 0.0;
    return (double)kPerElem[step] * (double)M * (double)N;
}

int gemm_tile_map(int64_t wg, int64_t batch, int64_t tiles_m, int64_t tiles_n, int64_t group_m, int64_t *b,
                  int64_t *tm, int64_t *tn)
{
    if (batch <= 0 || tiles_m <= 0 || tiles_n <= 0 || group_m < -tiles_m || wg < 0 ||
        wg >= batch * tiles_m * tiles_n || !b || !tm || !tn)
        return -1;
    const g5::TileCoord t = g5::tile_map(wg, batch, tiles_m, tiles_n, group_m);
    *b = t.b;
    *tm = t.tm;
    *tn = t.tn;
    return 0;
}

}  // extern "C"
