// g5_device.h -- device code shared by the kernel translation units of the
// dense-GEMM library: vector types, the bf16 rounding, the loaders, the
// LDS-writing buffer copies and swizzles, the LDS-staged epilogue and the
// bf16 LDS-ring kernel (k_bf16_ms) with its launcher over the ring
// variants.  Each .hip file instantiates the kernel configurations it
// launches, so the library's kernels compile in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>

#include "g5_common.h"

namespace g5 {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef long i64x2 __attribute__((ext_vector_type(2)));

#define G5_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

// ---------------------------------------------------------------- helpers

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// FP32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet bit set,
// payload kept), infinities keep their sign.  gfx950 converts a pair of
// floats in one instruction (v_cvt_pk_bf16_f32); over every binary32
// pattern, in both halves, it gives the same bits as the arithmetic rule
// (u + 0x7fff + bit 16 of u) >> 16 for non-NaN u and (u >> 16) | 0x40 for
// NaN (checked exhaustively on an MI355X), about a twelfth of its cost.
__device__ __forceinline__ uint32_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), in FP32 ("Operator & Runtime"
// §5.4.2 fuses it into the output tile), with the hardware reciprocal (about
// 1 ulp, far below the bf16 rounding that follows).  Large negative x gives
// e^-x = inf and a result of -0.
__device__ __forceinline__ float silu_f32(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3FN quantization of bf16 values against their row's (or column's)
// largest magnitude amax (page "Operator & Runtime" §5.4.3, Example 5-7): the code nearest
// to x * 448 / amax.  t = x * 448 is exact in binary32 (a bf16 significand
// times 7 * 64).  A quotient of two bf16 values sits either exactly on a
// midpoint between two E4M3FN values (at most 5 significant bits) or at
// least ~2^-13 of its size away from every midpoint, so any binary32
// quotient within ~2^-20 of the exact one that is exact at those midpoints
// gives, after the round-to-nearest-even conversion, the same code as the
// exact quotient.  Two such quotients:
//  - div: the correctly rounded division, clamped to +-448 (the conversion
//    turns larger values into NaN); defined for every amax > 0;
//  - fast: q0 = t * r with r = 1/amax correctly rounded, then one residual
//    step q0 + (t - q0 * amax) * r, both with single-rounding fmas
//    (Markstein's correction): exact whenever the quotient is, within ~1
//    ulp otherwise, and four instructions instead of a dozen.  For every
//    bf16 amax in [2^-126, 2^118] (x * 448 cannot overflow; the reciprocal
//    and the residual stay normal) and every bf16 x with |x| <= amax it
//    gives the code of div, never exceeds 448 in magnitude, and keeps the
//    sign of -0 (the residual is formed as q0 * amax - t and negated inside
//    the second fma): checked exhaustively on the host over all such pairs.
// A zero row (amax = 0) gives signed zeros.  Each quantizer takes the fast
// form when its amax is in range (uniform over a row) and div otherwise.
struct E4m3Quot {
    float amax, rcp;
    bool fast;
    __device__ __forceinline__ explicit E4m3Quot(float a)
        : amax(a), rcp(__frcp_rn(a)), fast(a >= 0x1p-126f && a <= 0x1p118f) {}
    __device__ __forceinline__ float q_fast(float x) const
    {
        const float t = x * 448.0f;
        const float q0 = t * rcp;
        const float e = __builtin_fmaf(q0, amax, -t);
        return __builtin_fmaf(-e, rcp, q0);
    }
    __device__ __forceinline__ float q_div(float x) const
    {
        const float y = amax > 0.0f ? __fdiv_rn(x * 448.0f, amax) : x * 0.0f;
        return y > 448.0f ? 448.0f : (y < -448.0f ? -448.0f : y);
    }
    // codes of 8 bf16 values (4 words, low half first), 4 per 32-bit word
    template <bool FAST>
    __device__ __forceinline__ uint32_t code4(uint32_t w0, uint32_t w1) const
    {
        auto q = [&](float x) { return FAST ? q_fast(x) : q_div(x); };
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_lo(w0)), q(bf16_hi(w0)), 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_lo(w1)), q(bf16_hi(w1)), pk, true);
        return (uint32_t)pk;
    }
    __device__ __forceinline__ uint32_t code1(float x) const
    {
        const float y = fast ? q_fast(x) : q_div(x);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xffu;
    }
};

// Fixed-range E4M3FN codes (page "Operator & Runtime" §5.3.1 stores Z with
// one fixed scale factor, a byte per element): for a bf16 value z, the code
// nearest to the binary32 quotient fl(z * 448 / amax), saturating at +-448,
// NaN giving 0x7f; amax > 0 is the call's range.  What is quantized is the
// bf16 value the unfused program stores (SwiGLU: bf16(t * u)), so the
// quotient is that of E4m3Quot: for a bf16 amax in [2^-126, 2^118], z is
// first clamped to [-amax, amax] (beyond, the code saturates; at +-amax the
// fast quotient is exactly +-448) and takes the fast quotient (checked
// exhaustively for bf16 |z| <= amax); other ranges take the division.  Both
// forms are selects, no branches.  The conversion writes 0xff for a NaN, so
// the bytes of NaN inputs are set to 0x7f afterwards.
struct E4m3Fixed {
    E4m3Quot q;
    bool fast;
    __device__ __forceinline__ explicit E4m3Fixed(float a)
        : q(a), fast(q.fast && (__float_as_uint(a) & 0xffffu) == 0u) {}
    // the value converted for z (a NaN z gives some value; its byte is replaced)
    template <bool FAST>
    __device__ __forceinline__ float quot(float z) const
    {
        return FAST ? q.q_fast(__builtin_amdgcn_fmed3f(z, -q.amax, q.amax)) : q.q_div(z);
    }
    template <bool FAST>
    __device__ __forceinline__ uint32_t code(float z) const
    {
        const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quot<FAST>(z), 0.0f, 0, false) & 0xffu;
        return z != z ? 0x7fu : c;
    }
    __device__ __forceinline__ uint32_t code(float z) const { return fast ? code<true>(z) : code<false>(z); }
    // the codes of 4 values in one word, the first in the lowest byte (two
    // pair conversions, into the low and the high half)
    template <bool FAST>
    __device__ __forceinline__ uint32_t code4(float a, float b, float c, float d) const
    {
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(quot<FAST>(a), quot<FAST>(b), 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(quot<FAST>(c), quot<FAST>(d), pk, true);
        const uint32_t m = (a != a ? 0xffu : 0u) | (b != b ? 0xff00u : 0u) | (c != c ? 0xff0000u : 0u) |
                           (d != d ? 0xff000000u : 0u);
        return ((uint32_t)pk & ~m) | (0x7f7f7f7fu & m);
    }
};

// Fused epilogues of a bf16 output chunk (8 values, already rounded once to
// bf16 from the FP32 sums: the rounding of the unfused program survives,
// §5.4.3).  SiLU: y = bf16(SiLU(g)).  SwiGLU (§5.3.1): z = bf16(t * u) with
// t = bf16(SiLU(g)); t and u are bf16, so t * u is exact in FP32 and z is
// rounded once.
__device__ __forceinline__ u32x4 epi_silu8(u32x4 g)
{
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = pack_bf16x2(silu_f32(bf16_lo(g[i])), silu_f32(bf16_hi(g[i])));
    return y;
}
__device__ __forceinline__ u32x4 epi_swiglu8(u32x4 g, u32x4 u)
{
    const u32x4 t = epi_silu8(g);
    u32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        z[i] = pack_bf16x2(bf16_lo(t[i]) * bf16_lo(u[i]), bf16_hi(t[i]) * bf16_hi(u[i]));
    return z;
}
// The product step alone: bf16(t * u) of 8 packed bf16 t and u (exact in
// FP32, rounded once).
__device__ __forceinline__ u32x4 mul8_bf16(u32x4 t, u32x4 u)
{
    u32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        z[i] = pack_bf16x2(bf16_lo(t[i]) * bf16_lo(u[i]), bf16_hi(t[i]) * bf16_hi(u[i]));
    return z;
}
// The fixed-range E4M3FN codes of 8 packed bf16 values (4 per word, the lowest column
// in the lowest byte).
template <bool FAST>
__device__ __forceinline__ u32x2 codes8_e4m3(u32x4 z, const E4m3Fixed &fq)
{
    return u32x2{fq.code4<FAST>(bf16_lo(z[0]), bf16_hi(z[0]), bf16_lo(z[1]), bf16_hi(z[1])),
                 fq.code4<FAST>(bf16_lo(z[2]), bf16_hi(z[2]), bf16_lo(z[3]), bf16_hi(z[3]))};
}
// The SwiGLU outputs of a chunk as codes: those of the bf16 outputs.
template <bool FAST>
__device__ __forceinline__ u32x2 epi_swiglu8_e4m3(u32x4 g, u32x4 u, const E4m3Fixed &fq)
{
    return codes8_e4m3<FAST>(epi_swiglu8(g, u), fq);
}

// One output element of the small-M kernels: the FP32 sum of batch entry
// b, or with the affine epilogue alpha * sum + bias[n] + beta * C[m][n]
// (C read only when beta != 0), rounded once to C's type.
__device__ __forceinline__ void store_out(const GemmArgs &p, int64_t b, int64_t m, int64_t n, float sum)
{
    const int64_t off = b * p.sC + m * p.ldc + n;
    if (p.affine) {
        float t = p.bias ? __uint_as_float((uint32_t)p.bias[n] << 16) : 0.f;
        if (p.beta != 0.f) {
            const float old = p.out_f32 ? ((const float *)p.C)[off]
                                        : __uint_as_float((uint32_t)((const uint16_t *)p.C)[off] << 16);
            t = __builtin_fmaf(p.beta, old, t);
        }
        sum = __builtin_fmaf(p.alpha, sum, t);
    }
    // SiLU of the bf16-rounded product, rounded again (as the ring kernels'
    // fused epilogue: the roundings of the unfused program)
    if (p.epi == EPI_SILU) sum = silu_f32(__uint_as_float(bf16_rne(sum) << 16));
    if (p.out_f32) ((float *)p.C)[off] = sum;
    else ((uint16_t *)p.C)[off] = (uint16_t)bf16_rne(sum);
}

// The SwiGLU output of the small-M kernels ("Operator & Runtime" §5.3.1):
// z = bf16(t * u) with t = bf16(SiLU(bf16(g))), u = bf16(u) -- the gate and
// up FP32 sums each rounded once as the unfused products would be; t * u is
// exact in FP32.
__device__ __forceinline__ void store_swiglu(const GemmArgs &p, int64_t b, int64_t m, int64_t n, float g, float u)
{
    const float t = __uint_as_float(bf16_rne(silu_f32(__uint_as_float(bf16_rne(g) << 16))) << 16);
    const float ub = __uint_as_float(bf16_rne(u) << 16);
    const int64_t off = b * p.sC + m * p.ldc + n;
    const uint32_t z = bf16_rne(t * ub);
    if (p.c_e4m3) ((uint8_t *)p.C)[off] = (uint8_t)E4m3Fixed(p.c_amax).code(__uint_as_float(z << 16));
    else ((uint16_t *)p.C)[off] = (uint16_t)z;
}

// Load 8 consecutive bf16 elements (one 16-byte chunk) starting at element
// `col` of a row, zero for elements at or beyond `limit` or when the row is
// out of range.  `align` is the byte alignment of the row start (16/8/4/2);
// col is a multiple of 8, so the chunk has the same alignment.
__device__ __forceinline__ u32x4 load_chunk8_bf16(const uint16_t *row, int64_t col, int64_t limit,
                                                  bool row_ok, int align)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!row_ok) return v;
    const uint16_t *p = row + col;
    if (col + 8 <= limit) {
        if (align >= 16) return *(const u32x4 *)p;
        if (align >= 8) {
            u32x2 lo = *(const u32x2 *)p, hi = *(const u32x2 *)(p + 4);
            v[0] = lo[0]; v[1] = lo[1]; v[2] = hi[0]; v[3] = hi[1];
            return v;
        }
        if (align >= 4) {
            const uint32_t *q = (const uint32_t *)p;
            v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
            return v;
        }
    }
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (col + i < limit) ? (uint32_t)p[i] : 0u;
    v[0] = e[0] | (e[1] << 16); v[1] = e[2] | (e[3] << 16);
    v[2] = e[4] | (e[5] << 16); v[3] = e[6] | (e[7] << 16);
    return v;
}

// Same for 4 consecutive floats (one 16-byte chunk of an fp32 row).
// Load 16 consecutive bytes (16 fp8 codes) starting at element `col` of a
// row, zero for elements at or beyond `limit` or when the row is out of
// range; `align` is the byte alignment of the row start (col is a multiple
// of 16).
__device__ __forceinline__ u32x4 load_chunk16_u8(const uint8_t *row, int64_t col, int64_t limit, bool row_ok,
                                                 int align)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!row_ok) return v;
    const uint8_t *p = row + col;
    if (col + 16 <= limit) {
        if (align >= 16) return *(const u32x4 *)p;
        if (align >= 4) {
            const uint32_t *q = (const uint32_t *)p;
            v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
            return v;
        }
    }
    uint32_t e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = (col + i < limit) ? (uint32_t)p[i] : 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = e[4 * w] | (e[4 * w + 1] << 8) | (e[4 * w + 2] << 16) | (e[4 * w + 3] << 24);
    return v;
}

__device__ __forceinline__ u32x4 load_chunk4_f32(const float *row, int64_t col, int64_t limit,
                                                 bool row_ok, int align)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!row_ok) return v;
    const float *p = row + col;
    if (col + 4 <= limit) {
        if (align >= 16) return *(const u32x4 *)p;
        if (align >= 8) {
            u32x2 lo = *(const u32x2 *)p, hi = *(const u32x2 *)(p + 2);
            v[0] = lo[0]; v[1] = lo[1]; v[2] = hi[0]; v[3] = hi[1];
            return v;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (col + i < limit) ? __float_as_uint(p[i]) : 0u;
    return v;
}

// Store 4 consecutive results of one row of C (columns n..n+3).  These are
// partial 128-byte lines, left to merge in L2 (non-temporal stores, which
// help the whole-line epilogue, measured slower here).
__device__ __forceinline__ void store4(void *Cbase, bool out_f32, int64_t ldc, int64_t m, int64_t n,
                                       f32x4 v, bool full, int64_t M, int64_t N, int align_c)
{
    if (out_f32) {
        float *c = (float *)Cbase + m * ldc + n;
        if (full && align_c >= 16) {
            *(f32x4 *)c = v;
            return;
        }
        if (m >= M) return;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n + j < N) c[j] = v[j];
    } else {
        uint16_t *c = (uint16_t *)Cbase + m * ldc + n;
        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        if (full && align_c >= 8) {
            u32x2 w = {lo, hi};
            *(u32x2 *)c = w;
            return;
        }
        if (m >= M) return;
        const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n + j < N) c[j] = e[j];
    }
}

// One wave-wide direct-to-LDS copy: lane i's 16 bytes at byte offset
// voff + soff of the buffer based at `base` land at lds + 16 i (bytes).
// The buffer base must be the same for every lane; num_records is set to the
// largest positive value, the aligned kernels' offsets stay far below it.
__device__ __forceinline__ void buffer_load_lds16(const void *base, uint32_t voff, uint32_t soff, void *lds)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, G5_LDS(void, lds), 16, voff, soff, 0, 0);
}

// The same copy issued as an instruction the compiler does not look into.
// Its waitcnt pass would otherwise treat every later LDS read as possibly
// aliasing the copy's destination and wait for all copies in flight
// (vmcnt(0)), which would serialise a multi-stage ring; the ring kernel
// accounts for its copies itself with explicit vmcnt waits.  M0 carries the
// LDS destination; one wait state separates its write from the load.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x4_t make_rsrc(const void *base, uint32_t num_records = 0x7fffffffu)
{
    const uint64_t b = (uint64_t)base;
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)((b >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int32_t)num_records);
    r[3] = 0x00020000;
    return r;
}
// BYTES is 16 (dwordx4) or 4 (dword): the LDS-writing buffer loads that
// gfx950 provides for these widths.
template <int BYTES>
__device__ __forceinline__ void dma(i32x4_t rsrc, uint32_t voff, uint32_t soff, const void *lds)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)G5_LDS(const void, lds));
    if (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :
                     : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
                     : "memory", "m0");
}

// s_waitcnt immediate (gfx9 layout): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4] (7 = no wait), lgkmcnt [11:8].
constexpr int waitcnt_imm(int vmcnt, int lgkmcnt)
{
    return (vmcnt & 0xf) | ((vmcnt >> 4) << 14) | (7 << 4) | ((lgkmcnt & 0xf) << 8);
}

// XOR swizzles of 16-byte chunk indices.
//  A slab rows hold 8 chunks (64 bf16 or 32 fp32): the chunk index is XORed
//  with row & 7, so the 16 rows that one fragment read touches (16 lanes,
//  same logical chunk) land on 8 distinct chunk positions -- measured
//  conflict-free for ds_read_b128 on gfx950 (4 LDS cycles per wave read).
__device__ __forceinline__ int swz_a(int row) { return row & 7; }
//  bf16 B slab rows (k) are read 4 rows x 32 bytes per 16 lanes by the
//  transposing read; XORing chunk bits 1..2 (a 32-byte segment inside an
//  aligned group of 4 segments) with this function of k spreads the 8 rows
//  {k0..k0+3, k0+8..k0+11} that 32 lanes read over distinct banks.
__device__ __forceinline__ int swz_b(int k) { return ((((k >> 1) & 1) | (((k >> 3) & 1) << 1))) << 1; }
//  The ring kernel's B slots: with BN = 192 the row pitch (384 bytes) puts
//  consecutive rows half the banks apart, so swz_b suffices.  When the row
//  pitch is a multiple of 256 bytes (BN % 128 == 0) every row starts on the
//  same bank, so the 8 rows read together get 8 distinct 32-byte segments:
//  chunk bits 1..3 are XORed with (k & 3) | ((k >> 3) & 1) << 2 (measured
//  bank conflicts, as a share of LDS cycles, with 128x128 tiles: batched
//  32 x 1024x1024x128 27% -> 0%, the FFN shape 40% -> 1.5%).
template <int BN>
__device__ __forceinline__ int swz_bn(int k)
{
    if constexpr (BN % 128 == 0) return ((k & 3) | (((k >> 3) & 1) << 2)) << 1;
    else return swz_b(k);
}

// Epilogue of whole tiles: the BM x BN results, held as acc[fn][fm] with
// lane (g, li) of wave (wm, wn) owning row wm*TM + 16 fm + li, columns
// wn*TN + 16 fn + 4 g .. +3, are written to LDS in row-major order (rows
// padded by 16 bytes against bank conflicts), then copied to C in 16-byte
// chunks with consecutive lanes on consecutive chunks of a row.  Tiles that
// do not fit in LDS at once go in passes of whole wave rows.  `lds` holds
// LDS_BYTES; every wave must have finished with it.  MASKED: only chunks of
// rows < M that end at or before column N are stored (N must be a multiple
// of the chunk's 16 / sizeof(TOut) elements, so no chunk straddles it).
template <int BM, int BN, int WGM, int WGN, int LDS_BYTES, typename TOut, bool MASKED, int EPI = EPI_NONE, int NFN,
          int NFM>
__device__ __forceinline__ void store_tile_via_lds(const f32x4 (&acc)[NFN][NFM], uint16_t *lds, void *Cb,
                                                   int64_t ldc, int64_t m0, int64_t n0, int64_t M, int64_t N,
                                                   const GemmArgs *pa = nullptr)
{
    static_assert(EPI == EPI_NONE || (EPI == EPI_AFFINE ? sizeof(TOut) == 4 : sizeof(TOut) == 2),
                  "SiLU and SwiGLU stage bf16; the affine epilogue stages the FP32 sums");
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int ESZ = (int)sizeof(TOut);
    constexpr int PITCH = BN * ESZ + 16;                     // bytes per staged row
    constexpr int CPR = BN * ESZ / 16;                       // 16-byte chunks per row
    constexpr int NT = WGM * WGN * 64;
    constexpr int FITS = LDS_BYTES / PITCH;                  // rows that fit
    constexpr int RP = FITS >= BM ? BM : (FITS >= BM / 2 ? BM / 2 : BM / 4);
    static_assert(RP % 16 == 0 && RP * PITCH <= LDS_BYTES, "staging passes");
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // offsets derived anew in every call (see RingTile::accumulate)
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, li = lane & 15;
    char *L = (char *)lds;
    // Affine epilogue: 8-column steps, APER per thread and pass.
    constexpr int AOPR = BN / 8;
    constexpr int APER = EPI == EPI_AFFINE ? (RP * AOPR + NT - 1) / NT : 1;
    u32x4 old0[APER], old1[APER];
#pragma unroll
    for (int pass = 0; pass < BM / RP; ++pass) {
        if constexpr (EPI == EPI_AFFINE) {
            // Load this pass's old C chunks first (beta != 0), so that their
            // latency overlaps the staging below.
            if (pa->beta != 0.f) {
                const bool f32o = pa->out_f32 != 0;
#pragma unroll
                for (int i = 0; i < APER; ++i) {
                    const int q = tid + i * NT;
                    if (APER * NT != RP * AOPR && q >= RP * AOPR) break;
                    const int r = q / AOPR, c = q % AOPR;
                    const int64_t m = m0 + pass * RP + r, n = n0 + (int64_t)c * 8;
                    if (MASKED && (m >= M || n + 8 > N)) continue;
                    const char *src = (const char *)Cb + (m * ldc + n) * (f32o ? 4 : 2);
                    old0[i] = *(const u32x4 *)src;
                    if (f32o) old1[i] = *(const u32x4 *)(src + 16);
                }
            }
        }
        // Each pass stages the 16-row accumulator blocks whose rows fall in
        // it (a wave's rows span several passes when a pass is shorter than
        // the wave tile).
        if (wm * TM / RP <= pass && (wm * TM + TM - 1) / RP >= pass) {
#pragma unroll
            for (int fn = 0; fn < NFN; ++fn)
#pragma unroll
                for (int fm = 0; fm < NFM; ++fm) {
                    if ((wm * TM + fm * 16) / RP != pass) continue;
                    const int r = wm * TM + fm * 16 + li - pass * RP;
                    const int c = wn * TN + fn * 16 + g * 4;
                    const f32x4 v = acc[fn][fm];
                    if (ESZ == 4) {
                        *(f32x4 *)(L + r * PITCH + c * 4) = v;
                    } else {
                        u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *(u32x2 *)(L + r * PITCH + c * 2) = w;
                    }
                }
        }
        __syncthreads();
        if constexpr (EPI == EPI_SWIGLU) {
            // Tile columns [0, BN/2) hold the gate product g, [BN/2, BN) the
            // up product u of the same BN/2 output columns starting at n0.
            // Fixed-range E4M3FN output (pa->c_e4m3): 8 codes, 8 bytes, per chunk.
            constexpr int OPR = CPR / 2;                     // output chunks per row
            if (pa->c_e4m3) {
                // (the quotient's form is fixed per call: one loop each)
                const E4m3Fixed fq(pa->c_amax);
                auto codes = [&](auto fast) {
                    for (int q = tid; q < RP * OPR; q += NT) {
                        const int r = q / OPR, c = q % OPR;
                        if (MASKED && (m0 + pass * RP + r >= M || n0 + (int64_t)(c + 1) * 8 > N)) continue;
                        const u32x4 g = *(const u32x4 *)(L + r * PITCH + c * 16);
                        const u32x4 u = *(const u32x4 *)(L + r * PITCH + (c + OPR) * 16);
                        char *dst = (char *)Cb + (m0 + pass * RP + r) * ldc + n0 + c * 8;
                        __builtin_nontemporal_store(epi_swiglu8_e4m3<decltype(fast)::value>(g, u, fq), (u32x2 *)dst);
                    }
                };
                if (fq.fast) codes(std::true_type{});
                else codes(std::false_type{});
            } else {
                for (int q = tid; q < RP * OPR; q += NT) {
                    const int r = q / OPR, c = q % OPR;
                    if (MASKED && (m0 + pass * RP + r >= M || n0 + (int64_t)(c + 1) * 8 > N)) continue;
                    const u32x4 g = *(const u32x4 *)(L + r * PITCH + c * 16);
                    const u32x4 u = *(const u32x4 *)(L + r * PITCH + (c + OPR) * 16);
                    char *dst = (char *)Cb + ((m0 + pass * RP + r) * ldc + n0) * 2 + c * 16;
                    __builtin_nontemporal_store(epi_swiglu8(g, u), (u32x4 *)dst);
                }
            }
        } else if constexpr (EPI == EPI_AFFINE) {
            // 8 columns per step: v = alpha * sum + (bias[n] + beta * C[m][n])
            // in FP32, rounded once to C's type (bf16 or float); the old C
            // chunks of this pass were loaded before the staging.
            const float alpha = pa->alpha, beta = pa->beta;
            const bool f32o = pa->out_f32 != 0;
#pragma unroll
            for (int i = 0; i < APER; ++i) {
                const int q = tid + i * NT;
                if (APER * NT != RP * AOPR && q >= RP * AOPR) break;
                const int r = q / AOPR, c = q % AOPR;
                const int64_t m = m0 + pass * RP + r, n = n0 + (int64_t)c * 8;
                if (MASKED && (m >= M || n + 8 > N)) continue;
                const f32x4 s0 = *(const f32x4 *)(L + r * PITCH + c * 32);
                const f32x4 s1 = *(const f32x4 *)(L + r * PITCH + c * 32 + 16);
                float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (pa->bias) {
                    const u32x4 bb = load_chunk8_bf16(pa->bias, n, N, true, pa->align_bias);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        t[2 * j] = bf16_lo(bb[j]);
                        t[2 * j + 1] = bf16_hi(bb[j]);
                    }
                }
                if (beta != 0.f) {
                    if (f32o) {
                        const f32x4 o0 = __builtin_bit_cast(f32x4, old0[i]), o1 = __builtin_bit_cast(f32x4, old1[i]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            t[j] = __builtin_fmaf(beta, o0[j], t[j]);
                            t[4 + j] = __builtin_fmaf(beta, o1[j], t[4 + j]);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            t[2 * j] = __builtin_fmaf(beta, bf16_lo(old0[i][j]), t[2 * j]);
                            t[2 * j + 1] = __builtin_fmaf(beta, bf16_hi(old0[i][j]), t[2 * j + 1]);
                        }
                    }
                }
                f32x4 v0, v1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v0[j] = __builtin_fmaf(alpha, s0[j], t[j]);
                    v1[j] = __builtin_fmaf(alpha, s1[j], t[4 + j]);
                }
                char *dst = (char *)Cb + (m * ldc + n) * (f32o ? 4 : 2);
                if (f32o) {
                    __builtin_nontemporal_store(v0, (f32x4 *)dst);
                    __builtin_nontemporal_store(v1, (f32x4 *)(dst + 16));
                } else {
                    const u32x4 w = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                     pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
                    __builtin_nontemporal_store(w, (u32x4 *)dst);
                }
            }
        } else {
            for (int q = tid; q < RP * CPR; q += NT) {
                const int r = q / CPR, c = q % CPR;
                if (MASKED && (m0 + pass * RP + r >= M || n0 + (int64_t)(c + 1) * (16 / ESZ) > N)) continue;
                u32x4 v = *(const u32x4 *)(L + r * PITCH + c * 16);
                if constexpr (EPI == EPI_SILU) v = epi_silu8(v);
                char *dst = (char *)Cb + ((m0 + pass * RP + r) * ldc + n0) * ESZ + c * 16;
                __builtin_nontemporal_store(v, (u32x4 *)dst);     // C is written once
            }
        }
        __syncthreads();
    }
}

// ================================================= bf16 MFMA ring kernel
//
// Tile BM x BN, 8 waves (two per SIMD, so one wave's MFMAs run while the
// other waits), wave tile (BM/WGM) x (BN/WGN).
//
// K is walked in stages of 32 through rings of LDS slots, NSA for A and NSB
// for B, so the copies of A stage k+NSA-1 and B stage k+NSB-1 are in flight
// while stage k is multiplied: the slab copies from L2 (and, on first touch,
// HBM) get several stages of compute to land ("4.1 Tối ưu hiệu năng toán tử
// GEMM trên CUDA" §9-§10 and "Operator & Runtime" §5.3.2 double buffering,
// deepened for gfx950's latency).  The two depths are independent because
// A and B are copied by different waves, each with its own vmcnt.
//  * Copies are buffer loads that write LDS directly (buffer_load ... lds):
//    one wave instruction moves 64 lanes x AV bytes of A (AV = 16, or 4 for
//    rows that are only 4- or 8-byte aligned) or 64 x 16 bytes of B into LDS, lane
//    i at byte AV*i, with no registers or ds_write instructions spent on
//    staging.  The slot's XOR swizzle is applied by choosing, per lane, which
//    global chunk lands in its position.  Waves 0..3 copy A, 4..7 copy B.
//  * A slot rows are 32 bf16 = 64 bytes (4 chunks), swizzled chunk ^
//    ((row >> 1) & 3), measured conflict-free for the fragment reads; B slot
//    rows are BN bf16, swizzled with swz_bn, read with ds_read_b64_tr_b16.
//  * Each wave waits for its own copies of the next stage (vmcnt counts
//    the copies still allowed in flight), then one barrier per stage.  The
//    loop is bounded by LDS traffic (copy writes plus fragment reads) and by
//    the copy path, not by copy latency: deeper rings measured no faster.  After
//    the barrier the next stage's fragments are read into the second
//    register set while the last TAIL MFMAs of the current stage run.
//  * MASKED: the buffer descriptors carry each operand's byte extent, so
//    reads past it return zero instead of faulting; rows of A at or beyond M
//    are sent out of range.  Columns of B beyond N and rows of A beyond M
//    only feed outputs that are never stored.  A K remainder (K % 32) is a
//    final stage loaded element by element with zero fill ("4.1" §4.5 and
//    "Operator & Runtime" §5.4.2: out-of-range elements contribute zero).
//  * EPI: EPI_SILU applies SiLU to each bf16-rounded output; EPI_SWIGLU
//    multiplies a merged gate|up weight B = [W_g | W_u] ([K, 2N]): the
//    tile's B slab takes its first BN/2 columns from W_g and the last BN/2
//    from the same columns of W_u, and the epilogue combines the two halves
//    into BN/2 columns of Z = bf16(bf16(SiLU(g)) * u).  Both need the
//    LDS-staged epilogue (16-byte aligned output rows, N % 8 == 0).
//  * EPI_AFFINE: C := alpha * sum + bias[n] + beta * C, from the FP32 sums
//    staged in LDS, rounded once to C's type (bf16 or float).
//  * SK: K is split over p.ksplit workgroups per tile (see GemmArgs); each
//    publishes its FP32 accumulators and the last to arrive adds the
//    partial tiles in slice order, so the result does not depend on which
//    workgroup finishes last ("Operator & Runtime" §5.2.4: partial sums over
//    split K, combined in a fixed order).
//  * BT: B is given transposed, Bt [N, K] row-major (element (k, n) at
//    Bt + n*ldb + k), the layout of a linear layer's weight and of the keys
//    of attention scores.  Its slab is then K-contiguous like A's: copied
//    and swizzled like A's, and read with ds_read_b128 instead of the
//    transposing read.
//  * AT: A is given transposed, At [K, M] row-major (element (m, k) at
//    At + k*lda + m), the layout of the activations in a weight gradient
//    X^T.dY.  Its slab (BK rows of BM columns m) is copied, swizzled and
//    read like B's, with the transposing read giving the K-contiguous A
//    fragments.  Needs 16-byte aligned rows of At and M % 8 == 0 or rows
//    padded to a multiple of 8 (the masked copy reads whole 16-byte chunks).
//  * F8: A and Bt hold E4M3FN codes (with BT): the same 64-byte slot rows
//    then carry 64 values of K per stage.  With an even stage count the
//    stages go in pairs through the double-rate fp8 instruction (below);
//    otherwise each 16-byte fragment feeds two v_mfma_f32_16x16x32_fp8_fp8
//    (the first takes bytes 0-7 of every lane, the second bytes 8-15: one
//    permutation of K, the same for both operands).  The FP32 sums are
//    multiplied by p.scale_a[row] and p.scale_b[column] (of the batch
//    entry) before the epilogue, plain or affine ("Operator & Runtime"
//    §5.4.3, Example 5-7: dequantization by the row's factor).
// One output tile of the bf16 LDS-ring kernel, as device functions that the
// tile kernels below call: `accumulate` multiplies K columns
// [kbase, kbase + K) of the tile's A row panel and B column panel into the
// FP32 accumulators (the LDS ring must be free on entry and is free again on
// return); `store` applies the fp8 factors and the epilogue and writes the
// tile to C through LDS.
template <int BM, int BN, int WGM, int WGN, int NSA, int NSB, int AV, bool MASKED, int EPI = EPI_NONE,
          bool BT = false, bool F8 = false, bool AT = false, bool QA = false>
struct RingTile {
    static constexpr int NWAVE = WGM * WGN;
    static constexpr int BK = 32;                                    // slot row: 32 bf16 = 64 bytes
    static constexpr int EB = F8 ? 1 : 2;                            // bytes per operand element
    static constexpr int KS = 64 / EB;                               // K per stage
    static_assert(!F8 || (BT && (EPI == EPI_NONE || EPI == EPI_AFFINE)), "fp8 operands: A and Bt, plain or affine epilogue");
    static_assert(!AT || (!F8 && !BT && AV == 16 && (EPI == EPI_NONE || EPI == EPI_AFFINE)),
                  "transposed A: bf16, B as [K, N], plain or affine epilogue");
    static_assert(!AT || ((BM / 8) % 8 == 0 && (BM % 128 != 0 || (BM / 8) % 16 == 0)), "At slot rows: whole swizzle groups");
    // QA: A is given as bf16 rows and quantized to E4M3FN codes on the way
    // into LDS (see accumulate); fp8 B codes given transposed, 4-slot rings.
    static_assert(!QA || (F8 && BT && !AT && EPI == EPI_NONE && NSA == 2 && NSB == 4 && AV == 16 &&
                          BM * 4 == WGM * WGN * 64),
                  "quantized-on-load A: fp8, Bt, 2 code slots and 4 B slots, one 16-code chunk per lane");
    static constexpr int TM = BM / WGM, TN = BN / WGN;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int NMFMA = FM * FN;
    static constexpr int TAIL = NMFMA / 2;                           // MFMAs run after the barrier
    static constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN;
    static constexpr int B_BASE = NSA * A_ELEMS;                     // B ring after the A ring (elements)
    // (QA: two stages of the bf16 A slab staged after the rings, 2 BM x 64
    // bf16 per stage)
    static constexpr int QA_STAGE_BYTES = QA ? BM * 64 * 2 : 0;
    static constexpr int LDS_BYTES = (NSA * A_ELEMS + NSB * B_ELEMS) * 2 + 2 * QA_STAGE_BYTES;
    static constexpr int A_INS = A_ELEMS * 2 / (64 * AV), B_INS = B_ELEMS * 2 / 1024;   // copy instructions
    static constexpr int A_W = NWAVE / 2, B_W = NWAVE / 2;           // copying waves per operand
    static constexpr int LA = A_INS / A_W, LB = B_INS / B_W;         // copies per wave per stage
    static constexpr int ROWS_PER_A = 64 * AV / 64;                  // A rows per copy instruction
    static_assert(NWAVE == 8, "two waves per SIMD");
    static_assert(AV == 16 || AV == 4, "A copy width");
    static_assert(A_INS % A_W == 0 && B_INS % B_W == 0, "slab split");
    static_assert((BN / 8) % 8 == 0 && (BN % 128 != 0 || (BN / 8) % 16 == 0), "B slot rows must be whole swizzle groups");
    static_assert((QA || NSA >= 3) && NSB >= 3 && LA * (NSA - 2) < 64 && LB * (NSB - 2) < 64, "vmcnt accounting");
    static_assert(TAIL > 0 && TAIL < NMFMA, "tail");
    static constexpr bool GLU = EPI == EPI_SWIGLU;
    static constexpr int HALF = BN / 2;                       // GLU: columns per weight half
    static_assert(!GLU || HALF % 8 == 0, "GLU halves must be whole chunks");
    static_assert(!(GLU && BT), "SwiGLU takes B as [K, 2N]");
    using Acc = f32x4[FN][FM];

    __device__ static __forceinline__ void zero(Acc &acc)
    {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    __device__ static __forceinline__ void accumulate(const GemmArgs &p, uint16_t *smem, const TileCoord &tc,
                                                      const int64_t kbase, const int64_t K, Acc &acc)
    {
    // The lane's offsets derive from the thread index anew in every call
    // (opaque to the compiler), so a kernel that calls this in a loop does
    // not keep them live in vector registers across the loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, li = lane & 15;
    // n0: first output column (GLU: first column of each weight half)
    const int64_t m0 = tc.tm * BM, n0 = tc.tn * (GLU ? HALF : BN);
    const int64_t M = p.M, N = p.N, lda = p.lda, ldb = p.ldb;
    const char *Abat = (const char *)p.A + (tc.b * p.sA + (AT ? kbase * lda : kbase)) * (QA ? 2 : EB);
    const char *Bbat = (const char *)p.B + (tc.b * p.sB + (BT ? kbase : kbase * ldb)) * EB;
    // Byte extents of this batch entry's operands from those bases (reads
    // past them return 0).
    // (At: the last row is read up to M rounded up to 8, which the host
    // guarantees is inside the allocation: M % 8 == 0 or padded rows.)
    const uint32_t a_bytes = !MASKED ? 0x7fffffffu
                             : AT    ? (uint32_t)(((p.K - kbase - 1) * lda + ((M + 7) & ~(int64_t)7)) * 2)
                                     : (uint32_t)(((M - 1) * lda + (p.K - kbase)) * (QA ? 2 : EB));
    const uint32_t b_bytes =
        !MASKED ? 0x7fffffffu
        : BT    ? (uint32_t)(((N - 1) * ldb + (p.K - kbase)) * EB)
                : (uint32_t)(((p.K - kbase - 1) * ldb + (GLU ? 2 * N : N)) * 2);
    // Global column of slot column c (a multiple of 8) of the B slab.
    auto b_col = [&](int c) -> int64_t { return GLU ? (c < HALF ? n0 + c : N + n0 + (c - HALF)) : n0 + c; };

    // Copy sources.  Offsets are bytes from the batch entry's base; the stage
    // adds k0 (A) or k0 rows (B) through the scalar offset.  A instruction r
    // covers slot rows ROWS_PER_A*r.. ; lane l lands in row ROWS_PER_A*r +
    // l/(64/ROWS_PER_A) at byte (l % (64/ROWS_PER_A))*AV of the row, and
    // holds the matching bytes of logical chunk (position ^ ((row>>1)&3)).
    const bool a_wave = wave < A_W;
    const int a_i0 = a_wave ? wave * LA : 0;
    uint32_t a_voff[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        if constexpr (AT) {
            // as B: 1024 bytes of the BK x BM slab (k rows of BM columns m) per instruction
            const int q = 1024 * (a_i0 + j) + 16 * lane;
            const int k = q / (BM * 2), pc = (q % (BM * 2)) / 16;
            a_voff[j] = (uint32_t)((k * lda + m0 + (pc ^ swz_bn<BM>(k)) * 8) * 2);
            continue;
        }
        constexpr int LPR = 64 / ROWS_PER_A;                  // lanes per 64-byte row
        const int row = ROWS_PER_A * (a_i0 + j) + lane / LPR;
        const int byte = (lane % LPR) * AV;                   // byte within the slot row
        const int chunk = (byte >> 4) ^ ((row >> 1) & 3);
        const uint32_t off = (uint32_t)((m0 + row) * lda * EB + chunk * 16 + (byte & 15));
        a_voff[j] = (MASKED && m0 + row >= M) ? 0x80000000u : off;
    }
    const int b_i0 = a_wave ? 0 : (wave - A_W) * LB;
    uint32_t b_voff[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        if constexpr (BT) {
            // as A: 16 slot rows (columns n) of 64 bytes per instruction
            const int row = 16 * (b_i0 + j) + lane / 4;
            const int chunk = (lane % 4) ^ ((row >> 1) & 3);
            const uint32_t off = (uint32_t)((n0 + row) * ldb * EB + chunk * 16);
            b_voff[j] = (MASKED && n0 + row >= N) ? 0x80000000u : off;
        } else {
            const int q = 1024 * (b_i0 + j) + 16 * lane;
            const int k = q / (BN * 2), pc = (q % (BN * 2)) / 16;
            b_voff[j] = (uint32_t)((k * ldb + b_col((pc ^ swz_bn<BN>(k)) * 8)) * 2);
        }
    }
    // The stage's offset moves the descriptor base (scalar arithmetic) and
    // shrinks its extent to match, so the scalar offset stays 0.
    // Each copying wave issues only its operand: A waves copy stage kt into
    // the A slot of stage ks (ks % NSA), B waves into B slot ks % NSB.
    auto issue = [&](int kt, int ks) {
        if (QA && a_wave) return;          // (QA: A goes through registers, qa_point below)
        if (a_wave) {
            uint16_t *sl = smem + (ks % NSA) * A_ELEMS;
            // 64 bytes of each A row, or BK rows of At, per stage
            const int64_t kstep = AT ? (int64_t)kt * BK * lda * 2 : (int64_t)kt * 64;
            const uint32_t adv = (uint32_t)kstep;
            const i32x4_t r = make_rsrc(Abat + kstep, a_bytes - adv);
#pragma unroll
            for (int j = 0; j < LA; ++j) dma<AV>(r, a_voff[j], 0, sl + (a_i0 + j) * (32 * AV));
        } else {
            uint16_t *sl = smem + B_BASE + (ks % NSB) * B_ELEMS;
            // bytes: 64 of each Bt row, or BK rows of B
            const int64_t kstep = BT ? (int64_t)kt * 64 : (int64_t)kt * BK * ldb * 2;
            const uint32_t adv = (uint32_t)kstep;
            const i32x4_t r = make_rsrc(Bbat + kstep, b_bytes - adv);
#pragma unroll
            for (int j = 0; j < LB; ++j) dma<16>(r, b_voff[j], 0, sl + (b_i0 + j) * 512);
        }
    };

    // Fragment read offsets within a slot (elements).
    int a_rd[FM], a_rd4[FM], b_rd[FN], b_rd4[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        if constexpr (AT) {
            // the transposing read of B's slab, with rows m in place of columns n
            const int k = g * 8 + (li >> 2);
            const int mcol = wm * TM + fm * 16 + (li & 3) * 4;
            const int c = mcol >> 3, half = (mcol >> 2) & 1;
            a_rd[fm] = k * BM + ((c ^ swz_bn<BM>(k)) * 8) + half * 4;
            a_rd4[fm] = (k + 4) * BM + ((c ^ swz_bn<BM>(k + 4)) * 8) + half * 4;
        } else {
            const int row = wm * TM + fm * 16 + li;
            a_rd[fm] = row * BK + ((g ^ ((row >> 1) & 3)) * 8);
            a_rd4[fm] = 0;
        }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        if constexpr (BT) {
            const int row = wn * TN + fn * 16 + li;
            b_rd[fn] = row * BK + ((g ^ ((row >> 1) & 3)) * 8);
            b_rd4[fn] = 0;
        } else {
            const int k = g * 8 + (li >> 2);
            const int ncol = wn * TN + fn * 16 + (li & 3) * 4;
            const int c = ncol >> 3, half = (ncol >> 2) & 1;
            b_rd[fn] = k * BN + ((c ^ swz_bn<BN>(k)) * 8) + half * 4;
            b_rd4[fn] = (k + 4) * BN + ((c ^ swz_bn<BN>(k + 4)) * 8) + half * 4;
        }
    }
    struct Frags {
        bf16x8 a[FM];
        bf16x8 b[FN];
    };
    // Fragments of stage kt (A slot kt % NSA, B slot kt % NSB).
    auto read_frags = [&](Frags &f, int kt) {
        const uint16_t *sa = smem + (kt % NSA) * A_ELEMS;
        const uint16_t *sb = smem + B_BASE + (kt % NSB) * B_ELEMS;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if constexpr (AT) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G5_LDS(i16x4, sa + a_rd[fm]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G5_LDS(i16x4, sa + a_rd4[fm]));
                f.a[fm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                f.a[fm] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sa + a_rd[fm]));
            }
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            if constexpr (BT) {
                f.b[fn] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sb + b_rd[fn]));
            } else {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G5_LDS(i16x4, sb + b_rd[fn]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G5_LDS(i16x4, sb + b_rd4[fn]));
                f.b[fn] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
    };

    auto mfma_range = [&](const Frags &f, int first, int count) {
#pragma unroll
        for (int t = 0; t < NMFMA; ++t) {
            if (t < first || t >= first + count) continue;
            const int fn = t / FM, fm = t % FM;
            if constexpr (F8) {
                const i64x2 a2 = __builtin_bit_cast(i64x2, f.a[fm]), b2 = __builtin_bit_cast(i64x2, f.b[fn]);
                acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(b2[0], a2[0], acc[fn][fm], 0, 0, 0);
                acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(b2[1], a2[1], acc[fn][fm], 0, 0, 0);
            } else {
                acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[fn], f.a[fm], acc[fn][fm], 0, 0, 0);
            }
        }
    };

    // Wait until this wave's copies of the next stage have landed -- at most
    // NSA-2 (A waves) or NSB-2 (B waves) stages of its copies may still be in
    // flight -- and its LDS reads are done, then the workgroup barrier.
    auto stage_barrier = [&]() {
        if constexpr (QA) {
            // at the barrier after point s the B stage s - 2 must have
            // landed; issued after it: 2 staging copies and LB B copies at
            // each of points s - 1 and s (4 + 2 LB), of which the oldest two
            // (stage s - 2's staging, already converted) may be waited for too
            if (a_wave) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2, 0));
            else __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LB + 2, 0));
        } else {
            if (a_wave) __builtin_amdgcn_s_waitcnt(waitcnt_imm(LA * (NSA - 2), 0));
            else __builtin_amdgcn_s_waitcnt(waitcnt_imm(LB * (NSB - 2), 0));
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");   // no LDS access moves across the barrier
    };

    const int KT = (int)(K / KS);                             // whole stages

    // QA: A arrives as bf16 rows [M, K] (p.A, row stride p.lda elements) with
    // each row's largest magnitude in p.amax_a[m], and is quantized on the
    // way into LDS by the row quantizer's rule (E4m3Quot: the code nearest
    // to x * 448 / amax), so the codes are those a separate quantization
    // pass would have written.  Lane tid owns one 16-code chunk
    // of each stage's A slab: tile row qa_r = tid / 4, K columns
    // 16 (tid % 4) .. + 15 of the stage.  Its 32 bytes of bf16 are copied by
    // two direct-to-LDS loads into a staging area that only this lane reads
    // (lane order, 16 bytes per lane per copy), one point ahead, then read
    // back, converted and written as 16 codes to the chunk's place in the
    // swizzled code slot.  At the point that copies B stage s: convert A
    // stage s - 2 (its staging landed: only this wave's B copies of the
    // previous point were issued after it), then copy A stage s - 1's bf16,
    // then B stage s.  Requires K % 64 == 0.
    const int qa_r = tid >> 2, qa_c = tid & 3;
    const bool qa_row = QA && m0 + qa_r < M;
    const uint32_t qa_off = qa_row ? (uint32_t)(((m0 + qa_r) * lda + 16 * qa_c) * 2) : 0x80000000u;
    const E4m3Quot qa_q(qa_row ? p.amax_a[m0 + qa_r] : 0.f);
    uint16_t *const qa_stage = smem + (NSA * A_ELEMS + NSB * B_ELEMS);
    auto qa_copy = [&](int st) {          // bf16 of stage st (clamped) into staging st % 2
        const int sc = st < KT ? st : KT - 1;
        const uint32_t adv = (uint32_t)sc * 128;
        const i32x4_t r = make_rsrc(Abat + adv, a_bytes - adv);
        uint16_t *dst = qa_stage + (st & 1) * (QA_STAGE_BYTES / 2) + wave * 512;
        dma<16>(r, qa_off, 0, dst);
        dma<16>(r, qa_off + 16, 0, dst + NWAVE * 512);
    };
    auto qa_convert = [&](int st) {       // staging st % 2 -> codes in A slot st % NSA
        const uint16_t *src = qa_stage + (st & 1) * (QA_STAGE_BYTES / 2) + tid * 8;
        const u32x4 lo = *(const u32x4 *)src, hi = *(const u32x4 *)(src + NWAVE * 512);
        u32x4 codes;
        if (qa_q.fast)
            codes = u32x4{qa_q.code4<true>(lo[0], lo[1]), qa_q.code4<true>(lo[2], lo[3]),
                          qa_q.code4<true>(hi[0], hi[1]), qa_q.code4<true>(hi[2], hi[3])};
        else
            codes = u32x4{qa_q.code4<false>(lo[0], lo[1]), qa_q.code4<false>(lo[2], lo[3]),
                          qa_q.code4<false>(hi[0], hi[1]), qa_q.code4<false>(hi[2], hi[3])};
        *(u32x4 *)(smem + (st % NSA) * A_ELEMS + qa_r * BK + ((qa_c ^ ((qa_r >> 1) & 3)) * 8)) = codes;
    };
    auto qa_point = [&](int s) {
        if (a_wave) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        else __builtin_amdgcn_s_waitcnt(waitcnt_imm(LB, 15));
        asm volatile("" ::: "memory");
        if (s - 2 < KT) qa_convert(s - 2);
        qa_copy(s - 1);
    };

    // A stage past the last reloads the last one, into the slot of the stage
    // it stands for, which is never read again.
    auto issue_clamped = [&](int ks) {
        // (QA: the point is B's stage number for every wave; A waves are
        // called with their A ring's stage, NSB - NSA behind)
        if constexpr (QA) qa_point(a_wave ? ks + NSB - NSA : ks);
        issue(ks < KT ? ks : KT - 1, ks);
    };
    Frags f0, f1;
    if (KT > 0) {
        if constexpr (QA) {
            // Prologue: bf16 A stages 0 and 1 and B stages 0..NSB-2; A stage
            // 0 converted once its staging landed (issued after it: A stage
            // 1's 2 copies and this wave's B copies), B stage 0 landed.
            qa_copy(0);
            qa_copy(1);
            if (!a_wave)
                for (int s2 = 0; s2 < NSB - 1; ++s2) issue(s2 < KT ? s2 : KT - 1, s2);
            if (a_wave) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2, 15));
            else __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 + LB * (NSB - 1), 15));
            asm volatile("" ::: "memory");
            qa_convert(0);
            if (a_wave) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2, 0));
            else __builtin_amdgcn_s_waitcnt(waitcnt_imm(LB * (NSB - 2), 0));
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        } else {
        // Prologue: A stages 0..NSA-2 and B stages 0..NSB-2 (clamped, see
        // below), stage 0 complete.
        const int NPRO = a_wave ? NSA - 1 : NSB - 1;
        for (int s2 = 0; s2 < NPRO; ++s2) issue_clamped(s2);
        stage_barrier();
        }
        read_frags(f0, 0);

        // One stage: copies for stage kt+NSA-1 (A waves) or kt+NSB-1 (B
        // waves), MFMAs, barrier, next fragments, tail.  Stages past the last
        // one reload the final stage into a slot nobody reads again, which
        // keeps the in-flight counts uniform.
        auto step = [&](int kt, Frags &fc, Frags &fnx) {
            issue_clamped(kt + (a_wave ? NSA : NSB) - 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_range(fc, 0, NMFMA - TAIL);
            __builtin_amdgcn_sched_barrier(0);
            stage_barrier();
            read_frags(fnx, kt + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_range(fc, NMFMA - TAIL, TAIL);
            __builtin_amdgcn_sched_barrier(0);
        };
        // F8 with an even stage count (not at 256x256, whose registers do
        // not hold both loops): stages in pairs.  The 16-byte fragments of
        // stages 2j and 2j+1 make each lane's 32 bytes of K for one
        // double-rate MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 on both
        // sides, unit block scales), the same permutation of K for both
        // operands; even stages only copy, wait and read fragments.
        constexpr bool F8_PAIRS = F8 && !(BM == 256 && BN == 256);
        bool paired = false;
        if constexpr (F8_PAIRS) {
            if (KT % 2 == 0) {
                paired = true;
                auto mfma_pair = [&](const Frags &lo, const Frags &hi) {
#pragma unroll
                    for (int t = 0; t < NMFMA; ++t) {
                        const int fn = t / FM, fm = t % FM;
                        const i32x4_t al = __builtin_bit_cast(i32x4_t, lo.a[fm]);
                        const i32x4_t ah = __builtin_bit_cast(i32x4_t, hi.a[fm]);
                        const i32x4_t bl = __builtin_bit_cast(i32x4_t, lo.b[fn]);
                        const i32x4_t bh = __builtin_bit_cast(i32x4_t, hi.b[fn]);
                        const i32x8_t a8 = __builtin_shufflevector(al, ah, 0, 1, 2, 3, 4, 5, 6, 7);
                        const i32x8_t b8 = __builtin_shufflevector(bl, bh, 0, 1, 2, 3, 4, 5, 6, 7);
                        acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[fn][fm], 0, 0, 0,
                                                                                       127, 0, 127);
                    }
                };
                for (int kt = 0; kt < KT; kt += 2) {
                    issue_clamped(kt + (a_wave ? NSA : NSB) - 1);
                    stage_barrier();
                    read_frags(f1, kt + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    issue_clamped(kt + (a_wave ? NSA : NSB));
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_pair(f0, f1);
                    __builtin_amdgcn_sched_barrier(0);
                    stage_barrier();
                    read_frags(f0, kt + 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (!paired) {
            int kt = 0;
            for (; kt + 1 < KT; kt += 2) {
                step(kt, f0, f1);
                step(kt + 1, f1, f0);
            }
            if (kt < KT) step(kt, f0, f1);
        }
    }
    if (!QA && MASKED && K % KS != 0) {
        // K remainder: every copy in flight lands first, then the last stage
        // is loaded element by element with zero fill into slot 0.
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int64_t k0 = (int64_t)KT * KS;
        uint16_t *sA = smem, *sB = smem + B_BASE;
        if constexpr (AT) {
            for (int q = tid; q < BK * (BM / 8); q += NWAVE * 64) {
                const int k = q / (BM / 8), c = q % (BM / 8);
                const u32x4 v = load_chunk8_bf16((const uint16_t *)Abat + (k0 + k) * lda + m0, 8 * c, M - m0,
                                                 k0 + k < K, p.align_a);
                *(u32x4 *)(sA + k * BM + ((c ^ swz_bn<BM>(k)) * 8)) = v;
            }
        } else
        for (int q = tid; q < BM * 4; q += NWAVE * 64) {
            const int row = q >> 2, c = q & 3;
            const u32x4 v = F8 ? load_chunk16_u8((const uint8_t *)Abat + (m0 + row) * lda, k0 + 16 * c, K,
                                                 m0 + row < M, p.align_a)
                               : load_chunk8_bf16((const uint16_t *)Abat + (m0 + row) * lda, k0 + 8 * c, K,
                                                  m0 + row < M, p.align_a);
            *(u32x4 *)(sA + row * BK + ((c ^ ((row >> 1) & 3)) * 8)) = v;
        }
        if constexpr (BT) {
            for (int q = tid; q < BN * 4; q += NWAVE * 64) {
                const int row = q >> 2, c = q & 3;
                const u32x4 v = F8 ? load_chunk16_u8((const uint8_t *)Bbat + (n0 + row) * ldb, k0 + 16 * c, K,
                                                     n0 + row < N, p.align_b)
                                   : load_chunk8_bf16((const uint16_t *)Bbat + (n0 + row) * ldb, k0 + 8 * c, K,
                                                      n0 + row < N, p.align_b);
                *(u32x4 *)(sB + row * BK + ((c ^ ((row >> 1) & 3)) * 8)) = v;
            }
        } else
        for (int q = tid; q < BK * (BN / 8); q += NWAVE * 64) {
            const int k = q / (BN / 8), c = q % (BN / 8);
            // GLU: chunk c of the up half is column n0 + 8c - HALF of W_u,
            // which lies at N + n0 + 8c - HALF of the merged row
            const bool up = GLU && 8 * c >= HALF;
            const int64_t base = up ? N + n0 - HALF : n0;
            const u32x4 v = load_chunk8_bf16((const uint16_t *)Bbat + (k0 + k) * ldb + base, 8 * c,
                                             up ? N - n0 + HALF : N - n0, k0 + k < K, p.align_b);
            *(u32x4 *)(sB + k * BN + ((c ^ swz_bn<BN>(k)) * 8)) = v;
        }
        __syncthreads();
        read_frags(f0, 0);
        mfma_range(f0, 0, NMFMA);
    }
    __builtin_amdgcn_s_waitcnt(0);

    }

    __device__ static __forceinline__ void store(const GemmArgs &p, uint16_t *smem, const TileCoord &tc, Acc &acc)
    {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, li = lane & 15;
    // n0: first output column (GLU: first column of each weight half)
    const int64_t m0 = tc.tm * BM, n0 = tc.tn * (GLU ? HALF : BN);
    const int64_t M = p.M, N = p.N, lda = p.lda, ldb = p.ldb;
    if constexpr (F8) {
        // Dequantization: the row's factor, then the column's, in FP32 (the
        // batch entry's factors).
        const float *scale_a = p.scale_a ? p.scale_a + tc.b * p.s_scale_a : nullptr;
        const float *scale_b = p.scale_b ? p.scale_b + tc.b * p.s_scale_b : nullptr;
        if (scale_a || scale_b) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int64_t m = m0 + wm * TM + fm * 16 + li;
                const float sa = (scale_a && m < M) ? scale_a[m] : 1.0f;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int64_t n = n0 + wn * TN + fn * 16 + g * 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float sb = (scale_b && n + i < N) ? scale_b[n + i] : 1.0f;
                        acc[fn][fm][i] = acc[fn][fm][i] * sa * sb;
                    }
                }
            }
        }
    }

    void *Cb = (char *)p.C + tc.b * p.sC * (p.c_e4m3 ? 1 : p.out_f32 ? 4 : 2);
    if (p.align_c >= 16 && (!MASKED || N % (p.out_f32 ? 4 : 8) == 0)) {
        // 16-byte aligned rows of C: stage the results through LDS (free
        // once every wave's copies and reads are done) and write whole
        // 16-byte chunks, consecutive lanes on consecutive chunks of a row,
        // so that every 128-byte line of C is written by one store.  Edge
        // tiles store only the chunks inside C, which needs N to be a whole
        // number of chunks.
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (EPI == EPI_AFFINE) {
            store_tile_via_lds<BM, BN, WGM, WGN, LDS_BYTES, float, MASKED, EPI>(acc, smem, Cb, p.ldc, m0, n0, M, N, &p);
        } else if constexpr (EPI != EPI_NONE) {
            store_tile_via_lds<BM, BN, WGM, WGN, LDS_BYTES, uint16_t, MASKED, EPI>(acc, smem, Cb, p.ldc, m0, n0, M, N,
                                                                                 &p);
        } else {
            if (p.out_f32) store_tile_via_lds<BM, BN, WGM, WGN, LDS_BYTES, float, MASKED>(acc, smem, Cb, p.ldc, m0, n0, M, N);
            else store_tile_via_lds<BM, BN, WGM, WGN, LDS_BYTES, uint16_t, MASKED>(acc, smem, Cb, p.ldc, m0, n0, M, N);
        }
        return;
    }
    if constexpr (EPI != EPI_NONE) return;   // the host never launches a fused epilogue without the staged store
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t m = m0 + wm * TM + fm * 16 + li;
            const int64_t n = n0 + wn * TN + fn * 16 + g * 4;
            if (MASKED && (m >= M || n >= N)) continue;
            const bool full = !MASKED || (n + 4 <= N);
            store4(Cb, p.out_f32 != 0, p.ldc, m, n, acc[fn][fm], full, M, N, p.align_c);
        }
    }
};

template <int BM, int BN, int WGM, int WGN, int NSA, int NSB, int AV, bool MASKED, int EPI = EPI_NONE,
          bool SK = false, bool BT = false, bool F8 = false, bool AT = false>
__global__ void __launch_bounds__(WGM *WGN * 64, 2) k_bf16_ms(GemmArgs p)
{
    using R = RingTile<BM, BN, WGM, WGN, NSA, NSB, AV, MASKED, EPI, BT, F8, AT>;
    constexpr int FM = R::FM, FN = R::FN, NWAVE = R::NWAVE, KS = R::KS;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[R::LDS_BYTES / 2];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t ntiles = p.batch * p.tiles_m * p.tiles_n;
    const int64_t wg = SK ? (int64_t)blockIdx.x % ntiles : (int64_t)blockIdx.x;
    const int slice = SK ? (int)((int64_t)blockIdx.x / ntiles) : 0;
    const TileCoord tc = tile_map(wg, p.batch, p.tiles_m, p.tiles_n, p.group_m);
    // This workgroup's part of K starts at kbase; the operand bases below are
    // moved there, so everything after this works on K columns from them.
    const int64_t kbase = SK ? (int64_t)slice * p.kt_per * KS : 0;
    const int64_t Kpart = SK && slice < p.ksplit - 1 ? (int64_t)p.kt_per * KS : p.K - kbase;
    f32x4 acc[FN][FM];
    R::zero(acc);
    R::accumulate(p, smem, tc, kbase, Kpart, acc);

    if constexpr (SK) {
        // Publish this slice's FP32 tile in register order (block, wave,
        // lane: each wave writes 1 KiB runs) with device-scope (sc1) stores,
        // wait for them, then count the arrival.  The workgroup that brings
        // the tile's counter to ksplit adds the slices 0, 1, ... in order
        // (its own from registers, bit-identical to what it stored), resets
        // the counter for the next call and stores the tile.  No fence: the
        // sc1 (device-scope) stores and loads of the partial tiles complete
        // at the device's coherence point, never in an XCD's private L2,
        // the wait and barrier retire every store before the counter
        // atomic (performed at that point) is issued, and the last arriver
        // loads only after reading the atomic's result.
        __shared__ unsigned sk_arrived;
        constexpr int TILE_F = BM * BN;
        float *tile_ws = p.ws_part + wg * p.ksplit * (int64_t)TILE_F;
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            tile_ws + (int64_t)slice * TILE_F, 0, TILE_F * 4, 0x00020000);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int off = (((fn * FM + fm) * NWAVE + wave) * 64 + lane) * 16;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[fn][fm]), wr, off, 0, 16);
            }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) sk_arrived = __hip_atomic_fetch_add(p.ws_cnt + wg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (sk_arrived != (unsigned)(p.ksplit - 1)) return;
        f32x4 tot[FN][FM];
        for (int s2 = 0; s2 < p.ksplit; ++s2) {
            const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
                tile_ws + (int64_t)s2 * TILE_F, 0, TILE_F * 4, 0x00020000);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int off = (((fn * FM + fm) * NWAVE + wave) * 64 + lane) * 16;
                    const f32x4 v = s2 == slice ? acc[fn][fm]
                                                : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 16));
                    tot[fn][fm] = s2 == 0 ? v : tot[fn][fm] + v;
                }
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = tot[fn][fm];
        if (tid == 0) __hip_atomic_store(p.ws_cnt + wg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    R::store(p, smem, tc, acc);
}

// Ring kernel variants 1-3 (16-byte A copies aligned / masked, 4-byte A copies masked).
template <int BM, int BN, int WGM, int WGN, int NSA, int NSB, int EPI, bool SK, bool BT, bool F8 = false,
          bool AT = false>
static hipError_t launch_ring(const GemmArgs &a, int variant, dim3 g, dim3 b, hipStream_t s)
{
    switch (variant) {
    case 1: hipLaunchKernelGGL((k_bf16_ms<BM, BN, WGM, WGN, NSA, NSB, 16, false, EPI, SK, BT, F8, AT>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_bf16_ms<BM, BN, WGM, WGN, NSA, NSB, 16, true, EPI, SK, BT, F8, AT>), g, b, 0, s, a); break;
    case 3:
        if constexpr (AT) return hipErrorInvalidValue;       // At rows are copied 16 bytes per lane only
        else hipLaunchKernelGGL((k_bf16_ms<BM, BN, WGM, WGN, NSA, NSB, 4, true, EPI, SK, BT, F8>), g, b, 0, s, a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace g5
