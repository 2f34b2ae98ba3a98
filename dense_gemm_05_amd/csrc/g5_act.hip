// g5_act.hip -- the activation chain of page "Operator & Runtime" §5.3.1
// (Example 5-4) on stored bf16 G and U: T = SiLU(G), Z = T (.) U, and Z
// quantized to E4M3FN with one fixed scale, each as its own step and fused.
// Every output element depends only on the inputs at its own position, so
// the work is a stream: HBM-bound, with no reuse for LDS or the matrix
// cores.  Each thread moves 16-byte chunks (8 bf16 values) of every operand,
// consecutive lanes on consecutive chunks of a row, with four chunks' loads
// issued before any of them is used; three persistent workgroups per CU walk
// the chunks and load the next four before storing the current ones;
// outputs go out with non-temporal stores (nothing reads them back in the
// call).  The element arithmetic is
// that of the fused GEMM epilogues (epi_silu8, mul8_bf16, epi_swiglu8,
// codes8_e4m3), so a chain step gives the same bits as the epilogue that
// fuses it.
#include <hip/hip_runtime.h>

#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

namespace {

constexpr int kActThreads = 256;
constexpr int kActUnroll = 4;   // chunks per thread, loads issued together
constexpr uint64_t kActGrid = 256 * 3;   // persistent workgroups: three per CU

constexpr bool act_two_inputs(int step) { return step == ACT_MUL || step == ACT_SWIGLU || step == ACT_SWIGLU_E4M3; }
constexpr bool act_codes(int step) { return step == ACT_QUANT || step == ACT_SWIGLU_E4M3; }

// One output chunk from the input chunks x0 (G, T or Z) and x1 (U).
template <int STEP, bool FAST>
__device__ __forceinline__ void act_store(void *dst, u32x4 x0, u32x4 x1, const E4m3Fixed &fq)
{
    if constexpr (STEP == ACT_SILU) __builtin_nontemporal_store(epi_silu8(x0), (u32x4 *)dst);
    else if constexpr (STEP == ACT_MUL) __builtin_nontemporal_store(mul8_bf16(x0, x1), (u32x4 *)dst);
    else if constexpr (STEP == ACT_SWIGLU) __builtin_nontemporal_store(epi_swiglu8(x0, x1), (u32x4 *)dst);
    else if constexpr (STEP == ACT_QUANT) __builtin_nontemporal_store(codes8_e4m3<FAST>(x0, fq), (u32x2 *)dst);
    else __builtin_nontemporal_store(epi_swiglu8_e4m3<FAST>(x0, x1, fq), (u32x2 *)dst);
}

// Whole 16-byte chunks: N % 8 == 0, every input row start 16-byte aligned,
// output rows 16-byte (bf16) or 8-byte (codes) aligned; M * N / 8 < 2^31.
// CONTIG: every operand's rows follow each other (ld == N), so chunk c sits
// at element 8c of each operand.  Persistent: a workgroup walks groups of
// kActUnroll chunks per thread, gridDim.x groups apart, and issues the next
// group's loads before it stores the current one.
template <int STEP, bool FAST, bool CONTIG>
__global__ void __launch_bounds__(kActThreads) k_act_vec(ActArgs a)
{
    constexpr bool TWO = act_two_inputs(STEP);
    constexpr int OB = act_codes(STEP) ? 1 : 2;   // output bytes per element
    const uint32_t cpr = (uint32_t)(a.N >> 3);
    const uint32_t total = (uint32_t)a.M * cpr;
    const E4m3Fixed fq(a.amax);
    const uint32_t stride = gridDim.x * (uint32_t)(kActThreads * kActUnroll);
    struct Group {
        u32x4 x0[kActUnroll], x1[kActUnroll];
        int64_t eo[kActUnroll];   // output element offsets of the chunks
    };
    auto load = [&](uint32_t first, Group &g) {
#pragma unroll
        for (int j = 0; j < kActUnroll; ++j) {
            const uint32_t c = first + (uint32_t)(j * kActThreads);
            int64_t e0, e1;
            if (CONTIG) {
                e0 = e1 = g.eo[j] = (int64_t)c * 8;
            } else {
                const uint32_t r = c / cpr, col = (c - r * cpr) * 8;
                e0 = (int64_t)r * a.ld0 + col;
                e1 = (int64_t)r * a.ld1 + col;
                g.eo[j] = (int64_t)r * a.ldo + col;
            }
            if (c < total) {
                g.x0[j] = __builtin_nontemporal_load((const u32x4 *)(a.in0 + e0));
                if constexpr (TWO) g.x1[j] = __builtin_nontemporal_load((const u32x4 *)(a.in1 + e1));
            }
        }
    };
    auto store = [&](uint32_t first, const Group &g) {
#pragma unroll
        for (int j = 0; j < kActUnroll; ++j) {
            const uint32_t c = first + (uint32_t)(j * kActThreads);
            if (c < total) act_store<STEP, FAST>((char *)a.out + g.eo[j] * OB, g.x0[j], TWO ? g.x1[j] : g.x0[j], fq);
        }
    };
    uint32_t first = blockIdx.x * (uint32_t)(kActThreads * kActUnroll) + threadIdx.x;
    Group cur, nxt;
    load(first, cur);
    // (total + stride < 2^32: the host keeps the chunk count below 2^31)
    for (; first < total; first += stride) {
        load(first + stride, nxt);
        store(first, cur);
        cur = nxt;
    }
}

// Any shape and alignment: one element per thread and step (grid-stride).
template <int STEP>
__global__ void __launch_bounds__(kActThreads) k_act_elem(ActArgs a)
{
    const int64_t total = a.M * a.N;
    const int64_t stride = (int64_t)gridDim.x * kActThreads;
    const E4m3Fixed fq(a.amax);
    for (int64_t q = (int64_t)blockIdx.x * kActThreads + threadIdx.x; q < total; q += stride) {
        const int64_t r = q / a.N, n = q - r * a.N;
        const float x = __uint_as_float((uint32_t)a.in0[r * a.ld0 + n] << 16);
        const float u = act_two_inputs(STEP) ? __uint_as_float((uint32_t)a.in1[r * a.ld1 + n] << 16) : 0.f;
        uint32_t v;   // the bf16 result (the codes' input for the quantizing steps)
        if constexpr (STEP == ACT_SILU) v = bf16_rne(silu_f32(x));
        else if constexpr (STEP == ACT_MUL) v = bf16_rne(x * u);
        else if constexpr (STEP == ACT_QUANT) v = __float_as_uint(x) >> 16;
        else v = bf16_rne(__uint_as_float(bf16_rne(silu_f32(x)) << 16) * u);
        if constexpr (act_codes(STEP)) ((uint8_t *)a.out)[r * a.ldo + n] = (uint8_t)fq.code(__uint_as_float(v << 16));
        else ((uint16_t *)a.out)[r * a.ldo + n] = (uint16_t)v;
    }
}

template <int STEP>
hipError_t launch_step(const ActArgs &a, bool vec, bool contig, hipStream_t s)
{
    if (vec) {
        const uint64_t chunks = (uint64_t)a.M * (uint64_t)(a.N >> 3);
        const uint64_t groups = (chunks + kActThreads * kActUnroll - 1) / (kActThreads * kActUnroll);
        const dim3 g((unsigned)(groups < kActGrid ? groups : kActGrid));
        // (the quotient's form is uniform over a call: one kernel each)
        bool fast = false;
        if constexpr (act_codes(STEP)) {
            const uint32_t bits = [&] { uint32_t b; __builtin_memcpy(&b, &a.amax, 4); return b; }();
            fast = (bits & 0xffffu) == 0u && a.amax >= 0x1p-126f && a.amax <= 0x1p118f;
        }
        if (contig) {
            if (fast) hipLaunchKernelGGL((k_act_vec<STEP, true, true>), g, dim3(kActThreads), 0, s, a);
            else hipLaunchKernelGGL((k_act_vec<STEP, false, true>), g, dim3(kActThreads), 0, s, a);
        } else {
            if (fast) hipLaunchKernelGGL((k_act_vec<STEP, true, false>), g, dim3(kActThreads), 0, s, a);
            else hipLaunchKernelGGL((k_act_vec<STEP, false, false>), g, dim3(kActThreads), 0, s, a);
        }
    } else {
        const int64_t total = a.M * a.N;
        const int64_t want = (total + kActThreads - 1) / kActThreads;
        const dim3 g((unsigned)(want < 256 * 16 ? want : 256 * 16));
        hipLaunchKernelGGL((k_act_elem<STEP>), g, dim3(kActThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_act_chain(int step, const ActArgs &a, bool vec, bool contig, hipStream_t s)
{
    switch (step) {
    case ACT_SILU: return launch_step<ACT_SILU>(a, vec, contig, s);
    case ACT_MUL: return launch_step<ACT_MUL>(a, vec, contig, s);
    case ACT_SWIGLU: return launch_step<ACT_SWIGLU>(a, vec, contig, s);
    case ACT_QUANT: return launch_step<ACT_QUANT>(a, vec, contig, s);
    case ACT_SWIGLU_E4M3: return launch_step<ACT_SWIGLU_E4M3>(a, vec, contig, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace g5
