// g5_streamk.hip -- the bf16 LDS-ring kernel with a persistent stream-K
// schedule: one workgroup per CU walks an equal share of all (output tile,
// 32-deep K stage) pairs, so that the matrix cores of every CU get the same
// number of stages whatever the tile count, and tiles whose K range is split
// between workgroups are finished by adding their partial tiles in a fixed
// order ("Operator & Runtime" §5.5.4: a persistent kernel walking tile
// tasks; §5.2.4: partial sums over a split reduction, combined in a fixed
// order; MUSA lesson m11-l5 case 1: the last block to finish completes the
// result).
#include <hip/hip_runtime.h>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

// A 64-bit value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uni64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Unit space: U = T x KT (T tiles, KT stages per tile), unit u = t * KT + k.
// Logical workgroup L owns units [lo(L), lo(L + 1)) with lo(L) = L * U / G.
__device__ __forceinline__ int64_t sk_lo(int64_t L, int64_t U, int64_t G) { return L * U / G; }
// The logical workgroup that owns unit u: the largest L with lo(L) <= u.
__device__ __forceinline__ int64_t sk_owner(int64_t u, int64_t U, int64_t G) { return ((u + 1) * G + U - 1) / U - 1; }

// Tile t -> (batch entry, tile row, tile column): column bands group_m
// tiles tall, walked column by column (the band order of tile_map, without
// its per-XCD regrouping: here consecutive logical workgroups, which own
// consecutive tiles, are placed on one XCD instead).
__device__ __forceinline__ TileCoord sk_tile(int64_t t, const GemmArgs &p)
{
    const int64_t per_batch = p.tiles_m * p.tiles_n;
    TileCoord c;
    c.b = t / per_batch;
    const int64_t r = t - c.b * per_batch;
    // (the diagnostic orders of tile_map, group_m <= 0, give bands of
    // |group_m| tiles, or of 1)
    const int64_t gm = p.group_m > 0 ? p.group_m : p.group_m < 0 ? -p.group_m : 1;
    const int64_t band_tiles = gm * p.tiles_n;
    const int64_t band = r / band_tiles;
    const int64_t first_m = band * gm;
    const int64_t rem_m = p.tiles_m - first_m;
    const int64_t h = rem_m < gm ? rem_m : gm;
    const int64_t rr = r - band * band_tiles;
    c.tm = first_m + rr % h;
    c.tn = rr / h;
    return c;
}

// grid = G <= U workgroups, one per CU, so that every workgroup owns at
// least one unit.  Workgroup w runs on XCD w % 8 and, when G is a multiple of
// 8, takes logical index L = (w % 8) * (G / 8) + w / 8, so
// each XCD owns one contiguous eighth of the unit space: its tiles share A
// row panels and B column panels in that XCD's L2, and the pieces of a split
// tile mostly meet on one XCD.
//
// A workgroup walks its units tile by tile (a "segment" per tile).  A segment
// that covers a whole tile is stored directly.  The pieces of a split tile
// (P of them, piece q covering the q-th K range) are combined as in the
// K-split ring kernel: every piece writes its FP32 tile to its slot with
// agent-scope (sc1) stores, waits for them, and counts itself on the tile's
// counter; the piece that brings the count to P adds pieces 0..P-1 in that
// order (its own from registers, the same bits it stored), resets the
// counter and stores the tile.  No workgroup ever waits for another.  A
// split piece is the first or the last segment of its workgroup (a segment
// between them covers a whole tile), so slot 2 L + (0: first, 1: last)
// holds it: the workspace has 2 G slots of BM x BN floats.
// Requires K % 32 == 0 (whole stages) and 16-byte aligned rows of A and B.
template <int BM, int BN, int WGM, int WGN, int NSA, int NSB, bool MASKED, int EPI, bool BT, bool AT>
__global__ void __launch_bounds__(WGM *WGN * 64, 2) k_bf16_sk(GemmArgs p)
{
    using R = RingTile<BM, BN, WGM, WGN, NSA, NSB, 16, MASKED, EPI, BT, false, AT>;
    constexpr int FM = R::FM, FN = R::FN, NWAVE = R::NWAVE, KS = R::KS;
    constexpr int TILE_F = BM * BN;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[R::LDS_BYTES / 2];
    __shared__ unsigned sk_arrived;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // Everything that steers the walk is uniform over the workgroup: held in
    // scalar registers, so that the accumulators keep the vector registers.
    const int64_t T = p.batch * p.tiles_m * p.tiles_n;
    const int64_t KT = p.K / KS;
    const int64_t U = T * KT, G = gridDim.x;
    const int64_t L = G % kNumXcd == 0 ? (int64_t)(blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd
                                       : (int64_t)blockIdx.x;
    const int64_t lo = uni64(sk_lo(L, U, G)), hi = uni64(sk_lo(L + 1, U, G));
    const int64_t t_first = uni64(lo / KT);
    for (int64_t u = lo; u < hi;) {
        const int64_t t = uni64(u / KT), a = uni64(u - t * KT);
        const int64_t b = uni64(hi - t * KT < KT ? hi - t * KT : KT);
        // The arguments are read again from the kernel-argument segment for
        // every segment (scalar loads) rather than held in scalar registers
        // across the walk, which the tile's own copy descriptors need.
        const GemmArgs *pp = &p;
        asm volatile("" : "+s"(pp));
        const TileCoord tc = sk_tile(t, *pp);
        f32x4 acc[FN][FM];
        R::zero(acc);
        R::accumulate(*pp, smem, tc, a * KS, (b - a) * KS, acc);
        bool finish = true;
        if (a != 0 || b != KT) {
            const int64_t wf = uni64(sk_owner(t * KT, U, G)), wl = uni64(sk_owner(t * KT + KT - 1, U, G));
            const int P = (int)(wl - wf + 1), piece = (int)(L - wf);
            float *slot = p.ws_part + (2 * L + (t == t_first ? 0 : 1)) * (int64_t)TILE_F;
            const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(slot, 0, TILE_F * 4, 0x00020000);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int off = (((fn * FM + fm) * NWAVE + wave) * 64 + lane) * 16;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[fn][fm]), wr, off, 0, 16);
                }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) sk_arrived = __hip_atomic_fetch_add(p.ws_cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (sk_arrived != (unsigned)(P - 1)) {
                finish = false;
            } else {
                // piece q belongs to logical workgroup wf + q; pieces after
                // the first start that workgroup's range (its first segment),
                // the first is wf's first segment only when its range starts
                // at this tile.  Each accumulator block is summed over the
                // pieces in order, in place.
                auto slot_of = [&](int q) {
                    const int64_t wq = wf + q;
                    const int segq = (q == 0 && sk_lo(wq, U, G) / KT != t) ? 1 : 0;
                    return __builtin_amdgcn_make_buffer_rsrc(p.ws_part + (2 * wq + segq) * (int64_t)TILE_F, 0,
                                                             TILE_F * 4, 0x00020000);
                };
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) {
                        const int off = (((fn * FM + fm) * NWAVE + wave) * 64 + lane) * 16;
                        f32x4 v = piece == 0 ? acc[fn][fm]
                                             : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(slot_of(0), off, 0, 16));
                        for (int q = 1; q < P; ++q)
                            v += q == piece ? acc[fn][fm]
                                            : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(slot_of(q), off, 0, 16));
                        acc[fn][fm] = v;
                        // one block's loads at a time: the other blocks' accumulators hold the registers
                        __builtin_amdgcn_s_waitcnt(0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                if (tid == 0) __hip_atomic_store(p.ws_cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (finish) R::store(*pp, smem, tc, acc);
        u = t * KT + b;
        __syncthreads();   // the LDS ring and staging area are free for the next segment
    }
}

template <int BM, int BN, int WGM, int WGN, int EPI, bool BT, bool AT>
static hipError_t launch_sk(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b(WGM * WGN * 64);
    if (variant == 1) hipLaunchKernelGGL((k_bf16_sk<BM, BN, WGM, WGN, 4, 4, false, EPI, BT, AT>), g, b, 0, s, a);
    else if (variant == 2) hipLaunchKernelGGL((k_bf16_sk<BM, BN, WGM, WGN, 4, 4, true, EPI, BT, AT>), g, b, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_streamk(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    switch (config_id) {
    case CFG_BF16_256x256: return launch_sk<256, 256, 2, 4, EPI_NONE, false, false>(a, variant, grid, s);
    case CFG_BF16_256x192: return launch_sk<256, 192, 2, 4, EPI_NONE, false, false>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace g5
