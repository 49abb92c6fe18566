// fm_ws.h — pieces of the weight-streaming products whose waves own adjacent 16-row weight tiles and share one LDS
// copy of the activation fragments (the bf16 lm_head argmax kernel, and the Q8_0 kernels' code decode and loads).
//
// A work-group of NW waves walks a k-range in chunks of 8 k-steps (256 columns) in lockstep:
//   * each wave holds NT bf16 weight tiles of 16 rows (NT = 2: the two matrices of a gated unit), row-staged: a chunk
//     of a tile is 8 row-contiguous instructions (2 rows x 512 bytes), parked in a wave-private LDS tile and read back
//     in the A layout of v_mfma_f32_16x16x32_bf16 (whole cache lines per instruction instead of the A layout's 16
//     half lines);
//   * the chunk's activation fragments (NB blocks of 16 rows, 16 KB each: k-step s at 2 KB, hi then lo) are read from
//     L2 once per work-group, each thread a 1 / NW share, into a double-buffered LDS slab.
// Q8_0 tables are streamed from a copy in the MFMA operand layout instead (launch_q8_tile_copy): their codes need no
// LDS staging; codes go exactly through the bf16 MFMA (int8 is exact in bf16) and each row's scale multiplies its
// step's product before it is accumulated.
#pragma once
#include "fm_device.h"

namespace ws {

constexpr int RS_PITCH = 33;   // uint4 per LDS row of a bf16 chunk: 32 + 1 pad (conflict-free A reads)

__device__ __forceinline__ uint32_t nt32(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint4 ldg_nt(const void* p) {
    const uint32_t* q = (const uint32_t*)p;
    return make_uint4(nt32(q), nt32(q + 1), nt32(q + 2), nt32(q + 3));
}
__device__ __forceinline__ bf16x8_t as_bf(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8 int8 codes -> 8 bf16 (exact)
__device__ __forceinline__ uint4 i8x8_bf16(uint2 c) {
    uint32_t w[2] = {c.x, c.y};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int b0 = ((int)(w[i] << (24 - 16 * j))) >> 24;
            int b1 = ((int)(w[i] << (16 - 16 * j))) >> 24;
            o[2 * i + j] = (__float_as_uint((float)b0) >> 16) | (__float_as_uint((float)b1) & 0xffff0000u);
        }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// ── bf16 ───────────────────────────────────────────────────────────────────────────────────────
template <int NW, int NT, int NB>
struct Regs {
    uint4 a[NT][8];         // the wave's NT tiles: 16 rows x 256 columns each
    uint4 b[NB * 16 / NW];  // this thread's share of the chunk's fragments
};

// W[n]: row 0 of the wave's tile n (row stride K elements); X: fragments (block b at X + b * K * 64); ch: chunk
template <int NW, int NT, int NB>
__device__ __forceinline__ void load(Regs<NW, NT, NB>& r, const uint16_t* const* W, int K, const uint8_t* X, int ch,
                                     int tid) {
    const int lane = tid & 63;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint16_t* E = W[n] + (size_t)(lane >> 5) * K + ch * 256 + (lane & 31) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) r.a[n][i] = ldg_nt(E + (size_t)(2 * i) * K);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint4* xb = (const uint4*)(X + (size_t)b * K * 64 + (size_t)ch * 8 * FRAG_STEP_BYTES);
#pragma unroll
        for (int j = 0; j < 16 / NW; ++j) r.b[b * (16 / NW) + j] = xb[tid + 64 * NW * j];
    }
}

// alds: the wave's [NT][16 * RS_PITCH] tile; blds: the slab buffer [NB * 1024] (uint4)
template <int NW, int NT, int NB>
__device__ __forceinline__ void stage(const Regs<NW, NT, NB>& r, uint4* alds, uint4* blds, int tid) {
    const int lane = tid & 63;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 8; ++i) alds[n * 16 * RS_PITCH + (2 * i + (lane >> 5)) * RS_PITCH + (lane & 31)] = r.a[n][i];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 16 / NW; ++j) blds[b * 1024 + tid + 64 * NW * j] = r.b[b * (16 / NW) + j];
}

template <int NT, int NB>
__device__ __forceinline__ void compute(const uint4* alds, const uint4* blds, f32x4_t (&acc)[NT][NB], int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const uint4 av = alds[n * 16 * RS_PITCH + r * RS_PITCH + 4 * i + g];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint4 bh = blds[b * 1024 + i * 128 + lane], bl = blds[b * 1024 + i * 128 + 64 + lane];
                acc[n][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(av), as_bf(bh), acc[n][b], 0, 0, 0);
                acc[n][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(av), as_bf(bl), acc[n][b], 0, 0, 0);
            }
        }
    }
}

}  // namespace ws
