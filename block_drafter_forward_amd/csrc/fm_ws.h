// fm_ws.h — pieces of the weight-streaming products whose waves own adjacent 16-row weight tiles and share one LDS
// copy of the activation fragments (the lm_head argmax kernel, and the skinny GEMM's tile-owning variant).
//
// A work-group of NW waves walks a k-range in chunks of 8 k-steps (256 columns) in lockstep:
//   * each wave holds NT weight tiles of 16 rows (NT = 2: the two matrices of a gated unit), row-staged: a chunk of a
//     bf16 tile is 8 row-contiguous instructions (2 rows x 512 bytes), of a Q8_0 tile 4 instructions (4 rows x 256
//     code bytes) plus one 16-byte load of each row's 8 scales; they are parked in a wave-private LDS tile and read
//     back in the A layout of v_mfma_f32_16x16x32_bf16 (whole cache lines per instruction instead of the A layout's
//     16 half lines);
//   * the chunk's activation fragments (NB blocks of 16 rows, 16 KB each: k-step s at 2 KB, hi then lo) are read from
//     L2 once per work-group, each thread a 1 / NW share, into a double-buffered LDS slab;
//   * Q8_0 codes go exactly through the bf16 MFMA (int8 is exact in bf16) and each row's scale multiplies its step's
//     product before it is accumulated.
#pragma once
#include "fm_device.h"

namespace ws {

constexpr int RS_PITCH = 33;   // uint4 per LDS row of a bf16 chunk: 32 + 1 pad (conflict-free A reads)
constexpr int Q8_PITCH = 17;   // uint4 per LDS row of a Q8_0 chunk: 16 + 1 pad

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

// ── Q8_0 (one block of activation rows) ─────────────────────────────────────────────────────────
template <int NW, int NT>
struct RegsQ8 {
    uint4 a[NT][4];   // 16 rows x 256 codes per tile
    uint4 sc[NT];     // lanes 0-15: row lane's 8 scales of the chunk
    uint4 b[16 / NW];
};

// C[n], Ds[n]: row 0 of tile n's codes (row stride K bytes) and scales (row stride K / 32 halves)
template <int NW, int NT>
__device__ __forceinline__ void load_q8(RegsQ8<NW, NT>& r, const int8_t* const* C, const uint16_t* const* Ds, int K,
                                        const uint8_t* X, int ch, int tid) {
    const int lane = tid & 63;
    const int nb = K >> 5;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int8_t* p = C[n] + (size_t)(lane >> 4) * K + ch * 256 + (lane & 15) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.a[n][i] = ldg_nt(p + (size_t)(4 * i) * K);
        // scales with an ordinary load: a 128-byte line of them serves 8 chunks and must stay in L2 meanwhile
        r.sc[n] = *(const uint4*)(Ds[n] + (size_t)(lane & 15) * nb + ch * 8);
    }
    const uint4* xb = (const uint4*)(X + (size_t)ch * 8 * FRAG_STEP_BYTES);
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) r.b[j] = xb[tid + 64 * NW * j];
}

// alds: the wave's [NT][16 * Q8_PITCH] code tile; slds: its [NT][8][16] scales (transposed: [step][row])
template <int NW, int NT>
__device__ __forceinline__ void stage_q8(const RegsQ8<NW, NT>& r, uint4* alds, uint16_t* slds, uint4* blds, int tid) {
    const int lane = tid & 63;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            alds[n * 16 * Q8_PITCH + (4 * i + (lane >> 4)) * Q8_PITCH + (lane & 15)] = r.a[n][i];
        if (lane < 16) {
            const uint32_t w[4] = {r.sc[n].x, r.sc[n].y, r.sc[n].z, r.sc[n].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                slds[n * 128 + (2 * e) * 16 + lane] = (uint16_t)(w[e] & 0xffffu);
                slds[n * 128 + (2 * e + 1) * 16 + lane] = (uint16_t)(w[e] >> 16);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) blds[tid + 64 * NW * j] = r.b[j];
}

template <int NT>
__device__ __forceinline__ void compute_q8(const uint4* alds, const uint16_t* slds, const uint4* blds,
                                           f32x4_t (&acc)[NT][1], int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 bh = blds[i * 128 + lane], bl = blds[i * 128 + 64 + lane];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const uint2 cv = ((const uint2*)(alds + n * 16 * Q8_PITCH + r * Q8_PITCH))[4 * i + g];
            const bf16x8_t A = as_bf(i8x8_bf16(cv));
            f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf(bh), p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf(bl), p, 0, 0, 0);
            const uint2 sv = *(const uint2*)(slds + n * 128 + i * 16 + 4 * g);
            acc[n][0][0] += f16_to_f32((uint16_t)(sv.x & 0xffffu)) * p[0];
            acc[n][0][1] += f16_to_f32((uint16_t)(sv.x >> 16)) * p[1];
            acc[n][0][2] += f16_to_f32((uint16_t)(sv.y & 0xffffu)) * p[2];
            acc[n][0][3] += f16_to_f32((uint16_t)(sv.y >> 16)) * p[3];
        }
    }
}

}  // namespace ws
