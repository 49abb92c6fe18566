// k_lm.hip — K5: the lm_head GEMM fused with a per-row argmax.
//
// z[t][v] = sum_k X[t][k] E[v][k] over the whole vocabulary, for the T <= 16 rows of one draft, and
// tok[t] = argmax_v z[t][v] (lowest index on ties). The flow-map page runs the target's verify-block matvec
// ("one read of the table") and then argmaxRows over materialised logits; here the logits never leave registers:
//   * the waves of a work-group own adjacent 16-row vocabulary tiles (the A operand of v_mfma_f32_16x16x32_bf16)
//     and walk the k-range in lockstep, streaming the table once from HBM; the 16 draft rows are the MFMA's N, as
//     hi/lo bf16 fragments staged once per work-group in LDS (32 rows of two batched drafts: two 16-row blocks,
//     each weight tile multiplied against both);
//   * the wave's best (value, index) per row is reduced across lanes with shuffles, then across the work-group's
//     waves in LDS, then across work-groups with one 64-bit atomicMax per row on an order-preserving key
//     (value bits, ~index), so ties resolve to the lowest index independent of scheduling;
//   * a one-work-group finalize kernel turns the keys into token ids and clears them for the next call.
// Q8_0 tables (the MTP head's lm_head): each k-step is one Q8_0 block; codes go exactly through the bf16 MFMA and
// the per-row scale multiplies the step's product.
#include "fm_device.h"
#include "fm_kernels.h"

#include <type_traits>

namespace {

__device__ __forceinline__ uint32_t nt32(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint4 ldg_nt(const void* p) {
    const uint32_t* q = (const uint32_t*)p;
    return make_uint4(nt32(q), nt32(q + 1), nt32(q + 2), nt32(q + 3));
}
__device__ __forceinline__ bf16x8_t as_bf(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

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

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Weights are row-staged: each chunk of 8 k-steps (256 columns) of a wave's 16 vocabulary rows is read as 8
// row-contiguous instructions (2 rows x 512 bytes), parked in a wave-private LDS tile and read back in the MFMA A
// layout -- whole cache lines per instruction instead of the A layout's 16 half lines.
constexpr int RS_PITCH = 33;   // uint4 per LDS row: 32 + 1 pad (conflict-free A reads)

// bf16 tables, row-staged weights + work-group-shared activations: the 4 waves of a work-group own 4 adjacent
// 16-row vocabulary tiles and walk the k-range in lockstep, so each chunk's activation fragments (8 k-steps,
// 16 KB) are read from L2 once per work-group (each thread one quarter of it) into a double-buffered LDS slab
// instead of once per wave. Weights and fragments of the next two chunks are in flight while one multiplies.
// NB blocks of 16 rows (bf16 tables): each chunk's fragments of every block go to the slab, block b at b * 1024
// (uint4), and each weight tile is multiplied against every block.
template <int NW, int NB>
struct WsRegs {
    uint4 a[8];             // this wave's 16 rows x 256 columns
    uint4 b[NB * 16 / NW];  // this thread's share of the chunk's fragments
};

template <int NW, int NB>
__device__ __forceinline__ void ws_load(WsRegs<NW, NB>& r, const LmArgs& a, int v0, int ch, int tid) {
    const int lane = tid & 63;
    const uint16_t* E = (const uint16_t*)a.E + (size_t)(v0 + (lane >> 5)) * a.K + ch * 256 + (lane & 31) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.a[i] = ldg_nt(E + (size_t)(2 * i) * a.K);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint4* xb = (const uint4*)(a.X + (size_t)b * a.K * 64 + (size_t)ch * 8 * FRAG_STEP_BYTES);
#pragma unroll
        for (int j = 0; j < 16 / NW; ++j) r.b[b * (16 / NW) + j] = xb[tid + 64 * NW * j];
    }
}

template <int NW, int NB>
__device__ __forceinline__ void ws_stage(const WsRegs<NW, NB>& r, uint4* alds, uint4* blds, int tid) {
    const int lane = tid & 63;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) alds[(2 * i + (lane >> 5)) * RS_PITCH + (lane & 31)] = r.a[i];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 16 / NW; ++j) blds[b * 1024 + tid + 64 * NW * j] = r.b[b * (16 / NW) + j];
}

template <int NB>
__device__ __forceinline__ void ws_compute(const uint4* alds, const uint4* blds, f32x4_t* acc, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 av = alds[r * RS_PITCH + 4 * i + g];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint4 bh = blds[b * 1024 + i * 128 + lane], bl = blds[b * 1024 + i * 128 + 64 + lane];
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(av), as_bf(bh), acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(av), as_bf(bl), acc[b], 0, 0, 0);
        }
    }
}

// Q8_0 tables, same structure: a chunk of 8 k-steps is 8 Q8_0 blocks per row, 256 code bytes (4 rows per
// 1 KB load instruction) and 8 f16 scales per row (one 16-byte load by lanes 0-15). Codes go to a wave-private LDS
// tile and come back as the A operand (8 codes = 8 bytes per lane, widened exactly to bf16); scales go to a
// transposed [step][row] LDS slab so a lane reads its 4 output rows' scales of a step in one 8-byte read; each step's
// product is scaled per row before it is accumulated.
constexpr int Q8_PITCH = 17;   // uint4 per LDS code row: 16 + 1 pad

struct WsRegsQ8 {
    uint4 a[4];   // 16 rows x 256 codes
    uint4 sc;     // lanes 0-15: row lane's 8 scales
    uint4 b[4];
};

template <int NW>
__device__ __forceinline__ void ws_load_q8(WsRegsQ8& r, const LmArgs& a, int v0, int ch, int tid) {
    const int lane = tid & 63;
    const int8_t* C = (const int8_t*)a.E + (size_t)(v0 + (lane >> 4)) * a.K + ch * 256 + (lane & 15) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = ldg_nt(C + (size_t)(4 * i) * a.K);
    const int nb = a.K >> 5;
    // scales with an ordinary load: a 128-byte line of them serves 8 chunks and must stay in L2 meanwhile
    r.sc = *(const uint4*)((const uint16_t*)a.Ed + (size_t)(v0 + (lane & 15)) * nb + ch * 8);
    const uint4* xb = (const uint4*)(a.X + (size_t)ch * 8 * FRAG_STEP_BYTES);
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) r.b[j] = xb[tid + 64 * NW * j];
}

template <int NW>
__device__ __forceinline__ void ws_stage_q8(const WsRegsQ8& r, uint4* alds, uint16_t* slds, uint4* blds, int tid) {
    const int lane = tid & 63;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) alds[(4 * i + (lane >> 4)) * Q8_PITCH + (lane & 15)] = r.a[i];
    if (lane < 16) {
        const uint32_t w[4] = {r.sc.x, r.sc.y, r.sc.z, r.sc.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            slds[(2 * e) * 16 + lane] = (uint16_t)(w[e] & 0xffffu);
            slds[(2 * e + 1) * 16 + lane] = (uint16_t)(w[e] >> 16);
        }
    }
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) blds[tid + 64 * NW * j] = r.b[j];
}

__device__ __forceinline__ void ws_compute_q8(const uint4* alds, const uint16_t* slds, const uint4* blds, f32x4_t& acc,
                                              int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint2 cv = ((const uint2*)(alds + r * Q8_PITCH))[4 * i + g];
        const bf16x8_t A = as_bf(i8x8_bf16(cv));
        const uint4 bh = blds[i * 128 + lane], bl = blds[i * 128 + 64 + lane];
        f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf(bh), p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf(bl), p, 0, 0, 0);
        const uint2 sv = *(const uint2*)(slds + i * 16 + 4 * g);
        acc[0] += f16_to_f32((uint16_t)(sv.x & 0xffffu)) * p[0];
        acc[1] += f16_to_f32((uint16_t)(sv.x >> 16)) * p[1];
        acc[2] += f16_to_f32((uint16_t)(sv.y & 0xffffu)) * p[2];
        acc[3] += f16_to_f32((uint16_t)(sv.y >> 16)) * p[3];
    }
}

// K % 512 == 0 (an even number of chunks), V % 16 == 0 (a tail work-group's extra waves redo the last tile).
// NB = 2 (bf16 only): rows 16 b + t of block b, every weight tile multiplied against both blocks.
template <int WT, int NW, int NB = 1>
__global__ __launch_bounds__(NW * 64) void lm_argmax_ws_kernel(LmArgs a) {
    static_assert(NB == 1 || WT == 0, "two row blocks: bf16 tables only");
    constexpr int APITCH = WT == 0 ? RS_PITCH : Q8_PITCH;
    __shared__ uint4 alds_all[NW][16 * APITCH];
    __shared__ uint16_t slds_all[NW][8 * 16];
    __shared__ uint4 blds_all[2][NB * 1024];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4;
    const int v0 = min((blockIdx.x * NW + wave) * 16, a.V - 16);   // tail waves redo the last tile (discarded)
    const bool own = (blockIdx.x * NW + wave) * 16 < a.V;
    uint4* alds = alds_all[wave];
    uint16_t* slds = slds_all[wave];
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nch = a.K >> 8;
    using Regs = typename std::conditional<WT == 0, WsRegs<NW, NB>, WsRegsQ8>::type;
    auto load = [&](Regs& r, int ch) {
        if constexpr (WT == 0) ws_load<NW, NB>(r, a, v0, ch, tid);
        else ws_load_q8<NW>(r, a, v0, ch, tid);
        // each chunk's loads stay together, in the prologue as in the loop: the wait before a chunk is staged is
        // the stricter of the loop header's two entries, and a prologue that interleaves the two chunks' loads
        // makes it wait for the next chunk's loads as well (vmcnt(1) instead of vmcnt(12))
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage = [&](const Regs& r, int buf) {
        if constexpr (WT == 0) ws_stage<NW, NB>(r, alds, blds_all[buf], tid);
        else ws_stage_q8<NW>(r, alds, slds, blds_all[buf], tid);
    };
    auto compute = [&](int buf) {
        if constexpr (WT == 0) ws_compute<NB>(alds, blds_all[buf], acc, lane);
        else ws_compute_q8(alds, slds, blds_all[buf], acc[0], lane);
    };
    Regs r0, r1;
    load(r0, 0);
    load(r1, 1);
    int ch = 0;
    for (; ch + 2 < nch; ch += 2) {
        stage(r0, 0);
        load(r0, ch + 2);
        __syncthreads();
        compute(0);
        stage(r1, 1);
        load(r1, ch + 3);
        __syncthreads();
        compute(1);
    }
    stage(r0, 0);
    __syncthreads();
    compute(0);
    stage(r1, 1);
    __syncthreads();
    compute(1);

    // lane holds z[row 16 b + lane % 16][v0 + 4 g + j] of block b
    __shared__ float wb[NW][NB * 16];
    __shared__ int wi[NW][NB * 16];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int t = 16 * b + (lane & 15);
        float best = -INFINITY;
        int bidx = 0x7fffffff;
        if (own) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int v = v0 + 4 * g + j;
                const float z = acc[b][j];
                if (a.logits && t < a.T) a.logits[(size_t)t * a.V + v] = z;
                if (z > best) { best = z; bidx = v; }
            }
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            const float ob = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bidx, o, 64);
            if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
        }
        if (lane < 16) { wb[wave][16 * b + lane] = best; wi[wave][16 * b + lane] = bidx; }
    }
    __syncthreads();
    if (tid < NB * 16 && tid < a.T) {
        float b = wb[0][tid];
        int bi = wi[0][tid];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            if (wb[w][tid] > b || (wb[w][tid] == b && wi[w][tid] < bi)) { b = wb[w][tid]; bi = wi[w][tid]; }
        if (bi != 0x7fffffff) {
            const unsigned long long key = ((unsigned long long)order_key(b) << 32) | (0xffffffffu - (uint32_t)bi);
            atomicMax(&a.best[tid], key);
        }
    }
}

__global__ void lm_finalize_kernel(unsigned long long* best, int T, int32_t* tokens) {
    const int t = threadIdx.x;
    if (t < T) {
        const unsigned long long k = best[t];
        tokens[t] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
        best[t] = 0ull;
    }
}

}  // namespace

hipError_t launch_lm_argmax(const LmArgs& a, int wtype, hipStream_t st) {
    // rows of a multiple of 512 (an even number of 8-step chunks) and whole 16-row vocabulary tiles; more than 16
    // activation rows (two blocks) on bf16 tables only
    if (a.T < 1 || a.T > 32 || (a.T > 16 && wtype != 0) || a.K % 512 || a.V % 16) return hipErrorInvalidValue;
    if (wtype == 0 && a.T > 16) lm_argmax_ws_kernel<0, 8, 2><<<(a.V + 127) / 128, 512, 0, st>>>(a);
    else if (wtype == 0) lm_argmax_ws_kernel<0, 4><<<(a.V + 63) / 64, 256, 0, st>>>(a);
    else lm_argmax_ws_kernel<1, 8><<<(a.V + 127) / 128, 512, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lm_finalize_kernel<<<1, 64, 0, st>>>(a.best, a.T, a.tokens);
    return hipGetLastError();
}
