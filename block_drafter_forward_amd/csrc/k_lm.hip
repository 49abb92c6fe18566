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
#include "fm_ws.h"

#include <type_traits>

namespace {

using ws::as_bf;

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// K % 512 == 0 (an even number of chunks), V % 16 == 0 (a tail work-group's extra waves redo the last tile).
// NB = 2 (bf16 only): rows 16 b + t of block b, every weight tile multiplied against both blocks.
template <int WT, int NW, int NB = 1>
__global__ __launch_bounds__(NW * 64) void lm_argmax_ws_kernel(LmArgs a) {
    static_assert(NB == 1 || WT == 0, "two row blocks: bf16 tables only");
    constexpr int APITCH = WT == 0 ? ws::RS_PITCH : ws::Q8_PITCH;
    __shared__ uint4 alds_all[NW][16 * APITCH];
    __shared__ uint16_t slds_all[NW][8 * 16];
    __shared__ uint4 blds_all[2][NB * 1024];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4;
    const int v0 = min((blockIdx.x * NW + wave) * 16, a.V - 16);   // tail waves redo the last tile (discarded)
    const bool own = (blockIdx.x * NW + wave) * 16 < a.V;
    uint4* alds = alds_all[wave];
    uint16_t* slds = slds_all[wave];
    f32x4_t acc[1][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[0][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nch = a.K >> 8;
    const uint16_t* const Wt[1] = {(const uint16_t*)a.E + (size_t)v0 * a.K};
    const int8_t* const Ct[1] = {(const int8_t*)a.E + (size_t)v0 * a.K};
    const uint16_t* const Dt[1] = {a.Ed ? (const uint16_t*)a.Ed + (size_t)v0 * (a.K >> 5) : nullptr};
    using Regs = typename std::conditional<WT == 0, ws::Regs<NW, 1, NB>, ws::RegsQ8<NW, 1>>::type;
    auto load = [&](Regs& r, int ch) {
        if constexpr (WT == 0) ws::load<NW, 1, NB>(r, Wt, a.K, a.X, ch, tid);
        else ws::load_q8<NW, 1>(r, Ct, Dt, a.K, a.X, ch, tid);
        // each chunk's loads stay together, in the prologue as in the loop: the wait before a chunk is staged is
        // the stricter of the loop header's two entries, and a prologue that interleaves the two chunks' loads
        // makes it wait for the next chunk's loads as well (vmcnt(1) instead of vmcnt(12))
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage = [&](const Regs& r, int buf) {
        if constexpr (WT == 0) ws::stage<NW, 1, NB>(r, alds, blds_all[buf], tid);
        else ws::stage_q8<NW, 1>(r, alds, slds, blds_all[buf], tid);
    };
    auto compute = [&](int buf) {
        if constexpr (WT == 0) ws::compute<1, NB>(alds, blds_all[buf], acc, lane);
        else ws::compute_q8<1>(alds, slds, blds_all[buf], acc, lane);
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
                const float z = acc[0][b][j];
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
