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
// the per-row scale multiplies the step's product. The table is streamed from a copy in the MFMA operand layout
// (q8_tile_copy_kernel, made once at create), so codes go from HBM straight into the registers that feed the matrix
// cores: no LDS staging of the weights, only of the activation fragments.
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

// bf16 tables. K % 512 == 0 (an even number of chunks), V % 16 == 0 (a tail work-group's extra waves redo the last
// tile). NB = 2: rows 16 b + t of block b, every weight tile multiplied against both blocks.
template <int NW, int NB = 1>
__global__ __launch_bounds__(NW * 64) void lm_argmax_ws_kernel(LmArgs a) {
    __shared__ uint4 alds_all[NW][16 * ws::RS_PITCH];
    __shared__ uint4 blds_all[2][NB * 1024];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4;
    const int v0 = min((blockIdx.x * NW + wave) * 16, a.V - 16);   // tail waves redo the last tile (discarded)
    const bool own = (blockIdx.x * NW + wave) * 16 < a.V;
    uint4* alds = alds_all[wave];
    f32x4_t acc[1][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[0][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nch = a.K >> 8;
    const uint16_t* const Wt[1] = {(const uint16_t*)a.E + (size_t)v0 * a.K};
    using Regs = ws::Regs<NW, 1, NB>;
    auto load = [&](Regs& r, int ch) {
        ws::load<NW, 1, NB>(r, Wt, a.K, a.X, ch, tid);
        // each chunk's loads stay together, in the prologue as in the loop: the wait before a chunk is staged is
        // the stricter of the loop header's two entries, and a prologue that interleaves the two chunks' loads
        // makes it wait for the next chunk's loads as well (vmcnt(1) instead of vmcnt(12))
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage = [&](const Regs& r, int buf) { ws::stage<NW, 1, NB>(r, alds, blds_all[buf], tid); };
    auto compute = [&](int buf) { ws::compute<1, NB>(alds, blds_all[buf], acc, lane); };
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

// Q8_0 tables in the MFMA operand layout (q8_tile_copy_kernel): a wave owns one 16-row vocabulary tile and walks
// the k-range in chunks of 256 columns (8 Q8_0 blocks), two chunks in flight. Per chunk a lane loads the 64 bytes
// of codes it multiplies (four 16-byte loads, each instruction 1 KB contiguous) and the 8 scales of its row; the
// chunk's activation fragments go through a double-buffered LDS slab shared by the work-group's 4 waves. The
// fragments are the MFMA's A operand and the codes its B operand, so a lane's output column is its own code row and
// each step's scale is one of the lane's own 8. Three work-groups per CU (at most 168 VGPRs). The MTP head's
// 248320 x 5120 table: 303 us per call row-major and staged through LDS (8 waves, one work-group per CU); from the
// copy, 267 us with three chunks in flight and two work-groups per CU, 252 us with two chunks and three.
constexpr int LMQ_NW = 4, LMQ_ST = 2;

__global__ __launch_bounds__(LMQ_NW * 64, 3) void lm_argmax_q8t_kernel(LmArgs a) {
    constexpr int NW = LMQ_NW, ST = LMQ_ST;
    __shared__ uint4 blds_all[2][1024];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int tile = blockIdx.x * NW + wave;
    const int v0 = min(tile * 16, a.V - 16);   // tail waves redo the last tile (discarded)
    const bool own = tile * 16 < a.V;
    const int nch = a.K >> 8;
    const uint8_t* Tq = (const uint8_t*)a.E + (size_t)(v0 >> 4) * nch * 4096 + lane * 16;
    const uint16_t* Ts = (const uint16_t*)a.Ed + (size_t)(v0 >> 4) * nch * 128 + r * 8;
    struct Regs {
        uint4 c[4];            // codes of steps 2i, 2i + 1 (8 each) in c[i]
        uint4 s;               // the row's 8 scales
        uint4 b[16 / NW];      // this thread's share of the chunk's fragments
    };
    auto load = [&](Regs& q, int ch) {   // nothing past the last chunk (a uniform branch)
        if (ch < nch) {
            const uint8_t* p = Tq + (size_t)ch * 4096;
#pragma unroll
            for (int i = 0; i < 4; ++i) q.c[i] = ws::ldg_nt(p + i * 1024);
            q.s = *(const uint4*)(Ts + (size_t)ch * 128);
            const uint4* xb = (const uint4*)(a.X + (size_t)ch * 8 * FRAG_STEP_BYTES);
#pragma unroll
            for (int j = 0; j < 16 / NW; ++j) q.b[j] = xb[tid + 64 * NW * j];
        }
        __builtin_amdgcn_sched_barrier(0);   // each chunk's loads stay together (one wait per chunk)
    };
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // chunk c's fragments go to slab c % 2: written after the barrier that follows the multiply of chunk c - 2
    auto step = [&](const Regs& q, int ch) {
        uint4* blds = blds_all[ch & 1];
#pragma unroll
        for (int j = 0; j < 16 / NW; ++j) blds[tid + 64 * NW * j] = q.b[j];
        __syncthreads();
        const uint32_t sw[4] = {q.s.x, q.s.y, q.s.z, q.s.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 xh = blds[i * 128 + lane], xl = blds[i * 128 + 64 + lane];
            const uint4 cc = q.c[i >> 1];
            const bf16x8_t B = as_bf(ws::i8x8_bf16((i & 1) ? make_uint2(cc.z, cc.w) : make_uint2(cc.x, cc.y)));
            f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(xh), B, p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(xl), B, p, 0, 0, 0);
            const float sc = f16_to_f32((uint16_t)((i & 1) ? (sw[i >> 1] >> 16) : (sw[i >> 1] & 0xffffu)));
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += sc * p[j];
        }
    };
    Regs q[ST];
#pragma unroll
    for (int u = 0; u < ST; ++u) load(q[u], u);
    int ch = 0;
    for (; ch + ST <= nch; ch += ST) {
#pragma unroll
        for (int u = 0; u < ST; ++u) {
            step(q[u], ch + u);
            load(q[u], ch + u + ST);
        }
    }
#pragma unroll
    for (int u = 0; u < ST - 1; ++u)
        if (ch + u < nch) step(q[u], ch + u);

    // lane holds z[row 4 g + j][v0 + r]: each row's best over the tile's 16 columns, then over the waves
    __shared__ float wb[NW][16];
    __shared__ int wi[NW][16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * g + j;
        float best = -INFINITY;
        int bidx = 0x7fffffff;
        if (own) {
            best = acc[j];
            bidx = v0 + r;
            if (a.logits && t < a.T) a.logits[(size_t)t * a.V + v0 + r] = acc[j];
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const float ob = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bidx, o, 64);
            if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
        }
        if (r == 0) { wb[wave][t] = best; wi[wave][t] = bidx; }
    }
    __syncthreads();
    if (tid < 16 && tid < a.T) {
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

// The MFMA operand layout of a Q8_0 table [M][K] (codes) + [M][K / 32] (f16 scales), M % 16 == 0, K % 256 == 0:
// for 16-row tile t and 256-column chunk c (nch = K / 256 chunks per row), at byte 4096 (t nch + c) of the codes,
// 4 pieces of 1 KB; in piece i, lane l = r + 16 g (r < 16, g < 4) holds 16 bytes: columns 256 c + 64 i + 8 g ... + 7
// of row 16 t + r, then the same 8 columns 32 further on (k-steps 2i and 2i + 1 of the chunk, k-group g). The
// scales at half 128 (t nch + c) + 8 r + s: row 16 t + r, Q8_0 block 8 c + s. One thread per 16 bytes of codes.
__global__ void q8_tile_copy_kernel(const int8_t* q, const uint16_t* d, int M, int K, uint8_t* oq, uint16_t* od) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int nch = K >> 8;
    if (i < (size_t)M * K / 16) {
        const int l = (int)(i & 63), pi = (int)((i >> 6) & 3);
        const size_t tc = i >> 8, t = tc / nch;
        const int c = (int)(tc - t * nch);
        const int8_t* src = q + (16 * t + (l & 15)) * (size_t)K + 256 * c + 64 * pi + 8 * (l >> 4);
        const uint2 lo = *(const uint2*)src, hi = *(const uint2*)(src + 32);
        *(uint4*)(oq + 16 * i) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    if (i < (size_t)M * nch) {   // (t, c, r): the row's 8 scales of the chunk
        const int r = (int)(i & 15);
        const size_t tc = i >> 4, t = tc / nch;
        const int c = (int)(tc - t * nch);
        const uint16_t* src = d + (16 * t + r) * (size_t)(K >> 5) + 8 * c;
#pragma unroll
        for (int e = 0; e < 8; ++e) od[8 * i + e] = src[e];
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
    if (wtype == 0 && a.T > 16) lm_argmax_ws_kernel<8, 2><<<(a.V + 127) / 128, 512, 0, st>>>(a);
    else if (wtype == 0) lm_argmax_ws_kernel<4><<<(a.V + 63) / 64, 256, 0, st>>>(a);
    else lm_argmax_q8t_kernel<<<(a.V + 16 * LMQ_NW - 1) / (16 * LMQ_NW), 64 * LMQ_NW, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lm_finalize_kernel<<<1, 64, 0, st>>>(a.best, a.T, a.tokens);
    return hipGetLastError();
}

hipError_t launch_q8_tile_copy(const int8_t* q, const uint16_t* d, int M, int K, uint8_t* oq, uint16_t* od,
                               hipStream_t st) {
    if (M < 16 || M % 16 || K < 256 || K % 256 || ((uintptr_t)q & 7) || ((uintptr_t)oq & 15) || ((uintptr_t)od & 15))
        return hipErrorInvalidValue;
    const size_t n = (size_t)M * K / 16;
    q8_tile_copy_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(q, d, M, K, oq, od);
    return hipGetLastError();
}
