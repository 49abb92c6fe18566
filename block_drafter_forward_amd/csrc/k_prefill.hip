// k_prefill.hip — K2: the MFMA GEMM of context prefill, C[r][n] = sum_k A[r][k] B[n][k].
//
// The one truly dense contraction of the path: the fusion of many context rows (fc / W_c over the concatenated
// taps, flashmap_drafter.js extendContext; module-dflash.ts #buildContext) and the per-layer K/V projections of the
// fused rows. Operands are f16 on v_mfma_f32_16x16x32_f16 with f32 accumulation: each row of f32 taps is scaled by a
// power of two that brings its largest magnitude into [2^14, 2^15) and rounded to f16 (2^-11 relative, four times
// finer than bf16; the scale is exact and undone on the f32 output row, so f16's range never limits the taps), bf16
// weights are widened to f16 exactly (up to f16's subnormal range, |error| <= 2^-25).
//
// Large problems (at least one 256 x 256 tile per CU) run prefill_dma_kernel: A and B are both f16 in HBM (the
// weights converted once when the drafter is created, the taps by the scaling pass before the product) and are streamed
// into LDS by the LDS-direct load (global_load_lds_dwordx4: no registers, no conversion on the way). A k-stage is 64
// k-values, so every row slice a load touches is one whole 128-byte line (measured: half-line slices moved half the
// bytes per second); in LDS a row is 8 chunks of 16 bytes with chunk c at slot c ^ (row & 7), which makes the
// 16 x 32 fragment reads conflict-free (measured with a read microbenchmark: 4 LDS cycles per 1 KB read). Two stage
// buffers (128 KB); 8 waves as 2 x 4 of 128 x 64; each wave reads the fragments of the next 32-k substep while the
// current one multiplies, so one barrier per stage is the only synchronisation.
// Small problems run prefill_kernel: 128 x 128 tiles of 4 waves, operands staged through registers (f16 rows, bf16
// weights widened on the way into LDS), two k-stages of loads in flight.
// Work-groups are remapped so each XCD owns a contiguous run of tiles, taken 8 row tiles at a time (the 8 row
// tiles of a group share B tiles and each A tile is shared by the group's column tiles, in that XCD's L2).
// Epilogues: f32 rows; a cache store (f16 / f32) at rows start + r, or into the f16 V cache's 32-position tiles
// (dimension-major inside a tile: 8-byte stores of 4 consecutive positions); or, for K, the per-head RMSNorm over the
// tile's columns (a head is 64 or 128 columns of the 256-wide tile) and interleaved RoPE at position start + r before
// the store -- the page's headNormRope + kvWrite, fused.
#include <algorithm>
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

// LDS row pitch of prefill_kernel's tiles (halves): 112 bytes. Measured against the other 16-byte-aligned pitches
// (80, 96, 144 bytes with two work-groups per CU): 80 bytes, the obvious padding, left the kernel at 5.4 LDS bank-
// conflict cycles per LDS instruction, and the 512-row FlashMap prefill took 255 us against 197 us at 112 bytes
// (the 2048-row KV-injection prefill 260 against 228 us).
constexpr int BK = 32, LDP = BK + 24;

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16);
}

// LDS-direct load of 16 bytes per lane: lane l's 16 bytes from g land at LDS byte lds + 16 l (lds is wave-uniform,
// passed in m0). Written as inline asm so that the compiler's wait bookkeeping leaves it alone: it cannot tell the
// two stage buffers apart and would otherwise wait for every load in flight before any LDS read; the kernel waits
// for these loads explicitly (wait_vm). Nothing else in the kernel uses m0.
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
    const unsigned la =
        __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)((__attribute__((address_space(3))) void*)lds));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory", "m0");
}

// s_waitcnt with vmcnt = n and the other counters at their maxima (gfx9 encoding), and with lgkmcnt = 0 only
template <int N> __device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// v[q] = C[row q][column c0 + t] on lane t of a quad (t = lane % 4) -> o[c] = C[row t][column c0 + c]: two
// exchanges between lane pairs (lane ^ 1, then lane ^ 2) by DPP quad permutations.
__device__ __forceinline__ float quad_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
}
// sum over the 16 lanes of a DPP row: pairs, quads, then the two mirrors
__device__ __forceinline__ float row16_sum(float s) {
    s += quad_xor1(s);
    s += quad_xor2(s);
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x141, 0xF, 0xF, true));
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x140, 0xF, 0xF, true));
    return s;
}
__device__ __forceinline__ void quad_transpose(const f32x4_t& v, int t, float (&o)[4]) {
    const bool odd = t & 1, hi = t & 2;
    // step 1: even lanes keep rows 0 and 2 and take the odd neighbour's (column + 1) values of those rows; odd lanes
    // keep rows 1 and 3 and take the even neighbour's (column - 1) values
    const float s0 = quad_xor1(odd ? v[0] : v[1]), s1 = quad_xor1(odd ? v[2] : v[3]);
    const float a0 = odd ? s0 : v[0], a1 = odd ? v[1] : s0;   // row t & 1, columns 2 (t >> 1) + 0, 1
    const float b0 = odd ? s1 : v[2], b1 = odd ? v[3] : s1;   // row (t & 1) + 2, same columns
    // step 2: lanes t and t ^ 2 complete one row each: row t & 1 for t < 2, row (t & 1) + 2 for t >= 2
    const float u0 = quad_xor2(hi ? a0 : b0), u1 = quad_xor2(hi ? a1 : b1);
    if (hi) { o[0] = u0; o[1] = u1; o[2] = b0; o[3] = b1; }
    else    { o[0] = a0; o[1] = a1; o[2] = u0; o[3] = u1; }
}

// acc[i][j][q] = C[r0 + wm*16*TI + 16 i + 4 (lane/16) + q][n0 + wn*64 + 16 j + lane%16]
// stage: null, or T * T * 2 bytes of LDS that no wave reads or loads into any more (f16 row tiles go out through it)
template <int T, int TI, int TJ, int NWN, bool STAGED>
__device__ __forceinline__ void prefill_epilogue(f32x4_t (&acc)[TI][TJ], const PrefillArgs& a, const PrefillGroup& G,
                                                 int r0, int n0, int wm, int wn, int lane, float (&nred)[NWN][T],
                                                 uint8_t* stage) {
    const int rq = 4 * (lane >> 4), cl = lane & 15;
    if (G.epi == PF_CACHE_K && G.knorm) {
        const int hd = a.hd;
        // with LDS to spare, the tile's T table rows (consecutive positions, T * hd floats <= T * T * 2 bytes) are
        // copied in one batch of loads instead of 4 * TI dependent rounds of loads from L2
        if constexpr (STAGED) {
            // one wave instruction moves 1 KB = 1024 / (4 hd) table rows; lane l takes 16 bytes of row l / (hd / 4)
            const int wave = threadIdx.x >> 6, rpi = 256 / hd, c16 = hd / 4;
            const int nins = T * hd * 4 / 1024, nw = blockDim.x >> 6;
            for (int ins = wave; ins < nins; ins += nw) {
                const int rl = ins * rpi + lane / c16, k = lane % c16;
                const int pos = a.start + min(r0 + rl, a.rows - 1);
                lds_load16(a.rope_pf + (size_t)pos * hd + 4 * k, stage + ins * 1024);
            }
            wait_vm<0>();
            __syncthreads();
        }
        const float* rtab = STAGED ? (const float*)stage : a.rope_pf;
        float ssq[TI][4];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < TJ; ++j) s += acc[i][j][q] * acc[i][j][q];
                ssq[i][q] = row16_sum(s);
            }
        if (hd == 128) {   // a head spans two waves along n
            if (cl == 0) {
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) nred[wn][wm * TI * 16 + 16 * i + rq + q] = ssq[i][q];
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rl = wm * TI * 16 + 16 * i + rq + q;
                    ssq[i][q] = nred[wn & ~1][rl] + nred[wn | 1][rl];
                }
        }
        // RoPE from the prefill copy of the table (rope_pf): per position, per 32-pair block b, per c = 0..7 the cos
        // then the sin of pairs 32 b + c + 8 j, j = 0..3 -- exactly this lane's four columns, two 16-byte loads per row
        const int dbase = (n0 + wn * 64) % hd;   // 0 or 64
        const int nb = hd / 64;
        float kw[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) kw[j] = bf16_to_f32(G.knorm[dbase + 16 * j + cl]);
        const float inv_hd = 1.f / (float)hd;
        const bool odd = cl & 1;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + wm * TI * 16 + 16 * i + rq + q;
                // v_rsq_f32 (~1 ulp): far below the f16 rounding of the cached K; 1 / hd is exact (hd = 64 or 128)
                const float rs = __builtin_amdgcn_rsqf(ssq[i][q] * inv_hd + a.eps);
                const size_t trow = STAGED ? (size_t)(r - r0) : (size_t)a.start + (r < a.rows ? r : 0);
                const float* tp = rtab + ((trow * nb + dbase / 64) * 8 + (cl >> 1)) * 8;
                const float4 cs = *(const float4*)tp, sn = *(const float4*)(tp + 4);
                const float cj[4] = {cs.x, cs.y, cs.z, cs.w}, sj[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const float v = acc[i][j][q] * rs * kw[j];
                    const float pv = quad_xor1(v);   // the other element of the pair (columns 2m, 2m + 1)
                    acc[i][j][q] = odd ? v * cj[j] + pv * sj[j] : v * cj[j] - pv * sj[j];
                }
            }
    }
    if (G.epi == PF_CACHE_VT) {   // a lane's 4 consecutive rows are 4 consecutive positions of one V dimension
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int rb = r0 + wm * TI * 16 + 16 * i + rq;
            const int pb = a.start + rb;
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int n = n0 + wn * 64 + 16 * j + cl;
                uint16_t* dst = (uint16_t*)G.out + ((size_t)(pb >> 5) * a.vt_ld + n) * 32 + (pb & 31);
                if (rb + 3 < a.rows && (pb & 3) == 0) {   // the 4 positions share a 32-position tile
                    *(uint2*)dst = make_uint2((uint32_t)f32_to_f16(acc[i][j][0]) | ((uint32_t)f32_to_f16(acc[i][j][1]) << 16),
                                              (uint32_t)f32_to_f16(acc[i][j][2]) | ((uint32_t)f32_to_f16(acc[i][j][3]) << 16));
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (rb + q < a.rows)
                            ((uint16_t*)G.out)[((size_t)((pb + q) >> 5) * a.vt_ld + n) * 32 + ((pb + q) & 31)] =
                                f32_to_f16(acc[i][j][q]);
                }
            }
        }
        return;
    }
    // Row stores: a 4 x 4 transpose inside each quad of lanes turns "4 rows of one column" into "4 consecutive
    // columns of one row", so each lane writes one 8-byte (f16) or 16-byte (f32) piece instead of four 2- or 4-byte
    // ones (measured: 2-byte stores made the K/V projection 25% slower than 8-byte ones).
    const int t = cl & 3, cq = cl & ~3;
    if (STAGED && G.epi != PF_F32 && a.kv_dtype == 0) {
        if (G.epi == PF_CACHE_K && G.knorm) __syncthreads();   // every wave is done with the table rows in LDS
        // f16 rows: the tile goes through LDS (row rl at rl * 2T bytes, 16-byte chunk k at slot k ^ (rl % 32)) and
        // out as whole row segments, 16 bytes per lane (measured: 32-byte pieces of rows 4 KB apart wrote slower than
        // the V cache's contiguous tiles)
        constexpr int RB = 2 * T, NCH = T / 8;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                float o[4];
                quad_transpose(acc[i][j], t, o);
                const int rl = wm * TI * 16 + 16 * i + rq + t, cl4 = wn * 64 + 16 * j + cq;
                *(uint2*)(stage + rl * RB + (((cl4 >> 3) ^ (rl & 31)) << 4) + ((cl4 >> 2) & 1) * 8) =
                    make_uint2(pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3]));
            }
        __syncthreads();
        for (int c = threadIdx.x; c < T * NCH; c += blockDim.x) {
            const int rl = c / NCH, k = c % NCH, r = r0 + rl;
            if (r < a.rows)
                *(uint4*)((uint16_t*)G.out + (size_t)(a.start + r) * a.ld + n0 + 8 * k) =
                    *(const uint4*)(stage + rl * RB + ((k ^ (rl & 31)) << 4));
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            float o[4];
            quad_transpose(acc[i][j], t, o);
            const int r = r0 + wm * TI * 16 + 16 * i + rq + t;
            const int n = n0 + wn * 64 + 16 * j + cq;
            if (r >= a.rows) continue;
            if (G.epi == PF_F32) {
                *(float4*)((float*)G.out + (size_t)r * a.ld + n) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
                const size_t off = (size_t)(a.start + r) * a.ld + n;
                if (a.kv_dtype == 0)
                    *(uint2*)((uint16_t*)G.out + off) = make_uint2(pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3]));
                else
                    *(float4*)((float*)G.out + off) = make_float4(o[0], o[1], o[2], o[3]);
            }
        }
}

// Tile T x T (T = 128: 4 waves as 2 x 2 of 64 x 64; T = 256: 8 waves as 2 x 4 of 128 x 64). Every thread stages
// 16 k-values of one f16 A row and one B row per k-stage; rows past the end of A are clamped (their results dropped).
// Two work-groups per CU (2 waves per SIMD, <= 256 registers a wave): without the bound the compiler keeps the
// accumulators in AGPRs next to 151 VGPRs and the kernel runs at one wave per SIMD, 25% slower.
template <int T>
__global__ __launch_bounds__(T * 2, 2) void prefill_kernel(PrefillArgs a) {
    constexpr int BM = T, BN = T, NWN = T / 64, TI = T == 128 ? 4 : 8, TJ = 4;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDP];
    __shared__ float nred[NWN][BM];

    int lin = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    // k split over work-groups: split s takes k in [s K / ksplit, (s + 1) K / ksplit) of every tile
    const int ks = a.ksplit > 1 ? a.ksplit : 1;
    const int split = lin / (total / ks);
    lin -= split * (total / ks);
    int gi = 0;
#pragma unroll 1
    for (int i = 1; i < a.ngroups; ++i)
        if (lin >= a.g[i].tile_begin) gi = i;
    PrefillGroup G = a.g[gi];
    if (ks > 1) G.out = (float*)G.out + (size_t)split * a.slab_stride;
    const int local = lin - G.tile_begin;
    const int mt = local / a.n_tiles, nt = local - mt * a.n_tiles;
    const int r0 = mt * BM, n0 = nt * BN;
    const void* Ap = G.A ? G.A : a.A;
    const int K = a.K;               // row stride of A and B
    const int kb = split * (K / ks);  // first k of this split

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / NWN, wn = wave % NWN;
    const int ldrow = tid >> 1, kofs = (tid & 1) * 16;
    const int arow = min(r0 + ldrow, a.rows - 1);

    struct PStage {
        uint4 rah[2], rb[2];
    };
    auto gload = [&](PStage& r, int kt) {
        const int k = kb + kt * BK + kofs;
        const uint4* p = (const uint4*)((const uint16_t*)Ap + (size_t)arow * K + k);
        r.rah[0] = p[0];
        r.rah[1] = p[1];
        const uint4* pb = (const uint4*)(G.B + (size_t)(n0 + ldrow) * K + k);
        r.rb[0] = pb[0];
        r.rb[1] = pb[1];
    };
    auto lstore = [&](const PStage& r, int buf) {
        *(uint4*)&As[buf][ldrow][kofs] = r.rah[0];
        *(uint4*)&As[buf][ldrow][kofs + 8] = r.rah[1];
        uint32_t w[8] = {r.rb[0].x, r.rb[0].y, r.rb[0].z, r.rb[0].w, r.rb[1].x, r.rb[1].y, r.rb[1].z, r.rb[1].w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = pack_f16x2(bf16_lo(w[i]), bf16_hi(w[i]));
        *(uint4*)&Bs[buf][ldrow][kofs] = make_uint4(o[0], o[1], o[2], o[3]);
        *(uint4*)&Bs[buf][ldrow][kofs + 8] = make_uint4(o[4], o[5], o[6], o[7]);
    };

    f32x4_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15, fk = 8 * (lane >> 4);
    auto mma = [&](int buf) {
        f16x8_t af[TI], bfr[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) af[i] = as_f16x8(*(const uint4*)&As[buf][wm * (TI * 16) + i * 16 + fr][fk]);
#pragma unroll
        for (int j = 0; j < TJ; ++j) bfr[j] = as_f16x8(*(const uint4*)&Bs[buf][wn * 64 + j * 16 + fr][fk]);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };

    // two k-stages in flight in registers while one multiplies from LDS; past the end a stage re-reads the
    // last one (no conditional load)
    const int nk = K / ks / BK;
    PStage s0, s1;
    gload(s0, 0);
    gload(s1, min(1, nk - 1));
    lstore(s0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        gload(s0, min(kt + 2, nk - 1));
        mma(0);
        lstore(s1, 1);
        __syncthreads();
        if (kt + 1 >= nk) break;
        gload(s1, min(kt + 3, nk - 1));
        mma(1);
        lstore(s0, 0);
        __syncthreads();
    }

    prefill_epilogue<T, TI, TJ, NWN, false>(acc, a, G, r0, n0, wm, wn, lane, nred, nullptr);
}

// ── 256 x 256 tiles from f16 operands, LDS-direct loads ──────────────────────────────────────────────────────────

// A bare s_barrier: __syncthreads() adds a release fence, which makes the compiler wait for every LDS-direct load in
// flight (vmcnt(0)) and would serialise the pipeline; the waits this kernel needs are explicit.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

template <int GM>
__global__ __launch_bounds__(512) void prefill_dma_kernel(PrefillArgs a) {
    constexpr int TI = 8, TJ = 4, NWN = 4;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][256 * 128];   // [stage][A | B][row][128 B]
    __shared__ float nred[NWN][256];

    const int total = gridDim.x;
    int lin = blockIdx.x;
    if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    int gi = 0;
#pragma unroll 1
    for (int i = 1; i < a.ngroups; ++i)
        if (lin >= a.g[i].tile_begin) gi = i;
    const PrefillGroup& G = a.g[gi];
    const int local = lin - G.tile_begin;
    const int grp = local / (GM * a.n_tiles);
    const int gm = min(GM, a.m_tiles - grp * GM);
    const int within = local - grp * GM * a.n_tiles;
    const int mt = grp * GM + within % gm, nt = within / gm;
    const int r0 = mt * 256, n0 = nt * 256;
    const uint16_t* Ap = (const uint16_t*)(G.A ? G.A : a.A);
    const int K = a.K;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 2, wn = wave & 3;
    // loads: wave w fills rows 32w .. 32w + 31 of the A and the B tile, 8 rows (1 KB of LDS) per instruction; lane l
    // takes row l / 8 of those 8 and writes LDS slot l % 8 of it, which holds chunk (l % 8) ^ (l / 8)
    const int lrow = lane >> 3, lch = (lane & 7) ^ lrow;
    const uint16_t* ga[4];
    const uint16_t* gb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ga[i] = Ap + (size_t)min(r0 + 32 * wave + 8 * i + lrow, a.rows - 1) * K + 8 * lch;
        gb[i] = G.B16 + (size_t)(n0 + 32 * wave + 8 * i + lrow) * K + 8 * lch;
    }
    auto issue = [&](int s, int buf) {
        const int k0 = s * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lds_load16(ga[i] + k0, &lds[buf][0][(32 * wave + 8 * i) * 128]);
            lds_load16(gb[i] + k0, &lds[buf][1][(32 * wave + 8 * i) * 128]);
        }
    };
    // fragment of k-half h: row l % 16 of a 16-row block, chunk 4h + l / 16, at slot chunk ^ (row & 7)
    const int fr = lane & 15, fq = lane >> 4;
    const int fo0 = fr * 128 + 16 * (fq ^ (fr & 7)), fo1 = fr * 128 + 16 * ((4 + fq) ^ (fr & 7));
    f32x4_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f16x8_t fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];
    auto rd = [&](f16x8_t* fa, f16x8_t* fb, int buf, int fo) {
#pragma unroll
        for (int i = 0; i < TI; ++i) fa[i] = *(const f16x8_t*)&lds[buf][0][(wm * 128 + 16 * i) * 128 + fo];
#pragma unroll
        for (int j = 0; j < TJ; ++j) fb[j] = *(const f16x8_t*)&lds[buf][1][(wn * 64 + 16 * j) * 128 + fo];
    };
    auto mm = [&](const f16x8_t* fa, const f16x8_t* fb) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    // Stage s lives in buffer s % 2. Iteration s: read substep 1's fragments of stage s, multiply substep 0; wait
    // until this wave's reads are done and stage s + 1 has landed, barrier (now every wave is done with buffer s % 2
    // and stage s + 1 is visible); load stage s + 2 into buffer s % 2, read stage s + 1's substep-0 fragments,
    // multiply substep 1. Past the end the loads re-read the last stage into a buffer nobody reads again, so every
    // iteration issues the same number of loads.
    const int nk = K / 64;
    issue(0, 0);
    issue(min(1, nk - 1), 1);
    wait_vm<8>();
    bar();
    rd(fa0, fb0, 0, fo0);
    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        rd(fa1, fb1, buf, fo1);
        mm(fa0, fb0);
        wait_lgkm0();
        wait_vm<0>();
        bar();
        issue(min(s + 2, nk - 1), buf);
        rd(fa0, fb0, buf ^ 1, fo0);
        mm(fa1, fb1);
    }
    wait_vm<0>();   // this wave's loads have landed; the barrier below covers every wave's
    __syncthreads();
    prefill_epilogue<256, TI, TJ, NWN, true>(acc, a, G, r0, n0, wm, wn, lane, nred, &lds[0][0][0]);
}

// Prefill copy of the interleaved-RoPE table: tab[p][i] = cos, tab[p][rdim/2 + i] = sin of pair i ->
// out[p][b][c][0..3] = cos of pairs 32 b + c + 8 j (j = 0..3), out[p][b][c][4..7] = their sin (values copied as is).
__global__ void rope_prefill_kernel(const float* __restrict__ tab, int P, int rdim, float* __restrict__ out) {
    const int half = rdim >> 1;
    const size_t n = (size_t)P * half;
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= n) return;
    const int p = (int)(id / half), i = (int)(id % half);
    const int b = i >> 5, w = i & 31, j = w >> 3, c = w & 7;
    float* o = out + (size_t)p * rdim + (size_t)(b * 8 + c) * 8;
    o[j] = tab[(size_t)p * rdim + i];
    o[4 + j] = tab[(size_t)p * rdim + half + i];
}

// Taps of one append -> f16, one work-group per row: the row's largest magnitude m picks a power of two s = 2^k with
// m s in [2^14, 2^15), the row is stored as f16(x s) (an exact scaling, then one rounding, so f16's range can
// neither overflow nor flush the row whatever its magnitude) and 1 / s goes to rscale[row], by which the consumer
// of the context projection multiplies that row's f32 output. A row whose largest magnitude is 0 or not finite
// keeps s = 1.
// The row is held in registers (NPT float4 per thread, all its loads in flight together), so it is read from HBM once
// (KT <= 1024 NPT).
template <int NPT>
__global__ __launch_bounds__(256) void taps_f16_kernel(const float* __restrict__ x, int KT, uint2* __restrict__ y,
                                                           float* __restrict__ rscale) {
    const int row = blockIdx.x, n4 = KT >> 2;
    const float4* p = (const float4*)(x + (size_t)row * KT);
    float4 v[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = threadIdx.x + 256 * j;
        v[j] = i < n4 ? p[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < NPT; ++j)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    __shared__ float red[4];
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int k = 0;
    if (m > 0.f && m <= 3.4028234e38f) {
        int ex;
        frexpf(m, &ex);   // m = f 2^ex, f in [0.5, 1): m 2^(15 - ex) in [2^14, 2^15)
        k = min(max(15 - ex, -100), 100);
    }
    const float s = ldexpf(1.f, k);
    if (threadIdx.x == 0) rscale[row] = ldexpf(1.f, -k);
    uint2* q = y + (size_t)row * n4;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = threadIdx.x + 256 * j;
        if (i < n4) q[i] = make_uint2(pack_f16x2(v[j].x * s, v[j].y * s), pack_f16x2(v[j].z * s, v[j].w * s));
    }
}

__global__ void bf16_to_f16_kernel(const uint2* __restrict__ x, size_t n4, uint2* __restrict__ y) {
    for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        const uint2 w = x[i];
        y[i] = make_uint2(pack_f16x2(bf16_lo(w.x), bf16_hi(w.x)), pack_f16x2(bf16_lo(w.y), bf16_hi(w.y)));
    }
}

}  // namespace

int prefill_tile(int rows, int N, int ngroups) {
    const long big_tiles = (long)((rows + 255) / 256) * (N / 256) * ngroups;
    return (N % 256 == 0 && big_tiles >= 256) ? 256 : 128;   // at least one 256-tile per CU
}

hipError_t launch_prefill(const PrefillArgs& a, int nwg, hipStream_t st) {
    const int T = prefill_tile(a.rows, a.N, a.ngroups);
    if (a.K % BK || a.N % T || a.rows < 1 || a.n_tiles != a.N / T || a.m_tiles != (a.rows + T - 1) / T ||
        a.ngroups < 1 || a.ngroups > PF_MAX_GROUPS)
        return hipErrorInvalidValue;
    if (a.ksplit > 1) {   // 128-tiles writing f32 partial slabs; nwg = tiles x ksplit
        if (T != 128 || a.K % (a.ksplit * BK) || nwg % a.ksplit || a.slab_stride < (long long)a.rows * a.ld)
            return hipErrorInvalidValue;
        for (int i = 0; i < a.ngroups; ++i)
            if (a.g[i].epi != PF_F32) return hipErrorInvalidValue;
    }
    for (int i = 0; i < a.ngroups; ++i)
        if (a.g[i].epi == PF_CACHE_K && a.g[i].knorm && (!a.rope_pf || a.rope_dims != a.hd || a.hd % 64))
            return hipErrorInvalidValue;
    if (T == 256) {   // f16 A and f16 copies of every group's B; 64-k stages
        if (a.K % 64) return hipErrorInvalidValue;
        for (int i = 0; i < a.ngroups; ++i)
            if (!a.g[i].B16) return hipErrorInvalidValue;
        prefill_dma_kernel<1><<<nwg, 512, 0, st>>>(a);
    } else {
        prefill_kernel<128><<<nwg, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_rope_prefill(const float* tab, int P, int rdim, float* out, hipStream_t st) {
    if (rdim % 64 || P < 1) return hipErrorInvalidValue;
    const size_t n = (size_t)P * (rdim / 2);
    rope_prefill_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(tab, P, rdim, out);
    return hipGetLastError();
}

hipError_t launch_taps_f16(const float* x, int n, int KT, uint16_t* y, float* rscale, hipStream_t st) {
    if (n < 1 || KT % 4 || ((uintptr_t)x & 15) || ((uintptr_t)y & 7)) return hipErrorInvalidValue;
    if (KT > TAPS_MAX_WIDTH) return hipErrorInvalidValue;
    taps_f16_kernel<16><<<n, 256, 0, st>>>(x, KT, (uint2*)y, rscale);
    return hipGetLastError();
}

hipError_t launch_bf16_to_f16(const uint16_t* x, size_t n, uint16_t* y, hipStream_t st) {
    if (n % 4 || ((uintptr_t)x & 7) || ((uintptr_t)y & 7)) return hipErrorInvalidValue;
    if (n == 0) return hipSuccess;
    const size_t n4 = n / 4;
    const int grid = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    bf16_to_f16_kernel<<<grid, 256, 0, st>>>((const uint2*)x, n4, (uint2*)y);
    return hipGetLastError();
}
