// k_prefill.hip — K2: the MFMA GEMM of context prefill, C[r][n] = sum_k A[r][k] B[n][k].
//
// The one truly dense contraction of the path: the fusion of many context rows (fc / W_c over the concatenated
// taps, flashmap_drafter.js extendContext; module-dflash.ts #buildContext) and the per-layer K/V projections of the
// fused rows. Operands are f16 on v_mfma_f32_16x16x32_f16 with f32 accumulation: the f32 taps are rounded to f16 on
// their way into LDS (2^-11 relative, four times finer than bf16), the bf16 weights are widened to f16 exactly (up
// to f16's subnormal range, |error| <= 2^-25). Tiles: 256 x 256 per work-group of 8 waves (2 x 4, 128 x 64 each,
// 32 accumulators of 16x16) when the problem has enough of them, else 128 x 128 per 4 waves; k-stages of 32
// double-buffered in LDS with a 16-byte row pad (conflict-free fragment reads), the next stage's global loads in
// flight while the current one computes. The larger tile halves the L2 traffic per flop. Two k-stages of global
// loads are in flight (registers) while a third multiplies from LDS: one stage of MFMAs alone does not cover the
// load latency (measured: 30% -> 40% of the f16 peak on the 8192-row K/V projections). Work-groups are remapped so
// each XCD owns a contiguous run of tiles (consecutive n-tiles of the same row block share their A rows in that
// XCD's L2).
// Epilogues: f32 rows; a cache store (f16 / f32) at rows start + r, or into the f16 V cache's 32-position tiles
// (dimension-major inside a tile: 8-byte stores of 4 consecutive positions); or, for K, the per-head RMSNorm over the tile's
// columns (a head is 64 or 128 columns of the 128-wide tile) and interleaved RoPE at position start + r before the
// store -- the page's headNormRope + kvWrite, fused.
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

constexpr int BK = 32, LDP = BK + 8;

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16);
}

// Tile T x T (T = 128: 4 waves as 2 x 2 of 64 x 64; T = 256: 8 waves as 2 x 4 of 128 x 64). Every thread stages
// 16 k-values of one A row and one B row per k-stage; rows past the end of A are clamped (their results dropped).
template <int AF32, int T>
__global__ __launch_bounds__(T * 2) void prefill_kernel(PrefillArgs a) {
    constexpr int BM = T, BN = T, NWN = T / 64, TI = T == 128 ? 4 : 8, TJ = 4;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDP];
    __shared__ float nred[NWN][BM];

    int lin = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    int gi = 0;
#pragma unroll 1
    for (int i = 1; i < a.ngroups; ++i)
        if (lin >= a.g[i].tile_begin) gi = i;
    const PrefillGroup& G = a.g[gi];
    const int local = lin - G.tile_begin;
    const int mt = local / a.n_tiles, nt = local - mt * a.n_tiles;
    const int r0 = mt * BM, n0 = nt * BN;
    const void* Ap = G.A ? G.A : a.A;
    const int K = a.K;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / NWN, wn = wave % NWN;
    const int ldrow = tid >> 1, kofs = (tid & 1) * 16;
    const int arow = min(r0 + ldrow, a.rows - 1);

    struct PStage {
        float4 ra[4];
        uint4 rah[2], rb[2];
    };
    auto gload = [&](PStage& r, int kt) {
        const int k = kt * BK + kofs;
        if constexpr (AF32) {
            const float4* p = (const float4*)((const float*)Ap + (size_t)arow * K + k);
#pragma unroll
            for (int i = 0; i < 4; ++i) r.ra[i] = p[i];
        } else {
            const uint4* p = (const uint4*)((const uint16_t*)Ap + (size_t)arow * K + k);
            r.rah[0] = p[0];
            r.rah[1] = p[1];
        }
        const uint4* pb = (const uint4*)(G.B + (size_t)(n0 + ldrow) * K + k);
        r.rb[0] = pb[0];
        r.rb[1] = pb[1];
    };
    auto lstore = [&](const PStage& r, int buf) {
        uint4 h0, h1;
        if constexpr (AF32) {
            h0 = make_uint4(pack_f16x2(r.ra[0].x, r.ra[0].y), pack_f16x2(r.ra[0].z, r.ra[0].w),
                            pack_f16x2(r.ra[1].x, r.ra[1].y), pack_f16x2(r.ra[1].z, r.ra[1].w));
            h1 = make_uint4(pack_f16x2(r.ra[2].x, r.ra[2].y), pack_f16x2(r.ra[2].z, r.ra[2].w),
                            pack_f16x2(r.ra[3].x, r.ra[3].y), pack_f16x2(r.ra[3].z, r.ra[3].w));
        } else {
            h0 = r.rah[0];
            h1 = r.rah[1];
        }
        *(uint4*)&As[buf][ldrow][kofs] = h0;
        *(uint4*)&As[buf][ldrow][kofs + 8] = h1;
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
    const int nk = K / BK;
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

    // acc[i][j][q] = C[r0 + wm*16*TI + 16 i + 4 (lane/16) + q][n0 + wn*64 + 16 j + lane%16]
    const int rq = 4 * (lane >> 4), cl = lane & 15;
    if (G.epi == PF_CACHE_K && G.knorm) {
        const int hd = a.hd;
        float ssq[TI][4];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < TJ; ++j) s += acc[i][j][q] * acc[i][j][q];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
                ssq[i][q] = s;
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
        const int half = a.rope_dims >> 1;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + wm * TI * 16 + 16 * i + rq + q;
                const float rs = 1.f / sqrtf(ssq[i][q] / (float)hd + a.eps);
                const int pos = a.start + (r < a.rows ? r : 0);
                const float* tr = a.rope_tab + (size_t)pos * a.rope_dims;
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const int n = n0 + wn * 64 + 16 * j + cl;
                    const int d = n % hd;
                    const float v = acc[i][j][q] * rs * bf16_to_f32(G.knorm[d]);
                    const float p = __shfl_xor(v, 1, 64);
                    const float c = tr[d >> 1], sn = tr[half + (d >> 1)];
                    acc[i][j][q] = (d & 1) ? v * c + p * sn : v * c - p * sn;
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
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + wm * TI * 16 + 16 * i + rq + q;
            if (r >= a.rows) continue;
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int n = n0 + wn * 64 + 16 * j + cl;
                const float v = acc[i][j][q];
                if (G.epi == PF_F32) {
                    ((float*)G.out)[(size_t)r * a.ld + n] = v;
                } else {
                    const size_t off = (size_t)(a.start + r) * a.ld + n;
                    if (a.kv_dtype == 0) ((uint16_t*)G.out)[off] = f32_to_f16(v);
                    else ((float*)G.out)[off] = v;
                }
            }
        }
}

}  // namespace

int prefill_tile(int rows, int N, int ngroups) {
    const long big_tiles = (long)((rows + 255) / 256) * (N / 256) * ngroups;
    return (N % 256 == 0 && big_tiles >= 256) ? 256 : 128;   // at least one 256-tile per CU
}

hipError_t launch_prefill(const PrefillArgs& a, int nwg, hipStream_t st) {
    const int T = prefill_tile(a.rows, a.N, a.ngroups);
    if (a.K % BK || a.N % T || a.rows < 1 || a.n_tiles != a.N / T || a.m_tiles != (a.rows + T - 1) / T)
        return hipErrorInvalidValue;
    if (T == 256) {
        if (a.a_f32) prefill_kernel<1, 256><<<nwg, 512, 0, st>>>(a);
        else prefill_kernel<0, 256><<<nwg, 512, 0, st>>>(a);
    } else {
        if (a.a_f32) prefill_kernel<1, 128><<<nwg, 256, 0, st>>>(a);
        else prefill_kernel<0, 128><<<nwg, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}
