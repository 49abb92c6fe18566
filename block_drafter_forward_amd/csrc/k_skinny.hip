// k_skinny.hip — K1: skinny-T (T <= 16) weight-streaming GEMM on the bf16 matrix cores of gfx950.
//
// Computes Y[t][m] = sum_k X[t][k] W[m][k] for the draft's 16 slots (or fewer rows), the product the flow-map page's
// gemvT17 / gemvT1 kernels and the MTP page's WG_Q8 compute: every weight byte is read from HBM exactly once.
// Design for CDNA4:
//   * the weight tile (16 rows x 32 k, 1 KB) is loaded straight into the A operand of v_mfma_f32_16x16x32_bf16:
//     lane l reads 16 contiguous bytes of row l % 16, so a wave reads 16 rows x 64 contiguous bytes per step;
//     loads are non-temporal (streamed, never reused);
//   * the activations are the B operand (16 slots = the MFMA's N), pre-split into bf16 hi + lo fragments by their
//     producer, so one k-step is two MFMAs and the f32 activations keep ~17 significant bits;
//   * a work-group is 4 waves on one 16-row tile, each wave a contiguous quarter of the k-range; up to 16 k-steps
//     a wave loads its whole range at once (all of it in flight), longer ranges stream in double-buffered stages;
//     the four 16x16 partial tiles are summed in LDS in a fixed order (deterministic), then the epilogue runs per
//     element;
//   * k is split across S work-groups when M alone gives too few work-groups to fill 256 CUs; the S partial slabs
//     are summed by the consumer kernel in a fixed order.
// Q8_0 weights (int8 codes + one f16 scale per 32 codes): a k-step is exactly one Q8_0 block, so the codes go
// through the MFMA exactly (int8 is exact in bf16) and each row's scale multiplies that step's partial product.
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

__device__ __forceinline__ uint4 ldg_nt(const uint4* p) {
    uint4 v;
    v.x = __builtin_nontemporal_load(&((const uint32_t*)p)[0]);
    v.y = __builtin_nontemporal_load(&((const uint32_t*)p)[1]);
    v.z = __builtin_nontemporal_load(&((const uint32_t*)p)[2]);
    v.w = __builtin_nontemporal_load(&((const uint32_t*)p)[3]);
    return v;
}
__device__ __forceinline__ uint2 ldg_nt2(const uint2* p) {
    uint2 v;
    v.x = __builtin_nontemporal_load(&((const uint32_t*)p)[0]);
    v.y = __builtin_nontemporal_load(&((const uint32_t*)p)[1]);
    return v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8 int8 codes -> 8 bf16 (exact).
__device__ __forceinline__ uint4 i8x8_to_bf16x8(uint2 c) {
    uint32_t w[2] = {c.x, c.y};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int b0 = ((int)(w[i] << (24 - 16 * j))) >> 24;
            int b1 = ((int)(w[i] << (16 - 16 * j))) >> 24;
            uint32_t f0 = __float_as_uint((float)b0) >> 16;
            uint32_t f1 = __float_as_uint((float)b1) & 0xffff0000u;
            o[2 * i + j] = f0 | f1;
        }
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// One pipeline stage: SKC k-steps of the wave's A tiles and B fragments, loaded without any condition (a
// conditional load makes the compiler wait for every outstanding load before the next MFMA).
template <int NT, int WT, int SKC>
struct SkStage {
    uint4 a[NT][SKC];    // bf16 weights; Q8_0 codes in .x/.y
    uint4 bh[SKC], bl[SKC];
    float sc[NT][SKC][4];
};

template <int NT, int WT, int SKC>
__device__ __forceinline__ void sk_load(SkStage<NT, WT, SKC>& st, const SkinnyGroup& G, int K, int m0, int s, int r,
                                        int g, int lane) {
    const uint8_t* xb = G.X + (size_t)s * FRAG_STEP_BYTES + lane * 16;
#pragma unroll
    for (int i = 0; i < SKC; ++i) {
        st.bh[i] = *(const uint4*)(xb + (size_t)i * FRAG_STEP_BYTES);
        st.bl[i] = *(const uint4*)(xb + (size_t)i * FRAG_STEP_BYTES + 1024);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if constexpr (WT == SKW_BF16) {
            const uint16_t* W = (const uint16_t*)(n == 0 ? G.W : G.W2) + (size_t)(m0 + r) * K;
#pragma unroll
            for (int i = 0; i < SKC; ++i) st.a[n][i] = ldg_nt((const uint4*)(W + kcol(s + i, g)));
        } else {
            const int8_t* C = (const int8_t*)(n == 0 ? G.W : G.W2);
            const uint16_t* Dd = (const uint16_t*)(n == 0 ? G.Wd : G.W2d);
            const uint2* cp = (const uint2*)(C + (size_t)(m0 + r) * K + (size_t)s * 32 + g * 8);
            const int nb = K >> 5;
#pragma unroll
            for (int i = 0; i < SKC; ++i) {
                const uint2 c = ldg_nt2(cp + i * 4);
                st.a[n][i] = make_uint4(c.x, c.y, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) st.sc[n][i][j] = f16_to_f32(Dd[(size_t)(m0 + 4 * g + j) * nb + s + i]);
            }
        }
    }
}

template <int NT, int WT, int SKC>
__device__ __forceinline__ void sk_compute(const SkStage<NT, WT, SKC>& st, f32x4_t* acc) {
#pragma unroll
    for (int i = 0; i < SKC; ++i) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if constexpr (WT == SKW_BF16) {
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.a[n][i]), as_bf16x8(st.bh[i]), acc[n], 0, 0, 0);
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.a[n][i]), as_bf16x8(st.bl[i]), acc[n], 0, 0, 0);
            } else {
                const bf16x8_t A = as_bf16x8(i8x8_to_bf16x8(make_uint2(st.a[n][i].x, st.a[n][i].y)));
                f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf16x8(st.bh[i]), p, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf16x8(st.bl[i]), p, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[n][j] += st.sc[n][i][j] * p[j];
            }
        }
    }
}

// Row-staged variant (bf16, KW a multiple of RC = 8 or 4): the MFMA A-operand pattern (16 rows x 64 bytes per load
// instruction) streams from HBM at about a third of the rate of row-contiguous reads. So each chunk of RC k-steps
// (32 RC columns) of the wave's 16-row tile is loaded as RC row-contiguous instructions (16 / RC rows x 64 RC bytes
// each: whole cache lines), parked in a wave-private LDS tile (row pitch padded by 16 bytes) and read back in the
// A layout; the next chunk's weights and activation fragments are in flight while the current one multiplies.
template <int NT, int RC, int NB>
struct RsStage {
    uint4 a[NT][RC];
    uint4 bh[NB][RC], bl[NB][RC];
};

template <int NT, int RC, int NB>
__device__ __forceinline__ void rs_load(RsStage<NT, RC, NB>& st, const SkinnyGroup& G, int K, int m0, int s,
                                        int lane) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint8_t* xb = G.X + (size_t)b * K * 64 + (size_t)s * FRAG_STEP_BYTES + lane * 16;
#pragma unroll
        for (int i = 0; i < RC; ++i) {
            st.bh[b][i] = *(const uint4*)(xb + (size_t)i * FRAG_STEP_BYTES);
            st.bl[b][i] = *(const uint4*)(xb + (size_t)i * FRAG_STEP_BYTES + 1024);
        }
    }
    constexpr int RPI = 16 / RC, LPR = 64 / RPI;   // rows per instruction, lanes per row
    const int sub = lane / LPR, piece = lane % LPR;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const uint16_t* W = (const uint16_t*)(n == 0 ? G.W : G.W2) + (size_t)(m0 + sub) * K + s * 32 + piece * 8;
#pragma unroll
        for (int i = 0; i < RC; ++i) st.a[n][i] = ldg_nt((const uint4*)(W + (size_t)(RPI * i) * K));
    }
}

template <int NT, int RC, int NB>
__device__ __forceinline__ void rs_compute(const RsStage<NT, RC, NB>& st, uint4* lds, f32x4_t (*acc)[NB], int lane) {
    constexpr int RPI = 16 / RC, LPR = 64 / RPI, PITCH = 4 * RC + 1;
    const int sub = lane / LPR, piece = lane % LPR, r = lane & 15, g = lane >> 4;
    __builtin_amdgcn_wave_barrier();   // the previous chunk's LDS reads stay before these writes
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < RC; ++i) lds[(n * 16 + RPI * i + sub) * PITCH + piece] = st.a[n][i];
    __builtin_amdgcn_wave_barrier();   // LDS is in order within a wave: the reads below see the writes
#pragma unroll
    for (int i = 0; i < RC; ++i) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const uint4 av = lds[(n * 16 + r) * PITCH + 4 * i + g];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                acc[n][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(st.bh[b][i]), acc[n][b],
                                                                    0, 0, 0);
                acc[n][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(st.bl[b][i]), acc[n][b],
                                                                    0, 0, 0);
            }
        }
    }
}

// Q8_0 row staging (KW a multiple of 8): a chunk of 8 k-steps is 8 Q8_0 blocks per row -- 256 code bytes (4 rows
// per 1 KB load instruction) and 8 f16 scales per row (lanes 0-15, one 16-byte load). Codes return from a
// wave-private LDS tile as the A operand (8 bytes per lane, widened exactly to bf16); the scales sit transposed
// [step][row] so a lane reads the scales of its 4 output rows for a step in one 8-byte read.
constexpr int Q8_PITCH = 17;   // uint4 per LDS code row: 16 + 1 pad

template <int NT>
struct RsStageQ8 {
    uint4 a[NT][4];
    uint4 sc[NT];
    uint4 bh[8], bl[8];
};

template <int NT>
__device__ __forceinline__ void rs_load_q8(RsStageQ8<NT>& st, const SkinnyGroup& G, int K, int m0, int s, int lane) {
    const uint8_t* xb = G.X + (size_t)s * FRAG_STEP_BYTES + lane * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        st.bh[i] = *(const uint4*)(xb + (size_t)i * FRAG_STEP_BYTES);
        st.bl[i] = *(const uint4*)(xb + (size_t)i * FRAG_STEP_BYTES + 1024);
    }
    const int nb = K >> 5;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int8_t* C = (const int8_t*)(n == 0 ? G.W : G.W2) + (size_t)(m0 + (lane >> 4)) * K + s * 32 + (lane & 15) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) st.a[n][i] = ldg_nt((const uint4*)(C + (size_t)(4 * i) * K));
        // scales with an ordinary load: a 128-byte line of them serves 8 chunks and must stay in L2 meanwhile
        st.sc[n] = *(const uint4*)((const uint16_t*)(n == 0 ? G.Wd : G.W2d) + (size_t)(m0 + (lane & 15)) * nb + s);
    }
}

template <int NT>
__device__ __forceinline__ void rs_compute_q8(const RsStageQ8<NT>& st, uint4* lds, uint16_t* slds, f32x4_t* acc,
                                              int lane) {
    const int r = lane & 15, g = lane >> 4;
    __builtin_amdgcn_wave_barrier();   // the previous chunk's LDS reads stay before these writes
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lds[(n * 16 + 4 * i + (lane >> 4)) * Q8_PITCH + (lane & 15)] = st.a[n][i];
        if (lane < 16) {
            const uint32_t w[4] = {st.sc[n].x, st.sc[n].y, st.sc[n].z, st.sc[n].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                slds[(n * 8 + 2 * e) * 16 + lane] = (uint16_t)(w[e] & 0xffffu);
                slds[(n * 8 + 2 * e + 1) * 16 + lane] = (uint16_t)(w[e] >> 16);
            }
        }
    }
    __builtin_amdgcn_wave_barrier();   // LDS is in order within a wave: the reads below see the writes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const uint2 cv = ((const uint2*)(lds + (n * 16 + r) * Q8_PITCH))[4 * i + g];
            const bf16x8_t A = as_bf16x8(i8x8_to_bf16x8(cv));
            f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf16x8(st.bh[i]), p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf16x8(st.bl[i]), p, 0, 0, 0);
            const uint2 sv = *(const uint2*)(slds + (n * 8 + i) * 16 + 4 * g);
            acc[n][0] += f16_to_f32((uint16_t)(sv.x & 0xffffu)) * p[0];
            acc[n][1] += f16_to_f32((uint16_t)(sv.x >> 16)) * p[1];
            acc[n][2] += f16_to_f32((uint16_t)(sv.y & 0xffffu)) * p[2];
            acc[n][3] += f16_to_f32((uint16_t)(sv.y >> 16)) * p[3];
        }
    }
}

// UP = 2: row-staged chunks of SKC (8 or 4) k-steps (bf16, KW % SKC == 0), double-buffered, last chunk peeled.
// UP = 1: the wave's whole k-range (SKC == KW steps) is loaded at once, then multiplied -- every byte of the wave
// in flight together. UP = 0: KW is a multiple of 2*SKC and stages are double-buffered (stage i+1 in flight while
// stage i computes), with the last pair peeled so the loop body carries no conditions.
// A single Q8_0 matrix fits two work-groups per CU (<= 256 registers a wave, no scratch); without the bound the
// compiler spends AGPRs and runs one wave per SIMD. Two matrices at once would spill, so they keep one.
// NB = 2 (two blocks of 16 activation rows against each weight tile) exists for bf16 with UP = 2 only.
template <int NT, int WT, int UP, int SKC, int NB = 1>
__global__ __launch_bounds__(256, (NT == 1 && WT == SKW_Q8_0) ? 2 : 1) void skinny_kernel(SkinnyArgs a) {
    static_assert(NB == 1 || (WT == SKW_BF16 && UP == 2), "two row blocks: row-staged bf16 only");
    const int bid = blockIdx.x;
    int gi = 0;
#pragma unroll 1
    for (int i = 1; i < a.ngroups; ++i)
        if (bid >= a.g[i].tile_begin) gi = i;
    const SkinnyGroup& G = a.g[gi];
    const int local = bid - G.tile_begin;
    const int rt = local / a.S;
    const int split = local - rt * a.S;
    const int m0 = rt * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int KW = a.KW;
    const int s0 = (split * 4 + wave) * KW;   // first k-step of this wave
    const int r = lane & 15, g = lane >> 4;
    const int K = a.K;

    f32x4_t accb[NT][NB];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int b = 0; b < NB; ++b) accb[n][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t* acc = &accb[0][0];   // the one-block paths (NB == 1): accb[n][0] is acc[n]

    if constexpr (UP == 2 && WT == SKW_Q8_0) {
        __shared__ uint4 q8_lds[4][NT * 16 * Q8_PITCH];
        __shared__ uint16_t q8_slds[4][NT * 8 * 16];
        uint4* lds = q8_lds[wave];
        uint16_t* slds = q8_slds[wave];
        RsStageQ8<NT> c0, c1;
        const int nch = KW / 8;
        rs_load_q8<NT>(c0, G, K, m0, s0, lane);
        int ch = 0;
        for (; ch + 2 < nch; ch += 2) {
            rs_load_q8<NT>(c1, G, K, m0, s0 + 8 * (ch + 1), lane);
            rs_compute_q8<NT>(c0, lds, slds, acc, lane);
            rs_load_q8<NT>(c0, G, K, m0, s0 + 8 * (ch + 2), lane);
            rs_compute_q8<NT>(c1, lds, slds, acc, lane);
        }
        if (ch + 1 < nch) {
            rs_load_q8<NT>(c1, G, K, m0, s0 + 8 * (ch + 1), lane);
            rs_compute_q8<NT>(c0, lds, slds, acc, lane);
            rs_compute_q8<NT>(c1, lds, slds, acc, lane);
        } else {
            rs_compute_q8<NT>(c0, lds, slds, acc, lane);
        }
    } else if constexpr (UP == 2) {
        __shared__ uint4 rs_lds[4][NT * 16 * (4 * SKC + 1)];
        uint4* lds = rs_lds[wave];
        RsStage<NT, SKC, NB> c0, c1;
        const int nch = KW / SKC;
        rs_load<NT, SKC, NB>(c0, G, K, m0, s0, lane);
        int ch = 0;
        for (; ch + 2 < nch; ch += 2) {
            rs_load<NT, SKC, NB>(c1, G, K, m0, s0 + SKC * (ch + 1), lane);
            rs_compute<NT, SKC, NB>(c0, lds, accb, lane);
            rs_load<NT, SKC, NB>(c0, G, K, m0, s0 + SKC * (ch + 2), lane);
            rs_compute<NT, SKC, NB>(c1, lds, accb, lane);
        }
        if (ch + 1 < nch) {
            rs_load<NT, SKC, NB>(c1, G, K, m0, s0 + SKC * (ch + 1), lane);
            rs_compute<NT, SKC, NB>(c0, lds, accb, lane);
            rs_compute<NT, SKC, NB>(c1, lds, accb, lane);
        } else {
            rs_compute<NT, SKC, NB>(c0, lds, accb, lane);
        }
    } else if constexpr (UP == 1) {
        SkStage<NT, WT, SKC> st;
        sk_load<NT, WT, SKC>(st, G, K, m0, s0, r, g, lane);
        sk_compute<NT, WT, SKC>(st, acc);
    } else {
        SkStage<NT, WT, SKC> st0, st1;
        sk_load<NT, WT, SKC>(st0, G, K, m0, s0, r, g, lane);
        int s = 0;
        for (; s + 2 * SKC < KW; s += 2 * SKC) {
            sk_load<NT, WT, SKC>(st1, G, K, m0, s0 + s + SKC, r, g, lane);
            sk_compute<NT, WT, SKC>(st0, acc);
            sk_load<NT, WT, SKC>(st0, G, K, m0, s0 + s + 2 * SKC, r, g, lane);
            sk_compute<NT, WT, SKC>(st1, acc);
        }
        sk_load<NT, WT, SKC>(st1, G, K, m0, s0 + s + SKC, r, g, lane);
        sk_compute<NT, WT, SKC>(st0, acc);
        sk_compute<NT, WT, SKC>(st1, acc);
    }

    // ── sum the four waves' tiles (fixed order), per block of rows ──
    __shared__ f32x4_t red[NT * NB][4][64];
    __shared__ float tile[NB][16][17];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int b = 0; b < NB; ++b) red[n * NB + b][wave][lane] = accb[n][b];
    __syncthreads();
    const int el = threadIdx.x & 63, rr = threadIdx.x >> 6;
    const int ml = 4 * (el >> 4) + rr;   // row of the tile
    const int t = el & 15;               // activation row (slot) within the block
    const int m = m0 + ml;
    const bool frag_mode = a.mode != SK_F32 && a.mode != SK_PARTIAL;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float v[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int q = n * NB + b;
            v[n] = ((red[q][0][el][rr] + red[q][1][el][rr]) + red[q][2][el][rr]) + red[q][3][el][rr];
        }
        const int row = 16 * b + t;
        if (a.mode == SK_F32) {
            if (t < a.T) {
                float bi = G.bias ? bf16_to_f32(G.bias[m]) : 0.f;
                ((float*)G.out)[(size_t)row * G.ld + m] = v[0] + bi;
            }
        } else if (a.mode == SK_PARTIAL) {
            if (t < a.T) ((float*)G.out)[(size_t)split * a.part_stride + (size_t)row * G.ld + m] = v[0];
        } else {
            float o;
            if (a.mode == SK_FRAG_GELU) {
                float bi = G.bias ? bf16_to_f32(G.bias[m]) : 0.f;
                o = gelu_erf(v[0] + bi);
            } else if (a.mode == SK_FRAG_GEGLU) {
                o = gelu_tanh(v[0]) * v[NT - 1];
            } else {
                o = silu(v[0]) * v[NT - 1];
            }
            tile[b][t][ml] = o;
        }
    }
    if (!frag_mode) return;
    __syncthreads();
    if (threadIdx.x < 32 * NB) {
        const int b = threadIdx.x >> 5, tt = (threadIdx.x >> 1) & 15, h = threadIdx.x & 1;
        if (tt < a.T) {
            float vals[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[e] = tile[b][tt][8 * h + e];
            frag_store8((uint8_t*)G.out + (size_t)b * G.M * 64, tt, m0 + 8 * h, vals);
        }
    }
}

template <int NT, int WT>
hipError_t launch_nt(const SkinnyArgs& a, int nwg, hipStream_t st) {
    const int KW = a.KW;
    dim3 grid(nwg), block(256);
    if (a.nb == 2) {   // two blocks of rows: chunks of 4 k-steps (the registers of two blocks' fragments)
        if constexpr (WT == SKW_BF16) {
            if (KW % 4 || a.T != 16) return hipErrorInvalidValue;
            skinny_kernel<NT, WT, 2, 4, 2><<<grid, block, 0, st>>>(a);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (a.nb != 1) return hipErrorInvalidValue;
    if (WT == SKW_BF16 && KW % 4 == 0) {
        if (KW % 8 == 0) skinny_kernel<NT, WT, 2, 8><<<grid, block, 0, st>>>(a);
        else skinny_kernel<NT, WT, 2, 4><<<grid, block, 0, st>>>(a);
        return hipGetLastError();
    }
    if (WT == SKW_Q8_0 && KW % 8 == 0) {
        skinny_kernel<NT, WT, 2, 8><<<grid, block, 0, st>>>(a);
        return hipGetLastError();
    }
#define SK_UP(n) case n: skinny_kernel<NT, WT, 1, n><<<grid, block, 0, st>>>(a); return hipGetLastError();
    switch (KW) {
        SK_UP(1) SK_UP(2) SK_UP(3) SK_UP(4) SK_UP(5) SK_UP(6) SK_UP(8) SK_UP(10) SK_UP(12) SK_UP(16)
    default: break;
    }
#undef SK_UP
    if (KW % 16 == 0) skinny_kernel<NT, WT, 0, 8><<<grid, block, 0, st>>>(a);
    else if (KW % 8 == 0) skinny_kernel<NT, WT, 0, 4><<<grid, block, 0, st>>>(a);
    else if (KW % 4 == 0) skinny_kernel<NT, WT, 0, 2><<<grid, block, 0, st>>>(a);
    else if (KW % 2 == 0) skinny_kernel<NT, WT, 0, 1><<<grid, block, 0, st>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const SkinnyArgs& a, int wtype, int nwg, hipStream_t st) {
    const bool glu = (a.mode == SK_FRAG_GEGLU || a.mode == SK_FRAG_SWIGLU);
    if (wtype == SKW_BF16) return glu ? launch_nt<2, SKW_BF16>(a, nwg, st) : launch_nt<1, SKW_BF16>(a, nwg, st);
    return glu ? launch_nt<2, SKW_Q8_0>(a, nwg, st) : launch_nt<1, SKW_Q8_0>(a, nwg, st);
}
