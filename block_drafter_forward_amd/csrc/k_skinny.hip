// k_skinny.hip — K1: skinny-T (T <= 16) weight-streaming GEMM on the bf16 matrix cores of gfx950.
//
// Computes Y[t][m] = sum_k X[t][k] W[m][k] for the draft's 16 slots (or fewer rows), the product the flow-map page's
// gemvT17 / gemvT1 kernels and the MTP page's WG_Q8 compute: every weight byte is read from HBM exactly once.
// Design for CDNA4, bf16 weights (skinny_kernel):
//   * the weight tile (16 rows x 32 k, 1 KB) is the A operand of v_mfma_f32_16x16x32_bf16, row-staged through a
//     wave-private LDS tile (whole cache lines per load instruction); loads are non-temporal (streamed, never reused);
//   * the activations are the B operand (16 slots = the MFMA's N), pre-split into bf16 hi + lo fragments by their
//     producer, so one k-step is two MFMAs and the f32 activations keep ~17 significant bits;
//   * a work-group is 4 waves on one 16-row tile, each wave a contiguous quarter of the k-range, its next chunk's
//     weights and fragments in flight while one multiplies; the four 16x16 partial tiles are summed in LDS in a fixed
//     order (deterministic), then the epilogue runs per element;
//   * k is split across S work-groups when M alone gives too few work-groups to fill 256 CUs; the S partial slabs
//     are summed by the consumer kernel in a fixed order.
// Q8_0 weights (int8 codes + one f16 scale per 32 codes: the MTP head), skinny_ws_kernel: a k-step is exactly one
// Q8_0 block, so the codes go through the MFMA exactly (int8 is exact in bf16) and each row's scale multiplies that
// step's partial product. Here the waves of a work-group own adjacent 16-row tiles and walk their k-range in lockstep,
// sharing one LDS copy of each chunk's activation fragments (fm_ws.h): a wave reads 4 KB of codes per chunk next to
// the 16 KB of fragments, so per-wave fragment reads would be four times the HBM bytes.
#include "fm_device.h"
#include "fm_kernels.h"
#include "fm_ws.h"
#include "fm_selfattn.h"

namespace {

__device__ __forceinline__ uint4 ldg_nt(const uint4* p) {
    uint4 v;
    v.x = __builtin_nontemporal_load(&((const uint32_t*)p)[0]);
    v.y = __builtin_nontemporal_load(&((const uint32_t*)p)[1]);
    v.z = __builtin_nontemporal_load(&((const uint32_t*)p)[2]);
    v.w = __builtin_nontemporal_load(&((const uint32_t*)p)[3]);
    return v;
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Device-coherent 16-byte store / load (written through / read past the non-coherent caches): buffer instructions
// with the device-coherent cache policy bit.
// base is wave-uniform (the buffer resource lives in scalar registers), idx the lane's float offset from it.
constexpr int SC1 = 16;
__device__ __forceinline__ void cst16(float* base, size_t idx, float4 v) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(
        u4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)}, r,
        (unsigned)(idx * 4), 0, SC1);
}
__device__ __forceinline__ float4 cld16(const float* base, size_t idx) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0x7fffffff, 0x00020000);
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (unsigned)(idx * 4), 0, SC1);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// LDS-direct load: lane l's 16 bytes from g land at lds + 16 l (lds wave-uniform, through m0). In inline asm, so
// the compiler's wait bookkeeping does not see it (a tracked LDS-direct load would make it wait for every load in
// flight at the next LDS read); its reader waits explicitly.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
    const unsigned la =
        __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)((__attribute__((address_space(3))) void*)lds));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory", "m0");
}

// One pipeline stage: SKC k-steps of the wave's A tiles and B fragments, loaded without any condition (a
// conditional load makes the compiler wait for every outstanding load before the next MFMA).
template <int NT, int WT, int SKC>
struct SkStage {
    uint4 a[NT][SKC];    // bf16 weights
    uint4 bh[SKC], bl[SKC];
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
        const uint16_t* W = (const uint16_t*)(n == 0 ? G.W : G.W2) + (size_t)(m0 + r) * K;
#pragma unroll
        for (int i = 0; i < SKC; ++i) st.a[n][i] = ldg_nt((const uint4*)(W + kcol(s + i, g)));
    }
}

template <int NT, int WT, int SKC>
__device__ __forceinline__ void sk_compute(const SkStage<NT, WT, SKC>& st, f32x4_t* acc) {
#pragma unroll
    for (int i = 0; i < SKC; ++i) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.a[n][i]), as_bf16x8(st.bh[i]), acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.a[n][i]), as_bf16x8(st.bl[i]), acc[n], 0, 0, 0);
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

// UP = 2: row-staged chunks of SKC (8 or 4) k-steps (bf16, KW % SKC == 0), double-buffered, last chunk peeled.
// UP = 1: the wave's whole k-range (SKC == KW steps) is loaded at once, then multiplied -- every byte of the wave
// in flight together. UP = 0: KW is a multiple of 2*SKC and stages are double-buffered (stage i+1 in flight while
// stage i computes), with the last pair peeled so the loop body carries no conditions.
// NB = 2 (two blocks of 16 activation rows against each weight tile) exists with UP = 2 only.
// EP, the epilogue's kind: EP_PLAIN, EP_LN (the LayerNorm fold of SkinnyArgs, one matrix) or EP_RESID (SK_RESID,
// one matrix). Every operand of the epilogue (bias, LayerNorm statistics and c1 / c2, the residual update's base,
// gate and scale) is loaded before the main loop, so the epilogue waits on no memory round trip of its own.
enum SkEpilogue { EP_PLAIN = 0, EP_LN = 1, EP_RESID = 2 };
template <int NT, int WT, int UP, int SKC, int NB = 1, int EP = EP_PLAIN>
__global__ __launch_bounds__(256, 1) void skinny_kernel(SkinnyArgs a) {
    static_assert(WT == SKW_BF16, "bf16 weights (Q8_0: skinny_ws_kernel)");
    static_assert(NB == 1 || UP == 2, "two row blocks: row-staged only");
    static_assert(EP == EP_PLAIN || EP == EP_LN || NT == 1, "the residual update takes one matrix");
    constexpr bool LN = EP == EP_LN;
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

    // ── epilogue operands, in flight with the first weights ──
    constexpr int R = 16 * NB;              // activation rows of the launch
    constexpr int NGQ = 256 / R;            // LayerNorm statistics: threads per row
    const int e_el = threadIdx.x & 63, e_rr = threadIdx.x >> 6;
    const int e_ml = 4 * (e_el >> 4) + e_rr;   // the element this thread finishes: tile row e_ml, activation row e_t
    const int e_t = e_el & 15, e_m = m0 + e_ml;
    constexpr bool resid = EP == EP_RESID;   // mode SK_RESID (checked by the launcher)
    const float e_bias = bf16_to_f32(*(G.bias ? G.bias + e_m : (const uint16_t*)a.zeros));   // no branch: no wait
    float e_base[NB], e_gate = 1.f, e_yf = 1.f;   // e_yf: x's factor in the next product's fragments
    if constexpr (resid) {
#pragma unroll
        for (int b = 0; b < NB; ++b) e_base[b] = a.rbase[(size_t)(16 * b + e_t) * a.rbase_ld + e_m];
        e_gate = *(a.rgate ? a.rgate + e_m : a.zeros);
        const float ys = *(a.ryscale ? a.ryscale + e_m : a.zeros);
        const float yw = bf16_to_f32(*(a.ryw ? a.ryw + e_m : (const uint16_t*)a.zeros));
        e_yf = a.ryw ? yw : 1.f + ys;
    }
    // LayerNorm statistics (float2 [ln_tiles][R], ln_tiles R / 128 KB) straight into LDS, 1 KB per wave instruction,
    // issued right after the first chunk's loads: loads complete in issue order, so the first chunk's wait covers
    // them too, and the statistics are reduced (ln_reduce) between the first chunk's products and the next chunk's
    // (after the statistics are reduced, the q | k | v product's self-attention tail reuses this LDS)
    __shared__ __attribute__((aligned(16))) float2 lnlds[LN ? LN_MAX_TILES * 16 : 1];
    float e_c1 = 0.f, e_c2 = 0.f;
    if constexpr (LN) {   // (an RMSNorm fold has no c12: zeros)
        e_c1 = *(G.c12 ? G.c12 + e_m : a.zeros);
        e_c2 = *(G.c12 ? G.c12 + G.M + e_m : a.zeros);
    }
    auto ln_prefetch = [&]() {
        if constexpr (LN) {
            const int nin = a.ln_tiles * R / 128;   // 1 KB pieces
            for (int i = wave; i < nin; i += 4)
                lds_dma16((const uint8_t*)a.ln_stats + (size_t)i * 1024 + lane * 16, (uint8_t*)lnlds + (size_t)i * 1024);
        }
    };

    f32x4_t accb[NT][NB];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int b = 0; b < NB; ++b) accb[n][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t* acc = &accb[0][0];   // the one-block paths (NB == 1): accb[n][0] is acc[n]

    // ── LayerNorm fold: each row's mean and rstd from its tiles' (mean, M2) in one pass, in a fixed order
    // (deterministic). Sums are taken about K = the row's first tile mean (Chan et al. with a shift):
    //   sum_j mean_j and S = sum_j (M2_j + 16 (mean_j - K)^2) = sum (x - K)^2;  M2 = S - n (mean - K)^2.
    // Thread (row, gq) takes tiles gq, gq + NGQ, ... (every LDS read in bounds and unconditional, the tiles past the
    // row's end masked); wave shuffles, then the four waves' sums through LDS. Run once, right after the first
    // chunk's products, while the next chunk's loads are in flight: its LDS reads take their base address from an
    // asm that consumes those products, so they cannot be scheduled before the wait for the first chunk, which (in
    // issue order) covers the statistics' LDS-direct loads. ──
    float e_mu[NB], e_rs[NB];
    __shared__ float lnred[LN ? 2 : 1][4][R];
    auto ln_reduce = [&]() {
        if constexpr (LN) {
            constexpr int NPT = LN_MAX_TILES / NB / NGQ;   // tiles per thread at most (16)
            int lbase = 0;
            float dep = accb[0][0][0];
            asm volatile("" : "+v"(lbase) : "v"(dep));
            __syncthreads();   // every wave's statistics have landed
            const float2* lp = lnlds + lbase;
            const int row = threadIdx.x % R, gq = threadIdx.x / R;
            const float kr = lp[row].x;
            float2 sv[NPT];
#pragma unroll
            for (int i = 0; i < NPT; ++i) sv[i] = lp[(gq + NGQ * i) * R + row];   // in bounds, past-the-row tiles too
            // every value an operand of an (empty) asm: the reads are issued together, none sunk into a branch
#pragma unroll
            for (int i = 0; i < NPT; ++i) asm volatile("" : "+v"(sv[i].x), "+v"(sv[i].y));
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int i = 0; i < NPT; ++i) {
                const bool ok = gq + NGQ * i < a.ln_tiles;
                const float dd = sv[i].x - kr;
                const float t2 = sv[i].y + 16.f * dd * dd;
                s1 += ok ? sv[i].x : 0.f;
                s2 += ok ? t2 : 0.f;
            }
            // lanes of one row within a wave: lane = gq_local R + row
#pragma unroll
            for (int o = R; o < 64; o <<= 1) {
                s1 += __shfl_xor(s1, o, 64);
                s2 += __shfl_xor(s2, o, 64);
            }
            if (lane < R) {
                lnred[0][wave][lane] = s1;
                lnred[1][wave][lane] = s2;
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int rw = 16 * b + e_t;
                const float mu =
                    (((lnred[0][0][rw] + lnred[0][1][rw]) + lnred[0][2][rw]) + lnred[0][3][rw]) * a.ln_inv;
                const float sq = ((lnred[1][0][rw] + lnred[1][1][rw]) + lnred[1][2][rw]) + lnred[1][3][rw];
                const float dk = mu - lp[rw].x;
                const float var = fmaxf((sq * a.ln_inv - 16.f * dk * dk) * (1.f / 16.f), 0.f);
                e_mu[b] = a.ln_rms ? 0.f : mu;
                e_rs[b] = 1.f / sqrtf((a.ln_rms ? var + mu * mu : var) + a.ln_eps);
            }
        }
    };

    if constexpr (UP == 2) {
        __shared__ uint4 rs_lds[4][NT * 16 * (4 * SKC + 1)];
        uint4* lds = rs_lds[wave];
        RsStage<NT, SKC, NB> c0, c1;
        const int nch = KW / SKC;
        rs_load<NT, SKC, NB>(c0, G, K, m0, s0, lane);
        ln_prefetch();
        int ch = 0;
        for (; ch + 2 < nch; ch += 2) {
            rs_load<NT, SKC, NB>(c1, G, K, m0, s0 + SKC * (ch + 1), lane);
            rs_compute<NT, SKC, NB>(c0, lds, accb, lane);
            if (ch == 0) ln_reduce();
            rs_load<NT, SKC, NB>(c0, G, K, m0, s0 + SKC * (ch + 2), lane);
            rs_compute<NT, SKC, NB>(c1, lds, accb, lane);
        }
        if (ch + 1 < nch) {
            rs_load<NT, SKC, NB>(c1, G, K, m0, s0 + SKC * (ch + 1), lane);
            rs_compute<NT, SKC, NB>(c0, lds, accb, lane);
            if (ch == 0) ln_reduce();
            rs_compute<NT, SKC, NB>(c1, lds, accb, lane);
        } else {
            rs_compute<NT, SKC, NB>(c0, lds, accb, lane);
            if (ch == 0) ln_reduce();
        }
    } else if constexpr (UP == 1) {
        SkStage<NT, WT, SKC> st;
        sk_load<NT, WT, SKC>(st, G, K, m0, s0, r, g, lane);
        ln_prefetch();
        sk_compute<NT, WT, SKC>(st, acc);
        ln_reduce();
    } else {
        SkStage<NT, WT, SKC> st0, st1;
        sk_load<NT, WT, SKC>(st0, G, K, m0, s0, r, g, lane);
        ln_prefetch();
        int s = 0;
        for (; s + 2 * SKC < KW; s += 2 * SKC) {
            sk_load<NT, WT, SKC>(st1, G, K, m0, s0 + s + SKC, r, g, lane);
            sk_compute<NT, WT, SKC>(st0, acc);
            if (s == 0) ln_reduce();
            sk_load<NT, WT, SKC>(st0, G, K, m0, s0 + s + 2 * SKC, r, g, lane);
            sk_compute<NT, WT, SKC>(st1, acc);
        }
        sk_load<NT, WT, SKC>(st1, G, K, m0, s0 + s + SKC, r, g, lane);
        sk_compute<NT, WT, SKC>(st0, acc);
        if (s == 0) ln_reduce();
        sk_compute<NT, WT, SKC>(st1, acc);
    }

    // ── sum the four waves' tiles (fixed order), per block of rows ──
    __shared__ f32x4_t red[NT * NB][4][64];
    __shared__ float tile[NB][16][17];
    __shared__ float xt[NB][16][17];   // SK_RESID: the tile's updated residual
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int b = 0; b < NB; ++b) red[n * NB + b][wave][lane] = accb[n][b];
    __syncthreads();
    const int el = e_el, rr = e_rr, ml = e_ml, t = e_t, m = e_m;
    const bool frag_mode = a.mode != SK_F32 && a.mode != SK_PARTIAL;
    // A residual update split over S work-groups: each split writes its partial tile with device-coherent stores
    // (written through to memory), waits until they are performed, then takes a ticket on the tile's counter. The
    // split that draws the last ticket adds the S partials in split order (deterministic), resets the counter for
    // the next launch and finishes the tile; the others are done. Nothing ever waits on another work-group.
    // The partial tiles go out and come back as 16-byte rows (thread q of a block: row q / 4, columns 4 (q % 4) ..),
    // staged through LDS: one write-through transaction per 16 bytes rather than one per element.
    float vsum[NB];
    if (resid && a.S > 1) {   // (resid: compile-time)
        __shared__ int ticket;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            vsum[b] = ((red[b][0][el][rr] + red[b][1][el][rr]) + red[b][2][el][rr]) + red[b][3][el][rr];
            tile[b][t][ml] = vsum[b];
        }
        __syncthreads();
        if (threadIdx.x < 64 * NB) {
            const int b = threadIdx.x >> 6, q = threadIdx.x & 63, tr = q >> 2, c4 = 4 * (q & 3);
            cst16(a.rpart, (size_t)split * a.part_stride + (size_t)(16 * b + tr) * G.M + m0 + c4,
                  make_float4(tile[b][tr][c4], tile[b][tr][c4 + 1], tile[b][tr][c4 + 2], tile[b][tr][c4 + 3]));
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partial stores are performed
        __syncthreads();                                    // and every thread's
        if (threadIdx.x == 0)
            ticket = (int)__hip_atomic_fetch_add(a.rtick + rt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (ticket != a.S - 1) return;   // another split finishes the tile
        if (threadIdx.x == 0) __hip_atomic_store(a.rtick + rt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float tot[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) tot[b] = 0.f;
        for (int sp = 0; sp < a.S; ++sp) {   // split order: the sum is the same whichever split finishes
            if (sp == split) {
#pragma unroll
                for (int b = 0; b < NB; ++b) tot[b] += vsum[b];
                continue;
            }
            if (threadIdx.x < 64 * NB) {   // the other split's tile, through LDS (xt: free until the epilogue)
                const int b = threadIdx.x >> 6, q = threadIdx.x & 63, tr = q >> 2, c4 = 4 * (q & 3);
                const float4 f = cld16(a.rpart, (size_t)sp * a.part_stride + (size_t)(16 * b + tr) * G.M + m0 + c4);
                xt[b][tr][c4] = f.x; xt[b][tr][c4 + 1] = f.y; xt[b][tr][c4 + 2] = f.z; xt[b][tr][c4 + 3] = f.w;
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < NB; ++b) tot[b] += xt[b][t][ml];
            __syncthreads();
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) vsum[b] = tot[b];
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float v[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int q = n * NB + b;
            v[n] = ((red[q][0][el][rr] + red[q][1][el][rr]) + red[q][2][el][rr]) + red[q][3][el][rr];
        }
        if (resid && a.S > 1) v[0] = vsum[b];
        const int row = 16 * b + t;
        if constexpr (LN) {   // rstd (acc - mean c1) + c2; the constant part once (split 0)
            v[0] = split == 0 ? e_rs[b] * (v[0] - e_mu[b] * e_c1) + e_c2 : e_rs[b] * v[0];
#pragma unroll
            for (int n = 1; n < NT; ++n) v[n] = e_rs[b] * v[n];   // (RMSNorm fold: no c1 / c2)
        }
        if (a.mode == SK_F32) {
            if (LN && a.sa.qkv) tile[b][t][ml] = v[0] + e_bias;   // stored device-coherent below, 16 bytes a thread
            else if (t < a.T) ((float*)G.out)[(size_t)row * G.ld + m] = v[0] + e_bias;
        } else if (a.mode == SK_PARTIAL) {
            if (t < a.T) ((float*)G.out)[(size_t)split * a.part_stride + (size_t)row * G.ld + m] = v[0];
        } else if (resid) {
            const float xn = e_base[b] + (a.rgate ? e_gate : 1.f) * (v[0] + e_bias);
            if (t < a.T) {
                a.rx[(size_t)row * a.rx_ld + m] = xn;
                if (a.rdebug) a.rdebug[(size_t)row * a.rx_ld + m] = xn;
            }
            xt[b][t][ml] = xn;
            tile[b][t][ml] = xn * e_yf;
        } else {
            float o;
            if (a.mode == SK_FRAG_GELU) {
                o = gelu_erf(v[0] + e_bias);
            } else if (a.mode == SK_FRAG_GEGLU) {
                o = gelu_tanh(v[0]) * v[NT - 1];
            } else {
                o = silu(v[0]) * v[NT - 1];
            }
            tile[b][t][ml] = o;
        }
    }
    if (!frag_mode) {
        if constexpr (LN) {
            if (a.sa.qkv) {   // q | k | v stored device-coherent: the head's last tile to arrive runs its attention
                __shared__ int sticket;
                __syncthreads();
                if (threadIdx.x < 64 * NB) {
                    const int b = threadIdx.x >> 6, q = threadIdx.x & 63, tr = q >> 2, c4 = 4 * (q & 3);
                    if (tr < a.T)
                        cst16((float*)G.out, (size_t)(16 * b + tr) * G.ld + m0 + c4,
                              make_float4(tile[b][tr][c4], tile[b][tr][c4 + 1], tile[b][tr][c4 + 2], tile[b][tr][c4 + 3]));
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's stores are performed
                __syncthreads();                                    // and every thread's
                const int head = m0 / a.sa.hd;
                if (threadIdx.x == 0)
                    sticket = (int)__hip_atomic_fetch_add(a.satick + head, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                if (sticket != 3 * (a.sa.hd / 16) - 1) return;   // another tile of the head finishes it
                if (threadIdx.x == 0) __hip_atomic_store(a.satick + head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                float* QK = (float*)lnlds;   // the statistics are reduced: the LDS is free
                float* Vs = QK + 32 * (a.sa.hd + 4);
                float(*Ps)[17] = (float(*)[17])(Vs + 16 * (a.sa.hd + 4));
                for (int b = 0; b < a.sa.nb; ++b) {
                    if (a.sa.hd == 128) sattn::head<128>(a.sa, head, b, QK, Vs, Ps);
                    else sattn::head<64>(a.sa, head, b, QK, Vs, Ps);
                }
            }
        }
        return;
    }
    __syncthreads();
    if (resid && threadIdx.x < R) {   // (mean, M2) of each row of x over the tile's 16 columns
        const int b = threadIdx.x >> 4, tt = threadIdx.x & 15;
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) sm += xt[b][tt][j];
        const float mean = sm * (1.f / 16.f);
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float dd = xt[b][tt][j] - mean;
            q += dd * dd;
        }
        ((float2*)a.rstats)[(size_t)(m0 >> 4) * R + threadIdx.x] = make_float2(mean, q);
    }
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

template <int NT, int WT, int EP>
hipError_t launch_nt_ep(const SkinnyArgs& a, int nwg, hipStream_t st) {
    const int KW = a.KW;
    dim3 grid(nwg), block(256);
    if (a.nb == 2) {   // two blocks of rows: chunks of 4 k-steps (the registers of two blocks' fragments)
        if constexpr (WT == SKW_BF16) {
            if (KW % 4 || a.T != 16) return hipErrorInvalidValue;
            skinny_kernel<NT, WT, 2, 4, 2, EP><<<grid, block, 0, st>>>(a);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (a.nb != 1) return hipErrorInvalidValue;
    if (KW % 4 == 0) {
        if (KW % 8 == 0) skinny_kernel<NT, WT, 2, 8, 1, EP><<<grid, block, 0, st>>>(a);
        else skinny_kernel<NT, WT, 2, 4, 1, EP><<<grid, block, 0, st>>>(a);
        return hipGetLastError();
    }
#define SK_UP(n) case n: skinny_kernel<NT, WT, 1, n, 1, EP><<<grid, block, 0, st>>>(a); return hipGetLastError();
    switch (KW) {
        SK_UP(1) SK_UP(2) SK_UP(3) SK_UP(5) SK_UP(6) SK_UP(10)
    default: break;
    }
#undef SK_UP
    if (KW > 16 && KW % 2 == 0) skinny_kernel<NT, WT, 0, 1, 1, EP><<<grid, block, 0, st>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int NT, int WT>
hipError_t launch_nt(const SkinnyArgs& a, int nwg, hipStream_t st) {
    if (a.ln_stats || a.mode == SK_RESID) {
        if constexpr (NT == 1)
            return a.ln_stats ? launch_nt_ep<1, WT, EP_LN>(a, nwg, st) : launch_nt_ep<1, WT, EP_RESID>(a, nwg, st);
        else if (a.ln_stats && a.ln_rms)
            return launch_nt_ep<NT, WT, EP_LN>(a, nwg, st);
        return hipErrorInvalidValue;
    }
    return launch_nt_ep<NT, WT, EP_PLAIN>(a, nwg, st);
}

// ── Q8_0: the tile-owning variant ──────────────────────────────────────────────────────────────
// The weights come in the MFMA operand layout (launch_q8_tile_copy: per 16-row tile and 256-column chunk, each lane's
// 64 bytes of codes contiguous, then its row's 8 scales), so codes go from HBM straight into the operand registers.
// A work-group is SK_WS_WAVES waves walking columns [split K / S, (split + 1) K / S) in chunks of 256, two chunks in
// flight per wave, each chunk's activation fragments staged once per work-group in a double-buffered LDS slab;
// three work-groups per CU (at most 168 VGPRs), so that the launches of 544 and 640 work-groups of the MTP head fit
// one round. The fragments are the MFMA's A operand and the codes its B operand: a lane's output column is its own
// code row, each k-step's scale one of its own 8. Wave w owns one 16-row tile: tile NW tg + w of its group, or for a
// gated unit (GLU) tile NW / 2 tg + w / 2 of the gate (w even) or of the up matrix (w odd), the pair combined
// through LDS at the end. Tail waves of a group's last work-group redo its last tile, their results dropped. Each
// wave's 16 x 16 tile is complete for its k-range, so no sum over waves: the epilogue goes straight from the
// accumulator (SK_PARTIAL: the split's slab).
template <bool GLU>
__global__ __launch_bounds__(SK_WS_WAVES * 64, 3) void skinny_ws_kernel(SkinnyArgs a) {
    constexpr int NW = SK_WS_WAVES, TPW = GLU ? NW / 2 : NW;   // tiles per work-group (of each matrix)
    constexpr int ST = 2;                                      // chunks in flight per wave
    __shared__ uint4 blds_all[2][1024];
    static_assert(sizeof(float) * NW * 16 * 17 <= sizeof(blds_all), "epilogue tile");
    float(*tile_all)[16][17] = (float(*)[16][17])&blds_all[0][0];   // after the last product
    const int bid = blockIdx.x;
    int gi = 0;
#pragma unroll 1
    for (int i = 1; i < a.ngroups; ++i)
        if (bid >= a.g[i].tile_begin) gi = i;
    const SkinnyGroup& G = a.g[gi];
    const int local = bid - G.tile_begin;
    const int tg = local / a.S, split = local - tg * a.S;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int ntile = G.M / 16, mt = tg * TPW + (GLU ? wave >> 1 : wave);
    const bool own = mt < ntile;
    const int m0 = min(mt, ntile - 1) * 16;
    const bool up = GLU && (wave & 1);
    const int K = a.K, ncht = K >> 8, nch = ncht / a.S, c0 = split * nch;   // chunks: per row, per split, first
    const size_t tc0 = (size_t)(m0 >> 4) * ncht + c0;
    const uint8_t* Tq = (const uint8_t*)(up ? G.W2 : G.W) + tc0 * 4096 + lane * 16;
    const uint16_t* Ts = (const uint16_t*)(up ? G.W2d : G.Wd) + tc0 * 128 + r * 8;
    const uint8_t* X = G.X + (size_t)c0 * 8 * FRAG_STEP_BYTES;
    struct Regs {
        uint4 c[4];            // codes of k-steps 2i, 2i + 1 (8 each) in c[i]
        uint4 s;               // the row's 8 scales
        uint4 b[16 / NW];      // this thread's share of the chunk's fragments
    };
    auto load = [&](Regs& q, int ch) {   // nothing past the last chunk (a uniform branch)
        if (ch < nch) {
            const uint8_t* p = Tq + (size_t)ch * 4096;
#pragma unroll
            for (int i = 0; i < 4; ++i) q.c[i] = ws::ldg_nt(p + i * 1024);
            q.s = *(const uint4*)(Ts + (size_t)ch * 128);
            const uint4* xb = (const uint4*)(X + (size_t)ch * 8 * FRAG_STEP_BYTES);
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
            const bf16x8_t B = ws::as_bf(ws::i8x8_bf16((i & 1) ? make_uint2(cc.z, cc.w) : make_uint2(cc.x, cc.y)));
            f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws::as_bf(xh), B, p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws::as_bf(xl), B, p, 0, 0, 0);
            const float sc = f16_to_f32((uint16_t)((i & 1) ? (sw[i >> 1] >> 16) : (sw[i >> 1] & 0xffffu)));
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += sc * p[j];
        }
    };
    // the RMSNorm fold: lane t < 16 takes row t's rstd over the segment holding this split's columns
    float rstd = 0.f;
    if (a.rms_ssq && r < a.T) {
        const float* qs = a.rms_ssq + ((size_t)((c0 * 256) / a.rms_seg) * 16 + r) * a.rms_nsl;
        float sum = 0.f;
        for (int i = 0; i < a.rms_nsl; ++i) sum += qs[i];
        rstd = 1.f / sqrtf(sum * a.rms_inv + a.rms_eps);
    }
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
    if (a.rms_ssq)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= __shfl(rstd, 4 * g + j, 64);

    // lane holds Y[t = 4 g + j][m0 + r]
    if (!GLU && (a.mode == SK_F32 || a.mode == SK_PARTIAL)) {
        if (!own) return;
        const int m = m0 + r;
        float* dst = (float*)G.out + m;
        float bias = 0.f;
        if (a.mode == SK_PARTIAL) dst += (size_t)split * a.part_stride;
        else if (G.bias) bias = bf16_to_f32(G.bias[m]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * g + j < a.T) dst[(size_t)(4 * g + j) * G.ld] = acc[j] + bias;
        return;
    }
    __syncthreads();   // every wave is done with the fragment slabs that tile_all reuses
#pragma unroll
    for (int j = 0; j < 4; ++j) tile_all[wave][4 * g + j][r] = acc[j];
    // from here the tile is read as [t = lane % 16][column 4 (lane / 16) + j]: other lanes' writes
    const int t = lane & 15, mc = m0 + 4 * g;
    if constexpr (GLU) {
        __syncthreads();   // the up tile of the pair is in its wave's LDS
        if (up) return;
        const float(*ut)[17] = tile_all[wave + 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = tile_all[wave][t][4 * g + j], u = ut[t][4 * g + j];
            tile_all[wave][t][4 * g + j] = a.mode == SK_FRAG_GEGLU ? gelu_tanh(v) * u : silu(v) * u;
        }
    } else {   // SK_FRAG_GELU
        __builtin_amdgcn_wave_barrier();   // LDS is in order within a wave: the reads below see the writes
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = tile_all[wave][t][4 * g + j];
            tile_all[wave][t][4 * g + j] = gelu_erf(v + (G.bias ? bf16_to_f32(G.bias[mc + j]) : 0.f));
        }
    }
    __builtin_amdgcn_wave_barrier();   // LDS is in order within a wave: the reads below see the writes
    if (lane < 32 && own) {
        const int tt = lane >> 1, h = lane & 1;
        if (tt < a.T) {
            float vals[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[e] = tile_all[wave][tt][8 * h + e];
            frag_store8((uint8_t*)G.out, tt, m0 + 8 * h, vals);
        }
    }
}

}  // namespace

hipError_t launch_skinny(const SkinnyArgs& a, int wtype, int nwg, hipStream_t st) {
    const bool glu = (a.mode == SK_FRAG_GEGLU || a.mode == SK_FRAG_SWIGLU);
    if (!a.zeros) return hipErrorInvalidValue;
    if (a.ln_stats) {   // the LayerNorm fold: bf16, one matrix, every group with its c1 / c2, not a residual update;
                        // the RMSNorm fold: bf16, one or two matrices (a gated unit), no c1 / c2
        if (wtype != SKW_BF16 || (glu && !a.ln_rms) || a.ln_tiles < 1 || a.ln_tiles > LN_MAX_TILES / a.nb ||
            a.mode == SK_RESID)
            return hipErrorInvalidValue;
        for (int i = 0; i < a.ngroups; ++i)
            if (!a.g[i].c12 != (a.ln_rms != 0)) return hipErrorInvalidValue;
    }
    if (a.sa.qkv &&   // the self-attention tail: a LayerNorm-folded unsplit q | k | v product of whole heads
        (!a.ln_stats || a.mode != SK_F32 || a.S != 1 || a.ngroups != 3 || !a.satick || a.nb != a.sa.nb ||
         (a.sa.hd != 64 && a.sa.hd != 128) || a.sa.T < 1 || a.sa.T > 16 || a.sa.D % a.sa.hd ||
         32 * (a.sa.hd + 4) * 4 + 16 * (a.sa.hd + 4) * 4 + 16 * 17 * 4 > LN_MAX_TILES * 16 * 8))
        return hipErrorInvalidValue;
    if (a.mode == SK_RESID && (wtype != SKW_BF16 || a.S < 1 || !a.rx || !a.rbase || !a.ryscale == !a.ryw || !a.rstats ||
                               a.ngroups != 1 || (a.S > 1 && (!a.rpart || !a.rtick))))
        return hipErrorInvalidValue;
    if (a.rms_ssq && (wtype != SKW_Q8_0 || a.rms_nsl < 1 || a.rms_seg < 256 || a.rms_seg % 256 ||
                      a.K % a.rms_seg || a.K / a.rms_seg > 2 || a.rms_seg % (a.K / a.S)))   // a split in one segment
        return hipErrorInvalidValue;
    if (wtype == SKW_BF16) return glu ? launch_nt<2, SKW_BF16>(a, nwg, st) : launch_nt<1, SKW_BF16>(a, nwg, st);
    if (a.mode == SK_RESID) return hipErrorInvalidValue;
    // Q8_0: whole chunks of 256 columns per split, one block of at most 16 rows, whole slabs (SK_F32 / FRAG: S = 1)
    if (a.nb != 1 || a.T < 1 || a.T > 16 || a.S < 1 || a.K % (256 * a.S) ||
        (a.mode != SK_PARTIAL && a.S != 1))
        return hipErrorInvalidValue;
    for (int i = 0; i < a.ngroups; ++i)
        if (a.g[i].M % 16 || !a.g[i].Wd || (glu && !a.g[i].W2d)) return hipErrorInvalidValue;
    if (glu) skinny_ws_kernel<true><<<nwg, SK_WS_WAVES * 64, 0, st>>>(a);
    else skinny_ws_kernel<false><<<nwg, SK_WS_WAVES * 64, 0, st>>>(a);
    return hipGetLastError();
}
