// k_attn.hip — K4: the drafter's attention kernels.
//
//  attn_split    up to 16 query rows of one head against one chunk of keys (cache rows, then optional extra f32
//                rows): scores, chunk max, exp-sum and the unnormalised P·V, written as a partial; both products run
//                on the matrix cores (f32 caches split into f16 hi + lo). Splitting the key
//                range across work-groups (flash-decoding) removes the page's 4096-key shared-memory cap and gives
//                long contexts enough work-groups; the queries' own head-norm + RoPE (or the sum of their split-K
//                partials) is rebuilt per work-group so it needs no extra launch.
//  attn_merge    log-sum-exp merge of the chunk partials (the online-softmax rescale of the MTP page's WG_ATTN),
//                optional sigmoid output gate, fragments out.
//  kv_final      context rows' K/V: per-head RMSNorm + RoPE on K, both rows stored to the cache (f16 or f32).
//  mtp_prep      MTP q/k head-norm + NEOX partial RoPE and the K/V cache write at pos0 + m (WG_QKPREP).
#include "fm_device.h"
#include "fm_kernels.h"

#include <type_traits>

namespace {

constexpr int MAX_QSLABS = 4;   // split-K slabs of q summed in the prologue

// native 4 x u32 vector: arrays of it stay in registers where arrays of the HIP uint4 class may not
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ── split-L attention on the matrix cores, one key run per wave (f16 cache, V tiled by 32 positions) ─
// A work-group of 4 waves builds the head's queries once (thread (query t, segment) holds hd/16 consecutive values:
// the sum of up to 4 split-K slabs, head-RMSNorm by a 16-lane shuffle, interleaved RoPE in the thread, f16 hi + lo
// into LDS); after one barrier each wave works alone on its own run of 32-key steps, with no further barrier:
//   loads   32 K rows and the head's block of the 32-position V tile (contiguous in the tiled cache) as whole 1 KB
//           instructions, one step ahead, parked in the wave's LDS tiles (keys past the end zeroed);
//   scores  Sᵀ[j][t] on v_mfma_f32_16x16x32_f16, A = K rows from LDS, B = the queries' hi and lo halves (kept in
//           registers for the whole run);
//   softmax online over the run: lanes of one query reduce by shuffles; the score accumulator of lane (t, g) holds
//           keys 4g..4g+3 and 16+4g..16+4g+3 of the step, exactly the 8 values the A operand of the 32-key P.V
//           product needs in that key order, so P never leaves registers (hi + lo halves);
//   P.V     B = V read from the wave's LDS tile in the same key order (two 8-byte reads per dimension tile).
// Each wave writes its run's (o, max, sum) partial; runs past the end write an empty one (max = -inf).
template <int HD>
__global__ __launch_bounds__(256) void attn_wave_kernel(AttnArgs a) {
    constexpr int QROW = HD + 8;                 // q LDS row (halfs)
    constexpr int KP = HD / 8 + 1;               // uint4 per LDS K row (+1 pad)
    constexpr int VP = 5;                        // uint4 per LDS V dimension row: 32 keys = 4, +1 pad
    constexpr int NS = HD / 32;                  // score k-steps
    constexpr int ND = HD / 16;                  // dimension tiles
    constexpr int RPI = 512 / HD;                // K rows per 1 KB load instruction
    constexpr int LPR = 64 / RPI;                // lanes per K row
    constexpr int KLD = 32 / RPI;                // K load instructions per step
    constexpr int VLD = HD / 16;                 // V load instructions per step (16 dimensions each)
    constexpr int QS = HD / 16;
    const int h = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nq = a.nq;
    const int kh = h / (a.heads / a.kv_heads);
    const QPrep& qp = a.qp;
    __shared__ u32x4_t Klds_all[4][32 * KP];
    __shared__ u32x4_t Vlds_all[4][HD * VP];
    static_assert(2 * 16 * QROW * 2 <= (int)sizeof(Klds_all), "q rows alias the K tiles");
    _Float16* Qh = (_Float16*)&Klds_all[0][0];   // the queries live in the K tiles until every wave holds them
    _Float16* Ql = Qh + 16 * QROW;
    u32x4_t* Klds = Klds_all[wave];
    u32x4_t* Vlds = Vlds_all[wave];

    const int ncache = a.key_hi - a.key_lo;
    const int nsteps = (ncache + 31) >> 5;
    const int run = blockIdx.x * 4 + wave;
    const int s_first = run * a.cpw;
    const int s_end = min(s_first + a.cpw, nsteps);   // may be <= s_first: an empty run

    u32x4_t kr[KLD], vr[VLD];
    auto load_step = [&](int st) {
        const int k0 = st * 32;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int row = i * RPI + lane / LPR;
            const int kidx = min(k0 + row, ncache - 1);
            kr[i] = *((const u32x4_t*)((const uint16_t*)a.kc + (size_t)(a.key_lo + kidx) * a.kv_ld + (size_t)kh * HD) +
                      lane % LPR);
        }
        // V: the step's 32-position tile, this head's HD dimensions x 64 bytes, contiguous (16 dims per instruction)
        const uint16_t* vt = (const uint16_t*)a.vc + ((size_t)((a.key_lo + k0) >> 5) * a.vt_ld + (size_t)kh * HD) * 32;
#pragma unroll
        for (int i = 0; i < VLD; ++i) vr[i] = *((const u32x4_t*)(vt + (16 * i) * 32) + lane);
    };
    load_step(min(s_first, nsteps - 1));

    // queries (once per work-group)
    {
        const int qt = tid >> 4, qseg = tid & 15, tq = min(qt, nq - 1);
        float q[QS], nw[QS], cs[QS / 2], sn[QS / 2];
        const float* src = qp.q + (size_t)tq * qp.q_ld + (size_t)h * qp.q_hs + qseg * QS;
        const int parts = qp.parts > 1 ? qp.parts : 1;
#pragma unroll
        for (int j = 0; j < QS; ++j) q[j] = 0.f;
#pragma unroll
        for (int pp = 0; pp < MAX_QSLABS; ++pp) {   // every slab load issued together; absent slabs re-read slab 0
            const float m = pp < parts ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < QS / 4; ++j) {
                const float4 f = ((const float4*)(src + (pp < parts ? pp : 0) * qp.pstride))[j];
                q[4 * j] += m * f.x; q[4 * j + 1] += m * f.y; q[4 * j + 2] += m * f.z; q[4 * j + 3] += m * f.w;
            }
        }
        const float* rt = qp.rope ? qp.rope_tab + (size_t)(qp.pos_base + tq) * HD + qseg * (QS / 2) : qp.zeros;
        const float* rs = qp.rope ? rt + HD / 2 : qp.zeros;
#pragma unroll
        for (int j = 0; j < QS / 2; ++j) { cs[j] = rt[j]; sn[j] = rs[j]; }
        const uint16_t* nb = qp.norm_bf16 ? qp.norm_bf16 + qseg * QS : (const uint16_t*)qp.zeros;
        const float* nf = qp.norm_f32 ? qp.norm_f32 + qseg * QS : qp.zeros;
#pragma unroll
        for (int j = 0; j < QS; ++j) nw[j] = qp.norm_bf16 ? bf16_to_f32(nb[j]) : nf[j];
        if (qp.norm_bf16 || qp.norm_f32) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < QS; ++j) ss += q[j] * q[j];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
            const float rr = 1.f / sqrtf(ss / (float)HD + qp.eps);
#pragma unroll
            for (int j = 0; j < QS; ++j) q[j] *= nw[j] * rr;
        }
        if (qp.rope) {
#pragma unroll
            for (int j = 0; j < QS / 2; ++j) {
                const float x0 = q[2 * j], x1 = q[2 * j + 1];
                q[2 * j] = x0 * cs[j] - x1 * sn[j];
                q[2 * j + 1] = x1 * cs[j] + x0 * sn[j];
            }
        }
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const float x = qt < nq ? q[j] : 0.f;
            const _Float16 hi = (_Float16)x;
            Qh[qt * QROW + qseg * QS + j] = hi;
            Ql[qt * QROW + qseg * QS + j] = (_Float16)(x - (float)hi);
        }
    }
    __syncthreads();
    f16x8_t qh[NS], ql[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        qh[s] = *(const f16x8_t*)(Qh + r * QROW + 32 * s + 8 * g);
        ql[s] = *(const f16x8_t*)(Ql + r * QROW + 32 * s + 8 * g);
    }
    __syncthreads();   // every wave holds its query operands: the K tiles are free

    float m_run = -INFINITY, l_run = 0.f;   // of query t = r (replicated over g)
    f32x4_t o[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int st = s_first; st < s_end; ++st) {
        const int k0 = st * 32;
        // park this step's K rows and V dimension rows (keys past the end zeroed) in the wave's LDS tiles
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < KLD; ++i) Klds[(i * RPI + lane / LPR) * KP + lane % LPR] = kr[i];
        {
            const int p = k0 + (lane & 3) * 8;
            u32x4_t msk = u32x4_t{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
            if (p + 8 > ncache) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    msk[e] = (p + 2 * e < ncache ? 0xffffu : 0u) | (p + 2 * e + 1 < ncache ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int i = 0; i < VLD; ++i) Vlds[(16 * i + (lane >> 2)) * VP + (lane & 3)] = vr[i] & msk;
        }
        __builtin_amdgcn_wave_barrier();
        load_step(min(st + 1, s_end - 1));   // the run's last step re-reads itself: no conditional load
        // scores of the step's two 16-key tiles
        f32x4_t sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const f16x8_t A = __builtin_bit_cast(f16x8_t, Klds[(16 * kt + r) * KP + 4 * s + g]);
                sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[s], sc[kt], 0, 0, 0);
                sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql[s], sc[kt], 0, 0, 0);
            }
        }
        // online softmax of query r over the step's keys 16 kt + 4 g + i
        float sv[2][4], cm = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kidx = k0 + 16 * kt + 4 * g + i;
                float v = sc[kt][i] * a.scale;
                if (kidx >= ncache) v = -INFINITY;
                if (a.causal_base >= 0 && a.key_lo + kidx > a.causal_base + r) v = -INFINITY;
                sv[kt][i] = v;
                cm = fmaxf(cm, v);
            }
        cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        const float m_new = fmaxf(m_run, cm);
        const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
        f16x8_t ph, pl;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = (m_new == -INFINITY) ? 0.f : expf(sv[kt][i] - m_new);
                const _Float16 hi = (_Float16)pv;
                ph[4 * kt + i] = hi;
                pl[4 * kt + i] = (_Float16)(pv - (float)hi);
                ls += pv;
            }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * alpha + ls;
        m_run = m_new;
        float al[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 4 * g + j, 64);
        // O = alpha O + P V, V from the LDS tile in the same key order as P
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint2* vrow = (const uint2*)(Vlds + (16 * dt + r) * VP);
            const uint2 v0 = vrow[g], v1 = vrow[4 + g];
            const f16x8_t B = __builtin_bit_cast(f16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
            for (int j = 0; j < 4; ++j) o[dt][j] *= al[j];
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, B, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, o[dt], 0, 0, 0);
        }
    }
    // the run's partial: unnormalised o, running max, running sum (an empty run: max -inf, sum 0, o 0)
    float* out = a.part + ((size_t)h * a.nchunks + run) * nq * (HD + 2);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 4 * g + j;
            if (t < nq) out[(size_t)t * (HD + 2) + 16 * dt + r] = o[dt][j];
        }
    if (g == 0 && r < nq) {
        out[(size_t)r * (HD + 2) + HD] = m_run;
        out[(size_t)r * (HD + 2) + HD + 1] = l_run;
    }
}

// ── split-L attention on the matrix cores (f32 cache, grouped queries) ─────────────────────────────
// One work-group = one kv head x one chunk of 32 keys (cache rows, then the optional extra f32 rows), 4 waves, for
// all G = heads / kv_heads query heads of the group at once (G * nq <= 16 QT rows, row t = head-in-group * nq + m),
// so each K/V element is read once per chunk. K and V are split f32 -> f16 hi + lo on their way into LDS (V
// transposed), the queries likewise; scores take K_hi q_hi + K_hi q_lo + K_lo q_hi on v_mfma_f32_16x16x32_f16
// (the lo * lo term is below 2^-22 relative), P.V likewise with P split hi + lo. Queries arrive ready (no head-norm,
// no RoPE: the MTP queries are prepared by mtp_prep, the KV-injection has neither). Writes the same per-chunk
// (o, max, sum) partials as the other split kernels.
// The transposed V tile's key order within dimension row dd: the four 8-key groups are permuted by dd / 16, so the
// 2-byte stores of one instruction (64 lanes on 64 consecutive dimensions of one key) spread over 4x more LDS banks
// (rows are 80 bytes apart: without it 16 lanes share a bank); an 8-key group stays contiguous for the 16-byte reads.
// Measured: the KV-injection draft 434 -> 419 us, the MTP pass over a 4096-row cache 527 -> 524 us.
__device__ __forceinline__ int vswz(int dd) { return 8 * ((dd >> 4) & 3); }

template <int HD, int QT>
__global__ __launch_bounds__(256) void attn_split_f32_mfma_kernel(AttnArgs a) {
    constexpr int C = 32;
    constexpr int KROW = HD + 8, VROW = C + 8, QROW = HD + 8, PROW = C + 8;
    constexpr int NQR = 16 * QT;                 // query rows held
    constexpr int V4 = HD / 4;                   // float4 per key row
    constexpr int LDK = C * V4 / 256;            // float4 of K (and of V) per thread
    constexpr int LDQ = NQR * V4 / 256;          // float4 of q per thread
    static_assert(LDK >= 1 && LDQ >= 1, "shape");
    // hd = 256 with one query tile: the two waves that compute scores read their query operands straight into
    // registers, and the query tiles leave LDS (96 -> 79 KB: two work-groups per CU instead of one; the MTP pass at
    // M = 1 over a 4096-row cache 419 -> 416 us). At hd = 128 (already three per CU) it cost 0.7 us per draft.
    constexpr bool QREG = QT == 1 && HD == 256;
    constexpr int NSQ = HD / 32;
    const int c = blockIdx.x, kh = blockIdx.y;
    const int nq = a.nq;
    const int G = a.heads / a.kv_heads;
    const int Q = G * nq;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const QPrep& qp = a.qp;
    __shared__ __attribute__((aligned(16))) _Float16 Kh[C * KROW], Kl[C * KROW];
    __shared__ __attribute__((aligned(16))) _Float16 Vth[HD * VROW], Vtl[HD * VROW];
    __shared__ __attribute__((aligned(16))) _Float16 Qh[QREG ? 8 : NQR * QROW], Ql[QREG ? 8 : NQR * QROW];
    __shared__ __attribute__((aligned(16))) _Float16 Ph[NQR * PROW], Pl[NQR * PROW];
    __shared__ float S[NQR][C + 1];

    const int ncache = a.key_hi - a.key_lo;
    const int ntot = ncache + a.nx;
    const int k0 = c * C;

    // 1. every global load up front
    float4 kr[LDK], vr[LDK], qr[LDQ];
#pragma unroll
    for (int i = 0; i < LDK; ++i) {
        const int u = tid + 256 * i, row = u / V4, c4 = u % V4;
        const int kidx = min(k0 + row, ntot - 1);
        const bool fc = kidx < ncache;
        const float* kb = fc ? (const float*)a.kc + (size_t)(a.key_lo + kidx) * a.kv_ld
                             : a.kx + (size_t)(kidx - ncache) * a.x_ld;
        const float* vb = fc ? (const float*)a.vc + (size_t)(a.key_lo + kidx) * a.kv_ld
                             : a.vx + (size_t)(kidx - ncache) * a.x_ld;
        kr[i] = *((const float4*)(kb + (size_t)kh * HD) + c4);
        vr[i] = *((const float4*)(vb + (size_t)kh * HD) + c4);
    }
    const int fr = lane & 15, fk = 8 * (lane >> 4);
    float4 qf[QREG ? 2 * NSQ : 1];   // QREG: this lane's query operand values (row fr, columns 32 s + fk .. + 7)
    if constexpr (QREG) {
        const int hl = fr / nq, m = fr - hl * nq;
        const float* src = fr < Q ? qp.q + (size_t)m * qp.q_ld + (size_t)(kh * G + hl) * qp.q_hs : qp.zeros;
        if (wave < 2)   // the score waves (a wave-uniform branch)
#pragma unroll
            for (int s = 0; s < NSQ; ++s) {
                qf[2 * s] = *(const float4*)(src + 32 * s + fk);
                qf[2 * s + 1] = *(const float4*)(src + 32 * s + fk + 4);
            }
    } else {
#pragma unroll
        for (int i = 0; i < LDQ; ++i) {
            const int u = tid + 256 * i, t = u / V4, c4 = u % V4;
            const int hl = t / nq, m = t - hl * nq;
            const float* src = t < Q ? qp.q + (size_t)m * qp.q_ld + (size_t)(kh * G + hl) * qp.q_hs : qp.zeros;
            qr[i] = *((const float4*)src + c4);
        }
    }
    // 2. hi/lo f16 splits into LDS: K row-major, V transposed (dim-major), queries row-major
#pragma unroll
    for (int i = 0; i < LDK; ++i) {
        const int u = tid + 256 * i, row = u / V4, d = 4 * (u % V4);
        const float kv[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
        const float vv[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const _Float16 hk = (_Float16)kv[e], hv = (_Float16)vv[e];
            Kh[row * KROW + d + e] = hk;
            Kl[row * KROW + d + e] = (_Float16)(kv[e] - (float)hk);
            const int vo = (d + e) * VROW + (row ^ vswz(d + e));
            Vth[vo] = hv;
            Vtl[vo] = (_Float16)(vv[e] - (float)hv);
        }
    }
#pragma unroll
    for (int i = 0; i < (QREG ? 0 : LDQ); ++i) {
        const int u = tid + 256 * i, t = u / V4, d = 4 * (u % V4);
        const float qv[4] = {qr[i].x, qr[i].y, qr[i].z, qr[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = t < Q ? qv[e] : 0.f;
            const _Float16 h = (_Float16)x;
            Qh[t * QROW + d + e] = h;
            Ql[t * QROW + d + e] = (_Float16)(x - (float)h);
        }
    }
    __syncthreads();
    // 3. scores Sᵀ[j][t]: (key tile, query tile) pairs over the waves
    for (int pr = wave; pr < 2 * QT; pr += 4) {
        const int kt = pr & 1, qt = pr >> 1;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < HD / 32; ++s) {
            const f16x8_t Ah = *(const f16x8_t*)(Kh + (kt * 16 + fr) * KROW + s * 32 + fk);
            const f16x8_t Al = *(const f16x8_t*)(Kl + (kt * 16 + fr) * KROW + s * 32 + fk);
            f16x8_t Bh, Bl;
            if constexpr (QREG) {
                const float x[8] = {qf[2 * s].x, qf[2 * s].y, qf[2 * s].z, qf[2 * s].w,
                                    qf[2 * s + 1].x, qf[2 * s + 1].y, qf[2 * s + 1].z, qf[2 * s + 1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 h = (_Float16)x[e];
                    Bh[e] = h;
                    Bl[e] = (_Float16)(x[e] - (float)h);
                }
            } else {
                Bh = *(const f16x8_t*)(Qh + (qt * 16 + fr) * QROW + s * 32 + fk);
                Bl = *(const f16x8_t*)(Ql + (qt * 16 + fr) * QROW + s * 32 + fk);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bh, acc, 0, 0, 0);
        }
        // lane holds keys j = 16 kt + 4 (lane / 16) + i for query row t = 16 qt + lane % 16
        const int t = qt * 16 + fr;
        const int m = t % nq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = kt * 16 + 4 * (lane >> 4) + i;
            const int kidx = k0 + j;
            float v = acc[i] * a.scale;
            if (kidx >= ntot) v = -INFINITY;
            if (a.causal_base >= 0 && kidx < ncache && a.key_lo + kidx > a.causal_base + m) v = -INFINITY;
            S[t][j] = v;
        }
    }
    __syncthreads();
    // 4. softmax statistics: 4 threads per query row, 8 keys each; P = exp(S - m) split hi/lo
    {
        const int t = tid >> 2, q4 = tid & 3;
        if (t < NQR) {
            float sv[C / 4], mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < C / 4; ++i) { sv[i] = S[t][q4 * (C / 4) + i]; mx = fmaxf(mx, sv[i]); }
            mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
            float l = 0.f;
#pragma unroll
            for (int i = 0; i < C / 4; ++i) {
                const float p = (mx == -INFINITY || t >= Q) ? 0.f : expf(sv[i] - mx);
                const _Float16 h = (_Float16)p;
                Ph[t * PROW + q4 * (C / 4) + i] = h;
                Pl[t * PROW + q4 * (C / 4) + i] = (_Float16)(p - (float)h);
                l += p;
            }
            l += __shfl_xor(l, 1, 64);
            l += __shfl_xor(l, 2, 64);
            if (q4 == 0 && t < Q) {
                const int hl = t / nq, m = t - hl * nq;
                float* out = a.part + (((size_t)(kh * G + hl) * a.nchunks + c) * nq + m) * (HD + 2);
                out[HD] = mx;
                out[HD + 1] = l;
            }
        }
    }
    __syncthreads();
    // 5. O = P V: (query tile, dim tile) pairs over the waves, one 32-key step each
    for (int pr = wave; pr < QT * (HD / 16); pr += 4) {
        const int qt = pr / (HD / 16), dt = pr % (HD / 16);
        const f16x8_t Ah = *(const f16x8_t*)(Ph + (qt * 16 + fr) * PROW + fk);
        const f16x8_t Al = *(const f16x8_t*)(Pl + (qt * 16 + fr) * PROW + fk);
        const int vo = (dt * 16 + fr) * VROW + (fk ^ vswz(dt * 16 + fr));
        const f16x8_t Bh = *(const f16x8_t*)(Vth + vo);
        const f16x8_t Bl = *(const f16x8_t*)(Vtl + vo);
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bh, acc, 0, 0, 0);
        // lane holds O[t = 16 qt + 4 (lane / 16) + i][d = 16 dt + lane % 16]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = qt * 16 + 4 * (lane >> 4) + i;
            if (t < Q) {
                const int hl = t / nq, m = t - hl * nq;
                a.part[(((size_t)(kh * G + hl) * a.nchunks + c) * nq + m) * (HD + 2) + dt * 16 + fr] = acc[i];
            }
        }
    }
}

// One work-group per (head, query row): thread (4-dim group, chunk group) folds its chunks with the online
// rescale, four chunks' loads in flight at a time; the chunk groups are then folded in LDS, one thread per
// dimension. NTH threads: 1024 when 256 would leave a thread more than two rounds of four chunks (many partials),
// so that every partial's load is in flight at once.
template <int HD, int NTH>
__global__ __launch_bounds__(NTH) void attn_merge_kernel(MergeArgs a) {
    constexpr int DV = HD / 4, G = NTH / DV;
    const int h = blockIdx.x, t = blockIdx.y;
    const int d4 = threadIdx.x % DV, cg = threadIdx.x / DV;
    const int nc = a.nchunks;
    const float* base = a.part + (size_t)h * nc * a.nq * (HD + 2) + (size_t)t * (HD + 2);
    const size_t cstride = (size_t)a.nq * (HD + 2);
    float M = -INFINITY, Ls = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = cg; c0 < nc; c0 += 4 * G) {
        float4 o[4];
        float m[4], l[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * G;
            const int cc = c < nc ? c : cg;
            const float* p = base + (size_t)cc * cstride;
            o[u] = *(const float4*)(p + 4 * d4);
            m[u] = c < nc ? p[HD] : -INFINITY;
            l[u] = p[HD + 1];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (m[u] == -INFINITY) continue;
            const float Mn = fmaxf(M, m[u]);
            const float a0 = (M == -INFINITY) ? 0.f : expf(M - Mn), a1 = expf(m[u] - Mn);
            Ls = Ls * a0 + l[u] * a1;
            O.x = O.x * a0 + o[u].x * a1; O.y = O.y * a0 + o[u].y * a1;
            O.z = O.z * a0 + o[u].z * a1; O.w = O.w * a0 + o[u].w * a1;
            M = Mn;
        }
    }
    __shared__ float sm[G], sl[G];
    __shared__ float so[G][HD];
    __shared__ float fo[HD];
    if (d4 == 0) { sm[cg] = M; sl[cg] = Ls; }
    so[cg][4 * d4] = O.x; so[cg][4 * d4 + 1] = O.y; so[cg][4 * d4 + 2] = O.z; so[cg][4 * d4 + 3] = O.w;
    __syncthreads();
    if (threadIdx.x < HD) {   // dimension d over the chunk groups, in group order
        const int d = threadIdx.x;
        float MM = -INFINITY;
#pragma unroll
        for (int g = 0; g < G; ++g) MM = fmaxf(MM, sm[g]);
        float L = 0.f, od = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float w = sm[g] == -INFINITY ? 0.f : expf(sm[g] - MM);
            L += w * sl[g];
            od += w * so[g][d];
        }
        fo[d] = od * (1.f / L);
    }
    __syncthreads();
    if (threadIdx.x < HD / 8) {
        const int d0 = threadIdx.x * 8;
        float o[8], gt[8];
        const float* gp = a.gate ? a.gate + (size_t)t * a.gate_ld + (size_t)h * a.gate_hs + d0 : nullptr;
#pragma unroll
        for (int e = 0; e < 8; ++e) gt[e] = gp ? gp[e] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[e] = fo[d0 + e];
            if (gp) o[e] *= sigmoidf(gt[e]);
        }
        frag_store8_rows(a.o_frag, a.heads * HD, a.row0 + t, h * HD + d0, o);
    }
}

// ── context K/V rows -> cache ────────────────────────────────────────────────────────────────────
__global__ __launch_bounds__(256) void kv_final_kernel(KVFinalArgs a) {
    const int t = blockIdx.x, l = blockIdx.y;
    const int D = a.D, hd = a.hd, per = hd >> 3;   // threads per head
    const int sn = a.stage_n ? a.stage_n : a.n;   // stage rows per group; this launch's rows start at stage_t0
    const float* krow = a.stage + ((size_t)(2 * l) * sn + a.stage_t0 + t) * D;
    const float* vrow = a.stage + ((size_t)(2 * l + 1) * sn + a.stage_t0 + t) * D;
    const size_t row = (size_t)(a.start + t) * D;
    const size_t kbase = (size_t)(2 * l) * a.max_ctx * D + row;
    const size_t vbase = (size_t)(2 * l + 1) * a.max_ctx * D + row;
    const uint16_t* nw = a.knorm[l];
    const uint16_t* nwp = nw ? nw : (const uint16_t*)a.zeros;
    const float* tr = nw ? a.rope_tab + (size_t)(a.start + t) * a.rope_dims : a.zeros;
    for (int slot = threadIdx.x; slot < D / 8; slot += 256) {
        const int i0 = slot * 8, d0 = i0 % hd;
        float k[8], v[8], wn[8], cs[4], sn[4];
        const int half = nw ? a.rope_dims >> 1 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) { k[e] = krow[i0 + e]; v[e] = vrow[i0 + e]; wn[e] = bf16_to_f32(nwp[d0 + e]); }
#pragma unroll
        for (int e = 0; e < 4; ++e) { cs[e] = tr[(d0 >> 1) + e]; sn[e] = tr[half + (d0 >> 1) + e]; }
        if (nw) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += k[e] * k[e];
            for (int o = 1; o < per; o <<= 1) ss += __shfl_xor(ss, o, 64);
            const float r = 1.f / sqrtf(ss / (float)hd + a.eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) k[e] *= wn[e] * r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float c = cs[e], s = sn[e];
                const float x0 = k[2 * e], x1 = k[2 * e + 1];
                k[2 * e] = x0 * c - x1 * s;
                k[2 * e + 1] = x1 * c + x0 * s;
            }
        }
        if (a.kv_dtype == 0) {
            uint32_t kw[4], vw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kw[e] = (uint32_t)f32_to_f16(k[2 * e]) | ((uint32_t)f32_to_f16(k[2 * e + 1]) << 16);
                vw[e] = (uint32_t)f32_to_f16(v[2 * e]) | ((uint32_t)f32_to_f16(v[2 * e + 1]) << 16);
            }
            *(uint4*)((uint16_t*)a.cache + kbase + i0) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
            // f16 V is tiled [pos / 32][dim][32]: dims i0 .. i0 + 7 of position start + t
            const int pos = a.start + t;
            uint16_t* vt = (uint16_t*)a.cache + (size_t)(2 * l + 1) * a.max_ctx * D +
                           ((size_t)(pos >> 5) * D + i0) * 32 + (pos & 31);
#pragma unroll
            for (int e = 0; e < 8; ++e) vt[e * 32] = (uint16_t)(vw[e >> 1] >> (16 * (e & 1)));
        } else {
            float* kc = (float*)a.cache + kbase + i0;
            float* vc = (float*)a.cache + vbase + i0;
#pragma unroll
            for (int e = 0; e < 8; ++e) { kc[e] = k[e]; vc[e] = v[e]; }
        }
    }
}

// ── MTP q/k preparation ──────────────────────────────────────────────────────────────────────────
__global__ __launch_bounds__(256) void mtp_prep_kernel(MtpPrepArgs a) {
    const int m = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
    const int HD = a.HD, NH = a.NH, NKV = a.NKV;
    const int pos = a.pos0 + m;
    __shared__ float red[4];
    __shared__ float sh[256];
    auto sum = [&](const float* p) {   // the S slabs of one element, in slab order
        float v = p[0];
        for (int s = 1; s < a.S; ++s) v += p[(size_t)s * a.slab];
        return v;
    };
    if (j >= NH + NKV) {
        const int vh = j - NH - NKV;
        if (tid < HD) a.vc[(size_t)pos * NKV * HD + vh * HD + tid] = sum(a.vt + (size_t)m * a.vt_ld + vh * HD + tid);
        return;
    }
    float x = 0.f, w = 0.f;
    if (tid < HD) {
        if (j < NH) {
            const size_t qi = (size_t)m * a.qf_ld + (size_t)j * 2 * HD + tid;
            x = sum(a.qf + qi);
            w = a.qn[tid];
            if (a.S > 1) ((float*)a.qf)[qi + HD] = sum(a.qf + qi + HD);   // the gate, for the merge
        } else {
            x = sum(a.kt + (size_t)m * a.kt_ld + (size_t)(j - NH) * HD + tid);
            w = a.kn[tid];
        }
    }
    const float ss = block_sum256(x * x, red);
    const float y = x * (1.f / sqrtf(ss / (float)HD + a.eps)) * w;
    sh[tid] = y;
    __syncthreads();
    float o = y;
    const int half = a.rot >> 1;
    if (tid < a.rot) {
        const int i = tid < half ? tid : tid - half;
        const float* tr = a.rope_tab + (size_t)pos * a.rot;
        const float c = tr[i], s = tr[half + i];
        o = tid < half ? y * c - sh[tid + half] * s : y * c + sh[tid - half] * s;
    }
    if (tid < HD) {
        if (j < NH) a.qout[(size_t)m * NH * HD + (size_t)j * HD + tid] = o;
        else a.kc[(size_t)pos * NKV * HD + (size_t)(j - NH) * HD + tid] = o;
    }
}

}  // namespace


// The f32-cache matrix-core kernel: head widths 128 / 256, queries ready-made, G * nq <= 48.
static bool f32_mfma_fits(const AttnArgs& a) {
    const int G = a.heads / a.kv_heads;
    return a.kv_dtype == 1 && (a.hd == 128 || a.hd == 256) && !a.qp.norm_bf16 && !a.qp.norm_f32 && !a.qp.rope &&
           a.qp.parts <= 1 && G * a.nq <= 48;
}

int attn_chunk_size(int hd, int kv_dtype, int nkeys, int heads) {
    (void)hd;
    (void)kv_dtype;
    (void)nkeys;
    (void)heads;
    return 32;   // the 32-key step of both matrix-core kernels
}

hipError_t launch_attn_split(const AttnArgs& a, hipStream_t st) {
    const int nkeys = a.key_hi - a.key_lo + a.nx;
    if (a.nq < 1 || a.nq > 16 || a.chunk != attn_chunk_size(a.hd, a.kv_dtype, nkeys, a.heads) || !a.qp.zeros ||
        !a.qp.q || nkeys < 1)
        return hipErrorInvalidValue;
    const int tc = (nkeys + a.chunk - 1) / a.chunk;
    // f16 caches: nchunks = key runs per head rounded up to whole 4-wave work-groups; f32 caches: one chunk each
    const int runs = (tc + a.cpw - 1) / a.cpw;
    if (a.cpw < 1 || (a.kv_dtype != 0 && (a.cpw != 1 || a.nchunks != tc)) ||
        (a.kv_dtype == 0 && a.nchunks != (runs + 3) / 4 * 4))
        return hipErrorInvalidValue;
    if (a.qp.rope && a.qp.rope_dims > (a.hd <= 128 ? a.hd : 128)) return hipErrorInvalidValue;
    if (a.nx > 0 && a.kv_dtype == 0) return hipErrorInvalidValue;   // extra rows are f32: f32 caches only
    if (a.qp.parts > MAX_QSLABS || (a.kv_dtype != 0 && a.qp.parts > 1)) return hipErrorInvalidValue;
    if (a.kv_dtype == 0) {
        if (a.qp.rope == 2 || (a.qp.rope == 1 && a.qp.rope_dims != a.hd) || a.nx > 0 || (a.key_lo & 31))
            return hipErrorInvalidValue;
        dim3 gw((a.nchunks + 3) / 4, a.heads);
        if (a.nchunks % 4) return hipErrorInvalidValue;
        switch (a.hd) {
        case 64: attn_wave_kernel<64><<<gw, 256, 0, st>>>(a); break;
        case 128: attn_wave_kernel<128><<<gw, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
        }
    } else if (f32_mfma_fits(a)) {
        const int rows = (a.heads / a.kv_heads) * a.nq;
        dim3 g2(a.nchunks, a.kv_heads);
        if (a.hd == 128) {   // the KV-injection drafter: no grouped queries, at most 16 rows
            if (rows > 16) return hipErrorInvalidValue;
            attn_split_f32_mfma_kernel<128, 1><<<g2, 256, 0, st>>>(a);
        } else {
            if (rows <= 16) attn_split_f32_mfma_kernel<256, 1><<<g2, 256, 0, st>>>(a);
            else if (rows <= 32) attn_split_f32_mfma_kernel<256, 2><<<g2, 256, 0, st>>>(a);
            else attn_split_f32_mfma_kernel<256, 3><<<g2, 256, 0, st>>>(a);
        }
    } else {
        return hipErrorInvalidValue;   // f32 caches: head widths 128 / 256 with ready-made queries
    }
    return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t st) {
    dim3 grid(a.heads, a.nq);
    if (a.hd != 64 && a.hd != 128 && a.hd != 256) return hipErrorInvalidValue;
    // more than two rounds of four chunks per thread at 256 threads (measured: the MTP pass over a 4096-row cache
    // 531 -> 526 us, the KV-injection draft 434 -> 432 us; at two rounds, the flow-map draft at L = 8193, 1024
    // threads were 4 us slower)
    // (head width 64 keeps the 256-thread kernel: no configuration reaches that many partials with it)
    const bool wide = a.hd >= 128 && a.nchunks > 8 * (256 / (a.hd / 4));
    if (wide) {
        if (a.hd == 128) attn_merge_kernel<128, 1024><<<grid, 1024, 0, st>>>(a);
        else attn_merge_kernel<256, 1024><<<grid, 1024, 0, st>>>(a);
    } else {
        if (a.hd == 64) attn_merge_kernel<64, 256><<<grid, 256, 0, st>>>(a);
        else if (a.hd == 128) attn_merge_kernel<128, 256><<<grid, 256, 0, st>>>(a);
        else attn_merge_kernel<256, 256><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_kv_final(const KVFinalArgs& a, hipStream_t st) {
    if (a.hd / 8 > 64 || a.layers > 16) return hipErrorInvalidValue;
    kv_final_kernel<<<dim3(a.n, a.layers), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_mtp_prep(const MtpPrepArgs& a, hipStream_t st) {
    if (a.HD > 256 || a.S < 1 || (a.S > 1 && a.slab < 1)) return hipErrorInvalidValue;
    mtp_prep_kernel<<<dim3(a.M, a.NH + 2 * a.NKV), 256, 0, st>>>(a);
    return hipGetLastError();
}
