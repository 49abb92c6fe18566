// k_attn.hip — K4: the drafter's attention kernels.
//
//  self_attn     flow-map self-attention over the T slots (one work-group per head): per-head q/k RMSNorm,
//                interleaved RoPE at the slots' positions, softmax(q kᵀ / sqrt(hd)) v with no mask
//                (flashmap_drafter.js: headNormRope, attnF32); o leaves as fragments for the o_proj GEMM.
//  attn_split    up to 16 query rows of one head against one chunk of keys (cache rows, then optional extra f32
//                rows): scores, chunk max, exp-sum and the unnormalised P·V, written as a partial. Splitting the key
//                range across work-groups (flash-decoding) removes the page's 4096-key shared-memory cap and gives
//                long contexts enough work-groups; the queries' own head-norm + RoPE (or the sum of their split-K
//                partials) is rebuilt per work-group so it needs no extra launch.
//  attn_merge    log-sum-exp merge of the chunk partials (the online-softmax rescale of the MTP page's WG_ATTN),
//                optional sigmoid output gate, fragments out.
//  kv_final      context rows' K/V: per-head RMSNorm + RoPE on K, both rows stored to the cache (f16 or f32).
//  mtp_prep      MTP q/k head-norm + NEOX partial RoPE and the K/V cache write at pos0 + m (WG_QKPREP).
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

__device__ __forceinline__ float ld_kv(const void* p, size_t i, int dt) {
    return dt == 0 ? f16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// ── self-attention ───────────────────────────────────────────────────────────────────────────────
__global__ __launch_bounds__(256) void self_attn_kernel(SelfAttnArgs a) {
    const int h = blockIdx.x;
    const int T = a.T, hd = a.hd, D = a.D;
    __shared__ float X[3][16][129];   // q, k, v rows of this head (hd <= 128)
    __shared__ float P[16][17];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 3 * T * hd; i += 256) {
        const int w = i / (T * hd), r = i % (T * hd), t = r / hd, d = r % hd;
        X[w][t][d] = a.qkv[(size_t)t * 3 * D + (size_t)w * D + (size_t)h * hd + d];
    }
    __syncthreads();
    // head RMSNorm of the q and k rows (one wave per row)
    for (int row = wave; row < 2 * T; row += 4) {
        const int w = row / T, t = row % T;
        const uint16_t* nw = w == 0 ? a.qn : a.kn;
        float ss = 0.f;
        for (int d = lane; d < hd; d += 64) ss += X[w][t][d] * X[w][t][d];
        ss = wave_sum(ss);
        const float r = 1.f / sqrtf(ss / (float)hd + a.eps);
        for (int d = lane; d < hd; d += 64) X[w][t][d] = X[w][t][d] * (bf16_to_f32(nw[d]) * r);
    }
    __syncthreads();
    // interleaved RoPE: pairs (2i, 2i+1) at position pos_base + t
    const int half = hd >> 1;
    for (int i = tid; i < 2 * T * half; i += 256) {
        const int row = i / half, pi = i % half, w = row / T, t = row % T;
        const float* tr = a.rope_tab + (size_t)(a.pos_base + t) * hd;
        const float c = tr[pi], s = tr[half + pi];
        const float x0 = X[w][t][2 * pi], x1 = X[w][t][2 * pi + 1];
        X[w][t][2 * pi] = x0 * c - x1 * s;
        X[w][t][2 * pi + 1] = x1 * c + x0 * s;
    }
    __syncthreads();
    {
        const int t = tid >> 4, u = tid & 15;
        if (t < T && u < T) {
            float s = 0.f;
            for (int d = 0; d < hd; ++d) s += X[0][t][d] * X[1][u][d];
            P[t][u] = s * a.scale;
        }
    }
    __syncthreads();
    if (tid < T) {
        float m = -INFINITY;
        for (int u = 0; u < T; ++u) m = fmaxf(m, P[tid][u]);
        float z = 0.f;
        for (int u = 0; u < T; ++u) { const float e = expf(P[tid][u] - m); P[tid][u] = e; z += e; }
        const float iz = 1.f / z;
        for (int u = 0; u < T; ++u) P[tid][u] *= iz;
    }
    __syncthreads();
    const int per = hd >> 3;
    for (int slot = tid; slot < T * per; slot += 256) {
        const int t = slot / per, d0 = (slot % per) * 8;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        for (int u = 0; u < T; ++u) {
            const float p = P[t][u];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += p * X[2][u][d0 + e];
        }
        frag_store8(a.o_frag, t, h * hd + d0, o);
    }
}

// ── query preparation shared by the split kernel ─────────────────────────────────────────────────
template <int HD>
__device__ void prep_queries(const QPrep& qp, int h, int nq, float (*qs)[HD]) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < nq * HD; i += 256) {
        const int t = i / HD, d = i % HD;
        const size_t off = (size_t)t * qp.q_ld + (size_t)h * qp.q_hs + d;
        float v;
        if (qp.part) {
            v = 0.f;
            for (int s = 0; s < qp.S; ++s) v += qp.part[(size_t)s * qp.part_stride + off];
        } else {
            v = qp.q[off];
        }
        qs[t][d] = v;
    }
    __syncthreads();
    if (qp.norm_bf16 || qp.norm_f32) {
        for (int t = wave; t < nq; t += 4) {
            float ss = 0.f;
            for (int d = lane; d < HD; d += 64) ss += qs[t][d] * qs[t][d];
            ss = wave_sum(ss);
            const float r = 1.f / sqrtf(ss / (float)HD + qp.eps);
            for (int d = lane; d < HD; d += 64)
                qs[t][d] *= (qp.norm_bf16 ? bf16_to_f32(qp.norm_bf16[d]) : qp.norm_f32[d]) * r;
        }
        __syncthreads();
    }
    if (qp.rope == 1) {
        const int half = HD / 2;
        for (int i = tid; i < nq * half; i += 256) {
            const int t = i / half, pi = i % half;
            const float* tr = qp.rope_tab + (size_t)(qp.pos_base + t) * qp.rope_dims;
            const float c = tr[pi], s = tr[half + pi];
            const float x0 = qs[t][2 * pi], x1 = qs[t][2 * pi + 1];
            qs[t][2 * pi] = x0 * c - x1 * s;
            qs[t][2 * pi + 1] = x1 * c + x0 * s;
        }
        __syncthreads();
    } else if (qp.rope == 2) {
        const int half = qp.rope_dims / 2;
        for (int i = tid; i < nq * half; i += 256) {
            const int t = i / half, pi = i % half;
            const float* tr = qp.rope_tab + (size_t)(qp.pos_base + t) * qp.rope_dims;
            const float c = tr[pi], s = tr[half + pi];
            const float x0 = qs[t][pi], x1 = qs[t][pi + half];
            qs[t][pi] = x0 * c - x1 * s;
            qs[t][pi + half] = x1 * c + x0 * s;
        }
        __syncthreads();
    }
}

// ── split-L attention ────────────────────────────────────────────────────────────────────────────
template <int HD>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
    constexpr int G = 256 / HD;            // key groups in the P·V pass
    const int c = blockIdx.x, h = blockIdx.y;
    const int nq = a.nq;
    const int kh = h / (a.heads / a.kv_heads);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    __shared__ float qs[16][HD];
    __shared__ float sc[16][256];
    __shared__ float red[G][16][HD];
    __shared__ float mrow[16], lrow[16];

    prep_queries<HD>(a.qp, h, nq, qs);

    const int ncache = a.key_hi - a.key_lo;
    const int ntot = ncache + a.nx;
    const int k0 = c * a.chunk;
    const int cnt = min(a.chunk, ntot - k0);

    // scores: thread j owns key k0 + j
    {
        float s[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) s[t] = 0.f;
        const bool valid = tid < cnt;
        if (valid) {
            const int kidx = k0 + tid;
            const bool from_cache = kidx < ncache;
            const size_t base = from_cache ? (size_t)(a.key_lo + kidx) * a.kv_ld + (size_t)kh * HD
                                           : (size_t)(kidx - ncache) * a.x_ld + (size_t)kh * HD;
            for (int d = 0; d < HD; d += 8) {
                float kk[8];
                if (from_cache) {
                    if (a.kv_dtype == 0) {
                        const uint4 raw = *(const uint4*)((const uint16_t*)a.kc + base + d);
                        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            kk[2 * e] = f16_to_f32((uint16_t)(w[e] & 0xffffu));
                            kk[2 * e + 1] = f16_to_f32((uint16_t)(w[e] >> 16));
                        }
                    } else {
                        const float4* p = (const float4*)((const float*)a.kc + base + d);
                        const float4 x0 = p[0], x1 = p[1];
                        kk[0] = x0.x; kk[1] = x0.y; kk[2] = x0.z; kk[3] = x0.w;
                        kk[4] = x1.x; kk[5] = x1.y; kk[6] = x1.z; kk[7] = x1.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kk[e] = a.kx[base + d + e];
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    if (t < nq) {
                        float acc = s[t];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc += qs[t][d + e] * kk[e];
                        s[t] = acc;
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                s[t] *= a.scale;
                if (a.causal_base >= 0 && from_cache && a.key_lo + kidx > a.causal_base + t) s[t] = -INFINITY;
            }
        }
        if (tid < 256) {
#pragma unroll
            for (int t = 0; t < 16; ++t)
                if (t < nq) sc[t][tid] = valid ? s[t] : -INFINITY;
        }
    }
    __syncthreads();
    // per-query max and exp-sum over the chunk (one wave per query row)
    for (int t = wave; t < nq; t += 4) {
        float m = -INFINITY;
        for (int j = lane; j < a.chunk; j += 64) m = fmaxf(m, sc[t][j]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < a.chunk; j += 64) {
            const float p = (m == -INFINITY) ? 0.f : expf(sc[t][j] - m);
            sc[t][j] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) { mrow[t] = m; lrow[t] = l; }
    }
    __syncthreads();
    // P·V: thread (d, key group kg)
    {
        const int d = tid % HD, kg = tid / HD;
        float o[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) o[t] = 0.f;
        for (int j = kg; j < cnt; j += G) {
            const int kidx = k0 + j;
            float vv;
            if (kidx < ncache) vv = ld_kv(a.vc, (size_t)(a.key_lo + kidx) * a.kv_ld + (size_t)kh * HD + d, a.kv_dtype);
            else vv = a.vx[(size_t)(kidx - ncache) * a.x_ld + (size_t)kh * HD + d];
#pragma unroll
            for (int t = 0; t < 16; ++t)
                if (t < nq) o[t] += sc[t][j] * vv;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t)
            if (t < nq) red[kg][t][d] = o[t];
    }
    __syncthreads();
    float* out = a.part + ((size_t)h * a.nchunks + c) * nq * (HD + 2);
    for (int i = tid; i < nq * HD; i += 256) {
        const int t = i / HD, d = i % HD;
        float v = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) v += red[g][t][d];
        out[(size_t)t * (HD + 2) + d] = v;
    }
    if (tid < nq) {
        out[(size_t)tid * (HD + 2) + HD] = mrow[tid];
        out[(size_t)tid * (HD + 2) + HD + 1] = lrow[tid];
    }
}

__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
    const int h = blockIdx.x;
    const int HD = a.hd, per = HD >> 3;
    const float* base = a.part + (size_t)h * a.nchunks * a.nq * (HD + 2);
    for (int slot = threadIdx.x; slot < a.nq * per; slot += 256) {
        const int t = slot / per, d0 = (slot % per) * 8;
        float M = -INFINITY;
        for (int c = 0; c < a.nchunks; ++c) M = fmaxf(M, base[((size_t)c * a.nq + t) * (HD + 2) + HD]);
        float l = 0.f, o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        for (int c = 0; c < a.nchunks; ++c) {
            const float* p = base + ((size_t)c * a.nq + t) * (HD + 2);
            const float mc = p[HD];
            const float w = (mc == -INFINITY) ? 0.f : expf(mc - M);
            l += w * p[HD + 1];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += w * p[d0 + e];
        }
        const float il = 1.f / l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[e] *= il;
            if (a.gate) o[e] *= sigmoidf(a.gate[(size_t)t * a.gate_ld + (size_t)h * a.gate_hs + d0 + e]);
        }
        frag_store8(a.o_frag, t, h * HD + d0, o);
    }
}

// ── context K/V rows -> cache ────────────────────────────────────────────────────────────────────
__global__ __launch_bounds__(256) void kv_final_kernel(KVFinalArgs a) {
    const int t = blockIdx.x, l = blockIdx.y;
    const int D = a.D, hd = a.hd, per = hd >> 3;   // threads per head
    const float* krow = a.stage + ((size_t)(2 * l) * a.n + t) * D;
    const float* vrow = a.stage + ((size_t)(2 * l + 1) * a.n + t) * D;
    const size_t row = (size_t)(a.start + t) * D;
    const size_t kbase = (size_t)(2 * l) * a.max_ctx * D + row;
    const size_t vbase = (size_t)(2 * l + 1) * a.max_ctx * D + row;
    const uint16_t* nw = a.knorm[l];
    for (int slot = threadIdx.x; slot < D / 8; slot += 256) {
        const int i0 = slot * 8, d0 = i0 % hd;
        float k[8], v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { k[e] = krow[i0 + e]; v[e] = vrow[i0 + e]; }
        if (nw) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += k[e] * k[e];
            for (int o = 1; o < per; o <<= 1) ss += __shfl_xor(ss, o, 64);
            const float r = 1.f / sqrtf(ss / (float)hd + a.eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) k[e] *= bf16_to_f32(nw[d0 + e]) * r;
            const float* tr = a.rope_tab + (size_t)(a.start + t) * a.rope_dims;
            const int half = a.rope_dims >> 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pi = (d0 >> 1) + e;
                const float c = tr[pi], s = tr[half + pi];
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
            *(uint4*)((uint16_t*)a.cache + vbase + i0) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
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
    if (j >= NH + NKV) {
        const int vh = j - NH - NKV;
        if (tid < HD) a.vc[(size_t)pos * NKV * HD + vh * HD + tid] = a.vt[(size_t)m * NKV * HD + vh * HD + tid];
        return;
    }
    float x = 0.f, w = 0.f;
    if (tid < HD) {
        if (j < NH) { x = a.qf[(size_t)m * NH * 2 * HD + (size_t)j * 2 * HD + tid]; w = a.qn[tid]; }
        else { x = a.kt[(size_t)m * NKV * HD + (size_t)(j - NH) * HD + tid]; w = a.kn[tid]; }
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

hipError_t launch_self_attn(const SelfAttnArgs& a, hipStream_t st) {
    if (a.hd > 128 || a.T > 16) return hipErrorInvalidValue;
    self_attn_kernel<<<a.heads, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_attn_split(const AttnArgs& a, hipStream_t st) {
    if (a.chunk > 256 || a.nq > 16) return hipErrorInvalidValue;
    dim3 grid(a.nchunks, a.heads);
    switch (a.hd) {
    case 64: attn_split_kernel<64><<<grid, 256, 0, st>>>(a); break;
    case 128: attn_split_kernel<128><<<grid, 256, 0, st>>>(a); break;
    case 256: attn_split_kernel<256><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t st) {
    attn_merge_kernel<<<a.heads, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_kv_final(const KVFinalArgs& a, hipStream_t st) {
    if (a.hd / 8 > 64 || a.layers > 16) return hipErrorInvalidValue;
    kv_final_kernel<<<dim3(a.n, a.layers), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_mtp_prep(const MtpPrepArgs& a, hipStream_t st) {
    if (a.HD > 256) return hipErrorInvalidValue;
    mtp_prep_kernel<<<dim3(a.M, a.NH + 2 * a.NKV), 256, 0, st>>>(a);
    return hipGetLastError();
}
