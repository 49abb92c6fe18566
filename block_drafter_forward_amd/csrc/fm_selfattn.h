// fm_selfattn.h — the flow-map self-attention of one head over the slots of one block of rows (the flow-map page's
// draft: headNormRope, then attnF32 over the block's own rows): per-head q / k RMSNorm, interleaved RoPE at the slots'
// positions, softmax(q kᵀ / sqrt(hd)) v with no mask, o out as fragments for the o_proj product.
//
// A work-group routine built for latency (the whole op is 16 x 16 x hd): the q, k, v rows of the head are read
// with 128-bit device-coherent loads (they were stored device-coherent by the other work-groups of the same
// launch), every load issued up front; thread (row, segment) holds hd/8 consecutive values of one q or k row, so the
// head-RMSNorm is an 8-lane shuffle reduction and the RoPE pairs stay inside the thread; then one LDS exchange for
// the scores (thread = (query, key), 16-lane softmax by shuffles) and one for P·V, whose 8 consecutive outputs per
// thread go straight out as fragments. All arithmetic in f32. Every thread of the work-group calls it.
#pragma once
#include "fm_device.h"
#include "fm_kernels.h"

namespace sattn {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int SC1 = 16;   // buffer-instruction cache policy bit: device-coherent

__device__ __forceinline__ float4 cld4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// LDS: QK [32 (HD + 4)] floats, Vs [16 (HD + 4)] floats, Ps [16][17] floats (16-byte aligned)
template <int HD>
__device__ __forceinline__ void head(const SelfAttnArgs& a, int h, int blk, float* QK, float* Vs, float (*Ps)[17]) {
    constexpr int SEG = HD / 8, VPT = HD / 16, QP = HD + 4;
    const int tid = threadIdx.x;
    const int T = a.T, D = a.D;
    // this block's rows of q | k | v, through a buffer resource (coherent loads need the buffer form)
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.qkv + (size_t)blk * 16 * 3 * D), 0, 0x7fffffff, 0x00020000);
    const int pos_base = blk ? a.pos_base1 : a.pos_base;
    const int row = tid >> 3, seg = tid & 7;   // q rows 0..15, k rows 16..31
    const int w = row >> 4, t = row & 15, tc = min(t, T - 1);
    float x[SEG], cs[SEG / 2], sn[SEG / 2], nw[SEG], v[VPT];
    {
        const uint32_t xo = (uint32_t)(((size_t)tc * 3 * D + (size_t)w * D + (size_t)h * HD + seg * SEG) * 4);
#pragma unroll
        for (int j = 0; j < SEG / 4; ++j) {
            const float4 f = cld4f(rq, xo + 16 * j);
            x[4 * j] = f.x; x[4 * j + 1] = f.y; x[4 * j + 2] = f.z; x[4 * j + 3] = f.w;
        }
        const float* rt = a.rope_tab + (size_t)(pos_base + tc) * HD + seg * (SEG / 2);
#pragma unroll
        for (int j = 0; j < SEG / 8; ++j) {
            const float4 c = ((const float4*)rt)[j], sv = ((const float4*)(rt + HD / 2))[j];
            cs[4 * j] = c.x; cs[4 * j + 1] = c.y; cs[4 * j + 2] = c.z; cs[4 * j + 3] = c.w;
            sn[4 * j] = sv.x; sn[4 * j + 1] = sv.y; sn[4 * j + 2] = sv.z; sn[4 * j + 3] = sv.w;
        }
        const uint16_t* n = (w ? a.kn : a.qn) + seg * SEG;
#pragma unroll
        for (int j = 0; j < SEG; ++j) nw[j] = bf16_to_f32(n[j]);
        const int vt = min(tid >> 4, T - 1), vp = tid & 15;
        const uint32_t vo = (uint32_t)(((size_t)vt * 3 * D + 2 * (size_t)D + (size_t)h * HD + vp * VPT) * 4);
#pragma unroll
        for (int j = 0; j < VPT / 4; ++j) {
            const float4 f = cld4f(rq, vo + 16 * j);
            v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < SEG; ++j) ss += x[j] * x[j];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    const float r = 1.f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int j = 0; j < SEG / 2; ++j) {
        const float x0 = x[2 * j] * (nw[2 * j] * r), x1 = x[2 * j + 1] * (nw[2 * j + 1] * r);
        x[2 * j] = x0 * cs[j] - x1 * sn[j];
        x[2 * j + 1] = x1 * cs[j] + x0 * sn[j];
    }
#pragma unroll
    for (int j = 0; j < SEG / 4; ++j)
        *(float4*)(QK + row * QP + seg * SEG + 4 * j) = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j)
        *(float4*)(Vs + (tid >> 4) * QP + (tid & 15) * VPT + 4 * j) =
            make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    __syncthreads();
    {
        const int qt = tid >> 4, u = tid & 15;
        const float* q = QK + qt * QP;
        const float* k = QK + (16 + u) * QP;
        float s = 0.f;
#pragma unroll 8
        for (int d = 0; d < HD; d += 4) {
            const float4 qa = *(const float4*)(q + d), kb = *(const float4*)(k + d);
            s += qa.x * kb.x + qa.y * kb.y + qa.z * kb.z + qa.w * kb.w;
        }
        s = u < T ? s * a.scale : -INFINITY;
        float m = s;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float e = u < T ? expf(s - m) : 0.f;
        float z = e;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
        Ps[qt][u] = e / z;
    }
    __syncthreads();
    if (tid < 2 * HD) {
        const int ot = tid / (HD / 8), d0 = (tid % (HD / 8)) * 8;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        for (int u = 0; u < T; ++u) {
            const float p = Ps[ot][u];
            const float4 v0 = *(const float4*)(Vs + u * QP + d0), v1 = *(const float4*)(Vs + u * QP + d0 + 4);
            o[0] += p * v0.x; o[1] += p * v0.y; o[2] += p * v0.z; o[3] += p * v0.w;
            o[4] += p * v1.x; o[5] += p * v1.y; o[6] += p * v1.z; o[7] += p * v1.w;
        }
        if (ot < T) frag_store8(a.o_frag + (size_t)blk * D * 64, ot, h * HD + d0, o);
    }
    __syncthreads();   // the LDS is free again when the routine returns
}

}  // namespace sattn
