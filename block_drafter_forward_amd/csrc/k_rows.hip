// k_rows.hip — K3 row kernels and K7 small kernels.
//
// rows_kernel: one work-group per activation row. It finishes the previous phase (base + gate * (sum of split-K
// partial slabs + bias): the gated residual of the flow-map page's gateAdd, or a plain residual), optionally keeps
// the updated residual stream, then normalises the row -- adaLN LayerNorm-modulation (lnMod) or RMSNorm
// (rmsRows / WG_NORM) -- and stores it as the hi/lo bf16 fragments the next skinny GEMM reads. Values stay in
// registers between the passes; reductions are wave shuffles plus one LDS exchange, in a fixed order.
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

__device__ __forceinline__ void ld8(const float* p, float* v) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8_bf16(const uint16_t* p, float* v) {
    const uint4 a = *(const uint4*)p;
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}
__device__ __forceinline__ void st8(float* p, const float* v) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Every global load of the row (base, S partial slabs, bias, per-row bias, gate, and the norm's parameters) is
// unconditional -- absent inputs read the workspace's zero row and are masked arithmetically -- and issued before
// the first arithmetic. (A load inside a data-dependent branch makes the compiler wait for all outstanding loads
// at the branch, which turned this kernel into a chain of serial memory round trips.)
template <int NS, int S>
__global__ __launch_bounds__(256) void rows_kernel(RowArgs a) {
    const int t = blockIdx.x;
    const int D = a.D;
    const int nslot = D >> 3;
    __shared__ float red[4];
    const float* zf = a.zeros;
    const uint16_t* zb = (const uint16_t*)a.zeros;
    // base: bf16 rows for t >= base_from, else f32 (init broadcast / in_rows / x / zero)
    const bool use_b16 = a.base_bf16 != nullptr && t >= a.base_from;
    const float* basef;
    size_t base_ld;
    if (a.init) { basef = a.init; base_ld = 0; }
    else if (a.in_rows) { basef = a.in_rows; base_ld = a.in_ld; }
    else if (a.x && !a.base_zero) { basef = a.x + (size_t)a.row0 * D; base_ld = D; }
    else { basef = zf; base_ld = 0; }
    const uint16_t* baseb = a.base_bf16 ? a.base_bf16 + (size_t)(use_b16 ? t - a.base_from : 0) * D : zb;
    const bool has_part = !(a.part_rows > 0 && t >= a.part_rows);
    const uint16_t* biasp = a.bias ? a.bias : zb;
    const uint16_t* rbias = a.row_bias_bf16 ? a.row_bias_bf16 + (size_t)t * D : zb;
    const float* gatep = a.gate ? a.gate : zf;
    const float* p0f = a.norm == ROW_LN_MOD ? a.scale : (a.w_f32 ? a.w_f32 : zf);
    const float* p1f = a.norm == ROW_LN_MOD ? a.shift : zf;
    const uint16_t* wb = a.w_bf16 ? a.w_bf16 : zb;
    const bool w_is_b16 = a.norm == ROW_RMS && a.w_bf16 != nullptr;
    const float rsc = a.row_scale ? a.row_scale[t] : 1.f;

    float v[NS][8], u[NS][8], gv[NS][8], p0[NS][8], p1[NS][8];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int slot = threadIdx.x + j * 256;
        const int i0 = (slot < nslot ? slot : 0) * 8;
        float bf[8], bb[8], pp[S > 0 ? S : 1][8], bi[8], rb[8], w16[8];
        ld8(basef + (size_t)t * base_ld + i0, bf);
        ld8_bf16(baseb + i0, bb);
#pragma unroll
        for (int s = 0; s < S; ++s) ld8(a.part + (size_t)s * a.part_stride + (size_t)t * D + i0, pp[s]);
        ld8_bf16(biasp + i0, bi);
        ld8_bf16(rbias + i0, rb);
        ld8(gatep + i0, gv[j]);
        ld8(p0f + i0, p0[j]);
        ld8(p1f + i0, p1[j]);
        ld8_bf16(wb + i0, w16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float uu = bi[e] + rb[e];
            if (has_part) {
#pragma unroll
                for (int s = 0; s < S; ++s) uu += pp[s][e];
            }
            u[j][e] = uu * rsc;
            v[j][e] = use_b16 ? bb[e] : bf[e];
            if (!a.gate) gv[j][e] = 1.f;
            if (w_is_b16) p0[j][e] = w16[e];
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int slot = threadIdx.x + j * 256;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] += gv[j][e] * u[j][e];
        if (slot < nslot) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += v[j][e];
            if (a.x) st8(a.x + (size_t)(t + a.row0) * D + slot * 8, v[j]);
            if (a.debug_x) st8(a.debug_x + (size_t)(t + a.row0) * D + slot * 8, v[j]);
        }
    }
    if (a.norm == ROW_NONE && !a.frag_out && !a.f32_out) return;

    float r = 1.f, mean = 0.f;
    if (a.norm == ROW_LN_MOD) {
        mean = block_sum256(sum, red) / (float)D;
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j)
            if ((int)threadIdx.x + j * 256 < nslot)
#pragma unroll
                for (int e = 0; e < 8; ++e) { const float d = v[j][e] - mean; q += d * d; }
        const float var = block_sum256(q, red) / (float)D;
        r = 1.f / sqrtf(var + a.eps);
    } else if (a.norm == ROW_RMS) {
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j)
            if ((int)threadIdx.x + j * 256 < nslot)
#pragma unroll
                for (int e = 0; e < 8; ++e) q += v[j][e] * v[j][e];
        const float ms = block_sum256(q, red) / (float)D;
        r = 1.f / sqrtf(ms + a.eps);
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int slot = threadIdx.x + j * 256;
        if (slot < nslot) {
            const int i0 = slot * 8;
            float h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (a.norm == ROW_LN_MOD) h[e] = (v[j][e] - mean) * r * (1.f + p0[j][e]) + p1[j][e];
                else if (a.norm == ROW_RMS) h[e] = v[j][e] * r * p0[j][e];
                else h[e] = v[j][e];
            }
            if (a.frag_out) frag_store8_rows(a.frag_out, a.frag_kw ? a.frag_kw : D, t + a.row0, a.frag_koff + i0, h);
            if (a.f32_out) st8(a.f32_out + (size_t)(t + (a.f32_local ? 0 : a.row0)) * a.out_ld + i0, h);
        }
    }
}

// The RMSNorm fold's producer (the MTP head): one wave per (row, 512-column slice, segment). Segment s's row is
// in[s] (or zero) plus, with one segment, the sum of the split partials; it is written to x if set, w[s] * row goes
// out as fragments at k offset s D, and the slice's sum of squares to ssq[s][row0 + t][slice]. The consumer takes
// rstd = 1 / sqrt(sum ssq / D + eps) of each row and segment and multiplies its product by it.
__global__ __launch_bounds__(64) void rms_seg_kernel(RmsSegArgs a) {
    const int t = blockIdx.x, sl = blockIdx.y, sg = blockIdx.z;
    const int D = a.D, row = a.row0 + t;
    const int i0 = (sl * 64 + (int)threadIdx.x) * 8;
    float q = 0.f;
    if (i0 < D) {
        float v[8], w[8];
        if (a.in[sg]) ld8(a.in[sg] + (size_t)t * a.in_ld + i0, v);
        else if (a.x_in) ld8(a.x + (size_t)row * D + i0, v);
        else
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        for (int sp = 0; sp < a.S; ++sp) {
            float pp[8];
            ld8(a.part + (size_t)sp * a.part_stride + (size_t)row * D + i0, pp);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += pp[e];
        }
        if (a.x) st8(a.x + (size_t)row * D + i0, v);
        ld8(a.w[sg] + i0, w);
        float h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            q += v[e] * v[e];
            h[e] = v[e] * w[e];
        }
        frag_store8_rows(a.frag, a.frag_kw, row, sg * D + i0, h);
    }
    q = wave_sum(q);
    if (threadIdx.x == 0) a.ssq[((size_t)sg * 16 + row) * gridDim.y + sl] = q;
}

// The rows whose products with a matrix W give the LayerNorm fold's c1 = sum_k (1 + s_k) W[m][k] and
// c2 = sum_k shift_k W[m][k]: for modulation j of the table (scale, shift, gate at mod + 3 j D), row 0 = 1 + scale
// and row 1 = shift as fragments at frag + j D 64 (a 16-row block; rows 2..15 zero).
__global__ void ln_fold_rows_kernel(const float* mod, int D, uint8_t* frag) {
    const int j = blockIdx.y;
    const int slot = blockIdx.x * 256 + threadIdx.x;
    if (slot * 8 >= D) return;
    const float* m = mod + (size_t)j * 3 * D + slot * 8;
    float v0[8], v1[8], z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        v0[e] = 1.f + m[e];
        v1[e] = m[D + e];
        z[e] = 0.f;
    }
    uint8_t* f = frag + (size_t)j * D * 64;
    frag_store8(f, 0, slot * 8, v0);
    frag_store8(f, 1, slot * 8, v1);
    for (int t = 2; t < 16; ++t) frag_store8(f, t, slot * 8, z);
}

__global__ void f32_to_frag_kernel(const float* x, int ld, int K, uint8_t* frag) {
    const int t = blockIdx.y;
    const int slot = blockIdx.x * 256 + threadIdx.x;
    if (slot * 8 >= K) return;
    float v[8];
    const float* p = x + (size_t)t * ld + slot * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e];
    frag_store8_rows(frag, K, t, slot * 8, v);
}

// Token ids outside [0, V) are clamped into the table (a device-side id cannot be validated by the host).
__device__ __forceinline__ size_t clamp_row(int32_t id, int V) { return (size_t)(id < 0 ? 0 : (id >= V ? V - 1 : id)); }

__global__ void gather_frag_kernel(const uint16_t* E, int V, int K, const int32_t* idx, uint8_t* frag,
                                   int frow) {
    const int slot = blockIdx.x * 256 + threadIdx.x;
    if (slot * 8 >= K) return;
    const size_t row = clamp_row(idx[0], V);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf16_to_f32(E[row * K + slot * 8 + e]);
    frag_store8(frag, frow, slot * 8, v);
}

__global__ void gather_f32_kernel(const uint16_t* E, int V, int K, const int32_t* idx, const uint16_t* add,
                                  float* out) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= K) return;
    const size_t row = clamp_row(idx[0], V);
    float v = bf16_to_f32(E[row * K + i]);
    if (add) v += bf16_to_f32(add[i]);
    out[i] = v;
}

// Row E[*idx] of a Q8_0 table ([V][K] int8 codes, [V][K/32] f16 scales) -> f32: d * q per element (exact in f32).
__global__ void gather_q8_f32_kernel(const int8_t* q, const uint16_t* dsc, int V, int K, const int32_t* idx,
                                     float* out) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= K) return;
    const size_t row = clamp_row(idx[0], V);
    out[i] = f16_to_f32(dsc[row * (K >> 5) + (i >> 5)]) * (float)q[row * K + i];
}

// Time conditioning of a jump s -> t (the flow-map page's timeConditioning), create-time work.
// Stage 1, one work-group: the sinusoidal embeddings of s and t (frequencies exp in f64 rounded to f32, angles as
// f32 products, cos / sin of those angles: the page's Math.fround steps), each through linear_1, SiLU, linear_2 of
// its MLP ([0] time_embed for s, [1] jump_embed for t); cond = SiLU(sum of the two).
__global__ __launch_bounds__(256) void tc_embed_kernel(TimeCondArgs a) {
    __shared__ float e[2][TC_MAX_DIM], h[2][TC_MAX_DIM], y[2][TC_MAX_DIM];
    const int tid = threadIdx.x, half = a.td / 2;
    for (int i = tid; i < half; i += 256)
        for (int w = 0; w < 2; ++w) {
            const float f = (float)exp(-log(10000.0) * (double)i / (double)half);
            const float ang = (a.times[w] * a.time_scale) * f;
            e[w][i] = (float)cos((double)ang);
            e[w][half + i] = (float)sin((double)ang);
        }
    __syncthreads();
    for (int m = tid; m < a.cd; m += 256)
        for (int w = 0; w < 2; ++w) {
            float acc = bf16_to_f32(a.l1b[w][m]);
            for (int k = 0; k < a.td; ++k) acc += bf16_to_f32(a.l1w[w][(size_t)m * a.td + k]) * e[w][k];
            h[w][m] = silu(acc);
        }
    __syncthreads();
    for (int m = tid; m < a.cd; m += 256)
        for (int w = 0; w < 2; ++w) {
            float acc = bf16_to_f32(a.l2b[w][m]);
            for (int k = 0; k < a.cd; ++k) acc += bf16_to_f32(a.l2w[w][(size_t)m * a.cd + k]) * h[w][k];
            y[w][m] = acc;
        }
    __syncthreads();
    for (int m = tid; m < a.cd; m += 256) a.cond[m] = silu(y[0][m] + y[1][m]);
}

// Stage 2: table row n (norm n) entry m = adaLN bias[m] + sum_k W_n[m][k] cond[k], one thread per entry.
__global__ __launch_bounds__(256) void tc_adaln_kernel(TimeCondArgs a) {
    __shared__ float c[TC_MAX_DIM];
    const int n = blockIdx.y, m = blockIdx.x * 256 + threadIdx.x;
    for (int k = threadIdx.x; k < a.cd; k += 256) c[k] = a.cond[k];
    __syncthreads();
    if (m >= a.rows) return;
    const uint16_t* wr = a.aw[n] + (size_t)m * a.cd;
    float acc = bf16_to_f32(a.ab[n][m]);
    for (int k = 0; k < a.cd; ++k) acc += bf16_to_f32(wr[k]) * c[k];
    a.table[(size_t)n * a.rows + m] = acc;
}

// Stage 2 with coalesced weight reads, for cond_dim a power of two in [16, 1024]: a row's dot product is split over
// LPR = cond_dim / 16 adjacent threads, each reading 16 consecutive bf16 weights (two 16-byte loads) against the
// matching 16 condition values, then summed by LPR-lane shuffles; a work-group covers 256 / LPR whole rows, so it
// reads contiguous rows (the table's 19 x 6144 x 256 weights stream at ~5 TB/s instead of one 512-byte row per
// thread read 2 bytes at a time).
template <int LPR>
__device__ __forceinline__ float tc_row_dot(const uint16_t* __restrict__ W, int K, int row, int seg, const float* x,
                                            bool live) {
    float acc = 0.f;
    if (live) {
        const uint4* p = (const uint4*)(W + (size_t)row * K + seg * 16);
        const uint4 w0 = p[0], w1 = p[1];
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const float* xs = x + seg * 16;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += bf16_lo(w[i]) * xs[2 * i] + bf16_hi(w[i]) * xs[2 * i + 1];
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
    return acc;
}

// Stage 1 over many work-groups, coalesced like stage 2 (time_dim and cond_dim powers of two in [16, 1024]):
// work-group (row block, w) embeds time w and computes its 256 / LT rows of h_w = SiLU(linear_1 e_w) into the
// scratch after the condition vector; then work-group (row block) computes its rows of both linear_2 outputs and
// cond = SiLU(y_0 + y_1).
template <int LT>
__global__ __launch_bounds__(256) void tc_hidden_kernel(TimeCondArgs a) {
    __shared__ __attribute__((aligned(16))) float e[TC_MAX_DIM];
    constexpr int RPI = 256 / LT;
    const int tid = threadIdx.x, w = blockIdx.y, half = a.td / 2, seg = tid % LT;
    for (int i = tid; i < half; i += 256) {
        const float f = (float)exp(-log(10000.0) * (double)i / (double)half);
        const float ang = (a.times[w] * a.time_scale) * f;
        e[i] = (float)cos((double)ang);
        e[half + i] = (float)sin((double)ang);
    }
    __syncthreads();
    const int m = blockIdx.x * RPI + tid / LT;
    const bool live = m < a.cd;
    const float acc = tc_row_dot<LT>(a.l1w[w], a.td, m, seg, e, live);
    if (live && seg == 0) a.cond[(size_t)(1 + w) * TC_MAX_DIM + m] = silu(acc + bf16_to_f32(a.l1b[w][m]));
}

template <int LC>
__global__ __launch_bounds__(256) void tc_cond_kernel(TimeCondArgs a) {
    __shared__ __attribute__((aligned(16))) float h[2][TC_MAX_DIM];
    constexpr int RPI = 256 / LC;
    const int tid = threadIdx.x, seg = tid % LC;
    for (int k = tid; k < a.cd; k += 256) {
        h[0][k] = a.cond[TC_MAX_DIM + k];
        h[1][k] = a.cond[2 * TC_MAX_DIM + k];
    }
    __syncthreads();
    const int m = blockIdx.x * RPI + tid / LC;
    const bool live = m < a.cd;
    const float y0 = tc_row_dot<LC>(a.l2w[0], a.cd, m, seg, h[0], live);
    const float y1 = tc_row_dot<LC>(a.l2w[1], a.cd, m, seg, h[1], live);
    if (live && seg == 0)
        a.cond[m] = silu((y0 + bf16_to_f32(a.l2b[0][m])) + (y1 + bf16_to_f32(a.l2b[1][m])));
}

template <int LC>
__global__ __launch_bounds__(256) void tc_adaln_seg_kernel(TimeCondArgs a) {
    __shared__ __attribute__((aligned(16))) float c[TC_MAX_DIM];
    constexpr int RPI = 256 / LC;
    const int n = blockIdx.y, tid = threadIdx.x, seg = tid % LC;
    for (int k = tid; k < a.cd; k += 256) c[k] = a.cond[k];
    __syncthreads();
    const int m = blockIdx.x * RPI + tid / LC;
    const bool live = m < a.rows;
    const float acc = tc_row_dot<LC>(a.aw[n], a.cd, m, seg, c, live);
    if (live && seg == 0) a.table[(size_t)n * a.rows + m] = acc + bf16_to_f32(a.ab[n][m]);
}

__global__ void colmean_stage1(const uint16_t* E, int V, int H, int R, float* scratch) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= H) return;
    const int per = (V + R - 1) / R;
    const int r0 = blockIdx.y * per, r1 = min(V, r0 + per);
    float s = 0.f;
    for (int r = r0; r < r1; ++r) s += bf16_to_f32(E[(size_t)r * H + col]);
    scratch[(size_t)blockIdx.y * H + col] = s;
}

__global__ void colmean_stage2(const float* scratch, int V, int H, int R, float* out) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= H) return;
    double s = 0.0;
    for (int r = 0; r < R; ++r) s += (double)scratch[(size_t)r * H + col];
    out[col] = (float)(s / (double)V);
}

__global__ void rope_table_kernel(float* tab, int P, int rdim, double theta) {
    const int half = rdim >> 1;
    const size_t n = (size_t)P * half;
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= n) return;
    const int p = (int)(id / half), i = (int)(id % half);
    const double a = (double)p * pow(theta, -2.0 * (double)i / (double)rdim);
    tab[(size_t)p * rdim + i] = (float)cos(a);
    tab[(size_t)p * rdim + half + i] = (float)sin(a);
}

// One wave that returns once `ticks` of the 100 MHz wall clock have passed since it started: queued ahead of a
// sequence of launches, it keeps the GPU busy while the host enqueues them, so they later run back to back.
__global__ void hold_kernel(uint64_t ticks) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int NS, int NSLAB>
__global__ __launch_bounds__(256) void rms_f16_kernel(const float* x, int D, const uint16_t* w, float eps,
                                                      uint16_t* out, long long slab_stride, const float* rscale) {
    const int t = blockIdx.x;
    const int nslot = D >> 3;
    __shared__ float red[4];
    float v[NS][8];
    float q = 0.f;
    const float rs = rscale ? rscale[t] : 1.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int slot = threadIdx.x + j * 256;
        if (slot < nslot) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
#pragma unroll
            for (int sl = 0; sl < NSLAB; ++sl) {   // partial slabs summed in a fixed order
                const float4* p = (const float4*)(x + (size_t)sl * slab_stride + (size_t)t * D + slot * 8);
                const float4 a0 = p[0], a1 = p[1];
                v[j][0] += a0.x; v[j][1] += a0.y; v[j][2] += a0.z; v[j][3] += a0.w;
                v[j][4] += a1.x; v[j][5] += a1.y; v[j][6] += a1.z; v[j][7] += a1.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[j][e] *= rs;
                q += v[j][e] * v[j][e];
            }
        }
    }
    const float r = 1.f / sqrtf(block_sum256(q, red) / (float)D + eps);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int slot = threadIdx.x + j * 256;
        if (slot < nslot) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = slot * 8 + 2 * e;
                o[e] = (uint32_t)f32_to_f16(v[j][2 * e] * r * bf16_to_f32(w[i])) |
                       ((uint32_t)f32_to_f16(v[j][2 * e + 1] * r * bf16_to_f32(w[i + 1])) << 16);
            }
            *(uint4*)(out + (size_t)t * D + slot * 8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

}  // namespace

template <int NS>
hipError_t launch_rows_ns(const RowArgs& a, hipStream_t st) {
    dim3 grid(a.T), block(256);
    switch (a.S) {
    case 0: rows_kernel<NS, 0><<<grid, block, 0, st>>>(a); break;
    case 1: rows_kernel<NS, 1><<<grid, block, 0, st>>>(a); break;
    case 2: rows_kernel<NS, 2><<<grid, block, 0, st>>>(a); break;
    case 3: rows_kernel<NS, 3><<<grid, block, 0, st>>>(a); break;
    case 4: rows_kernel<NS, 4><<<grid, block, 0, st>>>(a); break;
    case 5: rows_kernel<NS, 5><<<grid, block, 0, st>>>(a); break;
    case 6: rows_kernel<NS, 6><<<grid, block, 0, st>>>(a); break;
    case 7: rows_kernel<NS, 7><<<grid, block, 0, st>>>(a); break;
    case 8: rows_kernel<NS, 8><<<grid, block, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_rows(const RowArgs& a, hipStream_t st) {
    if (!a.zeros) return hipErrorInvalidValue;
    const int ns = (a.D / 8 + 255) / 256;
    switch (ns) {
    case 1: return launch_rows_ns<1>(a, st);
    case 2: return launch_rows_ns<2>(a, st);
    case 3: return launch_rows_ns<3>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ln_fold_rows(const float* mod, int D, int nmod, uint8_t* frag, hipStream_t st) {
    if (D % 32 || nmod < 1) return hipErrorInvalidValue;
    ln_fold_rows_kernel<<<dim3((D / 8 + 255) / 256, nmod), 256, 0, st>>>(mod, D, frag);
    return hipGetLastError();
}

hipError_t launch_f32_to_frag(const float* x, int ld, int T, int K, uint8_t* frag, hipStream_t st) {
    if (T < 1 || T > 32 || K % 32) return hipErrorInvalidValue;
    dim3 grid((K / 8 + 255) / 256, T);
    f32_to_frag_kernel<<<grid, 256, 0, st>>>(x, ld, K, frag);
    return hipGetLastError();
}

hipError_t launch_gather_frag(const uint16_t* E, int V, int K, const int32_t* idx, uint8_t* frag,
                              hipStream_t st, int row) {
    if (row < 0 || row >= 16) return hipErrorInvalidValue;
    gather_frag_kernel<<<(K / 8 + 255) / 256, 256, 0, st>>>(E, V, K, idx, frag, row);
    return hipGetLastError();
}

hipError_t launch_time_condition(const TimeCondArgs& a, hipStream_t st) {
    if (a.td < 2 || a.td % 2 || a.td > TC_MAX_DIM || a.cd < 1 || a.cd > TC_MAX_DIM || a.rows < 1 || a.nnorm < 1 ||
        a.nnorm > TC_MAX_NORMS)
        return hipErrorInvalidValue;
    // threads per row of the coalesced kernels (width / 16), 0 if the width does not fit them
    auto lanes = [](int k) { return (k >= 16 && k <= 1024 && (k & (k - 1)) == 0) ? k / 16 : 0; };
    const int lt = lanes(a.td), lc = lanes(a.cd);
    bool aligned = true;   // the coalesced kernels read 16-byte pieces of every weight row
    auto al = [&](const void* q) { aligned = aligned && ((uintptr_t)q & 15) == 0; };
    for (int w = 0; w < 2; ++w) { al(a.l1w[w]); al(a.l2w[w]); }
    for (int n = 0; n < a.nnorm; ++n) al(a.aw[n]);
    if (lt == 0 || lc == 0 || !aligned) {
        tc_embed_kernel<<<1, 256, 0, st>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        tc_adaln_kernel<<<dim3((a.rows + 255) / 256, a.nnorm), 256, 0, st>>>(a);
        return hipGetLastError();
    }
    const dim3 hgrid((a.cd + 256 / lt - 1) / (256 / lt), 2);
    switch (lt) {
    case 1: tc_hidden_kernel<1><<<hgrid, 256, 0, st>>>(a); break;
    case 2: tc_hidden_kernel<2><<<hgrid, 256, 0, st>>>(a); break;
    case 4: tc_hidden_kernel<4><<<hgrid, 256, 0, st>>>(a); break;
    case 8: tc_hidden_kernel<8><<<hgrid, 256, 0, st>>>(a); break;
    case 16: tc_hidden_kernel<16><<<hgrid, 256, 0, st>>>(a); break;
    case 32: tc_hidden_kernel<32><<<hgrid, 256, 0, st>>>(a); break;
    default: tc_hidden_kernel<64><<<hgrid, 256, 0, st>>>(a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int cgrid = (a.cd + 256 / lc - 1) / (256 / lc);
    switch (lc) {
    case 1: tc_cond_kernel<1><<<cgrid, 256, 0, st>>>(a); break;
    case 2: tc_cond_kernel<2><<<cgrid, 256, 0, st>>>(a); break;
    case 4: tc_cond_kernel<4><<<cgrid, 256, 0, st>>>(a); break;
    case 8: tc_cond_kernel<8><<<cgrid, 256, 0, st>>>(a); break;
    case 16: tc_cond_kernel<16><<<cgrid, 256, 0, st>>>(a); break;
    case 32: tc_cond_kernel<32><<<cgrid, 256, 0, st>>>(a); break;
    default: tc_cond_kernel<64><<<cgrid, 256, 0, st>>>(a); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((a.rows + 256 / lc - 1) / (256 / lc), a.nnorm);
    switch (lc) {
    case 1: tc_adaln_seg_kernel<1><<<grid, 256, 0, st>>>(a); break;
    case 2: tc_adaln_seg_kernel<2><<<grid, 256, 0, st>>>(a); break;
    case 4: tc_adaln_seg_kernel<4><<<grid, 256, 0, st>>>(a); break;
    case 8: tc_adaln_seg_kernel<8><<<grid, 256, 0, st>>>(a); break;
    case 16: tc_adaln_seg_kernel<16><<<grid, 256, 0, st>>>(a); break;
    case 32: tc_adaln_seg_kernel<32><<<grid, 256, 0, st>>>(a); break;
    default: tc_adaln_seg_kernel<64><<<grid, 256, 0, st>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t launch_gather_q8_f32(const int8_t* q, const uint16_t* dsc, int V, int K, const int32_t* idx, float* out,
                                hipStream_t st) {
    if (K % 32 || V < 1) return hipErrorInvalidValue;
    gather_q8_f32_kernel<<<(K + 255) / 256, 256, 0, st>>>(q, dsc, V, K, idx, out);
    return hipGetLastError();
}

hipError_t launch_gather_f32(const uint16_t* E, int V, int K, const int32_t* idx, const uint16_t* add, float* out,
                             hipStream_t st) {
    gather_f32_kernel<<<(K + 255) / 256, 256, 0, st>>>(E, V, K, idx, add, out);
    return hipGetLastError();
}

hipError_t launch_colmean(const uint16_t* E, int V, int H, float* scratch, int R, float* out, hipStream_t st) {
    colmean_stage1<<<dim3((H + 255) / 256, R), 256, 0, st>>>(E, V, H, R, scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    colmean_stage2<<<(H + 255) / 256, 256, 0, st>>>(scratch, V, H, R, out);
    return hipGetLastError();
}

hipError_t launch_rope_table(float* tab, int P, int rdim, double theta, hipStream_t st) {
    const size_t n = (size_t)P * (rdim / 2);
    rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(tab, P, rdim, theta);
    return hipGetLastError();
}

hipError_t launch_hold(uint64_t ticks, hipStream_t st) {
    hold_kernel<<<1, 64, 0, st>>>(ticks);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
    if (n == 0) return hipSuccess;
    fill_u32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
    return hipGetLastError();
}

template <int NSLAB>
hipError_t launch_rms_f16_s(const float* x, int n, int D, const uint16_t* w, float eps, uint16_t* out,
                            long long slab_stride, const float* rscale, hipStream_t st) {
    const int ns = (D / 8 + 255) / 256;
    switch (ns) {
    case 1: rms_f16_kernel<1, NSLAB><<<n, 256, 0, st>>>(x, D, w, eps, out, slab_stride, rscale); break;
    case 2: rms_f16_kernel<2, NSLAB><<<n, 256, 0, st>>>(x, D, w, eps, out, slab_stride, rscale); break;
    case 3: rms_f16_kernel<3, NSLAB><<<n, 256, 0, st>>>(x, D, w, eps, out, slab_stride, rscale); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_rms_f16(const float* x, int n, int D, const uint16_t* w, float eps, uint16_t* out, int nslab,
                          long long slab_stride, const float* rscale, hipStream_t st) {
    if (nslab > 1 && slab_stride < (long long)n * D) return hipErrorInvalidValue;
    switch (nslab) {
    case 1: return launch_rms_f16_s<1>(x, n, D, w, eps, out, 0, rscale, st);
    case 2: return launch_rms_f16_s<2>(x, n, D, w, eps, out, slab_stride, rscale, st);
    case 4: return launch_rms_f16_s<4>(x, n, D, w, eps, out, slab_stride, rscale, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rms_seg(const RmsSegArgs& a, hipStream_t st) {
    const int nsl = (a.D + 511) / 512;
    if (a.D % 32 || a.T < 1 || a.row0 < 0 || a.row0 + a.T > 16 || a.nseg < 1 || a.nseg > 2 || !a.w[0] ||
        (a.nseg == 2 && !a.w[1]) || !a.frag || !a.ssq || a.frag_kw < a.nseg * a.D || a.S < 0 || (a.S > 0 && !a.part) ||
        (a.x_in && !a.x) || ((a.S > 0 || a.x) && a.nseg != 1) || nsl != a.nsl)
        return hipErrorInvalidValue;
    rms_seg_kernel<<<dim3(a.T, nsl, a.nseg), 64, 0, st>>>(a);
    return hipGetLastError();
}
