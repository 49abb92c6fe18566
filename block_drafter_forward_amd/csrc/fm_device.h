// fm_device.h — device-side helpers shared by the gfx950 kernels: storage-format conversions, the MFMA
// activation-fragment layout, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ── bf16 / f16 ─────────────────────────────────────────────────────────────────────────────────
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two values split into their hi / lo bf16 terms, packed by pairs: hi = RNE(x), lo = RNE(x - hi) (x - hi is exact
// in f32), both rounded to nearest even by gfx950's v_cvt_pk_bf16_f32, one instruction per pair.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    const f32x2_t v = {a, b};
    const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    const f32x2_t r = v - __builtin_convertvector(h, f32x2_t);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, h);
    return (float)v;
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 v = (_Float16)f;
    return __builtin_bit_cast(uint16_t, v);
}

// ── activation fragments ───────────────────────────────────────────────────────────────────────
// A skinny activation matrix X[T <= 16][K] (K a multiple of 32) is stored as the B operand of
// v_mfma_f32_16x16x32_bf16, split into two bf16 terms x = hi + lo (|x - hi - lo| <= 2^-17 |x|):
//   k-step s = 2048 bytes = hi[64 lanes][8 bf16] then lo[64 lanes][8 bf16]; lane l = t + 16 g holds row t = l % 16.
// Column k = 32 s + 8 g + e of step s sits in lane group g, element e (the MFMA's own k order); Q8_0 weights: a step
// is one Q8_0 block.
// Rows t >= T are never read back by any consumer (MFMA columns are independent), so they need no clearing.
#define FRAG_STEP_BYTES 2048

// Column offset (within a weight row) of lane group g's 8 elements in k-step s.
__device__ __forceinline__ int kcol(int s, int g) { return (s << 5) + (g << 3); }

__device__ __forceinline__ size_t frag_offset(int t, int k) {   // byte offset of (t, k), k % 8 == 0
    return (size_t)(k >> 5) * FRAG_STEP_BYTES + (size_t)(t + 16 * ((k & 31) >> 3)) * 16;
}

// Store 8 consecutive values x[t][k .. k+7] (k % 8 == 0) as their hi/lo bf16 fragments.
__device__ __forceinline__ void frag_store8(uint8_t* frag, int t, int k, const float* v) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_pair(v[2 * i], v[2 * i + 1], hi[i], lo[i]);
    uint8_t* p = frag + frag_offset(t, k);
    *(uint4*)p = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *(uint4*)(p + 1024) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// A fragment matrix of T <= 32 rows is two of the above, one per 16 rows: rows 16 b .. 16 b + 15 of X[T][K] at byte
// offset b * K * 64 (K / 32 steps of 2 KB each).
__device__ __forceinline__ void frag_store8_rows(uint8_t* frag, int K, int t, int k, const float* v) {
    frag_store8(frag + (size_t)(t >> 4) * K * 64, t & 15, k, v);
}

// ── reductions ─────────────────────────────────────────────────────────────────────────────────
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
// Sum over the 256 threads of a block; `red` is __shared__ float[4]. Every thread gets the result.
__device__ __forceinline__ float block_sum256(float v, float* red) {
    v = wave_sum(v);
    int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// ── math ───────────────────────────────────────────────────────────────────────────────────────
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_tanh(float x) {
    const float c = 0.7978845608028654f;   // sqrt(2/pi)
    return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float silu(float x) { return x * sigmoidf(x); }
