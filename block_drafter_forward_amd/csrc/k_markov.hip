// k_markov.hip — the DSpark Markov correction and confidence head of the KV-injection drafter (the DFlash
// page, forwardRows' greedy loop): one launch per decode step, sequential over the block's rows because each step
// conditions on the token the previous step chose, plus one closing launch. Step k keeps its argmax in its own
// 64-bit key slot; step k + 1 reads its token from there, and its first work-group writes step k's token and
// confidence, so no step needs a launch of its own to finish.
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

// A float's bits reordered so that unsigned comparison follows float order (negatives flipped, positives with the
// sign bit set): the high half of the 64-bit argmax key, the low half the complement of the column.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ── DSpark Markov correction (KV-injection page, forwardRows' greedy loop) ────────────────────────
// One decode step k: scores[v] = z_k[v] + sum_j e1[j] w2[j][v] with e1 = w1[prev] (bf16 [V][r] rows, w2 bf16
// [r][V]), then the argmax over v into a 64-bit key (same order as the lm_head kernel). Each thread owns 4
// consecutive columns (one 8-byte load per w2 row), 16 rows' loads in flight; e1 goes through LDS as f32.
// V % 4 == 0; columns past V (the last work-group) are clamped and left out of the argmax.
__device__ __forceinline__ int key_token(unsigned long long key) {
    return (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
}

// the token step k conditions on: the anchor, then the token step k - 1 chose
__device__ __forceinline__ int markov_prev(const MarkovArgs& a, int k) {
    const int p = k == 0 ? a.anchor[0] : key_token(a.key[k - 1]);
    return min(max(p, 0), a.V - 1);
}

// step j's confidence sigmoid([block_j; e1] conf.w + conf.b), e1 the w1 row of the token step j conditioned on;
// the whole work-group takes part and every thread gets it (the same value in every work-group: same order of sums)
__device__ float markov_conf(const MarkovArgs& a, int j, float* red) {
    const int tid = threadIdx.x;
    const int prev = markov_prev(a, j);
    float s = 0.f;
    for (int i = tid; i < a.D; i += 256) s += a.block[(size_t)j * a.D + i] * bf16_to_f32(a.cw[i]);
    for (int i = tid; i < a.r; i += 256) s += bf16_to_f32(a.w1[(size_t)prev * a.r + i]) * bf16_to_f32(a.cw[a.D + i]);
    s = block_sum256(s, red);
    return 1.f / (1.f + expf(-(s + bf16_to_f32(a.cb[0]))));
}

// step j's token (from its key) and confidence
__device__ void markov_close(const MarkovArgs& a, int j, float* red) {
    const float c = markov_conf(a, j, red);
    if (threadIdx.x == 0) {
        a.tokens[j] = key_token(a.key[j]);
        a.conf[j] = c;
    }
}

__global__ __launch_bounds__(256) void markov_step_kernel(MarkovArgs a, int k) {
    __shared__ float e1[MARKOV_MAX_RANK];
    __shared__ float wb[4];
    __shared__ int wi[4];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (a.prune && k > 0) {
        // DFlash pruning: position k is dropped, and the block ends, when its confidence (which needs only the token
        // step k - 1 chose) is below thr[k]; then neither this step nor a later one streams the correction table
        if (*a.cut) return;   // an earlier step ended the block
        if (markov_conf(a, k, red) < a.thr[k]) {
            if (blockIdx.x == 0) {
                markov_close(a, k - 1, red);   // position k - 1 is kept
                if (tid == 0) *a.cut = k;
            }
            return;
        }
    }
    const int prev = markov_prev(a, k);
    for (int j = tid; j < a.r; j += 256) e1[j] = bf16_to_f32(a.w1[(size_t)prev * a.r + j]);
    __syncthreads();
    const int c0 = (blockIdx.x * 256 + tid) * 4;
    const bool own = c0 < a.V;
    const int cc = own ? c0 : a.V - 4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* w = a.w2 + cc;
    int j = 0;
    for (; j + 16 <= a.r; j += 16) {
        uint2 q[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) q[u] = *(const uint2*)(w + (size_t)(j + u) * a.V);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float e = e1[j + u];
            acc[0] += e * bf16_lo(q[u].x); acc[1] += e * bf16_hi(q[u].x);
            acc[2] += e * bf16_lo(q[u].y); acc[3] += e * bf16_hi(q[u].y);
        }
    }
    for (; j < a.r; ++j) {
        const uint2 q = *(const uint2*)(w + (size_t)j * a.V);
        const float e = e1[j];
        acc[0] += e * bf16_lo(q.x); acc[1] += e * bf16_hi(q.x);
        acc[2] += e * bf16_lo(q.y); acc[3] += e * bf16_hi(q.y);
    }
    const float4 zb = *(const float4*)(a.z + (size_t)k * a.V + cc);
    const float sc[4] = {zb.x + acc[0], zb.y + acc[1], zb.z + acc[2], zb.w + acc[3]};
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    if (own) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (a.scores) a.scores[(size_t)k * a.V + cc + c] = sc[c];
            if (sc[c] > best) { best = sc[c]; bidx = cc + c; }
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bidx, o, 64);
        if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
    }
    if (lane == 0) { wb[wave] = best; wi[wave] = bidx; }
    __syncthreads();
    if (tid == 0) {
        float b = wb[0];
        int bi = wi[0];
        for (int w2i = 1; w2i < 4; ++w2i)
            if (wb[w2i] > b || (wb[w2i] == b && wi[w2i] < bi)) { b = wb[w2i]; bi = wi[w2i]; }
        if (bi != 0x7fffffff) {
            const unsigned long long key = ((unsigned long long)order_key(b) << 32) | (0xffffffffu - (uint32_t)bi);
            atomicMax(&a.key[k], key);
        }
    }
    if (k > 0 && blockIdx.x == 0) markov_close(a, k - 1, red);   // the previous step's token and confidence
}

// The last step's token and confidence (unless pruning ended the block earlier: then the dropped positions get
// token -1 and confidence 0), the kept length, then every step's key and the cut cleared for the next call.
__global__ __launch_bounds__(256) void markov_finalize_kernel(MarkovArgs a, int last) {
    __shared__ float red[4];
    const int cut = a.prune ? *a.cut : 0;   // uniform
    if (cut == 0) markov_close(a, last, red);
    __syncthreads();
    const int t = threadIdx.x;
    if (cut > 0 && t >= cut && t <= last) {
        a.tokens[t] = -1;
        a.conf[t] = 0.f;
    }
    if (t == 0 && a.length) *a.length = cut > 0 ? cut : last + 1;
    if (t <= last) a.key[t] = 0ull;
    if (t == 0 && a.prune) *a.cut = 0;
}

}  // namespace

hipError_t launch_markov(const MarkovArgs& a, int rows, hipStream_t st) {
    if (a.r < 1 || a.r > MARKOV_MAX_RANK || a.V < 4 || a.V % 4 || rows < 1 || rows > 16 || (a.prune && !a.cut))
        return hipErrorInvalidValue;
    for (int k = 0; k < rows; ++k) {
        markov_step_kernel<<<(a.V / 4 + 255) / 256, 256, 0, st>>>(a, k);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    markov_finalize_kernel<<<1, 256, 0, st>>>(a, rows - 1);
    return hipGetLastError();
}
