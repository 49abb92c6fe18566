// k_draft.hip — K8: the flow-map draft block (the flow-map page's draft: the anchor slot, every DiT layer, the head)
// as one persistent kernel.
//
// Launched as one work-group per CU (the whole grid resident at once). Each work-group has DR_WAVES consumer waves
// and one producer wave:
//   * the producer streams, in the order the consumers will use them, every 8 KB chunk of weights (16 rows x 256
//     columns of a projection) and of the context K / V (32 keys of one head) this work-group needs during the
//     whole draft into a ring of DR_RING LDS slots, with LDS-direct loads (global_load_lds_dwordx4: no registers);
//     it runs ahead of the consumers across phase boundaries, so the weight stream of a projection overlaps the
//     latency-bound phases (norms, attention) before it. A slot carries a sequence number: the producer publishes
//     it once its loads have landed, the consumer releases it after its last read; the producer refills a slot only
//     after its release, and keeps at most DEPTH < DR_RING chunks unpublished, so it never waits on a consumer that
//     waits on it;
//   * the consumers run the phases of the draft in order. Work items of a phase are dealt to the work-groups
//     round-robin; between phases all work-groups meet at a grid barrier (one arrival counter per XCD label, no
//     cache flushes). Activations pass between work-groups through a write-once arena with device-coherent (sc1)
//     buffer stores and loads, so no L2 write-back or invalidate is ever needed;
//   * every wait (ring slot, consumer barrier, grid barrier) is bounded by a wall-clock deadline: on expiry the
//     work-group sets the error word and leaves, and the others follow at their next wait.
// The phases (per layer l; layer 0 starts at its cross-attention, the rest of it is the same for every draft):
//   A1   anchor_proj of the anchor's table row (k-split partial slabs)
//   A3X  the anchor row's cross K and V of layer l (its context row c = RMSNorm(A1 + bias) rebuilt per work-group)
//        together with the cross-attention of the 16 slots over the context keys [0, pos) (runs of 32-key steps)
//   M    per (head, slot): log-sum-exp merge of the runs and of the anchor key (its k head-norm + RoPE at pos), the
//        anchor's K / V written into the cache row pos
//   OC / R2 / F1 / F2: cross o_proj, residual + MLP LN-mod, fc1 + exact GELU, fc2
//   R0 / QKV / SA / O / R1 / QC (layers >= 1): residual + self LN-mod, q | k | v, self-attention, o_proj, residual +
//        cross LN-mod, cross q_proj
//   RF / HEAD: residual + final LN-mod, head (+ bias) -> hidden_out
#include "fm_device.h"
#include "fm_kernels.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int T = 16;                       // draft rows (slots)
constexpr int HD = 128;                     // head width of this kernel
constexpr int NTH = (DR_WAVES + 1) * 64;    // consumer waves + the producer
constexpr int NCT = DR_WAVES * 64;          // consumer threads
constexpr int DEPTH = 6;                    // producer chunks in flight before the oldest is published
constexpr int SC1 = 16;                     // buffer-instruction cache policy bit: device-coherent
constexpr int RING_OFF = 0, FLAG_OFF = DR_RING * DR_CHUNK, SCR_OFF = FLAG_OFF + 256;
static_assert(SCR_OFF + DR_SCRATCH == DR_LDS, "LDS layout");
static_assert(DEPTH < DR_RING, "the ring must be deeper than the chunks in flight");
static_assert(NCT == 256, "the consumer code is written for 256 threads");

enum Kind { PH_A1, PH_A3X, PH_M, PH_OC, PH_R2, PH_F1, PH_F2, PH_R0, PH_QKV, PH_SA, PH_O, PH_R1, PH_QC, PH_RF, PH_HEAD };

// The per-layer table is read through the constant address space (uniform scalar loads); data pointers are cast to
// the global address space, so no access becomes a FLAT instruction (which would count against the producer's
// load counter).
typedef __attribute__((address_space(4))) const DraftLayer CLayer;
__device__ __forceinline__ CLayer& layer(const DraftArgs& a, int l) { return ((CLayer*)a.L)[l]; }
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gp(const T* p) {
    return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gpw(T* p) {
    return (__attribute__((address_space(1))) T*)p;
}

// ── shared state of a work-group ────────────────────────────────────────────────────────────────
struct Ctx {
    int pos, nsteps, cpw, xgroups;   // this call: the anchor's position and the cross-attention split
    const int32_t* anchor;
    float* hidden_out;
    float* debug;
    uint8_t* lds;
    uint32_t *ready, *freed, *bar, *abort;
    __amdgpu_buffer_rsrc_t ar;   // the arena
    int g, wave, lane, tid;
    long long deadline;
    uint32_t bar_target;   // consumer-barrier arrivals expected so far
    uint32_t nbar;         // grid barriers passed
    int seq;               // ring chunks of this work-group enumerated so far
};

// The phase sequence, the one source of truth for both the producer and the consumers: A1; layer 0 from its
// cross-attention (A3X M OC R2 F1 F2); every further layer (R0 QKV SA O R1 QC A3X M OC R2 F1 F2); RF HEAD. One call
// site for fn (a loop over the phase index), so each phase's code exists once. fn returns false to stop.
__device__ __forceinline__ int tail_kind(int q) {   // a layer's phases from its cross-attention on
    switch (q) {
    case 0: return PH_A3X;
    case 1: return PH_M;
    case 2: return PH_OC;
    case 3: return PH_R2;
    case 4: return PH_F1;
    default: return PH_F2;
    }
}
__device__ __forceinline__ int head_kind(int q) {   // a layer's phases up to its cross-attention's q (layers >= 1)
    switch (q) {
    case 0: return PH_R0;
    case 1: return PH_QKV;
    case 2: return PH_SA;
    case 3: return PH_O;
    case 4: return PH_R1;
    default: return PH_QC;
    }
}
__device__ __forceinline__ void phase_at(const DraftArgs& a, int p, int& k, int& l) {
    const int np = 1 + 6 + 12 * (a.layers - 1) + 2;
    if (p == 0) { k = PH_A1; l = 0; return; }
    if (p == np - 2) { k = PH_RF; l = 0; return; }
    if (p == np - 1) { k = PH_HEAD; l = 0; return; }
    int q = p - 1;
    if (q < 6) { k = tail_kind(q); l = 0; return; }
    q -= 6;
    l = 1 + q / 12;
    q %= 12;
    k = q < 6 ? head_kind(q) : tail_kind(q - 6);
}
template <class Fn>
__device__ __forceinline__ void schedule(const DraftArgs& a, Fn&& fn) {
    const int np = 1 + 6 + 12 * (a.layers - 1) + 2;
    for (int p = 0; p < np; ++p) {
        int k, l;
        phase_at(a, p, k, l);
        if (!fn(__builtin_amdgcn_readfirstlane(k), __builtin_amdgcn_readfirstlane(l))) return;
    }
}

__device__ __forceinline__ int n_items(const DraftArgs& a, const Ctx& x, int k) {
    const int tD = a.D / 16;
    switch (k) {
    case PH_A1: return tD * a.S_a1;
    case PH_A3X: return a.H * x.xgroups + 2 * tD;
    case PH_M: return a.H * T;
    case PH_OC: return tD * a.S_oc;
    case PH_O: return tD * a.S_o;
    case PH_QC: return tD * a.S_qc;
    case PH_F1: return a.F / 16;
    case PH_F2: return tD * a.S_f2;
    case PH_QKV: return 3 * tD * a.S_qkv;
    case PH_SA: return a.H;
    case PH_HEAD: return a.Ht / 16;
    default: return T;   // the row phases
    }
}

// A projection's work item: output rows m .. m + 15 (of the phase's whole output row), columns k0 .. k0 + 256 nck.
struct GemmItem {
    const uint16_t* W;   // the tile's first row at column k0
    int K;               // weight row stride (elements)
    int nck;             // 256-column chunks
    int m;               // first output index
    int split;
    int k0;
};

__device__ __forceinline__ bool gemm_item(const DraftArgs& a, const Ctx& x, int k, int l, int item, GemmItem& g) {
    CLayer& L = layer(a, l);
    const int tD = a.D / 16;
    const uint16_t* W = nullptr;
    int K = a.D, S = 1, tiles = tD, goff = 0;
    switch (k) {
    case PH_A1: W = a.wap; K = a.Ht; S = a.S_a1; break;
    case PH_A3X: {
        item -= a.H * x.xgroups;   // the cross-attention items come first
        if (item < 0) return false;
        const int grp = item / tD;   // 0: the anchor's K row, 1: its V row
        W = grp ? L.wcv : L.wck;
        goff = grp * a.D;
        item -= grp * tD;
        break;
    }
    case PH_OC: W = L.woc; S = a.S_oc; break;
    case PH_O: W = L.wo; S = a.S_o; break;
    case PH_QC: W = L.wqc; S = a.S_qc; break;
    case PH_F1: W = L.w1; tiles = a.F / 16; break;
    case PH_F2: W = L.w2; K = a.F; S = a.S_f2; break;
    case PH_QKV: {
        const int s = item / (3 * tD), t = item % (3 * tD), grp = t / tD;
        g.split = s;
        g.K = a.D;
        g.nck = a.D / a.S_qkv / 256;
        g.k0 = s * (a.D / a.S_qkv);
        g.m = grp * a.D + (t % tD) * 16;
        g.W = (grp == 0 ? L.wq : grp == 1 ? L.wk : L.wv) + (size_t)((t % tD) * 16) * a.D + g.k0;
        return true;
    }
    case PH_HEAD: W = a.whead; tiles = a.Ht / 16; break;
    default: return false;
    }
    const int s = item / tiles, t = item % tiles;
    g.split = s;
    g.K = K;
    g.nck = K / S / 256;
    g.k0 = s * (K / S);
    g.m = goff + t * 16;
    g.W = W + (size_t)(t * 16) * K + g.k0;
    return true;
}

// Cross-attention item (head h, run group rg): run 4 rg + w belongs to consumer wave w and holds the 32-key steps
// [(4 rg + w) cpw, min((4 rg + w + 1) cpw, nsteps)). Chunk order: for each step index sl within a run, for each
// wave, that step's K chunk then its V chunk.
__device__ __forceinline__ bool x_exists(const Ctx& x, int rg, int w, int sl) {
    return (4 * rg + w) * x.cpw + sl < x.nsteps;
}
__device__ __forceinline__ int x_count(const Ctx& x, int rg, int sl) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < DR_WAVES; ++w) n += x_exists(x, rg, w, sl) ? 1 : 0;
    return n;
}

// ── memory helpers ──────────────────────────────────────────────────────────────────────────────
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4 ald16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1);
}
__device__ __forceinline__ float ald4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1));
}
// Activation reads through L2: every arena buffer is written once per launch (sc1, written through) before any
// work-group reads it, and each work-group invalidates its L2 at entry, so no L2 can hold a stale line of it.
__device__ __forceinline__ u32x4 cld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float cld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void ast16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SC1);
}
__device__ __forceinline__ void ast4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, SC1);
}
__device__ __forceinline__ void ald8f(__amdgpu_buffer_rsrc_t r, uint32_t off, float* v) {
    const u32x4 a = cld16(r, off), b = cld16(r, off + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = __uint_as_float(a[e]); v[4 + e] = __uint_as_float(b[e]); }
}
__device__ __forceinline__ void ast8f(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    ast16(r, off, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    ast16(r, off + 16, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
}
// x[t][k .. k+7] as hi / lo bf16 fragments (the layout of fm_device.h) in the arena
__device__ __forceinline__ void afrag8(__amdgpu_buffer_rsrc_t r, uint32_t base, int t, int k, const float* v) {
    u32x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h, l;
        split_pair(v[2 * i], v[2 * i + 1], h, l);
        hi[i] = h;
        lo[i] = l;
    }
    const uint32_t off = base + (uint32_t)frag_offset(t, k);
    ast16(r, off, hi);
    ast16(r, off + 1024, lo);
}
__device__ __forceinline__ void ld8g(const float* p, float* v) {
    const f32x4_t a = *gp((const f32x4_t*)p), b = *gp((const f32x4_t*)(p + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}
__device__ __forceinline__ void ld8b(const uint16_t* p, float* v) {
    const u32x4 a = *gp((const u32x4*)p);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[2 * e] = bf16_lo(a[e]); v[2 * e + 1] = bf16_hi(a[e]); }
}

// LDS-direct load of 16 bytes per lane (lane l's bytes land at lds + 16 l; lds is wave-uniform, in m0). Inline asm
// so that the compiler's own wait bookkeeping does not see these loads; the producer waits for them explicitly.
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
    const unsigned la =
        __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)((__attribute__((address_space(3))) void*)lds));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory", "m0");
}
template <int N> __device__ __forceinline__ void wait_vm() {   // vmcnt = N, other counters at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void cfence() { asm volatile("" ::: "memory"); }

// Byte offset, inside a chunk, of 16-byte piece q of row r. The XOR swizzles make the consumers' operand reads
// conflict-free; the producer fetches, for LDS position P, the global piece whose swizzled position is P.
__device__ __forceinline__ int w_piece(int r, int q) { return 16 * (r * 32 + (q ^ (r & 15))); }   // weights
__device__ __forceinline__ int k_piece(int r, int q) { return 16 * (r * 16 + (q ^ (r & 15))); }   // K: 32 keys
__device__ __forceinline__ int v_piece(int d, int q) { return 16 * (d * 4 + (q ^ ((d >> 2) & 3))); }   // V: [128][32]

__device__ __forceinline__ bool late(Ctx& x, const DraftArgs& a) {
    if (lds_ld(x.abort)) return true;
    if ((long long)__builtin_amdgcn_s_memrealtime() > x.deadline) {   // give up: tell the work-group and the host
        lds_st(x.abort, 1u);
        __hip_atomic_store(gpw(a.sync) + 8 * 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    return false;
}

// Barrier of the consumer waves only (the producer never joins): an LDS arrival counter.
__device__ __forceinline__ bool cbar(Ctx& x, const DraftArgs& a) {
    x.bar_target += DR_WAVES;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS writes are done
    if (x.lane == 0) __hip_atomic_fetch_add(x.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (lds_ld(x.bar) < x.bar_target) {
        if (late(x, a)) return false;
        __builtin_amdgcn_s_sleep(0);
    }
    cfence();
    return true;
}

// Grid barrier between phases: the work-group's stores are complete, one arrival on its XCD label's counter, then
// every consumer wave waits for all eight counters.
__device__ __forceinline__ bool grid_barrier(Ctx& x, const DraftArgs& a) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!cbar(x, a)) return false;
    if (x.wave == 0 && x.lane == 0)
        __hip_atomic_fetch_add(gpw(a.sync) + (x.g & 7) * 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t b = ++x.nbar;
    for (;;) {
        bool ok = true;
        if (x.lane < 8) {
            const uint32_t v = __hip_atomic_load(gpw(a.sync) + x.lane * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = v >= b * (uint32_t)((a.G - x.lane + 7) >> 3);
        }
        if (__all(ok)) break;
        if (late(x, a)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    cfence();
    return true;
}

__device__ __forceinline__ bool wait_chunk(Ctx& x, const DraftArgs& a, int q) {
    const uint32_t want = (uint32_t)(q / DR_RING) + 1u;
    uint32_t* r = x.ready + q % DR_RING;
    while (lds_ld(r) < want) {
        if (late(x, a)) return false;
        __builtin_amdgcn_s_sleep(0);
    }
    cfence();
    return true;
}
__device__ __forceinline__ void release_chunk(Ctx& x, int q) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of the slot have returned
    lds_st(x.freed + q % DR_RING, (uint32_t)(q / DR_RING) + 1u);
}
__device__ __forceinline__ const uint8_t* chunk_ptr(const Ctx& x, int q) {
    return x.lds + RING_OFF + (q % DR_RING) * DR_CHUNK;
}

// Sum over the 256 consumer threads; red is 8 floats of scratch (two banks, alternating by `turn`).
__device__ __forceinline__ bool csum(Ctx& x, const DraftArgs& a, float v, float* red, int& turn, float& out) {
    v = wave_sum(v);
    float* rb = red + 4 * (turn & 1);
    ++turn;
    if (x.lane == 0) rb[x.wave] = v;
    if (!cbar(x, a)) return false;
    out = (rb[0] + rb[1]) + (rb[2] + rb[3]);
    return true;
}

// ── producer ────────────────────────────────────────────────────────────────────────────────────
__device__ __forceinline__ void produce(Ctx& x, const DraftArgs& a) {
    int c = 0, pub = 0;
    const int lane = x.lane;
    auto publish = [&](int p) { lds_st(x.ready + p % DR_RING, (uint32_t)(p / DR_RING) + 1u); };
    // kind 0: weights, 16 rows x 256 columns, row stride `stride`; 1: K, 32 keys x 128, row stride `stride`;
    // 2: V, one head's 32-position tile block (128 x 32 contiguous)
    auto issue = [&](int kind, const uint16_t* p, int stride) -> bool {
        const uint32_t need = (uint32_t)(c / DR_RING);
        const uint32_t* fr = x.freed + c % DR_RING;
        while (lds_ld(fr) < need) {
            if (late(x, a)) return false;
            __builtin_amdgcn_s_sleep(0);
        }
        cfence();
        uint8_t* dst = x.lds + RING_OFF + (c % DR_RING) * DR_CHUNK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int P = 64 * j + lane;
            const uint16_t* src;
            if (kind == 0) {
                const int r = P >> 5, q = (P & 31) ^ (r & 15);
                src = p + (size_t)r * stride + 8 * q;
            } else if (kind == 1) {
                const int r = P >> 4, q = (P & 15) ^ (r & 15);
                src = p + (size_t)r * stride + 8 * q;
            } else {
                const int d = P >> 2, q = (P & 3) ^ ((d >> 2) & 3);
                src = p + d * 32 + 8 * q;
            }
            lds_load16(src, dst + j * 1024);
        }
        ++c;
        if (c - pub > DEPTH) {
            wait_vm<8 * DEPTH>();   // every chunk before the last DEPTH has landed
            publish(pub++);
        }
        return true;
    };
    schedule(a, [&](int k, int l) -> bool {
        const int n = n_items(a, x, k);
        CLayer& L = layer(a, l);
        for (int item = x.g; item < n; item += a.G) {
            GemmItem gi;
            if (gemm_item(a, x, k, l, item, gi)) {
                for (int j = 0; j < gi.nck; ++j)
                    if (!issue(0, gi.W + 256 * j, gi.K)) return false;
            } else if (k == PH_A3X) {   // cross-attention: the context keys of head h, run group rg
                const int h = item / x.xgroups, rg = item % x.xgroups;
                for (int sl = 0; sl < x.cpw; ++sl)
                    for (int w = 0; w < DR_WAVES; ++w) {
                        if (!x_exists(x, rg, w, sl)) continue;
                        const int st = (4 * rg + w) * x.cpw + sl;
                        if (!issue(1, L.kc + (size_t)(32 * st) * a.D + h * HD, a.D)) return false;
                        if (!issue(2, L.vc + ((size_t)st * a.D + h * HD) * 32, 0)) return false;
                    }
            }
        }
        return true;
    });
    wait_vm<0>();
    while (pub < c) publish(pub++);
}

// ── consumers: projections ──────────────────────────────────────────────────────────────────────
__device__ __forceinline__ bool rms_anchor_row(Ctx& x, const DraftArgs& a, float* cvec, float* red, int& turn) {
    // c = RMSNorm(sum of the anchor_proj slabs + bias; anchor_norm), one row, into LDS
    const int i0 = 8 * x.tid;
    const bool on = i0 < a.D;
    const int ii = on ? i0 : 0;
    float v[8], b[8], w[8];
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    for (int s = 0; s < a.S_a1; ++s) {
        float p[8];
        ald8f(x.ar, a.a1 + (uint32_t)((s * a.D + ii) * 4), p);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += p[e];
    }
    ld8b(a.bap + ii, b);
    ld8b(a.anorm + ii, w);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        v[e] += b[e];
        q += on ? v[e] * v[e] : 0.f;
    }
    float ss;
    if (!csum(x, a, q, red, turn, ss)) return false;
    const float r = 1.f / sqrtf(ss / (float)a.D + a.rms_eps);
    if (on) {
#pragma unroll
        for (int e = 0; e < 8; ++e) cvec[i0 + e] = v[e] * r * w[e];
    }
    return cbar(x, a);
}

__device__ __forceinline__ bool gemm_run(Ctx& x, const DraftArgs& a, int k, int l, const GemmItem& gi, bool& c_ready, int& turn) {
    CLayer& L = layer(a, l);
    const int r = x.lane & 15, g4 = x.lane >> 4;
    const int base = x.seq;
    x.seq += gi.nck;
    f32x4_t* red = (f32x4_t*)(x.lds + SCR_OFF);                 // [4][64]
    float* tile = (float*)(x.lds + SCR_OFF + 4096);              // [16][17]
    float* cvec = (float*)(x.lds + SCR_OFF + 4096 + 1088);       // [D]
    float* sred = (float*)(x.lds + SCR_OFF + 4096 + 1088 + 8192);   // [8]
    int src = 0;   // 0: arena fragments at xoff; 1: the anchor's table row; 2: the anchor context row c (LDS)
    uint32_t xoff = 0;
    switch (k) {
    case PH_A1: src = 1; break;
    case PH_A3X: src = 2; break;
    case PH_OC: xoff = L.mfrag; break;
    case PH_O: xoff = L.sao; break;
    case PH_QC: xoff = L.hc; break;
    case PH_F1: xoff = L.hm; break;
    case PH_F2: xoff = L.u; break;
    case PH_QKV: xoff = L.h0; break;
    default: xoff = a.hf; break;   // PH_HEAD
    }
    if (src == 2 && !c_ready) {
        if (!rms_anchor_row(x, a, cvec, sred, turn)) return false;
        c_ready = true;
    }
    int arow = 0;
    if (src == 1) {
        const int id = *gp(x.anchor);
        arow = id < 0 ? 0 : (id >= a.V ? a.V - 1 : id);   // ids outside the table are clamped into it
    }
    // B operands (the activations) of this wave's chunks j0 = wave, j1 = wave + 4 (nck <= 8), one chunk's worth of
    // registers: the second chunk's are loaded once the first chunk's products are issued
    u32x4 bh[8], bl[8];
    auto loadB = [&](int j, u32x4* h, u32x4* lo) {
        const int s0 = (gi.k0 >> 5) + 8 * j;   // first k-step of chunk j
        if (src == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t off = xoff + (uint32_t)((s0 + i) * FRAG_STEP_BYTES + x.lane * 16);
                h[i] = cld16(x.ar, off);
                lo[i] = cld16(x.ar, off + 1024);
            }
        } else if (src == 1) {   // bf16 row: hi = the value, lo = 0; rows 1..15 are zero
            const uint16_t* e = a.E + (size_t)arow * a.Ht + s0 * 32 + 8 * g4;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 v = *gp((const u32x4*)(e + 32 * i));
                h[i] = r == 0 ? v : u32x4{0u, 0u, 0u, 0u};
                lo[i] = u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float* cv = cvec + (s0 + i) * 32 + 8 * g4;
                uint32_t hh[4], ll[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    split_pair(r == 0 ? cv[2 * e] : 0.f, r == 0 ? cv[2 * e + 1] : 0.f, hh[e], ll[e]);
                h[i] = u32x4{hh[0], hh[1], hh[2], hh[3]};
                lo[i] = u32x4{ll[0], ll[1], ll[2], ll[3]};
            }
        }
    };
    const int j0 = x.wave, j1 = x.wave + DR_WAVES;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto mma_chunk = [&](int j) -> bool {
        if (!wait_chunk(x, a, base + j)) return false;
        const uint8_t* ch = chunk_ptr(x, base + j);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 A = *(const u32x4*)(ch + w_piece(r, 4 * i + g4));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                          __builtin_bit_cast(bf16x8_t, bh[i]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                          __builtin_bit_cast(bf16x8_t, bl[i]), acc, 0, 0, 0);
        }
        release_chunk(x, base + j);
        return true;
    };
    if (j0 < gi.nck) {
        loadB(j0, bh, bl);
        if (!mma_chunk(j0)) return false;
    }
    if (j1 < gi.nck) {
        loadB(j1, bh, bl);
        if (!mma_chunk(j1)) return false;
    }
    // the four waves' partial tiles, summed in a fixed order
    red[x.wave * 64 + x.lane] = acc;
    if (!cbar(x, a)) return false;
    const int el = x.tid & 63, rr = x.tid >> 6;
    const float v = ((red[el][rr] + red[64 + el][rr]) + red[128 + el][rr]) + red[192 + el][rr];
    const int t = el & 15, ml = 4 * (el >> 4) + rr, m = gi.m + ml;   // activation row t, output index m
    switch (k) {
    case PH_A1:
        if (t == 0) ast4(x.ar, a.a1 + (uint32_t)((gi.split * a.D + m) * 4), v);
        break;
    case PH_A3X:
        if (t == 0) ast4(x.ar, L.a3 + (uint32_t)(m * 4), v);
        break;
    case PH_HEAD:
        gpw(x.hidden_out)[(size_t)t * a.Ht + m] = v + bf16_to_f32(gp(a.bhead)[m]);
        break;
    case PH_F1: {
        tile[t * 17 + ml] = gelu_erf(v + bf16_to_f32(gp(L.b1)[m]));
        if (!cbar(x, a)) return false;
        if (x.tid < 32) {
            const int tt = x.tid >> 1, hh = x.tid & 1;
            float vals[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[e] = tile[tt * 17 + 8 * hh + e];
            afrag8(x.ar, L.u, tt, gi.m + 8 * hh, vals);
        }
        break;
    }
    default: {   // partial slabs [S][16][ld]: the tile through LDS, out as 16-byte pieces of its rows
        uint32_t dst;
        int ld = a.D;
        switch (k) {
        case PH_OC: dst = L.ocs; break;
        case PH_O: dst = L.os; break;
        case PH_QC: dst = L.qcs; break;
        case PH_F2: dst = L.f2s; break;
        default: dst = L.qkv; ld = 3 * a.D; break;   // PH_QKV
        }
        tile[t * 17 + ml] = v;
        if (!cbar(x, a)) return false;
        if (x.tid < 64) {
            const int tt = x.tid >> 2, c4 = 4 * (x.tid & 3);
            const float* tr = tile + tt * 17 + c4;
            ast16(x.ar, dst + (uint32_t)(((gi.split * T + tt) * ld + gi.m + c4) * 4),
                  u32x4{__float_as_uint(tr[0]), __float_as_uint(tr[1]), __float_as_uint(tr[2]), __float_as_uint(tr[3])});
        }
        break;
    }
    }
    return cbar(x, a);   // the scratch is free for the next item
}

// ── consumers: residual + norm rows ─────────────────────────────────────────────────────────────
__device__ __forceinline__ bool rows_run(Ctx& x, const DraftArgs& a, int k, int l, int t, int& turn) {
    const int D = a.D, i0 = 8 * x.tid;
    const bool on = i0 < D;
    const int ii = on ? i0 : 0;
    float* red = (float*)(x.lds + SCR_OFF);
    // base row, partial slabs (+ bias), gate, the LN-mod row, and where the results go
    int lp;                      // layer of the pending residual update
    int nrow_gate, nrow_ln;      // modulation rows: the gate's and the LN-mod's
    uint32_t part, xout, fout;
    int S;
    const uint16_t* bias = nullptr;
    bool base_global = false;
    uint32_t xin = 0;
    float* dbg = nullptr;
    switch (k) {
    case PH_R2:   // x = x_self + gate_ca (cross o_proj); h = LNmod_mlp(x)
        lp = l; part = layer(a, l).ocs; S = a.S_oc; nrow_gate = 3 * l + 1; nrow_ln = 3 * l + 2;
        base_global = l == 0; xin = l == 0 ? 0 : layer(a, l).xs;
        xout = layer(a, l).xm; fout = layer(a, l).hm;
        break;
    case PH_R0:   // x = x_mlp(l-1) + gate_mlp(l-1) (fc2 + b2); h = LNmod_sa(l)
        lp = l - 1; part = layer(a, lp).f2s; S = a.S_f2; bias = layer(a, lp).b2; nrow_gate = 3 * lp + 2; nrow_ln = 3 * l;
        xin = layer(a, lp).xm; xout = layer(a, l).x0; fout = layer(a, l).h0;
        if (x.debug) dbg = x.debug + ((size_t)lp * T + t) * D;
        break;
    case PH_R1:   // x = x0 + gate_sa (self o_proj); h = LNmod_ca(l)
        lp = l; part = layer(a, l).os; S = a.S_o; nrow_gate = 3 * l; nrow_ln = 3 * l + 1;
        xin = layer(a, l).x0; xout = layer(a, l).xs; fout = layer(a, l).hc;
        break;
    default:      // PH_RF: x = x_mlp(last) + gate_mlp(last) (fc2 + b2); h = LNmod_final
        lp = a.layers - 1; part = layer(a, lp).f2s; S = a.S_f2; bias = layer(a, lp).b2; nrow_gate = 3 * lp + 2;
        nrow_ln = 3 * a.layers; xin = layer(a, lp).xm; xout = a.xf; fout = a.hf;
        if (x.debug) dbg = x.debug + ((size_t)lp * T + t) * D;
        break;
    }
    (void)lp;
    float v[8], u[8], gt[8], sc[8], sh[8];
    if (base_global) ld8g(a.x1 + (size_t)t * D + ii, v);
    else ald8f(x.ar, xin + (uint32_t)((t * D + ii) * 4), v);
    for (int e = 0; e < 8; ++e) u[e] = 0.f;
    for (int s = 0; s < S; ++s) {
        float p[8];
        ald8f(x.ar, part + (uint32_t)(((s * T + t) * D + ii) * 4), p);
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] += p[e];
    }
    if (bias) {
        float b[8];
        ld8b(bias + ii, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] += b[e];
    }
    const float* mg = a.mod + (size_t)nrow_gate * 3 * D;
    const float* ml = a.mod + (size_t)nrow_ln * 3 * D;
    ld8g(mg + 2 * D + ii, gt);
    ld8g(ml + ii, sc);
    ld8g(ml + D + ii, sh);
    float s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        v[e] += gt[e] * u[e];
        s1 += on ? v[e] : 0.f;
    }
    if (on) {
        ast8f(x.ar, xout + (uint32_t)((t * D + i0) * 4), v);
        if (dbg) {
            *gpw((f32x4_t*)(dbg + i0)) = f32x4_t{v[0], v[1], v[2], v[3]};
            *gpw((f32x4_t*)(dbg + i0 + 4)) = f32x4_t{v[4], v[5], v[6], v[7]};
        }
    }
    float sum;
    if (!csum(x, a, s1, red, turn, sum)) return false;
    const float mean = sum / (float)D;
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float dd = v[e] - mean;
        s2 += on ? dd * dd : 0.f;
    }
    float var;
    if (!csum(x, a, s2, red, turn, var)) return false;
    const float rs = 1.f / sqrtf(var / (float)D + a.ln_eps);
    if (on) {
        float hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (v[e] - mean) * rs * (1.f + sc[e]) + sh[e];
        afrag8(x.ar, fout, t, i0, hv);
    }
    return true;
}

// ── consumers: self-attention of the 16 slots, one head ─────────────────────────────────────────
__device__ __forceinline__ bool self_run(Ctx& x, const DraftArgs& a, int l, int h) {
    constexpr int SEG = HD / 8, VPT = HD / 16, QP = HD + 4;
    CLayer& L = layer(a, l);
    const int D = a.D, tid = x.tid;
    float* QK = (float*)(x.lds + SCR_OFF);            // [32][QP]: q rows, then k rows
    float* Vs = QK + 32 * QP;                          // [16][QP]
    float* Ps = Vs + 16 * QP;                          // [16][17]
    const int row = tid >> 3, seg = tid & 7, w = row >> 4, t = row & 15;
    const uint32_t slab = (uint32_t)(T * 3 * D * 4);
    float xq[SEG], cs[SEG / 2], sn[SEG / 2], nw[SEG], v[VPT];
    for (int j = 0; j < SEG; ++j) xq[j] = 0.f;
    for (int s = 0; s < a.S_qkv; ++s) {
        const uint32_t off = L.qkv + s * slab + (uint32_t)((t * 3 * D + w * D + h * HD + seg * SEG) * 4);
#pragma unroll
        for (int j = 0; j < SEG / 4; ++j) {
            const u32x4 f = cld16(x.ar, off + 16 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) xq[4 * j + e] += __uint_as_float(f[e]);
        }
    }
    const float* rt = a.rope + (size_t)(x.pos + 1 + t) * HD + seg * (SEG / 2);
#pragma unroll
    for (int j = 0; j < SEG / 2; ++j) { cs[j] = gp(rt)[j]; sn[j] = gp(rt)[HD / 2 + j]; }
    const uint16_t* nb = (w ? L.kn : L.qn) + seg * SEG;
#pragma unroll
    for (int j = 0; j < SEG; ++j) nw[j] = bf16_to_f32(gp(nb)[j]);
    const int vt = tid >> 4, vp = tid & 15;
    for (int j = 0; j < VPT; ++j) v[j] = 0.f;
    for (int s = 0; s < a.S_qkv; ++s) {
        const uint32_t off = L.qkv + s * slab + (uint32_t)((vt * 3 * D + 2 * D + h * HD + vp * VPT) * 4);
#pragma unroll
        for (int j = 0; j < VPT / 4; ++j) {
            const u32x4 f = cld16(x.ar, off + 16 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * j + e] += __uint_as_float(f[e]);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < SEG; ++j) ss += xq[j] * xq[j];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    const float r = 1.f / sqrtf(ss / (float)HD + a.qk_eps);
#pragma unroll
    for (int j = 0; j < SEG / 2; ++j) {
        const float x0 = xq[2 * j] * (nw[2 * j] * r), x1 = xq[2 * j + 1] * (nw[2 * j + 1] * r);
        xq[2 * j] = x0 * cs[j] - x1 * sn[j];
        xq[2 * j + 1] = x1 * cs[j] + x0 * sn[j];
    }
#pragma unroll
    for (int j = 0; j < SEG / 4; ++j)
        *(float4*)(QK + row * QP + seg * SEG + 4 * j) = make_float4(xq[4 * j], xq[4 * j + 1], xq[4 * j + 2], xq[4 * j + 3]);
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j)
        *(float4*)(Vs + vt * QP + vp * VPT + 4 * j) = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    if (!cbar(x, a)) return false;
    {
        const int qt = tid >> 4, uu = tid & 15;
        const float* q = QK + qt * QP;
        const float* kk = QK + (16 + uu) * QP;
        float s = 0.f;
#pragma unroll 8
        for (int d = 0; d < HD; d += 4) {
            const float4 qa = *(const float4*)(q + d), kb = *(const float4*)(kk + d);
            s += qa.x * kb.x + qa.y * kb.y + qa.z * kb.z + qa.w * kb.w;
        }
        s *= a.scale;
        float m = s;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float e = expf(s - m);
        float z = e;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
        Ps[qt * 17 + uu] = e / z;
    }
    if (!cbar(x, a)) return false;
    {
        const int ot = tid / (HD / 8), d0 = (tid % (HD / 8)) * 8;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        for (int uu = 0; uu < T; ++uu) {
            const float p = Ps[ot * 17 + uu];
            const float4 v0 = *(const float4*)(Vs + uu * QP + d0), v1 = *(const float4*)(Vs + uu * QP + d0 + 4);
            o[0] += p * v0.x; o[1] += p * v0.y; o[2] += p * v0.z; o[3] += p * v0.w;
            o[4] += p * v1.x; o[5] += p * v1.y; o[6] += p * v1.z; o[7] += p * v1.w;
        }
        afrag8(x.ar, L.sao, ot, h * HD + d0, o);
    }
    return cbar(x, a);
}

// ── consumers: cross-attention over the context keys, one head, four runs (one per wave) ───────
__device__ __forceinline__ bool cross_run(Ctx& x, const DraftArgs& a, int l, int item) {
    constexpr int QROW = HD + 8, NS = HD / 32, ND = HD / 16;
    CLayer& L = layer(a, l);
    const int h = item / x.xgroups, rg = item % x.xgroups;
    const int tid = x.tid, lane = x.lane, r = lane & 15, g4 = lane >> 4;
    _Float16* Qh = (_Float16*)(x.lds + SCR_OFF);
    _Float16* Ql = Qh + 16 * QROW;
    // this item's chunk count, and where this wave's steps sit in the item's chunk order
    const int base = x.seq;
    int total = 0;
    for (int sl = 0; sl < x.cpw; ++sl) total += 2 * x_count(x, rg, sl);
    x.seq += total;
    {   // the 16 queries of head h: the sum of the q slabs, head RMSNorm, RoPE at pos + 1 + t, f16 hi + lo
        constexpr int QS = HD / 16;
        const int qt = tid >> 4, qseg = tid & 15;
        float q[QS], nw[QS], cs[QS / 2], sn[QS / 2];
        for (int j = 0; j < QS; ++j) q[j] = 0.f;
        if (l == 0) {
            for (int s = 0; s < a.q0c_slabs; ++s) {
                const float* p = a.q0c + s * a.q0c_stride + (size_t)qt * a.D + h * HD + qseg * QS;
                float f[8];
                ld8g(p, f);
#pragma unroll
                for (int j = 0; j < QS; ++j) q[j] += f[j];
            }
        } else {
            for (int s = 0; s < a.S_qc; ++s) {
                float f[8];
                ald8f(x.ar, L.qcs + (uint32_t)(((s * T + qt) * a.D + h * HD + qseg * QS) * 4), f);
#pragma unroll
                for (int j = 0; j < QS; ++j) q[j] += f[j];
            }
        }
        const float* rt = a.rope + (size_t)(x.pos + 1 + qt) * HD + qseg * (QS / 2);
#pragma unroll
        for (int j = 0; j < QS / 2; ++j) { cs[j] = gp(rt)[j]; sn[j] = gp(rt)[HD / 2 + j]; }
#pragma unroll
        for (int j = 0; j < QS; ++j) nw[j] = bf16_to_f32(gp(L.cqn)[qseg * QS + j]);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < QS; ++j) ss += q[j] * q[j];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
        const float rr = 1.f / sqrtf(ss / (float)HD + a.qk_eps);
#pragma unroll
        for (int j = 0; j < QS; ++j) q[j] *= nw[j] * rr;
#pragma unroll
        for (int j = 0; j < QS / 2; ++j) {
            const float x0 = q[2 * j], x1 = q[2 * j + 1];
            q[2 * j] = x0 * cs[j] - x1 * sn[j];
            q[2 * j + 1] = x1 * cs[j] + x0 * sn[j];
        }
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const _Float16 hi = (_Float16)q[j];
            Qh[qt * QROW + qseg * QS + j] = hi;
            Ql[qt * QROW + qseg * QS + j] = (_Float16)(q[j] - (float)hi);
        }
    }
    if (!cbar(x, a)) return false;
    f16x8_t qh[NS], ql[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        qh[s] = *(const f16x8_t*)(Qh + r * QROW + 32 * s + 8 * g4);
        ql[s] = *(const f16x8_t*)(Ql + r * QROW + 32 * s + 8 * g4);
    }
    const int w = x.wave, run = 4 * rg + w;
    const int ncache = x.pos;   // keys [0, pos): the anchor key at pos is merged later
    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int before = 0;   // chunks of the item before step sl's chunks
    for (int sl = 0; sl < x.cpw; ++sl) {
        const int cnt = x_count(x, rg, sl);
        if (x_exists(x, rg, w, sl)) {
            int mine = 0;
            for (int ww = 0; ww < w; ++ww) mine += x_exists(x, rg, ww, sl) ? 1 : 0;
            const int qk = base + before + 2 * mine, qv = qk + 1;
            const int st = run * x.cpw + sl, k0 = 32 * st;
            if (!wait_chunk(x, a, qk) || !wait_chunk(x, a, qv)) return false;
            const uint8_t* Kc = chunk_ptr(x, qk);
            const uint8_t* Vc = chunk_ptr(x, qv);
            f32x4_t sc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const f16x8_t A = *(const f16x8_t*)(Kc + k_piece(16 * kt + r, 4 * s + g4));
                    sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[s], sc[kt], 0, 0, 0);
                    sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql[s], sc[kt], 0, 0, 0);
                }
            }
            // online softmax of query r over the step's keys 16 kt + 4 g + i (keys past the context: -inf)
            float sv[2][4], cm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kidx = k0 + 16 * kt + 4 * g4 + i;
                    const float s = kidx < ncache ? sc[kt][i] * a.scale : -INFINITY;
                    sv[kt][i] = s;
                    cm = fmaxf(cm, s);
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
            for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 4 * g4 + j, 64);
            // V of keys past the context is masked to zero (it may hold anything)
            uint32_t mk0[2], mk1[2];
            {
                const int p0 = k0 + 4 * g4, p1 = k0 + 16 + 4 * g4;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    mk0[e] = (p0 + 2 * e < ncache ? 0xffffu : 0u) | (p0 + 2 * e + 1 < ncache ? 0xffff0000u : 0u);
                    mk1[e] = (p1 + 2 * e < ncache ? 0xffffu : 0u) | (p1 + 2 * e + 1 < ncache ? 0xffff0000u : 0u);
                }
            }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const int d = 16 * dt + r;
                const uint2 v0 = *(const uint2*)(Vc + v_piece(d, g4 >> 1) + 8 * (g4 & 1));
                const uint2 v1 = *(const uint2*)(Vc + v_piece(d, 2 + (g4 >> 1)) + 8 * (g4 & 1));
                const f16x8_t B = __builtin_bit_cast(
                    f16x8_t, make_uint4(v0.x & mk0[0], v0.y & mk0[1], v1.x & mk1[0], v1.y & mk1[1]));
#pragma unroll
                for (int j = 0; j < 4; ++j) o[dt][j] *= al[j];
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, B, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, o[dt], 0, 0, 0);
            }
            release_chunk(x, qk);
            release_chunk(x, qv);
        }
        before += 2 * cnt;
    }
    // this run's partial: unnormalised o, running max, running sum (an empty run: max -inf, sum 0, o 0)
    const int nruns = 4 * x.xgroups;
    const uint32_t po = L.xpart + (uint32_t)(((h * nruns + run) * T) * (HD + 2) * 4);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) ast4(x.ar, po + (uint32_t)(((4 * g4 + j) * (HD + 2) + 16 * dt + r) * 4), o[dt][j]);
    if (g4 == 0) {
        ast4(x.ar, po + (uint32_t)((r * (HD + 2) + HD) * 4), m_run);
        ast4(x.ar, po + (uint32_t)((r * (HD + 2) + HD + 1) * 4), l_run);
    }
    return cbar(x, a);   // the q tiles are free for the next item
}

// ── consumers: merge of the runs and the anchor key, one (head, slot) ───────────────────────────
__device__ __forceinline__ bool merge_run(Ctx& x, const DraftArgs& a, int l, int item, int& turn) {
    constexpr int DV = HD / 4, NG = 256 / DV;   // 32 threads per dimension set, 8 run groups
    CLayer& L = layer(a, l);
    const int h = item / T, t = item % T, tid = x.tid;
    float* so = (float*)(x.lds + SCR_OFF);        // [NG][HD]
    float* sm = so + NG * HD;                     // [NG]
    float* sl = sm + NG;                          // [NG]
    float* qa = sl + NG;                          // [HD] prepared q of slot t
    float* va = qa + HD;                          // [HD] the anchor's v
    float* red = va + HD;                         // [8]
    const int nruns = 4 * x.xgroups;
    // the runs' partials of (h, t)
    const int d4 = tid % DV, cg = tid / DV;
    float M = -INFINITY, Ls = 0.f;
    float O[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = cg; c < nruns; c += NG) {
        const uint32_t p = L.xpart + (uint32_t)((((h * nruns + c) * T) + t) * (HD + 2) * 4);
        const u32x4 ov = cld16(x.ar, p + 16 * d4);
        const float mv = cld4(x.ar, p + HD * 4), lv = cld4(x.ar, p + (HD + 1) * 4);
        if (mv == -INFINITY) continue;
        const float Mn = fmaxf(M, mv);
        const float a0 = (M == -INFINITY) ? 0.f : expf(M - Mn), a1 = expf(mv - Mn);
        Ls = Ls * a0 + lv * a1;
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] = O[e] * a0 + __uint_as_float(ov[e]) * a1;
        M = Mn;
    }
    if (d4 == 0) { sm[cg] = M; sl[cg] = Ls; }
#pragma unroll
    for (int e = 0; e < 4; ++e) so[cg * HD + 4 * d4 + e] = O[e];
    // the anchor key: threads 0..127 prepare q_t (dimension tid), threads 128..255 the anchor's k (tid - 128)
    const int d = tid & (HD - 1);
    const bool isk = tid >= HD;
    float xv = 0.f, vv = 0.f;
    if (!isk) {
        if (l == 0) {
            for (int s = 0; s < a.q0c_slabs; ++s) xv += gp(a.q0c)[s * a.q0c_stride + (size_t)t * a.D + h * HD + d];
        } else {
            for (int s = 0; s < a.S_qc; ++s) xv += cld4(x.ar, L.qcs + (uint32_t)(((s * T + t) * a.D + h * HD + d) * 4));
        }
        vv = cld4(x.ar, L.a3 + (uint32_t)((a.D + h * HD + d) * 4));
    } else {
        xv = cld4(x.ar, L.a3 + (uint32_t)((h * HD + d) * 4));
    }
    const float wnorm = bf16_to_f32(isk ? gp(L.ckn)[d] : gp(L.cqn)[d]);
    const int pp = isk ? x.pos : x.pos + 1 + t;
    const float cs = gp(a.rope)[(size_t)pp * HD + (d >> 1)], sn = gp(a.rope)[(size_t)pp * HD + HD / 2 + (d >> 1)];
    float sq = wave_sum(xv * xv);
    if (x.lane == 0) red[x.wave] = sq;
    if (!cbar(x, a)) return false;
    const float ssum = isk ? red[2] + red[3] : red[0] + red[1];
    const float y = xv * (1.f / sqrtf(ssum / (float)HD + a.qk_eps)) * wnorm;
    const float yp = __shfl_xor(y, 1, 64);   // the other member of the RoPE pair (2i, 2i + 1)
    const float yr = (d & 1) ? y * cs + yp * sn : y * cs - yp * sn;
    if (!isk) { qa[d] = yr; va[d] = vv; }
    if (isk && t == 0) {   // the anchor's K row (normed, rotated) and V row into the cache at pos
        gpw(L.kc)[(size_t)x.pos * a.D + h * HD + d] = f32_to_f16(yr);
    }
    if (!isk && t == 0) {
        gpw(L.vc)[((size_t)(x.pos >> 5) * a.D + h * HD + d) * 32 + (x.pos & 31)] = f32_to_f16(vv);
    }
    if (!cbar(x, a)) return false;
    float prod = isk ? qa[d] * yr : 0.f;
    float sc;
    if (!csum(x, a, prod, red + 4, turn, sc)) return false;
    sc *= a.scale;
    if (tid < HD / 8) {
        const int d0 = tid * 8;
        float MM = sc;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) MM = fmaxf(MM, sm[gg]);
        const float wa = expf(sc - MM);
        float Lt = wa, o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = wa * va[d0 + e];
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            const float wg = sm[gg] == -INFINITY ? 0.f : expf(sm[gg] - MM);
            Lt += wg * sl[gg];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += wg * so[gg * HD + d0 + e];
        }
        const float il = 1.f / Lt;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= il;
        afrag8(x.ar, L.mfrag, t, h * HD + d0, o);
    }
    return cbar(x, a);
}

__global__ __launch_bounds__(NTH, 1) void draft_kernel(const DraftArgs* __restrict__ ap, int pos,
                                                       const int32_t* anchor, float* hidden_out, float* debug) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const DraftArgs& a = *ap;
    Ctx x;
    x.pos = pos;
    draft_xsplit(pos, a.H, a.G, x.nsteps, x.cpw, x.xgroups);
    x.anchor = anchor;
    x.hidden_out = hidden_out;
    x.debug = debug;
    x.lds = lds;
    x.ready = (uint32_t*)(lds + FLAG_OFF);
    x.freed = x.ready + DR_RING;
    x.bar = x.freed + DR_RING;
    x.abort = x.bar + 1;
    x.ar = rsrc(a.arena);
    x.g = blockIdx.x;
    x.tid = threadIdx.x;
    x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform in a wave: scalar branches
    x.lane = threadIdx.x & 63;
    x.deadline = (long long)__builtin_amdgcn_s_memrealtime() + a.limit;
    x.bar_target = 0;
    x.nbar = 0;
    x.seq = 0;
    if (threadIdx.x < 2 * DR_RING + 2) lds_st(x.ready + threadIdx.x, 0u);
    __syncthreads();   // the only full-work-group barrier: the flags start at zero
    if (x.wave == DR_WAVES) {
        produce(x, a);
        return;
    }
    int turn = 0;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // no line of an earlier launch's arena stays in this L2
    schedule(a, [&](int k, int l) -> bool {
        const int n = n_items(a, x, k);
        bool c_ready = false;
        for (int item = x.g; item < n; item += a.G) {
            bool ok;
            GemmItem gi;
            if (gemm_item(a, x, k, l, item, gi)) ok = gemm_run(x, a, k, l, gi, c_ready, turn);
            else if (k == PH_A3X) ok = cross_run(x, a, l, item);
            else if (k == PH_M) ok = merge_run(x, a, l, item, turn);
            else if (k == PH_SA) ok = self_run(x, a, l, item);
            else ok = rows_run(x, a, k, l, item, turn);
            if (!ok) return false;
        }
        return k == PH_HEAD ? true : grid_barrier(x, a);
    });
}

}  // namespace

int draft_occupancy() {
    static int occ = -1;
    if (occ < 0) {
        int n = 0;
        if (hipFuncSetAttribute((const void*)draft_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, DR_LDS) !=
                hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, draft_kernel, NTH, DR_LDS) != hipSuccess)
            n = 0;
        occ = n;
    }
    return occ;
}

hipError_t launch_draft(const DraftArgs* args, int G, int pos, const int32_t* anchor, float* hidden_out, float* debug,
                        hipStream_t st) {
    if (!args || G < 1 || G > DR_MAX_WG || pos < 0 || !anchor || !hidden_out) return hipErrorInvalidValue;
    if (draft_occupancy() < 1) return hipErrorInvalidConfiguration;   // sets the kernel's LDS limit once
    draft_kernel<<<G, NTH, DR_LDS, st>>>(args, pos, anchor, hidden_out, debug);
    return hipGetLastError();
}
