// fm_api.cpp — the C ABI (include/fm.h): host-side validation, the device workspace plan and the launch sequence
// of every call. All validation happens before anything is enqueued; nothing here allocates device memory or
// synchronises a stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/fm.h"
#include "fm_kernels.h"

namespace {

thread_local std::string g_err;

fm_status fail(fm_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define HIPCHK(expr)                                                                                \
    do {                                                                                            \
        hipError_t e_ = (expr);                                                                     \
        if (e_ != hipSuccess) return fail(FM_E_HIP, "%s: %s", #expr, hipGetErrorString(e_));        \
    } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int TMAX = 16;          // rows of one skinny activation matrix
constexpr int FM_BATCH = 2;       // flow-map requests one batched draft takes (16 rows each)
constexpr int RTICK_MAX = 256;    // tiles of a split residual update (its output width / 16)
constexpr int SATICK_MAX = 64;    // heads of the self-attention tail
// the KV-injection residual updates run unsplit (64 work-groups at its width 1024: 435.9 us per draft against
// 445.8 us split in two with an arrival ticket and 452.8 us split in four)
constexpr int KVI_RESID_SPLIT = 1;
constexpr int QKV_SLABS = 4;      // split-K slabs the attention kernels sum while building q (and k, v)
constexpr int TARGET_WGS = 256;
constexpr int MTP_QKV_SPLIT = 2;   // k-split of the MTP head's q | k | v product (K / 256 chunks must divide by it)   // work-groups wanted per skinny launch (one per CU)
constexpr int PF_SPLIT_WGS = 512; // a k-split prefill launch stays within one round (two 128-tile work-groups per CU)
constexpr int PF_SPLIT_ROWS = 4096;  // prefill context rows kept for k-split slabs

// k-steps per wave the skinny kernel is built for: up to 16 loaded at once, longer ranges in even stages.
bool kw_ok(int kw) {
    return kw == 1 || kw == 2 || kw == 3 || kw == 4 || kw == 5 || kw == 6 || kw == 8 || kw == 10 || kw == 12 ||
           kw == 16 || (kw > 16 && kw % 2 == 0);
}

// k-split of a projection whose slabs the attention kernel sums itself (q, or the self-attention's q|k|v): the
// largest S <= QKV_SLABS leaving each wave whole row-staged chunks (4 k-steps); measured on MI355X this streams a
// 2048 x 2048 weight ~20% faster than the unsplit 128 work-groups.
int pick_qsplit(int K) {
    const int n4 = K / 128;
    for (int S = QKV_SLABS; S > 1; S >>= 1)
        if (n4 % S == 0 && (n4 / S) % 4 == 0) return S;
    return 1;
}

// k-split of a partial-output bf16 skinny GEMM (at most 8 slabs, the consumers' limit). Preference: enough
// work-groups (tiles * S >= TARGET_WGS) with a per-wave range that is a whole number of row-staged chunks
// (KW % 8 == 0); then enough work-groups with any supported range; else the largest supported S.
int pick_split(int M_total, int K) {
    const int n4 = K / 128, tiles = M_total / 16;
    int any_enough = -1, largest = -1;
    for (int S = 1; S <= std::min(8, n4); ++S) {
        if (n4 % S || !kw_ok(n4 / S)) continue;
        largest = S;
        if (tiles * S >= TARGET_WGS) {
            if ((n4 / S) % 8 == 0) return S;
            if (any_enough < 0) any_enough = S;
        }
    }
    return any_enough > 0 ? any_enough : largest;
}

// k-split of a Q8_0 projection (the tile-owning skinny variant): whole 256-column chunks per split, at most 8 slabs;
// the fewest splits that give twice TARGET_WGS work-groups, else the most.
int pick_split_ws(int groups, int K) {
    const int nch = K / 256;
    int S = 1;
    for (int s = 1; s <= std::min(8, nch); ++s) {
        if (nch % s) continue;
        S = s;
        if (groups * s >= 2 * TARGET_WGS) break;
    }
    return S;
}
int ws_groups(int M, bool glu = false) {
    const int tpw = glu ? SK_WS_WAVES / 2 : SK_WS_WAVES;   // tiles per work-group (of each matrix of a gated unit)
    return (M / 16 + tpw - 1) / tpw;
}

// ── the persistent draft kernel (k_draft.hip): which shapes it takes, its k-splits and its arena ─────
// Flow-map drafters with 128-wide heads, 16 slots, widths multiples of 256 up to 2048 (fc1 / head / the anchor's
// K and V take their whole k-range, at most 8 chunks of 256 per work-item).
bool draft_supported(const fm_config& c) {
    return c.variant == FM_VARIANT_FLOWMAP && c.head_dim == 128 && c.block == TMAX && c.dim % 256 == 0 &&
           c.dim <= 2048 && c.dim == c.heads * 128 && c.ffn % 256 == 0 && c.target_dim % 256 == 0;
}

// k-split of a projection in the persistent kernel: the split that minimises the chunks of the busiest work-group
// (items dealt round-robin over G), with at most 8 chunks (two per consumer wave) per item; ties to fewer slabs.
int pick_dsplit(int K, int tiles, int G) {
    const int nk = K / 256;
    int best = -1, best_cost = 0;
    for (int S = 1; S <= nk; ++S) {
        if (nk % S || nk / S > 8) continue;
        const int cost = ((tiles * S + G - 1) / G) * (nk / S);
        if (best < 0 || cost < best_cost) { best = S; best_cost = cost; }
    }
    return best;
}

struct DraftLayout {
    uint32_t a3, xpart, mfrag, ocs, xm, hm, u, f2s, x0, h0, qkv, sao, os, xs, hc, qcs;   // within a layer block
    uint32_t layer_bytes, a1, xf, hf, total, xpart_cap;
    int S_a1, S_qkv, S_o, S_qc, S_oc, S_f2;
};

DraftLayout draft_layout(const fm_config& c, int G) {
    DraftLayout L{};
    const int D = c.dim, tD = D / 16;
    L.S_a1 = pick_dsplit(c.target_dim, tD, G);
    L.S_qkv = pick_dsplit(D, 3 * tD, G);
    L.S_o = L.S_qc = L.S_oc = pick_dsplit(D, tD, G);
    L.S_f2 = pick_dsplit(c.ffn, tD, G);
    // the most cross-attention runs per head any position up to the last draftable one needs
    int cap = 4;
    const int pmax = c.max_ctx - c.block - 1;
    for (int pos = 0; pos <= pmax; pos += 32) {
        int ns, cpw, xg;
        draft_xsplit(pos, c.heads, G, ns, cpw, xg);
        cap = std::max(cap, 4 * xg);
        draft_xsplit(std::min(pos + 31, pmax), c.heads, G, ns, cpw, xg);
        cap = std::max(cap, 4 * xg);
    }
    L.xpart_cap = (uint32_t)cap;
    size_t off = 0;
    auto take = [&](size_t b) { const size_t o = off; off = align256(off + b); return (uint32_t)o; };
    const size_t rowf = (size_t)TMAX * D * 4, frag = (size_t)D * 64;
    L.a3 = take((size_t)2 * D * 4);
    L.xpart = take((size_t)c.heads * cap * TMAX * (c.head_dim + 2) * 4);
    L.mfrag = take(frag);
    L.ocs = take(L.S_oc * rowf);
    L.xm = take(rowf);
    L.hm = take(frag);
    L.u = take((size_t)c.ffn * 64);
    L.f2s = take(L.S_f2 * rowf);
    L.x0 = take(rowf);
    L.h0 = take(frag);
    L.qkv = take(L.S_qkv * 3 * rowf);
    L.sao = take(frag);
    L.os = take(L.S_o * rowf);
    L.xs = take(rowf);
    L.hc = take(frag);
    L.qcs = take(L.S_qc * rowf);
    L.layer_bytes = (uint32_t)off;
    off = (size_t)c.layers * L.layer_bytes;
    L.a1 = take((size_t)L.S_a1 * D * 4);
    L.xf = take(rowf);
    L.hf = take(frag);
    L.total = (uint32_t)off;
    return L;
}

// c1 / c2 of the LayerNorm fold (flow-map): per layer [q, k, v, cross q: 2 dim each][fc1: 2 ffn], then the head
// (2 target_dim); layer 0's first four are unused (its self-attention and cross q are cached at create)
size_t c12_floats(const fm_config& c) { return (size_t)c.layers * 2 * (4 * c.dim + c.ffn) + 2 * (size_t)c.target_dim; }
size_t c12_off(const fm_config& c, int l, int which) {   // which 0..3: q k v cross-q, 4: fc1; l == layers: head
    return (size_t)l * 2 * (4 * c.dim + c.ffn) + (size_t)2 * c.dim * which;
}

// The Q8_0 matrices of a configuration (the MTP head's) with their shapes [M][K]: each is copied at create into the
// MFMA operand layout (launch_q8_tile_copy) and registered under its name + ".qt" (codes) and ".dt" (scales).
struct Q8Mat {
    const char* name;
    int M, K;
};
std::vector<Q8Mat> q8_mats(const fm_config& c) {
    if (c.wtype != FM_W_Q8_0) return {};
    const int H = c.dim, qw = c.heads * 2 * c.head_dim, kw = c.kv_heads * c.head_dim;
    return {{"eh_proj", H, 2 * H},     {"attn_q", qw, H},       {"attn_k", kw, H},     {"attn_v", kw, H},
            {"attn_output", H, c.heads * c.head_dim},           {"ffn_gate", c.ffn, H}, {"ffn_up", c.ffn, H},
            {"ffn_down", H, c.ffn},    {"lm_head", c.vocab, c.target_dim}};
}

// ── workspace plan ──────────────────────────────────────────────────────────────────────────────
struct Plan {
    size_t best, mcut, zeros, rope, fragA, fragH, fragO, fragU, x, part, qkv, attnp, stage, h0, colsc, cmean, hc, pctx,
        pctxn, qout, apart, afrag, cfrag, w16, taps16, rope_pf, echain, q8t, ssq, blockn, zbase, tcond, qkv0, x1, q0c,
        rscale, modc, lnstats, c12, lnfrag, rtick, dargs, dlayers, dsync, arena, total;
    size_t zeros_bytes;
    int best_rows;           // argmax keys (one per row)
    size_t part_floats;      // capacity of the partial buffer
    size_t attnp_bytes;      // capacity of the attention partial buffer
    int rope_rows, rope_dims;
    int nchunk_max;
    size_t qkv_floats;
    int colR;
    int pctx_rows;           // rows of the prefill context buffer (>= max_ctx)
};

int kmax_frag(const fm_config& c) {
    int k = std::max({c.dim, c.target_dim, c.ffn, c.heads * c.head_dim, c.n_taps * c.target_dim});
    if (c.variant == FM_VARIANT_MTP) k = std::max(k, 2 * c.dim);
    return k;
}

int part_need(const fm_config& c) {   // floats per split slab row-set: max over partial uses of S * M
    int need = 0;
    const bool q8 = c.wtype == FM_W_Q8_0;
    auto use = [&](int M, int K) { need = std::max(need, (q8 ? pick_split_ws(ws_groups(M), K) : pick_split(M, K)) * M); };
    const int D = c.dim, Ht = c.target_dim;
    if (c.variant == FM_VARIANT_FLOWMAP) {
        use(D, c.n_taps * Ht); use(D, Ht); use(D, D); use(D, c.ffn);
    } else if (c.variant == FM_VARIANT_KVINJECT) {
        use(D, c.n_taps * Ht); use(D, Ht); use(D, D); use(D, c.ffn);
    } else {
        use(D, 2 * D); use(D, c.heads * c.head_dim); use(D, c.ffn);
    }
    return need;
}

Plan make_plan(const fm_config& c) {
    Plan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    const int D = c.dim;
    const bool fmv = c.variant == FM_VARIANT_FLOWMAP;
    const int RB = fmv ? FM_BATCH * TMAX : TMAX;   // rows of the block buffers (flow-map: two batched requests)
    p.best_rows = RB;
    p.best = take((size_t)RB * sizeof(unsigned long long));
    p.mcut = take(c.variant == FM_VARIANT_KVINJECT ? 4 : 0);   // the Markov decode's pruning cut (zero between calls)
    p.zeros_bytes = (size_t)std::max({kmax_frag(c), 2 * c.dim, c.target_dim, 256}) * 4;
    p.zeros = take(p.zeros_bytes);
    p.rope_dims = c.rope == FM_ROPE_NEOX ? c.rope_dims : c.head_dim;
    p.rope_rows = c.max_ctx + c.block + 2;
    p.rope = take(c.rope == FM_ROPE_NONE ? 0 : (size_t)p.rope_rows * p.rope_dims * 4);
    const size_t fragK = (size_t)kmax_frag(c) * 64;   // 2 KB per 32 k, per block of 16 rows
    p.fragA = take(fragK);
    p.fragH = take(fragK * (RB / TMAX));
    p.fragO = take(fragK * (RB / TMAX));
    p.fragU = take(fragK * (RB / TMAX));
    p.x = take((size_t)RB * D * 4);
    p.part_floats = (size_t)RB * part_need(c);
    p.part = take(p.part_floats * 4);
    int qkvw = 3 * D;
    if (c.variant == FM_VARIANT_MTP) qkvw = c.heads * 2 * c.head_dim + 2 * c.kv_heads * c.head_dim;
    p.qkv_floats = (size_t)QKV_SLABS * RB * qkvw;
    p.qkv = take(p.qkv_floats * 4);
    const int Lmax = c.max_ctx + c.block + 1;
    p.nchunk_max = (Lmax + 15) / 16;
    p.attnp_bytes = (size_t)c.heads * p.nchunk_max * TMAX * (c.head_dim + 2) * 4;
    p.attnp = take(p.attnp_bytes);
    p.stage = take((size_t)2 * c.layers * TMAX * D * 4);
    p.h0 = take((size_t)D * 4);
    p.colR = 64;
    p.colsc = take(c.variant == FM_VARIANT_FLOWMAP ? (size_t)p.colR * c.target_dim * 4 : 0);
    p.cmean = take((size_t)c.target_dim * 4);
    p.hc = take((size_t)TMAX * D * 4);
    const bool prefill = c.variant != FM_VARIANT_MTP;
    // prefill context rows; small prefills split the context projection's k-range, whose partial slabs need
    // up to PF_SPLIT_ROWS rows
    p.pctx_rows = std::max(c.max_ctx, PF_SPLIT_ROWS);
    p.pctx = take(prefill ? (size_t)p.pctx_rows * D * 4 : 0);
    p.pctxn = take(prefill ? (size_t)(c.variant == FM_VARIANT_KVINJECT ? c.layers : 1) * c.max_ctx * D * 2 : 0);
    // f16 copies of the prefill weights (the context projection, then K and V of every layer), made at create, and
    // of the taps of one append: the 256-tile prefill GEMM streams f16 operands straight into LDS
    const size_t KT = (size_t)c.n_taps * c.target_dim;
    p.w16 = take(prefill ? (KT * D + 2ull * c.layers * D * D) * 2 : 0);
    p.taps16 = take(prefill ? (size_t)c.max_ctx * KT * 2 : 0);
    // the prefill K epilogue's copy of the RoPE table (flow-map): each lane's cos / sin as two 16-byte loads
    p.rope_pf = take(c.variant == FM_VARIANT_FLOWMAP ? (size_t)p.rope_rows * p.rope_dims * 4 : 0);
    p.qout = take(c.variant == FM_VARIANT_MTP ? (size_t)TMAX * c.heads * c.head_dim * 4 : 0);
    // the flow-map anchor path's own buffers (its partials, the anchor row and the slot row as fragments)
    p.apart = take(fmv ? p.part_floats * 4 : 0);
    p.afrag = take(fmv ? (size_t)c.target_dim * 64 : 0);
    p.cfrag = take(fmv ? (size_t)c.dim * 64 : 0);
    // MTP chained passes: the embedding row of the previous draft token
    p.echain = take(c.variant == FM_VARIANT_MTP ? (size_t)c.dim * 4 : 0);
    // every Q8_0 matrix in the MFMA operand layout its kernels stream (codes, then scales, per matrix), copied at
    // create
    size_t q8b = 0;
    for (const Q8Mat& m : q8_mats(c)) q8b += align256((size_t)m.M * m.K) + align256((size_t)m.M * (m.K / 32) * 2);
    p.q8t = take(q8b);
    // the MTP head's RMSNorm folds: sums of squares per 512-column slice, [2 segments][16 rows][slices]
    p.ssq = take(c.variant == FM_VARIANT_MTP ? (size_t)2 * 16 * ((c.dim + 511) / 512) * 4 : 0);
    // KV-injection: the normed backbone rows of the last draft (the confidence head's input) and the base logits
    // of the Markov decode
    const bool kvi = c.variant == FM_VARIANT_KVINJECT;
    p.blockn = take(kvi ? (size_t)TMAX * c.dim * 4 : 0);
    p.zbase = take(kvi ? (size_t)c.block * c.vocab * 4 : 0);
    p.tcond = take(fmv ? (size_t)3 * TC_MAX_DIM * 4 : 0);   // time conditioning: cond, then the two hidden layers
    p.qkv0 = take(fmv ? (size_t)TMAX * 3 * c.dim * 4 : 0);   // layer 0's q | k | v of the zero-noise slot rows
    p.x1 = take(fmv ? (size_t)TMAX * c.dim * 4 : 0);          // layer 0's residual after its self-attention
    p.q0c = take(fmv ? (size_t)QKV_SLABS * TMAX * c.dim * 4 : 0);   // layer 0's cross-attention q (split-K slabs)
    p.rscale = take(prefill ? (size_t)c.max_ctx * 4 : 0);   // the power-of-two scale of each f16 tap row of an append
    // the handle's own modulation table (copied from the caller's at create, rewritten by time conditioning): the
    // layer-0 projections cached at create follow this table, so no other handle can change it under them
    p.modc = take(fmv ? (size_t)(3 * c.layers + 1) * 3 * c.dim * 4 : 0);
    // the LayerNorm fold of the flow-map draft: (mean, M2) of each 16-column tile of the residual rows (written by
    // each residual update, read by the next product), c1 / c2 of every product that takes a LayerNorm-modulated
    // row (layer l: q, k, v, cross q, fc1; then the head), and the fragments of the modulation rows they come from
    // (the KV-injection draft folds its RMSNorms the same way: statistics and arrival counters only)
    p.lnstats = take(fmv || kvi ? (size_t)(c.dim / 16) * FM_BATCH * TMAX * 8 : 0);
    p.c12 = take(fmv ? c12_floats(c) * 4 : 0);
    p.lnfrag = take(fmv ? (size_t)(3 * c.layers + 1) * c.dim * 64 : 0);
    // arrival counters: a split residual update's per tile, then the self-attention tail's per head
    p.rtick = take(fmv || kvi ? (size_t)(RTICK_MAX + SATICK_MAX) * 4 : 0);
    // the persistent draft kernel: its arguments and per-layer table (device copies), its barrier counters and its
    // activation arena (sized for the most work-groups it may run with)
    const bool pk = draft_supported(c);
    p.dargs = take(pk ? sizeof(DraftArgs) : 0);
    p.dlayers = take(pk ? (size_t)c.layers * sizeof(DraftLayer) : 0);
    p.dsync = take(pk ? (size_t)DR_SYNC_WORDS * 4 : 0);
    p.arena = take(pk ? draft_layout(c, DR_MAX_WG).total : 0);
    p.total = off;
    return p;
}

fm_status validate_config(const fm_config* c) {
    if (!c) return fail(FM_E_INVALID, "null config");
    if (c->variant < 0 || c->variant > 2) return fail(FM_E_INVALID, "unknown variant %d", c->variant);
    if (c->dim <= 0 || c->heads <= 0 || c->head_dim <= 0 || c->layers <= 0 || c->ffn <= 0 || c->block <= 0 ||
        c->target_dim <= 0 || c->vocab <= 0 || c->max_ctx <= 0 || c->kv_heads <= 0)
        return fail(FM_E_INVALID, "non-positive size in config");
    if (c->block > TMAX) return fail(FM_E_INVALID, "block %d exceeds %d rows", c->block, TMAX);
    if (c->layers > 16) return fail(FM_E_INVALID, "more than 16 layers");
    if (c->heads % c->kv_heads) return fail(FM_E_INVALID, "heads %% kv_heads != 0");
    if (c->variant != FM_VARIANT_MTP && c->dim != c->heads * c->head_dim)
        return fail(FM_E_INVALID, "dim %d != heads * head_dim", c->dim);
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
        return fail(FM_E_UNSUPPORTED, "head_dim %d (64, 128 or 256 supported)", c->head_dim);
    if (c->dim % 256 || c->target_dim % 256 || c->ffn % 256)
        return fail(FM_E_INVALID, "dim, target_dim and ffn must be multiples of 256");
    if (c->vocab % 16) return fail(FM_E_INVALID, "vocab must be a multiple of 16");
    if (c->target_dim % 512)   // the lm_head kernel walks its rows in pairs of 256-column chunks
        return fail(FM_E_UNSUPPORTED, "target_dim %d: the lm_head takes rows of a multiple of 512", c->target_dim);
    if (c->kv_dtype == FM_KV_F32 && c->head_dim != 128 && c->head_dim != 256)   // the f32-cache attention kernel
        return fail(FM_E_UNSUPPORTED, "head_dim %d with an f32 cache (128 or 256 supported)", c->head_dim);
    if (c->dim > 8 * 256 * 3) return fail(FM_E_UNSUPPORTED, "dim too large for the row kernels");
    switch (c->variant) {
    case FM_VARIANT_FLOWMAP:
        if (c->rope != FM_ROPE_INTERLEAVED || c->mlp != FM_MLP_GELU_ERF || c->wtype != FM_W_BF16 ||
            c->kv_dtype != FM_KV_F16 || c->head_dim > 128)
            return fail(FM_E_UNSUPPORTED, "flow-map needs interleaved RoPE, exact GELU, bf16, f16 cache, hd <= 128");
        if ((c->n_taps * c->target_dim) % 128) return fail(FM_E_INVALID, "tap width must be a multiple of 128");
        if (c->n_taps * c->target_dim > TAPS_MAX_WIDTH)
            return fail(FM_E_UNSUPPORTED, "tap width %d > %d", c->n_taps * c->target_dim, TAPS_MAX_WIDTH);
        if (c->max_ctx % 32) return fail(FM_E_INVALID, "an f16 cache needs max_ctx %% 32 == 0 (V is tiled by 32)");
        if (c->kv_heads != c->heads) return fail(FM_E_UNSUPPORTED, "the flow-map drafter has one K/V head per head");
        if (c->dim > 16 * LN_MAX_TILES)   // the LayerNorm fold's statistics: at most LN_MAX_TILES tiles per row
            return fail(FM_E_UNSUPPORTED, "flow-map dim %d > %d", c->dim, 16 * LN_MAX_TILES);
        break;
    case FM_VARIANT_KVINJECT:
        if (c->rope != FM_ROPE_NONE || c->mlp != FM_MLP_GEGLU_TANH || c->wtype != FM_W_BF16 ||
            c->kv_dtype != FM_KV_F32 || c->head_dim > 128)
            return fail(FM_E_UNSUPPORTED, "KV-inject needs no RoPE, tanh GeGLU, bf16, f32 cache, hd <= 128");
        if ((c->n_taps * c->target_dim) % 128) return fail(FM_E_INVALID, "tap width must be a multiple of 128");
        if (c->n_taps * c->target_dim > TAPS_MAX_WIDTH)
            return fail(FM_E_UNSUPPORTED, "tap width %d > %d", c->n_taps * c->target_dim, TAPS_MAX_WIDTH);
        if (c->kv_heads != c->heads) return fail(FM_E_UNSUPPORTED, "KV-inject attends with every head's own K/V");
        if (c->dim > 16 * LN_MAX_TILES)   // the RMSNorm fold's statistics: at most LN_MAX_TILES tiles per row
            return fail(FM_E_UNSUPPORTED, "KV-inject dim %d > %d", c->dim, 16 * LN_MAX_TILES);
        break;
    case FM_VARIANT_MTP:
        if (c->rope != FM_ROPE_NEOX || c->mlp != FM_MLP_SWIGLU || c->wtype != FM_W_Q8_0 || c->kv_dtype != FM_KV_F32)
            return fail(FM_E_UNSUPPORTED, "MTP needs NEOX RoPE, SwiGLU, Q8_0, f32 cache");
        if (c->head_dim != 256) return fail(FM_E_UNSUPPORTED, "MTP head_dim %d (256 supported)", c->head_dim);
        if (c->rope_dims <= 0 || c->rope_dims > c->head_dim || c->rope_dims % 2)
            return fail(FM_E_INVALID, "rope_dims");
        if (c->target_dim != c->dim) return fail(FM_E_INVALID, "MTP target_dim must equal dim");
        if ((c->heads * c->head_dim) % 256 || (c->kv_heads * c->head_dim) % 16)   // o_proj's k-range: whole chunks
            return fail(FM_E_INVALID, "MTP head widths");
        break;
    }
    return FM_OK;
}

}  // namespace

// ── handle ──────────────────────────────────────────────────────────────────────────────────────
struct fm_drafter {
    fm_config c;
    Plan p;
    std::map<std::string, const void*> w;
    uint8_t* ws;
    uint8_t* kv;
    int length;
    int draft_path = 0;       // 0 (automatic) and 1: one launch per phase, 2: the persistent kernel
    bool draft_ready = false; // the persistent kernel is set up for this handle (shape supported, grid resident)
    int G = 0;                // its work-groups
    DraftArgs dh{};           // host copies of its device-resident arguments (the sources of their uploads)
    DraftLayer dl[DR_MAX_LAYERS]{};
    // fm_profile_draft: while `rec` is set, every skinny launch's arguments are appended to it (and launched)
    std::vector<std::pair<SkinnyArgs, int>>* rec = nullptr;
    // the jump (s, t, time_dim, cond_dim, time_scale) the modulation table was last conditioned on (tc_set), else
    // the table is the one given at create: handles with the same weights and the same key hold the same table
    float tc_key[5] = {};
    bool tc_set = false;
    hipEvent_t ev[4] = {};
    ~fm_drafter() {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
    }

    template <class T> T* at(size_t off) const { return (T*)(ws + off); }
    const void* W(const std::string& n) const { auto it = w.find(n); return it == w.end() ? nullptr : it->second; }
    const uint16_t* B(const std::string& n) const { return (const uint16_t*)W(n); }
    const float* F(const std::string& n) const { return (const float*)W(n); }
    size_t kv_es() const { return c.kv_dtype == FM_KV_F16 ? 2 : 4; }
    void* kv_layer(int l, int which) const {   // which 0: K, 1: V
        return kv + ((size_t)(2 * l + which) * c.max_ctx * c.dim) * kv_es();
    }
    size_t tap_width() const { return (size_t)c.n_taps * c.target_dim; }
    // f16 copies of the prefill weights: the context projection [dim][n_taps * target_dim], then per layer K, V [dim][dim]
    const uint16_t* w16_ctx() const { return at<uint16_t>(p.w16); }
    const uint16_t* w16_kv(int l, int which) const {
        return at<uint16_t>(p.w16) + tap_width() * c.dim + (size_t)(2 * l + which) * c.dim * c.dim;
    }
};

namespace {

std::vector<std::string> required_names(const fm_config& c) {
    std::vector<std::string> n;
    char b[128];
    if (c.variant == FM_VARIANT_FLOWMAP) {
        n = {"fc.weight", "hidden_norm.weight", "anchor_proj.weight", "anchor_proj.bias", "anchor_norm.weight",
             "state_norm.weight", "x_embed.weight", "x_embed.bias", "head.weight", "head.bias", "lm_head.weight", "mod"};
        for (int l = 0; l < c.layers; ++l) {
            for (const char* br : {"self_attn", "cross_attn"}) {
                for (const char* p : {"q_proj", "k_proj", "v_proj", "o_proj", "q_norm", "k_norm"}) {
                    snprintf(b, sizeof b, "layers.%d.%s.%s.weight", l, br, p);
                    n.push_back(b);
                }
            }
            for (const char* p : {"mlp.fc1.weight", "mlp.fc1.bias", "mlp.fc2.weight", "mlp.fc2.bias"}) {
                snprintf(b, sizeof b, "layers.%d.%s", l, p);
                n.push_back(b);
            }
        }
    } else if (c.variant == FM_VARIANT_KVINJECT) {
        n = {"W_c", "ctx_norm", "tok_proj", "block_pos", "out_norm", "out_proj", "lm_head.weight"};
        if (c.block > 1) n.push_back("mask_emb");   // [block - 1][dim]: no rows in a one-row block
        for (int i = 0; i < c.layers; ++i)
            for (const char* p : {"attn_norm", "q", "k", "v", "o", "ff_norm", "gate", "up", "down"}) {
                snprintf(b, sizeof b, "bb.%d.%s", i, p);
                n.push_back(b);
            }
    } else {
        for (const char* p : {"eh_proj", "attn_q", "attn_k", "attn_v", "attn_output", "ffn_gate", "ffn_up", "ffn_down",
                              "lm_head"}) {
            n.push_back(std::string(p) + ".q");
            n.push_back(std::string(p) + ".d");
        }
        for (const char* p : {"attn_norm", "attn_q_norm", "attn_k_norm", "post_attention_norm", "shared_head_norm",
                              "enorm", "hnorm"})
            n.push_back(p);
    }
    return n;
}

// ── skinny GEMM helper ──────────────────────────────────────────────────────────────────────────
struct SkGroupDesc {
    const void* W;
    const void* Wd;
    const void* W2;
    const void* W2d;
    const uint16_t* bias;
    const uint8_t* X;
    void* out;
    int M;
    int ld;
    const float* c12 = nullptr;   // the LayerNorm fold's c1 / c2 of this group
};

// Optional epilogue work of a skinny launch (SkinnyArgs): the LayerNorm fold of a product whose input is a
// LayerNorm-modulated row (ln_stats), or the residual update of SK_RESID.
struct SkExtra {
    const float* ln_stats = nullptr;
    int ln_tiles = 0;
    float ln_eps = 0.f;
    float* rx = nullptr;
    int rx_ld = 0;
    const float* rbase = nullptr;
    int rbase_ld = 0;
    const float* rgate = nullptr;
    const float* ryscale = nullptr;
    float* rstats = nullptr;
    float* rdebug = nullptr;
    int ln_rms = 0;                  // the RMSNorm fold (no c1 / c2)
    const uint16_t* ryw = nullptr;   // SK_RESID: fragments of x w (the next RMSNorm's weight) instead of x (1 + s)
    SelfAttnArgs sa{};   // q | k | v with the self-attention tail (sa.qkv set)
    // Q8_0: the RMSNorm fold (SkinnyArgs.rms_*)
    const float* rms_ssq = nullptr;
    int rms_nsl = 0;
    int rms_seg = 0;
    float rms_inv = 0.f;
    float rms_eps = 0.f;
};

// Enqueue one skinny launch. For SK_PARTIAL the k-split is chosen here (returned through S_out); every other mode
// runs with S = 1 (the whole k-range in one work-group).
// Partial slabs go to the groups' own outputs; by default they are the shared partial buffer with slabs TMAX * M
// apart (M of the first group). A caller writing elsewhere passes the slab stride and the capacity (floats) there.
// nb = 2: two blocks of 16 activation rows (rows 16 b + t of the outputs; fragments of block b at X + b * K * 64),
// each weight tile multiplied against both; the k-split then keeps k-steps per wave a multiple of 4.
fm_status skinny(const fm_drafter* d, const std::vector<SkGroupDesc>& gs, int K, int T, int mode, int S_force,
                 int* S_out, hipStream_t st, long long pstride = 0, size_t cap_floats = 0, int nb = 1,
                 const SkExtra* ex = nullptr) {
    if (gs.empty() || gs.size() > SK_MAX_GROUPS) return fail(FM_E_INVALID, "skinny: %zu groups", gs.size());
    if (K % 128) return fail(FM_E_INVALID, "skinny: K %d not a multiple of 128", K);
    SkinnyArgs a{};
    const bool q8 = d->c.wtype == FM_W_Q8_0;
    const bool glu = mode == SK_FRAG_GEGLU || mode == SK_FRAG_SWIGLU;
    int tiles_total = 0, groups_total = 0;
    for (auto& g : gs) {
        tiles_total += g.M / 16;
        groups_total += ws_groups(g.M, glu);
    }
    int S = 1;
    if (q8) {   // the tile-owning variant: whole 256-column chunks per split
        if (nb != 1 || T > TMAX) return fail(FM_E_UNSUPPORTED, "skinny: Q8_0 takes one block of <= %d rows", TMAX);
        if (K % 256) return fail(FM_E_UNSUPPORTED, "skinny: Q8_0 needs K %% 256 == 0 (K %d)", K);
        if (mode == SK_PARTIAL) S = S_force > 0 ? S_force : pick_split_ws(groups_total, K);
        if (S < 1 || (K / 256) % S) return fail(FM_E_UNSUPPORTED, "skinny: no Q8_0 k-split %d for K %d", S, K);
    } else if (mode == SK_PARTIAL) {
        S = S_force > 0 ? S_force : pick_split(tiles_total * 16, K);
    } else if (mode == SK_RESID && S_force > 0) {
        S = S_force;   // the last split of each tile to arrive finishes it
    }
    if (q8) {
    } else if (nb == 2) {
        if (T != 16 || d->c.wtype != FM_W_BF16) return fail(FM_E_UNSUPPORTED, "skinny: two row blocks need bf16, T 16");
        while (S > 1 && ((K / 128) % S || (K / 128 / S) % 4)) --S;
        if ((K / 128 / S) % 4) return fail(FM_E_UNSUPPORTED, "skinny: two row blocks need K %% 512 == 0 (K %d)", K);
    } else if (nb != 1) {
        return fail(FM_E_INVALID, "skinny: %d row blocks", nb);
    }
    if (!q8 && (S < 1 || (K / 128) % S || !kw_ok(K / 128 / S)))
        return fail(FM_E_UNSUPPORTED, "skinny: no supported k-split for K %d (S %d)", K, S);
    a.ngroups = (int)gs.size();
    a.K = K;
    a.T = T;
    a.S = S;
    a.KW = q8 ? 0 : K / 128 / S;
    a.mode = mode;
    a.nb = nb;
    a.zeros = d->at<float>(d->p.zeros);
    if (ex) {
        a.ln_stats = ex->ln_stats;
        a.ln_tiles = ex->ln_tiles;
        a.ln_inv = ex->ln_tiles > 0 ? 1.f / (float)ex->ln_tiles : 0.f;
        a.ln_eps = ex->ln_eps;
        a.rx = ex->rx;
        a.rx_ld = ex->rx_ld;
        a.rbase = ex->rbase;
        a.rbase_ld = ex->rbase_ld;
        a.rgate = ex->rgate;
        a.ryscale = ex->ryscale;
        a.ryw = ex->ryw;
        a.ln_rms = ex->ln_rms;
        a.rstats = ex->rstats;
        a.rdebug = ex->rdebug;
        a.sa = ex->sa;
        a.rms_ssq = ex->rms_ssq;
        a.rms_nsl = ex->rms_nsl;
        a.rms_seg = ex->rms_seg;
        a.rms_inv = ex->rms_inv;
        a.rms_eps = ex->rms_eps;
        if (a.sa.qkv) a.satick = d->at<uint32_t>(d->p.rtick) + RTICK_MAX;
    }
    if (mode == SK_RESID && !ex) return fail(FM_E_INVALID, "skinny: a residual update needs its operands");
    if (mode == SK_RESID && S > 1) {
        a.rpart = d->at<float>(d->p.part);
        a.rtick = d->at<uint32_t>(d->p.rtick);
        a.part_stride = (long long)TMAX * nb * gs[0].M;
        if ((size_t)S * a.part_stride > d->p.part_floats) return fail(FM_E_INVALID, "skinny: partial buffer too small");
        if (gs[0].M / 16 > RTICK_MAX) return fail(FM_E_INVALID, "skinny: %d tiles > %d counters", gs[0].M / 16, RTICK_MAX);
    }
    int begin = 0;
    for (size_t i = 0; i < gs.size(); ++i) {
        const auto& g = gs[i];
        if (g.M % 16) return fail(FM_E_INVALID, "skinny: M %d not a multiple of 16", g.M);
        a.g[i] = SkinnyGroup{g.W, g.Wd, g.W2, g.W2d, g.bias, g.X, g.out, g.M, g.ld, begin, 0, g.c12};
        begin += (q8 ? ws_groups(g.M, glu) : g.M / 16) * S;   // work-groups of this group
    }
    if (mode == SK_PARTIAL) {
        a.part_stride = pstride > 0 ? pstride : (long long)TMAX * nb * gs[0].M;
        const size_t cap = cap_floats > 0 ? cap_floats : d->p.part_floats;
        if ((size_t)S * a.part_stride > cap) return fail(FM_E_INVALID, "skinny: partial buffer too small");
    }
    if (S_out) *S_out = S;
    if (d->rec) d->rec->push_back({a, begin});
    HIPCHK(launch_skinny(a, d->c.wtype == FM_W_Q8_0 ? SKW_Q8_0 : SKW_BF16, begin, st));
    return FM_OK;
}

RowArgs rows_base(const fm_drafter* d, int D, int T) {
    RowArgs r{};
    r.D = D;
    r.T = T;
    r.zeros = d->at<float>(d->p.zeros);
    return r;
}

fm_status rows(const RowArgs& r, hipStream_t st) {
    if (r.S > 8) return fail(FM_E_UNSUPPORTED, "row kernel: more than 8 partial slabs");
    HIPCHK(launch_rows(r, st));
    return FM_OK;
}

#define CHK(x)                        \
    do {                              \
        fm_status s_ = (x);           \
        if (s_ != FM_OK) return s_;   \
    } while (0)

// Attention of nq query rows over cache rows [key_lo, key_hi) (+ nx extra f32 rows), merged into o fragments.
fm_status attend(fm_drafter* d, const QPrep& qp, int nq, int layer_kv, int key_lo, int key_hi, const float* kx,
                 const float* vx, int nx, int x_ld, int causal_base, float scale, const float* gate, int gate_ld,
                 int gate_hs, uint8_t* o_frag, hipStream_t st, int o_row0 = 0) {
    const auto& c = d->c;
    AttnArgs a{};
    a.qp = qp;
    a.qp.zeros = d->at<float>(d->p.zeros);
    a.nq = nq;
    a.kv_dtype = c.kv_dtype;
    if (c.variant == FM_VARIANT_MTP) {
        const size_t w = (size_t)c.kv_heads * c.head_dim;
        a.kc = d->kv;
        a.vc = (const float*)d->kv + (size_t)c.max_ctx * w;
        a.kv_ld = (int)w;
    } else {
        a.kc = d->kv_layer(layer_kv, 0);
        a.vc = d->kv_layer(layer_kv, 1);
        a.kv_ld = c.dim;
        a.vt_ld = c.dim;   // f16 V is tiled [pos / 32][dim][32]
    }
    a.key_lo = key_lo;
    a.key_hi = key_hi;
    a.kx = kx;
    a.vx = vx;
    a.nx = nx;
    a.x_ld = x_ld;
    a.heads = c.heads;
    a.kv_heads = c.kv_heads;
    a.hd = c.head_dim;
    a.causal_base = causal_base;
    a.scale = scale;
    const int ntot = key_hi - key_lo + nx;
    a.chunk = attn_chunk_size(c.head_dim, c.kv_dtype, ntot, c.heads);
    const int tc = (ntot + a.chunk - 1) / a.chunk;
    if (c.kv_dtype == FM_KV_F16) {
        // the fewest 32-key steps per wave that keep the launch within one round of work-groups (one per CU): a
        // second partial round costs more than the longer runs (measured at L = 8193: 272 work-groups 791 us per
        // draft, 208 work-groups 759 us); more runs also make the merge read more partials
        a.cpw = 1;
        while (a.cpw < tc && c.heads * (((tc + a.cpw - 1) / a.cpw + 3) / 4) > TARGET_WGS) ++a.cpw;
        a.nchunks = ((tc + a.cpw - 1) / a.cpw + 3) / 4 * 4;
    } else {
        a.cpw = 1;
        a.nchunks = tc;
    }
    if ((size_t)c.heads * a.nchunks * TMAX * (c.head_dim + 2) * 4 > d->p.attnp_bytes)
        return fail(FM_E_INVALID, "attention partial buffer too small");
    a.part = d->at<float>(d->p.attnp);
    HIPCHK(launch_attn_split(a, st));
    MergeArgs m{};
    m.part = a.part;
    m.heads = c.heads;
    m.nchunks = a.nchunks;
    m.nq = nq;
    m.hd = c.head_dim;
    m.gate = gate;
    m.gate_ld = gate_ld;
    m.gate_hs = gate_hs;
    m.o_frag = o_frag;
    m.row0 = o_row0;
    HIPCHK(launch_attn_merge(m, st));
    return FM_OK;
}

// ── flow-map ────────────────────────────────────────────────────────────────────────────────────
// A operand of the context projection: the taps of the append as f16 rows, each scaled by a power of two that brings
// its largest magnitude into [2^14, 2^15) (launch_taps_f16); the scale is undone on the f32 output rows
// (d->p.rscale), so f16's range does not limit the taps.
// The context projection [n][K] x [K][D]: 128-tiles that fill less than one round of work-groups (two per CU) split
// their k-range over up to 4 work-groups per tile; the slabs go to ctx + s * n * D and the RMSNorm that follows
// sums them. Returns the slab count.
fm_status prefill_context(fm_drafter* d, const float* taps, int n, const uint16_t* w, const uint16_t* w16, float* ctx,
                          int* nslab, hipStream_t st);

fm_status prefill_taps(fm_drafter* d, const float* taps, int n, PrefillArgs& a, hipStream_t st) {
    uint16_t* t16 = d->at<uint16_t>(d->p.taps16);
    HIPCHK(launch_taps_f16(taps, n, (int)d->tap_width(), t16, d->at<float>(d->p.rscale), st));
    a.A = t16;
    return FM_OK;
}

fm_status prefill_context(fm_drafter* d, const float* taps, int n, const uint16_t* w, const uint16_t* w16, float* ctx,
                          int* nslab, hipStream_t st) {
    const int D = d->c.dim, KT = (int)d->tap_width();
    PrefillArgs a{};
    a.ngroups = 1;
    a.g[0] = PrefillGroup{nullptr, w, w16, nullptr, ctx, PF_F32, 0};
    CHK(prefill_taps(d, taps, n, a, st));
    a.rows = n;
    a.N = D;
    a.K = KT;
    a.ld = D;
    const int tile = prefill_tile(n, D, 1);
    a.m_tiles = (n + tile - 1) / tile;
    a.n_tiles = D / tile;
    const int tiles = a.m_tiles * a.n_tiles;
    int ks = 1;
    if (tile == 128)
        while (ks < 4 && 2 * ks * tiles <= PF_SPLIT_WGS && KT % (2 * ks * 32) == 0 && 2 * ks * n <= d->p.pctx_rows)
            ks *= 2;
    a.ksplit = ks;
    a.slab_stride = (long long)n * D;
    HIPCHK(launch_prefill(a, tiles * ks, st));
    *nslab = ks;
    return FM_OK;
}

std::string LW(int l, const char* s);
std::string BB(int i, const char* s);

// f16 copies of the prefill weights (bf16 -> f16 is exact down to f16's subnormal range)
fm_status prefill_weight_copies(fm_drafter* d, hipStream_t st) {
    const auto& c = d->c;
    const size_t DD = (size_t)c.dim * c.dim;
    const bool fmv = c.variant == FM_VARIANT_FLOWMAP;
    HIPCHK(launch_bf16_to_f16(d->B(fmv ? "fc.weight" : "W_c"), d->tap_width() * c.dim, (uint16_t*)d->w16_ctx(), st));
    for (int l = 0; l < c.layers; ++l)
        for (int w = 0; w < 2; ++w) {
            const std::string nm = fmv ? LW(l, w ? "cross_attn.v_proj.weight" : "cross_attn.k_proj.weight")
                                       : BB(l, w ? "v" : "k");
            HIPCHK(launch_bf16_to_f16(d->B(nm), DD, (uint16_t*)d->w16_kv(l, w), st));
        }
    return FM_OK;
}

std::string LW(int l, const char* s) {
    char b[128];
    snprintf(b, sizeof b, "layers.%d.%s", l, s);
    return b;
}

// c rows (fragments in fragH, T rows) -> every layer's K/V at rows start.. (skinny path, T <= 16). With `caches`
// (batched drafts), row t goes to the cache of handle caches[t] at its row starts[t] instead.
fm_status fm_kv_rows_small(fm_drafter* d, int T, int start, const uint8_t* cfrag, hipStream_t st,
                           fm_drafter* const* caches = nullptr, const int* starts = nullptr) {
    const auto& c = d->c;
    const int D = c.dim;
    std::vector<SkGroupDesc> gs;
    float* stage = d->at<float>(d->p.stage);
    for (int l = 0; l < c.layers; ++l) {
        gs.push_back({d->W(LW(l, "cross_attn.k_proj.weight")), nullptr, nullptr, nullptr, nullptr, cfrag,
                      stage + (size_t)(2 * l) * T * D, D, D});
        gs.push_back({d->W(LW(l, "cross_attn.v_proj.weight")), nullptr, nullptr, nullptr, nullptr, cfrag,
                      stage + (size_t)(2 * l + 1) * T * D, D, D});
    }
    // at most 12 groups per launch
    for (size_t i = 0; i < gs.size(); i += SK_MAX_GROUPS) {
        std::vector<SkGroupDesc> sub(gs.begin() + i, gs.begin() + std::min(gs.size(), i + SK_MAX_GROUPS));
        CHK(skinny(d, sub, D, T, SK_F32, 0, nullptr, st));
    }
    KVFinalArgs k{};
    k.stage = stage;
    k.n = T;
    k.D = D;
    k.heads = c.heads;
    k.hd = c.head_dim;
    k.layers = c.layers;
    for (int l = 0; l < c.layers; ++l) k.knorm[l] = d->B(LW(l, "cross_attn.k_norm.weight"));
    k.eps = c.qk_eps;
    k.rope_tab = d->at<float>(d->p.rope);
    k.rope_dims = d->p.rope_dims;
    k.start = start;
    k.cache = d->kv;
    k.max_ctx = c.max_ctx;
    k.kv_dtype = c.kv_dtype;
    k.zeros = d->at<float>(d->p.zeros);
    if (!caches) {
        HIPCHK(launch_kv_final(k, st));
        return FM_OK;
    }
    for (int t = 0; t < T; ++t) {   // one row into each request's own cache
        KVFinalArgs kt = k;
        kt.n = 1;
        kt.stage_n = T;
        kt.stage_t0 = t;
        kt.start = starts[t];
        kt.cache = caches[t]->kv;
        kt.max_ctx = caches[t]->c.max_ctx;
        HIPCHK(launch_kv_final(kt, st));
    }
    return FM_OK;
}

fm_status flowmap_append(fm_drafter* d, const float* taps, int n, int start, hipStream_t st) {
    const auto& c = d->c;
    const int D = c.dim, KT = c.n_taps * c.target_dim;
    if (n <= TMAX) {
        HIPCHK(launch_f32_to_frag(taps, KT, n, KT, d->at<uint8_t>(d->p.fragA), st));
        int S = 0;
        float* part = d->at<float>(d->p.part);
        CHK(skinny(d, {{d->W("fc.weight"), nullptr, nullptr, nullptr, nullptr, d->at<uint8_t>(d->p.fragA), part, D, D}},
                   KT, n, SK_PARTIAL, 0, &S, st));
        RowArgs r = rows_base(d, D, n);
        r.part = part;
        r.S = S;
        r.part_stride = (long long)TMAX * D;
        r.norm = ROW_RMS;
        r.w_bf16 = d->B("hidden_norm.weight");
        r.eps = c.rms_eps;
        r.frag_out = d->at<uint8_t>(d->p.fragH);
        CHK(rows(r, st));
        return fm_kv_rows_small(d, n, start, d->at<uint8_t>(d->p.fragH), st);
    }
    // prefill: MFMA GEMMs
    float* ctx = d->at<float>(d->p.pctx);
    uint16_t* ctxn = d->at<uint16_t>(d->p.pctxn);
    int nslab = 1;
    CHK(prefill_context(d, taps, n, d->B("fc.weight"), d->w16_ctx(), ctx, &nslab, st));
    HIPCHK(launch_rms_f16(ctx, n, D, d->B("hidden_norm.weight"), c.rms_eps, ctxn, nslab, (long long)n * D,
                          d->at<float>(d->p.rscale), st));
    for (int l0 = 0; l0 < c.layers; l0 += PF_MAX_GROUPS / 2) {
        PrefillArgs a{};
        const int nl = std::min(c.layers - l0, PF_MAX_GROUPS / 2);
        const int tile = prefill_tile(n, D, 2 * nl);
        const int mt = (n + tile - 1) / tile;
        const int per = mt * (D / tile);
        for (int j = 0; j < nl; ++j) {
            const int l = l0 + j;
            a.g[2 * j] = PrefillGroup{nullptr, d->B(LW(l, "cross_attn.k_proj.weight")), d->w16_kv(l, 0),
                                      d->B(LW(l, "cross_attn.k_norm.weight")), d->kv_layer(l, 0), PF_CACHE_K,
                                      (2 * j) * per};
            a.g[2 * j + 1] = PrefillGroup{nullptr, d->B(LW(l, "cross_attn.v_proj.weight")), d->w16_kv(l, 1), nullptr,
                                          d->kv_layer(l, 1), PF_CACHE_VT, (2 * j + 1) * per};
        }
        a.ngroups = 2 * nl;
        a.A = ctxn;
        a.rows = n;
        a.N = D;
        a.K = D;
        a.ld = D;
        a.hd = c.head_dim;
        a.eps = c.qk_eps;
        a.rope_tab = d->at<float>(d->p.rope);
        a.rope_pf = d->at<float>(d->p.rope_pf);
        a.rope_dims = d->p.rope_dims;
        a.start = start;
        a.kv_dtype = c.kv_dtype;
        a.vt_ld = D;
        a.m_tiles = mt;
        a.n_tiles = D / tile;
        HIPCHK(launch_prefill(a, 2 * nl * per, st));
    }
    return FM_OK;
}

// B (1 or 2) flow-map drafts in one pass: request b's anchor, position and context cache are handle ds[b]'s; its 16
// slots are rows 16 b .. 16 b + 15 of the pass (of hidden_out too). Every projection streams its weights once for
// all rows (two blocks of 16 activation rows against each weight tile); self-attention runs within each request's
// rows, cross-attention over each request's own cache, and each anchor slot goes into its own request's cache. The
// handles share the weights and the modulation table (checked by the caller), so the row kernels and layer 0's
// cached rows serve every request.
fm_status flowmap_draft_batch(fm_drafter* const* ds, int B, const fm_block_args* const* bas, float* hidden_out,
                              hipStream_t st) {
    fm_drafter* d = ds[0];
    const auto& c = d->c;
    const int D = c.dim, T = c.block, Ht = c.target_dim, H = c.heads, hd = c.head_dim;
    float* x = d->at<float>(d->p.x);
    const float* mod = d->at<float>(d->p.modc);
    uint8_t* fragH = d->at<uint8_t>(d->p.fragH);
    uint8_t* fragO = d->at<uint8_t>(d->p.fragO);
    uint8_t* fragU = d->at<uint8_t>(d->p.fragU);
    float* qkv = d->at<float>(d->p.qkv);
    const float* rope = d->at<float>(d->p.rope);
    const int Sq = pick_qsplit(D);
    float* debug = B == 1 ? bas[0]->debug_layers : nullptr;

    // anchor slots: anchor_norm(anchor_proj(E[anchor_b])) as row b, through every layer's k/v path into request b's
    // cache at its pos, on the caller's stream before layer 0. (Beside layer 0 on a second stream it was 37 us slower
    // per step: its 1,536-work-group K/V projections took the CUs layer 0's latency-bound kernels needed, and the
    // join cost another ~9 us.)
    {
        uint8_t* afrag = d->at<uint8_t>(d->p.afrag);
        uint8_t* cfrag = d->at<uint8_t>(d->p.cfrag);
        float* apart = d->at<float>(d->p.apart);
        for (int b = 0; b < B; ++b)
            HIPCHK(launch_gather_frag(d->B("lm_head.weight"), c.vocab, Ht, bas[b]->anchor, afrag, st, b));
        int Sa = 0;
        CHK(skinny(d, {{d->W("anchor_proj.weight"), nullptr, nullptr, nullptr, nullptr, afrag, apart, D, D}}, Ht, B,
                   SK_PARTIAL, 0, &Sa, st));
        RowArgs r = rows_base(d, D, B);
        r.part = apart;
        r.S = Sa;
        r.part_stride = (long long)TMAX * D;
        r.bias = d->B("anchor_proj.bias");
        r.norm = ROW_RMS;
        r.w_bf16 = d->B("anchor_norm.weight");
        r.eps = c.rms_eps;
        r.frag_out = cfrag;
        CHK(rows(r, st));
        if (B == 1) {
            CHK(fm_kv_rows_small(d, 1, bas[0]->pos, cfrag, st));
        } else {
            int starts[FM_BATCH];
            for (int b = 0; b < B; ++b) starts[b] = bas[b]->pos;
            CHK(fm_kv_rows_small(d, B, 0, cfrag, st, ds, starts));
        }
    }
    // The layers, with every LayerNorm folded into the product that takes its row (SkinnyArgs): each residual
    // update (o_proj, cross o_proj, fc2: unsplit, SK_RESID) writes x, the fragments of y = x (1 + scale) for the next
    // product and x's per-tile statistics; the next product (q | k | v, cross q, fc1, the head) applies
    // rstd (acc - mean c1) + c2. No row kernel runs between the layers.
    float2* stats = d->at<float2>(d->p.lnstats);
    const float* c12 = d->at<float>(d->p.c12);
    auto fold = [&]() {
        SkExtra e;
        e.ln_stats = (const float*)stats;
        e.ln_tiles = D / 16;
        e.ln_eps = c.ln_eps;
        return e;
    };
    auto resid = [&](const float* base, int base_ld, const float* gate, const float* next_mod, float* dbg) {
        SkExtra e;
        e.rx = x;
        e.rx_ld = D;
        e.rbase = base;
        e.rbase_ld = base_ld;
        e.rgate = gate;
        e.ryscale = next_mod;   // the next LayerNorm's scale row
        e.rstats = (float*)stats;
        e.rdebug = dbg;
        return e;
    };
    auto C12 = [&](int l, int which) { return c12 + c12_off(c, l, which); };
    int Sqb = Sq;             // split count of the cross q of layers >= 1 (two row blocks may take fewer)
    for (int l = 0; l < c.layers; ++l) {
        const float* m_sa = mod + (size_t)(3 * l) * 3 * D;
        const float* m_ca = mod + (size_t)(3 * l + 1) * 3 * D;
        const float* m_ml = mod + (size_t)(3 * l + 2) * 3 * D;
        // q | k | v of the self-attention LN-mod (x and its fragments from the previous layer's fc2); layer 0's are
        // the same for every draft (flowmap_layer0)
        if (l > 0) {
            SkExtra ef = fold();   // with the self-attention tail: the head's last q | k | v tile runs it
            ef.sa.qkv = qkv;
            ef.sa.T = T;
            ef.sa.D = D;
            ef.sa.heads = H;
            ef.sa.hd = hd;
            ef.sa.qn = d->B(LW(l, "self_attn.q_norm.weight"));
            ef.sa.kn = d->B(LW(l, "self_attn.k_norm.weight"));
            ef.sa.eps = c.qk_eps;
            ef.sa.rope_tab = rope;
            ef.sa.pos_base = bas[0]->pos + 1;
            ef.sa.pos_base1 = bas[B - 1]->pos + 1;
            ef.sa.nb = B;
            ef.sa.scale = 1.f / sqrtf((float)hd);
            ef.sa.o_frag = fragO;
            if (H > SATICK_MAX) return fail(FM_E_UNSUPPORTED, "more than %d heads", SATICK_MAX);
            std::vector<SkGroupDesc> g = {
                {d->W(LW(l, "self_attn.q_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, qkv, D, 3 * D},
                {d->W(LW(l, "self_attn.k_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, qkv + D, D, 3 * D},
                {d->W(LW(l, "self_attn.v_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, qkv + 2 * D, D,
                 3 * D}};
            for (int i = 0; i < 3; ++i) g[i].c12 = C12(l, i);
            CHK(skinny(d, g, D, T, SK_F32, 0, nullptr, st, 0, 0, B, &ef));
            // o_proj and the gated residual; fragments of the cross-attention LN-mod's x (1 + scale)
            const SkExtra er = resid(x, D, m_sa + 2 * D, m_ca, nullptr);
            CHK(skinny(d, {{d->W(LW(l, "self_attn.o_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragO, fragH, D,
                            0}},
                       D, T, SK_RESID, 0, nullptr, st, 0, 0, B, &er));
            // cross-attention q = cross q_proj(LN-mod(x)) (k-split slabs), per-head q_norm + RoPE inside the
            // attention kernel
            SkGroupDesc gq{d->W(LW(l, "cross_attn.q_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, qkv, D,
                           D};
            gq.c12 = C12(l, 3);
            const SkExtra efq = fold();
            CHK(skinny(d, {gq}, D, T, SK_PARTIAL, Sq, &Sqb, st, (long long)TMAX * B * D, d->p.qkv_floats, B, &efq));
        }
        for (int b = 0; b < B; ++b) {   // each request over its own cache rows [0, pos_b]
            QPrep qp{};
            qp.q = l == 0 ? d->at<float>(d->p.q0c) : qkv + (size_t)b * T * D;
            qp.q_ld = D;
            qp.q_hs = hd;
            qp.norm_bf16 = d->B(LW(l, "cross_attn.q_norm.weight"));
            qp.eps = c.qk_eps;
            qp.rope = 1;
            qp.rope_dims = d->p.rope_dims;
            qp.rope_tab = rope;
            qp.pos_base = bas[b]->pos + 1;
            qp.parts = l == 0 ? Sq : Sqb;
            qp.pstride = l == 0 ? (long long)TMAX * D : (long long)TMAX * B * D;
            CHK(attend(ds[b], qp, T, l, 0, bas[b]->pos + 1, nullptr, nullptr, 0, 0, -1, 1.f / sqrtf((float)hd), nullptr,
                       0, 0, fragO, st, b * T));
        }
        // cross o_proj and the gated residual (layer 0: on x1, the residual after its self-attention, the same row
        // for every slot); fragments of the MLP LN-mod's x (1 + scale)
        {
            const SkExtra er = l == 0 ? resid(d->at<float>(d->p.x1), 0, m_ca + 2 * D, m_ml, nullptr)
                                      : resid(x, D, m_ca + 2 * D, m_ml, nullptr);
            CHK(skinny(d, {{d->W(LW(l, "cross_attn.o_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragO, fragH,
                            D, 0}},
                       D, T, SK_RESID, 0, nullptr, st, 0, 0, B, &er));
        }
        // MLP: fc1 of the LN-mod + exact GELU (fused), fc2 + bias and the gated residual; fragments of the next
        // LayerNorm's x (1 + scale): the next layer's self-attention, or the final modulation
        {
            const SkExtra ef = fold();
            SkGroupDesc g1{d->W(LW(l, "mlp.fc1.weight")), nullptr, nullptr, nullptr, d->B(LW(l, "mlp.fc1.bias")), fragH,
                           fragU, c.ffn, 0};
            g1.c12 = C12(l, 4);
            CHK(skinny(d, {g1}, D, T, SK_FRAG_GELU, 0, nullptr, st, 0, 0, B, &ef));
            const float* next = l + 1 < c.layers ? mod + (size_t)(3 * (l + 1)) * 3 * D : mod + (size_t)(3 * c.layers) * 3 * D;
            const SkExtra er = resid(x, D, m_ml + 2 * D, next, debug ? debug + (size_t)l * T * D : nullptr);
            CHK(skinny(d, {{d->W(LW(l, "mlp.fc2.weight")), nullptr, nullptr, nullptr, d->B(LW(l, "mlp.fc2.bias")),
                            fragU, fragH, D, 0}},
                       c.ffn, T, SK_RESID, 2, nullptr, st, 0, 0, B, &er));
        }
    }
    // the head of the final LN-mod, + bias
    {
        const SkExtra ef = fold();
        SkGroupDesc gh{d->W("head.weight"), nullptr, nullptr, nullptr, d->B("head.bias"), fragH, hidden_out, Ht, Ht};
        gh.c12 = C12(c.layers, 0);
        CHK(skinny(d, {gh}, D, T, SK_F32, 0, nullptr, st, 0, 0, B, &ef));
    }
    return FM_OK;
}

fm_status flowmap_draft(fm_drafter* d, const fm_block_args* ba, float* hidden_out, hipStream_t st) {
    fm_drafter* ds[1] = {d};
    const fm_block_args* as[1] = {ba};
    return flowmap_draft_batch(ds, 1, as, hidden_out, st);
}

// Layer 0 of a draft starts every slot from the same row h0 with the same modulation, so its LN-mod and its q / k /
// v projections (before the head norms and RoPE, which the self-attention kernel applies at the slots' positions)
// are the same for every draft: computed here, at create and whenever the modulation table changes.
fm_status flowmap_layer0(fm_drafter* d, hipStream_t st) {
    const auto& c = d->c;
    const int D = c.dim, T = c.block;
    const float* m_sa = d->at<float>(d->p.modc);
    uint8_t* fragH = d->at<uint8_t>(d->p.fragH);
    float* q0 = d->at<float>(d->p.qkv0);
    RowArgs r = rows_base(d, D, T);
    r.init = d->at<float>(d->p.h0);
    r.norm = ROW_LN_MOD;
    r.scale = m_sa;
    r.shift = m_sa + D;
    r.eps = c.ln_eps;
    r.frag_out = fragH;
    CHK(rows(r, st));
    CHK(skinny(d,
               {{d->W(LW(0, "self_attn.q_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, q0, D, 3 * D},
                {d->W(LW(0, "self_attn.k_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, q0 + D, D, 3 * D},
                {d->W(LW(0, "self_attn.v_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH, q0 + 2 * D, D,
                 3 * D}},
               D, T, SK_F32, 0, nullptr, st));
    // Every slot's v row is the same and each query's softmax weights sum to 1, so layer 0's self-attention output
    // is v itself whatever the positions: o_proj(v), the residual x1 = h0 + gate * o_proj(v), its cross-attention
    // LN-mod and the cross-attention q projection (before its head norm and RoPE) are the same for every draft too.
    const float* m_ca = m_sa + 3 * D;
    uint8_t* fragO = d->at<uint8_t>(d->p.fragO);
    float* part = d->at<float>(d->p.part);
    const long long pstr = (long long)TMAX * D;
    HIPCHK(launch_f32_to_frag(q0 + 2 * D, 3 * D, T, D, fragO, st));
    int S = 0;
    CHK(skinny(d, {{d->W(LW(0, "self_attn.o_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragO, part, D, D}}, D,
               T, SK_PARTIAL, 0, &S, st));
    RowArgs r2 = rows_base(d, D, T);
    r2.x = d->at<float>(d->p.x1);
    r2.init = d->at<float>(d->p.h0);
    r2.part = part;
    r2.S = S;
    r2.part_stride = pstr;
    r2.gate = m_sa + 2 * D;
    r2.norm = ROW_LN_MOD;
    r2.scale = m_ca;
    r2.shift = m_ca + D;
    r2.eps = c.ln_eps;
    r2.frag_out = fragH;
    CHK(rows(r2, st));
    CHK(skinny(d, {{d->W(LW(0, "cross_attn.q_proj.weight")), nullptr, nullptr, nullptr, nullptr, fragH,
                    d->at<float>(d->p.q0c), D, D}},
               D, T, SK_PARTIAL, pick_qsplit(D), nullptr, st, pstr, (size_t)QKV_SLABS * TMAX * D));
    return FM_OK;
}

// c1 = sum_k (1 + scale_k) W[m][k] and c2 = sum_k shift_k W[m][k] of every product that takes a LayerNorm-modulated
// row in the draft, under the handle's modulation table (at create and whenever the table changes): each is one
// group of a two-row skinny product over the fragments of (1 + scale, shift).
fm_status flowmap_ln_fold(fm_drafter* d, hipStream_t st) {
    const auto& c = d->c;
    const int D = c.dim, L = c.layers;
    const float* mod = d->at<float>(d->p.modc);
    uint8_t* lf = d->at<uint8_t>(d->p.lnfrag);
    float* c12 = d->at<float>(d->p.c12);
    HIPCHK(launch_ln_fold_rows(mod, D, 3 * L + 1, lf, st));
    std::vector<SkGroupDesc> gs;
    auto flush = [&]() -> fm_status {
        if (!gs.empty()) CHK(skinny(d, gs, D, 2, SK_F32, 0, nullptr, st));
        gs.clear();
        return FM_OK;
    };
    auto add = [&](const std::string& w, int j, size_t off, int M) -> fm_status {
        if (gs.size() == SK_MAX_GROUPS) CHK(flush());
        gs.push_back({d->W(w), nullptr, nullptr, nullptr, nullptr, lf + (size_t)j * D * 64, c12 + off, M, M});
        return FM_OK;
    };
    for (int l = 0; l < L; ++l) {
        if (l > 0) {
            CHK(add(LW(l, "self_attn.q_proj.weight"), 3 * l, c12_off(c, l, 0), D));
            CHK(add(LW(l, "self_attn.k_proj.weight"), 3 * l, c12_off(c, l, 1), D));
            CHK(add(LW(l, "self_attn.v_proj.weight"), 3 * l, c12_off(c, l, 2), D));
            CHK(add(LW(l, "cross_attn.q_proj.weight"), 3 * l + 1, c12_off(c, l, 3), D));
        }
        CHK(add(LW(l, "mlp.fc1.weight"), 3 * l + 2, c12_off(c, l, 4), c.ffn));
    }
    CHK(add("head.weight", 3 * L, c12_off(c, L, 0), c.target_dim));
    return flush();
}

// Arguments of the persistent draft kernel, uploaded once: weights, cache rows, the handle's buffers and the arena
// layout for this device's work-group count. Leaves draft_ready false (the launches path serves the handle) when
// one work-group per CU does not fit.
fm_status draft_setup(fm_drafter* d, hipStream_t st) {
    const auto& c = d->c;
    if (!draft_supported(c)) return FM_OK;
    int dev = 0, ncu = 0;
    HIPCHK(hipGetDevice(&dev));
    HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    if (draft_occupancy() < 1 || ncu < 1) return FM_OK;
    d->G = std::min(ncu, DR_MAX_WG);
    const DraftLayout lay = draft_layout(c, d->G);
    const DraftLayout cap = draft_layout(c, DR_MAX_WG);   // the arena was sized with this one
    if (lay.total > cap.total) return FM_OK;
    const int D = c.dim;
    for (int l = 0; l < c.layers; ++l) {
        DraftLayer& L = d->dl[l];
        auto w = [&](const char* n) { return d->B(LW(l, n)); };
        L.wq = w("self_attn.q_proj.weight"); L.wk = w("self_attn.k_proj.weight"); L.wv = w("self_attn.v_proj.weight");
        L.wo = w("self_attn.o_proj.weight"); L.qn = w("self_attn.q_norm.weight"); L.kn = w("self_attn.k_norm.weight");
        L.wqc = w("cross_attn.q_proj.weight"); L.woc = w("cross_attn.o_proj.weight");
        L.cqn = w("cross_attn.q_norm.weight"); L.ckn = w("cross_attn.k_norm.weight");
        L.wck = w("cross_attn.k_proj.weight"); L.wcv = w("cross_attn.v_proj.weight");
        L.w1 = w("mlp.fc1.weight"); L.b1 = w("mlp.fc1.bias"); L.w2 = w("mlp.fc2.weight"); L.b2 = w("mlp.fc2.bias");
        L.kc = (uint16_t*)d->kv_layer(l, 0);
        L.vc = (uint16_t*)d->kv_layer(l, 1);
        const uint32_t b = (uint32_t)l * lay.layer_bytes;
        L.a3 = b + lay.a3; L.xpart = b + lay.xpart; L.mfrag = b + lay.mfrag; L.ocs = b + lay.ocs; L.xm = b + lay.xm;
        L.hm = b + lay.hm; L.u = b + lay.u; L.f2s = b + lay.f2s; L.x0 = b + lay.x0; L.h0 = b + lay.h0;
        L.qkv = b + lay.qkv; L.sao = b + lay.sao; L.os = b + lay.os; L.xs = b + lay.xs; L.hc = b + lay.hc;
        L.qcs = b + lay.qcs;
    }
    DraftArgs& a = d->dh;
    a.L = d->at<DraftLayer>(d->p.dlayers);
    a.layers = c.layers; a.D = D; a.H = c.heads; a.hd = c.head_dim; a.F = c.ffn; a.Ht = c.target_dim; a.V = c.vocab;
    a.mod = d->at<float>(d->p.modc);
    a.rope = d->at<float>(d->p.rope);
    a.wap = d->B("anchor_proj.weight"); a.bap = d->B("anchor_proj.bias"); a.anorm = d->B("anchor_norm.weight");
    a.E = d->B("lm_head.weight"); a.whead = d->B("head.weight"); a.bhead = d->B("head.bias");
    a.q0c = d->at<float>(d->p.q0c);
    a.q0c_slabs = pick_qsplit(D);
    a.q0c_stride = (long long)TMAX * D;
    a.x1 = d->at<float>(d->p.x1);
    a.ln_eps = c.ln_eps; a.rms_eps = c.rms_eps; a.qk_eps = c.qk_eps; a.scale = 1.f / sqrtf((float)c.head_dim);
    a.arena = d->at<uint8_t>(d->p.arena);
    a.a1 = lay.a1; a.xf = lay.xf; a.hf = lay.hf; a.xpart_cap = lay.xpart_cap;
    a.S_a1 = lay.S_a1; a.S_qkv = lay.S_qkv; a.S_o = lay.S_o; a.S_qc = lay.S_qc; a.S_oc = lay.S_oc; a.S_f2 = lay.S_f2;
    a.sync = d->at<uint32_t>(d->p.dsync);
    a.limit = 20000000;   // 0.2 s at the 100 MHz real-time clock: far beyond any draft; only a broken launch reaches it
    a.G = d->G;
    HIPCHK(hipMemcpyAsync(d->at<uint8_t>(d->p.dlayers), d->dl, (size_t)c.layers * sizeof(DraftLayer),
                          hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(d->at<uint8_t>(d->p.dargs), &d->dh, sizeof(DraftArgs), hipMemcpyHostToDevice, st));
    HIPCHK(launch_fill_u32(a.sync, DR_SYNC_WORDS, 0u, st));
    d->draft_ready = true;
    return FM_OK;
}

// The draft as one persistent kernel: clear its arrival counters (a fill kernel, so the pair can be captured in a
// graph), then one launch.
fm_status flowmap_draft_persistent(fm_drafter* d, const fm_block_args* ba, float* hidden_out, hipStream_t st) {
    int ns, cpw, xg;
    draft_xsplit(ba->pos, d->c.heads, d->G, ns, cpw, xg);
    if ((uint32_t)(4 * xg) > d->dh.xpart_cap) return fail(FM_E_INVALID, "cross-attention runs exceed the arena");
    HIPCHK(launch_fill_u32(d->dh.sync, 8 * 64, 0u, st));
    HIPCHK(launch_draft(d->at<DraftArgs>(d->p.dargs), d->G, ba->pos, ba->anchor, hidden_out, ba->debug_layers, st));
    return FM_OK;
}

fm_status flowmap_create(fm_drafter* d, hipStream_t st) {
    const auto& c = d->c;
    const int Ht = c.target_dim, D = c.dim;
    HIPCHK(launch_fill_u32(d->at<uint32_t>(d->p.rtick), RTICK_MAX + SATICK_MAX, 0u, st));   // each last arrival
                                                                                            // resets its own
    HIPCHK(hipMemcpyAsync(d->at<float>(d->p.modc), d->F("mod"), (size_t)(3 * c.layers + 1) * 3 * D * 4,
                          hipMemcpyDeviceToDevice, st));
    // zero-noise slot input h0 = x_embed(state_norm(mean row of E)) + b
    HIPCHK(launch_colmean(d->B("lm_head.weight"), c.vocab, Ht, d->at<float>(d->p.colsc), d->p.colR,
                          d->at<float>(d->p.cmean), st));
    RowArgs r = rows_base(d, Ht, 1);
    r.init = d->at<float>(d->p.cmean);
    r.norm = ROW_RMS;
    r.w_bf16 = d->B("state_norm.weight");
    r.eps = c.rms_eps;
    r.frag_out = d->at<uint8_t>(d->p.fragA);
    CHK(rows(r, st));
    CHK(skinny(d, {{d->W("x_embed.weight"), nullptr, nullptr, nullptr, d->B("x_embed.bias"), d->at<uint8_t>(d->p.fragA),
                    d->at<float>(d->p.h0), D, D}},
               Ht, 1, SK_F32, 0, nullptr, st));
    CHK(flowmap_layer0(d, st));
    CHK(flowmap_ln_fold(d, st));
    return draft_setup(d, st);
}

// ── KV-injection ────────────────────────────────────────────────────────────────────────────────
std::string BB(int i, const char* s) {
    char b[64];
    snprintf(b, sizeof b, "bb.%d.%s", i, s);
    return b;
}

fm_status kvinject_append(fm_drafter* d, const float* taps, int n, int start, hipStream_t st) {
    const auto& c = d->c;
    const int D = c.dim, KT = c.n_taps * c.target_dim;
    if (n <= TMAX) {
        HIPCHK(launch_f32_to_frag(taps, KT, n, KT, d->at<uint8_t>(d->p.fragA), st));
        int S = 0;
        float* part = d->at<float>(d->p.part);
        CHK(skinny(d, {{d->W("W_c"), nullptr, nullptr, nullptr, nullptr, d->at<uint8_t>(d->p.fragA), part, D, D}}, KT, n,
                   SK_PARTIAL, 0, &S, st));
        float* hc = d->at<float>(d->p.hc);
        RowArgs r = rows_base(d, D, n);
        r.part = part;
        r.S = S;
        r.part_stride = (long long)TMAX * D;
        r.norm = ROW_RMS;
        r.w_bf16 = d->B("ctx_norm");
        r.eps = c.rms_eps;
        r.f32_out = hc;
        r.out_ld = D;
        CHK(rows(r, st));
        // per layer: RMSNorm(H_ctx; attn_norm) -> K, V written straight into the f32 cache rows
        for (int i = 0; i < c.layers; ++i) {
            uint8_t* fr = i % 2 ? d->at<uint8_t>(d->p.fragO) : d->at<uint8_t>(d->p.fragH);
            RowArgs q = rows_base(d, D, n);
            q.in_rows = hc;
            q.in_ld = D;
            q.norm = ROW_RMS;
            q.w_bf16 = d->B(BB(i, "attn_norm"));
            q.eps = c.rms_eps;
            q.frag_out = fr;
            CHK(rows(q, st));
            CHK(skinny(d,
                       {{d->W(BB(i, "k")), nullptr, nullptr, nullptr, nullptr, fr,
                         (float*)d->kv_layer(i, 0) + (size_t)start * D, D, D},
                        {d->W(BB(i, "v")), nullptr, nullptr, nullptr, nullptr, fr,
                         (float*)d->kv_layer(i, 1) + (size_t)start * D, D, D}},
                       D, n, SK_F32, 0, nullptr, st));
        }
        return FM_OK;
    }
    float* ctx = d->at<float>(d->p.pctx);
    uint16_t* ctxn = d->at<uint16_t>(d->p.pctxn);
    int nslab = 1;
    CHK(prefill_context(d, taps, n, d->B("W_c"), d->w16_ctx(), ctx, &nslab, st));
    // H_ctx = RMSNorm(ctx; ctx_norm) in place (f32; split slabs summed into slab 0's rows, times the taps' row scales),
    // then per layer RMSNorm(H_ctx; attn_norm) -> f16
    {
        RowArgs r = rows_base(d, D, n);
        r.part = ctx;
        r.S = nslab;
        r.part_stride = (long long)n * D;
        r.row_scale = d->at<float>(d->p.rscale);
        r.norm = ROW_RMS;
        r.w_bf16 = d->B("ctx_norm");
        r.eps = c.rms_eps;
        r.f32_out = ctx;
        r.out_ld = D;
        CHK(rows(r, st));
    }
    for (int i = 0; i < c.layers; ++i)
        HIPCHK(launch_rms_f16(ctx, n, D, d->B(BB(i, "attn_norm")), c.rms_eps, ctxn + (size_t)i * c.max_ctx * D, 1, 0,
                              nullptr, st));
    for (int l0 = 0; l0 < c.layers; l0 += PF_MAX_GROUPS / 2) {
        PrefillArgs a{};
        const int nl = std::min(c.layers - l0, PF_MAX_GROUPS / 2);
        const int tile = prefill_tile(n, D, 2 * nl);
        const int mt = (n + tile - 1) / tile;
        const int per = mt * (D / tile);
        for (int j = 0; j < nl; ++j) {
            const int i = l0 + j;
            const uint16_t* Ai = ctxn + (size_t)i * c.max_ctx * D;
            a.g[2 * j] = PrefillGroup{Ai, d->B(BB(i, "k")), d->w16_kv(i, 0), nullptr, d->kv_layer(i, 0), PF_CACHE_V,
                                      (2 * j) * per};
            a.g[2 * j + 1] = PrefillGroup{Ai, d->B(BB(i, "v")), d->w16_kv(i, 1), nullptr, d->kv_layer(i, 1), PF_CACHE_V,
                                          (2 * j + 1) * per};
        }
        a.ngroups = 2 * nl;
        a.rows = n;
        a.N = D;
        a.K = D;
        a.ld = D;
        a.hd = c.head_dim;
        a.start = start;
        a.kv_dtype = c.kv_dtype;
        a.m_tiles = mt;
        a.n_tiles = D / tile;
        HIPCHK(launch_prefill(a, 2 * nl * per, st));
    }
    return FM_OK;
}

// B requests in one pass (B = 1: fm_draft_block): handle ds[b] holds request b's context cache, handle ds[0]'s
// workspace holds the B * block rows; every projection streams its weights once for all rows, each request attends
// over its own cache rows ++ its own block rows.
fm_status kvinject_draft_batch(fm_drafter* const* ds, int B, const int32_t* const* anchors, float* hidden_out,
                               float* debug_layers, hipStream_t st) {
    fm_drafter* d = ds[0];
    const auto& c = d->c;
    const int D = c.dim, G = c.block, T = B * G, Ht = c.target_dim, hd = c.head_dim;
    float* part = d->at<float>(d->p.part);
    float* x = d->at<float>(d->p.x);
    uint8_t* fragA = d->at<uint8_t>(d->p.fragA);
    uint8_t* fragH = d->at<uint8_t>(d->p.fragH);
    uint8_t* fragO = d->at<uint8_t>(d->p.fragO);
    uint8_t* fragU = d->at<uint8_t>(d->p.fragU);
    float* qkv = d->at<float>(d->p.qkv);
    const long long pstr = (long long)TMAX * D;

    // block rows of request b: H_d[0] = tok_proj(E[anchor_b]) + block_pos[0]; H_d[k] = mask_emb[k-1] + block_pos[k]
    for (int b = 0; b < B; ++b)
        HIPCHK(launch_gather_frag(d->B("lm_head.weight"), c.vocab, Ht, anchors[b], fragA, st, b));
    int S = 0;
    CHK(skinny(d, {{d->W("tok_proj"), nullptr, nullptr, nullptr, nullptr, fragA, part, D, D}}, Ht, B, SK_PARTIAL, 0,
               &S, st));
    for (int b = 0; b < B; ++b) {
        RowArgs r = rows_base(d, D, G);
        r.row0 = b * G;
        r.x = x;
        r.base_zero = 1;
        r.part = part + (size_t)b * D;   // tok_proj output row b feeds the request's row 0 only
        r.S = S;
        r.part_stride = pstr;
        r.part_rows = 1;
        r.base_bf16 = d->B("mask_emb");
        r.base_from = 1;
        r.row_bias_bf16 = d->B("block_pos");
        r.norm = ROW_RMS;
        r.w_bf16 = d->B(BB(0, "attn_norm"));
        r.eps = c.rms_eps;
        r.frag_out = fragH;
        CHK(rows(r, st));
    }
    const float scale = 1.f / sqrtf((float)hd);
    // Every RMSNorm inside the stack is folded (SkinnyArgs ln_rms): the residual updates of o and down (SK_RESID, gate
    // 1) write x, the fragments of x w for the next product (w: the next norm's weight) and x's per-tile statistics;
    // that product (the gate | up pair, the next layer's q | k | v) scales its rows by rstd. Layer 0's q | k | v takes
    // the normalised rows of the row kernel above, and the last layer's out_norm stays a row kernel (its f32 rows
    // feed the confidence head).
    float2* stats = d->at<float2>(d->p.lnstats);
    SkExtra fold;
    fold.ln_stats = (const float*)stats;
    fold.ln_tiles = D / 16;
    fold.ln_eps = c.rms_eps;
    fold.ln_rms = 1;
    auto resid = [&](const uint16_t* w_next, float* dbg) {
        SkExtra e;
        e.rx = x;
        e.rx_ld = D;
        e.rbase = x;
        e.rbase_ld = D;
        e.ryw = w_next;
        e.rstats = (float*)stats;
        e.rdebug = dbg;
        return e;
    };
    for (int i = 0; i < c.layers; ++i) {
        CHK(skinny(d,
                   {{d->W(BB(i, "q")), nullptr, nullptr, nullptr, nullptr, fragH, qkv, D, 3 * D},
                    {d->W(BB(i, "k")), nullptr, nullptr, nullptr, nullptr, fragH, qkv + D, D, 3 * D},
                    {d->W(BB(i, "v")), nullptr, nullptr, nullptr, nullptr, fragH, qkv + 2 * D, D, 3 * D}},
                   D, T, SK_F32, 0, nullptr, st, 0, 0, 1, i > 0 ? &fold : nullptr));
        // bidirectional attention of each request over [its context rows ++ its block rows]
        for (int b = 0; b < B; ++b) {
            float* qb = qkv + (size_t)b * G * 3 * D;
            QPrep qp{};
            qp.q = qb;
            qp.q_ld = 3 * D;
            qp.q_hs = hd;
            CHK(attend(ds[b], qp, G, i, 0, ds[b]->length, qb + D, qb + 2 * D, G, 3 * D, -1, scale, nullptr, 0, 0, fragO,
                       st, b * G));
        }
        // o and the residual; fragments of x ff_norm for the gated unit
        const SkExtra eo = resid(d->B(BB(i, "ff_norm")), nullptr);
        CHK(skinny(d, {{d->W(BB(i, "o")), nullptr, nullptr, nullptr, nullptr, fragO, fragH, D, 0}}, D, T, SK_RESID,
                   KVI_RESID_SPLIT, nullptr, st, 0, 0, 1, &eo));
        CHK(skinny(d, {{d->W(BB(i, "gate")), nullptr, d->W(BB(i, "up")), nullptr, nullptr, fragH, fragU, c.ffn, 0}},
                   D, T, SK_FRAG_GEGLU, 0, nullptr, st, 0, 0, 1, &fold));
        const bool last = i + 1 == c.layers;
        float* dbg = debug_layers ? debug_layers + (size_t)i * T * D : nullptr;
        if (!last) {   // down and the residual; fragments of x attn_norm of the next layer
            const SkExtra ed = resid(d->B(BB(i + 1, "attn_norm")), dbg);
            CHK(skinny(d, {{d->W(BB(i, "down")), nullptr, nullptr, nullptr, nullptr, fragU, fragH, D, 0}}, c.ffn, T,
                       SK_RESID, KVI_RESID_SPLIT, nullptr, st, 0, 0, 1, &ed));
            continue;
        }
        CHK(skinny(d, {{d->W(BB(i, "down")), nullptr, nullptr, nullptr, nullptr, fragU, part, D, D}}, c.ffn, T,
                   SK_PARTIAL, 0, &S, st));
        // residual + out_norm; each request's normed block rows are also kept in its own handle for the confidence
        // head (fm_markov_argmax on that handle)
        for (int b = 0; b < B; ++b) {
            RowArgs r = rows_base(d, D, G);
            r.row0 = b * G;
            r.x = x;
            r.part = part + (size_t)r.row0 * D;
            r.S = S;
            r.part_stride = pstr;
            if (dbg) r.debug_x = dbg;
            r.norm = ROW_RMS;
            r.w_bf16 = d->B("out_norm");
            r.eps = c.rms_eps;
            r.frag_out = fragH;
            r.f32_out = ds[b]->at<float>(ds[b]->p.blockn);
            r.f32_local = 1;
            r.out_ld = D;
            CHK(rows(r, st));
        }
    }
    CHK(skinny(d, {{d->W("out_proj"), nullptr, nullptr, nullptr, nullptr, fragH, hidden_out, Ht, Ht}}, D, T, SK_F32, 0,
               nullptr, st));
    return FM_OK;
}

fm_status kvinject_draft(fm_drafter* d, const fm_block_args* ba, float* hidden_out, hipStream_t st) {
    fm_drafter* ds[1] = {d};
    const int32_t* an[1] = {ba->anchor};
    return kvinject_draft_batch(ds, 1, an, hidden_out, ba->debug_layers, st);
}

// ── MTP ─────────────────────────────────────────────────────────────────────────────────────────
// B requests in one pass (B = 1: fm_draft_block): request b's M_b rows are rows off_b .. off_b + M_b - 1 of the
// pass (off_b = M_0 + ... + M_(b-1)), handle ds[b] holds its KV cache; the projections run once over all rows, the
// q/k preparation (with its cache write) and the causal attention run per request.
fm_status mtp_draft_batch(fm_drafter* const* ds, int B, const fm_block_args* const* as, float* hidden_out,
                          hipStream_t st) {
    fm_drafter* d = ds[0];
    const auto& c = d->c;
    const int H = c.dim, NH = c.heads, NKV = c.kv_heads, HD = c.head_dim;
    const int qw = NH * 2 * HD, kw = NKV * HD, qkvw = qw + 2 * kw;
    int off[TMAX + 1];
    off[0] = 0;
    for (int b = 0; b < B; ++b) off[b + 1] = off[b] + as[b]->rows;
    const int M = off[B];
    float* part = d->at<float>(d->p.part);
    float* x = d->at<float>(d->p.x);
    uint8_t* fragA = d->at<uint8_t>(d->p.fragA);
    uint8_t* fragH = d->at<uint8_t>(d->p.fragH);
    uint8_t* fragO = d->at<uint8_t>(d->p.fragO);
    uint8_t* fragU = d->at<uint8_t>(d->p.fragU);
    float* qkv = d->at<float>(d->p.qkv);
    float* qout = d->at<float>(d->p.qout);
    const long long pstr = (long long)TMAX * H;
    auto Q = [&](const char* n) { return d->W(std::string(n) + ".qt"); };   // the copies in the MFMA operand layout
    auto Dd = [&](const char* n) { return d->W(std::string(n) + ".dt"); };

    // The three RMSNorms that feed a Q8_0 product (enorm | hnorm before eh_proj, attn_norm, post_attention_norm)
    // are folded into it: a row kernel writes the fragments of w x and each 512-column slice's sum of squares, the
    // product scales its rows by their rstd. ssq holds one or two segments' sums ([segment][16][nsl]).
    float* ssq = d->at<float>(d->p.ssq);
    const int nsl = (H + 511) / 512;
    SkExtra fold{};
    fold.rms_ssq = ssq;
    fold.rms_nsl = nsl;
    fold.rms_seg = H;
    fold.rms_inv = 1.f / (float)H;
    fold.rms_eps = c.rms_eps;
    auto rms = [&](int nseg, const float* in0, const float* in1, int row0, int T, bool x_in, const float* w0,
                   const float* w1, int S, uint8_t* frag, int frag_kw) -> fm_status {
        RmsSegArgs r{};
        r.in[0] = in0;
        r.in[1] = in1;
        r.in_ld = H;
        r.x_in = x_in ? 1 : 0;
        r.x = nseg == 1 ? x : nullptr;
        r.part = S > 0 ? part : nullptr;
        r.part_stride = pstr;
        r.S = S;
        r.w[0] = w0;
        r.w[1] = w1;
        r.frag = frag;
        r.frag_kw = frag_kw;
        r.ssq = ssq;
        r.nsl = nsl;
        r.D = H;
        r.T = T;
        r.row0 = row0;
        r.nseg = nseg;
        HIPCHK(launch_rms_seg(r, st));
        return FM_OK;
    };
    // x = eh_proj([enorm(e); hnorm(h)])
    for (int b = 0; b < B; ++b)
        CHK(rms(2, as[b]->embed_rows, as[b]->prev_hidden, off[b], as[b]->rows, false, d->F("enorm"), d->F("hnorm"), 0,
                fragA, 2 * H));
    // eh_proj's splits each take columns of one norm's segment: an even split of the 2H columns
    int S = pick_split_ws(ws_groups(H), 2 * H);
    for (int s2 = S; S % 2 && s2 <= 8; ++s2)
        if ((2 * H / 256) % s2 == 0 && s2 % 2 == 0) S = s2;
    if (S % 2) S = 2;
    CHK(skinny(d, {{Q("eh_proj"), Dd("eh_proj"), nullptr, nullptr, nullptr, fragA, part, H, H}}, 2 * H, M, SK_PARTIAL,
               S, &S, st, 0, 0, 1, &fold));
    CHK(rms(1, nullptr, nullptr, 0, M, false, d->F("attn_norm"), nullptr, S, fragH, H));
    // q | gate, k, v as MTP_QKV_SPLIT partial slabs of [16][qkvw] (one work-group per four tiles would leave CUs
    // idle: 224 at the MTP shape), summed by mtp_prep
    int Sq = 0;
    CHK(skinny(d,
               {{Q("attn_q"), Dd("attn_q"), nullptr, nullptr, nullptr, fragH, qkv, qw, qkvw},
                {Q("attn_k"), Dd("attn_k"), nullptr, nullptr, nullptr, fragH, qkv + qw, kw, qkvw},
                {Q("attn_v"), Dd("attn_v"), nullptr, nullptr, nullptr, fragH, qkv + qw + kw, kw, qkvw}},
               H, M, SK_PARTIAL, MTP_QKV_SPLIT, &Sq, st, (long long)TMAX * qkvw, d->p.qkv_floats, 1, &fold));
    for (int b = 0; b < B; ++b) {
        fm_drafter* e = ds[b];
        float* qb = qkv + (size_t)off[b] * qkvw;
        MtpPrepArgs p{};
        p.qf = qb;
        p.kt = qb + qw;
        p.vt = qb + qw + kw;
        p.qf_ld = p.kt_ld = p.vt_ld = qkvw;
        p.S = Sq;
        p.slab = (long long)TMAX * qkvw;
        p.M = as[b]->rows;
        p.NH = NH;
        p.NKV = NKV;
        p.HD = HD;
        p.rot = c.rope_dims;
        p.qn = d->F("attn_q_norm");
        p.kn = d->F("attn_k_norm");
        p.eps = c.rms_eps;
        p.rope_tab = e->at<float>(e->p.rope);
        p.pos0 = as[b]->pos;
        p.qout = qout + (size_t)off[b] * NH * HD;
        p.kc = (float*)e->kv;
        p.vc = (float*)e->kv + (size_t)e->c.max_ctx * kw;
        HIPCHK(launch_mtp_prep(p, st));
        QPrep qp{};
        qp.q = qout + (size_t)off[b] * NH * HD;
        qp.q_ld = NH * HD;
        qp.q_hs = HD;
        CHK(attend(e, qp, as[b]->rows, 0, as[b]->kv_lo, as[b]->pos + as[b]->rows, nullptr, nullptr, 0, 0, as[b]->pos,
                   1.f / sqrtf((float)HD), qb + HD, qkvw, 2 * HD, fragO, st, off[b]));
    }
    CHK(skinny(d, {{Q("attn_output"), Dd("attn_output"), nullptr, nullptr, nullptr, fragO, part, H, H}}, NH * HD, M,
               SK_PARTIAL, 0, &S, st));
    CHK(rms(1, nullptr, nullptr, 0, M, true, d->F("post_attention_norm"), nullptr, S, fragH, H));
    CHK(skinny(d, {{Q("ffn_gate"), Dd("ffn_gate"), Q("ffn_up"), Dd("ffn_up"), nullptr, fragH, fragU, c.ffn, 0}}, H, M,
               SK_FRAG_SWIGLU, 0, nullptr, st, 0, 0, 1, &fold));
    CHK(skinny(d, {{Q("ffn_down"), Dd("ffn_down"), nullptr, nullptr, nullptr, fragU, part, H, H}}, c.ffn, M,
               SK_PARTIAL, 0, &S, st));
    {
        RowArgs r = rows_base(d, H, M);
        r.x = x;
        r.part = part;
        r.S = S;
        r.part_stride = pstr;
        if (B == 1 && as[0]->debug_layers) r.debug_x = as[0]->debug_layers;
        r.norm = ROW_RMS;
        r.w_f32 = d->F("shared_head_norm");
        r.eps = c.rms_eps;
        r.f32_out = hidden_out;
        r.out_ld = H;
        CHK(rows(r, st));
    }
    return FM_OK;
}

fm_status mtp_draft(fm_drafter* d, const fm_block_args* ba, float* hidden_out, hipStream_t st) {
    fm_drafter* ds[1] = {d};
    const fm_block_args* as[1] = {ba};
    return mtp_draft_batch(ds, 1, as, hidden_out, st);
}

fm_status kvinject_create(fm_drafter* d, hipStream_t st) {
    HIPCHK(launch_fill_u32(d->at<uint32_t>(d->p.rtick), RTICK_MAX + SATICK_MAX, 0u, st));   // each last arrival
    return FM_OK;                                                                              // resets its own
}

}  // namespace

// ── C ABI ───────────────────────────────────────────────────────────────────────────────────────
extern "C" {

size_t fm_kv_bytes(const fm_config* cfg) {
    if (validate_config(cfg) != FM_OK) return 0;
    const fm_config& c = *cfg;
    if (c.variant == FM_VARIANT_MTP) return 2 * (size_t)c.max_ctx * c.kv_heads * c.head_dim * 4;
    const size_t es = c.kv_dtype == FM_KV_F16 ? 2 : 4;
    return 2 * (size_t)c.layers * c.max_ctx * c.dim * es;
}

size_t fm_workspace_bytes(const fm_config* cfg) {
    if (validate_config(cfg) != FM_OK) return 0;
    return make_plan(*cfg).total;
}

fm_status fm_create(const fm_config* cfg, int32_t n_weights, const char* const* names, const void* const* ptrs,
                    void* kv_cache, void* workspace, void* stream, fm_drafter** out) {
    g_err.clear();
    if (!out) return fail(FM_E_INVALID, "null output handle pointer");
    *out = nullptr;
    CHK(validate_config(cfg));
    if (!kv_cache || !workspace) return fail(FM_E_INVALID, "null kv_cache or workspace");
    if (((uintptr_t)kv_cache & 255) || ((uintptr_t)workspace & 255))
        return fail(FM_E_INVALID, "kv_cache and workspace must be 256-byte aligned");
    if (n_weights < 0 || (n_weights > 0 && (!names || !ptrs))) return fail(FM_E_INVALID, "bad weight table");
    auto* d = new fm_drafter();
    d->c = *cfg;
    d->p = make_plan(*cfg);
    d->ws = (uint8_t*)workspace;
    d->kv = (uint8_t*)kv_cache;
    d->length = 0;
    for (int i = 0; i < n_weights; ++i) {
        if (!names[i]) { delete d; return fail(FM_E_INVALID, "null weight name at %d", i); }
        if (!ptrs[i]) { delete d; return fail(FM_E_INVALID, "null pointer for weight %s", names[i]); }
        d->w[names[i]] = ptrs[i];
    }
    for (const auto& n : required_names(*cfg))
        if (!d->W(n)) {
            delete d;
            return fail(FM_E_MISSING_WEIGHT, "missing weight '%s'", n.c_str());
        }
    if (cfg->variant == FM_VARIANT_KVINJECT && cfg->block < 1) { delete d; return fail(FM_E_INVALID, "gamma"); }
    for (const Q8Mat& m : q8_mats(*cfg))   // checked before any work is enqueued: the copies read codes 8 bytes a lane
        if (((uintptr_t)d->W(std::string(m.name) + ".q") & 7) || ((uintptr_t)d->W(std::string(m.name) + ".d") & 1)) {
            delete d;
            return fail(FM_E_INVALID, "%s.q must be 8-byte aligned and %s.d 2-byte aligned", m.name, m.name);
        }
    hipStream_t st = (hipStream_t)stream;
    fm_status s = FM_OK;
    do {
        if (launch_fill_u32(d->at<uint32_t>(d->p.best), 2 * (size_t)d->p.best_rows, 0u, st) != hipSuccess) {
            s = fail(FM_E_HIP, "fill");
            break;
        }
        if (cfg->variant == FM_VARIANT_KVINJECT && launch_fill_u32(d->at<uint32_t>(d->p.mcut), 1, 0u, st) != hipSuccess) {
            s = fail(FM_E_HIP, "fill");
            break;
        }
        if (launch_fill_u32(d->at<uint32_t>(d->p.zeros), d->p.zeros_bytes / 4, 0u, st) != hipSuccess) {
            s = fail(FM_E_HIP, "fill");
            break;
        }
        if (cfg->rope != FM_ROPE_NONE) {
            hipError_t e = launch_rope_table(d->at<float>(d->p.rope), d->p.rope_rows, d->p.rope_dims, cfg->rope_theta, st);
            if (e == hipSuccess && cfg->variant == FM_VARIANT_FLOWMAP)
                e = launch_rope_prefill(d->at<float>(d->p.rope), d->p.rope_rows, d->p.rope_dims,
                                        d->at<float>(d->p.rope_pf), st);
            if (e != hipSuccess) { s = fail(FM_E_HIP, "rope table: %s", hipGetErrorString(e)); break; }
        }
        if (cfg->variant != FM_VARIANT_MTP) {
            s = prefill_weight_copies(d, st);
            if (s != FM_OK) break;
        }
        size_t q8o = d->p.q8t;
        for (const Q8Mat& m : q8_mats(*cfg)) {
            const std::string n = m.name;
            uint8_t* oq = d->at<uint8_t>(q8o);
            q8o += align256((size_t)m.M * m.K);
            uint16_t* od = d->at<uint16_t>(q8o);
            q8o += align256((size_t)m.M * (m.K / 32) * 2);
            const hipError_t e = launch_q8_tile_copy((const int8_t*)d->W(n + ".q"), (const uint16_t*)d->W(n + ".d"),
                                                     m.M, m.K, oq, od, st);
            if (e != hipSuccess) {
                s = fail(FM_E_HIP, "Q8_0 copy of %s: %s", m.name, hipGetErrorString(e));
                break;
            }
            d->w[n + ".qt"] = oq;
            d->w[n + ".dt"] = od;
        }
        if (s != FM_OK) break;
        if (cfg->variant == FM_VARIANT_FLOWMAP) s = flowmap_create(d, st);
        else if (cfg->variant == FM_VARIANT_KVINJECT) s = kvinject_create(d, st);
    } while (0);
    if (s != FM_OK) { fm_destroy(d); return s; }
    *out = d;
    return FM_OK;
}

fm_status fm_context_append(fm_drafter* d, const float* taps, int32_t n, int32_t start, void* stream) {
    g_err.clear();
    if (!d) return fail(FM_E_INVALID, "null handle");
    if (d->c.variant == FM_VARIANT_MTP) return fail(FM_E_INVALID, "the MTP head has no context append");
    if (!taps) return fail(FM_E_INVALID, "null taps");
    if ((uintptr_t)taps & 15) return fail(FM_E_INVALID, "taps must be 16-byte aligned");
    if (n < 1) return fail(FM_E_INVALID, "n = %d < 1", n);
    if (start < 0 || start > d->length) return fail(FM_E_INVALID, "start %d outside [0, length %d]", start, d->length);
    if ((long long)start + n + d->c.block + 1 > d->c.max_ctx)
        return fail(FM_E_CONTEXT_FULL, "context full: start %d + n %d + block %d + 1 > max_ctx %d", start, n,
                    d->c.block, d->c.max_ctx);
    hipStream_t st = (hipStream_t)stream;
    fm_status s = d->c.variant == FM_VARIANT_FLOWMAP ? flowmap_append(d, taps, n, start, st)
                                                     : kvinject_append(d, taps, n, start, st);
    if (s == FM_OK) d->length = start + n;
    return s;
}

fm_status fm_draft_block(fm_drafter* d, const fm_block_args* a, float* hidden_out, void* stream) {
    g_err.clear();
    if (!d || !a || !hidden_out) return fail(FM_E_INVALID, "null argument");
    hipStream_t st = (hipStream_t)stream;
    const auto& c = d->c;
    if (c.variant == FM_VARIANT_FLOWMAP) {
        if (!a->anchor) return fail(FM_E_INVALID, "null anchor");
        if (a->pos < 0 || a->pos > d->length) return fail(FM_E_INVALID, "pos %d outside [0, length %d]", a->pos, d->length);
        if ((long long)a->pos + c.block + 1 > c.max_ctx) return fail(FM_E_CONTEXT_FULL, "pos %d + block + 1 > max_ctx", a->pos);
        if (d->draft_ready && d->draft_path == 2) return flowmap_draft_persistent(d, a, hidden_out, st);
        return flowmap_draft(d, a, hidden_out, st);
    }
    if (c.variant == FM_VARIANT_KVINJECT) {
        if (!a->anchor) return fail(FM_E_INVALID, "null anchor");
        return kvinject_draft(d, a, hidden_out, st);
    }
    if (!a->embed_rows || !a->prev_hidden) return fail(FM_E_INVALID, "null embed_rows / prev_hidden");
    if (a->rows < 1 || a->rows > c.block) return fail(FM_E_INVALID, "rows %d outside [1, %d]", a->rows, c.block);
    if (a->pos < 0 || a->kv_lo < 0 || a->kv_lo > a->pos)
        return fail(FM_E_INVALID, "need 0 <= kv_lo (%d) <= pos (%d)", a->kv_lo, a->pos);
    if ((long long)a->pos + a->rows > c.max_ctx)
        return fail(FM_E_CONTEXT_FULL, "pos %d + rows %d > KV cache rows %d", a->pos, a->rows, c.max_ctx);
    return mtp_draft(d, a, hidden_out, st);
}

fm_status fm_lm_argmax(fm_drafter* d, const float* hidden, int32_t rows, int32_t* tokens, float* logits, void* stream) {
    g_err.clear();
    if (!d || !hidden || !tokens) return fail(FM_E_INVALID, "null argument");
    // flow-map handles (bf16 tables) take the rows of a two-request batch
    const int rmax = d->c.variant == FM_VARIANT_FLOWMAP && d->c.wtype == FM_W_BF16 ? FM_BATCH * TMAX : TMAX;
    if (rows < 1 || rows > rmax) return fail(FM_E_INVALID, "rows %d outside [1, %d]", rows, rmax);
    hipStream_t st = (hipStream_t)stream;
    const int K = d->c.target_dim;
    uint8_t* fr = d->at<uint8_t>(d->p.fragH);
    HIPCHK(launch_f32_to_frag(hidden, K, rows, K, fr, st));
    LmArgs a{};
    const bool q8 = d->c.wtype == FM_W_Q8_0;
    a.E = q8 ? d->W("lm_head.qt") : d->W("lm_head.weight");
    a.Ed = q8 ? d->W("lm_head.dt") : nullptr;
    a.X = fr;
    a.V = d->c.vocab;
    a.K = K;
    a.T = rows;
    a.best = d->at<unsigned long long>(d->p.best);
    a.tokens = tokens;
    a.logits = logits;
    HIPCHK(launch_lm_argmax(a, q8 ? 1 : 0, st));
    return FM_OK;
}

fm_status fm_lm_argmax_static(fm_drafter* d, const float* hidden, int32_t rows, int32_t* tokens, void* stream) {
    g_err.clear();
    if (!d || !hidden || !tokens) return fail(FM_E_INVALID, "null argument");
    if (rows < 1 || rows > TMAX) return fail(FM_E_INVALID, "rows %d outside [1, %d]", rows, TMAX);
    const int K = d->c.target_dim;
    if ((size_t)256 + (size_t)K * 64 > STATIC_SCRATCH_BYTES)
        return fail(FM_E_INVALID, "target_dim %d: the static scratch holds fragments of rows up to %d wide", K,
                    (int)((STATIC_SCRATCH_BYTES - 256) / 64));
    hipError_t e = hipSuccess;
    uint8_t* s = (uint8_t*)static_scratch(&e);
    if (!s) return fail(FM_E_HIP, "static scratch: %s", hipGetErrorString(e));
    hipStream_t st = (hipStream_t)stream;
    unsigned long long* keys = (unsigned long long*)s;   // must start at zero: cleared by a kernel on every call
    uint8_t* fr = s + 256;
    HIPCHK(launch_fill_u32((uint32_t*)keys, 32, 0u, st));
    HIPCHK(launch_f32_to_frag(hidden, K, rows, K, fr, st));
    LmArgs a{};
    const bool q8 = d->c.wtype == FM_W_Q8_0;
    a.E = q8 ? d->W("lm_head.qt") : d->W("lm_head.weight");
    a.Ed = q8 ? d->W("lm_head.dt") : nullptr;
    a.X = fr;
    a.V = d->c.vocab;
    a.K = K;
    a.T = rows;
    a.best = keys;
    a.tokens = tokens;
    HIPCHK(launch_lm_argmax(a, q8 ? 1 : 0, st));
    return FM_OK;
}

fm_status fm_mtp_chain(fm_drafter* d, int32_t* tokens, const float* h, int32_t steps, int32_t pos, int32_t kv_lo,
                       float* hidden_out, void* stream) {
    g_err.clear();
    if (!d || !tokens || !h || !hidden_out) return fail(FM_E_INVALID, "null argument");
    const auto& c = d->c;
    if (c.variant != FM_VARIANT_MTP) return fail(FM_E_INVALID, "fm_mtp_chain needs an MTP drafter");
    if (steps < 1) return fail(FM_E_INVALID, "steps %d < 1", steps);
    if (pos < 0 || kv_lo < 0 || kv_lo > pos) return fail(FM_E_INVALID, "need 0 <= kv_lo (%d) <= pos (%d)", kv_lo, pos);
    if ((long long)pos + steps > c.max_ctx)
        return fail(FM_E_CONTEXT_FULL, "pos %d + steps %d > KV cache rows %d", pos, steps, c.max_ctx);
    hipStream_t st = (hipStream_t)stream;
    const int H = c.dim;
    float* e = d->at<float>(d->p.echain);
    const bool q8 = c.wtype == FM_W_Q8_0;
    for (int i = 0; i < steps; ++i) {
        // e = the previous draft token's table row; h = the previous pass's output (the caller's row first)
        if (q8)
            HIPCHK(launch_gather_q8_f32((const int8_t*)d->W("lm_head.q"), (const uint16_t*)d->W("lm_head.d"), c.vocab,
                                        H, tokens + i, e, st));
        else
            HIPCHK(launch_gather_f32(d->B("lm_head.weight"), c.vocab, H, tokens + i, nullptr, e, st));
        fm_block_args a{};
        a.rows = 1;
        a.pos = pos + i;
        a.kv_lo = kv_lo;
        a.embed_rows = e;
        a.prev_hidden = i == 0 ? h : hidden_out + (size_t)(i - 1) * H;
        CHK(mtp_draft(d, &a, hidden_out + (size_t)i * H, st));
        CHK(fm_lm_argmax(d, hidden_out + (size_t)i * H, 1, tokens + i + 1, nullptr, stream));
    }
    return FM_OK;
}

fm_status fm_markov_argmax(fm_drafter* d, const float* hidden, int32_t rows, const int32_t* anchor, int32_t rank,
                           int32_t* tokens, float* conf, float* scores, const float* thresholds, int32_t* length,
                           void* stream) {
    g_err.clear();
    if (!d || !hidden || !anchor || !tokens || !conf) return fail(FM_E_INVALID, "null argument");
    const auto& c = d->c;
    if (c.variant != FM_VARIANT_KVINJECT) return fail(FM_E_INVALID, "fm_markov_argmax needs a KV-injection drafter");
    if (rows < 1 || rows > c.block) return fail(FM_E_INVALID, "rows %d outside [1, %d]", rows, c.block);
    if (rank < 1 || rank > MARKOV_MAX_RANK) return fail(FM_E_INVALID, "rank %d outside [1, %d]", rank, MARKOV_MAX_RANK);
    if (c.vocab % 4) return fail(FM_E_UNSUPPORTED, "vocab %d not a multiple of 4", c.vocab);
    for (const char* n : {"markov.w1", "markov.w2", "conf.w", "conf.b"})
        if (!d->w.count(n)) return fail(FM_E_INVALID, "missing weight %s", n);
    hipStream_t st = (hipStream_t)stream;
    float* z = d->at<float>(d->p.zbase);
    // base logits of every row (the fused lm_head with its logits output; its own tokens are overwritten below)
    CHK(fm_lm_argmax(d, hidden, rows, tokens, z, stream));
    MarkovArgs a{};
    a.w1 = d->B("markov.w1");
    a.w2 = d->B("markov.w2");
    a.cw = d->B("conf.w");
    a.cb = d->B("conf.b");
    a.z = z;
    a.block = d->at<float>(d->p.blockn);
    a.anchor = anchor;
    a.tokens = tokens;
    a.conf = conf;
    a.scores = scores;
    a.key = d->at<unsigned long long>(d->p.best);
    a.V = c.vocab;
    a.r = rank;
    a.D = c.dim;
    a.prune = thresholds ? 1 : 0;
    for (int k = 0; thresholds && k < rows; ++k) a.thr[k] = thresholds[k];
    a.cut = d->at<int32_t>(d->p.mcut);
    a.length = length;
    HIPCHK(launch_markov(a, rows, st));   // the keys of rows [0, rows) were cleared by the lm_head's finalize
    return FM_OK;
}

fm_status fm_time_condition(fm_drafter* d, float s, float t, int32_t time_dim, int32_t cond_dim, float time_scale,
                            float* table_out, void* stream) {
    g_err.clear();
    if (!d) return fail(FM_E_INVALID, "null handle");
    const auto& c = d->c;
    if (c.variant != FM_VARIANT_FLOWMAP) return fail(FM_E_INVALID, "time conditioning needs a flow-map drafter");
    if (time_dim < 2 || time_dim % 2 || time_dim > TC_MAX_DIM || cond_dim < 1 || cond_dim > TC_MAX_DIM)
        return fail(FM_E_INVALID, "time_dim %d / cond_dim %d outside [2, %d] (time_dim even)", time_dim, cond_dim,
                    TC_MAX_DIM);
    const int nn = 3 * c.layers + 1;
    if (nn > TC_MAX_NORMS) return fail(FM_E_UNSUPPORTED, "%d norms", nn);
    TimeCondArgs a{};
    const char* pre[2] = {"time_embed", "jump_embed"};
    char b[128];
    auto need = [&](const char* n) -> const uint16_t* {
        auto it = d->w.find(n);
        return it == d->w.end() ? nullptr : (const uint16_t*)it->second;
    };
    for (int w = 0; w < 2; ++w) {
        snprintf(b, sizeof b, "%s.linear_1.weight", pre[w]); a.l1w[w] = need(b);
        snprintf(b, sizeof b, "%s.linear_1.bias", pre[w]);   a.l1b[w] = need(b);
        snprintf(b, sizeof b, "%s.linear_2.weight", pre[w]); a.l2w[w] = need(b);
        snprintf(b, sizeof b, "%s.linear_2.bias", pre[w]);   a.l2b[w] = need(b);
        if (!a.l1w[w] || !a.l1b[w] || !a.l2w[w] || !a.l2b[w]) return fail(FM_E_INVALID, "missing %s weights", pre[w]);
    }
    for (int n = 0; n < nn; ++n) {
        static const char* br[3] = {"self_attn", "cross_attn", "mlp"};
        if (n < 3 * c.layers) snprintf(b, sizeof b, "layers.%d.%s_adaln.linear.", n / 3, br[n % 3]);
        else snprintf(b, sizeof b, "final_adaln.linear.");
        const std::string base = b;
        a.aw[n] = need((base + "weight").c_str());
        a.ab[n] = need((base + "bias").c_str());
        if (!a.aw[n] || !a.ab[n]) return fail(FM_E_INVALID, "missing %sweight / bias", b);
    }
    a.times[0] = s;
    a.times[1] = t;
    a.time_scale = time_scale;
    a.td = time_dim;
    a.cd = cond_dim;
    a.rows = 3 * c.dim;
    a.nnorm = nn;
    a.cond = d->at<float>(d->p.tcond);
    a.table = d->at<float>(d->p.modc);   // the handle's own table: other handles sharing the weights keep theirs
    HIPCHK(launch_time_condition(a, (hipStream_t)stream));
    if (table_out)
        HIPCHK(hipMemcpyAsync(table_out, a.table, (size_t)nn * 3 * c.dim * 4, hipMemcpyDeviceToDevice,
                              (hipStream_t)stream));
    fm_status r = flowmap_layer0(d, (hipStream_t)stream);   // layer 0's projections follow the new table
    if (r == FM_OK) r = flowmap_ln_fold(d, (hipStream_t)stream);   // and so do the LayerNorm fold's c1 / c2
    if (r == FM_OK) {
        const float key[5] = {s, t, (float)time_dim, (float)cond_dim, time_scale};
        memcpy(d->tc_key, key, sizeof key);
        d->tc_set = true;
    }
    return r;
}

fm_status fm_draft_batch(fm_drafter* const* ds, int32_t B, const fm_block_args* args, float* hidden_out,
                         void* stream) {
    g_err.clear();
    if (!ds || !args || !hidden_out || B < 1) return fail(FM_E_INVALID, "null argument or B < 1");
    if (B > TMAX) return fail(FM_E_INVALID, "B %d > %d", B, TMAX);
    for (int b = 0; b < B; ++b)
        if (!ds[b]) return fail(FM_E_INVALID, "null handle %d", b);
    const auto& c = ds[0]->c;
    if (c.variant == FM_VARIANT_FLOWMAP && B > FM_BATCH)
        return fail(FM_E_UNSUPPORTED, "flow-map batches take at most %d requests", FM_BATCH);
    for (int b = 1; b < B; ++b) {
        const fm_drafter* e = ds[b];
        const auto& f = e->c;   // the shape of the block computation (max_ctx may differ: each cache is its own)
        if (f.variant != c.variant || f.dim != c.dim || f.heads != c.heads || f.head_dim != c.head_dim ||
            f.kv_heads != c.kv_heads || f.layers != c.layers || f.ffn != c.ffn || f.block != c.block ||
            f.target_dim != c.target_dim || f.n_taps != c.n_taps || f.vocab != c.vocab || f.mlp != c.mlp ||
            f.kv_dtype != c.kv_dtype || f.wtype != c.wtype || f.rms_eps != c.rms_eps || f.rope != c.rope ||
            f.rope_dims != c.rope_dims || f.rope_theta != c.rope_theta)
            return fail(FM_E_INVALID, "handle %d: another configuration", b);
        for (const auto& n : required_names(c)) {
            const auto& w0 = ds[0]->w;
            const auto& w1 = e->w;
            auto i0 = w0.find(n);
            auto i1 = w1.find(n);
            if (i0 == w0.end() || i1 == w1.end() || i0->second != i1->second)
                return fail(FM_E_INVALID, "handle %d: weight %s is not the same tensor", b, n.c_str());
        }
        for (int a = 0; a < b; ++a)
            if (ds[a] == e) return fail(FM_E_INVALID, "handle %d appears twice", b);
    }
    hipStream_t st = (hipStream_t)stream;
    if (c.variant == FM_VARIANT_FLOWMAP) {
        if (B > 1 && (c.block != TMAX || c.wtype != FM_W_BF16 || c.dim % 512 || c.ffn % 512 ||
                      c.dim > 16 * LN_MAX_TILES / FM_BATCH))
            return fail(FM_E_UNSUPPORTED, "flow-map batches need 16-slot blocks, bf16 weights, dim and ffn %% 512 == 0, "
                                          "dim <= %d", 16 * LN_MAX_TILES / FM_BATCH);
        const fm_block_args* as[FM_BATCH];
        for (int b = 0; b < B; ++b) {
            const fm_block_args* a = &args[b];
            const fm_drafter* e = ds[b];
            if (!a->anchor) return fail(FM_E_INVALID, "request %d: null anchor", b);
            if (a->pos < 0 || a->pos > e->length)
                return fail(FM_E_INVALID, "request %d: pos %d outside [0, length %d]", b, a->pos, e->length);
            if ((long long)a->pos + c.block + 1 > e->c.max_ctx)
                return fail(FM_E_CONTEXT_FULL, "request %d: pos %d + block + 1 > max_ctx", b, a->pos);
            if (e->tc_set != ds[0]->tc_set || (e->tc_set && memcmp(e->tc_key, ds[0]->tc_key, sizeof e->tc_key)))
                return fail(FM_E_INVALID, "handle %d: another modulation table (time conditioning)", b);
            as[b] = a;
        }
        return flowmap_draft_batch(ds, B, as, hidden_out, st);
    }
    if (c.variant == FM_VARIANT_KVINJECT) {
        if (B * c.block > TMAX) return fail(FM_E_INVALID, "B %d x block %d > %d rows", B, c.block, TMAX);
        const int32_t* an[TMAX];
        for (int b = 0; b < B; ++b) {
            if (!args[b].anchor) return fail(FM_E_INVALID, "request %d: null anchor", b);
            an[b] = args[b].anchor;
        }
        return kvinject_draft_batch(ds, B, an, hidden_out, nullptr, st);
    }
    const fm_block_args* as[TMAX];
    int rows_total = 0;
    for (int b = 0; b < B; ++b) {
        const fm_block_args* a = &args[b];
        if (!a->embed_rows || !a->prev_hidden) return fail(FM_E_INVALID, "request %d: null embed_rows / prev_hidden", b);
        if (a->rows < 1 || a->rows > c.block)
            return fail(FM_E_INVALID, "request %d: rows %d outside [1, %d]", b, a->rows, c.block);
        if (a->pos < 0 || a->kv_lo < 0 || a->kv_lo > a->pos)
            return fail(FM_E_INVALID, "request %d: need 0 <= kv_lo (%d) <= pos (%d)", b, a->kv_lo, a->pos);
        if ((long long)a->pos + a->rows > ds[b]->c.max_ctx)
            return fail(FM_E_CONTEXT_FULL, "request %d: pos %d + rows %d > KV cache rows %d", b, a->pos, a->rows,
                        ds[b]->c.max_ctx);
        rows_total += a->rows;
        as[b] = a;
    }
    if (rows_total > TMAX) return fail(FM_E_INVALID, "%d rows in all > %d", rows_total, TMAX);
    return mtp_draft_batch(ds, B, as, hidden_out, st);
}

fm_status fm_set_draft_path(fm_drafter* d, int32_t path) {
    g_err.clear();
    if (!d) return fail(FM_E_INVALID, "null handle");
    if (path < 0 || path > 2) return fail(FM_E_INVALID, "draft path %d (0 auto, 1 launches, 2 persistent)", path);
    if (path == 2 && !d->draft_ready)
        return fail(FM_E_UNSUPPORTED, "no persistent draft kernel for this drafter (shape or device)");
    d->draft_path = path;
    return FM_OK;
}

int32_t fm_draft_path(const fm_drafter* d) {
    if (!d) return -1;
    return (d->draft_ready && d->draft_path == 2) ? 2 : 1;
}

fm_status fm_device_status(fm_drafter* d, void* stream) {
    g_err.clear();
    if (!d) return fail(FM_E_INVALID, "null handle");
    if (!d->draft_ready) return FM_OK;
    HIPCHK(hipStreamSynchronize((hipStream_t)stream));
    uint32_t e = 0;
    uint32_t* w = d->dh.sync + 8 * 64;
    HIPCHK(hipMemcpy(&e, w, 4, hipMemcpyDeviceToHost));
    if (e) {
        const uint32_t z = 0;
        HIPCHK(hipMemcpy(w, &z, 4, hipMemcpyHostToDevice));
        return fail(FM_E_DEVICE, "a persistent draft launch gave up waiting (its results are not valid)");
    }
    return FM_OK;
}

fm_status fm_profile_draft(fm_drafter* d, const fm_block_args* a, float* hidden_out, int32_t reps, float* skinny_us,
                           int32_t* skinny_launches, float* draft_us, void* stream) {
    g_err.clear();
    if (!d || !a || !hidden_out || !skinny_us || !skinny_launches || !draft_us)
        return fail(FM_E_INVALID, "null argument");
    if (d->c.variant != FM_VARIANT_FLOWMAP) return fail(FM_E_UNSUPPORTED, "profile: flow-map drafters only");
    if (a->pos < 0 || a->pos + 1 > d->c.max_ctx) return fail(FM_E_INVALID, "pos %d outside the cache", a->pos);
    if (!a->anchor) return fail(FM_E_INVALID, "null anchor");
    if (reps < 1 || reps > 64) return fail(FM_E_INVALID, "reps %d outside [1, 64]", reps);
    hipStream_t st = (hipStream_t)stream;
    for (hipEvent_t& e : d->ev)
        if (!e) HIPCHK(hipEventCreate(&e));
    const int wt = d->c.wtype == FM_W_Q8_0 ? SKW_Q8_0 : SKW_BF16;
    // 1. one draft, recording its skinny launches
    std::vector<std::pair<SkinnyArgs, int>> rec;
    d->rec = &rec;
    const fm_status s = flowmap_draft(d, a, hidden_out, st);
    d->rec = nullptr;
    if (s != FM_OK) return s;
    // 2. the recorded skinny launches alone, `reps` times over, between two events; a hold kernel ahead of them
    // keeps the GPU busy while the host queues them, so they run back to back as in a draft
    HIPCHK(launch_hold(200000, st));   // 2 ms
    HIPCHK(hipEventRecord(d->ev[0], st));
    for (int r = 0; r < reps; ++r)
        for (const auto& l : rec) HIPCHK(launch_skinny(l.first, wt, l.second, st));
    HIPCHK(hipEventRecord(d->ev[1], st));
    // 3. the whole draft once more, the same way (its outputs are the call's outputs)
    HIPCHK(launch_hold(200000, st));
    HIPCHK(hipEventRecord(d->ev[2], st));
    CHK(flowmap_draft(d, a, hidden_out, st));
    HIPCHK(hipEventRecord(d->ev[3], st));
    HIPCHK(hipStreamSynchronize(st));
    float k1 = 0.f, tot = 0.f;
    HIPCHK(hipEventElapsedTime(&k1, d->ev[0], d->ev[1]));
    HIPCHK(hipEventElapsedTime(&tot, d->ev[2], d->ev[3]));
    *skinny_us = k1 * 1e3f / (float)reps;
    *skinny_launches = (int32_t)rec.size();
    *draft_us = tot * 1e3f;
    return FM_OK;
}

int32_t fm_context_length(const fm_drafter* d) { return d ? d->length : -1; }

void fm_destroy(fm_drafter* d) {
    if (!d) return;
    delete d;
}

const char* fm_last_error(void) { return g_err.c_str(); }

}  // extern "C"
