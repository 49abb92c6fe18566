// fm_kernels.h — argument blocks and host launchers of the gfx950 kernels (internal to libfm).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ── K1: skinny-T weight-streaming GEMM ─────────────────────────────────────────────────────────
// Y[t][m] = sum_k X[t][k] W[m][k] for t < T <= 16 (or, with nb = 2 blocks of activation rows, t < 32): weights
// streamed once from HBM straight into the A operand of v_mfma_f32_16x16x32_bf16 (16 rows x 32 k per step),
// activations read as hi/lo bf16 fragments (fm_device.h; block b of the rows at X + b * K * 64).
// A work-group is 4 waves on one 16-row tile, each wave a quarter of the group's k-range; the 4 partial tiles are
// summed in LDS. S > 1 splits k across work-groups; those write partial slabs the consumer sums in order. Output row
// t of block b is row 16 b + t of out (SK_F32, SK_PARTIAL) or of the output fragments (block b at out + b * M * 64).
enum SkinnyOut {
    SK_F32 = 0,        // out[t*ld + m] = acc + bias[m]
    SK_PARTIAL = 1,    // out[split*part_stride + t*ld + m] = acc
    SK_FRAG_GELU = 2,  // frag(out)[t][m] = gelu_erf(acc + bias[m])
    SK_FRAG_GEGLU = 3, // frag(out)[t][m] = gelu_tanh(acc_gate) * acc_up        (two weight tiles)
    SK_FRAG_SWIGLU = 4, // frag(out)[t][m] = silu(acc_gate) * acc_up            (two weight tiles)
    SK_RESID = 5        // residual update (bf16, one matrix): x[t][m] = base[t][m] + gate[m] (acc + bias[m]);
                        // frag(out)[t][m] = x[t][m] (1 + yscale[m]); (mean, M2) of x over each 16-column tile. With
                        // S > 1 the last split of a tile to arrive (an arrival counter) sums the splits and finishes it
};
enum SkinnyWType { SKW_BF16 = 0, SKW_Q8_0 = 1 };

#define SK_MAX_GROUPS 12
// Flow-map self-attention over the T slots of each block of rows, one head at a time (fm_selfattn.h): run by the
// q | k | v product's last work-group of each head (SkinnyArgs.sa); writes o as fragments.
struct SelfAttnArgs {
    const float* qkv;      // [rows][3D]: q | k | v (null: no self-attention)
    int T, D, heads, hd;
    const uint16_t* qn;    // q_norm, k_norm (bf16 [hd])
    const uint16_t* kn;
    float eps;
    const float* rope_tab;
    int pos_base;          // RoPE position of row 0 of block 0
    float scale;
    uint8_t* o_frag;
    int nb;                // blocks of T rows attending each within itself (1 or 2): block b's rows are rows 16 b + t
    int pos_base1;         //   of qkv (T = 16) and of the o fragments (K = D); its RoPE positions start at pos_base1
};

struct SkinnyGroup {
    const void* W;        // bf16 [M][K], or Q8_0 codes int8 [M][K]
    const void* Wd;       // Q8_0 scales f16 [M][K/32] (else null)
    const void* W2;       // second weight tile (GLU "up"), same format, or null
    const void* W2d;
    const uint16_t* bias; // bf16 [M] or null
    const uint8_t* X;     // activation fragments, K/32 steps
    void* out;
    int M;                // rows (multiple of 16)
    int ld;               // output row stride (elements)
    int tile_begin;       // first work-group of this group
    int pad;
    const float* c12;     // LayerNorm fold: c1 = c12[m], c2 = c12[M + m] (see SkinnyArgs), or null
};
struct SkinnyArgs {
    SkinnyGroup g[SK_MAX_GROUPS];
    int ngroups;
    int K;
    int T;
    int S;                // k-splits across work-groups
    int KW;               // k-steps per wave (K / 32 == S * 4 * KW), any value >= 1
    int mode;
    long long part_stride;
    int nb;               // blocks of 16 activation rows: 1, or 2 (bf16, KW % 4 == 0; T = 16 rows per block)
    const float* zeros;   // a zero row (the target of loads an epilogue does not use)
    // LayerNorm fold (bf16, one matrix): the activation fragments hold y = x (1 + s) of rows x whose LayerNorm with
    // modulation (x - mean) rstd (1 + s) + shift is the product's real input. ln_stats (float2 [ln_tiles][16 nb])
    // holds (mean, M2) of each 16-column tile of x (an SK_RESID epilogue's output); with c1 = sum_k (1 + s_k) W[m][k]
    // and c2 = sum_k shift_k W[m][k] (the group's c12), the epilogue takes rstd (acc - mean c1[m]) + c2[m] as the
    // product (SK_PARTIAL: split 0 adds the constant part, every split scales by rstd).
    // ln_rms: the fold of an RMSNorm instead (one or two matrices, no c12): the fragments hold y = x w (w the norm's
    // weight), and the epilogue takes rstd acc with rstd = 1 / sqrt(mean(x^2) + eps) from the same statistics.
    const float* ln_stats;
    int ln_tiles;         // x's width / 16 (at most LN_MAX_TILES / nb)
    float ln_inv;         // 1 / ln_tiles
    float ln_eps;
    int ln_rms;
    // SK_RESID
    float* rx;            // residual stream [rows][rx_ld], written (x above)
    int rx_ld;
    const float* rbase;   // base rows [rows][rbase_ld] (rbase_ld 0: one row for every row); may be rx
    int rbase_ld;
    const float* rgate;   // f32 [M] or null (gate 1)
    const float* ryscale; // f32 [M]: the next LayerNorm's modulation scale s (fragments of x (1 + s))
    const uint16_t* ryw;  // or bf16 [M]: the next RMSNorm's weight w (fragments of x w)
    float* rstats;        // float2 [M / 16][16 nb]: (mean, M2) of x over each 16-column tile, per row
    float* rdebug;        // optional copy of x (same layout)
    float* rpart;         // S > 1: the splits' partial tiles [S][rows][M] (slab stride part_stride)
    uint32_t* rtick;      // S > 1: one arrival counter per 16-row tile, zero between launches
    // q | k | v followed by the self-attention (SK_F32, the LayerNorm fold, three groups q, k, v of D rows each,
    // S = 1): the outputs are stored device-coherent, each tile's work-group takes a ticket on its head's counter
    // (satick[head], zero between launches), and the head's last arrival (3 hd / 16 of them) runs its attention
    SelfAttnArgs sa;
    uint32_t* satick;
    // RMSNorm fold of the Q8_0 variant: the fragments hold w x of rows x whose RMSNorm is the real input, rms_ssq the
    // sums of squares of x per 512-column slice (launch_rms_seg: [segment][16][rms_nsl]); a split's columns lie in
    // segment c / rms_seg, and the product of row t is scaled by 1 / sqrt(sum ssq * rms_inv + rms_eps)
    const float* rms_ssq;
    int rms_nsl;
    int rms_seg;
    float rms_inv;
    float rms_eps;
};
#define LN_MAX_TILES 256   // LayerNorm fold: x at most 4096 wide (2048 with two blocks of rows)
// Q8_0 weights run the tile-owning variant: a work-group of SK_WS_WAVES waves owns that many adjacent 16-row tiles
// of a group, or for a gated unit half as many tiles of each of its two matrices (tile_begin then counts work-groups:
// ceil(M / (16 SK_WS_WAVES)) x S per group, twice that for a gated unit) over a k-range of K / S columns (a multiple
// of 256), sharing one LDS copy of the activation fragments.
#define SK_WS_WAVES 4
hipError_t launch_skinny(const SkinnyArgs& a, int wtype, int n_workgroups, hipStream_t st);

// ── K3: row kernels (residual update + norm + fragment store) ─────────────────────────────────
enum RowNorm { ROW_NONE = 0, ROW_LN_MOD = 1, ROW_RMS = 2 };
struct RowArgs {
    float* x;              // residual stream [T][D] updated in place (or null)
    const float* init;     // if set, the row's base value is init[i] (broadcast over rows) instead of x
    const float* in_rows;  // if set, base value is in_rows[t*in_ld + i]
    int in_ld;
    const float* part;     // split partials [S][T][D] added (or null)
    long long part_stride;
    int S;
    const uint16_t* bias;  // bf16 [D] added with the partials (or null)
    const float* gate;     // f32 [D]: x = base + gate * update (null: gate 1)
    int norm;              // RowNorm
    const float* scale;    // LN-mod: LN(x) * (1 + scale) + shift
    const float* shift;
    const uint16_t* w_bf16;// RMSNorm weight (bf16) or
    const float* w_f32;    //   (f32)
    float eps;
    uint8_t* frag_out;     // normalised row -> fragments at k offset frag_koff (or null)
    int frag_koff;
    float* f32_out;        // normalised row as f32 [T][out_ld] (or null)
    int out_ld;
    float* debug_x;        // copy of the updated stream [T][D] (or null)
    int D;
    int T;
    int base_zero;         // base value 0 even when x is set (x is then only written)
    int part_rows;         // rows t >= part_rows take no partials (0: every row)
    const uint16_t* base_bf16;  // rows t >= base_from take their base from these bf16 rows [(t - base_from)][D]
    int base_from;
    const uint16_t* row_bias_bf16;  // bf16 [T][D] added to row t (or null)
    const float* zeros;    // a zero row of >= D floats (absent inputs read it; required)
    const float* row_scale;// if set, the partial sum of row t (slabs + biases) is multiplied by row_scale[t]
    int f32_local;         // 1: f32_out row t is at f32_out + t * out_ld (not row0 + t)
    int row0;              // row t of the launch is row row0 + t of x, debug_x, frag_out and f32_out (batched blocks)
    int frag_kw;           // width of the fragment matrix frag_out (0: D); rows >= 16 sit in its second block
};
hipError_t launch_rows(const RowArgs& a, hipStream_t st);

// The RMSNorm fold's producer: for rows row0 .. row0 + T - 1 (at most 16 in all) and nseg (1 or 2) segments of D
// columns, segment s's row v = in[s] row t (in_ld apart; null: x's row if x_in, else 0), plus with one segment the
// S split partials (row row0 + t of each [16][D] slab, part_stride floats apart); x (one segment) receives v; the
// fragments (width frag_kw) receive w[s] * v at k offset s D; ssq[(s 16 + row) nsl + slice] the sum of v^2 over
// each 512-column slice (nsl = ceil(D / 512)). The consumer (SkinnyArgs.rms_*) scales its product by
// 1 / sqrt(sum ssq / D + eps).
struct RmsSegArgs {
    const float* in[2];
    int in_ld;
    int x_in;              // 1: the base is x's row (segment 0, no in[0])
    float* x;
    const float* part;
    long long part_stride;
    int S;
    const float* w[2];     // f32 RMSNorm weights
    uint8_t* frag;
    int frag_kw;
    float* ssq;
    int nsl;
    int D, T, row0, nseg;
};
hipError_t launch_rms_seg(const RmsSegArgs& a, hipStream_t st);

// f32 rows [T][K] (row stride ld) -> fragments. T <= 32 (rows 16.. in the second block), K % 32 == 0.
hipError_t launch_f32_to_frag(const float* x, int ld, int T, int K, uint8_t* frag, hipStream_t st);
// fragments of (1 + scale, shift) of each of nmod modulations (scale, shift, gate rows of D) for the LayerNorm fold
hipError_t launch_ln_fold_rows(const float* mod, int D, int nmod, uint8_t* frag, hipStream_t st);
// bf16 row E[*idx] of a [V][K] table -> fragments (T = 1, lo = 0); ids are clamped to [0, V).
hipError_t launch_gather_frag(const uint16_t* E, int V, int K, const int32_t* idx, uint8_t* frag,
                              hipStream_t st, int row = 0);
// Time conditioning of a jump s -> t: the modulation table [nnorm][rows] (rows = 3 D: scale | shift | gate) from the
// time MLPs ([0] time_embed, [1] jump_embed: linear_1 bf16 [cd][td], linear_2 [cd][cd], biases) and one adaLN
// linear per norm (bf16 [rows][cd] + bias [rows]). cond is a [cd] f32 scratch vector.
#define TC_MAX_DIM 1024
#define TC_MAX_NORMS 49
struct TimeCondArgs {
    const uint16_t* l1w[2]; const uint16_t* l1b[2]; const uint16_t* l2w[2]; const uint16_t* l2b[2];
    const uint16_t* aw[TC_MAX_NORMS]; const uint16_t* ab[TC_MAX_NORMS];
    float times[2];        // s, t
    float time_scale;
    int td, cd, rows, nnorm;
    float* cond;           // [3 * TC_MAX_DIM]: the condition vector, then the time MLPs' hidden layers
    float* table;
};
hipError_t launch_time_condition(const TimeCondArgs& a, hipStream_t st);
// Q8_0 row E[*idx] -> f32 [K] (scale times code); ids are clamped to [0, V).
hipError_t launch_gather_q8_f32(const int8_t* q, const uint16_t* dsc, int V, int K, const int32_t* idx, float* out,
                                hipStream_t st);
// bf16 row E[*idx] -> f32 [K] (+ optional bf16 row added); ids are clamped to [0, V).
hipError_t launch_gather_f32(const uint16_t* E, int V, int K, const int32_t* idx, const uint16_t* add_bf16, float* out,
                             hipStream_t st);

// ── create-time kernels ────────────────────────────────────────────────────────────────────────
// Column mean of a bf16 table [V][H] -> f32 [H] (two deterministic stages; scratch holds R*H floats).
hipError_t launch_colmean(const uint16_t* E, int V, int H, float* scratch, int R, float* out, hipStream_t st);
// RoPE table rows p < P: [cos r/2 | sin r/2] of angle p * theta^(-2i/r), built in f64, stored f32.
hipError_t launch_rope_table(float* tab, int P, int r, double theta, hipStream_t st);
// Fill n 32-bit words with v.
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
// a one-wave kernel that returns after `ticks` of the 100 MHz wall clock
hipError_t launch_hold(uint64_t ticks, hipStream_t st);

// ── K4: attention ──────────────────────────────────────────────────────────────────────────────
struct QPrep {             // how a work-group builds its query rows for one head
    const float* q;        // q rows: q[t*q_ld + h*q_hs + d]
    int q_ld;
    int q_hs;
    const float* zeros;    // a zero row of >= 256 floats (absent inputs read it; required)
    const uint16_t* norm_bf16;  // head RMSNorm weight (bf16 or f32) or null
    const float* norm_f32;
    float eps;
    int rope;              // 0 none, 1 interleaved, 2 NEOX partial
    int rope_dims;
    const float* rope_tab; // rows [cos rope_dims/2 | sin rope_dims/2]
    int pos_base;          // query t sits at position pos_base + t
    int parts;             // q is the sum of this many split-K slabs (0 or 1: one), slab i at q + i * pstride
    long long pstride;     //   (honoured by the f16-cache kernel; the f32-cache kernel takes one slab)
};

struct AttnArgs {
    QPrep qp;
    int nq;                // query rows (<= 16)
    const void* kc;        // cache keys: row j at kc + j*kv_ld (element type by kv_dtype)
    const void* vc;        // cache values: f32 rows like the keys; f16 tiled [pos/32][vt_ld dims][32]
    int kv_ld;
    int vt_ld;
    int kv_dtype;          // 0 f16, 1 f32
    int key_lo, key_hi;    // cache rows [key_lo, key_hi)
    const float* kx;       // extra keys / values (f32 rows [nx][x_ld]) after the cache rows
    const float* vx;
    int nx, x_ld;
    int heads, kv_heads, hd;
    int causal_base;       // >= 0: query t sees cache row j only if j <= causal_base + t
    float scale;
    int chunk;             // keys per chunk: attn_chunk_size(hd, kv_dtype, keys, heads)
    int cpw;               // chunks per work-group (f16-cache kernel; the others take 1)
    int nchunks;           // work-groups per head = partials per head
    float* part;           // [heads][nchunks][nq][hd + 2]: unnormalised o, running max, sum
};
// Keys per work-group of the split kernel for a head width, cache type, key count and head count (the host sizes
// nchunks with it; the launcher checks that the two agree).
int attn_chunk_size(int hd, int kv_dtype, int nkeys, int heads);
hipError_t launch_attn_split(const AttnArgs& a, hipStream_t st);

struct MergeArgs {
    const float* part;
    int heads, nchunks, nq, hd;
    const float* gate;     // optional: o *= sigmoid(gate[t*gate_ld + h*gate_hs + d])
    int gate_ld, gate_hs;
    uint8_t* o_frag;       // o row row0 + t, k = h*hd + d (rows >= 16 in the second block of K = heads * hd)
    int row0;
};
hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t st);

// K/V rows -> cache: per group (layer) g: k rows from kbuf[g] (head RMSNorm + RoPE), v rows from vbuf[g];
// written at cache rows start .. start+n-1 as f16 or f32.
struct KVFinalArgs {
    const float* stage;    // [2*layers][n][D]: k of layer l at group 2l, v at 2l+1
    int n, D, heads, hd, layers;
    const uint16_t* knorm[16];     // per layer bf16 [hd] head-norm weight of K (null: no norm, no RoPE)
    float eps;
    const float* rope_tab;
    int rope_dims;
    int start;
    void* cache;           // layer l: K at l*2*max_ctx*D, V at (2l+1)*max_ctx*D (elements; f16 V tiled by 32)
    int max_ctx;
    int kv_dtype;
    const float* zeros;    // zero row (absent norm weights / RoPE read it)
    int stage_n;           // rows per group of stage (0: n), of which this launch takes rows stage_t0 ..
    int stage_t0;
};
hipError_t launch_kv_final(const KVFinalArgs& a, hipStream_t st);

// MTP: q/k head-norm + NEOX RoPE, K/V cache write at pos0 + m; q written to qout [M][NH*HD].
struct MtpPrepArgs {
    const float* qf; const float* kt; const float* vt;
    int qf_ld, kt_ld, vt_ld;   // row strides (elements)
    int S;                 // q | gate, k, v arrive as S split-K partial slabs, slab floats apart: summed here, and each
    long long slab;        // q head's summed gate written back into slab 0 (where the attention merge reads it)
    int M, NH, NKV, HD, rot;
    const float* qn; const float* kn;
    float eps;
    const float* rope_tab;
    int pos0;
    float* qout;
    float* kc; float* vc;  // [max_ctx][NKV*HD]
};
hipError_t launch_mtp_prep(const MtpPrepArgs& a, hipStream_t st);

// ── K5: lm_head + argmax ───────────────────────────────────────────────────────────────────────
struct LmArgs {
    const void* E;         // bf16 [V][K], or Q8_0 codes in the MFMA operand layout of launch_q8_tile_copy
    const void* Ed;        // Q8_0 scales in that layout, or null
    const uint8_t* X;      // fragments of the rows (rows 16.. in a second block at X + K * 64)
    int V, K, T;           // T <= 16, or <= 32 for bf16 tables
    unsigned long long* best;  // [T] packed (value, index) maxima, zero between calls
    int32_t* tokens;
    float* logits;         // optional [T][V]
};
hipError_t launch_lm_argmax(const LmArgs& a, int wtype, hipStream_t st);
// A Q8_0 table (codes [M][K], f16 scales [M][K / 32]) copied into the layout the Q8_0 lm_head kernel streams: per
// 16-row tile and 256-column chunk, 4 KB of codes in the order the MFMA's operand registers take them, then (in the
// scale array) 16 rows x 8 scales. oq: M K bytes, od: M K / 32 halves. M % 16 == 0, K % 256 == 0; q 8-byte aligned,
// oq and od 16-byte aligned.
hipError_t launch_q8_tile_copy(const int8_t* q, const uint16_t* d, int M, int K, uint8_t* oq, uint16_t* od,
                               hipStream_t st);

// The library's static scratch (fm_static.hip): a file-scope device array of STATIC_SCRATCH_BYTES on each GPU, for
// the entry point that allocates nothing. Returns its device address on the current device (looked up once per
// device with hipGetSymbolAddress), or null with *err set.
#define STATIC_SCRATCH_BYTES ((size_t)256 + (size_t)16 * 8192 * 4)   // 16 argmax keys, then fragments of K <= 8192
void* static_scratch(hipError_t* err);

// DSpark Markov decode step k (KV-injection drafter): scores = z_k + w1[prev] w2, argmax -> tokens[k], confidence
// sigmoid([block_k; w1[prev]] conf.w + conf.b) -> conf[k]; prev = anchor (k = 0) or tokens[k - 1].
#define MARKOV_MAX_RANK 1024
struct MarkovArgs {
    const uint16_t* w1;    // bf16 [V][r]
    const uint16_t* w2;    // bf16 [r][V]
    const uint16_t* cw;    // bf16 [D + r]
    const uint16_t* cb;    // bf16 [1]
    const float* z;        // base logits [rows][V]
    const float* block;    // normed backbone rows [rows][D]
    const int32_t* anchor; // device [1]
    int32_t* tokens;       // device [rows]
    float* conf;           // device [rows]
    float* scores;         // optional [rows][V]
    unsigned long long* key;  // [rows]: step k's argmax key; zero between calls
    int V, r, D;
    int prune;             // 1: confidence pruning with thr[] (positions k >= 1 with conf < thr[k] end the block)
    float thr[16];
    int32_t* cut;          // device [1]: the step that ended the block, 0 while none has; zero between calls
    int32_t* length;       // optional device [1]: positions kept
};
// The decode steps 0 .. rows - 1 (rows <= 16), step k's argmax in key[k] (key[0 .. rows) zero on entry, zero again
// on exit). With pruning, a step whose confidence falls below its threshold ends the block there: it and every later
// step do no work, their tokens are -1 and their confidences 0.
hipError_t launch_markov(const MarkovArgs& a, int rows, hipStream_t st);

// ── K2: MFMA prefill GEMM (f16 operands, f32 accumulate) ──────────────────────────────────────
// C[r][n] = sum_k A[r][k] B[n][k]; A f16 rows, B bf16 weights converted to f16 on the way into LDS (or their f16 copies).
enum PrefillEpi {
    PF_F32 = 0,     // C f32 [rows][ld]
    PF_CACHE_K = 1, // head RMSNorm + RoPE at position start + r, stored to the cache (f16/f32)
    PF_CACHE_V = 2, // stored to the cache
    PF_CACHE_VT = 3 // f16 V cache, tiled: position p, dim n at out[((p / 32) * vt_ld + n) * 32 + p % 32]
};
struct PrefillGroup {
    const void* A;         // this group's A rows (null: PrefillArgs.A)
    const uint16_t* B;     // bf16 [N][K]
    const uint16_t* B16;   // the same matrix as f16 [N][K] (256-tiles read this one)
    const uint16_t* knorm; // bf16 [hd] (PF_CACHE_K)
    void* out;             // f32 C or the cache row 0 of this layer's K or V
    int epi;
    int tile_begin;
};
#define PF_MAX_GROUPS 12
struct PrefillArgs {
    PrefillGroup g[PF_MAX_GROUPS];
    int ngroups;
    const void* A;         // f16 [rows][K]
    int rows, N, K, ld;
    int hd;
    float eps;
    const float* rope_tab;
    const float* rope_pf;  // PF_CACHE_K with knorm: the prefill copy of the RoPE table (launch_rope_prefill)
    int rope_dims;
    int start;
    int kv_dtype;
    int vt_ld;             // PF_CACHE_VT: dims per 32-position tile (the cache row width)
    int m_tiles, n_tiles;
    int ksplit;            // > 1 (128-tiles, PF_F32 groups only): the k-range is split over ksplit work-groups per
    long long slab_stride; //   tile; split s writes its partial product to out + s * slab_stride (floats)
};
// Tile edge (128 or 256) the launcher uses for rows x N x ngroups; the host sizes m_tiles, n_tiles and the
// groups' tile_begin with it. 256-tiles need every group's B16 and K % 64 == 0.
int prefill_tile(int rows, int N, int ngroups);
hipError_t launch_prefill(const PrefillArgs& a, int n_workgroups, hipStream_t st);
// Prefill copy of the interleaved-RoPE table [P][rdim] (rdim % 64 == 0): per position, per block of 32 pairs, per
// c = 0..7 the cos then the sin of pairs c, c + 8, c + 16, c + 24 of the block.
hipError_t launch_rope_prefill(const float* tab, int P, int rdim, float* out, hipStream_t st);
// n rows of f32 taps [n][KT] -> f16 rows y = f16(x s) with s = 2^k per row (the row's largest magnitude times s in
// [2^14, 2^15)); rscale[row] = 1 / s. KT % 4 == 0, KT <= TAPS_MAX_WIDTH.
#define TAPS_MAX_WIDTH 16384
hipError_t launch_taps_f16(const float* x, int n, int KT, uint16_t* y, float* rscale, hipStream_t st);
// y = f16(x) element-wise (exact for bf16 above f16's subnormal range), n % 4 == 0.
hipError_t launch_bf16_to_f16(const uint16_t* x, size_t n, uint16_t* y, hipStream_t st);

// Row RMSNorm of f32 rows [n][D] -> f16 rows [n][D] (prefill context); row t is rscale[t] times the sum of nslab
// (1, 2 or 4) partial slabs slab_stride floats apart (rscale: the taps' row scales, launch_taps_f16).
hipError_t launch_rms_f16(const float* x, int n, int D, const uint16_t* w, float eps, uint16_t* out, int nslab,
                          long long slab_stride, const float* rscale, hipStream_t st);

// ── K8: the flow-map draft block as one persistent kernel ──────────────────────────────────────
// One work-group per CU (DR_WAVES consumer waves + one producer wave). The producer streams every weight tile and the
// context K/V of the cross-attention through an LDS ring, running ahead of the consumers across phase boundaries;
// the consumers run the phases in order (anchor slot, the DiT layers, the head), exchanging activations through a
// write-once arena with device-coherent (sc1) stores and loads and per-XCD arrival counters between phases.
#define DR_MAX_LAYERS 16
#define DR_RING 16              // 8 KB ring slots
#define DR_CHUNK 8192
#define DR_WAVES 4              // consumer waves
#define DR_SCRATCH 27136        // consumer scratch bytes (the largest phase's)
#define DR_LDS (DR_RING * DR_CHUNK + 256 + DR_SCRATCH)
#define DR_MAX_WG 256
#define DR_SYNC_WORDS (8 * 64 + 64)   // 8 arrival counters 64 words apart, then the error word
struct DraftLayer {
    const uint16_t *wq, *wk, *wv, *wo, *qn, *kn;      // self-attention: projections [D][D], head norms [hd]
    const uint16_t *wqc, *woc, *cqn, *ckn, *wck, *wcv; // cross-attention: q / o projections, q / k head norms, k / v
    const uint16_t *w1, *b1, *w2, *b2;                 // MLP: fc1 [F][D] + bias, fc2 [D][F] + bias
    uint16_t* kc;                                      // f16 K cache [max_ctx][D]
    uint16_t* vc;                                      // f16 V cache, tiled [max_ctx / 32][D][32]
    // arena byte offsets of this layer's activations (each written once per launch)
    uint32_t a3, xpart, mfrag, ocs, xm, hm, u, f2s, x0, h0, qkv, sao, os, xs, hc, qcs;
};
struct DraftArgs {             // per handle, in device memory (written at create)
    const DraftLayer* L;       // device [layers]: the per-layer table
    int layers, D, H, hd, F, Ht, V;
    const float* mod;          // the handle's modulation table [(3 layers + 1)][scale D | shift D | gate D]
    const float* rope;         // [pos][cos hd/2 | sin hd/2]
    const uint16_t *wap, *bap, *anorm, *E, *whead, *bhead;
    const float* q0c;          // layer 0's cross-attention q (create time): q0c_slabs slabs q0c_stride floats apart
    int q0c_slabs;
    long long q0c_stride;
    const float* x1;           // layer 0's residual after its self-attention (create time), [16][D]
    float ln_eps, rms_eps, qk_eps, scale;
    uint8_t* arena;
    uint32_t a1, xf, hf;       // arena offsets: anchor_proj slabs, final residual, final LN-mod fragments
    uint32_t xpart_cap;        // cross-attention partial runs the arena holds per head
    int S_a1, S_qkv, S_o, S_qc, S_oc, S_f2;   // k-splits of the projections
    uint32_t* sync;            // DR_SYNC_WORDS: arrival counters (zero at launch), then the error word
    long long limit;           // wall-clock ticks (100 MHz) any wait may take before the launch gives up
    int G;                     // work-groups
};
// Split of the cross-attention over the context keys [0, pos) (nsteps 32-key steps): runs of cpw steps, four runs
// per work-group, xgroups work-groups per head, so that heads x xgroups fills about one work-group per CU.
__host__ __device__ inline void draft_xsplit(int pos, int H, int G, int& nsteps, int& cpw, int& xgroups) {
    nsteps = (pos + 31) / 32;
    cpw = (nsteps * H + 4 * G - 1) / (4 * G);
    if (cpw < 1) cpw = 1;
    xgroups = (nsteps + 4 * cpw - 1) / (4 * cpw);
}
// Work-groups of the persistent draft kernel one CU holds at once (0: it does not fit).
int draft_occupancy();
// args: device copy of the handle's DraftArgs; pos the anchor's position (cross-attention over [0, pos]).
hipError_t launch_draft(const DraftArgs* args, int G, int pos, const int32_t* anchor, float* hidden_out, float* debug,
                        hipStream_t st);
