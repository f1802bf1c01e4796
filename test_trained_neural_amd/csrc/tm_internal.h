// Internal structures shared by the C-ABI runtime (tm_api.hip) and the
// kernels (tm_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tmk {

// Event timing of launches (tm_timing_enable): while a timed call runs, its
// launch records this pair with the kernel's own dispatch (hipExtLaunchKernel),
// so the pair brackets the kernel's execution as the profiler sees it, not
// the host-side launch around it.  Set and consumed on the calling thread.
// A timed launch made of several kernels (a split product and its
// reduction) sets `parts` first: the start event goes with the first
// kernel's dispatch, the stop event with the last one's.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
    bool used = false;
    int parts = 1, seen = 0;
};
extern thread_local LaunchEvents g_launch_ev;

template <class K, class... A>
inline void launch_k(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, A... args) {
    if (g_launch_ev.start && !g_launch_ev.used) {
        const int k = ++g_launch_ev.seen;
        const bool last = k >= g_launch_ev.parts;
        if (last) g_launch_ev.used = true;
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, k == 1 ? g_launch_ev.start : nullptr,
                              last ? g_launch_ev.stop : nullptr, 0u, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
    }
}

constexpr int MAXL = 8;                 // deepest memory MLP supported
constexpr int MAX_CHUNK = 64;           // one wave lane per token in the scan
constexpr uint32_t STATE_MAGIC = 0x314D5354u;
constexpr uint32_t STATE_VERSION = 1;

// First 256 bytes of every state blob.
struct StateHeader {
    uint32_t magic;
    uint32_t version;
    uint64_t cfg_hash;
    int32_t batch;
    int32_t heads;
    int32_t nonfinite;      // sticky: set by the update kernel
    int32_t reserved0;
    long long position;     // tokens stored since init / import
    long long reserved[27];
};
static_assert(sizeof(StateHeader) == 256, "header is 256 bytes");

// Fragment-packed matrices ("packed" below).  An operand of the 16x16x32
// matrix instruction is fed as 16-row x 32-deep fragments in which lane l
// supplies row l % 16 and the 8 consecutive K values 8 * (l / 16) .. + 7.
// Packed storage puts those 8 values of the 64 lanes next to each other:
// element (r, k) of an R x K matrix (R padded to 16, K to 32) lives at
// pk(r, k, K / 32), and the fragment (row block rb, K step ks) of lane l
// starts at pkf(rb, ks, K / 32, l).  A wave's fragment load is then one
// contiguous 1 KB (2 KB for fp32) instead of 16 rows x 64 B: measured on
// MI355X, 59 vs 18.5 bytes per clock per CU.  Every operand the kernels
// produce for another kernel's matrix instructions is stored packed; for a
// B operand the "row" is the output column.
__host__ __device__ inline long pk(int r, int k, int nks) {
    return ((((long)(r >> 4) * nks + (k >> 5)) * 64 + (r & 15) + 16 * ((k & 31) >> 3)) << 3) + (k & 7);
}
__host__ __device__ inline long pkf(int rb, int ks, int nks, int lane) {
    return (((long)rb * nks + ks) * 64 + lane) << 3;
}
__host__ __device__ inline long pk_size(long rows, long cols) {
    return ((rows + 15) / 16 * 16) * ((cols + 31) / 32 * 32);
}

// Layer 0's M and S (d x h1) are stored in the matrix instruction's
// accumulator order: per 16-column block, per 16-row block, the 16 x 16 tile
// as 64 lanes x 4 consecutive rows (lane l: rows 4 * (l / 16) .. + 3 of
// column l % 16).  The first-layer workgroup that owns a column block then
// moves a wave's 16 x 16 block of M or S as one contiguous 1 KB float4
// access.  nrb = d / 16.
__host__ __device__ inline long cf0(int i, int j, int nrb) {
    return ((((long)(j >> 4) * nrb + (i >> 4)) * 64 + (j & 15) + 16 * ((i & 15) >> 2)) << 2) + (i & 3);
}

// Layer 1's M and S (h1 x d1) are stored in the accumulator order of its
// update computed transposed (rows: layer 1's outputs n, columns: its inputs
// j): per 16-row block of j, per 16-column block of n, lane l holds the 4
// consecutive outputs n = 4 * (l / 16) .. + 3 of input j = l % 16.  The
// first-layer workgroup that owns inputs j .. j+15 then moves each 16 x 16
// block as one contiguous 1 KB float4 access.  ncb = d1 / 16.
__host__ __device__ inline long cf1(int j, int n, int ncb) {
    return ((((long)(j >> 4) * ncb + (n >> 4)) * 64 + (j & 15) + 16 * ((n & 15) >> 2)) << 2) + (n & 3);
}

// Token-major arrays [batch][Tc][H][d]; gates use d = 1.
struct TokLayout {
    int Tc, H, d;
};

enum { EPI_HIDDEN = 0, EPI_OUT = 1, EPI_BWD = 2 };

// One matrix product of the chunk forward / backward, per stream s
// (blockIdx.z):  Z[r][n] = sum_k A[r][k] B[k][n], r < nrows, n < N, k < K.
// Rows r < n0 are queries, rows r >= n0 keys (t = r - n0 is the key's token
// inside the chunk); the backward has key rows only (n0 = 0).
enum { A_TOKENS = 0, A_ROWS = 1, A_PACKED = 2 };
enum { B_STRIDED = 0, B_ROWS = 1, B_PACKED = 2, B_CFRAG = 3, B_CF1 = 4 };
struct GemmArgs {
    int nrows, N, K;
    // A.  A_TOKENS: rows r < n0 are tokens (at0 + r) of a0, rows r >= n0
    // tokens (at1 + r - n0) of a1, both in the token layout tl.  A_ROWS: row
    // r at a0 + s*a_ss + r*a_ld.  A_PACKED: packed [rows][K] at a0 + s*a_ss.
    const void* a0;
    const void* a1;
    int n0, at0, at1, amode;
    long a_ss, a_ld;
    // B.  B_STRIDED: element (k, n) at b + s*b_ss + n + k*b_ld (row-major
    // [K][N]); B_ROWS: at b + s*b_ss + n*b_ld + k (row n contiguous in K);
    // B_PACKED: packed [N][K] at b + s*b_ss; B_CFRAG: layer 0's fp32 master
    // in accumulator order, cf0(k, n, K / 16), at b + s*b_ss; B_CF1: layer
    // 1's, cf1(k, n, N / 16).
    const void* b;
    long b_ss, b_ld;
    int bmode;
    TokLayout tl;
    int epi;
    // EPI_HIDDEN: act = SiLU(z) (operand type, packed [rows][N]); key rows
    //             also dsl[t][n] = SiLU'(z) and ht = act transposed (packed
    //             [N][bp]).
    // EPI_OUT   : query rows: y at token (yt0 + r) = z; key rows:
    //             Delta = 2 (z - v at token (vt0 + t)).
    // EPI_BWD   : Delta = z * dsl[t][n].
    // OUT / BWD write Delta (operand type, packed [b][N]) to dlp if set, and
    //             the theta-weighted transposed deltas dct = (c_t Delta)^T,
    //             ddt = (d_t Delta)^T (packed [N][bp]).
    void* act;
    long act_ss;
    float* dsl;
    long dsl_ss, dsl_ld;
    void* dlp;
    long dlp_ss;
    float* y;
    const void* v;
    int yt0, vt0;
    void* ht;
    void* dct;
    void* ddt;
    long tr_ss;               // per-stream stride of ht / dct / ddt
    int bp;
    const float* cc;          // c_t of the chunk's tokens: cc[s*coef_ss + t]
    const float* dc;
    long coef_ss;
    int xcd_streams;          // 1: each stream's tiles on one XCD (ns % 8 == 0)
};

// The theta-weighted gradient reduction of one chunk and the fused
// momentum / forgetting write, for every layer.  Grid: (tiles of all layers,
// streams); tiles are 64 x 64 blocks of W_l.  Operands arrive transposed
// (token-contiguous rows of bp tokens, valid below b).
struct UpdArgs {
    int L, b, bp;
    int din[MAXL], dout[MAXL];
    long off[MAXL];
    int tj[MAXL];
    int tbase[MAXL + 1];
    long P;
    float* M;
    float* S;
    void* Wt;                 // bf16 copy of M for the forward, packed [d_out][d_in] per layer
    const void* at[MAXL];     // at[l]: layer l's input key rows transposed, packed [d_in][bp]
    long at_ss[MAXL];
    const void* dct[MAXL];    // (c Delta_l)^T, packed [d_out][bp]
    const void* ddt[MAXL];    // (d Delta_l)^T
    long dt_ss[MAXL];
    const float* cs;          // per-chunk scalars (p_alpha, p_eta, s0, 0)
    long cs_ss;
    int chunk;
    int* flag;
};

// First-layer part of chunk step c, one launch (the update tiles of layers
// 2.. for chunk c-1 ride in the same launch).  One workgroup per JW = 16
// hidden units j: columns j of W_0 (full height) and rows j of W_1:
//   * if do_update: chunk c-1's update of those columns.  The first layer's
//     Delta for the columns is formed in place (depth >= 2) from layer 1's
//     Delta and rows j of layer 1's weights (at chunk c-1's start: their
//     update in this launch comes later or goes to the other buffer), or
//     read back (depth 1); theta-weighted, reduced against the chunk's keys
//     and folded into M and S (and, on the call's last update, the bf16 copy
//     of W_0);
//   * if do_fwd: chunk c's first-layer forward of [queries of chunk c-1;
//     keys of chunk c] through the freshly written columns;
//   * if do_update and depth >= 2: chunk c-1's update of rows j of W_1 (and
//     of their bf16 copy).
// K is split over the workgroup's waves (8; 4 for small widths in launches
// without workgroups of other roles) for the backward and the forward
// products (partial tiles summed in LDS), so no wave walks a long chain of
// dependent loads.
// Depth 2 with workgroups to spare: W_1's update moves to nw1 workgroups
// per stream of its own (a multiple of 8), after the nb1 first-layer blocks,
// each updating W1_JPW blocks of 16 rows.  They run beside the first-layer blocks, which
// still read W_1's rows at chunk c-1's start for the backward, so M_1 is read
// from m1_rd and its new value written to m1_wr, a second buffer (the two
// alternate over a call's updates).  Otherwise m1_rd == m1_wr, the state's
// own M_1, updated in place by the first-layer blocks.
constexpr int JW = 16;
constexpr int W1_JPW = 3;                // row blocks per W_1-update workgroup

struct FirstArgs {
    UpdArgs u;                // layers, state, chunk scalars, flag
    int dim, h1, nb1;
    // update tiles [upd_tile0, upd_tile0 + upd_ntiles) of the other layers
    // (chunk c-1), carried two or four per workgroup after the nb1 first-layer blocks
    int upd_tile0, upd_ntiles;
    int do_update, do_fwd, nq, nk;
    int chunk_prev;
    const void* kt_prev;      // keys of chunk c-1 transposed, packed [dim][bp]
    long kt_ss;
    const void* dlt2;         // Delta of layer 1 for chunk c-1 (operand type), packed [b][dout1]
    long dlt2_ss;
    int last_update;          // the call's last update: also write W_0's bf16 copy
    float* dsl1;              // SiLU'(z) of layer 0: read (chunk c-1), then written (chunk c)
    long dsl1_ss;
    const float* cc_prev;     // coefficients of chunk c-1's tokens
    const float* dc_prev;
    const float* cc_cur;      // coefficients of chunk c's tokens
    const float* dc_cur;
    long coef_ss;
    const void* xq;           // queries of chunk c-1, packed [b][dim] (rows r < nq)
    const void* xk;           // keys of chunk c, packed [b][dim] (rows r >= nq)
    long x_ss;
    TokLayout tl;             // token layout of y and v
    int tq0, tk0;
    void* act;                // layer-0 activations of the rows, packed [2b][h1]
    long act_ss;
    void* ht1;                // key rows of act transposed, packed [h1][bp]
    long ht_ss;
    // depth 1: the first layer is the last one
    float* y;
    const void* v;
    void* dct1;               // (c Delta)^T, (d Delta)^T of layer 0, packed [h1][bp]
    void* ddt1;
    long dt1_ss;
    // W_1 (depth >= 2): where its M is read and written (layer 1's first
    // element of stream 0, and the stream stride)
    const float* m1_rd;
    long m1_rd_ss;
    float* m1_wr;
    long m1_wr_ss;
    int nw1;                  // > 0: W_1's update in workgroups of its own
    int xcd_streams;          // 1: each stream's blocks on one XCD (grid (nb1, ns), ns % 8 == 0)
};

// Per call: the coefficient scan of every (stream, chunk); every chunk's
// keys transposed (packed [d][bp] per chunk) and its key and query rows
// packed ([b][d] per chunk).
struct ScanArgs {
    const float* theta;
    const float* eta;
    const float* alpha;
    TokLayout tl;             // d = 1
    int b, C, ns;
    float* cc;
    float* dc;
    long coef_ss;
    float* cs;
    long cs_ss;
    long long* position;
    long long add;
    const void* k;            // keys, token layout ktl
    const void* q;            // queries (may be null)
    TokLayout ktl;
    void* kt;                 // [s][chunk] packed [d][bp]
    void* xk;                 // [s][chunk] packed [b][d]
    void* xq;
    long xc;                  // elements of one chunk's packed rows
    int bp, kt_f32;
};

// The input side ("Titans, explained" steps 1, 4, 5): per token x (width D)
// the projections p_i = x W_i^T (i = key, value, query; W_i is [H*d][D], one
// row per output channel), a causal depthwise convolution of each channel
// over the last K <= 4 tokens (the tokens before the call come from the
// history the previous call left: its last K-1 projections, oldest first),
// l2-normalised keys and queries per head, and the gates sigmoid(x w_g + b_g).
constexpr int MAX_CONV = 4;
struct ProjArgs {
    const void* x;            // [B][T][D]
    const void* w;            // [3][H*d][D]
    const float* conv;        // [3][H*d][K]
    const float* wg;          // [3][H][D]
    const float* gb;          // [3]
    float* hist;              // [B][K-1][3][H*d] fp32, read by the projection kernel, then rewritten
    void* out[3];             // k, v, q: [B][T][H][d]
    float* gate[3];           // theta, eta, alpha: [B][T][H]
    int B, T, D, H, d, K;
};

// Per-token read (every query through the memory as its own token's write
// left it), per stream s (blockIdx.y).  With every gradient of chunk c at its
// start weights (M, S), the weights after token t of the chunk are
//     M_t = pm_t M + ps_t S - sum_{i <= t} c_ti G_i,   G_i = H_i^T Delta_i
// per layer, so a query row's layer product is
//     x_t M_t = pm_t x_t M + ps_t x_t S - sum_{i <= t} C_ti Delta_i,
//     C_ti = c_ti (x_t . H_i),
// the chunk start's products plus a causal b x b correction (the dual form
// of chunked linear attention).  Two kernels:
//   score  C of layer 0 (fp32, [16 ceil(b/16)][bp] per chunk, zeros off
//          the causal triangle and past the chunk) and pm_t, ps_t: they
//          depend on the inputs only, so one launch covers every chunk of
//          the call (blockIdx.z = chunk);
//   layer  one layer's rows: z = pm_t x M + ps_t x S - C Delta, then
//          SiLU(z) (packed [b][N], the next layer's x) or y = z (the last
//          layer).  Layer 0 forms its Delta in place: (Delta_1 W_1^T) .
//          SiLU'(z_0) for depth >= 2, 2 (k M - v) for depth 1; the layers
//          past it read Delta from the store's products and form their C in
//          place (the scores ride in the same K steps as x M and x S).
// c_ti, pm_t, ps_t come from the chunk's gates by the recurrences of the
// momentum and the forgetting (no ratios of running products).
enum { BL_CF0 = 0, BL_CF1 = 1, BL_ROW = 2, BL_CF1T = 3 };   // layout of an fp32 B operand
// where a layer's Delta (and C) come from: BUF Delta from dl and C formed in
// place (the layers past the first); BWD, OUT Delta formed in place and C
// from sc (layer 0)
enum { R3D_BUF = 0, R3D_BWD = 1, R3D_OUT = 2 };
struct R3Args {
    int b, bp, K, N;
    int bl;                   // BL_*: layout of the layer's M and S
    int dk;                   // R3D_*: Delta from dl (BUF), formed from Delta_1 (BWD) or from k M - v (OUT)
    const void* a;            // query rows, packed [b][K] (operand type); chunk z at a + z * a_cs
    long a_ss, a_cs;
    const void* hk;           // key rows of the layer's input, packed [b][K]
    long hk_ss, hk_cs;
    const float* M;           // fp32 M and S of the layer (stream strides m_ss, s_ss)
    const float* S;
    long m_ss, s_ss;
    const float* sc;          // layer 0: C, fp32 [16 ceil(b/16)][bp] (stream stride sc_ss, chunk stride sc_cs)
    long sc_ss, sc_cs;
    float* sco;               // score: where C is written (same strides)
    const void* dl;           // BUF: the key rows' Delta, packed [b][N]
    long dl_ss;
    const void* d1;           // BWD: Delta_1 of the key rows, packed [b][K1]; W_1's M at w1
    long d1_ss;
    int K1;
    const float* w1;
    long w1_ss;
    const float* dsl;         // BWD: SiLU'(z_0) of the key rows [b][dsl_ld]
    long dsl_ss, dsl_ld;
    const void* v;            // OUT: values of tokens vt0 + i
    int vt0;
    const float* theta;       // score, BUF: gates of tokens g0 + z b + t
    const float* eta;
    const float* alpha;
    TokLayout gl;
    int g0;
    float* pq;                // pm_t (t < b) then ps_t, per stream and chunk
    long pq_ss, pq_cs;
    void* out;                // layer, hidden: SiLU(z), packed [b][N] (operand type)
    long out_ss;
    float* y;                 // layer, last: y of tokens yt0 + t
    TokLayout tl;
    int yt0;
};

// ---- the backward through the store (tm_bwd.hip) ----
// Gradients of an outer loss through a call of tm_forward: a forward
// recompute that keeps every chunk-start state (canonical fp32 row-major
// layers, [c][stream][M_1..M_L, S_1..S_L]) and the key rows' activations,
// then a reverse sweep over the chunks.  All arithmetic is fp32.
//
// One matrix operand: element (r, c) of stream s is at
//   p + s * ss + r * ld + c                  (tok = 0, row-major fp32)
//   p + tok_off(tl, s, t0 + r) + c           (tok = 1, token layout; bf16
//                                             storage if bf, else fp32)
struct BMat {
    const void* p;
    long ss, ld;
    int tok, t0, bf;
};
// C[m][n] = sum_k A'[m][k] B'[k][n] per stream (blockIdx.z), with
// A' = A^T (A stored [k][m]) if ta, B' = B^T (B stored [n][k]) if tb.
//   dual 1: a second accumulator from B2 (same shape and transposition);
//   dual 2: both accumulators from B, row k scaled by sk0[k] and sk1[k].
// A second K segment (k2 > 0) adds sum_k A2'[m][k] B2s'[k][n] (same
// transpositions) to the first accumulator.  The epilogue (BE_*) combines
// the accumulators with the auxiliary operands x0, x1 into c0, c1.
enum {
    BE_STORE = 0,   // c0 = acc0
    BE_ACC,         // c0 += acc0
    BE_HID,         // c0 = z = acc0, c1 = SiLU(z)
    BE_OUTK,        // c0 = z = acc0, c1 = 2 (z - x0)
    BE_BWDK,        // c0 = g = acc0, c1 = g * SiLU'(x0)
    BE_QB,          // c0 = acc0 * SiLU'(x0)
    BE_ADDSTORE,    // c0 = acc0 + x0
    BE_HB,          // c1 += (acc0 + x0) * SiLU'(x1)
    BE_GP,          // c0 = -(rs0[r] acc0 + rs1[r] acc1); row partials of acc0 . x0, acc1 . x0
    BE_GQ,          // c0 = -(rs0[r] acc0 + rs1[r] acc1)
    BE_UPD,         // c0 = pa x0 + s0 x1 - acc0, c1 = pe x1 - acc1 (chunk scalars cs)
    BE_ADJ          // c0 = pa c0 + acc0, c1 = pe c1 + s0 c0 (old values); tile partials of
                    // <c0, x0>, <c1, x1>, <c0, x1> (old c0, c1)
};
struct BGemm {
    int m, n, k, k2;
    int ta, tb, dual, epi;
    TokLayout tl;
    BMat A, B, B2, A2, Bs2;
    BMat c0, c1, x0, x1;
    const float* sk0;         // dual 2: per-k scales (sk0 + s * sk_ss + k)
    const float* sk1;
    long sk_ss;
    const float* rs0;         // BE_GP, BE_GQ: per-row scales (rs0 + s * sk_ss + r)
    const float* rs1;
    const float* cs;          // chunk scalars of the stream: cs + s * cs_ss (pa, pe, s0)
    long cs_ss;
    float* part;              // BE_GP: [s][nt_part][2][64] at part + s * part_ss + (tile0 + bx) * 128
    long part_ss;             // BE_ADJ: [s][nt_part][3] at part + s * part_ss + (tile0 + tile) * 3
    int tile0;
    // split K (single-segment products only): splitk workgroups per tile
    // each sum a slice of K into acc (raw accumulators, 2 x 64 x 64 per
    // tile and slice); a second launch sums the slices in order and runs the
    // epilogue.  acc must hold bgemm_acc_floats(m, n, ns, splitk) floats.
    int splitk;
    float* acc;
};
long bgemm_acc_floats(int m, int n, int ns, int splitk);
// The split-K factor launch_bgemm will use for a product of this shape
// (1: no split).
int bgemm_splitk(int m, int n, int k, int k2, int epi, int ns);
hipError_t launch_bgemm(const BGemm& g, int ns, hipStream_t st);

// Element-wise steps of the reverse sweep over one chunk's b rows of width n
// (row-major [b][n]):
//   BW_U  : u = db * SiLU'(z), zb = db * g * SiLU''(z)
//   BW_OUT: zb = 2 db, dv (token layout) = -2 db
enum { BW_U = 0, BW_OUT = 1 };
struct BElem {
    int mode, b, n;
    const float* db;          // db, u, zb: per-stream stride ss
    const float* z;           // z, g: per-stream stride rss
    const float* g;
    float* u;
    float* zb;
    long ss, rss;
    float* dv;                // BW_OUT: token layout tl, tokens t0 ..
    TokLayout tl;
    int t0;
};
hipError_t launch_belem(const BElem& e, int ns, hipStream_t st);

// Per (stream, chunk): the chunk's coefficients from its gates (BC_FWD):
//   A_i = prod_{j>i} (1 - alpha_j), E_i = prod_{j>i} eta_j,
//   r_i = A_i + eta_{i+1} r_{i+1} (r_{b-1} = 1),
//   c_i = theta_i r_i, d_i = theta_i E_i, (p_alpha, p_eta, s0) =
//   ((1 - alpha_0) A_0, eta_0 E_0, eta_0 r_0);
// or (BC_BWD) the adjoint of those definitions: from the partial sums of
// cbar_i = -<Mbar_end, G_i>, dbar_i = -<Sbar_end, G_i>, pbar_alpha =
// <Mbar_end, M_0>, pbar_eta = <Sbar_end, S_0>, s0bar = <Mbar_end, S_0> to
// the gradients of theta, eta, alpha.
enum { BC_FWD = 0, BC_BWD = 1 };
struct BCoef {
    int mode, b, C;
    const float* theta;
    const float* eta;
    const float* alpha;
    TokLayout gl;             // gates: d = 1
    float* cc;                // [s][T]
    float* dc;
    long coef_ss;
    float* cs;                // [s][C][4]
    long cs_ss;
    const float* pgp;         // BC_BWD: row partials [s][c][ngp][2][64]
    int ngp;
    const float* pad;         // BC_BWD: tile partials [s][c][nad][3]
    int nad;
    float* dtheta;            // BC_BWD: gradients, gate layout
    float* deta;
    float* dalpha;
};
hipError_t launch_bcoef(const BCoef& a, int ns, hipStream_t st);

// ---- launchers (tm_r3.hip) ----
hipError_t launch_r3_score(const R3Args& r, int ns, int nchunks, int f32, hipStream_t st);
hipError_t launch_r3_layer(const R3Args& r, int ns, int f32, hipStream_t st);

// ---- launchers (tm_retrieve.hip) ----
// A retrieve pass's product of many query rows (bf16: tokens or packed rows
// times the packed bf16 copy; EPI_HIDDEN without SiLU' and transposes, or
// EPI_OUT with query rows only).
hipError_t launch_rows(const GemmArgs& g, int ns, hipStream_t st);

// Read-only retrieval of a depth-2 memory of width d <= 128 (bf16 operands),
// both layers in one launch: y = SiLU(q W_0) W_1 for rows t0 .. t0+nrows-1
// of every stream.  w: the stream's packed bf16 weights (W_0 packed [h][d],
// W_1 packed [d][h] at w + off1), stream stride w_ss elements.
struct Mlp2Args {
    const void* q;
    float* y;
    const void* w;
    long w_ss, off1;
    TokLayout tl;
    int t0, nrows, d, h;
    int xcd_streams;
};
bool mlp2_fits(int d, int h);
hipError_t launch_mlp2(const Mlp2Args& a, int ns, hipStream_t st);

// Memory-as-context wiring (tm_mac.hip).  Window: out [B][P+2S][D] (operand
// type) = [persistent [P][D]; recalled [B][S][D] fp32, rounded; segment
// [B][S][D]].  Gate: out [B][S][D] fp32 = segment (the attention output y,
// operand type) * recalled (the memory's fp32 read of y).
struct MacArgs {
    const void* persistent;
    const float* recalled;
    const void* segment;
    void* out;
    int B, S, P, D;
};
hipError_t launch_mac_window(const MacArgs& a, int f32, hipStream_t st);
hipError_t launch_mac_gate(const MacArgs& a, int f32, hipStream_t st);

// ---- launchers (tm_project.hip) ----
hipError_t launch_project(const ProjArgs& p, int f32, hipStream_t st);

// ---- launchers (tm_kernels.hip) ----
hipError_t launch_scan(const ScanArgs& a, hipStream_t st);
// fwd: op = 0 bf16 (A bf16, B = bf16 transposed copy), op = 1 fp32 (A fp32,
// B = fp32 master read with stride).  bwd: A fp32 deltas, B fp32 master.
hipError_t launch_fwd(const GemmArgs& g, int ns, int f32, hipStream_t st);
hipError_t launch_bwd(const GemmArgs& g, int ns, int f32, hipStream_t st);
hipError_t launch_first(const FirstArgs& a, int ns, int f32, hipStream_t st);
// export / import convert between the canonical row-major layers and the
// state layout (layer 0 of d0 x h1 and layer 1 of h1 x d1 in accumulator
// order; d1 = 0 for depth 1)
hipError_t launch_shadow(const UpdArgs& u, int ntiles, int ns, hipStream_t st);
// header + M = init (head s % H), S = 0, and the bf16 copy, in one pass
hipError_t launch_state_init(const UpdArgs& u, int ntiles, int ns, const float* init, int H, StateHeader* h,
                             uint64_t hash, int batch, int heads, hipStream_t st);
hipError_t launch_export(const float* M, const float* S, float* dst, long P, int ns, int d0, int h1,
                         int d1, hipStream_t st);
hipError_t launch_import(float* M, float* S, const float* src, long P, int ns, int d0, int h1, int d1,
                         hipStream_t st);
hipError_t launch_header(StateHeader* h, uint64_t hash, int batch, int heads,
                         hipStream_t st);

}  // namespace tmk
