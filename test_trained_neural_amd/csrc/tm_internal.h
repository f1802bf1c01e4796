// Internal structures shared by the C-ABI runtime (tm_api.hip) and the
// kernels (tm_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tmk {

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

// Token-major arrays [batch][Tc][H][d]; gates use d = 1.
struct TokLayout {
    int Tc, H, d;
};

enum { EPI_HIDDEN = 0, EPI_OUT = 1, EPI_BWD = 2 };

// One matrix product of the chunk forward / backward, per stream s
// (blockIdx.z):  Z[r][n] = sum_k A[r][k] B[k][n], r < nrows, n < N, k < K.
// Rows r < n0 are queries, rows r >= n0 keys (t = r - n0 is the key's token
// inside the chunk); the backward has key rows only (n0 = 0).
struct GemmArgs {
    int nrows, N, K;
    // A rows.  amode 0: rows r < n0 are tokens (at0 + r) of a0, rows r >= n0
    // tokens (at1 + r - n0) of a1, both in the token layout tl.  amode 1:
    // row r at a0 + s*a_ss + r*a_ld.
    const void* a0;
    const void* a1;
    int n0, at0, at1, amode;
    long a_ss, a_ld;
    // B element (k, n) at b + s*b_ss + n*b_ldn + k*b_ldk.
    const void* b;
    long b_ss, b_ldn, b_ldk;
    TokLayout tl;
    int epi;
    // EPI_HIDDEN: act[r][n] = SiLU(z) (operand type); key rows also
    //             dsl[t][n] = SiLU'(z) and the transposed copy ht[n][t] = act.
    // EPI_OUT   : query rows: y at token (yt0 + r) = z; key rows:
    //             dlt[t][n] = Delta = 2 (z - v at token (vt0 + t)).
    // EPI_BWD   : dlt[t][n] = Delta = z * dsl[t][n].
    // OUT / BWD also write the theta-weighted transposed deltas
    //             dct[n][t] = c_t Delta,  ddt[n][t] = d_t Delta  (operand type).
    // Transposed arrays have rows of bp (>= chunk, multiple of 32) tokens.
    void* act;
    long act_ss, act_ld;
    float* dsl;
    long dsl_ss, dsl_ld;
    float* dlt;
    long dlt_ss, dlt_ld;
    void* dltb;               // optional operand-type copy of dlt (same layout)
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
    void* Wt;                 // bf16 transposed copy, [d_out][d_in] per layer
    const void* at[MAXL];     // at[l]: layer l's input rows transposed, [d_in][bp]
    long at_ss[MAXL];
    const void* dct[MAXL];    // (c Delta_l)^T, [d_out][bp]
    const void* ddt[MAXL];    // (d Delta_l)^T
    long dt_ss[MAXL];
    const float* cs;          // per-chunk scalars (p_alpha, p_eta, s0, 0)
    long cs_ss;
    int chunk;
    int* flag;
    void* wr_next;            // if set: row-major copy (operand type) of layer 1's new weights
    long wr_ss;
};

// First-layer part of chunk step c (one launch; it runs concurrently with
// the update tiles of layers 1.. for chunk c-1).  One workgroup per JW-wide
// column block of the first weight matrix W_0 (full height):
//   * if do_update: chunk c-1's update of those columns.  The first layer's
//     Delta for the columns is formed in place (depth >= 2) from layer 1's
//     Delta and a row-major copy of layer 1's chunk-start weights, or read
//     back (depth 1); theta-weighted, reduced against the chunk's keys and
//     folded into M and S (and the bf16 copy of W_0);
//   * if do_fwd: chunk c's first-layer forward of [queries of chunk c-1;
//     keys of chunk c] through the freshly written columns.
// K is split over the workgroup's 4 waves for the backward and the forward
// products (partial tiles summed in LDS), so no wave walks a long chain of
// dependent loads.
constexpr int JW = 16;

struct FirstArgs {
    UpdArgs u;                // layers, state, chunk scalars, flag
    int dim, h1, nb1;
    int do_update, do_fwd, nq, nk;
    int chunk_prev;
    const void* kt_prev;      // keys of chunk c-1 transposed, [dim][bp]
    long kt_ss;
    const void* dlt2;         // Delta of layer 1 for chunk c-1 (operand type), [b][dout1]
    long dlt2_ss;
    const void* wr_prev;      // layer 1's weights at chunk c-1's start, [h1][dout1]
    long wr_ss;
    float* dsl1;              // SiLU'(z) of layer 0: read (chunk c-1), then written (chunk c)
    long dsl1_ss;
    const float* cc_prev;     // coefficients of chunk c-1's tokens
    const float* dc_prev;
    const float* cc_cur;      // coefficients of chunk c's tokens
    const float* dc_cur;
    long coef_ss;
    const void* xq;           // queries (rows r < nq are tokens tq0 + r)
    const void* xk;           // keys (rows r >= nq are tokens tk0 + r - nq)
    TokLayout tl;
    int tq0, tk0;
    void* act;                // layer-0 activations of the rows, [2b][h1]
    long act_ss;
    void* ht1;                // key rows of act transposed, [h1][bp]
    long ht_ss;
    // depth 1: the first layer is the last one
    float* y;
    const void* v;
    void* dct1;               // (c Delta)^T, (d Delta)^T of layer 0, [h1][bp]
    void* ddt1;
    long dt1_ss;
};

// Per call: the coefficient scan of every (stream, chunk) and the keys of
// every chunk transposed to kt[s][chunk][d][bp].
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
    TokLayout ktl;
    void* kt;
    int bp, kt_f32;
    int scan_blocks;          // blocks [0, scan_blocks) scan, the rest transpose
    // refresh of the row-major copy of layer 1's weights (depth >= 2)
    const float* w1_master;   // M of layer 1, stream stride w1_ss
    void* w1_copy;            // operand-type copy, same layout
    long w1_ss, w1_n;         // per-stream stride, elements per stream
    int tr_blocks;            // transpose blocks; copy blocks follow them
};

// ---- launchers (tm_kernels.hip) ----
hipError_t launch_scan(const ScanArgs& a, hipStream_t st);
// fwd: op = 0 bf16 (A bf16, B = bf16 transposed copy), op = 1 fp32 (A fp32,
// B = fp32 master read with stride).  bwd: A fp32 deltas, B fp32 master.
hipError_t launch_fwd(const GemmArgs& g, int ns, int f32, hipStream_t st);
hipError_t launch_bwd(const GemmArgs& g, int ns, int f32, hipStream_t st);
hipError_t launch_update(const UpdArgs& u, int ntiles, int ns, int f32, hipStream_t st);
hipError_t launch_first(const FirstArgs& a, int ns, int f32, hipStream_t st);
// update tiles [tile0, tile0 + ntiles) of every stream
hipError_t launch_update_range(const UpdArgs& u, int tile0, int ntiles, int ns, int f32, hipStream_t st);
hipError_t launch_init(float* M, float* S, const float* init, long P, int H, int ns,
                       hipStream_t st);
hipError_t launch_shadow(const UpdArgs& u, int ntiles, int ns, hipStream_t st);
hipError_t launch_export(const float* M, const float* S, float* dst, long P, int ns,
                         hipStream_t st);
hipError_t launch_import(float* M, float* S, const float* src, long P, int ns,
                         hipStream_t st);
hipError_t launch_header(StateHeader* h, uint64_t hash, int batch, int heads,
                         hipStream_t st);

}  // namespace tmk
