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
};

// ---- launchers (tm_kernels.hip) ----
hipError_t launch_scan(const ScanArgs& a, hipStream_t st);
// fwd: op = 0 bf16 (A bf16, B = bf16 transposed copy), op = 1 fp32 (A fp32,
// B = fp32 master read with stride).  bwd: A fp32 deltas, B fp32 master.
hipError_t launch_fwd(const GemmArgs& g, int ns, int f32, hipStream_t st);
hipError_t launch_bwd(const GemmArgs& g, int ns, int f32, hipStream_t st);
hipError_t launch_update(const UpdArgs& u, int ntiles, int ns, int f32, hipStream_t st);
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
