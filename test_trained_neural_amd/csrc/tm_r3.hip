// Per-token read of the Titans memory: every query of a chunk through the
// weights as its own token's write left them ("Attack of the Titans", the
// long-term memory section: a linear-attention output is a lookup in a matrix
// memory updated at every step; Technical Details / Parallel training: every
// gradient of a chunk sits at the chunk-start weights; "Titans, explained",
// steps 3-6).
//
// Unrolling S_u = eta_u S_{u-1} - theta_u G_u and M_u = (1 - alpha_u) M_{u-1}
// + S_u from the chunk start (M, S) to token t gives
//     M_t = pm_t M + ps_t S - sum_{i <= t} c_ti G_i,
//     pm_t = prod_{j <= t} (1 - alpha_j),
//     ps_t = sum_{u <= t} prod_{u < j <= t} (1 - alpha_j) prod_{j <= u} eta_j,
//     c_ti = theta_i sum_{i <= u <= t} prod_{u < j <= t} (1 - alpha_j) prod_{i < j <= u} eta_j,
// and with G_i = H_i^T Delta_i per layer, a query row's product with M_t is
// the chunk start's products plus a causal b x b correction:
//     x_t M_t = pm_t x_t M + ps_t x_t S - sum_{i <= t} c_ti (x_t . H_i) Delta_i.
// The three launch kinds (R3_DELTA, R3_SCORE, R3_LAYER) share one kernel:
// a workgroup of RW waves owns one 16-column block of the output for all of
// the chunk's rows and splits the 32-deep K steps over its waves; the
// partial tiles are summed in LDS in wave order.  Matrix products run on
// MFMA with fp32 accumulation; the state's fp32 M and S are rounded to the
// operand type on load.
#include "tm_device.h"

namespace tmk {

constexpr int RW = 4;      // waves of a workgroup
constexpr int RMR = 4;     // 16-row blocks: chunks of up to 64 tokens
constexpr int RTP = 17;    // padded LDS row of a partial tile
constexpr int R3_LDS = (RW * 3 * 16 * RMR * RTP + 3 * 64) * 4;

// 8 consecutive K values k0 .. k0 + 7 (k0 a multiple of 8) of column n of an
// fp32 B operand held in a layer's state layout.
template <int BL>
__device__ __forceinline__ f32x8 ldB(const float* B, int k0, int n, int K, int N) {
    if constexpr (BL == BL_CF0) {
        // B = W_0 [K][N] in accumulator order: 4 consecutive rows of a column
        // are one float4, the next 4 one 16-lane group (64 floats) later
        const float* p = B + cf0(k0, n, K >> 4);
        const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 64);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else if constexpr (BL == BL_CF1T) {
        // B[k][n] = W_1[n][k] (W_1 is [N][K]): 8 consecutive outputs of one input
        return ld8w1(B + cf1(n, k0, K >> 4));
    } else if constexpr (BL == BL_CF1) {
        // B = W_1 [K][N] in its accumulator order: consecutive inputs of one
        // output are 4 floats apart
        const float* p = B + cf1(k0, n, N >> 4);
        f32x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = p[4 * e];
        return u;
    } else {
        // row-major [K][N]
        f32x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = B[(long)(k0 + e) * N + n];
        return u;
    }
}

template <class OP, int BL, int KIND>
__global__ __launch_bounds__(RW * 64) void r3_kernel(R3Args r) {
    typedef typename Frag<OP>::T F;
    extern __shared__ __attribute__((aligned(16))) float red[];   // [RW][3][16 RMR][RTP], gates [3][64]
    float* gt = red + RW * 3 * 16 * RMR * RTP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.y;
    const int nb = blockIdx.x;                 // the workgroup's 16-column block
    const int n = nb * 16 + (lane & 15);       // this lane's B column
    const int kofs = 8 * (lane >> 4);
    const int b = r.b;
    const int mr = (b + 15) >> 4;
    const int nsk = r.K >> 5;
    constexpr int nseg = KIND == R3_LAYER ? 2 : 1;   // x M (and x S)
    const int nsb = KIND == R3_LAYER ? r.bp >> 5 : 0;  // C Delta
    const int nst = nseg * nsk + nsb;

    f32x4 acc[3][RMR];
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
        for (int m = 0; m < RMR; ++m) acc[g][m] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const OP* A = reinterpret_cast<const OP*>(r.a) + (long)s * r.a_ss;
    for (int st = wave; st < nst; st += RW) {
        if (st < nseg * nsk) {
            const int seg = st >= nsk ? 1 : 0;
            const int ks = st - seg * nsk;
            F bv;
            if constexpr (KIND == R3_SCORE) {
                // the key rows are the B columns; a block past the rows reads
                // the last valid block (its outputs are zeroed below)
                const int kb = nb < mr ? nb : mr - 1;
                bv = cvt<OP>(ld8(reinterpret_cast<const OP*>(r.hk) + (long)s * r.hk_ss + pkf(kb, ks, nsk, lane)));
            } else {
                const float* B = (seg ? r.S : r.M) + (long)s * r.ms_ss;
                bv = cvt<OP>(ldB<BL>(B, ks * 32 + kofs, n, r.K, r.N));
            }
#pragma unroll
            for (int m = 0; m < RMR; ++m) {
                if (m < mr) {
                    const F av = cvt<OP>(ld8(A + pkf(m, ks, nsk, lane)));
                    if (seg) mma(acc[1][m], av, bv);
                    else mma(acc[0][m], av, bv);
                }
            }
        } else {
            // the correction: C (packed [b][bp]) times the keys' Delta
            // (packed [b][N]); Delta rows past the chunk contribute zeros
            const int ks = st - nseg * nsk;
            const OP* D = reinterpret_cast<const OP*>(r.dl) + (long)s * r.dl_ss;
            F bv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = ks * 32 + kofs + e;
                const OP x = D[pk(i < b ? i : b - 1, n, r.N >> 5)];
                bv[e] = i < b ? x : (OP)0.0f;
            }
            const OP* Cs = reinterpret_cast<const OP*>(r.sc) + (long)s * r.sc_ss;
#pragma unroll
            for (int m = 0; m < RMR; ++m)
                if (m < mr) mma(acc[2][m], cvt<OP>(ld8(Cs + pkf(m, ks, nsb, lane))), bv);
        }
    }

    float* mine = red + wave * (3 * 16 * RMR * RTP);
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
        for (int m = 0; m < RMR; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mine[(g * 16 * RMR + m * 16 + 4 * (lane >> 4) + e) * RTP + (lane & 15)] = acc[g][m][e];
    if (KIND == R3_SCORE && tid < b) {
        const long go = tok_off(r.gl, s, r.g0 + tid);
        gt[tid] = r.theta[go];
        gt[64 + tid] = r.eta[go];
        gt[128 + tid] = r.alpha[go];
    }
    __syncthreads();

    const int rows = 16 * mr;
    for (int idx = tid; idx < rows * 16; idx += RW * 64) {
        const int t = idx >> 4, cl = idx & 15, col = nb * 16 + cl;
        float z[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < (KIND == R3_LAYER ? 3 : 1); ++g)
#pragma unroll
            for (int w = 0; w < RW; ++w) z[g] += red[(w * 3 * 16 * RMR + g * 16 * RMR + t) * RTP + cl];
        if constexpr (KIND == R3_SCORE) {
            // C[t][i] = c_ti (x_t . H_i) for i <= t < b; zeros elsewhere (the
            // padding of both dimensions included).  c_ti by the recurrence
            // w_i = A_i + eta_{i+1} w_{i+1}, A_i = prod_{i < j <= t} (1 - alpha_j),
            // from w_t = 1 down to i
            float val = 0.f;
            if (t < b && col <= t) {
                float Ap = 1.f, w = 1.f;
                for (int j = t; j > col; --j) {
                    Ap *= 1.0f - gt[128 + j];
                    w = __builtin_fmaf(gt[64 + j], w, Ap);
                }
                val = gt[col] * w * z[0];
            }
            reinterpret_cast<OP*>(r.out)[(long)s * r.out_ss + pk(t, col, r.bp >> 5)] = (OP)val;
        } else if (t < b) {
            if constexpr (KIND == R3_DELTA) {
                float d;
                if (r.v) {
                    // depth 1: the output layer's Delta = 2 (k M - v)
                    d = 2.0f * (z[0] - load1<OP>(r.v, tok_off(r.tl, s, r.vt0 + t) + col));
                } else {
                    d = z[0] * r.dsl[(long)s * r.dsl_ss + (long)t * r.dsl_ld + col];
                }
                reinterpret_cast<OP*>(r.out)[(long)s * r.out_ss + pk(t, col, r.N >> 5)] = (OP)d;
            } else {
                const float pm = r.pq[(long)s * r.pq_ss + t], ps = r.pq[(long)s * r.pq_ss + b + t];
                const float zz = __builtin_fmaf(pm, z[0], __builtin_fmaf(ps, z[1], -z[2]));
                if (r.y) {
                    r.y[tok_off(r.tl, s, r.yt0 + t) + col] = zz;
                } else {
                    reinterpret_cast<OP*>(r.out)[(long)s * r.out_ss + pk(t, col, r.N >> 5)] = (OP)(zz * sigmoid(zz));
                }
            }
        }
    }
    if (KIND == R3_SCORE && r.pq && nb == 0 && tid < b) {
        // pm_t and ps_t by the forward recurrences of the forgetting and the
        // momentum: ps_t = (1 - alpha_t) ps_{t-1} + prod_{j <= t} eta_j
        float pm = 1.f, ps = 0.f, E = 1.f;
        for (int j = 0; j <= tid; ++j) {
            pm *= 1.0f - gt[128 + j];
            E *= gt[64 + j];
            ps = __builtin_fmaf(1.0f - gt[128 + j], ps, E);
        }
        r.pq[(long)s * r.pq_ss + tid] = pm;
        r.pq[(long)s * r.pq_ss + b + tid] = ps;
    }
}

template <class OP, int BL, int KIND>
static void launch_as(const R3Args& r, int ns, hipStream_t st) {
    const int nblk = KIND == R3_SCORE ? r.bp / 16 : r.N / 16;
    hipLaunchKernelGGL((r3_kernel<OP, BL, KIND>), dim3(nblk, ns), dim3(RW * 64), R3_LDS, st, r);
}

template <class OP>
static hipError_t launch_op(const R3Args& r, int kind, int ns, hipStream_t st) {
    if (kind == R3_SCORE) {
        launch_as<OP, BL_ROW, R3_SCORE>(r, ns, st);
    } else if (kind == R3_DELTA) {
        if (r.bl == BL_CF0) launch_as<OP, BL_CF0, R3_DELTA>(r, ns, st);
        else if (r.bl == BL_CF1T) launch_as<OP, BL_CF1T, R3_DELTA>(r, ns, st);
        else return hipErrorInvalidValue;
    } else if (kind == R3_LAYER) {
        if (r.bl == BL_CF0) launch_as<OP, BL_CF0, R3_LAYER>(r, ns, st);
        else if (r.bl == BL_CF1) launch_as<OP, BL_CF1, R3_LAYER>(r, ns, st);
        else if (r.bl == BL_ROW) launch_as<OP, BL_ROW, R3_LAYER>(r, ns, st);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_r3(const R3Args& r, int kind, int ns, int f32, hipStream_t st) {
    // the shapes the kernel assumes: a chunk of 1 .. 64 tokens, bp = b
    // rounded up to 32, K a multiple of 32 and N of 16 (every layer width is
    // a multiple of 32)
    if (r.b < 1 || r.b > 16 * RMR || r.bp != (r.b + 31) / 32 * 32 || r.K < 32 || r.K % 32 != 0 ||
        r.N < 16 || r.N % 16 != 0 || ns < 1 || ns > 65535)
        return hipErrorInvalidValue;
    return f32 ? launch_op<float>(r, kind, ns, st) : launch_op<bf16>(r, kind, ns, st);
}

}  // namespace tmk
