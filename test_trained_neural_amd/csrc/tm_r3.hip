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
//
// Both kernels give a workgroup of 8 (or 16) waves one 16-column block of the output
// for all of the chunk's rows and split the 32-deep K steps over the waves in
// contiguous slices; each wave keeps its slice's operands in flight through a
// register ring of PF steps (steps past the slice re-load a valid address and
// are masked), and the partial tiles are summed in LDS in wave order.  Matrix
// products run on MFMA with fp32 accumulation (the state's fp32 M and S
// rounded to the operand type on load); the b x b correction and the Delta
// of layer 0 stay in fp32.
#include "tm_device.h"

namespace tmk {

constexpr int RW = 8;      // waves of a workgroup
constexpr int RMR = 4;     // 16-row blocks: chunks of up to 64 tokens
constexpr int RTP = 17;    // padded LDS row of a 16-column tile
constexpr int RCP = 68;    // LDS row of C and of Delta transposed (16-byte aligned)
constexpr int r3_score_lds(int sw) { return (sw * 64 * RTP + 3 * 64 + 64 * RTP) * 4; }
constexpr int R3_STAGE = 1024;   // floats of a wave's staging area (W_1's M and S blocks of one K step)
constexpr int R3_NSC = RMR * (RMR + 1) / 2;   // score tiles on and below the diagonal
constexpr int R3_LAYER_LDS = (2 * RW * 64 * RTP + RW * R3_STAGE + 64 * RCP + 16 * RCP + 2 * 64 + 3 * 64) * 4;
static_assert(RW * 64 * RTP + RW * R3_STAGE >= (RW / 2) * R3_NSC * 256, "score reduction space");

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

// A wave's contiguous slice [kb, ke) of nsk K steps; klast is a valid step
// for the ring's masked re-loads.
struct Slice {
    int spw, kb, ke, klast;
    __device__ Slice(int nsk, int wave, int nw) {
        spw = (nsk + nw - 1) / nw;
        kb = wave * spw;
        ke = min(nsk, kb + spw);
        klast = max(ke - 1, 0);
        if (klast >= nsk) klast = nsk - 1;
    }
};

// C = c_ti (x_t . H_i) of one layer for the 16 key columns i of block
// blockIdx.x and every query row t; chunk blockIdx.z of the launch.  SW
// waves (16 for long K: a chunk's launch has only ceil(b/16) workgroups per
// stream).
template <class OP, int SW>
__global__ __launch_bounds__(SW * 64) void r3_score_kernel(R3Args r) {
    typedef typename Frag<OP>::T F;
    constexpr int PF = sizeof(OP) == 2 ? 4 : 2;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* part = lds;                      // [SW][64][RTP]
    float* gt = part + SW * 64 * RTP;       // theta, eta, alpha of the chunk's tokens
    float* cf = gt + 3 * 64;                // [64][RTP]: c_ti for the block's 16 i
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.y, z = blockIdx.z, ib = blockIdx.x;
    const int b = r.b, mr = (b + 15) >> 4, nsk = r.K >> 5;
    const int hb = ib < mr ? ib : mr - 1;   // a block past the keys reads the last one (outputs zeroed)
    const OP* X = reinterpret_cast<const OP*>(r.a) + (long)s * r.a_ss + (long)z * r.a_cs;
    const OP* H = reinterpret_cast<const OP*>(r.hk) + (long)s * r.hk_ss + (long)z * r.hk_cs;
    float g[3] = {0.f, 0.f, 0.f};
    if (tid < b) {
        const long go = tok_off(r.gl, s, r.g0 + z * b + tid);
        g[0] = r.theta[go];
        g[1] = r.eta[go];
        g[2] = r.alpha[go];
    }
    const Slice sl(nsk, wave, SW);
    F xa[PF][RMR], hf[PF];
    auto load = [&](int p, int k) {
#pragma unroll
        for (int m = 0; m < RMR; ++m) xa[p][m] = ld8(X + pkf(m < mr ? m : mr - 1, k, nsk, lane));
        hf[p] = ld8(H + pkf(hb, k, nsk, lane));
    };
    f32x4 acc[RMR];
#pragma unroll
    for (int m = 0; m < RMR; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, min(sl.kb + p, sl.klast));
    for (int k = sl.kb; k < sl.kb + sl.spw; k += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const F bv = keep_if(hf[p], k + p < sl.ke);
#pragma unroll
            for (int m = 0; m < RMR; ++m) mma(acc[m], xa[p][m], bv);
            load(p, min(k + p + PF, sl.klast));
        }
    }
    float* mine = part + wave * 64 * RTP;
#pragma unroll
    for (int m = 0; m < RMR; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[(m * 16 + 4 * (lane >> 4) + e) * RTP + (lane & 15)] = acc[m][e];
    if (tid < b) {
        gt[tid] = g[0];
        gt[64 + tid] = g[1];
        gt[128 + tid] = g[2];
    }
    __syncthreads();
    const int i0 = ib * 16;
    if (tid < 64) {
        // row t of the coefficients: c_ti = theta_i w_i by w_i = A_i +
        // eta_{i+1} w_{i+1}, A_i = prod_{i < j <= t} (1 - alpha_j), from
        // w_t = A_t = 1 down (a fixed trip count: the gates are read the
        // same way by every lane, the rows differ by a select)
        // (every lane takes the same steps: rows above t hold the start
        // value, so the gate reads are unconditional and run ahead; no store
        // inside the walk)
        const int t = tid;
        float Ap = 1.f, wv = 1.f, cr[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) cr[e] = 0.f;
#pragma unroll
        for (int i = 63; i >= 0; --i) {
            if (i + 1 < 64) {
                const float ap = Ap * (1.0f - gt[128 + i + 1]);
                const float w = __builtin_fmaf(gt[64 + i + 1], wv, ap);
                Ap = i < t ? ap : 1.0f;
                wv = i < t ? w : 1.0f;
            }
            const float c = gt[i] * wv;
            cr[i & 15] = ((i >> 4) == ib && i <= t && t < b) ? c : cr[i & 15];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) cf[t * RTP + e] = cr[e];
    }
    if (r.pq && ib == 0 && tid >= 64 && tid < 64 + b) {
        // pm_t and ps_t by the forward recurrences of the forgetting and the
        // momentum: ps_t = (1 - alpha_t) ps_{t-1} + prod_{j <= t} eta_j
        const int t = tid - 64;
        float pm = 1.f, ps = 0.f, E = 1.f;
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const bool on = j <= t;
            const float a1 = 1.0f - gt[128 + j];
            const float e1 = E * gt[64 + j];
            pm = on ? pm * a1 : pm;
            ps = on ? __builtin_fmaf(a1, ps, e1) : ps;
            E = on ? e1 : E;
        }
        float* pq = r.pq + (long)s * r.pq_ss + (long)z * r.pq_cs;
        pq[t] = pm;
        pq[b + t] = ps;
    }
    __syncthreads();
    float* C = r.sco + (long)s * r.sc_ss + (long)z * r.sc_cs;
    for (int idx = tid; idx < 16 * mr * 16; idx += SW * 64) {
        const int t = idx >> 4, cl = idx & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < SW; ++w) sum += part[(w * 64 + t) * RTP + cl];
        // zeros past the causal triangle and the chunk (a select: rows of
        // the operands past the chunk are not defined)
        C[t * r.bp + i0 + cl] = (t < b && i0 + cl <= t) ? cf[t * RTP + cl] * sum : 0.f;
    }
}

// One layer's query rows for the 16 output columns of block blockIdx.x.
template <class OP, int BL, int DK>
__global__ __launch_bounds__(RW * 64) void r3_layer_kernel(R3Args r) {
    typedef typename Frag<OP>::T F;
    // ring depth within the register budget (the row-major layout's strided
    // loads carry an address per value; the key rows ride in the ring of the
    // layers that form their scores in place)
    constexpr int PF = sizeof(OP) == 2 ? ((DK == R3D_BWD && BL != BL_ROW) ? 3 : 2) : (DK == R3D_BUF ? 1 : 2);
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* zp = lds;                        // [RW][64][RTP]: pm x M + ps x S, per wave
    float* dp = zp + RW * 64 * RTP;         // [RW][64][RTP]: the Delta products, per wave
    float* stage = dp + RW * 64 * RTP;      // [RW][R3_STAGE]: W_1's blocks on their way to B fragments
    float* sred = dp;                       // (after the products) the score tiles' reduction: dp, stage
    float* cT = stage + RW * R3_STAGE;      // [64][RCP]: C
    float* dT = cT + 64 * RCP;              // [16][RCP]: Delta of the block's columns, transposed
    float* pmps = dT + 16 * RCP;            // pm_t, then ps_t
    float* gt = pmps + 2 * 64;              // BUF: theta, eta, alpha of the chunk's tokens
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.y, nb = blockIdx.x;
    const int n = nb * 16 + (lane & 15), kofs = 8 * (lane >> 4);
    const int b = r.b, mr = (b + 15) >> 4, nsk = r.K >> 5, nbp4 = r.bp >> 2;

    // the epilogue's operands, requested first: pm_t, ps_t, C (layer 0; the
    // layers past it form C in place from the gates) and the Delta of the
    // key rows (from memory for the layers past the first)
    if (tid < b) {
        pmps[tid] = r.pq[(long)s * r.pq_ss + tid];
        pmps[64 + tid] = r.pq[(long)s * r.pq_ss + b + tid];
        if constexpr (DK == R3D_BUF) {
            const long go = tok_off(r.gl, s, r.g0 + tid);
            gt[tid] = r.theta[go];
            gt[64 + tid] = r.eta[go];
            gt[128 + tid] = r.alpha[go];
        }
    }
    f32x4 cv[2];
    if constexpr (DK != R3D_BUF) {
        const float* Cg = r.sc + (long)s * r.sc_ss;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + q * RW * 64, t = idx / nbp4;
            cv[q] = *reinterpret_cast<const f32x4*>(Cg + (long)(t < 16 * mr ? t : 0) * r.bp + (idx % nbp4) * 4);
        }
    }
    // (BWD, OUT: SiLU'(z_0) or v of the Delta epilogue's elements)
    float dv[2] = {0.f, 0.f};
    if constexpr (DK == R3D_BWD || DK == R3D_OUT) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + q * RW * 64, i = idx >> 4, col = nb * 16 + (idx & 15);
            const int ic = i < b ? i : b - 1;
            if constexpr (DK == R3D_BWD)
                dv[q] = r.dsl[(long)s * r.dsl_ss + (long)ic * r.dsl_ld + col];
            else
                dv[q] = load1<OP>(r.v, tok_off(r.tl, s, r.vt0 + ic) + col);
        }
    }
    if constexpr (DK == R3D_BUF) {
        const OP* D = reinterpret_cast<const OP*>(r.dl) + (long)s * r.dl_ss;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + q * RW * 64, i = idx >> 4;
            const float x = (float)D[pk(i < b ? i : b - 1, nb * 16 + (idx & 15), r.N >> 5)];
            dv[q] = i < b ? x : 0.f;
        }
    }

    const OP* X = reinterpret_cast<const OP*>(r.a) + (long)s * r.a_ss;
    const OP* H = reinterpret_cast<const OP*>(r.hk) + (long)s * r.hk_ss;
    const float* Ms = r.M + (long)s * r.m_ss;
    const float* Ss = r.S + (long)s * r.s_ss;
    const Slice sl(nsk, wave, RW);
    F xa[PF][RMR], ha[PF][RMR];
    f32x8 bm[PF], bs[PF];
    auto load = [&](int p, int k) {
#pragma unroll
        for (int m = 0; m < RMR; ++m) {
            const int mm = m < mr ? m : mr - 1;
            xa[p][m] = ld8(X + pkf(mm, k, nsk, lane));
            if constexpr (DK != R3D_BWD) ha[p][m] = ld8(H + pkf(mm, k, nsk, lane));
        }
        if constexpr (BL == BL_CF1) {
            // the step's two 16 x 16 blocks (inputs 32k .. 32k+31, the
            // block's 16 outputs) are 1 KB each, contiguous: one float4 per
            // lane and block, rearranged through LDS before use
            const long o0 = ((long)(2 * k) * (r.N >> 4) + nb) * 256 + 4 * lane;
            const long o1 = o0 + (long)(r.N >> 4) * 256;
            const f32x4 m0 = *reinterpret_cast<const f32x4*>(Ms + o0), m1 = *reinterpret_cast<const f32x4*>(Ms + o1);
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(Ss + o0), s1 = *reinterpret_cast<const f32x4*>(Ss + o1);
            bm[p] = __builtin_shufflevector(m0, m1, 0, 1, 2, 3, 4, 5, 6, 7);
            bs[p] = __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            bm[p] = ldB<BL>(Ms, k * 32 + kofs, n, r.K, r.N);
            bs[p] = ldB<BL>(Ss, k * 32 + kofs, n, r.K, r.N);
        }
    };
    // layer 0 of a deeper memory: Delta_0 = (Delta_1 W_1^T) . SiLU'(z_0) of
    // the block's columns, over K1 = layer 1's outputs
    const int nsk1 = DK == R3D_BWD ? r.K1 >> 5 : 1;
    const Slice s1(nsk1, wave, RW);
    const OP* D1 = reinterpret_cast<const OP*>(r.d1) + (long)s * r.d1_ss;
    const float* W1 = r.w1 + (long)s * r.w1_ss;
    constexpr int PF1 = 2;   // (the Delta_0 ring is in flight beside the main one)
    F da[PF1][RMR];
    f32x8 wb[PF1];
    auto loadd = [&](int p, int k) {
#pragma unroll
        for (int m = 0; m < RMR; ++m) da[p][m] = ld8(D1 + pkf(m < mr ? m : mr - 1, k, nsk1, lane));
        wb[p] = ldB<BL_CF1T>(W1, k * 32 + kofs, n, r.K1, r.N);
    };

    f32x4 aM[RMR], aS[RMR], aD[RMR], aC[R3_NSC];
#pragma unroll
    for (int m = 0; m < RMR; ++m) aM[m] = aS[m] = aD[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < R3_NSC; ++q) aC[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, min(sl.kb + p, sl.klast));
    if constexpr (DK == R3D_BWD) {
#pragma unroll
        for (int p = 0; p < PF1; ++p) loadd(p, min(s1.kb + p, s1.klast));
    }
    for (int k = sl.kb; k < sl.kb + sl.spw; k += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const bool live = k + p < sl.ke;
            f32x8 rm = bm[p], rs = bs[p];
            if constexpr (BL == BL_CF1) {
                // slot l of a block holds outputs 4 (l / 16) .. + 3 of input
                // l % 16; this lane's B fragment is output n, inputs kofs .. + 7
                float* st = stage + wave * R3_STAGE;
                *reinterpret_cast<f32x4*>(st + 4 * lane) = __builtin_shufflevector(rm, rm, 0, 1, 2, 3);
                *reinterpret_cast<f32x4*>(st + 256 + 4 * lane) = __builtin_shufflevector(rm, rm, 4, 5, 6, 7);
                *reinterpret_cast<f32x4*>(st + 512 + 4 * lane) = __builtin_shufflevector(rs, rs, 0, 1, 2, 3);
                *reinterpret_cast<f32x4*>(st + 768 + 4 * lane) = __builtin_shufflevector(rs, rs, 4, 5, 6, 7);
                __builtin_amdgcn_wave_barrier();
                const int nl = lane & 15, src = 256 * (kofs >> 4) + 4 * ((kofs & 15) + 16 * (nl >> 2)) + (nl & 3);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    rm[e] = st[src + 4 * e];
                    rs[e] = st[512 + src + 4 * e];
                }
                __builtin_amdgcn_wave_barrier();
            }
            const F vm = cvt<OP>(keep_if(rm, live));
            const F vs = cvt<OP>(keep_if(rs, live));
#pragma unroll
            for (int m = 0; m < RMR; ++m) {
                mma(aM[m], xa[p][m], vm);
                mma(aS[m], xa[p][m], vs);
                if constexpr (DK == R3D_OUT) mma(aD[m], ha[p][m], vm);
            }
            if constexpr (DK == R3D_BUF) {
                // the scores x_t . H_i of query block m and key block j <= m
                const F* kf = ha[p];
#pragma unroll
                for (int m = 0; m < RMR; ++m)
#pragma unroll
                    for (int j = 0; j <= m; ++j) mma(aC[m * (m + 1) / 2 + j], xa[p][m], keep_if(kf[j], live));
            }
            load(p, min(k + p + PF, sl.klast));
        }
    }
    if constexpr (DK == R3D_BWD) {
        for (int k = s1.kb; k < s1.kb + s1.spw; k += PF1) {
#pragma unroll
            for (int p = 0; p < PF1; ++p) {
                const F vw = cvt<OP>(keep_if(wb[p], k + p < s1.ke));
#pragma unroll
                for (int m = 0; m < RMR; ++m) mma(aD[m], da[p][m], vw);
                loadd(p, min(k + p + PF1, s1.klast));
            }
        }
    }

    // C (or, formed in place, the score tiles) and the loaded Delta to LDS
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + q * RW * 64, t = idx / nbp4, c4 = (idx % nbp4) * 4;
        if constexpr (DK != R3D_BUF) {
            if (t < 16 * mr) {
#pragma unroll
                for (int e = 0; e < 4; ++e) cT[t * RCP + c4 + e] = cv[q][e];
            }
        }
        if constexpr (DK == R3D_BUF) dT[(idx & 15) * RCP + (idx >> 4)] = dv[q];
    }
    __syncthreads();   // pm_t, ps_t, the gates visible; every wave past its products
    if constexpr (DK == R3D_BUF) {
        // the score tiles summed over the waves in two rounds (waves 4..7
        // store, waves 0..3 add theirs; the slots sum in wave order below),
        // while wave 4 walks the coefficient rows into C's place
        f32x4* slot = reinterpret_cast<f32x4*>(sred) + (wave % (RW / 2)) * R3_NSC * 64 + lane;
        if (wave >= RW / 2) {
#pragma unroll
            for (int q = 0; q < R3_NSC; ++q) slot[q * 64] = aC[q];
        }
        __syncthreads();
        if (wave < RW / 2) {
#pragma unroll
            for (int q = 0; q < R3_NSC; ++q) {
                const f32x4 o = slot[q * 64];
#pragma unroll
                for (int e = 0; e < 4; ++e) aC[q][e] += o[e];
                slot[q * 64] = aC[q];
            }
        } else if (wave == RW / 2) {
            // row t: c_ti = theta_i w_i, w_i = A_i + eta_{i+1} w_{i+1},
            // A_i = prod_{i < j <= t} (1 - alpha_j), from w_t = A_t = 1
            // down; every lane takes the same steps (rows above t hold the
            // start value) and stores in groups of 16
            const int t = lane;
            float Ap = 1.f, wv = 1.f;
#pragma unroll
            for (int i0 = 48; i0 >= 0; i0 -= 16) {
                float cr[16];
#pragma unroll
                for (int e = 15; e >= 0; --e) {
                    const int i = i0 + e;
                    if (i + 1 < 64) {
                        const float ap = Ap * (1.0f - gt[128 + i + 1]);
                        const float w = __builtin_fmaf(gt[64 + i + 1], wv, ap);
                        Ap = i < t ? ap : 1.0f;
                        wv = i < t ? w : 1.0f;
                    }
                    cr[e] = gt[i] * wv;
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) cT[t * RCP + i0 + e] = cr[e];
            }
        }
        __syncthreads();
        // C = c_ti (x_t . H_i) on and below the diagonal inside the chunk,
        // zeros elsewhere (a select: rows past the chunk are not defined)
        for (int idx = tid; idx < 64 * 64; idx += RW * 64) {
            const int t = idx >> 6, i = idx & 63;
            float v = 0.f;
            if (t < b && i <= t) {
                const int q = (t >> 4) * ((t >> 4) + 1) / 2 + (i >> 4);
                const int ln = (i & 15) + 16 * ((t & 15) >> 2), e = t & 3;
                float sc = 0.f;
#pragma unroll
                for (int w = 0; w < RW / 2; ++w) sc += sred[((w * R3_NSC + q) * 64 + ln) * 4 + e];
                v = cT[t * RCP + i] * sc;
            }
            cT[t * RCP + i] = v;
        }
        // (the next barrier orders these writes before the correction)
    }
    float* zm = zp + wave * 64 * RTP;
    float* dm = dp + wave * 64 * RTP;
#pragma unroll
    for (int m = 0; m < RMR; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = m * 16 + 4 * (lane >> 4) + e;
            zm[t * RTP + (lane & 15)] = __builtin_fmaf(pmps[t], aM[m][e], pmps[64 + t] * aS[m][e]);
            if constexpr (DK != R3D_BUF) dm[t * RTP + (lane & 15)] = aD[m][e];
        }
    __syncthreads();
    if constexpr (DK != R3D_BUF) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + q * RW * 64, i = idx >> 4, cl = idx & 15;
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < RW; ++w) x += dp[(w * 64 + i) * RTP + cl];
            // (zeros past the chunk: the correction runs over whole float4s)
            dT[cl * RCP + i] = i >= b ? 0.f : DK == R3D_BWD ? x * dv[q] : 2.0f * (x - dv[q]);
        }
        __syncthreads();
    }
    for (int idx = tid; idx < b * 16; idx += RW * 64) {
        const int t = idx >> 4, cl = idx & 15, col = nb * 16 + cl;
        float zz = 0.f;
#pragma unroll
        for (int w = 0; w < RW; ++w) zz += zp[(w * 64 + t) * RTP + cl];
        // the correction over whole float4s of keys (C is zero past t and
        // the chunk, Delta past the chunk)
        const f32x4* cr = reinterpret_cast<const f32x4*>(cT + t * RCP);
        const f32x4* dr = reinterpret_cast<const f32x4*>(dT + cl * RCP);
        f32x4 c4 = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q <= (t >> 2); ++q) {
            const f32x4 cc = cr[q], dd = dr[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) c4[e] = __builtin_fmaf(cc[e], dd[e], c4[e]);
        }
        zz -= (c4[0] + c4[1]) + (c4[2] + c4[3]);
        if (r.y) {
            r.y[tok_off(r.tl, s, r.yt0 + t) + col] = zz;
        } else {
            reinterpret_cast<OP*>(r.out)[(long)s * r.out_ss + pk(t, col, r.N >> 5)] = (OP)(zz * sigmoid(zz));
        }
    }
}

// the shapes the kernels assume: a chunk of 1 .. 64 tokens, bp = b rounded
// up to 32, K (and K1) a multiple of 32 and N of 16 (every layer width is a
// multiple of 32)
static bool r3_shape_ok(const R3Args& r, int ns) {
    return r.b >= 1 && r.b <= 16 * RMR && r.bp == (r.b + 31) / 32 * 32 && r.K >= 32 && r.K % 32 == 0 &&
           r.N >= 16 && r.N % 16 == 0 && ns >= 1 && ns <= 65535;
}

hipError_t launch_r3_score(const R3Args& r, int ns, int nchunks, int f32, hipStream_t st) {
    if (!r3_shape_ok(r, ns) || nchunks < 1 || nchunks > 65535) return hipErrorInvalidValue;
    const dim3 grid(r.bp / 16, ns, nchunks);
    if (r.K >= 1024) {
        if (f32) launch_k((r3_score_kernel<float, 16>), grid, dim3(16 * 64), r3_score_lds(16), st, r);
        else launch_k((r3_score_kernel<bf16, 16>), grid, dim3(16 * 64), r3_score_lds(16), st, r);
    } else {
        if (f32) launch_k((r3_score_kernel<float, 8>), grid, dim3(8 * 64), r3_score_lds(8), st, r);
        else launch_k((r3_score_kernel<bf16, 8>), grid, dim3(8 * 64), r3_score_lds(8), st, r);
    }
    return hipGetLastError();
}

template <class OP, int BL, int DK>
static void launch_layer_as(const R3Args& r, int ns, hipStream_t st) {
    launch_k((r3_layer_kernel<OP, BL, DK>), dim3(r.N / 16, ns), dim3(RW * 64), R3_LAYER_LDS, st, r);
}

template <class OP>
static hipError_t launch_layer_op(const R3Args& r, int ns, hipStream_t st) {
    if (r.dk == R3D_BWD && r.bl == BL_CF0) launch_layer_as<OP, BL_CF0, R3D_BWD>(r, ns, st);
    else if (r.dk == R3D_OUT && r.bl == BL_CF0) launch_layer_as<OP, BL_CF0, R3D_OUT>(r, ns, st);
    else if (r.dk == R3D_BUF && r.bl == BL_CF1) launch_layer_as<OP, BL_CF1, R3D_BUF>(r, ns, st);
    else if (r.dk == R3D_BUF && r.bl == BL_ROW) launch_layer_as<OP, BL_ROW, R3D_BUF>(r, ns, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_r3_layer(const R3Args& r, int ns, int f32, hipStream_t st) {
    if (!r3_shape_ok(r, ns) || (r.dk == R3D_BWD && (r.K1 < 32 || r.K1 % 32 != 0))) return hipErrorInvalidValue;
    return f32 ? launch_layer_op<float>(r, ns, st) : launch_layer_op<bf16>(r, ns, st);
}

}  // namespace tmk
