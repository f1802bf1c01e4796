// The backward through the memory's store: the gradients of an outer loss
// with respect to a call's keys, values, queries, gates and starting state
// ("titans-pytorch analysis", Editorial conclusion: the loss backpropagates
// through the memory state; "Titans, explained", step 6: the chunked form
// that makes the memory trainable in parallel).
//
// Per chunk, with every gradient at the chunk-start weights M_0, the write
// is the closed form
//     S_end = p_eta S_0 - sum_i d_i G_i,   M_end = p_alpha M_0 + s0 S_0 - sum_i c_i G_i,
//     G_i = (per layer) h_i^T Delta_i,
// so its adjoint, given Mbar = dL/dM_end and Sbar = dL/dS_end, is
//     Mbar_0 = p_alpha Mbar + VJP_{M_0}( sum_i <Gbar_i, G_i> ),  Sbar_0 = p_eta Sbar + s0 Mbar,
//     Gbar_i = -(c_i Mbar + d_i Sbar),
//     cbar_i = -<Mbar, G_i>, dbar_i = -<Sbar, G_i>, pbar_alpha = <Mbar, M_0>,
//     pbar_eta = <Sbar, S_0>, s0bar = <Mbar, S_0>,
// and the coefficients' adjoint gives the gates' gradients.  The VJP runs
// back through each key row's forward and backward at M_0 (second order:
// SiLU'' appears).  This file holds the kernels: a tiled fp32 product with
// the sweep's epilogues, the element-wise steps, and the coefficients with
// their adjoint.  The launch sequence is in tm_api.hip.
#include "tm_device.h"

namespace tmk {
namespace {

constexpr int BT = 64;    // output tile: BT x BT, 256 threads of 4 x 4
constexpr int BKS = 16;   // K per LDS stage
constexpr int BPAD = 4;

__device__ __forceinline__ float silu_d(float z) {
    const float s = sigmoid(z);
    return s * (1.f + z * (1.f - s));
}
// d^2/dz^2 of z sigma(z) = sigma (1 - sigma) (2 + z (1 - 2 sigma))
__device__ __forceinline__ float silu_dd(float z) {
    const float s = sigmoid(z);
    return s * (1.f - s) * (2.f + z * (1.f - 2.f * s));
}

__device__ __forceinline__ long moff(const BMat& M, const TokLayout& tl, int s, int r, int c) {
    return M.tok ? tok_off(tl, s, M.t0 + r) + c : (long)s * M.ss + (long)r * M.ld + c;
}
__device__ __forceinline__ float mload(const BMat& M, const TokLayout& tl, int s, int r, int c) {
    const long o = moff(M, tl, s, r, c);
    return M.bf ? (float)reinterpret_cast<const bf16*>(M.p)[o] : reinterpret_cast<const float*>(M.p)[o];
}
__device__ __forceinline__ float* mptr(const BMat& M, const TokLayout& tl, int s, int r, int c) {
    return const_cast<float*>(reinterpret_cast<const float*>(M.p)) + moff(M, tl, s, r, c);
}

__global__ __launch_bounds__(256) void bgemm_kernel(BGemm g) {
    __shared__ float As[BKS][BT + BPAD];
    __shared__ float Bs[2][BKS][BT + BPAD];
    __shared__ float red[4][3];
    const int s = blockIdx.z;
    const int n0 = blockIdx.x * BT, m0 = blockIdx.y * BT;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    float acc0[4][4], acc1[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc0[i][j] = acc1[i][j] = 0.f;

    const int nseg = g.k2 > 0 ? 2 : 1;
    for (int seg = 0; seg < nseg; ++seg) {
        const BMat& A = seg ? g.A2 : g.A;
        const BMat& B = seg ? g.Bs2 : g.B;
        const int K = seg ? g.k2 : g.k;
        const bool two = seg == 0 && g.dual != 0;
        for (int k0 = 0; k0 < K; k0 += BKS) {
            for (int e = tid; e < BT * BKS; e += 256) {
                int mm, kk;
                if (g.ta) { mm = e & (BT - 1); kk = e / BT; }       // A stored [k][m]: m contiguous
                else { kk = e & (BKS - 1); mm = e / BKS; }          // A stored [m][k]: k contiguous
                const int gm = m0 + mm, gk = k0 + kk;
                float v = 0.f;
                if (gm < g.m && gk < K) v = g.ta ? mload(A, g.tl, s, gk, gm) : mload(A, g.tl, s, gm, gk);
                As[kk][mm] = v;
            }
            for (int e = tid; e < BT * BKS; e += 256) {
                int nn, kk;
                if (g.tb) { kk = e & (BKS - 1); nn = e / BKS; }     // B stored [n][k]
                else { nn = e & (BT - 1); kk = e / BT; }            // B stored [k][n]
                const int gn = n0 + nn, gk = k0 + kk;
                float v = 0.f, v2 = 0.f;
                if (gn < g.n && gk < K) {
                    v = g.tb ? mload(B, g.tl, s, gn, gk) : mload(B, g.tl, s, gk, gn);
                    if (seg == 0 && g.dual == 1)
                        v2 = g.tb ? mload(g.B2, g.tl, s, gn, gk) : mload(g.B2, g.tl, s, gk, gn);
                    if (seg == 0 && g.dual == 2) {
                        v2 = v * g.sk1[(long)s * g.sk_ss + gk];
                        v *= g.sk0[(long)s * g.sk_ss + gk];
                    }
                }
                Bs[0][kk][nn] = v;
                Bs[1][kk][nn] = v2;
            }
            __syncthreads();
#pragma unroll 4
            for (int kk = 0; kk < BKS; ++kk) {
                float a[4], b0[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
                for (int j = 0; j < 4; ++j) b0[j] = Bs[0][kk][tx * 4 + j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc0[i][j] = __builtin_fmaf(a[i], b0[j], acc0[i][j]);
                if (two) {
                    float b1[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) b1[j] = Bs[1][kk][tx * 4 + j];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc1[i][j] = __builtin_fmaf(a[i], b1[j], acc1[i][j]);
                }
            }
            __syncthreads();
        }
    }

    const TokLayout& tl = g.tl;
    const int rb = m0 + ty * 4, cb = n0 + tx * 4;
    if (g.epi == BE_GP) {
        // the tile holds rows 0 .. b-1 (m <= 64): each row's dot products of
        // the two accumulators with x0 over the tile's columns, reduced over
        // the 16 threads of the row group (lanes 16 ty' .. 16 ty' + 15)
        float pc[4], pd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pc[i] = pd[i] = 0.f;
            const int r = rb + i;
            if (r >= g.m) continue;
            const float cr = g.rs0[(long)s * g.sk_ss + r], dr = g.rs1[(long)s * g.sk_ss + r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = cb + j;
                if (n >= g.n) continue;
                const float x = mload(g.x0, tl, s, r, n);
                pc[i] = __builtin_fmaf(acc0[i][j], x, pc[i]);
                pd[i] = __builtin_fmaf(acc1[i][j], x, pd[i]);
                *mptr(g.c0, tl, s, r, n) = -__builtin_fmaf(cr, acc0[i][j], dr * acc1[i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) {
                pc[i] += __shfl_xor(pc[i], off, 64);
                pd[i] += __shfl_xor(pd[i], off, 64);
            }
        if (tx == 0) {
            float* o = g.part + (long)s * g.part_ss + (long)(g.tile0 + blockIdx.x) * 128;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[rb + i] = pc[i];
                o[64 + rb + i] = pd[i];
            }
        }
        return;
    }
    if (g.epi == BE_ADJ) {
        const float* cs = g.cs + (long)s * g.cs_ss;
        const float pa = cs[0], pe = cs[1], s0 = cs[2];
        float d0 = 0.f, d1 = 0.f, d2 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + i;
            if (r >= g.m) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = cb + j;
                if (n >= g.n) continue;
                float* pm = mptr(g.c0, tl, s, r, n);
                float* ps = mptr(g.c1, tl, s, r, n);
                const float mb = *pm, sb = *ps;
                const float mv = mload(g.x0, tl, s, r, n), sv = mload(g.x1, tl, s, r, n);
                d0 = __builtin_fmaf(mb, mv, d0);
                d1 = __builtin_fmaf(sb, sv, d1);
                d2 = __builtin_fmaf(mb, sv, d2);
                *pm = __builtin_fmaf(pa, mb, acc0[i][j]);
                *ps = __builtin_fmaf(pe, sb, s0 * mb);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            d0 += __shfl_xor(d0, off, 64);
            d1 += __shfl_xor(d1, off, 64);
            d2 += __shfl_xor(d2, off, 64);
        }
        const int wv = tid >> 6;
        if ((tid & 63) == 0) {
            red[wv][0] = d0;
            red[wv][1] = d1;
            red[wv][2] = d2;
        }
        __syncthreads();
        if (tid == 0) {
            float* o = g.part + (long)s * g.part_ss + (long)(g.tile0 + blockIdx.y * gridDim.x + blockIdx.x) * 3;
#pragma unroll
            for (int q = 0; q < 3; ++q) o[q] = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
        }
        return;
    }
    const float* cs = g.epi == BE_UPD ? g.cs + (long)s * g.cs_ss : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rb + i;
        if (r >= g.m) continue;
        float cr = 0.f, dr = 0.f;
        if (g.epi == BE_GQ) {
            cr = g.rs0[(long)s * g.sk_ss + r];
            dr = g.rs1[(long)s * g.sk_ss + r];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = cb + j;
            if (n >= g.n) continue;
            const float a0 = acc0[i][j];
            switch (g.epi) {
                case BE_STORE: *mptr(g.c0, tl, s, r, n) = a0; break;
                case BE_ACC: *mptr(g.c0, tl, s, r, n) += a0; break;
                case BE_HID:
                    *mptr(g.c0, tl, s, r, n) = a0;
                    *mptr(g.c1, tl, s, r, n) = a0 * sigmoid(a0);
                    break;
                case BE_OUTK:
                    *mptr(g.c0, tl, s, r, n) = a0;
                    *mptr(g.c1, tl, s, r, n) = 2.f * (a0 - mload(g.x0, tl, s, r, n));
                    break;
                case BE_BWDK:
                    *mptr(g.c0, tl, s, r, n) = a0;
                    *mptr(g.c1, tl, s, r, n) = a0 * silu_d(mload(g.x0, tl, s, r, n));
                    break;
                case BE_QB: *mptr(g.c0, tl, s, r, n) = a0 * silu_d(mload(g.x0, tl, s, r, n)); break;
                case BE_ADDSTORE: *mptr(g.c0, tl, s, r, n) = a0 + mload(g.x0, tl, s, r, n); break;
                case BE_HB:
                    *mptr(g.c1, tl, s, r, n) +=
                        (a0 + mload(g.x0, tl, s, r, n)) * silu_d(mload(g.x1, tl, s, r, n));
                    break;
                case BE_GQ: *mptr(g.c0, tl, s, r, n) = -__builtin_fmaf(cr, a0, dr * acc1[i][j]); break;
                case BE_UPD: {
                    const float mv = mload(g.x0, tl, s, r, n), sv = mload(g.x1, tl, s, r, n);
                    *mptr(g.c0, tl, s, r, n) = __builtin_fmaf(cs[0], mv, __builtin_fmaf(cs[2], sv, -a0));
                    *mptr(g.c1, tl, s, r, n) = __builtin_fmaf(cs[1], sv, -acc1[i][j]);
                    break;
                }
                default: break;
            }
        }
    }
}

__global__ __launch_bounds__(256) void belem_kernel(BElem e) {
    const int s = blockIdx.y;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)e.b * e.n) return;
    const int r = (int)(i / e.n), c = (int)(i - (long)r * e.n);
    const long o = (long)s * e.ss + i;
    const float db = e.db[o];
    if (e.mode == BW_U) {
        const long ro = (long)s * e.rss + i;
        const float z = e.z[ro];
        e.u[o] = db * silu_d(z);
        e.zb[o] = db * e.g[ro] * silu_dd(z);
    } else {
        e.zb[o] = 2.f * db;
        e.dv[tok_off(e.tl, s, e.t0 + r) + c] = -2.f * db;
    }
}

// One workgroup of 64 threads per (chunk, stream).  The recurrences run in
// thread 0 over the chunk's tokens in order (b <= 64 steps); the other
// threads only move data and sum the partials, each in a fixed order.
__global__ __launch_bounds__(64) void bcoef_kernel(BCoef a) {
    __shared__ float th[64], et[64], al[64], A[64], E[64], R[64];
    __shared__ float cb[64], dbb[64], Ab[64], Eb[64], rbb[64], etb[64], alb[64];
    __shared__ float dots[3];
    const int c = blockIdx.x, s = blockIdx.y, i = threadIdx.x, b = a.b;
    const int t = c * b + i;
    if (i < b) {
        const long gi = tok_off(a.gl, s, t);
        th[i] = a.theta[gi];
        et[i] = a.eta[gi];
        al[i] = a.alpha[gi];
    }
    if (a.mode == BC_BWD) {
        const long sc = (long)s * a.C + c;
        float pc = 0.f, pd = 0.f;
        if (i < b) {
            const float* p = a.pgp + sc * a.ngp * 128;
            for (int q = 0; q < a.ngp; ++q) {
                pc += p[q * 128 + i];
                pd += p[q * 128 + 64 + i];
            }
            // cbar_i = -<Mbar, G_i>, dbar_i = -<Sbar, G_i>
            cb[i] = -pc;
            dbb[i] = -pd;
        }
        float d3[3] = {0.f, 0.f, 0.f};
        const float* p = a.pad + sc * a.nad * 3;
        for (int q = i; q < a.nad; q += 64)
            for (int j = 0; j < 3; ++j) d3[j] += p[q * 3 + j];
        for (int j = 0; j < 3; ++j)
            for (int off = 32; off >= 1; off >>= 1) d3[j] += __shfl_xor(d3[j], off, 64);
        if (i == 0)
            for (int j = 0; j < 3; ++j) dots[j] = d3[j];
    }
    __syncthreads();
    if (i == 0) {
        A[b - 1] = 1.f;
        E[b - 1] = 1.f;
        R[b - 1] = 1.f;
        for (int j = b - 2; j >= 0; --j) {
            A[j] = A[j + 1] * (1.f - al[j + 1]);
            E[j] = E[j + 1] * et[j + 1];
            R[j] = A[j] + et[j + 1] * R[j + 1];
        }
        if (a.mode == BC_BWD) {
            for (int j = 0; j < b; ++j) {
                rbb[j] = cb[j] * th[j];
                Eb[j] = dbb[j] * th[j];
                Ab[j] = 0.f;
                etb[j] = 0.f;
                alb[j] = 0.f;
            }
            const float pab = dots[0], peb = dots[1], s0b = dots[2];
            // p_alpha = (1 - alpha_0) A_0, p_eta = eta_0 E_0, s0 = eta_0 r_0
            Ab[0] += pab * (1.f - al[0]);
            alb[0] -= pab * A[0];
            Eb[0] += peb * et[0];
            etb[0] += peb * E[0];
            rbb[0] += s0b * et[0];
            etb[0] += s0b * R[0];
            // the recurrences ran j = b-2 .. 0, each from j + 1: their
            // adjoints run j = 0 .. b-2
            for (int j = 0; j + 1 < b; ++j) {
                // r_j = A_j + eta_{j+1} r_{j+1}
                Ab[j] += rbb[j];
                etb[j + 1] += rbb[j] * R[j + 1];
                rbb[j + 1] += rbb[j] * et[j + 1];
                // E_j = E_{j+1} eta_{j+1}
                Eb[j + 1] += Eb[j] * et[j + 1];
                etb[j + 1] += Eb[j] * E[j + 1];
                // A_j = A_{j+1} (1 - alpha_{j+1})
                Ab[j + 1] += Ab[j] * (1.f - al[j + 1]);
                alb[j + 1] -= Ab[j] * A[j + 1];
            }
        }
    }
    __syncthreads();
    if (i < b) {
        if (a.mode == BC_FWD) {
            a.cc[(long)s * a.coef_ss + t] = th[i] * R[i];
            a.dc[(long)s * a.coef_ss + t] = th[i] * E[i];
            if (i == 0) {
                float* o = a.cs + (long)s * a.cs_ss + (long)c * 4;
                o[0] = (1.f - al[0]) * A[0];
                o[1] = et[0] * E[0];
                o[2] = et[0] * R[0];
                o[3] = 0.f;
            }
        } else {
            const long gi = tok_off(a.gl, s, t);
            // theta_i enters c_i = theta_i r_i and d_i = theta_i E_i
            a.dtheta[gi] = cb[i] * R[i] + dbb[i] * E[i];
            a.deta[gi] = etb[i];
            a.dalpha[gi] = alb[i];
        }
    }
}

}  // namespace

hipError_t launch_bgemm(const BGemm& g, int ns, hipStream_t st) {
    if (g.m <= 0 || g.n <= 0 || ns <= 0) return hipSuccess;
    if (g.epi == BE_GP && g.m > BT) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((g.n + BT - 1) / BT), (unsigned)((g.m + BT - 1) / BT), (unsigned)ns);
    launch_k(bgemm_kernel, grid, dim3(256), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_belem(const BElem& e, int ns, hipStream_t st) {
    const long n = (long)e.b * e.n;
    if (n <= 0 || ns <= 0) return hipSuccess;
    launch_k(belem_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)ns), dim3(256), 0, st, e);
    return hipGetLastError();
}

hipError_t launch_bcoef(const BCoef& a, int ns, hipStream_t st) {
    if (a.C <= 0 || ns <= 0) return hipSuccess;
    if (a.b < 1 || a.b > 64) return hipErrorInvalidValue;
    launch_k(bcoef_kernel, dim3((unsigned)a.C, (unsigned)ns), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace tmk
