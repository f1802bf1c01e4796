// HIP kernels for the Titans neural-memory store / retrieve on CDNA4 (gfx950).
//
// Per chunk of b tokens and per memory stream (one memory per sequence and
// head), the store is ("Titans, explained", steps 2-4 and 6; "Attack of the
// Titans", Parallel training):
//   1. forward of the keys through the chunk-start weights, with the queries
//      of the previous chunk riding along as extra rows (both read the same
//      weights),                                            -> gemm_kernel
//   2. backward of ||M(k) - v||^2 to every hidden layer,    -> gemm_kernel
//   3. the per-token gradients, weighted by coefficients of theta, eta and
//      alpha, reduced over the chunk and folded into S and M in one pass over
//      the state                                            -> update_kernel
// The coefficients come from a wave-level scan over the gates of each chunk
// (scan_kernel): the momentum is a linear recurrence and the forgetting a
// running product, and unrolling both over a chunk whose gradients all sit at
// the chunk-start weights gives
//     S_end = p_eta S_0 - sum_i d_i G_i,
//     M_end = p_alpha M_0 + s0 S_0 - sum_i c_i G_i,
// with A_i = prod_{j>i} (1 - alpha_j), E_i = prod_{j>i} eta_j,
// r_i = A_i + eta_{i+1} r_{i+1} (r_b = 1), c_i = theta_i r_i, d_i = theta_i E_i,
// p_alpha = prod (1 - alpha), p_eta = prod eta, s0 = eta_1 r_1.  Only products
// and sums appear (no ratios of running products, which underflow).
//
// Matrix products run on MFMA: v_mfma_f32_16x16x32_bf16 for the bf16 path
// and v_mfma_f32_16x16x4_f32 for the fp32 path, fp32 accumulation in both.
#include "tm_internal.h"

namespace tmk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <class OP> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 T; };
template <> struct Frag<float> { typedef f32x8 T; };   // also: 8 raw values of a storage type

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ f32x8 ld8(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 to_bf16(f32x8 v) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)v[j];
    return r;
}
__device__ __forceinline__ f32x8 to_f32(bf16x8 v) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (float)v[j];
    return r;
}

template <class OP> __device__ __forceinline__ typename Frag<OP>::T cvt(f32x8 v);
template <> __device__ __forceinline__ bf16x8 cvt<bf16>(f32x8 v) { return to_bf16(v); }
template <> __device__ __forceinline__ f32x8 cvt<float>(f32x8 v) { return v; }
template <class OP> __device__ __forceinline__ typename Frag<OP>::T cvt(bf16x8 v);
template <> __device__ __forceinline__ bf16x8 cvt<bf16>(bf16x8 v) { return v; }
template <> __device__ __forceinline__ f32x8 cvt<float>(bf16x8 v) { return to_f32(v); }

__device__ __forceinline__ f32x8 to_f32v(f32x8 v) { return v; }
__device__ __forceinline__ f32x8 to_f32v(bf16x8 v) { return to_f32(v); }

template <class OP> __device__ __forceinline__ typename Frag<OP>::T zero_frag() {
    typename Frag<OP>::T z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (OP)0.0f;
    return z;
}

// C += A B over one 32-deep slice of K.  Each lane supplies 8 consecutive K
// values of its A row and of its B column; A and B use the same K order, so
// how the instruction maps register slots to K does not matter.
__device__ __forceinline__ void mma(f32x4& c, bf16x8 a, bf16x8 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, f32x8 a, f32x8 b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ __forceinline__ long tok_off(const TokLayout& tl, int s, int t) {
    int bi = s / tl.H, hi = s - bi * tl.H;
    return ((long)bi * tl.Tc + t) * tl.H * (long)tl.d + (long)hi * tl.d;
}

template <class T> __device__ __forceinline__ void store1(void* p, long i, float x) {
    reinterpret_cast<T*>(p)[i] = (T)x;
}
template <class T> __device__ __forceinline__ float load1(const void* p, long i) {
    return (float)reinterpret_cast<const T*>(p)[i];
}

// ---------------------------------------------------------------------------
// Chunk forward / backward product.  A workgroup of W waves owns one tile of
// 64 rows x 16*NR columns and splits its K range over the waves (wave w takes
// the w-th contiguous slice of 32-deep steps); the W partial tiles are summed
// in LDS in a fixed order, so results are deterministic and no workgroup ever
// waits for another (cross-workgroup handoffs need device-scope fences, which
// serialise across the whole chip).  Each lane feeds the matrix cores from
// registers loaded straight from global memory (activations hit L2) through
// a PF-deep prefetch ring; the ring has no branches, steps past the end of a
// slice re-load a valid address and contribute zeros.
// OP: operand type; AT / BT: storage types of A / B; BKC: B contiguous in K.

constexpr int GEMM_RT = 64;   // rows per tile (4 row blocks of 16)

template <class OP> __device__ __forceinline__ void st8(OP* p, typename Frag<OP>::T v) {
    *reinterpret_cast<typename Frag<OP>::T*>(p) = v;
}
__device__ __forceinline__ void st8f(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = (f32x4){v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = (f32x4){v[4], v[5], v[6], v[7]};
}

// Row outputs of 8 consecutive columns c .. c+7 of row r; z becomes the
// value the transposed copy carries for key rows (the rounded activation,
// or Delta).
template <class OP>
__device__ __forceinline__ void gemm_store8(const GemmArgs& g, int s, int r, int c, float* z) {
    typedef typename Frag<OP>::T F;
    F o;
    if (g.epi == EPI_HIDDEN) {
        float sl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sg = sigmoid(z[e]);
            o[e] = (OP)(z[e] * sg);
            sl[e] = sg * (1.0f + z[e] * (1.0f - sg));
            z[e] = (float)o[e];
        }
        st8<OP>(reinterpret_cast<OP*>(g.act) + (long)s * g.act_ss + pk(r, c, g.N >> 5), o);
        if (r >= g.n0 && g.dsl) st8f(g.dsl + (long)s * g.dsl_ss + (long)(r - g.n0) * g.dsl_ld + c, sl);
        return;
    }
    int t = r;
    if (g.epi == EPI_OUT) {
        if (r < g.n0) {
            st8f(g.y + tok_off(g.tl, s, g.yt0 + r) + c, z);
            return;
        }
        t = r - g.n0;
        const f32x8 vv = to_f32v(ld8(reinterpret_cast<const OP*>(g.v) + tok_off(g.tl, s, g.vt0 + t) + c));
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = 2.0f * (z[e] - vv[e]);
    } else {
        const f32x8 sl = ld8(g.dsl + (long)s * g.dsl_ss + (long)r * g.dsl_ld + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = z[e] * sl[e];
    }
    if (g.dlp) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (OP)z[e];
        st8<OP>(reinterpret_cast<OP*>(g.dlp) + (long)s * g.dlp_ss + pk(t, c, g.N >> 5), o);
    }
}

template <class OP, class AT, class BT, bool BKC, int NR, int W, int PF>
__global__ __launch_bounds__(W * 64) void gemm_kernel(GemmArgs g) {
    typedef typename Frag<OP>::T F;
    constexpr int MR = GEMM_RT / 16;
    constexpr int NT = NR * 16;
    constexpr int NTP = NT + 1;            // padded LDS row
    extern __shared__ float red[];          // [W][GEMM_RT][NTP]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.z;
    const int row0 = blockIdx.y * GEMM_RT;
    const int col0 = blockIdx.x * NT;
    const int nsteps = g.K >> 5;
    const int spw = (nsteps + W - 1) / W;   // steps per wave
    const int kb = wave * spw;
    const int ke = min(nsteps, kb + spw);   // may be <= kb: the wave adds zeros
    const int klast = max(min(ke, nsteps) - 1, 0);

    f32x4 acc[MR][NR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n) acc[m][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // per-lane operand addresses at K step 0 and the distance of one step:
    // packed operands advance by one 64-lane fragment (512 elements)
    const int kofs = 8 * (lane >> 4);
    const AT* arow[MR];
    bool aok[MR];
    long astep = 32;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        int rb = (row0 >> 4) + m;
        aok[m] = rb * 16 + (lane & 15) < g.nrows;
        if (g.amode == A_PACKED) {
            if (rb * 16 >= g.nrows) rb = 0;   // a block past the rows: valid address, values dropped
            arow[m] = reinterpret_cast<const AT*>(g.a0) + (long)s * g.a_ss + pkf(rb, 0, nsteps, lane);
            astep = 512;
            continue;
        }
        int r = rb * 16 + (lane & 15);
        if (!aok[m]) r = g.nrows - 1;
        long off;
        const void* base = g.a0;
        if (g.amode == A_TOKENS) {
            if (r < g.n0) { off = tok_off(g.tl, s, g.at0 + r); }
            else { base = g.a1; off = tok_off(g.tl, s, g.at1 + r - g.n0); }
        } else {
            off = (long)s * g.a_ss + (long)r * g.a_ld;
        }
        arow[m] = reinterpret_cast<const AT*>(base) + off + kofs;
    }
    const BT* bcol[NR];
    bool bok[NR];
    long bstep = 32;
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        int cb = (col0 >> 4) + n;
        const int c = cb * 16 + (lane & 15);
        bok[n] = c < g.N;
        const BT* base = reinterpret_cast<const BT*>(g.b) + (long)s * g.b_ss;
        if (g.bmode == B_PACKED) {
            if (cb * 16 >= g.N) cb = 0;
            bcol[n] = base + pkf(cb, 0, nsteps, lane);
            bstep = 512;
        } else if (g.bmode == B_ROWS) {
            bcol[n] = base + (long)(bok[n] ? c : 0) * g.b_ld + kofs;
        } else {
            bcol[n] = base + (bok[n] ? c : 0) + (long)kofs * g.b_ld;
        }
    }
    // the ring holds raw storage vectors; conversion to the operand type
    // happens right before the matrix instruction, so loads stay in flight
    typedef typename Frag<AT>::T RA;
    typedef typename Frag<BT>::T RB;
    RA a[PF][MR];
    RB bb[PF][NR];
    auto load_step = [&](int p, int k) {
#pragma unroll
        for (int m = 0; m < MR; ++m) a[p][m] = ld8(arow[m] + k * astep);
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            if (BKC) {
                bb[p][n] = ld8(bcol[n] + k * bstep);
            } else {
                RB u;
                const BT* q = bcol[n] + (long)(k << 5) * g.b_ld;
#pragma unroll
                for (int j = 0; j < 8; ++j) u[j] = q[(long)j * g.b_ld];
                bb[p][n] = u;
            }
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load_step(p, min(kb + p, klast));
    for (int k = kb; k < kb + spw; k += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const bool live = k + p < ke;   // wave-uniform
            F av[MR], bv[NR];
#pragma unroll
            for (int m = 0; m < MR; ++m) av[m] = aok[m] ? cvt<OP>(a[p][m]) : zero_frag<OP>();
#pragma unroll
            for (int n = 0; n < NR; ++n) bv[n] = (live && bok[n]) ? cvt<OP>(bb[p][n]) : zero_frag<OP>();
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int n = 0; n < NR; ++n) mma(acc[m][n], av[m], bv[n]);
            load_step(p, min(k + p + PF, klast));
        }
    }

    // sum the W partial tiles in LDS, in wave order
    float* mine = red + wave * (GEMM_RT * NTP);
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mine[(m * 16 + 4 * (lane >> 4) + e) * NTP + n * 16 + (lane & 15)] = acc[m][n][e];
    __syncthreads();
    // pass 1: row outputs, 8 consecutive columns per thread (N is a multiple
    // of 32); the value for the transposed copy is left in slot 0
    for (int idx = tid; idx < GEMM_RT * (NT / 8); idx += W * 64) {
        const int rr = idx / (NT / 8), cc = (idx - rr * (NT / 8)) * 8;
        const int r = row0 + rr, c = col0 + cc;
        if (r >= g.nrows || c >= g.N) continue;
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) x += red[w * (GEMM_RT * NTP) + rr * NTP + cc + e];
            z[e] = x;
        }
        gemm_store8<OP>(g, s, r, c, z);
#pragma unroll
        for (int e = 0; e < 8; ++e) red[rr * NTP + cc + e] = z[e];
    }
    if (!g.ht && !g.dct) return;   // uniform: no transposed outputs (retrieve)
    __syncthreads();
    // pass 2: the key rows' transposed copies, packed [N][bp]: 8 tokens of
    // one column per thread, whole vectors where all 8 tokens are this
    // tile's rows (a group cut by the tile edge is stored element-wise)
    const int tlo = max(row0, g.n0) - g.n0, thi = min(row0 + GEMM_RT, g.nrows) - g.n0;
    if (thi <= tlo) return;
    const int g0 = tlo >> 3, ng = ((thi - 1) >> 3) - g0 + 1;
    const int nkb = g.bp >> 5;
    for (int idx = tid; idx < NT * ng; idx += W * 64) {
        const int cc = idx % NT, t8 = (g0 + idx / NT) * 8;
        const int c = col0 + cc;
        if (c >= g.N) continue;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t8 + e;
            x[e] = (t >= tlo && t < thi) ? red[(t + g.n0 - row0) * NTP + cc] : 0.f;
        }
        const long o = (long)s * g.tr_ss + pk(c, t8, nkb);
        const bool whole = t8 >= tlo && t8 + 8 <= thi;
        if (g.epi == EPI_HIDDEN) {
            OP* h = reinterpret_cast<OP*>(g.ht) + o;
            if (whole) {
                F v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (OP)x[e];
                st8<OP>(h, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t8 + e >= tlo && t8 + e < thi) h[e] = (OP)x[e];
            }
        } else {
            OP* pc = reinterpret_cast<OP*>(g.dct) + o;
            OP* pd = reinterpret_cast<OP*>(g.ddt) + o;
            const float* cf = g.cc + (long)s * g.coef_ss;
            const float* df = g.dc + (long)s * g.coef_ss;
            if (whole) {
                F vc, vd;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vc[e] = (OP)(cf[t8 + e] * x[e]);
                    vd[e] = (OP)(df[t8 + e] * x[e]);
                }
                st8<OP>(pc, vc);
                st8<OP>(pd, vd);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = t8 + e;
                    if (t >= tlo && t < thi) {
                        pc[e] = (OP)(cf[t] * x[e]);
                        pd[e] = (OP)(df[t] * x[e]);
                    }
                }
            }
        }
    }
}

// Pick the column width and wave count of one product: enough workgroups to
// cover the chip (about 192 tiles of 64 rows, ideally at least 3 steps per
// wave), wider tiles first so the activations are re-read from L2 less often.
static void pick(const GemmArgs& g, int ns, int& nr, int& w, bool allow16) {
    const int nsteps = g.K >> 5;
    const long nrt = (g.nrows + GEMM_RT - 1) / GEMM_RT;
    nr = 4;
    w = 4;
    auto wgs = [&](int nr_) { return (long)((g.N + 16 * nr_ - 1) / (16 * nr_)) * nrt * ns; };
    if (nsteps >= 8 * 3) w = 8;
    while (wgs(nr) < 192 && nr > 1) nr >>= 1;
    (void)allow16;
}

template <class OP, class AT, class BT, bool BKC, int NR, int W, int PF>
static void launch_one(const GemmArgs& g, int ns, hipStream_t st) {
    dim3 grid((g.N + NR * 16 - 1) / (NR * 16), (g.nrows + GEMM_RT - 1) / GEMM_RT, ns);
    const size_t lds = (size_t)W * GEMM_RT * (NR * 16 + 1) * 4;
    hipLaunchKernelGGL((gemm_kernel<OP, AT, BT, BKC, NR, W, PF>), grid, dim3(W * 64), lds, st, g);
}

template <class OP, class AT, class BT, bool BKC, int PF>
static hipError_t launch_gemm(const GemmArgs& g, int ns, hipStream_t st) {
    if (g.nrows <= 0 || g.N <= 0) return hipSuccess;
    int nr, w;
    // 16-wave workgroups cap a wave at 128 registers: only the narrowest
    // tile with 16-bit operands in storage fits the prefetch ring there
    pick(g, ns, nr, w, sizeof(AT) == 2 && sizeof(BT) == 2);
    if (w == 16) {
        launch_one<OP, AT, BT, BKC, 1, 16, PF>(g, ns, st);
    } else if (w == 8) {
        if (nr == 4) launch_one<OP, AT, BT, BKC, 4, 8, PF>(g, ns, st);
        else if (nr == 2) launch_one<OP, AT, BT, BKC, 2, 8, PF>(g, ns, st);
        else launch_one<OP, AT, BT, BKC, 1, 8, PF>(g, ns, st);
    } else {
        if (nr == 4) launch_one<OP, AT, BT, BKC, 4, 4, PF>(g, ns, st);
        else if (nr == 2) launch_one<OP, AT, BT, BKC, 2, 4, PF>(g, ns, st);
        else launch_one<OP, AT, BT, BKC, 1, 4, PF>(g, ns, st);
    }
    return hipGetLastError();
}

hipError_t launch_fwd(const GemmArgs& g, int ns, int f32, hipStream_t st) {
    if (f32) return launch_gemm<float, float, float, false, 2>(g, ns, st);
    return launch_gemm<bf16, bf16, bf16, true, 4>(g, ns, st);
}

hipError_t launch_bwd(const GemmArgs& g, int ns, int f32, hipStream_t st) {
    if (f32) return launch_gemm<float, float, float, true, 2>(g, ns, st);
    return launch_gemm<bf16, bf16, float, true, 2>(g, ns, st);
}

// ---------------------------------------------------------------------------
// Coefficient scan: one wave per (stream, chunk), lane i = token i of the chunk.

__device__ __forceinline__ float shdown(float x, int off) { return __shfl_down(x, off, 64); }

// Keys of one chunk, 64 features at a time, transposed through LDS into
// kt[s][chunk] (packed [d][bp]: rows are features, K runs over the chunk's
// tokens, zero past the chunk).
template <class T>
__device__ void transpose_keys(const ScanArgs& a, long blk) {
    typedef typename Frag<T>::T V;
    __shared__ float tile[64][65];
    const int d = a.ktl.d, ib = (d + 63) / 64;
    const int s = (int)(blk / ((long)a.C * ib));
    const long rem = blk - (long)s * a.C * ib;
    const int c = (int)(rem / ib), i0 = (int)(rem - (long)c * ib) * 64;
    const int tid = threadIdx.x;
    const T* k = reinterpret_cast<const T*>(a.k);
    for (int idx = tid; idx < 64 * 64; idx += 256) {
        const int t = idx >> 6, i = idx & 63;
        tile[t][i] = (t < a.b && i0 + i < d) ? (float)k[tok_off(a.ktl, s, c * a.b + t) + i0 + i] : 0.f;
    }
    __syncthreads();
    const int nkb = a.bp >> 5;
    T* kt = reinterpret_cast<T*>(a.kt) + ((long)s * a.C + c) * (long)d * a.bp;
    for (int idx = tid; idx < 4 * nkb * 64; idx += 256) {
        const int ln = idx & 63, ks = (idx >> 6) % nkb, rb = (idx >> 6) / nkb;
        const int i = rb * 16 + (ln & 15), t8 = ks * 32 + 8 * (ln >> 4);
        if (i0 + i >= d) continue;
        V v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (T)tile[t8 + e][i];
        *reinterpret_cast<V*>(kt + pkf((i0 >> 4) + rb, ks, nkb, ln)) = v;
    }
}

// One 16-token block of one chunk's keys or queries, packed ([b][d] per
// chunk: rows are tokens, K runs over the features; zero past the chunk).
template <class T>
__device__ void pack_rows(const ScanArgs& a, long blk) {
    typedef typename Frag<T>::T V;
    const int d = a.ktl.d, nbt = (a.b + 15) >> 4, nks = d >> 5;
    const int nkq = a.q ? 2 : 1;
    const int kq = (int)(blk % nkq);
    blk /= nkq;
    const int tb = (int)(blk % nbt);
    blk /= nbt;
    const int c = (int)(blk % a.C), s = (int)(blk / a.C);
    const T* src = reinterpret_cast<const T*>(kq ? a.q : a.k);
    T* dst = reinterpret_cast<T*>(kq ? a.xq : a.xk) + ((long)s * a.C + c) * a.xc;
    for (int idx = threadIdx.x; idx < nks * 64; idx += 256) {
        const int ln = idx & 63, ks = idx >> 6;
        const int t = tb * 16 + (ln & 15), i = ks * 32 + 8 * (ln >> 4);
        V v;
        if (t < a.b) {
            v = ld8(src + tok_off(a.ktl, s, c * a.b + t) + i);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (T)0.0f;
        }
        *reinterpret_cast<V*>(dst + pkf(tb, ks, nks, ln)) = v;
    }
}

// Layer 1's weights at the call start, in operand type and packed
// [din1][dout1] (rows are layer 1's inputs, K runs over its outputs).
template <class T>
__device__ void copy_layer1(const ScanArgs& a, long blk) {
    typedef typename Frag<T>::T V;
    const int nks = a.w1_dout >> 5;
    const long per = (long)(a.w1_din >> 4) * nks * 64;   // vectors per stream
    for (long e = blk * 256 + threadIdx.x; e < per * a.ns; e += 1024L * 256) {
        const long s = e / per, v = e - s * per;
        const int ln = (int)(v & 63);
        const long f = v >> 6;
        const int ks = (int)(f % nks), rb = (int)(f / nks);
        const int i = rb * 16 + (ln & 15), j = ks * 32 + 8 * (ln >> 4);
        const f32x8 w = ld8(a.w1_master + s * a.w1_ss + (long)i * a.w1_dout + j);
        V o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = (T)w[q];
        *reinterpret_cast<V*>(reinterpret_cast<T*>(a.w1_copy) + s * a.w1c_ss + (v << 3)) = o;
    }
}

__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
    const int x = (int)blockIdx.x;
    if (x >= a.scan_blocks + a.tr_blocks + a.pack_blocks) {
        const long blk = (long)x - a.scan_blocks - a.tr_blocks - a.pack_blocks;
        if (a.kt_f32) copy_layer1<float>(a, blk);
        else copy_layer1<bf16>(a, blk);
        return;
    }
    if (x >= a.scan_blocks + a.tr_blocks) {
        const long blk = (long)x - a.scan_blocks - a.tr_blocks;
        if (a.kt_f32) pack_rows<float>(a, blk);
        else pack_rows<bf16>(a, blk);
        return;
    }
    if (x >= a.scan_blocks) {
        const long blk = (long)x - a.scan_blocks;
        if (a.kt_f32) transpose_keys<float>(a, blk);
        else transpose_keys<bf16>(a, blk);
        return;
    }

    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.position) *a.position += a.add;
    const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= (long)a.ns * a.C) return;
    const int s = (int)(w / a.C), c = (int)(w - (long)s * a.C);
    const int b = a.b;
    const bool on = lane < b;
    const int t = c * b + lane;
    float th = 0.f, e = 1.f, oa = 1.f;
    if (on) {
        const long gi = tok_off(a.tl, s, t);
        th = a.theta[gi];
        e = a.eta[gi];
        oa = 1.0f - a.alpha[gi];
    }
    // inclusive suffix products over lanes i..63 (idle lanes contribute 1)
    float po = oa, pe = e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float o2 = shdown(po, off), e2 = shdown(pe, off);
        if (lane + off < 64) { po *= o2; pe *= e2; }
    }
    float A = shdown(po, 1), E = shdown(pe, 1);
    if (lane == 63) { A = 1.f; E = 1.f; }
    // r_i = A_i + eta_{i+1} r_{i+1}: suffix composition of x -> A_i + en_i x,
    // with en = 0 on the chunk's last token (r_{b-1} = 1) and beyond.
    float en = shdown(e, 1);
    if (lane + 1 >= b) en = 0.f;
    float fa = A, fm = en;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float a2 = shdown(fa, off), m2 = shdown(fm, off);
        if (lane + off < 64) { fa = fa + fm * a2; fm = fm * m2; }
    }
    const float r = fa;
    if (on) {
        a.cc[(long)s * a.coef_ss + t] = th * r;
        a.dc[(long)s * a.coef_ss + t] = th * E;
    }
    if (lane == 0) {
        float* o = a.cs + (long)s * a.cs_ss + (long)c * 4;
        o[0] = oa * A;   // p_alpha
        o[1] = e * E;    // p_eta
        o[2] = e * r;    // s0
        o[3] = 0.f;
    }
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    long waves = (long)a.ns * a.C;
    if (waves == 0) return hipSuccess;
    const long cp = a.w1_copy ? 1024 : 0;
    dim3 grid((unsigned)(a.scan_blocks + a.tr_blocks + a.pack_blocks + cp));
    hipLaunchKernelGGL(scan_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gradient reduction over the chunk + fused momentum / forgetting write.
// One workgroup per 64 x 64 tile of one layer's W (per stream):
//   U_M = H^T diag(c) Delta,  U_S = H^T diag(d) Delta   (K = the chunk's tokens)
//   S' = p_eta S - U_S,  M' = p_alpha M + s0 S - U_M,  Wt = bf16(M')^T.
// The producers left H^T, (c Delta)^T and (d Delta)^T token-contiguous, so
// each lane loads its 8 consecutive tokens straight from L2; the tile's M and
// S loads are issued first and overlap that work.  The results go through
// LDS once to switch from the matrix-core layout to row-contiguous float4
// accesses for M and S, and once more for the transposed bf16 copy.

template <class OP>
__device__ __forceinline__ typename Frag<OP>::T tok8(const OP* p, int t0, int b, bool full) {
    typedef typename Frag<OP>::T F;
    F v = cvt<OP>(ld8(p));
    if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (t0 + e >= b) v[e] = (OP)0.0f;
    }
    return v;
}

// tid: the thread's index among the tile's 256 threads.  A tile that is
// not live (padding of a workgroup that carries two tiles) computes on a
// valid tile and stores nothing; it still takes part in every barrier.
template <class OP>
__device__ void update_tile(const UpdArgs& u, int s, int tile, int tid, bool live, float (*UM)[65],
                            float (*US)[65]) {
    typedef typename Frag<OP>::T F;
    const int lane = tid & 63, wave = tid >> 6;
    int l = 0;
    while (l + 1 < u.L && tile >= u.tbase[l + 1]) ++l;
    tile -= u.tbase[l];
    const int ti = tile / u.tj[l], tj = tile - ti * u.tj[l];
    const int din = u.din[l], dout = u.dout[l];
    const int i0 = ti * 64, j0 = tj * 64;
    const int b = u.b, bp = u.bp;

    // U_M, U_S on the matrix cores: 4 waves as 2 x 2, 32 x 32 each
    const int wi = wave & 1, wj = wave >> 1;
    const int kofs = 8 * (lane >> 4);
    const int nkb = bp >> 5;
    const OP* A = reinterpret_cast<const OP*>(u.at[l]) + (long)s * u.at_ss[l];
    const OP* Bc = reinterpret_cast<const OP*>(u.dct[l]) + (long)s * u.dt_ss[l];
    const OP* Bd = reinterpret_cast<const OP*>(u.ddt[l]) + (long)s * u.dt_ss[l];
    int ab[2], bb[2];
    bool aok[2], bok[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        ab[m] = (i0 >> 4) + wi * 2 + m;     // 16-row blocks of W (packed operand rows)
        aok[m] = ab[m] * 16 < din;
        if (!aok[m]) ab[m] = 0;
        bb[m] = (j0 >> 4) + wj * 2 + m;
        bok[m] = bb[m] * 16 < dout;
        if (!bok[m]) bb[m] = 0;
    }
    // operand fragments first (vector loads complete in issue order, so
    // the matrix work below waits only for these), then this tile's M and
    // S, whose latency overlaps the matrix work and the LDS exchange
    // (every load is unconditional, from a clamped address, so the compiler
    // can wait for exactly the loads each step needs; unused values are
    // replaced by zeros)
    F fa[2][2], fc[2][2], fd[2][2];   // [k step][block]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int t0 = ks * 32 + kofs;
        const bool full = t0 + 8 <= b;
        const int kc = min(ks, nkb - 1);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            fa[ks][m] = tok8<OP>(A + pkf(ab[m], kc, nkb, lane), t0, b, full);
            fc[ks][m] = tok8<OP>(Bc + pkf(bb[m], kc, nkb, lane), t0, b, full);
            fd[ks][m] = tok8<OP>(Bd + pkf(bb[m], kc, nkb, lane), t0, b, full);
        }
    }
    float* Mp = u.M + (long)s * u.P + u.off[l];
    float* Sp = u.S + (long)s * u.P + u.off[l];
    f32x4 mreg[4], sreg[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q;
        const int gi = min(i0 + (idx >> 4), din - 1), gj = min(j0 + (idx & 15) * 4, dout - 4);
        const long o = (long)gi * dout + gj;
        mreg[q] = *reinterpret_cast<const f32x4*>(Mp + o);   // outside the layer: not used
        sreg[q] = *reinterpret_cast<const f32x4*>(Sp + o);
    }
    f32x4 am[2][2], as[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) { am[m][n] = (f32x4){0.f, 0.f, 0.f, 0.f}; as[m][n] = am[m][n]; }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        if (ks >= nkb) break;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const F av = aok[m] ? fa[ks][m] : zero_frag<OP>();
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                mma(am[m][n], av, bok[n] ? fc[ks][n] : zero_frag<OP>());
                mma(as[m][n], av, bok[n] ? fd[ks][n] : zero_frag<OP>());
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = wi * 32 + m * 16 + 4 * (lane >> 4) + e;
                const int c = wj * 32 + n * 16 + (lane & 15);
                UM[r][c] = am[m][n][e];
                US[r][c] = as[m][n][e];
            }
    __syncthreads();

    const float* csp = u.cs + (long)s * u.cs_ss + (long)u.chunk * 4;
    const float pa = csp[0], pe = csp[1], s0 = csp[2];
    bool bad = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q;
        const int i = idx >> 4, j = (idx & 15) * 4;
        const int gi = i0 + i, gj = j0 + j;
        if (live && gi < din && gj < dout) {
            const long o = (long)gi * dout + gj;
            const f32x4 m = mreg[q], sv = sreg[q];
            f32x4 mn, sn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sn[e] = pe * sv[e] - US[i][j + e];
                mn[e] = pa * m[e] + s0 * sv[e] - UM[i][j + e];
                bad |= !__builtin_isfinite(mn[e]) || !__builtin_isfinite(sn[e]);
                UM[i][j + e] = mn[e];
            }
            *reinterpret_cast<f32x4*>(Mp + o) = mn;
            *reinterpret_cast<f32x4*>(Sp + o) = sn;
        }
    }
    __syncthreads();
    // the tile of the bf16 forward copy Wt (packed [dout][din]): 4 column
    // blocks x 2 K steps x 64 lanes of 8 consecutive inputs, in memory order
    bf16* Wp = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P + u.off[l];
    for (int idx = tid; idx < 512; idx += 256) {
        const int ln = idx & 63, kk = (idx >> 6) & 1, jb = idx >> 7;
        const int jl = jb * 16 + (ln & 15), il = kk * 32 + 8 * (ln >> 4);
        if (live && j0 + jl < dout && i0 + il < din) {
            bf16x8 w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = (bf16)UM[il + e][jl];
            *reinterpret_cast<bf16x8*>(Wp + pkf((j0 >> 4) + jb, (i0 >> 5) + kk, din >> 5, ln)) = w;
        }
    }
    // layer 1's operand-type copy (packed [din][dout]) for the next chunk's
    // in-place backward of the first layer
    if (live && l == 1 && u.wr_next) {
        OP* wr = reinterpret_cast<OP*>(u.wr_next) + (long)s * u.wr_ss;
        for (int idx = tid; idx < 512; idx += 256) {
            const int ln = idx & 63, kk = (idx >> 6) & 1, ib = idx >> 7;
            const int il = ib * 16 + (ln & 15), jl = kk * 32 + 8 * (ln >> 4);
            if (i0 + il < din && j0 + jl < dout) {
                F w;
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = (OP)UM[il][jl + e];
                st8<OP>(wr + pkf((i0 >> 4) + ib, (j0 >> 5) + kk, dout >> 5, ln), w);
            }
        }
    }
    if (__ballot(bad) != 0 && lane == 0 && live) atomicOr(u.flag, 1);
}

template <class OP>
__global__ __launch_bounds__(256) void update_kernel(UpdArgs u) {
    __shared__ float UM[64][65];
    __shared__ float US[64][65];
    update_tile<OP>(u, blockIdx.y, blockIdx.x, threadIdx.x, true, UM, US);
}

hipError_t launch_update(const UpdArgs& u, int ntiles, int ns, int f32, hipStream_t st) {
    dim3 grid(ntiles, ns);
    if (f32) hipLaunchKernelGGL(update_kernel<float>, grid, dim3(256), 0, st, u);
    else hipLaunchKernelGGL(update_kernel<bf16>, grid, dim3(256), 0, st, u);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// First-layer part of a chunk step (see FirstArgs).

constexpr int WPAD = 8;     // LDS row padding (elements)
constexpr int RPAD = 1;     // LDS row padding of the partial-sum tiles (floats)
constexpr int FW = 8;       // waves of a first-layer workgroup

constexpr int FRED = FW / 2;   // partial tiles kept in LDS (two-round reduction)
constexpr size_t UPD_PAIR_LDS = 2 * 2 * 64 * 65 * 4;   // two update tiles: U_M, U_S each

static size_t first_lds_bytes(int dim, int bp, int f32) {
    const size_t e = f32 ? 4 : 2;
    return (size_t)JW * (dim + WPAD) * e + 2 * (size_t)JW * (bp + WPAD) * e +
           (size_t)FRED * 128 * (JW + RPAD) * 4;
}

// The waves' partial tiles acc (nb row blocks of 16 x JW) summed into FRED
// LDS slots in two rounds: waves FRED.. store theirs, waves 0..FRED-1 add
// their own.  Ends with a barrier; the caller sums the FRED slots.
template <int NB>
__device__ __forceinline__ void partial_tiles(float* red, const f32x4* acc, int nb, int rows, int wave, int lane,
                                              int RP) {
    const int g4 = 4 * (lane >> 4), jl = lane & 15;
    float* slot = red + (wave % FRED) * rows * RP;
    if (wave >= FRED) {
#pragma unroll
        for (int m = 0; m < NB; ++m)
            if (m < nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) slot[(16 * m + g4 + e) * RP + jl] = acc[m][e];
    }
    __syncthreads();
    if (wave < FRED) {
#pragma unroll
        for (int m = 0; m < NB; ++m)
            if (m < nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) slot[(16 * m + g4 + e) * RP + jl] += acc[m][e];
    }
    __syncthreads();
}

// Prefetch depths (in K steps or row blocks) of the first-layer workgroup:
// everything a wave needs is requested at kernel start when it fits the
// register file, so each phase waits for at most one round of memory.
template <class OP> struct FirstDepth;
template <> struct FirstDepth<bf16> { static constexpr int A = 2, B = 4, C = 2; };
template <> struct FirstDepth<float> { static constexpr int A = 1, B = 2, C = 1; };

template <class OP>
__global__ __launch_bounds__(FW * 64) void first_layer_kernel(FirstArgs a) {
    typedef typename Frag<OP>::T F;
    constexpr int PA = FirstDepth<OP>::A, PB = FirstDepth<OP>::B, PC = FirstDepth<OP>::C;
    constexpr int NT = FW * 64;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    if ((int)blockIdx.x >= a.nb1) {
        // the other layers' update tiles of chunk c-1, two per workgroup
        // (threads 0..255 and 256..511, each half with its own LDS tiles);
        // they touch nothing the first-layer blocks read or write
        const int half = threadIdx.x >> 8;
        int t = 2 * ((int)blockIdx.x - a.nb1) + half;
        const bool live = t < a.upd_ntiles;
        if (!live) t = a.upd_ntiles - 1;
        float(*UM)[65] = reinterpret_cast<float(*)[65]>(lds) + half * 128;
        update_tile<OP>(a.u, blockIdx.y, a.upd_tile0 + t, threadIdx.x & 255, live, UM, UM + 64);
        return;
    }
    const UpdArgs& u = a.u;
    const int s = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kofs = 8 * (lane >> 4), g4 = 4 * (lane >> 4);
    const int d = a.dim, h1 = a.h1, b = u.b, bp = u.bp;
    const int j0 = blockIdx.x * JW;
    const int jl = lane & 15, j = j0 + jl;   // the lane's column in B fragments / results
    const bool jok = j < h1;
    const int WP = d + WPAD, DP = bp + WPAD, RP = JW + RPAD;
    OP* Wn = reinterpret_cast<OP*>(lds);   // [JW][WP]: the block's columns of W_0, K-contiguous
    OP* DcT = Wn + JW * WP;                 // [JW][DP]: (c Delta_0)^T of chunk c-1
    OP* DdT = DcT + JW * DP;
    float* red = reinterpret_cast<float*>(DdT + JW * DP);   // [FRED][rows][RP] partial tiles
    float* M0 = u.M + (long)s * u.P;
    float* S0 = u.S + (long)s * u.P;
    bf16* Wt0 = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P;
    const OP* kt = reinterpret_cast<const OP*>(a.kt_prev) + (long)s * a.kt_ss;
    const bool upd = a.do_update;
    const bool bwd = upd && u.L >= 2;
    bool bad = false;

    // ================= every load of the kernel, in consumption order =================
    // (1) the in-place backward's operands: Delta_1 rows (4 token blocks) and
    //     the lane's column of W_1, K split over the waves
    const int K1 = bwd ? u.dout[1] : 32;
    const int nsA = K1 >> 5, qA = (nsA + FW - 1) / FW;
    const int kbA = wave * qA, keA = min(nsA, kbA + qA), klA = max(keA - 1, 0);
    const OP* Ad[4];
    bool tok[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        tok[m] = 16 * m + (lane & 15) < b;
        const int mb = 16 * m < b ? m : 0;   // token blocks past the chunk: valid address, dropped
        // without the backward: a harmless read of the first 2 KB of M
        Ad[m] = bwd ? reinterpret_cast<const OP*>(a.dlt2) + (long)s * a.dlt2_ss + pkf(mb, 0, nsA, lane)
                    : reinterpret_cast<const OP*>(M0) + lane * 8;
    }
    const OP* Bw = bwd ? reinterpret_cast<const OP*>(a.wr_prev) + (long)s * a.wr_ss + pkf(j0 >> 4, 0, nsA, lane)
                       : reinterpret_cast<const OP*>(M0) + lane * 8;
    // (every load below is unconditional and from a valid address, whether
    // or not this step uses it, so that the compiler waits for exactly the
    // loads each phase needs; the host points unused operands at valid memory)
    F ra[PA][4], rb[PA];
#pragma unroll
    for (int p = 0; p < PA; ++p) {
        const long k0 = (long)min(kbA + p, klA) << 9;
#pragma unroll
        for (int m = 0; m < 4; ++m) ra[p][m] = cvt<OP>(ld8(Ad[m] + k0));
        rb[p] = cvt<OP>(ld8(Bw + k0));
    }
    // (2) the backward epilogue's SiLU' and coefficients (2 elements per thread)
    constexpr int EA = 64 * JW / NT;
    float sl[EA], cv[EA], dv[EA];
#pragma unroll
    for (int q = 0; q < EA; ++q) {
        const int idx = tid + NT * q, t = min(idx / JW, b - 1), jj = j0 + idx % JW;
        sl[q] = *(bwd ? a.dsl1 + (long)s * a.dsl1_ss + (long)t * h1 + jj : M0 + (tid & 63));
        cv[q] = a.cc_prev[(long)s * a.coef_ss + t];
        dv[q] = a.dc_prev[(long)s * a.coef_ss + t];
    }
    // (3) the update's row blocks of this wave: keys^T fragments, M and S
    const int nrb = d >> 4;
    const int nkb = bp >> 5;
    const int mineB = upd ? (nrb - wave + FW - 1) / FW : 0;
    F kf[PB][2];
    float mr[PB][4], sr[PB][4];
    auto load_rb = [&](int p, int n) {
        // a wave without row blocks (mineB == 0) still loads a valid block
        const int rbk = min(wave + FW * max(min(n, mineB - 1), 0), nrb - 1);
        const int ib = 16 * rbk;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            kf[p][ks] = ks < nkb ? cvt<OP>(ld8(kt + pkf(rbk, ks, nkb, lane))) : zero_frag<OP>();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long o = (long)(ib + g4 + e) * h1 + (jok ? j : 0);
            mr[p][e] = M0[o];
            sr[p][e] = S0[o];
        }
    };
#pragma unroll
    for (int p = 0; p < PB; ++p) load_rb(p, p);
    // (4) the forward's rows (all 16-row blocks), K = dim split over the waves
    const int R = a.nq + a.nk;
    const int nrow = (R + 15) >> 4;
    const int nsC = d >> 5, qC = (nsC + FW - 1) / FW;
    const int kbC = wave * qC, keC = min(nsC, kbC + qC), klC = max(keC - 1, 0);
    // each lane's row: query rows of chunk c-1 first, then key rows of chunk
    // c, both packed per chunk
    const OP* Ax[8];
    bool rok[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        int r = 16 * m + (lane & 15);
        rok[m] = r < R;
        if (!rok[m]) r = R > 0 ? R - 1 : 0;
        const bool isq = r < a.nq;
        Ax[m] = reinterpret_cast<const OP*>(isq ? a.xq : a.xk) + (long)s * a.x_ss + pk(isq ? r : r - a.nq, kofs, nsC);
    }
    F rx[PC][8];
#pragma unroll
    for (int p = 0; p < PC; ++p)
#pragma unroll
        for (int m = 0; m < 8; ++m) rx[p][m] = cvt<OP>(ld8(Ax[m] + ((long)min(kbC + p, klC) << 9)));

    // ================= chunk c-1's update of the block's columns =================
    if (upd) {
        if (bwd) {
            // Delta_0 = (Delta_1 W_1^T) * SiLU'(z_0): 64 tokens x JW columns
            f32x4 acc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
            for (int k = kbA; k < kbA + qA; k += PA) {
#pragma unroll
                for (int p = 0; p < PA; ++p) {
                    const bool live = k + p < keA && k + p < kbA + qA;
                    const F bv = (live && jok) ? rb[p] : zero_frag<OP>();
#pragma unroll
                    for (int m = 0; m < 4; ++m) mma(acc[m], tok[m] ? ra[p][m] : zero_frag<OP>(), bv);
                    if (k + PA < kbA + qA) {   // wave-uniform: ring refill for long K
                        const long kn = (long)min(k + p + PA, klA) << 9;
#pragma unroll
                        for (int m = 0; m < 4; ++m) ra[p][m] = cvt<OP>(ld8(Ad[m] + kn));
                        rb[p] = cvt<OP>(ld8(Bw + kn));
                    }
                }
            }
            partial_tiles<4>(red, acc, 4, 64, wave, lane, RP);
#pragma unroll
            for (int q = 0; q < EA; ++q) {
                const int idx = tid + NT * q, t = idx / JW, cl = idx % JW;
                if (t >= bp) continue;
                float z = 0.f;
#pragma unroll
                for (int w = 0; w < FRED; ++w) z += red[(w * 64 + t) * RP + cl];
                const float dl = t < b ? z * sl[q] : 0.f;   // padding tokens: zero
                DcT[cl * DP + t] = (OP)(cv[q] * dl);
                DdT[cl * DP + t] = (OP)(dv[q] * dl);
            }
        } else {
            // depth 1: the previous chunk's forward left them in memory
            // (packed [h1][bp]; tokens past the chunk are zeroed here)
            for (int idx = tid; idx < JW * (bp >> 3); idx += NT) {
                const int cl = idx % JW, t8 = (idx / JW) * 8;
                const long o = (long)s * a.dt1_ss + pk(j0 + cl, t8, nkb);
                F vc = cvt<OP>(ld8(reinterpret_cast<const OP*>(a.dct1) + o));
                F vd = cvt<OP>(ld8(reinterpret_cast<const OP*>(a.ddt1) + o));
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t8 + e >= b) { vc[e] = (OP)0.0f; vd[e] = (OP)0.0f; }
                *reinterpret_cast<F*>(&DcT[cl * DP + t8]) = vc;
                *reinterpret_cast<F*>(&DdT[cl * DP + t8]) = vd;
            }
        }
        __syncthreads();

        // U = K^T diag(c) Delta_0 and the momentum / forgetting write, 16-row
        // blocks (block w, w+FW, ... for wave w)
        const float* csp = u.cs + (long)s * u.cs_ss + (long)a.chunk_prev * 4;
        const float pa = csp[0], pe = csp[1], s0 = csp[2];
        F bc[2], bd[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bool on = ks < nkb;
            bc[ks] = on ? *reinterpret_cast<const F*>(&DcT[jl * DP + ks * 32 + kofs]) : zero_frag<OP>();
            bd[ks] = on ? *reinterpret_cast<const F*>(&DdT[jl * DP + ks * 32 + kofs]) : zero_frag<OP>();
        }
        for (int n = 0; n < mineB; n += PB) {
#pragma unroll
            for (int p = 0; p < PB; ++p) {
                if (n + p < mineB) {   // wave-uniform
                    const int ib = 16 * (wave + FW * (n + p));
                    f32x4 um = (f32x4){0.f, 0.f, 0.f, 0.f}, us = um;
                    mma(um, kf[p][0], bc[0]);
                    mma(us, kf[p][0], bd[0]);
                    mma(um, kf[p][1], bc[1]);
                    mma(us, kf[p][1], bd[1]);
                    float mn[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float sn = pe * sr[p][e] - us[e];
                        mn[e] = pa * mr[p][e] + s0 * sr[p][e] - um[e];
                        bad |= jok && (!__builtin_isfinite(mn[e]) || !__builtin_isfinite(sn));
                        if (jok) {
                            const long o = (long)(ib + g4 + e) * h1 + j;
                            M0[o] = mn[e];
                            S0[o] = sn;
                        }
                        Wn[jl * WP + ib + g4 + e] = (OP)mn[e];
                    }
                    if (jok) {
                        // 4 consecutive inputs of output j: 8 contiguous bytes of packed Wt
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        *reinterpret_cast<bf16x4*>(Wt0 + pk(j, ib + g4, d >> 5)) =
                            (bf16x4){(bf16)mn[0], (bf16)mn[1], (bf16)mn[2], (bf16)mn[3]};
                    }
                }
                if (n + PB < mineB) load_rb(p, n + p + PB);   // wave-uniform refill
            }
        }
    } else if (a.do_fwd) {
        // first chunk of the call: the block's columns of the current W_0
        if (sizeof(OP) == 2) {
            for (int idx = tid; idx < JW * (d >> 3); idx += NT) {
                const int cl = idx % JW, i = (idx / JW) * 8;
                const int jj = j0 + cl;
                bf16x8 w = jj < h1 ? *reinterpret_cast<const bf16x8*>(Wt0 + pk(jj, i, d >> 5)) : zero_frag<bf16>();
                *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(Wn) + cl * WP + i) = w;
            }
        } else {
            for (int idx = tid; idx < JW * d; idx += NT) {
                const int i = idx / JW, cl = idx - i * JW;
                const int jj = j0 + cl;
                Wn[cl * WP + i] = jj < h1 ? (OP)M0[(long)i * h1 + jj] : (OP)0.0f;
            }
        }
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(u.flag, 1);
    if (!a.do_fwd) return;
    __syncthreads();

    // ================= chunk c's first-layer forward =================
    {
        f32x4 acc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int k = kbC; k < kbC + qC; k += PC) {
#pragma unroll
            for (int p = 0; p < PC; ++p) {
                const bool live = k + p < keC && k + p < kbC + qC;
                const int k0 = min(k + p, klC) << 5;
                F bv = *reinterpret_cast<const F*>(&Wn[jl * WP + k0 + kofs]);
                if (!live) bv = zero_frag<OP>();
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (m < nrow) mma(acc[m], rok[m] ? rx[p][m] : zero_frag<OP>(), bv);
                if (k + PC < kbC + qC) {   // wave-uniform ring refill
                    const long kn = (long)min(k + p + PC, klC) << 9;
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        if (m < nrow) rx[p][m] = cvt<OP>(ld8(Ax[m] + kn));
                }
            }
        }
        partial_tiles<8>(red, acc, nrow, 128, wave, lane, RP);
    }
    // z of every (row, column): the partial tiles summed into slot 0
    for (int idx = tid; idx < R * JW; idx += NT) {
        const int r = idx / JW, cl = idx - r * JW;
        float z = 0.f;
#pragma unroll
        for (int w = 0; w < FRED; ++w) z += red[(w * 128 + r) * RP + cl];
        red[r * RP + cl] = z;
    }
    __syncthreads();
    if (u.L >= 2) {
        // activations (packed [rows][h1]) and, for key rows, SiLU'(z)
        for (int idx = tid; idx < R * (JW / 8); idx += NT) {
            const int r = idx / (JW / 8), c8 = (idx % (JW / 8)) * 8, jj = j0 + c8;
            F hv;
            float sl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float z = red[r * RP + c8 + e];
                const float sg = sigmoid(z);
                hv[e] = (OP)(z * sg);
                sl[e] = sg * (1.0f + z * (1.0f - sg));
            }
            st8<OP>(reinterpret_cast<OP*>(a.act) + (long)s * a.act_ss + pk(r, jj, h1 >> 5), hv);
            if (r >= a.nq) st8f(a.dsl1 + (long)s * a.dsl1_ss + (long)(r - a.nq) * h1 + jj, sl);
        }
        // the key rows' activations transposed (packed [h1][bp], zero past the chunk)
        if (a.nk > 0) {
            for (int idx = tid; idx < JW * (bp >> 3); idx += NT) {
                const int cl = idx % JW, t8 = (idx / JW) * 8;
                F hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = t8 + e;
                    float h = 0.f;
                    if (t < a.nk) {
                        const float z = red[(a.nq + t) * RP + cl];
                        h = z * sigmoid(z);
                    }
                    hv[e] = (OP)h;
                }
                st8<OP>(reinterpret_cast<OP*>(a.ht1) + (long)s * a.ht_ss + pk(j0 + cl, t8, nkb), hv);
            }
        }
    } else {
        // depth 1: the first layer is the output layer
        for (int idx = tid; idx < a.nq * (JW / 8); idx += NT) {
            const int r = idx / (JW / 8), c8 = (idx % (JW / 8)) * 8;
            float z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = red[r * RP + c8 + e];
            st8f(a.y + tok_off(a.tl, s, a.tq0 + r) + j0 + c8, z);
        }
        if (a.nk > 0) {
            for (int idx = tid; idx < JW * (bp >> 3); idx += NT) {
                const int cl = idx % JW, t8 = (idx / JW) * 8, jj = j0 + cl;
                F vc, vd;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = t8 + e;
                    float xc = 0.f, xd = 0.f;
                    if (t < a.nk) {
                        const float z = red[(a.nq + t) * RP + cl];
                        const float dl = 2.0f * (z - load1<OP>(a.v, tok_off(a.tl, s, a.tk0 + t) + jj));
                        xc = a.cc_cur[(long)s * a.coef_ss + t] * dl;
                        xd = a.dc_cur[(long)s * a.coef_ss + t] * dl;
                    }
                    vc[e] = (OP)xc;
                    vd[e] = (OP)xd;
                }
                const long o = (long)s * a.dt1_ss + pk(jj, t8, nkb);
                st8<OP>(reinterpret_cast<OP*>(a.dct1) + o, vc);
                st8<OP>(reinterpret_cast<OP*>(a.ddt1) + o, vd);
            }
        }
    }
}

hipError_t launch_first(const FirstArgs& a, int ns, int f32, hipStream_t st) {
    const int pairs = (a.upd_ntiles + 1) / 2;
    dim3 grid(a.nb1 + pairs, ns);
    size_t lds = first_lds_bytes(a.dim, a.u.bp, f32);
    if (pairs > 0 && lds < UPD_PAIR_LDS) lds = UPD_PAIR_LDS;
    if (f32) hipLaunchKernelGGL(first_layer_kernel<float>, grid, dim3(FW * 64), lds, st, a);
    else hipLaunchKernelGGL(first_layer_kernel<bf16>, grid, dim3(FW * 64), lds, st, a);
    return hipGetLastError();
}

template <class OP>
__global__ __launch_bounds__(256) void update_range_kernel(UpdArgs u, int tile0) {
    __shared__ float UM[64][65];
    __shared__ float US[64][65];
    update_tile<OP>(u, blockIdx.y, tile0 + blockIdx.x, threadIdx.x, true, UM, US);
}

hipError_t launch_update_range(const UpdArgs& u, int tile0, int ntiles, int ns, int f32, hipStream_t st) {
    if (ntiles <= 0) return hipSuccess;
    dim3 grid(ntiles, ns);
    if (f32) hipLaunchKernelGGL(update_range_kernel<float>, grid, dim3(256), 0, st, u, tile0);
    else hipLaunchKernelGGL(update_range_kernel<bf16>, grid, dim3(256), 0, st, u, tile0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// State set-up, bf16 copy, export / import.

__global__ void init_kernel(float* M, float* S, const float* init, long P, int H, int ns) {
    const long n = (long)ns * P;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long s = i / P, p = i - s * P;
        M[i] = init[(s % H) * P + p];
        S[i] = 0.f;
    }
}

hipError_t launch_init(float* M, float* S, const float* init, long P, int H, int ns, hipStream_t st) {
    hipLaunchKernelGGL(init_kernel, dim3(2048), dim3(256), 0, st, M, S, init, P, H, ns);
    return hipGetLastError();
}

// Wt = bf16(M) packed [dout][din], per 64 x 64 tile (uses the layer / tile
// fields of UpdArgs).
__global__ __launch_bounds__(256) void shadow_kernel(UpdArgs u) {
    __shared__ float T[64][65];
    const int tid = threadIdx.x;
    const int s = blockIdx.y;
    int tile = blockIdx.x;
    int l = 0;
    while (l + 1 < u.L && tile >= u.tbase[l + 1]) ++l;
    tile -= u.tbase[l];
    const int ti = tile / u.tj[l], tj = tile - ti * u.tj[l];
    const int din = u.din[l], dout = u.dout[l];
    const int i0 = ti * 64, j0 = tj * 64;
    const float* Mp = u.M + (long)s * u.P + u.off[l];
    for (int idx = tid; idx < 64 * 64; idx += 256) {
        const int i = idx >> 6, j = idx & 63;
        T[i][j] = (i0 + i < din && j0 + j < dout) ? Mp[(long)(i0 + i) * dout + j0 + j] : 0.f;
    }
    __syncthreads();
    bf16* Wp = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P + u.off[l];
    for (int idx = tid; idx < 512; idx += 256) {
        const int ln = idx & 63, kk = (idx >> 6) & 1, jb = idx >> 7;
        const int jl = jb * 16 + (ln & 15), il = kk * 32 + 8 * (ln >> 4);
        if (j0 + jl < dout && i0 + il < din) {
            bf16x8 w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = (bf16)T[il + e][jl];
            *reinterpret_cast<bf16x8*>(Wp + pkf((j0 >> 4) + jb, (i0 >> 5) + kk, din >> 5, ln)) = w;
        }
    }
}

hipError_t launch_shadow(const UpdArgs& u, int ntiles, int ns, hipStream_t st) {
    hipLaunchKernelGGL(shadow_kernel, dim3(ntiles, ns), dim3(256), 0, st, u);
    return hipGetLastError();
}

__global__ void export_kernel(const float* M, const float* S, float* dst, long P, int ns) {
    const long n = (long)ns * P;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long s = i / P, p = i - s * P;
        dst[s * 2 * P + p] = M[i];
        dst[s * 2 * P + P + p] = S[i];
    }
}

__global__ void import_kernel(float* M, float* S, const float* src, long P, int ns) {
    const long n = (long)ns * P;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long s = i / P, p = i - s * P;
        M[i] = src[s * 2 * P + p];
        S[i] = src[s * 2 * P + P + p];
    }
}

hipError_t launch_export(const float* M, const float* S, float* dst, long P, int ns, hipStream_t st) {
    hipLaunchKernelGGL(export_kernel, dim3(2048), dim3(256), 0, st, M, S, dst, P, ns);
    return hipGetLastError();
}

hipError_t launch_import(float* M, float* S, const float* src, long P, int ns, hipStream_t st) {
    hipLaunchKernelGGL(import_kernel, dim3(2048), dim3(256), 0, st, M, S, src, P, ns);
    return hipGetLastError();
}

__global__ void header_kernel(StateHeader* h, uint64_t hash, int batch, int heads) {
    if (threadIdx.x == 0) {
        h->magic = STATE_MAGIC;
        h->version = STATE_VERSION;
        h->cfg_hash = hash;
        h->batch = batch;
        h->heads = heads;
        h->nonfinite = 0;
        h->reserved0 = 0;
        h->position = 0;
    }
}

hipError_t launch_header(StateHeader* h, uint64_t hash, int batch, int heads, hipStream_t st) {
    hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, st, h, hash, batch, heads);
    return hipGetLastError();
}

}  // namespace tmk
