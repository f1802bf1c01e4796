// HIP kernels for the Titans neural-memory store / retrieve on CDNA4 (gfx950).
//
// Per chunk of b tokens and per memory stream (one memory per sequence and
// head), the store is ("Titans, explained", steps 2-4 and 6; "Attack of the
// Titans", Parallel training): the forward of the keys through the
// chunk-start weights (with the queries of the previous chunk riding along as
// extra rows: both read the same weights), the backward of ||M(k) - v||^2 to
// every hidden layer, and the per-token gradients, weighted by coefficients
// of theta, eta and alpha, reduced over the chunk and folded into S and M in
// one pass over the state.  Per chunk step c the kernels are
//   first_layer_kernel  one workgroup per 16 hidden units j (per stream):
//                       chunk c-1's backward to layer 0 for the units (in
//                       place), the update of columns j of W_0 and rows j of
//                       W_1, and chunk c's layer-0 forward; update tiles of
//                       layers 2.. ride in the same launch (update_tile)
//   gemm_kernel         layers 1.. of chunk c's forward (the last one's
//                       epilogue gives y for the queries and Delta for the
//                       keys) and, for depth >= 3, the backward to layer 1
// and once per call scan_kernel (coefficients, packed operands).
// The coefficients come from a wave-level scan over the gates of each chunk:
// the momentum is a linear recurrence and the forgetting a running product,
// and unrolling both over a chunk whose gradients all sit at the chunk-start
// weights gives
//     S_end = p_eta S_0 - sum_i d_i G_i,
//     M_end = p_alpha M_0 + s0 S_0 - sum_i c_i G_i,
// with A_i = prod_{j>i} (1 - alpha_j), E_i = prod_{j>i} eta_j,
// r_i = A_i + eta_{i+1} r_{i+1} (r_b = 1), c_i = theta_i r_i, d_i = theta_i E_i,
// p_alpha = prod (1 - alpha), p_eta = prod eta, s0 = eta_1 r_1.  Only products
// and sums appear (no ratios of running products, which underflow).
//
// Matrix products run on MFMA: v_mfma_f32_16x16x32_bf16 for the bf16 path
// and v_mfma_f32_16x16x4_f32 for the fp32 path, fp32 accumulation in both.
#include "tm_device.h"

namespace tmk {

// ---------------------------------------------------------------------------
// Chunk forward / backward product.  A workgroup of W waves owns one tile of
// RT rows x 16*NR columns and splits its K range over the waves (wave w takes
// the w-th contiguous slice of 32-deep steps); the W partial tiles are summed
// in LDS in a fixed order, so results are deterministic and no workgroup ever
// waits for another (cross-workgroup handoffs need device-scope fences, which
// serialise across the whole chip).  Each lane feeds the matrix cores from
// registers loaded straight from global memory through a prefetch ring of PF
// steps, sized to the register budget; when a wave's slice fits the ring,
// all its loads are in flight at once.  The ring has no branches: steps past
// the end of a slice re-load a valid address and contribute zeros.  The
// epilogue's own operands (v or SiLU', the theta coefficients) are requested
// at kernel start too.
// OP: operand type; AT / BT: storage types of A / B; BM: B layout (B_*).

template <class OP> __device__ __forceinline__ void st8(OP* p, typename Frag<OP>::T v) {
    *reinterpret_cast<typename Frag<OP>::T*>(p) = v;
}
__device__ __forceinline__ void st8f(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = (f32x4){v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = (f32x4){v[4], v[5], v[6], v[7]};
}

// prefetch depth for a tile: about 96 registers of operand ring (8 values
// of each fragment per lane; a register holds 4 bytes)
constexpr int gemm_pf(int mr, int nr, int asz, int bsz) {
    const int per = (mr * asz + nr * bsz) * 2;   // registers per K step
    return 96 / per < 2 ? 2 : (96 / per > 8 ? 8 : 96 / per);
}

template <class OP, class AT, class BT, int BM, int RT, int NR, int W>
__global__ __launch_bounds__(W * 64) void gemm_kernel(GemmArgs g) {
    typedef typename Frag<OP>::T F;
    constexpr int MR = RT / 16;
    constexpr int NT = NR * 16;
    constexpr int NTP = NT + 1;            // padded LDS row
    constexpr int PF = gemm_pf(MR, NR, (int)sizeof(AT), (int)sizeof(BT));
    extern __shared__ float red[];          // [W][RT][NTP], then the tile's c, d coefficients
    float* coefs = red + W * RT * NTP;      // [2][RT]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the workgroup's stream and tile: the grid's own coordinates, or
    // (xcd_streams) remapped so that all tiles of a stream run on one XCD
    // (workgroups go to the 8 XCDs round-robin by linear id): the stream's
    // activations and weights are then fetched into one L2, not several
    int s = blockIdx.z, ty = blockIdx.y, tx = blockIdx.x;
    if (g.xcd_streams) {
        const int per = gridDim.x * gridDim.y;
        const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x, q = lin >> 3;
        s = (q / per) * 8 + (lin & 7);
        ty = (q % per) / gridDim.x;
        tx = (q % per) % gridDim.x;
    }
    const int row0 = ty * RT;
    const int col0 = tx * NT;
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
    constexpr long bstep = (BM == B_PACKED || BM == B_CFRAG) ? 512 : 32;
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        int cb = (col0 >> 4) + n;
        int c = cb * 16 + (lane & 15);
        bok[n] = c < g.N;
        if (!bok[n]) { cb = 0; c = lane & 15; }
        const BT* base = reinterpret_cast<const BT*>(g.b) + (long)s * g.b_ss;
        if constexpr (BM == B_PACKED) bcol[n] = base + pkf(cb, 0, nsteps, lane);
        else if constexpr (BM == B_ROWS) bcol[n] = base + (long)c * g.b_ld + kofs;
        else if constexpr (BM == B_CFRAG) bcol[n] = base + cf0(kofs, c, g.K >> 4);
        else if constexpr (BM == B_CF1) bcol[n] = base + cf1(kofs, c, g.N >> 4);
        else bcol[n] = base + c + (long)kofs * g.b_ld;
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
            if constexpr (BM == B_PACKED || BM == B_ROWS) {
                bb[p][n] = ld8(bcol[n] + k * bstep);
            } else if constexpr (BM == B_CF1) {
                // inputs kofs .. kofs+7 of output c: 8 lanes' slots, 4 floats apart
                const BT* q = bcol[n] + k * (2L * (g.N >> 4) * 256);
                RB u;
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] = q[4 * e];
                bb[p][n] = u;
            } else if constexpr (BM == B_CFRAG) {
                // rows kofs..kofs+3 and kofs+4..kofs+7 of the column: two
                // float4 one 16-lane group apart
                const BT* q = bcol[n] + k * bstep;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(q);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(q + 64);
                bb[p][n] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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

    // the epilogue's operands, requested now (unused ones read a valid
    // address): pass 1's first item (v or SiLU' of 8 columns of one row) and
    // the c, d coefficient of token (this thread's row) for pass 2
    typedef typename Frag<OP>::T RV;
    RV vpre;
    f32x8 spre;
    float cpre = 0.f, dpre = 0.f;
    {
        const int rr = tid / (NT / 8), cc = (tid % (NT / 8)) * 8;
        const int r = min(row0 + rr, g.nrows - 1), c = min(col0 + cc, g.N - 8);
        const int t = max(r - g.n0, 0);
        // v only where the product has key rows (their tokens vt0 .. vt0 + nk - 1)
        const bool keys = g.epi == EPI_OUT && g.v && g.nrows > g.n0;
        const OP* vp = keys ? reinterpret_cast<const OP*>(g.v) + tok_off(g.tl, s, g.vt0 + t) + c
                            : reinterpret_cast<const OP*>(g.b);
        vpre = ld8(vp);
        const float* sp = g.epi == EPI_BWD ? g.dsl + (long)s * g.dsl_ss + (long)r * g.dsl_ld + c
                                           : reinterpret_cast<const float*>(g.b);
        spre = ld8(sp);
        if (g.dct) {
            const int tt = min(max(row0 + (tid % RT) - g.n0, 0), g.nrows - g.n0 - 1);
            cpre = g.cc[(long)s * g.coef_ss + tt];
            dpre = g.dc[(long)s * g.coef_ss + tt];
        }
    }

    for (int k = kb; k < kb + spw; k += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            // steps past the wave's slice issue no matrix instruction
            // (wave-uniform; their ring slots still reload a valid address)
            if (k + p < ke) {
                F av[MR], bv[NR];
#pragma unroll
                for (int m = 0; m < MR; ++m) av[m] = aok[m] ? cvt<OP>(a[p][m]) : zero_frag<OP>();
#pragma unroll
                for (int n = 0; n < NR; ++n) bv[n] = bok[n] ? cvt<OP>(bb[p][n]) : zero_frag<OP>();
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int n = 0; n < NR; ++n) mma(acc[m][n], av[m], bv[n]);
            }
            load_step(p, min(k + p + PF, klast));
        }
    }

    // sum the W partial tiles in LDS, in wave order
    float* mine = red + wave * (RT * NTP);
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int n = 0; n < NR; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mine[(m * 16 + 4 * (lane >> 4) + e) * NTP + n * 16 + (lane & 15)] = acc[m][n][e];
    if (tid < RT) {
        coefs[tid] = cpre;
        coefs[RT + tid] = dpre;
    }
    __syncthreads();
    // pass 1: row outputs, 8 consecutive columns per thread (N is a multiple
    // of 32); the value for the transposed copy is left in slot 0
    for (int idx = tid; idx < RT * (NT / 8); idx += W * 64) {
        const int rr = idx / (NT / 8), cc = (idx - rr * (NT / 8)) * 8;
        const int r = row0 + rr, c = col0 + cc;
        if (r >= g.nrows || c >= g.N) continue;
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) x += red[w * (RT * NTP) + rr * NTP + cc + e];
            z[e] = x;
        }
        typename Frag<OP>::T o;
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
        } else if (g.epi == EPI_OUT && r < g.n0) {
            st8f(g.y + tok_off(g.tl, s, g.yt0 + r) + c, z);
        } else {
            const int t = r - g.n0;
            if (g.epi == EPI_OUT) {
                const f32x8 vv = to_f32v(idx == tid ? vpre : ld8(reinterpret_cast<const OP*>(g.v) +
                                                              tok_off(g.tl, s, g.vt0 + t) + c));
#pragma unroll
                for (int e = 0; e < 8; ++e) z[e] = 2.0f * (z[e] - vv[e]);
            } else {
                const f32x8 sl = idx == tid ? spre : ld8(g.dsl + (long)s * g.dsl_ss + (long)r * g.dsl_ld + c);
#pragma unroll
                for (int e = 0; e < 8; ++e) z[e] = z[e] * sl[e];
            }
            if (g.dlp) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (OP)z[e];
                st8<OP>(reinterpret_cast<OP*>(g.dlp) + (long)s * g.dlp_ss + pk(t, c, g.N >> 5), o);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) red[rr * NTP + cc + e] = z[e];
    }
    if (!g.ht && !g.dct) return;   // uniform: no transposed outputs (retrieve)
    __syncthreads();
    // pass 2: the key rows' transposed copies, packed [N][bp]: 8 tokens of
    // one column per thread, whole vectors where all 8 tokens are this
    // tile's rows (a group cut by the tile edge is stored element-wise)
    const int tlo = max(row0, g.n0) - g.n0, thi = min(row0 + RT, g.nrows) - g.n0;
    if (thi <= tlo) return;
    const int g0 = tlo >> 3, ng = ((thi - 1) >> 3) - g0 + 1;
    const int nkb = g.bp >> 5;
    for (int idx = tid; idx < NT * ng; idx += W * 64) {
        const int cc = idx % NT, t8 = (g0 + idx / NT) * 8;
        const int c = col0 + cc;
        if (c >= g.N) continue;
        float x[8];
        bool in[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t8 + e;
            in[e] = t >= tlo && t < thi;
            x[e] = in[e] ? red[(t + g.n0 - row0) * NTP + cc] : 0.f;
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
                    if (in[e]) h[e] = (OP)x[e];
            }
        } else {
            // the tile's coefficients, staged in LDS by row
            OP* pc = reinterpret_cast<OP*>(g.dct) + o;
            OP* pd = reinterpret_cast<OP*>(g.ddt) + o;
            F vc, vd;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int rr = min(max(t8 + e + g.n0 - row0, 0), RT - 1);
                vc[e] = (OP)(coefs[rr] * x[e]);
                vd[e] = (OP)(coefs[RT + rr] * x[e]);
            }
            if (whole) {
                st8<OP>(pc, vc);
                st8<OP>(pd, vd);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (in[e]) {
                        pc[e] = vc[e];
                        pd[e] = vd[e];
                    }
            }
        }
    }
}

// The tile shape and wave count of one product: prefer tiles whose K slice
// per wave fits the prefetch ring (one memory round trip) and enough
// workgroups to cover the chip, then the widest tile (activations re-read
// from L2 by fewer workgroups).
struct GemmShape {
    int rt, nr, w;
};

template <class AT, class BT>
static GemmShape pick(const GemmArgs& g, int ns) {
    const int nsteps = g.K >> 5;
    static const int cand[5][2] = {{64, 4}, {64, 2}, {32, 2}, {64, 1}, {32, 1}};
    GemmShape best{64, 1, 8};
    long best_score = -1;
    for (const auto& cd : cand) {
        const int rt = cd[0], nr = cd[1];
        const int pf = gemm_pf(rt / 16, nr, (int)sizeof(AT), (int)sizeof(BT));
        const int w = nsteps >= 16 ? 8 : 4;
        const int spw = (nsteps + w - 1) / w;
        const long wgs = (long)((g.N + 16 * nr - 1) / (16 * nr)) * ((g.nrows + rt - 1) / rt) * ns;
        // one round trip and a full chip first; then more workgroups; then
        // the wider tile (earlier candidates)
        const long score = (spw <= pf ? 4000000 : 0) + (wgs >= 192 ? 2000000 : 0) + (wgs < 192 ? wgs * 1000 : 0) +
                           (5 - (&cd - cand));
        if (score > best_score) {
            best_score = score;
            best = GemmShape{rt, nr, w};
        }
    }
    return best;
}

template <class OP, class AT, class BT, int BM, int RT, int NR, int W>
static void launch_one(const GemmArgs& g, int ns, hipStream_t st) {
    dim3 grid((g.N + NR * 16 - 1) / (NR * 16), (g.nrows + RT - 1) / RT, ns);
    const size_t lds = ((size_t)W * RT * (NR * 16 + 1) + 2 * RT) * 4;
    launch_k((gemm_kernel<OP, AT, BT, BM, RT, NR, W>), grid, dim3(W * 64), lds, st, g);
}

template <class OP, class AT, class BT, int BM, int RT, int W>
static void launch_nr(const GemmArgs& g, int ns, int nr, hipStream_t st) {
    if (nr == 4) launch_one<OP, AT, BT, BM, RT, 4, W>(g, ns, st);
    else if (nr == 2) launch_one<OP, AT, BT, BM, RT, 2, W>(g, ns, st);
    else launch_one<OP, AT, BT, BM, RT, 1, W>(g, ns, st);
}

template <class OP, class AT, class BT, int BM>
static hipError_t launch_gemm(const GemmArgs& g, int ns, hipStream_t st) {
    if (g.nrows <= 0 || g.N <= 0) return hipSuccess;
    if (g.xcd_streams && ns % 8 != 0) return hipErrorInvalidValue;
    const GemmShape sh = pick<AT, BT>(g, ns);
    if (sh.rt == 64) {
        if (sh.w == 8) launch_nr<OP, AT, BT, BM, 64, 8>(g, ns, sh.nr, st);
        else launch_nr<OP, AT, BT, BM, 64, 4>(g, ns, sh.nr, st);
    } else {
        if (sh.w == 8) launch_nr<OP, AT, BT, BM, 32, 8>(g, ns, sh.nr, st);
        else launch_nr<OP, AT, BT, BM, 32, 4>(g, ns, sh.nr, st);
    }
    return hipGetLastError();
}

hipError_t launch_fwd(const GemmArgs& g, int ns, int f32, hipStream_t st) {
    if (f32) {
        if (g.bmode == B_CFRAG) return launch_gemm<float, float, float, B_CFRAG>(g, ns, st);
        if (g.bmode == B_CF1) return launch_gemm<float, float, float, B_CF1>(g, ns, st);
        return launch_gemm<float, float, float, B_STRIDED>(g, ns, st);
    }
    return launch_gemm<bf16, bf16, bf16, B_PACKED>(g, ns, st);
}

hipError_t launch_bwd(const GemmArgs& g, int ns, int f32, hipStream_t st) {
    if (f32) return launch_gemm<float, float, float, B_ROWS>(g, ns, st);
    return launch_gemm<bf16, bf16, float, B_ROWS>(g, ns, st);
}

// ---------------------------------------------------------------------------
// Coefficient scan: one wave per (stream, chunk), lane i = token i of the chunk.

__device__ __forceinline__ float shdown(float x, int off) { return __shfl_down(x, off, 64); }

// The chunk's coefficients, one wave, lane i = token i (idle lanes past the
// chunk contribute the identity).
__device__ void scan_gates(const ScanArgs& a, int s, int c) {
    const int lane = threadIdx.x & 63;
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

// One workgroup per (stream, chunk, slice of SCAN_SLICE features): the
// slice's key and query rows of the chunk packed ([b][d] per chunk: rows are
// tokens, K runs over the features), its keys also transposed through LDS
// ([d][bp] per chunk: rows are features, K runs over the chunk's tokens), and
// in slice 0 the chunk's coefficients.  Every row is read once, 8 features
// (16 or 32 bytes) per lane; tokens past the chunk are zero.
constexpr int SCAN_SLICE = 128;

constexpr int SCAN_TP = SCAN_SLICE + 8;   // tile row pitch (elements)

template <class T>
__device__ void scan_rows(const ScanArgs& a, int s, int c, int f0, char* lds) {
    typedef typename Frag<T>::T V;
    T(*tile)[SCAN_TP] = reinterpret_cast<T(*)[SCAN_TP]>(lds);   // [token][feature of the slice]
    const int d = a.ktl.d, b = a.b, nks = d >> 5, nkb = a.bp >> 5;
    const int nf = min(SCAN_SLICE, d - f0), nbt = (b + 15) >> 4;
    const int items = nbt * (nf >> 5) * 64;   // 8-feature pieces per tensor (fragment order)
    // every piece of the thread (at most PER: a chunk of 64 tokens, a slice
    // of 128 features) is requested before any is stored: loads and stores
    // interleaved in a loop would wait a memory round trip per piece, the
    // compiler unable to move a load above a store that might alias it.
    // Keys first, then queries.
    constexpr int PER = (MAX_CHUNK / 16) * (SCAN_SLICE / 32) * 64 / 256;
    int po[PER], pt[PER], pf[PER];
    long ps[PER];
    bool live[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = threadIdx.x + 256 * u;
        const int ln = idx & 63, f = idx >> 6, ksl = f % (nf >> 5), tb = f / (nf >> 5);
        const int t = tb * 16 + (ln & 15), fl = ksl * 32 + 8 * (ln >> 4);
        live[u] = idx < items && t < b;
        // pieces past the chunk or the slice read a valid row and are zeroed
        ps[u] = tok_off(a.ktl, s, c * b + min(t, b - 1)) + f0 + (idx < items ? fl : 0);
        po[u] = idx < items ? pkf(tb, (f0 >> 5) + ksl, nks, ln) : -1;
        pt[u] = t;
        pf[u] = fl;
    }
    for (int kq = 0; kq < (a.q ? 2 : 1); ++kq) {
        const T* src = reinterpret_cast<const T*>(kq ? a.q : a.k);
        T* dst = reinterpret_cast<T*>(kq ? a.xq : a.xk) + ((long)s * a.C + c) * a.xc;
        V v[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) v[u] = keep_if(ld8(src + ps[u]), live[u]);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            if (po[u] < 0) continue;
            *reinterpret_cast<V*>(dst + po[u]) = v[u];
            if (kq == 0 && pt[u] < MAX_CHUNK) *reinterpret_cast<V*>(&tile[pt[u]][pf[u]]) = v[u];
        }
    }
    // rows of the tile past the packed ones (tokens up to bp) are zero
    for (int idx = threadIdx.x; idx < (a.bp - nbt * 16) * (nf >> 3); idx += 256) {
        const int t = nbt * 16 + idx / (nf >> 3), fl = (idx % (nf >> 3)) * 8;
        V z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (T)0.0f;
        *reinterpret_cast<V*>(&tile[t][fl]) = z;
    }
    __syncthreads();
    T* kt = reinterpret_cast<T*>(a.kt) + ((long)s * a.C + c) * (long)d * a.bp;
    for (int idx = threadIdx.x; idx < (nf >> 4) * nkb * 64; idx += 256) {
        const int ln = idx & 63, ks = (idx >> 6) % nkb, rb = (idx >> 6) / nkb;
        const int i = rb * 16 + (ln & 15), t8 = ks * 32 + 8 * (ln >> 4);
        V v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[t8 + e][i];
        *reinterpret_cast<V*>(kt + pkf((f0 >> 4) + rb, ks, nkb, ln)) = v;
    }
}

__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
    const int nsl = (a.ktl.d + SCAN_SLICE - 1) / SCAN_SLICE;
    const long x = blockIdx.x;
    const int sl = (int)(x % nsl);
    const long sc = x / nsl;
    const int c = (int)(sc % a.C), s = (int)(sc / a.C);
    if (x == 0 && threadIdx.x == 0 && a.position) *a.position += a.add;
    if (sl == 0 && threadIdx.x < 64) scan_gates(a, s, c);
    __shared__ __attribute__((aligned(16))) char lds[MAX_CHUNK * SCAN_TP * 4];
    if (a.kt_f32) scan_rows<float>(a, s, c, sl * SCAN_SLICE, lds);
    else scan_rows<bf16>(a, s, c, sl * SCAN_SLICE, lds);
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    const long blocks = (long)a.ns * a.C * ((a.ktl.d + SCAN_SLICE - 1) / SCAN_SLICE);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffL || a.b > MAX_CHUNK || a.bp > MAX_CHUNK || a.ktl.d % 32 != 0) return hipErrorInvalidValue;
    launch_k(scan_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
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

// 8 consecutive tokens t0 .. t0+7 of a transposed operand, zero past the
// chunk (selects, no branch: a branch here would make the compiler wait for
// every load in flight)
template <class OP>
__device__ __forceinline__ typename Frag<OP>::T tok8(const OP* p, int t0, int b) {
    typedef typename Frag<OP>::T F;
    F v = cvt<OP>(ld8(p));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t0 + e < b ? v[e] : (OP)0.0f;
    return v;
}

// One tile's loaded operands and state, between tile_load and tile_finish.
template <class OP>
struct TileIn {
    typedef typename Frag<OP>::T F;
    int din, dout, i0, j0;
    long off;
    float pa, pe, s0;
    bool aok[2], bok[2];
    F fa[2][2], fc[2][2], fd[2][2];   // [k step][block]
    f32x4 mreg[4], sreg[4];
};

// tid: the thread's index among the tile's 256 threads.  Every load of the
// tile, in consumption order: the chunk scalars, the operand fragments (the
// matrix work waits only for these), then the tile's M and S, whose latency
// overlaps the matrix work and the LDS exchange.  Every load is
// unconditional, from a clamped address, so the compiler waits for exactly
// the loads each step needs; unused values are replaced by zeros.
template <class OP>
__device__ __forceinline__ void tile_load(TileIn<OP>& T, const UpdArgs& u, int s, int tile, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    // the tile's layer and its parameters, picked by compare and select (an
    // index computed at run time into the kernel arguments would become a
    // chain of dependent memory loads)
    int l = 0;
#pragma unroll
    for (int q = 1; q < MAXL; ++q)
        if (q < u.L && tile >= u.tbase[q]) l = q;
    int tb = 0, tjn = 1, din = 32, dout = 32;
    long off = 0, at_ss = 0, dt_ss = 0;
    const void* atp = nullptr;
    const void* dcp = nullptr;
    const void* ddp = nullptr;
#pragma unroll
    for (int q = 0; q < MAXL; ++q)
        if (q == l) {
            tb = u.tbase[q];
            tjn = u.tj[q];
            din = u.din[q];
            dout = u.dout[q];
            off = u.off[q];
            atp = u.at[q];
            at_ss = u.at_ss[q];
            dcp = u.dct[q];
            ddp = u.ddt[q];
            dt_ss = u.dt_ss[q];
        }
    tile -= tb;
    const int ti = tile / tjn, tj = tile - ti * tjn;
    T.din = din;
    T.dout = dout;
    T.off = off;
    T.i0 = ti * 64;
    T.j0 = tj * 64;
    const int b = u.b, bp = u.bp;
    const float* csp = u.cs + (long)s * u.cs_ss + (long)u.chunk * 4;
    T.pa = csp[0];
    T.pe = csp[1];
    T.s0 = csp[2];
    // U_M, U_S on the matrix cores: 4 waves as 2 x 2, 32 x 32 each
    const int wi = wave & 1, wj = wave >> 1;
    const int kofs = 8 * (lane >> 4);
    const int nkb = bp >> 5;
    const OP* A = reinterpret_cast<const OP*>(atp) + (long)s * at_ss;
    const OP* Bc = reinterpret_cast<const OP*>(dcp) + (long)s * dt_ss;
    const OP* Bd = reinterpret_cast<const OP*>(ddp) + (long)s * dt_ss;
    int ab[2], bb[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        ab[m] = (T.i0 >> 4) + wi * 2 + m;     // 16-row blocks of W (packed operand rows)
        T.aok[m] = ab[m] * 16 < din;
        if (!T.aok[m]) ab[m] = 0;
        bb[m] = (T.j0 >> 4) + wj * 2 + m;
        T.bok[m] = bb[m] * 16 < dout;
        if (!T.bok[m]) bb[m] = 0;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int t0 = ks * 32 + kofs;
        const int kc = min(ks, nkb - 1);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            T.fa[ks][m] = tok8<OP>(A + pkf(ab[m], kc, nkb, lane), t0, b);
            T.fc[ks][m] = tok8<OP>(Bc + pkf(bb[m], kc, nkb, lane), t0, b);
            T.fd[ks][m] = tok8<OP>(Bd + pkf(bb[m], kc, nkb, lane), t0, b);
        }
    }
    const float* Mp = u.M + (long)s * u.P + off;
    const float* Sp = u.S + (long)s * u.P + off;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q;
        const int gi = min(T.i0 + (idx >> 4), din - 1), gj = min(T.j0 + (idx & 15) * 4, dout - 4);
        const long o = (long)gi * dout + gj;
        T.mreg[q] = *reinterpret_cast<const f32x4*>(Mp + o);   // outside the layer: not used
        T.sreg[q] = *reinterpret_cast<const f32x4*>(Sp + o);
    }
}

// The tile's products, the momentum / forgetting write and the bf16 copy.
// A tile that is not live (padding of a workgroup) computes on a valid tile
// and stores nothing; it still takes part in every barrier.
template <class OP>
__device__ void tile_finish(const TileIn<OP>& T, const UpdArgs& u, int s, int tid, bool live,
                            float (*UM)[65], float (*US)[65]) {
    typedef typename Frag<OP>::T F;
    const int lane = tid & 63, wave = tid >> 6;
    const int wi = wave & 1, wj = wave >> 1;
    const int nkb = u.bp >> 5;
    const int din = T.din, dout = T.dout, i0 = T.i0, j0 = T.j0;
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
            const F av = T.aok[m] ? T.fa[ks][m] : zero_frag<OP>();
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                mma(am[m][n], av, T.bok[n] ? T.fc[ks][n] : zero_frag<OP>());
                mma(as[m][n], av, T.bok[n] ? T.fd[ks][n] : zero_frag<OP>());
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

    float* Mp = u.M + (long)s * u.P + T.off;
    float* Sp = u.S + (long)s * u.P + T.off;
    bool bad = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q;
        const int i = idx >> 4, j = (idx & 15) * 4;
        const int gi = i0 + i, gj = j0 + j;
        if (live && gi < din && gj < dout) {
            const long o = (long)gi * dout + gj;
            const f32x4 m = T.mreg[q], sv = T.sreg[q];
            f32x4 mn, sn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sn[e] = mom_s(T.pe, sv[e], US[i][j + e]);
                mn[e] = mom_m(T.pa, m[e], T.s0, sv[e], UM[i][j + e]);
                bad |= !__builtin_isfinite(mn[e]) || !__builtin_isfinite(sn[e]);
                UM[i][j + e] = mn[e];
            }
            st_state(Mp + o, mn);
            st_state(Sp + o, sn);
        }
    }
    __syncthreads();
    // the tile of the bf16 forward copy Wt (packed [dout][din]): 4 column
    // blocks x 2 K steps x 64 lanes of 8 consecutive inputs, in memory order
    bf16* Wp = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P + T.off;
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
    // the LDS tiles are reused by the half's next tile
    __syncthreads();
    if (__ballot(bad) != 0 && lane == 0 && live) atomicOr(u.flag, 1);
}

// ---------------------------------------------------------------------------
// First-layer part of a chunk step (see FirstArgs).

constexpr int WPAD = 8;     // LDS row padding (elements)
constexpr int RPAD = 1;     // LDS row padding of the partial-sum tiles (floats)
constexpr int FW = 8;       // waves of a first-layer workgroup

// (a workgroup of NW waves keeps NW / 2 partial tiles in LDS: two-round reduction)
constexpr size_t UPD_TILE_LDS = 2 * 2 * 64 * 65 * 4;   // the two halves' update tiles: U_M, U_S each
// Update tiles per workgroup: two per half (both tiles' loads in flight
// together) where the register budget holds them, one per half in the
// half-occupancy (small) and fp32 variants.
__host__ __device__ constexpr int upd_tpw(bool f32, bool small) { return (!f32 && !small) ? 4 : 2; }

static size_t first_lds_bytes(int dim, int bp, int f32, int nw) {
    const size_t e = f32 ? 4 : 2;
    (void)bp;
    return (size_t)JW * (dim + WPAD) * e + 2 * (size_t)JW * (MAX_CHUNK + WPAD) * e +
           (size_t)(nw / 2) * 128 * (JW + RPAD) * 4;
}

// The waves' partial tiles acc (nb row blocks of 16 x JW) summed into FR
// LDS slots in two rounds: waves FR.. store theirs, waves 0..FR-1 add
// their own.  Ends with a barrier; the caller sums the FR slots.
template <int NB, int FR>
__device__ __forceinline__ void partial_tiles(float* red, const f32x4* acc, int nb, int rows, int wave, int lane,
                                              int RP) {
    const int g4 = 4 * (lane >> 4), jl = lane & 15;
    float* slot = red + (wave % FR) * rows * RP;
    if (wave >= FR) {
#pragma unroll
        for (int m = 0; m < NB; ++m)
            if (m < nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) slot[(16 * m + g4 + e) * RP + jl] = acc[m][e];
    }
    __syncthreads();
    if (wave < FR) {
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
// SMALL (dim and layer 1's outputs at most 128): with 8 waves every wave has
// one K step or row block per phase, so depth 1 everywhere and two
// workgroups per compute unit (the register budget halves); with 4 waves
// (launches without other roles) two row blocks and two W_1 blocks per
// wave, one K step, three workgroups per compute unit.
template <class OP, bool SMALL, int NW> struct FirstDepth;
template <> struct FirstDepth<bf16, false, 8> { static constexpr int A = 2, B = 3, C = 2, N = 3; };
template <> struct FirstDepth<float, false, 8> { static constexpr int A = 1, B = 2, C = 1, N = 3; };
template <class OP> struct FirstDepth<OP, true, 8> { static constexpr int A = 1, B = 1, C = 1, N = 1; };
template <class OP> struct FirstDepth<OP, true, 4> { static constexpr int A = 1, B = 2, C = 1, N = 2; };
constexpr int SMALL_DIM = 128;

// W_1's update as a workgroup role of its own (depth 2, with workgroups to
// spare): workgroup wg of stream s updates W1_JPW row blocks of W_1 for
// chunk c-1.  Workgroups go to the 8 XCDs round-robin by linear id, and a
// row block is given to a workgroup on the XCD of the first-layer block that
// reads those rows in the next launch, so that the rows are still in that
// XCD's L2: block jb sits at x = jb and this workgroup at x = nb1 + wg of the
// same grid row, so the row blocks jb = r, r + 8, ... with r = (nb1 + wg) mod 8
// are the candidates, W1_JPW of them per workgroup of that residue (nw1 is
// a multiple of 8).  Each block is computed transposed as in the first-layer
// blocks, U^T = (c Delta_1)^T H_1 (rows: layer 1's outputs n in 16-blocks
// nb = wave, wave + FW, ...; columns: the block's 16 inputs j; K: tokens).
// The (c Delta_1)^T fragments depend on the outputs only, so a wave loads
// them once for all its row blocks, and every row block's H_1 fragments and
// M / S values are requested at once, before any is used.  M_1 is read from
// m1_rd and written to m1_wr, never the buffer the first-layer blocks of the
// same launch read.  Row blocks past h1 re-read the last one and are dropped.
constexpr int W1_PN = 3;   // output blocks per wave held in registers
constexpr size_t W1_LDS = (size_t)FW * 16 * W1_PN * 24 * 2;   // the waves' bf16 tiles

template <class OP>
__device__ void w1_rows(const FirstArgs& a, int s, int wg, char* lds) {
    typedef typename Frag<OP>::T F;
    const UpdArgs& u = a.u;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kofs = 8 * (lane >> 4), g4 = 4 * (lane >> 4), jl = lane & 15;
    const int b = u.b, nkb = u.bp >> 5, h1 = a.h1;
    const int ncb1 = u.dout[1] >> 4;
    const int mine1 = (ncb1 - wave + FW - 1) / FW;
    const float* csp = u.cs + (long)s * u.cs_ss + (long)a.chunk_prev * 4;
    const float pa = csp[0], pe = csp[1], s0 = csp[2];
    const OP* at1 = reinterpret_cast<const OP*>(u.at[1]) + (long)s * u.at_ss[1];
    const OP* dc1 = reinterpret_cast<const OP*>(u.dct[1]) + (long)s * u.dt_ss[1];
    const OP* dd1 = reinterpret_cast<const OP*>(u.ddt[1]) + (long)s * u.dt_ss[1];
    const float* Mr = a.m1_rd + (long)s * a.m1_rd_ss;
    float* Mw = a.m1_wr + (long)s * a.m1_wr_ss;
    float* S1 = u.S + (long)s * u.P + u.off[1];
    bf16* Wt1 = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P + u.off[1];
    const int xr = (a.nb1 + wg) & 7, jb0 = xr + 8 * W1_JPW * (wg >> 3);   // row blocks jb0 + 8q
    bool bad = false;
    auto mso1 = [&](int jb, int nb) { return ((long)(jb * ncb1 + nb) * 64 + lane) * 4; };
    auto nbp = [&](int n) { return min(wave + FW * n, ncb1 - 1); };
    auto load_cd = [&](F* cf, F* df, int nb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int kc = min(ks, nkb - 1), t0 = ks * 32 + kofs;
            const F vc = tok8<OP>(dc1 + pkf(nb, kc, nkb, lane), t0, b);   // padding tokens: zero
            const F vd = tok8<OP>(dd1 + pkf(nb, kc, nkb, lane), t0, b);
            cf[ks] = keep_if(vc, ks < nkb);
            df[ks] = keep_if(vd, ks < nkb);
        }
    };
    // W_1's bf16 copy (packed: 8 consecutive inputs of one output per 16
    // bytes) goes out through a tile of the wave in LDS, since a lane holds 4
    // outputs of one input: 16 W1_PN rows (outputs) x 16 inputs per row block
    constexpr int TR = 24;   // tile row pitch (elements): rows stay 16-byte aligned
    bf16* tile = reinterpret_cast<bf16*>(lds) + wave * (16 * W1_PN * TR);
    // p >= 0: the fold's copy into tile rows 16p.., else straight to memory
    auto fold = [&](int jb, int nb, const F* cf, const F* df, const F* hf, f32x4 m, f32x4 sv, bool live, int p) {
        f32x4 um = (f32x4){0.f, 0.f, 0.f, 0.f}, us = um;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            mma(um, cf[ks], hf[ks]);
            mma(us, df[ks], hf[ks]);
        }
        f32x4 mn, sn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sn[e] = mom_s(pe, sv[e], us[e]);
            mn[e] = mom_m(pa, m[e], s0, sv[e], um[e]);
        }
        if (p >= 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[(16 * p + g4 + e) * TR + jl] = (bf16)mn[e];
        }
        if (live) {   // wave-uniform
            st_state(Mw + mso1(jb, nb), mn);
            st_state(S1 + mso1(jb, nb), sn);
            const int n0 = nb * 16 + g4;   // outputs n0 .. n0+3 of input j
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bad |= !__builtin_isfinite(mn[e]) || !__builtin_isfinite(sn[e]);
                if (p < 0) Wt1[pk(n0 + e, jb * 16 + jl, h1 >> 5)] = (bf16)mn[e];
            }
        }
    };
    // every load of the first two row blocks, in consumption order
    F c1f[W1_PN][2], d1f[W1_PN][2];
#pragma unroll
    for (int p = 0; p < W1_PN; ++p) load_cd(c1f[p], d1f[p], nbp(p));
    F hf[W1_JPW][2];
    f32x4 mr[W1_JPW][W1_PN], sr[W1_JPW][W1_PN];
    auto load_q = [&](int slot, int q) {
        const int jb = min(jb0 + 8 * q, a.nb1 - 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) hf[slot][ks] = cvt<OP>(ld8(at1 + pkf(jb, min(ks, nkb - 1), nkb, lane)));
#pragma unroll
        for (int p = 0; p < W1_PN; ++p) {
            mr[slot][p] = *reinterpret_cast<const f32x4*>(Mr + mso1(jb, nbp(p)));
            sr[slot][p] = *reinterpret_cast<const f32x4*>(S1 + mso1(jb, nbp(p)));
        }
    };
#pragma unroll
    for (int q = 0; q < W1_JPW; ++q) load_q(q, q);
#pragma unroll
    for (int q = 0; q < W1_JPW; ++q) {
        const int slot = q, jb = min(jb0 + 8 * q, a.nb1 - 1);
        const bool on = jb0 + 8 * q < a.nb1;
#pragma unroll
        for (int p = 0; p < W1_PN; ++p)
            fold(jb, nbp(p), c1f[p], d1f[p], hf[slot], mr[slot][p], sr[slot][p], on && p < mine1, p);
        // the tile's rows as whole 16-byte pieces (LDS operations of one wave
        // complete in order: no barrier)
        for (int c = lane; c < W1_PN * 32; c += 64) {
            const int row = c >> 1, half = c & 1, p = row >> 4;
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(&tile[row * TR + 8 * half]);
            if (on && p < mine1)
                *reinterpret_cast<bf16x8*>(Wt1 + pk(nbp(p) * 16 + (row & 15), jb * 16 + 8 * half, h1 >> 5)) = v;
        }
        for (int n = W1_PN; n < mine1; ++n) {   // layer 1 wider than 16 * FW * W1_PN outputs
            F cf[2], df[2];
            const int nb = nbp(n);
            load_cd(cf, df, nb);
            const f32x4 m = *reinterpret_cast<const f32x4*>(Mr + mso1(jb, nb));
            const f32x4 sv = *reinterpret_cast<const f32x4*>(S1 + mso1(jb, nb));
            fold(jb, nb, cf, df, hf[slot], m, sv, on, -1);
        }
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(u.flag, 1);
}

// UPD: chunk c-1's update runs (steps 1..C); FWD: chunk c's forward runs (a
// step with rows to push); DEEP: depth >= 2; SPLIT: W_1's update runs in
// workgroups of its own (w1_rows) instead of in the first-layer blocks.  The phases a launch runs are
// compile-time, so every load of a phase is unconditional and issued at the
// top in consumption order: a load whose only use sits behind a run-time
// branch would be moved down to that use, and a branch or loop around a use
// makes the compiler wait for every load in flight.
template <class OP, bool UPD, bool FWD, bool DEEP, bool SPLIT, bool SMALL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(SMALL ? (NW == 4 ? 3 : 4) : 1)))
void first_layer_kernel(FirstArgs a) {
    typedef typename Frag<OP>::T F;
    static_assert(NW == 8 || (NW == 4 && SMALL && !SPLIT), "4-wave workgroups: small dims, no other roles");
    constexpr int PA = FirstDepth<OP, SMALL, NW>::A, PB = FirstDepth<OP, SMALL, NW>::B, PC = FirstDepth<OP, SMALL, NW>::C;
    constexpr int NT = NW * 64;
    constexpr int FR = NW / 2;   // partial tiles kept in LDS
    constexpr bool BWD = UPD && DEEP;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    if ((int)blockIdx.x >= a.nb1) {
        if constexpr (SPLIT) {
            w1_rows<OP>(a, blockIdx.y, (int)blockIdx.x - a.nb1, lds);
            return;
        }
        // the other layers' update tiles of chunk c-1 (only launches that
        // update a memory of depth three or more have them), TPW per
        // workgroup: threads 0..255 and 256..511 each take TPW / 2 tiles with
        // LDS tiles of their own, every tile's loads requested before the
        // first is computed; they touch nothing the first-layer blocks read
        // or write
        if constexpr (UPD && DEEP && NW == 8) {
            const int half = threadIdx.x >> 8, tid = threadIdx.x & 255;
            constexpr int TPW = upd_tpw(sizeof(OP) == 4, SMALL);
            const int t0 = TPW * ((int)blockIdx.x - a.nb1) + half;   // tiles t0, t0 + 2, ...
            float(*UM)[65] = reinterpret_cast<float(*)[65]>(lds) + half * 128;
            TileIn<OP> T[TPW / 2];
#pragma unroll
            for (int q = 0; q < TPW / 2; ++q)
                tile_load<OP>(T[q], a.u, blockIdx.y, a.upd_tile0 + min(t0 + 2 * q, a.upd_ntiles - 1), tid);
#pragma unroll
            for (int q = 0; q < TPW / 2; ++q)
                tile_finish<OP>(T[q], a.u, blockIdx.y, tid, t0 + 2 * q < a.upd_ntiles, UM, UM + 64);
        }
        return;
    }
    const UpdArgs& u = a.u;
    // the workgroup's stream and column block: the grid's own coordinates,
    // or (xcd_streams) remapped so that all blocks of a stream run on one
    // XCD: the dispatcher deals workgroups to the 8 XCDs round-robin by
    // linear id, so XCD x gets the linear ids x, x + 8, ...; they are given
    // streams x, x + 8, ... (all nb1 blocks of each), and the operands every
    // block of a stream reads (the chunk's keys and rows, layer 1's Delta)
    // are fetched into one L2 instead of eight.
    int s = blockIdx.y, bx = blockIdx.x;
    if (a.xcd_streams) {
        const int lin = blockIdx.y * gridDim.x + blockIdx.x, q = lin >> 3;
        s = (q / a.nb1) * 8 + (lin & 7);
        bx = q % a.nb1;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kofs = 8 * (lane >> 4), g4 = 4 * (lane >> 4);
    const int d = a.dim, h1 = a.h1, b = u.b, bp = u.bp;
    const int j0 = bx * JW;
    const int jl = lane & 15, j = j0 + jl;   // the lane's column (h1 is a multiple of 16)
    const int WP = d + WPAD, RP = JW + RPAD;
    constexpr int DP = MAX_CHUNK + WPAD;     // rows hold every token slot of a chunk
    OP* Wn = reinterpret_cast<OP*>(lds);   // [JW][WP]: the block's columns of W_0, K-contiguous
    OP* DcT = Wn + JW * WP;                 // [JW][DP]: (c Delta_0)^T of chunk c-1
    OP* DdT = DcT + JW * DP;
    float* red = reinterpret_cast<float*>(DdT + JW * DP);   // [FR][rows][RP] partial tiles
    float* M0 = u.M + (long)s * u.P;
    float* S0 = u.S + (long)s * u.P;
    bf16* Wt0 = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P;
    bf16* Wt1 = Wt0 + (DEEP ? u.off[1] : 0);
    const OP* kt = reinterpret_cast<const OP*>(a.kt_prev) + (long)s * a.kt_ss;
    const int nrb = d >> 4;
    const int nkb = bp >> 5;
    bool bad = false;

    // ================= every load of the kernel, in consumption order =================
    // (0) the chunk scalars of chunk c-1
    float pa = 0.f, pe = 0.f, s0 = 0.f;
    if constexpr (UPD) {
        const float* csp = u.cs + (long)s * u.cs_ss + (long)a.chunk_prev * 4;
        pa = csp[0];
        pe = csp[1];
        s0 = csp[2];
    }
    // (1) the in-place backward's operands: Delta_1 rows (4 token blocks) and
    //     the lane's column of W_1, K split over the waves
    const int nsA = BWD ? u.dout[1] >> 5 : 1, qA = (nsA + NW - 1) / NW;
    const int kbA = wave * qA, keA = min(nsA, kbA + qA), klA = max(keA - 1, 0);
    const OP* Ad[4];
    const float* Bm = nullptr;
    bool tok[4];
    F ra[PA][4], rb[PA];
    if constexpr (BWD) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            tok[m] = 16 * m + (lane & 15) < b;
            const int mb = 16 * m < b ? m : 0;   // token blocks past the chunk: valid address, dropped
            Ad[m] = reinterpret_cast<const OP*>(a.dlt2) + (long)s * a.dlt2_ss + pkf(mb, 0, nsA, lane);
        }
        // W_1's rows j at chunk c-1's start (not yet updated in this launch)
        // from the fp32 master in accumulator order: outputs n .. n+3 and
        // n+4 .. n+7 of input j are two float4 one 16-lane group apart, and a
        // K step (32 outputs) is two 16-column blocks further on
        Bm = a.m1_rd + (long)s * a.m1_rd_ss + cf1(j, kofs, u.dout[1] >> 4);
#pragma unroll
        for (int p = 0; p < PA; ++p) {
            const long k0 = (long)min(kbA + p, klA) << 9;
#pragma unroll
            for (int m = 0; m < 4; ++m) ra[p][m] = cvt<OP>(ld8(Ad[m] + k0));
            rb[p] = cvt<OP>(ld8w1(Bm + k0));
        }
    }
    // (2) the backward epilogue's SiLU' and coefficients (2 elements per thread)
    constexpr int EA = MAX_CHUNK * JW / NT;
    float sl[EA], cv[EA], dv[EA];
    if constexpr (BWD) {
#pragma unroll
        for (int q = 0; q < EA; ++q) {
            const int idx = tid + NT * q, t = min(idx / JW, b - 1), jj = j0 + idx % JW;
            sl[q] = a.dsl1[(long)s * a.dsl1_ss + (long)t * h1 + jj];
            cv[q] = a.cc_prev[(long)s * a.coef_ss + t];
            dv[q] = a.dc_prev[(long)s * a.coef_ss + t];
        }
    }
    // (3) the update's row blocks of this wave (block wave + NW * p): keys^T
    //     fragments, M and S; blocks past the matrix are clamped and dropped
    const int mineB = (nrb - wave + NW - 1) / NW;
    // (the lane's 4 values of a 16 x 16 block of M or S are one float4 at
    // mso(rbk), the wave's block 1 KB contiguous)
    auto mso = [&](int rbk) { return ((long)(bx * nrb + rbk) * 64 + lane) * 4; };
    F kf[PB][2];
    f32x4 mr[PB], sr[PB];
    auto load_rb = [&](int p, int n) {
        const int rbk = min(wave + NW * n, nrb - 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            kf[p][ks] = keep_if(cvt<OP>(ld8(kt + pkf(rbk, min(ks, nkb - 1), nkb, lane))), ks < nkb);
        }
        mr[p] = *reinterpret_cast<const f32x4*>(M0 + mso(rbk));
        sr[p] = *reinterpret_cast<const f32x4*>(S0 + mso(rbk));
    };
    if constexpr (UPD) {
#pragma unroll
        for (int p = 0; p < PB; ++p) load_rb(p, p);
    }
    // (4) the forward's rows (all 16-row blocks), K = dim split over the
    //     waves; each lane's row: query rows of chunk c-1 first, then key rows
    //     of chunk c, both packed per chunk.  With a backward these loads are
    //     issued right after its products, once its operand registers are
    //     free (issued earlier, the prefetched set would not fit the register
    //     file), and still have the whole update phase to arrive.
    const int R = a.nq + a.nk;
    const int nsC = d >> 5, qC = (nsC + NW - 1) / NW;
    const int kbC = wave * qC, keC = min(nsC, kbC + qC), klC = max(keC - 1, 0);
    const OP* Ax[8];
    bool rok[8];
    F rx[PC][8];
    auto issue_rows = [&]() {
        if constexpr (FWD) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                int r = 16 * m + (lane & 15);
                rok[m] = r < R;
                if (!rok[m]) r = R - 1;
                const bool isq = r < a.nq;
                Ax[m] = reinterpret_cast<const OP*>(isq ? a.xq : a.xk) + (long)s * a.x_ss +
                        pk(isq ? r : r - a.nq, kofs, nsC);
            }
#pragma unroll
            for (int p = 0; p < PC; ++p)
#pragma unroll
                for (int m = 0; m < 8; ++m) rx[p][m] = cvt<OP>(ld8(Ax[m] + ((long)min(kbC + p, klC) << 9)));
        }
    };
    if constexpr (!BWD) issue_rows();

    // (5) chunk c-1's update of rows j0 .. j0+15 of W_1 (depth >= 2), its
    //     operands requested once the forward's registers are free.  It is
    //     computed transposed, U^T = (c Delta_1)^T H_1 (rows: layer 1's
    //     outputs n in 16-blocks nb = wave, wave + NW, ...; columns: the
    //     block's inputs j; K: tokens), so a lane's 4 results are outputs
    //     n .. n+3 of one input j: one float4 of M and S in their accumulator
    //     order.
    constexpr bool W1 = UPD && DEEP && !SPLIT;
    constexpr int PN = FirstDepth<OP, SMALL, NW>::N;   // n-blocks per wave held in registers
    const int d1 = DEEP ? u.dout[1] : 16, ncb1 = d1 >> 4;
    const int mine1 = (ncb1 - wave + NW - 1) / NW;
    F h1f[2], c1f[PN][2], d1f[PN][2];
    f32x4 m1r[PN], s1r[PN];
    const OP* at1 = DEEP ? reinterpret_cast<const OP*>(u.at[1]) + (long)s * u.at_ss[1] : nullptr;
    const OP* dc1 = DEEP ? reinterpret_cast<const OP*>(u.dct[1]) + (long)s * u.dt_ss[1] : nullptr;
    const OP* dd1 = DEEP ? reinterpret_cast<const OP*>(u.ddt[1]) + (long)s * u.dt_ss[1] : nullptr;
    const float* M1r = DEEP ? a.m1_rd + (long)s * a.m1_rd_ss : nullptr;
    float* M1w = DEEP ? a.m1_wr + (long)s * a.m1_wr_ss : nullptr;
    float* S1 = u.S + (long)s * u.P + (DEEP ? u.off[1] : 0);
    auto mso1 = [&](int nb) { return ((long)(bx * ncb1 + nb) * 64 + lane) * 4; };
    auto load_w1 = [&](int p, int n) {
        const int nb = min(wave + NW * n, ncb1 - 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int kc = min(ks, nkb - 1), t0 = ks * 32 + kofs;
            const F vc = tok8<OP>(dc1 + pkf(nb, kc, nkb, lane), t0, b);   // padding tokens: zero
            const F vd = tok8<OP>(dd1 + pkf(nb, kc, nkb, lane), t0, b);
            c1f[p][ks] = keep_if(vc, ks < nkb);
            d1f[p][ks] = keep_if(vd, ks < nkb);
        }
        m1r[p] = *reinterpret_cast<const f32x4*>(M1r + mso1(nb));
        s1r[p] = *reinterpret_cast<const f32x4*>(S1 + mso1(nb));
    };
    auto issue1 = [&]() {
        if constexpr (W1) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) h1f[ks] = cvt<OP>(ld8(at1 + pkf(bx, min(ks, nkb - 1), nkb, lane)));
#pragma unroll
            for (int p = 0; p < PN; ++p) load_w1(p, p);
        }
    };
    // the bf16 copy of the prefetched output blocks leaves through a
    // per-wave LDS tile in the partial-tile area (free once W_1's update
    // runs): a lane holds 4 outputs of one input, the copy stores 8
    // consecutive inputs of one output per 16 bytes
    constexpr int TR1 = 24;   // tile row pitch (elements): rows stay 16-byte aligned
    bf16* t1 = reinterpret_cast<bf16*>(red) + wave * (16 * PN * TR1);
    auto update1 = [&](int p, int n, bool live, bool tiled) {
        const int nb = min(wave + NW * n, ncb1 - 1);
        f32x4 um = (f32x4){0.f, 0.f, 0.f, 0.f}, us = um;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            mma(um, c1f[p][ks], h1f[ks]);
            mma(us, d1f[p][ks], h1f[ks]);
        }
        f32x4 mn, sn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sn[e] = mom_s(pe, s1r[p][e], us[e]);
            mn[e] = mom_m(pa, m1r[p][e], s0, s1r[p][e], um[e]);
        }
        if (live) {   // wave-uniform
            st_state(M1w + mso1(nb), mn);
            st_state(S1 + mso1(nb), sn);
            const int n0 = nb * 16 + g4;   // outputs n0 .. n0+3 of input j
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bad |= !__builtin_isfinite(mn[e]) || !__builtin_isfinite(sn[e]);
                if (tiled) t1[(16 * p + g4 + e) * TR1 + jl] = (bf16)mn[e];
                else Wt1[pk(n0 + e, j, h1 >> 5)] = (bf16)mn[e];
            }
        }
    };
    auto run1 = [&]() {
        if constexpr (W1) {
#pragma unroll
            for (int p = 0; p < PN; ++p) update1(p, p, p < mine1, true);
            // the tile's rows as whole 16-byte pieces (the LDS operations of
            // one wave complete in order: no barrier)
            for (int c = lane; c < PN * 32; c += 64) {
                const int row = c >> 1, half = c & 1, p = row >> 4;
                if (p < mine1) {
                    const int nb = min(wave + NW * p, ncb1 - 1);
                    const bf16x8 v = *reinterpret_cast<const bf16x8*>(&t1[row * TR1 + 8 * half]);
                    *reinterpret_cast<bf16x8*>(Wt1 + pk(nb * 16 + (row & 15), j0 + 8 * half, h1 >> 5)) = v;
                }
            }
            if constexpr (!SMALL)   // (SMALL: every output block prefetched)
            for (int n = PN; n < mine1; ++n) {
                load_w1(0, n);
                update1(0, n, true, false);
            }
        }
    };

    // ================= chunk c-1's update of the block's columns =================
    if constexpr (UPD) {
        if constexpr (BWD) {
            // Delta_0 = (Delta_1 W_1^T) * SiLU'(z_0): 64 tokens x JW columns.
            // The prefetched K steps straight-line, then (long K only) the
            // rest, each loaded and used
            f32x4 acc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < PA; ++p) {
                const F bv = keep_if(rb[p], kbA + p < keA);
#pragma unroll
                for (int m = 0; m < 4; ++m) mma(acc[m], tok[m] ? ra[p][m] : zero_frag<OP>(), bv);
            }
            if constexpr (!SMALL)   // (SMALL: one K step per wave)
            for (int k = kbA + PA; k < keA; ++k) {
                const long kn = (long)k << 9;
                F av[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) av[m] = cvt<OP>(ld8(Ad[m] + kn));
                const F bv = cvt<OP>(ld8w1(Bm + kn));
#pragma unroll
                for (int m = 0; m < 4; ++m) mma(acc[m], tok[m] ? av[m] : zero_frag<OP>(), bv);
            }
            issue_rows();
            partial_tiles<4, FR>(red, acc, 4, 64, wave, lane, RP);
            // theta-weighted, into LDS (token slots past the chunk get zeros)
#pragma unroll
            for (int q = 0; q < EA; ++q) {
                const int idx = tid + NT * q, t = idx / JW, cl = idx % JW;
                float z = 0.f;
#pragma unroll
                for (int w = 0; w < FR; ++w) z += red[(w * 64 + t) * RP + cl];
                const float dl = t < b ? z * sl[q] : 0.f;
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
                for (int e = 0; e < 8; ++e) {
                    vc[e] = t8 + e < b ? vc[e] : (OP)0.0f;
                    vd[e] = t8 + e < b ? vd[e] : (OP)0.0f;
                }
                *reinterpret_cast<F*>(&DcT[cl * DP + t8]) = vc;
                *reinterpret_cast<F*>(&DdT[cl * DP + t8]) = vd;
            }
        }
        __syncthreads();

        // U = K^T diag(c) Delta_0 and the momentum / forgetting write, 16-row
        // blocks (block w, w+NW, ... for wave w)
        F bc[2], bd[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bool on = ks < nkb;
            bc[ks] = on ? *reinterpret_cast<const F*>(&DcT[jl * DP + ks * 32 + kofs]) : zero_frag<OP>();
            bd[ks] = on ? *reinterpret_cast<const F*>(&DdT[jl * DP + ks * 32 + kofs]) : zero_frag<OP>();
        }
        auto update_rb = [&](int p, int n, bool live) {
            const int rbk = min(wave + NW * n, nrb - 1), ib = 16 * rbk;
            f32x4 um = (f32x4){0.f, 0.f, 0.f, 0.f}, us = um;
            mma(um, kf[p][0], bc[0]);
            mma(us, kf[p][0], bd[0]);
            mma(um, kf[p][1], bc[1]);
            mma(us, kf[p][1], bd[1]);
            f32x4 mn, sn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sn[e] = mom_s(pe, sr[p][e], us[e]);
                mn[e] = mom_m(pa, mr[p][e], s0, sr[p][e], um[e]);
            }
            if (live) {   // wave-uniform
                st_state(M0 + mso(rbk), mn);
                st_state(S0 + mso(rbk), sn);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bad |= !__builtin_isfinite(mn[e]) || !__builtin_isfinite(sn[e]);
                    Wn[jl * WP + ib + g4 + e] = (OP)mn[e];
                }
                // W_0's bf16 copy is read only by the next call's first step
                // and by retrieval (the forward here uses the columns in
                // LDS): written on the call's last update only.  4
                // consecutive inputs of output j: 8 contiguous bytes.
                if (a.last_update) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    *reinterpret_cast<bf16x4*>(Wt0 + pk(j, ib + g4, d >> 5)) =
                        (bf16x4){(bf16)mn[0], (bf16)mn[1], (bf16)mn[2], (bf16)mn[3]};
                }
            }
        };
        // the prefetched row blocks, then (dim above 16 * NW * PB only) the
        // rest, each loaded and used
#pragma unroll
        for (int p = 0; p < PB; ++p) update_rb(p, p, p < mineB);
        if constexpr (!SMALL)   // (SMALL: one row block per wave)
        for (int n = PB; n < mineB; ++n) {
            load_rb(0, n);
            update_rb(0, n, true);
        }

    } else if constexpr (FWD) {
        // first chunk of the call: the block's columns of the current W_0
        if constexpr (sizeof(OP) == 2) {
            for (int idx = tid; idx < JW * (d >> 3); idx += NT) {
                const int cl = idx % JW, i = (idx / JW) * 8;
                *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(Wn) + cl * WP + i) =
                    *reinterpret_cast<const bf16x8*>(Wt0 + pk(j0 + cl, i, d >> 5));
            }
        } else {
            for (int idx = tid; idx < JW * d; idx += NT) {
                const int i = idx / JW, cl = idx - i * JW;
                Wn[cl * WP + i] = (OP)M0[cf0(i, j0 + cl, nrb)];
            }
        }
    }
    if constexpr (!FWD) {
        issue1();
        run1();
        if (__ballot(bad) != 0 && lane == 0) atomicOr(u.flag, 1);
        return;
    }
    __syncthreads();

    // ================= chunk c's first-layer forward =================
    {
        f32x4 acc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
        // prefetched steps straight-line, then (long K only) load and use;
        // row blocks past the rows multiply zeros
#pragma unroll
        for (int p = 0; p < PC; ++p) {
            const int k0 = min(kbC + p, klC) << 5;
            F bv = *reinterpret_cast<const F*>(&Wn[jl * WP + k0 + kofs]);
            if (kbC + p >= keC) bv = zero_frag<OP>();
#pragma unroll
            for (int m = 0; m < 8; ++m) mma(acc[m], rok[m] ? rx[p][m] : zero_frag<OP>(), bv);
        }
        if constexpr (!SMALL)   // (SMALL: one K step per wave)
        for (int k = kbC + PC; k < keC; ++k) {
            F xv[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) xv[m] = cvt<OP>(ld8(Ax[m] + ((long)k << 9)));
            const F bv = *reinterpret_cast<const F*>(&Wn[jl * WP + (k << 5) + kofs]);
#pragma unroll
            for (int m = 0; m < 8; ++m) mma(acc[m], rok[m] ? xv[m] : zero_frag<OP>(), bv);
        }
        issue1();   // layer 1's rows: operands now, the update after the epilogue
        partial_tiles<8, FR>(red, acc, 8, 128, wave, lane, RP);
    }
    if constexpr (DEEP) {
        // z of every (row, column), summed from the partial tiles (slot
        // order), 4 columns of one row per thread: the activations (packed
        // [rows][h1]), SiLU'(z) of the key rows, and the key rows'
        // activations transposed into LDS (the (c Delta_0)^T area, free since
        // the update) for their packed [h1][bp] copy
        typedef OP OP4 __attribute__((ext_vector_type(4)));
        OP* hT = DcT;   // [JW][DP]
        for (int idx = tid; idx < R * (JW / 4); idx += NT) {
            const int r = idx / (JW / 4), c4 = (idx % (JW / 4)) * 4, jj = j0 + c4;
            OP4 hv;
            f32x4 sd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float z = 0.f;
#pragma unroll
                for (int w = 0; w < FR; ++w) z += red[(w * 128 + r) * RP + c4 + e];
                const float sg = sigmoid(z);
                hv[e] = (OP)(z * sg);
                sd[e] = sg * (1.0f + z * (1.0f - sg));
            }
            *reinterpret_cast<OP4*>(reinterpret_cast<OP*>(a.act) + (long)s * a.act_ss + pk(r, jj, h1 >> 5)) = hv;
            if (r >= a.nq) {
                *reinterpret_cast<f32x4*>(a.dsl1 + (long)s * a.dsl1_ss + (long)(r - a.nq) * h1 + jj) = sd;
#pragma unroll
                for (int e = 0; e < 4; ++e) hT[(c4 + e) * DP + r - a.nq] = hv[e];
            }
        }
        if (a.nk > 0) {   // uniform
            __syncthreads();
            for (int idx = tid; idx < JW * (bp >> 3); idx += NT) {
                const int cl = idx % JW, t8 = (idx / JW) * 8;
                F hv = *reinterpret_cast<const F*>(&hT[cl * DP + t8]);
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = t8 + e < a.nk ? hv[e] : (OP)0.0f;   // zero past the chunk
                st8<OP>(reinterpret_cast<OP*>(a.ht1) + (long)s * a.ht_ss + pk(j0 + cl, t8, nkb), hv);
            }
        }
    } else {
        // depth 1: the first layer is the output layer.  z of every (row,
        // column): the partial tiles summed into slot 0
        for (int idx = tid; idx < R * JW; idx += NT) {
            const int r = idx / JW, cl = idx - r * JW;
            float z = 0.f;
#pragma unroll
            for (int w = 0; w < FR; ++w) z += red[(w * 128 + r) * RP + cl];
            red[r * RP + cl] = z;
        }
        __syncthreads();
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
    if (a.nk == 0) __syncthreads();   // (uniform) the epilogue's reads of the partial tiles are done
    run1();
    if (__ballot(bad) != 0 && lane == 0) atomicOr(u.flag, 1);
}

static bool first_nw4_on() {
    static const int v = getenv("TM_FIRST4") ? atoi(getenv("TM_FIRST4")) : 1;
    return v != 0;
}

// The half-occupancy variant: bf16 with layer-0 and layer-1 widths within
// SMALL_DIM (the fp32 operand set does not fit half the register file).
static bool first_small(const FirstArgs& a, bool f32) {
    return !f32 && a.dim <= SMALL_DIM && (a.u.L < 2 || a.u.dout[1] <= SMALL_DIM);
}

// The small-dim variant with 4-wave workgroups: launches without workgroups
// of other roles (no W_1 workgroups, no update tiles).
static bool first_small4(const FirstArgs& a, bool f32) {
    return first_small(a, f32) && a.nw1 == 0 && a.upd_ntiles == 0 && first_nw4_on();
}

template <class OP, bool UPD, bool FWD>
static void launch_first_as(const FirstArgs& a, dim3 grid, size_t lds, hipStream_t st) {
    // (W_1's workgroups of their own: bf16 only; with fp32 operands that
    // variant's register set would spill)
    if constexpr (UPD && sizeof(OP) == 2) {
        if (a.nw1 > 0) {
            launch_k((first_layer_kernel<OP, true, FWD, true, true, false, 8>), grid, dim3(FW * 64), lds, st, a);
            return;
        }
    }
    const bool small = first_small(a, sizeof(OP) == 4);
    if constexpr (sizeof(OP) == 2) {
        if (small && first_small4(a, false)) {
            if (a.u.L >= 2)
                launch_k((first_layer_kernel<OP, UPD, FWD, true, false, true, 4>), grid, dim3(4 * 64), lds, st, a);
            else
                launch_k((first_layer_kernel<OP, UPD, FWD, false, false, true, 4>), grid, dim3(4 * 64), lds, st, a);
            return;
        }
        if (small) {
            if (a.u.L >= 2)
                launch_k((first_layer_kernel<OP, UPD, FWD, true, false, true, 8>), grid, dim3(FW * 64), lds, st, a);
            else
                launch_k((first_layer_kernel<OP, UPD, FWD, false, false, true, 8>), grid, dim3(FW * 64), lds, st, a);
            return;
        }
    }
    if (a.u.L >= 2)
        launch_k((first_layer_kernel<OP, UPD, FWD, true, false, false, 8>), grid, dim3(FW * 64), lds, st, a);
    else
        launch_k((first_layer_kernel<OP, UPD, FWD, false, false, false, 8>), grid, dim3(FW * 64), lds, st, a);
}

template <class OP>
static void launch_first_op(const FirstArgs& a, dim3 grid, size_t lds, hipStream_t st) {
    if (a.do_update && a.do_fwd) launch_first_as<OP, true, true>(a, grid, lds, st);
    else if (a.do_update) launch_first_as<OP, true, false>(a, grid, lds, st);
    else launch_first_as<OP, false, true>(a, grid, lds, st);
}

hipError_t launch_first(const FirstArgs& a, int ns, int f32, hipStream_t st) {
    if (!a.do_update && !a.do_fwd) return hipSuccess;
    if (a.nw1 > 0 && (f32 || !a.do_update || a.u.L != 2 || a.upd_ntiles != 0 || a.nw1 % 8 != 0 ||
                      (long)(a.nw1 / 8) * W1_JPW < (a.nb1 + 7) / 8 || a.m1_rd == a.m1_wr))
        return hipErrorInvalidValue;
    if (a.upd_ntiles > 0 && (!a.do_update || a.u.L < 3)) return hipErrorInvalidValue;
    if (a.xcd_streams && (a.nw1 > 0 || a.upd_ntiles > 0 || ns % 8 != 0)) return hipErrorInvalidValue;
    const int tpw = upd_tpw(f32, first_small(a, f32));
    const int nupd = (a.upd_ntiles + tpw - 1) / tpw;   // workgroups of update tiles
    dim3 grid(a.nb1 + (a.nw1 > 0 ? a.nw1 : nupd), ns);
    size_t lds = first_lds_bytes(a.dim, a.u.bp, f32, first_small4(a, f32) ? 4 : 8);
    if (nupd > 0 && lds < UPD_TILE_LDS) lds = UPD_TILE_LDS;
    if (a.nw1 > 0 && lds < W1_LDS) lds = W1_LDS;
    if (f32) launch_first_op<float>(a, grid, lds, st);
    else launch_first_op<bf16>(a, grid, lds, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// State set-up, bf16 copy, export / import.

// Position in the state of canonical element p (row-major layers) of one
// stream: layer 0 (d0 x h1) and layer 1 (h1 x d1, d1 = 0 for depth 1) in
// accumulator order, the other layers row-major.
__device__ __forceinline__ long state_pos(long p, int d0, int h1, int d1) {
    const long p0 = (long)d0 * h1;
    if (p < p0) {
        const int i = (int)(p / h1), j = (int)(p - (long)i * h1);
        return cf0(i, j, d0 >> 4);
    }
    if (p < p0 + (long)h1 * d1) {
        const long q = p - p0;
        const int j = (int)(q / d1), n = (int)(q - (long)j * d1);
        return p0 + cf1(j, n, d1 >> 4);
    }
    return p;
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
        const long o = l == 0 ? cf0(i0 + i, j0 + j, din >> 4)
                     : l == 1 ? cf1(i0 + i, j0 + j, dout >> 4) : (long)(i0 + i) * dout + j0 + j;
        T[i][j] = (i0 + i < din && j0 + j < dout) ? Mp[o] : 0.f;
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

// A fresh state in one pass: per 64 x 64 tile of one layer of one stream,
// the canonical init weights (head s % H) are read once through LDS and
// written to M in the layer's layout, to S as zeros and to the packed bf16
// copy; block (0, 0) also writes the header.
__global__ __launch_bounds__(256) void state_init_kernel(UpdArgs u, const float* init, int H, StateHeader* h,
                                                         uint64_t hash, int batch, int heads) {
    __shared__ float T[64][65];
    const int tid = threadIdx.x;
    const int s = blockIdx.y;
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
        h->magic = STATE_MAGIC;
        h->version = STATE_VERSION;
        h->cfg_hash = hash;
        h->batch = batch;
        h->heads = heads;
        h->nonfinite = 0;
        h->reserved0 = 0;
        h->position = 0;
    }
    int tile = blockIdx.x;
    int l = 0;
#pragma unroll
    for (int q = 1; q < MAXL; ++q)
        if (q < u.L && tile >= u.tbase[q]) l = q;
    int tb = 0, tjn = 1, din = 32, dout = 32;
    long off = 0;
#pragma unroll
    for (int q = 0; q < MAXL; ++q)
        if (q == l) {
            tb = u.tbase[q];
            tjn = u.tj[q];
            din = u.din[q];
            dout = u.dout[q];
            off = u.off[q];
        }
    tile -= tb;
    const int ti = tile / tjn, tj = tile - ti * tjn;
    const int i0 = ti * 64, j0 = tj * 64;
    const float* src = init + (long)(s % H) * u.P + off;
    f32x4 g[4];   // the tile's rows as float4 (dims are multiples of 32)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q, i = idx >> 4, j = (idx & 15) * 4;
        const bool in = i0 + i < din && j0 + j < dout;
        g[q] = *reinterpret_cast<const f32x4*>(src + (in ? (long)(i0 + i) * dout + j0 + j : 0));
        if (!in) g[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q, i = idx >> 4, j = (idx & 15) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) T[i][j + e] = g[q][e];
    }
    __syncthreads();
    float* Mp = u.M + (long)s * u.P + off;
    float* Sp = u.S + (long)s * u.P + off;
    // 1024 float4 of the tile, each at 4 consecutive positions of the
    // layer's layout: 4 rows of one column (layer 0), 4 outputs of one input
    // (layer 1, and the row-major layers)
    for (int k = tid; k < 1024; k += 256) {
        int i, j;
        f32x4 v;
        long o;
        if (l == 0) {
            j = k & 63;
            i = (k >> 6) * 4;
            v = (f32x4){T[i][j], T[i + 1][j], T[i + 2][j], T[i + 3][j]};
            o = cf0(i0 + i, j0 + j, din >> 4);
        } else {
            i = k & 63;
            j = (k >> 6) * 4;
            v = (f32x4){T[i][j], T[i][j + 1], T[i][j + 2], T[i][j + 3]};
            o = l == 1 ? cf1(i0 + i, j0 + j, dout >> 4) : (long)(i0 + i) * dout + j0 + j;
        }
        if (i0 + i < din && j0 + j < dout) {
            *reinterpret_cast<f32x4*>(Mp + o) = v;
            *reinterpret_cast<f32x4*>(Sp + o) = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
    }
    bf16* Wp = reinterpret_cast<bf16*>(u.Wt) + (long)s * u.P + off;
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

hipError_t launch_state_init(const UpdArgs& u, int ntiles, int ns, const float* init, int H, StateHeader* h,
                             uint64_t hash, int batch, int heads, hipStream_t st) {
    launch_k(state_init_kernel, dim3(ntiles, ns), dim3(256), 0, st, u, init, H, h, hash, batch, heads);
    return hipGetLastError();
}

hipError_t launch_shadow(const UpdArgs& u, int ntiles, int ns, hipStream_t st) {
    launch_k(shadow_kernel, dim3(ntiles, ns), dim3(256), 0, st, u);
    return hipGetLastError();
}

__global__ void export_kernel(const float* M, const float* S, float* dst, long P, int ns, int d0, int h1,
                              int d1) {
    const long n = (long)ns * P;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long s = i / P, p = i - s * P, q = s * P + state_pos(p, d0, h1, d1);
        dst[s * 2 * P + p] = M[q];
        dst[s * 2 * P + P + p] = S[q];
    }
}

__global__ void import_kernel(float* M, float* S, const float* src, long P, int ns, int d0, int h1,
                              int d1) {
    const long n = (long)ns * P;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long s = i / P, p = i - s * P, q = s * P + state_pos(p, d0, h1, d1);
        M[q] = src[s * 2 * P + p];
        S[q] = src[s * 2 * P + P + p];
    }
}

hipError_t launch_export(const float* M, const float* S, float* dst, long P, int ns, int d0, int h1, int d1,
                         hipStream_t st) {
    launch_k(export_kernel, dim3(2048), dim3(256), 0, st, M, S, dst, P, ns, d0, h1, d1);
    return hipGetLastError();
}

hipError_t launch_import(float* M, float* S, const float* src, long P, int ns, int d0, int h1, int d1,
                         hipStream_t st) {
    launch_k(import_kernel, dim3(2048), dim3(256), 0, st, M, S, src, P, ns, d0, h1, d1);
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
    launch_k(header_kernel, dim3(1), dim3(64), 0, st, h, hash, batch, heads);
    return hipGetLastError();
}

}  // namespace tmk
