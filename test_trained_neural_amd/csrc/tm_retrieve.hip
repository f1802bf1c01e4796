// Read-only retrieval's products on CDNA4 (gfx950): y = M(q) for up to 2048
// query rows per stream and pass, layer by layer through the bf16 copy of
// the weights ("Titans, explained", step 5: a forward pass with no write).
//
// With that many rows a layer is a plain tiled product: a workgroup of 4
// waves owns 64 rows x 16 NR columns, each wave 16 rows over the whole K
// range (no split over waves, so no partial tiles to sum), its operands
// streamed through a register ring of PF steps (steps past K re-load a valid
// address and are masked).  The epilogue applies SiLU and stores the next
// layer's packed activations (through a per-wave LDS tile, so the stores
// are 16-byte pieces of 8 consecutive columns), or writes y.  The chunk
// step's products (a few dozen rows per stream) use the split-K kernel in
// tm_kernels.hip instead.  A memory of depth 2 and width up to 128 takes
// mlp2_kernel below instead: both layers in one launch, no activations in
// memory.
#include "tm_device.h"

namespace tmk {

constexpr int RB_WAVES = 4;   // waves of a workgroup: 16 rows each

// TOK: A is the query token array (layer 0), else packed rows.
template <int NR, bool LAST, bool TOK>
__global__ __launch_bounds__(RB_WAVES * 64) void rows_kernel(GemmArgs g) {
    constexpr int PF = 4;
    constexpr int NC = NR * 16;
    __shared__ float tile[RB_WAVES][16][NC + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the stream and tile: the grid's coordinates, or (xcd_streams) remapped
    // so that all tiles of a stream run on one XCD (workgroups go to the 8
    // XCDs round-robin by linear id): a row block's operand rows and the
    // stream's weights are then fetched into one L2, not several
    int s = blockIdx.z, by = blockIdx.y, bx = blockIdx.x;
    if (g.xcd_streams) {
        const int per = gridDim.x * gridDim.y;
        const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x, q = lin >> 3;
        s = (q / per) * 8 + (lin & 7);
        by = (q % per) / gridDim.x;
        bx = (q % per) % gridDim.x;
    }
    const int r0 = by * (RB_WAVES * 16) + wave * 16;   // the wave's first row
    const int c0 = bx * NC;
    const int nsteps = g.K >> 5;
    const int kofs = 8 * (lane >> 4);

    // A: this lane's row (clamped into the rows: rows past them are dropped)
    const bf16* arow;
    long astep;
    if constexpr (TOK) {
        const int ra = min(r0 + (lane & 15), g.nrows - 1);
        arow = reinterpret_cast<const bf16*>(g.a0) + tok_off(g.tl, s, g.at0 + ra) + kofs;
        astep = 32;
    } else {
        const int rb = min(r0, g.nrows - 1) >> 4;
        arow = reinterpret_cast<const bf16*>(g.a0) + (long)s * g.a_ss + pkf(rb, 0, nsteps, lane);
        astep = 512;
    }
    const bf16* bcol[NR];
#pragma unroll
    for (int n = 0; n < NR; ++n)
        bcol[n] = reinterpret_cast<const bf16*>(g.b) + (long)s * g.b_ss + pkf((c0 >> 4) + n, 0, nsteps, lane);

    bf16x8 a[PF], bb[PF][NR];
    auto load = [&](int p, int k) {
        a[p] = ld8(arow + k * astep);
#pragma unroll
        for (int n = 0; n < NR; ++n) bb[p][n] = ld8(bcol[n] + (long)k * 512);
    };
    f32x4 acc[NR];
#pragma unroll
    for (int n = 0; n < NR; ++n) acc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, min(p, nsteps - 1));
    for (int k = 0; k < nsteps; k += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const bf16x8 av = keep_if(a[p], k + p < nsteps);
#pragma unroll
            for (int n = 0; n < NR; ++n) mma(acc[n], av, bb[p][n]);
            load(p, min(k + p + PF, nsteps - 1));
        }
    }

    if constexpr (LAST) {
        // y of the query rows (16 lanes write 16 consecutive outputs of a row)
#pragma unroll
        for (int n = 0; n < NR; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + 4 * (lane >> 4) + e;
                if (r < g.nrows) g.y[tok_off(g.tl, s, g.yt0 + r) + c0 + n * 16 + (lane & 15)] = acc[n][e];
            }
    } else {
        // SiLU, then the packed activations of the next layer, 8 consecutive
        // columns of one row per 16-byte store
#pragma unroll
        for (int n = 0; n < NR; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float z = acc[n][e];
                tile[wave][4 * (lane >> 4) + e][n * 16 + (lane & 15)] = z * sigmoid(z);
            }
        __syncthreads();
        bf16* act = reinterpret_cast<bf16*>(g.act) + (long)s * g.act_ss;
#pragma unroll
        for (int q = 0; q < NR / 2; ++q) {
            const int piece = lane + 64 * q, row = piece / (NC / 8), c8 = (piece % (NC / 8)) * 8;
            if (r0 + row < g.nrows) {
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (bf16)tile[wave][row][c8 + e];
                *reinterpret_cast<bf16x8*>(act + pk(r0 + row, c0 + c8, g.N >> 5)) = o;
            }
        }
    }
}

template <int NR, bool LAST>
static void launch_rows_as(const GemmArgs& g, int ns, hipStream_t st) {
    const dim3 grid(g.N / (NR * 16), (g.nrows + RB_WAVES * 16 - 1) / (RB_WAVES * 16), ns);
    if (g.amode == A_TOKENS) launch_k((rows_kernel<NR, LAST, true>), grid, dim3(RB_WAVES * 64), 0, st, g);
    else launch_k((rows_kernel<NR, LAST, false>), grid, dim3(RB_WAVES * 64), 0, st, g);
}

hipError_t launch_rows(const GemmArgs& g, int ns, hipStream_t st) {
    // bf16 operands: A as query tokens (no key rows) or packed rows, B the
    // packed bf16 copy; N a multiple of 32, K of 32
    if (g.nrows <= 0) return hipSuccess;
    if (g.bmode != B_PACKED || (g.amode != A_TOKENS && g.amode != A_PACKED) || g.n0 != g.nrows ||
        g.N % 32 != 0 || g.K % 32 != 0 || g.K <= 0 || ns < 1 || ns > 65535 || (g.xcd_streams && ns % 8 != 0))
        return hipErrorInvalidValue;
    const bool last = g.epi == EPI_OUT;
    if (!last && g.epi != EPI_HIDDEN) return hipErrorInvalidValue;
    if (g.N % 64 == 0) {
        if (last) launch_rows_as<4, true>(g, ns, st);
        else launch_rows_as<4, false>(g, ns, st);
    } else {
        if (last) launch_rows_as<2, true>(g, ns, st);
        else launch_rows_as<2, false>(g, ns, st);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Read-only retrieval of a depth-2 memory of width d <= 128 in one launch:
// y = SiLU(q W_0) W_1 with the hidden activations kept in registers.
//
// Both layers run transposed, H^T = W_0^T q^T and y^T = W_1^T H^T.  A lane's
// share of a layer-0 result tile is 4 rows of one token, and a layer-1 B
// fragment wants 8 consecutive hidden units of one token (lane group g of
// the 32-deep step: units 8g .. 8g+7).  So the two layer-0 tiles of a step
// take the step's hidden units in the order 8(i/4) + 4hb + i%4 for row i of
// tile hb: lane group g then holds units 8g .. 8g+3 in tile 0 and 8g+4 ..
// 8g+7 in tile 1, exactly its B fragment.  Only the rows of W_0's fragments
// are gathered in that order when the chunk is loaded; W_1's fragments are
// copied as they are stored, and nothing moves between the layers.
//
// A workgroup owns WAVES x TB 16-token blocks of one stream; a wave keeps its
// TB blocks of queries as B fragments (all d/32 steps) and TB x d/16
// accumulator tiles of y.  The weights stream through LDS in 64-hidden
// chunks, double buffered: chunk c+1's loads are in flight while chunk c
// computes, and each fragment read from LDS serves TB matrix instructions.
template <int D, int TB, int WAVES, int HC>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mlp2_kernel(Mlp2Args a) {
    constexpr int KS = D / 32, NB = D / 16, NT = WAVES * 64, SPC = HC / 32;
    constexpr int W0P = (HC / 16) * KS * 64;   // 16-byte pieces of a chunk's W_0 fragments
    constexpr int W1P = NB * SPC * 64;         // ... and of its W_1 fragments
    constexpr int CP = W0P + W1P;
    constexpr int RND = (CP + NT - 1) / NT;
    extern __shared__ __attribute__((aligned(16))) char lds[];   // 2 chunks of CP pieces
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, col = lane & 15;
    // the stream and row block: the grid's coordinates, or (xcd_streams) all
    // row blocks of a stream on one XCD, so its weights are fetched into one L2
    int s = blockIdx.y, bx = blockIdx.x;
    if (a.xcd_streams) {
        const int lin = blockIdx.y * gridDim.x + blockIdx.x, q8 = lin >> 3;
        s = (q8 / gridDim.x) * 8 + (lin & 7);
        bx = q8 % gridDim.x;
    }
    const bf16* w0 = reinterpret_cast<const bf16*>(a.w) + (long)s * a.w_ss;
    const bf16* w1 = w0 + a.off1;
    const int nks1 = a.h >> 5, nch = a.h / HC;
    const int r0 = (bx * WAVES + wave) * (TB * 16);   // the wave's first row

    // the wave's queries: B fragments of layer 0 (rows past the call are
    // clamped to a valid row and their results dropped)
    bf16x8 qf[TB][KS];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = min(r0 + 16 * tb + col, a.nrows - 1);
        const bf16* qp = reinterpret_cast<const bf16*>(a.q) + tok_off(a.tl, s, a.t0 + t) + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[tb][ks] = ld8(qp + 32 * ks);
    }

    // chunk c of the weights: W_0's fragments of the chunk's hidden units
    // (rows gathered in the order above), then W_1's fragments of the
    // chunk's K steps for every output block, as stored
    bf16x8 stg[RND];
    auto fetch = [&](int c) {
#pragma unroll
        for (int p = 0; p < RND; ++p) {
            const int o = p * NT + tid;
            if (o < W0P) {
                // A-fragment row i of the step's hidden block hb is hidden
                // unit 8(i/4) + 4hb + i%4 of the step: 8 consecutive inputs
                // of one hidden unit, contiguous in the packed copy
                const int f0 = o >> 6, L = o & 63, hbl = f0 / KS, ks = f0 % KS, i = L & 15;
                const int j = c * HC + 32 * (hbl >> 1) + 8 * (i >> 2) + 4 * (hbl & 1) + (i & 3);
                stg[p] = ld8(w0 + pk(j, 32 * ks + 8 * (L >> 4), KS));
            } else if (o < CP) {
                const int o1 = o - W0P, f = o1 >> 6;
                stg[p] = ld8(w1 + pkf(f / SPC, SPC * c + f % SPC, nks1, o1 & 63));
            }
        }
    };
    auto put = [&](char* buf) {
#pragma unroll
        for (int p = 0; p < RND; ++p) {
            const int o = p * NT + tid;
            if (o < CP) *reinterpret_cast<bf16x8*>(buf + o * 16) = stg[p];
        }
    };

    f32x4 yacc[NB][TB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) yacc[nb][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // A 32-hidden step: layer 0's fragments are read from LDS before its
    // products (all at once, so one LDS round trip per step), then step st-1's
    // layer-1 products (independent of this step's results), then this
    // step's SiLU, in stages across its 8 TB values per lane so that the
    // exponentials and reciprocals of different values overlap.
    auto layer0 = [&](const char* cur, int st, f32x4 (&hacc)[2][TB]) {
        bf16x8 w[2][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
                w[hb][ks] = *reinterpret_cast<const bf16x8*>(cur + (((2 * st + hb) * KS + ks) * 64 + lane) * 16);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) hacc[hb][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) mma(hacc[hb][tb], w[hb][ks], qf[tb][ks]);
    };
    auto silu = [&](const f32x4 (&hacc)[2][TB], bf16x8 (&hf)[TB]) {
        constexpr int NV = 8 * TB;
        float z[NV], e[NV];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[8 * tb + i] = hacc[0][tb][i];
                z[8 * tb + 4 + i] = hacc[1][tb][i];
            }
#pragma unroll
        for (int v = 0; v < NV; ++v) e[v] = __expf(-z[v]);
#pragma unroll
        for (int v = 0; v < NV; ++v) e[v] = __builtin_amdgcn_rcpf(1.0f + e[v]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 8; ++i) hf[tb][i] = (bf16)(z[8 * tb + i] * e[8 * tb + i]);
    };
    auto layer1 = [&](const char* l1, int st, const bf16x8 (&hf)[TB]) {
        bf16x8 w[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            w[nb] = *reinterpret_cast<const bf16x8*>(l1 + ((nb * SPC + st) * 64 + lane) * 16);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) mma(yacc[nb][tb], w[nb], hf[tb]);
    };
    fetch(0);
    put(lds);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const char* cur = lds + (c & 1) * (CP * 16);
        if (c + 1 < nch) fetch(c + 1);
        const char* l1 = cur + W0P * 16;
        // step st's layer-0 products go out before step st-1's layer-1
        // products, so the SiLU between the layers of a step waits behind
        // independent matrix work
        bf16x8 hf[2][TB];
#pragma unroll
        for (int st = 0; st < SPC; ++st) {
            f32x4 hacc[2][TB];
            layer0(cur, st, hacc);
            if (st > 0) layer1(l1, st - 1, hf[(st - 1) & 1]);
            silu(hacc, hf[st & 1]);
        }
        layer1(l1, SPC - 1, hf[(SPC - 1) & 1]);
        if (c + 1 < nch) put(lds + ((c + 1) & 1) * (CP * 16));
        __syncthreads();
    }
    // y: a lane holds outputs 16nb + 4g .. +3 of token r0 + 16tb + col
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = r0 + 16 * tb + col;
        if (t < a.nrows) {
            float* yp = a.y + tok_off(a.tl, s, a.t0 + t) + 4 * g;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4*>(yp + 16 * nb) = yacc[nb][tb];
        }
    }
}

bool mlp2_fits(int d, int h) { return d >= 32 && d <= 128 && d % 32 == 0 && h >= 64 && h % 64 == 0; }

template <int D, int TB, int WAVES, int HC>
static void launch_mlp2_as(const Mlp2Args& a, int ns, hipStream_t st) {
    constexpr int CP = (HC / 16) * (D / 32) * 64 + (D / 16) * (HC / 32) * 64;
    const dim3 grid((a.nrows + WAVES * TB * 16 - 1) / (WAVES * TB * 16), ns);
    launch_k((mlp2_kernel<D, TB, WAVES, HC>), grid, dim3(WAVES * 64), 2 * CP * 16, st, a);
}

// 4 waves of 2 token blocks (128 rows) per workgroup, 64-hidden chunks,
// layer 1 of a step behind layer 0 of the next: 2 workgroups per compute unit
// (232 registers a lane, 64 KB of LDS).  Measured on 64 streams of
// 128 -> 512 -> 128 over 32768 rows: 767 us; without the step pipelining
// 778 us; 8 waves with 128-hidden chunks 809 us; 4 token blocks a wave (one
// wave a SIMD) 1171 us.
template <int D>
static void launch_mlp2_d(const Mlp2Args& a, int ns, hipStream_t st) {
    launch_mlp2_as<D, 2, 4, 64>(a, ns, st);
}

hipError_t launch_mlp2(const Mlp2Args& a, int ns, hipStream_t st) {
    if (a.nrows <= 0) return hipSuccess;
    if (!mlp2_fits(a.d, a.h) || a.tl.d != a.d || ns < 1 || ns > 65535 || (a.xcd_streams && ns % 8 != 0))
        return hipErrorInvalidValue;
    switch (a.d) {
        case 32: launch_mlp2_d<32>(a, ns, st); break;
        case 64: launch_mlp2_d<64>(a, ns, st); break;
        case 96: launch_mlp2_d<96>(a, ns, st); break;
        default: launch_mlp2_d<128>(a, ns, st); break;
    }
    return hipGetLastError();
}

}  // namespace tmk
