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
// tm_kernels.hip instead.
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

}  // namespace tmk
