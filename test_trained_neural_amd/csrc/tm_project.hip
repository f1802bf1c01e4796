// HIP kernels of the Titans memory's input side on CDNA4 (gfx950): each
// token's model vector x to the key, value and query of every head
// (projections on the matrix cores, a short causal depthwise convolution with
// the stream's history carried across calls, l2-normalised keys and queries)
// and the three gates sigmoid(x w_g + b_g) ("Titans, explained", steps 1, 4
// and 5).
#include "tm_device.h"

namespace tmk {

// One workgroup per (batch row b, tile of RT tokens, projection i, head h):
// the head's d channels of projection i for tokens t0-3 .. t0+RT-1 on the
// matrix cores (K = D; the 3 rows before the tile feed the convolution),
// staged in LDS as fp32, then the convolution, the row norms (keys and
// queries) and the store.  Before the call's first token the rows come from
// the history.  Waves take 16-column blocks wave, wave + 8, ...; rows
// outside the call multiply zeros.
constexpr int PROJ_HALO = MAX_CONV - 1;

// The gates of RT tokens of batch row b: sigmoid(x w_g + b_g) for every
// gate g and head.  Wave w owns the RT/8 consecutive tokens from t0 + w*RT/8;
// a lane takes 8 consecutive inputs of each 512-input chunk of D.  The steps
// (gate-head gh, chunk) run in order and each issues the next step's loads
// before its own arithmetic and reduction, so a step costs about one load
// round trip; the two register buffers alternate by explicit unrolling.
template <class OP, int RT>
__device__ void gates_tile(const ProjArgs& a, int b, int t0) {
    constexpr int TPW = RT / 8;
    struct Buf {
        f32x8 w;
        f32x8 x[TPW];
    };
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tw = t0 + wave * TPW;
    const int nch = (a.D + 511) >> 9;
    const int nit = 3 * a.H * nch;
    const OP* xb = reinterpret_cast<const OP*>(a.x) + (long)b * a.T * a.D;
    auto load = [&](int it, Buf& o) {
        const int gh = it / nch, c = (it - gh * nch) * 512 + lane * 8;
        const bool ok = c < a.D;                     // D is a multiple of 8
        const int cc = ok ? c : 0;
        o.w = keep_if(ld8(a.wg + (long)gh * a.D + cc), ok);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            o.x[t] = keep_if(to_f32v(ld8(xb + (long)min(tw + t, a.T - 1) * a.D + cc)), ok);
    };
    float acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = 0.f;
    auto step = [&](int it, const Buf& cur, Buf& nxt) {
        if (it + 1 < nit) load(it + 1, nxt);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[t] += cur.x[t][e] * cur.w[e];
        const int gh = it / nch;
        if (it - gh * nch == nch - 1) {              // the gate's last chunk (wave-uniform)
            const int g = gh / a.H, h = gh - g * a.H;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) acc[t] += __shfl_xor(acc[t], off, 64);
                const int tok = tw + t;
                if (lane == 0 && tok < min(t0 + RT, a.T))
                    a.gate[g][((long)b * a.T + tok) * a.H + h] = sigmoid(acc[t] + a.gb[g]);
                acc[t] = 0.f;
            }
        }
    };
    Buf A, B;
    load(0, A);
    for (int it = 0; it < nit; it += 2) {
        step(it, A, B);
        if (it + 1 < nit) step(it + 1, B, A);
    }
}

template <class OP, int RT, int G>
__global__ __launch_bounds__(512) void project_kernel(ProjArgs a) {
    typedef typename Frag<OP>::T F;
    constexpr int NRB = (RT + PROJ_HALO + 15) / 16;   // row blocks of the staged tile
    constexpr int KC = sizeof(OP) == 2 ? 4 : 2;       // K steps (of 32) per staged chunk
    constexpr int AP = KC * 32 + 8;                   // staged row pitch (elements, 16-byte rows)
    constexpr int PPR = KC * 32 * (int)sizeof(OP) / 16;   // 16-byte pieces per staged row
    constexpr int NPC = NRB * 16 * PPR;               // pieces per chunk
    constexpr int NPT = (NPC + 511) / 512;            // per thread
    typedef __attribute__((ext_vector_type(4))) int I4;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kofs = 8 * (lane >> 4);
    const int b = blockIdx.z, i = blockIdx.y / a.H, h = blockIdx.y - i * a.H;
    const int t0 = blockIdx.x * RT, d = a.d, D = a.D, HD = a.H * a.d;
    if ((int)blockIdx.y == 3 * a.H) {   // the last grid row: the tile's gates
        gates_tile<OP, RT>(a, b, t0);
        return;
    }
    const int ncb = d >> 4, nks = D >> 5;
    const int DP = d + 4;                             // LDS row pitch (floats)
    float* P = reinterpret_cast<float*>(lds);         // [NRB*16][DP]: projections of rows t0-3 ..
    f32x4* taps = reinterpret_cast<f32x4*>(P + NRB * 16 * DP);   // [d]: the channels' taps (zero past K)
    OP* As = reinterpret_cast<OP*>(taps + d);         // [NRB*16][AP]: the staged x chunk
    const OP* x = reinterpret_cast<const OP*>(a.x) + (long)b * a.T * D;
    const OP* w = reinterpret_cast<const OP*>(a.w) + ((long)i * HD + (long)h * d) * D;

    // the x tile (token t0 - 3 + r, r < NRB*16) is staged through LDS one
    // chunk of KC*32 inputs at a time, read once per workgroup; rows outside
    // the call and inputs past D are zeros
    const int npass = (ncb + 8 * G - 1) / (8 * G);    // the same for every wave (barriers below)
    for (int pass = 0; pass < npass; ++pass) {
        const int c0 = wave + 8 * G * pass;
        f32x4 acc[NRB][G];
        const OP* brow[G];
        bool bok[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int cb = c0 + 8 * g;
            bok[g] = cb < ncb;
            brow[g] = w + (long)(min(cb, ncb - 1) * 16 + (lane & 15)) * D + kofs;
#pragma unroll
            for (int m = 0; m < NRB; ++m) acc[m][g] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        for (int k0 = 0; k0 < nks; k0 += KC) {
            // this chunk's weight fragments and staged pieces, all requested
            // before anything waits
            F bv[KC][G];
#pragma unroll
            for (int q = 0; q < KC; ++q)
#pragma unroll
                for (int g = 0; g < G; ++g) bv[q][g] = cvt<OP>(ld8(brow[g] + min(k0 + q, nks - 1) * 32));
            I4 pc[NPT];
#pragma unroll
            for (int n = 0; n < NPT; ++n) {
                const int pi = min(tid + 512 * n, NPC - 1), r = pi / PPR, c = (pi % PPR) * (16 / (int)sizeof(OP));
                const int u = t0 - PROJ_HALO + r, kk = k0 * 32 + c;
                const I4 v = *reinterpret_cast<const I4*>(x + (long)min(max(u, 0), a.T - 1) * D +
                                                          min(kk, D - 16 / (int)sizeof(OP)));
                pc[n] = keep_if(v, u >= 0 && u < a.T && kk < D);
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();   // the previous chunk's reads of As are done
#pragma unroll
            for (int n = 0; n < NPT; ++n) {
                const int pi = tid + 512 * n;
                if (pi < NPC) {
                    const int r = pi / PPR, c = (pi % PPR) * (16 / (int)sizeof(OP));
                    *reinterpret_cast<I4*>(As + r * AP + c) = pc[n];
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < KC; ++q) {
                const bool live = k0 + q < nks;
                F av[NRB];
#pragma unroll
                for (int m = 0; m < NRB; ++m)
                    av[m] = *reinterpret_cast<const F*>(As + (m * 16 + (lane & 15)) * AP + q * 32 + kofs);
#pragma unroll
                for (int m = 0; m < NRB; ++m)
#pragma unroll
                    for (int g = 0; g < G; ++g) mma(acc[m][g], av[m], keep_if(bv[q][g], live));
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
            if (bok[g])   // wave-uniform
#pragma unroll
                for (int m = 0; m < NRB; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        P[(m * 16 + 4 * (lane >> 4) + e) * DP + (c0 + 8 * g) * 16 + (lane & 15)] = acc[m][g][e];
    }
    __syncthreads();
    // rows before the call's first token: the history (projections of the
    // previous call's last K-1 tokens, oldest first)
    if (t0 < PROJ_HALO && a.K > 1) {
        for (int idx = tid; idx < PROJ_HALO * d; idx += 512) {
            const int r = idx / d, c = idx - r * d, u = t0 - PROJ_HALO + r;
            if (u < 0 && u >= -(a.K - 1))
                P[r * DP + c] = a.hist[(((long)b * (a.K - 1) + (a.K - 1 + u)) * 3 + i) * HD + (long)h * d + c];
        }
        __syncthreads();
    }
    for (int c = tid; c < d; c += 512) {
        const float* tp = a.conv + ((long)i * HD + (long)h * d + c) * a.K;
        f32x4 t4;
#pragma unroll
        for (int j = 0; j < MAX_CONV; ++j) t4[j] = j < a.K ? tp[j] : 0.f;
        taps[c] = t4;
    }
    __syncthreads();
    // the convolution, the row norms and the store: wave w owns rows
    // RPW*w .. RPW*w + RPW-1 of the tile, the LPR lanes of a row split its
    // channels (lane l: channels l, l + LPR, ...), so a row's sum of squares
    // needs log2(LPR) cross-lane steps
    constexpr int RPW = RT / 8, LPR = 64 / RPW, CPL = 1024 / LPR;
    const int r = RPW * wave + lane / LPR, lr = lane % LPR;
    const int ncl = (d - lr + LPR - 1) / LPR;          // this lane's channels
    float o[CPL];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lr + LPR * k;
        float acc = 0.f;
        if (k < ncl) {
            const f32x4 t4 = taps[c];
#pragma unroll
            for (int j = 0; j < MAX_CONV; ++j) acc += t4[j] * P[(r + PROJ_HALO - j) * DP + c];
        }
        o[k] = acc;
        ss += acc * acc;
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float scale = i != 1 ? __builtin_amdgcn_rcpf(fmaxf(sqrtf(ss), 1e-12f)) : 1.f;
    if (t0 + r < a.T) {
        OP* out = reinterpret_cast<OP*>(a.out[i]) + (((long)b * a.T + t0 + r) * a.H + h) * d;
#pragma unroll
        for (int k = 0; k < CPL; ++k)
            if (k < ncl) out[lr + LPR * k] = (OP)(o[k] * scale);
    }
}

// The new history: per channel of each projection, the projections of the
// call's last K-1 tokens (oldest first), or, where the call is shorter, the
// old history moved up.  One wave per (batch row, projection, channel),
// lanes split the width; each wave reads the old values it needs before it
// writes, and waves own disjoint channels.
template <class OP>
__global__ __launch_bounds__(256) void history_kernel(ProjArgs a) {
    const int HD = a.H * a.d, K1 = a.K - 1;
    const long wv = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wv >= (long)a.B * 3 * HD) return;   // wave-uniform
    const int n = (int)(wv % HD), i = (int)((wv / HD) % 3), b = (int)(wv / (3L * HD));
    float old[MAX_CONV - 1];
#pragma unroll
    for (int r = 0; r < MAX_CONV - 1; ++r)
        old[r] = (r < K1) ? a.hist[(((long)b * K1 + r) * 3 + i) * HD + n] : 0.f;
    const OP* w = reinterpret_cast<const OP*>(a.w) + ((long)i * HD + n) * a.D;
    float nw[MAX_CONV - 1];
#pragma unroll
    for (int r = 0; r < MAX_CONV - 1; ++r) {
        const int u = a.T - K1 + r;
        float v = 0.f;
        if (r < K1 && u >= 0) {   // wave-uniform
            const OP* x = reinterpret_cast<const OP*>(a.x) + ((long)b * a.T + u) * a.D;
            for (int c = lane; c < a.D; c += 64) v += (float)x[c] * (float)w[c];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        } else {
#pragma unroll
            for (int q = 0; q < MAX_CONV - 1; ++q)
                if (q == r + a.T) v = old[q];
        }
        nw[r] = v;
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < MAX_CONV - 1; ++r)
            if (r < K1) a.hist[(((long)b * K1 + r) * 3 + i) * HD + n] = nw[r];
    }
}

template <class OP, int RT, int G>
static void launch_project_g(const ProjArgs& p, hipStream_t st) {
    constexpr int NRB = (RT + PROJ_HALO + 15) / 16;
    constexpr int AP = (sizeof(OP) == 2 ? 4 : 2) * 32 + 8;
    const size_t lds = (size_t)NRB * 16 * (p.d + 4) * 4 + (size_t)p.d * 16 + (size_t)NRB * 16 * AP * sizeof(OP);
    if (lds > 64 * 1024)   // above the default dynamic LDS limit
        (void)hipFuncSetAttribute((const void*)project_kernel<OP, RT, G>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    dim3 grid((p.T + RT - 1) / RT, 3 * p.H + 1, p.B);   // + one grid row for the gates
    launch_k((project_kernel<OP, RT, G>), grid, dim3(512), lds, st, p);
}

// G: column blocks a wave holds per pass, as few as cover the head in one
// pass of the 8 waves (4 at most)
template <class OP, int RT>
static void launch_project_rt(const ProjArgs& p, hipStream_t st) {
    const int g = min(4, (p.d / 16 + 7) / 8);
    if (g == 1) launch_project_g<OP, RT, 1>(p, st);
    else if (g == 2) launch_project_g<OP, RT, 2>(p, st);
    else if (g == 3) launch_project_g<OP, RT, 3>(p, st);
    else launch_project_g<OP, RT, 4>(p, st);
}

hipError_t launch_project(const ProjArgs& p, int f32, hipStream_t st) {
    if (p.T == 0 || p.B == 0) return hipSuccess;
    if (p.d > 1024 || p.d % 32 != 0 || p.D % 32 != 0 || p.K < 1 || p.K > MAX_CONV) return hipErrorInvalidValue;
    // tiles of 32 tokens; 16 for the widest heads (the staged rows fill LDS)
    // and for calls whose 32-token grid would not cover the 256 compute
    // units (short calls: more, shorter workgroups finish sooner)
    const long grid32 = (long)((p.T + 31) / 32) * (3 * p.H + 1) * p.B;
    if (p.d <= 512 && grid32 >= 256) {
        if (f32) launch_project_rt<float, 32>(p, st);
        else launch_project_rt<bf16, 32>(p, st);
    } else {
        if (f32) launch_project_rt<float, 16>(p, st);
        else launch_project_rt<bf16, 16>(p, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.K == 1) return e;
    const long nw = (long)p.B * 3 * p.H * p.d;   // one wave each
    if (f32) launch_k(history_kernel<float>, dim3((unsigned)((nw + 3) / 4)), dim3(256), 0, st, p);
    else launch_k(history_kernel<bf16>, dim3((unsigned)((nw + 3) / 4)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace tmk
