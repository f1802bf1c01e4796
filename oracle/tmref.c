/*
 * tmref -- plain, slow fp64 CPU oracle for the Titans neural long-term memory.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or table with the HIP library.
 *
 * What it computes (sources are the five pages on Titans; "Titans, explained"
 * is the vibeengines.com page, "Attack of the Titans" the synthesis.ai post):
 *
 *  - The memory M is an MLP without biases: z_1 = x W_1, h_l = SiLU(z_l),
 *    z_{l+1} = h_l W_{l+1}, output y = z_L (row vectors, W_l is [d_in][d_out];
 *    the row convention of "k_t = x_t W_K" in "Titans, explained", step 1).
 *    depth 1 is the linear memory (one matrix).
 *  - Associative loss l(M; k, v) = ||M(k) - v||^2, summed over the output, no
 *    1/2 ("Titans, explained", step 2; its closing remark fixes the factor 2 of
 *    the linear gradient 2(M k - v) k^T).
 *  - Momentary surprise = gradient of that loss w.r.t. every weight, by plain
 *    backpropagation (step 2).
 *  - Momentum S_t = eta_t S_{t-1} - theta_t grad (step 3), then forgetting and
 *    write M_t = (1 - alpha_t) M_{t-1} + S_t with the new S_t (step 4).
 *  - Chunked form (step 6; "Attack of the Titans", Parallel training): the
 *    stream is cut into chunks of b tokens starting at the stream start, and
 *    every gradient inside a chunk is taken at the weights the chunk started
 *    with (t' = t - (t mod b)).  The momentum and forgetting recurrences above
 *    still run token by token; this file never uses a closed form for them.
 *  - Retrieval y = M(q) is a forward pass with no write (step 5).  In a
 *    combined store+retrieve call the queries of chunk c are read through the
 *    weights after chunk c has been written (read mode 0), or, the variant in
 *    which the queries read the memory before the chunk writes to it ("Attack
 *    of the Titans", the memory-as-context architecture), through the weights
 *    chunk c started with (read mode 1).  Read mode 2 reads every query
 *    through the memory right after its own token's write: inside a chunk the
 *    weights still move token by token (only the gradients sit at the chunk
 *    start), and query t sees them as they stand after token t, the way a
 *    linear-attention output is a lookup in a matrix memory updated at every
 *    step ("Attack of the Titans", the long-term memory section).
 *
 * Everything is fp64.  Inputs arrive as float32 arrays (bf16 inputs are passed
 * already widened, which is exact) and are widened to double on use.
 *
 * State layout (canonical, shared with the tests): per stream s = b*H + h,
 * 2P doubles: M_1 .. M_L then S_1 .. S_L, each W_l row-major [d_in][d_out].
 * Token arrays are [batch][n_tokens][heads][dim]; gates [batch][n_tokens][heads].
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* Loops over independent elements (the output columns of a product, the
 * rows of an outer product, the weights in the momentum and forgetting
 * updates) may be split over `n` threads when the library is built with
 * OpenMP: every element is still computed by one thread with its terms
 * summed in the order written, so the results are bitwise those of one
 * thread.  This only lets a workload with fewer streams than cores use the
 * spare cores; without OpenMP the pragma is ignored. */
#define TMREF_PRAGMA(x) _Pragma(#x)
#ifdef _OPENMP
#define PAR_FOR(n) TMREF_PRAGMA(omp parallel for schedule(static) num_threads(n) if ((n) > 1))
#else
#define PAR_FOR(n)
#endif

typedef struct {
    int dim, depth, expansion;
    int L;
    int din[8], dout[8];
    long off[9];          /* offset of W_l inside a P-vector; off[L] = P */
    int maxw;             /* widest layer output */
} mlp_t;

static int mlp_setup(mlp_t* m, int dim, int depth, int expansion) {
    if (dim <= 0 || depth < 1 || depth > 8 || expansion < 1) return -1;
    m->dim = dim; m->depth = depth; m->expansion = expansion; m->L = depth;
    int hid = depth == 1 ? dim : dim * expansion;
    m->off[0] = 0;
    m->maxw = dim > hid ? dim : hid;
    for (int l = 0; l < depth; l++) {
        m->din[l] = l == 0 ? dim : hid;
        m->dout[l] = l == depth - 1 ? dim : hid;
        m->off[l + 1] = m->off[l] + (long)m->din[l] * m->dout[l];
    }
    return 0;
}

static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Forward one row through the MLP.  act must hold (L+1)*maxw doubles and
 * pre must hold L*maxw doubles: act[l] is the input of layer l (act[0] = x),
 * pre[l] is layer l's pre-activation z.  Returns the output in out[dim].
 * nth: threads over blocks of output columns (each z[j] sums its inputs
 * i = 0, 1, ... in order either way). */
static void mlp_row_forward(const mlp_t* m, const double* W, const double* x,
                            double* act, double* pre, double* out, int nth) {
    int w = m->maxw;
    memcpy(act, x, sizeof(double) * m->dim);
    for (int l = 0; l < m->L; l++) {
        const double* Wl = W + m->off[l];
        const double* a = act + (long)l * w;
        double* z = pre + (long)l * w;
        int di = m->din[l], dn = m->dout[l];
        PAR_FOR(nth)
        for (int j0 = 0; j0 < dn; j0 += 64) {
            int j1 = j0 + 64 < dn ? j0 + 64 : dn;
            for (int j = j0; j < j1; j++) z[j] = 0.0;
            for (int i = 0; i < di; i++) {
                double ai = a[i];
                const double* row = Wl + (long)i * dn;
                for (int j = j0; j < j1; j++) z[j] += ai * row[j];
            }
        }
        double* nxt = act + (long)(l + 1) * w;
        if (l < m->L - 1) {
            for (int j = 0; j < dn; j++) nxt[j] = z[j] * sigm(z[j]);   /* SiLU */
        } else {
            memcpy(nxt, z, sizeof(double) * dn);
        }
    }
    memcpy(out, act + (long)m->L * w, sizeof(double) * m->dim);
}

/* Gradient of ||M(k) - v||^2 w.r.t. all weights, written to G (P doubles).
 * Scratch: act (L+1)*maxw, pre L*maxw, d0/d1 maxw each.  nth: threads over
 * rows (independent elements), as in mlp_row_forward. */
static double mlp_row_grad(const mlp_t* m, const double* W, const double* k,
                           const double* v, double* G, double* act, double* pre,
                           double* d0, double* d1, int nth) {
    int w = m->maxw;
    double* out = d1;
    mlp_row_forward(m, W, k, act, pre, out, nth);
    double loss = 0.0;
    /* dl/dy = 2 (y - v) */
    for (int j = 0; j < m->dim; j++) {
        double e = out[j] - v[j];
        loss += e * e;
        d0[j] = 2.0 * e;
    }
    double* delta = d0;   /* dl/dz_l for the current layer */
    double* other = d1;
    for (int l = m->L - 1; l >= 0; l--) {
        const double* a = act + (long)l * w;       /* input of layer l */
        int di = m->din[l], dn = m->dout[l];
        double* Gl = G + m->off[l];
        PAR_FOR(nth)
        for (int i = 0; i < di; i++) {
            double ai = a[i];
            double* row = Gl + (long)i * dn;
            for (int j = 0; j < dn; j++) row[j] = ai * delta[j];
        }
        if (l > 0) {
            /* dl/dh_{l-1} = delta W_l^T, then through SiLU'(z_{l-1}) */
            const double* Wl = W + m->off[l];
            const double* z = pre + (long)(l - 1) * w;
            PAR_FOR(nth)
            for (int i = 0; i < di; i++) {
                const double* row = Wl + (long)i * dn;
                double s = 0.0;
                for (int j = 0; j < dn; j++) s += row[j] * delta[j];
                double sg = sigm(z[i]);
                other[i] = s * sg * (1.0 + z[i] * (1.0 - sg));
            }
            double* t = delta; delta = other; other = t;
        }
    }
    return loss;
}

/* ---- exported single-row helpers (used by the oracle's own pin tests) ---- */

long tmref_param_count(int dim, int depth, int expansion) {
    mlp_t m;
    if (mlp_setup(&m, dim, depth, expansion)) return -1;
    return m.off[m.L];
}

int tmref_mlp_forward(int dim, int depth, int expansion, const double* W,
                      const double* x, double* y) {
    mlp_t m;
    if (mlp_setup(&m, dim, depth, expansion)) return -1;
    double* act = malloc(sizeof(double) * (size_t)(m.L + 1) * m.maxw);
    double* pre = malloc(sizeof(double) * (size_t)m.L * m.maxw);
    if (!act || !pre) { free(act); free(pre); return -2; }
    mlp_row_forward(&m, W, x, act, pre, y, 1);
    free(act); free(pre);
    return 0;
}

int tmref_mlp_grad(int dim, int depth, int expansion, const double* W,
                   const double* k, const double* v, double* G, double* loss) {
    mlp_t m;
    if (mlp_setup(&m, dim, depth, expansion)) return -1;
    double* act = malloc(sizeof(double) * (size_t)(m.L + 1) * m.maxw);
    double* pre = malloc(sizeof(double) * (size_t)m.L * m.maxw);
    double* d0 = malloc(sizeof(double) * (size_t)m.maxw);
    double* d1 = malloc(sizeof(double) * (size_t)m.maxw);
    if (!act || !pre || !d0 || !d1) { free(act); free(pre); free(d0); free(d1); return -2; }
    double l = mlp_row_grad(&m, W, k, v, G, act, pre, d0, d1, 1);
    if (loss) *loss = l;
    free(act); free(pre); free(d0); free(d1);
    return 0;
}

/* ---- the streaming store / retrieve ---- */

typedef struct {
    const mlp_t* m;
    int chunk, batch, heads, n_tokens;
    const float *k, *v, *q, *theta, *eta, *alpha;
    double* state;
    double* y;            /* NULL: store only */
    int retrieve_only;
    int read;                 /* 0: queries after the chunk's write; 1: before;
                                 2: each after its own token's write */
    int tid, nthreads;
    int inner;                /* threads per stream for its element loops */
    int err;
} job_t;

static void widen(double* dst, const float* src, int n) {
    for (int i = 0; i < n; i++) dst[i] = (double)src[i];
}

static void* run_streams(void* arg) {
    job_t* J = (job_t*)arg;
    const mlp_t* m = J->m;
    long P = m->off[m->L];
    int d = m->dim, H = J->heads, T = J->n_tokens, b = J->chunk;
    int w = m->maxw, nth = J->inner;
    double* M0 = malloc(sizeof(double) * (size_t)P);
    double* G = malloc(sizeof(double) * (size_t)P);
    double* act = malloc(sizeof(double) * (size_t)(m->L + 1) * w);
    double* pre = malloc(sizeof(double) * (size_t)m->L * w);
    double* d0 = malloc(sizeof(double) * (size_t)w);
    double* d1 = malloc(sizeof(double) * (size_t)w);
    double* kk = malloc(sizeof(double) * (size_t)d);
    double* vv = malloc(sizeof(double) * (size_t)d);
    double* out = malloc(sizeof(double) * (size_t)d);
    if (!M0 || !G || !act || !pre || !d0 || !d1 || !kk || !vv || !out) {
        J->err = -2;
        goto done;
    }
    for (int s = J->tid; s < J->batch * H; s += J->nthreads) {
        int bi = s / H, hi = s % H;
        double* M = J->state + (size_t)s * 2 * P;
        double* S = M + P;
        if (J->retrieve_only) {
            for (int t = 0; t < T; t++) {
                size_t row = ((size_t)bi * T + t) * H + hi;
                widen(kk, J->q + row * d, d);
                mlp_row_forward(m, M, kk, act, pre, out, nth);
                memcpy(J->y + row * d, out, sizeof(double) * d);
            }
            continue;
        }
        for (int c0 = 0; c0 < T; c0 += b) {
            /* weights at the start of the chunk: every gradient of the chunk
             * is taken here */
            memcpy(M0, M, sizeof(double) * (size_t)P);
            if (J->y && J->read == 1) {
                /* read the chunk's queries before the chunk writes */
                for (int t = c0; t < c0 + b; t++) {
                    size_t row = ((size_t)bi * T + t) * H + hi;
                    widen(kk, J->q + row * d, d);
                    mlp_row_forward(m, M, kk, act, pre, out, nth);
                    memcpy(J->y + row * d, out, sizeof(double) * d);
                }
            }
            for (int t = c0; t < c0 + b; t++) {
                size_t row = ((size_t)bi * T + t) * H + hi;
                widen(kk, J->k + row * d, d);
                widen(vv, J->v + row * d, d);
                mlp_row_grad(m, M0, kk, vv, G, act, pre, d0, d1, nth);
                double th = J->theta[row], et = J->eta[row], al = J->alpha[row];
                PAR_FOR(nth)
                for (long p = 0; p < P; p++) S[p] = et * S[p] - th * G[p];
                PAR_FOR(nth)
                for (long p = 0; p < P; p++) M[p] = (1.0 - al) * M[p] + S[p];
                if (J->y && J->read == 2) {
                    /* query t through the memory as token t left it */
                    widen(kk, J->q + row * d, d);
                    mlp_row_forward(m, M, kk, act, pre, out, nth);
                    memcpy(J->y + row * d, out, sizeof(double) * d);
                }
            }
            if (J->y && J->read == 0) {
                /* read the chunk's queries through the freshly written memory */
                for (int t = c0; t < c0 + b; t++) {
                    size_t row = ((size_t)bi * T + t) * H + hi;
                    widen(kk, J->q + row * d, d);
                    mlp_row_forward(m, M, kk, act, pre, out, nth);
                    memcpy(J->y + row * d, out, sizeof(double) * d);
                }
            }
        }
    }
done:
    free(M0); free(G); free(act); free(pre); free(d0); free(d1);
    free(kk); free(vv); free(out);
    return NULL;
}

static int run(int dim, int depth, int expansion, int chunk, int batch, int heads,
               int n_tokens, const float* k, const float* v, const float* q,
               const float* theta, const float* eta, const float* alpha,
               double* state, double* y, int retrieve_only, int read, int n_threads) {
    mlp_t m;
    if (mlp_setup(&m, dim, depth, expansion)) return -1;
    if (batch <= 0 || heads <= 0 || n_tokens < 0 || chunk <= 0) return -1;
    if (!retrieve_only && n_tokens % chunk) return -3;
    int ns = batch * heads;
    if (n_threads <= 0) n_threads = 1;
    /* one worker per stream; threads left over split each stream's loops */
    int inner = n_threads / (n_threads < ns ? n_threads : ns);
    if (n_threads > ns) n_threads = ns;
    job_t* jobs = calloc((size_t)n_threads, sizeof(job_t));
    pthread_t* th = calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    for (int i = 0; i < n_threads; i++) {
        job_t J = {&m, chunk, batch, heads, n_tokens, k, v, q, theta, eta, alpha,
                   state, y, retrieve_only, read, i, n_threads, inner, 0};
        jobs[i] = J;
    }
    for (int i = 1; i < n_threads; i++) pthread_create(&th[i], NULL, run_streams, &jobs[i]);
    run_streams(&jobs[0]);
    int err = 0;
    for (int i = 1; i < n_threads; i++) pthread_join(th[i], NULL);
    for (int i = 0; i < n_threads; i++) if (jobs[i].err) err = jobs[i].err;
    free(jobs); free(th);
    return err;
}

/* Store the call's n_tokens into the memory (and, if y != NULL, read the
 * queries: read = 0 chunk by chunk through the memory after the chunk's
 * write, read = 1 through the memory the chunk started with, read = 2 each
 * through the memory right after its own token's write).  state is
 * updated in place.  Returns 0, -1 (bad sizes or mode), -2 (out of memory),
 * -3 (n_tokens not a multiple of chunk). */
int tmref_forward_read(int dim, int depth, int expansion, int chunk, int batch, int heads,
                       int n_tokens, const float* k, const float* v, const float* q,
                       const float* theta, const float* eta, const float* alpha,
                       double* state, double* y, int read, int n_threads) {
    if (y && !q) return -1;
    if (read < 0 || read > 2) return -1;
    return run(dim, depth, expansion, chunk, batch, heads, n_tokens, k, v, q,
               theta, eta, alpha, state, y, 0, read, n_threads);
}

int tmref_forward(int dim, int depth, int expansion, int chunk, int batch, int heads,
                  int n_tokens, const float* k, const float* v, const float* q,
                  const float* theta, const float* eta, const float* alpha,
                  double* state, double* y, int n_threads) {
    return tmref_forward_read(dim, depth, expansion, chunk, batch, heads, n_tokens, k, v, q,
                              theta, eta, alpha, state, y, 0, n_threads);
}

/* Read only: y = M(q) for every query, the state untouched. */
int tmref_retrieve(int dim, int depth, int expansion, int batch, int heads,
                   int n_tokens, const double* state, const float* q, double* y,
                   int n_threads) {
    return run(dim, depth, expansion, 1, batch, heads, n_tokens, NULL, NULL, q,
               NULL, NULL, NULL, (double*)state, y, 1, 0, n_threads);
}
