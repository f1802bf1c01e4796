// C-ABI runtime of the neural-memory library: argument checks, the state
// and workspace layouts, and the per-call launch sequence (the chunk loop).
//
// State blob: [header 256 B][M fp32 ns*P][S fp32 ns*P][Wt bf16 ns*P], each
// region 256-byte aligned; per stream the layers follow each other.  In M and
// S, W_0 and W_1 are in matrix-instruction accumulator orders (cf0, cf1) and
// the other layers row-major [d_in][d_out]; Wt holds every layer fragment-packed
// [d_out][d_in].  Export and import convert to and from the canonical
// row-major form.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <thread>
#include <unordered_map>
#include <vector>

#include "../../include/tm.h"
#include "tm_internal.h"

using namespace tmk;

namespace tmk {
thread_local LaunchEvents g_launch_ev;
}

// Workspace of tm_forward_noalloc, for callers that cannot allocate device
// memory: a file-scope device array of SCRATCH_BYTES, one copy per GPU the
// library runs on, held until the process ends.  In host code `scratch` only
// names the symbol; its device address on the current GPU comes from
// hipGetSymbolAddress (scratch_address below) and is the only form passed to
// kernels.
constexpr size_t SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// A call's launch sequence replayed as a HIP graph: keyed by everything the
// kernels' arguments depend on (device, every pointer and every size).
struct GraphEntry {
    int dev, kind, batch, heads, n_tokens, dtype, opt, extra;
    const void* p[16];
    int seen;                    // sightings before capture
    hipGraphExec_t exec;
    unsigned long long last;     // LRU stamp
};

struct tm_ctx {
    std::mutex* gmu;
    std::vector<GraphEntry>* graphs;
    std::vector<std::pair<int, hipStream_t>>* capture_streams;
    // the backward's second stream per device, with its fork and join
    // events (independent products of a chunk run on both)
    struct Side {
        int dev;
        hipStream_t s;
        hipEvent_t fork, join;
        int idx;   // which of the device's extra streams
        std::thread::id tid;   // the host thread that uses it
    };
    std::vector<Side>* sides;
    unsigned long long stamp;
    int dim, depth, expansion, chunk, hidden, L;
    int din[MAXL], dout[MAXL];
    long off[MAXL + 1];
    long P;
    int tj[MAXL];
    int tbase[MAXL + 1];
    uint64_t hash;
};

namespace {

constexpr long RET_ROWS = 2048;   // query rows per stream per retrieve pass
constexpr int RET_TILED_ROWS = 256;   // from this many rows a retrieve pass uses the tiled product

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct StateLayout {
    size_t M, S, Wt, total;
};

// A call that runs its streams in groups (run_store) sees the state of
// streams s0 .. s0 + ns - 1 of a blob laid out for ns_total streams.
struct StateView {
    long s0, ns_total;
};
thread_local StateView g_sview{0, 0};

StateLayout state_layout(const tm_ctx* c, long ns) {
    const long N = g_sview.ns_total > 0 ? g_sview.ns_total : ns;
    const size_t s0 = g_sview.ns_total > 0 ? (size_t)g_sview.s0 : 0;
    StateLayout s;
    s.M = sizeof(StateHeader);
    s.S = s.M + al256((size_t)N * c->P * 4);
    s.Wt = s.S + al256((size_t)N * c->P * 4);
    s.total = s.Wt + al256((size_t)N * c->P * 2);
    s.M += s0 * c->P * 4;
    s.S += s0 * c->P * 4;
    s.Wt += s0 * c->P * 2;
    return s;
}

// Workspace of one call.  Every matrix-instruction operand that one kernel
// leaves for another is stored fragment-packed (pk() in tm_internal.h),
// sized in 4-byte elements so either operand type fits.
struct WsLayout {
    size_t cc, dc, cs, act[MAXL], dsl[MAXL], dlp[MAXL], kt, xk, xq, ht[MAXL], dct[MAXL], ddt[MAXL], ht1[2],
        m1x, r3x[2], r3c, r3p, ret[2], total;
    long coef_ss, cs_ss, act_ss, dsl_ss, dlp_ss[MAXL], kt_ss, x_ss, xc, ht_ss, dt_ss[MAXL], r3x_ss, r3c_ss, r3c_cs,
        r3p_ss, ret_ss, ret_rows;
    int bp, C;
};

WsLayout ws_layout(const tm_ctx* c, long ns, long T) {
    WsLayout w;
    memset(&w, 0, sizeof(w));
    const long b = c->chunk, C = (T + b - 1) / b, h = c->hidden;
    size_t o = 0;
    w.coef_ss = T;
    w.cc = o; o += al256((size_t)ns * T * 4);
    w.dc = o; o += al256((size_t)ns * T * 4);
    w.cs_ss = C * 4;
    w.cs = o; o += al256((size_t)ns * C * 16);
    // hidden layers: activations of [queries of chunk c-1; keys of chunk c]
    // (packed [2b][h]) and SiLU'(z) of the key rows (row-major [b][h])
    w.act_ss = pk_size(2 * b, h);
    w.dsl_ss = b * h;
    for (int l = 0; l + 1 < c->L; ++l) {
        w.act[l] = o; o += al256((size_t)ns * w.act_ss * 4);
        w.dsl[l] = o; o += al256((size_t)ns * w.dsl_ss * 4);
    }
    // Delta of layers 1.. (packed [b][dout]; layer 0's is formed in place)
    for (int l = 1; l < c->L; ++l) {
        w.dlp_ss[l] = pk_size(b, c->dout[l]);
        w.dlp[l] = o; o += al256((size_t)ns * w.dlp_ss[l] * 4);
    }
    // transposed operands of the update: packed [rows][bp]
    w.bp = (int)((b + 31) / 32 * 32);
    w.C = (int)C;
    w.kt_ss = C * c->dim * w.bp;
    w.kt = o; o += al256((size_t)ns * w.kt_ss * 4);
    // every chunk's key and query rows, packed [b][dim]
    w.xc = pk_size(b, c->dim);
    w.x_ss = C * w.xc;
    w.xk = o; o += al256((size_t)ns * w.x_ss * 4);
    w.xq = o; o += al256((size_t)ns * w.x_ss * 4);
    w.ht_ss = h * w.bp;
    for (int l = 0; l + 1 < c->L; ++l) {
        w.ht[l] = o; o += al256((size_t)ns * w.ht_ss * 4);
    }
    for (int l = 0; l < c->L; ++l) {
        w.dt_ss[l] = (long)c->dout[l] * w.bp;
        w.dct[l] = o; o += al256((size_t)ns * w.dt_ss[l] * 4);
        w.ddt[l] = o; o += al256((size_t)ns * w.dt_ss[l] * 4);
    }
    // the first layer's transposed key-row activations, alternating between
    // the chunk being written and the chunk being reduced
    for (int i = 0; i < 2; ++i) {
        w.ht1[i] = o; o += al256((size_t)ns * w.ht_ss * 4);
    }
    // depth 2: W_1's M in the other buffer of an update in workgroups of
    // its own (the state's layout, stream stride P_1)
    if (c->L == 2) {
        w.m1x = o; o += al256((size_t)ns * c->din[1] * c->dout[1] * 4);
    }
    // per-token read: the query rows' hidden layers (ping-pong, packed
    // [b][h]), the correction's coefficient-scaled scores (packed [b][bp]) and
    // the rows' pm_t, ps_t
    if (c->L >= 2) {
        w.r3x_ss = pk_size(b, h);
        for (int i = 0; i < 2; ++i) {
            w.r3x[i] = o; o += al256((size_t)ns * w.r3x_ss * 4);
        }
    }
    // C of layer 0 for every chunk of the call (fp32 [16 ceil(b/16)][bp]
    // each; the other layers form theirs in place); pm_t, ps_t of every chunk
    w.r3c_cs = ((b + 15) / 16 * 16) * w.bp;
    w.r3c_ss = C * w.r3c_cs;
    w.r3c = o; o += al256((size_t)ns * w.r3c_ss * 4);
    w.r3p_ss = C * 2 * b;
    w.r3p = o; o += al256((size_t)ns * w.r3p_ss * 4);
    size_t fwd_total = o;
    // retrieve: ping-pong activations of up to RET_ROWS query rows (packed)
    w.ret_rows = T < RET_ROWS ? T : RET_ROWS;
    w.ret_ss = pk_size(w.ret_rows, h);
    size_t r = 0;
    if (c->L > 1) {
        w.ret[0] = r; r += al256((size_t)ns * w.ret_ss * 4);
        w.ret[1] = r; r += al256((size_t)ns * w.ret_ss * 4);
    }
    w.total = fwd_total > r ? fwd_total : r;
    if (w.total == 0) w.total = 256;
    return w;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

uint64_t fnv(uint64_t h, uint64_t x) {
    for (int i = 0; i < 8; ++i) { h ^= (x >> (8 * i)) & 0xff; h *= 1099511628211ull; }
    return h;
}

tm_status hip_status(hipError_t e) { return e == hipSuccess ? TM_OK : TM_ERR_HIP; }

// Host-side record of every state blob that tm_state_init or
// tm_state_import set up in this process: the configuration hash, batch and
// heads its header holds.  The compute calls look their state up here before
// launching anything, so a blob made for another configuration, batch or
// head count (or never set up) is refused with TM_ERR_STATE instead of being
// read or written past its end on the device.  Keyed by the device address
// (unique across devices); a blob set up again under another shape replaces
// its record.
struct StateRec {
    uint64_t hash;
    int batch, heads;
};
std::mutex g_smu;
std::unordered_map<uintptr_t, StateRec>* g_states = nullptr;

void state_register(const tm_ctx* c, const void* st, int batch, int heads) {
    std::lock_guard<std::mutex> g(g_smu);
    if (!g_states) g_states = new std::unordered_map<uintptr_t, StateRec>;
    (*g_states)[(uintptr_t)st] = StateRec{c->hash, batch, heads};
}

// TM_OK if `st` was set up for this configuration, batch and heads.
tm_status state_lookup(const tm_ctx* c, const void* st, int batch, int heads) {
    std::lock_guard<std::mutex> g(g_smu);
    if (!g_states) return TM_ERR_STATE;
    auto it = g_states->find((uintptr_t)st);
    if (it == g_states->end()) return TM_ERR_STATE;
    const StateRec& r = it->second;
    return r.hash == c->hash && r.batch == batch && r.heads == heads ? TM_OK : TM_ERR_STATE;
}

// TM_LOG=1 prints each call's configuration and launch plan to stderr once
// per distinct call shape; TM_LOG=2 also prints graph captures and replays.
// (each switch is read once, by a thread-safe static initialisation)
int log_level() {
    static const int lvl = [] {
        const char* e = getenv("TM_LOG");
        return e ? atoi(e) : 0;
    }();
    return lvl;
}

// compute units of the current device (queried once per device)
hipError_t compute_units(int* out) {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> g(mu);
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (cache[dev] == 0) {
        e = hipDeviceGetAttribute(&cache[dev], hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    *out = cache[dev];
    return hipSuccess;
}

// Device address of `scratch` on the current GPU, looked up once per device
// (with that device current) and kept.
hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

// ---- optional per-launch timing (tm_timing_enable / tm_timing_read) ----
// (class 3 is unused: the update of layers 1.. rides in the first-layer launch)
enum {
    K_SCAN = 0, K_FWD = 1, K_BWD = 2, K_FIRST = 4, K_R3 = 5, K_PROJ = 6, K_MAC = 7,
    K_BSTATE = 8,   // tm_backward: the launches that stream the state (recompute's write, adjoint update)
    K_BREST = 9,    // tm_backward: its other products, element-wise steps and coefficients
    K_CLASSES = 10
};
struct Timed {
    hipEvent_t a, b;
    int kind;
};
std::mutex g_tmu;
int g_timing = 0;   // bit mask of timed kernel classes
std::vector<Timed> g_pending;
std::vector<hipEvent_t> g_pool;
double g_ms[K_CLASSES];
long long g_n[K_CLASSES];

hipEvent_t pool_get() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// The launch inside `launch` records the pair with its own dispatch
// (launch_k); a launch that turned out to be empty records nothing and is
// not counted.
template <class F>
hipError_t timed(int kind, hipStream_t st, F&& launch) {
    (void)st;
    bool on;
    {
        std::lock_guard<std::mutex> g(g_tmu);
        on = (g_timing >> kind) & 1;
    }
    if (!on) return launch();
    hipEvent_t a, b;
    {
        std::lock_guard<std::mutex> g(g_tmu);
        a = pool_get();
        b = pool_get();
    }
    if (!a || !b) return hipErrorOutOfMemory;
    g_launch_ev = LaunchEvents{a, b, false};
    const hipError_t e = launch();
    const bool used = g_launch_ev.used;
    g_launch_ev = LaunchEvents{};
    std::lock_guard<std::mutex> g(g_tmu);
    if (e != hipSuccess || !used) {
        g_pool.push_back(a);
        g_pool.push_back(b);
        return e;
    }
    g_pending.push_back(Timed{a, b, kind});
    return hipSuccess;
}

// ---- TM_LOG diagnostics ----
thread_local bool g_log_plan = false;   // the running launch sequence prints its plan

const char* kind_name(int kind) {
    switch (kind) {
        case 0: return "tm_state_init";
        case 1: return "tm_store";
        case 2: return "tm_forward";
        case 3: return "tm_retrieve";
        case 4: return "tm_forward_ex(read before write)";
        case 5: return "tm_project";
        case 6: return "tm_forward_ex(read per token)";
        case 7: return "tm_backward";
    }
    return "?";
}

void log_call(const tm_ctx* c, const GraphEntry& k) {
    fprintf(stderr,
            "[tm] new call shape: %s, memory dim %d depth %d expansion %d chunk %d (P = %ld), batch %d, heads %d, "
            "n_tokens %d, %s\n",
            kind_name(k.kind), c->dim, c->depth, c->expansion, c->chunk, c->P, k.batch, k.heads, k.n_tokens,
            k.dtype == TM_BF16 ? "bf16" : "fp32");
}

// ---- graph replay of repeated calls ----
// process-wide switches, set by the *_enable calls from any thread
std::atomic<bool> g_graphs{true};
std::atomic<bool> g_w1_split{true};       // tm_w1_split_enable
std::atomic<bool> g_store_groups{true};   // tm_store_groups_enable
// TM_XCD_STREAMS=0 turns the first-layer blocks' grouping by XCD off (for
// comparing the two mappings; the results are bitwise the same)
bool xcd_streams_on() {
    static const bool on = [] {
        const char* e = getenv("TM_XCD_STREAMS");
        return !(e && e[0] == '0');
    }();
    return on;
}
constexpr size_t MAX_GRAPHS = 16;

// Runs `launch(stream)`.  A call whose key has been seen before is captured
// once into a graph on a private stream and from then on replayed on the
// caller's stream; first sightings and timed runs launch directly.
template <class F>
tm_status with_graph(const tm_ctx* cc, GraphEntry key, hipStream_t st, F&& launch) {
    tm_ctx* c = const_cast<tm_ctx*>(cc);
    bool timing;
    {
        std::lock_guard<std::mutex> g(g_tmu);
        timing = g_timing != 0;
    }
    if (!g_graphs || timing) return launch(st);
    if (hipGetDevice(&key.dev) != hipSuccess) return TM_ERR_HIP;
    const int lvl = log_level();
    std::unique_lock<std::mutex> lk(*c->gmu);
    GraphEntry* hit = nullptr;
    for (GraphEntry& e : *c->graphs) {
        if (e.dev == key.dev && e.kind == key.kind && e.batch == key.batch && e.heads == key.heads &&
            e.n_tokens == key.n_tokens && e.dtype == key.dtype && e.opt == key.opt && e.extra == key.extra &&
            memcmp(e.p, key.p, sizeof(key.p)) == 0) {
            hit = &e;
            break;
        }
    }
    if (!hit) {
        if (c->graphs->size() >= MAX_GRAPHS) {
            size_t lru = 0;
            for (size_t i = 1; i < c->graphs->size(); ++i)
                if ((*c->graphs)[i].last < (*c->graphs)[lru].last) lru = i;
            if ((*c->graphs)[lru].exec) (void)hipGraphExecDestroy((*c->graphs)[lru].exec);
            c->graphs->erase(c->graphs->begin() + lru);
        }
        key.seen = 1;
        key.exec = nullptr;
        key.last = ++c->stamp;
        c->graphs->push_back(key);
        lk.unlock();
        if (lvl >= 1) log_call(c, key);
        g_log_plan = lvl >= 1;
        tm_status rc = launch(st);
        g_log_plan = false;
        return rc;
    }
    hit->last = ++c->stamp;
    if (lvl >= 2)
        fprintf(stderr, "[tm] %s call %s (batch %d, heads %d, n_tokens %d)\n", hit->exec ? "replay" : "capture",
                kind_name(key.kind), key.batch, key.heads, key.n_tokens);
    if (!hit->exec) {
        hipStream_t cs = nullptr;
        for (auto& pr : *c->capture_streams)
            if (pr.first == key.dev) cs = pr.second;
        if (!cs) {
            if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return TM_ERR_HIP;
            c->capture_streams->push_back({key.dev, cs});
        }
        hipGraph_t graph = nullptr;
        if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) return TM_ERR_HIP;
        tm_status rc = launch(cs);
        hipError_t e = hipStreamEndCapture(cs, &graph);
        if (rc != TM_OK || e != hipSuccess) {
            if (graph) (void)hipGraphDestroy(graph);
            return rc != TM_OK ? rc : TM_ERR_HIP;
        }
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess) return TM_ERR_HIP;
        hit->exec = exec;
    }
    return hipGraphLaunch(hit->exec, st) == hipSuccess ? TM_OK : TM_ERR_HIP;
}

GraphEntry make_key(int kind, int batch, int heads, int n_tokens, int dtype,
                    std::initializer_list<const void*> ptrs) {
    GraphEntry k;
    memset(&k, 0, sizeof(k));
    k.kind = kind;
    k.batch = batch;
    k.heads = heads;
    k.n_tokens = n_tokens;
    k.dtype = dtype;
    k.opt = (g_w1_split ? 1 : 0) | (g_store_groups ? 2 : 0);   // the switches that change the launches
    int i = 0;
    for (const void* p : ptrs) k.p[i++] = p;
    return k;
}

// Layer / tile fields shared by the update and the bf16-copy kernels.
UpdArgs base_upd(const tm_ctx* c, char* state, long ns) {
    UpdArgs u;
    memset(&u, 0, sizeof(u));
    StateLayout sl = state_layout(c, ns);
    u.L = c->L;
    u.b = c->chunk;
    for (int l = 0; l < c->L; ++l) {
        u.din[l] = c->din[l];
        u.dout[l] = c->dout[l];
        u.off[l] = c->off[l];
        u.tj[l] = c->tj[l];
    }
    for (int l = 0; l <= c->L; ++l) u.tbase[l] = c->tbase[l];
    u.P = c->P;
    u.M = reinterpret_cast<float*>(state + sl.M);
    u.S = reinterpret_cast<float*>(state + sl.S);
    u.Wt = state + sl.Wt;
    u.flag = &reinterpret_cast<StateHeader*>(state)->nonfinite;
    return u;
}

tm_status check_common(const tm_ctx* c, const void* state, int batch, int heads, int n_tokens,
                       tm_dtype dtype, const void* ws) {
    if (!c || !state || !ws) return TM_ERR_INVALID;
    if (batch <= 0 || heads <= 0 || n_tokens < 0) return TM_ERR_INVALID;
    if ((long)batch * heads > 65535) return TM_ERR_INVALID;   // grid.y / grid.z limit
    if (dtype != TM_F32 && dtype != TM_BF16) return TM_ERR_DTYPE;
    if (!aligned(state, 256) || !aligned(ws, 256)) return TM_ERR_INVALID;
    return TM_OK;
}

bool tok_ok(const void* p) { return p && aligned(p, 16); }
bool gate_ok(const void* p) { return p && aligned(p, 4); }

// Forward of `rows` rows (q rows first, then k rows) of one chunk step, or of
// a retrieve pass, through every layer at the current weights.
struct FwdRows {
    int nq, nk;        // q rows, k rows
    const void* q;     // q token array (input layout) or nullptr
    int tq;            // first q token
    const void* k;
    int tk;
    const void* v;
    float* y;
    const float* m1;   // fp32 path: layer 1's master if not the state's (stream stride m1_ss)
    long m1_ss;
};

tm_status run_forward_layers(const tm_ctx* c, char* state, long ns, const WsLayout& w, char* ws,
                             const TokLayout& tl, const FwdRows& fr, bool f32, bool retrieve,
                             hipStream_t st, int l_begin = 0) {
    StateLayout sl = state_layout(c, ns);
    const int rows = fr.nq + fr.nk;
    if (rows == 0) return TM_OK;
    for (int l = l_begin; l < c->L; ++l) {
        GemmArgs g;
        memset(&g, 0, sizeof(g));
        g.nrows = rows;
        g.N = c->dout[l];
        g.K = c->din[l];
        g.tl = tl;
        g.n0 = fr.nq;
        if (l == 0) {
            g.amode = A_TOKENS;
            g.a0 = fr.q;
            g.at0 = fr.tq;
            g.a1 = fr.k;
            g.at1 = fr.tk;
        } else {
            g.amode = A_PACKED;
            if (retrieve) {
                g.a0 = ws + w.ret[(l - 1) & 1];
                g.a_ss = w.ret_ss;
            } else {
                g.a0 = ws + w.act[l - 1];
                g.a_ss = w.act_ss;
            }
        }
        if (f32) {
            // fp32 operands straight from the fp32 master: row-major [din][dout],
            // layers 0 and 1 in accumulator order
            g.bmode = l == 0 ? B_CFRAG : l == 1 ? B_CF1 : B_STRIDED;
            g.b = state + sl.M + (size_t)c->off[l] * 4;
            g.b_ss = c->P;
            g.b_ld = c->dout[l];
            if (l == 1 && fr.m1) {
                g.b = fr.m1;
                g.b_ss = fr.m1_ss;
            }
        } else {
            g.bmode = B_PACKED;
            g.b = state + sl.Wt + (size_t)c->off[l] * 2;
            g.b_ss = c->P;
        }
        if (l + 1 < c->L) {
            g.epi = EPI_HIDDEN;
            if (retrieve) {
                g.act = ws + w.ret[l & 1];
                g.act_ss = w.ret_ss;
                // retrieve rows are all q rows: no SiLU' is stored
                g.dsl = nullptr;
            } else {
                g.act = ws + w.act[l];
                g.act_ss = w.act_ss;
                g.dsl = reinterpret_cast<float*>(ws + w.dsl[l]);
                g.dsl_ss = w.dsl_ss;
                g.dsl_ld = c->hidden;
                g.ht = ws + w.ht[l];
                g.tr_ss = w.ht_ss;
                g.bp = w.bp;
            }
        } else {
            g.epi = EPI_OUT;
            g.y = fr.y;
            g.yt0 = fr.tq;
            g.v = fr.v;
            g.vt0 = fr.tk;
            if (!retrieve && fr.nk > 0) {
                if (l >= 1) {
                    g.dlp = ws + w.dlp[l];
                    g.dlp_ss = w.dlp_ss[l];
                }
                g.dct = ws + w.dct[l];
                g.ddt = ws + w.ddt[l];
                g.tr_ss = w.dt_ss[l];
                g.bp = w.bp;
                g.cc = reinterpret_cast<const float*>(ws + w.cc) + fr.tk;
                g.dc = reinterpret_cast<const float*>(ws + w.dc) + fr.tk;
                g.coef_ss = w.coef_ss;
            }
        }
        // (a retrieve pass of many rows: a plain tiled product, no split K)
        const bool big = retrieve && !f32 && rows >= RET_TILED_ROWS;
        g.xcd_streams = xcd_streams_on() && ns % 8 == 0 && ns >= 8 ? 1 : 0;
        hipError_t e = timed(K_FWD, st, [&] {
            return big ? launch_rows(g, (int)ns, st) : launch_fwd(g, (int)ns, f32 ? 1 : 0, st);
        });
        if (e != hipSuccess) return TM_ERR_HIP;
    }
    return TM_OK;
}

// Backward of chunk ci through layers L-1 .. 2: Delta_{l-1} from Delta_l
// (the first layer's Delta is formed inside the next step kernel).
tm_status run_backward(const tm_ctx* c, char* state, long ns, const WsLayout& w, char* ws,
                       const TokLayout& tl, int ci, bool f32, hipStream_t st) {
    const int b = c->chunk;
    StateLayout sl = state_layout(c, ns);
    for (int l = c->L - 1; l >= 2; --l) {
        GemmArgs g;
        memset(&g, 0, sizeof(g));
        g.nrows = b;
        g.N = c->din[l];
        g.K = c->dout[l];
        g.tl = tl;
        g.amode = A_PACKED;
        g.a0 = ws + w.dlp[l];
        g.a_ss = w.dlp_ss[l];
        g.n0 = 0;   // key rows only
        // B[k][n] = W_l[n][k]: row n of the fp32 master, contiguous in K
        g.bmode = B_ROWS;
        g.b = state + sl.M + (size_t)c->off[l] * 4;
        g.b_ss = c->P;
        g.b_ld = c->dout[l];
        g.epi = EPI_BWD;
        g.dsl = reinterpret_cast<float*>(ws + w.dsl[l - 1]);
        g.dsl_ss = w.dsl_ss;
        g.dsl_ld = c->hidden;
        g.dlp = ws + w.dlp[l - 1];
        g.dlp_ss = w.dlp_ss[l - 1];
        g.dct = ws + w.dct[l - 1];
        g.ddt = ws + w.ddt[l - 1];
        g.tr_ss = w.dt_ss[l - 1];
        g.bp = w.bp;
        g.cc = reinterpret_cast<const float*>(ws + w.cc) + ci * b;
        g.dc = reinterpret_cast<const float*>(ws + w.dc) + ci * b;
        g.coef_ss = w.coef_ss;
        g.xcd_streams = xcd_streams_on() && ns % 8 == 0 && ns >= 8 ? 1 : 0;
        hipError_t e = timed(K_BWD, st, [&] { return launch_bwd(g, (int)ns, f32 ? 1 : 0, st); });
        if (e != hipSuccess) return TM_ERR_HIP;
    }
    return TM_OK;
}

// Per-token read, once per call: C of layer 0 and pm_t, ps_t for every
// chunk (they depend on the inputs only).
tm_status run_token_scores(const tm_ctx* c, long ns, const WsLayout& w, char* ws, const float* theta,
                           const float* eta, const float* alpha, int n_tokens, int heads, bool f32,
                           hipStream_t st) {
    R3Args r;
    memset(&r, 0, sizeof(r));
    r.b = c->chunk;
    r.bp = w.bp;
    r.K = c->dim;
    r.N = c->dout[0];
    r.a = ws + w.xq;
    r.a_ss = w.x_ss;
    r.a_cs = w.xc;
    r.hk = ws + w.xk;
    r.hk_ss = w.x_ss;
    r.hk_cs = w.xc;
    r.sco = reinterpret_cast<float*>(ws + w.r3c);
    r.sc_ss = w.r3c_ss;
    r.sc_cs = w.r3c_cs;
    r.theta = theta;
    r.eta = eta;
    r.alpha = alpha;
    r.gl = TokLayout{n_tokens, heads, 1};
    r.pq = reinterpret_cast<float*>(ws + w.r3p);
    r.pq_ss = w.r3p_ss;
    r.pq_cs = 2 * c->chunk;
    if (timed(K_R3, st, [&] { return launch_r3_score(r, (int)ns, w.C, f32 ? 1 : 0, st); }) != hipSuccess)
        return TM_ERR_HIP;
    return TM_OK;
}

// Per-token read of chunk ci (every query through the memory as its own
// token's write left it), between the chunk's forward / backward and the
// step that writes it, so the state still holds the chunk-start weights: one
// launch per layer (layer 0 forms its Delta in place and reads its C from
// the call's score launch; the layers past it form their C in place); the
// last layer writes y.
tm_status run_token_read(const tm_ctx* c, char* state, long ns, const WsLayout& w, char* ws,
                         const TokLayout& tl, int ci, const void* v, const float* theta, const float* eta,
                         const float* alpha, float* y, int n_tokens, int heads, const float* m1, long m1_ss,
                         bool f32, hipStream_t st) {
    const int b = c->chunk;
    const size_t esz = f32 ? 4 : 2;
    StateLayout sl = state_layout(c, ns);
    const float* Mst = reinterpret_cast<const float*>(state + sl.M);
    const float* Sst = reinterpret_cast<const float*>(state + sl.S);
    float* cbuf = reinterpret_cast<float*>(ws + w.r3c);
    for (int l = 0; l < c->L; ++l) {
        R3Args r;
        memset(&r, 0, sizeof(r));
        r.b = b;
        r.bp = w.bp;
        r.K = c->din[l];
        r.N = c->dout[l];
        r.tl = tl;
        if (l == 0) {
            r.a = ws + w.xq + (size_t)ci * w.xc * esz;
            r.a_ss = w.x_ss;
            r.hk = ws + w.xk + (size_t)ci * w.xc * esz;
            r.hk_ss = w.x_ss;
            r.sc = cbuf + (size_t)ci * w.r3c_cs;
        } else {
            // the keys' rows of the store's forward (no query rows: keys from
            // row 0); the layer forms its C in place from them and the gates
            r.a = ws + w.r3x[(l - 1) & 1];
            r.a_ss = w.r3x_ss;
            r.hk = ws + w.act[l - 1];
            r.hk_ss = w.act_ss;
            r.theta = theta;
            r.eta = eta;
            r.alpha = alpha;
            r.gl = TokLayout{n_tokens, heads, 1};
            r.g0 = ci * b;
        }
        r.sc_ss = w.r3c_ss;
        r.pq = reinterpret_cast<float*>(ws + w.r3p) + (size_t)ci * 2 * b;
        r.pq_ss = w.r3p_ss;
        r.bl = l == 0 ? BL_CF0 : l == 1 ? BL_CF1 : BL_ROW;
        // (layer 1's M where this step's update wrote it)
        r.M = l == 1 ? m1 : Mst + c->off[l];
        r.m_ss = l == 1 ? m1_ss : c->P;
        r.S = Sst + c->off[l];
        r.s_ss = c->P;
        if (l > 0) {
            r.dk = R3D_BUF;
            r.dl = ws + w.dlp[l];
            r.dl_ss = w.dlp_ss[l];
        } else if (c->L == 1) {
            r.dk = R3D_OUT;
            r.v = v;
            r.vt0 = ci * b;
        } else {
            r.dk = R3D_BWD;
            r.d1 = ws + w.dlp[1];
            r.d1_ss = w.dlp_ss[1];
            r.K1 = c->dout[1];
            r.w1 = m1;
            r.w1_ss = m1_ss;
            r.dsl = reinterpret_cast<const float*>(ws + w.dsl[0]);
            r.dsl_ss = w.dsl_ss;
            r.dsl_ld = c->hidden;
        }
        if (l + 1 < c->L) {
            r.out = ws + w.r3x[l & 1];
            r.out_ss = w.r3x_ss;
        } else {
            r.y = y;
            r.yt0 = ci * b;
        }
        if (timed(K_R3, st, [&] { return launch_r3_layer(r, (int)ns, f32 ? 1 : 0, st); }) != hipSuccess)
            return TM_ERR_HIP;
    }
    return TM_OK;
}

// The context's extra stream `idx` (0, 1, ...) on the current device for
// the calling host thread (default priority), with its fork and join
// events; created on first use.  (Per thread: two threads that recorded
// one fork event in turn could let one's extra stream start on the other's
// point.)
tm_status side_stream(const tm_ctx* c, tm_ctx::Side* out, int idx = 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TM_ERR_HIP;
    tm_ctx* cm = const_cast<tm_ctx*>(c);
    // (a lock of its own: the graph cache's lock is held while a call is
    // captured)
    static std::mutex side_mu;
    std::lock_guard<std::mutex> lk(side_mu);
    const std::thread::id tid = std::this_thread::get_id();
    for (auto& sd : *cm->sides)
        if (sd.dev == dev && sd.idx == idx && sd.tid == tid) {
            *out = sd;
            return TM_OK;
        }
    tm_ctx::Side sd{dev, nullptr, nullptr, nullptr, idx, tid};
    if (hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) != hipSuccess) return TM_ERR_HIP;
    if (hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&sd.join, hipEventDisableTiming) != hipSuccess) {
        if (sd.fork) (void)hipEventDestroy(sd.fork);
        (void)hipStreamDestroy(sd.s);
        return TM_ERR_HIP;
    }
    cm->sides->push_back(sd);
    *out = sd;
    return TM_OK;
}

// The call's chunk loop.  Step c (0..C) is one launch of the step kernel:
// chunk c-1's update of every layer (the first layer's Delta formed in
// place) and chunk c's first-layer forward of [queries of chunk c-1; keys of
// chunk c]; then the forward of layers 1.. for the same rows (their last
// layer writes y for the queries and Delta for the keys) and, for depth >= 3,
// the backward down to layer 1.  Step C only finishes chunk C-1.
tm_status run_chain(const tm_ctx* c, void* state_v, const void* k, const void* v, const void* q,
                    const float* theta, const float* eta, const float* alpha, float* y, int batch,
                    int heads, int n_tokens, tm_dtype dtype, void* ws_v, hipStream_t st, int read,
                    bool add_position) {
    char* state = static_cast<char*>(state_v);
    char* ws = static_cast<char*>(ws_v);
    const long ns = (long)batch * heads;
    const int b = c->chunk, C = n_tokens / b;
    const bool f32 = dtype == TM_F32;
    const size_t esz = f32 ? 4 : 2;
    WsLayout w = ws_layout(c, ns, n_tokens);
    TokLayout tl{n_tokens, heads, c->dim};

    ScanArgs sa;
    memset(&sa, 0, sizeof(sa));
    sa.theta = theta;
    sa.eta = eta;
    sa.alpha = alpha;
    sa.tl = TokLayout{n_tokens, heads, 1};
    sa.b = b;
    sa.C = C;
    sa.ns = (int)ns;
    sa.cc = reinterpret_cast<float*>(ws + w.cc);
    sa.dc = reinterpret_cast<float*>(ws + w.dc);
    sa.coef_ss = w.coef_ss;
    sa.cs = reinterpret_cast<float*>(ws + w.cs);
    sa.cs_ss = w.cs_ss;
    sa.position = add_position ? &reinterpret_cast<StateHeader*>(state)->position : nullptr;
    sa.add = n_tokens;
    sa.k = k;
    sa.q = q;
    sa.ktl = tl;
    sa.kt = ws + w.kt;
    sa.xk = ws + w.xk;
    sa.xq = ws + w.xq;
    sa.xc = w.xc;
    sa.bp = w.bp;
    sa.kt_f32 = f32 ? 1 : 0;
    if (timed(K_SCAN, st, [&] { return launch_scan(sa, st); }) != hipSuccess) return TM_ERR_HIP;
    if (read == TM_READ_PER_TOKEN && q) {
        tm_status rc = run_token_scores(c, ns, w, ws, theta, eta, alpha, n_tokens, heads, f32, st);
        if (rc != TM_OK) return rc;
    }

    FirstArgs a;
    memset(&a, 0, sizeof(a));
    a.u = base_upd(c, state, ns);
    a.u.bp = w.bp;
    a.u.cs = reinterpret_cast<const float*>(ws + w.cs);
    a.u.cs_ss = w.cs_ss;
    for (int l = 2; l < c->L; ++l) {
        a.u.at[l] = ws + w.ht[l - 1];
        a.u.at_ss[l] = w.ht_ss;
    }
    if (c->L >= 2) a.u.at_ss[1] = w.ht_ss;
    for (int l = 0; l < c->L; ++l) {
        a.u.dct[l] = ws + w.dct[l];
        a.u.ddt[l] = ws + w.ddt[l];
        a.u.dt_ss[l] = w.dt_ss[l];
    }
    a.dim = c->dim;
    a.h1 = c->dout[0];
    a.nb1 = (a.h1 + JW - 1) / JW;
    a.kt_ss = w.kt_ss;
    a.dlt2_ss = c->L >= 2 ? w.dlp_ss[1] : 0;
    a.dlt2 = c->L >= 2 ? (const void*)(ws + w.dlp[1]) : nullptr;
    a.dsl1 = c->L >= 2 ? reinterpret_cast<float*>(ws + w.dsl[0]) : nullptr;
    a.dsl1_ss = w.dsl_ss;
    a.coef_ss = w.coef_ss;
    a.x_ss = w.x_ss;
    a.tl = tl;
    a.act = c->L >= 2 ? ws + w.act[0] : nullptr;
    a.act_ss = w.act_ss;
    a.ht_ss = w.ht_ss;
    a.y = y;
    a.v = v;
    a.dct1 = ws + w.dct[0];
    a.ddt1 = ws + w.ddt[0];
    a.dt1_ss = w.dt_ss[0];
    // layers 0 and 1 are updated by the first-layer blocks; layers 2.. by
    // update tiles in the same launch
    const int tile2 = c->tbase[c->L > 2 ? 2 : c->L];
    const int ntile_rest = c->tbase[c->L] - tile2;
    // depth 2: W_1's update in workgroups of its own when they add no round
    // of workgroups to the launch (one workgroup per compute unit: the
    // first-layer blocks are register-bound).  Those steps read M_1 from one buffer
    // and write the other; the buffers alternate so that the call's last
    // update writes the state's (with an odd number of updates, the first
    // one runs in place in the first-layer blocks).
    float* m1_state = c->L >= 2 ? a.u.M + c->off[1] : nullptr;
    float* m1_ws = c->L == 2 ? reinterpret_cast<float*>(ws + w.m1x) : nullptr;
    const long p1 = c->L >= 2 ? (long)c->din[1] * c->dout[1] : 0;
    int nw1 = 0;
    if (c->L == 2 && g_w1_split && !f32) {
        // a multiple of 8 workgroups, W1_JPW row blocks each per XCD residue
        const int n1 = 8 * (((a.nb1 + 7) / 8 + W1_JPW - 1) / W1_JPW);
        int cus = 0;
        if (compute_units(&cus) != hipSuccess) return TM_ERR_HIP;
        const long nsa = g_sview.ns_total > 0 ? g_sview.ns_total : ns;   // every chain's streams
        if ((nsa * (a.nb1 + n1) + cus - 1) / cus <= (nsa * a.nb1 + cus - 1) / cus) nw1 = n1;
    }

    if (g_log_plan)
        fprintf(stderr,
                "[tm] plan: %d chunks of %d over %ld streams; 1 scan launch%s, then %d steps of 1 first-layer "
                "launch (%d blocks/stream, %d W_1 blocks/stream, %d update tiles of layers 2..) + %d product "
                "launches + %d backward launches%s; workspace %zu bytes\n",
                C, b, ns, read == TM_READ_PER_TOKEN && q ? " + 1 score launch" : "", C + 1, a.nb1, nw1, ntile_rest,
                c->L - 1, c->L >= 3 ? c->L - 2 : 0, read == TM_READ_PER_TOKEN && q ? " + L read launches" : "",
                w.total);

    for (int ci = 0; ci <= C; ++ci) {
        // queries: chunk ci-1's through the memory after its write (rows of
        // step ci), or chunk ci's through the memory before its write (the
        // same rows as chunk ci's keys)
        const int cq = read == TM_READ_BEFORE_WRITE ? ci : ci - 1;
        // (per-token: the queries go through run_token_read, not these rows)
        const bool has_q = q && read != TM_READ_PER_TOKEN && cq >= 0 && cq < C;
        a.do_update = ci >= 1;
        a.last_update = ci == C;
        a.nq = has_q ? b : 0;
        a.nk = ci < C ? b : 0;
        a.do_fwd = a.nq + a.nk > 0;
        a.chunk_prev = ci - 1;
        a.u.chunk = ci - 1;
        a.tq0 = cq * b;
        a.tk0 = ci * b;
        // steps that skip a part still get valid addresses for its operands
        // (the step kernel loads them unconditionally and drops the values)
        const int cprev = ci >= 1 ? ci - 1 : 0;
        a.xq = has_q ? ws + w.xq + (size_t)cq * w.xc * esz : nullptr;
        a.xk = ws + w.xk + (size_t)(ci < C ? ci : 0) * w.xc * esz;
        a.kt_prev = ws + w.kt + (size_t)cprev * c->dim * w.bp * esz;
        a.cc_prev = reinterpret_cast<const float*>(ws + w.cc) + cprev * b;
        a.dc_prev = reinterpret_cast<const float*>(ws + w.dc) + cprev * b;
        a.cc_cur = reinterpret_cast<const float*>(ws + w.cc) + (ci < C ? ci : 0) * b;
        a.dc_cur = reinterpret_cast<const float*>(ws + w.dc) + (ci < C ? ci : 0) * b;
        if (c->L >= 2) {
            a.u.at[1] = ws + w.ht1[(ci - 1) & 1];
            a.ht1 = ws + w.ht1[ci & 1];
        }
        if (!a.do_update && !a.do_fwd) continue;
        // one launch: the first-layer blocks plus chunk c-1's update tiles of
        // the other layers (independent of each other)
        a.upd_tile0 = tile2;
        a.upd_ntiles = a.do_update ? ntile_rest : 0;
        // many streams, no workgroups of other roles: each stream's blocks on
        // one XCD (its shared operands fetched into one L2)
        a.xcd_streams = xcd_streams_on() && ns % 8 == 0 && ns >= 8 && a.upd_ntiles == 0 ? 1 : 0;
        a.m1_rd = m1_state;
        a.m1_wr = m1_state;
        a.m1_rd_ss = a.m1_wr_ss = c->P;
        a.nw1 = 0;
        if (nw1 > 0 && a.do_update && (ci >= 2 || C % 2 == 0)) {
            a.xcd_streams = 0;
            const bool to_ws = (C - ci + 1) % 2 == 0;   // updates left, this one included
            a.nw1 = nw1;
            a.m1_rd = to_ws ? m1_state : m1_ws;
            a.m1_rd_ss = to_ws ? c->P : p1;
            a.m1_wr = to_ws ? m1_ws : m1_state;
            a.m1_wr_ss = to_ws ? p1 : c->P;
        }
        if (timed(K_FIRST, st, [&] { return launch_first(a, (int)ns, f32 ? 1 : 0, st); }) != hipSuccess)
            return TM_ERR_HIP;
        if (a.do_fwd && c->L >= 2) {
            FwdRows fr{};
            fr.nq = a.nq;
            fr.q = q;
            fr.tq = a.tq0;
            fr.nk = a.nk;
            fr.k = k;
            fr.tk = a.tk0;
            fr.v = v;
            fr.y = y;
            fr.m1 = a.m1_wr;   // M_1 after this step's update (wherever it was written)
            fr.m1_ss = a.m1_wr_ss;
            tm_status rc = run_forward_layers(c, state, ns, w, ws, tl, fr, f32, false, st, 1);
            if (rc != TM_OK) return rc;
        }
        if (ci < C && c->L >= 3) {
            tm_status rc = run_backward(c, state, ns, w, ws, tl, ci, f32, st);
            if (rc != TM_OK) return rc;
        }
        if (ci < C && read == TM_READ_PER_TOKEN && q) {
            tm_status rc = run_token_read(c, state, ns, w, ws, tl, ci, v, theta, eta, alpha, y, n_tokens, heads,
                                          a.m1_wr, a.m1_wr_ss, f32, st);
            if (rc != TM_OK) return rc;
        }
    }
    return TM_OK;
}

// Batch groups of a store: the call's batches split into G groups whose
// chunk chains run on G streams at once (the caller's and the context's
// extra streams), so that one chain's kernels fill the idle compute units
// of another's launch tails and gaps.  The chains are independent (each
// stream's recurrence is its own) and run the launches of one chain over
// fewer streams, so the results are bitwise those of one chain.
// Two chains when the call has at least 16 streams and an even batch (with
// fewer streams each launch of one chain is short and latency-bound, and
// running two side by side only adds contention); measured on the 8 x 8-head
// dim-128 memory: +9% tokens/s with two chains, -5% with four.
// TM_STORE_GROUPS=1, 2, 4 or 8 overrides the choice (for comparison).
constexpr int MAX_GROUPS = 8;
int store_groups(int batch, int heads) {
    static const int env = [] {
        const char* e = getenv("TM_STORE_GROUPS");
        return e && (e[0] == '1' || e[0] == '2' || e[0] == '4' || e[0] == '8') && e[1] == 0 ? e[0] - '0' : -1;
    }();
    if (!g_store_groups) return 1;
    const int G = env > 0 ? env : ((long)batch * heads >= 16 ? 2 : 1);
    return batch % G == 0 ? G : 1;
}

// Sets the state view for one group and clears it on every return path.
struct ViewGuard {
    ViewGuard(long s0, long total) { g_sview = StateView{s0, total}; }
    ~ViewGuard() { g_sview = StateView{0, 0}; }
};

size_t store_ws_bytes(const tm_ctx* c, int batch, int heads, int n_tokens) {
    size_t need = ws_layout(c, (long)batch * heads, n_tokens).total;
    for (int G = 2; G <= MAX_GROUPS; G *= 2)
        if (batch % G == 0)
            need = std::max(need, G * al256(ws_layout(c, (long)(batch / G) * heads, n_tokens).total));
    return need;
}

// `groups` = 0: the choice above; 1: one chain (no extra stream).
tm_status run_store(const tm_ctx* c, void* state, const void* k, const void* v, const void* q,
                    const float* theta, const float* eta, const float* alpha, float* y, int batch,
                    int heads, int n_tokens, tm_dtype dtype, void* ws_v, hipStream_t st,
                    int read = TM_READ_AFTER_WRITE, int groups = 0) {
    const int G = groups == 1 ? 1 : store_groups(batch, heads);
    if (G == 1) return run_chain(c, state, k, v, q, theta, eta, alpha, y, batch, heads, n_tokens, dtype, ws_v, st,
                                 read, true);
    tm_ctx::Side side[MAX_GROUPS - 1];
    for (int g = 1; g < G; ++g)
        if (side_stream(c, &side[g - 1], g - 1) != TM_OK) return TM_ERR_HIP;
    // the extra streams forked so far are joined back on every path (a
    // capture must end with every stream it reached joined)
    int forked = 1;
    auto join = [&]() {
        bool ok = true;
        for (int g = 1; g < forked; ++g)
            ok = hipEventRecord(side[g - 1].join, side[g - 1].s) == hipSuccess &&
                 hipStreamWaitEvent(st, side[g - 1].join, 0) == hipSuccess && ok;
        return ok;
    };
    for (int g = 1; g < G; ++g) {
        if (hipEventRecord(side[g - 1].fork, st) != hipSuccess) break;
        if (hipStreamWaitEvent(side[g - 1].s, side[g - 1].fork, 0) != hipSuccess) break;
        forked = g + 1;
    }
    if (forked < G) {
        (void)join();
        return TM_ERR_HIP;
    }
    const int bg = batch / G;
    const size_t esz = dtype == TM_F32 ? 4 : 2;
    const size_t tok = (size_t)n_tokens * heads * c->dim, gate = (size_t)n_tokens * heads;
    const size_t wsg = al256(ws_layout(c, (long)bg * heads, n_tokens).total);
    tm_status rc = TM_OK;
    for (int g = 0; g < G && rc == TM_OK; ++g) {
        const size_t b0 = (size_t)g * bg;
        auto off = [&](const void* p, size_t n) -> const void* {
            return p ? static_cast<const char*>(p) + b0 * n : nullptr;
        };
        ViewGuard view((long)b0 * heads, (long)batch * heads);
        rc = run_chain(c, state, off(k, tok * esz), off(v, tok * esz), off(q, tok * esz),
                       static_cast<const float*>(off(theta, gate * 4)), static_cast<const float*>(off(eta, gate * 4)),
                       static_cast<const float*>(off(alpha, gate * 4)),
                       y ? y + b0 * tok : nullptr, bg, heads, n_tokens, dtype, static_cast<char*>(ws_v) + g * wsg,
                       g == 0 ? st : side[g - 1].s, read, g == 0);
    }
    const bool joined = join();
    if (rc != TM_OK) return rc;
    return joined ? TM_OK : TM_ERR_HIP;
}

// ---- the backward through the store (tm_backward) ----
// Workspace: every chunk-start state (canonical fp32, [chunk][stream][2P],
// C + 1 of them), the chunks' coefficients, each (stream, chunk)'s key-row
// record from the recompute, the reverse sweep's per-stream scratch, and
// the partial sums behind the gates' gradients.  Sizes in 4-byte elements.
struct BwdLayout {
    size_t tape, cc, dc, cs, key, scr, pgp, pad, acc, acc2, total;
    long tape_cs;               // elements per chunk slot (ns * 2P)
    long rec;                   // elements of one (stream, chunk) key record
    long hk[MAXL], zk[MAXL], dk[MAXL], gk[MAXL];   // offsets inside a record
    long scr_ss;                // per-stream elements of the sweep's scratch
    long hq[MAXL], zq[MAXL], dq[MAXL], db[MAXL], hb[MAXL], u[MAXL], zb[MAXL];
    int ngp, nad, gpbase[MAXL], adbase[MAXL];
    int C;
};

BwdLayout bwd_layout(const tm_ctx* c, long ns, long T) {
    BwdLayout w;
    memset(&w, 0, sizeof(w));
    const long b = c->chunk, C = T / b;
    w.C = (int)C;
    size_t o = 0;
    w.tape_cs = ns * 2 * c->P;
    w.tape = o; o += al256((size_t)(C + 1) * w.tape_cs * 4);
    w.cc = o; o += al256((size_t)ns * T * 4);
    w.dc = o; o += al256((size_t)ns * T * 4);
    w.cs = o; o += al256((size_t)ns * C * 16);
    // key record: h_l (l >= 1; h_0 is the keys themselves), z_l, Delta_l,
    // and g_l = Delta_l W_l^T (l >= 1), each [b][width] row-major
    long r = 0;
    for (int l = 0; l < c->L; ++l) {
        if (l >= 1) { w.hk[l] = r; r += b * c->din[l]; }
        w.zk[l] = r; r += b * c->dout[l];
        w.dk[l] = r; r += b * c->dout[l];
        if (l >= 1) { w.gk[l] = r; r += b * c->din[l]; }
    }
    w.rec = r;
    w.key = o; o += al256((size_t)ns * C * r * 4);
    // sweep scratch per stream: the queries' h, z and backpropagated delta,
    // and the key rows' Deltabar, hbar (from the surprise's adjoint), u and zbar
    r = 0;
    for (int l = 0; l < c->L; ++l) {
        if (l >= 1) { w.hq[l] = r; r += b * c->din[l]; }
        if (l + 1 < c->L) { w.zq[l] = r; r += b * c->dout[l]; w.dq[l] = r; r += b * c->dout[l]; }
        w.db[l] = r; r += b * c->dout[l];
        w.hb[l] = r; r += b * c->din[l];
        if (l >= 1) { w.u[l] = r; r += b * c->din[l]; }
        w.zb[l] = r; r += b * c->dout[l];
    }
    w.scr_ss = r;
    w.scr = o; o += al256((size_t)ns * r * 4);
    for (int l = 0; l < c->L; ++l) {
        w.gpbase[l] = w.ngp;
        w.ngp += (c->dout[l] + 63) / 64;
        w.adbase[l] = w.nad;
        w.nad += ((c->din[l] + 63) / 64) * ((c->dout[l] + 63) / 64);
    }
    w.pgp = o; o += al256((size_t)ns * C * w.ngp * 128 * 4);
    w.pad = o; o += al256((size_t)ns * C * w.nad * 3 * 4);
    // split-K partial tiles of the largest split product (b rows by a layer
    // width, either direction; the queries' weight gradient, K = b)
    long acc = 0;
    for (int l = 0; l < c->L; ++l) {
        const int di = c->din[l], dn = c->dout[l];
        const int shapes[3][3] = {{(int)b, dn, di}, {(int)b, di, dn}, {di, dn, (int)b}};
        for (const auto& sh : shapes) {
            const long f = bgemm_acc_floats(sh[0], sh[1], (int)ns, bgemm_splitk(sh[0], sh[1], sh[2], 0, BE_STORE, (int)ns));
            acc = f > acc ? f : acc;
        }
    }
    w.acc = o; o += al256((size_t)acc * 4);
    w.acc2 = o; o += al256((size_t)acc * 4);   // the second stream's
    w.total = o > 0 ? o : 256;
    return w;
}

BMat rowm(const void* p, long ss, long ld) {
    BMat m;
    memset(&m, 0, sizeof(m));
    m.p = p;
    m.ss = ss;
    m.ld = ld;
    return m;
}
BMat tokm(const void* p, int t0, int bf) {
    BMat m;
    memset(&m, 0, sizeof(m));
    m.p = p;
    m.tok = 1;
    m.t0 = t0;
    m.bf = bf;
    return m;
}

tm_status run_bwd(const tm_ctx* c, const void* state, const void* k, const void* v, const void* q,
                  const float* theta, const float* eta, const float* alpha, const float* dy, float* dst,
                  float* dk, float* dv, float* dq, float* dth, float* det, float* dal, int batch, int heads,
                  int T, tm_dtype dtype, int read, void* ws_v, hipStream_t st) {
    const long ns = (long)batch * heads, P = c->P;
    const int b = c->chunk, C = T / b, L = c->L;
    const int bf = dtype == TM_BF16 ? 1 : 0;
    BwdLayout w = bwd_layout(c, ns, T);
    char* ws = static_cast<char*>(ws_v);
    float* tape = reinterpret_cast<float*>(ws + w.tape);
    float* cc = reinterpret_cast<float*>(ws + w.cc);
    float* dc = reinterpret_cast<float*>(ws + w.dc);
    float* cs = reinterpret_cast<float*>(ws + w.cs);
    float* key = reinterpret_cast<float*>(ws + w.key);
    float* scr = reinterpret_cast<float*>(ws + w.scr);
    float* pgp = reinterpret_cast<float*>(ws + w.pgp);
    float* pad = reinterpret_cast<float*>(ws + w.pad);
    const TokLayout tl{T, heads, c->dim};
    const TokLayout gl{T, heads, 1};
    if (g_log_plan)
        fprintf(stderr,
                "[tm] backward plan: %d chunks of %d over %ld streams; recompute 3L-1 = %d launches per chunk, "
                "reverse sweep about 9L = %d per chunk; workspace %zu bytes\n",
                C, b, ns, 3 * L - 1, 9 * L, w.total * 1);

    float* accbuf = reinterpret_cast<float*>(ws + w.acc);
    float* accbuf2 = reinterpret_cast<float*>(ws + w.acc2);
    // the second stream (default priority) and its fork / join events; under
    // graph capture the fork joins it to the capture and the products on
    // it become parallel branches of the graph
    tm_ctx::Side side{-1, nullptr, nullptr, nullptr};
    if (side_stream(c, &side) != TM_OK) return TM_ERR_HIP;
    hipStream_t s2 = side.s;
    auto fork = [&]() -> bool {
        return hipEventRecord(side.fork, st) == hipSuccess && hipStreamWaitEvent(s2, side.fork, 0) == hipSuccess;
    };
    auto join = [&]() -> bool {
        return hipEventRecord(side.join, s2) == hipSuccess && hipStreamWaitEvent(st, side.join, 0) == hipSuccess;
    };
    // a product on the main stream, or (second) on the second stream with
    // its own split-K partial tiles
    auto gemm = [&](BGemm g, int kind, bool second = false) -> bool {
        g.splitk = bgemm_splitk(g.m, g.n, g.k, g.k2, g.epi, (int)ns);
        g.acc = second ? accbuf2 : accbuf;
        hipStream_t gs = second ? s2 : st;
        return timed(kind, gs, [&] { return launch_bgemm(g, (int)ns, gs); }) == hipSuccess;
    };
    auto base = [&](int m, int n, int kk, int ta, int tb, int epi) {
        BGemm g;
        memset(&g, 0, sizeof(g));
        g.m = m;
        g.n = n;
        g.k = kk;
        g.ta = ta;
        g.tb = tb;
        g.epi = epi;
        g.tl = tl;
        return g;
    };
    // layer l of a chunk-start state slot: M (S = 1: S), [din][dout] row-major
    auto slot = [&](int ci, int l, int S) {
        return rowm(tape + (size_t)ci * w.tape_cs + (S ? P : 0) + c->off[l], 2 * P, c->dout[l]);
    };
    auto adj = [&](int l, int S) { return rowm(dst + (S ? P : 0) + c->off[l], 2 * P, c->dout[l]); };
    auto rec = [&](int ci, long off, int width) { return rowm(key + (size_t)ci * w.rec + off, (long)C * w.rec, width); };
    auto sc = [&](long off, int width) { return rowm(scr + off, w.scr_ss, width); };
    auto keys = [&](int ci) { return tokm(k, ci * b, bf); };
    auto hkey = [&](int ci, int l) { return l == 0 ? keys(ci) : rec(ci, w.hk[l], c->din[l]); };

    // the starting state, canonical, into slot 0
    {
        StateLayout sl = state_layout(c, ns);
        const char* s8 = static_cast<const char*>(state);
        if (timed(K_BREST, st, [&] {
                return launch_export(reinterpret_cast<const float*>(s8 + sl.M), reinterpret_cast<const float*>(s8 + sl.S),
                                     tape, P, (int)ns, c->din[0], c->dout[0], L > 1 ? c->dout[1] : 0, st);
            }) != hipSuccess)
            return TM_ERR_HIP;
    }
    // every chunk's coefficients
    BCoef co;
    memset(&co, 0, sizeof(co));
    co.mode = BC_FWD;
    co.b = b;
    co.C = C;
    co.theta = theta;
    co.eta = eta;
    co.alpha = alpha;
    co.gl = gl;
    co.cc = cc;
    co.dc = dc;
    co.coef_ss = T;
    co.cs = cs;
    co.cs_ss = (long)C * 4;
    if (timed(K_BREST, st, [&] { return launch_bcoef(co, (int)ns, st); }) != hipSuccess) return TM_ERR_HIP;

    // ---- recompute: chunk by chunk, keeping every chunk-start state ----
    for (int ci = 0; ci < C; ++ci) {
        // the key rows' forward at M_0 (z, h; the last layer's Delta = 2 (z - v))
        for (int l = 0; l < L; ++l) {
            const bool last = l + 1 == L;
            BGemm g = base(b, c->dout[l], c->din[l], 0, 0, last ? BE_OUTK : BE_HID);
            g.A = hkey(ci, l);
            g.B = slot(ci, l, 0);
            g.c0 = rec(ci, w.zk[l], c->dout[l]);
            g.c1 = last ? rec(ci, w.dk[l], c->dout[l]) : rec(ci, w.hk[l + 1], c->din[l + 1]);
            if (last) g.x0 = tokm(v, ci * b, bf);
            if (!gemm(g, K_BREST)) return TM_ERR_HIP;
        }
        // their backward: g_l = Delta_l W_l^T, Delta_{l-1} = g_l * SiLU'(z_{l-1})
        for (int l = L - 1; l >= 1; --l) {
            BGemm g = base(b, c->din[l], c->dout[l], 0, 1, BE_BWDK);
            g.A = rec(ci, w.dk[l], c->dout[l]);
            g.B = slot(ci, l, 0);
            g.c0 = rec(ci, w.gk[l], c->din[l]);
            g.c1 = rec(ci, w.dk[l - 1], c->dout[l - 1]);
            g.x0 = rec(ci, w.zk[l - 1], c->dout[l - 1]);
            if (!gemm(g, K_BREST)) return TM_ERR_HIP;
        }
        // the write: M_end = p_alpha M_0 + s0 S_0 - H^T diag(c) Delta,
        // S_end = p_eta S_0 - H^T diag(d) Delta, into the next slot (the
        // layers' writes are independent: odd layers on the second stream)
        if (L > 1 && !fork()) return TM_ERR_HIP;
        for (int l = 0; l < L; ++l) {
            BGemm g = base(c->din[l], c->dout[l], b, 1, 0, BE_UPD);
            g.dual = 2;
            g.A = hkey(ci, l);
            g.B = rec(ci, w.dk[l], c->dout[l]);
            g.sk0 = cc + (size_t)ci * b;
            g.sk1 = dc + (size_t)ci * b;
            g.sk_ss = T;
            g.x0 = slot(ci, l, 0);
            g.x1 = slot(ci, l, 1);
            g.c0 = slot(ci + 1, l, 0);
            g.c1 = slot(ci + 1, l, 1);
            g.cs = cs + (size_t)ci * 4;
            g.cs_ss = (long)C * 4;
            if (!gemm(g, K_BSTATE, (l & 1) != 0)) return TM_ERR_HIP;
        }
        if (L > 1 && !join()) return TM_ERR_HIP;
    }

    // ---- reverse sweep ----
    // the queries of chunk ci read slot wq: forward of their rows, backprop
    // of dy down to dq, and their weights' gradient added to Mbar
    auto query_steps = [&](int ci, int wq) -> bool {
        for (int l = 0; l + 1 < L; ++l) {
            BGemm g = base(b, c->dout[l], c->din[l], 0, 0, BE_HID);
            g.A = l == 0 ? tokm(q, ci * b, bf) : sc(w.hq[l], c->din[l]);
            g.B = slot(wq, l, 0);
            g.c0 = sc(w.zq[l], c->dout[l]);
            g.c1 = sc(w.hq[l + 1], c->din[l + 1]);
            if (!gemm(g, K_BREST)) return false;
        }
        auto dqm = [&](int l) { return l == L - 1 ? tokm(dy, ci * b, 0) : sc(w.dq[l], c->dout[l]); };
        for (int l = L - 1; l >= 0; --l) {
            BGemm g = base(b, c->din[l], c->dout[l], 0, 1, l > 0 ? BE_QB : BE_STORE);
            g.A = dqm(l);
            g.B = slot(wq, l, 0);
            if (l > 0) {
                g.c0 = sc(w.dq[l - 1], c->dout[l - 1]);
                g.x0 = sc(w.zq[l - 1], c->dout[l - 1]);
            } else {
                g.c0 = tokm(dq, ci * b, 0);
            }
            if (!gemm(g, K_BREST)) return false;
        }
        // (each layer's gradient goes to its own Mbar: odd layers on the
        // second stream)
        if (L > 1 && !fork()) return false;
        for (int l = 0; l < L; ++l) {
            BGemm g = base(c->din[l], c->dout[l], b, 1, 0, BE_ACC);
            g.A = l == 0 ? tokm(q, ci * b, bf) : sc(w.hq[l], c->din[l]);
            g.B = dqm(l);
            g.c0 = adj(l, 0);
            if (!gemm(g, K_BREST, (l & 1) != 0)) return false;
        }
        return L == 1 || join();
    };

    for (int ci = C - 1; ci >= 0; --ci) {
        if (read == TM_READ_AFTER_WRITE && !query_steps(ci, ci + 1)) return TM_ERR_HIP;
        // the surprise's adjoint Gbar_i = -(c_i Mbar + d_i Sbar), through
        // G_l = h_l^T Delta_l: Deltabar_l = -(c h_l Mbar_l + d h_l Sbar_l) (with
        // the row sums behind cbar, dbar), hbar_l = -(c Delta_l Mbar_l^T + d Delta_l Sbar_l^T);
        // the hbar products (independent of the Deltabar ones) on the second stream
        if (!fork()) return TM_ERR_HIP;
        for (int l = 0; l < L; ++l) {
            BGemm g = base(b, c->dout[l], c->din[l], 0, 0, BE_GP);
            g.dual = 1;
            g.A = hkey(ci, l);
            g.B = adj(l, 0);
            g.B2 = adj(l, 1);
            g.rs0 = cc + (size_t)ci * b;
            g.rs1 = dc + (size_t)ci * b;
            g.sk_ss = T;
            g.x0 = rec(ci, w.dk[l], c->dout[l]);
            g.c0 = sc(w.db[l], c->dout[l]);
            g.part = pgp + (size_t)ci * w.ngp * 128;
            g.part_ss = (long)C * w.ngp * 128;
            g.tile0 = w.gpbase[l];
            if (!gemm(g, K_BREST)) return TM_ERR_HIP;
            BGemm h = base(b, c->din[l], c->dout[l], 0, 1, BE_GQ);
            h.dual = 1;
            h.A = rec(ci, w.dk[l], c->dout[l]);
            h.B = adj(l, 0);
            h.B2 = adj(l, 1);
            h.rs0 = cc + (size_t)ci * b;
            h.rs1 = dc + (size_t)ci * b;
            h.sk_ss = T;
            h.c0 = sc(w.hb[l], c->din[l]);
            if (!gemm(h, K_BREST, true)) return TM_ERR_HIP;
        }
        if (!join()) return TM_ERR_HIP;
        // back through the key rows' backward (layers 1 .. L-1 in order)
        for (int l = 1; l < L; ++l) {
            BElem e;
            memset(&e, 0, sizeof(e));
            e.mode = BW_U;
            e.b = b;
            e.n = c->din[l];
            e.db = scr + w.db[l - 1];
            e.z = key + (size_t)ci * w.rec + w.zk[l - 1];
            e.g = key + (size_t)ci * w.rec + w.gk[l];
            e.u = scr + w.u[l];
            e.zb = scr + w.zb[l - 1];
            e.ss = w.scr_ss;
            e.rss = (long)C * w.rec;
            // then Deltabar_l += u_l W_l (from g_l = Delta_l W_l^T)
            BGemm g = base(b, c->dout[l], c->din[l], 0, 0, BE_ACC);
            g.A = sc(w.u[l], c->din[l]);
            g.B = slot(ci, l, 0);
            g.c0 = sc(w.db[l], c->dout[l]);
            if (timed(K_BREST, st, [&] { return launch_belem(e, (int)ns, st); }) != hipSuccess) return TM_ERR_HIP;
            if (!gemm(g, K_BREST)) return TM_ERR_HIP;
        }
        {
            BElem e;
            memset(&e, 0, sizeof(e));
            e.mode = BW_OUT;
            e.b = b;
            e.n = c->dout[L - 1];
            e.db = scr + w.db[L - 1];
            e.zb = scr + w.zb[L - 1];
            e.ss = w.scr_ss;
            e.dv = dv;
            e.tl = tl;
            e.t0 = ci * b;
            if (timed(K_BREST, st, [&] { return launch_belem(e, (int)ns, st); }) != hipSuccess) return TM_ERR_HIP;
        }
        // back through the key rows' forward (layers L-1 .. 0): hbar_l =
        // hbar_l(surprise) + zbar_l W_l^T, zbar_{l-1} += hbar_l SiLU'(z_{l-1}); dk
        for (int l = L - 1; l >= 0; --l) {
            BGemm g = base(b, c->din[l], c->dout[l], 0, 1, l > 0 ? BE_HB : BE_ADDSTORE);
            g.A = sc(w.zb[l], c->dout[l]);
            g.B = slot(ci, l, 0);
            g.x0 = sc(w.hb[l], c->din[l]);
            if (l > 0) {
                g.x1 = rec(ci, w.zk[l - 1], c->dout[l - 1]);
                g.c1 = sc(w.zb[l - 1], c->dout[l - 1]);
            } else {
                g.c0 = tokm(dk, ci * b, 0);
            }
            if (!gemm(g, K_BREST)) return TM_ERR_HIP;
        }
        // Mbar_0 = p_alpha Mbar + h^T zbar + u^T Delta, Sbar_0 = p_eta Sbar + s0 Mbar,
        // with the sums behind the chunk scalars' adjoints (layers
        // independent: odd layers on the second stream)
        if (L > 1 && !fork()) return TM_ERR_HIP;
        for (int l = 0; l < L; ++l) {
            BGemm g = base(c->din[l], c->dout[l], b, 1, 0, BE_ADJ);
            g.A = hkey(ci, l);
            g.B = sc(w.zb[l], c->dout[l]);
            if (l >= 1) {
                g.k2 = b;
                g.A2 = sc(w.u[l], c->din[l]);
                g.Bs2 = rec(ci, w.dk[l], c->dout[l]);
            }
            g.c0 = adj(l, 0);
            g.c1 = adj(l, 1);
            g.x0 = slot(ci, l, 0);
            g.x1 = slot(ci, l, 1);
            g.cs = cs + (size_t)ci * 4;
            g.cs_ss = (long)C * 4;
            g.part = pad + (size_t)ci * w.nad * 3;
            g.part_ss = (long)C * w.nad * 3;
            g.tile0 = w.adbase[l];
            if (!gemm(g, K_BSTATE, (l & 1) != 0)) return TM_ERR_HIP;
        }
        if (L > 1 && !join()) return TM_ERR_HIP;
        if (read == TM_READ_BEFORE_WRITE && !query_steps(ci, ci)) return TM_ERR_HIP;
    }
    // the gates' gradients, every chunk
    co.mode = BC_BWD;
    co.pgp = pgp;
    co.ngp = w.ngp;
    co.pad = pad;
    co.nad = w.nad;
    co.dtheta = dth;
    co.deta = det;
    co.dalpha = dal;
    if (timed(K_BREST, st, [&] { return launch_bcoef(co, (int)ns, st); }) != hipSuccess) return TM_ERR_HIP;
    return TM_OK;
}

}  // namespace

extern "C" {

tm_status tm_create(int dim, int depth, int expansion, int chunk, tm_ctx** out) {
    if (!out) return TM_ERR_INVALID;
    *out = nullptr;
    if (dim < 32 || dim % 32 != 0 || dim > 1024) return TM_ERR_INVALID;
    if (depth < 1 || depth > MAXL) return TM_ERR_INVALID;
    if (expansion < 1 || (long)dim * expansion > 65536) return TM_ERR_INVALID;
    if (chunk < 1 || chunk > MAX_CHUNK) return TM_ERR_INVALID;
    tm_ctx* c = new (std::nothrow) tm_ctx;
    if (!c) return TM_ERR_INVALID;
    memset(c, 0, sizeof(*c));
    c->gmu = new (std::nothrow) std::mutex;
    c->graphs = new (std::nothrow) std::vector<GraphEntry>;
    c->capture_streams = new (std::nothrow) std::vector<std::pair<int, hipStream_t>>;
    c->sides = new (std::nothrow) std::vector<tm_ctx::Side>;
    if (!c->gmu || !c->graphs || !c->capture_streams || !c->sides) {
        delete c->gmu;
        delete c->graphs;
        delete c->capture_streams;
        delete c->sides;
        delete c;
        return TM_ERR_INVALID;
    }
    c->dim = dim;
    c->depth = depth;
    c->expansion = depth > 1 ? expansion : 1;
    c->chunk = chunk;
    c->hidden = depth > 1 ? dim * expansion : dim;
    c->L = depth;
    c->off[0] = 0;
    c->tbase[0] = 0;
    for (int l = 0; l < depth; ++l) {
        c->din[l] = l == 0 ? dim : c->hidden;
        c->dout[l] = l == depth - 1 ? dim : c->hidden;
        c->off[l + 1] = c->off[l] + (long)c->din[l] * c->dout[l];
        c->tj[l] = (c->dout[l] + 63) / 64;
        c->tbase[l + 1] = c->tbase[l] + ((c->din[l] + 63) / 64) * c->tj[l];
    }
    c->P = c->off[depth];
    uint64_t h = 1469598103934665603ull;
    h = fnv(h, (uint64_t)dim);
    h = fnv(h, (uint64_t)depth);
    h = fnv(h, (uint64_t)c->expansion);
    h = fnv(h, (uint64_t)chunk);
    c->hash = h;
    *out = c;
    return TM_OK;
}

void tm_destroy(tm_ctx* ctx) {
    if (!ctx) return;
    for (GraphEntry& e : *ctx->graphs)
        if (e.exec) (void)hipGraphExecDestroy(e.exec);
    for (auto& pr : *ctx->capture_streams) (void)hipStreamDestroy(pr.second);
    for (auto& sd : *ctx->sides) {
        (void)hipEventDestroy(sd.fork);
        (void)hipEventDestroy(sd.join);
        (void)hipStreamDestroy(sd.s);
    }
    delete ctx->graphs;
    delete ctx->capture_streams;
    delete ctx->sides;
    delete ctx->gmu;
    delete ctx;
}

size_t tm_param_count(const tm_ctx* c) { return c ? (size_t)c->P : 0; }

tm_status tm_config(const tm_ctx* c, int* dim, int* depth, int* expansion, int* chunk) {
    if (!c) return TM_ERR_INVALID;
    if (dim) *dim = c->dim;
    if (depth) *depth = c->depth;
    if (expansion) *expansion = c->expansion;
    if (chunk) *chunk = c->chunk;
    return TM_OK;
}

size_t tm_state_bytes(const tm_ctx* c, int batch, int heads) {
    if (!c || batch <= 0 || heads <= 0) return 0;
    return state_layout(c, (long)batch * heads).total;
}

size_t tm_workspace_bytes(const tm_ctx* c, int batch, int heads, int n_tokens) {
    if (!c || batch <= 0 || heads <= 0 || n_tokens < 0) return 0;
    return store_ws_bytes(c, batch, heads, n_tokens > 0 ? n_tokens : 1);
}

tm_status tm_state_init(const tm_ctx* c, void* state, int batch, int heads, const float* init,
                        void* stream) {
    if (!c || !state || !init || batch <= 0 || heads <= 0) return TM_ERR_INVALID;
    if ((long)batch * heads > 65535) return TM_ERR_INVALID;
    if (!aligned(state, 256) || !aligned(init, 4)) return TM_ERR_INVALID;
    const long ns = (long)batch * heads;
    char* s = static_cast<char*>(state);
    tm_status rc = with_graph(c, make_key(0, batch, heads, 0, 0, {state, init}), static_cast<hipStream_t>(stream),
                              [&](hipStream_t st) {
        UpdArgs u = base_upd(c, s, ns);
        return hip_status(launch_state_init(u, c->tbase[c->L], (int)ns, init, heads,
                                            reinterpret_cast<StateHeader*>(s), c->hash, batch, heads, st));
    });
    if (rc == TM_OK) state_register(c, state, batch, heads);
    return rc;
}

tm_status tm_store(const tm_ctx* c, void* state, const void* k, const void* v, const float* theta,
                   const float* eta, const float* alpha, int batch, int heads, int n_tokens,
                   tm_dtype dtype, void* ws, void* stream) {
    tm_status rc = check_common(c, state, batch, heads, n_tokens, dtype, ws);
    if (rc != TM_OK) return rc;
    if (n_tokens == 0) return TM_OK;   // nothing to store: the token pointers are not examined
    if (!tok_ok(k) || !tok_ok(v) || !gate_ok(theta) || !gate_ok(eta) || !gate_ok(alpha))
        return TM_ERR_INVALID;
    if (n_tokens % c->chunk != 0) return TM_ERR_SHAPE;
    if (state_lookup(c, state, batch, heads) != TM_OK) return TM_ERR_STATE;
    return with_graph(c, make_key(1, batch, heads, n_tokens, dtype, {state, k, v, theta, eta, alpha, ws}),
                      static_cast<hipStream_t>(stream), [&](hipStream_t st) {
        return run_store(c, state, k, v, nullptr, theta, eta, alpha, nullptr, batch, heads, n_tokens,
                         dtype, ws, st);
    });
}

tm_status tm_forward_ex(const tm_ctx* c, void* state, const void* k, const void* v, const void* q,
                        const float* theta, const float* eta, const float* alpha, float* y, int batch,
                        int heads, int n_tokens, tm_dtype dtype, tm_read read, void* ws, void* stream) {
    tm_status rc = check_common(c, state, batch, heads, n_tokens, dtype, ws);
    if (rc != TM_OK) return rc;
    if (read != TM_READ_AFTER_WRITE && read != TM_READ_BEFORE_WRITE && read != TM_READ_PER_TOKEN)
        return TM_ERR_INVALID;
    if (n_tokens == 0) return TM_OK;
    if (!tok_ok(k) || !tok_ok(v) || !tok_ok(q) || !tok_ok(y) || !gate_ok(theta) || !gate_ok(eta) ||
        !gate_ok(alpha))
        return TM_ERR_INVALID;
    if (n_tokens % c->chunk != 0) return TM_ERR_SHAPE;
    if (state_lookup(c, state, batch, heads) != TM_OK) return TM_ERR_STATE;
    const int kind = read == TM_READ_BEFORE_WRITE ? 4 : read == TM_READ_PER_TOKEN ? 6 : 2;
    return with_graph(c, make_key(kind, batch, heads, n_tokens, dtype, {state, k, v, q, theta, eta, alpha, y, ws}),
                      static_cast<hipStream_t>(stream), [&](hipStream_t st) {
        return run_store(c, state, k, v, q, theta, eta, alpha, y, batch, heads, n_tokens, dtype, ws, st,
                         (int)read);
    });
}

tm_status tm_project(const tm_ctx* c, const void* x, int model_dim, const void* w_kvq, const float* conv,
                     int conv_len, const float* w_gate, const float* gate_bias, float* history, void* k,
                     void* v, void* q, float* theta, float* eta, float* alpha, int batch, int heads,
                     int n_tokens, tm_dtype dtype, void* stream) {
    if (!c) return TM_ERR_INVALID;
    if (dtype != TM_F32 && dtype != TM_BF16) return TM_ERR_DTYPE;
    if (batch <= 0 || heads <= 0 || n_tokens < 0 || model_dim < 32 || model_dim % 32 != 0 ||
        conv_len < 1 || conv_len > MAX_CONV || (long)batch * n_tokens > 0x7fffffffL ||
        (long)heads * c->dim > 65536)
        return TM_ERR_INVALID;
    if (!tok_ok(x) || !tok_ok(w_kvq) || !gate_ok(conv) || !tok_ok(w_gate) || !gate_ok(gate_bias) ||
        (conv_len > 1 && !gate_ok(history)))
        return TM_ERR_INVALID;
    if (n_tokens == 0) return TM_OK;
    if (!tok_ok(k) || !tok_ok(v) || !tok_ok(q) || !gate_ok(theta) || !gate_ok(eta) || !gate_ok(alpha))
        return TM_ERR_INVALID;
    GraphEntry key = make_key(5, batch, heads, n_tokens, dtype, {x, w_kvq, conv, w_gate, gate_bias, history, k, v,
                                                               q, theta, eta, alpha});
    key.extra = model_dim * 8 + conv_len;
    ProjArgs p;
    memset(&p, 0, sizeof(p));
    p.x = x;
    p.w = w_kvq;
    p.conv = conv;
    p.wg = w_gate;
    p.gb = gate_bias;
    p.hist = history;
    p.out[0] = k;
    p.out[1] = v;
    p.out[2] = q;
    p.gate[0] = theta;
    p.gate[1] = eta;
    p.gate[2] = alpha;
    p.B = batch;
    p.T = n_tokens;
    p.D = model_dim;
    p.H = heads;
    p.d = c->dim;
    p.K = conv_len;
    return with_graph(c, key, static_cast<hipStream_t>(stream), [&](hipStream_t st) {
        // (timed: the projection kernel, the first of the two launches)
        return timed(K_PROJ, st, [&] { return launch_project(p, dtype == TM_F32 ? 1 : 0, st); }) == hipSuccess
                   ? TM_OK
                   : TM_ERR_HIP;
    });
}

tm_status tm_forward(const tm_ctx* c, void* state, const void* k, const void* v, const void* q,
                     const float* theta, const float* eta, const float* alpha, float* y, int batch,
                     int heads, int n_tokens, tm_dtype dtype, void* ws, void* stream) {
    return tm_forward_ex(c, state, k, v, q, theta, eta, alpha, y, batch, heads, n_tokens, dtype,
                         TM_READ_AFTER_WRITE, ws, stream);
}

size_t tm_backward_workspace_bytes(const tm_ctx* c, int batch, int heads, int n_tokens) {
    if (!c || batch <= 0 || heads <= 0 || n_tokens < 0) return 0;
    return bwd_layout(c, (long)batch * heads, n_tokens).total;
}

tm_status tm_backward(const tm_ctx* c, const void* state, const void* k, const void* v, const void* q,
                      const float* theta, const float* eta, const float* alpha, const float* dy, float* dstate,
                      float* dk, float* dv, float* dq, float* dtheta, float* deta, float* dalpha, int batch,
                      int heads, int n_tokens, tm_dtype dtype, tm_read read, void* ws, void* stream) {
    tm_status rc = check_common(c, state, batch, heads, n_tokens, dtype, ws);
    if (rc != TM_OK) return rc;
    if (read != TM_READ_AFTER_WRITE && read != TM_READ_BEFORE_WRITE) return TM_ERR_INVALID;
    if (!dstate || !aligned(dstate, 16)) return TM_ERR_INVALID;
    if (n_tokens == 0) return TM_OK;   // the call is the identity on the state
    if (!tok_ok(k) || !tok_ok(v) || !tok_ok(q) || !tok_ok(dy) || !tok_ok(dk) || !tok_ok(dv) || !tok_ok(dq) ||
        !gate_ok(theta) || !gate_ok(eta) || !gate_ok(alpha) || !gate_ok(dtheta) || !gate_ok(deta) ||
        !gate_ok(dalpha))
        return TM_ERR_INVALID;
    if (n_tokens % c->chunk != 0) return TM_ERR_SHAPE;
    if (state_lookup(c, state, batch, heads) != TM_OK) return TM_ERR_STATE;
    GraphEntry key = make_key(7, batch, heads, n_tokens, dtype,
                              {state, k, v, q, theta, eta, alpha, dy, dstate, dk, dv, dq, dtheta, deta, dalpha, ws});
    key.extra = (int)read;
    return with_graph(c, key, static_cast<hipStream_t>(stream), [&](hipStream_t st) {
        return run_bwd(c, state, k, v, q, theta, eta, alpha, dy, dstate, dk, dv, dq, dtheta, deta, dalpha, batch,
                       heads, n_tokens, dtype, (int)read, ws, st);
    });
}

tm_status tm_forward_noalloc(const tm_ctx* c, void* state, const void* k, const void* v, const void* q,
                             const float* theta, const float* eta, const float* alpha, float* y, int batch,
                             int heads, int n_tokens, tm_dtype dtype, void* stream) {
    if (!c || !state) return TM_ERR_INVALID;
    if (batch <= 0 || heads <= 0 || n_tokens < 0) return TM_ERR_INVALID;
    if ((long)batch * heads > 65535) return TM_ERR_INVALID;
    if (dtype != TM_F32 && dtype != TM_BF16) return TM_ERR_DTYPE;
    if (!aligned(state, 256)) return TM_ERR_INVALID;
    if (n_tokens == 0) return TM_OK;
    if (!tok_ok(k) || !tok_ok(v) || !tok_ok(q) || !tok_ok(y) || !gate_ok(theta) || !gate_ok(eta) ||
        !gate_ok(alpha))
        return TM_ERR_INVALID;
    if (n_tokens % c->chunk != 0) return TM_ERR_SHAPE;
    if (state_lookup(c, state, batch, heads) != TM_OK) return TM_ERR_STATE;
    // (the size tm_workspace_bytes reports, though one chain needs no more
    // than ws_layout's total)
    if (store_ws_bytes(c, batch, heads, n_tokens) > SCRATCH_BYTES) return TM_ERR_SCRATCH;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return TM_ERR_HIP;
    // direct launches (no graph capture: instantiating a graph may allocate)
    return run_store(c, state, k, v, q, theta, eta, alpha, y, batch, heads, n_tokens, dtype, ws,
                     static_cast<hipStream_t>(stream), TM_READ_AFTER_WRITE, 1);
}

tm_status tm_retrieve(const tm_ctx* c, const void* state_v, const void* q, float* y, int batch,
                      int heads, int n_tokens, tm_dtype dtype, void* ws_v, void* stream) {
    tm_status rc = check_common(c, state_v, batch, heads, n_tokens, dtype, ws_v);
    if (rc != TM_OK) return rc;
    if (n_tokens == 0) return TM_OK;
    if (!tok_ok(q) || !tok_ok(y)) return TM_ERR_INVALID;
    if (state_lookup(c, state_v, batch, heads) != TM_OK) return TM_ERR_STATE;
    char* state = const_cast<char*>(static_cast<const char*>(state_v));   // read only below
    char* ws = static_cast<char*>(ws_v);
    const long ns = (long)batch * heads;
    return with_graph(c, make_key(3, batch, heads, n_tokens, dtype, {state_v, q, y, ws_v}),
                      static_cast<hipStream_t>(stream), [&](hipStream_t st) {
        WsLayout w = ws_layout(c, ns, n_tokens);
        TokLayout tl{n_tokens, heads, c->dim};
        if (dtype == TM_BF16 && c->L == 2 && mlp2_fits(c->dim, c->hidden)) {
            // both layers in one launch over every query row (no workspace)
            StateLayout sl = state_layout(c, ns);
            Mlp2Args a{};
            a.q = q;
            a.y = y;
            a.w = state + sl.Wt;
            a.w_ss = c->P;
            a.off1 = c->off[1];
            a.tl = tl;
            a.t0 = 0;
            a.nrows = n_tokens;
            a.d = c->dim;
            a.h = c->hidden;
            a.xcd_streams = xcd_streams_on() && ns % 8 == 0 && ns >= 8 ? 1 : 0;
            return hip_status(timed(K_FWD, st, [&] { return launch_mlp2(a, (int)ns, st); }));
        }
        for (long p0 = 0; p0 < n_tokens; p0 += w.ret_rows) {
            FwdRows fr{};
            fr.nq = (int)((n_tokens - p0) < w.ret_rows ? (n_tokens - p0) : w.ret_rows);
            fr.q = q;
            fr.tq = (int)p0;
            fr.nk = 0;
            fr.k = nullptr;
            fr.tk = 0;
            fr.v = nullptr;
            fr.y = y;
            tm_status r2 = run_forward_layers(c, state, ns, w, ws, tl, fr, dtype == TM_F32, true, st);
            if (r2 != TM_OK) return r2;
        }
        return TM_OK;
    });
}

tm_status tm_mac_window(const void* persistent, int n_persist, const float* recalled, const void* segment,
                        void* window, int batch, int seg_len, int model_dim, tm_dtype dtype, void* stream) {
    if (dtype != TM_F32 && dtype != TM_BF16) return TM_ERR_DTYPE;
    if (batch <= 0 || seg_len <= 0 || n_persist < 0 || model_dim < 32 || model_dim % 32 != 0 ||
        (long)batch * (n_persist + 2L * seg_len) * model_dim > (1L << 40))
        return TM_ERR_INVALID;
    if (!tok_ok(recalled) || !tok_ok(segment) || !tok_ok(window) || (n_persist > 0 && !tok_ok(persistent)))
        return TM_ERR_INVALID;
    MacArgs a{persistent, recalled, segment, window, batch, seg_len, n_persist, model_dim};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(timed(K_MAC, st, [&] { return launch_mac_window(a, dtype == TM_F32 ? 1 : 0, st); }));
}

tm_status tm_mac_gate(const void* y, const float* mem, float* out, int batch, int seg_len, int model_dim,
                      tm_dtype dtype, void* stream) {
    if (dtype != TM_F32 && dtype != TM_BF16) return TM_ERR_DTYPE;
    if (batch <= 0 || seg_len <= 0 || model_dim < 32 || model_dim % 32 != 0 ||
        (long)batch * seg_len * model_dim > (1L << 40))
        return TM_ERR_INVALID;
    if (!tok_ok(y) || !tok_ok(mem) || !tok_ok(out)) return TM_ERR_INVALID;
    MacArgs a{nullptr, mem, y, out, batch, seg_len, 0, model_dim};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(timed(K_MAC, st, [&] { return launch_mac_gate(a, dtype == TM_F32 ? 1 : 0, st); }));
}

tm_status tm_state_export(const tm_ctx* c, const void* state, int batch, int heads, float* dst,
                          void* stream) {
    if (!c || !state || !dst || batch <= 0 || heads <= 0) return TM_ERR_INVALID;
    if (!aligned(state, 256) || !aligned(dst, 4)) return TM_ERR_INVALID;
    if (state_lookup(c, state, batch, heads) != TM_OK) return TM_ERR_STATE;
    const long ns = (long)batch * heads;
    StateLayout sl = state_layout(c, ns);
    const char* s = static_cast<const char*>(state);
    return hip_status(launch_export(reinterpret_cast<const float*>(s + sl.M),
                                    reinterpret_cast<const float*>(s + sl.S), dst, c->P, (int)ns, c->din[0],
                                    c->dout[0], c->L > 1 ? c->dout[1] : 0, static_cast<hipStream_t>(stream)));
}

tm_status tm_state_import(const tm_ctx* c, void* state, int batch, int heads, const float* src,
                          void* stream) {
    if (!c || !state || !src || batch <= 0 || heads <= 0) return TM_ERR_INVALID;
    if ((long)batch * heads > 65535) return TM_ERR_INVALID;
    if (!aligned(state, 256) || !aligned(src, 4)) return TM_ERR_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const long ns = (long)batch * heads;
    char* s = static_cast<char*>(state);
    UpdArgs u = base_upd(c, s, ns);
    if (launch_header(reinterpret_cast<StateHeader*>(s), c->hash, batch, heads, st) != hipSuccess)
        return TM_ERR_HIP;
    if (launch_import(u.M, u.S, src, c->P, (int)ns, c->din[0], c->dout[0], c->L > 1 ? c->dout[1] : 0, st) !=
        hipSuccess)
        return TM_ERR_HIP;
    if (launch_shadow(u, c->tbase[c->L], (int)ns, st) != hipSuccess) return TM_ERR_HIP;
    state_register(c, state, batch, heads);
    return TM_OK;
}

tm_status tm_state_check(const tm_ctx* c, const void* state, int batch, int heads, int* nonfinite,
                         long long* position, void* stream) {
    if (!c || !state || batch <= 0 || heads <= 0) return TM_ERR_INVALID;
    StateHeader h;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&h, state, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return TM_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return TM_ERR_HIP;
    if (h.magic != STATE_MAGIC || h.version != STATE_VERSION || h.cfg_hash != c->hash ||
        h.batch != batch || h.heads != heads)
        return TM_ERR_STATE;
    if (nonfinite) *nonfinite = h.nonfinite;
    if (position) *position = h.position;
    return TM_OK;
}

tm_status tm_graphs_enable(int on) {
    g_graphs = on != 0;
    return TM_OK;
}

tm_status tm_store_groups_enable(int on) {
    g_store_groups = on != 0;
    return TM_OK;
}

tm_status tm_w1_split_enable(int on) {
    g_w1_split = on != 0;
    return TM_OK;
}

tm_status tm_timing_enable(int class_mask) {
    std::lock_guard<std::mutex> g(g_tmu);
    g_timing = class_mask & ((1 << K_CLASSES) - 1);
    return TM_OK;
}

tm_status tm_timing_read(int kind, double* total_ms, long long* launches) {
    if (kind < 0 || kind >= K_CLASSES) return TM_ERR_INVALID;
    std::vector<Timed> todo;
    {
        std::lock_guard<std::mutex> g(g_tmu);
        todo.swap(g_pending);
    }
    tm_status rc = TM_OK;
    double ms[K_CLASSES] = {0};
    long long n[K_CLASSES] = {0};
    for (const Timed& t : todo) {
        float x = 0.f;
        if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&x, t.a, t.b) != hipSuccess) {
            rc = TM_ERR_HIP;
            continue;
        }
        ms[t.kind] += x;
        n[t.kind] += 1;
    }
    std::lock_guard<std::mutex> g(g_tmu);
    for (const Timed& t : todo) {
        g_pool.push_back(t.a);
        g_pool.push_back(t.b);
    }
    for (int i = 0; i < K_CLASSES; ++i) {
        g_ms[i] += ms[i];
        g_n[i] += n[i];
    }
    if (total_ms) *total_ms = g_ms[kind];
    if (launches) *launches = g_n[kind];
    g_ms[kind] = 0;
    g_n[kind] = 0;
    return rc;
}

const char* tm_status_str(tm_status s) {
    switch (s) {
        case TM_OK: return "ok";
        case TM_ERR_INVALID: return "invalid argument";
        case TM_ERR_SHAPE: return "n_tokens is not a multiple of the chunk size";
        case TM_ERR_DTYPE: return "unknown dtype";
        case TM_ERR_STATE: return "state header does not match the memory configuration";
        case TM_ERR_HIP: return "HIP runtime error";
        case TM_ERR_SCRATCH: return "the call needs more workspace than the library's scratch array holds";
    }
    return "unknown status";
}

}  // extern "C"
