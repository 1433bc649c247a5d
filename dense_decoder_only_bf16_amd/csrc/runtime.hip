// Host runtime behind the C ABI in include/nc.h: model and KV-cache objects, argument
// checks, workspace management and the per-layer launch schedule of prefill and decode.
//
// Schedule of one layer (the block structure of the yelogs.com launch write-up's
// architecture answer; plain pre-norm residual reading):
//   QKV product (raw, fp32)  -> QKV finish: row norm scale, RoPE, QK-norm, KV-cache write
//   attention (prefill: flash kernel; decode: one kernel over balanced runs of 64-key
//   blocks that merges rows cut between runs itself)
//   O product  + residual epilogue (x += ., dtype copy of x, per-row sum of squares)
//   FC product + norm scale + ReLU^2 epilogue
//   PROJ product + residual epilogue
// then the LM head with norm scale and softcap.  Prefill uses the 256x256 MFMA tile with
// the epilogues fused (the QKV finish is a separate row kernel).  Decode (M = batch rows)
// uses the weight-streaming decode products with the elementwise epilogues fused (at most
// 32 rows: K split over the waves of one workgroup, the QKV finish in the QKV product's
// epilogue; more rows: 256- or 128-column workgroups with K split across workgroups, a split-K
// finish kernel, and a separate QKV finish kernel); the LM head's launch also advances the
// row lengths.  The whole decode step is
// captured once per (token buffer, logit buffer) pair as a HIP graph and replayed.
// The L2 caches of the chip's dies are not coherent with each other, so a device-wide
// fence costs a write-back and invalidation of a die's L2.  Reductions across workgroups
// are separate launches, except where data passes through device-scope stores and loads
// and an arrival counter or ready flag, with no fence: the decode down-projection's K
// slices, the fused QKV finish's head tiles, and the decode attention's partial states
// (whose merging workgroup waits, bounded, only for runs dispatched before it).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/nc.h"
#include "kernels.h"

using namespace nc;

thread_local LaunchStamp nc::t_stamp = {};

namespace {

thread_local std::string g_err;

nc_status fail(nc_status code, const std::string& msg) {
    g_err = msg;
    return code;
}

#define HIP_TRY(expr)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail(e_ == hipErrorOutOfMemory ? NC_ERR_OOM : NC_ERR_DEVICE,              \
                        std::string(#expr) + ": " + hipGetErrorString(e_));                  \
    } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- kernel timing (diagnostics): every launch of one class of kernels gets a pair of HIP
// events that its dispatch stamps with the kernel's start and end (hipExtLaunchKernel).
// While a class is timed, decode steps launch their kernels one by one instead of replaying
// a captured graph, since stamped launches cannot be captured.
struct TimingPair {  // one timed operation: its kernels' event pairs and its work
    hipEvent_t ev[NC_MAX_STAMPS][2];
    int n;
    double bytes, flops;
};
struct Timing {
    int cls = NC_KC_NONE;
    std::vector<TimingPair> pending;  // launches not yet read
    long long launches = 0;
    double ms = 0, bytes = 0, flops = 0;
};
Timing g_tm;

void timing_release(TimingPair& tp) {
    for (int i = 0; i < NC_MAX_STAMPS; ++i)
        for (int j = 0; j < 2; ++j)
            if (tp.ev[i][j]) (void)hipEventDestroy(tp.ev[i][j]);
}

}  // namespace

struct nc_model {
    nc_config cfg;
    DType dt;
    size_t esz;
    int device;
    void* arena = nullptr;
    const void* wte = nullptr;
    const void* lm = nullptr;
    int e8_lm = 0;
    struct Layer {
        const void *wqkv, *wo, *wfc, *wproj;
        int e8_fc = 0, e8_proj = 0;  // exponents of the e4m3 weight copies (compensated prefill)
    };
    std::vector<Layer> layers;
    float* rope_cos = nullptr;
    float* rope_sin = nullptr;
    std::vector<int> windows;  // per-layer sliding window, -1: the whole causal context
    struct Extras {            // the later version's blocks (nc_model_set_extras)
        bool on = false;
        std::vector<float> lam, mu;  // residual scaling per layer
        void* smear_gate = nullptr;
        int smear_ch = 0;
        float smear_lambda = 0.f;
        int backout_layer = -1;
        float backout_lambda = 0.f;
        std::vector<void*> ve, ve_gate;  // per layer (null: none)
        int ve_ch = 0;
    } ex;
    int live_kv = 0;
};

// Workspace of the forward: every buffer the kernels use beyond the inputs, the outputs,
// the weights and the cache.  One block, laid out by ws_layout for `cap_m` token rows; the
// same layout is carved from library-allocated memory (nc_kv) or from the static array of
// the allocation-free decode entry point.
struct Ws {
    long long cap_m = 0;
    int ss_parts_max = 0;
    void* base = nullptr;     // the block (null: none)
    float* x = nullptr;       // [M][d] fp32 residual
    void* act = nullptr;      // [M][d] dtype copy of x
    float* ss_a = nullptr;    // [parts][M] sums of squares feeding the QKV / LM-head norm
    float* ss_b = nullptr;    // [parts][M] sums of squares feeding the MLP norm
    float* qkv = nullptr;     // [M][(H+2 nkv) hd] raw products
    void* q = nullptr;        // [M][H][hd]
    void* y = nullptr;        // [M][H hd] attention output
    void* u = nullptr;        // [M][d_ff] MLP hidden
    void* act_lo = nullptr;   // bf16 only: low parts of the MLP operands (compensated
    void* u_lo = nullptr;     // products): x - bf16(x) after attention, u - bf16(u)
    float* apart = nullptr;   // decode attention partial states
    int32_t* actr = nullptr;  // decode attention ready flags, one per (row, K/V head) and slot
    int32_t* fctr = nullptr;  // decode QKV finish in the product's epilogue: arrival counters per head slot
    float* dpart = nullptr;   // decode projections: split-K arrival counters, then partials
    float* tpart = nullptr;   // prefill products (bf16): partial sums of the tail split's K halves
    int32_t* tctr = nullptr;  // and their arrival counters / ready flags (2 per tile slot)
    float* x0 = nullptr;      // later-version blocks: stream before layer 0's scaling [M][d]
    float* xb = nullptr;      // and the backout source [M][d]
    int32_t* tokbuf = nullptr;   // the rows' clamped tokens (value embeddings) [M]
    ResidExtra* rx_dev = nullptr;  // per layer: the PROJ residual's blocks (decode)
    ValueEmbed* ve_dev = nullptr;  // per layer: the value embedding (decode)
    long long dpart_elems = 0;
    long long apart_elems = 0;
    long long actr_elems = 0;
    int apart_slots = 0;      // partial slots per (row, K/V head) unit
    size_t bytes = 0;         // size of the block
};

struct nc_kv {
    nc_model* m;
    int B, max_seq, S;  // S: allocated positions per row (stride), multiple of 64
    void* kcache = nullptr;  // [L][B][nkv][S][hd]
    void* vcache = nullptr;  // [L][B][nkv][hd][S]
    int32_t* lens_dev = nullptr;
    std::vector<int32_t> lens_host;
    int32_t* hist = nullptr;  // [B][S] tokens by position (only with smear)
    Ws ws;  // workspace, library-allocated (grown on demand)
    // decode step captured as a HIP graph, keyed by the caller's token/logit buffers
    bool use_graph = true;
    hipStream_t cap_stream = nullptr;
    struct Graph {
        const void* tokens;
        const void* logits;
        const void* next;  // greedy picks written in the same graph (null: none)
        hipGraphExec_t exec;
    };
    std::vector<Graph> graphs;
};

namespace {

void drop_graph(nc_kv::Graph& g) {
    (void)hipGraphExecDestroy(g.exec);
}

void drop_graphs(nc_kv* kv) {
    for (auto& g : kv->graphs) drop_graph(g);
    kv->graphs.clear();
}

void ws_free(nc_kv* kv) {
    drop_graphs(kv);  // captured graphs point into the workspace
    if (kv->ws.base) (void)hipFree(kv->ws.base);
    kv->ws = Ws{};
}

// RESID extras of layer l's MLP residual (PROJ): the next layer's scaling, the backout
// source when the next layer is the backout layer, the backout itself after the last.
ResidExtra proj_resid_extra(const nc_model* m, const Ws& ws, int l) {
    const nc_model::Extras& ex = m->ex;
    ResidExtra r{};
    r.ra = 1.f;
    if (!ex.on) return r;
    r.x0 = ws.x0;
    if (l + 1 < m->cfg.n_layer) {
        r.ra = ex.lam[l + 1];
        r.rb = ex.mu[l + 1];
        if (l + 1 == ex.backout_layer) r.xb_out = ws.xb;
    } else if (ex.backout_layer >= 0) {
        r.xb = ws.xb;
        r.rc = -ex.backout_lambda;
    }
    return r;
}

// Value embedding of layer l (ve null: none); the tokens are those the embedding kernel
// recorded for the rows of the current call.
ValueEmbed value_embed(const nc_model* m, const Ws& ws, int l) {
    ValueEmbed v{};
    if (!m->ex.on || !m->ex.ve[l]) return v;
    v.ve = m->ex.ve[l]; v.ve_gate = m->ex.ve_gate[l]; v.ve_ch = m->ex.ve_ch; v.vocab = m->cfg.vocab;
    v.tok = ws.tokbuf; v.xin = ws.x; v.xin_stride = m->cfg.d_model;
    return v;
}

// Layout of the workspace for M token rows of a cache of B rows and S positions, carved
// from `base` (null: sizes only, every pointer offset from 0).  Each buffer starts at a
// 256-byte boundary; ws.bytes is the total.
Ws ws_layout(const nc_model* m, int B, int S, long long M, void* base) {
    const nc_config& c = m->cfg;
    const size_t es = m->esz;
    Ws w{};
    w.cap_m = M;
    const long long d = c.d_model, hq = (long long)c.n_head * c.head_dim;
    const long long nqkv = (long long)(c.n_head + 2 * c.n_kv_head) * c.head_dim;
    // row statistics come in parts of one per output tile of the producing product
    w.ss_parts_max = (c.d_model + dec_gemm_tile_n() - 1) / dec_gemm_tile_n();
    // dtype activations that decode stores blocked hold whole 32-row blocks
    const long long Mr = (M + 31) / 32 * 32;
    size_t off = 0;
    auto take = [&](long long bytes) -> void* {
        void* p = (char*)base + off;
        off += align_up((size_t)std::max(bytes, 0LL), 256);
        return p;
    };
    w.x = (float*)take(M * d * 4);
    w.act = take(Mr * d * es);
    w.ss_a = (float*)take((long long)w.ss_parts_max * M * 4);
    w.ss_b = (float*)take((long long)w.ss_parts_max * M * 4);
    w.qkv = (float*)take(M * nqkv * 4);
    w.q = take(M * hq * es);
    w.y = take(Mr * hq * es);
    w.u = take(Mr * c.d_ff * es);
    if (m->dt == BF16) {
        w.act_lo = take(Mr * d * es);
        w.u_lo = take(Mr * c.d_ff * es);
    }
    const nc_model::Extras& ex = m->ex;
    if (ex.on) {
        w.x0 = (float*)take(M * d * 4);
        if (ex.backout_layer >= 0) w.xb = (float*)take(M * d * 4);
        w.tokbuf = (int32_t*)take(M * 4);
        w.rx_dev = (ResidExtra*)take(c.n_layer * (long long)sizeof(ResidExtra));
        w.ve_dev = (ValueEmbed*)take(c.n_layer * (long long)sizeof(ValueEmbed));
    }
    const int units = B * c.n_kv_head;  // (row, K/V head) pairs of decode attention
    w.apart_slots = attn_decode_slots(units, S);
    w.apart_elems = (long long)units * w.apart_slots * 16 * (c.head_dim + 2);
    w.apart = (float*)take(w.apart_elems * 4);
    w.actr_elems = (long long)units * w.apart_slots;
    w.actr = (int32_t*)take(w.actr_elems * 4);
    w.fctr = (int32_t*)take(DEC_FIN_SLOTS * 4);
    {   // split-K partials of the decode projections (M = batch rows)
        const int hqv = c.n_head * c.head_dim, nq = (c.n_head + 2 * c.n_kv_head) * c.head_dim;
        w.dpart_elems = std::max({dec_gemm_part_elems(m->dt, EPI_STORE, B, nq, c.d_model),
                                  dec_gemm_part_elems(m->dt, EPI_RESID, B, c.d_model, hqv),
                                  dec_gemm_part_elems(m->dt, EPI_RELU2, B, c.d_ff, c.d_model),
                                  dec_gemm_part_elems(m->dt, EPI_RESID, B, c.d_model, c.d_ff),
                                  dec_gemm_part_elems(m->dt, EPI_SOFTCAP, B, c.vocab, c.d_model)});
        w.dpart = w.dpart_elems > 0 ? (float*)take(w.dpart_elems * 4) : nullptr;
    }
    if (m->dt == BF16 && M > 1024) {  // prefill sizes only (32 MB); decode rows never need it
        w.tpart = (float*)take((long long)GEMM_TAIL_SLOTS * GEMM_TAIL_FLOATS * 4);
        w.tctr = (int32_t*)take(2LL * GEMM_TAIL_SLOTS * 4);
    }
    w.bytes = off;
    w.base = base;
    return w;
}

// Grow the workspace to hold M token rows.
nc_status ws_ensure(nc_kv* kv, long long M) {
    if (M <= kv->ws.cap_m) return NC_OK;
    HIP_TRY(hipDeviceSynchronize());
    ws_free(kv);
    const size_t bytes = ws_layout(kv->m, kv->B, kv->S, M, nullptr).bytes;
    void* base = nullptr;
    HIP_TRY(hipMalloc(&base, bytes));
    Ws w = ws_layout(kv->m, kv->B, kv->S, M, base);
    // the attention ready flags and the split-K arrival counters start at zero, and every
    // launch leaves them so
    hipError_t e = hipMemset(w.actr, 0, (size_t)w.actr_elems * 4);
    if (e == hipSuccess) e = hipMemset(w.fctr, 0, DEC_FIN_SLOTS * 4);
    if (e == hipSuccess && w.dpart) e = hipMemset(w.dpart, 0, DEC_PART_CTRS * 4);
    if (e == hipSuccess && w.tctr) e = hipMemset(w.tctr, 0, 2 * GEMM_TAIL_SLOTS * 4);
    if (e == hipSuccess && kv->m->ex.on) {  // the per-layer blocks that decode kernels read through pointers
        const nc_config& c = kv->m->cfg;
        std::vector<ResidExtra> rx(c.n_layer);
        std::vector<ValueEmbed> ve(c.n_layer);
        for (int l = 0; l < c.n_layer; ++l) {
            rx[l] = proj_resid_extra(kv->m, w, l);
            ve[l] = value_embed(kv->m, w, l);
        }
        e = hipMemcpy(w.rx_dev, rx.data(), rx.size() * sizeof(ResidExtra), hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(w.ve_dev, ve.data(), ve.size() * sizeof(ValueEmbed), hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) {
        (void)hipFree(base);
        return fail(NC_ERR_DEVICE, std::string("workspace setup: ") + hipGetErrorString(e));
    }
    kv->ws = w;
    return NC_OK;
}

nc_status check_cfg(const nc_config* c) {
    if (!c) return fail(NC_ERR_INVALID_ARG, "cfg is NULL");
    if (c->n_layer < 1 || c->d_model < 1 || c->n_head < 1 || c->head_dim < 1 || c->d_ff < 1 ||
        c->vocab < 1 || c->max_seq < 1)
        return fail(NC_ERR_INVALID_ARG, "all sizes must be positive");
    if (c->dtype != NC_F32 && c->dtype != NC_BF16) return fail(NC_ERR_INVALID_ARG, "dtype must be NC_F32 or NC_BF16");
    if (c->n_kv_head < 1 || c->n_head % c->n_kv_head)
        return fail(NC_ERR_INVALID_ARG, "n_kv_head must be >= 1 and divide n_head");
    if (c->n_head / c->n_kv_head > 16)
        return fail(NC_ERR_UNSUPPORTED, "more than 16 query heads per K/V head is not supported by the decode attention kernel");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(NC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if ((long long)c->n_head * c->head_dim != c->d_model) return fail(NC_ERR_INVALID_ARG, "d_model must equal n_head * head_dim");
    if (c->d_model % 64 || c->d_ff % 64) return fail(NC_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
    if (c->d_model > 4096) return fail(NC_ERR_UNSUPPORTED, "d_model > 4096 is not supported");
    if (!(c->softcap > 0.f) || !(c->norm_eps >= 0.f) || !(c->rope_base > 0.f))
        return fail(NC_ERR_INVALID_ARG, "softcap and rope_base must be > 0, norm_eps >= 0");
    if (c->max_seq > (1 << 24)) return fail(NC_ERR_INVALID_ARG, "max_seq too large");
    return NC_OK;
}

nc_status check_device(int* dev_out) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n < 1) return fail(NC_ERR_DEVICE, "no HIP device available");
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(NC_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", gfx950 required");
    *dev_out = dev;
    return NC_OK;
}

nc_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NC_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    return NC_OK;
}
#define LAUNCH(expr)                                \
    do {                                            \
        nc_status s_ = launched((expr), #expr);     \
        if (s_ != NC_OK) return s_;                 \
    } while (0)

// Launch `fn` (returning hipError_t); if kernel class `cls` is being timed, bracket it with
// an event pair on `st` that carries its algorithmic bytes and flops.
// `kernels` = number of kernels `fn` launches through NC_TLAUNCH (at most NC_MAX_STAMPS).
// Set while the allocation-free decode step enqueues: no timing events are created.
thread_local bool t_untimed = false;

template <typename F>
hipError_t timed(int cls, double bytes, double flops, hipStream_t st, F fn, int kernels = 1) {
    (void)st;
    if (g_tm.cls != cls || t_untimed) return fn();
    TimingPair tp = {};
    tp.bytes = bytes;
    tp.flops = flops;
    hipError_t e = hipSuccess;
    for (int i = 0; i < kernels && e == hipSuccess; ++i)
        for (int j = 0; j < 2 && e == hipSuccess; ++j) e = hipEventCreate(&tp.ev[i][j]);
    if (e == hipSuccess) {
        t_stamp = {};
        for (int i = 0; i < kernels; ++i) {
            t_stamp.ev[i][0] = tp.ev[i][0];
            t_stamp.ev[i][1] = tp.ev[i][1];
        }
        t_stamp.avail = kernels;
        e = fn();
        tp.n = t_stamp.used;
        t_stamp = {};
    }
    if (e != hipSuccess) {
        timing_release(tp);
        return e;
    }
    g_tm.pending.push_back(tp);
    return hipSuccess;
}

// (query, key) pairs a prefill of T tokens at positions off .. off + T - 1 attends to:
// sum over positions p of min(p + 1, w + 1) (w < 0: p + 1).
double visible_pairs(long long off, long long T, int w) {
    if (w < 0) return (double)T * off + (double)T * (T + 1) / 2.0;
    const long long n1 = std::min(std::max((long long)w - off, 0LL), T);  // positions p < w
    return (double)n1 * off + (double)n1 * (n1 + 1) / 2.0 + (double)(T - n1) * (w + 1.0);
}

// Algorithmic bytes of a decode projection: weights, activations (both parts of a
// compensated operand), and the epilogue's outputs (RESID also reads x; low parts where
// written); flops 2 M N K of the model (the extra MFMAs of the low part are not counted).
nc_status decode_gemm(nc_kv* kv, Epi epi, const DecGemmArgs& a, hipStream_t st, const DecFinishArgs* fin = nullptr) {
    const double es = (double)kv->m->esz, M = a.M, N = a.N, K = a.K;
    double out = 0;
    if (epi == EPI_STORE || epi == EPI_SOFTCAP) out = M * N * 4;
    else if (epi == EPI_RELU2) out = M * N * es;
    else out = M * N * (8 + es);
    if (a.out_lo) out += M * N * es;
    const double bytes = N * K * es + M * K * es * (a.A_lo ? 2 : 1) + out;
    LAUNCH(timed(NC_KC_DECODE_GEMM, bytes, 2 * M * N * K, st,
                 [&] { return launch_dec_gemm(kv->m->dt, epi, a, st, 0, fin); }, 2));
    return NC_OK;
}

// Prefill projection: flops 2 M N K of the model; bytes: A (and its one-byte e4m3 low part
// when compensated), weights and the outputs once (low parts one byte each).
hipError_t prefill_gemm(nc_model* m, Epi epi, const GemmArgs& g, hipStream_t st) {
    const double es = (double)m->esz, M = g.M, N = g.N, K = g.K;
    const double out = ((epi == EPI_STORE || epi == EPI_SOFTCAP) ? M * N * 4
                        : (epi == EPI_RELU2 ? M * N * es : M * N * (8 + es))) +
                       (g.out_lo ? M * N : 0);
    return timed(NC_KC_PREFILL_GEMM, M * K * es + (g.A_lo ? M * K : 0) + N * K * es + out, 2 * M * N * K, st,
                 [&] { return launch_gemm(m->dt, epi, g, st); });
}

// Embedding of M = B T token rows (positions lens[b] + t), with the later-version blocks'
// smear, x0 and layer-0 scaling when they are on.
EmbedArgs embed_args(nc_model* m, nc_kv* kv, const Ws& ws, const int32_t* tokens, int M, int T, bool blocked) {
    const nc_config& c = m->cfg;
    const nc_model::Extras& ex = m->ex;
    EmbedArgs e{};
    e.tok = tokens; e.M = M; e.T = T; e.wte = m->wte; e.vocab = c.vocab; e.d = c.d_model;
    e.eps = c.norm_eps; e.scale0 = 1.f;
    e.x = ws.x; e.act = ws.act; e.ss = ws.ss_a; e.blocked = blocked;
    e.lens = kv->lens_dev; e.hist = kv->hist; e.S = kv->S;
    if (ex.on) {
        e.scale0 = ex.lam[0] + ex.mu[0];
        e.x0 = ws.x0;
        if (ex.backout_layer == 0) e.xb = ws.xb;
        e.smear_gate = ex.smear_gate; e.smear_ch = ex.smear_ch; e.smear_lambda = ex.smear_lambda;
        e.tok_out = ws.tokbuf;
    }
    return e;
}

// Enqueue one decode step (everything after the host-side checks) on `st`.
nc_status enqueue_decode(nc_model* m, nc_kv* kv, const Ws& ws, const int32_t* tokens, float* logits, hipStream_t st) {
    const nc_config& c = m->cfg;
    const int B = kv->B;
    const int d = c.d_model, H = c.n_head, hd = c.head_dim, F = c.d_ff, V = c.vocab, nkv = c.n_kv_head;
    const int nqkv = (H + 2 * nkv) * hd;
    const size_t per_layer = (size_t)B * nkv * kv->S * hd * m->esz;
    const int parts_d = (d + dec_gemm_tile_n() - 1) / dec_gemm_tile_n();
    const int ss = (int)ws.cap_m;
    nc_status s;

    LAUNCH(launch_embed(m->dt, embed_args(m, kv, ws, tokens, B, 1, true), st));
    int ss_a_parts = 1;
    for (int l = 0; l < c.n_layer; ++l) {
        const nc_model::Layer& L = m->layers[l];
        void* kc = (char*)kv->kcache + l * per_layer;
        void* vtc = (char*)kv->vcache + l * per_layer;
        DecGemmArgs a{};
        a.M = B; a.eps = c.norm_eps; a.cap = c.softcap; a.ss_stride = ss; a.part = ws.dpart;
        // QKV product and its finish (norm scale, RoPE + QK-norm at lens[b], the query heads
        // to ws.q, the new key / value into the cache): for at most 32 rows in the product's
        // epilogue; otherwise the product leaves its K slices apart and the finish kernel
        // adds them
        a.A = ws.act; a.W = L.wqkv; a.N = nqkv; a.K = d;
        a.out_f32 = ws.qkv; a.ldo = nqkv;
        {
            const int sl = dec_gemm_store_slices(m->dt, B, nqkv, d);
            DecFinishArgs fa{};
            fa.part = sl ? ws.dpart + DEC_PART_CTRS : ws.qkv; fa.splits = sl ? sl : 1;
            fa.z_stride = (long long)B * nqkv;
            fa.ss_in = ws.ss_a; fa.ss_in_parts = ss_a_parts; fa.ss_stride = ss; fa.norm_dim = d;
            fa.eps = c.norm_eps; fa.lens = kv->lens_dev; fa.rope_cos = m->rope_cos; fa.rope_sin = m->rope_sin;
            fa.q = ws.q; fa.kc = kc; fa.vtc = vtc;
            fa.vemb = (m->ex.on && m->ex.ve[l]) ? ws.ve_dev + l : nullptr;
            fa.head_ctr = ws.fctr;
            fa.B = B; fa.H = H; fa.hd = hd; fa.nkv = nkv; fa.S = kv->S;
            if (dec_gemm_fuses_finish(m->dt, B, hd, H + 2 * nkv)) {
                if ((s = decode_gemm(kv, EPI_STORE, a, st, &fa)) != NC_OK) return s;
            } else {
                if ((s = decode_gemm(kv, EPI_STORE, a, st)) != NC_OK) return s;
                // timed with the projections: it also adds the product's K slices (bytes: the
                // raw product read once, q / k / v written)
                LAUNCH(timed(NC_KC_DECODE_GEMM, (double)B * nqkv * (4 + m->esz), 0, st,
                             [&] { return launch_qkv_finish_decode(m->dt, fa, st); }));
            }
        }
        // attention over the cache
        DecAttnArgs at{};
        at.q = ws.q; at.lens = kv->lens_dev; at.kc = kc; at.vtc = vtc; at.part = ws.apart; at.flags = ws.actr;
        at.y = ws.y;
        at.B = B; at.H = H; at.hd = hd; at.S = kv->S; at.nkv = nkv; at.max_slots = ws.apart_slots;
        at.window = m->windows[l];
        {   // bytes: the K/V read for every row (its visible positions, the new one
            // included) of each K/V head, q in and y out; flops 4 hd per (query head, key) pair
            const double es = (double)m->esz;
            double keys = 0;
            for (int b = 0; b < B; ++b)
                keys += at.window < 0 ? kv->lens_host[b] + 1 : std::min(kv->lens_host[b], at.window) + 1;
            const double by = keys * nkv * hd * 2 * es + 2.0 * B * H * hd * es;
            LAUNCH(timed(NC_KC_DECODE_ATTN, by, 4.0 * H * hd * keys, st,
                         [&] { return launch_attn_decode(m->dt, at, st); }));
        }
        // O + residual
        DecGemmArgs o = a;
        o.A = ws.y; o.W = L.wo; o.N = d; o.K = H * hd;
        o.out_f32 = ws.x; o.out_t = ws.act; o.ldo = d; o.ss_out = ws.ss_b;
        o.out_lo = ws.act_lo;
        if ((s = decode_gemm(kv, EPI_RESID, o, st)) != NC_OK) return s;
        // FC + norm scale + relu^2 (compensated operand)
        DecGemmArgs f = a;
        f.A = ws.act; f.A_lo = ws.act_lo; f.W = L.wfc; f.N = F; f.K = d;
        f.out_t = ws.u; f.out_lo = ws.u_lo; f.ldo = F; f.ss_in = ws.ss_b; f.ss_in_parts = parts_d;
        if ((s = decode_gemm(kv, EPI_RELU2, f, st)) != NC_OK) return s;
        // PROJ + residual (compensated operand)
        DecGemmArgs pj = a;
        pj.A = ws.u; pj.A_lo = ws.u_lo; pj.W = L.wproj; pj.N = d; pj.K = F;
        pj.out_f32 = ws.x; pj.out_t = ws.act; pj.ldo = d; pj.ss_out = ws.ss_a;
        pj.rx = m->ex.on ? ws.rx_dev + l : nullptr;
        if (l == c.n_layer - 1) pj.out_lo = ws.act_lo;  // the LM head's operand is compensated
        if ((s = decode_gemm(kv, EPI_RESID, pj, st)) != NC_OK) return s;
        ss_a_parts = parts_d;
    }
    DecGemmArgs h{};
    h.M = B; h.eps = c.norm_eps; h.cap = c.softcap; h.ss_stride = ss; h.part = ws.dpart;
    h.A = ws.act; h.A_lo = ws.act_lo; h.W = m->lm; h.N = V; h.K = d;
    h.out_f32 = logits; h.ldo = V; h.ss_in = ws.ss_a; h.ss_in_parts = ss_a_parts;
    h.lens_inc = kv->lens_dev;  // the step's last kernel also advances every row by one
    if ((s = decode_gemm(kv, EPI_SOFTCAP, h, st)) != NC_OK) return s;
    return NC_OK;
}

}  // namespace

extern "C" {

int32_t nc_abi_version(void) { return NC_ABI_VERSION; }

const char* nc_last_error(void) { return g_err.c_str(); }

nc_status nc_model_create(const nc_config* cfg, const void* const* weights, nc_model** out) {
    try {
        if (!out) return fail(NC_ERR_INVALID_ARG, "out is NULL");
        *out = nullptr;
        nc_status s = check_cfg(cfg);
        if (s != NC_OK) return s;
        if (!weights) return fail(NC_ERR_INVALID_ARG, "weights is NULL");
        const int nw = 6 * cfg->n_layer + 2;
        for (int i = 0; i < nw; ++i)
            if (!weights[i]) return fail(NC_ERR_INVALID_ARG, "weight pointer " + std::to_string(i) + " is NULL");
        int dev = 0;
        s = check_device(&dev);
        if (s != NC_OK) return s;
        for (int i = 0; i < nw; ++i) {  // kernels read the weights directly: device memory only
            hipPointerAttribute_t attr;
            if (hipPointerGetAttributes(&attr, weights[i]) != hipSuccess ||
                (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)) {
                (void)hipGetLastError();
                return fail(NC_ERR_INVALID_ARG, "weight pointer " + std::to_string(i) + " is not device memory");
            }
        }

        nc_model* m = new nc_model();
        m->cfg = *cfg;
        m->windows.assign(cfg->n_layer, -1);
        m->dt = cfg->dtype == NC_BF16 ? BF16 : F32;
        m->esz = cfg->dtype == NC_BF16 ? 2 : 4;
        m->device = dev;
        const size_t d = cfg->d_model, hd = cfg->head_dim, H = cfg->n_head, V = cfg->vocab, F = cfg->d_ff;
        const size_t nkv = cfg->n_kv_head;
        const size_t es = m->esz;
        // projection weights are stored MFMA-blocked (kernels.h); the embedding stays row-major
        const size_t sz_emb = align_up(V * d * es, 256);
        const size_t sz_qkv = align_up((size_t)blocked_elems((int)((H + 2 * nkv) * hd), (int)d) * es, 256);
        const size_t sz_o = align_up((size_t)blocked_elems((int)d, (int)(H * hd)) * es, 256);
        const size_t sz_fc = align_up((size_t)blocked_elems((int)F, (int)d) * es, 256);
        const size_t sz_pj = align_up((size_t)blocked_elems((int)d, (int)F) * es, 256);
        const size_t sz_lm = align_up((size_t)blocked_elems((int)V, (int)d) * es, 256);
        const size_t total = sz_emb + sz_lm + cfg->n_layer * (sz_qkv + sz_o + sz_fc + sz_pj);
        hipError_t e = hipMalloc(&m->arena, total);
        if (e != hipSuccess) {
            delete m;
            return fail(NC_ERR_OOM, std::string("weight arena: ") + hipGetErrorString(e));
        }
        char* p = (char*)m->arena;
        hipError_t ce = hipMemcpy(p, weights[0], V * d * es, hipMemcpyDefault);
        m->wte = p;
        p += sz_emb;
        m->layers.resize(cfg->n_layer);
        const size_t qrows_bytes = (size_t)blocked_elems((int)(H * hd), (int)d) * es;  // H*hd is a multiple of 32
        const size_t krows_bytes = (size_t)blocked_elems((int)(nkv * hd), (int)d) * es;  // hd is too
        for (int l = 0; l < cfg->n_layer && ce == hipSuccess; ++l) {
            const void* const* w = weights + 1 + 6 * l;
            nc_model::Layer& L = m->layers[l];
            L.wqkv = p;
            ce = launch_repack(m->dt, w[0], p, (int)(H * hd), (int)d, 0);
            if (ce == hipSuccess) ce = launch_repack(m->dt, w[1], p + qrows_bytes, (int)(nkv * hd), (int)d, 0);
            if (ce == hipSuccess)
                ce = launch_repack(m->dt, w[2], p + qrows_bytes + krows_bytes, (int)(nkv * hd), (int)d, 0);
            p += sz_qkv;
            L.wo = p;
            if (ce == hipSuccess) ce = launch_repack(m->dt, w[3], p, (int)d, (int)(H * hd), 0);
            p += sz_o;
            L.wfc = p;
            if (ce == hipSuccess) ce = launch_repack(m->dt, w[4], p, (int)F, (int)d, 0);
            p += sz_fc;
            L.wproj = p;
            if (ce == hipSuccess) ce = launch_repack(m->dt, w[5], p, (int)d, (int)F, 0);
            p += sz_pj;
        }
        if (ce == hipSuccess) ce = launch_repack(m->dt, weights[nw - 1], p, (int)V, (int)d, 0);
        m->lm = p;
        if (ce == hipSuccess && m->dt == BF16) {
            // largest |w| of the compensated products' weights (MLP and LM head): the exponent
            // of their e4m3 copies in the prefill's low-part product
            const int L = cfg->n_layer;
            unsigned* amax = nullptr;
            ce = hipMalloc((void**)&amax, (2 * L + 1) * sizeof(unsigned));
            if (ce == hipSuccess) ce = hipMemset(amax, 0, (2 * L + 1) * sizeof(unsigned));
            for (int l = 0; l < L && ce == hipSuccess; ++l) {
                const void* const* w = weights + 1 + 6 * l;
                ce = launch_absmax(w[4], (long long)F * d, amax + 2 * l, 0);
                if (ce == hipSuccess) ce = launch_absmax(w[5], (long long)d * F, amax + 2 * l + 1, 0);
            }
            if (ce == hipSuccess) ce = launch_absmax(weights[nw - 1], (long long)V * d, amax + 2 * L, 0);
            std::vector<unsigned> h(2 * L + 1, 0);
            if (ce == hipSuccess) ce = hipMemcpy(h.data(), amax, h.size() * sizeof(unsigned), hipMemcpyDeviceToHost);
            if (amax) (void)hipFree(amax);
            auto as_float = [](unsigned u) { float f; std::memcpy(&f, &u, 4); return f; };
            for (int l = 0; l < L && ce == hipSuccess; ++l) {
                m->layers[l].e8_fc = lo8_weight_exp(as_float(h[2 * l]));
                m->layers[l].e8_proj = lo8_weight_exp(as_float(h[2 * l + 1]));
            }
            m->e8_lm = lo8_weight_exp(as_float(h[2 * L]));
        }
        if (ce == hipSuccess) ce = hipDeviceSynchronize();
        // RoPE tables: angle p * base^(-2i/hd), evaluated in double, stored fp32.
        const size_t half = hd / 2, S = cfg->max_seq;
        std::vector<float> hc(S * half), hs(S * half);
        for (size_t i = 0; i < half; ++i) {
            const double inv = std::pow((double)cfg->rope_base, -2.0 * (double)i / (double)hd);
            for (size_t t = 0; t < S; ++t) {
                const double a = (double)t * inv;
                hc[t * half + i] = (float)std::cos(a);
                hs[t * half + i] = (float)std::sin(a);
            }
        }
        if (ce == hipSuccess) ce = hipMalloc((void**)&m->rope_cos, S * half * 4);
        if (ce == hipSuccess) ce = hipMalloc((void**)&m->rope_sin, S * half * 4);
        if (ce == hipSuccess) ce = hipMemcpy(m->rope_cos, hc.data(), S * half * 4, hipMemcpyHostToDevice);
        if (ce == hipSuccess) ce = hipMemcpy(m->rope_sin, hs.data(), S * half * 4, hipMemcpyHostToDevice);
        if (ce != hipSuccess) {
            nc_model_free(m);
            return fail(ce == hipErrorOutOfMemory ? NC_ERR_OOM : NC_ERR_DEVICE,
                        std::string("model upload: ") + hipGetErrorString(ce));
        }
        *out = m;
        return NC_OK;
    } catch (const std::bad_alloc&) {
        return fail(NC_ERR_OOM, "host allocation failed");
    } catch (...) {
        return fail(NC_ERR_DEVICE, "unexpected exception");
    }
}

namespace {
void extras_free(nc_model::Extras& ex) {
    if (ex.smear_gate) (void)hipFree(ex.smear_gate);
    for (void* p : ex.ve)
        if (p) (void)hipFree(p);
    for (void* p : ex.ve_gate)
        if (p) (void)hipFree(p);
    ex = nc_model::Extras{};
}

bool is_device_ptr(const void* p) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

// Library-owned copy of `bytes` of device memory.
hipError_t dev_copy(const void* src, size_t bytes, void** dst) {
    hipError_t e = hipMalloc(dst, bytes);
    if (e == hipSuccess) e = hipMemcpy(*dst, src, bytes, hipMemcpyDeviceToDevice);
    return e;
}
}  // namespace

void nc_model_free(nc_model* m) {
    if (!m) return;
    (void)hipDeviceSynchronize();
    extras_free(m->ex);
    if (m->arena) (void)hipFree(m->arena);
    if (m->rope_cos) (void)hipFree(m->rope_cos);
    if (m->rope_sin) (void)hipFree(m->rope_sin);
    delete m;
}

nc_status nc_model_set_windows(nc_model* m, const int32_t* windows) {
    try {
        if (!m || !windows) return fail(NC_ERR_INVALID_ARG, "NULL argument");
        if (m->live_kv != 0) return fail(NC_ERR_STATE, "windows can only change while the model has no kv object");
        std::vector<int> w(windows, windows + m->cfg.n_layer);
        for (int& x : w) x = x < 0 ? -1 : x;
        m->windows = std::move(w);
        return NC_OK;
    } catch (const std::bad_alloc&) {
        return fail(NC_ERR_OOM, "host allocation failed");
    }
}

nc_status nc_model_set_extras(nc_model* m, const nc_extras* x) {
    try {
        if (!m) return fail(NC_ERR_INVALID_ARG, "model is NULL");
        if (m->live_kv != 0) return fail(NC_ERR_STATE, "extras can only change while the model has no kv object");
        const nc_config& c = m->cfg;
        const int L = c.n_layer, lim = std::min(64, c.d_model);
        if (x) {
            if (x->smear_gate_dev && (x->smear_channels < 1 || x->smear_channels > lim))
                return fail(NC_ERR_INVALID_ARG, "smear_channels must be in [1, min(64, d_model)]");
            if (x->backout_layer < -1 || x->backout_layer >= L) return fail(NC_ERR_INVALID_ARG, "backout_layer out of range");
            if (x->smear_gate_dev && !is_device_ptr(x->smear_gate_dev))
                return fail(NC_ERR_INVALID_ARG, "smear_gate_dev is not device memory");
            if (x->ve_dev) {
                if (!x->ve_gate_dev) return fail(NC_ERR_INVALID_ARG, "ve_gate_dev is NULL");
                bool any = false;
                for (int l = 0; l < L; ++l) {
                    if (!x->ve_dev[l]) continue;
                    any = true;
                    if (!is_device_ptr(x->ve_dev[l]) || !x->ve_gate_dev[l] || !is_device_ptr(x->ve_gate_dev[l]))
                        return fail(NC_ERR_INVALID_ARG, "value embedding of layer " + std::to_string(l) +
                                                            ": table or gate is not device memory");
                }
                if (any && (x->ve_channels < 1 || x->ve_channels > lim))
                    return fail(NC_ERR_INVALID_ARG, "ve_channels must be in [1, min(64, d_model)]");
            }
        }
        (void)hipDeviceSynchronize();
        extras_free(m->ex);
        if (!x) return NC_OK;
        nc_model::Extras& ex = m->ex;
        ex.on = true;
        ex.lam.assign(L, 1.f);
        ex.mu.assign(L, 0.f);
        if (x->resid_lambda_host) ex.lam.assign(x->resid_lambda_host, x->resid_lambda_host + L);
        if (x->x0_lambda_host) ex.mu.assign(x->x0_lambda_host, x->x0_lambda_host + L);
        ex.backout_layer = x->backout_layer;
        ex.backout_lambda = x->backout_lambda;
        ex.ve.assign(L, nullptr);
        ex.ve_gate.assign(L, nullptr);
        hipError_t e = hipSuccess;
        if (x->smear_gate_dev) {
            ex.smear_ch = x->smear_channels;
            ex.smear_lambda = x->smear_lambda;
            e = dev_copy(x->smear_gate_dev, (size_t)ex.smear_ch * m->esz, &ex.smear_gate);
        }
        if (x->ve_dev) {
            ex.ve_ch = x->ve_channels;
            const size_t tb = (size_t)c.vocab * c.n_kv_head * c.head_dim * m->esz;
            const size_t gb = (size_t)c.n_kv_head * ex.ve_ch * m->esz;
            for (int l = 0; l < L && e == hipSuccess; ++l) {
                if (!x->ve_dev[l]) continue;
                e = dev_copy(x->ve_dev[l], tb, &ex.ve[l]);
                if (e == hipSuccess) e = dev_copy(x->ve_gate_dev[l], gb, &ex.ve_gate[l]);
            }
        }
        if (e != hipSuccess) {
            extras_free(m->ex);
            return fail(e == hipErrorOutOfMemory ? NC_ERR_OOM : NC_ERR_DEVICE,
                        std::string("extras copy: ") + hipGetErrorString(e));
        }
        return NC_OK;
    } catch (const std::bad_alloc&) {
        extras_free(m->ex);
        return fail(NC_ERR_OOM, "host allocation failed");
    }
}

nc_status nc_kv_create(nc_model* m, int32_t batch, int32_t max_seq, nc_kv** out) {
    try {
        if (!out) return fail(NC_ERR_INVALID_ARG, "out is NULL");
        *out = nullptr;
        if (!m) return fail(NC_ERR_INVALID_ARG, "model is NULL");
        if (batch < 1 || max_seq < 1) return fail(NC_ERR_INVALID_ARG, "batch and max_seq must be >= 1");
        if (max_seq > m->cfg.max_seq) return fail(NC_ERR_INVALID_ARG, "max_seq exceeds the model's max_seq");
        if (max_seq > 32768) return fail(NC_ERR_UNSUPPORTED, "cache capacity above 32768 positions is not supported");
        nc_kv* kv = new nc_kv();
        kv->m = m;
        kv->B = batch;
        kv->max_seq = max_seq;
        kv->S = (int)align_up(max_seq, 64);
        kv->lens_host.assign(batch, 0);
        const char* ng = std::getenv("NC_DECODE_GRAPH");
        kv->use_graph = !(ng && ng[0] == '0');
        const nc_config& c = m->cfg;
        const size_t bytes = (size_t)c.n_layer * batch * c.n_kv_head * kv->S * c.head_dim * m->esz;
        hipError_t e = hipMalloc(&kv->kcache, bytes);
        if (e == hipSuccess) e = hipMalloc(&kv->vcache, bytes);
        if (e == hipSuccess) e = hipMalloc((void**)&kv->lens_dev, batch * sizeof(int32_t));
        if (e == hipSuccess) e = hipMemset(kv->kcache, 0, bytes);
        if (e == hipSuccess) e = hipMemset(kv->vcache, 0, bytes);
        if (e == hipSuccess) e = hipMemset(kv->lens_dev, 0, batch * sizeof(int32_t));
        if (e == hipSuccess && m->ex.smear_gate) {
            e = hipMalloc((void**)&kv->hist, (size_t)batch * kv->S * sizeof(int32_t));
            if (e == hipSuccess) e = hipMemset(kv->hist, 0, (size_t)batch * kv->S * sizeof(int32_t));
        }
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            if (kv->kcache) (void)hipFree(kv->kcache);
            if (kv->vcache) (void)hipFree(kv->vcache);
            if (kv->lens_dev) (void)hipFree(kv->lens_dev);
            if (kv->hist) (void)hipFree(kv->hist);
            delete kv;
            return fail(e == hipErrorOutOfMemory ? NC_ERR_OOM : NC_ERR_DEVICE,
                        std::string("kv allocation: ") + hipGetErrorString(e));
        }
        m->live_kv++;
        *out = kv;
        return NC_OK;
    } catch (const std::bad_alloc&) {
        return fail(NC_ERR_OOM, "host allocation failed");
    } catch (...) {
        return fail(NC_ERR_DEVICE, "unexpected exception");
    }
}

void nc_kv_free(nc_kv* kv) {
    if (!kv) return;
    (void)hipDeviceSynchronize();
    ws_free(kv);
    if (kv->cap_stream) (void)hipStreamDestroy(kv->cap_stream);
    if (kv->kcache) (void)hipFree(kv->kcache);
    if (kv->vcache) (void)hipFree(kv->vcache);
    if (kv->lens_dev) (void)hipFree(kv->lens_dev);
    if (kv->hist) (void)hipFree(kv->hist);
    kv->m->live_kv--;
    delete kv;
}

nc_status nc_kv_set_lens(nc_kv* kv, const int32_t* lens) {
    if (!kv || !lens) return fail(NC_ERR_INVALID_ARG, "NULL argument");
    for (int b = 0; b < kv->B; ++b)
        if (lens[b] < 0 || lens[b] > kv->lens_host[b])
            return fail(NC_ERR_INVALID_ARG, "lens may only shrink (0 <= new <= current)");
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipMemcpy(kv->lens_dev, lens, kv->B * sizeof(int32_t), hipMemcpyHostToDevice));
    std::copy(lens, lens + kv->B, kv->lens_host.begin());
    return NC_OK;
}

nc_status nc_kv_get_lens(const nc_kv* kv, int32_t* lens) {
    if (!kv || !lens) return fail(NC_ERR_INVALID_ARG, "NULL argument");
    std::copy(kv->lens_host.begin(), kv->lens_host.end(), lens);
    return NC_OK;
}

nc_status nc_kv_export(nc_kv* kv, int32_t layer, void* k_out, void* v_out, void* stream) {
    if (!kv || !k_out || !v_out) return fail(NC_ERR_INVALID_ARG, "NULL argument");
    const nc_config& c = kv->m->cfg;
    if (layer < 0 || layer >= c.n_layer) return fail(NC_ERR_INVALID_ARG, "layer out of range");
    const size_t per_layer = (size_t)kv->B * c.n_kv_head * kv->S * c.head_dim * kv->m->esz;
    const char* kc = (const char*)kv->kcache + layer * per_layer;
    const char* vc = (const char*)kv->vcache + layer * per_layer;
    // the cache is [B][n_kv_head][...] per layer: export (row, K/V head) pairs as rows
    LAUNCH(launch_kv_export(kv->m->dt, c.head_dim, kc, vc, k_out, v_out, kv->B * c.n_kv_head, kv->S, kv->max_seq,
                            (hipStream_t)stream));
    return NC_OK;
}

nc_status nc_sample(const float* logits, int32_t B, int32_t V, float temperature, int32_t top_k,
                    const float* u, int32_t* out, void* stream) {
    if (!logits || !out) return fail(NC_ERR_INVALID_ARG, "NULL argument");
    if (B < 1 || V < 1) return fail(NC_ERR_INVALID_ARG, "B and V must be >= 1");
    if (!(temperature > 0.f)) {
        LAUNCH(launch_argmax(logits, B, V, out, (hipStream_t)stream));
        return NC_OK;
    }
    if (!u) return fail(NC_ERR_INVALID_ARG, "u is NULL");
    if (V > (1 << 20)) return fail(NC_ERR_UNSUPPORTED, "sampling supports V <= 2^20");
    const double scale = 1.4426950408889634 / (double)temperature;
    if (!(scale < 3.0e38)) return fail(NC_ERR_INVALID_ARG, "temperature too small");
    LAUNCH(launch_sample(logits, B, V, (float)scale, top_k, u, out, (hipStream_t)stream));
    return NC_OK;
}

nc_status nc_kv_copy_rows(nc_kv* dst, const int32_t* dst_rows, nc_kv* src, const int32_t* src_rows,
                          int32_t n, void* stream) {
    try {
        if (!dst || !src) return fail(NC_ERR_INVALID_ARG, "NULL argument");
        if (dst->m != src->m) return fail(NC_ERR_INVALID_ARG, "the caches belong to different models");
        if (n < 0) return fail(NC_ERR_INVALID_ARG, "n must be >= 0");
        if (n == 0) return NC_OK;
        if (!dst_rows || !src_rows) return fail(NC_ERR_INVALID_ARG, "NULL row list");
        std::vector<char> is_dst(dst->B, 0);
        for (int i = 0; i < n; ++i) {
            if (dst_rows[i] < 0 || dst_rows[i] >= dst->B || src_rows[i] < 0 || src_rows[i] >= src->B)
                return fail(NC_ERR_INVALID_ARG, "row index out of range");
            if (is_dst[dst_rows[i]]) return fail(NC_ERR_INVALID_ARG, "a destination row appears twice");
            is_dst[dst_rows[i]] = 1;
            if (src->lens_host[src_rows[i]] > dst->max_seq)
                return fail(NC_ERR_CAPACITY, "a source row is longer than the destination's max_seq");
        }
        if (dst == src)
            for (int i = 0; i < n; ++i)
                if (is_dst[src_rows[i]]) return fail(NC_ERR_INVALID_ARG, "a row is both a source and a destination");
        const nc_config& c = dst->m->cfg;
        hipStream_t st = (hipStream_t)stream;
        for (int i0 = 0; i0 < n; i0 += KvRowCopy::MAX) {
            KvRowCopy rc{};
            rc.n = std::min(n - i0, KvRowCopy::MAX);
            for (int i = 0; i < rc.n; ++i) {
                rc.dst[i] = dst_rows[i0 + i];
                rc.src[i] = src_rows[i0 + i];
                rc.len[i] = src->lens_host[src_rows[i0 + i]];
            }
            LAUNCH(launch_kv_copy_rows(rc, src->kcache, src->vcache, dst->kcache, dst->vcache, c.n_layer,
                                       c.n_kv_head, c.head_dim, (int)dst->m->esz, src->B, src->S, dst->B,
                                       dst->S, dst->lens_dev, src->hist, dst->hist, st));
        }
        for (int i = 0; i < n; ++i) dst->lens_host[dst_rows[i]] = src->lens_host[src_rows[i]];
        return NC_OK;
    } catch (const std::bad_alloc&) {
        return fail(NC_ERR_OOM, "host allocation failed");
    } catch (...) {
        return fail(NC_ERR_DEVICE, "unexpected exception");
    }
}

nc_status nc_argmax(const float* logits, int32_t B, int32_t V, int32_t* out, void* stream) {
    if (!logits || !out) return fail(NC_ERR_INVALID_ARG, "NULL argument");
    if (B < 1 || V < 1) return fail(NC_ERR_INVALID_ARG, "B and V must be >= 1");
    LAUNCH(launch_argmax(logits, B, V, out, (hipStream_t)stream));
    return NC_OK;
}

nc_status nc_prefill(nc_model* m, const int32_t* tokens, int32_t B, int32_t T, nc_kv* kv,
                     float* logits, void* stream) {
    try {
        if (!m || !tokens || !kv) return fail(NC_ERR_INVALID_ARG, "NULL argument");
        if (kv->m != m) return fail(NC_ERR_INVALID_ARG, "kv belongs to another model");
        if (B != kv->B) return fail(NC_ERR_INVALID_ARG, "B differs from the cache's batch");
        if (T < 1) return fail(NC_ERR_INVALID_ARG, "T must be >= 1");
        for (int b = 0; b < B; ++b)
            if ((long long)kv->lens_host[b] + T > kv->max_seq)
                return fail(NC_ERR_CAPACITY, "a row's length + T exceeds the cache's max_seq");
        const long long M = (long long)B * T;
        nc_status s = ws_ensure(kv, M);
        if (s != NC_OK) return s;
        hipStream_t st = (hipStream_t)stream;
        const nc_config& c = m->cfg;
        const int d = c.d_model, H = c.n_head, hd = c.head_dim, F = c.d_ff, V = c.vocab, nkv = c.n_kv_head;
        const int nqkv = (H + 2 * nkv) * hd;
        const int tn = gemm_tile_n();
        const int parts_d = (d + tn - 1) / tn;
        const size_t per_layer = (size_t)B * nkv * kv->S * hd * m->esz;
        const int Mi = (int)M;

        // bf16 activations of prefill are stored blocked, the layout the products read
        LAUNCH(launch_embed(m->dt, embed_args(m, kv, kv->ws, tokens, Mi, T, m->dt == BF16), st));
        int ss_a_parts = 1;
        for (int l = 0; l < c.n_layer; ++l) {
            const nc_model::Layer& L = m->layers[l];
            GemmArgs g{};
            g.M = Mi; g.lda = d; g.k_split = 1; g.eps = c.norm_eps; g.cap = c.softcap;
            g.tail_part = kv->ws.tpart; g.tail_ctr = kv->ws.tctr;
            // QKV raw product
            g.A = kv->ws.act; g.B = L.wqkv; g.N = nqkv; g.K = d; g.Npad = nqkv;
            g.out_f32 = kv->ws.qkv; g.ldo = nqkv; g.z_stride = 0;
            LAUNCH(prefill_gemm(m, EPI_STORE, g, st));
            QkvPostArgs qa{};
            qa.part = kv->ws.qkv; qa.splits = 1; qa.z_stride = 0; qa.M = Mi; qa.T = T; qa.H = H; qa.hd = hd; qa.nkv = nkv;
            qa.ss_in = kv->ws.ss_a; qa.ss_in_parts = ss_a_parts; qa.ss_stride = (int)kv->ws.cap_m; qa.norm_dim = d;
            qa.lens = kv->lens_dev; qa.rope_cos = m->rope_cos; qa.rope_sin = m->rope_sin;
            qa.q = kv->ws.q; qa.kc = (char*)kv->kcache + l * per_layer; qa.vtc = (char*)kv->vcache + l * per_layer;
            qa.S = kv->S; qa.eps = c.norm_eps;
            qa.vemb = value_embed(m, kv->ws, l);
            LAUNCH(launch_qkv_post(m->dt, qa, st));
            {   // causal attention flops: 4 hd per visible (query, key) pair and head; bytes:
                // q in, y out, and every key/value a query of the row sees, read once
                const int w = m->windows[l];
                double vis = 0, keys = 0;
                for (int b = 0; b < B; ++b) {
                    const long long off = kv->lens_host[b];
                    vis += visible_pairs(off, T, w);
                    keys += (double)(off + T - (w < 0 ? 0 : std::max(0LL, off - w)));
                }
                const double fl = 4.0 * H * hd * vis;
                const double by = ((double)B * T * 2 * H + keys * 2 * nkv) * hd * m->esz;
                LAUNCH(timed(NC_KC_PREFILL_ATTN, by, fl, st, [&] {
                    return launch_attn_prefill(m->dt, hd, kv->ws.q, qa.kc, qa.vtc, kv->ws.y, B, T, H, nkv, kv->S, w,
                                               kv->lens_dev, st);
                }));
            }
            // O product + residual
            g.A = kv->ws.y; g.lda = H * hd; g.B = L.wo; g.N = d; g.K = H * hd; g.Npad = d;
            g.out_f32 = kv->ws.x; g.out_t = kv->ws.act; g.ldo = d; g.ss_out = kv->ws.ss_b; g.ss_stride = (int)kv->ws.cap_m;
            g.A_lo = nullptr; g.out_lo = kv->ws.act_lo;
            LAUNCH(prefill_gemm(m, EPI_RESID, g, st));
            // FC + norm + relu^2 (compensated operand)
            g.A = kv->ws.act; g.lda = d; g.B = L.wfc; g.N = F; g.K = d; g.Npad = F;
            g.out_t = kv->ws.u; g.ldo = F; g.ss_in = kv->ws.ss_b; g.ss_in_parts = parts_d; g.ss_stride = (int)kv->ws.cap_m;
            g.A_lo = kv->ws.act_lo; g.out_lo = kv->ws.u_lo; g.w8_exp = L.e8_fc;
            LAUNCH(prefill_gemm(m, EPI_RELU2, g, st));
            // PROJ + residual (compensated operand)
            g.A = kv->ws.u; g.lda = F; g.B = L.wproj; g.N = d; g.K = F; g.Npad = d;
            g.out_f32 = kv->ws.x; g.out_t = kv->ws.act; g.ldo = d; g.ss_out = kv->ws.ss_a; g.ss_stride = (int)kv->ws.cap_m;
            g.A_lo = kv->ws.u_lo; g.w8_exp = L.e8_proj;
            g.out_lo = (l == c.n_layer - 1) ? kv->ws.act_lo : nullptr;  // LM head operand, compensated
            g.rx = proj_resid_extra(m, kv->ws, l);
            LAUNCH(prefill_gemm(m, EPI_RESID, g, st));
            g.A_lo = nullptr;
            g.rx = ResidExtra{};
            ss_a_parts = parts_d;
        }
        if (logits) {
            GemmArgs g{};
            g.A = kv->ws.act; g.A_lo = kv->ws.act_lo; g.w8_exp = m->e8_lm; g.lda = d; g.B = m->lm; g.M = Mi; g.N = V; g.K = d;
            g.Npad = (V + 31) / 32 * 32; g.k_split = 1;
            g.tail_part = kv->ws.tpart; g.tail_ctr = kv->ws.tctr;
            g.out_f32 = logits; g.ldo = V; g.ss_in = kv->ws.ss_a; g.ss_in_parts = ss_a_parts;
            g.ss_stride = (int)kv->ws.cap_m; g.eps = c.norm_eps; g.cap = c.softcap;
            LAUNCH(prefill_gemm(m, EPI_SOFTCAP, g, st));
        }
        LAUNCH(launch_lens_add(kv->lens_dev, B, T, -1, st));
        for (int32_t& n : kv->lens_host) n += T;
        return NC_OK;
    } catch (...) {
        return fail(NC_ERR_DEVICE, "unexpected exception");
    }
}

}  // extern "C"

namespace {
// One decode step, with the greedy picks of its logits into `next` when next is not null,
// eager or as a replay of the graph captured for (tokens, logits, next).
nc_status decode_impl(nc_model* m, const int32_t* tokens, int32_t B, nc_kv* kv, float* logits,
                      int32_t* next, void* stream) {
    try {
        if (!m || !tokens || !kv || !logits) return fail(NC_ERR_INVALID_ARG, "NULL argument");
        if (kv->m != m) return fail(NC_ERR_INVALID_ARG, "kv belongs to another model");
        if (B != kv->B) return fail(NC_ERR_INVALID_ARG, "B differs from the cache's batch");
        if (B > 128) return fail(NC_ERR_UNSUPPORTED, "decode supports at most 128 rows");
        for (int b = 0; b < B; ++b)
            if (kv->lens_host[b] + 1 > kv->max_seq) return fail(NC_ERR_CAPACITY, "a row is full (lens + 1 > max_seq)");
        nc_status s = ws_ensure(kv, B);
        if (s != NC_OK) return s;
        hipStream_t st = (hipStream_t)stream;
        auto enqueue = [&](hipStream_t q) {
            nc_status r = enqueue_decode(m, kv, kv->ws, tokens, logits, q);
            if (r == NC_OK && next) {
                const hipError_t e = launch_argmax(logits, B, m->cfg.vocab, next, q);
                if (e != hipSuccess) r = fail(NC_ERR_DEVICE, std::string("argmax: ") + hipGetErrorString(e));
            }
            return r;
        };
        if (!kv->use_graph || g_tm.cls != NC_KC_NONE) {
            s = enqueue(st);
        } else {
            hipGraphExec_t exec = nullptr;
            for (const nc_kv::Graph& g : kv->graphs)
                if (g.tokens == tokens && g.logits == logits && g.next == next) {
                    exec = g.exec;
                    break;
                }
            if (!exec) {
                if (!kv->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&kv->cap_stream, hipStreamNonBlocking));
                HIP_TRY(hipStreamBeginCapture(kv->cap_stream, hipStreamCaptureModeThreadLocal));
                s = enqueue(kv->cap_stream);
                hipGraph_t graph = nullptr;
                hipError_t e = hipStreamEndCapture(kv->cap_stream, &graph);
                if (s != NC_OK || e != hipSuccess) {
                    if (graph) (void)hipGraphDestroy(graph);
                    if (s != NC_OK) return s;
                }
                if (e != hipSuccess) return fail(NC_ERR_DEVICE, std::string("decode capture: ") + hipGetErrorString(e));
                e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
                (void)hipGraphDestroy(graph);
                if (e != hipSuccess) {
                    return fail(NC_ERR_DEVICE, std::string("graph instantiate: ") + hipGetErrorString(e));
                }
                if (kv->graphs.size() >= 8) {  // keep a handful of buffer pairs
                    // the oldest graph may still be queued or running on some stream:
                    // let the device drain before its executable is destroyed
                    e = hipDeviceSynchronize();
                    if (e != hipSuccess) {
                        (void)hipGraphExecDestroy(exec);
                        return fail(NC_ERR_DEVICE, std::string("graph eviction: ") + hipGetErrorString(e));
                    }
                    drop_graph(kv->graphs.front());
                    kv->graphs.erase(kv->graphs.begin());
                }
                kv->graphs.push_back({tokens, logits, next, exec});
            }
            HIP_TRY(hipGraphLaunch(exec, st));
        }
        if (s != NC_OK) return s;
        for (int b = 0; b < B; ++b) kv->lens_host[b] += 1;
        return NC_OK;
    } catch (...) {
        return fail(NC_ERR_DEVICE, "unexpected exception");
    }
}
}  // namespace

extern "C" {

nc_status nc_decode_step(nc_model* m, const int32_t* tokens, int32_t B, nc_kv* kv, float* logits,
                         void* stream) {
    return decode_impl(m, tokens, B, kv, logits, nullptr, stream);
}

nc_status nc_decode_greedy(nc_model* m, const int32_t* tokens, int32_t B, nc_kv* kv, float* logits,
                           int32_t* next, void* stream) {
    if (!next) return fail(NC_ERR_INVALID_ARG, "next is NULL");
    return decode_impl(m, tokens, B, kv, logits, next, stream);
}

}  // extern "C"

// ---- allocation-free decode step, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the workspace of the step
// lives in this file-scope device array.  Each GPU that loads the library holds its own
// copy until the process ends; its device address is looked up once per device.
static __device__ __align__(256) unsigned char scratch[NC_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};

nc_status scratch_of_device(void** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(NC_ERR_UNSUPPORTED, "device index beyond the supported range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(NC_ERR_DEVICE, std::string("scratch address: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NC_OK;
}
}  // namespace

extern "C" {

nc_status nc_decode_step_static(nc_model* m, const int32_t* tokens, int32_t B, nc_kv* kv, float* logits,
                                void* stream) {
    try {
        if (!m || !tokens || !kv || !logits) return fail(NC_ERR_INVALID_ARG, "NULL argument");
        if (kv->m != m) return fail(NC_ERR_INVALID_ARG, "kv belongs to another model");
        if (B != kv->B) return fail(NC_ERR_INVALID_ARG, "B differs from the cache's batch");
        if (B > 128) return fail(NC_ERR_UNSUPPORTED, "decode supports at most 128 rows");
        if (m->ex.on)
            return fail(NC_ERR_UNSUPPORTED, "the allocation-free decode step does not take the later-version blocks");
        for (int b = 0; b < B; ++b)
            if (kv->lens_host[b] + 1 > kv->max_seq) return fail(NC_ERR_CAPACITY, "a row is full (lens + 1 > max_seq)");
        const size_t need = ws_layout(m, kv->B, kv->S, B, nullptr).bytes;
        if (need > NC_STATIC_SCRATCH_BYTES)
            return fail(NC_ERR_CAPACITY, "the step's workspace (" + std::to_string(need) + " bytes) exceeds the " +
                                             std::to_string((size_t)NC_STATIC_SCRATCH_BYTES) + "-byte static array");
        void* base = nullptr;
        nc_status s = scratch_of_device(&base);
        if (s != NC_OK) return s;
        const Ws w = ws_layout(m, kv->B, kv->S, B, base);
        hipStream_t st = (hipStream_t)stream;
        // the array keeps the last call's contents: the attention ready flags and the
        // split-K arrival counters must start at zero
        LAUNCH(launch_zero_i32(w.actr, w.actr_elems, st));
        LAUNCH(launch_zero_i32(w.fctr, DEC_FIN_SLOTS, st));
        if (w.dpart) LAUNCH(launch_zero_i32((int32_t*)w.dpart, DEC_PART_CTRS, st));
        t_untimed = true;
        s = enqueue_decode(m, kv, w, tokens, logits, st);
        t_untimed = false;
        if (s != NC_OK) return s;
        for (int b = 0; b < B; ++b) kv->lens_host[b] += 1;
        return NC_OK;
    } catch (...) {
        t_untimed = false;
        return fail(NC_ERR_DEVICE, "unexpected exception");
    }
}

nc_status nc_timing_enable(int32_t kernel_class) {
    if (kernel_class < NC_KC_NONE || kernel_class > NC_KC_DECODE_ATTN)
        return fail(NC_ERR_INVALID_ARG, "unknown kernel class");
    HIP_TRY(hipDeviceSynchronize());
    for (auto& tp : g_tm.pending) timing_release(tp);
    g_tm.pending.clear();
    g_tm.cls = kernel_class;
    g_tm.launches = 0;
    g_tm.ms = g_tm.bytes = g_tm.flops = 0;
    return NC_OK;
}

nc_status nc_timing_read(nc_timing* out) {
    if (!out) return fail(NC_ERR_INVALID_ARG, "out is NULL");
    HIP_TRY(hipDeviceSynchronize());
    auto add = [](TimingPair& tp) -> hipError_t {
        float ms = 0.f;
        for (int i = 0; i < tp.n; ++i) {
            float t = 0.f;
            hipError_t e = hipEventElapsedTime(&t, tp.ev[i][0], tp.ev[i][1]);
            if (e != hipSuccess) return e;
            ms += t;
        }
        g_tm.launches++;
        g_tm.ms += ms;
        g_tm.bytes += tp.bytes;
        g_tm.flops += tp.flops;
        return hipSuccess;
    };
    hipError_t err = hipSuccess;
    for (auto& tp : g_tm.pending) {
        if (err == hipSuccess) err = add(tp);
        timing_release(tp);
    }
    g_tm.pending.clear();
    if (err != hipSuccess) return fail(NC_ERR_DEVICE, std::string("event timing: ") + hipGetErrorString(err));
    out->launches = g_tm.launches;
    out->ms = g_tm.ms;
    out->bytes = g_tm.bytes;
    out->flops = g_tm.flops;
    return NC_OK;
}

}  // extern "C"
