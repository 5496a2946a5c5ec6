// Host side of the Talker decode step (include/qp_talker.h).  Included once,
// at the end of qp.hip, so that it shares the weight uploader and the batched
// product launcher with the predictor.
#pragma once

#include "qp_talker.h"
#include "qp_talker_kernels.h"

struct qp_talker {
    int device = 0;
    qp_talker_geometry g{};
    int wt = 0;                       // kernel weight format
    std::vector<void*> allocs;
    struct Layer {
        qp::tiled::FMat qkv{}, o{}, gate{}, up{}, down{};
        const float* attn_norm = nullptr;
        const float* ffn_norm = nullptr;
        const float* q_norm = nullptr;
        const float* k_norm = nullptr;
    };
    std::vector<Layer> layers;
    qp::tiled::FMat head{};
    const float* out_norm = nullptr;
    uint16_t* kc = nullptr;           // [n_slots][L][nkv][max_ctx][hd]
    uint16_t* vc = nullptr;
    float* rope_cos = nullptr;        // [max_ctx][hd/2]
    float* rope_sin = nullptr;
    float* x = nullptr;               // [max_batch][d]
    float* ss = nullptr;              // [max_batch][d/16]
    float* qkv = nullptr;             // [max_batch][nqkv]
    uint16_t* xg = nullptr;           // max_batch rows (rounded up to 16) of width d, fragment order
    uint16_t* ao = nullptr;           // ... of width nq*hd, fragment order
    uint16_t* hb = nullptr;           // ... of width F, fragment order
    unsigned long long* keys = nullptr;  // [max_batch][vocab/16]
    float* apart = nullptr;           // attention partials [max_batch][nq][max_split][hd+2]
    int max_split = 0;
    unsigned* actr = nullptr;         // [max_batch][nkv]
    // split-K scratch of the products: none (the Talker has no projection
    // of H, the one product that splits K), so t_nctr = 0 keeps KS = 1
    float* t_part = nullptr;
    size_t t_part_floats = 0;
    unsigned* t_ctr = nullptr;
    size_t t_nctr = 0;
    unsigned* err = nullptr;
    unsigned last_flags = 0;
    // a step without the logits hook replays a graph prepared by
    // qp_talker_create for the smallest batch bucket that holds its rows
    // (attention grid for max_ctx; the call's row count and split limit are
    // read from st_live), reading and writing handle-owned staging buffers;
    // the graphs are kept until qp_talker_destroy
    struct StepGraph {
        int B = 0;
        hipGraph_t graph = nullptr;
        hipGraphExec_t exec = nullptr;
    };
    std::vector<StepGraph> graphs;
    hipStream_t cap_stream = nullptr;
    int* st_live = nullptr;           // {split limit, rows} of the replayed call
    float* st_x = nullptr;            // [max_batch][d]
    int* st_slots = nullptr;          // [max_batch]
    int* st_pos = nullptr;            // [max_batch]
    float* st_H = nullptr;            // [max_batch][d]
    int* st_q0 = nullptr;             // [max_batch]
};

namespace {

// 64 positions per attention split (a B = 1 step over 1,024 positions of
// history: 1.27 ms against 1.32 with 32-position chunks; 128 and 256 were
// slower)
constexpr int kTalkerCh = qp::talker::kMaxCh;

qp_status validate_talker(const qp_talker_geometry* g) {
    if (g->d_model <= 0 || g->n_layers < 0 || g->n_q_heads <= 0 || g->n_kv_heads <= 0 || g->head_dim <= 0 ||
        g->d_ffn <= 0 || g->vocab <= 0)
        return fail(QP_ERR_GEOMETRY, "non-positive talker dimension");
    if (g->n_q_heads != g->n_kv_heads && g->n_q_heads != 2 * g->n_kv_heads)
        return fail(QP_ERR_GEOMETRY, "n_q_heads must equal n_kv_heads or twice it");
    if (g->head_dim != 64 && g->head_dim != 128) return fail(QP_ERR_GEOMETRY, "head_dim must be 64 or 128");
    if (g->d_model % 256 || (g->n_q_heads * g->head_dim) % 256 || g->d_ffn % 256 || g->vocab % 32 ||
        ((g->n_q_heads + 2 * g->n_kv_heads) * g->head_dim) % 32)
        return fail(QP_ERR_SHAPE, "d_model, n_q_heads*head_dim and d_ffn must be multiples of 256, vocab of 32");
    if (!(g->rms_eps > 0.f) || !(g->rope_base > 1.f)) return fail(QP_ERR_GEOMETRY, "rms_eps must be > 0, rope_base > 1");
    if (g->weight_dtype != QP_WEIGHT_BF16 && g->weight_dtype != QP_WEIGHT_Q8_0 && g->weight_dtype != QP_WEIGHT_Q4_0)
        return fail(QP_ERR_DTYPE, "talker weights must be bf16, Q8_0 or Q4_0");
    if (g->max_batch < 1 || g->n_slots < 1 || g->max_ctx < 1 || g->max_ctx > (1 << 20))
        return fail(QP_ERR_GEOMETRY, "max_batch and n_slots must be >= 1, max_ctx in [1, 2^20]");
    return QP_OK;
}

// attention split of a step: 64-position chunks, their number rounded up to
// a power of two (chunks past a request's history exit at once), so that a
// growing history changes the launch shape only when it doubles
void talker_split(int max_len, int* ch_out, int* nsplit_out) {
    const int ch = kTalkerCh;
    int ns = 1;
    while (ns * ch < max_len) ns *= 2;
    *ch_out = ch;
    *nsplit_out = ns;
}

template <int WT>
qp_status talker_launch(qp_talker* t, int B, const float* x, const int* slots, const int* pos, int ch, int nsplit,
                        float* H_out, int* q0_out, float* logits_out, hipStream_t stream,
                        const int* live = nullptr) {
    namespace T = qp::tiled;
    namespace K = qp::talker;
    const qp_talker_geometry& G = t->g;
    const int d = G.d_model, L = G.n_layers, hd = G.head_dim;
    const int qd = G.n_q_heads * hd, nqkv = (G.n_q_heads + 2 * G.n_kv_heads) * hd, nss = d / 16;
    const int R = G.n_q_heads / G.n_kv_heads;
    if (nsplit > t->max_split) return fail(QP_ERR_INVALID_ARG, "attention split table too small");

    // the bf16 activations' layout for this batch (qp::tiled::act_index)
    const int frag = B >= T::kFragMinRows ? 1 : 0;
    K::InArgs ia{d, x, t->x, t->xg, t->ss, L > 0 ? t->layers[0].attn_norm : t->out_norm, frag};
    hipLaunchKernelGGL(K::k_input, dim3(B), dim3(K::kThreadsK), 0, stream, ia);
    K::AttnArgs aa{};
    aa.nkv = G.n_kv_heads;
    aa.nqkv = nqkv;
    aa.qd = qd;
    aa.L = L;
    aa.max_ctx = G.max_ctx;
    aa.n_slots = G.n_slots;
    aa.ch = ch;
    aa.nsplit = nsplit;
    aa.eps = G.rms_eps;
    aa.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(hd)));
    aa.qkv = t->qkv;
    aa.rope_cos = t->rope_cos;
    aa.rope_sin = t->rope_sin;
    aa.slots = slots;
    aa.pos = pos;
    aa.kc = t->kc;
    aa.vc = t->vc;
    aa.part = t->apart;
    aa.ctr = t->actr;
    aa.ao = t->ao;
    aa.frag = frag;
    aa.err = t->err;
    aa.live = live;
    T::GemmArgs g{};
    for (int l = 0; l < L; ++l) {
        const qp_talker::Layer& Ly = t->layers[l];
        const float* g_after = l + 1 < L ? t->layers[l + 1].attn_norm : t->out_norm;
        // q, k, v = W_qkv . RMSNorm(x)
        g = T::GemmArgs{};
        g.eps = G.rms_eps;
        g.frag = frag;
        g.M = B;
        g.a = t->xg;
        g.lda = d;
        g.ss_in = t->ss;
        g.nss = nss;
        g.N = nqkv;
        g.K = d;
        g.w0 = Ly.qkv;
        g.out = t->qkv;
        g.ldo = nqkv;
        tiled_gemm<WT, T::SRC_BF16_NORM, T::EPI_SCALE>(t, g, stream);
        // attention over each request's history
        aa.l = l;
        aa.q_norm = Ly.q_norm;
        aa.k_norm = Ly.k_norm;
        const dim3 ag(nsplit, G.n_kv_heads, B);
        if (hd == 128) {
            if (R == 2) hipLaunchKernelGGL((K::k_attn<128, 2>), ag, dim3(K::kThreadsK), 0, stream, aa);
            else hipLaunchKernelGGL((K::k_attn<128, 1>), ag, dim3(K::kThreadsK), 0, stream, aa);
        } else {
            if (R == 2) hipLaunchKernelGGL((K::k_attn<64, 2>), ag, dim3(K::kThreadsK), 0, stream, aa);
            else hipLaunchKernelGGL((K::k_attn<64, 1>), ag, dim3(K::kThreadsK), 0, stream, aa);
        }
        // x += W_o . attention; publishes bf16(ffn_norm * x)
        g = T::GemmArgs{};
        g.eps = G.rms_eps;
        g.frag = frag;
        g.M = B;
        g.a = t->ao;
        g.lda = qd;
        g.N = d;
        g.K = qd;
        g.w0 = Ly.o;
        g.out = t->x;
        g.ldo = d;
        g.xg = t->xg;
        g.g_next = Ly.ffn_norm;
        g.ss_out = t->ss;
        tiled_gemm<WT, T::SRC_BF16, T::EPI_RESID>(t, g, stream);
        // h = silu(W_g . RMSNorm(x)) * (W_u . RMSNorm(x)), bf16
        g = T::GemmArgs{};
        g.eps = G.rms_eps;
        g.frag = frag;
        g.M = B;
        g.a = t->xg;
        g.lda = d;
        g.ss_in = t->ss;
        g.nss = nss;
        g.N = G.d_ffn;
        g.K = d;
        g.w0 = Ly.gate;
        g.w1 = Ly.up;
        g.outb = t->hb;
        tiled_gemm<WT, T::SRC_BF16_NORM, T::EPI_SWIGLU>(t, g, stream);
        // x += W_d . h; publishes the next reader's operand
        g = T::GemmArgs{};
        g.eps = G.rms_eps;
        g.frag = frag;
        g.M = B;
        g.a = t->hb;
        g.lda = G.d_ffn;
        g.N = d;
        g.K = G.d_ffn;
        g.w0 = Ly.down;
        g.out = t->x;
        g.ldo = d;
        g.xg = t->xg;
        g.g_next = g_after;
        g.ss_out = t->ss;
        tiled_gemm<WT, T::SRC_BF16, T::EPI_RESID>(t, g, stream);
    }
    // codec head . RMSNorm(x): per-tile argmax keys (and the logits)
    g = T::GemmArgs{};
    g.eps = G.rms_eps;
    g.frag = frag;
    g.M = B;
    g.a = t->xg;
    g.lda = d;
    g.ss_in = t->ss;
    g.nss = nss;
    g.N = G.vocab;
    g.K = d;
    g.w0 = t->head;
    g.keys = t->keys;
    if (logits_out) {
        g.logits = logits_out;
        g.logit_ld = G.vocab;
    }
    const int nkt = tiled_gemm<WT, T::SRC_BF16_NORM, T::EPI_ARGMAX>(t, g, stream);
    K::FinArgs fa{d, nkt, G.rms_eps, t->x, t->ss, t->out_norm, t->keys, H_out, q0_out};
    hipLaunchKernelGGL(K::k_final, dim3(B), dim3(K::kThreadsK), 0, stream, fa);
    qp_status st = QP_OK;
    if (!check_hip(hipGetLastError(), "talker kernel launch", &st)) return st;
    return QP_OK;
}

// Capture one step of batch bucket Bk (attention grid for max_ctx) and
// instantiate it.
template <int WT>
qp_status talker_capture(qp_talker* t, int Bk) {
    qp_status st = QP_OK;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (!check_hip(hipStreamBeginCapture(t->cap_stream, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture", &st))
        return st;
    const qp_status lst = talker_launch<WT>(t, Bk, t->st_x, t->st_slots, t->st_pos, kTalkerCh, t->max_split, t->st_H,
                                            t->st_q0, nullptr, t->cap_stream, t->st_live);
    const hipError_t ce = hipStreamEndCapture(t->cap_stream, &graph);
    if (lst != QP_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return lst;
    }
    if (!check_hip(ce, "hipStreamEndCapture", &st)) return st;
    if (!check_hip(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "hipGraphInstantiate", &st)) {
        (void)hipGraphDestroy(graph);
        return st;
    }
    qp_talker::StepGraph sg;
    sg.B = Bk;
    sg.graph = graph;
    sg.exec = exec;
    t->graphs.push_back(sg);
    return QP_OK;
}

qp_status talker_prepare_graphs(qp_talker* t) {
    qp_status st = QP_OK;
    if (!check_hip(hipStreamCreateWithFlags(&t->cap_stream, hipStreamNonBlocking), "hipStreamCreate", &st)) return st;
    for (int Bk : batch_buckets(t->g.max_batch)) {
        switch (t->wt) {
            case WT_BF16: st = talker_capture<WT_BF16>(t, Bk); break;
            case WT_Q8: st = talker_capture<WT_Q8>(t, Bk); break;
            default: st = talker_capture<WT_Q4>(t, Bk); break;
        }
        if (st != QP_OK) return st;
    }
    return QP_OK;
}

// A step without the logits hook: stage the call's rows (padding rows of the
// bucket zeroed), write its limits, replay the bucket's prepared graph and
// copy B rows of H and q0 back.  Nothing is captured or freed here.
qp_status talker_launch_graph(qp_talker* t, int B, const float* x, const int* slots, const int* pos, int nsplit,
                              float* H_out, int* q0_out, hipStream_t stream) {
    qp_status st = QP_OK;
    const qp_talker::StepGraph* sg = nullptr;
    for (const auto& e : t->graphs)
        if (e.B >= B && (!sg || e.B < sg->B)) sg = &e;
    if (!sg) return fail(QP_ERR_HIP, "no prepared talker graph for B=" + std::to_string(B));
    const size_t d = static_cast<size_t>(t->g.d_model), Bk = static_cast<size_t>(sg->B);
    stage32(x, t->st_x, static_cast<size_t>(B) * d, Bk * d, stream);
    stage32(slots, t->st_slots, static_cast<size_t>(B), Bk, stream);
    stage32(pos, t->st_pos, static_cast<size_t>(B), Bk, stream);
    hipLaunchKernelGGL(qp::talker::k_set_live, dim3(1), dim3(64), 0, stream, t->st_live, nsplit, B);
    if (!check_hip(hipGraphLaunch(sg->exec, stream), "hipGraphLaunch", &st)) return st;
    copy32(t->st_H, H_out, static_cast<size_t>(B) * d, stream);
    copy32(t->st_q0, q0_out, static_cast<size_t>(B), stream);
    if (!check_hip(hipGetLastError(), "staging copy launch", &st)) return st;
    return QP_OK;
}

void talker_free(qp_talker* t) {
    for (void* p : t->allocs) (void)hipFree(p);
    t->allocs.clear();
}

// Wait for the device (no replay is in flight after that), then free the
// graphs, the capture stream, every buffer and the handle.
void talker_destroy(qp_talker* t) {
    {
        DeviceGuard guard(t->device);
        (void)hipDeviceSynchronize();
        for (auto& e : t->graphs) {
            if (e.exec) (void)hipGraphExecDestroy(e.exec);
            if (e.graph) (void)hipGraphDestroy(e.graph);
        }
        t->graphs.clear();
        if (t->cap_stream) (void)hipStreamDestroy(t->cap_stream);
        t->cap_stream = nullptr;
        talker_free(t);
    }
    delete t;
}

}  // namespace

extern "C" {

qp_status qp_talker_create(const qp_talker_weights* w, const qp_talker_geometry* g, int32_t device,
                           qp_talker** out) {
    if (!out) return fail(QP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w || !g) return fail(QP_ERR_INVALID_ARG, "weights or geometry is NULL");
    qp_status st = validate_talker(g);
    if (st != QP_OK) return st;
    if (!w->output_norm || !w->codec_head || (g->n_layers > 0 && !w->layers))
        return fail(QP_ERR_INVALID_ARG, "missing talker weights");
    for (int l = 0; l < g->n_layers; ++l) {
        const qp_layer_weights& lw = w->layers[l];
        if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.q_norm || !lw.k_norm || !lw.ffn_norm ||
            !lw.w_gate || !lw.w_up || !lw.w_down)
            return fail(QP_ERR_INVALID_ARG, "missing weights in talker layer " + std::to_string(l));
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
        return fail(QP_ERR_INVALID_ARG, "no such HIP device");
    DeviceGuard guard(device);
    qp_talker* t = new qp_talker();
    t->device = device;
    t->g = *g;
    const int hostwt = g->weight_dtype == QP_WEIGHT_BF16 ? WT_BF16 : (g->weight_dtype == QP_WEIGHT_Q8_0 ? WT_Q8 : WT_Q4);
    t->wt = hostwt;
    const int d = g->d_model, L = g->n_layers, hd = g->head_dim, F = g->d_ffn;
    const int qd = g->n_q_heads * hd, kd = g->n_kv_heads * hd, nqkv = qd + 2 * kd;
    Uploader up{&t->allocs};
    for (int l = 0; l < L && up.st == QP_OK; ++l) {
        const qp_layer_weights& lw = w->layers[l];
        qp_talker::Layer Ly;
        Ly.qkv = up.fragments(Uploader::build({lw.wq, lw.wk, lw.wv}, {qd, kd, kd}, d, hostwt));
        Ly.o = up.fragments(Uploader::build({lw.wo}, {d}, qd, hostwt));
        Ly.gate = up.fragments(Uploader::build({lw.w_gate}, {F}, d, hostwt));
        Ly.up = up.fragments(Uploader::build({lw.w_up}, {F}, d, hostwt));
        Ly.down = up.fragments(Uploader::build({lw.w_down}, {d}, F, hostwt));
        Ly.attn_norm = static_cast<const float*>(up.upload(lw.attn_norm, sizeof(float) * d));
        Ly.q_norm = static_cast<const float*>(up.upload(lw.q_norm, sizeof(float) * hd));
        Ly.k_norm = static_cast<const float*>(up.upload(lw.k_norm, sizeof(float) * hd));
        Ly.ffn_norm = static_cast<const float*>(up.upload(lw.ffn_norm, sizeof(float) * d));
        t->layers.push_back(Ly);
    }
    t->head = up.fragments(Uploader::build({w->codec_head}, {g->vocab}, d, hostwt));
    t->out_norm = static_cast<const float*>(up.upload(w->output_norm, sizeof(float) * d));
    // RoPE table, fp64 then rounded: angle(p, i) = p * base^(-2i/hd)
    const int half = hd / 2;
    std::vector<float> rc(static_cast<size_t>(g->max_ctx) * half), rs(rc.size());
    for (int p = 0; p < g->max_ctx; ++p)
        for (int i = 0; i < half; ++i) {
            const double ang = p * std::pow(static_cast<double>(g->rope_base), -2.0 * i / hd);
            rc[static_cast<size_t>(p) * half + i] = static_cast<float>(std::cos(ang));
            rs[static_cast<size_t>(p) * half + i] = static_cast<float>(std::sin(ang));
        }
    t->rope_cos = static_cast<float*>(up.upload(rc.data(), rc.size() * 4));
    t->rope_sin = static_cast<float*>(up.upload(rs.data(), rs.size() * 4));
    const size_t kvn = static_cast<size_t>(g->n_slots) * L * g->n_kv_heads * g->max_ctx * hd;
    t->kc = static_cast<uint16_t*>(up.alloc(kvn * 2));
    t->vc = static_cast<uint16_t*>(up.alloc(kvn * 2));
    const size_t mb = static_cast<size_t>(g->max_batch);
    t->x = static_cast<float*>(up.alloc(mb * d * 4));
    t->ss = static_cast<float*>(up.alloc(mb * (d / 16) * 4));
    t->qkv = static_cast<float*>(up.alloc(mb * nqkv * 4));
    // the products' bf16 operands in fragment order: whole row fragments
    const size_t mb16 = (mb + 15) / 16 * 16;
    t->xg = static_cast<uint16_t*>(up.alloc(mb16 * d * 2));
    t->ao = static_cast<uint16_t*>(up.alloc(mb16 * qd * 2));
    t->hb = static_cast<uint16_t*>(up.alloc(mb16 * F * 2));
    t->keys = static_cast<unsigned long long*>(up.alloc(mb * (g->vocab / 16) * 8));
    t->max_split = 1;   // split counts are powers of two
    while (t->max_split * kTalkerCh < g->max_ctx) t->max_split *= 2;
    t->apart = static_cast<float*>(up.alloc(mb * g->n_q_heads * t->max_split * (hd + 2) * 4));
    t->actr = static_cast<unsigned*>(up.alloc(mb * g->n_kv_heads * 4));
    t->err = static_cast<unsigned*>(up.alloc(256));
    t->st_x = static_cast<float*>(up.alloc(mb * d * 4));
    t->st_slots = static_cast<int*>(up.alloc(mb * 4));
    t->st_pos = static_cast<int*>(up.alloc(mb * 4));
    t->st_H = static_cast<float*>(up.alloc(mb * d * 4));
    t->st_q0 = static_cast<int*>(up.alloc(mb * 4));
    t->st_live = static_cast<int*>(up.alloc(2 * 4));
    if (up.st == QP_OK) {
        // counters start (and are left) at zero; the cache starts cleared
        if (!check_hip(hipMemset(t->actr, 0, mb * g->n_kv_heads * 4), "hipMemset", &st) ||
            !check_hip(hipMemset(t->err, 0, 256), "hipMemset", &st) ||
            !check_hip(hipMemset(t->kc, 0, kvn * 2), "hipMemset", &st) ||
            !check_hip(hipMemset(t->vc, 0, kvn * 2), "hipMemset", &st) ||
            !check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize", &st))
            up.st = st;
    }
    if (up.st != QP_OK) {
        const qp_status s2 = up.st;
        if (!up.msg.empty()) (void)fail(s2, up.msg);
        talker_free(t);
        delete t;
        return s2;
    }
    // every graph a later step can replay, built now so that no step
    // captures, instantiates or frees one
    st = talker_prepare_graphs(t);
    if (st != QP_OK) {
        talker_destroy(t);
        return st;
    }
    *out = t;
    return QP_OK;
}

qp_status qp_talker_load_history(qp_talker* t, int32_t slot, int32_t n, const uint16_t* k, const uint16_t* v,
                                 void* stream) {
    if (!t) return fail(QP_ERR_INVALID_ARG, "talker is NULL");
    if (slot < 0 || slot >= t->g.n_slots) return fail(QP_ERR_INVALID_ARG, "slot outside [0, n_slots)");
    if (n < 0 || n > t->g.max_ctx) return fail(QP_ERR_INVALID_ARG, "n outside [0, max_ctx]");
    if (n == 0 || t->g.n_layers == 0) return QP_OK;
    if (!k || !v) return fail(QP_ERR_INVALID_ARG, "NULL history pointer");
    DeviceGuard guard(t->device);
    hipLaunchKernelGGL(qp::talker::k_load_history, dim3(1024), dim3(256), 0, static_cast<hipStream_t>(stream), k, v,
                       t->kc, t->vc, slot, n, t->g.n_layers, t->g.n_kv_heads, t->g.head_dim, t->g.max_ctx);
    qp_status st = QP_OK;
    if (!check_hip(hipGetLastError(), "history copy launch", &st)) return st;
    return QP_OK;
}

qp_status qp_talker_step(qp_talker* t, int32_t B, const float* x, const int32_t* slots, const int32_t* pos,
                         int32_t max_len, float* H_out, int32_t* q0_out, float* logits_out, void* stream) {
    if (!t) return fail(QP_ERR_INVALID_ARG, "talker is NULL");
    if (B < 0 || B > t->g.max_batch)
        return fail(QP_ERR_BATCH, "B=" + std::to_string(B) + " outside [0, " + std::to_string(t->g.max_batch) + "]");
    if (max_len < 1 || max_len > t->g.max_ctx) return fail(QP_ERR_INVALID_ARG, "max_len outside [1, max_ctx]");
    if (B == 0) return QP_OK;
    if (!x || !slots || !pos || !H_out || !q0_out) return fail(QP_ERR_INVALID_ARG, "NULL input or output pointer");
    DeviceGuard guard(t->device);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int ch = 0, ns = 0;
    talker_split(max_len, &ch, &ns);
    if (logits_out) {
        switch (t->wt) {
            case WT_BF16: return talker_launch<WT_BF16>(t, B, x, slots, pos, ch, ns, H_out, q0_out, logits_out, s);
            case WT_Q8: return talker_launch<WT_Q8>(t, B, x, slots, pos, ch, ns, H_out, q0_out, logits_out, s);
            default: return talker_launch<WT_Q4>(t, B, x, slots, pos, ch, ns, H_out, q0_out, logits_out, s);
        }
    }
    return talker_launch_graph(t, B, x, slots, pos, ns, H_out, q0_out, s);
}

qp_status qp_talker_get_error(qp_talker* t) {
    if (!t) return fail(QP_ERR_INVALID_ARG, "talker is NULL");
    DeviceGuard guard(t->device);
    qp_status st = QP_OK;
    if (!check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize", &st)) return st;
    unsigned flags = 0;
    if (!check_hip(hipMemcpy(&flags, t->err, 4, hipMemcpyDeviceToHost), "hipMemcpy", &st)) return st;
    t->last_flags = flags;
    if (flags == 0) return QP_OK;
    if (!check_hip(hipMemset(t->err, 0, 4), "hipMemset", &st)) return st;
    char hex[16];
    std::snprintf(hex, sizeof(hex), "0x%x", flags);
    return fail(QP_ERR_DEVICE_FLAG, std::string("talker device flags ") + hex);
}

uint32_t qp_talker_last_device_flags(qp_talker* t) { return t ? t->last_flags : 0u; }

void qp_talker_destroy(qp_talker* t) {
    if (!t) return;
    talker_destroy(t);
}

}  // extern "C"
