// C ABI of libhf: argument validation, workspace layout and kernel launches.
// Every entry point validates all of its arguments before enqueuing anything, so a
// failing call has no side effect; the reason is kept per thread for hf_last_error().
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "hf_internal.h"

namespace {

thread_local std::string g_last_error;

hf_status fail(hf_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

hf_status ok() {
    g_last_error.clear();
    return HF_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxElems = (int64_t)1 << 31;

hf_status check_dims(const hf_dims *d) {
    if (!d) return fail(HF_ERR_NULL, "dims is NULL");
    if (d->B < 1 || d->H < 1) return fail(HF_ERR_SHAPE, "B=%d H=%d must be >= 1", d->B, d->H);
    if (d->D != 64 && d->D != 128) return fail(HF_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", d->D);
    if (d->T < 8 || d->T % 8) return fail(HF_ERR_UNSUPPORTED, "T=%d must be a positive multiple of 8", d->T);
    if (d->C < 1 || d->W < d->C) return fail(HF_ERR_SHAPE, "need 1 <= C <= W (C=%d W=%d)", d->C, d->W);
    if (d->bq != 16 && d->bq != 32 && d->bq != 64)
        return fail(HF_ERR_UNSUPPORTED, "bq=%d (supported: 16, 32, 64)", d->bq);
    if (d->bk != 16 && d->bk != 32 && d->bk != 64 && d->bk != 128)
        return fail(HF_ERR_UNSUPPORTED, "bk=%d (supported: 16, 32, 64, 128)", d->bk);
    const int64_t ring = (int64_t)d->B * d->H * d->W * d->T * d->D;
    if (ring >= kMaxElems) return fail(HF_ERR_UNSUPPORTED, "ring of %lld elements exceeds 2^31", (long long)ring);
    const int64_t nkb = cdiv((int64_t)d->W * d->T, d->bk);
    if (nkb > kMaxKeyBlocks)
        return fail(HF_ERR_UNSUPPORTED, "window of %lld key blocks exceeds %d", (long long)nkb, kMaxKeyBlocks);
    return HF_OK;
}

hf_status check_ring(const hf_dims *d, const hf_kv_ring *r) {
    if (!r) return fail(HF_ERR_NULL, "ring is NULL");
    if (!r->k_dev || !r->vg_dev) return fail(HF_ERR_NULL, "ring storage pointer is NULL");
    if (r->head < 0 || r->head >= d->W) return fail(HF_ERR_RING_STATE, "ring head=%d outside [0, W=%d)", r->head, d->W);
    if (r->n_committed < 0 || r->n_committed > d->W - d->C)
        return fail(HF_ERR_RING_STATE, "ring n_committed=%d outside [0, W-C=%d]", r->n_committed, d->W - d->C);
    return HF_OK;
}

struct Geometry {
    int BH, Nq, Nk, nqb, nkb;
};

Geometry geometry(const hf_dims *d, const hf_kv_ring *r) {
    Geometry g;
    g.BH = d->B * d->H;
    g.Nq = d->C * d->T;
    g.Nk = (r->n_committed + d->C) * d->T;
    g.nqb = (int)cdiv(g.Nq, d->bq);
    g.nkb = (int)cdiv(g.Nk, d->bk);
    return g;
}

// Workspace layout (offsets 256-byte aligned):
//   [absorb partials]  [qbar fp64]  [kbar fp64]  [S^T bf16]  [z copy fp32]
//   [frame-pooled keys fp64, up to kMaxHierFrames frames]  [per key block frame parts fp64]
struct WsLayout {
    size_t absorb, qbar, kbar, st, zc, fbar, part, total;
};

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const hf_dims *d) {
    const int BH = d->B * d->H;
    const int64_t nqb = cdiv((int64_t)d->C * d->T, d->bq);
    const int64_t nkb = cdiv((int64_t)d->W * d->T, d->bk);
    WsLayout w;
    w.absorb = 0;
    w.qbar = al(hf_absorb_workspace_bytes(BH, d->D));
    w.kbar = w.qbar + al((size_t)BH * nqb * d->D * sizeof(double));
    w.st = w.kbar + al((size_t)BH * nkb * d->D * sizeof(double));
    w.zc = w.st + al((size_t)BH * d->D * d->D * sizeof(uint16_t));
    w.fbar = w.zc + al((size_t)BH * d->D * sizeof(float));
    const int frames = d->W < kMaxHierFrames ? d->W : kMaxHierFrames;
    w.part = w.fbar + al((size_t)BH * frames * d->D * sizeof(double));
    w.total = w.part + al((size_t)BH * nkb * 2 * d->D * sizeof(double));
    return w;
}

hf_status check_ws(const hf_dims *d, void *ws, size_t bytes) {
    const size_t need = ws_layout(d).total;
    if (!ws) return fail(HF_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (bytes < need) return fail(HF_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", bytes, need);
    return HF_OK;
}

char *wsp(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

hf_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(HF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return HF_OK;
}

// --- enqueue helpers (arguments already validated)

hf_append_args append_args(const hf_dims *d, const hf_kv_ring *r, const void *kc, const void *vc) {
    hf_append_args a{};
    a.BH = d->B * d->H;
    a.D = d->D;
    a.T = d->T;
    a.W = d->W;
    a.head = r->head;
    a.first_frame = r->n_committed;
    a.C = d->C;
    a.k_cur = static_cast<const uint16_t *>(kc);
    a.v_cur = static_cast<const uint16_t *>(vc);
    a.ring_k = static_cast<uint16_t *>(r->k_dev);
    a.ring_vg = static_cast<uint16_t *>(r->vg_dev);
    return a;
}

hipError_t enqueue_append(const hf_dims *d, const hf_kv_ring *r, const void *kc, const void *vc, hipStream_t s) {
    return hf_launch_ring_append(append_args(d, r, kc, vc), s);
}

hipError_t enqueue_select(const hf_dims *d, const void *q, const hf_kv_ring *r, int top_k, int32_t *idx,
                          double *scores, void *ws, hipStream_t s, int top_frames = 0, int32_t *fidx = nullptr,
                          double *fscores = nullptr, const hf_state_args *prep = nullptr,
                          const hf_append_args *app = nullptr) {
    const Geometry g = geometry(d, r);
    const WsLayout L = ws_layout(d);
    hf_select_args a{};
    a.BH = g.BH;
    a.D = d->D;
    a.T = d->T;
    a.W = d->W;
    a.head = r->head;
    a.Nq = g.Nq;
    a.Nk = g.Nk;
    a.bq = d->bq;
    a.bk = d->bk;
    a.nqb = g.nqb;
    a.nkb = g.nkb;
    a.top_k = top_k;
    a.q = static_cast<const uint16_t *>(q);
    a.ring_k = static_cast<const uint16_t *>(r->k_dev);
    a.qbar = reinterpret_cast<double *>(wsp(ws, L.qbar));
    a.kbar = reinterpret_cast<double *>(wsp(ws, L.kbar));
    a.idx = idx;
    a.scores = scores;
    a.nfr = r->n_committed + d->C;
    a.top_frames = top_frames;
    a.fbar = reinterpret_cast<double *>(wsp(ws, L.fbar));
    a.part = reinterpret_cast<double *>(wsp(ws, L.part));
    a.fidx = fidx;
    a.fscores = fscores;
    if (prep) {
        a.prep = *prep;
        a.prep_tiles = a.BH * (d->D / 32) * (d->D / 32);
    }
    if (app) {
        a.app = *app;
        a.app_tiles = hf_append_tiles(*app);
        a.k_cur = app->k_cur;
        a.ncom = r->n_committed;
    }
    return hf_launch_block_select(a, s);
}

// The state pass of a step: readout operands (S^T bf16, z copy) from the state as it is,
// and, when `absorb_tokens` > 0, the absorb partials already in the workspace added in.
// `step_absorb`: the partials come from a step's absorb (its own split count).
hf_state_args state_args(const hf_dims *d, float *S, float *z, bool readout, int64_t absorb_tokens, void *ws,
                         bool step_absorb = false) {
    const WsLayout L = ws_layout(d);
    hf_state_args a{};
    a.BH = d->B * d->H;
    a.D = d->D;
    a.S = S;
    a.z = z;
    a.part = absorb_tokens > 0 ? reinterpret_cast<const float *>(wsp(ws, L.absorb)) : nullptr;
    a.P = absorb_tokens <= 0 ? 0
          : (step_absorb ? hf_step_absorb_splits(a.BH, d->D, absorb_tokens) : hf_absorb_splits(a.BH, d->D, absorb_tokens));
    a.st = readout ? reinterpret_cast<uint16_t *>(wsp(ws, L.st)) : nullptr;
    a.zc = readout ? reinterpret_cast<float *>(wsp(ws, L.zc)) : nullptr;
    return a;
}

hipError_t enqueue_state(const hf_dims *d, float *S, float *z, bool readout, int64_t absorb_tokens, void *ws,
                         hipStream_t s, bool step_absorb = false) {
    return hf_launch_state(state_args(d, S, z, readout, absorb_tokens, ws, step_absorb), s);
}

// Attention (+ readout from the prepared S^T / z copy when `readout`).
hipError_t enqueue_attn(const hf_dims *d, const void *q, const hf_kv_ring *r, const int32_t *idx, int top_k,
                        bool readout, float eps, float *out, void *ws, hipStream_t s, float *lse = nullptr,
                        const hf_rope *rope = nullptr, int64_t absorb_tok = 0) {
    const Geometry g = geometry(d, r);
    const WsLayout L = ws_layout(d);
    hf_attn_args a{};
    a.BH = g.BH;
    a.D = d->D;
    a.T = d->T;
    a.W = d->W;
    a.head = r->head;
    a.Nq = g.Nq;
    a.Nk = g.Nk;
    a.bq = d->bq;
    a.bk = d->bk;
    a.nqb = g.nqb;
    a.nkb = g.nkb;
    a.top_k = top_k;
    a.q = static_cast<const uint16_t *>(q);
    a.ring_k = static_cast<const uint16_t *>(r->k_dev);
    a.ring_vg = static_cast<const uint16_t *>(r->vg_dev);
    a.idx = idx;
    a.st = readout ? reinterpret_cast<const uint16_t *>(wsp(ws, L.st)) : nullptr;
    a.zc = readout ? reinterpret_cast<const float *>(wsp(ws, L.zc)) : nullptr;
    a.eps = eps;
    a.out = out;
    a.lse = lse;
    a.ncom = r->n_committed;
    if (rope) {
        a.rope_dt = rope->temporal_dims;
        a.rope_cap = rope->cap;
        a.rope_c1 = (float)(-2.0 * std::log2((double)rope->base) / rope->temporal_dims);
    }
    if (absorb_tok > 0) {   // the step's evicted tokens: split partials by extra workgroups of this launch
        a.ab_E = (int)absorb_tok;
        a.ab_part = reinterpret_cast<float *>(wsp(ws, L.absorb));
    }
    return hf_launch_sparse_attn(a, s);
}

// Absorb partial sums of row-major evicted tokens (k, v) into the workspace.
hipError_t enqueue_absorb_partial(const hf_dims *d, const void *k, const void *v, int64_t n_tok, void *ws,
                                  hipStream_t s) {
    hf_absorb_args a{};
    a.BH = d->B * d->H;
    a.D = d->D;
    a.n_tok = n_tok;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.part = reinterpret_cast<float *>(wsp(ws, ws_layout(d).absorb));
    if (hf_absorb_partial_floats(a.BH, a.D, hf_absorb_splits(a.BH, a.D, n_tok)) * sizeof(float) >
        hf_absorb_workspace_bytes(a.BH, a.D))
        return hipErrorInvalidValue;
    return hf_launch_absorb_partial(a, s);
}

hipError_t record(const hf_step_events *ev, int i, hipStream_t s) {
    if (ev && ev->ev[i]) return hipEventRecord(ev->ev[i], s);
    return hipSuccess;
}

}  // namespace

extern "C" {

int hf_abi_version(void) { return HF_ABI_VERSION; }

hf_status hf_cag_schedule(int32_t n_chunks, const int32_t *n_kb, double s_base, double s_target, double s_max,
                          int32_t *top_k, double *sparsity, double *beta) {
    if (!n_kb || !top_k) return fail(HF_ERR_NULL, "n_kb/top_k is NULL");
    if (n_chunks < 1) return fail(HF_ERR_SHAPE, "n_chunks=%d must be >= 1", n_chunks);
    auto unit = [](double x) { return x >= 0.0 && x < 1.0; };   // also rejects NaN
    if (!unit(s_base) || !unit(s_target) || !unit(s_max))
        return fail(HF_ERR_SHAPE, "s_base, s_target and s_max must lie in [0, 1)");
    for (int i = 0; i < n_chunks; ++i)
        if (n_kb[i] < 1) return fail(HF_ERR_SHAPE, "n_kb[%d]=%d must be >= 1", i, n_kb[i]);
    hf_status st = hf_cag_schedule_impl(n_chunks, n_kb, s_base, s_target, s_max, top_k, sparsity, beta);
    return st == HF_OK ? ok() : st;
}

const char *hf_status_str(hf_status s) {
    switch (s) {
        case HF_OK: return "HF_OK";
        case HF_ERR_NULL: return "HF_ERR_NULL";
        case HF_ERR_SHAPE: return "HF_ERR_SHAPE";
        case HF_ERR_UNSUPPORTED: return "HF_ERR_UNSUPPORTED";
        case HF_ERR_RING_STATE: return "HF_ERR_RING_STATE";
        case HF_ERR_WORKSPACE: return "HF_ERR_WORKSPACE";
        case HF_ERR_HIP: return "HF_ERR_HIP";
    }
    return "HF_ERR_UNKNOWN";
}

const char *hf_last_error(void) { return g_last_error.c_str(); }

hf_status hf_workspace_size(const hf_dims *d, int32_t top_k, size_t *bytes) {
    hf_status st = check_dims(d);
    if (st != HF_OK) return st;
    if (!bytes) return fail(HF_ERR_NULL, "bytes is NULL");
    (void)top_k;
    *bytes = ws_layout(d).total;
    return ok();
}

hf_status hf_ring_init(const hf_dims *d, void *k_store, void *vg_store, hf_kv_ring *out) {
    const hf_status st = check_dims(d);
    if (st != HF_OK) return st;
    if (!k_store || !vg_store || !out) return fail(HF_ERR_NULL, "k_store/vg_store/out is NULL");
    *out = hf_kv_ring{k_store, vg_store, 0, 0};
    return ok();
}

hf_status hf_ring_append(const hf_dims *d, const hf_kv_ring *ring, const void *k_cur, const void *v_cur,
                         hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_ring(d, ring);
    if (st != HF_OK) return st;
    if (!k_cur || !v_cur) return fail(HF_ERR_NULL, "k_cur/v_cur is NULL");
    st = hip_status(enqueue_append(d, ring, k_cur, v_cur, stream), "ring append launch");
    return st == HF_OK ? ok() : st;
}

hf_status hf_block_select(const hf_dims *d, const void *q, const hf_kv_ring *ring, int32_t top_k, int32_t *idx,
                          double *scores, void *ws, size_t ws_bytes, hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_ring(d, ring);
    if (st != HF_OK) return st;
    if (!q || !idx) return fail(HF_ERR_NULL, "q/idx is NULL");
    const Geometry g = geometry(d, ring);
    if (top_k < 1 || top_k > g.nkb) return fail(HF_ERR_SHAPE, "top_k=%d outside [1, n_kb=%d]", top_k, g.nkb);
    st = check_ws(d, ws, ws_bytes);
    if (st != HF_OK) return st;
    st = hip_status(enqueue_select(d, q, ring, top_k, idx, scores, ws, stream), "block select launch");
    return st == HF_OK ? ok() : st;
}

hf_status hf_block_select_hier(const hf_dims *d, const void *q, const hf_kv_ring *ring, int32_t top_frames,
                               int32_t top_k, int32_t *idx, int32_t *frames, double *scores, double *frame_scores,
                               void *ws, size_t ws_bytes, hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_ring(d, ring);
    if (st != HF_OK) return st;
    if (!q || !idx) return fail(HF_ERR_NULL, "q/idx is NULL");
    const Geometry g = geometry(d, ring);
    const int nfr = ring->n_committed + d->C;
    if (nfr > kMaxHierFrames)
        return fail(HF_ERR_UNSUPPORTED, "window of %d frames exceeds %d for the hierarchical selection", nfr,
                    kMaxHierFrames);
    if (d->bk > d->T) return fail(HF_ERR_UNSUPPORTED, "hierarchical selection needs bk <= T (bk=%d T=%d)", d->bk, d->T);
    if (top_frames < 1 || top_frames > nfr)
        return fail(HF_ERR_SHAPE, "top_frames=%d outside [1, frames in the window=%d]", top_frames, nfr);
    // any top_frames distinct frames touch at least this many key blocks
    const int64_t per_frame = cdiv(d->T, d->bk);
    const int64_t least = (int64_t)top_frames * per_frame - (top_frames - 1);
    const int64_t kmax = least < g.nkb ? least : g.nkb;
    if (top_k < 1 || top_k > kmax)
        return fail(HF_ERR_SHAPE, "top_k=%d outside [1, %lld] (key blocks guaranteed inside %d frames)", top_k,
                    (long long)kmax, top_frames);
    st = check_ws(d, ws, ws_bytes);
    if (st != HF_OK) return st;
    st = hip_status(enqueue_select(d, q, ring, top_k, idx, scores, ws, stream, top_frames, frames, frame_scores),
                    "hierarchical block select launch");
    return st == HF_OK ? ok() : st;
}

static hf_status check_rope(const hf_dims *d, const hf_rope *r) {
    if (!r) return fail(HF_ERR_NULL, "rope is NULL");
    const int dt = r->temporal_dims;
    if (dt != 16 && dt != 32) return fail(HF_ERR_SHAPE, "rope temporal_dims=%d: need 16 or 32", dt);
    if (r->cap < 0 || r->cap > 1024) return fail(HF_ERR_SHAPE, "rope cap=%d outside [0, 1024]", r->cap);
    if (!(r->base > 1.f) || !std::isfinite(r->base)) return fail(HF_ERR_SHAPE, "rope base must be finite and > 1");
    return HF_OK;
}

static hf_status sparse_window_attn(const hf_dims *d, const void *q, const hf_kv_ring *ring, const int32_t *idx,
                                    int32_t top_k, const float *S, const float *z, float eps, float *out, float *lse,
                                    void *ws, size_t ws_bytes, hipStream_t stream, const hf_rope *rope = nullptr) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_ring(d, ring);
    if (st != HF_OK) return st;
    if (!q || !idx || !out) return fail(HF_ERR_NULL, "q/idx/out is NULL");
    if ((S == nullptr) != (z == nullptr)) return fail(HF_ERR_NULL, "S and z must both be given or both be NULL");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(HF_ERR_SHAPE, "eps must be finite and >= 0");
    const Geometry g = geometry(d, ring);
    if (top_k < 1 || top_k > g.nkb) return fail(HF_ERR_SHAPE, "top_k=%d outside [1, n_kb=%d]", top_k, g.nkb);
    st = check_ws(d, ws, ws_bytes);
    if (st != HF_OK) return st;
    hipError_t e = S ? enqueue_state(d, const_cast<float *>(S), const_cast<float *>(z), true, 0, ws, stream) : hipSuccess;
    if (e == hipSuccess) e = enqueue_attn(d, q, ring, idx, top_k, S != nullptr, eps, out, ws, stream, lse, rope);
    st = hip_status(e, "sparse attention launch");
    return st == HF_OK ? ok() : st;
}

hf_status hf_sparse_window_attn(const hf_dims *d, const void *q, const hf_kv_ring *ring, const int32_t *idx,
                                int32_t top_k, const float *S, const float *z, float eps, float *out, void *ws,
                                size_t ws_bytes, hipStream_t stream) {
    return sparse_window_attn(d, q, ring, idx, top_k, S, z, eps, out, nullptr, ws, ws_bytes, stream);
}

hf_status hf_sparse_window_attn_lse(const hf_dims *d, const void *q, const hf_kv_ring *ring, const int32_t *idx,
                                    int32_t top_k, const float *S, const float *z, float eps, float *out, float *lse,
                                    void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!lse) return fail(HF_ERR_NULL, "lse is NULL");
    return sparse_window_attn(d, q, ring, idx, top_k, S, z, eps, out, lse, ws, ws_bytes, stream);
}

hf_status hf_sparse_window_attn_rope(const hf_dims *d, const void *q, const hf_kv_ring *ring, const int32_t *idx,
                                     int32_t top_k, const float *S, const float *z, float eps, const hf_rope *rope,
                                     float *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_rope(d, rope);
    if (st != HF_OK) return st;
    return sparse_window_attn(d, q, ring, idx, top_k, S, z, eps, out, nullptr, ws, ws_bytes, stream, rope);
}

hf_status hf_backward_workspace_size(const hf_dims *d, int32_t top_k, size_t *bytes) {
    hf_status st = check_dims(d);
    if (st != HF_OK) return st;
    if (!bytes) return fail(HF_ERR_NULL, "bytes is NULL");
    const int64_t nkb = cdiv((int64_t)d->W * d->T, d->bk);
    if (top_k < 1 || top_k > nkb) return fail(HF_ERR_SHAPE, "top_k=%d outside [1, %lld]", top_k, (long long)nkb);
    *bytes = hf_bwd_workspace_bytes(d->B * d->H, d->D, d->C * d->T, d->W * d->T, d->bq, d->bk, top_k);
    return ok();
}

hf_status hf_hybrid_attn_backward(const hf_dims *d, const void *q, const hf_kv_ring *ring, const int32_t *idx,
                                  int32_t top_k, const float *S, const float *z, float eps, const float *out,
                                  const float *lse, const float *dout, float *dq, float *dk, float *dv, float *dS,
                                  float *dz, void *ws, size_t ws_bytes, hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_ring(d, ring);
    if (st != HF_OK) return st;
    if (!q || !idx || !S || !z || !out || !lse || !dout) return fail(HF_ERR_NULL, "an input pointer is NULL");
    if (!dq || !dk || !dv || !dS || !dz) return fail(HF_ERR_NULL, "an output pointer is NULL");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(HF_ERR_SHAPE, "eps must be finite and >= 0");
    const Geometry g = geometry(d, ring);
    if (top_k < 1 || top_k > g.nkb) return fail(HF_ERR_SHAPE, "top_k=%d outside [1, n_kb=%d]", top_k, g.nkb);
    const size_t need = hf_bwd_workspace_bytes(g.BH, d->D, g.Nq, g.Nk, d->bq, d->bk, top_k);
    if (!ws) return fail(HF_ERR_WORKSPACE, "backward workspace is NULL (need %zu bytes)", need);
    if (ws_bytes < need) return fail(HF_ERR_WORKSPACE, "backward workspace of %zu bytes, need %zu", ws_bytes, need);
    hf_bwd_args a{};
    a.BH = g.BH;
    a.D = d->D;
    a.T = d->T;
    a.W = d->W;
    a.head = ring->head;
    a.Nq = g.Nq;
    a.Nk = g.Nk;
    a.bq = d->bq;
    a.bk = d->bk;
    a.nqb = g.nqb;
    a.nkb = g.nkb;
    a.top_k = top_k;
    a.q = static_cast<const uint16_t *>(q);
    a.ring_k = static_cast<const uint16_t *>(ring->k_dev);
    a.ring_vg = static_cast<const uint16_t *>(ring->vg_dev);
    a.idx = idx;
    a.S = S;
    a.z = z;
    a.out = out;
    a.lse = lse;
    a.dout = dout;
    a.eps = eps;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dS = dS;
    a.dz = dz;
    hf_bwd_layout(a, ws);
    st = hip_status(hf_launch_attn_backward(a, stream), "backward launch");
    return st == HF_OK ? ok() : st;
}

hf_status hf_linear_absorb_backward(const hf_dims *d, const void *k_ev, const void *v_ev, int64_t n_tok,
                                    const float *dS, const float *dz, float *dk, float *dv, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st != HF_OK) return st;
    if (n_tok < 0) return fail(HF_ERR_SHAPE, "n_tok=%lld < 0", (long long)n_tok);
    if (!dS || !dz) return fail(HF_ERR_NULL, "dS/dz is NULL");
    if (n_tok > 0 && (!k_ev || !v_ev || !dk || !dv)) return fail(HF_ERR_NULL, "k_ev/v_ev/dk/dv is NULL");
    if ((int64_t)d->B * d->H * n_tok * d->D >= kMaxElems)
        return fail(HF_ERR_UNSUPPORTED, "evicted tensors exceed 2^31 elements");
    st = check_ws(d, ws, ws_bytes);
    if (st != HF_OK) return st;
    if (ws_bytes < (size_t)4 * d->B * d->H * d->D * d->D)
        return fail(HF_ERR_WORKSPACE, "workspace of %zu bytes is below 4 B H D^2", ws_bytes);
    if (n_tok == 0) return ok();
    hf_absorb_bwd_args a{};
    a.BH = d->B * d->H;
    a.D = d->D;
    a.n_tok = n_tok;
    a.k = static_cast<const uint16_t *>(k_ev);
    a.v = static_cast<const uint16_t *>(v_ev);
    a.dS = dS;
    a.dz = dz;
    a.sb = static_cast<uint16_t *>(ws);
    a.stb = a.sb + (size_t)a.BH * d->D * d->D;
    a.dk = dk;
    a.dv = dv;
    st = hip_status(hf_launch_absorb_backward(a, stream), "absorb backward launch");
    return st == HF_OK ? ok() : st;
}

hf_status hf_linear_absorb(const hf_dims *d, const void *k_ev, const void *v_ev, int64_t n_tok, float *S, float *z,
                           void *ws, size_t ws_bytes, hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st != HF_OK) return st;
    if (n_tok < 0) return fail(HF_ERR_SHAPE, "n_tok=%lld < 0", (long long)n_tok);
    if (!S || !z) return fail(HF_ERR_NULL, "S/z is NULL");
    if (n_tok > 0 && (!k_ev || !v_ev)) return fail(HF_ERR_NULL, "k_ev/v_ev is NULL");
    if ((int64_t)d->B * d->H * n_tok * d->D >= kMaxElems)
        return fail(HF_ERR_UNSUPPORTED, "evicted tensors exceed 2^31 elements");
    st = check_ws(d, ws, ws_bytes);
    if (st != HF_OK) return st;
    if (n_tok == 0) return ok();
    hipError_t e = enqueue_absorb_partial(d, k_ev, v_ev, n_tok, ws, stream);
    if (e == hipSuccess) e = enqueue_state(d, S, z, false, n_tok, ws, stream);
    st = hip_status(e, "absorb launch");
    return st == HF_OK ? ok() : st;
}

}  // extern "C"

// Validation of a step's arguments, workspace aside (sets the error message).
hf_status hf_step_validate(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur,
                           const hf_kv_ring *ring, int32_t top_k, uint32_t flags, const float *S, const float *z,
                           float eps, const int32_t *idx, const float *out) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_ring(d, ring);
    if (st != HF_OK) return st;
    if (!q || !idx || !out) return fail(HF_ERR_NULL, "q/idx/out is NULL");
    if ((k_cur == nullptr) != (v_cur == nullptr)) return fail(HF_ERR_NULL, "give both k_cur and v_cur or neither");
    if ((S == nullptr) != (z == nullptr)) return fail(HF_ERR_NULL, "S and z must both be given or both be NULL");
    if ((flags & HF_STEP_COMMIT) && !S) return fail(HF_ERR_NULL, "HF_STEP_COMMIT needs S and z");
    if (flags & ~HF_STEP_COMMIT) return fail(HF_ERR_SHAPE, "unknown flags 0x%x", flags);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(HF_ERR_SHAPE, "eps must be finite and >= 0");
    const Geometry g = geometry(d, ring);
    if (top_k < 1 || top_k > g.nkb) return fail(HF_ERR_SHAPE, "top_k=%d outside [1, n_kb=%d]", top_k, g.nkb);
    return HF_OK;
}

// Bytes at the start of the workspace layout that a step uses (everything before the
// hierarchical selection's buffers); dims already validated.
size_t hf_step_workspace_bytes(const hf_dims *d) { return ws_layout(d).fbar; }

hf_status hf_fail_unsupported(const char *msg, size_t need, size_t have) {
    return fail(HF_ERR_UNSUPPORTED, "%s: needs %zu bytes, holds %zu", msg, need, have);
}

hf_status hf_fail_hip(hipError_t e, const char *what) { return hip_status(e, what); }

// Enqueue a validated step on `ws` (at least hf_step_workspace_bytes bytes).
hf_status hf_step_enqueue(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur, hf_kv_ring *ring,
                          int32_t top_k, uint32_t flags, float *S, float *z, float eps, const hf_rope *rope,
                          int32_t *idx, float *out, void *ws, const hf_step_events *events, hipStream_t stream) {
    // Order: select -- its pool launch also takes the readout operands from the state as it
    // is, its score + top-k launch also appends the chunk to the ring; attention with the
    // fused readout, whose launch also forms the absorb partials of the frames this step
    // evicts (still in the ring until the next append); the state pass that adds them.
    hf_kv_ring next = *ring;
    int evict = 0;
    if (flags & HF_STEP_COMMIT) {
        next.n_committed += d->C;
        evict = next.n_committed - (d->W - d->C);
        if (evict < 0) evict = 0;
        next.head = (next.head + evict) % d->W;
        next.n_committed -= evict;
    }
    const int64_t evict_tok = (int64_t)evict * d->T;
    hipError_t e = record(events, 0, stream);
    if (e == hipSuccess) e = record(events, 1, stream);
    // the readout operands are extra workgroups of the selection's pool launch (which reads
    // the current chunk's keys from k_cur), the ring append those of its score launch
    const hf_state_args prep = S ? state_args(d, S, z, true, 0, ws) : hf_state_args{};
    const hf_append_args app = k_cur ? append_args(d, ring, k_cur, v_cur) : hf_append_args{};
    if (e == hipSuccess)
        e = enqueue_select(d, q, ring, top_k, idx, nullptr, ws, stream, 0, nullptr, nullptr, S ? &prep : nullptr,
                           k_cur ? &app : nullptr);
    if (e == hipSuccess) e = record(events, 2, stream);
    if (e == hipSuccess) e = record(events, 3, stream);
    // attention with the fused readout; extra workgroups of the same launch form the split
    // partial sums of the evicted frames (the oldest window frames, which the append does not
    // touch), beside the attention -- the readout reads the copy of the state the pool launch
    // made -- and the state pass adds them to (S, z) in split order
    if (e == hipSuccess)
        e = enqueue_attn(d, q, ring, idx, top_k, S != nullptr, eps, out, ws, stream, nullptr, rope, evict_tok);
    if (e == hipSuccess) e = record(events, 4, stream);
    if (e == hipSuccess && evict_tok > 0) e = enqueue_state(d, S, z, false, evict_tok, ws, stream, true);
    if (e == hipSuccess) e = record(events, 5, stream);
    if (e != hipSuccess) return hip_status(e, "hybrid step launch");
    *ring = next;
    return ok();
}

static hf_status hybrid_step(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur, hf_kv_ring *ring,
                             int32_t top_k, uint32_t flags, float *S, float *z, float eps, const hf_rope *rope,
                             int32_t *idx, float *out, void *ws, size_t ws_bytes, const hf_step_events *events,
                             hipStream_t stream) {
    hf_status st = hf_step_validate(d, q, k_cur, v_cur, ring, top_k, flags, S, z, eps, idx, out);
    if (st == HF_OK) st = check_ws(d, ws, ws_bytes);
    if (st != HF_OK) return st;
    return hf_step_enqueue(d, q, k_cur, v_cur, ring, top_k, flags, S, z, eps, rope, idx, out, ws, events, stream);
}

extern "C" {

hf_status hf_hybrid_step(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur, hf_kv_ring *ring,
                         int32_t top_k, uint32_t flags, float *S, float *z, float eps, int32_t *idx, float *out,
                         void *ws, size_t ws_bytes, const hf_step_events *events, hipStream_t stream) {
    return hybrid_step(d, q, k_cur, v_cur, ring, top_k, flags, S, z, eps, nullptr, idx, out, ws, ws_bytes, events,
                       stream);
}

hf_status hf_hybrid_step_rope(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur, hf_kv_ring *ring,
                              int32_t top_k, uint32_t flags, float *S, float *z, float eps, const hf_rope *rope,
                              int32_t *idx, float *out, void *ws, size_t ws_bytes, const hf_step_events *events,
                              hipStream_t stream) {
    hf_status st = check_dims(d);
    if (st == HF_OK) st = check_rope(d, rope);
    if (st != HF_OK) return st;
    return hybrid_step(d, q, k_cur, v_cur, ring, top_k, flags, S, z, eps, rope, idx, out, ws, ws_bytes, events,
                       stream);
}

}  // extern "C"
