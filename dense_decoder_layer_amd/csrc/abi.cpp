// The C ABI: admission, weight packing, workspace planning, the prefill
// stack runner and the device KV mirror.  Host logic only; every step of the
// layer runs in the kernels launched from here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "internal.h"

#include <algorithm>

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Why a layer is not served, or nullptr when it is ("frink-models 0.29.0
// src/decoder/cuda_prefill.rs", try_cuda_prefill_dense_stack and
// cuda_prefill_layer; "frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_shape_ok; "frink-models 0.49.0 src/fused_layer.rs",
// "What it refuses").
const char* why_unsupported(const ddl_layer_desc* d) {
    if (!d) return "null layer description";
    if (d->d_model <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 ||
        d->d_ff <= 0)
        return "non-positive shape";
    if (d->act != DDL_ACT_SWIGLU && d->act != DDL_ACT_GELU) return "unknown FFN activation";
    if (d->post_norm_eps != d->rms_eps) return "post-norm epsilon differs from rms_eps";
    if (d->v_head_dim != d->head_dim) return "v_head_dim differs from head_dim";
    if (d->window < 0) return "negative sliding window";
    if (d->has_sinks) return "attention sinks";
    if (d->has_alibi) return "ALiBi";
    if (d->has_lora) return "LoRA adapter attached";
    if (d->rope_enabled) {
        const int rd = d->rope_rot_dim == 0 ? d->head_dim : d->rope_rot_dim;
        if (d->rope_layout != DDL_ROPE_NEOX && d->rope_layout != DDL_ROPE_NORM)
            return "unknown RoPE layout";
        if (rd < 2 || rd % 2 || rd > d->head_dim) return "RoPE width not even or above head_dim";
        // a thread of the QKV post-step holds channels e and e + 32k of a head
        if (d->rope_layout == DDL_ROPE_NEOX && (rd / 2) % 32)
            return "Neox RoPE width not a multiple of 64";
        if (!std::isfinite(d->rope_mscale)) return "RoPE attention factor not finite";
        if (!(d->rope_theta > 0.0)) return "RoPE theta not positive";
        if (d->rope_freq_factors)
            for (int i = 0; i < rd / 2; ++i)
                if (!(d->rope_freq_factors[i] > 0.0f) || !std::isfinite(d->rope_freq_factors[i]))
                    return "RoPE frequency factor not positive and finite";
    }
    if (d->head_dim != 64 && d->head_dim != 128) return "head_dim other than 64 or 128";
    if (d->n_heads % d->n_kv_heads != 0) return "n_heads not a multiple of n_kv_heads";
    if (d->d_model % 128 != 0) return "d_model not a multiple of 128";
    if (d->d_model > 4096) return "d_model above 4096 (the row norm holds a row in registers)";
    if (d->d_ff % 64 != 0) return "d_ff not a multiple of 64";
    if (!(d->attn_softcap >= 0.0f)) return "negative softcap";
    const int nqkv = (d->gated ? 2 : 1) * d->n_heads * d->head_dim + 2 * d->n_kv_heads * d->head_dim;
    if (nqkv % 128 != 0) return "q/k/v width not a multiple of 128";
    return nullptr;
}

struct BlobLayout {
    size_t hdr, g_attn, g_ffn, bqkv, qn, kn, freq, gpa, gpf, wqkv, wo, wgu, wd, total;
    int nqkv;
};

void blob_layout(const ddl_layer_desc* d, BlobLayout* L) {
    const size_t dm = d->d_model, qw = (size_t)d->n_heads * d->head_dim,
                 kw = (size_t)d->n_kv_heads * d->head_dim, f = d->d_ff;
    L->nqkv = (int)((d->gated ? 2 : 1) * qw + 2 * kw);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    L->hdr = take(sizeof(BlobHeader));
    L->g_attn = take(dm * 4);
    L->g_ffn = take(dm * 4);
    L->bqkv = take(d->has_qkv_bias ? (size_t)L->nqkv * 4 : 0);
    L->qn = take(d->has_qk_norm ? (size_t)d->head_dim * 4 : 0);
    L->kn = take(d->has_qk_norm ? (size_t)d->head_dim * 4 : 0);
    const int rd = d->rope_rot_dim == 0 ? d->head_dim : d->rope_rot_dim;
    L->freq = take(d->rope_enabled && d->rope_freq_factors ? (size_t)(rd / 2) * 4 : 0);
    L->gpa = take(d->has_post_attn_norm ? dm * 4 : 0);
    L->gpf = take(d->has_post_ffn_norm ? dm * 4 : 0);
    L->wqkv = take((size_t)L->nqkv * dm * 2);
    L->wo = take(dm * qw * 2);
    L->wgu = take(2 * f * dm * 2);
    L->wd = take(dm * f * 2);
    L->total = o;
}

// Per-call scratch in the caller's workspace.
struct WsLayout {
    size_t rope, h, qkv, q16, o16, x1, a16, k16, vt16, part, total;
    int tcap;
};

int staged_rows(int B, int S) {
    const int nblk = (B + 31) / 32;
    return ((S + 32 * (nblk + 1)) + 31) / 32 * 32;
}

WsLayout ws_layout(const ddl_layer* L, int B, int S) {
    WsLayout w;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    w.tcap = staged_rows(B, S);
    w.rope = take((size_t)B * (L->hd / 2) * sizeof(float2));
    w.h = take((size_t)B * L->d * 2);
    w.qkv = take((size_t)B * L->nqkv * 4);
    w.q16 = take((size_t)B * L->hq * L->hd * 2);
    w.o16 = take((size_t)B * L->hq * L->hd * 2);
    w.x1 = take((size_t)B * L->d * 4);
    w.a16 = take((size_t)B * L->f * 2);
    w.k16 = take((size_t)L->hkv * w.tcap * L->hd * 2);
    w.vt16 = take((size_t)L->hkv * w.tcap * L->hd * 2);
    // split-K partials, reused by the QKV, wo and down projections in turn.
    // A smaller batch may split more ways, so the region covers every batch
    // up to B (the split only changes at multiples of the 64-row tile).
    size_t part = 0;
    for (int b = 64; b < B + 64; b += 64) {
        const int bb = std::min(b, B);
        const size_t pq = (size_t)(gemm_splits(bb, L->nqkv, L->d, EPI_F32) - 1) * bb * L->nqkv;
        const size_t po = (size_t)(gemm_splits(bb, L->d, L->hq * L->hd, EPI_RESID) - 1) * bb * L->d;
        const size_t pd = (size_t)(gemm_splits(bb, L->d, L->f, EPI_RESID) - 1) * bb * L->d;
        part = std::max(part, std::max(pq, std::max(po, pd)));
    }
    w.part = take(part * 4);
    w.total = o;
    return w;
}

// Layers of one run share the shapes the workspace is laid out for and the
// model's one epsilon (a norm kernel may finish one layer and start the
// next); per-layer options (RoPE, activation, window, softcap, extras,
// sandwich norms) may differ.
bool same_run_shape(const ddl_layer* a, const ddl_layer* b) {
    return a->d == b->d && a->hq == b->hq && a->hkv == b->hkv && a->hd == b->hd && a->f == b->f &&
           a->gated == b->gated && a->eps == b->eps;
}

// Two rotating layers whose position tables are the same.
bool same_rope(const ddl_layer* a, const ddl_layer* b) {
    return a->rope_on && b->rope_on && a->theta == b->theta && a->rot_dim == b->rot_dim &&
           a->mscale == b->mscale && a->freq_host == b->freq_host;
}

size_t elem_bytes(int dtype) { return dtype == DDL_DTYPE_BF16 ? 2 : 4; }

const void* offset_rows(const void* p, int dtype, size_t elems) {
    return static_cast<const char*>(p) + elems * elem_bytes(dtype);
}

}  // namespace

extern "C" {

const char* ddl_last_error(void) { return g_err.c_str(); }

ddl_ctx* ddl_ctx_create(const ddl_ctx_opts* opts) {
    ddl_ctx* c = new (std::nothrow) ddl_ctx;
    if (!c) return nullptr;
    c->min_batch = 4;
    c->fault_after_admission = 0;
    c->attn_form = DDL_ATTN_AUTO;
    if (opts) {
        if (opts->min_batch > 0) c->min_batch = opts->min_batch;
        c->fault_after_admission = opts->fault_after_admission;
        if (opts->attn_form == DDL_ATTN_ONE_HEAD || opts->attn_form == DDL_ATTN_SHARED)
            c->attn_form = opts->attn_form;
    }
    return c;
}

namespace {
void probe_release(ddl_ctx* c) {
    for (hipEvent_t e : c->probe_events) hipEventDestroy(e);
    c->probe_events.clear();
    c->probe_kind = -1;
    c->probe_max = c->probe_count = 0;
}
}  // namespace

void ddl_ctx_destroy(ddl_ctx* ctx) {
    if (!ctx) return;
    probe_release(ctx);
    delete ctx;
}

int ddl_probe_enable(ddl_ctx* ctx, int kind, int max_launches) {
    if (!ctx || kind < 0 || kind >= DDL_K_COUNT || max_launches < 0)
        return fail(DDL_ERR_INVALID, "bad probe arguments");
    probe_release(ctx);
    if (max_launches == 0) return 1;
    ctx->probe_events.resize(2 * (size_t)max_launches, nullptr);
    for (hipEvent_t& e : ctx->probe_events) {
        if (hipEventCreate(&e) != hipSuccess) {
            probe_release(ctx);
            return fail(DDL_ERR_DEVICE, "hipEventCreate failed");
        }
    }
    ctx->probe_kind = kind;
    ctx->probe_max = max_launches;
    return 1;
}

int ddl_probe_read(ddl_ctx* ctx, float* ms_out, int cap) {
    if (!ctx || (cap > 0 && !ms_out)) return fail(DDL_ERR_INVALID, "bad probe arguments");
    const int n = ctx->probe_count;
    for (int i = 0; i < n; ++i) {
        hipError_t e = hipEventSynchronize(ctx->probe_events[2 * i + 1]);
        float ms = 0.f;
        if (!e) e = hipEventElapsedTime(&ms, ctx->probe_events[2 * i], ctx->probe_events[2 * i + 1]);
        if (e) return fail(DDL_ERR_DEVICE, std::string("probe: ") + hipGetErrorString(e));
        if (i < cap) ms_out[i] = ms;
    }
    ctx->probe_count = 0;
    return n;
}

int ddl_layer_supported(const ddl_layer_desc* desc) {
    const char* why = why_unsupported(desc);
    if (why) {
        g_err = why;
        return 0;
    }
    return 1;
}

size_t ddl_layer_blob_bytes(const ddl_layer_desc* desc) {
    if (why_unsupported(desc)) return 0;
    BlobLayout L;
    blob_layout(desc, &L);
    return L.total;
}

int ddl_layer_pack(ddl_ctx* ctx, const ddl_layer_desc* d, const ddl_layer_weights* w,
                   void* dev_blob, size_t blob_bytes, void* stream, ddl_layer** out) {
    if (!ctx || !out) return fail(DDL_ERR_INVALID, "null context or output handle");
    if (const char* why = why_unsupported(d)) return fail(DDL_DECLINED, why);
    if (!w || !dev_blob) return fail(DDL_ERR_INVALID, "null weights or blob");
    if (w->dtype != DDL_DTYPE_F32 && w->dtype != DDL_DTYPE_BF16)
        return fail(DDL_ERR_INVALID, "unknown weight dtype");
    if (!w->wq || !w->wk || !w->wv || !w->wo || !w->wg || !w->wu || !w->wd || !w->g_attn ||
        !w->g_ffn)
        return fail(DDL_ERR_INVALID, "a required weight pointer is null");
    if (d->has_qkv_bias && (!w->bq || !w->bk || !w->bv))
        return fail(DDL_ERR_INVALID, "q/k/v bias pointers are null");
    if (d->has_qk_norm && (!w->q_norm || !w->k_norm))
        return fail(DDL_ERR_INVALID, "q/k norm pointers are null");
    if ((d->has_post_attn_norm && !w->g_post_attn) || (d->has_post_ffn_norm && !w->g_post_ffn))
        return fail(DDL_ERR_INVALID, "post-norm gain pointers are null");
    BlobLayout B;
    blob_layout(d, &B);
    if (blob_bytes < B.total) return fail(DDL_ERR_INVALID, "blob smaller than ddl_layer_blob_bytes");
    if ((reinterpret_cast<uintptr_t>(dev_blob) & 255) != 0)
        return fail(DDL_ERR_INVALID, "blob not 256-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(dev_blob);
    ddl_layer* L = new (std::nothrow) ddl_layer;
    if (!L) return fail(DDL_ERR_INVALID, "out of host memory");
    L->d = d->d_model;
    L->hq = d->n_heads;
    L->hkv = d->n_kv_heads;
    L->hd = d->head_dim;
    L->f = d->d_ff;
    L->nqkv = B.nqkv;
    L->gated = d->gated;
    L->has_bias = d->has_qkv_bias;
    L->has_qk_norm = d->has_qk_norm;
    L->rope_on = d->rope_enabled;
    L->act = d->act;
    L->window = d->window;
    L->eps = d->rms_eps;
    L->softcap = d->attn_softcap;
    L->theta = d->rope_theta;
    L->rope_layout = d->rope_layout;
    L->rot_dim = d->rope_rot_dim == 0 ? d->head_dim : d->rope_rot_dim;
    L->mscale = d->rope_mscale;
    L->freq = nullptr;
    if (d->rope_enabled && d->rope_freq_factors) {
        L->freq_host.assign(d->rope_freq_factors, d->rope_freq_factors + L->rot_dim / 2);
        L->freq = reinterpret_cast<float*>(base + B.freq);
    }
    L->blob_bytes = B.total;
    L->hdr = reinterpret_cast<BlobHeader*>(base + B.hdr);
    L->g_attn = reinterpret_cast<float*>(base + B.g_attn);
    L->g_ffn = reinterpret_cast<float*>(base + B.g_ffn);
    L->bqkv = d->has_qkv_bias ? reinterpret_cast<float*>(base + B.bqkv) : nullptr;
    L->q_norm = d->has_qk_norm ? reinterpret_cast<float*>(base + B.qn) : nullptr;
    L->k_norm = d->has_qk_norm ? reinterpret_cast<float*>(base + B.kn) : nullptr;
    L->g_post_attn = d->has_post_attn_norm ? reinterpret_cast<float*>(base + B.gpa) : nullptr;
    L->g_post_ffn = d->has_post_ffn_norm ? reinterpret_cast<float*>(base + B.gpf) : nullptr;
    L->wqkv = reinterpret_cast<f16*>(base + B.wqkv);
    L->wo = reinterpret_cast<f16*>(base + B.wo);
    L->wgu = reinterpret_cast<f16*>(base + B.wgu);
    L->wd = reinterpret_cast<f16*>(base + B.wd);

    const int dt = w->dtype;
    const size_t dm = L->d, qw = (size_t)L->hq * L->hd, kw = (size_t)L->hkv * L->hd, f = L->f;
    const size_t wq_rows = (L->gated ? 2 : 1) * qw;
    hipError_t e = hipMemsetAsync(L->hdr, 0, sizeof(BlobHeader), s);
    uint32_t* amax = L->hdr->absmax_bits;
    if (!e) e = launch_absmax(w->wq, dt, wq_rows * dm, amax + MAT_QKV, s);
    if (!e) e = launch_absmax(w->wk, dt, kw * dm, amax + MAT_QKV, s);
    if (!e) e = launch_absmax(w->wv, dt, kw * dm, amax + MAT_QKV, s);
    if (!e) e = launch_absmax(w->wo, dt, dm * qw, amax + MAT_O, s);
    if (!e) e = launch_absmax(w->wg, dt, f * dm, amax + MAT_GU, s);
    if (!e) e = launch_absmax(w->wu, dt, f * dm, amax + MAT_GU, s);
    if (!e) e = launch_absmax(w->wd, dt, dm * f, amax + MAT_D, s);
    if (!e) e = launch_finalize_scales(L->hdr, s);
    // stacked q/k/v(/gate) rows
    if (!e) e = launch_convert_rows(w->wq, dt, (int)qw, (int)dm, L->wqkv, 0, 0, L->hdr, MAT_QKV, s);
    if (!e) e = launch_convert_rows(w->wk, dt, (int)kw, (int)dm, L->wqkv, (int)qw, 0, L->hdr, MAT_QKV, s);
    if (!e) e = launch_convert_rows(w->wv, dt, (int)kw, (int)dm, L->wqkv, (int)(qw + kw), 0, L->hdr, MAT_QKV, s);
    if (!e && L->gated)
        e = launch_convert_rows(offset_rows(w->wq, dt, qw * dm), dt, (int)qw, (int)dm, L->wqkv,
                                (int)(qw + 2 * kw), 0, L->hdr, MAT_QKV, s);
    if (!e) e = launch_convert_rows(w->wo, dt, (int)dm, (int)qw, L->wo, 0, 0, L->hdr, MAT_O, s);
    if (!e) e = launch_convert_rows(w->wg, dt, (int)f, (int)dm, L->wgu, 0, 1, L->hdr, MAT_GU, s);
    if (!e) e = launch_convert_rows(w->wu, dt, (int)f, (int)dm, L->wgu, 0, 2, L->hdr, MAT_GU, s);
    if (!e) e = launch_convert_rows(w->wd, dt, (int)dm, (int)f, L->wd, 0, 0, L->hdr, MAT_D, s);
    if (!e) e = hipMemcpyAsync(L->g_attn, w->g_attn, dm * 4, hipMemcpyDefault, s);
    if (!e) e = hipMemcpyAsync(L->g_ffn, w->g_ffn, dm * 4, hipMemcpyDefault, s);
    if (!e && L->has_bias) {
        e = hipMemsetAsync(L->bqkv, 0, (size_t)L->nqkv * 4, s);
        if (!e) e = hipMemcpyAsync(L->bqkv, w->bq, qw * 4, hipMemcpyDefault, s);
        if (!e) e = hipMemcpyAsync(L->bqkv + qw, w->bk, kw * 4, hipMemcpyDefault, s);
        if (!e) e = hipMemcpyAsync(L->bqkv + qw + kw, w->bv, kw * 4, hipMemcpyDefault, s);
    }
    if (!e && L->g_post_attn)
        e = hipMemcpyAsync(L->g_post_attn, w->g_post_attn, dm * 4, hipMemcpyDefault, s);
    if (!e && L->g_post_ffn)
        e = hipMemcpyAsync(L->g_post_ffn, w->g_post_ffn, dm * 4, hipMemcpyDefault, s);
    if (!e && L->freq)   // from the handle's own copy: the caller's array may go away
        e = hipMemcpyAsync(L->freq, L->freq_host.data(), L->freq_host.size() * 4,
                           hipMemcpyHostToDevice, s);
    if (!e && L->has_qk_norm) {
        e = hipMemcpyAsync(L->q_norm, w->q_norm, (size_t)L->hd * 4, hipMemcpyDefault, s);
        if (!e) e = hipMemcpyAsync(L->k_norm, w->k_norm, (size_t)L->hd * 4, hipMemcpyDefault, s);
    }
    if (e) {
        delete L;
        return fail(DDL_ERR_DEVICE, std::string("pack: ") + hipGetErrorString(e));
    }
    *out = L;
    return 1;
}

void ddl_layer_destroy(ddl_layer* layer) { delete layer; }

size_t ddl_workspace_bytes(const ddl_layer* const* layers, int n, int max_batch,
                           int max_start_pos) {
    if (!layers || n <= 0 || max_batch <= 0 || max_start_pos < 0) return 0;
    size_t need = 0;
    for (int i = 0; i < n; ++i) {
        if (!layers[i]) return 0;
        const size_t t = ws_layout(layers[i], max_batch, max_start_pos).total;
        if (t > need) need = t;
    }
    return need;
}

int ddl_prefill_dense_stack(ddl_ctx* ctx, const float* hidden, const ddl_layer* const* layers,
                            int n_layers, int batch, int start_pos, const float* const* prefix_k,
                            const float* const* prefix_v, const int* prefix_rows,
                            float* hidden_out, float* const* k_rows, float* const* v_rows,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (!ctx || !layers || n_layers <= 0 || !hidden || !hidden_out || !k_rows || !v_rows ||
        !prefix_rows)
        return fail(DDL_ERR_INVALID, "null argument");
    if (start_pos < 0) return fail(DDL_ERR_INVALID, "negative start_pos");
    if (batch < ctx->min_batch || batch <= 0)
        return fail(DDL_DECLINED, "batch below the context's min_batch");
    if (!layers[0]) return fail(DDL_ERR_INVALID, "null layer 0");

    // The longest run of consecutive layers this call serves.
    int run = 0;
    std::string stop;
    for (int l = 0; l < n_layers; ++l) {
        const ddl_layer* L = layers[l];
        if (!L) { stop = "null layer"; break; }
        if (prefix_rows[l] != start_pos) { stop = "cache rows differ from start_pos"; break; }
        if (l > 0 && !same_run_shape(L, layers[0])) { stop = "layer shape differs from the run"; break; }
        if (start_pos > 0 && (!prefix_k || !prefix_v || !prefix_k[l] || !prefix_v[l]))
            return fail(DDL_ERR_INVALID, "null prefix pointer with start_pos > 0");
        if (!k_rows[l] || !v_rows[l]) return fail(DDL_ERR_INVALID, "null K/V row output");
        ++run;
    }
    if (run == 0) return fail(DDL_DECLINED, "layer 0 not served: " + stop);
    const ddl_layer* L0 = layers[0];
    if (!gemm_shape_ok(batch, L0->nqkv, L0->d, EPI_F32))
        return fail(DDL_DECLINED, "shape not served by the GEMM tiles");
    const WsLayout W = ws_layout(L0, batch, start_pos);
    if (!workspace || workspace_bytes < W.total)
        return fail(DDL_ERR_WORKSPACE, "workspace smaller than ddl_workspace_bytes");
    if (ctx->fault_after_admission)
        return fail(DDL_ERR_INJECTED, "injected fault after admission");

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    float2* rope = reinterpret_cast<float2*>(ws + W.rope);
    f16* h = reinterpret_cast<f16*>(ws + W.h);
    float* qkv = reinterpret_cast<float*>(ws + W.qkv);
    f16* q16 = reinterpret_cast<f16*>(ws + W.q16);
    f16* o16 = reinterpret_cast<f16*>(ws + W.o16);
    float* x1 = reinterpret_cast<float*>(ws + W.x1);
    f16* a16 = reinterpret_cast<f16*>(ws + W.a16);
    f16* k16 = reinterpret_cast<f16*>(ws + W.k16);
    f16* vt16 = reinterpret_cast<f16*>(ws + W.vt16);
    float* part = reinterpret_cast<float*>(ws + W.part);
    const int d = L0->d, hq = L0->hq, hkv = L0->hkv, hd = L0->hd, f = L0->f, nqkv = L0->nqkv;
    // K splits of the projections (gate/up never splits); a split GEMM's
    // partial sums are added by the kernel that consumes its output: the QKV
    // post-step, the FFN norm, the next layer's attention norm, and after
    // the run's last down projection a closing row kernel.
    const int sp_qkv = gemm_splits(batch, nqkv, d, EPI_F32);
    const int sp_wo = gemm_splits(batch, d, hq * hd, EPI_RESID);
    const int sp_down = gemm_splits(batch, d, f, EPI_RESID);
    int pending = 0;                  // partials of the last down projection
    const float* pending_gpost = nullptr;   // its layer's post-FFN gain: hidden_out holds the raw branch

    hipError_t e = hipSuccess;
    const ddl_layer* table_of = nullptr;   // layer whose RoPE description the table holds
    for (int l = 0; l < run && !e; ++l) {
        const ddl_layer* L = layers[l];
        if (L->rope_on && !(table_of && same_rope(L, table_of))) {
            e = launch_rope_table(rope, batch, start_pos, L->rot_dim, L->theta, L->freq, L->mscale, s);
            table_of = L;
            if (e) break;
        }
        // the first layer reads the caller's hidden (no partials: never written)
        float* x = l == 0 ? const_cast<float*>(hidden) : hidden_out;
        // attention branch: x1 = x + wo . attn(rope(qkv(rms_norm(x)))); a
        // sandwich-norm layer adds rms_norm(wo . attn) * g_post_attn instead.
        // This norm also finishes the previous layer: its down partials, and
        // with a post-FFN norm x = x1 + rms_norm(branch) * g_post_ffn.
        {
            ProbeScope p(ctx, DDL_K_RMSNORM, s);
            e = launch_rmsnorm_f16(x, L->g_attn, h, batch, d, L->eps, part, pending,
                                   pending_gpost ? x1 : nullptr, pending_gpost, s);
        }
        if (!e && start_pos > 0) {
            StagePrefixArgs sp{};
            sp.pk = prefix_k[l]; sp.pv = prefix_v[l];
            sp.S = start_pos; sp.hkv = hkv; sp.hd = hd;
            sp.k16 = k16; sp.vt16 = vt16; sp.tcap = W.tcap;
            e = launch_stage_prefix(sp, s);
        }
        if (!e) {
            GemmArgs g{};
            g.A = h; g.lda = d; g.W = L->wqkv; g.ldw = d;
            g.M = batch; g.N = nqkv; g.K = d;
            g.inv_scale = &L->hdr->inv_scale[MAT_QKV];
            g.C = qkv; g.ldc = nqkv; g.P = part;
            ProbeScope p(ctx, DDL_K_GEMM_QKV, s);
            e = launch_gemm(g, EPI_F32, sp_qkv, s);
        }
        if (!e) {
            QkvPostArgs q{};
            q.qkv = qkv; q.nqkv = nqkv; q.part = part; q.nparts = sp_qkv - 1;
            q.bias = L->bqkv; q.q_norm = L->q_norm; q.k_norm = L->k_norm;
            q.rope = L->rope_on ? rope : nullptr;
            q.rope_layout = L->rope_layout;
            q.rope_half = L->rot_dim / 2;
            q.B = batch; q.S = start_pos; q.hq = hq; q.hkv = hkv; q.hd = hd; q.gated = L->gated;
            q.eps = L->eps;
            q.q16 = q16; q.k_rows = k_rows[l]; q.v_rows = v_rows[l];
            q.k16 = k16; q.vt16 = vt16; q.tcap = W.tcap;
            ProbeScope p(ctx, DDL_K_QKV_POST, s);
            e = launch_qkv_post(q, s);
        }
        if (!e) {
            AttnPrefillArgs a{};
            a.q16 = q16; a.k16 = k16; a.vt16 = vt16; a.tcap = W.tcap;
            a.gate = L->gated ? qkv + (size_t)(hq + 2 * hkv) * hd : nullptr;
            a.gate_ld = nqkv;
            a.o16 = o16;
            a.B = batch; a.S = start_pos; a.hq = hq; a.hkv = hkv; a.hd = hd;
            a.softcap = L->softcap;
            a.window = L->window;
            a.form = ctx->attn_form;
            ProbeScope p(ctx, DDL_K_ATTN_PREFILL, s);
            e = launch_attn_prefill(a, s);
        }
        if (!e) {
            GemmArgs g{};
            g.A = o16; g.lda = hq * hd; g.W = L->wo; g.ldw = hq * hd;
            g.M = batch; g.N = d; g.K = hq * hd;
            g.inv_scale = &L->hdr->inv_scale[MAT_O];
            g.C = x1; g.ldc = d; g.R = L->g_post_attn ? nullptr : x; g.ldr = d; g.P = part;
            ProbeScope p(ctx, DDL_K_GEMM_WO, s);
            e = launch_gemm(g, EPI_RESID, sp_wo, s);
        }
        // FFN branch: out = x1 + down(silu(gate(h2)) * up(h2)), h2 = rms_norm(x1)
        if (!e) {
            ProbeScope p(ctx, DDL_K_RMSNORM, s);
            e = launch_rmsnorm_f16(x1, L->g_ffn, h, batch, d, L->eps, part, sp_wo - 1,
                                   L->g_post_attn ? x : nullptr, L->g_post_attn, s);
        }
        if (!e) {
            GemmArgs g{};
            g.A = h; g.lda = d; g.W = L->wgu; g.ldw = d;
            g.M = batch; g.N = 2 * f; g.K = d;
            g.inv_scale = &L->hdr->inv_scale[MAT_GU];
            g.H = a16; g.ldh = f;
            ProbeScope p(ctx, DDL_K_GEMM_GATE_UP, s);
            e = launch_gemm(g, L->act == DDL_ACT_GELU ? EPI_GEGLU : EPI_SWIGLU, 1, s);
        }
        if (!e) {
            GemmArgs g{};
            g.A = a16; g.lda = f; g.W = L->wd; g.ldw = f;
            g.M = batch; g.N = d; g.K = f;
            g.inv_scale = &L->hdr->inv_scale[MAT_D];
            g.C = hidden_out; g.ldc = d; g.R = L->g_post_ffn ? nullptr : x1; g.ldr = d; g.P = part;
            ProbeScope p(ctx, DDL_K_GEMM_DOWN, s);
            e = launch_gemm(g, EPI_RESID, sp_down, s);
            pending = sp_down - 1;
            pending_gpost = L->g_post_ffn;
        }
    }
    if (!e && (pending > 0 || pending_gpost)) {
        // the last down projection's partials, and a post-FFN norm's residual
        ProbeScope p(ctx, DDL_K_RMSNORM, s);
        e = launch_rmsnorm_f16(hidden_out, nullptr, nullptr, batch, d, layers[run - 1]->eps, part,
                               pending, x1, pending_gpost, s);
    }
    if (e) return fail(DDL_ERR_DEVICE, std::string("prefill launch: ") + hipGetErrorString(e));
    g_err.clear();
    return run;
}

// ---- mirror ------------------------------------------------------------------

size_t ddl_mirror_bytes(int n_kv_heads, int head_dim, int capacity) {
    if (n_kv_heads <= 0 || head_dim <= 0 || capacity <= 0) return 0;
    return 2 * align256((size_t)capacity * n_kv_heads * head_dim * 4);
}

int ddl_mirror_init(ddl_mirror** out, void* dev_buf, size_t buf_bytes, int n_kv_heads,
                    int head_dim, int capacity) {
    if (!out || !dev_buf) return fail(DDL_ERR_INVALID, "null mirror handle or buffer");
    const size_t need = ddl_mirror_bytes(n_kv_heads, head_dim, capacity);
    if (need == 0 || buf_bytes < need) return fail(DDL_ERR_INVALID, "mirror buffer too small");
    ddl_mirror* m = new (std::nothrow) ddl_mirror;
    if (!m) return fail(DDL_ERR_INVALID, "out of host memory");
    m->k = static_cast<float*>(dev_buf);
    m->v = reinterpret_cast<float*>(static_cast<char*>(dev_buf) + need / 2);
    m->hkv = n_kv_heads;
    m->hd = head_dim;
    m->cap = capacity;
    m->seq_len = 0;
    *out = m;
    return 1;
}

int ddl_mirror_upload(ddl_mirror* m, const float* k, const float* v, int rows, void* stream) {
    if (!m) return fail(DDL_ERR_INVALID, "null mirror");
    if (rows < 0 || rows > m->cap || (rows > 0 && (!k || !v))) {
        m->seq_len = -1;
        return fail(DDL_ERR_INVALID, "upload rows exceed the mirror capacity or null source");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t bytes = (size_t)rows * m->hkv * m->hd * 4;
    hipError_t e = hipSuccess;
    if (bytes) {
        e = hipMemcpyAsync(m->k, k, bytes, hipMemcpyDefault, s);
        if (!e) e = hipMemcpyAsync(m->v, v, bytes, hipMemcpyDefault, s);
    }
    if (e) {
        m->seq_len = -1;
        return fail(DDL_ERR_DEVICE, std::string("mirror upload: ") + hipGetErrorString(e));
    }
    m->seq_len = rows;
    return 1;
}

int ddl_mirror_seq_len(const ddl_mirror* m) { return m ? m->seq_len : -1; }
int ddl_mirror_capacity(const ddl_mirror* m) { return m ? m->cap : 0; }
void ddl_mirror_invalidate(ddl_mirror* m) {
    if (m) m->seq_len = -1;
}
void ddl_mirror_destroy(ddl_mirror* m) { delete m; }

int ddl_mirror_plan_capacity(int rows, int planned) {
    if (rows < 0) return fail(DDL_ERR_INVALID, "negative rows");
    const long want = (long)rows + 1;
    if (planned > 0 && planned >= want) return planned;
    long cap = 1;
    while (cap < want) cap <<= 1;
    if (cap < 512) cap = 512;
    if (cap > 0x40000000L) return fail(DDL_ERR_INVALID, "capacity overflow");
    return (int)cap;
}

// ---- decode attention layer ----------------------------------------------------

namespace {
struct AttnWs {
    size_t pm, pl, po, o, x1, a, qkv, q, rdev, total;
};
// Partials are sized for the largest split count, so one workspace serves
// every row count.
AttnWs attn_ws(const ddl_layer* L) {
    const int splits = DECODE_MAX_SPLITS;
    AttnWs w;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    w.pm = take((size_t)L->hq * splits * 4);
    w.pl = take((size_t)L->hq * splits * 4);
    w.po = take((size_t)L->hq * splits * L->hd * 4);
    w.o = take((size_t)L->hq * L->hd * 4);
    w.x1 = take((size_t)L->d * 4);
    w.a = take((size_t)L->f * 4);
    w.qkv = take((size_t)L->nqkv * 4);      // ddl_decode_layer's head
    w.q = take((size_t)L->hq * L->hd * 4);
    w.rdev = take(sizeof(int));             // a decode graph's device row count
    w.total = o;
    return w;
}

// The refusals of the single-token path, before any device work
// ("frink-models 0.38.0 src/decoder/device_attention.rs": the mirror is
// trusted only while it holds exactly the cache's rows and needs room for
// one more; device_attention_shape_ok: no sliding window).  True when the
// call is declined (the reason is in the last error).
bool decode_rows_refused(const ddl_mirror* m, int host_rows) {
    if (m->seq_len != host_rows) {
        fail(DDL_DECLINED, "mirror is stale (seq_len differs from the cache's rows)");
        return true;
    }
    if (host_rows < 0 || m->cap < host_rows + 1) {
        fail(DDL_DECLINED, "mirror capacity below rows + 1");
        return true;
    }
    return false;
}

// The shape half of the refusals (the same for every row count).
bool decode_shape_refused(const ddl_mirror* m, int n_heads, const ddl_layer* L) {
    auto no = [](const char* why) {
        fail(DDL_DECLINED, why);
        return true;
    };
    if (n_heads != L->hq || m->hkv != L->hkv || m->hd != L->hd)
        return no("head shape differs between call, layer and mirror");
    if (!decode_group_ok(L->hq, L->hkv, L->hd))
        return no("query-head group size not served");
    if (!gemv_shape_ok(L->d) || !gemv_shape_ok(L->f) || !gemv_shape_ok(L->hq * L->hd))
        return no("GEMV width not served");
    if (L->window != 0) return no("sliding-window layer");
    // the decode tail's GEMVs add the residual in their epilogue: a layer
    // with sandwich norms takes the host path
    if (L->g_post_attn || L->g_post_ffn) return no("post-attention/post-FFN norm");
    return false;
}

bool decode_refused(const ddl_mirror* m, int host_rows, int n_heads, const ddl_layer* L) {
    return decode_rows_refused(m, host_rows) || decode_shape_refused(m, n_heads, L);
}

// Attention against the mirror (appending row host_rows) and the tail:
// x1 = x + wo . o; out = x1 + down(act(gate(h2)) * up(h2)), h2 = rms_norm(x1).
// With rdev the row count is read from device memory (a captured step) and
// the split plan is the one for the mirror's full capacity.
hipError_t attn_and_tail(ddl_ctx* ctx, ddl_mirror* m, int host_rows, const float* q,
                         const float* k, const float* v, const float* gate, float softcap,
                         const ddl_layer* L, const float* residual, float* out, char* ws,
                         const AttnWs& W, hipStream_t s, int* rdev = nullptr) {
    float* o = reinterpret_cast<float*>(ws + W.o);
    float* x1 = reinterpret_cast<float*>(ws + W.x1);
    float* a = reinterpret_cast<float*>(ws + W.a);
    DecodeAttnArgs d{};
    d.q = q; d.knew = k; d.vnew = v; d.mk = m->k; d.mv = m->v; d.gate = gate;
    d.part_m = reinterpret_cast<float*>(ws + W.pm);
    d.part_l = reinterpret_cast<float*>(ws + W.pl);
    d.part_o = reinterpret_cast<float*>(ws + W.po);
    d.o = o;
    d.R = host_rows; d.hq = L->hq; d.hkv = L->hkv; d.hd = L->hd;
    d.R_dev = rdev;
    decode_split_plan(L->hq, L->hkv, L->hd, rdev ? m->cap : host_rows + 1, &d.n_splits,
                      &d.rows_per_split);
    d.softcap = softcap;
    hipError_t e;
    {
        ProbeScope p(ctx, DDL_K_DECODE_ATTN, s);
        e = launch_decode_attn(d, s);
    }
    if (!e) {   // x1 = x + wo . o
        GemvArgs g{};
        g.W = L->wo; g.K = L->hq * L->hd; g.N = L->d;
        g.inv_scale = &L->hdr->inv_scale[MAT_O];
        g.x = o; g.r = residual; g.y = x1;
        ProbeScope p(ctx, DDL_K_GEMV_WO, s);
        e = launch_gemv(g, GV_RESID, s);
    }
    if (!e) {   // a = act(gate(h2)) * up(h2), h2 = rms_norm(x1) * g_ffn
        GemvArgs g{};
        g.W = L->wgu; g.K = L->d; g.N = L->f;
        g.inv_scale = &L->hdr->inv_scale[MAT_GU];
        g.x = x1; g.norm_g = L->g_ffn; g.eps = L->eps; g.y = a;
        g.gelu = L->act == DDL_ACT_GELU;
        ProbeScope p(ctx, DDL_K_GEMV_GATE_UP, s);
        e = launch_gemv(g, GV_SWIGLU, s);
    }
    if (!e) {   // out = x1 + down . a
        GemvArgs g{};
        g.W = L->wd; g.K = L->f; g.N = L->d;
        g.inv_scale = &L->hdr->inv_scale[MAT_D];
        g.x = a; g.r = x1; g.y = out;
        ProbeScope p(ctx, DDL_K_GEMV_DOWN, s);
        e = launch_gemv(g, GV_RESID, s);
    }
    return e;
}
}  // namespace

size_t ddl_attn_workspace_bytes(const ddl_layer* layer, int capacity) {
    if (!layer || capacity <= 0) return 0;
    return attn_ws(layer).total;
}

int ddl_attn_layer(ddl_ctx* ctx, ddl_mirror* m, int host_rows, const float* q, const float* k,
                   const float* v, const float* gate, int n_heads, float softcap,
                   const ddl_layer* L, const float* residual, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (!ctx || !m || !q || !k || !v || !L || !residual || !out)
        return fail(DDL_ERR_INVALID, "null argument");
    if (decode_refused(m, host_rows, n_heads, L)) return DDL_DECLINED;
    if (!(softcap >= 0.0f)) return fail(DDL_ERR_INVALID, "negative softcap");
    const AttnWs W = attn_ws(L);
    if (!workspace || workspace_bytes < W.total)
        return fail(DDL_ERR_WORKSPACE, "workspace smaller than ddl_attn_workspace_bytes");
    if (ctx->fault_after_admission) {
        m->seq_len = -1;
        return fail(DDL_ERR_INJECTED, "injected fault after admission");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = attn_and_tail(ctx, m, host_rows, q, k, v, gate, softcap, L, residual, out,
                                       static_cast<char*>(workspace), W, s);
    if (e) {
        m->seq_len = -1;
        return fail(DDL_ERR_DEVICE, std::string("attn_layer launch: ") + hipGetErrorString(e));
    }
    m->seq_len = host_rows + 1;
    g_err.clear();
    return 1;
}

}  // extern "C"

// ---- ddl_attn_layer without a caller workspace -----------------------------------
// For callers that cannot allocate device memory.  The decode scratch (split
// partials, attention output, x1, FFN activations) lives in this file-scope
// device array instead of a caller workspace; every call on a GPU shares that
// GPU's copy.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in symbol): its device address is looked up once
// per device, with that device current, and kept below.
namespace {
__device__ __align__(256) char scratch[DDL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, or nullptr (message set).
char* scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(DDL_ERR_DEVICE, "no current HIP device for the decode scratch");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(DDL_ERR_DEVICE, std::string("decode scratch address: ") + hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int ddl_attn_layer_noalloc(ddl_ctx* ctx, ddl_mirror* m, int host_rows, const float* q,
                           const float* k, const float* v, const float* gate, int n_heads,
                           float softcap, const ddl_layer* L, const float* residual, float* out,
                           void* stream) {
    if (!ctx || !m || !q || !k || !v || !L || !residual || !out)
        return fail(DDL_ERR_INVALID, "null argument");
    if (decode_refused(m, host_rows, n_heads, L)) return DDL_DECLINED;
    if (!(softcap >= 0.0f)) return fail(DDL_ERR_INVALID, "negative softcap");
    const AttnWs W = attn_ws(L);
    if (W.total > DDL_NOALLOC_SCRATCH_BYTES)
        return fail(DDL_ERR_WORKSPACE,
                    "layer needs " + std::to_string(W.total) +
                        " bytes of decode scratch, above the fixed DDL_NOALLOC_SCRATCH_BYTES (" +
                        std::to_string((size_t)DDL_NOALLOC_SCRATCH_BYTES) +
                        "); use ddl_attn_layer with a workspace");
    char* ws = scratch_of_current_device();
    if (!ws) return DDL_ERR_DEVICE;
    if (ctx->fault_after_admission) {
        m->seq_len = -1;
        return fail(DDL_ERR_INJECTED, "injected fault after admission");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = attn_and_tail(ctx, m, host_rows, q, k, v, gate, softcap, L, residual, out,
                                       ws, W, s);
    if (e) {
        m->seq_len = -1;
        return fail(DDL_ERR_DEVICE, std::string("attn_layer_noalloc launch: ") + hipGetErrorString(e));
    }
    m->seq_len = host_rows + 1;
    g_err.clear();
    return 1;
}

}  // extern "C"

namespace {
// One whole decode step (head, attention, tail) on s; with rdev the row
// count and the position are read from device memory.
hipError_t decode_step(ddl_ctx* ctx, ddl_mirror* m, int host_rows, const float* hidden,
                       const ddl_layer* L, float* out, float* k_row, float* v_row, char* ws,
                       const AttnWs& W, hipStream_t s, int* rdev) {
    float* qkv = reinterpret_cast<float*>(ws + W.qkv);
    float* q = reinterpret_cast<float*>(ws + W.q);
    hipError_t e;
    {   // qkv = [Wq; Wk; Wv(; Wgate)] . (rms_norm(x) * g_attn)
        GemvArgs g{};
        g.W = L->wqkv; g.K = L->d; g.N = L->nqkv;
        g.inv_scale = &L->hdr->inv_scale[MAT_QKV];
        g.x = hidden; g.norm_g = L->g_attn; g.eps = L->eps; g.r = nullptr; g.y = qkv;
        ProbeScope p(ctx, DDL_K_GEMV_QKV, s);
        e = launch_gemv(g, GV_RESID, s);
    }
    if (!e) {
        DecodeHeadArgs h{};
        h.qkv = qkv; h.bias = L->bqkv; h.q_norm = L->q_norm; h.k_norm = L->k_norm; h.eps = L->eps;
        h.rope_on = L->rope_on; h.rope_layout = L->rope_layout; h.rot_dim = L->rot_dim;
        h.theta = L->theta; h.freq = L->freq; h.mscale = L->mscale;
        h.pos = host_rows; h.pos_dev = rdev; h.hq = L->hq; h.hkv = L->hkv; h.hd = L->hd;
        h.q = q; h.k_row = k_row; h.v_row = v_row;
        ProbeScope p(ctx, DDL_K_DECODE_HEAD, s);
        e = launch_decode_head(h, s);
    }
    if (!e) {
        const float* gate = L->gated ? qkv + (size_t)(L->hq + 2 * L->hkv) * L->hd : nullptr;
        e = attn_and_tail(ctx, m, host_rows, q, k_row, v_row, gate, L->softcap, L, hidden, out, ws,
                          W, s, rdev);
    }
    return e;
}
}  // namespace

extern "C" {

int ddl_decode_layer(ddl_ctx* ctx, ddl_mirror* m, int host_rows, const float* hidden,
                     const ddl_layer* L, float* out, float* k_row, float* v_row,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (!ctx || !m || !hidden || !L || !out || !k_row || !v_row)
        return fail(DDL_ERR_INVALID, "null argument");
    if (decode_refused(m, host_rows, L->hq, L)) return DDL_DECLINED;
    if (!gemv_shape_ok(L->d) || L->nqkv % 32) return fail(DDL_DECLINED, "GEMV width not served");
    const AttnWs W = attn_ws(L);
    if (!workspace || workspace_bytes < W.total)
        return fail(DDL_ERR_WORKSPACE, "workspace smaller than ddl_attn_workspace_bytes");
    if (ctx->fault_after_admission) {
        m->seq_len = -1;
        return fail(DDL_ERR_INJECTED, "injected fault after admission");
    }
    const hipError_t e = decode_step(ctx, m, host_rows, hidden, L, out, k_row, v_row,
                                     static_cast<char*>(workspace), W,
                                     static_cast<hipStream_t>(stream), nullptr);
    if (e) {
        m->seq_len = -1;
        return fail(DDL_ERR_DEVICE, std::string("decode_layer launch: ") + hipGetErrorString(e));
    }
    m->seq_len = host_rows + 1;
    g_err.clear();
    return 1;
}

}  // extern "C"

// ---- a decode step captured once and replayed per token -----------------------
struct ddl_decode_graph {
    ddl_mirror* m;
    const ddl_layer* L;
    hipStream_t capture;     // the stream the step was captured on
    hipGraph_t graph;
    hipGraphExec_t exec;
    int* rdev;               // device row count, in the caller's workspace
    int shadow;              // the count rdev holds once enqueued work is done; -1 unknown
};

namespace {
void graph_release(ddl_decode_graph* g) {
    if (g->exec) hipGraphExecDestroy(g->exec);
    if (g->graph) hipGraphDestroy(g->graph);
    if (g->capture) hipStreamDestroy(g->capture);
    delete g;
}
}  // namespace

extern "C" {

int ddl_decode_graph_create(ddl_ctx* ctx, ddl_mirror* m, const ddl_layer* L,
                            const float* hidden, float* out, float* k_row, float* v_row,
                            void* workspace, size_t workspace_bytes, ddl_decode_graph** out_graph) {
    if (!ctx || !m || !L || !hidden || !out || !k_row || !v_row || !out_graph)
        return fail(DDL_ERR_INVALID, "null argument");
    if (decode_shape_refused(m, L->hq, L)) return DDL_DECLINED;
    if (!gemv_shape_ok(L->d) || L->nqkv % 32) return fail(DDL_DECLINED, "GEMV width not served");
    const AttnWs W = attn_ws(L);
    if (!workspace || workspace_bytes < W.total)
        return fail(DDL_ERR_WORKSPACE, "workspace smaller than ddl_attn_workspace_bytes");
    ddl_decode_graph* g = new (std::nothrow) ddl_decode_graph{};
    if (!g) return fail(DDL_ERR_INVALID, "out of host memory");
    g->m = m;
    g->L = L;
    char* ws = static_cast<char*>(workspace);
    g->rdev = reinterpret_cast<int*>(ws + W.rdev);
    g->shadow = -1;
    // capture on a stream of the library's own (the caller's may be the
    // null stream, which cannot be captured), with the launch probes off
    hipError_t e = hipStreamCreateWithFlags(&g->capture, hipStreamNonBlocking);
    if (!e) e = hipStreamBeginCapture(g->capture, hipStreamCaptureModeRelaxed);
    if (!e) {
        const int kind = ctx->probe_kind;
        ctx->probe_kind = -1;
        const hipError_t le = decode_step(ctx, m, 0, hidden, L, out, k_row, v_row, ws, W,
                                          g->capture, g->rdev);
        ctx->probe_kind = kind;
        e = hipStreamEndCapture(g->capture, &g->graph);
        if (!e) e = le;
    }
    if (!e) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    if (e) {
        graph_release(g);
        return fail(DDL_ERR_DEVICE, std::string("decode graph capture: ") + hipGetErrorString(e));
    }
    *out_graph = g;
    g_err.clear();
    return 1;
}

int ddl_decode_graph_launch(ddl_ctx* ctx, ddl_decode_graph* g, int host_rows, void* stream) {
    if (!ctx || !g) return fail(DDL_ERR_INVALID, "null argument");
    ddl_mirror* m = g->m;
    if (decode_rows_refused(m, host_rows)) return DDL_DECLINED;
    if (ctx->fault_after_admission) {
        m->seq_len = -1;
        return fail(DDL_ERR_INJECTED, "injected fault after admission");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // the device count follows the graph's own replays; anything else that
    // moved the mirror (an upload, an eager step) is caught up first
    if (g->shadow != host_rows) e = launch_set_int(g->rdev, host_rows, s);
    if (!e) e = hipGraphLaunch(g->exec, s);
    if (e) {
        m->seq_len = -1;
        g->shadow = -1;
        return fail(DDL_ERR_DEVICE, std::string("decode graph launch: ") + hipGetErrorString(e));
    }
    g->shadow = host_rows + 1;
    m->seq_len = host_rows + 1;
    g_err.clear();
    return 1;
}

void ddl_decode_graph_destroy(ddl_decode_graph* g) {
    if (g) graph_release(g);
}

}  // extern "C"
