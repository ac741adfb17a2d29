/*
 * ddl.h -- resident dense decoder-layer stack for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Two operations:
 *
 *   ddl_prefill_dense_stack  batched prefill of a run of consecutive dense
 *                            Llama-style layers, kept on the device between
 *                            layers, returning the new hidden rows and each
 *                            layer's K/V rows.
 *   ddl_attn_layer           one token's attention layer (attention, gate,
 *                            wo, residual, FFN norm, SwiGLU FFN, residual)
 *                            against a device mirror of the host KV cache.
 *
 * Sources (the pages describe the host side of these operations):
 *   [P1] "frink-models 0.29.0 src/decoder/cuda_prefill.rs" -- module doc,
 *        try_cuda_prefill_dense_stack, cuda_prefill_layer.
 *   [P2] "frink-models 0.38.0 src/decoder/device_attention.rs" -- module doc
 *        ("Why this is the last one", "The mirror, and why it cannot go
 *        stale"), device_attention_layer, device_attention_shape_ok,
 *        ensure_attn_mirror.
 *   [P3] "frink-models 0.49.0 src/fused_layer.rs" -- module doc ("What it
 *        refuses, and why the list is written out"), LayerFfnParts::for_layer.
 *
 * Conventions (all calls):
 *   - Device pointers unless a parameter says "host".  The library never
 *     allocates device memory: weights blobs, workspaces, mirrors and
 *     outputs are caller-owned buffers (PyTorch tensors in the Python
 *     binding).  Host-side handles (ddl_ctx, ddl_layer, ddl_mirror) are
 *     allocated by the library and released by the matching destroy call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     every device operation of a call is enqueued on it, asynchronously.
 *   - Matrices are row-major [out][in] (y = W x); activations are
 *     token-major; a K/V row is [n_kv_heads][head_dim] fp32.
 *   - Return codes: > 0 served (the meaning is per call), 0 = DECLINED (no
 *     device work was enqueued, every output and cache untouched; [P1]
 *     try_cuda_prefill_dense_stack answers None before touching the device),
 *     < 0 = error after admission (see ddl_last_error(); [P1] a launch that
 *     fails after admission is reported once and the caller's caches stay
 *     untouched because the caller pushes rows only on success).
 *   - Thread-compatible per ddl_ctx: distinct contexts may be used from
 *     distinct threads; one context must not be used by two threads at once.
 */
#ifndef DDL_H
#define DDL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDL_DECLINED 0
#define DDL_ERR_INVALID (-1)   /* bad argument (null pointer, size, shape) */
#define DDL_ERR_DEVICE (-2)    /* a HIP call or kernel launch failed */
#define DDL_ERR_INJECTED (-3)  /* the test hook fault_after_admission fired */
#define DDL_ERR_WORKSPACE (-4) /* workspace smaller than the call needs */

enum { DDL_ACT_SWIGLU = 0, DDL_ACT_GELU = 1 };
enum { DDL_ROPE_NEOX = 0, DDL_ROPE_NORM = 1 };
enum { DDL_DTYPE_F32 = 0, DDL_DTYPE_BF16 = 1 };

typedef struct ddl_ctx ddl_ctx;
typedef struct ddl_layer ddl_layer;
typedef struct ddl_mirror ddl_mirror;

/* Context options.  min_batch: smallest batch the prefill serves ([P1]
 * try_cuda_prefill_dense_stack declines batches under four; default 4).
 * fault_after_admission: test hook -- a call that passes admission returns
 * DDL_ERR_INJECTED before enqueueing any device work.
 * attn_form: which prefill attention kernel form runs (a measurement and
 * test aid; results agree to rounding): DDL_ATTN_AUTO (0, the default: one
 * head per workgroup on small grids, a GQA group's heads sharing each K/V
 * tile on large ones), DDL_ATTN_ONE_HEAD, DDL_ATTN_SHARED (falls back to
 * one head when a KV head has a single query head). */
enum { DDL_ATTN_AUTO = 0, DDL_ATTN_ONE_HEAD = 1, DDL_ATTN_SHARED = 2 };
typedef struct {
    int min_batch;
    int fault_after_admission;
    int attn_form;
} ddl_ctx_opts;

/* Create / destroy a context.  opts may be NULL (defaults).  Creating a
 * context touches no device.  Returns NULL only when out of host memory. */
ddl_ctx* ddl_ctx_create(const ddl_ctx_opts* opts);
void ddl_ctx_destroy(ddl_ctx* ctx);

/* One layer's description ([P1] cuda_prefill_layer: the layer descriptor
 * and the attention parameters; [P2] device_attention_shape_ok).  Every
 * field must be answered: a layer with anything the kernels do not
 * implement is declined, never silently dropped ([P3] "What it refuses").
 *   served: act DDL_ACT_SWIGLU or DDL_ACT_GELU (gated GELU, exact erf form;
 *   [P1] try_cuda_prefill_dense_stack names it); post_norm_eps == rms_eps;
 *   v_head_dim == head_dim; window >= 0 (0 = none; W > 0: the token at
 *   position p sees keys p-W+1 .. p); post-attention / post-FFN (sandwich)
 *   norms; no sinks, ALiBi or LoRA; rope disabled, or Neox / Norm layout
 *   with rot_dim (0 = head_dim) even and at most head_dim -- for Neox a
 *   multiple of 64 -- any positive frequency factors ([rot_dim/2], host,
 *   copied at pack time) and any finite attention factor mscale (on the
 *   rotated channels); head_dim in {64, 128}; n_heads a multiple of
 *   n_kv_heads; d_model a multiple of 128 and at most 4096; d_ff a multiple
 *   of 64; the stacked q/k/v(/gate) width a multiple of 128; softcap >= 0.
 *   ddl_attn_layer and ddl_decode_layer further need n_heads / n_kv_heads
 *   in {1, 2, 3, 4, 8}, no window and no sandwich norms
 *   and d_model, d_ff, n_heads*head_dim at most 15872 (declined otherwise). */
typedef struct {
    int d_model, n_heads, n_kv_heads, head_dim, v_head_dim, d_ff;
    float rms_eps, post_norm_eps;
    int act;                      /* DDL_ACT_* */
    int rope_enabled;             /* 0: the layer does not rotate */
    double rope_theta;
    int rope_layout;              /* DDL_ROPE_* */
    int rope_rot_dim;             /* 0 means head_dim */
    float rope_mscale;            /* attention factor on rotated channels */
    const float* rope_freq_factors; /* host, [rot_dim/2] or NULL */
    float attn_softcap;           /* 0: none; else s <- c*tanh(s/c) */
    int gated;                    /* wq is [q ; gate], o *= sigmoid(gate) */
    int has_qkv_bias, has_qk_norm;
    int window;                   /* sliding window; 0 = none */
    int has_post_attn_norm, has_post_ffn_norm, has_sinks, has_alibi, has_lora;
} ddl_layer_desc;

/* A layer's weights as the caller holds them (device pointers).  Matrices
 * of element type `dtype` (DDL_DTYPE_F32 or DDL_DTYPE_BF16 bit patterns):
 *   wq [(gated ? 2 : 1) * n_heads*head_dim][d_model]   rows [q ; gate]
 *   wk, wv [n_kv_heads*head_dim][d_model]
 *   wo [d_model][n_heads*head_dim]
 *   wg, wu [d_ff][d_model];  wd [d_model][d_ff]
 * fp32 vectors: g_attn, g_ffn [d_model]; bq [n_heads*head_dim], bk, bv
 * [n_kv_heads*head_dim] (when has_qkv_bias); q_norm, k_norm [head_dim]
 * (when has_qk_norm); g_post_attn, g_post_ffn [d_model] (when
 * has_post_attn_norm / has_post_ffn_norm: the sandwich norms' gains). */
typedef struct {
    int dtype;
    const void *wq, *wk, *wv, *wo, *wg, *wu, *wd;
    const float *g_attn, *g_ffn;
    const float *bq, *bk, *bv;
    const float *q_norm, *k_norm;
    const float *g_post_attn, *g_post_ffn;
} ddl_layer_weights;

/* 1 if the layer is one the kernels serve, 0 if not (pure host predicate;
 * the reason is in ddl_last_error()).  [P1] cuda_prefill_layer answers
 * None for a layer the launch does not serve, and [P3] LayerFfnParts::
 * for_layer names every field so none is dropped unanswered: the same
 * question, asked before any device memory is committed. */
int ddl_layer_supported(const ddl_layer_desc* desc);

/* Device bytes of one layer's packed weights (0 if not supported): the
 * device-resident form of the norm gains, extras and seven projections that
 * [P1] cuda_prefill_layer borrows through each matrix's device view
 * (`view(...)`, None when a matrix has none).  The caller allocates them. */
size_t ddl_layer_blob_bytes(const ddl_layer_desc* desc);

/* [P1] cuda_prefill_layer: the launch borrows each projection through a
 * device view of its storage and the norm gains and extras as they are.
 * Packs a layer's weights into the caller-owned device blob `dev_blob`
 * (blob_bytes >= ddl_layer_blob_bytes(desc)), on `stream`: matrices are
 * stored as fp16 holding the given values times a per-matrix power of two,
 * q/k/v stacked into one matrix and gate/up interleaved in 16-row blocks.
 * The source buffers may be freed once the stream has passed the call.
 * *out receives a host handle that borrows `dev_blob` (which must outlive
 * it).  Returns 1, 0 (declined: layer not supported, *out untouched) or < 0. */
int ddl_layer_pack(ddl_ctx* ctx, const ddl_layer_desc* desc,
                   const ddl_layer_weights* w, void* dev_blob, size_t blob_bytes,
                   void* stream, ddl_layer** out);
void ddl_layer_destroy(ddl_layer* layer);

/* [P1] module doc: the hidden batch stays on the device between layers and
 * every step between the seven matmuls of a layer is a kernel, so the
 * intermediates live in device memory for the length of the call only.
 * Workspace bytes a prefill of up to max_batch tokens at a start position of
 * up to max_start_pos needs over `n` layers (0 on bad arguments).  The
 * workspace holds the per-layer intermediates (normed rows, q/k/v, attention
 * output, SwiGLU activations) and the layer's keys and values staged as
 * fp16; its contents do not outlive a call. */
size_t ddl_workspace_bytes(const ddl_layer* const* layers, int n, int max_batch,
                           int max_start_pos);

/* Batched prefill of the longest servable run of consecutive layers
 * ([P1] module doc and try_cuda_prefill_dense_stack).
 *   hidden      [batch][d_model] fp32 in (device)
 *   layers      host array of n_layers packed layers
 *   start_pos   rows already in every layer's cache (positions of the new
 *               tokens are start_pos .. start_pos+batch-1)
 *   prefix_k/v  host arrays of n_layers device pointers, each
 *               [start_pos][n_kv_heads*head_dim] fp32: the cache rows, used
 *               as they are (already rotated); may be NULL when start_pos==0
 *   prefix_rows host array of n_layers row counts of those caches; a layer
 *               whose count is not start_pos ends the run ([P1]
 *               cuda_prefill_layer requires positions == rows == start_pos)
 *   hidden_out  [batch][d_model] fp32 out; may alias hidden
 *   k_rows/v_rows host arrays of n_layers device pointers, each
 *               [batch][n_kv_heads*head_dim] fp32 out: the rows the caller
 *               pushes into its cache, row b for token b (post bias, QK-norm
 *               and RoPE for K)
 *   workspace   device, workspace_bytes >= ddl_workspace_bytes(layers,
 *               n_layers, batch, start_pos) (else DDL_ERR_WORKSPACE)
 * Returns run_len > 0 (layers 0..run_len-1 ran; hidden_out is the output
 * of layer run_len-1 and k_rows/v_rows[0..run_len-1] are written), 0 when
 * declined (batch < min_batch, layer 0 not servable or its prefix count
 * differs), < 0 on error. */
int ddl_prefill_dense_stack(ddl_ctx* ctx, const float* hidden,
                            const ddl_layer* const* layers, int n_layers,
                            int batch, int start_pos,
                            const float* const* prefix_k,
                            const float* const* prefix_v,
                            const int* prefix_rows, float* hidden_out,
                            float* const* k_rows, float* const* v_rows,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* ---- the device KV mirror ([P2] "The mirror, and why it cannot go stale",
 * ensure_attn_mirror) ----------------------------------------------------
 * A caller-owned device buffer holding K rows then V rows,
 * [capacity][n_kv_heads*head_dim] fp32 each, plus a host handle with its
 * seq_len (rows it holds; -1 = stale).  The host cache stays authoritative:
 * the mirror is trusted only while seq_len equals the cache's row count,
 * and anything else is fixed by re-uploading the whole history. */
size_t ddl_mirror_bytes(int n_kv_heads, int head_dim, int capacity);
/* *out borrows dev_buf (buf_bytes >= ddl_mirror_bytes(...)); seq_len = 0. */
int ddl_mirror_init(ddl_mirror** out, void* dev_buf, size_t buf_bytes,
                    int n_kv_heads, int head_dim, int capacity);
/* Copies `rows` K and V rows (host or device memory, [rows][kv_width] fp32)
 * into the mirror on `stream` and sets seq_len = rows.  Returns 1, or < 0
 * (rows > capacity, bad pointer; seq_len then becomes -1). */
int ddl_mirror_upload(ddl_mirror* m, const float* k, const float* v, int rows,
                      void* stream);
int ddl_mirror_seq_len(const ddl_mirror* m);
int ddl_mirror_capacity(const ddl_mirror* m);
void ddl_mirror_invalidate(ddl_mirror* m);   /* seq_len = -1 */
/* The capacity a mirror for a cache of `rows` rows should have ([P2]
 * ensure_attn_mirror): the cache's planned capacity when it is at least
 * rows+1 (planned <= 0: none), else max(next_pow2(rows+1), 512). */
int ddl_mirror_plan_capacity(int rows, int planned);
void ddl_mirror_destroy(ddl_mirror* m);

/* Workspace bytes of ddl_attn_layer and ddl_decode_layer for a layer (the
 * same for every row count up to `capacity`). */
size_t ddl_attn_workspace_bytes(const ddl_layer* layer, int capacity);

/* One token's attention layer in one submission against the mirror
 * ([P2] device_attention_layer).
 *   host_rows  rows in the caller's host cache; DECLINED unless the mirror
 *              holds exactly that many (seq_len == host_rows) and has room
 *              for one more
 *   q          [n_heads*head_dim] fp32, rotated and QK-normed
 *   k, v       [n_kv_heads*head_dim] fp32, this token's rows (k rotated)
 *   gate       [n_heads*head_dim] fp32 or NULL; o *= sigmoid(gate)
 *   softcap    0 = none, else s <- c*tanh(s/c)
 *   layer      packed layer supplying wo, the FFN norm, gate/up/down and
 *              the head shape (n_heads must equal the layer's)
 *   residual   [d_model] fp32, the layer input x
 *   out        [d_model] fp32, x1 + ffn(rms_norm(x1)) with x1 = x + wo.o
 * Returns 1 (served: k/v appended at row host_rows, seq_len = host_rows+1;
 * the caller pushes k/v into its host cache so rows == seq_len again), 0
 * (declined, nothing enqueued, mirror unchanged) or < 0 (error; the mirror
 * is marked stale so the next use re-uploads). */
int ddl_attn_layer(ddl_ctx* ctx, ddl_mirror* mirror, int host_rows,
                   const float* q, const float* k, const float* v,
                   const float* gate, int n_heads, float softcap,
                   const ddl_layer* layer, const float* residual, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ddl_attn_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same refusals, kernels and results, with no workspace argument.  The
 * decode scratch is a fixed device array of DDL_NOALLOC_SCRATCH_BYTES
 * inside the library, one copy per GPU, held until the process ends; the
 * call allocates nothing (no hipMalloc, hipFree or allocating library call).
 * A layer whose scratch (ddl_attn_workspace_bytes) exceeds that size
 * returns DDL_ERR_WORKSPACE with nothing enqueued -- 32 query heads of 128
 * with hidden 4096 and FFN 14336 need about 4.3 MB.  Every call on one GPU
 * uses the same array: calls that overlap on one GPU (other streams, other
 * threads, other contexts) race and give undefined results; calls ordered
 * on one stream are fine.  Returns as ddl_attn_layer. */
#define DDL_NOALLOC_SCRATCH_BYTES (6u << 20)
int ddl_attn_layer_noalloc(ddl_ctx* ctx, ddl_mirror* mirror, int host_rows,
                           const float* q, const float* k, const float* v,
                           const float* gate, int n_heads, float softcap,
                           const ddl_layer* layer, const float* residual,
                           float* out, void* stream);

/* One token's whole decoder layer against the mirror, every step on the
 * device: the head ([P1] cuda_prefill_layer's attention norm, stacked
 * q/k/v(/gate) projection, extras and RoPE description) feeding the
 * attention and tail of ddl_attn_layer -- the "one submission a layer" of
 * [P3] (module doc, "Why") and [P2] device_attention_layer with q/k/v
 * computed on the device instead of handed in.
 *   host_rows  rows in the caller's host cache (the token's position);
 *              declined unless the mirror's seq_len equals it and its
 *              capacity is at least host_rows + 1
 *   hidden     [d_model] fp32 (device): the layer input (also the residual)
 *   out        [d_model] fp32 (device): the layer output; may alias hidden
 *   k_row, v_row [n_kv_heads*head_dim] fp32 (device) out: this token's K row
 *              (biased, QK-normed, rotated at position host_rows) and V row,
 *              the rows the caller pushes into its host cache
 *   workspace  >= ddl_attn_workspace_bytes(layer, capacity)
 * The layer's softcap, gate, RoPE, extras and FFN activation are the packed
 * layer's own.  Declines like ddl_attn_layer (and for the same layers).
 * Returns 1 (served: the mirror holds the new row, seq_len = host_rows+1),
 * 0 (declined, nothing touched) or < 0 (error: the mirror is marked
 * stale). */
int ddl_decode_layer(ddl_ctx* ctx, ddl_mirror* m, int host_rows,
                     const float* hidden, const ddl_layer* layer, float* out,
                     float* k_row, float* v_row, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ---- the decode step as one submission --------------------------------------
 * [P3] module doc ("Why"): the cost of a decode token is the number of
 * submissions, one per layer at best; [P2] device_attention_layer runs the
 * whole attention layer "in one submission".  ddl_decode_graph_create
 * captures one ddl_decode_layer step (its seven kernels) as a HIP graph,
 * bound to this mirror, layer and these buffers (their addresses are baked
 * in: hidden is read, out/k_row/v_row written, at every replay).  The row
 * count the step attends over lives in device memory (in the workspace) and
 * the attention's split plan is sized for the mirror's capacity, so one
 * graph serves every row count up to it.  Declines like ddl_decode_layer
 * for the shape; returns 1 and *graph, 0, or < 0.  Nothing is enqueued.
 *   hidden, out, k_row, v_row, workspace: as ddl_decode_layer's, device
 *   memory that must stay in place (and workspace unshared) while the graph
 *   exists. */
typedef struct ddl_decode_graph ddl_decode_graph;
int ddl_decode_graph_create(ddl_ctx* ctx, ddl_mirror* mirror, const ddl_layer* layer,
                            const float* hidden, float* out, float* k_row,
                            float* v_row, void* workspace, size_t workspace_bytes,
                            ddl_decode_graph** graph);
/* Replays the step for the token at position host_rows on `stream`: the same
 * results, appended row and mirror bookkeeping as ddl_decode_layer with the
 * graph's buffers.  Declines (nothing enqueued) unless the mirror's seq_len
 * equals host_rows and its capacity is at least host_rows + 1.  When the
 * mirror moved since the graph's last replay (an upload, an eager step) one
 * small kernel first sets the device row count.  Returns 1, 0 or < 0 (the
 * mirror is then marked stale). */
int ddl_decode_graph_launch(ddl_ctx* ctx, ddl_decode_graph* graph, int host_rows,
                            void* stream);
void ddl_decode_graph_destroy(ddl_decode_graph* graph);

/* ---- launch timing probe (a measurement aid) -------------------------------
 * Kernel classes of the two operations. */
enum {
    DDL_K_RMSNORM = 0,        /* attention and FFN RMS norms */
    DDL_K_GEMM_QKV = 1,       /* stacked q/k/v(/gate) projection */
    DDL_K_QKV_POST = 2,       /* bias, QK norm, RoPE, K/V rows */
    DDL_K_ATTN_PREFILL = 3,   /* causal GQA attention */
    DDL_K_GEMM_WO = 4,        /* wo projection + residual */
    DDL_K_GEMM_GATE_UP = 5,   /* gate/up projection + SwiGLU */
    DDL_K_GEMM_DOWN = 6,      /* down projection + residual */
    DDL_K_DECODE_ATTN = 7,    /* decode attention (split + combine) */
    DDL_K_GEMV_WO = 8,
    DDL_K_GEMV_GATE_UP = 9,
    DDL_K_GEMV_DOWN = 10,
    DDL_K_GEMV_QKV = 11,      /* decode head: RMS norm + stacked q/k/v(/gate) GEMV */
    DDL_K_DECODE_HEAD = 12,   /* decode head: bias, QK norm, RoPE */
    DDL_K_COUNT = 13
};
/* While enabled, each launch of class `kind` made through `ctx` is
 * bracketed by two HIP events recorded on the call's stream, for at most
 * max_launches launches (max_launches = 0 disables; events are created
 * here, on the current device).  Returns 1 or < 0. */
int ddl_probe_enable(ddl_ctx* ctx, int kind, int max_launches);
/* Waits for the recorded events, writes the duration (ms) of each bracketed
 * launch to ms_out (up to cap entries, host memory) and returns how many
 * launches were recorded since ddl_probe_enable (the count then restarts
 * from 0), or < 0 on error. */
int ddl_probe_read(ddl_ctx* ctx, float* ms_out, int cap);

/* The calling thread's last error or decline reason ("" if none).  [P1]
 * warn_once prints each distinct decline message once per process; here
 * the library only records the message and the caller de-duplicates. */
const char* ddl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DDL_H */
