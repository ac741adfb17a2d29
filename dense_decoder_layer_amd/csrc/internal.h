// Host-side structures of the library and the kernel launchers' signatures.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ddl.h"

typedef _Float16 f16;

#include <vector>

struct ddl_ctx {
    int min_batch;
    int fault_after_admission;
    int attn_form;                      // DDL_ATTN_*
    // launch timing probe
    int probe_kind = -1, probe_max = 0, probe_count = 0;
    std::vector<hipEvent_t> probe_events;   // 2 per launch: start, end
};

// Brackets one launch of class `kind` with probe events when enabled.
struct ProbeScope {
    ddl_ctx* c;
    hipStream_t s;
    int slot = -1;
    ProbeScope(ddl_ctx* ctx, int kind, hipStream_t stream) : c(ctx), s(stream) {
        if (c->probe_kind == kind && c->probe_count < c->probe_max) {
            slot = c->probe_count++;
            (void)hipEventRecord(c->probe_events[2 * slot], s);
        }
    }
    ~ProbeScope() {
        if (slot >= 0) (void)hipEventRecord(c->probe_events[2 * slot + 1], s);
    }
};

// Device header at the start of a packed layer blob.  absmax_bits are
// filled by the pack kernels (max |w| of each packed matrix, as the bits
// of a non-negative float so an integer max is exact); shift/inv_scale
// are derived from them: a matrix is stored as fp16(w * 2^shift) and the
// GEMM epilogue multiplies by inv_scale = 2^-shift.
enum { MAT_QKV = 0, MAT_O = 1, MAT_GU = 2, MAT_D = 3, MAT_COUNT = 4 };
struct BlobHeader {
    uint32_t absmax_bits[MAT_COUNT];
    int32_t shift[MAT_COUNT];
    float inv_scale[MAT_COUNT];
    uint32_t pad[52];
};
static_assert(sizeof(BlobHeader) == 256, "header is one 256-byte line");

// A packed layer: shapes plus device pointers into the caller's blob.
// Matrices (logical [rows][cols], y = W x):
//   wqkv [nqkv][d]   rows: q (hq*hd), k (hkv*hd), v (hkv*hd), gate (hq*hd, gated)
//   wo   [d][hq*hd]
//   wgu  [2*f][d]    gate/up interleaved in 16-row blocks: block 2j = gate
//                    rows 16j..16j+15, block 2j+1 = up rows 16j..16j+15
//   wd   [d][f]
// each stored in MFMA-fragment order: the 32 x 16 block (rows 32nb..,
// cols 16kb..) is 512 consecutive fp16 at ((nb * cols/16) + kb) * 512, and
// inside it element (32nb + r, 16kb + c) sits at (r + 32*(c/8)) * 8 + c%8 --
// lane r + 32*(c/8) of a v_mfma_f32_32x32x16_f16 B operand holds it.
struct ddl_layer {
    int d, hq, hkv, hd, f, nqkv;
    int gated, has_bias, has_qk_norm, rope_on;
    int act;                     // DDL_ACT_SWIGLU or DDL_ACT_GELU (gated GELU)
    int window;                  // sliding window (keys per query), 0 = none
    float eps, softcap;
    double theta;
    int rope_layout, rot_dim;    // DDL_ROPE_*, rotated channels per head
    float mscale;                // attention factor on the rotated channels
    std::vector<float> freq_host;   // frequency factors (empty: none), host copy
    float* freq;                 // the same in the blob, [rot_dim/2] or null
    size_t blob_bytes;
    BlobHeader* hdr;
    float *g_attn, *g_ffn, *bqkv, *q_norm, *k_norm;
    float *g_post_attn, *g_post_ffn;   // sandwich-norm gains, or null
    f16 *wqkv, *wo, *wgu, *wd;
};

struct ddl_mirror {
    float* k;   // [cap][hkv*hd]
    float* v;
    int hkv, hd, cap, seq_len;
};

// ---- launchers (each enqueues on `s`; return hipGetLastError()) ----------

enum { EPI_F32 = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_GEGLU = 3 };

struct GemmArgs {
    const f16* A; int lda;      // [M][K]
    const f16* W; int ldw;      // [N][K]
    int M, N, K;
    const float* inv_scale;     // device scalar, multiplies the accumulator
    float* C; int ldc;          // EPI_F32, EPI_RESID output
    const float* R; int ldr;    // EPI_RESID residual input (may alias C; null: C = acc)
    f16* H; int ldh;            // EPI_SWIGLU / EPI_GEGLU output [M][N/2]
    // Split-K (EPI_F32, EPI_RESID): slice 0 of the K range applies the
    // epilogue to C; slice z > 0 stores its raw scaled sum to
    // P + (z - 1) * M * ldc, [M][ldc], which the consumer adds in.
    float* P;
};
// W in MFMA-fragment order (see ddl_layer); N % 128 == 0, K % 64 == 0.
// splits: gemm_splits(...) slices; P must hold (splits - 1) * M * ldc floats.
hipError_t launch_gemm(const GemmArgs& a, int epi, int splits, hipStream_t s);
bool gemm_shape_ok(int M, int N, int K, int epi);
// The K split launch_gemm is to be called with for this shape (1 = none).
int gemm_splits(int M, int N, int K, int epi);

// h = fp16(rms_norm(x) * g), one row of d values per token.  With
// nparts > 0, x first gets the split-K partials part[z * rows * d + row * d +
// col] (z < nparts) added.  With gpost, that sum y becomes base + rms_norm(y)
// * gpost (a sandwich norm's residual add).  x is written back when either
// applies; h may be null (no second norm).
hipError_t launch_rmsnorm_f16(float* x, const float* g, f16* h, int rows, int d, float eps,
                              const float* part, int nparts, const float* base,
                              const float* gpost, hipStream_t s);

// tab[b][i] = m * (cos, sin) of (start_pos + b) * theta^(-2i/rot_dim) / freq[i]
// for the rot_dim/2 rotated pairs i (freq may be null: factors of 1).
hipError_t launch_rope_table(float2* tab, int batch, int start_pos, int rot_dim, double theta,
                             const float* freq, float mscale, hipStream_t s);

// Staged fp16 K/V of one layer for the attention kernel, tcap rows per KV
// head (a multiple of 32, at least S + 32*(ceil(B/32)+1)):
//   k16  [hkv][tcap][hd]   key j = cached row j (j < S) or new row j - S
//   vt16 [hkv][hd][tcap]   the same values transposed, key j at position
//                          vt_pos(j): within each aligned group of 16 keys,
//                          keys 8..11 and 4..7 trade places, so that the 8
//                          keys one lane of the attention's V^T operand needs
//                          (4g..4g+3 and 8+4g..8+4g+3, g = 0 or 1) are the
//                          16 contiguous bytes at position 8g
__host__ __device__ inline int vt_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }
struct QkvPostArgs {
    const float* part; int nparts;       // split-K partials of qkv, [nparts][B][nqkv]
    float* qkv; int nqkv;               // [B][nqkv] GEMM output (a gated layer's
                                        // gate columns get the partials added in place)
    const float* bias;                  // [nqkv] or null
    const float* q_norm; const float* k_norm;   // [hd] or null
    const float2* rope;                 // [B][rope_half] (launch_rope_table) or null
    int rope_layout;                    // DDL_ROPE_NEOX: pairs (i, i + rope_half);
                                        // DDL_ROPE_NORM: pairs (2i, 2i + 1); i < rope_half
    int rope_half;                      // rotated pairs per head (rot_dim / 2)
    int B, S, hq, hkv, hd, gated; float eps;
    f16* q16;                           // [B][hq*hd]
    float* k_rows; float* v_rows;       // [B][hkv*hd]
    f16* k16; f16* vt16; int tcap;
};
hipError_t launch_qkv_post(const QkvPostArgs& a, hipStream_t s);

struct StagePrefixArgs {
    const float* pk; const float* pv;   // [S][hkv*hd]
    int S, hkv, hd;
    f16* k16; f16* vt16; int tcap;
};
hipError_t launch_stage_prefix(const StagePrefixArgs& a, hipStream_t s);

struct AttnPrefillArgs {
    const f16* q16;                      // [B][hq*hd]
    const f16* k16; const f16* vt16; int tcap;   // staged keys/values (QkvPostArgs)
    const float* gate; int gate_ld;      // gate (B rows, stride gate_ld) or null
    f16* o16;                            // [B][hq*hd]
    int B, S, hq, hkv, hd;
    float softcap;
    int window;                          // > 0: token at position p sees keys p-window+1 .. p
    int form;                            // DDL_ATTN_*
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s);

// packing
hipError_t launch_absmax(const void* src, int dtype, size_t n, uint32_t* out_bits,
                         hipStream_t s);
hipError_t launch_finalize_scales(BlobHeader* hdr, hipStream_t s);
// Converts a [rows][cols] matrix into fp16 rows of dst, a matrix of
// dst_rows x cols stored in MFMA-fragment order: mode 0: dst row =
// row_offset + r; mode 1/2: gate/up interleave (gate / up).
hipError_t launch_convert_rows(const void* src, int dtype, int rows, int cols, f16* dst,
                               int row_offset, int mode, const BlobHeader* hdr, int mat,
                               hipStream_t s);
// Offset (in elements) of element (r, c) of a fragment-ordered matrix with
// `cols` columns.
__host__ __device__ inline size_t frag_index(int r, int c, int cols) {
    return ((size_t)(r >> 5) * (cols >> 4) + (c >> 4)) * 512 + ((r & 31) + 32 * ((c >> 3) & 1)) * 8 +
           (c & 7);
}

// decode (one token against the mirror)
constexpr int DECODE_MAX_SPLITS = 256;
struct DecodeAttnArgs {
    const float* q;                      // [hq*hd]
    const float* knew; const float* vnew; // [hkv*hd] this token's rows
    float* mk; float* mv;                // mirror [cap][hkv*hd]; row R is written
    const float* gate;                   // [hq*hd] or null
    float* part_m; float* part_l;        // [hq][n_splits]
    float* part_o;                       // [hq][n_splits][hd]
    float* o;                            // [hq*hd] merged, normalised, gated
    int R, hq, hkv, hd;
    int n_splits, rows_per_split;
    float softcap;
    // Non-null: the row count lives in device memory and R is read from it
    // (a step replayed from a graph); rows per split (other row widths) are
    // then derived in the kernel, and the combine kernel advances the count
    // by one after every read of it has happened.
    int* R_dev;
};
bool decode_group_ok(int hq, int hkv, int hd);
constexpr int DECODE_ROWS_SPLITS = 184;   // split cap of the row-per-wave kernel
bool decode_rows_kernel_ok(int hq, int hkv, int hd);
void decode_split_plan(int hq, int hkv, int hd, int rows_total, int* n_splits, int* rows_per_split);
hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s);
// *dst = value (one thread): the device row count of a replayed decode step
hipError_t launch_set_int(int* dst, int value, hipStream_t s);

enum { GV_RESID = 0, GV_SWIGLU = 1 };
struct GemvArgs {
    const f16* W; int K;         // [rows][K] fragment-ordered weights (gate/up interleaved for GV_SWIGLU)
    int N;                       // outputs
    const float* inv_scale;      // device scalar
    const float* x;              // [K]
    const float* norm_g; float eps;   // RMS-norm x first when norm_g != null
    const float* r;              // [N] residual (GV_RESID; null: y = W x)
    float* y;                    // [N]
    int gelu;                    // GV_SWIGLU: gelu(gate) * up instead of silu(gate) * up
};
bool gemv_shape_ok(int K);

// The single-token head: q/k/v heads of the stacked projection output ->
// q [hq*hd], k_row, v_row [hkv*hd] (bias, Q/K norm, RoPE at pos).
struct DecodeHeadArgs {
    const float* qkv;                    // [nqkv] projection of the normed row
    const float* bias;                   // [nqkv] or null
    const float* q_norm; const float* k_norm;   // [hd] or null
    float eps;
    int rope_on, rope_layout, rot_dim; double theta; const float* freq; float mscale;
    int pos, hq, hkv, hd;
    const int* pos_dev;                  // non-null: the position is read from here
    float* q; float* k_row; float* v_row;
};
hipError_t launch_decode_head(const DecodeHeadArgs& a, hipStream_t s);
hipError_t launch_gemv(const GemvArgs& a, int epi, hipStream_t s);
