// Row-wise steps between the matmuls, and the weight-packing kernels.
//
// RMSNorm follows the plain weighted RMS norm of a pre-norm layer
// ("frink-models 0.49.0 src/fused_layer.rs", LayerFfnParts::for_layer; one
// epsilon per layer, "frink-models 0.29.0 src/decoder/cuda_prefill.rs",
// try_cuda_prefill_dense_stack): h = x / sqrt(mean(x^2) + eps) * g.
// The QKV post-step applies the layer's optional q/k/v biases and per-head
// Q/K RMS norms, then RoPE at position start_pos + b (cuda_prefill.rs,
// cuda_prefill_layer: AttnExtras and the RoPE description), and writes the
// K/V rows the call returns.
#include "common.h"
#include "internal.h"

namespace {

// One 256-thread block per row; d % 4 == 0, d <= 4096.  The row and the
// gains are loaded once into registers (one memory round trip), reduced,
// normalised and stored as fp16.
constexpr int RMS_V4 = 4;   // float4s per thread: 256 * 4 * 4 = 4096 columns

// With nparts > 0 the split-K partials of the GEMM that produced x are
// added first (in slice order).  With gpost (a sandwich-norm layer's
// post-attention or post-FFN gain, "frink-models 0.29.0
// src/decoder/cuda_prefill.rs", cuda_prefill_layer: post_attn_norm,
// post_ffn_norm) that sum is the branch output y and the row becomes
// base + rms_norm(y) * gpost, the residual added after the branch's own norm.
// The row is written back to x when it changed; h (null: skipped) gets
// fp16(rms_norm(row) * g).
__global__ __launch_bounds__(256) void rmsnorm_f16_kernel(float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          f16* __restrict__ h, int d, float eps,
                                                          const float* __restrict__ part,
                                                          int nparts, size_t pstride,
                                                          const float* __restrict__ base,
                                                          const float* __restrict__ gpost) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    float4* xr = reinterpret_cast<float4*>(x + row * d);
    const int n4 = d >> 2;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 v[RMS_V4];
#pragma unroll
    for (int k = 0; k < RMS_V4; ++k) {
        const int i = threadIdx.x + k * 256;
        v[k] = i < n4 ? xr[i] : zero;
    }
    if (nparts > 0) {
        for (int z = 0; z < nparts; ++z) {
            const float4* pr = reinterpret_cast<const float4*>(part + z * pstride + row * d);
#pragma unroll
            for (int k = 0; k < RMS_V4; ++k) {
                const int i = threadIdx.x + k * 256;
                if (i < n4) {
                    const float4 q = pr[i];
                    v[k].x += q.x; v[k].y += q.y; v[k].z += q.z; v[k].w += q.w;
                }
            }
        }
    }
    auto row_scale = [&]() {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < RMS_V4; ++k)
            ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
        ss = block_sum_256(ss, red);
        return 1.0f / sqrtf(ss / (float)d + eps);
    };
    if (gpost) {
        const float r = row_scale();
        const float4* br = reinterpret_cast<const float4*>(base + row * d);
        const float4* pg = reinterpret_cast<const float4*>(gpost);
#pragma unroll
        for (int k = 0; k < RMS_V4; ++k) {
            const int i = threadIdx.x + k * 256;
            if (i < n4) {
                const float4 b = br[i], gp = pg[i];
                v[k] = make_float4(b.x + v[k].x * r * gp.x, b.y + v[k].y * r * gp.y,
                                   b.z + v[k].z * r * gp.z, b.w + v[k].w * r * gp.w);
            }
        }
    }
    if (nparts > 0 || gpost) {
#pragma unroll
        for (int k = 0; k < RMS_V4; ++k) {
            const int i = threadIdx.x + k * 256;
            if (i < n4) xr[i] = v[k];
        }
    }
    if (!h) return;
    const float4* gr = reinterpret_cast<const float4*>(g);
    const float r = row_scale();
    half4* hr = reinterpret_cast<half4*>(h + row * d);
#pragma unroll
    for (int k = 0; k < RMS_V4; ++k) {
        const int i = threadIdx.x + k * 256;
        if (i < n4) {
            const float4 w = gr[i];
            hr[i] = half4{(f16)(v[k].x * r * w.x), (f16)(v[k].y * r * w.y),
                          (f16)(v[k].z * r * w.z), (f16)(v[k].w * r * w.w)};
        }
    }
}

// cos/sin of rotated pair i at position start_pos + b, times the attention
// factor m; the angle is computed in fp64: (start_pos + b) * theta^(-2i/rot_dim)
// divided by the pair's frequency factor when the layer has them
// ("frink-models 0.29.0 src/decoder/cuda_prefill.rs", cuda_prefill_layer:
// theta, freq_factors, rot_dim, mscale).
__global__ void rope_table_kernel(float2* tab, int batch, int start_pos, int rot_dim,
                                  double theta, const float* freq, float mscale) {
    const int half = rot_dim / 2;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= batch * half) return;
    const int b = idx / half, i = idx - b * half;
    double inv = pow(theta, -2.0 * (double)i / (double)rot_dim);
    if (freq) inv /= (double)freq[i];
    const double ang = (double)(start_pos + b) * inv;
    tab[idx] = make_float2((float)(mscale * cos(ang)), (float)(mscale * sin(ang)));
}

// One 256-thread block per (block of 32 tokens, head slot).  Slots: [0, hq)
// q heads, [hq, hq+hkv) k heads, [hq+hkv, hq+2hkv) v heads, then (a gated
// layer with split-K partials only) the gate heads, whose summed columns are
// written back into the projection for the attention to read.  Thread t
// takes token t/8 and, for i = 0 .. HD/32-1, the four head elements
// 32i + 4(t%8) .. +3: the eight threads of a token read its 128-byte runs
// together, and the Neox partner of element e (e < HD/2) is element
// e + HD/2 of the same thread.
// q goes to q16 (fp16), k to the K rows (fp32) and to K16[g][S+b] (fp16),
// v to the V rows (fp32) and, transposed through LDS, to Vt16[g][e][S+b].
// Block index nblk (one past the last token block) zero-fills K16/Vt16 rows
// [S+32*nblk, S+32*nblk+32), so every 32-key tile the attention reads is
// finite.  NP: split-K partial slices added (in slice order).
template <int HD, int NP>
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs p) {
    constexpr int NG = HD / 32;          // float4 groups per thread
    __shared__ f16 vt[HD][33];
    const int tid = threadIdx.x, tl = tid >> 3, part = tid & 7;
    const int blk = blockIdx.x, slot = blockIdx.y;
    const int nblk = (p.B + 31) / 32;
    const int b = blk * 32 + tl;
    const bool is_q = slot < p.hq, is_k = !is_q && slot < p.hq + p.hkv;
    const bool is_v = !is_q && !is_k && slot < p.hq + 2 * p.hkv;
    const bool is_gate = !is_q && !is_k && !is_v;
    const int g = is_k ? slot - p.hq : (is_v ? slot - p.hq - p.hkv : 0);
    const int eoff = part * 4;           // element 32*i + eoff + c
    const bool valid = blk < nblk && b < p.B;
    if (blk == nblk && !is_k && !is_v) return;
    if (is_gate && !valid) return;

    float4 x[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int col0 = slot * HD + eoff;   // q, k, v, gate slots are contiguous columns
    if (valid) {
        const float* src = p.qkv + (size_t)b * p.nqkv + col0;
        float4 q[NP > 0 ? NP : 1][NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) x[i] = *reinterpret_cast<const float4*>(src + 32 * i);
#pragma unroll
        for (int z = 0; z < NP; ++z) {
            const float* ps = p.part + ((size_t)z * p.B + b) * p.nqkv + col0;
#pragma unroll
            for (int i = 0; i < NG; ++i) q[z][i] = *reinterpret_cast<const float4*>(ps + 32 * i);
        }
#pragma unroll
        for (int z = 0; z < NP; ++z)
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                x[i].x += q[z][i].x; x[i].y += q[z][i].y; x[i].z += q[z][i].z; x[i].w += q[z][i].w;
            }
        if (is_gate) {
            float* dst = p.qkv + (size_t)b * p.nqkv + col0;
#pragma unroll
            for (int i = 0; i < NG; ++i) *reinterpret_cast<float4*>(dst + 32 * i) = x[i];
            return;
        }
        if (p.bias) {
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const float4 c = *reinterpret_cast<const float4*>(p.bias + col0 + 32 * i);
                x[i].x += c.x; x[i].y += c.y; x[i].z += c.z; x[i].w += c.w;
            }
        }
    }
    if (is_q || is_k) {
        const float* gn = is_q ? p.q_norm : p.k_norm;
        if (gn) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < NG; ++i) ss += x[i].x * x[i].x + x[i].y * x[i].y + x[i].z * x[i].z + x[i].w * x[i].w;
            ss += __shfl_xor(ss, 1, 64);
            ss += __shfl_xor(ss, 2, 64);
            ss += __shfl_xor(ss, 4, 64);
            const float r = 1.0f / sqrtf(ss / (float)HD + p.eps);
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const float4 c = *reinterpret_cast<const float4*>(gn + eoff + 32 * i);
                x[i].x = x[i].x * r * c.x; x[i].y = x[i].y * r * c.y;
                x[i].z = x[i].z * r * c.z; x[i].w = x[i].w * r * c.w;
            }
        }
        if (p.rope) {
            const float* cs = reinterpret_cast<const float*>(p.rope + (size_t)(valid ? b : 0) * p.rope_half);
            if (p.rope_layout == DDL_ROPE_NEOX) {
                // pair (e, e + rope_half), rope_half = 32k: element e = 32i + eoff + c
                // (i < k) pairs with x[i + k] of the same thread; angle index e
                const int k = p.rope_half / 32;
#pragma unroll
                for (int i = 0; i < NG / 2; ++i) {
                    if (i >= k) break;
                    const float4 c01 = *reinterpret_cast<const float4*>(cs + 2 * (32 * i + eoff));
                    const float4 c23 = *reinterpret_cast<const float4*>(cs + 2 * (32 * i + eoff) + 4);
                    const float4 a = x[i];
#pragma unroll
                    for (int j = 0; j < NG; ++j) {       // x[i + k], with k not a compile-time value
                        if (j != i + k) continue;
                        const float4 o = x[j];
                        x[i] = make_float4(a.x * c01.x - o.x * c01.y, a.y * c01.z - o.y * c01.w,
                                           a.z * c23.x - o.z * c23.y, a.w * c23.z - o.w * c23.w);
                        x[j] = make_float4(a.x * c01.y + o.x * c01.x, a.y * c01.w + o.y * c01.z,
                                           a.z * c23.y + o.z * c23.x, a.w * c23.w + o.w * c23.z);
                    }
                }
            } else {
                // adjacent pairs (2j, 2j + 1) = (x, y) and (z, w) of a float4; pair
                // j = e/2 rotates while j < rope_half
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const int j0 = (32 * i + eoff) >> 1;
                    if (j0 < p.rope_half) {
                        const float2 c0 = *reinterpret_cast<const float2*>(cs + 2 * j0);
                        const float a = x[i].x, o = x[i].y;
                        x[i].x = a * c0.x - o * c0.y;
                        x[i].y = a * c0.y + o * c0.x;
                    }
                    if (j0 + 1 < p.rope_half) {
                        const float2 c1 = *reinterpret_cast<const float2*>(cs + 2 * (j0 + 1));
                        const float a = x[i].z, o = x[i].w;
                        x[i].z = a * c1.x - o * c1.y;
                        x[i].w = a * c1.y + o * c1.x;
                    }
                }
            }
        }
    }
    auto h4 = [](float4 v) { return half4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w}; };
    if (is_q) {
        if (valid) {
            f16* dst = p.q16 + (size_t)b * p.hq * HD + slot * HD + eoff;
#pragma unroll
            for (int i = 0; i < NG; ++i) *reinterpret_cast<half4*>(dst + 32 * i) = h4(x[i]);
        }
        return;
    }
    const size_t key = (size_t)p.S + b;            // row in the staged K/V
    if (is_k) {
        if (valid) {
            float* dst = p.k_rows + (size_t)b * p.hkv * HD + g * HD + eoff;
#pragma unroll
            for (int i = 0; i < NG; ++i) *reinterpret_cast<float4*>(dst + 32 * i) = x[i];
        }
        f16* kd = p.k16 + ((size_t)g * p.tcap + key) * HD + eoff;
#pragma unroll
        for (int i = 0; i < NG; ++i) *reinterpret_cast<half4*>(kd + 32 * i) = h4(x[i]);   // zeros past B
        return;
    }
    // v
    if (valid) {
        float* dst = p.v_rows + (size_t)b * p.hkv * HD + g * HD + eoff;
#pragma unroll
        for (int i = 0; i < NG; ++i) *reinterpret_cast<float4*>(dst + 32 * i) = x[i];
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int e = 32 * i + eoff;
        vt[e][tl] = (f16)x[i].x;
        vt[e + 1][tl] = (f16)x[i].y;
        vt[e + 2][tl] = (f16)x[i].z;
        vt[e + 3][tl] = (f16)x[i].w;
    }
    __syncthreads();
    // row e of Vt16 gets this block's 32 keys at their positions vt_pos(key):
    // when the block's first key is 16-aligned its keys fill its own 32
    // positions, written as 16-byte stores of 8 positions; else one key at a
    // time (a 16-key group then spans two writers, each writing its keys)
    if ((p.S & 15) == 0) {
        for (int idx = tid; idx < HD * 4; idx += 256) {
            const int e = idx >> 2, t0 = (idx & 3) * 8;
            half8 w;
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = vt[e][vt_pos(t0 + u)];
            *reinterpret_cast<half8*>(p.vt16 + ((size_t)g * HD + e) * p.tcap + p.S + blk * 32 + t0) = w;
        }
    } else {
        for (int idx = tid; idx < HD * 32; idx += 256) {
            const int e = idx >> 5, t = idx & 31;
            p.vt16[((size_t)g * HD + e) * p.tcap + vt_pos(p.S + blk * 32 + t)] = vt[e][t];
        }
    }
}

// Cached rows [0, S) of one layer into the staged fp16 layouts: K16[g][j]
// and Vt16[g][e][vt_pos(j)].  One block per (32 rows, KV head).
template <int HD>
__global__ __launch_bounds__(256) void stage_prefix_kernel(StagePrefixArgs p) {
    __shared__ f16 vt[HD][33];
    const int blk = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int kvw = p.hkv * HD;
    for (int idx = tid; idx < 32 * HD / 4; idx += 256) {
        const int t = idx / (HD / 4), e = (idx % (HD / 4)) * 4;
        const int j = blk * 32 + t;
        float4 k = make_float4(0.f, 0.f, 0.f, 0.f), v = k;
        if (j < p.S) {
            k = *reinterpret_cast<const float4*>(p.pk + (size_t)j * kvw + g * HD + e);
            v = *reinterpret_cast<const float4*>(p.pv + (size_t)j * kvw + g * HD + e);
            *reinterpret_cast<half4*>(p.k16 + ((size_t)g * p.tcap + j) * HD + e) =
                half4{(f16)k.x, (f16)k.y, (f16)k.z, (f16)k.w};
        }
        vt[e][t] = (f16)v.x;
        vt[e + 1][t] = (f16)v.y;
        vt[e + 2][t] = (f16)v.z;
        vt[e + 3][t] = (f16)v.w;
    }
    __syncthreads();
    for (int idx = tid; idx < HD * 32; idx += 256) {
        const int e = idx >> 5, t = idx & 31, j = blk * 32 + t;
        if (j < p.S) p.vt16[((size_t)g * HD + e) * p.tcap + vt_pos(j)] = vt[e][t];
    }
}

// ---- packing ---------------------------------------------------------------

__device__ __forceinline__ float load_weight(const void* src, int dtype, size_t i) {
    return dtype == DDL_DTYPE_BF16 ? bf16_bits_to_float(static_cast<const uint16_t*>(src)[i])
                                   : static_cast<const float*>(src)[i];
}

__global__ __launch_bounds__(256) void absmax_kernel(const void* src, int dtype, size_t n,
                                                     uint32_t* out_bits) {
    float m = 0.f;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        m = fmaxf(m, fabsf(load_weight(src, dtype, i)));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomicMax(out_bits, __float_as_uint(m));
}

// shift = 14 - e where max|w| = f * 2^e, f in [0.5, 1): max|w| * 2^shift < 2^14.
__global__ void finalize_scales_kernel(BlobHeader* hdr) {
    const int i = threadIdx.x;
    if (i >= MAT_COUNT) return;
    const float m = __uint_as_float(hdr->absmax_bits[i]);
    int sh = 0;
    if (m > 0.f) {
        int e;
        frexpf(m, &e);
        sh = 14 - e;
        sh = sh < -24 ? -24 : (sh > 40 ? 40 : sh);
    }
    hdr->shift[i] = sh;
    hdr->inv_scale[i] = ldexpf(1.0f, -sh);
}

__global__ __launch_bounds__(256) void convert_rows_kernel(const void* src, int dtype, int rows,
                                                           int cols, f16* dst, int row_offset,
                                                           int mode, const BlobHeader* hdr,
                                                           int mat) {
    const int sh = hdr->shift[mat];
    const size_t n = (size_t)rows * cols;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const int r = (int)(i / cols), c = (int)(i - (size_t)r * cols);
        int dr = row_offset + r;
        if (mode != 0) dr = (r >> 4) * 32 + (mode - 1) * 16 + (r & 15);
        dst[frag_index(dr, c, cols)] = (f16)ldexpf(load_weight(src, dtype, i), sh);
    }
}

int grid_for(size_t n) {
    size_t g = (n + 255) / 256;
    return (int)(g > 8192 ? 8192 : (g < 1 ? 1 : g));
}

}  // namespace

hipError_t launch_rmsnorm_f16(float* x, const float* g, f16* h, int rows, int d, float eps,
                              const float* part, int nparts, const float* base,
                              const float* gpost, hipStream_t s) {
    if (d % 4 || d > 256 * 4 * RMS_V4 || (nparts > 0 && !part) || (gpost && !base) || (h && !g))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3(rows), dim3(256), 0, s, x, g, h, d, eps, part,
                       nparts, (size_t)rows * d, base, gpost);
    return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int batch, int start_pos, int rot_dim, double theta,
                             const float* freq, float mscale, hipStream_t s) {
    if (rot_dim < 2 || rot_dim % 2) return hipErrorInvalidValue;
    const int n = batch * (rot_dim / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tab, batch,
                       start_pos, rot_dim, theta, freq, mscale);
    return hipGetLastError();
}

namespace {
template <int HD>
hipError_t launch_qkv_post_hd(const QkvPostArgs& a, dim3 grid, hipStream_t s) {
    switch (a.nparts) {
        case 0: hipLaunchKernelGGL((qkv_post_kernel<HD, 0>), grid, dim3(256), 0, s, a); break;
        case 1: hipLaunchKernelGGL((qkv_post_kernel<HD, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((qkv_post_kernel<HD, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((qkv_post_kernel<HD, 3>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_qkv_post(const QkvPostArgs& a, hipStream_t s) {
    // at most three partial slices (a four-way K split)
    if (a.nparts < 0 || a.nparts > 3 || (a.nparts > 0 && !a.part)) return hipErrorInvalidValue;
    // rotated pairs: Neox needs rope_half a multiple of 32 (a thread holds
    // both channels of its pairs), Norm any count up to hd/2
    if (a.rope && (a.rope_half < 1 || 2 * a.rope_half > a.hd ||
                   (a.rope_layout == DDL_ROPE_NEOX && a.rope_half % 32) ||
                   (a.rope_layout != DDL_ROPE_NEOX && a.rope_layout != DDL_ROPE_NORM)))
        return hipErrorInvalidValue;
    // the gate heads (a gated layer's second q half) take part only to get
    // their split-K partials added
    const int slots = a.hq + 2 * a.hkv + (a.gated && a.nparts > 0 ? a.hq : 0);
    const dim3 grid((a.B + 31) / 32 + 1, slots);
    if (a.hd == 128) return launch_qkv_post_hd<128>(a, grid, s);
    if (a.hd == 64) return launch_qkv_post_hd<64>(a, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_stage_prefix(const StagePrefixArgs& a, hipStream_t s) {
    if (a.S <= 0) return hipSuccess;
    const dim3 grid((a.S + 31) / 32, a.hkv);
    if (a.hd == 128)
        hipLaunchKernelGGL(stage_prefix_kernel<128>, grid, dim3(256), 0, s, a);
    else if (a.hd == 64)
        hipLaunchKernelGGL(stage_prefix_kernel<64>, grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_absmax(const void* src, int dtype, size_t n, uint32_t* out_bits,
                         hipStream_t s) {
    hipLaunchKernelGGL(absmax_kernel, dim3(grid_for(n)), dim3(256), 0, s, src, dtype, n,
                       out_bits);
    return hipGetLastError();
}

hipError_t launch_finalize_scales(BlobHeader* hdr, hipStream_t s) {
    hipLaunchKernelGGL(finalize_scales_kernel, dim3(1), dim3(64), 0, s, hdr);
    return hipGetLastError();
}

hipError_t launch_convert_rows(const void* src, int dtype, int rows, int cols, f16* dst,
                               int row_offset, int mode, const BlobHeader* hdr, int mat,
                               hipStream_t s) {
    hipLaunchKernelGGL(convert_rows_kernel, dim3(grid_for((size_t)rows * cols)), dim3(256), 0, s,
                       src, dtype, rows, cols, dst, row_offset, mode, hdr, mat);
    return hipGetLastError();
}
