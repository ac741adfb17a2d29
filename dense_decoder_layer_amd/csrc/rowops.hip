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
// added first (in slice order) and the sum is written back to x.
__global__ __launch_bounds__(256) void rmsnorm_f16_kernel(float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          f16* __restrict__ h, int d, float eps,
                                                          const float* __restrict__ part,
                                                          int nparts, size_t pstride) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    float4* xr = reinterpret_cast<float4*>(x + row * d);
    const float4* gr = reinterpret_cast<const float4*>(g);
    const int n4 = d >> 2;
    float4 v[RMS_V4], w[RMS_V4];
#pragma unroll
    for (int k = 0; k < RMS_V4; ++k) {
        const int i = threadIdx.x + k * 256;
        v[k] = i < n4 ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        w[k] = i < n4 ? gr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
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
#pragma unroll
        for (int k = 0; k < RMS_V4; ++k) {
            const int i = threadIdx.x + k * 256;
            if (i < n4) xr[i] = v[k];
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < RMS_V4; ++k) ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    ss = block_sum_256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    half4* hr = reinterpret_cast<half4*>(h + row * d);
#pragma unroll
    for (int k = 0; k < RMS_V4; ++k) {
        const int i = threadIdx.x + k * 256;
        if (i < n4)
            hr[i] = half4{(f16)(v[k].x * r * w[k].x), (f16)(v[k].y * r * w[k].y),
                          (f16)(v[k].z * r * w[k].z), (f16)(v[k].w * r * w[k].w)};
    }
}

// cos/sin of pair i at position start_pos + b, angle computed in fp64:
// (start_pos + b) * theta^(-2i/rot_dim).
__global__ void rope_table_kernel(float2* tab, int batch, int start_pos, int half, int rot_dim,
                                  double theta) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= batch * half) return;
    const int b = idx / half, i = idx - b * half;
    const double inv = pow(theta, -2.0 * (double)i / (double)rot_dim);
    const double ang = (double)(start_pos + b) * inv;
    tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// One 256-thread block per (block of 32 tokens, head slot).  Slots: [0, hq)
// q heads, [hq, hq+hkv) k heads, [hq+hkv, hq+2hkv) v heads (a gated layer's
// gate columns are read by the attention straight from the projection).  Thread t takes token t/8 and head elements
// [(t%8)*HD/8, +HD/8); the Neox partner of element e (e < HD/2) lives in
// thread t^4.
// q goes to q16 (fp16), k to the K rows (fp32) and to K16[g][S+b] (fp16),
// v to the V rows (fp32) and, transposed through LDS, to Vt16[g][e][S+b].
// Block index nblk (one past the last
// token block) zero-fills K16/Vt16 rows [S+32*nblk, S+32*nblk+32), so every
// 32-key tile the attention reads is finite.
template <int HD>
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs p) {
    constexpr int EPT = HD / 8;          // elements per thread
    __shared__ f16 vt[HD][33];
    const int tid = threadIdx.x, tl = tid >> 3, part = tid & 7;
    const int blk = blockIdx.x, slot = blockIdx.y;
    const int nblk = (p.B + 31) / 32;
    const int b = blk * 32 + tl;
    const bool is_q = slot < p.hq, is_k = !is_q && slot < p.hq + p.hkv;
    const bool is_v = !is_q && !is_k && slot < p.hq + 2 * p.hkv;
    const bool is_gate = !is_q && !is_k && !is_v;     // launched only with partials to add
    const int g = is_k ? slot - p.hq : (is_v ? slot - p.hq - p.hkv : 0);
    const int e0 = part * EPT;
    const bool valid = blk < nblk && b < p.B;
    if (blk == nblk && !is_k && !is_v) return;
    if (is_gate && !valid) return;

    float x[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) x[i] = 0.f;
    const int col0 = slot * HD + e0;     // q, k, v, gate slots are contiguous columns
    if (valid) {
        const float* src = p.qkv + (size_t)b * p.nqkv + col0;
#pragma unroll
        for (int i = 0; i < EPT; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(src + i);
            x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
        }
        for (int z = 0; z < p.nparts; ++z) {
            const float* ps = p.part + ((size_t)z * p.B + b) * p.nqkv + col0;
#pragma unroll
            for (int i = 0; i < EPT; i += 4) {
                const float4 v = *reinterpret_cast<const float4*>(ps + i);
                x[i] += v.x; x[i + 1] += v.y; x[i + 2] += v.z; x[i + 3] += v.w;
            }
        }
        if (is_gate) {          // the attention reads the gate from the projection
            float* dst = p.qkv + (size_t)b * p.nqkv + col0;
#pragma unroll
            for (int i = 0; i < EPT; i += 4)
                *reinterpret_cast<float4*>(dst + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
            return;
        }
        if (p.bias) {
#pragma unroll
            for (int i = 0; i < EPT; ++i) x[i] += p.bias[col0 + i];
        }
    }
    if (is_q || is_k) {
        const float* gn = is_q ? p.q_norm : p.k_norm;
        if (gn) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < EPT; ++i) ss += x[i] * x[i];
            ss += __shfl_xor(ss, 1, 64);
            ss += __shfl_xor(ss, 2, 64);
            ss += __shfl_xor(ss, 4, 64);
            const float r = 1.0f / sqrtf(ss / (float)HD + p.eps);
#pragma unroll
            for (int i = 0; i < EPT; ++i) x[i] = x[i] * r * gn[e0 + i];
        }
        if (p.rope) {
            const bool first = part < 4;          // holds the a of the pairs (a, b)
            const int ebase = (first ? e0 : e0 - HD / 2);
            const float2* cs = p.rope + (size_t)(valid ? b : 0) * (HD / 2) + ebase;
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const float other = __shfl_xor(x[i], 4, 64);
                const float2 c = cs[i];
                x[i] = first ? x[i] * c.x - other * c.y : other * c.y + x[i] * c.x;
            }
        }
    }
    if (is_q) {
        if (valid) {
            half8* dst = reinterpret_cast<half8*>(p.q16 + (size_t)b * p.hq * HD + slot * HD + e0);
#pragma unroll
            for (int i = 0; i < EPT; i += 8)
                dst[i / 8] = half8{(f16)x[i], (f16)x[i + 1], (f16)x[i + 2], (f16)x[i + 3],
                                   (f16)x[i + 4], (f16)x[i + 5], (f16)x[i + 6], (f16)x[i + 7]};
        }
        return;
    }
    const size_t key = (size_t)p.S + b;            // row in the staged K/V
    if (is_k) {
        if (valid) {
            float* dst = p.k_rows + (size_t)b * p.hkv * HD + g * HD + e0;
#pragma unroll
            for (int i = 0; i < EPT; i += 4)
                *reinterpret_cast<float4*>(dst + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
        }
        half8* kd = reinterpret_cast<half8*>(p.k16 + ((size_t)g * p.tcap + key) * HD + e0);
#pragma unroll
        for (int i = 0; i < EPT; i += 8)                      // zeros past B
            kd[i / 8] = half8{(f16)x[i], (f16)x[i + 1], (f16)x[i + 2], (f16)x[i + 3],
                              (f16)x[i + 4], (f16)x[i + 5], (f16)x[i + 6], (f16)x[i + 7]};
        return;
    }
    // v
    if (valid) {
        float* dst = p.v_rows + (size_t)b * p.hkv * HD + g * HD + e0;
#pragma unroll
        for (int i = 0; i < EPT; i += 4)
            *reinterpret_cast<float4*>(dst + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) vt[e0 + i][tl] = (f16)x[i];
    __syncthreads();
    // row e of Vt16 gets this block's 32 keys
    for (int idx = tid; idx < HD * 32; idx += 256) {
        const int e = idx >> 5, t = idx & 31;
        p.vt16[((size_t)g * HD + e) * p.tcap + p.S + blk * 32 + t] = vt[e][t];
    }
}

// Cached rows [0, S) of one layer into the staged fp16 layouts: K16[g][j]
// and Vt16[g][e][j].  One block per (32 rows, KV head).
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
        if (j < p.S) p.vt16[((size_t)g * HD + e) * p.tcap + j] = vt[e][t];
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
                              const float* part, int nparts, hipStream_t s) {
    if (d % 4 || d > 256 * 4 * RMS_V4 || (nparts > 0 && !part)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3(rows), dim3(256), 0, s, x, g, h, d, eps, part,
                       nparts, (size_t)rows * d);
    return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int batch, int start_pos, int half, int rot_dim,
                             double theta, hipStream_t s) {
    const int n = batch * half;
    hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tab, batch,
                       start_pos, half, rot_dim, theta);
    return hipGetLastError();
}

hipError_t launch_qkv_post(const QkvPostArgs& a, hipStream_t s) {
    if (a.nparts > 0 && !a.part) return hipErrorInvalidValue;
    // the gate heads (a gated layer's second q half) take part only to get
    // their split-K partials added
    const int slots = a.hq + 2 * a.hkv + (a.gated && a.nparts > 0 ? a.hq : 0);
    const dim3 grid((a.B + 31) / 32 + 1, slots);
    if (a.hd == 128)
        hipLaunchKernelGGL(qkv_post_kernel<128>, grid, dim3(256), 0, s, a);
    else if (a.hd == 64)
        hipLaunchKernelGGL(qkv_post_kernel<64>, grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
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
