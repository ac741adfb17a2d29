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

// One 256-thread block per row; d % 4 == 0.
__global__ __launch_bounds__(256) void rmsnorm_f16_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          f16* __restrict__ h, int d, float eps) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + row * d);
    const float4* gr = reinterpret_cast<const float4*>(g);
    const int n4 = d >> 2;
    float ss = 0.f;
    for (int i = threadIdx.x; i < n4; i += 256) {
        const float4 v = xr[i];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block_sum_256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    half4* hr = reinterpret_cast<half4*>(h + row * d);
    for (int i = threadIdx.x; i < n4; i += 256) {
        const float4 v = xr[i], w = gr[i];
        hr[i] = half4{(f16)(v.x * r * w.x), (f16)(v.y * r * w.y), (f16)(v.z * r * w.z),
                      (f16)(v.w * r * w.w)};
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

// One wave per (token, head slot): slots [0, hq) are q heads, [hq, hq+hkv)
// k heads, [hq+hkv, hq+2*hkv) v heads.  Lane l holds the Neox pair
// (l, l + hd/2); for hd = 64 lanes 32..63 only take part in the reductions.
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs p) {
    const int lane = threadIdx.x & 63;
    const int slots = p.hq + 2 * p.hkv;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= p.B * slots) return;
    const int b = item / slots, slot = item - b * slots;
    const int half = p.hd >> 1;
    const bool active = lane < half;
    const int col0 = slot * p.hd;     // q, k, v slots are contiguous columns
    const float* src = p.qkv + (size_t)b * p.nqkv + col0;
    float x0 = 0.f, x1 = 0.f;
    if (active) {
        x0 = src[lane];
        x1 = src[lane + half];
        if (p.bias) {
            x0 += p.bias[col0 + lane];
            x1 += p.bias[col0 + lane + half];
        }
    }
    const bool is_q = slot < p.hq, is_k = !is_q && slot < p.hq + p.hkv;
    if (is_q || is_k) {
        const float* gn = is_q ? p.q_norm : p.k_norm;
        if (gn) {
            const float ss = wave_sum(x0 * x0 + x1 * x1);
            const float r = 1.0f / sqrtf(ss / (float)p.hd + p.eps);
            if (active) {
                x0 = x0 * r * gn[lane];
                x1 = x1 * r * gn[lane + half];
            }
        }
        if (p.rope && active) {
            const float2 cs = p.rope[(size_t)b * half + lane];
            const float y0 = x0 * cs.x - x1 * cs.y;
            const float y1 = x0 * cs.y + x1 * cs.x;
            x0 = y0;
            x1 = y1;
        }
    }
    if (!active) return;
    if (is_q) {
        f16* dst = p.q16 + (size_t)b * p.hq * p.hd + slot * p.hd;
        dst[lane] = (f16)x0;
        dst[lane + half] = (f16)x1;
    } else {
        const int g = is_k ? slot - p.hq : slot - p.hq - p.hkv;
        float* dst = (is_k ? p.k_rows : p.v_rows) + (size_t)b * p.hkv * p.hd + g * p.hd;
        dst[lane] = x0;
        dst[lane + half] = x1;
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
        dst[(size_t)dr * cols + c] = (f16)ldexpf(load_weight(src, dtype, i), sh);
    }
}

int grid_for(size_t n) {
    size_t g = (n + 255) / 256;
    return (int)(g > 8192 ? 8192 : (g < 1 ? 1 : g));
}

}  // namespace

hipError_t launch_rmsnorm_f16(const float* x, const float* g, f16* h, int rows, int d, float eps,
                              hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3(rows), dim3(256), 0, s, x, g, h, d, eps);
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
    const int items = a.B * (a.hq + 2 * a.hkv);
    hipLaunchKernelGGL(qkv_post_kernel, dim3((items + 3) / 4), dim3(256), 0, s, a);
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
