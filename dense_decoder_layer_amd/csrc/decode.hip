// One token's attention layer against the device KV mirror
// ("frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_layer: attention over the mirror, output gate, wo,
// residual, FFN norm, FFN, residual, in one submission; the gate is the
// half split off a double-width wq; q/k/v arrive rotated and QK-normed).
// The layer tail is x + ffn(rms_norm(x + branch)) with one dense SwiGLU
// expert ("frink-models 0.49.0 src/fused_layer.rs", module doc).
//
// Attention is split over rows: workgroup (split, kv head) walks rows
// [r0, r1) of the mirror, plus the token's own row (index R, read from the
// k/v arguments and written into the mirror by the one workgroup whose range
// holds it), for all query heads of the KV head's group.  Rows are read as
// fp32 with 16 lanes per row (two 256-byte coalesced segments per row for
// head_dim 128) and the softmax is online per lane group; the groups and
// waves are merged in a fixed order and one unnormalised partial (m, l, o)
// per (query head, split) goes to the workspace.  A second kernel merges
// the splits in order, normalises and applies the gate.  Everything is
// fp32 with fp16 weights widened on load.
#include "common.h"
#include "internal.h"

namespace {

template <int HD, int G>
__global__ __launch_bounds__(256) void decode_attn_split_kernel(DecodeAttnArgs p) {
    constexpr int DPL = HD / 16;        // dims per lane (16 lanes per row)
    constexpr int NF4 = HD / 64;        // float4 chunks per lane: dims j*64 + sub*4 .. +3
    __shared__ float sm[4][G], sl[4][G];
    __shared__ float so[4][G][HD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, sub = lane & 15;
    const int split = blockIdx.x, g = blockIdx.y;
    const int kvw = p.hkv * HD;
    const int nrows = p.R + 1;
    const int r0 = split * p.rows_per_split;
    const int r1 = min(r0 + p.rows_per_split, nrows);
    const float LOG2E = 1.4426950408889634f;
    const float scale = 1.0f / sqrtf((float)HD);

    auto dim_of = [&](int i) { return (i >> 2) * 64 + sub * 4 + (i & 3); };

    float q[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < DPL; ++i) q[h][i] = p.q[(size_t)(g * G + h) * HD + dim_of(i)];

    float m[G], l[G], o[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[h][i] = 0.f;
    }

    for (int base = r0; base < r1; base += 16) {
        const int r = base + wave * 4 + grp;
        const bool valid = r < r1;
        float kx[DPL], vx[DPL];
        const float* ksrc = nullptr;
        const float* vsrc = nullptr;
        if (valid) {
            if (r < p.R) {
                ksrc = p.mk + (size_t)r * kvw + g * HD;
                vsrc = p.mv + (size_t)r * kvw + g * HD;
            } else {
                ksrc = p.knew + g * HD;
                vsrc = p.vnew + g * HD;
            }
        }
#pragma unroll
        for (int j = 0; j < NF4; ++j) {
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (valid) {
                kk = *reinterpret_cast<const float4*>(ksrc + j * 64 + sub * 4);
                vv = *reinterpret_cast<const float4*>(vsrc + j * 64 + sub * 4);
            }
            kx[4 * j] = kk.x; kx[4 * j + 1] = kk.y; kx[4 * j + 2] = kk.z; kx[4 * j + 3] = kk.w;
            vx[4 * j] = vv.x; vx[4 * j + 1] = vv.y; vx[4 * j + 2] = vv.z; vx[4 * j + 3] = vv.w;
        }
        if (valid && r == p.R) {   // append this token's row to the mirror
#pragma unroll
            for (int j = 0; j < NF4; ++j) {
                const size_t at = (size_t)r * kvw + g * HD + j * 64 + sub * 4;
                *reinterpret_cast<float4*>(p.mk + at) =
                    make_float4(kx[4 * j], kx[4 * j + 1], kx[4 * j + 2], kx[4 * j + 3]);
                *reinterpret_cast<float4*>(p.mv + at) =
                    make_float4(vx[4 * j], vx[4 * j + 1], vx[4 * j + 2], vx[4 * j + 3]);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < DPL; ++i) s += q[h][i] * kx[i];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            s += __shfl_xor(s, 8, 64);
            s *= scale;
            if (p.softcap > 0.f) s = p.softcap * tanhf(s / p.softcap);
            s = valid ? s * LOG2E : -INFINITY;
            const float m_new = fmaxf(m[h], s);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2f(m[h] - m_use);
            const float pr = exp2f(s - m_use);
            l[h] = l[h] * alpha + pr;
            m[h] = m_new;
#pragma unroll
            for (int i = 0; i < DPL; ++i) o[h][i] = o[h][i] * alpha + pr * vx[i];
        }
    }

    // merge the four lane groups of the wave (xor 16, then xor 32)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], off, 64);
            const float lo = __shfl_xor(l[h], off, 64);
            const float mn = fmaxf(m[h], mo);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float a = exp2f(m[h] - mu), b = exp2f(mo - mu);
            l[h] = l[h] * a + lo * b;
            m[h] = mn;
#pragma unroll
            for (int i = 0; i < DPL; ++i) {
                const float oo = __shfl_xor(o[h][i], off, 64);
                o[h][i] = o[h][i] * a + oo * b;
            }
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (sub == 0) {
                sm[wave][h] = m[h];
                sl[wave][h] = l[h];
            }
#pragma unroll
            for (int i = 0; i < DPL; ++i) so[wave][h][dim_of(i)] = o[h][i];
        }
    }
    __syncthreads();
    // merge the four waves and write this split's partial
    for (int t = tid; t < G * HD; t += 256) {
        const int h = t / HD, d = t - h * HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][h]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = exp2f(sm[w][h] - Mu);
            L += sl[w][h] * a;
            O += so[w][h][d] * a;
        }
        const int qh = g * G + h;
        const size_t slot = (size_t)qh * p.n_splits + split;
        p.part_o[slot * HD + d] = O;
        if (d == 0) {
            p.part_m[slot] = M;
            p.part_l[slot] = L;
        }
    }
}

// One block per query head, one thread per dim: merge the splits in order,
// normalise, gate.
template <int HD>
__global__ __launch_bounds__(HD) void decode_attn_combine_kernel(DecodeAttnArgs p) {
    const int h = blockIdx.x, d = threadIdx.x;
    const size_t base = (size_t)h * p.n_splits;
    float M = -INFINITY;
    for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, p.part_m[base + s]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < p.n_splits; ++s) {
        const float a = exp2f(p.part_m[base + s] - M);
        L += p.part_l[base + s] * a;
        O += p.part_o[(base + s) * HD + d] * a;
    }
    float r = O / L;
    if (p.gate) r *= 1.0f / (1.0f + expf(-p.gate[(size_t)h * HD + d]));
    p.o[(size_t)h * HD + d] = r;
}

// y = W x (fp16 weights times inv_scale, fp32 x) with fused epilogues; W in
// MFMA-fragment order.  One 512-thread workgroup per 32-row block: x (RMS-
// normed first when norm_g is set) is staged in LDS, the eight waves split
// the 16-column blocks of K round-robin, and lane l accumulates row l % 32
// over columns 16kb + 8*(l/32) .. +7 of each 1 KB fragment block it loads
// (one fully coalesced load per block).  The halves of a row meet with one
// shuffle, the waves in LDS, in a fixed order.
constexpr int GV_WAVES = 8;
constexpr int GV_MAXK = 15872;  // largest K the LDS stage holds (62 KB of dynamic LDS)

template <int EPI>
__global__ __launch_bounds__(GV_WAVES * 64) void gemv_kernel(GemvArgs p) {
    extern __shared__ float xs[];   // [K]
    __shared__ float red[GV_WAVES][32];
    __shared__ float wsum[GV_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < p.K; i += GV_WAVES * 64) xs[i] = p.x[i];
    if (p.norm_g) {
        float ss = 0.f;
        for (int i = tid; i < p.K; i += GV_WAVES * 64) ss += p.x[i] * p.x[i];
        ss = wave_sum(ss);
        if (lane == 0) wsum[wave] = ss;
        __syncthreads();
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < GV_WAVES; ++w) t += wsum[w];
        const float r = 1.0f / sqrtf(t / (float)p.K + p.eps);
        for (int i = tid; i < p.K; i += GV_WAVES * 64) xs[i] = xs[i] * r * p.norm_g[i];
    }
    __syncthreads();
    const int nb = blockIdx.x;
    const int kblocks = p.K >> 4;
    const f16* wb = p.W + (size_t)nb * kblocks * 512 + lane * 8;
    const float* xl = xs + 8 * (lane >> 5);
    float acc = 0.f;
    int kb = wave;
    for (; kb + 3 * GV_WAVES < kblocks; kb += 4 * GV_WAVES) {
        half8 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const half8*>(wb + (size_t)(kb + u * GV_WAVES) * 512);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float* xv = xl + (kb + u * GV_WAVES) * 16;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += (float)w[u][j] * xv[j];
        }
    }
    for (; kb < kblocks; kb += GV_WAVES) {
        const half8 w = *reinterpret_cast<const half8*>(wb + (size_t)kb * 512);
        const float* xv = xl + kb * 16;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += (float)w[j] * xv[j];
    }
    acc += __shfl_xor(acc, 32, 64);
    if (lane < 32) red[wave][lane] = acc;
    __syncthreads();
    if (tid >= 32) return;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) y += red[w][tid];
    y *= *p.inv_scale;
    if constexpr (EPI == GV_SWIGLU) {
        // rows 32nb + t: t < 16 gate, t >= 16 up, of output 16nb + t % 16
        const float other = __shfl_xor(y, 16, 64);
        if (tid < 16) p.y[nb * 16 + tid] = y / (1.0f + expf(-y)) * other;
    } else {
        const int row = nb * 32 + tid;
        p.y[row] = p.r[row] + y;
    }
}

template <int HD>
hipError_t launch_split_hd(const DecodeAttnArgs& a, int G, hipStream_t s) {
    const dim3 grid(a.n_splits, a.hkv);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_attn_split_kernel<HD, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_attn_split_kernel<HD, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((decode_attn_split_kernel<HD, 3>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_attn_split_kernel<HD, 4>), grid, dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_attn_split_kernel<HD, 8>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e) return e;
    hipLaunchKernelGGL(decode_attn_combine_kernel<HD>, dim3(a.hq), dim3(HD), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool decode_group_ok(int hq, int hkv, int hd) {
    if (hkv <= 0 || hq % hkv) return false;
    const int G = hq / hkv;
    return (hd == 64 || hd == 128) && (G == 1 || G == 2 || G == 3 || G == 4 || G == 8);
}

void decode_split_plan(int rows_total, int* n_splits, int* rows_per_split) {
    int splits = (rows_total + 63) / 64;
    if (splits > DECODE_MAX_SPLITS) splits = DECODE_MAX_SPLITS;
    if (splits < 1) splits = 1;
    int per = (rows_total + splits - 1) / splits;
    per = (per + 15) / 16 * 16;
    *n_splits = (rows_total + per - 1) / per;
    *rows_per_split = per;
}

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    if (a.hd == 128) return launch_split_hd<128>(a, G, s);
    if (a.hd == 64) return launch_split_hd<64>(a, G, s);
    return hipErrorInvalidValue;
}

bool gemv_shape_ok(int K) { return K > 0 && K % 16 == 0 && K <= GV_MAXK; }

hipError_t launch_gemv(const GemvArgs& a, int epi, hipStream_t s) {
    if (!gemv_shape_ok(a.K)) return hipErrorInvalidValue;
    // GV_SWIGLU: N outputs from 2N packed rows; GV_RESID: N rows
    const int rows = epi == GV_SWIGLU ? 2 * a.N : a.N;
    if (rows % 32) return hipErrorInvalidValue;
    const dim3 grid(rows / 32);
    if (epi == GV_SWIGLU)
        hipLaunchKernelGGL(gemv_kernel<GV_SWIGLU>, grid, dim3(GV_WAVES * 64), a.K * sizeof(float), s, a);
    else
        hipLaunchKernelGGL(gemv_kernel<GV_RESID>, grid, dim3(GV_WAVES * 64), a.K * sizeof(float), s, a);
    return hipGetLastError();
}
