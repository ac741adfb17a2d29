// One token's attention layer against the device KV mirror
// ("frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_layer: attention over the mirror, output gate, wo,
// residual, FFN norm, FFN, residual, in one submission; the gate is the
// half split off a double-width wq; q/k/v arrive rotated and QK-normed).
// The layer tail is x + ffn(rms_norm(x + branch)) with one dense SwiGLU
// expert ("frink-models 0.49.0 src/fused_layer.rs", module doc).
//
// Attention is split over rows.  Main kernel (KV row width hkv*hd of 256,
// 512 or 1024 floats): one wave reads whole mirror rows -- all KV heads, so
// each load instruction covers contiguous 128-byte runs of the row -- with
// hd/DPL lanes per KV head and DPL dims per lane, and keeps an online
// softmax (running max m, sum l, unnormalised o) for every query head of
// the lane's KV head.  Split s of n takes rows s, s+n, s+2n, ... (wave w of
// the split every 8th of them), so at any moment the whole grid streams one
// contiguous window of the mirror.  The token's own row (index R) comes
// from the k/v arguments and the wave that takes it also writes it into the
// mirror.  The eight waves merge through LDS in a fixed tree and one
// unnormalised partial (m, l, o) per (query head, split) goes to the
// workspace.  Other row widths use a kernel with one KV head per workgroup
// (16 lanes per row, contiguous row ranges per split).  A second kernel
// merges the splits in a fixed order, normalises and applies the gate.
// Everything is fp32 with fp16 weights widened on load.
#include "common.h"
#include "internal.h"

namespace {

constexpr int ROWS_WAVES = 8;      // waves per workgroup of the row-per-wave kernel

template <int HD, int DPL, int G>
__global__ __launch_bounds__(ROWS_WAVES * 64) void decode_attn_rows_kernel(DecodeAttnArgs p) {
    constexpr int NW = ROWS_WAVES;
    constexpr int LPH = HD / DPL;            // lanes per KV head
    constexpr int HKV = 64 / LPH;            // KV heads of a row
    constexpr int HQ = HKV * G;
    constexpr int NC = DPL / 4;              // 16-byte chunks per lane
    static_assert(LPH * HKV == 64 && DPL % 4 == 0 && G * DPL <= 64, "row covers the wave");
    __shared__ float so[NW / 2][HQ][HD];
    __shared__ float sml[NW / 2][HQ][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPH, sub = lane % LPH;
    const int kvw = HKV * HD;
    const int R = p.R_dev ? *p.R_dev : p.R;
    const int nrows = R + 1;
    const int split = blockIdx.x, ns = p.n_splits;
    const float LOG2E = 1.4426950408889634f;
    // chunk c of the lane: dims c*4*LPH + sub*4 .. +3 of KV head g; q is
    // pre-scaled by log2(e)/sqrt(hd), so logits come out in the exp2 domain
    const float qs = LOG2E / sqrtf((float)HD);
    float q[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float4 v = *reinterpret_cast<const float4*>(p.q + (size_t)(g * G + h) * HD + c * 4 * LPH + sub * 4);
            q[h][4 * c] = v.x * qs; q[h][4 * c + 1] = v.y * qs;
            q[h][4 * c + 2] = v.z * qs; q[h][4 * c + 3] = v.w * qs;
        }
    float m[G], l[G], o[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[h][i] = 0.f;
    }
    const float cap = p.softcap, inv_cap = cap > 0.f ? 1.0f / cap : 0.f;
    for (int r = split + ns * wave; r < nrows; r += ns * NW) {
        const float* ks = r < R ? p.mk + (size_t)r * kvw : p.knew;
        const float* vs = r < R ? p.mv + (size_t)r * kvw : p.vnew;
        float kx[DPL], vx[DPL];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float4 kk = *reinterpret_cast<const float4*>(ks + g * HD + c * 4 * LPH + sub * 4);
            const float4 vv = *reinterpret_cast<const float4*>(vs + g * HD + c * 4 * LPH + sub * 4);
            kx[4 * c] = kk.x; kx[4 * c + 1] = kk.y; kx[4 * c + 2] = kk.z; kx[4 * c + 3] = kk.w;
            vx[4 * c] = vv.x; vx[4 * c + 1] = vv.y; vx[4 * c + 2] = vv.z; vx[4 * c + 3] = vv.w;
        }
        if (r == R) {   // append this token's row to the mirror
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const size_t at = (size_t)r * kvw + g * HD + c * 4 * LPH + sub * 4;
                *reinterpret_cast<float4*>(p.mk + at) = make_float4(kx[4 * c], kx[4 * c + 1], kx[4 * c + 2], kx[4 * c + 3]);
                *reinterpret_cast<float4*>(p.mv + at) = make_float4(vx[4 * c], vx[4 * c + 1], vx[4 * c + 2], vx[4 * c + 3]);
            }
        }
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < DPL; ++i) a += q[h][i] * kx[i];
#pragma unroll
            for (int off = 1; off < LPH; off <<= 1) a += __shfl_xor(a, off, 64);
            sc[h] = a;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float v = sc[h];
            if (cap > 0.f) v = cap * LOG2E * tanhf(v * (inv_cap / LOG2E));
            const float m_new = fmaxf(m[h], v);
            const float alpha = exp2f(m[h] - m_new);     // m_new is finite: v is
            const float pr = exp2f(v - m_new);
            l[h] = l[h] * alpha + pr;
            m[h] = m_new;
#pragma unroll
            for (int i = 0; i < DPL; ++i) o[h][i] = o[h][i] * alpha + pr * vx[i];
        }
    }
    // waves [half, 2*half) hand their state to waves [0, half) through LDS
    auto put = [&](int slot) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) so[slot][g * G + h][c * 4 * LPH + sub * 4 + i] = o[h][4 * c + i];
            if (sub == 0) {
                sml[slot][g * G + h][0] = m[h];
                sml[slot][g * G + h][1] = l[h];
            }
        }
    };
    auto take = [&](int slot) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = sml[slot][g * G + h][0], lo = sml[slot][g * G + h][1];
            const float mn = fmaxf(m[h], mo);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float a = exp2f(m[h] - mu), b = exp2f(mo - mu);
            l[h] = l[h] * a + lo * b;
            m[h] = mn;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[h][4 * c + i] = o[h][4 * c + i] * a + so[slot][g * G + h][c * 4 * LPH + sub * 4 + i] * b;
        }
    };
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) put(wave - half);
        __syncthreads();
        if (wave < half) take(wave);
        __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const size_t slot = (size_t)(g * G + h) * ns + split;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                *reinterpret_cast<float4*>(p.part_o + slot * HD + c * 4 * LPH + sub * 4) =
                    make_float4(o[h][4 * c], o[h][4 * c + 1], o[h][4 * c + 2], o[h][4 * c + 3]);
            if (sub == 0) {
                p.part_m[slot] = m[h];
                p.part_l[slot] = l[h];
            }
        }
    }
}

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
    const int R = p.R_dev ? *p.R_dev : p.R;
    const int nrows = R + 1;
    // with the count in device memory the split count is fixed (by the
    // mirror's capacity) and the rows are dealt out here, 16 at a time
    const int per = p.R_dev ? (((nrows + p.n_splits - 1) / p.n_splits + 15) / 16) * 16 : p.rows_per_split;
    const int r0 = split * per;
    const int r1 = min(r0 + per, nrows);
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

    // U groups of 16 rows per pass: every load of the pass is issued before
    // any of its arithmetic, so each lane keeps 4*U 16-byte loads in flight
    constexpr int U = 4;
    for (int base = r0; base < r1; base += 16 * U) {
        float kx[U][DPL], vx[U][DPL];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * 16 + wave * 4 + grp;
            valid[u] = r < r1;
            const float* ksrc = r < R ? p.mk + (size_t)r * kvw + g * HD : p.knew + g * HD;
            const float* vsrc = r < R ? p.mv + (size_t)r * kvw + g * HD : p.vnew + g * HD;
#pragma unroll
            for (int j = 0; j < NF4; ++j) {
                float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
                if (valid[u]) {
                    kk = *reinterpret_cast<const float4*>(ksrc + j * 64 + sub * 4);
                    vv = *reinterpret_cast<const float4*>(vsrc + j * 64 + sub * 4);
                }
                kx[u][4 * j] = kk.x; kx[u][4 * j + 1] = kk.y; kx[u][4 * j + 2] = kk.z; kx[u][4 * j + 3] = kk.w;
                vx[u][4 * j] = vv.x; vx[u][4 * j + 1] = vv.y; vx[u][4 * j + 2] = vv.z; vx[u][4 * j + 3] = vv.w;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * 16 + wave * 4 + grp;
            if (valid[u] && r == R) {   // append this token's row to the mirror
#pragma unroll
                for (int j = 0; j < NF4; ++j) {
                    const size_t at = (size_t)r * kvw + g * HD + j * 64 + sub * 4;
                    *reinterpret_cast<float4*>(p.mk + at) =
                        make_float4(kx[u][4 * j], kx[u][4 * j + 1], kx[u][4 * j + 2], kx[u][4 * j + 3]);
                    *reinterpret_cast<float4*>(p.mv + at) =
                        make_float4(vx[u][4 * j], vx[u][4 * j + 1], vx[u][4 * j + 2], vx[u][4 * j + 3]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float sc = 0.f;
#pragma unroll
                for (int i = 0; i < DPL; ++i) sc += q[h][i] * kx[u][i];
                sc += __shfl_xor(sc, 1, 64);
                sc += __shfl_xor(sc, 2, 64);
                sc += __shfl_xor(sc, 4, 64);
                sc += __shfl_xor(sc, 8, 64);
                sc *= scale;
                if (p.softcap > 0.f) sc = p.softcap * tanhf(sc / p.softcap);
                sc = valid[u] ? sc * LOG2E : -INFINITY;
                const float m_new = fmaxf(m[h], sc);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = exp2f(m[h] - m_use);
                const float pr = exp2f(sc - m_use);
                l[h] = l[h] * alpha + pr;
                m[h] = m_new;
#pragma unroll
                for (int i = 0; i < DPL; ++i) o[h][i] = o[h][i] * alpha + pr * vx[u][i];
            }
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

// Merge of the splits: block (query head, 32-dim slice) of 1024 threads =
// 32 dims x 32 groups of at most 8 splits (n_splits <= 256), so every load
// of the kernel is issued in one round; each group merges its splits, the
// groups meet in LDS in a fixed order; normalise, gate.
constexpr int COMBINE_GROUPS = 32;
static_assert(COMBINE_GROUPS * 8 >= DECODE_MAX_SPLITS, "eight splits per group at most");

template <int HD>
__global__ __launch_bounds__(COMBINE_GROUPS * 32) void decode_attn_combine_kernel(DecodeAttnArgs p) {
    __shared__ float sm_[COMBINE_GROUPS], sl_[COMBINE_GROUPS], so_[COMBINE_GROUPS][33];
    const int h = blockIdx.x, d0 = blockIdx.y * 32, tid = threadIdx.x;
    const int d = tid & 31, grp = tid >> 5;
    const int ns = p.n_splits;
    const size_t base = (size_t)h * ns;
    const int per = (ns + COMBINE_GROUPS - 1) / COMBINE_GROUPS;
    const int s0 = grp * per, s1 = min(ns, s0 + per);
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const bool ok = s0 + u < s1;
        mv[u] = ok ? p.part_m[base + s0 + u] : -INFINITY;
        lv[u] = ok ? p.part_l[base + s0 + u] : 0.f;
        ov[u] = ok ? p.part_o[(base + s0 + u) * HD + d0 + d] : 0.f;
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, mv[u]);
    const float mu = m == -INFINITY ? 0.f : m;
    float l = 0.f, O = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const float w = exp2f(mv[u] - mu);
        l += lv[u] * w;
        O += ov[u] * w;
    }
    if (d == 0) {
        sm_[grp] = m;
        sl_[grp] = l;
    }
    so_[grp][d] = O;
    __syncthreads();
    if (tid < 32) {
        float M = -INFINITY;
        for (int gq = 0; gq < COMBINE_GROUPS; ++gq) M = fmaxf(M, sm_[gq]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float L = 0.f, T = 0.f;
        for (int gq = 0; gq < COMBINE_GROUPS; ++gq) {
            const float w = exp2f(sm_[gq] - Mu);
            L += sl_[gq] * w;
            T += so_[gq][tid] * w;
        }
        float r = T / L;
        if (p.gate) r *= 1.0f / (1.0f + expf(-p.gate[(size_t)h * HD + d0 + tid]));
        p.o[(size_t)h * HD + d0 + tid] = r;
        // a replayed step: the head and the attention kernels, which read
        // the count, have finished (stream order), so it advances here
        if (p.R_dev && h == 0 && blockIdx.y == 0 && tid == 0) p.R_dev[0] = p.R_dev[0] + 1;
    }
}

// y = W x (fp16 weights times inv_scale, fp32 x) with fused epilogues; W in
// MFMA-fragment order.  x (RMS-normed first when norm_g is set) is staged
// in LDS and the eight waves of a workgroup split the 16-column blocks of K
// round-robin, one fully coalesced load per fragment block.
//  RH = 1: one workgroup per 32-row block; lane l accumulates row l % 32
//          over columns 16kb + 8*(l/32) .. +7 of each 1 KB block it loads.
//  RH = 2: two workgroups per 32-row block, one per 16-row half (for the
//          residual projections, whose 32-row blocks are fewer than the
//          CUs).  One load covers that half of two consecutive blocks: lane
//          l takes row 16h + l % 16, column half (l/16) % 2, block kb + l/32
//          (two 256-byte runs per block).
// A wave issues its loads NL at a time, all of a chunk back to back before
// any is used, and the first chunk before x is staged (x's own loads go out
// first: the counter completes loads in order).  Past the wave's last block a chunk repeats that
// block (a wave-uniform clamp instead of a branch, which would make the
// compiler wait for every load) and counts it with weight 0.
// Lanes of a row meet by shuffles, the waves in LDS, in a fixed order.
constexpr int GV_WAVES = 8;
constexpr int GV_MAXK = 15872;  // largest K the LDS stage holds (62 KB of dynamic LDS)

template <int EPI, int RH, int NL, int XV>
__global__ __launch_bounds__(GV_WAVES * 64) void gemv_kernel(GemvArgs p) {
    static_assert(RH == 1 || (RH == 2 && EPI == GV_RESID), "row halves only for the residual form");
    extern __shared__ float xs[];   // [K]
    __shared__ float red[GV_WAVES][32];
    __shared__ float wsum[GV_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = blockIdx.x / RH, hsel = blockIdx.x % RH;
    const int kblocks = p.K >> 4;
    // this wave's loads j = 0 .. nload-1: block kb0 + j * kstep (RH = 2: and
    // the next one, for the lanes with kofs = 1; kblocks is even there)
    const int kofs = RH == 1 ? 0 : lane >> 5;
    const f16* wb;
    const float* xl;
    int kb0, kstep;
    if constexpr (RH == 1) {
        wb = p.W + (size_t)nb * kblocks * 512 + lane * 8;
        xl = xs + 8 * (lane >> 5);
        kb0 = wave;
        kstep = GV_WAVES;
    } else {
        const int khalf = (lane >> 4) & 1;
        const int fl = (lane & 15) + 16 * hsel + 32 * khalf;      // lane within the 1 KB block
        wb = p.W + ((size_t)nb * kblocks + kofs) * 512 + fl * 8;
        xl = xs + kofs * 16 + 8 * khalf;
        kb0 = 2 * wave;
        kstep = 2 * GV_WAVES;
    }
    const int nload = kblocks > kb0 ? (kblocks - kb0 + kstep - 1) / kstep : 0;
    auto block_of = [&](int j) { return nload > 0 ? kb0 + min(j, nload - 1) * kstep : 0; };
    half8 w[NL];
    auto issue = [&](int c0) {
#pragma unroll
        for (int u = 0; u < NL; ++u) w[u] = *reinterpret_cast<const half8*>(wb + (size_t)block_of(c0 + u) * 512);
        __builtin_amdgcn_sched_barrier(0);   // keep the chunk's loads together, ahead of their use
    };
    float acc = 0.f;
    auto use = [&](int c0) {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const float* xv = xl + block_of(c0 + u) * 16;
            float d = 0.f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) d += (float)w[u][jj] * xv[jj];
            acc += (c0 + u < nload ? 1.0f : 0.0f) * d;
        }
    };

    // x first (XV float4 a thread, clamped in range), then the weights: the
    // counter completes loads in order, so x can be used while the weight
    // loads are still in flight
    const int k4 = p.K >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(p.x);
    float4 xr[XV], gr[XV];
#pragma unroll
    for (int v = 0; v < XV; ++v) xr[v] = x4[min(tid + v * GV_WAVES * 64, k4 - 1)];
    if (p.norm_g) {
#pragma unroll
        for (int v = 0; v < XV; ++v)
            gr[v] = reinterpret_cast<const float4*>(p.norm_g)[min(tid + v * GV_WAVES * 64, k4 - 1)];
    }
    issue(0);
    float r = 1.0f;
    if (p.norm_g) {
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < XV; ++v)
            if (tid + v * GV_WAVES * 64 < k4)
                ss += xr[v].x * xr[v].x + xr[v].y * xr[v].y + xr[v].z * xr[v].z + xr[v].w * xr[v].w;
        ss = wave_sum(ss);
        if (lane == 0) wsum[wave] = ss;
        __syncthreads();
        float t = 0.f;
#pragma unroll
        for (int v = 0; v < GV_WAVES; ++v) t += wsum[v];
        r = 1.0f / sqrtf(t / (float)p.K + p.eps);
    }
    float4* xs4 = reinterpret_cast<float4*>(xs);
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int i4 = tid + v * GV_WAVES * 64;
        if (i4 < k4) {
            float4 y = xr[v];
            if (p.norm_g)
                y = make_float4(y.x * r * gr[v].x, y.y * r * gr[v].y, y.z * r * gr[v].z,
                                y.w * r * gr[v].w);
            xs4[i4] = y;
        }
    }
    __syncthreads();
    use(0);
    for (int c0 = NL; c0 < nload; c0 += NL) {
        issue(c0);
        use(c0);
    }
    if constexpr (RH == 1) {
        acc += __shfl_xor(acc, 32, 64);
        if (lane < 32) red[wave][lane] = acc;
    } else {
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        if (lane < 16) red[wave][lane] = acc;
    }
    __syncthreads();
    constexpr int ROWS = 32 / RH;
    if (tid >= ROWS) return;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) y += red[w][tid];
    y *= *p.inv_scale;
    if constexpr (EPI == GV_SWIGLU) {
        // rows 32nb + t: t < 16 gate, t >= 16 up, of output 16nb + t % 16
        const float other = __shfl_xor(y, 16, 64);
        const float act = p.gelu ? 0.5f * y * (1.0f + erff(y * 0.7071067811865476f))
                                 : y / (1.0f + expf(-y));
        if (tid < 16) p.y[nb * 16 + tid] = act * other;
    } else {
        const int row = nb * 32 + hsel * 16 + tid;
        p.y[row] = p.r ? p.r[row] + y : y;
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
    return hipGetLastError();
}

template <int HD, int DPL>
hipError_t launch_rows_dpl(const DecodeAttnArgs& a, int G, hipStream_t s) {
    const dim3 grid(a.n_splits), block(ROWS_WAVES * 64);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_attn_rows_kernel<HD, DPL, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_attn_rows_kernel<HD, DPL, 2>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((decode_attn_rows_kernel<HD, DPL, 3>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_attn_rows_kernel<HD, DPL, 4>), grid, block, 0, s, a); break;
        case 8:
            if constexpr (8 * DPL <= 64) {
                hipLaunchKernelGGL((decode_attn_rows_kernel<HD, DPL, 8>), grid, block, 0, s, a);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int HD>
hipError_t launch_rows_hd(const DecodeAttnArgs& a, int G, hipStream_t s) {
    switch (a.hkv * HD) {
        case 256: return launch_rows_dpl<HD, 4>(a, G, s);
        case 512: return launch_rows_dpl<HD, 8>(a, G, s);
        case 1024: return launch_rows_dpl<HD, 16>(a, G, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_group_ok(int hq, int hkv, int hd) {
    if (hkv <= 0 || hq % hkv) return false;
    const int G = hq / hkv;
    return (hd == 64 || hd == 128) && (G == 1 || G == 2 || G == 3 || G == 4 || G == 8);
}

bool decode_rows_kernel_ok(int hq, int hkv, int hd) {
    const int w = hkv * hd, G = hq / hkv;
    return (w == 256 || w == 512 || (w == 1024 && G <= 4));
}

void decode_split_plan(int hq, int hkv, int hd, int rows_total, int* n_splits, int* rows_per_split) {
    if (decode_rows_kernel_ok(hq, hkv, hd)) {
        // interleaved rows: a split is any 1/n of them.  At 32K rows,
        // 176..200 workgroups of eight waves measured best; from about 208
        // the time rises by a tenth
        int splits = (rows_total + 63) / 64;
        splits = splits < 1 ? 1 : (splits > DECODE_ROWS_SPLITS ? DECODE_ROWS_SPLITS : splits);
        *n_splits = splits;
        *rows_per_split = (rows_total + splits - 1) / splits;
        return;
    }
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
    if (a.n_splits < 1 || a.n_splits > DECODE_MAX_SPLITS || a.hd % 32) return hipErrorInvalidValue;
    const bool rows = decode_rows_kernel_ok(a.hq, a.hkv, a.hd);
    hipError_t e;
    if (a.hd == 128) e = rows ? launch_rows_hd<128>(a, G, s) : launch_split_hd<128>(a, G, s);
    else if (a.hd == 64) e = rows ? launch_rows_hd<64>(a, G, s) : launch_split_hd<64>(a, G, s);
    else return hipErrorInvalidValue;
    if (e) return e;
    const dim3 grid(a.hq, a.hd / 32);
    if (a.hd == 128)
        hipLaunchKernelGGL(decode_attn_combine_kernel<128>, grid, dim3(COMBINE_GROUPS * 32), 0, s, a);
    else
        hipLaunchKernelGGL(decode_attn_combine_kernel<64>, grid, dim3(COMBINE_GROUPS * 32), 0, s, a);
    return hipGetLastError();
}

namespace {
// The single-token head of a layer: one block per q, k or v head of the
// stacked projection (gate heads are used as they are), one thread per
// channel.  Bias, then the per-head Q/K RMS norm, then RoPE at position
// p.pos ("frink-models 0.29.0 src/decoder/cuda_prefill.rs",
// cuda_prefill_layer: the extras and the RoPE description -- the same order
// as the prefill's QKV post-step); the rotation partner of a channel comes
// through LDS.  Angles in fp64, then cos/sin times the attention factor in
// fp32.
template <int HD>
__global__ __launch_bounds__(HD) void decode_head_kernel(DecodeHeadArgs p) {
    __shared__ float xs[HD];
    __shared__ float part[HD / 64];
    const int slot = blockIdx.x, e = threadIdx.x;
    const bool is_q = slot < p.hq, is_v = slot >= p.hq + p.hkv;
    const int col = slot * HD + e;
    float x = p.qkv[col];
    if (p.bias) x += p.bias[col];
    if (!is_v) {
        const float* gn = is_q ? p.q_norm : p.k_norm;
        if (gn) {
            const float ss = wave_sum(x * x);
            if ((e & 63) == 0) part[e >> 6] = ss;
            __syncthreads();
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < HD / 64; ++w) t += part[w];
            x = x * (1.0f / sqrtf(t / (float)HD + p.eps)) * gn[e];
        }
        if (p.rope_on) {
            xs[e] = x;
            __syncthreads();
            const int rd = p.rot_dim, half = rd / 2;
            if (e < rd) {
                int i, partner;
                bool first;
                if (p.rope_layout == DDL_ROPE_NEOX) {
                    first = e < half;
                    i = first ? e : e - half;
                    partner = first ? e + half : e - half;
                } else {
                    first = (e & 1) == 0;
                    i = e >> 1;
                    partner = e ^ 1;
                }
                double inv = pow(p.theta, -2.0 * (double)i / (double)rd);
                if (p.freq) inv /= (double)p.freq[i];
                const double ang = (double)(p.pos_dev ? *p.pos_dev : p.pos) * inv;
                const float c = (float)(p.mscale * cos(ang)), sn = (float)(p.mscale * sin(ang));
                const float xp = xs[partner];
                // pair (a, b) -> (a c - b s, a s + b c)
                x = first ? x * c - xp * sn : xp * sn + x * c;
            }
        }
    }
    if (is_q)
        p.q[col] = x;
    else if (!is_v)
        p.k_row[(slot - p.hq) * HD + e] = x;
    else
        p.v_row[(slot - p.hq - p.hkv) * HD + e] = x;
}
}  // namespace

hipError_t launch_decode_head(const DecodeHeadArgs& a, hipStream_t s) {
    if (a.rope_on && (a.rot_dim < 2 || a.rot_dim % 2 || a.rot_dim > a.hd)) return hipErrorInvalidValue;
    const dim3 grid(a.hq + 2 * a.hkv);
    if (a.hd == 128)
        hipLaunchKernelGGL(decode_head_kernel<128>, grid, dim3(128), 0, s, a);
    else if (a.hd == 64)
        hipLaunchKernelGGL(decode_head_kernel<64>, grid, dim3(64), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

namespace {
__global__ void set_int_kernel(int* dst, int value) {
    if (threadIdx.x == 0) dst[0] = value;
}
}  // namespace

hipError_t launch_set_int(int* dst, int value, hipStream_t s) {
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(64), 0, s, dst, value);
    return hipGetLastError();
}

bool gemv_shape_ok(int K) { return K > 0 && K % 16 == 0 && K <= GV_MAXK; }
static_assert(GV_MAXK <= 8 * 4 * GV_WAVES * 64, "x staging covers the largest K");

namespace {
// Loads a wave keeps in flight per chunk: the smallest of 8, 16, 24, 32 that
// covers the wave's blocks, else 32 (more chunks).
// ... and float4 of x a thread: XV * 2048 >= K.
template <int EPI, int RH, int NL>
hipError_t launch_gemv_xv(const GemvArgs& a, int grid, size_t lds, hipStream_t s) {
    const dim3 block(GV_WAVES * 64);
    const int xv = (a.K + 4 * GV_WAVES * 64 - 1) / (4 * GV_WAVES * 64);
    if (xv <= 1) hipLaunchKernelGGL((gemv_kernel<EPI, RH, NL, 1>), dim3(grid), block, lds, s, a);
    else if (xv <= 2) hipLaunchKernelGGL((gemv_kernel<EPI, RH, NL, 2>), dim3(grid), block, lds, s, a);
    else if (xv <= 4) hipLaunchKernelGGL((gemv_kernel<EPI, RH, NL, 4>), dim3(grid), block, lds, s, a);
    else hipLaunchKernelGGL((gemv_kernel<EPI, RH, NL, 8>), dim3(grid), block, lds, s, a);
    return hipGetLastError();
}

// Loads a wave keeps in flight per chunk: 8 (4 when a wave has no more
// blocks).  Measured at the decode shapes (hidden 4096, FFN 14336): chunks
// of 8 took gate/up from 51.4 to 45.5 us and down from 27.9 to 25.3 us
// against chunks of 32 -- smaller chunks leave registers for four
// workgroups a CU, whose round trips then overlap; 4 and 6 were no better.
template <int EPI, int RH>
hipError_t launch_gemv_nl(const GemvArgs& a, int grid, size_t lds, hipStream_t s) {
    const int kblocks = a.K >> 4, kstep = RH == 1 ? GV_WAVES : 2 * GV_WAVES;
    const int nload = (kblocks + kstep - 1) / kstep;   // wave 0's, the most of any wave
    if (nload <= 4) return launch_gemv_xv<EPI, RH, 4>(a, grid, lds, s);
    return launch_gemv_xv<EPI, RH, 8>(a, grid, lds, s);
}
}  // namespace

hipError_t launch_gemv(const GemvArgs& a, int epi, hipStream_t s) {
    if (!gemv_shape_ok(a.K)) return hipErrorInvalidValue;
    // GV_SWIGLU: N outputs from 2N packed rows; GV_RESID: N rows
    const int rows = epi == GV_SWIGLU ? 2 * a.N : a.N;
    if (rows % 32) return hipErrorInvalidValue;
    const size_t lds = a.K * sizeof(float);
    if (epi == GV_SWIGLU) return launch_gemv_nl<GV_SWIGLU, 1>(a, rows / 32, lds, s);
    // under two rounds of row blocks on 256 CUs: 16-row halves (their loads
    // take block pairs, so K is a multiple of 32 there)
    if (rows / 32 < 512 && a.K % 32 == 0) return launch_gemv_nl<GV_RESID, 2>(a, rows / 16, lds, s);
    return launch_gemv_nl<GV_RESID, 1>(a, rows / 32, lds, s);
}
