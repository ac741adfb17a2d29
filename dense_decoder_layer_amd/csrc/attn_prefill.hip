// Causal GQA attention of B new tokens over S cached rows plus the new rows
// ("frink-models 0.29.0 src/decoder/cuda_prefill.rs", cuda_prefill_layer:
// the attention parameters -- head counts, 1/sqrt(head_dim) scale, optional
// logit softcap, the cache prefix and start_pos; the output gate is the one
// of "frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_layer).
//
// Flash-style: a 256-thread workgroup takes 64 queries of one query head
// (16 per wave) and walks the keys in tiles of 32, keeping a running max and
// sum per query (online softmax, base-2 exponentials).  K and V tiles are
// read as fp32 rows -- from the caller's prefix for key j < S, from this
// call's K/V rows after -- rounded to fp16 into LDS, K row-major and V
// transposed.  Both products run on v_mfma_f32_16x16x32_f16 in transposed
// form, S^T = K Q^T and O^T += V^T P^T, so every lane holds the scores and
// the output columns of exactly one query: the softmax statistics of a query
// live in the four lanes l, l^16, l^32, l^48 and the rescale factor is one
// scalar per lane.  Tiles wholly above a wave's last query are skipped;
// masked scores are -inf and contribute exact zeros, so a token's outputs do
// not depend on the values of later tokens.
#include "common.h"
#include "internal.h"

namespace {

constexpr int KT = 32;   // keys per tile

template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnPrefillArgs p) {
    constexpr int HC = HD / 8;          // 16-byte chunks per K row in LDS
    constexpr int VT_LD = KT + 4;       // V^T row stride (halves), keeps 8-byte reads aligned
    constexpr int KS = HD / 32;         // MFMA k-steps over the head dimension
    constexpr int HB = HD / 16;         // 16-row blocks of O^T
    constexpr int LOADS = KT * HD / 4 / 256;
    __shared__ half8 Ks[KT * HC];
    __shared__ f16 Vt[HD * VT_LD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
    const int qt = gridDim.x - 1 - blockIdx.x;      // longest rows first
    const int h = blockIdx.y;
    const int g = h / (p.hq / p.hkv);
    const int kvw = p.hkv * HD;
    const int q0 = qt * 64;
    const int qrow = q0 + wave * 16 + (lane & 15);  // this lane's query token
    const int qpos = p.S + qrow;
    const int nkeys = p.S + p.B;
    const int kv_end = min(p.S + q0 + 64, nkeys);
    const int wave_last = p.S + q0 + wave * 16 + 15;
    const float LOG2E = 1.4426950408889634f;
    const float scale = 1.0f / sqrtf((float)HD);

    half8 qf[KS];
    const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = qrow < p.B ? *reinterpret_cast<const half8*>(
                                  p.q16 + (size_t)qrow * p.hq * HD + h * HD + ks * 32 + 8 * grp)
                            : zero8;

    floatx4 o[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    for (int k0 = 0; k0 < kv_end; k0 += KT) {
        float4 kr[LOADS], vr[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int idx = i * 256 + tid, key = idx / (HD / 4), c4 = idx % (HD / 4);
            const int j = k0 + key;
            const float* ks = nullptr;
            const float* vs = nullptr;
            if (j < p.S) {
                ks = p.pk + (size_t)j * kvw;
                vs = p.pv + (size_t)j * kvw;
            } else if (j < nkeys) {
                ks = p.nk + (size_t)(j - p.S) * kvw;
                vs = p.nv + (size_t)(j - p.S) * kvw;
            }
            kr[i] = ks ? *reinterpret_cast<const float4*>(ks + g * HD + c4 * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
            vr[i] = vs ? *reinterpret_cast<const float4*>(vs + g * HD + c4 * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();   // the previous tile's readers are done
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int idx = i * 256 + tid, key = idx / (HD / 4), c4 = idx % (HD / 4);
            half4* kd = reinterpret_cast<half4*>(&Ks[key * HC + ((c4 >> 1) ^ (key & 7))]) + (c4 & 1);
            *kd = half4{(f16)kr[i].x, (f16)kr[i].y, (f16)kr[i].z, (f16)kr[i].w};
            f16* vd = &Vt[(c4 * 4) * VT_LD + key];
            vd[0] = (f16)vr[i].x;
            vd[VT_LD] = (f16)vr[i].y;
            vd[2 * VT_LD] = (f16)vr[i].z;
            vd[3 * VT_LD] = (f16)vr[i].w;
        }
        __syncthreads();
        if (k0 > wave_last) continue;   // wave-uniform: every key of the tile is masked

        floatx4 st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            st[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int key = kb * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = ks * 4 + grp;
                st[kb] = mfma16x16x32(Ks[key * HC + (c ^ (key & 7))], qf[ks], st[kb]);
            }
        }
        // lane holds S^T[key = kb*16 + 4*grp + e][query = lane & 15]
        float s[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kpos = k0 + kb * 16 + 4 * grp + e;
                float v = st[kb][e] * scale;
                if (p.softcap > 0.f) v = p.softcap * tanhf(v / p.softcap);
                v *= LOG2E;
                if (kpos > qpos || kpos >= nkeys) v = -INFINITY;
                s[kb * 4 + e] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m - m_use);
        float psum = 0.f;
        half8 pf;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float pv = exp2f(s[i] - m_use);
            psum += pv;
            pf[i] = (f16)pv;
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l = l * alpha + psum;
        m = m_new;
        // P^T operand: element i of lane group grp is key (i < 4 ? 4*grp + i
        // : 16 + 4*grp + i - 4); the V^T operand uses the same key order.
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const f16* vrow = &Vt[(hb * 16 + (lane & 15)) * VT_LD];
            const half4 lo = *reinterpret_cast<const half4*>(vrow + 4 * grp);
            const half4 hi = *reinterpret_cast<const half4*>(vrow + 16 + 4 * grp);
            const half8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[hb] = o[hb] * alpha;
            o[hb] = mfma16x16x32(vf, pf, o[hb]);
        }
    }

    if (qrow >= p.B) return;
    const float inv_l = 1.0f / l;
    f16* dst = p.o16 + (size_t)qrow * p.hq * HD + h * HD;
    const float* gt = p.gate ? p.gate + (size_t)qrow * p.gate_ld + h * HD : nullptr;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int d0 = hb * 16 + 4 * grp;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = o[hb][e] * inv_l;
            if (gt) r[e] *= 1.0f / (1.0f + expf(-gt[d0 + e]));
        }
        *reinterpret_cast<half4*>(dst + d0) = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
    }
}

}  // namespace

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
    const dim3 grid((a.B + 63) / 64, a.hq);
    if (a.hd == 128)
        hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), 0, s, a);
    else if (a.hd == 64)
        hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
