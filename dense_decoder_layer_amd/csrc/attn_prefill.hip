// Causal GQA attention of B new tokens over S cached rows plus the new rows
// ("frink-models 0.29.0 src/decoder/cuda_prefill.rs", cuda_prefill_layer:
// the attention parameters -- head counts, 1/sqrt(head_dim) scale, optional
// logit softcap, the cache prefix and start_pos; the output gate is the one
// of "frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_layer).
//
// Flash-style, one wave per workgroup: the wave takes 32 queries of one
// query head and walks the keys of its KV head in tiles of 32 with a running
// max and sum per query (online softmax, base-2 exponentials).  Keys and
// values were staged once per layer as fp16: K16 [kv head][key][hd] and
// Vt16 [kv head][hd][key].  Tiles move global -> LDS by DMA
// (global_load_lds_dwordx4) through a 3-stage ring, so the next tiles are in
// flight while one is used; a single wave needs no barriers.  Both products
// run on v_mfma_f32_32x32x16_f16 in transposed form: S^T = K Q^T gives every
// lane 16 scores of one query (its partner lane l^32 holds the other 16), and
// those probabilities are directly the B operand of O^T += V^T P^T; the
// rescale factor of a query is one scalar per lane.  Tiles wholly above the
// wave's last query are not visited; masked scores are -inf and contribute
// exact zeros, so a token's outputs do not depend on later tokens' values.
#include "common.h"
#include "internal.h"

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int KT = 32;    // keys per tile
constexpr int NS = 3;     // LDS ring stages

__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
#endif
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int HD>
__global__ __launch_bounds__(64) void attn_prefill_kernel(AttnPrefillArgs p) {
    constexpr int KCH = HD / 8;                  // 16-byte chunks per K row
    constexpr int K_BYTES = KT * HD * 2;         // K tile [32 keys][HD]
    constexpr int V_BYTES = HD * KT * 2;         // V^T tile [HD][32 keys]
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int K_INSTR = K_BYTES / 1024, V_INSTR = V_BYTES / 1024;
    constexpr int PER = K_INSTR + V_INSTR;       // DMA instructions per tile
    constexpr int KS = HD / 16;                  // k-steps of S^T over the head dim
    constexpr int HB = HD / 32;                  // 32-row blocks of O^T
    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

    const int lane = threadIdx.x, g2 = lane >> 5, ql = lane & 31;
    const int qt = gridDim.x - 1 - blockIdx.x;     // longest rows first
    const int h = blockIdx.y;
    const int g = h / (p.hq / p.hkv);
    const int q0 = qt * 32;
    const int qrow = q0 + ql;                      // this lane's query token
    const int qpos = p.S + qrow;
    const int nkeys = p.S + p.B;
    const int kv_end = min(p.S + q0 + 32, nkeys);  // keys the wave can see
    const int ntiles = (kv_end + KT - 1) / KT;
    const float LOG2E = 1.4426950408889634f;
    const float scale = 1.0f / sqrtf((float)HD);

    // Per-lane DMA sources.  K: instruction j covers rows 4j..4j+3 (HD=128)
    // or 8j..8j+7 (HD=64); lane chunk (l % KCH) ^ (row % 8) keeps the K rows
    // XOR-swizzled.  V^T: instruction j covers hd rows 16j..16j+15, four
    // 16-byte chunks (8 keys) each; chunk c of row r sits at c ^ ((r/2) % 4).
    const f16* kbase = p.k16 + (size_t)g * p.tcap * HD;
    const f16* vbase = p.vt16 + (size_t)g * HD * p.tcap;
    const uint32_t sm = (uint32_t)(uintptr_t)smem;
    size_t koff[K_INSTR], voff[V_INSTR];
#pragma unroll
    for (int j = 0; j < K_INSTR; ++j) {
        const int r = j * (64 / KCH) + lane / KCH;
        koff[j] = (size_t)r * HD + (((lane % KCH) ^ (r & 7)) * 8);
    }
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
        const int r = j * 16 + (lane >> 2);
        voff[j] = (size_t)r * p.tcap + (((lane & 3) ^ ((r >> 1) & 3)) * 8);
    }
    auto issue = [&](int tile, int slot) {
        const uint32_t sb = sm + slot * STAGE;
        const size_t k0 = (size_t)tile * KT;
#pragma unroll
        for (int j = 0; j < K_INSTR; ++j) dma16(kbase + k0 * HD + koff[j], sb + j * 1024);
#pragma unroll
        for (int j = 0; j < V_INSTR; ++j) dma16(vbase + k0 + voff[j], sb + K_BYTES + j * 1024);
    };

    // Q^T operand: lane holds Q[qrow][ks*16 + 8*g2 .. +7]
    half8 qf[KS];
    const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = qrow < p.B ? *reinterpret_cast<const half8*>(p.q16 + (size_t)qrow * p.hq * HD +
                                                                h * HD + ks * 16 + 8 * g2)
                            : zero8;

    floatx16 o[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    issue(0, 0);
    issue(min(1, ntiles - 1), 1);
    for (int t = 0; t < ntiles; ++t) {
        const int slot = t % NS;
        // the tile after next goes into the slot used two tiles ago (or the
        // last tile again, into that already-used slot: same wait count on
        // every path)
        issue(min(t + 2, ntiles - 1), (t + 2) % NS);
        wait_vmcnt<2 * PER>();            // tile t has landed in LDS
        asm volatile("" ::: "memory");
        const half8* Ks = reinterpret_cast<const half8*>(smem + slot * STAGE);
        const f16* Vs = reinterpret_cast<const f16*>(smem + slot * STAGE + K_BYTES);
        const int k0 = t * KT;

        // S^T[key][query]: A = K rows, B = Q^T
        floatx16 st;
#pragma unroll
        for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks * 2 + g2;
            st = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ks[ql * KCH + (c ^ (ql & 7))], qf[ks], st,
                                                        0, 0, 0);
        }
        // lane holds key k0 + 8*(e/4) + 4*g2 + e%4 of query qrow
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int kpos = k0 + 8 * (e >> 2) + 4 * g2 + (e & 3);
            float v = st[e] * scale;
            if (p.softcap > 0.f) v = p.softcap * tanhf(v / p.softcap);
            v *= LOG2E;
            if (kpos > qpos || kpos >= nkeys) v = -INFINITY;
            st[e] = v;
            tmax = fmaxf(tmax, v);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m - m_use);
        float psum = 0.f;
        half8 pf[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float pv = exp2f(st[e] - m_use);
            psum += pv;
            pf[e >> 3][e & 7] = (f16)pv;
        }
        psum += __shfl_xor(psum, 32, 64);
        l = l * alpha + psum;
        m = m_new;
        // O^T[hd][query] += V^T P^T.  P^T operand kh: element j of lane group
        // g2 is key kh*16 + (j < 4 ? 4*g2 + j : 8 + 4*g2 + j - 4), which is
        // exactly score e = 8*kh + j above; the V^T operand reads the same keys.
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int r = hb * 32 + ql;
            const f16* vrow = Vs + r * KT;
            const int sw = (r >> 1) & 3;
            o[hb] = o[hb] * alpha;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const half4 lo = *reinterpret_cast<const half4*>(vrow + (((2 * kh) ^ sw) * 8) + 4 * g2);
                const half4 hi = *reinterpret_cast<const half4*>(vrow + (((2 * kh + 1) ^ sw) * 8) + 4 * g2);
                const half8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kh], o[hb], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();

    if (qrow >= p.B) return;
    const float inv_l = 1.0f / l;
    f16* dst = p.o16 + (size_t)qrow * p.hq * HD + h * HD;
    const float* gt = p.gate ? p.gate + (size_t)qrow * p.gate_ld + h * HD : nullptr;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = hb * 32 + 8 * q4 + 4 * g2;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r[e] = o[hb][q4 * 4 + e] * inv_l;
                if (gt) r[e] *= 1.0f / (1.0f + expf(-gt[d0 + e]));
            }
            *reinterpret_cast<half4*>(dst + d0) = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
        }
}

}  // namespace

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
    if (a.tcap % 32 || a.tcap < a.S + a.B) return hipErrorInvalidValue;
    const dim3 grid((a.B + 31) / 32, a.hq);
    if (a.hd == 128)
        hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(64), 0, s, a);
    else if (a.hd == 64)
        hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(64), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
