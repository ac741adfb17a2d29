// Causal GQA attention of B new tokens over S cached rows plus the new rows
// ("frink-models 0.29.0 src/decoder/cuda_prefill.rs", cuda_prefill_layer:
// the attention parameters -- head counts, 1/sqrt(head_dim) scale, optional
// logit softcap, the cache prefix and start_pos; the output gate is the one
// of "frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_layer).
//
// Flash-style: a workgroup takes 32 queries of one query head; its NW waves
// split the key tiles of the KV head round-robin (wave w takes tiles w,
// w+NW, ...), each with a running max and sum per query (online softmax,
// base-2 exponentials), and merge their partial states through LDS in a
// fixed order at the end.
//
// Keys and values were staged once per layer as fp16: K16 [kv head][key][hd]
// and Vt16 [kv head][hd][key].  Tiles move global -> LDS by DMA
// (global_load_lds_dwordx4) through a small ring per wave, so the next tile
// is in flight while one is used; each wave owns its ring, so the loop needs
// no barriers.  Both products run on v_mfma_f32_32x32x16_f16 in transposed
// form: S^T = K Q^T gives every lane 16 scores of one query (its partner lane
// l^32 holds the other 16), and those probabilities are directly the B
// operand of O^T += V^T P^T; the rescale factor of a query is one scalar per
// lane.  The running max is raised only when a tile exceeds it by a margin,
// so rescaling O is rare.  Tiles wholly above the wave's last query are not
// visited; only tiles on the diagonal or past the last key apply the causal
// mask, and masked scores are -inf and contribute exact zeros, so a token's
// outputs do not depend on later tokens' values.  With a sliding window W
// (cuda_prefill_layer's `window`) the token at position p sees keys
// p-W+1 .. p: tiles wholly below the block's first window are not visited and
// the tiles across its lower edge are masked too.
#include "common.h"
#include "internal.h"

#include <atomic>

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int KT = 32;    // keys per tile
constexpr int RING = 2;   // LDS ring stages per wave (tiles in flight + 1)

// Waves per workgroup.  Two waves with two-stage rings (64 KB of LDS at
// head_dim 128) let two workgroups share a CU; measured best against one
// wave with three stages and three or four waves with two or three stages.
template <int HD>
constexpr int attn_waves() { return 2; }
template <int HD, int NW, int NSTAGE = RING>
constexpr int attn_lds_bytes() { return NW * NSTAGE * (2 * KT * HD * 2); }

// log2-domain headroom of the running max: it is raised only when a tile's
// max exceeds it by more than this, so the rescale of O is rare; P stays
// <= 2^8, exact enough in fp16 (11-bit significand at any magnitude)
constexpr float MAX_SLACK = 8.0f;

// tanh from one exp2: sign(x) (1 - t) / (1 + t), t = 2^(-2|x| log2 e)
__device__ __forceinline__ float tanh_exp2(float x) {
    const float t = __builtin_amdgcn_exp2f(-2.8853900817779268f * fabsf(x));
    return copysignf((1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t), x);
}

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

template <int HD, bool CAP, int NW, int NS = RING>
__global__ __launch_bounds__(NW * 64) void attn_prefill_kernel(AttnPrefillArgs p) {
    constexpr int KCH = HD / 8;                  // 16-byte chunks per K row
    constexpr int K_BYTES = KT * HD * 2;         // K tile [32 keys][HD]
    constexpr int V_BYTES = HD * KT * 2;         // V^T tile [HD][32 keys]
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int K_INSTR = K_BYTES / 1024, V_INSTR = V_BYTES / 1024;
    constexpr int PER = K_INSTR + V_INSTR;       // DMA instructions per tile
    constexpr int KS = HD / 16;                  // k-steps of S^T over the head dim
    constexpr int HB = HD / 32;                  // 32-row blocks of O^T
    extern __shared__ __attribute__((aligned(1024))) char smem_all[];
    static_assert(NW == 1 || (NW - 1) * (HD * 32 + 64) * 4 <= NW * NS * STAGE, "merge fits the rings");

    const int lane = threadIdx.x & 63, g2 = lane >> 5, ql = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS addresses stay scalar
    char* smem = smem_all + wave * NS * STAGE;
    // Grid (hq, query blocks): the longest rows are dispatched first, and
    // consecutive workgroups (which the dispatcher deals out to the XCDs in
    // turn) are different heads of one query block, so every XCD gets an
    // equal share of the long rows.
    const int qt = gridDim.y - 1 - blockIdx.y;
    const int h = blockIdx.x;
    const int g = h / (p.hq / p.hkv);
    const int q0 = qt * 32;
    const int qrow = q0 + ql;                      // this lane's query token
    const int qpos = p.S + qrow;
    const int nkeys = p.S + p.B;
    const int kv_end = min(p.S + q0 + 32, nkeys);  // keys the wave can see
    const int ntiles = (kv_end + KT - 1) / KT;
    // first key of the block's first query's window; tiles before its tile
    // hold no visible key for any query of the block
    const int win_lo = p.window > 0 ? max(p.S + q0 - p.window + 1, 0) : 0;
    const int t0 = win_lo / KT;
    const int my_n = ntiles - t0 > wave ? (ntiles - t0 - wave + NW - 1) / NW : 0;   // this wave's tiles
    auto tile_of = [&](int i) { return t0 + wave + i * NW; };
    // keys below this bound are outside the last query's window: a tile
    // starting below it may hold keys outside some query's window
    const int win_edge = p.window > 0 ? p.S + q0 + 32 - p.window : -1;
    const float LOG2E = 1.4426950408889634f;
    const float scale = 1.0f / sqrtf((float)HD);
    // exp2-domain logit: c * s, or capl * tanh(s * ic) with a softcap
    const float c = scale * LOG2E;
    const float capl = p.softcap * LOG2E, ic = CAP ? scale / p.softcap : 0.f;

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

    if (my_n > 0) {
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) issue(tile_of(min(j, my_n - 1)), j);
    }
    for (int i = 0; i < my_n; ++i) {
        const int slot = i % NS;
        // tile i+NS-1 goes into the slot used one tile ago (or the wave's
        // last tile again, into an already-used slot: the same wait count on
        // every path)
        issue(tile_of(min(i + NS - 1, my_n - 1)), (i + NS - 1) % NS);
        wait_vmcnt<(NS - 1) * PER>();     // tile i has landed in LDS
        asm volatile("" ::: "memory");
        const half8* Ks = reinterpret_cast<const half8*>(smem + slot * STAGE);
        const f16* Vs = reinterpret_cast<const f16*>(smem + slot * STAGE + K_BYTES);
        const int k0 = tile_of(i) * KT;

        // S^T[key][query]: A = K rows, B = Q^T; two independent chains
        floatx16 st0, st1;
#pragma unroll
        for (int e = 0; e < 16; ++e) st0[e] = st1[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            const int c0 = ks * 2 + g2, c1 = c0 + 2;
            st0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ks[ql * KCH + (c0 ^ (ql & 7))], qf[ks], st0, 0, 0, 0);
            st1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ks[ql * KCH + (c1 ^ (ql & 7))], qf[ks + 1], st1, 0, 0, 0);
        }
        // lane holds key k0 + 8*(e/4) + 4*g2 + e%4 of query qrow.  Without a
        // softcap the scores stay raw (the exp2-domain scale c > 0 keeps
        // their order) and c is folded into the exponent's fma below.
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float r = st0[e] + st1[e];
            sv[e] = CAP ? capl * tanh_exp2(r * ic) : r;
        }
        // only a tile that reaches past the block's first query or past the
        // last key needs the mask (a wave-uniform test)
        if (k0 + KT - 1 > p.S + q0 || k0 + KT > nkeys || k0 < win_edge) {
            const int klo = p.window > 0 ? qpos - p.window : -1;   // keys <= klo are outside the window
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int kpos = k0 + 8 * (e >> 2) + 4 * g2 + (e & 3);
                sv[e] = ((kpos <= qpos) & (kpos < nkeys) & (kpos > klo)) ? sv[e] : -INFINITY;
            }
        }
        float tmax = sv[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sv[e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        if constexpr (!CAP) tmax *= c;
        // raise the running max (and rescale l and O) only past the slack;
        // the branch is uniform over the wave
        const bool grow = tmax > m + MAX_SLACK;
        if (__ballot(grow)) {
            // lanes that keep their max scale by 1; from -inf the factor is 0
            const float alpha = grow ? __builtin_amdgcn_exp2f(m - tmax) : 1.0f;
            l *= alpha;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) o[hb] = o[hb] * alpha;
            if (grow) m = tmax;
        }
        const float m_use = m == -INFINITY ? 0.f : m;                 // every key so far masked
        float psum = 0.f;
        half8 pf[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float pv = __builtin_amdgcn_exp2f(CAP ? sv[e] - m_use : fmaf(sv[e], c, -m_use));
            psum += pv;
            pf[e >> 3][e & 7] = (f16)pv;
        }
        psum += __shfl_xor(psum, 32, 64);
        l += psum;
        // O^T[hd][query] += V^T P^T.  P^T operand kh: element j of lane group
        // g2 is key kh*16 + (j < 4 ? 4*g2 + j : 8 + 4*g2 + j - 4), which is
        // exactly score e = 8*kh + j above; the V^T operand reads the same keys.
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int r = hb * 32 + ql;
            const f16* vrow = Vs + r * KT;
            const int sw = (r >> 1) & 3;
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

    // merge: waves 1..NW-1 leave (m, l, O^T) in LDS, wave 0 folds them in
    // order.  Every wave's DMA has landed, so the rings can be reused.
    __syncthreads();
    float* mbuf = reinterpret_cast<float*>(smem_all);                 // [NW-1][32]
    float* lbuf = mbuf + (NW - 1) * 32;                               // [NW-1][32]
    float* obuf = lbuf + (NW - 1) * 32;                               // [NW-1][HD][32]
    if (wave > 0) {
        if (g2 == 0) {
            mbuf[(wave - 1) * 32 + ql] = m;
            lbuf[(wave - 1) * 32 + ql] = l;
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = hb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
                obuf[((size_t)(wave - 1) * HD + r) * 32 + ql] = o[hb][e];
            }
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 1; w < NW; ++w) {
        const float mo = mbuf[(w - 1) * 32 + ql], lo = lbuf[(w - 1) * 32 + ql];
        // finite: the tile holding a query's own key is visited by one of
        // the waves; a wave that saw no visible key has m = -inf, l = 0, O = 0
        const float mn = fmaxf(m, mo);
        const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float b = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        l = l * a + lo * b;
        m = mn;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = hb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
                o[hb][e] = o[hb][e] * a + obuf[((size_t)(w - 1) * HD + r) * 32 + ql] * b;
            }
    }

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

namespace {
template <int HD, bool CAP>
hipError_t launch_hd(const AttnPrefillArgs& a, hipStream_t s) {
    constexpr int NW = attn_waves<HD>();
    constexpr int lds = attn_lds_bytes<HD, NW, RING>();
    // the rings may take more than the default 64 KB of dynamic LDS; the
    // attribute is set once per device (idempotent if two threads race)
    static std::atomic<bool> set_on[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !set_on[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefill_kernel<HD, CAP, NW>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) set_on[dev].store(true, std::memory_order_release);
    }
    const dim3 grid(a.hq, (a.B + 31) / 32);
    hipLaunchKernelGGL((attn_prefill_kernel<HD, CAP, NW>), grid, dim3(NW * 64), lds, s, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
    if (a.tcap % 32 || a.tcap < a.S + a.B || a.window < 0) return hipErrorInvalidValue;
    const bool cap = a.softcap > 0.f;
    if (a.hd == 128) return cap ? launch_hd<128, true>(a, s) : launch_hd<128, false>(a, s);
    if (a.hd == 64) return cap ? launch_hd<64, true>(a, s) : launch_hd<64, false>(a, s);
    return hipErrorInvalidValue;
}
