// Causal GQA attention of B new tokens over S cached rows plus the new rows
// ("frink-models 0.29.0 src/decoder/cuda_prefill.rs", cuda_prefill_layer:
// the attention parameters -- head counts, 1/sqrt(head_dim) scale, optional
// logit softcap, the cache prefix and start_pos; the output gate is the one
// of "frink-models 0.38.0 src/decoder/device_attention.rs",
// device_attention_layer).
//
// Flash-style, one workgroup per (G query heads, block of 32 queries): one
// head, or G <= 6 heads of one KV head's group (the whole group or an equal
// part of it), which then share every key/value tile: a tile is staged into
// LDS once and read by the G waves of one head each.  The key
// tiles are split round-robin over NKS groups of G waves (group s takes tiles
// s, s+NKS, ...), each with a running max and sum per query (online
// softmax, base-2 exponentials); the groups merge their partial states
// through LDS in a fixed order at the end.
//
// Keys and values were staged once per layer as fp16: K16 [kv head][key][hd]
// and Vt16 [kv head][hd][key], the keys of each 16-key group ordered so that
// a lane's V^T operand is one 16-byte LDS read.  Each key split owns a two-stage LDS ring.
// With one head per workgroup a wave runs through its own tiles with no
// barrier, the next tile's DMA (global_load_lds_dwordx4) in flight while one
// is used.  With G heads the split's G waves share each tile's DMA, and the
// workgroup steps through the tiles in lockstep with one barrier per tile,
// after which the next tile's DMA goes into the slot the previous one left.  Both products run on v_mfma_f32_32x32x16_f16 in transposed
// form: S^T = K Q^T gives every lane 16 scores of one query (its partner lane
// l^32 holds the other 16), and those probabilities are directly the B
// operand of O^T += V^T P^T; the rescale factor of a query is one scalar per
// lane.  The running max is raised only when a tile exceeds it by a margin,
// so rescaling O is rare.  Tiles wholly above the block's last query are not
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

// log2-domain headroom of the running max: it is raised only when a tile's
// max exceeds it by more than this, so the rescale of O is rare; P stays
// <= 2^8, exact enough in fp16 (11-bit significand at any magnitude)
constexpr float MAX_SLACK = 8.0f;

template <int HD>
constexpr int stage_bytes() { return 2 * KT * HD * 2; }   // K tile + V^T tile
// one partial state (O^T [HD][32] plus m and l of 32 queries) in the merge
template <int HD>
constexpr int state_floats() { return HD * 32 + 64; }
constexpr int NS = 2;     // LDS ring stages per key split

template <int HD, int G, int NKS>
constexpr int attn_lds_bytes() {
    constexpr int ring = NKS * NS * stage_bytes<HD>();
    constexpr int merge = (NKS - 1) * G * state_floats<HD>() * 4;
    return ring > merge ? ring : merge;
}

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

template <int HD, bool CAP, int G, int NKS>
__global__ __launch_bounds__(G * NKS * 64) void attn_prefill_kernel(AttnPrefillArgs p) {
    constexpr int KCH = HD / 8;                  // 16-byte chunks per K row
    constexpr int K_BYTES = KT * HD * 2;         // K tile [32 keys][HD]
    constexpr int STAGE = stage_bytes<HD>();     // K tile, then V^T tile [HD][32 keys]
    constexpr int K_INSTR = K_BYTES / 1024;      // 1 KB DMA instructions of the K tile
    constexpr int NDMA = STAGE / 1024;           // ... of the whole tile
    constexpr int PER = (NDMA + G - 1) / G;      // per wave (a few waves repeat one)
    constexpr int KS = HD / 16;                  // k-steps of S^T over the head dim
    constexpr int HB = HD / 32;                  // 32-row blocks of O^T
    static_assert(NKS >= 1 && NKS <= 4, "key splits: 1 to 4");
    static_assert(G * NKS <= 12, "at most 12 waves (168 VGPRs each)");
    static_assert(attn_lds_bytes<HD, G, NKS>() <= 160 * 1024, "LDS");
    extern __shared__ __attribute__((aligned(1024))) char smem_all[];

    const int lane = threadIdx.x & 63, g2 = lane >> 5, ql = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS addresses stay scalar
    const int split = wave / G, j = wave % G;     // key split, query head within the group
    char* ring = smem_all + split * NS * STAGE;
    // Grid (query-head groups, query blocks): the longest rows are
    // dispatched first, and consecutive workgroups (which the dispatcher
    // deals out to the XCDs in turn) are different heads of one query block,
    // so every XCD gets an equal share of the long rows.
    const int qt = gridDim.y - 1 - blockIdx.y;
    // blockIdx.x = KV head * (parts of its group) + part: the workgroup's
    // first query head is blockIdx.x * G
    const int h = blockIdx.x * G + j;
    const int g = h / (p.hq / p.hkv);
    const int q0 = qt * 32;
    const int qrow = q0 + ql;                      // this lane's query token
    const int qpos = p.S + qrow;
    const int nkeys = p.S + p.B;
    const int kv_end = min(p.S + q0 + 32, nkeys);  // keys the block can see
    const int ntiles = (kv_end + KT - 1) / KT;
    // first key of the block's first query's window; tiles before its tile
    // hold no visible key for any query of the block
    const int win_lo = p.window > 0 ? max(p.S + q0 - p.window + 1, 0) : 0;
    const int t0 = win_lo / KT;
    const int n_all = ntiles - t0;
    const int iters = (n_all + NKS - 1) / NKS;                 // the same for every wave
    const int my_n = n_all > split ? (n_all - split + NKS - 1) / NKS : 0;   // this split's tiles
    auto tile_of = [&](int i) { return t0 + split + i * NKS; };
    // keys below this bound are outside the last query's window: a tile
    // starting below it may hold keys outside some query's window
    const int win_edge = p.window > 0 ? p.S + q0 + 32 - p.window : -1;
    const float LOG2E = 1.4426950408889634f;
    const float scale = 1.0f / sqrtf((float)HD);
    // exp2-domain logit: c * s, or capl * tanh(s * ic) with a softcap
    const float c = scale * LOG2E;
    const float capl = p.softcap * LOG2E, ic = CAP ? scale / p.softcap : 0.f;

    // This wave's share of a tile's DMA: instructions j, j+G, ... of the
    // NDMA (the last ones repeat instruction j when NDMA is not a multiple of
    // G: the same bytes to the same place).  K instruction d covers rows
    // RPI*d .. RPI*d + RPI-1 (RPI = 64/KCH rows: 4 at HD=128, 8 at HD=64);
    // lane l takes row RPI*d + l/KCH and chunk (l % KCH) ^ (row % KCH), so
    // the 16 rows one pass of a fragment read touches sit in 16 (HD=128) or
    // 8 (HD=64) different chunk positions.  V^T instruction v = d - K_INSTR
    // covers hd rows 16v .. 16v+15, four 16-byte chunks (8 keys) each; chunk
    // c of row r sits at c ^ ((r/4) % 4), so the four rows of a pass that
    // share banks (r, r+4, r+8, r+12) read four different positions.  Both
    // offsets are a per-lane part plus a part of d: the K swizzle of row
    // RPI*d + l/KCH is (l % KCH) ^ (l/KCH) ^ (RPI*d % KCH), and (r/4) % 4 =
    // (l/16) % 4 for every v.
    constexpr int RPI = 64 / KCH;
    const f16* kbase = p.k16 + (size_t)g * p.tcap * HD;
    const f16* vbase = p.vt16 + (size_t)g * HD * p.tcap;
    const int kswz = (lane % KCH) ^ (lane / KCH);
    const int krow = (lane / KCH) * HD;
    auto k_ofs = [&](int d) {   // d wave-uniform
        return (size_t)d * RPI * HD + krow + ((kswz ^ ((RPI * d) & (KCH - 1))) * 8);
    };
    const int vofs = (lane >> 2) * p.tcap + (((lane & 3) ^ ((lane >> 4) & 3)) * 8);
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
    auto issue = [&](int tile, int slot) {
        const size_t k0 = (size_t)tile * KT;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int d0 = j + r * G;
            const int d = d0 < NDMA ? d0 : j;     // wave-uniform
            const f16* src = d < K_INSTR
                ? kbase + k0 * HD + k_ofs(d)
                : vbase + k0 + (size_t)(d - K_INSTR) * 16 * p.tcap + vofs;
            dma16(src, ring_lds + slot * STAGE + d * 1024);
        }
    };

    // the first tile's DMA goes out before the Q loads
    if (my_n > 0) issue(tile_of(0), 0);

    // Q^T operand: lane holds Q[qrow][h][ks*16 + 8*g2 .. +7]
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

    // One head per workgroup (G == 1): each wave owns its ring and runs
    // through its own tiles with no barrier, issuing tile i+NS-1 (past its
    // last tile: the last one again, into a slot it has finished with, so
    // every step waits for the same count) before it waits for tile i.
    // Shared rings (G > 1): the workgroup steps through the tiles in lockstep.
    for (int i = 0; i < (G == 1 ? my_n : iters); ++i) {
        if constexpr (G == 1) {
            issue(tile_of(min(i + NS - 1, my_n - 1)), (i + NS - 1) % NS);
            wait_vmcnt<(NS - 1) * PER>();
            asm volatile("" ::: "memory");
        } else {
            // this wave's share of tile i has landed (nothing newer is in
            // flight); the barrier makes every wave's share visible and ends
            // every wave's reads of tile i-1, whose slot then takes tile i+1
            wait_vmcnt<0>();
            __syncthreads();
            if (i + 1 < my_n) issue(tile_of(i + 1), (i + 1) % NS);
            if (i >= my_n) continue;
        }
        const int slot = i % NS;
        const half8* Ks = reinterpret_cast<const half8*>(ring + slot * STAGE);
        const f16* Vs = reinterpret_cast<const f16*>(ring + slot * STAGE + K_BYTES);
        const int k0 = tile_of(i) * KT;

        // S^T[key][query]: A = K rows, B = Q^T; with one wave per SIMD two
        // independent chains, else one (the other waves fill the gaps and
        // the registers are needed)
        constexpr int CH = G * NKS >= 8 ? 1 : 2;
        floatx16 st[CH];
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
#pragma unroll
            for (int e = 0; e < 16; ++e) st[ch][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cc = ks * 2 + g2;
            st[ks % CH] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ks[ql * KCH + (cc ^ (ql & (KCH - 1)))], qf[ks],
                                                                 st[ks % CH], 0, 0, 0);
        }
        // lane holds key k0 + 8*(e/4) + 4*g2 + e%4 of query qrow.  Without a
        // softcap the scores stay raw (the exp2-domain scale c > 0 keeps
        // their order) and c is folded into the exponent's fma below.
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float r = CH == 2 ? st[0][e] + st[CH - 1][e] : st[0][e];
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
        // O^T[hd][query] += V^T P^T.  P^T operand kh: element jj of lane group
        // g2 is key kh*16 + (jj < 4 ? 4*g2 + jj : 8 + 4*g2 + jj - 4), which is
        // exactly score e = 8*kh + jj above; the V^T operand reads the same keys.
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int r = hb * 32 + ql;
            const f16* vrow = Vs + r * KT;
            const int sw = (r >> 2) & 3;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                // the staged key order puts this lane's 8 keys in chunk 2kh + g2
                const half8 vf = *reinterpret_cast<const half8*>(vrow + (((2 * kh + g2) ^ sw) * 8));
                o[hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kh], o[hb], 0, 0, 0);
            }
        }
    }

    // Merge the splits of each head in a fixed order: splits 1 .. NKS-1
    // leave (m, l, O^T) in LDS and split 0 folds them in one after another.
    // Once every DMA has landed (the one-head path may still have repeats of
    // its last tile in flight) the rings can be reused.
    if constexpr (NKS > 1) {
        float* states = reinterpret_cast<float*>(smem_all);
        wait_vmcnt<0>();
        __syncthreads();
        if (split > 0) {
            float* st = states + ((split - 1) * G + j) * state_floats<HD>();
            if (g2 == 0) {
                st[ql] = m;
                st[32 + ql] = l;
            }
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = hb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
                    st[64 + r * 32 + ql] = o[hb][e];
                }
        }
        __syncthreads();
        if (split > 0) return;
#pragma unroll 1
        for (int w = 1; w < NKS; ++w) {
            const float* st = states + ((w - 1) * G + j) * state_floats<HD>();
            const float mo = st[ql], lo = st[32 + ql];
            // finite: the tile holding a query's own key is visited by one of
            // the splits; a split that saw no visible key has m = -inf, l = 0, O = 0
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
                    o[hb][e] = o[hb][e] * a + st[64 + r * 32 + ql] * b;
                }
        }
    }

    if (split != 0 || qrow >= p.B) return;
    const float inv_l = 1.0f / l;
    f16* out = p.o16 + (size_t)qrow * p.hq * HD + h * HD;
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
            *reinterpret_cast<half4*>(out + d0) = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
        }
}

template <int HD, bool CAP, int G, int NKS>
hipError_t launch_cfg(const AttnPrefillArgs& a, hipStream_t s) {
    constexpr int lds = attn_lds_bytes<HD, G, NKS>();
    // the rings may take more than the default 64 KB of dynamic LDS; the
    // attribute is set once per device (idempotent if two threads race)
    static std::atomic<bool> set_on[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !set_on[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefill_kernel<HD, CAP, G, NKS>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) set_on[dev].store(true, std::memory_order_release);
    }
    const dim3 grid(a.hq / G, (a.B + 31) / 32);
    hipLaunchKernelGGL((attn_prefill_kernel<HD, CAP, G, NKS>), grid, dim3(G * NKS * 64), lds, s, a);
    return hipGetLastError();
}

// Measured at 3B width (24 query / 8 KV heads of 128), rocprof averages:
// at 512 new tokens one head per workgroup with two waves takes 14.7 us
// against 18.5 us for three heads sharing tiles (nine waves, one workgroup
// per CU: the heaviest query block's three heads then queue on one CU), and
// 42.6 against 46.5 us over a 1536-row prefix; at 8B width and 4096 tokens
// (1024 packed workgroups) sharing takes 219 us against 356 us.  So: one
// head per workgroup while the packed grid would be under two rounds of
// 256 CUs, shared tiles beyond.  Both use two key splits and two-stage rings
// (64 KB of LDS: two workgroups per CU).
template <int HD, bool CAP, int G>
hipError_t launch_group(const AttnPrefillArgs& a, hipStream_t s) {
    const int packed_wgs = (a.hq / G) * ((a.B + 31) / 32);
    const bool shared = a.form == DDL_ATTN_SHARED ||
                        (a.form != DDL_ATTN_ONE_HEAD && packed_wgs >= 512);
    if (G == 1 || !shared) return launch_cfg<HD, CAP, 1, 2>(a, s);
    return launch_cfg<HD, CAP, G, 2>(a, s);
}

// Query heads per shared-tile workgroup: the largest of 6, 4, 3, 2, 1 that
// divides the GQA group (a group of 8 takes two workgroups of 4 per KV head).
template <int HD, bool CAP>
hipError_t launch_hd(const AttnPrefillArgs& a, hipStream_t s) {
    const int group = a.hq / a.hkv;
    if (group % 6 == 0) return launch_group<HD, CAP, 6>(a, s);
    if (group % 4 == 0) return launch_group<HD, CAP, 4>(a, s);
    if (group % 3 == 0) return launch_group<HD, CAP, 3>(a, s);
    if (group % 2 == 0) return launch_group<HD, CAP, 2>(a, s);
    return launch_group<HD, CAP, 1>(a, s);
}
}  // namespace

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
    if (a.tcap % 32 || a.tcap < a.S + a.B || a.window < 0 || a.hkv <= 0 || a.hq % a.hkv)
        return hipErrorInvalidValue;
    const bool cap = a.softcap > 0.f;
    if (a.hd == 128) return cap ? launch_hd<128, true>(a, s) : launch_hd<128, false>(a, s);
    if (a.hd == 64) return cap ? launch_hd<64, true>(a, s) : launch_hd<64, false>(a, s);
    return hipErrorInvalidValue;
}
