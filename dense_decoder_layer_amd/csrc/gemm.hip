// fp16 MFMA GEMM with fused epilogues for the layer's projections:
//   C[M][N] = A[M][K] * W[N][K]^T * inv_scale
// A holds token-major activations (normed rows, attention output or SwiGLU
// output, rounded to fp16); W is a packed weight matrix whose fp16 values are
// the layer's weights times 2^shift (inv_scale undoes it).
//
// Epilogues (the steps between the matmuls of a layer, fused into the
// matmul that produces their input):
//   EPI_F32     store fp32 (the stacked q/k/v/gate projection)
//   EPI_RESID   C = R + acc (wo and down projections plus the residual;
//               with R null, C = acc for a layer whose branch is normed first).
//               The residual tile is read before the k-loop (9 us of exposed
//               latency per launch when read in the epilogue)
//   EPI_SWIGLU  W rows are gate/up interleaved in 16-row blocks; store
//               fp16 silu(gate) * up into H[M][N/2]
//   EPI_GEGLU   the same with the exact GELU, gate * Phi(gate), in place of
//               silu (the GELU-gated FFN of "frink-models 0.29.0
//               src/decoder/cuda_prefill.rs", try_cuda_prefill_dense_stack)
//
// Design (gfx950, v_mfma_f32_32x32x16_f16):
//  * W is stored in MFMA-fragment order (see the packing kernels): the
//    32 x 16 block (rows 32nb.., k 16kb..) is 1 KB in which lane l's B
//    operand -- row 32nb + l%32, k 16kb + 8*(l/32) .. +7 -- sits at byte
//    16*l.  A wave loads each weight fragment with one fully coalesced
//    1 KB global load straight into registers; weights never touch LDS.
//  * The activation tile (BM rows x 64 k) is shared by the workgroup's
//    waves: its 16-byte chunks are loaded into registers NS-1 k-tiles
//    ahead (consecutive threads take consecutive chunks of a row, so the
//    loads coalesce) and written into a 2-slot LDS ring one step before
//    use, chunk c of row r at position c ^ (r % 8), so the fragment reads
//    of 8 consecutive lanes (one row each, same chunk) hit distinct banks.
//    Every load of the kernel is an ordinary register load, so the
//    hardware returns them in issue order and one counter tracks them.
//  * A stage spans 64 k (128 for the six-wave 64 x 192 tiles, where
//    halving the barriers per K measured 11-21% faster).
//  * Per k-tile: issue the loads of k-tile kt+NS-1, multiply k-tile kt,
//    write k-tile kt+1's activations into the other LDS slot, barrier.
//    For the K of the hot projections the k-loop is unrolled at compile
//    time (straight-line code, so the compiler's own waits on the register
//    loads are exact); other K run a generic loop.
//  * Workgroups of the same weight tile are dispatched to the same XCD.
#include "common.h"
#include "internal.h"

#include <type_traits>
#include <utility>

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;   // k granularity of the shapes; a kernel's stage takes BKT = 64 or 128

__device__ __forceinline__ floatx16 mfma32x32x16(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Waits for this wave's LDS writes (s_waitcnt lgkmcnt(0); gfx9 encoding:
// vmcnt[3:0] + [15:14], expcnt[6:4], lgkmcnt[11:8], the others at maximum),
// then the workgroup barrier; no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 (straight-line code).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

// Accumulator layout of a 32x32 MFMA tile: lane l holds column l % 32 of
// rows 8*(e/4) + 4*(l/32) + e%4 for e = 0..15.
// The residual tile of a wave (EPI_RESID, K slice 0), read into registers
// before the k-loop so its memory latency hides behind the MFMAs instead of
// being exposed at the end (R may alias C: each element is read and written
// by the same lane, and no other workgroup writes this tile of C).
template <int MI, int NI, int EPI>
struct ResidTile {
    float v[EPI == EPI_RESID ? MI : 1][EPI == EPI_RESID ? NI : 1][16];
};

template <int MI, int NI, int EPI>
__device__ __forceinline__ void load_resid(const GemmArgs& p, ResidTile<MI, NI, EPI>& rt, int row0,
                                           int col0, int lane, bool full, int split) {
    if constexpr (EPI == EPI_RESID) {
        const int rbase = row0 + 4 * (lane >> 5), cl = lane & 31;
        const bool use = split == 0 && p.R;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                    rt.v[i][j][e] = use && (full || row < p.M)
                                        ? p.R[(size_t)row * p.ldr + col0 + j * 32 + cl] : 0.f;
                }
    }
}

template <int MI, int NI, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, floatx16 (&acc)[MI][NI], int row0,
                                         int col0, int lane, bool full, int split,
                                         const ResidTile<MI, NI, EPI>& rt) {
    const float sc = *p.inv_scale;
    const int rbase = row0 + 4 * (lane >> 5);
    const int cl = lane & 31;
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_GEGLU) {
        // a 32-column tile holds gate block 2q (lanes 0..15 of the columns)
        // and up block 2q+1 (lanes 16..31) of the same 16 outputs
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int fcol = ((col0 + j * 32) >> 1) + (cl & 15);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                float a[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float v = acc[i][j][e] * sc;
                    const float other = __shfl_xor(v, 16, 64);   // lane l^16 holds the partner
                    // silu from the hardware exp2 and reciprocal (~1 ulp each, far
                    // below the fp16 rounding of the output); the library expf and
                    // IEEE divide cost ~6 us of VALU per launch at 512 x 16384
                    const float act = EPI == EPI_GEGLU
                                          ? 0.5f * v * (1.0f + erff(v * 0.7071067811865476f))
                                          : v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
                    a[e] = act * other;
                }
                if (cl < 16) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                        if (full || row < p.M) p.H[(size_t)row * p.ldh + fcol] = (f16)a[e];
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int col = col0 + j * 32 + cl;
                float v[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = acc[i][j][e] * sc;
                if (split > 0) {         // a later K slice: raw partial for the consumer
                    float* P = p.P + (size_t)(split - 1) * p.M * p.ldc;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                        if (full || row < p.M) P[(size_t)row * p.ldc + col] = v[e];
                    }
                    continue;
                }
                if constexpr (EPI == EPI_RESID) {   // zeros when R is null (raw branch output)
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] += rt.v[i][j][e];
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                    if (full || row < p.M) p.C[(size_t)row * p.ldc + col] = v[e];
                }
            }
    }
}

// Workgroup of WGM x WGN waves, tile BM x (WN*WGN); wave tile (BM/WGM) x WN.
// The grid is tiles x splits; slice z takes k-tiles [z*nk, (z+1)*nk).
// NK > 0: nk == NK, straight-line k-loop; NK == 0: generic loop.
template <int BM, int WN, int WGM, int WGN, int NS, int EPI, int NK, int BKT>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_kernel(GemmArgs p, int splits) {
    constexpr int KC = BKT / 8;                     // 16-byte chunks per activation row of a stage
    constexpr int NT = WGM * WGN * 64, BN = WN * WGN, WM = BM / WGM;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int A_TOT = BM * KC;                  // 16-byte activation chunks per k-tile
    constexpr int A_CH = (A_TOT + NT - 1) / NT;     // per thread (six waves: the last one partial)
    constexpr int STAGE = BM * BKT * 2;
    static_assert(MI >= 1 && NI >= 1, "wave tile below 32x32");
    static_assert(A_CH >= 1, "activation chunks");
    static_assert(NS >= 2 && NS <= 4, "pipeline depth");
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int mt = (p.M + BM - 1) / BM, nt = p.N / BN, total = mt * nt * splits;
    int bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int tile = bid % (mt * nt), split = bid / (mt * nt);
    const int m0 = (tile % mt) * BM, n0 = (tile / mt) * BN;
    const int nk = NK > 0 ? NK : p.K / BKT / splits;
    const int kt0 = split * nk;                    // this slice's first k-tile

    const f16* a_src[A_CH];
    int a_dst[A_CH];                                // half8 index in an LDS slot
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int idx = i * NT + tid;
        const bool ok = A_CH * NT == A_TOT || idx < A_TOT;   // past the tile: loads row 0, never stored
        const int r = ok ? idx / KC : 0, c = idx % KC;
        a_src[i] = p.A + (size_t)min(m0 + r, p.M - 1) * p.lda + (size_t)kt0 * BKT + c * 8;   // rows past M: discarded outputs
        a_dst[i] = ok ? r * KC + (c ^ (r & 7)) : -1;
    }
    const f16* wfrag[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j)
        wfrag[j] = p.W + ((size_t)((n0 + wn * WN) / 32 + j) * (p.K / 16) + (size_t)kt0 * (BKT / 16)) * 512 + lane * 8;

    half8 areg[NS][A_CH];
    half8 breg[NS][NI][BKT / 16];
    auto issue = [&](int kt, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            areg[slot][i] = *reinterpret_cast<const half8*>(a_src[i] + (size_t)kt * BKT);
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int ks = 0; ks < BKT / 16; ++ks)
                breg[slot][j][ks] = *reinterpret_cast<const half8*>(wfrag[j] + (size_t)(kt * (BKT / 16) + ks) * 512);
    };
    auto commit = [&](auto slot_c, int buf) {
        constexpr int slot = decltype(slot_c)::value;
        half8* As = reinterpret_cast<half8*>(smem + buf * STAGE);
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            if (A_CH * NT == A_TOT || a_dst[i] >= 0) As[a_dst[i]] = areg[slot][i];
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // One k-tile: issue k-tile kt+NS-1 into the register slot consumed one
    // step ago (past the end, the last k-tile again: in bounds, never used),
    // multiply from LDS buffer kt%2, write k-tile kt+1 into the other buffer
    // (last read two steps ago, before the previous barrier), barrier.
    auto step = [&](int kt, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        issue(min(kt + NS - 1, nk - 1), std::integral_constant<int, (slot + NS - 1) % NS>());
        const half8* As = reinterpret_cast<const half8*>(smem + (kt & 1) * STAGE);
        half8 af[2][MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int r = wm * WM + i * 32 + (lane & 31), c = lane >> 5;
            af[0][i] = As[r * KC + (c ^ (r & 7))];
        }
#pragma unroll
        for (int ks = 0; ks < BKT / 16; ++ks) {
            if (ks + 1 < BKT / 16) {
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const int r = wm * WM + i * 32 + (lane & 31), c = (ks + 1) * 2 + (lane >> 5);
                    af[(ks + 1) & 1][i] = As[r * KC + (c ^ (r & 7))];
                }
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = mfma32x32x16(af[ks & 1][i], breg[slot][j][ks], acc[i][j]);
        }
        commit(std::integral_constant<int, (slot + 1) % NS>(), (kt + 1) & 1);
        lds_barrier();
    };

    ResidTile<MI, NI, EPI> rt;
    load_resid<MI, NI, EPI>(p, rt, m0 + wm * WM, n0 + wn * WN, lane, m0 + BM <= p.M, split);
    issue(0, std::integral_constant<int, 0>());
    if constexpr (NS > 2) issue(min(1, nk - 1), std::integral_constant<int, 1>());
    if constexpr (NS > 3) issue(min(2, nk - 1), std::integral_constant<int, 2>());
    commit(std::integral_constant<int, 0>(), 0);
    lds_barrier();
    if constexpr (NK > 0) {
        static_for<NK>([&](auto kc) {
            constexpr int kt = decltype(kc)::value;
            step(kt, std::integral_constant<int, kt % NS>());
        });
    } else {
        for (int kt = 0; kt < nk; kt += NS) {
            step(kt, std::integral_constant<int, 0>());
            if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1 % NS>());
            if constexpr (NS > 2) if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2 % NS>());
            if constexpr (NS > 3) if (kt + 3 < nk) step(kt + 3, std::integral_constant<int, 3 % NS>());
        }
    }
    epilogue<MI, NI, EPI>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, m0 + BM <= p.M, split, rt);
}

// The 128 x 256 eight-wave tile on v_mfma_f32_16x16x32_f16, for gate/up at
// large M (862 -> 810 us on the 8B layer at 4096 tokens against the
// 32x32x16 form, one box; at 512 tokens the 32x32x16 form is as fast or
// faster, and for the residual projections at 4096 tokens this form
// measured no faster).  Wave tile 128 x 32 = 8 x 2 tiles of 16 x 16.
// A fragment (16 rows x 32 k): lane l holds row l % 16, chunk l / 16 of
// the 32-wide window, read from the same swizzled LDS tile as above.
// B fragment (32 k x 16 columns): lane l holds column l % 16 and k
// 8(l/16) .. +7 of the window, which in the 32 x 16 fragment blocks sits
// in block 2w + (l/32), lane 16 jj + l % 16 + 32 ((l/16) % 2): one 16-byte
// load a lane, in 256-byte runs.  Accumulator: lane l holds column l % 16
// of rows 4(l/16) .. +3; in a gate/up tile, 16-column tile 0 is the gate
// and tile 1 the up half of the same 16 outputs, so SwiGLU pairs them
// within the lane.
template <int NS, int EPI, int NK>
__global__ __launch_bounds__(512) void gemm16_kernel(GemmArgs p) {
    static_assert(EPI == EPI_SWIGLU || EPI == EPI_GEGLU, "gate/up epilogues only");
    constexpr int BM = 128, BN = 256, BKT = 64, KC = 8, NT = 512, WN = 32;
    constexpr int A_TOT = BM * KC, A_CH = A_TOT / NT, STAGE = BM * BKT * 2;
    constexpr int MT = BM / 16, NTL = WN / 16, KW = BKT / 32;   // 16x16 tiles, k32 windows
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mt = (p.M + BM - 1) / BM, nt = p.N / BN, total = mt * nt;
    int bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int m0 = (bid % mt) * BM, n0 = (bid / mt) * BN;
    const int nk = NK > 0 ? NK : p.K / BKT;

    const f16* a_src[A_CH];
    int a_dst[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int idx = i * NT + tid;
        const int r = idx / KC, c = idx % KC;
        a_src[i] = p.A + (size_t)min(m0 + r, p.M - 1) * p.lda + c * 8;
        a_dst[i] = r * KC + (c ^ (r & 7));
    }
    // B: the wave's 32 columns are fragment block (n0 + 32 wave) / 32
    const int q = lane >> 4;
    const f16* wbase = p.W + ((size_t)((n0 + wave * WN) / 32) * (p.K / 16) + (q >> 1)) * 512 +
                       ((lane & 15) + 32 * (q & 1)) * 8;

    half8 areg[NS][A_CH];
    half8 breg[NS][KW][NTL];
    auto issue = [&](int kt, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            areg[slot][i] = *reinterpret_cast<const half8*>(a_src[i] + (size_t)kt * BKT);
#pragma unroll
        for (int w = 0; w < KW; ++w)
#pragma unroll
            for (int jj = 0; jj < NTL; ++jj)
                breg[slot][w][jj] = *reinterpret_cast<const half8*>(wbase + (size_t)(kt * (BKT / 16) + 2 * w) * 512 + jj * 16 * 8);
    };
    auto commit = [&](auto slot_c, int buf) {
        constexpr int slot = decltype(slot_c)::value;
        half8* As = reinterpret_cast<half8*>(smem + buf * STAGE);
#pragma unroll
        for (int i = 0; i < A_CH; ++i) As[a_dst[i]] = areg[slot][i];
    };

    floatx4 acc[MT][NTL];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto step = [&](int kt, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        issue(min(kt + NS - 1, nk - 1), std::integral_constant<int, (slot + NS - 1) % NS>());
        const half8* As = reinterpret_cast<const half8*>(smem + (kt & 1) * STAGE);
#pragma unroll
        for (int w = 0; w < KW; ++w) {
            half8 af[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int r = i * 16 + (lane & 15), c = w * 4 + q;
                af[i] = As[r * KC + (c ^ (r & 7))];
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NTL; ++j) acc[i][j] = mfma16x16x32(af[i], breg[slot][w][j], acc[i][j]);
        }
        commit(std::integral_constant<int, (slot + 1) % NS>(), (kt + 1) & 1);
        lds_barrier();
    };

    const int col0 = n0 + wave * WN;
    const bool full = m0 + BM <= p.M;
    static_assert(NS == 3, "three-deep register prefetch");
    issue(0, std::integral_constant<int, 0>());
    issue(min(1, nk - 1), std::integral_constant<int, 1>());
    commit(std::integral_constant<int, 0>(), 0);
    lds_barrier();
    if constexpr (NK > 0) {
        static_for<NK>([&](auto kc) {
            constexpr int kt = decltype(kc)::value;
            step(kt, std::integral_constant<int, kt % NS>());
        });
    } else {
        for (int kt = 0; kt < nk; kt += NS) {
            step(kt, std::integral_constant<int, 0>());
            if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>());
            if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>());
        }
    }

    const float sc = *p.inv_scale;
    const int fcol = (col0 >> 1) + (lane & 15);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float g = acc[i][0][e] * sc, u = acc[i][1][e] * sc;
            const float act = EPI == EPI_GEGLU
                                  ? 0.5f * g * (1.0f + erff(g * 0.7071067811865476f))
                                  : g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
            const int row = m0 + i * 16 + 4 * q + e;
            if (full || row < p.M) p.H[(size_t)row * p.ldh + fcol] = (f16)(act * u);
        }
}

constexpr int MF16_MIN_M = 2048;   // the 16x16x32 form from here on

template <int EPI>
hipError_t launch16(const GemmArgs& a, hipStream_t s) {
    const dim3 grid(((a.M + 127) / 128) * (a.N / 256)), block(512);
    switch (a.K / 64) {
        case 48: hipLaunchKernelGGL((gemm16_kernel<3, EPI, 48>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((gemm16_kernel<3, EPI, 64>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((gemm16_kernel<3, EPI, 0>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int BM, int WN, int WGM, int WGN, int NS, int EPI, int NK, int BKT>
hipError_t launch_cfg(const GemmArgs& a, int splits, hipStream_t s) {
    const int mt = (a.M + BM - 1) / BM, nt = a.N / (WN * WGN);
    hipLaunchKernelGGL((gemm_kernel<BM, WN, WGM, WGN, NS, EPI, NK, BKT>), dim3(mt * nt * splits),
                       dim3(WGM * WGN * 64), 0, s, a, splits);
    return hipGetLastError();
}

// The k-tile counts per slice of the hot shapes get the straight-line loop.
template <int BM, int WN, int WGM, int WGN, int NS, int EPI, int BKT = 64>
hipError_t launch_nk(const GemmArgs& a, int splits, hipStream_t s) {
    switch (a.K / BKT / splits) {
        case 8: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 8, BKT>(a, splits, s);
        case 12: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 12, BKT>(a, splits, s);
        case 16: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 16, BKT>(a, splits, s);
        case 24: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 24, BKT>(a, splits, s);
        case 32: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 32, BKT>(a, splits, s);
        case 48: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 48, BKT>(a, splits, s);
        case 64: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 64, BKT>(a, splits, s);
        case 128: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 128, BKT>(a, splits, s);
        default: return launch_cfg<BM, WN, WGM, WGN, NS, EPI, 0, BKT>(a, splits, s);
    }
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K, int epi) {
    (void)epi;
    return M > 0 && N > 0 && K > 0 && N % 128 == 0 && K % BK == 0;
}

// Tiles and K splits (measured on MI355X at the 512-token shapes).  At
// these shapes the narrow projections are limited by how many CUs their grid
// fills, so the plan aims at one 8- or 6-wave workgroup per CU:
//  * gate/up: 128 x 256 tiles, eight waves of 128 x 32 sharing one
//    activation tile, 3-deep register prefetch (a third fewer bytes per flop
//    than two 128 x 128 workgroups on a CU).  Never split (SwiGLU/GELU need
//    the whole sum).
//  * stacked QKV: the same tile, K split so the grid comes closest to 256
//    workgroups (80 tiles at 512 tokens: three slices, 240 workgroups; 23 us
//    against 28 us with two).
//    From 2048 rows the gate/up tile is issued as 16x16x32 MFMAs
//    (gemm16_kernel below).
//  * wo and down, width a multiple of 192: 64 x 192 tiles of six waves,
//    split to fill 256 workgroups (two slices at 512 tokens).  For down this
//    matches the four-way split of 64 x 128 tiles in time with one partial
//    sum instead of three for the next norm to add.
//  * wo and down at large M, once 128 x 256 tiles alone fill the CUs (4096
//    tokens): the gate/up tile with the residual epilogue, unsplit (8B
//    layer: down 641 -> 504 us, wo 193 -> 161 us against 64 x 256 tiles).
//  * other residual shapes: 64 x 128 tiles (four waves, three workgroups fit
//    a CU) split until 768 workgroup slots fill, each slice keeping at least
//    24 k-tiles; 64 x 256 tiles of eight waves where that gives fewer than
//    four slices.
//  * Anything else: 64 x 128 tiles, gate/up 128 x 128.
namespace {
enum Tile { T64x128, T128x128, T128x256, T64x256, T64x192, T128x256R };
struct Plan {
    Tile tile;
    int splits;
};

int split_count(int tiles, int slots, int nk) {
    int splits = 1;
    while (splits < 4 && tiles * splits * 2 <= slots && nk % (splits * 2) == 0 &&
           nk / (splits * 2) >= 24)
        splits *= 2;
    return splits;
}

// The K split in 1..4 that brings tiles * split closest to `slots` without
// passing it, each slice keeping at least 16 k-tiles.
int fill_split(int tiles, int slots, int nk) {
    int best = 1;
    for (int s = 2; s <= 4; ++s)
        if (tiles * s <= slots && nk % s == 0 && nk / s >= 16) best = s;
    return best;
}

Plan gemm_plan(int M, int N, int K, int epi) {
    const int nk = K / BK;
    if (epi == EPI_SWIGLU || epi == EPI_GEGLU) return {N % 256 == 0 && M > 64 ? T128x256 : T128x128, 1};
    if (epi == EPI_F32 && N % 256 == 0 && M > 64)
        return {T128x256, fill_split(((M + 127) / 128) * (N / 256), 256, nk)};
    // large M: the gate/up tile, which fills the CUs without a K split
    if (epi == EPI_RESID && N % 256 == 0 && ((M + 127) / 128) * (N / 256) >= 256)
        return {T128x256R, 1};
    if (epi == EPI_RESID && N % 192 == 0 && M > 64 && ((M + 63) / 64) * (N / 192) <= 256)
        return {T64x192, fill_split(((M + 63) / 64) * (N / 192), 256, nk)};
    const int splits = split_count(((M + 63) / 64) * (N / 128), 768, nk);
    if (epi == EPI_RESID && splits < 4 && N % 256 == 0)
        return {T64x256, split_count(((M + 63) / 64) * (N / 256), 256, nk)};
    return {T64x128, splits};
}
}  // namespace

int gemm_splits(int M, int N, int K, int epi) {
    if (!gemm_shape_ok(M, N, K, epi)) return 1;
    return gemm_plan(M, N, K, epi).splits;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, int splits, hipStream_t s) {
    if (!gemm_shape_ok(a.M, a.N, a.K, epi)) return hipErrorInvalidValue;
    if (splits < 1 || (a.K / BK) % splits ||
        (splits > 1 && (!a.P || epi == EPI_SWIGLU || epi == EPI_GEGLU)))
        return hipErrorInvalidValue;
    const Tile t = gemm_plan(a.M, a.N, a.K, epi).tile;
    if (t == T128x256 && (epi == EPI_SWIGLU || epi == EPI_GEGLU) && a.M >= MF16_MIN_M)
        return epi == EPI_SWIGLU ? launch16<EPI_SWIGLU>(a, s) : launch16<EPI_GEGLU>(a, s);
    switch (epi) {
        case EPI_SWIGLU:
            if (t == T128x256) return launch_nk<128, 32, 1, 8, 3, EPI_SWIGLU>(a, 1, s);
            return launch_nk<128, 32, 1, 4, 4, EPI_SWIGLU>(a, 1, s);
        case EPI_GEGLU:
            if (t == T128x256) return launch_nk<128, 32, 1, 8, 3, EPI_GEGLU>(a, 1, s);
            return launch_nk<128, 32, 1, 4, 4, EPI_GEGLU>(a, 1, s);
        case EPI_F32:
            if (t == T128x256) return launch_nk<128, 32, 1, 8, 3, EPI_F32>(a, splits, s);
            return launch_nk<64, 32, 1, 4, 4, EPI_F32>(a, splits, s);
        case EPI_RESID:
            if (t == T64x192)   // 128-wide k stages where a slice divides (wo 24 -> 19 us, down 41 -> 36 us in a harness)
                return (a.K / splits) % 128 == 0 ? launch_nk<64, 32, 1, 6, 3, EPI_RESID, 128>(a, splits, s)
                                                 : launch_nk<64, 32, 1, 6, 3, EPI_RESID>(a, splits, s);
            if (t == T64x256) return launch_nk<64, 32, 1, 8, 3, EPI_RESID>(a, splits, s);
            if (t == T128x256R) return launch_nk<128, 32, 1, 8, 3, EPI_RESID>(a, splits, s);
            return launch_nk<64, 32, 1, 4, 4, EPI_RESID>(a, splits, s);
    }
    return hipErrorInvalidValue;
}
