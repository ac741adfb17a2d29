// fp16 MFMA GEMM with fused epilogues for the layer's projections:
//   C[M][N] = A[M][K] * W[N][K]^T * inv_scale
// A holds token-major activations (normed rows, attention output or SwiGLU
// output, rounded to fp16); W holds a packed weight matrix [out][in] whose
// fp16 values are the layer's weights times 2^shift (inv_scale undoes it).
// Both operands are K-contiguous, so A and W fragments are read alike.
//
// Epilogues (the steps between the matmuls of a layer, fused into the
// matmul that produces their input):
//   EPI_F32     store fp32 (the stacked q/k/v/gate projection)
//   EPI_RESID   C = R + acc (wo and down projections plus the residual)
//   EPI_SWIGLU  W rows are gate/up interleaved in 16-row blocks; store
//               fp16 silu(gate) * up into H[M][N/2]
//
// Tiling (gfx950): a workgroup of WGM x WGN waves computes a BM x BN tile;
// each wave owns a (BM/WGM) x (BN/WGN) block of v_mfma_f32_32x32x16_f16
// tiles.  K advances 64 at a time through an NS-stage ring in LDS that is
// filled by global_load_lds_dwordx4 (global memory straight into LDS, no
// VGPR staging), so NS-1 stages are in flight while one is consumed.  One
// DMA instruction writes 1 KB = 8 LDS rows of 128 B, lane l at byte 16*l;
// the lane fetches the 16-byte chunk (l % 8) ^ (row % 8) of its row, which
// leaves every row XOR-swizzled so the fragment reads of 8 consecutive
// lanes (one row each, same chunk) hit distinct banks.
#include "common.h"
#include "internal.h"

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int K_ALIGN = 64;     // every K the library passes is a multiple of this

__device__ __forceinline__ floatx16 mfma32x32x16(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// bytes [16l, 16l+16) after the wave-uniform LDS address `lds`.  The size-16
// form exists on gfx950 only, so the host compilation pass (which checks the
// builtin against a generic target) does not see it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
#endif
}

// s_waitcnt with only vmcnt limited (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Accumulator layout of a 32x32 MFMA tile: lane l holds column l % 32 of
// rows 8*(e/4) + 4*(l/32) + e%4 for e = 0..15.
template <int BM, int WM, int WN, int MI, int NI, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, floatx16 (&acc)[MI][NI], int m0, int n0,
                                         int wm, int wn, int lane, int split) {
    const float sc = *p.inv_scale;
    const int rbase = m0 + wm * WM + 4 * (lane >> 5);
    const int cl = lane & 31;
    const bool full = m0 + BM <= p.M;      // no row of the tile is past M
    if constexpr (EPI == EPI_SWIGLU) {
        // 32-column MFMA tile j holds gate block 2q (lanes 0..15 of the
        // column range) and up block 2q+1 (lanes 16..31) for 16 outputs
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int col0 = n0 + wn * WN + j * 32;      // multiple of 32
                const int fcol = (col0 >> 1) + (cl & 15);
                float a[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float v = acc[i][j][e] * sc;
                    const float other = __shfl_xor(v, 16, 64);   // lane l^16 holds the partner
                    a[e] = v / (1.0f + expf(-v)) * other;
                }
                if (cl < 16) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                        if (full || row < p.M) p.H[(size_t)row * p.ldh + fcol] = (f16)a[e];
                    }
                }
            }
    } else if (split > 0) {
        float* P = p.P + (size_t)(split - 1) * p.M * p.N;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int col = n0 + wn * WN + j * 32 + cl;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                    if (full || row < p.M) P[(size_t)row * p.N + col] = acc[i][j][e] * sc;
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int col = n0 + wn * WN + j * 32 + cl;
                float v[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = acc[i][j][e] * sc;
                if constexpr (EPI == EPI_RESID) {
                    if (full) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                            v[e] += p.R[(size_t)row * p.ldr + col];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                            if (row < p.M) v[e] += p.R[(size_t)row * p.ldr + col];
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
                    if (full || row < p.M) p.C[(size_t)row * p.ldc + col] = v[e];
                }
            }
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int NS, int EPI>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_f16_kernel(GemmArgs p) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;       // wave tile
    constexpr int MI = WM / 32, NI = WN / 32;         // 32x32 MFMA tiles per wave
    constexpr int CHUNKS = BK / 8;                    // 16-byte chunks per LDS row
    constexpr int ROW_BYTES = BK * 2;
    constexpr int RPI = 64 / CHUNKS;                  // rows per 1 KB DMA instruction
    constexpr int A_INSTR = BM / RPI / NW, B_INSTR = BN / RPI / NW;   // DMA instructions per wave per stage
    constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
    static_assert(BK == 64 || BK == 128, "k-tile");
    static_assert(MI >= 1 && NI >= 1, "wave tile below 32x32");
    static_assert(A_INSTR >= 1 && B_INSTR >= 1 && A_INSTR * NW * RPI == BM && B_INSTR * NW * RPI == BN,
                  "tile rows must split evenly into DMA blocks per wave");
    static_assert(EPI != EPI_SWIGLU || (WN % 32) == 0, "swiglu pairs 16-column blocks");
    static_assert(NS >= 2 && NS <= 4, "pipeline depth");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // Tile order: the workgroups of one weight tile (all M tiles of one N
    // tile) are consecutive in the logical order, and the logical order is
    // laid out XCD by XCD (dispatch sends workgroup i to XCD i % 8), so a
    // weight tile is fetched into one XCD's L2 and reused there.
    // Split-K: split z takes k-tiles [z*kper, (z+1)*kper); split 0 runs the
    // epilogue, the others store raw fp32 partials that the consumer adds.
    const int mt = (p.M + BM - 1) / BM, nt = p.N / BN;
    const int total = mt * nt * p.splits;
    int bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int m0 = (bid % mt) * BM, n0 = ((bid / mt) % nt) * BN, split = bid / (mt * nt);
    const int kper = p.K / BK / p.splits;
    const size_t kbase = (size_t)split * kper * BK;

    // Per-lane DMA source offsets (in halves) for each of this wave's
    // instructions; only k0 changes from stage to stage.
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    size_t a_off[A_INSTR], b_off[B_INSTR];
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j) {
        const int r = (wave * A_INSTR + j) * RPI + lane / CHUNKS;
        const int c = (lane % CHUNKS) ^ (r & 7);
        const int row = min(m0 + r, p.M - 1);   // rows past M feed only discarded outputs
        a_off[j] = (size_t)row * p.lda + kbase + c * 8;
    }
#pragma unroll
    for (int j = 0; j < B_INSTR; ++j) {
        const int r = (wave * B_INSTR + j) * RPI + lane / CHUNKS;
        const int c = (lane % CHUNKS) ^ (r & 7);
        b_off[j] = (size_t)(n0 + r) * p.ldw + kbase + c * 8;
    }
    auto issue = [&](int kt, int slot) {
        const int k0 = kt * BK;
        const uint32_t sbase = smem_base + slot * STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < A_INSTR; ++j)
            dma16(p.A + a_off[j] + k0, sbase + (wave * A_INSTR + j) * 1024);
#pragma unroll
        for (int j = 0; j < B_INSTR; ++j)
            dma16(p.W + b_off[j] + k0, sbase + BM * ROW_BYTES + (wave * B_INSTR + j) * 1024);
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = kper;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) issue(s, s);

    constexpr int PER_STAGE = A_INSTR + B_INSTR;
    constexpr int KSTEPS = BK / 16;
    half8 af[2][MI], bf[2][NI];
    auto frags = [&](const half8* As, const half8* Bs, int ks, int buf) {
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int r = wm * WM + i * 32 + (lane & 31);
            af[buf][i] = As[r * CHUNKS + (c ^ (r & 7))];
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int r = wn * WN + j * 32 + (lane & 31);
            bf[buf][j] = Bs[r * CHUNKS + (c ^ (r & 7))];
        }
    };
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once at most (stages issued after it) loads are pending
        const int after = min(NS - 2, nk - 1 - kt);
        if (after >= 2) wait_vmcnt<2 * PER_STAGE>();
        else if (after == 1) wait_vmcnt<PER_STAGE>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();   // every wave's part of stage kt is in LDS, and
                                        // every wave is done reading stage kt-1
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);

        const half8* As = reinterpret_cast<const half8*>(smem + (kt % NS) * STAGE_BYTES);
        const half8* Bs = As + BM * (ROW_BYTES / 16);
        frags(As, Bs, 0, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks + 1 < KSTEPS) frags(As, Bs, ks + 1, (ks + 1) & 1);   // next k-step's reads in flight
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = mfma32x32x16(af[ks & 1][i], bf[ks & 1][j], acc[i][j]);
        }
    }

    epilogue<BM, WM, WN, MI, NI, EPI>(p, acc, m0, n0, wm, wn, lane, split);
}


template <int BM, int BN, int BK, int WGM, int WGN, int NS, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    constexpr int lds = NS * (BM + BN) * BK * 2;
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_f16_kernel<BM, BN, BK, WGM, WGN, NS, EPI>),
            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e) return e;
        configured = true;
    }
    if (a.splits < 1 || (a.K / BK) % a.splits || a.K % BK || a.N % BN) return hipErrorInvalidValue;
    if (EPI == EPI_SWIGLU && a.splits != 1) return hipErrorInvalidValue;
    const int mt = (a.M + BM - 1) / BM, nt = a.N / BN;
    hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, BK, WGM, WGN, NS, EPI>), dim3(mt * nt * a.splits),
                       dim3(WGM * WGN * 64), lds, s, a);
    return hipGetLastError();
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K, int epi) {
    (void)epi;
    return M > 0 && N > 0 && K > 0 && N % 128 == 0 && K % K_ALIGN == 0;
}

// Tile configuration and split-K factor of one projection.  The gate/up
// projection (N = 2*d_ff) has tiles enough for 256 CUs; the others at
// prefill batch sizes do not, so their K range is split 2 or 4 ways when
// that leaves at least 8 (16) k-tiles per split.
GemmPlan gemm_plan(int M, int N, int K, int epi) {
    GemmPlan pl{GEMM_CFG_128x128, 1};
    if (epi == EPI_SWIGLU) {
        if (M >= 256) pl.cfg = GEMM_CFG_256x128;
        return pl;
    }
    const int tiles = ((M + 127) / 128) * (N / 128);
    const int nk = K / 64;
    if (tiles < 256) {
        if (tiles <= 128 && nk % 4 == 0 && nk / 4 >= 16) pl.splits = 4;
        else if (nk % 2 == 0 && nk / 2 >= 8) pl.splits = 2;
    }
    return pl;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t s) {
    if (!gemm_shape_ok(a.M, a.N, a.K, epi)) return hipErrorInvalidValue;
    const GemmPlan pl = gemm_plan(a.M, a.N, a.K, epi);
    GemmArgs g = a;
    g.splits = pl.splits;
    if (g.splits > 1 && !g.P) return hipErrorInvalidValue;
    if (pl.cfg == GEMM_CFG_256x128) {
        switch (epi) {
            case EPI_F32: return launch_tile<256, 128, 64, 4, 2, 2, EPI_F32>(g, s);
            case EPI_RESID: return launch_tile<256, 128, 64, 4, 2, 2, EPI_RESID>(g, s);
            case EPI_SWIGLU: return launch_tile<256, 128, 64, 4, 2, 2, EPI_SWIGLU>(g, s);
        }
    } else {
        switch (epi) {
            case EPI_F32: return launch_tile<128, 128, 64, 4, 2, 2, EPI_F32>(g, s);
            case EPI_RESID: return launch_tile<128, 128, 64, 4, 2, 2, EPI_RESID>(g, s);
            case EPI_SWIGLU: return launch_tile<128, 128, 64, 4, 2, 2, EPI_SWIGLU>(g, s);
        }
    }
    return hipErrorInvalidValue;
}
