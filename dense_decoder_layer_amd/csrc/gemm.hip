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
// Tiling: a 256-thread workgroup computes a BM x BN tile, four waves in a
// 2x2 grid, each wave (BM/2) x (BN/2) of v_mfma_f32_16x16x32_f16 tiles.
// K advances 64 at a time through a double-buffered LDS stage; the 16-byte
// chunks of each LDS row are XOR-swizzled by the row index so the
// fragment reads of 8 consecutive lanes hit distinct banks.
#include "common.h"
#include "internal.h"

namespace {

constexpr int BK = 64;            // halves of K per stage
constexpr int CHUNKS = BK / 8;    // 16-byte chunks per LDS row

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_f16_kernel(GemmArgs p) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int A_LOADS = BM * CHUNKS / 256;
    constexpr int B_LOADS = BN * CHUNKS / 256;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for 256 threads");
    static_assert(EPI != EPI_SWIGLU || (NI % 2) == 0, "swiglu pairs 16-column blocks");
    __shared__ half8 As[2][BM * CHUNKS];
    __shared__ half8 Bs[2][BN * CHUNKS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Tile order: the workgroups of one weight tile (all M tiles of one N
    // tile) are consecutive in the logical order, and the logical order is
    // laid out XCD by XCD (dispatch sends workgroup i to XCD i % 8), so a
    // weight tile is fetched into one XCD's L2 and reused there.
    const int mt = (p.M + BM - 1) / BM, nt = p.N / BN;
    const int total = mt * nt;
    int bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int m0 = (bid % mt) * BM, n0 = (bid / mt) * BN;

    half8 ra[A_LOADS], rb[B_LOADS];
    const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int idx = i * 256 + tid, r = idx / CHUNKS, c = idx % CHUNKS;
            const int row = m0 + r;
            ra[i] = row < p.M
                        ? *reinterpret_cast<const half8*>(p.A + (size_t)row * p.lda + k0 + c * 8)
                        : zero8;
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int idx = i * 256 + tid, r = idx / CHUNKS, c = idx % CHUNKS;
            rb[i] = *reinterpret_cast<const half8*>(p.W + (size_t)(n0 + r) * p.ldw + k0 + c * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int idx = i * 256 + tid, r = idx / CHUNKS, c = idx % CHUNKS;
            As[buf][r * CHUNKS + (c ^ (r & 7))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int idx = i * 256 + tid, r = idx / CHUNKS, c = idx % CHUNKS;
            Bs[buf][r * CHUNKS + (c ^ (r & 7))] = rb[i];
        }
    };

    floatx4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            half8 af[MI], bf[NI];
            const int c = ks * 4 + (lane >> 4);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int r = wm * WM + i * 16 + (lane & 15);
                af[i] = As[cur][r * CHUNKS + (c ^ (r & 7))];
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int r = wn * WN + j * 16 + (lane & 15);
                bf[j] = Bs[cur][r * CHUNKS + (c ^ (r & 7))];
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Accumulator layout of a 16x16 MFMA tile: lane l holds rows
    // 4*(l/16) + e (e = 0..3) of column l % 16.
    const float sc = *p.inv_scale;
    const int rbase = m0 + wm * WM + 4 * (lane >> 4);
    const int cbase = n0 + wn * WN + (lane & 15);
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; j += 2) {
                const int fcol = ((n0 + wn * WN + j * 16) >> 5) * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = rbase + i * 16 + e;
                    if (row < p.M) {
                        const float g = acc[i][j][e] * sc, u = acc[i][j + 1][e] * sc;
                        p.H[(size_t)row * p.ldh + fcol] = (f16)(g / (1.0f + expf(-g)) * u);
                    }
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = rbase + i * 16 + e, col = cbase + j * 16;
                    if (row < p.M) {
                        float v = acc[i][j][e] * sc;
                        if constexpr (EPI == EPI_RESID) v += p.R[(size_t)row * p.ldr + col];
                        p.C[(size_t)row * p.ldc + col] = v;
                    }
                }
    }
}

template <int BM, int BN, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    const int mt = (a.M + BM - 1) / BM, nt = a.N / BN;
    hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, EPI>), dim3(mt * nt), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K, int epi) {
    (void)epi;
    return M > 0 && N > 0 && K > 0 && N % 128 == 0 && K % BK == 0;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t s) {
    if (!gemm_shape_ok(a.M, a.N, a.K, epi)) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_F32: return launch_tile<128, 128, EPI_F32>(a, s);
        case EPI_RESID: return launch_tile<128, 128, EPI_RESID>(a, s);
        case EPI_SWIGLU: return launch_tile<128, 128, EPI_SWIGLU>(a, s);
    }
    return hipErrorInvalidValue;
}
