// Time-parallel input projection of one layer, both directions in one GEMM, on gfx950 FP32
// MFMA (speakrs 0.6.0, page `lstmproj.rs`: module doc, `InputProjection::enqueue` — x·Wᵀ
// for all steps at once, with W's gate rows permuted per hidden unit).
//
//   gates[m][n] = bias[n] + sum_k x[m][k] · w[n][k]      m < rows, n < 1024, k < in
//
// x is row-major [rows][in] (in = 60 or 256, rows = windows·steps), w the packed weights
// [1024][kpad] (row d·512 + 4j + g, zero padded to kpad), bias [1024] = Wb + Rb.
//
// Design for CDNA4:
//  * 128x128 output tile per 256-thread workgroup, 4 waves of 64x64, each a 4x4 grid of
//    v_mfma_f32_16x16x4_f32 tiles (FP32 in, FP32 accumulate).
//  * K steps of 32 staged through LDS, double buffered. Both operands are stored K-major per
//    row with a 36-float stride, so a ds_read_b128 of 8 consecutive rows touches 32 distinct
//    banks.
//  * Inside one MFMA the K slots are permuted: lane group g (lanes 16g..16g+15) supplies
//    k = k0 + 4g + e in the e-th of four consecutive MFMAs, so each lane fetches four
//    consecutive K values of its row with one ds_read_b128. A and B use the same
//    permutation, so the product is unchanged.
//  * Workgroup ids are remapped so each XCD (ids congruent mod 8) runs a contiguous run of
//    tiles: the eight column tiles of a row block share that XCD's L2 for their A rows.
//  * The per-row K order is fixed and independent of the row's position, so a row's gates
//    are bitwise the same whatever the batch.
#include "bilstm_internal.h"

namespace bl {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = kProjTileM;
constexpr int BN = kProjTileN;
constexpr int BK = kProjTileK;
constexpr int kStride = BK + 4;                    // LDS row stride, floats
constexpr int kLoadsPerThread = BM * BK / 4 / kProjThreads;  // float4 per operand per thread

static_assert(BM == 128 && BN == 128 && BK == 32 && kProjThreads == 256, "tile shape");
static_assert(kLoadsPerThread == 4, "loads per thread");

__global__ __launch_bounds__(kProjThreads) void projection_kernel(ProjArgs a) {
    __shared__ __attribute__((aligned(16))) float lds_a[2][BM * kStride];
    __shared__ __attribute__((aligned(16))) float lds_b[2][BN * kStride];

    const int nwg = gridDim.x;  // a multiple of 8
    const int wg = blockIdx.x;
    const int tile = (wg & 7) * (nwg >> 3) + (wg >> 3);
    if (tile >= a.tiles) return;
    constexpr int kColTiles = kGateCols / BN;
    const int m0 = (tile / kColTiles) * BM;
    const int n0 = (tile % kColTiles) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    v4f ra[kLoadsPerThread], rb[kLoadsPerThread];

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int j = 0; j < kLoadsPerThread; ++j) {
            const int f = tid + kProjThreads * j;
            const int row = f >> 3;
            const int k = k0 + (f & 7) * 4;
            const int m = m0 + row;
            v4f va = {0.f, 0.f, 0.f, 0.f};
            if (m < a.rows && k < a.in) {
                va = *reinterpret_cast<const v4f *>(a.x + static_cast<size_t>(m) * a.in + k);
            }
            ra[j] = va;
            rb[j] = *reinterpret_cast<const v4f *>(a.w + static_cast<size_t>(n0 + row) * a.kpad + k);
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kLoadsPerThread; ++j) {
            const int f = tid + kProjThreads * j;
            const int row = f >> 3;
            const int c = (f & 7) * 4;
            *reinterpret_cast<v4f *>(&lds_a[buf][row * kStride + c]) = ra[j];
            *reinterpret_cast<v4f *>(&lds_b[buf][row * kStride + c]) = rb[j];
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int ksteps = a.kpad / BK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    const int frag_row = lane & 15;
    const int frag_k = (lane >> 4) * 4;
    for (int kt = 0; kt < ksteps; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < ksteps) load_tiles((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            v4f af[4], bf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[t] = *reinterpret_cast<const v4f *>(
                    &lds_a[cur][(wm * 64 + t * 16 + frag_row) * kStride + ks * 16 + frag_k]);
                bf[t] = *reinterpret_cast<const v4f *>(
                    &lds_b[cur][(wn * 64 + t * 16 + frag_row) * kStride + ks * 16 + frag_k]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 4; ++tj)
                        acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[ti][e], bf[tj][e],
                                                                          acc[ti][tj], 0, 0, 0);
        }
        if (kt + 1 < ksteps) store_tiles(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: lane l of a 16x16 MFMA tile holds rows 4·(l/16) + r, r = 0..3, column l % 16.
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
        const int n = n0 + wn * 64 + tj * 16 + (lane & 15);
        const float bv = a.bias[n];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + ti * 16 + (lane >> 4) * 4 + r;
                if (m < a.rows) a.gates[static_cast<size_t>(m) * kGateCols + n] = acc[ti][tj][r] + bv;
            }
        }
    }
}

}  // namespace

hipError_t launch_projection(const ProjArgs &args, hipStream_t stream) {
    if (args.tiles <= 0) return hipSuccess;
    const int nwg = (args.tiles + 7) / 8 * 8;
    hipLaunchKernelGGL(projection_kernel, dim3(nwg), dim3(kProjThreads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace bl
