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
//  * Persistent: 256-thread workgroups walk the 128x128 output tiles q = wq, wq + grid, ...,
//    one or two per CU (190 VGPRs, 72 KB of LDS each), whichever takes fewer tile rounds at
//    the measured rates: two on a CU finish a round of two tiles in about 1.87 times a lone
//    workgroup's tile time, so two win unless the last round is mostly empty. The walk is XCD-ordered: the
//    ids congruent mod 8 run on one XCD, and the workgroups of one XCD take consecutive tiles,
//    so the eight column tiles of a row block are computed on the same XCD and share its L2
//    for their x rows.
//  * Four waves of 64x64, each a 2x2 grid of v_mfma_f32_32x32x2_f32 blocks (FP32 in, FP32
//    accumulate in AGPRs). The 32x32x2 form keeps the matrix pipe busy with one wave per SIMD
//    and few independent accumulators (measured 147 TFLOP/s in a pure MFMA loop).
//  * K steps of 32 staged through LDS, double buffered, with a 36-float row stride
//    (conflict-free ds_read_b128). Inside an MFMA group of four, lane half h supplies
//    k = k0 + 4h + e in the e-th MFMA, so every lane fetches four consecutive K values of its
//    row with one ds_read_b128; A and B use the same permutation, so the product is unchanged.
//    Fragments of the next group are read while the current group's MFMAs run.
//  * The next tile's first K step is loaded during the current tile's last one.
//  * Output: a finished tile's sums (plus bias) go straight to memory; with two workgroups on
//    a CU the other one's products fill the matrix pipe meanwhile. (Holding the sums until the
//    next tile's K steps, to overlap the stores with one workgroup per CU, measured slower.)
//    In the 32x32 output layout one store instruction writes two full 128-byte row segments.
//  * Every row's K order is fixed and independent of the row's position and of the grid, so a
//    row's gates are bitwise the same whatever the batch, the number of workgroups or the
//    tile order. (Layers with 256 inputs: reverse-direction columns sum the reverse half of K
//    first, kstep_at.)
//  * Streamed order (projection_stream_kernel): the recurrences run at the same time on
//    other CUs, this layer's reading the gates step by step and the previous layer's still
//    writing this layer's input. Tiles then cover `group_windows` windows × `chunk`
//    consecutive recurrence steps of one direction, numbered in the order the recurrence reads
//    them; beside the previous layer, a workgroup with several tiles first walks down from the
//    chunks whose rows exist first (the middle ones), then takes the rest in that order
//    (protocol.h). Each tile waits for each K half of its rows before summing it, is computed on its own,
//    stored with agent-scope stores and, once those have completed, published by one counter
//    increment. Its K steps go from memory straight into a 4-stage LDS ring (buffer loads with
//    the LDS bit, rows swizzled instead of padded), three steps ahead of the products, with
//    explicit counter waits and bare barriers.
#include <algorithm>
#include <vector>
#include <type_traits>

#include "bilstm_internal.h"

namespace bl {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Raw buffer resource, word 3 of the descriptor for the gfx9 family (no format conversion),
// and the cache-policy bit of an agent-scope (sc1) access.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCachePolicySc1 = 16;
constexpr unsigned int kOutOfRange = 0x80000000u;  // a buffer offset past every buffer here


constexpr int BM = kProjTileM;
constexpr int BN = kProjTileN;
constexpr int BK = kProjTileK;
constexpr int kStride = BK + 4;                              // LDS row stride, floats
constexpr int kThreadsPerRow = BK / 4;                       // float4 loads along K per row
constexpr int kLoadsPerThread = BM * BK / 4 / kProjThreads;  // float4 per operand per thread
constexpr int kGroups = BK / 8;                              // MFMA groups (K = 8 each) per K step

static_assert(BM == 128 && BN == 128 && BK == 32 && kProjThreads == 256, "tile shape");
static_assert(kLoadsPerThread == 4, "loads per thread");
static_assert(2 * 2 * BM * kStride * sizeof(float) == kProjLdsBytes, "LDS size");

// K step taken at position kt of a tile whose first gate column is n0. A layer after the
// first reads the previous layer's output, forward h in k < 128 and reverse h in k >= 128;
// its reverse-direction columns sum the reverse half first. For the rows of a reverse chunk
// that is the half the previous layer finishes first (its reverse direction reaches late times
// early), as the forward half is for a forward chunk, so the streamed order can sum the first
// half before the second exists.
template <int KSTEPS>
__device__ __forceinline__ int kstep_at(int n0, int kt) {
    if constexpr (KSTEPS * BK == kWidth) {
        return n0 >= kGates ? (kt + KSTEPS / 2) % KSTEPS : kt;
    } else {
        return kt;
    }
}

template <int KSTEPS>
__global__ __launch_bounds__(kProjThreads, 2) void projection_kernel(ProjArgs a) {
    __shared__ __attribute__((aligned(16))) float lds_a[2][BM * kStride];
    __shared__ __attribute__((aligned(16))) float lds_b[2][BN * kStride];

    const int nwg = gridDim.x;  // a multiple of 8
    const int per_xcd = nwg >> 3;
    const int first = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    constexpr int kColTiles = kGateCols / BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    // ---- global -> registers -> LDS staging of one K step -----------------------------------
    v4f ra[kLoadsPerThread], rb[kLoadsPerThread];
    auto load = [&](int m0, int n0, int k0) {
#pragma unroll
        for (int j = 0; j < kLoadsPerThread; ++j) {
            const int f = tid + kProjThreads * j;
            const int row = f / kThreadsPerRow;
            const int k = k0 + (f % kThreadsPerRow) * 4;
            const int m = m0 + row;
            v4f va = {0.f, 0.f, 0.f, 0.f};
            if (m < a.rows && k < a.in) {
                va = *reinterpret_cast<const v4f *>(a.x + static_cast<size_t>(m) * a.in + k);
            }
            ra[j] = va;
            rb[j] = *reinterpret_cast<const v4f *>(a.w + static_cast<size_t>(n0 + row) * a.kpad + k);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kLoadsPerThread; ++j) {
            const int f = tid + kProjThreads * j;
            const int off = (f / kThreadsPerRow) * kStride + (f % kThreadsPerRow) * 4;
            *reinterpret_cast<v4f *>(&lds_a[buf][off]) = ra[j];
            *reinterpret_cast<v4f *>(&lds_b[buf][off]) = rb[j];
        }
    };

    // ---- MFMA fragments: lane l holds row l % 32 of a 32-row block, K quarter 4·(l / 32) ----
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 4;
    auto frags = [&](int buf, int g, v4f (&af)[2], v4f (&bf)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            af[t] = *reinterpret_cast<const v4f *>(
                &lds_a[buf][(wm * 64 + t * 32 + frag_row) * kStride + g * 8 + frag_k]);
            bf[t] = *reinterpret_cast<const v4f *>(
                &lds_b[buf][(wn * 64 + t * 32 + frag_row) * kStride + g * 8 + frag_k]);
        }
    };

    // ---- a finished tile's sums plus bias to the gates (in the 32x32 output layout register r
    // of lane l is row 8·(r / 4) + 4·(l / 32) + r % 4, column l % 32 of the block; one store
    // instruction writes two full 128-byte row segments). The other workgroup on the CU
    // multiplies meanwhile.
    auto finish = [&](int m0, int n0, const v16f (&acc)[2][2]) {
        auto put = [&](auto full_tag) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + wn * 64 + j * 32 + (lane & 31);
                const float bv = a.bias[n];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                        if (decltype(full_tag)::value || m < a.rows) {
                            a.gates[static_cast<size_t>(m) * kGateCols + n] = acc[i][j][r] + bv;
                        }
                    }
            }
        };
        if (m0 + BM <= a.rows) {
            put(std::true_type{});
        } else {
            put(std::false_type{});
        }
    };

    int q = first;
    int base = 0;  // LDS buffer of the tile's first K step
    if (q < a.tiles) {
        const int n0 = (q % kColTiles) * BN;
        load((q / kColTiles) * BM, n0, kstep_at<KSTEPS>(n0, 0) * BK);
        store(0);
    }
    __syncthreads();
    v4f af[2][2], bf[2][2];
    frags(0, 0, af[0], bf[0]);

    for (; q < a.tiles; q += nwg) {
        const int m0 = (q / kColTiles) * BM;
        const int n0 = (q % kColTiles) * BN;
        const int qn = q + nwg;
        const bool next = qn < a.tiles;

        v16f acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
        for (int kt = 0; kt < KSTEPS; ++kt) {
            const int cur = (base + kt) & 1;
            const bool more = kt + 1 < KSTEPS;
            // the next K step of this tile, or the first K step of the next tile
            if (more) {
                load(m0, n0, kstep_at<KSTEPS>(n0, kt + 1) * BK);
            } else if (next) {
                const int nn = (qn % kColTiles) * BN;
                load((qn / kColTiles) * BM, nn, kstep_at<KSTEPS>(nn, 0) * BK);
            }
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                const int p = g & 1;
                if (g + 1 < kGroups) frags(cur, g + 1, af[p ^ 1], bf[p ^ 1]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[p][i][e], bf[p][j][e],
                                                                             acc[i][j], 0, 0, 0);
            }
            if (more || next) store(cur ^ 1);
            __syncthreads();
            if (more || next) frags(cur ^ 1, 0, af[0], bf[0]);
        }

        finish(m0, n0, acc);
        base = (base + KSTEPS) & 1;
    }
}


// ---- split-precision variant ---------------------------------------------------------------
//
// The same projection with every FP32 operand split into bf16 parts and the products of the
// parts accumulated in FP32 on the bf16 matrix cores (a bf16 x bf16 product is exact in FP32).
// Each part is the round-to-nearest-even bf16 of what the earlier parts leave: a_0 = bf16(a),
// a_1 = bf16(a - a_0), a_2 = bf16(a - a_0 - a_1) (each difference is exact in FP32), and each
// part removes all but 2^-8 of the remainder, so after P parts |a - sum a_p| <= 2^-8P·|a|.
//   PARTS = 2: three products per K chunk, a_0·b_0 + a_0·b_1 + a_1·b_0 (the dropped a_1·b_1 and
//     the residuals stay below 3·2^-16·|a·b|):
//     |gates - exact| <= (3·2^-16·(1 + 2^-7) + (3K + 2)·2^-24) · sum_k |x_k w_k|;
//   PARTS = 3: six products, every a_p·b_q with p + q <= 2 (the dropped a_1·b_2, a_2·b_1,
//     a_2·b_2 and the residuals stay below 4·2^-24·|a·b|(1 + 2^-7)): the truncation is then
//     of the order of one FP32 rounding per product,
//     |gates - exact| <= (4·2^-24·(1 + 2^-7) + (6K + 2)·2^-24) · sum_k |x_k w_k|.
// W arrives already split (PARTS [1024][kpad] bf16 planes, packed at plan creation); x is
// split in registers on its way into LDS. v_mfma_f32_32x32x16_bf16: lane l supplies row (or
// column) l % 32 and eight consecutive k of half l / 32 of a 16-wide K chunk, for A and B alike.
//
// Layout for gfx950: two 256-thread workgroups per CU (each wave shares its SIMD with a wave of
// the other workgroup, which issues its matrix products while this one splits, waits or
// stores), each walking 128x128 tiles like projection_kernel. A stage of the LDS ring is one
// 16-wide K chunk: PARTS planes of x and PARTS planes of W, 128 rows of 32 bytes each, the two
// 16-byte halves of row r stored in swapped order when bit 2 xor bit 3 of r is set: a
// fragment read serves 16 lanes (16 consecutive rows, one half) per LDS cycle over 64 banks,
// and those 16 halves then fill the 256 bytes once (with bit 2 alone, rows r and r + 8 met on
// the same banks: two cycles per 16 lanes, measured as bank conflicts). Three stages: the W
// planes of the chunk two ahead go from memory straight into LDS (buffer loads with the LDS
// bit, no registers); the x rows go into registers four chunks ahead (their first read comes
// from memory, not L2), and the x rows of the next chunk are split into their parts and
// written to LDS while the matrix products of the current chunk run. The stage walk runs on
// across tiles, so a tile's first chunks are loaded during the previous tile's last ones.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSplitThreads = 256;
constexpr int kSplitStages = 3;
constexpr int kSplitPlane = BM * 16;  // bf16 elements of one plane of one stage

// bf16 element offset, within a plane, of the 16-byte half h of row r
__device__ __forceinline__ int split_half(int r, int h) { return h ^ ((r >> 2) & 1) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int split_slot(int r, int h) { return r * 16 + (split_half(r, h) << 3); }

// Wait until at most n of this wave's vector memory operations are outstanding (n <= 7; any
// other n waits for all of them).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
        case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// Stage s of a split-kernel workgroup's walk: its tile's first row and gate column and its K
// offset. The workgroup's tiles are first, first + nwg, ...; a stage past its last one gives a
// tile past the last tile, which has no rows.
struct SplitStage {
    int m0, n0, k0;
};
template <int KSTEPS>
__device__ __forceinline__ SplitStage split_stage(int s, int first, int nwg) {
    constexpr int NC = 2 * KSTEPS;
    const int q = first + (s / NC) * nwg;
    const int j = s % NC;
    SplitStage t;
    t.m0 = (q / (kGateCols / BN)) * BM;
    t.n0 = (q % (kGateCols / BN)) * BN;
    t.k0 = kstep_at<KSTEPS>(t.n0, j >> 1) * BK + (j & 1) * 16;
    return t;
}

template <int KSTEPS, int PARTS>
__global__ __launch_bounds__(kSplitThreads, 2) void projection_split_kernel(ProjArgs a) {
    static_assert(PARTS == 2 || PARTS == 3, "two or three bf16 parts");
    constexpr int NC = 2 * KSTEPS;                      // 16-wide K chunks per tile
    constexpr int kStage = 2 * PARTS * kSplitPlane;     // x planes, then W planes
    constexpr bool kMaskK = KSTEPS * BK != kWidth;      // layer 0: k past the 60 inputs reads 0
    // one LDS array (the ring, then the bias): with a second one the compiler waits for every
    // LDS-bound load before each ring read, as it then tells the arrays apart but not the slots.
    // At least kProjLdsBytes (two parts need less): a recurrence workgroup's LDS reservation
    // keeps any projection workgroup of that size off its CU.
    constexpr int kRingElems = kSplitStages * kStage + 2 * kGateCols;
    constexpr int kLdsElems = kRingElems * 2 >= static_cast<int>(kProjLdsBytes) ? kRingElems
                                                                               : static_cast<int>(kProjLdsBytes) / 2;
    __shared__ __attribute__((aligned(16))) __bf16 ring[kLdsElems];
    float *const sbias = reinterpret_cast<float *>(ring + kSplitStages * kStage);

    const int nwg = gridDim.x;  // a multiple of 8
    const int per_xcd = nwg >> 3;
    const int first = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    constexpr int kColTiles = kGateCols / BN;
    const int my_tiles = first < a.tiles ? (a.tiles - first + nwg - 1) / nwg : 0;
    const int stages = my_tiles * NC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    // W: each wave fills 32 rows of each plane, lane i the 16-byte slot i % 2 of row i / 2
    const int wrow = wave * 32 + (lane >> 1);
    const unsigned int wlane = (static_cast<unsigned int>(wrow) * a.kpad + 8 * split_half(wrow, lane & 1)) * 2u;
    // x: this thread's two float4 of a stage, rows tid / 4 and tid / 4 + 64, k = 4·(tid % 4)
    const int xq = tid & 3;
    const int xrow = tid >> 2;

    // stage s's W planes into ring stage `slot` (from L2: W is small and read by every tile)
    auto issue_w = [&](int s, int slot) {
        const SplitStage t = split_stage<KSTEPS>(s, first, nwg);
        __bf16 *const sb = ring + slot * kStage + PARTS * kSplitPlane + wave * 512;
#pragma unroll
        for (int p = 0; p < PARTS; ++p) {
            // (the descriptor is made here: an array of descriptors, or a helper producing one,
            // keeps the host pass from emitting the kernel's launch stub)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16 *>(p == 0 ? a.w_hi : (p == 1 ? a.w_lo : a.w_lo2)), 0,
                                                  kGateCols * a.kpad * 2, kBufferRsrcWord3),
                sb + p * kSplitPlane, 16, wlane + static_cast<unsigned int>(t.n0) * a.kpad * 2u, t.k0 * 2, 0, 0);
        }
    };
    // stage s's x rows into registers (from memory the first time a row block is read: these go
    // out four stages ahead). Rows past the last one read zeros (the buffer ends at the tile's
    // last row), and so does every stage past the workgroup's last one, which keeps the number
    // of memory operations between two waits the same on every path.
    auto issue_x = [&](int s, v4f (&xv)[2]) {
        const SplitStage t = split_stage<KSTEPS>(s, first, nwg);
        // (uniform; readfirstlane keeps the clamp, which has no scalar form, off the vector
        // registers, so the descriptor stays scalar)
        const int rows = __builtin_amdgcn_readfirstlane(max(0, min(BM, a.rows - t.m0)));
        const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.x + static_cast<size_t>(t.m0) * a.in), 0, rows * a.in * 4, kBufferRsrcWord3);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const unsigned int off = (static_cast<unsigned int>(xrow + 64 * i) * a.in + t.k0 + 4 * xq) * 4u;
            const bool in_k = !kMaskK || t.k0 + 4 * xq < a.in;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrsrc, in_k ? off : kOutOfRange, 0, 0);
            xv[i] = __builtin_bit_cast(v4f, v);
        }
    };
    // x rows of a stage, split into their parts (two values per packed conversion, as split8),
    // into ring stage `slot`
    auto put_x = [&](int slot, const v4f (&xv)[2]) {
        __bf16 *const sa = ring + slot * kStage;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = xrow + 64 * i;
            const int off = split_slot(r, xq >> 1) + (xq & 1) * 4;
            bf16x4 part[PARTS];
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                float ra = xv[i][e];
                float rb = xv[i][e + 1];
#pragma unroll
                for (int p = 0; p < PARTS; ++p) {
                    const bf16x2 pk = __builtin_convertvector(f32x2{ra, rb}, bf16x2);
                    part[p][e] = pk[0];
                    part[p][e + 1] = pk[1];
                    if (p + 1 < PARTS) {
                        const unsigned int u = __builtin_bit_cast(unsigned int, pk);
                        ra -= __builtin_bit_cast(float, u << 16);          // exact
                        rb -= __builtin_bit_cast(float, u & 0xFFFF0000u);  // exact
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < PARTS; ++p) *reinterpret_cast<bf16x4 *>(sa + p * kSplitPlane + off) = part[p];
        }
    };

    const int fr = lane & 31;
    const int flane = split_slot(fr, lane >> 5);  // rows of a block start at multiples of 32
    v16f acc[2][2];
    auto zero = [&] {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    };
    // the six (three) products of the parts of one chunk, in the order every split kernel uses
    auto products = [&](int slot) {
        const __bf16 *const sa = ring + slot * kStage;
        const __bf16 *const sb = sa + PARTS * kSplitPlane;
        bf16x8 af[PARTS][2], bf[PARTS][2];
#pragma unroll
        for (int p = 0; p < PARTS; ++p)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[p][t] = *reinterpret_cast<const bf16x8 *>(sa + p * kSplitPlane + (wm * 64 + t * 32) * 16 + flane);
                bf[p][t] = *reinterpret_cast<const bf16x8 *>(sb + p * kSplitPlane + (wn * 64 + t * 32) * 16 + flane);
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][i], bf[0][j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][i], bf[1][j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1][i], bf[0][j], acc[i][j], 0, 0, 0);
                if constexpr (PARTS == 3) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1][i], bf[1][j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][i], bf[2][j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[2][i], bf[0][j], acc[i][j], 0, 0, 0);
                }
            }
    };
    // A finished tile: sums plus bias to the gates. The buffer ends at the tile's last row, so
    // rows past the last one are not written; the row and column offsets of an element are a
    // per-lane base plus a constant (in the 32x32 output layout one store instruction writes two
    // full 128-byte row segments).
    auto finish = [&](int s) {
        const int q = first + (s / NC) * nwg;
        const int m0 = (q / kColTiles) * BM;
        const int n0 = (q % kColTiles) * BN;
        const int rows = __builtin_amdgcn_readfirstlane(max(0, min(BM, a.rows - m0)));
        const __amdgpu_buffer_rsrc_t grsrc = __builtin_amdgcn_make_buffer_rsrc(
            a.gates + static_cast<size_t>(m0) * kGateCols, 0, rows * kGateCols * 4, kBufferRsrcWord3);
        const int col = n0 + wn * 64 + fr;
        const unsigned int goff = static_cast<unsigned int>((wm * 64 + (lane >> 5) * 4) * kGateCols + col) * 4u;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float bv = sbias[col + j * 32];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, acc[i][j][r] + bv), grsrc,
                                                          goff,
                                                          ((i * 32 + (r >> 2) * 8 + (r & 3)) * kGateCols + j * 32) * 4,
                                                          0);
                }
        }
        zero();
    };
    // Stage s: issue stage s + 2's W and stage s + 4's x (into the registers stage s's x left),
    // the products of stage s, then stage s + 1's x into LDS; the barrier at the end makes stage
    // s + 1 whole (every wave's W loads landed, every wave's x written) and frees stage s's slot.
    // Per stage the loads go out in the order W(s + 2), x(s + 4), so when stage s + 1's W and x
    // have landed, only x(s + 3), W(s + 2) and x(s + 4) may still be in flight. The stages past
    // the last one load into slots nobody reads again (x as zeros, W rows in bounds).
    constexpr int kAfter = PARTS + 4;
    auto step = [&](int s, v4f (&x_next)[2], v4f (&x_far)[2]) {
        issue_w(s + 2, (s + 2) % kSplitStages);
        issue_x(s + 4, x_far);
        products(s % kSplitStages);
        wait_vm(kAfter);
        put_x((s + 1) % kSplitStages, x_next);
        if (s % NC == NC - 1) finish(s);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0: the x parts are in LDS
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if (stages == 0) return;
    for (int n = tid; n < kGateCols; n += kSplitThreads) sbias[n] = a.bias[n];
    zero();
    // the loads of stages 0 and 1 in the steady order (x(0) and x(1) first)
    v4f x0[2], x1[2], x2[2], x3[2];
    issue_x(0, x0);
    issue_x(1, x1);
    issue_w(0, 0);
    issue_x(2, x2);
    issue_w(1, 1);
    issue_x(3, x3);
    wait_vm(kAfter);
    put_x(0, x0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // stage s's x is in register set s % 4, as stage s + 4's will be. A tile has a multiple of
    // four stages, so stages is one too.
    for (int s = 0; s < stages; s += 4) {
        step(s, x1, x0);
        step(s + 1, x2, x1);
        step(s + 2, x3, x2);
        step(s + 3, x0, x3);
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(0x0F70);
}


// ---- streamed order ------------------------------------------------------------------------
//
// The same MFMA blocks as projection_kernel over the streamed row blocks (StreamLayout in the
// internal header). A tile's first K steps are loaded once its first half exists (during the
// previous tile's last K steps if it already does), its second half once that exists, and its
// outputs are stored and published as soon as its K loop ends, so no finished tile waits
// behind the inputs of the next one. Every row sums its K terms in the same order as
// projection_kernel, so the gates are bitwise the same.

// Row block of streamed tile q: first window, first step, chunk, direction, first gate
// column, width in gate columns and publication counter.
struct StreamTile {
    int w0, s0, c, dir, n0, width, counter;
};

// The tiles of chunk 0 come first, `split` of them per 128 gate columns: narrower tiles spread
// the first chunk after a layer boundary over more workgroups. The other chunks follow in
// 128-column tiles.
__device__ __forceinline__ StreamTile stream_tile(const ProjArgs &a, int q) {
    const int first_tiles = 2 * a.groups * (kGates / BN) * a.split;
    int ct, rest, id, width;
    if (q < first_tiles) {
        const int per = (kGates / BN) * a.split;
        ct = q % per;
        rest = q / per;
        width = BN / a.split;
        id = rest / a.groups;  // direction
    } else {
        const int r = q - first_tiles;
        ct = r & 3;
        rest = r >> 2;
        width = BN;
        id = rest / a.groups + 2;  // chunk · 2 + direction
    }
    const int g = rest % a.groups;
    StreamTile t;
    t.dir = id & 1;
    t.c = id >> 1;
    t.w0 = g * a.group_windows;
    t.s0 = t.c * a.chunk;
    t.n0 = t.dir * kGates + ct * width;
    t.width = width;
    t.counter = (t.c * 2 + t.dir) * a.groups + g;
    return t;
}

// Gate row of local row r of a streamed tile, or -1 when r falls past the batch or the steps.
__device__ __forceinline__ int stream_row(const ProjArgs &a, const StreamTile &t, int r) {
    const int w = t.w0 + (r >> a.chunk_shift);
    const int s = t.s0 + (r & (a.chunk - 1));
    if (w >= a.batch || s >= a.steps) return -1;
    return w * a.steps + (t.dir == 0 ? s : a.steps - 1 - s);
}

// Inputs written by the previous layer's recurrence during this kernel: a K half of a tile's
// rows exists once the direction that writes it has published enough steps for each of the
// tile's windows. Lane 2i + d of a wave watches window w0 + i, direction d (the other lanes
// watch nothing); the tile's first half is written by direction t.dir (kstep_at).
__device__ __forceinline__ const unsigned long long *watched_word(const ProjArgs &a, const StreamTile &t, int lane) {
    const int w = t.w0 + (lane >> 1);
    if (a.progress == nullptr || lane >= 2 * a.group_windows || w >= a.batch) return nullptr;
    return a.progress + kProgressStride * (2 * w + (lane & 1));
}

// Whether this lane's word, `seen`, lets the first (second) half of the tile's rows be read.
__device__ __forceinline__ bool half_ready(const ProjArgs &a, const StreamTile &t, int lane, unsigned long long seen,
                                          bool first) {
    if (watched_word(a, t, lane) == nullptr || ((lane & 1) == t.dir) != first) return true;
    const int need = first ? stream_near(a.steps, a.chunk, t.c) : stream_far(a.steps, a.chunk, t.c);
    return progress_reached(seen, a.progress_pass, static_cast<uint32_t>(need));
}

// Wait until the first (second) half of the tile's rows exists; the wave goes on when all its
// lanes have seen it.
__device__ __forceinline__ void wait_half(const ProjArgs &a, const StreamTile &t, int lane, bool first,
                                          bool &timed_out) {
    const unsigned long long *p = watched_word(a, t, lane);
    if (p == nullptr || timed_out || ((lane & 1) == t.dir) != first) return;
    if (half_ready(a, t, lane, __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), first)) return;
    const unsigned long long t0 = wall_clock64();
    while (true) {
        __builtin_amdgcn_s_sleep(2);
        if (half_ready(a, t, lane, __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), first)) break;
        if (wall_clock64() - t0 > a.timeout_ticks) {
            report_timeout(a.error, kErrProgress);
            timed_out = true;
            break;
        }
    }
}

template <int TN>
struct TileWidth {
    static constexpr int value = TN;
};

// LDS staging of the streamed kernel. A K step of a tile is 128 rows of x and 128 rows of W,
// 32 floats each, written from memory straight into LDS by buffer loads with the LDS bit, so
// no registers hold them on the way and four K steps can be in flight. Row r's eight 16-byte
// chunks are stored swizzled, chunk c in slot c ^ ((r >> 1) & 7): the 32 rows one fragment
// read touches then fall on distinct banks without padding. One wave instruction fills 8 rows
// (64 lanes x 16 bytes, lane i in slot i % 8 of row 8n + i / 8), so lane i fetches chunk
// (i % 8) ^ ((row >> 1) & 7) of its row. An out-of-range offset loads zeros (rows past the
// batch or the steps, k past the input width, W rows past the last gate).
constexpr int kStages = 4;                        // K steps in the LDS ring
constexpr int kStageFloats = 2 * BM * BK;         // x rows, then W rows

__device__ __forceinline__ int swizzled(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 2); }

// Wait until at most 8·n of this wave's vector memory operations are outstanding (n = K steps
// issued after the one waited for, each 8 loads per wave, and nothing else issued since).
// They complete in issue order. s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8] (7 and 15 = no wait).
__device__ __forceinline__ void wait_steps_after(int n) {
    n *= 8;
    if (n >= 24) {
        __builtin_amdgcn_s_waitcnt(0x4F78);  // vmcnt 24
    } else if (n >= 16) {
        __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt 16
    } else if (n >= 8) {
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt 8
    } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
    }
}

// Eight consecutive FP32 values (two LDS chunks) split into PARTS bf16 parts, each the bf16 of
// what the earlier parts leave: the same parts the plain split kernel and the plan produce.
// Two values at a time: one packed conversion per pair and part, and the part back in FP32
// from its bits (a shift for the low half, a mask for the high one). Converting one value at a
// time and packing the parts afterwards took a third more VALU operations, and the streamed
// three-part projection 12 % longer.
template <int PARTS>
__device__ __forceinline__ void split8(v4f lo, v4f hi, bf16x8 (&out)[PARTS]) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        float ra = e < 4 ? lo[e] : hi[e - 4];
        float rb = e < 4 ? lo[e + 1] : hi[e - 3];
#pragma unroll
        for (int pl = 0; pl < PARTS; ++pl) {
            const bf16x2 p = __builtin_convertvector(f32x2{ra, rb}, bf16x2);
            out[pl][e] = p[0];
            out[pl][e + 1] = p[1];
            if (pl + 1 < PARTS) {
                const unsigned int u = __builtin_bit_cast(unsigned int, p);
                ra -= __builtin_bit_cast(float, u << 16);          // exact
                rb -= __builtin_bit_cast(float, u & 0xFFFF0000u);  // exact
            }
        }
    }
}

// PARTS = 0: FP32 MFMA products; 2 or 3: split precision as projection_split_kernel, the
// FP32 operands split in registers after the LDS ring.
template <int KSTEPS, int PARTS>
__global__ __launch_bounds__(kProjThreads, 1) void projection_stream_kernel(ProjArgs a, unsigned int lead0) {
    // The K-step ring, then thread 0's walk state and the two tiles it chose for the whole
    // workgroup. One LDS object: with a second one the compiler no longer tells the ring's
    // fragment reads from the loads still writing later stages and waits for all of them.
    constexpr int kWalkFloats = 16;
    static_assert(sizeof(StreamWalk) <= 12 * sizeof(float) && alignof(StreamWalk) <= sizeof(float), "walk state");
    __shared__ __attribute__((aligned(16))) float lds[kStages * kStageFloats + kWalkFloats];
    StreamWalk &walk_state = *reinterpret_cast<StreamWalk *>(&lds[kStages * kStageFloats]);
    int *const order_slot = reinterpret_cast<int *>(&lds[kStages * kStageFloats + 12]);
    // K steps loaded ahead of the one being multiplied
    constexpr int LA = KSTEPS > kStages - 1 ? kStages - 1 : KSTEPS;
    constexpr int kHalf = KSTEPS / 2;
    constexpr bool kHalves = KSTEPS * BK == kWidth;  // inputs written by the previous layer

    const int nwg = gridDim.x;  // a multiple of 8
    const int per_xcd = nwg >> 3;
    const int first = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Inputs written while this kernel runs are read with agent-scope (sc1) loads.
    const bool coherent = a.progress != nullptr;
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.x), 0, static_cast<int>(static_cast<unsigned int>(a.steps) * a.batch * a.in * 4),
        kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.w), 0, kGateCols * a.kpad * 4, kBufferRsrcWord3);

    // this lane's row and chunk in each of its four load instructions per operand
    int lrow[4], lchunk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lrow[i] = wave * 32 + 8 * i + (lane >> 3);
        lchunk[i] = (lane & 7) ^ ((lrow[i] >> 1) & 7);
    }
    // byte offsets of those rows' chunks at K = 0 in x and W for the current and the next tile
    // (the K offset goes in the scalar offset of each load)
    unsigned int xoff[4], woff[4], xoff_next[4], woff_next[4];
    auto offsets_of = [&](const StreamTile &t, unsigned int (&xo)[4], unsigned int (&wo)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = stream_row(a, t, lrow[i]);
            xo[i] = r >= 0 ? (static_cast<unsigned int>(r) * a.in + 4 * lchunk[i]) * 4u : kOutOfRange;
            const int n = t.n0 + lrow[i];
            wo[i] = n < kGateCols ? (static_cast<unsigned int>(n) * a.kpad + 4 * lchunk[i]) * 4u : kOutOfRange;
        }
    };
    // one K step (K offset k0) into LDS stage `stage`
    auto issue = [&](int stage, const unsigned int (&xo)[4], const unsigned int (&wo)[4], int k0) {
        float *sa = &lds[stage * kStageFloats];
        const int kb = k0 * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // layer 0: k past the 60 inputs reads zeros, not the next row
            const unsigned int off = (KSTEPS * BK == kWidth || k0 + 4 * lchunk[i] < a.in) ? xo[i] : kOutOfRange;
            if (coherent) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, sa + (wave * 4 + i) * 256, 16, off, kb, 0,
                                                         kCachePolicySc1);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, sa + (wave * 4 + i) * 256, 16, off, kb, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, sa + BM * BK + (wave * 4 + i) * 256, 16, wo[i], kb, 0, 0);
        }
    };
    const int frag_row = lane & 31;

    bool timed_out = false;
    // The next tile's first K steps are loaded during the current tile's last ones when its
    // first half already exists (known from a progress read at the current tile's start); else
    // the tile waits for it when it starts. The current tile's second half is loaded as the
    // ring frees when it exists; else, after the first half's last products, once it does.
    bool staged = false;  // the tile's first LA K steps are already issued
    int sbase = 0;        // LDS stage of the tile's first K step

    // One tile TN gate columns wide. The four waves split it WM x WN, each a grid of NI x NJ
    // blocks of 32 x 32 (128 columns: 2 x 2 waves of 64 x 64; 64: 2 x 2 of 64 x 32; 32: 4 x 1
    // of 32 x 32). Every block runs the same MFMA sequence over K whatever the width, so a
    // gate's sum does not depend on the tile it falls in.
    // The workgroup's tiles first + k·nwg, k = 0 .. my_tiles - 1, in the walk's order (protocol.h:
    // with lead0 > 0 the tiles whose rows exist first while the previous layer still runs).
    const int my_tiles = first < a.tiles ? (a.tiles - first + nwg - 1) / nwg : 0;
    const bool walk = kHalves && lead0 > 0 && a.progress != nullptr && my_tiles > 1;
    auto tile_of = [&](int k) { return stream_tile(a, first + k * nwg); };
    // steps of the previous layer both directions of a window have run, from their words
    auto both_directions = [&](unsigned long long s0, unsigned long long s1) {
        const uint32_t p0 = progress_steps(s0, a.progress_pass, static_cast<uint32_t>(a.steps));
        const uint32_t p1 = progress_steps(s1, a.progress_pass, static_cast<uint32_t>(a.steps));
        return p0 < p1 ? p0 : p1;
    };

    auto run = [&](const StreamTile &t, const StreamTile &tn, bool next, int taken, auto width_tag) {
        constexpr int TN = decltype(width_tag)::value;
        constexpr int WN = TN >= 64 ? 2 : 1;
        constexpr int WM = 4 / WN;
        constexpr int NI = BM / WM / 32;
        constexpr int NJ = TN / WN / 32;
        const int row0 = (wave / WN) * (BM / WM);
        const int col0 = (wave % WN) * (TN / WN);
        const int n0 = t.n0;

        float sbias[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) sbias[j] = a.bias[n0 + col0 + j * 32 + (lane & 31)];

        // progress of this tile's and of the next tile's windows, read before any K step of
        // this tile is issued (so every later wait counts K steps only)
        const unsigned long long *pc = watched_word(a, t, lane);
        const unsigned long long seen_cur =
            pc != nullptr ? __hip_atomic_load(pc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : ~0ull;
        const unsigned long long *pn = next ? watched_word(a, tn, lane) : nullptr;
        const unsigned long long seen_next =
            pn != nullptr ? __hip_atomic_load(pn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : ~0ull;

        // a whole number of rings per tile: every tile starts at stage 0 (compile-time stages)
        auto stage_of = [&](int g) {
            return KSTEPS % kStages == 0 ? g & (kStages - 1) : (sbase + g) & (kStages - 1);
        };
        if (!staged) {
            wait_half(a, t, lane, true, timed_out);
            offsets_of(t, xoff, woff);
#pragma unroll
            for (int g = 0; g < LA; ++g) issue(stage_of(g), xoff, woff, kstep_at<KSTEPS>(n0, g) * BK);
        }
        int last = LA - 1;  // last K step issued (steps of the next tile count from KSTEPS)
        // whether the second half exists and whether the next tile's first half does: decided
        // where first needed, long after the progress reads were issued
        bool second_ok = !kHalves;
        bool prefetch = false;
        bool late = false;

        v16f acc[NI][NJ];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        staged = false;
#pragma unroll
        for (int kt = 0; kt < KSTEPS; ++kt) {
            // this wave's loads of step kt have landed; then every wave's have, and every wave
            // is done with the stage step kt - 1 used. A bare barrier: the fence of
            // __syncthreads would wait for every load in flight, the later steps' too.
            wait_steps_after(last - kt);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            // refill that stage with step kt + LA: of this tile, or of the next one
            const int g = kt + LA;
            if (kHalves && g == kHalf) second_ok = __all(half_ready(a, t, lane, seen_cur, false));
            if (g == KSTEPS) prefetch = next && __all(half_ready(a, tn, lane, seen_next, true));
            if (g < KSTEPS) {
                if (kHalves && g >= kHalf && !second_ok) {
                    late = true;
                } else {
                    issue(stage_of(g), xoff, woff, kstep_at<KSTEPS>(n0, g) * BK);
                    last = g;
                }
            } else if (prefetch) {
                if (g == KSTEPS) offsets_of(tn, xoff_next, woff_next);
                issue(stage_of(g), xoff_next, woff_next, kstep_at<KSTEPS>(tn.n0, g - KSTEPS) * BK);
                last = g;
                staged = true;
            }
            // products of step kt. The fragment addresses are recomputed every step from an
            // opaque copy of the lane's row (a few ALU operations): hoisted out of the loops,
            // they took over a hundred registers across the stages and tile widths.
            const float *sa = &lds[stage_of(kt) * kStageFloats];
            const float *sb = sa + BM * BK;
            int fr = frag_row;
            asm volatile("" : "+v"(fr));
            if constexpr (PARTS != 0) {
                // two 16-wide K chunks; lane half h supplies k = 16c + 8h .. 16c + 8h + 7, the
                // LDS chunks 4c + 2h and 4c + 2h + 1 of its row; the six (three) products of the
                // parts in the order of projection_split_kernel
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int c0 = 4 * c + 2 * (lane >> 5);
                    bf16x8 pa[NI][PARTS], pb[NJ][PARTS];
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int r = row0 + i * 32 + fr;
                        split8<PARTS>(*reinterpret_cast<const v4f *>(&sa[swizzled(r, c0)]),
                                      *reinterpret_cast<const v4f *>(&sa[swizzled(r, c0 + 1)]), pa[i]);
                    }
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int r = col0 + j * 32 + fr;
                        split8<PARTS>(*reinterpret_cast<const v4f *>(&sb[swizzled(r, c0)]),
                                      *reinterpret_cast<const v4f *>(&sb[swizzled(r, c0 + 1)]), pb[j]);
                    }
#pragma unroll
                    for (int i = 0; i < NI; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j) {
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i][0], pb[j][0], acc[i][j], 0, 0, 0);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i][0], pb[j][1], acc[i][j], 0, 0, 0);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i][1], pb[j][0], acc[i][j], 0, 0, 0);
                            if constexpr (PARTS == 3) {
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i][1], pb[j][1], acc[i][j], 0, 0, 0);
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i][0], pb[j][2], acc[i][j], 0, 0, 0);
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i][2], pb[j][0], acc[i][j], 0, 0, 0);
                            }
                        }
                }
            } else {
            v4f af[2][NI], bf[2][NJ];
            auto frags = [&](int gq, v4f (&fa)[NI], v4f (&fb)[NJ]) {
                const int c = 2 * gq + (lane >> 5);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    fa[i] = *reinterpret_cast<const v4f *>(&sa[swizzled(row0 + i * 32 + fr, c)]);
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    fb[j] = *reinterpret_cast<const v4f *>(&sb[swizzled(col0 + j * 32 + fr, c)]);
                }
            };
            frags(0, af[0], bf[0]);
#pragma unroll
            for (int gq = 0; gq < kGroups; ++gq) {
                const int p = gq & 1;
                if (gq + 1 < kGroups) frags(gq + 1, af[p ^ 1], bf[p ^ 1]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < NI; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[p][i][e], bf[p][j][e],
                                                                             acc[i][j], 0, 0, 0);
            }
            }
            // the second half held back: after the first half's last products, wait for it
            // and load every step of it the ring has room for
            if (kHalves && kt == kHalf - 1 && late) {
                wait_half(a, t, lane, false, timed_out);
#pragma unroll
                for (int h = kHalf; h <= kt + LA && h < KSTEPS; ++h) {
                    issue(stage_of(h), xoff, woff, kstep_at<KSTEPS>(n0, h) * BK);
                    last = h;
                }
                late = false;
                second_ok = true;
            }
        }
        sbase = (sbase + KSTEPS) & (kStages - 1);
        if (staged) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xoff[i] = xoff_next[i];
                woff[i] = woff_next[i];
            }
        }

        // store with agent-scope stores; once every wave's stores have completed, publish.
        // Row r of block i is local row lb + i·32 + (r / 4)·8 + r % 4 (lb from an opaque copy,
        // so the row arithmetic is not hoisted out of the tile loop into registers). A 32-row
        // block lies in one window (chunks are 32 steps or more), so its rows are consecutive
        // steps: gate row = the block's first row's, plus or minus the step offset.
        int lb = row0 + (lane >> 5) * 4;
        asm volatile("" : "+v"(lb));
        float *const gcol = a.gates + n0 + col0 + (lane & 31);
        const bool full = t.w0 + a.group_windows <= a.batch && t.s0 + a.chunk <= a.steps;
        const int dstep = t.dir == 0 ? 1 : -1;
        int bm0[NI], bw[NI], bs0[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int lr0 = lb + i * 32;                  // local row of r = 0
            bw[i] = t.w0 + (lr0 >> a.chunk_shift);        // the block's window
            bs0[i] = t.s0 + (lr0 & (a.chunk - 1));        // step of r = 0
            bm0[i] = bw[i] * a.steps + (t.dir == 0 ? bs0[i] : a.steps - 1 - bs0[i]);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ds = (r >> 2) * 8 + (r & 3);
                if (full || (bw[i] < a.batch && bs0[i] + ds < a.steps)) {
                    float *const p = gcol + static_cast<ptrdiff_t>(bm0[i] + dstep * ds) * kGateCols;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        __hip_atomic_store(p + j * 32, acc[i][j][r] + sbias[j], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        // the tile after the next one, from the progress this tile's start saw (lanes 0 and 1
        // of wave 0 watch both directions of the tile's first window)
        const unsigned long long seen_other = __shfl(seen_cur, 1);
        if (tid == 0 && next) {
            const uint32_t p = walk ? both_directions(seen_cur, seen_other) : 0u;
            order_slot[0] = stream_walk_after(walk_state, taken, p,
                                              static_cast<uint32_t>(chunk_need(a.steps, a.chunk, t.c)));
        }
        __syncthreads();
        // the tiles of a counter's chunk add kReadyPerPass per pass in all: TN / 32 each
        if (tid == 0) {
            __hip_atomic_fetch_add(a.ready + t.counter, static_cast<unsigned int>(TN / 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    if (tid == 0) {
        const int mid = walk ? stream_walk_mid(my_tiles, a.steps, a.chunk, [&](int k) { return tile_of(k).c; }) : 0;
        stream_walk_init(walk_state, my_tiles, mid, a.steps, lead0, walk);
        uint32_t p = 0;
        if (walk) {
            const unsigned long long *w0 = a.progress + kProgressStride * 2 * tile_of(0).w0;
            p = both_directions(__hip_atomic_load(w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                __hip_atomic_load(w0 + kProgressStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        stream_walk_start(walk_state, p, order_slot[0], order_slot[1]);
    }
    __syncthreads();
    // order_slot[0] is rewritten at the end of the next tile, after every wave has read it here.
    // The tiles are the same in every lane: read into scalar registers, so that everything
    // derived from them (row blocks, K offsets, the width dispatch) stays scalar.
    int kcur = __builtin_amdgcn_readfirstlane(order_slot[0]);
    int knext = __builtin_amdgcn_readfirstlane(order_slot[1]);
    for (int taken = 0; kcur >= 0; ++taken) {
        const StreamTile t = tile_of(kcur);
        const bool next = knext >= 0;
        const StreamTile tn = tile_of(next ? knext : kcur);
        if (t.width == BN) {
            run(t, tn, next, taken, TileWidth<BN>{});
        } else if (t.width == BN / 2) {
            run(t, tn, next, taken, TileWidth<BN / 2>{});
        } else {
            run(t, tn, next, taken, TileWidth<BN / 4>{});
        }
        // written by thread 0 before the tile's last barrier
        const int kafter = next ? __builtin_amdgcn_readfirstlane(order_slot[0]) : -1;
        kcur = knext;
        knext = kafter;
    }
}


// ---- matrix-core rate probe ------------------------------------------------------------------
//
// The rate the projection's peak rests on: two 256-thread workgroups per CU, each wave running
// `iters` rounds of 16 MFMAs over four independent 32x32 accumulators, operands in registers
// from `in` (4096 floats). KIND 0: v_mfma_f32_32x32x16_bf16; 1: v_mfma_f32_32x32x2f32. The
// operand values matter: the matrix pipes run slower on random data than on zeros.
template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(const float *in, float *out, int iters) {
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    v16f acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    if constexpr (KIND == 0) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[t][e] = static_cast<__bf16>(in[(gid * 32 + t * 8 + e) & 4095]);
                b[t][e] = static_cast<__bf16>(in[(gid * 32 + 16 + t * 8 + e) & 4095]);
            }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], acc[1], 0, 0, 0);
                acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], acc[2], 0, 0, 0);
                acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc[3], 0, 0, 0);
            }
        }
    } else {
        v4f a[2], b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[t][e] = in[(gid * 16 + t * 4 + e) & 4095];
                b[t][e] = in[(gid * 16 + 8 + t * 4 + e) & 4095];
            }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0][u], b[0][u], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0][u], b[1][u], acc[1], 0, 0, 0);
                acc[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1][u], b[0][u], acc[2], 0, 0, 0);
                acc[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1][u], b[1][u], acc[3], 0, 0, 0);
            }
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[i][r];
    out[gid] = sum;
}

}  // namespace

// The walk's assumed lead and the tiles per workgroup from which the walk is used. The lead is
// the previous layer's steps per streamed tile: about 40 for the three-part split (17-18 us per
// tile beside the recurrence) and 20-25 for FP32 products, at 0.44-0.46 us per step.
constexpr unsigned int kWalkLead = 64;
constexpr int kWalkMinTiles = 8;

hipError_t launch_projection(const ProjArgs &args, int workgroups, hipStream_t stream) {
    if (args.tiles <= 0) return hipSuccess;
    // a multiple of 8 (the XCD-ordered walk), at most one workgroup per tile group of 8
    int nwg = std::min(workgroups, (args.tiles + 7) / 8 * 8);
    nwg = std::max(8, nwg / 8 * 8);
    if (args.chunk > 0) {
        // streamed order: FP32 MFMA or split precision (W as FP32, split in registers)
        if (args.ready == nullptr || args.chunk * args.group_windows != kProjTileM ||
            (1 << args.chunk_shift) != args.chunk ||
            (args.split_parts != 0 && args.split_parts != 2 && args.split_parts != 3)) {
            return hipErrorInvalidValue;
        }
        // Beside the previous layer's recurrence (progress words), workgroups with several tiles
        // walk: the tiles whose rows exist first (protocol.h), assuming kWalkLead steps of that
        // layer per tile until one is measured. With fewer tiles per workgroup the projection
        // ends well before the recurrence that reads it, and the plain order is kept.
        const int per_wg = (args.tiles + nwg - 1) / nwg;
        const unsigned int lead0 = args.progress != nullptr && per_wg >= kWalkMinTiles ? kWalkLead : 0u;
#define BL_STREAM(KS, PARTS) \
    hipLaunchKernelGGL((projection_stream_kernel<KS, PARTS>), dim3(nwg), dim3(kProjThreads), 0, stream, args, lead0)
        switch ((args.kpad / kProjTileK) * 4 + args.split_parts) {
            case 2 * 4 + 0: BL_STREAM(2, 0); break;
            case 2 * 4 + 2: BL_STREAM(2, 2); break;
            case 2 * 4 + 3: BL_STREAM(2, 3); break;
            case 8 * 4 + 0: BL_STREAM(8, 0); break;
            case 8 * 4 + 2: BL_STREAM(8, 2); break;
            case 8 * 4 + 3: BL_STREAM(8, 3); break;
            default:
                return hipErrorInvalidValue;
        }
#undef BL_STREAM
        return hipGetLastError();
    }
    if (args.split_parts != 0) {
        if (args.w_hi == nullptr || args.w_lo == nullptr || (args.split_parts == 3) != (args.w_lo2 != nullptr)) {
            return hipErrorInvalidValue;
        }
        const bool three = args.split_parts == 3;
        // two workgroups per CU
        const int nsplit = std::max(8, std::min(2 * workgroups, (args.tiles + 7) / 8 * 8) / 8 * 8);
        switch (args.kpad / kProjTileK) {
            case 2:
                if (three) {
                    hipLaunchKernelGGL((projection_split_kernel<2, 3>), dim3(nsplit), dim3(kSplitThreads), 0, stream,
                                       args);
                } else {
                    hipLaunchKernelGGL((projection_split_kernel<2, 2>), dim3(nsplit), dim3(kSplitThreads), 0, stream,
                                       args);
                }
                break;
            case 8:
                if (three) {
                    hipLaunchKernelGGL((projection_split_kernel<8, 3>), dim3(nsplit), dim3(kSplitThreads), 0, stream,
                                       args);
                } else {
                    hipLaunchKernelGGL((projection_split_kernel<8, 2>), dim3(nsplit), dim3(kSplitThreads), 0, stream,
                                       args);
                }
                break;
            default:
                return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // One or two workgroups per CU, whichever needs less time by tile rounds: two on a CU
    // finish a round of two tiles in about 1.87 times one tile's time alone (measured).
    int nfp32 = nwg;
    {
        const int two = std::max(8, std::min(2 * workgroups, (args.tiles + 7) / 8 * 8) / 8 * 8);
        const long r1 = (args.tiles + nwg - 1) / nwg;
        const long r2 = (args.tiles + two - 1) / two;
        if (15 * r2 < 8 * r1) nfp32 = two;
    }
    switch (args.kpad / kProjTileK) {
        case 2:
            hipLaunchKernelGGL(projection_kernel<2>, dim3(nfp32), dim3(kProjThreads), 0, stream, args);
            break;
        case 8:
            hipLaunchKernelGGL(projection_kernel<8>, dim3(nfp32), dim3(kProjThreads), 0, stream, args);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


hipError_t run_mfma_probe(int kind, int data, int iters, int cu_count, double *tflops, double *ms) {
    const int workgroups = 2 * cu_count;
    const size_t threads = static_cast<size_t>(workgroups) * 256;
    std::vector<float> host(4096);
    unsigned int st = 12345u;
    for (float &v : host) {
        st = st * 1664525u + 1013904223u;
        v = data == 0 ? 0.0f : data == 1 ? 1.0f : static_cast<float>(st >> 8) / 8388608.0f - 1.0f;
    }
    float *in = nullptr, *out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipMalloc(&in, host.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&out, threads * sizeof(float));
    if (e == hipSuccess) e = hipMemcpy(in, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    float elapsed = 0.0f;
    for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {  // the first launch warms up
        e = hipEventRecord(e0, nullptr);
        if (kind == 0) {
            hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(workgroups), dim3(256), 0, nullptr, in, out, iters);
        } else {
            hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(workgroups), dim3(256), 0, nullptr, in, out, iters);
        }
        if (e == hipSuccess) e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        if (e == hipSuccess) e = hipEventElapsedTime(&elapsed, e0, e1);
    }
    if (e0 != nullptr) (void)hipEventDestroy(e0);
    if (e1 != nullptr) (void)hipEventDestroy(e1);
    if (in != nullptr) (void)hipFree(in);
    if (out != nullptr) (void)hipFree(out);
    if (e != hipSuccess) return e;
    const double flop_per_mfma = kind == 0 ? 32.0 * 32 * 16 * 2 : 32.0 * 32 * 2 * 2;
    const double flops = static_cast<double>(threads / 64) * iters * 16 * flop_per_mfma;
    *ms = elapsed;
    *tflops = flops / (elapsed * 1e-3) / 1e12;
    return hipSuccess;
}

}  // namespace bl
