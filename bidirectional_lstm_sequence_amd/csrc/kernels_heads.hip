// The segmentation heads after the stack, fused into one kernel on gfx950 (speakrs 0.6.0,
// page `segdense.rs`, `Site` doc: linear0 256 -> 128 and linear1 128 -> 128, each with bias
// and LeakyReLU, then linear2 128 -> 7 with bias and log-softmax; row-major [k][n] weights).
//
//   h0 = leaky(y · W0 + b0)      [rows][128]
//   h1 = leaky(h0 · W1 + b1)     [rows][128]
//   out = log_softmax(h1 · W2 + b2) over each row's 7 classes
//
// One 256-thread workgroup takes 32 rows through all three layers; h0 and h1 never leave
// LDS, so HBM sees the stack's output read once and the log-probabilities written once. Its
// 67 KB of LDS let two workgroups share a CU, and 32-row tiles spread a batch evenly over the
// CUs (589 tiles for 32 windows of 589 frames, against 295 of 64 rows, which left the second
// round of a 256-CU chip mostly empty).
//  * linear0 and linear1: FP32 MFMA (v_mfma_f32_32x32x2_f32), four waves of 32x32 (one column
//    block each), K steps of 32 through double-buffered LDS tiles (36-float rows:
//    conflict-free ds_read_b128); lane half h supplies k = k0 + 4h + e in the e-th MFMA of a
//    group, for A and B alike. The weights arrive transposed ([n][k]) from the host packer so
//    both operands read along k.
//  * classifier: 32 rows x 8 class slots (7 used) on the VALU, eight lanes per row, one class
//    each; log-softmax with DPP reductions over the eight lanes (xor 1, xor 2, then the
//    half-row mirror) of the row maximum and of the sum of exponentials:
//    out = z - m - log(sum exp(z - m)).
// Each output's summation order is fixed and independent of the row's position.
#include "bilstm_internal.h"

namespace bl {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kRows = kHeadTileRows;      // rows per workgroup
constexpr int kThreads = kHeadThreads;
constexpr int kK = 32;                    // K step
constexpr int kStride = kK + 4;           // LDS row stride of a K-step tile, floats
constexpr int kHStride = kHeadMid + 4;    // LDS row stride of h0 / h1, floats

static_assert(kRows == 32 && kThreads == 256 && kHeadMid == 128, "tile shape");

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float leaky(float v, float slope) { return v >= 0.0f ? v : slope * v; }

template <int N>
struct Const {
    static constexpr int value = N;
};

__global__ __launch_bounds__(kThreads, 2) void heads_kernel(HeadArgs a) {
    __shared__ __attribute__((aligned(16))) float tile_a[2][kRows * kStride];
    __shared__ __attribute__((aligned(16))) float tile_b[2][kHeadMid * kStride];  // later h1
    __shared__ __attribute__((aligned(16))) float h0s[kRows * kHStride];
    __shared__ __attribute__((aligned(16))) float w2s[kHeadClassSlots * kHeadMid];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave;  // 32-column block of this wave
    const long m0 = static_cast<long>(blockIdx.x) * kRows;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 4;

    // classifier weights [8][128] (slot 7 zero) into LDS
    for (int i = tid; i < kHeadClassSlots * kHeadMid / 4; i += kThreads) {
        reinterpret_cast<v4f *>(w2s)[i] = reinterpret_cast<const v4f *>(a.w2t)[i];
    }

    // One MFMA layer: acc (column block wn) = A[32 rows][K] · Bᵀ, B [128][K] from global
    // (transposed weights), A either from global (y) or from h0 in LDS.
    v16f acc;
    // The global loads of K step kt + kAhead are issued at step kt into a register ring, so
    // several steps' loads are in flight while the MFMAs run (one step ahead, a tile's latency
    // was its K steps' load round trips: about 20 us for any tile).
    constexpr int kAhead = 3;
    auto gemm = [&](const float *bt, auto ksteps_c, auto a_global_c) {
        constexpr int ksteps = decltype(ksteps_c)::value;
        constexpr bool a_global = decltype(a_global_c)::value != 0;
        constexpr int kdim = ksteps * kK;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        v4f ra[kAhead], rb[kAhead][4];
        auto load = [&](int slot, int k0) {
            if constexpr (a_global) {
                const long m = m0 + (tid >> 3);
                const int k = k0 + (tid & 7) * 4;
                v4f v = {0.f, 0.f, 0.f, 0.f};
                if (m < a.rows) v = *reinterpret_cast<const v4f *>(a.y + m * kHeadIn + k);
                ra[slot] = v;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = tid + kThreads * i;
                rb[slot][i] = *reinterpret_cast<const v4f *>(bt + static_cast<size_t>(f >> 3) * kdim + k0 + (f & 7) * 4);
            }
        };
        auto store = [&](int slot, int buf) {
            if constexpr (a_global) *reinterpret_cast<v4f *>(&tile_a[buf][(tid >> 3) * kStride + (tid & 7) * 4]) = ra[slot];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = tid + kThreads * i;
                *reinterpret_cast<v4f *>(&tile_b[buf][(f >> 3) * kStride + (f & 7) * 4]) = rb[slot][i];
            }
        };
        // step 0 into LDS; steps 1 .. kAhead into the ring (slot (s - 1) % kAhead holds step s)
        load(0, 0);
        store(0, 0);
#pragma unroll
        for (int st = 1; st <= kAhead; ++st)
            if (st < ksteps) load((st - 1) % kAhead, st * kK);
        __syncthreads();
#pragma unroll
        for (int kt = 0; kt < ksteps; ++kt) {
            const int cur = kt & 1;
#pragma unroll
            for (int g = 0; g < kK / 8; ++g) {
                v4f af;
                if constexpr (a_global) {
                    af = *reinterpret_cast<const v4f *>(&tile_a[cur][frag_row * kStride + g * 8 + frag_k]);
                } else {
                    af = *reinterpret_cast<const v4f *>(&h0s[frag_row * kHStride + kt * kK + g * 8 + frag_k]);
                }
                const v4f bf = *reinterpret_cast<const v4f *>(&tile_b[cur][(wn * 32 + frag_row) * kStride + g * 8 + frag_k]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], acc, 0, 0, 0);
            }
            if (kt + 1 < ksteps) {
                // step kt + 1 from its ring slot into the other LDS buffer, then step
                // kt + 1 + kAhead into the freed slot
                const int slot = kt % kAhead;
                store(slot, cur ^ 1);
                if (kt + 1 + kAhead < ksteps) load(slot, (kt + 1 + kAhead) * kK);
            }
            __syncthreads();
        }
    };
    // bias + LeakyReLU of the MFMA sums into an LDS row buffer [32][132]
    auto finish = [&](const float *bias, float *dst) {
        const int n = wn * 32 + (lane & 31);
        const float bv = bias[n];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            dst[row * kHStride + n] = leaky(acc[r] + bv, a.slope);
        }
    };

    gemm(a.w0t, Const<kHeadIn / kK>{}, Const<1>{});
    finish(a.b0, h0s);
    __syncthreads();
    gemm(a.w1t, Const<kHeadMid / kK>{}, Const<0>{});
    float *h1s = &tile_b[0][0];  // the B tiles are free once linear1's last K step is done
    finish(a.b1, h1s);
    __syncthreads();

    // classifier and log-softmax: eight lanes per row, lane c takes class c (slot 7 unused)
    const int row = tid >> 3;
    const int c = tid & 7;
    const bool valid = c < kHeadClasses;  // class 7 is padding
    float z = a.b2[valid ? c : 0];
#pragma unroll 4
    for (int k4 = 0; k4 < kHeadMid / 4; ++k4) {
        const v4f hv = *reinterpret_cast<const v4f *>(&h1s[row * kHStride + 4 * k4]);
        const v4f wv = *reinterpret_cast<const v4f *>(&w2s[c * kHeadMid + 4 * k4]);
        z = fmaf(hv[0], wv[0], z);
        z = fmaf(hv[1], wv[1], z);
        z = fmaf(hv[2], wv[2], z);
        z = fmaf(hv[3], wv[3], z);
    }
    // the maximum and the sum over the row's lanes: xor 1, xor 2 (quad_perm), then the
    // half-row mirror, which pairs each lane with one of the other quad
    float mx = valid ? z : -__builtin_huge_valf();
    mx = fmaxf(mx, dpp<0xB1>(mx));   // quad_perm 1,0,3,2
    mx = fmaxf(mx, dpp<0x4E>(mx));   // quad_perm 2,3,0,1
    mx = fmaxf(mx, dpp<0x141>(mx));  // row_half_mirror
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kLn2 = 0.6931471805599453f;
    float se = valid ? __builtin_amdgcn_exp2f((z - mx) * kLog2e) : 0.0f;
    se = se + dpp<0xB1>(se);
    se = se + dpp<0x4E>(se);
    se = se + dpp<0x141>(se);
    const float lse = mx + __builtin_amdgcn_logf(se) * kLn2;
    const long m = m0 + row;
    if (m < a.rows && valid) a.out[m * kHeadClasses + c] = z - lse;
}

}  // namespace

hipError_t launch_heads(const HeadArgs &args, hipStream_t stream) {
    if (args.rows <= 0) return hipSuccess;
    const long blocks = (args.rows + kHeadTileRows - 1) / kHeadTileRows;
    hipLaunchKernelGGL(heads_kernel, dim3(static_cast<unsigned int>(blocks)), dim3(kHeadThreads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace bl
