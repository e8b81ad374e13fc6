// Persistent, step-serial LSTM recurrence of one layer on gfx950, the exchange clear and the
// exchange latency probe (speakrs 0.6.0, page `lstmproj.rs`: module doc — one launch per
// direction runs that direction's whole recurrence with the recurrent weights held on chip;
// `RecurrencePlan` doc — several workgroups per window tile split the units and exchange h,
// or one workgroup holds the whole matrix and needs no exchange; `Exchange` and
// `clear_state` — flagged words zeroed before a pass).
//
// Work split. A launch covers `tile_count` tiles of BT windows for one direction (or both,
// gridDim.y = 2). Each tile is served by KG workgroups; workgroup `member` owns hidden
// units [member·U, (member+1)·U), U = 128/KG, i.e. the 4U packed gate rows 4j+g of R, held
// in VGPRs for the whole launch. Inside a workgroup, Q lanes (adjacent in the wave) share a
// unit: lane q holds the unit's four gate rows over K chunks [q·16/Q, (q+1)·16/Q) of the
// 16 eight-element chunks of h.
//
// One step s (t = s forward, T-1-s reverse):
//  1. every lane: 4·BT dot products of its rows with its h chunks (h_{t-1} from LDS);
//  2. the canonical sum: each chunk summed in k order from 0, chunks combined by a fixed
//     balanced binary tree — in-lane for the lower levels, DPP butterflies across the Q
//     lanes for the upper ones. The tree is the same for every KG, so every workgroup
//     split gives bitwise identical results;
//  3. lane q < BT (window q of the tile): a = gate input + sum; i, f, o = σ, g = tanh;
//     c = f·c + i·g; h = o·tanh(c); h goes to LDS, to the output and, when KG > 1, to the
//     exchange as one 64-bit word {flag, h};
//  4. KG > 1: the other workgroups' h words of step s are polled until their flag is
//     flag_base + s + 1 and copied into LDS (step-parity double buffer);
//  5. one workgroup barrier.
//
// Gate inputs are prefetched several steps ahead. With KG = 1 every window lane keeps a
// register ring. With KG > 1, waves that poll must not hold outstanding prefetches (the
// poll's wait would drain them), so wave 0 prefetches the workgroup's gates into an LDS
// ring and does not poll; waves 1.. poll.
//
// Waits are bounded: a poll that sees no progress for `timeout_ticks` wall-clock ticks
// sets the error word and stops waiting, so the grid always drains.
#include "bilstm_internal.h"

namespace bl {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kRing = 4;  // prefetch depth in steps

template <int KG>
struct Split {
    static constexpr int U = kHidden / KG;                         // units per workgroup
    static constexpr int Q = KG == 1 ? 4 : (KG == 2 ? 8 : 16);     // lanes per unit
    static constexpr int NT = U * Q;                               // threads
    static constexpr int NCH = 16 / Q;                             // K chunks per lane
};

// Padded h index: 4 floats of padding after every 32, so the four K quarters of h start on
// different LDS banks.
__device__ __forceinline__ int hpad(int k) { return k + (k >> 5) * 4; }
constexpr int kHPad = kHidden + kHidden / 8;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// e^{-a} for a >= 0, on the hardware exp2.
__device__ __forceinline__ float exp_neg(float a) {
    return __builtin_amdgcn_exp2f(a * -1.4426950408889634f);
}

// σ(z) = 1/(1+e^{-z}), evaluated through e^{-|z|} so it never overflows.
__device__ __forceinline__ float sigmoid_f(float z) {
    const float e = exp_neg(fabsf(z));
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return z >= 0.0f ? r : e * r;
}

// tanh(z) = sign(z)·(1 - e^{-2|z|})/(1 + e^{-2|z|}).
__device__ __forceinline__ float tanh_f(float z) {
    const float e = exp_neg(2.0f * fabsf(z));
    const float t = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    return copysignf(t, z);
}

template <int BT>
__device__ __forceinline__ float pick(const float (&v)[BT], int b) {
    float r = v[0];
#pragma unroll
    for (int i = 1; i < BT; ++i) r = (b == i) ? v[i] : r;
    return r;
}

__device__ __forceinline__ unsigned long long load_word(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_word(unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KG, int BT>
__global__ __launch_bounds__(Split<KG>::NT) void recurrence_kernel(RecurArgs a) {
    using S = Split<KG>;
    constexpr int U = S::U, Q = S::Q, NT = S::NT, NCH = S::NCH;

    // ---- which tile, member and direction ------------------------------------------------
    int tile, member;
    if constexpr (KG == 1) {
        tile = blockIdx.x;
        member = 0;
    } else {
        // ids congruent mod 8 share an XCD: keep a tile's KG workgroups on one XCD
        const int slot = blockIdx.x >> 3;
        tile = (slot / KG) * 8 + (blockIdx.x & 7);
        member = slot % KG;
    }
    if (tile >= a.tile_count) return;  // grid padding; uniform over the workgroup
    tile += a.tile_first;
    const int dir = a.direction + blockIdx.y;
    const int steps = a.steps;

    const int tid = threadIdx.x;
    const int u = tid / Q;
    const int q = tid % Q;
    const int ug = member * U + u;  // global hidden unit of this lane

    __shared__ __attribute__((aligned(16))) float hs[2][kHPad * BT];
    __shared__ __attribute__((aligned(16))) float gs[KG > 1 ? 2 : 1][KG > 1 ? U * 4 * BT : 4];

    // ---- recurrent weights into VGPRs ------------------------------------------------------
    float rr[4][NCH][8];
    {
        const float *rdir = a.r + static_cast<size_t>(dir) * kGates * kHidden;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int chunk = q * NCH + c;
                const v4f *p = reinterpret_cast<const v4f *>(
                    rdir + static_cast<size_t>(4 * ug + g) * kHidden + chunk * 8);
                const v4f lo = p[0], hi = p[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rr[g][c][e] = lo[e];
                    rr[g][c][4 + e] = hi[e];
                }
            }
    }

    // h_{-1} = 0
    for (int i = tid; i < 2 * kHPad * BT; i += NT) (&hs[0][0])[i] = 0.0f;

    const bool window_lane = q < BT;
    const int win = tile * BT + (window_lane ? q : 0);
    const bool valid = window_lane && win < a.batch;
    const size_t gate_col = static_cast<size_t>(dir) * kGates;
    auto time_of = [&](int s) { return dir == 0 ? s : steps - 1 - s; };

    // KG == 1: per-lane register ring of this lane's float4 of gates.
    v4f ring[kRing];
    // KG > 1: wave 0 stages the workgroup's gates; lane j of wave 0 moves float4 j, j + 64 ...
    constexpr int kStageVec = KG > 1 ? (U * BT + 63) / 64 : 1;
    v4f stage[kRing][kStageVec];
    const bool stager = (KG > 1) && (tid < 64);

    auto gate_ptr = [&](int w, int s) {
        return a.gates + (static_cast<size_t>(w) * steps + time_of(s)) * kGateCols + gate_col;
    };
    // float4 j of the workgroup's per-step gates: window j / U, unit member·U + j % U
    auto stage_load = [&](int j, int s) -> v4f {
        const int bw = tile * BT + j / U;
        if (j >= U * BT || bw >= a.batch || s >= steps) return v4f{0.f, 0.f, 0.f, 0.f};
        return *reinterpret_cast<const v4f *>(gate_ptr(bw, s) + 4 * (member * U + j % U));
    };

    if constexpr (KG == 1) {
#pragma unroll
        for (int p = 0; p < kRing; ++p) {
            ring[p] = v4f{0.f, 0.f, 0.f, 0.f};
            if (valid && p < steps) ring[p] = *reinterpret_cast<const v4f *>(gate_ptr(win, p) + 4 * ug);
        }
    } else {
        if (stager) {
            // step 0 straight into LDS slot 0; steps 1..kRing into the register ring
#pragma unroll
            for (int v = 0; v < kStageVec; ++v) {
                const int j = tid + 64 * v;
                if (j < U * BT) *reinterpret_cast<v4f *>(&gs[0][4 * j]) = stage_load(j, 0);
            }
#pragma unroll
            for (int p = 0; p < kRing; ++p)
#pragma unroll
                for (int v = 0; v < kStageVec; ++v) stage[p][v] = stage_load(tid + 64 * v, p + 1);
        }
    }
    __syncthreads();

    unsigned long long *xdir = nullptr;
    if constexpr (KG > 1) {
        xdir = a.exchange + (static_cast<size_t>(dir) * a.tiles + tile) * 2 * kHidden * BT;
    }
    float cst = 0.0f;  // cell state of (unit ug, window q) on window lanes
    bool timed_out = false;

    for (int s0 = 0; s0 < steps; s0 += kRing) {
#pragma unroll
        for (int p = 0; p < kRing; ++p) {
            const int s = s0 + p;
            if (s < steps) {
                const int cur = s & 1;
                const int nxt = cur ^ 1;

                // (1) partial dot products over this lane's chunks
                float acc[4][NCH][BT];
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int chunk = q * NCH + c;
                    const float *hp = &hs[cur][hpad(chunk * 8) * BT];
                    float hv[8 * BT];
#pragma unroll
                    for (int v = 0; v < 2 * BT; ++v) {
                        const v4f t4 = *reinterpret_cast<const v4f *>(hp + 4 * v);
                        hv[4 * v + 0] = t4[0];
                        hv[4 * v + 1] = t4[1];
                        hv[4 * v + 2] = t4[2];
                        hv[4 * v + 3] = t4[3];
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int b = 0; b < BT; ++b) {
                            float sacc = rr[g][c][0] * hv[b];
#pragma unroll
                            for (int e = 1; e < 8; ++e) sacc = fmaf(rr[g][c][e], hv[e * BT + b], sacc);
                            acc[g][c][b] = sacc;
                        }
                }

                // (2) canonical tree: in-lane levels, then DPP butterflies over the Q lanes
                float sum[4][BT];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int b = 0; b < BT; ++b) {
                        float v;
                        if constexpr (NCH == 4) {
                            v = (acc[g][0][b] + acc[g][1][b]) + (acc[g][2][b] + acc[g][3][b]);
                        } else if constexpr (NCH == 2) {
                            v = acc[g][0][b] + acc[g][1][b];
                        } else {
                            v = acc[g][0][b];
                        }
                        if constexpr (Q >= 2) v = v + dpp<0xB1>(v);   // quad_perm 1,0,3,2
                        if constexpr (Q >= 4) v = v + dpp<0x4E>(v);   // quad_perm 2,3,0,1
                        if constexpr (Q >= 8) v = v + dpp<0x141>(v);  // row_half_mirror
                        if constexpr (Q >= 16) v = v + dpp<0x140>(v); // row_mirror
                        sum[g][b] = v;
                    }

                // (3) the cell update on window lanes
                const unsigned int flag = a.flag_base + static_cast<unsigned int>(s) + 1u;
                float hval = 0.0f;
                if (window_lane) {
                    v4f gi;
                    if constexpr (KG == 1) {
                        gi = ring[p];
                    } else {
                        gi = *reinterpret_cast<const v4f *>(&gs[cur][4 * (q * U + u)]);
                    }
                    const float ai = gi[0] + pick<BT>(sum[0], q);
                    const float af = gi[1] + pick<BT>(sum[1], q);
                    const float ag = gi[2] + pick<BT>(sum[2], q);
                    const float ao = gi[3] + pick<BT>(sum[3], q);
                    const float ig = sigmoid_f(ai);
                    const float fg = sigmoid_f(af);
                    const float gg = tanh_f(ag);
                    const float og = sigmoid_f(ao);
                    cst = fmaf(fg, cst, ig * gg);
                    hval = og * tanh_f(cst);
                    hs[nxt][hpad(ug) * BT + q] = hval;
                    if constexpr (KG > 1) {
                        const unsigned long long word =
                            (static_cast<unsigned long long>(flag) << 32) | __float_as_uint(hval);
                        store_word(xdir + (static_cast<size_t>(cur) * kHidden + ug) * BT + q, word);
                    }
                }

                if constexpr (KG == 1) {
                    // refill this ring slot with step s + kRing
                    if (valid && s + kRing < steps) {
                        ring[p] = *reinterpret_cast<const v4f *>(gate_ptr(win, s + kRing) + 4 * ug);
                    }
                } else {
                    if (stager) {
                        // stage[p] holds step s+1 (loaded kRing steps ago): into LDS slot nxt,
                        // then load step s + 1 + kRing in its place
#pragma unroll
                        for (int v = 0; v < kStageVec; ++v) {
                            const int j = tid + 64 * v;
                            if (j < U * BT) *reinterpret_cast<v4f *>(&gs[nxt][4 * j]) = stage[p][v];
                            stage[p][v] = stage_load(j, s + 1 + kRing);
                        }
                    } else {
                        // (4) gather the other workgroups' h of step s
                        constexpr int kOthers = (kHidden - U) * BT;
                        const unsigned long long *xs = xdir + static_cast<size_t>(cur) * kHidden * BT;
                        for (int idx = tid - 64; idx < kOthers; idx += NT - 64) {
                            const int uo = idx / BT;
                            const int b = idx - uo * BT;
                            const int ugo = uo < member * U ? uo : uo + U;
                            const unsigned long long *wp = xs + static_cast<size_t>(ugo) * BT + b;
                            unsigned long long w = load_word(wp);
                            if (static_cast<unsigned int>(w >> 32) != flag && !timed_out) {
                                const unsigned long long t0 = wall_clock64();
                                while (true) {
                                    w = load_word(wp);
                                    if (static_cast<unsigned int>(w >> 32) == flag) break;
                                    if (wall_clock64() - t0 > a.timeout_ticks) {
                                        atomicOr(a.error, 1u);
                                        timed_out = true;
                                        break;
                                    }
                                }
                            }
                            hs[nxt][hpad(ugo) * BT + b] = __uint_as_float(static_cast<unsigned int>(w));
                        }
                    }
                }

                if (valid) {
                    a.y[(static_cast<size_t>(win) * steps + time_of(s)) * kWidth + dir * kHidden + ug] = hval;
                }
                __syncthreads();
            }
        }
    }
}

__global__ void exchange_clear_kernel(unsigned long long *words, size_t count) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        words[i] = 0ull;
    }
}

// Ping-pong between workgroup 0 and workgroup `partner` of the grid; the others exit.
// Word 0 carries A->B, word 16 (another 128-byte line) B->A; the flag is the round number.
__global__ void exchange_probe_kernel(unsigned long long *words, int partner, int rounds,
                                      unsigned long long timeout_ticks, unsigned long long *out) {
    const int wg = blockIdx.x;
    if (wg != 0 && wg != partner) return;
    if (threadIdx.x != 0) return;
    const bool is_a = wg == 0;
    unsigned long long *mine = words + (is_a ? 0 : 16);
    unsigned long long *theirs = words + (is_a ? 16 : 0);
    const unsigned int xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11));
    unsigned long long t_start = 0, t_end = 0;
    bool ok = true;
    for (int r = 1; r <= rounds && ok; ++r) {
        if (is_a) {
            if (r == 1) t_start = wall_clock64();
            store_word(mine, static_cast<unsigned long long>(r) << 32);
        }
        const unsigned long long t0 = wall_clock64();
        while (static_cast<unsigned int>(load_word(theirs) >> 32) != static_cast<unsigned int>(r)) {
            if (wall_clock64() - t0 > timeout_ticks) {
                ok = false;
                break;
            }
        }
        if (!is_a) store_word(mine, static_cast<unsigned long long>(r) << 32);
    }
    t_end = wall_clock64();
    if (is_a) {
        out[0] = t_end - t_start;
        out[1] = ok ? 1ull : 0ull;
        out[2] = xcc;
    } else {
        out[3] = xcc;
        out[4] = ok ? 1ull : 0ull;
    }
}

template <int KG, int BT>
hipError_t launch_typed(const RecurArgs &args, int directions, hipStream_t stream) {
    using S = Split<KG>;
    const int nwg = KG == 1 ? args.tile_count : (args.tile_count + 7) / 8 * 8 * KG;
    hipLaunchKernelGGL((recurrence_kernel<KG, BT>), dim3(nwg, directions), dim3(S::NT), 0, stream, args);
    return hipGetLastError();
}

template <int KG, int BT>
hipError_t occupancy_typed(int *per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, recurrence_kernel<KG, BT>, Split<KG>::NT, 0);
}

#define BL_FOR_EACH_SPLIT(X) \
    X(1, 1) X(1, 2) X(1, 4) X(2, 1) X(2, 2) X(2, 4) X(4, 1) X(4, 2) X(4, 4) X(8, 1) X(8, 2) X(8, 4) \
    X(16, 1) X(16, 2) X(16, 4)

}  // namespace

hipError_t launch_recurrence(int groups, int tile, const RecurArgs &args, int directions,
                             hipStream_t stream) {
    if (args.tile_count <= 0) return hipSuccess;
#define BL_CASE(KG, BT) \
    if (groups == KG && tile == BT) return launch_typed<KG, BT>(args, directions, stream);
    BL_FOR_EACH_SPLIT(BL_CASE)
#undef BL_CASE
    return hipErrorInvalidValue;
}

hipError_t recurrence_occupancy(int groups, int tile, int *per_cu) {
#define BL_CASE(KG, BT) \
    if (groups == KG && tile == BT) return occupancy_typed<KG, BT>(per_cu);
    BL_FOR_EACH_SPLIT(BL_CASE)
#undef BL_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_exchange_clear(unsigned long long *words, size_t count, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    const size_t blocks = (count + 255) / 256;
    const unsigned int grid = static_cast<unsigned int>(blocks < 1024 ? blocks : 1024);
    hipLaunchKernelGGL(exchange_clear_kernel, dim3(grid), dim3(256), 0, stream, words, count);
    return hipGetLastError();
}

hipError_t run_exchange_probe(int same_xcd, int round_trips, unsigned long long timeout_ticks,
                              double ticks_per_ns, double *one_way_ns, int *xcd_a, int *xcd_b) {
    unsigned long long *words = nullptr;
    unsigned long long *out = nullptr;
    hipError_t e = hipMalloc(&words, 64 * sizeof(unsigned long long));
    if (e != hipSuccess) return e;
    e = hipMalloc(&out, 8 * sizeof(unsigned long long));
    if (e != hipSuccess) {
        (void)hipFree(words);
        return e;
    }
    unsigned long long host[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    e = hipMemset(words, 0, 64 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemset(out, 0, 8 * sizeof(unsigned long long));
    if (e == hipSuccess) {
        // ids 0 and 8 share an XCD when workgroups are dealt round-robin over 8 XCDs; 0 and 1 do not
        const int partner = same_xcd ? 8 : 1;
        hipLaunchKernelGGL(exchange_probe_kernel, dim3(16), dim3(64), 0, nullptr, words, partner,
                           round_trips, timeout_ticks, out);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(host, out, sizeof(host), hipMemcpyDeviceToHost);
    (void)hipFree(words);
    (void)hipFree(out);
    if (e != hipSuccess) return e;
    if (host[1] != 1 || host[4] != 1) return hipErrorLaunchTimeOut;
    *one_way_ns = static_cast<double>(host[0]) / ticks_per_ns / (2.0 * round_trips);
    *xcd_a = static_cast<int>(host[2]);
    *xcd_b = static_cast<int>(host[3]);
    return hipSuccess;
}

}  // namespace bl
