// Persistent, step-serial LSTM recurrence of one layer on gfx950, the exchange clear and the
// exchange latency probe (speakrs 0.6.0, page `lstmproj.rs`: module doc — one launch per
// direction runs that direction's whole recurrence with the recurrent weights held on chip;
// `RecurrencePlan` doc — several workgroups per window tile split the units and exchange h,
// or, on the A100 variant, a single block keeps all of R and exchanges nothing; `Exchange`
// and `clear_state` — flagged words zeroed before a pass).
//
// Work split. A launch covers `tile_count` tiles of BT windows for one direction (or both,
// gridDim.y = 2). Each tile is served by KG workgroups; workgroup `member` owns hidden
// units [member·U, (member+1)·U), U = 128/KG, i.e. the 4U packed gate rows 4j+g of R, held
// in VGPRs for the whole launch. Eight adjacent lanes share two units (8 gate rows): lane l
// of the group holds all 8 rows over the K eighth [16l, 16l+16) — 128 values — so a lane
// reads only 16·BT values of h per step (half of what a K quarter per lane would need; the LDS
// reads of h co-limit the step). Its register slot s holds row l ^ slot_row(s), which turns
// the group's reduction into a reduce-scatter with no selects; lane l ends with row l, so
// each quad holds one unit's gates i, f, g, o.
//
// One step s (t = s forward, T-1-s reverse):
//  1. every lane: 8·BT dot products of its rows with its eighth of h_{t-1} (from LDS), each
//     summed in k order from the first product;
//  2. reduce-scatter over the group with DPP (partners l ^ 7, l ^ 2, l ^ 1): lane l ends with
//     row l's full sum, combined in one fixed order for every split and tile;
//  3. lane q: a = gate input + sum; the activation of gate q (σ for i, f, o; tanh for g,
//     as 2σ(2a) - 1); the lane of window b collects the four activations, updates
//     c = f·c + i·g and h = o·tanh(c), and writes h to LDS, to the output and, when KG > 1,
//     to the exchange as one 64-bit word {flag, h};
//  4. KG > 1: the other workgroups' h words of step s are polled until their flag is
//     flag_base + s + 1 and copied into LDS (step-parity double buffer);
//  5. one workgroup barrier.
//
// Gate inputs are prefetched several steps ahead. With KG = 1 every lane keeps a register
// ring. With KG > 1, waves that poll must not hold outstanding prefetches (the poll's wait
// would drain them), so wave 0 prefetches the workgroup's gates into an LDS ring and does not
// poll; waves 1.. poll.
//
// Streamed gates (STREAM, KG = 1): the layer's projection runs at the same time on other CUs
// and publishes the gates chunk by chunk. Before the gate loads of a group of kRing steps are
// issued, the chunk counter read one group earlier must show the chunk published (else the
// wave polls until it does); the counter of the group after next is read at the same point,
// so in the steady state no wave ever waits for a counter. Gate loads are agent-scope loads,
// which see the projection's agent-scope stores once its counter shows them complete. In
// turn the output is written with agent-scope stores and each window's progress (steps whose
// output has completed) is published every kRing steps, for the next layer's projection when
// it runs beside this recurrence. One launch can run several layers this way
// (recurrence_stream_kernel): a workgroup that has finished a layer moves on to the next
// with the same tile and direction.
//
// Waits are bounded: a poll that sees no progress for `timeout_ticks` wall-clock ticks
// sets the error word and stops waiting, so the grid always drains.
#include <algorithm>
#include <vector>

#include "bilstm_internal.h"

namespace bl {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// Prefetch depth in steps: gate loads of step s are issued at step s - depth. Streamed gates
// are read with agent-scope loads, which go past the L2, so they are issued further ahead, as
// they are for single-window tiles, whose steps are shortest (measured: 8 steps 0.472 against
// 4 steps 0.480 us per step; for two-window tiles 4 steps is better). Streamed one-window
// tiles take 16: their group start (chunk counter check, progress word) then comes every 16
// steps (measured: b32 forward 1.121 -> 1.112 ms; the plain kernel is 0.6 % slower with 16;
// a 32-step ring is slower again, 1.114 -> 1.127 ms).
// A chunk (32, 64 or 128 steps) is always a whole number of rings.
constexpr int kRingPlain = 4;
constexpr int kRingOne = 8;
constexpr int kRingStreamOne = 16;

// LDS index of h element f = k·BT + b (unit k, window b of the tile): 4 floats of padding
// after every 64, so the eight K eighths a wave reads (16·BT consecutive elements each) start
// on distinct banks.
__device__ __forceinline__ int hidx(int f) { return f + 4 * (f >> 6); }
template <int BT>
constexpr int kHLen = kHidden * BT + 4 * (kHidden * BT / 64);

// Register slot s of a lane holds row l ^ slot_row(s) of its 8-lane group (l = lane in the
// group): s = 4·b1 + 2·b2 + b3 maps to 7·b1 ^ 2·b2 ^ b3, the partners of the three reduction
// levels (half-row mirror l ^ 7, then l ^ 2, then l ^ 1).
__host__ __device__ constexpr int slot_row(int s) { return ((s & 4) ? 7 : 0) ^ ((s & 2) ? 2 : 0) ^ (s & 1); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kXor1 = 0xB1;       // quad_perm 1,0,3,2
constexpr int kXor2 = 0x4E;       // quad_perm 2,3,0,1
constexpr int kMirror8 = 0x141;   // row_half_mirror: lane l of each 8 reads lane 7 - l = l ^ 7
template <int L>
constexpr int kBcast = L * 0x55;  // quad_perm L,L,L,L: every lane reads quad lane L

// Activations on the hardware exp2 and reciprocal: σ(a) = 1/(1 + 2^(-a·log2 e)) and
// tanh(a) = 2σ(2a) - 1. The recurrent rows arrive pre-multiplied by -log2 e (i, f, o) or
// -2·log2 e (g) (kGateExpScale), and the gate input is scaled the same way, so a gate's sum is
// already the exponent z and rcp(1 + 2^z) is σ (i, f, o) or (tanh + 1)/2 (g). For z -> +inf,
// 2^z overflows to +inf and the reciprocal returns the exact limit 0, so no clamp is needed.
__device__ __forceinline__ float rcp_one_plus_exp2(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

template <int BT>
__device__ __forceinline__ float pick(const float (&v)[BT], int b) {
    // v[b] as a register vector element: a chain of selects over the array's elements is
    // turned by the optimizer into an indexed load from a stack copy of the array
    if constexpr (BT == 1) {
        return v[0];
    } else {
        typedef float vec_t __attribute__((ext_vector_type(BT)));
        vec_t x;
#pragma unroll
        for (int i = 0; i < BT; ++i) x[i] = v[i];
        return x[b];
    }
}

__device__ __forceinline__ unsigned long long load_word(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_word(unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N>
struct Slot {
    static constexpr int value = N;
};

// f(Slot<P>{}) for P = FIRST .. LAST - 1, as straight-line code.
template <int FIRST, int LAST, typename F>
__device__ __forceinline__ void for_slots(F &&f) {
    if constexpr (FIRST < LAST) {
        f(Slot<FIRST>{});
        for_slots<FIRST + 1, LAST>(f);
    }
}

// One layer's recurrence for this workgroup's tile and direction. `timed_out` is set once a
// wait has given up; every later wait of the workgroup then returns at once.
template <int KG, int BT, bool STREAM>
__device__ __forceinline__ void recurrence_layer(const RecurArgs &a, bool &timed_out) {
    constexpr int U = kHidden / KG;  // units per workgroup
    constexpr int NT = 4 * U;        // threads
    static_assert(KG == 1 || NT >= 128, "a polling wave besides the staging wave");
    static_assert(!STREAM || KG == 1, "streamed gates: single-workgroup tiles only");
    constexpr int kRing = STREAM && BT == 1 ? kRingStreamOne : (STREAM || (KG == 1 && BT == 1)) ? kRingOne : kRingPlain;

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
    const int u = tid >> 2;
    const int q = tid & 3;
    const int ug = member * U + u;  // global hidden unit of this quad
    const int win0 = tile * BT;
    // Window this lane writes: lane q < BT takes window q of the tile; the other lanes of the
    // quad, and lanes of windows past the batch, duplicate window 0 (always valid) so every
    // lane runs the same straight-line code and their stores are idempotent.
    const int qe = (q < BT && win0 + q < a.batch) ? q : 0;

    __shared__ __attribute__((aligned(16))) float hs[2][kHLen<BT>];
    __shared__ __attribute__((aligned(16))) float gs[KG > 1 ? 2 : 1][KG > 1 ? U * 4 * BT : 4];

    // ---- recurrent weights into VGPRs: slot s = row l ^ slot_row(s) of the lane's 8-lane
    // group (the group's rows are units 2·grp, 2·grp + 1 × gates i, f, g, o), K eighth l ------
    const int l8 = tid & 7;
    float rr[8][16];
    {
        const float *rgrp = a.r + (static_cast<size_t>(dir) * kGates + 4 * (member * U) + 8 * (tid >> 3)) * kHidden;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const v4f *p = reinterpret_cast<const v4f *>(rgrp + static_cast<size_t>(l8 ^ slot_row(sl)) * kHidden + 16 * l8);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const v4f x = p[v];
                rr[sl][4 * v + 0] = x[0];
                rr[sl][4 * v + 1] = x[1];
                rr[sl][4 * v + 2] = x[2];
                rr[sl][4 * v + 3] = x[3];
            }
        }
    }

    // h_{-1} = 0
    for (int i = tid; i < 2 * kHLen<BT>; i += NT) (&hs[0][0])[i] = 0.0f;

    auto time_of = [&](int s) { return dir == 0 ? s : steps - 1 - s; };
    // Gate input of gate q, unit ug, window b of the tile at step s. Steps past the end and
    // windows past the batch read in-bounds stand-ins (last step, window 0) whose values
    // nobody uses, so the loads need no branch.
    const size_t gate_col = static_cast<size_t>(dir) * kGates + 4 * ug + q;
    auto gate_in = [&](int b, int s) -> float {
        const int w = (win0 + b < a.batch) ? win0 + b : win0;
        const int sc = s < steps ? s : steps - 1;
        const float *p = a.gates + (static_cast<size_t>(w) * steps + time_of(sc)) * kGateCols + gate_col;
        if constexpr (STREAM) {
            return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            return *p;
        }
    };

    // STREAM: publication counter of the chunk holding step s (clamped to the last step) for
    // this tile's window group and direction
    const unsigned int *ready_tile =
        STREAM ? a.ready + static_cast<size_t>(dir) * a.groups + win0 / a.group_windows : nullptr;
    auto ready_ptr = [&](int s) {
        const int sc = s < steps ? s : steps - 1;
        return ready_tile + static_cast<unsigned int>(sc >> a.chunk_shift) * (2u * a.groups);
    };
    auto read_ready = [&](int s) -> unsigned int {
        return __hip_atomic_load(ready_ptr(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto published = [&](unsigned int v) { return chunk_published(v, a.ready_target); };
    // The counter read one group ahead: even lanes read the chunk of step s, odd lanes the one
    // after. The per-lane address keeps the value in a vector register across the group (a
    // value the compiler sees as uniform would be moved to a scalar register at once, which
    // waits for the load, and with it for every gate prefetch, right after it is issued).
    const int lane_chunk = (tid & 1) * a.chunk;
    auto read_ready_ahead = [&](int s) -> unsigned int {
        return __hip_atomic_load(ready_ptr(s + lane_chunk), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // Wait until the chunk of step s is published; `seen` is what read_ready_ahead(s) returned,
    // checked in lane 0 (an even lane) with a scalar compare.
    auto wait_ready = [&](unsigned int seen, int s) {
        if (__builtin_expect(published(__builtin_amdgcn_readfirstlane(seen)) || timed_out, 1)) return;
        const unsigned long long t0 = wall_clock64();
        while (true) {
            __builtin_amdgcn_s_sleep(1);
            if (published(read_ready(s))) break;
            if (wall_clock64() - t0 > a.timeout_ticks) {
                report_timeout(a.error, kErrCounter);
                timed_out = true;
                break;
            }
        }
    };
    unsigned int ready_seen = 0;  // counter of the chunk of the group after the current one
    // STREAM: progress[window][dir] = progress_pass | steps whose output stores have completed,
    // for every window of the tile (read by the next layer's projection). Written by wave 0
    // (`publisher`, a wave-uniform test, so no lane mask is set up); its lanes store the same
    // word.
    unsigned long long *const progress_tile = STREAM ? a.progress + kProgressStride * (2 * win0 + dir) : nullptr;
    const unsigned long long progress_pass = a.progress_pass;
    const bool publisher = __builtin_amdgcn_readfirstlane(tid) == 0;
    auto publish = [&](unsigned int done) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (win0 + b < a.batch) {
                __hip_atomic_store(progress_tile + kProgressStride * 2 * b, progress_word(progress_pass, done), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };
    float *const ycol = a.y + static_cast<size_t>(win0 + qe) * steps * kWidth + dir * kHidden + ug;
    // Single-workgroup tiles (KG = 1): the gate row of the next refill and the output row of
    // the current step are uniform pointers moved by one row per step (a scalar add; the
    // refill stops at the last step), instead of addresses rebuilt from the step index every
    // step: that arithmetic sat between the cell update and the barrier (measured: streamed
    // b32 forward 1.192 -> 1.159 ms, plain one-window recurrence -2 %, two-window -3.5 %).
    constexpr bool kRowPtrs = KG == 1;
    const long gate_row_step = dir == 0 ? kGateCols : -static_cast<long>(kGateCols);
    const long y_row_step = dir == 0 ? kWidth : -static_cast<long>(kWidth);
    const float *gate_row = a.gates + (static_cast<size_t>(win0) * steps + time_of(max(0, min(kRing, steps - 1)))) * kGateCols;
    float *y_row = a.y + (static_cast<size_t>(win0) * steps + time_of(0)) * kWidth;
    const int gate_off = static_cast<int>(gate_col);
    const size_t y_off = static_cast<size_t>(qe) * steps * kWidth + dir * kHidden + ug;
    // window b's gate rows relative to window 0's (windows past the batch read window 0's)
    size_t win_off[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) win_off[b] = win0 + b < a.batch ? static_cast<size_t>(b) * steps * kGateCols : 0;

    // KG == 1: per-lane register ring of gate inputs.
    float ring[kRing][BT];
    // KG > 1: wave 0 stages the workgroup's gates; lane j of wave 0 moves float4 j, j + 64 ...
    // (float4 j = window j / U, unit member·U + j % U)
    constexpr int kStageVec = KG > 1 ? (U * BT + 63) / 64 : 1;
    v4f stage[kRing][kStageVec];
    const bool stager = (KG > 1) && (tid < 64);
    auto stage_load = [&](int j, int s) -> v4f {
        const int w = win0 + j / U;
        if (j >= U * BT || w >= a.batch || s >= steps) return v4f{0.f, 0.f, 0.f, 0.f};
        return *reinterpret_cast<const v4f *>(
            a.gates + (static_cast<size_t>(w) * steps + time_of(s)) * kGateCols +
            static_cast<size_t>(dir) * kGates + 4 * (member * U + j % U));
    };

    if constexpr (KG == 1) {
        if constexpr (STREAM) {
            wait_ready(read_ready_ahead(0), 0);
            ready_seen = read_ready_ahead(kRing);
        }
#pragma unroll
        for (int p = 0; p < kRing; ++p)
#pragma unroll
            for (int b = 0; b < BT; ++b) ring[p][b] = gate_in(b, p);
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
    // Drain the prologue's loads (R, the first gate inputs) here, once. Left outstanding, they
    // make the compiler's wait counting conservative inside the step loop, where it would then
    // wait for every in-flight load — including the gate prefetches — at each step.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    unsigned long long *xdir = nullptr;
    if constexpr (KG > 1) {
        xdir = a.exchange + (static_cast<size_t>(dir) * a.tiles + tile) * 2 * kHidden * BT;
    }
    const bool is_g = q == 2;
    const float zscale = is_g ? kGateExpScale[2] : kGateExpScale[0];  // of gate q
    // The cell state is kept multiplied by kCellScale = -2·log2 e, the factor tanh's exponent
    // needs, so no multiply stands between c and its exponential.
    constexpr float kCellScale = kGateExpScale[2];
    float cst = 0.0f;  // kCellScale · cell state of (unit ug, window qe)

    // One step s; P is the step's slot in the prefetch ring (s mod kRing), a compile-time
    // constant so the ring stays in registers.
    auto step = [&](int s, auto slot) {
        constexpr int P = decltype(slot)::value;
        const int cur = s & 1;
        const int nxt = cur ^ 1;


        // (1) partial dot products of the lane's 8 rows over its K eighth; slot 0 (row l of the
        // group = gate q of unit ug) starts from that gate's scaled input, so the reduction
        // below yields the whole exponent
        float zin[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            float gin;
            if constexpr (KG == 1) {
                // Plain one-window kernel: keep the slot's use at its own step. Otherwise the
                // scheduler computes later slots' scaled inputs early, which waits for loads
                // issued only two steps before (vmcnt) instead of the ring's full depth.
                if constexpr (!STREAM && BT == 1) asm volatile("" : "+v"(ring[P][b]));
                gin = ring[P][b];
            } else {
                gin = gs[cur][4 * (b * U + u) + q];
            }
            zin[b] = gin * zscale;
        }
        float acc[8][BT];
        {
            const float *hp = &hs[cur][hidx(16 * l8 * BT)];
            // every LDS read of h first, so their latencies overlap (the FMAs then wait for
            // each in turn). Left to itself the compiler spaced them out in the streamed and
            // multi-window kernels; there a scheduling barrier keeps them together (measured:
            // streamed b32 forward 1.30 -> 1.298 ms, two windows 0.998 -> 0.955 us per step),
            // while it slows the plain one-window kernel (0.471 -> 0.491 us), already in order.
            // Four windows' h (64 registers) would not fit beside R and the 32 sums: there the compiler
            // schedules the reads.
            constexpr bool kUpfront = BT <= 2;
            v4f hv[kUpfront ? 4 * BT : 1];
            if constexpr (kUpfront) {
#pragma unroll
                for (int v = 0; v < 4 * BT; ++v) hv[v] = *reinterpret_cast<const v4f *>(hp + 4 * v);
                if constexpr (STREAM || BT > 1) __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (STREAM && P == 0) {
                // This group refills the ring with steps s + kRing .. s + 2·kRing - 1 (one
                // chunk): check the counter read a group ago, and read the one for the next
                // group. Done while the h reads above are in flight (measured: streamed b32
                // forward 1.150 -> 1.144 ms against doing it before them).
                wait_ready(ready_seen, s + kRing);
                ready_seen = read_ready_ahead(s + 2 * kRing);
                // Publish this tile's progress. Every wave has passed the previous step's
                // barrier and, before it, waited for the gate load issued kRing steps earlier;
                // vector memory operations complete in issue order, so every output store of
                // the steps before s - 2·kRing has completed.
                if (publisher) publish(static_cast<unsigned int>(s >= 2 * kRing ? s - 2 * kRing : 0));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int v = 0; v < 4 * BT; ++v) {
                const v4f h4 = kUpfront ? hv[v] : *reinterpret_cast<const v4f *>(hp + 4 * v);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int idx = 4 * v + e;  // = k_local·BT + b
                    const int kk = idx / BT;
                    const int b = idx % BT;
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) {
                        acc[sl][b] = kk != 0   ? fmaf(rr[sl][kk], h4[e], acc[sl][b])
                                     : sl == 0 ? fmaf(rr[0][0], h4[e], zin[b])
                                               : rr[sl][0] * h4[e];
                    }
                }
            }
        }

        // (2) reduce-scatter over the 8-lane group: lane l keeps row l's exponent (gate q of
        // unit ug), its eighths combined level by level with the partners l ^ 7, l ^ 2, l ^ 1
        float sum[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            float t[4];
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) t[sl] = acc[sl][b] + dpp<kMirror8>(acc[sl + 4][b]);
            const float u0 = t[0] + dpp<kXor2>(t[2]);
            const float u1 = t[1] + dpp<kXor2>(t[3]);
            sum[b] = u0 + dpp<kXor1>(u1);
        }

        // (3) σ of gate q for each window (i, f, o are read as they are; lane 2 turns its
        // value r into kCellScale·tanh = kCellScale·(2r - 1), one fma beside the broadcasts of
        // i and f), then every lane updates the cell of window qe
        float sig[BT], gsc[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            sig[b] = rcp_one_plus_exp2(sum[b]);
            gsc[b] = fmaf(2.0f * kCellScale, sig[b], -kCellScale);
        }
        float ig[BT], fg[BT], gg[BT], og[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            ig[b] = dpp<kBcast<0>>(sig[b]);
            fg[b] = dpp<kBcast<1>>(sig[b]);
            gg[b] = dpp<kBcast<2>>(gsc[b]);
            og[b] = dpp<kBcast<3>>(sig[b]);
        }
        const float i_w = pick<BT>(ig, qe), f_w = pick<BT>(fg, qe);
        const float g_w = pick<BT>(gg, qe), o_w = pick<BT>(og, qe);
        cst = fmaf(f_w, cst, i_w * g_w);
        // h = o·tanh(c) = 2o·rcp(1 + 2^(kCellScale·c)) - o
        const float hval = fmaf(o_w + o_w, rcp_one_plus_exp2(cst), -o_w);

        // h to LDS for the next step (lanes of one window write the same value)
        hs[nxt][hidx(ug * BT + qe)] = hval;
        const unsigned int flag = exchange_flag(a.flag_base, s);
        if constexpr (KG > 1) {
            if (q < BT) {
                store_word(xdir + exchange_index(s, ug, q, kHidden, BT), exchange_word(flag, __float_as_uint(hval)));
            }
        }

        if constexpr (KG == 1) {
            // refill this ring slot with step s + kRing
            if constexpr (kRowPtrs) {
#pragma unroll
                for (int b = 0; b < BT; ++b) {
                    const float *gp = gate_row + win_off[b] + gate_off;
                    ring[P][b] = STREAM ? __hip_atomic_load(gp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *gp;
                }
                gate_row = s + kRing + 1 < steps ? gate_row + gate_row_step : gate_row;
            } else {
#pragma unroll
                for (int b = 0; b < BT; ++b) ring[P][b] = gate_in(b, s + kRing);
            }
        } else {
            if (stager) {
                // stage[P] holds step s+1 (loaded kRing steps ago): into LDS slot nxt, then
                // load step s + 1 + kRing in its place
#pragma unroll
                for (int v = 0; v < kStageVec; ++v) {
                    const int j = tid + 64 * v;
                    if (j < U * BT) *reinterpret_cast<v4f *>(&gs[nxt][4 * j]) = stage[P][v];
                    stage[P][v] = stage_load(j, s + 1 + kRing);
                }
            } else {
                // (4) gather the other workgroups' h of step s
                constexpr int kOthers = (kHidden - U) * BT;
                const unsigned int expect = flag + a.flag_skew;
                for (int idx = tid - 64; idx < kOthers; idx += NT - 64) {
                    const int uo = idx / BT;
                    const int b = idx - uo * BT;
                    const int ugo = uo < member * U ? uo : uo + U;
                    const unsigned long long *wp = xdir + exchange_index(s, ugo, b, kHidden, BT);
                    unsigned long long w = load_word(wp);
                    if (word_flag(w) != expect && !timed_out) {
                        const unsigned long long t0 = wall_clock64();
                        while (true) {
                            w = load_word(wp);
                            if (word_flag(w) == expect) break;
                            if (wall_clock64() - t0 > a.timeout_ticks) {
                                report_timeout(a.error, kErrExchange);
                                timed_out = true;
                                break;
                            }
                        }
                    }
                    hs[nxt][hidx(ugo * BT + b)] = __uint_as_float(word_value(w));
                }
            }
        }

        float *const yp = kRowPtrs ? y_row + y_off : ycol + static_cast<size_t>(time_of(s)) * kWidth;
        if constexpr (STREAM) {
            __hip_atomic_store(yp, hval, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            *yp = hval;
        }
        if constexpr (kRowPtrs) y_row += y_row_step;
        __syncthreads();
    };

    // Full groups of kRing steps run as straight-line code (no per-step guards), which keeps
    // the compiler's memory-wait counting exact; the last partial group is guarded.
    int s0 = 0;
    for (; s0 + kRing <= steps; s0 += kRing) {
        for_slots<0, kRing>([&](auto slot) { step(s0 + decltype(slot)::value, slot); });
    }
    for_slots<0, kRing - 1>([&](auto slot) {
        if (s0 + decltype(slot)::value < steps) step(s0 + decltype(slot)::value, slot);
    });
    if constexpr (STREAM) {
        // every wave's output stores have completed: the whole sequence is published
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (publisher) publish(static_cast<unsigned int>(steps));
    }
}

// A workgroup is 512 / KG threads, i.e. 2 / KG waves per SIMD, and one workgroup runs per CU:
// telling the compiler so keeps it from trading the step's latency for a higher occupancy
// (squeezed to fit 3 waves, it serialized the LDS reads of h).
template <int KG, int BT>
__global__ __launch_bounds__(4 * (kHidden / KG)) __attribute__((amdgpu_waves_per_eu(KG == 1 ? 2 : 1, KG == 1 ? 2 : 1)))
void recurrence_kernel(RecurArgs a) {
    bool timed_out = false;
    recurrence_layer<KG, BT, false>(a, timed_out);
}

// Streamed gates: the recurrences of `layers` consecutive layers in one launch. Each
// workgroup keeps its tile and direction and goes from one layer to the next by itself: it
// reloads R and waits for the next layer's first chunk, which the next projection computes
// once every window of the chunk has finished this layer in both directions. No workgroup
// waits for another layer's launch, so the gap between layers is that first chunk's latency.
template <int BT>
__global__ __launch_bounds__(4 * kHidden) __attribute__((amdgpu_waves_per_eu(2, 2)))
void recurrence_stream_kernel(RecurStack st) {
    bool timed_out = false;
    if (st.stamps != nullptr && threadIdx.x == 0) atomicMax(st.stamps + kLayers, ~wall_clock64());
    for (int l = 0; l < st.layers; ++l) {
        recurrence_layer<1, BT, true>(st.layer[l], timed_out);
        // the layer ends with a workgroup barrier
        if (st.stamps != nullptr && threadIdx.x == 0) atomicMax(st.stamps + l, wall_clock64());
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
        const unsigned long long word = static_cast<unsigned long long>(r) << 32;
        if (is_a) {
            if (r == 1) t_start = wall_clock64();
            store_word(mine, word);
        }
        const unsigned long long t0 = wall_clock64();
        while (true) {
            const unsigned long long v = load_word(theirs);
            if (static_cast<unsigned int>(v >> 32) == static_cast<unsigned int>(r)) break;
            if (wall_clock64() - t0 > timeout_ticks) {
                ok = false;
                break;
            }
        }
        if (!is_a) store_word(mine, word);
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

// FMA issue rate: each wave runs `iters` rounds of 128 FMAs over 8 independent accumulators per
// lane, the shape of the recurrence's product loop (128 FMAs per lane and step, 8 sums). The
// workgroup's waves are dealt over the CU's four SIMDs, so a workgroup of 256·w threads puts w
// waves on each. Thread 0 records the elapsed shader clocks and wall-clock ticks of the timed
// loop, between two barriers.
__global__ __launch_bounds__(1024) void fma_rate_kernel(int iters, float seed, unsigned long long *out, float *sink) {
    // acc += w·h with register operands, as the recurrence's products (v_fmac_f32)
    float acc[8], w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc[i] = seed * static_cast<float>(i + 1) + 1e-7f * static_cast<float>(threadIdx.x);
        w[i] = 1e-3f * seed * static_cast<float>(i + 2);
    }
    float h = seed + 1e-9f * static_cast<float>(threadIdx.x);
    __syncthreads();
    const unsigned long long t0 = __builtin_readcyclecounter();
    const unsigned long long w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[i], h, acc[i]);
        asm volatile("" : "+v"(h));  // a fresh operand each round: the products are not hoisted
    }
    __syncthreads();
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long w1 = wall_clock64();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = w1 - w0;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += acc[i];
    if (sum == 12345.0f) sink[threadIdx.x] = sum;  // keeps the products live; never true here
}

template <int KG, int BT>
hipError_t launch_typed(const RecurArgs &args, int directions, size_t lds, hipStream_t stream) {
    const int nwg = KG == 1 ? args.tile_count : (args.tile_count + 7) / 8 * 8 * KG;
    if (args.chunk > 0) {
        if constexpr (KG == 1) {
            RecurStack st{};
            st.layer[0] = args;
            st.layers = 1;
            hipLaunchKernelGGL((recurrence_stream_kernel<BT>), dim3(nwg, directions), dim3(recur_threads(KG)), lds,
                               stream, st);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((recurrence_kernel<KG, BT>), dim3(nwg, directions), dim3(recur_threads(KG)), lds, stream,
                       args);
    return hipGetLastError();
}

template <int KG, int BT>
hipError_t allow_lds_typed(size_t bytes) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&recurrence_kernel<KG, BT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
    if (e != hipSuccess || KG != 1) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&recurrence_stream_kernel<BT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

template <int KG, int BT>
hipError_t occupancy_typed(int *per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, recurrence_kernel<KG, BT>, recur_threads(KG), 0);
}

#define BL_FOR_EACH_SPLIT(X) X(1, 1) X(1, 2) X(1, 4) X(2, 1) X(2, 2) X(2, 4) X(4, 1) X(4, 2) X(4, 4)

}  // namespace

hipError_t launch_recurrence(int groups, int tile, const RecurArgs &args, int directions,
                             size_t dynamic_lds, hipStream_t stream) {
    if (args.tile_count <= 0) return hipSuccess;
#define BL_CASE(KG, BT) \
    if (groups == KG && tile == BT) return launch_typed<KG, BT>(args, directions, dynamic_lds, stream);
    BL_FOR_EACH_SPLIT(BL_CASE)
#undef BL_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_recurrence_stack(int tile, const RecurStack &stack, size_t dynamic_lds, hipStream_t stream) {
    const RecurArgs &a = stack.layer[0];
    if (stack.layers < 1 || stack.layers > kLayers || a.tile_count <= 0 || a.direction != 0) {
        return hipErrorInvalidValue;
    }
    for (int l = 0; l < stack.layers; ++l) {
        const RecurArgs &b = stack.layer[l];
        if (b.chunk <= 0 || b.tile_first != a.tile_first || b.tile_count != a.tile_count || b.direction != 0) {
            return hipErrorInvalidValue;
        }
    }
    const dim3 grid(a.tile_count, 2);
    switch (tile) {
        case 1:
            hipLaunchKernelGGL(recurrence_stream_kernel<1>, grid, dim3(recur_threads(1)), dynamic_lds, stream, stack);
            break;
        case 2:
            hipLaunchKernelGGL(recurrence_stream_kernel<2>, grid, dim3(recur_threads(1)), dynamic_lds, stream, stack);
            break;
        case 4:
            hipLaunchKernelGGL(recurrence_stream_kernel<4>, grid, dim3(recur_threads(1)), dynamic_lds, stream, stack);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t recurrence_allow_lds(int groups, int tile, size_t bytes) {
#define BL_CASE(KG, BT) \
    if (groups == KG && tile == BT) return allow_lds_typed<KG, BT>(bytes);
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

hipError_t run_fma_probe(int waves_per_simd, int workgroups, int iters, double wall_khz, double *clocks_per_fma,
                         double *ghz) {
    unsigned long long *out = nullptr;
    float *sink = nullptr;
    hipError_t e = hipMalloc(&out, 2 * static_cast<size_t>(workgroups) * sizeof(unsigned long long));
    if (e != hipSuccess) return e;
    e = hipMalloc(&sink, 1024 * sizeof(float));
    if (e != hipSuccess) {
        (void)hipFree(out);
        return e;
    }
    std::vector<unsigned long long> host(2 * static_cast<size_t>(workgroups));
    hipLaunchKernelGGL(fma_rate_kernel, dim3(workgroups), dim3(256 * waves_per_simd), 0, nullptr, iters, 0.5f, out,
                       sink);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(host.data(), out, host.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    (void)hipFree(out);
    (void)hipFree(sink);
    if (e != hipSuccess) return e;
    // the median workgroup: clocks per wave64 FMA per SIMD, and shader clocks per wall-clock tick
    std::vector<double> cpf(workgroups), rate(workgroups);
    const double fmas_per_simd = static_cast<double>(waves_per_simd) * iters * 128.0;
    for (int g = 0; g < workgroups; ++g) {
        cpf[g] = static_cast<double>(host[2 * g]) / fmas_per_simd;
        rate[g] = host[2 * g + 1] > 0 ? static_cast<double>(host[2 * g]) / static_cast<double>(host[2 * g + 1]) : 0.0;
    }
    std::nth_element(cpf.begin(), cpf.begin() + workgroups / 2, cpf.end());
    std::nth_element(rate.begin(), rate.begin() + workgroups / 2, rate.end());
    *clocks_per_fma = cpf[workgroups / 2];
    *ghz = rate[workgroups / 2] * wall_khz * 1e-6;
    return hipSuccess;
}

}  // namespace bl
