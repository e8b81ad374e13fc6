// Internal declarations shared by the host plan code and the HIP kernels of the
// bidirectional LSTM library. Not part of the public ABI (include/bilstm.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "protocol.h"

namespace bl {

constexpr int kHidden = 128;               // H
constexpr int kGates = 512;                // 4H gate rows per direction
constexpr int kGateCols = 1024;            // both directions side by side in the gate buffer
constexpr int kWidth = 256;                // 2H
constexpr int kFeatures = 60;
constexpr int kLayers = 4;

// Projection GEMM tile (rows x gate columns) and K step.
constexpr int kProjTileM = 128;
constexpr int kProjTileN = 128;
constexpr int kProjTileK = 32;
constexpr int kProjThreads = 256;
// LDS of one projection workgroup (two stages of A and B tiles, rows padded to 36 floats) and
// of one CU.
constexpr size_t kProjLdsBytes = 2 * 2 * kProjTileM * (kProjTileK + 4) * sizeof(float);
constexpr size_t kCuLdsBytes = 160 * 1024;

// Batch slices of a forward pass (concurrent chains of layers on their own streams). A HIP
// process gets 4 hardware queues by default; streams beyond that share queues and serialize
// (measured: 4 slices ran slower than 1), so the automatic choice stays at 2.
constexpr int kMaxSlices = 8;
constexpr int kAutoSlices = 2;

inline int padded_input(int in) { return (in + kProjTileK - 1) / kProjTileK * kProjTileK; }

// bilstm_options.projection values
constexpr int kProjectionAuto = 0;    // the plan's rule (host_pack_schedule.cpp)
constexpr int kProjectionVendor = 1;  // hipBLASLt, FP32 compute (comparator)
constexpr int kProjectionSplit2 = 2;  // two bf16 parts, three products
constexpr int kProjectionSplit3 = 3;  // three bf16 parts, six products
constexpr int kProjectionFp32 = 4;    // FP32 MFMA products

// Factor of each gate's pre-activation in the exponent of its activation, by gate (i, f, g,
// o): σ(a) = 1/(1 + 2^(-a·log2 e)) and tanh(a) = 2/(1 + 2^(-2a·log2 e)) - 1. The plan stores the
// recurrent rows multiplied by these factors (rounded to fp32).
__host__ __device__ constexpr float gate_exp_scale(int gate) {
    return gate == 2 ? -2.8853900817779268f : -1.4426950408889634f;
}
__device__ constexpr float kGateExpScale[4] = {gate_exp_scale(0), gate_exp_scale(1), gate_exp_scale(2),
                                               gate_exp_scale(3)};

// Threads per recurrence workgroup for `groups` workgroups per (direction, tile): four lanes
// per hidden unit.
inline int recur_threads(int groups) { return 4 * (kHidden / groups); }

// Exchange words of one direction: [tiles][2 parities][128 units][tile] u64 words.
inline size_t exchange_words_per_direction(int tiles, int tile) {
    return static_cast<size_t>(tiles) * 2 * kHidden * tile;
}

// Watchdog reports. A wait that gives up stores 1 into the word of its kind; the plan keeps
// the words in host-mapped coherent memory, so the host reads them without a device
// synchronization, and the next call on the plan reports them.
constexpr int kErrExchange = 0;  // a recurrence exchange wait (flagged h words)
constexpr int kErrCounter = 1;   // a recurrence wait for a chunk counter (streamed gates)
constexpr int kErrProgress = 2;  // a projection wait for the previous layer's progress
constexpr int kErrWords = 4;

struct ProjArgs {
    const float *x;      // [rows][in]
    const float *w;      // [1024][kpad]
    const __bf16 *w_hi;  // split-precision mode: [1024][kpad] bf16(w), else nullptr
    const __bf16 *w_lo;  //                       [1024][kpad] bf16(w - bf16(w))
    const __bf16 *w_lo2; // three parts: [1024][kpad] bf16 of what the first two leave, else nullptr
    int split_parts;     // 0: FP32 MFMA; 2 or 3: bf16 parts (the streamed kernel splits W itself)
    const float *bias;   // [1024]
    float *gates;        // [rows][1024]
    int rows;
    int in;
    int kpad;
    int row_tiles;       // ceil(rows / kProjTileM)
    int tiles;           // row_tiles * (1024 / kProjTileN)
    // Streamed order (chunk > 0): tiles follow the recurrence's consumption order and each
    // finished tile is published on `ready` (layout below). chunk = 0: plain row-major tiles.
    int chunk;           // recurrence steps per tile row block (128 / group_windows)
    int chunk_shift;     // log2(chunk)
    int group_windows;   // windows per tile row block
    int groups;          // ceil(batch / group_windows)
    int split;           // tiles of chunk 0 per 128 gate columns (stream_split)
    int batch;
    int steps;
    unsigned int *ready;      // [chunks][2][groups] publication counters
    // Inputs written by the previous layer's recurrence while this projection runs
    // (progress != nullptr): before each K half of a tile's rows is read, each of its windows'
    // progress word in the direction that wrote that half must reach progress_pass | steps the
    // rows need (see StreamLayout); the rows are then read with agent-scope loads.
    const unsigned long long *progress;  // [batch][2], kProgressStride words apart
    unsigned long long progress_pass;    // (previous layer's pass number) << 32
    unsigned int *error;                 // [kErrWords] watchdog reports
    unsigned long long timeout_ticks;
};

struct RecurArgs {
    const float *gates;            // [batch*steps][1024], bias included
    const float *r;                // [2][512][128] packed rows 4j+g
    float *y;                      // [batch][steps][256]
    unsigned long long *exchange;  // [2][tiles][2][128][tile] words (groups > 1)
    unsigned int *error;           // [kErrWords] watchdog reports
    int batch;
    int steps;
    int direction;                 // direction of blockIdx.y == 0
    int tiles;                     // window tiles in the whole batch
    int tile_first;                // first tile of this launch
    int tile_count;                // tiles in this launch
    unsigned int flag_base;        // flags of this layer are flag_base + s + 1
    unsigned int flag_skew;        // added to the flag a wait expects: 0, or a value no
                                   // producer writes (forced-timeout tests)
    unsigned long long timeout_ticks;  // watchdog, in wall-clock ticks
    // Streamed gates (chunk > 0): before reading the gates of steps [c·chunk, (c+1)·chunk) of
    // window group g, wait until ready[(c·2 + dir)·groups + g] reaches ready_target.
    const unsigned int *ready;
    int chunk;                     // a power of two
    int chunk_shift;               // log2(chunk)
    int group_windows;
    int groups;
    unsigned int ready_target;
    // Streamed gates: the output is written with agent-scope stores and, every few steps, each
    // window's progress[window][dir] = progress_pass | (steps whose output has completed).
    unsigned long long *progress;
    unsigned long long progress_pass;
};

// Streamed gates: the recurrences of `layers` consecutive layers (layer[0] first) in one
// launch of tile_count tiles × both directions; every entry has chunk > 0, direction 0 and the
// same tiles.
struct RecurStack {
    RecurArgs layer[kLayers];
    int layers;
    // Phase timing, or nullptr: stamps[l] = the latest end of layer l over the workgroups and
    // stamps[kLayers] = ~(the earliest start), in wall-clock ticks (atomic maxima over words
    // cleared to zero before the launch).
    unsigned long long *stamps;
};

// Segmentation heads after the stack: 256 -> 128 -> 128 -> 7 (class slots padded to 8).
constexpr int kHeadIn = 256;
constexpr int kHeadMid = 128;
constexpr int kHeadClasses = 7;
constexpr int kHeadClassSlots = 8;
constexpr int kHeadTileRows = 32;
constexpr int kHeadThreads = 256;

struct HeadArgs {
    const float *y;    // [rows][256]
    float *out;        // [rows][7]
    const float *w0t;  // [128][256]  linear0 weight transposed ([n][k])
    const float *b0;   // [128]
    const float *w1t;  // [128][128]
    const float *b1;   // [128]
    const float *w2t;  // [8][128]    classifier weight transposed, slot 7 zero
    const float *b2;   // [7]
    float slope;       // LeakyReLU negative slope
    long rows;
};

// StreamLayout. Streamed projection: each layer's projection runs beside the recurrences
// and publishes its gates chunk by chunk in the order the recurrence reads them. A tile row
// block holds `group_windows` windows × `chunk` steps (128 rows): row r is window
// g·group_windows + r / chunk at step s = c·chunk + r % chunk of direction d, i.e. time s
// (forward) or steps - 1 - s (reverse); rows past the batch or past the last step are
// skipped. The walk goes chunk by chunk, the order the recurrence reads them. Chunk 0 comes
// first, in tiles of 128 / split columns: tile q = (d·groups + g)·4·split + column tile,
// columns d·512 + (128 / split)·(column tile). Then chunks c >= 1 in tiles of 128 columns:
// tile 2·groups·4·split + ((c·2 + d - 2)·groups + g)·4 + column tile. Narrow first tiles
// spread the chunk a layer boundary waits for over more workgroups. A tile of width W adds
// W / 32 to ready[(c·2 + d)·groups + g] once all its gates are stored with agent-scope stores
// and those stores have completed, so a pass adds kReadyPerPass to every counter.
// A tile of layer l + 1 reads the times of its chunk, all 256 columns, of layer l's output:
// forward output (k < 128) up to the chunk's last time t_hi (written at forward step t_hi) and
// reverse output (k >= 128) down to its first time t_lo (written at reverse step T-1-t_lo).
// For chunk c of direction d, layer l's direction d must have run stream_near(c) = min(c·chunk
// + chunk, T) steps and its other direction stream_far(c) = T - c·chunk steps. A tile of
// direction d sums the K half of direction d first (forward half first for d = 0, reverse
// half first for d = 1, in every FP32 projection kernel, so the sums are the same bits), so it
// waits for stream_near(c) of direction d before its first half and stream_far(c) of the other
// before its second: the first halves are ready early in layer l, and at its end only the
// second halves of the first chunks are left.
static_assert(kReadyPerPass == kGates / 32, "a pass adds width / 32 per tile over 512 columns");
// Tiles of chunk 0 per 128 gate columns: as many as keep every one of them in the first round
// of `workgroups` persistent projection workgroups (1, 2 or 4).
inline int stream_split(int groups, int workgroups) {
    int split = 4;
    while (split > 1 && 2 * groups * (kGates / kProjTileN) * split > workgroups) split /= 2;
    return split;
}
// Persistent workgroups of a streamed projection: the CUs the recurrence's workgroups (one
// per CU) leave free, a multiple of 8, at least 8.
inline int stream_projection_workgroups(int cu_count, int recur_tiles, int recur_groups) {
    const int free_cus = (cu_count - 2 * recur_tiles * recur_groups) / 8 * 8;
    return free_cus > 8 ? free_cus : 8;
}
// Tiles of a streamed projection pass.
inline int stream_tiles(int chunks, int groups, int split) {
    return (chunks - 1 + split) * 2 * groups * (kGates / kProjTileN);
}
inline int stream_chunks(int steps, int chunk) { return (steps + chunk - 1) / chunk; }
// Progress words one 128-byte line apart: each window's direction has its own line, so the
// recurrence's stores and the projection's polls of different windows never share one.
constexpr int kProgressStride = 16;
__host__ __device__ inline int stream_near(int steps, int chunk, int c) {
    return c * chunk + chunk < steps ? c * chunk + chunk : steps;
}
__host__ __device__ inline int stream_far(int steps, int chunk, int c) { return steps - c * chunk; }

// Launchers (kernels_*.hip). They return the launch's hipError_t.
hipError_t launch_heads(const HeadArgs &args, hipStream_t stream);
#ifdef __HIP__  // HIP-language sources only; the host .cpp files include this header as C++
// Report a wait that gave up (one system-scope store; the host may be reading the word).
__device__ __forceinline__ void report_timeout(unsigned int *error, int kind) {
    __hip_atomic_store(error + kind, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
#endif
// The projection on `workgroups` persistent workgroups (one per CU; rounded to a multiple of 8).
// The streamed kernel's 128 KB K-step ring keeps two of its workgroups off one CU (2 · 128 KB
// > 160 KB), so its persistent grid spreads one per CU.
hipError_t launch_projection(const ProjArgs &args, int workgroups, hipStream_t stream);
hipError_t launch_recurrence(int groups, int tile, const RecurArgs &args, int directions,
                             size_t dynamic_lds, hipStream_t stream);
// The streamed recurrences of several layers in one launch (single-workgroup tiles of `tile`
// windows).
hipError_t launch_recurrence_stack(int tile, const RecurStack &stack, size_t dynamic_lds, hipStream_t stream);
// Allow `bytes` of dynamic LDS per recurrence workgroup of this split.
hipError_t recurrence_allow_lds(int groups, int tile, size_t bytes);
hipError_t launch_exchange_clear(unsigned long long *words, size_t count, hipStream_t stream);
hipError_t recurrence_occupancy(int groups, int tile, int *per_cu);
hipError_t run_exchange_probe(int same_xcd, int round_trips, unsigned long long timeout_ticks,
                              double ticks_per_ns, double *one_way_ns, int *xcd_a, int *xcd_b);
hipError_t run_fma_probe(int waves_per_simd, int workgroups, int iters, double wall_khz, double *clocks_per_fma,
                         double *ghz);
// matrix-core rate: kind 0 bf16 32x32x16, 1 FP32 32x32x2; data 0 zeros, 1 ones, 2 uniform [-1, 1)
hipError_t run_mfma_probe(int kind, int data, int iters, int cu_count, double *tflops, double *ms);

}  // namespace bl
