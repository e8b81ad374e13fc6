// The C ABI of the library: plan creation (weight packing, scratch, side stream), the
// forward pass and the per-phase entry points (speakrs 0.6.0, page `lstmproj.rs`:
// `with_recurrence`, `Oxide::enqueue`, `Oxide::recur`, `clear_state`, `check_len`, `to_u32`).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/bilstm.h"
#include "bilstm_host.h"

namespace bl {

namespace {
thread_local std::string g_last_error;

// Watchdog of a recurrence wait, in milliseconds. A step normally takes microseconds; the
// limit only has to end a wait whose producer can never arrive.
constexpr double kWatchdogMs = 2000.0;
}  // namespace

bilstm_status fail(bilstm_status status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

bilstm_status check_len(const char *context, size_t expected, size_t actual) {
    if (expected == actual) return BILSTM_OK;
    return fail(BILSTM_BUFFER_LENGTH, "%s: expected %zu elements, got %zu", context, expected, actual);
}

}  // namespace bl

using namespace bl;

struct bilstm_plan {
    int device = 0;
    uint32_t batch = 0;
    uint32_t steps = 0;
    size_t rows = 0;
    bilstm_plan_info info{};
    int in[kLayers] = {kFeatures, kWidth, kWidth, kWidth};
    int kpad[kLayers] = {0, 0, 0, 0};
    float *w[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    float *r[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    float *bias[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    uint16_t *w_hi[kLayers] = {nullptr, nullptr, nullptr, nullptr};  // split precision: bf16(w)
    uint16_t *w_lo[kLayers] = {nullptr, nullptr, nullptr, nullptr};  //   bf16(w - bf16(w))
    uint16_t *w_lo2[kLayers] = {nullptr, nullptr, nullptr, nullptr}; //   three parts: the third
    float *gates = nullptr;
    unsigned long long *exchange = nullptr;
    size_t exchange_words = 0;
    unsigned int *error = nullptr;       // device address of the watchdog reports
    unsigned int *error_host = nullptr;  // the same kErrWords words, host-mapped
    hipEvent_t done = nullptr;           // recorded on the caller's stream at the end of every call
    uint32_t clears = 0;                 // clears of the exchange words or streamed counters
    hipStream_t side = nullptr;
    hipEvent_t fork[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t join[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    bool phase_events = false;
    hipEvent_t ev_start = nullptr;
    hipEvent_t ev_proj[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t ev_recur[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t ev_launch0[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t ev_launch1[kLayers] = {nullptr, nullptr, nullptr, nullptr};
    bool phases_recorded = false;
    bool phases_streamed = false;  // the recorded forward streamed its gates
    // batch slices: each runs its own chain of layers on its own stream
    hipStream_t slice_stream[kMaxSlices] = {};
    hipEvent_t slice_fork = nullptr;
    hipEvent_t slice_first[kMaxSlices] = {};  // after the slice's first projection
    hipEvent_t slice_join[kMaxSlices] = {};
    // streamed gates: the projection's stream, the second layer buffer, the chunk counters
    hipStream_t proj_stream = nullptr;
    hipEvent_t proj_fork = nullptr;
    hipEvent_t proj_join = nullptr;
    hipEvent_t layer_done[kLayers] = {nullptr, nullptr, nullptr, nullptr};  // no layer overlap
    hipEvent_t proj_done[kLayers] = {nullptr, nullptr, nullptr, nullptr};   // kernels one at a time
    float *ybuf = nullptr;                 // [rows][256]: output of layers 0 and 2
    float *gates_odd = nullptr;            // [rows][1024]: gates of layers 1 and 3
    // chunk counters of the two gate buffers (two per word): buffer b at b·ready_words
    unsigned long long *ready = nullptr;
    size_t ready_words = 0;
    unsigned long long *progress = nullptr;  // [batch][2] recurrence progress words
    unsigned long long *stamps = nullptr;    // phase timing of a one-launch recurrence (after progress)
    bool phases_fused = false;               // the recorded forward ran its recurrences as one launch
    int stream_groups = 0;
    int stream_chunks = 0;
    uint32_t ready_passes[2] = {0, 0};  // streamed passes per gate buffer since the last clear
    uint32_t layer_pass = 0;            // streamed layer passes since the last clear
    bool ready_dirty = false;    // a streamed pass failed to enqueue: zero the counters first
    int proj_workgroups_streamed = 0;
    size_t reserve_lds = 0;  // dynamic LDS of a recurrence workgroup (keeps its CU to itself)
    LibraryProjection *library = nullptr;  // vendor-GEMM projection (comparator), if chosen
    int proj_workgroups = 0;         // CUs for the persistent projection on an idle GPU
    int proj_workgroups_sliced = 0;  // ... beside the other slices' recurrences
    uint32_t epoch = 0;  // flags of the next pass start above this value
    unsigned long long timeout_ticks = 0;
    unsigned int flag_skew = 0;
    double watchdog_ms = 0.0;
    double wall_khz = 0.0;  // wall-clock ticks per millisecond
    uint64_t device_bytes = 0;
};

namespace {

// float -> bf16 bits, round to nearest even (the weights are finite)
uint16_t bf16_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, sizeof(u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

float bf16_value(uint16_t h) {
    const uint32_t u = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &u, sizeof(f));
    return f;
}

// Make `device` current for the scope and restore the caller's device afterwards.
class DeviceScope {
public:
    explicit DeviceScope(int device) {
        ok_ = hipGetDevice(&saved_) == hipSuccess;
        err_ = hipSetDevice(device);
    }
    ~DeviceScope() {
        if (ok_) (void)hipSetDevice(saved_);
    }
    hipError_t error() const { return err_; }

private:
    int saved_ = 0;
    bool ok_ = false;
    hipError_t err_ = hipSuccess;
};

#define BL_HIP(expr, context)                                                                \
    do {                                                                                     \
        hipError_t bl_e_ = (expr);                                                           \
        if (bl_e_ != hipSuccess) {                                                           \
            return fail(BILSTM_HIP_ERROR, "%s: %s failed: %s", context, #expr,               \
                        hipGetErrorString(bl_e_));                                           \
        }                                                                                    \
    } while (0)

template <typename T>
bilstm_status device_alloc(bilstm_plan *p, T **out, size_t count, const char *what) {
    void *ptr = nullptr;
    const size_t bytes = count * sizeof(T) > 0 ? count * sizeof(T) : 16;
    hipError_t e = hipMalloc(&ptr, bytes);
    if (e != hipSuccess) {
        return fail(BILSTM_HIP_ERROR, "plan_create: hipMalloc of %zu bytes for %s failed: %s", bytes,
                    what, hipGetErrorString(e));
    }
    *out = static_cast<T *>(ptr);
    p->device_bytes += bytes;
    return BILSTM_OK;
}

void release(bilstm_plan *p) {
    if (p == nullptr) return;
    DeviceScope scope(p->device);
    (void)hipDeviceSynchronize();
    for (int l = 0; l < kLayers; ++l) {
        if (p->w[l]) (void)hipFree(p->w[l]);
        if (p->r[l]) (void)hipFree(p->r[l]);
        if (p->bias[l]) (void)hipFree(p->bias[l]);
        if (p->w_hi[l]) (void)hipFree(p->w_hi[l]);
        if (p->w_lo[l]) (void)hipFree(p->w_lo[l]);
        if (p->w_lo2[l]) (void)hipFree(p->w_lo2[l]);
        if (p->fork[l]) (void)hipEventDestroy(p->fork[l]);
        if (p->join[l]) (void)hipEventDestroy(p->join[l]);
        if (p->ev_proj[l]) (void)hipEventDestroy(p->ev_proj[l]);
        if (p->ev_recur[l]) (void)hipEventDestroy(p->ev_recur[l]);
        if (p->ev_launch0[l]) (void)hipEventDestroy(p->ev_launch0[l]);
        if (p->ev_launch1[l]) (void)hipEventDestroy(p->ev_launch1[l]);
    }
    if (p->ev_start) (void)hipEventDestroy(p->ev_start);
    for (int i = 0; i < kMaxSlices; ++i) {
        if (p->slice_stream[i]) (void)hipStreamDestroy(p->slice_stream[i]);
        if (p->slice_first[i]) (void)hipEventDestroy(p->slice_first[i]);
        if (p->slice_join[i]) (void)hipEventDestroy(p->slice_join[i]);
    }
    if (p->slice_fork) (void)hipEventDestroy(p->slice_fork);
    if (p->proj_fork) (void)hipEventDestroy(p->proj_fork);
    if (p->proj_join) (void)hipEventDestroy(p->proj_join);
    for (int l = 0; l < kLayers; ++l) {
        if (p->layer_done[l]) (void)hipEventDestroy(p->layer_done[l]);
        if (p->proj_done[l]) (void)hipEventDestroy(p->proj_done[l]);
    }
    if (p->proj_stream) (void)hipStreamDestroy(p->proj_stream);
    if (p->ybuf) (void)hipFree(p->ybuf);
    if (p->gates_odd) (void)hipFree(p->gates_odd);
    if (p->ready) (void)hipFree(p->ready);
    if (p->progress) (void)hipFree(p->progress);
    if (p->library) library_projection_destroy(p->library);
    if (p->gates) (void)hipFree(p->gates);
    if (p->exchange) (void)hipFree(p->exchange);
    if (p->error_host) (void)hipHostFree(p->error_host);
    if (p->done) (void)hipEventDestroy(p->done);
    if (p->side) (void)hipStreamDestroy(p->side);
    delete p;
}

bool is_gfx950(int device) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return false;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t a_bytes, const void *b, size_t b_bytes) {
    const auto x = reinterpret_cast<uintptr_t>(a);
    const auto y = reinterpret_cast<uintptr_t>(b);
    return x < y + b_bytes && y < x + a_bytes;
}

// Reserve `count` flag values for the next pass. Stale words must never match a flag a wait
// expects (speakrs 0.6.0, page `lstmproj.rs`, `clear_state`, where the words are zeroed at the
// start of every pass). Here they are zeroed at plan creation and whenever the 32-bit flag
// space would wrap; in between, each pass uses flag values above every earlier pass's.
bilstm_status reserve_flags(bilstm_plan *p, uint32_t count, hipStream_t stream, uint32_t *base) {
    if (p->exchange == nullptr) {
        *base = 0;
        return BILSTM_OK;
    }
    uint32_t epoch = p->epoch;
    bool clear = false;
    const uint32_t first = reserve_flag_range(epoch, count, clear);
    if (clear) {
        BL_HIP(launch_exchange_clear(p->exchange, p->exchange_words, stream), "exchange clear");
        ++p->clears;
    }
    p->epoch = epoch;
    *base = first;
    return BILSTM_OK;
}

// The projection of rows [row_first, row_first + rows) of x into the same rows of gates.
// streamed: the whole batch in the recurrence's order, published on the plan's counters.
bilstm_status enqueue_projection(bilstm_plan *p, int layer, const float *x, float *gates,
                                 hipStream_t stream, size_t row_first, size_t rows, int workgroups,
                                 bool streamed = false, int buffer = 0) {
    if (p->library != nullptr) {
        // the vendor GEMM was planned for the whole batch, which it always runs unsliced
        if (row_first != 0 || rows != p->rows) {
            return fail(BILSTM_UNSUPPORTED, "projection: the vendor GEMM runs the whole batch only");
        }
        return library_projection_run(p->library, layer, x, p->w[layer], gates, stream);
    }
    ProjArgs args{};
    args.x = x + row_first * p->in[layer];
    args.w = p->w[layer];
    args.w_hi = reinterpret_cast<const __bf16 *>(p->w_hi[layer]);
    args.w_lo = reinterpret_cast<const __bf16 *>(p->w_lo[layer]);
    args.w_lo2 = reinterpret_cast<const __bf16 *>(p->w_lo2[layer]);
    args.split_parts = p->info.projection == kProjectionSplit2 ? 2 : p->info.projection == kProjectionSplit3 ? 3 : 0;
    args.bias = p->bias[layer];
    args.gates = gates + row_first * kGateCols;
    args.rows = static_cast<int>(rows);
    args.in = p->in[layer];
    args.kpad = p->kpad[layer];
    args.row_tiles = static_cast<int>((rows + kProjTileM - 1) / kProjTileM);
    args.tiles = args.row_tiles * (kGateCols / kProjTileN);
    if (streamed) {
        const int chunk = p->info.stream_chunk;
        args.chunk = chunk;
        while ((1 << args.chunk_shift) < chunk) ++args.chunk_shift;
        args.group_windows = kProjTileM / chunk;
        args.groups = p->stream_groups;
        args.batch = static_cast<int>(p->batch);
        args.steps = static_cast<int>(p->steps);
        args.ready = reinterpret_cast<unsigned int *>(p->ready + buffer * p->ready_words);
        args.split = p->info.stream_split;
        args.tiles = stream_tiles(p->stream_chunks, args.groups, args.split);
        args.error = p->error;
        args.timeout_ticks = p->timeout_ticks;
        if (layer > 0 && p->info.stream_overlap) {
            // the previous layer's recurrence, running now, still writes the input: each tile
            // waits for its rows
            args.progress = p->progress;
            args.progress_pass = progress_pass_bits(p->layer_pass - 1);
        }
    }
    BL_HIP(launch_projection(args, workgroups, stream), "projection launch");
    return BILSTM_OK;
}

// Both directions' recurrence of one layer over window tiles [tile_lo, tile_hi) (speakrs
// 0.6.0, page `lstmproj.rs`, `Oxide::recur`: the reverse direction on the side stream when
// the schedule allows it, joined back before the next layer).
RecurArgs recurrence_args(const bilstm_plan *p, int layer, const float *gates, float *y, uint32_t flag_base,
                          bool streamed, int buffer) {
    const bilstm_plan_info &s = p->info;
    RecurArgs base{};
    base.gates = gates;
    base.r = p->r[layer];
    base.y = y;
    base.exchange = p->exchange;
    base.error = p->error;
    base.batch = static_cast<int>(p->batch);
    base.steps = static_cast<int>(p->steps);
    base.tiles = s.recur_tiles;
    base.flag_base = flag_base;
    base.timeout_ticks = p->timeout_ticks;
    base.flag_skew = p->flag_skew;
    if (streamed) {
        base.ready = reinterpret_cast<const unsigned int *>(p->ready + buffer * p->ready_words);
        base.chunk = s.stream_chunk;
        base.chunk_shift = 0;
        while ((1 << base.chunk_shift) < base.chunk) ++base.chunk_shift;
        base.group_windows = kProjTileM / s.stream_chunk;
        base.groups = p->stream_groups;
        // a forced timeout expects a count no pass reaches
        base.ready_target = ready_target(p->ready_passes[buffer], p->flag_skew);
        base.progress = p->progress;
        base.progress_pass = progress_pass_bits(p->layer_pass);
    }
    return base;
}

bilstm_status enqueue_recurrence(bilstm_plan *p, int layer, const float *gates, float *y,
                                 uint32_t flag_base, hipStream_t stream, bool layer_events,
                                 int tile_lo, int tile_hi, bool streamed = false, int buffer = 0) {
    const bilstm_plan_info &s = p->info;
    const RecurArgs base = recurrence_args(p, layer, gates, y, flag_base, streamed, buffer);
    const int per_launch = (s.recur_tiles + s.recur_launches - 1) / s.recur_launches;
    const size_t lds = p->reserve_lds;
    // With phase events on, the first launch on the caller's stream is bracketed by its own
    // event pair, so its duration can be read separately from the phase.
    const bool mark = p->phase_events && layer_events;
    auto launch_direction = [&](int direction, int directions, hipStream_t on) -> bilstm_status {
        for (int first = tile_lo; first < tile_hi; first += per_launch) {
            RecurArgs a = base;
            a.direction = direction;
            a.tile_first = first;
            a.tile_count = std::min(per_launch, tile_hi - first);
            const bool bracket = mark && on == stream && direction == 0 && first == tile_lo;
            if (bracket) BL_HIP(hipEventRecord(p->ev_launch0[layer], stream), "phase event");
            BL_HIP(launch_recurrence(s.recur_groups, s.recur_tile, a, directions, lds, on), "recurrence launch");
            if (bracket) BL_HIP(hipEventRecord(p->ev_launch1[layer], stream), "phase event");
        }
        return BILSTM_OK;
    };

    bilstm_status st;
    if (s.concurrent == 2) {
        return launch_direction(0, 2, stream);
    }
    if (s.concurrent == 1) {
        BL_HIP(hipEventRecord(p->fork[layer], stream), "fork");
        BL_HIP(hipStreamWaitEvent(p->side, p->fork[layer], 0), "fork wait");
        st = launch_direction(0, 1, stream);
        if (st == BILSTM_OK) st = launch_direction(1, 1, p->side);
        // join the side stream back, also when a launch failed
        hipError_t e = hipEventRecord(p->join[layer], p->side);
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, p->join[layer], 0);
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(p->side);
            if (st == BILSTM_OK) st = fail(BILSTM_HIP_ERROR, "recurrence join: %s", hipGetErrorString(e));
        }
        return st;
    }
    if ((st = launch_direction(0, 1, stream)) != BILSTM_OK) return st;
    return launch_direction(1, 1, stream);
}

// The stack with streamed gates. Every projection runs on the plan's projection stream and
// every recurrence on the caller's stream: the recurrence of layer l waits for the chunks its
// projection publishes. With layer overlap the projection of layer l + 1 starts as soon as
// layer l's projection is done and waits for the rows layer l's recurrence publishes; without,
// it waits on an event for layer l's recurrence to end. Gates alternate between two buffers and
// layer outputs between the plan's layer buffer (layers 0, 2) and y (1, 3), so a projection
// never overwrites gates a running recurrence reads, nor a recurrence rows a running
// projection reads.
bilstm_status forward_streamed(bilstm_plan *p, const float *x, float *y, hipStream_t stream, uint32_t base) {
    bilstm_status st;
    if (stream_counters_need_clear(p->layer_pass, p->ready_passes, p->ready_dirty)) {
        // counters out of step with the pass counts (a failed enqueue), or close to wrapping
        BL_HIP(launch_exchange_clear(p->ready, 2 * p->ready_words, stream), "counter clear");
        BL_HIP(launch_exchange_clear(p->progress, kProgressStride * 2 * static_cast<size_t>(p->batch), stream),
               "progress clear");
        p->ready_passes[0] = p->ready_passes[1] = 0;
        p->layer_pass = 0;
        p->ready_dirty = false;
        ++p->clears;
    }
    BL_HIP(hipEventRecord(p->proj_fork, stream), "projection fork");
    BL_HIP(hipStreamWaitEvent(p->proj_stream, p->proj_fork, 0), "projection fork wait");
    // From here on the projection stream is forked: whatever happens, join it back into the
    // caller's stream before returning, so the caller's stream order covers every projection
    // already enqueued (the next pass's counter clear must not overtake them).
    struct Join {
        bilstm_plan *p;
        hipStream_t stream;
        bool armed = true;
        ~Join() {
            if (!armed) return;
            if (hipEventRecord(p->proj_join, p->proj_stream) == hipSuccess) {
                (void)hipStreamWaitEvent(stream, p->proj_join, 0);
            } else {
                (void)hipStreamSynchronize(p->proj_stream);
            }
        }
    } join{p, stream};
    if (p->phase_events) BL_HIP(hipEventRecord(p->ev_start, stream), "phase event");
    // the four recurrences in one launch
    const bool one_launch = p->info.stream_fused != 0;
    RecurStack stack{};
    for (int l = 0; l < kLayers; ++l) {
        const int buffer = l % 2;
        const float *in = l == 0 ? x : (l % 2 == 1 ? p->ybuf : y);
        float *out = l % 2 == 0 ? p->ybuf : y;
        float *gates = buffer == 0 ? p->gates : p->gates_odd;
        ++p->layer_pass;
        ++p->ready_passes[buffer];
        if (!p->info.stream_overlap && l > 0) {
            BL_HIP(hipStreamWaitEvent(p->proj_stream, p->layer_done[l - 1], 0), "layer wait");
        }
        if ((st = enqueue_projection(p, l, in, gates, p->proj_stream, 0, p->rows, p->proj_workgroups_streamed, true,
                                     buffer)) != BILSTM_OK) {
            return st;
        }
        if (p->phase_events) BL_HIP(hipEventRecord(p->ev_proj[l], p->proj_stream), "phase event");
        if (p->info.stream_serial) {
            // kernels one at a time: this layer's recurrence after its whole projection
            BL_HIP(hipEventRecord(p->proj_done[l], p->proj_stream), "projection event");
            BL_HIP(hipStreamWaitEvent(stream, p->proj_done[l], 0), "projection wait");
        }
        if (one_launch) {
            RecurArgs &a = stack.layer[l];
            a = recurrence_args(p, l, gates, out, base + l * p->steps, true, buffer);
            a.direction = 0;
            a.tile_first = 0;
            a.tile_count = p->info.recur_tiles;
            continue;
        }
        if ((st = enqueue_recurrence(p, l, gates, out, base + l * p->steps, stream, true, 0, p->info.recur_tiles,
                                     true, buffer)) != BILSTM_OK) {
            return st;
        }
        if (!p->info.stream_overlap) BL_HIP(hipEventRecord(p->layer_done[l], stream), "layer event");
        if (p->phase_events) BL_HIP(hipEventRecord(p->ev_recur[l], stream), "phase event");
    }
    if (one_launch) {
        stack.layers = kLayers;
        if (p->phase_events) {
            // the launch between its own events; stamps split it into layers
            BL_HIP(launch_exchange_clear(p->stamps, kLayers + 1, stream), "stamp clear");
            stack.stamps = p->stamps;
            BL_HIP(hipEventRecord(p->ev_launch0[0], stream), "phase event");
        }
        BL_HIP(launch_recurrence_stack(p->info.recur_tile, stack, p->reserve_lds, stream), "recurrence launch");
        if (p->phase_events) {
            BL_HIP(hipEventRecord(p->ev_launch1[0], stream), "phase event");
            BL_HIP(hipEventRecord(p->ev_recur[kLayers - 1], stream), "phase event");
        }
    }
    join.armed = false;
    BL_HIP(hipEventRecord(p->proj_join, p->proj_stream), "projection join");
    BL_HIP(hipStreamWaitEvent(stream, p->proj_join, 0), "projection join wait");
    p->phases_recorded = p->phase_events;
    p->phases_streamed = true;
    p->phases_fused = one_launch;
    return BILSTM_OK;
}

// The stack without streamed gates: per layer the projection, then the recurrence, each
// batch slice as its own chain of layers on its own stream (slice 0 on the caller's stream).
bilstm_status forward_sliced(bilstm_plan *plan, const float *x, float *y, hipStream_t stream, uint32_t base) {
    const bilstm_plan_info &info = plan->info;
    const int slices = info.slices;
    bilstm_status st;
    if (slices > 1) {
        // fork: every slice stream starts after the caller's prior work
        BL_HIP(hipEventRecord(plan->slice_fork, stream), "slice fork");
        for (int i = 1; i < slices; ++i) {
            BL_HIP(hipStreamWaitEvent(plan->slice_stream[i], plan->slice_fork, 0), "slice fork wait");
        }
    }
    // From here on the slice streams are forked: join every one back into the caller's
    // stream before returning, also when an enqueue fails part way.
    struct Join {
        bilstm_plan *p;
        hipStream_t stream;
        int slices;
        bilstm_status join() {
            bilstm_status r = BILSTM_OK;
            for (int i = 1; i < slices; ++i) {
                hipError_t e = hipEventRecord(p->slice_join[i], p->slice_stream[i]);
                if (e == hipSuccess) e = hipStreamWaitEvent(stream, p->slice_join[i], 0);
                if (e != hipSuccess) {
                    (void)hipStreamSynchronize(p->slice_stream[i]);
                    if (r == BILSTM_OK) r = fail(BILSTM_HIP_ERROR, "slice join: %s", hipGetErrorString(e));
                }
            }
            slices = 0;
            return r;
        }
        ~Join() { (void)join(); }
    } joiner{plan, stream, slices};
    if (plan->phase_events) BL_HIP(hipEventRecord(plan->ev_start, stream), "phase event");
    for (int l = 0; l < kLayers; ++l) {
        for (int i = 0; i < slices; ++i) {
            // slice i holds windows [w0, w1); its chain runs on its own stream
            const uint32_t w0 = static_cast<uint32_t>(i) * info.slice_windows;
            const uint32_t w1 = std::min<uint32_t>(plan->batch, w0 + info.slice_windows);
            hipStream_t on = i > 0 ? plan->slice_stream[i] : stream;
            // The first projections run one slice after another, so the slices' recurrences
            // start staggered and each later projection meets recurrences, not projections.
            if (slices > 1 && l == 0 && i > 0) {
                BL_HIP(hipStreamWaitEvent(on, plan->slice_first[i - 1], 0), "slice stagger");
            }
            // every layer after the first reads the previous layer's complete output from y
            if ((st = enqueue_projection(plan, l, l == 0 ? x : y, plan->gates, on,
                                         static_cast<size_t>(w0) * plan->steps,
                                         static_cast<size_t>(w1 - w0) * plan->steps,
                                         slices > 1 ? plan->proj_workgroups_sliced : plan->proj_workgroups)) !=
                BILSTM_OK) {
                return st;
            }
            if (slices > 1 && l == 0) BL_HIP(hipEventRecord(plan->slice_first[i], on), "slice stagger");
            if (plan->phase_events && i == 0) BL_HIP(hipEventRecord(plan->ev_proj[l], on), "phase event");
            const int t0 = static_cast<int>(w0 / info.recur_tile);
            const int t1 = static_cast<int>((w1 + info.recur_tile - 1) / info.recur_tile);
            if ((st = enqueue_recurrence(plan, l, plan->gates, y, base + l * plan->steps, on, i == 0, t0, t1)) !=
                BILSTM_OK) {
                return st;
            }
            if (plan->phase_events && i == 0) BL_HIP(hipEventRecord(plan->ev_recur[l], on), "phase event");
        }
    }
    // join: the caller's stream waits for every other slice
    if ((st = joiner.join()) != BILSTM_OK) return st;
    plan->phases_recorded = plan->phase_events;
    plan->phases_streamed = false;
    plan->phases_fused = false;
    return BILSTM_OK;
}

// A watchdog report of an earlier call, read from the host-mapped words without a device
// synchronization: cleared and returned as BILSTM_TIMEOUT, so a caller that never calls
// bilstm_check still learns that an output it may have consumed is invalid.
bilstm_status take_timeout_report(bilstm_plan *p, const char *context) {
    volatile unsigned int *words = p->error_host;
    unsigned int seen = 0;
    for (int k = 0; k < kErrWords; ++k) seen |= words[k] != 0 ? 1u << k : 0u;
    if (seen == 0) return BILSTM_OK;
    for (int k = 0; k < kErrWords; ++k) words[k] = 0;
    // a pass that timed out may have left its counters or progress words out of step with the
    // pass counts: the next streamed pass clears them first
    if (seen & ((1u << kErrCounter) | (1u << kErrProgress))) p->ready_dirty = true;
    return fail(BILSTM_TIMEOUT,
                "%s: a wait of an earlier call on this plan hit its %.3f ms watchdog (%s%s%s); that call's "
                "outputs are invalid; nothing was enqueued",
                context, p->watchdog_ms, (seen & (1u << kErrExchange)) ? "exchange " : "",
                (seen & (1u << kErrCounter)) ? "chunk counter " : "", (seen & (1u << kErrProgress)) ? "progress" : "");
}

// Event flags. An event that only orders this plan's streams on its own device needs no
// system-scope fence (by default every record writes back and invalidates the L2, several
// microseconds on the stream each time, and the next kernel starts on a cold cache); nor does
// an event that only times. `done`, which the host waits on, keeps the default.
constexpr unsigned int kOrderEvent = hipEventDisableTiming | hipEventDisableSystemFence;
constexpr unsigned int kTimingEvent = hipEventDisableSystemFence;

// The end of a call that enqueued work: the plan's completion event goes on the caller's
// stream (after any join), whatever `st` is, so bilstm_check waits for all of it.
bilstm_status mark_done(bilstm_plan *p, hipStream_t stream, bilstm_status st, const char *context) {
    const hipError_t e = hipEventRecord(p->done, stream);
    if (st == BILSTM_OK && e != hipSuccess) {
        return fail(BILSTM_HIP_ERROR, "%s: completion event: %s", context, hipGetErrorString(e));
    }
    return st;
}

bilstm_status check_plan_buffers(const char *context, const bilstm_plan *p, const void *a,
                                 const void *b) {
    if (p == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "%s: plan is NULL", context);
    if (a == nullptr || b == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "%s: NULL buffer", context);
    if (!aligned16(a) || !aligned16(b)) {
        return fail(BILSTM_INVALID_ARGUMENT, "%s: buffers must be 16-byte aligned", context);
    }
    return BILSTM_OK;
}

}  // namespace

extern "C" {

const char *bilstm_last_error(void) { return g_last_error.c_str(); }

bilstm_status bilstm_plan_create_ex(int device, uint32_t batch, uint32_t steps,
                                    const bilstm_layer layers[BILSTM_LAYERS],
                                    const bilstm_options *options, bilstm_plan **out) {
    if (out == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "plan_create: out is NULL");
    *out = nullptr;
    if (layers == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "plan_create: layers is NULL");
    if (batch == 0 || steps == 0) {
        return fail(BILSTM_INVALID_ARGUMENT, "plan_create: batch (%u) and steps (%u) must be >= 1", batch, steps);
    }
    const uint64_t rows = static_cast<uint64_t>(batch) * steps;
    if (rows * kGateCols > 0xFFFFFFFFull) {
        return fail(BILSTM_DIMENSION_OVERFLOW, "plan_create: batch*steps*1024 = %llu exceeds 32 bits",
                    static_cast<unsigned long long>(rows * kGateCols));
    }
    if (4ull * steps + 2 > 0xFFFFFFFFull) {
        return fail(BILSTM_DIMENSION_OVERFLOW, "plan_create: steps %u too large for the step flags", steps);
    }
    for (int l = 0; l < kLayers; ++l) {
        const size_t in = l == 0 ? kFeatures : kWidth;
        const bilstm_layer &L = layers[l];
        if (L.w == nullptr || L.r == nullptr || L.b == nullptr) {
            return fail(BILSTM_INVALID_ARGUMENT, "plan_create: layer %d has a NULL weight pointer", l);
        }
        char ctx[64];
        bilstm_status s;
        std::snprintf(ctx, sizeof(ctx), "plan_create layer %d W", l);
        if ((s = check_len(ctx, 2 * kGates * in, L.w_len)) != BILSTM_OK) return s;
        std::snprintf(ctx, sizeof(ctx), "plan_create layer %d R", l);
        if ((s = check_len(ctx, 2ull * kGates * kHidden, L.r_len)) != BILSTM_OK) return s;
        std::snprintf(ctx, sizeof(ctx), "plan_create layer %d B", l);
        if ((s = check_len(ctx, 4ull * kGates, L.b_len)) != BILSTM_OK) return s;
    }

    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count == 0) {
        return fail(BILSTM_UNSUPPORTED, "plan_create: no HIP device (%s)", hipGetErrorString(e));
    }
    if (device < 0 || device >= count) {
        return fail(BILSTM_INVALID_ARGUMENT, "plan_create: device %d out of range (%d devices)", device, count);
    }
    if (!is_gfx950(device)) {
        return fail(BILSTM_UNSUPPORTED, "plan_create: device %d is not a gfx950 (MI355X) GPU", device);
    }
    DeviceScope scope(device);
    BL_HIP(scope.error(), "plan_create: hipSetDevice");

    auto *p = new bilstm_plan();
    p->device = device;
    p->batch = batch;
    p->steps = steps;
    p->rows = rows;
    auto fail_release = [&](bilstm_status s) {
        release(p);
        return s;
    };

    int cu_count = 0;
    int wall_khz = 0;
    e = hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, device);
    if (e != hipSuccess || cu_count <= 0 || wall_khz <= 0) {
        return fail_release(fail(BILSTM_HIP_ERROR, "plan_create: device attributes: %s", hipGetErrorString(e)));
    }
    const int32_t wd_us = options != nullptr ? options->watchdog_us : 0;
    const double watchdog_ms = wd_us > 0 ? wd_us / 1000.0 : (wd_us < 0 ? 0.0 : kWatchdogMs);
    p->timeout_ticks = static_cast<unsigned long long>(watchdog_ms * wall_khz);
    p->wall_khz = wall_khz;
    p->watchdog_ms = watchdog_ms;
    // watchdog_us = -1: every wait expects a flag that no producer ever writes, so its first
    // poll misses and it gives up at once: a forced, deterministic timeout
    p->flag_skew = wd_us < 0 ? 0x80000000u : 0u;

    // choose the split, then size the launches from the chosen kernel's occupancy
    bilstm_plan_info info{};
    bilstm_options choose{};
    if (options != nullptr) choose = *options;
    choose.concurrent = -1;  // the concurrency request is checked once the occupancy is known
    bilstm_status st = schedule(batch, steps, cu_count, 1, &choose, &info);
    if (st != BILSTM_OK) return fail_release(st);
    int per_cu = 0;
    e = recurrence_occupancy(info.recur_groups, info.recur_tile, &per_cu);
    if (e != hipSuccess || per_cu <= 0) {
        return fail_release(fail(BILSTM_HIP_ERROR, "plan_create: recurrence occupancy: %s (%d per CU)",
                                 hipGetErrorString(e), per_cu));
    }
    bilstm_options fixed{};
    if (options != nullptr) fixed = *options;
    fixed.recur_groups = info.recur_groups;
    fixed.recur_tile = info.recur_tile;
    st = schedule(batch, steps, cu_count, per_cu, &fixed, &info);
    if (st != BILSTM_OK) return fail_release(st);
    info.proj_tile_m = kProjTileM;
    info.proj_tile_n = kProjTileN;
    p->info = info;
    // The projection's persistent grid counts CUs (its launch puts one or two workgroups on
    // each): every CU, or beside the recurrences of the other slices (each of their workgroups
    // keeps a CU to itself) the CUs they leave free.
    p->proj_workgroups = cu_count;
    {
        const int slice_tiles = (info.slice_windows + info.recur_tile - 1) / info.recur_tile;
        const int busy = 2 * slice_tiles * info.recur_groups * (info.slices - 1);
        p->proj_workgroups_sliced = std::max(8, cu_count - busy);
    }

    // pack and upload the weights
    for (int l = 0; l < kLayers; ++l) {
        p->kpad[l] = padded_input(p->in[l]);
        std::vector<float> w(static_cast<size_t>(kGateCols) * p->kpad[l]);
        std::vector<float> r(2ull * kGates * kHidden);
        std::vector<float> b(kGateCols);
        pack_layer(layers[l], p->in[l], w.data(), r.data(), b.data());
        // recurrent rows scaled into the exponent of their gate's activation (row 4j + g)
        for (size_t row = 0; row < 2ull * kGates; ++row) {
            const float scale = gate_exp_scale(static_cast<int>(row % 4));
            for (int k = 0; k < kHidden; ++k) r[row * kHidden + k] *= scale;
        }
        if ((st = device_alloc(p, &p->w[l], w.size(), "W")) != BILSTM_OK) return fail_release(st);
        if ((st = device_alloc(p, &p->r[l], r.size(), "R")) != BILSTM_OK) return fail_release(st);
        if ((st = device_alloc(p, &p->bias[l], b.size(), "bias")) != BILSTM_OK) return fail_release(st);
        e = hipMemcpy(p->w[l], w.data(), w.size() * sizeof(float), hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(p->r[l], r.data(), r.size() * sizeof(float), hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(p->bias[l], b.data(), b.size() * sizeof(float), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            return fail_release(fail(BILSTM_HIP_ERROR, "plan_create: weight upload: %s", hipGetErrorString(e)));
        }
        if (info.projection == kProjectionSplit2 || info.projection == kProjectionSplit3) {
            // split precision: w = part 0 + part 1 (+ part 2) + a residual below 2^-8P·|w|, each
            // part the bf16 of what the earlier ones leave (every difference exact in fp32)
            const int parts = info.projection == kProjectionSplit3 ? 3 : 2;
            std::vector<uint16_t> plane[3];
            for (int pl = 0; pl < parts; ++pl) plane[pl].resize(w.size());
            for (size_t i = 0; i < w.size(); ++i) {
                float rest = w[i];
                for (int pl = 0; pl < parts; ++pl) {
                    plane[pl][i] = bf16_rne(rest);
                    rest -= bf16_value(plane[pl][i]);
                }
            }
            uint16_t **dst[3] = {&p->w_hi[l], &p->w_lo[l], &p->w_lo2[l]};
            for (int pl = 0; pl < parts; ++pl) {
                if ((st = device_alloc(p, dst[pl], plane[pl].size(), "W part")) != BILSTM_OK) return fail_release(st);
                e = hipMemcpy(*dst[pl], plane[pl].data(), plane[pl].size() * sizeof(uint16_t), hipMemcpyHostToDevice);
                if (e != hipSuccess) {
                    return fail_release(fail(BILSTM_HIP_ERROR, "plan_create: weight upload: %s", hipGetErrorString(e)));
                }
            }
        }
    }

    if ((st = device_alloc(p, &p->gates, rows * kGateCols, "gates")) != BILSTM_OK) return fail_release(st);
    if (info.projection == kProjectionVendor) {
        if ((st = library_projection_create(static_cast<long>(rows), p->in, p->kpad, p->bias, &p->library)) !=
            BILSTM_OK) {
            return fail_release(st);
        }
    }
    // watchdog reports: host-mapped, coherent words the kernels store into and the host reads
    // without synchronizing
    e = hipHostMalloc(reinterpret_cast<void **>(&p->error_host), kErrWords * sizeof(unsigned int),
                      hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) {
        p->error_host = nullptr;
        return fail_release(fail(BILSTM_HIP_ERROR, "plan_create: hipHostMalloc of the watchdog words: %s",
                                 hipGetErrorString(e)));
    }
    std::memset(p->error_host, 0, kErrWords * sizeof(unsigned int));
    e = hipHostGetDevicePointer(reinterpret_cast<void **>(&p->error), p->error_host, 0);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->done, hipEventDisableTiming);
    if (info.recur_groups > 1) {
        p->exchange_words = 2 * exchange_words_per_direction(info.recur_tiles, info.recur_tile);
        if ((st = device_alloc(p, &p->exchange, p->exchange_words, "exchange")) != BILSTM_OK) {
            return fail_release(st);
        }
        if (e == hipSuccess) e = hipMemset(p->exchange, 0, p->exchange_words * sizeof(unsigned long long));
    }
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking);
    for (int l = 0; l < kLayers && e == hipSuccess; ++l) {
        e = hipEventCreateWithFlags(&p->fork[l], kOrderEvent);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->join[l], kOrderEvent);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_proj[l], kTimingEvent);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_recur[l], kTimingEvent);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_launch0[l], kTimingEvent);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_launch1[l], kTimingEvent);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_start, kTimingEvent);
    if (info.slices > 1) {
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->slice_fork, kOrderEvent);
        for (int i = 0; i < info.slices && e == hipSuccess; ++i) {
            // slice 0 runs on the caller's stream; each other slice gets a stream of its own
            if (i > 0) e = hipStreamCreateWithFlags(&p->slice_stream[i], hipStreamNonBlocking);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&p->slice_first[i], kOrderEvent);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&p->slice_join[i], kOrderEvent);
        }
        // A recurrence workgroup claims enough LDS that no projection workgroup fits beside it
        // on its CU (every projection kernel of the library takes at least kProjLdsBytes): the
        // projections of other slices then run only on CUs no recurrence uses, and the
        // latency-bound recurrence keeps its CU's issue slots and LDS to itself.
        if (e == hipSuccess) {
            p->reserve_lds = kCuLdsBytes - kProjLdsBytes + 4096;
            e = recurrence_allow_lds(info.recur_groups, info.recur_tile, p->reserve_lds);
        }
    }
    if (e == hipSuccess && info.pipeline) {
        // streamed gates: the second layer buffer, the chunk counters (zeroed), the projection's
        // stream and the events that order it against the recurrence
        const int group_windows = kProjTileM / info.stream_chunk;
        p->stream_groups = static_cast<int>((batch + group_windows - 1) / group_windows);
        p->stream_chunks = stream_chunks(static_cast<int>(steps), info.stream_chunk);
        const size_t counters = static_cast<size_t>(p->stream_chunks) * 2 * p->stream_groups;
        p->ready_words = (counters + 1) / 2;
        if ((st = device_alloc(p, &p->ybuf, rows * kWidth, "layer buffer")) != BILSTM_OK) return fail_release(st);
        if ((st = device_alloc(p, &p->gates_odd, rows * kGateCols, "second gate buffer")) != BILSTM_OK) {
            return fail_release(st);
        }
        if ((st = device_alloc(p, &p->ready, 2 * p->ready_words, "chunk counters")) != BILSTM_OK) return fail_release(st);
        // the progress words, then one line of phase stamps
        if ((st = device_alloc(p, &p->progress, kProgressStride * (2 * static_cast<size_t>(batch) + 1),
                               "progress words")) != BILSTM_OK) {
            return fail_release(st);
        }
        p->stamps = p->progress + kProgressStride * 2 * static_cast<size_t>(batch);
        e = hipMemset(p->ready, 0, 2 * p->ready_words * sizeof(unsigned long long));
        if (e == hipSuccess) {
            e = hipMemset(p->progress, 0, kProgressStride * 2 * static_cast<size_t>(batch) * sizeof(unsigned long long));
        }
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->proj_stream, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->proj_fork, kOrderEvent);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&p->proj_join, kOrderEvent);
        for (int l = 0; l < kLayers && e == hipSuccess; ++l) {
            e = hipEventCreateWithFlags(&p->layer_done[l], kOrderEvent);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&p->proj_done[l], kOrderEvent);
        }
        // Each recurrence workgroup claims enough LDS that no projection workgroup fits beside
        // it, and each streamed projection workgroup enough that no second one shares its CU:
        // the projection's persistent grid then takes exactly the CUs the recurrence leaves.
        if (e == hipSuccess) {
            p->reserve_lds = kCuLdsBytes - kProjLdsBytes + 4096;
            e = recurrence_allow_lds(info.recur_groups, info.recur_tile, p->reserve_lds);
        }
        p->proj_workgroups_streamed = stream_projection_workgroups(cu_count, info.recur_tiles, info.recur_groups);
    }
    if (e == hipSuccess && options != nullptr && options->near_wrap != 0) {
        // Test hook: flags and pass numbers start just below their clear thresholds (those of
        // reserve_flags and forward_streamed), so the first forward runs near the top of their
        // range and the second one clears. The counters hold kReadyPerPass per pass so far.
        const uint32_t count = kLayers * steps;
        p->epoch = 0xFFFFFFFFu - 1u - count - count / 2;
        p->ready_passes[0] = p->ready_passes[1] = kReadyPassLimit - 1;
        p->layer_pass = kLayerPassLimit - (kLayers - 1);
        if (p->ready != nullptr) {
            e = hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(p->ready),
                             static_cast<int>(ready_target(kReadyPassLimit - 1, 0)),
                             4 * p->ready_words);
        }
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        return fail_release(fail(BILSTM_HIP_ERROR, "plan_create: scratch setup: %s", hipGetErrorString(e)));
    }
    p->info.device_bytes = p->device_bytes;
    *out = p;
    return BILSTM_OK;
}

bilstm_status bilstm_plan_create(int device, uint32_t batch, uint32_t steps,
                                 const bilstm_layer layers[BILSTM_LAYERS], bilstm_plan **out) {
    return bilstm_plan_create_ex(device, batch, steps, layers, nullptr, out);
}

bilstm_status bilstm_forward(bilstm_plan *plan, const float *x, size_t x_len, float *y,
                             size_t y_len, void *stream_ptr) {
    bilstm_status st = check_plan_buffers("forward", plan, x, y);
    if (st != BILSTM_OK) return st;
    if ((st = check_len("forward input", plan->rows * kFeatures, x_len)) != BILSTM_OK) return st;
    if ((st = check_len("forward output", plan->rows * kWidth, y_len)) != BILSTM_OK) return st;
    if (overlap(x, x_len * sizeof(float), y, y_len * sizeof(float))) {
        return fail(BILSTM_INVALID_ARGUMENT, "forward: input and output overlap");
    }
    auto stream = static_cast<hipStream_t>(stream_ptr);
    DeviceScope scope(plan->device);
    BL_HIP(scope.error(), "forward: hipSetDevice");
    if ((st = take_timeout_report(plan, "forward")) != BILSTM_OK) return st;

    uint32_t base = 0;
    if ((st = reserve_flags(plan, kLayers * plan->steps, stream, &base)) != BILSTM_OK) return st;
    if (plan->info.pipeline) {
        st = forward_streamed(plan, x, y, stream, base);
        if (st != BILSTM_OK) plan->ready_dirty = true;
    } else {
        st = forward_sliced(plan, x, y, stream, base);
    }
    return mark_done(plan, stream, st, "forward");
}

bilstm_status bilstm_project(bilstm_plan *plan, int layer, const float *x, size_t x_len,
                             float *gates, size_t gates_len, void *stream_ptr) {
    bilstm_status st = check_plan_buffers("project", plan, x, gates);
    if (st != BILSTM_OK) return st;
    if (layer < 0 || layer >= kLayers) return fail(BILSTM_INVALID_ARGUMENT, "project: layer %d out of range", layer);
    if ((st = check_len("project input", plan->rows * plan->in[layer], x_len)) != BILSTM_OK) return st;
    if ((st = check_len("project gates", plan->rows * kGateCols, gates_len)) != BILSTM_OK) return st;
    DeviceScope scope(plan->device);
    BL_HIP(scope.error(), "project: hipSetDevice");
    if ((st = take_timeout_report(plan, "project")) != BILSTM_OK) return st;
    auto stream = static_cast<hipStream_t>(stream_ptr);
    st = enqueue_projection(plan, layer, x, gates, stream, 0, plan->rows, plan->proj_workgroups);
    return mark_done(plan, stream, st, "project");
}

bilstm_status bilstm_recur(bilstm_plan *plan, int layer, const float *gates, size_t gates_len,
                           float *y, size_t y_len, void *stream_ptr) {
    bilstm_status st = check_plan_buffers("recur", plan, gates, y);
    if (st != BILSTM_OK) return st;
    if (layer < 0 || layer >= kLayers) return fail(BILSTM_INVALID_ARGUMENT, "recur: layer %d out of range", layer);
    if ((st = check_len("recur gates", plan->rows * kGateCols, gates_len)) != BILSTM_OK) return st;
    if ((st = check_len("recur output", plan->rows * kWidth, y_len)) != BILSTM_OK) return st;
    auto stream = static_cast<hipStream_t>(stream_ptr);
    DeviceScope scope(plan->device);
    BL_HIP(scope.error(), "recur: hipSetDevice");
    if ((st = take_timeout_report(plan, "recur")) != BILSTM_OK) return st;
    uint32_t base = 0;
    if ((st = reserve_flags(plan, plan->steps, stream, &base)) != BILSTM_OK) return st;
    st = enqueue_recurrence(plan, layer, gates, y, base, stream, false, 0, plan->info.recur_tiles);
    return mark_done(plan, stream, st, "recur");
}

bilstm_status bilstm_plan_get_info(const bilstm_plan *plan, bilstm_plan_info *info) {
    if (plan == nullptr || info == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "get_info: NULL argument");
    *info = plan->info;
    info->clears = plan->clears;
    return BILSTM_OK;
}

bilstm_status bilstm_check(bilstm_plan *plan) {
    if (plan == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "check: plan is NULL");
    DeviceScope scope(plan->device);
    BL_HIP(scope.error(), "check: hipSetDevice");
    // the plan's last call only: its completion event, after every join into the caller's
    // stream (a never-recorded event is complete)
    BL_HIP(hipEventSynchronize(plan->done), "check");
    return take_timeout_report(plan, "check");
}

bilstm_status bilstm_set_phase_events(bilstm_plan *plan, int enable) {
    if (plan == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "set_phase_events: plan is NULL");
    plan->phase_events = enable != 0;
    return BILSTM_OK;
}

bilstm_status bilstm_phase_times(bilstm_plan *plan, float *ms, size_t n) {
    if (plan == nullptr || ms == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "phase_times: NULL argument");
    if (n < 3 * kLayers) return fail(BILSTM_BUFFER_LENGTH, "phase_times: need %d values, got %zu", 3 * kLayers, n);
    if (!plan->phases_recorded) {
        return fail(BILSTM_INVALID_ARGUMENT, "phase_times: no forward ran with phase events enabled");
    }
    DeviceScope scope(plan->device);
    BL_HIP(scope.error(), "phase_times: hipSetDevice");
    BL_HIP(hipEventSynchronize(plan->ev_recur[kLayers - 1]), "phase_times");
    if (plan->phases_fused) {
        // One recurrence launch for the four layers, between its own events (duration L, end
        // E from the forward's start). The stamps place each layer's end inside it: layer l
        // ends at E - L·(1 - f_l), f_l = (its end - the launch's start) / (the last layer's end
        // - the launch's start) on the GPU's wall clock; its share of the launch is L·(f_l -
        // f_{l-1}).
        unsigned long long st[kLayers + 1];
        BL_HIP(hipMemcpy(st, plan->stamps, sizeof(st), hipMemcpyDeviceToHost), "phase_times");
        const unsigned long long t0 = ~st[kLayers];
        if (st[kLayers] == 0 || st[kLayers - 1] <= t0) {
            return fail(BILSTM_HIP_ERROR, "phase_times: the recurrence launch left no stamps");
        }
        float e_end = 0.0f, l_dur = 0.0f;
        BL_HIP(hipEventElapsedTime(&e_end, plan->ev_start, plan->ev_launch1[0]), "phase_times");
        BL_HIP(hipEventElapsedTime(&l_dur, plan->ev_launch0[0], plan->ev_launch1[0]), "phase_times");
        const double span = static_cast<double>(st[kLayers - 1] - t0);
        double before = 0.0;
        for (int l = 0; l < kLayers; ++l) {
            BL_HIP(hipEventElapsedTime(&ms[l], plan->ev_start, plan->ev_proj[l]), "phase_times");
            const double f = st[l] > t0 ? std::min(1.0, static_cast<double>(st[l] - t0) / span) : 0.0;
            ms[kLayers + l] = static_cast<float>(e_end - l_dur * (1.0 - f));
            ms[2 * kLayers + l] = static_cast<float>(l_dur * (f - before));
            before = f;
        }
        return BILSTM_OK;
    }
    for (int l = 0; l < kLayers; ++l) {
        // streamed: the end of every phase from the forward's start (the phases of a layer and
        // of its neighbours overlap); else each phase's own duration
        hipEvent_t before = plan->phases_streamed || l == 0 ? plan->ev_start : plan->ev_recur[l - 1];
        BL_HIP(hipEventElapsedTime(&ms[l], before, plan->ev_proj[l]), "phase_times");
        BL_HIP(hipEventElapsedTime(&ms[kLayers + l], plan->phases_streamed ? plan->ev_start : plan->ev_proj[l],
                                   plan->ev_recur[l]),
               "phase_times");
        BL_HIP(hipEventElapsedTime(&ms[2 * kLayers + l], plan->ev_launch0[l], plan->ev_launch1[l]), "phase_times");
    }
    return BILSTM_OK;
}

void bilstm_destroy(bilstm_plan *plan) { release(plan); }

bilstm_status bilstm_probe_exchange(int device, int same_xcd, int32_t round_trips, double *one_way_ns,
                                    int32_t *xcd_a, int32_t *xcd_b) {
    if (one_way_ns == nullptr || xcd_a == nullptr || xcd_b == nullptr) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_exchange: NULL output");
    }
    if (round_trips <= 0 || round_trips > 1000000) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_exchange: round_trips %d out of range", round_trips);
    }
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_exchange: no device %d", device);
    }
    if (!is_gfx950(device)) return fail(BILSTM_UNSUPPORTED, "probe_exchange: device %d is not gfx950", device);
    DeviceScope scope(device);
    BL_HIP(scope.error(), "probe_exchange: hipSetDevice");
    int wall_khz = 0;
    BL_HIP(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, device), "probe_exchange");
    const double ticks_per_ns = wall_khz / 1.0e6;
    const auto timeout = static_cast<unsigned long long>(kWatchdogMs * wall_khz);
    int a = -1, b = -1;
    hipError_t e = run_exchange_probe(same_xcd, round_trips, timeout, ticks_per_ns, one_way_ns, &a, &b);
    if (e == hipErrorLaunchTimeOut) return fail(BILSTM_TIMEOUT, "probe_exchange: watchdog fired");
    BL_HIP(e, "probe_exchange");
    *xcd_a = a;
    *xcd_b = b;
    return BILSTM_OK;
}

bilstm_status bilstm_probe_fma_rate(int device, int waves_per_simd, int32_t workgroups, int32_t iterations,
                                    double *clocks_per_fma, double *ghz) {
    if (clocks_per_fma == nullptr || ghz == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "probe_fma_rate: NULL output");
    if (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_fma_rate: waves_per_simd %d is not 1, 2 or 4", waves_per_simd);
    }
    if (workgroups < 1 || workgroups > 4096 || iterations < 1 || iterations > 1000000) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_fma_rate: workgroups %d or iterations %d out of range", workgroups,
                    iterations);
    }
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_fma_rate: no device %d", device);
    }
    if (!is_gfx950(device)) return fail(BILSTM_UNSUPPORTED, "probe_fma_rate: device %d is not gfx950", device);
    DeviceScope scope(device);
    BL_HIP(scope.error(), "probe_fma_rate: hipSetDevice");
    int wall_khz = 0;
    BL_HIP(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, device), "probe_fma_rate");
    BL_HIP(run_fma_probe(waves_per_simd, workgroups, iterations, wall_khz, clocks_per_fma, ghz), "probe_fma_rate");
    return BILSTM_OK;
}

bilstm_status bilstm_probe_mfma_rate(int device, int kind, int data, int32_t iterations, double *tflops, double *ms) {
    if (tflops == nullptr || ms == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "probe_mfma_rate: NULL output");
    if (kind != 0 && kind != 1) return fail(BILSTM_INVALID_ARGUMENT, "probe_mfma_rate: kind %d is not 0 or 1", kind);
    if (data < 0 || data > 2) return fail(BILSTM_INVALID_ARGUMENT, "probe_mfma_rate: data %d is not 0, 1 or 2", data);
    if (iterations < 1 || iterations > 1000000) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_mfma_rate: iterations %d out of range", iterations);
    }
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) {
        return fail(BILSTM_INVALID_ARGUMENT, "probe_mfma_rate: no device %d", device);
    }
    if (!is_gfx950(device)) return fail(BILSTM_UNSUPPORTED, "probe_mfma_rate: device %d is not gfx950", device);
    DeviceScope scope(device);
    BL_HIP(scope.error(), "probe_mfma_rate: hipSetDevice");
    int cu_count = 0;
    BL_HIP(hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, device), "probe_mfma_rate");
    BL_HIP(run_mfma_probe(kind, data, iterations, cu_count, tflops, ms), "probe_mfma_rate");
    return BILSTM_OK;
}

}  // extern "C"
