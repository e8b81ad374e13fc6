// Host-only parts of the library: the weight packer and the recurrence schedule. Neither
// touches the GPU, so both are exported for tests that run without a device.
#include <algorithm>
#include <cstring>

#include "../../include/bilstm.h"
#include "bilstm_host.h"

namespace bl {

// Packed gate row of source row `src` (gate g = src / 128, unit j = src % 128): 4j + g, i.e.
// unit j's i, f, g and o rows sit next to each other (speakrs 0.6.0, page `lstmproj.rs`,
// module doc: the projection's gate columns are reordered per hidden unit).
static inline int packed_row(int src) { return 4 * (src % kHidden) + src / kHidden; }

bilstm_status pack_layer(const bilstm_layer &layer, int in, float *w_out, float *r_out,
                         float *bias_out) {
    const int kpad = padded_input(in);
    std::memset(w_out, 0, sizeof(float) * static_cast<size_t>(kGateCols) * kpad);
    for (int d = 0; d < 2; ++d) {
        for (int src = 0; src < kGates; ++src) {
            const int row = d * kGates + packed_row(src);
            const float *w = layer.w + (static_cast<size_t>(d) * kGates + src) * in;
            std::memcpy(w_out + static_cast<size_t>(row) * kpad, w, sizeof(float) * in);
            const float *r = layer.r + (static_cast<size_t>(d) * kGates + src) * kHidden;
            std::memcpy(r_out + (static_cast<size_t>(d) * kGates + packed_row(src)) * kHidden, r,
                        sizeof(float) * kHidden);
            const float wb = layer.b[(static_cast<size_t>(d) * 2 + 0) * kGates + src];
            const float rb = layer.b[(static_cast<size_t>(d) * 2 + 1) * kGates + src];
            bias_out[row] = wb + rb;  // one fp32 round-to-nearest addition
        }
    }
    return BILSTM_OK;
}

// ---- the projection rule ------------------------------------------------------------------
//
// The input projection runs either as FP32 MFMA products or split into three bf16 parts per
// operand with six bf16 MFMA products (speakrs 0.6.0, page `lstmproj.rs`, `projection_rule`:
// reduced-precision tensor projections only where enough rows amortize them and where they
// were accurate enough on the device; `tf32_projection_accurate`: accurate means within 1.1x
// the reference library's error against an f64 reference). Here the split is used only where
// it is both accurate and faster for the forward:
//  * accuracy: development checks on MI355X (the five synthetic workloads, whole outputs
//    against the fp64 oracle) put the stack's largest error with the three-part split at 0.94
//    to 0.98 times the FP32 kernel's (b8 0.98, b32 0.94, b256 0.95, b64_t4096 0.98), within
//    the 1.1 factor; the two-part split measured 2.5 to 4.3 times and is never chosen;
//  * amortization: at least kSplitMinRows projection rows, the pages' small-projection
//    threshold (below it the FP32 kernel is kept);
//  * speed: the projection must be on the forward's critical path. Unstreamed, it runs between
//    the recurrences, so it always is. Streamed beside the recurrence, the FP32 kernel keeps up
//    while each recurrence step asks at most kStreamFp32FlopPerCu flops of each CU the
//    recurrence leaves (measured: about 0.40 TFLOP/s per CU beside a one-window step of about
//    0.46 us); beyond that the layer runs at the projection's pace.
// The rule is a function of the workload and the device only (the plan's schedule with every
// option left to the plan), so every plan for one workload computes the same gates, whatever
// its streaming, slices or recurrence split.
constexpr unsigned long long kSplitMinRows = 2048;
constexpr double kStreamFp32FlopPerCu = 184.0e3;

// Whether the three-part split stayed within 1.1x the FP32 kernel's error on this device: every
// workload the development checks ran on gfx950 did.
static bool split_projection_accurate(uint32_t batch, uint32_t steps) {
    (void)batch;
    (void)steps;
    return true;
}

static int auto_projection(uint32_t batch, uint32_t steps, int cu_count) {
    const unsigned long long rows = static_cast<unsigned long long>(batch) * steps;
    if (rows < kSplitMinRows || !split_projection_accurate(batch, steps)) return kProjectionFp32;
    // the default recurrence schedule: one workgroup per tile and direction, each alone on a CU,
    // the fewest windows per tile that let both directions fit the GPU at once
    long long tiles = (static_cast<long long>(batch) + 3) / 4;
    for (int t : {1, 2, 4}) {
        const long long n = (static_cast<long long>(batch) + t - 1) / t;
        if (2 * n <= cu_count) {
            tiles = n;
            break;
        }
    }
    const long long rec_wgs = 2 * tiles;
    const bool streamed = rec_wgs + 8 <= cu_count && 4 * rec_wgs <= 3LL * cu_count;
    if (!streamed) return kProjectionSplit3;
    const int free_cus = stream_projection_workgroups(cu_count, static_cast<int>(tiles), 1);
    const double flop_per_step = 2.0 * kGateCols * kWidth * static_cast<double>(batch);
    return flop_per_step / free_cus > kStreamFp32FlopPerCu ? kProjectionSplit3 : kProjectionFp32;
}

static bool valid_groups(int g) { return g == 1 || g == 2 || g == 4; }
static bool valid_tile(int t) { return t == 1 || t == 2 || t == 4; }

bilstm_status schedule(uint32_t batch, uint32_t steps, int cu_count, int per_cu,
                       const bilstm_options *opt, bilstm_plan_info *info) {
    if (batch == 0 || steps == 0) {
        return fail(BILSTM_INVALID_ARGUMENT, "schedule: batch (%u) and steps (%u) must be >= 1", batch, steps);
    }
    if (cu_count <= 0 || per_cu <= 0) {
        return fail(BILSTM_INVALID_ARGUMENT, "schedule: cu_count (%d) and per_cu (%d) must be >= 1",
                    cu_count, per_cu);
    }
    if (opt != nullptr) {
        if (opt->near_wrap != 0 && opt->near_wrap != 1) {
            return fail(BILSTM_INVALID_ARGUMENT, "options: near_wrap %d is not 0 or 1", opt->near_wrap);
        }
        if (opt->pipeline < 0 || opt->pipeline > 5) {
            return fail(BILSTM_INVALID_ARGUMENT, "options: pipeline %d is not one of 0..5", opt->pipeline);
        }
        if (opt->projection < 0 || opt->projection > kProjectionFp32) {
            return fail(BILSTM_INVALID_ARGUMENT, "options: projection %d is not one of 0..%d", opt->projection,
                        kProjectionFp32);
        }
        if (opt->slices < 0 || opt->slices > kMaxSlices) {
            return fail(BILSTM_INVALID_ARGUMENT, "options: slices %d is not in 0..%d", opt->slices, kMaxSlices);
        }
        if (opt->recur_groups != 0 && !valid_groups(opt->recur_groups)) {
            return fail(BILSTM_UNSUPPORTED, "options: recur_groups %d is not one of 1, 2, 4",
                        opt->recur_groups);
        }
        if (opt->recur_tile != 0 && !valid_tile(opt->recur_tile)) {
            return fail(BILSTM_UNSUPPORTED, "options: recur_tile %d is not one of 1, 2, 4", opt->recur_tile);
        }
        if (opt->watchdog_us < -1) {
            return fail(BILSTM_INVALID_ARGUMENT, "options: watchdog_us %d is below -1", opt->watchdog_us);
        }
        if (opt->concurrent < -1 || opt->concurrent > 2) {
            return fail(BILSTM_INVALID_ARGUMENT, "options: concurrent %d is not -1, 0, 1 or 2", opt->concurrent);
        }
    }
    const int capacity = cu_count * per_cu;
    const int want_groups = (opt != nullptr) ? opt->recur_groups : 0;
    const int want_tile = (opt != nullptr) ? opt->recur_tile : 0;
    const int want_conc = (opt != nullptr) ? opt->concurrent : -1;

    // Workgroups per tile: by default a single workgroup keeps all of R for its direction, so
    // no h has to cross workgroups; the split variants pay a measured ~0.45 us per step for
    // the cross-CU hand-off and are slower at every batch size.
    const int groups = want_groups != 0 ? want_groups : 1;
    // Windows per tile: the fewest that let both directions' grids fit the GPU at once.
    int tile = want_tile;
    if (tile == 0) {
        tile = 4;
        for (int t : {1, 2, 4}) {
            const long long tiles = (static_cast<long long>(batch) + t - 1) / t;
            if (2 * tiles * groups <= capacity) {
                tile = t;
                break;
            }
        }
    }
    const int tiles = static_cast<int>((static_cast<long long>(batch) + tile - 1) / tile);
    const long long grid = static_cast<long long>(tiles) * groups;

    // Workgroups of a tile wait for each other when groups > 1, so each launch's grid must
    // fit the resident capacity; both directions run at once only if both grids fit together.
    int launches = 1;
    if (groups > 1) {
        const int per_launch = std::max(1, capacity / groups);
        if (groups > capacity) {
            return fail(BILSTM_UNSUPPORTED, "schedule: %d workgroups per tile exceed the resident capacity %d",
                        groups, capacity);
        }
        launches = (tiles + per_launch - 1) / per_launch;
    }
    const bool joint_fits = groups == 1 || 2 * grid <= capacity;
    int concurrent;
    if (want_conc == -1) {
        // Both directions in one launch when they fit together: on MI355X this measured ~23 us
        // per layer faster than the side stream's event fork and join.
        concurrent = joint_fits ? 2 : 0;
    } else {
        concurrent = want_conc;
        if (concurrent != 0 && !joint_fits) {
            return fail(BILSTM_UNSUPPORTED,
                        "schedule: concurrent directions need both grids (2 x %lld workgroups) resident "
                        "together, capacity is %d", grid, capacity);
        }
    }

    const int want_slices = (opt != nullptr) ? opt->slices : 0;
    const int want_projection = (opt != nullptr) ? opt->projection : kProjectionAuto;
    const int projection = want_projection != kProjectionAuto ? want_projection : auto_projection(batch, steps, cu_count);

    // Streamed gates: each layer's projection runs beside its own recurrence, on the CUs the
    // recurrence leaves free (every recurrence workgroup keeps a CU to itself), and never waits
    // for it; only the recurrence waits, for chunks the projection publishes. The projection
    // needs CUs of its own (8 at least), single-workgroup tiles (no cross-workgroup waits in
    // the recurrence besides the counters) and one of the library's own kernels (FP32 or split).
    const int want_pipe = (opt != nullptr) ? opt->pipeline : 0;
    const long long rec_wgs = 2 * grid;
    const bool pipe_possible = groups == 1 && projection != kProjectionVendor && want_slices <= 1 && rec_wgs + 8 <= cu_count;
    bool pipeline = false;
    if (want_pipe >= 2) {
        if (!pipe_possible) {
            return fail(BILSTM_UNSUPPORTED,
                        "schedule: streamed gates need recur_groups = 1, the library's own projection, slices <= 1 and at "
                        "least 8 CUs beside the recurrence's %lld workgroups (%d CUs)", rec_wgs, cu_count);
        }
        pipeline = true;
    } else if (want_pipe == 0) {
        // auto: when the recurrence leaves at least half of the CUs to the projection. Measured
        // on MI355X at 589 steps, unstreamed against streamed: 1 window 1.187 -> 1.168 ms,
        // 2 windows 1.228 -> 1.174, 4 windows 1.240 -> 1.179, 32 windows 1.405 -> 1.202,
        // 48 windows 1.60 -> 1.19, 64 windows 1.48 -> 1.31 (and 64 x 4096 10.2 -> 7.9). With
        // fewer CUs left the streamed projection sets the pace: 72 windows 1.56 against 1.64,
        // 80 windows 1.61 against 2.06, 96 windows 1.81 against 3.54.
        pipeline = pipe_possible && concurrent == 2 && 2 * rec_wgs <= static_cast<long long>(cu_count);
    }
    // windows per projection row block: up to 4, a multiple of the recurrence tile, so a
    // recurrence tile never spans two row blocks; chunk = 128 / that many steps
    int group_windows = 1;
    if (pipeline) {
        while (group_windows < 4 && group_windows < static_cast<long long>(batch)) group_windows *= 2;
        group_windows = std::max(group_windows, tile);
    }

    // Batch slices: while one slice's recurrence runs (on 2·tiles/slices of the CUs), another
    // slice's projection uses the CUs it leaves idle. Only single-workgroup tiles: a split
    // tile's workgroups wait for each other, and two slices' launches partly resident at once
    // could then wait on each other for good.
    int slices = 1;
    if (pipeline) {
        // the streamed projection already runs beside the recurrence
    } else if (want_slices > 1) {
        if (groups != 1 || concurrent == 1 || projection == kProjectionVendor) {
            return fail(BILSTM_UNSUPPORTED,
                        "schedule: %d slices need recur_groups = 1, concurrent != 1 and the library's own "
                        "projection", want_slices);
        }
        slices = want_slices;
    } else if (want_slices == 0 && groups == 1 && concurrent != 1 && projection != kProjectionVendor) {
        // auto: slice when the recurrence leaves at least half of the CUs idle
        if (2 * grid * 2 <= cu_count && static_cast<long long>(batch) >= 2LL * tile) slices = kAutoSlices;
    }
    // windows per slice: a whole number of tiles
    const long long tiles_per_slice = (static_cast<long long>(tiles) + slices - 1) / slices;
    const int slice_windows = static_cast<int>(std::min<long long>(tiles_per_slice * tile, batch));
    slices = static_cast<int>((static_cast<long long>(batch) + slice_windows - 1) / slice_windows);

    info->batch = batch;
    info->steps = steps;
    info->slices = slices;
    info->slice_windows = slice_windows;
    info->projection = projection;
    info->pipeline = pipeline ? 1 : 0;
    info->stream_chunk = pipeline ? kProjTileM / group_windows : 0;
    info->stream_split =
        pipeline ? stream_split(static_cast<int>((batch + group_windows - 1) / group_windows),
                                stream_projection_workgroups(cu_count, static_cast<int>(tiles), groups))
                 : 0;
    // The next layer's projection starts during this layer's recurrence unless asked not to
    // (3): measured faster both where the recurrence sets the pace (b32: 1.44 -> 1.39 ms) and
    // where the projection does (b64_t4096: 10.45 -> 10.32 ms).
    info->stream_overlap = pipeline && want_pipe != 3 && want_pipe != 5 ? 1 : 0;
    info->stream_serial = pipeline && want_pipe == 5 ? 1 : 0;
    // 4: the four layers' recurrences as one launch, when one launch holds both directions of
    // every tile. A layer boundary waits for the next layer's first chunk either way, which
    // outlasts a kernel launch: on earlier builds a launch per layer measured faster, on the
    // current one the single launch is 0.3-0.6 % faster at 1-32 windows (b32 1.1205 against
    // 1.1167 ms). It is not the default because the HBM counters of the recurrence cannot be
    // taken for it: counter collection runs kernels one at a time, and the single launch waits
    // for projections that run beside it.
    info->stream_fused = info->stream_overlap && concurrent == 2 && launches == 1 && want_pipe == 4 ? 1 : 0;
    info->recur_groups = groups;
    info->recur_tile = tile;
    info->recur_tiles = tiles;
    info->recur_threads = recur_threads(groups);
    info->recur_launches = launches;
    info->concurrent = concurrent;
    info->cu_count = cu_count;
    info->recur_capacity = capacity;
    return BILSTM_OK;
}

}  // namespace bl

extern "C" bilstm_status bilstm_pack_layer(const bilstm_layer *layer, uint32_t in, float *w_out,
                                           size_t w_out_len, float *r_out, size_t r_out_len,
                                           float *bias_out, size_t bias_out_len) {
    using namespace bl;
    if (layer == nullptr || w_out == nullptr || r_out == nullptr || bias_out == nullptr ||
        layer->w == nullptr || layer->r == nullptr || layer->b == nullptr) {
        return fail(BILSTM_INVALID_ARGUMENT, "pack_layer: NULL pointer");
    }
    if (in == 0 || in % 4 != 0 || in > 4096) {
        return fail(BILSTM_INVALID_ARGUMENT, "pack_layer: input width %u must be a positive multiple of 4", in);
    }
    const size_t kpad = static_cast<size_t>(padded_input(static_cast<int>(in)));
    bilstm_status s;
    if ((s = check_len("pack_layer W", 2ull * kGates * in, layer->w_len)) != BILSTM_OK) return s;
    if ((s = check_len("pack_layer R", 2ull * kGates * kHidden, layer->r_len)) != BILSTM_OK) return s;
    if ((s = check_len("pack_layer B", 4ull * kGates, layer->b_len)) != BILSTM_OK) return s;
    if ((s = check_len("pack_layer packed W", kGateCols * kpad, w_out_len)) != BILSTM_OK) return s;
    if ((s = check_len("pack_layer packed R", 2ull * kGates * kHidden, r_out_len)) != BILSTM_OK) return s;
    if ((s = check_len("pack_layer packed bias", kGateCols, bias_out_len)) != BILSTM_OK) return s;
    return pack_layer(*layer, static_cast<int>(in), w_out, r_out, bias_out);
}

extern "C" bilstm_status bilstm_schedule(uint32_t batch, uint32_t steps, int32_t cu_count,
                                         int32_t per_cu, const bilstm_options *options,
                                         bilstm_plan_info *info) {
    if (info == nullptr) return bl::fail(BILSTM_INVALID_ARGUMENT, "schedule: info is NULL");
    std::memset(info, 0, sizeof(*info));
    info->proj_tile_m = bl::kProjTileM;
    info->proj_tile_n = bl::kProjTileN;
    return bl::schedule(batch, steps, cu_count, per_cu, options, info);
}
