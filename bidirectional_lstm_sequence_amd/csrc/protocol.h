// The publication protocols between concurrently running workgroups, as plain functions shared
// by the HIP kernels, the host plan code and the CPU model of the protocols
// (protocol_model.cpp, which runs them on std::thread producers and consumers). No GPU types.
//
// 1. Exchange words (recurrence split over KG workgroups per window tile; speakrs 0.6.0, page
//    `lstmproj.rs`, `Exchange` doc, `DirectionLaunch` doc and `clear_state`). The producer of
//    hidden unit j publishes h_t of step s as one 64-bit word {flag, h bits} in the buffer of
//    parity s mod 2; flag = flag_base + s + 1, where flag_base = epoch + layer·T grows across the
//    layers of a pass and across passes, so a word left by an earlier step, layer or pass never
//    carries the flag a later wait expects. The words are zeroed at plan creation and whenever
//    the next pass's flags would pass 2^32 - 1 (the epoch then restarts at 0); zero never
//    matches, because every flag is at least 1.
// 2. Chunk counters (streamed gates). The projection adds a tile's width / 32 to the counter of
//    (chunk, direction, window group) once the tile's gates are stored; a pass adds
//    kReadyPerPass to every counter. Pass n of a counter waits until it reaches n·kReadyPerPass,
//    compared as a signed 32-bit difference, so the comparison needs no clear while the counts
//    stay below 2^31; the plan clears counters and pass counts well before that.
// 3. Progress words (streamed gates, the next layer's projection beside this layer's
//    recurrence): {layer pass << 32 | steps whose output has completed}, one per window and
//    direction. A reader of layer pass p needs a word >= (p << 32 | steps it needs): words of
//    earlier passes are smaller whatever their step count.
// 4. Tile order of a streamed projection workgroup beside the previous layer's recurrence:
//    the tiles whose rows exist first, then the rest in consumption order (section 4 below).
#pragma once

#include <cstdint>

#ifdef __HIP__  // HIP-language sources; the CPU model compiles this header as plain C++
#define BL_HD __host__ __device__
#else
#define BL_HD
#endif

namespace bl {

constexpr int kGatesPerDirection = 512;
// Counter increments per pass: every tile of a chunk adds its width / 32, over 512 columns.
constexpr int kReadyPerPass = kGatesPerDirection / 32;

// ---- 1. exchange words ----------------------------------------------------------------------
BL_HD inline uint32_t exchange_flag(uint32_t flag_base, int step) {
    return flag_base + static_cast<uint32_t>(step) + 1u;
}
BL_HD inline uint64_t exchange_word(uint32_t flag, uint32_t value_bits) {
    return (static_cast<uint64_t>(flag) << 32) | value_bits;
}
BL_HD inline uint32_t word_flag(uint64_t word) { return static_cast<uint32_t>(word >> 32); }
BL_HD inline uint32_t word_value(uint64_t word) { return static_cast<uint32_t>(word); }
// Index of (parity of `step`, unit, window b) in one tile's [2][128][tile] words.
BL_HD inline int exchange_index(int step, int unit, int b, int hidden, int tile) {
    return ((step & 1) * hidden + unit) * tile + b;
}

// The flag range of the next pass: `count` = layers · steps flags above `epoch`. Returns the
// pass's flag_base and advances `epoch`; sets `clear` when the words must be zeroed first
// (the range would pass 2^32 - 1), in which case the range starts again at 0.
inline uint32_t reserve_flag_range(uint32_t &epoch, uint32_t count, bool &clear) {
    clear = static_cast<uint64_t>(epoch) + count + 1 > 0xFFFFFFFFull;
    if (clear) epoch = 0;
    const uint32_t base = epoch;
    epoch += count;
    return base;
}

// ---- 2. chunk counters ----------------------------------------------------------------------
// The value pass `passes` (1 for the first pass after a clear) waits for; `skew` is 0, or a
// value no pass reaches (forced-timeout tests).
BL_HD inline uint32_t ready_target(uint32_t passes, uint32_t skew) {
    return passes * static_cast<uint32_t>(kReadyPerPass) + skew;
}
BL_HD inline bool chunk_published(uint32_t counter, uint32_t target) {
    return static_cast<int32_t>(counter - target) >= 0;
}
// Counter of (chunk c, direction d, window group g) among `groups` groups.
BL_HD inline int counter_index(int c, int d, int g, int groups) { return (c * 2 + d) * groups + g; }
// Pass counts above which the counters, progress words and counts are cleared.
constexpr uint32_t kReadyPassLimit = 0x03FFFFFFu;
constexpr uint32_t kLayerPassLimit = 0x0FFFFFF0u;
inline bool stream_counters_need_clear(uint32_t layer_pass, const uint32_t ready_passes[2], bool dirty) {
    return dirty || layer_pass > kLayerPassLimit || ready_passes[0] > kReadyPassLimit ||
           ready_passes[1] > kReadyPassLimit;
}

// ---- 3. progress words ----------------------------------------------------------------------
BL_HD inline uint64_t progress_pass_bits(uint32_t layer_pass) { return static_cast<uint64_t>(layer_pass) << 32; }
BL_HD inline uint64_t progress_word(uint64_t pass_bits, uint32_t done) { return pass_bits | done; }
BL_HD inline bool progress_reached(uint64_t seen, uint64_t pass_bits, uint32_t need) {
    return seen >= (pass_bits | need);
}
// Steps of pass `pass_bits` that a word shows: 0 for a word of an earlier pass, all `steps` for
// one of a later pass (that pass can only start once this one has ended).
BL_HD inline uint32_t progress_steps(uint64_t seen, uint64_t pass_bits, uint32_t steps) {
    if (seen < pass_bits) return 0;
    if ((seen >> 32) > (pass_bits >> 32)) return steps;
    const uint32_t done = static_cast<uint32_t>(seen);
    return done < steps ? done : steps;
}

// ---- 4. tile order of a streamed projection workgroup ---------------------------------------
// A persistent workgroup's streamed tiles k = 0 .. n-1 are numbered in the recurrence's
// consumption order (their chunk never falls as k rises). Tile k can be computed once the
// previous layer has run chunk_need(c_k) steps in both directions: the rows of the middle
// chunks exist from about half of that layer on, those of the first and of the last chunk only
// at its end. Taken in consumption order, a workgroup's first tile (chunk 0) holds it through
// the whole second half of the previous layer. The walk instead starts at `mid`, the last tile
// of least need, and goes down (mid, mid - 1, ...) while the tile being chosen would still end
// before the previous layer does; the remaining tiles then follow in consumption order
// (0 .. lo - 1, then mid + 1 .. n - 1), so chunk 0 starts just before its rows are complete.
// Every tile is taken once, and a tile's sums do not depend on when it is taken.
BL_HD inline int chunk_need(int steps, int chunk, int c) {
    const int near = c * chunk + chunk < steps ? c * chunk + chunk : steps;  // own direction
    const int far = steps - c * chunk;                                      // the other one
    return near > far ? near : far;
}

// The last tile of least need; chunk_of(k) is tile k's chunk. near - far rises with the chunk,
// so the least need is at the first tile where near >= far or at the tile before it.
template <class ChunkOf>
BL_HD inline int stream_walk_mid(int n, int steps, int chunk, ChunkOf chunk_of) {
    int a = 0, b = n;
    while (a < b) {
        const int m = (a + b) / 2;
        const int c = chunk_of(m);
        const int near = c * chunk + chunk < steps ? c * chunk + chunk : steps;
        if (near >= steps - c * chunk) {
            b = m;
        } else {
            a = m + 1;
        }
    }
    if (a == n) return n - 1;
    if (a > 0 && chunk_need(steps, chunk, chunk_of(a - 1)) < chunk_need(steps, chunk, chunk_of(a))) return a - 1;
    // the last tile of tile a's chunk
    const int c = chunk_of(a);
    int lo = a, hi = n;
    while (lo < hi) {
        const int m = (lo + hi) / 2;
        if (chunk_of(m) > c) {
            hi = m;
        } else {
            lo = m + 1;
        }
    }
    return lo - 1;
}

struct StreamWalk {
    int n;                   // the workgroup's tiles
    int lo, hi;              // the walk has taken tiles [lo, hi)
    int next_in_order;       // the next tile in consumption order, [lo, hi) skipped
    int steps;               // of the previous layer
    bool walking;
    uint32_t lead0;          // steps of the previous layer per tile, assumed until measured
    uint32_t lead;           // the largest measured so far
    uint32_t last_progress;  // progress seen at the previous tile's start
    uint32_t last_need;      // the previous tile's chunk_need
};

// walk = false: plain consumption order.
BL_HD inline void stream_walk_init(StreamWalk &w, int n, int mid, int steps, uint32_t lead0, bool walk) {
    w.n = n;
    w.lo = mid + 1;
    w.hi = mid + 1;
    w.next_in_order = 0;
    w.steps = steps;
    w.walking = walk && n > 1;
    w.lead0 = lead0;
    w.lead = 0;
    w.last_progress = 0;
    w.last_need = 0;
}

// The next tile (-1: none left). `progress` = steps the previous layer had run when the
// estimate starts, `lead` = steps it runs per tile of this workgroup, `horizon` = tiles from
// that moment to the end of the tile being chosen.
BL_HD inline int stream_walk_next(StreamWalk &w, uint32_t progress, uint32_t lead, int horizon) {
    if (w.walking) {
        if (w.lo > 0 && static_cast<uint64_t>(progress) + static_cast<uint64_t>(horizon) * lead <
                            static_cast<uint64_t>(w.steps)) {
            return --w.lo;
        }
        w.walking = false;
    }
    if (w.next_in_order == w.lo) w.next_in_order = w.hi;
    return w.next_in_order < w.n ? w.next_in_order++ : -1;
}

// Steps the previous layer ran during one tile: from the tile's start (progress `before`), or
// from when its rows were complete (`ready_at`) if it waited for them, to `now`.
BL_HD inline uint32_t stream_walk_lead(uint32_t now, uint32_t before, uint32_t ready_at) {
    const uint32_t from = before > ready_at ? before : ready_at;
    return now > from ? now - from : 0;
}

// A workgroup's first two tiles, chosen at its start (previous layer at `progress`): the first
// ends one tile from now, the second two.
BL_HD inline void stream_walk_start(StreamWalk &w, uint32_t progress, int &first, int &second) {
    first = stream_walk_next(w, progress, w.lead0, 1);
    second = first < 0 ? -1 : stream_walk_next(w, progress, w.lead0, 2);
}

// At the end of the workgroup's i-th tile (i = 0 first), whose start saw `progress` and whose
// rows needed `need` steps: the tile after the next one, which ends three tiles after that
// start. From the second tile on, the lead is the largest one measured.
BL_HD inline int stream_walk_after(StreamWalk &w, int i, uint32_t progress, uint32_t need) {
    uint32_t lead = w.lead0;
    if (i > 0) {
        const uint32_t m = stream_walk_lead(progress, w.last_progress, w.last_need);
        w.lead = m > w.lead ? m : w.lead;
        lead = w.lead;
    }
    w.last_progress = progress;
    w.last_need = need;
    return stream_walk_next(w, progress, lead, 3);
}

}  // namespace bl
