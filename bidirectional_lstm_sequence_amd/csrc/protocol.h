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

}  // namespace bl
