// CPU model of the publication protocols of protocol.h, run on std::thread producers and
// consumers over std::atomic words (host only; built with g++, also under ThreadSanitizer).
//
// Each scenario drives the same functions the kernels and the plan use — flag values and word
// layout of the h exchange, flag-range reservation and its clear, counter targets and their
// signed comparison, the counters' clear rule, progress words — with random delays between
// operations so that producers and consumers interleave differently from run to run. Every
// value a consumer accepts is checked against the one its producer wrote for that step and
// pass; stale words (left by an earlier step, layer or pass, or planted before the run) must
// never be accepted, and a producer that never publishes must end every wait on it at the
// watchdog, after which all threads finish.
//
// Producers publish with release stores / read-modify-writes and consumers observe with
// acquire loads: the order the kernels obtain on the GPU by waiting for their stores to
// complete before publishing (s_waitcnt) and by issuing their reads only after the observed
// value arrived. The model checks the protocols' logic (values, parities, targets, wrap
// clears, watchdogs), not the GPU's memory model.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "protocol.h"

namespace {

using Clock = std::chrono::steady_clock;

struct Rng {
    uint64_t s;
    explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
    uint32_t next() {
        s ^= s << 13;
        s ^= s >> 7;
        s ^= s << 17;
        return static_cast<uint32_t>(s >> 11);
    }
    // a short random pause: nothing, a yield, or a spin of up to a few hundred iterations
    void pause() {
        const uint32_t r = next() % 16;
        if (r < 10) return;
        if (r < 13) {
            std::this_thread::yield();
            return;
        }
        volatile uint32_t sink = 0;
        for (uint32_t i = 0, n = next() % 400; i < n; ++i) sink = sink + i;
    }
};

// The value a producer publishes: distinct for every (pass, layer, step, unit, window), never
// the bit pattern a planted stale word carries (stale words have the top bit set, these not).
uint32_t value_of(uint32_t pass, uint32_t layer, uint32_t step, uint32_t unit, uint32_t b) {
    uint64_t h = (static_cast<uint64_t>(pass) << 40) ^ (static_cast<uint64_t>(layer) << 32) ^
                 (static_cast<uint64_t>(step) << 12) ^ (static_cast<uint64_t>(unit) << 4) ^ b;
    h *= 0xD6E8FEB86659FD93ull;
    h ^= h >> 29;
    return static_cast<uint32_t>(h) & 0x7FFFFFFFu;
}

// Bounded wait: poll `ready()` until it holds or `ms` milliseconds pass.
template <typename F>
bool wait_until(F &&ready, int ms, Rng &rng) {
    if (ready()) return true;
    const auto t0 = Clock::now();
    while (true) {
        rng.pause();
        if (ready()) return true;
        if (Clock::now() - t0 > std::chrono::milliseconds(ms)) return false;
    }
}

}  // namespace

extern "C" {

typedef struct {
    uint64_t accepted;      // words, chunks or progress values a consumer accepted
    uint64_t wrong_values;  // accepted values that were not what the producer wrote for it
    uint64_t timeouts;      // waits that gave up at the watchdog
    uint64_t clears;        // clears the host-side logic ordered
    uint64_t passes;        // passes run
} bilstm_model_result;

// h exchange of one window tile of `tile` windows split over `groups` member threads (`units`
// hidden units in all), `layers` layers of `steps` steps per pass, `passes` passes. The flag
// epoch starts at `start_epoch`. stale_fill = 1 plants, before the first pass, words whose
// flags lie in [1, start_epoch] (or anywhere when start_epoch is 0) and whose values are never
// a producer's. Member `missing` (-1: none) publishes nothing from step `missing_from` of its
// first layer on. `skew` is added to every expected flag (forced timeouts).
int bilstm_model_exchange(int groups, int units, int tile, int steps, int layers, int passes,
                          uint32_t start_epoch, int stale_fill, int missing, int missing_from, uint32_t skew,
                          int watchdog_ms, uint32_t seed, bilstm_model_result *out) {
    if (out == nullptr || groups < 1 || units % groups != 0 || tile < 1 || steps < 1 || layers < 1 || passes < 1) {
        return 1;
    }
    std::memset(out, 0, sizeof(*out));
    const int per = units / groups;
    std::vector<std::atomic<uint64_t>> words(static_cast<size_t>(2) * units * tile);
    for (auto &w : words) w.store(0, std::memory_order_relaxed);
    Rng host(seed);
    if (stale_fill) {
        for (auto &w : words) {
            const uint32_t f = start_epoch > 0 ? 1 + host.next() % start_epoch : host.next();
            w.store(bl::exchange_word(f, 0x80000000u | host.next()), std::memory_order_relaxed);
        }
    }
    std::atomic<uint64_t> accepted{0}, wrong{0}, timeouts{0};
    uint32_t epoch = start_epoch;
    for (int p = 0; p < passes; ++p) {
        bool clear = false;
        const uint32_t base = bl::reserve_flag_range(epoch, static_cast<uint32_t>(layers * steps), clear);
        if (clear) {
            // the clear kernel runs on the stream before the pass
            for (auto &w : words) w.store(0, std::memory_order_relaxed);
            ++out->clears;
        }
        for (int l = 0; l < layers; ++l) {
            // one launch: every member of the tile, joined at its end
            const uint32_t flag_base = base + static_cast<uint32_t>(l * steps);
            std::vector<std::thread> members;
            for (int m = 0; m < groups; ++m) {
                members.emplace_back([&, m] {
                    Rng rng(seed * 1000003u + static_cast<uint32_t>(p * 131 + l * 17 + m));
                    bool timed_out = false;
                    for (int s = 0; s < steps; ++s) {
                        const uint32_t flag = bl::exchange_flag(flag_base, s);
                        const bool silent = m == missing && p == 0 && l == 0 && s >= missing_from;
                        for (int u = m * per; u < (m + 1) * per && !silent; ++u) {
                            for (int b = 0; b < tile; ++b) {
                                rng.pause();
                                words[bl::exchange_index(s, u, b, units, tile)].store(
                                    bl::exchange_word(flag, value_of(p, l, s, u, b)), std::memory_order_release);
                            }
                        }
                        // gather the other members' h of step s
                        for (int u = 0; u < units; ++u) {
                            if (u / per == m) continue;
                            for (int b = 0; b < tile; ++b) {
                                std::atomic<uint64_t> &wp = words[bl::exchange_index(s, u, b, units, tile)];
                                uint64_t w = wp.load(std::memory_order_acquire);
                                const uint32_t expect = flag + skew;
                                if (bl::word_flag(w) != expect && !timed_out) {
                                    const bool ok = wait_until(
                                        [&] {
                                            w = wp.load(std::memory_order_acquire);
                                            return bl::word_flag(w) == expect;
                                        },
                                        watchdog_ms, rng);
                                    if (!ok) {
                                        timed_out = true;
                                        timeouts.fetch_add(1);
                                    }
                                }
                                if (bl::word_flag(w) == expect) {
                                    accepted.fetch_add(1);
                                    if (bl::word_value(w) != value_of(p, l, s, u, b)) wrong.fetch_add(1);
                                }
                            }
                        }
                    }
                });
            }
            for (auto &t : members) t.join();
        }
        ++out->passes;
    }
    out->accepted = accepted.load();
    out->wrong_values = wrong.load();
    out->timeouts = timeouts.load();
    return 0;
}

// Chunk counters of the streamed gates: `passes` passes of one gate buffer for `groups` window
// groups × 2 directions × `chunks` chunks. Per pass, `workers` projection threads walk the
// tiles in the streamed order (chunk 0 in tiles of 128 / split columns, the others 128 wide;
// 512 columns per direction), store each tile's values, then add width / 32 to its counter;
// one recurrence thread per (direction, group) waits for each chunk in turn and checks every
// value of it. The pass count starts at `start_passes` with the counters holding what that
// many passes left (the plan's state after so many passes); the plan's clear rule is applied
// before every pass. Tile `missing` of the first pass (-1: none) is never published. `skew` is
// added to every target (forced timeouts).
int bilstm_model_counters(int groups, int chunks, int split, int workers, int passes, uint32_t start_passes,
                          int missing, uint32_t skew, int watchdog_ms, uint32_t seed, bilstm_model_result *out) {
    if (out == nullptr || groups < 1 || chunks < 1 || workers < 1 || passes < 1 ||
        (split != 1 && split != 2 && split != 4)) {
        return 1;
    }
    std::memset(out, 0, sizeof(*out));
    constexpr int kCols = bl::kGatesPerDirection;  // gate columns per direction
    constexpr int kVals = 4;                       // values per 32 columns of a (chunk, dir, group)
    const int ncounters = chunks * 2 * groups;
    std::vector<std::atomic<uint32_t>> counters(ncounters);
    // plain memory: only the counters order the projection's stores before the recurrence's loads
    std::vector<uint32_t> vals(static_cast<size_t>(ncounters) * (kCols / 32) * kVals, 0x80000000u);
    uint32_t ready_passes[2] = {start_passes, start_passes};
    uint32_t layer_pass = start_passes;
    for (auto &c : counters) c.store(bl::ready_target(start_passes, 0), std::memory_order_relaxed);
    // the tiles of one pass in the streamed order: (chunk, dir, group, first column, width)
    struct Tile {
        int c, d, g, col, width;
    };
    std::vector<Tile> tiles;
    for (int d = 0; d < 2; ++d)
        for (int g = 0; g < groups; ++g)
            for (int q = 0; q < 4 * split; ++q) tiles.push_back({0, d, g, q * (128 / split), 128 / split});
    for (int c = 1; c < chunks; ++c)
        for (int d = 0; d < 2; ++d)
            for (int g = 0; g < groups; ++g)
                for (int q = 0; q < 4; ++q) tiles.push_back({c, d, g, q * 128, 128});
    std::atomic<uint64_t> accepted{0}, wrong{0}, timeouts{0};
    bool dirty = false;  // the last pass timed out: its counters may lag behind the pass count
    for (int p = 0; p < passes; ++p) {
        if (bl::stream_counters_need_clear(layer_pass, ready_passes, dirty)) {
            for (auto &c : counters) c.store(0, std::memory_order_relaxed);
            ready_passes[0] = ready_passes[1] = 0;
            layer_pass = 0;
            ++out->clears;
        }
        ++layer_pass;
        const uint32_t pass = ++ready_passes[0];
        const uint32_t target = bl::ready_target(pass, skew);
        const uint64_t timeouts_before = timeouts.load();
        std::atomic<int> next_tile{0};
        std::vector<std::thread> threads;
        // the recurrence's waits start first, and the projection's workers a moment later, so a
        // wait that let a chunk through too early would read it before it is written
        for (int d = 0; d < 2; ++d) {
            for (int g = 0; g < groups; ++g) {
                threads.emplace_back([&, d, g] {
                    Rng rng(seed * 104729u + static_cast<uint32_t>(p * 31 + d * 7 + g));
                    bool timed_out = false;
                    for (int c = 0; c < chunks; ++c) {
                        const int counter = bl::counter_index(c, d, g, groups);
                        bool ok = bl::chunk_published(counters[counter].load(std::memory_order_acquire), target);
                        if (!ok && !timed_out) {
                            ok = wait_until(
                                [&] {
                                    return bl::chunk_published(counters[counter].load(std::memory_order_acquire),
                                                               target);
                                },
                                watchdog_ms, rng);
                            if (!ok) {
                                timed_out = true;
                                timeouts.fetch_add(1);
                            }
                        }
                        if (!ok) continue;
                        accepted.fetch_add(1);
                        for (int k = 0; k < kCols / 32; ++k) {
                            for (int v = 0; v < kVals; ++v) {
                                const uint32_t got = vals[(static_cast<size_t>(counter) * (kCols / 32) + k) * kVals + v];
                                if (got != (value_of(pass, 0, c, k, v) ^ static_cast<uint32_t>(counter << 8))) {
                                    wrong.fetch_add(1);
                                }
                            }
                        }
                    }
                });
            }
        }
        for (int w = 0; w < workers; ++w) {
            threads.emplace_back([&, w] {
                Rng rng(seed * 7919u + static_cast<uint32_t>(p * 257 + w));
                std::this_thread::sleep_for(std::chrono::milliseconds(2));
                for (int q; (q = next_tile.fetch_add(1)) < static_cast<int>(tiles.size());) {
                    const Tile &t = tiles[q];
                    if (p == 0 && q == missing) continue;
                    const int counter = bl::counter_index(t.c, t.d, t.g, groups);
                    for (int k = t.col / 32; k < (t.col + t.width) / 32; ++k) {
                        for (int v = 0; v < kVals; ++v) {
                            rng.pause();
                            vals[(static_cast<size_t>(counter) * (kCols / 32) + k) * kVals + v] =
                                value_of(pass, 0, t.c, k, v) ^ static_cast<uint32_t>(counter << 8);
                        }
                    }
                    counters[counter].fetch_add(static_cast<uint32_t>(t.width / 32), std::memory_order_release);
                }
            });
        }
        for (auto &t : threads) t.join();
        // a pass whose waits timed out leaves the plan to clear the counters before the next one
        dirty = timeouts.load() != timeouts_before;
        ++out->passes;
    }
    out->accepted = accepted.load();
    out->wrong_values = wrong.load();
    out->timeouts = timeouts.load();
    return 0;
}

// Progress words: a recurrence thread per (window, direction) writes its output of layer pass
// `layer_pass` step by step and publishes {pass << 32 | steps done} every `every` steps; a
// projection thread per window reads, for each chunk of `chunk` steps, the rows it needs once
// the words show them done (forward steps up to the chunk's end, reverse steps down to its
// start, as the next layer's tiles do) and checks them. Before the pass the words hold the
// previous pass's final words (all steps done), which must not let any read through. Window
// `missing` (-1: none) never publishes; its reader must end at the watchdog.
int bilstm_model_progress(int windows, int steps, int chunk, int every, uint32_t layer_pass, int missing,
                          int watchdog_ms, uint32_t seed, bilstm_model_result *out) {
    if (out == nullptr || windows < 1 || steps < 1 || chunk < 1 || every < 1 || layer_pass < 1) return 1;
    std::memset(out, 0, sizeof(*out));
    std::vector<std::atomic<uint64_t>> words(static_cast<size_t>(windows) * 2);
    // plain memory: only the progress words order the recurrence's stores before the loads
    std::vector<uint32_t> outputs(static_cast<size_t>(windows) * 2 * steps, 0x80000000u);
    const uint64_t stale = bl::progress_word(bl::progress_pass_bits(layer_pass - 1), static_cast<uint32_t>(steps));
    for (auto &w : words) w.store(stale, std::memory_order_relaxed);
    const uint64_t bits = bl::progress_pass_bits(layer_pass);
    std::atomic<uint64_t> accepted{0}, wrong{0}, timeouts{0};
    std::vector<std::thread> threads;
    for (int w = 0; w < windows; ++w) {
        for (int d = 0; d < 2; ++d) {
            threads.emplace_back([&, w, d] {
                if (w == missing) return;
                Rng rng(seed * 31337u + static_cast<uint32_t>(w * 2 + d));
                // the readers are already waiting: a wait that let rows through too early reads
                // them before they are written
                std::this_thread::sleep_for(std::chrono::milliseconds(2));
                for (int s = 0; s < steps; ++s) {
                    const int t = d == 0 ? s : steps - 1 - s;
                    rng.pause();
                    outputs[(static_cast<size_t>(w) * 2 + d) * steps + t] = value_of(layer_pass, d, t, w, 0);
                    if ((s + 1) % every == 0 || s + 1 == steps) {
                        words[static_cast<size_t>(w) * 2 + d].store(
                            bl::progress_word(bits, static_cast<uint32_t>(s + 1)), std::memory_order_release);
                    }
                }
            });
        }
        threads.emplace_back([&, w] {
            Rng rng(seed * 65537u + static_cast<uint32_t>(w));
            bool timed_out = false;
            for (int c = 0; c * chunk < steps && !timed_out; ++c) {
                // rows of times [c·chunk, min(c·chunk + chunk, T)): the forward direction must have
                // run up to the chunk's end, the reverse one down to its start
                const uint32_t need[2] = {static_cast<uint32_t>(std::min(c * chunk + chunk, steps)),
                                          static_cast<uint32_t>(steps - c * chunk)};
                for (int d = 0; d < 2 && !timed_out; ++d) {
                    std::atomic<uint64_t> &word = words[static_cast<size_t>(w) * 2 + d];
                    const bool ok = wait_until(
                        [&] { return bl::progress_reached(word.load(std::memory_order_acquire), bits, need[d]); },
                        watchdog_ms, rng);
                    if (!ok) {
                        timed_out = true;
                        timeouts.fetch_add(1);
                        break;
                    }
                    accepted.fetch_add(1);
                    for (int t = c * chunk; t < std::min(c * chunk + chunk, steps); ++t) {
                        const uint32_t got = outputs[(static_cast<size_t>(w) * 2 + d) * steps + t];
                        if (got != value_of(layer_pass, d, t, w, 0)) wrong.fetch_add(1);
                    }
                }
            }
        });
    }
    for (auto &t : threads) t.join();
    out->accepted = accepted.load();
    out->wrong_values = wrong.load();
    out->timeouts = timeouts.load();
    out->passes = 1;
    return 0;
}

// The tile order of one streamed projection workgroup, chosen with the walk functions as the
// kernel chooses it, against a previous layer that runs `rate` steps per unit of time from time
// 0 (both directions alike). The workgroup starts at `start`; a tile starts computing once its
// rows exist and takes `tile_time`. chunks[k] is tile k's chunk (never falling); lead0 = 0:
// plain consumption order. Writes order[i] (the i-th tile taken) and begin[k] / end[k] (when
// tile k computed) and returns the number of tiles taken: -1 for bad arguments, -2 when a tile
// out of range or one already taken comes up.
int bilstm_model_stream_walk(int n, const int *chunks, int steps, int chunk, uint32_t lead0, double rate,
                             double start, double tile_time, int *order, double *begin, double *end) {
    if (n < 0 || chunks == nullptr || steps < 1 || chunk < 1 || rate <= 0.0 || tile_time <= 0.0 ||
        order == nullptr || begin == nullptr || end == nullptr) {
        return -1;
    }
    for (int k = 1; k < n; ++k) {
        if (chunks[k] < chunks[k - 1]) return -1;
    }
    auto progress_at = [&](double t) {
        const double s = std::floor(rate * t);
        return static_cast<uint32_t>(s <= 0.0 ? 0.0 : s >= steps ? steps : s);
    };
    auto chunk_of = [&](int k) { return chunks[k]; };
    bl::StreamWalk w;
    const int mid = lead0 > 0 && n > 0 ? bl::stream_walk_mid(n, steps, chunk, chunk_of) : 0;
    bl::stream_walk_init(w, n, mid, steps, lead0, lead0 > 0);
    double t = start;
    int cur, next;
    bl::stream_walk_start(w, progress_at(t), cur, next);
    std::vector<char> taken(static_cast<size_t>(n), 0);
    int i = 0;
    while (cur >= 0) {
        if (i >= n || cur >= n || taken[static_cast<size_t>(cur)]) return -2;
        taken[static_cast<size_t>(cur)] = 1;
        order[i] = cur;
        const uint32_t seen = progress_at(t);  // read at the tile's start
        const int need = bl::chunk_need(steps, chunk, chunks[cur]);
        begin[cur] = std::max(t, need / rate);
        end[cur] = begin[cur] + tile_time;
        const int after = next >= 0 ? bl::stream_walk_after(w, i, seen, static_cast<uint32_t>(need)) : -1;
        t = end[cur];
        cur = next;
        next = after;
        ++i;
    }
    return i;
}

}  // extern "C"

#ifdef BILSTM_MODEL_MAIN
// Stand-alone driver (the ThreadSanitizer build): every scenario once; exit status 0 when each
// accepted value was its producer's and watchdogs fired exactly where a producer was missing.
#include <cstdio>

// The walk against a layout: every tile taken once, in the walk's shape (mid, mid - 1, ..., lo,
// then 0 .. lo - 1, then mid + 1 .. n - 1; plain consumption order when lead0 = 0).
static bool walk_is_whole(int n, const int *chunks, int steps, int chunk, uint32_t lead0, double rate, double start,
                          double tile_time, std::vector<int> &order, std::vector<double> &end) {
    order.assign(static_cast<size_t>(n), -1);
    std::vector<double> begin(static_cast<size_t>(n));
    end.assign(static_cast<size_t>(n), 0.0);
    if (bilstm_model_stream_walk(n, chunks, steps, chunk, lead0, rate, start, tile_time, order.data(), begin.data(),
                                 end.data()) != n) {
        return false;
    }
    int i = 0;
    const int mid = order[0];
    while (i < n && order[static_cast<size_t>(i)] == mid - i) ++i;  // the walk down from order[0]
    const int lo = mid - i + 1;
    if (lead0 == 0 && mid != 0) return false;
    std::vector<int> want;
    if (lead0 == 0) {
        for (int k = 0; k < n; ++k) want.push_back(k);
    } else {
        for (int k = mid; k >= lo; --k) want.push_back(k);
        for (int k = 0; k < lo; ++k) want.push_back(k);
        for (int k = mid + 1; k < n; ++k) want.push_back(k);
    }
    return want == order;
}

// The next layer's recurrence reading chunk c once its tile has ended (one tile per chunk).
static double consumer_end(const std::vector<double> &end, double start, double chunk_time) {
    double t = start;
    for (double e : end) t = std::max(t, e) + chunk_time;
    return t;
}

static int walk_checks() {
    int failures = 0;
    auto expect = [&](const char *name, bool ok) {
        std::printf("%-40s %s\n", name, ok ? "ok" : "FAIL");
        failures += ok ? 0 : 1;
    };
    // 4096 steps of 32-step chunks, one tile per chunk: the previous layer takes 1810 time
    // units, a tile 17.6, and the workgroup starts at 900
    std::vector<int> chunks(128);
    for (int k = 0; k < 128; ++k) chunks[static_cast<size_t>(k)] = k;
    const double rate = 4096.0 / 1810.0;
    std::vector<int> plain, walked;
    std::vector<double> plain_end, walked_end;
    const bool whole = walk_is_whole(128, chunks.data(), 4096, 32, 0, rate, 900.0, 17.6, plain, plain_end) &&
                       walk_is_whole(128, chunks.data(), 4096, 32, 64, rate, 900.0, 17.6, walked, walked_end);
    expect("walk, every tile once", whole);
    // chunks 63 and 64 need 2080 steps each: the walk starts at the later
    expect("walk, starts at the last tile of least need", whole && walked[0] == 64);
    expect("walk, chunk 0 no later", whole && walked_end[0] <= plain_end[0]);
    expect("walk, the next layer ends earlier",
           whole && consumer_end(walked_end, 1810.0, 1810.0 / 128) < 0.95 * consumer_end(plain_end, 1810.0, 1810.0 / 128));
    // a workgroup's tiles on chunks 0, 2, 5, 8, 11, 14, 17 of 589 steps: chunk 8 needs least
    const int few[] = {0, 2, 5, 8, 11, 14, 17};
    expect("walk, seven tiles", walk_is_whole(7, few, 589, 32, 64, 589.0 / 270.0, 0.0, 10.0, walked, walked_end) &&
                                    walked[0] == 3);
    // random layouts, rates and starts
    Rng rng(77);
    bool all = true;
    for (int trial = 0; trial < 300 && all; ++trial) {
        const int n = 1 + static_cast<int>(rng.next() % 200);
        const int chunk = 8 << (rng.next() % 4);
        const int steps = 1 + static_cast<int>(rng.next() % 5000);
        const int nchunks = (steps + chunk - 1) / chunk;
        std::vector<int> layout(static_cast<size_t>(n));
        for (int k = 0; k < n; ++k) layout[static_cast<size_t>(k)] = static_cast<int>(rng.next() % nchunks);
        std::sort(layout.begin(), layout.end());
        const double r = 0.5 + (rng.next() % 1000) / 200.0;
        const double start = (rng.next() % 1000) / 1000.0 * steps / r;
        const double tau = 0.5 + (rng.next() % 100);
        const uint32_t lead0 = trial % 3 == 0 ? 0u : 1u + rng.next() % 200;
        all = walk_is_whole(n, layout.data(), steps, chunk, lead0, r, start, tau, walked, walked_end);
    }
    expect("walk, random layouts", all);
    // the lead counts from when the tile's rows were complete
    expect("walk, lead from readiness", bl::stream_walk_lead(100, 40, 70) == 30 && bl::stream_walk_lead(100, 80, 70) == 20 &&
                                            bl::stream_walk_lead(50, 40, 70) == 0);
    return failures;
}

// argv[1]: the watchdog of the scenarios where every producer publishes, in ms (default 2000)
int main(int argc, char **argv) {
    const int wd = argc > 1 ? std::atoi(argv[1]) : 2000;
    int failures = 0;
    auto expect = [&](const char *name, const bilstm_model_result &r, bool want_timeouts) {
        const bool ok = r.wrong_values == 0 && (want_timeouts ? r.timeouts > 0 : r.timeouts == 0) && r.accepted > 0;
        std::printf("%-40s accepted %llu wrong %llu timeouts %llu clears %llu %s\n", name,
                    static_cast<unsigned long long>(r.accepted), static_cast<unsigned long long>(r.wrong_values),
                    static_cast<unsigned long long>(r.timeouts), static_cast<unsigned long long>(r.clears),
                    ok ? "ok" : "FAIL");
        failures += ok ? 0 : 1;
    };
    bilstm_model_result r;
    bilstm_model_exchange(4, 32, 2, 40, 4, 3, 0, 1, -1, 0, 0, wd, 1, &r);
    expect("exchange 4 members, stale words", r, false);
    bilstm_model_exchange(2, 16, 1, 30, 4, 3, 0xFFFFFFFFu - 200u, 1, -1, 0, 0, wd, 2, &r);
    expect("exchange across the flag wrap", r, false);
    bilstm_model_exchange(4, 32, 1, 20, 2, 1, 0, 0, 2, 5, 0, 50, 3, &r);
    expect("exchange, a member goes silent", r, true);
    bilstm_model_counters(3, 5, 2, 4, 4, 0, -1, 0, wd, 4, &r);
    expect("counters", r, false);
    bilstm_model_counters(2, 4, 4, 3, 4, bl::kReadyPassLimit - 1, -1, 0, wd, 5, &r);
    expect("counters across the clear", r, false);
    bilstm_model_counters(2, 4, 1, 3, 1, 0, 9, 0, 50, 6, &r);
    expect("counters, a tile never published", r, true);
    bilstm_model_progress(4, 120, 32, 8, 7, -1, wd, 7, &r);
    expect("progress, stale final words", r, false);
    bilstm_model_progress(3, 64, 16, 4, 2, 1, 50, 8, &r);
    expect("progress, a window never published", r, true);
    failures += walk_checks();
    return failures == 0 ? 0 : 1;
}
#endif
