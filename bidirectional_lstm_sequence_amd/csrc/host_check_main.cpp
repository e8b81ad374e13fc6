// Host-side check of the library for the sanitizer build (AddressSanitizer, UndefinedBehavior
// Sanitizer on the host code only): the packer, the schedule over a grid of shapes and options,
// and every entry point's argument checks, none of which needs a GPU. With no GPU present the
// calls that reach the device return an error status, which is checked too. Exit status 0 when
// every call returned what it should.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/bilstm.h"

namespace {

int failures = 0;

void expect(bool ok, const char *what) {
    if (!ok) {
        std::printf("FAIL %s (last error: %s)\n", what, bilstm_last_error());
        ++failures;
    }
}

struct Weights {
    std::vector<float> w[BILSTM_LAYERS], r[BILSTM_LAYERS], b[BILSTM_LAYERS];
    bilstm_layer layers[BILSTM_LAYERS];
    Weights() {
        unsigned s = 12345u;
        auto rnd = [&s] {
            s = s * 1664525u + 1013904223u;
            return static_cast<float>(s >> 8) / 16777216.0f - 0.5f;
        };
        for (int l = 0; l < BILSTM_LAYERS; ++l) {
            const size_t in = l == 0 ? BILSTM_FEATURES : BILSTM_WIDTH;
            w[l].resize(2 * BILSTM_GATES * in);
            r[l].resize(2 * BILSTM_GATES * BILSTM_HIDDEN);
            b[l].resize(4 * BILSTM_GATES);
            for (auto *v : {&w[l], &r[l], &b[l]})
                for (float &x : *v) x = rnd();
            layers[l] = {w[l].data(), w[l].size(), r[l].data(), r[l].size(), b[l].data(), b[l].size()};
        }
    }
};

void check_packer(const Weights &wt) {
    for (int l = 0; l < 2; ++l) {
        const uint32_t in = l == 0 ? BILSTM_FEATURES : BILSTM_WIDTH;
        const uint32_t kpad = (in + 31) / 32 * 32;
        std::vector<float> w(1024 * kpad), r(2 * 512 * 128), b(1024);
        expect(bilstm_pack_layer(&wt.layers[l], in, w.data(), w.size(), r.data(), r.size(), b.data(), b.size()) ==
                   BILSTM_OK,
               "pack_layer");
        // row 4j + g of direction d holds source row g·128 + j
        for (int d = 0; d < 2; ++d)
            for (int src = 0; src < 512; ++src) {
                const int row = d * 512 + 4 * (src % 128) + src / 128;
                expect(std::memcmp(&w[static_cast<size_t>(row) * kpad], &wt.w[l][(static_cast<size_t>(d) * 512 + src) * in],
                                   in * sizeof(float)) == 0,
                       "pack_layer row");
            }
        expect(bilstm_pack_layer(&wt.layers[l], in, w.data(), w.size() - 1, r.data(), r.size(), b.data(), b.size()) ==
                   BILSTM_BUFFER_LENGTH,
               "pack_layer short buffer");
    }
}

void check_schedule() {
    long calls = 0;
    for (uint32_t batch : {1u, 2u, 3u, 7u, 8u, 31u, 32u, 33u, 64u, 100u, 128u, 255u, 256u, 257u, 520u, 1024u})
        for (uint32_t steps : {1u, 2u, 7u, 16u, 33u, 589u, 4096u})
            for (int cus : {8, 80, 256, 304})
                for (int per_cu : {1, 2, 4})
                    for (int groups : {0, 1, 2, 4})
                        for (int tile : {0, 1, 2, 4})
                            for (int pipeline : {0, 1, 2, 3, 4})
                                for (int slices : {0, 1, 2, 3}) {
                                    bilstm_options o{};
                                    o.recur_groups = groups;
                                    o.recur_tile = tile;
                                    o.concurrent = -1;
                                    o.pipeline = pipeline;
                                    o.slices = slices;
                                    bilstm_plan_info info{};
                                    const bilstm_status st = bilstm_schedule(batch, steps, cus, per_cu, &o, &info);
                                    ++calls;
                                    if (st != BILSTM_OK) continue;
                                    // every launch of a split tile fits the resident capacity
                                    const int per_launch =
                                        (info.recur_tiles + info.recur_launches - 1) / info.recur_launches;
                                    expect(info.recur_groups == 1 ||
                                               static_cast<long>(per_launch) * info.recur_groups <= cus * per_cu,
                                           "schedule capacity");
                                    expect(static_cast<long>(info.recur_tiles) * info.recur_tile >= batch,
                                           "schedule covers the batch");
                                }
    bilstm_plan_info info{};
    expect(bilstm_schedule(0, 5, 256, 1, nullptr, &info) == BILSTM_INVALID_ARGUMENT, "schedule batch 0");
    std::printf("schedule: %ld calls\n", calls);
}

void check_entry_points(const Weights &wt) {
    bilstm_plan *plan = nullptr;
    expect(bilstm_plan_create(0, 2, 3, nullptr, &plan) == BILSTM_INVALID_ARGUMENT && plan == nullptr,
           "plan_create NULL layers");
    expect(bilstm_plan_create(0, 0, 3, wt.layers, &plan) == BILSTM_INVALID_ARGUMENT, "plan_create batch 0");
    bilstm_layer bad[BILSTM_LAYERS];
    std::memcpy(bad, wt.layers, sizeof(bad));
    bad[2].r_len -= 1;
    expect(bilstm_plan_create(0, 2, 3, bad, &plan) == BILSTM_BUFFER_LENGTH, "plan_create short R");
    bilstm_options o{};
    o.near_wrap = 3;
    expect(bilstm_plan_create_ex(0, 2, 3, wt.layers, &o, &plan) != BILSTM_OK, "plan_create bad option");
    expect(bilstm_plan_create(0, 0x10000u, 0x10000u, wt.layers, &plan) == BILSTM_DIMENSION_OVERFLOW,
           "plan_create overflow");
    // a well-formed request: without a gfx950 device it fails cleanly, with one it succeeds
    const bilstm_status st = bilstm_plan_create(0, 2, 3, wt.layers, &plan);
    expect(st == BILSTM_OK || st == BILSTM_UNSUPPORTED || st == BILSTM_HIP_ERROR, "plan_create status");
    bilstm_destroy(plan);
    bilstm_destroy(nullptr);
    float dummy[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
    expect(bilstm_forward(nullptr, dummy, 4, dummy, 4, nullptr) == BILSTM_INVALID_ARGUMENT, "forward NULL plan");
    expect(bilstm_project(nullptr, 0, dummy, 4, dummy, 4, nullptr) == BILSTM_INVALID_ARGUMENT, "project NULL plan");
    expect(bilstm_recur(nullptr, 0, dummy, 4, dummy, 4, nullptr) == BILSTM_INVALID_ARGUMENT, "recur NULL plan");
    expect(bilstm_check(nullptr) == BILSTM_INVALID_ARGUMENT, "check NULL plan");
    expect(bilstm_plan_get_info(nullptr, nullptr) == BILSTM_INVALID_ARGUMENT, "get_info NULL");
    float ms[12];
    expect(bilstm_phase_times(nullptr, ms, 12) == BILSTM_INVALID_ARGUMENT, "phase_times NULL");
    // the entry point that allocates nothing: its argument checks come before any device call
    std::vector<float> x(3 * 5 * 60), y(3 * 5 * 256);
    expect(bilstm_forward_noalloc(0, 3, 5, nullptr, x.data(), x.size(), y.data(), y.size(), nullptr) ==
               BILSTM_INVALID_ARGUMENT,
           "forward_noalloc NULL layers");
    expect(bilstm_forward_noalloc(0, 3, 5, wt.layers, x.data(), x.size() - 1, y.data(), y.size(), nullptr) ==
               BILSTM_BUFFER_LENGTH,
           "forward_noalloc short x");
    expect(bilstm_forward_noalloc(0, 40, 589, wt.layers, x.data(), 40 * 589 * 60, y.data(), 40 * 589 * 256, nullptr) ==
               BILSTM_DIMENSION_OVERFLOW,
           "forward_noalloc beyond its scratch");
    expect(bilstm_forward_noalloc(0, 3, 5, wt.layers, x.data(), x.size(), x.data(), y.size(), nullptr) ==
               BILSTM_INVALID_ARGUMENT,
           "forward_noalloc overlap");
    double ta = 0.0, tb = 0.0;
    expect(bilstm_probe_mfma_rate(0, 2, 0, 10, &ta, &tb) == BILSTM_INVALID_ARGUMENT, "probe_mfma_rate kind");
    expect(bilstm_probe_mfma_rate(0, 0, 0, 10, nullptr, &tb) == BILSTM_INVALID_ARGUMENT, "probe_mfma_rate NULL");
    expect(bilstm_probe_fma_rate(0, 3, 1, 10, &ta, &tb) == BILSTM_INVALID_ARGUMENT, "probe_fma_rate waves");
    bilstm_heads *heads = nullptr;
    expect(bilstm_heads_create(0, nullptr, &heads) == BILSTM_INVALID_ARGUMENT, "heads_create NULL");
    bilstm_heads_destroy(nullptr);
    expect(std::strlen(bilstm_last_error()) > 0, "last_error text");
}

}  // namespace

int main() {
    Weights wt;
    check_packer(wt);
    check_schedule();
    check_entry_points(wt);
    std::printf("host checks: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
