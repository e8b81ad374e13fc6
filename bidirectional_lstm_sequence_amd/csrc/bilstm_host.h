// Host-side helpers shared by the library's C++ sources: error recording, length checks,
// the weight packer and the recurrence schedule.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/bilstm.h"
#include "bilstm_internal.h"

namespace bl {

// Record a formatted message for bilstm_last_error() and return `status`.
bilstm_status fail(bilstm_status status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// A buffer or dimension must hold exactly what the stack needs (speakrs 0.6.0, page
// `lstmproj.rs`, `check_len`).
bilstm_status check_len(const char *context, size_t expected, size_t actual);

// Pack one layer (lengths already checked): W rows into [1024][kpad], R into [2][512][128]
// with rows 4j + g, bias into [1024] = Wb + Rb.
bilstm_status pack_layer(const bilstm_layer &layer, int in, float *w_out, float *r_out, float *bias_out);

// Choose the recurrence split for `batch` windows; fills the recur_* fields, concurrent,
// cu_count and recur_capacity of `info`.
bilstm_status schedule(uint32_t batch, uint32_t steps, int cu_count, int per_cu,
                       const bilstm_options *opt, bilstm_plan_info *info);

// The projection through hipBLASLt (comparator for the hand-written kernel), full batch only.
struct LibraryProjection;
bilstm_status library_projection_create(long rows, const int in[kLayers], const int kpad[kLayers],
                                        float *const bias[kLayers], LibraryProjection **out);
bilstm_status library_projection_run(LibraryProjection *lp, int layer, const float *x, const float *w,
                                     float *gates, hipStream_t stream);
void library_projection_destroy(LibraryProjection *lp);

}  // namespace bl
