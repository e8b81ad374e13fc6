/*
 * Oracle of the four-layer bidirectional LSTM stack: a plain, slow, single-threaded CPU
 * implementation written from the definition.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
 * baseline call it. The HIP library never links, loads or calls it, and it shares no code,
 * header or table with the HIP library.
 *
 * Source of what is computed: the speakrs 0.6.0 page `lstmproj.rs` (module doc,
 * `PackedLayer` doc, `Oxide::enqueue`, `DirectionLaunch` doc) and the `lstm.rs` page
 * (module doc). The pages fix the data flow (a time-parallel projection x·Wᵀ, then a
 * step-serial recurrence per direction; the reverse direction on columns H..2H-1), the
 * tensor shapes (W [2][512][in], R [2][512][128], B with Wb and Rb, bias = Wb + Rb) and
 * that each layer feeds the next. They never write the cell equations, so the cell is the
 * standard LSTM with gate rows in the order i, f, g, o (PyTorch's `nn.LSTM`), zero initial
 * state, sigmoid on i, f, o and tanh on g and on the cell output.
 *
 * Two builds of the same body (lstm_body.inc):
 *   *_f64  double accumulation, activations and inter-layer values: the reference.
 *   *_f32  float throughout: diagnostic, to show the intrinsic fp32 noise floor.
 *
 * The segmentation heads after the stack (the `segdense.rs` page: linear0, linear1 and the
 * classifier with their LeakyReLU and log-softmax epilogues) are in the same body.
 *
 * Pins (tests/test_oracle_pins.py): a hand-derived one-unit closed form, agreement with
 * torch.nn.LSTM in float64, |h| < 1, the R = 0 scan closed form and per-step independence
 * with the forget gate off, and time-reversal symmetry with the directions swapped; for the
 * heads, a hand-derived one-unit case, agreement with torch's linear / leaky_relu /
 * log_softmax in float64, normalisation and shift invariance of the log-softmax.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define REAL double
#define EXPR exp
#define TANHR tanh
#define LOGR log
#define NAME(x) x##_f64
#include "lstm_body.inc"
#undef REAL
#undef EXPR
#undef TANHR
#undef LOGR
#undef NAME

#define REAL float
#define EXPR expf
#define TANHR tanhf
#define LOGR logf
#define NAME(x) x##_f32
#include "lstm_body.inc"
#undef REAL
#undef EXPR
#undef TANHR
#undef LOGR
#undef NAME
