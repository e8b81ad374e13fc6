/*
 * bilstm.h — C ABI of the MI355X (gfx950) four-layer bidirectional LSTM stack.
 *
 * The stack is the one of the speakrs 0.6.0 segmentation model (page `lstmproj.rs`,
 * module doc and `PackedLayer` doc): hidden size H = 128, 4H = 512 gate rows per direction,
 * input width 60 in the first layer and 256 (forward and reverse hidden states side by
 * side) in the others, four layers, fp32 throughout. Per layer it runs a time-parallel input
 * projection x·Wᵀ + (Wb + Rb) for every step of both directions, then a step-serial
 * recurrence per direction with the recurrent matrix held on chip, the reverse direction
 * concurrently with the forward one; the next layer waits for both.
 *
 * Cell (the pages give the data flow, not the equations; this is the standard LSTM cell
 * with PyTorch's gate order): a = x_t·Wᵀ + Wb + Rb + R·h_{t-1}, rows in blocks i, f, g, o;
 * i, f, o = σ(a), g = tanh(a); c_t = f c_{t-1} + i g; h_t = o tanh(c_t); h_0 = c_0 = 0.
 * Direction 0 runs t = 0..T-1 and writes output columns 0..127; direction 1 runs
 * t = T-1..0 and writes columns 128..255 (page `lstmproj.rs`, `DirectionLaunch` doc).
 *
 * Conventions shared by every entry point
 *  - No C++ types cross this boundary. Device buffers are plain pointers to device memory
 *    of the plan's device; host buffers are plain host pointers. Lengths are element counts
 *    and are checked exactly (page `lstmproj.rs`, `check_len`): a mismatch returns
 *    BILSTM_BUFFER_LENGTH; a size that does not fit the kernels' 32-bit indices returns
 *    BILSTM_DIMENSION_OVERFLOW (page `lstmproj.rs`, `to_u32`).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Device work is
 *    enqueued asynchronously on it; the plan's own side stream is joined back into it
 *    before the call returns, so the caller's stream order covers all of the plan's work.
 *  - On failure every call returns a nonzero bilstm_status and records a message for
 *    bilstm_last_error(). Nothing is enqueued when validation fails.
 *  - A plan serves one batch size and one sequence length (page `lstmproj.rs`, `Oxide`
 *    doc). It owns its scratch (gate buffer, exchange words), so two calls on the same
 *    plan must not run concurrently; calls on different plans may.
 */
#ifndef BILSTM_H
#define BILSTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BILSTM_HIDDEN 128   /* H */
#define BILSTM_GATES 512    /* 4H gate rows per direction */
#define BILSTM_FEATURES 60  /* input width of the first layer */
#define BILSTM_WIDTH 256    /* 2H: output width of every layer, input width of layers 1..3 */
#define BILSTM_LAYERS 4

typedef struct bilstm_plan bilstm_plan; /* opaque; created and owned by the library */

typedef enum {
    BILSTM_OK = 0,
    BILSTM_INVALID_ARGUMENT = 1,   /* NULL pointer, bad layer index, misaligned buffer ... */
    BILSTM_BUFFER_LENGTH = 2,      /* a length differs from the one the plan needs */
    BILSTM_DIMENSION_OVERFLOW = 3, /* a size exceeds the kernels' 32-bit indexing */
    BILSTM_UNSUPPORTED = 4,        /* not a gfx950 device, or an option this build lacks */
    BILSTM_HIP_ERROR = 5,          /* a HIP runtime call failed (message has the HIP error) */
    BILSTM_TIMEOUT = 6             /* a recurrence wait hit its watchdog (see bilstm_check) */
} bilstm_status;

/*
 * One layer's weights, HOST pointers, PyTorch nn.LSTM layout (page `lstmproj.rs`,
 * `with_recurrence`: W is 2·512·in, R is 2·512·128, B is 4·512):
 *   w [2][512][in]   direction 0 = forward (weight_ih_l{k}), 1 = reverse (weight_ih_l{k}_reverse),
 *                    rows in blocks of 128: i, f, g, o; in = 60 for layer 0, else 256
 *   r [2][512][128]  weight_hh
 *   b [2][2][512]    per direction: Wb (bias_ih) then Rb (bias_hh)
 * The library copies and repacks them at plan creation; the caller keeps ownership.
 */
typedef struct {
    const float *w;
    size_t w_len;
    const float *r;
    size_t r_len;
    const float *b;
    size_t b_len;
} bilstm_layer;

/*
 * Plan options (page `lstmproj.rs`, `with_recurrence`: an explicit recurrence plan, so
 * different kernels can run the same batch). Zero / -1 fields mean "the plan's choice".
 */
typedef struct {
    int32_t recur_groups; /* workgroups per (direction, window tile): 1, 2 or 4; 0 = auto */
    int32_t recur_tile;   /* windows per tile: 1, 2 or 4; 0 = auto */
    int32_t concurrent;   /* directions: -1 auto (2 when both grids fit together, else 0),
                             0 serially on the caller's stream, 1 reverse on the
                             plan's side stream joined back by events, 2 both directions in one
                             launch on the caller's stream */
    int32_t watchdog_us;  /* bound of one recurrence wait in microseconds; 0 = 2 s; -1 =
                             forced timeout for failure-handling tests: every exchange wait
                             expects a flag no producer writes and gives up on its first poll.
                             A wait that hits its bound sets the plan's error flag
                             (bilstm_check) and stops waiting; the kernels still finish */
    int32_t slices;       /* batch slices for bilstm_forward: the windows are cut into this many
                             contiguous slices, each run as its own chain of layers on its own
                             stream, so one slice's projection overlaps other slices'
                             recurrences on the CUs the recurrence leaves idle. Windows are
                             independent, so the output does not depend on it (bitwise).
                             0 = auto (2 when the recurrence leaves at least half of the CUs
                             idle, else 1), 1 = off, at most 8 (beyond the process's hardware
                             queues, 4 by default, streams share queues and run one after
                             another); needs recur_groups = 1, concurrent != 1 and the
                             library's own projection (projection != 1) */
    int32_t projection;   /* input projection:
                             0 = the plan's rule (default; speakrs 0.6.0, page `lstmproj.rs`,
                                 `projection_rule`): 3 where the split is accurate on this device
                                 (development checks: within 1.1x the FP32 kernel's largest error
                                 against an fp64 reference on every workload measured), at least
                                 2048 projection rows amortize it and the projection is on the
                                 forward's critical path (unstreamed, or streamed with more work per
                                 recurrence step than the FP32 kernel keeps up with on the CUs the
                                 recurrence leaves); else 4. A function of batch, steps and the
                                 device only, so every plan for one workload computes the same gates;
                             1 = the vendor GEMM (hipBLASLt, FP32 compute, bias epilogue) as a
                                 comparator, run unsliced and unstreamed;
                             2 = the own kernel in split precision, two bf16 parts per FP32
                                 operand, three bf16 MFMA products per K chunk (a0·b0 + a0·b1 +
                                 a1·b0) accumulated in FP32:
                                 |error| <= (3·2^-16·(1 + 2^-7) + (3K + 2)·2^-24)·sum|x·w| per gate;
                             3 = three bf16 parts, six products (every ap·bq with p + q <= 2):
                                 |error| <= (4·2^-24·(1 + 2^-7) + (6K + 2)·2^-24)·sum|x·w| per gate,
                                 the truncation of the order of one FP32 rounding per product;
                             4 = the own kernel's FP32 MFMA products:
                                 |error| <= (K + 2)·2^-24·sum|x·w| per gate */
    int32_t pipeline;     /* streamed gates for bilstm_forward: each layer's projection runs beside
                             that layer's recurrence on the CUs the recurrence leaves free, computes
                             the gates in the order the recurrence reads them (chunks of steps,
                             per direction) and publishes each chunk through a counter the
                             recurrence polls; the next layer's projection can start while this
                             layer's recurrence still runs, reading the rows it has published.
                             Gates alternate between two plan-owned buffers and layer outputs
                             between y and a plan-owned buffer, so no kernel overwrites data a
                             running one still reads. The output is bitwise the same as without
                             it.
                             0 = auto (on when recur_groups = 1, concurrent = 2, the
                             recurrence's grid leaves at least half of the CUs free and the
                             projection is the library's own), 1 = off,
                             2 = on (BILSTM_UNSUPPORTED unless recur_groups = 1, projection != 1,
                             slices <= 1 and at least 8 CUs stay free), with the next layer's
                             projection starting during this layer's recurrence; 3 = on, with it
                             starting after this layer's recurrence; 4 = as 2, with the four
                             layers' recurrences as one launch where possible
                             (bilstm_plan_info.stream_fused), not a launch per layer; 5 = as 3,
                             and each layer's recurrence also starts only after that layer's
                             projection has finished: the same streamed kernels run one at a
                             time (for profilers that serialize kernels, e.g. counter
                             collection), none of them ever waiting for another.
                             Every wait on a counter is bounded by the watchdog like every other
                             wait: if the GPU is shared with other work that keeps a kernel from
                             running, bilstm_check reports BILSTM_TIMEOUT instead of hanging */
    int32_t near_wrap;    /* test hook for the clear paths: 1 = the flag epoch of the exchange
                             words and the pass numbers of the streamed gates' counters and
                             progress words start just below the values at which the plan clears
                             those words and starts again from zero (the counters are filled to
                             match), so the first forward runs with flags and counts near the top
                             of their range and the second one runs the clears (speakrs 0.6.0,
                             page `lstmproj.rs`, `clear_state`). 0 = off */
} bilstm_options;

/* What a plan chose; filled by bilstm_plan_get_info. */
typedef struct {
    uint32_t batch;
    uint32_t steps;
    int32_t recur_groups;    /* workgroups per (direction, tile) */
    int32_t recur_tile;      /* windows per tile */
    int32_t recur_tiles;     /* number of window tiles */
    int32_t recur_threads;   /* threads per recurrence workgroup */
    int32_t recur_launches;  /* launches per direction per layer */
    int32_t concurrent;      /* 0 serial, 1 side stream, 2 one launch for both directions */
    int32_t proj_tile_m;     /* projection output tile, rows */
    int32_t proj_tile_n;     /* projection output tile, gate columns */
    int32_t cu_count;        /* compute units of the device */
    int32_t recur_capacity;  /* recurrence workgroups the device keeps resident at once */
    uint64_t device_bytes;   /* device memory the plan owns */
    int32_t slices;          /* batch slices bilstm_forward runs as concurrent chains */
    int32_t slice_windows;   /* windows per slice (the last slice may hold fewer) */
    int32_t projection;      /* the projection the plan runs (never 0): 1 vendor GEMM, 2 and 3 own
                                split-precision kernel with two or three bf16 parts, 4 own FP32 MFMA */
    int32_t pipeline;        /* 1 when bilstm_forward streams the gates (see bilstm_options) */
    int32_t stream_chunk;    /* streamed gates: recurrence steps per published chunk (128 /
                                windows per projection row block); 0 when not streamed */
    int32_t stream_overlap;  /* streamed gates: 1 when the next layer's projection starts during
                                this layer's recurrence, 0 when after it */
    int32_t stream_split;    /* streamed gates: tiles per 128 gate columns of each layer's first
                                chunk (1, 2 or 4), the chunk a layer boundary waits for: narrower
                                tiles spread it over more workgroups; 0 when not streamed */
    int32_t stream_fused;    /* streamed gates: 1 when the four layers' recurrences run as one
                                launch (pipeline = 4, concurrent = 2, recur_launches = 1); each
                                workgroup then moves from a layer to the next by itself */
    int32_t stream_serial;   /* streamed gates: 1 when pipeline = 5 (kernels one at a time) */
    uint32_t clears;         /* times the plan has cleared its exchange words or its streamed
                                counters and progress words since creation (before the 32-bit flag
                                or pass space would wrap, or after a failed enqueue) */
} bilstm_plan_info;

/*
 * Create a plan for `batch` windows of `steps` frames on HIP device `device`, packing the
 * four layers' weights (page `lstmproj.rs`, `with_recurrence`: gate rows permuted so rows
 * 4j..4j+3 hold hidden unit j's i, f, g, o; bias folded to Wb + Rb).
 * Returns BILSTM_UNSUPPORTED on a device other than gfx950. *out receives the plan.
 * batch and steps must be >= 1; batch·steps·256 must fit 32 bits.
 */
bilstm_status bilstm_plan_create(int device, uint32_t batch, uint32_t steps,
                                 const bilstm_layer layers[BILSTM_LAYERS], bilstm_plan **out);

/* As bilstm_plan_create, with explicit options (NULL = defaults). */
bilstm_status bilstm_plan_create_ex(int device, uint32_t batch, uint32_t steps,
                                    const bilstm_layer layers[BILSTM_LAYERS],
                                    const bilstm_options *options, bilstm_plan **out);

/*
 * The whole stack (page `lstmproj.rs`, `Oxide::enqueue`).
 *   x [batch][steps][60]  device, fp32, 16-byte aligned; read only; x_len = batch·steps·60
 *   y [batch][steps][256] device, fp32, 16-byte aligned; y_len = batch·steps·256
 * y doubles as the inter-layer buffer. Without streamed gates it is updated in place layer by
 * layer: a layer's projection has consumed all of the previous layer's output by the time its
 * recurrence starts writing (page `lstmproj.rs`, module doc). With streamed gates
 * (bilstm_options.pipeline) a layer's projection still reads while its recurrence writes, so
 * layers 0 and 2 write a plan-owned buffer and layers 1 and 3 write y.
 * x and y must not overlap. Asynchronous on `stream`.
 */
bilstm_status bilstm_forward(bilstm_plan *plan, const float *x, size_t x_len, float *y,
                             size_t y_len, void *stream);

/*
 * One layer's input projection alone (page `lstmproj.rs`, `InputProjection::enqueue`),
 * into a caller buffer in the plan's gate layout:
 *   x     [batch·steps][in]   device; in = 60 for layer 0, else 256
 *   gates [batch·steps][1024] device; column d·512 + 4j + g holds direction d, hidden unit j,
 *         gate g (0 i, 1 f, 2 g, 3 o), bias Wb + Rb included.
 */
bilstm_status bilstm_project(bilstm_plan *plan, int layer, const float *x, size_t x_len,
                             float *gates, size_t gates_len, void *stream);

/*
 * One layer's recurrence alone, both directions (page `lstmproj.rs`, `Oxide::recur`),
 * from gate pre-activations in the layout bilstm_project writes, into
 *   y [batch][steps][256] device.
 */
bilstm_status bilstm_recur(bilstm_plan *plan, int layer, const float *gates, size_t gates_len,
                           float *y, size_t y_len, void *stream);

/* Fill *info with the plan's choices. */
bilstm_status bilstm_plan_get_info(const bilstm_plan *plan, bilstm_plan_info *info);

/*
 * Wait until the work of the plan's last call (bilstm_forward, bilstm_project or bilstm_recur)
 * has finished — an event the call recorded on its stream, so work of other streams is not
 * waited for — and report whether a wait of any earlier call hit its watchdog
 * (BILSTM_TIMEOUT: the outputs of the call that timed out are invalid). Clears the report.
 * Blocks the calling thread.
 *
 * The kernels write a timeout report into host-mapped memory, so it reaches the caller
 * without this call as well: bilstm_forward, bilstm_project and bilstm_recur first look at it
 * and, if a wait of an earlier call on the plan has timed out and finished, clear the report
 * and return BILSTM_TIMEOUT without enqueueing anything (the next call runs normally).
 */
bilstm_status bilstm_check(bilstm_plan *plan);

/*
 * Per-phase timing (page `lstmproj.rs`: the `LstmPhases` hooks around the projection and
 * the recurrence of each layer). When enabled, bilstm_forward records HIP events on
 * `stream` around each phase. bilstm_phase_times then waits for the last forward and
 * writes 12 values in milliseconds: projection of layers 0..3; recurrence phase of layers
 * 0..3 (both directions, including any join); duration of the first recurrence launch on the
 * caller's stream of layers 0..3 (the launch running both directions when they share one
 * launch, else the forward direction's). n must be >= 12. With streamed gates the phases of a
 * layer and of its neighbours overlap: the first 8 values are then the time from the forward's
 * start to the end of each projection and of each recurrence. When the four recurrences run
 * as one launch (bilstm_plan_info.stream_fused), that launch is timed by its own event pair
 * and split into layers by wall-clock stamps the kernel records (each layer's latest end over
 * the workgroups): the last 4 values are then each layer's share of the launch (from the
 * previous layer's end, or the launch's start) and sum to its duration.
 */
bilstm_status bilstm_set_phase_events(bilstm_plan *plan, int enable);
bilstm_status bilstm_phase_times(bilstm_plan *plan, float *ms, size_t n);

/* Release everything the plan owns. Waits for its work first. NULL is a no-op. */
void bilstm_destroy(bilstm_plan *plan);

/* Text of the last error recorded on the calling thread ("" if none). */
const char *bilstm_last_error(void);

/* ---- the stack without a plan, for callers that cannot allocate ------------------- */

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The whole stack, as bilstm_forward computes it, with
 * no plan: this call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   layers  the four layers' weights as DEVICE pointers on `device` (same layout and lengths as
 *           bilstm_layer; read only, 4-byte aligned)
 *   x       [batch][steps][60]  device, fp32, 16-byte aligned; x_len = batch·steps·60
 *   y       [batch][steps][256] device, fp32, 16-byte aligned; y_len = batch·steps·256; also the
 *           inter-layer buffer (updated in place layer by layer); must not overlap x
 * Its scratch — the packed weights (repacked from `layers` by every call) and the gate
 * pre-activations — is one static device array of 96 MiB per device, taken by the first call
 * on that device and held until the process ends, so batch·steps is limited to 23,227 rows
 * (e.g. 39 windows of 589 frames); larger calls return BILSTM_DIMENSION_OVERFLOW. Calls that
 * overlap on one device race on that array (serialize them, e.g. on one stream); calls on
 * different devices do not. Runs the projection and the single-workgroup recurrence on
 * `stream`, both directions per layer in one launch, with FP32 projection products: the output
 * is bitwise the same as a plan's bilstm_forward for the same inputs wherever the plan computes
 * its projection with FP32 products (bilstm_options.projection = 4, or the plan's rule where it
 * chooses them: every workload of up to 48 windows of 589 frames).
 */
bilstm_status bilstm_forward_noalloc(int device, uint32_t batch, uint32_t steps,
                                     const bilstm_layer layers[BILSTM_LAYERS], const float *x, size_t x_len,
                                     float *y, size_t y_len, void *stream);

/* ---- segmentation heads after the stack ------------------------------------------- */

/*
 * The segmentation model's dense heads that consume the stack's output (speakrs 0.6.0, page
 * `segdense.rs`, `Site` doc and `dimensions()`), fused into one kernel:
 *   h0  = LeakyReLU(y · W0 + b0)      W0 [256][128]  row-major [k][n], as the page's layout
 *   h1  = LeakyReLU(h0 · W1 + b1)     W1 [128][128]
 *   out = log_softmax(h1 · W2 + b2)   W2 [128][7], over each row's 7 classes
 * The page gives no LeakyReLU slope; the caller passes it (PyTorch's default is 0.01).
 * All pointers HOST, float32; the library copies and repacks them.
 */
typedef struct bilstm_heads bilstm_heads; /* opaque; created and owned by the library */

typedef struct {
    const float *w0;
    size_t w0_len; /* 256·128 */
    const float *b0;
    size_t b0_len; /* 128 */
    const float *w1;
    size_t w1_len; /* 128·128 */
    const float *b1;
    size_t b1_len; /* 128 */
    const float *w2;
    size_t w2_len; /* 128·7 */
    const float *b2;
    size_t b2_len; /* 7 */
    float slope;   /* LeakyReLU negative slope */
} bilstm_head_weights;

/* Pack the heads' weights onto HIP device `device` (gfx950 only; BILSTM_UNSUPPORTED else). */
bilstm_status bilstm_heads_create(int device, const bilstm_head_weights *weights, bilstm_heads **out);

/*
 * The heads over every row of the stack's output:
 *   y   [rows][256] device, fp32, 16-byte aligned; y_len = rows·256 (any rows >= 0; with
 *                   rows = 0 the call does nothing and the pointers may be NULL)
 *   out [rows][7]   device, fp32: log-probabilities; out_len = rows·7
 * Asynchronous on `stream`; y and out must not overlap. A call may run concurrently with
 * other calls on the same heads object (it owns no scratch).
 */
bilstm_status bilstm_heads_forward(bilstm_heads *heads, const float *y, size_t y_len, float *out,
                                   size_t out_len, void *stream);

/* Release the heads' device memory (waits for the device first). NULL is a no-op. */
void bilstm_heads_destroy(bilstm_heads *heads);

/* ---- host-only helpers: no GPU call, usable without a device ---------------------- */

/*
 * The weight packer alone (page `lstmproj.rs`, `with_recurrence`: pack_input_directions,
 * pack_directions, pack_bias), host to host:
 *   w_out    [1024][kpad]      row d·512 + 4j + g = w[d][g·128 + j][0..in), zero padded
 *                              to kpad = in rounded up to a multiple of 32
 *   r_out    [2][512][128]     row 4j + g of direction d = r[d][g·128 + j]
 *   bias_out [1024]            bias_out[d·512 + 4j + g] = Wb[d][g·128+j] + Rb[d][g·128+j] (fp32)
 * Returns BILSTM_BUFFER_LENGTH if a length is wrong (w_out_len must be 1024·kpad).
 */
bilstm_status bilstm_pack_layer(const bilstm_layer *layer, uint32_t in, float *w_out,
                                size_t w_out_len, float *r_out, size_t r_out_len,
                                float *bias_out, size_t bias_out_len);

/*
 * The recurrence schedule for `batch` windows on a device with `cu_count` compute units
 * whose recurrence kernel keeps `per_cu` workgroups resident per CU (page `lstmproj.rs`,
 * `RecurrencePlan` and its `Schedule`): fills `info` fields recur_* and concurrent.
 * `options` may be NULL. Every launch's grid fits the resident capacity when workgroups
 * of a tile wait for each other (recur_groups > 1).
 */
bilstm_status bilstm_schedule(uint32_t batch, uint32_t steps, int32_t cu_count, int32_t per_cu,
                              const bilstm_options *options, bilstm_plan_info *info);

/* ---- measurement ------------------------------------------------------------------- */

/*
 * Exchange latency probe: two workgroups pass a flagged 64-bit word back and forth
 * `round_trips` times through global memory, the same kind of word the recurrence's
 * hidden-state exchange uses. same_xcd = 1 places both on one XCD, 0 on two XCDs.
 * Both sides use agent-scope relaxed 64-bit atomics, as the recurrence does: on gfx950 these
 * are the accesses that make one CU's store visible to another CU's load.
 * Writes the mean one-way latency in nanoseconds and the XCD id each side ran on.
 */
bilstm_status bilstm_probe_exchange(int device, int same_xcd, int32_t round_trips,
                                    double *one_way_ns, int32_t *xcd_a, int32_t *xcd_b);

/*
 * FMA issue-rate probe, the rate the recurrence's on-chip bound rests on: one or `workgroups`
 * workgroups of 256·waves_per_simd threads (waves_per_simd = 1, 2 or 4 waves on each of a CU's
 * four SIMDs) each run `iterations` rounds of 128 FP32 FMAs over 8 independent accumulators per
 * lane, the shape of the recurrence's product loop. Writes the median workgroup's shader clocks
 * per wave64 FMA per SIMD and its shader clock in GHz (shader clocks over wall-clock time).
 */
bilstm_status bilstm_probe_fma_rate(int device, int waves_per_simd, int32_t workgroups, int32_t iterations,
                                    double *clocks_per_fma, double *ghz);

/*
 * Matrix-core rate probe, the rate the projection's peak rests on: two 256-thread workgroups
 * per CU, every wave running `iterations` rounds of 16 MFMAs over four independent 32x32
 * accumulators with its operands in registers. kind 0: v_mfma_f32_32x32x16_bf16 (the split
 * projection's instruction); 1: v_mfma_f32_32x32x2f32 (the FP32 projection's). data 0: zero
 * operands, 1: ones, 2: uniform in [-1, 1) (a fixed sequence): the matrix pipes run slower on
 * random operands. Writes the rate in TFLOP/s and the timed launch's milliseconds. Allocates
 * and frees a few kilobytes of device memory; synchronizes the device.
 */
bilstm_status bilstm_probe_mfma_rate(int device, int kind, int data, int32_t iterations, double *tflops, double *ms);

#ifdef __cplusplus
}
#endif

#endif /* BILSTM_H */
