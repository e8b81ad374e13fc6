// The whole stack for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): bilstm_forward_noalloc.
//
// It runs the same kernels as a plan without streamed gates — the FP32-MFMA projection, then
// the single-workgroup recurrence of both directions in one launch, per layer, all on the
// caller's stream — but owns no plan. Everything a plan would allocate lives in `scratch`, one
// file-scope device array of kStaticScratchBytes per device: each call packs the caller's
// device-resident weights into it (gate interleave, bias fold, K padding and the recurrent
// rows' exponent scale, as plan creation does on the host: speakrs 0.6.0, page `lstmproj.rs`,
// `with_recurrence` and `PackedLayer` doc), then uses its tail for the gate pre-activations.
// Every call on a device shares that device's array: two calls that overlap on one device
// race. Each call rewrites every byte it reads, so nothing carries over between calls.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/bilstm.h"
#include "bilstm_host.h"

namespace bl {
namespace {

// Layout of the array: four layers' packed W ([1024][64] for layer 0, [1024][256] after it),
// their packed, scaled R ([2][512][128] each) and folded bias ([1024] each), the watchdog
// words, then the gates [rows][1024] of up to kStaticMaxRows rows.
constexpr size_t kStaticScratchBytes = size_t{96} << 20;
constexpr size_t kW0Floats = static_cast<size_t>(kGateCols) * 64;
constexpr size_t kWnFloats = static_cast<size_t>(kGateCols) * kWidth;
constexpr size_t kRFloats = 2ull * kGates * kHidden;
constexpr size_t kWOffset[kLayers] = {0, kW0Floats, kW0Floats + kWnFloats, kW0Floats + 2 * kWnFloats};
constexpr size_t kROffset = kW0Floats + 3 * kWnFloats;  // in floats
constexpr size_t kBiasOffset = kROffset + kLayers * kRFloats;
constexpr size_t kErrOffset = kBiasOffset + kLayers * static_cast<size_t>(kGateCols);
constexpr size_t kGatesOffset = (kErrOffset + kErrWords + 63) / 64 * 64;  // 256-byte aligned
constexpr size_t kStaticMaxRows =
    (kStaticScratchBytes - kGatesOffset * sizeof(float)) / (static_cast<size_t>(kGateCols) * sizeof(float));
static_assert(kGatesOffset * sizeof(float) < kStaticScratchBytes, "scratch too small for the weights");

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

// What the first call on a device sets up, with that device current.
struct DeviceState {
    bool ready = false;
    bilstm_status status = BILSTM_OK;
    char message[256] = {0};
    float *base = nullptr;  // the device address of `scratch` on this device
    int cu_count = 0;
    int per_cu[3] = {0, 0, 0};  // resident single-workgroup recurrence workgroups per CU, tile 1, 2, 4
    unsigned long long timeout_ticks = 0;
};
std::mutex g_mutex;
DeviceState g_state[kMaxDevices];

struct PackSources {
    const float *w[kLayers];
    const float *r[kLayers];
    const float *b[kLayers];
};

// One element of the packed weights per thread (grid-stride): W row d·512 + 4j + g holds
// source row g·128 + j of direction d, zero past the input width; R row 4j + g likewise,
// multiplied by gate g's exponent factor; bias = Wb + Rb, one fp32 addition. The same
// arithmetic as the host packer, so a plan and this entry point hold the same bits.
__global__ __launch_bounds__(256) void pack_weights_kernel(PackSources src, float *base) {
    constexpr size_t kWTotal = kROffset;
    constexpr size_t kRTotal = kLayers * kRFloats;
    constexpr size_t kBTotal = kLayers * static_cast<size_t>(kGateCols);
    constexpr size_t kTotal = kWTotal + kRTotal + kBTotal + kErrWords;
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < kTotal;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        if (i < kWTotal) {
            const int l = i < kW0Floats ? 0 : 1 + static_cast<int>((i - kW0Floats) / kWnFloats);
            const int in = l == 0 ? kFeatures : kWidth;
            const int kpad = l == 0 ? 64 : kWidth;
            const size_t e = i - kWOffset[l];
            const int row = static_cast<int>(e / kpad), k = static_cast<int>(e % kpad);
            const int d = row / kGates, j = (row % kGates) / 4, g = row % 4;
            base[i] = k < in ? src.w[l][(static_cast<size_t>(d) * kGates + g * kHidden + j) * in + k] : 0.0f;
        } else if (i < kWTotal + kRTotal) {
            const size_t e = i - kWTotal;
            const int l = static_cast<int>(e / kRFloats);
            const size_t el = e % kRFloats;
            const int row = static_cast<int>(el / kHidden), k = static_cast<int>(el % kHidden);
            const int d = row / kGates, j = (row % kGates) / 4, g = row % 4;
            base[i] = src.r[l][(static_cast<size_t>(d) * kGates + g * kHidden + j) * kHidden + k] * gate_exp_scale(g);
        } else if (i < kWTotal + kRTotal + kBTotal) {
            const size_t e = i - kWTotal - kRTotal;
            const int l = static_cast<int>(e / kGateCols), n = static_cast<int>(e % kGateCols);
            const int d = n / kGates, j = (n % kGates) / 4, g = n % 4;
            const float *b = src.b[l] + static_cast<size_t>(d) * 2 * kGates;
            base[i] = b[g * kHidden + j] + b[kGates + g * kHidden + j];
        } else {
            reinterpret_cast<unsigned int *>(base)[i] = 0u;  // watchdog words
        }
    }
}

bilstm_status setup_device(int device, DeviceState &st) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return fail(BILSTM_HIP_ERROR, "forward_noalloc: device properties: %s", hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        return fail(BILSTM_UNSUPPORTED, "forward_noalloc: device %d is not a gfx950 (MI355X) GPU", device);
    }
    // the device address of this device's copy of the array (the name itself is a host-side
    // stand-in and must never reach a kernel)
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
        return fail(BILSTM_HIP_ERROR, "forward_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    }
    int wall_khz = 0;
    e = hipDeviceGetAttribute(&st.cu_count, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, device);
    for (int t = 0; t < 3 && e == hipSuccess; ++t) e = recurrence_occupancy(1, 1 << t, &st.per_cu[t]);
    if (e != hipSuccess) return fail(BILSTM_HIP_ERROR, "forward_noalloc: device attributes: %s", hipGetErrorString(e));
    st.base = static_cast<float *>(ptr);
    st.timeout_ticks = static_cast<unsigned long long>(2000.0 * wall_khz);
    return BILSTM_OK;
}

bool aligned(const void *p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

}  // namespace
}  // namespace bl

using namespace bl;

extern "C" bilstm_status bilstm_forward_noalloc(int device, uint32_t batch, uint32_t steps,
                                                const bilstm_layer layers[BILSTM_LAYERS], const float *x,
                                                size_t x_len, float *y, size_t y_len, void *stream_ptr) {
    if (layers == nullptr || x == nullptr || y == nullptr) {
        return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: NULL argument");
    }
    if (device < 0 || device >= kMaxDevices) {
        return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: device %d out of range", device);
    }
    if (batch == 0 || steps == 0) {
        return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: batch (%u) and steps (%u) must be >= 1", batch, steps);
    }
    const uint64_t rows = static_cast<uint64_t>(batch) * steps;
    if (rows > kStaticMaxRows) {
        return fail(BILSTM_DIMENSION_OVERFLOW,
                    "forward_noalloc: batch*steps = %llu rows exceed the static scratch's %zu rows (%zu MiB per "
                    "device); use a plan (bilstm_plan_create) for larger batches",
                    static_cast<unsigned long long>(rows), kStaticMaxRows, kStaticScratchBytes >> 20);
    }
    bilstm_status s;
    if ((s = check_len("forward_noalloc input", rows * kFeatures, x_len)) != BILSTM_OK) return s;
    if ((s = check_len("forward_noalloc output", rows * kWidth, y_len)) != BILSTM_OK) return s;
    if (!aligned(x, 16) || !aligned(y, 16)) {
        return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: x and y must be 16-byte aligned");
    }
    const auto xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
    if (xa < ya + y_len * sizeof(float) && ya < xa + x_len * sizeof(float)) {
        return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: input and output overlap");
    }
    PackSources src{};
    for (int l = 0; l < kLayers; ++l) {
        const bilstm_layer &L = layers[l];
        const size_t in = l == 0 ? kFeatures : kWidth;
        if (L.w == nullptr || L.r == nullptr || L.b == nullptr || !aligned(L.w, 4) || !aligned(L.r, 4) ||
            !aligned(L.b, 4)) {
            return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: layer %d has a NULL or misaligned weight pointer", l);
        }
        char ctx[64];
        std::snprintf(ctx, sizeof(ctx), "forward_noalloc layer %d W", l);
        if ((s = check_len(ctx, 2 * kGates * in, L.w_len)) != BILSTM_OK) return s;
        std::snprintf(ctx, sizeof(ctx), "forward_noalloc layer %d R", l);
        if ((s = check_len(ctx, 2ull * kGates * kHidden, L.r_len)) != BILSTM_OK) return s;
        std::snprintf(ctx, sizeof(ctx), "forward_noalloc layer %d B", l);
        if ((s = check_len(ctx, 4ull * kGates, L.b_len)) != BILSTM_OK) return s;
        src.w[l] = L.w;
        src.r[l] = L.r;
        src.b[l] = L.b;
    }

    int saved = 0;
    const bool restore = hipGetDevice(&saved) == hipSuccess;
    if (hipSetDevice(device) != hipSuccess) return fail(BILSTM_INVALID_ARGUMENT, "forward_noalloc: no device %d", device);
    struct Restore {
        bool on;
        int dev;
        ~Restore() {
            if (on) (void)hipSetDevice(dev);
        }
    } restore_device{restore, saved};

    DeviceState st;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        DeviceState &ds = g_state[device];
        if (!ds.ready) {
            ds.status = setup_device(device, ds);
            if (ds.status != BILSTM_OK) std::snprintf(ds.message, sizeof(ds.message), "%s", bilstm_last_error());
            ds.ready = true;
        }
        st = ds;
    }
    if (st.status != BILSTM_OK) return fail(st.status, "%s", st.message);

    // The schedule a plan without streamed gates or slices would choose.
    bilstm_options opt{};
    opt.recur_groups = 1;
    opt.concurrent = -1;
    opt.slices = 1;
    opt.pipeline = 1;
    bilstm_plan_info info{};
    if ((s = schedule(batch, steps, st.cu_count, 1, &opt, &info)) != BILSTM_OK) return s;
    const int per_cu = st.per_cu[info.recur_tile == 1 ? 0 : info.recur_tile == 2 ? 1 : 2];
    opt.recur_tile = info.recur_tile;
    if ((s = schedule(batch, steps, st.cu_count, per_cu > 0 ? per_cu : 1, &opt, &info)) != BILSTM_OK) return s;

    auto stream = static_cast<hipStream_t>(stream_ptr);
    float *const base = st.base;
    float *const gates = base + kGatesOffset;
    unsigned int *const error = reinterpret_cast<unsigned int *>(base + kErrOffset);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(2048), dim3(256), 0, stream, src, base);
    hipError_t e = hipGetLastError();
    for (int l = 0; l < kLayers && e == hipSuccess; ++l) {
        ProjArgs pa{};
        pa.x = l == 0 ? x : y;
        pa.w = base + kWOffset[l];
        pa.bias = base + kBiasOffset + static_cast<size_t>(l) * kGateCols;
        pa.gates = gates;
        pa.rows = static_cast<int>(rows);
        pa.in = l == 0 ? kFeatures : kWidth;
        pa.kpad = l == 0 ? 64 : kWidth;
        pa.row_tiles = static_cast<int>((rows + kProjTileM - 1) / kProjTileM);
        pa.tiles = pa.row_tiles * (kGateCols / kProjTileN);
        pa.error = error;
        pa.timeout_ticks = st.timeout_ticks;
        e = launch_projection(pa, st.cu_count, stream);
        if (e != hipSuccess) break;
        RecurArgs ra{};
        ra.gates = gates;
        ra.r = base + kROffset + static_cast<size_t>(l) * kRFloats;
        ra.y = y;
        ra.error = error;
        ra.batch = static_cast<int>(batch);
        ra.steps = static_cast<int>(steps);
        ra.tiles = info.recur_tiles;
        ra.timeout_ticks = st.timeout_ticks;
        const int per_launch = (info.recur_tiles + info.recur_launches - 1) / info.recur_launches;
        for (int direction = 0; direction < 2 && e == hipSuccess; direction += info.concurrent == 2 ? 2 : 1) {
            for (int first = 0; first < info.recur_tiles && e == hipSuccess; first += per_launch) {
                RecurArgs a = ra;
                a.direction = direction;
                a.tile_first = first;
                a.tile_count = std::min(per_launch, info.recur_tiles - first);
                e = launch_recurrence(1, info.recur_tile, a, info.concurrent == 2 ? 2 : 1, 0, stream);
            }
        }
    }
    if (e != hipSuccess) return fail(BILSTM_HIP_ERROR, "forward_noalloc: launch: %s", hipGetErrorString(e));
    return BILSTM_OK;
}
