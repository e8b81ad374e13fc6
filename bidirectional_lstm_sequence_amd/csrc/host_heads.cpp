// C ABI of the segmentation heads after the stack (speakrs 0.6.0, page `segdense.rs`, `Site`
// doc and `dimensions()`: linear0, linear1 and the classifier with their epilogues): weight
// packing at creation, one fused launch per call.
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "../../include/bilstm.h"
#include "bilstm_host.h"

using namespace bl;

struct bilstm_heads {
    int device = 0;
    float slope = 0.0f;
    float *w0t = nullptr;
    float *b0 = nullptr;
    float *w1t = nullptr;
    float *b1 = nullptr;
    float *w2t = nullptr;
    float *b2 = nullptr;
};

namespace {

void release_heads(bilstm_heads *h) {
    if (h == nullptr) return;
    int saved = 0;
    const bool have = hipGetDevice(&saved) == hipSuccess;
    (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    for (float *p : {h->w0t, h->b0, h->w1t, h->b1, h->w2t, h->b2}) {
        if (p) (void)hipFree(p);
    }
    if (have) (void)hipSetDevice(saved);
    delete h;
}

bool gfx950(int device) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return false;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

// [k][n] row-major -> [n_slots][k], slots past n zero
std::vector<float> transpose(const float *w, int k, int n, int n_slots) {
    std::vector<float> t(static_cast<size_t>(n_slots) * k, 0.0f);
    for (int kk = 0; kk < k; ++kk) {
        for (int nn = 0; nn < n; ++nn) t[static_cast<size_t>(nn) * k + kk] = w[static_cast<size_t>(kk) * n + nn];
    }
    return t;
}

}  // namespace

extern "C" {

bilstm_status bilstm_heads_create(int device, const bilstm_head_weights *w, bilstm_heads **out) {
    if (out == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "heads_create: out is NULL");
    *out = nullptr;
    if (w == nullptr || w->w0 == nullptr || w->b0 == nullptr || w->w1 == nullptr || w->b1 == nullptr ||
        w->w2 == nullptr || w->b2 == nullptr) {
        return fail(BILSTM_INVALID_ARGUMENT, "heads_create: NULL weight pointer");
    }
    bilstm_status st;
    if ((st = check_len("heads_create W0", static_cast<size_t>(kHeadIn) * kHeadMid, w->w0_len)) != BILSTM_OK) return st;
    if ((st = check_len("heads_create b0", kHeadMid, w->b0_len)) != BILSTM_OK) return st;
    if ((st = check_len("heads_create W1", static_cast<size_t>(kHeadMid) * kHeadMid, w->w1_len)) != BILSTM_OK) return st;
    if ((st = check_len("heads_create b1", kHeadMid, w->b1_len)) != BILSTM_OK) return st;
    if ((st = check_len("heads_create W2", static_cast<size_t>(kHeadMid) * kHeadClasses, w->w2_len)) != BILSTM_OK) return st;
    if ((st = check_len("heads_create b2", kHeadClasses, w->b2_len)) != BILSTM_OK) return st;
    if (!(w->slope == w->slope)) return fail(BILSTM_INVALID_ARGUMENT, "heads_create: slope is NaN");
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count == 0) {
        return fail(BILSTM_UNSUPPORTED, "heads_create: no HIP device (%s)", hipGetErrorString(e));
    }
    if (device < 0 || device >= count) {
        return fail(BILSTM_INVALID_ARGUMENT, "heads_create: device %d out of range (%d devices)", device, count);
    }
    if (!gfx950(device)) return fail(BILSTM_UNSUPPORTED, "heads_create: device %d is not a gfx950 (MI355X) GPU", device);
    int saved = 0;
    const bool have = hipGetDevice(&saved) == hipSuccess;
    e = hipSetDevice(device);
    if (e != hipSuccess) return fail(BILSTM_HIP_ERROR, "heads_create: hipSetDevice: %s", hipGetErrorString(e));

    auto *h = new bilstm_heads();
    h->device = device;
    h->slope = w->slope;
    const std::vector<float> w0t = transpose(w->w0, kHeadIn, kHeadMid, kHeadMid);
    const std::vector<float> w1t = transpose(w->w1, kHeadMid, kHeadMid, kHeadMid);
    const std::vector<float> w2t = transpose(w->w2, kHeadMid, kHeadClasses, kHeadClassSlots);
    struct Up {
        float **dst;
        const float *src;
        size_t n;
    } ups[] = {{&h->w0t, w0t.data(), w0t.size()}, {&h->b0, w->b0, static_cast<size_t>(kHeadMid)},
               {&h->w1t, w1t.data(), w1t.size()}, {&h->b1, w->b1, static_cast<size_t>(kHeadMid)},
               {&h->w2t, w2t.data(), w2t.size()}, {&h->b2, w->b2, static_cast<size_t>(kHeadClasses)}};
    for (const Up &u : ups) {
        e = hipMalloc(reinterpret_cast<void **>(u.dst), u.n * sizeof(float));
        if (e == hipSuccess) e = hipMemcpy(*u.dst, u.src, u.n * sizeof(float), hipMemcpyHostToDevice);
        if (e != hipSuccess) break;
    }
    if (have) (void)hipSetDevice(saved);
    if (e != hipSuccess) {
        release_heads(h);
        return fail(BILSTM_HIP_ERROR, "heads_create: weight upload: %s", hipGetErrorString(e));
    }
    *out = h;
    return BILSTM_OK;
}

bilstm_status bilstm_heads_forward(bilstm_heads *heads, const float *y, size_t y_len, float *out,
                                   size_t out_len, void *stream) {
    if (heads == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "heads_forward: heads is NULL");
    if (y_len == 0 && out_len == 0) return BILSTM_OK;  // no rows: nothing to do
    if (y == nullptr || out == nullptr) return fail(BILSTM_INVALID_ARGUMENT, "heads_forward: NULL buffer");
    if ((reinterpret_cast<uintptr_t>(y) & 15u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0) {
        return fail(BILSTM_INVALID_ARGUMENT, "heads_forward: y must be 16-byte aligned and out 4-byte aligned");
    }
    if (y_len % kHeadIn != 0) {
        return fail(BILSTM_BUFFER_LENGTH, "heads_forward input: expected a multiple of %d elements, got %zu",
                    kHeadIn, y_len);
    }
    const size_t rows = y_len / kHeadIn;
    bilstm_status st;
    if ((st = check_len("heads_forward output", rows * kHeadClasses, out_len)) != BILSTM_OK) return st;
    if (rows > 0x7FFFFFFFull / kHeadIn) {
        return fail(BILSTM_DIMENSION_OVERFLOW, "heads_forward: %zu rows exceed the kernel's indexing", rows);
    }
    const uintptr_t yb = reinterpret_cast<uintptr_t>(y), ob = reinterpret_cast<uintptr_t>(out);
    if (yb < ob + out_len * sizeof(float) && ob < yb + y_len * sizeof(float)) {
        return fail(BILSTM_INVALID_ARGUMENT, "heads_forward: input and output overlap");
    }
    int saved = 0;
    const bool have = hipGetDevice(&saved) == hipSuccess;
    hipError_t e = hipSetDevice(heads->device);
    if (e == hipSuccess) {
        HeadArgs a{};
        a.y = y;
        a.out = out;
        a.w0t = heads->w0t;
        a.b0 = heads->b0;
        a.w1t = heads->w1t;
        a.b1 = heads->b1;
        a.w2t = heads->w2t;
        a.b2 = heads->b2;
        a.slope = heads->slope;
        a.rows = static_cast<long>(rows);
        e = launch_heads(a, static_cast<hipStream_t>(stream));
    }
    if (have) (void)hipSetDevice(saved);
    if (e != hipSuccess) return fail(BILSTM_HIP_ERROR, "heads_forward: launch: %s", hipGetErrorString(e));
    return BILSTM_OK;
}

void bilstm_heads_destroy(bilstm_heads *heads) { release_heads(heads); }

}  // extern "C"
