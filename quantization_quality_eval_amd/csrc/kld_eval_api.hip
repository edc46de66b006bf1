// Host side of the C ABI declared in include/kld_eval.h: handle lifetime,
// argument validation, stream/event ordering, latched asynchronous errors and
// the summary copy-back. All computation happens in the HIP kernels
// (kld_row.hip, kld_reduce.hip).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <new>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "kld_eval.h"
#include "kld_kernels.h"

namespace {

constexpr uint32_t kMagic = 0x4b4c4445u;  // "KLDE"
constexpr int64_t kMaxRowsPerLaunch = int64_t{1} << 30;

thread_local std::string g_last_error;
std::mutex g_live_mu;
std::set<const kld_eval*> g_live;

kld_status fail(kld_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

std::string hip_msg(const char* what, hipError_t e) {
    return std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
}

}  // namespace

struct kld_eval {
    uint32_t magic = kMagic;
    int device = 0;
    int64_t vocab = 0;
    int64_t max_rows = 0;
    int32_t base_type = 0;
    int32_t quant_type = 0;
    // per-token buffers, max_rows each
    float* kld = nullptr;
    uint8_t* match = nullptr;
    int32_t* argmax_b = nullptr;
    int32_t* argmax_q = nullptr;
    float* lse_b = nullptr;
    float* lse_q = nullptr;
    // reduction partials and result
    double* part_sum = nullptr;
    double* part_max = nullptr;
    int64_t* part_max_row = nullptr;
    int64_t* part_match = nullptr;
    kldk::DevSummary* dsum = nullptr;
    kldk::DevSummary* hsum = nullptr;  // pinned host
    std::mutex mu;
    std::vector<std::pair<hipStream_t, hipEvent_t>> events;  // last work recorded per stream
    hipError_t sticky = hipSuccess;
};

namespace {

bool live(const kld_eval* h) {
    if (!h) return false;
    std::lock_guard<std::mutex> g(g_live_mu);
    return g_live.count(h) != 0 && h->magic == kMagic;
}

// Makes the handle's device current for the lifetime of the guard.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            switched = (err == hipSuccess);
        }
    }
    ~DeviceGuard() {
        if (switched) (void)hipSetDevice(prev);
    }
};

void free_all(kld_eval* h) {
    void* dev_ptrs[] = {h->kld, h->match, h->argmax_b, h->argmax_q, h->lse_b, h->lse_q,
                        h->part_sum, h->part_max, h->part_max_row, h->part_match, h->dsum};
    for (void* p : dev_ptrs)
        if (p) (void)hipFree(p);
    if (h->hsum) (void)hipHostFree(h->hsum);
    for (auto& se : h->events) (void)hipEventDestroy(se.second);
    h->events.clear();
}

kld_status latch(kld_eval* h, const char* what, hipError_t e) {
    {
        std::lock_guard<std::mutex> g(h->mu);
        if (h->sticky == hipSuccess) h->sticky = e;
    }
    return fail(KLD_ERR_HIP, hip_msg(what, e));
}

kld_status check_sticky(kld_eval* h) {
    std::lock_guard<std::mutex> g(h->mu);
    if (h->sticky != hipSuccess) return fail(KLD_ERR_HIP, hip_msg("earlier asynchronous error", h->sticky));
    return KLD_OK;
}

// Record that work was enqueued on `s` for this handle.
hipError_t record(kld_eval* h, hipStream_t s) {
    std::lock_guard<std::mutex> g(h->mu);
    for (auto& se : h->events)
        if (se.first == s) return hipEventRecord(se.second, s);
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    h->events.emplace_back(s, ev);
    return hipEventRecord(ev, s);
}

// Order `s` after all work recorded on other streams.
hipError_t wait_all(kld_eval* h, hipStream_t s) {
    std::lock_guard<std::mutex> g(h->mu);
    for (auto& se : h->events) {
        if (se.first == s) continue;
        hipError_t e = hipStreamWaitEvent(s, se.second, 0);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class T>
hipError_t dalloc(T** p, int64_t n) {
    return hipMalloc(reinterpret_cast<void**>(p), static_cast<size_t>(n) * sizeof(T));
}

}  // namespace

extern "C" {

kld_status kld_eval_create(kld_eval** out, int64_t vocab, int64_t max_rows, int32_t base_dtype,
                           int32_t quant_dtype) {
    if (!out) return fail(KLD_ERR_INVALID_ARG, "kld_eval_create: out is NULL");
    *out = nullptr;
    if (vocab < 1 || vocab > INT32_MAX)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_create: vocab must be in [1, 2^31-1]");
    if (max_rows < 1 || max_rows > (int64_t{1} << 40))
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_create: max_rows must be in [1, 2^40]");
    if ((base_dtype != KLD_DTYPE_F32 && base_dtype != KLD_DTYPE_BF16) ||
        (quant_dtype != KLD_DTYPE_F32 && quant_dtype != KLD_DTYPE_BF16))
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_create: dtype must be KLD_DTYPE_F32 or KLD_DTYPE_BF16");
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) return fail(KLD_ERR_NO_DEVICE, "kld_eval_create: no HIP device visible");
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KLD_ERR_NO_DEVICE, hip_msg("kld_eval_create: hipGetDevice", e));
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(KLD_ERR_HIP, hip_msg("kld_eval_create: hipGetDeviceProperties", e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(KLD_ERR_UNSUPPORTED_ARCH,
                    std::string("kld_eval_create: built for gfx950, device is ") + prop.gcnArchName);
    const char* inj = std::getenv("KLD_EVAL_FAIL_ALLOC");
    if (inj && std::strcmp(inj, "1") == 0)
        return fail(KLD_ERR_OUT_OF_MEMORY, "kld_eval_create: allocation failure injected (KLD_EVAL_FAIL_ALLOC=1)");

    kld_eval* h = new (std::nothrow) kld_eval;
    if (!h) return fail(KLD_ERR_OUT_OF_MEMORY, "kld_eval_create: host allocation failed");
    h->device = dev;
    h->vocab = vocab;
    h->max_rows = max_rows;
    h->base_type = base_dtype;
    h->quant_type = quant_dtype;
    const int64_t np = kldk::reduce_partials(max_rows);
    hipError_t a = hipSuccess;
    if (a == hipSuccess) a = dalloc(&h->kld, max_rows);
    if (a == hipSuccess) a = dalloc(&h->match, max_rows);
    if (a == hipSuccess) a = dalloc(&h->argmax_b, max_rows);
    if (a == hipSuccess) a = dalloc(&h->argmax_q, max_rows);
    if (a == hipSuccess) a = dalloc(&h->lse_b, max_rows);
    if (a == hipSuccess) a = dalloc(&h->lse_q, max_rows);
    if (a == hipSuccess) a = dalloc(&h->part_sum, np);
    if (a == hipSuccess) a = dalloc(&h->part_max, np);
    if (a == hipSuccess) a = dalloc(&h->part_max_row, np);
    if (a == hipSuccess) a = dalloc(&h->part_match, np);
    if (a == hipSuccess) a = dalloc(&h->dsum, 1);
    if (a == hipSuccess) a = hipHostMalloc(reinterpret_cast<void**>(&h->hsum), sizeof(kldk::DevSummary), 0);
    if (a != hipSuccess) {
        free_all(h);
        delete h;
        (void)hipGetLastError();
        return fail(KLD_ERR_OUT_OF_MEMORY, hip_msg("kld_eval_create: allocation", a));
    }
    {
        std::lock_guard<std::mutex> g(g_live_mu);
        g_live.insert(h);
    }
    *out = h;
    return KLD_OK;
}

kld_status kld_eval_rows(kld_eval* h, const void* base, const void* quant, int64_t n_rows, int64_t row_offset,
                         float* kld_out, uint8_t* match_out, int32_t* argmax_base_out, int32_t* argmax_quant_out,
                         void* stream) {
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_rows: invalid or destroyed handle");
    if (n_rows < 0 || row_offset < 0) return fail(KLD_ERR_INVALID_ARG, "kld_eval_rows: negative n_rows or row_offset");
    if (n_rows == 0) return KLD_OK;
    if (!base || !quant) return fail(KLD_ERR_INVALID_ARG, "kld_eval_rows: base or quant is NULL");
    if (row_offset > h->max_rows || n_rows > h->max_rows - row_offset)
        return fail(KLD_ERR_RANGE, "kld_eval_rows: row_offset + n_rows exceeds max_rows");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_rows: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t sb = h->base_type == KLD_DTYPE_F32 ? 4 : 2;
    const size_t sq = h->quant_type == KLD_DTYPE_F32 ? 4 : 2;
    for (int64_t done = 0; done < n_rows; done += kMaxRowsPerLaunch) {
        const int64_t n = std::min(kMaxRowsPerLaunch, n_rows - done);
        kldk::RowOut o;
        o.kld = h->kld;
        o.match = h->match;
        o.argmax_b = h->argmax_b;
        o.argmax_q = h->argmax_q;
        o.lse_b = h->lse_b;
        o.lse_q = h->lse_q;
        o.kld_out = kld_out ? kld_out + done : nullptr;
        o.match_out = match_out ? match_out + done : nullptr;
        o.argmax_b_out = argmax_base_out ? argmax_base_out + done : nullptr;
        o.argmax_q_out = argmax_quant_out ? argmax_quant_out + done : nullptr;
        const char* pb = static_cast<const char*>(base) + static_cast<size_t>(done) * h->vocab * sb;
        const char* pq = static_cast<const char*>(quant) + static_cast<size_t>(done) * h->vocab * sq;
        hipError_t e = kldk::launch_rows(h->base_type, h->quant_type, pb, pq, h->vocab, n, row_offset + done,
                                         h->max_rows, o, s);
        if (e != hipSuccess) return latch(h, "kld_eval_rows: kernel launch", e);
    }
    hipError_t e = record(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_rows: event record", e);
    return KLD_OK;
}

kld_status kld_eval_reduce(kld_eval* h, int64_t n_rows, kld_eval_summary* out, void* stream) {
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_reduce: invalid or destroyed handle");
    if (!out) return fail(KLD_ERR_INVALID_ARG, "kld_eval_reduce: out is NULL");
    if (n_rows < 0) return fail(KLD_ERR_INVALID_ARG, "kld_eval_reduce: negative n_rows");
    if (n_rows == 0) return fail(KLD_ERR_EMPTY, "kld_eval_reduce: zero rows");
    if (n_rows > h->max_rows) return fail(KLD_ERR_RANGE, "kld_eval_reduce: n_rows exceeds max_rows");
    kld_status st = check_sticky(h);
    if (st != KLD_OK) return st;
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_reduce: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = wait_all(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_reduce: stream wait", e);
    e = kldk::launch_reduce(h->kld, h->match, n_rows, h->part_sum, h->part_max, h->part_max_row, h->part_match,
                            h->dsum, s);
    if (e != hipSuccess) return latch(h, "kld_eval_reduce: kernel launch", e);
    e = hipMemcpyAsync(h->hsum, h->dsum, sizeof(kldk::DevSummary), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return latch(h, "kld_eval_reduce: summary copy", e);
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return latch(h, "kld_eval_reduce: synchronize", e);
    const kldk::DevSummary d = *h->hsum;
    out->n_rows = d.n_rows;
    out->kld_sum = d.kld_sum;
    out->kld_mean = d.kld_sum / static_cast<double>(d.n_rows);
    out->kld_max = d.kld_max;
    out->kld_max_row = d.kld_max_row;
    out->n_match = d.n_match;
    out->same_top1 = static_cast<double>(d.n_match) / static_cast<double>(d.n_rows);
    return KLD_OK;
}

kld_status kld_eval_copy_lse(kld_eval* h, int64_t row_offset, int64_t n_rows, float* lse_base_out,
                             float* lse_quant_out, void* stream) {
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_copy_lse: invalid or destroyed handle");
    if (n_rows < 0 || row_offset < 0)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_copy_lse: negative n_rows or row_offset");
    if (row_offset > h->max_rows || n_rows > h->max_rows - row_offset)
        return fail(KLD_ERR_RANGE, "kld_eval_copy_lse: row_offset + n_rows exceeds max_rows");
    if (n_rows == 0) return KLD_OK;
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_copy_lse: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = wait_all(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_copy_lse: stream wait", e);
    const size_t bytes = static_cast<size_t>(n_rows) * sizeof(float);
    if (lse_base_out) {
        e = hipMemcpyAsync(lse_base_out, h->lse_b + row_offset, bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return latch(h, "kld_eval_copy_lse: copy", e);
    }
    if (lse_quant_out) {
        e = hipMemcpyAsync(lse_quant_out, h->lse_q + row_offset, bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return latch(h, "kld_eval_copy_lse: copy", e);
    }
    return KLD_OK;
}

kld_status kld_eval_destroy(kld_eval* h) {
    if (!h) return KLD_OK;
    {
        std::lock_guard<std::mutex> g(g_live_mu);
        if (!g_live.count(h) || h->magic != kMagic)
            return fail(KLD_ERR_BAD_HANDLE, "kld_eval_destroy: invalid or already destroyed handle");
        g_live.erase(h);
    }
    kld_status st = KLD_OK;
    {
        DeviceGuard dg(h->device);
        for (auto& se : h->events) {
            hipError_t e = hipEventSynchronize(se.second);
            if (e != hipSuccess && h->sticky == hipSuccess) h->sticky = e;
        }
        if (h->sticky != hipSuccess) st = fail(KLD_ERR_HIP, hip_msg("kld_eval_destroy: latched error", h->sticky));
        free_all(h);
    }
    h->magic = 0;
    delete h;
    return st;
}

const char* kld_eval_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
