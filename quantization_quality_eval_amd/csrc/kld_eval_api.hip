// Host side of the C ABI declared in include/kld_eval.h: handle lifetime,
// argument validation, stream/event ordering, latched asynchronous errors and
// the summary copy-back. All computation happens in the HIP kernels
// (kld_row.hip, kld_reduce.hip, kld_grad.hip, kld_topk.hip; kld_probe.hip for
// the read-bandwidth probe).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <cmath>
#include <new>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "kld_eval.h"
#include "kld_kernels.h"
#include "kld_probe.h"

#ifdef KLD_EVAL_ROCTX
#include <rocprofiler-sdk-roctx/roctx.h>
#endif

namespace {

constexpr uint32_t kMagic = 0x4b4c4445u;  // "KLDE"

// A named roctx range over one call of the C ABI (its argument checks and
// enqueues on the host; the kernels it launches show in a kernel trace), for
// `rocprofv3 --marker-trace`. Only builds made with KLD_EVAL_ROCTX defined
// (and linked with the roctx library) emit it; in the default build it is
// empty and the library does not depend on roctx.
struct CallRange {
#ifdef KLD_EVAL_ROCTX
    explicit CallRange(const char* name) { roctxRangePushA(name); }
    ~CallRange() { roctxRangePop(); }
#else
    explicit CallRange(const char*) {}
#endif
    CallRange(const CallRange&) = delete;
    CallRange& operator=(const CallRange&) = delete;
};

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

// Reduction workspace: tile descriptors and partials (device), segment tables
// and results (device), and their pinned host staging. Sized at create for
// one segment over max_rows rows; grown by the first call that needs more.
struct ReduceSpace {
    int64_t cap_tiles = 0;
    int64_t cap_segs = 0;
    kldk::ReduceTile* tiles = nullptr;
    kldk::Partial* parts = nullptr;
    int64_t* seg_tile = nullptr;  // cap_segs + 1
    int64_t* seg_rows = nullptr;  // cap_segs
    kldk::DevSummary* res = nullptr;
    unsigned int* done = nullptr;  // ticket counter of the one-launch reduction (zero between launches)
    kldk::ReduceTile* h_tiles = nullptr;  // pinned host staging
    int64_t* h_seg_tile = nullptr;
    int64_t* h_seg_rows = nullptr;
    kldk::DevSummary* h_res = nullptr;
    kldk::DevSummary* h_res_dev = nullptr;  // h_res as the device addresses it
    // Segment offsets whose tile and segment tables are on the device (empty:
    // none); a reduction over the same offsets skips their upload.
    std::vector<int64_t> uploaded;
    // Segment offsets whose results h_res holds, and the handle's row-write
    // count they reflect (kNoResults: none). A reduction over the same offsets
    // with no row write since returns them as they are.
    std::vector<int64_t> res_offsets;
    uint64_t res_writes = UINT64_MAX;
};
constexpr uint64_t kNoResults = UINT64_MAX;

struct kld_eval {
    uint32_t magic = kMagic;
    int device = 0;
    int64_t vocab = 0;
    int64_t max_rows = 0;
    int32_t base_type = 0;
    int32_t quant_type = 0;
    int64_t max_lds = 0;  // LDS bytes one workgroup may use on this device
    // per-token buffers, max_rows each
    float* kld = nullptr;
    uint8_t* match = nullptr;
    int32_t* argmax_b = nullptr;
    int32_t* argmax_q = nullptr;
    double* lse_b = nullptr;
    double* lse_q = nullptr;
    float* logp_b = nullptr;
    float* logp_q = nullptr;
    float* dp = nullptr;
    uint8_t* tok_state = nullptr;
    uint8_t* retake = nullptr;    // conditioning flags of the row pass (rows it evaluated a second time)
    double* topk_coef = nullptr;  // 3 per row, rows evaluated from a stored top-K form: P + R, (P + R) Q_rest - R, lse_rest
    ReduceSpace rs;
    std::mutex reduce_mu;  // one reduction at a time per handle (shared workspace)
    std::mutex mu;
    std::vector<std::pair<hipStream_t, hipEvent_t>> events;  // last work recorded per stream
    uint64_t row_writes = 0;  // calls so far that wrote per-token rows (under mu, with their events)
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

void free_space(ReduceSpace& rs) {
    void* dev_ptrs[] = {rs.tiles, rs.parts, rs.seg_tile, rs.seg_rows, rs.res, rs.done};
    for (void* p : dev_ptrs)
        if (p) (void)hipFree(p);
    void* host_ptrs[] = {rs.h_tiles, rs.h_seg_tile, rs.h_seg_rows, rs.h_res};
    for (void* p : host_ptrs)
        if (p) (void)hipHostFree(p);
    rs = ReduceSpace{};
}

void free_all(kld_eval* h) {
    void* dev_ptrs[] = {h->kld, h->match, h->argmax_b, h->argmax_q, h->lse_b, h->lse_q,
                        h->logp_b, h->logp_q, h->dp, h->tok_state, h->retake, h->topk_coef};
    for (void* p : dev_ptrs)
        if (p) (void)hipFree(p);
    free_space(h->rs);
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

// Record that work was enqueued on `s` for this handle; `writes_rows` counts
// a call that wrote per-token rows.
hipError_t record(kld_eval* h, hipStream_t s, bool writes_rows = false) {
    std::lock_guard<std::mutex> g(h->mu);
    if (writes_rows) ++h->row_writes;
    for (auto& se : h->events)
        if (se.first == s) return hipEventRecord(se.second, s);
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    h->events.emplace_back(s, ev);
    return hipEventRecord(ev, s);
}

// Order `s` after all work recorded on other streams; `writes_seen` receives
// the row-write count of the work so ordered.
hipError_t wait_all(kld_eval* h, hipStream_t s, uint64_t* writes_seen = nullptr) {
    std::lock_guard<std::mutex> g(h->mu);
    if (writes_seen) *writes_seen = h->row_writes;
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

template <class T>
hipError_t halloc(T** p, int64_t n) {
    return hipHostMalloc(reinterpret_cast<void**>(p), static_cast<size_t>(n) * sizeof(T), 0);
}

// Make the workspace hold n_tiles tiles and n_segs segments. Called with the
// handle's reduce_mu held and the handle's device current. A reduction
// enqueued by kld_eval_reduce_async may still be running on the old buffers,
// so the device is synchronized before they are freed (growth happens only
// for segmented reductions beyond the create-time size).
hipError_t reserve(ReduceSpace& rs, int64_t n_tiles, int64_t n_segs) {
    if (n_tiles <= rs.cap_tiles && n_segs <= rs.cap_segs) return hipSuccess;
    if (rs.cap_tiles > 0) {
        const hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return e;
    }
    ReduceSpace nw;
    nw.cap_tiles = std::max<int64_t>(std::max<int64_t>(n_tiles, rs.cap_tiles), 1);
    nw.cap_segs = std::max<int64_t>(n_segs, rs.cap_segs);
    hipError_t a = dalloc(&nw.tiles, nw.cap_tiles);
    if (a == hipSuccess) a = dalloc(&nw.parts, nw.cap_tiles);
    if (a == hipSuccess) a = dalloc(&nw.seg_tile, nw.cap_segs + 1);
    if (a == hipSuccess) a = dalloc(&nw.seg_rows, nw.cap_segs);
    if (a == hipSuccess) a = dalloc(&nw.res, nw.cap_segs);
    if (a == hipSuccess) a = halloc(&nw.h_tiles, nw.cap_tiles);
    if (a == hipSuccess) a = halloc(&nw.h_seg_tile, nw.cap_segs + 1);
    if (a == hipSuccess) a = halloc(&nw.h_seg_rows, nw.cap_segs);
    if (a == hipSuccess) a = halloc(&nw.h_res, nw.cap_segs);
    if (a == hipSuccess) a = dalloc(&nw.done, 1);
    if (a == hipSuccess) a = hipMemset(nw.done, 0, sizeof(unsigned int));
    if (a == hipSuccess) a = hipHostGetDevicePointer(reinterpret_cast<void**>(&nw.h_res_dev), nw.h_res, 0);
    if (a != hipSuccess) {
        free_space(nw);
        (void)hipGetLastError();
        return a;
    }
    free_space(rs);
    rs = nw;
    return hipSuccess;
}

int64_t count_tiles(const int64_t* off, int64_t n_segs) {
    int64_t n = 0;
    for (int64_t k = 0; k < n_segs; ++k) n += (off[k + 1] - off[k] + kldk::kReduceTileRows - 1) / kldk::kReduceTileRows;
    return n;
}

// Run the reduction over segments [off[s], off[s+1]) and leave the results in
// rs.h_res[0 .. n_segs). The caller holds reduce_mu, has validated `off` and
// has reserved the workspace for it. One segment starting at row 0 is reduced
// in a single launch that writes the sums straight into the pinned h_res;
// several segments use the tile and segment tables (uploaded when the offsets
// changed), two launches and a copy back. Both give the same bits.
hipError_t run_reduce(kld_eval* h, const int64_t* off, int64_t n_segs, hipStream_t s) {
    ReduceSpace& rs = h->rs;
    uint64_t seen = 0;
    hipError_t e = wait_all(h, s, &seen);
    if (e != hipSuccess) return e;
    const bool same = rs.res_offsets.size() == static_cast<size_t>(n_segs + 1) &&
                      std::equal(off, off + n_segs + 1, rs.res_offsets.begin());
    if (same && rs.res_writes == seen) return hipSuccess;  // h_res already holds these results
    rs.res_writes = kNoResults;
    rs.res_offsets.clear();
    const kldk::RowIn in{h->kld, h->match, h->logp_b, h->logp_q, h->dp, h->tok_state};
    const int64_t whole = off[n_segs] - off[0];
    if (n_segs == 1 && off[0] == 0 && whole >= 1 &&
        (whole + kldk::kReduceTileRows - 1) / kldk::kReduceTileRows <= kldk::reduce_fused_max_tiles()) {
        e = kldk::launch_reduce_fused(in, whole, rs.parts, rs.done, rs.h_res_dev, nullptr, s);
        if (e != hipSuccess) return e;
    } else {
        int64_t t = 0;
        for (int64_t k = 0; k < n_segs; ++k) {
            rs.h_seg_tile[k] = t;
            rs.h_seg_rows[k] = off[k + 1] - off[k];
            for (int64_t r = off[k]; r < off[k + 1]; r += kldk::kReduceTileRows)
                rs.h_tiles[t++] = kldk::ReduceTile{r, std::min(r + kldk::kReduceTileRows, off[k + 1])};
        }
        rs.h_seg_tile[n_segs] = t;
        const int64_t n_tiles = t;
        const bool uploaded = rs.uploaded.size() == static_cast<size_t>(n_segs + 1) &&
                              std::equal(off, off + n_segs + 1, rs.uploaded.begin());
        if (!uploaded) {
            rs.uploaded.clear();  // set again once the upload below has completed
            if (n_tiles > 0) {
                e = hipMemcpyAsync(rs.tiles, rs.h_tiles, static_cast<size_t>(n_tiles) * sizeof(kldk::ReduceTile),
                                   hipMemcpyHostToDevice, s);
                if (e != hipSuccess) return e;
            }
            e = hipMemcpyAsync(rs.seg_tile, rs.h_seg_tile, static_cast<size_t>(n_segs + 1) * sizeof(int64_t),
                               hipMemcpyHostToDevice, s);
            if (e != hipSuccess) return e;
            e = hipMemcpyAsync(rs.seg_rows, rs.h_seg_rows, static_cast<size_t>(n_segs) * sizeof(int64_t),
                               hipMemcpyHostToDevice, s);
            if (e != hipSuccess) return e;
        }
        e = kldk::launch_reduce(in, rs.tiles, n_tiles, rs.seg_tile, rs.seg_rows, n_segs, rs.parts, rs.res, s);
        if (e != hipSuccess) return e;
        e = hipMemcpyAsync(rs.h_res, rs.res, static_cast<size_t>(n_segs) * sizeof(kldk::DevSummary),
                           hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return e;
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return e;
        if (!uploaded) rs.uploaded.assign(off, off + n_segs + 1);
        rs.res_offsets.assign(off, off + n_segs + 1);
        rs.res_writes = seen;
        return hipSuccess;
    }
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    rs.res_offsets.assign(off, off + n_segs + 1);
    rs.res_writes = seen;
    return hipSuccess;
}

void to_summary(const kldk::DevSummary& d, kld_eval_summary* o) {
    const double n = static_cast<double>(d.n_rows);
    o->n_rows = d.n_rows;
    o->kld_sum = d.kld_sum;
    o->kld_mean = d.n_rows > 0 ? d.kld_sum / n : NAN;
    o->kld_max = d.kld_max;
    o->kld_max_row = d.n_rows > 0 ? d.kld_max_row : -1;
    o->n_match = d.n_match;
    o->same_top1 = d.n_rows > 0 ? static_cast<double>(d.n_match) / n : NAN;
}

void to_token_summary(const kldk::DevSummary& d, kld_eval_token_summary* o) {
    o->n_scored = d.n_scored;
    o->n_invalid = d.n_invalid;
    o->logp_base_sum = d.logp_b_sum;
    o->logp_quant_sum = d.logp_q_sum;
    if (d.n_scored > 0) {
        const double n = static_cast<double>(d.n_scored);
        o->ppl_base = std::exp(-d.logp_b_sum / n);
        o->ppl_quant = std::exp(-d.logp_q_sum / n);
        // the same ratio as one exponential: finite where both perplexities overflow
        o->ppl_ratio = std::exp((d.logp_b_sum - d.logp_q_sum) / n);
        o->dp_mean = d.dp_sum / n;
        o->dp_rms = std::sqrt(d.dp2_sum / n);
    } else {
        o->ppl_base = o->ppl_quant = o->ppl_ratio = o->dp_mean = o->dp_rms = NAN;
    }
}

}  // namespace

namespace {

// Workspace of kld_eval_compare_noalloc: the reduction partials, one per tile
// of kReduceTileRows rows, for at most kNoAllocMaxRows rows (4096 partials of
// 80 B, 320 KiB). A file-scope device array: each GPU the library runs on
// holds its own copy from module load until the process ends, so the entry
// point never allocates. Host code must use the address hipGetSymbolAddress
// gives on each device, never this name (a host-side stand-in).
constexpr int64_t kNoAllocMaxRows = int64_t{1} << 22;
constexpr int64_t kNoAllocMaxTiles = kNoAllocMaxRows / kldk::kReduceTileRows;
static __device__ __align__(256) kldk::Partial scratch[kNoAllocMaxTiles];

// Per device: the device address of `scratch`, resolved on the first call on
// that device (with it current), and whether the device is a gfx950.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
kldk::Partial* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_checked[kMaxDevices] = {};

kld_status noalloc_scratch(int dev, kldk::Partial** out) {
    const char* who = "kld_eval_compare_noalloc";
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": device index beyond the supported 64");
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_checked[dev]) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(KLD_ERR_HIP, hip_msg(who, e));
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return fail(KLD_ERR_UNSUPPORTED_ARCH, std::string(who) + ": built for gfx950, device is " +
                                                      prop.gcnArchName);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(KLD_ERR_HIP, hip_msg("kld_eval_compare_noalloc: hipGetSymbolAddress(scratch)",
                                             e != hipSuccess ? e : hipErrorInvalidSymbol));
        }
        g_scratch_ptr[dev] = static_cast<kldk::Partial*>(p);
        g_scratch_checked[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return KLD_OK;
}

}  // namespace

extern "C" {

kld_status kld_eval_create(kld_eval** out, int64_t vocab, int64_t max_rows, int32_t base_dtype,
                           int32_t quant_dtype) {
    const CallRange range_("kld_eval_create");
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
    h->max_lds = static_cast<int64_t>(prop.sharedMemPerBlock);
    h->vocab = vocab;
    h->max_rows = max_rows;
    h->base_type = base_dtype;
    h->quant_type = quant_dtype;
    hipError_t a = hipSuccess;
    if (a == hipSuccess) a = dalloc(&h->kld, max_rows);
    if (a == hipSuccess) a = dalloc(&h->match, max_rows);
    if (a == hipSuccess) a = dalloc(&h->argmax_b, max_rows);
    if (a == hipSuccess) a = dalloc(&h->argmax_q, max_rows);
    if (a == hipSuccess) a = dalloc(&h->lse_b, max_rows);
    if (a == hipSuccess) a = dalloc(&h->lse_q, max_rows);
    if (a == hipSuccess) a = dalloc(&h->logp_b, max_rows);
    if (a == hipSuccess) a = dalloc(&h->logp_q, max_rows);
    if (a == hipSuccess) a = dalloc(&h->dp, max_rows);
    if (a == hipSuccess) a = dalloc(&h->tok_state, max_rows);
    if (a == hipSuccess) a = dalloc(&h->retake, max_rows);
    if (a == hipSuccess) a = hipMemset(h->retake, 0, static_cast<size_t>(max_rows));  // no row written yet
    if (a == hipSuccess) a = dalloc(&h->topk_coef, 3 * max_rows);
    if (a == hipSuccess)
        a = reserve(h->rs, (max_rows + kldk::kReduceTileRows - 1) / kldk::kReduceTileRows, 1);
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

}  // extern "C"

namespace {

// Shared body of the row calls. start / stop (may be null) go to the first and
// the last launch of the call, which record them themselves.
kld_status rows_impl(kld_eval* h, const void* base, const void* quant, const int32_t* tokens, int64_t n_rows,
                     int64_t row_offset, float* kld_out, uint8_t* match_out, int32_t* argmax_base_out,
                     int32_t* argmax_quant_out, float* logp_base_out, float* logp_quant_out, float* dp_out,
                     void* stream, hipEvent_t start, hipEvent_t stop) {
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
    const int64_t per_launch = kldk::rows_max_per_launch();
    for (int64_t done = 0; done < n_rows; done += per_launch) {
        const int64_t n = std::min(per_launch, n_rows - done);
        kldk::RowOut o{};
        o.kld = h->kld;
        o.match = h->match;
        o.argmax_b = h->argmax_b;
        o.argmax_q = h->argmax_q;
        o.lse_b = h->lse_b;
        o.lse_q = h->lse_q;
        o.logp_b = h->logp_b;
        o.logp_q = h->logp_q;
        o.dp = h->dp;
        o.tok_state = h->tok_state;
        o.retake = h->retake;
        o.tokens = tokens ? tokens + done : nullptr;
        o.kld_out = kld_out ? kld_out + done : nullptr;
        o.match_out = match_out ? match_out + done : nullptr;
        o.argmax_b_out = argmax_base_out ? argmax_base_out + done : nullptr;
        o.argmax_q_out = argmax_quant_out ? argmax_quant_out + done : nullptr;
        o.logp_b_out = logp_base_out ? logp_base_out + done : nullptr;
        o.logp_q_out = logp_quant_out ? logp_quant_out + done : nullptr;
        o.dp_out = dp_out ? dp_out + done : nullptr;
        const char* pb = static_cast<const char*>(base) + static_cast<size_t>(done) * h->vocab * sb;
        const char* pq = static_cast<const char*>(quant) + static_cast<size_t>(done) * h->vocab * sq;
        hipError_t e = kldk::launch_rows(h->base_type, h->quant_type, pb, pq, h->vocab, n, row_offset + done,
                                         h->max_rows, o, s, done == 0 ? start : nullptr,
                                         done + n == n_rows ? stop : nullptr);
        if (e != hipSuccess) return latch(h, "kld_eval_rows: kernel launch", e);
    }
    hipError_t e = record(h, s, true);
    if (e != hipSuccess) return latch(h, "kld_eval_rows: event record", e);
    return KLD_OK;
}

}  // namespace

extern "C" {

kld_status kld_eval_rows_tokens(kld_eval* h, const void* base, const void* quant, const int32_t* tokens,
                                int64_t n_rows, int64_t row_offset, float* kld_out, uint8_t* match_out,
                                int32_t* argmax_base_out, int32_t* argmax_quant_out, float* logp_base_out,
                                float* logp_quant_out, float* dp_out, void* stream) {
    const CallRange range_("kld_eval_rows_tokens");
    return rows_impl(h, base, quant, tokens, n_rows, row_offset, kld_out, match_out, argmax_base_out,
                     argmax_quant_out, logp_base_out, logp_quant_out, dp_out, stream, nullptr, nullptr);
}

kld_status kld_eval_rows(kld_eval* h, const void* base, const void* quant, int64_t n_rows, int64_t row_offset,
                         float* kld_out, uint8_t* match_out, int32_t* argmax_base_out, int32_t* argmax_quant_out,
                         void* stream) {
    const CallRange range_("kld_eval_rows");
    return rows_impl(h, base, quant, nullptr, n_rows, row_offset, kld_out, match_out, argmax_base_out,
                     argmax_quant_out, nullptr, nullptr, nullptr, stream, nullptr, nullptr);
}

kld_status kld_eval_rows_timed(kld_eval* h, const void* base, const void* quant, int64_t n_rows,
                               int64_t row_offset, float* kld_out, uint8_t* match_out, int32_t* argmax_base_out,
                               int32_t* argmax_quant_out, void* stream, void* start_event, void* stop_event) {
    const CallRange range_("kld_eval_rows_timed");
    return rows_impl(h, base, quant, nullptr, n_rows, row_offset, kld_out, match_out, argmax_base_out,
                     argmax_quant_out, nullptr, nullptr, nullptr, stream, static_cast<hipEvent_t>(start_event),
                     static_cast<hipEvent_t>(stop_event));
}

}  // extern "C"

namespace {

// Shared body of the reductions: validation done by the caller; runs the
// segments and leaves their results in h->rs.h_res.
kld_status reduce_common(kld_eval* h, const char* who, const int64_t* off, int64_t n_segs, void* stream) {
    kld_status st = check_sticky(h);
    if (st != KLD_OK) return st;
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, who, dg.err);
    hipError_t e = reserve(h->rs, count_tiles(off, n_segs), n_segs);
    if (e != hipSuccess) return fail(KLD_ERR_OUT_OF_MEMORY, hip_msg(who, e));
    e = run_reduce(h, off, n_segs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return latch(h, who, e);
    return KLD_OK;
}

kld_status check_reduce_args(kld_eval* h, const char* who, int64_t n_rows, const void* out) {
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, std::string(who) + ": invalid or destroyed handle");
    if (!out) return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": out is NULL");
    if (n_rows < 0) return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": negative n_rows");
    if (n_rows == 0) return fail(KLD_ERR_EMPTY, std::string(who) + ": zero rows");
    if (n_rows > h->max_rows) return fail(KLD_ERR_RANGE, std::string(who) + ": n_rows exceeds max_rows");
    return KLD_OK;
}

}  // namespace

extern "C" {

kld_status kld_eval_reduce(kld_eval* h, int64_t n_rows, kld_eval_summary* out, void* stream) {
    const CallRange range_("kld_eval_reduce");
    kld_status st = check_reduce_args(h, "kld_eval_reduce", n_rows, out);
    if (st != KLD_OK) return st;
    std::lock_guard<std::mutex> g(h->reduce_mu);
    const int64_t off[2] = {0, n_rows};
    st = reduce_common(h, "kld_eval_reduce", off, 1, stream);
    if (st != KLD_OK) return st;
    to_summary(h->rs.h_res[0], out);
    return KLD_OK;
}

kld_status kld_eval_reduce_async(kld_eval* h, int64_t n_rows, kld_eval_summary* out, void* stream) {
    const CallRange range_("kld_eval_reduce_async");
    const char* who = "kld_eval_reduce_async";
    kld_status st = check_reduce_args(h, who, n_rows, out);
    if (st != KLD_OK) return st;
    if ((n_rows + kldk::kReduceTileRows - 1) / kldk::kReduceTileRows > kldk::reduce_fused_max_tiles())
        return fail(KLD_ERR_RANGE, std::string(who) + ": n_rows beyond one launch of the reduction");
    std::lock_guard<std::mutex> g(h->reduce_mu);
    st = check_sticky(h);
    if (st != KLD_OK) return st;
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, who, dg.err);
    hipError_t e = reserve(h->rs, (n_rows + kldk::kReduceTileRows - 1) / kldk::kReduceTileRows, 1);
    if (e != hipSuccess) return fail(KLD_ERR_OUT_OF_MEMORY, hip_msg(who, e));
    hipStream_t s = static_cast<hipStream_t>(stream);
    e = wait_all(h, s);
    if (e != hipSuccess) return latch(h, who, e);
    const kldk::RowIn in{h->kld, h->match, h->logp_b, h->logp_q, h->dp, h->tok_state};
    e = kldk::launch_reduce_fused(in, n_rows, h->rs.parts, h->rs.done, nullptr, out, s);
    if (e != hipSuccess) return latch(h, who, e);
    // later reductions on other streams share the workspace: they order after this one
    e = record(h, s);
    if (e != hipSuccess) return latch(h, who, e);
    return KLD_OK;
}

kld_status kld_eval_reduce_tokens(kld_eval* h, int64_t n_rows, kld_eval_token_summary* out, void* stream) {
    const CallRange range_("kld_eval_reduce_tokens");
    kld_status st = check_reduce_args(h, "kld_eval_reduce_tokens", n_rows, out);
    if (st != KLD_OK) return st;
    std::lock_guard<std::mutex> g(h->reduce_mu);
    const int64_t off[2] = {0, n_rows};
    st = reduce_common(h, "kld_eval_reduce_tokens", off, 1, stream);
    if (st != KLD_OK) return st;
    to_token_summary(h->rs.h_res[0], out);
    return KLD_OK;
}

kld_status kld_eval_reduce_segments(kld_eval* h, const int64_t* offsets, int64_t n_segments,
                                    kld_eval_summary* kld_out, kld_eval_token_summary* tok_out, void* stream) {
    const CallRange range_("kld_eval_reduce_segments");
    const char* who = "kld_eval_reduce_segments";
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, std::string(who) + ": invalid or destroyed handle");
    if (!offsets) return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": offsets is NULL");
    if (n_segments < 1 || n_segments > (int64_t{1} << 30))
        return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": n_segments must be in [1, 2^30]");
    for (int64_t k = 0; k <= n_segments; ++k) {
        if (offsets[k] < 0 || offsets[k] > h->max_rows)
            return fail(KLD_ERR_RANGE, std::string(who) + ": offset outside [0, max_rows]");
        if (k > 0 && offsets[k] < offsets[k - 1])
            return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": offsets decrease");
    }
    std::lock_guard<std::mutex> g(h->reduce_mu);
    kld_status st = reduce_common(h, who, offsets, n_segments, stream);
    if (st != KLD_OK) return st;
    for (int64_t k = 0; k < n_segments; ++k) {
        if (kld_out) to_summary(h->rs.h_res[k], kld_out + k);
        if (tok_out) to_token_summary(h->rs.h_res[k], tok_out + k);
    }
    return KLD_OK;
}

kld_status kld_eval_copy_lse(kld_eval* h, int64_t row_offset, int64_t n_rows, float* lse_base_out,
                             float* lse_quant_out, void* stream) {
    const CallRange range_("kld_eval_copy_lse");
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
    if (lse_base_out) {
        e = kldk::launch_lse_to_f32(h->lse_b + row_offset, lse_base_out, n_rows, s);
        if (e != hipSuccess) return latch(h, "kld_eval_copy_lse: kernel launch", e);
    }
    if (lse_quant_out) {
        e = kldk::launch_lse_to_f32(h->lse_q + row_offset, lse_quant_out, n_rows, s);
        if (e != hipSuccess) return latch(h, "kld_eval_copy_lse: kernel launch", e);
    }
    return KLD_OK;
}

kld_status kld_eval_copy_row_flags(kld_eval* h, int64_t row_offset, int64_t n_rows, uint8_t* flags_out,
                                   void* stream) {
    const CallRange range_("kld_eval_copy_row_flags");
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_copy_row_flags: invalid or destroyed handle");
    if (n_rows < 0 || row_offset < 0)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_copy_row_flags: negative n_rows or row_offset");
    if (row_offset > h->max_rows || n_rows > h->max_rows - row_offset)
        return fail(KLD_ERR_RANGE, "kld_eval_copy_row_flags: row_offset + n_rows exceeds max_rows");
    if (n_rows == 0) return KLD_OK;
    if (!flags_out) return fail(KLD_ERR_INVALID_ARG, "kld_eval_copy_row_flags: flags_out is NULL");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_copy_row_flags: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = wait_all(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_copy_row_flags: stream wait", e);
    e = hipMemcpyAsync(flags_out, h->retake + row_offset, static_cast<size_t>(n_rows), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return latch(h, "kld_eval_copy_row_flags: copy", e);
    return KLD_OK;
}

kld_status kld_eval_grad(kld_eval* h, const void* base, const void* quant, int64_t n_rows, int64_t row_offset,
                         double scale, void* grad_out, int32_t grad_dtype, void* stream) {
    const CallRange range_("kld_eval_grad");
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_grad: invalid or destroyed handle");
    if (n_rows < 0 || row_offset < 0) return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad: negative n_rows or row_offset");
    if (grad_dtype != KLD_DTYPE_F32 && grad_dtype != KLD_DTYPE_BF16)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad: grad_dtype must be KLD_DTYPE_F32 or KLD_DTYPE_BF16");
    if (!std::isfinite(scale)) return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad: scale is not finite");
    if (row_offset > h->max_rows || n_rows > h->max_rows - row_offset)
        return fail(KLD_ERR_RANGE, "kld_eval_grad: row_offset + n_rows exceeds max_rows");
    if (n_rows == 0) return KLD_OK;
    if (!base || !quant || !grad_out) return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad: base, quant or grad_out is NULL");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_grad: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = wait_all(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_grad: stream wait", e);
    e = kldk::launch_grad(h->base_type, h->quant_type, grad_dtype, base, quant, h->lse_b, h->lse_q, h->vocab, n_rows,
                          row_offset, static_cast<float>(scale), grad_out, s);
    if (e != hipSuccess) return latch(h, "kld_eval_grad: kernel launch", e);
    e = record(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_grad: event record", e);
    return KLD_OK;
}

kld_status kld_eval_topk_compress(kld_eval* h, const void* base, int64_t n_rows, int32_t k, int32_t* idx_out,
                                  float* logp_out, float* rest_out, void* stream) {
    const CallRange range_("kld_eval_topk_compress");
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_topk_compress: invalid or destroyed handle");
    if (n_rows < 0) return fail(KLD_ERR_INVALID_ARG, "kld_eval_topk_compress: negative n_rows");
    if (k < 1 || k > kldk::topk_max_k() || k > h->vocab)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_topk_compress: k must be in [1, min(vocab, 1024)]");
    if (n_rows == 0) return KLD_OK;
    if (!base || !idx_out || !logp_out || !rest_out)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_topk_compress: NULL pointer");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_topk_compress: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = kldk::launch_topk_compress(h->base_type, base, h->vocab, n_rows, k, idx_out, logp_out, rest_out, s);
    if (e != hipSuccess) return latch(h, "kld_eval_topk_compress: kernel launch", e);
    e = record(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_topk_compress: event record", e);
    return KLD_OK;
}

kld_status kld_eval_rows_topk(kld_eval* h, const int32_t* topk_idx, const float* topk_logp, const float* topk_rest,
                              int32_t k, const void* quant, int64_t n_rows, int64_t row_offset, float* kld_out,
                              uint8_t* match_out, int32_t* argmax_base_out, int32_t* argmax_quant_out, void* stream) {
    const CallRange range_("kld_eval_rows_topk");
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_rows_topk: invalid or destroyed handle");
    if (n_rows < 0 || row_offset < 0)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_rows_topk: negative n_rows or row_offset");
    if (k < 1 || k > kldk::topk_max_k() || k > h->vocab)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_rows_topk: k must be in [1, min(vocab, 1024)]");
    const int64_t lds = (h->vocab + 31) / 32 * 4 + kldk::kTopkEvalStaticLds;
    if (lds > h->max_lds)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_rows_topk: vocab too large for the on-chip token map of this device");
    if (row_offset > h->max_rows || n_rows > h->max_rows - row_offset)
        return fail(KLD_ERR_RANGE, "kld_eval_rows_topk: row_offset + n_rows exceeds max_rows");
    if (n_rows == 0) return KLD_OK;
    if (!topk_idx || !topk_logp || !topk_rest || !quant)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_rows_topk: NULL pointer");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_rows_topk: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    kldk::RowOut o{};
    o.kld = h->kld;
    o.match = h->match;
    o.argmax_b = h->argmax_b;
    o.argmax_q = h->argmax_q;
    o.lse_b = h->lse_b;
    o.lse_q = h->lse_q;
    o.logp_b = h->logp_b;
    o.logp_q = h->logp_q;
    o.dp = h->dp;
    o.tok_state = h->tok_state;
    o.topk_coef = h->topk_coef;
    o.kld_out = kld_out;
    o.match_out = match_out;
    o.argmax_b_out = argmax_base_out;
    o.argmax_q_out = argmax_quant_out;
    hipError_t e = kldk::launch_topk_eval(h->quant_type, topk_idx, topk_logp, topk_rest, k, quant, h->vocab, n_rows,
                                          row_offset, o, s);
    if (e != hipSuccess) return latch(h, "kld_eval_rows_topk: kernel launch", e);
    e = record(h, s, true);
    if (e != hipSuccess) return latch(h, "kld_eval_rows_topk: event record", e);
    return KLD_OK;
}

kld_status kld_eval_grad_topk(kld_eval* h, const int32_t* topk_idx, const float* topk_logp, int32_t k,
                              const void* quant, int64_t n_rows, int64_t row_offset, double scale, void* grad_out,
                              int32_t grad_dtype, void* stream) {
    const CallRange range_("kld_eval_grad_topk");
    if (!live(h)) return fail(KLD_ERR_BAD_HANDLE, "kld_eval_grad_topk: invalid or destroyed handle");
    if (n_rows < 0 || row_offset < 0)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad_topk: negative n_rows or row_offset");
    if (k < 1 || k > kldk::topk_max_k() || k > h->vocab)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad_topk: k must be in [1, min(vocab, 1024)]");
    if (grad_dtype != KLD_DTYPE_F32 && grad_dtype != KLD_DTYPE_BF16)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad_topk: grad_dtype must be KLD_DTYPE_F32 or KLD_DTYPE_BF16");
    if (!std::isfinite(scale)) return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad_topk: scale is not finite");
    if (row_offset > h->max_rows || n_rows > h->max_rows - row_offset)
        return fail(KLD_ERR_RANGE, "kld_eval_grad_topk: row_offset + n_rows exceeds max_rows");
    if (n_rows == 0) return KLD_OK;
    if (!topk_idx || !topk_logp || !quant || !grad_out)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_grad_topk: NULL pointer");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return latch(h, "kld_eval_grad_topk: set device", dg.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = wait_all(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_grad_topk: stream wait", e);
    e = kldk::launch_topk_grad(h->quant_type, grad_dtype, topk_idx, topk_logp, k, quant, h->vocab, n_rows,
                               row_offset, h->lse_q, h->topk_coef, static_cast<float>(scale), grad_out, s);
    if (e != hipSuccess) return latch(h, "kld_eval_grad_topk: kernel launch", e);
    e = record(h, s);
    if (e != hipSuccess) return latch(h, "kld_eval_grad_topk: event record", e);
    return KLD_OK;
}

kld_status kld_eval_compare_noalloc(const void* base, const void* quant, int64_t vocab, int64_t n_rows,
                                    int32_t base_dtype, int32_t quant_dtype, float* kld_out, uint8_t* match_out,
                                    int32_t* argmax_base_out, int32_t* argmax_quant_out,
                                    kld_eval_summary* summary_out, void* stream) {
    const CallRange range_("kld_eval_compare_noalloc");
    const char* who = "kld_eval_compare_noalloc";
    if (vocab < 1 || vocab > INT32_MAX) return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": vocab must be in [1, 2^31-1]");
    if ((base_dtype != KLD_DTYPE_F32 && base_dtype != KLD_DTYPE_BF16) ||
        (quant_dtype != KLD_DTYPE_F32 && quant_dtype != KLD_DTYPE_BF16))
        return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": dtype must be KLD_DTYPE_F32 or KLD_DTYPE_BF16");
    if (n_rows < 0) return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": negative n_rows");
    if (n_rows == 0) return fail(KLD_ERR_EMPTY, std::string(who) + ": zero rows");
    if (n_rows > kNoAllocMaxRows)
        return fail(KLD_ERR_RANGE, std::string(who) + ": n_rows exceeds the workspace limit of 4194304 rows per call");
    if (!base || !quant || !kld_out || !match_out || !summary_out)
        return fail(KLD_ERR_INVALID_ARG, std::string(who) + ": base, quant, kld_out, match_out or summary_out is NULL");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KLD_ERR_NO_DEVICE, hip_msg(who, e));
    kldk::Partial* parts = nullptr;
    kld_status st = noalloc_scratch(dev, &parts);
    if (st != KLD_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t sb = base_dtype == KLD_DTYPE_F32 ? 4 : 2;
    const size_t sq = quant_dtype == KLD_DTYPE_F32 ? 4 : 2;
    const int64_t per_launch = kldk::rows_max_per_launch();
    for (int64_t done = 0; done < n_rows; done += per_launch) {
        const int64_t n = std::min(per_launch, n_rows - done);
        kldk::RowOut o{};  // no handle: per-token results straight into the caller's arrays
        o.kld = kld_out;
        o.match = match_out;
        o.argmax_b = argmax_base_out;
        o.argmax_q = argmax_quant_out;
        const char* pb = static_cast<const char*>(base) + static_cast<size_t>(done) * vocab * sb;
        const char* pq = static_cast<const char*>(quant) + static_cast<size_t>(done) * vocab * sq;
        // the launch shape is keyed on the call's row count: the results equal
        // those of a handle created with max_rows = n_rows
        e = kldk::launch_rows(base_dtype, quant_dtype, pb, pq, vocab, n, done, n_rows, o, s);
        if (e != hipSuccess) return fail(KLD_ERR_HIP, hip_msg("kld_eval_compare_noalloc: row kernel launch", e));
    }
    const kldk::RowIn in{kld_out, match_out, nullptr, nullptr, nullptr, nullptr};
    e = kldk::launch_reduce_whole(in, n_rows, parts, summary_out, s);
    if (e != hipSuccess) return fail(KLD_ERR_HIP, hip_msg("kld_eval_compare_noalloc: reduction launch", e));
    return KLD_OK;
}

kld_status kld_eval_read_probe(const void* a, const void* b, int64_t n_rows, int64_t row_bytes,
                               int32_t waves_per_row, uint32_t* sink, void* stream, void* start_event,
                               void* stop_event) {
    const CallRange range_("kld_eval_read_probe");
    if (n_rows < 0) return fail(KLD_ERR_INVALID_ARG, "kld_eval_read_probe: negative n_rows");
    if (row_bytes <= 0 || row_bytes % 16 != 0)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_read_probe: row_bytes must be a positive multiple of 16");
    if (waves_per_row != 1 && waves_per_row != 4)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_read_probe: waves_per_row must be 1 or 4");
    if (n_rows == 0) return KLD_OK;
    if (!a || !sink) return fail(KLD_ERR_INVALID_ARG, "kld_eval_read_probe: a or sink is NULL");
    if (reinterpret_cast<uintptr_t>(a) % 16 != 0 || reinterpret_cast<uintptr_t>(b) % 16 != 0)
        return fail(KLD_ERR_INVALID_ARG, "kld_eval_read_probe: a and b must be 16-byte aligned");
    const hipError_t e =
        kldk::launch_read_probe(a, b, n_rows, row_bytes, waves_per_row, sink, static_cast<hipStream_t>(stream),
                                static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
    if (e != hipSuccess) return fail(KLD_ERR_HIP, hip_msg("kld_eval_read_probe: kernel launch", e));
    return KLD_OK;
}

kld_status kld_eval_destroy(kld_eval* h) {
    const CallRange range_("kld_eval_destroy");
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
