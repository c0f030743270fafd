// C ABI of libwqmm: argument validation, M routing, route counters, launches.
// The contract (layouts, ownership, errors) is documented in include/wqmm.h.
#include "../../include/wqmm.h"
#include "wq_internal.h"

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

namespace wq {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];
hipError_t g_dev_err[kMaxDevices];

std::atomic<int> g_forced_route{WQ_ROUTE_AUTO};
std::atomic<uint64_t> g_route_count[6];

int trace_flag() {
    static const int v = [] {
        const char *e = std::getenv("WQ_TRACE");
        return (e && e[0] && std::strcmp(e, "0") != 0) ? 1 : 0;
    }();
    return v;
}
}  // namespace

bool trace_enabled() { return trace_flag() != 0; }

hipError_t device_info(DeviceInfo *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_dev_once[dev], [dev] {
        int cus = 0;
        g_dev_err[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        g_dev[dev].cus = cus > 0 ? cus : 1;
    });
    *out = g_dev[dev];
    return g_dev_err[dev];
}

namespace {
// One cached buffer per (device, stream): work on one stream is ordered by the
// stream itself, so a reuse needs no event (an event record costs about 3 us
// of GPU time on MI355X).  Up to kStreamSlots streams per device are cached.
struct StreamScratch {
    bool live = false;
    hipStream_t stream = nullptr;
    void *ptr = nullptr;
    size_t bytes = 0;
};
struct DevScratch {
    std::mutex mu;
    StreamScratch slot[kStreamSlots];
};
DevScratch g_scratch[kMaxDevices];
}  // namespace

hipError_t ScratchLease::acquire(size_t bytes, hipStream_t s, void **ptr) {
    *ptr = nullptr;
    s_ = s;
    hipError_t e = hipGetDevice(&dev_);
    if (e != hipSuccess) return e;
    if (dev_ < 0 || dev_ >= kMaxDevices) return hipErrorInvalidDevice;
    DevScratch &d = g_scratch[dev_];
    StreamScratch *slot = nullptr;
    if (bytes <= kScratchCacheBytes) {
        d.mu.lock();
        held_ = true;
        for (StreamScratch &x : d.slot)
            if (x.live && x.stream == s) slot = &x;
        if (!slot)
            for (StreamScratch &x : d.slot)
                if (!x.live) {
                    slot = &x;
                    slot->live = true;
                    slot->stream = s;
                    break;
                }
        if (!slot) {  // every slot taken by another stream
            d.mu.unlock();
            held_ = false;
        }
    }
    if (!slot) {
        e = hipMallocAsync(&priv_, bytes, s);
        if (e == hipSuccess) *ptr = priv_;
        return e;
    }
    if (bytes > slot->bytes) {
        // Grow (at least double) on this stream, after its earlier uses.
        size_t want = slot->bytes * 2 > bytes ? slot->bytes * 2 : bytes;
        if (want > kScratchCacheBytes) want = kScratchCacheBytes;
        want = (want + 4095) & ~size_t(4095);
        if (slot->ptr) {
            e = hipFreeAsync(slot->ptr, s);
            slot->ptr = nullptr;
            slot->bytes = 0;
            if (e != hipSuccess) return e;
        }
        e = hipMallocAsync(&slot->ptr, want, s);
        if (e != hipSuccess) {
            slot->ptr = nullptr;
            return e;
        }
        slot->bytes = want;
    }
    *ptr = slot->ptr;
    slot_ = static_cast<int>(slot - d.slot);
    return hipSuccess;
}

hipError_t ScratchLease::release() {
    hipError_t e = hipSuccess;
    if (priv_) {
        e = hipFreeAsync(priv_, s_);
        priv_ = nullptr;
    }
    if (held_) {
        held_ = false;
        g_scratch[dev_].mu.unlock();
    }
    return e;
}

ScratchLease::~ScratchLease() { (void)release(); }

// The allocation-free workspace: one fixed array per GPU, in device memory the
// code object brings along when the library is loaded on that GPU.  Host code
// never uses the array's name as an address: it takes the device address with
// hipGetSymbolAddress once per device (that device current) and passes that.
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {
std::once_flag g_noalloc_once[kMaxDevices];
void *g_noalloc_ptr[kMaxDevices];
hipError_t g_noalloc_err[kMaxDevices];
}  // namespace

// Device address of the current device's workspace (looked up on its first use).
hipError_t noalloc_workspace(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_noalloc_once[dev], [dev] {
        void *p = nullptr;
        g_noalloc_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_noalloc_ptr[dev] = g_noalloc_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_noalloc_err[dev] != hipSuccess) return g_noalloc_err[dev];
    *ptr = g_noalloc_ptr[dev];
    return *ptr ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace wq

namespace {

bool mul_ok(int64_t x, int64_t y, int64_t *out) { return !__builtin_mul_overflow(x, y, out); }

bool overlaps(const void *p, int64_t pbytes, const void *q, int64_t qbytes) {
    if (!p || !q || pbytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
    return a0 < b0 + static_cast<uintptr_t>(qbytes) && b0 < a0 + static_cast<uintptr_t>(pbytes);
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

bool known_format(int fmt) { return fmt == WQ_FMT_F16 || fmt == WQ_FMT_Q8_0 || fmt == WQ_FMT_Q4_0; }

bool known_epilogue(int epi) { return epi == WQ_EPI_NONE || epi == WQ_EPI_RESIDUAL || epi == WQ_EPI_SWIGLU; }

// Validates a product call.  Returns WQ_OK with *noop = true when nothing is
// to be done (m == 0 or n == 0), WQ_OK with *noop = false when a launch
// follows, or an error status.  The weights have n rows, or 2n for SWIGLU.
int validate(const float *a, const void *b, const float *c, int64_t m, int64_t n, int64_t k, int fmt,
             bool *noop, int epi = WQ_EPI_NONE) {
    *noop = false;
    if (!known_epilogue(epi)) return WQ_ERR_EPILOGUE;
    if (!known_format(fmt)) return WQ_ERR_FORMAT;
    if (m < 0 || n < 0 || k < 0) return WQ_ERR_SHAPE;
    if (m == 0 || n == 0) {
        *noop = true;
        return WQ_OK;
    }
    if (fmt != WQ_FMT_F16 && (k == 0 || k % 32 != 0)) return WQ_ERR_K;
    int64_t a_elems, c_elems, b_bytes, a_bytes, c_bytes, nw;
    if (!mul_ok(n, epi == WQ_EPI_SWIGLU ? 2 : 1, &nw)) return WQ_ERR_SHAPE;
    if (!mul_ok(m, k, &a_elems) || !mul_ok(a_elems, 4, &a_bytes)) return WQ_ERR_SHAPE;
    if (!mul_ok(m, n, &c_elems) || !mul_ok(c_elems, 4, &c_bytes)) return WQ_ERR_SHAPE;
    int64_t glu_bytes;  // the M == 1 route's scratch: [m, 2n] f32 sums
    if (epi == WQ_EPI_SWIGLU && !mul_ok(c_bytes, 2, &glu_bytes)) return WQ_ERR_SHAPE;
    if (fmt == WQ_FMT_F16) {
        int64_t nk;
        if (!mul_ok(nw, k, &nk) || !mul_ok(nk, 2, &b_bytes)) return WQ_ERR_SHAPE;
    } else {
        if (!mul_ok(nw, (k / 32) * (fmt == WQ_FMT_Q8_0 ? 34 : 18), &b_bytes)) return WQ_ERR_SHAPE;
    }
    if (!c) return WQ_ERR_NULL;
    if (k > 0 && (!a || !b)) return WQ_ERR_NULL;
    if (!aligned(c, 4) || (a && !aligned(a, 4)) || (b && !aligned(b, 2))) return WQ_ERR_ALIGN;
    if (k > 0 && (overlaps(c, c_bytes, a, a_bytes) || overlaps(c, c_bytes, b, b_bytes))) return WQ_ERR_ALIAS;
    return WQ_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_LAUNCH; }

// M == 1: the decode GEMV; small M: weight-streaming kernels; larger M: the
// LDS-tiled GEMM on the f16 matrix cores (A as hi / lo halves).  Quantized
// weights with K % 256 == 0 take the f16 matrix-core stream for M <= 16 (its
// time hardly depends on M: measured on MI355X at (N, K) = (11008, 4096) and
// (4096, 11008) it beats the tiled products up to M = 16); other quantized
// shapes take the fp32 small-M kernel up to M = 4, f16 weights up to M = 8
// (crossovers measured on the same shapes).  Calls the tiled f16 product cannot
// take (K % 32 != 0, misaligned a or b) go to the fp32 GEMM at launch.
constexpr int64_t kSkinnyRows = 16;  // rows of A per small-M launch
int auto_route(int64_t m, int64_t k, int fmt) {
    if (m <= 1) return WQ_ROUTE_GEMV;
    if (fmt == WQ_FMT_F16) return m <= 8 ? WQ_ROUTE_SKINNY : WQ_ROUTE_GEMM_HL;
    if (k % 256 == 0) return m <= 16 ? WQ_ROUTE_STREAM : WQ_ROUTE_GEMM_HL;  // alignment is checked at launch
    return m <= 4 ? WQ_ROUTE_SKINNY : WQ_ROUTE_GEMM_HL;  // Q4_0 as Q8_0
}
bool known_route(int r) {
    return r == WQ_ROUTE_GEMV || r == WQ_ROUTE_GEMM || r == WQ_ROUTE_SKINNY || r == WQ_ROUTE_STREAM ||
           r == WQ_ROUTE_GEMM_HL;
}

// Kernel-side epilogue code of a wq_epilogue value.
int kernel_epi(int epi) {
    return epi == WQ_EPI_RESIDUAL ? wq::kEpiResidual : epi == WQ_EPI_SWIGLU ? wq::kEpiGlu : wq::kEpiNone;
}

// The M rule, except that two Q8_0 rows of A the register-chunk GEMV takes in
// one launch with at most three units per wave go to the GEMV route (faster
// than the weight stream there).  a and b may be NULL: the shape alone decides.
int pick_route(const float *a, const void *b, int64_t m, int64_t n, int64_t k, int fmt, int epi) {
    const int route = auto_route(m, k, fmt);
    if (route == WQ_ROUTE_STREAM &&
        wq::gemv_q_rows_auto(a, static_cast<const uint8_t *>(b), fmt, m, n, k, kernel_epi(epi)))
        return WQ_ROUTE_GEMV;
    return route;
}

// The GEMV route (M == 1; 2 <= M <= 4 quantized rows where the register-chunk
// kernel takes them in one launch; forced otherwise): else one GEMV launch
// per row of A, each applying the epilogue itself.
int run_gemv(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, hipStream_t s,
             int epi) {
    const int ke = kernel_epi(epi);
    const auto *b8 = static_cast<const uint8_t *>(b);
    if (fmt != WQ_FMT_F16 && m >= 2) {
        hipError_t e = hipSuccess;
        if (wq::launch_gemv_q_rows(a, b8, fmt, c, m, n, k, s, ke, &e)) {
            if (e != hipSuccess) return WQ_ERR_LAUNCH;
            wq::g_route_count[WQ_ROUTE_GEMV].fetch_add(1, std::memory_order_relaxed);
            return WQ_OK;
        }
    }
    for (int64_t i = 0; i < m; ++i) {
        const float *ai = a + i * k;
        float *ci = c + i * n;
        hipError_t e = (fmt == WQ_FMT_F16)    ? wq::launch_gemv_f16(ai, static_cast<const uint16_t *>(b), ci, n, k, s, ke)
                       : (fmt == WQ_FMT_Q8_0) ? wq::launch_gemv_q8_0(ai, b8, ci, n, k, s, ke)
                                              : wq::launch_gemv_q4_0(ai, b8, ci, n, k, s, ke);
        if (e != hipSuccess) return WQ_ERR_LAUNCH;
        wq::g_route_count[WQ_ROUTE_GEMV].fetch_add(1, std::memory_order_relaxed);
    }
    return WQ_OK;
}

int run_gemm(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, hipStream_t s,
             int epi) {
    hipError_t e = wq::launch_gemm(a, b, fmt, c, m, n, k, s, kernel_epi(epi));
    if (e != hipSuccess) return WQ_ERR_LAUNCH;
    wq::g_route_count[WQ_ROUTE_GEMM].fetch_add(1, std::memory_order_relaxed);
    return WQ_OK;
}

// The tiled product on the f16 matrix cores where it applies (K % 32 == 0,
// 16-byte aligned a and b, quantized weights under 2 GiB); anything else takes
// the fp32 GEMM.
int run_gemm_hl(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, hipStream_t s,
                int epi) {
    if (!wq::hgemm_ok(a, b, fmt, m, epi == WQ_EPI_SWIGLU ? 2 * n : n, k)) return run_gemm(a, b, c, m, n, k, fmt, s, epi);
    if (wq::launch_hgemm(a, b, fmt, c, m, n, k, s, kernel_epi(epi)) != hipSuccess) return WQ_ERR_LAUNCH;
    wq::g_route_count[WQ_ROUTE_GEMM_HL].fetch_add(1, std::memory_order_relaxed);
    return WQ_OK;
}

// One small-M launch per block of up to kSkinnyRows rows of A: the staged
// quantized kernel where it applies (K % 256 == 0, 16-byte aligned operands),
// else the general one.
int run_skinny(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, hipStream_t s,
               int epi) {
    for (int64_t i = 0; i < m; i += kSkinnyRows) {
        const int64_t rows = m - i < kSkinnyRows ? m - i : kSkinnyRows;
        const float *ai = a + i * k;
        hipError_t e = wq::smallm_ok(ai, b, fmt, rows, k)
                           ? wq::launch_smallm(ai, b, fmt, c + i * n, rows, n, k, s, kernel_epi(epi))
                           : wq::launch_skinny(ai, b, fmt, c + i * n, rows, n, k, s, kernel_epi(epi));
        if (e != hipSuccess) return WQ_ERR_LAUNCH;
        wq::g_route_count[WQ_ROUTE_SKINNY].fetch_add(1, std::memory_order_relaxed);
    }
    return WQ_OK;
}

// The f16 matrix-core weight stream, one launch per block of up to 16 rows of
// A, where it applies (Q8_0 / Q4_0, K % 256 == 0, 16-byte aligned operands, no
// SwiGLU); anything else takes the small-M route.
int run_stream(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, hipStream_t s,
               int epi) {
    const int ke = kernel_epi(epi);
    bool ok = ke != wq::kEpiGlu;
    for (int64_t i = 0; ok && i < m; i += kSkinnyRows)
        ok = wq::wstream_ok(a + i * k, b, fmt, m - i < kSkinnyRows ? m - i : kSkinnyRows, n, k);
    if (!ok) return run_skinny(a, b, c, m, n, k, fmt, s, epi);
    for (int64_t i = 0; i < m; i += kSkinnyRows) {
        const int64_t rows = m - i < kSkinnyRows ? m - i : kSkinnyRows;
        if (wq::launch_wstream(a + i * k, b, fmt, c + i * n, rows, n, k, s, ke) != hipSuccess) return WQ_ERR_LAUNCH;
        wq::g_route_count[WQ_ROUTE_STREAM].fetch_add(1, std::memory_order_relaxed);
    }
    return WQ_OK;
}

// K == 0 (f16 only): the empty sum, c = 0.
int run_zero(float *c, int64_t m, int64_t n, hipStream_t s) {
    return status_of(wq::launch_fill_zero(c, m * n, s));
}

// Validated product with an epilogue on the route the M rule (or the forced
// route) picks.
int run_routed(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, int epi,
               hipStream_t s) {
    if (k == 0) return epi == WQ_EPI_RESIDUAL ? WQ_OK : run_zero(c, m, n, s);  // silu(0) * 0 = 0
    int route = wq::g_forced_route.load(std::memory_order_relaxed);
    if (route == WQ_ROUTE_AUTO) route = pick_route(a, b, m, n, k, fmt, epi);
    if (route == WQ_ROUTE_GEMV) return run_gemv(a, b, c, m, n, k, fmt, s, epi);
    if (route == WQ_ROUTE_SKINNY) return run_skinny(a, b, c, m, n, k, fmt, s, epi);
    if (route == WQ_ROUTE_STREAM) return run_stream(a, b, c, m, n, k, fmt, s, epi);
    if (route == WQ_ROUTE_GEMM_HL) return run_gemm_hl(a, b, c, m, n, k, fmt, s, epi);
    return run_gemm(a, b, c, m, n, k, fmt, s, epi);
}

}  // namespace

extern "C" {

int wq_abi_version(void) { return 108; }

const char *wq_status_str(int status) {
    switch (status) {
        case WQ_OK: return "ok";
        case WQ_ERR_NULL: return "a required pointer is NULL";
        case WQ_ERR_SHAPE: return "negative dimension or byte count overflow";
        case WQ_ERR_K: return "Q8_0 needs K > 0 and K % 32 == 0";
        case WQ_ERR_FORMAT: return "unknown weight format";
        case WQ_ERR_ALIGN: return "misaligned pointer (a, c need 4 bytes; b needs 2)";
        case WQ_ERR_LAUNCH: return "HIP kernel launch failed";
        case WQ_ERR_ALIAS: return "output overlaps an input";
        case WQ_ERR_ROUTE: return "unknown route";
        case WQ_ERR_EPILOGUE: return "unknown epilogue";
        case WQ_ERR_TOPK: return "top-k count outside 1 .. WQ_TOPK_MAX";
        case WQ_ERR_WORKSPACE: return "request needs more than the fixed no-allocation workspace";
        default: return "unknown status";
    }
}

int wq_gemv_f16(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k, void *stream) {
    bool noop;
    int st = validate(a, b, c, 1, n, k, WQ_FMT_F16, &noop);
    if (st != WQ_OK || noop) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 0) return run_zero(c, 1, n, s);
    return run_gemv(a, b, c, 1, n, k, WQ_FMT_F16, s, WQ_EPI_NONE);
}

int wq_gemv_q8_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, void *stream) {
    bool noop;
    int st = validate(a, b, c, 1, n, k, WQ_FMT_Q8_0, &noop);
    if (st != WQ_OK || noop) return st;
    return run_gemv(a, b, c, 1, n, k, WQ_FMT_Q8_0, static_cast<hipStream_t>(stream), WQ_EPI_NONE);
}

int wq_gemv_q4_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, void *stream) {
    bool noop;
    int st = validate(a, b, c, 1, n, k, WQ_FMT_Q4_0, &noop);
    if (st != WQ_OK || noop) return st;
    return run_gemv(a, b, c, 1, n, k, WQ_FMT_Q4_0, static_cast<hipStream_t>(stream), WQ_EPI_NONE);
}

int wq_gemm_f16(const float *a, const uint16_t *b, float *c, int64_t m, int64_t n, int64_t k, void *stream) {
    bool noop;
    int st = validate(a, b, c, m, n, k, WQ_FMT_F16, &noop);
    if (st != WQ_OK || noop) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 0) return run_zero(c, m, n, s);
    return run_gemm(a, b, c, m, n, k, WQ_FMT_F16, s, WQ_EPI_NONE);
}

int wq_gemm_q8_0(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, void *stream) {
    bool noop;
    int st = validate(a, b, c, m, n, k, WQ_FMT_Q8_0, &noop);
    if (st != WQ_OK || noop) return st;
    return run_gemm(a, b, c, m, n, k, WQ_FMT_Q8_0, static_cast<hipStream_t>(stream), WQ_EPI_NONE);
}

int wq_gemm_q4_0(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, void *stream) {
    bool noop;
    int st = validate(a, b, c, m, n, k, WQ_FMT_Q4_0, &noop);
    if (st != WQ_OK || noop) return st;
    return run_gemm(a, b, c, m, n, k, WQ_FMT_Q4_0, static_cast<hipStream_t>(stream), WQ_EPI_NONE);
}

int wq_matmul(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, void *stream) {
    return wq_matmul_ex(a, b, c, m, n, k, fmt, WQ_EPI_NONE, stream);
}

int wq_matmul_ex(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt, int epi,
                 void *stream) {
    bool noop;
    int st = validate(a, b, c, m, n, k, fmt, &noop, epi);
    if (st != WQ_OK || noop) return st;
    return run_routed(a, b, c, m, n, k, fmt, epi, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {
int validate_lm_head_topk(const float *a, const void *b, int64_t n, int64_t k, int fmt, int topk,
                          const float *vals, const uint32_t *ids) {
    if (!known_format(fmt)) return WQ_ERR_FORMAT;
    if (n < 0 || k < 0) return WQ_ERR_SHAPE;
    if (topk < 1 || topk > WQ_TOPK_MAX) return WQ_ERR_TOPK;
    if (n >= static_cast<int64_t>(WQ_TOPK_NO_ID)) return WQ_ERR_SHAPE;  // ids must stay below the sentinel
    if (fmt != WQ_FMT_F16 && (k == 0 || k % 32 != 0)) return WQ_ERR_K;
    int64_t nk, b_bytes;
    if (fmt == WQ_FMT_F16) {
        if (!mul_ok(n, k, &nk) || !mul_ok(nk, 2, &b_bytes)) return WQ_ERR_SHAPE;
    } else if (!mul_ok(n, (k / 32) * (fmt == WQ_FMT_Q8_0 ? 34 : 18), &b_bytes)) {
        return WQ_ERR_SHAPE;
    }
    if (!vals || !ids) return WQ_ERR_NULL;
    if (n > 0 && k > 0 && (!a || !b)) return WQ_ERR_NULL;
    if (!aligned(vals, 4) || !aligned(ids, 4) || (a && !aligned(a, 4)) || (b && !aligned(b, 2))) return WQ_ERR_ALIGN;
    const int64_t a_bytes = 4 * k, o_bytes = 4LL * topk;
    if (overlaps(vals, o_bytes, ids, o_bytes)) return WQ_ERR_ALIAS;
    for (const void *o : {static_cast<const void *>(vals), static_cast<const void *>(ids)})
        if (overlaps(o, o_bytes, a, a_bytes) || overlaps(o, o_bytes, b, b_bytes)) return WQ_ERR_ALIAS;
    return WQ_OK;
}
}  // namespace

extern "C" {

int wq_lm_head_topk(const float *a, const void *b, int64_t n, int64_t k, int fmt, int topk, float *vals,
                    uint32_t *ids, void *stream) {
    const int st = validate_lm_head_topk(a, b, n, k, fmt, topk, vals, ids);
    if (st != WQ_OK) return st;
    // n == 0 or K == 0 still go through the kernels: the lists are then all
    // sentinels (n == 0) or all logits are 0 (K == 0, f16).
    return status_of(wq::launch_lm_head_topk(a, b, fmt, n, k, topk, vals, ids, static_cast<hipStream_t>(stream)));
}

int wq_lm_head_topk_noalloc(const float *a, const void *b, int64_t n, int64_t k, int fmt, int topk, float *vals,
                            uint32_t *ids, void *stream) {
    const int st = validate_lm_head_topk(a, b, n, k, fmt, topk, vals, ids);
    if (st != WQ_OK) return st;
    wq::DeviceInfo di;
    if (wq::device_info(&di) != hipSuccess) return WQ_ERR_LAUNCH;
    const size_t need = wq::lm_head_topk_scratch_bytes(a, b, fmt, n, k, topk, di.cus);
    if (need > wq::kNoAllocBytes) return WQ_ERR_WORKSPACE;
    void *ws = nullptr;
    if (wq::noalloc_workspace(&ws) != hipSuccess) return WQ_ERR_LAUNCH;
    return status_of(wq::launch_lm_head_topk(a, b, fmt, n, k, topk, vals, ids, static_cast<hipStream_t>(stream), ws,
                                             wq::kNoAllocBytes));
}

size_t wq_noalloc_workspace_bytes(void) { return wq::kNoAllocBytes; }

int wq_topk(const float *logits, int64_t n, int topk, float *vals, uint32_t *ids, void *stream) {
    if (n < 0) return WQ_ERR_SHAPE;
    if (topk < 1 || topk > WQ_TOPK_MAX) return WQ_ERR_TOPK;
    if (n >= static_cast<int64_t>(WQ_TOPK_NO_ID)) return WQ_ERR_SHAPE;
    if (!vals || !ids || (n > 0 && !logits)) return WQ_ERR_NULL;
    if (!aligned(vals, 4) || !aligned(ids, 4) || (logits && !aligned(logits, 4))) return WQ_ERR_ALIGN;
    const int64_t o_bytes = 4LL * topk;
    if (overlaps(vals, o_bytes, ids, o_bytes) || overlaps(vals, o_bytes, logits, 4 * n) ||
        overlaps(ids, o_bytes, logits, 4 * n))
        return WQ_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    wq::ScratchLease lease;
    void *scratch = nullptr;
    if (lease.acquire(static_cast<size_t>(wq::kTopkGroups) * topk * sizeof(wq::TopkCand), s, &scratch) !=
        hipSuccess)
        return WQ_ERR_LAUNCH;
    int st = status_of(wq::launch_topk_merge(nullptr, 0, logits, n, topk, static_cast<wq::TopkCand *>(scratch),
                                             vals, ids, s));
    if (lease.release() != hipSuccess && st == WQ_OK) st = WQ_ERR_LAUNCH;
    return st;
}

int wq_decode_attention(const float *q, const void *k_cache, const void *v_cache, float *out, int64_t cache_len,
                        int head_dim, int num_q_heads, int num_kv_heads, int kv_fmt, float scale, void *stream) {
    if (kv_fmt != WQ_KV_F32 && kv_fmt != WQ_KV_F16) return WQ_ERR_FORMAT;
    if (cache_len < 0 || num_q_heads < 1 || num_kv_heads < 1) return WQ_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return WQ_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > WQ_ATTN_MAX_GROUP) return WQ_ERR_SHAPE;
    const int64_t elem = kv_fmt == WQ_KV_F32 ? 4 : 2;
    int64_t cache_elems, cache_bytes;
    if (!mul_ok(cache_len, static_cast<int64_t>(num_kv_heads) * head_dim, &cache_elems) ||
        !mul_ok(cache_elems, elem, &cache_bytes))
        return WQ_ERR_SHAPE;
    if (!q || !out || (cache_len > 0 && (!k_cache || !v_cache))) return WQ_ERR_NULL;
    if (!aligned(q, 4) || !aligned(out, 4) || (k_cache && !aligned(k_cache, 16)) ||
        (v_cache && !aligned(v_cache, 16)))
        return WQ_ERR_ALIGN;
    const int64_t qo_bytes = static_cast<int64_t>(num_q_heads) * head_dim * 4;
    if (overlaps(out, qo_bytes, q, qo_bytes) || overlaps(out, qo_bytes, k_cache, cache_bytes) ||
        overlaps(out, qo_bytes, v_cache, cache_bytes))
        return WQ_ERR_ALIAS;
    return status_of(wq::launch_decode_attention(q, k_cache, v_cache, kv_fmt, out, cache_len, head_dim, num_q_heads,
                                                 num_kv_heads, scale, static_cast<hipStream_t>(stream)));
}

int wq_pack_f16(const float *w, uint16_t *out, int64_t count, void *stream) {
    if (count < 0) return WQ_ERR_SHAPE;
    if (count == 0) return WQ_OK;
    if (count > INT64_MAX / 4) return WQ_ERR_SHAPE;
    if (!w || !out) return WQ_ERR_NULL;
    if (!aligned(w, 4) || !aligned(out, 2)) return WQ_ERR_ALIGN;
    if (overlaps(w, count * 4, out, count * 2)) return WQ_ERR_ALIAS;
    return status_of(wq::launch_pack_f16(w, out, count, static_cast<hipStream_t>(stream)));
}

int wq_quantize_q8_0(const float *w, uint8_t *out, int64_t count, void *stream) {
    if (count < 0) return WQ_ERR_SHAPE;
    if (count % 32 != 0) return WQ_ERR_K;
    if (count == 0) return WQ_OK;
    if (count > INT64_MAX / 4) return WQ_ERR_SHAPE;
    if (!w || !out) return WQ_ERR_NULL;
    if (!aligned(w, 4) || !aligned(out, 2)) return WQ_ERR_ALIGN;
    if (overlaps(w, count * 4, out, count / 32 * 34)) return WQ_ERR_ALIAS;
    return status_of(wq::launch_quantize_q8_0(w, out, count, static_cast<hipStream_t>(stream)));
}

int wq_read_probe(const void *p, int64_t bytes, uint32_t *out, int variant, void *stream) {
    if (bytes < 0 || bytes % 16 != 0 || variant < 0 || variant > 3) return WQ_ERR_SHAPE;
    if (bytes == 0) return WQ_OK;
    if (!p || !out) return WQ_ERR_NULL;
    if (!aligned(p, 16) || !aligned(out, 4)) return WQ_ERR_ALIGN;
    if (overlaps(out, (bytes + 1023) / 1024 * 4, p, bytes)) return WQ_ERR_ALIAS;
    return status_of(wq::launch_read_probe(p, bytes, out, variant, static_cast<hipStream_t>(stream)));
}

int wq_route_for(int64_t m, int64_t n, int64_t k, int fmt) {
    if (!known_format(fmt)) return -WQ_ERR_FORMAT;
    if (m < 0 || n < 0 || k < 0) return -WQ_ERR_SHAPE;
    if (fmt != WQ_FMT_F16 && m > 0 && n > 0 && (k == 0 || k % 32 != 0)) return -WQ_ERR_K;
    return pick_route(nullptr, nullptr, m, n, k, fmt, WQ_EPI_NONE);
}

int wq_gemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits) {
    if (!known_format(fmt)) return WQ_ERR_FORMAT;
    if (m <= 0 || n <= 0 || k <= 0 || cus <= 0) return WQ_ERR_SHAPE;
    if (fmt != WQ_FMT_F16 && k % 32 != 0) return WQ_ERR_K;
    if (!bm || !bn || !splits) return WQ_ERR_NULL;
    wq::gemm_plan(m, n, k, fmt, cus, bm, bn, splits);
    return WQ_OK;
}

int wq_set_gemm_plan(int bm, int bn, int splits) {
    return wq::set_gemm_plan_override(bm, bn, splits) ? WQ_OK : WQ_ERR_SHAPE;
}

int wq_hgemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits) {
    if (!known_format(fmt)) return WQ_ERR_FORMAT;
    if (m <= 0 || n <= 0 || k <= 0 || cus <= 0) return WQ_ERR_SHAPE;
    if (k % 32 != 0) return WQ_ERR_K;
    if (!bm || !bn || !splits) return WQ_ERR_NULL;
    wq::hgemm_plan(m, n, k, fmt, cus, bm, bn, splits);
    return WQ_OK;
}

int wq_set_hgemm_plan(int bm, int bn, int splits) {
    return wq::set_hgemm_plan_override(bm, bn, splits) ? WQ_OK : WQ_ERR_SHAPE;
}

int wq_set_gemv_plan(int rb, int nf, int nr) {
    return wq::set_gemv_plan_override(rb, nf, nr) ? WQ_OK : WQ_ERR_SHAPE;
}

int wq_set_stream_plan(int shape, int splits) {
    return wq::set_wstream_plan_override(shape, splits) ? WQ_OK : WQ_ERR_SHAPE;
}

int wq_set_attn_partition(int64_t tokens) {
    if (tokens < 0) return WQ_ERR_SHAPE;
    wq::set_attn_partition_override(tokens);
    return WQ_OK;
}

int wq_set_forced_route(int route) {
    if (route != WQ_ROUTE_AUTO && !known_route(route)) return -WQ_ERR_ROUTE;
    return wq::g_forced_route.exchange(route);
}

uint64_t wq_route_count(int route) {
    if (!known_route(route)) return 0;
    return wq::g_route_count[route].load(std::memory_order_relaxed);
}

void wq_reset_route_counts(void) {
    for (auto &x : wq::g_route_count) x.store(0, std::memory_order_relaxed);
}

}  // extern "C"
