// C ABI of the gfx950 EXL3 trellis tile encoder: context, validation,
// batching of the kernel chain within the scratch bound, and the host-side
// golden-section scale search.
//
// Sources: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
// section 1 (the pass-1 / traceback / pass-2 / traceback chain per tile),
// section 2 (scratch bounded up front, admission before any work, batches
// that leave results unchanged), section 8 (rms and the wrapped-diagonal tile
// sample with the highest- and lowest-energy tiles for the scale search);
// "JEV-9B EXL3 K=2 (mul1) Checkpoint" model card, section 2 (golden-section
// scale search).  Host control runs in binary64 with a fixed summation order
// (ascending tile index), so the chosen scale does not depend on batching.
#include "exl3.h"
#include "exl3_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <vector>

// ---- Device scratch of exl3_encode_tiles_noalloc ----
// One batch of the encode chain: the backpointers of up to 256 tiles (K = 1..3,
// 1,044,480 B each) or 512 tiles (K = 4, 522,240 B each), then the pass-1 end
// state (uint16), X (uint16) and pass-2 path cost (float) of up to 512 tiles.
// Each GPU the library is loaded on holds its own copy until the process ends.
// Host code never passes this name to a kernel: it is a host-side stand-in;
// the device address comes from hipGetSymbolAddress, looked up once per device
// when a context is created there (noalloc_setup below).
constexpr size_t kNoAllocBpBytes =
    (size_t)EXL3_NOALLOC_MAX_TILES * exl3::kSlots * exl3::kLanes * sizeof(uint32_t);
static_assert((size_t)EXL3_NOALLOC_MAX_TILES_K4 * exl3::kSlots * exl3::kLanes * sizeof(uint16_t) ==
                  kNoAllocBpBytes, "K = 4 batches fill the same backpointer bytes");
constexpr size_t kNoAllocBookTiles = EXL3_NOALLOC_MAX_TILES_K4;
constexpr size_t kNoAllocBytes = kNoAllocBpBytes + kNoAllocBookTiles * (2 + 2 + 4);
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

// State of a golden-section scale search run on the device: the bracket
// [a, b], its two points and their scores, the reductions done, which point
// the next score belongs to (0: p, 1: q), and the scale of the next probe
// (after the last reduction: the result).
struct GssDev {
    double a, b, p, q, fp, fq;
    int it, pending;
    float scale;
};

struct exl3_ctx {
    int device = 0;
    int n_cu = 256;
    hipStream_t stream = nullptr;
    // second stream (default priority) for the last partial round of a
    // scale-search probe, with the events that order it against `stream`
    hipStream_t aux = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // orders a new stream after the work already enqueued on the old one
    hipEvent_t ev_switch = nullptr;
    size_t scratch_limit = 0;
    uint16_t *d_levels = nullptr;
    void *d_bp = nullptr;
    size_t bp_cap = 0;
    uint16_t *d_end = nullptr;
    uint16_t *d_X = nullptr;
    float *d_cost = nullptr;
    size_t small_cap = 0;
    int32_t *d_idx = nullptr;
    size_t idx_cap = 0;
    float *d_wreg = nullptr;
    size_t wreg_cap = 0;
    float *d_sumsq = nullptr;
    size_t sumsq_cap = 0;
    float *d_sse = nullptr;
    size_t sse_cap = 0;
    // grid search: the tile indices and per-tile scales of a batch of points
    int32_t *d_bidx = nullptr;
    size_t bidx_cap = 0;
    float *d_bscale = nullptr;
    size_t bscale_cap = 0;
    int *d_flag = nullptr;
    GssDev *d_gss = nullptr;
    // pinned host staging for the read-backs (sign checks, tile energies, the
    // chosen scale, per-tile errors): a copy into it is a DMA queued behind the
    // work on the stream, where a pageable destination is staged by the
    // runtime only once the stream has drained
    void *h_pin = nullptr;
    size_t pin_cap = 0;
    // LDLQ: error of the quantized spans (tile-major), one span's target,
    // dequantized values and container words
    float *d_err_tiles = nullptr;
    size_t err_tiles_cap = 0;
    float *d_span_target = nullptr;
    size_t span_target_cap = 0;
    float *d_span_what = nullptr;
    size_t span_what_cap = 0;
    uint16_t *d_span_packed = nullptr;
    size_t span_packed_cap = 0;
    // binary16 whole-matrix path: the sample's binary32 tiles, binary16
    // encoder inputs, and the probes' container words
    float *d_gs = nullptr;
    size_t gs_cap = 0;
    uint16_t *d_x16 = nullptr;
    size_t x16_cap = 0;
    uint16_t *d_pk = nullptr;
    size_t pk_cap = 0;
    // within-tile order of tile-major arrays: 256 bytes position -> element,
    // then 256 bytes element -> position; has_order is false for the natural
    // order (the kernels then take null tables)
    uint8_t *d_order = nullptr;
    bool has_order = false;
    std::string err;
    // optional per-launch timing (HIP events on the context's stream)
    struct Timed {
        int kind;
        int64_t tiles;
        hipEvent_t start, stop;
        hipStream_t stream;
    };
    bool timing = false;
    std::vector<Timed> timed;
};

namespace {

// 64 GiB: 65,536 tiles' backpointers, the final encode of a 4096 x 4096
// matrix in one batch (8 batches of 8,192 tiles measured 1-2 % slower: each
// batch boundary leaves the chip mostly idle through two tracebacks)
constexpr size_t kDefaultScratch = (size_t)64 << 30;

int fail(exl3_ctx *ctx, int code, const char *fmt, ...) {
    if (ctx) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        ctx->err = buf;
    }
    return code;
}

#define EXL3_HIP(ctx, call)                                                              \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess)                                                            \
            return fail((ctx), EXL3_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// Grow-only device buffer.  Waits for the stream before releasing the old one.
template <typename T>
int ensure(exl3_ctx *ctx, T *&ptr, size_t &cap, size_t count) {
    if (count <= cap && ptr) return EXL3_OK;
    if (ptr) {
        EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
        EXL3_HIP(ctx, hipFree(ptr));
        ptr = nullptr;
        cap = 0;
    }
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, std::max<size_t>(count, 1) * sizeof(T));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, EXL3_ENOMEM, "device allocation of %zu bytes failed: %s",
                    count * sizeof(T), hipGetErrorString(e));
    }
    ptr = static_cast<T *>(p);
    cap = count;
    return EXL3_OK;
}

int set_device(exl3_ctx *ctx) {
    EXL3_HIP(ctx, hipSetDevice(ctx->device));
    return EXL3_OK;
}

// Per-device address of `scratch` (null until looked up), and the error of a
// failed lookup.
std::mutex g_noalloc_mu;
std::vector<void *> g_noalloc_ptr;
std::vector<hipError_t> g_noalloc_err;

// Once per device, with that device current: look up the device address of
// the static scratch.  Runs at context creation (which may allocate host
// memory for the table); a failure is kept and reported by the entry point.
void noalloc_setup(int device) {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    if ((size_t)device < g_noalloc_ptr.size() &&
        (g_noalloc_ptr[(size_t)device] || g_noalloc_err[(size_t)device] != hipSuccess))
        return;
    if ((size_t)device >= g_noalloc_ptr.size()) {
        g_noalloc_ptr.resize((size_t)device + 1, nullptr);
        g_noalloc_err.resize((size_t)device + 1, hipSuccess);
    }
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        g_noalloc_err[(size_t)device] = e != hipSuccess ? e : hipErrorInvalidSymbol;
        return;
    }
    g_noalloc_ptr[(size_t)device] = p;
}

// The looked-up address for this device (no allocation, no HIP call).
void *noalloc_ptr(int device, hipError_t *err) {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    if ((size_t)device >= g_noalloc_ptr.size()) {
        *err = hipErrorNotInitialized;
        return nullptr;
    }
    *err = g_noalloc_err[(size_t)device];
    return g_noalloc_ptr[(size_t)device];
}

bool k_supported(int K) { return K >= 1 && K <= 4; }

const uint8_t *tile_order(const exl3_ctx *ctx) { return ctx->has_order ? ctx->d_order : nullptr; }
const uint8_t *tile_order_inv(const exl3_ctx *ctx) {
    return ctx->has_order ? ctx->d_order + 256 : nullptr;
}

// Every array argument must lie inside one allocation that the context's GPU
// can address (its device memory, managed memory or pinned host memory) and
// span the bytes the call touches.  Plain host memory, another device's
// memory or a buffer that ends too early is rejected before any launch, where
// a kernel would otherwise fault.  A sub-range of a larger allocation (a
// caching allocator's segment) is measured against that allocation.
int check_span(exl3_ctx *ctx, const void *p, size_t bytes, const char *name) {
    if (!p || bytes == 0) return EXL3_OK;
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof a);
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, EXL3_EINVAL, "%s (%p) is not memory the GPU can address", name, p);
    }
    if (a.type == hipMemoryTypeUnregistered)
        return fail(ctx, EXL3_EINVAL, "%s (%p) is host memory unknown to HIP, not device memory",
                    name, p);
    if (a.type == hipMemoryTypeDevice && a.device != ctx->device)
        return fail(ctx, EXL3_EINVAL, "%s is on device %d, the context on device %d", name,
                    a.device, ctx->device);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, EXL3_EINVAL, "%s (%p) lies in no allocation", name, p);
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < b || q - b > size || bytes > size - (q - b))
        return fail(ctx, EXL3_EINVAL,
                    "%s: %zu bytes from %p run past the end of its allocation (%zu bytes from %p)",
                    name, bytes, p, size, base);
    return EXL3_OK;
}

// Host-side tables (codebooks) must not be device memory.
int check_host(exl3_ctx *ctx, const void *p, const char *name) {
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof a);
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return EXL3_OK;
    }
    if (a.type == hipMemoryTypeDevice)
        return fail(ctx, EXL3_EINVAL, "%s (%p) is device memory; a host array is expected", name,
                    p);
    return EXL3_OK;
}

void clear_timing(exl3_ctx *ctx) {
    for (auto &r : ctx->timed) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    ctx->timed.clear();
}

// Bracket one launch with events when timing is on (on the stream the launch
// goes to).  Returns the record index (or -1); close_timed() records the stop
// event.
int open_timed(exl3_ctx *ctx, int kind, int64_t tiles, hipStream_t s = nullptr) {
    if (!ctx->timing) return -1;
    exl3_ctx::Timed r{kind, tiles, nullptr, nullptr, s ? s : ctx->stream};
    if (hipEventCreate(&r.start) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    if (hipEventCreate(&r.stop) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipEventDestroy(r.start);
        return -1;
    }
    (void)hipEventRecord(r.start, r.stream);
    ctx->timed.push_back(r);
    return (int)ctx->timed.size() - 1;
}

void close_timed(exl3_ctx *ctx, int id) {
    if (id >= 0) (void)hipEventRecord(ctx->timed[(size_t)id].stop, ctx->timed[(size_t)id].stream);
}

int ensure_small(exl3_ctx *ctx, size_t n) {
    if (n <= ctx->small_cap && ctx->d_end && ctx->d_X && ctx->d_cost) return EXL3_OK;
    if (ctx->d_end || ctx->d_X || ctx->d_cost) {
        EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
        (void)hipFree(ctx->d_end);
        (void)hipFree(ctx->d_X);
        (void)hipFree(ctx->d_cost);
        ctx->d_end = nullptr;
        ctx->d_X = nullptr;
        ctx->d_cost = nullptr;
        ctx->small_cap = 0;
    }
    size_t m = std::max<size_t>(n, 1);
    if (hipMalloc((void **)&ctx->d_end, m * sizeof(uint16_t)) != hipSuccess ||
        hipMalloc((void **)&ctx->d_X, m * sizeof(uint16_t)) != hipSuccess ||
        hipMalloc((void **)&ctx->d_cost, m * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, EXL3_ENOMEM, "device allocation of per-tile bookkeeping failed");
    }
    ctx->small_cap = m;
    return EXL3_OK;
}

// Admission of a batch of tiles: the largest number whose backpointer scratch
// fits the context's bound (whole rounds of one tile per compute unit when
// several batches are needed, so no batch ends in a mostly idle round).  If the
// device allocation fails, the batch is halved and tried again; the scratch is
// released before each attempt, never held twice.  Results do not depend on
// the batch size.
int admit_batch(exl3_ctx *ctx, int64_t n, int K, int64_t *batch_out) {
    const size_t per_tile = exl3::bp_bytes_per_tile(K);
    const size_t max_batch = ctx->scratch_limit / per_tile;
    if (max_batch == 0)
        return fail(ctx, EXL3_ENOMEM, "scratch limit %zu B is below one tile's %zu B",
                    ctx->scratch_limit, per_tile);
    int64_t batch = (int64_t)std::min<size_t>((size_t)n, max_batch);
    if (batch < n && batch > ctx->n_cu) batch -= batch % ctx->n_cu;
    bool retried = false;
    for (;;) {
        size_t bytes_cap = ctx->bp_cap;
        char *bp = static_cast<char *>(ctx->d_bp);
        int rc = ensure(ctx, bp, bytes_cap, (size_t)batch * per_tile);
        ctx->d_bp = bp;
        ctx->bp_cap = bytes_cap;
        if (rc == EXL3_OK) break;
        if (rc != EXL3_ENOMEM || batch == 1) return rc;
        batch = std::max<int64_t>(1, batch / 2);
        if (batch > ctx->n_cu) batch -= batch % ctx->n_cu;
        retried = true;
    }
    int rc = ensure_small(ctx, (size_t)batch);
    if (rc != EXL3_OK) return rc;
    if (retried) ctx->err.clear();     // the failed attempts are not the call's error
    *batch_out = batch;
    return EXL3_OK;
}

int ensure_aux(exl3_ctx *ctx) {
    if (ctx->aux) return EXL3_OK;
    EXL3_HIP(ctx, hipStreamCreateWithFlags(&ctx->aux, hipStreamNonBlocking));
    EXL3_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_fork, hipEventDisableTiming));
    EXL3_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_join, hipEventDisableTiming));
    return EXL3_OK;
}

// Path costs of n sample tiles (scale-search probe) when they fill some whole
// rounds of one tile per compute unit plus a small remainder: the remainder's
// chain runs on the second stream, so its pass 1 shares a round with the main
// part's pass 2 instead of leaving the chip idle for a round of its own.
int probe_split(exl3_ctx *ctx, const float *x, const int32_t *idx, int64_t n, int K, float scale,
                const float *scale_dev, float *cost_out, bool scale_per_tile) {
    const int64_t rem = n % ctx->n_cu, a = n - rem;
    const size_t per_tile = exl3::bp_bytes_per_tile(K);
    char *bp = static_cast<char *>(ctx->d_bp);
    int rc;
    if ((rc = ensure_aux(ctx)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, hipEventRecord(ctx->ev_fork, ctx->stream));
    EXL3_HIP(ctx, hipStreamWaitEvent(ctx->aux, ctx->ev_fork, 0));
    struct Part {
        hipStream_t s;
        int64_t first, count;
    } parts[2] = {{ctx->stream, 0, a}, {ctx->aux, a, rem}};
    // the remainder's forward launches are timed as their own kind: they run
    // beside the main part's, so their durations overlap other launches
    for (const Part &p : parts) {
        int id = open_timed(ctx, p.s == ctx->stream ? EXL3_KERNEL_FWD1 : EXL3_KERNEL_FWD_SIDE,
                            p.count, p.s);
        const float *sd = scale_dev && scale_per_tile ? scale_dev + p.first : scale_dev;
        EXL3_HIP(ctx, exl3::launch_viterbi_fwd(K, 1, x, idx + p.first, 0, p.count, ctx->d_levels,
                                               scale, sd, nullptr, bp + p.first * per_tile,
                                               ctx->d_end + p.first, nullptr, p.s,
                                               scale_per_tile));
        close_timed(ctx, id);
    }
    for (const Part &p : parts) {
        int id = open_timed(ctx, EXL3_KERNEL_TB1, p.count, p.s);
        EXL3_HIP(ctx, exl3::launch_traceback(K, 1, false, bp + p.first * per_tile, p.count,
                                             ctx->d_end + p.first, ctx->d_X + p.first, nullptr,
                                             nullptr, 0, nullptr, 0.0f, nullptr, nullptr,
                                             nullptr, nullptr, p.s));
        close_timed(ctx, id);
        id = open_timed(ctx, p.s == ctx->stream ? EXL3_KERNEL_FWD_COST : EXL3_KERNEL_FWD_SIDE,
                        p.count, p.s);
        const float *sd = scale_dev && scale_per_tile ? scale_dev + p.first : scale_dev;
        EXL3_HIP(ctx, exl3::launch_viterbi_fwd(K, 3, x, idx + p.first, 0, p.count, ctx->d_levels,
                                               scale, sd, ctx->d_X + p.first,
                                               bp + p.first * per_tile, nullptr,
                                               cost_out + p.first, p.s, scale_per_tile));
        close_timed(ctx, id);
    }
    EXL3_HIP(ctx, hipEventRecord(ctx->ev_join, ctx->aux));
    EXL3_HIP(ctx, hipStreamWaitEvent(ctx->stream, ctx->ev_join, 0));
    return EXL3_OK;
}

// One step of the golden-section scale search on the device, after probe k,
// with the operations of the host form in the same order (so the same scale,
// bit for bit): the probe's score is the binary64 sum of the sample's path
// costs in ascending tile order.  Probe 0 scores p0 and probe 1 q0; every
// later probe scores the point the previous reduction set.  From probe 1 on,
// one reduction follows; the binary32 value of its new point is the next
// probe's scale, and after the last reduction the scale is the midpoint of
// the bracket (the result).  One lane: the sum is a chain of dependent
// additions anyway.
__global__ void __launch_bounds__(64)
gss_step_kernel(GssDev *__restrict__ st, const float *__restrict__ costs, int64_t cnt, double a0,
                double b0, double p0, double q0, double g, int iters, int k) {
    if (threadIdx.x != 0) return;
    double f = 0.0;
    for (int64_t i = 0; i < cnt; ++i) f += (double)costs[i];
    GssDev s;
    if (k == 0) {
        s = GssDev{a0, b0, p0, q0, f, 0.0, 0, 0, (float)q0};
        *st = s;
        return;
    }
    s = *st;
    if (k == 1 || s.pending == 1) s.fq = f;
    else s.fp = f;
    if (s.it < iters) {
        if (s.fp < s.fq) {
            s.b = s.q;
            s.q = s.p;
            s.fq = s.fp;
            s.p = s.b - (s.b - s.a) * g;
            s.pending = 0;
            s.scale = (float)s.p;
        } else {
            s.a = s.p;
            s.p = s.q;
            s.fp = s.fq;
            s.q = s.a + (s.b - s.a) * g;
            s.pending = 1;
            s.scale = (float)s.q;
        }
        ++s.it;
    }
    if (s.it == iters) s.scale = (float)((s.a + s.b) / 2.0);
    *st = s;
}

// The pass-1 / traceback / pass-2 (/ traceback) chain over n tiles, batched so
// that the backpointers of one batch fit the scratch bound.  With cost_only,
// only the pass-2 path costs are produced (scale-search probes); with
// scale_dev, the forward passes read the scale from device memory.
int encode_chain(exl3_ctx *ctx, const float *x, const int32_t *idx, int64_t n, int K,
                 float scale, uint16_t *packed, uint16_t *states, float *sse, float *w_hat,
                 float *cost_only, const float *scale_dev = nullptr,
                 bool scale_per_tile = false) {
    if (n == 0) return EXL3_OK;
    // the traceback dequantizes at the host's scale: a device scale is for
    // path costs only
    if (scale_dev && !cost_only) return fail(ctx, EXL3_EINVAL, "device scale without cost_only");
    int64_t batch = 0;
    int rc;
    if ((rc = admit_batch(ctx, n, K, &batch)) != EXL3_OK) return rc;
    if (cost_only && idx && batch == n && n > ctx->n_cu && n % ctx->n_cu != 0 &&
        n % ctx->n_cu <= ctx->n_cu / 8)
        return probe_split(ctx, x, idx, n, K, scale, scale_dev, cost_only, scale_per_tile);
    for (int64_t i0 = 0; i0 < n; i0 += batch) {
        const int64_t nb = std::min<int64_t>(batch, n - i0);
        const int32_t *idx_b = idx ? idx + i0 : nullptr;
        const float *sd = scale_dev && scale_per_tile ? scale_dev + i0 : scale_dev;
        int id = open_timed(ctx, EXL3_KERNEL_FWD1, nb);
        EXL3_HIP(ctx, exl3::launch_viterbi_fwd(K, 1, x, idx_b, i0, nb, ctx->d_levels, scale, sd,
                                               nullptr, ctx->d_bp, ctx->d_end, nullptr,
                                               ctx->stream, scale_per_tile));
        close_timed(ctx, id);
        id = open_timed(ctx, EXL3_KERNEL_TB1, nb);
        EXL3_HIP(ctx, exl3::launch_traceback(K, 1, false, ctx->d_bp, nb, ctx->d_end, ctx->d_X, nullptr,
                                             nullptr, 0, nullptr, 0.0f, nullptr, nullptr,
                                             nullptr, nullptr, ctx->stream));
        close_timed(ctx, id);
        id = open_timed(ctx, cost_only ? EXL3_KERNEL_FWD_COST : EXL3_KERNEL_FWD2, nb);
        EXL3_HIP(ctx, exl3::launch_viterbi_fwd(K, cost_only ? 3 : 2, x, idx_b, i0, nb,
                                               ctx->d_levels, scale, sd,
                                               ctx->d_X, ctx->d_bp, nullptr,
                                               cost_only ? cost_only + i0 : ctx->d_cost,
                                               ctx->stream, scale_per_tile));
        close_timed(ctx, id);
        if (!cost_only) {
            id = open_timed(ctx, EXL3_KERNEL_TB2, nb);
            EXL3_HIP(ctx, exl3::launch_traceback(K, 2, false, ctx->d_bp, nb, ctx->d_X, nullptr, x,
                                                 idx_b, i0, ctx->d_levels, scale, packed,
                                                 states, sse, w_hat, ctx->stream));
            close_timed(ctx, id);
        }
    }
    return EXL3_OK;
}

// The same chain in binary16 arithmetic: costs come out of pass 2 directly.
// With x32 given (the binary32 weights of the same tiles), the traceback also
// dequantizes at `scale` and sums the binary32 squared errors (sse, w_hat).
int encode_chain_f16(exl3_ctx *ctx, const uint16_t *x, int64_t n, int K, uint16_t *packed,
                     uint16_t *states, uint16_t *cost, const float *x32 = nullptr,
                     float scale = 0.0f, float *sse = nullptr, float *w_hat = nullptr) {
    if (n == 0) return EXL3_OK;
    int64_t batch = 0;
    int rc;
    if ((rc = admit_batch(ctx, n, K, &batch)) != EXL3_OK) return rc;
    uint16_t *cost_tmp = reinterpret_cast<uint16_t *>(ctx->d_cost);
    // A batch a few tiles past a whole round of the compute units (one tile each
    // at K = 1..3; the scale search's sample): the remainder runs on a second
    // stream beside the main part, three tile-pass times instead of four (as
    // in probe_split)
    if (K <= 3 && batch == n && n > ctx->n_cu && n % ctx->n_cu != 0 &&
        n % ctx->n_cu <= ctx->n_cu / 8) {
        const int64_t rem = n % ctx->n_cu, a = n - rem;
        const size_t per_tile = exl3::bp_bytes_per_tile(K);
        char *bp = static_cast<char *>(ctx->d_bp);
        if ((rc = ensure_aux(ctx)) != EXL3_OK) return rc;
        EXL3_HIP(ctx, hipEventRecord(ctx->ev_fork, ctx->stream));
        EXL3_HIP(ctx, hipStreamWaitEvent(ctx->aux, ctx->ev_fork, 0));
        struct Part {
            hipStream_t s;
            int64_t first, count;
        } parts[2] = {{ctx->stream, 0, a}, {ctx->aux, a, rem}};
        for (const Part &p : parts) {
            int id = open_timed(ctx, p.s == ctx->stream ? EXL3_KERNEL_FWD1 : EXL3_KERNEL_FWD_SIDE,
                                p.count, p.s);
            EXL3_HIP(ctx, exl3::launch_viterbi_fwd_f16(K, 1, x, p.first, p.count, ctx->d_levels,
                                                       nullptr, bp + p.first * per_tile,
                                                       ctx->d_end + p.first, nullptr, p.s));
            close_timed(ctx, id);
        }
        for (const Part &p : parts) {
            int id = open_timed(ctx, EXL3_KERNEL_TB1, p.count, p.s);
            EXL3_HIP(ctx, exl3::launch_traceback(K, 1, true, bp + p.first * per_tile, p.count,
                                                 ctx->d_end + p.first, ctx->d_X + p.first,
                                                 nullptr, nullptr, 0, nullptr, 0.0f, nullptr,
                                                 nullptr, nullptr, nullptr, p.s));
            close_timed(ctx, id);
            id = open_timed(ctx, p.s == ctx->stream ? EXL3_KERNEL_FWD2 : EXL3_KERNEL_FWD_SIDE,
                            p.count, p.s);
            EXL3_HIP(ctx, exl3::launch_viterbi_fwd_f16(K, 2, x, p.first, p.count, ctx->d_levels,
                                                       ctx->d_X + p.first,
                                                       bp + p.first * per_tile, nullptr,
                                                       (cost ? cost : cost_tmp) + p.first, p.s));
            close_timed(ctx, id);
            id = open_timed(ctx, EXL3_KERNEL_TB2, p.count, p.s);
            EXL3_HIP(ctx, exl3::launch_traceback(K, 2, true, bp + p.first * per_tile, p.count,
                                                 ctx->d_X + p.first, nullptr, x32, nullptr,
                                                 p.first, ctx->d_levels, scale, packed, states,
                                                 sse, w_hat, p.s));
            close_timed(ctx, id);
        }
        EXL3_HIP(ctx, hipEventRecord(ctx->ev_join, ctx->aux));
        EXL3_HIP(ctx, hipStreamWaitEvent(ctx->stream, ctx->ev_join, 0));
        return EXL3_OK;
    }
    for (int64_t i0 = 0; i0 < n; i0 += batch) {
        const int64_t nb = std::min<int64_t>(batch, n - i0);
        int id = open_timed(ctx, EXL3_KERNEL_FWD1, nb);
        EXL3_HIP(ctx, exl3::launch_viterbi_fwd_f16(K, 1, x, i0, nb, ctx->d_levels, nullptr,
                                                   ctx->d_bp, ctx->d_end, nullptr, ctx->stream));
        close_timed(ctx, id);
        id = open_timed(ctx, EXL3_KERNEL_TB1, nb);
        EXL3_HIP(ctx, exl3::launch_traceback(K, 1, true, ctx->d_bp, nb, ctx->d_end, ctx->d_X,
                                             nullptr, nullptr, 0, nullptr, 0.0f, nullptr,
                                             nullptr, nullptr, nullptr, ctx->stream));
        close_timed(ctx, id);
        id = open_timed(ctx, EXL3_KERNEL_FWD2, nb);
        EXL3_HIP(ctx, exl3::launch_viterbi_fwd_f16(K, 2, x, i0, nb, ctx->d_levels, ctx->d_X,
                                                   ctx->d_bp, nullptr,
                                                   cost ? cost + i0 : cost_tmp, ctx->stream));
        close_timed(ctx, id);
        id = open_timed(ctx, EXL3_KERNEL_TB2, nb);
        EXL3_HIP(ctx, exl3::launch_traceback(K, 2, true, ctx->d_bp, nb, ctx->d_X, nullptr,
                                             x32, nullptr, i0, ctx->d_levels, scale, packed,
                                             states, sse, w_hat, ctx->stream));
        close_timed(ctx, id);
    }
    return EXL3_OK;
}

// The pinned staging buffer, at least `bytes` long (the stream is idle when
// it is replaced: every use synchronizes before reading it).
int pinned(exl3_ctx *ctx, size_t bytes, void **out) {
    if (bytes > ctx->pin_cap) {
        if (ctx->h_pin) {
            EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
            (void)hipHostFree(ctx->h_pin);
            ctx->h_pin = nullptr;
            ctx->pin_cap = 0;
        }
        const size_t cap = std::max<size_t>(bytes, 1 << 20);
        EXL3_HIP(ctx, hipHostMalloc(&ctx->h_pin, cap, hipHostMallocDefault));
        ctx->pin_cap = cap;
    }
    *out = ctx->h_pin;
    return EXL3_OK;
}

// Device-to-host read-backs of up to two arrays through the pinned buffer, one
// synchronization; returns the host copies (valid until the next read-back).
int read_back(exl3_ctx *ctx, const void *d0, size_t b0, const void *d1, size_t b1,
              const void **h0, const void **h1 = nullptr) {
    const size_t off1 = (b0 + 255) / 256 * 256;
    void *h;
    int rc;
    if ((rc = pinned(ctx, off1 + b1, &h)) != EXL3_OK) return rc;
    char *hc = static_cast<char *>(h);
    if (b0) EXL3_HIP(ctx, hipMemcpyAsync(hc, d0, b0, hipMemcpyDeviceToHost, ctx->stream));
    if (b1) EXL3_HIP(ctx, hipMemcpyAsync(hc + off1, d1, b1, hipMemcpyDeviceToHost, ctx->stream));
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    *h0 = hc;
    if (h1) *h1 = hc + off1;
    return EXL3_OK;
}

// Sign vectors must hold exactly +1 or -1 (copied to the host to check, both
// with one synchronization; d1 may be null).
int check_signs(exl3_ctx *ctx, const float *d0, int n0, const char *name0,
                const float *d1 = nullptr, int n1 = 0, const char *name1 = nullptr) {
    const void *p0, *p1;
    int rc;
    if ((rc = read_back(ctx, d0, (size_t)n0 * sizeof(float), d1,
                        d1 ? (size_t)n1 * sizeof(float) : 0, &p0, &p1)) != EXL3_OK)
        return rc;
    const float *h0 = static_cast<const float *>(p0), *h1 = static_cast<const float *>(p1);
    for (int i = 0; i < n0; ++i)
        if (h0[i] != 1.0f && h0[i] != -1.0f)
            return fail(ctx, EXL3_EINVAL, "%s[%d] = %g is not +1 or -1", name0, i, (double)h0[i]);
    for (int i = 0; d1 && i < n1; ++i)
        if (h1[i] != 1.0f && h1[i] != -1.0f)
            return fail(ctx, EXL3_EINVAL, "%s[%d] = %g is not +1 or -1", name1, i, (double)h1[i]);
    return EXL3_OK;
}

int check_matrix_args(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                      int had_block, const float *su, const float *sv) {
    if (!w || !su || !sv) return fail(ctx, EXL3_EINVAL, "null weight or sign pointer");
    if (w_dtype != EXL3_F32 && w_dtype != EXL3_BF16)
        return fail(ctx, EXL3_EINVAL, "weight dtype %d is not EXL3_F32 or EXL3_BF16", w_dtype);
    if (had_block != 64 && had_block != 128)
        return fail(ctx, EXL3_EUNSUPPORTED, "Hadamard block %d (supported: 64, 128)", had_block);
    if (rows <= 0 || cols <= 0 || rows % had_block || cols % had_block)
        return fail(ctx, EXL3_EINVAL, "shape %d x %d is not a positive multiple of %d", rows,
                    cols, had_block);
    return EXL3_OK;
}

}  // namespace

extern "C" {

const char *exl3_version(void) { return "exl3-gfx950 0.1"; }

size_t exl3_scratch_per_tile(int K) {
    return k_supported(K) ? exl3::bp_bytes_per_tile(K) : 0;
}

int exl3_ctx_create(exl3_ctx **out, int device, void *hip_stream, size_t scratch_bytes) {
    if (!out) return EXL3_EINVAL;
    *out = nullptr;
    exl3_ctx *ctx = new (std::nothrow) exl3_ctx();
    if (!ctx) return EXL3_ENOMEM;
    ctx->device = device;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    ctx->scratch_limit = scratch_bytes ? scratch_bytes : kDefaultScratch;
    if (hipSetDevice(device) != hipSuccess) {
        (void)hipGetLastError();
        delete ctx;
        return EXL3_EHIP;
    }
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess &&
        n_cu > 0)
        ctx->n_cu = n_cu;
    noalloc_setup(device);
    std::vector<uint16_t> lv(65536);
    exl3::build_mul1_levels(lv.data());
    if (hipMalloc((void **)&ctx->d_levels, 65536 * sizeof(uint16_t)) != hipSuccess ||
        hipMalloc((void **)&ctx->d_flag, sizeof(int)) != hipSuccess ||
        hipMalloc((void **)&ctx->d_gss, sizeof(GssDev)) != hipSuccess ||
        hipMemcpy(ctx->d_levels, lv.data(), 65536 * sizeof(uint16_t), hipMemcpyHostToDevice) !=
            hipSuccess) {
        (void)hipGetLastError();
        exl3_ctx_destroy(ctx);
        return EXL3_EHIP;
    }
    *out = ctx;
    return EXL3_OK;
}

void exl3_ctx_destroy(exl3_ctx *ctx) {
    if (!ctx) return;
    (void)hipSetDevice(ctx->device);
    (void)hipStreamSynchronize(ctx->stream);
    if (ctx->aux) (void)hipStreamSynchronize(ctx->aux);
    clear_timing(ctx);
    if (ctx->ev_fork) (void)hipEventDestroy(ctx->ev_fork);
    if (ctx->ev_join) (void)hipEventDestroy(ctx->ev_join);
    if (ctx->ev_switch) (void)hipEventDestroy(ctx->ev_switch);
    if (ctx->aux) (void)hipStreamDestroy(ctx->aux);
    if (ctx->h_pin) (void)hipHostFree(ctx->h_pin);
    void *bufs[] = {ctx->d_levels,      ctx->d_bp,          ctx->d_end,         ctx->d_X,
                    ctx->d_cost,        ctx->d_idx,         ctx->d_wreg,        ctx->d_sumsq,
                    ctx->d_sse,         ctx->d_flag,        ctx->d_err_tiles,   ctx->d_span_target,
                    ctx->d_span_what,   ctx->d_span_packed, ctx->d_gs,          ctx->d_x16,
                    ctx->d_pk,          ctx->d_order,       ctx->d_gss,         ctx->d_bidx,
                    ctx->d_bscale};
    for (void *p : bufs)
        if (p) (void)hipFree(p);
    delete ctx;
}

const char *exl3_last_error(const exl3_ctx *ctx) { return ctx ? ctx->err.c_str() : ""; }

int exl3_ctx_set_stream(exl3_ctx *ctx, void *hip_stream) {
    if (!ctx) return EXL3_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (s == ctx->stream) return EXL3_OK;
    // work already enqueued on the old stream may still use the context's
    // buffers: the new stream waits for it (no host synchronization)
    int rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    if (!ctx->ev_switch)
        EXL3_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_switch, hipEventDisableTiming));
    EXL3_HIP(ctx, hipEventRecord(ctx->ev_switch, ctx->stream));
    EXL3_HIP(ctx, hipStreamWaitEvent(s, ctx->ev_switch, 0));
    ctx->stream = s;
    return EXL3_OK;
}

int exl3_ctx_set_timing(exl3_ctx *ctx, int enable) {
    if (!ctx) return EXL3_EINVAL;
    int rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    clear_timing(ctx);
    ctx->timing = enable != 0;
    return EXL3_OK;
}

int exl3_ctx_read_timing(exl3_ctx *ctx, int kind, double *total_ms, int64_t *launches,
                         int64_t *tiles) {
    if (!ctx || !total_ms || !launches || !tiles) return fail(ctx, EXL3_EINVAL, "null argument");
    int rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    double ms = 0.0;
    int64_t nl = 0, nt = 0;
    for (auto &r : ctx->timed) {
        if (r.kind != kind) continue;
        float e = 0.0f;
        EXL3_HIP(ctx, hipEventElapsedTime(&e, r.start, r.stop));
        ms += e;
        nl += 1;
        nt += r.tiles;
    }
    *total_ms = ms;
    *launches = nl;
    *tiles = nt;
    return EXL3_OK;
}

int exl3_set_codebook(exl3_ctx *ctx, const uint16_t *levels_fp16_host) {
    if (!ctx) return EXL3_EINVAL;
    int rc;
    if (levels_fp16_host && (rc = check_host(ctx, levels_fp16_host, "levels")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    std::vector<uint16_t> lv(65536);
    if (levels_fp16_host) {
        for (int i = 0; i < 65536; ++i) {
            if ((levels_fp16_host[i] & 0x7C00u) == 0x7C00u)
                return fail(ctx, EXL3_EINVAL, "level %d is NaN or Inf", i);
            lv[(size_t)i] = levels_fp16_host[i];
        }
    } else {
        exl3::build_mul1_levels(lv.data());
    }
    EXL3_HIP(ctx, hipMemcpyAsync(ctx->d_levels, lv.data(), 65536 * sizeof(uint16_t),
                                 hipMemcpyHostToDevice, ctx->stream));
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    return EXL3_OK;
}

int exl3_set_codebook_kind(exl3_ctx *ctx, int kind) {
    if (!ctx) return EXL3_EINVAL;
    std::vector<uint16_t> lv(65536);
    switch (kind) {
        case EXL3_CB_MUL1: exl3::build_mul1_levels(lv.data()); break;
        case EXL3_CB_MCG: exl3::build_mcg_levels(lv.data()); break;
        case EXL3_CB_3INST: exl3::build_3inst_levels(lv.data()); break;
        default: return fail(ctx, EXL3_EUNSUPPORTED, "codebook kind %d (supported: 0, 1, 2)", kind);
    }
    int rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, hipMemcpyAsync(ctx->d_levels, lv.data(), 65536 * sizeof(uint16_t),
                                 hipMemcpyHostToDevice, ctx->stream));
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    return EXL3_OK;
}

int exl3_set_tile_order(exl3_ctx *ctx, const uint8_t *order_host) {
    if (!ctx) return EXL3_EINVAL;
    int rc;
    uint8_t tab[512];
    bool identity = true;
    if (order_host) {
        if ((rc = check_host(ctx, order_host, "order")) != EXL3_OK) return rc;
        bool seen[256] = {};
        for (int t = 0; t < 256; ++t) {
            const uint8_t e = order_host[t];
            if (seen[e])
                return fail(ctx, EXL3_EINVAL,
                            "order is not a permutation of 0..255 (element %d appears twice)",
                            (int)e);
            seen[e] = true;
            tab[t] = e;
            tab[256 + e] = (uint8_t)t;
            identity = identity && e == t;
        }
    }
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    if (identity) {
        ctx->has_order = false;
        return EXL3_OK;
    }
    if (!ctx->d_order) {
        void *p = nullptr;
        hipError_t e = hipMalloc(&p, sizeof tab);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ctx, EXL3_ENOMEM, "device allocation of the order table failed: %s",
                        hipGetErrorString(e));
        }
        ctx->d_order = static_cast<uint8_t *>(p);
    }
    // in stream order: work already enqueued keeps reading the previous table
    EXL3_HIP(ctx, hipMemcpyAsync(ctx->d_order, tab, sizeof tab, hipMemcpyHostToDevice,
                                 ctx->stream));
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    ctx->has_order = true;
    return EXL3_OK;
}

int exl3_get_codebook(exl3_ctx *ctx, uint16_t *levels_fp16_host) {
    if (!ctx || !levels_fp16_host) return fail(ctx, EXL3_EINVAL, "null argument");
    int rc;
    if ((rc = check_host(ctx, levels_fp16_host, "levels")) != EXL3_OK) return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, hipMemcpyAsync(levels_fp16_host, ctx->d_levels, 65536 * sizeof(uint16_t),
                                 hipMemcpyDeviceToHost, ctx->stream));
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    return EXL3_OK;
}

int exl3_regularize(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                    int had_block, const float *su, const float *sv, float *w_reg,
                    int out_layout, float *tile_sumsq, int *nonfinite) {
    if (!ctx) return EXL3_EINVAL;
    int rc;
    if ((rc = check_matrix_args(ctx, w, w_dtype, rows, cols, had_block, su, sv)) != EXL3_OK)
        return rc;
    if (!w_reg) return fail(ctx, EXL3_EINVAL, "null output");
    if (out_layout != EXL3_ROW_MAJOR && out_layout != EXL3_TILE_MAJOR)
        return fail(ctx, EXL3_EINVAL, "layout %d", out_layout);
    const size_t nel = (size_t)rows * cols, ntiles = nel / 256;
    if ((rc = check_span(ctx, w, nel * (w_dtype == EXL3_BF16 ? 2 : 4), "w")) != EXL3_OK ||
        (rc = check_span(ctx, su, (size_t)rows * sizeof(float), "su")) != EXL3_OK ||
        (rc = check_span(ctx, sv, (size_t)cols * sizeof(float), "sv")) != EXL3_OK ||
        (rc = check_span(ctx, w_reg, nel * sizeof(float), "w_reg")) != EXL3_OK ||
        (rc = check_span(ctx, tile_sumsq, ntiles * sizeof(float), "tile_sumsq")) != EXL3_OK ||
        (rc = check_span(ctx, nonfinite, sizeof(int), "nonfinite")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    const int id = open_timed(ctx, EXL3_KERNEL_REGULARIZE, (int64_t)ntiles);
    EXL3_HIP(ctx, exl3::launch_regularize(w, w_dtype, rows, cols, had_block, su, sv, w_reg,
                                          out_layout, tile_sumsq, nonfinite, tile_order(ctx),
                                          ctx->n_cu, ctx->stream));
    close_timed(ctx, id);
    return EXL3_OK;
}

int exl3_unregularize(exl3_ctx *ctx, const float *w_reg, int in_layout, int rows, int cols,
                      int had_block, const float *su, const float *sv, float *out) {
    if (!ctx) return EXL3_EINVAL;
    if (!w_reg || !su || !sv || !out) return fail(ctx, EXL3_EINVAL, "null pointer");
    if (in_layout != EXL3_ROW_MAJOR && in_layout != EXL3_TILE_MAJOR)
        return fail(ctx, EXL3_EINVAL, "layout %d", in_layout);
    if (had_block != 64 && had_block != 128)
        return fail(ctx, EXL3_EUNSUPPORTED, "Hadamard block %d (supported: 64, 128)", had_block);
    if (rows <= 0 || cols <= 0 || rows % had_block || cols % had_block)
        return fail(ctx, EXL3_EINVAL, "shape %d x %d is not a positive multiple of %d", rows,
                    cols, had_block);
    const size_t bytes = (size_t)rows * cols * sizeof(float);
    const char *ib = reinterpret_cast<const char *>(w_reg), *ob = reinterpret_cast<const char *>(out);
    if (ob < ib + bytes && ib < ob + bytes) return fail(ctx, EXL3_EINVAL, "out overlaps w_reg");
    int rc;
    if ((rc = check_span(ctx, w_reg, bytes, "w_reg")) != EXL3_OK ||
        (rc = check_span(ctx, su, (size_t)rows * sizeof(float), "su")) != EXL3_OK ||
        (rc = check_span(ctx, sv, (size_t)cols * sizeof(float), "sv")) != EXL3_OK ||
        (rc = check_span(ctx, out, bytes, "out")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, exl3::launch_unregularize(w_reg, in_layout, rows, cols, had_block, su, sv, out,
                                            tile_order(ctx), ctx->stream));
    return EXL3_OK;
}

int exl3_channel_normalize(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                           const float *su, double floor, float *w_norm, float *su_folded,
                           double *row_rms) {
    if (!ctx) return EXL3_EINVAL;
    if (!w || !su || !w_norm || !su_folded)
        return fail(ctx, EXL3_EINVAL, "null weight, sign or output pointer");
    if (w_dtype != EXL3_F32 && w_dtype != EXL3_BF16)
        return fail(ctx, EXL3_EINVAL, "weight dtype %d is not EXL3_F32 or EXL3_BF16", w_dtype);
    if (rows <= 0 || cols <= 0) return fail(ctx, EXL3_EINVAL, "shape %d x %d", rows, cols);
    if (!(floor > 0.0) || !std::isfinite(floor))
        return fail(ctx, EXL3_EINVAL, "zero-channel floor %g is not finite and positive", floor);
    const size_t in_bytes = (size_t)rows * cols * (w_dtype == EXL3_BF16 ? 2 : 4);
    const char *wb = static_cast<const char *>(w), *ob = reinterpret_cast<const char *>(w_norm);
    if (ob < wb + in_bytes && wb < ob + (size_t)rows * cols * sizeof(float))
        return fail(ctx, EXL3_EINVAL, "w_norm overlaps w");
    int rc;
    if ((rc = check_span(ctx, w, in_bytes, "w")) != EXL3_OK ||
        (rc = check_span(ctx, su, (size_t)rows * sizeof(float), "su")) != EXL3_OK ||
        (rc = check_span(ctx, w_norm, (size_t)rows * cols * sizeof(float), "w_norm")) !=
            EXL3_OK ||
        (rc = check_span(ctx, su_folded, (size_t)rows * sizeof(float), "su_folded")) !=
            EXL3_OK ||
        (rc = check_span(ctx, row_rms, (size_t)rows * sizeof(double), "row_rms")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    if ((rc = check_signs(ctx, su, rows, "su")) != EXL3_OK) return rc;
    const int id = open_timed(ctx, EXL3_KERNEL_CHANNEL, 0);
    EXL3_HIP(ctx, exl3::launch_channel_normalize(w, w_dtype, rows, cols, su, floor, w_norm,
                                                 su_folded, row_rms, ctx->stream));
    close_timed(ctx, id);
    return EXL3_OK;
}

int exl3_encode_tiles(exl3_ctx *ctx, const float *x, int64_t n, int K, float scale,
                      uint16_t *packed, uint16_t *states, float *tile_sse) {
    if (!ctx) return EXL3_EINVAL;
    if (!k_supported(K)) return fail(ctx, EXL3_EUNSUPPORTED, "K = %d (supported: 1, 2, 3, 4)", K);
    if (n < 0) return fail(ctx, EXL3_EINVAL, "n = %lld", (long long)n);
    if (n > 0 && (!x || !packed)) return fail(ctx, EXL3_EINVAL, "null input or output");
    if (!std::isfinite(scale)) return fail(ctx, EXL3_EINVAL, "scale is not finite");
    if (n > (int64_t)INT32_MAX) return fail(ctx, EXL3_EINVAL, "too many tiles");
    int rc;
    const size_t nt = (size_t)n;
    if ((rc = check_span(ctx, x, nt * 256 * sizeof(float), "x")) != EXL3_OK ||
        (rc = check_span(ctx, packed, nt * 16 * K * sizeof(uint16_t), "packed")) != EXL3_OK ||
        (rc = check_span(ctx, states, nt * 256 * sizeof(uint16_t), "states")) != EXL3_OK ||
        (rc = check_span(ctx, tile_sse, nt * sizeof(float), "tile_sse")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    return encode_chain(ctx, x, nullptr, n, K, scale, packed, states, tile_sse, nullptr, nullptr);
}

int exl3_encode_tiles_noalloc(exl3_ctx *ctx, const float *x, int64_t n, int K, float scale,
                              uint16_t *packed, uint16_t *states, float *tile_sse) {
    if (!ctx) return EXL3_EINVAL;
    if (!k_supported(K)) return fail(ctx, EXL3_EUNSUPPORTED, "K = %d (supported: 1, 2, 3, 4)", K);
    if (n < 0) return fail(ctx, EXL3_EINVAL, "n = %lld", (long long)n);
    const int64_t max_n = K == 4 ? EXL3_NOALLOC_MAX_TILES_K4 : EXL3_NOALLOC_MAX_TILES;
    if (n > max_n)
        return fail(ctx, EXL3_EINVAL,
                    "n = %lld tiles exceeds the %lld the static scratch holds at K = %d "
                    "(call again for the rest)", (long long)n, (long long)max_n, K);
    if (n > 0 && (!x || !packed)) return fail(ctx, EXL3_EINVAL, "null input or output");
    if (!std::isfinite(scale)) return fail(ctx, EXL3_EINVAL, "scale is not finite");
    int rc;
    const size_t nt = (size_t)n;
    if ((rc = check_span(ctx, x, nt * 256 * sizeof(float), "x")) != EXL3_OK ||
        (rc = check_span(ctx, packed, nt * 16 * K * sizeof(uint16_t), "packed")) != EXL3_OK ||
        (rc = check_span(ctx, states, nt * 256 * sizeof(uint16_t), "states")) != EXL3_OK ||
        (rc = check_span(ctx, tile_sse, nt * sizeof(float), "tile_sse")) != EXL3_OK)
        return rc;
    if (n == 0) return EXL3_OK;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    hipError_t e = hipSuccess;
    char *base = static_cast<char *>(noalloc_ptr(ctx->device, &e));
    if (!base)
        return fail(ctx, EXL3_EHIP, "the static scratch of device %d is not available: %s",
                    ctx->device, hipGetErrorString(e));
    // layout: backpointers, then end states, X and path costs of the batch;
    // every word the chain reads was written earlier in this call, so nothing
    // needs clearing
    void *bp = base;
    uint16_t *d_end = reinterpret_cast<uint16_t *>(base + kNoAllocBpBytes);
    uint16_t *d_X = d_end + kNoAllocBookTiles;
    float *d_cost = reinterpret_cast<float *>(d_X + kNoAllocBookTiles);
    hipStream_t s = ctx->stream;
    EXL3_HIP(ctx, exl3::launch_viterbi_fwd(K, 1, x, nullptr, 0, n, ctx->d_levels, scale, nullptr,
                                           nullptr, bp, d_end, nullptr, s));
    EXL3_HIP(ctx, exl3::launch_traceback(K, 1, false, bp, n, d_end, d_X, nullptr, nullptr, 0,
                                         nullptr, 0.0f, nullptr, nullptr, nullptr, nullptr, s));
    EXL3_HIP(ctx, exl3::launch_viterbi_fwd(K, 2, x, nullptr, 0, n, ctx->d_levels, scale, nullptr,
                                           d_X, bp, nullptr, d_cost, s));
    EXL3_HIP(ctx, exl3::launch_traceback(K, 2, false, bp, n, d_X, nullptr, x, nullptr, 0,
                                         ctx->d_levels, scale, packed, states, tile_sse, nullptr,
                                         s));
    return EXL3_OK;
}

int exl3_encode_tiles_f16(exl3_ctx *ctx, const uint16_t *x, int64_t n, int K, uint16_t *packed,
                          uint16_t *states, uint16_t *cost) {
    if (!ctx) return EXL3_EINVAL;
    if (!k_supported(K)) return fail(ctx, EXL3_EUNSUPPORTED, "K = %d (supported: 1, 2, 3, 4)", K);
    if (n < 0) return fail(ctx, EXL3_EINVAL, "n = %lld", (long long)n);
    if (n > 0 && (!x || !packed)) return fail(ctx, EXL3_EINVAL, "null input or output");
    if (n > (int64_t)INT32_MAX) return fail(ctx, EXL3_EINVAL, "too many tiles");
    int rc;
    const size_t nt = (size_t)n;
    if ((rc = check_span(ctx, x, nt * 256 * sizeof(uint16_t), "x")) != EXL3_OK ||
        (rc = check_span(ctx, packed, nt * 16 * K * sizeof(uint16_t), "packed")) != EXL3_OK ||
        (rc = check_span(ctx, states, nt * 256 * sizeof(uint16_t), "states")) != EXL3_OK ||
        (rc = check_span(ctx, cost, nt * sizeof(uint16_t), "cost")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    return encode_chain_f16(ctx, x, n, K, packed, states, cost);
}

int exl3_decode_tiles(exl3_ctx *ctx, const uint16_t *packed, int64_t n, int K, float scale,
                      float *out) {
    if (!ctx) return EXL3_EINVAL;
    if (K < 1 || K > 8) return fail(ctx, EXL3_EUNSUPPORTED, "K = %d (supported: 1..8)", K);
    if (n < 0) return fail(ctx, EXL3_EINVAL, "n = %lld", (long long)n);
    if (n > 0 && (!packed || !out)) return fail(ctx, EXL3_EINVAL, "null input or output");
    if (!std::isfinite(scale)) return fail(ctx, EXL3_EINVAL, "scale is not finite");
    if (n > (int64_t)INT32_MAX) return fail(ctx, EXL3_EINVAL, "too many tiles");
    int rc;
    const size_t nt = (size_t)n;
    if ((rc = check_span(ctx, packed, nt * 16 * K * sizeof(uint16_t), "packed")) != EXL3_OK ||
        (rc = check_span(ctx, out, nt * 256 * sizeof(float), "out")) != EXL3_OK)
        return rc;
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    const int id = open_timed(ctx, EXL3_KERNEL_DECODE, n);
    EXL3_HIP(ctx, exl3::launch_decode(packed, n, K, scale, ctx->d_levels, out, ctx->n_cu,
                                      ctx->stream));
    close_timed(ctx, id);
    return EXL3_OK;
}

}  // extern "C"

namespace {

// Grid + parabolic search for the multiplier of the rms ("EXL3 Intel Arc
// Quantizer" README, Core Implemented Architecture section 8): coarse points
// lo + k*step on the subsample (least objective, lowest on ties), fine points
// g_c + m*fine_step on the full sample, then the vertex of the parabola through
// an interior fine minimum and its neighbours; at least `floor`.
template <typename FS, typename FF>
double grid_search(const exl3_grid &grid, FS f_sub, FF f_full) {
    // f_sub, f_full: the objectives of a list of points (one batch each)
    const long n_c = std::lround((grid.coarse_hi - grid.coarse_lo) / grid.coarse_step);
    std::vector<double> gc;
    for (long k = 0; k <= n_c; ++k) gc.push_back(grid.coarse_lo + (double)k * grid.coarse_step);
    const std::vector<double> vc = f_sub(gc);
    double g_c = gc[0], best = vc[0];
    for (size_t k = 1; k < gc.size(); ++k)
        if (vc[k] < best) {
            best = vc[k];
            g_c = gc[k];
        }
    const long M = std::lround(grid.fine_radius / grid.fine_step);
    std::vector<double> gs;
    for (long m = -M; m <= M; ++m) gs.push_back(g_c + (double)m * grid.fine_step);
    const std::vector<double> fs = f_full(gs);
    size_t ib = 0;
    for (size_t i = 1; i < fs.size(); ++i)
        if (fs[i] < fs[ib]) ib = i;
    double g = gs[ib];
    if (ib > 0 && ib + 1 < fs.size()) {
        const double fm = fs[ib - 1], f0 = fs[ib], fp = fs[ib + 1];
        const double d = fm - 2.0 * f0 + fp;
        if (d > 0.0) g = gs[ib] + grid.fine_step * (fm - fp) / (2.0 * d);
    }
    return std::max(g, grid.floor);
}

// Validation, regularization (tile-major, into the context), statistics and the
// scale (fixed or golden-section search on the tile sample): the common front
// of the whole-matrix calls.
int regularize_and_choose_scale(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                                int K, int had_block, const float *su, const float *sv,
                                const exl3_gss *gss, const exl3_grid *grid, float fixed_scale,
                                uint16_t *packed, float *scale_out, float *scale_chosen,
                                const float *w_hat, const float *tile_out, const float *L,
                                bool f16 = false) {
    if (!ctx) return EXL3_EINVAL;
    int rc;
    if ((rc = check_matrix_args(ctx, w, w_dtype, rows, cols, had_block, su, sv)) != EXL3_OK)
        return rc;
    if (!k_supported(K)) return fail(ctx, EXL3_EUNSUPPORTED, "K = %d (supported: 1, 2, 3, 4)", K);
    if (!packed || !scale_out) return fail(ctx, EXL3_EINVAL, "null output");
    if (grid) {
        const double n_c = grid->coarse_step > 0.0
                               ? (grid->coarse_hi - grid->coarse_lo) / grid->coarse_step : -1.0;
        const double n_f = grid->fine_step > 0.0 ? grid->fine_radius / grid->fine_step : -1.0;
        if (!(grid->coarse_lo > 0.0) || !(n_c >= 0.0) || n_c > 1000.0 || grid->stride < 1 ||
            !(n_f >= 0.0) || n_f > 1000.0 || !(grid->floor >= 0.0) || !std::isfinite(grid->floor))
            return fail(ctx, EXL3_EINVAL, "grid search {%g..%g step %g, stride %d, +-%g step %g, "
                        "floor %g}", grid->coarse_lo, grid->coarse_hi, grid->coarse_step,
                        grid->stride, grid->fine_radius, grid->fine_step, grid->floor);
    } else if (gss) {
        if (gss->iters < 1 || gss->iters > 64 || !(gss->lo > 0.0) || !(gss->hi > gss->lo) ||
            !std::isfinite(gss->hi))
            return fail(ctx, EXL3_EINVAL, "scale search {iters %d, lo %g, hi %g}", gss->iters,
                        gss->lo, gss->hi);
    } else if (!std::isfinite(fixed_scale)) {
        return fail(ctx, EXL3_EINVAL, "fixed scale is not finite");
    }
    {
        const size_t nel = (size_t)rows * cols, nt = nel / 256;
        if ((rc = check_span(ctx, w, nel * (w_dtype == EXL3_BF16 ? 2 : 4), "w")) != EXL3_OK ||
            (rc = check_span(ctx, su, (size_t)rows * sizeof(float), "su")) != EXL3_OK ||
            (rc = check_span(ctx, sv, (size_t)cols * sizeof(float), "sv")) != EXL3_OK ||
            (rc = check_span(ctx, packed, nt * 16 * K * sizeof(uint16_t), "packed")) !=
                EXL3_OK ||
            (rc = check_span(ctx, w_hat, nel * sizeof(float), "w_hat")) != EXL3_OK ||
            (rc = check_span(ctx, tile_out, nt * sizeof(float), "per-tile output")) !=
                EXL3_OK ||
            (rc = check_span(ctx, L, (size_t)cols * cols * sizeof(float), "L")) != EXL3_OK)
            return rc;
    }
    if ((rc = set_device(ctx)) != EXL3_OK) return rc;
    if ((rc = check_signs(ctx, su, rows, "su", sv, cols, "sv")) != EXL3_OK) return rc;

    const int TR = rows / 16, TC = cols / 16;
    const int64_t ntiles = (int64_t)TR * TC;
    const size_t nel = (size_t)rows * cols;
    if ((rc = ensure(ctx, ctx->d_wreg, ctx->wreg_cap, nel)) != EXL3_OK) return rc;
    if ((rc = ensure(ctx, ctx->d_sumsq, ctx->sumsq_cap, (size_t)ntiles)) != EXL3_OK) return rc;

    // 1. regularize (tile-major) with per-tile energy and the non-finite flag
    EXL3_HIP(ctx, hipMemsetAsync(ctx->d_flag, 0, sizeof(int), ctx->stream));
    int reg_id = open_timed(ctx, EXL3_KERNEL_REGULARIZE, ntiles);
    EXL3_HIP(ctx, exl3::launch_regularize(w, w_dtype, rows, cols, had_block, su, sv, ctx->d_wreg,
                                          EXL3_TILE_MAJOR, ctx->d_sumsq, ctx->d_flag,
                                          tile_order(ctx), ctx->n_cu, ctx->stream));
    close_timed(ctx, reg_id);
    const void *p_sumsq, *p_flag;
    if ((rc = read_back(ctx, ctx->d_sumsq, (size_t)ntiles * sizeof(float), ctx->d_flag,
                        sizeof(int), &p_sumsq, &p_flag)) != EXL3_OK)
        return rc;
    if (*static_cast<const int *>(p_flag))
        return fail(ctx, EXL3_ENONFINITE, "weight matrix holds NaN or Inf");
    // read in place: the next read-back (the chosen scale) comes after its last use
    const float *sumsq = static_cast<const float *>(p_sumsq);

    // 2. rms in binary64, ascending tile order
    double total = 0.0;
    for (int64_t i = 0; i < ntiles; ++i) total += (double)sumsq[i];
    const double rms = std::sqrt(total / (double)nel);

    // 3. scale
    float scale = fixed_scale;
    if (gss || grid) {
        if (rms == 0.0) {
            scale = 0.0f;
        } else {
            // sample: wrapped diagonal + highest / lowest energy (lowest index on ties)
            std::set<int64_t> pick;
            for (int i = 0; i < std::max(TR, TC); ++i)
                pick.insert((int64_t)(i % TR) * TC + (i % TC));
            int64_t imax = 0, imin = 0;
            for (int64_t i = 1; i < ntiles; ++i) {
                if (sumsq[i] > sumsq[imax]) imax = i;
                if (sumsq[i] < sumsq[imin]) imin = i;
            }
            pick.insert(imax);
            pick.insert(imin);
            std::vector<int32_t> sample(pick.begin(), pick.end());
            const int64_t ns = (int64_t)sample.size();
            // device index list: the sample, then (grid search) every stride-th entry of it
            std::vector<int32_t> idx_all(sample);
            int64_t ns_sub = 0;
            if (grid)
                for (size_t i = 0; i < sample.size(); i += (size_t)grid->stride, ++ns_sub)
                    idx_all.push_back(sample[i]);
            if ((rc = ensure(ctx, ctx->d_idx, ctx->idx_cap, idx_all.size())) != EXL3_OK) return rc;
            if ((rc = ensure(ctx, ctx->d_sse, ctx->sse_cap,
                             std::max<size_t>((size_t)ns, (size_t)ntiles))) != EXL3_OK)
                return rc;
            EXL3_HIP(ctx, hipMemcpyAsync(ctx->d_idx, idx_all.data(),
                                         idx_all.size() * sizeof(int32_t),
                                         hipMemcpyHostToDevice, ctx->stream));
            std::vector<float> costs((size_t)ns);
            int err = EXL3_OK;
            if (f16) {
                // binary16 probes work on a contiguous copy of the sample
                if ((rc = ensure(ctx, ctx->d_gs, ctx->gs_cap, (size_t)ns * 256)) != EXL3_OK ||
                    (rc = ensure(ctx, ctx->d_x16, ctx->x16_cap, (size_t)ns * 256)) != EXL3_OK ||
                    (rc = ensure(ctx, ctx->d_pk, ctx->pk_cap, (size_t)ns * 16 * K)) != EXL3_OK)
                    return rc;
                EXL3_HIP(ctx, exl3::launch_gather_tiles(ctx->d_wreg, ctx->d_idx, ns, ctx->d_gs,
                                                        ctx->stream));
            }
            // binary16 mode: the binary64 sum, in ascending tile order, of the
            // sample's path costs at scale (float)s (the search on fp16(w / s);
            // the traceback scores the dequantized tiles in binary32)
            auto objective_f16 = [&](double s) -> double {
                if (err != EXL3_OK) return 0.0;
                const int64_t cnt = ns;
                hipError_t e = exl3::launch_to_f16(ctx->d_gs, nullptr, cnt, (float)s, ctx->d_x16,
                                                   ctx->stream);
                int r = e == hipSuccess
                            ? encode_chain_f16(ctx, ctx->d_x16, cnt, K, ctx->d_pk, nullptr,
                                               nullptr, ctx->d_gs, (float)s, ctx->d_sse)
                            : fail(ctx, EXL3_EHIP, "binary16 inputs: %s", hipGetErrorString(e));
                if (r == EXL3_OK) {
                    hipError_t e = hipMemcpyAsync(costs.data(), ctx->d_sse,
                                                  (size_t)cnt * sizeof(float),
                                                  hipMemcpyDeviceToHost, ctx->stream);
                    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
                    if (e != hipSuccess)
                        r = fail(ctx, EXL3_EHIP, "scale-search readback: %s",
                                 hipGetErrorString(e));
                }
                if (r != EXL3_OK) {
                    err = r;
                    return 0.0;
                }
                double f = 0.0;
                for (int64_t i = 0; i < cnt; ++i) f += (double)costs[(size_t)i];
                return f;
            };
            // grid search (binary32): the objective of each scale in ss, the
            // binary64 sum in ascending tile order of the path costs of the tiles
            // idx_all[off .. off + cnt) at (float)s.  Every point's tiles go in
            // one batch, each tile with its point's scale (a tile's cost does not
            // depend on what else is in the batch), with one read-back.
            auto objectives_on = [&](const std::vector<double> &ss, int64_t off,
                                     int64_t cnt) -> std::vector<double> {
                std::vector<double> f(ss.size(), 0.0);
                if (err != EXL3_OK) return f;
                const size_t np = ss.size(), nt = np * (size_t)cnt;
                std::vector<int32_t> bidx(nt);
                std::vector<float> bscale(nt);
                for (size_t q = 0; q < np; ++q)
                    for (int64_t i = 0; i < cnt; ++i) {
                        bidx[q * (size_t)cnt + (size_t)i] = idx_all[(size_t)(off + i)];
                        bscale[q * (size_t)cnt + (size_t)i] = (float)ss[q];
                    }
                int r;
                if ((r = ensure(ctx, ctx->d_bidx, ctx->bidx_cap, nt)) != EXL3_OK ||
                    (r = ensure(ctx, ctx->d_bscale, ctx->bscale_cap, nt)) != EXL3_OK ||
                    (r = ensure(ctx, ctx->d_sse, ctx->sse_cap, nt)) != EXL3_OK) {
                    err = r;
                    return f;
                }
                hipError_t e = hipMemcpyAsync(ctx->d_bidx, bidx.data(), nt * sizeof(int32_t),
                                              hipMemcpyHostToDevice, ctx->stream);
                if (e == hipSuccess)
                    e = hipMemcpyAsync(ctx->d_bscale, bscale.data(), nt * sizeof(float),
                                       hipMemcpyHostToDevice, ctx->stream);
                if (e != hipSuccess) {
                    err = fail(ctx, EXL3_EHIP, "scale-search batch: %s", hipGetErrorString(e));
                    (void)hipStreamSynchronize(ctx->stream);   // bidx, bscale read by then
                    return f;
                }
                r = encode_chain(ctx, ctx->d_wreg, ctx->d_bidx, (int64_t)nt, K, 0.0f, nullptr,
                                 nullptr, nullptr, nullptr, ctx->d_sse, ctx->d_bscale, true);
                const void *pc = nullptr;
                // (read_back synchronizes the stream: the uploads are done by then)
                if (r == EXL3_OK)
                    r = read_back(ctx, ctx->d_sse, nt * sizeof(float), nullptr, 0, &pc);
                if (r != EXL3_OK) {
                    err = r;
                    (void)hipStreamSynchronize(ctx->stream);   // bidx, bscale read by then
                    return f;
                }
                const float *c = static_cast<const float *>(pc);
                for (size_t q = 0; q < np; ++q) {
                    double sum = 0.0;
                    for (int64_t i = 0; i < cnt; ++i)
                        sum += (double)c[q * (size_t)cnt + (size_t)i];
                    f[q] = sum;
                }
                return f;
            };
            if (grid) {
                auto scaled = [&](const std::vector<double> &ms) {
                    std::vector<double> ss;
                    for (double m : ms) ss.push_back(m * rms);
                    return ss;
                };
                const double mult = grid_search(
                    *grid,
                    [&](const std::vector<double> &ms) {
                        return objectives_on(scaled(ms), ns, ns_sub);
                    },
                    [&](const std::vector<double> &ms) { return objectives_on(scaled(ms), 0, ns); });
                if (err != EXL3_OK) return err;
                *scale_chosen = (float)(mult * rms);
                return EXL3_OK;
            }
            const double g = (std::sqrt(5.0) - 1.0) / 2.0;
            double a = gss->lo * rms, b = gss->hi * rms;
            double p = b - (b - a) * g, q = a + (b - a) * g;
            if (!f16) {
                // The whole search enqueued at once, no host round trip between
                // probes: each probe after the first reads its scale from device
                // memory, written by the search step before it (the result is
                // read back once, at the end).  The last reduction's point is
                // not scored (the result never reads it): iters + 1 probes.
                const int probes = gss->iters >= 1 ? gss->iters + 1 : 2;
                const float *scale_dev = &ctx->d_gss->scale;
                for (int k = 0; k < probes; ++k) {
                    if ((rc = encode_chain(ctx, ctx->d_wreg, ctx->d_idx, ns, K, (float)p, nullptr,
                                           nullptr, nullptr, nullptr, ctx->d_sse,
                                           k == 0 ? nullptr : scale_dev)) != EXL3_OK)
                        return rc;
                    hipLaunchKernelGGL(gss_step_kernel, dim3(1), dim3(64), 0, ctx->stream,
                                       ctx->d_gss, ctx->d_sse, ns, a, b, p, q, g, gss->iters, k);
                    EXL3_HIP(ctx, hipGetLastError());
                }
                const void *p_scale;
                if ((rc = read_back(ctx, scale_dev, sizeof(float), nullptr, 0, &p_scale)) !=
                    EXL3_OK)
                    return rc;
                *scale_chosen = *static_cast<const float *>(p_scale);
                return EXL3_OK;
            }
            // The result is the midpoint of the last bracket, which the last
            // reduction sets before its new point is scored: that score can
            // never be read, so it is not computed (iters + 1 probes in all).
            double fp = objective_f16(p), fq = objective_f16(q);
            for (int it = 0; it < gss->iters && err == EXL3_OK; ++it) {
                const bool last = it + 1 == gss->iters;
                if (fp < fq) {
                    b = q;
                    q = p;
                    fq = fp;
                    p = b - (b - a) * g;
                    if (!last) fp = objective_f16(p);
                } else {
                    a = p;
                    p = q;
                    fp = fq;
                    q = a + (b - a) * g;
                    if (!last) fq = objective_f16(q);
                }
            }
            if (err != EXL3_OK) return err;
            scale = (float)((a + b) / 2.0);
        }
    }

    *scale_chosen = scale;
    return EXL3_OK;
}

// Final encode of every tile of the regularized matrix at the chosen scale,
// the mean squared error in binary64 (ascending tile order) and the scale.
int encode_whole_matrix(exl3_ctx *ctx, int rows, int cols, int K, float scale, uint16_t *packed,
                        float *scale_out, double *mse_out, float *w_hat, float *tile_sse) {
    int rc;
    const int64_t ntiles = (int64_t)(rows / 16) * (cols / 16);
    const size_t nel = (size_t)rows * cols;
    // 4. final encode of every tile at the chosen scale
    float *sse_dev = tile_sse;
    if (!sse_dev) {
        if ((rc = ensure(ctx, ctx->d_sse, ctx->sse_cap, (size_t)ntiles)) != EXL3_OK) return rc;
        sse_dev = ctx->d_sse;
    }
    if ((rc = encode_chain(ctx, ctx->d_wreg, nullptr, ntiles, K, scale, packed, nullptr, sse_dev,
                           w_hat, nullptr)) != EXL3_OK)
        return rc;
    if (mse_out) {
        const void *p;
        if ((rc = read_back(ctx, sse_dev, (size_t)ntiles * sizeof(float), nullptr, 0, &p)) !=
            EXL3_OK)
            return rc;
        const float *sse = static_cast<const float *>(p);
        double tot = 0.0;
        for (int64_t i = 0; i < ntiles; ++i) tot += (double)sse[i];
        *mse_out = tot / (double)nel;
    }
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    *scale_out = scale;
    return EXL3_OK;
}

}  // namespace

extern "C" {

int exl3_quantize_matrix(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols, int K,
                         int had_block, const float *su, const float *sv, const exl3_gss *gss,
                         float fixed_scale, uint16_t *packed, float *scale_out, double *mse_out,
                         float *w_hat, float *tile_sse) {
    float scale = 0.0f;
    int rc = regularize_and_choose_scale(ctx, w, w_dtype, rows, cols, K, had_block, su, sv, gss,
                                         nullptr, fixed_scale, packed, scale_out, &scale, w_hat,
                                         tile_sse, nullptr);
    if (rc != EXL3_OK) return rc;
    return encode_whole_matrix(ctx, rows, cols, K, scale, packed, scale_out, mse_out, w_hat,
                               tile_sse);
}

int exl3_quantize_matrix_grid(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                              int K, int had_block, const float *su, const float *sv,
                              const exl3_grid *grid, uint16_t *packed, float *scale_out,
                              double *mse_out, float *w_hat, float *tile_sse) {
    if (!ctx) return EXL3_EINVAL;
    if (!grid) return fail(ctx, EXL3_EINVAL, "null grid");
    float scale = 0.0f;
    int rc = regularize_and_choose_scale(ctx, w, w_dtype, rows, cols, K, had_block, su, sv,
                                         nullptr, grid, 0.0f, packed, scale_out, &scale, w_hat,
                                         tile_sse, nullptr);
    if (rc != EXL3_OK) return rc;
    return encode_whole_matrix(ctx, rows, cols, K, scale, packed, scale_out, mse_out, w_hat,
                               tile_sse);
}

int exl3_quantize_matrix_f16(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                             int K, int had_block, const float *su, const float *sv,
                             const exl3_gss *gss, float fixed_scale, uint16_t *packed,
                             float *scale_out, double *mse_out, float *w_hat, float *tile_sse) {
    if (!ctx) return EXL3_EINVAL;
    float scale = 0.0f;
    int rc = regularize_and_choose_scale(ctx, w, w_dtype, rows, cols, K, had_block, su, sv, gss,
                                         nullptr, fixed_scale, packed, scale_out, &scale, w_hat,
                                         tile_sse, nullptr, true);
    if (rc != EXL3_OK) return rc;
    const int64_t ntiles = (int64_t)(rows / 16) * (cols / 16);
    const size_t nel = (size_t)rows * cols;
    float *sse_dev = tile_sse;
    if (!sse_dev) {
        if ((rc = ensure(ctx, ctx->d_sse, ctx->sse_cap, (size_t)ntiles)) != EXL3_OK) return rc;
        sse_dev = ctx->d_sse;
    }
    if ((rc = ensure(ctx, ctx->d_x16, ctx->x16_cap, (size_t)ntiles * 256)) != EXL3_OK) return rc;
    EXL3_HIP(ctx, exl3::launch_to_f16(ctx->d_wreg, nullptr, ntiles, scale, ctx->d_x16,
                                      ctx->stream));
    if ((rc = encode_chain_f16(ctx, ctx->d_x16, ntiles, K, packed, nullptr, nullptr, ctx->d_wreg,
                               scale, sse_dev, w_hat)) != EXL3_OK)
        return rc;
    const void *p_sse;
    if ((rc = read_back(ctx, sse_dev, (size_t)ntiles * sizeof(float), nullptr, 0, &p_sse)) !=
        EXL3_OK)
        return rc;
    const float *sse = static_cast<const float *>(p_sse);
    if (mse_out) {
        double tot = 0.0;
        for (int64_t i = 0; i < ntiles; ++i) tot += (double)sse[i];
        *mse_out = tot / (double)nel;
    }
    *scale_out = scale;
    return EXL3_OK;
}

int exl3_quantize_matrix_ldlq(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                              int K, int had_block, const float *su, const float *sv,
                              const exl3_gss *gss, float fixed_scale, const float *L,
                              uint16_t *packed, float *scale_out, double *mse_out, float *w_hat,
                              float *tile_err) {
    if (!ctx) return EXL3_EINVAL;
    if (!L) return fail(ctx, EXL3_EINVAL, "null factor L");
    float scale = 0.0f;
    int rc = regularize_and_choose_scale(ctx, w, w_dtype, rows, cols, K, had_block, su, sv, gss,
                                         nullptr, fixed_scale, packed, scale_out, &scale, w_hat,
                                         tile_err, L);
    if (rc != EXL3_OK) return rc;
    const int TR = rows / 16, TC = cols / 16;
    const int64_t ntiles = (int64_t)TR * TC;
    const size_t nel = (size_t)rows * cols;
    if ((rc = ensure(ctx, ctx->d_err_tiles, ctx->err_tiles_cap, nel)) != EXL3_OK) return rc;
    if ((rc = ensure(ctx, ctx->d_span_target, ctx->span_target_cap, (size_t)TR * 256)) != EXL3_OK)
        return rc;
    if ((rc = ensure(ctx, ctx->d_span_what, ctx->span_what_cap, (size_t)TR * 256)) != EXL3_OK)
        return rc;
    if ((rc = ensure(ctx, ctx->d_span_packed, ctx->span_packed_cap, (size_t)TR * 16 * K)) !=
        EXL3_OK)
        return rc;
    float *err_dev = tile_err;
    if (!err_dev) {
        if ((rc = ensure(ctx, ctx->d_sse, ctx->sse_cap, (size_t)ntiles)) != EXL3_OK) return rc;
        err_dev = ctx->d_sse;
    }
    // spans from the last tile column to the first: target, encode, commit
    for (int j = TC - 1; j >= 0; --j) {
        EXL3_HIP(ctx, exl3::launch_ldlq_target(ctx->d_wreg, ctx->d_err_tiles, L, TR, TC, j,
                                               tile_order_inv(ctx),
                                               ctx->d_span_target, ctx->stream));
        if ((rc = encode_chain(ctx, ctx->d_span_target, nullptr, TR, K, scale, ctx->d_span_packed,
                               nullptr, nullptr, ctx->d_span_what, nullptr)) != EXL3_OK)
            return rc;
        EXL3_HIP(ctx, exl3::launch_ldlq_commit(ctx->d_wreg, ctx->d_span_what, ctx->d_span_packed,
                                               TR, TC, j, K, packed, ctx->d_err_tiles, w_hat,
                                               err_dev, ctx->stream));
    }
    if (mse_out) {
        const void *p_err;
        if ((rc = read_back(ctx, err_dev, (size_t)ntiles * sizeof(float), nullptr, 0, &p_err)) !=
            EXL3_OK)
            return rc;
        const float *err = static_cast<const float *>(p_err);
        double tot = 0.0;
        for (int64_t i = 0; i < ntiles; ++i) tot += (double)err[i];
        *mse_out = tot / (double)nel;
    }
    EXL3_HIP(ctx, hipStreamSynchronize(ctx->stream));
    *scale_out = scale;
    return EXL3_OK;
}

}  // extern "C"
