// api.hip -- the extern "C" entry points declared in include/fp8q.h.
//
// Host-side validation happens before any HIP call, so argument errors are
// reported without touching the device; valid calls only enqueue kernels on
// the caller's stream.  Messages for the last error are thread-local.
//
// Reduction scratch.  Calls that reduce over a grid (an amax, the cast
// statistics) fold per-block partials in a small scratch slot and finish with
// a one-block kernel that reads the slot and leaves it zero.  The slots are
// one device global, `scratch` below: kScratchSlots slots of 6 KiB on every
// device the library runs on, held until the process ends.  The library never
// allocates device memory.  Each stream that runs a reducing call gets a slot
// of its own on first use (a host-side table, no device work), so calls on
// different streams never share partials; a host mutex per slot is held while
// one call enqueues its kernels, so calls from several host threads on one
// stream cannot interleave their partials.  A device with more than
// kScratchSlots such streams returns FP8Q_EUNSUPPORTED.
//
// FP8Q_DEBUG (environment, read once): when set to a non-empty value other
// than "0", every call prints one line to stderr -- the entry point, its sizes
// and formats, the stream and scratch slot, and the status with its message.
// The line is written after the kernels are enqueued; it never waits for the
// device.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <thread>
#include <utility>

#include "fp8q.h"
#include "fp8q_launch.h"

// Every device's reduction scratch (zero-initialised when the code object is
// loaded on the device).  Host code never takes this name as a device
// address: the address on the current device comes from hipGetSymbolAddress.
static __device__ __align__(256) fp8q::GridScratch scratch[fp8q::kScratchSlots];

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return FP8Q_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(FP8Q_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool debug_enabled()
{
    static const bool on = [] {
        const char *v = std::getenv("FP8Q_DEBUG");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// ------------------------------------------------------ scratch slots ----
constexpr int kMaxDevices = 64;

struct Slot {
    std::mutex mu;      // held across the launches of one call
    bool dirty = false; // a failed call may have left partials in the slot
    uint32_t tag = 0;   // the tag of the slot's last call (tags are nonzero)
};

// Bound on a finishing block's polling rounds (fp8q_set_finish_poll_rounds).
std::atomic<uint32_t> g_poll_rounds{fp8q::kPollRounds};

struct StreamKey {
    hipStream_t s;
    std::thread::id thread; // only for the per-thread default stream, whose handle is shared
    bool operator<(const StreamKey &o) const { return s != o.s ? s < o.s : thread < o.thread; }
};

struct DeviceScratch {
    std::once_flag once;
    hipError_t err = hipSuccess;
    fp8q::GridScratch *base = nullptr; // address of `scratch` on this device
    Slot slots[fp8q::kScratchSlots];
    std::map<StreamKey, int> slot_of; // guarded by g_table_mu
};

DeviceScratch g_devices[kMaxDevices];
std::mutex g_table_mu;

// The scratch slot of the current device and stream `s`, locked for the
// duration of one call.
class ScratchLease {
public:
    // FP8Q_OK, or an error status with its message set
    int acquire(const char *fn, hipStream_t s)
    {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_status(e, fn);
        if (dev < 0 || dev >= kMaxDevices) return fail(FP8Q_EUNSUPPORTED, "%s: device %d out of range", fn, dev);
        DeviceScratch &d = g_devices[dev];
        // once per device, with that device current
        std::call_once(d.once, [&d] { d.err = hipGetSymbolAddress((void **)&d.base, HIP_SYMBOL(scratch)); });
        if (d.err != hipSuccess) return hip_status(d.err, fn);
        int idx;
        {
            std::lock_guard<std::mutex> lock(g_table_mu);
            const StreamKey key{s, s == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
            auto it = d.slot_of.find(key);
            if (it != d.slot_of.end()) {
                idx = it->second;
            } else {
                if ((int)d.slot_of.size() >= fp8q::kScratchSlots)
                    return fail(FP8Q_EUNSUPPORTED,
                                "%s: more than %d streams on device %d have run reducing calls (scratch slots)", fn,
                                fp8q::kScratchSlots, dev);
                idx = (int)d.slot_of.size();
                d.slot_of.emplace(key, idx);
            }
        }
        slot_ = &d.slots[idx];
        lock_ = std::unique_lock<std::mutex>(slot_->mu);
        index_ = idx;
        gs = d.base + idx;
        if (slot_->dirty) {
            e = fp8q::launch_clear_scratch(gs, s);
            if (e != hipSuccess) return hip_status(e, fn);
            slot_->dirty = false;
        }
        if (++slot_->tag == 0) ++slot_->tag;
        tag = slot_->tag;
        return FP8Q_OK;
    }
    // record the outcome of the call's launches
    int settle(int status)
    {
        if (slot_ && status != FP8Q_OK) slot_->dirty = true;
        return status;
    }
    int index() const { return index_; }
    fp8q::GridScratch *gs = nullptr;
    uint32_t tag = 0;

private:
    Slot *slot_ = nullptr;
    int index_ = -1;
    std::unique_lock<std::mutex> lock_;
};

// One entry-point call: its optional scratch lease and its debug line.
class Call {
public:
    Call(const char *fn, void *stream) : fn_(fn), stream_(stream) { args_[0] = '\0'; }
    ~Call()
    {
        if (!debug_enabled()) return;
        std::fprintf(stderr, "fp8q: %s(%s) stream=%p slot=%d -> %d%s%s\n", fn_, args_, stream_, lease_.index(),
                     status_, status_ ? " " : "", status_ ? g_err : "");
        std::fflush(stderr);
    }
    // sizes and formats for the debug line (formatted only when it is on)
    void args(const char *fmt, ...)
    {
        if (!debug_enabled()) return;
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(args_, sizeof(args_), fmt, ap);
        va_end(ap);
    }
    int scratch(fp8q::GridScratch **gs)
    {
        const int st = lease_.acquire(fn_, (hipStream_t)stream_);
        *gs = st == FP8Q_OK ? lease_.gs : nullptr;
        return st;
    }
    // the slot, this call's tag and the polling bound of its finishing block
    int scratch(fp8q::Reduce *r)
    {
        const int st = lease_.acquire(fn_, (hipStream_t)stream_);
        *r = st == FP8Q_OK ? fp8q::Reduce{lease_.gs, lease_.tag, g_poll_rounds.load(std::memory_order_relaxed)}
                           : fp8q::Reduce{nullptr, 0u, 0u};
        return st;
    }
    int ret(int status)
    {
        status_ = lease_.settle(status);
        return status_;
    }
    int launched(hipError_t e) { return ret(hip_status(e, fn_)); }

private:
    const char *fn_;
    void *stream_;
    char args_[192];
    int status_ = FP8Q_OK;
    ScratchLease lease_;
};

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_fmt(int32_t f) { return f == FP8Q_E4M3FN || f == FP8Q_E5M2; }
bool valid_dtype(int32_t d) { return d == FP8Q_F32 || d == FP8Q_BF16; }
int64_t dsize(int32_t d) { return d == FP8Q_F32 ? 4 : 2; }

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Scale-source checks shared by the per-tensor quantizers.
int check_scale_src(const char *fn, const float *amax_in, const float *scale_inv_in, const float *scale_inv_out,
                    const float *scale_out, const float *amax_out)
{
    if ((amax_in == nullptr) == (scale_inv_in == nullptr))
        return fail(FP8Q_EINVAL, "%s: exactly one of amax_in / scale_inv_in must be given", fn);
    const float *in = amax_in ? amax_in : scale_inv_in;
    if (!aligned(in, 4)) return fail(FP8Q_EINVAL, "%s: scale input not 4-byte aligned", fn);
    const float *outs[3] = {scale_inv_out, scale_out, amax_out};
    for (const float *o : outs) {
        if (!o) continue;
        if (!aligned(o, 4)) return fail(FP8Q_EINVAL, "%s: scalar output not 4-byte aligned", fn);
        if (o == in) return fail(FP8Q_EINVAL, "%s: a scalar output aliases the scale input", fn);
    }
    if ((scale_inv_out && (scale_inv_out == scale_out || scale_inv_out == amax_out)) ||
        (scale_out && scale_out == amax_out))
        return fail(FP8Q_EINVAL, "%s: scalar outputs alias each other", fn);
    return FP8Q_OK;
}

fp8q::ScaleSrc make_src(const float *amax_in, int32_t margin, const float *scale_inv_in)
{
    return fp8q::ScaleSrc{amax_in, scale_inv_in, (int)margin};
}

} // namespace

extern "C" const char *fp8q_last_error(void) { return g_err; }

static int fp8q_clock_monitor_impl(uint64_t *out, const uint32_t *stop, void *stream)
{
    const char *fn = "fp8q_clock_monitor";
    if (!out || !aligned(out, 8)) return fail(FP8Q_EINVAL, "%s: out must be an 8-byte aligned pointer", fn);
    if (!stop || !aligned(stop, 4)) return fail(FP8Q_EINVAL, "%s: stop must be a 4-byte aligned pointer", fn);
    if (overlap(out, 8 * (3 * fp8q::kClockBlocks + 1), stop, 4))
        return fail(FP8Q_EINVAL, "%s: stop overlaps out", fn);
    return hip_status(fp8q::launch_clock_monitor(out, stop, (hipStream_t)stream), fn);
}

extern "C" int fp8q_clock_monitor(uint64_t *out, const uint32_t *stop, void *stream)
{
    Call c("fp8q_clock_monitor", stream);
    return c.ret(fp8q_clock_monitor_impl(out, stop, stream));
}

extern "C" int fp8q_set_finish_poll_rounds(uint32_t rounds, uint32_t *previous)
{
    const uint32_t was = g_poll_rounds.exchange(rounds == 0xFFFFFFFFu ? fp8q::kPollRounds : rounds);
    if (previous) *previous = was;
    return ok();
}

static int fp8_amax_impl(Call &c, const void *x, int32_t dtype, int64_t n, float *amax, void *stream)
{
    const char *fn = "fp8_amax";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (n < 0) return fail(FP8Q_EINVAL, "%s: negative n", fn);
    if (!amax || !aligned(amax, 4)) return fail(FP8Q_EINVAL, "%s: amax must be a 4-byte aligned pointer", fn);
    if (n > 0 && (!x || !aligned(x, 16))) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
    if (overlap(x, n * dsize(dtype), amax, 4)) return fail(FP8Q_EINVAL, "%s: amax overlaps x", fn);
    fp8q::Reduce r{};
    const int st = c.scratch(&r);
    if (st) return st;
    return hip_status(fp8q::launch_amax(x, dtype, n, amax, r, (hipStream_t)stream), fn);
}

extern "C" int fp8_amax(const void *x, int32_t dtype, int64_t n, float *amax, void *stream)
{
    Call c("fp8_amax", stream);
    c.args("dtype=%lld n=%lld", (long long)dtype, (long long)n);
    return c.ret(fp8_amax_impl(c, x, dtype, n, amax, stream));
}

// fp8_quantize_tensor and, with stats, fp8_quantize_tensor_stats
static int quantize_tensor(Call &c, const char *fn, const void *x, int32_t dtype, int64_t n, int32_t fmt,
                           const float *amax_in, int32_t margin, const float *scale_inv_in, uint8_t *q,
                           float *scale_inv_out, float *scale_out, float *amax_out, uint64_t *stats, void *stream)
{
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (n < 0) return fail(FP8Q_EINVAL, "%s: negative n", fn);
    int st = check_scale_src(fn, amax_in, scale_inv_in, scale_inv_out, scale_out, amax_out);
    if (st) return st;
    if (stats) {
        const float *scalars[4] = {amax_in ? amax_in : scale_inv_in, scale_inv_out, scale_out, amax_out};
        if (!aligned(stats, 8)) return fail(FP8Q_EINVAL, "%s: stats must be an 8-byte aligned pointer", fn);
        for (const float *p : scalars)
            if (overlap(stats, 32, p, p ? 4 : 0)) return fail(FP8Q_EINVAL, "%s: stats overlaps a scalar", fn);
    }
    if (n > 0) {
        if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
        if (!q || !aligned(q, 16)) return fail(FP8Q_EINVAL, "%s: q must be a 16-byte aligned pointer", fn);
        if (overlap(x, n * dsize(dtype), q, n)) return fail(FP8Q_EINVAL, "%s: q overlaps x", fn);
        if (stats && (overlap(x, n * dsize(dtype), stats, 32) || overlap(q, n, stats, 32)))
            return fail(FP8Q_EINVAL, "%s: stats overlaps x or q", fn);
    }
    fp8q::Reduce r{};
    if (amax_out || stats) {
        const int st = c.scratch(&r);
        if (st) return st;
    }
    return hip_status(fp8q::launch_cast(x, dtype, n, fmt, make_src(amax_in, margin, scale_inv_in), q, scale_inv_out,
                                        scale_out, amax_out, stats, r, (hipStream_t)stream),
                      fn);
}

static int fp8_quantize_tensor_impl(Call &c, const void *x, int32_t dtype, int64_t n, int32_t fmt,
                                    const float *amax_in, int32_t margin, const float *scale_inv_in, uint8_t *q,
                                    float *scale_inv_out, float *scale_out, float *amax_out, void *stream)
{
    return quantize_tensor(c, "fp8_quantize_tensor", x, dtype, n, fmt, amax_in, margin, scale_inv_in, q, scale_inv_out,
                           scale_out, amax_out, nullptr, stream);
}

extern "C" int fp8_quantize_tensor(const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *amax_in,
                                   int32_t margin, const float *scale_inv_in, uint8_t *q, float *scale_inv_out,
                                   float *scale_out, float *amax_out, void *stream)
{
    Call c("fp8_quantize_tensor", stream);
    c.args("dtype=%lld n=%lld fmt=%lld margin=%lld", (long long)dtype, (long long)n, (long long)fmt, (long long)margin);
    return c.ret(fp8_quantize_tensor_impl(c, x, dtype, n, fmt, amax_in, margin, scale_inv_in, q, scale_inv_out, scale_out, amax_out, stream));
}

static int fp8_quantize_tensor_stats_impl(Call &c, const void *x, int32_t dtype, int64_t n, int32_t fmt,
                                          const float *amax_in, int32_t margin, const float *scale_inv_in, uint8_t *q,
                                          float *scale_inv_out, float *scale_out, float *amax_out, uint64_t *stats,
                                          void *stream)
{
    const char *fn = "fp8_quantize_tensor_stats";
    if (!stats) return fail(FP8Q_EINVAL, "%s: stats must be given", fn);
    return quantize_tensor(c, fn, x, dtype, n, fmt, amax_in, margin, scale_inv_in, q, scale_inv_out, scale_out, amax_out,
                           stats, stream);
}

extern "C" int fp8_quantize_tensor_stats(const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *amax_in,
                                         int32_t margin, const float *scale_inv_in, uint8_t *q, float *scale_inv_out,
                                         float *scale_out, float *amax_out, uint64_t *stats, void *stream)
{
    Call c("fp8_quantize_tensor_stats", stream);
    c.args("dtype=%lld n=%lld fmt=%lld margin=%lld", (long long)dtype, (long long)n, (long long)fmt, (long long)margin);
    return c.ret(fp8_quantize_tensor_stats_impl(c, x, dtype, n, fmt, amax_in, margin, scale_inv_in, q, scale_inv_out, scale_out, amax_out, stats, stream));
}

static int fp8_dequantize_impl(Call &c, const uint8_t *q, int32_t fmt, int64_t n, const float *scale_inv, float *y, void *stream)
{
    const char *fn = "fp8_dequantize";
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (n < 0) return fail(FP8Q_EINVAL, "%s: negative n", fn);
    if (!scale_inv || !aligned(scale_inv, 4)) return fail(FP8Q_EINVAL, "%s: scale_inv must be 4-byte aligned", fn);
    if (n > 0) {
        if (!q || !aligned(q, 16)) return fail(FP8Q_EINVAL, "%s: q must be a 16-byte aligned pointer", fn);
        if (!y || !aligned(y, 16)) return fail(FP8Q_EINVAL, "%s: y must be a 16-byte aligned pointer", fn);
        if (overlap(q, n, y, 4 * n)) return fail(FP8Q_EINVAL, "%s: y overlaps q", fn);
    }
    return hip_status(fp8q::launch_dequant(q, fmt, n, scale_inv, y, (hipStream_t)stream), fn);
}

extern "C" int fp8_dequantize(const uint8_t *q, int32_t fmt, int64_t n, const float *scale_inv, float *y, void *stream)
{
    Call c("fp8_dequantize", stream);
    c.args("fmt=%lld n=%lld", (long long)fmt, (long long)n);
    return c.ret(fp8_dequantize_impl(c, q, fmt, n, scale_inv, y, stream));
}

static int fp8_quantize_rowwise_colwise_impl(Call &c, const void *x, int32_t dtype, int64_t rows, int64_t cols,
                                             int32_t fmt, const float *amax_in, int32_t margin,
                                             const float *scale_inv_in, uint8_t *q_row, uint8_t *q_col,
                                             float *scale_inv_out, float *scale_out, float *amax_out, void *stream)
{
    const char *fn = "fp8_quantize_rowwise_colwise";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (rows < 0 || cols < 0) return fail(FP8Q_EINVAL, "%s: negative shape", fn);
    if (rows % 16 || cols % 16) return fail(FP8Q_EUNSUPPORTED, "%s: rows and cols must be multiples of 16", fn);
    if (!q_row && !q_col) return fail(FP8Q_EINVAL, "%s: at least one of q_row / q_col is needed", fn);
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31)
        return fail(FP8Q_EUNSUPPORTED, "%s: a dimension exceeds 2^31", fn);
    int st = check_scale_src(fn, amax_in, scale_inv_in, scale_inv_out, scale_out, amax_out);
    if (st) return st;
    const int64_t n = rows * cols;
    if (n > 0) {
        if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
        if ((q_row && !aligned(q_row, 16)) || (q_col && !aligned(q_col, 16)))
            return fail(FP8Q_EINVAL, "%s: q_row / q_col must be 16-byte aligned", fn);
        if (overlap(x, n * dsize(dtype), q_row, n) || overlap(x, n * dsize(dtype), q_col, n) ||
            overlap(q_row, n, q_col, n))
            return fail(FP8Q_EINVAL, "%s: output buffers overlap", fn);
    }
    fp8q::Reduce r{};
    if (amax_out) {
        const int st = c.scratch(&r);
        if (st) return st;
    }
    return hip_status(fp8q::launch_rowwise_colwise(x, dtype, rows, cols, fmt, make_src(amax_in, margin, scale_inv_in),
                                                   q_row, q_col, scale_inv_out, scale_out, amax_out, r,
                                                   (hipStream_t)stream),
                      fn);
}

extern "C" int fp8_quantize_rowwise_colwise(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt,
                                            const float *amax_in, int32_t margin, const float *scale_inv_in,
                                            uint8_t *q_row, uint8_t *q_col, float *scale_inv_out, float *scale_out,
                                            float *amax_out, void *stream)
{
    Call c("fp8_quantize_rowwise_colwise", stream);
    c.args("dtype=%lld rows=%lld cols=%lld fmt=%lld margin=%lld", (long long)dtype, (long long)rows, (long long)cols, (long long)fmt, (long long)margin);
    return c.ret(fp8_quantize_rowwise_colwise_impl(c, x, dtype, rows, cols, fmt, amax_in, margin, scale_inv_in, q_row, q_col, scale_inv_out, scale_out, amax_out, stream));
}

static int fp8_quantize_block_impl(Call &c, const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt,
                                   int32_t block_rows, uint8_t *q_row, float *s_row, uint8_t *q_col, float *s_col,
                                   void *stream)
{
    const char *fn = "fp8_quantize_block";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (block_rows != 1 && block_rows != 128) return fail(FP8Q_EINVAL, "%s: block_rows must be 1 or 128", fn);
    if (rows < 0 || cols < 0) return fail(FP8Q_EINVAL, "%s: negative shape", fn);
    if (rows % 128 || cols % 128) return fail(FP8Q_EUNSUPPORTED, "%s: rows and cols must be multiples of 128", fn);
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31)
        return fail(FP8Q_EUNSUPPORTED, "%s: a dimension exceeds 2^31", fn);
    if ((q_col == nullptr) != (s_col == nullptr)) return fail(FP8Q_EINVAL, "%s: give both q_col and s_col or neither", fn);
    const int64_t n = rows * cols;
    if (n == 0) return ok();
    if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
    if (!q_row || !aligned(q_row, 16) || !s_row || !aligned(s_row, 4))
        return fail(FP8Q_EINVAL, "%s: q_row (16-byte) and s_row (4-byte) must be aligned pointers", fn);
    if (q_col && (!aligned(q_col, 16) || !aligned(s_col, 4)))
        return fail(FP8Q_EINVAL, "%s: q_col / s_col misaligned", fn);
    const int64_t ns_row = (rows / block_rows) * (cols / 128) * 4;
    const int64_t ns_col = (block_rows == 128 ? (cols / 128) * (rows / 128) : cols * (rows / 128)) * 4;
    if (overlap(x, n * dsize(dtype), q_row, n) || overlap(x, n * dsize(dtype), q_col, n) || overlap(q_row, n, q_col, n) ||
        overlap(s_row, ns_row, s_col, ns_col) || overlap(q_row, n, s_row, ns_row) || overlap(q_col, n, s_col, ns_col) ||
        overlap(x, n * dsize(dtype), s_row, ns_row) || overlap(x, n * dsize(dtype), s_col, ns_col))
        return fail(FP8Q_EINVAL, "%s: buffers overlap", fn);
    return hip_status(fp8q::launch_block(x, dtype, rows, cols, fmt, block_rows, q_row, s_row, q_col, s_col,
                                         (hipStream_t)stream),
                      fn);
}

extern "C" int fp8_quantize_block(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt,
                                  int32_t block_rows, uint8_t *q_row, float *s_row, uint8_t *q_col, float *s_col,
                                  void *stream)
{
    Call c("fp8_quantize_block", stream);
    c.args("dtype=%lld rows=%lld cols=%lld fmt=%lld block_rows=%lld", (long long)dtype, (long long)rows, (long long)cols, (long long)fmt, (long long)block_rows);
    return c.ret(fp8_quantize_block_impl(c, x, dtype, rows, cols, fmt, block_rows, q_row, s_row, q_col, s_col, stream));
}

static int fp8_quantize_mx_impl(Call &c, const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt,
                                uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col, void *stream)
{
    const char *fn = "fp8_quantize_mx";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (rows < 0 || cols < 0) return fail(FP8Q_EINVAL, "%s: negative shape", fn);
    if (rows % 128 || cols % 128) return fail(FP8Q_EUNSUPPORTED, "%s: rows and cols must be multiples of 128", fn);
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31)
        return fail(FP8Q_EUNSUPPORTED, "%s: a dimension exceeds 2^31", fn);
    if ((q_col == nullptr) != (s_col == nullptr)) return fail(FP8Q_EINVAL, "%s: give both q_col and s_col or neither", fn);
    const int64_t n = rows * cols;
    if (n == 0) return ok();
    if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
    if (!q_row || !aligned(q_row, 16) || !s_row || !aligned(s_row, 4))
        return fail(FP8Q_EINVAL, "%s: q_row must be a 16-byte aligned pointer and s_row 4-byte aligned", fn);
    if (s_col && !aligned(s_col, 4)) return fail(FP8Q_EINVAL, "%s: s_col must be 4-byte aligned", fn);
    if (q_col && !aligned(q_col, 16)) return fail(FP8Q_EINVAL, "%s: q_col misaligned", fn);
    const int64_t ns = n / 32; // scale bytes of either layout
    const int64_t nx = n * dsize(dtype);
    if (overlap(x, nx, q_row, n) || overlap(x, nx, q_col, n) || overlap(q_row, n, q_col, n) ||
        overlap(s_row, ns, s_col, ns) || overlap(q_row, n, s_row, ns) || overlap(q_col, n, s_col, ns) ||
        overlap(q_row, n, s_col, ns) || overlap(q_col, n, s_row, ns) || overlap(x, nx, s_row, ns) ||
        overlap(x, nx, s_col, ns))
        return fail(FP8Q_EINVAL, "%s: buffers overlap", fn);
    return hip_status(fp8q::launch_mx(x, dtype, rows, cols, fmt, q_row, s_row, q_col, s_col, (hipStream_t)stream), fn);
}

extern "C" int fp8_quantize_mx(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt, uint8_t *q_row,
                               uint8_t *s_row, uint8_t *q_col, uint8_t *s_col, void *stream)
{
    Call c("fp8_quantize_mx", stream);
    c.args("dtype=%lld rows=%lld cols=%lld fmt=%lld", (long long)dtype, (long long)rows, (long long)cols, (long long)fmt);
    return c.ret(fp8_quantize_mx_impl(c, x, dtype, rows, cols, fmt, q_row, s_row, q_col, s_col, stream));
}

static int fp8_update_scale_delayed_impl(Call &c, float *hist, int32_t history_len, int32_t n_cols, int32_t col,
                                         const float *new_amax, int64_t step, int32_t fmt, int32_t margin,
                                         int32_t algo, float *scale, float *scale_inv, void *stream)
{
    const char *fn = "fp8_update_scale_delayed";
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (algo != FP8Q_ALGO_MAX && algo != FP8Q_ALGO_MOST_RECENT)
        return fail(FP8Q_EINVAL, "%s: unknown algo %d", fn, (int)algo);
    if (history_len < 1 || n_cols < 1 || col < 0 || col >= n_cols)
        return fail(FP8Q_EINVAL, "%s: need history_len >= 1 and 0 <= col < n_cols", fn);
    if (step < 0) return fail(FP8Q_EINVAL, "%s: negative step", fn);
    if (!hist || !new_amax || !scale || !scale_inv || !aligned(hist, 4) || !aligned(new_amax, 4) ||
        !aligned(scale, 4) || !aligned(scale_inv, 4))
        return fail(FP8Q_EINVAL, "%s: hist, new_amax, scale, scale_inv must be 4-byte aligned pointers", fn);
    const int64_t nh = (int64_t)history_len * n_cols * 4;
    if (overlap(hist, nh, scale, 4 * n_cols) || overlap(hist, nh, scale_inv, 4 * n_cols) ||
        overlap(scale, 4 * n_cols, scale_inv, 4 * n_cols) || overlap(new_amax, 4, scale, 4 * n_cols) ||
        overlap(new_amax, 4, scale_inv, 4 * n_cols))
        return fail(FP8Q_EINVAL, "%s: state buffers overlap", fn);
    return hip_status(fp8q::launch_delayed(hist, history_len, n_cols, col, new_amax, step, fmt, margin, algo, scale,
                                           scale_inv, (hipStream_t)stream),
                      fn);
}

extern "C" int fp8_update_scale_delayed(float *hist, int32_t history_len, int32_t n_cols, int32_t col,
                                        const float *new_amax, int64_t step, int32_t fmt, int32_t margin,
                                        int32_t algo, float *scale, float *scale_inv, void *stream)
{
    Call c("fp8_update_scale_delayed", stream);
    c.args("history_len=%lld n_cols=%lld col=%lld step=%lld fmt=%lld margin=%lld algo=%lld", (long long)history_len, (long long)n_cols, (long long)col, (long long)step, (long long)fmt, (long long)margin, (long long)algo);
    return c.ret(fp8_update_scale_delayed_impl(c, hist, history_len, n_cols, col, new_amax, step, fmt, margin, algo, scale, scale_inv, stream));
}

static int fp8_quantize_delayed_impl(Call &c, const void *x, int32_t dtype, int64_t n, int32_t fmt, float *hist,
                                     int32_t history_len, int32_t n_cols, int32_t col, int64_t step, int32_t fmt_next,
                                     int32_t margin, int32_t algo, float *scale, float *scale_inv, uint8_t *q,
                                     float *q_scale_inv_out, float *amax_out, void *stream)
{
    const char *fn = "fp8_quantize_delayed";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt) || !valid_fmt(fmt_next)) return fail(FP8Q_EINVAL, "%s: unknown format", fn);
    if (n < 0) return fail(FP8Q_EINVAL, "%s: negative n", fn);
    if (algo != FP8Q_ALGO_MAX && algo != FP8Q_ALGO_MOST_RECENT)
        return fail(FP8Q_EINVAL, "%s: unknown algo %d", fn, (int)algo);
    if (history_len < 1 || n_cols < 1 || col < 0 || col >= n_cols)
        return fail(FP8Q_EINVAL, "%s: need history_len >= 1 and 0 <= col < n_cols", fn);
    if (step < 0) return fail(FP8Q_EINVAL, "%s: negative step", fn);
    if (!hist || !scale || !scale_inv || !aligned(hist, 4) || !aligned(scale, 4) || !aligned(scale_inv, 4))
        return fail(FP8Q_EINVAL, "%s: hist, scale, scale_inv must be 4-byte aligned pointers", fn);
    if ((q_scale_inv_out && !aligned(q_scale_inv_out, 4)) || (amax_out && !aligned(amax_out, 4)))
        return fail(FP8Q_EINVAL, "%s: scalar outputs must be 4-byte aligned", fn);
    const int64_t nh = (int64_t)history_len * n_cols * 4;
    if (overlap(hist, nh, scale, 4 * n_cols) || overlap(hist, nh, scale_inv, 4 * n_cols) ||
        overlap(scale, 4 * n_cols, scale_inv, 4 * n_cols) || overlap(q_scale_inv_out, 4, hist, nh) ||
        overlap(q_scale_inv_out, 4, scale, 4 * n_cols) || overlap(q_scale_inv_out, 4, scale_inv, 4 * n_cols) ||
        overlap(amax_out, 4, hist, nh) || overlap(amax_out, 4, scale, 4 * n_cols) ||
        overlap(amax_out, 4, scale_inv, 4 * n_cols) || (amax_out && amax_out == q_scale_inv_out))
        return fail(FP8Q_EINVAL, "%s: state and scalar buffers overlap", fn);
    if (n > 0) {
        if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
        if (!q || !aligned(q, 16)) return fail(FP8Q_EINVAL, "%s: q must be a 16-byte aligned pointer", fn);
        if (overlap(x, n * dsize(dtype), q, n)) return fail(FP8Q_EINVAL, "%s: q overlaps x", fn);
        const void *state[5] = {hist, scale, scale_inv, q_scale_inv_out, amax_out};
        const int64_t state_bytes[5] = {nh, 4 * n_cols, 4 * n_cols, 4, 4};
        for (int i = 0; i < 5; ++i)
            if (overlap(x, n * dsize(dtype), state[i], state_bytes[i]) || overlap(q, n, state[i], state_bytes[i]))
                return fail(FP8Q_EINVAL, "%s: x or q overlaps the scaling state or a scalar output", fn);
    }
    fp8q::Reduce r{};
    const int st = c.scratch(&r);
    if (st) return st;
    return hip_status(fp8q::launch_delayed_step(x, dtype, n, fmt, hist, history_len, n_cols, col, step, fmt_next, margin,
                                                algo, scale, scale_inv, q, q_scale_inv_out, amax_out, r,
                                                (hipStream_t)stream),
                      fn);
}

extern "C" int fp8_quantize_delayed(const void *x, int32_t dtype, int64_t n, int32_t fmt, float *hist,
                                    int32_t history_len, int32_t n_cols, int32_t col, int64_t step, int32_t fmt_next,
                                    int32_t margin, int32_t algo, float *scale, float *scale_inv, uint8_t *q,
                                    float *q_scale_inv_out, float *amax_out, void *stream)
{
    Call c("fp8_quantize_delayed", stream);
    c.args("dtype=%lld n=%lld fmt=%lld history_len=%lld n_cols=%lld col=%lld step=%lld fmt_next=%lld margin=%lld algo=%lld", (long long)dtype, (long long)n, (long long)fmt, (long long)history_len, (long long)n_cols, (long long)col, (long long)step, (long long)fmt_next, (long long)margin, (long long)algo);
    return c.ret(fp8_quantize_delayed_impl(c, x, dtype, n, fmt, hist, history_len, n_cols, col, step, fmt_next, margin, algo, scale, scale_inv, q, q_scale_inv_out, amax_out, stream));
}

static int fp8_quantize_hybrid_impl(Call &c, const void *x, int32_t dtype, int64_t rows, int64_t cols,
                                    int32_t row_fmt, int32_t col_fmt, int32_t col_source, const float *amax_in,
                                    int32_t row_margin, int32_t col_margin, const float *row_scale_inv_in,
                                    const float *col_scale_inv_in, uint8_t *q_row, uint8_t *q_col,
                                    float *row_scale_inv_out, float *col_scale_inv_out, float *amax_out, void *stream)
{
    const char *fn = "fp8_quantize_hybrid";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(row_fmt) || !valid_fmt(col_fmt)) return fail(FP8Q_EINVAL, "%s: unknown format", fn);
    if (col_source != FP8Q_COLSRC_ORIGINAL && col_source != FP8Q_COLSRC_ROWWISE_DEQUANTIZED)
        return fail(FP8Q_EINVAL, "%s: unknown columnwise source %d", fn, (int)col_source);
    if (rows < 0 || cols < 0) return fail(FP8Q_EINVAL, "%s: negative shape", fn);
    if (rows % 16 || cols % 16) return fail(FP8Q_EUNSUPPORTED, "%s: rows and cols must be multiples of 16", fn);
    if (rows * cols > 0 && !q_row && !q_col)
        return fail(FP8Q_EINVAL, "%s: at least one of q_row / q_col is needed", fn);
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31)
        return fail(FP8Q_EUNSUPPORTED, "%s: a dimension exceeds 2^31", fn);
    const bool given = row_scale_inv_in || col_scale_inv_in;
    if (amax_in ? given : !(row_scale_inv_in && col_scale_inv_in))
        return fail(FP8Q_EINVAL, "%s: give either amax_in or both row_scale_inv_in and col_scale_inv_in", fn);
    const float *ins[3] = {amax_in, row_scale_inv_in, col_scale_inv_in};
    const float *outs[3] = {row_scale_inv_out, col_scale_inv_out, amax_out};
    for (const float *p : ins)
        if (p && !aligned(p, 4)) return fail(FP8Q_EINVAL, "%s: scale input not 4-byte aligned", fn);
    for (int i = 0; i < 3; ++i) {
        if (!outs[i]) continue;
        if (!aligned(outs[i], 4)) return fail(FP8Q_EINVAL, "%s: scalar output not 4-byte aligned", fn);
        for (const float *p : ins)
            if (outs[i] == p) return fail(FP8Q_EINVAL, "%s: a scalar output aliases a scale input", fn);
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return fail(FP8Q_EINVAL, "%s: scalar outputs alias each other", fn);
    }
    const int64_t n = rows * cols;
    if (n > 0) {
        if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
        if ((q_row && !aligned(q_row, 16)) || (q_col && !aligned(q_col, 16)))
            return fail(FP8Q_EINVAL, "%s: q_row / q_col must be 16-byte aligned", fn);
        if (overlap(x, n * dsize(dtype), q_row, n) || overlap(x, n * dsize(dtype), q_col, n) ||
            overlap(q_row, n, q_col, n))
            return fail(FP8Q_EINVAL, "%s: output buffers overlap", fn);
        for (const float *p : ins)
            if (overlap(q_row, n, p, 4) || overlap(q_col, n, p, 4))
                return fail(FP8Q_EINVAL, "%s: an output buffer overlaps a scale input", fn);
        for (const float *p : outs)
            if (overlap(x, n * dsize(dtype), p, 4) || overlap(q_row, n, p, 4) || overlap(q_col, n, p, 4))
                return fail(FP8Q_EINVAL, "%s: a scalar output overlaps x or the codes", fn);
    }
    fp8q::Reduce r{};
    if (amax_out) {
        const int st = c.scratch(&r);
        if (st) return st;
    }
    const fp8q::ScaleSrc src{amax_in, row_scale_inv_in, (int)row_margin};
    const fp8q::ScaleSrc src_col{amax_in, col_scale_inv_in, (int)col_margin};
    return hip_status(fp8q::launch_hybrid(x, dtype, rows, cols, row_fmt, col_fmt, col_source, src, src_col, q_row,
                                          q_col, row_scale_inv_out, col_scale_inv_out, amax_out, r,
                                          (hipStream_t)stream),
                      fn);
}

extern "C" int fp8_quantize_hybrid(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t row_fmt,
                                   int32_t col_fmt, int32_t col_source, const float *amax_in, int32_t row_margin,
                                   int32_t col_margin, const float *row_scale_inv_in, const float *col_scale_inv_in,
                                   uint8_t *q_row, uint8_t *q_col, float *row_scale_inv_out, float *col_scale_inv_out,
                                   float *amax_out, void *stream)
{
    Call c("fp8_quantize_hybrid", stream);
    c.args("dtype=%lld rows=%lld cols=%lld row_fmt=%lld col_fmt=%lld col_source=%lld row_margin=%lld col_margin=%lld", (long long)dtype, (long long)rows, (long long)cols, (long long)row_fmt, (long long)col_fmt, (long long)col_source, (long long)row_margin, (long long)col_margin);
    return c.ret(fp8_quantize_hybrid_impl(c, x, dtype, rows, cols, row_fmt, col_fmt, col_source, amax_in, row_margin, col_margin, row_scale_inv_in, col_scale_inv_in, q_row, q_col, row_scale_inv_out, col_scale_inv_out, amax_out, stream));
}

// bytes of the scale buffer of one direction's copy of a [rows][cols] tensor
// under a block sub-quantizer, rows and cols being the copy's own (x^T's for
// the columnwise copy)
static int64_t subq_scale_bytes(int32_t recipe, int64_t rows, int64_t cols)
{
    if (recipe == FP8Q_SUBQ_PER_TENSOR) return 4;
    if (recipe == FP8Q_SUBQ_BLOCK_128x128) return (rows / 128) * (cols / 128) * 4;
    if (recipe == FP8Q_SUBQ_BLOCK_1x128) return rows * (cols / 128) * 4;
    return rows * (cols / 32);
}

static bool valid_subq(int32_t r)
{
    return r == FP8Q_SUBQ_BLOCK_128x128 || r == FP8Q_SUBQ_BLOCK_1x128 || r == FP8Q_SUBQ_MXFP8 ||
           r == FP8Q_SUBQ_PER_TENSOR;
}

static int fp8_quantize_hybrid_blockwise_impl(Call &c, const void *x, int32_t dtype, int64_t rows, int64_t cols,
                                              int32_t row_recipe, int32_t row_fmt, uint8_t *q_row, void *s_row,
                                              int32_t col_recipe, int32_t col_fmt, int32_t col_source,
                                              uint8_t *q_col, void *s_col, const float *amax_in, int32_t margin,
                                              const float *scale_inv_in, void *stream)
{
    const char *fn = "fp8_quantize_hybrid_blockwise";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(row_fmt) || !valid_fmt(col_fmt)) return fail(FP8Q_EINVAL, "%s: unknown format", fn);
    if (!valid_subq(row_recipe) || !valid_subq(col_recipe))
        return fail(FP8Q_EINVAL, "%s: unknown sub-quantizer (row %d, col %d)", fn, (int)row_recipe, (int)col_recipe);
    if (col_source != FP8Q_COLSRC_ORIGINAL && col_source != FP8Q_COLSRC_ROWWISE_DEQUANTIZED)
        return fail(FP8Q_EINVAL, "%s: unknown columnwise source %d", fn, (int)col_source);
    // a per-tensor direction takes its scale from amax_in (current scaling
    // with margin) or scale_inv_in; only one direction may be per-tensor
    const int n_tensor = (row_recipe == FP8Q_SUBQ_PER_TENSOR) + (col_recipe == FP8Q_SUBQ_PER_TENSOR);
    if (n_tensor == 2)
        return fail(FP8Q_EINVAL, "%s: two per-tensor directions are fp8_quantize_hybrid's; here at most one", fn);
    if (n_tensor == 1 && (amax_in == nullptr) == (scale_inv_in == nullptr))
        return fail(FP8Q_EINVAL, "%s: the per-tensor direction needs exactly one of amax_in / scale_inv_in", fn);
    if (n_tensor == 0 && (amax_in || scale_inv_in))
        return fail(FP8Q_EINVAL, "%s: amax_in / scale_inv_in serve a per-tensor direction only", fn);
    if ((amax_in && !aligned(amax_in, 4)) || (scale_inv_in && !aligned(scale_inv_in, 4)))
        return fail(FP8Q_EINVAL, "%s: amax_in / scale_inv_in must be 4-byte aligned", fn);
    if (col_recipe == FP8Q_SUBQ_PER_TENSOR && col_source == FP8Q_COLSRC_ROWWISE_DEQUANTIZED && amax_in)
        return fail(FP8Q_EUNSUPPORTED,
                    "%s: per-tensor columns of the dequantized rows need a given scale_inv_in (their amax is not "
                    "known before the pass)", fn);
    if (rows < 0 || cols < 0) return fail(FP8Q_EINVAL, "%s: negative shape", fn);
    if (rows % 128 || cols % 128) return fail(FP8Q_EUNSUPPORTED, "%s: rows and cols must be multiples of 128", fn);
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31)
        return fail(FP8Q_EUNSUPPORTED, "%s: a dimension exceeds 2^31", fn);
    if ((q_row == nullptr) != (s_row == nullptr)) return fail(FP8Q_EINVAL, "%s: give both q_row and s_row or neither", fn);
    if ((q_col == nullptr) != (s_col == nullptr)) return fail(FP8Q_EINVAL, "%s: give both q_col and s_col or neither", fn);
    const int64_t n = rows * cols;
    if (n == 0) return ok();
    if (!q_row && !q_col) return fail(FP8Q_EINVAL, "%s: at least one of the two copies is needed", fn);
    if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
    if ((q_row && !aligned(q_row, 16)) || (q_col && !aligned(q_col, 16)))
        return fail(FP8Q_EINVAL, "%s: q_row / q_col must be 16-byte aligned", fn);
    if ((s_row && !aligned(s_row, 4)) || (s_col && !aligned(s_col, 4)))
        return fail(FP8Q_EINVAL, "%s: s_row / s_col must be 4-byte aligned", fn);
    const void *buf[7] = {x, amax_in, scale_inv_in, q_row, s_row, q_col, s_col};
    const int64_t len[7] = {n * dsize(dtype), 4, 4, n, subq_scale_bytes(row_recipe, rows, cols), n,
                            subq_scale_bytes(col_recipe, cols, rows)};
    for (int i = 3; i < 7; ++i) // the outputs against every other buffer
        for (int j = 0; j < i; ++j)
            if (overlap(buf[i], len[i], buf[j], len[j])) return fail(FP8Q_EINVAL, "%s: buffers overlap", fn);
    const fp8q::ScaleSrc pt{amax_in, scale_inv_in, (int)margin};
    return hip_status(fp8q::launch_hybrid_blockwise(x, dtype, rows, cols, row_recipe, row_fmt, q_row, s_row,
                                                    col_recipe, col_fmt, q_col, s_col,
                                                    col_source == FP8Q_COLSRC_ROWWISE_DEQUANTIZED, pt,
                                                    (hipStream_t)stream),
                      fn);
}

extern "C" int fp8_quantize_hybrid_blockwise(const void *x, int32_t dtype, int64_t rows, int64_t cols,
                                             int32_t row_recipe, int32_t row_fmt, uint8_t *q_row, void *s_row,
                                             int32_t col_recipe, int32_t col_fmt, int32_t col_source, uint8_t *q_col,
                                             void *s_col, const float *amax_in, int32_t margin,
                                             const float *scale_inv_in, void *stream)
{
    Call c("fp8_quantize_hybrid_blockwise", stream);
    c.args("dtype=%lld rows=%lld cols=%lld row_recipe=%lld row_fmt=%lld col_recipe=%lld col_fmt=%lld col_source=%lld "
           "margin=%lld",
           (long long)dtype, (long long)rows, (long long)cols, (long long)row_recipe, (long long)row_fmt,
           (long long)col_recipe, (long long)col_fmt, (long long)col_source, (long long)margin);
    return c.ret(fp8_quantize_hybrid_blockwise_impl(c, x, dtype, rows, cols, row_recipe, row_fmt, q_row, s_row,
                                                    col_recipe, col_fmt, col_source, q_col, s_col, amax_in, margin,
                                                    scale_inv_in, stream));
}

static int fp8_cast_stats_impl(Call &c, const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *scale_inv,
                               uint64_t *stats, void *stream)
{
    const char *fn = "fp8_cast_stats";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (n < 0) return fail(FP8Q_EINVAL, "%s: negative n", fn);
    if (!scale_inv || !aligned(scale_inv, 4)) return fail(FP8Q_EINVAL, "%s: scale_inv must be 4-byte aligned", fn);
    if (!stats || !aligned(stats, 8)) return fail(FP8Q_EINVAL, "%s: stats must be an 8-byte aligned pointer", fn);
    if (overlap(stats, 32, scale_inv, 4)) return fail(FP8Q_EINVAL, "%s: stats overlaps scale_inv", fn);
    if (n > 0) {
        if (!x || !aligned(x, 16)) return fail(FP8Q_EINVAL, "%s: x must be a 16-byte aligned pointer", fn);
        if (overlap(x, n * dsize(dtype), stats, 32)) return fail(FP8Q_EINVAL, "%s: stats overlaps x", fn);
    }
    fp8q::GridScratch *gs = nullptr;
    const int st = c.scratch(&gs);
    if (st) return st;
    return hip_status(fp8q::launch_cast_stats(x, dtype, n, fmt, scale_inv, stats, gs, (hipStream_t)stream), fn);
}

extern "C" int fp8_cast_stats(const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *scale_inv,
                              uint64_t *stats, void *stream)
{
    Call c("fp8_cast_stats", stream);
    c.args("dtype=%lld n=%lld fmt=%lld", (long long)dtype, (long long)n, (long long)fmt);
    return c.ret(fp8_cast_stats_impl(c, x, dtype, n, fmt, scale_inv, stats, stream));
}

static int fp8_quantize_error_feedback_impl(Call &c, const void *g, int32_t dtype, float *residual, int64_t n,
                                            int32_t fmt, const float *scale_inv, uint8_t *q, float *amax_out,
                                            void *stream)
{
    const char *fn = "fp8_quantize_error_feedback";
    if (!valid_dtype(dtype)) return fail(FP8Q_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: unknown format %d", fn, (int)fmt);
    if (n < 0) return fail(FP8Q_EINVAL, "%s: negative n", fn);
    if (!scale_inv || !aligned(scale_inv, 4)) return fail(FP8Q_EINVAL, "%s: scale_inv must be 4-byte aligned", fn);
    if (amax_out && (!aligned(amax_out, 4) || amax_out == scale_inv))
        return fail(FP8Q_EINVAL, "%s: amax_out misaligned or aliasing scale_inv", fn);
    if (n > 0) {
        if (!g || !aligned(g, 16)) return fail(FP8Q_EINVAL, "%s: g must be a 16-byte aligned pointer", fn);
        if (!residual || !aligned(residual, 16))
            return fail(FP8Q_EINVAL, "%s: residual must be a 16-byte aligned pointer", fn);
        if (!q || !aligned(q, 16)) return fail(FP8Q_EINVAL, "%s: q must be a 16-byte aligned pointer", fn);
        const int64_t ng = n * dsize(dtype);
        if (overlap(g, ng, residual, 4 * n) || overlap(g, ng, q, n) || overlap(residual, 4 * n, q, n))
            return fail(FP8Q_EINVAL, "%s: g, residual and q overlap", fn);
        if (overlap(g, ng, scale_inv, 4) || overlap(residual, 4 * n, scale_inv, 4) || overlap(q, n, scale_inv, 4) ||
            overlap(g, ng, amax_out, 4) || overlap(residual, 4 * n, amax_out, 4) || overlap(q, n, amax_out, 4))
            return fail(FP8Q_EINVAL, "%s: a tensor overlaps scale_inv or amax_out", fn);
    }
    fp8q::Reduce r{};
    if (amax_out) {
        const int st = c.scratch(&r);
        if (st) return st;
    }
    return hip_status(
        fp8q::launch_error_feedback(g, dtype, residual, n, fmt, scale_inv, q, amax_out, r, (hipStream_t)stream), fn);
}

extern "C" int fp8_quantize_error_feedback(const void *g, int32_t dtype, float *residual, int64_t n, int32_t fmt,
                                           const float *scale_inv, uint8_t *q, float *amax_out, void *stream)
{
    Call c("fp8_quantize_error_feedback", stream);
    c.args("dtype=%lld n=%lld fmt=%lld", (long long)dtype, (long long)n, (long long)fmt);
    return c.ret(fp8_quantize_error_feedback_impl(c, g, dtype, residual, n, fmt, scale_inv, q, amax_out, stream));
}

// Shared body of the two GEMM entry points.  c_type: FP8Q_F32, FP8Q_BF16,
// FP8Q_OUT_E4M3FN or FP8Q_OUT_E5M2 (the last two only from the fused call).
static int scaled_gemm(Call &c, const char *fn, const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B,
                       int32_t fb, const float *sB, int64_t M, int64_t N, int64_t K, int32_t mode, const float *bias,
                       int32_t act, void *C, int32_t c_type, const float *c_scale_inv, float *amax_out, void *stream)
{
    if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(FP8Q_EINVAL, "%s: unknown operand format", fn);
    if (mode != FP8Q_PER_TENSOR && mode != FP8Q_BLOCK_1x128_128x128 && mode != FP8Q_BLOCK_1x128_1x128 &&
        mode != FP8Q_MXFP8)
        return fail(FP8Q_EINVAL, "%s: unknown scaling mode %d", fn, (int)mode);
    if (act != FP8Q_ACT_NONE && act != FP8Q_ACT_RELU && act != FP8Q_ACT_GELU)
        return fail(FP8Q_EINVAL, "%s: unknown activation %d", fn, (int)act);
    const bool fp8_out = c_type == FP8Q_OUT_E4M3FN || c_type == FP8Q_OUT_E5M2;
    if (M < 0 || N < 0 || K < 0) return fail(FP8Q_EINVAL, "%s: negative shape", fn);
    if (M % 128 || N % 128 || K % 128) return fail(FP8Q_EUNSUPPORTED, "%s: M, N, K must be multiples of 128", fn);
    if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31)
        return fail(FP8Q_EUNSUPPORTED, "%s: a dimension exceeds 2^31", fn);
    // a block's operand panel (256 rows of K bytes) is addressed with 32-bit
    // buffer offsets, and the grid is one block per 256x256 output tile
    if (K > (int64_t)1 << 22) return fail(FP8Q_EUNSUPPORTED, "%s: K exceeds 2^22", fn);
    if ((M / 256 + 1) * (N / 256 + 1) > (int64_t)INT32_MAX)
        return fail(FP8Q_EUNSUPPORTED, "%s: more than 2^31 output tiles", fn);
    if (!sA || !sB || !aligned(sA, 4) || !aligned(sB, 4))
        return fail(FP8Q_EINVAL, "%s: sA and sB must be 4-byte aligned pointers", fn);
    if (amax_out && !aligned(amax_out, 4)) return fail(FP8Q_EINVAL, "%s: amax_out misaligned", fn);
    if (fp8_out && (!c_scale_inv || !aligned(c_scale_inv, 4)))
        return fail(FP8Q_EINVAL, "%s: an FP8 output needs a 4-byte aligned c_scale_inv", fn);
    if (!fp8_out && c_scale_inv) return fail(FP8Q_EINVAL, "%s: c_scale_inv is only for an FP8 output", fn);
    if (bias && !aligned(bias, 16)) return fail(FP8Q_EINVAL, "%s: bias must be 16-byte aligned", fn);
    if (M == 0 || N == 0) {
        if (amax_out) return hip_status(fp8q::launch_fill_u32(reinterpret_cast<uint32_t *>(amax_out), 0u,
                                                              (hipStream_t)stream), fn);
        return ok();
    }
    if (!C || !aligned(C, 16)) return fail(FP8Q_EINVAL, "%s: C must be a 16-byte aligned pointer", fn);
    if (K > 0 && (!A || !B || !aligned(A, 16) || !aligned(B, 16)))
        return fail(FP8Q_EINVAL, "%s: A and B must be 16-byte aligned pointers", fn);
    const int64_t c_bytes = M * N * (fp8_out ? 1 : dsize(c_type));
    if (overlap(C, c_bytes, A, M * K) || overlap(C, c_bytes, B, N * K) || overlap(C, c_bytes, amax_out, 4) ||
        overlap(C, c_bytes, bias, 4 * N) || overlap(C, c_bytes, c_scale_inv, 4))
        return fail(FP8Q_EINVAL, "%s: C overlaps an input", fn);
    if (overlap(amax_out, 4, bias, 4 * N) || overlap(amax_out, 4, c_scale_inv, 4))
        return fail(FP8Q_EINVAL, "%s: amax_out overlaps an input", fn);
    fp8q::GridScratch *gs = nullptr;
    if (amax_out) {
        const int st = c.scratch(&gs);
        if (st) return st;
    }
    // kernel output kinds: 0 bf16, 1 fp32, 2 E4M3FN codes, 3 E5M2 codes
    const int out_kind = c_type == FP8Q_BF16 ? 0 : c_type == FP8Q_F32 ? 1 : c_type == FP8Q_OUT_E4M3FN ? 2 : 3;
    return hip_status(fp8q::launch_gemm(A, fa, sA, B, fb, sB, M, N, K, mode, C, out_kind, bias, act, c_scale_inv,
                                        amax_out, gs, (hipStream_t)stream),
                      fn);
}

static int fp8_scaled_gemm_impl(Call &c, const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B, int32_t fb,
                                const float *sB, int64_t M, int64_t N, int64_t K, int32_t mode, void *C,
                                int32_t c_dtype, float *amax_out, void *stream)
{
    const char *fn = "fp8_scaled_gemm";
    if (!valid_dtype(c_dtype)) return fail(FP8Q_EINVAL, "%s: unknown output dtype %d", fn, (int)c_dtype);
    return scaled_gemm(c, fn, A, fa, sA, B, fb, sB, M, N, K, mode, nullptr, FP8Q_ACT_NONE, C, c_dtype, nullptr, amax_out,
                       stream);
}

extern "C" int fp8_scaled_gemm(const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B, int32_t fb,
                               const float *sB, int64_t M, int64_t N, int64_t K, int32_t mode, void *C,
                               int32_t c_dtype, float *amax_out, void *stream)
{
    Call c("fp8_scaled_gemm", stream);
    c.args("fa=%lld fb=%lld M=%lld N=%lld K=%lld mode=%lld c_dtype=%lld", (long long)fa, (long long)fb, (long long)M, (long long)N, (long long)K, (long long)mode, (long long)c_dtype);
    return c.ret(fp8_scaled_gemm_impl(c, A, fa, sA, B, fb, sB, M, N, K, mode, C, c_dtype, amax_out, stream));
}

static int fp8_scaled_gemm_fused_impl(Call &c, const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B,
                                      int32_t fb, const float *sB, int64_t M, int64_t N, int64_t K, int32_t mode,
                                      const float *bias, int32_t act, void *C, int32_t c_type,
                                      const float *c_scale_inv, float *amax_out, void *stream)
{
    const char *fn = "fp8_scaled_gemm_fused";
    if (!valid_dtype(c_type) && c_type != FP8Q_OUT_E4M3FN && c_type != FP8Q_OUT_E5M2)
        return fail(FP8Q_EINVAL, "%s: unknown output type %d", fn, (int)c_type);
    return scaled_gemm(c, fn, A, fa, sA, B, fb, sB, M, N, K, mode, bias, act, C, c_type, c_scale_inv, amax_out, stream);
}

extern "C" int fp8_scaled_gemm_fused(const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B, int32_t fb,
                                     const float *sB, int64_t M, int64_t N, int64_t K, int32_t mode,
                                     const float *bias, int32_t act, void *C, int32_t c_type,
                                     const float *c_scale_inv, float *amax_out, void *stream)
{
    Call c("fp8_scaled_gemm_fused", stream);
    c.args("fa=%lld fb=%lld M=%lld N=%lld K=%lld mode=%lld act=%lld c_type=%lld", (long long)fa, (long long)fb, (long long)M, (long long)N, (long long)K, (long long)mode, (long long)act, (long long)c_type);
    return c.ret(fp8_scaled_gemm_fused_impl(c, A, fa, sA, B, fb, sB, M, N, K, mode, bias, act, C, c_type, c_scale_inv, amax_out, stream));
}

