// C ABI of the submconv library: argument validation, rulebook lifetime,
// kernel dispatch.  Every argument check here runs before any HIP call, so
// invalid calls fail without touching the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "common.h"

namespace sc {
int build_map(const int32_t *coords, submconv_rulebook *rb, hipStream_t stream);
int launch_forward(const void *feats, const void *w, const float *bias,
                   const submconv_rulebook *rb, void *out, int cin, int cout, int dtype, int flip,
                   int variant, hipStream_t s);
int input_order_table(const submconv_rulebook *rb, int32_t *out, hipStream_t s);
int64_t win_plan_ints(int64_t n);
int subdivide(const int32_t *coords, const void *feats, int64_t n, int c, int dtype,
              int32_t *out_coords, void *out_feats, hipStream_t s);
int space_to_depth(const int32_t *coords, const void *feats, int64_t n, int c, int dtype, int res,
                   int batch, int32_t *out_coords, void *out_feats, uint8_t *out_mask,
                   int64_t *out_m, hipStream_t s);
int depth_to_space(const int32_t *cc, const void *cf, const uint8_t *mask, int64_t m, int c,
                   int dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s);
int upsample_masked(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n, int c, int dtype,
                    int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s);
int upsample_masked_noalloc(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n, int c,
                            int dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, hipStream_t s);
size_t noalloc_expand_bytes(int64_t m);
int downsample(const int32_t *coords, const void *feats, int64_t n, int c, int dtype, int res, int batch,
               int mean, int32_t *out_coords, void *out_feats, int64_t *out_m, hipStream_t s);
int classify_5d(const int64_t *shape, int hint, int *layout);
int weight_convert(const void *src, int layout, int cout, int cin, int dtype, int flip, void *dst, hipStream_t s);

static thread_local char g_err[512];

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

// Pinned host blocks of a host thread: the status read-back buffer and the status
// mailbox.  A thread's blocks go back to a process-wide list when the thread exits
// (no HIP call there: the runtime may already be shutting down) and are handed to the
// next thread that needs one, so short-lived threads do not pile up pinned memory.
namespace {
struct PinnedSet {
    DevStatus *pinned = nullptr;   // read-back buffer
    size_t pinned_bytes = 0;
    Mailbox *mb = nullptr;         // host address of the mailbox
    Mailbox *mb_dev = nullptr;     // its device address
    uint32_t seq = 0;              // the last sequence number used on it
};
std::mutex g_pinned_mu;
std::vector<PinnedSet> g_pinned_free;
struct PinnedHolder {
    PinnedSet p;
    PinnedHolder()
    {
        std::lock_guard<std::mutex> lk(g_pinned_mu);
        if (!g_pinned_free.empty()) {
            p = g_pinned_free.back();
            g_pinned_free.pop_back();
        }
    }
    ~PinnedHolder()
    {
        if (!p.pinned && !p.mb) return;
        std::lock_guard<std::mutex> lk(g_pinned_mu);
        g_pinned_free.push_back(p);
    }
};
thread_local PinnedHolder g_pin;
}  // namespace

int read_status_counts(const DevStatus *d, int64_t ncounts, DevStatus *h, uint64_t *sum, hipStream_t stream)
{
    const size_t bytes = sizeof(DevStatus) + (size_t)ncounts * 4;
    PinnedSet &ps = g_pin.p;
    if (ps.pinned_bytes < bytes) {  // grows to the largest read-back seen on this thread
        if (ps.pinned) (void)hipHostFree(ps.pinned);
        ps.pinned = nullptr;
        ps.pinned_bytes = 0;
        const size_t want = bytes < 4096 ? 4096 : bytes;
        SC_HIP(hipHostMalloc((void **)&ps.pinned, want, hipHostMallocDefault));
        ps.pinned_bytes = want;
    }
    SC_HIP(hipMemcpyAsync(ps.pinned, d, bytes, hipMemcpyDeviceToHost, stream));
    SC_HIP(hipStreamSynchronize(stream));
    *h = *ps.pinned;
    uint64_t t = 0;
    const uint32_t *c = (const uint32_t *)(ps.pinned + 1);
    for (int64_t i = 0; i < ncounts; ++i) t += c[i];
    if (sum) *sum = t;
    return SUBMCONV_OK;
}

int read_status(const DevStatus *d, DevStatus *h, hipStream_t stream)
{
    return read_status_counts(d, 0, h, nullptr, stream);
}

int mailbox_acquire(Mailbox **mb, uint32_t *seq)
{
    PinnedSet &ps = g_pin.p;
    if (!ps.mb) {
        // coherent: the device's stores reach host memory while the kernel runs; portable:
        // usable from every device
        Mailbox *h = nullptr;
        SC_HIP(hipHostMalloc((void **)&h, sizeof(Mailbox),
                             hipHostMallocCoherent | hipHostMallocMapped | hipHostMallocPortable));
        __atomic_store_n(&h->seq, 0u, __ATOMIC_RELAXED);
        void *dp = nullptr;
        if (hipHostGetDevicePointer(&dp, h, 0) != hipSuccess) {
            (void)hipHostFree(h);
            return fail(SUBMCONV_E_HIP, "hipHostGetDevicePointer failed for the status mailbox");
        }
        ps.mb = h;
        ps.mb_dev = (Mailbox *)dp;
        ps.seq = 0;
    }
    // the sequence goes on from the mailbox's last one (it may come from an exited thread),
    // so a stale post never matches; never 0, the initial value
    ps.seq = ps.seq + 1 ? ps.seq + 1 : 1;
    *mb = ps.mb_dev;
    *seq = ps.seq;
    return SUBMCONV_OK;
}

int mailbox_wait(Mailbox *mb_dev, uint32_t seq, DevStatus *h, hipStream_t stream)
{
    (void)mb_dev;
    Mailbox *mb = g_pin.p.mb;
    // poll for up to ~2 ms (a build of a few million voxels takes well under that); past
    // it, or if the post never comes (a failed launch), synchronise and check once more
    const auto t0 = std::chrono::steady_clock::now();
    bool seen = false;
    for (uint32_t it = 0;; ++it) {
        if (__atomic_load_n(&mb->seq, __ATOMIC_ACQUIRE) == seq) {
            seen = true;
            break;
        }
        if ((it & 255u) == 255u && std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(2000)) break;
    }
    if (!seen) {
        SC_HIP(hipStreamSynchronize(stream));
        if (__atomic_load_n(&mb->seq, __ATOMIC_ACQUIRE) != seq)
            return fail(SUBMCONV_E_HIP, "the build's status was not posted");
    }
    *h = DevStatus{};
    h->flags = mb->flags;
    h->taps = mb->taps;
    h->count = mb->count;
    return SUBMCONV_OK;
}

// Device memory of the library (rulebooks and scratch) comes from a block cache.
// The driver's stream-ordered allocator costs tens to hundreds of microseconds of
// host time per call for large blocks, and a map build allocates and frees its
// scratch every time; so freed blocks are kept per device and handed out again for
// requests of up to their size and at least half of it.
//
// Ordering: a block freed while work queued on a stream may still use it carries an
// event recorded on that stream at the free.  Whoever takes the block next makes its
// own stream wait for that event (hipStreamWaitEvent), so a block can move between
// streams, and a stream destroyed meanwhile leaves no dangling ordering.  Blocks
// freed right after their stream was synchronised carry no event.  Blocks of the
// caller's stream are preferred, so the usual wait is on an event of the same stream.
// The cache holds at most g_cap bytes per device (submconv_set_cache_limit; 2 GiB by
// default); beyond that, freed blocks go back to the driver.  submconv_release_cache
// empties it.
namespace {
struct Cached {
    void *p;
    size_t bytes;
    int device;
    hipStream_t stream;  // where it was freed (preference only)
    hipEvent_t ev;       // completes when that stream's prior work is done; nullptr: idle
};
std::mutex g_cache_mu;
size_t g_cap = size_t(2) << 30;
std::unordered_map<void *, std::pair<size_t, int>> g_live;  // block -> (bytes, device)
std::vector<Cached> g_free;
std::vector<std::pair<int, hipEvent_t>> g_events;  // spare events, by device
size_t g_cached[64];

size_t size_class(size_t bytes)  // 8 classes per power of two: at most 12.5% slack
{
    bytes = (bytes + 255) & ~size_t(255);
    size_t top = 256;
    while (top < bytes) top <<= 1;
    const size_t step = top >= 2048 ? top / 16 : 128;
    return (bytes + step - 1) / step * step;
}

void put_event(int device, hipEvent_t ev)  // caller holds g_cache_mu
{
    if (ev) g_events.push_back({device, ev});
}

hipEvent_t get_event(int device)  // caller holds g_cache_mu; current device == device
{
    for (size_t i = 0; i < g_events.size(); ++i)
        if (g_events[i].first == device) {
            hipEvent_t ev = g_events[i].second;
            g_events[i] = g_events.back();
            g_events.pop_back();
            return ev;
        }
    hipEvent_t ev = nullptr;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return nullptr;
    return ev;
}

// Return blocks to the driver once their last use has finished.  Caller holds g_cache_mu.
void release_cached(int device)
{
    int cur = -1;
    (void)hipGetDevice(&cur);
    for (size_t i = 0; i < g_free.size();) {
        Cached &b = g_free[i];
        if (device < 0 || b.device == device) {
            if (b.ev) (void)hipEventSynchronize(b.ev);
            if (b.device != cur && hipSetDevice(b.device) == hipSuccess) cur = b.device;
            (void)hipFreeAsync(b.p, nullptr);  // its last use has finished (event above)
            put_event(b.device, b.ev);
            if (b.device >= 0 && b.device < 64) g_cached[b.device] -= b.bytes;
            g_free[i] = g_free.back();
            g_free.pop_back();
        } else {
            ++i;
        }
    }
}
}  // namespace

int dev_alloc(void **p, size_t bytes, hipStream_t stream)
{
    *p = nullptr;
    bytes = size_class(bytes == 0 ? 256 : bytes);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SUBMCONV_E_HIP, "hipGetDevice failed");
    {
        std::lock_guard<std::mutex> lock(g_cache_mu);
        size_t best = SIZE_MAX;
        for (size_t i = 0; i < g_free.size(); ++i) {
            const Cached &b = g_free[i];
            if (b.device != dev || b.bytes < bytes || b.bytes / 2 > bytes) continue;
            if (best == SIZE_MAX) { best = i; continue; }
            const Cached &c = g_free[best];
            const bool bs = b.stream == stream, cs = c.stream == stream;
            if ((bs && !cs) || (bs == cs && b.bytes < c.bytes)) best = i;
        }
        if (best != SIZE_MAX) {
            Cached b = g_free[best];
            if (b.ev && hipStreamWaitEvent(stream, b.ev, 0) != hipSuccess)
                return fail(SUBMCONV_E_HIP, "hipStreamWaitEvent failed");
            put_event(dev, b.ev);
            *p = b.p;
            g_live[*p] = {b.bytes, dev};
            if (dev < 64) g_cached[dev] -= b.bytes;
            g_free[best] = g_free.back();
            g_free.pop_back();
            return SUBMCONV_OK;
        }
    }
    hipError_t e = hipMallocAsync(p, bytes, stream);
    if (e == hipErrorOutOfMemory) {  // give the cached blocks back and try once more
        {
            std::lock_guard<std::mutex> lock(g_cache_mu);
            release_cached(dev);
        }
        e = hipMallocAsync(p, bytes, stream);
    }
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(e == hipErrorOutOfMemory ? SUBMCONV_E_OOM : SUBMCONV_E_HIP,
                    "device allocation of %zu bytes: %s", bytes, hipGetErrorString(e));
    }
    std::lock_guard<std::mutex> lock(g_cache_mu);
    g_live[*p] = {bytes, dev};
    return SUBMCONV_OK;
}

static void dev_release(void *p, hipStream_t stream, bool idle)
{
    if (!p) return;
    std::lock_guard<std::mutex> lock(g_cache_mu);
    auto it = g_live.find(p);
    if (it == g_live.end()) {  // not from dev_alloc: hand it to the driver
        (void)hipFreeAsync(p, stream);
        return;
    }
    const size_t bytes = it->second.first;
    const int dev = it->second.second;
    g_live.erase(it);
    int cur = -1;
    if (dev >= 0 && dev < 64 && g_cached[dev] + bytes <= g_cap && hipGetDevice(&cur) == hipSuccess && cur == dev) {
        hipEvent_t ev = nullptr;
        if (!idle) {
            ev = get_event(dev);
            if (!ev || hipEventRecord(ev, stream) != hipSuccess) {
                put_event(dev, ev);
                (void)hipFreeAsync(p, stream);
                return;
            }
        }
        g_free.push_back({p, bytes, dev, stream, ev});
        g_cached[dev] += bytes;
    } else {
        (void)hipFreeAsync(p, stream);
    }
}

void dev_free(void *p, hipStream_t stream) { dev_release(p, stream, false); }

void dev_free_idle(void *p, hipStream_t stream) { dev_release(p, stream, true); }

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const char *x = (const char *)a, *y = (const char *)b;
    return x < y + nb && y < x + na;
}

static size_t elem_size(int dtype) { return dtype == SUBMCONV_F32 ? 4 : 2; }

}  // namespace sc

using namespace sc;

extern "C" {

const char *submconv_version(void) { return "submconv 0.1 gfx950"; }

const char *submconv_status_string(int status)
{
    switch (status) {
    case SUBMCONV_OK: return "ok";
    case SUBMCONV_E_INVALID_ARG: return "invalid argument";
    case SUBMCONV_E_COORD_RANGE: return "coordinate out of range";
    case SUBMCONV_E_DUPLICATE: return "duplicate coordinate";
    case SUBMCONV_E_UNSUPPORTED: return "unsupported configuration";
    case SUBMCONV_E_ALIAS: return "output aliases an input";
    case SUBMCONV_E_OOM: return "out of device memory";
    case SUBMCONV_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *submconv_last_error(void) { return g_err; }

int submconv_build_map(const int32_t *coords, int64_t n, int32_t res, int32_t batch, void *stream,
                       submconv_rulebook **out_rb)
{
    if (!out_rb) return fail(SUBMCONV_E_INVALID_ARG, "out_rb is NULL");
    *out_rb = nullptr;
    if (n < 0 || n >= (int64_t(1) << 31)) return fail(SUBMCONV_E_INVALID_ARG, "n = %lld outside [0, 2^31)", (long long)n);
    if (n > 0 && !coords) return fail(SUBMCONV_E_INVALID_ARG, "coords is NULL");
    if (n > 0 && !aligned16(coords)) return fail(SUBMCONV_E_INVALID_ARG, "coords must be 16-byte aligned");
    if (res < 1) return fail(SUBMCONV_E_INVALID_ARG, "res = %d must be >= 1", res);
    if (batch < 1) return fail(SUBMCONV_E_INVALID_ARG, "batch = %d must be >= 1", batch);
    const int rb = bits_for(res) > 0 ? bits_for(res) : 1;
    const int nbits = 3 * rb + bits_for(batch);
    if (nbits > 64) return fail(SUBMCONV_E_UNSUPPORTED, "res %d and batch %d need %d key bits (max 64)", res, batch, nbits);
    hipStream_t s = (hipStream_t)stream;

    submconv_rulebook *r = new (std::nothrow) submconv_rulebook();
    if (!r) return fail(SUBMCONV_E_OOM, "host allocation failed");
    r->n = n;
    r->res = res;
    r->batch = batch;
    r->rb = rb;
    r->nbits = nbits;
    r->key_bytes = nbits <= 32 ? 4 : 8;
    r->taps = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) { delete r; return fail(SUBMCONV_E_HIP, "hipGetDevice failed"); }
    r->device = dev;
    int st = SUBMCONV_OK;
    r->ngroups = (n + 31) / 32;
    r->nbr_in = nullptr;

    const size_t kbytes = (((size_t)n * r->key_bytes) + 255) & ~size_t(255);
    const size_t pbytes = (((size_t)n * 4) + 255) & ~size_t(255);
    // +1 KB: kernels copy table rows in 16-byte chunks that may run past the last row
    const size_t nbytes = ((((size_t)n * NBR_INTS * 4) + 255) & ~size_t(255)) + 1024;
    const size_t mbytes = (((size_t)r->ngroups * GWIN_INTS * 4) + 255) & ~size_t(255);
    const size_t lbytes = (size_t)win_plan_ints(n) * 4 + 256;
    r->block_bytes = kbytes + pbytes + nbytes + mbytes + lbytes;
    st = dev_alloc(&r->block, r->block_bytes, s);
    if (st != SUBMCONV_OK) { delete r; return st; }
    r->keys = r->block;
    r->perm = (int32_t *)((char *)r->block + kbytes);
    r->nbr_sp = (int32_t *)((char *)r->block + kbytes + pbytes);
    r->gwin = (int32_t *)((char *)r->block + kbytes + pbytes + nbytes);
    r->plan = (int32_t *)((char *)r->block + kbytes + pbytes + nbytes + mbytes);
    if (n > 0) {
        st = build_map(coords, r, s);
        if (st != SUBMCONV_OK) {
            dev_free(r->block, s);
            delete r;
            return st;
        }
    }
    *out_rb = r;
    return SUBMCONV_OK;
}

int submconv_rulebook_neighbors(submconv_rulebook *rb, void *stream, const int32_t **nbr, int64_t *n)
{
    if (!rb || !nbr || !n) return fail(SUBMCONV_E_INVALID_ARG, "NULL argument");
    if (!rb->nbr_in && rb->n > 0) {
        void *p = nullptr;
        SC_CHECK(dev_alloc(&p, (size_t)rb->n * 27 * 4, (hipStream_t)stream));
        const int st = input_order_table(rb, (int32_t *)p, (hipStream_t)stream);
        if (st != SUBMCONV_OK) { dev_free(p, (hipStream_t)stream); return st; }
        rb->nbr_in = (int32_t *)p;
    }
    *nbr = rb->nbr_in;
    *n = rb->n;
    return SUBMCONV_OK;
}

int submconv_rulebook_copy_neighbors(const submconv_rulebook *rb, int32_t *dst, void *stream)
{
    if (!rb) return fail(SUBMCONV_E_INVALID_ARG, "rulebook is NULL");
    if (rb->n == 0) return SUBMCONV_OK;
    if (!dst) return fail(SUBMCONV_E_INVALID_ARG, "dst is NULL");
    const size_t bytes = (size_t)rb->n * 27 * 4;
    if (overlaps(dst, bytes, rb->block, rb->block_bytes)) return fail(SUBMCONV_E_ALIAS, "dst overlaps the rulebook");
    return input_order_table(rb, dst, (hipStream_t)stream);
}

int submconv_rulebook_info(const submconv_rulebook *rb, int64_t *n, int32_t *res, int32_t *batch,
                           int64_t *taps_present)
{
    if (!rb) return fail(SUBMCONV_E_INVALID_ARG, "rulebook is NULL");
    if (n) *n = rb->n;
    if (res) *res = rb->res;
    if (batch) *batch = rb->batch;
    if (taps_present) *taps_present = rb->taps;
    return SUBMCONV_OK;
}

int submconv_rulebook_free(submconv_rulebook *rb, void *stream)
{
    if (!rb) return SUBMCONV_OK;
    dev_free(rb->nbr_in, (hipStream_t)stream);
    dev_free(rb->block, (hipStream_t)stream);
    delete rb;
    return SUBMCONV_OK;
}

int submconv_forward_variant(const void *feats, const void *weight, const float *bias,
                             const submconv_rulebook *rb, void *out, int32_t cin, int32_t cout,
                             int32_t dtype, int32_t flip, int32_t variant, void *stream)
{
    if (!rb) return fail(SUBMCONV_E_INVALID_ARG, "rulebook is NULL");
    if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
    if (cin < 1 || cin > 1024 || cout < 1 || cout > 1024)
        return fail(SUBMCONV_E_UNSUPPORTED, "channel counts %d -> %d outside 1..1024", cin, cout);
    if (flip != 0 && flip != 1) return fail(SUBMCONV_E_INVALID_ARG, "flip must be 0 or 1");
    if (variant < SUBMCONV_KERNEL_AUTO || variant > SUBMCONV_KERNEL_PERSISTENT)
        return fail(SUBMCONV_E_INVALID_ARG, "unknown kernel variant %d", variant);
    const int64_t n = rb->n;
    if (n == 0) return SUBMCONV_OK;
    if (!feats || !weight || !out) return fail(SUBMCONV_E_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(feats) || !aligned16(weight) || !aligned16(out) || (bias && !aligned16(bias)))
        return fail(SUBMCONV_E_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const size_t es = elem_size(dtype);
    const size_t fb = (size_t)n * cin * es, wb = (size_t)cout * 27 * cin * es, ob = (size_t)n * cout * es;
    if (overlaps(out, ob, feats, fb) || overlaps(out, ob, weight, wb) ||
        (bias && overlaps(out, ob, bias, (size_t)cout * 4)))
        return fail(SUBMCONV_E_ALIAS, "out overlaps feats, weight or bias");
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev != rb->device)
        return fail(SUBMCONV_E_INVALID_ARG, "rulebook lives on device %d, current device is %d", rb->device, dev);
    return launch_forward(feats, weight, bias, rb, out, cin, cout, dtype, flip, variant,
                          (hipStream_t)stream);
}

int submconv_forward(const void *feats, const void *weight, const float *bias,
                     const submconv_rulebook *rb, void *out, int32_t cin, int32_t cout,
                     int32_t dtype, int32_t flip, void *stream)
{
    return submconv_forward_variant(feats, weight, bias, rb, out, cin, cout, dtype, flip,
                                    SUBMCONV_KERNEL_AUTO, stream);
}

int submconv_subdivide(const int32_t *coords, const void *feats, int64_t n, int32_t c,
                       int32_t dtype, int32_t *out_coords, void *out_feats, void *stream)
{
    if (n < 0 || n >= (int64_t(1) << 28)) return fail(SUBMCONV_E_INVALID_ARG, "n = %lld outside [0, 2^28)", (long long)n);
    if (n == 0) return SUBMCONV_OK;
    if (!coords || !out_coords) return fail(SUBMCONV_E_INVALID_ARG, "NULL coordinate pointer");
    if (!aligned16(coords) || !aligned16(out_coords)) return fail(SUBMCONV_E_INVALID_ARG, "coordinate pointers must be 16-byte aligned");
    if (overlaps(out_coords, (size_t)n * 128, coords, (size_t)n * 16)) return fail(SUBMCONV_E_ALIAS, "out_coords overlaps coords");
    if (feats) {
        if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
        if (c < 1 || c > 65536) return fail(SUBMCONV_E_INVALID_ARG, "c = %d", c);
        if (!out_feats) return fail(SUBMCONV_E_INVALID_ARG, "out_feats is NULL");
        const size_t es = elem_size(dtype);
        if (((uintptr_t)feats | (uintptr_t)out_feats) & (((size_t)c * es) % 4 == 0 ? 3u : 1u))
            return fail(SUBMCONV_E_INVALID_ARG, "feature pointers misaligned");
        if (overlaps(out_feats, (size_t)n * 8 * c * es, feats, (size_t)n * c * es))
            return fail(SUBMCONV_E_ALIAS, "out_feats overlaps feats");
    }
    return subdivide(coords, feats, n, c, dtype, out_coords, out_feats, (hipStream_t)stream);
}

int submconv_space_to_depth(const int32_t *coords, const void *feats, int64_t n, int32_t c,
                            int32_t dtype, int32_t res, int32_t batch, int32_t *out_coords,
                            void *out_feats, uint8_t *out_mask, int64_t *out_m, void *stream)
{
    if (!out_m) return fail(SUBMCONV_E_INVALID_ARG, "out_m is NULL");
    *out_m = 0;
    if (n < 0 || n >= (int64_t(1) << 31)) return fail(SUBMCONV_E_INVALID_ARG, "n = %lld outside [0, 2^31)", (long long)n);
    if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
    if (c < 1 || c > 65536) return fail(SUBMCONV_E_INVALID_ARG, "c = %d", c);
    if (res < 1 || batch < 1) return fail(SUBMCONV_E_INVALID_ARG, "res and batch must be >= 1");
    if (n == 0) return SUBMCONV_OK;
    if (!coords || !feats || !out_coords || !out_feats) return fail(SUBMCONV_E_INVALID_ARG, "NULL pointer");
    if (!aligned16(coords) || !aligned16(out_coords)) return fail(SUBMCONV_E_INVALID_ARG, "coordinate pointers must be 16-byte aligned");
    const size_t es = elem_size(dtype);
    if (overlaps(out_feats, (size_t)n * 8 * c * es, feats, (size_t)n * c * es) ||
        overlaps(out_coords, (size_t)n * 16, coords, (size_t)n * 16))
        return fail(SUBMCONV_E_ALIAS, "an output overlaps an input");
    return space_to_depth(coords, feats, n, c, dtype, res, batch, out_coords, out_feats, out_mask,
                          out_m, (hipStream_t)stream);
}

int submconv_depth_to_space(const int32_t *coarse_coords, const void *coarse_feats,
                            const uint8_t *mask, int64_t m, int32_t c, int32_t dtype,
                            int32_t *out_coords, void *out_feats, int64_t *out_n, void *stream)
{
    if (!out_n) return fail(SUBMCONV_E_INVALID_ARG, "out_n is NULL");
    *out_n = 0;
    if (m < 0 || m >= (int64_t(1) << 28)) return fail(SUBMCONV_E_INVALID_ARG, "m = %lld outside [0, 2^28)", (long long)m);
    if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
    if (c < 1 || c > 65536) return fail(SUBMCONV_E_INVALID_ARG, "c = %d", c);
    if (m == 0) return SUBMCONV_OK;
    if (!coarse_coords || !coarse_feats || !out_coords || !out_feats) return fail(SUBMCONV_E_INVALID_ARG, "NULL pointer");
    if (!aligned16(coarse_coords) || !aligned16(out_coords)) return fail(SUBMCONV_E_INVALID_ARG, "coordinate pointers must be 16-byte aligned");
    const size_t es = elem_size(dtype);
    if (overlaps(out_feats, (size_t)m * 8 * c * es, coarse_feats, (size_t)m * 8 * c * es) ||
        overlaps(out_coords, (size_t)m * 128, coarse_coords, (size_t)m * 16))
        return fail(SUBMCONV_E_ALIAS, "an output overlaps an input");
    return depth_to_space(coarse_coords, coarse_feats, mask, m, c, dtype, out_coords, out_feats,
                          out_n, (hipStream_t)stream);
}

static int check_upsample_masked(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n,
                                 int32_t c, int32_t dtype, int32_t *out_coords, void *out_feats, int64_t *out_n,
                                 int64_t max_n)
{
    if (!out_n) return fail(SUBMCONV_E_INVALID_ARG, "out_n is NULL");
    *out_n = 0;
    if (n < 0 || n >= (int64_t(1) << 28)) return fail(SUBMCONV_E_INVALID_ARG, "n = %lld outside [0, 2^28)", (long long)n);
    if (n > max_n) return fail(SUBMCONV_E_UNSUPPORTED, "n = %lld above the limit %lld", (long long)n, (long long)max_n);
    if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
    if (c < 1 || c > 65536) return fail(SUBMCONV_E_INVALID_ARG, "c = %d", c);
    if (n == 0) return SUBMCONV_OK;
    if (!coords || !feats || !mask || !out_coords || !out_feats) return fail(SUBMCONV_E_INVALID_ARG, "NULL pointer");
    if (!aligned16(coords) || !aligned16(out_coords)) return fail(SUBMCONV_E_INVALID_ARG, "coordinate pointers must be 16-byte aligned");
    const size_t es = elem_size(dtype);
    if (overlaps(out_feats, (size_t)n * 8 * c * es, feats, (size_t)n * c * es) ||
        overlaps(out_coords, (size_t)n * 128, coords, (size_t)n * 16) ||
        overlaps(out_feats, (size_t)n * 8 * c * es, mask, (size_t)n * 8) ||
        overlaps(out_coords, (size_t)n * 128, mask, (size_t)n * 8))
        return fail(SUBMCONV_E_ALIAS, "an output overlaps an input");
    return SUBMCONV_OK;
}

int submconv_upsample_masked(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n, int32_t c,
                             int32_t dtype, int32_t *out_coords, void *out_feats, int64_t *out_n, void *stream)
{
    SC_CHECK(check_upsample_masked(coords, feats, mask, n, c, dtype, out_coords, out_feats, out_n, int64_t(1) << 28));
    if (n == 0) return SUBMCONV_OK;
    return upsample_masked(coords, feats, mask, n, c, dtype, out_coords, out_feats, out_n, (hipStream_t)stream);
}

int submconv_upsample_masked_noalloc(const int32_t *coords, const void *feats, const uint8_t *mask, int64_t n,
                                     int32_t c, int32_t dtype, int32_t *out_coords, void *out_feats,
                                     int64_t *out_n, void *stream)
{
    static_assert(SUBMCONV_NOALLOC_MAX_N >= 1, "limit");
    SC_CHECK(check_upsample_masked(coords, feats, mask, n, c, dtype, out_coords, out_feats, out_n,
                                   SUBMCONV_NOALLOC_MAX_N));
    if (n == 0) return SUBMCONV_OK;
    if (noalloc_expand_bytes(n) > SUBMCONV_NOALLOC_SCRATCH_BYTES)  // cannot happen for n <= the limit
        return fail(SUBMCONV_E_UNSUPPORTED, "n = %lld does not fit the scratch array", (long long)n);
    return upsample_masked_noalloc(coords, feats, mask, n, c, dtype, out_coords, out_feats, out_n,
                                   (hipStream_t)stream);
}

int submconv_downsample(const int32_t *coords, const void *feats, int64_t n, int32_t c, int32_t dtype, int32_t res,
                        int32_t batch, int32_t mode, int32_t *out_coords, void *out_feats, int64_t *out_m,
                        void *stream)
{
    if (!out_m) return fail(SUBMCONV_E_INVALID_ARG, "out_m is NULL");
    *out_m = 0;
    if (n < 0 || n >= (int64_t(1) << 31)) return fail(SUBMCONV_E_INVALID_ARG, "n = %lld outside [0, 2^31)", (long long)n);
    if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
    if (mode != SUBMCONV_POOL_MAX && mode != SUBMCONV_POOL_MEAN) return fail(SUBMCONV_E_INVALID_ARG, "mode %d", mode);
    if (c < 1 || c > 65536) return fail(SUBMCONV_E_INVALID_ARG, "c = %d", c);
    if (res < 1 || batch < 1) return fail(SUBMCONV_E_INVALID_ARG, "res and batch must be >= 1");
    if (n == 0) return SUBMCONV_OK;
    if (!coords || !feats || !out_coords || !out_feats) return fail(SUBMCONV_E_INVALID_ARG, "NULL pointer");
    if (!aligned16(coords) || !aligned16(out_coords)) return fail(SUBMCONV_E_INVALID_ARG, "coordinate pointers must be 16-byte aligned");
    const size_t es = elem_size(dtype);
    if (overlaps(out_feats, (size_t)n * c * es, feats, (size_t)n * c * es) ||
        overlaps(out_coords, (size_t)n * 16, coords, (size_t)n * 16))
        return fail(SUBMCONV_E_ALIAS, "an output overlaps an input");
    return downsample(coords, feats, n, c, dtype, res, batch, mode == SUBMCONV_POOL_MEAN, out_coords, out_feats,
                      out_m, (hipStream_t)stream);
}

int submconv_classify_5d(const int64_t *shape, int32_t hint, int32_t *layout)
{
    if (!shape || !layout) return fail(SUBMCONV_E_INVALID_ARG, "NULL pointer");
    int l = SUBMCONV_LAYOUT_UNKNOWN;
    const int status = classify_5d(shape, hint, &l);
    *layout = l;
    return status;
}

int submconv_weight_convert(const void *src, int32_t layout, int32_t cout, int32_t cin, int32_t dtype, int32_t flip,
                            void *dst, void *stream)
{
    if (layout != SUBMCONV_LAYOUT_KRSC && layout != SUBMCONV_LAYOUT_OIDHW)
        return fail(SUBMCONV_E_INVALID_ARG, "layout %d", layout);
    if (dtype != SUBMCONV_F32 && dtype != SUBMCONV_BF16) return fail(SUBMCONV_E_UNSUPPORTED, "dtype %d", dtype);
    if (cout < 1 || cin < 1 || (int64_t)cout * cin > (int64_t(1) << 24))
        return fail(SUBMCONV_E_INVALID_ARG, "cout = %d, cin = %d", cout, cin);
    if (!src || !dst) return fail(SUBMCONV_E_INVALID_ARG, "NULL pointer");
    const size_t bytes = (size_t)cout * 27 * cin * elem_size(dtype);
    if (overlaps(dst, bytes, src, bytes)) return fail(SUBMCONV_E_ALIAS, "dst overlaps src");
    return weight_convert(src, layout, cout, cin, dtype, flip, dst, (hipStream_t)stream);
}

int submconv_release_cache(int32_t device)
{
    std::lock_guard<std::mutex> lock(g_cache_mu);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(SUBMCONV_E_HIP, "hipGetDevice failed");
    release_cached(device);
    (void)hipSetDevice(cur);
    (void)hipDeviceSynchronize();  // the frees are queued on the null stream; let them land
    return SUBMCONV_OK;
}

int submconv_set_cache_limit(int64_t bytes)
{
    if (bytes < 0) return fail(SUBMCONV_E_INVALID_ARG, "cache limit %lld < 0", (long long)bytes);
    std::lock_guard<std::mutex> lock(g_cache_mu);
    g_cap = (size_t)bytes;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(SUBMCONV_E_HIP, "hipGetDevice failed");
    for (int d = 0; d < 64; ++d)  // shrink: drop cached blocks of devices above the new limit
        if (g_cached[d] > g_cap) release_cached(d);
    (void)hipSetDevice(cur);
    return SUBMCONV_OK;
}

}  // extern "C"
