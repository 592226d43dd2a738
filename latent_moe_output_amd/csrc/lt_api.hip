// lt_api.hip -- C ABI of liblatenttail.so: validation, scratch, dispatch.
//
// The entry point follows [PR50383 Key source snippets, `_shard_up_proj_tail`]
// on one GPU: reduce the routed partials (locally, over n_partials), norm,
// narrow W rows and out columns to [c0, c0+n), add the projection in place.
// The token-count dispatcher mirrors the tier choice of [PR50383
// Implementation, item 1], reduced to the two single-GPU paths:
//   T <= skinny_max  -> one weight-streaming launch per 64 tokens (32 when
//                       L > 1024) (k_skinny)
//   T >  skinny_max  -> k_sum_rmsnorm into a scratch latent, then k_gemm
//                       (one partial without the norm: k_gemm reads it as is).
// lt_latent_tail_residual runs the same path with the decoder layer's
// residual update fused into the epilogue of the projection kernel.
// The pages' own fallback is silent ([PR51253 Implementation, item 2]); a
// library cannot fall back to a path it does not own, so every violated
// precondition is an explicit status code returned before any launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <thread>
#include <tuple>
#include <utility>
#include <vector>

#include "latent_tail.h"
#include "lt_internal.h"

namespace {

constexpr int64_t kDefaultSkinnyMax = 64;

std::atomic<int64_t> g_skinny_max{-1};
// timing events of lt_set_kernel_events, per calling thread
thread_local void *g_ev_before = nullptr;
thread_local void *g_ev_after = nullptr;

// Records the timing event `ev` (if set) on `s`.
bool record_hook(void *ev, hipStream_t s)
{
    return !ev || hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s) == hipSuccess;
}

int64_t default_skinny_max()
{
    static const int64_t v = [] {
        const char *e = std::getenv("LT_SKINNY_MAX_T");
        if (e && *e) {
            char *end = nullptr;
            long long x = std::strtoll(e, &end, 10);
            if (end && *end == '\0' && x >= 0) return (int64_t)x;
        }
        return kDefaultSkinnyMax;
    }();
    return v;
}

int64_t skinny_max()
{
    int64_t v = g_skinny_max.load(std::memory_order_relaxed);
    return v < 0 ? default_skinny_max() : v;
}

// ---- scratch: one [T][L] bf16 latent buffer per (device, stream) ----------
// hipStreamPerThread is one handle that names a different stream in every
// host thread, so for it the calling thread is part of the key.
struct ScratchKey {
    int dev;
    uintptr_t stream;
    std::thread::id tid;
    bool operator<(const ScratchKey &o) const
    {
        return std::tie(dev, stream, tid) < std::tie(o.dev, o.stream, o.tid);
    }
};
struct Scratch {
    void *ptr = nullptr;
    size_t bytes = 0;
};
// g_mu guards the map and every buffer in it.  A caller holds it from
// looking a buffer up until the kernels that use it are enqueued, so two
// calls on one stream from different threads never interleave their norm
// and GEMM kernels on one buffer.
std::mutex g_mu;
std::map<ScratchKey, Scratch> g_scratch;
// Buffers that a larger one replaced.  Kernels already queued, and graphs
// captured earlier, may still read and write them, so they stay allocated
// until lt_release_scratch (growth neither frees nor synchronises).
std::vector<std::pair<int, void *>> g_retired;

ScratchKey scratch_key(int dev, hipStream_t stream)
{
    return {dev, reinterpret_cast<uintptr_t>(stream),
            stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
}

// Returns a scratch buffer of at least `bytes` for (current device, stream).
// The caller holds g_mu.  Sizes are powers of two from 1 MiB, so the retired
// buffers of a stream never add up to more than its current one.
int ensure_scratch(size_t bytes, hipStream_t stream, void **out_ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LT_ERR_HIP;
    Scratch &s = g_scratch[scratch_key(dev, stream)];
    if (s.bytes >= bytes) {
        *out_ptr = s.ptr;
        return LT_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return LT_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return LT_ERR_NO_MEMORY;  // never allocate in capture
    size_t want = (size_t)1 << 20;
    while (want < bytes) {
        if (want > SIZE_MAX / 2) return LT_ERR_NO_MEMORY;
        want <<= 1;
    }
    const hipError_t pending = hipPeekAtLastError();
    void *p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
        if (pending == hipSuccess) (void)hipGetLastError();   // only the error this call set
        return LT_ERR_NO_MEMORY;
    }
    if (s.ptr) g_retired.emplace_back(dev, s.ptr);
    s.ptr = p;
    s.bytes = want;
    *out_ptr = p;
    return LT_OK;
}

// ---- the fixed scratch of lt_latent_tail_noalloc ---------------------------
// One [T][L] bf16 latent of at most LT_NOALLOC_MAX_LATENT elements per
// device, held for the life of the process.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns for the current device (g_noalloc_ptr), never
// the array's name.  Every noalloc call on a device shares its array.
static __device__ __align__(256) uint16_t scratch[LT_NOALLOC_MAX_LATENT];

constexpr int kMaxDevices = 64;
void *g_noalloc_ptr[kMaxDevices] = {};   // guarded by g_mu

// Device address of the current device's `scratch`, resolved once per
// device (no allocation).  The caller holds g_mu.
int noalloc_scratch(void **out_ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LT_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LT_ERR_UNSUPPORTED;
    if (!g_noalloc_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LT_ERR_HIP;
        g_noalloc_ptr[dev] = p;
    }
    *out_ptr = g_noalloc_ptr[dev];
    return LT_OK;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool mul_ok(int64_t a, int64_t b, int64_t *r)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *r = a * b;
    return true;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

const char *lt_status_string(int status)
{
    switch (status) {
    case LT_OK: return "LT_OK";
    case LT_ERR_INVALID_ARG: return "LT_ERR_INVALID_ARG: argument out of range, NULL or overlapping";
    case LT_ERR_UNSUPPORTED: return "LT_ERR_UNSUPPORTED: latent width or alignment not handled";
    case LT_ERR_NO_MEMORY: return "LT_ERR_NO_MEMORY: scratch could not be allocated";
    case LT_ERR_HIP: return "LT_ERR_HIP: HIP call or kernel launch failed";
    case LT_ERR_SCRATCH_LIMIT:
        return "LT_ERR_SCRATCH_LIMIT: T*L exceeds the fixed scratch of lt_latent_tail_noalloc";
    default: return "unknown lt status";
    }
}

const char *lt_version(void) { return "liblatenttail 0.2.0 gfx950"; }

int64_t lt_set_skinny_max_tokens(int64_t t)
{
    const int64_t prev = skinny_max();
    g_skinny_max.store(t < 0 ? -1 : t, std::memory_order_relaxed);
    return prev;
}

int64_t lt_get_skinny_max_tokens(void) { return skinny_max(); }

int lt_set_kernel_events(void *before, void *after)
{
    g_ev_before = before;
    g_ev_after = after;
    return LT_OK;
}

int lt_path_for(int64_t T, int64_t n)
{
    if (T <= 0 || n <= 0) return 0;
    return T <= skinny_max() ? 1 : 2;
}

int lt_reserve(int64_t max_T, int64_t L, void *stream)
{
    if (max_T < 0 || L < 1) return LT_ERR_INVALID_ARG;
    int64_t elems = 0;
    if (!mul_ok(max_T, L, &elems) || elems > INT64_MAX / 2) return LT_ERR_INVALID_ARG;
    if (elems == 0) return LT_OK;
    void *p = nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return ensure_scratch((size_t)elems * 2, reinterpret_cast<hipStream_t>(stream), &p);
}

int lt_release_scratch(void)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LT_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (hipDeviceSynchronize() != hipSuccess) return LT_ERR_HIP;
    for (auto it = g_scratch.begin(); it != g_scratch.end();) {
        if (it->first.dev == dev) {
            if (it->second.ptr && hipFree(it->second.ptr) != hipSuccess) return LT_ERR_HIP;
            it = g_scratch.erase(it);
        } else {
            ++it;
        }
    }
    for (auto it = g_retired.begin(); it != g_retired.end();) {
        if (it->first == dev) {
            if (hipFree(it->second) != hipSuccess) return LT_ERR_HIP;
            it = g_retired.erase(it);
        } else {
            ++it;
        }
    }
    return LT_OK;
}

}  // extern "C"

namespace {

// The tail, with the residual update when `res` is set (its pointers
// validated by the caller and not yet offset by c0).  With `fixed` the
// large-token path's latent goes to the device's fixed `scratch` array
// (nothing is allocated); otherwise to the stream's growable buffer.
int tail_impl(const void *partials, int n_partials, int64_t T, int64_t L, const void *norm_w,
              float eps, const void *W, int64_t H, int64_t c0, int64_t n, void *out,
              int64_t ld_out, const lt::Resid *res_in, void *stream, bool fixed)
{
    // ---- sizes and window
    if (n_partials < 1 || T < 0 || L < 1 || H < 1 || c0 < 0 || n < 0 || c0 > H || n > H - c0 ||
        ld_out < H)
        return LT_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.f) return LT_ERR_INVALID_ARG;
    if (L % 8 != 0 || L > LT_MAX_L) return LT_ERR_UNSUPPORTED;
    if (T == 0 || n == 0) return LT_OK;
    if (!partials || !W || !out) return LT_ERR_INVALID_ARG;

    int64_t tl = 0, ptl = 0, hl = 0, tld = 0;
    if (!mul_ok(T, L, &tl) || !mul_ok(tl, n_partials, &ptl) || !mul_ok(H, L, &hl) ||
        !mul_ok(T - 1, ld_out, &tld) || tld > INT64_MAX - H || ptl > INT64_MAX / 2 ||
        hl > INT64_MAX / 2 || tld + H > INT64_MAX / 2)
        return LT_ERR_INVALID_ARG;
    if (n > 0x7FFFFFFF || L > 0x7FFFFFFF) return LT_ERR_UNSUPPORTED;

    // ---- alignment (16-byte vector loads of every input row)
    if (!aligned(partials, 16) || !aligned(W, 16) || (norm_w && !aligned(norm_w, 16)) ||
        !aligned(out, 2))
        return LT_ERR_UNSUPPORTED;

    // ---- out must not alias an input
    const size_t out_bytes = (size_t)(tld + H) * 2;
    if (ranges_overlap(out, out_bytes, partials, (size_t)ptl * 2) ||
        ranges_overlap(out, out_bytes, W, (size_t)hl * 2) ||
        ranges_overlap(out, out_bytes, norm_w, (size_t)L * 2))
        return LT_ERR_INVALID_ARG;

    // ---- the residual buffers: prefix is read, resid written (resid may be
    // the prefix buffer itself, with the same stride)
    lt::Resid res_win{};
    const lt::Resid *res = nullptr;
    if (res_in) {
        const lt::Resid &r = *res_in;
        if (!r.prefix || !r.resid || r.ld_prefix < c0 + n || r.ld_resid < c0 + n)
            return LT_ERR_INVALID_ARG;
        int64_t tp = 0, tr = 0;
        if (!mul_ok(T - 1, r.ld_prefix, &tp) || !mul_ok(T - 1, r.ld_resid, &tr) ||
            tp > INT64_MAX / 4 || tr > INT64_MAX / 4)
            return LT_ERR_INVALID_ARG;
        if (!aligned(r.prefix, 2) || !aligned(r.resid, 2)) return LT_ERR_UNSUPPORTED;
        const size_t pb = (size_t)(tp + c0 + n) * 2, rb = (size_t)(tr + c0 + n) * 2;
        const size_t ob = (size_t)(tld + H) * 2;
        const bool same = r.resid == r.prefix && r.ld_resid == r.ld_prefix;
        if (ranges_overlap(r.resid, rb, partials, (size_t)ptl * 2) ||
            ranges_overlap(r.resid, rb, W, (size_t)hl * 2) ||
            ranges_overlap(r.resid, rb, norm_w, (size_t)L * 2) ||
            ranges_overlap(r.resid, rb, out, ob) || ranges_overlap(r.prefix, pb, out, ob) ||
            (!same && ranges_overlap(r.resid, rb, r.prefix, pb)))
            return LT_ERR_INVALID_ARG;
        res_win = {r.prefix + c0, r.ld_prefix, r.resid + c0, r.ld_resid};
        res = &res_win;
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint16_t *part = static_cast<const uint16_t *>(partials);
    const uint16_t *nw = static_cast<const uint16_t *>(norm_w);
    const uint16_t *Wn = static_cast<const uint16_t *>(W) + c0 * L;
    uint16_t *outn = static_cast<uint16_t *>(out) + c0;

    if (T <= skinny_max()) {
        const int per = lt::skinny_tokens_per_launch((int)L);
        if (!record_hook(g_ev_before, s)) return LT_ERR_HIP;
        for (int64_t tb = 0; tb < T; tb += per) {
            const int tc = (int)((T - tb) < per ? (T - tb) : per);
            lt::Resid rb{};
            if (res)
                rb = {res->prefix + tb * res->ld_prefix, res->ld_prefix,
                      res->resid + tb * res->ld_resid, res->ld_resid};
            hipError_t e = lt::launch_skinny(part + tb * L, tl, n_partials, tc, (int)L, nw, eps,
                                             Wn, (int)n, outn + tb * ld_out, ld_out,
                                             res ? &rb : nullptr, s);
            if (e != hipSuccess) return LT_ERR_HIP;
        }
        return record_hook(g_ev_after, s) ? LT_OK : LT_ERR_HIP;
    }

    // one partial and no norm: the latent is the partial itself (its bf16
    // storage round trip is exact), so the GEMM reads it in place
    if (n_partials == 1 && !nw) {
        if (!record_hook(g_ev_before, s)) return LT_ERR_HIP;
        if (lt::launch_gemm(part, T, (int)L, Wn, (int)n, outn, ld_out, res, s) != hipSuccess)
            return LT_ERR_HIP;
        return record_hook(g_ev_after, s) ? LT_OK : LT_ERR_HIP;
    }

    if (fixed && tl > (int64_t)LT_NOALLOC_MAX_LATENT) return LT_ERR_SCRATCH_LIMIT;
    // the scratch stays locked until both kernels that use it are enqueued
    std::lock_guard<std::mutex> lock(g_mu);
    void *buf = nullptr;
    int st = fixed ? noalloc_scratch(&buf) : ensure_scratch((size_t)tl * 2, s, &buf);
    if (st != LT_OK) return st;
    uint16_t *y = static_cast<uint16_t *>(buf);
    if (lt::launch_sum_rmsnorm(part, tl, n_partials, T, (int)L, nw, eps, y, s) != hipSuccess)
        return LT_ERR_HIP;
    if (!record_hook(g_ev_before, s)) return LT_ERR_HIP;
    if (lt::launch_gemm(y, T, (int)L, Wn, (int)n, outn, ld_out, res, s) != hipSuccess)
        return LT_ERR_HIP;
    return record_hook(g_ev_after, s) ? LT_OK : LT_ERR_HIP;
}

}  // namespace

extern "C" {

int lt_latent_tail(const void *partials, int n_partials, int64_t T, int64_t L,
                   const void *norm_w, float eps, const void *W, int64_t H, int64_t c0,
                   int64_t n, void *out, int64_t ld_out, void *stream)
{
    return tail_impl(partials, n_partials, T, L, norm_w, eps, W, H, c0, n, out, ld_out, nullptr,
                     stream, false);
}

int lt_latent_tail_noalloc(const void *partials, int n_partials, int64_t T, int64_t L,
                           const void *norm_w, float eps, const void *W, int64_t H, int64_t c0,
                           int64_t n, void *out, int64_t ld_out, void *stream)
{
    return tail_impl(partials, n_partials, T, L, norm_w, eps, W, H, c0, n, out, ld_out, nullptr,
                     stream, true);
}

int lt_latent_tail_residual(const void *partials, int n_partials, int64_t T, int64_t L,
                            const void *norm_w, float eps, const void *W, int64_t H, int64_t c0,
                            int64_t n, void *out, int64_t ld_out, const void *prefix,
                            int64_t ld_prefix, void *resid, int64_t ld_resid, void *stream)
{
    const lt::Resid r{static_cast<const uint16_t *>(prefix), ld_prefix,
                      static_cast<uint16_t *>(resid), ld_resid};
    return tail_impl(partials, n_partials, T, L, norm_w, eps, W, H, c0, n, out, ld_out, &r,
                     stream, false);
}

int lt_attn_res_zero_block(void *prefix, const void *delta, int64_t T, int64_t H,
                           void *block_residual, int64_t num_slots, int64_t block_idx,
                           const void *norm_w, float eps, void *out, void *stream)
{
    if (T < 0 || H < 1 || num_slots < 0 || block_idx >= num_slots || block_idx < -1)
        return LT_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.f) return LT_ERR_INVALID_ARG;
    if (H % 8 != 0 || H > LT_ATTN_RES_MAX_H) return LT_ERR_UNSUPPORTED;
    if (T == 0) return LT_OK;
    if (T > 0x7FFFFFFF) return LT_ERR_UNSUPPORTED;
    const bool write_block = block_idx >= 0;
    if (!prefix || !out || (write_block && !block_residual)) return LT_ERR_INVALID_ARG;
    int64_t th = 0, tsh = 0;
    if (!mul_ok(T, H, &th) || th > INT64_MAX / 4 || !mul_ok(th, num_slots, &tsh) ||
        tsh > INT64_MAX / 4)
        return LT_ERR_INVALID_ARG;
    if (!aligned(prefix, 16) || !aligned(out, 16) || (delta && !aligned(delta, 16)) ||
        (norm_w && !aligned(norm_w, 16)) || (write_block && !aligned(block_residual, 16)))
        return LT_ERR_UNSUPPORTED;
    // out and the block are written, the prefix too when there is a delta:
    // none of them may overlap another buffer
    const size_t rb = (size_t)th * 2, bb = (size_t)tsh * 2, wb = (size_t)H * 2;
    const void *blk = write_block ? block_residual : nullptr;
    if (ranges_overlap(out, rb, prefix, rb) || ranges_overlap(out, rb, delta, rb) ||
        ranges_overlap(out, rb, norm_w, wb) || ranges_overlap(out, rb, blk, bb) ||
        ranges_overlap(blk, bb, prefix, rb) || ranges_overlap(blk, bb, delta, rb) ||
        ranges_overlap(blk, bb, norm_w, wb) || ranges_overlap(prefix, rb, delta, rb) ||
        ranges_overlap(prefix, rb, norm_w, wb))
        return LT_ERR_INVALID_ARG;
    uint16_t *slot = write_block ? static_cast<uint16_t *>(block_residual) + block_idx * H
                                 : nullptr;
    const hipError_t e = lt::launch_attn_res(
        static_cast<uint16_t *>(prefix), static_cast<const uint16_t *>(delta), T, (int)H, slot,
        num_slots * H, static_cast<const uint16_t *>(norm_w), eps, static_cast<uint16_t *>(out),
        reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? LT_OK : LT_ERR_HIP;
}

}  // extern "C"
