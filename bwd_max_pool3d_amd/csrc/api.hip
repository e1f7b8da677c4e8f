// api.hip -- the C ABI declared in include/mp3d.h: argument checks, the
// choice of kernel, launch planning, and error reporting.
//
// Every check runs before the first launch, so a failing call writes
// nothing.  The library allocates no device memory: all buffers belong to
// the caller, and the only per-process state is the cached LDS limit of
// each device and the per-thread error message.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../../include/mp3d.h"
#include "dtype.hpp"
#include "idxsrc.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

thread_local char g_msg[256] = "";

// mp3d_time_next_call: events armed for the next call on this thread
thread_local LaunchTiming g_timing = {nullptr, nullptr};

// Disarms the kernel-time events when a C-ABI call returns, whether or not
// it launched anything.
struct TimingScope {
    ~TimingScope() { g_timing = {nullptr, nullptr}; }
};

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return code;
}

// MP3D_SMALL=0 turns the small-tensor kernels off, so that the general
// kernels can be exercised on small inputs (read on every call).
bool small_enabled()
{
    const char *v = getenv("MP3D_SMALL");
    return !(v && strcmp(v, "0") == 0);
}

// MP3D_TWO_PASS=1: the index-free backward takes the two-pass form whenever
// a workspace is given (tests use it to reach that form on any shape).
bool two_pass_forced()
{
    const char *v = getenv("MP3D_TWO_PASS");
    return v && strcmp(v, "1") == 0;
}

bool log_enabled()
{
    static int on = -1;
    if (on < 0) {
        const char *v = getenv("MP3D_LOG");
        on = (v && *v && strcmp(v, "0") != 0) ? 1 : 0;
    }
    return on == 1;
}

constexpr int64_t kInt32Max = 2147483647;

// Shared checks of shapes and pointers; fills the per-plane sizes of g.
int check_common(int dtype, int64_t N, int64_t C, int64_t D, int64_t H, int64_t W)
{
    if (dtype != MP3D_F32 && dtype != MP3D_F16 && dtype != MP3D_BF16 && dtype != MP3D_F64)
        return fail(MP3D_EDTYPE, "dtype %d is not MP3D_F32, MP3D_F16, MP3D_BF16 or MP3D_F64",
                    dtype);
    if (N < 0 || C < 0)
        return fail(MP3D_EINVAL, "N=%lld and C=%lld must be >= 0", (long long)N, (long long)C);
    if (D <= 0 || H <= 0 || W <= 0)
        return fail(MP3D_EINVAL, "spatial extents must be >= 1 (D=%lld H=%lld W=%lld)",
                    (long long)D, (long long)H, (long long)W);
    if (D > kInt32Max || H > kInt32Max || W > kInt32Max || D * H > kInt32Max ||
        D * H * W > kInt32Max)
        return fail(MP3D_EOVERFLOW, "D*H*W exceeds the int32 index range");
    const int64_t plane = D * H * W;
    if (N > 0 && C > ((int64_t)1 << 62) / N / plane)
        return fail(MP3D_EOVERFLOW, "N*C*D*H*W exceeds 2^62 elements");
    return MP3D_OK;
}

int set_fixed_axis(Axis *a, int64_t X, int32_t k, int32_t s, const char *name)
{
    if (k <= 0 || s <= 0)
        return fail(MP3D_EINVAL, "kernel and stride on %s must be >= 1 (got %d, %d)", name, k, s);
    if (X < k)
        return fail(MP3D_EINVAL, "kernel %d exceeds extent %lld on %s", k, (long long)X, name);
    *a = Axis::make((int32_t)X, (int32_t)((X - k) / s + 1), k, s);
    return MP3D_OK;
}

// Output extent of a fixed axis with padding and dilation: floor mode
// counts the windows whose span fits the padded axis; ceil mode also keeps
// a last partial window if it starts inside the input or the left padding.
// -1 if not even one window fits.
int64_t fixed_out_ex(int64_t X, int64_t k, int64_t s, int64_t pad, int64_t dil, bool ceil_mode)
{
    const int64_t ext = (k - 1) * dil + 1, room = X + 2 * pad - ext;
    if (room < 0) return -1;
    int64_t O = (ceil_mode ? (room + s - 1) / s : room / s) + 1;
    if (ceil_mode && (O - 1) * s >= X + pad) --O;
    return O;
}

// Validation shared by the padded / dilated entry points.
int check_fixed_ex(int64_t X, int64_t k, int64_t s, int64_t pad, int64_t dil, const char *name)
{
    if (k <= 0 || s <= 0)
        return fail(MP3D_EINVAL, "kernel and stride on %s must be >= 1 (got %lld, %lld)", name,
                    (long long)k, (long long)s);
    if (pad < 0 || dil <= 0)
        return fail(MP3D_EINVAL, "padding on %s must be >= 0 and dilation >= 1 (got %lld, %lld)",
                    name, (long long)pad, (long long)dil);
    if ((k - 1) * dil + 1 > kInt32Max || X + 2 * pad > kInt32Max)
        return fail(MP3D_EOVERFLOW, "window span or padded extent on %s exceeds int32", name);
    const int64_t ext = (k - 1) * dil + 1;
    if (2 * pad > k)
        return fail(MP3D_EINVAL, "padding %lld on %s exceeds half the kernel %lld",
                    (long long)pad, name, (long long)k);
    if (X + 2 * pad < ext)
        return fail(MP3D_EINVAL, "window span %lld exceeds the padded extent %lld on %s",
                    (long long)ext, (long long)(X + 2 * pad), name);
    return MP3D_OK;
}

// A fixed axis with padding and dilation whose output extent O is given:
// it must be the floor-mode or the ceil-mode extent.
int set_fixed_axis_ex(Axis *a, int64_t X, int32_t k, int32_t s, int32_t pad, int32_t dil,
                      int64_t O, const char *name)
{
    int rc = check_fixed_ex(X, k, s, pad, dil, name);
    if (rc) return rc;
    const int64_t lo = fixed_out_ex(X, k, s, pad, dil, false), hi = fixed_out_ex(X, k, s, pad, dil, true);
    if (O != lo && O != hi)
        return fail(MP3D_EINVAL, "output extent %lld on %s is neither %lld (floor) nor %lld (ceil)",
                    (long long)O, name, (long long)lo, (long long)hi);
    *a = Axis::make((int32_t)X, (int32_t)O, k, s, pad, dil);
    return MP3D_OK;
}

int set_adaptive_axis(Axis *a, int64_t X, int32_t O, const char *name)
{
    if (O <= 0)
        return fail(MP3D_EINVAL, "output extent on %s must be >= 1 (got %d)", name, O);
    *a = Axis::make((int32_t)X, O, 0, 0);
    return MP3D_OK;
}

int finish_geom(Geom *g, int64_t N, int64_t C)
{
    const int64_t out = (int64_t)g->ax[0].O * g->ax[1].O * g->ax[2].O;
    if ((int64_t)g->ax[0].O * g->ax[1].O > kInt32Max || out > kInt32Max)
        return fail(MP3D_EOVERFLOW, "OD*OH*OW exceeds the int32 range");
    g->planes = N * C;
    g->in_plane = g->ax[0].X * g->ax[1].X * g->ax[2].X;
    g->out_plane = (int32_t)out;
    if (g->planes > 0 && g->planes > ((int64_t)1 << 62) / out)
        return fail(MP3D_EOVERFLOW, "N*C*OD*OH*OW exceeds 2^62 elements");
    return MP3D_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return MP3D_OK;
    return fail(MP3D_EHIP, "%s: %s (hipError %d)", what, hipGetErrorString(e), (int)e);
}

template <typename T, typename IT>
int run_forward(const void *x, void *y, IT *idx, const Geom &g, hipStream_t s)
{
    FixedPlan fp;
    if (plan_fixed(g, (int)sizeof(typename T::raw), x, y, idx, &fp)) {
        if (log_enabled())
            fprintf(stderr, "[mp3d] forward fixed dtype=%d k=%d s=%d threads=%u vec_store=%d\n",
                    T::code, g.ax[0].k, g.ax[0].s, fp.nthreads, fp.vec_store);
        return hip_status(launch_forward_fixed<T, IT>(x, y, idx, fp, s), "forward fixed launch");
    }
    // tiny tensors: one thread per output, every load at once, no barrier
    // (latency, not bandwidth, is their cost)
    SmallPlan sp;
    const bool tiny = g.planes * (int64_t)g.in_plane <= kTinyInputs;
    const bool small = small_enabled() && plan_small_forward(g, &sp);
    ColPlan cp;
    if (!(tiny && small) && plan_col(g, (int)sizeof(typename T::raw), x, &cp)) {
        if (log_enabled())
            fprintf(stderr, "[mp3d] forward column dtype=%d tod=%d tiles=%u maxkd=%d lds=%u\n",
                    T::code, cp.tod, cp.ntiles, cp.maxkd, cp.lds_bytes);
        return hip_status(launch_forward_col<T, IT>(x, y, idx, cp, s), "forward column launch");
    }
    if (small) {
        if (log_enabled()) fprintf(stderr, "[mp3d] forward small dtype=%d outputs=%u\n", T::code, sp.total);
        return hip_status(launch_forward_small<T, IT>(x, y, idx, sp, s), "forward small launch");
    }
    FwdPlan p;
    if (plan_forward(g, (int)sizeof(typename T::raw), &p)) {
        if (log_enabled())
            fprintf(stderr, "[mp3d] forward tile dtype=%d tile=(%d,%d,%d) tiles=%lld lds=%u\n",
                    T::code, p.tod, p.toh, p.tow, (long long)p.ntiles, p.lds_bytes);
        return hip_status(launch_forward_tile<T, IT>(x, y, idx, p, s), "forward tile launch");
    }
    if (log_enabled()) fprintf(stderr, "[mp3d] forward direct dtype=%d\n", T::code);
    return hip_status(launch_forward_direct<T, IT>(x, y, idx, g, s), "forward direct launch");
}

template <typename T, typename IT>
int run_forward_ex(const void *x, void *y, IT *idx, const Geom &g, hipStream_t s)
{
    ExPlan p;
    plan_ex(g, &p);
    if (log_enabled())
        fprintf(stderr, "[mp3d] forward general dtype=%d idx=%d taps<=3:%d outputs=%lld\n", T::code,
                (int)sizeof(IT) * 8, p.km == 3, (long long)p.total);
    return hip_status(launch_forward_ex<T, IT>(x, y, idx, p, s), "forward general launch");
}

template <typename T, typename IT>
int forward_it(const void *x, void *y, IT *idx, const Geom &g, hipStream_t s)
{
    // dilated windows take the general kernel; padded and ceil-mode windows
    // of dilation 1 are clipped spans, which the column, tile, small and
    // direct kernels scan as they are.  float64: the general kernel for
    // windows of at most 3 taps per axis (all 27 loads issued at once;
    // measured slightly faster there), else the column kernel (binary64
    // partials) where it applies, else the general kernel.
    if constexpr (std::is_same<T, F64>::value) {
        ColPlan cp;
        if (g.contiguous() && !(max_taps(g.ax[0]) <= 3 && max_taps(g.ax[1]) <= 3 &&
                                max_taps(g.ax[2]) <= 3) &&
            plan_col(g, (int)sizeof(typename T::raw), x, &cp)) {
            if (log_enabled())
                fprintf(stderr, "[mp3d] forward column dtype=%d tod=%d tiles=%u maxkd=%d lds=%u\n",
                        T::code, cp.tod, cp.ntiles, cp.maxkd, cp.lds_bytes);
            return hip_status(launch_forward_col<T, IT>(x, y, idx, cp, s), "forward column launch");
        }
        return run_forward_ex<T, IT>(x, y, idx, g, s);
    } else {
        if (!g.contiguous()) return run_forward_ex<T, IT>(x, y, idx, g, s);
        return run_forward<T, IT>(x, y, idx, g, s);
    }
}

template <typename T>
int forward_t(const void *x, void *y, void *idx, int idx_type, const Geom &g, hipStream_t s)
{
    if (idx_type == MP3D_IDX_I64) return forward_it<T, int64_t>(x, y, (int64_t *)idx, g, s);
    return forward_it<T, int32_t>(x, y, (int32_t *)idx, g, s);
}

int forward(const void *x, void *y, void *idx, int idx_type, int dtype, const Geom &g,
            hipStream_t s)
{
    if (g.planes == 0) return MP3D_OK;
    if (!x || !y) return fail(MP3D_EINVAL, "null tensor pointer");   // idx NULL: values only
    switch (dtype) {
    case MP3D_F32: return forward_t<F32>(x, y, idx, idx_type, g, s);
    case MP3D_F16: return forward_t<F16>(x, y, idx, idx_type, g, s);
    case MP3D_F64: return forward_t<F64>(x, y, idx, idx_type, g, s);
    default: return forward_t<BF16>(x, y, idx, idx_type, g, s);
    }
}

enum class BwdPath { gather, accumulate, ordered };

template <typename S> struct is_array_src : std::false_type {};
template <typename IT> struct is_array_src<IdxArray<IT>> : std::true_type {};
template <typename S> struct is_recompute_src : std::false_type {};
template <typename T> struct is_recompute_src<IdxRecompute<T>> : std::true_type {};

// The gather and small-tensor kernels visit every window of each input
// element, so they take only index arrays; a recomputed or checked argmax
// goes to the slab / box kernels, which ask once per window.
template <typename T, typename Src>
int run_backward(const void *gy, const Src &src, void *gx, const Geom &g, BwdPath path,
                 hipStream_t s)
{
    if constexpr (is_array_src<Src>::value) {
        if (path == BwdPath::gather) {
            GatherPlan p;
            plan_gather(g, &p);
            if (log_enabled()) fprintf(stderr, "[mp3d] backward gather dtype=%d\n", T::code);
            return hip_status(launch_backward_gather<T, Src>(gy, src, gx, p, s),
                              "backward gather launch");
        }
        SmallPlan sp;
        if (small_enabled() && plan_small_backward(g, &sp)) {
            if (log_enabled())
                fprintf(stderr, "[mp3d] backward small dtype=%d inputs=%u\n", T::code, sp.total);
            return hip_status(launch_backward_small<T, Src>(gy, src, gx, sp, s),
                              "backward small launch");
        }
    }
    const bool ordered = path == BwdPath::ordered;
    if constexpr (is_array_src<Src>::value) {
        // The owner-gather slab gives the ascending-order fold, with no
        // atomics and no phases: the ordered path takes it wherever it
        // applies.  (As the accumulate path it measured slower than the
        // compare-and-swap slab on both large overlapping workloads: 104
        // against 94 us and 100 against 63 us.)
        OwnerPlan op;
        if (ordered && plan_owner(g, (int)sizeof(typename T::raw), &op)) {
            if (log_enabled())
                fprintf(stderr, "[mp3d] backward owner-gather dtype=%d slab=%d tiles=%lld "
                        "threads=%d lds=%u\n", T::code, op.td, (long long)op.ntiles,
                        op.threads, op.lds_bytes);
            return hip_status(launch_backward_owner<T, Src>(gy, src, gx, op, s),
                              "backward owner-gather launch");
        }
    }
    if constexpr (is_recompute_src<Src>::value) {
        // index-free, any order: the column stages recompute the argmax
        RcPlan rp;
        if (!ordered && plan_rc(g, (int)sizeof(typename T::raw), (int)sizeof(typename T::acc),
                                src.x, &rp)) {
            if (log_enabled())
                fprintf(stderr, "[mp3d] backward index-free column dtype=%d slab=%d tiles=%u lds=%u "
                        "slots=%d maxkd=%d small3=%d\n",
                        T::code, rp.td, rp.ntiles, rp.lds_bytes, rp.slots, rp.maxkd, rp.small3);
            return hip_status(launch_backward_rc<T>(src.x, src.y, gy, gx, rp, s),
                              "backward index-free launch");
        }
    }
    BwdPlan p;
    if (plan_backward(g, ordered, (int)sizeof(typename T::acc), &p)) {

        if (log_enabled())
            fprintf(stderr, "[mp3d] backward %s%s dtype=%d box=(%d,%d,%d) tiles=%lld lds=%u phases=%d\n",
                    ordered ? "ordered slab" : "accumulate",
                    is_array_src<Src>::value ? "" : is_recompute_src<Src>::value
                                                        ? " (argmax recomputed)"
                                                        : " (argmax checked)",
                    T::code, p.td, p.th,
                    p.tw, (long long)p.ntiles, p.lds_bytes, p.nphase);
        return hip_status(launch_backward_tile<T, Src>(gy, src, gx, p, s), "backward tile launch");
    }
    OrdPlan op;
    plan_ordered(g, &op);
    if (log_enabled()) fprintf(stderr, "[mp3d] backward ordered gather dtype=%d\n", T::code);
    return hip_status(launch_backward_ordered<T, Src>(gy, src, gx, op, s), "backward ordered launch");
}

template <typename T>
IdxRecompute<T> recompute_src(const void *x, const void *y, const Geom &g)
{
    IdxRecompute<T> r;
    r.x = (const typename T::raw *)x;
    r.y = (const typename T::raw *)y;
    r.g = g;
    r.fast32 = g.planes * (int64_t)g.out_plane < ((int64_t)1 << 31);
    ExPlan ep;                                   // its tap-count test
    plan_ex(g, &ep);
    r.km3 = ep.km == 3;
    r.w8 = max_taps(g.ax[2]) <= 8;
    r.plane_div = FastDiv((uint32_t)g.out_plane);
    r.ow_div = FastDiv((uint32_t)g.ax[2].O);
    r.oh_div = FastDiv((uint32_t)g.ax[1].O);
    return r;
}

template <typename T>
IdxChecked<T> checked_src(const void *x, const void *y, const void *yf, const int32_t *idxf,
                          const Geom &g)
{
    IdxChecked<T> r;
    r.idxf = idxf;
    r.yf = (const typename T::raw *)yf;
    r.x = (const typename T::raw *)x;
    r.y = (const typename T::raw *)y;
    r.g = g;
    r.ow_div = FastDiv((uint32_t)g.ax[2].O);
    r.oh_div = FastDiv((uint32_t)g.ax[1].O);
    return r;
}

// Workspace of the two-pass index-free backward: the forward's maximum
// (storage type) then its int32 argmax, each part starting on 256 bytes.
struct WsLayout {
    size_t y_bytes, bytes;
};

WsLayout ws_layout(int64_t outputs, int es)
{
    const size_t yb = ((size_t)outputs * (size_t)es + 255) & ~(size_t)255;
    return {yb, yb + (size_t)outputs * 4};
}

// Windows tile an axis -- each position in exactly one window, the one
// given by p / (X/O) -- for adaptive windows when O divides X, and for
// fixed windows when stride == X/O and kernel <= stride.
bool axis_tiles(const Axis &a)
{
    if (a.X % a.O != 0 || !a.plain()) return false;
    if (a.k == 0) return true;
    return a.s == a.X / a.O && a.k <= a.s;
}

// Axes of the padded / dilated entry points: kernel[a] == stride[a] == 0
// selects adaptive windows with extent O (padding 0 and dilation 1 there);
// otherwise fixed windows.  pad and dilation may be NULL (0 and 1).
int set_axes_ex(Geom *g, int64_t D, int64_t H, int64_t W, int32_t od, int32_t oh, int32_t ow,
                const int32_t *kernel, const int32_t *stride, const int32_t *pad,
                const int32_t *dilation)
{
    if (!kernel || !stride) return fail(MP3D_EINVAL, "kernel and stride arrays must not be NULL");
    const int64_t X[3] = {D, H, W};
    const int32_t O[3] = {od, oh, ow};
    const char *names[3] = {"D", "H", "W"};
    for (int a = 0; a < 3; ++a) {
        const int32_t pa = pad ? pad[a] : 0, dl = dilation ? dilation[a] : 1;
        int rc;
        if (kernel[a] == 0 && stride[a] == 0) {
            if (pa != 0 || dl != 1)
                return fail(MP3D_EINVAL, "adaptive axis %s takes padding 0 and dilation 1", names[a]);
            if ((rc = set_adaptive_axis(&g->ax[a], X[a], O[a], names[a]))) return rc;
        } else if ((rc = set_fixed_axis_ex(&g->ax[a], X[a], kernel[a], stride[a], pa, dl, O[a],
                                           names[a]))) {
            return rc;
        }
    }
    return MP3D_OK;
}

// Shared by the backward entry points.  idx_type < 0: no index array, the
// argmax is recomputed from x and y (x, y then required).
// A workspace (ws, with idx_type < 0) takes the two-pass index-free
// backward: the forward into the workspace, then the argmax checked
// against y.
int backward(const void *gy, const void *idx, int idx_type, const void *x, const void *y,
             void *gx, int dtype, Geom &g, int64_t N, int64_t C, int overlap, hipStream_t s,
             void *ws = nullptr, size_t ws_bytes = 0)
{
    int rc;
    if (overlap < -1 || overlap > 2)
        return fail(MP3D_EINVAL, "overlap must be -1, 0, 1 or 2 (got %d)", overlap);
    if ((rc = finish_geom(&g, N, C))) return rc;
    const bool tiles = axis_tiles(g.ax[0]) && axis_tiles(g.ax[1]) && axis_tiles(g.ax[2]);
    if (overlap == 0 && !tiles)
        return fail(MP3D_ENOTDIV, "overlap=0 needs windows that tile every axis");
    if (g.planes == 0) return MP3D_OK;
    if (!gy || !gx || (idx_type >= 0 ? !idx : (!x || !y)))
        return fail(MP3D_EINVAL, "null tensor pointer");
    // the gather is already the ordered sum (one window per input)
    const BwdPath path = overlap == 0 || ((overlap == -1 || overlap == 2) && tiles)
                             ? BwdPath::gather
                             : overlap == 2 ? BwdPath::ordered : BwdPath::accumulate;
    if (idx_type < 0) {
        // with windows that tile, every input has at most one contribution:
        // the accumulate path gives the gather's (and the ordered) result
        const BwdPath rp = path == BwdPath::ordered ? BwdPath::ordered : BwdPath::accumulate;
        const int es = dtype == MP3D_F64 ? 8 : dtype == MP3D_F32 ? 4 : 2;
        const WsLayout L = ws_layout(g.planes * (int64_t)g.out_plane, es);
        if (ws && ws_bytes < L.bytes)
            return fail(MP3D_EWORKSPACE, "workspace of %zu bytes; this call needs %zu", ws_bytes,
                        L.bytes);
        if (ws && (uintptr_t)ws % 16)
            return fail(MP3D_EWORKSPACE, "workspace must be 16-byte aligned");
        // the two-pass form, except for small tensors (one launch instead
        // of two) and where the fused one-pass kernel takes slabs of 4
        // slices or more (there it measured as fast or faster: each window
        // is recomputed by few slabs)
        RcPlan rcp;
        const bool small = g.planes * (int64_t)g.in_plane < ((int64_t)1 << 22);
        const bool fused_wide = rp != BwdPath::ordered &&
                                plan_rc(g, es, es == 8 ? 8 : 4, x, &rcp) && rcp.td >= 4;
        if (ws && (two_pass_forced() || (!small && !fused_wide))) {
            if (log_enabled()) fprintf(stderr, "[mp3d] index-free backward: two passes\n");
            void *yf = ws;
            int32_t *idxf = (int32_t *)((char *)ws + L.y_bytes);
            if ((rc = forward(x, yf, idxf, MP3D_IDX_I32, dtype, g, s))) return rc;
            switch (dtype) {
            case MP3D_F32: return run_backward<F32>(gy, checked_src<F32>(x, y, yf, idxf, g), gx, g, rp, s);
            case MP3D_F16: return run_backward<F16>(gy, checked_src<F16>(x, y, yf, idxf, g), gx, g, rp, s);
            case MP3D_F64: return run_backward<F64>(gy, checked_src<F64>(x, y, yf, idxf, g), gx, g, rp, s);
            default: return run_backward<BF16>(gy, checked_src<BF16>(x, y, yf, idxf, g), gx, g, rp, s);
            }
        }
        switch (dtype) {
        case MP3D_F32: return run_backward<F32>(gy, recompute_src<F32>(x, y, g), gx, g, rp, s);
        case MP3D_F16: return run_backward<F16>(gy, recompute_src<F16>(x, y, g), gx, g, rp, s);
        case MP3D_F64: return run_backward<F64>(gy, recompute_src<F64>(x, y, g), gx, g, rp, s);
        default: return run_backward<BF16>(gy, recompute_src<BF16>(x, y, g), gx, g, rp, s);
        }
    }
    if (idx_type == MP3D_IDX_I64) {
        const IdxArray<int64_t> ix{(const int64_t *)idx};
        switch (dtype) {
        case MP3D_F32: return run_backward<F32>(gy, ix, gx, g, path, s);
        case MP3D_F16: return run_backward<F16>(gy, ix, gx, g, path, s);
        case MP3D_F64: return run_backward<F64>(gy, ix, gx, g, path, s);
        default: return run_backward<BF16>(gy, ix, gx, g, path, s);
        }
    }
    const IdxArray<int32_t> ix{(const int32_t *)idx};
    switch (dtype) {
    case MP3D_F32: return run_backward<F32>(gy, ix, gx, g, path, s);
    case MP3D_F16: return run_backward<F16>(gy, ix, gx, g, path, s);
    case MP3D_F64: return run_backward<F64>(gy, ix, gx, g, path, s);
    default: return run_backward<BF16>(gy, ix, gx, g, path, s);
    }
}

// Scratch of mp3d_backward_recompute_static: the two-pass index-free
// backward's workspace in device memory of the library's own, for callers
// that cannot allocate.  Each device holds its own copy until the process
// ends.  In host code the array's name is only a stand-in: its device
// address, per device, comes from hipGetSymbolAddress (scratch_address).
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The current device's address of `scratch`, looked up once per device
// with that device current; nullptr (and the message set) on failure.
void *scratch_address()
{
    static std::mutex mu;
    static void *cache[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        hip_status(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= 64) {
        fail(MP3D_EHIP, "device %d beyond the 64 the scratch table holds", dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        cache[dev] = ptr;
    }
    return cache[dev];
}

}  // namespace

LaunchTiming &launch_timing() { return g_timing; }

int device_cus()
{
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cache[dev] = v;
    }
    return cache[dev];
}

size_t lds_limit()
{
    static std::mutex mu;
    static size_t cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        cache[dev] = (size_t)v;
    }
    return cache[dev];
}

}  // namespace mp3d

using namespace mp3d;

extern "C" {

int mp3d_out_size(int64_t X, int32_t k, int32_t s, int64_t *out)
{
    if (!out) return fail(MP3D_EINVAL, "out is NULL");
    if (k <= 0 || s <= 0) return fail(MP3D_EINVAL, "kernel and stride must be >= 1");
    if (X < k) return fail(MP3D_EINVAL, "kernel %d exceeds extent %lld", k, (long long)X);
    *out = (X - k) / s + 1;
    return MP3D_OK;
}

int mp3d_out_size_ex(int64_t X, int32_t k, int32_t s, int32_t pad, int32_t dilation, int ceil_mode,
                     int64_t *out)
{
    if (!out) return fail(MP3D_EINVAL, "out is NULL");
    if (ceil_mode != 0 && ceil_mode != 1) return fail(MP3D_EINVAL, "ceil_mode must be 0 or 1");
    if (X <= 0 || X > kInt32Max) return fail(MP3D_EINVAL, "extent %lld out of range", (long long)X);
    int rc = check_fixed_ex(X, k, s, pad, dilation, "the axis");
    if (rc) return rc;
    *out = fixed_out_ex(X, k, s, pad, dilation, ceil_mode == 1);
    return MP3D_OK;
}

int mp3d_forward(const void *x, void *y, int32_t *idx, int dtype, int64_t N, int64_t C,
                 int64_t D, int64_t H, int64_t W, int32_t kd, int32_t kh, int32_t kw,
                 int32_t sd, int32_t sh, int32_t sw, void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    Geom g;
    if ((rc = set_fixed_axis(&g.ax[0], D, kd, sd, "D"))) return rc;
    if ((rc = set_fixed_axis(&g.ax[1], H, kh, sh, "H"))) return rc;
    if ((rc = set_fixed_axis(&g.ax[2], W, kw, sw, "W"))) return rc;
    if ((rc = finish_geom(&g, N, C))) return rc;
    return forward(x, y, idx, MP3D_IDX_I32, dtype, g, (hipStream_t)stream);
}

int amp3d_forward(const void *x, void *y, int32_t *idx, int dtype, int64_t N, int64_t C,
                  int64_t D, int64_t H, int64_t W, int32_t od, int32_t oh, int32_t ow,
                  void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    Geom g;
    if ((rc = set_adaptive_axis(&g.ax[0], D, od, "D"))) return rc;
    if ((rc = set_adaptive_axis(&g.ax[1], H, oh, "H"))) return rc;
    if ((rc = set_adaptive_axis(&g.ax[2], W, ow, "W"))) return rc;
    if ((rc = finish_geom(&g, N, C))) return rc;
    return forward(x, y, idx, MP3D_IDX_I32, dtype, g, (hipStream_t)stream);
}

int mp3d_forward_ex(const void *x, void *y, void *idx, int dtype, int idx_type, int64_t N,
                    int64_t C, int64_t D, int64_t H, int64_t W, int32_t od, int32_t oh,
                    int32_t ow, const int32_t *kernel, const int32_t *stride, const int32_t *pad,
                    const int32_t *dilation, void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    if (idx_type != MP3D_IDX_I32 && idx_type != MP3D_IDX_I64)
        return fail(MP3D_EDTYPE, "idx_type %d is not MP3D_IDX_I32 or MP3D_IDX_I64", idx_type);
    Geom g;
    if ((rc = set_axes_ex(&g, D, H, W, od, oh, ow, kernel, stride, pad, dilation))) return rc;
    if ((rc = finish_geom(&g, N, C))) return rc;
    return forward(x, y, idx, idx_type, dtype, g, (hipStream_t)stream);
}

int mp3d_backward(const void *gy, const int32_t *idx, void *gx, int dtype, int64_t N,
                  int64_t C, int64_t D, int64_t H, int64_t W, int32_t od, int32_t oh,
                  int32_t ow, int32_t kd, int32_t kh, int32_t kw, int32_t sd, int32_t sh,
                  int32_t sw, int overlap, void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    const int64_t X[3] = {D, H, W};
    const int32_t O[3] = {od, oh, ow}, K[3] = {kd, kh, kw}, S[3] = {sd, sh, sw};
    const char *names[3] = {"D", "H", "W"};
    Geom g;
    for (int a = 0; a < 3; ++a) {
        if (K[a] == 0 && S[a] == 0) {
            if ((rc = set_adaptive_axis(&g.ax[a], X[a], O[a], names[a]))) return rc;
        } else {
            if ((rc = set_fixed_axis(&g.ax[a], X[a], K[a], S[a], names[a]))) return rc;
            if (g.ax[a].O != O[a])
                return fail(MP3D_EINVAL,
                            "output extent %d on %s does not match (X-k)/s+1 = %d", O[a],
                            names[a], g.ax[a].O);
        }
    }
    return backward(gy, idx, MP3D_IDX_I32, nullptr, nullptr, gx, dtype, g, N, C, overlap,
                    (hipStream_t)stream);
}

int mp3d_backward_ex(const void *gy, const void *idx, void *gx, int dtype, int idx_type,
                     int64_t N, int64_t C, int64_t D, int64_t H, int64_t W, int32_t od,
                     int32_t oh, int32_t ow, const int32_t *kernel, const int32_t *stride,
                     const int32_t *pad, const int32_t *dilation, int overlap, void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    if (idx_type != MP3D_IDX_I32 && idx_type != MP3D_IDX_I64)
        return fail(MP3D_EDTYPE, "idx_type %d is not MP3D_IDX_I32 or MP3D_IDX_I64", idx_type);
    Geom g;
    if ((rc = set_axes_ex(&g, D, H, W, od, oh, ow, kernel, stride, pad, dilation))) return rc;
    return backward(gy, idx, idx_type, nullptr, nullptr, gx, dtype, g, N, C, overlap,
                    (hipStream_t)stream);
}

int mp3d_backward_recompute(const void *x, const void *y, const void *gy, void *gx, int dtype,
                            int64_t N, int64_t C, int64_t D, int64_t H, int64_t W, int32_t od,
                            int32_t oh, int32_t ow, const int32_t *kernel, const int32_t *stride,
                            const int32_t *pad, const int32_t *dilation, int overlap,
                            void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    Geom g;
    if ((rc = set_axes_ex(&g, D, H, W, od, oh, ow, kernel, stride, pad, dilation))) return rc;
    return backward(gy, nullptr, -1, x, y, gx, dtype, g, N, C, overlap, (hipStream_t)stream);
}

int mp3d_recompute_workspace_size(int dtype, int64_t N, int64_t C, int32_t od, int32_t oh,
                                  int32_t ow, size_t *bytes)
{
    if (!bytes) return fail(MP3D_EINVAL, "bytes is NULL");
    if (dtype < MP3D_F32 || dtype > MP3D_F64)
        return fail(MP3D_EDTYPE, "dtype %d is not one of MP3D_F32/F16/BF16/F64", dtype);
    if (N < 0 || C < 0 || od <= 0 || oh <= 0 || ow <= 0)
        return fail(MP3D_EINVAL, "N, C must be >= 0 and the output extents >= 1");
    const int64_t per = (int64_t)od * oh * ow;
    if (per > kInt32Max || (N && C && (N > INT64_MAX / C || N * C > (INT64_MAX / 16) / per)))
        return fail(MP3D_EOVERFLOW, "output size out of range");
    const int es = dtype == MP3D_F64 ? 8 : dtype == MP3D_F32 ? 4 : 2;
    *bytes = ws_layout(N * C * per, es).bytes;
    return MP3D_OK;
}

int mp3d_backward_recompute_ws(const void *x, const void *y, const void *gy, void *gx, int dtype,
                               int64_t N, int64_t C, int64_t D, int64_t H, int64_t W, int32_t od,
                               int32_t oh, int32_t ow, const int32_t *kernel,
                               const int32_t *stride, const int32_t *pad,
                               const int32_t *dilation, int overlap, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    Geom g;
    if ((rc = set_axes_ex(&g, D, H, W, od, oh, ow, kernel, stride, pad, dilation))) return rc;
    return backward(gy, nullptr, -1, x, y, gx, dtype, g, N, C, overlap, (hipStream_t)stream,
                    workspace, workspace_bytes);
}


int mp3d_backward_recompute_static(const void *x, const void *y, const void *gy, void *gx,
                                   int dtype, int64_t N, int64_t C, int64_t D, int64_t H,
                                   int64_t W, int32_t od, int32_t oh, int32_t ow,
                                   const int32_t *kernel, const int32_t *stride,
                                   const int32_t *pad, const int32_t *dilation, int overlap,
                                   void *stream)
{
    TimingScope timing_scope;
    int rc = check_common(dtype, N, C, D, H, W);
    if (rc) return rc;
    Geom g;
    if ((rc = set_axes_ex(&g, D, H, W, od, oh, ow, kernel, stride, pad, dilation))) return rc;
    size_t need = 0;
    if ((rc = mp3d_recompute_workspace_size(dtype, N, C, od, oh, ow, &need))) return rc;
    if (need > kScratchBytes)
        return fail(MP3D_EWORKSPACE, "this call needs %zu bytes of workspace; the library's "
                    "static scratch holds %zu (use mp3d_backward_recompute_ws)", need,
                    kScratchBytes);
    void *ws = nullptr;
    if (N * C > 0 && !(ws = scratch_address())) return MP3D_EHIP;
    return backward(gy, nullptr, -1, x, y, gx, dtype, g, N, C, overlap, (hipStream_t)stream,
                    ws, kScratchBytes);
}

int mp3d_time_next_call(void *start_event, void *stop_event)
{
    if (!stop_event && start_event) return fail(MP3D_EINVAL, "start event without a stop event");
    g_timing = {(hipEvent_t)start_event, (hipEvent_t)stop_event};
    return MP3D_OK;
}

int mp3d_backward_workspace_bytes(int dtype, int idx_type, int64_t N, int64_t C, int32_t od,
                                  int32_t oh, int32_t ow, size_t *bytes)
{
    if (!bytes) return fail(MP3D_EINVAL, "bytes is NULL");
    if (idx_type != MP3D_IDX_I32 && idx_type != MP3D_IDX_I64 && idx_type != MP3D_IDX_NONE)
        return fail(MP3D_EDTYPE, "idx_type %d is not MP3D_IDX_I32, MP3D_IDX_I64 or MP3D_IDX_NONE",
                    idx_type);
    if (idx_type == MP3D_IDX_NONE) return mp3d_recompute_workspace_size(dtype, N, C, od, oh, ow, bytes);
    if (dtype < MP3D_F32 || dtype > MP3D_F64)
        return fail(MP3D_EDTYPE, "dtype %d is not one of MP3D_F32/F16/BF16/F64", dtype);
    if (N < 0 || C < 0 || od <= 0 || oh <= 0 || ow <= 0)
        return fail(MP3D_EINVAL, "N, C must be >= 0 and the output extents >= 1");
    *bytes = 0;                      // every index-array path keeps its accumulator in LDS
    return MP3D_OK;
}

const char *mp3d_strerror(int code)
{
    switch (code) {
    case MP3D_OK: return "success";
    case MP3D_EINVAL: return "invalid argument";
    case MP3D_EDTYPE: return "unsupported dtype";
    case MP3D_ENOTDIV: return "windows do not tile every axis";
    case MP3D_EOVERFLOW: return "size exceeds the index range";
    case MP3D_EHIP: return "HIP runtime error";
    case MP3D_EWORKSPACE: return "workspace too small or misaligned";
    default: return "unknown status";
    }
}

const char *mp3d_last_error(void) { return g_msg; }

}  // extern "C"
