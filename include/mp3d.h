/*
 * mp3d.h -- C ABI of libmp3d: 3-D max pooling over NCDHW tensors on AMD
 * Instinct MI355X (gfx950).
 *
 * Operations:
 *  - forward, fixed windows: "Struct Maxpool3dForward" (teenygrad API docs),
 *    the description under the struct: one output per window, no padding,
 *    and per axis O = (X - K) / STRIDE + 1 with integer division.  Window o
 *    covers [o*STRIDE, o*STRIDE + K).
 *  - forward, adaptive windows, and the backward: "[KernelGen][MThreads]
 *    Add adaptive_max_pool3d_backward Moore Threads specialized operator"
 *    (FlagGems-Experimental PR #308), Summary.  The backward sends each
 *    output window's gradient to the input position of that window's
 *    argmax.  When every spatial axis divides evenly the windows tile the
 *    input and each input is reached by at most one window (a gather with a
 *    single write per input); otherwise windows overlap and contributions
 *    add (a zero-filled accumulator plus an atomic scatter).  The page
 *    prints no window formula; this library takes window o of O over an
 *    axis of length X to cover [floor(o*X/O), ceil((o+1)*X/O)).
 *
 * Semantics fixed here where the pages are silent:
 *  - A window is scanned d, then h, then w, ascending.  The argmax is the
 *    first element in that order that is not smaller than any other: ties
 *    go to the earlier element, -0 and +0 tie, and NaN counts as larger
 *    than every number (the first NaN wins).  y holds that element's bits.
 *  - idx is int32, flat within one plane: (d*H + h)*W + w.
 *  - The backward accumulates in binary32 from +0 and rounds the sum once,
 *    to nearest-even, into the storage type (float64: in binary64, no
 *    rounding).
 *
 * Layout and ownership: every tensor is contiguous NCDHW in device memory
 * owned by the caller; the library never allocates or frees.  x and gx
 * hold N*C*D*H*W elements; y, idx and gy hold N*C*OD*OH*OW.  Outputs must
 * not alias inputs, and each pointer is aligned to its element size.
 * dtype selects the storage type of x, y, gy and gx
 * (MP3D_F32, MP3D_F16, MP3D_BF16, MP3D_F64); idx is int32 (int64 through
 * the _ex entry points).
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Calls enqueue their kernels and return without synchronising;
 * device faults surface at the caller's next synchronisation.  A call only
 * launches kernels on `stream` (no allocation, memset or synchronisation),
 * so calls can be recorded under stream capture into a HIP graph and
 * replayed.
 *
 * Errors: every call returns MP3D_OK (0) or an error code.  All argument
 * checks run before the first launch, so a call that fails leaves every
 * output untouched.  mp3d_last_error() gives a message for the calling
 * thread's most recent failure.  N*C == 0 is a valid no-op.
 */
#ifndef MP3D_H
#define MP3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mp3d_status {
    MP3D_OK = 0,
    MP3D_EINVAL = 1,    /* null pointer with work to do, a size, kernel,
                           stride or output extent <= 0, a window larger
                           than its axis, or inconsistent shapes */
    MP3D_EDTYPE = 2,    /* dtype is not one of MP3D_F32/F16/BF16/F64, or idx_type
                           not one of MP3D_IDX_I32/I64 */
    MP3D_ENOTDIV = 3,   /* overlap = 0 asked for, but the windows do not
                           tile every axis (see mp3d_backward) */
    MP3D_EOVERFLOW = 4, /* D*H*W > INT32_MAX (int32 idx impossible) or an
                           element count beyond 2^62 */
    MP3D_EHIP = 5,      /* a HIP launch failed; the message names it */
    MP3D_EWORKSPACE = 6 /* a workspace smaller than its size query, or not
                           16-byte aligned */
};

/* Storage types.  float16 and bfloat16 values are compared and gradients
 * accumulated in binary32; float64 in binary64 (PR #308 page, Testing:
 * that implementation leaves float64 to a generic fallback; here it is a
 * dtype of its own, served by the general kernels). */
enum mp3d_dtype { MP3D_F32 = 0, MP3D_F16 = 1, MP3D_BF16 = 2, MP3D_F64 = 3 };

/* Index element type of the _ex entry points (the others use int32).
 * MP3D_IDX_NONE names the index-free backward in the workspace query. */
enum mp3d_index { MP3D_IDX_NONE = -1, MP3D_IDX_I32 = 0, MP3D_IDX_I64 = 1 };

/* Forward with fixed windows (teenygrad "Struct Maxpool3dForward",
 * description): kernel (kd, kh, kw), stride (sd, sh, sw), no padding.
 * Output extents are (D-kd)/sd+1, (H-kh)/sh+1, (W-kw)/sw+1; the caller
 * sizes y and idx from mp3d_out_size.  Writes y (dtype) and idx (int32).
 * idx may be NULL: then only y is written (values-only forward, for callers
 * that need no backward; y is the same as with idx).  MP3D_EINVAL if x or
 * y is NULL with work to do, any kernel or stride is <= 0 or a kernel
 * exceeds its axis. */
int mp3d_forward(const void *x, void *y, int32_t *idx, int dtype,
                 int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                 int32_t kd, int32_t kh, int32_t kw,
                 int32_t sd, int32_t sh, int32_t sw, void *stream);

/* Forward with adaptive windows (PR #308, Summary): output extents
 * (od, oh, ow), each >= 1 (an extent larger than its axis is allowed; the
 * windows then have width 1 or 2 and overlap).  Writes y and idx; idx may
 * be NULL, as for mp3d_forward. */
int amp3d_forward(const void *x, void *y, int32_t *idx, int dtype,
                  int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                  int32_t od, int32_t oh, int32_t ow, void *stream);

/* Backward (PR #308, Summary): gx[p] = sum of gy[o] over the outputs o
 * whose idx[o] == p, in binary32 from +0, rounded once to dtype (float64:
 * binary64); +0 where no output points.  Every element of gx is written.
 *
 * (N, C, D, H, W) is the input shape; (od, oh, ow) the shape of gy and
 * idx.  The window rule is given per axis so that the library knows which
 * windows can reach a block of gx: kd/kh/kw and sd/sh/sw > 0 select fixed
 * windows on that axis (od must then equal (D-kd)/sd+1, and so on); a
 * kernel and stride of 0 select adaptive windows on that axis.
 *
 * overlap selects the path:
 *   0  gather: one pass over gx, no accumulator, no atomics.  Valid only
 *      when the windows tile every axis: X % O == 0 and, for fixed windows,
 *      stride == X / O and kernel <= stride.  Otherwise MP3D_ENOTDIV.
 *   1  accumulate: zero-filled binary32 accumulator, atomic scatter of gy
 *      at idx, one rounding store.  Valid for every geometry.  The order
 *      of the additions into one element is not fixed, so an element
 *      reached by three or more outputs may differ in its last bits from
 *      run to run.  Small tensors (at most 2^20 input elements, each in at
 *      most two windows per axis) take an ordered gather instead: the same
 *      sums, added in ascending output order, with no accumulator.
 *   2  ordered: every element is the binary32 sum of its contributions in
 *      ascending output order, from +0, rounded once -- the same bits on
 *      every run.  Valid for every geometry: the gather when the windows
 *      tile, else the ordered gather for small tensors, else slabs whose
 *      contributions are added rank by rank (no atomics), else the ordered
 *      gather at any size (slower: loads one after another).
 *  -1  choose: 0 when valid, else 1.
 * Each idx[o] must lie inside window o, as the forward produces it; idx
 * values outside [0, D*H*W) are ignored (never written, never a fault),
 * and in-range values outside their window give unspecified but
 * memory-safe results. */
int mp3d_backward(const void *gy, const int32_t *idx, void *gx, int dtype,
                  int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                  int32_t od, int32_t oh, int32_t ow,
                  int32_t kd, int32_t kh, int32_t kw,
                  int32_t sd, int32_t sh, int32_t sw,
                  int overlap, void *stream);

/* Fixed-window output extent (X - k)/s + 1 into *out.  MP3D_EINVAL if
 * k <= 0, s <= 0, X < k or out is NULL. */
int mp3d_out_size(int64_t X, int32_t k, int32_t s, int64_t *out);

/* --- Padding, dilation, ceil mode and int64 indices ------------------
 *
 * The pages define fixed windows without padding ("Struct
 * Maxpool3dForward", teenygrad, description).  These entry points widen
 * that surface; the reading taken where the pages are silent: window o on
 * an axis takes the k taps o*s - pad + j*dil (0 <= j < k), which span
 * (k-1)*dil + 1 positions (the effective kernel of the FlagGems
 * conv_transpose2d PR page, Implementation); a tap outside the axis is
 * padding and is never taken.  y is still the first maximum in d, h, w
 * scan order (NaN first) and idx its flat plane position.  A window whose
 * taps all fall in the padding (only possible when the dilation steps over
 * the whole axis) gives y = -inf and idx = -1.
 *
 * Per axis: kernel k >= 1, stride s >= 1, pad >= 0, dilation >= 1,
 * 2*pad <= k (as torch requires), and the span must fit the padded axis:
 * X + 2*pad >= (k-1)*dil + 1.  Otherwise MP3D_EINVAL. */

/* Index-free backward: the same sums as mp3d_backward_ex, with each
 * window's argmax recomputed from the forward's input x and output y
 * instead of read from an index array, so that a caller can run the
 * values-only forward (idx = NULL) and keep no index at all (the teenygrad
 * kernel ABI passes no index buffer, "Struct Maxpool3dForward", Kernel
 * trait; its backward receives the forward's inputs and output,
 * RuntimeOp).  The argmax of window o is its first tap, in d, h, w scan
 * order, whose element equals y[o] (the first NaN when y[o] is NaN): the
 * forward's own argmax whenever y is what the forward wrote.  A window with
 * no such tap contributes nothing.  x: (N, C, D, H, W); y and gy:
 * (N, C, od, oh, ow); geometry arrays and overlap as for mp3d_backward_ex
 * (overlap 0 and -1 take the accumulate kernels, which give the gather's
 * result on tiling windows).  Reads x once per window that reaches a slab
 * of gx: slower than the index path, and no index traffic. */
int mp3d_backward_recompute(const void *x, const void *y, const void *gy, void *gx, int dtype,
                            int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                            int32_t od, int32_t oh, int32_t ow,
                            const int32_t *kernel, const int32_t *stride,
                            const int32_t *pad, const int32_t *dilation,
                            int overlap, void *stream);

/* Bytes of workspace mp3d_backward_recompute_ws needs for N*C planes of
 * od*oh*ow outputs of dtype: the forward's maximum in the storage type,
 * rounded up to 256 bytes, then its int32 argmax.  Into *bytes. */
int mp3d_recompute_workspace_size(int dtype, int64_t N, int64_t C, int32_t od, int32_t oh,
                                  int32_t ow, size_t *bytes);

/* The index-free backward of mp3d_backward_recompute (same arguments, same
 * result bit for bit in the ordered mode and within the same bounds
 * otherwise) in two passes through a caller's device workspace: the
 * forward runs on x into the workspace (its maximum yf and argmax), then
 * the backward takes the argmax of window o from there wherever y[o]
 * equals yf[o] (both NaN, or equal as numbers: then every tap equal to
 * y[o] is a maximum of the window and the first of them is the forward's
 * argmax) and scans window o of x where it does not.  For callers who can
 * lend transient device memory (a fraction of x: yf and an int32 per
 * output) but keep no index between forward and backward; faster than
 * the one-pass form where windows overlap and slabs of gx are thin.
 * workspace: device memory of workspace_bytes >=
 * mp3d_recompute_workspace_size(...), 16-byte aligned (else MP3D_EINVAL),
 * overlapping none of x, y, gy, gx;
 * its contents on entry do not matter and are overwritten; the caller
 * owns it and may reuse it once the stream has passed this call.
 * workspace NULL: the one-pass mp3d_backward_recompute.  A smaller
 * workspace_bytes: MP3D_EINVAL.  The one-pass form still runs, and the
 * workspace stays untouched, where it measured as fast: tensors under 2^22
 * elements, and geometries whose one-pass slabs hold 4 or more slices of
 * gx (environment MP3D_TWO_PASS=1 takes two passes regardless). */
int mp3d_backward_recompute_ws(const void *x, const void *y, const void *gy, void *gx, int dtype,
                               int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                               int32_t od, int32_t oh, int32_t ow,
                               const int32_t *kernel, const int32_t *stride,
                               const int32_t *pad, const int32_t *dilation,
                               int overlap, void *workspace, size_t workspace_bytes,
                               void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * two-pass index-free backward of mp3d_backward_recompute_ws, same
 * arguments and same results, with the workspace taken from a static
 * device array of the library (128 MiB; each GPU the library runs on holds
 * its own copy until the process ends) instead of from the caller.  No
 * allocation and no free happen in this call.  A call whose workspace
 * (mp3d_recompute_workspace_size) exceeds 128 MiB fails with
 * MP3D_EWORKSPACE before any launch.  Every call on one GPU shares that
 * GPU's array: calls that may overlap in time on one GPU (several streams,
 * several host threads) race on it and must be serialised by the caller.
 * Nothing in the array needs to start at any value: the forward pass
 * writes all of it that the backward pass reads. */
int mp3d_backward_recompute_static(const void *x, const void *y, const void *gy, void *gx,
                                   int dtype, int64_t N, int64_t C, int64_t D, int64_t H,
                                   int64_t W, int32_t od, int32_t oh, int32_t ow,
                                   const int32_t *kernel, const int32_t *stride,
                                   const int32_t *pad, const int32_t *dilation, int overlap,
                                   void *stream);

/* Output extent into *out.  ceil_mode 0: (X + 2*pad - span)/s + 1, rounded
 * down.  ceil_mode 1: rounded up, less one if that last window would start
 * at or beyond X + pad (so every window starts inside the input or the
 * left padding). */
int mp3d_out_size_ex(int64_t X, int32_t k, int32_t s, int32_t pad, int32_t dilation,
                     int ceil_mode, int64_t *out);

/* Forward with padding and dilation (kernel, stride, pad and dilation are
 * arrays of 3, d/h/w; pad and dilation may be NULL for 0 and 1).  An axis
 * with kernel = stride = 0 uses adaptive windows (as amp3d_forward) with
 * padding 0 and dilation 1.  (od, oh, ow) are the output extents: on a
 * fixed axis each must be the floor-mode or the ceil-mode extent of
 * mp3d_out_size_ex, and that choice is the ceil mode.  idx_type selects
 * int32 or int64 idx; idx may be NULL (values only).  With no padding,
 * dilation 1 and int32 idx the result is that of mp3d_forward /
 * amp3d_forward, by the same kernels. */
int mp3d_forward_ex(const void *x, void *y, void *idx, int dtype, int idx_type,
                    int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                    int32_t od, int32_t oh, int32_t ow,
                    const int32_t *kernel, const int32_t *stride,
                    const int32_t *pad, const int32_t *dilation, void *stream);

/* Backward for the geometries of mp3d_forward_ex: the same sums as
 * mp3d_backward (the result depends only on gy and idx; the window rule
 * tells the library which windows can reach a block of gx), with idx of
 * idx_type.  int64 idx values outside the plane are ignored.  overlap as
 * for mp3d_backward; overlap 0 needs no padding, dilation 1 and tiling
 * windows.  The ordered path (overlap 2) adds rank by rank only for
 * contiguous windows (dilation 1) and otherwise takes the ordered
 * gather. */
int mp3d_backward_ex(const void *gy, const void *idx, void *gx, int dtype, int idx_type,
                     int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                     int32_t od, int32_t oh, int32_t ow,
                     const int32_t *kernel, const int32_t *stride,
                     const int32_t *pad, const int32_t *dilation,
                     int overlap, void *stream);

/* Workspace bytes a backward needs for N*C planes of od*oh*ow outputs of
 * dtype, into *bytes: 0 for every backward that reads an index array
 * (idx_type MP3D_IDX_I32 or MP3D_IDX_I64: their accumulators, tables and
 * staged slabs live in LDS, so mp3d_backward and mp3d_backward_ex take no
 * workspace), and for the index-free backward (MP3D_IDX_NONE) the size of
 * mp3d_recompute_workspace_size, the workspace its two-pass form takes.
 * MP3D_EDTYPE for another dtype or idx_type, MP3D_EINVAL for negative N or
 * C, an output extent < 1 or a NULL bytes.  Host arithmetic only. */
int mp3d_backward_workspace_bytes(int dtype, int idx_type, int64_t N, int64_t C, int32_t od,
                                  int32_t oh, int32_t ow, size_t *bytes);

/* Kernel timing of the next call (a measurement aid, for benchmarks).  The
 * next call on the calling thread that launches kernels records
 * start_event when its first kernel starts and stop_event when its last
 * kernel ends (hipExtLaunchKernel's kernel-time events), so that
 * hipEventElapsedTime(start_event, stop_event) gives that call's kernel
 * time without the overhead of separate event records around it.  The
 * events are the caller's (hipEvent_t from hipEventCreate, passed as
 * void*).  Only the next call is timed: every launching call disarms the
 * events when it returns, whether or not it launched anything (a call that
 * launches nothing records neither event).  stop_event NULL disarms;
 * start_event without stop_event is MP3D_EINVAL. */
int mp3d_time_next_call(void *start_event, void *stop_event);

/* Text for a status code (static storage). */
const char *mp3d_strerror(int code);

/* Message for the calling thread's most recent failed call ("" if none). */
const char *mp3d_last_error(void);

/* Environment (read by the library, never required):
 *   MP3D_LOG=1    print the kernel path chosen for each call to stderr.
 *   MP3D_SMALL=0  never use the small-tensor kernels (for testing the
 *                 general kernels on small inputs; read on every call). */

#ifdef __cplusplus
}
#endif

#endif /* MP3D_H */
