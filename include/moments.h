/*
 * moments.h - C ABI of the MI355X (gfx950) physical-frame state-moments library.
 *
 * The operation (burn-mamba "recalculated.rs" source page, moments_phys_fwd and
 * the Mamba3MomentsBackendExt trait; "backward.rs" source page, module doc
 * "Gradient math" and moments_phys_bwd):
 *
 *   per (b,h) chain, with V = min(valid_len, s), decays da <= 0 typical,
 *     h~[t] = exp(da_t) h~[t-1] + sum_c xhat[t,c] (outer) bhat[t,c],  h~[-1] = h0
 *   computed chunkwise: a = inclusive cumsum of da inside a chunk,
 *     h~[t] = exp(a_t) h_- + sum_{j<=t,c} exp(a_t - a_j) xhat[j,c] (outer) bhat[j,c]
 *   then de-rotated along the state-rank axis, c_t = M_t h~[t] row by row:
 *     complex pairwise : pairs (2i, 2i+1), i < rope_dim/2, angle rot[b,t,h,i],
 *                        (x, y) -> (cos x + sin y, -sin x + cos y)     (R(-theta))
 *     complex half     : pairs (i, r/2 + i), same 2x2 block
 *     quaternion       : 4-blocks 4j..4j+3, j < quat_blocks, left Hamilton
 *                        product by Q = rot[b,t,h,j,:] = (w,x,y,z)
 *     coordinates outside the rotated width pass through unchanged;
 *   and the masked moments over t < V (V per sequence with desc->valid_lens):
 *     m2[b,h]     = sum_t c_t^T c_t                       ([r, r])
 *     m1[b,h,p,:] = sum_t c_t[p, :]                       ([p, r], per state row)
 *   The pages' pooled first moment m1[b,h,r] is m1.sum over p; its cotangent is
 *   d_m1 broadcast over p.
 *
 * moments_bwd returns the vector-Jacobian product of (m2, m1) with cotangents
 * (d_m2, d_m1) with respect to xhat, bhat, da, rot (the cumulative angles or
 * quaternions, unconstrained) and h0. Gradients at positions t >= V are exactly
 * zero. Nothing is kept between calls: the backward recomputes the states.
 *
 * Layouts: every tensor is dense row-major (C order), device memory, aligned to
 * at least 16 bytes:
 *   xhat[b,s,c,h,p]  bhat[b,s,c,h,r]  da[b,s,h]
 *   rot[b,s,h,rope_dim/2] (complex) | rot[b,s,h,quat_blocks,4] (quaternion)
 *   h0[b,h,p,r]  m2[b,h,r,r]  m1[b,h,p,r]  d_m2[b,h,r,r]  d_m1[b,h,p,r]
 * The five float inputs share one dtype (desc->dtype); gradients are written in
 * that dtype; m2, m1, d_m2 and d_m1 are float32. Arithmetic accumulates in fp32.
 *
 * Ownership: the caller allocates every buffer, including the workspace, and
 * keeps them alive until the work queued on `stream` (a hipStream_t, NULL = the
 * default stream) has finished. The library allocates no device memory, keeps
 * no state between calls, and fully overwrites every output it is given.
 *
 * Errors: functions return 0 on success or a negative MOMENTS_E* code; nothing
 * is launched when a call fails validation. moments_strerror() names a code;
 * moments_last_hip_error() returns the hipError_t behind MOMENTS_EHIP.
 *
 * Debug check: with the environment variable MOMENTS_CHECK_FINITE set (to
 * anything but "" or "0", read at every call), moments_fwd* and moments_bwd*
 * scan their outputs after the work (m2 and m1; every gradient they wrote),
 * wait for the stream, and return MOMENTS_ENONFINITE if one holds a NaN or an
 * infinity (the pages sanitise m2 and m1 at the end of moments_phys_fwd,
 * "recalculated.rs" source page; the sanitiser's body is not on the pages and
 * is read as this check). The flag lives in the last 256 bytes of the workspace.
 */
#ifndef MOMENTS_H
#define MOMENTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOMENTS_OK = 0,
  MOMENTS_EINVAL = -1,     /* bad descriptor, NULL required pointer, misalignment */
  MOMENTS_ENOTSUP = -2,    /* shape outside what the compiled kernels cover */
  MOMENTS_EWORKSPACE = -3, /* workspace_bytes below moments_workspace_size() */
  MOMENTS_EHIP = -4,       /* a HIP launch or runtime call failed */
  MOMENTS_ESCRATCH = -5,   /* moments_fwd_static: the problem needs more scratch than it has */
  MOMENTS_ENONFINITE = -6  /* debug check (MOMENTS_CHECK_FINITE set): an output is not finite */
};

typedef enum { MOMENTS_F32 = 0, MOMENTS_BF16 = 1 } moments_dtype;

typedef enum {
  MOMENTS_ROT_NONE = 0,
  MOMENTS_ROT_COMPLEX_PAIRWISE = 1,
  MOMENTS_ROT_COMPLEX_HALF = 2,
  MOMENTS_ROT_QUATERNION = 3
} moments_rot_kind;

typedef struct {
  int64_t b, s, c, h, p, r; /* batch, sequence, channels, heads, rows, state rank */
  int64_t chunk_len;        /* the caller's chunk length l: 1 <= l, s % l == 0 */
  int64_t valid_len;        /* positions >= valid_len are padding; >= s acts as s */
  int32_t dtype;            /* moments_dtype */
  int32_t rot_kind;         /* moments_rot_kind */
  int64_t rope_dim;         /* complex modes: rotated coordinates, even, <= r */
  int64_t quat_blocks;      /* quaternion mode: J, 4*J <= r */
  /* Per-sequence valid lengths (ragged batch), or NULL: a device array of b
   * int32; sequence bi uses V_bi = min(max(valid_lens[bi], 0), valid_len, s)
   * in place of the batch-wide min(valid_len, s), which still bounds every
   * sequence and sizes the workspaces ("recalculated.rs" page, chunk_mask and
   * the trait's valid_len: one scalar there; here the masks, and so the
   * gradients that are exactly zero, follow each sequence's own length).
   * The array is read by the kernels (device memory, alive until the queued
   * work has finished); the host never reads it. */
  const int32_t* valid_lens;
} moments_desc;

/* Host-only check of a descriptor (no GPU needed). Returns 0, MOMENTS_EINVAL or
 * MOMENTS_ENOTSUP. Supported: 1 <= r <= 128, 1 <= c <= 4, p >= 1, any s, b, h;
 * half-split needs r even; rope_dim/2 <= r/2 there. */
int moments_validate(const moments_desc* desc);

/* Bytes of device workspace moments_fwd (is_bwd = 0) or moments_bwd (is_bwd = 1)
 * needs for this descriptor, or a negative error code. */
int64_t moments_workspace_size(const moments_desc* desc, int is_bwd);

/* Forward: m2, m1 (float32) from the five inputs. rot may be NULL only for
 * MOMENTS_ROT_NONE; h0 may be NULL (zero initial state). */
int moments_fwd(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                const void* rot, const void* h0, float* m2, float* m1, void* workspace,
                size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same operation, arguments and results as moments_fwd,
 * but the kernels' scratch (boundary carries and per-workgroup partial moments)
 * lives in a static device array of MOMENTS_STATIC_SCRATCH_BYTES (64 MiB), one
 * copy per GPU, held until the process ends. Calls no hipMalloc, hipFree or
 * allocating library routine. Problems whose forward workspace
 * (moments_workspace_size(desc, 0)) exceeds that size return MOMENTS_ESCRATCH
 * without launching anything. Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (concurrent streams or host threads) race; calls
 * ordered on one stream are safe. The first call on a device looks up the
 * array's address there. With per-kernel timing enabled it creates HIP events. */
#define MOMENTS_STATIC_SCRATCH_BYTES (64ull << 20)
int moments_fwd_static(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                       const void* rot, const void* h0, float* m2, float* m1, void* stream);

/* Backward: the VJP of (m2, m1) with cotangents d_m2 [b,h,r,r] (need not be
 * symmetric; only d_m2 + d_m2^T enters) and d_m1 [b,h,p,r]. Any gradient
 * pointer may be NULL (not wanted); d_rot must be NULL for MOMENTS_ROT_NONE. */
int moments_bwd(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                const void* rot, const void* h0, const float* d_m2, const float* d_m1,
                void* d_xhat, void* d_bhat, void* d_da, void* d_rot, void* d_h0,
                void* workspace, size_t workspace_bytes, void* stream);

/* Saved-carry variant ("backward.rs" source page, module doc and
 * boundary_carries: the backward needs the state entering every chunk, which
 * the pages recompute with a cheap chunk-level pass; "recalculated.rs" module
 * doc: the node itself keeps only its inputs). moments_fwd_save is moments_fwd
 * that also leaves those boundary states in a caller buffer `saved`;
 * moments_bwd_saved is moments_bwd that reads them from there instead of
 * recomputing them (it skips the carry pass). The results equal the plain
 * calls up to rounding (the states reach the buffer through the forward's own
 * arithmetic).
 *
 * `saved` holds, at kernel-chunk granularity (moments_kernel_chunk_len()
 * tokens; NK = ceil(min(valid_len, s) / that) chunks per chain):
 *   float32 states [b*h][NK][p][r] entering each chunk (entry 0 is h0, or
 *   zeros), columns in the library's internal order (the caller's order, except
 *   that half-split pairs (i, r/2+i) sit at (2i, 2i+1)), then, at the next
 *   256-byte boundary, float32 chunk decays [b*h][NK] (exp of the sum of da over
 *   the chunk; the last chunk's entry is not used).
 * Treat it as opaque: fill it with moments_fwd_save and pass it, unchanged and
 * with the same descriptor and inputs, to moments_bwd_saved. Its size is
 * moments_saved_size(desc) bytes (about 4 * b*h*NK*p*r), device memory, 16-byte
 * aligned, owned by the caller. A saved buffer below that size returns
 * MOMENTS_EWORKSPACE, a NULL one MOMENTS_EINVAL. Workspaces are those of
 * moments_fwd and moments_bwd. For bf16 with c = 4 the backward walks token
 * pairs, with chunk boundaries of its own, and runs its own carry pass: there
 * moments_bwd_saved validates the buffer but does not read it. */
int64_t moments_saved_size(const moments_desc* desc);
int moments_fwd_save(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                     const void* rot, const void* h0, float* m2, float* m1, void* saved,
                     size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream);
int moments_bwd_saved(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                      const void* rot, const void* h0, const void* saved, size_t saved_bytes,
                      const float* d_m2, const float* d_m1, void* d_xhat, void* d_bhat, void* d_da,
                      void* d_rot, void* d_h0, void* workspace, size_t workspace_bytes, void* stream);

/* Rotation-sequence producer: builds the cumulative rotation that moments_fwd
 * and moments_bwd take (rot) from per-token increments ("recalculated.rs"
 * source page: RotPrim carries cumulative angles [b,s,h,a] or cumulative unit
 * quaternions [b,s,h,J,4]; quat_mul_prim is the Hamilton product on the packed
 * (w,x,y,z) axis). The pages do not print this step; it is read as
 *   complex modes : rot[b,t,h,i] = sum_{t' <= t} inc[b,t',h,i]
 *   quaternion    : rot[b,t,h,j] = N(rot[b,t-1,h,j] (x) inc[b,t,h,j]),
 *                   rot[b,-1,h,j] = 1, N(v) = v / |v|
 * (left-to-right composition, renormalised every step; for unit increments N
 * changes nothing in exact arithmetic, for any nonzero increments the result is
 * the normalised product inc[0] (x) ... (x) inc[t]). Every position t < s is
 * produced (valid_len is not read). Quaternion increments must be nonzero.
 *
 * Reads desc->b, s, h, dtype, rot_kind (not MOMENTS_ROT_NONE), rope_dim (complex
 * modes: a = rope_dim/2 angles per head) or quat_blocks; the other fields are
 * ignored. inc and rot have rot's layout from moments_fwd ([b,s,h,a] or
 * [b,s,h,J,4], row-major, desc->dtype, 16-byte aligned device memory) and must
 * not overlap. Sums and products run in fp32. Returns MOMENTS_EINVAL for a bad
 * descriptor, NULL or misaligned pointers, MOMENTS_ENOTSUP for b > 65535 or
 * more than 2^24 chains per token (h * a or h * J) or 2^30 in all (times b),
 * MOMENTS_EWORKSPACE below moments_rot_workspace_size(); empty shapes (b, s or h
 * zero) launch nothing and accept NULL pointers. */
int64_t moments_rot_workspace_size(const moments_desc* desc, int is_bwd);
int moments_rot_fwd(const moments_desc* desc, const void* inc, void* rot, void* workspace,
                    size_t workspace_bytes, void* stream);

/* VJP of the producer: d_inc from d_rot (the cotangent of rot, e.g. the d_rot
 * moments_bwd returns) and the same increments inc:
 *   complex modes : d_inc[t] = sum_{t' >= t} d_rot[t']
 *   quaternion    : the reverse-mode derivative of the renormalised product;
 *                   d_inc[t] is orthogonal to inc[t] (rescaling an increment
 *                   leaves rot unchanged).
 * Same layouts, dtype, alignment and errors as moments_rot_fwd; inc, d_rot and
 * d_inc must not overlap. */
int moments_rot_bwd(const moments_desc* desc, const void* inc, const void* d_rot, void* d_inc,
                    void* workspace, size_t workspace_bytes, void* stream);

const char* moments_strerror(int code);
int moments_last_hip_error(void);

/* Tokens per kernel chunk. The kernels split every chain into chunks of this
 * many tokens whatever desc->chunk_len is: the chunked states equal the per-token
 * recurrence at any chunk length ("backward.rs" page, module doc "Gradient
 * math": the decays are products of exp(da) over the tokens in between), so
 * only the rounding differs. Host-only. */
int64_t moments_kernel_chunk_len(void);

/* Diagnostics: per-kernel timing. While enabled (on != 0), each kernel launch
 * of moments_fwd / moments_bwd is bracketed by two HIP events recorded on the
 * caller's stream (the stream the kernel runs on); disabled by default.
 * moments_profile_read() waits for the recorded events, folds them into
 * per-kernel totals and reports kernel `id` (0 <= id < the returned count):
 * its name, number of timed launches and summed milliseconds. It returns the
 * number of kernel ids, or a negative error code. Not thread-safe with
 * concurrent fwd/bwd calls from other host threads. */
int moments_profile_enable(int on);
int moments_profile_read(int id, const char** name, int64_t* launches, double* total_ms);
void moments_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MOMENTS_H */
