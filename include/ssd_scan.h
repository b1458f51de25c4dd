/*
 * ssd_scan.h - C ABI of the chunked state-space-duality (SSD) scan forward
 * pass on AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h; g = h / (H/G) is the B/C group):
 *
 *   h_{-1}  = init_state[b,h]            (P x N, or zero when init_state is NULL)
 *   h_t     = exp(da[b,t,h]) * R(theta[b,t,h]) h_{t-1}
 *             + sum_{r<R} x[b,t,r,h,:] (outer) B[b,t,r,g,:]
 *   y[b,t,r,h,p] = sum_n C[b,t,r,g,n] * h_t[p,n] + D[h] * x[b,t,r,h,p]
 *   final_state[b,h] = h_{T-1}
 *
 * R(theta) turns every state pair (2k, 2k+1) by the plane rotation
 * [[cos, -sin], [sin, cos]] of angle theta[b,t,h,k] (identity when theta is
 * NULL). Sources, by page and section:
 *  - burn-mamba "mamba3/ssd/serial.rs", ssd_serial with stages k1 (chunk
 *    cumsum of da), k2 (C B^T on the rank-fused rows), k3 (chunk states),
 *    k4 (serial state passing) and k5 (chunk scan Y_diag + Y_off): the
 *    multi-rank (MIMO) chunked form, inputs pre-scaled (dt enters only via da),
 *    the K5 mask keeping the whole R x R diagonal block, no skip inside.
 *  - LeetGPU "SSM Selective Scan" write-up, problem statement: the skip term
 *    D * x and the starting state of zero.
 *  - "mamba3/scan.py", module docstring and cumulative_angles / rotate_by:
 *    the data-dependent rotation, folded into B and C by inclusive cumulative
 *    angles Phi_t (B~ = R(-Phi_t) B, C~ = R(-Phi_t) C); the returned
 *    final_state is the physical state h_{T-1} = R(Phi_{T-1}) g_{T-1}.
 *  - burn-mamba "modules/misc/segsum.rs": decays are exponentials of
 *    differences of prefix sums, masked before exp.
 *
 * Layouts: dense, row-major, device memory.
 *   x           [b, T, R, H, P]   in_dtype (fp32 or bf16)
 *   da          [b, T, H]         fp32, finite and <= 0 (log of the decay)
 *   B, C        [b, T, R, G, N]   in_dtype
 *   D           [H]               fp32, may be NULL (no skip term)
 *   init_state  [b, H, P, N]      fp32, may be NULL (zero initial state)
 *   theta       [b, T, H, N/2]    fp32, may be NULL (no rotation)
 *   y           [b, T, R, H, P]   fp32, written in full
 *   final_state [b, H, P, N]      fp32, written in full
 * x, B, C, init_state, y and final_state must be 16-byte aligned; da, D and
 * theta 4-byte aligned.
 *
 * Ownership: the caller owns every buffer and keeps inputs alive until the
 * work enqueued on `stream` has completed. Nothing is retained after return.
 * Scratch (the head-shared C B^T tile pack, and segment states when the
 * sequence is split; see ssd_workspace_bytes) is the library's: one device
 * buffer per (device, stream), allocated on first use, grown when a call
 * needs more (hipMalloc, after the old buffer's last use has finished) and
 * kept until the process ends. Each call orders its kernels after the
 * previous call that used the buffer (an event), so calls are asynchronous.
 * Calls on different streams use different buffers; calls on one stream are
 * ordered by it.
 * final_state may be the same pointer as init_state (in-place state update);
 * any other overlap between an output and another buffer is SSD_ERR_ALIAS.
 *
 * Errors: every argument, the launch plan and the scratch buffer are checked
 * or obtained on the host before the first kernel is enqueued. On every error
 * status except SSD_ERR_HIP no kernel is launched and no output is touched.
 * SSD_ERR_HIP (a failed HIP call) can come after part of the call's kernels
 * were enqueued; y and final_state are then unspecified.
 * The call is asynchronous: it returns after enqueueing on `stream` (a
 * hipStream_t; NULL means the null stream) without synchronising.
 * Different streams may call concurrently (host threads included); they
 * share only the scratch cache's bookkeeping, which is locked.
 *
 * Supported envelope (SSD_ERR_UNSUPPORTED outside it):
 *   P in {16, 32, 64, 128}; N in {16, 32, 64, 128, 256};
 *   R in {1, 2, 4, 8, 16}; in_dtype fp32 or bf16.
 */
#ifndef SSD_SCAN_H
#define SSD_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
    int64_t batch;    /* b >= 1 */
    int64_t seqlen;   /* T >= 1 time steps */
    int64_t nheads;   /* H >= 1 */
    int64_t headdim;  /* P */
    int64_t dstate;   /* N */
    int64_t ngroups;  /* G >= 1, H % G == 0 */
    int32_t in_dtype; /* ssd_dtype of x, B and C */
} ssd_dims;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,    /* a required pointer (x, da, B, C, y, final_state, dims) is NULL */
    SSD_ERR_BAD_SHAPE = 2,   /* T < 1, b/H/P/N/G < 1, H % G != 0, chunk_len < 1, R < 1, odd N with theta */
    SSD_ERR_UNSUPPORTED = 3, /* valid but outside the kernels' envelope, or a misaligned pointer */
    SSD_ERR_ALIAS = 4,       /* an output overlaps another buffer (final_state == init_state is allowed) */
    SSD_ERR_HIP = 5,         /* a HIP call or kernel launch failed */
    SSD_ERR_WORKSPACE = 6    /* ssd_forward_noalloc: the problem needs more scratch than
                                SSD_NOALLOC_SCRATCH_BYTES */
} ssd_status;

/* Launch choices that do not change the result beyond rounding. */
typedef struct {
    int32_t segments;        /* 0: automatic. k >= 1: split every sequence into k
                                segments that run in parallel, joined by a state
                                carry pass (clamped to the number of 32-row tiles) */
    int32_t block_slices;    /* 0: automatic. k >= 1: each workgroup of the
                                shared-B/C walk owns k consecutive 16-column
                                slices of one time row flattened over
                                (head, headdim) within a B/C group; k must be
                                1, 2, 4, 6, 8 or 10, divide
                                (nheads / ngroups) * headdim / 16 and have a
                                kernel for (dstate, dtype), else
                                SSD_ERR_UNSUPPORTED. Ignored when theta is given
                                (rotation walks one head per workgroup). */
    int32_t reserved[2];     /* must be zero */
    void *walk_events[2];    /* NULL, NULL: none. Two hipEvent_t (cast to void*)
                                created by the caller: the library records
                                walk_events[0] on the stream just before the
                                launch of the output walk (the kernel that
                                writes y and final_state, which dominates the
                                call's time) and walk_events[1] just after
                                it, so the caller can time that kernel alone.
                                Both or neither must be given, else
                                SSD_ERR_BAD_SHAPE; a failed record is
                                SSD_ERR_HIP. */
} ssd_launch_opts;

/*
 * Forward chunked SSD scan (see the header comment for the definition).
 *   d          problem sizes and the dtype of x, B, C
 *   chunk_len  chunk length in time steps (>= 1). The result is the same for
 *              every chunk length up to rounding, because the chunked form is
 *              exact; the kernels walk 32-row tiles (32/R time steps) and
 *              accept any chunk_len >= 1.
 *   R          MIMO rank (writes per time step)
 *   stream     hipStream_t cast to void*, or NULL
 */
ssd_status ssd_forward(const ssd_dims *d, const void *x, const float *da,
                       const void *B, const void *C, const float *D,
                       const float *init_state, int64_t chunk_len, int64_t R,
                       const float *theta, float *y, float *final_state,
                       void *stream);

/* ssd_forward with explicit launch options (NULL opts = automatic). */
ssd_status ssd_forward_ex(const ssd_dims *d, const void *x, const float *da,
                          const void *B, const void *C, const float *D,
                          const float *init_state, int64_t chunk_len, int64_t R,
                          const float *theta, float *y, float *final_state,
                          const ssd_launch_opts *opts, void *stream);

/* Bytes of scratch ssd_forward needs for this problem with automatic launch
 * options: the larger of the plans without and with rotation (the shared
 * C B^T tile pack, plus segment states when the sequence is split). The
 * library takes it from its per-(device, stream) cache (ssd_forward_ex) or
 * from its fixed array (ssd_forward_noalloc). Returns 0 for invalid arguments. */
size_t ssd_workspace_bytes(const ssd_dims *d, int64_t chunk_len, int64_t R);

/*
 * Diagonal selective scan (Mamba-1 form), LeetGPU "SSM Selective Scan"
 * write-up, problem statement: per batch b, channel d and state n, from a
 * zero state,
 *   h[n]      = exp(delta[b,t,d] * A[d,n]) * h[n] + delta[b,t,d] * B[b,t,n] * u[b,t,d]
 *   y[b,t,d]  = sum_n C[b,t,n] * h[n] + skip[d] * u[b,t,d]
 * (the decay is diagonal per (d, n); B and C are shared by every channel).
 *
 * Layouts: dense, row-major, fp32, device memory, 4-byte aligned.
 *   u, delta  [batch, seq_len, d_model]
 *   A         [d_model, d_state]
 *   B, C      [batch, seq_len, d_state]
 *   skip      [d_model]
 *   y         [batch, seq_len, d_model], written in full
 * Sizes: batch in 1..65535, seq_len >= 1, d_model in 1..2^22, d_state in
 * 1..64 (SSD_ERR_UNSUPPORTED above these bounds). Ownership, asynchrony and scratch are as
 * for ssd_forward: the sequence is cut into chunks that run in parallel and
 * are joined by a carry pass through the per-(device, stream) scratch buffer.
 * Errors: SSD_ERR_NULL_ARG for a NULL pointer, SSD_ERR_BAD_SHAPE for a size
 * below 1, SSD_ERR_ALIAS when y overlaps an input, SSD_ERR_UNSUPPORTED for
 * a misaligned pointer or sizes outside the envelope; nothing is enqueued on
 * any of these.
 */
ssd_status ssd_selective_scan(const float *u, const float *delta, const float *A,
                              const float *B, const float *C, const float *skip,
                              float *y, int64_t batch, int64_t seq_len,
                              int64_t d_model, int64_t d_state, void *stream);

/* ssd_selective_scan with launch options (NULL opts = automatic):
 *   segments      0: automatic; k >= 1: cut every sequence into chunks of
 *                 ceil(seq_len / k') steps, k' = min(k, seq_len, 4096) (the
 *                 last chunk may be shorter; there are at most k' chunks)
 *   block_slices  must be 0 (SSD_ERR_UNSUPPORTED otherwise)
 *   reserved      must be zero (SSD_ERR_BAD_SHAPE otherwise)
 *   walk_events   recorded just before and just after the output pass (the
 *                 kernel that writes y); both or neither (SSD_ERR_BAD_SHAPE)
 * The result does not depend on the options beyond rounding. */
ssd_status ssd_selective_scan_ex(const float *u, const float *delta, const float *A,
                                 const float *B, const float *C, const float *skip,
                                 float *y, int64_t batch, int64_t seq_len,
                                 int64_t d_model, int64_t d_state,
                                 const ssd_launch_opts *opts, void *stream);

/*
 * Mamba-3 trapezoid (two-write) forward. "mamba3/scan.py", module docstring
 * and scan_forward (whose comment cites the Mamba-3 paper's eq. 11), and
 * burn-mamba "mamba3/moments.rs", build_moments_input (previous-token
 * entries). Per batch b and head h (group g = h / (H/G)):
 *
 *   W_t  = sum_r x[b,t,r,h,:] (outer) B[b,t,r,g,:]
 *   W_-1 = sum_r prev_x[b,r,h,:] (outer) prev_B[b,r,g,:]   (zero when NULL)
 *   h_t  = R(theta[b,t,h]) (exp(da[b,t,h]) h_{t-1} + beta[b,t,h] W_{t-1})
 *          + gamma[b,t,h] W_t
 *   y[b,t,r,h,p] = sum_n C[b,t,r,g,n] h_t[p,n]        (no skip term)
 *   h_-1 = init_state (or zero), final_state = h_{T-1}
 *
 * The previous step's write is turned by theta_t with the decayed state
 * (it enters the cumulative frame at the previous step's angle).
 * Arguments as ssd_forward_ex (without D), plus:
 *   beta, gamma  [b, T, H] fp32, 4-byte aligned
 *   prev_x       [b, R, H, P] in_dtype, 16-byte aligned, may be NULL
 *   prev_B       [b, R, G, N] in_dtype, 16-byte aligned; NULL exactly when
 *                prev_x is (SSD_ERR_NULL_ARG otherwise)
 *   batch * seqlen must stay below 2^31 (SSD_ERR_UNSUPPORTED)
 * Runs as the single-write scan over 2T sub-steps (decay then turn), which
 * writes y for the odd sub-steps only, so the envelope is ssd_forward's at
 * seqlen 2T; opts apply to that scan (walk events bracket its output walk).
 * Where the scan takes its rotating column walk (bf16, rotation, headdim 64
 * or 128, dstate 64 or 128, R >= 4) that walk reads the sub-steps straight
 * from x, B, C and theta and applies beta and gamma in fp32. Other shapes
 * first expand the sub-step inputs into scratch; with bf16 inputs that stores
 * beta_t x_{t-1} and gamma_t x_t as bf16, one extra rounding (at most 2^-9
 * relative) of the scaled x.
 * Scratch: the sub-step inputs (about 2x x, B, C, da and theta in bytes) in
 * a second per-(device, stream) buffer of the library, besides
 * ssd_forward's own.
 */
ssd_status ssd_trapezoid_forward(const ssd_dims *d, const void *x, const float *da,
                                 const void *B, const void *C, const float *beta,
                                 const float *gamma, const void *prev_x, const void *prev_B,
                                 const float *init_state, int64_t chunk_len, int64_t R,
                                 const float *theta, float *y, float *final_state,
                                 const ssd_launch_opts *opts, void *stream);

/*
 * Physical-frame state moments, burn-mamba "mamba3/moments.rs", module
 * documentation (per-token states, de-rotated to the physical frame, plain
 * real sums masked to valid_len) and state_moments_phys. For every batch b
 * and head h, with h_t the physical state (P x N) after step t:
 *
 *   m2[b,h][n][n'] = sum_{t < valid_len} sum_p h_t[p][n] h_t[p][n']
 *   m1[b,h][n]     = sum_{t < valid_len} sum_p h_t[p][n]
 *
 * (count = valid_len * P samples per (b, h)). h_t follows
 *   - with beta and gamma NULL: the recurrence of ssd_forward,
 *     h_t = exp(da_t) R(theta_t) h_{t-1} + sum_r x_{t,r} (outer) B_{t,r};
 *   - with beta and gamma: the Mamba-3 trapezoid of ssd_trapezoid_forward,
 *     with the optional previous-token entries prev_x, prev_B.
 * Steps t >= valid_len still advance the state but are not counted (their
 * inputs cannot change the result). C, y and D play no part.
 * Arguments: as ssd_forward / ssd_trapezoid_forward (same layouts and
 * dtypes), plus
 *   valid_len   1 <= valid_len <= seqlen, else SSD_ERR_BAD_SHAPE
 *   m2          [b, H, N, N] fp32, written in full (symmetric), 16-byte aligned
 *   m1          [b, H, N]    fp32, written in full
 * Envelope: as ssd_forward with dstate <= 128; theta 16-byte aligned.
 * Errors: SSD_ERR_NULL_ARG for a NULL required pointer or a lone beta/gamma or
 * prev_x/prev_B; SSD_ERR_BAD_SHAPE also for prev_x without beta; SSD_ERR_ALIAS
 * when m2 or m1 overlaps an input or each other. Ownership, scratch and
 * asynchrony as ssd_trapezoid_forward (the state passes of the forward give
 * each segment its entering state).
 */
ssd_status ssd_state_moments(const ssd_dims *d, const void *x, const float *da, const void *B,
                             const float *beta, const float *gamma, const void *prev_x,
                             const void *prev_B, const float *init_state, int64_t R,
                             const float *theta, int64_t valid_len, float *m2, float *m1,
                             void *stream);

/*
 * Gradients of the scan ("mamba3/scan.py", verify(): the backward of the fast
 * scan is checked against the token recurrence; burn-mamba
 * "mamba3/moments.rs", module documentation: states recomputed in the
 * backward rather than stored). For the recurrence of ssd_forward (no chunk
 * length: the result does not depend on one), given dy = dL/dy and
 * dfinal = dL/dfinal_state, with h_t the physical state after step t,
 * a_t = exp(da_t) and H_t = dL/dh_t:
 *
 *   H_t   = a_{t+1} R(theta_{t+1})^T H_{t+1} + sum_r dy_{t,r} (outer) C_{t,r}
 *           (H_{T-1} from dfinal)
 *   dx[b,t,r,h,p] = sum_n H_t[p,n] B[b,t,r,g,n] + D[h] dy[b,t,r,h,p]
 *   dB[b,t,r,g,n] = sum_{h in g} sum_p H_t[p,n] x[b,t,r,h,p]
 *   dC[b,t,r,g,n] = sum_{h in g} sum_p dy[b,t,r,h,p] h_t[p,n]
 *   dda[b,t,h]    = sum_{s >= t} sum_{p,n} H_s[p,n] (h_s - W_s)[p,n]
 *                   (W_s the write of step s), as a reverse cumulative sum
 *   dtheta[b,t,h,k] = the same sum for the turn of pair k (2-D cross products)
 *   dinit[b,h]    = a_0 R(theta_0)^T H_0
 *   dD[h]         = sum_{b,t,r,p} dy x
 *
 * Arguments: d, x, da, B, C, D, init_state, R, theta as ssd_forward_ex (same
 * layouts, dtypes and alignment; no chunk length), plus
 *   dy      [b, T, R, H, P] fp32, 16-byte aligned
 *   dfinal  [b, H, P, N] fp32, 16-byte aligned, or NULL (zero)
 *   dx      [b, T, R, H, P] fp32, 16-byte aligned
 *   dda     [b, T, H] fp32
 *   dB, dC  [b, T, R, G, N] fp32
 *   dtheta  [b, T, H, N/2] fp32: required exactly when theta is given
 *   dinit   [b, H, P, N] fp32, 16-byte aligned, or NULL (not wanted)
 *   dD      [H] fp32: required exactly when D is given
 * Every output is written in full (none accumulates into what it held).
 * Envelope: as ssd_forward with dstate <= 128 (SSD_ERR_UNSUPPORTED beyond).
 * Errors: SSD_ERR_NULL_ARG for a NULL required pointer or a dtheta/dD that
 * does not match theta/D; SSD_ERR_ALIAS when an output overlaps an input or
 * another output. Ownership and asynchrony as ssd_forward; scratch: the
 * forward's segment states, per-head partial sums of dB and dC
 * (2 b H T R N fp32) and the backward's segment states, in a separate
 * per-(device, stream) buffer of the library.
 * Streams: the recomputation of the forward direction (the forward's state
 * passes and the walk that gives the dC partials and the final state) runs on
 * a second stream that the library creates once per device (default
 * priority), forked from `stream` after the work already queued there and
 * joined back into it before the first kernel that reads its results; to the
 * caller the call is ordered on `stream` alone. Calls on one device take
 * turns enqueueing on that second stream (a lock held from fork to join).
 */
ssd_status ssd_backward(const ssd_dims *d, const void *x, const float *da, const void *B,
                        const void *C, const float *D, const float *init_state, int64_t R,
                        const float *theta, const float *dy, const float *dfinal, float *dx,
                        float *dda, float *dB, float *dC, float *dtheta, float *dinit, float *dD,
                        void *stream);

/*
 * ssd_forward_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments, result and launch plan as ssd_forward_ex (bitwise the same
 * output), but the scratch (C B^T tile pack, segment states; the bytes
 * ssd_workspace_bytes reports for the plan) lives in a fixed device array of
 * SSD_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. The call makes no hipMalloc, hipFree or other
 * allocating call; the first call on a device looks up that device's copy of
 * the array once (hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's array and leaves the last call's
 * contents in it: calls that may overlap on one GPU (different streams or
 * host threads without ordering between them) race and must not be made.
 * Calls ordered on one stream are safe.
 * Errors: as ssd_forward_ex, plus SSD_ERR_WORKSPACE when the plan needs more
 * than SSD_NOALLOC_SCRATCH_BYTES (nothing is launched); SSD_ERR_HIP when the
 * array's address cannot be found.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ssd_status ssd_forward_noalloc(const ssd_dims *d, const void *x, const float *da,
                               const void *B, const void *C, const float *D,
                               const float *init_state, int64_t chunk_len, int64_t R,
                               const float *theta, float *y, float *final_state,
                               const ssd_launch_opts *opts, void *stream);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char *ssd_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* SSD_SCAN_H */
