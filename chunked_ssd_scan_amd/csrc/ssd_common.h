// Helpers shared by the chunked SSD scan (ssd_scan.hip) and the diagonal
// selective scan (sel_scan.hip), both linked into libssd_scan.so.
#ifndef SSD_COMMON_H
#define SSD_COMMON_H

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "ssd_scan.h"

namespace ssd_detail {

constexpr float kLog2e = 1.4426950408889634f;

// Buffer resource over `bytes` bytes at `base` (raw addressing, stride 0).
// Loads past `bytes` return zero and stores past it are dropped, which the
// kernels use for ragged tails and for rows beyond a segment's range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOOB = 0x80000000u;  // lane offset that always falls outside a range

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Span {
    uintptr_t lo, hi;
};

inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

inline Span span_of(const void* p, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + (uintptr_t)bytes};
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Scratch of at least `bytes` for `stream` on the current device, cached per
// (device, stream, slot) and ordered after its previous use; nullptr on
// failure. *entry identifies it for scratch_release, which marks the end of
// this call's use on the stream (defined in ssd_scan.hip). A call that runs
// another entry point inside it keeps its own buffers in another slot.
enum { kSlotWork = 0, kSlotExpand = 1, kSlotMoments = 2, kSlotBackward = 3 };
void* scratch_acquire(hipStream_t stream, size_t bytes, int* entry, int slot = kSlotWork);
bool scratch_release(int entry);

// Compute units of the current device (256 if the query fails).
int device_cus();

// The shape checks of ssd_forward (sizes, envelope, dtype; defined in
// ssd_scan.hip).
ssd_status forward_shape_status(const ssd_dims* d, int64_t chunk_len, int64_t R, bool has_theta);

// ssd_forward_ex; with ysub = 1 (seqlen even) y keeps only the odd time
// steps, step 2s + 1 written as step s of a y with seqlen / 2 steps (defined
// in ssd_scan.hip).
ssd_status forward_impl(const ssd_dims* d, const void* x, const float* da, const void* B,
                        const void* C, const float* D, const float* init_state, int64_t chunk_len,
                        int64_t R, const float* theta, float* y, float* final_state,
                        const ssd_launch_opts* opts, void* stream, int ysub);

// ssd_forward_ex in two phases. forward_plan checks every argument and picks
// the launch plan (host only: no HIP call but device queries); ws_bytes is the
// workspace the launch needs. forward_launch enqueues the kernels with a
// workspace of at least ws_bytes (may be null when ws_bytes is 0); it fails
// only on a HIP error, possibly after part of the work was enqueued.
struct Plan {
    int64_t b, T, H, P, N, G, R, NP;
    int dtype, S, nsub, Qt, log2R;
    int SF;    // state-pass segments per output segment (the state pass divides finer)
    int kind;  // kernel path: general walk or column-block walk
    int W;     // column-block width in 16-column slices (column-block walk)
};
struct FwdPlan {
    Plan pl;
    bool rot, cols, shared;
    size_t ws_bytes;
    int ysub;
};
ssd_status forward_plan(const ssd_dims* d, const void* x, const float* da, const void* B,
                        const void* C, const float* D, const float* init_state, int64_t chunk_len,
                        int64_t R, const float* theta, float* y, float* final_state,
                        const ssd_launch_opts* opts, int ysub, FwdPlan* out);
// The trapezoid's own inputs, when the rotating column walk stages its
// sub-steps straight from the source arrays (forward_launch with trap set:
// the plan is for 2T sub-steps; x, B, C, theta have T steps, da is the
// per-sub-step da, with scale, the per-sub-step write scale).
struct TrapSrc {
    const float* scale;      // [b][2T][H]
    const void* prev_x;      // may be null (with prev_B)
    const void* prev_B;
};
ssd_status forward_launch(const FwdPlan& fp, const void* x, const float* da, const void* B,
                          const void* C, const float* D, const float* init_state, const float* theta,
                          float* y, float* final_state, void* ws, void* const* walk_events,
                          hipStream_t hs, const TrapSrc* trap = nullptr);
// forward_plan without the argument checks (shape, options and pointers are
// the caller's to check): the launch plan and workspace of problem d.
ssd_status forward_plan_shape(const ssd_dims* d, int64_t R, bool rot, const ssd_launch_opts* opts, int ysub,
                              FwdPlan* out);

// The trapezoid's sub-step inputs (trap_scan.hip): every step t of the
// two-write recurrence becomes sub-steps 2t (decay, the previous write scaled
// by beta) and 2t + 1 (turn by theta, this write scaled by gamma). The
// expanded arrays live in a workspace: trap_expand_bytes sizes it (C may be
// left out), trap_expand_setup points the output arrays into it, and
// trap_expand_launch enqueues the expansion kernel.
struct TrapExpand {
    const void* x;
    const float* da;
    const void* B;
    const void* C;           // may be null: no C^ is built
    const float* beta;
    const float* gamma;
    const void* prev_x;
    const void* prev_B;
    const float* theta;
    void* xh;                // [b][2T][R][H][P]
    float* dah;              // [b][2T][H]
    void* Bh;                // [b][2T][R][G][N]
    void* Ch;                // [b][2T][R][G][N], or null
    float* thh;              // [b][2T][H][N/2], or null
    int64_t b, T, R, H, P, G, N;
    int esz;                 // bytes per x/B/C element (2: bf16, 4: fp32)
};
size_t trap_expand_bytes(const TrapExpand& a);
void trap_expand_setup(TrapExpand* a, void* ws);
ssd_status trap_expand_launch(const TrapExpand& a, hipStream_t hs);

// The forward's state passes alone (pass A and the carry), for callers that
// need the state entering every segment: states_plan makes the forward's
// launch plan for (d, R, rot) and the workspace those passes need;
// states_launch enqueues them (nothing when the plan has one segment) and
// returns in *ws_state the [b*H][S*SF][P][N] entering states (nullptr with
// one segment: the caller starts from init_state).
ssd_status states_plan(const ssd_dims* d, int64_t R, bool rot, Plan* pl, size_t* ws_bytes);
ssd_status states_launch(const Plan& pl, bool rot, const void* x, const float* da, const void* B,
                         const float* init_state, const float* theta, void* ws, hipStream_t hs,
                         float** ws_state);

// Kernel addresses for a launch plan, nullptr when no instantiation fits
// (defined in the instantiation units ssd_walk_{bf16,f32}.hip and
// ssd_cols_{bf16,f32}.hip). mode 1: state-only pass, 0: output pass; ysub:
// the output pass that keeps only odd steps of y.
void* select_walk_bf16(bool rot, int mode, int P, int NP);
void* select_walk_f32(bool rot, int mode, int P, int NP);
void* select_cols_bf16(int mode, int w, int NP, bool ysub);
void* select_cols_f32(int mode, int w, int NP, bool ysub);
void* select_cols_rot_bf16(int mode, int w, int NP, bool ysub);
void* cb_pack_bf16(int NP);
void* cb_pack_f32(int NP);

}  // namespace ssd_detail

#endif  // SSD_COMMON_H
