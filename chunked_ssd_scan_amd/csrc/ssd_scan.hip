// Chunked SSD scan forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// A workgroup walks the tiles of one sequence segment in order. A tile is 32
// rank-fused rows (32/R time steps). Per tile it runs the chunk algorithm of
// burn-mamba "mamba3/ssd/serial.rs" (k1..k5) on that tile:
//   K1  inclusive prefix sum of da over the tile (wave shuffles)
//   K2  C B^T on the tile's fused rows (MFMA), turned into the decay matrix
//       L o CB with L[i,j] = exp(cum_i - cum_j) when step(i) >= step(j)
//       (masked before exp, burn-mamba "modules/misc/segsum.rs")
//   K5  y = exp(cum_i) C h_in + (L o CB) x   (+ D x, folded into L's diagonal)
//   K3+K4  h <- exp(cum_last) h + sum_j exp(cum_last - cum_j) x_j (outer) B_j
// The running state h (P x N fp32) never leaves the accumulator registers:
// each wave holds 16 state columns p for every n, so the K4 state passing
// between tiles is a register update, not a memory round trip.
//
// Two walks: the column-block walk (no rotation) gives a workgroup W
// consecutive 16-column slices of the time rows flattened over (head, p)
// within one B/C group, so its x and y rows are contiguous and the B, C and
// C B^T tiles it stages serve every head it touches; the general walk (any
// rotation, or shapes the former does not fit) gives a workgroup one head.
//
// With a rotation ("mamba3/scan.py", cumulative_angles / rotate_by), B and C
// are turned by R(-Phi_t) while they are staged into LDS, Phi being the
// inclusive cumulative angle from the segment start; the final state is
// turned back by R(Phi) to the physical frame.
//
// Long sequences with few (batch, head) pairs are split into S segments:
// pass A computes each segment's end state from zero (state-only walk),
// pass B carries states across segments (h_{s+1} = e^{Lambda_s} R(Phi_s) h_s
// + local_s), pass C walks every segment from its carried state and writes y.
//
// MFMA usage: v_mfma_f32_16x16x32_bf16 for bf16 inputs and
// v_mfma_f32_16x16x4_f32 for fp32 inputs. Lane layouts (16x16 output tile):
//   A operand: lane l holds row l%16, reduction slots 8*(l/16) .. +7
//   B operand: lane l holds col l%16, the same reduction slots
//   D output : lane l holds col l%16, rows 4*(l/16) .. +3
// Any bijection between (lane group, slot) and the reduction index is valid
// as long as A and B use the same one; the kernels pick the bijection that
// lets accumulator registers be reused directly as operands.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ssd_kernels.h"

namespace ssd_detail {

// Scratch is cached per (device, stream) and grows on demand. Stream-ordered
// allocation (hipMallocAsync / hipFreeAsync) would block the host while the
// stream has work in flight, serialising the caller with the device. Calls
// on one stream are ordered by the stream; each call also waits (on the
// device) for the last call that used the buffer, which keeps a stream handle
// that is destroyed and reissued from racing with the old stream's work.
// Buffers live until the process ends.
struct ScratchEntry {
    int dev;
    hipStream_t stream;
    int slot;
    void* ptr;
    size_t bytes;
    hipEvent_t last;    // recorded after the last call that used ptr
};

std::mutex g_scratch_mu;
ScratchEntry g_scratch[256];
int g_scratch_n = 0;

// Scratch of at least `bytes` for `stream` on the current device, ordered
// after its previous use; nullptr on failure. *entry identifies it for
// scratch_release.
void* scratch_acquire(hipStream_t stream, size_t bytes, int* entry, int slot) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    int i = 0;
    while (i < g_scratch_n &&
           !(g_scratch[i].dev == dev && g_scratch[i].stream == stream && g_scratch[i].slot == slot))
        ++i;
    if (i == g_scratch_n) {
        if (g_scratch_n == 256) return nullptr;
        ScratchEntry& e = g_scratch[g_scratch_n];
        e.dev = dev;
        e.stream = stream;
        e.slot = slot;
        e.ptr = nullptr;
        e.bytes = 0;
        if (hipEventCreateWithFlags(&e.last, hipEventDisableTiming) != hipSuccess) return nullptr;
        ++g_scratch_n;
    }
    ScratchEntry& e = g_scratch[i];
    if (e.bytes < bytes) {
        // grow: wait for the old buffer's last use, then replace it
        if (e.ptr) {
            if (hipEventSynchronize(e.last) != hipSuccess || hipFree(e.ptr) != hipSuccess) return nullptr;
            e.ptr = nullptr;
            e.bytes = 0;
        }
        if (hipMalloc(&e.ptr, bytes) != hipSuccess) {
            e.ptr = nullptr;
            return nullptr;
        }
        e.bytes = bytes;
    } else if (hipStreamWaitEvent(stream, e.last, 0) != hipSuccess) {
        return nullptr;
    }
    *entry = i;
    return e.ptr;
}

// Marks the end of this call's use of the scratch on its stream.
bool scratch_release(int entry) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchEntry& e = g_scratch[entry];
    return hipEventRecord(e.last, e.stream) == hipSuccess;
}

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
    return n;
}

}  // namespace ssd_detail

namespace {

using namespace ssd_detail;

// Pass B: carry states across segments, one thread per state pair (p, k).
//   c_0 = init (or 0);  c_{s+1} = exp(Lambda_s) R(Phi_s) c_s + local_s
// over the S segments of the state pass, for s < upto. On entry ws_state slot
// s+1 holds local_s (segment s from a zero state); on exit slot s holds c_s,
// the state entering segment s (slot 0: a copy of init).
__global__ __launch_bounds__(256) void ssd_carry_kernel(const float* __restrict__ init,
                                                       float* __restrict__ ws_state,
                                                       const float* __restrict__ ws_misc,
                                                       int64_t P, int64_t N, int S, int upto, int rot) {
    const int64_t bh = blockIdx.y;
    const int64_t pair = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (pair >= P * (N / 2)) return;
    const int64_t p = pair / (N / 2), kk = pair % (N / 2);
    const int64_t off = p * N + 2 * kk;
    float c0 = 0.f, c1 = 0.f;
    if (init) {
        c0 = init[bh * P * N + off];
        c1 = init[bh * P * N + off + 1];
    }
    float* st0 = ws_state + bh * S * P * N + off;
    st0[0] = c0;
    st0[1] = c1;
    for (int s = 0; s < upto; ++s) {
        const float* misc = ws_misc + (bh * S + s) * (1 + N / 2);
        float* st = ws_state + (bh * S + s + 1) * P * N + off;
        const float dec = __expf(misc[0]);
        if (rot) {
            float sn, cs;
            sincosf(misc[1 + kk], &sn, &cs);
            const float r0 = cs * c0 - sn * c1, r1 = sn * c0 + cs * c1;
            c0 = r0;
            c1 = r1;
        }
        c0 = dec * c0 + st[0];
        c1 = dec * c1 + st[1];
        st[0] = c0;
        st[1] = c1;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

constexpr int kLdsLimit = 160 * 1024;

// Column-block widths (16-column slices per workgroup), preferred first.
constexpr int kColsWidths[] = {10, 8, 6, 4, 2, 1};

// ysub selects the output-pass instantiations that keep only odd steps of y
void* select_cols(int dtype, int mode, int w, int NP, bool ysub = false) {
    return dtype == SSD_BF16 ? select_cols_bf16(mode, w, NP, ysub) : select_cols_f32(mode, w, NP, ysub);
}

// Rotating column walk: bf16 only.
void* select_cols_rot(int dtype, int mode, int w, int NP, bool ysub = false) {
    return dtype == SSD_BF16 ? select_cols_rot_bf16(mode, w, NP, ysub) : nullptr;
}

void* select_walk(int dtype, bool rot, int mode, int P, int NP) {
    return dtype == SSD_BF16 ? select_walk_bf16(rot, mode, P, NP) : select_walk_f32(rot, mode, P, NP);
}

void* cb_pack_sel(int dtype, int NP) { return dtype == SSD_BF16 ? cb_pack_bf16(NP) : cb_pack_f32(NP); }

enum PathKind { kWalkPath = 0, kColsPath = 1 };

bool is_pow2_in(int64_t v, int64_t lo, int64_t hi) {
    if (v < lo || v > hi) return false;
    return (v & (v - 1)) == 0;
}


ssd_status check_shape(const ssd_dims* d, int64_t chunk_len, int64_t R, bool has_theta) {
    if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1)
        return SSD_ERR_BAD_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (chunk_len < 1 || R < 1) return SSD_ERR_BAD_SHAPE;
    if (has_theta && (d->dstate % 2)) return SSD_ERR_BAD_SHAPE;
    if (d->in_dtype != SSD_F32 && d->in_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (!is_pow2_in(d->headdim, 16, 128)) return SSD_ERR_UNSUPPORTED;
    if (!is_pow2_in(d->dstate, 16, 256)) return SSD_ERR_UNSUPPORTED;
    if (!is_pow2_in(R, 1, 16)) return SSD_ERR_UNSUPPORTED;
    // sizes must stay addressable with 64-bit offsets and 32-bit tile counts
    const int64_t TR = d->seqlen * R;
    if (TR > ((int64_t)1 << 40) || d->batch * d->nheads > ((int64_t)1 << 30)) return SSD_ERR_UNSUPPORTED;
    if ((TR + kRows - 1) / kRows > ((int64_t)1 << 30)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Segments per sequence: aim at >= `target` workgroups of `units` per
// segment, but keep >= 4 tiles per segment (each segment boundary costs a
// state-only pass over the preceding tiles).
int auto_segments(int64_t units, int nsub, int64_t target) {
    int64_t want = (target + units - 1) / units;
    int64_t cap = nsub / 4;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want > 256) want = 256;
    return (int)(want < 1 ? 1 : want);
}



// Scratch layout: [segment states | segment Lambda/Phi | C B^T tile pack]
struct WsLayout {
    size_t state, misc, pack, total;
};

WsLayout workspace_layout(const Plan& pl, bool no_pack) {
    WsLayout w{0, 0, 0, 0};
    const size_t bh = (size_t)(pl.b * pl.H), sa = (size_t)pl.S * pl.SF;
    if (pl.S > 1) {
        w.state = align256(bh * sa * pl.P * pl.N * sizeof(float));
        w.misc = align256(bh * sa * (1 + pl.N / 2) * sizeof(float));
    }
    if (!no_pack) w.pack = align256((size_t)(pl.b * pl.G) * pl.nsub * 768 * sizeof(float));
    w.total = w.state + w.misc + w.pack;
    return w;
}


// Most heads one block of w slices touches within a group.
int64_t block_heads(const Plan& pl, int w) {
    const int64_t sph = pl.P / 16, nb = (pl.H / pl.G) * sph / w;
    int64_t most = 0;
    for (int64_t j = 0; j < nb && j < sph; ++j) {   // the pattern repeats every sph blocks
        const int64_t n = (j * w + w - 1) / sph - (j * w) / sph + 1;
        if (n > most) most = n;
    }
    return most;
}

bool cols_ok(const Plan& pl, int w) {
    const int64_t slices = (pl.H / pl.G) * (pl.P / 16);
    return w >= 1 && slices % w == 0 && block_heads(pl, w) <= cols_max_heads(w) &&
           select_cols(pl.dtype, 0, w, (int)pl.NP) && select_cols(pl.dtype, 1, w, (int)pl.NP);
}

// The rotating column walk takes one head per block, R >= 4 (a 4-row group of
// a tile is one time step) and a rotation table of (32 / R) steps x dstate / 2
// pairs per tile.
bool cols_rot_ok(const Plan& pl) {
    const int w = (int)(pl.P / 16);
    return pl.N >= 64 && pl.R >= 4 && (int64_t)pl.Qt * (pl.NP / 2) <= kRotEntries &&
           select_cols_rot(pl.dtype, 0, w, (int)pl.NP) && select_cols_rot(pl.dtype, 1, w, (int)pl.NP);
}

// Kernel path, column-block width and segments. `w_req` and `segments` are
// the caller's launch options (0 = automatic).
ssd_status make_plan(const ssd_dims* d, int64_t R, bool rot, int segments, int w_req, Plan* out) {
    Plan pl;
    pl.b = d->batch; pl.T = d->seqlen; pl.H = d->nheads; pl.P = d->headdim;
    pl.N = d->dstate; pl.G = d->ngroups; pl.R = R;
    pl.NP = pl.N < 32 ? 32 : pl.N;
    pl.dtype = d->in_dtype;
    pl.Qt = (int)(kRows / R);
    pl.log2R = 0;
    while ((1 << pl.log2R) < R) ++pl.log2R;
    pl.nsub = (int)((pl.T * R + kRows - 1) / kRows);
    pl.kind = kWalkPath;
    pl.W = 0;
    pl.SF = 1;

    // the column-block walk addresses a segment with 32-bit offsets: keep
    // each segment, with the tiles prefetched past its end, under 2^30 bytes
    const int64_t esz = pl.dtype == SSD_BF16 ? 2 : 4;
    int64_t row_bytes = pl.H * pl.P * 4 > pl.G * pl.N * esz ? pl.H * pl.P * 4 : pl.G * pl.N * esz;
    if (rot && pl.H * pl.N * 2 > row_bytes) row_bytes = pl.H * pl.N * 2;   // theta rows, per step
    const int64_t max_tiles = ((int64_t)1 << 30) / (kRows * row_bytes) - 4;
    const int cus = device_cus();
    if (rot && max_tiles >= 1 && cols_rot_ok(pl)) {
        pl.W = (int)(pl.P / 16);
        pl.kind = kColsPath;
    } else if (!rot && max_tiles >= 1) {
        const int64_t slices = pl.b * pl.G * (pl.H / pl.G) * (pl.P / 16);
        if (w_req > 0) {
            if (!cols_ok(pl, w_req)) return SSD_ERR_UNSUPPORTED;
            pl.W = w_req;
        } else {
            // The widest block whose workgroups, multiplied by the segments
            // that auto_segments adds when the blocks alone are too few, fill
            // whole rounds of the device (at least 3/4 of the last round);
            // else the width that fills best. A narrow block leaves a CU too
            // little work to hide latency, which costs more than the extra
            // state pass of the segments.
            double best_fill = -1.0;
            for (int w : kColsWidths) {
                if (!cols_ok(pl, w)) continue;
                const int64_t blocks = slices / w;
                const int64_t wgs = blocks * auto_segments(blocks, pl.nsub, cus);
                const int64_t rounds = (wgs + cus - 1) / cus;
                const double fill = (double)wgs / (double)(rounds * cus);
                if (fill > best_fill) {
                    best_fill = fill;
                    pl.W = w;
                }
                if (fill >= 0.75) {
                    pl.W = w;
                    break;
                }
            }
        }
        if (pl.W > 0) pl.kind = kColsPath;
    } else if (w_req > 0 && !rot) {
        return SSD_ERR_UNSUPPORTED;
    }
    int64_t min_segments = 1, units = pl.b * pl.H, target = 2 * cus;
    if (pl.kind == kColsPath) {
        min_segments = (pl.nsub + max_tiles - 1) / max_tiles;
        units = pl.b * pl.H * (pl.P / 16) / pl.W;
        target = cus;
        if (rot) {
            // one-head blocks are small: fill every workgroup slot of the device
            int per_cu = 0;
            void* fn = select_cols_rot(pl.dtype, 0, pl.W, (int)pl.NP);
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * (pl.W + cols_mem_waves(pl.W, true)), 0) ==
                    hipSuccess && per_cu > 1)
                target = (int64_t)cus * per_cu;
        }
    }
    pl.S = segments > 0 ? segments : auto_segments(units, pl.nsub, target);
    if (pl.S > pl.nsub) pl.S = pl.nsub;
    if (pl.S < min_segments) pl.S = (int)min_segments;
    if (pl.S < 1) pl.S = 1;
    // The state pass runs over all but the last segment; when halving its
    // segments still leaves one workgroup per CU at most, it divides each
    // segment in two (the carry pass then joins twice as many segments, and
    // the output pass starts from every other carried state). Measured: the
    // rotated Mamba-3 workload's state pass goes from 128 to 256 workgroups of
    // half the length (0.56 -> 0.45 ms a call); where the halves would need a
    // second round of workgroups it does not pay.
    pl.SF = 1;
    if (pl.S > 1 && pl.nsub / (2 * pl.S) >= 4 && units * (2 * pl.S - 2) <= (int64_t)cus) pl.SF = 2;
    *out = pl;
    return SSD_OK;
}

// Tile walks: the column-block walk (ssd_cols_kernel, shared B/C) or the
// general walk (ssd_walk_kernel, which also handles rotation).
template <typename Args>
ssd_status launch_walk(const Plan& pl, int mode, bool rot, const Args& args, hipStream_t st) {
    void* fn = nullptr;
    int64_t nwg = pl.b * pl.H * args.seg_items;
    unsigned threads = (unsigned)(4 * pl.P);
    if (pl.kind == kColsPath) {
        const bool ysub = args.ysub != 0;
        fn = rot ? select_cols_rot(pl.dtype, mode, pl.W, (int)pl.NP, ysub)
                 : select_cols(pl.dtype, mode, pl.W, (int)pl.NP, ysub);
        nwg = pl.b * args.seg_items * pl.H * (pl.P / 16) / pl.W;
        threads = (unsigned)(64 * (pl.W + cols_mem_waves(pl.W, rot)));
    } else {
        fn = select_walk(pl.dtype, rot, mode, (int)pl.P, (int)pl.NP);
    }
    if (!fn) return SSD_ERR_UNSUPPORTED;
    if (nwg < 1 || nwg > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    dim3 grid((unsigned)nwg), block(threads);
    Args a = args;
    void* kargs[] = {&a};
    if (hipLaunchKernel(fn, grid, block, kargs, 0, st) != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

// Pass A (segment end states) and pass B (carry): with S > 1 segments,
// ws_state slot s of every (batch, head) then holds the physical state
// entering state-pass segment s (S SF of them; slot 0 a copy of init_state).
template <typename Args>
ssd_status run_state_passes(const Plan& pl, bool rot, Args args, const float* init_state, hipStream_t hs) {
    ssd_status rs = SSD_OK;
    const int SA = pl.S * pl.SF;   // segments of the state pass
    args.SF = pl.SF;
    if (pl.S > 1) {
        args.S = SA;
        args.seg_items = SA - pl.SF;
        rs = launch_walk(pl, 1, rot, args, hs);
        if (rs == SSD_OK) {
            dim3 grid((unsigned)((pl.P * (pl.N / 2) + 255) / 256), (unsigned)(pl.b * pl.H));
            hipLaunchKernelGGL(ssd_carry_kernel, grid, dim3(256), 0, hs, init_state, args.ws_state,
                               args.ws_misc, pl.P, pl.N, SA, SA - pl.SF, rot ? 1 : 0);
            if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
        }
    }
    return rs;
}

// Pass A (segment end states), pass B (carry), pass C (outputs).
template <typename Args>
ssd_status run_passes(const Plan& pl, bool rot, Args args, const float* init_state, hipStream_t hs,
                      void* const* walk_events) {
    args.SF = pl.SF;
    ssd_status rs = run_state_passes(pl, rot, args, init_state, hs);
    if (rs == SSD_OK) {
        args.S = pl.S;
        args.seg_items = pl.S;
        const bool timed = walk_events && walk_events[0];
        if (timed && hipEventRecord(reinterpret_cast<hipEvent_t>(walk_events[0]), hs) != hipSuccess)
            return SSD_ERR_HIP;
        rs = launch_walk(pl, 0, rot, args, hs);
        if (rs == SSD_OK && timed && hipEventRecord(reinterpret_cast<hipEvent_t>(walk_events[1]), hs) != hipSuccess)
            rs = SSD_ERR_HIP;
    }
    return rs;
}

}  // namespace

namespace ssd_detail {

ssd_status forward_shape_status(const ssd_dims* d, int64_t chunk_len, int64_t R, bool has_theta) {
    return check_shape(d, chunk_len, R, has_theta);
}

}  // namespace ssd_detail

extern "C" {

const char* ssd_status_str(int32_t status) {
    switch (status) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG";
        case SSD_ERR_BAD_SHAPE: return "SSD_ERR_BAD_SHAPE";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
        case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS";
        case SSD_ERR_HIP: return "SSD_ERR_HIP";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    }
    return "unknown status";
}

size_t ssd_workspace_bytes(const ssd_dims* d, int64_t chunk_len, int64_t R) {
    if (!d || check_shape(d, chunk_len, R, false) != SSD_OK) return 0;
    // the larger of the plans without and with rotation
    Plan pl, pr;
    if (make_plan(d, R, false, 0, 0, &pl) != SSD_OK) return 0;
    const size_t plain = workspace_layout(pl, pl.kind == kWalkPath).total;
    if (d->dstate % 2 || make_plan(d, R, true, 0, 0, &pr) != SSD_OK) return plain;
    const size_t rotated = workspace_layout(pr, true).total;
    return plain > rotated ? plain : rotated;
}

ssd_status ssd_forward_ex(const ssd_dims* d, const void* x, const float* da, const void* B,
                          const void* C, const float* D, const float* init_state,
                          int64_t chunk_len, int64_t R, const float* theta, float* y,
                          float* final_state, const ssd_launch_opts* opts, void* stream) {
    return ssd_detail::forward_impl(d, x, da, B, C, D, init_state, chunk_len, R, theta, y,
                                    final_state, opts, stream, 0);
}

}  // extern "C"

namespace ssd_detail {

ssd_status forward_plan(const ssd_dims* d, const void* x, const float* da, const void* B,
                        const void* C, const float* D, const float* init_state, int64_t chunk_len,
                        int64_t R, const float* theta, float* y, float* final_state,
                        const ssd_launch_opts* opts, int ysub, FwdPlan* out) {
    if (!d || !x || !da || !B || !C || !y || !final_state) return SSD_ERR_NULL_ARG;
    if (ysub && (d->seqlen % 2)) return SSD_ERR_BAD_SHAPE;
    ssd_status st = check_shape(d, chunk_len, R, theta != nullptr);
    if (st != SSD_OK) return st;
    if (opts) {
        if (opts->segments < 0 || opts->block_slices < 0) return SSD_ERR_BAD_SHAPE;
        for (int i = 0; i < 2; ++i)
            if (opts->reserved[i] != 0) return SSD_ERR_BAD_SHAPE;
        if ((opts->walk_events[0] == nullptr) != (opts->walk_events[1] == nullptr)) return SSD_ERR_BAD_SHAPE;
    }
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(final_state, 16) || (init_state && !aligned(init_state, 16)) || !aligned(da, 4) ||
        (D && !aligned(D, 4)) || (theta && !aligned(theta, 4)))
        return SSD_ERR_UNSUPPORTED;

    const int64_t b = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate,
                  G = d->ngroups;
    const int64_t esz = d->in_dtype == SSD_BF16 ? 2 : 4;
    const Span sy = span_of(y, (ysub ? b * T / 2 : b * T) * R * H * P * 4);
    const Span sf = span_of(final_state, b * H * P * N * 4);
    const Span ins[] = {span_of(x, b * T * R * H * P * esz), span_of(da, b * T * H * 4),
                        span_of(B, b * T * R * G * N * esz), span_of(C, b * T * R * G * N * esz),
                        D ? span_of(D, H * 4) : Span{0, 0},
                        init_state ? span_of(init_state, b * H * P * N * 4) : Span{0, 0},
                        theta ? span_of(theta, b * T * H * (N / 2) * 4) : Span{0, 0}};
    if (overlap(sy, sf)) return SSD_ERR_ALIAS;
    for (int i = 0; i < 7; ++i) {
        if (ins[i].hi == 0) continue;
        if (overlap(sy, ins[i])) return SSD_ERR_ALIAS;
        const bool same_state = (i == 5) && (const void*)final_state == (const void*)init_state;
        if (!same_state && overlap(sf, ins[i])) return SSD_ERR_ALIAS;
    }

    return forward_plan_shape(d, R, theta != nullptr, opts, ysub, out);
}

ssd_status forward_plan_shape(const ssd_dims* d, int64_t R, bool rot, const ssd_launch_opts* opts, int ysub,
                              FwdPlan* out) {
    FwdPlan fp;
    fp.rot = rot;
    ssd_status st = make_plan(d, R, fp.rot, opts ? opts->segments : 0, opts ? opts->block_slices : 0, &fp.pl);
    if (st != SSD_OK) return st;
    // column-block walk (C B^T tile pack shared by the heads of a group unless
    // rotated), or the general walk for shapes it does not cover
    fp.cols = fp.pl.kind == kColsPath;
    fp.shared = fp.cols && !fp.rot;
    if (fp.shared) {
        const void* pk = cb_pack_sel(fp.pl.dtype, (int)fp.pl.NP);
        if (!pk || fp.pl.b * fp.pl.G * fp.pl.nsub > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    }
    fp.ws_bytes = workspace_layout(fp.pl, !fp.shared).total;
    fp.ysub = ysub;
    *out = fp;
    return SSD_OK;
}

ssd_status forward_launch(const FwdPlan& fp, const void* x, const float* da, const void* B,
                          const void* C, const float* D, const float* init_state, const float* theta,
                          float* y, float* final_state, void* ws, void* const* walk_events,
                          hipStream_t hs, const TrapSrc* trap) {
    // the rotating column walk's odd-step output mode is the trapezoid's
    // sub-step walk, and the trapezoid's sources need that walk
    if ((trap != nullptr) != (fp.cols && fp.rot && fp.ysub != 0)) return SSD_ERR_UNSUPPORTED;
    const Plan& pl = fp.pl;
    const WsLayout wl = workspace_layout(pl, !fp.shared);
    char* wsc = static_cast<char*>(ws);
    float* ws_state = pl.S > 1 ? reinterpret_cast<float*>(wsc) : nullptr;
    float* ws_misc = pl.S > 1 ? reinterpret_cast<float*>(wsc + wl.state) : nullptr;
    float* ws_pack = fp.shared ? reinterpret_cast<float*>(wsc + wl.state + wl.misc) : nullptr;
    const int64_t T = pl.T, H = pl.H, G = pl.G, N = pl.N, R = pl.R, P = pl.P;

    ssd_status rs = SSD_OK;
    if (!fp.cols) {
        WalkArgs args;
        memset(&args, 0, sizeof(args));
        args.x = x; args.da = da; args.B = B; args.C = C; args.D = D;
        args.init = init_state; args.theta = theta; args.y = y; args.final_state = final_state;
        args.T = T; args.H = H; args.G = G; args.N = N; args.R = R;
        args.S = pl.S; args.nsub = pl.nsub; args.log2R = pl.log2R; args.Qt = pl.Qt;
        args.ws_state = ws_state; args.ws_misc = ws_misc;
        args.ysub = fp.ysub;
        rs = run_passes(pl, fp.rot, args, init_state, hs, walk_events);
    } else {
        // without rotation K2 runs once per (batch, group, tile), shared by
        // every head of the group; the rotating walk forms it per head
        if (fp.shared) {
            void* pk = cb_pack_sel(pl.dtype, (int)pl.NP);
            const int64_t ntiles = pl.b * pl.G * pl.nsub;
            const void* Bp = B;
            const void* Cp = C;
            int64_t TRv = T * R, Gv = G, Nv = N;
            int nsub = pl.nsub, l2r = pl.log2R;
            void* kargs[] = {(void*)&Bp, (void*)&Cp, (void*)&ws_pack, (void*)&TRv, (void*)&Gv, (void*)&Nv, (void*)&nsub, (void*)&l2r};
            if (hipLaunchKernel(pk, dim3((unsigned)ntiles), dim3(64), kargs, 0, hs) != hipSuccess) rs = SSD_ERR_HIP;
        }
        if (rs == SSD_OK) {
            TileArgs args;
            memset(&args, 0, sizeof(args));
            args.x = x; args.da = da; args.B = B; args.C = C; args.D = D;
            args.init = init_state; args.y = y; args.final_state = final_state;
            args.T = T; args.H = H; args.G = G; args.N = N; args.R = R; args.P = P;
            args.S = pl.S; args.nsub = pl.nsub; args.log2R = pl.log2R; args.Qt = pl.Qt;
            args.ws_state = ws_state; args.ws_misc = ws_misc; args.cbpack = ws_pack;
            args.theta = theta;
            args.NB = (int)((pl.H / pl.G) * (pl.P / 16) / pl.W);
            args.ysub = fp.ysub;
            if (trap) {
                args.scale = trap->scale;
                args.prev_x = trap->prev_x; args.prev_B = trap->prev_B;
            }
            rs = run_passes(pl, fp.rot, args, init_state, hs, walk_events);
        }
    }
    return rs;
}

ssd_status forward_impl(const ssd_dims* d, const void* x, const float* da, const void* B,
                        const void* C, const float* D, const float* init_state, int64_t chunk_len,
                        int64_t R, const float* theta, float* y, float* final_state,
                        const ssd_launch_opts* opts, void* stream, int ysub) {
    FwdPlan fp;
    ssd_status st = forward_plan(d, x, da, B, C, D, init_state, chunk_len, R, theta, y, final_state,
                                 opts, ysub, &fp);
    if (st != SSD_OK) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    void* ws = nullptr;
    int ws_entry = -1;
    if (fp.ws_bytes) {
        ws = scratch_acquire(hs, fp.ws_bytes, &ws_entry);
        if (!ws) return SSD_ERR_HIP;
    }
    ssd_status rs = forward_launch(fp, x, da, B, C, D, init_state, theta, y, final_state, ws,
                                   opts ? opts->walk_events : nullptr, hs);
    if (ws && !scratch_release(ws_entry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    return rs;
}

ssd_status states_plan(const ssd_dims* d, int64_t R, bool rot, Plan* pl, size_t* ws_bytes) {
    ssd_status st = make_plan(d, R, rot, 0, 0, pl);
    if (st != SSD_OK) return st;
    *ws_bytes = workspace_layout(*pl, true).total;
    return SSD_OK;
}

ssd_status states_launch(const Plan& pl, bool rot, const void* x, const float* da, const void* B,
                         const float* init_state, const float* theta, void* ws, hipStream_t hs,
                         float** ws_state) {
    const WsLayout wl = workspace_layout(pl, true);
    char* wsc = static_cast<char*>(ws);
    float* wstate = pl.S > 1 ? reinterpret_cast<float*>(wsc) : nullptr;
    float* wmisc = pl.S > 1 ? reinterpret_cast<float*>(wsc + wl.state) : nullptr;
    *ws_state = wstate;
    if (pl.S == 1) return SSD_OK;
    const int64_t T = pl.T, H = pl.H, G = pl.G, N = pl.N, R = pl.R, P = pl.P;
    if (pl.kind != kColsPath) {
        WalkArgs args;
        memset(&args, 0, sizeof(args));
        args.x = x; args.da = da; args.B = B; args.C = B;
        args.init = init_state; args.theta = theta;
        args.T = T; args.H = H; args.G = G; args.N = N; args.R = R;
        args.S = pl.S; args.nsub = pl.nsub; args.log2R = pl.log2R; args.Qt = pl.Qt;
        args.ws_state = wstate; args.ws_misc = wmisc;
        return run_state_passes(pl, rot, args, init_state, hs);
    }
    TileArgs args;
    memset(&args, 0, sizeof(args));
    args.x = x; args.da = da; args.B = B; args.C = B;
    args.init = init_state;
    args.T = T; args.H = H; args.G = G; args.N = N; args.R = R; args.P = P;
    args.S = pl.S; args.nsub = pl.nsub; args.log2R = pl.log2R; args.Qt = pl.Qt;
    args.ws_state = wstate; args.ws_misc = wmisc;
    args.theta = theta;
    args.NB = (int)((pl.H / pl.G) * (pl.P / 16) / pl.W);
    return run_state_passes(pl, rot, args, init_state, hs);
}

}  // namespace ssd_detail

extern "C" {

ssd_status ssd_forward(const ssd_dims* d, const void* x, const float* da, const void* B,
                       const void* C, const float* D, const float* init_state, int64_t chunk_len,
                       int64_t R, const float* theta, float* y, float* final_state, void* stream) {
    return ssd_forward_ex(d, x, da, B, C, D, init_state, chunk_len, R, theta, y, final_state,
                          nullptr, stream);
}


}  // extern "C"

// ---------------------------------------------------------------------------
// No-allocation entry point: the scratch is this fixed device array. Each GPU
// that runs the library holds its own copy at its own address; host code uses
// that address (looked up once per device), never the array's name.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_noalloc_mu;
constexpr int kMaxDevices = 64;
void* g_noalloc_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch` (looked up on the first
// call on each device); nullptr when the lookup fails.
void* noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_noalloc_ptr[dev] = ptr;
    }
    return g_noalloc_ptr[dev];
}

}  // namespace

extern "C" ssd_status ssd_forward_noalloc(const ssd_dims* d, const void* x, const float* da,
                                          const void* B, const void* C, const float* D,
                                          const float* init_state, int64_t chunk_len, int64_t R,
                                          const float* theta, float* y, float* final_state,
                                          const ssd_launch_opts* opts, void* stream) {
    ssd_detail::FwdPlan fp;
    ssd_status st = ssd_detail::forward_plan(d, x, da, B, C, D, init_state, chunk_len, R, theta, y,
                                             final_state, opts, 0, &fp);
    if (st != SSD_OK) return st;
    if (fp.ws_bytes > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
    void* ws = nullptr;
    if (fp.ws_bytes) {
        ws = noalloc_scratch();
        if (!ws) return SSD_ERR_HIP;
    }
    return ssd_detail::forward_launch(fp, x, da, B, C, D, init_state, theta, y, final_state, ws,
                                      opts ? opts->walk_events : nullptr,
                                      reinterpret_cast<hipStream_t>(stream));
}
