// Mamba-3 trapezoid (two-write) forward for AMD Instinct MI355X (gfx950).
//
// Per batch b and head h ("mamba3/scan.py", docstring and scan_forward, the
// Mamba-3 paper's eq. 11 as that code cites it; burn-mamba
// "mamba3/moments.rs", build_moments_input for the previous-token entries):
//   W_t = sum_r x_t (outer) B_t,   W_-1 from prev_x, prev_B (or zero)
//   h_t = R(theta_t) (exp(da_t) h_{t-1} + beta_t W_{t-1}) + gamma_t W_t
//   y_t = C_t h_t
// Every step splits into two sub-steps of the single-write scan:
//   2t    : decay exp(da_t), no rotation, write beta_t x_{t-1} (outer) B_{t-1}
//   2t+1  : no decay, rotation theta_t, write gamma_t x_t (outer) B_t, read C_t
// which gives h_{2t+1} = R(theta_t)(exp(da_t) h + beta_t W_{t-1}) + gamma_t W_t,
// exactly the step above. So the trapezoid runs as the single-write scan on a
// sequence of 2T sub-steps: B and C stay per group, the rotation and the
// chunked kernels are the SSD path's own. This file builds the sub-step
// inputs and calls the scan, which stores only the odd sub-steps' y.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ssd_common.h"

namespace {

using namespace ssd_detail;

// 16 bytes of x scaled by w: 8 bf16 or 4 fp32 lanes, rounded back to the
// stored type (bf16: round to nearest even)
__device__ __forceinline__ uint4 scale16(uint4 v, float w, bool bf) {
    uint32_t u[4] = {v.x, v.y, v.z, v.w};
    if (bf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(u[i] << 16) * w, hi = __uint_as_float(u[i] & 0xffff0000u) * w;
            const __bf16 l = (__bf16)lo, h = (__bf16)hi;
            u[i] = (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(__uint_as_float(u[i]) * w);
    }
    return make_uint4(u[0], u[1], u[2], u[3]);
}

// One workgroup per (batch, step) row; builds sub-steps 2t and 2t+1:
//   x^_{2t} = beta_t x_{t-1} (prev_x at t = 0),  x^_{2t+1} = gamma_t x_t
//   B^_{2t} = B_{t-1} (prev_B at t = 0),         B^_{2t+1} = B_t
//   C^_{2t} = C^_{2t+1} = C_t                    (sub-step 2t's y is not kept)
//   da^_{2t} = da_t, da^_{2t+1} = 0;  theta^_{2t} = 0, theta^_{2t+1} = theta_t
// x, B and C rows move in 16-byte vectors (rows are multiples of 32 bytes).
__global__ __launch_bounds__(256) void trap_expand_rows(TrapExpand a) {
    const int64_t bt = blockIdx.x;
    const int64_t bb = bt / a.T, t = bt - bb * a.T;
    const int64_t o = bb * 2 * a.T + 2 * t;            // row of sub-step 2t
    const bool bf = a.esz == 2;
    const int per = 16 / a.esz;                        // elements per vector
    // x
    const int64_t xrow = a.R * a.H * a.P, xv = xrow * a.esz / 16, hp = a.H * a.P;
    const uint4* x = static_cast<const uint4*>(a.x);
    const uint4* xprev = t > 0 ? x + (bt - 1) * xv : (a.prev_x ? static_cast<const uint4*>(a.prev_x) + bb * xv : nullptr);
    uint4* xh = static_cast<uint4*>(a.xh);
    for (int64_t j = threadIdx.x; j < xv; j += blockDim.x) {
        const int64_t h = ((j * per) % hp) / a.P;      // a vector never straddles two heads
        const float be = a.beta[bt * a.H + h], ga = a.gamma[bt * a.H + h];
        const uint4 cur = x[bt * xv + j];
        const uint4 prv = xprev ? xprev[j] : make_uint4(0, 0, 0, 0);
        xh[o * xv + j] = scale16(prv, be, bf);
        xh[(o + 1) * xv + j] = scale16(cur, ga, bf);
    }
    // B, C
    const int64_t bv = a.R * a.G * a.N * a.esz / 16;
    const uint4* B = static_cast<const uint4*>(a.B);
    const uint4* C = static_cast<const uint4*>(a.C);
    const uint4* bprev = t > 0 ? B + (bt - 1) * bv : (a.prev_B ? static_cast<const uint4*>(a.prev_B) + bb * bv : nullptr);
    uint4* Bh = static_cast<uint4*>(a.Bh);
    uint4* Ch = static_cast<uint4*>(a.Ch);
    for (int64_t j = threadIdx.x; j < bv; j += blockDim.x) {
        Bh[o * bv + j] = bprev ? bprev[j] : make_uint4(0, 0, 0, 0);
        Bh[(o + 1) * bv + j] = B[bt * bv + j];
        if (Ch) {
            const uint4 c = C[bt * bv + j];
            Ch[o * bv + j] = c;
            Ch[(o + 1) * bv + j] = c;
        }
    }
    // da, theta
    for (int64_t j = threadIdx.x; j < a.H; j += blockDim.x) {
        a.dah[o * a.H + j] = a.da[bt * a.H + j];
        a.dah[(o + 1) * a.H + j] = 0.f;
    }
    if (a.thh) {
        const int64_t tr = a.H * (a.N / 2);
        for (int64_t j = threadIdx.x; j < tr; j += blockDim.x) {
            a.thh[o * tr + j] = 0.f;
            a.thh[(o + 1) * tr + j] = a.theta[bt * tr + j];
        }
    }
}

// Per sub-step da and write scale of the trapezoid, for the rotating column
// walk, which stages x, B, C and theta from the source arrays itself: element
// (b, t, h) gives sub-steps 2t (da_t, beta_t) and 2t + 1 (0, gamma_t).
__global__ __launch_bounds__(256) void trap_da_scale(const float* __restrict__ da, const float* __restrict__ beta,
                                                    const float* __restrict__ gamma, float* __restrict__ dah,
                                                    float* __restrict__ sch, int64_t T, int64_t H, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t h = i % H, bt = i / H, t = bt % T, b = bt / T;
    const int64_t e = (b * 2 * T + 2 * t) * H + h, o = e + H;
    dah[e] = da[i];
    dah[o] = 0.f;
    sch[e] = beta[i];
    sch[o] = gamma[i];
}

}  // namespace

namespace ssd_detail {

size_t trap_expand_bytes(const TrapExpand& a) {
    const size_t nx = align256((size_t)(a.b * 2 * a.T * a.R * a.H * a.P) * a.esz);
    const size_t nbc = align256((size_t)(a.b * 2 * a.T * a.R * a.G * a.N) * a.esz);
    const size_t nda = align256((size_t)(a.b * 2 * a.T * a.H) * 4);
    const size_t nth = a.theta ? align256((size_t)(a.b * 2 * a.T * a.H * (a.N / 2)) * 4) : 0;
    return nx + (a.C ? 2 : 1) * nbc + nda + nth;
}

void trap_expand_setup(TrapExpand* a, void* ws) {
    char* w = static_cast<char*>(ws);
    const size_t nx = align256((size_t)(a->b * 2 * a->T * a->R * a->H * a->P) * a->esz);
    const size_t nbc = align256((size_t)(a->b * 2 * a->T * a->R * a->G * a->N) * a->esz);
    const size_t nda = align256((size_t)(a->b * 2 * a->T * a->H) * 4);
    a->xh = w;
    a->Bh = w + nx;
    a->Ch = a->C ? w + nx + nbc : nullptr;
    char* rest = w + nx + (a->C ? 2 : 1) * nbc;
    a->dah = reinterpret_cast<float*>(rest);
    a->thh = a->theta ? reinterpret_cast<float*>(rest + nda) : nullptr;
}

ssd_status trap_expand_launch(const TrapExpand& a, hipStream_t hs) {
    hipLaunchKernelGGL(trap_expand_rows, dim3((unsigned)(a.b * a.T)), dim3(256), 0, hs, a);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace ssd_detail

extern "C" {

ssd_status ssd_trapezoid_forward(const ssd_dims* d, const void* x, const float* da, const void* B,
                                 const void* C, const float* beta, const float* gamma,
                                 const void* prev_x, const void* prev_B, const float* init_state,
                                 int64_t chunk_len, int64_t R, const float* theta, float* y,
                                 float* final_state, const ssd_launch_opts* opts, void* stream) {
    if (!d || !x || !da || !B || !C || !beta || !gamma || !y || !final_state) return SSD_ERR_NULL_ARG;
    if ((prev_x == nullptr) != (prev_B == nullptr)) return SSD_ERR_NULL_ARG;
    ssd_status st = forward_shape_status(d, chunk_len, R, theta != nullptr);
    if (st != SSD_OK) return st;
    if (d->seqlen > ((int64_t)1 << 39) || d->batch * d->seqlen > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    ssd_dims d2 = *d;
    d2.seqlen = 2 * d->seqlen;
    st = forward_shape_status(&d2, chunk_len, R, theta != nullptr);
    if (st != SSD_OK) return st;
    if (opts) {
        if (opts->segments < 0 || opts->block_slices < 0) return SSD_ERR_BAD_SHAPE;
        for (int i = 0; i < 2; ++i)
            if (opts->reserved[i] != 0) return SSD_ERR_BAD_SHAPE;
        if ((opts->walk_events[0] == nullptr) != (opts->walk_events[1] == nullptr)) return SSD_ERR_BAD_SHAPE;
    }
    const int64_t b = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate,
                  G = d->ngroups;
    const int64_t esz = d->in_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(final_state, 16) || (init_state && !aligned(init_state, 16)))
        return SSD_ERR_UNSUPPORTED;
    if (!aligned(da, 4) || !aligned(beta, 4) || !aligned(gamma, 4) || (theta && !aligned(theta, 4)) ||
        (prev_x && !aligned(prev_x, 16)) || (prev_B && !aligned(prev_B, 16)))
        return SSD_ERR_UNSUPPORTED;
    const Span sy = span_of(y, b * T * R * H * P * 4);
    const Span sf = span_of(final_state, b * H * P * N * 4);
    const Span ins[] = {span_of(x, b * T * R * H * P * esz), span_of(da, b * T * H * 4),
                        span_of(B, b * T * R * G * N * esz), span_of(C, b * T * R * G * N * esz),
                        span_of(beta, b * T * H * 4), span_of(gamma, b * T * H * 4),
                        prev_x ? span_of(prev_x, b * R * H * P * esz) : Span{0, 0},
                        prev_B ? span_of(prev_B, b * R * G * N * esz) : Span{0, 0},
                        init_state ? span_of(init_state, b * H * P * N * 4) : Span{0, 0},
                        theta ? span_of(theta, b * T * H * (N / 2) * 4) : Span{0, 0}};
    if (overlap(sy, sf)) return SSD_ERR_ALIAS;
    for (const Span& si : ins) {
        if (overlap(sy, si)) return SSD_ERR_ALIAS;
        const bool same_init = init_state && si.lo == reinterpret_cast<uintptr_t>(init_state);
        if (!same_init && overlap(sf, si)) return SSD_ERR_ALIAS;
    }
    if (init_state && reinterpret_cast<const void*>(init_state) != reinterpret_cast<const void*>(final_state) &&
        overlap(sf, span_of(init_state, b * H * P * N * 4)))
        return SSD_ERR_ALIAS;

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    {
        // the rotating column walk stages the sub-steps from the source arrays
        // itself (write scales in fp32, nothing expanded through HBM)
        FwdPlan fp;
        ssd_status ps = forward_plan_shape(&d2, R, theta != nullptr, opts, 1, &fp);
        if (ps != SSD_OK) return ps;
        if (fp.cols && fp.rot) {
            // per sub-step da (da_t, 0) and write scale (beta_t, gamma_t)
            const size_t half = align256((size_t)(b * 2 * T * H) * 4);
            int sentry = -1;
            char* sws = static_cast<char*>(scratch_acquire(hs, 2 * half, &sentry, kSlotExpand));
            if (!sws) return SSD_ERR_HIP;
            void* fws = nullptr;
            int fentry = -1;
            ssd_status rs = SSD_OK;
            if (fp.ws_bytes) {
                fws = scratch_acquire(hs, fp.ws_bytes, &fentry);
                if (!fws) rs = SSD_ERR_HIP;
            }
            float* dah = reinterpret_cast<float*>(sws);
            float* sch = reinterpret_cast<float*>(sws + half);
            if (rs == SSD_OK) {
                const int64_t n = b * T * H;
                hipLaunchKernelGGL(trap_da_scale, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, hs, da, beta, gamma,
                                   dah, sch, T, H, n);
                if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
            }
            const TrapSrc ts{sch, prev_x, prev_B};
            if (rs == SSD_OK)
                rs = forward_launch(fp, x, dah, B, C, nullptr, init_state, theta, y, final_state, fws,
                                    opts ? opts->walk_events : nullptr, hs, &ts);
            if (fws && !scratch_release(fentry) && rs == SSD_OK) rs = SSD_ERR_HIP;
            if (!scratch_release(sentry) && rs == SSD_OK) rs = SSD_ERR_HIP;
            return rs;
        }
    }

    // other shapes: the sub-step inputs in the expansion slot
    TrapExpand a;
    memset(&a, 0, sizeof(a));
    a.x = x; a.da = da; a.B = B; a.C = C; a.beta = beta; a.gamma = gamma;
    a.prev_x = prev_x; a.prev_B = prev_B; a.theta = theta;
    a.b = b; a.T = T; a.R = R; a.H = H; a.P = P; a.G = G; a.N = N;
    a.esz = (int)esz;
    int entry = -1;
    void* ws = scratch_acquire(hs, trap_expand_bytes(a), &entry, kSlotExpand);
    if (!ws) return SSD_ERR_HIP;
    trap_expand_setup(&a, ws);

    // plan the scan over the 2T sub-steps (and take its scratch) before the
    // expansion is enqueued, so that a rejected plan launches nothing
    FwdPlan fp;
    ssd_status rs = forward_plan(&d2, a.xh, a.dah, a.Bh, a.Ch, nullptr, init_state, chunk_len, R,
                                 a.thh, y, final_state, opts, 1, &fp);
    void* fws = nullptr;
    int fentry = -1;
    if (rs == SSD_OK && fp.ws_bytes) {
        fws = scratch_acquire(hs, fp.ws_bytes, &fentry);
        if (!fws) rs = SSD_ERR_HIP;
    }
    if (rs == SSD_OK) rs = trap_expand_launch(a, hs);
    if (rs == SSD_OK)
        rs = forward_launch(fp, a.xh, a.dah, a.Bh, a.Ch, nullptr, init_state, a.thh, y, final_state,
                            fws, opts ? opts->walk_events : nullptr, hs);
    if (fws && !scratch_release(fentry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    if (!scratch_release(entry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    return rs;
}

}  // extern "C"
