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
// exactly the step above. So the trapezoid runs as ssd_forward_ex on a
// sequence of 2T sub-steps: B and C stay per group, the rotation and the
// chunked kernels are the SSD path's own. This file builds the sub-step
// inputs, calls the scan, and keeps the odd sub-steps' y.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ssd_common.h"

namespace {

using namespace ssd_detail;

__device__ __forceinline__ float load_as_f(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_as_f(const uint16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void store_from_f(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_from_f(uint16_t* p, int64_t i, float v) {
    const __bf16 h = (__bf16)v;                       // round to nearest even
    p[i] = __builtin_bit_cast(uint16_t, h);
}

struct ExpandArgs {
    const void* x;
    const float* da;
    const void* B;
    const void* C;
    const float* beta;
    const float* gamma;
    const void* prev_x;
    const void* prev_B;
    const float* theta;
    void* xh;        // [b][2T][R][H][P]
    float* dah;      // [b][2T][H]
    void* Bh;        // [b][2T][R][G][N]
    void* Ch;        // [b][2T][R][G][N]
    float* thh;      // [b][2T][H][N/2], or null
    int64_t b, T, R, H, P, G, N;
};

// x^: sub-step 2t takes beta_t x_{t-1} (prev_x at t = 0), 2t+1 takes gamma_t x_t
template <typename TI>
__global__ __launch_bounds__(256) void trap_expand_x(ExpandArgs a) {
    const int64_t row = a.R * a.H * a.P, hp = a.H * a.P;
    const int64_t total = a.b * a.T * row;
    const TI* x = static_cast<const TI*>(a.x);
    const TI* px = static_cast<const TI*>(a.prev_x);
    TI* xh = static_cast<TI*>(a.xh);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bt = i / row, e = i - bt * row;
        const int64_t bb = bt / a.T, t = bt - bb * a.T;
        const int64_t h = (e % hp) / a.P;
        const int64_t sh = bt * a.H + h;
        float prev = 0.f;
        if (t > 0) prev = load_as_f(x, i - row);
        else if (px) prev = load_as_f(px, bb * row + e);
        const int64_t o = (bb * 2 * a.T + 2 * t) * row + e;
        store_from_f(xh, o, a.beta[sh] * prev);
        store_from_f(xh, o + row, a.gamma[sh] * load_as_f(x, i));
    }
}

// B^, C^ (raw element copies): B^_{2t} = B_{t-1} (prev_B at t = 0),
// B^_{2t+1} = B_t, C^_{2t} = C^_{2t+1} = C_t (sub-step 2t's y is not kept)
template <typename TI>
__global__ __launch_bounds__(256) void trap_expand_bc(ExpandArgs a) {
    const int64_t row = a.R * a.G * a.N;
    const int64_t total = a.b * a.T * row;
    const TI* B = static_cast<const TI*>(a.B);
    const TI* C = static_cast<const TI*>(a.C);
    const TI* pB = static_cast<const TI*>(a.prev_B);
    TI* Bh = static_cast<TI*>(a.Bh);
    TI* Ch = static_cast<TI*>(a.Ch);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bt = i / row, e = i - bt * row;
        const int64_t bb = bt / a.T, t = bt - bb * a.T;
        TI prev = (TI)0;
        if (t > 0) prev = B[i - row];
        else if (pB) prev = pB[bb * row + e];
        const int64_t o = (bb * 2 * a.T + 2 * t) * row + e;
        const TI c = C[i];
        Bh[o] = prev;
        Bh[o + row] = B[i];
        Ch[o] = c;
        Ch[o + row] = c;
    }
}

// da^ and theta^: sub-step 2t decays by da_t without turning, 2t+1 turns by
// theta_t without decaying
__global__ __launch_bounds__(256) void trap_expand_da_theta(ExpandArgs a) {
    const int64_t K = a.N / 2;
    const int64_t total = a.b * a.T * a.H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bt = i / a.H, h = i - bt * a.H;
        const int64_t bb = bt / a.T, t = bt - bb * a.T;
        const int64_t o = (bb * 2 * a.T + 2 * t) * a.H + h;
        a.dah[o] = a.da[i];
        a.dah[o + a.H] = 0.f;
        if (a.thh) {
            for (int64_t k = 0; k < K; ++k) {
                a.thh[o * K + k] = 0.f;
                a.thh[(o + a.H) * K + k] = a.theta[i * K + k];
            }
        }
    }
}

// y_t = y^_{2t+1}; rows of R*H*P floats, a multiple of 4
__global__ __launch_bounds__(256) void trap_gather_y(const float4* yh, float4* y, int64_t b, int64_t T,
                                                     int64_t row4) {
    const int64_t total = b * T * row4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bt = i / row4, e = i - bt * row4;
        const int64_t bb = bt / T, t = bt - bb * T;
        y[i] = yh[(bb * 2 * T + 2 * t + 1) * row4 + e];
    }
}

unsigned grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    const int64_t cap = 256 * 64;     // grid-stride beyond 64 blocks per CU
    if (g > cap) g = cap;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

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
    if (d->seqlen > ((int64_t)1 << 39)) return SSD_ERR_UNSUPPORTED;
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
        (prev_x && !aligned(prev_x, (uintptr_t)esz)) || (prev_B && !aligned(prev_B, (uintptr_t)esz)))
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

    // sub-step inputs and the sub-step y in the expansion slot
    const size_t nx = align256((size_t)(b * 2 * T * R * H * P) * esz);
    const size_t nbc = align256((size_t)(b * 2 * T * R * G * N) * esz);
    const size_t nda = align256((size_t)(b * 2 * T * H) * 4);
    const size_t nth = theta ? align256((size_t)(b * 2 * T * H * (N / 2)) * 4) : 0;
    const size_t ny = align256((size_t)(b * 2 * T * R * H * P) * 4);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    int entry = -1;
    char* ws = static_cast<char*>(scratch_acquire(hs, nx + 2 * nbc + nda + nth + ny, &entry, kSlotExpand));
    if (!ws) return SSD_ERR_HIP;
    ExpandArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x; a.da = da; a.B = B; a.C = C; a.beta = beta; a.gamma = gamma;
    a.prev_x = prev_x; a.prev_B = prev_B; a.theta = theta;
    a.xh = ws;
    a.Bh = ws + nx;
    a.Ch = ws + nx + nbc;
    a.dah = reinterpret_cast<float*>(ws + nx + 2 * nbc);
    a.thh = theta ? reinterpret_cast<float*>(ws + nx + 2 * nbc + nda) : nullptr;
    float* yh = reinterpret_cast<float*>(ws + nx + 2 * nbc + nda + nth);
    a.b = b; a.T = T; a.R = R; a.H = H; a.P = P; a.G = G; a.N = N;

    ssd_status rs = SSD_OK;
    const bool bf = d->in_dtype == SSD_BF16;
    if (bf) {
        hipLaunchKernelGGL(trap_expand_x<uint16_t>, dim3(grid_for(b * T * R * H * P)), dim3(256), 0, hs, a);
        hipLaunchKernelGGL(trap_expand_bc<uint16_t>, dim3(grid_for(b * T * R * G * N)), dim3(256), 0, hs, a);
    } else {
        hipLaunchKernelGGL(trap_expand_x<float>, dim3(grid_for(b * T * R * H * P)), dim3(256), 0, hs, a);
        hipLaunchKernelGGL(trap_expand_bc<float>, dim3(grid_for(b * T * R * G * N)), dim3(256), 0, hs, a);
    }
    hipLaunchKernelGGL(trap_expand_da_theta, dim3(grid_for(b * T * H)), dim3(256), 0, hs, a);
    if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
    if (rs == SSD_OK)
        rs = ssd_forward_ex(&d2, a.xh, a.dah, a.Bh, a.Ch, nullptr, init_state, chunk_len, R, a.thh, yh,
                            final_state, opts, stream);
    if (rs == SSD_OK) {
        const int64_t row4 = R * H * P / 4;
        hipLaunchKernelGGL(trap_gather_y, dim3(grid_for(b * T * row4)), dim3(256), 0, hs,
                           reinterpret_cast<const float4*>(yh), reinterpret_cast<float4*>(y), b, T, row4);
        if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
    }
    if (!scratch_release(entry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    return rs;
}

}  // extern "C"
