// Device code of the chunked SSD scan: the tile walks and the C B^T pack,
// as templates. Each translation unit that includes this file compiles only
// the instantiations it takes the address of (ssd_walk_*.hip, ssd_cols_*.hip);
// ssd_scan.hip uses the argument structs and constants for the host side.
#ifndef SSD_KERNELS_H
#define SSD_KERNELS_H

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ssd_common.h"

namespace {


using namespace ssd_detail;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kRows = 32;  // fused rows per tile

// ---------------------------------------------------------------------------
// element type helpers: TI = uint16_t (bf16 bits) or float
// ---------------------------------------------------------------------------
template <typename TI> struct Ops;

template <> struct Ops<uint16_t> {
    typedef bf16x8 frag;
    static constexpr int kPad = 8;  // 16 bytes of row padding in LDS
    __device__ static inline float to_f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
    __device__ static inline uint16_t from_f(float f) {
        __bf16 b = (__bf16)f;
        return __builtin_bit_cast(uint16_t, b);
    }
    // 8 contiguous elements
    __device__ static inline frag ld8(const uint16_t* p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
    }
    // elements p[0..3] and p[16..19]
    __device__ static inline frag ld4x2(const uint16_t* p) {
        uint2 a = *reinterpret_cast<const uint2*>(p);
        uint2 b = *reinterpret_cast<const uint2*>(p + 16);
        uint4 v = make_uint4(a.x, a.y, b.x, b.y);
        return __builtin_bit_cast(frag, v);
    }
    __device__ static inline void unpack(frag f, float* o) {
        uint4 v = __builtin_bit_cast(uint4, f);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static inline frag pack(const float* v) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (__bf16)v[i];
        return f;
    }
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Ops<float> {
    typedef f32x8 frag;
    static constexpr int kPad = 4;
    __device__ static inline float to_f(float v) { return v; }
    __device__ static inline float from_f(float f) { return f; }
    __device__ static inline frag ld8(const float* p) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        frag f = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        return f;
    }
    __device__ static inline frag ld4x2(const float* p) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 16);
        frag f = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        return f;
    }
    __device__ static inline void unpack(frag f, float* o) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = f[i];
    }
    __device__ static inline frag pack(const float* v) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = v[i];
        return f;
    }
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
};

// State row permutation. State tile t (16 rows) holds, in accumulator row
// rho = 4*q + v, the state index n = phi(t, rho). With this order the two
// tiles 2s and 2s+1 of one lane form, slot for slot, the standard reduction
// layout of n in [32s, 32s+32): slot e of lane group q is n = 32s + 8q + e.
__device__ __forceinline__ int phi_row(int t, int rho) {
    return 32 * (t >> 1) + 8 * (rho >> 2) + 4 * (t & 1) + (rho & 3);
}

// Workgroups are dispatched round-robin over the 8 XCDs. Give each XCD a
// contiguous range of work items so that heads sharing B/C tiles (same batch,
// segment and group) share one L2.
__device__ __forceinline__ int xcd_item(int wg, int nwg) {
    const int q = nwg >> 3, r = nwg & 7;
    const int xcd = wg & 7, j = wg >> 3;
    return (xcd < r) ? xcd * (q + 1) + j : r * (q + 1) + (xcd - r) * q + j;
}

struct WalkArgs {
    const void* x;
    const float* da;
    const void* B;
    const void* C;
    const float* D;
    const float* init;     // segment-0 initial state [b,H,P,N] or null
    const float* theta;    // [b,T,H,N/2] or null
    float* y;
    float* final_state;
    float* ws_state;       // [b*H][S][P][N] segment states / carries
    float* ws_misc;        // [b*H][S][1 + N/2]: Lambda, Phi per pair
    int64_t T, H, G, N, R;
    int S;                 // segments of this launch's division of the sequence
    int seg_items;         // segments this launch covers
    int SF;                // output pass: state-pass segments per segment
    int nsub;              // tiles per sequence
    int log2R;
    int Qt;                // time steps per tile (32 / R)
    int ysub;              // 1: y keeps only the odd time steps, as step (t - 1) / 2
};

// ---------------------------------------------------------------------------
// The tile walk. MODE 0: output pass (y, final state). MODE 1: state-only
// pass (segment end states for the carry).
// ---------------------------------------------------------------------------
template <typename TI, int P, int NP, bool ROT, int MODE>
__global__ __launch_bounds__(4 * P) void ssd_walk_kernel(WalkArgs a) {
    using O = Ops<TI>;
    typedef typename O::frag frag;
    constexpr int W = P / 16;          // waves
    constexpr int NT = 64 * W;         // threads
    constexpr int F = kRows;
    constexpr int PAD = O::kPad;
    constexpr int LDR = NP + PAD;      // row-major tile row stride (elements)
    constexpr int LDT = F + PAD;       // transposed tile row stride
    constexpr int NTILE = NP / 16;     // state tiles per wave
    constexpr int KS = NP / 32;        // reduction steps over n
    constexpr bool OUT = (MODE == 0);

    __shared__ __attribute__((aligned(16))) TI sC[OUT ? F * LDR : 1];
    __shared__ __attribute__((aligned(16))) TI sB[OUT ? F * LDR : 1];
    __shared__ __attribute__((aligned(16))) TI sBt[NP * LDT];
    __shared__ __attribute__((aligned(16))) TI sXt[P * LDT];
    __shared__ float sCum[F], sEin[F], sW[F], sCarry[1];
    __shared__ float sPhi[ROT ? NP / 2 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int q = lane >> 4, l16 = lane & 15;
    const int p0 = wv * 16;

    const int64_t T = a.T, H = a.H, N = a.N, R = a.R;
    const int S = a.S;
    const int nwg = gridDim.x;
    const int item = xcd_item(blockIdx.x, nwg);
    const int h = (int)(item % H);
    const int bs = (int)(item / H);
    const int seg = bs % a.seg_items;
    const int b = bs / a.seg_items;
    const int64_t grp = h / (H / a.G);
    const int64_t bh = (int64_t)b * H + h;
    const int k0 = (int)(((int64_t)seg * a.nsub) / S);
    const int k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    const int64_t TR = T * R;
    const int log2R = a.log2R;
    const int Qt = a.Qt;

    const TI* xg = static_cast<const TI*>(a.x);
    const TI* Bg = static_cast<const TI*>(a.B);
    const TI* Cg = static_cast<const TI*>(a.C);

    // ---- initial state (physical; the segment's rotation frame starts at 0)
    f32x4 hs[NTILE];
    {
        // S == 1: the caller's initial state. S > 1: the carry pass has stored
        // the state entering every segment (segment 0 included) in ws slot seg,
        // so init_state is never read here and may alias final_state.
        const float* src = nullptr;
        if (OUT) {
            if (S == 1)
                src = a.init ? a.init + bh * P * N : nullptr;
            else
                src = a.ws_state + (bh * S + seg) * a.SF * P * N;
        }
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = phi_row(t, 4 * q + v);
                hs[t][v] = (src && n < N) ? src[(int64_t)(p0 + l16) * N + n] : 0.f;
            }
        }
    }

    const float Dh = (OUT && a.D) ? a.D[h] : 0.f;
    float lam = 0.f;  // sum of da over the segment (wave 0, lane 0)

    // ---- staging registers (non-rotated B/C and x are prefetched one tile ahead)
    constexpr int XU = (sizeof(TI) == 2) ? 16 * (P / 4) : F * (P / 4);         // x units
    constexpr int XPT = (XU + NT - 1) / NT;
    constexpr int BU = (sizeof(TI) == 2) ? 16 * (NP / 4) : F * (NP / 4);       // B units
    constexpr int BPT = (BU + NT - 1) / NT;
    constexpr int CU = F * NP * (int)sizeof(TI) / 16;                           // C 16B units
    constexpr int CPT = (CU + NT - 1) / NT;
    uint4 rx[XPT];
    uint4 rb[ROT ? 1 : BPT];
    uint4 rc[(ROT || !OUT) ? 1 : CPT];
    float rda = 0.f;

    // rotation bookkeeping: slot = (pair block of 16, time group of Qt/4)
    constexpr int RSLOTS = (NP / 2) * 4;
    constexpr int RPT = ROT ? (RSLOTS + NT - 1) / NT : 1;
    float phib[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) phib[m] = 0.f;

    auto row_x = [&](int64_t fr) -> const TI* { return xg + ((b * TR + fr) * H + h) * P; };
    auto row_bc = [&](const TI* base, int64_t fr) -> const TI* { return base + ((b * TR + fr) * a.G + grp) * N; };

    auto stage_load = [&](int k) {
        const int64_t fbase = (int64_t)k * F;
#pragma unroll
        for (int m = 0; m < XPT; ++m) {
            const int u = tid + m * NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (u < XU) {
                if (sizeof(TI) == 2) {
                    const int ra = u / (P / 4), c = u % (P / 4);
                    const int64_t f0 = fbase + 2 * ra;
                    if (f0 < TR) {
                        uint2 lo = *reinterpret_cast<const uint2*>(row_x(f0) + 4 * c);
                        v.x = lo.x; v.y = lo.y;
                    }
                    if (f0 + 1 < TR) {
                        uint2 hi = *reinterpret_cast<const uint2*>(row_x(f0 + 1) + 4 * c);
                        v.z = hi.x; v.w = hi.y;
                    }
                } else {
                    const int f = u / (P / 4), c = u % (P / 4);
                    if (fbase + f < TR) v = *reinterpret_cast<const uint4*>(row_x(fbase + f) + 4 * c);
                }
            }
            rx[m] = v;
        }
        if (!ROT) {
#pragma unroll
            for (int m = 0; m < BPT; ++m) {
                const int u = tid + m * NT;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (u < BU) {
                    if (sizeof(TI) == 2) {
                        const int ra = u / (NP / 4), c = u % (NP / 4);
                        const int64_t f0 = fbase + 2 * ra;
                        if (4 * c < N) {
                            if (f0 < TR) {
                                uint2 lo = *reinterpret_cast<const uint2*>(row_bc(Bg, f0) + 4 * c);
                                v.x = lo.x; v.y = lo.y;
                            }
                            if (f0 + 1 < TR) {
                                uint2 hi = *reinterpret_cast<const uint2*>(row_bc(Bg, f0 + 1) + 4 * c);
                                v.z = hi.x; v.w = hi.y;
                            }
                        }
                    } else {
                        const int f = u / (NP / 4), c = u % (NP / 4);
                        if (4 * c < N && fbase + f < TR)
                            v = *reinterpret_cast<const uint4*>(row_bc(Bg, fbase + f) + 4 * c);
                    }
                }
                rb[m] = v;
            }
            if (OUT) {
                constexpr int EPU = 16 / (int)sizeof(TI);   // elements per 16B unit
#pragma unroll
                for (int m = 0; m < CPT; ++m) {
                    const int u = tid + m * NT;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (u < CU) {
                        const int f = u / (NP / EPU), c = u % (NP / EPU);
                        if (EPU * c < N && fbase + f < TR)
                            v = *reinterpret_cast<const uint4*>(row_bc(Cg, fbase + f) + EPU * c);
                    }
                    rc[m] = v;
                }
            }
        }
        if (wv == 0) {
            const int64_t t = (int64_t)k * Qt + lane;
            rda = (lane < Qt && t < T) ? a.da[(b * T + t) * H + h] : 0.f;
        }
    };

    auto stage_store = [&](int k) {
        // x -> sXt (transposed: p rows, fused-row columns)
#pragma unroll
        for (int m = 0; m < XPT; ++m) {
            const int u = tid + m * NT;
            if (u < XU) {
                const uint4 v = rx[m];
                if (sizeof(TI) == 2) {
                    const int ra = u / (P / 4), c = u % (P / 4);
                    uint32_t* d0 = reinterpret_cast<uint32_t*>(sXt + (4 * c) * LDT + 2 * ra);
                    const uint32_t lo[2] = {v.x, v.y}, hi[2] = {v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wl = lo[e >> 1], wh = hi[e >> 1];
                        const uint32_t pr = (e & 1) ? ((wl >> 16) | (wh & 0xffff0000u))
                                                    : ((wl & 0xffffu) | (wh << 16));
                        *reinterpret_cast<uint32_t*>(reinterpret_cast<TI*>(d0) + e * LDT) = pr;
                    }
                } else {
                    const int f = u / (P / 4), c = u % (P / 4);
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<uint32_t*>(sXt + (4 * c + e) * LDT + f) = w4[e];
                }
            }
        }
        if (!ROT) {
#pragma unroll
            for (int m = 0; m < BPT; ++m) {
                const int u = tid + m * NT;
                if (u < BU) {
                    const uint4 v = rb[m];
                    if (sizeof(TI) == 2) {
                        const int ra = u / (NP / 4), c = u % (NP / 4);
                        if (OUT) {
                            *reinterpret_cast<uint2*>(sB + (2 * ra) * LDR + 4 * c) = make_uint2(v.x, v.y);
                            *reinterpret_cast<uint2*>(sB + (2 * ra + 1) * LDR + 4 * c) = make_uint2(v.z, v.w);
                        }
                        const uint32_t lo[2] = {v.x, v.y}, hi[2] = {v.z, v.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t wl = lo[e >> 1], wh = hi[e >> 1];
                            const uint32_t pr = (e & 1) ? ((wl >> 16) | (wh & 0xffff0000u))
                                                        : ((wl & 0xffffu) | (wh << 16));
                            *reinterpret_cast<uint32_t*>(sBt + (4 * c + e) * LDT + 2 * ra) = pr;
                        }
                    } else {
                        const int f = u / (NP / 4), c = u % (NP / 4);
                        if (OUT) *reinterpret_cast<uint4*>(sB + f * LDR + 4 * c) = v;
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            *reinterpret_cast<uint32_t*>(sBt + (4 * c + e) * LDT + f) = w4[e];
                    }
                }
            }
            if (OUT) {
                constexpr int EPU = 16 / (int)sizeof(TI);
#pragma unroll
                for (int m = 0; m < CPT; ++m) {
                    const int u = tid + m * NT;
                    if (u < CU) {
                        const int f = u / (NP / EPU), c = u % (NP / EPU);
                        *reinterpret_cast<uint4*>(sC + f * LDR + EPU * c) = rc[m];
                    }
                }
            }
        } else {
            // Rotated B (and C): per (pair k, time group) slot, a prefix sum of
            // theta over the group's steps, a cross-group scan by shuffles, then
            // B~ = R(-Phi) B, C~ = R(-Phi) C for every rank of those steps.
            const int64_t fbase = (int64_t)k * F;
            const int TPG = (Qt + 3) / 4;
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int slot = tid + m * NT;
                const int kk = (slot >> 6) * 16 + (slot & 15);
                const int tg = (slot & 63) >> 4;
                const bool kvalid = (slot < RSLOTS) && (2 * kk < N);
                float part[8];
                float run = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tl = tg * TPG + j;
                    const int64_t t = (int64_t)k * Qt + tl;
                    float th = 0.f;
                    if (j < TPG && tl < Qt && t < T && kvalid)
                        th = a.theta[((b * T + t) * H + h) * (N / 2) + kk];
                    run += th;
                    part[j] = run;
                }
                // inclusive scan of group totals across the 4 groups of this block
                float tot = run;
                float u1 = __shfl_up(tot, 16);
                if (tg >= 1) tot += u1;
                float u2 = __shfl_up(tot, 32);
                if (tg >= 2) tot += u2;
                const float excl = tot - run;
                const float all = __shfl(tot, (lane & 15) + 48);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tl = tg * TPG + j;
                    if (j < TPG && tl < Qt && slot < RSLOTS && kk < NP / 2) {
                        float sn = 0.f, cs = 1.f;
                        if (kvalid) sincosf(phib[m] + excl + part[j], &sn, &cs);
                        for (int r = 0; r < (int)R; ++r) {
                            const int f = tl * (int)R + r;
                            const int64_t fr = fbase + f;
                            float b0 = 0.f, b1 = 0.f, c0 = 0.f, c1 = 0.f;
                            if (kvalid && fr < TR) {
                                const TI* pb = row_bc(Bg, fr) + 2 * kk;
                                b0 = O::to_f(pb[0]); b1 = O::to_f(pb[1]);
                                if (OUT) {
                                    const TI* pc = row_bc(Cg, fr) + 2 * kk;
                                    c0 = O::to_f(pc[0]); c1 = O::to_f(pc[1]);
                                }
                            }
                            // R(-phi): (a, b) -> (cos a + sin b, -sin a + cos b)
                            const TI rb0 = O::from_f(cs * b0 + sn * b1);
                            const TI rb1 = O::from_f(cs * b1 - sn * b0);
                            sBt[(2 * kk) * LDT + f] = rb0;
                            sBt[(2 * kk + 1) * LDT + f] = rb1;
                            if (OUT) {
                                sB[f * LDR + 2 * kk] = rb0;
                                sB[f * LDR + 2 * kk + 1] = rb1;
                                sC[f * LDR + 2 * kk] = O::from_f(cs * c0 + sn * c1);
                                sC[f * LDR + 2 * kk + 1] = O::from_f(cs * c1 - sn * c0);
                            }
                        }
                    }
                }
                phib[m] += all;
            }
        }
        // K1: inclusive prefix of da over the tile's time steps (wave 0)
        if (wv == 0) {
            float v = rda;
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
                const float u = __shfl_up(v, o);
                if (lane >= o) v += u;
            }
            const float last = __shfl(v, Qt - 1);
            const float cf = __shfl(v, (lane & 31) >> log2R);
            if (lane < F) {
                sCum[lane] = cf;
                sEin[lane] = __expf(cf);
                sW[lane] = __expf(last - cf);
            }
            if (lane == 0) {
                sCarry[0] = __expf(last);
                lam += last;
            }
        }
    };

    // ---- the walk
    stage_load(k0);
    stage_store(k0);
    __syncthreads();
    for (int k = k0; k < k1; ++k) {
        if (k + 1 < k1) stage_load(k + 1);

        if (OUT) {
            // K5 off-diagonal term and K2 tiles, one reduction step over n at a time
            f32x4 yacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            f32x4 cb00 = {0.f, 0.f, 0.f, 0.f}, cb01 = cb00, cb11 = cb00;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float hv[8];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    hv[v] = hs[2 * s][v];
                    hv[4 + v] = hs[2 * s + 1][v];
                }
                const frag hA = O::pack(hv);
                const frag c0 = O::ld8(sC + (l16) * LDR + 32 * s + 8 * q);
                const frag c1 = O::ld8(sC + (16 + l16) * LDR + 32 * s + 8 * q);
                const frag b0 = O::ld8(sB + (l16) * LDR + 32 * s + 8 * q);
                const frag b1 = O::ld8(sB + (16 + l16) * LDR + 32 * s + 8 * q);
                yacc[0] = O::mma(hA, c0, yacc[0]);
                yacc[1] = O::mma(hA, c1, yacc[1]);
                cb00 = O::mma(b0, c0, cb00);
                cb01 = O::mma(b0, c1, cb01);
                cb11 = O::mma(b1, c1, cb11);
            }
            // exp(cum_i) on the off-diagonal term (column i of y^T)
            {
                const float e0 = sEin[l16], e1 = sEin[16 + l16];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    yacc[0][v] *= e0;
                    yacc[1][v] *= e1;
                }
            }
            // decay matrix L o CB^T: element (j = 16J + 4q + v, i = 16I + l16)
            float m00[4], m01[4], m11[4];
            {
                const float ci0 = sCum[l16], ci1 = sCum[16 + l16];
                const int ti0 = l16 >> log2R, ti1 = (16 + l16) >> log2R;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j0 = 4 * q + v, j1 = 16 + 4 * q + v;
                    const float cj0 = sCum[j0], cj1 = sCum[j1];
                    const int tj0 = j0 >> log2R, tj1 = j1 >> log2R;
                    m00[v] = (ti0 >= tj0) ? cb00[v] * __expf(ci0 - cj0) : 0.f;
                    m01[v] = (ti1 >= tj0) ? cb01[v] * __expf(ci1 - cj0) : 0.f;
                    m11[v] = (ti1 >= tj1) ? cb11[v] * __expf(ci1 - cj1) : 0.f;
                    if (j0 == l16) m00[v] += Dh;
                    if (j1 == 16 + l16) m11[v] += Dh;
                }
            }
            // K5 diagonal block: y^T[p, i] += sum_j x^T[p, j] (L o CB^T)[j, i]
            {
                const frag xa = O::ld4x2(sXt + (p0 + l16) * LDT + 4 * q);
                float mv0[8], mv1[8];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    mv0[v] = m00[v];
                    mv0[4 + v] = 0.f;        // rows j >= 16 never reach i < 16
                    mv1[v] = m01[v];
                    mv1[4 + v] = m11[v];
                }
                yacc[0] = O::mma(xa, O::pack(mv0), yacc[0]);
                yacc[1] = O::mma(xa, O::pack(mv1), yacc[1]);
            }
            // store y: lane holds y[row i][p0 + 4q .. +3]
            const int64_t fbase = (int64_t)k * F;
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                const int64_t fr = fbase + 16 * I + l16;
                // with ysub, only odd steps are kept: row fr = t R + r goes to
                // ((t - 1) / 2) R + r of a y with T / 2 steps
                const int64_t st = fr >> log2R;
                if (fr < TR && (!a.ysub || (st & 1))) {
                    const int64_t yr = a.ysub ? (((st >> 1) << log2R) | (fr & ((1 << log2R) - 1))) : fr;
                    const int64_t ytr = a.ysub ? TR / 2 : TR;
                    float* dst = a.y + ((b * ytr + yr) * H + h) * P + p0 + 4 * q;
                    *reinterpret_cast<f32x4*>(dst) = yacc[I];
                }
            }
        }

        // K3 + K4: h <- exp(cum_last) h + sum_j w_j x_j (outer) B_j
        {
            const float carry = sCarry[0];
            float xv[8], wv8[8];
            O::unpack(O::ld8(sXt + (p0 + l16) * LDT + 8 * q), xv);
#pragma unroll
            for (int e = 0; e < 8; ++e) wv8[e] = sW[8 * q + e];
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[e] *= wv8[e];
            const frag xw = O::pack(xv);
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
#pragma unroll
                for (int v = 0; v < 4; ++v) hs[t][v] *= carry;
                const frag bt = O::ld8(sBt + phi_row(t, l16) * LDT + 8 * q);
                hs[t] = O::mma(bt, xw, hs[t]);
            }
        }

        __syncthreads();
        if (k + 1 < k1) {
            stage_store(k + 1);
            __syncthreads();
        }
    }

    // ---- epilogue: rotate the state back to the physical frame
    if (ROT) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int slot = tid + m * NT;
            const int kk = (slot >> 6) * 16 + (slot & 15);
            const int tg = (slot & 63) >> 4;
            if (slot < RSLOTS && tg == 0 && kk < NP / 2) sPhi[kk] = phib[m];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int v = 0; v < 4; v += 2) {
                const int n = phi_row(t, 4 * q + v);   // even: pair (n, n+1)
                float sn, cs;
                sincosf(sPhi[n >> 1], &sn, &cs);
                const float g0 = hs[t][v], g1 = hs[t][v + 1];
                hs[t][v] = cs * g0 - sn * g1;
                hs[t][v + 1] = sn * g0 + cs * g1;
            }
        }
    }
    float* dstate = nullptr;
    if (OUT) {
        if (seg == S - 1) dstate = a.final_state + bh * P * N;
    } else {
        dstate = a.ws_state + (bh * S + seg + 1) * P * N;
        float* misc = a.ws_misc + (bh * S + seg) * (1 + N / 2);
        if (tid == 0) misc[0] = lam;
        if (ROT) {
            for (int kk = tid; kk < N / 2; kk += NT) misc[1 + kk] = sPhi[kk];
        }
    }
    if (dstate) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = phi_row(t, 4 * q + v);
                if (n < N) dstate[(int64_t)(p0 + l16) * N + n] = hs[t][v];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Shared-B/C path (no rotation): B and C do not depend on the head, so the
// K2 product C B^T of every tile is computed once per (batch, group, tile) by
// ssd_cb_pack_kernel and reused by all heads of the group. The tile walk then
// only stages row-major x, B, C tiles; operands that run along time (x^T, B^T)
// come from the LDS transpose read (ds_read_b64_tr_b16).
// ---------------------------------------------------------------------------

// One wave per (batch, group, tile): CB^T for the three 16x16 blocks
// (J, I) = (0,0), (0,1), (1,1) of the 32x32 tile, K = N, stored in
// accumulator lane order: pack[tile][blk][lane][4] (fp32).
template <typename TI, int NP>
__global__ __launch_bounds__(64) void ssd_cb_pack_kernel(const void* __restrict__ Bv,
                                                         const void* __restrict__ Cv,
                                                         float* __restrict__ pack, int64_t TR,
                                                         int64_t G, int64_t N, int nsub, int log2R) {
    using O = Ops<TI>;
    typedef typename O::frag frag;
    constexpr int KS = NP / 32;
    const TI* Bg = static_cast<const TI*>(Bv);
    const TI* Cg = static_cast<const TI*>(Cv);
    const int lane = threadIdx.x, q = lane >> 4, l16 = lane & 15;
    const int64_t tile = blockIdx.x;                  // (b*G + g)*nsub + k
    const int64_t bg = tile / nsub;
    const int k = (int)(tile % nsub);
    const int64_t b = bg / G, g = bg % G;
    const int64_t f0 = (int64_t)k * kRows;
    auto row = [&](const TI* base, int r) -> const TI* { return base + ((b * TR + f0 + r) * G + g) * N; };
    const bool ok0 = f0 + l16 < TR, ok1 = f0 + 16 + l16 < TR;
    f32x4 c00 = {0.f, 0.f, 0.f, 0.f}, c01 = c00, c11 = c00;
    const frag zero = O::pack((const float[8]){0, 0, 0, 0, 0, 0, 0, 0});
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int n = 32 * s + 8 * q;
        const bool nok = n < N;
        const frag b0 = (ok0 && nok) ? O::ld8(row(Bg, l16) + n) : zero;
        const frag b1 = (ok1 && nok) ? O::ld8(row(Bg, 16 + l16) + n) : zero;
        const frag c0 = (ok0 && nok) ? O::ld8(row(Cg, l16) + n) : zero;
        const frag c1 = (ok1 && nok) ? O::ld8(row(Cg, 16 + l16) + n) : zero;
        c00 = O::mma(b0, c0, c00);
        c01 = O::mma(b0, c1, c01);
        c11 = O::mma(b1, c1, c11);
    }
    // causal block mask (step(i) >= step(j)), applied here so that the walk
    // multiplies by exp2(min(cum_i - cum_j, 0)) without a compare
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        if ((l16 >> log2R) < ((4 * q + v) >> log2R)) c00[v] = 0.f;
        if (((16 + l16) >> log2R) < ((16 + 4 * q + v) >> log2R)) c11[v] = 0.f;
    }
    f32x4* dst = reinterpret_cast<f32x4*>(pack + tile * 768) + lane;
    dst[0] = c00;
    dst[64] = c01;
    dst[128] = c11;
}

struct TileArgs {
    const void* x;
    const float* da;
    const void* B;
    const void* C;
    const float* D;
    const float* init;
    float* y;
    float* final_state;
    float* ws_state;
    float* ws_misc;
    const float* cbpack;   // from ssd_cb_pack_kernel (output pass without rotation)
    const float* theta;    // [b,T,H,N/2] or null (rotation walk only)
    int64_t T, H, G, N, R, P;
    int S, seg_items, nsub, log2R, Qt;
    int SF;                // output pass: state-pass segments per segment
    int NB;                // column blocks per B/C group
    int ysub;              // 1: y keeps only the odd time steps, as step (t - 1) / 2
    // trapezoid sub-steps (the rotating walk with YS): T counts sub-steps;
    // x, B, C, theta have T / 2 steps, and sub-step s takes x and B of step
    // (s - 1) >> 1 (prev_x, prev_B before step 0), C of step s >> 1 and theta
    // on odd sub-steps; da and the write scale (beta on even, gamma on odd
    // sub-steps) come per sub-step in da and scale
    const float* scale;    // [b,T,H]
    const void* prev_x;    // [b,R,H,P] or null
    const void* prev_B;    // [b,R,G,N] or null
};

// Operand whose reduction index runs down the rows of a row-major LDS tile:
// lane (q, i) receives rows r0+q4 .. r0+q4+3 and r1+q4 .. r1+q4+3 (q4 = 4q)
// of column col(i) = cb(i >> 2) + (i & 3). bf16: two ds_read_b64_tr_b16, where
// within each 16-lane group lane s reads 4 elements at row r + (s >> 2),
// column cb(s & 3). fp32: eight single-element reads.
template <typename TI> struct RowRuns;

template <> struct RowRuns<uint16_t> {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    __device__ static inline bf16x8 load(const uint16_t* tile, int ld, int r0, int r1, int cb_src,
                                         int /*col_own*/, int lane) {
        const int s = lane & 15;
        const uint16_t* p0 = tile + (r0 + (s >> 2)) * ld + cb_src;
        const uint16_t* p1 = tile + (r1 + (s >> 2)) * ld + cb_src;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    }
};

template <> struct RowRuns<float> {
    __device__ static inline f32x8 load(const float* tile, int ld, int r0, int r1, int /*cb_src*/,
                                        int col_own, int /*lane*/) {
        f32x8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = tile[(r0 + e) * ld + col_own];
            f[4 + e] = tile[(r1 + e) * ld + col_own];
        }
        return f;
    }
};

// Row stride (elements) of a row-major LDS tile whose transposed operands are
// read by row runs: a 16-lane group reads 4 consecutive rows, each at column
// offsets {0, 8, 16, 24} + {0..3} elements of one 32-column block. Pick the
// smallest padding (a multiple of 16 bytes) for which those 4 row slices fall
// in distinct 4-byte banks of the 64-bank LDS.
template <typename TI>
constexpr int tr_row_stride(int ncols) {
    constexpr int esz = (int)sizeof(TI);
    const int row_dw = ncols * esz / 4;
    for (int pad16 = 0; pad16 < 16; ++pad16) {
        const int sdw = row_dw + 4 * pad16;
        bool used[64] = {};
        bool ok = true;
        for (int r = 0; r < 4 && ok; ++r)
            for (int c = 0; c < 4 && ok; ++c)
                for (int w = 0; w < 2 * (esz == 2 ? 1 : 2) && ok; ++w) {
                    const int bank = (r * sdw + (8 * c * esz) / 4 + w) & 63;
                    if (used[bank]) ok = false;
                    used[bank] = true;
                }
        if (ok) return ncols + pad16 * 16 / esz;
    }
    return ncols + 16 / esz;
}

// Row stride (elements) of the rotating walk's B tile, which is read both by
// row runs (as for tr_row_stride) and along rows as 8-byte halves of 16-byte
// fragments (the head's C B^T blocks), and written that way: the smallest
// stride whose row runs fall in distinct banks and whose byte stride is 8
// modulo 16 (the class that serves row reads without bank conflicts, as for
// c_row_stride).
template <typename TI>
constexpr int rot_b_row_stride(int ncols) {
    constexpr int esz = (int)sizeof(TI);
    const int row_dw = ncols * esz / 4;
    for (int pad = 2; pad < 64; pad += 4) {
        const int sdw = row_dw + pad;
        bool used[64] = {};
        bool ok = true;
        for (int r = 0; r < 4 && ok; ++r)
            for (int c = 0; c < 4 && ok; ++c)
                for (int w = 0; w < 2 * (esz == 2 ? 1 : 2) && ok; ++w) {
                    const int bank = (r * sdw + (8 * c * esz) / 4 + w) & 63;
                    if (used[bank]) ok = false;
                    used[bank] = true;
                }
        if (ok) return ncols + pad * 4 / esz;
    }
    return ncols + 8 / esz;
}

// Row stride (elements) of the per-head x tile of the grouped walk, read as
// the x^T operand by row runs starting at 16-column slices: bf16 lanes of one
// 16-lane group read 4 consecutive rows, 8 dwords each; fp32 lane groups read
// rows 4 apart, 16 dwords each. Smallest padding (a multiple of 16 bytes) that
// puts those row slices in distinct banks.
template <typename TI>
constexpr int x_row_stride(int ncols) {
    constexpr int esz = (int)sizeof(TI);
    const int row_dw = ncols * esz / 4;
    const int rstep = esz == 2 ? 1 : 4, width = esz == 2 ? 8 : 16;
    for (int pad16 = 0; pad16 < 16; ++pad16) {
        const int sdw = row_dw + 4 * pad16;
        bool used[64] = {};
        bool ok = true;
        for (int r = 0; r < 4 && ok; ++r)
            for (int w = 0; w < width && ok; ++w) {
                const int bank = (r * rstep * sdw + w) & 63;
                if (used[bank]) ok = false;
                used[bank] = true;
            }
        if (ok) return ncols + pad16 * 16 / esz;
    }
    return ncols + 16 / esz;
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row-15 broadcast); lanes 0..31 are the only ones used.
__device__ __forceinline__ float wave_prefix32(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    return v;
}

template <typename TI> struct MBlock;
template <> struct MBlock<uint16_t> { typedef uint2 type; };
template <> struct MBlock<float> { typedef float4 type; };

template <typename TI>
__device__ __forceinline__ typename MBlock<TI>::type pack_m(float a, float b, float c, float d) {
    if constexpr (sizeof(TI) == 2) {
        typedef __attribute__((ext_vector_type(2))) float f32x2;
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
        const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
        return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    } else {
        return make_float4(a, b, c, d);
    }
}

template <typename TI>
__device__ __forceinline__ typename Ops<TI>::frag join_m(typename MBlock<TI>::type lo,
                                                       typename MBlock<TI>::type hi) {
    if constexpr (sizeof(TI) == 2) {
        return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    } else {
        f32x8 f = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        return f;
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

constexpr float kInv2Pi = 0.15915494309189535f;

// phi - 2 pi k with k = round(phi / 2 pi): the running angle kept in
// [-pi, pi] so that its fp32 sums keep their absolute precision. 2 pi is split
// into a head with few significant bits (k * head is exact) and a tail
// (Cody and Waite's argument reduction).
__device__ __forceinline__ float wrap_angle(float phi) {
    const float k = rintf(phi * kInv2Pi);
    phi = fmaf(-k, 6.28125f, phi);
    return fmaf(-k, 1.9353071795864769e-3f, phi);
}


// ---------------------------------------------------------------------------
// Column-block tile walk (shared B/C, no rotation). Flatten each time row of
// x and y over (head, p) and cut the columns of one B/C group into slices of
// 16; a workgroup owns W consecutive slices (one wave each), possibly
// spanning several heads. Its x and y rows are then contiguous runs of 16 W
// columns, and the B, C and C B^T tiles it stages serve every head it touches.
// Wave w keeps the state columns p in [p0, p0 + 16) of its head h and scans
// that head's decays itself. y goes through LDS and leaves as whole rows of
// the block, one tile after it is computed.
// ---------------------------------------------------------------------------

// Row stride (floats) of the staged y block: eight consecutive rows written at
// one 16-byte column by the MFMA output layout fall in distinct banks.
constexpr int y_row_stride(int ncols) {
    for (int pad = 0; pad < 64; pad += 4) {
        const int s = ncols + pad;
        bool used[64] = {};
        bool ok = true;
        for (int r = 0; r < 8 && ok; ++r)
            for (int w = 0; w < 4 && ok; ++w) {
                const int bank = (r * s + w) & 63;
                if (used[bank]) ok = false;
                used[bank] = true;
            }
        if (ok) return s;
    }
    return ncols + 4;
}

// Most heads a block of W slices may touch: W / 2 + 1 when every head has at
// least two slices (headdim >= 32). The host checks the actual count.
// Row stride (elements) of the staged C tile, read along rows as 16-byte
// fragments (rows l16 of a 16-lane group). Measured on gfx950: rows whose
// byte stride is 8 modulo 16 serve these reads without bank conflicts, 16-byte
// multiples do not (they run at about 60%). Rows are then only 8-byte aligned.
template <typename TI>
constexpr int c_row_stride(int ncols) { return ncols + 8 / (int)sizeof(TI); }

// 8 consecutive elements from an 8-byte aligned LDS address, as an MFMA operand.
template <typename TI>
__device__ __forceinline__ typename Ops<TI>::frag ld8_a8(const TI* p) {
    const uint2* q = reinterpret_cast<const uint2*>(p);
    if constexpr (sizeof(TI) == 2) {
        const uint2 a = q[0], b = q[1];
        return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
    } else {
        const uint2 a = q[0], b = q[1], c = q[2], d = q[3];
        f32x8 f = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(b.x), __uint_as_float(b.y),
                   __uint_as_float(c.x), __uint_as_float(c.y), __uint_as_float(d.x), __uint_as_float(d.y)};
        return f;
    }
}

constexpr int cols_max_heads(int W) { return W / 2 + 1; }

// Rotation tables of the rotating column walk hold (time step, pair) entries
// of one tile: at most this many, i.e. (32 / R) * dstate / 2 <= kRotEntries.
constexpr int kRotEntries = 512;
// row (one time step) of a memory wave's rotation table: per pair group of two
// state pairs, the four rows of its 4x4 turning matrix (8 bytes each)
// (plus 4 entries, so that the rows of the four time steps a 16-lane group
// reads start 8 banks apart)
constexpr int rot_row_stride(int NP) { return (NP / 4) * 4 + 4; }

template <typename TI, int NP, int W, bool ROT>
constexpr int cols_lds_bytes(int mode) {
    constexpr int esz = (int)sizeof(TI), epu = 16 / esz, F = kRows, CW = 16 * W;
    constexpr int MH = ROT ? 1 : cols_max_heads(W);
    constexpr int ldx = x_row_stride<TI>(CW), ldc = c_row_stride<TI>(NP);
    constexpr int ldb = ROT ? rot_b_row_stride<TI>(NP) : tr_row_stride<TI>(NP);
    constexpr int mbytes = (int)sizeof(typename MBlock<TI>::type);
    const int out = mode == 0;
    return 2 * (F * ldx + epu) * esz + 2 * (F * ldb + epu) * esz +
           (out ? 2 * (F * ldc + epu) * esz + 2 * (F * y_row_stride(CW) + 4) * 4 +
                      (ROT ? 0 : 2 * (768 + 4) * 4 + 2 * MH * 3 * 64 * mbytes)
                : 0) +
           4 * MH * (3 * F + 1) * 4 + 4 * F * (ROT ? 1 : 8) * 4 +
           (ROT ? 4 * (kRotEntries / (NP / 2) / 2) * rot_row_stride(NP) * 8 + (NP / 2) * 4 : 0);
}

// Memory waves per workgroup of the column-block walk: they issue every global
// load of the walk (x, and the B, C, C B^T and da tiles), so the W compute
// waves work from LDS and registers and only store y. The rotating walk runs
// four, one per SIMD, each turning one 16-row block of B or C.
constexpr int cols_mem_waves(int W, bool rot) { return rot ? 4 : (W >= 4 ? 2 : 1); }

// YS (output pass only): y keeps only the odd time steps (TileArgs::ysub).
template <typename TI, int NP, int W, int MODE, bool ROT, bool YS = false>
__global__ __launch_bounds__(64 * (W + cols_mem_waves(W, ROT))) void ssd_cols_kernel(TileArgs a) {
    using O = Ops<TI>;
    typedef typename O::frag frag;
    typedef typename MBlock<TI>::type mblk;
    constexpr int MW = cols_mem_waves(W, ROT);
    static_assert(!ROT || (W & (W - 1)) == 0, "the rotating walk deals tiles to a power-of-two wave count");
    constexpr int NTM = 64 * MW;                   // memory threads
    constexpr int NTC = 64 * W;                    // compute threads
    constexpr int F = kRows;
    constexpr int ESZ = (int)sizeof(TI);
    constexpr int CW = 16 * W;                     // columns per workgroup
    constexpr int MH = ROT ? 1 : cols_max_heads(W);  // a rotating block is one head
    constexpr int LDX = x_row_stride<TI>(CW);
    constexpr int LDB = ROT ? rot_b_row_stride<TI>(NP) : tr_row_stride<TI>(NP);
    constexpr int LDC = c_row_stride<TI>(NP);      // rows 8 bytes off 16-byte alignment
    constexpr int LDY = y_row_stride(CW);
    constexpr int NTILE = NP / 16;
    constexpr int KS = NP / 32;
    constexpr bool OUT = (MODE == 0);
    constexpr int EPU = 16 / ESZ;
    constexpr int XUR = CW / EPU, BUR = NP / EPU, YUR = CW / 4;   // 16-byte units per row
    constexpr int XU = F * XUR, BU = F * BUR, CBU = 768 * 4 / 16, YU = F * YUR;
    constexpr int XPT = (XU + NTM - 1) / NTM;                                       // per memory thread
    constexpr int DAH = ROT ? 1 : 8;               // heads per staged da step
    constexpr int CBPM = (CBU + NTM - 1) / NTM, DPM = (F * DAH + NTM - 1) / NTM;  // per memory thread
    constexpr int BPM = (BU + NTM - 1) / NTM;

    __shared__ __attribute__((aligned(16))) TI sX[2][F * LDX + EPU];
    __shared__ __attribute__((aligned(16))) TI sB[2][F * LDB + EPU];
    __shared__ __attribute__((aligned(16))) TI sC[OUT ? 2 : 1][OUT ? F * LDC + EPU : 1];
    __shared__ __attribute__((aligned(16))) float sCB[(OUT && !ROT) ? 2 : 1][(OUT && !ROT) ? 768 + 4 : 1];
    __shared__ __attribute__((aligned(16))) float sY[OUT ? 2 : 1][OUT ? F * LDY + 4 : 1];
    __shared__ __attribute__((aligned(16))) mblk sM[(OUT && !ROT) ? 2 : 1][(OUT && !ROT) ? MH * 3 * 64 : 1];
    // per-head tile vectors, ring of 4 tiles: cumulative log2-decay, exp2 of
    // it, the weight that carries row j to the tile end, and the tile decay
    __shared__ __attribute__((aligned(16))) float sCum[4][MH][F], sEin[4][MH][F], sW[4][MH][F];
    __shared__ float sCarry[4][MH];
    // da of the block's heads, staged by the memory waves: [tile ring][step][head]
    __shared__ __attribute__((aligned(16))) float sDa[4][kRows][DAH];
    // trapezoid: per sub-step write scale (beta or gamma), same ring
    __shared__ float sSc[ROT ? 4 : 1][ROT ? kRows : 1];
    // rotation: each memory wave's table for the time steps of its 16-row
    // block: per step and pair group (2 state pairs), the four rows of the bf16
    // matrix that turns them by R(-Phi), Phi the angle from the segment start;
    // Phi at the segment end
    constexpr int RSTR = rot_row_stride(NP);
    constexpr int QTM = ROT ? kRotEntries / (NP / 2) : 1;        // most steps per tile
    __shared__ __attribute__((aligned(16))) uint2 sRot[ROT ? 4 : 1][ROT ? (QTM / 2) * RSTR : 1];
    __shared__ float sPhi[ROT ? NP / 2 : 1];
    __shared__ float sLam[ROT ? W : 1];   // partial sums of da per compute wave

    const int tid = threadIdx.x;
    // wave index made visibly uniform, so per-head pointers stay scalar
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;
    const bool memw = wv >= W;                     // memory wave
    const int mt = tid - 64 * W;                   // memory thread index (memory waves)
    const int mw = wv - W;                         // memory wave index
    const int cwv = memw ? 0 : wv;                 // compute wave index (0 for memory waves)

    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, R = a.R, P = a.P;
    const int64_t TR = T * R;
    const int S = a.S;
    const int SPH = (int)(P >> 4);                 // slices per head
    const int NB = a.NB;                           // column blocks per B/C group
    int item = xcd_item(blockIdx.x, gridDim.x);
    const int jb = item % NB;
    item /= NB;
    const int64_t grp = item % G;
    item /= (int)G;
    const int seg = item % a.seg_items;
    const int b = item / a.seg_items;
    const int64_t col0 = grp * (H / G) * P + (int64_t)jb * CW;   // first flattened (h, p) column
    const int s0 = jb * W;                                       // first slice of the block
    const int hb0 = s0 / SPH;                                    // its head, within the group
    const int nhb = (s0 + W - 1) / SPH - hb0 + 1;                // heads the block touches
    const int64_t hfirst = grp * (H / G) + hb0;
    const int slice = s0 + cwv;                                  // this compute wave's slice
    const int hl = slice / SPH - hb0;                            // its head within the block
    const int64_t h = hfirst + hl;
    const int p0 = (slice % SPH) * 16;
    const int64_t bh = (int64_t)b * H + h;
    const int k0 = (int)(((int64_t)seg * a.nsub) / S);
    const int k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    const int log2R = a.log2R;
    const int Qt = a.Qt;
    const int nk = k1 - k0;

    // Buffer resources span the segment's valid rows; per lane a fixed 32-bit
    // offset advances by a per-tile step. Rows past the segment (ragged tail,
    // tiles prefetched beyond k1) fall outside the resource: loads return 0,
    // stores are dropped. The host keeps every segment's span below 2^30 bytes.
    const int64_t xrow_el = H * P, brow_el = G * N;
    const int64_t row0 = (int64_t)k0 * F;
    const int64_t row_end = ((int64_t)k1 * F < TR) ? (int64_t)k1 * F : TR;
    const int64_t vrows = row_end - row0;                    // >= 1

    // K1 of tile k for head hd of the block (prefix of da over the tile's
    // fused rows, in base 2), from the da the memory waves staged. Lane f < 32
    // takes step f >> log2R for the first rank of each step (0 for the others),
    // so the scan over fused rows yields cum per row.
    const bool da_lane = (lane < F) && ((lane & ((1 << log2R) - 1)) == 0);
    float lam = 0.f;   // sum of da over the segment (lane 0 of the scanning wave)
    auto scan_head = [&](int k, int hd) {
        const float dv = da_lane ? sDa[k & 3][lane >> log2R][hd] : 0.f;
        const float cum = wave_prefix32(dv);
        const float last = __shfl(cum, F - 1);
        const float c2 = cum * kLog2e, l2 = last * kLog2e;
        if (lane < F) {
            sCum[k & 3][hd][lane] = c2;
            sEin[k & 3][hd][lane] = __builtin_amdgcn_exp2f(c2);
            sW[k & 3][hd][lane] = __builtin_amdgcn_exp2f(l2 - c2);
        }
        if (lane == 0) sCarry[k & 3][hd] = __builtin_amdgcn_exp2f(l2);
        lam += last;
    };

    // trapezoid source geometry: a tile of Qt sub-steps covers Qt / 2 source
    // steps (16 source rows); x and B resources start one step before the
    // segment (its first even sub-step reads the previous step), except in the
    // first segment, whose step -1 comes from prev_x / prev_B
    constexpr bool trap = ROT && YS;            // the rotating walk with YS runs trapezoid sub-steps
    const int64_t Ts = trap ? T / 2 : T;                          // source steps
    const int64_t sb = trap ? (int64_t)k0 * (Qt >> 1) : 0;       // segment's first source step
    const int64_t se = trap ? (((int64_t)k1 * (Qt >> 1) < Ts) ? (int64_t)k1 * (Qt >> 1) : Ts) : 0;
    const int adj = (trap && k0 > 0) ? 1 : 0;
    const bool first_seg = trap && k0 == 0;

    if (memw) {
        // ============ memory waves: x, B, C, C B^T and da staged into LDS ============
        const int64_t xr0 = trap ? (sb - adj) * R : row0, xvr = trap ? (se - sb + adj) * R : vrows;
        const auto rs_x = make_rsrc(static_cast<const TI*>(a.x) + (b * Ts * R + xr0) * xrow_el + col0,
                                    (uint32_t)(((xvr - 1) * xrow_el + CW) * ESZ));
        const uint32_t xstep = (uint32_t)((trap ? (F >> 1) : F) * xrow_el * ESZ);
        uint32_t xgoff[XPT], xpoff[XPT];
        int xloff[XPT];
#pragma unroll
        for (int m = 0; m < XPT; ++m) {
            const int u = mt + m * NTM;
            const int r = u / XUR, col = (u % XUR) * EPU;
            int srow = r;
            if (trap) {
                const int sl = r >> log2R, rr = r & ((1 << log2R) - 1);
                srow = (((sl - 1) >> 1) + adj) * (int)R + rr;   // may be -R..-1: out of range
                xpoff[m] = (u < XU && sl == 0) ? (uint32_t)((rr * xrow_el + col) * ESZ) : kOOB;
            } else {
                xpoff[m] = kOOB;
            }
            xgoff[m] = (u < XU) ? (uint32_t)((int64_t)(srow * xrow_el + col) * ESZ) : kOOB;
            xloff[m] = (u < XU) ? r * LDX + col : F * LDX;
        }
        uint4 rx[2][XPT];            // x of tile t in slot t & 1
        auto load_x = [&](int slot, int k) {
            const uint32_t o = (uint32_t)k * xstep;
#pragma unroll
            for (int m = 0; m < XPT; ++m)   // non-temporal: x is read once (plain walk)
                rx[slot][m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, xgoff[m] + o, 0, trap ? 0 : 2));
        };
        // trapezoid, first segment: sub-step 0 writes prev_x, whose units the
        // first load_x left zero (out of range); called once, after it
        auto patch_x0 = [&](int slot) {
            if constexpr (trap) {
                if (!first_seg || !a.prev_x) return;
                const auto rs_px = make_rsrc(static_cast<const TI*>(a.prev_x) + b * R * xrow_el + col0,
                                             (uint32_t)(((R - 1) * xrow_el + CW) * ESZ));
#pragma unroll
                for (int m = 0; m < XPT; ++m) {
                    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_px, xpoff[m], 0, 0));
                    rx[slot][m].x |= v.x;
                    rx[slot][m].y |= v.y;
                    rx[slot][m].z |= v.z;
                    rx[slot][m].w |= v.w;
                }
            }
        };
        auto store_x = [&](int slot, int buf) {
#pragma unroll
            for (int m = 0; m < XPT; ++m) *reinterpret_cast<uint4*>(&sX[buf][xloff[m]]) = rx[slot][m];
        };
        // da of tile t in slot t & 1: element (step, head) of the block's heads,
        // lane-contiguous along the heads of a step (one short run per step)
        // da (and, for the trapezoid, the write scale) per step of the walk
        const int64_t step0 = (int64_t)k0 * Qt;
        const int64_t vsteps = (((int64_t)k1 * Qt < T) ? (int64_t)k1 * Qt : T) - step0;
        const auto rs_da = make_rsrc(a.da + (b * T + step0) * H + hfirst, (uint32_t)(((vsteps - 1) * H + nhb) * 4));
        const uint32_t dastep = (uint32_t)(Qt * H * 4);
        uint32_t daoff[DPM];
#pragma unroll
        for (int m = 0; m < DPM; ++m) {
            const int u = mt + m * NTM, st = u / DAH, hd = u % DAH;
            daoff[m] = (st < Qt && hd < nhb) ? (uint32_t)((st * H + hd) * 4) : kOOB;
        }
        float rda[2][DPM], rsc[2][trap ? DPM : 1];
        auto load_da = [&](int slot, int k) {
            const uint32_t o = (uint32_t)k * dastep;
#pragma unroll
            for (int m = 0; m < DPM; ++m)
                rda[slot][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_da, daoff[m] + o, 0, 0));
            if constexpr (trap) {
                const auto rs_sc = make_rsrc(a.scale + (b * T + step0) * H + hfirst, (uint32_t)(((vsteps - 1) * H + nhb) * 4));
#pragma unroll
                for (int m = 0; m < DPM; ++m)
                    rsc[slot][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_sc, daoff[m] + o, 0, 0));
            }
        };
        auto store_da = [&](int slot, int k) {
#pragma unroll
            for (int m = 0; m < DPM; ++m) {
                // (the shared walk's units fill the ring slot exactly; an
                // unneeded guard there costs registers)
                if (!ROT || mt + m * NTM < F * DAH) (&sDa[k & 3][0][0])[mt + m * NTM] = rda[slot][m];
                if constexpr (trap) {
                    if (mt + m * NTM < F) sSc[k & 3][mt + m * NTM] = rsc[slot][m];
                }
            }
        };
        // B and C of tile t: one register slot, refilled a tile ahead
        const uint32_t bspan = (uint32_t)(((vrows - 1) * brow_el + N) * ESZ);
        const auto rs_b = make_rsrc(static_cast<const TI*>(a.B) + (b * TR + row0) * brow_el + grp * N, bspan);
        const auto rs_c = make_rsrc(static_cast<const TI*>(a.C) + (b * TR + row0) * brow_el + grp * N, bspan);
        const uint32_t bstep = (uint32_t)(F * brow_el * ESZ);
        if constexpr (!ROT) {
            // C B^T blocks of tile t in slot t & 1 (768 floats = CBU 16-byte units)
            const auto rs_cb = make_rsrc(OUT ? a.cbpack + ((int64_t)(b * G + grp) * a.nsub + k0) * 768 : a.da,
                                         OUT ? (uint32_t)((k1 - k0) * 768 * 4) : 0u);
            uint32_t cbgoff[CBPM];
            int cbloff[CBPM];
    #pragma unroll
            for (int m = 0; m < CBPM; ++m) {
                const int u = mt + m * NTM;
                cbgoff[m] = (u < CBU) ? (uint32_t)(u * 16) : kOOB;
                cbloff[m] = (u < CBU) ? u * 4 : 768;
            }
            float4 rcb[2][CBPM];
            auto load_cb = [&](int slot, int k) {
                if (OUT) {
                    const uint32_t o = (uint32_t)k * (768 * 4);
    #pragma unroll
                    for (int m = 0; m < CBPM; ++m)
                        rcb[slot][m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs_cb, cbgoff[m] + o, 0, 0));
                }
            };
            auto store_cb = [&](int slot, int k) {
                if (OUT) {
    #pragma unroll
                    for (int m = 0; m < CBPM; ++m) *reinterpret_cast<float4*>(&sCB[k & 1][cbloff[m]]) = rcb[slot][m];
                }
            };
            // thread mt takes column unit mt % BUR of rows mt / BUR + m (NTM / BUR):
            // the offsets advance by a fixed stride per unit
            static_assert(NTM % BUR == 0, "memory threads cover whole B rows");
            constexpr int RPM = NTM / BUR;               // rows per memory pass
            const int br0 = mt / BUR, bcol = (mt % BUR) * EPU;
            const bool bcol_ok = bcol < N;
            const uint32_t bgo0 = (uint32_t)((br0 * brow_el + bcol) * ESZ);
            const uint32_t bgstride = (uint32_t)(RPM * brow_el * ESZ);
            const int blo0 = br0 * LDB + bcol, clo0 = br0 * LDC + bcol;
            uint4 rb[BPM], rc[BPM];
            auto load_bc = [&](int k) {
                const uint32_t ob = (uint32_t)k * bstep;
    #pragma unroll
                for (int m = 0; m < BPM; ++m) {
                    const uint32_t go = (bcol_ok && br0 + m * RPM < F) ? bgo0 + m * bgstride + ob : kOOB;
                    rb[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_b, go, 0, 0));
                    if (OUT) rc[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_c, go, 0, 0));
                }
            };
            auto store_bc = [&](int buf) {
    #pragma unroll
                for (int m = 0; m < BPM; ++m) {
                    if (br0 + m * RPM >= F) continue;
                    *reinterpret_cast<uint4*>(&sB[buf][blo0 + m * RPM * LDB]) = rb[m];
                    if (OUT) {
                        // two 8-byte halves: C rows are only 8-byte aligned
                        uint2* d = reinterpret_cast<uint2*>(&sC[buf][clo0 + m * RPM * LDC]);
                        d[0] = make_uint2(rc[m].x, rc[m].y);
                        d[1] = make_uint2(rc[m].z, rc[m].w);
                    }
                }
            };
            // x is staged in registers two tiles ahead and in LDS one tile ahead
            // (buffer = tile parity). The C B^T blocks and da run one tile further
            // ahead, for the compute waves' decay matrices and scans. Each register
            // slot is refilled right after it is drained. Barriers match the
            // compute waves' one for one.
            load_bc(0);
            load_x(0, 0);
            load_x(1, 1);
            load_cb(0, 0);
            load_cb(1, 1);
            load_da(0, 0);
            load_da(1, 1);
            store_bc(0);
            load_bc(1);
            store_x(0, 0);
            load_x(0, 2);
            store_cb(0, 0);
            load_cb(0, 2);
            store_cb(1, 1);
            load_cb(1, 3);
            store_da(0, 0);
            load_da(0, 2);
            store_da(1, 1);
            load_da(1, 3);
            __syncthreads();             // da of tiles 0, 1 for the compute waves' scans
            store_da(0, 2);
            load_da(0, 4);
            __syncthreads();
            __syncthreads();
            int k = 0;
            for (; k < nk; k += 2) {
                store_bc(1);             // B, C of tile k+1
                load_bc(k + 2);
                store_x(1, 1);           // x of tile k+1
                load_x(1, k + 3);
                store_cb(0, k + 2);
                load_cb(0, k + 4);
                store_da(1, k + 3);
                load_da(1, k + 5);
                __syncthreads();
                store_bc(0);             // B, C of tile k+2
                load_bc(k + 3);
                store_x(0, 0);           // x of tile k+2
                load_x(0, k + 4);
                store_cb(1, k + 3);
                load_cb(1, k + 5);
                store_da(0, k + 4);
                load_da(0, k + 6);
                __syncthreads();
            }
        } else {
            // ---- rotation: each memory wave turns one 16-row block of B or C
            // by R(-Phi) on its way to LDS (the state pass needs B only); the
            // compute waves form K2 (C B^T) from the turned tiles.
            static_assert(MW == 4, "the rotating walk runs four memory waves");
            // their turn of the next tile is the longer chain of a tile: issue
            // ahead of the compute wave sharing the SIMD
            __builtin_amdgcn_s_setprio(1);
            constexpr int NPP = NP / 2;                  // state pairs
            static_assert(NPP <= 64, "one lane per state pair");
            const int gmat = mw >> 1, grb = mw & 1;      // matrix (0 = B, 1 = C) and row block
            const bool gon = OUT || gmat == 0;
            const int grow = 16 * grb + l16;             // this lane's row of the tile
            // trapezoid: the source row of this lane's sub-step row (B: step
            // (s - 1) >> 1 from a resource one step early unless first segment;
            // C: step s >> 1), tiles 16 source rows apart
            int gsrc = grow;
            uint32_t gpoff = kOOB;
            if (trap) {
                const int sl = grow >> log2R, rr = grow & ((1 << log2R) - 1);
                gsrc = (gmat ? (sl >> 1) : ((sl - 1) >> 1) + adj) * (int)R + rr;
                if (gmat == 0 && sl == 0) gpoff = (uint32_t)((rr * brow_el + 8 * q) * ESZ);
            }
            const uint32_t goff = gon ? (uint32_t)((int64_t)(gsrc * brow_el + 8 * q) * ESZ) : kOOB;
            const int64_t gr0 = gmat ? sb * R : (sb - adj) * R, gvr = gmat ? (se - sb) * R : (se - sb + adj) * R;
            const auto rs_g = trap ? make_rsrc(static_cast<const TI*>(gmat ? a.C : a.B) + (b * Ts * R + gr0) * brow_el + grp * N,
                                               (uint32_t)(((gvr - 1) * brow_el + N) * ESZ))
                                   : (gmat ? rs_c : rs_b);
            const uint32_t gstep = trap ? (uint32_t)((F >> 1) * brow_el * ESZ) : bstep;
            // B / C fragments and angles of tile t in register slot t & 1,
            // loaded a full tile before they are used
            uint4 rf[2][KS];
            auto load_frags = [&](int slot, int k) {
                const uint32_t o = (uint32_t)k * gstep;
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    rf[slot][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_g, goff + s * 64 + o, 0, 0));
            };
            // trapezoid, first segment: sub-step 0 writes prev_B (out of range
            // in the first load_frags); called once, after it
            auto patch_frags0 = [&](int slot) {
                if constexpr (trap) {
                    if (!first_seg || gmat != 0 || !a.prev_B) return;
                    const auto rs_pg = make_rsrc(static_cast<const TI*>(a.prev_B) + b * R * brow_el + grp * N,
                                                 (uint32_t)(((R - 1) * brow_el + N) * ESZ));
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                      rs_pg, gpoff == kOOB ? kOOB : gpoff + s * 64, 0, 0));
                        rf[slot][s].x |= v.x;
                        rf[slot][s].y |= v.y;
                        rf[slot][s].z |= v.z;
                        rf[slot][s].w |= v.w;
                    }
                }
            };
            // angles: every memory wave keeps, per pair (lane), the running
            // angle from the segment start (wrapped to [-pi, pi]) and tables
            // (cos, sin) at the time steps of its own row block
            const int spb = 16 >> log2R;                 // time steps per 16-row block
            const int st0 = grb * spb;
            const int64_t NH2 = N / 2;
            const int64_t th0 = trap ? sb : step0, thv = trap ? se - sb : vsteps;
            const auto rs_th = make_rsrc(a.theta + ((b * Ts + th0) * H + hfirst) * NH2,
                                         (uint32_t)((((thv - 1) * H) * NH2 + NH2) * 4));
            const uint32_t throw_b = (uint32_t)(H * NH2 * 4);
            const uint32_t thstep = (uint32_t)((trap ? (Qt >> 1) : Qt) * H * NH2 * 4);
            const uint32_t thoff = (gon && lane < NH2) ? (uint32_t)(lane * 4) : kOOB;
            float rth[2][QTM], carry = 0.f;
            // theta of sub-step st: step st (plain) or, for the trapezoid, step
            // st >> 1 on odd sub-steps and no turn on even ones
            auto load_th = [&](int slot, int k) {
                const uint32_t o = (uint32_t)k * thstep;
#pragma unroll
                for (int st = 0; st < QTM; ++st) {
                    const bool on = st < Qt && (!trap || (st & 1));
                    const uint32_t so = trap ? (uint32_t)(st >> 1) * throw_b : (uint32_t)st * throw_b;
                    rth[slot][st] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                  rs_th, on ? thoff + so + o : kOOB, 0, 0));
                }
            };
            uint2* tab = sRot[mw];
            // table of the tile whose angles are in rth, then B~ / C~ of that
            // tile into buffer buf (the table is this wave's own: no barrier).
            // The turn is a 4x4x4 MFMA per pair group: its 16 blocks are 4-lane
            // groups, i.e. 4 consecutive rows of one time step (R >= 4) and the
            // same 2 pairs. Block row e of the matrix (lane 4b + e) is
            //   e = 0: (c0, s0, 0, 0)   e = 1: (-s0, c0, 0, 0)
            //   e = 2: (0, 0, c1, s1)   e = 3: (0, 0, -s1, c1)
            // and lane 4b + r contributes its own row r of B or C, so that
            // lane 4b + r receives out[r][e] = sum_k M[e][k] in[r][k] in slot e.
            auto rotate_tile = [&](int buf, int slot) {
                if (!gon) return;
                float run = 0.f;
#pragma unroll
                for (int st = 0; st < QTM; ++st) {
                    if (st < Qt) {
                        run += rth[slot][st];
                        if (st >= st0 && st < st0 + spb) {
                            // the hardware sine and cosine take revolutions
                            const float rev = (carry + run) * kInv2Pi;
                            const float c = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
                            if (lane < NPP) {
                                const uint32_t cs = pack_bf16x2(c, sn), ms = pack_bf16x2(-sn, c);
                                const int h = lane & 1;
                                uint2* e0 = tab + (st - st0) * RSTR + (lane >> 1) * 4 + 2 * h;
                                e0[0] = h ? make_uint2(0u, cs) : make_uint2(cs, 0u);
                                e0[1] = h ? make_uint2(0u, ms) : make_uint2(ms, 0u);
                            }
                        }
                    }
                }
                carry = wrap_angle(carry + run);
                typedef __attribute__((ext_vector_type(4))) short s16x4;
                const uint2* trow = tab + (l16 >> log2R) * RSTR + (lane & 3);
                // the state pass, where the memory waves set the pace: every
                // table row of the turn read before its first store, so that
                // the reads are in flight together (the output walk keeps
                // them interleaved, which measured faster there)
                uint2 mr[OUT ? 1 : KS][2];
                if constexpr (!OUT) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        mr[s][0] = trow[(8 * s + 2 * q) * 4];
                        mr[s][1] = trow[(8 * s + 2 * q + 1) * 4];
                    }
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    // pair groups 8 s + 2 q and 8 s + 2 q + 1 of this row's step
                    uint2 m0, m1;
                    if constexpr (!OUT) {
                        m0 = mr[s][0];
                        m1 = mr[s][1];
                    } else {
                        m0 = trow[(8 * s + 2 * q) * 4];
                        m1 = trow[(8 * s + 2 * q + 1) * 4];
                    }
                    const uint4 w = rf[slot][s];
                    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                        __builtin_bit_cast(s16x4, m0), __builtin_bit_cast(s16x4, make_uint2(w.x, w.y)), zero4, 0, 0, 0);
                    const f32x4 d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                        __builtin_bit_cast(s16x4, m1), __builtin_bit_cast(s16x4, make_uint2(w.z, w.w)), zero4, 0, 0, 0);
                    const uint4 r = make_uint4(pack_bf16x2(d0[0], d0[1]), pack_bf16x2(d0[2], d0[3]),
                                               pack_bf16x2(d1[0], d1[1]), pack_bf16x2(d1[2], d1[3]));
                    if (gmat == 0) {
                        uint2* d = reinterpret_cast<uint2*>(&sB[buf][grow * LDB + 32 * s + 8 * q]);
                        d[0] = make_uint2(r.x, r.y);
                        d[1] = make_uint2(r.z, r.w);
                    } else {
                        uint2* d = reinterpret_cast<uint2*>(&sC[buf][grow * LDC + 32 * s + 8 * q]);
                        d[0] = make_uint2(r.x, r.y);
                        d[1] = make_uint2(r.z, r.w);
                    }
                }
            };
            // Tile t is turned and stored during tile t-1; its angles and B/C
            // fragments are loaded during tile t-3, as soon as their register
            // slot drains, so that more than a tile of work covers the latency.
            load_frags(0, 0);
            patch_frags0(0);
            load_th(0, 0);
            load_frags(1, 1);
            load_th(1, 1);
            load_x(0, 0);
            patch_x0(0);
            load_x(1, 1);
            load_da(0, 0);
            load_da(1, 1);
            store_x(0, 0);
            load_x(0, 2);
            store_da(0, 0);
            load_da(0, 2);
            store_da(1, 1);
            load_da(1, 3);
            rotate_tile(0, 0);
            load_frags(0, 2);
            load_th(0, 2);
            __syncthreads();             // da of tiles 0, 1; B~, C~, x of tile 0
            store_da(0, 2);
            load_da(0, 4);
            __syncthreads();
            __syncthreads();
            int k = 0;
            for (; k < nk; k += 2) {
                rotate_tile(1, 1);       // tile k+1
                load_frags(1, k + 3);
                load_th(1, k + 3);
                store_x(1, 1);
                load_x(1, k + 3);
                store_da(1, k + 3);
                load_da(1, k + 5);
                __syncthreads();
                rotate_tile(0, 0);       // tile k+2
                load_frags(0, k + 4);
                load_th(0, k + 4);
                store_x(0, 0);
                load_x(0, k + 4);
                store_da(0, k + 4);
                load_da(0, k + 6);
                __syncthreads();
            }
            // the angle at the segment end (tiles past it add zero)
            if (mw == 0 && lane < NH2) {
                sPhi[lane] = carry;
                if (!OUT) a.ws_misc[(((int64_t)b * H + hfirst) * S + seg) * (1 + NH2) + 1 + lane] = carry;
            }
            __syncthreads();
        }
        return;
    }

    // ================= compute waves =================
    // wave w < nhb scans the decays of head hfirst + w
    const bool scanner = wv < nhb;
    // this wave's y fragment in the staged block: rows 16 I + l16, columns
    // 16 wv + 4 q .. + 3
    const int ysoff = l16 * LDY + 16 * wv + 4 * q;
    // y of tile k leaves from the staged block during tile k+1, in whole
    // 16-byte units of the block's rows, spread over the compute threads
    // (their barrier wait has room for it; the memory waves have less)
    constexpr int YPC = (YU + NTC - 1) / NTC;
    // with ysub, y holds only the odd steps (a tile starts at an even step,
    // 32 / R being even): local row r = j R + k of an odd step j goes to
    // compact row (j >> 1) R + k, half a tile of rows per tile
    constexpr int ys = YS ? 1 : 0;
    const auto rs_y = make_rsrc(a.y + (b * (TR >> ys) + (row0 >> ys)) * xrow_el + col0,
                                (uint32_t)((((vrows >> ys) - 1) * xrow_el + CW) * 4));
    const uint32_t ystep = (uint32_t)((F >> ys) * xrow_el * 4);
    uint32_t ygoff[YPC];
    int yloff[YPC];
#pragma unroll
    for (int m = 0; m < YPC; ++m) {
        const int u = tid + m * NTC;
        const int r = u / YUR, col = (u % YUR) * 4;
        const int j = r >> log2R;
        const bool keep = u < YU && (!ys || (j & 1));
        const int yr = ys ? (((j >> 1) << log2R) | (r & ((1 << log2R) - 1))) : r;
        ygoff[m] = keep ? (uint32_t)((yr * xrow_el + col) * 4) : kOOB;
        yloff[m] = (u < YU) ? r * LDY + col : F * LDY;
    }
    // global stores of the y block staged in sY[buf] by tile k; the first
    // flush (tile -1) wraps to an offset beyond the resource and is dropped
    auto flush_y = [&](int buf, int k) {
        if (OUT) {
            const uint32_t o = (uint32_t)k * ystep;
#pragma unroll
            for (int m = 0; m < YPC; ++m) {
                const float4 v = *reinterpret_cast<const float4*>(&sY[buf][yloff[m]]);
                // non-temporal: y is written once and never read back here
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs_y, ygoff[m] + o, 0, 2);
            }
        }
    };
    // the scanning waves: wave w < nhb scans head hfirst + w; in the rotating
    // walk (one head) the compute waves take the tiles in turn
    auto scan = [&](int k) {
        if constexpr (ROT) {
            if (wv == (k & (W - 1))) scan_head(k, 0);
        } else {
            if (scanner) scan_head(k, wv);
        }
    };

    // ---- state (physical frame)
    f32x4 hs[NTILE];
    {
        const float* src = nullptr;
        if (OUT) {
            if (S == 1)
                src = a.init ? a.init + bh * P * N : nullptr;
            else
                src = a.ws_state + (bh * S + seg) * a.SF * P * N;
        }
        // unconditional loads (clamped index), then one select: lets the
        // loads issue back to back
        const float* row = (src ? src : a.da) + (src ? (int64_t)(p0 + l16) * N : 0);
        const int nmax = src ? (int)N - 1 : 0;
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = phi_row(t, 4 * q + v);
                const float val = row[n < nmax ? n : nmax];
                hs[t][v] = (src && n < N) ? val : 0.f;
            }
        }
    }

    // Decay matrices M = (C B^T o L) (+ D on the diagonal) of tile k for
    // every head of the block, one (head, 16x16 block) unit per compute wave:
    // element (j = 16 J + 4 q + v, i = 16 I + l16) of blocks (0,0), (0,1),
    // (1,1). The pack already zeroes C B^T where step(i) < step(j), and cum is
    // non-increasing, so exp2(min(cum_i - cum_j, 0)) is exact where it counts.
    constexpr int UPW = (3 * MH + W - 1) / W;      // units per compute wave
    float Du[UPW];
#pragma unroll
    for (int r = 0; r < UPW; ++r) {
        const int u = wv + W * r;
        Du[r] = (OUT && a.D && u < 3 * nhb && (u % 3) != 1) ? a.D[hfirst + u / 3] : 0.f;
    }
    float dsel[4];                                 // one-hot: this lane's diagonal slot
#pragma unroll
    for (int v = 0; v < 4; ++v) dsel[v] = (l16 == 4 * q + v) ? 1.f : 0.f;
    const float Dr = (ROT && OUT && a.D) ? a.D[h] : 0.f;   // D of the rotating block's head
    auto build_m = [&](int k) {
        if constexpr (OUT && !ROT) {
#pragma unroll
            for (int r = 0; r < UPW; ++r) {
                const int u = wv + W * r;
                if (u < 3 * nhb) {
                    const int uh = u / 3, blk = u - 3 * uh;
                    const int J = blk == 2 ? 1 : 0, I = blk == 0 ? 0 : 1;
                    const float* cum = sCum[k & 3][uh];
                    const float4 cb = *reinterpret_cast<const float4*>(&sCB[k & 1][blk * 256 + lane * 4]);
                    const float4 cj = *reinterpret_cast<const float4*>(&cum[16 * J + 4 * q]);
                    const float ci = cum[16 * I + l16];
                    const float cbv[4] = {cb.x, cb.y, cb.z, cb.w}, cjv[4] = {cj.x, cj.y, cj.z, cj.w};
                    float mv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        mv[v] = fmaf(dsel[v], Du[r], cbv[v] * __builtin_amdgcn_exp2f(fminf(ci - cjv[v], 0.f)));
                    sM[k & 1][u * 64 + lane] = pack_m<TI>(mv[0], mv[1], mv[2], mv[3]);
                }
            }
        }
    };

    auto compute = [&](int buf, int k) {
        const TI* tB = sB[buf];
        const int vb = k & 3;
        // x^T operand: rows j in {4q..4q+3} and {16+4q..16+4q+3}, column 16 wv + i
        const frag xa = RowRuns<TI>::load(sX[buf], LDX, 4 * q, 16 + 4 * q, 16 * wv + 4 * (lane & 3),
                                          16 * wv + l16, lane);
        if (OUT) {
            const TI* tC = sC[buf];
            f32x4 yacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            // rotating walk: K2 of the block's head from the turned tiles,
            // blocks (J, I) = (0,0), (0,1), (1,1) of C B^T (rows j, columns i)
            f32x4 cb00 = {0.f, 0.f, 0.f, 0.f}, cb01 = cb00, cb11 = cb00;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float hv[8];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    hv[v] = hs[2 * s][v];
                    hv[4 + v] = hs[2 * s + 1][v];
                }
                const frag hA = O::pack(hv);
                if constexpr (ROT) {
                    const frag c0 = ld8_a8<TI>(tC + l16 * LDC + 32 * s + 8 * q);
                    const frag c1 = ld8_a8<TI>(tC + (16 + l16) * LDC + 32 * s + 8 * q);
                    yacc[0] = O::mma(hA, c0, yacc[0]);
                    yacc[1] = O::mma(hA, c1, yacc[1]);
                    const frag b0 = ld8_a8<TI>(tB + l16 * LDB + 32 * s + 8 * q);
                    const frag b1 = ld8_a8<TI>(tB + (16 + l16) * LDB + 32 * s + 8 * q);
                    cb00 = O::mma(b0, c0, cb00);
                    cb01 = O::mma(b0, c1, cb01);
                    cb11 = O::mma(b1, c1, cb11);
                } else {
                    yacc[0] = O::mma(hA, ld8_a8<TI>(tC + l16 * LDC + 32 * s + 8 * q), yacc[0]);
                    yacc[1] = O::mma(hA, ld8_a8<TI>(tC + (16 + l16) * LDC + 32 * s + 8 * q), yacc[1]);
                }
            }
            const float e0 = sEin[vb][hl][l16], e1 = sEin[vb][hl][16 + l16];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                yacc[0][v] *= e0;
                yacc[1][v] *= e1;
            }
            mblk m00, m01, m11;
            if constexpr (!ROT) {
                const mblk* mb = &sM[k & 1][hl * 3 * 64 + lane];
                m00 = mb[0];
                m01 = mb[64];
                m11 = mb[128];
            } else {
                // the block's one head: its decay matrices from its C B^T
                // blocks, zero where step(i) < step(j) (cum is non-increasing,
                // so exp2(min(cum_i - cum_j, 0)) is exact where it counts)
                const float* cum = sCum[vb][0];
                const float4 cj0 = *reinterpret_cast<const float4*>(&cum[4 * q]);
                const float4 cj1 = *reinterpret_cast<const float4*>(&cum[16 + 4 * q]);
                const float ci0 = cum[l16], ci1 = cum[16 + l16];
                const float cjv0[4] = {cj0.x, cj0.y, cj0.z, cj0.w}, cjv1[4] = {cj1.x, cj1.y, cj1.z, cj1.w};
                float v0[4], v1[4], v2[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool k00 = (l16 >> log2R) >= ((4 * q + v) >> log2R);
                    const bool k11 = ((16 + l16) >> log2R) >= ((16 + 4 * q + v) >> log2R);
                    v0[v] = fmaf(dsel[v], Dr, k00 ? cb00[v] * __builtin_amdgcn_exp2f(fminf(ci0 - cjv0[v], 0.f)) : 0.f);
                    v1[v] = cb01[v] * __builtin_amdgcn_exp2f(fminf(ci1 - cjv0[v], 0.f));
                    v2[v] = fmaf(dsel[v], Dr, k11 ? cb11[v] * __builtin_amdgcn_exp2f(fminf(ci1 - cjv1[v], 0.f)) : 0.f);
                }
                if (trap) {
                    // the source rows' write scales (source rows 4q + v and
                    // 16 + 4q + v, one time step each since R >= 4)
                    const float s0 = sSc[vb][(4 * q) >> log2R], s1 = sSc[vb][(16 + 4 * q) >> log2R];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        v0[v] *= s0;
                        v1[v] *= s0;
                        v2[v] *= s1;
                    }
                }
                m00 = pack_m<TI>(v0[0], v0[1], v0[2], v0[3]);
                m01 = pack_m<TI>(v1[0], v1[1], v1[2], v1[3]);
                m11 = pack_m<TI>(v2[0], v2[1], v2[2], v2[3]);
            }
            const mblk zz = pack_m<TI>(0.f, 0.f, 0.f, 0.f);
            yacc[0] = O::mma(xa, join_m<TI>(m00, zz), yacc[0]);
            yacc[1] = O::mma(xa, join_m<TI>(m01, m11), yacc[1]);
#pragma unroll
            for (int I = 0; I < 2; ++I)
                *reinterpret_cast<f32x4*>(&sY[buf][ysoff + 16 * I * LDY]) = yacc[I];
        }
        // K3 + K4: decay the state over the tile and add the tile's writes
        float xv[8];
        O::unpack(xa, xv);
        const float4 w0 = *reinterpret_cast<const float4*>(&sW[vb][hl][4 * q]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sW[vb][hl][16 + 4 * q]);
        xv[0] *= w0.x; xv[1] *= w0.y; xv[2] *= w0.z; xv[3] *= w0.w;
        xv[4] *= w1.x; xv[5] *= w1.y; xv[6] *= w1.z; xv[7] *= w1.w;
        if constexpr (ROT) {
            if (trap) {
                const float s0 = sSc[vb][(4 * q) >> log2R], s1 = sSc[vb][(16 + 4 * q) >> log2R];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xv[e] *= s0;
                    xv[4 + e] *= s1;
                }
            }
        }
        const frag xw = O::pack(xv);
        const float carry = sCarry[vb][hl];
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
            // B^T operand rows n = phi(t, i): column base for 4-lane group a
            const int cbs = 32 * (t >> 1) + 8 * (lane & 3) + 4 * (t & 1);
            const int cown = 32 * (t >> 1) + 8 * (l16 >> 2) + 4 * (t & 1) + (l16 & 3);
            const frag bt = RowRuns<TI>::load(tB, LDB, 4 * q, 16 + 4 * q, cbs, cown, lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) hs[t][v] *= carry;
            hs[t] = O::mma(bt, xw, hs[t]);
        }
    };

    // ---- pipeline (barriers match the memory waves' one for one). B and C
    // are staged in registers two tiles ahead and in LDS one tile ahead
    // (buffer = tile parity); the da scans and the memory waves' C B^T blocks
    // run one tile further ahead, so that the decay matrices of tile k+1 are
    // built, once per head, while tile k is computed. Each register slot is
    // refilled right after it is drained. Memory counters retire in issue
    // order, and each step waits only for the oldest group in flight.
    __syncthreads();                 // da of tiles 0, 1 staged
    scan(0);
    scan(1);
    __syncthreads();
    build_m(0);
    __syncthreads();
    for (int k = 0; k < nk; k += 2) {
        flush_y(1, k - 1);
        scan(k + 2);
        build_m(k + 1);
        compute(0, k);
        __syncthreads();
        flush_y(0, k);
        scan(k + 3);
        build_m(k + 2);
        compute(1, k + 1);
        __syncthreads();
    }
    flush_y(1, ((nk + 1) & ~1) - 1);   // the last tile walked (past nk when nk is odd: dropped)

    if constexpr (ROT) {
        // back to the physical frame: h = R(Phi_end) g, Phi_end from the
        // memory waves' angle walk. The segment's sum of da, from the
        // compute waves' partial sums, goes to wave 0.
        if (lane == 0) sLam[wv] = lam;
        __syncthreads();
        if (wv == 0) {
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) tot += sLam[w];
            lam = tot;
        }
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int v = 0; v < 4; v += 2) {
                const int n = phi_row(t, 4 * q + v);   // even: pair (n, n + 1)
                float sn, cs;
                sincosf(sPhi[n >> 1], &sn, &cs);
                const float g0 = hs[t][v], g1 = hs[t][v + 1];
                hs[t][v] = cs * g0 - sn * g1;
                hs[t][v + 1] = sn * g0 + cs * g1;
            }
        }
    }

    // ---- epilogue
    float* dstate = nullptr;
    if (OUT) {
        if (seg == S - 1) dstate = a.final_state + bh * P * N;
    } else {
        dstate = a.ws_state + (bh * S + seg + 1) * P * N;
        // Lambda of the segment, by the wave that scanned the head
        if (scanner && lane == 0) a.ws_misc[(((int64_t)b * H + hfirst + wv) * S + seg) * (1 + N / 2)] = lam;
    }
    if (dstate) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = phi_row(t, 4 * q + v);
                if (n < N) dstate[(int64_t)(p0 + l16) * N + n] = hs[t][v];
            }
        }
    }
}

}  // namespace

#endif  // SSD_KERNELS_H
