// Backward of the chunked SSD scan for AMD Instinct MI355X (gfx950).
//
// Gradients of a loss with respect to x, da, B, C, theta, init_state and D,
// given dy and the final-state gradient dfinal ("mamba3/scan.py", verify():
// the backward is checked against the recurrence, separately from the
// forward; burn-mamba "mamba3/moments.rs", module documentation: the
// recompute discipline, states re-materialised instead of kept). Per
// (batch, head), with h_t the physical state after step t and
// H_t = dL/dh_t (h_t = a_t R(theta_t) h_{t-1} + sum_r x_{t,r} (outer) B_{t,r},
// a_t = exp(da_t)):
//
//   H_t       = a_{t+1} R(theta_{t+1})^T H_{t+1} + sum_r dy_{t,r} (outer) C_{t,r}
//               (H_{T-1} starts from dfinal)
//   dx_{t,r}  = H_t B_{t,r} + D dy_{t,r}          dinit = a_0 R(theta_0)^T H_0
//   dB_{t,r}  = sum_p H_t[p,:] x_{t,r}[p]          (summed over a group's heads)
//   dC_{t,r}  = sum_p dy_{t,r}[p] h_t[p,:]         (summed over a group's heads)
//   dD        = sum dy . x
//   dda_t     = sum_{s >= t} (sum_r C_s . dC_s - sum_r B_s . dB_s)   (per head)
//               + <dfinal, h_{T-1}>
//   dtheta_t,k = sum_{s >= t} sum_r [(dC_2k C_2k+1 - dC_2k+1 C_2k) + (dB_2k B_2k+1 - dB_2k+1 B_2k)]
//               + sum_p (dfinal_2k+1 h_2k - dfinal_2k h_2k+1)          (per head)
//
// The last two follow from the chain rule: the decay of step t multiplies
// every pair (write before t, read at or after t) once, so its gradient is a
// reverse cumulative sum of per-step inner products; the turn of a state pair
// likewise, with the 2-D cross product (J = d R / d theta at zero). So no
// kernel pairs a state with its gradient: dC needs only the states (a walk
// forwards in time), dx and dB only the state gradients (a walk backwards),
// each with its own segment states from a state pass and a carry.
//
// The step walks (fp32 inputs, headdim 128) step one time step at a time with
// the state in registers as 16 x 16 MFMA accumulators, a workgroup per (batch,
// head, group of at most 64 state rows p, segment), two memory waves staging
// each 32-row tile; the chunked walks (bf16, headdim <= 64) take a tile at a
// time with four memory waves.
// Contractions over p (dC, dB) need the layout D[p][n] (lanes across n); the
// contraction over n (dx) needs D[n][p] (lanes across p), so the backward walk
// keeps its state gradient in both layouts and updates both.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ssd_common.h"
#include "ssd_step.h"

namespace {

using namespace ssd_detail;
using namespace ssd_step;

constexpr int kTileRows = 32;        // fused rows (step, rank) staged per tile
constexpr int kPadRows = 4;          // zero rows after a tile (reads past its last step)
constexpr int kRowGroup = 64;        // most state rows p per workgroup
constexpr int kMemWaves = 2;
constexpr int kMaxWaves = kRowGroup / 16 + kMemWaves;
// Memory waves of the chunked walks: four. With rotation they also turn B and
// C while staging (measured on the Mamba-3 MIMO layer four took the call from
// 3.48 to 2.89 ms); without it four instead of two took the 2.7B layer's call
// from 3.46 to 3.33 ms (forward-direction walk) and 3.21 ms (both walks). The
// backward walk without rotation is then held to 128 VGPRs (four waves per
// SIMD), so that two workgroups of eight waves still fit a CU; with rotation
// that limit spills more and was slower (MIMO layer 1.77 -> 2.15 ms), so it
// keeps three waves per SIMD.
constexpr int bwdc_mem_waves(bool) { return 4; }
constexpr int bwdc_fwd_mem_waves(bool) { return 4; }
constexpr int bwdc_bwd_waves_per_simd(bool rot) { return rot ? 3 : 4; }

struct BwdArgs {
    const void* x;
    const float* da;
    const void* B;
    const void* C;
    const float* theta;     // [b,T,H,N/2] or null
    const float* dy;        // [b,T,R,H,P] fp32
    const float* D;         // [H] or null
    const float* init;      // [b,H,P,N] or null
    const float* dfinal;    // [b,H,P,N] or null
    const float* seg_in;    // entering (adjoint) states [b*H][S*SF][P][N] (forward walk) or
                            // [b*H][S][P][N] (backward walk), null with one segment
    float* seg_out;         // backward state pass: local adjoints [b*H][S][P][N]
    void* part;             // per-head partials [b][T*R][H][npg][N] (dC or dB): heads interleaved per row;
                            // fp32 from the step walks, bf16 from the chunked walks
    float* dx;              // [b,T,R,H,P]
    float* dinit;           // [b,H,P,N] or null
    float* final_state;     // forward walk: h_{T-1} [b,H,P,N]
    float* dDp;             // [b*H][npg][S] partial sums of dy . x
    int64_t T, H, G, N, R, P;
    int PG, S, SF, nsub, Qt, log2R;
    const float* phi;       // [b,T,H,N/2] cumulative angles (chunked walks with rotation), or null
};

// Staging of one 32-row tile by the memory waves: x, dy (as TI), B, C rows,
// and per step the decay a = exp(da) and (cos, sin) of every state pair's turn.
template <typename TI, int NP, bool WANT_X, bool WANT_B, bool WANT_C, int MW = kMemWaves>
struct Stage {
    static constexpr int ESZ = (int)sizeof(TI);
    static constexpr int EPU = 16 / ESZ;
    static constexpr int LDX = kRowGroup + 16 / ESZ;   // x and dy rows (a row group)
    static constexpr int LDB = NP + 16 / ESZ;          // B and C rows
    static constexpr int PAD = ESZ == 2 ? kPadRows : 0;  // the fp32 path reads no row past a step
    static constexpr int ROWS = kTileRows + PAD;
    static constexpr int NH = NP / 2;
    static constexpr int NTM = 64 * MW;
    static constexpr int XR = (kTileRows * kRowGroup / EPU + NTM - 1) / NTM;   // 16-byte units per memory thread
    static constexpr int DYR = (kTileRows * kRowGroup / 4 + NTM - 1) / NTM;    // dy: 4 floats per unit
    static constexpr int BRG = (kTileRows * NP / EPU + NTM - 1) / NTM;
    static constexpr int THR = (kTileRows * NH / 4 + NTM - 1) / NTM;
};

// The staging buffers, each two tiles ([2][ROWS][ld]) flattened.
template <typename TI>
struct StageMem {
    TI* sX;
    TI* sDy;
    TI* sB;
    TI* sC;
    float2* sCs;
    float* sA;
};

template <typename TI>
__device__ __forceinline__ float to_f32(TI v) {
    if constexpr (sizeof(TI) == 2) return __uint_as_float((uint32_t)v << 16);
    else return v;
}

// One memory thread's staging of tile k into registers (load) and LDS (store).
// RAW: no rotation staged, and da kept as is (the chunked walks scan it)
// instead of as the decay exp(da). TURN (bf16): B and C rows stored turned
// into the folded frame, B~ = R(-Phi_t) B, with Phi from a.phi.
template <typename TI, int NP, bool WANT_X, bool WANT_B, bool WANT_C, bool RAW = false, bool TURN = false,
          int MW = kMemWaves>
struct Stager {
    using St = Stage<TI, NP, WANT_X, WANT_B, WANT_C, MW>;
    uint4 rx[WANT_X ? St::XR : 1];
    float4 rdy[St::DYR];
    uint4 rb[WANT_B ? St::BRG : 1];
    uint4 rc[WANT_C ? St::BRG : 1];
    // the angles of a unit's pairs: B and C units of one row share them
    static constexpr bool OWN_PC = TURN && WANT_C && !WANT_B;
    float4 rpb[(TURN && WANT_B) ? St::BRG : 1], rpc[OWN_PC ? St::BRG : 1];
    float4 rth[St::THR];
    float rda;

    // the 4 pairs of v turned by R(-Phi): (e0, e1) -> (c e0 + s e1, c e1 - s e0)
    __device__ static uint4 turn(uint4 v, float4 ph) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const float pv[4] = {ph.x, ph.y, ph.z, ph.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e0 = __uint_as_float(w[i] << 16), e1 = __uint_as_float(w[i] & 0xffff0000u);
            const float rev = pv[i] * kInv2Pi;
            const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
            const float n0 = fmaf(cs, e0, sn * e1), n1 = fmaf(cs, e1, -sn * e0);
            o[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)n0) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)n1) << 16);
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    }

    // a load at a byte offset from a tile's base (the base is uniform, the
    // offset a 32-bit lane value)
    template <typename V, typename E>
    __device__ static V at(const E* base, uint32_t byteoff) {
        return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + byteoff);
    }

    __device__ void load(const BwdArgs& a, int k, int mt, int64_t b, int64_t h, int64_t g, int pbase) {
        const int64_t T = a.T, H = a.H, G = a.G, N = a.N, P = a.P, TR = a.T * a.R;
        const int64_t f0 = (int64_t)k * kTileRows, rem = TR - f0;   // rows r < rem are in range
        const int PG = a.PG;
        const int xur = PG / St::EPU, dur = PG / 4, nbu = (int)(N / St::EPU), thu = (int)(N / 8);
        // the unit counts per row are powers of two (P and N are): shifts, not divisions
        const int xurs = __builtin_ctz(xur), durs = __builtin_ctz(dur), nbus = __builtin_ctz(nbu),
                  thus = __builtin_ctz(thu);
        // rows of x and dy are H P elements apart, rows of B and C G N
        const uint32_t xrs = (uint32_t)(H * P), brs = (uint32_t)(G * N);
        if constexpr (WANT_X) {
            const TI* xt = static_cast<const TI*>(a.x) + ((b * TR + f0) * H + h) * P + pbase;
#pragma unroll
            for (int m = 0; m < St::XR; ++m) {
                const int u = mt + m * St::NTM, r = u >> xurs, c = (u & (xur - 1)) * St::EPU;
                rx[m] = (u < kTileRows * xur && r < rem) ? at<uint4>(xt, ((uint32_t)r * xrs + c) * sizeof(TI))
                                                         : make_uint4(0, 0, 0, 0);
            }
        }
        {
            const float* dyt = a.dy + ((b * TR + f0) * H + h) * P + pbase;
#pragma unroll
            for (int m = 0; m < St::DYR; ++m) {
                const int u = mt + m * St::NTM, r = u >> durs, c = (u & (dur - 1)) * 4;
                rdy[m] = (u < kTileRows * dur && r < rem) ? at<float4>(dyt, ((uint32_t)r * xrs + c) * 4u)
                                                          : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        // with TURN, the angles of the tile's steps: row r is step f0 / R + r / R
        const float* pht = nullptr;
        if constexpr (TURN) pht = a.phi + ((b * T + (f0 >> a.log2R)) * H + h) * (N / 2);
        const uint32_t prs = (uint32_t)(H * (N / 2));
        if constexpr (WANT_B) {
            const TI* Bt = static_cast<const TI*>(a.B) + ((b * TR + f0) * G + g) * N;
#pragma unroll
            for (int m = 0; m < St::BRG; ++m) {
                const int u = mt + m * St::NTM, r = u >> nbus, c = (u & (nbu - 1)) * St::EPU;
                const bool ok = u < kTileRows * nbu && r < rem;
                rb[m] = ok ? at<uint4>(Bt, ((uint32_t)r * brs + c) * sizeof(TI)) : make_uint4(0, 0, 0, 0);
                if constexpr (TURN)
                    rpb[m] = ok ? at<float4>(pht, (((uint32_t)r >> a.log2R) * prs + c / 2) * 4u)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        if constexpr (WANT_C) {
            const TI* Ct = static_cast<const TI*>(a.C) + ((b * TR + f0) * G + g) * N;
#pragma unroll
            for (int m = 0; m < St::BRG; ++m) {
                const int u = mt + m * St::NTM, r = u >> nbus, c = (u & (nbu - 1)) * St::EPU;
                const bool ok = u < kTileRows * nbu && r < rem;
                rc[m] = ok ? at<uint4>(Ct, ((uint32_t)r * brs + c) * sizeof(TI)) : make_uint4(0, 0, 0, 0);
                if constexpr (OWN_PC)
                    rpc[m] = ok ? at<float4>(pht, (((uint32_t)r >> a.log2R) * prs + c / 2) * 4u)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        const int64_t t0 = (int64_t)k * a.Qt;
        if constexpr (!RAW) {
            const float* tht = a.theta ? a.theta + ((b * T + t0) * H + h) * (N / 2) : nullptr;
#pragma unroll
            for (int m = 0; m < St::THR; ++m) {
                const int u = mt + m * St::NTM, st = u >> thus, c = (u & (thu - 1)) * 4;
                rth[m] = (tht && st < a.Qt && t0 + st < T) ? at<float4>(tht, ((uint32_t)st * prs + c) * 4u)
                                                           : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        const float* dat = a.da + (b * T + t0) * H + h;
        rda = (mt < a.Qt && t0 + mt < T) ? at<float>(dat, (uint32_t)mt * (uint32_t)H * 4u) : 0.f;
    }

    __device__ void store(const StageMem<TI>& s, const BwdArgs& a, int buf, int mt) {
        // the chunked walks read no row past a tile: their buffers hold 32 rows
        constexpr int RW = RAW ? kTileRows : St::ROWS;
        constexpr int XS = RW * St::LDX, BS = RW * St::LDB;
        const int PG = a.PG, N = (int)a.N;
        const int xur = PG / St::EPU, dur = PG / 4, nbu = N / St::EPU, thu = N / 8;
        const int xurs = __builtin_ctz(xur), durs = __builtin_ctz(dur), nbus = __builtin_ctz(nbu),
                  thus = __builtin_ctz(thu);
        if constexpr (WANT_X) {
#pragma unroll
            for (int m = 0; m < St::XR; ++m) {
                const int u = mt + m * St::NTM, r = u >> xurs, c = (u & (xur - 1)) * St::EPU;
                if (u < kTileRows * xur) *reinterpret_cast<uint4*>(&s.sX[buf * XS + r * St::LDX + c]) = rx[m];
            }
        }
#pragma unroll
        for (int m = 0; m < St::DYR; ++m) {
            const int u = mt + m * St::NTM, r = u >> durs, c = (u & (dur - 1)) * 4;
            if (u < kTileRows * dur) {
                TI* d = &s.sDy[buf * XS + r * St::LDX + c];
                if constexpr (sizeof(TI) == 2) {
                    d[0] = __builtin_bit_cast(uint16_t, (__bf16)rdy[m].x);
                    d[1] = __builtin_bit_cast(uint16_t, (__bf16)rdy[m].y);
                    d[2] = __builtin_bit_cast(uint16_t, (__bf16)rdy[m].z);
                    d[3] = __builtin_bit_cast(uint16_t, (__bf16)rdy[m].w);
                } else {
                    *reinterpret_cast<float4*>(d) = rdy[m];
                }
            }
        }
        if constexpr (WANT_B) {
#pragma unroll
            for (int m = 0; m < St::BRG; ++m) {
                const int u = mt + m * St::NTM, r = u >> nbus, c = (u & (nbu - 1)) * St::EPU;
                if (u < kTileRows * nbu)
                    *reinterpret_cast<uint4*>(&s.sB[buf * BS + r * St::LDB + c]) = TURN ? turn(rb[m], rpb[m]) : rb[m];
            }
        }
        if constexpr (WANT_C) {
#pragma unroll
            for (int m = 0; m < St::BRG; ++m) {
                const int u = mt + m * St::NTM, r = u >> nbus, c = (u & (nbu - 1)) * St::EPU;
                if (u < kTileRows * nbu)
                    *reinterpret_cast<uint4*>(&s.sC[buf * BS + r * St::LDB + c]) = TURN ? turn(rc[m], OWN_PC ? rpc[m] : rpb[m]) : rc[m];
            }
        }
#pragma unroll
        for (int m = 0; m < (RAW ? 0 : St::THR); ++m) {
            const int u = mt + m * St::NTM, st = u >> thus, c = (u & (thu - 1)) * 4;
            if (st < a.Qt) {
                const float v4[4] = {rth[m].x, rth[m].y, rth[m].z, rth[m].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float rev = v4[e] * kInv2Pi;
                    s.sCs[buf * kTileRows * St::NH + st * St::NH + c + e] =
                        make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
                }
            }
        }
        if constexpr (RAW) {
            // the first memory wave: the tile's decay sums for the compute
            // waves, per fused row m: cum_m (the sum of da over the tile's
            // steps up to m's), e^{cum_m} and e^{last - cum_m}, last = cum_31;
            // lanes 32 .. 63 repeat lanes 0 .. 31
            if (mt < 64) {
                const int m = mt & 31, rmask = (1 << a.log2R) - 1;
                float v = __shfl(rda, m >> a.log2R);
                if (m & rmask) v = 0.f;
#pragma unroll
                for (int o = 1; o < kTileRows; o <<= 1) {
                    const float u = __shfl_up(v, o);
                    if (m >= o) v += u;
                }
                const float last = __shfl(v, kTileRows - 1);
                if (mt < kTileRows) {
                    float* d = s.sA + buf * 3 * kTileRows;
                    d[m] = v;
                    d[kTileRows + m] = __expf(v);
                    d[2 * kTileRows + m] = __expf(last - v);
                }
            }
        } else {
            if (mt < a.Qt) s.sA[buf * kTileRows + mt] = __expf(rda);
        }
    }
};

// The contraction operand of one step: rows m of a 16-row block of the tile
// that belong to step s (fused rows s R .. s R + R - 1), zero elsewhere;
// k = 4 (lane / 16) .. + 3 of the 16 columns at `col`.
template <typename TI>
__device__ __forceinline__ s16x4 step_rows(const TI* tile, int ld, int blk, int r_lo, int r_hi, int col, int lane) {
    const int m = 16 * blk + (lane & 15);
    const s16x4 z = {0, 0, 0, 0};
    if (m < r_lo || m >= r_hi) return z;
    return row4(reinterpret_cast<const uint16_t*>(tile) + m * ld + col + 4 * (lane >> 4));
}

// A compute wave's share of per-head rows [32][NP] (two row blocks of NT
// accumulator tiles) into the reduction buffer: wave 0 stores, the others add
// in wave order, one barrier between waves (the caller's).
template <int NT>
__device__ __forceinline__ void put_share(float* sZ, const f32x4 (&z)[2][NT], bool first, int lane) {
    constexpr int NP = 16 * NT;
    const int q = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float* zp = &sZ[(16 * i + 4 * q + v) * NP + 16 * c + l16];
                *zp = first ? z[i][c][v] : *zp + z[i][c][v];
            }
}

// The reduced rows of a tile (those before TR) to the head's partial, whose
// rows are rs elements apart (the partials interleave the heads per row).
template <int NP>
__device__ __forceinline__ void copy_rows(const float* sZ, float* dst, int64_t f0, int64_t TR, int N, int64_t rs,
                                          int tid, int nthr) {
    const int nu = N / 4;
    for (int i = tid; i < kTileRows * nu; i += nthr) {
        const int r = i / nu, c = (i % nu) * 4;
        if (f0 + r < TR)
            *reinterpret_cast<float4*>(dst + (f0 + r) * rs + c) = *reinterpret_cast<const float4*>(&sZ[r * NP + c]);
    }
}

// ------------------------------------------------------------------------
// Forward walk: the states h_t, and per head dC_{t,r} = sum_p dy h_t[p,:]
// over the workgroup's rows p; the final state.
//
// Per tile: the memory waves stage tile k + 1 into the free buffer while the
// compute waves walk tile k, then nw barriers (the shares added in wave order)
// and one after the copy to the partial.
// ------------------------------------------------------------------------
template <typename TI, int NP>
__global__ __launch_bounds__(64 * kMaxWaves) void ssd_bwd_forward_kernel(BwdArgs a) {
    using St = Stage<TI, NP, true, true, false>;
    constexpr bool BF = sizeof(TI) == 2;
    constexpr int NT = NP / 16, LDX = St::LDX, LDB = St::LDB, NH = St::NH, ROWS = St::ROWS, PAD = St::PAD;
    __shared__ __attribute__((aligned(16))) TI sX[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sDy[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sB[2][ROWS * LDB];
    __shared__ __attribute__((aligned(16))) float2 sCs[2][kTileRows * NH];
    __shared__ float sA[2][kTileRows];
    __shared__ __attribute__((aligned(16))) float sZ[kTileRows * NP];
    const StageMem<TI> sm{&sX[0][0], &sDy[0][0], &sB[0][0], nullptr, &sCs[0][0], &sA[0][0]};

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, R = a.R, P = a.P, TR = T * R;
    const int PG = a.PG, nw = PG >> 4, S = a.S, npg = (int)(P / PG), Qt = a.Qt, Ri = (int)R;
    const bool memw = wv >= nw;
    const int mt = tid - 64 * nw;
    int item = blockIdx.x;
    const int seg = item % S;
    item /= S;
    const int pg = item % npg;
    const int64_t bh = item / npg;
    const int64_t b = bh / H, h = bh % H, g = h / (H / G);
    const int k0 = (int)(((int64_t)seg * a.nsub) / S), k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    const int pbase = pg * PG;
    float* dst = static_cast<float*>(a.part) + ((b * TR * H + h) * npg + pg) * N;   // [b][TR][H][npg][N]

    if constexpr (PAD > 0)
        for (int i = tid; i < 2 * PAD * LDX; i += nthr) {
            sX[i / (PAD * LDX)][kTileRows * LDX + i % (PAD * LDX)] = TI(0);
            sDy[i / (PAD * LDX)][kTileRows * LDX + i % (PAD * LDX)] = TI(0);
        }
    for (int i = tid; i < 2 * ROWS * LDB; i += nthr) sB[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
    __syncthreads();

    if (memw) {
        Stager<TI, NP, true, true, false> st;
        st.load(a, k0, mt, b, h, g, pbase);
        st.store(sm, a, 0, mt);
        __syncthreads();
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            if (k + 1 < k1) {
                st.load(a, k + 1, mt, b, h, g, pbase);
                st.store(sm, a, buf ^ 1, mt);
            }
            for (int w = 0; w < nw; ++w) __syncthreads();
            copy_rows<NP>(sZ, dst, (int64_t)k * kTileRows, TR, (int)N, H * npg * N, tid, nthr);
            __syncthreads();
        }
        return;
    }

    // ---- compute waves: state tiles D[p][n] of rows p0 .. p0 + 15
    const int p0 = pbase + 16 * wv, xcol = 16 * wv;
    f32x4 hs[NT];
    {
        const float* src = (S == 1) ? a.init : a.seg_in;
        const int64_t off = (S == 1) ? bh * P * N : (bh * S + seg) * (int64_t)a.SF * P * N;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                hs[c][v] = (src && n < N) ? src[off + (int64_t)(p0 + 4 * q + v) * N + n] : 0.f;
        }
    }
    const int kr0 = (4 * q < Ri) ? 4 * q : 0;
    __syncthreads();
    for (int k = k0; k < k1; ++k) {
        const int buf = (k - k0) & 1;
        f32x4 z[2][NT];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int c = 0; c < NT; ++c) z[i][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < Qt; ++s) {
            const int64_t t = (int64_t)k * Qt + s;
            if (t >= T) break;
            // decay and turn: h <- a R(theta) h
            const float at = sA[buf][s];
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int n = 16 * c + l16;
                const float2 cs = (n < N) ? sCs[buf][s * NH + (n >> 1)] : make_float2(1.f, 0.f);
                const float self = at * cs.x, part = (n & 1) ? at * cs.y : -at * cs.y;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float pv = swap_pair(hs[c][v]);
                    hs[c][v] = fmaf(self, hs[c][v], part * pv);
                }
            }
            const int row = s * Ri;
            const int blk = row >> 4;
            if constexpr (BF) {
                // the rank-R write x (outer) B
                s16x4 xa = tr_rows4(reinterpret_cast<const uint16_t*>(sX[buf]), LDX, row + kr0, xcol, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * q + e >= Ri) xa[e] = 0;
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const s16x4 bb = tr_rows4(reinterpret_cast<const uint16_t*>(sB[buf]), LDB, row + kr0, 16 * c, lane);
                    hs[c] = mma16(xa, bb, hs[c]);
                }
                // dC share: rows of this step, dy (k = p) times the state tiles
                const s16x4 dya = step_rows<TI>(sDy[buf], LDX, blk, row, row + Ri, xcol, lane);
                if (blk == 0) {
#pragma unroll
                    for (int c = 0; c < NT; ++c) z[0][c] = mma16(dya, pack4_bf16(hs[c]), z[0][c]);
                } else {
#pragma unroll
                    for (int c = 0; c < NT; ++c) z[1][c] = mma16(dya, pack4_bf16(hs[c]), z[1][c]);
                }
            } else {
                for (int j = 0; 4 * j < Ri; ++j) {
                    const int r = 4 * j + q, rr = r < Ri ? r : 0;
                    const float xv = r < Ri ? (float)sX[buf][(row + rr) * LDX + xcol + l16] : 0.f;
#pragma unroll
                    for (int c = 0; c < NT; ++c)
                        hs[c] = mma4f(xv, (float)sB[buf][(row + rr) * LDB + 16 * c + l16], hs[c]);
                }
                const int m = 16 * blk + l16;
                const bool mine = m >= row && m < row + Ri;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float dv = mine ? (float)sDy[buf][m * LDX + xcol + 4 * q + v] : 0.f;
                    if (blk == 0) {
#pragma unroll
                        for (int c = 0; c < NT; ++c) z[0][c] = mma4f(dv, hs[c][v], z[0][c]);
                    } else {
#pragma unroll
                        for (int c = 0; c < NT; ++c) z[1][c] = mma4f(dv, hs[c][v], z[1][c]);
                    }
                }
            }
        }
        for (int w = 0; w < nw; ++w) {
            if (wv == w) put_share<NT>(sZ, z, w == 0, lane);
            __syncthreads();
        }
        copy_rows<NP>(sZ, dst, (int64_t)k * kTileRows, TR, (int)N, H * npg * N, tid, nthr);
        __syncthreads();
    }
    if (seg == S - 1 && a.final_state) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (n < N) a.final_state[bh * P * N + (int64_t)(p0 + 4 * q + v) * N + n] = hs[c][v];
        }
    }
}

// ------------------------------------------------------------------------
// Backward walk (tiles and steps in reverse): the state gradient in both
// layouts, Hp = D[p][n] (for dB) and Hn = D[n][p] (for dx). MODE 1: the
// segment's own contribution at its left end (from a zero gradient), for the
// carry; MODE 0: dx, the head's dB partial, the dy . x partial, dinit.
// ------------------------------------------------------------------------
template <typename TI, int NP, int MODE>
__global__ __launch_bounds__(64 * kMaxWaves) void ssd_bwd_backward_kernel(BwdArgs a) {
    constexpr bool OUT = MODE == 0;
    using St = Stage<TI, NP, OUT, OUT, true>;
    constexpr bool BF = sizeof(TI) == 2;
    constexpr int NT = NP / 16, LDX = St::LDX, LDB = St::LDB, NH = St::NH, ROWS = St::ROWS, PAD = St::PAD;
    __shared__ __attribute__((aligned(16))) TI sX[2][OUT ? ROWS * LDX : 8];
    __shared__ __attribute__((aligned(16))) TI sDy[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sB[2][OUT ? ROWS * LDB : 8];
    __shared__ __attribute__((aligned(16))) TI sC[2][ROWS * LDB];
    __shared__ __attribute__((aligned(16))) float2 sCs[2][kTileRows * NH];
    __shared__ float sA[2][kTileRows];
    __shared__ __attribute__((aligned(16))) float sZ[OUT ? kTileRows * NP : 4];
    __shared__ float sDd[kRowGroup / 16];
    const StageMem<TI> sm{&sX[0][0], &sDy[0][0], &sB[0][0], &sC[0][0], &sCs[0][0], &sA[0][0]};

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, R = a.R, P = a.P, TR = T * R;
    const int PG = a.PG, nw = PG >> 4, S = a.S, npg = (int)(P / PG), Qt = a.Qt, Ri = (int)R;
    const bool memw = wv >= nw;
    const int mt = tid - 64 * nw;
    int item = blockIdx.x;
    const int seg = item % S;
    item /= S;
    const int pg = item % npg;
    const int64_t bh = item / npg;
    const int64_t b = bh / H, h = bh % H, g = h / (H / G);
    const int k0 = (int)(((int64_t)seg * a.nsub) / S), k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    // the state pass: the first segment's local gradient is never used (the
    // carry starts from dfinal), so its workgroups leave at once, together
    if (!OUT && seg == 0) return;
    const int pbase = pg * PG;
    float* dst = OUT ? static_cast<float*>(a.part) + ((b * TR * H + h) * npg + pg) * N : nullptr;

    if constexpr (PAD > 0)
        for (int i = tid; i < 2 * PAD * LDX; i += nthr) {
            if (OUT) sX[i / (PAD * LDX)][kTileRows * LDX + i % (PAD * LDX)] = TI(0);
            sDy[i / (PAD * LDX)][kTileRows * LDX + i % (PAD * LDX)] = TI(0);
        }
    for (int i = tid; i < 2 * ROWS * LDB; i += nthr) {
        if (OUT) sB[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
        sC[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
    }
    __syncthreads();

    if (memw) {
        Stager<TI, NP, OUT, OUT, true> st;
        if (k1 > k0) {
            st.load(a, k1 - 1, mt, b, h, g, pbase);
            st.store(sm, a, 0, mt);
        }
        __syncthreads();
        for (int k = k1 - 1; k >= k0; --k) {
            const int buf = (k1 - 1 - k) & 1;
            if (k > k0) {
                st.load(a, k - 1, mt, b, h, g, pbase);
                st.store(sm, a, buf ^ 1, mt);
            }
            if constexpr (OUT) {
                for (int w = 0; w < nw; ++w) __syncthreads();
                copy_rows<NP>(sZ, dst, (int64_t)k * kTileRows, TR, (int)N, H * npg * N, tid, nthr);
            }
            __syncthreads();
        }
        __syncthreads();                           // the dy . x shares
        return;
    }

    // ---- compute waves
    const int p0 = pbase + 16 * wv, xcol = 16 * wv;
    f32x4 hp[NT], hn[NT];                          // D[p][n] and D[n][p] tiles
    {
        const float* src = nullptr;
        int64_t off = 0;
        if (OUT) {
            if (seg == S - 1) {
                src = a.dfinal;
                off = bh * P * N;
            } else {
                src = a.seg_in;
                off = (bh * S + seg) * P * N;
            }
        }
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                hp[c][v] = (src && n < N) ? src[off + (int64_t)(p0 + 4 * q + v) * N + n] : 0.f;
                const int nn = 16 * c + 4 * q + v;
                hn[c][v] = (src && nn < N) ? src[off + (int64_t)(p0 + l16) * N + nn] : 0.f;
            }
        }
    }
    const int kr0 = (4 * q < Ri) ? 4 * q : 0;
    const float Dh = (OUT && a.D) ? a.D[h] : 0.f;
    float dd = 0.f;                                // this lane's share of sum dy . x
    __syncthreads();
    for (int k = k1 - 1; k >= k0; --k) {
        const int buf = (k1 - 1 - k) & 1;
        f32x4 zb[2][OUT ? NT : 1], zx[2];
        if constexpr (OUT) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                zx[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NT; ++c) zb[i][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        }
        for (int s = Qt - 1; s >= 0; --s) {
            const int64_t t = (int64_t)k * Qt + s;
            if (t >= T) continue;
            const int row = s * Ri;
            const int blk = row >> 4;
            // the reads of step t: H += sum_r dy_{t,r} (outer) C_{t,r}
            if constexpr (BF) {
                s16x4 dyM = tr_rows4(reinterpret_cast<const uint16_t*>(sDy[buf]), LDX, row + kr0, xcol, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * q + e >= Ri) dyM[e] = 0;
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    s16x4 cc = tr_rows4(reinterpret_cast<const uint16_t*>(sC[buf]), LDB, row + kr0, 16 * c, lane);
                    hp[c] = mma16(dyM, cc, hp[c]);     // D[p][n]: A = dy^T (rows p), B = C
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q + e >= Ri) cc[e] = 0;
                    hn[c] = mma16(cc, dyM, hn[c]);     // D[n][p]: A = C^T (rows n), B = dy
                }
            } else {
                for (int j = 0; 4 * j < Ri; ++j) {
                    const int r = 4 * j + q, rr = r < Ri ? r : 0;
                    const float dv = r < Ri ? (float)sDy[buf][(row + rr) * LDX + xcol + l16] : 0.f;
#pragma unroll
                    for (int c = 0; c < NT; ++c) {
                        const float cv = r < Ri ? (float)sC[buf][(row + rr) * LDB + 16 * c + l16] : 0.f;
                        hp[c] = mma4f(dv, cv, hp[c]);
                        hn[c] = mma4f(cv, dv, hn[c]);
                    }
                }
            }
            if constexpr (OUT) {
                // dx rows of step t: B (k = n) times Hn; dB share: x (k = p) times Hp
                if constexpr (BF) {
                    const s16x4 xs = step_rows<TI>(sX[buf], LDX, blk, row, row + Ri, xcol, lane);
#pragma unroll
                    for (int c = 0; c < NT; ++c) {
                        const s16x4 bs = step_rows<TI>(sB[buf], LDB, blk, row, row + Ri, 16 * c, lane);
                        if (blk == 0) {
                            zx[0] = mma16(bs, pack4_bf16(hn[c]), zx[0]);
                            zb[0][c] = mma16(xs, pack4_bf16(hp[c]), zb[0][c]);
                        } else {
                            zx[1] = mma16(bs, pack4_bf16(hn[c]), zx[1]);
                            zb[1][c] = mma16(xs, pack4_bf16(hp[c]), zb[1][c]);
                        }
                    }
                } else {
                    const int m = 16 * blk + l16;
                    const bool mine = m >= row && m < row + Ri;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float xv = mine ? (float)sX[buf][m * LDX + xcol + 4 * q + v] : 0.f;
#pragma unroll
                        for (int c = 0; c < NT; ++c) {
                            const float bv = mine ? (float)sB[buf][m * LDB + 16 * c + 4 * q + v] : 0.f;
                            if (blk == 0) {
                                zx[0] = mma4f(bv, hn[c][v], zx[0]);
                                zb[0][c] = mma4f(xv, hp[c][v], zb[0][c]);
                            } else {
                                zx[1] = mma4f(bv, hn[c][v], zx[1]);
                                zb[1][c] = mma4f(xv, hp[c][v], zb[1][c]);
                            }
                        }
                    }
                }
            }
            // into step t - 1: H <- a_t R(theta_t)^T H
            const float at = sA[buf][s];
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int n = 16 * c + l16;
                const float2 cs = (n < N) ? sCs[buf][s * NH + (n >> 1)] : make_float2(1.f, 0.f);
                const float self = at * cs.x, part = (n & 1) ? -at * cs.y : at * cs.y;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float pv = swap_pair(hp[c][v]);
                    hp[c][v] = fmaf(self, hp[c][v], part * pv);
                }
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    const int nn = 16 * c + 4 * q + v;   // even: pair (nn, nn + 1) in this lane
                    const float2 cp = (nn < N) ? sCs[buf][s * NH + (nn >> 1)] : make_float2(1.f, 0.f);
                    const float e0 = hn[c][v], e1 = hn[c][v + 1];
                    hn[c][v] = at * fmaf(cp.x, e0, cp.y * e1);
                    hn[c][v + 1] = at * fmaf(cp.x, e1, -cp.y * e0);
                }
            }
        }
        if constexpr (OUT) {
            // dx = zx + D dy for the tile's rows, this wave's 16 columns (dy and
            // the dy . x sum from the fp32 dy)
            const int64_t f0 = (int64_t)k * kTileRows;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * i + 4 * q + v;
                    if (f0 + r < TR) {
                        const int64_t o = ((b * TR + f0 + r) * H + h) * P + p0 + l16;
                        const float dyv = a.dy[o];
                        a.dx[o] = fmaf(Dh, dyv, zx[i][v]);
                        dd = fmaf(dyv, to_f32(sX[buf][r * LDX + xcol + l16]), dd);
                    }
                }
            for (int w = 0; w < nw; ++w) {
                if (wv == w) put_share<NT>(sZ, zb, w == 0, lane);
                __syncthreads();
            }
            copy_rows<NP>(sZ, dst, f0, TR, (int)N, H * npg * N, tid, nthr);
        }
        __syncthreads();
    }
    // the state gradient at the segment's left end (after its first step's
    // decay and turn): the carry's local term (MODE 1), or dinit (segment 0)
    float* out = nullptr;
    if (!OUT && seg > 0) out = a.seg_out + (bh * S + seg) * P * N;
    if (OUT && seg == 0 && a.dinit) out = a.dinit + bh * P * N;
    if (out) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (n < N) out[(int64_t)(p0 + 4 * q + v) * N + n] = hp[c][v];
        }
    }
    if constexpr (OUT) {
        for (int o = 32; o >= 1; o >>= 1) dd += __shfl_xor(dd, o);
        if (lane == 0) sDd[wv] = dd;
    }
    __syncthreads();
    if (OUT && tid == 0) {
        float acc = 0.f;
        for (int w = 0; w < nw; ++w) acc += sDd[w];
        a.dDp[(bh * npg + pg) * S + seg] = acc;
    }
}

// ------------------------------------------------------------------------
// Chunked walks (bf16 inputs, no rotation, headdim <= 64): one workgroup per
// (batch, head, segment) holds the whole head. Per 32-row tile, with cum_m the
// inclusive sum of da over the tile's steps up to row m's step:
//   forward:  dC  = e^{cum} o (dy h_in) + (G o L) B,   G = dy x^T (rows m, j)
//             h  <- e^{cum_last} h + (w o x)^T B,     w_j = e^{cum_last - cum_j}
//   backward: dx  = w o (B H^T) + (CB^T o L')^T dy     (CB^T)[j][m] = C_j . B_m
//             dB  = w o (x H)   + (G^T o L'^T) C
//             H  <- e^{cum_last} H + (e^{cum} o dy)^T C
// with H the state gradient entering the tile from its right, L the causal
// decay e^{cum_m - cum_j} (step(j) <= step(m)) and L' its transpose. The
// 32 x 32 products are three 16 x 16 blocks each, built by one wave per block
// and shared through LDS.
// ------------------------------------------------------------------------

constexpr int kLdm = 24;             // row stride of a staged 16 x 16 block (bf16)

// A tile's decay sums, staged per fused row m by the memory waves: cum_m at
// [m], e^{cum_m} at [32 + m] and e^{last - cum_m} at [64 + m].
constexpr int kCumE = kTileRows, kCumW = 2 * kTileRows;

// D[m][j] = sum_k ta[mrow0 + m][k] tb[jrow0 + j][k] over k < K: rows of two
// row-major bf16 tiles dotted along their columns (K a multiple of 16)
__device__ __forceinline__ f32x4 rows_dot(const uint16_t* ta, int lda, int mrow0, const uint16_t* tb, int ldb,
                                          int jrow0, int K, int lane) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int l16 = lane & 15, q = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 16)
        acc = mma16(row4(ta + (mrow0 + l16) * lda + k0 + 4 * q), row4(tb + (jrow0 + l16) * ldb + k0 + 4 * q), acc);
    return acc;
}

// One 16 x 16 block (rows m in block mb, columns j in block jb) of a 32 x 32
// tile matrix, decay-masked: upper (step(j) >= step(m), factor e^{cum_j - cum_m})
// or lower (step(j) <= step(m), e^{cum_m - cum_j}); stored as bf16 [m][j].
__device__ __forceinline__ void put_masked(uint16_t* dst, f32x4 acc, int mb, int jb, bool upper, const float* cum,
                                           int log2R, int lane) {
    const int l16 = lane & 15, q = lane >> 4;
    const int j = 16 * jb + l16;
    const float cj = cum[j];
    const float4 c4 = *reinterpret_cast<const float4*>(cum + 16 * mb + 4 * q);
    const float cmv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 16 * mb + 4 * q + v;
        const float cm = cmv[v];
        const int sm = m >> log2R, sj = j >> log2R;
        float val = 0.f;
        if (upper ? (sj >= sm) : (sj <= sm)) val = acc[v] * __expf(upper ? cj - cm : cm - cj);
        dst[(4 * q + v) * kLdm + l16] = __builtin_bit_cast(uint16_t, (__bf16)val);
    }
}

// the A operand of rows m = 16 mb + (lane % 16), columns 4 (lane / 16) .. + 3
// of a staged block
__device__ __forceinline__ s16x4 blk_rows(const uint16_t* blk, int lane) {
    return row4(blk + (lane & 15) * kLdm + 4 * (lane >> 4));
}

__device__ __forceinline__ s16x4 scale4(s16x4 v, float a, float b, float c, float d) {
    f32x4 f = {__uint_as_float((uint32_t)(uint16_t)v[0] << 16) * a, __uint_as_float((uint32_t)(uint16_t)v[1] << 16) * b,
               __uint_as_float((uint32_t)(uint16_t)v[2] << 16) * c, __uint_as_float((uint32_t)(uint16_t)v[3] << 16) * d};
    return pack4_bf16(f);
}

// Products of contraction length 32 (v_mfma_f32_16x16x32_bf16, twice the work
// of the 16 x 16 x 16 form in the same cycles). Operand layout: lane l holds
// row (A) or column (B) l % 16 and k = 8 (l / 16) .. + 7; the result as mma16.
typedef __attribute__((ext_vector_type(8))) short s16x8;

__device__ __forceinline__ f32x4 mma32(s16x8 a, s16x8 b, f32x4 c) {
    typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// eight consecutive elements of one row (16 bytes, 16-byte aligned)
__device__ __forceinline__ s16x8 row8(const uint16_t* p) { return *reinterpret_cast<const s16x8*>(p); }

__device__ __forceinline__ s16x8 cat8(s16x4 lo, s16x4 hi) {
    return (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// rows r0 .. r0 + 7 of column colbase + (lane % 16) of a row-major tile
__device__ __forceinline__ s16x8 tr_rows8(const uint16_t* tile, int ld, int r0, int colbase, int lane) {
    return cat8(tr_rows4(tile, ld, r0, colbase, lane), tr_rows4(tile, ld, r0 + 4, colbase, lane));
}

__device__ __forceinline__ s16x8 scale8(s16x8 v, float4 a, float4 b) {
    const s16x4 lo = scale4((s16x4){v[0], v[1], v[2], v[3]}, a.x, a.y, a.z, a.w);
    const s16x4 hi = scale4((s16x4){v[4], v[5], v[6], v[7]}, b.x, b.y, b.z, b.w);
    return cat8(lo, hi);
}

// A operand of the 16 x 32 block row [left | right] of two staged 16 x 16
// blocks; a null half is zero (a block the causal mask removes)
__device__ __forceinline__ s16x8 blk_pair(const uint16_t* left, const uint16_t* right, int lane) {
    const int l16 = lane & 15, q = lane >> 4;
    const uint16_t* blk = q < 2 ? left : right;
    s16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (blk) v = row8(blk + l16 * kLdm + 8 * (q & 1));
    return v;
}

// rows_dot with contraction length 32 (K a multiple of 32)
template <int K>
__device__ __forceinline__ f32x4 rows_dot32(const uint16_t* ta, int lda, int mrow0, const uint16_t* tb, int ldb,
                                            int jrow0, int lane) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int l16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32)
        acc = mma32(row8(ta + (mrow0 + l16) * lda + k0 + 8 * q), row8(tb + (jrow0 + l16) * ldb + k0 + 8 * q), acc);
    return acc;
}

// A compute wave's share of per-head rows [32][NP] in its own LDS slot, in
// accumulator order: fragment (i, c, lane) holds rows 16 i + 4 q + v of
// column 16 c + l16.
template <int NT>
__device__ __forceinline__ void put_frags(float4* slot, const f32x4 (&z)[2][NT], int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < NT; ++c)
            slot[(i * NT + c) * 64 + lane] = make_float4(z[i][c][0], z[i][c][1], z[i][c][2], z[i][c][3]);
}

// The nw slots added in wave order and stored as the rows f0 + r (< TR) of dst.
template <int NT>
__device__ __forceinline__ void sum_frags(const float4* slots, int nw, float* dst, int64_t f0, int64_t TR, int N,
                                          int64_t rs, int tid, int nthr) {
    constexpr int NF = 2 * NT * 64;
    for (int f = tid; f < NF; f += nthr) {
        float4 acc = slots[f];
        for (int w = 1; w < nw; ++w) {
            const float4 v = slots[w * NF + f];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const int ln = f & 63, ic = f >> 6, i = ic / NT, c = ic % NT;
        const int n = 16 * c + (ln & 15), r0 = 16 * i + 4 * (ln >> 4);
        if (n >= N) continue;
        const float av[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (f0 + r0 + v < TR) dst[(f0 + r0 + v) * rs + n] = av[v];
    }
}


// Frame changes of state tiles: every state pair (2k, 2k+1) turned by
// R(sgn Phi[k]) (phirow: the angles of one step, one head). Layout D[p][n]
// (pairs in neighbouring lanes) and D[n][p] (pairs in one lane).
template <int NT>
__device__ __forceinline__ void turn_pn(f32x4 (&hs)[NT], const float* phirow, int N, float sgn, int lane) {
    const int l16 = lane & 15;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int n = 16 * c + l16;
        const float rev = (n < N ? phirow[n >> 1] : 0.f) * sgn * kInv2Pi;
        const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
        const float part = (n & 1) ? sn : -sn;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float pv = swap_pair(hs[c][v]);
            hs[c][v] = fmaf(cs, hs[c][v], part * pv);
        }
    }
}

template <int NT>
__device__ __forceinline__ void turn_np(f32x4 (&hn)[NT], const float* phirow, int N, float sgn, int lane) {
    const int q = lane >> 4;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
            const int nn = 16 * c + 4 * q + v;
            const float rev = (nn < N ? phirow[nn >> 1] : 0.f) * sgn * kInv2Pi;
            const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
            const float e0 = hn[c][v], e1 = hn[c][v + 1];
            hn[c][v] = fmaf(cs, e0, -sn * e1);
            hn[c][v + 1] = fmaf(sn, e0, cs * e1);
        }
}

// The state entering a tile, as bf16 [n][p] (row stride kLdh): every compute
// wave puts its rows p0 .. p0 + 15 (accumulator layout D[p][n]) so that each
// wave can contract over all p for its own column tiles.
constexpr int kLdh = kRowGroup + 8;

template <int NT>
__device__ __forceinline__ void put_state(uint16_t* sH, const f32x4 (&hs)[NT], int p0, int lane) {
    const int q = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int c = 0; c < NT; ++c) *reinterpret_cast<s16x4*>(sH + (16 * c + l16) * kLdh + p0 + 4 * q) = pack4_bf16(hs[c]);
}

// Rows [f0, f0 + 32) of a row-major fp32 array (row stride rs floats, `base`
// at row 0) as a buffer resource that ends at row TR: stores to later rows are
// dropped and loads from them read zero, with no branch. The byte range fits
// 32 bits (the host checks 32 H max(P, N) 4 bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rows(const float* base, int64_t f0, int64_t TR, int64_t rs) {
    const int64_t rem = TR - f0, rows = rem < kTileRows ? rem : kTileRows;
    return make_rsrc(base + f0 * rs, (uint32_t)(rows * rs * 4));
}

// The same rows of a row-major bf16 array.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rows16(const uint16_t* base, int64_t f0, int64_t TR,
                                                              int64_t rs) {
    const int64_t rem = TR - f0, rows = rem < kTileRows ? rem : kTileRows;
    return make_rsrc(base + f0 * rs, (uint32_t)(rows * rs * 2));
}

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4v;

// A tile computed transposed (the product's operands swapped, so that a lane
// holds row l16 and the four columns 4 q .. 4 q + 3 of a 16-column tile):
// rows i16 + l16 (i16 = 0, 16), rounded to bf16 (to nearest even), one 8-byte
// store per row from the lane's byte offset voff (row l16, column 4 q)
__device__ __forceinline__ void store_tile_cols16(__amdgpu_buffer_rsrc_t rsrc, const f32x4& z0, const f32x4& z1,
                                                  uint32_t voff, uint32_t rowb, uint32_t colb) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4_bf16(z0)), rsrc, voff, colb, 0);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4_bf16(z1)), rsrc, voff, colb + 16 * rowb, 0);
}

// Forward direction: the head's dC partial rows and the final state. ROT: in
// the folded frame g = R(-Phi) h (B~, C~ turned while staged; the partial
// rows are dC~, turned back in the reduction). Each compute wave keeps rows
// p0 .. p0 + 15 of the state and, for the partial, takes the column tiles
// c = wv, wv + nw, ... with the contraction over every p read from the staged
// entering state.
template <int NP, bool ROT>
__global__ __launch_bounds__(64 * (kRowGroup / 16 + bwdc_fwd_mem_waves(ROT))) void ssd_bwdc_forward_kernel(BwdArgs a) {
    using TI = uint16_t;
    constexpr int MW = bwdc_fwd_mem_waves(ROT);
    using St = Stage<TI, NP, true, true, false, MW>;
    constexpr int NT = NP / 16, LDX = St::LDX, LDB = St::LDB, ROWS = kTileRows;
    __shared__ __attribute__((aligned(16))) TI sX[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sDy[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sB[2][ROWS * LDB];
    __shared__ __attribute__((aligned(16))) float sA[2][3 * kTileRows];
    __shared__ __attribute__((aligned(16))) uint16_t sM[3][16 * kLdm];
    __shared__ __attribute__((aligned(16))) uint16_t sH[NP * kLdh];
    const StageMem<TI> sm{&sX[0][0], &sDy[0][0], &sB[0][0], nullptr, nullptr, &sA[0][0]};

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, R = a.R, P = a.P, TR = T * R;
    const int nw = (int)(P >> 4), S = a.S, Qt = a.Qt, log2R = a.log2R;
    const bool memw = wv >= nw;
    const int mt = tid - 64 * nw;
    const int seg = blockIdx.x % S;
    const int64_t bh = blockIdx.x / S;
    const int64_t b = bh / H, h = bh % H, g = h / (H / G);
    const int k0 = (int)(((int64_t)seg * a.nsub) / S), k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    uint16_t* dst = static_cast<uint16_t*>(a.part) + (b * TR * H + h) * N;   // [b][TR][H][N], bf16
    const int64_t rs = H * N;
    // lane byte offset of the partial tiles (computed transposed): row l16, column 4 q
    const uint32_t prow = (uint32_t)((l16 * rs + 4 * q) * 2), rowb = (uint32_t)(rs * 2);

    // columns n >= N of B, p >= P of x and dy, and of the staged state stay
    // zero (the contractions over p always run over the 64 rows of a group)
    for (int i = tid; i < 2 * ROWS * LDB; i += blockDim.x) sB[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
    for (int i = tid; i < 2 * ROWS * LDX; i += blockDim.x) {
        sX[i / (ROWS * LDX)][i % (ROWS * LDX)] = TI(0);
        sDy[i / (ROWS * LDX)][i % (ROWS * LDX)] = TI(0);
    }
    for (int i = tid; i < NP * kLdh; i += blockDim.x) sH[i] = 0;
    __syncthreads();

    if (memw) {
        Stager<TI, NP, true, true, false, true, ROT, MW> st;
        if (k1 > k0) {
            st.load(a, k0, mt, b, h, g, 0);
            st.store(sm, a, 0, mt);
            if (k0 + 1 < k1) st.load(a, k0 + 1, mt, b, h, g, 0);
        }
        __syncthreads();
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            if (k + 1 < k1) {
                st.store(sm, a, buf ^ 1, mt);
                if (k + 2 < k1) st.load(a, k + 2, mt, b, h, g, 0);
            }
            __syncthreads();                               // blocks built, entering state put
            __syncthreads();                               // tile walked
        }
        return;
    }

    const int p0 = 16 * wv;
    f32x4 hs[NT];                                  // D[p][n]: rows p0 + 4q + v, column 16c + l16
    {
        const float* src = (S == 1) ? a.init : a.seg_in;
        const int64_t off = (S == 1) ? bh * P * N : (bh * S + seg) * (int64_t)a.SF * P * N;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                hs[c][v] = (src && n < N) ? src[off + (int64_t)(p0 + 4 * q + v) * N + n] : 0.f;
        }
        // the physical state entering a later segment, into the folded frame
        if (ROT && S > 1 && seg > 0)
            turn_pn<NT>(hs, a.phi + ((b * T + (int64_t)k0 * Qt - 1) * H + h) * (N / 2), (int)N, -1.f, lane);
    }
    __syncthreads();
    for (int k = k0; k < k1; ++k) {
        const int buf = (k - k0) & 1;
        const uint16_t* tX = reinterpret_cast<const uint16_t*>(sX[buf]);
        const uint16_t* tDy = reinterpret_cast<const uint16_t*>(sDy[buf]);
        const uint16_t* tB = reinterpret_cast<const uint16_t*>(sB[buf]);
        const float* cum = sA[buf];
        put_state<NT>(sH, hs, p0, lane);
        // G o L blocks (0,0), (1,0), (1,1): rows m of dy against rows j of x
        for (int u = wv; u < 3; u += nw) {
            const int mb = u == 0 ? 0 : 1, jb = u == 2 ? 1 : 0;
            const f32x4 gacc = rows_dot32<kRowGroup>(tDy, LDX, 16 * mb, tX, LDX, 16 * jb, lane);
            put_masked(sM[u], gacc, mb, jb, false, cum, log2R, lane);
        }
        __syncthreads();
        // dC = e^{cum_m} (dy h_in) + (G o L) B on the wave's column tiles,
        // computed transposed (lane: step row 16 i + l16, four columns)
        float ein[2];
        s16x8 dya[2][kRowGroup / 32];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            ein[i] = cum[kCumE + 16 * i + l16];
#pragma unroll
            for (int kb = 0; kb < kRowGroup / 32; ++kb)
                dya[i][kb] = row8(tDy + (16 * i + l16) * LDX + 32 * kb + 8 * q);
        }
        // block rows [G o L (0,0) | 0] and [(1,0) | (1,1)]
        const s16x8 m0 = blk_pair(sM[0], nullptr, lane), m1 = blk_pair(sM[1], sM[2], lane);
        const auto prs = tile_rows16(dst, (int64_t)k * kTileRows, TR, rs);
        // the wave's dC column tiles c = wv, wv + nw, ...
        auto dc_tile = [&](int c) {
            f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < kRowGroup / 32; ++kb) {
                const s16x8 hb = row8(sH + (16 * c + l16) * kLdh + 32 * kb + 8 * q);
                z0 = mma32(hb, dya[0][kb], z0);
                z1 = mma32(hb, dya[1][kb], z1);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                z0[v] *= ein[0];
                z1[v] *= ein[1];
            }
            const s16x8 bb = tr_rows8(tB, LDB, 8 * q, 16 * c, lane);
            z0 = mma32(bb, m0, z0);
            z1 = mma32(bb, m1, z1);
            store_tile_cols16(prs, z0, z1, prow, rowb, 32u * c);
        };
        if (NT % (kRowGroup / 16) == 0 && nw == kRowGroup / 16 && N == NP) {
            // four compute waves and every column tile in range: unrolled, so
            // that one tile's LDS reads overlap the other's products
#pragma unroll
            for (int j = 0; j < NT / (kRowGroup / 16); ++j) dc_tile(wv + (kRowGroup / 16) * j);
        } else {
            // N is a multiple of 16: a column tile is all in range or all out
            for (int c = wv; c < NT && 16 * c < N; c += nw) dc_tile(c);
        }
        // h <- e^{last} h + (w o x)^T B, contracted over the tile's 32 rows
        const float carry = cum[kCumE + kTileRows - 1];
        const s16x8 xw = scale8(tr_rows8(tX, LDX, 8 * q, p0, lane),
                                *reinterpret_cast<const float4*>(cum + kCumW + 8 * q),
                                *reinterpret_cast<const float4*>(cum + kCumW + 8 * q + 4));
#pragma unroll
        for (int c = 0; c < NT; ++c) {
#pragma unroll
            for (int v = 0; v < 4; ++v) hs[c][v] *= carry;
            hs[c] = mma32(xw, tr_rows8(tB, LDB, 8 * q, 16 * c, lane), hs[c]);
        }
        __syncthreads();                           // tile walked: its buffers and sH free
    }
    if (seg == S - 1 && a.final_state) {
        if (ROT) turn_pn<NT>(hs, a.phi + ((b * T + T - 1) * H + h) * (N / 2), (int)N, 1.f, lane);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (n < N) a.final_state[bh * P * N + (int64_t)(p0 + 4 * q + v) * N + n] = hs[c][v];
        }
    }
}

// Backward direction (tiles in reverse). MODE 1: only the state gradient, from
// zero, to the segment's left end (the carry's local term); MODE 0: dx, the
// head's dB partial, the dy . x partial and dinit. ROT: the gradient of the
// folded state G = R(-Phi) H, converted at the segment ends. Each compute wave
// keeps rows p0 .. p0 + 15 of the state gradient; MODE 0 stages the entering
// one as bf16 [n][p], read transposed for dx and, for the dB partial on the
// wave's column tiles c = wv, wv + nw, ..., contracted over every p.
template <int NP, int MODE, bool ROT>
__global__ __launch_bounds__(64 * (kRowGroup / 16 + bwdc_mem_waves(ROT)))
__attribute__((amdgpu_waves_per_eu(bwdc_bwd_waves_per_simd(ROT)))) void ssd_bwdc_backward_kernel(BwdArgs a) {
    using TI = uint16_t;
    constexpr bool OUT = MODE == 0;
    constexpr int MW = bwdc_mem_waves(ROT);
    using St = Stage<TI, NP, OUT, OUT, true, MW>;
    constexpr int NT = NP / 16, LDX = St::LDX, LDB = St::LDB, ROWS = kTileRows;
    __shared__ __attribute__((aligned(16))) TI sX[2][OUT ? ROWS * LDX : 8];
    __shared__ __attribute__((aligned(16))) TI sDy[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sB[2][OUT ? ROWS * LDB : 8];
    __shared__ __attribute__((aligned(16))) TI sC[2][ROWS * LDB];
    __shared__ __attribute__((aligned(16))) float sA[2][3 * kTileRows];
    __shared__ __attribute__((aligned(16))) uint16_t sM[OUT ? 6 : 1][16 * kLdm];
    __shared__ __attribute__((aligned(16))) uint16_t sH[OUT ? NP * kLdh : 8];
    __shared__ float sDd[kRowGroup / 16];
    const StageMem<TI> sm{&sX[0][0], &sDy[0][0], &sB[0][0], &sC[0][0], nullptr, &sA[0][0]};

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, R = a.R, P = a.P, TR = T * R;
    const int nw = (int)(P >> 4), S = a.S, Qt = a.Qt, log2R = a.log2R;
    const bool memw = wv >= nw;
    const int mt = tid - 64 * nw;
    const int seg = blockIdx.x % S;
    const int64_t bh = blockIdx.x / S;
    const int64_t b = bh / H, h = bh % H, g = h / (H / G);
    const int k0 = (int)(((int64_t)seg * a.nsub) / S), k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    // the state pass: the first segment's local gradient is never used (the
    // carry starts from dfinal), so its workgroups leave at once, together
    if (!OUT && seg == 0) return;
    uint16_t* dst = OUT ? static_cast<uint16_t*>(a.part) + (b * TR * H + h) * N : nullptr;   // bf16
    const int64_t rs = H * N;
    // lane byte offsets (+ uniform steps): the partial tiles at row l16,
    // column 4 q (stride H N, bf16); dy and dx at rows l16 and 16 + l16,
    // columns p0 + 4 q .. p0 + 4 q + 3 (stride H P, fp32). The dx stores take
    // the whole offset in the lane register and a zero scalar offset: for a
    // 16-byte store in that form the compiler keeps the next instruction from
    // overwriting the store's data registers, which it does not do for a
    // register scalar offset
    const uint32_t prow = (uint32_t)((l16 * rs + 4 * q) * 2), rowb = (uint32_t)(rs * 2);
    const uint32_t xrow0 = (uint32_t)((l16 * H * P + 16 * wv + 4 * q) * 4), xrowb = (uint32_t)(H * P * 4);
    const uint32_t xrow1 = xrow0 + 16u * xrowb;
    const float* dyh = a.dy + (b * TR * H + h) * P;
    float* dxh = OUT ? a.dx + (b * TR * H + h) * P : nullptr;

    // columns n >= N of B and C, p >= P of x and dy, and of the staged state
    // stay zero (the contractions over p always run over the 64 rows of a group)
    for (int i = tid; i < 2 * ROWS * LDB; i += blockDim.x) {
        if (OUT) sB[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
        sC[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
    }
    for (int i = tid; i < 2 * ROWS * LDX; i += blockDim.x) {
        if (OUT) sX[i / (ROWS * LDX)][i % (ROWS * LDX)] = TI(0);
        sDy[i / (ROWS * LDX)][i % (ROWS * LDX)] = TI(0);
    }
    if (OUT)
        for (int i = tid; i < NP * kLdh; i += blockDim.x) sH[i] = 0;
    __syncthreads();

    if (memw) {
        Stager<TI, NP, OUT, OUT, true, true, ROT, MW> st;
        if (k1 > k0) {
            st.load(a, k1 - 1, mt, b, h, g, 0);
            st.store(sm, a, 0, mt);
            if (k1 - 2 >= k0) st.load(a, k1 - 2, mt, b, h, g, 0);
        }
        __syncthreads();
        for (int k = k1 - 1; k >= k0; --k) {
            const int buf = (k1 - 1 - k) & 1;
            if (k > k0) {
                st.store(sm, a, buf ^ 1, mt);
                if (k - 2 >= k0) st.load(a, k - 2, mt, b, h, g, 0);
            }
            if constexpr (OUT) __syncthreads();                // blocks built, entering state put
            __syncthreads();                                   // tile walked
        }
        __syncthreads();                                       // the dy . x shares
        return;
    }

    const int p0 = 16 * wv;
    f32x4 hp[NT];                                  // D[p][n]: rows p0 + 4q + v, column 16c + l16
    {
        const float* src = nullptr;
        int64_t off = 0;
        if (OUT) {
            if (seg == S - 1) {
                src = a.dfinal;
                off = bh * P * N;
            } else {
                src = a.seg_in;
                off = (bh * S + seg) * P * N;
            }
        }
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) hp[c][v] = (src && n < N) ? src[off + (int64_t)(p0 + 4 * q + v) * N + n] : 0.f;
        }
        // the physical gradient at the segment's last step, into the folded frame
        if (ROT && OUT && src) {
            const int64_t tl = (((int64_t)k1 * Qt < T) ? (int64_t)k1 * Qt : T) - 1;
            turn_pn<NT>(hp, a.phi + ((b * T + tl) * H + h) * (N / 2), (int)N, -1.f, lane);
        }
    }
    const float Dh = (OUT && a.D) ? a.D[h] : 0.f;
    float dd = 0.f;
    __syncthreads();
    for (int k = k1 - 1; k >= k0; --k) {
        const int buf = (k1 - 1 - k) & 1;
        const uint16_t* tDy = reinterpret_cast<const uint16_t*>(sDy[buf]);
        const uint16_t* tC = reinterpret_cast<const uint16_t*>(sC[buf]);
        const float* cum = sA[buf];
        if constexpr (OUT) {
            const uint16_t* tX = reinterpret_cast<const uint16_t*>(sX[buf]);
            const uint16_t* tB = reinterpret_cast<const uint16_t*>(sB[buf]);
            // the tile's fp32 dy (for D dy and the dy . x sum), loaded now, used
            // last; rows past TR read zero
            const int64_t f0 = (int64_t)k * kTileRows;
            const auto xrs = tile_rows(dyh, f0, TR, H * P), drs = tile_rows(dxh, f0, TR, H * P);
            float4 dyr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                dyr[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xrs, i ? xrow1 : xrow0, 0, 0));
            put_state<NT>(sH, hp, p0, lane);
            // upper blocks (0,0), (0,1), (1,1): CB' = B_m . C_j (jobs 0-2) and
            // G' = x_m . dy_j (jobs 3-5), masked by step(j) >= step(m)
            for (int u = wv; u < 6; u += nw) {
                const int ub = u % 3, mb = ub == 2 ? 1 : 0, jb = ub == 0 ? 0 : 1;
                const f32x4 acc = u < 3 ? rows_dot32<NP>(tB, LDB, 16 * mb, tC, LDB, 16 * jb, lane)
                                        : rows_dot32<kRowGroup>(tX, LDX, 16 * mb, tDy, LDX, 16 * jb, lane);
                put_masked(sM[u], acc, mb, jb, true, cum, log2R, lane);
            }
            __syncthreads();
            // the tiles below are computed transposed: the lane's step row is 16 i + l16
            float wl[2];                           // e^{last - cum_m}
#pragma unroll
            for (int i = 0; i < 2; ++i) wl[i] = cum[kCumW + 16 * i + l16];
            // dx = w o (B H^T) + (CB' o L') dy over this wave's p
            f32x4 zx[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                zx[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c2 = 0; c2 < NT / 2; ++c2) {
                    const s16x8 bs = row8(tB + (16 * i + l16) * LDB + 32 * c2 + 8 * q);
                    zx[i] = mma32(tr_rows8(sH, kLdh, 32 * c2 + 8 * q, p0, lane), bs, zx[i]);
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) zx[i][v] *= wl[i];
            }
            {
                // block rows [CB' (0,0) | (0,1)] and [0 | (1,1)] against dy's 32 rows
                const s16x8 d8 = tr_rows8(tDy, LDX, 8 * q, p0, lane);
                zx[0] = mma32(d8, blk_pair(sM[0], sM[1], lane), zx[0]);
                zx[1] = mma32(d8, blk_pair(nullptr, sM[2], lane), zx[1]);
            }
            // dx rows (rows past TR dropped; their dy and x are zero), stored before
            // the dB partial rows so that using dy waits on no partial store
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float dv[4] = {dyr[i].x, dyr[i].y, dyr[i].z, dyr[i].w};
                const s16x4 xv = row4(reinterpret_cast<const uint16_t*>(sX[buf]) + (16 * i + l16) * LDX + p0 + 4 * q);
                f32x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    o[v] = fmaf(Dh, dv[v], zx[i][v]);
                    dd = fmaf(dv[v], __uint_as_float((uint32_t)(uint16_t)xv[v] << 16), dd);
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, o), drs, i ? xrow1 : xrow0, 0, 0);
            }
            // dB partial = w o (x H) + (G' o L') C on the wave's column tiles
            {
                s16x8 xs[2][kRowGroup / 32];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int kb = 0; kb < kRowGroup / 32; ++kb)
                        xs[i][kb] = row8(tX + (16 * i + l16) * LDX + 32 * kb + 8 * q);
                // block rows [G' (0,0) | (0,1)] and [0 | (1,1)]
                const s16x8 g0 = blk_pair(sM[3], sM[4], lane), g1 = blk_pair(nullptr, sM[5], lane);
                const auto prs = tile_rows16(dst, f0, TR, rs);
                // the wave's dB column tiles c = wv, wv + nw, ...
                auto db_tile = [&](int c) {
                    f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < kRowGroup / 32; ++kb) {
                        const s16x8 hb = row8(sH + (16 * c + l16) * kLdh + 32 * kb + 8 * q);
                        z0 = mma32(hb, xs[0][kb], z0);
                        z1 = mma32(hb, xs[1][kb], z1);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        z0[v] *= wl[0];
                        z1[v] *= wl[1];
                    }
                    const s16x8 cc = tr_rows8(tC, LDB, 8 * q, 16 * c, lane);
                    z0 = mma32(cc, g0, z0);
                    z1 = mma32(cc, g1, z1);
                    store_tile_cols16(prs, z0, z1, prow, rowb, 32u * c);
                };
                if (NT % (kRowGroup / 16) == 0 && nw == kRowGroup / 16 && N == NP) {
                    // four compute waves and every column tile in range: unrolled, so
                    // that one tile's LDS reads overlap the other's products
#pragma unroll
                    for (int j = 0; j < NT / (kRowGroup / 16); ++j) db_tile(wv + (kRowGroup / 16) * j);
                } else {
                    // N is a multiple of 16: a column tile is all in range or all out
                    for (int c = wv; c < NT && 16 * c < N; c += nw) db_tile(c);
                }
            }
        }
        // H <- e^{last} H + (e^{cum} o dy)^T C, contracted over the tile's 32 rows
        const float carry = cum[kCumE + kTileRows - 1];
        const s16x8 ed = scale8(tr_rows8(tDy, LDX, 8 * q, p0, lane),
                                *reinterpret_cast<const float4*>(cum + kCumE + 8 * q),
                                *reinterpret_cast<const float4*>(cum + kCumE + 8 * q + 4));
#pragma unroll
        for (int c = 0; c < NT; ++c) {
#pragma unroll
            for (int v = 0; v < 4; ++v) hp[c][v] *= carry;
            hp[c] = mma32(ed, tr_rows8(tC, LDB, 8 * q, 16 * c, lane), hp[c]);
        }
        __syncthreads();                           // tile walked: its buffers and sH free
    }
    float* out = nullptr;
    if (!OUT && seg > 0) out = a.seg_out + (bh * S + seg) * P * N;
    if (OUT && seg == 0 && a.dinit) out = a.dinit + bh * P * N;
    // back to the physical frame at step k0 Qt - 1 (none before step 0)
    if (ROT && out && seg > 0)
        turn_pn<NT>(hp, a.phi + ((b * T + (int64_t)k0 * Qt - 1) * H + h) * (N / 2), (int)N, 1.f, lane);
    if (out) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = 16 * c + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (n < N) out[(int64_t)(p0 + 4 * q + v) * N + n] = hp[c][v];
        }
    }
    if constexpr (OUT) {
        for (int o = 32; o >= 1; o >>= 1) dd += __shfl_xor(dd, o);
        if (lane == 0) sDd[wv] = dd;
    }
    __syncthreads();
    if (OUT && tid == 0) {
        float acc = 0.f;
        for (int w = 0; w < nw; ++w) acc += sDd[w];
        a.dDp[bh * S + seg] = acc;
    }
}

// Per (batch, head, segment): Lambda = sum of da and Phi[k] = sum of theta over
// the segment's steps (thread k < N/2: Phi[k]; thread N/2: Lambda).
__global__ __launch_bounds__(128) void ssd_bwd_segsums(const float* __restrict__ da, const float* __restrict__ theta,
                                                      const float* __restrict__ phi, float* __restrict__ sums,
                                                      int64_t T, int64_t H, int64_t N, int S, int nsub, int Qt) {
    const int64_t bh = blockIdx.x / S;
    const int seg = blockIdx.x % S;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t0 = ((int64_t)seg * nsub / S) * Qt, t1raw = ((int64_t)(seg + 1) * nsub / S) * Qt;
    const int64_t t1 = t1raw < T ? t1raw : T;
    const int k = threadIdx.x;
    float acc = 0.f;
    if (k < N / 2) {
        if (phi) {
            // from the cumulative angles: Phi[t1 - 1] - Phi[t0 - 1] (mod 2 pi)
            acc = phi[((b * T + t1 - 1) * H + h) * (N / 2) + k] -
                  (t0 > 0 ? phi[((b * T + t0 - 1) * H + h) * (N / 2) + k] : 0.f);
        } else if (theta) {
#pragma unroll 8
            for (int64_t t = t0; t < t1; ++t) acc += theta[((b * T + t) * H + h) * (N / 2) + k];
        }
        sums[(bh * S + seg) * (N / 2 + 1) + k] = acc;
    }
    // Lambda: the whole workgroup, strided, then reduced in a fixed order
    __shared__ float sl[2];
    float lam = 0.f;
    for (int64_t t = t0 + k; t < t1; t += blockDim.x) lam += da[(b * T + t) * H + h];
    for (int o = 32; o >= 1; o >>= 1) lam += __shfl_xor(lam, o);
    if ((k & 63) == 0) sl[k >> 6] = lam;
    __syncthreads();
    if (k == 0) sums[(bh * S + seg) * (N / 2 + 1) + N / 2] = sl[0] + sl[1];
}

// Reverse carry, one thread per (p, state pair): c_{S-1} = dfinal (or 0);
// c_s = e^{Lambda_{s+1}} R(Phi_{s+1})^T c_{s+1} + local_{s+1}, the gradient
// entering segment s from the right, into slot s of seg_in.
__global__ __launch_bounds__(256) void ssd_bwd_carry(const float* __restrict__ dfinal, const float* __restrict__ local,
                                                    const float* __restrict__ sums, float* __restrict__ seg_in,
                                                    int64_t P, int64_t N, int S) {
    const int64_t bh = blockIdx.y;
    const int64_t pair = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (pair >= P * (N / 2)) return;
    const int64_t p = pair / (N / 2), kk = pair % (N / 2), off = p * N + 2 * kk;
    float c0 = dfinal ? dfinal[bh * P * N + off] : 0.f, c1 = dfinal ? dfinal[bh * P * N + off + 1] : 0.f;
    for (int s = S - 1; s >= 0; --s) {
        if (s < S - 1) {
            const float* sm = sums + (bh * S + s + 1) * (N / 2 + 1);
            const float dec = __expf(sm[N / 2]);
            float sn, cs;
            sincosf(sm[kk], &sn, &cs);
            const float* lo = local + (bh * S + s + 1) * P * N + off;
            const float r0 = cs * c0 + sn * c1, r1 = -sn * c0 + cs * c1;
            c0 = dec * r0 + lo[0];
            c1 = dec * r1 + lo[1];
        }
        float* d = seg_in + (bh * S + s) * P * N + off;
        d[0] = c0;
        d[1] = c1;
    }
}

// The sum over the 64 lanes, in every lane: DPP row shifts leave each 16-lane
// row's total in its lane 15, the row broadcasts add rows 0 and 2 into rows 1
// and 3 and then lane 31 into rows 2 and 3, so that lane 63 holds the total.
__device__ __forceinline__ float wave_sum64(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Two consecutive entries (a state pair) of a row: bf16 or fp32 storage.
// bf16 rows (the chunked walks' partials, read once) load with the
// non-temporal hint.
__device__ __forceinline__ float2 ld_pair(const uint16_t* p, uint32_t pair) {
    const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + pair);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ float2 ld_pair(const float* p, uint32_t pair) {
    return reinterpret_cast<const float2*>(p)[pair];
}

// dB and dC of every group (the heads' and row groups' partials added in
// order) and, per head and step, the inner products and pair cross products
// of the decay and turn gradients. One workgroup of 4 waves per (batch,
// step); lane k takes the state pair (2k, 2k + 1). The ranks go in blocks of
// RM: wave w takes the heads w, w + 4, ... of a group, HU of them at a time,
// and keeps its sums of dB and dC for each rank of the block in registers.
// The four waves' sums meet in LDS and are added in wave order. A head's
// decay and turn terms add up over the ranks of a block in registers and over
// blocks in its own output slot. With phi the partials are of the folded
// frame and are turned back by R(Phi_t) first. Loads take clamped, in-bounds
// indexes and are masked after, so that all of a pass's loads are in flight
// together. PT is the partials' storage type (bf16 from the chunked walks).
template <typename TI, typename PT, int RM, int HU>
__global__ __launch_bounds__(256) void ssd_bwd_reduce(const PT* __restrict__ pC, const PT* __restrict__ pB,
                                                     const void* __restrict__ Bv, const void* __restrict__ Cv,
                                                     float* __restrict__ dB, float* __restrict__ dC,
                                                     float* __restrict__ hv, float* __restrict__ th,
                                                     int64_t T, int64_t H, int64_t G, int64_t N, int64_t R, int npg,
                                                     int rot, const float* __restrict__ phi) {
    __shared__ __attribute__((aligned(16))) float sred[2][4][RM][128];
    const int64_t bt = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t HG = H / G;
    // this step's rows: R ranks x H heads x npg row groups x N partials, and
    // R ranks x G groups x N entries of B, C, dB and dC; offsets in them fit 32 bits
    const int64_t row0 = bt * R;
    const PT* pBt = pB + row0 * H * npg * N;
    const PT* pCt = pC + row0 * H * npg * N;
    const TI* Bt = static_cast<const TI*>(Bv) + row0 * G * N;
    const TI* Ct = static_cast<const TI*>(Cv) + row0 * G * N;
    float* dBt = dB + row0 * G * N;
    float* dCt = dC + row0 * G * N;
    const float* phit = phi ? phi + bt * H * (N / 2) : nullptr;
    float* tht = th + bt * H * (N / 2);
    // without phi the angle loads read the first word of the partials, unused: no branch
    const float* phs = phit ? phit : reinterpret_cast<const float*>(pBt);
    const uint32_t phm = phit ? 0xffffffffu : 0u;
    const uint32_t Hu = (uint32_t)H, Gu = (uint32_t)G, NP2 = (uint32_t)(N / 2), npu = (uint32_t)npg;
    const bool kok = (uint32_t)lane < NP2;
    const uint32_t kc = kok ? (uint32_t)lane : 0;
    const float2 zero2 = make_float2(0.f, 0.f);
    for (uint32_t g = 0; g < Gu; ++g) {
        for (int64_t r0 = 0; r0 < R; r0 += RM) {
            float2 sb[RM], sc[RM], bn[RM], cn[RM];
            bool ok[RM];
            uint32_t rc[RM];
#pragma unroll
            for (int k = 0; k < RM; ++k) {
                const bool rin = r0 + k < R;
                rc[k] = rin ? (uint32_t)(r0 + k) : 0;
                ok[k] = rin && kok;
                sb[k] = zero2;
                sc[k] = zero2;
                const uint32_t i = (rc[k] * Gu + g) * NP2 + kc;
                const float2 bv = ld_pair(Bt, i), cv = ld_pair(Ct, i);
                bn[k] = ok[k] ? bv : zero2;
                cn[k] = ok[k] ? cv : zero2;
            }
            const uint32_t hend = (g + 1) * (uint32_t)HG;
            for (uint32_t h0 = g * (uint32_t)HG + w; h0 < hend; h0 += 4 * HU) {
                // heads h0 + 4 j of this pass; past the group's end they are
                // clamped to h0 and their terms are dropped
                uint32_t hj[HU];
                bool hok[HU];
#pragma unroll
                for (int j = 0; j < HU; ++j) {
                    hok[j] = h0 + 4 * j < hend;
                    hj[j] = hok[j] ? h0 + 4 * j : h0;
                }
                float2 db[HU][RM], dc[HU][RM];
                float ph[HU];
#pragma unroll
                for (int j = 0; j < HU; ++j) {
                    ph[j] = phs[(hj[j] * NP2 + kc) & phm];
#pragma unroll
                    for (int k = 0; k < RM; ++k) {
                        const uint32_t i = (rc[k] * Hu + hj[j]) * npu * NP2 + kc;
                        db[j][k] = ld_pair(pBt, i);
                        dc[j][k] = ld_pair(pCt, i);
                    }
                }
                for (uint32_t pg = 1; pg < npu; ++pg)
#pragma unroll
                    for (int j = 0; j < HU; ++j)
#pragma unroll
                        for (int k = 0; k < RM; ++k) {
                            const uint32_t i = ((rc[k] * Hu + hj[j]) * npu + pg) * NP2 + kc;
                            const float2 b2 = ld_pair(pBt, i), c2 = ld_pair(pCt, i);
                            db[j][k].x += b2.x;
                            db[j][k].y += b2.y;
                            dc[j][k].x += c2.x;
                            dc[j][k].y += c2.y;
                        }
#pragma unroll
                for (int j = 0; j < HU; ++j) {
                    float cs = 1.f, sn = 0.f;
                    if (phit) {
                        const float rev = ph[j] * kInv2Pi;
                        cs = __builtin_amdgcn_cosf(rev);
                        sn = __builtin_amdgcn_sinf(rev);
                    }
                    float hvacc = 0.f, thacc = 0.f;
#pragma unroll
                    for (int k = 0; k < RM; ++k) {
                        float2 bd = db[j][k], cd = dc[j][k];
                        if (!(ok[k] && hok[j])) bd = cd = zero2;
                        if (phit) {
                            // partials of the folded frame: dB = R(Phi_t) dB~, dC = R(Phi_t) dC~
                            bd = make_float2(fmaf(cs, bd.x, -sn * bd.y), fmaf(cs, bd.y, sn * bd.x));
                            cd = make_float2(fmaf(cs, cd.x, -sn * cd.y), fmaf(cs, cd.y, sn * cd.x));
                        }
                        sb[k].x += bd.x;
                        sb[k].y += bd.y;
                        sc[k].x += cd.x;
                        sc[k].y += cd.y;
                        hvacc = fmaf(cn[k].x, cd.x, fmaf(cn[k].y, cd.y, fmaf(-bn[k].x, bd.x, fmaf(-bn[k].y, bd.y, hvacc))));
                        // (dC_2k C_2k+1 - dC_2k+1 C_2k) + (dB_2k B_2k+1 - dB_2k+1 B_2k)
                        if (rot) thacc += (cd.x * cn[k].y - cd.y * cn[k].x) + (bd.x * bn[k].y - bd.y * bn[k].x);
                    }
                    if (!hok[j]) continue;
                    hvacc = wave_sum64(hvacc);
                    const int64_t ht = bt * H + hj[j];
                    if (lane == 0) hv[ht] = r0 == 0 ? hvacc : hv[ht] + hvacc;
                    if (rot && kok) {
                        float* q = tht + hj[j] * NP2 + lane;
                        *q = r0 == 0 ? thacc : *q + thacc;
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < RM; ++k) {
                *reinterpret_cast<float2*>(&sred[0][w][k][2 * lane]) = sb[k];
                *reinterpret_cast<float2*>(&sred[1][w][k][2 * lane]) = sc[k];
            }
            __syncthreads();
            for (int i = tid; i < RM * 128; i += 256) {
                const int k = i >> 7, n = i & 127;
                if (n >= N || r0 + k >= R) continue;
                const float vb = sred[0][0][k][n] + sred[0][1][k][n] + sred[0][2][k][n] + sred[0][3][k][n];
                const float vc = sred[1][0][k][n] + sred[1][1][k][n] + sred[1][2][k][n] + sred[1][3][k][n];
                const uint32_t o = ((uint32_t)(r0 + k) * Gu + g) * (uint32_t)N + n;
                dBt[o] = vb;
                dCt[o] = vc;
            }
            __syncthreads();
        }
    }
}

// the blocks of the reduction (16 pair loads in flight per wave and pass):
// one rank and eight heads, two ranks and four heads, or four ranks and two
template <typename TI, typename PT>
void* bwd_reduce_for(int64_t R) {
    if (R <= 1) return reinterpret_cast<void*>(&ssd_bwd_reduce<TI, PT, 1, 4>);
    if (R == 2) return reinterpret_cast<void*>(&ssd_bwd_reduce<TI, PT, 2, 2>);
    return reinterpret_cast<void*>(&ssd_bwd_reduce<TI, PT, 4, 1>);
}

// dda and dtheta are reverse cumulative sums over the steps of the per-step
// terms (column k < N/2: the turn of pair k; column N/2: the decay), plus the
// final state's terms at the last step. Four kernels: the final state's terms
// and dD (per (batch, head)), the sums of chunks of kScanChunk steps, each
// chunk's carry (the final terms plus the sums of the chunks after it, one
// wave per (batch, head, column)), and the scan of each chunk from its carry.
constexpr int kScanChunk = 64;
constexpr int kCarryBlock = 16;   // chunks whose sums a carry thread loads at once

// Phi[b,t,h,k] = sum over s <= t of theta[b,s,h,k], kept in [-pi, pi] (the
// running sum is wrapped each step so that it keeps its absolute precision;
// 2 pi split into a head exact in few bits and a tail, as in Cody and
// Waite's argument reduction). Three kernels over chunks of kScanChunk steps:
// the chunks' sums, the angle entering each chunk (one thread per (batch,
// head, pair) walking the chunks), then each chunk's scan from it.
// Thread -> (batch-head, chunk, pair), pairs fastest.
__device__ __forceinline__ float wrap_2pi(float v) {
    const float m = rintf(v * kInv2Pi);
    return fmaf(-m, 1.9353071795864769e-3f, fmaf(-m, 6.28125f, v));
}

__global__ __launch_bounds__(256) void ssd_bwd_phi_sums(const float* __restrict__ theta, float* __restrict__ psum,
                                                       int64_t T, int64_t H, int64_t NH, int nchunk, int64_t items) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= items) return;
    const int64_t k = i % NH, ch = (i / NH) % nchunk, bh = i / (NH * nchunk), h = bh % H, b = bh / H;
    const int64_t t0 = ch * (int64_t)kScanChunk, t1 = t0 + kScanChunk < T ? t0 + kScanChunk : T;
    float acc = 0.f;
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) acc += theta[((b * T + t) * H + h) * NH + k];
    psum[i] = wrap_2pi(acc);
}

// the chunks' sums replaced in place by the angle entering each chunk
__global__ __launch_bounds__(256) void ssd_bwd_phi_carry(float* __restrict__ psum, int64_t NH, int nchunk,
                                                        int64_t items) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= items) return;
    const int64_t k = i % NH, bh = i / NH;
    float* col = psum + bh * nchunk * NH + k;
    float run = 0.f;
    // blocks of kCarryBlock chunks: every load of a block is issued before its
    // stores (same array), so that they are in flight together
    for (int c0 = 0; c0 < nchunk; c0 += kCarryBlock) {
        float v[kCarryBlock];
#pragma unroll
        for (int j = 0; j < kCarryBlock; ++j) v[j] = c0 + j < nchunk ? col[(int64_t)(c0 + j) * NH] : 0.f;
#pragma unroll
        for (int j = 0; j < kCarryBlock; ++j) {
            if (c0 + j < nchunk) col[(int64_t)(c0 + j) * NH] = run;
            run = wrap_2pi(run + v[j]);
        }
    }
}

__global__ __launch_bounds__(256) void ssd_bwd_phi(const float* __restrict__ theta, const float* __restrict__ pin,
                                                  float* __restrict__ phi, int64_t T, int64_t H, int64_t NH,
                                                  int nchunk, int64_t items) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= items) return;
    const int64_t k = i % NH, ch = (i / NH) % nchunk, bh = i / (NH * nchunk), h = bh % H, b = bh / H;
    float run = pin[i];
    const int64_t t0 = ch * (int64_t)kScanChunk, t1 = t0 + kScanChunk < T ? t0 + kScanChunk : T;
    // the loads do not depend on the running angle: unrolled, several are in flight
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t o = ((b * T + t) * H + h) * NH + k;
        run = wrap_2pi(run + theta[o]);
        phi[o] = run;
    }
}

__global__ __launch_bounds__(128) void ssd_bwd_final_terms(const float* __restrict__ dfinal,
                                                          const float* __restrict__ fin,
                                                          const float* __restrict__ dDp, float* __restrict__ ft,
                                                          float* __restrict__ dD, int64_t B_, int64_t H, int64_t P,
                                                          int64_t N, int nparts) {
    // lane k takes the state pair (2k, 2k + 1) of rows p = half, half + 2, ...:
    // dfinal . fin over the pair, and the pair's cross product
    const int64_t bh = blockIdx.x, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, k = tid & 63, half = tid >> 6, nc = (int)(N / 2 + 1);
    __shared__ float sdot[2], scr[2][64];
    float dot = 0.f, cr = 0.f;
    if (dfinal && k < N / 2) {
        const float2* df = reinterpret_cast<const float2*>(dfinal + bh * P * N) + k;
        const float2* fi = reinterpret_cast<const float2*>(fin + bh * P * N) + k;
#pragma unroll 4
        for (int64_t p = half; p < P; p += 2) {
            const float2 a = df[p * (N / 2)], c = fi[p * (N / 2)];
            dot = fmaf(a.x, c.x, fmaf(a.y, c.y, dot));
            cr += a.y * c.x - a.x * c.y;
        }
    }
    dot = wave_sum64(dot);
    if (k == 0) sdot[half] = dot;
    scr[half][k] = cr;
    __syncthreads();
    if (tid < N / 2) {
        ft[bh * nc + tid] = scr[0][tid] + scr[1][tid];
    } else if (tid == N / 2) {
        ft[bh * nc + tid] = sdot[0] + sdot[1];
    } else if (tid == N / 2 + 1 && dD && b == 0) {
        float acc = 0.f;
        for (int64_t bb = 0; bb < B_; ++bb)
            for (int i = 0; i < nparts; ++i) acc += dDp[(bb * H + h) * nparts + i];
        dD[h] = acc;
    }
}

// the value of column k at step t (k < N/2: th, k == N/2: hv)
__device__ __forceinline__ float step_term(const float* hv, const float* th, int64_t b, int64_t t, int64_t T,
                                           int64_t H, int64_t h, int64_t N, int k) {
    return k < N / 2 ? th[((b * T + t) * H + h) * (N / 2) + k] : hv[(b * T + t) * H + h];
}

// Thread item of the chunked reverse scans: the column k (a pair's angle term,
// or the decay term at k = N/2) fastest, then the head, the chunk and the batch,
// so that a wave's per-step loads and stores of one step are contiguous over
// heads (or columns)
__device__ __forceinline__ int scan_item(int64_t it, int ncols, int k0, int64_t H, int nchunk, int64_t* h,
                                         int* ch, int64_t* b) {
    const int k = k0 + (int)(it % ncols);
    const int64_t r = it / ncols;
    *h = r % H;
    *ch = (int)((r / H) % nchunk);
    *b = r / (H * nchunk);
    return k;
}

__global__ __launch_bounds__(128) void ssd_bwd_chunk_sums(const float* __restrict__ hv, const float* __restrict__ th,
                                                         float* __restrict__ csum, int64_t T, int64_t H, int64_t N,
                                                         int nchunk, int k0, int64_t items) {
    const int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (it >= items) return;
    const int nc = (int)(N / 2 + 1), ncols = nc - k0;
    int ch;
    int64_t b, h;
    const int k = scan_item(it, ncols, k0, H, nchunk, &h, &ch, &b);
    const int64_t bh = b * H + h;
    const int64_t t0 = (int64_t)ch * kScanChunk, t1 = t0 + kScanChunk < T ? t0 + kScanChunk : T;
    float acc = 0.f;
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) acc += step_term(hv, th, b, t, T, H, h, N, k);
    csum[(bh * nchunk + ch) * nc + k] = acc;
}

// the chunks' sums replaced in place by each chunk's carry: the final terms
// plus the sums of the chunks after it. One wave per (batch, head, column):
// lane l takes the chunks [l per, l per + per), per = ceil(nchunk / 64); the
// lanes' totals are summed from the last lane down by shuffles, then each lane
// walks its chunks from its last one, storing the carries.
__global__ __launch_bounds__(256) void ssd_bwd_chunk_carry(const float* __restrict__ ft, float* __restrict__ csum,
                                                          int nchunk, int nc, int k0, int64_t items) {
    const int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (it >= items) return;   // whole waves
    const int lane = threadIdx.x & 63;
    const int ncols = nc - k0;
    const int k = k0 + (int)(it % ncols);
    const int64_t bh = it / ncols;
    float* col = csum + bh * nchunk * nc + k;
    const int per = (nchunk + 63) >> 6;
    const int c0 = lane * per, c1 = c0 + per < nchunk ? c0 + per : nchunk;
    float tot = 0.f;
    for (int c = c0; c < c1; ++c) tot += col[(int64_t)c * nc];
    // inclusive sums over this lane and the lanes after it; the carry into a
    // lane's chunks is the next lane's
    float suf = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_down(suf, d, 64);
        suf += lane + d < 64 ? o : 0.f;
    }
    const float after = __shfl_down(suf, 1, 64);
    float acc = ft[bh * nc + k] + (lane < 63 ? after : 0.f);
    for (int c = c1 - 1; c >= c0; --c) {
        const float v = col[(int64_t)c * nc];
        col[(int64_t)c * nc] = acc;
        acc += v;
    }
}

__global__ __launch_bounds__(128) void ssd_bwd_chunk_scan(const float* __restrict__ hv, const float* __restrict__ th,
                                                         const float* __restrict__ carry, float* __restrict__ dda,
                                                         float* __restrict__ dtheta, int64_t T, int64_t H, int64_t N,
                                                         int nchunk, int k0, int64_t items) {
    const int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (it >= items) return;
    const int nc = (int)(N / 2 + 1), ncols = nc - k0;
    int ch;
    int64_t b, h;
    const int k = scan_item(it, ncols, k0, H, nchunk, &h, &ch, &b);
    const int64_t bh = b * H + h;
    float acc = carry[(bh * nchunk + ch) * nc + k];
    const int64_t t0 = (int64_t)ch * kScanChunk, t1 = t0 + kScanChunk < T ? t0 + kScanChunk : T;
    float* out = k < N / 2 ? dtheta : dda;
#pragma unroll 8
    for (int64_t t = t1 - 1; t >= t0; --t) {
        acc += step_term(hv, th, b, t, T, H, h, N, k);
        if (k < N / 2) out[((b * T + t) * H + h) * (N / 2) + k] = acc;
        else out[(b * T + t) * H + h] = acc;
    }
}

template <typename TI>
void* bwd_forward_np(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_bwd_forward_kernel<TI, 32>);
        case 64: return reinterpret_cast<void*>(&ssd_bwd_forward_kernel<TI, 64>);
        case 128: return reinterpret_cast<void*>(&ssd_bwd_forward_kernel<TI, 128>);
    }
    return nullptr;
}

template <bool ROT>
void* bwdc_forward_np(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_bwdc_forward_kernel<32, ROT>);
        case 64: return reinterpret_cast<void*>(&ssd_bwdc_forward_kernel<64, ROT>);
        case 128: return reinterpret_cast<void*>(&ssd_bwdc_forward_kernel<128, ROT>);
    }
    return nullptr;
}

template <int MODE, bool ROT>
void* bwdc_backward_np(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_bwdc_backward_kernel<32, MODE, ROT>);
        case 64: return reinterpret_cast<void*>(&ssd_bwdc_backward_kernel<64, MODE, ROT>);
        case 128: return reinterpret_cast<void*>(&ssd_bwdc_backward_kernel<128, MODE, ROT>);
    }
    return nullptr;
}

template <typename TI, int MODE>
void* bwd_backward_np(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_bwd_backward_kernel<TI, 32, MODE>);
        case 64: return reinterpret_cast<void*>(&ssd_bwd_backward_kernel<TI, 64, MODE>);
        case 128: return reinterpret_cast<void*>(&ssd_bwd_backward_kernel<TI, 128, MODE>);
    }
    return nullptr;
}

// A second stream per device for the forward-direction chain (the forward's
// state passes and the forward-direction walk), which reads nothing the
// backward chain writes: the two chains run side by side and each fills the
// other's last round of workgroups. Created on first use with default
// priority; a call holds the lock from the fork to the join, so calls on one
// device take their turns on it.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

ssd_status side_stream(SideStream** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
    SideStream& ss = g_side[dev];
    if (!ss.fork && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) {
        ss.fork = nullptr;
        return SSD_ERR_HIP;
    }
    if (!ss.join && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
        ss.join = nullptr;
        return SSD_ERR_HIP;
    }
    if (!ss.s && hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) {
        ss.s = nullptr;
        return SSD_ERR_HIP;
    }
    *out = &ss;
    return SSD_OK;
}

}  // namespace

extern "C" ssd_status ssd_backward(const ssd_dims* d, const void* x, const float* da, const void* B,
                                   const void* C, const float* D, const float* init_state, int64_t R,
                                   const float* theta, const float* dy, const float* dfinal, float* dx,
                                   float* dda, float* dB, float* dC, float* dtheta, float* dinit, float* dD,
                                   void* stream) {
    if (!d || !x || !da || !B || !C || !dy || !dx || !dda || !dB || !dC) return SSD_ERR_NULL_ARG;
    if ((theta == nullptr) != (dtheta == nullptr) || (D == nullptr) != (dD == nullptr)) return SSD_ERR_NULL_ARG;
    ssd_status st = forward_shape_status(d, 1, R, theta != nullptr);
    if (st != SSD_OK) return st;
    if (d->dstate > 128) return SSD_ERR_UNSUPPORTED;
    const int64_t b = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
    const int64_t esz = d->in_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dy, 16) || !aligned(dx, 16) ||
        (init_state && !aligned(init_state, 16)) || (dfinal && !aligned(dfinal, 16)) ||
        (dinit && !aligned(dinit, 16)) || (theta && !aligned(theta, 16)) || !aligned(da, 4) ||
        !aligned(dda, 4) || !aligned(dB, 4) || !aligned(dC, 4) || (dtheta && !aligned(dtheta, 4)) ||
        (D && !aligned(D, 4)) || (dD && !aligned(dD, 4)))
        return SSD_ERR_UNSUPPORTED;
    const Span outs[] = {span_of(dx, b * T * R * H * P * 4), span_of(dda, b * T * H * 4),
                         span_of(dB, b * T * R * G * N * 4), span_of(dC, b * T * R * G * N * 4),
                         dtheta ? span_of(dtheta, b * T * H * (N / 2) * 4) : Span{0, 0},
                         dinit ? span_of(dinit, b * H * P * N * 4) : Span{0, 0},
                         dD ? span_of(dD, H * 4) : Span{0, 0}};
    const Span ins[] = {span_of(x, b * T * R * H * P * esz), span_of(da, b * T * H * 4),
                        span_of(B, b * T * R * G * N * esz), span_of(C, b * T * R * G * N * esz),
                        D ? span_of(D, H * 4) : Span{0, 0},
                        init_state ? span_of(init_state, b * H * P * N * 4) : Span{0, 0},
                        theta ? span_of(theta, b * T * H * (N / 2) * 4) : Span{0, 0},
                        span_of(dy, b * T * R * H * P * 4),
                        dfinal ? span_of(dfinal, b * H * P * N * 4) : Span{0, 0}};
    for (int i = 0; i < 7; ++i) {
        if (outs[i].hi == 0) continue;
        for (int j = i + 1; j < 7; ++j)
            if (outs[j].hi && overlap(outs[i], outs[j])) return SSD_ERR_ALIAS;
        for (const Span& si : ins)
            if (si.hi && overlap(outs[i], si)) return SSD_ERR_ALIAS;
    }

    // the forward's plan gives the segments (and, with more than one, the
    // states entering them from its state passes)
    const bool rot = theta != nullptr;
    Plan pl;
    size_t st_bytes = 0;
    st = states_plan(d, R, rot, &pl, &st_bytes);
    if (st != SSD_OK) return st;
    const int NP = (int)pl.NP;
    const bool bf = d->in_dtype == SSD_BF16;
    // bf16 without rotation and a whole head per workgroup: the chunked walks;
    // otherwise the step-by-step walks
    const bool chunked = bf && P <= kRowGroup;
    void* kf = chunked ? (rot ? bwdc_forward_np<true>(NP) : bwdc_forward_np<false>(NP))
                       : bf ? bwd_forward_np<uint16_t>(NP) : bwd_forward_np<float>(NP);
    void* kb0 = chunked ? (rot ? bwdc_backward_np<0, true>(NP) : bwdc_backward_np<0, false>(NP))
                        : bf ? bwd_backward_np<uint16_t, 0>(NP) : bwd_backward_np<float, 0>(NP);
    void* kb1 = chunked ? (rot ? bwdc_backward_np<1, true>(NP) : bwdc_backward_np<1, false>(NP))
                        : bf ? bwd_backward_np<uint16_t, 1>(NP) : bwd_backward_np<float, 1>(NP);
    // partials: bf16 from the chunked walks, fp32 from the step walks
    void* kr = chunked ? bwd_reduce_for<uint16_t, uint16_t>(R)
                       : bf ? bwd_reduce_for<uint16_t, float>(R) : bwd_reduce_for<float, float>(R);
    if (!kf || !kb0 || !kb1) return SSD_ERR_UNSUPPORTED;
    const int PG = (int)(P < kRowGroup ? P : kRowGroup), npg = (int)(P / PG);
    if (chunked && npg != 1) return SSD_ERR_UNSUPPORTED;
    const int S = pl.S;
    const int64_t nwg = b * H * npg * S;
    if (nwg > 0x7fffffff || b * T > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (R * H * npg * N > 0x7fffffff) return SSD_ERR_UNSUPPORTED;   // one step's partials, 32-bit offsets
    // a tile's rows of x, dy, B, C and its steps' angles: 32-bit byte offsets
    if ((int64_t)kTileRows * H * (P > N ? P : N) * 4 > 0xffffffffLL) return SSD_ERR_UNSUPPORTED;
    if ((b * H * ((T + kScanChunk - 1) / kScanChunk) * (N / 2 + 1) + 127) / 128 > 0x7fffffff)
        return SSD_ERR_UNSUPPORTED;

    // workspace: forward state passes | partial dC | partial dB | final state |
    // per-step terms (hv, th) | dD partials | backward segment states, locals, sums
    const size_t n_part = (size_t)(b * H * npg) * (size_t)(T * R * N);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    const size_t o_states = take(st_bytes);
    const size_t psz = chunked ? 2 : 4;                // bytes per partial entry
    const size_t o_pC = take(n_part * psz), o_pB = take(n_part * psz);
    const size_t o_fin = take((size_t)(b * H * P * N) * 4);
    const size_t o_hv = take((size_t)(b * T * H) * 4);
    const size_t o_th = take(rot ? (size_t)(b * T * H * (N / 2)) * 4 : 4);
    const size_t o_dd = take((size_t)(b * H * npg * S) * 4);
    const size_t o_segin = take(S > 1 ? (size_t)(b * H * S * P * N) * 4 : 4);
    const size_t o_local = take(S > 1 ? (size_t)(b * H * S * P * N) * 4 : 4);
    const size_t o_sums = take(S > 1 ? (size_t)(b * H * S * (N / 2 + 1)) * 4 : 4);
    const int64_t nchunks = (T + kScanChunk - 1) / kScanChunk;
    const size_t o_ft = take((size_t)(b * H * (N / 2 + 1)) * 4);
    const bool cphi = chunked && rot;                  // the folded frame's angles
    const size_t o_phi = take(cphi ? (size_t)(b * T * H * (N / 2)) * 4 : 4);
    const size_t o_csum = take((size_t)(b * H * nchunks * (N / 2 + 1)) * 4);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    int entry = -1;
    char* ws = static_cast<char*>(scratch_acquire(hs, off, &entry, kSlotBackward));
    if (!ws) return SSD_ERR_HIP;
    float* fin = reinterpret_cast<float*>(ws + o_fin);

    BwdArgs ba;
    memset(&ba, 0, sizeof(ba));
    ba.x = x; ba.da = da; ba.B = B; ba.C = C; ba.theta = theta; ba.dy = dy; ba.D = D;
    ba.init = init_state; ba.dfinal = dfinal; ba.dx = dx; ba.dinit = dinit;
    ba.T = T; ba.H = H; ba.G = G; ba.N = N; ba.R = R; ba.P = P;
    ba.PG = PG; ba.S = S; ba.SF = pl.SF; ba.nsub = pl.nsub; ba.Qt = pl.Qt; ba.log2R = pl.log2R;
    float* phi = cphi ? reinterpret_cast<float*>(ws + o_phi) : nullptr;
    ba.phi = phi;
    // the chunked walks with rotation run four memory waves, the others two
    const dim3 grid((unsigned)nwg), block((unsigned)(64 * (PG / 16 + (chunked ? bwdc_mem_waves(rot) : kMemWaves))));
    const dim3 fblock((unsigned)(64 * (PG / 16 + (chunked ? bwdc_fwd_mem_waves(rot) : kMemWaves))));

    // 0. the cumulative angles (chunked walks with rotation)
    ssd_status rs = SSD_OK;
    if (cphi) {
        // chunk sums of theta in the dda scan's chunk-sum buffer (free until then)
        const int nch = (int)((T + kScanChunk - 1) / kScanChunk);
        const int64_t n = b * H * nch * (N / 2);
        float* psum = reinterpret_cast<float*>(ws + o_csum);
        const int64_t nk = b * H * (N / 2);
        hipLaunchKernelGGL(ssd_bwd_phi_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, hs, theta, psum, T, H,
                           N / 2, nch, n);
        hipLaunchKernelGGL(ssd_bwd_phi_carry, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, hs, psum, N / 2, nch,
                           nk);
        hipLaunchKernelGGL(ssd_bwd_phi, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, hs, theta, psum, phi, T, H,
                           N / 2, nch, n);
        if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
    }
    // fork: the forward-direction chain on the side stream, after everything
    // the caller's stream holds so far (inputs, the angles)
    std::unique_lock<std::mutex> side_lock(g_side_mu);
    SideStream* side = nullptr;
    hipStream_t fs = hs;
    if (rs == SSD_OK) rs = side_stream(&side);
    if (rs == SSD_OK) {
        if (hipEventRecord(side->fork, hs) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
            rs = SSD_ERR_HIP;
        else
            fs = side->s;
    }
    // 1. forward walk: states from the forward's state passes, dC partials, final state
    float* fws_state = nullptr;
    if (rs == SSD_OK) rs = states_launch(pl, rot, x, da, B, init_state, theta, ws + o_states, fs, &fws_state);
    if (rs == SSD_OK) {
        BwdArgs fa = ba;
        fa.seg_in = fws_state;
        fa.part = ws + o_pC;
        fa.final_state = fin;
        void* kargs[] = {&fa};
        if (hipLaunchKernel(kf, grid, fblock, kargs, 0, fs) != hipSuccess) rs = SSD_ERR_HIP;
    }
    // 2. backward state pass and reverse carry (more than one segment)
    float* seg_in = reinterpret_cast<float*>(ws + o_segin);
    if (rs == SSD_OK && S > 1) {
        hipLaunchKernelGGL(ssd_bwd_segsums, dim3((unsigned)(b * H * S)), dim3(128), 0, hs, da, theta, phi,
                           reinterpret_cast<float*>(ws + o_sums), T, H, N, S, pl.nsub, pl.Qt);
        if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
        if (rs == SSD_OK) {
            BwdArgs la = ba;
            la.seg_out = reinterpret_cast<float*>(ws + o_local);
            void* kargs[] = {&la};
            if (hipLaunchKernel(kb1, grid, block, kargs, 0, hs) != hipSuccess) rs = SSD_ERR_HIP;
        }
        if (rs == SSD_OK) {
            dim3 cg((unsigned)((P * (N / 2) + 255) / 256), (unsigned)(b * H));
            hipLaunchKernelGGL(ssd_bwd_carry, cg, dim3(256), 0, hs, dfinal,
                               reinterpret_cast<const float*>(ws + o_local),
                               reinterpret_cast<const float*>(ws + o_sums), seg_in, P, N, S);
            if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
        }
    }
    // 3. backward walk: dx, dB partials, dD partials, dinit
    if (rs == SSD_OK) {
        BwdArgs oa = ba;
        oa.seg_in = S > 1 ? seg_in : nullptr;
        oa.part = ws + o_pB;
        oa.dDp = reinterpret_cast<float*>(ws + o_dd);
        void* kargs[] = {&oa};
        if (hipLaunchKernel(kb0, grid, block, kargs, 0, hs) != hipSuccess) rs = SSD_ERR_HIP;
    }
    // join: the caller's stream waits for the forward-direction chain (the
    // reduction reads its dC partials, the final terms its final state)
    if (fs != hs && (hipEventRecord(side->join, fs) != hipSuccess || hipStreamWaitEvent(hs, side->join, 0) != hipSuccess))
        rs = SSD_ERR_HIP;
    side_lock.unlock();
    // 4. group sums and per-step terms; 5. reverse cumulative sums
    if (rs == SSD_OK) {
        const void* pC = ws + o_pC;
        const void* pB = ws + o_pB;
        float* hv = reinterpret_cast<float*>(ws + o_hv);
        float* th = reinterpret_cast<float*>(ws + o_th);
        int64_t Tv = T, Hv = H, Gv = G, Nv = N, Rv = R;
        int npgv = npg, rotv = rot ? 1 : 0;
        const float* phiv = phi;
        void* kargs[] = {(void*)&pC, (void*)&pB, (void*)&B, (void*)&C, (void*)&dB, (void*)&dC, (void*)&hv,
                         (void*)&th, (void*)&Tv, (void*)&Hv, (void*)&Gv, (void*)&Nv, (void*)&Rv, (void*)&npgv,
                         (void*)&rotv, (void*)&phiv};
        if (hipLaunchKernel(kr, dim3((unsigned)(b * T)), dim3(256), kargs, 0, hs) != hipSuccess) rs = SSD_ERR_HIP;
        // final-state terms and dD; chunk sums; chunk carries; chunk scans
        // (columns from k0: all pairs with rotation, only the decay column without)
        const int nc = (int)(N / 2 + 1), nchunk = (int)((T + kScanChunk - 1) / kScanChunk);
        const int k0 = rot ? 0 : (int)(N / 2);
        float* ft = reinterpret_cast<float*>(ws + o_ft);
        float* csum = reinterpret_cast<float*>(ws + o_csum);
        if (rs == SSD_OK) {
            hipLaunchKernelGGL(ssd_bwd_final_terms, dim3((unsigned)(b * H)), dim3(128), 0, hs, dfinal, fin,
                               reinterpret_cast<const float*>(ws + o_dd), ft, dD, b, H, P, N, npg * S);
            const int64_t items = b * H * nchunk * (int64_t)(nc - k0);
            const dim3 sgrid((unsigned)((items + 127) / 128));
            const int64_t citems = b * H * (int64_t)(nc - k0);
            hipLaunchKernelGGL(ssd_bwd_chunk_sums, sgrid, dim3(128), 0, hs, hv, th, csum, T, H, N, nchunk, k0, items);
            hipLaunchKernelGGL(ssd_bwd_chunk_carry, dim3((unsigned)((citems + 3) / 4)), dim3(256), 0, hs, ft, csum,
                               nchunk, nc, k0, citems);
            hipLaunchKernelGGL(ssd_bwd_chunk_scan, sgrid, dim3(128), 0, hs, hv, th, csum, dda, dtheta, T, H, N,
                               nchunk, k0, items);
            if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
        }
    }
    if (!scratch_release(entry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    return rs;
}
