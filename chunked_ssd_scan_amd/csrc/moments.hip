// Physical-frame state moments for AMD Instinct MI355X (gfx950).
//
// burn-mamba "mamba3/moments.rs", module documentation (steps 1-4: the
// per-token states of a chunk, their de-rotation to the physical frame, the
// plain real m2/m1 sums masked to valid_len) and state_moments_phys: for every
// (batch, head), with h_t the physical state (P x N) after step t,
//   m2[n][n'] = sum_{t < valid_len} sum_p h_t[p][n] h_t[p][n']
//   m1[n]     = sum_{t < valid_len} sum_p h_t[p][n]
// Every per-token state is needed (the page explains why no closed form
// exists once the state turns), so the kernel materialises them one step at
// a time, in registers, and never stores them.
//
// The recurrence is stepped in the physical frame, h_t = e^{da_t} R(theta_t)
// h_{t-1} + sum_r x_{t,r} (outer) B_{t,r}: the turn of each state pair is two
// multiply-adds against the neighbouring lane (a DPP swap), so no cumulative
// angle and no de-rotation are needed. The Mamba-3 trapezoid runs as the
// sub-step sequence of trap_scan.hip (sub-step 2t: decay and the beta write;
// 2t + 1: turn and the gamma write); only odd sub-steps are counted.
//
// Layout: state rows p evolve independently, so a workgroup walks one
// (batch, head, group of at most 64 rows p, segment). Its compute wave w holds
// rows p in [p0 + 16w, p0 + 16w + 16) for every n, as 16 x 16 accumulator tiles
// D[p][n] (lane l: column n = 16c + l % 16, rows p = 4 (l / 16) .. + 3); two
// memory waves stage each tile's x, B, theta and da into LDS. In that layout
// the accumulators of one step are, as they stand, both operands of the Gram
// MFMA D[n][n'] += sum_p h[p][n] h[p][n'] (k = p), so each wave adds its 16
// rows' share of every upper-triangle block of m2 with one MFMA per block and
// step, and the workgroup sums its waves' shares at the end. Segments start
// from the state the forward's state pass and carry give them; a last kernel
// adds the row groups' and segments' sums and mirrors the upper blocks.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ssd_common.h"
#include "ssd_step.h"

namespace {

using namespace ssd_detail;
using namespace ssd_step;

constexpr int kTileRows = 32;        // fused rows staged per tile (32 / R steps)
constexpr int kPadRows = 4;          // zero rows after a tile: reads past its last step
constexpr int kRowGroup = 64;        // most state rows p per workgroup
constexpr int kMemWaves = 4;         // waves that stage the tiles (four: 3.55 -> 3.47 ms against two)

struct MomArgs {
    const void* x;
    const float* da;
    const void* B;
    const float* theta;      // [b,T,H,N/2] or null
    const float* init;       // [b,H,P,N] or null
    const float* ws_state;   // [b*H][S*SF][P][N] entering states, or null (one segment)
    float* part;             // [b*H][row groups][S][blocks * 256 + NP] sums
    int64_t T, H, G, N, R, P;
    int PG;                  // state rows per workgroup (a row group)
    int S, SF, nsub, Qt;
    int64_t limit;           // step t counts when t < limit and (t & smask) == smask
    int smask;
};

// upper-triangle block index of (a, b), a <= b < nt
__host__ __device__ constexpr int ublk(int a, int b, int nt) { return a * nt - a * (a - 1) / 2 + (b - a); }

template <typename TI, int NP>
__global__ __launch_bounds__(64 * (kRowGroup / 16 + kMemWaves)) void ssd_moments_kernel(MomArgs a) {
    constexpr int ESZ = (int)sizeof(TI);
    constexpr bool BF = ESZ == 2;
    constexpr int NT = NP / 16;                    // 16-column state tiles
    constexpr int NB2 = NT * (NT + 1) / 2;         // upper-triangle blocks of m2
    constexpr int LDX = kRowGroup + 16 / ESZ;      // staged x row stride (elements)
    constexpr int LDB = NP + 16 / ESZ;             // staged B row stride
    constexpr int ROWS = kTileRows + kPadRows;
    constexpr int NH = NP / 2;                     // state pairs
    constexpr int EPU = 16 / ESZ;                  // elements per 16-byte unit
    constexpr int NTM = 64 * kMemWaves;            // memory threads
    // staging units per memory thread: x rows of the group, B rows, theta
    constexpr int XR = (kTileRows * kRowGroup / EPU + NTM - 1) / NTM;
    constexpr int BRG = (kTileRows * NP / EPU + NTM - 1) / NTM;
    constexpr int THR = (kTileRows * NH / 4 + NTM - 1) / NTM;

    __shared__ __attribute__((aligned(16))) TI sX[2][ROWS * LDX];
    __shared__ __attribute__((aligned(16))) TI sB[2][ROWS * LDB];
    // per step and state pair: e^{da} cos and e^{da} sin of the step's decay
    // and angle (the memory waves evaluate them while staging)
    __shared__ __attribute__((aligned(16))) float2 sCS[2][kTileRows * NH];
    __shared__ __attribute__((aligned(16))) float sRed[NB2 * 256 + NP];

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, R = a.R, P = a.P;
    const int64_t TR = T * R;
    const int PG = a.PG;
    const int nw = PG >> 4;                        // compute waves
    const bool memw = wv >= nw;
    const int mt = tid - 64 * nw;                  // memory thread index
    const int S = a.S;
    const int npg = (int)(P / PG);
    int item = blockIdx.x;
    const int seg = item % S;
    item /= S;
    const int pg = item % npg;
    const int64_t bh = item / npg;
    const int64_t b = bh / H, h = bh % H, g = h / (H / G);
    const int k0 = (int)(((int64_t)seg * a.nsub) / S);
    const int k1 = (int)(((int64_t)(seg + 1) * a.nsub) / S);
    const int Qt = a.Qt;
    const int Ri = (int)R;
    const int pbase = pg * PG;                     // first state row of the group

    // zero the pad rows of both buffers (read past a tile's last step), and
    // the B columns past N (state tiles beyond dstate)
    for (int i = tid; i < 2 * kPadRows * LDX; i += nthr)
        sX[i / (kPadRows * LDX)][kTileRows * LDX + i % (kPadRows * LDX)] = TI(0);
    for (int i = tid; i < 2 * ROWS * LDB; i += nthr) sB[i / (ROWS * LDB)][i % (ROWS * LDB)] = TI(0);
    // the angles of pairs past N/2 are never staged: they stay zero, so that
    // every lane reads its pair's angle without a guard
    for (int i = tid; i < 2 * kTileRows * NH; i += nthr) (&sCS[0][0])[i] = make_float2(0.f, 0.f);
    __syncthreads();

    // ---- staging (memory waves): tile k's x rows [32][PG], B rows [32][N],
    // theta [Qt][N/2] and da [Qt] (as e^{da} times the cos and sin of each
    // angle); rows past the sequence are zero (identity steps)
    const TI* xg = static_cast<const TI*>(a.x);
    const TI* Bg = static_cast<const TI*>(a.B);
    const int xur = PG / EPU, nbu = (int)((N + EPU - 1) / EPU), thu = (int)((N / 2 + 3) / 4);
    uint4 rx[XR], rb[BRG], rth[THR];
    float rda[THR];
    auto load_tile = [&](int k) {
        const int64_t f0 = (int64_t)k * kTileRows;
#pragma unroll
        for (int m = 0; m < XR; ++m) {
            const int u = mt + m * NTM, r = u / xur, c = (u % xur) * EPU;
            rx[m] = (u < kTileRows * xur && f0 + r < TR)
                        ? *reinterpret_cast<const uint4*>(xg + ((b * TR + f0 + r) * H + h) * P + pbase + c)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < BRG; ++m) {
            const int u = mt + m * NTM, r = u / nbu, c = (u % nbu) * EPU;
            rb[m] = (u < kTileRows * nbu && f0 + r < TR)
                        ? *reinterpret_cast<const uint4*>(Bg + ((b * TR + f0 + r) * G + g) * N + c)
                        : make_uint4(0, 0, 0, 0);
        }
        const int64_t t0 = (int64_t)k * Qt;
#pragma unroll
        for (int m = 0; m < THR; ++m) {
            const int u = mt + m * NTM, st = u / thu, c = (u % thu) * 4;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (a.theta && st < Qt && t0 + st < T) {
                const float* src = a.theta + ((b * T + t0 + st) * H + h) * (N / 2) + c;
                if (c + 4 <= N / 2) v = *reinterpret_cast<const uint4*>(src);
            }
            rth[m] = v;
            rda[m] = (st < Qt && t0 + st < T) ? a.da[(b * T + t0 + st) * H + h] : 0.f;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int m = 0; m < XR; ++m) {
            const int u = mt + m * NTM, r = u / xur, c = (u % xur) * EPU;
            if (u < kTileRows * xur) *reinterpret_cast<uint4*>(&sX[buf][r * LDX + c]) = rx[m];
        }
#pragma unroll
        for (int m = 0; m < BRG; ++m) {
            const int u = mt + m * NTM, r = u / nbu, c = (u % nbu) * EPU;
            if (u < kTileRows * nbu) *reinterpret_cast<uint4*>(&sB[buf][r * LDB + c]) = rb[m];
        }
#pragma unroll
        for (int m = 0; m < THR; ++m) {
            const int u = mt + m * NTM, st = u / thu, c = (u % thu) * 4;
            if (st < Qt) {
                // the hardware sine and cosine take revolutions
                const float th[4] = {__uint_as_float(rth[m].x), __uint_as_float(rth[m].y), __uint_as_float(rth[m].z),
                                     __uint_as_float(rth[m].w)};
                const float al = __expf(rda[m]);
                float4* d = reinterpret_cast<float4*>(&sCS[buf][st * NH + c]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float r0 = th[2 * j] * kInv2Pi, r1 = th[2 * j + 1] * kInv2Pi;
                    d[j] = make_float4(al * __builtin_amdgcn_cosf(r0), al * __builtin_amdgcn_sinf(r0),
                                       al * __builtin_amdgcn_cosf(r1), al * __builtin_amdgcn_sinf(r1));
                }
            }
        }
    };

    // Memory waves and compute waves run separate loops with the same
    // barriers (one after each tile's compute, one after each staging), so
    // that neither keeps the other's registers live.
    if (memw) {
        load_tile(k0);
        store_tile(0);
        __syncthreads();
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            if (k + 1 < k1) load_tile(k + 1);
            __syncthreads();                       // tile k computed
            if (k + 1 < k1) {
                store_tile(buf ^ 1);
                __syncthreads();
            }
        }
        for (int i = tid; i < NB2 * 256 + NP; i += nthr) sRed[i] = 0.f;
        __syncthreads();
        for (int w = 0; w < nw; ++w) __syncthreads();
    } else {
        // ---- state entering the segment: D[p][n] tiles of this wave's 16 rows
        const int p0 = pbase + 16 * wv;
        f32x4 hs[NT];
        {
            const float* src = nullptr;
            if (S == 1)
                src = a.init ? a.init + bh * P * N : nullptr;
            else
                src = a.ws_state + (bh * S + seg) * (int64_t)a.SF * P * N;
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int n = 16 * c + l16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int p = p0 + 4 * q + v;
                    hs[c][v] = (src && n < N) ? src[(int64_t)p * N + n] : 0.f;
                }
            }
        }
        f32x4 m2p[NB2];
#pragma unroll
        for (int i = 0; i < NB2; ++i) m2p[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
        float m1p[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) m1p[c] = 0.f;

        // rows of one step hold the R ranks; the K slots 4q + e of the write
        // MFMA beyond R are zero. Lane groups with no rank read the step's
        // first rows.
        const int kr0 = (4 * q < Ri) ? 4 * q : 0;
        // the K slots of the write: x slot 4q + e and B row e count when they
        // hold one of the step's R ranks (bit masks, applied without a branch)
        s16x4 xmask, bmask;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xmask[e] = (4 * q + e < Ri) ? (short)-1 : (short)0;
            bmask[e] = (e < Ri) ? (short)-1 : (short)0;
        }
        const int xcol = 16 * wv;                  // this wave's columns in the staged x tile

        __syncthreads();                           // tile k0 staged
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            for (int s = 0; s < Qt; ++s) {
                const int64_t t = (int64_t)k * Qt + s;
                if (t >= T) break;
                // decay and turn of every state pair, against the partner lane
                float cs_self[NT], cs_part[NT];
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const int n = 16 * c + l16;
                    const float2 csn = sCS[buf][s * NH + (n >> 1)];
                    cs_self[c] = csn.x;
                    cs_part[c] = (n & 1) ? csn.y : -csn.y;
                }
#pragma unroll
                for (int c = 0; c < NT; ++c) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float pv = swap_pair(hs[c][v]);
                        hs[c][v] = fmaf(cs_self[c], hs[c][v], cs_part[c] * pv);
                    }
                }
                // this step's rank-R write
                const int row = s * Ri;
                if constexpr (BF) {
                    const s16x4 xa = tr_rows4(reinterpret_cast<const uint16_t*>(sX[buf]), LDX, row + kr0, xcol, lane) &
                                     xmask;
#pragma unroll
                    for (int c = 0; c < NT; ++c) {
                        const s16x4 bb =
                            tr_rows4(reinterpret_cast<const uint16_t*>(sB[buf]), LDB, row + kr0, 16 * c, lane) & bmask;
                        hs[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xa, bb, hs[c], 0, 0, 0);
                    }
                } else {
                    for (int j = 0; 4 * j < Ri; ++j) {
                        const int r = 4 * j + q;
                        const int rr = r < Ri ? r : 0;
                        const float xv = r < Ri ? (float)sX[buf][(row + rr) * LDX + xcol + l16] : 0.f;
#pragma unroll
                        for (int c = 0; c < NT; ++c) {
                            const float bv = (float)sB[buf][(row + rr) * LDB + 16 * c + l16];
                            hs[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, bv, hs[c], 0, 0, 0);
                        }
                    }
                }
                // the sums, over the steps that count
                if (t < a.limit && (t & a.smask) == a.smask) {
#pragma unroll
                    for (int c = 0; c < NT; ++c) m1p[c] += (hs[c][0] + hs[c][1]) + (hs[c][2] + hs[c][3]);
                    if constexpr (BF) {
                        s16x4 hb[NT];
#pragma unroll
                        for (int c = 0; c < NT; ++c) hb[c] = pack4_bf16(hs[c]);
#pragma unroll
                        for (int ta = 0; ta < NT; ++ta)
#pragma unroll
                            for (int tb = ta; tb < NT; ++tb)
                                m2p[ublk(ta, tb, NT)] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                    hb[ta], hb[tb], m2p[ublk(ta, tb, NT)], 0, 0, 0);
                    } else {
#pragma unroll
                        for (int ta = 0; ta < NT; ++ta)
#pragma unroll
                            for (int tb = ta; tb < NT; ++tb)
#pragma unroll
                                for (int v = 0; v < 4; ++v)
                                    m2p[ublk(ta, tb, NT)] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                        hs[ta][v], hs[tb][v], m2p[ublk(ta, tb, NT)], 0, 0, 0);
                    }
                }
            }
            __syncthreads();                       // tile k computed
            if (k + 1 < k1) __syncthreads();       // tile k + 1 staged
        }

        // ---- the workgroup's sums: the compute waves' shares added in wave order
        for (int i = tid; i < NB2 * 256 + NP; i += nthr) sRed[i] = 0.f;
        __syncthreads();
        for (int w = 0; w < nw; ++w) {
            if (wv == w) {
#pragma unroll
                for (int i = 0; i < NB2; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) sRed[i * 256 + (4 * q + v) * 16 + l16] += m2p[i][v];
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    float s1 = m1p[c] + __shfl_xor(m1p[c], 16);
                    s1 += __shfl_xor(s1, 32);
                    if (q == 0) sRed[NB2 * 256 + 16 * c + l16] += s1;
                }
            }
            __syncthreads();
        }
    }
    float* dst = a.part + ((bh * npg + pg) * S + seg) * (int64_t)(NB2 * 256 + NP);
    for (int i = tid; i < NB2 * 256 + NP; i += nthr) dst[i] = sRed[i];
}

// m2 [b*H][N][N] and m1 [b*H][N]: the sums of the row groups and segments
// (ng = groups x segments, consecutive per (batch, head)) added in order, the
// lower blocks mirrored from the upper ones.
template <int NP>
__global__ __launch_bounds__(256) void ssd_moments_final(const float* __restrict__ part, float* __restrict__ m2,
                                                        float* __restrict__ m1, int64_t N, int ng) {
    constexpr int NT = NP / 16, NB2 = NT * (NT + 1) / 2, STRIDE = NB2 * 256 + NP;
    const int64_t bh = blockIdx.x;
    const float* src = part + bh * ng * (int64_t)STRIDE;
    for (int64_t i = threadIdx.x; i < N * N; i += blockDim.x) {
        const int n = (int)(i / N), n2 = (int)(i % N);
        int ta = n >> 4, tb = n2 >> 4, ra = n & 15, rb = n2 & 15;
        if (ta > tb) {
            const int t0 = ta; ta = tb; tb = t0;
            const int r0 = ra; ra = rb; rb = r0;
        }
        const int off = ublk(ta, tb, NT) * 256 + ra * 16 + rb;
        float acc = 0.f;
        for (int s = 0; s < ng; ++s) acc += src[(int64_t)s * STRIDE + off];
        m2[bh * N * N + i] = acc;
    }
    for (int64_t n = threadIdx.x; n < N; n += blockDim.x) {
        float acc = 0.f;
        for (int s = 0; s < ng; ++s) acc += src[(int64_t)s * STRIDE + NB2 * 256 + n];
        m1[bh * N + n] = acc;
    }
}

template <typename TI>
void* moments_kernel_np(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_moments_kernel<TI, 32>);
        case 64: return reinterpret_cast<void*>(&ssd_moments_kernel<TI, 64>);
        case 128: return reinterpret_cast<void*>(&ssd_moments_kernel<TI, 128>);
    }
    return nullptr;
}

void* moments_final_np(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_moments_final<32>);
        case 64: return reinterpret_cast<void*>(&ssd_moments_final<64>);
        case 128: return reinterpret_cast<void*>(&ssd_moments_final<128>);
    }
    return nullptr;
}

}  // namespace

extern "C" ssd_status ssd_state_moments(const ssd_dims* d, const void* x, const float* da, const void* B,
                                        const float* beta, const float* gamma, const void* prev_x,
                                        const void* prev_B, const float* init_state, int64_t R,
                                        const float* theta, int64_t valid_len, float* m2, float* m1,
                                        void* stream) {
    if (!d || !x || !da || !B || !m2 || !m1) return SSD_ERR_NULL_ARG;
    if ((beta == nullptr) != (gamma == nullptr) || (prev_x == nullptr) != (prev_B == nullptr))
        return SSD_ERR_NULL_ARG;
    const bool trap = beta != nullptr;
    if (prev_x && !trap) return SSD_ERR_BAD_SHAPE;
    ssd_status st = forward_shape_status(d, 1, R, theta != nullptr);
    if (st != SSD_OK) return st;
    if (valid_len < 1 || valid_len > d->seqlen) return SSD_ERR_BAD_SHAPE;
    if (d->dstate > 128) return SSD_ERR_UNSUPPORTED;
    const int64_t b = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate,
                  G = d->ngroups;
    ssd_dims d2 = *d;
    if (trap) {
        if (d->seqlen > ((int64_t)1 << 39) || d->batch * d->seqlen > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
        d2.seqlen = 2 * d->seqlen;
        st = forward_shape_status(&d2, 1, R, theta != nullptr);
        if (st != SSD_OK) return st;
    }
    const int64_t esz = d->in_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(x, 16) || !aligned(B, 16) || (init_state && !aligned(init_state, 16)) ||
        !aligned(m2, 16) || !aligned(m1, 4) || !aligned(da, 4) || (theta && !aligned(theta, 16)) ||
        (beta && (!aligned(beta, 4) || !aligned(gamma, 4))) ||
        (prev_x && (!aligned(prev_x, 16) || !aligned(prev_B, 16))))
        return SSD_ERR_UNSUPPORTED;
    const Span s2 = span_of(m2, b * H * N * N * 4), s1 = span_of(m1, b * H * N * 4);
    const Span ins[] = {span_of(x, b * T * R * H * P * esz), span_of(da, b * T * H * 4),
                        span_of(B, b * T * R * G * N * esz),
                        beta ? span_of(beta, b * T * H * 4) : Span{0, 0},
                        gamma ? span_of(gamma, b * T * H * 4) : Span{0, 0},
                        prev_x ? span_of(prev_x, b * R * H * P * esz) : Span{0, 0},
                        prev_B ? span_of(prev_B, b * R * G * N * esz) : Span{0, 0},
                        init_state ? span_of(init_state, b * H * P * N * 4) : Span{0, 0},
                        theta ? span_of(theta, b * T * H * (N / 2) * 4) : Span{0, 0}};
    if (overlap(s2, s1)) return SSD_ERR_ALIAS;
    for (const Span& si : ins) {
        if (si.hi == 0) continue;
        if (overlap(s2, si) || overlap(s1, si)) return SSD_ERR_ALIAS;
    }

    const bool rot = theta != nullptr;
    const ssd_dims& dd = trap ? d2 : *d;
    Plan pl;
    size_t st_bytes = 0;
    st = states_plan(&dd, R, rot, &pl, &st_bytes);
    if (st != SSD_OK) return st;
    const int NP = (int)pl.NP;
    void* kfn = d->in_dtype == SSD_BF16 ? moments_kernel_np<uint16_t>(NP) : moments_kernel_np<float>(NP);
    void* ffn = moments_final_np(NP);
    if (!kfn || !ffn) return SSD_ERR_UNSUPPORTED;
    // a workgroup per (batch, head, group of at most 64 state rows, segment)
    const int PG = (int)(P < kRowGroup ? P : kRowGroup);
    const int npg = (int)(P / PG);
    const int64_t nthr = 64 * (PG / 16 + kMemWaves);
    const int64_t nwg = b * H * npg * pl.S;
    if (nwg > 0x7fffffff) return SSD_ERR_UNSUPPORTED;

    const int nt = NP / 16;
    const size_t part_bytes = align256((size_t)nwg * (size_t)(nt * (nt + 1) / 2 * 256 + NP) * 4);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    TrapExpand ex;
    memset(&ex, 0, sizeof(ex));
    int xentry = -1;
    const void* sx = x;
    const float* sda = da;
    const void* sB = B;
    const float* sth = theta;
    if (trap) {
        ex.x = x; ex.da = da; ex.B = B; ex.C = nullptr; ex.beta = beta; ex.gamma = gamma;
        ex.prev_x = prev_x; ex.prev_B = prev_B; ex.theta = theta;
        ex.b = b; ex.T = T; ex.R = R; ex.H = H; ex.P = P; ex.G = G; ex.N = N; ex.esz = (int)esz;
        void* xw = scratch_acquire(hs, trap_expand_bytes(ex), &xentry, kSlotExpand);
        if (!xw) return SSD_ERR_HIP;
        trap_expand_setup(&ex, xw);
        sx = ex.xh; sda = ex.dah; sB = ex.Bh; sth = ex.thh;
    }
    int mentry = -1;
    char* mw = static_cast<char*>(scratch_acquire(hs, align256(st_bytes) + part_bytes, &mentry, kSlotMoments));
    ssd_status rs = mw ? SSD_OK : SSD_ERR_HIP;
    if (rs == SSD_OK && trap) rs = trap_expand_launch(ex, hs);
    float* ws_state = nullptr;
    if (rs == SSD_OK) rs = states_launch(pl, rot, sx, sda, sB, init_state, sth, mw, hs, &ws_state);
    float* part = mw ? reinterpret_cast<float*>(mw + align256(st_bytes)) : nullptr;
    if (rs == SSD_OK) {
        MomArgs ma;
        memset(&ma, 0, sizeof(ma));
        ma.x = sx; ma.da = sda; ma.B = sB; ma.theta = sth; ma.init = init_state; ma.ws_state = ws_state;
        ma.part = part;
        ma.T = dd.seqlen; ma.H = H; ma.G = G; ma.N = N; ma.R = R; ma.P = P; ma.PG = PG;
        ma.S = pl.S; ma.SF = pl.SF; ma.nsub = pl.nsub; ma.Qt = pl.Qt;
        ma.limit = trap ? 2 * valid_len : valid_len;
        ma.smask = trap ? 1 : 0;
        void* kargs[] = {&ma};
        if (hipLaunchKernel(kfn, dim3((unsigned)nwg), dim3((unsigned)nthr), kargs, 0, hs) != hipSuccess)
            rs = SSD_ERR_HIP;
    }
    if (rs == SSD_OK) {
        const float* pp = part;
        int64_t Nv = N;
        int ng = npg * pl.S;
        void* fargs[] = {(void*)&pp, (void*)&m2, (void*)&m1, (void*)&Nv, (void*)&ng};
        if (hipLaunchKernel(ffn, dim3((unsigned)(b * H)), dim3(256), fargs, 0, hs) != hipSuccess) rs = SSD_ERR_HIP;
    }
    if (mw && !scratch_release(mentry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    if (xentry >= 0 && !scratch_release(xentry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    return rs;
}
