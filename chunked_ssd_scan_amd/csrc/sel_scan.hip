// Diagonal selective scan (Mamba-1 form) for AMD Instinct MI355X (gfx950).
//
// LeetGPU "SSM Selective Scan" write-up, problem statement: per batch b,
// channel d and state n, from a zero state,
//   h[n] <- exp(delta[b,t,d] A[d,n]) h[n] + delta[b,t,d] B[b,t,n] u[b,t,d]
//   y[b,t,d] = sum_n C[b,t,n] h[n] + skip[d] u[b,t,d]
// The decay differs per (d, n), so unlike the SSD scan there is no matrix
// shared across channels and no contraction for MFMA: the work is one
// exponential and a handful of fp32 VALU operations per (t, d, n), and the
// kernels are bound by VALU issue.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ssd_common.h"

namespace {

using namespace ssd_detail;

// ---------------------------------------------------------------------------
// One lane per (batch, channel) holds the N states in registers. u, delta
// and y rows are contiguous over the 64 channels of a wave; the B and C rows
// of a block of steps are the same for every lane and are staged through LDS
// and read as broadcasts. The sequence is cut into K chunks that run in
// parallel: pass 1 walks each chunk from zero and keeps its end state and its
// sum of delta, pass 2 carries the states across chunks (the decay over a
// chunk is exp(A[d,n] sum delta)), pass 3 walks each chunk again from its
// carried state and writes y.
// ---------------------------------------------------------------------------
struct SelArgs {
    const float* u;
    const float* delta;
    const float* A;
    const float* B;
    const float* C;
    const float* skip;
    float* y;
    float* ws_h;     // [b][K][N][D]: chunk end states (pass 1), then carried states (pass 2)
    float* ws_s;     // [b][K][D]: sum of delta over the chunk
    int64_t T, Dm, N;
    int64_t Lc;      // steps per chunk (the last may be shorter)
    int K;           // chunks, ceil(T / Lc)
    int Kw;          // chunks this launch walks (the state pass skips the last)
    int DG;          // 64-channel groups
};

// Steps per block: a block's B and C rows (TB * NN floats each) take two
// loads per lane; u and delta of the next block are in flight in registers
// while the current one is computed.
template <int NN>
constexpr int sel_block_steps() { return 128 / NN; }

template <int NN, int MODE>   // MODE 1: chunk states; MODE 0: outputs
__global__ __launch_bounds__(64) void sel_scan_kernel(SelArgs a) {
    constexpr int TB = sel_block_steps<NN>();
    constexpr int PER = TB * NN / 64;                    // B (and C) values each lane stages
    __shared__ float4 sBC4[2][2][TB * NN / 4];           // [buffer][B, C][step * NN + n]
    const int lane = threadIdx.x;
    int item = blockIdx.x;
    const int dg = item % a.DG;
    item /= a.DG;
    const int k = item % a.Kw;
    const int b = item / a.Kw;
    const int64_t T = a.T, Dm = a.Dm, N = a.N;
    const int64_t d = (int64_t)dg * 64 + lane;
    const bool dok = d < Dm;
    const int64_t dd = dok ? d : Dm - 1;                 // clamped for loads
    const int64_t t0 = (int64_t)k * a.Lc, t1 = t0 + a.Lc < T ? t0 + a.Lc : T;
    const int nblk = (int)((t1 - t0 + TB - 1) / TB);
    // A rows of this wave's channels and, past the first chunk, the entering
    // states: one load each, states past N and channels past Dm read as zero
    const int64_t hrow = ((int64_t)b * a.K + k) * N;      // ws_h row of (b, k, n = 0)
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.A + (int64_t)dg * 64 * N, (uint32_t)((Dm - (int64_t)dg * 64) * N * 4));
    const __amdgpu_buffer_rsrc_t rH = make_rsrc(a.ws_h + hrow * Dm + (int64_t)dg * 64, (uint32_t)(N * Dm * 4 - (int64_t)dg * 256));
    float A2[NN], h[NN];
#pragma unroll
    for (int n = 0; n < NN; ++n) {
        const uint32_t ao = n < N ? (uint32_t)((lane * N + n) * 4) : kOOB;
        A2[n] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rA, ao, 0, 0)) * kLog2e;
        h[n] = 0.f;
    }
    if (MODE == 0 && k > 0) {
#pragma unroll
        for (int n = 0; n < NN; ++n) {
            const uint32_t ho = n < N ? (uint32_t)(n * Dm * 4) + (uint32_t)lane * 4 : kOOB;
            h[n] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rH, ho, 0, 0));
        }
    }
    const float sk = (MODE == 0) ? a.skip[dd] : 0.f;
    // per-lane byte offsets: u/delta rows are Dm floats apart; B/C staging
    // element e = lane + 64 j sits at (step e / NN, state e % NN)
    const uint32_t DmB = (uint32_t)(Dm * 4);
    const uint32_t uoff = dok ? (uint32_t)lane * 4 : kOOB;
    uint32_t bcoff[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j, st = e / NN, n = e % NN;
        bcoff[j] = n < N ? (uint32_t)((st * N + n) * 4) : kOOB;
    }
    float pu[TB], pd[TB], pb[PER], pc[PER];
    // loads of one block; rows past the chunk read as zero (outside the range)
    auto fetch = [&](int blk) {
        const int64_t tb = t0 + (int64_t)blk * TB;
        const int64_t rows = t1 - tb < TB ? t1 - tb : TB;
        const int64_t ue = ((int64_t)b * T + tb) * Dm + (int64_t)dg * 64;
        const uint32_t ubytes = (uint32_t)(rows * Dm * 4 - (int64_t)dg * 256);
        const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.u + ue, ubytes);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.delta + ue, ubytes);
#pragma unroll
        for (int st = 0; st < TB; ++st) {
            const uint32_t o = uoff + (uint32_t)st * DmB;
            pu[st] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ru, o, 0, 0));
            pd[st] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o, 0, 0));
        }
        const int64_t be = ((int64_t)b * T + tb) * N;
        const uint32_t bbytes = (uint32_t)(rows * N * 4);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B + be, bbytes);
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C + be, bbytes);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            pb[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, bcoff[j], 0, 0));
            if (MODE == 0) pc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, bcoff[j], 0, 0));
            else pc[j] = 0.f;
        }
    };
    fetch(0);
    float dsum = 0.f;
    for (int blk = 0; blk < nblk; ++blk) {
        float cu[TB], cd[TB];
#pragma unroll
        for (int s = 0; s < TB; ++s) {
            cu[s] = pu[s];
            cd[s] = pd[s];
        }
        float* sB = reinterpret_cast<float*>(sBC4[blk & 1][0]);
        float* sC = reinterpret_cast<float*>(sBC4[blk & 1][1]);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            sB[lane + 64 * j] = pb[j];
            if (MODE == 0) sC[lane + 64 * j] = pc[j];
        }
        __syncthreads();
        if (blk + 1 < nblk) fetch(blk + 1);
        // rows past the chunk were loaded as zeros: delta = 0 turns the step
        // into h = 1 * h + 0, so only the store of y needs the row bound
        const int64_t tb = t0 + (int64_t)blk * TB;
        const int rows = (int)(t1 - tb < TB ? t1 - tb : TB);
        // up to 32 states the B (and C) row of step s + 1 is read from LDS
        // while step s is computed; at 64 the extra registers cost more
        // occupancy than the overlap gains
        constexpr bool kAhead = NN <= 32;
        const float4* B4 = sBC4[blk & 1][0];
        const float4* C4 = sBC4[blk & 1][1];
        float4 nb[NN / 4], nc[NN / 4];
        if constexpr (kAhead) {
#pragma unroll
            for (int q = 0; q < NN / 4; ++q) {
                nb[q] = B4[q];
                nc[q] = MODE == 0 ? C4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int s = 0; s < TB; ++s) {
            const float dl = cd[s], uu = cu[s], su = dl * uu;
            float4 cb[NN / 4], cc[NN / 4];
            if constexpr (kAhead) {
#pragma unroll
                for (int q = 0; q < NN / 4; ++q) {
                    cb[q] = nb[q];
                    cc[q] = nc[q];
                }
                if (s + 1 < TB) {
#pragma unroll
                    for (int q = 0; q < NN / 4; ++q) {
                        nb[q] = B4[(s + 1) * (NN / 4) + q];
                        if (MODE == 0) nc[q] = C4[(s + 1) * (NN / 4) + q];
                    }
                }
            }
            float acc0 = sk * uu, acc1 = 0.f;
#pragma unroll
            for (int q = 0; q < NN / 4; ++q) {
                // without the read-ahead each 16-byte read sits next to its use
                const float4 bq = kAhead ? cb[q] : B4[s * (NN / 4) + q];
                const float4 cq = kAhead ? cc[q] : (MODE == 0 ? C4[s * (NN / 4) + q] : make_float4(0.f, 0.f, 0.f, 0.f));
                const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
                const float cv[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 4 * q + i;
                    h[n] = fmaf(__builtin_amdgcn_exp2f(dl * A2[n]), h[n], su * bv[i]);
                    if (MODE == 0) {
                        if (i & 1) acc1 = fmaf(cv[i], h[n], acc1);
                        else acc0 = fmaf(cv[i], h[n], acc0);
                    }
                }
            }
            dsum += dl;
            if (MODE == 0 && dok && s < rows) a.y[((int64_t)b * T + tb + s) * Dm + d] = acc0 + acc1;
        }
    }
    if (MODE == 1) {
#pragma unroll
        for (int n = 0; n < NN; ++n) {
            const uint32_t ho = (n < N && dok) ? (uint32_t)(n * Dm * 4) + (uint32_t)lane * 4 : kOOB;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, h[n]), rH, ho, 0, 0);
        }
        if (dok) a.ws_s[((int64_t)b * a.K + k) * Dm + d] = dsum;
    }
}

// Pass 2: across chunks the state follows c_{k+1} = exp(A[d,n] s_k) c_k + l_k
// (l_k: chunk k's end state from zero, s_k: its sum of delta), an affine scan.
// A workgroup takes 64 channels of one (batch, state) and cuts the chunks into
// blockDim.y runs: each run folds its chunks from zero (phase 1), one thread
// per channel joins the runs in order (phase 2), and each run walks its chunks
// again from its true entering state, storing it per chunk (phase 3). The
// decay across a run is exp(A[d,n] times the run's sum of s_k), so the join
// needs one exponential per run. Slot k of ws_h holds l_k on entry and the
// state entering chunk k on exit (slot 0: zero, never read).
constexpr int kCarryBatch = 8;
constexpr int kCarryRuns = 16;

__global__ __launch_bounds__(64 * kCarryRuns) void sel_carry_kernel(SelArgs a) {
    __shared__ float sL[kCarryRuns][64], sS[kCarryRuns][64];
    const int lane = threadIdx.x, g = threadIdx.y, runs = blockDim.y;
    const int64_t Dm = a.Dm, N = a.N;
    int item = blockIdx.x;
    const int dg = item % a.DG;
    item /= a.DG;
    const int64_t n = item % N;
    const int b = (int)(item / N);
    const int64_t d = (int64_t)dg * 64 + lane;
    const bool dok = d < Dm;
    const int64_t dd = dok ? d : Dm - 1;
    const float a2 = a.A[dd * N + n] * kLog2e;
    const int nk = a.K - 1;                            // chunks whose end state is carried
    const int per = (nk + runs - 1) / runs;
    const int k0 = min(nk, g * per), k1 = min(nk, k0 + per);
    const int64_t hstep = N * Dm;
    float* hp = a.ws_h + ((int64_t)b * a.K * N + n) * Dm + dd;
    const float* sp = a.ws_s + (int64_t)b * a.K * Dm + dd;

    // folds chunks [k0, k1) into c; with `store`, writes the entering state
    // of each chunk first. The next kCarryBatch chunks load while the current
    // ones are folded.
    auto walk = [&](float c, bool store, float& ssum) {
        float nl[kCarryBatch], ns[kCarryBatch];
        auto fetch = [&](int kb) {
#pragma unroll
            for (int j = 0; j < kCarryBatch; ++j) {
                const int kk = kb + j < k1 ? kb + j : k1 - 1;
                nl[j] = hp[kk * hstep];
                ns[j] = sp[kk * Dm];
            }
        };
        if (k1 > k0) fetch(k0);
        for (int kb = k0; kb < k1; kb += kCarryBatch) {
            float cl[kCarryBatch], cs[kCarryBatch];
#pragma unroll
            for (int j = 0; j < kCarryBatch; ++j) {
                cl[j] = nl[j];
                cs[j] = ns[j];
            }
            if (kb + kCarryBatch < k1) fetch(kb + kCarryBatch);
#pragma unroll
            for (int j = 0; j < kCarryBatch; ++j) {
                if (kb + j < k1) {
                    if (store && dok) hp[(kb + j) * hstep] = c;
                    c = fmaf(__builtin_amdgcn_exp2f(a2 * cs[j]), c, cl[j]);
                    ssum += cs[j];
                }
            }
        }
        return c;
    };
    // a run of at most kCarryBatch chunks is loaded once and kept in
    // registers for phase 3
    const bool one_batch = per <= kCarryBatch;
    float kl[kCarryBatch], ks[kCarryBatch];
    float ssum = 0.f;
    if (one_batch) {
        float c = 0.f;
#pragma unroll
        for (int j = 0; j < kCarryBatch; ++j) {
            const bool in = k0 + j < k1;
            const int kk = in ? k0 + j : k0;          // k0 <= K - 1: a valid slot
            const float l = hp[kk * hstep], sv = sp[kk * Dm];
            kl[j] = in ? l : 0.f;
            ks[j] = in ? sv : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kCarryBatch; ++j) {
            c = fmaf(__builtin_amdgcn_exp2f(a2 * ks[j]), c, kl[j]);
            ssum += ks[j];
        }
        sL[g][lane] = c;
    } else {
        sL[g][lane] = walk(0.f, false, ssum);
    }
    sS[g][lane] = ssum;
    __syncthreads();
    if (g == 0) {
        float run = 0.f;
        for (int r = 0; r < runs; ++r) {
            const float l = sL[r][lane];
            sL[r][lane] = run;
            run = fmaf(__builtin_amdgcn_exp2f(a2 * sS[r][lane]), run, l);
        }
    }
    __syncthreads();
    float c = sL[g][lane];
    if (one_batch) {
#pragma unroll
        for (int j = 0; j < kCarryBatch; ++j) {
            if (k0 + j < k1) {
                if (dok) hp[(k0 + j) * hstep] = c;
                c = fmaf(__builtin_amdgcn_exp2f(a2 * ks[j]), c, kl[j]);
            }
        }
    } else {
        float unused = 0.f;
        c = walk(c, true, unused);
    }
    if (k1 == nk && k1 > k0 && dok) hp[nk * hstep] = c;
}

// Runs per carry workgroup: about the square root of the carried chunks.
int sel_carry_runs(int K) {
    int r = 1;
    while (r < kCarryRuns && r * r < K - 1) r *= 2;
    return r;
}

template <int MODE>
void* sel_ptr(int64_t N) {
    if (N <= 16) return reinterpret_cast<void*>(&sel_scan_kernel<16, MODE>);
    if (N <= 32) return reinterpret_cast<void*>(&sel_scan_kernel<32, MODE>);
    if (N <= 64) return reinterpret_cast<void*>(&sel_scan_kernel<64, MODE>);
    return nullptr;
}

// Steps per block of the kernel that serves d_state N.
int64_t sel_steps_per_block(int64_t N) { return N <= 16 ? 8 : N <= 32 ? 4 : 2; }

static_assert(sel_block_steps<16>() == 8 && sel_block_steps<32>() == 4 && sel_block_steps<64>() == 2,
              "host and kernel block lengths differ");

// Chunk length (automatic): about 24 waves per CU over both passes' grids,
// so that every SIMD has several waves to interleave; chunks of at least 64
// steps (shorter ones cost more in per-chunk loads and in the carry than they
// gain in balance) and a whole number of blocks (a partial block costs as
// much as a full one); at most 1024 chunks.
constexpr int64_t kSelMaxChunks = 4096;    // explicit counts are clamped here

int64_t sel_chunk_len(int64_t b, int64_t T, int64_t DG, int64_t N, int cus) {
    const int64_t tb = sel_steps_per_block(N);
    const int64_t kt = (24 * (int64_t)cus + b * DG - 1) / (b * DG);
    int64_t lc = tb * ((T + kt * tb - 1) / (kt * tb));
    if (lc < 64) lc = 64;
    if ((T + lc - 1) / lc > 1024) lc = tb * (((T + 1023) / 1024 + tb - 1) / tb);
    return lc;
}

}  // namespace

extern "C" {

ssd_status ssd_selective_scan_ex(const float* u, const float* delta, const float* A, const float* B,
                                 const float* C, const float* skip, float* y, int64_t batch,
                                 int64_t seq_len, int64_t d_model, int64_t d_state,
                                 const ssd_launch_opts* opts, void* stream) {
    if (!u || !delta || !A || !B || !C || !skip || !y) return SSD_ERR_NULL_ARG;
    if (batch < 1 || seq_len < 1 || d_model < 1 || d_state < 1) return SSD_ERR_BAD_SHAPE;
    if (opts) {
        if (opts->segments < 0 || opts->block_slices < 0) return SSD_ERR_BAD_SHAPE;
        for (int i = 0; i < 2; ++i)
            if (opts->reserved[i] != 0) return SSD_ERR_BAD_SHAPE;
        if ((opts->walk_events[0] == nullptr) != (opts->walk_events[1] == nullptr)) return SSD_ERR_BAD_SHAPE;
        if (opts->block_slices != 0) return SSD_ERR_UNSUPPORTED;
    }
    // d_model bound: a chunk's states (d_state x d_model floats) and a block's
    // u/delta rows must stay below 2^31 bytes of buffer offset
    if (d_state > 64 || batch > 65535 || d_model > ((int64_t)1 << 22)) return SSD_ERR_UNSUPPORTED;
    const float* ins[] = {u, delta, A, B, C, skip};
    for (const float* p : ins)
        if (!aligned(p, 4)) return SSD_ERR_UNSUPPORTED;
    if (!aligned(y, 4)) return SSD_ERR_UNSUPPORTED;
    const int64_t b = batch, T = seq_len, Dm = d_model, N = d_state;
    const Span sy = span_of(y, b * T * Dm * 4);
    const Span sins[] = {span_of(u, b * T * Dm * 4), span_of(delta, b * T * Dm * 4), span_of(A, Dm * N * 4),
                         span_of(B, b * T * N * 4), span_of(C, b * T * N * 4), span_of(skip, Dm * 4)};
    for (const Span& si : sins)
        if (overlap(sy, si)) return SSD_ERR_ALIAS;
    if (b * T * Dm > ((int64_t)1 << 40)) return SSD_ERR_UNSUPPORTED;

    SelArgs a;
    memset(&a, 0, sizeof(a));
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.skip = skip; a.y = y;
    a.T = T; a.Dm = Dm; a.N = N;
    a.DG = (int)((Dm + 63) / 64);
    if (opts && opts->segments > 0) {
        const int64_t cap = T < kSelMaxChunks ? T : kSelMaxChunks;
        const int64_t want = opts->segments < cap ? opts->segments : cap;
        a.Lc = (T + want - 1) / want;
    } else {
        a.Lc = sel_chunk_len(b, T, a.DG, N, device_cus());
    }
    a.K = (int)((T + a.Lc - 1) / a.Lc);
    const int64_t nwg = b * a.K * a.DG;
    if (nwg > 0x7fffffff || b * N * a.DG > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    void* ws = nullptr;
    int ws_entry = -1;
    if (a.K > 1) {
        const size_t hbytes = align256((size_t)(b * a.K) * N * Dm * sizeof(float));
        ws = scratch_acquire(hs, hbytes + (size_t)(b * a.K) * Dm * sizeof(float), &ws_entry);
        if (!ws) return SSD_ERR_HIP;
        a.ws_h = static_cast<float*>(ws);
        a.ws_s = reinterpret_cast<float*>(static_cast<char*>(ws) + hbytes);
    }
    ssd_status rs = SSD_OK;
    void* kargs[] = {&a};
    if (a.K > 1) {
        a.Kw = a.K - 1;     // the last chunk's end state is never needed
        if (hipLaunchKernel(sel_ptr<1>(N), dim3((unsigned)(b * a.Kw * a.DG)), dim3(64), kargs, 0, hs) != hipSuccess)
            rs = SSD_ERR_HIP;
        if (rs == SSD_OK) {
            const int runs = sel_carry_runs(a.K);
            hipLaunchKernelGGL(sel_carry_kernel, dim3((unsigned)(b * N * a.DG)), dim3(64, runs), 0, hs, a);
            if (hipGetLastError() != hipSuccess) rs = SSD_ERR_HIP;
        }
    }
    a.Kw = a.K;
    const bool timed = opts && opts->walk_events[0];
    if (rs == SSD_OK && timed && hipEventRecord(reinterpret_cast<hipEvent_t>(opts->walk_events[0]), hs) != hipSuccess)
        rs = SSD_ERR_HIP;
    if (rs == SSD_OK &&
        hipLaunchKernel(sel_ptr<0>(N), dim3((unsigned)nwg), dim3(64), kargs, 0, hs) != hipSuccess)
        rs = SSD_ERR_HIP;
    if (rs == SSD_OK && timed && hipEventRecord(reinterpret_cast<hipEvent_t>(opts->walk_events[1]), hs) != hipSuccess)
        rs = SSD_ERR_HIP;
    if (ws && !scratch_release(ws_entry) && rs == SSD_OK) rs = SSD_ERR_HIP;
    return rs;
}


ssd_status ssd_selective_scan(const float* u, const float* delta, const float* A, const float* B,
                              const float* C, const float* skip, float* y, int64_t batch,
                              int64_t seq_len, int64_t d_model, int64_t d_state, void* stream) {
    return ssd_selective_scan_ex(u, delta, A, B, C, skip, y, batch, seq_len, d_model, d_state,
                                 nullptr, stream);
}

}  // extern "C"
