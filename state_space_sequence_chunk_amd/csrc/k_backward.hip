// Backward pass: orchestration and the kernels that do not depend on the state shape
// (reverse carry over chunks, the per-(batch, head) suffix sum, the sums over heads).
// The per-chunk kernels are templates in backward.h, instantiated per input dtype in
// k_backward_bf16.hip and k_backward_f32.hip.
#include "backward.h"

namespace ssd {

hipError_t launch_bwd_chunks_bf16(const BwdArgs& a, int batch, int P, int S, bool f, bool r,
                                  bool v, hipStream_t st);
hipError_t launch_bwd_chunks_f32(const BwdArgs& a, int batch, int P, int S, bool f, bool r,
                                 bool v, hipStream_t st);
hipError_t launch_bwd_mfma_bf16(const BwdArgs& a, int batch, int P, int S, hipStream_t st);
hipError_t launch_bwd_dR_mfma_bf16(const BwdArgs& a, int batch, int P, int S, hipStream_t st);

// ---- reverse carry over chunks: R_c (gradient at chunk c's end), dh0 -------------------
// In place over the per-chunk sums: reads dR_c, stores R_c, then R <- 2^{G_last} R + dR_c.
__global__ __launch_bounds__(64) void bwd_carry_kernel(float* __restrict__ R,
                                                        const float* __restrict__ G,
                                                        const float* __restrict__ dfinal,
                                                        float* __restrict__ dh0, int L, int T,
                                                        int nC, int PS) {
    const int per_bh = PS / 256;
    const size_t bh = blockIdx.x / per_bh;
    const int e = (blockIdx.x % per_bh) * 256 + threadIdx.x * 4;
    f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
    if (dfinal) r = *(const f32x4*)(dfinal + bh * PS + e);
    const float* gr = G + bh * L;
    float* base = R + bh * nC * (size_t)PS + e;
    for (int c = nC - 1; c >= 0; --c) {
        float* p = base + (size_t)c * PS;
        const f32x4 d = *(const f32x4*)p;
        *(f32x4*)p = r;
        const float dec = exp2_fast(gr[min((c + 1) * T, L) - 1]);
        r = dec * r + d;
    }
    if (dh0) *(f32x4*)(dh0 + bh * PS + e) = r;
}

// ---- per (batch, head): the suffix sum for the log-decay gradient, ddt, dA and dD -------
// da_t = sum_{t' >= t} (q_t' - dt_t' v_t') + <dfinal, final>. 1024 threads per (batch,
// head), each a contiguous run of tokens; the runs' totals are combined with wave prefix
// scans (DPP) and one LDS pass over the 16 wave totals.
constexpr int kScanThreads = 1024, kScanWaves = kScanThreads / 64;

// Sum over the workgroup (every thread gets the total); `red` holds kScanWaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) t += red[w];
    return t;
}

__global__ __launch_bounds__(kScanThreads) void bwd_scan_kernel(
    const float* __restrict__ q, const float* __restrict__ v, const float* __restrict__ dyx,
    const float* __restrict__ dt_t, const float* __restrict__ A, const float* __restrict__ dfinal,
    const float* __restrict__ fin, float* __restrict__ ddt, float* __restrict__ dA_bh,
    float* __restrict__ dD_bh, int L, int H, int PS) {
    __shared__ float s_red[kScanWaves], s_wave[kScanWaves];
    const int bh = blockIdx.x, h = bh % H, b = bh / H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // <dfinal, final>
    float cst = 0.f;
    if (dfinal)
        for (int i = tid; i < PS; i += kScanThreads)
            cst += dfinal[(size_t)bh * PS + i] * fin[(size_t)bh * PS + i];
    cst = block_sum(cst, s_red);
    // this thread's run of tokens and its total
    const int per = (L + kScanThreads - 1) / kScanThreads;
    const int ta = min(tid * per, L), tz = min(ta + per, L);
    const size_t o = (size_t)bh * L;
    // tokens in batches of 8 so that each batch's loads are in flight together
    constexpr int NB = 8;
    float run = 0.f;
    for (int tb = ta; tb < tz; tb += NB) {
        float tq[NB], td[NB], tv[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const bool ok = tb + k < tz;
            tq[k] = ok ? q[o + tb + k] : 0.f;
            td[k] = ok ? dt_t[o + tb + k] : 0.f;
            tv[k] = ok ? v[o + tb + k] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) run += tq[k] - td[k] * tv[k];
    }
    // sum of the runs after this thread's: total - inclusive prefix
    const float incl = wave_inclusive_scan(run);
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    float before = 0.f, total = 0.f;  // wave totals before this wave; all of them
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) {
        const float x = s_wave[w];
        before += w < wv ? x : 0.f;
        total += x;
    }
    float suffix = cst + total - (before + incl);
    const float ah = A[h];
    float pa = 0.f, pd = 0.f;
    // the same batches, last to first; token tb + k of a batch
    const int nbat = (tz - ta + NB - 1) / NB;
    for (int bi = nbat - 1; bi >= 0; --bi) {
        const int tb = ta + bi * NB;
        float tq[NB], td[NB], tv[NB], tx[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const bool ok = tb + k < tz;
            tq[k] = ok ? q[o + tb + k] : 0.f;
            td[k] = ok ? dt_t[o + tb + k] : 0.f;
            tv[k] = ok ? v[o + tb + k] : 0.f;
            tx[k] = ok ? dyx[o + tb + k] : 0.f;
        }
#pragma unroll
        for (int k = NB - 1; k >= 0; --k) {
            if (tb + k >= tz) continue;
            suffix += tq[k] - td[k] * tv[k];
            ddt[((size_t)b * L + tb + k) * H + h] = tv[k] + ah * suffix;
            pa += td[k] * suffix;
            pd += tx[k];
        }
    }
    pa = block_sum(pa, s_red);
    pd = block_sum(pd, s_red);
    if (tid == 0) {
        dA_bh[bh] = pa;
        dD_bh[bh] = pd;
    }
}

// ---- sums over the heads of each group (dB, dC) and over the batch (dA, dD) ------------
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ dBh,
                                                         const float* __restrict__ dCh,
                                                         float* __restrict__ dB,
                                                         float* __restrict__ dC, size_t nBG,
                                                         int hpg, int S) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // over [B, L, G, S]
    if (i >= nBG) return;
    const size_t s = i % S, blg = i / S;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < hpg; ++k) {
        const size_t j = (blg * hpg + k) * S + s;
        sb += dBh[j];
        sc += dCh[j];
    }
    dB[i] = sb;
    dC[i] = sc;
}

__global__ __launch_bounds__(256) void bwd_reduce_heads_kernel(const float* __restrict__ dA_bh,
                                                               const float* __restrict__ dD_bh,
                                                               float* __restrict__ dA,
                                                               float* __restrict__ dD, int B,
                                                               int H) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float sa = 0.f, sd = 0.f;
    for (int b = 0; b < B; ++b) {
        sa += dA_bh[(size_t)b * H + h];
        sd += dD_bh[(size_t)b * H + h];
    }
    dA[h] = sa;
    if (dD) dD[h] = sd;
}


__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

static hipError_t fill_zero(float* p, size_t n, hipStream_t s) {
    if (!p || n == 0) return hipSuccess;
    fill_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
    return hipGetLastError();
}

// Heads per workgroup of the matrix-core kernels: the largest divisor of the heads per
// group that still leaves a workgroup for every compute unit.
static int bwd_heads_per_block(int B, int nC, int H, int hpg) {
    int best = 1;
    for (int nh = 1; nh <= hpg; ++nh)
        if (hpg % nh == 0 && (long)B * nC * (H / nh) >= 256) best = nh;
    return best;
}

int bwd_partials_per_group(int in_dtype, const Dims& d) {
    const int hpg = d.nheads / d.ngroups;
    if (bwd_mfma_chunk(in_dtype, d.headdim, d.dstate) == d.chunk)
        return hpg / bwd_heads_per_block(d.batch, d.nchunks(), d.nheads, hpg);
    return hpg;
}

hipError_t launch_backward(int in_dtype, const BwdLaunch& k, const Dims& d, hipStream_t s) {
    const int B = d.batch, L = d.seqlen, H = d.nheads, P = d.headdim, S = d.dstate;
    const int G = d.ngroups, T = d.chunk, nC = d.nchunks(), PS = P * S;
    const int hpg = H / G;
    hipError_t e;
    if (L == 0) {  // no tokens: final = h0, so dh0 = dfinal; nothing else moves
        if (k.dh0) {
            e = launch_state_init(k.dfinal, k.dh0, d, s);
            if (e != hipSuccess) return e;
        }
        e = fill_zero(k.dA, H, s);
        if (e != hipSuccess) return e;
        return fill_zero(k.dD, H, s);
    }
    // forward quantities: cumulative decay, fp32 chunk-initial states, final state
    e = launch_cumsum(in_dtype, k.dt, k.A, k.ws.G, k.ws.dt_t, d, s);
    if (e != hipSuccess) return e;
    e = launch_chunk_state(in_dtype, k.x, k.B, k.A, k.ws.dt_t, k.ws.R, d, s);
    if (e != hipSuccess) return e;
    e = launch_state_carry(kF32, k.ws.R, k.ws.G, k.h0, k.ws.Hc, k.ws.fin, d, s);
    if (e != hipSuccess) return e;

    BwdArgs a;
    a.x = k.x; a.dt = k.dt; a.Bm = k.B; a.Cm = k.C; a.A = k.A; a.D = k.D; a.dy = k.dy;
    a.Gc = k.ws.G; a.dtt = k.ws.dt_t;
    a.Hc = k.ws.Hc; a.R = k.ws.R; a.dx = k.dx;
    a.dBh = hpg == 1 ? k.dB : k.ws.dBh;
    a.dCh = hpg == 1 ? k.dC : k.ws.dCh;
    a.v = k.ws.v; a.q = k.ws.q; a.dyx = k.ws.dyx;
    a.L = L; a.H = H; a.G = G; a.T = T; a.NH = 1;
    auto chunks = [&](bool f, bool r, bool v) {
        return in_dtype == kBF16 ? launch_bwd_chunks_bf16(a, B, P, S, f, r, v, s)
                                 : launch_bwd_chunks_f32(a, B, P, S, f, r, v, s);
    };
    // bf16 inputs with a matrix-core plan for this shape (run at its own chunk length,
    // which the caller has put in d): dC, dB and dx as chunked products; otherwise the
    // fp32 token walks
    const bool mfma = bwd_mfma_chunk(in_dtype, P, S) == T;
    // dB, dC partials to sum per group (per head with the walks; per block of a.NH heads,
    // summed inside the kernels, with the matrix-core path)
    const int parts = bwd_partials_per_group(in_dtype, d);
    if (mfma) {
        a.NH = hpg / parts;
        a.dBh = parts == 1 ? k.dB : k.ws.dBh;
        a.dCh = parts == 1 ? k.dC : k.ws.dCh;
    }
    // per-chunk sums dR_c (over the consumed increments), and with the walks the forward
    // walk (dC, q)
    if (mfma) e = launch_bwd_dR_mfma_bf16(a, B, P, S, s);
    else e = chunks(true, true, false);
    if (e != hipSuccess) return e;
    bwd_carry_kernel<<<B * H * (PS / 256), 64, 0, s>>>(k.ws.R, k.ws.G, k.dfinal, k.dh0, L, T, nC,
                                                       PS);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (mfma) {
        e = launch_bwd_mfma_bf16(a, B, P, S, s);
    } else {
        e = chunks(false, false, true);
    }
    if (e != hipSuccess) return e;
    bwd_scan_kernel<<<B * H, kScanThreads, 0, s>>>(k.ws.q, k.ws.v, k.ws.dyx, k.ws.dt_t, k.A, k.dfinal,
                                          k.ws.fin, k.ddt, k.ws.dA_bh, k.ws.dD_bh, L, H, PS);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (parts > 1) {
        const size_t n = (size_t)B * L * G * S;
        bwd_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(k.ws.dBh, k.ws.dCh, k.dB,
                                                                      k.dC, n, parts, S);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    bwd_reduce_heads_kernel<<<(H + 255) / 256, 256, 0, s>>>(k.ws.dA_bh, k.ws.dD_bh, k.dA, k.dD,
                                                            B, H);
    return hipGetLastError();
}

}  // namespace ssd
