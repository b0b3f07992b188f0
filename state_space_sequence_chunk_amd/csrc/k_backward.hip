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

// ---- reverse carry over chunks: R_c (gradient at chunk c's end), dh0, anchors -----------
// In place over the per-chunk sums: reads dR_c, stores R_c, then R <- 2^{G_last} R + dR_c.
// R_c is the gradient reaching the state after chunk c (Hc_{c+1}, or the final state for
// the last chunk) from everything later, so <R_c, Hc_{c+1}> is the log-decay gradient at
// the first token after chunk c (da_t = alpha_t <Lam_t, h_{t-1}>). Each wave adds up its
// 256 elements of that inner product and stores it as one of the PS/256 partials of
// chunk c; the suffix sums for da then start from these anchors at every chunk end
// instead of running over the whole sequence, which keeps their rounding local to a
// chunk (over the whole sequence it grows with its length).
// dR_c and H_{c+1} are read once and R_c written once here (R_c is read again only by
// later kernels, long after it has left the caches), so all three go through
// non-temporal accesses.
constexpr int kCarryBatch = 8;  // chunks whose loads are in flight together

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__global__ __launch_bounds__(64) void bwd_carry_kernel(float* __restrict__ R,
                                                        const float* __restrict__ G,
                                                        const float* __restrict__ Hc,
                                                        const float* __restrict__ fin,
                                                        const float* __restrict__ dfinal,
                                                        float* __restrict__ dh0,
                                                        float* __restrict__ anc, int L, int T,
                                                        int nC, int PS) {
    const int per_bh = PS / 256;
    const size_t bh = blockIdx.x / per_bh;
    const int slot = blockIdx.x % per_bh;
    const int e = slot * 256 + threadIdx.x * 4;
    f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
    if (dfinal) r = *(const f32x4*)(dfinal + bh * PS + e);
    const float* gr = G + bh * L;
    float* base = R + bh * nC * (size_t)PS + e;
    const float* hbase = Hc + bh * nC * (size_t)PS + e;
    const f32x4 hfin = *(const f32x4*)(fin + bh * PS + e);
    float* ap = anc + bh * nC * (size_t)per_bh + slot;
    for (int c0 = nC - 1; c0 >= 0; c0 -= kCarryBatch) {
        f32x4 d[kCarryBatch], hn[kCarryBatch];
        float dec[kCarryBatch];
#pragma unroll
        for (int u = 0; u < kCarryBatch; ++u) {
            const int c = c0 - u;
            if (c >= 0) {
                d[u] = __builtin_nontemporal_load((const f32x4*)(base + (size_t)c * PS));
                hn[u] = c + 1 < nC
                            ? __builtin_nontemporal_load((const f32x4*)(hbase + (size_t)(c + 1) * PS))
                            : hfin;
                dec[u] = exp2_fast(gr[min((c + 1) * T, L) - 1]);
            }
        }
        float part[kCarryBatch];
#pragma unroll
        for (int u = 0; u < kCarryBatch; ++u) {
            const int c = c0 - u;
            part[u] = 0.f;
            if (c >= 0) {
                __builtin_nontemporal_store(r, (f32x4*)(base + (size_t)c * PS));
                part[u] = r[0] * hn[u][0] + r[1] * hn[u][1] + r[2] * hn[u][2] + r[3] * hn[u][3];
                r = dec[u] * r + d[u];
            }
        }
#pragma unroll
        for (int u = 0; u < kCarryBatch; ++u) {
            const float tot = wave_sum(part[u]);
            if (threadIdx.x == 0 && c0 - u >= 0) ap[(size_t)(c0 - u) * per_bh] = tot;
        }
    }
    if (dh0) *(f32x4*)(dh0 + bh * PS + e) = r;
}

// ---- per (batch, head): the suffix sums for the log-decay gradient, ddt, dA and dD ------
// Within chunk c, da_t = a_c + sum_{t' >= t in chunk c} (q_t' - dt_t' v_t'), where the
// anchor a_c = <R_c, state after chunk c> is the sum of the chunk's PS/256 partials (for
// the last chunk R = dfinal and the state is the final one, so a = <dfinal, final>).
// ddt_t = v_t + A da_t; dA = sum_t dt_t da_t; dD = sum_t dy_t . x_t. One workgroup of
// 16 waves per (batch, head); the waves take the chunks in turn, each lane a run of
// T/64 consecutive tokens, and a wave prefix scan (DPP) gives the sums over later lanes.
constexpr int kScanThreads = 1024, kScanWaves = kScanThreads / 64;

// Sum over the workgroup (every thread gets the total); `red` holds kScanWaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) t += red[w];
    return t;
}

template <int K>  // tokens per lane: T / 64
__global__ __launch_bounds__(kScanThreads) void bwd_scan_kernel(
    const float* __restrict__ q, const float* __restrict__ v, const float* __restrict__ dyx,
    const float* __restrict__ dt_t, const float* __restrict__ A, const float* __restrict__ anc,
    float* __restrict__ ddt, float* __restrict__ dA_bh, float* __restrict__ dD_bh, int L, int H,
    int nC, int per_bh) {
    __shared__ float s_red[kScanWaves];
    constexpr int T = 64 * K;
    const int bh = blockIdx.x, h = bh % H, b = bh / H;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const size_t o = (size_t)bh * L;
    const float ah = A[h];
    float pa = 0.f, pd = 0.f;
    for (int c = wv; c < nC; c += kScanWaves) {
        // the anchor: sum of the chunk's partials
        const float* ap = anc + ((size_t)bh * nC + c) * per_bh;
        float a = 0.f;
        for (int i = lane; i < per_bh; i += 64) a += ap[i];
        a = wave_sum(a);
        // this lane's tokens t0 + K lane + k (zero past the sequence's end)
        const int t0 = c * T + K * lane;
        float tq[K], tv[K], td[K], tw[K];
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool ok = t0 + k < L;
            tq[k] = ok ? q[o + t0 + k] : 0.f;
            tv[k] = ok ? v[o + t0 + k] : 0.f;
            td[k] = ok ? dt_t[o + t0 + k] : 0.f;
            pd += ok ? dyx[o + t0 + k] : 0.f;
            tw[k] = tq[k] - td[k] * tv[k];
            run += tw[k];
        }
        // sum over the later lanes of the chunk: wave total - inclusive prefix
        const float incl = wave_inclusive_scan(run);
        const float total = __shfl(incl, 63, 64);
        float suffix = a + (total - incl);
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
            suffix += tw[k];
            if (t0 + k < L) {
                ddt[((size_t)b * L + t0 + k) * H + h] = tv[k] + ah * suffix;
                pa += td[k] * suffix;
            }
        }
    }
    pa = block_sum(pa, s_red);
    pd = block_sum(pd, s_red);
    if (threadIdx.x == 0) {
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
    if (state_scan_preferred(in_dtype, d)) {  // the single pass, where it is the faster
        e = launch_state_scan(kF32, k.x, k.B, k.A, k.ws.dt_t, k.h0, k.ws.Hc, k.ws.fin, d, s);
        if (e != hipSuccess) return e;
    } else {
        e = launch_chunk_state(in_dtype, k.x, k.B, k.A, k.ws.dt_t, k.ws.R, d, s);
        if (e != hipSuccess) return e;
        e = launch_state_carry(kF32, k.ws.R, k.ws.G, k.h0, k.ws.Hc, k.ws.fin, d, s);
        if (e != hipSuccess) return e;
    }

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
    bwd_carry_kernel<<<B * H * (PS / 256), 64, 0, s>>>(k.ws.R, k.ws.G, k.ws.Hc, k.ws.fin,
                                                       k.dfinal, k.dh0, k.ws.anc, L, T, nC, PS);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (mfma) {
        e = launch_bwd_mfma_bf16(a, B, P, S, s);
    } else {
        e = chunks(false, false, true);
    }
    if (e != hipSuccess) return e;
    {
        auto scan = T == 64 ? bwd_scan_kernel<1> : T == 128 ? bwd_scan_kernel<2> : bwd_scan_kernel<4>;
        scan<<<B * H, kScanThreads, 0, s>>>(k.ws.q, k.ws.v, k.ws.dyx, k.ws.dt_t, k.A, k.ws.anc,
                                            k.ddt, k.ws.dA_bh, k.ws.dD_bh, L, H, nC, PS / 256);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
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
