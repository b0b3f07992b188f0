// Backward pass of the SSD recurrence (kernel templates; instantiated in k_backward_*.hip).
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Mamba-2 architecture" (the recurrence) differentiated in reverse mode.
// With Lam_t = dL/dH_t (H_t the [P][S] state after token t, all later uses included):
//     Lam_t = dy_t (outer) C_t + exp(a_{t+1}) Lam_{t+1}
//     dx_t  = D dy_t + dt_t Lam_t B_t,   dB_t = dt_t Lam_t^T x_t,   dC_t = H_t^T dy_t
// and the gradient of the log decays a_t = A dt_t is a suffix sum of per-token scalars:
//     dL/da_t = sum_{t' >= t} (q_t' - dt_t' v_t') + <dfinal, final>,
//     q_t = dy_t . (H_t C_t),   v_t = x_t . (Lam_t B_t)
// (expand <Lam_t, exp(a_t) H_{t-1}> = <Lam_t, H_t> - dt_t v_t and telescope). Then
//     ddt_t = v_t + A dL/da_t,   dA = sum_t dt_t dL/da_t,   dD = sum_t dy_t . x_t.
//
// Chunked like the forward pass: the state entering each chunk (H_c) comes from the
// forward state pass, and the gradient arriving at each chunk's end from later tokens,
// R_c, from a reverse carry over per-chunk sums dR_c = sum_{t in c} 2^{G_t} dy_t C_t^T
// (G_t the inclusive log2 decay from the chunk's start): R_{c-1} = 2^{G_last} R_c + dR_c,
// R_{last} = dfinal, dh0 = R_{-1}. Inside a chunk each (batch, chunk, head) walks its
// tokens: forward from H_c for dC and q, backward from R_c for dx, dB and v.
//
// gfx950 mapping: one workgroup of NW waves per (batch, chunk, head); wave w owns the
// state columns [w*S/NW, (w+1)*S/NW) and each lane an RR x NC tile of them (at most 128
// fp32 values in registers). Sums over a row (dx) or a column (dB, dC) of the state are
// lane shuffles inside the wave; the per-token sums that span waves (dx, v and q when
// NW > 1) go through LDS once per 32 tokens. All arithmetic is fp32.
#pragma once

#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

template <int P, int S>
struct BwdCfg {
    static constexpr int NW = (P * S + 8191) / 8192;  // waves per workgroup
    static constexpr int SB = S / NW;                 // state columns per wave
    static constexpr int E = P * SB / 64;             // state values per lane
    static constexpr int RR = E < 8 ? E : 8;          // rows per lane
    static constexpr int NC = E / RR;                 // columns per lane
    static constexpr int RB = P / RR;                 // row blocks
    static constexpr int CB = 64 / RB;                // column blocks
    // tokens per cross-wave reduction (keeps the LDS partials of dx within 32 KiB)
    static constexpr int TS = NW * P * 32 * 4 > 32768 ? 16 : 32;
    static_assert(CB * NC == SB && RB * CB == 64 && RR * RB == P, "lane tiling");
};

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* p, float* out) {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f32(p[i]);
}

// Sum over the lanes whose index differs only in bits LO, 2 LO, ... below HI.
template <int LO, int HI>
__device__ __forceinline__ float lane_sum(float v) {
#pragma unroll
    for (int m = LO; m < HI; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

struct BwdArgs {
    const void* x;    // [B, L, H, P] in_dtype
    const void* dt;   // [B, L, H] in_dtype
    const void* Bm;   // [B, L, G, S] in_dtype
    const void* Cm;   // [B, L, G, S] in_dtype
    const float* A;   // [H]
    const float* D;   // [H] or null
    const float* dy;  // [B, L, H, P]
    const float* Gc;  // [B, H, L] per-chunk cumulative log2 decay
    const float* dtt; // [B, H, L] dt (fp32)
    const float* Hc;  // [B, H, nC, P, S] chunk-initial states (fp32)
    float* R;         // [B, H, nC, P, S] dR_c, then R_c
    float* dx;        // [B, L, H, P]
    float* dBh;       // [B, L, H, S] dB of each head (dB itself with one head per group)
    float* dCh;       // [B, L, H, S]
    float* v;         // [B, H, L]
    float* q;         // [B, H, L]
    float* dyx;       // [B, H, L]
    int L, H, G, T;
    int NH;           // heads per workgroup of the matrix-core kernels (divides H / G)
};

struct BwdUnit {
    int b, c, h, g, wave, lane, rb, cb, p0, s0, t0, t1, nC;
};

template <int P, int S>
__device__ __forceinline__ BwdUnit bwd_unit(const BwdArgs& a) {
    using Cfg = BwdCfg<P, S>;
    BwdUnit u;
    u.nC = (a.L + a.T - 1) / a.T;
    u.h = blockIdx.x % a.H;
    u.c = (blockIdx.x / a.H) % u.nC;
    u.b = blockIdx.x / (a.H * u.nC);
    u.g = u.h / (a.H / a.G);
    u.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u.lane = threadIdx.x & 63;
    u.rb = u.lane / Cfg::CB;
    u.cb = u.lane % Cfg::CB;
    u.p0 = u.rb * Cfg::RR;
    u.s0 = u.wave * Cfg::SB + u.cb * Cfg::NC;
    u.t0 = u.c * a.T;
    u.t1 = min(u.t0 + a.T, a.L);
    return u;
}

// ---- forward walk: dC_t = H_t^T dy_t and q_t = dy_t . H_t C_t ------------------------
template <typename TIn, int P, int S>
__global__ __launch_bounds__(256) void bwd_fwd_kernel(BwdArgs a) {
    using Cfg = BwdCfg<P, S>;
    constexpr int RR = Cfg::RR, NC = Cfg::NC, CB = Cfg::CB, RB = Cfg::RB, NW = Cfg::NW;
    constexpr int TS = Cfg::TS;
    __shared__ float s_q[NW][TS];
    const TIn* x = (const TIn*)a.x;
    const TIn* dt = (const TIn*)a.dt;
    const TIn* Bm = (const TIn*)a.Bm;
    const TIn* Cm = (const TIn*)a.Cm;
    const BwdUnit u = bwd_unit<P, S>(a);
    const int L = a.L, H = a.H, G = a.G;
    const float ah = a.A[u.h] * kLog2e;

    float Hs[RR][NC];
    const float* hc = a.Hc + ((((size_t)u.b * H + u.h) * u.nC + u.c) * P + u.p0) * S + u.s0;
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int k = 0; k < NC; ++k) Hs[r][k] = hc[(size_t)r * S + k];

    for (int tb = u.t0; tb < u.t1; tb += TS) {
        const int te = min(tb + TS, u.t1);
        for (int t = tb; t < te; ++t) {
            const size_t bt = (size_t)u.b * L + t;
            const float dtv = to_f32(dt[bt * H + u.h]);
            const float al = exp2_fast(ah * dtv);
            float xr[RR], dyr[RR], br[NC], cr[NC];
            load_vec<TIn, RR>(x + (bt * H + u.h) * P + u.p0, xr);
            load_vec<float, RR>(a.dy + (bt * H + u.h) * P + u.p0, dyr);
            load_vec<TIn, NC>(Bm + (bt * G + u.g) * S + u.s0, br);
            load_vec<TIn, NC>(Cm + (bt * G + u.g) * S + u.s0, cr);
            float z[NC];
#pragma unroll
            for (int k = 0; k < NC; ++k) z[k] = 0.f;
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                const float w = dtv * xr[r];
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    Hs[r][k] = al * Hs[r][k] + w * br[k];
                    z[k] += Hs[r][k] * dyr[r];
                }
            }
            float qp = 0.f;
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                z[k] = lane_sum<CB, 64>(z[k]);  // over the row blocks: the whole column
                qp += z[k] * cr[k];
            }
            qp = lane_sum<1, CB>(qp);  // over this wave's columns
            float* dc = a.dCh + (bt * H + u.h) * S + u.s0;
#pragma unroll
            for (int k = 0; k < NC; ++k)
                if (k % RB == u.rb) dc[k] = z[k];
            if constexpr (NW == 1) {
                if (u.lane == 0) a.q[((size_t)u.b * H + u.h) * L + t] = qp;
            } else {
                if (u.lane == 0) s_q[u.wave][t - tb] = qp;
            }
        }
        if constexpr (NW > 1) {
            __syncthreads();
            if ((int)threadIdx.x < te - tb) {
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) s += s_q[w][threadIdx.x];
                a.q[((size_t)u.b * H + u.h) * L + tb + threadIdx.x] = s;
            }
            __syncthreads();
        }
    }
}

// ---- per-chunk sums for the reverse carry: dR_c = sum_t 2^{G_t} dy_t C_t^T ---------------
template <typename TIn, int P, int S>
__global__ __launch_bounds__(256) void bwd_dR_kernel(BwdArgs a) {
    using Cfg = BwdCfg<P, S>;
    constexpr int RR = Cfg::RR, NC = Cfg::NC;
    const TIn* dt = (const TIn*)a.dt;
    const TIn* Cm = (const TIn*)a.Cm;
    const BwdUnit u = bwd_unit<P, S>(a);
    const int L = a.L, H = a.H, G = a.G;
    const float ah = a.A[u.h] * kLog2e;
    float acc[RR][NC];
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int k = 0; k < NC; ++k) acc[r][k] = 0.f;
    float w = 1.f;  // 2^{G_t}: the decay from the chunk's start through token t
    for (int t = u.t0; t < u.t1; ++t) {
        const size_t bt = (size_t)u.b * L + t;
        w *= exp2_fast(ah * to_f32(dt[bt * H + u.h]));
        float dyr[RR], cr[NC];
        load_vec<float, RR>(a.dy + (bt * H + u.h) * P + u.p0, dyr);
        load_vec<TIn, NC>(Cm + (bt * G + u.g) * S + u.s0, cr);
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const float wd = w * dyr[r];
#pragma unroll
            for (int k = 0; k < NC; ++k) acc[r][k] += wd * cr[k];
        }
    }
    float* out = a.R + ((((size_t)u.b * H + u.h) * u.nC + u.c) * P + u.p0) * S + u.s0;
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int k = 0; k < NC; ++k) out[(size_t)r * S + k] = acc[r][k];
}

// ---- reverse walk: dx_t, dB_t (this head), v_t = x_t . Lam_t B_t, dy_t . x_t ------------
template <typename TIn, int P, int S>
__global__ __launch_bounds__(256) void bwd_rev_kernel(BwdArgs a) {
    using Cfg = BwdCfg<P, S>;
    constexpr int RR = Cfg::RR, NC = Cfg::NC, CB = Cfg::CB, RB = Cfg::RB, NW = Cfg::NW;
    constexpr int TS = Cfg::TS;
    __shared__ float s_u[NW > 1 ? NW : 1][TS][P];
    __shared__ float s_v[NW][TS];
    const TIn* x = (const TIn*)a.x;
    const TIn* dt = (const TIn*)a.dt;
    const TIn* Bm = (const TIn*)a.Bm;
    const TIn* Cm = (const TIn*)a.Cm;
    const BwdUnit u = bwd_unit<P, S>(a);
    const int L = a.L, H = a.H, G = a.G;
    const float ah = a.A[u.h] * kLog2e;
    const float dval = a.D ? a.D[u.h] : 0.f;
    const size_t bhL = ((size_t)u.b * H + u.h) * L;

    float Lam[RR][NC];
    const float* rc = a.R + ((((size_t)u.b * H + u.h) * u.nC + u.c) * P + u.p0) * S + u.s0;
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int k = 0; k < NC; ++k) Lam[r][k] = rc[(size_t)r * S + k];

    float carry = 1.f;  // exp(a_{t+1}): the step from the token after t (1 at the chunk end)
    for (int te = u.t1; te > u.t0; te -= TS) {
        const int tb = max(te - TS, u.t0);
        for (int t = te - 1; t >= tb; --t) {
            const size_t bt = (size_t)u.b * L + t;
            const float dtv = to_f32(dt[bt * H + u.h]);
            float xr[RR], dyr[RR], br[NC], cr[NC];
            load_vec<TIn, RR>(x + (bt * H + u.h) * P + u.p0, xr);
            load_vec<float, RR>(a.dy + (bt * H + u.h) * P + u.p0, dyr);
            load_vec<TIn, NC>(Bm + (bt * G + u.g) * S + u.s0, br);
            load_vec<TIn, NC>(Cm + (bt * G + u.g) * S + u.s0, cr);
            float ur[RR], wc[NC];
#pragma unroll
            for (int k = 0; k < NC; ++k) wc[k] = 0.f;
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                ur[r] = 0.f;
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    Lam[r][k] = carry * Lam[r][k] + dyr[r] * cr[k];
                    ur[r] += Lam[r][k] * br[k];
                    wc[k] += Lam[r][k] * xr[r];
                }
            }
            carry = exp2_fast(ah * dtv);
            // dB_t of this head: column sums over the row blocks, times dt
            float vp = 0.f;
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                wc[k] = lane_sum<CB, 64>(wc[k]);
                vp += wc[k] * br[k];
            }
            vp = lane_sum<1, CB>(vp);  // v_t over this wave's columns
            float* db = a.dBh + (bt * H + u.h) * S + u.s0;
#pragma unroll
            for (int k = 0; k < NC; ++k)
                if (k % RB == u.rb) db[k] = dtv * wc[k];
            // dy_t . x_t over all rows (each row block once)
            float dx_dot = 0.f;
#pragma unroll
            for (int r = 0; r < RR; ++r) dx_dot += dyr[r] * xr[r];
            dx_dot = lane_sum<CB, 64>(dx_dot);
            if (u.wave == 0 && u.lane == 0) a.dyx[bhL + t] = dx_dot;
            // row sums of Lam B over this wave's columns
#pragma unroll
            for (int r = 0; r < RR; ++r) ur[r] = lane_sum<1, CB>(ur[r]);
            if constexpr (NW == 1) {
                float* dxr = a.dx + (bt * H + u.h) * P + u.p0;
#pragma unroll
                for (int r = 0; r < RR; ++r)
                    if (r % CB == u.cb) dxr[r] = dval * dyr[r] + dtv * ur[r];
                if (u.lane == 0) a.v[bhL + t] = vp;
            } else {
#pragma unroll
                for (int r = 0; r < RR; ++r)
                    if (r % CB == u.cb) s_u[u.wave][t - tb][u.p0 + r] = ur[r];
                if (u.lane == 0) s_v[u.wave][t - tb] = vp;
            }
        }
        if constexpr (NW > 1) {
            __syncthreads();
            for (int e = threadIdx.x; e < (te - tb) * P; e += NW * 64) {
                const int tt = e / P, p = e % P;
                const size_t bt = (size_t)u.b * L + tb + tt;
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) s += s_u[w][tt][p];
                const float dtv = to_f32(dt[bt * H + u.h]);
                a.dx[(bt * H + u.h) * P + p] = dval * a.dy[(bt * H + u.h) * P + p] + dtv * s;
            }
            if ((int)threadIdx.x < te - tb) {
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) s += s_v[w][threadIdx.x];
                a.v[bhL + tb + threadIdx.x] = s;
            }
            __syncthreads();
        }
    }
}

// ---- launch helpers -----------------------------------------------------------------------
template <typename TIn, int P, int S>
hipError_t run_bwd_chunks(const BwdArgs& a, int batch, bool fwd_walk, bool dR, bool rev_walk,
                          hipStream_t stream) {
    using Cfg = BwdCfg<P, S>;
    const int nC = (a.L + a.T - 1) / a.T;
    const int nblocks = batch * nC * a.H;
    if (fwd_walk) bwd_fwd_kernel<TIn, P, S><<<nblocks, 64 * Cfg::NW, 0, stream>>>(a);
    if (dR) bwd_dR_kernel<TIn, P, S><<<nblocks, 64 * Cfg::NW, 0, stream>>>(a);
    if (rev_walk) bwd_rev_kernel<TIn, P, S><<<nblocks, 64 * Cfg::NW, 0, stream>>>(a);
    return hipGetLastError();
}

template <typename TIn, int P>
hipError_t bwd_by_s(const BwdArgs& a, int batch, int S, bool f, bool r, bool v, hipStream_t st) {
    switch (S) {
        case 16: return run_bwd_chunks<TIn, P, 16>(a, batch, f, r, v, st);
        case 32: return run_bwd_chunks<TIn, P, 32>(a, batch, f, r, v, st);
        case 64: return run_bwd_chunks<TIn, P, 64>(a, batch, f, r, v, st);
        case 128: return run_bwd_chunks<TIn, P, 128>(a, batch, f, r, v, st);
        case 256: return run_bwd_chunks<TIn, P, 256>(a, batch, f, r, v, st);
    }
    return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t bwd_chunks(const BwdArgs& a, int batch, int P, int S, bool f, bool r, bool v,
                      hipStream_t st) {
    switch (P) {
        case 16: return bwd_by_s<TIn, 16>(a, batch, S, f, r, v, st);
        case 32: return bwd_by_s<TIn, 32>(a, batch, S, f, r, v, st);
        case 64: return bwd_by_s<TIn, 64>(a, batch, S, f, r, v, st);
        case 128: return bwd_by_s<TIn, 128>(a, batch, S, f, r, v, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ssd
