// Stage 2a, multi-head form: each chunk's own contribution to the state that leaves it,
// for a block of heads of one B group per workgroup (kernel template; instantiated in
// k_chunk_state_mh_*.hip).
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Mamba-2 architecture" (the log-space jump formula) and section
// "Kernel 2: fwd_pass_state" (operand fusion before the matrix product):
//     dS_c[p][s] = sum_{j in chunk} (dt_j 2^{G_last - G_j} x_j[p]) B_j[s]
// with the exponent summed from the chunk's end (so its rounding is relative to the
// exponents that dominate the state).
//
// gfx950 mapping: one workgroup of 8 waves per (batch, chunk, block of NH heads). The
// chunk's B rows are staged once in LDS and shared by the NH heads; each head's x rows
// are double-buffered in LDS and the next head's rows are loaded while the current head's
// products run, with one barrier per head. B and x fragments (tokens along K) come from
// the gfx950 transposing LDS read. The fused operand dt_j 2^{...} x_j[p] is formed in fp32
// and, for bf16 inputs, split into a bf16 high part and a bf16 remainder (two MFMAs
// against the exact bf16 B), which keeps ~16 significant bits. Wave 0 forms each head's
// decay weights with a single-wave DPP scan while the other waves work.
#pragma once

#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int P, int S, int T>
struct StateMhCfg {
    static constexpr int NTHR = 512, NWAVE = 8;
    static constexpr int NPT = P / 16, NST = S / 16;
    static constexpr int WPT = NPT >= NWAVE ? 1 : NWAVE / NPT;  // waves per p-tile
    static constexpr int MST = (NST + WPT - 1) / WPT;           // s-tiles per wave
    static constexpr int VE = 16 / (int)sizeof(TIn);
    static constexpr int XS = col_stride<TIn>(P), BS = col_stride<TIn>(S);
    static constexpr int NXV = (T * P / VE + NTHR - 1) / NTHR;  // x vectors per thread
    static constexpr int NBV = (T * S / VE + NTHR - 1) / NTHR;  // B vectors per thread
    static constexpr int PER = T / 64;                          // tokens per lane in the scan
    static constexpr size_t X_BYTES = (size_t)T * XS * sizeof(TIn);
    static constexpr size_t W_BYTES = (size_t)T * sizeof(float);
    static constexpr size_t B_BYTES = (size_t)T * BS * sizeof(TIn);
    static constexpr size_t LDS_BYTES = B_BYTES + 2 * (X_BYTES + W_BYTES);
    static constexpr bool FITS = LDS_BYTES <= 163840 && NPT <= NWAVE;
};

template <typename TIn, int P, int S, int T>
__global__ __launch_bounds__(512) void chunk_state_mh_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ dt_t, float* __restrict__ dS, int L, int H, int ngroups, int NH) {
    using Cfg = StateMhCfg<TIn, P, S, T>;
    constexpr int VE = Cfg::VE, XS = Cfg::XS, BS = Cfg::BS, NTHR = Cfg::NTHR, PER = Cfg::PER;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    TIn* s_b = (TIn*)smem;  // [T][BS]
    auto s_x = [&](int k) { return (TIn*)(smem + Cfg::B_BYTES + k * (Cfg::X_BYTES + Cfg::W_BYTES)); };
    auto s_w = [&](int k) {
        return (float*)(smem + Cfg::B_BYTES + k * (Cfg::X_BYTES + Cfg::W_BYTES) + Cfg::X_BYTES);
    };

    const int nC = (L + T - 1) / T;
    const int nhb = H / NH;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = id % nhb;
    const int c = (id / nhb) % nC;
    const int b = id / (nhb * nC);
    const int h_first = hb * NH;
    const int g = h_first / (H / ngroups);  // NH divides the heads per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int t0 = c * T;
    const int rows = min(T, L - t0);  // real tokens of this chunk; the rest count as zeros
    const int HP = H * P;
    const int pt = wave / Cfg::WPT;          // this wave's p-tile
    const int st0 = wave % Cfg::WPT;         // first s-tile; stride WPT
    const bool active = pt < Cfg::NPT;

    // x rows past the chunk's real tokens lie outside the descriptor and load as zeros
    const BufRsrc rx = make_rsrc(x + ((size_t)b * L + t0) * HP, (uint32_t)(rows * HP * sizeof(TIn)));
    const BufRsrc rdt = make_rsrc(dt_t + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));

    // ---- per-head staging --------------------------------------------------------------
    Vec16 px[Cfg::NXV];
    float pdt[PER];
    auto load_head = [&](int h) {
#pragma unroll
        for (int i = 0; i < Cfg::NXV; ++i) {
            const int v = tid + i * NTHR;
            if (v < T * P / VE) {
                const int r = v / (P / VE), col = (v % (P / VE)) * VE;
                px[i] = buf_load16(rx, (uint32_t)((r * HP + col) * sizeof(TIn)),
                                   (uint32_t)(h * P * sizeof(TIn)));
            }
        }
        if (wave == 0) {  // wave 0 scans the head's decay; lane holds tokens T-1-(PER*lane+k)
            const uint32_t o = (uint32_t)(((size_t)h * L + t0) * sizeof(float));
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int t = T - 1 - (PER * lane + k);
                pdt[k] = t < rows ? buf_load_f32(rdt, t * 4, o) : 0.f;
            }
        }
    };
    auto store_head = [&](int h, int kb) {
        TIn* bx = s_x(kb);
#pragma unroll
        for (int i = 0; i < Cfg::NXV; ++i) {
            const int v = tid + i * NTHR;
            if (v < T * P / VE) {
                const int r = v / (P / VE), col = (v % (P / VE)) * VE;
                *(Vec16*)(bx + r * XS + col) = px[i];
            }
        }
        if (wave == 0) {
            // w_t = dt_t 2^{log2(e) sum_{k>t} A dt_k}: scanned from the chunk's end
            const float ah = A[h];
            float pre[PER], run = 0.f;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                pre[k] = run;
                run += ah * pdt[k];
            }
            const float excl = wave_shift_up1(wave_inclusive_scan(run));
            float* bw = s_w(kb);
#pragma unroll
            for (int k = 0; k < PER; ++k)
                bw[T - 1 - (PER * lane + k)] = pdt[k] * exp2_fast((excl + pre[k]) * kLog2e);
        }
    };

    // ---- prologue: B rows, first head --------------------------------------------------
    load_head(h_first);
    {
        const TIn* bg = Bm + (((size_t)b * L + t0) * ngroups + g) * S;
        const size_t grow = (size_t)ngroups * S;
        Vec16 pb[Cfg::NBV];
#pragma unroll
        for (int i = 0; i < Cfg::NBV; ++i) {
            const int v = tid + i * NTHR;
            if (v < T * S / VE) {
                const int r = v / (S / VE), col = (v % (S / VE)) * VE;
                pb[i] = r < rows ? *(const Vec16*)(bg + (size_t)r * grow + col) : Vec16{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::NBV; ++i) {
            const int v = tid + i * NTHR;
            if (v < T * S / VE) {
                const int r = v / (S / VE), col = (v % (S / VE)) * VE;
                *(Vec16*)(s_b + r * BS + col) = pb[i];
            }
        }
    }
    store_head(h_first, 0);
    __syncthreads();

    for (int hh = 0; hh < NH; ++hh) {
        const int h = h_first + hh;
        const int kb = hh & 1;
        const TIn* bx = s_x(kb);
        const float* bw = s_w(kb);
        if (hh + 1 < NH) load_head(h + 1);  // in flight while this head's products run

        f32x4 acc[Cfg::MST];
#pragma unroll
        for (int m = 0; m < Cfg::MST; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (active) {
            // slot (g4, v) carries token 32 ks + 16 (v/4) + 4 g4 + v%4 (two column reads)
            for (int ks = 0; ks < T / 32; ++ks) {
                const int r_lo = ks * 32 + 4 * g4, r_hi = r_lo + 16;
                Frag<TIn> bf[Cfg::MST];
#pragma unroll
                for (int m = 0; m < Cfg::MST; ++m) {
                    const int st = st0 + Cfg::WPT * m;
                    if (st < Cfg::NST) {
                        if constexpr (sizeof(TIn) == 2) {
                            const bf16x4 a = lds_col4(s_b, BS, r_lo, st * 16, lane);
                            const bf16x4 q = lds_col4(s_b, BS, r_hi, st * 16, lane);
                            bf[m].v = __builtin_shufflevector(a, q, 0, 1, 2, 3, 4, 5, 6, 7);
                        } else {
#pragma unroll
                            for (int v = 0; v < 8; ++v)
                                bf[m].v[v] = s_b[((v < 4 ? r_lo : r_hi) + (v & 3)) * BS + st * 16 + l16];
                        }
                    }
                }
                const f32x4 w_lo = *(const f32x4*)(bw + r_lo);
                const f32x4 w_hi = *(const f32x4*)(bw + r_hi);
                float xw[8];
                if constexpr (sizeof(TIn) == 2) {
                    const bf16x4 a = lds_col4(bx, XS, r_lo, pt * 16, lane);
                    const bf16x4 q = lds_col4(bx, XS, r_hi, pt * 16, lane);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        xw[v] = to_f32(a[v]) * w_lo[v];
                        xw[v + 4] = to_f32(q[v]) * w_hi[v];
                    }
                    Frag<bf16> hi, lo;
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        hi.v[v] = from_f32<bf16>(xw[v]);
                        lo.v[v] = from_f32<bf16>(xw[v] - to_f32(hi.v[v]));
                    }
#pragma unroll
                    for (int m = 0; m < Cfg::MST; ++m) {
                        if (st0 + Cfg::WPT * m < Cfg::NST) {
                            mma(acc[m], hi, bf[m]);
                            mma(acc[m], lo, bf[m]);
                        }
                    }
                } else {
                    Frag<float> a;
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const int r = (v < 4 ? r_lo : r_hi) + (v & 3);
                        a.v[v] = to_f32(bx[r * XS + pt * 16 + l16]) * (v < 4 ? w_lo[v & 3] : w_hi[v & 3]);
                    }
#pragma unroll
                    for (int m = 0; m < Cfg::MST; ++m)
                        if (st0 + Cfg::WPT * m < Cfg::NST) mma(acc[m], a, bf[m]);
                }
            }
            // dS[b, h, c, p, s]: element (row p = 16 pt + 4 g4 + r, column s) of tile m,
            // through a descriptor over this head's P x S block alone (a batch row's
            // increments may exceed what 32-bit offsets reach)
            const BufRsrc rds = make_rsrc(dS + (((size_t)b * H + h) * nC + c) * P * S,
                                          (uint32_t)(P * S * sizeof(float)));
#pragma unroll
            for (int m = 0; m < Cfg::MST; ++m) {
                const int st = st0 + Cfg::WPT * m;
                if (st < Cfg::NST) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        buf_store_f32(acc[m][r], rds,
                                      (uint32_t)(((pt * 16 + 4 * g4 + r) * S + st * 16 + l16) * 4), 0u);
                }
            }
        }
        if (hh + 1 < NH) store_head(h + 1, kb ^ 1);  // the other buffer is free
        __syncthreads();
    }
}

// Heads per workgroup: the largest divisor of the heads per group that still leaves one
// workgroup per CU on 256 CUs.
inline int state_heads_per_block(const Dims& d) {
    const int hpg = d.nheads / d.ngroups;
    const long units = (long)d.batch * d.nchunks() * d.nheads;
    int best = 1;
    for (int nh = 1; nh <= hpg; ++nh)
        if (hpg % nh == 0 && units / nh >= 256) best = nh;
    return best;
}

// Launches the multi-head kernel when its LDS plan fits; returns false (and launches
// nothing) otherwise.
template <typename TIn, int P, int S, int T>
bool run_state_mh(const void* x, const void* Bm, const float* A, const float* dt_t, float* dS,
                  const Dims& d, hipStream_t stream, hipError_t* err) {
    using Cfg = StateMhCfg<TIn, P, S, T>;
    if constexpr (!Cfg::FITS) {
        return false;
    } else {
        auto kern = chunk_state_mh_kernel<TIn, P, S, T>;
        if (Cfg::LDS_BYTES > 65536) {
            *err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)Cfg::LDS_BYTES);
            if (*err != hipSuccess) return true;
        }
        const int nh = state_heads_per_block(d);
        const int nblocks = d.batch * d.nchunks() * (d.nheads / nh);
        kern<<<nblocks, Cfg::NTHR, Cfg::LDS_BYTES, stream>>>((const TIn*)x, (const TIn*)Bm, A,
                                                            dt_t, dS, d.seqlen, d.nheads,
                                                            d.ngroups, nh);
        *err = hipGetLastError();
        return true;
    }
}

template <typename TIn, int P, int S>
bool state_mh_by_t(const void* x, const void* Bm, const float* A, const float* dt_t, float* dS,
                   const Dims& d, hipStream_t s, hipError_t* e) {
    switch (d.chunk) {
        case 64: return run_state_mh<TIn, P, S, 64>(x, Bm, A, dt_t, dS, d, s, e);
        case 128: return run_state_mh<TIn, P, S, 128>(x, Bm, A, dt_t, dS, d, s, e);
        case 256: return run_state_mh<TIn, P, S, 256>(x, Bm, A, dt_t, dS, d, s, e);
    }
    return false;
}

template <typename TIn, int P>
bool state_mh_by_s(const void* x, const void* Bm, const float* A, const float* dt_t, float* dS,
                   const Dims& d, hipStream_t s, hipError_t* e) {
    switch (d.dstate) {
        case 16: return state_mh_by_t<TIn, P, 16>(x, Bm, A, dt_t, dS, d, s, e);
        case 32: return state_mh_by_t<TIn, P, 32>(x, Bm, A, dt_t, dS, d, s, e);
        case 64: return state_mh_by_t<TIn, P, 64>(x, Bm, A, dt_t, dS, d, s, e);
        case 128: return state_mh_by_t<TIn, P, 128>(x, Bm, A, dt_t, dS, d, s, e);
        case 256: return state_mh_by_t<TIn, P, 256>(x, Bm, A, dt_t, dS, d, s, e);
    }
    return false;
}

template <typename TIn>
bool state_mh_by_p(const void* x, const void* Bm, const float* A, const float* dt_t, float* dS,
                   const Dims& d, hipStream_t s, hipError_t* e) {
    switch (d.headdim) {
        case 16: return state_mh_by_s<TIn, 16>(x, Bm, A, dt_t, dS, d, s, e);
        case 32: return state_mh_by_s<TIn, 32>(x, Bm, A, dt_t, dS, d, s, e);
        case 64: return state_mh_by_s<TIn, 64>(x, Bm, A, dt_t, dS, d, s, e);
        case 128: return state_mh_by_s<TIn, 128>(x, Bm, A, dt_t, dS, d, s, e);
    }
    return false;
}

}  // namespace ssd
