// Stage 2a: each chunk's own contribution to the state that leaves it (one workgroup per
// (batch, chunk, head); the multi-head form in chunk_state_mh.h is preferred when it fits).
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Mamba-2 architecture" (the log-space jump formula) and section
// "Kernel 2: fwd_pass_state" (operand fusion before the matrix product): the state
// after a chunk is 2^{G_last} times the state before it plus
//     dS_c[p][s] = sum_{j in chunk} (dt_j * 2^{G_last - G_j} * x_j[p]) * B_j[s],
// a P x S product with the chunk's tokens as the contraction index. This kernel
// computes dS_c for every (batch, chunk, head) in parallel; the short sequential
// carry across chunks is a separate streaming kernel (k_state_carry.hip). The page
// instead walks the chunks sequentially inside one program per state tile; splitting
// lets all matrix-core work run over batch*chunks*heads workgroups, which fills the
// 256 CUs even when batch*heads is small.
//
// gfx950 mapping: one 256-thread workgroup per (batch, chunk, head); tokens are
// staged 64 at a time in LDS (x rows and B rows, padded), with the next block's
// global loads in flight during the current block's MFMAs. The fused operand
// w_j x_j[p] is formed in fp32; for bf16 inputs it is split into a bf16 high part and
// a bf16 remainder, each multiplied by the exact bf16 B (two MFMAs), which keeps the
// product at ~16 significant bits instead of bf16's 8. fp32 inputs use fp32 MFMA.
// Slot (g, v) of a fragment carries token 16*(v/4) + 4*g + v%4 of the 32-token step:
// four consecutive rows per half, which is what one gfx950 transposing LDS read
// (ds_read_b64_tr_b16) delivers from the row-major tiles, so a bf16 fragment costs two
// LDS instructions instead of eight 2-byte reads.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kTK = 64;  // tokens per LDS block

template <typename TIn, int P, int S>
struct StateCfg {
    static constexpr int NPT = P / 16, NST = S / 16;
    static constexpr int WPP = NPT >= 4 ? 1 : 4 / NPT;                   // waves per p-tile
    static constexpr int MPT = NPT >= 4 ? NPT / 4 : 1;                   // p-tiles per wave
    static constexpr int MST = NPT >= 4 ? NST : (NST + WPP - 1) / WPP;   // s-tiles per wave
    static constexpr int VE = 16 / (int)sizeof(TIn);                     // elements per 16 B
    static constexpr int XS = col_stride<TIn>(P), BS = col_stride<TIn>(S);  // LDS row strides
    static constexpr int XVEC = kTK * P / VE, BVEC = kTK * S / VE;
    static constexpr int XPT = (XVEC + 255) / 256, BPT = (BVEC + 255) / 256;
};

template <typename TIn, int P, int S>
__global__ __launch_bounds__(256) void chunk_state_kernel(const TIn* __restrict__ x,
                                                          const TIn* __restrict__ Bm,
                                                          const float* __restrict__ A,
                                                          const float* __restrict__ dt_t,
                                                          float* __restrict__ dS, int L, int H,
                                                          int ngroups, int T) {
    using Cfg = StateCfg<TIn, P, S>;
    __shared__ __attribute__((aligned(16))) float s_w[256];
    __shared__ __attribute__((aligned(16))) TIn s_x[kTK * Cfg::XS];
    __shared__ __attribute__((aligned(16))) TIn s_b[kTK * Cfg::BS];

    const int nC = (L + T - 1) / T;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int h = id % H;
    const int c = (id / H) % nC;
    const int b = id / (H * nC);
    const int g = h / (H / ngroups);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int g4 = lane >> 4, l16 = lane & 15;
    const int t0 = c * T;
    const int rows = min(T, L - t0);  // real tokens of this chunk; the rest count as zeros
    const size_t bh = (size_t)b * H + h;

    // w_j = dt_j * 2^{log2(e) * sum_{k=j+1}^{T-1} A dt_k}: the decay from token j to the end
    // of the chunk (the page's G_last - G_j). It is summed from the chunk's end backwards
    // (thread tid holds token T-1-tid), so its rounding error is relative to the small
    // exponents that dominate the state rather than to the chunk's whole cumulative decay.
    {
        __shared__ float s_tot[4];
        const float* dc = dt_t + bh * L + t0;
        const float ah = A[h];
        const int t = T - 1 - tid;
        const float dtv = tid < T && t < rows ? dc[t] : 0.f;
        const float a = ah * dtv;
        const float incl = wave_inclusive_scan(a);
        const float excl = wave_shift_up1(incl);
        if (lane == 63) s_tot[wave] = incl;
        __syncthreads();
        float off = 0.f;
        for (int w2 = 0; w2 < wave; ++w2) off += s_tot[w2];
        if (tid < T) s_w[t] = dtv * exp2_fast((off + excl) * kLog2e);
    }

    const TIn* xg = x + (((size_t)b * L + t0) * H + h) * P;
    const TIn* bg = Bm + (((size_t)b * L + t0) * ngroups + g) * S;
    const size_t xrow = (size_t)H * P, brow = (size_t)ngroups * S;

    Vec16 xr[Cfg::XPT], br[Cfg::BPT];
#define SSD_GLOAD(kb)                                                                     \
    {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < Cfg::XPT; ++i) {                            \
            const int v = tid + i * 256;                                                  \
            if (v < Cfg::XVEC) {                                                          \
                const int r = v / (P / Cfg::VE), col = (v % (P / Cfg::VE)) * Cfg::VE;     \
                const int tr = (kb) * kTK + r;                                            \
                xr[i] = tr < rows ? *(const Vec16*)(xg + (size_t)tr * xrow + col)         \
                                  : Vec16{0u, 0u, 0u, 0u};                                \
            }                                                                             \
        }                                                                                 \
        _Pragma("unroll") for (int i = 0; i < Cfg::BPT; ++i) {                            \
            const int v = tid + i * 256;                                                  \
            if (v < Cfg::BVEC) {                                                          \
                const int r = v / (S / Cfg::VE), col = (v % (S / Cfg::VE)) * Cfg::VE;     \
                const int tr = (kb) * kTK + r;                                            \
                br[i] = tr < rows ? *(const Vec16*)(bg + (size_t)tr * brow + col)         \
                                  : Vec16{0u, 0u, 0u, 0u};                                \
            }                                                                             \
        }                                                                                 \
    }

    const int pt_w = Cfg::NPT >= 4 ? wave : wave / Cfg::WPP;   // first p-tile of this wave
    const int pt_step = 4;                                     // p-tile stride when NPT >= 4
    const int st_w = Cfg::NPT >= 4 ? 0 : wave % Cfg::WPP;      // first s-tile of this wave
    const int st_step = Cfg::NPT >= 4 ? 1 : Cfg::WPP;          // s-tile stride

    f32x4 acc[Cfg::MPT][Cfg::MST];
#pragma unroll
    for (int n = 0; n < Cfg::MPT; ++n)
#pragma unroll
        for (int m = 0; m < Cfg::MST; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nKB = T / kTK;
    SSD_GLOAD(0)
    for (int kb = 0; kb < nKB; ++kb) {
        __syncthreads();  // previous block's LDS reads are done (and s_w is visible)
#pragma unroll
        for (int i = 0; i < Cfg::XPT; ++i) {
            const int v = tid + i * 256;
            if (v < Cfg::XVEC) {
                const int r = v / (P / Cfg::VE), col = (v % (P / Cfg::VE)) * Cfg::VE;
                *(Vec16*)(s_x + r * Cfg::XS + col) = xr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::BPT; ++i) {
            const int v = tid + i * 256;
            if (v < Cfg::BVEC) {
                const int r = v / (S / Cfg::VE), col = (v % (S / Cfg::VE)) * Cfg::VE;
                *(Vec16*)(s_b + r * Cfg::BS + col) = br[i];
            }
        }
        __syncthreads();
        if (kb + 1 < nKB) SSD_GLOAD(kb + 1)
#pragma unroll
        for (int ks = 0; ks < kTK / 32; ++ks) {
            const int r_lo = ks * 32 + 4 * g4, r_hi = r_lo + 16;  // rows of items 0-3, 4-7
            Frag<TIn> bf[Cfg::MST];
#pragma unroll
            for (int m = 0; m < Cfg::MST; ++m) {
                const int st = st_w + st_step * m;
                if (st < Cfg::NST) {
                    if constexpr (sizeof(TIn) == 2) {
                        const bf16x4 a = lds_col4(s_b, Cfg::BS, r_lo, st * 16, lane);
                        const bf16x4 c = lds_col4(s_b, Cfg::BS, r_hi, st * 16, lane);
                        bf[m].v = __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
                    } else {
#pragma unroll
                        for (int v = 0; v < 8; ++v)
                            bf[m].v[v] = s_b[((v < 4 ? r_lo : r_hi) + (v & 3)) * Cfg::BS +
                                             st * 16 + l16];
                    }
                }
            }
            const f32x4 w_lo = *(const f32x4*)(s_w + kb * kTK + r_lo);
            const f32x4 w_hi = *(const f32x4*)(s_w + kb * kTK + r_hi);
#pragma unroll
            for (int n = 0; n < Cfg::MPT; ++n) {
                const int pt = pt_w + pt_step * n;
                float xw[8];
                if constexpr (sizeof(TIn) == 2) {
                    const bf16x4 a = lds_col4(s_x, Cfg::XS, r_lo, pt * 16, lane);
                    const bf16x4 c = lds_col4(s_x, Cfg::XS, r_hi, pt * 16, lane);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        xw[v] = to_f32(a[v]) * w_lo[v];
                        xw[v + 4] = to_f32(c[v]) * w_hi[v];
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const int r = (v < 4 ? r_lo : r_hi) + (v & 3);
                        xw[v] = to_f32(s_x[r * Cfg::XS + pt * 16 + l16]) *
                                (v < 4 ? w_lo[v & 3] : w_hi[v & 3]);
                    }
                }
                if constexpr (sizeof(TIn) == 2) {
                    Frag<bf16> hi, lo;
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        hi.v[v] = from_f32<bf16>(xw[v]);
                        lo.v[v] = from_f32<bf16>(xw[v] - to_f32(hi.v[v]));
                    }
#pragma unroll
                    for (int m = 0; m < Cfg::MST; ++m) {
                        if (st_w + st_step * m < Cfg::NST) {
                            mma(acc[n][m], hi, bf[m]);
                            mma(acc[n][m], lo, bf[m]);
                        }
                    }
                } else {
                    Frag<float> a;
#pragma unroll
                    for (int v = 0; v < 8; ++v) a.v[v] = xw[v];
#pragma unroll
                    for (int m = 0; m < Cfg::MST; ++m)
                        if (st_w + st_step * m < Cfg::NST) mma(acc[n][m], a, bf[m]);
                }
            }
        }
    }
#undef SSD_GLOAD

    float* out = dS + (bh * nC + c) * (size_t)(P * S);
#pragma unroll
    for (int n = 0; n < Cfg::MPT; ++n) {
        const int pt = pt_w + pt_step * n;
#pragma unroll
        for (int m = 0; m < Cfg::MST; ++m) {
            const int st = st_w + st_step * m;
            if (st < Cfg::NST) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    out[(pt * 16 + 4 * g4 + r) * S + st * 16 + l16] = acc[n][m][r];
            }
        }
    }
}

template <typename TIn, int P, int S>
static hipError_t run_state(const void* x, const void* Bm, const float* A, const float* dt_t,
                            float* dS, const Dims& d, hipStream_t stream) {
    const int nblocks = d.batch * d.nchunks() * d.nheads;
    chunk_state_kernel<TIn, P, S><<<nblocks, 256, 0, stream>>>(
        (const TIn*)x, (const TIn*)Bm, A, dt_t, dS, d.seqlen, d.nheads, d.ngroups, d.chunk);
    return hipGetLastError();
}

template <typename TIn, int P>
static hipError_t state_by_s(const void* x, const void* Bm, const float* A, const float* dt_t,
                             float* dS, const Dims& d, hipStream_t st) {
    switch (d.dstate) {
        case 16: return run_state<TIn, P, 16>(x, Bm, A, dt_t, dS, d, st);
        case 32: return run_state<TIn, P, 32>(x, Bm, A, dt_t, dS, d, st);
        case 64: return run_state<TIn, P, 64>(x, Bm, A, dt_t, dS, d, st);
        case 128: return run_state<TIn, P, 128>(x, Bm, A, dt_t, dS, d, st);
        case 256: return run_state<TIn, P, 256>(x, Bm, A, dt_t, dS, d, st);
    }
    return hipErrorInvalidValue;
}

template <typename TIn>
static hipError_t state_by_p(const void* x, const void* Bm, const float* A, const float* dt_t,
                             float* dS, const Dims& d, hipStream_t st) {
    switch (d.headdim) {
        case 16: return state_by_s<TIn, 16>(x, Bm, A, dt_t, dS, d, st);
        case 32: return state_by_s<TIn, 32>(x, Bm, A, dt_t, dS, d, st);
        case 64: return state_by_s<TIn, 64>(x, Bm, A, dt_t, dS, d, st);
        case 128: return state_by_s<TIn, 128>(x, Bm, A, dt_t, dS, d, st);
    }
    return hipErrorInvalidValue;
}

bool launch_chunk_state_mh_bf16(const void*, const void*, const float*, const float*, float*,
                                const Dims&, hipStream_t, hipError_t*);
bool launch_chunk_state_mh_f32(const void*, const void*, const float*, const float*, float*,
                               const Dims&, hipStream_t, hipError_t*);

// The multi-head form (B rows staged once per workgroup, x double-buffered per head) is
// used whenever its LDS plan fits; otherwise one workgroup per (batch, chunk, head).
hipError_t launch_chunk_state(int in_dtype, const void* x, const void* Bm, const float* A,
                              const float* dt_t, float* dS, const Dims& d, hipStream_t stream) {
    hipError_t err = hipSuccess;
    if (in_dtype == kBF16) {
        if (launch_chunk_state_mh_bf16(x, Bm, A, dt_t, dS, d, stream, &err)) return err;
        return state_by_p<bf16>(x, Bm, A, dt_t, dS, d, stream);
    }
    if (launch_chunk_state_mh_f32(x, Bm, A, dt_t, dS, d, stream, &err)) return err;
    return state_by_p<float>(x, Bm, A, dt_t, dS, d, stream);
}

}  // namespace ssd
