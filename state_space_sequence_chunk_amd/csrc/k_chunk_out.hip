// Stage 3: fused per-chunk output.
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Mamba-2 architecture" (the decayed chunk-output formula) and section
// "Kernel 3: compute_out". For chunk c, token rows i and columns j of the chunk:
//     y_i = 2^{G_i} C_i . S_c  +  sum_{j <= i} 2^{G_i - G_j} (C_i . B_j) dt_j x_j  +  D x_i
// where S_c is the chunk-initial state. The interaction C B^T, its decay and the causal
// mask exist only in registers; decays of masked (j > i) pairs are removed by selection,
// never by multiplying, so an overflowing 2^{positive} cannot reach y.
//
// gfx950 mapping: one workgroup of chunk/32 waves per (batch, chunk, head). The chunk's
// x rows are staged once in LDS (padded rows) for the W x product and the skip term.
// Wave w owns the 16-row tiles w and (chunk/16 - 1 - w), which balances the causal
// triangle. Per row tile it:
//   1. multiplies C_i (held in registers for the whole kernel) by the chunk-initial
//      state (K = dstate) and scales each row by 2^{G_i};
//   2. for every pair of 16-column tiles (j <= i), forms S^T = B_j C_i^T on the matrix
//      core (K = dstate). In the accumulator layout each lane then holds one row i and
//      four j's per tile, exactly the A-operand layout of the next product, so the decay,
//      dt_j and the mask are applied in registers and the tile is rounded once to the
//      input dtype and fed straight into y += W x (K = 32 tokens) with no LDS round trip;
//   3. adds D x_i and writes y in fp32.
// B_j rows are read from global memory (they are shared by every head of the group and
// stay in L2). The page's matrix-core operand swap for Blackwell does not apply: gfx950
// MFMA takes both operands from VGPRs.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kOutPad = 16;  // LDS row padding (elements)

// 8 consecutive elements of a row into a fragment (zeros when !valid).
__device__ __forceinline__ void load8(Frag<bf16>& f, const bf16* p, bool valid) {
    if (valid) f.v = *(const bf16x8*)p;
    else f.v = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
}
__device__ __forceinline__ void load8(Frag<float>& f, const float* p, bool valid) {
    if (valid) {
        const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
        f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        f.v = f32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
}

// State fragment in the input's MFMA type. A bf16 product with fp32 states splits each
// value into bf16 high and low parts (two products).
template <typename TIn, typename TS> struct StateFrag {
    static constexpr bool kSplit = false;
    Frag<TIn> hi, lo;
    __device__ __forceinline__ void load(const TS* p, bool valid) {
        if constexpr (sizeof(TIn) == sizeof(TS)) {
            load8(hi, (const TIn*)p, valid);
        } else {  // fp32 product, bf16 states: widen exactly
            Frag<bf16> t;
            load8(t, (const bf16*)p, valid);
#pragma unroll
            for (int v = 0; v < 8; ++v) hi.v[v] = to_f32(t.v[v]);
        }
    }
};
template <> struct StateFrag<bf16, float> {
    static constexpr bool kSplit = true;
    Frag<bf16> hi, lo;
    __device__ __forceinline__ void load(const float* p, bool valid) {
        Frag<float> t;
        load8(t, p, valid);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            hi.v[v] = (bf16)t.v[v];
            lo.v[v] = (bf16)(t.v[v] - to_f32(hi.v[v]));
        }
    }
};

template <typename TIn, typename TS, int P, int S>
__global__ __launch_bounds__(512) void chunk_out_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ Bm, const TIn* __restrict__ Cm,
    const float* __restrict__ G, const float* __restrict__ dt_t, const TS* __restrict__ states,
    const float* __restrict__ Dv, float* __restrict__ y, int L, int H, int ngroups, int T) {
    constexpr int NPT = P / 16;
    constexpr int NKS = (S + 31) / 32;  // K = dstate steps of 32 (S = 16 pads with zeros)
    constexpr int XS = P + kOutPad;
    constexpr int VE = 16 / (int)sizeof(TIn);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    TIn* s_x = (TIn*)smem;                                    // [T][XS]
    float* s_g = (float*)(smem + (size_t)T * XS * sizeof(TIn));  // [T]
    float* s_dt = s_g + T;                                     // [T]

    const int nC = L / T;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int h = id % H;
    const int c = (id / H) % nC;
    const int b = id / (H * nC);
    const int g = h / (H / ngroups);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int NW = T / 32;
    const int nthr = 2 * T;
    const int t0 = c * T;
    const size_t bh = (size_t)b * H + h;

    {  // stage x rows, G and dt of this chunk
        const TIn* xg = x + (((size_t)b * L + t0) * H + h) * P;
        const size_t xrow = (size_t)H * P;
        constexpr int VPR = P / VE;
        for (int v = tid; v < T * VPR; v += nthr) {
            const int r = v / VPR, col = (v % VPR) * VE;
            *(Vec16*)(s_x + r * XS + col) = *(const Vec16*)(xg + r * xrow + col);
        }
        for (int t = tid; t < T; t += nthr) {
            s_g[t] = G[bh * L + t0 + t];
            s_dt[t] = dt_t[bh * L + t0 + t];
        }
    }

    const int its[2] = {wave, 2 * NW - 1 - wave};
    const size_t grow = (size_t)ngroups * S;
    const TIn* cg = Cm + (((size_t)b * L + t0) * ngroups + g) * S;
    const TIn* bg = Bm + (((size_t)b * L + t0) * ngroups + g) * S;

    // C rows of both row tiles, K = dstate, kept in registers.
    Frag<TIn> cf[2][NKS];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int s0 = ks * 32 + g4 * 8;
            load8(cf[q][ks], cg + (size_t)(its[q] * 16 + l16) * grow + s0, s0 < S);
        }

    f32x4 yacc[2][NPT];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) yacc[q][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // 1. carried state: C_i . S_c (rows i, columns p), K = dstate
    const TS* sp = states + (bh * nC + c) * (size_t)(P * S);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int s0 = ks * 32 + g4 * 8;
            StateFrag<TIn, TS> hf;
            hf.load(sp + (size_t)(pt * 16 + l16) * S + s0, s0 < S);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                mma(yacc[q][pt], cf[q][ks], hf.hi);
                if constexpr (StateFrag<TIn, TS>::kSplit) mma(yacc[q][pt], cf[q][ks], hf.lo);
            }
        }
    }

    __syncthreads();  // s_x, s_g, s_dt are ready

#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = exp2_fast(s_g[its[q] * 16 + 4 * g4 + r]);
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) yacc[q][pt][r] *= sc;
        }

    // 2. within-chunk term, two 16-column tiles (32 tokens) per step
    const int itmax = its[1];
    for (int kp = 0; 2 * kp <= itmax; ++kp) {
        Frag<TIn> bfj[2][NKS];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int jt = 2 * kp + jj;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int s0 = ks * 32 + g4 * 8;
                load8(bfj[jj][ks], bg + (size_t)(jt * 16 + l16) * grow + s0,
                      s0 < S && jt <= itmax);
            }
        }
        // x fragments: slot (g4, v) carries token j = 32kp + 16(v/4) + 4 g4 + v%4
        Frag<TIn> xf[NPT];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const int j = 32 * kp + 16 * (v >> 2) + 4 * g4 + (v & 3);
                xf[pt].v[v] = s_x[j * XS + pt * 16 + l16];
            }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int it = its[q];
            if (it < 2 * kp) continue;
            const int i = it * 16 + l16;
            const float gi = s_g[i];
            float wv[8];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int jt = 2 * kp + jj;
                f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
                if (jt <= it) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) mma(st, bfj[jj][ks], cf[q][ks]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jt * 16 + 4 * g4 + r;
                    const float e = exp2_fast(gi - s_g[j]) * s_dt[j];
                    wv[jj * 4 + r] = (i >= j) ? st[r] * e : 0.f;
                }
            }
            Frag<TIn> wf;
#pragma unroll
            for (int v = 0; v < 8; ++v) wf.v[v] = from_f32<TIn>(wv[v]);
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) mma(yacc[q][pt], wf, xf[pt]);
        }
    }

    // 3. skip term and store
    const float dh = Dv ? Dv[h] : 0.f;
    float* yb = y + (((size_t)b * L + t0) * H + h) * P;
    const size_t yrow = (size_t)H * P;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = its[q] * 16 + 4 * g4 + r;
                const int p = pt * 16 + l16;
                yb[(size_t)i * yrow + p] = yacc[q][pt][r] + dh * to_f32(s_x[i * XS + p]);
            }
}

template <typename TIn, typename TS, int P, int S>
static hipError_t run_out(const void* x, const void* Bm, const void* Cm, const float* G,
                          const float* dt_t, const void* states, const float* D, float* y,
                          const Dims& d, hipStream_t stream) {
    const int T = d.chunk;
    const size_t smem = (size_t)T * (P + kOutPad) * sizeof(TIn) + 2 * (size_t)T * sizeof(float);
    auto kern = chunk_out_kernel<TIn, TS, P, S>;
    if (smem > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    const int nblocks = d.batch * d.nchunks() * d.nheads;
    kern<<<nblocks, 2 * T, smem, stream>>>((const TIn*)x, (const TIn*)Bm, (const TIn*)Cm, G,
                                           dt_t, (const TS*)states, D, y, d.seqlen, d.nheads,
                                           d.ngroups, T);
    return hipGetLastError();
}

template <typename TIn, typename TS, int P>
static hipError_t out_by_s(const void* x, const void* Bm, const void* Cm, const float* G,
                           const float* dt_t, const void* st, const float* D, float* y,
                           const Dims& d, hipStream_t s) {
    switch (d.dstate) {
        case 16: return run_out<TIn, TS, P, 16>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 32: return run_out<TIn, TS, P, 32>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 64: return run_out<TIn, TS, P, 64>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 128: return run_out<TIn, TS, P, 128>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 256: return run_out<TIn, TS, P, 256>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
    }
    return hipErrorInvalidValue;
}

template <typename TIn, typename TS>
static hipError_t out_by_p(const void* x, const void* Bm, const void* Cm, const float* G,
                           const float* dt_t, const void* st, const float* D, float* y,
                           const Dims& d, hipStream_t s) {
    switch (d.headdim) {
        case 16: return out_by_s<TIn, TS, 16>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 32: return out_by_s<TIn, TS, 32>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 64: return out_by_s<TIn, TS, 64>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 128: return out_by_s<TIn, TS, 128>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_out(int in_dtype, int states_dtype, const void* x, const void* Bm,
                            const void* Cm, const float* G, const float* dt_t, const void* states,
                            const float* D, float* y, const Dims& d, hipStream_t s) {
    if (in_dtype == kBF16) {
        if (states_dtype == kBF16) return out_by_p<bf16, bf16>(x, Bm, Cm, G, dt_t, states, D, y, d, s);
        return out_by_p<bf16, float>(x, Bm, Cm, G, dt_t, states, D, y, d, s);
    }
    if (states_dtype == kBF16) return out_by_p<float, bf16>(x, Bm, Cm, G, dt_t, states, D, y, d, s);
    return out_by_p<float, float>(x, Bm, Cm, G, dt_t, states, D, y, d, s);
}

}  // namespace ssd
