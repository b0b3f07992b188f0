// Recurrent decode step: one token of the recurrence on a carried state.
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Mamba-2 architecture": the recurrent form updates a fixed-size state per
// token, which is what makes the model cheap for sequential inference; for batch b,
// head h (group g = h / (H/G)):
//     state[p][s] <- exp(A_h dt) state[p][s] + dt x[p] B[s]
//     y[p]         = sum_s state[p][s] C[s] + D_h x[p]          (y reads the new state)
// The state is the fp32 [P][S] state that the chunked forward pass returns as its final
// state, so a prefill by ssd_forward continues token by token here.
//
// gfx950 mapping: the step is a read-modify-write of the state (8 bytes of HBM traffic per
// element against 4 flops); at decode sizes (a few MB) its time is mostly the latency of
// one round trip to memory. Each 256-thread workgroup owns a contiguous slice of one
// (batch, head) state of up to 256 x ROWS x 4 floats; a thread owns 4 consecutive state
// columns (one 16-byte load and store) of up to ROWS rows, and issues all its rows' loads
// before using any. The S/4 threads that share a row are adjacent lanes of one wave, so y's
// sum over s is a butterfly over those lanes (no LDS, no barrier). ROWS is 2, or 1 where
// two rows per thread would leave fewer workgroups than compute units (measured on the
// 2.7B layer's 160 states: 3.9 us with 2 rows, 4.0 with 1; on the article's 32 states:
// 2.7 us with 2 rows, 2.4 with 1).
#include <algorithm>
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kDecodeThreads = 256;

template <typename TIn, int S, int ROWS>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ dt, const float* __restrict__ A,
    const TIn* __restrict__ Bm, const TIn* __restrict__ Cm, const float* __restrict__ Dv,
    float* __restrict__ state, float* __restrict__ y, int H, int P, int ngroups, int vpw) {
    constexpr int RL = S / 4;  // lanes per state row
    const int per_bh = P * RL / vpw;
    const int bh = blockIdx.x / per_bh;
    const int v0 = (blockIdx.x % per_bh) * vpw;
    const int b = bh / H, h = bh % H;
    const int g = h / (H / ngroups);
    const float dtv = to_f32(dt[bh]);
    const float decay = exp2_fast(A[h] * dtv * kLog2e);
    const float dval = Dv ? Dv[h] : 0.f;
    const TIn* xr = x + (size_t)bh * P;
    const TIn* br = Bm + ((size_t)b * ngroups + g) * S;
    const TIn* cr = Cm + ((size_t)b * ngroups + g) * S;
    float* st = state + (size_t)bh * P * S;

    const int lane_s = (threadIdx.x % RL) * 4;  // first state column of this thread
    float bs[4], cs[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bs[k] = to_f32(br[lane_s + k]);
        cs[k] = to_f32(cr[lane_s + k]);
    }
    // vpw is a multiple of 64, so each wave is either wholly inside or wholly outside
    // the slice for a given j (the row butterfly below needs its whole lane group)
    f32x4 sv[ROWS];
    float xv[ROWS];
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        const int t = threadIdx.x + kDecodeThreads * j;
        if (t < vpw) {
            sv[j] = *(const f32x4*)(st + (size_t)(v0 + t) * 4);
            xv[j] = to_f32(xr[(v0 + t) / RL]);
        }
    }
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        const int t = threadIdx.x + kDecodeThreads * j;
        if (t < vpw) {
            const int v = v0 + t, p = v / RL;
            const float u = dtv * xv[j];
            f32x4 s = sv[j];
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                s[k] = decay * s[k] + u * bs[k];
                part += s[k] * cs[k];
            }
            *(f32x4*)(st + (size_t)v * 4) = s;
            // sum over the RL lanes of this row (aligned groups within one wave)
#pragma unroll
            for (int off = RL / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, RL);
            if (threadIdx.x % RL == 0) y[(size_t)bh * P + p] = part + dval * xv[j];
        }
    }
}

template <typename TIn>
static hipError_t decode_by_s(const void* x, const void* dt, const float* A, const void* Bm,
                              const void* Cm, const float* D, float* state, float* y,
                              const Dims& d, hipStream_t stream) {
    const int vecs = d.headdim * d.dstate / 4;  // per (batch, head)
    // two rows per thread unless that leaves fewer workgroups than compute units
    const int rows = (long)d.batch * d.nheads * vecs / (2 * kDecodeThreads) >= 256 ? 2 : 1;
    const int vpw = std::min(vecs, rows * kDecodeThreads);
    const int nblocks = d.batch * d.nheads * (vecs / vpw);
    auto go = [&](auto kern) {
        kern<<<nblocks, kDecodeThreads, 0, stream>>>((const TIn*)x, (const TIn*)dt, A,
                                                     (const TIn*)Bm, (const TIn*)Cm, D, state, y,
                                                     d.nheads, d.headdim, d.ngroups, vpw);
        return hipGetLastError();
    };
    auto by_s = [&](auto rows_c) -> hipError_t {
        constexpr int R = decltype(rows_c)::value;
        switch (d.dstate) {
            case 16: return go(decode_kernel<TIn, 16, R>);
            case 32: return go(decode_kernel<TIn, 32, R>);
            case 64: return go(decode_kernel<TIn, 64, R>);
            case 128: return go(decode_kernel<TIn, 128, R>);
            case 256: return go(decode_kernel<TIn, 256, R>);
        }
        return hipErrorInvalidValue;
    };
    return rows == 2 ? by_s(std::integral_constant<int, 2>{}) : by_s(std::integral_constant<int, 1>{});
}

hipError_t launch_decode(int in_dtype, const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* D, float* state, float* y,
                         const Dims& d, hipStream_t stream) {
    if (in_dtype == kBF16) return decode_by_s<bf16>(x, dt, A, Bm, Cm, D, state, y, d, stream);
    return decode_by_s<float>(x, dt, A, Bm, Cm, D, state, y, d, stream);
}

}  // namespace ssd
