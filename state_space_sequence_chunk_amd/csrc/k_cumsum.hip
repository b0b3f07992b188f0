// Stage 1: per-chunk cumulative decay in base-2 log space.
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Kernel 1: Computing cumulative sums": for each chunk the kernel forms
// a = A[h] * dt[b,t,h], takes its inclusive running sum inside the chunk (restarting at
// every chunk) and multiplies by log2(e) so later stages can use exp2. The output goes
// to the head-major [batch, head, token] layout (section "Mamba-2 performance
// optimization", GMEM layout), together with dt itself widened to fp32 in that layout.
//
// gfx950 mapping: one 256-thread workgroup per (chunk, 16-head tile, batch). The dt
// tile is staged through LDS transposed to [head][token]; then one wave scans one head
// at a time: each lane sums chunk/64 consecutive tokens serially and the 64 lane totals
// are combined with a DPP wave scan (row_shr + row_bcast), with no LDS round trip.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kCumsumHeads = 16;

template <typename TIn>
__global__ __launch_bounds__(256) void cumsum_kernel(const TIn* __restrict__ dt,
                                                     const float* __restrict__ A,
                                                     float* __restrict__ G,
                                                     float* __restrict__ dt_t, int L, int H,
                                                     int T) {
    __shared__ float s_dt[kCumsumHeads][256 + 1];
    const int c = blockIdx.x;
    const int h_base = blockIdx.y * kCumsumHeads;
    const int b = blockIdx.z;
    const int nh = min(kCumsumHeads, H - h_base);
    const int t0 = c * T;

    for (int e = threadIdx.x; e < T * kCumsumHeads; e += 256) {
        const int t = e / kCumsumHeads, hh = e % kCumsumHeads;
        float v = 0.f;
        if (hh < nh) v = to_f32(dt[((size_t)b * L + t0 + t) * H + h_base + hh]);
        s_dt[hh][t] = v;
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int per = T / 64;  // 1, 2 or 4 tokens per lane
    for (int hh = wave; hh < nh; hh += 4) {
        const int h = h_base + hh;
        const float ah = A[h];
        float part[4];
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < per) {
                run += ah * s_dt[hh][lane * per + k];
                part[k] = run;
            }
        }
        const float incl = wave_inclusive_scan(run);
        // exclusive prefix = inclusive prefix of the previous lane (DPP wave_shr:1)
        const float excl = wave_shift_up1(incl);
        const size_t base = ((size_t)b * H + h) * L + t0 + lane * per;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < per) {
                G[base + k] = (excl + part[k]) * kLog2e;
                if (dt_t) dt_t[base + k] = s_dt[hh][lane * per + k];
            }
        }
    }
}

hipError_t launch_cumsum(int in_dtype, const void* dt, const float* A, float* G, float* dt_t,
                         const Dims& d, hipStream_t stream) {
    dim3 grid(d.nchunks(), (d.nheads + kCumsumHeads - 1) / kCumsumHeads, d.batch);
    if (in_dtype == kBF16)
        cumsum_kernel<bf16><<<grid, 256, 0, stream>>>((const bf16*)dt, A, G, dt_t, d.seqlen,
                                                      d.nheads, d.chunk);
    else
        cumsum_kernel<float><<<grid, 256, 0, stream>>>((const float*)dt, A, G, dt_t, d.seqlen,
                                                       d.nheads, d.chunk);
    return hipGetLastError();
}

}  // namespace ssd
