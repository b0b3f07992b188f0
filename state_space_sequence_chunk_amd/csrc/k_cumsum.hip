// Stage 1: per-chunk cumulative decay in base-2 log space.
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Kernel 1: Computing cumulative sums": for each chunk the kernel forms
// a = A[h] * dt[b,t,h], takes its inclusive running sum inside the chunk (restarting at
// every chunk) and multiplies by log2(e) so later stages can use exp2. The output goes
// to the head-major [batch, head, token] layout (section "Mamba-2 performance
// optimization", GMEM layout), together with dt itself widened to fp32 in that layout.
//
// gfx950 mapping. One 512-thread workgroup per (chunk, head block, batch). A head block
// is a run of up to 56 whole heads, so the workgroup's slice of dt is `chunk` row
// segments of head-block width (80 contiguous bytes for 40 bf16 heads). Each thread
// issues its 16-byte loads in unrolled batches of eight before using any of them, so a
// workgroup waits for about one HBM round trip rather than one per element. The slice is
// transposed through LDS to [head][token]; then each wave scans whole heads: a lane sums
// chunk/64 consecutive tokens serially and the 64 lane totals are combined with a DPP
// wave scan (row_shr + row_bcast). G and dt_t leave as one contiguous 16-, 8- or 4-byte
// store per lane, so each wave writes a full 1 KiB row segment per head.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kCumsumThreads = 512;
constexpr int kCumsumMaxHeads = 56;  // 56 * 257 * 4 B < 64 KiB of LDS at chunk 256

// Number of input elements one load brings in: 16 bytes when every head block's row
// segment is 16-byte aligned and a whole number of vectors, else one element.
template <typename TIn> constexpr int cumsum_vec() { return 16 / (int)sizeof(TIn); }

template <typename TIn, int VW>
__device__ __forceinline__ void unpack(const Vec16& v, float* out) {
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            out[2 * q] = __uint_as_float(v[q] << 16);
            out[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __uint_as_float(v[q]);
    }
}

template <typename TIn, int T, int VW>
__global__ __launch_bounds__(kCumsumThreads) void cumsum_kernel(
    const TIn* __restrict__ dt, const float* __restrict__ A, float* __restrict__ G,
    float* __restrict__ dt_t, int L, int H, int hb) {
    extern __shared__ float s_dt[];  // [hb][T + 1]
    constexpr int LD = T + 1;
    constexpr int PER = T / 64;  // tokens per lane in the scan
    constexpr int R = 8;         // loads in flight per thread
    const int c = blockIdx.x, b = blockIdx.z;
    const int h0 = blockIdx.y * hb;
    const int nh = min(hb, H - h0);
    const int t0 = c * T;
    const int rows = min(T, L - t0);  // real tokens; a partial last chunk is zero-padded
    const int groups = nh / VW;  // vectors per token row (nh % VW == 0 by the host plan)
    const int nvec = T * groups;
    const TIn* src = dt + ((size_t)b * L + t0) * H + h0;

    for (int base = threadIdx.x; base < nvec; base += R * kCumsumThreads) {
        if constexpr (VW > 1) {
            Vec16 v[R];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int e = base + k * kCumsumThreads;
                if (e < nvec) {
                    const int t = e / groups, gi = e - t * groups;
                    v[k] = t < rows ? *(const Vec16*)(src + (size_t)t * H + gi * VW)
                                    : Vec16{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int e = base + k * kCumsumThreads;
                if (e < nvec) {
                    const int t = e / groups, gi = e - t * groups;
                    float f[VW];
                    unpack<TIn, VW>(v[k], f);
#pragma unroll
                    for (int q = 0; q < VW; ++q) s_dt[(gi * VW + q) * LD + t] = f[q];
                }
            }
        } else {
            float v[R];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int e = base + k * kCumsumThreads;
                if (e < nvec) {
                    const int t = e / groups;
                    v[k] = t < rows ? to_f32(src[(size_t)t * H + (e - t * groups)]) : 0.f;
                }
            }
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int e = base + k * kCumsumThreads;
                if (e < nvec) {
                    const int t = e / groups;
                    s_dt[(e - t * groups) * LD + t] = v[k];
                }
            }
        }
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    for (int hh = wave; hh < nh; hh += kCumsumThreads / 64) {
        const int h = h0 + hh;
        float d[PER], g[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) d[k] = s_dt[hh * LD + lane * PER + k];
        chunk_log2_decay<PER>(d, A[h], g);
        const size_t o = ((size_t)b * H + h) * L + t0 + lane * PER;
        if (rows < T || (L & 3) != 0) {
            // partial chunk, or rows not 16-byte aligned: element stores of the real tokens
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                if (lane * PER + k < rows) {
                    G[o + k] = g[k];
                    if (dt_t) dt_t[o + k] = d[k];
                }
            }
        } else if constexpr (PER == 4) {
            *(float4*)(G + o) = make_float4(g[0], g[1], g[2], g[3]);
            if (dt_t) *(float4*)(dt_t + o) = make_float4(d[0], d[1], d[2], d[3]);
        } else if constexpr (PER == 2) {
            *(float2*)(G + o) = make_float2(g[0], g[1]);
            if (dt_t) *(float2*)(dt_t + o) = make_float2(d[0], d[1]);
        } else {
            G[o] = g[0];
            if (dt_t) dt_t[o] = d[0];
        }
    }
}

// Head-block plan: about four workgroups per CU (1024 in all) where the batch and chunk
// count alone do not give that many, whole vectors per row segment, and at most
// kCumsumMaxHeads heads per block.
struct CumsumPlan {
    int hb, nsplit, vw;
};

static CumsumPlan cumsum_plan(const Dims& d, int esize) {
    const int vmax = 16 / esize;
    const int vw = (d.nheads % vmax == 0) ? vmax : 1;
    const long long units = (long long)d.batch * d.nchunks();
    int want = (int)((1024 + units - 1) / units);
    want = std::max(1, std::min(want, d.nheads / vw));
    int hb = (d.nheads + want - 1) / want;
    hb = (hb + vw - 1) / vw * vw;
    hb = std::min(hb, kCumsumMaxHeads);
    return {hb, (d.nheads + hb - 1) / hb, vw};
}

template <typename TIn, int T>
static hipError_t launch_cumsum_t(const TIn* dt, const float* A, float* G, float* dt_t,
                                  const Dims& d, hipStream_t stream) {
    const CumsumPlan p = cumsum_plan(d, sizeof(TIn));
    const dim3 grid(d.nchunks(), p.nsplit, d.batch);
    const size_t lds = (size_t)p.hb * (T + 1) * sizeof(float);
    if (p.vw > 1)
        cumsum_kernel<TIn, T, cumsum_vec<TIn>()><<<grid, kCumsumThreads, lds, stream>>>(
            dt, A, G, dt_t, d.seqlen, d.nheads, p.hb);
    else
        cumsum_kernel<TIn, T, 1><<<grid, kCumsumThreads, lds, stream>>>(dt, A, G, dt_t,
                                                                         d.seqlen, d.nheads, p.hb);
    return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_cumsum_d(const void* dt, const float* A, float* G, float* dt_t,
                                  const Dims& d, hipStream_t stream) {
    const TIn* p = (const TIn*)dt;
    switch (d.chunk) {
        case 64: return launch_cumsum_t<TIn, 64>(p, A, G, dt_t, d, stream);
        case 128: return launch_cumsum_t<TIn, 128>(p, A, G, dt_t, d, stream);
        case 256: return launch_cumsum_t<TIn, 256>(p, A, G, dt_t, d, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cumsum(int in_dtype, const void* dt, const float* A, float* G, float* dt_t,
                         const Dims& d, hipStream_t stream) {
    if (in_dtype == kBF16) return launch_cumsum_d<bf16>(dt, A, G, dt_t, d, stream);
    return launch_cumsum_d<float>(dt, A, G, dt_t, d, stream);
}

}  // namespace ssd
