// HBM stream probes (declared in include/ssd_probe.h): grid-stride read, write, copy and
// mixed read/write kernels of 16-byte vectors, each thread keeping UNR of them in flight per iteration, so
// that the measured rate is the DRAM's rather than a latency limit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssd_probe.h"

namespace {

typedef uint32_t V4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

template <bool NT>
__device__ __forceinline__ V4 ld(const V4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(V4* p, V4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Vector i of iteration k of workgroup w: the UNR vectors of one thread are kThreads apart,
// so each load instruction of a wave covers 1 KB of consecutive bytes.
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const V4* __restrict__ src, size_t n,
                                                            V4* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
    V4 acc = {0u, 0u, 0u, 0u};
    size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
    for (; base + (kUnroll - 1) * kThreads < n; base += stride) {
        V4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = ld<NT>(src + base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (int u = 0; u < kUnroll; ++u)  // the ragged end of the buffer
        if (base + u * kThreads < n) acc ^= ld<NT>(src + base + u * kThreads);
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == acc[3]) *sink = acc;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_write_kernel(V4* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
    const V4 v = {0x3f800000u, 0u, 0x3f800000u, 0u};
    size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
    for (; base + (kUnroll - 1) * kThreads < n; base += stride) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) st<NT>(dst + base + u * kThreads, v);
    }
    for (int u = 0; u < kUnroll; ++u)
        if (base + u * kThreads < n) st<NT>(dst + base + u * kThreads, v);
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const V4* __restrict__ src,
                                                            V4* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
    size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
    for (; base + (kUnroll - 1) * kThreads < n; base += stride) {
        V4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = ld<NT>(src + base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) st<NT>(dst + base + u * kThreads, v[u]);
    }
    for (int u = 0; u < kUnroll; ++u)
        if (base + u * kThreads < n) st<NT>(dst + base + u * kThreads, ld<NT>(src + base + u * kThreads));
}

// Reads nr vectors and writes nw in one pass: index i of n = max(nr, nw) reads vector
// i * nr / n and writes vector i * nw / n (each vector of the shorter buffer is touched by
// one or more consecutive indices, so the loads and stores stay in the same proportion all
// along the run). The written value depends on the loaded one, so no load can be dropped.
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_mix_kernel(const V4* __restrict__ src, size_t nr,
                                                           V4* __restrict__ dst, size_t nw,
                                                           size_t n) {
    const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
    const V4 k = {0x3f800000u, 0u, 0x3f800000u, 0u};
    for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n;
         base += stride) {
        V4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + u * kThreads;
            v[u] = (i < n && nr) ? ld<NT>(src + i * nr / n) : k;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + u * kThreads;
            if (i < n && nw) st<NT>(dst + i * nw / n, v[u] ^ k);
        }
    }
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

ssd_status check(size_t bytes, int mode, int workgroups) {
    if (bytes == 0 || bytes % 16 != 0 || workgroups < 0) return SSD_ERR_SHAPE;
    if (mode != 0 && mode != 1) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

unsigned grid_of(size_t n, int workgroups) {
    if (workgroups > 0) return (unsigned)workgroups;
    const size_t per = (size_t)kThreads * kUnroll;
    const size_t need = (n + per - 1) / per;
    return (unsigned)(need < 2048 ? need : 2048);  // 8 per compute unit
}

ssd_status done() { return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

}  // namespace

extern "C" {

ssd_status ssd_probe_read(const void* src, size_t bytes, void* sink, int mode, int workgroups,
                          void* stream) {
    if (!src || !sink) return SSD_ERR_NULL;
    if (!al16(src) || !al16(sink)) return SSD_ERR_ALIGN;
    const ssd_status s = check(bytes, mode, workgroups);
    if (s != SSD_OK) return s;
    const size_t n = bytes / 16;
    const unsigned g = grid_of(n, workgroups);
    if (mode) probe_read_kernel<true><<<g, kThreads, 0, (hipStream_t)stream>>>((const V4*)src, n, (V4*)sink);
    else probe_read_kernel<false><<<g, kThreads, 0, (hipStream_t)stream>>>((const V4*)src, n, (V4*)sink);
    return done();
}

ssd_status ssd_probe_write(void* dst, size_t bytes, int mode, int workgroups, void* stream) {
    if (!dst) return SSD_ERR_NULL;
    if (!al16(dst)) return SSD_ERR_ALIGN;
    const ssd_status s = check(bytes, mode, workgroups);
    if (s != SSD_OK) return s;
    const size_t n = bytes / 16;
    const unsigned g = grid_of(n, workgroups);
    if (mode) probe_write_kernel<true><<<g, kThreads, 0, (hipStream_t)stream>>>((V4*)dst, n);
    else probe_write_kernel<false><<<g, kThreads, 0, (hipStream_t)stream>>>((V4*)dst, n);
    return done();
}

ssd_status ssd_probe_copy(const void* src, void* dst, size_t bytes, int mode, int workgroups,
                          void* stream) {
    if (!src || !dst) return SSD_ERR_NULL;
    if (!al16(src) || !al16(dst)) return SSD_ERR_ALIGN;
    const ssd_status s = check(bytes, mode, workgroups);
    if (s != SSD_OK) return s;
    const size_t n = bytes / 16;
    const unsigned g = grid_of(n, workgroups);
    if (mode) probe_copy_kernel<true><<<g, kThreads, 0, (hipStream_t)stream>>>((const V4*)src, (V4*)dst, n);
    else probe_copy_kernel<false><<<g, kThreads, 0, (hipStream_t)stream>>>((const V4*)src, (V4*)dst, n);
    return done();
}

ssd_status ssd_probe_mix(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                         int mode, int workgroups, void* stream) {
    if ((read_bytes && !src) || (write_bytes && !dst)) return SSD_ERR_NULL;
    if (!al16(src) || !al16(dst)) return SSD_ERR_ALIGN;
    const size_t big = read_bytes > write_bytes ? read_bytes : write_bytes;
    if (read_bytes % 16 != 0 || write_bytes % 16 != 0) return SSD_ERR_SHAPE;
    const ssd_status s = check(big, mode, workgroups);
    if (s != SSD_OK) return s;
    const size_t nr = read_bytes / 16, nw = write_bytes / 16, n = big / 16;
    const unsigned g = grid_of(n, workgroups);
    if (mode)
        probe_mix_kernel<true><<<g, kThreads, 0, (hipStream_t)stream>>>((const V4*)src, nr, (V4*)dst, nw, n);
    else
        probe_mix_kernel<false><<<g, kThreads, 0, (hipStream_t)stream>>>((const V4*)src, nr, (V4*)dst, nw, n);
    return done();
}

}  // extern "C"
