// Device-side building blocks for the gfx950 SSD kernels: element types, MFMA operand
// fragments, conversions, base-2 exponential and a wave64 DPP prefix scan.
//
// MFMA fragment convention (16x16 output tiles, K = 32 per step)
// ---------------------------------------------------------------
// A "fragment" is the 8 values one lane contributes to a K=32 step. Lane l has
// row/column index (l & 15) of its operand and "slot group" g = l >> 4 (0..3); its
// item v (0..7) fills slot (g, v). Each kernel decides which k (token or state index)
// each slot (g, v) carries; the A and B fragments of one product always use the same
// assignment, so the sum over k is the same whatever order the matrix core walks the
// slots in.
//   bf16 : one v_mfma_f32_16x16x32_bf16 per step (8 bf16 per lane and operand).
//   fp32 : eight v_mfma_f32_16x16x4_f32 per step; the v-th one takes item v of every
//          lane (so slot (g, v) is row k = g of the v-th product).
// The 16x16 fp32 accumulator tile holds element (row 4*g + r, column l & 15) in
// register r (0..3) of lane l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int v = 0; v < 8; ++v)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[v], b.v[v], acc, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// 2^x with the hardware transcendental unit (v_exp_f32). Very negative x gives 0;
// large positive x gives +inf, which callers select away and never multiply.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// four row_shr steps scan each row of 16 lanes, then row_bcast:15 and row_bcast:31 carry
// row totals into the later rows. Lanes whose DPP source is outside the row keep `old`
// (0 here), which is the additive identity.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    int x = __float_as_int(v);
#define SSD_DPP_ADD(ctrl, rmask)                                                        \
    {                                                                                   \
        int t = __builtin_amdgcn_update_dpp(0, x, ctrl, rmask, 0xf, false);             \
        x = __float_as_int(__int_as_float(x) + __int_as_float(t));                      \
    }
    SSD_DPP_ADD(0x111, 0xf)  // row_shr:1
    SSD_DPP_ADD(0x112, 0xf)  // row_shr:2
    SSD_DPP_ADD(0x114, 0xf)  // row_shr:4
    SSD_DPP_ADD(0x118, 0xf)  // row_shr:8
    SSD_DPP_ADD(0x142, 0xa)  // row_bcast:15 into rows 1 and 3
    SSD_DPP_ADD(0x143, 0xc)  // row_bcast:31 into rows 2 and 3
#undef SSD_DPP_ADD
    return __int_as_float(x);
}

// Value of the previous lane (lane 0 gets 0): turns an inclusive scan into an exclusive one
// without a subtraction (DPP wave_shr:1).
__device__ __forceinline__ float wave_shift_up1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, false));
}

// Per-chunk cumulative decay of one head, one wave: lane l holds the chunk's tokens
// l*PER .. l*PER+PER-1 (d = dt, fp32). G[t] = log2(e) * sum of A dt over the chunk's tokens
// up to t (inclusive): a serial sum over the lane's tokens, then a DPP scan of the lane
// totals. Every kernel that forms G calls this, so they agree bit for bit.
template <int PER>
__device__ __forceinline__ void chunk_log2_decay(const float (&d)[PER], float ah, float (&g)[PER]) {
    float part[PER];
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        run += ah * d[k];
        part[k] = run;
    }
    // exclusive prefix of the lane totals = inclusive prefix of the previous lane
    const float excl = wave_shift_up1(wave_inclusive_scan(run));
    {
        // G is a rounded product wherever it is used: a caller that goes on to subtract it
        // must not have the multiply fused into that subtraction (an FMA would skip the
        // rounding and give other bits than a G read back from memory)
#pragma clang fp contract(off)
#pragma unroll
        for (int k = 0; k < PER; ++k) g[k] = (excl + part[k]) * kLog2e;
    }
}

// LDS row strides (in elements) chosen against bank conflicts on 64 four-byte banks.
//  - col_stride: for ds_read_b64_tr_b16 column reads, where the 32 lanes served together
//    read 8 consecutive rows x 32 bytes: the row stride in words must be an odd multiple
//    of 8 so those rows land on disjoint 8-bank windows (fp32 tiles, read one element per
//    lane from rows 4 apart, need a stride of 4 mod 16 words instead).
//  - row_stride: for 16-byte row reads by 16 lanes of 16 different rows: stride = 4 mod 8
//    words spreads the rows over disjoint 4-bank windows.
template <typename T> constexpr int col_stride(int n) {
    return sizeof(T) == 2 ? (n == 16 ? 16 : n + 16) : n + 4;
}
template <typename T> constexpr int row_stride(int n) { return sizeof(T) == 2 ? n + 8 : n + 4; }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Column read through the gfx950 transposing LDS load (ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane s supplies the address of 4 consecutive elements and lane j
// receives element (j & 3) from lanes (j >> 2) + 4k, k = 0..3. Pointing lane s at row
// r0 + (s >> 2), column c0 + 4 (s & 3) of a row-major matrix therefore hands lane j the
// column c0 + j of rows r0 .. r0 + 3. r0 may differ between the four 16-lane groups.
// `base` must be the start of a __shared__ array; ld is its row stride in elements.
__device__ __forceinline__ bf16x4 lds_col4(const bf16* base, int ld, int r0, int c0, int lane) {
    const int s = lane & 15;
    const bf16* p = base + (r0 + (s >> 2)) * ld + c0 + 4 * (s & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(__attribute__((address_space(3))) bf16*)p);
}

// Buffer-resource addressing: a 128-bit descriptor (base in SGPRs, size in bytes) plus a
// 32-bit per-lane offset and a 32-bit uniform offset, so loads and stores need no 64-bit
// per-lane address arithmetic. Accesses at or beyond `bytes` are dropped (stores) or
// return zero (loads) by the hardware range check. Word 3 = 0x00020000 is the raw 32-bit
// data format of the gfx9 family.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// The b32 buffer builtins move raw 32-bit patterns (integers); floats are bit-cast.
__device__ __forceinline__ void buf_store_f32(float v, BufRsrc r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}

// 16-byte vector type for cooperative global<->LDS copies.
typedef uint32_t Vec16 __attribute__((ext_vector_type(4)));

// 16-byte buffer store with the whole byte offset in the per-lane offset and a constant 0
// in the uniform (SGPR) offset field. A store of more than 8 bytes reads its data
// registers after issue, so they must not be rewritten for two wait states. The compiler
// inserts those wait states only when the uniform offset is not a register; with a
// register there it let the next VALU or MFMA instruction overwrite the data registers
// at once, and on gfx950 that corrupted what the store wrote (seen in the segmented state
// kernel's recorded states). Keeping the uniform offset 0 keeps the wait states.
__device__ __forceinline__ void buf_store16(Vec16 v, BufRsrc r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0u, 0);
}
__device__ __forceinline__ Vec16 buf_load16(BufRsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ float buf_load_f32(BufRsrc r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Workgroup barrier that orders LDS only: this wave's global loads and stores in flight
// stay in flight (__syncthreads' workgroup-scope release fence would first wait for all
// of them to complete). For barriers that only hand over data staged in LDS.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Map a linear workgroup id so that consecutive logical ids run on the same XCD:
// hardware hands workgroups to the 8 XCDs round-robin, so logical id
// (xcd * per_xcd + k) is given to hardware id (k * 8 + xcd). Consecutive logical ids
// (neighbouring heads of one chunk, which read the same B/C rows) then share an L2.
__device__ __forceinline__ int xcd_remap(int hw_id, int nblocks) {
    if (nblocks % 8 != 0) return hw_id;
    const int per_xcd = nblocks / 8;
    return (hw_id % 8) * per_xcd + hw_id / 8;
}

}  // namespace ssd
