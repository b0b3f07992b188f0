// Stage 3: fused per-chunk output (kernel template; instantiated in k_chunk_out_*.hip).
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Mamba-2 architecture" (the decayed chunk-output formula) and section
// "Kernel 3: compute_out". For chunk c, token rows i and columns j of the chunk:
//     y_i = 2^{G_i} C_i . S_c  +  sum_{j <= i} 2^{G_i - G_j} (C_i . B_j) dt_j x_j  +  D x_i
// where S_c is the chunk-initial state. The interaction C B^T, its decay and the causal
// mask exist only in registers; decays of masked (j > i) pairs are removed by selection,
// never by multiplying, so an overflowing 2^{positive} cannot reach y.
//
// gfx950 mapping
// --------------
// One workgroup of T/32 waves handles one (batch, chunk) and a block of NH heads of one
// B/C group, one head after another:
//  - Wave w owns row tiles w and T/16-1-w, which splits the causal triangle evenly; C's
//    rows of those tiles stay in VGPRs for the whole workgroup.
//  - The interaction tiles S^T = B_j C_i^T (16 x 16, j-tile <= i-tile, K = dstate) do not
//    depend on the head. When they fit, the workgroup computes them once (B staged in LDS
//    when it fits too, else read from L2) and keeps them in LDS in the accumulator layout
//    (each lane reads back its own four values with one 8- or 16-byte load), so every head
//    reuses them; otherwise each head recomputes them.
//  - Per head, x's chunk rows, the chunk-initial state, G, dt and u_j = dt_j 2^{G_e - G_j}
//    (e = last token of j's 16-token tile) sit in LDS; the next head's copies are loaded
//    into registers while the current head computes and are written to LDS after it, so
//    HBM reads overlap the matrix work.
//  - In the S^T accumulator layout each lane holds one row i and four j's per tile --
//    exactly the A-operand layout of y += W x -- so the decay (2^{G_i - G_e} u_j off the
//    diagonal, exact with the causal mask on it) is applied in registers and W is rounded
//    once to the input dtype and used directly; x's token-axis fragments come from the
//    gfx950 transposing LDS read.
//  - The carried-state term C_i . S_c (K = dstate) is scaled per row by 2^{G_i}; D x_i
//    is added and y is written in fp32.
// The page's operand swap for Blackwell's tensor memory does not apply: gfx950 MFMA takes
// both operands from VGPRs.
#pragma once

#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

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

// State fragment in the input's MFMA type. With bf16 inputs and fp32 states each value is
// split into a bf16 high part and a bf16 remainder (two products).
template <typename TIn, typename TS> struct StateFrag {
    static constexpr bool kSplit = false;
    Frag<TIn> hi, lo;
    __device__ __forceinline__ void load(const TS* p, bool valid) { load8(hi, p, valid); }
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

template <typename TIn, typename TS, int P, int S, int T, bool SEGC = false>
struct OutCfg {
    static constexpr int NW = T / 32, NTHR = 2 * T, NIT = T / 16;
    static constexpr int NPT = P / 16, NKS = (S + 31) / 32;
    static constexpr int NTILE = NIT * (NIT + 1) / 2;  // lower-triangular 16 x 16 tiles
    static constexpr int XS = col_stride<TIn>(P);   // x rows (read by columns)
    static constexpr int SS = row_stride<TS>(S);    // state rows (read by rows)
    static constexpr int BS = row_stride<TIn>(S);   // B rows (read by rows)
    static constexpr int VE = 16 / (int)sizeof(TIn), VES = 16 / (int)sizeof(TS);
    static constexpr int NXV = T * P / VE / NTHR;                       // x vectors / thread
    static constexpr int NSV = (P * S / VES + NTHR - 1) / NTHR;         // state vectors / thread
    static constexpr int NBV = T * S / VE / NTHR;                       // B vectors / thread
    static constexpr size_t X_BYTES = (size_t)T * XS * sizeof(TIn);
    static constexpr size_t ST_BYTES = (size_t)P * SS * sizeof(TS);
    static constexpr size_t GD_BYTES = 3 * (size_t)T * sizeof(float);  // G, dt, u
    static constexpr size_t HEAD_BYTES = X_BYTES + ST_BYTES + GD_BYTES;  // per-head region
    static constexpr size_t B_BYTES = (size_t)T * BS * sizeof(TIn);
    // the tiles plus one all-zero tile that stands in for tiles above the diagonal
    static constexpr size_t TILE_BYTES = (size_t)(NTILE + 1) * 256 * sizeof(TIn);
    // SEGC: each head's log2 decay from its segment's start (up to 256 heads) after the rest
    static constexpr size_t DEC_BYTES = SEGC ? 256 * sizeof(float) : 0;
    static constexpr size_t LDS_MAX = 163840 - DEC_BYTES;
    // interaction tiles shared by the heads of a workgroup
    static constexpr bool SHARED = HEAD_BYTES + TILE_BYTES <= LDS_MAX;
    // B staged in LDS: in SHARED mode only while the tiles are built (over the per-head
    // region), otherwise next to the per-head region for the whole kernel
    static constexpr bool B_IN_LDS =
        SHARED ? (B_BYTES > HEAD_BYTES ? B_BYTES : HEAD_BYTES) + TILE_BYTES <= LDS_MAX
               : HEAD_BYTES + B_BYTES <= LDS_MAX;
    static constexpr size_t REGION0 =
        SHARED ? (B_IN_LDS && B_BYTES > HEAD_BYTES ? B_BYTES : HEAD_BYTES) : HEAD_BYTES;
    // SHARED mode with B too large for LDS: the tiles are built in passes over runs of
    // B_PASS 16-row j-tiles, each run's B rows staged over the per-head region (free until
    // the first head is staged); B_PASS is the largest divisor of NIT whose rows fit there.
    // 0 when B is staged whole or the tiles are not shared.
    static constexpr size_t BT_BYTES = (size_t)16 * BS * sizeof(TIn);  // one j-tile's B rows
    static constexpr int pass_tiles() {
        if (!SHARED || B_IN_LDS) return 0;
        int best = 0;
        for (int n = 1; n < NIT; ++n)
            if (NIT % n == 0 && n * BT_BYTES <= HEAD_BYTES) best = n;
        return best;
    }
    static constexpr int B_PASS = pass_tiles();
    static constexpr int NBVP = B_PASS * 16 * S / VE / NTHR;  // B vectors / thread and pass
    static constexpr size_t BASE_BYTES =
        SHARED ? REGION0 + TILE_BYTES : HEAD_BYTES + (B_IN_LDS ? B_BYTES : 0);
    // fp32 y leaves through a per-wave LDS scratch of 16 rows x 32 columns (two p-tiles), so
    // that each store instruction writes whole 128-byte row pieces; only where the scratch
    // fits without lowering the workgroups resident per CU (the bf16-y instances of the
    // same shape carry it unused, so that every instance of a shape has one launch plan)
    static constexpr size_t Y_OFF = (BASE_BYTES + DEC_BYTES + 15) / 16 * 16;
    static constexpr int YST = 36;  // scratch row stride in floats (rows 16 banks apart)
    static constexpr size_t Y_SCR_BYTES = (size_t)NW * 16 * YST * 4;
    // (measured: at 128-token chunks the article's shape went from 90 to 68 us; at 256 the
    // 2.7B layer ran 1% slower, so the 8-wave form keeps the direct stores)
    static constexpr bool Y_STAGE = NPT % 2 == 0 && T <= 128 && Y_OFF + Y_SCR_BYTES <= 163840 &&
                                    163840 / (Y_OFF + Y_SCR_BYTES) ==
                                        163840 / (BASE_BYTES + DEC_BYTES);
    static constexpr size_t LDS_BYTES = Y_STAGE ? Y_OFF + Y_SCR_BYTES : BASE_BYTES + DEC_BYTES;
    // minimum waves per SIMD asked of the register allocator: two for the shapes that fit
    // them without spilling (bf16 inputs and states up to P 64, S 128; fp32 up to P 64,
    // S 64, 128-token chunks), so that two workgroups share a compute unit where LDS allows
    static constexpr int WPE = ((sizeof(TIn) == 2 && sizeof(TS) == 2 && P <= 64 && S <= 128) ||
                                (sizeof(TIn) == 4 && P <= 64 && S <= 64 && T <= 128))
                                   ? 2
                                   : 1;
};

// y element store through a buffer descriptor: fp32, or bf16 rounded to nearest even.
__device__ __forceinline__ void store_y(float v, float*, BufRsrc r, uint32_t voff, uint32_t soff) {
    buf_store_f32(v, r, voff, soff);
}
__device__ __forceinline__ void store_y(float v, bf16*, BufRsrc r, uint32_t voff, uint32_t soff) {
    const bf16 b = from_f32<bf16>(v);
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b), r, voff, soff, 0);
}

// SEGC: the chunk states are relative to the start of their segment of seg_chunks chunks
// (see state_seg.h); the state of chunk c in segment k >= 1 is states[c] +
// 2^{dec_in[c]} seg_in[k], formed in fp32 while the state is staged and rounded once.
template <typename TIn, typename TS, typename TY, int P, int S, int T, bool SEGC = false>
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(OutCfg<TIn, TS, P, S, T, SEGC>::WPE))) void chunk_out_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ Bm, const TIn* __restrict__ Cm,
    const float* __restrict__ G, const float* __restrict__ dt_t, const TS* __restrict__ states,
    const float* __restrict__ Dv, TY* __restrict__ y, int L, int H, int ngroups, int NH,
    const TS* __restrict__ seg_in, const float* __restrict__ dec_in, int seg_chunks) {
    using Cfg = OutCfg<TIn, TS, P, S, T, SEGC>;
    static_assert(!SEGC || sizeof(TS) == 2, "segment-relative states are bf16");
    constexpr int NPT = Cfg::NPT, NKS = Cfg::NKS, XS = Cfg::XS, SS = Cfg::SS, BS = Cfg::BS;
    constexpr int VE = Cfg::VE, VES = Cfg::VES, NTHR = Cfg::NTHR;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    TIn* s_x = (TIn*)smem;                                                  // [T][XS]
    TS* s_st = (TS*)(smem + Cfg::X_BYTES);                                  // [P][SS]
    float* s_g = (float*)(smem + Cfg::X_BYTES + Cfg::ST_BYTES);             // [T]
    float* s_dt = s_g + T;                                                  // [T]
    float* s_u = s_dt + T;                                                  // [T]
    // B rows: over the per-head region (SHARED, prologue only) or after it
    TIn* s_b = (TIn*)(smem + (Cfg::SHARED ? 0 : Cfg::HEAD_BYTES));         // [T][BS]
    TIn* s_tiles = (TIn*)(smem + Cfg::REGION0);                            // [NTILE+1][64][4]
    float* s_dec = (float*)(smem + Cfg::BASE_BYTES);                       // [NH] (SEGC)

    const int nC = (L + T - 1) / T;
    const int nhb = H / NH;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = id % nhb;
    const int c = (id / nhb) % nC;
    const int b = id / (nhb * nC);
    const int h_first = hb * NH;
    const int g = h_first / (H / ngroups);  // NH divides the heads per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int g4 = lane >> 4, l16 = lane & 15;
    const int t0 = c * T;
    // real tokens of this chunk; a partial last chunk is computed as if padded with zero
    // tokens (dt = 0 keeps G at its last real value), and its padded rows are not stored
    const int rows = min(T, L - t0);
    const int HP = H * P;
    const size_t grow = (size_t)ngroups * S;
    const TIn* cg = Cm + (((size_t)b * L + t0) * ngroups + g) * S;
    const TIn* bg = Bm + (((size_t)b * L + t0) * ngroups + g) * S;
    const int its[2] = {wave, Cfg::NIT - 1 - wave};

    // buffer descriptors over this chunk's rows of x and y (all heads) and the
    // per-(batch, head) decay rows; per-head offsets go in the uniform offset operand
    // (x and y rows past the real tokens lie outside these descriptors: loads return zeros
    // and stores are dropped). Each head's chunk-initial state gets a descriptor of its
    // own, so the states of a batch row may exceed what 32-bit offsets reach.
    const BufRsrc rx = make_rsrc(x + ((size_t)b * L + t0) * HP, (uint32_t)(rows * HP * sizeof(TIn)));
    const BufRsrc ry = make_rsrc(y + ((size_t)b * L + t0) * HP, (uint32_t)(rows * HP * sizeof(TY)));
    const BufRsrc rg = make_rsrc(G + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));
    const BufRsrc rdt = make_rsrc(dt_t + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));

    // ---- per-head staging: global -> registers (prefetch) -> LDS ----------------------
    Vec16 px[Cfg::NXV], pst[Cfg::NSV];
    float pg = 0.f, pdt = 0.f, pge = 0.f;
    // segment correction (SEGC): entering state of this chunk's segment and its decay
    const int seg = SEGC ? c / seg_chunks : 0;
    const bool corr = SEGC && seg > 0;  // workgroup-uniform
    const int nseg = SEGC ? (nC + seg_chunks - 1) / seg_chunks : 0;
    Vec16 psi[SEGC ? Cfg::NSV : 1];
    float pdec = 0.f;
    // (below kSegCut the correction adds exactly nothing and seg_in is not read at all)
    auto load_head = [&](int h) {
#pragma unroll
        for (int i = 0; i < Cfg::NXV; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / (P / VE), col = (v % (P / VE)) * VE;
            px[i] = buf_load16(rx, (uint32_t)((r * HP + col) * sizeof(TIn)),
                               (uint32_t)(h * P * sizeof(TIn)));
        }
        const BufRsrc rst = make_rsrc(states + (((size_t)b * H + h) * nC + c) * P * S,
                                      (uint32_t)(P * S * sizeof(TS)));
#pragma unroll
        for (int i = 0; i < Cfg::NSV; ++i) {
            const int v = tid + i * NTHR;
            if (v < P * S / VES) pst[i] = buf_load16(rst, (uint32_t)(v * 16), 0u);
        }
        if constexpr (SEGC) {
            if (corr) {
                // the first head's decay from global memory, the others' from LDS (staged
                // by the prologue)
                pdec = h == h_first ? dec_in[((size_t)b * H + h) * nC + c] : s_dec[h - h_first];
                if (pdec >= kSegCut) {
                    const BufRsrc rsi = make_rsrc(seg_in + (((size_t)b * H + h) * nseg + seg) * P * S,
                                                  (uint32_t)(P * S * sizeof(TS)));
#pragma unroll
                    for (int i = 0; i < Cfg::NSV; ++i) {
                        const int v = tid + i * NTHR;
                        if (v < P * S / VES) psi[i] = buf_load16(rsi, (uint32_t)(v * 16), 0u);
                    }
                }
            }
        }
        if (tid < T) {
            const uint32_t o = (uint32_t)(((size_t)h * L + t0) * sizeof(float));
            pg = buf_load_f32(rg, min(tid, rows - 1) * 4, o);
            pdt = tid < rows ? buf_load_f32(rdt, tid * 4, o) : 0.f;
            pge = buf_load_f32(rg, min(tid | 15, rows - 1) * 4, o);  // G at the tile's last token
        }
    };
    auto store_head = [&]() {
#pragma unroll
        for (int i = 0; i < Cfg::NXV; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / (P / VE), col = (v % (P / VE)) * VE;
            *(Vec16*)(s_x + r * XS + col) = px[i];
        }
        if constexpr (SEGC) {
            if (corr && pdec >= kSegCut) {
                const float f = exp2_fast(pdec);
#pragma unroll
                for (int i = 0; i < Cfg::NSV; ++i) {
                    const bf16x8 l8 = __builtin_bit_cast(bf16x8, pst[i]);
                    const bf16x8 s8 = __builtin_bit_cast(bf16x8, psi[i]);
                    bf16x8 o;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(to_f32(l8[e]) + f * to_f32(s8[e]));
                    pst[i] = __builtin_bit_cast(Vec16, o);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::NSV; ++i) {
            const int v = tid + i * NTHR;
            if (v < P * S / VES) {
                const int r = v / (S / VES), col = (v % (S / VES)) * VES;
                *(Vec16*)(s_st + r * SS + col) = pst[i];
            }
        }
        if (tid < T) {
            s_g[tid] = pg;
            s_dt[tid] = pdt;
            // u_j = dt_j 2^{G_e - G_j}, e = last token of j's tile: the decay from j to the
            // end of its tile (<= 1), shared by every row tile below it
            s_u[tid] = pdt * exp2_fast(pge - pg);
        }
    };

    // ---- prologue: C rows (registers), interaction tiles (LDS), first head ------------
    Frag<TIn> cf[2][NKS];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int s0 = ks * 32 + g4 * 8;
            load8(cf[q][ks], cg + (size_t)(its[q] * 16 + l16) * grow + s0,
                  s0 < S && its[q] * 16 + l16 < rows);
        }
    if constexpr (Cfg::B_IN_LDS) {
        Vec16 pb[Cfg::NBV];
#pragma unroll
        for (int i = 0; i < Cfg::NBV; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / (S / VE), col = (v % (S / VE)) * VE;
            pb[i] = r < rows ? *(const Vec16*)(bg + (size_t)r * grow + col) : Vec16{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < Cfg::NBV; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / (S / VE), col = (v % (S / VE)) * VE;
            *(Vec16*)(s_b + r * BS + col) = pb[i];
        }
    }
    // B_PASS: the B rows of j-tiles j0 .. j0 + B_PASS - 1 into s_b (rows past the chunk's
    // real tokens as zeros)
    auto stage_b_pass = [&](int j0) {
        if constexpr (Cfg::B_PASS > 0) {
            Vec16 pb[Cfg::NBVP];
#pragma unroll
            for (int i = 0; i < Cfg::NBVP; ++i) {
                const int v = tid + i * NTHR;
                const int r = j0 * 16 + v / (S / VE), col = (v % (S / VE)) * VE;
                pb[i] = r < rows ? *(const Vec16*)(bg + (size_t)r * grow + col)
                                 : Vec16{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < Cfg::NBVP; ++i) {
                const int v = tid + i * NTHR;
                const int r = v / (S / VE), col = (v % (S / VE)) * VE;
                *(Vec16*)(s_b + r * BS + col) = pb[i];
            }
        }
    };
    if constexpr (Cfg::B_PASS > 0) stage_b_pass(0);
    // B rows of j-tile jt as the A operand of S^T = B_j C_i^T (lane: row j, 8 dstate values);
    // j0: the first j-tile staged in s_b
    auto load_bfrag = [&](Frag<TIn>& f, int jt, int ks, int j0 = 0) {
        const int s0 = ks * 32 + g4 * 8;
        if constexpr (Cfg::B_IN_LDS || Cfg::B_PASS > 0)
            load8(f, s_b + ((jt - j0) * 16 + l16) * BS + s0, s0 < S);
        else
            load8(f, bg + (size_t)(jt * 16 + l16) * grow + s0, s0 < S && jt * 16 + l16 < rows);
    };
    auto tile_ptr = [&](int q, int jt) {  // this lane's 4 values of tile (its[q], jt)
        const int k = jt <= its[q] ? its[q] * (its[q] + 1) / 2 + jt : Cfg::NTILE;
        return s_tiles + ((size_t)k * 64 + lane) * 4;
    };
    load_head(h_first);  // in flight while the tiles are built
    if constexpr (SEGC) {
        // the block's decays from the segment's start, read by the later heads' loads
        if (corr && tid < NH) s_dec[tid] = dec_in[((size_t)b * H + h_first + tid) * nC + c];
    }
    if constexpr (Cfg::SHARED) {
        // build this wave's interaction tiles once for all heads of the workgroup (in
        // passes over runs of j-tiles when only a run's B rows fit in LDS)
        constexpr int JB = Cfg::B_PASS > 0 ? Cfg::B_PASS : Cfg::NIT;
        const int itmax = its[1];
        // every wave runs every pass (the barriers inside), with no tiles where j0 > itmax
        for (int j0 = 0; j0 < Cfg::NIT; j0 += JB) {
            if constexpr (Cfg::B_PASS > 0) {
                if (j0 > 0) {
                    lds_barrier();  // every wave is done with the previous run's rows
                    stage_b_pass(j0);
                }
            }
            if constexpr (Cfg::B_IN_LDS || Cfg::B_PASS > 0) lds_barrier();
            for (int jt = j0; jt <= min(itmax, j0 + JB - 1); ++jt) {
                f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    Frag<TIn> bfr;
                    load_bfrag(bfr, jt, ks, j0);
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        if (jt <= its[q]) mma(st[q], bfr, cf[q][ks]);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (jt > its[q]) continue;
                    TIn* dst = tile_ptr(q, jt);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[r] = from_f32<TIn>(st[q][r]);
                }
            }
        }
        if (wave == 0) {
            TIn* z = s_tiles + ((size_t)Cfg::NTILE * 64 + lane) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) z[r] = from_f32<TIn>(0.f);
        }
        lds_barrier();  // tiles written; the B rows (if staged) may now be overwritten
    }
    store_head();
    lds_barrier();

    // y offsets (bytes) of this lane's 8 rows within the chunk, for column l16 of head 0
    uint32_t yoff[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            yoff[q][r] = (uint32_t)(((its[q] * 16 + 4 * g4 + r) * HP + l16) * sizeof(TY));

    for (int hh = 0; hh < NH; ++hh) {
        const int h = h_first + hh;
        if (hh + 1 < NH) load_head(h + 1);  // in flight while this head computes

        f32x4 yacc[2][NPT];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) yacc[q][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // 1. carried state: C_i . S_c over dstate, then row scale 2^{G_i}
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int s0 = ks * 32 + g4 * 8;
                StateFrag<TIn, TS> hf;
                hf.load(s_st + (pt * 16 + l16) * SS + s0, s0 < S);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    mma(yacc[q][pt], cf[q][ks], hf.hi);
                    if constexpr (StateFrag<TIn, TS>::kSplit) mma(yacc[q][pt], cf[q][ks], hf.lo);
                }
            }
        }
        float gi[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            gi[q] = s_g[its[q] * 16 + l16];
            const f32x4 g4v = *(const f32x4*)(s_g + its[q] * 16 + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sc = exp2_fast(g4v[r]);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) yacc[q][pt][r] *= sc;
            }
        }

        // 2. within the chunk, two 16-column tiles (32 tokens) per step
        const int itmax = its[1];
        for (int kp = 0; 2 * kp <= itmax; ++kp) {
            // S^T tiles (rows j of the two column tiles, columns i of both row tiles);
            // tiles above the diagonal read as zeros
            f32x4 st[2][2];
            if constexpr (Cfg::SHARED) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const TIn* src = tile_ptr(q, 2 * kp + jj);
                        if constexpr (sizeof(TIn) == 2) {
                            const bf16x4 t4 = *(const bf16x4*)src;
#pragma unroll
                            for (int r = 0; r < 4; ++r) st[q][jj][r] = to_f32(t4[r]);
                        } else {
                            st[q][jj] = *(const f32x4*)src;
                        }
                    }
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) st[q][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
                // one B fragment is live at a time and feeds both row tiles
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int jt = 2 * kp + jj;
                    if (jt > itmax) continue;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        Frag<TIn> bfr;
                        load_bfrag(bfr, jt, ks);
#pragma unroll
                        for (int q = 0; q < 2; ++q)
                            if (jt <= its[q]) mma(st[q][jj], bfr, cf[q][ks]);
                    }
                }
            }
            // x fragments: slot (g4, v) carries token j = 32kp + 16(v/4) + 4 g4 + v%4,
            // matching the rows the S^T accumulator holds in each lane
            Frag<TIn> xf[NPT];
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                if constexpr (sizeof(TIn) == 2) {
                    const bf16x4 lo4 = lds_col4(s_x, XS, 32 * kp + 4 * g4, pt * 16, lane);
                    const bf16x4 hi4 = lds_col4(s_x, XS, 32 * kp + 16 + 4 * g4, pt * 16, lane);
                    xf[pt].v = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const int j = 32 * kp + 16 * (v >> 2) + 4 * g4 + (v & 3);
                        xf[pt].v[v] = s_x[j * XS + pt * 16 + l16];
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int it = its[q];
                if (it < 2 * kp) continue;
                float w[8];
                // off the diagonal every i is past the tile's last token e:
                // decay = 2^{G_i - G_e} u_j. Above the diagonal the tile is zero and the
                // clamped exponent keeps the factor finite.
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int jt = 2 * kp + jj;
                    const float v = exp2_fast(fminf(gi[q] - s_g[jt * 16 + 15], 0.f));
                    const f32x4 u = *(const f32x4*)(s_u + jt * 16 + 4 * g4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[jj * 4 + r] = st[q][jj][r] * (v * u[r]);
                }
                if ((it >> 1) == kp) {
                    // the diagonal tile (the first of the pair when it is even): exact decay
                    // with the causal mask, by selection
                    const bool lo = (it & 1) == 0;
                    const int i = it * 16 + l16;
                    const int j0 = it * 16 + 4 * g4;
                    const f32x4 gj = *(const f32x4*)(s_g + j0);
                    const f32x4 dj = *(const f32x4*)(s_dt + j0);
                    f32x4 e4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) e4[r] = exp2_fast(gi[q] - gj[r]) * dj[r];
                    if (lo) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w[r] = (i >= j0 + r) ? st[q][0][r] * e4[r] : 0.f;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w[4 + r] = (i >= j0 + r) ? st[q][1][r] * e4[r] : 0.f;
                    }
                }
                Frag<TIn> wf;
#pragma unroll
                for (int v = 0; v < 8; ++v) wf.v[v] = from_f32<TIn>(w[v]);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) mma(yacc[q][pt], wf, xf[pt]);
            }
        }

        // 3. skip term and store (x of this lane's rows i by a column read)
        const float dh = Dv ? Dv[h] : 0.f;
        const uint32_t yh = (uint32_t)(h * P * sizeof(TY));
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                float xi[4];
                if constexpr (sizeof(TIn) == 2) {
                    const bf16x4 x4 = lds_col4(s_x, XS, its[q] * 16 + 4 * g4, pt * 16, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) xi[r] = to_f32(x4[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        xi[r] = s_x[(its[q] * 16 + 4 * g4 + r) * XS + pt * 16 + l16];
                }
                if constexpr (Cfg::Y_STAGE && sizeof(TY) == 4) {
                    // into this wave's scratch (rows of the row tile, two p-tiles wide);
                    // after each pair, 16-byte reads give each lane four consecutive
                    // columns and 8 lanes cover a 128-byte row piece
                    float* scr = (float*)(smem + Cfg::Y_OFF) + wave * 16 * Cfg::YST;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        scr[(4 * g4 + r) * Cfg::YST + (pt & 1) * 16 + l16] = yacc[q][pt][r] + dh * xi[r];
                    if (pt & 1) {
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const int v = i * 64 + lane, rr = v >> 3, c4 = (v & 7) * 4;
                            const f32x4 o = *(const f32x4*)(scr + rr * Cfg::YST + c4);
                            buf_store16(__builtin_bit_cast(Vec16, o), ry,
                                        (uint32_t)((((its[q] * 16 + rr) * HP) + h * P +
                                                    (pt - 1) * 16 + c4) * sizeof(float)));
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        store_y(yacc[q][pt][r] + dh * xi[r], y, ry,
                                yoff[q][r] + pt * 16 * (uint32_t)sizeof(TY), yh);
                }
            }

        lds_barrier();  // every wave is done with this head's LDS copies
        if (hh + 1 < NH) {
            store_head();
            lds_barrier();
        }
    }
}

// Heads per workgroup. Each workgroup pays a fixed prologue (C rows, B rows, the
// interaction tiles), so it should serve as many heads as possible -- but the grid must
// still cover every CU with as many resident workgroups as fit. Pick the largest divisor
// of the heads per group whose grid still gives every CU its resident workgroups.
inline int heads_per_block(const Dims& d, size_t lds_bytes, int max_nh = 1 << 30) {
    const int hpg = d.nheads / d.ngroups;
    const long units = (long)d.batch * d.nchunks() * d.nheads;
    const long per_cu = std::max<long>(1, std::min<long>(163840 / (long)std::max<size_t>(lds_bytes, 1),
                                                         32 / (d.chunk / 32)));
    const long want = 256L * per_cu;  // workgroups that fill 256 CUs once
    int best = 1;
    for (int nh = 1; nh <= hpg; ++nh)
        if (hpg % nh == 0 && units / nh >= want && nh <= max_nh) best = nh;
    return best;
}

// The launch plan of chunk_out_kernel for a shape (host-only): heads per workgroup, whether
// the interaction tiles are shared by the workgroup's heads, and the matrix-core flops the
// launch executes (each mma() call is 2 x 16 x 16 x 32 flops, on bf16 16x16x32 or eight
// fp32 16x16x4 instructions): the tiles (once per workgroup when shared, else per head),
// per head the carried-state product C_i . S_c (twice with split fp32 states) and the
// masked products W x over the row tiles' column-tile pairs.
template <typename TIn, typename TS, int P, int S, int T, bool SEGC>
OutPlan out_plan_t(const Dims& d) {
    using Cfg = OutCfg<TIn, TS, P, S, T, SEGC>;
    const int nh = heads_per_block(d, Cfg::LDS_BYTES, SEGC ? 256 : 1 << 30);
    const double nblocks = (double)d.batch * d.nchunks() * (d.nheads / nh);
    long pairs = 0;  // column-tile pairs of every row tile
    for (int it = 0; it < Cfg::NIT; ++it) pairs += it / 2 + 1;
    const long tiles = (long)Cfg::NTILE * Cfg::NKS;
    const long per_head = (long)Cfg::NIT * Cfg::NPT * Cfg::NKS * (StateFrag<TIn, TS>::kSplit ? 2 : 1) +
                          (long)Cfg::NPT * pairs;
    const double calls = (Cfg::SHARED ? (double)tiles : (double)tiles * nh) + (double)per_head * nh;
    return OutPlan{nh, Cfg::SHARED, calls * nblocks * 2.0 * 16 * 16 * 32, (double)Cfg::LDS_BYTES};
}

template <typename TIn, typename TS, typename TY, int P, int S, int T, bool SEGC = false>
hipError_t run_out(const void* x, const void* Bm, const void* Cm, const float* G,
                   const float* dt_t, const void* states, const float* D, void* y,
                   const Dims& d, hipStream_t stream, const void* seg_in = nullptr,
                   const float* dec_in = nullptr, int seg_chunks = 0) {
    using Cfg = OutCfg<TIn, TS, P, S, T, SEGC>;
    auto kern = chunk_out_kernel<TIn, TS, TY, P, S, T, SEGC>;
    if (Cfg::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)Cfg::LDS_BYTES);
        if (e != hipSuccess) return e;
    }
    // SEGC: the block's decays are staged in LDS for at most 256 heads
    const int nh = heads_per_block(d, Cfg::LDS_BYTES, SEGC ? 256 : 1 << 30);
    const int nblocks = d.batch * d.nchunks() * (d.nheads / nh);
    kern<<<nblocks, 2 * T, Cfg::LDS_BYTES, stream>>>((const TIn*)x, (const TIn*)Bm,
                                                     (const TIn*)Cm, G, dt_t,
                                                     (const TS*)states, D, (TY*)y, d.seqlen,
                                                     d.nheads, d.ngroups, nh, (const TS*)seg_in,
                                                     dec_in, seg_chunks);
    return hipGetLastError();
}

template <typename TIn, typename TS, typename TY, int P, int S>
hipError_t out_by_t(const void* x, const void* Bm, const void* Cm, const float* G,
                    const float* dt_t, const void* st, const float* D, void* y, const Dims& d,
                    hipStream_t s) {
    switch (d.chunk) {
        case 64: return run_out<TIn, TS, TY, P, S, 64>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 128: return run_out<TIn, TS, TY, P, S, 128>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 256: return run_out<TIn, TS, TY, P, S, 256>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
    }
    return hipErrorInvalidValue;
}

template <typename TIn, typename TS, typename TY, int P>
hipError_t out_by_s(const void* x, const void* Bm, const void* Cm, const float* G,
                    const float* dt_t, const void* st, const float* D, void* y, const Dims& d,
                    hipStream_t s) {
    switch (d.dstate) {
        case 16: return out_by_t<TIn, TS, TY, P, 16>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 32: return out_by_t<TIn, TS, TY, P, 32>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 64: return out_by_t<TIn, TS, TY, P, 64>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 128: return out_by_t<TIn, TS, TY, P, 128>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 256: return out_by_t<TIn, TS, TY, P, 256>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
    }
    return hipErrorInvalidValue;
}

template <typename TIn, typename TS, typename TY>
hipError_t out_by_p(const void* x, const void* Bm, const void* Cm, const float* G,
                    const float* dt_t, const void* st, const float* D, void* y, const Dims& d,
                    hipStream_t s) {
    switch (d.headdim) {
        case 16: return out_by_s<TIn, TS, TY, 16>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 32: return out_by_s<TIn, TS, TY, 32>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 64: return out_by_s<TIn, TS, TY, 64>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
        case 128: return out_by_s<TIn, TS, TY, 128>(x, Bm, Cm, G, dt_t, st, D, y, d, s);
    }
    return hipErrorInvalidValue;
}

// Segment-relative chunk states (bf16 inputs and states), for the shapes the segmented
// state pass is built for (headdim 64, dstate 64, 128 or 256).
template <typename TY>
hipError_t out_seg(const void* x, const void* Bm, const void* Cm, const float* G,
                   const float* dt_t, const void* st, const void* seg_in, const float* dec_in,
                   int seg_chunks, const float* D, void* y, const Dims& d, hipStream_t s) {
#define SSD_OUT_SEG(p, s_, t)                                                                  \
    if (d.headdim == p && d.dstate == s_ && d.chunk == t)                                      \
        return run_out<bf16, bf16, TY, p, s_, t, true>(x, Bm, Cm, G, dt_t, st, D, y, d, s,     \
                                                       seg_in, dec_in, seg_chunks);
    SSD_OUT_SEG(64, 64, 64) SSD_OUT_SEG(64, 64, 128) SSD_OUT_SEG(64, 64, 256)
    SSD_OUT_SEG(64, 128, 64) SSD_OUT_SEG(64, 128, 128) SSD_OUT_SEG(64, 128, 256)
    SSD_OUT_SEG(64, 256, 64) SSD_OUT_SEG(64, 256, 128) SSD_OUT_SEG(64, 256, 256)
#undef SSD_OUT_SEG
    return hipErrorInvalidValue;
}

}  // namespace ssd
