// Backward pass on the matrix cores (bf16 inputs): the per-chunk products of the gradient
// written as causal decayed products, one kernel template for three of them.
//
// Inside chunk c (tokens t, s of the chunk; G the inclusive log2 decay from the chunk's
// start, G_e its value at the last real token; H_c the state entering the chunk and R_c
// the gradient arriving at its end), the chain rule through the recurrence of page
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile",
// section "Mamba-2 architecture", gives
//     dC_t  = 2^{G_t} H_c^T dy_t       + sum_{s <= t} 2^{G_t - G_s} dt_s (dy_t . x_s) B_s
//     dB_s  = dt_s [2^{G_e - G_s} R_c^T x_s + sum_{t >= s} 2^{G_t - G_s} (x_s . dy_t) C_t]
//     dxh_s = 2^{G_e - G_s} R_c B_s    + sum_{t >= s} 2^{G_t - G_s} (B_s . C_t) dy_t
// with dx_s = D dy_s + dt_s dxh_s. Each is
//     out_i = scale_i Q_i . Z  +  sum_{j causal to i} 2^{+-(G_i - G_j)} w_j (Q_i . K_j) V_j
// ("causal" is j <= i forward in time for dC, j >= i backward in time for dB and dxh):
//     op   Q    K    V    Z (state, [N][KD])   w     scale
//     dC   dy   x    B    H_c^T                dt    2^{G_i}
//     dB   x    dy   C    R_c^T                1     2^{G_e - G_i}   (times dt_i after)
//     dxh  B    C    dy   R_c                  1     2^{G_e - G_i}
// The epilogues also form q_t = C_t . dC_t (dC op), and v_s = x_s . dxh_s, dy_s . x_s and
// dx (dxh op), the per-token scalars of the decay gradient.
//
// gfx950 mapping: one workgroup per (batch, chunk, block of NH heads of one group), the
// heads one after another (the next head's rows loading while the current one computes),
// with T/32 pairs of row tiles and NSPLIT waves per pair; K rows, V rows, Q rows (dC, dB;
// dxh's Q, B's rows, stays in registers), the state (bf16 high and low parts of its fp32
// values) and G, dt in LDS. Wave pair w owns row tiles w and T/16-1-w (equal causal
// work). For each 32-wide block of j it builds the two 16x16 tiles Z^T[j][i] = K_j . Q_i
// on MFMA with Q's row fragments; the accumulator layout of Z^T (lane: column i, four
// consecutive j) is the A-operand layout of out += W V, so the decay, mask and w are
// applied in registers and W is split into bf16 high and low parts; V's token-axis
// fragments come from the transposing LDS read. dy (fp32) enters the MFMAs split the same
// way (as Q of dC, K of dB and V of dxh); everything accumulates in fp32.
#pragma once

#include <type_traits>

#include "backward.h"

namespace ssd {

enum BwdOp { kOpC = 0, kOpB = 1, kOpX = 2 };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values as packed bf16 high parts (round to nearest even) and packed bf16
// remainders: one packed conversion each, the high parts widened back by bit operations.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    const uint32_t hu = __builtin_bit_cast(uint32_t, h);
    const float ah = __uint_as_float(hu << 16), bh = __uint_as_float(hu & 0xffff0000u);
    hi = hu;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a - ah, b - bh}, bf16x2_t));
}

// Eight fp32 values (two f32x4) as a bf16x8 of high parts and one of remainders.
__device__ __forceinline__ void split8(const f32x4& u, const f32x4& w, bf16x8& hi, bf16x8& lo) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split2(u[0], u[1], h0, l0);
    split2(u[2], u[3], h1, l1);
    split2(w[0], w[1], h2, l2);
    split2(w[2], w[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, (u32x4){h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, (u32x4){l0, l1, l2, l3});
}

template <int OP, int P, int S, int T>
struct BmCfg {
    static constexpr bool REV = OP != kOpC;
    static constexpr int KD = OP == kOpX ? S : P;  // contraction of Q . K and of Q . Z
    static constexpr int N = OP == kOpX ? P : S;   // output width
    // dy (fp32) is the operand split into bf16 high and low parts: Q of dC, K of dB, V of dxh
    static constexpr bool QSPLIT = OP == kOpC, KSPLIT = OP == kOpB, VSPLIT = OP == kOpX;
    // T/32 pairs of row tiles; NSPLIT waves per pair, each taking NNH of the output's 16-wide
    // column tiles (at most 4, so the accumulators leave room for two waves per SIMD)
    static constexpr int NSPLIT = N / 64 > 2 ? N / 64 : 2;
    static constexpr int NIT = T / 16, NW = T / 32, NTHR = 64 * NW * NSPLIT;
    static constexpr int NKS = KD / 32, NNT = N / 16, NNH = NNT / NSPLIT;
    static constexpr int KS = row_stride<bf16>(KD);  // K rows and Z rows (read by rows)
    static constexpr int VS = col_stride<bf16>(N);   // V rows (read by columns)
    static constexpr size_t K_BYTES = (size_t)T * KS * 2;  // each part
    static constexpr size_t V_BYTES = (size_t)T * VS * 2;  // each part
    static constexpr size_t Z_BYTES = (size_t)N * KS * 2;  // each part
    // dxh: x's rows of the head for the epilogue's x . dxh and dy . x (its D dy and dy . x
    // take dy as the sum of its bf16 high and low parts in V, within 2^-17 of dy); the row
    // stride (4 mod 8 words) puts the four rows 4 apart that a read touches on disjoint
    // banks
    static constexpr int XR = row_stride<bf16>(P);
    static constexpr size_t X_BYTES = OP == kOpX ? (size_t)T * XR * 2 : 0;
    // dC, dB: Q's rows of the head (read by rows, like K; dy split into two parts)
    static constexpr size_t Q_BYTES = OP == kOpX ? 0 : (size_t)T * KS * 2 * (QSPLIT ? 2 : 1);
    static constexpr size_t LDS_BYTES = K_BYTES * (KSPLIT ? 2 : 1) + V_BYTES * (VSPLIT ? 2 : 1) +
                                        2 * Z_BYTES + 3 * (size_t)T * 4 +
                                        2 * NSPLIT * (size_t)T * 4 + X_BYTES + Q_BYTES;
    static constexpr bool FITS = LDS_BYTES <= 163840 && KD % 32 == 0 && NNT % NSPLIT == 0;
};

// 8 consecutive values as bf16 (high part) and, for fp32 sources, the bf16 remainders
__device__ __forceinline__ void ld8_split(const bf16* p, bf16x8& hi, bf16x8& lo) {
    hi = *(const bf16x8*)p;
    lo = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
}
__device__ __forceinline__ void ld8_split(const float* p, bf16x8& hi, bf16x8& lo) {
    split8(*(const f32x4*)p, *(const f32x4*)(p + 4), hi, lo);
}

// Rows [0, NROWS) x NCOLS (a multiple of 8) of a row-major source, staged into LDS as bf16
// (and, with SPLIT, the bf16 remainders of fp32 values): load() puts every load of the
// calling thread in flight at once, store() converts and writes after they land. Rows at
// or past `rows` are zero.
template <typename TSrc, int NTHR, int NROWS, int NCOLS, bool SPLIT>
struct Stager {
    static constexpr int PER = NCOLS / 8, NVEC = NROWS * PER;
    static constexpr int NV = (NVEC + NTHR - 1) / NTHR;
    static constexpr bool F32 = sizeof(TSrc) == 4;
    f32x4 raw[F32 ? 2 * NV : NV];
    // Every thread issues the same number of loads, with no branch around them, so that
    // the compiler's waits for later loads count exactly; rows at or past `rows` lie
    // outside the descriptor and read as zeros, as do the slots past the tile (offset
    // 2^31).
    __device__ __forceinline__ void load(const TSrc* src, size_t sstride, int rows, int tid) {
        const BufRsrc rs = make_rsrc(src, (uint32_t)((size_t)rows * sstride * sizeof(TSrc)));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / PER, col = (v % PER) * 8;
            const uint32_t off =
                v < NVEC ? (uint32_t)(((size_t)r * sstride + col) * sizeof(TSrc)) : 0x80000000u;
            if constexpr (F32) {
                raw[2 * i] = __builtin_bit_cast(f32x4, buf_load16(rs, off, 0u));
                raw[2 * i + 1] = __builtin_bit_cast(f32x4, buf_load16(rs, off + 16u, 0u));
            } else {
                raw[i] = __builtin_bit_cast(f32x4, buf_load16(rs, off, 0u));
            }
        }
    }
    // fp32 sources: the values as they are (row stride dstride floats)
    __device__ __forceinline__ void store_f32(float* dst, int dstride, int tid) const {
        static_assert(F32, "fp32 source only");
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NTHR;
            if (v >= NVEC) continue;
            const int r = v / PER, col = (v % PER) * 8;
            *(f32x4*)(dst + r * dstride + col) = raw[2 * i];
            *(f32x4*)(dst + r * dstride + col + 4) = raw[2 * i + 1];
        }
    }
    __device__ __forceinline__ void store(bf16* dst, bf16* dst_lo, int dstride, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NTHR;
            if (v >= NVEC) continue;
            const int r = v / PER, col = (v % PER) * 8;
            if constexpr (F32) {
                bf16x8 hi, lo;
                split8(raw[2 * i], raw[2 * i + 1], hi, lo);
                *(bf16x8*)(dst + r * dstride + col) = hi;
                if constexpr (SPLIT) *(bf16x8*)(dst_lo + r * dstride + col) = lo;
            } else {
                *(f32x4*)(dst + r * dstride + col) = raw[i];
            }
        }
    }
};

// The state [P][S] (fp32) transposed into LDS: Z[s][p], high and low bf16 parts. Each
// thread takes two neighbouring rows p, p + 1 and four columns, so the lanes of a wave
// write consecutive 4-byte words of a Z row (a pair of bf16 values each). The groups of
// four columns are taken in the order 0, 2, 1, 3 within each run of four groups, so that
// at headdim 64 the two halves of a wave write Z rows 8 apart (288 words: disjoint banks)
// rather than 4 apart (144 words: half the banks shared).
__device__ __forceinline__ int col_group(int sg) {
    return (sg & ~3) | ((sg & 1) << 1) | ((sg >> 1) & 1);
}
template <int NTHR, int P, int S>
struct StateTStager {
    static constexpr int NVEC = (P / 2) * (S / 4), NV = (NVEC + NTHR - 1) / NTHR;
    static_assert((S / 4) % 4 == 0, "column groups are permuted in runs of four");
    f32x4 raw[2 * NV];
    __device__ __forceinline__ void load(const float* src, int tid) {
        const BufRsrc rs = make_rsrc(src, (uint32_t)(P * S * sizeof(float)));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NTHR;
            const int p = 2 * (v % (P / 2)), s0 = 4 * col_group(v / (P / 2));
            // unconditional loads (see Stager::load); slots past the state read zeros
            const uint32_t off = v < NVEC ? (uint32_t)((p * S + s0) * sizeof(float)) : 0x80000000u;
            raw[2 * i] = __builtin_bit_cast(f32x4, buf_load16(rs, off, 0u));
            raw[2 * i + 1] = __builtin_bit_cast(f32x4, buf_load16(rs, off + (uint32_t)(S * sizeof(float)), 0u));
        }
    }
    __device__ __forceinline__ void store(bf16* zh, bf16* zl, int ks, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NTHR;
            if (v >= NVEC) continue;
            const int p = 2 * (v % (P / 2)), s0 = 4 * col_group(v / (P / 2));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t hw, lw;
                split2(raw[2 * i][k], raw[2 * i + 1][k], hw, lw);
                *(uint32_t*)(zh + (s0 + k) * ks + p) = hw;
                *(uint32_t*)(zl + (s0 + k) * ks + p) = lw;
            }
        }
    }
};

template <int OP, int P, int S, int T>
__global__ __attribute__((amdgpu_flat_work_group_size(1, BmCfg<OP, P, S, T>::NTHR))) void bwd_mfma_kernel(
    BwdArgs a) {
    using Cfg = BmCfg<OP, P, S, T>;
    constexpr int N = Cfg::N, KD = Cfg::KD, NKS = Cfg::NKS, NNH = Cfg::NNH;
    constexpr int KS = Cfg::KS, VS = Cfg::VS, NTHR = Cfg::NTHR, NIT = Cfg::NIT;
    constexpr bool REV = Cfg::REV, QSPLIT = Cfg::QSPLIT, KSPLIT = Cfg::KSPLIT,
                   VSPLIT = Cfg::VSPLIT;
    constexpr bool SUM = OP != kOpX;  // output summed over the workgroup's heads

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* sp = smem;
    bf16* s_k = (bf16*)sp;                               // [T][KS]
    sp += Cfg::K_BYTES;
    bf16* s_kl = KSPLIT ? (bf16*)sp : nullptr;           // [T][KS] low parts of K
    sp += KSPLIT ? Cfg::K_BYTES : 0;
    bf16* s_v = (bf16*)sp;                               // [T][VS]
    sp += Cfg::V_BYTES;
    bf16* s_vl = VSPLIT ? (bf16*)sp : nullptr;           // [T][VS] low parts of V
    sp += VSPLIT ? Cfg::V_BYTES : 0;
    bf16* s_zh = (bf16*)sp;                              // [N][KS]
    bf16* s_zl = s_zh + N * KS;                          // [N][KS]
    sp += 2 * Cfg::Z_BYTES;
    float* s_g = (float*)sp;                             // [T]
    float* s_dt = s_g + T;                               // [T]
    float* s_u = s_dt + T;                               // [T] per-token decay factors
    float* s_red = s_u + T;                              // [NSPLIT][2][T] row-sum partials
    bf16* s_xr = (bf16*)(s_red + 2 * Cfg::NSPLIT * T);   // dxh: [T][XR] x rows
    bf16* s_q = (bf16*)((unsigned char*)s_xr + Cfg::X_BYTES);  // dC, dB: [T][KS] Q rows
    bf16* s_ql = QSPLIT ? s_q + T * KS : nullptr;        // dC: [T][KS] low parts of Q

    // workgroup: (batch, chunk, block of NH heads of one group)
    const int L = a.L, H = a.H, NG = a.G, NH = a.NH;
    const int nC = (L + T - 1) / T, nhb = H / NH;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = id % nhb, c = (id / nhb) % nC, b = id / (nhb * nC);
    const int h_first = hb * NH;
    const int g = h_first / (H / NG);  // NH divides the heads per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wid % Cfg::NW, part = wid / Cfg::NW;  // row-tile pair, column part
    const int nt0 = part * NNH;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int t0 = c * T, rows = min(T, L - t0);
    const size_t HP = (size_t)H * P, GS = (size_t)NG * S;
    const size_t tok0 = (size_t)b * L + t0;
    const bf16* br = (const bf16*)a.Bm + (tok0 * NG + g) * S;  // stride GS
    const bf16* cr = (const bf16*)a.Cm + (tok0 * NG + g) * S;  // stride GS
    auto xr_of = [&](int h) { return (const bf16*)a.x + (tok0 * H + h) * P; };  // stride HP
    auto dyr_of = [&](int h) { return a.dy + (tok0 * H + h) * P; };             // stride HP
    auto bhl_of = [&](int h) { return ((size_t)b * H + h) * L + t0; };
    auto zsrc_of = [&](int h) {
        return (OP == kOpC ? a.Hc : a.R) + (((size_t)b * H + h) * nC + c) * P * S;
    };

    // ---- staging ----------------------------------------------------------------------
    // Shared by the heads: V = B (dC), V = C (dB), K = C (dxh). Per head: K = x (dC),
    // K = dy (dB), V = dy (dxh), the state Z (high/low bf16), G and dt. The next head's
    // loads are in flight while the current head computes.
    using KSrc = std::conditional_t<OP == kOpB, float, bf16>;
    using VSrc = std::conditional_t<OP == kOpX, float, bf16>;
    using ZStage = std::conditional_t<OP == kOpX, Stager<float, NTHR, P, S, true>,
                                      StateTStager<NTHR, P, S>>;
    Stager<KSrc, NTHR, T, KD, KSPLIT> stk;
    Stager<VSrc, NTHR, T, N, VSPLIT> stv;
    Stager<bf16, NTHR, T, P, false> stx;  // dxh: x rows
    using QSrc = std::conditional_t<OP == kOpC, float, bf16>;
    Stager<QSrc, NTHR, T, KD, QSPLIT> stq;  // dC, dB: Q rows (dy, x)
    ZStage stz;
    // G at this token and at the start (backward in time) or end (forward) of its 16-token
    // tile; u = 2^{G - G_start}, or dt 2^{G_end - G}: the decay from the tile's edge (<= 1)
    float pg = 0.f, pdt = 0.f, pge = 0.f;
    // dxh: D of the head, loaded with its rows (zero when D is absent: a descriptor of no
    // bytes), so that no load outside the prefetch is issued, and waited for, per head
    float pdv = 0.f, dval = 0.f;
    const BufRsrc rD = make_rsrc(a.D, a.D ? (uint32_t)(H * sizeof(float)) : 0u);
    auto load_head = [&](int h) {
        if constexpr (OP == kOpX) pdv = buf_load_f32(rD, (uint32_t)(h * 4), 0u);
        if constexpr (OP == kOpC) stk.load(xr_of(h), HP, rows, tid);
        else if constexpr (OP == kOpB) stk.load(dyr_of(h), HP, rows, tid);
        else stv.load(dyr_of(h), HP, rows, tid);
        if constexpr (OP == kOpX) stx.load(xr_of(h), HP, rows, tid);
        if constexpr (OP == kOpC) stq.load(dyr_of(h), HP, rows, tid);
        if constexpr (OP == kOpB) stq.load(xr_of(h), HP, rows, tid);
        if constexpr (OP == kOpX) stz.load(zsrc_of(h), S, P, tid);
        else stz.load(zsrc_of(h), tid);
        // (every thread loads, those past T harmlessly: no branch around the loads)
        const BufRsrc rg = make_rsrc(a.Gc + bhl_of(h), (uint32_t)(rows * sizeof(float)));
        const BufRsrc rd = make_rsrc(a.dtt + bhl_of(h), (uint32_t)(rows * sizeof(float)));
        const int tt = tid & (T - 1);
        pg = buf_load_f32(rg, (uint32_t)(min(tt, rows - 1) * 4), 0u);
        pdt = buf_load_f32(rd, (uint32_t)(tt * 4), 0u);  // zero past the real tokens
        pge = buf_load_f32(rg, (uint32_t)(min(REV ? (tt & ~15) : (tt | 15), rows - 1) * 4), 0u);
    };
    auto store_head = [&]() {
        dval = pdv;
        if constexpr (OP == kOpX) {
            stv.store(s_v, s_vl, VS, tid);
            stx.store(s_xr, nullptr, Cfg::XR, tid);
        } else {
            stk.store(s_k, s_kl, KS, tid);
            stq.store(s_q, s_ql, KS, tid);
        }
        stz.store(s_zh, s_zl, KS, tid);
        if (tid < T) {
            s_g[tid] = pg;
            s_dt[tid] = pdt;
            s_u[tid] = REV ? exp2_fast(pg - pge) : pdt * exp2_fast(pge - pg);
        }
    };
    if constexpr (OP == kOpC) stv.load(br, GS, rows, tid);
    else if constexpr (OP == kOpB) stv.load(cr, GS, rows, tid);
    else stk.load(cr, GS, rows, tid);
    load_head(h_first);
    if constexpr (OP == kOpX) stk.store(s_k, nullptr, KS, tid);
    else stv.store(s_v, nullptr, VS, tid);
    store_head();
    lds_barrier();

    const uint32_t row0s[2] = {(uint32_t)(wave * 16 + 4 * g4),
                               (uint32_t)((NIT - 1 - wave) * 16 + 4 * g4)};
    // dC: C's values at this lane's output elements (the same for every head)
    float cval[SUM && OP == kOpC ? 2 : 1][NNH][4];
    if constexpr (OP == kOpC) {
        const BufRsrc rc = make_rsrc(cr, (uint32_t)(rows * GS * 2));
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < NNH; ++j) {
                    const uint32_t vc = (row0s[qi] + r) * (uint32_t)(GS * 2) + l16 * 2;
                    const uint16_t cb =
                        __builtin_amdgcn_raw_buffer_load_b16(rc, vc + (nt0 + j) * 32, 0, 0);
                    cval[qi][j][r] = to_f32(__builtin_bit_cast(bf16, cb));
                }
    }
    f32x4 tot[SUM ? 2 : 1][NNH];  // sums over the heads (dC, dB)
#pragma unroll
    for (int qi = 0; qi < (SUM ? 2 : 1); ++qi)
#pragma unroll
        for (int j = 0; j < NNH; ++j) tot[qi][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Q's rows (lane: row I0 + l16, k = 32 ks + 8 g4 + v): for dC (dy, split) and dB (x)
    // staged in LDS with the head's other rows; for dxh B's rows, the same for every head,
    // loaded once for both row tiles. So the head loop issues no loads but the next head's,
    // at its top, and every wait inside a head leaves them in flight (vector-memory
    // operations complete in issue order). Every memory operation of the loop is issued on
    // every path (at the last head the loads repeat the current head and go unused; the
    // per-row sums are stored through descriptors that drop the rows past the chunk), so
    // the compiler's counted waits never fall back to waiting for everything.
    f32x4 qkeep[OP == kOpX ? 2 : 1][OP == kOpX ? NKS : 1];
    if constexpr (OP == kOpX) {
        const BufRsrc rq = make_rsrc(br, (uint32_t)(rows * GS * 2));
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
            const int qrow = (qi == 0 ? wave : NIT - 1 - wave) * 16 + l16;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qkeep[qi][ks] = __builtin_bit_cast(
                    f32x4, buf_load16(rq, (uint32_t)((qrow * GS + ks * 32 + g4 * 8) * 2), 0u));
        }
    }

#pragma unroll 1
    for (int hh = 0; hh < NH; ++hh) {
        const int h = h_first + hh;
        load_head(hh + 1 < NH ? h + 1 : h);
        const float g_end = s_g[T - 1];     // = G at the last real token
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
            const int it = qi == 0 ? wave : NIT - 1 - wave;  // this wave's row tiles
            const int I0 = it * 16;
            const int qrow = I0 + l16;
            Frag<bf16> qf[NKS], ql[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if constexpr (OP == kOpX) {
                    qf[ks].v = __builtin_bit_cast(bf16x8, qkeep[qi][ks]);
                } else {
                    const int o = qrow * KS + ks * 32 + g4 * 8;
                    qf[ks].v = *(const bf16x8*)(s_q + o);
                    if constexpr (QSPLIT) ql[ks].v = *(const bf16x8*)(s_ql + o);
                }
            }
            const uint32_t row0 = row0s[qi];
            f32x4 acc[NNH];  // output columns 16 (nt0 + j) + l16
#pragma unroll
            for (int j = 0; j < NNH; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            // carried-state term Q_i . Z, scaled per row
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int j = 0; j < NNH; ++j) {
                    const int o = ((nt0 + j) * 16 + l16) * KS + ks * 32 + g4 * 8;
                    Frag<bf16> zh, zl;
                    zh.v = *(const bf16x8*)(s_zh + o);
                    zl.v = *(const bf16x8*)(s_zl + o);
                    mma(acc[j], qf[ks], zh);
                    mma(acc[j], qf[ks], zl);
                    if constexpr (QSPLIT) mma(acc[j], ql[ks], zh);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gi = s_g[I0 + 4 * g4 + r];
                const float sc = exp2_fast(REV ? g_end - gi : gi);
#pragma unroll
                for (int j = 0; j < NNH; ++j) acc[j][r] *= sc;
            }
            // intra-chunk term over 32-wide blocks of j
            const float gi = s_g[qrow];
            const int jp_lo = REV ? it / 2 : 0, jp_hi = REV ? NIT / 2 - 1 : it / 2;
#pragma unroll 1
            for (int jp = jp_lo; jp <= jp_hi; ++jp) {
                const int J0 = jp * 32;
                f32x4 zt[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int o = (J0 + jt * 16 + l16) * KS + ks * 32 + g4 * 8;
                        Frag<bf16> kf;
                        kf.v = *(const bf16x8*)(s_k + o);
                        mma(zt[jt], kf, qf[ks]);
                        if constexpr (QSPLIT) mma(zt[jt], kf, ql[ks]);
                        if constexpr (KSPLIT) {
                            kf.v = *(const bf16x8*)(s_kl + o);
                            mma(zt[jt], kf, qf[ks]);
                        }
                    }
                // W[i][j] in the A-operand layout (row i = qrow, item 4 jt + r <-> j), split
                // into bf16 high and low parts. Off the diagonal tile the decay is a row
                // factor (one exp) times the staged per-token factor u_j, both <= 1; on it
                // each element is exact, with the causal mask; tiles on the far side of
                // the diagonal are zero.
                // (dB keeps the per-element form everywhere: the factored form's extra
                // branches push its registers past the two-waves-per-SIMD budget.)
                Frag<bf16> wf, wl;
                uint32_t wh[4], wlo[4];
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    const int tj = jp * 2 + jt;  // j-tile (wave-uniform, as is it)
                    const int jb = J0 + jt * 16 + 4 * g4;
                    f32x4 w4 = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (OP == kOpB || tj == it) {
                        const f32x4 gj = *(const f32x4*)(s_g + jb);
                        f32x4 wj = f32x4{1.f, 1.f, 1.f, 1.f};
                        if constexpr (!REV) wj = *(const f32x4*)(s_dt + jb);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool keep = REV ? jb + r >= qrow : jb + r <= qrow;
                            const float e = exp2_fast(REV ? gj[r] - gi : gi - gj[r]);
                            w4[r] = keep ? e * wj[r] * zt[jt][r] : 0.f;
                        }
                    } else if (REV ? tj > it : tj < it) {
                        const float gref = s_g[J0 + jt * 16 + (REV ? 0 : 15)];
                        const float rr = exp2_fast(REV ? gref - gi : gi - gref);
                        const f32x4 u4 = *(const f32x4*)(s_u + jb);
#pragma unroll
                        for (int r = 0; r < 4; ++r) w4[r] = (rr * u4[r]) * zt[jt][r];
                    }
                    split2(w4[0], w4[1], wh[2 * jt], wlo[2 * jt]);
                    split2(w4[2], w4[3], wh[2 * jt + 1], wlo[2 * jt + 1]);
                }
                wf.v = __builtin_bit_cast(bf16x8, (u32x4){wh[0], wh[1], wh[2], wh[3]});
                wl.v = __builtin_bit_cast(bf16x8, (u32x4){wlo[0], wlo[1], wlo[2], wlo[3]});
#pragma unroll
                for (int j = 0; j < NNH; ++j) {
                    const int n0 = (nt0 + j) * 16;
                    Frag<bf16> vf;
                    vf.v = __builtin_shufflevector(lds_col4(s_v, VS, J0 + 4 * g4, n0, lane),
                                                   lds_col4(s_v, VS, J0 + 16 + 4 * g4, n0, lane),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
                    mma(acc[j], wf, vf);
                    mma(acc[j], wl, vf);
                    if constexpr (VSPLIT) {
                        vf.v = __builtin_shufflevector(
                            lds_col4(s_vl, VS, J0 + 4 * g4, n0, lane),
                            lds_col4(s_vl, VS, J0 + 16 + 4 * g4, n0, lane), 0, 1, 2, 3, 4, 5,
                            6, 7);
                        mma(acc[j], wf, vf);
                    }
                }
            }
            // ---- this head's contribution: element (row I0 + 4 g4 + r, column
            // 16 (nt0 + j) + l16) of the tile
            float red[4] = {0.f, 0.f, 0.f, 0.f}, red2[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (OP == kOpC) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < NNH; ++j) {
                        red[r] += acc[j][r] * cval[qi][j][r];
                        tot[qi][j][r] += acc[j][r];
                    }
            } else if constexpr (OP == kOpB) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dti = s_dt[row0 + r];
#pragma unroll
                    for (int j = 0; j < NNH; ++j) tot[qi][j][r] += dti * acc[j][r];
                }
            } else {
                // rows sit in the per-lane offset, the head in the uniform one; rows of a
                // partial chunk past its real tokens fall outside the descriptors
                const BufRsrc rdx = make_rsrc(a.dx + tok0 * HP, (uint32_t)(rows * HP * 4));
                const uint32_t hp4 = (uint32_t)(HP * 4), soff4 = (uint32_t)(h * P * 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t vo = (row0 + r) * hp4 + l16 * 4;
                    const float dtr = s_dt[row0 + r];
#pragma unroll
                    for (int j = 0; j < NNH; ++j) {
                        const int nt = nt0 + j;
                        const float o = acc[j][r];
                        const int e = (row0 + r) * VS + nt * 16 + l16;
                        const float dyv = to_f32(s_v[e]) + to_f32(s_vl[e]);
                        const float xv = to_f32(s_xr[(row0 + r) * Cfg::XR + nt * 16 + l16]);
                        buf_store_f32(dval * dyv + dtr * o, rdx, vo + nt * 64, soff4);
                        red[r] += xv * o;
                        red2[r] += xv * dyv;
                    }
                }
            }
            if constexpr (OP != kOpB) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma unroll
                    for (int m = 1; m < 16; m <<= 1) {
                        red[r] += __shfl_xor(red[r], m, 64);
                        if constexpr (OP == kOpX) red2[r] += __shfl_xor(red2[r], m, 64);
                    }
                    // this part's partial row sums; the parts are added below
                    if (l16 == 0) {
                        s_red[(part * 2) * T + row0 + r] = red[r];
                        s_red[(part * 2 + 1) * T + row0 + r] = red2[r];
                    }
                }
            }
        }
        lds_barrier();  // every wave is done with this head's LDS and partials
        if constexpr (OP != kOpB) {
            const size_t bhl = bhl_of(h);
            const int tt = tid & (T - 1);
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int q = 0; q < Cfg::NSPLIT; ++q) {
                s0 += s_red[(2 * q) * T + tt];
                s1 += s_red[(2 * q + 1) * T + tt];
            }
            const uint32_t off = tid < rows ? (uint32_t)(tid * 4) : 0x80000000u;
            const uint32_t nb = (uint32_t)(rows * 4);
            if constexpr (OP == kOpC) {
                buf_store_f32(s0, make_rsrc(a.q + bhl, nb), off, 0u);
            } else {
                buf_store_f32(s0, make_rsrc(a.v + bhl, nb), off, 0u);
                buf_store_f32(s1, make_rsrc(a.dyx + bhl, nb), off, 0u);
            }
        }
        if (hh + 1 < NH) store_head();
        lds_barrier();
    }

    // ---- dC, dB: the sum over this workgroup's heads, [B, L, H / NH, S] (the output itself
    // when the workgroup holds all heads of its group)
    if constexpr (SUM) {
        float* outp = (OP == kOpC ? a.dCh : a.dBh) + tok0 * nhb * S;
        const BufRsrc ro = make_rsrc(outp, (uint32_t)(rows * nhb * S * 4));
        const uint32_t hs4 = (uint32_t)(nhb * S * 4), soff = (uint32_t)(hb * S * 4);
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t vo = (row0s[qi] + r) * hs4 + l16 * 4;
#pragma unroll
                for (int j = 0; j < NNH; ++j)
                    buf_store_f32(tot[qi][j][r], ro, vo + (nt0 + j) * 64, soff);
            }
    }
}

// ---- per-chunk sums for the reverse carry: dR_c = sum_t 2^{G_t} dy_t C_t^T -------------
// One workgroup of T/32 waves per (batch, chunk, block of `nhr` heads of one group). The
// group's C rows are staged in LDS once; per head the rows 2^{G_t} dy_t (fp32, split into
// bf16 high and low parts) are written to LDS as [t][.], and the next head's rows load
// into registers while the current head's products run. Each output tile [16 p x 16 s]
// contracts over the chunk's tokens with both operands read down the token axis by the
// transposing LDS read (token slot (g, v) <-> t = 4 g + v, 16 + 4 g + v - 4 in each
// 32-token step, the same for both operands). Every load and store is issued on every
// path (rows past the chunk read zeros through the descriptors; the last head re-loads
// its own rows), so the compiler's waits stay counted.
template <int P, int S, int T>
struct DrCfg {
    static constexpr int NW = T / 32, NTHR = 64 * NW;
    static constexpr int YS = col_stride<bf16>(P), CS = col_stride<bf16>(S);
    static constexpr size_t Y_BYTES = (size_t)T * YS * 2;  // each part
    static constexpr size_t C_BYTES = (size_t)T * CS * 2;
    static constexpr size_t LDS_BYTES = 2 * Y_BYTES + C_BYTES;
    static constexpr bool FITS = LDS_BYTES <= 163840 && P % 16 == 0 && S % 16 == 0;
};

template <int P, int S, int T>
__global__ __launch_bounds__(2 * T) void bwd_dR_mfma_kernel(BwdArgs a, int nhr) {
    using Cfg = DrCfg<P, S, T>;
    constexpr int YS = Cfg::YS, CS = Cfg::CS, NTHR = Cfg::NTHR, NW = Cfg::NW;
    constexpr int NPT = P / 16, NST = S / 16, NTILE = NPT * NST;
    // whole loops with compile-time trip counts, so the compiler counts the stores issued
    // after the next head's loads and its waits for those loads leave the stores in flight
    static_assert(NTILE % NW == 0, "tiles per wave");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16* s_yh = (bf16*)smem;                              // [T][YS]
    bf16* s_yl = (bf16*)(smem + Cfg::Y_BYTES);             // [T][YS]
    bf16* s_c = (bf16*)(smem + 2 * Cfg::Y_BYTES);          // [T][CS]

    const int L = a.L, H = a.H, NG = a.G;
    const int nC = (L + T - 1) / T, nhb = H / nhr;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = id % nhb, c = (id / nhb) % nC, b = id / (nhb * nC);
    const int h_first = hb * nhr;
    const int g = h_first / (H / NG);  // nhr divides the heads per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int t0 = c * T, rows = min(T, L - t0);
    const size_t HP = (size_t)H * P, GS = (size_t)NG * S;
    const size_t tok0 = (size_t)b * L + t0;
    const bf16* cr = (const bf16*)a.Cm + (tok0 * NG + g) * S;

    // one head's rows of dy (fp32) and its per-token log2 decays G_t, in registers
    constexpr int PER = P / 8, NVY = T * PER / NTHR;
    static_assert(T * PER % NTHR == 0, "dy vectors per thread");
    f32x4 ry[2 * NVY];
    float wt[NVY];
    auto load_dy = [&](int h) {
        const BufRsrc rd = make_rsrc(a.dy + (tok0 * H + h) * P, (uint32_t)(rows * HP * 4));
        const BufRsrc rg = make_rsrc(a.Gc + ((size_t)b * H + h) * L + t0, (uint32_t)(rows * 4));
#pragma unroll
        for (int i = 0; i < NVY; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / PER, col = (v % PER) * 8;
            const uint32_t o = (uint32_t)((r * HP + col) * 4);
            ry[2 * i] = __builtin_bit_cast(f32x4, buf_load16(rd, o, 0u));
            ry[2 * i + 1] = __builtin_bit_cast(f32x4, buf_load16(rd, o + 16u, 0u));
            wt[i] = buf_load_f32(rg, (uint32_t)(r * 4), 0u);
        }
    };
    Stager<bf16, NTHR, T, S, false> stc;
    stc.load(cr, GS, rows, tid);
    load_dy(h_first);
    stc.store(s_c, nullptr, CS, tid);

#pragma unroll 1
    for (int hh = 0; hh < nhr; ++hh) {
        const int h = h_first + hh;
        if (hh > 0) lds_barrier();  // every wave is done with the previous head's rows
        // the weighted split: 2^{G_t} dy_t as bf16 high and low parts
#pragma unroll
        for (int i = 0; i < NVY; ++i) {
            const int v = tid + i * NTHR;
            const int r = v / PER, col = (v % PER) * 8;
            const float w = exp2_fast(wt[i]);
            bf16x8 hi, lo;
            split8(w * ry[2 * i], w * ry[2 * i + 1], hi, lo);
            *(bf16x8*)(s_yh + r * YS + col) = hi;
            *(bf16x8*)(s_yl + r * YS + col) = lo;
        }
        lds_barrier();
        load_dy(hh + 1 < nhr ? h + 1 : h);  // in flight during this head's products
        // (kept ahead of the products and stores: the scheduler would otherwise sink the
        // loads among the stores, and the wait for them at the next head would then wait
        // for this head's stores as well)
        __builtin_amdgcn_sched_barrier(0);

        const BufRsrc ro = make_rsrc(a.R + (((size_t)b * H + h) * nC + c) * P * S,
                                     (uint32_t)(P * S * 4));
#pragma unroll
        for (int k = 0; k < NTILE / NW; ++k) {
            const int tile = wave + k * NW;
            const int p0 = (tile / NST) * 16, s0 = (tile % NST) * 16;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < T; k0 += 32) {
                Frag<bf16> yh, yl, cf;
                yh.v = __builtin_shufflevector(lds_col4(s_yh, YS, k0 + 4 * g4, p0, lane),
                                               lds_col4(s_yh, YS, k0 + 16 + 4 * g4, p0, lane),
                                               0, 1, 2, 3, 4, 5, 6, 7);
                yl.v = __builtin_shufflevector(lds_col4(s_yl, YS, k0 + 4 * g4, p0, lane),
                                               lds_col4(s_yl, YS, k0 + 16 + 4 * g4, p0, lane),
                                               0, 1, 2, 3, 4, 5, 6, 7);
                cf.v = __builtin_shufflevector(lds_col4(s_c, CS, k0 + 4 * g4, s0, lane),
                                               lds_col4(s_c, CS, k0 + 16 + 4 * g4, s0, lane),
                                               0, 1, 2, 3, 4, 5, 6, 7);
                mma(acc, yh, cf);
                mma(acc, yl, cf);
            }
            // element (row p0 + 4 g4 + r, column s0 + l16)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                buf_store_f32(acc[r], ro, (uint32_t)(((p0 + 4 * g4 + r) * S + s0 + l16) * 4), 0u);
        }
    }
}

// Heads per dR workgroup: the largest divisor of the heads per group that leaves at least
// two workgroups per compute unit (512), so C's rows are staged once for that many heads.
inline int dr_heads_per_block(int batch, int nC, int H, int hpg) {
    int best = 1;
    for (int d = 1; d <= hpg; ++d)
        if (hpg % d == 0 && (long)batch * nC * (H / d) >= 512) best = d;
    return best;
}

template <int P, int S, int T>
hipError_t run_bwd_dR_mfma(const BwdArgs& a, int batch, hipStream_t stream) {
    using Cfg = DrCfg<P, S, T>;
    auto kern = bwd_dR_mfma_kernel<P, S, T>;
    if (Cfg::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)Cfg::LDS_BYTES);
        if (e != hipSuccess) return e;
    }
    const int nC = (a.L + T - 1) / T;
    const int nhr = dr_heads_per_block(batch, nC, a.H, a.H / a.G);
    kern<<<batch * nC * (a.H / nhr), 2 * T, Cfg::LDS_BYTES, stream>>>(a, nhr);
    return hipGetLastError();
}

template <int OP, int P, int S, int T>
hipError_t run_bwd_mfma(const BwdArgs& a, int batch, hipStream_t stream) {
    using Cfg = BmCfg<OP, P, S, T>;
    auto kern = bwd_mfma_kernel<OP, P, S, T>;
    if (Cfg::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)Cfg::LDS_BYTES);
        if (e != hipSuccess) return e;
    }
    const int nC = (a.L + T - 1) / T;
    kern<<<batch * nC * (a.H / a.NH), Cfg::NTHR, Cfg::LDS_BYTES, stream>>>(a);
    return hipGetLastError();
}

template <int P, int S, int T>
constexpr bool bwd_mfma_fits() {
    return BmCfg<kOpC, P, S, T>::FITS && BmCfg<kOpB, P, S, T>::FITS &&
           BmCfg<kOpX, P, S, T>::FITS && DrCfg<P, S, T>::FITS;
}

template <int P, int S, int T>
hipError_t run_bwd_mfma_all(const BwdArgs& a, int batch, hipStream_t st) {
    hipError_t e = run_bwd_mfma<kOpC, P, S, T>(a, batch, st);
    if (e == hipSuccess) e = run_bwd_mfma<kOpB, P, S, T>(a, batch, st);
    if (e == hipSuccess) e = run_bwd_mfma<kOpX, P, S, T>(a, batch, st);
    return e;
}

}  // namespace ssd
