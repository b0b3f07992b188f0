// Stage 2 in one pass: the chunk-initial states by a sequential scan over chunks, with each
// chunk's own contribution formed on the fly (kernel template for bf16 inputs; instances
// in k_state_scan_bf16*.hip). An alternative to the chunk_state + state_carry pair for
// shapes with many (batch, head) pairs and whole chunks only (seqlen a multiple of the
// chunk length).
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Kernel 2: fwd_pass_state": one program walks the chunks of a sequence in
// order, keeps the running state on chip, records it as the state entering each chunk,
// and advances it by the jump formula (section "Mamba-2 architecture"):
//     S_{c+1}[p][s] = 2^{g_c} S_c[p][s] + sum_{j in chunk c} x_j[p] (dt_j 2^{G_last - G_j} B_j[s])
// where g_c is the chunk's total log2 decay. Both exponents are summed from the chunk's
// end, so their rounding is relative to the terms that dominate the state.
//
// gfx950 mapping. One workgroup of 8 waves per (batch, head, slice of PT rows of the
// head dimension); the running state lives in the waves' MFMA accumulator layout in fp32
// registers for the whole sequence and never goes to HBM except as the recorded per-chunk
// states and the final state. Tokens stream through LDS in sub-blocks of TB rows (x slice
// and the group's B rows), double-buffered: the next sub-block's 16-byte global loads are
// in flight while the current one's products run, with one barrier per sub-block. The
// contraction over tokens is dS^T = (w o B)^T x on bf16 MFMA (16x16x32): both operands
// come from the transposing LDS read (tokens along K). The fused operand w_j B_j[s] is
// formed in fp32 and split into a bf16 high part and a bf16 remainder (two MFMAs against
// the exact bf16 x), which keeps about 16 significant bits. The accumulator holds four
// consecutive state columns s of one row p per lane, so every recorded state leaves as
// one 8- or 16-byte store per lane. Wave 0 forms the next chunk's weights with a
// single-wave DPP suffix scan while the other waves finish the current chunk.
#pragma once

#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// Position of 16-byte granule q of row r in an unpadded bf16 LDS tile with GR granules per
// row. The tiles are read by ds_read_b64_tr_b16, where 32 lanes read 8 consecutive rows x
// 2 granules (an aligned pair); XOR-ing the pair index with a per-row value spreads those
// 16 granules over all 64 banks.
template <int GR>
__device__ __forceinline__ int swz(int r) {
    constexpr int RPL = GR >= 16 ? 1 : 16 / GR;  // rows per 256-byte bank line
    constexpr int MASK = (GR >= 16 ? 16 : GR) / 2 - 1;
    return 2 * ((r / RPL) & MASK);
}

// Byte offset, within a swizzled bf16 tile of GR granules per row, of the 8 bytes that
// lane s of a 16-lane group supplies to a transposing read (ds_read_b64_tr_b16) of rows
// r0 .. r0+3 and columns c0 .. c0+15: lane j then receives column c0 + j of those rows.
template <int GR>
__device__ __forceinline__ uint32_t tr_off(int r0, int c0, int lane) {
    const int s = lane & 15;
    const int r = r0 + (s >> 2);
    const int q = (c0 >> 3) + ((s & 3) >> 1);
    return (uint32_t)((r * GR + (q ^ swz<GR>(r))) * 16 + 8 * (s & 1));
}

__device__ __forceinline__ bf16x4 lds_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(__attribute__((address_space(3))) bf16*)(const bf16*)p);
}

// s_waitcnt that waits until at most N vector-memory operations of this wave are
// outstanding (gfx9 encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same wait with a wave-uniform count n (LO .. HI): a binary search over the
// immediates, scalar branches only.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_upto(int n) {
    if constexpr (LO == HI) {
        wait_vm<LO>();
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n <= MID) wait_vm_upto<LO, MID>(n);
        else wait_vm_upto<MID + 1, HI>(n);
    }
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane l
// writes lds + 16 l, where `lds` (wave-uniform) goes through M0. Written as inline
// assembly so that the compiler, which cannot tell which LDS bytes the copy writes, does
// not drain every copy in flight before each LDS read; completion is tracked by hand
// with wait_vm. M0 is restored afterwards; s_nop covers the M0-to-LDS-DMA hazard.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
    const uint32_t l = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l), "v"(src)
        : "memory");
}

template <typename TIn, typename TS, int P, int S, int T, int PT, int TB, int R>
struct ScanCfg {
    static constexpr int NTHR = 512, NWAVE = 8;
    static constexpr int NPT = PT / 16, NST = S / 16;
    // Waves split the row tiles p of the slice; the WPT waves that share a row tile split
    // its column tiles s. Each wave forms the weighted x operand of its own row tiles
    // once per step and reuses it for all of its column tiles.
    static constexpr bool ROWS = NPT >= NWAVE;
    static constexpr int MP = ROWS ? NPT / NWAVE : 1;     // row tiles per wave
    static constexpr int WPT = ROWS ? 1 : NWAVE / NPT;    // waves per row tile
    static constexpr int MS = ROWS ? NST : (NST + WPT - 1) / WPT;  // column tiles per wave
    static constexpr bool EVEN = ROWS || NST % WPT == 0;  // every wave has MS column tiles
    static constexpr int ES = (int)sizeof(TIn), VE = 16 / ES;
    static constexpr int GRX = PT * ES / 16, GRB = S * ES / 16;  // granules per row
    static constexpr int SLOT_X = TB * GRX, SLOT_B = TB * GRB;    // granules per slot
    static constexpr int NI_X = SLOT_X / 64, NI_B = SLOT_B / 64;  // 1 KiB wave loads
    static constexpr int NI = NI_X + NI_B;
    static constexpr int N_HI = (NI + NWAVE - 1) / NWAVE, N_LO = NI / NWAVE;
    static constexpr int KB = T / TB;   // sub-blocks per chunk
    static constexpr int PER = T / 64;  // tokens per lane in the weight scan
    static constexpr size_t SLOT_BYTES = (size_t)(SLOT_X + SLOT_B) * 16;
    static constexpr size_t W_OFF = (size_t)R * SLOT_BYTES;
    static constexpr size_t DT_OFF = W_OFF + 2 * (size_t)T * sizeof(float);
    static constexpr size_t G_OFF = DT_OFF + (size_t)R * T * sizeof(float);
    static constexpr size_t LDS_BYTES = G_OFF + 2 * 16;
    static constexpr bool FITS = LDS_BYTES <= 163840 && PT <= P && TB <= T &&
                                 SLOT_X % 64 == 0 && SLOT_B % 64 == 0 && R >= 2 &&
                                 N_HI * (R - 2) < 64 && T * 4 <= 1024;
};

template <typename TIn, typename TS, int P, int S, int T, int PT, int TB, int R>
__global__ __launch_bounds__(512) void state_scan_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ dt_t, const float* __restrict__ h0, TS* __restrict__ states,
    float* __restrict__ final_state, int L, int H, int ngroups) {
    static_assert(sizeof(TIn) == 2, "bf16 inputs only");
    using Cfg = ScanCfg<TIn, TS, P, S, T, PT, TB, R>;
    constexpr int VE = Cfg::VE, PER = Cfg::PER, GRX = Cfg::GRX, GRB = Cfg::GRB;
    constexpr int MS = Cfg::MS, MP = Cfg::MP, KB = Cfg::KB, NI = Cfg::NI, NI_X = Cfg::NI_X;
    constexpr int NP = P / PT;
    constexpr uint32_t XK = 32 * GRX * 16, BK = 32 * GRB * 16;  // bytes per 32 rows
    constexpr uint32_t B0 = Cfg::SLOT_X * 16;                    // B tile within a slot

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    auto slot = [&](int k) { return smem + (size_t)k * Cfg::SLOT_BYTES; };
    auto s_w = [&](int k) { return (float*)(smem + Cfg::W_OFF + k * T * sizeof(float)); };
    auto s_dt = [&](int c) { return (float*)(smem + Cfg::DT_OFF + (c % R) * T * sizeof(float)); };
    float* s_g = (float*)(smem + Cfg::G_OFF);  // [2] chunk log2 decays (16-byte slots)

    const int nC = L / T;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int pp = id % NP;
    const int h = (id / NP) % H;
    const int b = id / (NP * H);
    const int g = h / (H / ngroups);
    const int p0 = pp * PT;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;

    // this wave's tiles: row tiles p_tile(m) (within the slice), column tiles s_tile(m)
    auto p_tile = [&](int m) { return Cfg::ROWS ? wave * MP + m : wave % Cfg::NPT; };
    auto s_tile = [&](int m) { return Cfg::ROWS ? m : wave / Cfg::NPT + Cfg::WPT * m; };
    auto s_ok = [&](int m) { return Cfg::EVEN || s_tile(m) < Cfg::NST; };

    const size_t xrow = (size_t)H * P, brow = (size_t)ngroups * S;
    const TIn* xb = x + ((size_t)b * L * H + h) * P + p0;
    const TIn* bb = Bm + ((size_t)b * L * ngroups + g) * S;
    const float* dtb = dt_t + ((size_t)b * H + h) * L;
    const size_t bh = (size_t)b * H + h;
    const float ah = A[h];

    // running state, accumulator layout: (s = 16 s_tile + 4 g4 + r, p = p0 + 16 p_tile + l16)
    f32x4 st[MS][MP], acc[MS][MP];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int mp = 0; mp < MP; ++mp) {
            acc[ms][mp] = f32x4{0.f, 0.f, 0.f, 0.f};
            st[ms][mp] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (h0 && s_ok(ms)) {
                const int p = p0 + 16 * p_tile(mp) + l16, s = 16 * s_tile(ms) + 4 * g4;
                st[ms][mp] = *(const f32x4*)(h0 + (bh * P + p) * S + s);
            }
            // consume the loaded state here, so the compiler's wait for these loads comes
            // before the scan rather than inside it
            asm volatile("" ::"v"(st[ms][mp]));
        }

    const int N_SUB = nC * KB;  // sub-blocks in the sequence
    // sub-block s2 is the last of its chunk and the next chunk's dt is loaded with it
    auto has_dt = [&](int s2) { return (s2 + 1) % KB == 0 && (s2 + 1) / KB < nC; };

    // ---- per-lane offsets, fixed for the whole scan ------------------------------------
    // global element offset of each of this wave's 1 KiB loads (load j = wave + 8 m fills
    // slot granules 64 j .. 64 j + 63; lane l granule 64 j + l), relative to sub-block 0
    uint32_t doff[Cfg::N_HI];
#pragma unroll
    for (int m = 0; m < Cfg::N_HI; ++m) {
        const int j = wave + Cfg::NWAVE * m;
        doff[m] = 0;
        if (j < NI_X) {
            const int gpos = j * 64 + lane, r = gpos / GRX, pos = gpos % GRX;
            doff[m] = (uint32_t)(r * xrow + (pos ^ swz<GRX>(r)) * VE);
        } else if (j < NI) {
            const int gpos = (j - NI_X) * 64 + lane, r = gpos / GRB, pos = gpos % GRB;
            doff[m] = (uint32_t)(r * brow + (pos ^ swz<GRB>(r)) * VE);
        }
    }
    // LDS byte offsets of this lane's transposing reads at k-step 0 (k-step ks adds ks*XK
    // or ks*BK: the swizzle repeats every 32 rows)
    uint32_t xo[MP][2], bo[MS][2];
#pragma unroll
    for (int mp = 0; mp < MP; ++mp)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) xo[mp][hh] = tr_off<GRX>(4 * g4 + 16 * hh, 16 * p_tile(mp), lane);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            bo[ms][hh] = B0 + tr_off<GRB>(4 * g4 + 16 * hh, s_ok(ms) ? 16 * s_tile(ms) : 0, lane);

    // ---- sub-block i (tokens i*TB ..) straight from global memory into ring slot i % R --
    auto issue_dt = [&](int c) {  // dt of chunk c, T fp32 values, by wave 0
        if (wave == 0 && lane < T / 4) dma16(dtb + (size_t)c * T + 4 * lane, s_dt(c));
    };
    auto issue = [&](int i) {
        // the next chunk's dt goes ahead of a chunk's last sub-block, so the wait for that
        // sub-block also covers it
        if (has_dt(i)) issue_dt((i + 1) / KB);
        unsigned char* sl = slot(i % R);
        const size_t t0 = (size_t)i * TB;
        const TIn* xt = xb + t0 * xrow;
        const TIn* bt = bb + t0 * brow;
#pragma unroll
        for (int m = 0; m < Cfg::N_HI; ++m) {
            const int j = wave + Cfg::NWAVE * m;
            if (j < NI) dma16((j < NI_X ? xt : bt) + doff[m], sl + j * 1024);
        }
    };
    // Wait until this wave's loads of sub-block i are done. Vector-memory operations
    // complete in issue order, so everything this wave issued after them may stay in
    // flight: the loads of the later sub-blocks already issued (R-2 of them, fewer at the
    // end), the dt loads issued with those, and the state stores of the chunk ends passed
    // since sub-block i was issued (in iteration i-R+1, ahead of that iteration's stores).
    const int n_ld = (wave < NI % Cfg::NWAVE || NI % Cfg::NWAVE == 0) ? Cfg::N_HI : Cfg::N_LO;
    int n_st = 0;  // state stores per chunk end (one 8- or 16-byte store per tile)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) n_st += s_ok(ms) ? MP : 0;
    auto wait_for = [&](int i) {
        const int later = min(R - 2, N_SUB - 1 - i);
        int n = n_ld * later;
        if (wave == 0)
            for (int s2 = i + 1; s2 <= i + later; ++s2) n += has_dt(s2) ? 1 : 0;
        for (int j = max(0, i - R + 1); j < i; ++j) n += ((j + 1) % KB == 0) ? n_st : 0;
        wait_vm_upto<0, 63>(min(n, 63));
    };

    // ---- per-chunk weights (wave 0): lane holds tokens T-1-(PER*lane+k) -------------------
    auto make_w = [&](int c) {
        if (wave == 0) {
            const float* dtc = s_dt(c);
            float pdt[PER];
#pragma unroll
            for (int k = 0; k < PER; ++k) pdt[k] = dtc[T - 1 - (PER * lane + k)];
            // w_t = dt_t 2^{log2(e) sum_{k>t} A dt_k}; the chunk's decay sums every token
            float pre[PER], run = 0.f;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                pre[k] = run;
                run += ah * pdt[k];
            }
            const float incl = wave_inclusive_scan(run);
            const float excl = wave_shift_up1(incl);
            float* bw = s_w(c & 1);
#pragma unroll
            for (int k = 0; k < PER; ++k)
                bw[T - 1 - (PER * lane + k)] = pdt[k] * exp2_fast((excl + pre[k]) * kLog2e);
            const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
            if (lane == 0) s_g[(c & 1) * 4] = total * kLog2e;
        }
    };

    // ---- one sub-block's products: acc += B^T (w o x) over its TB tokens ----------------
    auto compute = [&](int i, int c, int k) {
        const unsigned char* sl = slot(i % R);
        const float* sw = s_w(c & 1) + k * TB + 4 * g4;
#pragma unroll
        for (int ks = 0; ks < TB / 32; ++ks) {
            // slot (g4, v) carries token 32 ks + 16 (v/4) + 4 g4 + v%4 (two column reads)
            const f32x4 w_lo = *(const f32x4*)(sw + ks * 32);
            const f32x4 w_hi = *(const f32x4*)(sw + ks * 32 + 16);
            Frag<bf16> hi[MP], lo[MP];
#pragma unroll
            for (int mp = 0; mp < MP; ++mp) {
                const bf16x4 a = lds_tr(sl + xo[mp][0] + ks * XK);
                const bf16x4 q = lds_tr(sl + xo[mp][1] + ks * XK);
                float xw[8];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    xw[v] = to_f32(a[v]) * w_lo[v];
                    xw[v + 4] = to_f32(q[v]) * w_hi[v];
                }
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    hi[mp].v[v] = from_f32<bf16>(xw[v]);
                    lo[mp].v[v] = from_f32<bf16>(xw[v] - to_f32(hi[mp].v[v]));
                }
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                if (s_ok(ms)) {
                    Frag<bf16> bf;
                    const bf16x4 a = lds_tr(sl + bo[ms][0] + ks * BK);
                    const bf16x4 q = lds_tr(sl + bo[ms][1] + ks * BK);
                    bf.v = __builtin_shufflevector(a, q, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int mp = 0; mp < MP; ++mp) {
                        mma(acc[ms][mp], bf, hi[mp]);
                        mma(acc[ms][mp], bf, lo[mp]);
                    }
                }
            }
        }
    };

    // ---- record the running state (fp32 accumulator layout) to `dst` --------------------
    auto store_state = [&](auto* dst) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int mp = 0; mp < MP; ++mp) {
                if (!s_ok(ms)) continue;
                const int p = p0 + 16 * p_tile(mp) + l16, s = 16 * s_tile(ms) + 4 * g4;
                const f32x4 v = st[ms][mp];
                if constexpr (sizeof(*dst) == 2) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = from_f32<bf16>(v[r]);
                    *(bf16x4*)(dst + (size_t)p * S + s) = o;
                } else {
                    *(f32x4*)(dst + (size_t)p * S + s) = v;
                }
            }
    };

    // ---- the scan ---------------------------------------------------------------------
    // Iteration i: wait for sub-block i, barrier (every wave is done with sub-block i-1,
    // whose slot the next issue reuses), issue sub-block i+R-1, compute sub-block i.
    const int N = N_SUB;
    issue_dt(0);
    wait_vm<0>();
    make_w(0);
    for (int i = 0; i < R - 1 && i < N; ++i) issue(i);
    for (int i = 0; i < N; ++i) {
        const int c = i / KB, k = i - c * KB;
        wait_for(i);
        lds_barrier();
        if (i + R - 1 < N) issue(i + R - 1);
        compute(i, c, k);
        if (k == KB - 1) {
            store_state(states + (bh * nC + c) * (size_t)P * S);
            const float decay = exp2_fast(s_g[(c & 1) * 4]);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int mp = 0; mp < MP; ++mp) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) st[ms][mp][r] = decay * st[ms][mp][r] + acc[ms][mp][r];
                    acc[ms][mp] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            if (c + 1 < nC) make_w(c + 1);  // into the other weight buffer
        }
    }
    if (final_state) store_state(final_state + bh * (size_t)P * S);
}

// ---- plans and launch -------------------------------------------------------------------
// Sub-block length and ring depth: 128 tokens (capped by the chunk) in 3 slots, shorter
// sub-blocks where that ring does not fit in LDS.
struct ScanPlan {
    int tb, ring;
};

template <typename TS, int P, int S, int T, int PT>
constexpr ScanPlan scan_plan() {
    constexpr int tb0 = T < 128 ? T : 128;
    if constexpr (ScanCfg<bf16, TS, P, S, T, PT, tb0, 3>::FITS) return {tb0, 3};
    else if constexpr (ScanCfg<bf16, TS, P, S, T, PT, 64, 3>::FITS) return {64, 3};
    else if constexpr (ScanCfg<bf16, TS, P, S, T, PT, 32, 3>::FITS) return {32, 3};
    else return {32, 2};
}

// Rows of the head dimension per workgroup: 64, or 32 where 64-row slices would leave
// compute units without a workgroup.
inline int scan_rows_per_block(const Dims& d) {
    const long bh = (long)d.batch * d.nheads;
    return bh * (d.headdim / 64) >= 256 ? 64 : 32;
}

template <typename TS, int P, int S, int T, int PT>
hipError_t run_scan(const void* x, const void* Bm, const float* A, const float* dt_t,
                    const float* h0, void* states, float* fin, const Dims& d, hipStream_t stream) {
    constexpr ScanPlan plan = scan_plan<TS, P, S, T, PT>();
    using Cfg = ScanCfg<bf16, TS, P, S, T, PT, plan.tb, plan.ring>;
    static_assert(Cfg::FITS, "state scan LDS plan does not fit");
    auto kern = state_scan_kernel<bf16, TS, P, S, T, PT, plan.tb, plan.ring>;
    if (Cfg::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)Cfg::LDS_BYTES);
        if (e != hipSuccess) return e;
    }
    const int nblocks = d.batch * d.nheads * (P / PT);
    kern<<<nblocks, Cfg::NTHR, Cfg::LDS_BYTES, stream>>>((const bf16*)x, (const bf16*)Bm, A, dt_t,
                                                        h0, (TS*)states, fin, d.seqlen, d.nheads,
                                                        d.ngroups);
    return hipGetLastError();
}

template <typename TS, int P, int S, int T>
hipError_t scan_by_pt(const void* x, const void* Bm, const float* A, const float* dt_t,
                      const float* h0, void* st, float* fin, const Dims& d, hipStream_t s) {
    if (scan_rows_per_block(d) == 64) return run_scan<TS, P, S, T, 64>(x, Bm, A, dt_t, h0, st, fin, d, s);
    return run_scan<TS, P, S, T, 32>(x, Bm, A, dt_t, h0, st, fin, d, s);
}

template <typename TS, int P, int S>
hipError_t scan_by_t(const void* x, const void* Bm, const float* A, const float* dt_t,
                     const float* h0, void* st, float* fin, const Dims& d, hipStream_t s) {
    switch (d.chunk) {
        case 64: return scan_by_pt<TS, P, S, 64>(x, Bm, A, dt_t, h0, st, fin, d, s);
        case 128: return scan_by_pt<TS, P, S, 128>(x, Bm, A, dt_t, h0, st, fin, d, s);
        case 256: return scan_by_pt<TS, P, S, 256>(x, Bm, A, dt_t, h0, st, fin, d, s);
    }
    return hipErrorInvalidValue;
}

template <typename TS, int P>
hipError_t scan_by_s(const void* x, const void* Bm, const float* A, const float* dt_t,
                     const float* h0, void* st, float* fin, const Dims& d, hipStream_t s) {
    switch (d.dstate) {
        case 64: return scan_by_t<TS, P, 64>(x, Bm, A, dt_t, h0, st, fin, d, s);
        case 128: return scan_by_t<TS, P, 128>(x, Bm, A, dt_t, h0, st, fin, d, s);
        case 256: return scan_by_t<TS, P, 256>(x, Bm, A, dt_t, h0, st, fin, d, s);
    }
    return hipErrorInvalidValue;
}

// bf16 inputs, headdim 64 or 128, dstate 64, 128 or 256 (see state_scan_supported)
template <typename TS>
hipError_t scan_by_p(const void* x, const void* Bm, const float* A, const float* dt_t,
                     const float* h0, void* st, float* fin, const Dims& d, hipStream_t s) {
    switch (d.headdim) {
        case 64: return scan_by_s<TS, 64>(x, Bm, A, dt_t, h0, st, fin, d, s);
        case 128: return scan_by_s<TS, 128>(x, Bm, A, dt_t, h0, st, fin, d, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ssd
