// Stage 2 by segments: the chunk-initial states of a run of consecutive chunks, with the
// running state of a block of heads kept on chip (kernel template for bf16 inputs;
// instances in k_state_seg_bf16.hip).
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Kernel 2: fwd_pass_state" (the state kernel walks the chunks in order,
// records the state entering each chunk and advances it by the jump formula of section
// "Mamba-2 architecture"):
//     S_{c+1}[p][s] = 2^{g_c} S_c[p][s] + sum_{j in chunk c} x_j[p] (dt_j 2^{G_last - G_j} B_j[s])
// Because the recurrence is linear in the state, a walk over segment k (chunks
// kK .. kK+K-1) may start from zero instead of the true entering state S_in(k):
//     S_c = L_c + 2^{D_c} S_in(k),    D_c = sum of g over the segment's chunks before c,
// where L_c is the state the walk from zero records. Segment 0 starts from h0, so its
// recorded states are the true ones. The walk writes L_c (rounded to bf16 like the
// states the output kernel consumes), D_c, the segment's own end state E_k (fp32) and its
// total decay; a small sequential kernel then carries S_in(k+1) = 2^{D_k} S_in(k) + E_k
// across segments (and gives the final state), and the output kernel adds 2^{D_c} S_in(k)
// while staging each chunk's state. The per-chunk increments never go to HBM.
//
// gfx950 mapping: one workgroup of 8 waves (one per CU), or of 4 waves (two per CU) where
// its LDS plan fits in half a CU, per (batch, segment, block of NH heads of one B group).
// Each head's running state (P x S fp32) is spread over the waves in the MFMA
// accumulator layout and stays in registers for the whole segment. A step is one (chunk,
// 64-token sub-block) for all NH heads: the sub-block's B rows, staged in LDS once, give
// each wave its B fragments once per 32 tokens, and those feed every head's products. B
// rows and every head's x rows are double-buffered in LDS by step parity and go there
// straight from memory (direct-to-LDS buffer loads, no registers), issued at the top of
// the step before, right after the barrier that freed the buffers; the tiles are unpadded
// with their 16-byte pieces swizzled per row, so the transposing reads stay free of bank
// conflicts. dt loads into registers a step ahead and becomes the head's decay weights (at
// a chunk's first sub-block) at the end of the step before, so the end of a step is a
// single barrier, which also waits for the direct loads. The contraction over the tokens is dS^T = B^T (w o x) on bf16 MFMA 16x16x32
// with both operands from the transposing LDS read; the fused operand w_j x_j is formed in
// fp32 and split into a bf16 high part and a bf16 remainder (two MFMAs against the exact
// bf16 B). The accumulator holds four consecutive state columns s of one row p per lane;
// a swap between lanes 16 apart gives each lane eight, so each recorded state leaves as
// 16-byte stores (64 contiguous bytes of each of 16 rows per instruction). Wave hh forms
// head hh's weights, once per chunk, with a single-wave DPP suffix scan.
#pragma once

#include <algorithm>
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int V> using IntC = std::integral_constant<int, V>;

// f(IntC<I>{}) for I = B .. E-1, unrolled at compile time.
template <int B, int E> struct StaticFor {
    template <class F> __device__ __forceinline__ static void run(F&& f) {
        if constexpr (B < E) {
            f(IntC<B>{});
            StaticFor<B + 1, E>::run(f);
        }
    }
};

// TB: tokens per step (a sub-block of the chunk). NW: waves per workgroup, 8 (one
// workgroup per CU) or 4 (two per CU when the LDS plan takes at most half the CU's 160 KB).
// A step is one (chunk, sub-block) for all NH heads of the workgroup: the sub-block's B
// fragments are read from LDS once per step and feed every head's products.
template <int P, int S, int T, int TB, int NW = 8>
struct SegCfg {
    static constexpr int NTHR = 64 * NW, NWAVE = NW;
    static constexpr int NSUB = T / TB;  // sub-blocks (steps) per chunk
    static constexpr int NPT = P / 16, NST = S / 16;
    static constexpr int WPT = NPT >= NWAVE ? 1 : NWAVE / NPT;  // waves per p-tile
    static constexpr int MST = (NST + WPT - 1) / WPT;           // s-tiles per wave
    static constexpr int XRB = P * 2, BRB = S * 2;  // row bytes of the x and B tiles
    static constexpr int NXI = TB * XRB / 1024 / NW;  // direct loads per wave and head (x)
    static constexpr int NBI = TB * BRB / 1024 / NW;  // direct loads per wave (B)
    static constexpr int PER = T / 64;                          // tokens per lane in the scan
    static constexpr size_t X_BYTES = (size_t)TB * XRB;  // one head's rows
    static constexpr size_t W_BYTES = (size_t)T * sizeof(float);       // one chunk's weights
    static constexpr size_t B_BYTES = (size_t)TB * BRB;
    // B and every head's x rows double-buffered by step parity; weights per (chunk parity,
    // head)
    static constexpr size_t lds_bytes(int nh) {
        return 2 * B_BYTES + 2 * (size_t)nh * X_BYTES + 2 * (size_t)nh * W_BYTES;
    }
    static constexpr size_t LDS_BYTES = lds_bytes(2);
    static constexpr int STATE_REGS = MST * 4;
    // (the x and B tiles of a step split into whole 1 KB direct loads per wave, so that no
    // load of the step loop sits under a condition: there the compiler cannot count the
    // memory operations issued after a load and waits for all of them; the swizzle covers
    // rows of 128 bytes and more)
    static constexpr bool FITS = lds_bytes(1) <= 163840 && NPT <= NWAVE && NST % WPT == 0 &&
                                 T % TB == 0 && TB % 32 == 0 && (TB * XRB) % (1024 * NW) == 0 &&
                                 (TB * BRB) % (1024 * NW) == 0 && (P == 64 || P == 128) &&
                                 S >= 64;
};

// Swizzled tiles: the 16-byte piece c of row r sits at piece position c ^ swz(r), so that the
// 8 rows x 2 pieces that 32 lanes read together through the transposing LDS read fall on
// distinct banks without row padding (rows of 128 bytes: two rows per 64 banks; of 256 bytes
// or more: a row per 64 banks).
template <int RB> __device__ __forceinline__ int swz(int r) {
    return RB == 128 ? 2 * ((r >> 1) & 3) : 2 * (r & 7);
}
template <int RB>
__device__ __forceinline__ bf16x4 lds_col4_sw(const bf16* base, int r0, int c0, int lane) {
    const int s = lane & 15;
    const int r = r0 + (s >> 2), col = c0 + 4 * (s & 3);
    const bf16* p = base + r * (RB / 2) + (((col >> 3) ^ swz<RB>(r)) << 3) + (col & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(__attribute__((address_space(3))) bf16*)p);
}
// Rows row0 .. row0 + (NW NI 1024 / RB) - 1 of a row-major bf16 matrix (row stride gstride
// elements) straight into a swizzled LDS tile: wave w issues the direct-to-LDS loads of
// pieces (w NI + k) 64 + lane, k < NI (lane L of a load lands 16 L bytes past its base).
template <int RB, int NI>
__device__ __forceinline__ void dma_tile(bf16* lds, BufRsrc r, int row0, uint32_t gstride,
                                         uint32_t soff, int wave, int lane) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        const int n = (wave * NI + k) * 64 + lane;
        const int rr = n / (RB / 16), pp = n % (RB / 16);
        const int c = pp ^ swz<RB>(rr);
        const uint32_t voff = ((uint32_t)(row0 + rr) * gstride + (uint32_t)c * 8u) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + (wave * NI + k) * 512), 16, voff,
            soff, 0, 0);
    }
}

// (the 4-wave form asks the register allocator for two waves per SIMD: two workgroups per
// compute unit)
template <int P, int S, int T, int TB, int NW, int NH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1))) void state_seg_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ G, const float* __restrict__ dt_t, const float* __restrict__ h0,
    bf16* __restrict__ states, float* __restrict__ seg_end, float* __restrict__ dec_in,
    float* __restrict__ dec_seg, int L, int H, int ngroups, int K) {
    using Cfg = SegCfg<P, S, T, TB, NW>;
    constexpr int PER = Cfg::PER, XRB = Cfg::XRB, BRB = Cfg::BRB;
    constexpr int MST = Cfg::MST, WPT = Cfg::WPT, NSUB = Cfg::NSUB;
    constexpr int SPC = NSUB;  // steps per chunk

    // one LDS object per buffer parity, so that the compiler sees the direct loads into
    // one parity's buffers and the reads of the other's as disjoint (it waits for a direct
    // load before a read of LDS that it cannot show to be elsewhere)
    __shared__ __attribute__((aligned(16))) bf16 sB0[TB * S], sB1[TB * S];   // [TB][S] swizzled
    __shared__ __attribute__((aligned(16))) bf16 sX0[NH * TB * P], sX1[NH * TB * P];  // [NH][TB][P]
    __shared__ __attribute__((aligned(16))) float sW[2 * NH * T];
    auto s_b = [&](auto k_c) { return decltype(k_c)::value ? sB1 : sB0; };
    auto s_x = [&](auto k_c, int hh) { return (decltype(k_c)::value ? sX1 : sX0) + hh * TB * P; };
    auto s_w = [&](int par, int hh) { return sW + (par * NH + hh) * T; };  // [T] one (chunk, head)

    const int nC = (L + T - 1) / T;
    const int nseg = (nC + K - 1) / K;
    const int nhb = H / NH;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = id % nhb;
    const int seg = (id / nhb) % nseg;
    const int b = id / (nhb * nseg);
    const int h_first = hb * NH;
    const int g = h_first / (H / ngroups);  // NH divides the heads per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int HP = H * P;
    const size_t grow = (size_t)ngroups * S;
    const int pt = wave / WPT;
    const int st0 = (wave % WPT) * MST;
    const int c_first = seg * K;
    const int nck = min(K, nC - c_first);
    const int p = pt * 16 + l16;
    const bool odd_g4 = (g4 & 1) != 0;
    const uint32_t st_off =
        (uint32_t)((p * S + (odd_g4 ? (st0 + 1) * 16 + 4 * (g4 - 1) : st0 * 16 + 4 * g4)) *
                   sizeof(bf16));
    static_assert(MST % 2 == 0, "recorded states are written as tile pairs");
    static_assert(Cfg::NXI >= 1 && Cfg::NBI >= 1, "a step's rows split evenly over the waves");

    const BufRsrc rdt = make_rsrc(dt_t + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));
    const BufRsrc rg = make_rsrc(G + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));
    auto rows_of = [&](int c) { return min(T, L - c * T); };
    auto rdec_in = [&](int h) {  // the (batch, head) row of chunk decays
        return make_rsrc(dec_in + ((size_t)b * H + h) * nC, (uint32_t)(nC * sizeof(float)));
    };
    auto x_rsrc = [&](int c) {
        return make_rsrc(x + ((size_t)b * L + (size_t)c * T) * HP,
                         (uint32_t)(rows_of(c) * HP * sizeof(bf16)));
    };

    // ---- staging --------------------------------------------------------------------------
    // B rows and every head's x rows go straight from memory into the LDS buffers of the
    // next step (issued at the top of the step before, after the barrier that freed them);
    // the chunk decay two steps ahead and dt one step ahead go to registers, dt into the
    // weight slot (at a chunk's first sub-block) at the end of the step before.
    float pdt[NH][PER];
    float gls[2][NH];
    auto load_g = [&](auto set_c, int c) {
        constexpr int q = decltype(set_c)::value;
        const int rows = rows_of(c);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const uint32_t o = (uint32_t)(((size_t)(h_first + hh) * L + (size_t)c * T) * sizeof(float));
            gls[q][hh] = buf_load_f32(rg, (uint32_t)((rows - 1) * 4), o);
        }
    };
    auto dma_rows = [&](auto kb, int c, int sub) {
        const int rows = rows_of(c);
        const BufRsrc rb = make_rsrc(Bm + (((size_t)b * L + (size_t)c * T) * ngroups + g) * S,
                                     (uint32_t)(((size_t)(rows - 1) * grow + S) * sizeof(bf16)));
        dma_tile<BRB, Cfg::NBI>(s_b(kb), rb, sub * TB, (uint32_t)grow, 0u, wave, lane);
        const BufRsrc rx = x_rsrc(c);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
            dma_tile<XRB, Cfg::NXI>(s_x(kb, hh), rx, sub * TB, (uint32_t)HP,
                                    (uint32_t)((h_first + hh) * P * sizeof(bf16)), wave, lane);
    };
    auto load_dt = [&](int c) {
        const int rows = rows_of(c);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const uint32_t o = (uint32_t)(((size_t)(h_first + hh) * L + (size_t)c * T) * sizeof(float));
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int t = T - 1 - (PER * lane + k);
                pdt[hh][k] = buf_load_f32(rdt, (uint32_t)(t < rows ? t * 4 : 0x80000000u), o);
            }
        }
    };
    // at a chunk's first sub-block wave hh turns head hh's dt into its weights, in the slot
    // of the chunk's parity
    auto store_w = [&](int c, int sub) {
        if (sub == 0) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                if (wave != hh % NW) continue;
                // w_t = dt_t 2^{log2(e) sum_{k>t} A dt_k}: scanned from the chunk's end
                const float ah = A[h_first + hh];
                float pre[PER], run = 0.f;
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    pre[k] = run;
                    run += ah * pdt[hh][k];
                }
                const float excl = wave_shift_up1(wave_inclusive_scan(run));
                float* bw = s_w(c & 1, hh);
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    bw[T - 1 - (PER * lane + k)] = pdt[hh][k] * exp2_fast((excl + pre[k]) * kLog2e);
            }
        }
    };

    // ---- running states: h0 for segment 0, zero otherwise -------------------------------
    f32x4 acc[NH][MST];
    float dacc[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        dacc[hh] = 0.f;
#pragma unroll
        for (int m = 0; m < MST; ++m) {
            const int s = (st0 + m) * 16 + 4 * g4;
            if (seg == 0 && h0)
                acc[hh][m] = *(const f32x4*)(h0 + (((size_t)b * H + h_first + hh) * P + p) * S + s);
            else
                acc[hh][m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // ---- one step: sub-block u of chunk ci, register set / LDS buffers q ----------------
    auto step = [&](auto u_c, auto q_c, int ci) {
        constexpr int u = decltype(u_c)::value, q = decltype(q_c)::value;
        constexpr int sub = u;
        constexpr int u1 = (u + 1) % SPC, dc1 = (u + 1) / SPC;
        constexpr int dc2 = (u + 2) / SPC;  // the chunk two steps ahead
        const int c = c_first + ci;
        float gl[NH];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) gl[hh] = gls[q][hh];  // before set q is reloaded
        // the next step's rows into LDS buffers q^1 (last read by the previous step, which
        // ended at a barrier); dt for the next step, the chunk decay two steps ahead; past
        // the segment's end the loads repeat its last chunk and are never used
        const int c1 = min(c + dc1, c_first + nck - 1);
        dma_rows(IntC<q ^ 1>{}, c1, u1);
        load_dt(c1);
        load_g(q_c, min(c + dc2, c_first + nck - 1));
        __builtin_amdgcn_sched_barrier(0);

        if constexpr (sub == 0) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                const int h = h_first + hh;
                const BufRsrc rst = make_rsrc(states + (((size_t)b * H + h) * nC + c) * (size_t)P * S,
                                              (uint32_t)(P * S * sizeof(bf16)));
#pragma unroll
                for (int m = 0; m < MST; m += 2) {
                    bf16x4 o0, o1;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        o0[r] = from_f32<bf16>(acc[hh][m][r]);
                        o1[r] = from_f32<bf16>(acc[hh][m + 1][r]);
                    }
                    const u32x2 a = __builtin_bit_cast(u32x2, o0), a1 = __builtin_bit_cast(u32x2, o1);
                    const u32x2 send = odd_g4 ? a : a1;
                    u32x2 recv;
                    recv[0] = (uint32_t)__shfl_xor((int)send[0], 16);
                    recv[1] = (uint32_t)__shfl_xor((int)send[1], 16);
                    const u32x2 first = odd_g4 ? recv : a, second = odd_g4 ? a1 : recv;
                    const Vec16 out = Vec16{first[0], first[1], second[0], second[1]};
                    buf_store16(out, rst, st_off + (uint32_t)(m * 16 * sizeof(bf16)));
                }
                // one lane writes the decay (the others' offsets lie outside the
                // descriptor and their stores are dropped): no store under a condition
                buf_store_f32(dacc[hh], rdec_in(h), tid == 0 ? (uint32_t)(c * sizeof(float)) : 0x80000000u, 0u);
                dacc[hh] += gl[hh];
                const float dec = exp2_fast(gl[hh]);
#pragma unroll
                for (int m = 0; m < MST; ++m) acc[hh][m] *= dec;
            }
        }

        const bf16* bb = s_b(q_c);
        // slot (g4, v) carries token 32 ks + 16 (v/4) + 4 g4 + v%4 (two column reads)
#pragma unroll 2
        for (int ks = 0; ks < TB / 32; ++ks) {
            const int r_lo = ks * 32 + 4 * g4, r_hi = r_lo + 16;
            Frag<bf16> bf[MST];
#pragma unroll
            for (int m = 0; m < MST; ++m) {
                const int st = st0 + m;
                const bf16x4 a = lds_col4_sw<BRB>(bb, r_lo, st * 16, lane);
                const bf16x4 q4 = lds_col4_sw<BRB>(bb, r_hi, st * 16, lane);
                bf[m].v = __builtin_shufflevector(a, q4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                const bf16* bx = s_x(q_c, hh);
                const float* bw = s_w(c & 1, hh) + sub * TB;
                const f32x4 w_lo = *(const f32x4*)(bw + r_lo);
                const f32x4 w_hi = *(const f32x4*)(bw + r_hi);
                const bf16x4 a = lds_col4_sw<XRB>(bx, r_lo, pt * 16, lane);
                const bf16x4 q4 = lds_col4_sw<XRB>(bx, r_hi, pt * 16, lane);
                Frag<bf16> hi, lo;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float x0 = to_f32(a[v]) * w_lo[v], x1 = to_f32(q4[v]) * w_hi[v];
                    hi.v[v] = from_f32<bf16>(x0);
                    hi.v[v + 4] = from_f32<bf16>(x1);
                    lo.v[v] = from_f32<bf16>(x0 - to_f32(hi.v[v]));
                    lo.v[v + 4] = from_f32<bf16>(x1 - to_f32(hi.v[v + 4]));
                }
#pragma unroll
                for (int m = 0; m < MST; ++m) {
                    mma(acc[hh][m], bf[m], hi);
                    mma(acc[hh][m], bf[m], lo);
                }
            }
        }
        // the next chunk's weights (at its first sub-block)
        store_w(c + dc1, u1);
        lds_barrier();  // the next step's rows have landed; every wave is done with buffers q
    };

    // ---- prologue: steps 0 and 1 loaded, step 0 in LDS ----------------------------------
    dma_rows(IntC<0>{}, c_first, 0);
    load_dt(c_first);
    load_g(IntC<0>{}, c_first);
    load_g(IntC<1>{}, min(c_first + 1 / SPC, c_first + nck - 1));
    store_w(c_first, 0);
    lds_barrier();

    constexpr int CPP = SPC % 2 == 0 ? 1 : 2;  // chunks per pass
    for (int ci = 0; ci < nck; ci += CPP) {
        StaticFor<0, SPC>::run([&](auto u_c) {
            constexpr int u = decltype(u_c)::value;
            step(u_c, IntC<(u & 1)>{}, ci);
        });
        if constexpr (CPP == 2) {
            if (ci + 1 < nck) {
                StaticFor<0, SPC>::run([&](auto u_c) {
                    constexpr int u = decltype(u_c)::value;
                    step(u_c, IntC<((SPC + u) & 1)>{}, ci + 1);
                });
            }
        }
    }

    // ---- the segment's own end state and total decay ------------------------------------
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        const int h = h_first + hh;
        float* dst = seg_end + (((size_t)b * H + h) * nseg + seg) * (size_t)P * S;
#pragma unroll
        for (int m = 0; m < MST; ++m) {
            const int s = (st0 + m) * 16 + 4 * g4;
            *(f32x4*)(dst + (size_t)p * S + s) = acc[hh][m];
        }
        if (tid == 0) dec_seg[((size_t)b * H + h) * nseg + seg] = dacc[hh];
    }
}

// Carry across segments: S_in(0) = end of segment 0 (which started from h0);
// S_in(k+1) = 2^{D_k} S_in(k) + E_k; the state after the last segment is the final state.
// S_in(k) for k >= 1 is stored in bf16 for the output kernel. One wave per 256 state
// elements of one (batch, head), 4 per lane.
__global__ __launch_bounds__(64) void seg_carry_kernel(const float* __restrict__ seg_end,
                                                       const float* __restrict__ dec_seg,
                                                       bf16* __restrict__ seg_in,
                                                       float* __restrict__ fin, int nseg,
                                                       int PS) {
    const int per_bh = PS / 256;
    const size_t bh = blockIdx.x / per_bh;
    const int e = (blockIdx.x % per_bh) * 256 + threadIdx.x * 4;
    const float* src = seg_end + bh * nseg * (size_t)PS + e;
    bf16* dst = seg_in + bh * nseg * (size_t)PS + e;
    f32x4 hv = *(const f32x4*)src;
    for (int k = 1; k < nseg; ++k) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = from_f32<bf16>(hv[r]);
        *(bf16x4*)(dst + (size_t)k * PS) = o;
        hv = exp2_fast(dec_seg[bh * nseg + k]) * hv + *(const f32x4*)(src + (size_t)k * PS);
    }
    if (fin) *(f32x4*)(fin + bh * PS + e) = hv;
}


// True chunk-initial states from segment-relative ones, in place: for the chunks of
// segments k >= 1, S_c = bf16(L_c + 2^{D_c} S_in(k)) with the fp32 arithmetic the output
// kernel uses when it forms the same sum while staging a state, so either route gives the
// same bits; chunks with D_c below kSegCut are left as they are. One workgroup of 256
// threads per (batch, head, chunk), 16-byte accesses.
__global__ __launch_bounds__(256) void seg_correct_kernel(bf16* __restrict__ states,
                                                          const bf16* __restrict__ seg_in,
                                                          const float* __restrict__ dec_in,
                                                          int nC, int K, int nseg, int PS) {
    const int c = blockIdx.x % nC;
    const size_t bh = blockIdx.x / nC;
    const int k = c / K;
    if (k == 0) return;
    const float dec = dec_in[bh * nC + c];
    if (!(dec >= kSegCut)) return;
    const float f = exp2_fast(dec);
    bf16x8* st = (bf16x8*)(states + (bh * nC + c) * (size_t)PS);
    const bf16x8* si = (const bf16x8*)(seg_in + (bh * nseg + k) * (size_t)PS);
    for (int v = threadIdx.x; v < PS / 8; v += 256) {
        const bf16x8 l8 = st[v], s8 = si[v];
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(to_f32(l8[e]) + f * to_f32(s8[e]));
        st[v] = o;
    }
}

}  // namespace ssd
