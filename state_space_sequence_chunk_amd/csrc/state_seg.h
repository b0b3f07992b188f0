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
// its LDS plan fits in half a CU, per (batch, segment, block of NH heads of one B group). Each head's running state (P x S fp32) is spread over the waves in the MFMA
// accumulator layout and stays in registers for the whole segment. A step is one (chunk,
// sub-block of TB tokens, head); TB is the whole chunk unless the chunk's B rows would not
// fit in LDS (dstate 256 with 256-token chunks: TB = 128). Per sub-block the group's B
// rows are staged in LDS once and shared by the NH heads; per step the x rows and the
// decay weights are double-buffered in LDS, the loads two steps ahead (and, at a
// sub-block's last head, the next sub-block's B rows) in flight while the current
// products run. The contraction over the tokens is dS^T = B^T (w o x) on bf16 MFMA
// 16x16x32 with both operands from the transposing LDS read; the fused operand w_j x_j is
// formed in fp32 and split into a bf16 high part and a bf16 remainder (two MFMAs against
// the exact bf16 B). The accumulator holds four consecutive state columns s of one row p
// per lane; a swap between lanes 16 apart gives each lane eight, so each recorded state
// leaves as 16-byte stores (64 contiguous bytes of each of 16 rows per instruction). Wave
// 0 forms each head's weights, once per chunk, with a single-wave DPP suffix scan.
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
// workgroup per CU) or 4 (two per CU when the LDS plan takes at most half the CU's 160 KB:
// two independent workgroups do not run in step, so one's VALU and LDS work overlaps the
// other's products).
template <int P, int S, int T, int TB, int NW = 8>
struct SegCfg {
    static constexpr int NTHR = 64 * NW, NWAVE = NW;
    static constexpr int NSUB = T / TB;  // sub-blocks per chunk
    static constexpr int NPT = P / 16, NST = S / 16;
    static constexpr int WPT = NPT >= NWAVE ? 1 : NWAVE / NPT;  // waves per p-tile
    static constexpr int MST = (NST + WPT - 1) / WPT;           // s-tiles per wave
    static constexpr int VE = 8;                                // bf16 per 16 bytes
    static constexpr int XS = col_stride<bf16>(P), BS = col_stride<bf16>(S);
    static constexpr int NXV = (TB * P / VE + NTHR - 1) / NTHR;  // x vectors per thread
    static constexpr int NBV = (TB * S / VE + NTHR - 1) / NTHR;  // B vectors per thread
    static constexpr int PER = T / 64;                          // tokens per lane in the scan
    static constexpr size_t X_BYTES = (size_t)TB * XS * sizeof(bf16);
    static constexpr size_t W_BYTES = (size_t)T * sizeof(float);  // one chunk's weights
    static constexpr size_t B_BYTES = (size_t)TB * BS * sizeof(bf16);
    // weight slots: one per x buffer when a step is a whole chunk; otherwise one per head
    // of the block (up to 8 heads with 8 waves, 2 with 4) and chunk parity, since a head's
    // weights serve all its sub-blocks
    static constexpr int NWS = NSUB == 1 ? 2 : (NW == 4 ? 4 : 16);
    static constexpr size_t LDS_BYTES = B_BYTES + 2 * X_BYTES + NWS * W_BYTES;
    // registers per head for the running state (fp32 per lane)
    static constexpr int STATE_REGS = MST * 4;
    static constexpr bool FITS = LDS_BYTES <= 163840 && NPT <= NWAVE && NST % WPT == 0 &&
                                 T % TB == 0 && TB % 32 == 0;
};

template <int P, int S, int T, int TB, int NW, int NH>
__global__ __launch_bounds__(64 * NW) void state_seg_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ G, const float* __restrict__ dt_t, const float* __restrict__ h0,
    bf16* __restrict__ states, float* __restrict__ seg_end, float* __restrict__ dec_in,
    float* __restrict__ dec_seg, int L, int H, int ngroups, int K) {
    using Cfg = SegCfg<P, S, T, TB, NW>;
    constexpr int VE = Cfg::VE, XS = Cfg::XS, BS = Cfg::BS, NTHR = Cfg::NTHR, PER = Cfg::PER;
    constexpr int MST = Cfg::MST, WPT = Cfg::WPT, NSUB = Cfg::NSUB;
    constexpr int SPC = NSUB * NH;  // steps per chunk
    static_assert(NSUB == 1 || NH <= Cfg::NWS / 2, "weight slots");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16* s_b = (bf16*)smem;  // [TB][BS] B rows of the current sub-block
    auto s_x = [&](int k) { return (bf16*)(smem + Cfg::B_BYTES + k * Cfg::X_BYTES); };  // [TB][XS]
    auto s_w = [&](int k) {  // [T] weights of one (chunk, head)
        return (float*)(smem + Cfg::B_BYTES + 2 * Cfg::X_BYTES + k * Cfg::W_BYTES);
    };

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
    const int pt = wave / WPT;   // this wave's p-tile
    // this wave's s-tiles: MST adjacent ones, so that each 128-byte piece of a recorded
    // state row comes from one wave's back-to-back stores (whole lines reach L2 together,
    // never two waves' halves of one line)
    const int st0 = (wave % WPT) * MST;
    const int c_first = seg * K;
    const int nck = min(K, nC - c_first);  // chunks of this segment
    const int p = pt * 16 + l16;           // this lane's state row (accumulator column)
    // byte offset of this lane's 8 recorded columns for the first tile pair (see the record
    // step: even slot groups take columns 16 st0 + 4 g4 .., odd ones 16 (st0+1) + 4 (g4-1) ..)
    const bool odd_g4 = (g4 & 1) != 0;
    const uint32_t st_off =
        (uint32_t)((p * S + (odd_g4 ? (st0 + 1) * 16 + 4 * (g4 - 1) : st0 * 16 + 4 * g4)) *
                   sizeof(bf16));
    static_assert(MST % 2 == 0, "recorded states are written as tile pairs");

    const BufRsrc rdt = make_rsrc(dt_t + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));
    const BufRsrc rg = make_rsrc(G + (size_t)b * H * L, (uint32_t)((size_t)H * L * sizeof(float)));
    auto rows_of = [&](int c) { return min(T, L - c * T); };
    // x rows past a chunk's real tokens lie outside its descriptor and load as zeros
    auto x_rsrc = [&](int c) {
        return make_rsrc(x + ((size_t)b * L + (size_t)c * T) * HP,
                         (uint32_t)(rows_of(c) * HP * sizeof(bf16)));
    };

    // ---- staging: global -> registers (prefetch, two steps deep) -> LDS -----------------
    // A step is one (chunk, sub-block, head) of the segment, heads fastest, in order (with
    // TB = T: one (chunk, head)). Step j's x rows, dt and chunk
    // decay are loaded into register set j % 2 at the start of step j-2 and moved to LDS
    // buffer j % 2 (wave 0 turning dt into the weights) at the start of step j-1, after
    // that step's own loads are issued; so the staging overlaps the products and the end
    // of a step is a single barrier. The next sub-block's B rows are loaded during a
    // sub-block's last head and replace the current ones between two barriers at its end.
    Vec16 px[2][Cfg::NXV], pb[Cfg::NBV];
    float pdt[2][PER];
    float gls[2] = {0.f, 0.f};  // each set's chunk decay g (log2): G at the chunk's last real token
    auto load_head = [&](auto set_c, int c, int sub, int h) {
        constexpr int q = decltype(set_c)::value;
        const int rows = rows_of(c);
        const BufRsrc rx = x_rsrc(c);
#pragma unroll
        for (int i = 0; i < Cfg::NXV; ++i) {
            const int v = tid + i * NTHR;
            if (v < TB * P / VE) {
                const int r = sub * TB + v / (P / VE), col = (v % (P / VE)) * VE;
                px[q][i] = buf_load16(rx, (uint32_t)((r * HP + col) * sizeof(bf16)),
                                      (uint32_t)(h * P * sizeof(bf16)));
            }
        }
        const uint32_t o = (uint32_t)(((size_t)h * L + (size_t)c * T) * sizeof(float));
        gls[q] = buf_load_f32(rg, (uint32_t)((rows - 1) * 4), o);
        // dt for wave 0's scan (lane holds tokens T-1-(PER*lane+k)); every wave issues the
        // same loads so that all waves count the same memory operations per step
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int t = T - 1 - (PER * lane + k);
            pdt[q][k] = buf_load_f32(rdt, (uint32_t)(t < rows ? t * 4 : 0x80000000u), o);
        }
    };
    // B rows of sub-block sub of chunk c through a descriptor over the chunk's real rows
    // (padded rows read zeros)
    auto load_b = [&](int c, int sub) {
        const int rows = rows_of(c);
        const BufRsrc rb = make_rsrc(Bm + (((size_t)b * L + (size_t)c * T) * ngroups + g) * S,
                                     (uint32_t)(((size_t)(rows - 1) * grow + S) * sizeof(bf16)));
#pragma unroll
        for (int i = 0; i < Cfg::NBV; ++i) {
            const int v = tid + i * NTHR;
            if (v < TB * S / VE) {
                const int r = sub * TB + v / (S / VE), col = (v % (S / VE)) * VE;
                pb[i] = buf_load16(rb, (uint32_t)(((size_t)r * grow + col) * sizeof(bf16)), 0u);
            }
        }
    };
    auto store_b = [&]() {
#pragma unroll
        for (int i = 0; i < Cfg::NBV; ++i) {
            const int v = tid + i * NTHR;
            if (v < TB * S / VE) {
                const int r = v / (S / VE), col = (v % (S / VE)) * VE;
                *(Vec16*)(s_b + r * BS + col) = pb[i];
            }
        }
    };
    // register set q -> LDS buffer q (x rows); at a chunk's first sub-block wave 0 also
    // turns the chunk's dt into the head's weights, in weight slot ws
    auto store_head = [&](auto set_c, int h, bool first_sub, int ws) {
        constexpr int q = decltype(set_c)::value;
        bf16* bx = s_x(q);
#pragma unroll
        for (int i = 0; i < Cfg::NXV; ++i) {
            const int v = tid + i * NTHR;
            if (v < TB * P / VE) {
                const int r = v / (P / VE), col = (v % (P / VE)) * VE;
                *(Vec16*)(bx + r * XS + col) = px[q][i];
            }
        }
        if (wave == 0 && first_sub) {
            // w_t = dt_t 2^{log2(e) sum_{k>t} A dt_k}: scanned from the chunk's end
            const float ah = A[h];
            float pre[PER], run = 0.f;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                pre[k] = run;
                run += ah * pdt[q][k];
            }
            const float excl = wave_shift_up1(wave_inclusive_scan(run));
            float* bw = s_w(ws);
#pragma unroll
            for (int k = 0; k < PER; ++k)
                bw[T - 1 - (PER * lane + k)] = pdt[q][k] * exp2_fast((excl + pre[k]) * kLog2e);
        }
    };

    // ---- running states: h0 for segment 0, zero otherwise -------------------------------
    // tile m of head hh: element (row s = 16 st + 4 g4 + r, column p) in register r
    f32x4 acc[NH][MST];
    float dacc[NH];  // log2 decay from the segment's start (wave-uniform)
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

    // weight slot of head hh in chunk c: per x buffer q when a step is a whole chunk,
    // otherwise per (chunk parity, head)
    auto wslot = [&](int q, int hh, int c) { return NSUB == 1 ? q : (c & 1) * NH + hh; };

    // ---- one step: step u of chunk ci (sub-block u / NH, head u % NH), set / buffer q ----
    auto step = [&](auto u_c, auto q_c, int ci) {
        constexpr int u = decltype(u_c)::value, q = decltype(q_c)::value;
        constexpr int hh = u % NH, sub = u / NH;
        constexpr int u1 = (u + 1) % SPC, dc1 = (u + 1) / SPC;  // the next step
        constexpr int u2 = (u + 2) % SPC, dc2 = (u + 2) / SPC;  // the step two ahead
        const int c = c_first + ci, h = h_first + hh;
        const bool next = ci + dc1 < nck;  // a next step in this segment
        const float gl = gls[q];  // this step's chunk decay, before set q is reloaded
        // Every step issues its loads unconditionally (past the segment's end they repeat its
        // last chunk and are never used), so no wait before a use depends on a runtime branch
        // and the loads two steps ahead stay in flight. The next sub-block's B rows go first:
        // vector-memory waits are in issue order, so the wait for them at this step's end
        // then leaves the loads two steps ahead in flight.
        if constexpr (hh == NH - 1) {  // the next sub-block's B rows
            if constexpr (sub + 1 < NSUB) load_b(c, sub + 1);
            else load_b(next ? c + 1 : c, 0);
        }
        load_head(q_c, min(c + dc2, c_first + nck - 1), u2 / NH, h_first + u2 % NH);
        // stage the next step now (its loads were issued a step ago): LDS buffer q^1 was
        // last read by the previous step, which ended at a barrier; the next step reads
        // it after this step's barrier. Past the segment's end the copy is never read.
        constexpr IntC<q ^ 1> q1{};
        store_head(q1, h_first + u1 % NH, u1 / NH == 0, wslot(q ^ 1, u1 % NH, c + dc1));

        if constexpr (sub == 0) {
            // record the state entering chunk c (from the segment's start), then advance it.
            // For each pair of adjacent tiles (m, m+1) the lanes 16 apart (slot groups 2k and
            // 2k+1) swap one tile's four values, so that the even lane holds columns
            // 16(st0+m) + 4 g4 .. +7 and the odd one 16(st0+m+1) + 4(g4-1) .. +7: one 16-byte
            // store per lane writes 64 contiguous bytes of each of the 16 rows.
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
            if (tid == 0) dec_in[((size_t)b * H + h) * nC + c] = dacc[hh];
            dacc[hh] += gl;
            const float dec = exp2_fast(gl);
    #pragma unroll
            for (int m = 0; m < MST; ++m) acc[hh][m] *= dec;

        }

        const bf16* bx = s_x(q);
        const float* bw = s_w(wslot(q, hh, c)) + sub * TB;
        // slot (g4, v) carries token 32 ks + 16 (v/4) + 4 g4 + v%4 (two column reads)
#pragma unroll 2
        for (int ks = 0; ks < TB / 32; ++ks) {
            const int r_lo = ks * 32 + 4 * g4, r_hi = r_lo + 16;
            Frag<bf16> bf[MST];
#pragma unroll
            for (int m = 0; m < MST; ++m) {
                const int st = st0 + m;
                const bf16x4 a = lds_col4(s_b, BS, r_lo, st * 16, lane);
                const bf16x4 q4 = lds_col4(s_b, BS, r_hi, st * 16, lane);
                bf[m].v = __builtin_shufflevector(a, q4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            const f32x4 w_lo = *(const f32x4*)(bw + r_lo);
            const f32x4 w_hi = *(const f32x4*)(bw + r_hi);
            const bf16x4 a = lds_col4(bx, XS, r_lo, pt * 16, lane);
            const bf16x4 q4 = lds_col4(bx, XS, r_hi, pt * 16, lane);
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

        // hand over to the next step (at a sub-block's end, after the B rows are replaced)
        if constexpr (hh + 1 < NH) {
            lds_barrier();
        } else {
            if (next) {
                lds_barrier();  // every wave is done with this sub-block's B rows
                store_b();
                lds_barrier();
            }
        }
    };

    // ---- prologue: the first sub-block's B rows, steps 0 and 1 loaded, step 0 in LDS ----
    load_head(IntC<0>{}, c_first, 0, h_first);
    load_head(IntC<1>{}, min(c_first + 1 / SPC, c_first + nck - 1), (1 % SPC) / NH,
              h_first + (1 % SPC) % NH);
    load_b(c_first, 0);
    store_b();
    store_head(IntC<0>{}, h_first, true, wslot(0, 0, c_first));
    lds_barrier();

    // ---- main loop: each step's set known at compile time (one chunk per pass when a
    // chunk has an even number of steps, two when it is odd) ------------------------------
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
