// Segmented state pass for bf16 inputs: plan choice, workspace layout and launches
// (kernels in state_seg.h).
#include "state_seg.h"

namespace ssd {

namespace {

constexpr int kSegHeads[] = {1, 2, 3, 4, 5, 6, 8};  // instantiated heads per workgroup

// The kernel form for a shape: 64-token steps; 4 waves, two workgroups per CU, where the
// LDS plan of two heads fits in half a CU (80 KB) and a head's running state takes at
// most 32 registers per lane (dstate up to 128); otherwise 8 waves, one workgroup per CU.
template <int P, int S, int T>
struct SegPick {
    static constexpr int TB = 64;
    using Cfg4 = SegCfg<P, S, T, TB, 4>;
    static constexpr bool DUAL = Cfg4::FITS && Cfg4::lds_bytes(2) <= 81920 && P * S <= 64 * 128;
    static constexpr int NW = DUAL ? 4 : 8;
    using Cfg = SegCfg<P, S, T, TB, NW>;
    static constexpr int SLOTS = DUAL ? 512 : 256;  // workgroups resident on 256 CUs
    // running-state registers per lane the plan allows: no spills, and with 4 waves at
    // most 256 registers per wave so that two workgroups stay resident
    static constexpr int MAX_STATE_REGS = DUAL ? 64 : 80;
    // heads whose x buffers and weight slots fit the form's LDS share
    static constexpr size_t LDS_CAP = DUAL ? 81920 : 163840;
    static constexpr int MAX_HEADS = Cfg::lds_bytes(8) <= LDS_CAP   ? 8
                                     : Cfg::lds_bytes(4) <= LDS_CAP ? 4
                                     : Cfg::lds_bytes(2) <= LDS_CAP ? 2
                                                                    : 1;
};
template <int P, int S, int T> using SegCfgFor = typename SegPick<P, S, T>::Cfg;

// Whether the shape has a kernel form; its workgroup slots per round, state-register and
// head limits, threads and sub-blocks per chunk.
struct SegForm {
    bool fits;
    int slots, max_state_regs, max_heads, nthr, nsub;
};
SegForm seg_form(int P, int S, int T) {
    switch (P * 1000000 + S * 1000 + T) {
#define SSD_SEG_FITS(p, s, t)                                                              \
    case p * 1000000 + s * 1000 + t:                                                       \
        return SegForm{SegCfgFor<p, s, t>::FITS, SegPick<p, s, t>::SLOTS,                  \
                       SegPick<p, s, t>::MAX_STATE_REGS, SegPick<p, s, t>::MAX_HEADS,      \
                       SegCfgFor<p, s, t>::NTHR, SegCfgFor<p, s, t>::NSUB};
        SSD_SEG_FITS(64, 64, 64) SSD_SEG_FITS(64, 64, 128) SSD_SEG_FITS(64, 64, 256)
        SSD_SEG_FITS(64, 128, 64) SSD_SEG_FITS(64, 128, 128) SSD_SEG_FITS(64, 128, 256)
        SSD_SEG_FITS(64, 256, 64) SSD_SEG_FITS(64, 256, 128) SSD_SEG_FITS(64, 256, 256)
#undef SSD_SEG_FITS
    }
    return SegForm{false, 0, 0, 0, 0, 0};
}

template <int P, int S, int T, int NH>
hipError_t run_seg(const void* x, const void* Bm, const float* A, const float* G,
                   const float* dt_t, const float* h0, void* states, const SegPlan& pl,
                   const SegBuffers& sb, const Dims& d, hipStream_t stream) {
    using Pick = SegPick<P, S, T>;
    using Cfg = typename Pick::Cfg;
    auto kern = state_seg_kernel<P, S, T, Pick::TB, Pick::NW, NH>;
    const int nblocks = d.batch * pl.nseg * (d.nheads / NH);
    kern<<<nblocks, Cfg::NTHR, 0, stream>>>(
        (const bf16*)x, (const bf16*)Bm, A, G, dt_t, h0, (bf16*)states, sb.seg_end, sb.dec_in,
        sb.dec_seg, d.seqlen, d.nheads, d.ngroups, pl.chunks);
    return hipGetLastError();
}

template <int P, int S, int T>
hipError_t seg_by_nh(const void* x, const void* Bm, const float* A, const float* G,
                     const float* dt_t, const float* h0, void* st, const SegPlan& pl,
                     const SegBuffers& sb, const Dims& d, hipStream_t s) {
    using Pick = SegPick<P, S, T>;
    if constexpr (!Pick::Cfg::FITS) {
        return hipErrorInvalidValue;
    } else {
        // head counts the plan can choose for this form (others are not instantiated)
        constexpr int RPH = P * S / Pick::Cfg::NTHR;  // state registers per head and lane
        switch (pl.heads) {
#define SSD_SEG_NH(n)                                                                          \
    case n:                                                                                    \
        if constexpr (n <= Pick::MAX_HEADS && n * RPH <= Pick::MAX_STATE_REGS)                 \
            return run_seg<P, S, T, n>(x, Bm, A, G, dt_t, h0, st, pl, sb, d, s);               \
        break;
            SSD_SEG_NH(1) SSD_SEG_NH(2) SSD_SEG_NH(3) SSD_SEG_NH(4) SSD_SEG_NH(5) SSD_SEG_NH(6)
            SSD_SEG_NH(8)
#undef SSD_SEG_NH
        }
        return hipErrorInvalidValue;
    }
}

template <int P, int S>
hipError_t seg_by_t(const void* x, const void* Bm, const float* A, const float* G,
                    const float* dt_t, const float* h0, void* st, const SegPlan& pl,
                    const SegBuffers& sb, const Dims& d, hipStream_t s) {
    switch (d.chunk) {
        case 64: return seg_by_nh<P, S, 64>(x, Bm, A, G, dt_t, h0, st, pl, sb, d, s);
        case 128: return seg_by_nh<P, S, 128>(x, Bm, A, G, dt_t, h0, st, pl, sb, d, s);
        case 256: return seg_by_nh<P, S, 256>(x, Bm, A, G, dt_t, h0, st, pl, sb, d, s);
    }
    return hipErrorInvalidValue;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

// Plan: heads per workgroup (a divisor of the heads per group whose running states fit
// in registers) and chunks per segment (at least 2 unless the sequence has one
// chunk). Workgroups are resident one or two per CU (the form's LDS plan), so the grid
// runs in rounds of 256 or 512 workgroups; with two per CU, a last round that leaves
// every CU at most one workgroup takes 0.9 of a full one. A workgroup's work is counted
// in (64-token sub-block, head) units, plus 0.2 of a unit per sub-block for the B rows its
// heads share, 2 per head (entering and end states) and 2 per workgroup; each segment adds
// 0.3 for its carry and correction. These weights were fitted to measured forward times
// over plans for five layer shapes (dstate 64 to 256, 8 to 80 heads, chunks of 64 to 256
// tokens). Ties go to longer segments (fewer corrections downstream).
bool state_seg_plan(int in_dtype, int states_dtype, const Dims& d, SegPlan* out) {
    if (in_dtype != kBF16 || states_dtype != kBF16) return false;
    const SegForm f = seg_form(d.headdim, d.dstate, d.chunk);
    if (!f.fits) return false;
    const int nC = d.nchunks();
    if (nC < 1) return false;
    const int hpg = d.nheads / d.ngroups;
    const int regs_per_head = d.headdim * d.dstate / f.nthr;
    double best = 1e300;
    SegPlan bp{0, 0, 0};
    for (int nh : kSegHeads) {
        // register budget of the two-step prefetch (no spills): the form's state-register
        // limit per lane, its weight slots, and, with 8 waves, eight heads only with
        // chunks shorter than 256 tokens
        if (hpg % nh != 0 || nh * regs_per_head > f.max_state_regs || nh > f.max_heads ||
            (f.slots == 256 && nh == 8 && d.chunk == 256))
            continue;
        for (int k = (nC == 1 ? 1 : 2); k <= nC; ++k) {
            const int nseg = (nC + k - 1) / k;
            const long wgs = (long)d.batch * nseg * (d.nheads / nh);
            double rounds = (double)((wgs + f.slots - 1) / f.slots);
            if (f.slots == 512 && wgs % 512 != 0 && wgs % 512 <= 256) rounds -= 0.1;
            const double steps = (double)k * f.nsub;
            const double cost = rounds * (nh * steps + 0.2 * steps + 2.0 * nh + 2.0) + 0.3 * nseg;
            if (cost < best - 1e-9 || (cost < best + 1e-9 && k > bp.chunks)) {
                best = cost;
                bp = SegPlan{nh, k, nseg};
            }
        }
    }
    if (bp.heads == 0) return false;
    *out = bp;
    return true;
}

// Workspace: segment end states [B,H,nseg,P,S] fp32, entering states [B,H,nseg,P,S] bf16,
// per-chunk decays [B,H,nC] and per-segment decays [B,H,nseg] fp32.
size_t state_seg_ws_bytes(const Dims& d, const SegPlan& pl) {
    const size_t bh = (size_t)d.batch * d.nheads, ps = (size_t)d.headdim * d.dstate;
    return round256(bh * pl.nseg * ps * 4) + round256(bh * pl.nseg * ps * 2) +
           round256(bh * d.nchunks() * 4) + round256(bh * pl.nseg * 4);
}

SegBuffers state_seg_buffers(void* ws, const Dims& d, const SegPlan& pl) {
    const size_t bh = (size_t)d.batch * d.nheads, ps = (size_t)d.headdim * d.dstate;
    char* w = (char*)ws;
    SegBuffers sb;
    sb.seg_end = (float*)w;
    w += round256(bh * pl.nseg * ps * 4);
    sb.seg_in = (void*)w;
    w += round256(bh * pl.nseg * ps * 2);
    sb.dec_in = (float*)w;
    w += round256(bh * d.nchunks() * 4);
    sb.dec_seg = (float*)w;
    return sb;
}

hipError_t launch_state_seg(const void* x, const void* Bm, const float* A, const float* G,
                            const float* dt_t, const float* h0, void* states,
                            float* final_state, const SegPlan& pl, const SegBuffers& sb,
                            const Dims& d, hipStream_t stream) {
    hipError_t e = hipErrorInvalidValue;
    switch (d.headdim * 1000 + d.dstate) {
        case 64064: e = seg_by_t<64, 64>(x, Bm, A, G, dt_t, h0, states, pl, sb, d, stream); break;
        case 64128: e = seg_by_t<64, 128>(x, Bm, A, G, dt_t, h0, states, pl, sb, d, stream); break;
        case 64256: e = seg_by_t<64, 256>(x, Bm, A, G, dt_t, h0, states, pl, sb, d, stream); break;
    }
    if (e != hipSuccess) return e;
    if (pl.nseg == 1 && !final_state) return hipSuccess;
    const int PS = d.headdim * d.dstate;  // a multiple of 256 for every instantiated size
    const int nblocks = d.batch * d.nheads * (PS / 256);
    seg_carry_kernel<<<nblocks, 64, 0, stream>>>(sb.seg_end, sb.dec_seg, (bf16*)sb.seg_in,
                                                  final_state, pl.nseg, PS);
    return hipGetLastError();
}

hipError_t launch_seg_correct(void* states, const SegPlan& pl, const SegBuffers& sb,
                              const Dims& d, hipStream_t stream) {
    if (pl.nseg == 1) return hipSuccess;  // every chunk is in segment 0: already true states
    const long nblocks = (long)d.batch * d.nheads * d.nchunks();
    seg_correct_kernel<<<(unsigned)nblocks, 256, 0, stream>>>(
        (bf16*)states, (const bf16*)sb.seg_in, sb.dec_in, d.nchunks(), pl.chunks, pl.nseg,
        d.headdim * d.dstate);
    return hipGetLastError();
}

}  // namespace ssd
