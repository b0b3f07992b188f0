// Single-pass state kernel: which shapes it covers, when the forward pass takes it, and
// the dispatch on the recorded states' dtype (instances in k_state_scan_bf16*.hip).
#include "ssd_launch.h"

namespace ssd {

hipError_t launch_state_scan_bf16(const void*, const void*, const float*, const float*,
                                  const float*, void*, float*, const Dims&, hipStream_t);
hipError_t launch_state_scan_bf16_f32(const void*, const void*, const float*, const float*,
                                      const float*, void*, float*, const Dims&, hipStream_t);

bool state_scan_supported(int in_dtype, const Dims& d) {
    return in_dtype == kBF16 && (d.headdim == 64 || d.headdim == 128) &&
           (d.dstate == 64 || d.dstate == 128 || d.dstate == 256) && d.seqlen > 0 &&
           d.seqlen % d.chunk == 0;
}

// The single pass runs one 512-thread workgroup per (batch, head, 64-row slice), one per
// compute unit at a time (its LDS ring takes 96-144 KB), so it runs in rounds of 256
// workgroups, each costing about the same whatever its fill, while the two-kernel pass
// costs in proportion to the slices. Measured on MI355X with bf16 states (batch x tokens
// at the workloads' head shapes), a round costs as much as the two-kernel pass on 190
// slices at dstate 128 and on 148 at dstate 256; the single pass is taken when the last
// round is full enough to win with a margin: 0.75 of 256 slices (0.6 at dstate 256).
// Below 256 slices it would run 32-row slices, which re-read B for each half of a head
// and lost by 1.4-1.7x in every case measured.
bool state_scan_preferred(int in_dtype, const Dims& d) {
    if (!state_scan_supported(in_dtype, d)) return false;
    constexpr long kComputeUnits = 256;
    const long w = (long)d.batch * d.nheads * (d.headdim / 64);
    if (w < kComputeUnits) return false;
    const long rounds = (w + kComputeUnits - 1) / kComputeUnits;
    const double fill = (double)w / (double)(rounds * kComputeUnits);
    return fill >= (d.dstate == 256 ? 0.6 : 0.75);
}

hipError_t launch_state_scan(int states_dtype, const void* x, const void* Bm, const float* A,
                             const float* dt_t, const float* h0, void* states,
                             float* final_state, const Dims& d, hipStream_t s) {
    if (states_dtype == kBF16)
        return launch_state_scan_bf16(x, Bm, A, dt_t, h0, states, final_state, d, s);
    return launch_state_scan_bf16_f32(x, Bm, A, dt_t, h0, states, final_state, d, s);
}

}  // namespace ssd
