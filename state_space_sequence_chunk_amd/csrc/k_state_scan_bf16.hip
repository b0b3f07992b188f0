// Single-pass state kernel instances for bf16 inputs and bf16 chunk-initial states
// (template in state_scan.h).
#include "state_scan.h"

namespace ssd {

hipError_t launch_state_scan_bf16(const void* x, const void* Bm, const float* A,
                                  const float* dt_t, const float* h0, void* states, float* fin,
                                  const Dims& d, hipStream_t s) {
    return scan_by_p<bf16>(x, Bm, A, dt_t, h0, states, fin, d, s);
}

}  // namespace ssd
