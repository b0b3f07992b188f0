// Backward per-chunk kernel instances for float inputs (templates in backward.h).
#include "backward.h"

namespace ssd {

hipError_t launch_bwd_chunks_f32(const BwdArgs& a, int batch, int P, int S, bool f, bool r,
                                  bool v, hipStream_t st) {
    return bwd_chunks<float>(a, batch, P, S, f, r, v, st);
}

}  // namespace ssd
