// Backward per-chunk kernel instances for bf16 inputs (templates in backward.h).
#include "backward.h"

namespace ssd {

hipError_t launch_bwd_chunks_bf16(const BwdArgs& a, int batch, int P, int S, bool f, bool r,
                                  bool v, hipStream_t st) {
    return bwd_chunks<bf16>(a, batch, P, S, f, r, v, st);
}

}  // namespace ssd
