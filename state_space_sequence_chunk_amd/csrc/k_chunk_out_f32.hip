// Stage 3 kernel instances for inputs float and chunk-initial states float (template in chunk_out.h).
#include "chunk_out.h"

namespace ssd {

hipError_t launch_chunk_out_f32(const void* x, const void* Bm, const void* Cm, const float* G,
                             const float* dt_t, const void* states, const float* D, void* y,
                             const Dims& d, hipStream_t s) {
    return out_by_p<float, float, float>(x, Bm, Cm, G, dt_t, states, D, y, d, s);
}

}  // namespace ssd
