// Stage 2a multi-head kernel instances for float inputs (template in chunk_state_mh.h).
#include "chunk_state_mh.h"

namespace ssd {

bool launch_chunk_state_mh_f32(const void* x, const void* Bm, const float* A, const float* dt_t,
                            float* dS, const Dims& d, hipStream_t s, hipError_t* err) {
    return state_mh_by_p<float>(x, Bm, A, dt_t, dS, d, s, err);
}

}  // namespace ssd
