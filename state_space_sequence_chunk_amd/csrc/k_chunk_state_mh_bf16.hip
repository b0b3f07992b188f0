// Stage 2a multi-head kernel instances for bf16 inputs (template in chunk_state_mh.h).
#include "chunk_state_mh.h"

namespace ssd {

bool launch_chunk_state_mh_bf16(const void* x, const void* Bm, const float* A, const float* dt_t,
                            float* dS, const Dims& d, hipStream_t s, hipError_t* err) {
    return state_mh_by_p<bf16>(x, Bm, A, dt_t, dS, d, s, err);
}

}  // namespace ssd
