// Stage 3 kernel instances over segment-relative bf16 chunk states, fp32 and bf16 y
// (template in chunk_out.h).
#include "chunk_out.h"

namespace ssd {

hipError_t launch_chunk_out_seg(int out_dtype, const void* x, const void* Bm, const void* Cm,
                                const float* G, const float* dt_t, const void* states,
                                const void* seg_in, const float* dec_in, int seg_chunks,
                                const float* D, void* y, const Dims& d, hipStream_t s) {
    if (out_dtype == kBF16)
        return out_seg<bf16>(x, Bm, Cm, G, dt_t, states, seg_in, dec_in, seg_chunks, D, y, d, s);
    return out_seg<float>(x, Bm, Cm, G, dt_t, states, seg_in, dec_in, seg_chunks, D, y, d, s);
}

}  // namespace ssd
