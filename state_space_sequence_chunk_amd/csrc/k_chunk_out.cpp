// Stage 3 dispatch on the input, state and output dtypes.
#include "ssd_launch.h"

namespace ssd {

hipError_t launch_chunk_out_bf16(const void*, const void*, const void*, const float*, const float*,
                                 const void*, const float*, void*, const Dims&, hipStream_t);
hipError_t launch_chunk_out_bf16_f32(const void*, const void*, const void*, const float*,
                                     const float*, const void*, const float*, void*, const Dims&,
                                     hipStream_t);
hipError_t launch_chunk_out_bf16_ybf16(const void*, const void*, const void*, const float*,
                                       const float*, const void*, const float*, void*,
                                       const Dims&, hipStream_t);
hipError_t launch_chunk_out_f32(const void*, const void*, const void*, const float*, const float*,
                                const void*, const float*, void*, const Dims&, hipStream_t);

hipError_t launch_chunk_out(int in_dtype, int states_dtype, int out_dtype, const void* x,
                            const void* Bm, const void* Cm, const float* G, const float* dt_t,
                            const void* states, const float* D, void* y, const Dims& d,
                            hipStream_t s) {
    if (out_dtype == kBF16) {
        if (in_dtype == kBF16 && states_dtype == kBF16)
            return launch_chunk_out_bf16_ybf16(x, Bm, Cm, G, dt_t, states, D, y, d, s);
        return hipErrorInvalidValue;
    }
    if (in_dtype == kBF16 && states_dtype == kBF16)
        return launch_chunk_out_bf16(x, Bm, Cm, G, dt_t, states, D, y, d, s);
    if (in_dtype == kBF16 && states_dtype == kF32)
        return launch_chunk_out_bf16_f32(x, Bm, Cm, G, dt_t, states, D, y, d, s);
    if (in_dtype == kF32 && states_dtype == kF32)
        return launch_chunk_out_f32(x, Bm, Cm, G, dt_t, states, D, y, d, s);
    return hipErrorInvalidValue;
}

}  // namespace ssd
