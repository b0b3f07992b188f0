// Stage 3 dispatch on the input, state and output dtypes, and the host-side plan query.
#include "chunk_out.h"

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

namespace {
template <typename TIn, typename TS, bool SEGC, int P, int S>
bool plan_t(const Dims& d, OutPlan* o) {
    switch (d.chunk) {
        case 64: *o = out_plan_t<TIn, TS, P, S, 64, SEGC>(d); return true;
        case 128: *o = out_plan_t<TIn, TS, P, S, 128, SEGC>(d); return true;
        case 256: *o = out_plan_t<TIn, TS, P, S, 256, SEGC>(d); return true;
    }
    return false;
}
template <typename TIn, typename TS, bool SEGC, int P>
bool plan_s(const Dims& d, OutPlan* o) {
    switch (d.dstate) {
        case 16: return plan_t<TIn, TS, SEGC, P, 16>(d, o);
        case 32: return plan_t<TIn, TS, SEGC, P, 32>(d, o);
        case 64: return plan_t<TIn, TS, SEGC, P, 64>(d, o);
        case 128: return plan_t<TIn, TS, SEGC, P, 128>(d, o);
        case 256: return plan_t<TIn, TS, SEGC, P, 256>(d, o);
    }
    return false;
}
template <typename TIn, typename TS, bool SEGC>
bool plan_p(const Dims& d, OutPlan* o) {
    switch (d.headdim) {
        case 16: return plan_s<TIn, TS, SEGC, 16>(d, o);
        case 32: return plan_s<TIn, TS, SEGC, 32>(d, o);
        case 64: return plan_s<TIn, TS, SEGC, 64>(d, o);
        case 128: return plan_s<TIn, TS, SEGC, 128>(d, o);
    }
    return false;
}
}  // namespace

bool chunk_out_plan(int in_dtype, int states_dtype, bool segc, const Dims& d, OutPlan* o) {
    if (in_dtype == kBF16 && states_dtype == kBF16)
        return segc ? plan_p<bf16, bf16, true>(d, o) : plan_p<bf16, bf16, false>(d, o);
    if (segc) return false;
    if (in_dtype == kBF16 && states_dtype == kF32) return plan_p<bf16, float, false>(d, o);
    if (in_dtype == kF32 && states_dtype == kF32) return plan_p<float, float, false>(d, o);
    return false;
}

}  // namespace ssd
