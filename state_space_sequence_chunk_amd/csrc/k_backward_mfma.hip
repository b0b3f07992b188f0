// Matrix-core backward kernels (bf16 inputs; templates in bwd_mfma.h), and the chunk
// length they run at. The backward pass may use a chunk length of its own: the chunked
// form is exact for any length, and 64 or 128 tokens keep the split operands in LDS.
// Shapes with no plan here take the fp32 token walks at the caller's chunk length.
#include "bwd_mfma.h"

namespace ssd {

// 128 tokens where the plan fits (64 for headdim 128, whose 128-token dx kernel would
// spill registers)
template <int P, int S>
constexpr int mfma_chunk() {
    return P <= 64 && bwd_mfma_fits<P, S, 128>() ? 128 : bwd_mfma_fits<P, S, 64>() ? 64 : 0;
}

template <int P, int S>
static hipError_t mfma_run(const BwdArgs& a, int batch, hipStream_t st) {
    constexpr int T = mfma_chunk<P, S>();
    if constexpr (T == 0) {
        return hipErrorInvalidValue;
    } else {
        if (a.T != T) return hipErrorInvalidValue;
        return run_bwd_mfma_all<P, S, T>(a, batch, st);
    }
}

#define SSD_BWD_SHAPES(X) X(64, 64) X(64, 128) X(64, 256) X(128, 64) X(128, 128)

// Chunk length of the matrix-core plan for this shape, 0 when there is none.
int bwd_mfma_chunk(int in_dtype, int P, int S) {
    if (in_dtype != kBF16) return 0;
#define SSD_CHUNK(PP, SS) \
    if (P == PP && S == SS) return mfma_chunk<PP, SS>();
    SSD_BWD_SHAPES(SSD_CHUNK)
#undef SSD_CHUNK
    return 0;
}

template <int P, int S>
static hipError_t dr_run(const BwdArgs& a, int batch, hipStream_t st) {
    constexpr int T = mfma_chunk<P, S>();
    if constexpr (T == 0) {
        return hipErrorInvalidValue;
    } else {
        if (a.T != T) return hipErrorInvalidValue;
        return run_bwd_dR_mfma<P, S, T>(a, batch, st);
    }
}

// dC, dB and dx for bf16 inputs; a.T must be bwd_mfma_chunk's choice for the shape.
hipError_t launch_bwd_mfma_bf16(const BwdArgs& a, int batch, int P, int S, hipStream_t st) {
#define SSD_RUN(PP, SS) \
    if (P == PP && S == SS) return mfma_run<PP, SS>(a, batch, st);
    SSD_BWD_SHAPES(SSD_RUN)
#undef SSD_RUN
    return hipErrorInvalidValue;
}

// The per-chunk sums dR_c (into a.R) for bf16 inputs, at the same chunk length.
hipError_t launch_bwd_dR_mfma_bf16(const BwdArgs& a, int batch, int P, int S, hipStream_t st) {
#define SSD_RUN(PP, SS) \
    if (P == PP && S == SS) return dr_run<PP, SS>(a, batch, st);
    SSD_BWD_SHAPES(SSD_RUN)
#undef SSD_RUN
    return hipErrorInvalidValue;
}

}  // namespace ssd
