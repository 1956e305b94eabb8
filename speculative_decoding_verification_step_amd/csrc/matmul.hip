// Dispatch of the weight-streaming matmuls to a kernel family.  Each launch
// below opens a timing scope with its algorithmic bytes (weights once +
// activations + outputs; a residual is read and written) and flops.
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

hipError_t launch_gemv(const MatmulArgs& a, hipStream_t stream);
hipError_t launch_mfma_skinny(const MatmulArgs& a, hipStream_t stream);
hipError_t launch_mfma_tiled(const MatmulArgs& a, hipStream_t stream);

namespace {

const char* scope_name(int kind, int epi) {
    static const char* names[3][3] = {
        {"gemv_valu.up_silu", "gemv_valu.down_residual", "gemv_valu.head"},
        {"mfma_skinny.up_silu", "mfma_skinny.down_residual", "mfma_skinny.head"},
        {"mfma_tiled.up_silu", "mfma_tiled.down_residual", "mfma_tiled.head"},
    };
    return names[kind][epi];
}

}  // namespace

hipError_t launch_matmul(const MatmulArgs& a, int kind, hipStream_t stream) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (kind < 0 || kind > 2 || a.epi < 0 || a.epi > 2) return hipErrorInvalidValue;
    MatmulArgs b = a;
    b.name = a.name ? a.name : scope_name(kind, a.epi);
    switch (kind) {
        case kGemvValu: return launch_gemv(b, stream);
        case kMfmaSkinny: return launch_mfma_skinny(b, stream);
        default: return launch_mfma_tiled(b, stream);
    }
}

}  // namespace sv

namespace sv {

double matmul_bytes(const MatmulArgs& a, int rows) {
    const double es = a.bf16 ? 2.0 : 4.0;
    const double out_es = a.epi == kEpiSilu ? es : 4.0;
    return (double)a.N * a.K * es + (double)rows * a.K * es +
           (double)rows * a.N * out_es * (a.epi == kEpiResidual ? 2 : 1);
}

}  // namespace sv
