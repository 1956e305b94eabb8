// Host-side pieces of the dense verification forward shared by the C-ABI
// sources (include/spec_verify.h, include/spec_verify_cycle.h): the model
// handle, workspace sizes and the enqueue sequences.  Nothing here
// allocates, synchronises or reads device data.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kernels.hpp"
#include "spec_verify.h"

struct sv_model {
    sv_model_desc desc;
};

namespace sv {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int hip_fail(hipError_t e, const char* what);
bool temp_ok(float T);

// Workspace of run_forward for M rows, and of run_accept for B requests of
// K drafts over a vocabulary of V.
size_t forward_bytes(const sv_model_desc& d, int M);
size_t accept_bytes(int B, int K, int V);

// Forward of M rows of hidden [M, d] fp32 to logits [M, V] fp32; the
// verification's vocabulary stage.  Arguments are checked by the callers.
int run_forward(const sv_model_desc& d, const float* hidden, int M, float* logits, char* ws,
                hipStream_t s);
int run_accept(const float* tl, const float* dl, const int32_t* x, int B, int K, int V, float T,
               uint64_t seed, uint32_t step, int32_t* out, int32_t* al, float* p_at, float* q_at,
               char* ws, hipStream_t s);
// Host checks of spec_verify_accept's arguments (sizes, temperature, null
// pointers); SV_OK or the failure recorded for spec_verify_last_error.
int check_accept_args(const float* tl, const float* dl, const int32_t* x, int B, int K, int V,
                      float T, const int32_t* out, const int32_t* al);

}  // namespace sv
