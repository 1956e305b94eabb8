// spec_verify_accept_noalloc: the rejection-sampling stage for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its scratch -- the per-chunk
// softmax statistics, draw-weight sums and per-request draw parameters that
// spec_verify_accept keeps in the caller's workspace -- lives in a static
// device array of kScratchBytes per GPU, held until the process ends.
//
// The array's host-side name is only a handle: kernels receive the device
// address that hipGetSymbolAddress resolves, once per device with that
// device current, on the first call there.  Every call on a GPU shares that
// GPU's array, so calls that overlap on one GPU race; nothing in it needs to
// start at zero (each call writes every statistic and draw value before it
// reads it).
#include <mutex>

#include "host.hpp"
#include "kernels.hpp"
#include "model.hpp"
#include "spec_verify.h"

namespace sv {

namespace {

constexpr size_t kScratchBytes = SV_ACCEPT_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];       // device address of `scratch`, per device

// Device address of the current device's scratch array (resolved on the
// first call on that device).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SV_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SV_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

}  // namespace

}  // namespace sv

using namespace sv;

extern "C" int spec_verify_accept_noalloc(const float* target_logits, const float* draft_logits,
                                          const int32_t* draft_tokens, int32_t B, int32_t K,
                                          int32_t V, float temperature, uint64_t seed,
                                          uint32_t step, int32_t* out_tokens,
                                          int32_t* accept_len, float* p_at_draft,
                                          float* q_at_draft, void* stream) {
    int rc = check_accept_args(target_logits, draft_logits, draft_tokens, B, K, V, temperature,
                               out_tokens, accept_len);
    if (rc != SV_OK || B == 0) return rc;
    const size_t need = accept_bytes(B, K, V);
    if (need > kScratchBytes)
        return fail(SV_ERR_WORKSPACE,
                    "B=%d K=%d V=%d needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use spec_verify_accept with a workspace)",
                    B, K, V, need, kScratchBytes);
    void* p = nullptr;
    rc = scratch_address(&p);
    if (rc != SV_OK) return rc;
    return run_accept(target_logits, draft_logits, draft_tokens, B, K, V, temperature, seed, step,
                      out_tokens, accept_len, p_at_draft, q_at_draft, static_cast<char*>(p),
                      static_cast<hipStream_t>(stream));
}
