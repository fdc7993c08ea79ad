// Decode attention that allocates nothing and takes no workspace: the chunk
// partials of attn_decode_quant live in a library-owned device array instead
// of a caller workspace.  For callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` is one file-scope device array; each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the name `scratch` is only a host-side stand-in, so the device address
// of the current GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what the
// kernels receive.  Every call on one GPU shares its copy: calls that overlap
// on one GPU (two streams, two host threads) race on it.  Nothing in it must
// start at zero: the decode kernels write every partial the combine reads in
// the same call.
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr size_t kScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device ordinal

// Device address of the current GPU's copy of `scratch` (looked up on the
// first call on that device, with the device current).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status attn_decode_quant_noalloc(const kvq_cache* kv, const float* q,
                                                int32_t n_q_heads, float sm_scale, float* out,
                                                float* lse, void* stream) {
    AttnPlan plan;
    const kvq_status rs = decode_request(kv, q, n_q_heads, out, lse, plan);
    if (rs != KVQ_OK) return rs;
    // a decode whose wide (all heads per workgroup) plan does not fit runs
    // per head group, whose partials do
    if (plan.ws_bytes > kScratchBytes && plan.heads_per_blk == 64) plan = make_plan(*kv, n_q_heads, 1, q, false);
    if (plan.ws_bytes > kScratchBytes) return KVQ_ERR_SCRATCH;
    void* ws = nullptr;
    if (plan.ws_bytes > 0 && scratch_address(&ws) != hipSuccess) return KVQ_ERR_LAUNCH;
    const hipError_t e = launch_attention(*kv, plan, q, 1, n_q_heads, -1, sm_scale, out, lse, ws,
                                          (hipStream_t)stream);
    return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}
