// sv_sample_noalloc: sv_sample with its scratch in a static device array
// instead of a caller-supplied workspace, for callers that cannot allocate
// device memory. The kernels are those of sv_sample; they take the array's
// device address as they take the workspace pointer there.
#include <mutex>

#include "sv_internal.h"

namespace sv {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The scratch. Each GPU the library runs on holds its own copy at its own
// address for the life of the process. In host code the name is only a
// stand-in: kernels are given the address hipGetSymbolAddress returns for the
// current device, never the name.
static __device__ __align__(256) char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];   // per device, looked up on first use

// The device address of `scratch` on the current device (nullptr on failure).
static char* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return (char*)g_scratch_ptr[dev];
}

}  // namespace sv

using namespace sv;

extern "C" int sv_sample_noalloc(const sv_problem* prob, const int32_t* parent,
                                 const int32_t* node_token, const float* logits,
                                 const float* draft_logits, const float* uniforms,
                                 const float* temperature, int32_t* accept_len,
                                 int32_t* accept_path, int32_t* out_tokens, int32_t* seq_status,
                                 const sv_debug* dbg, sv_stream_t stream) {
  Plan P;
  int rc = make_plan(prob, &P, /*sampling_only=*/true);
  if (rc != SV_OK) return rc;
  rc = check_sample_args(P, parent, node_token, logits, draft_logits, uniforms, temperature,
                         accept_len, accept_path, out_tokens, seq_status);
  if (rc != SV_OK) return rc;
  if (P.total > kScratchBytes) return SV_ERR_SCRATCH;
  char* ws = scratch_on_current_device();
  if (ws == nullptr) return SV_ERR_HIP;
  return sample_call(P, parent, node_token, logits, draft_logits, uniforms, temperature,
                     accept_len, accept_path, out_tokens, seq_status, dbg, ws,
                     (hipStream_t)stream);
}
