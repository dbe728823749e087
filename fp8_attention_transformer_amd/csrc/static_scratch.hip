// sage_attn_fwd_static: the attention forward of sage_attn_fwd with its
// workspace in a fixed device array of the library, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Declared in include/sage.h.
#include "sage.h"

#include <mutex>

#include <hip/hip_runtime.h>

namespace {

constexpr size_t kScratchBytes = SAGE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The prepass buffers of every call of sage_attn_fwd_static on a GPU.  Each
// GPU the library runs on holds its own copy until the process ends.  In host
// code this name only stands for the symbol: the device address of a GPU's
// copy comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

extern "C" sage_status sage_attn_fwd_static(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                                            int D, int causal, float sm_scale, int qk_bits, int smooth_v,
                                            sage_dtype in_dtype, sage_dtype out_dtype, hipStream_t stream) {
  const size_t need = sage_workspace_bytes(B, H, N, D);
  if (need == 0) return SAGE_ERR_INVALID;
  if (need > kScratchBytes) return SAGE_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  // first call on this device (it is current): the address of its copy
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess || !g_ptr[dev]) return SAGE_ERR_HIP;
  // Nothing in the array needs to start at zero: the prepass writes every
  // element the fused kernel reads.
  return sage_attn_fwd(q, k, v, o, B, H, N, D, causal, sm_scale, qk_bits, smooth_v, in_dtype, out_dtype, g_ptr[dev],
                       kScratchBytes, stream);
}
