// attn_bwd_noalloc: the backward with its workspace in a static device array
// instead of a caller buffer, for callers that cannot allocate (graph
// capture, serving loops).  The kernels are attn_bwd's; only the workspace
// pointer differs.
#include <mutex>

#include "launch.h"
#include "sdpa_attn.h"

namespace {

// The scratch: one copy per GPU, loaded with the library's code object.
// Host code never uses the name as an address (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, per device, below.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of the current device's scratch, looked up on the first
// call on that device (with it current) and kept.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::call_once(g_once[dev], [dev] {
    void* ptr = nullptr;
    g_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_err[dev] != hipSuccess || !g_scratch[dev]) return ATTN_ERR_HIP;
  *out = g_scratch[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd_noalloc(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
                                const void* d_o, const float* lse, const float* softmax_offset,
                                const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk, void* dv,
                                float* d_softmax_offset, void* stream) {
  // Host checks before any HIP call: the problem, the pointers, the size.
  const int rc = attn_validate(p);
  if (rc != ATTN_OK) return rc;
  if (p->dtype == ATTN_FP8) return ATTN_ERR_UNSUPPORTED;  // the bf16 / fp32 backward only
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (attn_bwd_workspace_size(p) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int e = scratch_ptr(&ws);
  if (e != ATTN_OK) return e;
  // The minimum workspace size: dQ recomputes S and dP, as attn_bwd does with
  // a workspace of attn_bwd_workspace_size bytes (no stored dS).
  return sdpa::bwd_run(0, p, q, k, v, o, d_o, lse, softmax_offset, seqlens, seq_offsets, dq, dk, dv,
                       d_softmax_offset, ws, attn_bwd_workspace_size(p), stream, nullptr);
}
