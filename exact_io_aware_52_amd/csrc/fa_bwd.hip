// Backward-pass instances for 16-bit inputs (bf16, fp16), the dispatch, and
// the device-resident scratch of the allocation-free backward entry point.
#include <mutex>

#include "fa_bwd_impl.h"

namespace fa {

hipError_t launch_backward_f32(const Problem& p, const BwdTensors& t);  // fa_bwd_f32.hip

hipError_t launch_backward(const Problem& p, const BwdTensors& t) {
  if (p.chunk_blocks > 0) {  // block-sparse split (16-bit types; checked by the caller)
    switch (p.dtype * 1000 + p.d) {
      case 1 * 1000 + 64: return launch_bwd_t<_Float16, 64, false, true>(p, t);
      case 1 * 1000 + 128: return launch_bwd_t<_Float16, 128, false, true>(p, t);
      case 2 * 1000 + 64: return launch_bwd_t<__bf16, 64, false, true>(p, t);
      case 2 * 1000 + 128: return launch_bwd_t<__bf16, 128, false, true>(p, t);
    }
    return hipErrorInvalidValue;
  }
  switch (p.dtype * 1000 + p.d) {
    case 0 * 1000 + 64:
    case 0 * 1000 + 128: return launch_backward_f32(p, t);
    case 1 * 1000 + 64:
      return p.grad_f32 ? launch_bwd_t<_Float16, 64, true>(p, t) : launch_bwd_t<_Float16, 64>(p, t);
    case 1 * 1000 + 128:
      return p.grad_f32 ? launch_bwd_t<_Float16, 128, true>(p, t)
                        : launch_bwd_t<_Float16, 128>(p, t);
    case 2 * 1000 + 64:
      return p.grad_f32 ? launch_bwd_t<__bf16, 64, true>(p, t) : launch_bwd_t<__bf16, 64>(p, t);
    case 2 * 1000 + 128:
      return p.grad_f32 ? launch_bwd_t<__bf16, 128, true>(p, t) : launch_bwd_t<__bf16, 128>(p, t);
  }
  return hipErrorInvalidValue;
}

// Scratch for fa_backward_noalloc: the backward workspace (-D and
// LSE * log2(e), 8 bytes per query row) in a file-scope device array, so that
// callers that cannot allocate need not supply one.  Each GPU the library
// runs on holds its own copy until the process ends.  Its address on a
// device comes from hipGetSymbolAddress, taken once per device with that
// device current; host code never passes the array's own name to a kernel
// (on the host that name is only a stand-in, not a device address).
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_workspace(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
