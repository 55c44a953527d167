// Backward-pass instances for 16-bit inputs (bf16, fp16) and the dispatch.
#include "fa_bwd_impl.h"

namespace fa {

hipError_t launch_backward_f32(const Problem& p, const BwdTensors& t);  // fa_bwd_f32.hip

hipError_t launch_backward(const Problem& p, const BwdTensors& t) {
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

}  // namespace fa
