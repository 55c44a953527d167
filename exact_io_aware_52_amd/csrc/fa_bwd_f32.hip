// Backward-pass instances for fp32 inputs (the accuracy path).  Built without
// the VGPR-form matrix-core option (see build_lib.py).
#include "fa_bwd_impl.h"

namespace fa {

hipError_t launch_backward_f32(const Problem& p, const BwdTensors& t) {
  if (p.d == 64) return launch_bwd_t<float, 64>(p, t);
  if (p.d == 128) return launch_bwd_t<float, 128>(p, t);
  return hipErrorInvalidValue;
}

}  // namespace fa
