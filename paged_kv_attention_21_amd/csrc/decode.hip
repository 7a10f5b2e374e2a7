// Decode dispatch: picks the (element type, head size) instance of the decode
// kernels (compiled separately in decode_<type>_d<size>.hip, whose kernels are
// defined in decode_impl.h).

#include "decode_impl.h"

namespace pka {

PKA_DECODE_FOR_ALL(PKA_DECODE_EXTERN)

hipError_t launch_decode(const DecodeArgs& a, int mode, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim == 64) return launch_decode_td<BF16, 64>(a, mode, stream);
    if (a.head_dim == 128) return launch_decode_td<BF16, 128>(a, mode, stream);
    if (a.head_dim == 256) return launch_decode_td<BF16, 256>(a, mode, stream);
  } else {
    if (a.head_dim == 64) return launch_decode_td<F16, 64>(a, mode, stream);
    if (a.head_dim == 128) return launch_decode_td<F16, 128>(a, mode, stream);
    if (a.head_dim == 256) return launch_decode_td<F16, 256>(a, mode, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const ReduceArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim == 64) return launch_splitk_reduce_td<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_splitk_reduce_td<BF16, 128>(a, stream);
    if (a.head_dim == 256) return launch_splitk_reduce_td<BF16, 256>(a, stream);
  } else {
    if (a.head_dim == 64) return launch_splitk_reduce_td<F16, 64>(a, stream);
    if (a.head_dim == 128) return launch_splitk_reduce_td<F16, 128>(a, stream);
    if (a.head_dim == 256) return launch_splitk_reduce_td<F16, 256>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pka
