// Decode kernels for f16 at head size 256 (one translation unit per
// (element type, head size), so the instances compile in parallel).

#include "decode_impl.h"

namespace pka {
PKA_DECODE_INSTANTIATE(F16, 256)
}  // namespace pka
