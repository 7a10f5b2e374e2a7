// Decode kernels for f16 at head size 64 (one translation unit per
// (element type, head size), so the instances compile in parallel).

#include "decode_impl.h"

namespace pka {
PKA_DECODE_INSTANTIATE(F16, 64)
}  // namespace pka
