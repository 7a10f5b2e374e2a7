// Decode kernels for bf16 at head size 128 (one translation unit per
// (element type, head size), so the instances compile in parallel).

#include "decode_impl.h"

namespace pka {
PKA_DECODE_INSTANTIATE(BF16, 128)
}  // namespace pka
