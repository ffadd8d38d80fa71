// Transpose kernel instances for 1-byte elements (see transpose.hpp).
#include "transpose.hpp"

namespace tc {
TC_TRANSPOSE_DISPATCH(1)
}  // namespace tc
