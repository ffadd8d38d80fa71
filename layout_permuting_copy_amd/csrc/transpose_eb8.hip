// Transpose kernel instances for 8-byte elements (see transpose.hpp).
#include "transpose.hpp"

namespace tc {
TC_TRANSPOSE_DISPATCH(8)
}  // namespace tc
