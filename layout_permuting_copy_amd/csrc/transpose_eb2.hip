// Transpose kernel instances for 2-byte elements (see transpose.hpp).
#include "transpose.hpp"

namespace tc {
TC_TRANSPOSE_DISPATCH(2)
}  // namespace tc
