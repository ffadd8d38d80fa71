// Transpose kernel instances for 16-byte elements (see transpose.hpp).
#include "transpose.hpp"

namespace tc {
TC_TRANSPOSE_DISPATCH(16)
}  // namespace tc
