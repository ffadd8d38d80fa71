// Transpose kernel instances for 4-byte elements (see transpose.hpp).
#include "transpose.hpp"

namespace tc {
TC_TRANSPOSE_DISPATCH(4)
}  // namespace tc
