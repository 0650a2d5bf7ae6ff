// Sparse attention backward (placeholder until the kernels land).
#include "bsa_internal.h"

namespace bsa {

BackwardWs carve_backward(const Problem& p, int64_t capacity, void* ws, size_t* bytes) {
  (void)p; (void)capacity; (void)ws;
  *bytes = 0;
  return BackwardWs{};
}

hipError_t launch_backward(const Problem&, const void*, const void*, const void*, const void*, const void*,
                           const float*, float, const bsa_csr*, void*, void*, void*, const BackwardWs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace bsa
