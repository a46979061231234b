// Instantiations of the log-linear gated DeltaNet forward: io type x key
// dimension N x value dimension P.
#include "loglin_gdn.hpp"

namespace loglin {

template <class T>
GdnFn lookup_gdn_t(int N, int P) {
#define LOGLIN_GCASE(NN, PP) \
  if (N == NN && P == PP) return &launch_gdn<T, NN, PP>;
  LOGLIN_GCASE(16, 16) LOGLIN_GCASE(16, 32) LOGLIN_GCASE(16, 64)
  LOGLIN_GCASE(32, 16) LOGLIN_GCASE(32, 32) LOGLIN_GCASE(32, 64)
  LOGLIN_GCASE(64, 16) LOGLIN_GCASE(64, 32) LOGLIN_GCASE(64, 64)
  LOGLIN_GCASE(128, 16) LOGLIN_GCASE(128, 32) LOGLIN_GCASE(128, 64)
#undef LOGLIN_GCASE
  return nullptr;
}

GdnFn lookup_gdn(int dtype, int N, int P) {
  return dtype == 1 ? lookup_gdn_t<bf16>(N, P) : lookup_gdn_t<float>(N, P);
}

}  // namespace loglin
