// One instantiation unit per (io type, chunk); the build compiles this file
// six times with LOGLIN_IO (bf16 | f32) and LOGLIN_CHUNK (16 | 32 | 64) set.
#include "loglin_launch.hpp"

#if !defined(LOGLIN_IO) || !defined(LOGLIN_CHUNK)
#error "LOGLIN_IO and LOGLIN_CHUNK must be defined"
#endif

#define LOGLIN_NAME2(io, c) lookup_##io##_##c
#define LOGLIN_NAME(io, c) LOGLIN_NAME2(io, c)
#define LOGLIN_TYPE_bf16 bf16
#define LOGLIN_TYPE_f32 float
#define LOGLIN_TYPE2(io) LOGLIN_TYPE_##io
#define LOGLIN_TYPE(io) LOGLIN_TYPE2(io)

namespace loglin {
LaunchFn LOGLIN_NAME(LOGLIN_IO, LOGLIN_CHUNK)(int P, int N) {
  return lookup<LOGLIN_TYPE(LOGLIN_IO), LOGLIN_CHUNK>(P, N);
}
}  // namespace loglin
