// One backward instantiation unit per (io type, chunk); the build compiles
// this file with LOGLIN_IO (bf16 | f32) and LOGLIN_CHUNK set (bf16 chunks
// 32 and 64, f32 chunks 16, 32 and 64).
#include "loglin_bwd.hpp"

#if !defined(LOGLIN_IO) || !defined(LOGLIN_CHUNK)
#error "LOGLIN_IO and LOGLIN_CHUNK must be defined"
#endif

#define LOGLIN_BNAME2(io, c) lookup_bwd_##io##_##c
#define LOGLIN_BNAME(io, c) LOGLIN_BNAME2(io, c)
#define LOGLIN_TYPE_bf16 bf16
#define LOGLIN_TYPE_f32 float
#define LOGLIN_TYPE2(io) LOGLIN_TYPE_##io
#define LOGLIN_TYPE(io) LOGLIN_TYPE2(io)

namespace loglin {
BwdFn LOGLIN_BNAME(LOGLIN_IO, LOGLIN_CHUNK)(int P, int N) {
  return lookup_bwd<LOGLIN_TYPE(LOGLIN_IO), LOGLIN_CHUNK>(P, N);
}
}  // namespace loglin
