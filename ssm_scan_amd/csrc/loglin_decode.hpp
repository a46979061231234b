// One-token decode step of log-linear Mamba-2: declarations shared by the
// host unit and the kernel unit.
#pragma once

#include <cstdint>

namespace loglin {

struct DecodeParams {
  const void* X;      // [B, H, P]  io type, token t
  const void* Bm;     // [B, G, N]
  const void* Cm;     // [B, G, N]
  const float* log_a; // [B, H]
  const void* lam;    // [B, H, L]
  void* out;          // [B, H, P]
  float* S;           // [B, H, LL, P/4, N, 4] level states (fp32, stored without their decay)
  float* gd;          // [B, H, 2, LL] per-level decay factors; bank t & 1 is read at step t
  int batch, nheads, ngroups, nlevels, ll;
  int64_t t;
};

using DecodeFn = int (*)(const DecodeParams&, void* stream);

// Launcher for (io dtype, P, N); nullptr when the shape is not supported.
DecodeFn lookup_decode(int dtype, int P, int N);

}  // namespace loglin
