// Kernel launch sequence for one (io type, chunk, P, N) instantiation.
#pragma once

#include "loglin_device.hpp"
#include "loglin_out2.hpp"

namespace loglin {

using LaunchFn = int (*)(const Params&, hipStream_t, void* const*);

inline int pad8(int n) { return (n + 7) & ~7; }

inline void record(void* const* ev, int i, hipStream_t st) {
  if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), st);
}

template <class T, int C, int P, int N, int HP>
void launch_output(Params pr, hipStream_t st) {
  using Cfg = OutCfg<T, C, P, N, HP>;
  pr.total = pr.batch * pr.ns * (pr.nheads / HP);
  const size_t shm = (size_t)HP * C * lam_words(pr.ll, (int)sizeof(T)) * 4;
  if (pr.lmask == ~0ull)
    hipLaunchKernelGGL((output_kernel<T, C, P, N, HP, false>), dim3(pad8(pr.total)), dim3(Cfg::NT), shm, st, pr);
  else
    hipLaunchKernelGGL((output_kernel<T, C, P, N, HP, true>), dim3(pad8(pr.total)), dim3(Cfg::NT), shm, st, pr);
}

// Returns 0 or hipError_t of the first failing launch (caller maps it).
template <class T, int C, int P, int N>
int launch_forward(const Params& base, hipStream_t st, void* const* ev) {
  using Tl = Tiles<T, C, P, N>;
  Params pr = base;
  // the bf16 output pass for 64-token chunks and 64 columns reads slots in
  // natural state order; the other instantiations in state order
  constexpr bool OUT2 = sizeof(T) == 2 && C == 64 && P == 64 && (N == 64 || N == 128);
  const bool use2 = OUT2 && pr.hp != 2;
  pr.nat = use2 ? 1 : 0;
  record(ev, 0, st);
  // Levels above a segment (c + m + 1 and up) need the state pass and the
  // scan; a level mask without them (the unfused per-level variant) skips
  // both.
  const int c_log = __builtin_ctz(C);
  const bool above = (c_log + pr.m + 1 >= 64) ? false : (pr.lmask >> (c_log + pr.m + 1)) != 0;
  if (pr.ns > 1 && above) {
    // bf16 heads of one group share their B rows in one work-group
    constexpr bool SPAIRS = sizeof(T) == 2;
    if (OUT2 && use2 && (pr.nheads / pr.ngroups) % 2 == 0) {
      // the output pass's shape: the same LDS layouts as there
      constexpr int NN = OUT2 ? N : 128;
      pr.total = pr.batch * pr.ns * (pr.nheads / 2);
      hipLaunchKernelGGL((state2_kernel<NN>), dim3(pad8(pr.total)), dim3(512), 0, st, pr);
    } else if (SPAIRS && (pr.nheads / pr.ngroups) % 2 == 0) {
      pr.total = pr.batch * pr.ns * (pr.nheads / 2);
      hipLaunchKernelGGL((state_kernel<T, C, P, N, SPAIRS ? 2 : 1>), dim3(pad8(pr.total)),
                         dim3(2 * Tl::NT), 0, st, pr);
    } else {
      pr.total = pr.batch * pr.nheads * pr.ns;
      hipLaunchKernelGGL((state_kernel<T, C, P, N, 1>), dim3(pad8(pr.total)), dim3(Tl::NT), 0, st, pr);
    }
    record(ev, 1, st);
    constexpr int E = 16 / (int)sizeof(T);  // state elements per scan thread
    static_assert((P * N) % (64 * E) == 0, "a scan wave covers 64 E state elements");
    dim3 g2((P * N + E * SCAN_NT - 1) / (E * SCAN_NT), pr.batch * pr.nheads);
    dim3 g3(P * N / (64 * E), pr.batch * pr.nheads);  // one wave's elements per work-group
    if (pr.ns <= SCAN_RMAX * SCAN_L)  // ranges of SCAN_L segments side by side
      hipLaunchKernelGGL((scan_range_kernel<T, N, SCAN_L>), g3, dim3(64 * ((pr.ns + SCAN_L - 1) / SCAN_L)), 0, st,
                         pr, P * N);
    else if (pr.ns < (1 << 10))  // a stack of 10 block sums covers fewer than 2^10 segments
      hipLaunchKernelGGL((scan_kernel<T, N, 10>), g2, dim3(SCAN_NT), 0, st, pr, P * N);
    else
      hipLaunchKernelGGL((scan_kernel<T, N, MAX_DEPTH>), g2, dim3(SCAN_NT), 0, st, pr, P * N);
  } else {
    record(ev, 1, st);
  }
  record(ev, 2, st);
  // pairs of heads of one group (shared B, C and scores) where requested;
  // the host only accepts that for bf16 with 64 columns
  constexpr bool PAIRS = sizeof(T) == 2 && P == 64;
  if (use2) {
    constexpr int NN = OUT2 ? N : 128;
    // batch x groups of 8 segments x 8 XCDs x heads (see output2_kernel)
    const int grid = pr.batch * ((pr.ns + 7) / 8) * 8 * pr.nheads;
    const size_t shm = (size_t)C * lam_words(pr.ll, 2) * 4;
    if (pr.lmask == ~0ull)
      hipLaunchKernelGGL((output2_kernel<NN, false>), dim3(grid), dim3(256), shm, st, pr);
    else
      hipLaunchKernelGGL((output2_kernel<NN, true>), dim3(grid), dim3(256), shm, st, pr);
  } else if (PAIRS && pr.hp == 2)
    launch_output<T, C, P, N, PAIRS ? 2 : 1>(pr, st);
  else
    launch_output<T, C, P, N, 1>(pr, st);
  record(ev, 3, st);
  return (int)hipGetLastError();
}

template <class T, int C>
LaunchFn lookup(int P, int N) {
#define LOGLIN_CASE(PP, NN) \
  if (P == PP && N == NN) return &launch_forward<T, C, PP, NN>;
  LOGLIN_CASE(16, 32) LOGLIN_CASE(16, 64) LOGLIN_CASE(16, 128)
  LOGLIN_CASE(32, 32) LOGLIN_CASE(32, 64) LOGLIN_CASE(32, 128)
  LOGLIN_CASE(64, 32) LOGLIN_CASE(64, 64) LOGLIN_CASE(64, 128)
  if constexpr (sizeof(T) == 4) {
    LOGLIN_CASE(16, 16) LOGLIN_CASE(32, 16) LOGLIN_CASE(64, 16)
  }
#undef LOGLIN_CASE
  return nullptr;
}

// Defined in one translation unit per (io type, chunk).
LaunchFn lookup_bf16_16(int P, int N);
LaunchFn lookup_bf16_32(int P, int N);
LaunchFn lookup_bf16_64(int P, int N);
LaunchFn lookup_f32_16(int P, int N);
LaunchFn lookup_f32_32(int P, int N);
LaunchFn lookup_f32_64(int P, int N);

}  // namespace loglin
