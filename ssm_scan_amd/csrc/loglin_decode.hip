// One-token decode step of log-linear Mamba-2 on gfx950.
//
// Log-linear attention write-up (yoousoft.com/industry/3746), section
// "log-linear attention" and "special structure: tree partition": decoding
// keeps one state per Fenwick bucket of the prefix, O(log T) of them, and
// the output weights the bucket memories by the token's level weights.  A
// bucket state is sum over its tokens s of decay(s -> t) B_s X_s^T (N x P).
// From t-1 to t, with z = trailing zeros of t (t > 0), the buckets of
// levels 0..z merge into level z+1, levels 1..z empty, every older bucket
// decays by a_t, and level 0 becomes {t}:
//   y_t = sum_l lambda[t, l] S_l^T C_t.
//
// Each level is stored as (S_l, g_l) with true state g_l S_l: the decay of
// untouched levels is a scalar update, so a step reads each occupied level
// once (for y and for the merge) and writes only levels 0 and z+1.  The
// g banks alternate by step parity, so the step that writes them never
// reads them.
#include <hip/hip_runtime.h>

#include "loglin.h"
#include "loglin_decode.hpp"
#include "loglin_device.hpp"

namespace loglin {

// grid: batch * heads * (P / 16) work-groups of 256 threads.  Thread
// (r, u) = (tid / 4, tid % 4) owns columns 16 pb + 4u .. +3 of the rows
// n = r + 64 k.
template <class T, int P, int N>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams dp) {
  constexpr int PB = P / 16;
  constexpr int RK = (N + 63) / 64;  // rows per thread
  const int tid = threadIdx.x, u = tid & 3, rr = tid >> 2;
  const int pb = blockIdx.x % PB;
  const int bh = blockIdx.x / PB;
  const int H = dp.nheads, G = dp.ngroups, LL = dp.ll, L = dp.nlevels;
  const int b = bh / H, h = bh % H, grp = h / (H / G);
  const int64_t t = dp.t;
  const int z = t > 0 ? __builtin_ctzll((unsigned long long)t) : -1;  // levels 0..z merge into z+1
  const float a = expf(dp.log_a[bh]);
  const T* lam = static_cast<const T*>(dp.lam) + (int64_t)bh * L;
  const T* Cv = static_cast<const T*>(dp.Cm) + ((int64_t)b * G + grp) * N;
  const T* Bv = static_cast<const T*>(dp.Bm) + ((int64_t)b * G + grp) * N;
  const T* Xv = static_cast<const T*>(dp.X) + (int64_t)bh * P;
  const float* gold = dp.gd + ((int64_t)bh * 2 + (t & 1)) * LL;
  float* S = dp.S + (int64_t)bh * LL * N * P;
  const int c0 = 16 * pb + 4 * u;  // first of this thread's 4 columns

  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = to_f(Xv[c0 + i]);
  float cn[RK], bn[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int n = rr + 64 * k;
    cn[k] = n < N ? to_f(Cv[n]) : 0.f;
    bn[k] = n < N ? to_f(Bv[n]) : 0.f;
  }
  const float lam_merge = z >= 0 ? to_f(lam[z + 1]) : 0.f;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 merged[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) merged[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (t > 0) {
    for (int l = 0; l < LL; ++l) {  // uniform loop; empty levels are skipped
      const float gl = gold[l];
      if (gl == 0.f || l == z + 1) continue;
      const bool merge = l <= z;
      const float w = (merge ? lam_merge : to_f(lam[l])) * a * gl;
      const float* Sl = S + (int64_t)l * N * P;
#pragma unroll
      for (int k = 0; k < RK; ++k) {
        const int n = rr + 64 * k;
        if (n < N) {
          const f32x4 s = *reinterpret_cast<const f32x4*>(Sl + n * P + c0);
          acc += (w * cn[k]) * s;
          if (merge) merged[k] += gl * s;
        }
      }
    }
  }
  // new level 0: the token itself, S_0 = B_t X_t^T
  {
    float bc = 0.f;
#pragma unroll
    for (int k = 0; k < RK; ++k) bc += bn[k] * cn[k];
    const float w0 = to_f(lam[0]) * bc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += w0 * x[i];
  }

  // the merged level and level 0, stored without decay factor
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int n = rr + 64 * k;
    if (n < N) {
      if (z >= 0) *reinterpret_cast<f32x4*>(S + ((int64_t)(z + 1) * N + n) * P + c0) = merged[k];
      *reinterpret_cast<f32x4*>(S + (int64_t)n * P + c0) = f32x4{bn[k] * x[0], bn[k] * x[1], bn[k] * x[2], bn[k] * x[3]};
    }
  }

  // reduce acc over the 64 row groups: lanes with equal u within a wave,
  // then the four waves through LDS
#pragma unroll
  for (int d = 4; d < 64; d <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], d, 64);
  }
  __shared__ f32x4 part[4][4];
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < 4) part[wave][lane] = acc;
  __syncthreads();
  if (tid < 4) {
    f32x4 y = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
    T* o = static_cast<T*>(dp.out) + (int64_t)bh * P + 16 * pb + 4 * tid;
    store4(o, y);
  }
  // decay factors for the next step (one work-group per head writes them)
  if (pb == 0 && tid < LL) {
    const int l = tid;
    float gn;
    if (l == 0) gn = 1.f;
    else if (t == 0 || l <= z) gn = 0.f;
    else if (l == z + 1) gn = a;
    else gn = gold[l] * a;
    dp.gd[((int64_t)bh * 2 + ((t + 1) & 1)) * LL + l] = gn;
  }
}

template <class T, int P, int N>
int launch_decode(const DecodeParams& dp, void* stream) {
  const int grid = dp.batch * dp.nheads * (P / 16);
  hipLaunchKernelGGL((decode_kernel<T, P, N>), dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dp);
  return (int)hipGetLastError();
}

template <class T>
DecodeFn lookup_decode_t(int P, int N) {
#define LOGLIN_DCASE(PP, NN) \
  if (P == PP && N == NN) return &launch_decode<T, PP, NN>;
  LOGLIN_DCASE(16, 32) LOGLIN_DCASE(16, 64) LOGLIN_DCASE(16, 128)
  LOGLIN_DCASE(32, 32) LOGLIN_DCASE(32, 64) LOGLIN_DCASE(32, 128)
  LOGLIN_DCASE(64, 32) LOGLIN_DCASE(64, 64) LOGLIN_DCASE(64, 128)
  if constexpr (sizeof(T) == 4) {
    LOGLIN_DCASE(16, 16) LOGLIN_DCASE(32, 16) LOGLIN_DCASE(64, 16)
  }
#undef LOGLIN_DCASE
  return nullptr;
}

DecodeFn lookup_decode(int dtype, int P, int N) {
  return dtype == LOGLIN_BF16 ? lookup_decode_t<bf16>(P, N) : lookup_decode_t<float>(P, N);
}

}  // namespace loglin
