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

// grid: batch * heads * (P / 4) work-groups of 128 threads: thread n owns
// row n of the 4 columns 4 pq .. 4 pq + 3 (rows n >= N idle), so a level
// costs one 16-byte read per thread and many small work-groups spread the
// step over the CUs.  A level state is stored column-quad major,
// [P/4][N][4], so a work-group's reads of a level are one contiguous run.
template <class T, int P, int N>
__global__ __launch_bounds__(128) void decode_kernel(DecodeParams dp) {
  constexpr int PQ = P / 4;
  static_assert(N <= 128, "one row per thread");
  const int n = threadIdx.x;
  const bool row = n < N;
  const int pq = blockIdx.x % PQ;
  const int bh = blockIdx.x / PQ;
  const int H = dp.nheads, G = dp.ngroups, LL = dp.ll, L = dp.nlevels;
  const int b = bh / H, h = bh % H, grp = h / (H / G);
  const int64_t t = dp.t;
  const int z = t > 0 ? __builtin_ctzll((unsigned long long)t) : -1;  // levels 0..z merge into z+1
  const float a = expf(dp.log_a[bh]);
  const T* lam = static_cast<const T*>(dp.lam) + (int64_t)bh * L;
  const T* Xv = static_cast<const T*>(dp.X) + (int64_t)bh * P;
  const float* gold = dp.gd + ((int64_t)bh * 2 + (t & 1)) * LL;
  float* S = dp.S + (int64_t)bh * LL * N * P;
  const int c0 = 4 * pq;  // first of the work-group's 4 columns

  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = to_f(Xv[c0 + i]);
  const int64_t gb = ((int64_t)b * G + grp) * N;
  const float cn = row ? to_f(static_cast<const T*>(dp.Cm)[gb + n]) : 0.f;
  const float bn = row ? to_f(static_cast<const T*>(dp.Bm)[gb + n]) : 0.f;
  const float lam_merge = z >= 0 ? to_f(lam[z + 1]) : 0.f;

  // new level 0, the token itself (S_0 = B_t X_t^T), then every occupied
  // older level; the levels 0..z also merge into level z+1
  f32x4 acc = (to_f(lam[0]) * bn * cn) * f32x4{x[0], x[1], x[2], x[3]};
  f32x4 merged = {0.f, 0.f, 0.f, 0.f};
  if (t > 0 && row) {
    constexpr int U = 8;  // levels whose loads are in flight together
    for (int l0 = 0; l0 < LL; l0 += U) {  // uniform; empty levels load nothing
      f32x4 sv[U];
      float gv[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int l = l0 + i;
        gv[i] = (l < LL && l != z + 1) ? gold[l] : 0.f;
        sv[i] = gv[i] != 0.f ? *reinterpret_cast<const f32x4*>(S + (((int64_t)l * PQ + pq) * N + n) * 4)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int l = l0 + i;
        if (gv[i] != 0.f) {
          const bool merge = l <= z;
          const float w = (merge ? lam_merge : to_f(lam[l])) * a * gv[i];
          acc += (w * cn) * sv[i];
          if (merge) merged += gv[i] * sv[i];
        }
      }
    }
  }
  if (row) {  // the merged level and level 0, stored without decay factor
    if (z >= 0) *reinterpret_cast<f32x4*>(S + (((int64_t)(z + 1) * PQ + pq) * N + n) * 4) = merged;
    *reinterpret_cast<f32x4*>(S + ((int64_t)pq * N + n) * 4) =
        f32x4{bn * x[0], bn * x[1], bn * x[2], bn * x[3]};
  }

  // sum over the rows: each wave by shuffles, then the two waves in LDS
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], d, 64);
  }
  __shared__ f32x4 part[2];
  if ((n & 63) == 0) part[n >> 6] = acc;
  __syncthreads();
  if (n == 0) {
    T* o = static_cast<T*>(dp.out) + (int64_t)bh * P + c0;
    store4(o, part[0] + part[1]);
  }
  // decay factors for the next step (one work-group per head writes them)
  if (pq == 0 && n < LL) {
    const int l = n;
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
  const int grid = dp.batch * dp.nheads * (P / 4);
  hipLaunchKernelGGL((decode_kernel<T, P, N>), dim3(grid), dim3(128), 0,
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
