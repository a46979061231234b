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

  // The loads that depend on nothing are issued together, unconditionally
  // (idle rows read row N - 1) and kept in the io type until all are out: a
  // load under a branch, or one converted as soon as it is issued, makes
  // the thread wait for it before the next goes out.
  const int64_t gb = ((int64_t)b * G + grp) * N;
  const int nr = row ? n : N - 1;
  T xr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xr[i] = Xv[c0 + i];
  const T cr = static_cast<const T*>(dp.Cm)[gb + nr];
  const T br = static_cast<const T*>(dp.Bm)[gb + nr];
  const T lr0 = lam[0], lrm = lam[z >= 0 ? z + 1 : 0];
  constexpr int U = 16;  // levels whose loads are in flight together
  float gr[U];
  T lr[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int l = min(i, LL - 1);
    gr[i] = gold[l];
    lr[i] = lam[l];
  }

  // every occupied older level (S_l^T, C applied at the end), then the new
  // level 0, the token itself (S_0 = B_t X_t^T); the levels 0..z also merge
  // into level z+1
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 merged = {0.f, 0.f, 0.f, 0.f};
  if (t > 0 && row) {
    // Before step t the buckets are those of the prefix 0 .. t-1: level 0
    // and, for l >= 1, level l where bit l-1 of t-1 is set (level z+1 is
    // empty).  Known from t alone, so the state loads need not wait for the
    // decay factors; a bucket whose factor has underflowed to 0 adds 0.
    const unsigned long long occ = ((unsigned long long)(t - 1) << 1) | 1ull;
    for (int l0 = 0; l0 < LL; l0 += U) {  // uniform; empty levels load nothing
      f32x4 sv[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int l = l0 + i;
        sv[i] = (l < LL && ((occ >> l) & 1ull))
                    ? *reinterpret_cast<const f32x4*>(S + (((int64_t)l * PQ + pq) * N + n) * 4)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float gv[U], lv[U];  // decay factor and lambda of each level
#pragma unroll
      for (int i = 0; i < U; ++i) {
        gv[i] = l0 == 0 ? gr[i] : gold[min(l0 + i, LL - 1)];
        // the factors are uniform (scalar loads): taking them here, after
        // the state loads have gone out, keeps the compiler from loading
        // and waiting for each one next to its use
        asm volatile("" : "+v"(gv[i]));
        lv[i] = l0 == 0 ? to_f(lr[i]) : to_f(lam[min(l0 + i, LL - 1)]);
      }
      const float lam_merge = z >= 0 ? to_f(lrm) : 0.f;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int l = l0 + i;
        if (l < LL && ((occ >> l) & 1ull)) {
          const bool merge = l <= z;
          const float w = (merge ? lam_merge : lv[i]) * a * gv[i];
          acc += w * sv[i];
          if (merge) merged += gv[i] * sv[i];
        }
      }
    }
  }
  const float cn = row ? to_f(cr) : 0.f;
  const float bn = row ? to_f(br) : 0.f;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = to_f(xr[i]);
  acc = cn * (acc + (to_f(lr0) * bn) * f32x4{x[0], x[1], x[2], x[3]});
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
