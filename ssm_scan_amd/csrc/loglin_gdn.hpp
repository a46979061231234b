// Device code of the log-linear gated DeltaNet forward for gfx950 (MI355X).
//
// Method: log-linear attention write-up (yoousoft.com/industry/3746),
// section "log-linear generalisation of Mamba-2 and gated DeltaNet": the
// model keeps gated DeltaNet's transition A_t = alpha_t (I - beta_t k_t
// k_t^T) on every Fenwick level state and weights the levels by lambda.
// Equivalently O = (G ⊙ M^H) V with G the gated DeltaNet attention matrix,
// G[t, s] = beta_s (gamma_t / gamma_s) q_t^T H_t ... H_{s+1} k_s, H = I - beta k k^T.
//
// Chunked form (chunk of C tokens, gamma_t = exp(cumulative log alpha from
// the chunk start to t), Gamma[t][s] = gamma_t / gamma_s for s <= t):
//   L   = strictly lower part of diag(beta) (K K^T ⊙ Gamma)
//   Th  = (I + L)^{-1}                        (unit lower triangular)
//   G   = tril(Q K^T ⊙ Gamma) Th diag(beta)    intra-chunk attention
//   U   = Th diag(beta) V,  W = Th diag(beta gamma) K
//   Qe  = diag(gamma) Q - G diag(gamma) K      queries seen by older state
//   Kh  = diag(gamma_C / gamma) K
// A state S held at the chunk start contributes Qe S to the outputs and
// becomes gamma_C S - Kh^T (W S) at the chunk end; the chunk's own tokens
// leave Kh^T U.  Intra-chunk outputs are (G ⊙ lambda-by-level) V.  Older
// tokens are grouped at chunk granularity by the Fenwick rule (chunk level
// m holds the chunks i with bit_length(j xor i) = m for the current chunk
// j, token level c + m), each level's state propagated like S above.
//
// One work-group per (batch, head, 16 value columns): the columns of a
// delta-rule state evolve independently.  It walks the chunks in order with
// the chunk-level states in registers (thread-owned slices of N x 16).
// The per-chunk algebra is plain fp32 on LDS tiles.
#pragma once

#include "loglin_device.hpp"

namespace loglin {

struct GdnParams {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const void* lam;
  void* out;
  int batch, seqlen, nheads, nlevels, ll, nc;
};

constexpr int GDN_C = 32;     // tokens per chunk
constexpr int GDN_PB = 16;    // value columns per work-group
constexpr int GDN_NT = 256;   // threads per work-group
constexpr int GDN_KMAX = 16;  // chunk levels 1..GDN_KMAX-1 held in registers
constexpr int GDN_LMAX = 32;  // token levels per lambda row

template <class T, int N, int P>
__global__ __launch_bounds__(GDN_NT) void gdn_kernel(GdnParams pr) {
  constexpr int C = GDN_C, PB = GDN_PB, NT = GDN_NT, c_log = 5;
  static_assert((1 << c_log) == C, "chunk");
  constexpr int NS = N + 1;            // padded row stride: rows read across lanes
  constexpr int EPT = N * PB / NT;     // state elements per thread
  constexpr int TPR = PB / EPT;        // threads per state row
  static_assert(EPT >= 1 && PB % EPT == 0 && P % PB == 0, "state slicing");
  __shared__ float qs[C][NS];  // q, then the effective queries Qe
  __shared__ float ks[C][NS];
  __shared__ float wm[C][NS];
  __shared__ float vs[C][PB];
  __shared__ float am[C][C + 1], lm[C][C + 1], tm[C][C + 1], gm[C][C + 1];
  __shared__ float um[C][PB], os[C][PB];
  __shared__ float xy[2 * C][PB];
  __shared__ float zs[N][PB];
  __shared__ float lam_s[C][GDN_LMAX];
  __shared__ float cum[C], gam[C], bet[C], khs[C];

  const int nblk = P / PB;
  const int wg = blockIdx.x;
  const int pblk = wg % nblk, bh = wg / nblk;
  const int H = pr.nheads, L = pr.nlevels, ll = pr.ll;
  const int b = bh / H, h = bh % H, p0 = pblk * PB;
  const int64_t T_ = pr.seqlen;
  const int tid = threadIdx.x;
  const int zn = tid / TPR, zp = (tid % TPR) * EPT;  // this thread's state slice
  const T* qg = static_cast<const T*>(pr.q);
  const T* kg = static_cast<const T*>(pr.k);
  const T* vg = static_cast<const T*>(pr.v);
  const T* lg = static_cast<const T*>(pr.lam);
  T* og = static_cast<T*>(pr.out);

  float Z[GDN_KMAX][EPT];  // chunk-level states (index = level; 0 unused)
#pragma unroll
  for (int m = 0; m < GDN_KMAX; ++m)
#pragma unroll
    for (int e = 0; e < EPT; ++e) Z[m][e] = 0.f;

  for (int j = 0; j < pr.nc; ++j) {
    const int64_t t0 = (int64_t)j * C;
    // ---- this chunk's rows
    for (int i = tid; i < C * N; i += NT) {
      const int t = i / N, n = i % N;
      const int64_t row = ((int64_t)b * T_ + t0 + t) * H + h;
      qs[t][n] = to_f(qg[row * N + n]);
      ks[t][n] = to_f(kg[row * N + n]);
    }
    for (int i = tid; i < C * PB; i += NT) {
      const int t = i / PB, p = i % PB;
      vs[t][p] = to_f(vg[(((int64_t)b * T_ + t0 + t) * H + h) * P + p0 + p]);
    }
    for (int i = tid; i < C * ll; i += NT) {
      const int t = i / ll, l = i % ll;
      lam_s[t][l] = to_f(lg[(((int64_t)b * T_ + t0 + t) * H + h) * L + l]);
    }
    if (tid < 64) {  // inclusive cumulative log alpha over the chunk
      const int64_t gi = ((int64_t)b * T_ + t0 + (tid < C ? tid : 0)) * H + h;
      float x = tid < C ? pr.log_alpha[gi] : 0.f;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(x, d, 64);
        if (tid >= d) x += o;
      }
      if (tid < C) {
        cum[tid] = x;
        gam[tid] = expf(x);
        bet[tid] = pr.beta[gi];
      }
    }
    __syncthreads();
    if (tid < C) khs[tid] = expf(cum[C - 1] - cum[tid]);  // gamma_C / gamma_t
    // ---- tril(Q K^T ⊙ Gamma) and L = strictly lower diag(beta)(K K^T ⊙ Gamma)
    for (int i = tid; i < C * C; i += NT) {
      const int t = i / C, s = i % C;
      float a = 0.f, l = 0.f;
      if (s <= t) {
        float dq = 0.f, dk = 0.f;
        for (int n = 0; n < N; ++n) {
          dq += qs[t][n] * ks[s][n];
          dk += ks[t][n] * ks[s][n];
        }
        const float g = expf(cum[t] - cum[s]);
        a = dq * g;
        if (s < t) l = bet[t] * dk * g;
      }
      am[t][s] = a;
      lm[t][s] = l;
    }
    __syncthreads();
    // ---- Th = (I + L)^{-1}, one column per thread, forward substitution
    if (tid < C) {
      const int jc = tid;
      for (int i = 0; i < C; ++i) {
        float x = i == jc ? 1.f : 0.f;
        if (i > jc)
          for (int m = jc; m < i; ++m) x -= lm[i][m] * tm[m][jc];
        tm[i][jc] = x;
      }
    }
    __syncthreads();
    // ---- G = tril(Q K^T ⊙ Gamma) Th diag(beta), U = Th diag(beta) V,
    //      W = Th diag(beta gamma) K
    for (int i = tid; i < C * C; i += NT) {
      const int t = i / C, s = i % C;
      float g = 0.f;
      if (s <= t) {
        for (int m = s; m <= t; ++m) g += am[t][m] * tm[m][s];
        g *= bet[s];
      }
      gm[t][s] = g;
    }
    for (int i = tid; i < C * PB; i += NT) {
      const int r = i / PB, p = i % PB;
      float u = 0.f;
      for (int s = 0; s <= r; ++s) u += tm[r][s] * bet[s] * vs[s][p];
      um[r][p] = u;
    }
    for (int i = tid; i < C * N; i += NT) {
      const int r = i / N, n = i % N;
      float w = 0.f;
      for (int s = 0; s <= r; ++s) w += tm[r][s] * (bet[s] * gam[s]) * ks[s][n];
      wm[r][n] = w;
    }
    __syncthreads();
    // ---- Qe = diag(gamma) Q - G diag(gamma) K (in place), intra outputs
    for (int i = tid; i < C * N; i += NT) {
      const int t = i / N, n = i % N;
      float x = gam[t] * qs[t][n];
      for (int s = 0; s <= t; ++s) x -= gm[t][s] * gam[s] * ks[s][n];
      qs[t][n] = x;
    }
    for (int i = tid; i < C * PB; i += NT) {
      const int t = i / PB, p = i % PB;
      float o = 0.f;
      for (int s = 0; s <= t; ++s) o += gm[t][s] * lam_s[t][bit_length((unsigned)(t ^ s))] * vs[s][p];
      os[t][p] = o;
    }
    __syncthreads();
    // ---- chunk levels whose bit is set in j: outputs, then propagation.
    // The loop body is large, so it is not unrolled; the level's state is
    // moved in and out of zc through uniform branches with constant indices
    // (a runtime index into Z would move Z to scratch memory).
    const float gC = gam[C - 1];
    for (unsigned act = (unsigned)j; act; act &= act - 1u) {
      const int m = __builtin_ctz(act) + 1;  // uniform
      float zc[EPT];
#pragma unroll
      for (int m2 = 1; m2 < GDN_KMAX; ++m2)
        if (m2 == m) {
#pragma unroll
          for (int e = 0; e < EPT; ++e) zc[e] = Z[m2][e];
        }
#pragma unroll
      for (int e = 0; e < EPT; ++e) zs[zn][zp + e] = zc[e];
      __syncthreads();
      for (int i = tid; i < 2 * C * PB; i += NT) {  // Qe Z (rows < C), W Z (rows >= C)
        const int r = i / PB, p = i % PB;
        const float* a = r < C ? qs[r] : wm[r - C];
        float x = 0.f;
        for (int n = 0; n < N; ++n) x += a[n] * zs[n][p];
        xy[r][p] = x;
      }
      __syncthreads();
      for (int i = tid; i < C * PB; i += NT) {
        const int t = i / PB, p = i % PB;
        os[t][p] += lam_s[t][c_log + m] * xy[t][p];
      }
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float acc = gC * zc[e];
        for (int r = 0; r < C; ++r) acc -= khs[r] * ks[r][zn] * xy[C + r][zp + e];
        zc[e] = acc;
      }
#pragma unroll
      for (int m2 = 1; m2 < GDN_KMAX; ++m2)
        if (m2 == m) {
#pragma unroll
          for (int e = 0; e < EPT; ++e) Z[m2][e] = zc[e];
        }
      __syncthreads();  // zs and xy are reused by the next level
    }
    // ---- the chunk's own tokens, then the Fenwick merge for chunk j + 1
    float own[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      float acc = 0.f;
      for (int r = 0; r < C; ++r) acc += khs[r] * ks[r][zn] * um[r][zp + e];
      own[e] = acc;
    }
    if (j + 1 < pr.nc) {
      const int z = __builtin_ctz((unsigned)(j + 1));
#pragma unroll
      for (int m = 1; m < GDN_KMAX; ++m)
        if (m <= z) {
#pragma unroll
          for (int e = 0; e < EPT; ++e) {
            own[e] += Z[m][e];
            Z[m][e] = 0.f;
          }
        }
#pragma unroll
      for (int m = 1; m < GDN_KMAX; ++m)
        if (m == z + 1) {
#pragma unroll
          for (int e = 0; e < EPT; ++e) Z[m][e] = own[e];
        }
    }
    for (int i = tid; i < C * PB; i += NT) {
      const int t = i / PB, p = i % PB;
      og[(((int64_t)b * T_ + t0 + t) * H + h) * P + p0 + p] = from_f<T>(os[t][p]);
    }
    __syncthreads();  // the next chunk restages every tile
  }
}

using GdnFn = int (*)(const GdnParams&, hipStream_t);

template <class T, int N, int P>
int launch_gdn(const GdnParams& pr, hipStream_t st) {
  const int blocks = pr.batch * pr.nheads * (P / GDN_PB);
  hipLaunchKernelGGL((gdn_kernel<T, N, P>), dim3(blocks), dim3(GDN_NT), 0, st, pr);
  return (int)hipGetLastError();
}

GdnFn lookup_gdn(int dtype, int N, int P);

}  // namespace loglin
