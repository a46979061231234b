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
// Two passes.  gdn_chunk_kernel, one work-group per (batch, head, chunk),
// all chunks at once: T^, G, U, W, Qe and the intra-chunk outputs, to the
// workspace in fp32.  gdn_scan_kernel, one work-group per (batch, head, 16
// value columns; the columns of a delta-rule state evolve independently),
// walks the chunks in order with the chunk-level states in registers (in
// the layout the state update's MFMA leaves them), reads each chunk's Qe,
// W, K, U and intra outputs (loaded into registers one chunk ahead), adds
// the level terms and writes the outputs.  Its barriers wait for LDS
// traffic only (lds_barrier): __syncthreads() would also wait for the
// next chunk's loads in flight.  Every product is a
// v_mfma_f32_16x16x4f32 tile over XOR-swizzled fp32 LDS tiles (fp32 keeps
// the delta rule's corrections exact to fp32); the triangular inverse is
// blocked (8 -> 16 -> 32) so that every thread takes part.
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
  float* qe;  // [batch*nheads*nc, C, N]  effective queries
  float* w;   // [batch*nheads*nc, C, N]  W
  float* u;   // [batch*nheads*nc, C, P]  U
  float* oi;  // [batch*nheads*nc, C, P]  intra-chunk outputs
  float* kh;  // [batch*nheads*nc, C]     gamma_C / gamma_t
  float* gc;  // [batch*nheads*nc]        gamma_C
  int batch, seqlen, nheads, nlevels, ll, nc;
};

constexpr int GDN_C = 32;     // tokens per chunk
constexpr int GDN_PB = 16;    // value columns per work-group of the scan
constexpr int GDN_NT = 256;   // threads per work-group of the chunk pass (4 waves)
constexpr int GDN_SNT = 512;  // threads per work-group of the level pass (8 waves)
constexpr int GDN_KMAX = 16;  // chunk levels 1..GDN_KMAX-1 held in registers
constexpr int GDN_LMAX = 32;  // token levels per lambda row
constexpr int GDN_LB = 4;     // chunk levels the level pass handles per batch

// ------------------------------------------------------------ pass 1

// Eight consecutive io-type elements as fp32 (one 16-byte load for bf16).
template <class T>
__device__ inline void load8f(const T* p, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[e + 4] = b[e];
    }
  }
}
__device__ inline void store8f(float* lo, float* hi, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(lo) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(hi) = f32x4{x[4], x[5], x[6], x[7]};
}

template <class T, int N, int P>
__global__ __launch_bounds__(GDN_NT) void gdn_chunk_kernel(GdnParams pr) {
  using M = Mfma<float>;  // 16x16x4 fp32: A row r / B column r, contraction element g
  constexpr int C = GDN_C, NT = GDN_NT, c_log = 5;
  static_assert((1 << c_log) == C && N % 16 == 0 && P % 16 == 0, "tile shapes");
  constexpr int NTILE = N / 16, PT = P / 16;
  using LN = Rows<float, N>;
  using LC = Rows<float, C>;
  using LV = Rows<float, P>;
  __shared__ __attribute__((aligned(16))) float qf[C * N];
  __shared__ __attribute__((aligned(16))) float kf[C * N];
  __shared__ __attribute__((aligned(16))) float am[C * C];  // tril(Q K^T ⊙ Gamma)
  __shared__ __attribute__((aligned(16))) float lm[C * C];  // L
  __shared__ __attribute__((aligned(16))) float tm[C * C];  // Th = (I + L)^-1
  __shared__ __attribute__((aligned(16))) float gm[C * C];  // G
  __shared__ __attribute__((aligned(16))) float gl[C * C];  // G ⊙ lambda by level
  __shared__ __attribute__((aligned(16))) float pt[C * C];  // block-inverse temporary
  __shared__ __attribute__((aligned(16))) float vf[C * P];
  __shared__ __attribute__((aligned(16))) float vb[C * P];  // diag(beta) V
  __shared__ float lam_s[C][8];                              // intra-chunk levels 0..c
  __shared__ float cum[C], gam[C], bet[C], bg[C];

  const int item = blockIdx.x;  // (batch*head) * nc + chunk
  const int bh = item / pr.nc, j = item % pr.nc;
  const int H = pr.nheads, L = pr.nlevels;
  const int b = bh / H, h = bh % H;
  const int64_t T_ = pr.seqlen, t0 = (int64_t)j * C;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const T* qg = static_cast<const T*>(pr.q);
  const T* kg = static_cast<const T*>(pr.k);
  const T* vg = static_cast<const T*>(pr.v);
  const T* lg = static_cast<const T*>(pr.lam);

  for (int i = tid; i < C * N / 8; i += NT) {  // eight keys / queries per thread and step
    const int t = (8 * i) / N, n = (8 * i) % N;
    const int64_t row = ((int64_t)b * T_ + t0 + t) * H + h;
    float x[8];
    load8f(qg + row * N + n, x);
    store8f(qf + LN::at(t, n), qf + LN::at(t, n + 4), x);
    load8f(kg + row * N + n, x);
    store8f(kf + LN::at(t, n), kf + LN::at(t, n + 4), x);
  }
  for (int i = tid; i < C * (c_log + 1); i += NT) {
    const int t = i / (c_log + 1), l = i % (c_log + 1);
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
    const float tot = __shfl(x, C - 1, 64);
    if (tid < C) {
      const float be = pr.beta[gi];
      cum[tid] = x;
      gam[tid] = expf(x);
      bet[tid] = be;
      bg[tid] = be * expf(x);
      pr.kh[(int64_t)item * C + tid] = expf(tot - x);  // gamma_C / gamma_t
      if (tid == 0) pr.gc[item] = expf(tot);
    }
  }
  __syncthreads();
  for (int i = tid; i < C * P / 8; i += NT) {
    const int t = (8 * i) / P, p = (8 * i) % P;
    float x[8], y[8];
    load8f(vg + (((int64_t)b * T_ + t0 + t) * H + h) * P + p, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = bet[t] * x[e];
    store8f(vf + LV::at(t, p), vf + LV::at(t, p + 4), x);
    store8f(vb + LV::at(t, p), vb + LV::at(t, p + 4), y);
  }
  // ---- Q K^T and K K^T, masked: wave w owns the 16x16 tile (w >> 1, w & 1)
  {
    const int tb = wave >> 1, sb = wave & 1;
    f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
    if (sb <= tb) {
#pragma unroll 8
      for (int n0 = 0; n0 < N; n0 += 4) {
        const float bk = frag_along<float, LN>(kf, 16 * sb + r, n0, g);
        sq = M::mma(frag_along<float, LN>(qf, 16 * tb + r, n0, g), bk, sq);
        sk = M::mma(frag_along<float, LN>(kf, 16 * tb + r, n0, g), bk, sk);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, s = 16 * sb + r;
      const float gr = s <= t ? expf(cum[t] - cum[s]) : 0.f;
      am[LC::at(t, s)] = sq[i] * gr;
      lm[LC::at(t, s)] = s < t ? bet[t] * sk[i] * gr : 0.f;
    }
  }
  __syncthreads();
  // ---- Th = (I + L)^-1, blocked: 8x8 diagonal blocks by substitution,
  // then [[A, 0], [B, D]]^-1 = [[A^-1, 0], [-D^-1 B A^-1, D^-1]] at 16, 32
  if (tid < C) {  // column jc of its 8x8 diagonal block, in registers
    const int jc = tid, blk = jc & ~7, jj = jc & 7;
    float x[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      float v = ii == jj ? 1.f : 0.f;
#pragma unroll
      for (int mm = 0; mm < ii; ++mm) v -= lm[LC::at(blk + ii, blk + mm)] * x[mm];
      x[ii] = ii < jj ? 0.f : v;  // above the diagonal: zero
    }
    for (int i = 0; i < C; ++i) {
      float v = 0.f;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) v = i == blk + ii ? x[ii] : v;
      tm[LC::at(i, jc)] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hb = 8; hb < C; hb *= 2) {  // half block size: 8, then 16
    const int cnt = (C / (2 * hb)) * hb * hb;
    for (int i = tid; i < cnt; i += NT) {  // B A^-1 (rows in the lower half, columns in the upper)
      const int blk = i / (hb * hb), e = i % (hb * hb);
      const int row = blk * 2 * hb + hb + e / hb, col = blk * 2 * hb + e % hb;
      float x = 0.f;
      for (int m = col; m < blk * 2 * hb + hb; ++m) x += lm[LC::at(row, m)] * tm[LC::at(m, col)];
      pt[LC::at(row, col)] = x;
    }
    __syncthreads();
    for (int i = tid; i < cnt; i += NT) {  // the lower-left block: -D^-1 (B A^-1)
      const int blk = i / (hb * hb), e = i % (hb * hb);
      const int row = blk * 2 * hb + hb + e / hb, col = blk * 2 * hb + e % hb;
      float x = 0.f;
      for (int m = blk * 2 * hb + hb; m <= row; ++m) x -= tm[LC::at(row, m)] * pt[LC::at(m, col)];
      tm[LC::at(row, col)] = x;
    }
    __syncthreads();
  }
  // ---- G = tril(Q K^T ⊙ Gamma) Th diag(beta) and G ⊙ lambda
  {
    const int tb = wave >> 1, sb = wave & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m0 = 0; m0 < C; m0 += 4)
      acc = M::mma(frag_along<float, LC>(am, 16 * tb + r, m0, g),
                   frag_down<float, LC>(tm, m0, 16 * sb, g, r), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, s = 16 * sb + r;
      const float gv = s <= t ? acc[i] * bet[s] : 0.f;
      gm[LC::at(t, s)] = gv;
      gl[LC::at(t, s)] = s <= t ? gv * lam_s[t][bit_length((unsigned)(t ^ s))] : 0.f;
    }
  }
  // ---- U = Th diag(beta) V and W = Th diag(beta gamma) K, straight to the
  //      workspace (row tile tile & 1, column tile tile >> 1)
  float* ug = pr.u + (int64_t)item * C * P;
  float* wg = pr.w + (int64_t)item * C * N;
  for (int tile = wave; tile < 2 * PT; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < C; s0 += 4)
      acc = M::mma(frag_along<float, LC>(tm, 16 * tb + r, s0, g),
                   frag_down<float, LV>(vb, s0, 16 * cb, g, r), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) ug[(16 * tb + 4 * g + i) * P + 16 * cb + r] = acc[i];
  }
  for (int tile = wave; tile < 2 * NTILE; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < C; s0 += 4)
      acc = M::mma(frag_along<float, LC>(tm, 16 * tb + r, s0, g) * bg[s0 + g],
                   frag_down<float, LN>(kf, s0, 16 * cb, g, r), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) wg[(16 * tb + 4 * g + i) * N + 16 * cb + r] = acc[i];
  }
  __syncthreads();  // gm and gl are complete
  // ---- Qe = diag(gamma) Q - G diag(gamma) K and the intra outputs (G ⊙ lambda) V
  float* qeg = pr.qe + (int64_t)item * C * N;
  float* oig = pr.oi + (int64_t)item * C * P;
  for (int tile = wave; tile < 2 * NTILE; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < C; s0 += 4)
      acc = M::mma(frag_along<float, LC>(gm, 16 * tb + r, s0, g) * gam[s0 + g],
                   frag_down<float, LN>(kf, s0, 16 * cb, g, r), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, n = 16 * cb + r;
      qeg[t * N + n] = gam[t] * qf[LN::at(t, n)] - acc[i];
    }
  }
  for (int tile = wave; tile < 2 * PT; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < C; s0 += 4)
      acc = M::mma(frag_along<float, LC>(gl, 16 * tb + r, s0, g),
                   frag_down<float, LV>(vf, s0, 16 * cb, g, r), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) oig[(16 * tb + 4 * g + i) * P + 16 * cb + r] = acc[i];
  }
}

// ------------------------------------------------------------ pass 2

// One chunk's operands of the level pass, loaded into registers one chunk
// ahead and then stored to LDS: Qe, W and K (C x N), U and the intra outputs
// for this work-group's 16 columns, gamma_C / gamma_t, and lambda rows.
template <class T, int N, int P, int NT_>
struct GdnStage {
  static constexpr int C = GDN_C, PB = GDN_PB, NT = NT_;
  static constexpr int NV = (C * PB + NT - 1) / NT;  // U / intra-output values per thread
  static constexpr int NQ4 = C * N / 4;  // float4 groups of a C x N tile
  static constexpr int NQ = (NQ4 + NT - 1) / NT;  // per thread
  static constexpr int NL = (C * GDN_LMAX + NT - 1) / NT;
  f32x4 qe[NQ], w[NQ], k[NQ];
  float u2[NV], o2[NV], khv, gcv;
  T lam[NL];  // raw: converted (and zeroed past the level count) when staged
  __device__ inline void load(const GdnParams& pr, int item, int b, int h, int64_t t0, int p0, int tid) {
    const float* qeg = pr.qe + (int64_t)item * C * N;
    const float* wg = pr.w + (int64_t)item * C * N;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q * NT + tid >= NQ4) break;
      const int e = (q * NT + tid) * 4, t = e / N, n = e % N;
      qe[q] = *reinterpret_cast<const f32x4*>(qeg + e);
      w[q] = *reinterpret_cast<const f32x4*>(wg + e);
      const T* kr = static_cast<const T*>(pr.k) + (((int64_t)b * pr.seqlen + t0 + t) * pr.nheads + h) * N + n;
      if constexpr (sizeof(T) == 2) {  // four keys: one 8-byte load
        const bf16x4 kv = *reinterpret_cast<const bf16x4*>(kr);
#pragma unroll
        for (int c = 0; c < 4; ++c) k[q][c] = (float)kv[c];
      } else {
        k[q] = *reinterpret_cast<const f32x4*>(kr);
      }
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) {  // C x 16 = 512 values
      const int e = q * NT + tid, t = e / PB, p = e % PB;
      u2[q] = e < C * PB ? pr.u[((int64_t)item * C + t) * P + p0 + p] : 0.f;
      o2[q] = e < C * PB ? pr.oi[((int64_t)item * C + t) * P + p0 + p] : 0.f;
    }
    const T* lg = static_cast<const T*>(pr.lam);
#pragma unroll
    for (int q = 0; q < NL; ++q) {  // unconditional loads: nothing waits for them here
      const int e = q * NT + tid, t = min(e / GDN_LMAX, C - 1), l = min(e % GDN_LMAX, pr.ll - 1);
      lam[q] = lg[(((int64_t)b * pr.seqlen + t0 + t) * pr.nheads + h) * pr.nlevels + l];
    }
    khv = tid < C ? pr.kh[(int64_t)item * C + tid] : 0.f;
    gcv = pr.gc[item];
  }
};

// Layout of the level pass's K tile (C x N fp32): the 16-byte blocks of row
// t are XOR-swizzled by 4 (t mod 4), masked to the N / 4 blocks of a row.
// Its only reads take rows j0 + g (j0 a multiple of 4) and columns
// 16 nb + r, so for N >= 64 a wave's 64 lanes meet 64 different banks; the
// staging writes fill whole rows.
template <int N>
struct KRows {
  __device__ static inline int at(int row, int c) {
    return row * N + ((((c >> 2) ^ (((row & 3) << 2) & (N / 4 - 1))) << 2) | (c & 3));
  }
};

template <class T, int N, int P>
__global__ __launch_bounds__(GDN_SNT) void gdn_scan_kernel(GdnParams pr) {
  using M = Mfma<float>;
  constexpr int C = GDN_C, PB = GDN_PB, NT = GDN_SNT, NWV = NT / 64, c_log = 5;
  static_assert(PB == 16 && N % 16 == 0 && P % PB == 0, "tile shapes");
  constexpr int NTILE = N / 16;                // 16-row blocks of a state
  constexpr int NTW = (NTILE + NWV - 1) / NWV;  // of them per wave (waves past NTILE own none)
  using LN = Rows<float, N>;
  using LP = Rows<float, PB>;
  using St = GdnStage<T, N, P, NT>;
  __shared__ __attribute__((aligned(16))) float qf[C * N];  // Qe
  __shared__ __attribute__((aligned(16))) float wf[C * N];  // W
  __shared__ __attribute__((aligned(16))) float kf[C * N];  // K
  __shared__ __attribute__((aligned(16))) float us[C * PB];  // U
  __shared__ __attribute__((aligned(16))) float ys[GDN_LB * C * PB];  // W Z of a batch of levels
  // outputs of the chunk: the intra part and the even batch slots' levels
  // in os, the odd slots' levels in os1 (each written by one wave per row
  // block: no two waves add to one entry)
  __shared__ __attribute__((aligned(16))) float os[C * PB];
  __shared__ __attribute__((aligned(16))) float os1[C * PB];
  __shared__ __attribute__((aligned(16))) float zs[GDN_LB * N * PB];  // a batch of level states
  __shared__ float lam_s[C][GDN_LMAX];
  __shared__ float khs[C];

  const int nblk = P / PB;
  const int pblk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
  const int H = pr.nheads;
  const int b = bh / H, h = bh % H, p0 = pblk * PB;
  const int64_t T_ = pr.seqlen;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* og = static_cast<T*>(pr.out);

  // chunk-level states: wave w owns rows [16 (NTW w + u), +16) of N, all 16
  // columns, as MFMA result tiles (lane: rows 4 g + i, column r)
  f32x4 Z[GDN_KMAX][NTW];
#pragma unroll
  for (int m = 0; m < GDN_KMAX; ++m)
#pragma unroll
    for (int u = 0; u < NTW; ++u) Z[m][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  St st;
  st.load(pr, bh * pr.nc, b, h, 0, p0, tid);
  for (int j = 0; j < pr.nc; ++j) {
    const int64_t t0 = (int64_t)j * C;
    // ---- this chunk's operands into LDS, then the next chunk's loads
#pragma unroll
    for (int q = 0; q < St::NQ; ++q) {
      if (q * NT + tid >= St::NQ4) break;
      const int e = (q * NT + tid) * 4, t = e / N, n = e % N;
      store16(qf + LN::at(t, n), st.qe[q]);
      store16(wf + LN::at(t, n), st.w[q]);
      store16(kf + KRows<N>::at(t, n), st.k[q]);
    }
#pragma unroll
    for (int q = 0; q < St::NV; ++q) {
      const int e = q * NT + tid, t = e / PB, p = e % PB;
      if (e < C * PB) {
        us[LP::at(t, p)] = st.u2[q];
        os[LP::at(t, p)] = st.o2[q];
        os1[LP::at(t, p)] = 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < St::NL; ++q) {
      const int e = q * NT + tid;
      if (e < C * GDN_LMAX) lam_s[e / GDN_LMAX][e % GDN_LMAX] = e % GDN_LMAX < pr.ll ? to_f(st.lam[q]) : 0.f;
    }
    if (tid < C) khs[tid] = st.khv;
    const float gC = st.gcv;
    lds_barrier();
    if (j + 1 < pr.nc) st.load(pr, bh * pr.nc + j + 1, b, h, t0 + C, p0, tid);

    // ---- chunk levels whose bit is set in j, up to GDN_LB at a time (three
    // barriers per batch): their states to LDS, then Qe Z (outputs) and W Z,
    // then the propagation.  The body is not unrolled; a level's state moves
    // in and out of registers through uniform branches with constant indices
    // (a runtime index into Z would move Z to scratch memory).
    for (unsigned act = (unsigned)j; act;) {
      int ms[GDN_LB];
      int nbat = 0;
      unsigned bmask = 0;  // bit m: level m is in the batch, at slot popcount(bmask & (2^m - 1))
#pragma unroll
      for (int q = 0; q < GDN_LB; ++q) {
        ms[q] = act ? __builtin_ctz(act) + 1 : 0;  // uniform; 0: no level
        if (act) {
          bmask |= 1u << ms[q];
          act &= act - 1u;
          ++nbat;
        }
      }
#pragma unroll
      for (int m2 = 1; m2 < GDN_KMAX; ++m2)
        if ((bmask >> m2) & 1u) {
          const int q = __builtin_popcount(bmask & ((1u << m2) - 1u));
#pragma unroll
          for (int u = 0; u < NTW; ++u)
            if (NTW * wave + u < NTILE) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                zs[q * N * PB + LP::at(16 * (NTW * wave + u) + 4 * g + i, r)] = Z[m2][u][i];
            }
        }
      lds_barrier();
      {  // wave w: Qe Z (outputs) for w mod 4 < 2, else W Z; row block
         // w mod 2; batch slots q = w / 4, w / 4 + 2
        const bool qe = (wave & 2) == 0;
        const float* a = qe ? qf : wf;
        const int rb = wave & 1, q0 = wave >> 2;
        float* od = q0 ? os1 : os;
#pragma unroll
        for (int q = q0; q < GDN_LB; q += 2) {
          if (q >= nbat) break;
          const float* zq = zs + q * N * PB;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
          for (int n0 = 0; n0 < N; n0 += 4)
            acc = M::mma(frag_along<float, LN>(a, 16 * rb + r, n0, g),
                         frag_down<float, LP>(zq, n0, 0, g, r), acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * rb + 4 * g + i;
            if (qe)
              od[LP::at(t, r)] += lam_s[t][c_log + ms[q]] * acc[i];
            else
              ys[q * C * PB + LP::at(t, r)] = acc[i];
          }
        }
      }
      lds_barrier();
      // Z <- gamma_C Z - Kh^T (W Z)
#pragma unroll
      for (int m2 = 1; m2 < GDN_KMAX; ++m2)
        if ((bmask >> m2) & 1u) {
          const int q = __builtin_popcount(bmask & ((1u << m2) - 1u));
#pragma unroll
          for (int u = 0; u < NTW; ++u) {
            const int nb = NTW * wave + u;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (nb < NTILE) {  // uniform
#pragma unroll
              for (int j0 = 0; j0 < C; j0 += 4)
                acc = M::mma(kf[KRows<N>::at(j0 + g, 16 * nb + r)] * khs[j0 + g],
                             frag_down<float, LP>(ys + q * C * PB, j0, 0, g, r), acc);
            }
            Z[m2][u] = gC * Z[m2][u] - acc;
          }
        }
      lds_barrier();  // zs and ys are reused by the next batch
    }
    // ---- the chunk's own tokens (Kh^T U), then the Fenwick merge for j + 1
    f32x4 own[NTW];
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int nb = NTW * wave + u;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (nb < NTILE) {  // uniform
#pragma unroll
        for (int j0 = 0; j0 < C; j0 += 4)
          acc = M::mma(kf[KRows<N>::at(j0 + g, 16 * nb + r)] * khs[j0 + g],
                       frag_down<float, LP>(us, j0, 0, g, r), acc);
      }
      own[u] = acc;
    }
    if (j + 1 < pr.nc) {
      const int z = __builtin_ctz((unsigned)(j + 1));
#pragma unroll
      for (int m = 1; m < GDN_KMAX; ++m)
        if (m <= z) {
#pragma unroll
          for (int u = 0; u < NTW; ++u) {
            own[u] += Z[m][u];
            Z[m][u] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
      for (int m = 1; m < GDN_KMAX; ++m)
        if (m == z + 1) {
#pragma unroll
          for (int u = 0; u < NTW; ++u) Z[m][u] = own[u];
        }
    }
    for (int i = tid; i < C * PB; i += NT) {
      const int t = i / PB, p = i % PB;
      og[(((int64_t)b * T_ + t0 + t) * H + h) * P + p0 + p] = from_f<T>(os[LP::at(t, p)] + os1[LP::at(t, p)]);
    }
    lds_barrier();  // the next chunk restages every tile
  }
}


// ---- the level pass for bf16 inputs: products as bf16 hi / lo pairs

// 64-byte rows of bf16 (32 elements, four 16-byte blocks): block b of row
// `row` sits at b ^ (row / 4 mod 4), so the 16 rows of an MFMA operand read
// at one logical block meet 16 different groups of four banks.
struct R32 {
  __device__ static inline int at(int row, int c) {
    return row * 32 + ((((c >> 3) ^ (row >> 2)) & 3) << 3) + (c & 7);
  }
};
template <int N>
using GdnRowsN = std::conditional_t<N == 32, R32, Rows<bf16, N>>;

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits.
__device__ inline void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}
__device__ inline void split_store4(bf16* hi, bf16* lo, int off, const f32x4& v) {
  bf16x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16 x = (bf16)v[i];
    h[i] = x;
    l[i] = (bf16)(v[i] - (float)x);
  }
  *reinterpret_cast<bf16x4*>(hi + off) = h;
  *reinterpret_cast<bf16x4*>(lo + off) = l;
}
// a . b with a = ah + al, b = bh + bl: ah bh + ah bl + al bh (the al bl term
// is below the pair's precision)
__device__ inline f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
  using M = Mfma<bf16>;
  c = M::mma(ah, bh, c);
  c = M::mma(ah, bl, c);
  return M::mma(al, bh, c);
}

// Same walk as gdn_scan_kernel.  Every product runs on
// v_mfma_f32_16x16x32_bf16 with each fp32 operand split into a bf16 hi / lo
// pair (about 16 significant bits per operand instead of fp32's 24): three
// products per step for two split operands, two where K, exact in bf16,
// meets a split one.  Kh = diag(gamma_C / gamma) K never forms: the state
// update subtracts K^T (diag(gamma_C / gamma) W Z) and the chunk's own
// tokens add K^T (diag(gamma_C / gamma) U), the scale applied to the fp32
// W Z and U before they are split.
//
// A chunk's operands (Qe and W rows in fp32, K rows in bf16, this
// work-group's 16 columns of U and of the intra outputs) are copied into
// LDS by global_load_lds_dwordx4, one chunk ahead into the other of two
// buffers, in XOR-swizzled row layouts: no registers hold them in flight
// and no staging pass rewrites them.  Each wave reads its Qe or W row
// fragments (fp32, split in registers) and its K^T fragments (transposing
// reads) once per chunk and keeps them for every level.  The level states,
// W Z and U are staged transposed (rows of the 16 value columns); the level
// states stay fp32 in registers and only their copies for the products are
// split.  Lambda rows, gamma_C / gamma_t and the odd batch slots' output
// sums are double-buffered by chunk parity too, so a chunk ends without a
// barrier.
template <int N, int P>
__global__ __launch_bounds__(GDN_SNT) void gdn_scan_bf16_kernel(GdnParams pr) {
  using T = bf16;
  using M = Mfma<bf16>;
  using frag = bf16x8;
  constexpr int C = GDN_C, PB = GDN_PB, NT = GDN_SNT, NWV = NT / 64, c_log = 5;
  static_assert(C == 32 && PB == 16 && N % 32 == 0 && P % PB == 0, "tile shapes");
  constexpr int NTILE = N / 16;                 // 16-row blocks of a state
  constexpr int NTW = (NTILE + NWV - 1) / NWV;  // of them per wave
  constexpr int NKK = N / 32;                   // contraction steps over the key dimension
  constexpr int NL = (C * GDN_LMAX + NT - 1) / NT;
  using LN = GdnRowsN<N>;     // level states (transposed)
  using LF = Rows<float, N>;  // Qe and W rows
  using LK = Rows<bf16, N>;   // K rows
  using LP = Rows<float, PB>;  // U, the intra outputs and the output sums: 16 columns
  __shared__ __attribute__((aligned(16))) float qf[2][C * N];    // Qe
  __shared__ __attribute__((aligned(16))) float wf[2][C * N];    // W
  __shared__ __attribute__((aligned(16))) bf16 kb[2][C * N];     // K
  __shared__ __attribute__((aligned(16))) float uf[2][C * PB];   // U
  __shared__ __attribute__((aligned(16))) float of[2][C * PB];   // intra outputs + even batch slots
  __shared__ __attribute__((aligned(16))) float os1[2][C * PB];  // odd batch slots
  __shared__ __attribute__((aligned(16))) float khs[2][C];       // gamma_C / gamma_t
  __shared__ float lam_s[2][C][GDN_LMAX];
  __shared__ __attribute__((aligned(16))) bf16 zth[GDN_LB * PB * N], ztl[GDN_LB * PB * N];  // Z^T
  __shared__ __attribute__((aligned(16))) bf16 yth[GDN_LB * PB * C], ytl[GDN_LB * PB * C];  // (W Z)^T

  const int nblk = P / PB;
  const int pblk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
  const int H = pr.nheads;
  const int b = bh / H, h = bh % H, p0 = pblk * PB;
  const int64_t T_ = pr.seqlen;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* og = static_cast<T*>(pr.out);
  const T* kg = static_cast<const T*>(pr.k);
  const T* lg = static_cast<const T*>(pr.lam);
  // products: wave w forms Qe Z (outputs) for w mod 4 < 2, else W Z, for
  // token rows [16 (w mod 2), +16) and batch slots w / 4, w / 4 + 2
  const bool qe_wave = (wave & 2) == 0;
  const int rbw = wave & 1, q0w = wave >> 2;

  // chunk j's copies into buffer j mod 2 (U by waves 6 and 7, the intra
  // outputs by waves 4 and 5: the first waves copy a Qe and W piece more),
  // its lambda rows and gamma_C / gamma_t into registers
  T lam[NL];  // raw: converted (and zeroed past the level count) when staged
  float khv = 0.f;
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int item = bh * pr.nc + j, buf = j & 1;
    const int64_t t0 = (int64_t)j * C;
    rows_to_lds<float, C, N, NWV>(pr.qe + (int64_t)item * C * N, N, qf[buf], wave, lane);
    rows_to_lds<float, C, N, NWV>(pr.w + (int64_t)item * C * N, N, wf[buf], wave, lane);
    rows_to_lds<T, C, N, NWV>(kg + (((int64_t)b * T_ + t0) * H + h) * N, (int64_t)H * N, kb[buf], wave, lane);
    rows_to_lds<float, C, PB, NWV>(pr.u + (int64_t)item * C * P + p0, P, uf[buf], (wave + 2) & (NWV - 1), lane);
    rows_to_lds<float, C, PB, NWV>(pr.oi + (int64_t)item * C * P + p0, P, of[buf], (wave + 4) & (NWV - 1), lane);
    // unconditional loads at clamped indices: a load under a branch whose
    // value is converted there makes the wave wait for every copy in flight
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int e = q * NT + tid, t = min(e / GDN_LMAX, C - 1), l = min(e % GDN_LMAX, pr.ll - 1);
      lam[q] = lg[(((int64_t)b * T_ + t0 + t) * H + h) * pr.nlevels + l];
    }
    khv = pr.kh[(int64_t)item * C + (tid & (C - 1))];
  };

  f32x4 Z[GDN_KMAX][NTW];
#pragma unroll
  for (int m = 0; m < GDN_KMAX; ++m)
#pragma unroll
    for (int u = 0; u < NTW; ++u) Z[m][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  for (int j = 0; j < pr.nc; ++j) {
    const int64_t t0 = (int64_t)j * C;
    const int buf = j & 1;
    const float gC = pr.gc[bh * pr.nc + j];
    float* const ofb = of[buf];
    float* const os1b = os1[buf];
    const float* const khb = khs[buf];
    // ---- this chunk's lambda rows and scales into LDS, then the next chunk's copies
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies and loads of the chunk have landed
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int e = q * NT + tid;
      if (e < C * GDN_LMAX) lam_s[buf][e / GDN_LMAX][e % GDN_LMAX] = e % GDN_LMAX < pr.ll ? to_f(lam[q]) : 0.f;
    }
    if (tid < C) khs[buf][tid] = khv;
    for (int i = tid; i < C * PB; i += NT) os1b[i] = 0.f;
    lds_barrier();  // every wave's copies have landed; the other buffer is free
    if (j + 1 < pr.nc) issue(j + 1);
    // this chunk's operand fragments of the wave: Qe or W rows, split
    frag ah[NKK], al[NKK];
    {
      const float* a_s = qe_wave ? qf[buf] : wf[buf];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(a_s + LF::at(16 * rbw + r, 32 * kk + 8 * g));
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(a_s + LF::at(16 * rbw + r, 32 * kk + 8 * g + 4));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 hi, lo;
          split_bf16(e < 4 ? x0[e] : x1[e - 4], hi, lo);
          ah[kk][e] = hi;
          al[kk][e] = lo;
        }
      }
    }
    frag kt[NTW];  // K^T fragments: rows 16 nb + r of K^T, tokens 8 g ..
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int nb = NTW * wave + u;
      kt[u] = nb < NTILE ? frag_down_bf16<LK>(kb[buf], 0, 16 * nb, g, r) : frag{};
    }

    // ---- chunk levels whose bit is set in j, up to GDN_LB at a time
    for (unsigned act = (unsigned)j; act;) {
      int ms[GDN_LB];
      int nbat = 0;
      unsigned bmask = 0;  // bit m: level m is in the batch, at slot popcount(bmask & (2^m - 1))
#pragma unroll
      for (int q = 0; q < GDN_LB; ++q) {
        ms[q] = act ? __builtin_ctz(act) + 1 : 0;  // uniform; 0: no level
        if (act) {
          bmask |= 1u << ms[q];
          act &= act - 1u;
          ++nbat;
        }
      }
      // level states of the batch, transposed and split
#pragma unroll
      for (int m2 = 1; m2 < GDN_KMAX; ++m2)
        if ((bmask >> m2) & 1u) {
          const int q = __builtin_popcount(bmask & ((1u << m2) - 1u));
#pragma unroll
          for (int u = 0; u < NTW; ++u)
            if (NTW * wave + u < NTILE)
              split_store4(zth, ztl, q * PB * N + LN::at(r, 16 * (NTW * wave + u) + 4 * g), Z[m2][u]);
        }
      lds_barrier();
      {
        float* od = q0w ? os1b : ofb;
#pragma unroll
        for (int q = q0w; q < GDN_LB; q += 2) {
          if (q >= nbat) break;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const int o = q * PB * N + LN::at(r, 32 * kk + 8 * g);
            acc = mma3(ah[kk], al[kk], *reinterpret_cast<const frag*>(zth + o),
                       *reinterpret_cast<const frag*>(ztl + o), acc);
          }
          if (qe_wave) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = 16 * rbw + 4 * g + i;
              od[LP::at(t, r)] += lam_s[buf][t][c_log + ms[q]] * acc[i];
            }
          } else {  // diag(gamma_C / gamma) W Z
            const f32x4 ks = *reinterpret_cast<const f32x4*>(khb + 16 * rbw + 4 * g);
            split_store4(yth, ytl, q * PB * C + R32::at(r, 16 * rbw + 4 * g), acc * ks);
          }
        }
      }
      lds_barrier();
      // Z <- gamma_C Z - K^T (diag(gamma_C / gamma) W Z)
#pragma unroll
      for (int m2 = 1; m2 < GDN_KMAX; ++m2)
        if ((bmask >> m2) & 1u) {
          const int q = __builtin_popcount(bmask & ((1u << m2) - 1u));
          const int o = q * PB * C + R32::at(r, 8 * g);
          const frag yh = *reinterpret_cast<const frag*>(yth + o);
          const frag yl = *reinterpret_cast<const frag*>(ytl + o);
#pragma unroll
          for (int u = 0; u < NTW; ++u)
            if (NTW * wave + u < NTILE)
              Z[m2][u] = gC * Z[m2][u] - M::mma(kt[u], yl, M::mma(kt[u], yh, f32x4{0.f, 0.f, 0.f, 0.f}));
        }
      lds_barrier();  // zt and yt are reused by the next batch
    }
    // ---- the chunk's own tokens, K^T (diag(gamma_C / gamma) U), then the
    // Fenwick merge for j + 1
    f32x4 own[NTW];
    {
      // U^T fragment: column p0 + r, tokens 8 g .. 8 g + 7
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(khb + 8 * g);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(khb + 8 * g + 4);
      frag uh, ul;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 hi, lo;
        split_bf16(uf[buf][LP::at(8 * g + e, r)] * (e < 4 ? k0[e] : k1[e - 4]), hi, lo);
        uh[e] = hi;
        ul[e] = lo;
      }
#pragma unroll
      for (int u = 0; u < NTW; ++u)
        own[u] = NTW * wave + u < NTILE ? M::mma(kt[u], ul, M::mma(kt[u], uh, f32x4{0.f, 0.f, 0.f, 0.f}))
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (j + 1 < pr.nc) {
      const int z = __builtin_ctz((unsigned)(j + 1));
#pragma unroll
      for (int m = 1; m < GDN_KMAX; ++m)
        if (m <= z) {
#pragma unroll
          for (int u = 0; u < NTW; ++u) {
            own[u] += Z[m][u];
            Z[m][u] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
      for (int m = 1; m < GDN_KMAX; ++m)
        if (m == z + 1) {
#pragma unroll
          for (int u = 0; u < NTW; ++u) Z[m][u] = own[u];
        }
    }
    for (int i = tid; i < C * PB; i += NT) {
      const int t = i / PB, p = i % PB;
      og[(((int64_t)b * T_ + t0 + t) * H + h) * P + p0 + p] = from_f<T>(ofb[LP::at(t, p)] + os1b[LP::at(t, p)]);
    }
    // No barrier: the next chunk stages lambda, the scales and the odd
    // slots' sums in the other parity's buffers, its first batch writes Z^T
    // only after its first barrier, and the copies into this chunk's
    // buffers start after that barrier too.
  }
}

// ---- the chunk pass for bf16 inputs

// A operand of a 16x16x32 bf16 product from an fp32 C x C tile (LDS, Rows
// layout): lane (g, r) takes row `row`, columns 8 g .. 8 g + 7, each scaled
// by sc[column], split into a bf16 hi / lo pair.
__device__ inline void split_a32(const float* tile, const float* sc, int row, int g, bf16x8& hi, bf16x8& lo) {
  using LC = Rows<float, GDN_C>;
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(tile + LC::at(row, 8 * g));
  const f32x4 a1 = *reinterpret_cast<const f32x4*>(tile + LC::at(row, 8 * g + 4));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (e < 4 ? a0[e] : a1[e - 4]) * (sc ? sc[8 * g + e] : 1.f);
    const bf16 h = (bf16)x;
    hi[e] = h;
    lo[e] = (bf16)(x - (float)h);
  }
}

// Same work as gdn_chunk_kernel.  Q, K and V are bf16 already, so Q K^T and
// K K^T run on v_mfma_f32_16x16x32_bf16 exactly (fp32 accumulation), and the
// products of an fp32 C x C factor with K or V (W, U, Qe, the intra outputs)
// split the fp32 factor into a bf16 hi / lo pair against the exact bf16
// operand (two products per tile, one contraction step of 32 tokens).  The
// triangular inverse and G stay fp32.  Q, K and V are staged in bf16, which
// halves their LDS.
template <int N, int P>
__global__ __launch_bounds__(GDN_NT) void gdn_chunk_bf16_kernel(GdnParams pr) {
  using T = bf16;
  using MF = Mfma<float>;
  using MB = Mfma<bf16>;
  using frag = bf16x8;
  constexpr int C = GDN_C, NT = GDN_NT, c_log = 5;
  static_assert(C == 32 && N % 32 == 0 && P % 16 == 0, "tile shapes");
  constexpr int NTILE = N / 16, PT = P / 16;
  using LN = GdnRowsN<N>;
  using LV = std::conditional_t<P == 32, R32, Rows<bf16, P>>;
  using LC = Rows<float, C>;
  __shared__ __attribute__((aligned(16))) bf16 qb[C * N];
  __shared__ __attribute__((aligned(16))) bf16 kb[C * N];
  __shared__ __attribute__((aligned(16))) bf16 vbf[C * P];
  __shared__ __attribute__((aligned(16))) float am[C * C];  // tril(Q K^T ⊙ Gamma)
  __shared__ __attribute__((aligned(16))) float lm[C * C];  // L
  __shared__ __attribute__((aligned(16))) float tm[C * C];  // Th = (I + L)^-1
  __shared__ __attribute__((aligned(16))) float gm[C * C];  // G
  __shared__ __attribute__((aligned(16))) float gl[C * C];  // G ⊙ lambda by level
  __shared__ __attribute__((aligned(16))) float pt[C * C];  // block-inverse temporary
  __shared__ float lam_s[C][8];                              // intra-chunk levels 0..c
  __shared__ float cum[C], gam[C], bet[C], bg[C];

  const int item = blockIdx.x;  // (batch*head) * nc + chunk
  const int bh = item / pr.nc, j = item % pr.nc;
  const int H = pr.nheads, L = pr.nlevels;
  const int b = bh / H, h = bh % H;
  const int64_t T_ = pr.seqlen, t0 = (int64_t)j * C;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const T* qg = static_cast<const T*>(pr.q);
  const T* kg = static_cast<const T*>(pr.k);
  const T* vg = static_cast<const T*>(pr.v);
  const T* lg = static_cast<const T*>(pr.lam);

  for (int i = tid; i < C * N / 8; i += NT) {  // eight keys / queries per thread and step
    const int t = (8 * i) / N, n = (8 * i) % N;
    const int64_t row = ((int64_t)b * T_ + t0 + t) * H + h;
    *reinterpret_cast<bf16x8*>(qb + LN::at(t, n)) = *reinterpret_cast<const bf16x8*>(qg + row * N + n);
    *reinterpret_cast<bf16x8*>(kb + LN::at(t, n)) = *reinterpret_cast<const bf16x8*>(kg + row * N + n);
  }
  for (int i = tid; i < C * P / 8; i += NT) {
    const int t = (8 * i) / P, p = (8 * i) % P;
    *reinterpret_cast<bf16x8*>(vbf + LV::at(t, p)) =
        *reinterpret_cast<const bf16x8*>(vg + (((int64_t)b * T_ + t0 + t) * H + h) * P + p);
  }
  for (int i = tid; i < C * (c_log + 1); i += NT) {
    const int t = i / (c_log + 1), l = i % (c_log + 1);
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
    const float tot = __shfl(x, C - 1, 64);
    if (tid < C) {
      const float be = pr.beta[gi];
      cum[tid] = x;
      gam[tid] = expf(x);
      bet[tid] = be;
      bg[tid] = be * expf(x);
      pr.kh[(int64_t)item * C + tid] = expf(tot - x);  // gamma_C / gamma_t
      if (tid == 0) pr.gc[item] = expf(tot);
    }
  }
  __syncthreads();
  // ---- Q K^T and K K^T, masked: wave w owns the 16x16 tile (w >> 1, w & 1)
  {
    const int tb = wave >> 1, sb = wave & 1;
    f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
    if (sb <= tb) {
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) {
        const frag bk = *reinterpret_cast<const frag*>(kb + LN::at(16 * sb + r, 32 * kk + 8 * g));
        sq = MB::mma(*reinterpret_cast<const frag*>(qb + LN::at(16 * tb + r, 32 * kk + 8 * g)), bk, sq);
        sk = MB::mma(*reinterpret_cast<const frag*>(kb + LN::at(16 * tb + r, 32 * kk + 8 * g)), bk, sk);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, s = 16 * sb + r;
      const float gr = s <= t ? expf(cum[t] - cum[s]) : 0.f;
      am[LC::at(t, s)] = sq[i] * gr;
      lm[LC::at(t, s)] = s < t ? bet[t] * sk[i] * gr : 0.f;
    }
  }
  __syncthreads();
  // ---- Th = (I + L)^-1, blocked: 8x8 diagonal blocks by substitution,
  // then [[A, 0], [B, D]]^-1 = [[A^-1, 0], [-D^-1 B A^-1, D^-1]] at 16, 32
  if (tid < C) {  // column jc of its 8x8 diagonal block, in registers
    const int jc = tid, blk = jc & ~7, jj = jc & 7;
    float x[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      float v = ii == jj ? 1.f : 0.f;
#pragma unroll
      for (int mm = 0; mm < ii; ++mm) v -= lm[LC::at(blk + ii, blk + mm)] * x[mm];
      x[ii] = ii < jj ? 0.f : v;  // above the diagonal: zero
    }
    for (int i = 0; i < C; ++i) {
      float v = 0.f;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) v = i == blk + ii ? x[ii] : v;
      tm[LC::at(i, jc)] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hb = 8; hb < C; hb *= 2) {  // half block size: 8, then 16
    const int cnt = (C / (2 * hb)) * hb * hb;
    for (int i = tid; i < cnt; i += NT) {  // B A^-1 (rows in the lower half, columns in the upper)
      const int blk = i / (hb * hb), e = i % (hb * hb);
      const int row = blk * 2 * hb + hb + e / hb, col = blk * 2 * hb + e % hb;
      float x = 0.f;
      for (int m = col; m < blk * 2 * hb + hb; ++m) x += lm[LC::at(row, m)] * tm[LC::at(m, col)];
      pt[LC::at(row, col)] = x;
    }
    __syncthreads();
    for (int i = tid; i < cnt; i += NT) {  // the lower-left block: -D^-1 (B A^-1)
      const int blk = i / (hb * hb), e = i % (hb * hb);
      const int row = blk * 2 * hb + hb + e / hb, col = blk * 2 * hb + e % hb;
      float x = 0.f;
      for (int m = blk * 2 * hb + hb; m <= row; ++m) x -= tm[LC::at(row, m)] * pt[LC::at(m, col)];
      tm[LC::at(row, col)] = x;
    }
    __syncthreads();
  }
  // ---- G = tril(Q K^T ⊙ Gamma) Th diag(beta) and G ⊙ lambda (fp32)
  {
    const int tb = wave >> 1, sb = wave & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m0 = 0; m0 < C; m0 += 4)
      acc = MF::mma(frag_along<float, LC>(am, 16 * tb + r, m0, g),
                    frag_down<float, LC>(tm, m0, 16 * sb, g, r), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, s = 16 * sb + r;
      const float gv = s <= t ? acc[i] * bet[s] : 0.f;
      gm[LC::at(t, s)] = gv;
      gl[LC::at(t, s)] = s <= t ? gv * lam_s[t][bit_length((unsigned)(t ^ s))] : 0.f;
    }
  }
  // ---- U = Th diag(beta) V and W = Th diag(beta gamma) K, straight to the
  //      workspace (row tile tile & 1, column tile tile >> 1)
  float* ug = pr.u + (int64_t)item * C * P;
  float* wg = pr.w + (int64_t)item * C * N;
  for (int tile = wave; tile < 2 * PT; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    frag ah, al;
    split_a32(tm, bet, 16 * tb + r, g, ah, al);
    const frag bv = frag_down_bf16<LV>(vbf, 0, 16 * cb, g, r);
    f32x4 acc = MB::mma(ah, bv, f32x4{0.f, 0.f, 0.f, 0.f});
    acc = MB::mma(al, bv, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) ug[(16 * tb + 4 * g + i) * P + 16 * cb + r] = acc[i];
  }
  for (int tile = wave; tile < 2 * NTILE; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    frag ah, al;
    split_a32(tm, bg, 16 * tb + r, g, ah, al);
    const frag bk = frag_down_bf16<LN>(kb, 0, 16 * cb, g, r);
    f32x4 acc = MB::mma(ah, bk, f32x4{0.f, 0.f, 0.f, 0.f});
    acc = MB::mma(al, bk, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) wg[(16 * tb + 4 * g + i) * N + 16 * cb + r] = acc[i];
  }
  __syncthreads();  // gm and gl are complete
  // ---- Qe = diag(gamma) Q - G diag(gamma) K and the intra outputs (G ⊙ lambda) V
  float* qeg = pr.qe + (int64_t)item * C * N;
  float* oig = pr.oi + (int64_t)item * C * P;
  for (int tile = wave; tile < 2 * NTILE; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    frag ah, al;
    split_a32(gm, gam, 16 * tb + r, g, ah, al);
    const frag bk = frag_down_bf16<LN>(kb, 0, 16 * cb, g, r);
    f32x4 acc = MB::mma(ah, bk, f32x4{0.f, 0.f, 0.f, 0.f});
    acc = MB::mma(al, bk, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, n = 16 * cb + r;
      qeg[t * N + n] = gam[t] * (float)qb[LN::at(t, n)] - acc[i];
    }
  }
  for (int tile = wave; tile < 2 * PT; tile += 4) {
    const int tb = tile & 1, cb = tile >> 1;
    frag ah, al;
    split_a32(gl, nullptr, 16 * tb + r, g, ah, al);
    const frag bv = frag_down_bf16<LV>(vbf, 0, 16 * cb, g, r);
    f32x4 acc = MB::mma(ah, bv, f32x4{0.f, 0.f, 0.f, 0.f});
    acc = MB::mma(al, bv, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) oig[(16 * tb + 4 * g + i) * P + 16 * cb + r] = acc[i];
  }
}

using GdnFn = int (*)(const GdnParams&, hipStream_t);

template <class T, int N, int P>
int launch_gdn(const GdnParams& pr, hipStream_t st) {
  const int items = pr.batch * pr.nheads * pr.nc;
  if constexpr (sizeof(T) == 2 && N % 32 == 0)
    hipLaunchKernelGGL((gdn_chunk_bf16_kernel<N, P>), dim3(items), dim3(GDN_NT), 0, st, pr);
  else
    hipLaunchKernelGGL((gdn_chunk_kernel<T, N, P>), dim3(items), dim3(GDN_NT), 0, st, pr);
  const int blocks = pr.batch * pr.nheads * (P / GDN_PB);
  if constexpr (sizeof(T) == 2 && N % 32 == 0)
    hipLaunchKernelGGL((gdn_scan_bf16_kernel<N, P>), dim3(blocks), dim3(GDN_SNT), 0, st, pr);
  else
    hipLaunchKernelGGL((gdn_scan_kernel<T, N, P>), dim3(blocks), dim3(GDN_SNT), 0, st, pr);
  return (int)hipGetLastError();
}

GdnFn lookup_gdn(int dtype, int N, int P);

}  // namespace loglin
