// Device code of the log-linear Mamba-2 forward for gfx950 (MI355X).
//
// Method: log-linear attention write-up (yoousoft.com/industry/3746),
// sections "special structure: tree partition" (mask M^H built from Fenwick
// levels and per-level weights lambda) and "efficient training algorithm"
// (M^H = block-diagonal intra-chunk part + one low-rank term per higher
// level; the intra part is a dense C x C block, the inter part is handled
// by state passing over chunks, O(log(T/C)) levels of O(T) work each).
//
// Three passes, all on the caller's stream:
//   1. state_kernel   reduce each segment of 2^m chunks to one N x P state
//                     S_q = sum_s exp(decay s -> end of segment) B_s X_s^T
//                     (MFMA over the tokens), plus its total log-decay;
//   2. scan_kernel    Fenwick-ordered up-sweep over the segment states in
//                     fp32: slot q receives the decayed sum of the largest
//                     aligned block of segments ending at q (the lower half a
//                     later segment reads at that level);
//   3. output_kernel  per chunk: the dense intra-chunk block (levels
//                     0..log2 C) on MFMA, then every inter-chunk level whose
//                     bit is set in the chunk index, fused in one pass:
//                     Y^T += diag(lambda_t^l exp(Lambda_t + D_l)) (Z_l^T C^T).
//
// Matrix-core conventions (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32,
// 64-wide wavefront): lane = 16*g + r.  Operand A supplies row r and
// contraction elements [KPL*g, KPL*g + KPL) of each KB-wide step; operand B
// supplies column r with the same contraction elements; the 16x16 fp32
// result gives lane (g, r) rows 4g..4g+3 of column r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loglin {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Upper bound on Fenwick depth over segments (supports 2^16 segments).
constexpr int MAX_DEPTH = 16;

struct Params {
  const void* X;
  const void* Bm;
  const void* Cm;
  const float* log_a;
  const void* lam;
  void* out;
  float* seg_state;  // [batch*nheads, ns, P, N] fp32, fragment order
  float* seg_decay;  // [batch*nheads, ns]
  void* slots;       // [batch*nheads, ns, P, N] io type, fragment order
  float* gap_decay;  // [batch*nheads, ns, ks + 1]
  int batch, seqlen, nheads, ngroups, nlevels;
  int nc;     // chunks
  int kc;     // log2(nc): number of inter-chunk levels
  int m;      // log2(chunks per segment)
  int ns;     // segments
  int ks;     // log2(ns)
  int ll;     // levels used: log2(seqlen) + 1
  int total;  // logical work-groups of the kernel being launched
};

// ------------------------------------------------------------ MFMA traits

template <class T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int KB = 32;  // contraction length of one instruction
  static constexpr int KPL = 8;  // contraction elements held by one lane
  using frag = bf16x8;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Contraction over the state dimension uses the order in which the state
  // MFMA leaves rows in registers (4 consecutive rows per lane, two 16-row
  // blocks per step).  Fragment element j of lane group g at step kk holds
  // state row state_row(kk, g, j); a state stored in memory puts row n at
  // position state_pos(n) of its P-row, so one lane reads KPL contiguous
  // elements.
  __host__ __device__ static constexpr int state_row(int kk, int g, int j) {
    return 32 * kk + 16 * (j >> 2) + 4 * g + (j & 3);
  }
  __host__ __device__ static constexpr int state_pos(int n) {
    return 32 * (n >> 5) + 8 * ((n & 15) >> 2) + 4 * ((n & 31) >> 4) + (n & 3);
  }
  // Fragment element (kk, j) of a lane is row state_row(kk, g, j) = element
  // s_i of 16-row tile s_nb of the state MFMA result held by the same lane.
  __host__ __device__ static constexpr int s_nb(int kk, int j) { return 2 * kk + (j >> 2); }
  __host__ __device__ static constexpr int s_i(int, int j) { return j & 3; }
  __device__ static inline float ex(float x) { return __expf(x); }
};

template <>
struct Mfma<float> {
  static constexpr int KB = 4;
  static constexpr int KPL = 1;
  using frag = float;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __host__ __device__ static constexpr int state_row(int kk, int g, int) {
    return 16 * (kk >> 2) + 4 * g + (kk & 3);
  }
  __host__ __device__ static constexpr int state_pos(int n) {
    return 16 * (n >> 4) + 4 * (n & 3) + ((n & 15) >> 2);
  }
  __host__ __device__ static constexpr int s_nb(int kk, int) { return kk >> 2; }
  __host__ __device__ static constexpr int s_i(int kk, int) { return kk & 3; }
  __device__ static inline float ex(float x) { return expf(x); }
};

__device__ inline float to_f(bf16 x) { return (float)x; }
__device__ inline float to_f(float x) { return x; }
template <class T>
__device__ inline T from_f(float x);
template <>
__device__ inline bf16 from_f<bf16>(float x) { return (bf16)x; }
template <>
__device__ inline float from_f<float>(float x) { return x; }

template <class T>
struct alignas(16) Vec16 {
  static constexpr int n = 16 / sizeof(T);
  T e[n];
};

template <class T>
__device__ inline T frag_elem(const typename Mfma<T>::frag& f, int j);
template <>
__device__ inline bf16 frag_elem<bf16>(const bf16x8& f, int j) { return f[j]; }
template <>
__device__ inline float frag_elem<float>(const float& f, int) { return f; }
template <class T>
__device__ inline void set_frag_elem(typename Mfma<T>::frag& f, int j, T v);
template <>
__device__ inline void set_frag_elem<bf16>(bf16x8& f, int j, bf16 v) { f[j] = v; }
template <>
__device__ inline void set_frag_elem<float>(float& f, int, float v) { f = v; }

template <class T>
__device__ inline typename Mfma<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Mfma<T>::frag*>(p);
}

// B operand over the state dimension, read from a token row of C in state
// order (see Mfma::state_row).
__device__ inline bf16x8 load_state_frag(const bf16* row, int kk, int g) {
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * kk + 4 * g);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * kk + 16 + 4 * g);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline float load_state_frag(const float* row, int kk, int g) {
  return row[Mfma<float>::state_row(kk, g, 0)];
}

__device__ inline void store4(bf16* p, f32x4 v) {
  bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ inline void store4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

__device__ inline int bit_length(unsigned x) {
  return x ? 32 - __builtin_clz(x) : 0;
}

// Work-groups are dealt to the 8 XCDs round-robin by id; give each XCD a
// contiguous range of logical tiles so neighbours share its L2.  The grid is
// padded to a multiple of 8 and ids past `total` exit.
__device__ inline int xcd_tile(int bid, int nblocks) {
  int per = nblocks >> 3;
  return (bid & 7) * per + (bid >> 3);
}

template <class T, int C, int P, int N>
struct Tiles {
  using M = Mfma<T>;
  static constexpr int KB = M::KB, KPL = M::KPL;
  static constexpr int NW = P / 16;  // one wave per 16-column block of X
  static constexpr int NT = NW * 64;
  static constexpr int TB = C / 16, PB = P / 16, NB = N / 16;
  static constexpr int KC = C < KB ? KB : C;  // token contraction, padded
  static constexpr int NKT = KC / KB;
  static constexpr int NKN = N / KB;
  static constexpr int XS = KC + 16 / (int)sizeof(T);  // LDS row stride
  static constexpr int VEC = 16 / (int)sizeof(T);
  static_assert(C % 16 == 0 && P % 16 == 0 && N % KB == 0, "tile sizes");
  static_assert(C <= 64, "one wave scans a chunk");
};

// Inclusive prefix sum of log_a over one chunk into cum[0..C), staged in LDS.
template <int C>
__device__ inline void chunk_cumsum(const float* log_a, float* cum, int64_t row0,
                                    int H, int h, int tid) {
  if (tid < 64) {
    float v = tid < C ? log_a[(row0 + tid) * H + h] : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      float o = __shfl_up(v, d, 64);
      if (tid >= d) v += o;
    }
    if (tid < C) cum[tid] = v;
  }
}

// X rows of one chunk -> xt[p][tau] (transposed), bf16/fp32 as stored.
template <class T, int C, int P, int N>
__device__ inline void load_xt(const T* X, T* xt, int64_t row0, int H, int h,
                               int tid) {
  using Tl = Tiles<T, C, P, N>;
  constexpr int PV = P / Tl::VEC;
  for (int idx = tid; idx < C * PV; idx += Tl::NT) {
    int tau = idx / PV, pv = idx - tau * PV;
    Vec16<T> v = *reinterpret_cast<const Vec16<T>*>(
        X + ((row0 + tau) * H + h) * P + pv * Tl::VEC);
#pragma unroll
    for (int e = 0; e < Tl::VEC; ++e) xt[(pv * Tl::VEC + e) * Tl::XS + tau] = v.e[e];
  }
}

// ------------------------------------------------------------- pass 1

// One work-group per (batch, head, segment).  Wave w owns state columns
// [16w, 16w+16) and all N rows, as NB 16x16 fp32 tiles.
template <class T, int C, int P, int N>
__global__ __launch_bounds__((Tiles<T, C, P, N>::NT)) void state_kernel(Params pr) {
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
  __shared__ __attribute__((aligned(16))) T bwt[N * Tl::XS];
  __shared__ __attribute__((aligned(16))) T xt[P * Tl::XS];
  __shared__ float cum[C];

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= pr.total) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int H = pr.nheads, G = pr.ngroups;
  const int q = tile % pr.ns;
  const int bh = tile / pr.ns;
  const int h = bh % H, b = bh / H;
  const int grp = h / (H / G);
  const T* X = static_cast<const T*>(pr.X);
  const T* Bm = static_cast<const T*>(pr.Bm);
  const int seg = 1 << pr.m;

  if (Tl::KC > C) {  // zero the contraction padding once
    for (int idx = tid; idx < (N + P) * (Tl::KC - C); idx += Tl::NT) {
      int row = idx / (Tl::KC - C), col = C + idx % (Tl::KC - C);
      if (row < N) bwt[row * Tl::XS + col] = from_f<T>(0.f);
      else xt[(row - N) * Tl::XS + col] = from_f<T>(0.f);
    }
  }

  f32x4 S[Tl::NB];
#pragma unroll
  for (int nb = 0; nb < Tl::NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float seg_sum = 0.f;

  for (int jl = 0; jl < seg; ++jl) {
    const int j = q * seg + jl;
    if (j >= pr.nc) break;  // last segment of a ragged chunk count
    const int64_t row0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    chunk_cumsum<C>(pr.log_a, cum, row0, H, h, tid);
    __syncthreads();
    const float atot = cum[C - 1];
    constexpr int NV = N / Tl::VEC;
    for (int idx = tid; idx < C * NV; idx += Tl::NT) {
      int tau = idx / NV, nv = idx - tau * NV;
      Vec16<T> v = *reinterpret_cast<const Vec16<T>*>(
          Bm + ((row0 + tau) * G + grp) * N + nv * Tl::VEC);
      float w = M::ex(atot - cum[tau]);
#pragma unroll
      for (int e = 0; e < Tl::VEC; ++e)
        bwt[(nv * Tl::VEC + e) * Tl::XS + tau] = from_f<T>(to_f(v.e[e]) * w);
    }
    load_xt<T, C, P, N>(X, xt, row0, H, h, tid);
    __syncthreads();
    if (jl > 0) {
      const float dec = M::ex(atot);
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb) S[nb] *= dec;
    }
#pragma unroll
    for (int kt = 0; kt < Tl::NKT; ++kt) {
      auto bf = load_frag<T>(xt + (16 * wave + r) * Tl::XS + kt * Tl::KB + g * Tl::KPL);
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb) {
        auto af = load_frag<T>(bwt + (16 * nb + r) * Tl::XS + kt * Tl::KB + g * Tl::KPL);
        S[nb] = M::mma(af, bf, S[nb]);
      }
    }
    seg_sum += atot;
    __syncthreads();
  }

  float* dst = pr.seg_state + ((int64_t)bh * pr.ns + q) * (P * N) + (16 * wave + r) * N;
#pragma unroll
  for (int nb = 0; nb < Tl::NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[M::state_pos(16 * nb + 4 * g + i)] = S[nb][i];
  if (tid == 0) pr.seg_decay[(int64_t)bh * pr.ns + q] = seg_sum;
}

// ------------------------------------------------------------- pass 2

// grid (ceil(P*N/256), batch*nheads).  Each thread owns one state element
// and sweeps the segments in order, keeping a Fenwick stack of block sums in
// fp32 registers: after segment q the top entry is the sum over the largest
// aligned block of segments ending at q, decayed to q's end.  That block is
// the lower half a later segment reads at level trailing_ones(q) + 1.
template <class T>
__global__ __launch_bounds__(256) void scan_kernel(Params pr, int pn) {
  using M = Mfma<T>;
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const bool valid = e < pn;
  const float* src = pr.seg_state + (int64_t)bh * pr.ns * pn;
  const float* dec = pr.seg_decay + (int64_t)bh * pr.ns;
  T* dst = static_cast<T*>(pr.slots) + (int64_t)bh * pr.ns * pn;

  // Gap decays: for segment q and segment level k (1..ks), the log-decay
  // over the segments from the start of q's 2^(k-1)-aligned block to q-1.
  if (blockIdx.x == 0 && threadIdx.x < pr.ks) {
    const int k = threadIdx.x + 1;
    const int mask = (1 << (k - 1)) - 1;
    float run = 0.f;
    float* gd = pr.gap_decay + (int64_t)bh * pr.ns * (pr.ks + 1);
    for (int q = 0; q < pr.ns; ++q) {
      if ((q & mask) == 0) run = 0.f;
      gd[q * (pr.ks + 1) + k] = run;
      run += dec[q];
    }
  }

  float stk[MAX_DEPTH], stka[MAX_DEPTH];
#pragma unroll
  for (int i = 0; i < MAX_DEPTH; ++i) stk[i] = stka[i] = 0.f;
  constexpr int U = 8;  // segments whose loads are in flight together
  const int nq = pr.ns - 1;  // the last segment is never read
  for (int q0 = 0; q0 < nq; q0 += U) {
    float vb[U], db[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u;
      vb[u] = (valid && q < nq) ? src[(int64_t)q * pn + e] : 0.f;
      db[u] = q < nq ? dec[q] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u;
      if (q >= nq) break;
      float v = vb[u];
      float acur = db[u];
      const int z = __builtin_ctz(~(unsigned)q);  // trailing ones of q
#pragma unroll
      for (int i = 0; i < MAX_DEPTH; ++i) {
        if (i < z) {
          v = M::ex(acur) * stk[i] + v;
          acur += stka[i];
        }
      }
#pragma unroll
      for (int i = 0; i < MAX_DEPTH; ++i) {
        if (i == z) {
          stk[i] = v;
          stka[i] = acur;
        }
      }
      if (valid) dst[(int64_t)q * pn + e] = from_f<T>(v);
    }
  }
}

// ------------------------------------------------------------- pass 3

// Largest segment depth m (chunks per segment 2^m) the output pass keeps a
// register stack for.
constexpr int MAX_SEG_LOG2 = 3;

// One work-group per (batch, segment of 2^m chunks, head); the chunks of the
// segment are processed in order.  Wave w owns output columns [16w, 16w+16)
// of the head for all C tokens of a chunk (TB tiles of Y^T), and the same
// columns of every chunk state it builds.
//
// Inter-chunk level k of chunk j reads the lower half of j's 2^k-chunk
// block.  For k > m that block is a run of whole segments: its sum is slot
// ((q >> ks) << ks) + 2^(ks-1) - 1 of pass 2 (ks = k - m), shared by every
// chunk of the segment.  For k <= m it lies inside the segment: the wave
// keeps a Fenwick stack of those block sums, entry e holding the block of
// 2^e chunks that ends just before the current chunk, as MFMA A-operand
// fragments.  The state MFMA leaves a lane exactly the rows its own
// fragments need, so the stack never crosses lanes.
template <class T, int C, int P, int N>
__global__ __launch_bounds__((Tiles<T, C, P, N>::NT), 2) void output_kernel(Params pr) {
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int RS = N + Tl::VEC;  // row stride of the staged B and C rows
  constexpr int NBU = C * N / Tl::VEC;  // 16-byte units of a chunk of B or C
  constexpr int MM = MAX_SEG_LOG2;
  __shared__ __attribute__((aligned(16))) T xt[P * Tl::XS];
  __shared__ __attribute__((aligned(16))) T wt[C * Tl::XS];
  __shared__ __attribute__((aligned(16))) T bsh[C * RS];  // B rows
  __shared__ __attribute__((aligned(16))) T csh[C * RS];  // C rows
  __shared__ __attribute__((aligned(16))) T bwt[N * Tl::XS];  // (B w)^T
  __shared__ float cum[C];
  extern __shared__ float lam_s[];  // [C][ll]

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= pr.total) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int H = pr.nheads, G = pr.ngroups, L = pr.nlevels, LL = pr.ll;
  const int h = tile % H;
  const int q = (tile / H) % pr.ns;
  const int b = tile / (H * pr.ns);
  const int grp = h / (H / G);
  const int bh = b * H + h;
  const int c_log = __builtin_ctz(C);
  const int m = pr.m;
  const int seg = 1 << m;
  const int j0 = q * seg;
  const int nch = min(seg, pr.nc - j0);
  const T* X = static_cast<const T*>(pr.X);
  const T* Bm = static_cast<const T*>(pr.Bm);
  const T* Cm = static_cast<const T*>(pr.Cm);
  const T* lam = static_cast<const T*>(pr.lam);
  const T* slots = static_cast<const T*>(pr.slots);
  T* out = static_cast<T*>(pr.out);

  if (Tl::KC > C) {  // contraction padding of X^T, W and (B w)^T stays zero
    for (int idx = tid; idx < (C + P + N) * (Tl::KC - C); idx += Tl::NT) {
      int row = idx / (Tl::KC - C), col = C + idx % (Tl::KC - C);
      if (row < C) wt[row * Tl::XS + col] = from_f<T>(0.f);
      else if (row < C + P) xt[(row - C) * Tl::XS + col] = from_f<T>(0.f);
      else bwt[(row - C - P) * Tl::XS + col] = from_f<T>(0.f);
    }
  }

  frag zl[MM][Tl::NKN];  // local Fenwick stack (entry e: 2^e chunks)
  float zla[MM];         // total log-decay of each entry's block
  float dloc[MM + 1];    // log-decay from a local block's end to the chunk
#pragma unroll
  for (int e = 0; e < MM; ++e) zla[e] = 0.f;
#pragma unroll
  for (int k = 0; k <= MM; ++k) dloc[k] = 0.f;
  float accseg = 0.f;  // log-decay from the segment start to the chunk
  const float* gap = pr.ks > 0 ? pr.gap_decay + ((int64_t)bh * pr.ns + q) * (pr.ks + 1) : nullptr;

  for (int jl = 0; jl < nch; ++jl) {
    const int j = j0 + jl;
    const int64_t row0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const bool need_state = jl + 1 < nch;

    // ---- stage the chunk: cumulative log-decay, lambda, X^T, B and C rows
    chunk_cumsum<C>(pr.log_a, cum, row0, H, h, tid);
    for (int idx = tid; idx < C * LL; idx += Tl::NT) {
      int tau = idx / LL, l = idx - tau * LL;
      lam_s[idx] = to_f(lam[((row0 + tau) * H + h) * L + l]);
    }
    load_xt<T, C, P, N>(X, xt, row0, H, h, tid);
    constexpr int NV = N / Tl::VEC;
    for (int idx = tid; idx < NBU; idx += Tl::NT) {
      const int tau = idx / NV, nv = idx - tau * NV;
      const int64_t go = ((row0 + tau) * G + grp) * N + nv * Tl::VEC;
      *reinterpret_cast<Vec16<T>*>(bsh + tau * RS + nv * Tl::VEC) =
          *reinterpret_cast<const Vec16<T>*>(Bm + go);
      *reinterpret_cast<Vec16<T>*>(csh + tau * RS + nv * Tl::VEC) =
          *reinterpret_cast<const Vec16<T>*>(Cm + go);
    }
    __syncthreads();
    const float atot = cum[C - 1];

    // ---- (B w)^T for this chunk's state, w_s = exp(atot - cum_s)
    if (need_state) {
      for (int idx = tid; idx < NBU; idx += Tl::NT) {
        const int tau = idx / NV, nv = idx - tau * NV;
        const Vec16<T> v = *reinterpret_cast<const Vec16<T>*>(bsh + tau * RS + nv * Tl::VEC);
        const float w = M::ex(atot - cum[tau]);
#pragma unroll
        for (int e = 0; e < Tl::VEC; ++e)
          bwt[(nv * Tl::VEC + e) * Tl::XS + tau] = from_f<T>(to_f(v.e[e]) * w);
      }
    }

    // ---- intra-chunk weights W[t][s], from the transposed scores B C^T
    for (int u = wave; u < Tl::TB * Tl::TB; u += Tl::NW) {
      const int tb = u / Tl::TB, sb = u - tb * Tl::TB;
      const int t = 16 * tb + r;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (sb <= tb) {
        const T* brow = bsh + (16 * sb + r) * RS + g * Tl::KPL;
        const T* crow = csh + t * RS + g * Tl::KPL;
#pragma unroll
        for (int kk = 0; kk < Tl::NKN; ++kk)
          acc = M::mma(load_frag<T>(brow + kk * Tl::KB), load_frag<T>(crow + kk * Tl::KB), acc);
      }
      f32x4 wv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * sb + 4 * g + i;
        wv[i] = (s <= t) ? acc[i] * M::ex(cum[t] - cum[s]) * lam_s[t * LL + bit_length(t ^ s)]
                         : 0.f;
      }
      store4(wt + t * Tl::XS + 16 * sb + 4 * g, wv);
    }
    __syncthreads();

    // ---- output tiles: intra block, then every active inter-chunk level
    f32x4 Y[Tl::TB];
#pragma unroll
    for (int tb = 0; tb < Tl::TB; ++tb) {
      Y[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < Tl::NKT; ++kt) {
        if (kt * Tl::KB < 16 * (tb + 1)) {
          auto af = load_frag<T>(xt + (16 * wave + r) * Tl::XS + kt * Tl::KB + g * Tl::KPL);
          auto bf = load_frag<T>(wt + (16 * tb + r) * Tl::XS + kt * Tl::KB + g * Tl::KPL);
          Y[tb] = M::mma(af, bf, Y[tb]);
        }
      }
    }
    frag cf[Tl::TB][Tl::NKN];  // C^T fragments in state order
#pragma unroll
    for (int tb = 0; tb < Tl::TB; ++tb)
#pragma unroll
      for (int kk = 0; kk < Tl::NKN; ++kk)
        cf[tb][kk] = load_state_frag(csh + (16 * tb + r) * RS, kk, g);

    auto add_level = [&](const frag* zf, int level, float D) {
#pragma unroll
      for (int tb = 0; tb < Tl::TB; ++tb) {
        f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Tl::NKN; ++kk) tmp = M::mma(zf[kk], cf[tb][kk], tmp);
        const int t = 16 * tb + r;
        const float sc = lam_s[t * LL + level] * M::ex(cum[t] + D);
        Y[tb] += sc * tmp;
      }
    };

    for (int ks = 1; ks <= pr.ks; ++ks) {  // levels above the segment
      if (!((q >> (ks - 1)) & 1)) continue;
      const int qs = ((q >> ks) << ks) + (1 << (ks - 1)) - 1;
      const T* zrow = slots + (((int64_t)bh * pr.ns + qs) * P + 16 * wave + r) * N + g * Tl::KPL;
      frag zf[Tl::NKN];
#pragma unroll
      for (int kk = 0; kk < Tl::NKN; ++kk) zf[kk] = load_frag<T>(zrow + kk * Tl::KB);
      add_level(zf, c_log + m + ks, gap[ks] + accseg);
    }
#pragma unroll
    for (int e = 0; e < MM; ++e) {  // levels inside the segment
      if (e < m && ((jl >> e) & 1)) add_level(zl[e], c_log + e + 1, dloc[e + 1]);
    }

#pragma unroll
    for (int tb = 0; tb < Tl::TB; ++tb) {
      const int t = 16 * tb + r;
      store4(out + ((row0 + t) * H + h) * P + 16 * wave + 4 * g, Y[tb]);
    }

    // ---- this chunk's state, pushed on the local Fenwick stack
    if (need_state) {
      f32x4 S[Tl::NB];
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < Tl::NKT; ++kt) {
        auto bf = load_frag<T>(xt + (16 * wave + r) * Tl::XS + kt * Tl::KB + g * Tl::KPL);
#pragma unroll
        for (int nb = 0; nb < Tl::NB; ++nb) {
          auto af = load_frag<T>(bwt + (16 * nb + r) * Tl::XS + kt * Tl::KB + g * Tl::KPL);
          S[nb] = M::mma(af, bf, S[nb]);
        }
      }
      // merge with the entries of the blocks this chunk completes
      const int z = __builtin_ctz(~(unsigned)jl);  // trailing ones of jl
      float cur_a = atot;
#pragma unroll
      for (int e = 0; e < MM; ++e) {
        if (e < z) {
          const float dec = M::ex(cur_a);
#pragma unroll
          for (int kk = 0; kk < Tl::NKN; ++kk)
#pragma unroll
            for (int jj = 0; jj < Tl::KPL; ++jj)
              S[M::s_nb(kk, jj)][M::s_i(kk, jj)] += dec * to_f(frag_elem<T>(zl[e][kk], jj));
          cur_a += zla[e];
        }
      }
#pragma unroll
      for (int e = 0; e < MM; ++e) {
        if (e == z) {
#pragma unroll
          for (int kk = 0; kk < Tl::NKN; ++kk)
#pragma unroll
            for (int jj = 0; jj < Tl::KPL; ++jj)
              set_frag_elem<T>(zl[e][kk], jj, from_f<T>(S[M::s_nb(kk, jj)][M::s_i(kk, jj)]));
          zla[e] = cur_a;
        }
      }
    }

    // ---- running log-decays for the next chunk
    accseg += atot;
#pragma unroll
    for (int k = 1; k <= MM; ++k) {
      dloc[k] += atot;
      if (((jl + 1) & ((1 << (k - 1)) - 1)) == 0) dloc[k] = 0.f;
    }
    __syncthreads();  // LDS is restaged by the next chunk
  }
}

}  // namespace loglin
