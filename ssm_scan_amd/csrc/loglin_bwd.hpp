// Device code of the log-linear Mamba-2 backward pass for gfx950 (MI355X).
//
// Method: log-linear attention write-up (yoousoft.com/industry/3746),
// sections "special structure: tree partition" (O = (C B^T ⊙ M^H) X with
// M^H[t, s] = prod_{r=s+1..t} a_r * lambda[t, level(t, s)]) and "efficient
// training algorithm" (intra-chunk blocks plus one low-rank term per chunk
// level).  The write-up gives no backward formulas; these are the calculus
// of that definition.  With S = C B^T, D = dO X^T and G = M ⊙ S ⊙ D:
//
//   dX_s = sum_t (M ⊙ S)[t, s] dO_t     dB_s = sum_t (M ⊙ D)[t, s] C_t
//   dC_t = sum_s (M ⊙ D)[t, s] B_s      dlambda[t, l] = dO_t . Y^(l)_t
//   dlog_a_r = sum_{t >= r} (dO_t . O_t - X_t . dX_t)
//
// (G's row sums are dO_t . O_t and its column sums X_s . dX_s, and log a_r
// enters the entries with s < r <= t.)  dB and dC sum over the heads of a
// group.
//
// Chunk level k (token level c + k, C = 2^c) pairs the lower and upper
// halves of each aligned block of 2^k chunks.  Queries in the upper half
// read the lower half's state (forward direction: key B, value X, lambda of
// the query); keys in the lower half receive from the upper half (reverse
// direction: key C, value dO, and lambda[t, c + k] of the upper half's
// tokens, which is why those states are per level).  Launches:
//   1. bwd_atot_kernel          per-chunk total log-decay, bwd_cuma_kernel
//                               their fp64 prefix sums;
//   2. forward direction: bwd_zst_group_kernel, per aligned group of 8
//                               chunks, the lower halves of levels 1-4 as
//                               nested blocks of the chunk states, and
//                               bwd_zst_up_kernel the levels above from the
//                               groups' totals;
//                               reverse direction: bwd_level_state_kernel,
//                               per (level, pair, piece of <= 8 chunks), the
//                               decayed sum over the piece's chunks of the
//                               upper half;
//   3. bwd_level_reduce_kernel  reverse pieces -> one state per (level,
//                               pair), fp32;
//   4. bwd_dq_kernel            per (group, chunk): dC and each head's
//                               dlambda, from the intra block and the
//                               lower-half states;
//   5. bwd_dkv_kernel           per (group, chunk): each head's dX, and dB,
//                               from the intra block and the upper-half states
//                               (a work-group takes the group's heads in turn
//                               and sums their dB or dC in registers);
//   6. bwd_dloga_part_kernel, bwd_dloga_kernel   suffix sums of dO.O - X.dX.
#pragma once

#include "loglin_device.hpp"
#include "loglin_out2.hpp"

namespace loglin {

struct BwdParams {
  const void* X;
  const void* Bm;
  const void* Cm;
  const float* log_a;
  const void* lam;
  const void* dO;
  void* dX;
  void* dB;
  void* dC;
  float* dloga;
  void* dlam;
  float* atot;    // [batch*nheads, nc]
  double* cuma;   // [batch*nheads, nc + 1] exclusive prefix sums of atot
  float* part_f;  // [batch*nheads, ceil(nc / 8), N, P] fp32, totals of the groups of 8 chunks
  float* part_r;  // [batch*nheads, npart, N, P] fp32, upper-half pieces
  float* zst;     // [batch*nheads, nstate, N, P] lower-half sums (level-state form, below)
  float* rst;     // [batch*nheads, nstate, N, P] upper-half sums (level-state form)
  float* term1;   // [batch*nheads, seqlen] dO_t . O_t
  float* term2;   // [batch*nheads, seqlen] X_t . dX_t
  int batch, seqlen, nheads, ngroups, nlevels;
  int nc, kc, ll;
  int npart, nstate;  // per (batch, head)
  int nstate_direct;  // states of the levels whose half is one piece (listed first)
};

// Pieces of at most BWD_PIECE chunks bound the serial work of one
// work-group in the level-state pass.
constexpr int BWD_PIECE = 8;
// Levels held per token row in LDS (sequences up to 2^31 tokens).
constexpr int BWD_LMAX = 32;

// Pairs at chunk level k whose upper half holds at least one chunk.
__host__ __device__ inline int bwd_pairs(int nc, int k) {
  const int half = 1 << (k - 1);
  return nc > half ? (nc + half - 1) >> k : 0;  // ceil((nc - half) / 2^k), a shift: no division
}
// Pieces per half at chunk level k.
__host__ __device__ inline int bwd_pieces(int k) {
  return ((1 << (k - 1)) + BWD_PIECE - 1) / BWD_PIECE;
}
// Flat piece index (levels in order, then pairs, then pieces) -> parts.
__device__ inline void bwd_piece_of(int item, int nc, int kc, int& k, int& pair, int& pc) {
  for (k = 1; k <= kc; ++k) {
    const int np = bwd_pieces(k), cnt = bwd_pairs(nc, k) * np;
    if (item < cnt) {
      pair = item / np;
      pc = item % np;
      return;
    }
    item -= cnt;
  }
  k = pair = pc = 0;  // not reached for item < npart
}
// Flat state index (levels in order, then pairs) -> parts, and back.
__device__ inline void bwd_state_of(int item, int nc, int kc, int& k, int& pair) {
  for (k = 1; k <= kc; ++k) {
    const int cnt = bwd_pairs(nc, k);
    if (item < cnt) {
      pair = item;
      return;
    }
    item -= cnt;
  }
  k = pair = 0;
}
__device__ inline int bwd_state_index(int nc, int k, int pair) {
  int s = 0;
  for (int k2 = 1; k2 < k; ++k2) s += bwd_pairs(nc, k2);
  return s + pair;
}
__device__ inline int bwd_piece_base(int nc, int k) {
  int s = 0;
  for (int k2 = 1; k2 < k; ++k2) s += bwd_pairs(nc, k2) * bwd_pieces(k2);
  return s;
}

// R token rows of W elements (global row stride grs) into LDS, Rows layout.
template <class T, int R, int W, int NT>
__device__ inline void rows_load(const T* g, int64_t grs, T* lds, int tid) {
  using L = Rows<T, W>;
  constexpr int PIECES = R * L::NBLK;
#pragma unroll
  for (int i0 = 0; i0 < PIECES; i0 += NT) {
    const int i = i0 + tid;
    if (i < PIECES) {
      const int row = i / L::NBLK, pb = i % L::NBLK;
      store16(lds + L::at(row, pb * L::VEC), load16(g + (int64_t)row * grs + pb * L::VEC));
    }
  }
}

// One chunk's state S[n][p] += sum_t key[t][n] w[t] val[t][p] for this wave's
// 16 columns (the forward's chunk_state_mma), with w[t] val[t][p] split into
// hi and lo bf16 fragments for bf16 io (the split of the level states, see
// state_put4).
template <class T, int C, int P, int N>
__device__ inline void chunk_state_mma_split(const T* ks, const T* vs, const float* w, f32x4* S,
                                             int wave, int g, int r) {
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
#pragma unroll
  for (int kt = 0; kt < Tl::NKT; ++kt) {
    if constexpr (sizeof(T) == 2) {
      const auto f = frag_down<T, Rows<T, P>>(vs, kt * Tl::KB, 16 * wave, g, r);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + kt * Tl::KB + 8 * g);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + kt * Tl::KB + 8 * g + 4);
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = (float)f[j] * w0[j], v1 = (float)f[j + 4] * w1[j];
        hi[j] = (bf16)v0;
        hi[j + 4] = (bf16)v1;
        lo[j] = (bf16)(v0 - (float)hi[j]);
        lo[j + 4] = (bf16)(v1 - (float)hi[j + 4]);
      }
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb) {
        const auto af = frag_down<T, Rows<T, N>>(ks, kt * Tl::KB, 16 * nb, g, r);
        S[nb] = M::mma(af, hi, S[nb]);
        S[nb] = M::mma(af, lo, S[nb]);
      }
    } else {
      const auto bf = frag_down_scaled<T, Rows<T, P>>(vs, w, kt * Tl::KB, 16 * wave, g, r);
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb)
        S[nb] = M::mma(frag_down<T, Rows<T, N>>(ks, kt * Tl::KB, 16 * nb, g, r), bf, S[nb]);
    }
  }
}

// sum over the 16 lanes r of a lane group (MFMA result columns)
__device__ inline float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// A DPP lane move within rows of 16 lanes (every source lane in range).
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Four sums at once over the 16 lanes of each lane row: afterwards lane r
// holds the total of v[[0, 2, 1, 3][r mod 4]].  Two exchanges inside each
// lane quad halve the values a lane carries (quad_perm [1,0,3,2], then
// [2,3,0,1]); two rotations of the row by 4 and 8 lanes add the four quads.
__device__ inline float sum16x4(const f32x4& v, int r) {
  const bool o1 = (r & 1) != 0, o2 = (r & 2) != 0;
  const float s0 = (o1 ? v[2] : v[0]) + dpp_mov<0xb1>(o1 ? v[0] : v[2]);
  const float s1 = (o1 ? v[3] : v[1]) + dpp_mov<0xb1>(o1 ? v[1] : v[3]);
  float k = (o2 ? s1 : s0) + dpp_mov<0x4e>(o2 ? s0 : s1);
  k += dpp_mov<0x124>(k);  // row_ror:4
  k += dpp_mov<0x128>(k);  // row_ror:8
  return k;
}

// ------------------------------------------------------------ launch 1

template <class T, int C>
__global__ __launch_bounds__(64) void bwd_atot_kernel(BwdParams pr) {
  __shared__ float cum[64], ecum[64], wst[64];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / pr.nheads, h = bh % pr.nheads;
  const float la =
      tid < C ? pr.log_a[((int64_t)b * pr.seqlen + (int64_t)j * C + tid) * pr.nheads + h] : 0.f;
  chunk_decays<T, C>(la, cum, ecum, wst, tid);  // the same sums the chunk passes form
  __syncthreads();
  if (tid == 0) pr.atot[(int64_t)bh * pr.nc + j] = cum[C - 1];
}

// grid (batch*nheads), 1024 threads: cuma[j] = sum_{m < j} atot[m] in fp64,
// so that any range of chunk log-decays (a level's gap) is one subtraction
// with no cancellation at fp32 resolution.
constexpr int BWD_SCAN_NT = 1024;
template <class T>  // (a template so that every unit's copy is a weak symbol)
__global__ __launch_bounds__(BWD_SCAN_NT) void bwd_cuma_kernel(BwdParams pr) {
  __shared__ double sh[BWD_SCAN_NT];
  const int bh = blockIdx.x, tid = threadIdx.x, nc = pr.nc;
  const int per = (nc + BWD_SCAN_NT - 1) / BWD_SCAN_NT;
  const int lo = min(tid * per, nc), hi = min(lo + per, nc);
  const float* at = pr.atot + (int64_t)bh * nc;
  double tot = 0.0;
  for (int m = lo; m < hi; ++m) tot += at[m];
  sh[tid] = tot;
  __syncthreads();
  for (int d = 1; d < BWD_SCAN_NT; d <<= 1) {  // inclusive prefix sums over threads
    const double v = tid >= d ? sh[tid - d] : 0.0;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  double run = tid ? sh[tid - 1] : 0.0;
  double* ca = pr.cuma + (int64_t)bh * (nc + 1);
  for (int m = lo; m < hi; ++m) {
    ca[m] = run;
    run += at[m];
  }
  if (tid == BWD_SCAN_NT - 1) ca[nc] = sh[BWD_SCAN_NT - 1];
}

// Token tiles of one chunk staged through registers: every global load of
// the four tiles is issued before the first LDS store, so the work-group
// waits for one memory latency instead of one per load.  The loads are
// unconditional (a short tile's spare lanes load its last piece again and
// store nothing): a load under a branch into a register that lives across
// the branch makes the next one wait for it.
template <class T, int R, int W, int NT>
struct RowsStage {
  using L = Rows<T, W>;
  static constexpr int PIECES = R * L::NBLK;
  static constexpr int IT = (PIECES + NT - 1) / NT;
  vec16_t<T> v[IT];
  __device__ inline void load(const T* g, int64_t grs, int tid) {
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int i = PIECES % NT == 0 ? q * NT + tid : min(q * NT + tid, PIECES - 1);
      v[q] = load16(g + (int64_t)(i / L::NBLK) * grs + (i % L::NBLK) * L::VEC);
    }
  }
  __device__ inline void store(T* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int i = q * NT + tid;
      if (i < PIECES) store16(lds + L::at(i / L::NBLK, (i % L::NBLK) * L::VEC), v[q]);
    }
  }
};

// A tile of R token rows staged in LDS in the Rows layout, written to global
// rows (row stride grs elements) 16 bytes a lane: one store instruction per
// lane and 16-byte piece instead of one per element.
template <class T, int R, int W, int NT>
__device__ inline void rows_from_lds(const T* lds, T* g, int64_t grs, int tid) {
  using L = Rows<T, W>;
  constexpr int PIECES = R * L::NBLK;
#pragma unroll
  for (int q = 0; q < (PIECES + NT - 1) / NT; ++q) {
    const int i = q * NT + tid;
    if (PIECES % NT == 0 || i < PIECES) {
      const int row = i / L::NBLK, blk = i % L::NBLK;
      store16(g + (int64_t)row * grs + blk * L::VEC, load16(lds + L::at(row, blk * L::VEC)));
    }
  }
}

// Level weights' gradients of C token rows (L per row, row stride H L), the
// first ll of each row from LDS and zeros past them; 16 bytes a lane when
// the rows are whole 16-byte pieces.
template <class T, int C, int LMAX, int NT>
__device__ inline void dlam_rows_out(const float (*dl)[LMAX], T* g, int H, int L, int ll, int tid) {
  constexpr int VEC = 16 / (int)sizeof(T);
  if (L % VEC == 0) {  // uniform
    for (int i = tid; i < C * (L / VEC); i += NT) {
      const int t = i / (L / VEC), l0 = (i % (L / VEC)) * VEC;
      vec16_t<T> v;
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = from_f<T>(l0 + e < ll ? dl[t][l0 + e] : 0.f);
      store16(g + (int64_t)t * H * L + l0, v);
    }
  } else {
    for (int i = tid; i < C * L; i += NT) {
      const int t = i / L, l = i % L;
      g[(int64_t)t * H * L + l] = from_f<T>(l < ll ? dl[t][l] : 0.f);
    }
  }
}

// Level states (zst, rst) as the chunk passes take them: for bf16 io a pair
// of bf16 planes, hi = rnd(v) and lo = rnd(v - hi), each [N][P], which the
// products use as two bf16 operands, so that they keep about 16 bits of the
// fp32 state; for fp32 io the fp32 values [N][P].  Same bytes either way;
// element (n, p) is at n P + p.  The 16 bits matter for dlog_a: it is a
// suffix sum over the whole sequence of dO_t . O_t - X_t . dX_t, two terms
// formed through different states (the lower-half state against dO, the
// upper-half state against B and X); with the states rounded to bf16 their
// mismatch near every chunk boundary would accumulate along the sequence.
//
// Four consecutive elements idx .. idx + 3 of a state in that form.
template <class T, int N, int P>
__device__ inline void state_put4(float* st, int idx, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    bf16* hp = reinterpret_cast<bf16*>(st);
    bf16x4 hv, lv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hv[e] = (bf16)v[e];
      lv[e] = (bf16)(v[e] - (float)hv[e]);
    }
    *reinterpret_cast<bf16x4*>(hp + idx) = hv;
    *reinterpret_cast<bf16x4*>(hp + N * P + idx) = lv;
  } else {
    *reinterpret_cast<f32x4*>(st + idx) = v;
  }
}

// A wave's NB 16x16 tiles of a state (MFMA layout: lane (g, r) holds rows
// 16 nb + 4 g + i, i < 4, of column col0 + r) in the level-state form.  For
// bf16 the two lanes of a pair (r, r + 1) swap one value of each tile, so
// that each writes two adjacent columns of two rows, four bytes a store:
// the even lane rows 4 g and 4 g + 2, the odd lane rows 4 g + 1 and 4 g + 3.
template <class T, int N, int P, int NB>
__device__ inline void state_put_tiles(float* st, const f32x4* S, int col0, int g, int r) {
  if constexpr (sizeof(T) == 2) {
    bf16* hp = reinterpret_cast<bf16*>(st);
    const bool odd = (r & 1) != 0;
    const int pc = col0 + (r & ~1);  // the pair's first column
    auto put2 = [&](int idx, float x, float y) __attribute__((always_inline)) {
      const bf16 hx = (bf16)x, hy = (bf16)y;
      const bf16 lx = (bf16)(x - (float)hx), ly = (bf16)(y - (float)hy);
      *reinterpret_cast<bf16x2*>(hp + idx) = bf16x2{hx, hy};
      *reinterpret_cast<bf16x2*>(hp + N * P + idx) = bf16x2{lx, ly};
    };
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // the even lane receives the odd lane's rows 0 and 2, the odd lane the
      // even lane's rows 1 and 3
      const float a = dpp_mov<0xb1>(odd ? S[nb][0] : S[nb][1]);
      const float c = dpp_mov<0xb1>(odd ? S[nb][2] : S[nb][3]);
      const int n0 = 16 * nb + 4 * g + (odd ? 1 : 0);
      put2(n0 * P + pc, odd ? a : S[nb][0], odd ? S[nb][1] : a);
      put2((n0 + 2) * P + pc, odd ? c : S[nb][2], odd ? S[nb][3] : c);
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[(16 * nb + 4 * g + i) * P + col0 + r] = S[nb][i];
  }
}

// The same tiles (bf16) staged in LDS planes hl, ll ([N][P] each, the level
// state's two planes), so that the state can go out in whole lines
// (state_lds_out, after a barrier).
template <int N, int P, int NB>
__device__ inline void state_tiles_to_lds(bf16* hl, bf16* ll, const f32x4* S, int col0, int g, int r) {
  const bool odd = (r & 1) != 0;
  const int pc = col0 + (r & ~1);
  auto put2 = [&](int idx, float x, float y) __attribute__((always_inline)) {
    const bf16 hx = (bf16)x, hy = (bf16)y;
    *reinterpret_cast<bf16x2*>(hl + idx) = bf16x2{hx, hy};
    *reinterpret_cast<bf16x2*>(ll + idx) = bf16x2{(bf16)(x - (float)hx), (bf16)(y - (float)hy)};
  };
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float a = dpp_mov<0xb1>(odd ? S[nb][0] : S[nb][1]);
    const float c = dpp_mov<0xb1>(odd ? S[nb][2] : S[nb][3]);
    const int n0 = 16 * nb + 4 * g + (odd ? 1 : 0);
    put2(n0 * P + pc, odd ? a : S[nb][0], odd ? S[nb][1] : a);
    put2((n0 + 2) * P + pc, odd ? c : S[nb][2], odd ? S[nb][3] : c);
  }
}
// The staged planes out as one level state, 16 bytes a thread (NTH threads,
// thread index t).
template <int N, int P, int NTH>
__device__ inline void state_lds_out(float* st, const bf16* hl, const bf16* ll, int t) {
  constexpr int PP = N * P / 8;  // 16-byte pieces per plane
  bf16* hp = reinterpret_cast<bf16*>(st);
#pragma unroll
  for (int i0 = 0; i0 < 2 * PP; i0 += NTH) {
    const int i = i0 + t;
    if ((2 * PP) % NTH == 0 || i < 2 * PP) {
      const int plane = i / PP, off = (i % PP) * 8;
      store16(hp + plane * (N * P) + off, load16((plane ? ll : hl) + off));
    }
  }
}

// ------------------------------------------------------------ launch 2

// grid (npart, batch*nheads).  Wave w owns state columns [16 w, 16 w + 16)
// and all N rows (NB tiles of 16x16 fp32), as in the forward's state pass.
// Forward direction (REV false): chunks of the piece in order, key B, value
// X, weight exp(decay s -> chunk end); acc <- exp(Atot_j) acc + chunk state,
// so the result is decayed to the end of the piece.  Reverse: chunks in
// reverse order, key C, value dO, weight lambda[t, c + k] exp(decay from the
// chunk start to t); acc <- exp(Atot_j) acc + chunk state, decayed to the
// start of the piece.  A level whose half is a single piece writes its state
// directly; other levels write partials for bwd_level_reduce_kernel.  The
// next chunk's rows are loaded into registers while the current one is used.
template <class T, int C, int P, int N, bool REV>
__global__ __launch_bounds__((Tiles<T, C, P, N>::NT)) void bwd_level_state_kernel(BwdParams pr) {
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
  constexpr int NT = Tl::NT;
  static_assert(Tl::KC == C, "token tiles are not padded here");
  static_assert(REV, "forward-direction states come from bwd_zst_group_kernel (part_f holds group totals)");
  __shared__ __attribute__((aligned(16))) T ksh[C * N];
  __shared__ __attribute__((aligned(16))) T vsh[C * P];
  __shared__ __attribute__((aligned(16))) float cum[64], ecum[64], wst[64], wsh[64];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, H = pr.nheads, G = pr.ngroups, L = pr.nlevels;
  const int b = bh / H, h = bh % H, grp = h / (H / G);
  const int64_t T_ = pr.seqlen;
  int k, pair, pc;
  bwd_piece_of(blockIdx.x, pr.nc, pr.kc, k, pair, pc);
  const int half = 1 << (k - 1);
  const int base = pair * 2 * half + (REV ? half : 0);  // first chunk of the half
  const int lo = base + pc * BWD_PIECE;
  if (lo >= pr.nc) return;  // uniform: a piece past the sequence (the reduce skips it)
  const int hi = min(min(lo + BWD_PIECE, base + half), pr.nc);
  constexpr int c_log = ilog2c(C);

  f32x4 S[Tl::NB];
#pragma unroll
  for (int nb = 0; nb < Tl::NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  RowsStage<T, C, N, NT> sk;
  RowsStage<T, C, P, NT> sv;
  // issue the loads of chunk j's rows; returns its log a and lambda value
  // for this thread's token (by value: see the scan pass on loop-carried
  // values held through references).  Both loads are unconditional and
  // lambda stays in the io type until it is used: converting it here would
  // make the wave wait for the rows in flight.
  struct Next {
    float la;
    T lam;
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)j * C;
    const T* kg = static_cast<const T*>(REV ? pr.Cm : pr.Bm) + (((int64_t)b * T_ + t0) * G + grp) * N;
    const T* vg = static_cast<const T*>(REV ? pr.dO : pr.X) + (((int64_t)b * T_ + t0) * H + h) * P;
    sk.load(kg, (int64_t)G * N, tid);
    sv.load(vg, (int64_t)H * P, tid);
    const int tt = tid < C ? tid : 0;
    Next v;
    v.la = pr.log_a[((int64_t)b * T_ + t0 + tt) * H + h];
    v.lam = REV ? static_cast<const T*>(pr.lam)[(((int64_t)b * T_ + t0 + tt) * H + h) * L + c_log + k]
                : from_f<T>(0.f);
    return v;
  };
  const int n = hi - lo;
  Next nxt = {0.f, from_f<T>(0.f)};
  if (n > 0) nxt = issue(REV ? hi - 1 : lo);
  for (int step = 0; step < n; ++step) {
    sk.store(ksh, tid);
    sv.store(vsh, tid);
    const float la = tid < C ? nxt.la : 0.f, lamv = to_f(nxt.lam);
    if (step + 1 < n) nxt = issue(REV ? hi - 2 - step : lo + step + 1);
    chunk_decays<T, C>(la, cum, ecum, wst, tid);
    lds_barrier();
    if (tid < C) wsh[tid] = REV ? lamv * ecum[tid] : wst[tid];
    lds_barrier();
    const float dec = M::ex(cum[C - 1]);
#pragma unroll
    for (int nb = 0; nb < Tl::NB; ++nb) S[nb] *= dec;
    chunk_state_mma_split<T, C, P, N>(ksh, vsh, wsh, S, wave, g, r);
    lds_barrier();  // the next chunk restages the tiles
  }
  if (bwd_pieces(k) == 1) {  // the level's state itself
    float* dst = (REV ? pr.rst : pr.zst) + ((int64_t)bh * pr.nstate + bwd_state_index(pr.nc, k, pair)) * (N * P);
    state_put_tiles<T, N, P, Tl::NB>(dst, S, 16 * wave, g, r);
  } else {  // an fp32 partial for the reduce
    float* dst = (REV ? pr.part_r : pr.part_f) + ((int64_t)bh * pr.npart + blockIdx.x) * (N * P);
#pragma unroll
    for (int nb = 0; nb < Tl::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * nb + 4 * g + i) * P + 16 * wave + r] = S[nb][i];
  }
}

// The reverse-direction pieces for the output pass's shape (bf16, 64-token
// chunks, P = 64, N = 64 or 128), in that pass's LDS layouts: C rows in
// 272-byte rows, dO rows with the lane-keyed swizzle, so every transposing
// operand read is a lane base plus an immediate.  One work-group per (piece,
// batch, two heads of a group), eight waves: wave w serves head w / 4 and
// its state columns [16 (w mod 4), +16); the heads share one copy of the C
// rows.  The piece's log-decays and level weights are copied once, up front,
// and each chunk's weights are formed while the chunk after it (the walk
// runs backwards) is being reduced.  What it computes is
// bwd_level_state_kernel's reverse direction.
template <int N>
__global__ __launch_bounds__(512, 2) void bwd_level_state2_kernel(BwdParams pr) {
  using O = Out2<N>;
  using M = Mfma<bf16>;
  constexpr int C = O::C, P = O::P, NB = O::NB, BROW = O::BROW, BBLK = O::BBLK, BINST = O::BINST;
  constexpr int NWT = 8;
  constexpr int c_log = 6;
  __shared__ __attribute__((aligned(16))) unsigned char csh0[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char csh1[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char dsh0[2][C * P * 2];
  __shared__ __attribute__((aligned(16))) unsigned char dsh1[2][C * P * 2];
  // per head: the piece's log-decays and level-weight words (by position in
  // the piece), and per chunk parity the decays and the weights
  __shared__ __attribute__((aligned(16))) float las[2][BWD_PIECE * C];
  __shared__ __attribute__((aligned(16))) unsigned lws[2][BWD_PIECE * C];
  __shared__ __attribute__((aligned(16))) float cum[2][2][C], ecum[2][2][C], wst[2][2][C], wsh[2][2][C];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NWT);
  const int hh = wave >> 2, wv = wave & 3;
  const int g = lane >> 4, r = lane & 15;
  const int H = pr.nheads, G = pr.ngroups, L = pr.nlevels;
  const int b = blockIdx.y / (H / 2), h0 = 2 * (blockIdx.y % (H / 2));
  const int h = h0 + hh, grp = h0 / (H / G);
  const int bh = b * H + h;
  const int64_t T_ = pr.seqlen;
  int k, pair, pc;
  bwd_piece_of(blockIdx.x, pr.nc, pr.kc, k, pair, pc);
  const int half = 1 << (k - 1);
  const int base = pair * 2 * half + half;  // first chunk of the upper half
  const int lo = base + pc * BWD_PIECE;
  if (lo >= pr.nc) return;  // uniform: a piece past the sequence (the reduce skips it)
  const int hi = min(min(lo + BWD_PIECE, base + half), pr.nc);
  const int n = hi - lo;
  const int lev = c_log + k;
  const bf16* Cg = static_cast<const bf16*>(pr.Cm);
  const bf16* Dg = static_cast<const bf16*>(pr.dO);

  // C^T transposing reads: + (32 kt + 4 hh) BROW + 32 nb
  const unsigned o_bt = (8 * g + (r >> 2)) * BROW + 8 * (r & 3);
  // dO^T transposing reads: + (32 kt + 4 hh) 128
  const int keyx = ((r >> 3) & 1) | ((g & 1) << 1);
  const unsigned o_xt = (8 * g + (r >> 2)) * 128 + 16 * ((2 * wv + ((r & 3) >> 1)) ^ (2 * keyx)) +
                        8 * (r & 1);
  const unsigned rs_c = (unsigned)G * N * 2, rs_d = (unsigned)H * P * 2;
  auto cc_off = [&](int inst) __attribute__((always_inline)) {
    const unsigned pos = (unsigned)(inst * 64 + lane);
    const unsigned rho = pos / BBLK;
    const unsigned blk = min(pos - rho * BBLK, (unsigned)(BBLK - 2));
    return __umul24(rho, rs_c) + 16u * blk;
  };
  auto cd_off = [&](int kx) __attribute__((always_inline)) {
    const int pos = (wv + 4 * kx) * 64 + lane;
    const int rho = pos >> 3, phys = pos & 7;
    const int key = ((rho >> 1) & 1) | (((rho >> 3) & 1) << 1);
    return __umul24((unsigned)rho, rs_d) + 16u * (phys ^ (2 * key));
  };
  auto issue = [&](int j, unsigned char* cs, unsigned char (*ds)[C * P * 2]) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * T_ + (int64_t)j * C;
    const bf16* csrc = Cg + (r0 * G + grp) * N;
    const bf16* dsrc = Dg + (r0 * H + h) * P;
#pragma unroll
    for (int kx = 0; kx < (BINST + NWT - 1) / NWT; ++kx)
      if (BINST % NWT == 0 || wave + NWT * kx < BINST)
        dma_16x64_at(csrc, cc_off(wave + NWT * kx), lds_addr(cs) + (wave + NWT * kx) * 1024u);
#pragma unroll
    for (int kx = 0; kx < O::XINST_W; ++kx) dma_16x64_at(dsrc, cd_off(kx), lds_addr(ds[hh]) + (wv + 4 * kx) * 1024u);
  };

  // The piece's log-decays and the words holding its level weights
  // lambda[t, c + k] (lane t, one 4-byte word each; the element's parity
  // picks the half): wave 0 of each head.
  const int64_t t_lo = (int64_t)b * T_ + (int64_t)lo * C;
  const int64_t e0 = (t_lo * H + h) * L + lev;  // element of the piece's first token
  if (wv == 0) {
    const float* lsrc = pr.log_a + t_lo * H + h;
    const unsigned* wsrc = static_cast<const unsigned*>(pr.lam) + (e0 >> 1);
#pragma unroll
    for (int kx = 0; kx < BWD_PIECE; ++kx)
      if (kx < n) {
        dma_4x64_at(lsrc, (unsigned)((kx * C + lane) * H) * 4u, lds_addr(&las[hh][kx * C]));
        const unsigned wo = (unsigned)(((e0 & 1) + (int64_t)(kx * C + lane) * H * L) >> 1);
        dma_4x64_at(wsrc, wo * 4u, lds_addr(&lws[hh][kx * C]));
      }
  }
  // decays and weights of the chunk at position jp of the piece (wave 0)
  auto weights = [&](int jp, int par) __attribute__((always_inline)) {
    chunk_decays<bf16, C>(las[hh][jp * C + lane], cum[hh][par], ecum[hh][par], wst[hh][par], lane);
    const unsigned wd = lws[hh][jp * C + lane];
    const bool upper = ((e0 + (int64_t)(jp * C + lane) * H * L) & 1) != 0;
    const float lam = __uint_as_float(upper ? (wd & 0xffff0000u) : (wd << 16));
    wsh[hh][par][lane] = lam * ecum[hh][par][lane];
  };

  f32x4 S[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(hi - 1, csh0, dsh0);
  auto step = [&](auto cur_c, int s) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value;
    const int jp = n - 1 - s;  // position of this step's chunk in the piece
    const unsigned char* cs = CUR ? csh1 : csh0;
    const unsigned char* ds = CUR ? dsh1[hh] : dsh0[hh];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the chunk have landed
    if (s == 0 && wv == 0) weights(jp, 0);  // (later chunks' are formed a step ahead)
    lds_barrier();
    if (s + 1 < n)  // the other buffers were released by the previous barrier
      issue(lo + jp - 1, CUR ? csh0 : csh1, CUR ? dsh0 : dsh1);
    if (s > 0) {
      const float dec = M::ex(cum[hh][CUR][C - 1]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) S[nb] *= dec;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // dO rows scaled by the weights, split into hi and lo bf16 parts
      const unsigned char* px = ds + o_xt + 32 * kt * 128;
      const bf16x8 xt = cat8(lds_read8_tr(px), lds_read8_tr(px + 4 * 128));
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wsh[hh][CUR][32 * kt + 8 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wsh[hh][CUR][32 * kt + 8 * g + 4]);
      bf16x8 vh, vl;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float v0 = (float)xt[jj] * w0[jj], v1 = (float)xt[jj + 4] * w1[jj];
        vh[jj] = (bf16)v0;
        vh[jj + 4] = (bf16)v1;
        vl[jj] = (bf16)(v0 - (float)vh[jj]);
        vl[jj + 4] = (bf16)(v1 - (float)vh[jj + 4]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const unsigned char* pb = cs + o_bt + 32 * kt * BROW + 32 * nb;
        const bf16x8 af = cat8(lds_read8_tr(pb), lds_read8_tr(pb + 4 * BROW));
        S[nb] = M::mma(af, vh, S[nb]);
        S[nb] = M::mma(af, vl, S[nb]);
      }
    }
    if (s + 1 < n && wv == 0) weights(jp - 1, CUR ^ 1);
    lds_barrier();
  };
  for (int s = 0; s < n; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < n) step(std::integral_constant<int, 1>{}, s + 1);
  }
  if (bwd_pieces(k) == 1) {  // the level's state itself, through LDS (the last barrier freed it)
    float* dst = pr.rst + ((int64_t)bh * pr.nstate + bwd_state_index(pr.nc, k, pair)) * (N * P);
    bf16* hl = reinterpret_cast<bf16*>(hh ? &dsh0[0][0] : csh0);
    bf16* ll = reinterpret_cast<bf16*>(hh ? &dsh1[0][0] : csh1);
    state_tiles_to_lds<N, P, NB>(hl, ll, S, 16 * wv, g, r);
    lds_barrier();
    state_lds_out<N, P, 256>(dst, hl, ll, 64 * wv + lane);
  } else {  // an fp32 partial for the reduce
    float* dst = pr.part_r + ((int64_t)bh * pr.npart + blockIdx.x) * (N * P);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * nb + 4 * g + i) * P + 16 * wv + r] = S[nb][i];
  }
}

// Forward-direction level states (key B, value X) without re-reading the
// token rows per level.  The lower half of chunk level k at pair p is the
// aligned block of 2^(k-1) chunks starting at chunk p 2^k, summed decayed to
// its end; such blocks nest, so one walk over the chunks builds all of them:
// after chunk c the aligned blocks of 2^e chunks ending at c are complete
// for e up to the trailing ones of c (the Fenwick rule), a completed block
// whose bit e is 0 is the lower half of level e + 1 (stored when its upper
// half exists) and waits for its right sibling, and the sibling folds it in
// decayed by its own total log-decay.
//
// grid (ceil(nc / 8), batch*nheads): the blocks inside one aligned group of
// 8 chunks (levels 1 to 4), from the group's chunk states; the totals of
// the full groups go to part_f for bwd_zst_up_kernel when there are levels
// above 4.
template <class T, int C, int P, int N>
__global__ __launch_bounds__((Tiles<T, C, P, N>::NT)) void bwd_zst_group_kernel(BwdParams pr) {
  using Tl = Tiles<T, C, P, N>;
  constexpr int NT = Tl::NT, NB = Tl::NB;
  static_assert(Tl::KC == C, "token tiles are not padded here");
  __shared__ __attribute__((aligned(16))) T ksh[C * N];
  __shared__ __attribute__((aligned(16))) T vsh[C * P];
  __shared__ __attribute__((aligned(16))) float cum[64], ecum[64], wst[64];
  // a level state on its way out (bf16 io: its two planes)
  __shared__ __attribute__((aligned(16))) bf16 zs_hi[sizeof(T) == 2 ? N * P : 8], zs_lo[sizeof(T) == 2 ? N * P : 8];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, H = pr.nheads, G = pr.ngroups;
  const int b = bh / H, h = bh % H, grp = h / (H / G);
  const int64_t T_ = pr.seqlen;
  const int g8 = blockIdx.x, c0 = 8 * g8, c1 = min(c0 + 8, pr.nc);
  const double* ca = pr.cuma + (int64_t)bh * (pr.nc + 1);
  float* zst = pr.zst + (int64_t)bh * pr.nstate * (N * P);
  // a level state (uniform call: a barrier inside; at most one per chunk, and
  // the loop's barriers separate one from the next)
  auto put = [&](float* dst, const f32x4* S) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
      state_tiles_to_lds<N, P, NB>(zs_hi, zs_lo, S, 16 * wave, g, r);
      lds_barrier();
      state_lds_out<N, P, NT>(dst, zs_hi, zs_lo, tid);
    } else {
      state_put_tiles<T, N, P, NB>(dst, S, 16 * wave, g, r);
    }
  };
  auto put_f32 = [&](float* dst, const f32x4* S) __attribute__((always_inline)) {  // a group total
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * nb + 4 * g + i) * P + 16 * wave + r] = S[nb][i];
  };
  RowsStage<T, C, N, NT> sk;
  RowsStage<T, C, P, NT> sv;
  float la_n = 0.f;  // next chunk's log a for this thread's token
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)j * C;
    sk.load(static_cast<const T*>(pr.Bm) + (((int64_t)b * T_ + t0) * G + grp) * N, (int64_t)G * N, tid);
    sv.load(static_cast<const T*>(pr.X) + (((int64_t)b * T_ + t0) * H + h) * P, (int64_t)H * P, tid);
    la_n = pr.log_a[((int64_t)b * T_ + t0 + (tid < C ? tid : 0)) * H + h];
  };
  f32x4 stk[3][NB];  // left blocks of 1, 2 and 4 chunks waiting for their siblings
  issue(c0);
  for (int c = c0; c < c1; ++c) {
    sk.store(ksh, tid);
    sv.store(vsh, tid);
    const float la = tid < C ? la_n : 0.f;
    if (c + 1 < c1) issue(c + 1);
    chunk_decays<T, C>(la, cum, ecum, wst, tid);
    lds_barrier();
    f32x4 cur[NB];  // this chunk's state, decayed to its end
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) cur[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    chunk_state_mma_split<T, C, P, N>(ksh, vsh, wst, cur, wave, g, r);
    lds_barrier();  // the next chunk restages the tiles
    const int i = c - c0;
    bool open = true;  // uniform
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!open) continue;
      if (e == 3) {  // the whole group (i = 7): lower half of level 4 when even
        if (pr.kc >= 5) put_f32(pr.part_f + ((int64_t)bh * ((pr.nc + 7) >> 3) + g8) * (N * P), cur);
        if (!(g8 & 1) && (g8 >> 1) < bwd_pairs(pr.nc, 4))
          put(zst + (int64_t)bwd_state_index(pr.nc, 4, g8 >> 1) * (N * P), cur);
        open = false;
      } else if (!((i >> e) & 1)) {  // a left block: lower half of level e + 1
        const int k = e + 1, pair = c >> k;
        if (pair < bwd_pairs(pr.nc, k)) put(zst + (int64_t)bwd_state_index(pr.nc, k, pair) * (N * P), cur);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) stk[e][nb] = cur[nb];
        open = false;
      } else {  // a right block: its left sibling, decayed across it, folds in
        const float dec = __expf((float)(ca[c + 1] - ca[c + 1 - (1 << e)]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) cur[nb] = dec * stk[e][nb] + cur[nb];
      }
    }
  }
}

// grid (N P / 1024, batch*nheads), 256 threads: the lower halves of chunk
// levels 5 and up, by the same walk over the full groups' totals (a block
// of 2^z groups completed at group q is the lower half of level z + 4).
// Each thread owns four consecutive state elements of every block; the
// totals of 16 groups are loaded at a time.
constexpr int BWD_UP_DEPTH = 24;  // group levels: chunk levels up to 27
template <class T, int P, int N>
__global__ __launch_bounds__(256) void bwd_zst_up_kernel(BwdParams pr) {
  constexpr int D = BWD_UP_DEPTH, U = 16;
  const int bh = blockIdx.y;
  const int e4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e4 >= N * P) return;
  const int ng = pr.nc >> 3;  // full groups
  const float* gt = pr.part_f + (int64_t)bh * ((pr.nc + 7) >> 3) * (N * P) + e4;
  const double* ca = pr.cuma + (int64_t)bh * (pr.nc + 1);
  float* zst = pr.zst + (int64_t)bh * pr.nstate * (N * P);
  f32x4 stk[D];
#pragma unroll
  for (int e = 0; e < D; ++e) stk[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < ng; q0 += U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const f32x4*>(gt + (int64_t)min(q0 + u, ng - 1) * (N * P));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u;
      if (q >= ng) break;  // uniform
      const int z = __builtin_ctz(~(unsigned)q);  // trailing ones of q
      f32x4 cur = v[u];
      // Unrolled into uniform branches, one per entry, so that every stack
      // index is a constant and the stack stays in registers.
#pragma unroll
      for (int e = 0; e < D; ++e)
        if (e < z) cur = __expf((float)(ca[8 * (q + 1)] - ca[8 * (q + 1 - (1 << e))])) * stk[e] + cur;
      const int k = z + 4, pair = (8 * (q + 1 - (1 << z))) >> k;
      if (z >= 1 && k <= pr.kc && pair < bwd_pairs(pr.nc, k))
        state_put4<T, N, P>(zst + (int64_t)bwd_state_index(pr.nc, k, pair) * (N * P), e4, cur);
#pragma unroll
      for (int e = 0; e < D; ++e)
        if (e == z) stk[e] = cur;
    }
  }
}

// ------------------------------------------------------------ launch 3

// grid (nstate, batch*nheads), 256 threads.  Combines the pieces of one
// half: forward, each piece decayed from its end to the end of the half
// (pieces from last to first); reverse, from the start of the half to the
// piece's start (pieces in order).  Writes the fp32 state, row-major [N][P].
template <class T, int P, int N, bool REV>
__global__ __launch_bounds__(256) void bwd_level_reduce_kernel(BwdParams pr) {
  static_assert(REV, "forward-direction states come from the block walk, not from pieces");
  constexpr int Q4 = N * P / 4;              // float4 groups of a state
  constexpr int EPT = (Q4 + 255) / 256;      // per thread
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int sidx = pr.nstate_direct + blockIdx.x;  // only levels with several pieces
  int k, pair;
  bwd_state_of(sidx, pr.nc, pr.kc, k, pair);
  const int half = 1 << (k - 1);
  const int base = pair * 2 * half + (REV ? half : 0);
  const int np = bwd_pieces(k);
  const int pbase = bwd_piece_base(pr.nc, k) + pair * np;
  const float* at = pr.atot + (int64_t)bh * pr.nc;
  const float* part = (REV ? pr.part_r : pr.part_f) + ((int64_t)bh * pr.npart + pbase) * (N * P);
  f32x4 acc[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  float run = 0.f;  // log-decay between the piece and the reference point
  for (int s = 0; s < np; ++s) {
    const int pcs = REV ? s : np - 1 - s;
    const int clo = base + pcs * BWD_PIECE;
    if (clo >= pr.nc) break;  // uniform: pieces past the sequence hold nothing and are not written
    const int chi = min(min(clo + BWD_PIECE, base + half), pr.nc);
    const float w = Mfma<T>::ex(run);
#pragma unroll
    for (int q = 0; q < EPT; ++q)
      if (q * 256 + tid < Q4)
        acc[q] += w * *reinterpret_cast<const f32x4*>(part + (int64_t)pcs * (N * P) + (q * 256 + tid) * 4);
    float pt = 0.f;  // the piece's total log-decay (uniform)
    for (int m = clo; m < chi; ++m) pt += at[m];
    run += pt;
  }
  float* dst = (REV ? pr.rst : pr.zst) + ((int64_t)bh * pr.nstate + sidx) * (N * P);
#pragma unroll
  for (int q = 0; q < EPT; ++q)
    if (q * 256 + tid < Q4) state_put4<T, N, P>(dst, (q * 256 + tid) * 4, acc[q]);
}

// ------------------------------------------------------------ launches 4, 5

// LDS bytes of the two chunk passes (the host only instantiates shapes that
// fit the 160 KB of a CU).
// Work split of the chunk passes' products with the state dimension (see
// bwd_dq_kernel).
template <class T, int C>
struct ChunkSplit {
  static constexpr int NWR = C / 16, NW = 2 * NWR;
  // 16-row blocks per wave (fp32 keeps one: its operands take four times the
  // registers per contraction step)
  static constexpr int RPW = (sizeof(T) == 2 && NWR >= 2) ? 2 : 1;
  static constexpr int NRG = NWR / RPW;         // row groups
  static constexpr int NCG = NW / NRG;          // column groups
};

template <class T, int C, int P, int N>
constexpr int bwd_dq_lds() {
  return (int)sizeof(T) * (2 * C * N + 2 * C * P + C * C + (sizeof(T) == 2 ? 2 : 1) * N * P) +
         4 * (C * (C + 1) + 2 * C * BWD_LMAX + 4 * 64 + BWD_LMAX + 2 * ChunkSplit<T, C>::NCG * 64);
}
template <class T, int C, int P, int N>
constexpr int bwd_dkv_lds() {
  return (int)sizeof(T) * (2 * C * N + 2 * C * P + 2 * C * C + (sizeof(T) == 2 ? 2 : 1) * N * P) +
         4 * (C * (C + 1) + C * 8 + (C / 8) * 64 + ChunkSplit<T, C>::NCG * 64 + 3 * 64 + BWD_LMAX);
}

// S = C B^T and D = dO X^T for the query rows [16 rb, +16) of the chunk,
// the tiles sb = half, half + 2, ... (tiles above the diagonal block are
// skipped), then the mask
// M[t, s] = exp(cum_t - cum_s) lambda[t, level(t, s)] for s <= t:
// wm = M ⊙ S (if WANT_WS), wd = M ⊙ D in the io type, and optionally
// E ⊙ S ⊙ D or G = M ⊙ S ⊙ D in fp32.
template <class T, int C, int P, int N, int LW, bool WANT_WS, bool WANT_ESD, bool WANT_G>
__device__ inline void bwd_intra_scores(const T* csh, const T* bsh, const T* xsh, const T* osh,
                                        const float* cum, const float (*lam_s)[LW], T* wm, T* wd,
                                        float (*esd)[C + 1], int rb, int half, int g, int r) {
  using M = Mfma<T>;
  using LN = Rows<T, N>;
  using LP = Rows<T, P>;
  using LC = Rows<T, C>;
  constexpr int KB = M::KB, TB = C / 16;
  const int tw = 16 * rb;
#pragma unroll
  for (int sb0 = 0; sb0 < TB; sb0 += 2) {
    const int sb = sb0 + half;  // the two waves of a row block take alternate tiles
    if (TB % 2 != 0 && sb >= TB) break;  // (never for an even tile count)
    f32x4 s4 = {0.f, 0.f, 0.f, 0.f}, d4 = {0.f, 0.f, 0.f, 0.f};
    if (sb <= rb) {
#pragma unroll
      for (int kk = 0; kk < N / KB; ++kk)
        s4 = M::mma(frag_along<T, LN>(csh, tw + r, kk * KB, g),
                    frag_along<T, LN>(bsh, 16 * sb + r, kk * KB, g), s4);
#pragma unroll
      for (int kk = 0; kk < P / KB; ++kk)
        d4 = M::mma(frag_along<T, LP>(osh, tw + r, kk * KB, g),
                    frag_along<T, LP>(xsh, 16 * sb + r, kk * KB, g), d4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tw + 4 * g + i, s = 16 * sb + r;
      float e = 0.f, m = 0.f;
      if (s <= t) {
        e = M::ex(cum[t] - cum[s]);
        m = e * lam_s[t][bit_length((unsigned)(t ^ s))];
      }
      if constexpr (WANT_WS) wm[LC::at(t, s)] = from_f<T>(m * s4[i]);
      wd[LC::at(t, s)] = from_f<T>(m * d4[i]);
      if constexpr (WANT_ESD) esd[t][s] = e * s4[i] * d4[i];
      if constexpr (WANT_G) esd[t][s] = m * s4[i] * d4[i];
    }
  }
}

// A level state (the form of state_put4) prefetched into registers, then
// stored to LDS as the hi and lo tiles the products read.
template <class T, int N, int P, int NT>
struct StateStage {
  using L = Rows<T, P>;
  static constexpr int PIECES = N * L::NBLK;  // 16-byte io-type pieces
  static constexpr int IT = (PIECES + NT - 1) / NT;
  static constexpr int F4 = L::VEC / 4;  // float4 per piece
  // bf16: the hi and lo pieces of the level state's two planes; fp32: the
  // values (see state_put4)
  f32x4 v[IT][F4];
  __device__ inline void load(const float* g, int tid) {  // unconditional: see RowsStage
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int i = PIECES % NT == 0 ? q * NT + tid : min(q * NT + tid, PIECES - 1);
      if constexpr (sizeof(T) == 2) {
        const bf16* hp = reinterpret_cast<const bf16*>(g) + (int64_t)i * L::VEC;
        v[q][0] = *reinterpret_cast<const f32x4*>(hp);
        v[q][1] = *reinterpret_cast<const f32x4*>(hp + N * P);
      } else {
        const float* src = g + (int64_t)(i / L::NBLK) * P + (i % L::NBLK) * L::VEC;
#pragma unroll
        for (int f = 0; f < F4; ++f) v[q][f] = *reinterpret_cast<const f32x4*>(src + 4 * f);
      }
    }
  }
  __device__ inline void store(T* hi, T* lo, int tid) const {
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int i = q * NT + tid;
      if (i < PIECES) {
        const int o = L::at(i / L::NBLK, (i % L::NBLK) * L::VEC);
        if constexpr (sizeof(T) == 2) {
          store16(hi + o, __builtin_bit_cast(bf16x8, v[q][0]));
          store16(lo + o, __builtin_bit_cast(bf16x8, v[q][1]));
        } else {
          store16(hi + o, v[q][0]);
        }
      }
    }
  }
};

// The thread index through an opaque move: values derived from it inside a
// persistent loop are recomputed per iteration instead of being hoisted out
// of the loop and held in registers across it.
__device__ inline int opaque_tid() {
  int v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"((int)threadIdx.x));
  return v;
}

// Chunk passes: persistent work-groups, as many as fit on the device at
// once (a multiple of 8).  The (batch*head, chunk) tiles are split into 8
// contiguous ranges, one per XCD (work-group b runs on XCD b mod 8).  At
// step m the L work-groups of an XCD take the range's tiles [m L, m L + L),
// work-group l the tile m L + (l + m) mod L: the ones running together work
// on neighbouring chunks of one head and share its level states in L2, and
// each work-group meets every chunk index residue mod L in turn (a chunk's
// level count depends on its index bits, so a fixed residue would load some
// work-groups far more than others).  Each work-group prefetches the next
// tile's token rows into registers while it computes the current one.
// Work items of the chunk passes: tiles (batch * group, chunk), each taken
// by one work-group for every head of the group in turn, so that the heads'
// dB and dC contributions add up in registers (no per-head shares and no
// group-sum pass; the order of the sum is fixed: head order).
struct BwdItem {
  int bh, j, b, h, grp, hi;
};
struct BwdItems {
  int hpg, nc, H, G;
  __device__ explicit BwdItems(const BwdParams& pr)
      : hpg(pr.nheads / pr.ngroups), nc(pr.nc), H(pr.nheads), G(pr.ngroups) {}
  __device__ BwdItem at(int item) const {
    BwdItem x;
    const int tile = item / hpg;
    x.hi = item - tile * hpg;
    const int bg = tile / nc;
    x.j = tile - bg * nc;
    x.b = bg / G;
    x.grp = bg - x.b * G;
    x.h = x.grp * hpg + x.hi;
    x.bh = x.b * H + x.h;
    return x;
  }
  // the work-group's item at step mi (its tile at step mi / hpg), or -1
  template <class CT>
  __device__ int item(const CT& ct, int mi) const {
    const int t = ct.tile(mi / hpg);
    return t < 0 ? -1 : t * hpg + mi % hpg;
  }
};

struct ChunkTiles {
  int base, end, L, l;
  __device__ explicit ChunkTiles(int total) {
    const int x = (int)(blockIdx.x & 7);
    const int per = (total + 7) >> 3;
    l = (int)(blockIdx.x >> 3);
    L = (int)(gridDim.x >> 3);
    base = x * per;
    end = min(total, base + per);
  }
  __device__ bool more(int m) const { return base + m * L < end; }  // step m exists
  __device__ int tile(int m) const {  // this work-group's tile at step m, or -1
    const int t = base + m * L + (l + m) % L;
    return t < end ? t : -1;
  }
};

// Two waves per 16-row block (C / 8 waves; two waves per SIMD hide more
// latency than one).  The score tiles go as in bwd_intra_scores.  The
// products with the state dimension (the intra dC product and every chunk
// level's) give each wave RPW = 2 adjacent 16-row blocks (1 for a 16-token
// chunk) and every NCG-th 16-column tile: a state fragment read from LDS
// then serves two row blocks, which halves the LDS reads of the level
// states against one row block per wave.  dC_t = sum_s (M ⊙ D)[t, s] B_s
// within the chunk plus, for each chunk level k whose bit is set in j,
// lambda[t, c+k] exp(decay) (Z_k dO_t) with Z_k the lower half's state;
// dlambda[t, l] = the level-l bucket sum of E S D inside the chunk, and
// exp(decay) C_t . (Z_k dO_t) at level c + k: each column group's share of
// the row sum is staged in LDS and the NCG shares are added in a fixed order.
// The next level's state is loaded into registers while the current one
// is used.
constexpr int bwd_chunk_threads(int C) { return C / 16 * 128; }
template <class T, int C, int P, int N>
__global__ __launch_bounds__(bwd_chunk_threads(C)) void bwd_dq_kernel(BwdParams pr) {
  using M = Mfma<T>;
  using LN = Rows<T, N>;
  using LP = Rows<T, P>;
  using LC = Rows<T, C>;
  using CS = ChunkSplit<T, C>;
  constexpr int NWR = CS::NWR, NW = CS::NW, NT = NW * 64, KB = M::KB, NB = N / 16;
  constexpr int RPW = CS::RPW, NRG = CS::NRG, NCG = CS::NCG;
  constexpr int NBW = (NB + NCG - 1) / NCG;  // column tiles per wave in the state products
  constexpr int c_log = ilog2c(C);
  __shared__ __attribute__((aligned(16))) T csh[C * N];
  __shared__ __attribute__((aligned(16))) T bsh[C * N];
  __shared__ __attribute__((aligned(16))) T xsh[C * P];
  __shared__ __attribute__((aligned(16))) T osh[C * P];
  __shared__ __attribute__((aligned(16))) T wsh[C * C];
  __shared__ __attribute__((aligned(16))) T zsh[N * P];
  __shared__ __attribute__((aligned(16))) T zlo[sizeof(T) == 2 ? N * P : 1];
  __shared__ float esd[C][C + 1];
  __shared__ float lam_s[C][BWD_LMAX];
  __shared__ float dlam_s[C][BWD_LMAX];
  __shared__ float red[2][NCG][64];  // a chunk level's row sums per column group (two levels in flight)
  __shared__ float cum[64], ecum[64], wst[64], term_s[64], gap_s[BWD_LMAX];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int half = wave >= NWR ? 1 : 0, rb = wave - half * NWR;
  const int rg = wave % NRG, cg = wave / NRG;  // state products: row group, column group
  const int H = pr.nheads, G = pr.ngroups, L = pr.nlevels;
  const int64_t T_ = pr.seqlen;
  const ChunkTiles ct(pr.batch * G * pr.nc);
  // lambda rows: every level the sequence reaches (ll <= BWD_LMAX), one
  // register per (row, level slot) of the BWD_LMAX-wide rows (NT = 8 C)
  constexpr int LIT = C * BWD_LMAX / NT;
  static_assert(C * BWD_LMAX % NT == 0, "whole rows of level slots per thread");
  const int ll = pr.ll;
  RowsStage<T, C, N, NT> sc, sb;
  RowsStage<T, C, P, NT> sx, so;
  T lv_[LIT];
  float la = 0.f;
  double ca_hi = 0.0, ca_lo = 0.0;
  const BwdItems it(pr);
  auto load_rows = [&](int item) {  // token rows of an item into registers
    const int tid = opaque_tid();
    const BwdItem x = it.at(item);
    const int bh = x.bh, j = x.j, b = x.b, h = x.h, grp = x.grp;
    const int64_t t0 = (int64_t)j * C;
    // the group's C and B rows (loaded for every head, a branch here would
    // make the compiler wait for them; staged only for the first)
    sc.load(static_cast<const T*>(pr.Cm) + (((int64_t)b * T_ + t0) * G + grp) * N, (int64_t)G * N, tid);
    sb.load(static_cast<const T*>(pr.Bm) + (((int64_t)b * T_ + t0) * G + grp) * N, (int64_t)G * N, tid);
    sx.load(static_cast<const T*>(pr.X) + (((int64_t)b * T_ + t0) * H + h) * P, (int64_t)H * P, tid);
    so.load(static_cast<const T*>(pr.dO) + (((int64_t)b * T_ + t0) * H + h) * P, (int64_t)H * P, tid);
    const T* lg = static_cast<const T*>(pr.lam) + (((int64_t)b * T_ + t0) * H + h) * L;
#pragma unroll
    for (int q = 0; q < LIT; ++q) {  // element i: row i / BWD_LMAX, level i mod BWD_LMAX
      const int i = q * NT + tid;
      const int l = min(i % BWD_LMAX, ll - 1);  // unconditional (see RowsStage): levels past ll repeat the last
      lv_[q] = lg[(int64_t)(i / BWD_LMAX) * H * L + l];
    }
    la = pr.log_a[((int64_t)b * T_ + t0 + min(tid, C - 1)) * H + h];
    // level k's gap (lane k - 1): log-decay from the end of the lower half
    // to chunk j, from the prefix sums at j and at the first chunk of j's
    // upper half at level k
    const double* ca = pr.cuma + (int64_t)bh * (pr.nc + 1);
    const int kl = tid < pr.kc ? tid : 0;
    ca_hi = ca[j];
    ca_lo = ca[(j >> kl) << kl];
  };
  f32x4 dc[RPW][NBW];  // row block RPW rg + rr, column tile cg + NCG q: summed over the group's heads
  if (it.item(ct, 0) >= 0) load_rows(it.item(ct, 0));
  for (int mi = 0; ct.more(mi / it.hpg); ++mi) {
  const int item = it.item(ct, mi), next = it.item(ct, mi + 1);
  if (item < 0) continue;  // uniform: the last step has fewer tiles than work-groups
  const int tid = opaque_tid(), lane = tid & 63, g = lane >> 4, r = lane & 15;
  const BwdItem x = it.at(item);
  const int bh = x.bh, j = x.j, b = x.b, h = x.h;
  const int64_t t0 = (int64_t)j * C;
  const unsigned act0 = (unsigned)j & ((1u << pr.kc) - 1u);  // active chunk levels (bit k-1)
  const float gap = tid < pr.kc && ((act0 >> tid) & 1u) ? (float)(ca_hi - ca_lo) : 0.f;

  if (x.hi == 0) {  // later heads of the group find the C and B rows in place
    sc.store(csh, tid);
    sb.store(bsh, tid);
  }
  sx.store(xsh, tid);
  so.store(osh, tid);
#pragma unroll
  for (int q = 0; q < LIT; ++q) {
    const int i = q * NT + tid, row = i / BWD_LMAX, l = i % BWD_LMAX;
    if (l < ll) {
      lam_s[row][l] = to_f(lv_[q]);
      dlam_s[row][l] = 0.f;
    }
  }
  if (tid < pr.kc) gap_s[tid + 1] = gap;
  chunk_decays<T, C>(tid < C ? la : 0.f, cum, ecum, wst, tid);
  lds_barrier();
  // the states of the first two active levels are requested now, each later
  // one two levels ahead of its use; then the next tile's rows
  StateStage<T, N, P, NT> st0, st1;  // two named buffers: no runtime array index
  auto state_of = [&](int kk) {
    return pr.zst + ((int64_t)bh * pr.nstate + bwd_state_index(pr.nc, kk, j >> kk)) * (N * P);
  };
  unsigned act = act0;
  int k = act ? __builtin_ctz(act) + 1 : 0;
  unsigned act2 = act ? act & (act - 1u) : 0u;
  const int k2 = act2 ? __builtin_ctz(act2) + 1 : 0;
  if (k) st0.load(state_of(k), tid);
  if (k2) st1.load(state_of(k2), tid);
  if (next >= 0) load_rows(next);

  bwd_intra_scores<T, C, P, N, BWD_LMAX, false, true, false>(csh, bsh, xsh, osh, cum, lam_s,
                                                             nullptr, wsh, esd, rb, half, g, r);
  lds_barrier();

  // intra-chunk levels: the level-l bucket of t (l >= 1) is the 2^(l-1) keys
  // below t's aligned 2^l block boundary, present when bit l-1 of t is set;
  // wave w sums the levels l = w mod NW.  Each level's loop has its length
  // fixed at compile time, so its LDS reads go out together (a loop of
  // runtime length waits for one read per key: 32 for the top level)
  static_for<0, c_log + 1>([&](auto lc) __attribute__((always_inline)) {
    constexpr int l = decltype(lc)::value;
    if (l % NW == wave && lane < C) {
      const int t = lane;
      float v = 0.f;
      if constexpr (l == 0) {
        v = esd[t][t];
      } else if ((t >> (l - 1)) & 1) {
        const int lo = t & ~((1 << l) - 1);
#pragma unroll
        for (int s = 0; s < (1 << (l - 1)); ++s) v += esd[t][lo + s];
      }
      dlam_s[t][l] = v;
    }
  });

  if (x.hi == 0) {  // the group's first head: its dC sum starts
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int q = 0; q < NBW; ++q) dc[rr][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kt = 0; kt < C / KB; ++kt) {  // keys s; entries with s > t are zero
    typename M::frag a[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) a[rr] = frag_along<T, LC>(wsh, 16 * (RPW * rg + rr) + r, kt * KB, g);
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int nb = cg + NCG * q;
      if (NB % NCG == 0 || nb < NB) {
        const auto bf = frag_down<T, LN>(bsh, kt * KB, 16 * nb, g, r);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) dc[rr][q] = M::mma(a[rr], bf, dc[rr][q]);
      }
    }
  }
  lds_barrier();  // dlam_s of the intra levels is written
  if (tid < C) {
    float tsum = 0.f;
    for (int l = 0; l <= c_log; ++l) tsum += lam_s[tid][l] * dlam_s[tid][l];
    term_s[tid] = tsum;
  }

  // operands every chunk level reuses: this wave's dO fragments, and its C
  // values at the positions of u's result tiles (for dlambda)
  typename M::frag ao[RPW][P / KB];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
    for (int kp = 0; kp < P / KB; ++kp) ao[rr][kp] = frag_along<T, LP>(osh, 16 * (RPW * rg + rr) + r, kp * KB, g);
  f32x4 cv[RPW][NBW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
    for (int q = 0; q < NBW; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cv[rr][q][i] = (NB % NCG == 0 || cg + NCG * q < NB)
                           ? to_f(csh[LN::at(16 * (RPW * rg + rr) + 4 * g + i, 16 * (cg + NCG * q) + r)])
                           : 0.f;
  // dlambda and dlog_a terms of a chunk level from its column groups' row sums
  auto finish_level = [&](int kk, int rbuf) {
    if (tid < C) {
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < NCG; ++c) sum += red[rbuf][c][tid];
      const int lv = c_log + kk;
      const float dl = M::ex(cum[tid] + gap_s[kk]) * sum;
      dlam_s[tid][lv] = dl;
      term_s[tid] += lam_s[tid][lv] * dl;
    }
  };

  int buf = 0, pk = 0;  // pk: the previous level, whose row sums wait in red[buf ^ 1]
  while (k) {
    if (buf == 0)  // uniform
      st0.store(zsh, zlo, tid);
    else
      st1.store(zsh, zlo, tid);
    if (pk) finish_level(pk, buf ^ 1);
    lds_barrier();
    act &= act - 1u;
    const int kn = act ? __builtin_ctz(act) + 1 : 0;
    const unsigned a3 = act ? act & (act - 1u) : 0u;
    const int k3 = a3 ? __builtin_ctz(a3) + 1 : 0;  // two levels ahead
    if (k3) {
      if (buf == 0)
        st0.load(state_of(k3), tid);
      else
        st1.load(state_of(k3), tid);
    }
    f32x4 u[RPW][NBW];  // u[t][n] = sum_p dO[t][p] Z[n][p]
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int q = 0; q < NBW; ++q) u[rr][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kp = 0; kp < P / KB; ++kp) {
#pragma unroll
      for (int q = 0; q < NBW; ++q) {
        const int nb = cg + NCG * q;
        if (NB % NCG == 0 || nb < NB) {
          const auto zh = frag_along<T, LP>(zsh, 16 * nb + r, kp * KB, g);
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) u[rr][q] = M::mma(ao[rr][kp], zh, u[rr][q]);
          if constexpr (sizeof(T) == 2) {
            const auto zl = frag_along<T, LP>(zlo, 16 * nb + r, kp * KB, g);
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr) u[rr][q] = M::mma(ao[rr][kp], zl, u[rr][q]);
          }
        }
      }
    }
    const int lv = c_log + k;
    const float egk = M::ex(gap_s[k]);  // e^(gap + Lambda_t) = e^gap e^(Lambda_t): one exponential per level
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int tw = 16 * (RPW * rg + rr);
      f32x4 part;  // this wave's share of C_t . u_t, per row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tw + 4 * g + i;
        const float wt = ecum[t] * egk;
        float pt = 0.f;
#pragma unroll
        for (int q = 0; q < NBW; ++q)
          if (NB % NCG == 0 || cg + NCG * q < NB) pt += u[rr][q][i] * cv[rr][q][i];
        part[i] = pt;
        const float lk = lam_s[t][lv];
#pragma unroll
        for (int q = 0; q < NBW; ++q) dc[rr][q][i] += (lk * wt) * u[rr][q][i];
      }
      // lanes r < 4 of lane group g hold the row sums of t = tw + 4 g +
      // [0, 2, 1, 3][r]: this column group's share
      const float rs = sum16x4(part, r);
      if (r < 4) red[buf][cg][tw + 4 * g + (((r & 1) << 1) | (r >> 1))] = rs;
    }
    lds_barrier();  // zsh is restaged by the next level; red[buf] is complete
    pk = k;
    k = kn;
    buf ^= 1;
  }
  if (pk) finish_level(pk, buf ^ 1);

  // after the group's last head: the dC tile through LDS (csh: every wave
  // is done with the C rows), then out by rows
  const bool last = x.hi == it.hpg - 1;  // uniform
  lds_barrier();
  if (last) {
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int q = 0; q < NBW; ++q)
        if (NB % NCG == 0 || cg + NCG * q < NB) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            csh[LN::at(16 * (RPW * rg + rr) + 4 * g + i, 16 * (cg + NCG * q) + r)] = from_f<T>(dc[rr][q][i]);
        }
  }
  lds_barrier();  // dlam_s and the dC tile are complete
  if (last)
    rows_from_lds<T, C, N, NT>(csh, static_cast<T*>(pr.dC) + (((int64_t)b * T_ + t0) * G + x.grp) * N,
                               (int64_t)G * N, tid);
  dlam_rows_out<T, C, BWD_LMAX, NT>(dlam_s, static_cast<T*>(pr.dlam) + (((int64_t)b * T_ + t0) * H + h) * L, H,
                                    L, pr.ll, tid);
  if (tid < C) pr.term1[(int64_t)bh * T_ + t0 + tid] = term_s[tid];
  lds_barrier();  // the next tile restages every LDS array
  }
}

// The mask epilogue runs per query row block as in bwd_dq_kernel; then, as
// there, each wave takes RPW adjacent 16-row blocks of keys and every
// NCG-th 16-column tile of P and of N (a level-state fragment read from LDS
// serves both row blocks): dX_s = sum_t (M ⊙ S)[t, s] dO_t and
// dB_s = sum_t (M ⊙ D)[t, s] C_t within the chunk, plus, for each chunk level
// k whose bit is clear in i and whose upper half exists,
// exp(decay s -> end of the lower half) (R_k^T B_s, R_k X_s) with R_k the
// upper half's state (lambda already on its tokens).
template <class T, int C, int P, int N>
__global__ __launch_bounds__(bwd_chunk_threads(C)) void bwd_dkv_kernel(BwdParams pr) {
  using M = Mfma<T>;
  using LN = Rows<T, N>;
  using LP = Rows<T, P>;
  using LC = Rows<T, C>;
  using CS = ChunkSplit<T, C>;
  constexpr int NWR = CS::NWR, NW = CS::NW, NT = NW * 64, KB = M::KB, NB = N / 16, PB = P / 16;
  constexpr int RPW = CS::RPW, NRG = CS::NRG, NCG = CS::NCG;
  constexpr int NBW = (NB + NCG - 1) / NCG, PBW = (PB + NCG - 1) / NCG;  // column tiles per wave
  constexpr int c_log = ilog2c(C);
  __shared__ __attribute__((aligned(16))) T csh[C * N];
  __shared__ __attribute__((aligned(16))) T bsh[C * N];
  __shared__ __attribute__((aligned(16))) T xsh[C * P];
  __shared__ __attribute__((aligned(16))) T osh[C * P];
  __shared__ __attribute__((aligned(16))) T wsh[C * C];
  __shared__ __attribute__((aligned(16))) T vsh[C * C];
  __shared__ __attribute__((aligned(16))) T rsh[N * P];
  __shared__ __attribute__((aligned(16))) T rlo[sizeof(T) == 2 ? N * P : 1];
  __shared__ float gsh[C][C + 1];
  __shared__ float lam_s[C][8];
  __shared__ float colpart[NW][64];
  __shared__ float xpart[NCG][64];  // X_s . (chunk-level dX_s), per column group
  __shared__ float cum[64], ecum[64], wst[64], gap_s[BWD_LMAX];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int half = wave >= NWR ? 1 : 0, rb = wave - half * NWR;
  const int rg = wave % NRG, cg = wave / NRG;  // state products: row group, column group
  const int H = pr.nheads, G = pr.ngroups, L = pr.nlevels;
  const int64_t T_ = pr.seqlen;
  const ChunkTiles ct(pr.batch * G * pr.nc);
  constexpr int LIT = (C * (c_log + 1) + NT - 1) / NT;
  RowsStage<T, C, N, NT> sc, sb;
  RowsStage<T, C, P, NT> sx, so;
  T lv_[LIT];
  float la = 0.f;
  double ca_hi = 0.0, ca_lo = 0.0;
  const BwdItems it(pr);
  auto load_rows = [&](int item) {  // token rows of an item into registers
    const int tid = opaque_tid();
    const BwdItem x = it.at(item);
    const int bh = x.bh, ich = x.j, b = x.b, h = x.h, grp = x.grp;
    const int64_t t0 = (int64_t)ich * C;
    // the group's C and B rows (loaded for every head, a branch here would
    // make the compiler wait for them; staged only for the first)
    sc.load(static_cast<const T*>(pr.Cm) + (((int64_t)b * T_ + t0) * G + grp) * N, (int64_t)G * N, tid);
    sb.load(static_cast<const T*>(pr.Bm) + (((int64_t)b * T_ + t0) * G + grp) * N, (int64_t)G * N, tid);
    sx.load(static_cast<const T*>(pr.X) + (((int64_t)b * T_ + t0) * H + h) * P, (int64_t)H * P, tid);
    so.load(static_cast<const T*>(pr.dO) + (((int64_t)b * T_ + t0) * H + h) * P, (int64_t)H * P, tid);
    const T* lg = static_cast<const T*>(pr.lam) + (((int64_t)b * T_ + t0) * H + h) * L;
#pragma unroll
    for (int q = 0; q < LIT; ++q) {
      const int i = q * NT + tid;
      const int ic = min(i, C * (c_log + 1) - 1);  // unconditional (see RowsStage)
      lv_[q] = lg[(int64_t)(ic / (c_log + 1)) * H * L + ic % (c_log + 1)];
    }
    la = pr.log_a[((int64_t)b * T_ + t0 + min(tid, C - 1)) * H + h];
    // level k's gap (lane k - 1): log-decay from the end of chunk i to the
    // end of its lower half, from the prefix sums at the first chunk of the
    // upper half at level k (clamped for lanes whose level is inactive) and
    // after chunk i
    const double* ca = pr.cuma + (int64_t)bh * (pr.nc + 1);
    const int kl = tid < pr.kc ? tid : 0;
    ca_hi = ca[min(((ich >> kl) + 1) << kl, pr.nc)];
    ca_lo = ca[ich + 1];
  };
  f32x4 db[RPW][NBW];  // dB of the chunk, summed over the group's heads
  if (it.item(ct, 0) >= 0) load_rows(it.item(ct, 0));
  for (int mi = 0; ct.more(mi / it.hpg); ++mi) {
  const int item = it.item(ct, mi), next = it.item(ct, mi + 1);
  if (item < 0) continue;  // uniform: the last step has fewer tiles than work-groups
  const int tid = opaque_tid(), lane = tid & 63, g = lane >> 4, r = lane & 15;
  const BwdItem x = it.at(item);
  const int bh = x.bh, i_ch = x.j, b = x.b, h = x.h;
  const int64_t t0 = (int64_t)i_ch * C;
  // active chunk levels (bit k-1): i in a lower half whose upper half exists
  unsigned act0 = 0;
  for (int k = 1; k <= pr.kc; ++k)
    if (!((i_ch >> (k - 1)) & 1) && ((((i_ch >> (k - 1)) + 1) << (k - 1)) < pr.nc)) act0 |= 1u << (k - 1);
  const float gap = tid < pr.kc && ((act0 >> tid) & 1u) ? (float)(ca_hi - ca_lo) : 0.f;

  if (x.hi == 0) {  // later heads of the group find the C and B rows in place
    sc.store(csh, tid);
    sb.store(bsh, tid);
  }
  sx.store(xsh, tid);
  so.store(osh, tid);
#pragma unroll
  for (int q = 0; q < LIT; ++q) {
    const int i = q * NT + tid;
    if (i < C * (c_log + 1)) lam_s[i / (c_log + 1)][i % (c_log + 1)] = to_f(lv_[q]);
  }
  if (tid < pr.kc) gap_s[tid + 1] = gap;
  chunk_decays<T, C>(tid < C ? la : 0.f, cum, ecum, wst, tid);
  lds_barrier();
  // the states of the first two active levels are requested now, each later
  // one two levels ahead of its use; then the next tile's rows
  StateStage<T, N, P, NT> st0, st1;  // two named buffers: no runtime array index
  auto state_of = [&](int kk) {
    return pr.rst + ((int64_t)bh * pr.nstate + bwd_state_index(pr.nc, kk, i_ch >> kk)) * (N * P);
  };
  unsigned act = act0;
  int k = act ? __builtin_ctz(act) + 1 : 0;
  unsigned act2 = act ? act & (act - 1u) : 0u;
  const int k2 = act2 ? __builtin_ctz(act2) + 1 : 0;
  if (k) st0.load(state_of(k), tid);
  if (k2) st1.load(state_of(k2), tid);
  if (next >= 0) load_rows(next);

  bwd_intra_scores<T, C, P, N, 8, true, false, true>(csh, bsh, xsh, osh, cum, lam_s, wsh, vsh,
                                                     gsh, rb, half, g, r);
  lds_barrier();
  // X_s . dX_s within the chunk is the column sum of G: taken in fp32 from
  // the same entries whose row sums form dO_t . O_t, so that the two terms of
  // dlog_a agree where they overlap (the rounding of M ⊙ S to the io type for
  // the dX product would otherwise enter one term and not the other).  Wave w
  // sums the rows t = w mod NW.
  if (lane < C) {  // rows in a loop of fixed length: the reads go out together
    float cs = 0.f;
#pragma unroll
    for (int i = 0; i < (C + NW - 1) / NW; ++i) {
      const int t = wave + i * NW;
      if (t >= lane && t < C) cs += gsh[t][lane];
    }
    colpart[wave][lane] = cs;
  }

  // dX: intra-chunk part, chunk-level part; dB (row block RPW rg + rr,
  // column tile cg + NCG q of P or of N)
  f32x4 dx[RPW][PBW], dxe[RPW][PBW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
#pragma unroll
    for (int q = 0; q < PBW; ++q) dx[rr][q] = dxe[rr][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (x.hi == 0) {  // the group's first head: its dB sum starts
#pragma unroll
      for (int q = 0; q < NBW; ++q) db[rr][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int kt = 0; kt < C / KB; ++kt) {  // queries t; entries with t < s are zero
    typename M::frag aw[RPW], av[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      aw[rr] = frag_down<T, LC>(wsh, kt * KB, 16 * (RPW * rg + rr), g, r);
      av[rr] = frag_down<T, LC>(vsh, kt * KB, 16 * (RPW * rg + rr), g, r);
    }
#pragma unroll
    for (int q = 0; q < PBW; ++q)
      if (PB % NCG == 0 || cg + NCG * q < PB) {
        const auto bo = frag_down<T, LP>(osh, kt * KB, 16 * (cg + NCG * q), g, r);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) dx[rr][q] = M::mma(aw[rr], bo, dx[rr][q]);
      }
#pragma unroll
    for (int q = 0; q < NBW; ++q)
      if (NB % NCG == 0 || cg + NCG * q < NB) {
        const auto bc = frag_down<T, LN>(csh, kt * KB, 16 * (cg + NCG * q), g, r);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) db[rr][q] = M::mma(av[rr], bc, db[rr][q]);
      }
  }

  // this wave's B and X row fragments, the A operands of every chunk level
  // (B's for bf16 only: fp32 fragments hold one element each, and N / 4 of
  // them per row block would not fit in registers)
  constexpr bool HOLD_B = sizeof(T) == 2;
  typename M::frag abf[RPW][HOLD_B ? N / KB : 1], axf[RPW][P / KB];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    if constexpr (HOLD_B) {
#pragma unroll
      for (int kn2 = 0; kn2 < N / KB; ++kn2)
        abf[rr][kn2] = frag_along<T, LN>(bsh, 16 * (RPW * rg + rr) + r, kn2 * KB, g);
    }
#pragma unroll
    for (int kp = 0; kp < P / KB; ++kp) axf[rr][kp] = frag_along<T, LP>(xsh, 16 * (RPW * rg + rr) + r, kp * KB, g);
  }

  int buf = 0;
  while (k) {
    if (buf == 0)  // uniform
      st0.store(rsh, rlo, tid);
    else
      st1.store(rsh, rlo, tid);
    lds_barrier();
    act &= act - 1u;
    const int kn = act ? __builtin_ctz(act) + 1 : 0;
    const unsigned a3 = act ? act & (act - 1u) : 0u;
    const int k3 = a3 ? __builtin_ctz(a3) + 1 : 0;  // two levels ahead
    if (k3) {
      if (buf == 0)
        st0.load(state_of(k3), tid);
      else
        st1.load(state_of(k3), tid);
    }
    f32x4 tx[RPW][PBW], tb[RPW][NBW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
#pragma unroll
      for (int q = 0; q < PBW; ++q) tx[rr][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < NBW; ++q) tb[rr][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kn2 = 0; kn2 < N / KB; ++kn2) {  // tx[s][p] = sum_n B[s][n] R[n][p]
      typename M::frag ab[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr)
        ab[rr] = HOLD_B ? abf[rr][HOLD_B ? kn2 : 0] : frag_along<T, LN>(bsh, 16 * (RPW * rg + rr) + r, kn2 * KB, g);
#pragma unroll
      for (int q = 0; q < PBW; ++q) {
        const int pb = cg + NCG * q;
        if (PB % NCG == 0 || pb < PB) {
          const auto rh = frag_down<T, LP>(rsh, kn2 * KB, 16 * pb, g, r);
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) tx[rr][q] = M::mma(ab[rr], rh, tx[rr][q]);
          if constexpr (sizeof(T) == 2) {
            const auto rl = frag_down<T, LP>(rlo, kn2 * KB, 16 * pb, g, r);
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr) tx[rr][q] = M::mma(ab[rr], rl, tx[rr][q]);
          }
        }
      }
    }
#pragma unroll
    for (int kp = 0; kp < P / KB; ++kp) {  // tb[s][n] = sum_p X[s][p] R[n][p]
#pragma unroll
      for (int q = 0; q < NBW; ++q) {
        const int nb = cg + NCG * q;
        if (NB % NCG == 0 || nb < NB) {
          const auto rh = frag_along<T, LP>(rsh, 16 * nb + r, kp * KB, g);
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) tb[rr][q] = M::mma(axf[rr][kp], rh, tb[rr][q]);
          if constexpr (sizeof(T) == 2) {
            const auto rl = frag_along<T, LP>(rlo, 16 * nb + r, kp * KB, g);
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr) tb[rr][q] = M::mma(axf[rr][kp], rl, tb[rr][q]);
          }
        }
      }
    }
    const float egk = M::ex(gap_s[k]);  // e^(decay s -> chunk end + gap) as a product: one exponential per level
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * (RPW * rg + rr) + 4 * g + i;
        const float w = wst[s] * egk;
#pragma unroll
        for (int q = 0; q < PBW; ++q) dxe[rr][q][i] += w * tx[rr][q][i];
#pragma unroll
        for (int q = 0; q < NBW; ++q) db[rr][q][i] += w * tb[rr][q][i];
      }
    lds_barrier();  // rsh is restaged by the next level
    k = kn;
    buf ^= 1;
  }
  // the dX tile and, after the group's last head, the dB tile through LDS
  // (osh and csh: every wave is done with the dO and C rows), then out by rows
  const bool last = x.hi == it.hpg - 1;  // uniform
  lds_barrier();
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int sw = 16 * (RPW * rg + rr);
    f32x4 part;  // X_s . (chunk-level part of dX_s), this wave's columns
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = sw + 4 * g + i;
      float pt = 0.f;
#pragma unroll
      for (int q = 0; q < PBW; ++q) {
        const int pb = cg + NCG * q;
        if (PB % NCG == 0 || pb < PB) {
          pt += dxe[rr][q][i] * to_f(xsh[LP::at(s, 16 * pb + r)]);
          osh[LP::at(s, 16 * pb + r)] = from_f<T>(dx[rr][q][i] + dxe[rr][q][i]);
        }
      }
      part[i] = pt;
      if (last) {
#pragma unroll
        for (int q = 0; q < NBW; ++q)
          if (NB % NCG == 0 || cg + NCG * q < NB) csh[LN::at(s, 16 * (cg + NCG * q) + r)] = from_f<T>(db[rr][q][i]);
      }
    }
    // lanes r < 4 of lane group g hold the row sums of s = sw + 4 g + [0, 2, 1, 3][r]
    const float rs = sum16x4(part, r);
    if (r < 4) xpart[cg][sw + 4 * g + (((r & 1) << 1) | (r >> 1))] = rs;
  }
  lds_barrier();  // colpart, xpart and the dX and dB tiles are complete
  rows_from_lds<T, C, P, NT>(osh, static_cast<T*>(pr.dX) + (((int64_t)b * T_ + t0) * H + h) * P, (int64_t)H * P,
                             tid);
  if (last)
    rows_from_lds<T, C, N, NT>(csh, static_cast<T*>(pr.dB) + (((int64_t)b * T_ + t0) * G + x.grp) * N,
                               (int64_t)G * N, tid);
  if (tid < C) {
    float cs = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) cs += colpart[w][tid];
    float xs = 0.f;
#pragma unroll
    for (int c = 0; c < NCG; ++c) xs += xpart[c][tid];
    pr.term2[(int64_t)bh * T_ + t0 + tid] = cs + xs;
  }
  lds_barrier();  // the next tile restages every LDS array
  }
}

// ------------------------------------------------------------ launch 6

// dlog_a[t] = sum_{t' >= t} (term1 - term2), in fp64, over segments of
// whole 1024-token blocks (at most DLOGA_SEGS per (batch, head)): first each
// segment's total, then per segment the sum of the later segments' totals
// and a suffix scan of the segment, block by block from its end.  Token
// reads are coalesced; the totals reuse the chunk passes' prefix-sum region
// (nc + 1 doubles per head, at least the segment count: free by now).
constexpr int DLOGA_SEGS = 64;
__host__ __device__ inline int dloga_nseg(int64_t T) {
  const int64_t n = (T + 4095) / 4096;
  return (int)(n < DLOGA_SEGS ? n : DLOGA_SEGS);
}
__device__ inline int64_t dloga_segt(int64_t T, int nseg) {
  return ((T + nseg - 1) / nseg + BWD_SCAN_NT - 1) / BWD_SCAN_NT * BWD_SCAN_NT;
}

// grid (nseg, batch*nheads), 256 threads: segment totals.
template <class T>  // (a template so that every unit's copy is a weak symbol)
__global__ __launch_bounds__(256) void bwd_dloga_part_kernel(BwdParams pr) {
  __shared__ double wsum[4];
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int64_t T_ = pr.seqlen;
  const int nseg = gridDim.x;
  const int64_t segt = dloga_segt(T_, nseg);
  const int64_t lo = (int64_t)s * segt, hi = min(lo + segt, T_);
  const float* t1 = pr.term1 + (int64_t)bh * T_;
  const float* t2 = pr.term2 + (int64_t)bh * T_;
  double acc = 0.0;
  for (int64_t t = lo + tid; t < hi; t += 256) acc += (double)t1[t] - (double)t2[t];
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) pr.cuma[(int64_t)bh * nseg + s] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// grid (nseg, batch*nheads), 1024 threads: one segment's suffix sums.
template <class T>
__global__ __launch_bounds__(BWD_SCAN_NT) void bwd_dloga_kernel(BwdParams pr) {
  constexpr int NT = BWD_SCAN_NT, NWV = NT / 64;
  __shared__ double wsum[2][NWV];  // wave totals of a block, by block parity
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = pr.nheads, b = bh / H, h = bh % H;
  const int64_t T_ = pr.seqlen;
  const int nseg = gridDim.x;
  const int64_t segt = dloga_segt(T_, nseg);
  const int64_t lo = (int64_t)s * segt, hi = min(lo + segt, T_);
  const float* t1 = pr.term1 + (int64_t)bh * T_;
  const float* t2 = pr.term2 + (int64_t)bh * T_;
  double carry = 0.0;  // the later segments, then the later blocks
  for (int s2 = nseg - 1; s2 > s; --s2) carry += pr.cuma[(int64_t)bh * nseg + s2];
  const int64_t nblk = hi > lo ? (hi - lo + NT - 1) / NT : 0;
  float a1 = 0.f, a2 = 0.f;  // this thread's token of the next block (clamped: no branch)
  auto ld = [&](int64_t blk) __attribute__((always_inline)) {
    const int64_t t = min(lo + blk * NT + tid, hi - 1);
    a1 = t1[t];
    a2 = t2[t];
  };
  if (nblk > 0) ld(nblk - 1);
  for (int64_t blk = nblk - 1, it = 0; blk >= 0; --blk, ++it) {
    const int64_t t = lo + blk * NT + tid;
    double v = t < hi ? (double)a1 - (double)a2 : 0.0;
    if (blk > 0) ld(blk - 1);
    for (int d = 1; d < 64; d <<= 1) {  // inclusive suffix sums within the wave
      const double o = __shfl_down(v, d, 64);
      if (lane + d < 64) v += o;
    }
    if (lane == 0) wsum[it & 1][w] = v;
    __syncthreads();
    double after = carry, total = carry;
#pragma unroll
    for (int w2 = 0; w2 < NWV; ++w2) {
      const double x = wsum[it & 1][w2];
      total += x;
      if (w2 > w) after += x;
    }
    if (t < hi) pr.dloga[((int64_t)b * T_ + t) * H + h] = (float)(v + after);
    carry = total;
  }
}

// ------------------------------------------------------------ launch sequence

using BwdFn = int (*)(const BwdParams&, hipStream_t);

// Grid of a persistent chunk pass: the work-groups the current device holds
// at once (compute units x resident work-groups per unit), a multiple of 8
// (one share per XCD), at most one per tile rounded up to 8.
inline int bwd_chunk_grid(const void* kernel, int C, int tiles) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, bwd_chunk_threads(C), 0) != hipSuccess ||
      per <= 0)
    per = 1;
  const int fill = (cus * per) & ~7;
  const int need = (tiles + 7) & ~7;
  return fill < 8 ? 8 : (need < fill ? need : fill);
}
template <class K>
inline int bwd_chunk_grid(K* kernel, int C, int tiles) {
  return bwd_chunk_grid(reinterpret_cast<const void*>(kernel), C, tiles);
}

template <class T, int C, int P, int N>
int launch_backward(const BwdParams& pr, hipStream_t st) {
  using Tl = Tiles<T, C, P, N>;
  const int bh = pr.batch * pr.nheads;
  hipLaunchKernelGGL((bwd_atot_kernel<T, C>), dim3(pr.nc, bh), dim3(64), 0, st, pr);
  hipLaunchKernelGGL((bwd_cuma_kernel<T>), dim3(bh), dim3(BWD_SCAN_NT), 0, st, pr);
  if (pr.npart > 0) {
    // forward direction: blocks of the chunk states, levels 1-4 per group of
    // 8 chunks, then the levels above from the groups' totals
    hipLaunchKernelGGL((bwd_zst_group_kernel<T, C, P, N>), dim3((pr.nc + 7) / 8, bh), dim3(Tl::NT), 0, st, pr);
    if (pr.kc >= 5)
      hipLaunchKernelGGL((bwd_zst_up_kernel<T, P, N>), dim3((N * P + 1023) / 1024, bh), dim3(256), 0, st, pr);
    // reverse direction: per (level, pair, piece), the pieces then reduced
    constexpr bool LS2 = sizeof(T) == 2 && C == 64 && P == 64 && (N == 64 || N == 128);
    if (LS2 && (pr.nheads / pr.ngroups) % 2 == 0)  // the output pass's shape: its layouts, heads in pairs
      hipLaunchKernelGGL((bwd_level_state2_kernel<LS2 ? N : 128>), dim3(pr.npart, bh / 2), dim3(512), 0, st, pr);
    else
      hipLaunchKernelGGL((bwd_level_state_kernel<T, C, P, N, true>), dim3(pr.npart, bh), dim3(Tl::NT), 0, st, pr);
    if (pr.nstate > pr.nstate_direct)
      hipLaunchKernelGGL((bwd_level_reduce_kernel<T, P, N, true>),
                         dim3(pr.nstate - pr.nstate_direct, bh), dim3(256), 0, st, pr);
  }
  const int tiles = pr.nc * pr.batch * pr.ngroups;  // (batch * group, chunk), every head of the group in turn
  hipLaunchKernelGGL((bwd_dq_kernel<T, C, P, N>), dim3(bwd_chunk_grid(bwd_dq_kernel<T, C, P, N>, C, tiles)),
                     dim3(bwd_chunk_threads(C)), 0, st, pr);
  hipLaunchKernelGGL((bwd_dkv_kernel<T, C, P, N>), dim3(bwd_chunk_grid(bwd_dkv_kernel<T, C, P, N>, C, tiles)),
                     dim3(bwd_chunk_threads(C)), 0, st, pr);
  const int nseg = dloga_nseg(pr.seqlen);
  hipLaunchKernelGGL((bwd_dloga_part_kernel<T>), dim3(nseg, bh), dim3(256), 0, st, pr);
  hipLaunchKernelGGL((bwd_dloga_kernel<T>), dim3(nseg, bh), dim3(BWD_SCAN_NT), 0, st, pr);
  return (int)hipGetLastError();
}

// Shapes with a backward instantiation: bf16 needs P >= 32 and chunk >= 32
// (one MFMA step of 32 along the token and head dimensions); both chunk
// passes must fit in a CU's 160 KB of LDS.
template <class T, int C, int P, int N>
constexpr bool bwd_supported() {
  constexpr int KB = Mfma<T>::KB;
  return P >= KB && C >= KB && N >= KB &&
         bwd_dq_lds<T, C, P, N>() <= 160 * 1024 && bwd_dkv_lds<T, C, P, N>() <= 160 * 1024;
}

template <class T, int C>
BwdFn lookup_bwd(int P, int N) {
#define LOGLIN_BCASE(PP, NN)                                            \
  if constexpr (bwd_supported<T, C, PP, NN>())                          \
    if (P == PP && N == NN) return &launch_backward<T, C, PP, NN>;
  LOGLIN_BCASE(16, 16) LOGLIN_BCASE(16, 32) LOGLIN_BCASE(16, 64) LOGLIN_BCASE(16, 128)
  LOGLIN_BCASE(32, 16) LOGLIN_BCASE(32, 32) LOGLIN_BCASE(32, 64) LOGLIN_BCASE(32, 128)
  LOGLIN_BCASE(64, 16) LOGLIN_BCASE(64, 32) LOGLIN_BCASE(64, 64) LOGLIN_BCASE(64, 128)
#undef LOGLIN_BCASE
  return nullptr;
}

// Defined in one translation unit per (io type, chunk).
BwdFn lookup_bwd_bf16_32(int P, int N);
BwdFn lookup_bwd_bf16_64(int P, int N);
BwdFn lookup_bwd_f32_16(int P, int N);
BwdFn lookup_bwd_f32_32(int P, int N);
BwdFn lookup_bwd_f32_64(int P, int N);

}  // namespace loglin
