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

#include <type_traits>

namespace loglin {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Upper bound on Fenwick depth over segments (supports 2^16 segments).
constexpr int MAX_DEPTH = 16;

// Level weights of one chunk sit in LDS as 32-bit words copied straight
// from the lambda tensor: token t owns words [t W, t W + W) starting at the
// word that holds its first weight.  W is odd, so 16 consecutive tokens read
// 16 different banks.  bf16 rows may start in the upper half of a word.
__host__ __device__ inline int lam_words(int ll, int esize) {
  return esize == 4 ? (ll | 1) : (((ll + 1) / 2 + 1) | 1);
}

struct Params {
  const void* X;
  const void* Bm;
  const void* Cm;
  const float* log_a;
  const void* lam;
  void* out;
  void* seg_state;   // [batch*nheads, ns, P, N] io type, natural or state order
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
  int hp;     // heads per work-group of the output pass (1 or 2)
  unsigned long long lmask;  // levels the output includes (bit l: level l)
  int total;  // logical work-groups of the kernel being launched
  int nat;    // segment states and slots in natural state order (1) or state order (0)
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

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 16 bytes of T as a register vector.
template <class T>
struct Vec;
template <>
struct Vec<bf16> {
  using v16 = bf16x8;
  using v2 = bf16x2;
};
template <>
struct Vec<float> {
  using v16 = f32x4;
  using v2 = f32x2;
};
template <class T>
using vec16_t = typename Vec<T>::v16;
template <class T>
using vec2_t = typename Vec<T>::v2;

template <class T>
__device__ inline vec16_t<T> load16(const T* p) {
  return *reinterpret_cast<const vec16_t<T>*>(p);
}
template <class T>
__device__ inline void store16(T* p, vec16_t<T> v) {
  *reinterpret_cast<vec16_t<T>*>(p) = v;
}
template <class T>
__device__ inline void store_pair(T* p, T a, T b) {
  vec2_t<T> v = {a, b};
  *reinterpret_cast<vec2_t<T>*>(p) = v;
}

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

__device__ inline void store4(bf16* p, f32x4 v) {
  bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ inline void store4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// Work-group barrier for LDS producer / consumer hand-offs.  It waits for
// this wave's LDS operations only: __syncthreads() also waits for every
// outstanding global load (its fence is not address-space aware), which
// would stall on the asynchronous global->LDS prefetch of the next chunk.
// Tiles filled by global_load_lds are published with an explicit
// s_waitcnt before the barrier that precedes their first read.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
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
  static constexpr int VEC = 16 / (int)sizeof(T);
  // LDS arrays indexed [row][token] (X^T, W, (B w)^T): for bf16 with 64
  // tokens the rows are unpadded and the 16-byte blocks of a row are XOR-
  // swizzled by ((row >> 3) ^ row) & 7, which keeps both the token-pair
  // transposing stores and the MFMA operand loads free of bank conflicts;
  // other shapes use a 16-byte row pad.
  static constexpr bool SWZ = sizeof(T) == 2 && KC == 64;
  static constexpr int XS = SWZ ? KC : KC + VEC;  // LDS row stride
  __device__ static inline int col(int row, int c) {
    if constexpr (SWZ) return (((c >> 3) ^ (row >> 3) ^ row) & 7) << 3 | (c & 7);
    else return c;
  }
  __device__ static inline int at(int row, int c) { return row * XS + col(row, c); }
  static_assert(C % 16 == 0 && P % 16 == 0 && N % KB == 0, "tile sizes");
  static_assert(C <= 64, "one wave scans a chunk");
};

// Per-token quantities of one chunk, staged in LDS by wave 0:
//   cum[t]  inclusive prefix sum of log a over the chunk (fp32),
//   ecum[t] = exp(cum[t])            (decay from the chunk start to t),
//   wst[t]  = exp(cum[C-1] - cum[t]) (decay from t to the chunk end).
// The prefix sum runs on DPP lane moves inside the wave (no LDS round
// trips): shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the
// last lane of each row is added to the rows after it (row_bcast:15 and
// row_bcast:31).  Only the first C lanes are used.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_shift_add(float v) {
  // lanes whose source is outside the move (or whose row is masked off)
  // add the old value 0
  const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false);
  return v + __builtin_bit_cast(float, t);
}
template <int C>
__device__ inline float wave_prefix_sum(float v) {
  v = dpp_shift_add<0x111, 0xf>(v);  // row_shr:1
  v = dpp_shift_add<0x112, 0xf>(v);  // row_shr:2
  v = dpp_shift_add<0x114, 0xf>(v);  // row_shr:4
  v = dpp_shift_add<0x118, 0xf>(v);  // row_shr:8
  if constexpr (C > 16) v = dpp_shift_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  if constexpr (C > 32) v = dpp_shift_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <class T, int C>
__device__ inline void chunk_decays(float la, float* cum, float* ecum, float* wst, int tid) {
  if (tid < 64) {  // one whole wave: the lane moves need every lane active
    const float v = wave_prefix_sum<C>(la);
    const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), C - 1));
    if (tid < C) {
      cum[tid] = v;
      ecum[tid] = Mfma<T>::ex(v);
      wst[tid] = Mfma<T>::ex(tot - v);
    }
  }
}

// A tile of token rows (B, C or X of one chunk) staged in LDS unpadded, W
// elements per row, with the 16-byte blocks of row t XOR-swizzled by a key
// k(t).  The reads it serves: 16 rows x one block (row-wise MFMA operands,
// 16 lanes per LDS cycle), the state-order 8-byte halves of 16 rows, and
// the transposing 8-byte reads of rows {R..R+3} and {R+8..R+11} x two
// neighbouring blocks (32 lanes per LDS cycle); the output rows are written
// 8 bytes a lane and read back 16.  For bf16 the keys keep all of these
// free of bank conflicts (checked against a model of 64 four-byte banks):
//   256-byte rows (16 blocks, a row spans every bank): k(t) must differ
//     between the 16 rows of an aligned group, and k(t)/2 between the eight
//     rows of one transposing read: k = 2 (t mod 4) + 8 (t/8 mod 2) + (t/4 mod 2);
//   128-byte rows (8 blocks, two rows per bank sweep): k must differ
//     between the even (and between the odd) rows of an aligned group of
//     16, and k/2 between the even (odd) rows of one transposing read:
//     k = 2 (t/2 mod 2) + 4 (t/8 mod 2) + (t/4 mod 2).
// Other shapes use k(t) = t mod (blocks per row).
template <class T, int W>
struct Rows {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int NBLK = W / VEC;
  // physical 16-byte block of logical block b in row `row` (an involution)
  __device__ static inline int blk(int row, int b) {
    if constexpr (sizeof(T) == 2 && NBLK == 16)
      return b ^ (((row & 3) << 1) | (((row >> 3) & 1) << 3) | ((row >> 2) & 1));
    else if constexpr (sizeof(T) == 2 && NBLK == 8)
      return b ^ ((((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2) | ((row >> 2) & 1));
    else
      return (b ^ row) & (NBLK - 1);
  }
  __device__ static inline int at(int row, int c) {
    return row * W + blk(row, c / VEC) * VEC + (c % VEC);
  }
};

// Level slots (pass 2 output, pass 3 input) are stored in the order the
// output pass loads them as MFMA A operands: for each 16-row block w of the
// P rows and contraction step kk, the 64 lanes' KPL-element fragments lie
// back to back (lane 16 g + r at position 4 r + g), so every load
// instruction of a wave reads whole cache lines.  Element (p, n) of a state
// in state order (n = state_pos of the state row) goes to slot_index(p, n).
template <class T, int N>
__host__ __device__ constexpr int slot_index(int p, int n) {
  using M = Mfma<T>;
  constexpr int NKN = N / M::KB;
  const int w = p >> 4, r = p & 15, kk = n / M::KB, g = (n % M::KB) / M::KPL, j = n % M::KPL;
  return ((w * NKN + kk) * 64 + r * 4 + g) * M::KPL + j;
}
// First element of lane (g, r)'s fragment at step kk of row block w.
template <class T, int N>
__host__ __device__ constexpr int slot_frag(int w, int kk, int g, int r) {
  using M = Mfma<T>;
  return ((w * (N / M::KB) + kk) * 64 + r * 4 + g) * M::KPL;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* global_ptr_t;

// One global_load_lds_dwordx4: lane i copies 16 bytes from its own global
// address to LDS address lds_base + 16 i.  Issued from inline assembly so
// that the compiler does not track it: its wait analysis cannot tell LDS
// arrays apart for these copies and would otherwise stall every later LDS
// read on the copy in flight.  Callers publish the data with s_waitcnt
// vmcnt(0) and a barrier before the first read of the destination.
__device__ inline void dma_16x64(const void* src, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

// Same with global_load_lds_dword: lane i copies 4 bytes to lds_byte + 4 i.
__device__ inline void dma_4x64(const void* src, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

// The same two copies from a uniform base address (scalar registers) plus
// a 32-bit per-lane byte offset: the per-lane address arithmetic stays
// 32-bit.  The base must be the same in every lane (it is read from the
// first active one).
__device__ inline unsigned long long uniform_addr(const void* p) {
  const unsigned long long a = (unsigned long long)(uintptr_t)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
__device__ inline void dma_16x64_at(const void* base, unsigned off, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(uniform_addr(base)), "s"(m0)
               : "memory", "m0");
}
__device__ inline void dma_4x64_at(const void* base, unsigned off, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(uniform_addr(base)), "s"(m0)
               : "memory", "m0");
}

// Byte address of an LDS array element in the LDS aperture (32 bits).
__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(lds_ptr_t)const_cast<void*>(p);
}

// Copy R token rows of W elements (global row stride `grs` elements) into
// LDS in the Rows layout with global_load_lds_dwordx4: lane i of an
// instruction writes the 16 bytes at M0 + 16 i, so each instruction fills
// 1 KB of LDS and every lane fetches the global block that belongs there.
// The copy is asynchronous: s_waitcnt and a barrier precede any read.
// g is uniform; R rows of the stride fit 32-bit byte offsets (the host
// bounds heads and state sizes far below that).  The row offset is a 24-bit
// multiply (full rate; a 32-bit one takes four passes): rows are below 64
// and the host's bounds keep the row stride below 2^22 bytes.
template <class T, int R, int W, int NW>
__device__ inline void rows_to_lds(const T* g, int64_t grs, T* lds, int wave, int lane) {
  using L = Rows<T, W>;
  constexpr int PIECES = R * L::NBLK;  // 16-byte pieces of the tile
  constexpr int INSTS = (PIECES + 63) / 64;
  const int ws = __builtin_amdgcn_readfirstlane(wave);  // uniform: keep it scalar
  __builtin_assume(ws >= 0 && ws < NW);
  const unsigned rs = (unsigned)grs * (unsigned)sizeof(T);  // row stride in bytes
#pragma unroll
  for (int k = 0; k < (INSTS + NW - 1) / NW; ++k) {
    const int inst = ws + k * NW;
    const int piece = inst * 64 + lane;
    if ((INSTS % NW == 0 || inst < INSTS) && (PIECES % 64 == 0 || piece < PIECES)) {
      // (lanes past a short tile write nothing)
      const int row = piece / L::NBLK, pb = piece % L::NBLK;
      const int lb = L::blk(row, pb);  // logical block that lands in physical block pb
      dma_16x64_at(g, __umul24((unsigned)row, rs) + (unsigned)(lb * 16), lds_addr(lds) + inst * 1024u);
    }
  }
}

// Copy BYTES contiguous bytes (a multiple of 16) into LDS unchanged.
template <int BYTES, int NW>
__device__ inline void flat_to_lds(const void* g, void* lds, int wave, int lane) {
  constexpr int PIECES = BYTES / 16;
  constexpr int INSTS = (PIECES + 63) / 64;
  const int ws = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int k = 0; k < (INSTS + NW - 1) / NW; ++k) {
    const int inst = ws + k * NW;
    const int piece = inst * 64 + lane;
    if (inst < INSTS && piece < PIECES)
      dma_16x64(static_cast<const char*>(g) + piece * 16, lds_addr(lds) + inst * 1024u);
  }
}

// ---- MFMA operand fragments from LDS tiles (lane = 16 g + r)

// Contraction along a row: elements [k0 + KPL g, k0 + KPL g + KPL) of row
// `row` (one 16-byte read for bf16).
template <class T, class Lay>
__device__ inline typename Mfma<T>::frag frag_along(const T* tile, int row, int k0, int g) {
  return load_frag<T>(tile + Lay::at(row, k0 + g * Mfma<T>::KPL));
}

// Contraction down the rows: lane (g, r) receives tile[k0 + KPL g + j][c0 + r]
// for j < KPL.  For bf16 this is two ds_read_b64_tr_b16: within each group
// of 16 lanes, lane i = 4q + p receives element p of the 8-byte pieces that
// lanes q, q+4, q+8, q+12 address; lane s addresses row kb + s/4 at column
// c0 + 4 (s mod 4), so lane i gets rows kb..kb+3 of column c0 + i.
template <class Lay>
__device__ inline bf16x8 frag_down_bf16(const bf16* tile, int k0, int c0, int g, int r) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16* lp;
  const int kb = k0 + 8 * g + (r >> 2), c = c0 + 4 * (r & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(void*)(tile + Lay::at(kb, c)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(void*)(tile + Lay::at(kb + 4, c)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <class T, class Lay>
__device__ inline typename Mfma<T>::frag frag_down(const T* tile, int k0, int c0, int g, int r) {
  if constexpr (sizeof(T) == 2) return frag_down_bf16<Lay>(tile, k0, c0, g, r);
  else return tile[Lay::at(k0 + g, c0 + r)];
}

// frag_down of a token-row tile with row k scaled by w[k] (fp32 math).
template <class T, class Lay>
__device__ inline typename Mfma<T>::frag frag_down_scaled(const T* tile, const float* w, int k0,
                                                          int c0, int g, int r) {
  auto f = frag_down<T, Lay>(tile, k0, c0, g, r);
  if constexpr (sizeof(T) == 2) {
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + k0 + 8 * g);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + k0 + 8 * g + 4);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = (bf16)((float)f[j] * w0[j]);
      o[j + 4] = (bf16)((float)f[j + 4] * w1[j]);
    }
    return o;
  } else {
    return f * w[k0 + g];
  }
}

// State-order B-operand fragment (see Mfma::state_row) of token row `row`.
template <class T, int N>
__device__ inline typename Mfma<T>::frag rows_state_frag(const T* tile, int row, int kk, int g) {
  using L = Rows<T, N>;
  if constexpr (sizeof(T) == 2) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(tile + L::at(row, 32 * kk + 4 * g));
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(tile + L::at(row, 32 * kk + 16 + 4 * g));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    return tile[L::at(row, Mfma<float>::state_row(kk, g, 0))];
  }
}

// One chunk's state S[n][p] = sum_t B[t][n] w[t] X[t][p] for this wave's 16
// columns of X (all N rows of S), accumulated into S (NB tiles of 16x16).
template <class T, int C, int P, int N>
__device__ inline void chunk_state_mma(const T* bs, const T* xs, const float* w, f32x4* S,
                                       int wave, int g, int r) {
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
#pragma unroll
  for (int kt = 0; kt < Tl::NKT; ++kt) {  // rows C..KC-1 of the tiles are zero
    const auto bf = frag_down_scaled<T, Rows<T, P>>(xs, w, kt * Tl::KB, 16 * wave, g, r);
#pragma unroll
    for (int nb = 0; nb < Tl::NB; ++nb) {
      const auto af = frag_down<T, Rows<T, N>>(bs, kt * Tl::KB, 16 * nb, g, r);
      S[nb] = M::mma(af, bf, S[nb]);
    }
  }
}

// ------------------------------------------------------------- pass 1

// One work-group per (batch, segment, HS heads of one group).  Wave w
// serves head w / (P/16) and owns its state columns [16 (w mod P/16), +16)
// and all N rows, as NB 16x16 fp32 tiles.  The heads of a group read the
// same B rows, so with HS = 2 one copy of them in LDS serves both.  B and X
// rows go straight to LDS, double-buffered: the next chunk's rows are
// requested as soon as the current chunk's have landed.
template <class T, int C, int P, int N, int HS>
__global__ __launch_bounds__((HS * Tiles<T, C, P, N>::NT), (HS * Tiles<T, C, P, N>::NW / 2))
void state_kernel(Params pr) {
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
  constexpr int KC = Tl::KC;  // token rows of a tile; rows C..KC-1 stay zero
  constexpr int NT = HS * Tl::NT;
  // Two named buffers (not one 2-D array) so that the compiler can tell the
  // asynchronous fill of one from reads of the other and does not wait.
  __shared__ __attribute__((aligned(1024))) T bsh0[KC * N];
  __shared__ __attribute__((aligned(1024))) T bsh1[KC * N];
  __shared__ __attribute__((aligned(1024))) T xsh0[HS * KC * P];
  __shared__ __attribute__((aligned(1024))) T xsh1[HS * KC * P];
  __shared__ __attribute__((aligned(16))) float cum[HS * C], ecum[HS * C], wst[HS * KC];

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= pr.total) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = wave / Tl::NW, wv = wave % Tl::NW;
  const int g = lane >> 4, r = lane & 15;
  const int H = pr.nheads, G = pr.ngroups;
  if (KC > C) {
    for (int i = tid; i < (KC - C) * (N + HS * P); i += NT) {
      const int rr = C + i / (N + HS * P), c = i % (N + HS * P);
      if (c < N) {
        bsh0[rr * N + c] = bsh1[rr * N + c] = from_f<T>(0.f);
      } else {
        const int x = c - N, o = (x / P) * KC * P + rr * P + x % P;
        xsh0[o] = xsh1[o] = from_f<T>(0.f);
      }
    }
    for (int i = tid; i < HS * (KC - C); i += NT) wst[(i / (KC - C)) * KC + C + i % (KC - C)] = 0.f;
  }
  // heads of one group next to each other (they read the same B rows), then
  // groups, then segments: the work-groups running together on an XCD (a
  // contiguous range of tiles) cover every head of a few segments and share
  // each token's log-decay line (32 heads' log-decays per 128 bytes)
  const int hpg = H / G, npair = hpg / HS;
  const int pi = tile % npair;
  const int grp = (tile / npair) % G;
  const int q = (tile / (npair * G)) % pr.ns;
  const int b = tile / (npair * G * pr.ns);
  const int h0 = grp * hpg + pi * HS;
  const int h = h0 + hh;
  const int bh = b * H + h;
  const T* X = static_cast<const T*>(pr.X);
  const T* Bm = static_cast<const T*>(pr.Bm);
  const int seg = 1 << pr.m;
  const int j0 = q * seg;
  const int nch = min(seg, pr.nc - j0);
  float* cum_h = cum + hh * C;
  float* ecum_h = ecum + hh * C;
  float* wst_h = wst + hh * KC;

  f32x4 S[Tl::NB];
#pragma unroll
  for (int nb = 0; nb < Tl::NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float seg_sum = 0.f;

  auto issue = [&](int j, T* bs, T* xs) __attribute__((always_inline)) {
    const int64_t row0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    rows_to_lds<T, C, N, HS * Tl::NW>(Bm + (row0 * G + grp) * N, (int64_t)G * N, bs, wave, lane);
#pragma unroll
    for (int k = 0; k < HS; ++k)
      rows_to_lds<T, C, P, HS * Tl::NW>(X + (row0 * H + h0 + k) * P, (int64_t)H * P, xs + k * KC * P,
                                        wave, lane);
  };
  // log-decays of each head, loaded and scanned by its first wave
  auto load_la = [&](int j) __attribute__((always_inline)) {
    const int64_t rn = (int64_t)b * pr.seqlen + (int64_t)j * C;
    return (wv == 0 && lane < C) ? pr.log_a[(rn + lane) * H + h] : 0.f;
  };
  float la = load_la(j0);
  issue(j0, bsh0, xsh0);
  // one chunk per call; CUR selects the buffer pair at compile time
  auto step = [&](auto cur_c, int jl) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value;
    T* bs = CUR ? bsh1 : bsh0;
    T* xs = (CUR ? xsh1 : xsh0) + hh * KC * P;
    if (wv == 0) chunk_decays<T, C>(la, cum_h, ecum_h, wst_h, lane);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rows of the chunk have landed
    lds_barrier();
    if (jl + 1 < nch) {  // the other buffer was released by the previous barrier
      issue(j0 + jl + 1, CUR ? bsh0 : bsh1, CUR ? xsh0 : xsh1);
      la = load_la(j0 + jl + 1);
    }
    const float atot = cum_h[C - 1];
    if (jl > 0) {
      const float dec = M::ex(atot);
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb) S[nb] *= dec;
    }
    // lane addresses rebuilt per chunk rather than held across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    chunk_state_mma<T, C, P, N>(bs, xs, wst_h, S, wv, ln >> 4, ln & 15);
    seg_sum += atot;
    lds_barrier();
  };
  for (int jl = 0; jl < nch; jl += 2) {
    step(std::integral_constant<int, 0>{}, jl);
    if (jl + 1 < nch) step(std::integral_constant<int, 1>{}, jl + 1);
  }

  // the segment state in the io type (fp32 accumulation; the level scan
  // sums in fp32 and its slots are stored in the io type as well)
  T* dst = static_cast<T*>(pr.seg_state) + ((int64_t)bh * pr.ns + q) * (P * N) + (16 * wv + r) * N;
  if (pr.nat) {  // row n at position n
#pragma unroll
    for (int nb = 0; nb < Tl::NB; ++nb) store4(dst + 16 * nb + 4 * g, S[nb]);
  } else {
#pragma unroll
    for (int nb = 0; nb < Tl::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[M::state_pos(16 * nb + 4 * g + i)] = from_f<T>(S[nb][i]);
  }
  if (wv == 0 && lane == 0) pr.seg_decay[(int64_t)bh * pr.ns + q] = seg_sum;
}

// ------------------------------------------------------------- pass 2

// grid (ceil(P*N/(128 E)), batch*nheads), 128 threads.  Each thread owns E
// consecutive state elements (16 bytes per segment: E = 8 for bf16, 4 for
// fp32) and sweeps the segments in order, keeping a Fenwick stack of block
// sums in fp32 registers: after segment q the top entry is the sum over the
// largest aligned block of segments ending at q, decayed to q's end.  That
// block is the lower half a later segment reads at level trailing_ones(q) +
// 1.  The E elements share a state row, so they land in E consecutive slot
// positions.  D bounds the stack depth: the host passes ns < 2^D.
//
// Before segment q the live entries are the set bits of q (entry i: a block
// of 2^i segments), so the log-decay from the start of q's 2^(k-1)-aligned
// block to q's start is the sum of the live entries' decays below bit k-1;
// the stack's decays are the same in every thread, so threads 0..ks of the
// first work-group of each (batch, head) write one level's gap each.
//
// Loads run SCAN_U segments ahead through a per-wave LDS ring, filled by
// global_load_lds (lane i's 16 bytes land at ring slot + 16 i, and lane i
// reads back only those).  In registers the prefetch would be copied around
// the loop by the register allocator (the stack pushes loaded values), and
// each copy waits for its load.  The segment log-decays are staged in LDS
// too, SCAN_DEC at a time: as scalar loads their waits would complete out
// of order and also wait for the prefetch.
constexpr int SCAN_NT = 128;
constexpr int SCAN_U = 16;
constexpr int SCAN_DEC = 1024;

// s_waitcnt on the vector memory counter alone.  Written as inline assembly
// with a memory clobber so that no LDS read of the copied data is moved
// above it (the builtin form does not order memory accesses).
template <int NV>
__device__ inline void wait_vm() {
  static_assert(NV >= 0 && NV < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV) : "memory");
}

template <class T, int N, int D>
__global__ __launch_bounds__(SCAN_NT) void scan_kernel(Params pr, int pn) {
  using M = Mfma<T>;
  constexpr int U = SCAN_U;
  constexpr int E = 16 / (int)sizeof(T);  // state elements per thread
  static_assert(SCAN_DEC % U == 0, "decay tiles hold whole batches");
  __shared__ float dec_s[SCAN_DEC];
  __shared__ f32x4 ring[SCAN_NT / 64][U][64];
  const int bh = blockIdx.y;
  const int ns = pr.ns;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float* dec = pr.seg_decay + (int64_t)bh * ns;
  // pn is a multiple of 64 E, so a wave's elements are all valid or all idle
  const int e = (blockIdx.x * SCAN_NT + threadIdx.x) * E;
  const bool valid = e < pn;
  const bool gap_lane = blockIdx.x == 0 && (int)threadIdx.x <= pr.ks;
  const T* src = static_cast<const T*>(pr.seg_state) + (int64_t)bh * ns * pn;
  T* dst = static_cast<T*>(pr.slots) + (int64_t)bh * ns * pn;
  float* gd = pr.gap_decay + (int64_t)bh * ns * (pr.ks + 1);
  const int di = valid ? slot_index<T, N>(e / N, e % N) : 0;

  // E fp32 values of a state element run (the copy's 16 bytes widened)
  struct Run {
    float v[E];
  };
  auto widen = [](const f32x4& raw) __attribute__((always_inline)) {
    Run x;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int c = 0; c < E; ++c) x.v[c] = (float)h[c];
    } else {
#pragma unroll
      for (int c = 0; c < E; ++c) x.v[c] = raw[c];
    }
    return x;
  };
  Run stk[D];
  float stka[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
#pragma unroll
    for (int c = 0; c < E; ++c) stk[i].v[c] = 0.f;
    stka[i] = 0.f;
  }
  // Every prefetch is issued, so that each wave's count of memory operations
  // per segment is fixed: the segment index is clamped to the last one
  // stored, ns - 2 (the pass runs for ns > 1), and idle lanes read element 0.
  // What such a copy holds is only ever pushed by the final segment, whose
  // result no one reads.
  const int ec = valid ? e : 0;
  auto prefetch = [&](int q, int slot) __attribute__((always_inline)) {
    dma_16x64(src + (int64_t)min(q, ns - 2) * pn + ec, lds_addr(&ring[wv][slot][0]));
  };
  auto refill = [&](int q0) __attribute__((always_inline)) {  // uniform
    __syncthreads();
    for (int i = threadIdx.x; i < SCAN_DEC && q0 + i < ns; i += SCAN_NT) dec_s[i] = dec[q0 + i];
    __syncthreads();
  };
  // one segment: fold the stack entries below its level in, push, store
  auto step = [&](Run v, int q) __attribute__((always_inline)) {
    float acur = dec_s[q % SCAN_DEC];
    const int z = __builtin_ctz(~(unsigned)q);  // trailing ones of q (uniform)
    if (gap_lane) {  // lane k writes level k's gap; one store, no loop
      float run = 0.f;
#pragma unroll
      for (int i = 0; i + 1 < D; ++i)
        if (i + 1 < (int)threadIdx.x && ((q >> i) & 1)) run += stka[i];
      gd[q * (pr.ks + 1) + threadIdx.x] = run;
    }
    // Unrolled into uniform branches, one per entry, so that every stack
    // index is a constant and the stack stays in registers (a loop with an
    // early exit lets the compiler sink the push into one store at a
    // runtime index, which moves the stack to scratch memory).
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (i < z) {
        const float w = M::ex(acur);
#pragma unroll
        for (int c = 0; c < E; ++c) v.v[c] = w * stk[i].v[c] + v.v[c];
        acur += stka[i];
      }
    }
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (i == z) {
        stk[i] = v;
        stka[i] = acur;
      }
    }
    if (valid && q < ns - 1) {
      if constexpr (sizeof(T) == 2) {
        bf16x8 o;
#pragma unroll
        for (int c = 0; c < E; ++c) o[c] = (bf16)v.v[c];
        store16(dst + (int64_t)q * pn + di, o);
      } else {
        store4(dst + (int64_t)q * pn + di, f32x4{v.v[0], v.v[1], v.v[2], v.v[3]});
      }
    }
  };

#pragma unroll
  for (int u = 0; u < U; ++u) prefetch(u, u);
  const int nfull = ns / U * U;
  for (int q0 = 0; q0 < nfull; q0 += U) {
    if (q0 % SCAN_DEC == 0) refill(q0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // Memory operations this wave issued after segment q0+u's copy: the
      // U-1 later copies, and in a valid wave the slot stores of the U-1
      // segments since (none in the first batch).  The first work-group's
      // gap stores only add to the count, which makes the wait longer.
      if (valid && q0 > 0)
        wait_vm<2 * U - 2>();
      else
        wait_vm<U - 1>();
      const Run v = widen(ring[wv][u][lane]);
      step(v, q0 + u);
      prefetch(q0 + U + u, u);  // v has been used, so its slot is free
    }
  }
  // The last ns mod U segments: their copies were issued by the final batch
  // (or the prologue) into slots 0, 1, ...
  wait_vm<0>();
  if (nfull < ns && nfull % SCAN_DEC == 0) refill(nfull);
  for (int q = nfull; q < ns; ++q) step(widen(ring[wv][q - nfull][lane]), q);
}

// The same level scan for up to SCAN_RMAX L segments, split into ranges of
// L segments that run side by side, one wave per range (work-group = the
// ranges of one run of 64 E state elements).  A slot is the sum over an
// aligned block of segments, and every block of at most L segments lies in
// one range, so each wave sweeps its range with a stack of depth log2 L,
// starting empty.  The blocks that span ranges are the slots of a range's
// last segment when the range index is odd (2^t ranges for t trailing ones
// of the index): they are formed after the sweeps from the ranges' totals,
// exchanged through LDS.  The gaps of levels above log2 L + 1 likewise add
// the log-decays of whole ranges to the range-local prefix.  All of a
// wave's copies are issued before its first step (L is a compile-time
// count, and the sweep is unrolled, so every stack index is a constant).
constexpr int SCAN_RMAX = 16;
constexpr int SCAN_L = 16;

template <class T, int N, int L>
__global__ __launch_bounds__(64 * SCAN_RMAX) void scan_range_kernel(Params pr, int pn) {
  using M = Mfma<T>;
  constexpr int E = 16 / (int)sizeof(T);  // state elements per lane
  constexpr int J = ilog2c(L);
  static_assert(L == (1 << J) && E % 4 == 0, "ranges of 2^J segments");
  __shared__ f32x4 tot_s[SCAN_RMAX][E / 4][64];  // range totals, fp32
  __shared__ float tdec_s[SCAN_RMAX];              // range log-decays
  const int bh = blockIdx.y, ns = pr.ns, ks = pr.ks;
  const int lane = threadIdx.x & 63;
  const int r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's range
  const int q0 = r * L;
  const int e = (blockIdx.x * 64 + lane) * E;  // the grid covers pn exactly
  const T* src = static_cast<const T*>(pr.seg_state) + (int64_t)bh * ns * pn + e;
  T* dst = static_cast<T*>(pr.slots) + (int64_t)bh * ns * pn + slot_index<T, N>(e / N, e % N);
  const float* dec = pr.seg_decay + (int64_t)bh * ns;
  float* gd = pr.gap_decay + (int64_t)bh * ns * (ks + 1);
  const bool gap_lane = blockIdx.x == 0 && lane <= ks;  // lane k writes level k's gap

  struct Run {
    float v[E];
  };
  auto widen = [](const f32x4& raw) __attribute__((always_inline)) {
    Run x;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int c = 0; c < E; ++c) x.v[c] = (float)h[c];
    } else {
#pragma unroll
      for (int c = 0; c < E; ++c) x.v[c] = raw[c];
    }
    return x;
  };
  auto put = [&](int q, const Run& v) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
      bf16x8 o;
#pragma unroll
      for (int c = 0; c < E; ++c) o[c] = (bf16)v.v[c];
      store16(dst + (int64_t)q * pn, o);
    } else {
      store4(dst + (int64_t)q * pn, f32x4{v.v[0], v.v[1], v.v[2], v.v[3]});
    }
  };

  // the range's copies and log-decays (segments past the end repeat the
  // last one; nothing they give is stored)
  f32x4 raw[L];
  float dq[L];
#pragma unroll
  for (int u = 0; u < L; ++u) {
    const int qc = min(q0 + u, ns - 1);
    raw[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)qc * pn);
    dq[u] = dec[qc];
  }
  Run stk[J + 1];
  float stka[J + 1];
  float pre[L];  // log-decay from the range's start to segment q0 + u
#pragma unroll
  for (int i = 0; i <= J; ++i) stka[i] = 0.f;
  static_for<0, L>([&](auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    constexpr int z = __builtin_ctz(~(unsigned)u);  // trailing ones of u
    const int q = q0 + u;
    // live entries before segment q: the set bits of u
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < J; ++i)
      if ((u >> i) & 1) run += (i + 1 < lane || lane > J + 1) ? stka[i] : 0.f;
    pre[u] = run;
    if (gap_lane && lane <= J + 1 && q < ns) gd[q * (ks + 1) + lane] = run;
    Run v = widen(raw[u]);
    float acur = dq[u];
#pragma unroll
    for (int i = 0; i < z; ++i) {
      const float w = M::ex(acur);
#pragma unroll
      for (int c = 0; c < E; ++c) v.v[c] = w * stk[i].v[c] + v.v[c];
      acur += stka[i];
    }
    stk[z] = v;
    stka[z] = acur;
    // the last segment's block spans ranges when r is odd (formed below)
    if (q < ns - 1 && (u < L - 1 || (r & 1) == 0)) put(q, v);
  });

  // range totals to LDS
#pragma unroll
  for (int c4 = 0; c4 < E / 4; ++c4)
    tot_s[r][c4][lane] = f32x4{stk[J].v[4 * c4], stk[J].v[4 * c4 + 1], stk[J].v[4 * c4 + 2], stk[J].v[4 * c4 + 3]};
  if (lane == 0) tdec_s[r] = stka[J];
  __syncthreads();

  const int qe = q0 + L - 1;
  if ((r & 1) && qe < ns - 1) {  // block of 2^t ranges ending with this one
    const int t = __builtin_ctz(~(unsigned)r);
    Run acc = stk[J];
    float a = stka[J];
    for (int rr = r - 1; rr > r - (1 << t); --rr) {
      const float w = M::ex(a);
#pragma unroll
      for (int c4 = 0; c4 < E / 4; ++c4) {
        const f32x4 x = tot_s[rr][c4][lane];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc.v[4 * c4 + c] = w * x[c] + acc.v[4 * c4 + c];
      }
      a += tdec_s[rr];
    }
    put(qe, acc);
  }
  if (gap_lane && lane > J + 1) {
    // level k = lane: its aligned block starts at range (r >> (k-1-J)) << (k-1-J)
    const int sh = lane - 1 - J;
    float rp = 0.f;
    for (int rr = (r >> sh) << sh; rr < r; ++rr) rp += tdec_s[rr];
#pragma unroll
    for (int u = 0; u < L; ++u)
      if (q0 + u < ns) gd[(q0 + u) * (ks + 1) + lane] = pre[u] + rp;
  }
}

// ------------------------------------------------------------- pass 3

// Largest segment depth m (chunks per segment 2^m) the output pass keeps a
// register stack for.
constexpr int MAX_SEG_LOG2 = 3;

// Score tiles of the intra-chunk block in the order they are dealt
// round-robin to the waves, so that every wave has a like share of the
// dearest tiles before the barrier that follows: the diagonal ones (a
// level and a causality test per element), then the tiles below them, then
// the strictly upper tiles the intra product reads, as zeros.  With 32
// tokens per MFMA contraction (bf16) token block tb reads columns up to the
// end of its 32-token half, so those are (tb, tb + 1) for even tb; with 4
// (fp32) it reads no upper tile.
template <int TB, int KB>
struct ScoreTiles {
  static constexpr int NO = TB * (TB - 1) / 2;       // below the diagonal
  static constexpr int NZ = KB == 32 ? TB / 2 : 0;  // upper tiles read as zeros
  static constexpr int N = TB + NO + NZ;
};
template <int TB, int KB>
__device__ inline void score_tile(int u, int& tb, int& sb) {
  static_assert(KB == 32 || KB == 4, "contraction lengths");
  if constexpr (TB == 4 && KB == 32) {
    // 64-token chunks (4 diagonal D, 6 lower O and 2 zero Z tiles): four
    // O, the four D, then O, O, Z, Z.  Dealt to 4 waves: D+2O, D+2O,
    // D+O+Z, D+O+Z; to 8 waves (two heads): 2O, 2O, O+Z, O+Z, D, D, D, D.
    // (one nibble 4 tb + sb per tile, in scalar arithmetic: an indexed
    // constant array would be a memory load whose wait also waits for the
    // copies in flight)
    constexpr unsigned long long order = 0xb1edfa50c984ull;
    const unsigned e = (unsigned)(order >> (4 * u)) & 15u;
    tb = (int)(e >> 2);
    sb = (int)(e & 3);
    return;
  }
  if (u < TB) {
    tb = sb = u;
    return;
  }
  u -= TB;
  if (u < ScoreTiles<TB, KB>::NO) {  // row-major: (1,0), (2,0), (2,1), (3,0), ...
    tb = 1;
    while (u >= tb) {
      u -= tb;
      ++tb;
    }
    sb = u;
    return;
  }
  tb = 2 * (u - ScoreTiles<TB, KB>::NO);
  sb = tb + 1;
}

// One work-group per (batch, segment of 2^m chunks, HP heads of one group);
// the chunks of the segment are processed in order.  The HP heads share
// the group's B and C rows and the scores C B^T; wave w serves head
// w / (P/16) and owns its output columns [16 (w mod P/16), +16) for all C
// tokens of a chunk (TB tiles of Y^T), and the same columns of every chunk
// state it builds.
//
// Inter-chunk level k of chunk j reads the lower half of j's 2^k-chunk
// block.  For k > m that block is a run of whole segments: its sum is slot
// ((q >> ks) << ks) + 2^(ks-1) - 1 of pass 2 (ks = k - m), shared by every
// chunk of the segment.  The first RZ of those slots stay in registers for
// the whole segment; the others are fetched per chunk.  For k <= m the block
// lies inside the segment: the wave keeps a Fenwick stack of those block
// sums, entry e holding the block of 2^e chunks that ends just before the
// current chunk, as MFMA A-operand fragments.  The state MFMA leaves a lane
// exactly the rows its own fragments need, so the stack never crosses
// lanes.
//
// B and X rows are double-buffered in LDS (bf16): the next chunk's rows are
// requested right after the current chunk's first barrier.  C rows are
// single-buffered and refilled once the output tiles have read them.
template <class T, int C, int P, int N, int HP>
struct OutCfg {
  using Tl = Tiles<T, C, P, N>;
  static constexpr int NWH = Tl::NW;    // waves per head
  static constexpr int NTW = HP * NWH;  // waves per work-group
  static constexpr int NT = NTW * 64;
  static constexpr int NBUF = sizeof(T) == 2 ? 2 : 1;
  static constexpr int KC = Tl::KC;
  // slots above the segment held in registers for the whole segment
  static constexpr int RZ = sizeof(T) == 2 ? 3 : 1;
  static constexpr int MIN_BLOCKS = HP == 1 ? 2 : 1;
};

// MASKED: only the levels in pr.lmask enter the output (a separate
// instantiation, so the full pass pays nothing for the option).
template <class T, int C, int P, int N, int HP, bool MASKED>
__global__ __launch_bounds__((OutCfg<T, C, P, N, HP>::NT), (OutCfg<T, C, P, N, HP>::MIN_BLOCKS))
void output_kernel(Params pr) {
  using Cfg = OutCfg<T, C, P, N, HP>;
  using Tl = Tiles<T, C, P, N>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  using RB = Rows<T, N>;
  using RX = Rows<T, P>;
  constexpr int MM = MAX_SEG_LOG2;
  constexpr int NBUF = Cfg::NBUF;
  constexpr int RZ = Cfg::RZ;
  constexpr int NTW = Cfg::NTW;
  constexpr int KC = Tl::KC;  // token rows of the B / X tiles; rows C..KC-1 stay zero
  constexpr int GS = MAX_DEPTH + 1;
  // B and X rows, two named buffers each (bf16; fp32 uses only the first)
  // so that the compiler can tell the asynchronous fill of one from reads
  // of the other and does not wait for it.  X, W and the per-token arrays
  // hold HP heads back to back.
  __shared__ __attribute__((aligned(1024))) T bsh0[KC * N];
  __shared__ __attribute__((aligned(1024))) T bsh1[NBUF == 2 ? KC * N : 1];
  __shared__ __attribute__((aligned(1024))) T xsh0[HP * KC * P];
  __shared__ __attribute__((aligned(1024))) T xsh1[NBUF == 2 ? HP * KC * P : 1];
  __shared__ __attribute__((aligned(1024))) T csh[C * N];          // C rows
  // W[t][s] of each head; after the intra product, the head's output tile
  // [t][P] (Rows layout) on its way to memory
  constexpr int WTS = C * Tl::XS > C * P ? C * Tl::XS : C * P;
  __shared__ __attribute__((aligned(16))) T wt[HP * WTS];
  __shared__ __attribute__((aligned(16))) float cum[HP * C], ecum[HP * C], wst[HP * KC];
  __shared__ float gap_s[HP * GS];     // gap log-decays of this segment
  extern __shared__ unsigned lam_w[];  // [HP][C][lam_words]: level weights

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= pr.total) return;
  const int tid0 = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);  // uniform: keep it scalar
  const int hh = wave / Cfg::NWH;  // head of this wave within the work-group
  static_assert(WTS >= C * Tl::XS, "W buffer");
  const int wv = wave % Cfg::NWH;  // its 16-column block
  if (KC > C) {  // contraction padding of the token tiles and of W stays zero
    for (int i = tid0; i < (KC - C) * (N + HP * P); i += Cfg::NT) {
      const int rr = C + i / (N + HP * P), c = i % (N + HP * P);
      if (c < N) {
        bsh0[rr * N + c] = from_f<T>(0.f);
        if constexpr (NBUF == 2) bsh1[rr * N + c] = from_f<T>(0.f);
      } else {
        const int x = c - N, o = (x / P) * KC * P + rr * P + x % P;
        xsh0[o] = from_f<T>(0.f);
        if constexpr (NBUF == 2) xsh1[o] = from_f<T>(0.f);
      }
    }
    for (int i = tid0; i < HP * C * (KC - C); i += Cfg::NT) {
      const int row = i / (KC - C), k = row / C;  // head-major rows of W
      wt[k * WTS + (row % C) * Tl::XS + C + i % (KC - C)] = from_f<T>(0.f);
    }
    for (int i = tid0; i < HP * (KC - C); i += Cfg::NT) wst[(i / (KC - C)) * KC + C + i % (KC - C)] = 0.f;
  }
  const int H = pr.nheads, G = pr.ngroups, L = pr.nlevels, LL = pr.ll;
  const int LW = lam_words(LL, (int)sizeof(T));
  // Heads of one group next to each other (they share B and C), then
  // segments, then groups: the work-groups resident on one XCD at a time
  // cover few heads and many segments, so the level slots they read stay
  // in that XCD's L2.  Segments are dealt from the last one down: a segment
  // whose index has more set bits has more levels above it to apply, so the
  // longer work-groups start first and the shorter ones fill the tail.
  const int hpg = H / G, npair = hpg / HP;
  const int pi = tile % npair;
  const int q = pr.ns - 1 - (tile / npair) % pr.ns;
  const int grp = (tile / (npair * pr.ns)) % G;
  const int b = tile / (npair * pr.ns * G);
  const int h0 = grp * hpg + pi * HP;  // first head of the work-group
  const int h = h0 + hh;               // head of this wave
  const int bh = b * H + h;
  const int c_log = __builtin_ctz(C);
  const int m = pr.m;
  const int seg = 1 << m;
  const int j0 = q * seg;
  const int nch = min(seg, pr.nc - j0);
  const T* X = static_cast<const T*>(pr.X);
  const T* Bm = static_cast<const T*>(pr.Bm);
  const T* Cm = static_cast<const T*>(pr.Cm);
  const T* slots = static_cast<const T*>(pr.slots);
  T* out = static_cast<T*>(pr.out);
  float* cum_h = cum + hh * C;
  float* ecum_h = ecum + hh * C;
  float* wst_h = wst + hh * KC;
  const float* gap_h = gap_s + hh * GS;

  frag zl[MM][Tl::NKN];  // local Fenwick stack (entry e: 2^e chunks)
  float zla[MM];         // total log-decay of each entry's block
  float dloc[MM + 1];    // log-decay from a local block's end to the chunk
#pragma unroll
  for (int e = 0; e < MM; ++e) zla[e] = 0.f;
#pragma unroll
  for (int k = 0; k <= MM; ++k) dloc[k] = 0.f;
  float accseg = 0.f;  // log-decay from the segment start to the chunk
  if (pr.ks > 0) {     // read after the first barrier
    for (int i = tid0; i < HP * (pr.ks + 1); i += Cfg::NT) {
      const int k = i / (pr.ks + 1), l = i % (pr.ks + 1);
      gap_s[k * GS + l] = pr.gap_decay[((int64_t)(b * H + h0 + k) * pr.ns + q) * (pr.ks + 1) + l];
    }
  }
  const unsigned ext_mask = (unsigned)q & ((1u << pr.ks) - 1u);  // active levels above
  auto slot_of = [&](int hd, int ks) __attribute__((always_inline)) {
    const int qs = ((q >> ks) << ks) + (1 << (ks - 1)) - 1;
    return slots + ((int64_t)(b * H + hd) * pr.ns + qs) * P * N;
  };
  // levels past the resident ones are fetched per chunk
  unsigned stream_mask = ext_mask;
#pragma unroll
  for (int i = 0; i < RZ; ++i) stream_mask &= stream_mask - 1;
  // the segment's lowest RZ level slots, in registers for all its chunks
  frag zres[RZ][Tl::NKN];
  {
    const int lane = tid0 & 63, r = lane & 15, g = lane >> 4;
    unsigned mk = ext_mask;
#pragma unroll
    for (int i = 0; i < RZ; ++i) {
      if (mk) {
        const T* zr = slot_of(h, __builtin_ctz(mk) + 1) + slot_frag<T, N>(wv, 0, g, r);
        mk &= mk - 1;
#pragma unroll
        for (int kk = 0; kk < Tl::NKN; ++kk) zres[i][kk] = load_frag<T>(zr + kk * 64 * Tl::KPL);
      }
    }
  }

  float la = 0.f;
  auto issue_bx = [&](int j, T* bs, T* xs, int lane) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    rows_to_lds<T, C, N, NTW>(Bm + (r0 * G + grp) * N, (int64_t)G * N, bs, wave, lane);
#pragma unroll
    for (int k = 0; k < HP; ++k)
      rows_to_lds<T, C, P, NTW>(X + (r0 * H + h0 + k) * P, (int64_t)H * P, xs + k * KC * P, wave, lane);
  };
  auto issue_c = [&](int j, int lane) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    rows_to_lds<T, C, N, NTW>(Cm + (r0 * G + grp) * N, (int64_t)G * N, csh, wave, lane);
  };
  auto issue_regs = [&](int j, int tid) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const int lane = tid & 63, r = lane & 15, g = lane >> 4;
    // the last wave of each head: the first issues the odd level-weight copy
    la = (wv == Cfg::NWH - 1 && lane < C) ? pr.log_a[(r0 + lane) * H + h] : 0.f;
  };
  // level weights of chunk j into lam_w (the last word of the tensor bounds
  // the copy: a row's padding words may run past the end)
  const int64_t lam_last_word = ((int64_t)pr.batch * pr.seqlen * H * L * (int64_t)sizeof(T) - 4) / 4;
  // idx / LW in float: idx < 2^13 and the exact quotient of idx + 1/2 lies
  // at least 1/(2 LW) from an integer, far beyond the rounding error
  const float inv_lw = 1.f / (float)LW;
  auto issue_lam = [&](int j, int lane) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const int64_t eb = (r0 * H + h0) * L;  // element index of the chunk's first row
    const int64_t wb = sizeof(T) == 4 ? eb : (eb >> 1);
    const int par0 = sizeof(T) == 4 ? 0 : (int)(eb & 1);
    const unsigned* base = static_cast<const unsigned*>(pr.lam) + wb;
    const unsigned lim = (unsigned)min(lam_last_word - wb, (int64_t)0x7fffffff);
    const int words = HP * C * LW;
    for (int inst = __builtin_amdgcn_readfirstlane(wave); inst * 64 < words; inst += NTW) {
      const int idx = inst * 64 + lane;
      if (idx < words) {
        const int tw = (int)(((float)idx + 0.5f) * inv_lw), w = idx - tw * LW;  // tw = head * C + token
        const int k = tw / C, t = tw - k * C;
        // element offset of the row from eb (24-bit multiplies: t < 64 and
        // the host bounds H by 4096 and L by 64)
        const int x = (int)__umul24((unsigned)t, (unsigned)(H * L)) + (int)__umul24((unsigned)k, (unsigned)L);
        unsigned ow = (unsigned)((sizeof(T) == 4 ? x : ((x + par0) >> 1)) + w);
        ow = ow < lim ? ow : lim;
        dma_4x64_at(base, ow * 4u, lds_addr(lam_w) + inst * 256u);
      }
    }
  };
  // weight of level lvl for token t of head h0 + k in the current chunk;
  // par: the row starts in the upper half of its first word (bf16, odd
  // level count)
  const unsigned long long lmask = MASKED ? pr.lmask : ~0ull;
  auto lam_at = [&](int k, int t, int lvl, int par) __attribute__((always_inline)) -> float {
    const int row = k * C + t;
    float v;
    if constexpr (sizeof(T) == 4) {
      v = __uint_as_float(lam_w[row * LW + lvl]);
    } else {
      const unsigned short* hw = reinterpret_cast<const unsigned short*>(lam_w);
      v = __uint_as_float((unsigned)hw[2 * row * LW + par + lvl] << 16);
    }
    if constexpr (MASKED) return (lmask >> lvl) & 1 ? v : 0.f;  // left-out levels weigh 0
    return v;
  };
  const bool intra_on = !MASKED || (lmask & ((2ull << c_log) - 1)) != 0;  // levels 0..log2 C
  // levels inside the segment (log2 C + 1 .. log2 C + m): the local stack
  const bool local_on = !MASKED || ((lmask >> (c_log + 1)) & ((1ull << m) - 1)) != 0;
  const int lpar = sizeof(T) == 2 ? (L & 1) : 0;
  issue_bx(j0, bsh0, xsh0, tid0 & 63);
  issue_c(j0, tid0 & 63);
  issue_lam(j0, tid0 & 63);
  issue_regs(j0, tid0);

  // one chunk per call; CUR selects the B / X buffer pair at compile time
  auto step = [&](auto cur_c, int jl) __attribute__((always_inline)) {
    constexpr int CUR = NBUF == 2 ? decltype(cur_c)::value : 0;
    T* bs = CUR ? bsh1 : bsh0;
    T* xsb = CUR ? xsh1 : xsh0;
    T* bs_next = NBUF == 2 ? (CUR ? bsh0 : bsh1) : bsh0;
    T* xs_next = NBUF == 2 ? (CUR ? xsh0 : xsh1) : xsh0;
    const int j = j0 + jl;
    const int64_t row0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const bool need_state = jl + 1 < nch;  // a next chunk: prefetch it, push this one's state
    // Recompute lane-dependent LDS addresses inside the loop instead of
    // keeping dozens of them live across it (they would be spilled).
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g = lane >> 4, r = lane & 15;
    const T* xs = xsb + hh * KC * P;

    // ---- per-token decays of the chunk (last wave of each head)
    if (wv == Cfg::NWH - 1) chunk_decays<T, C>(la, cum_h, ecum_h, wst_h, lane);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rows of the chunk have landed
    lds_barrier();
    if (NBUF == 2 && need_state) issue_bx(j + 1, bs_next, xs_next, lane);  // other pair is free
    const float atot = cum_h[C - 1];

    // ---- intra-chunk weights W[t][s] of every head, from the shared
    // transposed scores B C^T
    constexpr int NSC = ScoreTiles<Tl::TB, Tl::KB>::N;
    for (int u = intra_on ? wave : NSC; u < NSC; u += NTW) {
      int tb, sb;
      score_tile<Tl::TB, Tl::KB>(u, tb, sb);
      const int t = 16 * tb + r;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (sb <= tb) {
#pragma unroll
        for (int kk = 0; kk < Tl::NKN; ++kk)
          acc = M::mma(frag_along<T, RB>(bs, 16 * sb + r, kk * Tl::KB, g),
                       frag_along<T, RB>(csh, t, kk * Tl::KB, g), acc);
      }
#pragma unroll
      for (int k = 0; k < HP; ++k) {
        f32x4 wv4 = {0.f, 0.f, 0.f, 0.f};
        if (sb < tb) {
          // Below the diagonal blocks every s precedes t, and t XOR s =
          // 16 (tb XOR sb) + (r XOR (s mod 16)) has bit length
          // 4 + bitlen(tb XOR sb) across the whole tile: one level weight.
          const float ct_ = cum[k * C + t];
          const int par = lpar & ((((int)row0 + t) & H) ^ (h0 + k));  // parity of (row0 + t) H + h0 + k
          const float lt = lam_at(k, t, 4 + bit_length((unsigned)(tb ^ sb)), par);
          const f32x4 cs4 = *reinterpret_cast<const f32x4*>(cum + k * C + 16 * sb + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) wv4[i] = acc[i] * M::ex(ct_ - cs4[i]) * lt;
        } else if (sb == tb) {
          const float ct_ = cum[k * C + t];
          const int par = lpar & ((((int)row0 + t) & H) ^ (h0 + k));  // parity of (row0 + t) H + h0 + k
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = 16 * sb + 4 * g + i;
            wv4[i] = (s <= t) ? acc[i] * M::ex(ct_ - cum[k * C + s]) *
                                    lam_at(k, t, bit_length(t ^ s), par)
                              : 0.f;
          }
        }
        store4(wt + k * WTS + Tl::at(t, 16 * sb + 4 * g), wv4);
      }
    }
    lds_barrier();

    // ---- output tiles: intra block, then every active inter-chunk level
    {
      T* wth = wt + hh * WTS;
      const int par_r = lpar & ((((int)row0 + r) & H) ^ h);  // parity of (row0 + r) H + h: token 16 tb + r
      f32x4 Y[Tl::TB];
#pragma unroll
      for (int tb = 0; tb < Tl::TB; ++tb) {
        Y[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < Tl::NKT; ++kt) {
          if (intra_on && kt * Tl::KB < 16 * (tb + 1)) {
            auto af = frag_down<T, RX>(xs, kt * Tl::KB, 16 * wv, g, r);
            auto bf = load_frag<T>(wth + Tl::at(16 * tb + r, kt * Tl::KB + g * Tl::KPL));
            Y[tb] = M::mma(af, bf, Y[tb]);
          }
        }
      }
      // level weight of token 16 tb + r times e^(Lambda_t + D)
      auto level_scale = [&](int tb, int level, float eD) __attribute__((always_inline)) {
        const int t = 16 * tb + r;
        // 16 tb keeps the parity of the row start: H * 16 tb is even
        return lam_at(hh, t, level, par_r) * ecum_h[t] * eD;
      };

      // Levels whose slots are in registers (the segment's resident ones and
      // the local stack), one token block at a time: its C^T fragments are
      // read once and serve all of them.
      float eres[RZ];
      int lres[RZ];
      {
        unsigned mk = ext_mask;
#pragma unroll
        for (int i = 0; i < RZ; ++i) {
          const int ks = mk ? __builtin_ctz(mk) + 1 : 1;
          mk &= mk - 1;
          lres[i] = c_log + m + ks;
          eres[i] = M::ex(gap_h[ks] + accseg);
        }
      }
      const int nres = min(__builtin_popcount(ext_mask), RZ);
      float eloc[MM];
#pragma unroll
      for (int e = 0; e < MM; ++e) eloc[e] = M::ex(dloc[e + 1]);
#pragma unroll
      for (int tb = 0; tb < Tl::TB; ++tb) {
        frag cf[Tl::NKN];  // C^T fragments of the block, in state order
#pragma unroll
        for (int kk = 0; kk < Tl::NKN; ++kk) cf[kk] = rows_state_frag<T, N>(csh, 16 * tb + r, kk, g);
        // Every level's scale of the block is read up front, whether or not
        // the level is active (an inactive one reads a weight of the row,
        // clamped to the levels it holds, and is never used), so that no
        // product waits on a weight read issued just before it.
        float sres[RZ], sloc[MM];
#pragma unroll
        for (int i = 0; i < RZ; ++i) sres[i] = level_scale(tb, min(lres[i], LL - 1), eres[i]);
#pragma unroll
        for (int e = 0; e < MM; ++e) sloc[e] = level_scale(tb, min(c_log + e + 1, LL - 1), eloc[e]);
#pragma unroll
        for (int i = 0; i < RZ; ++i) {
          if (i < nres && (!MASKED || ((lmask >> lres[i]) & 1))) {
            f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < Tl::NKN; ++kk) tmp = M::mma(zres[i][kk], cf[kk], tmp);
            Y[tb] += sres[i] * tmp;
          }
        }
#pragma unroll
        for (int e = 0; e < MM; ++e) {  // levels inside the segment
          if (e < m && ((jl >> e) & 1) && (!MASKED || ((lmask >> (c_log + e + 1)) & 1))) {
            f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < Tl::NKN; ++kk) tmp = M::mma(zl[e][kk], cf[kk], tmp);
            Y[tb] += sloc[e] * tmp;
          }
        }
      }

      // The remaining levels above the segment (rare: a segment index with
      // more than RZ set bits), from memory; C^T comes from LDS again.
      unsigned mask = stream_mask;
      while (mask) {
        const int ks = __builtin_ctz(mask) + 1;
        mask &= mask - 1;
        if (MASKED && !((lmask >> (c_log + m + ks)) & 1)) continue;
        frag zcur[Tl::NKN];
        const T* zr = slot_of(h, ks) + slot_frag<T, N>(wv, 0, g, r);
#pragma unroll
        for (int kk = 0; kk < Tl::NKN; ++kk) zcur[kk] = load_frag<T>(zr + kk * 64 * Tl::KPL);
        const float eD = M::ex(gap_h[ks] + accseg);
#pragma unroll
        for (int tb = 0; tb < Tl::TB; ++tb) {
          f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Tl::NKN; ++kk)
            tmp = M::mma(zcur[kk], rows_state_frag<T, N>(csh, 16 * tb + r, kk, g), tmp);
          Y[tb] += level_scale(tb, c_log + m + ks, eD) * tmp;
        }
      }
      // Stage the tile in LDS (W is consumed; the barrier below also tells
      // that every wave has read its C^T fragments) so that each token's
      // output row leaves as whole cache lines.
#pragma unroll
      for (int tb = 0; tb < Tl::TB; ++tb) store4(wth + RX::at(16 * tb + r, 16 * wv + 4 * g), Y[tb]);
    }
    lds_barrier();
    {
      constexpr int VEC = 16 / (int)sizeof(T), NBP = P / VEC, PIECES = C * NBP;
      const T* ys = wt + hh * WTS;
#pragma unroll
      for (int pc0 = 0; pc0 < PIECES; pc0 += Cfg::NWH * 64) {
        const int pc = pc0 + wv * 64 + lane;
        if (PIECES % (Cfg::NWH * 64) == 0 || pc < PIECES) {
          const int t = pc / NBP, bb = pc % NBP;
          store16(out + ((row0 + t) * H + h) * P + bb * VEC, load16(ys + RX::at(t, bb * VEC)));
        }
      }
    }

    if (need_state) {
      issue_c(j + 1, lane);
      issue_lam(j + 1, lane);
      issue_regs(j + 1, tid);  // land during the state MFMAs
    }
    if (need_state && local_on) {
      // ---- this chunk's state, pushed on the local Fenwick stack
      f32x4 S[Tl::NB];
#pragma unroll
      for (int nb = 0; nb < Tl::NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      chunk_state_mma<T, C, P, N>(bs, xs, wst_h, S, wv, g, r);
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
    lds_barrier();  // LDS is restaged by the next chunk
    if (NBUF == 1 && need_state) issue_bx(j + 1, bs_next, xs_next, lane);
  };
  for (int jl = 0; jl < nch; jl += 2) {
    step(std::integral_constant<int, 0>{}, jl);
    if (jl + 1 < nch) step(std::integral_constant<int, 1>{}, jl + 1);
  }
}

}  // namespace loglin
