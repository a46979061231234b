// Output pass of the log-linear Mamba-2 forward for bf16, 64-token chunks
// and 64 value columns (the write-up's benchmark shape: head dim 64, state
// 64 or 128, chunk 64), laid out so that every LDS operand read is one
// lane register plus an immediate offset.
//
// What it computes is the output_kernel's (loglin_device.hpp): per chunk,
// the dense intra-chunk block (levels 0..6) and every inter-chunk level
// whose bit is set in the chunk index, fused in one pass (log-linear
// attention write-up, sections "special structure: tree partition" and
// "efficient training algorithm"; its Fig 4 level fusion).  One work-group
// per (batch, segment of 2^m chunks, head), four waves; wave w owns output
// columns [16 w, 16 w + 16) of every chunk and the same columns of every
// chunk state.
//
// LDS layouts (bank model: 64 four-byte banks; 16 lanes per cycle for
// 16-byte reads, 32 for 8-byte ones):
//   B and C rows  272-byte rows (256 bytes of data, one 16-byte pad block).
//                 The row-wise reads (scores, level products) give lane
//                 (g, r) 16 bytes of row 16 x + r at byte 64 kk + 16 g: row r
//                 starts 16 r bytes further round the banks, so the 16 lanes
//                 of a cycle hit 16 distinct 16-byte bank groups.  The
//                 transposing reads of the chunk state (rows 8 g + r / 4,
//                 bytes 8 (r mod 4) + 32 nb) meet two-way conflicts there.
//                 Contractions over the state dimension use the natural
//                 order: lane group g holds elements 32 kk + 8 g .. + 7.
//   X rows        128-byte rows, 16-byte blocks XOR-swizzled by
//                 2 (bit 1 of the row | bit 3 of the row << 1): the
//                 transposing reads (rows 8 g + r / 4 + 4 h, columns
//                 16 w + 4 (r mod 4)) are conflict-free and the key depends
//                 on lane bits only.  The output tile is staged in the same
//                 place and layout: a wave writes only the columns it read.
//   W[t][s]       128-byte rows, 16-byte blocks XOR-swizzled by
//                 (t / 2) mod 8: the row-wise operand reads and the score
//                 epilogue's writes are conflict-free.
#pragma once

#include "loglin_device.hpp"

namespace loglin {

template <int N>
struct Out2 {
  static constexpr int C = 64, P = 64, TB = 4, NW = 4, NT = 256;
  static constexpr int NKN = N / 32;  // 32-wide contraction steps over the state
  static constexpr int NB = N / 16;   // 16-row tiles of a chunk state
  static constexpr int BROW = 2 * N + 16;           // bytes per B / C row in LDS
  static constexpr int BBLK = BROW / 16;            // 16-byte blocks per row (last: pad)
  static constexpr int BINST = C * BBLK / 64;       // copy instructions per B / C tile
  static constexpr int BINST_W = (BINST + NW - 1) / NW;
  static constexpr int XINST = C * P * 2 / 1024;    // copy instructions per X tile
  static constexpr int XINST_W = XINST / NW;
  static_assert(C * BBLK % 64 == 0, "B / C tiles fill whole copy instructions");
  static_assert(XINST % NW == 0, "X tiles split evenly over the waves");
};

// 8 bytes of LDS at a byte address (ds_read_b64)
__device__ inline bf16x4 lds_read8(const unsigned char* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}
// transposing 8-byte read (ds_read_b64_tr_b16)
__device__ inline bf16x4 lds_read8_tr(const unsigned char* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16* lp;
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(void*)p));
}
__device__ inline bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// bf16 weight at a byte address of LDS, as fp32
__device__ inline float lds_bf16(const unsigned char* p) {
  return __uint_as_float((unsigned)*reinterpret_cast<const unsigned short*>(p) << 16);
}
__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float LOG2E = 1.4426950408889634f;

// Score tiles of a 64-token chunk dealt to the four waves: the diagonal
// tile (w, w) and, below it, (1,0) (2,0) | (2,1) (3,0) | (3,1) | (3,2); the
// two upper tiles W X reads as zeros, (0,1) and (2,3), go to waves 2 and 3.
// Entry: tb * 4 + sb, with tb < sb marking a zero tile.
template <int W>
struct WaveTiles;
template <>
struct WaveTiles<0> {
  static constexpr int n = 3;
  static constexpr int t[3] = {0, 4, 8};  // D(0,0) L(1,0) L(2,0)
};
template <>
struct WaveTiles<1> {
  static constexpr int n = 3;
  static constexpr int t[3] = {5, 9, 12};  // D(1,1) L(2,1) L(3,0)
};
template <>
struct WaveTiles<2> {
  static constexpr int n = 3;
  static constexpr int t[3] = {10, 13, 1};  // D(2,2) L(3,1) Z(0,1)
};
template <>
struct WaveTiles<3> {
  static constexpr int n = 3;
  static constexpr int t[3] = {15, 14, 11};  // D(3,3) L(3,2) Z(2,3)
};

template <int N, bool MASKED>
__global__ __launch_bounds__(256, 2) void output2_kernel(Params pr) {
  using O = Out2<N>;
  using M = Mfma<bf16>;
  using frag = bf16x8;
  constexpr int C = O::C, P = O::P, TB = O::TB, NKN = O::NKN, NB = O::NB;
  constexpr int BROW = O::BROW, BBLK = O::BBLK;
  constexpr int MM = MAX_SEG_LOG2;  // levels inside a segment (local stack)
  constexpr int RZ = 3;             // level slots above the segment held in registers
  constexpr int GS = MAX_DEPTH + 1;
  __shared__ __attribute__((aligned(16))) unsigned char bsh0[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char bsh1[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char csh[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char xsh0[C * P * 2];
  __shared__ __attribute__((aligned(16))) unsigned char xsh1[C * P * 2];
  __shared__ __attribute__((aligned(16))) unsigned char wsh[C * C * 2];
  // per-token decays, by chunk parity (a chunk's last reads of them and the
  // next chunk's writes need no barrier between them)
  __shared__ __attribute__((aligned(16))) float c2s2[2][C], e2s2[2][C], w2s2[2][C];
  __shared__ float gap_s[GS];
  extern __shared__ unsigned lam_w[];  // [C][LW] level weights, 32-bit words

  // Work-group -> (segment, head).  The hardware deals work-groups to the 8
  // XCDs round-robin by id.  XCD x takes its u-th group of 8 segments
  // (counted from the last) at offset (u + x) mod 8, so over u every XCD
  // meets every offset and every group: the same mix of segment indices,
  // whose set bits decide a segment's level count, the longest first.  It
  // runs all heads of a segment in turn, heads of one group next to each
  // other (they read the same B and C rows), so the work-groups running
  // together on an XCD cover every head of one or two segments and share
  // each token's log-decay and level-weight lines (a 128-byte line holds
  // 32 heads' log-decays).
  const int H = pr.nheads;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int ng8 = (pr.ns + 7) >> 3;  // groups of 8 segments per batch entry
  const int slot = kx / H;
  const int b = slot / ng8, u = slot % ng8;
  const int qd = 8 * u + ((u + xcd) & 7);  // segment, counted from the last
  if (b >= pr.batch || qd >= pr.ns) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int G = pr.ngroups, L = pr.nlevels, LL = pr.ll;
  const int LW = lam_words(LL, 2);
  const int hpg = H / G;
  const int h = kx % H;
  const int grp = h / hpg;
  const int q = pr.ns - 1 - qd;
  const int bh = b * H + h;
  const int c_log = 6;
  const int m = pr.m;
  const int seg = 1 << m;
  const int j0 = q * seg;
  const int nch = min(seg, pr.nc - j0);
  const bf16* Xg = static_cast<const bf16*>(pr.X);
  const bf16* Bg = static_cast<const bf16*>(pr.Bm);
  const bf16* Cg = static_cast<const bf16*>(pr.Cm);
  const bf16* slots = static_cast<const bf16*>(pr.slots);
  bf16* outg = static_cast<bf16*>(pr.out);

  // ---- lane constants (byte offsets into the LDS tiles)
  // B / C row-wise reads: + 16 x BROW + 64 kk
  const unsigned o_row = r * BROW + 16 * g;
  // B^T transposing reads: + (32 kt + 4 hh) BROW + 32 nb
  const unsigned o_bt = (8 * g + (r >> 2)) * BROW + 8 * (r & 3);
  // X^T transposing reads: + (32 kt + 4 hh) 128
  const int keyx = ((r >> 3) & 1) | ((g & 1) << 1);
  const unsigned o_xt = (8 * g + (r >> 2)) * 128 + 16 * ((2 * wv + ((r & 3) >> 1)) ^ (2 * keyx)) +
                        8 * (r & 1);
  // output tile staged in X's layout: row 16 tb + r, columns 16 wv + 4 g
  const int keyy = ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
  const unsigned o_yst = r * 128 + 16 * ((2 * wv + (g >> 1)) ^ (2 * keyy)) + 8 * (g & 1);
  // W reads (row 16 tb + r, 16-byte block 4 kt + g): + 2048 tb
  const int kw = (r >> 1) & 7;
  const unsigned o_w0 = r * 128 + 16 * (g ^ kw);
  const unsigned o_w1 = r * 128 + 16 * ((4 + g) ^ kw);
  // level weights of token r of a token block: + 4 LW 16 tb + 2 level.  The
  // row of token t starts in the upper half of its first word when its
  // element offset ((row0 + t) H + h) L is odd; row0 is even.
  const int lpar = L & 1;
  const int par = lpar & ((r & H) ^ h);
  const unsigned o_lam = 4u * LW * r + 2u * par;

  // copy pieces: lane byte offsets from the chunk's first row (a pad block
  // repeats the row's last block)
  const unsigned rs_bc = (unsigned)G * N * 2, rs_x = (unsigned)H * P * 2;
  auto cbc_off = [&](int k) __attribute__((always_inline)) {
    const unsigned pos = (unsigned)((wv + 4 * k) * 64 + lane);
    const unsigned rho = pos / BBLK;
    const unsigned blk = min(pos - rho * BBLK, (unsigned)(BBLK - 2));
    return __umul24(rho, rs_bc) + 16u * blk;
  };
  auto cx_off = [&](int k) __attribute__((always_inline)) {
    const int pos = (wv + 4 * k) * 64 + lane;
    const int rho = pos >> 3, phys = pos & 7;
    const int key = ((rho >> 1) & 1) | (((rho >> 3) & 1) << 1);
    return __umul24((unsigned)rho, rs_x) + 16u * (phys ^ (2 * key));
  };
  auto issue_bx = [&](int j, unsigned char* bs, unsigned char* xs) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const bf16* bsrc = Bg + (r0 * G + grp) * N;
    const bf16* xsrc = Xg + (r0 * H + h) * P;
#pragma unroll
    for (int k = 0; k < O::BINST_W; ++k)
      if (O::BINST % 4 == 0 || wv + 4 * k < O::BINST)
        dma_16x64_at(bsrc, cbc_off(k), lds_addr(bs) + (wv + 4 * k) * 1024u);
#pragma unroll
    for (int k = 0; k < O::XINST_W; ++k) dma_16x64_at(xsrc, cx_off(k), lds_addr(xs) + (wv + 4 * k) * 1024u);
  };
  auto issue_c = [&](int j) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const bf16* csrc = Cg + (r0 * G + grp) * N;
#pragma unroll
    for (int k = 0; k < O::BINST_W; ++k)
      if (O::BINST % 4 == 0 || wv + 4 * k < O::BINST)
        dma_16x64_at(csrc, cbc_off(k), lds_addr(csh) + (wv + 4 * k) * 1024u);
  };
  // level weights of chunk j into lam_w (see output_kernel: the last word of
  // the tensor bounds the copy)
  const int64_t lam_last_word = ((int64_t)pr.batch * pr.seqlen * H * L * 2 - 4) / 4;
  const float inv_lw = 1.f / (float)LW;
  auto issue_lam = [&](int j) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const int64_t eb = (r0 * H + h) * L;
    const int64_t wb = eb >> 1;
    const int par0 = (int)(eb & 1);
    const unsigned* base = static_cast<const unsigned*>(pr.lam) + wb;
    const unsigned lim = (unsigned)min(lam_last_word - wb, (int64_t)0x7fffffff);
    const int words = C * LW;
    for (int inst = wv; inst * 64 < words; inst += 4) {
      const int idx = inst * 64 + lane;
      if (idx < words) {
        const int t = (int)(((float)idx + 0.5f) * inv_lw), w = idx - t * LW;
        const int x = (int)__umul24((unsigned)t, (unsigned)(H * L));
        unsigned ow = (unsigned)(((x + par0) >> 1) + w);
        ow = ow < lim ? ow : lim;
        dma_4x64_at(base, ow * 4u, lds_addr(lam_w) + inst * 256u);
      }
    }
  };
  float la = 0.f;
  auto load_la = [&](int j) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    la = (wv == 3) ? pr.log_a[(r0 + lane) * H + h] : 0.f;
  };

  // ---- level bookkeeping (see output_kernel)
  frag zl[MM][NKN];  // local Fenwick stack, entry e: the 2^e chunks before
  float zla[MM];
  float dloc[MM + 1];
#pragma unroll
  for (int e = 0; e < MM; ++e) zla[e] = 0.f;
#pragma unroll
  for (int k = 0; k <= MM; ++k) dloc[k] = 0.f;
  float accseg = 0.f;
  if (pr.ks > 0)
    for (int i = tid; i < pr.ks + 1; i += 256)
      gap_s[i] = pr.gap_decay[((int64_t)bh * pr.ns + q) * (pr.ks + 1) + i];
  const unsigned ext_mask = (unsigned)q & ((1u << pr.ks) - 1u);
  auto slot_of = [&](int ks) __attribute__((always_inline)) {
    const int qs = ((q >> ks) << ks) + (1 << (ks - 1)) - 1;
    return slots + ((int64_t)bh * pr.ns + qs) * P * N;
  };
  unsigned stream_mask = ext_mask;
#pragma unroll
  for (int i = 0; i < RZ; ++i) stream_mask &= stream_mask - 1;
  frag zres[RZ][NKN];
  int lres[RZ];
  const int nres = min(__builtin_popcount(ext_mask), RZ);
  {
    unsigned mk = ext_mask;
#pragma unroll
    for (int i = 0; i < RZ; ++i) {
      const int ks = mk ? __builtin_ctz(mk) + 1 : 1;
      lres[i] = c_log + m + ks;
      if (mk) {
        const bf16* zr = slot_of(ks) + slot_frag<bf16, N>(wv, 0, g, r);
#pragma unroll
        for (int kk = 0; kk < NKN; ++kk) zres[i][kk] = load_frag<bf16>(zr + kk * 64 * 8);
      } else {
#pragma unroll
        for (int kk = 0; kk < NKN; ++kk) zres[i][kk] = frag{};
      }
      mk &= mk - 1;
    }
  }
  const unsigned long long lmask = MASKED ? pr.lmask : ~0ull;
  const bool intra_on = !MASKED || (lmask & 0x7full) != 0;
  const bool local_on = !MASKED || ((lmask >> 7) & ((1ull << m) - 1)) != 0;

  // diagonal score tiles: level bit_length(r ^ s) and causality s <= r of
  // the lane's four elements s = 4 g + i, the same in every diagonal tile
  unsigned o_dl[4];
  unsigned long long keep[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 4 * g + i;
    o_dl[i] = o_lam + 2u * (unsigned)bit_length((unsigned)(r ^ s));
    keep[i] = __ballot(s <= r);
  }

  issue_bx(j0, bsh0, xsh0);
  issue_c(j0);
  issue_lam(j0);
  load_la(j0);

  // one chunk; Q = jl mod 4 (jl's low bits fix which local levels it reads
  // and where it pushes its state), CUR = jl mod 2 (the buffer parity)
  auto step = [&](auto q_c, int jl) __attribute__((always_inline)) {
    constexpr int Q = decltype(q_c)::value;
    constexpr int CUR = Q & 1;
    unsigned char* bs = CUR ? bsh1 : bsh0;
    unsigned char* xs = CUR ? xsh1 : xsh0;
    const int j = j0 + jl;
    const int64_t row0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const bool has_next = jl + 1 < nch;
    float* c2s = c2s2[CUR];
    float* e2s = e2s2[CUR];
    float* w2s = w2s2[CUR];

    // ---- chunk decays (last wave): log2-scaled prefix sums, e^Lambda_t and
    // the decay from t to the chunk end
    if (wv == 3) {
      const float v = wave_prefix_sum<C>(la) * LOG2E;
      const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), C - 1));
      c2s[lane] = v;
      e2s[lane] = fexp2(v);
      w2s[lane] = fexp2(tot - v);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the chunk have landed
    lds_barrier();
    if (has_next) issue_bx(j + 1, CUR ? bsh0 : bsh1, CUR ? xsh0 : xsh1);
    const float atot = c2s[C - 1] * (1.f / LOG2E);  // chunk log-decay (natural log)

    // ---- scores B C^T of this wave's tiles, masked into W[t][s]
    if (intra_on) {
      auto tiles = [&](auto wc) __attribute__((always_inline)) {
        using WT = WaveTiles<decltype(wc)::value>;
#pragma unroll
        for (int u = 0; u < WT::n; ++u) {
          const int tb = WT::t[u] >> 2, sb = WT::t[u] & 3;
          unsigned char* wrow = wsh + (16 * tb + r) * 128 + 8 * (g & 1);
          const int wblk = (2 * sb + (g >> 1)) ^ kw;
          if (tb < sb) {  // upper tile read as zeros by W X
            *reinterpret_cast<bf16x4*>(wrow + 16 * wblk) = bf16x4{};
            continue;
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKN; ++kk) {
            const unsigned char* pb = bs + o_row + 16 * sb * BROW + 64 * kk;
            const unsigned char* pc = csh + o_row + 16 * tb * BROW + 64 * kk;
            acc = M::mma(*reinterpret_cast<const frag*>(pb), *reinterpret_cast<const frag*>(pc), acc);
          }
          // lane (g, r): t = 16 tb + r, s = 16 sb + 4 g + i
          const float ct = c2s[16 * tb + r];
          const f32x4 cs = *reinterpret_cast<const f32x4*>(&c2s[16 * sb + 4 * g]);
          const unsigned char* lrow = reinterpret_cast<const unsigned char*>(lam_w) + 64u * LW * tb;
          f32x4 wv4;
          if (tb > sb) {
            // t XOR s = 16 (tb XOR sb) + (r XOR s mod 16): one level for the tile
            const int lev = 4 + bit_length((unsigned)(tb ^ sb));
            const float lt = (!MASKED || ((lmask >> lev) & 1)) ? lds_bf16(lrow + o_lam + 2 * lev) : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv4[i] = acc[i] * fexp2(ct - cs[i]) * lt;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float lt = lds_bf16(lrow + o_dl[i]);
              if constexpr (MASKED) {
                const int lev = bit_length((unsigned)(r ^ (4 * g + i)));
                lt = ((lmask >> lev) & 1) ? lt : 0.f;
              }
              const float v = acc[i] * fexp2(ct - cs[i]) * lt;
              wv4[i] = ((keep[i] >> lane) & 1) ? v : 0.f;
            }
          }
          bf16x4 o4 = {(bf16)wv4[0], (bf16)wv4[1], (bf16)wv4[2], (bf16)wv4[3]};
          *reinterpret_cast<bf16x4*>(wrow + 16 * wblk) = o4;
        }
      };
      switch (wv) {
        case 0: tiles(std::integral_constant<int, 0>{}); break;
        case 1: tiles(std::integral_constant<int, 1>{}); break;
        case 2: tiles(std::integral_constant<int, 2>{}); break;
        default: tiles(std::integral_constant<int, 3>{}); break;
      }
    }
    lds_barrier();

    // ---- X^T fragments of this wave's columns (W X and the chunk state)
    frag xt[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const unsigned char* p = xs + o_xt + 32 * kt * 128;
      xt[kt] = cat8(lds_read8_tr(p), lds_read8_tr(p + 4 * 128));
    }
    // ---- intra block: Y^T = X^T W^T
    f32x4 Y[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      Y[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (intra_on) {
        Y[tb] = M::mma(xt[0], *reinterpret_cast<const frag*>(wsh + o_w0 + 2048 * tb), Y[tb]);
        if (tb >= 2) Y[tb] = M::mma(xt[1], *reinterpret_cast<const frag*>(wsh + o_w1 + 2048 * tb), Y[tb]);
      }
    }

    // ---- inter-chunk levels, two token blocks at a time: C^T fragments of
    // the pair are read once and serve every level
    float eres[RZ];
#pragma unroll
    for (int i = 0; i < RZ; ++i) eres[i] = __expf(gap_s[lres[i] - c_log - m] + accseg);
    float eloc[MM];
#pragma unroll
    for (int e = 0; e < MM; ++e) eloc[e] = __expf(dloc[e + 1]);
    const unsigned char* lam_b = reinterpret_cast<const unsigned char*>(lam_w);
    frag cf[2][NKN];
    float e2t[2];
    auto load_cf = [&](int half) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tb = 2 * half + u;
#pragma unroll
        for (int kk = 0; kk < NKN; ++kk) {
          cf[u][kk] = *reinterpret_cast<const frag*>(csh + o_row + 16 * tb * BROW + 64 * kk);
        }
        e2t[u] = e2s[16 * tb + r];
      }
    };
    // one level's product for token blocks 2 half and 2 half + 1
    auto level = [&](const frag(&z)[NKN], int lev, float eD, int half) __attribute__((always_inline)) {
      const unsigned char* lp = lam_b + o_lam + 2 * lev;
      f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKN; ++kk) {
        t0 = M::mma(z[kk], cf[0][kk], t0);
        t1 = M::mma(z[kk], cf[1][kk], t1);
      }
      const float s0 = lds_bf16(lp + 64u * LW * (2 * half)) * (e2t[0] * eD);
      const float s1 = lds_bf16(lp + 64u * LW * (2 * half + 1)) * (e2t[1] * eD);
      Y[2 * half] += s0 * t0;
      Y[2 * half + 1] += s1 * t1;
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      load_cf(half);
#pragma unroll
      for (int i = 0; i < RZ; ++i)
        if (i < nres && (!MASKED || ((lmask >> lres[i]) & 1))) level(zres[i], lres[i], eres[i], half);
#pragma unroll
      for (int e = 0; e < MM; ++e)
        if (e < m && (e < 2 ? ((Q >> e) & 1) != 0 : ((jl >> e) & 1) != 0) &&
            (!MASKED || ((lmask >> (c_log + e + 1)) & 1)))
          level(zl[e], c_log + e + 1, eloc[e], half);
    }
    // levels above the segment past the resident ones (a segment index with
    // more than RZ set bits): each slot is fetched once per chunk, the C^T
    // fragments are read from LDS again
    {
      unsigned mask = stream_mask;
      while (mask) {
        const int ks = __builtin_ctz(mask) + 1;
        mask &= mask - 1;
        if (MASKED && !((lmask >> (c_log + m + ks)) & 1)) continue;
        frag zc[NKN];
        const bf16* zr = slot_of(ks) + slot_frag<bf16, N>(wv, 0, g, r);
#pragma unroll
        for (int kk = 0; kk < NKN; ++kk) zc[kk] = load_frag<bf16>(zr + kk * 64 * 8);
        const float eD = __expf(gap_s[ks] + accseg);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          load_cf(half);
          level(zc, c_log + m + ks, eD, half);
        }
      }
    }

    // ---- stage the output tile in X's place (this wave's columns only)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      bf16x4 o4 = {(bf16)Y[tb][0], (bf16)Y[tb][1], (bf16)Y[tb][2], (bf16)Y[tb][3]};
      *reinterpret_cast<bf16x4*>(xs + o_yst + 2048 * tb) = o4;
    }
    lds_barrier();  // every wave has staged its columns and read C, W, lambda
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pos = (wv + 4 * k) * 64 + lane;  // 16-byte piece of the tile
      const int t = pos >> 3, phys = pos & 7;
      const int key = ((t >> 1) & 1) | (((t >> 3) & 1) << 1);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(xs + pos * 16);
      *reinterpret_cast<bf16x8*>(outg + ((row0 + t) * H + h) * P + 8 * (phys ^ (2 * key))) = v;
    }
    if (has_next) {
      issue_c(j + 1);
      issue_lam(j + 1);
      load_la(j + 1);
    }

    // ---- this chunk's state, pushed on the local Fenwick stack
    if (has_next && local_on) {
      f32x4 S[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // X rows scaled by the decay to the chunk end: token 32 kt + 8 g + jj
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(&w2s[32 * kt + 8 * g]);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(&w2s[32 * kt + 8 * g + 4]);
        frag xw;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          xw[jj] = (bf16)((float)xt[kt][jj] * w0[jj]);
          xw[jj + 4] = (bf16)((float)xt[kt][jj + 4] * w1[jj]);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const unsigned char* p = bs + o_bt + 32 * kt * BROW + 32 * nb;
          S[nb] = M::mma(cat8(lds_read8_tr(p), lds_read8_tr(p + 4 * BROW)), xw, S[nb]);
          if (nb % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      // The state MFMA leaves lane (g, r) rows 16 nb + 4 g + i of column
      // 16 wv + r.  A natural-order fragment of step kk needs rows 32 kk +
      // 8 g .. + 7: rows 8 (g mod 2) + j of tile 2 kk + g / 2, which lane
      // groups 2 (g mod 2) and 2 (g mod 2) + 1 hold.  Two lane swaps per
      // register pair move them there: the upper 32 lanes of tile 2 kk with
      // the lower 32 of tile 2 kk + 1, then the odd 16-lane rows of the first
      // register with the even rows of the second.
      f32x4 Sn[NKN][2];  // natural order: [kk][j / 4][j mod 4]
#pragma unroll
      for (int kk = 0; kk < NKN; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(S[2 * kk][i]),
                                                            __float_as_uint(S[2 * kk + 1][i]), false, false);
          const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
          Sn[kk][0][i] = __uint_as_float(s16[0]);
          Sn[kk][1][i] = __uint_as_float(s16[1]);
        }
      // merge with the entries of the blocks this chunk completes
      // trailing ones of jl: fixed by Q while a next chunk exists (a segment
      // has at most 8 chunks, so jl = 7 has none)
      constexpr int z = Q == 1 ? 1 : (Q == 3 ? 2 : 0);
      float cur_a = atot;
#pragma unroll
      for (int e = 0; e < MM; ++e) {
        if (e < z) {
          const float dec = __expf(cur_a);
#pragma unroll
          for (int kk = 0; kk < NKN; ++kk)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) Sn[kk][jj >> 2][jj & 3] += dec * (float)zl[e][kk][jj];
          cur_a += zla[e];
        }
      }
#pragma unroll
      for (int e = 0; e < MM; ++e) {
        if (e == z) {
#pragma unroll
          for (int kk = 0; kk < NKN; ++kk)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) zl[e][kk][jj] = (bf16)Sn[kk][jj >> 2][jj & 3];
          zla[e] = cur_a;
        }
      }
    }

    // ---- running log-decays for the next chunk
    accseg += atot;
#pragma unroll
    for (int k = 1; k <= MM; ++k) {
      dloc[k] += atot;
      if (((Q + 1) & ((1 << (k - 1)) - 1)) == 0) dloc[k] = 0.f;
    }
    // No barrier here: the next chunk writes only the other parity's decays
    // before its first barrier, and every tile it overwrites after that
    // barrier was last read before this chunk's staging barrier or, for B
    // and X, two chunks back.
  };
  for (int jl = 0; jl < nch; jl += 4) {
    step(std::integral_constant<int, 0>{}, jl);
    if (jl + 1 < nch) step(std::integral_constant<int, 1>{}, jl + 1);
    if (jl + 2 < nch) step(std::integral_constant<int, 2>{}, jl + 2);
    if (jl + 3 < nch) step(std::integral_constant<int, 3>{}, jl + 3);
  }
}

// State pass for the same shape, in the output pass's LDS layouts: the
// transposing reads of B (272-byte rows) and X (128-byte rows, lane-keyed
// swizzle) are a lane base plus an immediate, so the only per-chunk address
// work is the copies'.  One work-group per (batch, segment, two heads of a
// group), eight waves: wave w serves head w / 4 and its state columns
// [16 (w mod 4), +16), all N rows.  The heads share one copy of the B rows.
// The segment's log-decays are copied once, up front, and each chunk's
// decays are formed while the chunk before it is being reduced; the states
// go out through LDS, whole 128-byte lines at a time.
// What it computes is state_kernel's (loglin_device.hpp): each segment's
// state, decayed to the segment's end, in natural row order, and the
// segment's log-decay.
template <int N>
__global__ __launch_bounds__(512, 2) void state2_kernel(Params pr) {
  using O = Out2<N>;
  using M = Mfma<bf16>;
  constexpr int C = O::C, P = O::P, NB = O::NB, BROW = O::BROW, BBLK = O::BBLK, BINST = O::BINST;
  constexpr int NWT = 8;
  constexpr int SEG = 1 << MAX_SEG_LOG2;
  constexpr int SROW = 2 * N + 16;  // bytes per staged state row (one pad block)
  static_assert(P * SROW <= C * BROW, "a head's state fits one B buffer");
  __shared__ __attribute__((aligned(16))) unsigned char bsh0[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char bsh1[C * BROW];
  __shared__ __attribute__((aligned(16))) unsigned char xsh0[2][C * P * 2];
  __shared__ __attribute__((aligned(16))) unsigned char xsh1[2][C * P * 2];
  // per head: the segment's log-decays, and the chunk decays by chunk parity
  __shared__ __attribute__((aligned(16))) float las[2][SEG * C];
  __shared__ __attribute__((aligned(16))) float cum[2][2][C], ecum[2][2][C], wst[2][2][C];

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= pr.total) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NWT);
  const int hh = wave >> 2, wv = wave & 3;
  const int g = lane >> 4, r = lane & 15;
  const int H = pr.nheads, G = pr.ngroups;
  // heads of one group next to each other, then groups, then segments (as
  // state_kernel)
  const int hpg = H / G, npair = hpg / 2;
  const int pi = tile % npair;
  const int grp = (tile / npair) % G;
  const int q = (tile / (npair * G)) % pr.ns;
  const int b = tile / (npair * G * pr.ns);
  const int h0 = grp * hpg + pi * 2;
  const int h = h0 + hh;
  const int bh = b * H + h;
  const int seg = 1 << pr.m;
  const int j0 = q * seg;
  const int nch = min(seg, pr.nc - j0);
  const bf16* Xg = static_cast<const bf16*>(pr.X);
  const bf16* Bg = static_cast<const bf16*>(pr.Bm);

  // B^T transposing reads: + (32 kt + 4 hh) BROW + 32 nb
  const unsigned o_bt = (8 * g + (r >> 2)) * BROW + 8 * (r & 3);
  // X^T transposing reads: + (32 kt + 4 hh) 128
  const int keyx = ((r >> 3) & 1) | ((g & 1) << 1);
  const unsigned o_xt = (8 * g + (r >> 2)) * 128 + 16 * ((2 * wv + ((r & 3) >> 1)) ^ (2 * keyx)) +
                        8 * (r & 1);
  // copy pieces (byte offsets from the chunk's first row; a B pad block
  // repeats the row's last block)
  const unsigned rs_bc = (unsigned)G * N * 2, rs_x = (unsigned)H * P * 2;
  auto cbc_off = [&](int inst) __attribute__((always_inline)) {
    const unsigned pos = (unsigned)(inst * 64 + lane);
    const unsigned rho = pos / BBLK;
    const unsigned blk = min(pos - rho * BBLK, (unsigned)(BBLK - 2));
    return __umul24(rho, rs_bc) + 16u * blk;
  };
  auto cx_off = [&](int k) __attribute__((always_inline)) {
    const int pos = (wv + 4 * k) * 64 + lane;
    const int rho = pos >> 3, phys = pos & 7;
    const int key = ((rho >> 1) & 1) | (((rho >> 3) & 1) << 1);
    return __umul24((unsigned)rho, rs_x) + 16u * (phys ^ (2 * key));
  };
  auto issue = [&](int j, unsigned char* bs, unsigned char (*xs)[C * P * 2]) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)b * pr.seqlen + (int64_t)j * C;
    const bf16* bsrc = Bg + (r0 * G + grp) * N;
    const bf16* xsrc = Xg + (r0 * H + h) * P;
#pragma unroll
    for (int k = 0; k < (BINST + NWT - 1) / NWT; ++k)
      if (BINST % NWT == 0 || wave + NWT * k < BINST)
        dma_16x64_at(bsrc, cbc_off(wave + NWT * k), lds_addr(bs) + (wave + NWT * k) * 1024u);
#pragma unroll
    for (int k = 0; k < O::XINST_W; ++k) dma_16x64_at(xsrc, cx_off(k), lds_addr(xs[hh]) + (wv + 4 * k) * 1024u);
  };

  // the segment's log-decays of this head: wave 0 copies chunk k's, lane t
  // token t (one 4-byte element per lane)
  if (wv == 0) {
    const float* lsrc = pr.log_a + ((int64_t)b * pr.seqlen + (int64_t)j0 * C) * H + h;
#pragma unroll
    for (int k = 0; k < SEG; ++k)
      if (k < nch) dma_4x64_at(lsrc, (unsigned)((k * C + lane) * H) * 4u, lds_addr(&las[hh][k * C]));
  }
  f32x4 S[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) S[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float seg_sum = 0.f;
  issue(j0, bsh0, xsh0);
  auto step = [&](auto cur_c, int jl) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value;
    const unsigned char* bs = CUR ? bsh1 : bsh0;
    const unsigned char* xs = CUR ? xsh1[hh] : xsh0[hh];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the chunk have landed
    if (jl == 0 && wv == 0)  // (later chunks' decays are formed a step ahead)
      chunk_decays<bf16, C>(las[hh][lane], cum[hh][0], ecum[hh][0], wst[hh][0], lane);
    lds_barrier();
    if (jl + 1 < nch)  // the other buffers were released by the previous barrier
      issue(j0 + jl + 1, CUR ? bsh0 : bsh1, CUR ? xsh0 : xsh1);
    const float atot = cum[hh][CUR][C - 1];
    if (jl > 0) {
      const float dec = M::ex(atot);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) S[nb] *= dec;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // X rows scaled by the decay to the chunk end: token 32 kt + 8 g + jj
      const unsigned char* px = xs + o_xt + 32 * kt * 128;
      const bf16x8 xt = cat8(lds_read8_tr(px), lds_read8_tr(px + 4 * 128));
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wst[hh][CUR][32 * kt + 8 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wst[hh][CUR][32 * kt + 8 * g + 4]);
      bf16x8 xw;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        xw[jj] = (bf16)((float)xt[jj] * w0[jj]);
        xw[jj + 4] = (bf16)((float)xt[jj + 4] * w1[jj]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const unsigned char* pb = bs + o_bt + 32 * kt * BROW + 32 * nb;
        S[nb] = M::mma(cat8(lds_read8_tr(pb), lds_read8_tr(pb + 4 * BROW)), xw, S[nb]);
      }
    }
    if (jl + 1 < nch && wv == 0)
      chunk_decays<bf16, C>(las[hh][(jl + 1) * C + lane], cum[hh][CUR ^ 1], ecum[hh][CUR ^ 1],
                            wst[hh][CUR ^ 1], lane);
    seg_sum += atot;
    lds_barrier();
  };
  for (int jl = 0; jl < nch; jl += 2) {
    step(std::integral_constant<int, 0>{}, jl);
    if (jl + 1 < nch) step(std::integral_constant<int, 1>{}, jl + 1);
  }

  // The state in natural row order (row n of column p at p N + n), staged
  // in the B buffers (one per head; the last barrier released them) and
  // written out in whole rows.
  unsigned char* stg = hh ? bsh1 : bsh0;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16x4 o4 = {(bf16)S[nb][0], (bf16)S[nb][1], (bf16)S[nb][2], (bf16)S[nb][3]};
    *reinterpret_cast<bf16x4*>(stg + (16 * wv + r) * SROW + 2 * (16 * nb + 4 * g)) = o4;
  }
  lds_barrier();
  constexpr int RB = 2 * N / 16;  // 16-byte blocks per state row
  unsigned char* dst = reinterpret_cast<unsigned char*>(static_cast<bf16*>(pr.seg_state) +
                                                        ((int64_t)bh * pr.ns + q) * (P * N));
#pragma unroll
  for (int k = 0; k < P * RB / 256; ++k) {
    const int piece = (wv + 4 * k) * 64 + lane;  // this head's 16-byte pieces
    const int p = piece / RB, blk = piece % RB;
    *reinterpret_cast<bf16x8*>(dst + piece * 16) = *reinterpret_cast<const bf16x8*>(stg + p * SROW + 16 * blk);
  }
  if (wv == 0 && lane == 0) pr.seg_decay[(int64_t)bh * pr.ns + q] = seg_sum;
}

}  // namespace loglin
