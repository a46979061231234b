// Host side of the C ABI declared in include/loglin.h: argument checks,
// workspace plan and dispatch to the (io type, chunk, P, N) instantiation.
// Every check runs before the first HIP call.
#include "loglin.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "loglin_bwd.hpp"
#include "loglin_decode.hpp"
#include "loglin_gdn.hpp"
#include "loglin_launch.hpp"

namespace {

using loglin::Params;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_log2(int64_t x) {
  int k = 0;
  while ((int64_t(1) << k) < x) ++k;
  return k;
}

bool supported_shape(int dtype, int64_t P, int64_t N) {
  const bool p_ok = P == 16 || P == 32 || P == 64;
  const bool n_ok = N == 32 || N == 64 || N == 128 || (dtype == LOGLIN_F32 && N == 16);
  return p_ok && n_ok;
}

struct Plan {
  int nc, kc, m, ns, ks, ll, hp;
  size_t off_state, off_decay, off_slots, off_gap, bytes;
};

int check_dims(const loglin_dims* d, int chunk, const loglin_opts* o, Plan* pl) {
  if (!d) return LOGLIN_ERR_NULL;
  if (d->reserved != 0) return LOGLIN_ERR_DIM;
  if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->ngroups <= 0 ||
      d->headdim <= 0 || d->dstate <= 0 || d->nlevels <= 0)
    return LOGLIN_ERR_DIM;
  if (d->io_dtype != LOGLIN_F32 && d->io_dtype != LOGLIN_BF16) return LOGLIN_ERR_DTYPE;
  if (chunk != 16 && chunk != 32 && chunk != 64) return LOGLIN_ERR_CHUNK;
  if (d->seqlen % chunk) return LOGLIN_ERR_SEQ_CHUNK;
  if (d->nheads % d->ngroups) return LOGLIN_ERR_GROUPS;
  // Limits of the int32 index math and of the launch grids.
  if (d->seqlen > (int64_t(1) << 30) || d->nheads > 4096 || d->nlevels > 64 ||
      d->batch * d->nheads > 65535)
    return LOGLIN_ERR_DIM;
  const int64_t nc = d->seqlen / chunk;
  if (d->batch * nc * d->nheads > (int64_t(1) << 30)) return LOGLIN_ERR_DIM;
  if (d->nlevels < ceil_log2(d->seqlen) + 1) return LOGLIN_ERR_LEVELS;
  if (!supported_shape(d->io_dtype, d->headdim, d->dstate)) return LOGLIN_ERR_SHAPE;

  // A chunk count that is not a power of two needs no special case: every
  // block a chunk reads lies before it.
  const int kc = ceil_log2(nc);
  int m = kc < loglin::MAX_SEG_LOG2 ? kc : loglin::MAX_SEG_LOG2;
  // heads of one group per output work-group: one unless asked for two
  // (two measured slower on the 32K workload)
  const bool pairs_ok = d->io_dtype == LOGLIN_BF16 && d->headdim == 64 &&
                        (d->nheads / d->ngroups) % 2 == 0;
  int hp = 1;
  if (o) {
    if (o->heads_per_block < 0 || o->heads_per_block > 2) return LOGLIN_ERR_OPTS;
    if (o->heads_per_block == 2 && !pairs_ok) return LOGLIN_ERR_OPTS;
    if (o->heads_per_block > 0) hp = o->heads_per_block;
    if (o->seg_log2 < -1 || o->seg_log2 > loglin::MAX_SEG_LOG2) return LOGLIN_ERR_OPTS;
    if (o->seg_log2 > kc) return LOGLIN_ERR_OPTS;
    if (o->seg_log2 >= 0) m = o->seg_log2;
  }
  const int64_t ns = (nc + (int64_t(1) << m) - 1) >> m;
  const int ks = ceil_log2(ns);
  if (ks > loglin::MAX_DEPTH) return LOGLIN_ERR_DIM;

  pl->nc = (int)nc;
  pl->kc = kc;
  pl->m = m;
  pl->ns = (int)ns;
  pl->ks = ks;
  pl->ll = ceil_log2(d->seqlen) + 1;
  pl->hp = hp;
  const size_t bh = (size_t)(d->batch * d->nheads);
  const size_t pn = (size_t)(d->headdim * d->dstate);
  const size_t esz = d->io_dtype == LOGLIN_BF16 ? 2 : 4;
  size_t off = 0;
  if (ns > 1) {  // levels above one segment exist
    pl->off_state = off;
    off = round_up(off + bh * ns * pn * esz);
    pl->off_decay = off;
    off = round_up(off + bh * ns * sizeof(float));
    pl->off_slots = off;
    off = round_up(off + bh * ns * pn * esz);
    pl->off_gap = off;
    off = round_up(off + bh * ns * (ks + 1) * sizeof(float));
  } else {
    pl->off_state = pl->off_decay = pl->off_slots = pl->off_gap = 0;
  }
  pl->bytes = off;
  return LOGLIN_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

int check_all(const void* X, const void* B, const void* C, const float* log_a,
              const void* lambda, int chunk, const void* out, const loglin_dims* dims,
              const void* ws, size_t ws_bytes, const loglin_opts* opts, Plan* pl) {
  int rc = check_dims(dims, chunk, opts, pl);
  if (rc) return rc;
  if (!X || !B || !C || !log_a || !lambda || !out) return LOGLIN_ERR_NULL;
  if (misaligned(X) || misaligned(B) || misaligned(C) || misaligned(log_a) ||
      misaligned(lambda) || misaligned(out))
    return LOGLIN_ERR_ALIGN;
  if (pl->bytes > 0) {
    if (!ws || ws_bytes < pl->bytes) return LOGLIN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return LOGLIN_ERR_ALIGN;
  }
  return LOGLIN_OK;
}

loglin::LaunchFn pick(int dtype, int chunk, int P, int N) {
  using namespace loglin;
  if (dtype == LOGLIN_BF16) {
    if (chunk == 16) return lookup_bf16_16(P, N);
    if (chunk == 32) return lookup_bf16_32(P, N);
    if (chunk == 64) return lookup_bf16_64(P, N);
  } else {
    if (chunk == 16) return lookup_f32_16(P, N);
    if (chunk == 32) return lookup_f32_32(P, N);
    if (chunk == 64) return lookup_f32_64(P, N);
  }
  return nullptr;
}

loglin::BwdFn pick_bwd(int dtype, int chunk, int P, int N) {
  using namespace loglin;
  if (dtype == LOGLIN_BF16) {  // chunk 16 is below one bf16 MFMA step
    if (chunk == 32) return lookup_bwd_bf16_32(P, N);
    if (chunk == 64) return lookup_bwd_bf16_64(P, N);
  } else {
    if (chunk == 16) return lookup_bwd_f32_16(P, N);
    if (chunk == 32) return lookup_bwd_f32_32(P, N);
    if (chunk == 64) return lookup_bwd_f32_64(P, N);
  }
  return nullptr;
}

// Backward workspace: chunk log-decays and their fp64 prefix sums, the
// totals of the groups of 8 chunks (forward direction), the reverse
// direction's piece partials, both directions' level states (fp32) and the
// two per-token terms of dlog_a; each region 256-byte aligned.
struct BwdPlan {
  int nc, kc, ll, npart, nstate, nstate_direct;
  size_t off_atot, off_cuma, off_pf, off_pr, off_z, off_r, off_t1, off_t2, bytes;
};

int check_bwd_dims(const loglin_dims* d, int chunk, BwdPlan* pl) {
  Plan fp;
  int rc = check_dims(d, chunk, nullptr, &fp);
  if (rc) return rc;
  if (fp.ll > loglin::BWD_LMAX) return LOGLIN_ERR_DIM;
  // chunk levels above 4 are walked over groups of 8 chunks with a stack of
  // BWD_UP_DEPTH block sums
  if (fp.kc > loglin::BWD_UP_DEPTH + 2) return LOGLIN_ERR_DIM;
  if (!pick_bwd(d->io_dtype, chunk, (int)d->headdim, (int)d->dstate)) return LOGLIN_ERR_SHAPE;
  pl->nc = fp.nc;
  pl->kc = fp.kc;
  pl->ll = fp.ll;
  int64_t npart = 0, nstate = 0, ndirect = 0;
  for (int k = 1; k <= fp.kc; ++k) {
    npart += (int64_t)loglin::bwd_pairs(fp.nc, k) * loglin::bwd_pieces(k);
    nstate += loglin::bwd_pairs(fp.nc, k);
    if (loglin::bwd_pieces(k) == 1) ndirect += loglin::bwd_pairs(fp.nc, k);
  }
  pl->nstate_direct = (int)ndirect;
  pl->npart = (int)npart;
  pl->nstate = (int)nstate;
  const size_t bh = (size_t)(d->batch * d->nheads);
  const size_t pn = (size_t)(d->headdim * d->dstate);
  size_t off = 0;
  pl->off_atot = off;
  off = round_up(off + bh * fp.nc * sizeof(float));
  pl->off_cuma = off;
  off = round_up(off + bh * (fp.nc + 1) * sizeof(double));
  pl->off_pf = off;  // totals of the groups of 8 chunks (levels above 4)
  off = round_up(off + bh * (fp.kc >= 5 ? (size_t)(fp.nc + 7) / 8 : 0) * pn * sizeof(float));
  pl->off_pr = off;
  off = round_up(off + bh * npart * pn * sizeof(float));
  pl->off_z = off;
  off = round_up(off + bh * nstate * pn * sizeof(float));
  pl->off_r = off;
  off = round_up(off + bh * nstate * pn * sizeof(float));
  pl->off_t1 = off;
  off = round_up(off + bh * d->seqlen * sizeof(float));
  pl->off_t2 = off;
  off = round_up(off + bh * d->seqlen * sizeof(float));
  pl->bytes = off;
  return LOGLIN_OK;
}

// Log-linear gated DeltaNet forward: one query and key per head (ngroups
// equals nheads), chunks of GDN_C tokens, chunk levels held in registers.
// Workspace of the gated DeltaNet forward: per (batch, head, chunk) the
// effective queries and W (C x N), U and the intra outputs (C x P), the
// chunk's decay ratios and total decay, fp32, each region 256-byte aligned.
struct GdnPlan {
  size_t off_qe, off_w, off_u, off_oi, off_kh, off_gc, bytes;
};

int check_gdn(const loglin_dims* d, int* ll, int* nc) {
  if (!d) return LOGLIN_ERR_NULL;
  if (d->reserved != 0) return LOGLIN_ERR_DIM;
  if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->ngroups <= 0 ||
      d->headdim <= 0 || d->dstate <= 0 || d->nlevels <= 0)
    return LOGLIN_ERR_DIM;
  if (d->io_dtype != LOGLIN_F32 && d->io_dtype != LOGLIN_BF16) return LOGLIN_ERR_DTYPE;
  if (d->ngroups != d->nheads) return LOGLIN_ERR_GROUPS;
  if (d->seqlen % loglin::GDN_C) return LOGLIN_ERR_SEQ_CHUNK;
  if (d->seqlen > (int64_t(1) << 30) || d->nheads > 4096 || d->nlevels > 64 ||
      d->batch * d->nheads * 4 > (int64_t(1) << 30))
    return LOGLIN_ERR_DIM;
  const int l = ceil_log2(d->seqlen) + 1;
  if (d->nlevels < l) return LOGLIN_ERR_LEVELS;
  const int64_t n = d->seqlen / loglin::GDN_C;
  if (l > loglin::GDN_LMAX || ceil_log2(n) > loglin::GDN_KMAX - 1) return LOGLIN_ERR_DIM;
  if (!loglin::lookup_gdn(d->io_dtype, (int)d->dstate, (int)d->headdim)) return LOGLIN_ERR_SHAPE;
  *ll = l;
  *nc = (int)n;
  return LOGLIN_OK;
}

GdnPlan gdn_plan(const loglin_dims* d, int nc) {
  const size_t items = (size_t)(d->batch * d->nheads) * nc;
  const size_t C = loglin::GDN_C;
  GdnPlan pl;
  size_t off = 0;
  pl.off_qe = off;
  off = round_up(off + items * C * d->dstate * sizeof(float));
  pl.off_w = off;
  off = round_up(off + items * C * d->dstate * sizeof(float));
  pl.off_u = off;
  off = round_up(off + items * C * d->headdim * sizeof(float));
  pl.off_oi = off;
  off = round_up(off + items * C * d->headdim * sizeof(float));
  pl.off_kh = off;
  off = round_up(off + items * C * sizeof(float));
  pl.off_gc = off;
  off = round_up(off + items * sizeof(float));
  pl.bytes = off;
  return pl;
}

// Decode state: level states fp32 [B, H, LL, P/4, N, 4], then the two banks of
// per-level decay factors [B, H, 2, LL]; each region 256-byte aligned.
struct DecodePlan {
  int ll;
  size_t off_g, bytes;
};

int check_decode(const loglin_dims* d, DecodePlan* pl) {
  if (!d) return LOGLIN_ERR_NULL;
  if (d->reserved != 0) return LOGLIN_ERR_DIM;
  if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->ngroups <= 0 ||
      d->headdim <= 0 || d->dstate <= 0 || d->nlevels <= 0)
    return LOGLIN_ERR_DIM;
  if (d->io_dtype != LOGLIN_F32 && d->io_dtype != LOGLIN_BF16) return LOGLIN_ERR_DTYPE;
  if (d->nheads % d->ngroups) return LOGLIN_ERR_GROUPS;
  if (d->seqlen > (int64_t(1) << 40) || d->nheads > 4096 || d->nlevels > 64 ||
      d->batch * d->nheads > (int64_t(1) << 24))
    return LOGLIN_ERR_DIM;
  const int ll = ceil_log2(d->seqlen) + 1;
  if (d->nlevels < ll) return LOGLIN_ERR_LEVELS;
  if (!supported_shape(d->io_dtype, d->headdim, d->dstate)) return LOGLIN_ERR_SHAPE;
  if (ll > 128) return LOGLIN_ERR_DIM;  // one thread per level writes the decay factors
  pl->ll = ll;
  const size_t bh = (size_t)(d->batch * d->nheads);
  pl->off_g = round_up(bh * ll * (size_t)(d->headdim * d->dstate) * sizeof(float));
  pl->bytes = round_up(pl->off_g + bh * 2 * ll * sizeof(float));
  return LOGLIN_OK;
}

}  // namespace

extern "C" {

size_t loglin_decode_state_bytes(const loglin_dims* dims) {
  DecodePlan pl;
  return check_decode(dims, &pl) ? 0 : pl.bytes;
}

int loglin_decode_step(void* state, int64_t t, const void* X, const void* B, const void* C,
                       const float* log_a, const void* lambda, void* out,
                       const loglin_dims* dims, void* stream) {
  DecodePlan pl;
  int rc = check_decode(dims, &pl);
  if (rc) return rc;
  if (t < 0 || t >= dims->seqlen) return LOGLIN_ERR_DIM;
  if (!state || !X || !B || !C || !log_a || !lambda || !out) return LOGLIN_ERR_NULL;
  // one token's rows are small: inputs need only element alignment
  const uintptr_t es = dims->io_dtype == LOGLIN_BF16 ? 2 : 4;
  auto off = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; };
  if (off(X, es) || off(B, es) || off(C, es) || off(lambda, es) || off(log_a, 4) ||
      misaligned(out) || off(state, kAlign))
    return LOGLIN_ERR_ALIGN;
  loglin::DecodeFn fn = loglin::lookup_decode(dims->io_dtype, (int)dims->headdim, (int)dims->dstate);
  if (!fn) return LOGLIN_ERR_SHAPE;
  loglin::DecodeParams dp{};
  dp.X = X;
  dp.Bm = B;
  dp.Cm = C;
  dp.log_a = log_a;
  dp.lam = lambda;
  dp.out = out;
  dp.S = static_cast<float*>(state);
  dp.gd = reinterpret_cast<float*>(static_cast<char*>(state) + pl.off_g);
  dp.batch = (int)dims->batch;
  dp.nheads = (int)dims->nheads;
  dp.ngroups = (int)dims->ngroups;
  dp.nlevels = (int)dims->nlevels;
  dp.ll = pl.ll;
  dp.t = t;
  return fn(dp, stream) ? LOGLIN_ERR_HIP : LOGLIN_OK;
}

size_t loglin_workspace_bytes_ex(const loglin_dims* dims, int chunk, const loglin_opts* opts) {
  Plan pl;
  return check_dims(dims, chunk, opts, &pl) ? 0 : pl.bytes;
}

size_t loglin_workspace_bytes(const loglin_dims* dims, int chunk) {
  return loglin_workspace_bytes_ex(dims, chunk, nullptr);
}

int loglin_plan_seg_log2(const loglin_dims* dims, int chunk, const loglin_opts* opts) {
  Plan pl;
  int rc = check_dims(dims, chunk, opts, &pl);
  return rc ? rc : pl.m;
}

int loglin_validate(const void* X, const void* B, const void* C, const float* log_a,
                    const void* lambda, int chunk, const void* out, const loglin_dims* dims,
                    const void* workspace, size_t workspace_bytes, const loglin_opts* opts) {
  Plan pl;
  return check_all(X, B, C, log_a, lambda, chunk, out, dims, workspace, workspace_bytes,
                   opts, &pl);
}

int loglin_fwd_ex(const void* X, const void* B, const void* C, const float* log_a,
                  const void* lambda, int chunk, void* out, const loglin_dims* dims,
                  void* workspace, size_t workspace_bytes, void* stream,
                  const loglin_opts* opts) {
  Plan pl;
  int rc = check_all(X, B, C, log_a, lambda, chunk, out, dims, workspace, workspace_bytes,
                     opts, &pl);
  if (rc) return rc;
  loglin::LaunchFn fn = pick(dims->io_dtype, chunk, (int)dims->headdim, (int)dims->dstate);
  if (!fn) return LOGLIN_ERR_SHAPE;

  Params pr{};
  pr.X = X;
  pr.Bm = B;
  pr.Cm = C;
  pr.log_a = log_a;
  pr.lam = lambda;
  pr.out = out;
  char* ws = static_cast<char*>(workspace);
  if (pl.bytes > 0) {
    pr.seg_state = ws + pl.off_state;
    pr.seg_decay = reinterpret_cast<float*>(ws + pl.off_decay);
    pr.slots = ws + pl.off_slots;
    pr.gap_decay = reinterpret_cast<float*>(ws + pl.off_gap);
  }
  pr.batch = (int)dims->batch;
  pr.seqlen = (int)dims->seqlen;
  pr.nheads = (int)dims->nheads;
  pr.ngroups = (int)dims->ngroups;
  pr.nlevels = (int)dims->nlevels;
  pr.nc = pl.nc;
  pr.kc = pl.kc;
  pr.m = pl.m;
  pr.ns = pl.ns;
  pr.ks = pl.ks;
  pr.ll = pl.ll;
  pr.hp = pl.hp;
  pr.lmask = (opts && opts->level_mask) ? opts->level_mask : ~0ull;
  void* const* ev = opts ? opts->stage_events : nullptr;
  int herr = fn(pr, static_cast<hipStream_t>(stream), ev);
  return herr ? LOGLIN_ERR_HIP : LOGLIN_OK;
}

int loglin_fwd(const void* X, const void* B, const void* C, const float* log_a,
               const void* lambda, int chunk, void* out, const loglin_dims* dims,
               void* workspace, size_t workspace_bytes, void* stream) {
  return loglin_fwd_ex(X, B, C, log_a, lambda, chunk, out, dims, workspace, workspace_bytes,
                       stream, nullptr);
}

size_t loglin_bwd_workspace_bytes(const loglin_dims* dims, int chunk) {
  BwdPlan pl;
  return check_bwd_dims(dims, chunk, &pl) ? 0 : pl.bytes;
}

int loglin_bwd(const void* X, const void* B, const void* C, const float* log_a,
               const void* lambda, const void* dO, int chunk, void* dX, void* dB, void* dC,
               float* dlog_a, void* dlambda, const loglin_dims* dims, void* workspace,
               size_t workspace_bytes, void* stream) {
  BwdPlan pl;
  int rc = check_bwd_dims(dims, chunk, &pl);
  if (rc) return rc;
  if (!X || !B || !C || !log_a || !lambda || !dO || !dX || !dB || !dC || !dlog_a || !dlambda ||
      !workspace)
    return !workspace && X && B && C && log_a && lambda && dO && dX && dB && dC && dlog_a &&
                   dlambda
               ? LOGLIN_ERR_WORKSPACE
               : LOGLIN_ERR_NULL;
  if (misaligned(X) || misaligned(B) || misaligned(C) || misaligned(log_a) ||
      misaligned(lambda) || misaligned(dO) || misaligned(dX) || misaligned(dB) ||
      misaligned(dC) || misaligned(dlog_a) || misaligned(dlambda))
    return LOGLIN_ERR_ALIGN;
  if (workspace_bytes < pl.bytes) return LOGLIN_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return LOGLIN_ERR_ALIGN;
  loglin::BwdFn fn = pick_bwd(dims->io_dtype, chunk, (int)dims->headdim, (int)dims->dstate);
  char* ws = static_cast<char*>(workspace);
  loglin::BwdParams pr{};
  pr.X = X;
  pr.Bm = B;
  pr.Cm = C;
  pr.log_a = log_a;
  pr.lam = lambda;
  pr.dO = dO;
  pr.dX = dX;
  pr.dB = dB;
  pr.dC = dC;
  pr.dloga = dlog_a;
  pr.dlam = dlambda;
  pr.atot = reinterpret_cast<float*>(ws + pl.off_atot);
  pr.cuma = reinterpret_cast<double*>(ws + pl.off_cuma);
  pr.part_f = reinterpret_cast<float*>(ws + pl.off_pf);
  pr.part_r = reinterpret_cast<float*>(ws + pl.off_pr);
  pr.zst = reinterpret_cast<float*>(ws + pl.off_z);
  pr.rst = reinterpret_cast<float*>(ws + pl.off_r);
  pr.term1 = reinterpret_cast<float*>(ws + pl.off_t1);
  pr.term2 = reinterpret_cast<float*>(ws + pl.off_t2);
  pr.batch = (int)dims->batch;
  pr.seqlen = (int)dims->seqlen;
  pr.nheads = (int)dims->nheads;
  pr.ngroups = (int)dims->ngroups;
  pr.nlevels = (int)dims->nlevels;
  pr.nc = pl.nc;
  pr.kc = pl.kc;
  pr.ll = pl.ll;
  pr.npart = pl.npart;
  pr.nstate = pl.nstate;
  pr.nstate_direct = pl.nstate_direct;
  return fn(pr, static_cast<hipStream_t>(stream)) ? LOGLIN_ERR_HIP : LOGLIN_OK;
}

size_t loglin_gdn_workspace_bytes(const loglin_dims* dims) {
  int ll = 0, nc = 0;
  if (check_gdn(dims, &ll, &nc)) return 0;
  return gdn_plan(dims, nc).bytes;
}

int loglin_gdn_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                   const float* beta, const void* lambda, void* out, const loglin_dims* dims,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int ll = 0, nc = 0;
  int rc = check_gdn(dims, &ll, &nc);
  if (rc) return rc;
  if (!q || !k || !v || !log_alpha || !beta || !lambda || !out) return LOGLIN_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(log_alpha) ||
      misaligned(beta) || misaligned(lambda) || misaligned(out))
    return LOGLIN_ERR_ALIGN;
  const GdnPlan pl = gdn_plan(dims, nc);
  if (!workspace || workspace_bytes < pl.bytes) return LOGLIN_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return LOGLIN_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  loglin::GdnParams pr{};
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.log_alpha = log_alpha;
  pr.beta = beta;
  pr.lam = lambda;
  pr.out = out;
  pr.qe = reinterpret_cast<float*>(ws + pl.off_qe);
  pr.w = reinterpret_cast<float*>(ws + pl.off_w);
  pr.u = reinterpret_cast<float*>(ws + pl.off_u);
  pr.oi = reinterpret_cast<float*>(ws + pl.off_oi);
  pr.kh = reinterpret_cast<float*>(ws + pl.off_kh);
  pr.gc = reinterpret_cast<float*>(ws + pl.off_gc);
  pr.batch = (int)dims->batch;
  pr.seqlen = (int)dims->seqlen;
  pr.nheads = (int)dims->nheads;
  pr.nlevels = (int)dims->nlevels;
  pr.ll = ll;
  pr.nc = nc;
  loglin::GdnFn fn = loglin::lookup_gdn(dims->io_dtype, (int)dims->dstate, (int)dims->headdim);
  return fn(pr, static_cast<hipStream_t>(stream)) ? LOGLIN_ERR_HIP : LOGLIN_OK;
}

const char* loglin_strerror(int code) {
  switch (code) {
    case LOGLIN_OK: return "success";
    case LOGLIN_ERR_NULL: return "a required pointer is NULL";
    case LOGLIN_ERR_DIM: return "a dimension is non-positive or too large";
    case LOGLIN_ERR_CHUNK: return "chunk must be 16, 32 or 64";
    case LOGLIN_ERR_SEQ_CHUNK: return "seqlen must be a multiple of chunk";
    case LOGLIN_ERR_GROUPS: return "nheads must be a multiple of ngroups";
    case LOGLIN_ERR_LEVELS: return "nlevels must be at least ceil(log2 seqlen) + 1";
    case LOGLIN_ERR_DTYPE: return "io_dtype must be LOGLIN_F32 or LOGLIN_BF16";
    case LOGLIN_ERR_WORKSPACE: return "workspace is NULL or too small";
    case LOGLIN_ERR_ALIGN: return "a pointer is not 16-byte aligned (workspace: 256)";
    case LOGLIN_ERR_SHAPE: return "unsupported (headdim, dstate) for this dtype";
    case LOGLIN_ERR_HIP: return "a HIP launch failed";
    case LOGLIN_ERR_OPTS: return "an option is out of range";
    case LOGLIN_ERR_SCRATCH:
      return "the workspace exceeds the fixed scratch array of loglin_fwd_noalloc";
    default: return "unknown error code";
  }
}

int loglin_event_create(void** event) {
  if (!event) return LOGLIN_ERR_NULL;
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return LOGLIN_ERR_HIP;
  *event = e;
  return LOGLIN_OK;
}

int loglin_event_destroy(void* event) {
  if (!event) return LOGLIN_ERR_NULL;
  return hipEventDestroy(static_cast<hipEvent_t>(event)) == hipSuccess ? LOGLIN_OK
                                                                        : LOGLIN_ERR_HIP;
}

int loglin_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return LOGLIN_ERR_NULL;
  return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start),
                             static_cast<hipEvent_t>(stop)) == hipSuccess
             ? LOGLIN_OK
             : LOGLIN_ERR_HIP;
}

}  // extern "C"
