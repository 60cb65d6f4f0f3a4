// Host side of libforge: argument validation, per-call scalars, dispatch.
// Implements include/forge.h.

#include "../../include/forge.h"

#include <cmath>
#include <cstdint>
#include <cstring>

#include "forge_internal.h"

static_assert(FORGE_GROUP_MAX == forge::GROUP_MAX, "group size of the ABI and the kernels");
static_assert(FORGE_DGRAD_SCRATCH_BYTES == forge::DGRAD_SCRATCH_BYTES, "scratch size of the ABI and the kernels");
static_assert(FORGE_QUOTIENT_COUNTS == forge::QUOTIENT_CHECK_BLOCKS * 8, "quotient check counters of the ABI and the kernel");

namespace {

using namespace forge;

constexpr uint32_t kGolden = 0x9E3779B9u;
constexpr uint64_t kMaxExtent = 1ull << 48;   // largest byte extent of one matrix

// MurmurHash3 32-bit finaliser (Appleby, public domain).
uint32_t fmix32_host(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// Stochastic-rounding key of one stored tensor: the 64-bit step and seed are
// folded in as four 32-bit words, each through the finaliser.
uint32_t sr_key(uint64_t seed, uint64_t step, uint32_t tensor_id) {
  uint32_t k = fmix32_host((uint32_t)(step >> 32) + kGolden * (tensor_id + 1u));
  k = fmix32_host((uint32_t)step ^ k);
  k = fmix32_host((uint32_t)(seed >> 32) ^ k);
  k = fmix32_host((uint32_t)seed ^ k);
  return k;
}

int elem_size(int dtype) {
  switch (dtype) {
    case FORGE_F32: return 4;
    case FORGE_BF16: return 2;
    case FORGE_S8:
    case FORGE_U8:
    case FORGE_E4M3: return 1;
    default: return 0;
  }
}

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};

Range mat_range(const forge_mat& m) {
  Range r;
  if (m.rows <= 0 || m.cols <= 0 || m.data == nullptr) return r;
  const uint64_t n = (uint64_t)(m.rows - 1) * (uint64_t)m.ld + (uint64_t)m.cols;
  r.lo = (uintptr_t)m.data;
  r.hi = r.lo + (uintptr_t)(n * (uint64_t)elem_size(m.dtype));
  return r;
}

Range raw_range(const void* p, uint64_t bytes) {
  Range r;
  if (p == nullptr || bytes == 0) return r;
  r.lo = (uintptr_t)p;
  r.hi = r.lo + (uintptr_t)bytes;
  return r;
}

bool overlap(const Range& a, const Range& b) {
  if (a.empty() || b.empty()) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

bool finite(double x) { return std::isfinite(x); }

// Shape / dtype / pointer checks of one matrix.
forge_status check_mat(const forge_mat& m, int64_t rows, int64_t cols) {
  if (m.rows != rows || m.cols != cols) return FORGE_E_SHAPE;
  if (m.rows < 0 || m.cols < 0) return FORGE_E_SHAPE;
  if (m.ld < m.cols || (m.cols > 0 && m.ld < 1)) return FORGE_E_SHAPE;
  const int es = elem_size(m.dtype);
  if (es == 0) return FORGE_E_DTYPE;
  if (m.rows > 0 && m.cols > 0) {
    // byte extent ((rows - 1) ld + cols) es: no wrap-around, at most 2^48
    // (so that every row offset the kernels form in 64 bits is exact)
    uint64_t ext = 0;
    if (__builtin_mul_overflow((uint64_t)(m.rows - 1), (uint64_t)m.ld, &ext) ||
        __builtin_add_overflow(ext, (uint64_t)m.cols, &ext) || __builtin_mul_overflow(ext, (uint64_t)es, &ext) ||
        ext > kMaxExtent)
      return FORGE_E_SHAPE;
    if (m.data == nullptr) return FORGE_E_NULL;
    if (!aligned(m.data, es)) return FORGE_E_ALIGN;
  }
  return FORGE_OK;
}

struct Plan {
  int64_t BT = 0, N = 0, K = 0;
  int in_fmt = -1, w_fmt = -1, m_fmt = -1, v_fmt = FMT_NONE;
  int block = 0;
  bool empty = false;  // N == 0 or K == 0: nothing to do
};

forge_status check_state(const forge_state& s, int64_t N, int64_t K, bool first, Plan& pl) {
  forge_status st = check_mat(s.q, N, K);
  if (st != FORGE_OK) return st;
  const int dt = s.q.dtype;
  // 8-bit codes with block scales: S8 (first moment) / U8 (second) / E4M3 (either)
  const bool int8 = (first ? dt == FORGE_S8 : dt == FORGE_U8) || dt == FORGE_E4M3;
  if (!(dt == FORGE_F32 || dt == FORGE_BF16 || int8)) return FORGE_E_DTYPE;
  if (int8) {
    if (!(s.block == 32 || s.block == 64 || s.block == 128)) return FORGE_E_SHAPE;
    if (K % s.block != 0) return FORGE_E_SHAPE;
    if (N > 0 && K > 0) {
      if (s.scale == nullptr) return FORGE_E_NULL;
      if (!aligned(s.scale, 4)) return FORGE_E_ALIGN;
    }
    if (pl.block != 0 && pl.block != s.block) return FORGE_E_UNSUPPORTED;
    pl.block = s.block;
  } else if (s.scale != nullptr) {
    return FORGE_E_DTYPE;  // a scale array only makes sense for int8 codes
  }
  return FORGE_OK;
}

// Memory written by a call (W, m, v and their scale arrays) and read-only inputs (X, dY).
void layer_ranges(const forge_mat* X, const forge_mat* dY, const forge_mat* W, const forge_state* m,
                  const forge_state* v, const Plan& pl, Range (&outs)[5], Range (&ins)[2]) {
  outs[0] = mat_range(*W);
  outs[1] = m ? mat_range(m->q) : Range();
  outs[2] = v ? mat_range(v->q) : Range();
  outs[3] = (m && m->scale) ? raw_range(m->scale, (uint64_t)pl.N * (uint64_t)(pl.K / (m->block ? m->block : 1)) * 4)
                            : Range();
  outs[4] = (v && v->scale) ? raw_range(v->scale, (uint64_t)pl.N * (uint64_t)(pl.K / (v->block ? v->block : 1)) * 4)
                            : Range();
  ins[0] = mat_range(*X);
  ins[1] = mat_range(*dY);
}

// wq: the weight as an E4M3 state (codes + block scales; W == &wq->q), or
// NULL for a bf16 / fp32 weight.
forge_status validate(const forge_mat* X, const forge_mat* dY, const forge_mat* W, const forge_state* m,
                      const forge_state* v, const forge_hyper* h, int64_t step, Plan& pl,
                      const forge_state* wq = nullptr) {
  if (!X || !dY || !W || !h) return FORGE_E_NULL;
  // optimizer and which states it keeps
  const int o = h->opt;
  if (o < FORGE_ADAMW || o > FORGE_SGD) return FORGE_E_HYPER;
  if (h->round != FORGE_ROUND_RNE && h->round != FORGE_ROUND_SR) return FORGE_E_HYPER;
  if (opt_has_m(o) && !m) return FORGE_E_NULL;
  if (opt_has_v(o) && !v) return FORGE_E_NULL;
  if ((!opt_has_m(o) && m) || (!opt_has_v(o) && v)) return FORGE_E_UNSUPPORTED;
  if (step < 1) return FORGE_E_STEP;
  // hyper-parameters: all finite; the ones the optimizer uses in range
  if (!finite(h->lr) || !finite(h->beta1) || !finite(h->beta2) || !finite(h->eps) || !finite(h->weight_decay))
    return FORGE_E_HYPER;
  if (h->lr < 0 || h->weight_decay < 0) return FORGE_E_HYPER;
  const bool adam_like = o == FORGE_ADAMW || o == FORGE_NADAM || o == FORGE_RADAM;
  const bool uses_b1 = adam_like || o == FORGE_LION || o == FORGE_SGDM;
  const bool uses_b2 = adam_like || o == FORGE_LION || o == FORGE_RMSPROP;
  const bool uses_eps = adam_like || o == FORGE_RMSPROP || o == FORGE_ADAGRAD;
  if (uses_b1 && (h->beta1 < 0 || h->beta1 >= 1)) return FORGE_E_HYPER;
  if (uses_b2 && (h->beta2 < 0 || h->beta2 >= 1)) return FORGE_E_HYPER;
  if (uses_eps && !(h->eps > 0)) return FORGE_E_HYPER;
  // shapes
  pl.BT = X->rows;
  pl.K = X->cols;
  pl.N = dY->cols;
  if (pl.BT < 0 || pl.N < 0 || pl.K < 0) return FORGE_E_SHAPE;
  if (dY->rows != pl.BT) return FORGE_E_SHAPE;
  forge_status st;
  if ((st = check_mat(*X, pl.BT, pl.K)) != FORGE_OK) return st;
  if ((st = check_mat(*dY, pl.BT, pl.N)) != FORGE_OK) return st;
  if ((st = check_mat(*W, pl.N, pl.K)) != FORGE_OK) return st;
  if (X->dtype != dY->dtype) return FORGE_E_DTYPE;
  if (X->dtype != FORGE_F32 && X->dtype != FORGE_BF16) return FORGE_E_DTYPE;
  if (wq) {
    if (W->dtype != FORGE_E4M3) return FORGE_E_DTYPE;
    if (!(wq->block == 32 || wq->block == 64 || wq->block == 128)) return FORGE_E_SHAPE;
    if (pl.K % wq->block != 0) return FORGE_E_SHAPE;
    if (pl.N > 0 && pl.K > 0) {
      if (wq->scale == nullptr) return FORGE_E_NULL;
      if (!aligned(wq->scale, 4)) return FORGE_E_ALIGN;
    }
    pl.block = wq->block;
  } else if (W->dtype != FORGE_F32 && W->dtype != FORGE_BF16) {
    return FORGE_E_DTYPE;
  }
  if (m && (st = check_state(*m, pl.N, pl.K, true, pl)) != FORGE_OK) return st;
  if (v && (st = check_state(*v, pl.N, pl.K, false, pl)) != FORGE_OK) return st;
  // size limits: 32-bit flat SR index and 32-bit tile / token counters
  if ((uint64_t)pl.N * (uint64_t)pl.K >= (1ull << 32)) return FORGE_E_SHAPE;
  if (pl.BT >= (1ll << 31) || pl.N >= (1ll << 31) || pl.K >= (1ll << 31)) return FORGE_E_SHAPE;
  const int64_t tiles = ((pl.N + 127) / 128) * ((pl.K + 127) / 128);
  if (tiles >= (1ll << 31)) return FORGE_E_SHAPE;
  // aliasing: outputs must not overlap inputs or each other
  Range outs[5], ins[2];
  layer_ranges(X, dY, W, m, v, pl, outs, ins);
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlap(outs[i], ins[j])) return FORGE_E_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return FORGE_E_ALIAS;
  }
  if (wq && wq->scale) {   // the weight's block scales are written too
    const Range rs = raw_range(wq->scale, (uint64_t)pl.N * (uint64_t)(pl.K / wq->block) * 4);
    for (const Range& r : outs)
      if (overlap(rs, r)) return FORGE_E_ALIAS;
    for (const Range& r : ins)
      if (overlap(rs, r)) return FORGE_E_ALIAS;
  }
  pl.in_fmt = X->dtype;
  pl.w_fmt = W->dtype;
  pl.m_fmt = m ? m->q.dtype : FMT_NONE;
  pl.v_fmt = v ? v->q.dtype : FMT_NONE;
  if (!combo_supported(pl.in_fmt, pl.w_fmt, h->opt, pl.m_fmt, pl.v_fmt)) return FORGE_E_UNSUPPORTED;
  pl.empty = (pl.N == 0 || pl.K == 0);
  return FORGE_OK;
}

// X and dY of a call that has no weight (gradient accumulation).
forge_status validate_inputs(const forge_mat* X, const forge_mat* dY, Plan& pl) {
  if (!X || !dY) return FORGE_E_NULL;
  pl.BT = X->rows;
  pl.K = X->cols;
  pl.N = dY->cols;
  if (pl.BT < 0 || pl.N < 0 || pl.K < 0) return FORGE_E_SHAPE;
  if (dY->rows != pl.BT) return FORGE_E_SHAPE;
  forge_status st;
  if ((st = check_mat(*X, pl.BT, pl.K)) != FORGE_OK) return st;
  if ((st = check_mat(*dY, pl.BT, pl.N)) != FORGE_OK) return st;
  if (X->dtype != dY->dtype) return FORGE_E_DTYPE;
  if (X->dtype != FORGE_F32 && X->dtype != FORGE_BF16) return FORGE_E_DTYPE;
  if ((uint64_t)pl.N * (uint64_t)pl.K >= (1ull << 32)) return FORGE_E_SHAPE;
  if (pl.BT >= (1ll << 31) || pl.N >= (1ll << 31) || pl.K >= (1ll << 31)) return FORGE_E_SHAPE;
  pl.in_fmt = X->dtype;
  pl.empty = (pl.N == 0 || pl.K == 0);
  return FORGE_OK;
}

// The fp32 gradient accumulator of forge_wgrad_accumulate / _step_accumulated.
forge_status check_acc(const forge_mat* acc, int64_t N, int64_t K) {
  if (!acc) return FORGE_E_NULL;
  const forge_status st = check_mat(*acc, N, K);
  if (st != FORGE_OK) return st;
  if (acc->dtype != FORGE_F32) return FORGE_E_DTYPE;
  return FORGE_OK;
}

bool vec_ok(const void* p, int64_t ld, int elems, int es) {
  return p == nullptr || (aligned(p, elems * es) && (ld % elems) == 0);
}

// Row pitch small enough for the aligned epilogue's 32-bit per-thread
// offsets (up to 32 rows of a pass, 2^26 bytes each, plus the columns).
bool pitch_ok(int64_t ld, int es) { return (uint64_t)ld * (uint64_t)es <= (1ull << 26); }

// dX = dY W: shapes, dtypes, limits, aliasing; fills the launch arguments.
// wq: the weight as an E4M3 state (W == &wq->q), or NULL.
forge_status check_dgrad(const forge_mat* dY, const forge_mat* W, const forge_mat* dX, DgArgs& g, bool& fast,
                         const forge_state* wq = nullptr) {
  if (!dY || !W || !dX) return FORGE_E_NULL;
  const int64_t BT = dY->rows, N = dY->cols, K = W->cols;
  if (BT < 0 || N < 0 || K < 0) return FORGE_E_SHAPE;
  forge_status st;
  if ((st = check_mat(*dY, BT, N)) != FORGE_OK) return st;
  if ((st = check_mat(*W, N, K)) != FORGE_OK) return st;
  if ((st = check_mat(*dX, BT, K)) != FORGE_OK) return st;
  for (const forge_mat* t : {dY, W, dX}) {
    if (t == W && wq) {
      if (t->dtype != FORGE_E4M3) return FORGE_E_DTYPE;
    } else if (t->dtype != FORGE_F32 && t->dtype != FORGE_BF16) {
      return FORGE_E_DTYPE;
    }
  }
  if (BT >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31)) return FORGE_E_SHAPE;
  if (((BT + 127) / 128) * ((K + 127) / 128) >= (1ll << 31)) return FORGE_E_SHAPE;
  Range rws;
  if (wq) {
    if (!(wq->block == 32 || wq->block == 64 || wq->block == 128) || K % wq->block != 0) return FORGE_E_SHAPE;
    if (N > 0 && K > 0) {
      if (wq->scale == nullptr) return FORGE_E_NULL;
      if (!aligned(wq->scale, 4)) return FORGE_E_ALIGN;
    }
    rws = raw_range(wq->scale, (uint64_t)N * (uint64_t)(K / wq->block) * 4);
  }
  const Range out = mat_range(*dX);
  if (overlap(out, mat_range(*dY)) || overlap(out, mat_range(*W)) || overlap(out, rws)) return FORGE_E_ALIAS;
  std::memset(&g, 0, sizeof(g));
  g.dY = dY->data; g.lddy = dY->ld;
  g.W = W->data; g.ldw = W->ld;
  g.dX = dX->data; g.ldx = dX->ld;
  g.BT = (int32_t)BT; g.N = (int32_t)N; g.K = (int32_t)K;
  g.tiles_m = (int32_t)((BT + 127) / 128);
  g.tiles_k = (int32_t)((K + 127) / 128);
  g.in_fmt = dY->dtype; g.w_fmt = W->dtype; g.dx_fmt = dX->dtype;
  g.vec_out = vec_ok(dX->data, dX->ld, 4, elem_size(dX->dtype)) ? 1 : 0;
  g.splits = 1;
  g.ws = nullptr;
  g.wsc = wq ? wq->scale : nullptr;
  g.wblock = wq ? wq->block : 0;
  fast = dY->dtype == FORGE_BF16 && W->dtype == FORGE_BF16 && N % 8 == 0 && K % 8 == 0 &&
         vec_ok(dY->data, dY->ld, 8, 2) && vec_ok(W->data, W->ld, 8, 2) &&
         (uint64_t)BT * (uint64_t)dY->ld * 2 < (1ull << 31) && (uint64_t)N * (uint64_t)W->ld * 2 < (1ull << 31);
  return FORGE_OK;
}

// The activation half of a launch: X, dY, sizes, tile counts, loader choice.
void input_args(const forge_mat* X, const forge_mat* dY, const Plan& pl, KArgs& a) {
  a.X = X->data; a.ldx = X->ld;
  a.dY = dY->data; a.lddy = dY->ld;
  a.BT = (int32_t)pl.BT; a.N = (int32_t)pl.N; a.K = (int32_t)pl.K;
  a.tiles_n = (int32_t)((pl.N + 127) / 128);
  a.tiles_k = (int32_t)((pl.K + 127) / 128);
  // 16-byte vector loads of 8 bf16 / 4 fp32 activations
  const int ies = elem_size(pl.in_fmt), ivec = 16 / ies;
  a.vec_in = (vec_ok(X->data, X->ld, ivec, ies) && vec_ok(dY->data, dY->ld, ivec, ies)) ? 1 : 0;
  // direct-to-LDS mainloop: 16-byte aligned bf16 rows, feature counts that
  // are multiples of 8 (a chunk is all inside or all outside), and byte
  // offsets that fit the 32-bit buffer addressing
  a.dma_ok = (pl.in_fmt == FORGE_BF16 && a.vec_in && pl.N % 8 == 0 && pl.K % 8 == 0 &&
              (uint64_t)pl.BT * (uint64_t)dY->ld * 2 < (1ull << 31) &&
              (uint64_t)pl.BT * (uint64_t)X->ld * 2 < (1ull << 31)) ? 1 : 0;
  a.lddw = pl.K;
}

// An fp32 G buffer (accumulator) as the launch's dW.
void acc_args(forge_mat* acc, KArgs& a) {
  a.dW = acc->data;
  a.lddw = acc->ld;
  a.dw_fmt = FMT_F32;
  a.vec_dw = (vec_ok(acc->data, acc->ld, 4, 4) && pitch_ok(acc->ld, 4)) ? 1 : 0;
}

KArgs make_args(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m, forge_state* v,
                const forge_hyper* h, int64_t step, uint64_t seed, const Plan& pl) {
  KArgs a;
  std::memset(&a, 0, sizeof(a));
  input_args(X, dY, pl, a);
  a.W = W->data; a.ldw = W->ld;
  if (m) { a.m = m->q.data; a.ldm = m->q.ld; a.ms = m->scale; }
  if (v) { a.v = v->q.data; a.ldv = v->q.ld; a.vs = v->scale; }
  a.block = pl.block ? pl.block : 128;
  // 4-element state accesses (16 B fp32, 8 B bf16, 4 B int8)
  bool vs = vec_ok(W->data, W->ld, 4, elem_size(pl.w_fmt)) && pitch_ok(W->ld, elem_size(pl.w_fmt));
  if (m) vs = vs && vec_ok(m->q.data, m->q.ld, 4, elem_size(pl.m_fmt)) && pitch_ok(m->q.ld, elem_size(pl.m_fmt));
  if (v) vs = vs && vec_ok(v->q.data, v->q.ld, 4, elem_size(pl.v_fmt)) && pitch_ok(v->q.ld, elem_size(pl.v_fmt));
  a.vec_state = vs ? 1 : 0;
  // scalars, in double, rounded once
  const double lr = h->lr, b1 = h->beta1, b2 = h->beta2, wd = h->weight_decay;
  EpiConst& c = a.c;
  c.lr = (float)lr;
  c.b1 = (float)b1;
  c.b2 = (float)b2;
  c.omb1 = (float)(1.0 - b1);
  c.omb2 = (float)(1.0 - b2);
  c.eps = (float)h->eps;
  c.decay = (float)(1.0 - lr * wd);
  c.wd = (float)wd;
  const double t = (double)step;
  const int o = h->opt;
  const bool adam_like = o == FORGE_ADAMW || o == FORGE_NADAM || o == FORGE_RADAM;
  c.bc1 = adam_like ? (float)(1.0 / (1.0 - std::pow(b1, t))) : 1.0f;
  c.lrbc1 = adam_like ? (float)(lr / (1.0 - std::pow(b1, t))) : 0.0f;
  c.bc2s = (o == FORGE_ADAMW || o == FORGE_NADAM) ? (float)(1.0 / std::sqrt(1.0 - std::pow(b2, t))) : 1.0f;
  if (o == FORGE_NADAM) {
    // momentum schedule mu_i = b1 (1 - 0.5 * 0.96^(psi i)), psi = 0.004, and
    // its running product over i = 1..t (+1), in double in increasing i;
    // once the product is below 2^-60, 1 - product is 1 in double and the
    // remaining factors cannot change it
    const double psi = 0.004;
    auto mu = [&](double i) { return b1 * (1.0 - 0.5 * std::pow(0.96, i * psi)); };
    double prod = 1.0;
    for (int64_t i = 1; i <= step && prod >= 0x1p-60; ++i) prod *= mu((double)i);
    if (prod < 0x1p-60) prod = 0.0;
    const double mu_t = mu(t), mu_next = mu(t + 1.0);
    c.na1 = (float)(mu_next / (1.0 - prod * mu_next));
    c.na2 = (float)((1.0 - mu_t) / (1.0 - prod));
  }
  if (o == FORGE_RADAM) {
    const double b2t = std::pow(b2, t);
    const double rho_inf = 2.0 / (1.0 - b2) - 1.0;
    const double rho_t = rho_inf - 2.0 * t * b2t / (1.0 - b2t);
    c.rect = rho_t > 5.0 ? 1 : 0;
    if (c.rect) {
      const double r = std::sqrt((rho_t - 4.0) * (rho_t - 2.0) * rho_inf / ((rho_inf - 4.0) * (rho_inf - 2.0) * rho_t));
      c.rc = (float)(r * std::sqrt(1.0 - b2t) / (1.0 - std::pow(b1, t)));
    }
  }
  c.keyW = sr_key(seed, (uint64_t)step, 0);
  c.keyM = sr_key(seed, (uint64_t)step, 1);
  c.keyV = sr_key(seed, (uint64_t)step, 2);
  c.sr = h->round == FORGE_ROUND_SR ? 0xFFFFFFFFu : 0u;
  return a;
}

}  // namespace

extern "C" {

namespace {
thread_local hipError_t g_last_hip = hipSuccess;

forge_status hip_status(hipError_t e) {
  if (e == hipSuccess) return FORGE_OK;
  g_last_hip = e;
  return FORGE_E_HIP;
}
}  // namespace

forge_status forge_wgrad_check(const forge_mat* X, const forge_mat* dY, const forge_mat* W, const forge_state* m,
                               const forge_state* v, const forge_hyper* h, int64_t step) {
  Plan pl;
  return validate(X, dY, W, m, v, h, step, pl);
}

forge_status forge_wgrad_step(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m, forge_state* v,
                              const forge_hyper* h, int64_t step, uint64_t seed, void* stream) {
  Plan pl;
  forge_status st = validate(X, dY, W, m, v, h, step, pl);
  if (st != FORGE_OK || pl.empty) return st;
  const KArgs a = make_args(X, dY, W, m, v, h, step, seed, pl);
  return hip_status(launch_fused(a, pl.in_fmt, pl.w_fmt, h->opt, pl.m_fmt, pl.v_fmt, (hipStream_t)stream));
}

forge_status forge_wgrad_step_fp8w(const forge_mat* X, const forge_mat* dY, forge_state* W, forge_state* m,
                                   forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed, void* stream) {
  if (!W) return FORGE_E_NULL;
  Plan pl;
  forge_status st = validate(X, dY, &W->q, m, v, h, step, pl, W);
  if (st != FORGE_OK || pl.empty) return st;
  KArgs a = make_args(X, dY, &W->q, m, v, h, step, seed, pl);
  a.wsc = W->scale;
  return hip_status(launch_fused_fp8w(a, h->opt, pl.m_fmt, pl.v_fmt, (hipStream_t)stream));
}

forge_status forge_wgrad_check_fp8w(const forge_mat* X, const forge_mat* dY, const forge_state* W,
                                    const forge_state* m, const forge_state* v, const forge_hyper* h, int64_t step) {
  if (!W) return FORGE_E_NULL;
  Plan pl;
  return validate(X, dY, &W->q, m, v, h, step, pl, W);
}

forge_status forge_dgrad_fp8w(const forge_mat* dY, const forge_state* W, forge_mat* dX, void* stream) {
  if (!W) return FORGE_E_NULL;
  DgArgs g;
  bool fast = false;
  const forge_status st = check_dgrad(dY, &W->q, dX, g, fast, W);
  if (st != FORGE_OK) return st;
  // the bf16 matrix-core kernel: 16-byte rows of dY (8 bf16) and W (16
  // codes), whole 16-byte segments, buffer offsets within 32 bits
  const int64_t N = dY->cols, K = W->q.cols;
  const bool fast8 = dY->dtype == FORGE_BF16 && N % 8 == 0 && K % 16 == 0 && vec_ok(dY->data, dY->ld, 8, 2) &&
                     vec_ok(W->q.data, W->q.ld, 16, 1) && (uint64_t)dY->rows * (uint64_t)dY->ld * 2 < (1ull << 31) &&
                     (uint64_t)N * (uint64_t)W->q.ld < (1ull << 31) &&
                     (uint64_t)N * (uint64_t)(K / W->block) * 4 < (1ull << 31);
  return hip_status(launch_dgrad_fp8w(g, fast8, (hipStream_t)stream));
}

forge_status forge_wgrad_step_group(const forge_layer* layers, int32_t n, const forge_hyper* h, int64_t step,
                                    void* stream) {
  if (n < 1 || n > FORGE_GROUP_MAX) return FORGE_E_SHAPE;
  if (!layers || !h) return FORGE_E_NULL;
  Plan pl[FORGE_GROUP_MAX];
  for (int i = 0; i < n; ++i) {
    const forge_layer& L = layers[i];
    const forge_status st = validate(L.X, L.dY, L.W, L.m, L.v, h, step, pl[i]);
    if (st != FORGE_OK) return st;
  }
  // one kernel instantiation serves the group: identical formats
  int ref = -1;
  for (int i = 0; i < n; ++i) {
    if (pl[i].empty) continue;
    if (ref < 0) { ref = i; continue; }
    const Plan& a = pl[ref];
    const Plan& b = pl[i];
    if (a.in_fmt != b.in_fmt || a.w_fmt != b.w_fmt || a.m_fmt != b.m_fmt || a.v_fmt != b.v_fmt ||
        a.block != b.block)
      return FORGE_E_UNSUPPORTED;
  }
  if (ref < 0) return FORGE_OK;
  // layers are independent: nothing one layer writes may overlap any buffer of another
  Range outs[FORGE_GROUP_MAX][5], ins[FORGE_GROUP_MAX][2];
  for (int i = 0; i < n; ++i) {
    const forge_layer& L = layers[i];
    layer_ranges(L.X, L.dY, L.W, L.m, L.v, pl[i], outs[i], ins[i]);
  }
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      if (i == j) continue;
      for (int p = 0; p < 5; ++p) {
        for (int q = 0; q < 5; ++q)
          if (overlap(outs[i][p], outs[j][q])) return FORGE_E_ALIAS;
        for (int q = 0; q < 2; ++q)
          if (overlap(outs[i][p], ins[j][q])) return FORGE_E_ALIAS;
      }
    }
  // eligible layers share one launch; the others get their own
  GroupArgs g;
  std::memset(&g, 0, sizeof(g));
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    if (pl[i].empty) continue;
    const forge_layer& L = layers[i];
    const KArgs a = make_args(L.X, L.dY, L.W, L.m, L.v, h, step, L.seed, pl[i]);
    if (group_eligible(a, pl[i].in_fmt)) {
      g.layer[g.n] = a;
      g.first_tile[g.n] = (int32_t)tiles;
      tiles += (int64_t)a.tiles_n * a.tiles_k;
      ++g.n;
    } else {
      const forge_status st =
          hip_status(launch_fused(a, pl[i].in_fmt, pl[i].w_fmt, h->opt, pl[i].m_fmt, pl[i].v_fmt, (hipStream_t)stream));
      if (st != FORGE_OK) return st;
    }
  }
  if (g.n == 0) return FORGE_OK;
  g.first_tile[g.n] = (int32_t)tiles;
  return hip_status(launch_fused_group(g, pl[ref].w_fmt, h->opt, pl[ref].m_fmt, pl[ref].v_fmt, (hipStream_t)stream));
}

forge_status forge_wgrad_unfused(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m,
                                 forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed, void* dW,
                                 int32_t dW_dtype, void* stream) {
  Plan pl;
  forge_status st = validate(X, dY, W, m, v, h, step, pl);
  if (st != FORGE_OK) return st;
  if (dW_dtype != FORGE_F32 && dW_dtype != FORGE_BF16) return FORGE_E_DTYPE;
  if (pl.empty) return FORGE_OK;
  if (dW == nullptr) return FORGE_E_NULL;
  if (!aligned(dW, 16)) return FORGE_E_ALIGN;
  const Range ws = raw_range(dW, (uint64_t)pl.N * (uint64_t)pl.K * (uint64_t)elem_size(dW_dtype));
  Range outs[5], ins[2];
  layer_ranges(X, dY, W, m, v, pl, outs, ins);
  for (const Range& r : outs)
    if (overlap(ws, r)) return FORGE_E_ALIAS;
  for (const Range& r : ins)
    if (overlap(ws, r)) return FORGE_E_ALIAS;
  KArgs a = make_args(X, dY, W, m, v, h, step, seed, pl);
  a.dW = dW;
  a.dw_fmt = dW_dtype == FORGE_F32 ? FMT_F32 : FMT_BF16;
  a.vec_dw = ((pl.K % 4) == 0 && pitch_ok(pl.K, 4)) ? 1 : 0;   // the workspace is 16-byte aligned with ld = K
  hipError_t e = launch_gemm(a, pl.in_fmt, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_step(a, pl.w_fmt, h->opt, pl.m_fmt, pl.v_fmt, (hipStream_t)stream);
  return hip_status(e);
}

forge_status forge_wgrad_accumulate(const forge_mat* X, const forge_mat* dY, forge_mat* acc, int32_t first,
                                    void* stream) {
  Plan pl;
  forge_status st = validate_inputs(X, dY, pl);
  if (st != FORGE_OK) return st;
  if ((st = check_acc(acc, pl.N, pl.K)) != FORGE_OK) return st;
  const Range ra = mat_range(*acc);
  if (overlap(ra, mat_range(*X)) || overlap(ra, mat_range(*dY))) return FORGE_E_ALIAS;
  if (pl.empty) return FORGE_OK;
  KArgs a;
  std::memset(&a, 0, sizeof(a));
  input_args(X, dY, pl, a);
  acc_args(acc, a);
  a.dw_add = first ? 0 : 1;
  return hip_status(launch_gemm(a, pl.in_fmt, (hipStream_t)stream));
}

forge_status forge_wgrad_step_accumulated(const forge_mat* X, const forge_mat* dY, forge_mat* acc, forge_mat* W,
                                          forge_state* m, forge_state* v, const forge_hyper* h, int64_t step,
                                          uint64_t seed, void* stream) {
  Plan pl;
  forge_status st = validate(X, dY, W, m, v, h, step, pl);
  if (st != FORGE_OK) return st;
  if ((st = check_acc(acc, pl.N, pl.K)) != FORGE_OK) return st;
  Range outs[5], ins[2];
  layer_ranges(X, dY, W, m, v, pl, outs, ins);
  const Range ra = mat_range(*acc);
  for (const Range& r : outs)
    if (overlap(ra, r)) return FORGE_E_ALIAS;
  for (const Range& r : ins)
    if (overlap(ra, r)) return FORGE_E_ALIAS;
  if (pl.empty) return FORGE_OK;
  KArgs a = make_args(X, dY, W, m, v, h, step, seed, pl);
  acc_args(acc, a);
  // aligned bf16: one fused kernel adds the accumulator to the tile in the
  // epilogue; otherwise this micro-batch is added into the accumulator and
  // the step reads it back (the same fp32 addition, so the same result)
  if (pl.in_fmt == FORGE_BF16 && a.dma_ok && a.vec_state && a.vec_dw && pl.K % 4 == 0)
    return hip_status(launch_fused_acc(a, pl.w_fmt, h->opt, pl.m_fmt, pl.v_fmt, (hipStream_t)stream));
  a.dw_add = 1;
  hipError_t e = launch_gemm(a, pl.in_fmt, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_step(a, pl.w_fmt, h->opt, pl.m_fmt, pl.v_fmt, (hipStream_t)stream);
  return hip_status(e);
}

forge_status forge_dgrad(const forge_mat* dY, const forge_mat* W, forge_mat* dX, void* stream) {
  DgArgs g;
  bool fast = false;
  const forge_status st = check_dgrad(dY, W, dX, g, fast);
  if (st != FORGE_OK) return st;
  return hip_status(launch_dgrad(g, fast, (hipStream_t)stream));
}

int64_t forge_dgrad_workspace_bytes(int64_t BT, int64_t N, int64_t K) {
  if (BT <= 0 || N <= 0 || K <= 0 || BT >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31)) return 0;
  const int s = dgrad_splits(BT, N, K);
  return s > 1 ? (int64_t)s * BT * K * 4 : 0;
}

// The workspace of the split dX kernel, checked against every buffer of the
// call (`others`), and the split recorded in g; no-op where no split applies.
static forge_status attach_dgrad_workspace(DgArgs& g, bool fast, void* workspace, int64_t workspace_bytes,
                                           const Range* others, int n_others) {
  if (workspace_bytes < 0) return FORGE_E_SHAPE;
  const int64_t need = forge_dgrad_workspace_bytes(g.BT, g.N, g.K);
  if (!fast || need == 0) return FORGE_OK;
  if (!workspace) return FORGE_E_NULL;
  if (workspace_bytes < need) return FORGE_E_SHAPE;
  if (!aligned(workspace, 16)) return FORGE_E_ALIGN;
  const Range rw = raw_range(workspace, (uint64_t)need);
  for (int i = 0; i < n_others; ++i)
    if (overlap(rw, others[i])) return FORGE_E_ALIAS;
  g.splits = dgrad_splits(g.BT, g.N, g.K);
  g.ws = static_cast<float*>(workspace);
  return FORGE_OK;
}

forge_status forge_dgrad_split(const forge_mat* dY, const forge_mat* W, forge_mat* dX, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  DgArgs g;
  bool fast = false;
  forge_status st = check_dgrad(dY, W, dX, g, fast);
  if (st != FORGE_OK) return st;
  const Range others[3] = {mat_range(*dY), mat_range(*W), mat_range(*dX)};
  if ((st = attach_dgrad_workspace(g, fast, workspace, workspace_bytes, others, 3)) != FORGE_OK) return st;
  return hip_status(launch_dgrad(g, fast, (hipStream_t)stream));
}

forge_status forge_dgrad_split_noalloc(const forge_mat* dY, const forge_mat* W, forge_mat* dX, void* stream) {
  DgArgs g;
  bool fast = false;
  const forge_status st = check_dgrad(dY, W, dX, g, fast);
  if (st != FORGE_OK) return st;
  const int64_t need = fast ? forge_dgrad_workspace_bytes(g.BT, g.N, g.K) : 0;
  if (need > FORGE_DGRAD_SCRATCH_BYTES) return FORGE_E_SCRATCH;
  if (need > 0) g.splits = dgrad_splits(g.BT, g.N, g.K);
  return hip_status(launch_dgrad_scratch(g, fast, (hipStream_t)stream));
}

static forge_status backward_step(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m,
                                  forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed, forge_mat* dX,
                                  bool split, void* workspace, int64_t workspace_bytes, void* stream) {
  Plan pl;
  forge_status st = validate(X, dY, W, m, v, h, step, pl);
  if (st != FORGE_OK) return st;
  DgArgs g;
  bool fast = false;
  if ((st = check_dgrad(dY, W, dX, g, fast)) != FORGE_OK) return st;
  Range outs[5], ins[2];
  layer_ranges(X, dY, W, m, v, pl, outs, ins);
  const Range rx = mat_range(*dX);
  for (const Range& r : outs)
    if (overlap(rx, r)) return FORGE_E_ALIAS;
  for (const Range& r : ins)
    if (overlap(rx, r)) return FORGE_E_ALIAS;
  if (split) {
    const Range others[8] = {outs[0], outs[1], outs[2], outs[3], outs[4], ins[0], ins[1], rx};
    if ((st = attach_dgrad_workspace(g, fast, workspace, workspace_bytes, others, 8)) != FORGE_OK) return st;
  }
  // stream order is the contract: dX reads W before the fused step rewrites it
  hipError_t e = launch_dgrad(g, fast, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  if (pl.empty) return FORGE_OK;
  const KArgs a = make_args(X, dY, W, m, v, h, step, seed, pl);
  return hip_status(launch_fused(a, pl.in_fmt, pl.w_fmt, h->opt, pl.m_fmt, pl.v_fmt, (hipStream_t)stream));
}

forge_status forge_backward_step(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m, forge_state* v,
                                 const forge_hyper* h, int64_t step, uint64_t seed, forge_mat* dX, void* stream) {
  return backward_step(X, dY, W, m, v, h, step, seed, dX, false, nullptr, 0, stream);
}

forge_status forge_backward_step_split(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m,
                                       forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed,
                                       forge_mat* dX, void* workspace, int64_t workspace_bytes, void* stream) {
  return backward_step(X, dY, W, m, v, h, step, seed, dX, true, workspace, workspace_bytes, stream);
}

forge_status forge_debug_sr_bf16(const float* in, uint16_t* out, int64_t n, uint64_t seed, int64_t step,
                                 uint32_t tensor_id, void* stream) {
  if (n < 0 || (uint64_t)n >= (1ull << 32)) return FORGE_E_SHAPE;
  if (step < 1) return FORGE_E_STEP;
  if (n == 0) return FORGE_OK;
  if (!in || !out) return FORGE_E_NULL;
  if (!aligned(in, 4) || !aligned(out, 2)) return FORGE_E_ALIGN;
  if (overlap(raw_range(in, (uint64_t)n * 4), raw_range(out, (uint64_t)n * 2))) return FORGE_E_ALIAS;
  const uint32_t key = sr_key(seed, (uint64_t)step, tensor_id);
  return hip_status(launch_debug_sr(in, out, (uint32_t)n, key, (hipStream_t)stream));
}

forge_status forge_debug_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0 || (uint64_t)n >= (1ull << 32)) return FORGE_E_SHAPE;
  if (n == 0) return FORGE_OK;
  if (!in || !out) return FORGE_E_NULL;
  if (!aligned(in, 4)) return FORGE_E_ALIGN;
  if (overlap(raw_range(in, (uint64_t)n * 4), raw_range(out, (uint64_t)n))) return FORGE_E_ALIAS;
  return hip_status(launch_debug_e4m3(in, out, (uint32_t)n, (hipStream_t)stream));
}

forge_status forge_debug_e4m3_sr(const float* in, uint8_t* out, int64_t n, uint64_t seed, int64_t step,
                                 void* stream) {
  if (n < 0 || (uint64_t)n >= (1ull << 32)) return FORGE_E_SHAPE;
  if (step < 1) return FORGE_E_STEP;
  if (n == 0) return FORGE_OK;
  if (!in || !out) return FORGE_E_NULL;
  if (!aligned(in, 4)) return FORGE_E_ALIGN;
  if (overlap(raw_range(in, (uint64_t)n * 4), raw_range(out, (uint64_t)n))) return FORGE_E_ALIAS;
  return hip_status(launch_debug_e4m3_sr(in, out, (uint32_t)n, sr_key(seed, (uint64_t)step, 0), (hipStream_t)stream));
}

forge_status forge_debug_quotients(uint64_t* counts, void* stream) {
  if (!counts) return FORGE_E_NULL;
  if (!aligned(counts, 8)) return FORGE_E_ALIGN;
  return hip_status(launch_debug_quotients(reinterpret_cast<unsigned long long*>(counts), (hipStream_t)stream));
}

forge_status forge_debug_quant(const float* in, uint8_t* codes, float* scales, int64_t rows, int64_t cols,
                               int32_t dtype, int32_t second_moment, int32_t block, void* stream) {
  if (dtype != FORGE_S8 && dtype != FORGE_U8 && dtype != FORGE_E4M3) return FORGE_E_DTYPE;
  if (second_moment != 0 && second_moment != 1) return FORGE_E_DTYPE;
  if ((dtype == FORGE_S8 && second_moment) || (dtype == FORGE_U8 && !second_moment)) return FORGE_E_DTYPE;
  if (!(block == 32 || block == 64 || block == 128)) return FORGE_E_SHAPE;
  if (rows < 0 || cols < 0 || cols % block != 0) return FORGE_E_SHAPE;
  if ((uint64_t)rows * (uint64_t)cols >= (1ull << 32) || rows >= (1ll << 31) || cols >= (1ll << 31))
    return FORGE_E_SHAPE;
  if (rows == 0 || cols == 0) return FORGE_OK;
  if (!in || !codes || !scales) return FORGE_E_NULL;
  if (!aligned(in, 4) || !aligned(codes, 4) || !aligned(scales, 4)) return FORGE_E_ALIGN;
  const uint64_t n = (uint64_t)rows * (uint64_t)cols;
  const Range ri = raw_range(in, n * 4), rc = raw_range(codes, n), rs = raw_range(scales, n / (uint64_t)block * 4);
  if (overlap(ri, rc) || overlap(ri, rs) || overlap(rc, rs)) return FORGE_E_ALIAS;
  return hip_status(launch_debug_quant(in, codes, scales, (int)rows, (int)cols, dtype, second_moment != 0, block,
                                       (hipStream_t)stream));
}

forge_status forge_debug_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return FORGE_E_SHAPE;
  if (bytes == 0) return FORGE_OK;
  if (!src || !dst) return FORGE_E_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FORGE_E_ALIGN;
  if (overlap(raw_range(src, (uint64_t)bytes), raw_range(dst, (uint64_t)bytes))) return FORGE_E_ALIAS;
  return hip_status(launch_debug_copy(src, dst, (uint64_t)bytes, (hipStream_t)stream));
}

forge_status forge_debug_state_stream(uint16_t* W, float* m, float* v, int64_t N, int64_t K, void* stream) {
  if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FORGE_E_SHAPE;
  if ((uint64_t)N * (uint64_t)K >= (1ull << 32) || N >= (1ll << 31) || K >= (1ll << 31)) return FORGE_E_SHAPE;
  if (N == 0 || K == 0) return FORGE_OK;
  if (!W || !m || !v) return FORGE_E_NULL;
  if (!aligned(W, 8) || !aligned(m, 16) || !aligned(v, 16)) return FORGE_E_ALIGN;
  const uint64_t n = (uint64_t)N * (uint64_t)K;
  const Range rw = raw_range(W, 2 * n), rm = raw_range(m, 4 * n), rv = raw_range(v, 4 * n);
  if (overlap(rw, rm) || overlap(rw, rv) || overlap(rm, rv)) return FORGE_E_ALIAS;
  return hip_status(launch_debug_state_stream(W, m, v, (int)N, (int)K, (hipStream_t)stream));
}

forge_status forge_debug_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20)) return FORGE_E_SHAPE;
  if (!out) return FORGE_E_NULL;
  if (!aligned(out, 4)) return FORGE_E_ALIGN;
  return hip_status(launch_debug_mfma(out, blocks, iters, (hipStream_t)stream));
}

const char* forge_last_error(void) { return hipGetErrorString(g_last_hip); }

const char* forge_status_str(forge_status s) {
  switch (s) {
    case FORGE_OK: return "FORGE_OK";
    case FORGE_E_NULL: return "FORGE_E_NULL: a required pointer is NULL";
    case FORGE_E_SHAPE: return "FORGE_E_SHAPE: shapes disagree or exceed a limit";
    case FORGE_E_DTYPE: return "FORGE_E_DTYPE: dtype not allowed here";
    case FORGE_E_ALIGN: return "FORGE_E_ALIGN: misaligned pointer";
    case FORGE_E_STEP: return "FORGE_E_STEP: step must be >= 1";
    case FORGE_E_HYPER: return "FORGE_E_HYPER: invalid optimizer or hyper-parameter";
    case FORGE_E_ALIAS: return "FORGE_E_ALIAS: an output overlaps another buffer";
    case FORGE_E_UNSUPPORTED: return "FORGE_E_UNSUPPORTED: combination not implemented";
    case FORGE_E_HIP: return "FORGE_E_HIP: HIP launch error";
    case FORGE_E_SCRATCH: return "FORGE_E_SCRATCH: the call needs more than the static scratch array holds";
  }
  return "unknown forge_status";
}

const char* forge_version(void) { return "forge-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
