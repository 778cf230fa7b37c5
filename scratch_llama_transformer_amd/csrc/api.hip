// C ABI of libslt: argument checks, the planner (parameter layout, activation
// arena and scratch offsets), and the forward / backward walks that enqueue the
// kernels of rowops.hip, gemm.hip and attention.hip on the caller's stream.
//
// Hephaistos, "Design notes": flat parameter buffer with per-tensor (offset,
// length), an activation arena filled by the forward, the backward as a
// straight reverse walk over it.  strata: a planner that sizes parameters and
// memory and validates the configuration before anything runs.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "slt_internal.h"

namespace slt {

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }

slt_status fail(slt_status code, const std::string& msg) {
  set_error(msg);
  return code;
}

slt_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SLT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return SLT_OK;
}

#define SLT_TRY(expr)                    \
  do {                                   \
    slt_status _st = (expr);             \
    if (_st != SLT_OK) return _st;       \
  } while (0)

static inline int64_t a256(int64_t b) { return (b + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// Launch timing by class (slt_timing / slt_timing_read), for measurement:
// while it is on, a pair of HIP events brackets every launch of a class on
// the stream that launch runs on; the pairs are kept until they are read.
// ---------------------------------------------------------------------------
enum { TM_FWD = 0, TM_DX = 1, TM_DW = 2, TM_AFWD = 3, TM_ABWD = 4 };
struct TmRec {
  int cls;
  hipEvent_t a, b;
};
static std::mutex g_tm_mu;
static std::atomic<bool> g_tm_on{false};
static std::vector<TmRec> g_tm_recs;
static std::vector<hipEvent_t> g_tm_pool;  // events for reuse (kept until the process ends)

static hipEvent_t tm_event() {  // with g_tm_mu held
  if (!g_tm_pool.empty()) {
    hipEvent_t e = g_tm_pool.back();
    g_tm_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

struct Timed {
  int cls;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(int c, hipStream_t st) : cls(c), s(st) {
    if (!g_tm_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_tm_mu);
    a = tm_event();
    b = tm_event();
    if (!a || !b || hipEventRecord(a, s) != hipSuccess) {
      (void)hipGetLastError();
      drop_locked();
    }
  }
  // the bracketed call launched nothing: forget the pair
  void drop() {
    if (!a && !b) return;
    std::lock_guard<std::mutex> lk(g_tm_mu);
    drop_locked();
  }
  void drop_locked() {
    if (a) g_tm_pool.push_back(a);
    if (b) g_tm_pool.push_back(b);
    a = b = nullptr;
  }
  ~Timed() {
    if (!a) return;
    const bool ok = hipEventRecord(b, s) == hipSuccess;
    if (!ok) (void)hipGetLastError();
    std::lock_guard<std::mutex> lk(g_tm_mu);
    if (ok) g_tm_recs.push_back(TmRec{cls, a, b});
    else drop_locked();
  }
};

// ---------------------------------------------------------------------------
// Planner
// ---------------------------------------------------------------------------
struct LayerP {
  int64_t norm1 = -1, norm1b = -1, qkvw = -1, wo = -1, norm2 = -1, w1 = -1, w3 = -1, w2 = -1, fcin = -1, wout = -1;
};

struct LayerA {
  int64_t n1, r1, mu1, qkv, o, ores, lse, n2, r2, ab, h;  // byte offsets in the arena (-1: absent)
};

struct Plan {
  slt_config c;
  int d, N, qd, kd, qkv_w, in_w, ou_w;
  bool llama, bf;
  int64_t es;  // element size of activations / compute weights
  std::vector<slt_tensor> tensors;
  std::vector<LayerP> lp;
  int64_t wte, normf, normfb = -1, head, n_params;
  // arena
  std::vector<int64_t> xs;
  std::vector<LayerA> la;
  int64_t nf, rf, muf, z, cs, act_bytes;
  // scratch
  // Gradient buffers the layer weight gradients read run in three sets (set
  // l % 3 for layer l; dx of set l % 3 holds the gradient at layer l's
  // output), since those products run one layer behind the backward walk on
  // a second stream.  dy1 / dy2: masked output gradients of the dropped
  // projections (dropout on).
  int64_t dx[3], dx2[3], dbig[3], dqkv[3], dy1[3], dy2[3];
  int64_t rowloss, dmid, dn, delta, normws, normws_each, embws, gemmws, gemmws_bytes, scratch_bytes;
  int dbig_w, dmid_w;
};

static slt_status validate(const slt_config* c) {
  if (!c) return fail(SLT_EINVAL, "config is NULL");
  if (c->V <= 0 || c->C <= 0 || c->H <= 0 || c->Hkv <= 0 || c->L <= 0 || c->T <= 0 || c->B <= 0 || c->F <= 0)
    return fail(SLT_EINVAL, "all of V, C, H, Hkv, L, T, B, F must be positive");
  if (c->C % c->H) return fail(SLT_EINVAL, "C must be a multiple of H (C = H * d)");
  if (c->H % c->Hkv) return fail(SLT_EINVAL, "H must be a multiple of Hkv");
  const int d = c->C / c->H;
  if (c->R < 0 || c->R > d || (c->R & 1)) return fail(SLT_EINVAL, "R must be even and 0 <= R <= d");
  if (d > 64) return fail(SLT_EUNSUPPORTED, "head dimension above 64");
  if (c->rope_mode != SLT_ROPE_HALF && c->rope_mode != SLT_ROPE_PAIRS) return fail(SLT_EINVAL, "bad rope_mode");
  if (c->block != SLT_BLOCK_LLAMA && c->block != SLT_BLOCK_PARALLEL) return fail(SLT_EINVAL, "bad block");
  if (c->act != SLT_F32 && c->act != SLT_BF16) return fail(SLT_EINVAL, "bad act dtype");
  if (c->C > 4096 || (c->C % 8 && c->C > 512)) return fail(SLT_EUNSUPPORTED, "C above 4096 (or above 512 unaligned)");
  if (!(c->eps >= 0.f) || !(c->rope_base > 0.f)) return fail(SLT_EINVAL, "eps must be >= 0 and rope_base > 0");
  if (!(c->dropout >= 0.f && c->dropout < 1.f)) return fail(SLT_EINVAL, "dropout must satisfy 0 <= p < 1");
  const int64_t N = (int64_t)c->B * c->T;
  if (N > (1 << 30) || (int64_t)c->V * c->C > ((int64_t)1 << 40)) return fail(SLT_EUNSUPPORTED, "sizes too large");
  return SLT_OK;
}

static void add_tensor(Plan& p, const std::string& name, int64_t rows, int64_t cols, int32_t decay, int64_t& off) {
  slt_tensor t;
  memset(&t, 0, sizeof(t));
  snprintf(t.name, sizeof(t.name), "%s", name.c_str());
  t.offset = off;
  t.rows = rows;
  t.cols = cols;
  t.numel = rows * cols;
  t.decay = decay;
  p.tensors.push_back(t);
  off += t.numel;
}

static slt_status make_plan(const slt_config* cfg, Plan& p) {
  SLT_TRY(validate(cfg));
  const slt_config& c = *cfg;
  p.c = c;
  p.d = c.C / c.H;
  p.N = c.B * c.T;
  p.qd = c.H * p.d;
  p.kd = c.Hkv * p.d;
  p.qkv_w = p.qd + 2 * p.kd;
  p.llama = c.block == SLT_BLOCK_LLAMA;
  p.bf = c.act == SLT_BF16;
  p.es = p.bf ? 2 : 4;
  p.in_w = p.llama ? 2 * c.F : p.qkv_w + c.F;
  p.ou_w = p.qd + c.F;

  // parameters (every tensor decays: the pages exclude none)
  int64_t off = 0;
  p.tensors.clear();
  p.lp.assign(c.L, LayerP{});
  p.wte = off;
  add_tensor(p, "wte", c.V, c.C, 1, off);
  for (int l = 0; l < c.L; ++l) {
    const std::string pre = "h" + std::to_string(l) + ".";
    LayerP& L = p.lp[l];
    if (p.llama) {
      L.norm1 = off; add_tensor(p, pre + "attn_norm", 1, c.C, 1, off);
      L.qkvw = off; add_tensor(p, pre + "qkvw", p.qkv_w, c.C, 1, off);
      L.wo = off; add_tensor(p, pre + "w_o", c.C, p.qd, 1, off);
      L.norm2 = off; add_tensor(p, pre + "mlp_norm", 1, c.C, 1, off);
      L.w1 = off; add_tensor(p, pre + "w1", c.F, c.C, 1, off);
      L.w3 = off; add_tensor(p, pre + "w3", c.F, c.C, 1, off);
      L.w2 = off; add_tensor(p, pre + "w2", c.C, c.F, 1, off);
    } else {
      L.norm1 = off; add_tensor(p, pre + "ln_g", 1, c.C, 1, off);
      L.norm1b = off; add_tensor(p, pre + "ln_b", 1, c.C, 1, off);
      L.qkvw = off; add_tensor(p, pre + "qkvw", p.qkv_w, c.C, 1, off);
      L.fcin = off; add_tensor(p, pre + "fc_in", c.F, c.C, 1, off);
      L.wout = off; add_tensor(p, pre + "w_out", c.C, p.ou_w, 1, off);
    }
  }
  if (p.llama) {
    p.normf = off; add_tensor(p, "norm_f", 1, c.C, 1, off);
  } else {
    p.normf = off; add_tensor(p, "lnf_g", 1, c.C, 1, off);
    p.normfb = off; add_tensor(p, "lnf_b", 1, c.C, 1, off);
  }
  p.head = off;
  add_tensor(p, "lm_head", c.V, c.C, 1, off);
  p.n_params = off;

  // activation arena
  const int64_t N = p.N, es = p.es, C = c.C;
  int64_t a = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = a;
    a += a256(bytes);
    return o;
  };
  const int nx = p.llama ? 2 * c.L + 1 : c.L + 1;
  p.xs.resize(nx);
  for (int i = 0; i < nx; ++i) p.xs[i] = take(N * C * es);
  p.la.resize(c.L);
  for (int l = 0; l < c.L; ++l) {
    LayerA& A = p.la[l];
    A.n1 = take(N * C * es);
    A.r1 = take(N * 4);
    A.mu1 = p.llama ? -1 : take(N * 4);
    A.lse = take((int64_t)c.B * c.H * c.T * 4);
    A.ores = p.bf ? take(N * p.qd * es) : -1;  // bf16 rounding residual of the attention output
    if (p.llama) {
      A.qkv = take(N * p.qkv_w * es);
      A.o = take(N * p.qd * es);
      A.n2 = take(N * C * es);
      A.r2 = take(N * 4);
      A.ab = take(N * 2 * c.F * es);
      A.h = take(N * c.F * es);
    } else {
      A.qkv = take(N * p.in_w * es);   // [q | k | v | fc_in pre-activation]
      A.o = take(N * p.ou_w * es);     // [attention output | gelu output]
      A.n2 = A.r2 = A.ab = A.h = -1;
    }
  }
  p.nf = take(N * C * es);
  p.rf = take(N * 4);
  p.muf = p.llama ? -1 : take(N * 4);
  p.z = take(N * (int64_t)c.V * es);
  p.cs = take((int64_t)c.T * std::max(c.R, 2) * 4);
  p.act_bytes = a;

  // scratch
  p.dbig_w = p.llama ? std::max(2 * c.F, p.qkv_w) : p.in_w;
  p.dmid_w = p.llama ? std::max(c.F, p.qd) : p.ou_w;
  int64_t s = 0;
  auto takes = [&](int64_t bytes) {
    const int64_t o = s;
    s += a256(bytes);
    return o;
  };
  p.rowloss = takes(N * 4);
  for (int k = 0; k < 3; ++k) {
    p.dx[k] = takes(N * C * es);
    p.dx2[k] = takes(N * C * es);  // residual-stream gradient between the two sub-blocks of a layer
    p.dbig[k] = takes(N * p.dbig_w * es);
    p.dqkv[k] = p.llama ? takes(N * p.qkv_w * es) : -1;  // kept apart from dbig until the layer's dW launch
    p.dy1[k] = c.dropout > 0.f ? takes(N * C * es) : -1;
    p.dy2[k] = c.dropout > 0.f && p.llama ? takes(N * C * es) : -1;
  }
  p.dmid = takes(N * p.dmid_w * es);
  p.dn = takes(N * C * es);
  p.delta = takes(attention_bwd_ws(c.B, c.H, c.T));
  // one partial buffer per norm of the backward (final norm, then two per
  // layer): their column sums run on the second stream, behind the walk
  p.normws_each = a256(norm_bwd_ws(p.N, c.C));
  p.normws = takes(p.normws_each * (2 * (int64_t)c.L + 1));
  p.embws = takes(embedding_bwd_ws(N, c.V));
  // split-K partials of the weight gradients
  p.gemmws_bytes = 64ll << 20;
  p.gemmws = takes(p.gemmws_bytes);
  p.scratch_bytes = s;
  return SLT_OK;
}

// ---------------------------------------------------------------------------
// GEMM helpers for the three forms
// ---------------------------------------------------------------------------
struct Ctx {
  const Plan& p;
  hipStream_t s;
  char* acts;
  char* scr;
  const char* params;
  int dt;  // activation dtype
  GradW gw{};  // how parameter gradients are written (scale, accumulate)
  void* A(int64_t off) const { return acts + off; }
  void* S(int64_t off) const { return scr + off; }
  const void* P(int64_t off) const { return params + off * p.es; }
};

// Inverted dropout of one site of one layer (0: embedding output, 1:
// attention projection output, 2: MLP output, 3: attention weights); off
// when p = 0.  A kept
// element is scaled by 1/(1-p) rounded to fp32; the mask bit of element e
// compares one Philox-4x32-10 word with floor(p 2^32) (drop_mult).
static Drop make_drop(const slt_config& c, int site, int layer) {
  Drop d;
  if (!(c.dropout > 0.f)) return d;
  d.on = true;
  d.thr = (uint32_t)floor((double)c.dropout * 4294967296.0);
  d.scale = (float)(1.0 / (1.0 - (double)c.dropout));
  d.k0 = (uint32_t)c.dropout_seed;
  d.k1 = (uint32_t)(c.dropout_seed >> 32);
  d.site = site;
  d.layer = layer;
  return d;
}

// y[M, N] = drop(x[M, K] W[N, K]^T) (+ R)
static slt_status proj(const Ctx& x, int M, int N, int K, const void* X, int64_t ldx, const void* W, void* Y,
                       int64_t ldy, const void* R, int64_t ldr, Drop drop = {}) {
  GemmArgs g{M, N, K, X, ldx, true, W, (int64_t)K, true, Y, ldy, R, ldr, x.dt, x.dt, nullptr, 0};
  g.drop = drop;
  Timed tm(TM_FWD, x.s);
  return launch_gemm(g, x.s);
}

// dX[M, K] = dY[M, N] W[N, K]   (W row stride ldw)
static slt_status proj_dx(const Ctx& x, int M, int N, int K, const void* dY, int64_t lddy, const void* W,
                          int64_t ldw, void* dX, int64_t lddx) {
  GemmArgs g{M, K, N, dY, lddy, true, W, ldw, false, dX, lddx, nullptr, 0, x.dt, x.dt, nullptr, 0};
  Timed tm(TM_DX, x.s);
  return launch_gemm(g, x.s);
}

// dW[N, K] = alpha dY[M, N]^T X[M, K] (+ dW when accumulating)  (fp32 out, row stride ldw)
static slt_status proj_dw(const Ctx& x, int M, int N, int K, const void* dY, int64_t lddy, const void* X,
                          int64_t ldx, float* dW, int64_t ldw) {
  GemmArgs g{N, K, M, dY, lddy, false, X, ldx, false, dW, ldw, x.gw.accumulate ? dW : nullptr, ldw, x.dt, SLT_F32,
             reinterpret_cast<float*>(x.S(x.p.gemmws)), x.p.gemmws_bytes};
  g.alpha = x.gw.alpha;
  return launch_gemm(g, x.s);
}

// [a | b] = n [W1; W3]^T and h = swiglu(a, b): one fused launch where the
// fused kernel applies (bf16, wide enough grids), else the projection and the
// element kernel.
static slt_status mlp_in(int M, int F, int C, const void* n, const void* w13, char* ab, void* h, int dt,
                         hipStream_t s) {
  if (dt == SLT_BF16) {
    Timed tm(TM_FWD, s);
    const slt_status st = launch_gemm_swiglu_fwd(M, F, C, n, C, w13, ab, 2 * F, h, F, s);
    if (st != SLT_EUNSUPPORTED) return st;
    tm.drop();
  }
  GemmArgs g{M, 2 * F, C, n, C, true, w13, C, true, ab, 2 * F, nullptr, 0, dt, dt, nullptr, 0};
  {
    Timed tm(TM_FWD, s);
    SLT_TRY(launch_gemm(g, s));
  }
  const int64_t es = dt == SLT_BF16 ? 2 : 4;
  return launch_swiglu_fwd(ab, ab + F * es, h, M, F, 2 * F, 2 * F, F, dt, s);
}

// y = n W^T over N columns and u = gelu(y[:, col0:]).
static slt_status proj_gelu(int M, int N, int K, const void* n, const void* w, char* y, int64_t ldy, int col0,
                            char* u, int64_t ldu, int dt, hipStream_t s) {
  GemmArgs g{M, N, K, n, K, true, w, K, true, y, ldy, nullptr, 0, dt, dt, nullptr, 0};
  {
    Timed tm(TM_FWD, s);
    SLT_TRY(launch_gemm(g, s));
  }
  const int64_t es = dt == SLT_BF16 ? 2 : 4;
  return launch_gelu_fwd(y + col0 * es, u, M, N - col0, ldy, ldu, dt, s);
}

// Whether the step stores q and k rotated: the bf16 attention kernels read
// them rotated and rounded once (RoPE in the QKV projection's epilogue).
static bool rope_in_projection(const Plan& p) { return flash_eligible(p.c.act, p.d); }

// y[M, N] = n W^T (row stride ldy) whose first (H + Hkv) d columns are the q
// and k heads, RoPE'd by row position m % T before the one rounding: the
// projection's epilogue where it applies, else the plain product and RoPE in
// place.  R = 0: the plain product.
static slt_status rope_proj(int M, int N, int K, const void* n, const void* w, char* y, int64_t ldy, int T, int H,
                            int Hkv, int d, int R, int mode, const float* cs, int dt, hipStream_t s) {
  GemmArgs g{M, N, K, n, K, true, w, K, true, y, ldy, nullptr, 0, dt, dt, nullptr, 0};
  if (R == 0) {
    Timed tm(TM_FWD, s);
    return launch_gemm(g, s);
  }
  RopeEpi r;
  r.cs = cs;
  r.T = T;
  r.d = d;
  r.R = R;
  r.end = (H + Hkv) * d;
  r.half = mode == SLT_ROPE_HALF;
  {
    Timed tm(TM_FWD, s);
    const slt_status st = launch_gemm_rope(g, r, s);
    if (st != SLT_EUNSUPPORTED) return st;
    tm.drop();
  }
  {
    Timed tm(TM_FWD, s);
    SLT_TRY(launch_gemm(g, s));
  }
  const int64_t es = dt == SLT_BF16 ? 2 : 4;
  SLT_TRY(launch_rope(y, ldy, y, ldy, M, T, H, d, R, mode, cs, 1.0f, dt, s));
  return launch_rope(y + (int64_t)H * d * es, ldy, y + (int64_t)H * d * es, ldy, M, T, Hkv, d, R, mode, cs, 1.0f,
                     dt, s);
}

static slt_status proj_rope(const Plan& p, const Ctx& x, int M, int N, int K, const void* n, const void* w, char* y,
                            int64_t ldy, const float* cs) {
  const slt_config& c = p.c;
  return rope_proj(M, N, K, n, w, y, ldy, c.T, c.H, c.Hkv, p.d, c.R, c.rope_mode, cs, x.dt, x.s);
}

// [da | db] from dh = dY W2 (stored in dh_buf) and the cached [a | b].
static slt_status mlp_in_bwd(int M, int F, int C, const void* dy, const void* w2, const char* ab, char* dab,
                             void* dh_buf, int dt, hipStream_t s) {
  GemmArgs g{M, F, C, dy, C, true, w2, F, false, dh_buf, F, nullptr, 0, dt, dt, nullptr, 0};
  {
    Timed tm(TM_DX, s);
    SLT_TRY(launch_gemm(g, s));
  }
  const int64_t es = dt == SLT_BF16 ? 2 : 4;
  return launch_swiglu_bwd(ab, ab + F * es, dh_buf, dab, dab + F * es, M, F, 2 * F, 2 * F, F, 2 * F, 2 * F, dt, s);
}

// Weight gradients deferred to the end of a layer's backward walk, so that
// they run as one grouped launch (every product fits the grouped kernel) or
// else one GEMM each, in the order they were added.
struct DwList {
  struct Item {
    int M, N, K;
    const void* dY;
    int64_t lddy;
    const void* X;
    int64_t ldx;
    float* dW;
    int64_t ldw;
  };
  Item it[6];
  int n = 0;
  // dW[N, K] = dY[M, N]^T X[M, K]
  void add(int M, int N, int K, const void* dY, int64_t lddy, const void* X, int64_t ldx, float* dW, int64_t ldw) {
    it[n++] = Item{M, N, K, dY, lddy, X, ldx, dW, ldw};
  }
};

static slt_status flush_dw(const Ctx& x, DwList& L) {
  Timed tm(TM_DW, x.s);
  bool group = x.dt == SLT_BF16 && L.n > 1;
  GroupItem g[6];
  for (int i = 0; i < L.n && group; ++i) {
    const DwList::Item& t = L.it[i];
    g[i] = GroupItem{t.N, t.K, t.dY, t.lddy, t.X, t.ldx, t.dW, t.ldw, x.gw.alpha, x.gw.accumulate};
    group = t.M == L.it[0].M && gemm_group_ok(g[i], t.M);
  }
  if (group) {
    SLT_TRY(launch_gemm_group(g, L.n, L.it[0].M, reinterpret_cast<float*>(x.S(x.p.gemmws)), x.p.gemmws_bytes, x.s));
  } else {
    for (int i = 0; i < L.n; ++i) {
      const DwList::Item& t = L.it[i];
      SLT_TRY(proj_dw(x, t.M, t.N, t.K, t.dY, t.lddy, t.X, t.ldx, t.dW, t.ldw));
    }
  }
  L.n = 0;
  return SLT_OK;
}

// ---------------------------------------------------------------------------
// Forward and backward walks
// ---------------------------------------------------------------------------
static slt_status forward(const Plan& p, const Ctx& x, const int32_t* tok, float* loss) {
  const slt_config& c = p.c;
  const int N = p.N, C = c.C;
  const int64_t ldt = c.T + 1;
  float* cs = reinterpret_cast<float*>(x.A(p.cs));
  const bool rot = rope_in_projection(p);
  if (c.R > 0) SLT_TRY(launch_rope_table(c.T, c.R, c.rope_base, cs, x.s));
  SLT_TRY(launch_embedding_fwd(tok, c.B, c.T, ldt, x.P(p.wte), x.A(p.xs[0]), c.V, C, x.dt, x.s, make_drop(c, 0, 0)));
  for (int l = 0; l < c.L; ++l) {
    const LayerP& W = p.lp[l];
    const LayerA& A = p.la[l];
    AttnArgs at{};
    at.B = c.B; at.T = c.T; at.H = c.H; at.Hkv = c.Hkv; at.d = p.d; at.R = c.R; at.rope_mode = c.rope_mode;
    at.dtype = x.dt; at.cs = cs;
    at.lse = reinterpret_cast<float*>(x.A(A.lse));
    at.ores_out = A.ores >= 0 ? x.A(A.ores) : nullptr;
    at.qk_rotated = rot;
    at.drop = make_drop(c, 3, l);
    if (p.llama) {
      void* xin = x.A(p.xs[2 * l]);
      void* xmid = x.A(p.xs[2 * l + 1]);
      void* xout = x.A(p.xs[2 * l + 2]);
      SLT_TRY(launch_rmsnorm_fwd(xin, x.P(W.norm1), x.A(A.n1), (float*)x.A(A.r1), N, C, c.eps, x.dt, x.s));
      if (rot)
        SLT_TRY(proj_rope(p, x, N, p.qkv_w, C, x.A(A.n1), x.P(W.qkvw), (char*)x.A(A.qkv), p.qkv_w, cs));
      else
        SLT_TRY(proj(x, N, p.qkv_w, C, x.A(A.n1), C, x.P(W.qkvw), x.A(A.qkv), p.qkv_w, nullptr, 0));
      char* qkv = (char*)x.A(A.qkv);
      at.q = qkv; at.k = qkv + p.qd * p.es; at.v = qkv + (p.qd + p.kd) * p.es;
      at.ldq = at.ldk = at.ldv = p.qkv_w;
      at.out = x.A(A.o); at.ldo = p.qd;
      {
        Timed tm(TM_AFWD, x.s);
        SLT_TRY(launch_attention_fwd(at, x.s));
      }
      SLT_TRY(proj(x, N, C, p.qd, x.A(A.o), p.qd, x.P(W.wo), xmid, C, xin, C, make_drop(c, 1, l)));
      SLT_TRY(launch_rmsnorm_fwd(xmid, x.P(W.norm2), x.A(A.n2), (float*)x.A(A.r2), N, C, c.eps, x.dt, x.s));
      SLT_TRY(mlp_in(N, c.F, C, x.A(A.n2), x.P(W.w1), (char*)x.A(A.ab), x.A(A.h), x.dt, x.s));
      SLT_TRY(proj(x, N, C, c.F, x.A(A.h), c.F, x.P(W.w2), xout, C, xmid, C, make_drop(c, 2, l)));
    } else {
      void* xin = x.A(p.xs[l]);
      void* xout = x.A(p.xs[l + 1]);
      SLT_TRY(launch_layernorm_fwd(xin, x.P(W.norm1), x.P(W.norm1b), x.A(A.n1), (float*)x.A(A.mu1),
                                   (float*)x.A(A.r1), N, C, c.eps, x.dt, x.s));
      char* qkv = (char*)x.A(A.qkv);
      char* ou = (char*)x.A(A.o);
      // [q | k | v | a] = n W^T (q and k RoPE'd in the epilogue when the
      // attention reads them rotated) and u = gelu(a) into [o | u]
      if (rot) {
        SLT_TRY(proj_rope(p, x, N, p.in_w, C, x.A(A.n1), x.P(W.qkvw), qkv, p.in_w, cs));
        SLT_TRY(launch_gelu_fwd(qkv + p.qkv_w * p.es, ou + p.qd * p.es, N, c.F, p.in_w, p.ou_w, x.dt, x.s));
      } else {
        SLT_TRY(proj_gelu(N, p.in_w, C, x.A(A.n1), x.P(W.qkvw), qkv, p.in_w, p.qkv_w, ou + p.qd * p.es, p.ou_w, x.dt,
                          x.s));
      }
      at.q = qkv; at.k = qkv + p.qd * p.es; at.v = qkv + (p.qd + p.kd) * p.es;
      at.ldq = at.ldk = at.ldv = p.in_w;
      at.out = ou; at.ldo = p.ou_w;
      {
        Timed tm(TM_AFWD, x.s);
        SLT_TRY(launch_attention_fwd(at, x.s));
      }
      SLT_TRY(proj(x, N, C, p.ou_w, ou, p.ou_w, x.P(W.wout), xout, C, xin, C, make_drop(c, 1, l)));
    }
  }
  void* xf = x.A(p.xs.back());
  if (p.llama)
    SLT_TRY(launch_rmsnorm_fwd(xf, x.P(p.normf), x.A(p.nf), (float*)x.A(p.rf), N, C, c.eps, x.dt, x.s));
  else
    SLT_TRY(launch_layernorm_fwd(xf, x.P(p.normf), x.P(p.normfb), x.A(p.nf), (float*)x.A(p.muf),
                                 (float*)x.A(p.rf), N, C, c.eps, x.dt, x.s));
  SLT_TRY(proj(x, N, c.V, C, x.A(p.nf), C, x.P(p.head), x.A(p.z), c.V, nullptr, 0));
  SLT_TRY(launch_softmax_xent(x.A(p.z), c.V, tok, c.B, c.T, ldt, c.V, loss, nullptr, x.dt, x.S(p.rowloss), x.s));
  return SLT_OK;
}

// A second stream per device for the work of the backward that nothing in
// the walk reads (the layer weight gradients, the norm-gain column sums, the
// token sort of the embedding gradient), and the events that order it
// against the walk's stream: `ready` is recorded on the walk's stream before
// each launch there, done[k] after the launch that reads buffer set k,
// sort_done after the sort, fin after the last launch of a walk.  Created on
// first use (default priority, non-blocking); host calls that enqueue
// backward walks on one device take turns (mutex), so an event is never
// re-recorded before the waits on its last record are enqueued.
struct DwStream {
  hipStream_t s = nullptr;
  hipEvent_t ready = nullptr, done[3] = {nullptr, nullptr, nullptr}, sort_done = nullptr, fin = nullptr;
};
static std::mutex g_dw_mu;

static DwStream* dw_stream() {
  static std::map<int, DwStream> per_dev;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  auto it = per_dev.find(dev);
  if (it == per_dev.end()) {
    DwStream a;
    // The events only order the two streams of one device: a device-scope
    // release suffices, not the system-scope fence (write-back and invalidate
    // for host visibility) of a default event.  The caller's own
    // synchronisation still makes the results visible to the host.
    const unsigned ef = hipEventDisableTiming | hipEventDisableSystemFence;
    bool ok = hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&a.ready, ef) == hipSuccess;
    for (int k = 0; k < 3 && ok; ++k) ok = hipEventCreateWithFlags(&a.done[k], ef) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&a.sort_done, ef) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&a.fin, ef) == hipSuccess;
    if (!ok) {  // fall back to the walk's stream (what was created stays until exit)
      a = DwStream{};
      (void)hipGetLastError();
    }
    it = per_dev.emplace(dev, a).first;
  }
  return it->second.s ? &it->second : nullptr;
}

static slt_status hip_ok(hipError_t e, const char* what) {
  return e == hipSuccess ? SLT_OK : fail(SLT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// AdamW folded into the backward (slt_backward_adamw): each layer's update
// is enqueued as soon as its gradients are final.
struct AdamArgs {
  float* master;
  uint16_t* shadow;
  float *m, *v;
  int64_t t;
  float lr, b1, b2, eps, wd;
  const uint8_t* mask;
};

static slt_status backward(const Plan& p, const Ctx& x, const int32_t* tok, float* grads,
                           const AdamArgs* opt = nullptr) {
  const slt_config& c = p.c;
  const int N = p.N, C = c.C;
  const int64_t ldt = c.T + 1;
  const float* cs = reinterpret_cast<const float*>(x.A(p.cs));
  void* dn = x.S(p.dn);
  char* dmid = (char*)x.S(p.dmid);
  DwList dws;

  // The weight gradients of layer l run on the second stream while the walk
  // goes on through layer l-1; before the walk writes a buffer set again it
  // waits for the last launch that reads it.
  std::lock_guard<std::mutex> lock(g_dw_mu);
  DwStream* aux = dw_stream();
  Ctx xw = x;
  if (aux) xw.s = aux->s;
  // Whatever path leaves this function, the caller's stream ends after all
  // of the second stream's work (on an error return too, so that the
  // caller's next call cannot overwrite buffers that work still reads).
  struct Join {
    DwStream* aux;
    hipStream_t s;
    ~Join() {
      if (aux && hipEventRecord(aux->fin, aux->s) == hipSuccess) (void)hipStreamWaitEvent(s, aux->fin, 0);
    }
  } join{aux, x.s};
  bool pending[3] = {false, false, false};
  auto wait_set = [&](int k) -> slt_status {
    if (!aux || !pending[k]) return SLT_OK;
    pending[k] = false;
    return hip_ok(hipStreamWaitEvent(x.s, aux->done[k], 0), "backward: stream wait");
  };
  // partials of norm k (0: final norm, 2 l + 1: the layer's second, 2 l + 2:
  // its first) and their column sums, on the second stream when there is one
  auto nws = [&](int k) { return static_cast<char*>(x.S(p.normws)) + k * p.normws_each; };
  // AdamW over parameters [off, end) on stream s (ranges start on 4-element
  // boundaries, or one update of the whole buffer runs at the end)
  bool ranges_ok = opt != nullptr && p.lp[0].norm1 % 4 == 0 && p.normf % 4 == 0;
  for (int l = 0; l < c.L && ranges_ok; ++l) ranges_ok = p.lp[l].norm1 % 4 == 0;
  auto adam = [&](int64_t off, int64_t end, hipStream_t s) -> slt_status {
    if (!opt || !ranges_ok || end <= off) return SLT_OK;
    return launch_adamw(end - off, opt->master + off, opt->shadow ? opt->shadow + off : nullptr, grads + off,
                        opt->m + off, opt->v + off, opt->t, opt->lr, opt->b1, opt->b2, opt->eps, opt->wd,
                        opt->mask ? opt->mask + off : nullptr, nullptr, s);
  };
  // Second-stream work that only waits for the walk up to some point (a
  // norm's column sums of its partials, a layer's AdamW update once all its
  // gradients are final) is queued here and enqueued, in order, behind the
  // next weight-gradient launch, so that one event per layer hands the
  // second stream everything the walk has finished (each record costs the
  // walk's stream an idle gap of a few microseconds).
  struct SideTask {
    int k;  // >= 0: column sums of norm k into dg (and db); -1: AdamW over [off, end)
    float *dg, *db;
    int64_t off, end;
  };
  SideTask side_q[8];
  int side_n = 0;
  auto run_side = [&](const SideTask& t) -> slt_status {
    if (t.k >= 0) return launch_norm_colsum(nws(t.k), N, C, t.dg, t.db, xw.s, x.gw);
    return adam(t.off, t.end, xw.s);
  };
  auto side = [&](const SideTask& t) -> slt_status {
    if (!aux) return t.k >= 0 ? SLT_OK : run_side(t);  // one stream: the norm launch summed its partials itself
    if (side_n == 8) return fail(SLT_EINVAL, "backward: second-stream queue full");
    side_q[side_n++] = t;
    return SLT_OK;
  };
  auto drain_side = [&]() -> slt_status {
    for (int i = 0; i < side_n; ++i) SLT_TRY(run_side(side_q[i]));
    side_n = 0;
    return SLT_OK;
  };
  // hand the queue to the second stream now, behind an event of its own
  auto flush_side = [&]() -> slt_status {
    if (!aux || side_n == 0) return SLT_OK;
    SLT_TRY(hip_ok(hipEventRecord(aux->ready, x.s), "backward: event record"));
    SLT_TRY(hip_ok(hipStreamWaitEvent(aux->s, aux->ready, 0), "backward: stream wait"));
    return drain_side();
  };
  auto norm_sums = [&](int k, float* dg, float* db) -> slt_status { return side(SideTask{k, dg, db, 0, 0}); };
  auto side_adam = [&](int64_t off, int64_t end) -> slt_status { return side(SideTask{-1, nullptr, nullptr, off, end}); };
  const bool defer = aux != nullptr;
  auto launch_dw = [&](int k) -> slt_status {
    if (aux) {
      SLT_TRY(hip_ok(hipEventRecord(aux->ready, x.s), "backward: event record"));
      SLT_TRY(hip_ok(hipStreamWaitEvent(aux->s, aux->ready, 0), "backward: stream wait"));
    }
    SLT_TRY(flush_dw(xw, dws));
    if (aux) {
      SLT_TRY(hip_ok(hipEventRecord(aux->done[k], aux->s), "backward: event record"));
      pending[k] = true;
    }
    return drain_side();
  };

  // the token sort of the embedding gradient (tokens only) runs on the second
  // stream while the walk goes on; `sort_done` orders the final sums after it
  bool sort_ahead = false;
  if (aux) {
    SLT_TRY(hip_ok(hipEventRecord(aux->ready, x.s), "backward: event record"));
    SLT_TRY(hip_ok(hipStreamWaitEvent(aux->s, aux->ready, 0), "backward: stream wait"));
    SLT_TRY(launch_embedding_sort(tok, c.B, c.T, ldt, c.V, x.S(p.embws), aux->s));
    SLT_TRY(hip_ok(hipEventRecord(aux->sort_done, aux->s), "backward: event record"));
    sort_ahead = true;
  }

  // lm_head and final norm (its weight gradient joins the last layer's launch)
  void* dxL = x.S(p.dx[(c.L - 1) % 3]);
  dws.add(N, c.V, C, x.A(p.z), c.V, x.A(p.nf), C, grads + p.head, C);
  SLT_TRY(proj_dx(x, N, c.V, C, x.A(p.z), c.V, x.P(p.head), C, dn, C));
  if (p.llama)
    SLT_TRY(launch_rmsnorm_bwd(x.A(p.xs.back()), x.P(p.normf), (const float*)x.A(p.rf), dn, nullptr, dxL,
                               grads + p.normf, N, C, x.dt, nws(0), x.s, x.gw, defer));
  else
    SLT_TRY(launch_layernorm_bwd(x.A(p.xs.back()), x.P(p.normf), (const float*)x.A(p.muf),
                                 (const float*)x.A(p.rf), dn, nullptr, dxL, grads + p.normf, grads + p.normfb, N, C,
                                 x.dt, nws(0), x.s, x.gw, defer));
  SLT_TRY(norm_sums(0, grads + p.normf, p.llama ? nullptr : grads + p.normfb));

  for (int l = c.L - 1; l >= 0; --l) {
    const LayerP& W = p.lp[l];
    const LayerA& A = p.la[l];
    const int sl = l % 3, si = (l + 2) % 3;  // this layer's set; the set of the gradient at its input
    SLT_TRY(wait_set(sl));
    void* dx = x.S(p.dx[sl]);          // gradient at the layer's output
    void* dxi = x.S(p.dx[si]);         // gradient at its input (the next layer down's output)
    void* dx2 = x.S(p.dx2[sl]);
    char* dbig = (char*)x.S(p.dbig[sl]);
    AttnArgs at{};
    at.B = c.B; at.T = c.T; at.H = c.H; at.Hkv = c.Hkv; at.d = p.d; at.R = c.R; at.rope_mode = c.rope_mode;
    at.dtype = x.dt; at.cs = cs;
    at.lse_in = (const float*)x.A(A.lse);
    at.delta = (float*)x.S(p.delta);
    at.ores_in = A.ores >= 0 ? x.A(A.ores) : nullptr;
    at.qk_rotated = rope_in_projection(p);
    at.drop = make_drop(c, 3, l);
    char* qkv = (char*)x.A(A.qkv);
    if (p.llama) {
      // dx: gradient at x_out, read by the layer's weight gradients;
      // dx2: gradient at x_mid; dbig: [da | db]; dqkv: [dq | dk | dv].
      char* dqkv = (char*)x.S(p.dqkv[sl]);
      // x_out = x_mid + drop(h W2^T): the product's gradient is dx times the mask
      const void* dy2 = dx;
      if (p.dy2[sl] >= 0) {
        SLT_TRY(launch_drop_apply(dx, x.S(p.dy2[sl]), N, C, x.dt, make_drop(c, 2, l), x.s));
        dy2 = x.S(p.dy2[sl]);
      }
      dws.add(N, C, c.F, dy2, C, x.A(A.h), c.F, grads + W.w2, c.F);
      SLT_TRY(mlp_in_bwd(N, c.F, C, dy2, x.P(W.w2), (const char*)x.A(A.ab), dbig, dmid, x.dt, x.s));
      dws.add(N, 2 * c.F, C, dbig, 2 * c.F, x.A(A.n2), C, grads + W.w1, C);
      SLT_TRY(proj_dx(x, N, 2 * c.F, C, dbig, 2 * c.F, x.P(W.w1), C, dn, C));
      SLT_TRY(launch_rmsnorm_bwd(x.A(p.xs[2 * l + 1]), x.P(W.norm2), (const float*)x.A(A.r2), dn, dx, dx2,
                                 grads + W.norm2, N, C, x.dt, nws(2 * l + 1), x.s, x.gw, defer));
      SLT_TRY(norm_sums(2 * l + 1, grads + W.norm2, nullptr));
      // x_mid = x_in + drop(o W_o^T)
      const void* dy1 = dx2;
      if (p.dy1[sl] >= 0) {
        SLT_TRY(launch_drop_apply(dx2, x.S(p.dy1[sl]), N, C, x.dt, make_drop(c, 1, l), x.s));
        dy1 = x.S(p.dy1[sl]);
      }
      dws.add(N, C, p.qd, dy1, C, x.A(A.o), p.qd, grads + W.wo, p.qd);
      SLT_TRY(proj_dx(x, N, C, p.qd, dy1, C, x.P(W.wo), p.qd, dmid, p.qd));
      at.q = qkv; at.k = qkv + p.qd * p.es; at.v = qkv + (p.qd + p.kd) * p.es;
      at.ldq = at.ldk = at.ldv = p.qkv_w;
      at.o = x.A(A.o); at.ldo = p.qd;
      at.dout = dmid; at.lddo = p.qd;
      at.dq = dqkv; at.dk = dqkv + p.qd * p.es; at.dv = dqkv + (p.qd + p.kd) * p.es;
      at.lddq = at.lddk = at.lddv = p.qkv_w;
      {
        Timed tm(TM_ABWD, x.s);
        SLT_TRY(launch_attention_bwd(at, x.s));
      }
      dws.add(N, p.qkv_w, C, dqkv, p.qkv_w, x.A(A.n1), C, grads + W.qkvw, C);
      SLT_TRY(launch_dw(sl));
      if (l == c.L - 1) SLT_TRY(side_adam(p.normf, p.n_params));  // final norm and lm_head are final
      SLT_TRY(proj_dx(x, N, p.qkv_w, C, dqkv, p.qkv_w, x.P(W.qkvw), C, dn, C));
      SLT_TRY(wait_set(si));
      SLT_TRY(launch_rmsnorm_bwd(x.A(p.xs[2 * l]), x.P(W.norm1), (const float*)x.A(A.r1), dn, dx2, dxi,
                                 grads + W.norm1, N, C, x.dt, nws(2 * l + 2), x.s, x.gw, defer));
      SLT_TRY(norm_sums(2 * l + 2, grads + W.norm1, nullptr));
      SLT_TRY(side_adam(W.norm1, l + 1 < c.L ? p.lp[l + 1].norm1 : p.normf));  // the layer's gradients are final
      // the second stream ends the step with the first layer's weight
      // gradients: give it this layer's queue first, not behind them
      if (l == 1) SLT_TRY(flush_side());
    } else {
      char* ou = (char*)x.A(A.o);
      // x_out = x_in + drop([o | u] W_out^T)
      const void* dy1 = dx;
      if (p.dy1[sl] >= 0) {
        SLT_TRY(launch_drop_apply(dx, x.S(p.dy1[sl]), N, C, x.dt, make_drop(c, 1, l), x.s));
        dy1 = x.S(p.dy1[sl]);
      }
      dws.add(N, C, p.ou_w, dy1, C, ou, p.ou_w, grads + W.wout, p.ou_w);
      SLT_TRY(proj_dx(x, N, C, p.ou_w, dy1, C, x.P(W.wout), p.ou_w, dmid, p.ou_w));
      SLT_TRY(launch_gelu_bwd(qkv + p.qkv_w * p.es, dmid + p.qd * p.es, dbig + p.qkv_w * p.es, N, c.F, p.in_w,
                              p.ou_w, p.in_w, x.dt, x.s));
      at.q = qkv; at.k = qkv + p.qd * p.es; at.v = qkv + (p.qd + p.kd) * p.es;
      at.ldq = at.ldk = at.ldv = p.in_w;
      at.o = ou; at.ldo = p.ou_w;
      at.dout = dmid; at.lddo = p.ou_w;
      at.dq = dbig; at.dk = dbig + p.qd * p.es; at.dv = dbig + (p.qd + p.kd) * p.es;
      at.lddq = at.lddk = at.lddv = p.in_w;
      {
        Timed tm(TM_ABWD, x.s);
        SLT_TRY(launch_attention_bwd(at, x.s));
      }
      dws.add(N, p.in_w, C, dbig, p.in_w, x.A(A.n1), C, grads + W.qkvw, C);
      SLT_TRY(launch_dw(sl));
      if (l == c.L - 1) SLT_TRY(side_adam(p.normf, p.n_params));  // final norm and lm_head are final
      SLT_TRY(proj_dx(x, N, p.in_w, C, dbig, p.in_w, x.P(W.qkvw), C, dn, C));
      SLT_TRY(wait_set(si));
      SLT_TRY(launch_layernorm_bwd(x.A(p.xs[l]), x.P(W.norm1), (const float*)x.A(A.mu1), (const float*)x.A(A.r1),
                                   dn, dx, dxi, grads + W.norm1, grads + W.norm1b, N, C, x.dt, nws(2 * l + 2), x.s,
                                   x.gw, defer));
      SLT_TRY(norm_sums(2 * l + 2, grads + W.norm1, grads + W.norm1b));
      SLT_TRY(side_adam(W.norm1, l + 1 < c.L ? p.lp[l + 1].norm1 : p.normf));  // the layer's gradients are final
      // the second stream ends the step with the first layer's weight
      // gradients: give it this layer's queue first, not behind them
      if (l == 1) SLT_TRY(flush_side());
    }
  }
  SLT_TRY(flush_side());  // the first layer's norm sums and update
  if (sort_ahead) SLT_TRY(hip_ok(hipStreamWaitEvent(x.s, aux->sort_done, 0), "backward: stream wait"));
  SLT_TRY(launch_embedding_bwd(tok, c.B, c.T, ldt, x.S(p.dx[2]), grads + p.wte, c.V, C, x.dt, x.S(p.embws), x.s,
                               x.gw, make_drop(c, 0, 0), sort_ahead));
  SLT_TRY(adam(p.wte, p.lp[0].norm1, x.s));
  // the walk's stream ends after everything on the second stream (in order
  // there, so one event after the last launch covers it all)
  if (aux) {
    join.aux = nullptr;
    SLT_TRY(hip_ok(hipEventRecord(aux->fin, aux->s), "backward: event record"));
    SLT_TRY(hip_ok(hipStreamWaitEvent(x.s, aux->fin, 0), "backward: stream wait"));
  }
  if (opt && !ranges_ok)  // offsets not on 4-element boundaries: one update at the end
    SLT_TRY(launch_adamw(p.n_params, opt->master, opt->shadow, grads, opt->m, opt->v, opt->t, opt->lr, opt->b1,
                         opt->b2, opt->eps, opt->wd, opt->mask, nullptr, x.s));
  return SLT_OK;
}

static bool is_dtype(int32_t d) { return d == SLT_F32 || d == SLT_BF16; }

// ---------------------------------------------------------------------------
// Key/value-cache forward: buffers for B sequences, Tq new rows each, and a
// cache of Tmax positions.  The cache holds per layer K then V
// ([B, Hkv, Tmax, d] each, activation type), then the RoPE table of Tmax
// positions (fp32).
// ---------------------------------------------------------------------------
struct CachePlan {
  int64_t kv, table, bytes;  // one K or V block, table offset, total cache bytes
  int64_t x0, x1, n, r, mu, qkv, qrot, o, ab, h, lse, rot, part, ws_bytes;
};

static CachePlan cache_plan(const Plan& p, int B, int Tq, int Tmax) {
  const slt_config& c = p.c;
  CachePlan q;
  q.kv = a256((int64_t)B * c.Hkv * Tmax * p.d * p.es);
  q.table = 2 * c.L * q.kv;
  q.bytes = q.table + a256((int64_t)Tmax * std::max(c.R, 2) * 4);
  const int64_t M = (int64_t)B * Tq, es = p.es, C = c.C;
  int64_t a = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = a;
    a += a256(bytes);
    return o;
  };
  q.x0 = take(M * C * es);
  q.x1 = take(M * C * es);
  q.n = take(M * C * es);
  q.r = take(M * 4);
  q.mu = take(M * 4);
  q.qkv = take(M * (p.llama ? p.qkv_w : p.in_w) * es);
  q.qrot = take(M * p.qd * 4);
  q.o = take(M * (p.llama ? p.qd : p.ou_w) * es);
  q.ab = p.llama ? take(M * 2 * c.F * es) : -1;
  q.h = p.llama ? take(M * c.F * es) : -1;
  q.lse = take((int64_t)B * c.H * Tq * 4);
  q.rot = flash_eligible(c.act, p.d) ? take(flash_rot_elems(B, Tq, c.H, c.Hkv, p.d) * 2) : -1;  // prefill's rotated q, k
  q.part = take(decode_attention_ws(B, Tq, c.H, c.Hkv, p.d, Tmax));
  q.ws_bytes = a;
  return q;
}

// Tq new tokens per sequence at positions pos0 .. pos0 + Tq - 1.  A prompt
// of 16 or more tokens at pos0 = 0 runs the training forward's attention on
// the projections; every other call attends over the cache.
static slt_status forward_cached(const Plan& p, const Ctx& x, const CachePlan& q, const int32_t* tok, int B, int Tq,
                                 int64_t ldt, int pos0, char* cache, int Tmax, bool last_only, void* logits,
                                 int64_t ldz) {
  const slt_config& c = p.c;
  const int M = B * Tq, C = c.C;
  float* cs = reinterpret_cast<float*>(cache + q.table);
  if (c.R > 0 && pos0 == 0) SLT_TRY(launch_rope_table(Tmax, c.R, c.rope_base, cs, x.s));
  const bool prefill = pos0 == 0 && Tq >= 16;
  void* xa = x.A(q.x0);
  void* xb = x.A(q.x1);
  SLT_TRY(launch_embedding_fwd(tok, B, Tq, ldt, x.P(p.wte), xa, c.V, C, x.dt, x.s));
  for (int l = 0; l < c.L; ++l) {
    const LayerP& W = p.lp[l];
    char* Kc = cache + 2 * l * q.kv;
    char* Vc = Kc + q.kv;
    char* qkv = (char*)x.A(q.qkv);
    char* ou = (char*)x.A(q.o);
    const int64_t ldqkv = p.llama ? p.qkv_w : p.in_w, ldo = p.llama ? p.qd : p.ou_w;
    if (p.llama)
      SLT_TRY(launch_rmsnorm_fwd(xa, x.P(W.norm1), x.A(q.n), (float*)x.A(q.r), M, C, c.eps, x.dt, x.s));
    else
      SLT_TRY(launch_layernorm_fwd(xa, x.P(W.norm1), x.P(W.norm1b), x.A(q.n), (float*)x.A(q.mu), (float*)x.A(q.r),
                                   M, C, c.eps, x.dt, x.s));
    if (p.llama)
      SLT_TRY(proj(x, M, (int)ldqkv, C, x.A(q.n), C, x.P(W.qkvw), qkv, ldqkv, nullptr, 0));
    else  // [q | k | v | a] and u = gelu(a) into [o | u]
      SLT_TRY(proj_gelu(M, (int)ldqkv, C, x.A(q.n), x.P(W.qkvw), qkv, ldqkv, p.qkv_w, ou + p.qd * p.es, ldo, x.dt,
                        x.s));
    SLT_TRY(launch_kv_append(qkv, ldqkv, (float*)x.A(q.qrot), B, Tq, pos0, c.H, c.Hkv, p.d, c.R, c.rope_mode, cs, Kc,
                             Vc, Tmax, x.dt, x.s));
    if (prefill) {
      AttnArgs at{};
      at.B = B; at.T = Tq; at.H = c.H; at.Hkv = c.Hkv; at.d = p.d; at.R = c.R; at.rope_mode = c.rope_mode;
      at.dtype = x.dt; at.cs = cs;
      at.lse = (float*)x.A(q.lse);
      at.qk_rotated = false;
      at.rot = q.rot >= 0 ? x.A(q.rot) : nullptr;
      at.q = qkv; at.k = qkv + p.qd * p.es; at.v = qkv + (p.qd + p.kd) * p.es;
      at.ldq = at.ldk = at.ldv = ldqkv;
      at.out = ou; at.ldo = ldo;
      {
        Timed tm(TM_AFWD, x.s);
        SLT_TRY(launch_attention_fwd(at, x.s));
      }
    } else {
      SLT_TRY(launch_attention_decode((const float*)x.A(q.qrot), Kc, Vc, ou, ldo, B, Tq, pos0, c.H, c.Hkv, p.d, Tmax,
                                      x.dt, (float*)x.A(q.part), x.s));
    }
    if (p.llama) {
      SLT_TRY(proj(x, M, C, p.qd, ou, p.qd, x.P(W.wo), xb, C, xa, C));
      SLT_TRY(launch_rmsnorm_fwd(xb, x.P(W.norm2), x.A(q.n), (float*)x.A(q.r), M, C, c.eps, x.dt, x.s));
      SLT_TRY(mlp_in(M, c.F, C, x.A(q.n), x.P(W.w1), (char*)x.A(q.ab), x.A(q.h), x.dt, x.s));
      SLT_TRY(proj(x, M, C, c.F, x.A(q.h), c.F, x.P(W.w2), xa, C, xb, C));
    } else {
      SLT_TRY(proj(x, M, C, p.ou_w, ou, p.ou_w, x.P(W.wout), xb, C, xa, C));
      std::swap(xa, xb);
    }
  }
  if (p.llama)
    SLT_TRY(launch_rmsnorm_fwd(xa, x.P(p.normf), x.A(q.n), (float*)x.A(q.r), M, C, c.eps, x.dt, x.s));
  else
    SLT_TRY(launch_layernorm_fwd(xa, x.P(p.normf), x.P(p.normfb), x.A(q.n), (float*)x.A(q.mu), (float*)x.A(q.r), M,
                                 C, c.eps, x.dt, x.s));
  if (last_only)
    return proj(x, B, c.V, C, (char*)x.A(q.n) + (int64_t)(Tq - 1) * C * p.es, (int64_t)Tq * C, x.P(p.head), logits,
                ldz, nullptr, 0);
  return proj(x, M, c.V, C, x.A(q.n), C, x.P(p.head), logits, ldz, nullptr, 0);
}

}  // namespace slt

using namespace slt;

// ---------------------------------------------------------------------------
// Exported entry points
// ---------------------------------------------------------------------------
extern "C" {

slt_status slt_timing(int32_t on) {
  g_tm_on.store(on != 0);
  return SLT_OK;
}

slt_status slt_timing_read(double* ms, int64_t* launches, int32_t nclass) {
  if (!ms || !launches || nclass < 0) return fail(SLT_EINVAL, "timing_read: NULL output or negative class count");
  for (int i = 0; i < nclass; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  std::lock_guard<std::mutex> lk(g_tm_mu);
  hipError_t err = hipSuccess;
  for (const TmRec& r : g_tm_recs) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess && err == hipSuccess) err = e;
    if (e == hipSuccess && r.cls < nclass) {
      ms[r.cls] += t;
      launches[r.cls] += 1;
    }
    g_tm_pool.push_back(r.a);
    g_tm_pool.push_back(r.b);
  }
  g_tm_recs.clear();
  if (err != hipSuccess) return fail(SLT_EHIP, std::string("timing_read: ") + hipGetErrorString(err));
  return SLT_OK;
}

const char* slt_last_error(void) { return g_err.c_str(); }

const char* slt_version(void) { return "slt 0.1 (gfx950)"; }

slt_status slt_validate(const slt_config* cfg) { return validate(cfg); }

slt_status slt_param_layout(const slt_config* cfg, slt_tensor* out, int32_t cap, int32_t* n_tensors,
                            int64_t* n_params) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!n_tensors || !n_params) return fail(SLT_EINVAL, "n_tensors and n_params must not be NULL");
  *n_tensors = (int32_t)p.tensors.size();
  *n_params = p.n_params;
  if (out) {
    if (cap < 0) return fail(SLT_EINVAL, "cap must be >= 0");
    for (int i = 0; i < (int)p.tensors.size() && i < cap; ++i) out[i] = p.tensors[i];
  }
  return SLT_OK;
}

slt_status slt_workspace_bytes(const slt_config* cfg, int64_t* act_bytes, int64_t* scratch_bytes) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!act_bytes || !scratch_bytes) return fail(SLT_EINVAL, "output pointers must not be NULL");
  *act_bytes = p.act_bytes;
  *scratch_bytes = p.scratch_bytes;
  return SLT_OK;
}

slt_status slt_model_init(const slt_config* cfg, uint64_t seed, float std, float out_scale, float* master,
                          void* stream) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!master) return fail(SLT_EINVAL, "master is NULL");
  hipStream_t s = as_stream(stream);
  for (const slt_tensor& t : p.tensors) {
    const std::string name(t.name);
    auto ends = [&](const char* suf) {
      const size_t n = strlen(suf);
      return name.size() >= n && name.compare(name.size() - n, n, suf) == 0;
    };
    int kind = 0;
    float v = std;
    if (ends("norm") || ends("norm_f") || ends("ln_g") || ends("lnf_g")) {
      kind = 1; v = 1.0f;
    } else if (ends("ln_b") || ends("lnf_b")) {
      kind = 1; v = 0.0f;
    } else if (ends("w_o") || ends("w2") || ends("w_out")) {
      v = std * out_scale;
    }
    SLT_TRY(launch_model_init_range(master + t.offset, t.numel, t.offset, seed, v, kind, s));
  }
  return SLT_OK;
}

slt_status slt_cast_bf16(const float* src, uint16_t* dst, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!src || !dst))) return fail(SLT_EINVAL, "cast: bad arguments");
  if (n == 0) return SLT_OK;
  return launch_cast_bf16(src, dst, n, as_stream(stream));
}

slt_status slt_forward_loss(const slt_config* cfg, const void* params, const int32_t* tokens, void* acts,
                            void* scratch, float* loss, void* stream) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!params || !tokens || !acts || !scratch || !loss) return fail(SLT_EINVAL, "forward_loss: NULL pointer");
  Ctx x{p, as_stream(stream), (char*)acts, (char*)scratch, (const char*)params, cfg->act};
  return forward(p, x, tokens, loss);
}

slt_status slt_backward(const slt_config* cfg, const void* params, const int32_t* tokens, void* acts, void* scratch,
                        float* grads, void* stream) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!params || !tokens || !acts || !scratch || !grads) return fail(SLT_EINVAL, "backward: NULL pointer");
  Ctx x{p, as_stream(stream), (char*)acts, (char*)scratch, (const char*)params, cfg->act};
  return backward(p, x, tokens, grads);
}

slt_status slt_backward_adamw(const slt_config* cfg, const void* params, const int32_t* tokens, void* acts,
                              void* scratch, float* grads, float* master, uint16_t* shadow, float* m, float* v,
                              int64_t t, float lr, float beta1, float beta2, float eps, float wd,
                              const uint8_t* decay_mask, void* stream) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!params || !tokens || !acts || !scratch || !grads || !master || !m || !v)
    return fail(SLT_EINVAL, "backward_adamw: NULL pointer");
  if (cfg->act == SLT_BF16 && !shadow) return fail(SLT_EINVAL, "backward_adamw: bf16 configurations need the shadow");
  if (t < 1) return fail(SLT_EINVAL, "backward_adamw: t must be >= 1");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f))
    return fail(SLT_EINVAL, "backward_adamw: betas must lie in [0, 1) and eps >= 0");
  auto al16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  if (!al16(master) || !al16(grads) || !al16(m) || !al16(v) || (shadow && reinterpret_cast<uintptr_t>(shadow) % 8) ||
      (decay_mask && reinterpret_cast<uintptr_t>(decay_mask) % 4))
    return fail(SLT_EINVAL, "backward_adamw: buffers must be 16-byte aligned (shadow 8, mask 4)");
  Ctx x{p, as_stream(stream), (char*)acts, (char*)scratch, (const char*)params, cfg->act};
  const AdamArgs opt{master, shadow, m, v, t, lr, beta1, beta2, eps, wd, decay_mask};
  return backward(p, x, tokens, grads, &opt);
}

slt_status slt_backward_accumulate(const slt_config* cfg, const void* params, const int32_t* tokens, void* acts,
                                   void* scratch, float* grads, float scale, const float* loss, float* loss_sum,
                                   void* stream) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (!params || !tokens || !acts || !scratch || !grads) return fail(SLT_EINVAL, "backward_accumulate: NULL pointer");
  if (!(scale == scale)) return fail(SLT_EINVAL, "backward_accumulate: scale is NaN");
  if ((loss == nullptr) != (loss_sum == nullptr))
    return fail(SLT_EINVAL, "backward_accumulate: loss and loss_sum are both given or both NULL");
  Ctx x{p, as_stream(stream), (char*)acts, (char*)scratch, (const char*)params, cfg->act};
  x.gw.alpha = scale;
  x.gw.accumulate = true;
  if (loss) SLT_TRY(launch_scalar_axpy(loss_sum, scale, loss, x.s));
  return backward(p, x, tokens, grads);
}

slt_status slt_adamw_step(int64_t n, float* master, uint16_t* shadow, const float* grads, float* m, float* v,
                          int64_t t, float lr, float beta1, float beta2, float eps, float wd,
                          const uint8_t* decay_mask, const float* grad_scale, void* stream) {
  if (n < 0) return fail(SLT_EINVAL, "adamw: n < 0");
  if (n == 0) return SLT_OK;
  if (!master || !grads || !m || !v) return fail(SLT_EINVAL, "adamw: NULL pointer");
  if (t < 1) return fail(SLT_EINVAL, "adamw: t must be >= 1");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f))
    return fail(SLT_EINVAL, "adamw: betas must lie in [0, 1) and eps >= 0");
  auto al16 = [](const void* q) { return q == nullptr || reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  if (!al16(master) || !al16(grads) || !al16(m) || !al16(v) || (shadow && reinterpret_cast<uintptr_t>(shadow) % 8) ||
      (decay_mask && reinterpret_cast<uintptr_t>(decay_mask) % 4))
    return fail(SLT_EINVAL, "adamw: buffers must be 16-byte aligned (shadow 8, mask 4)");
  if (grad_scale && reinterpret_cast<uintptr_t>(grad_scale) % 4) return fail(SLT_EINVAL, "adamw: misaligned grad_scale");
  return launch_adamw(n, master, shadow, grads, m, v, t, lr, beta1, beta2, eps, wd, decay_mask, grad_scale,
                      as_stream(stream));
}

int64_t slt_clip_workspace_bytes(void) { return grad_norm_ws(); }

slt_status slt_clip_grad_norm(int64_t n, const float* grads, int32_t kind, float max_norm, float* norm, float* scale,
                              void* workspace, void* stream) {
  if (n < 0) return fail(SLT_EINVAL, "clip_grad_norm: n < 0");
  if (kind != SLT_NORM_L2 && kind != SLT_NORM_LINF) return fail(SLT_EINVAL, "clip_grad_norm: bad kind");
  if (!(max_norm > 0.f)) return fail(SLT_EINVAL, "clip_grad_norm: max_norm must be > 0");
  if ((n > 0 && !grads) || !workspace) return fail(SLT_EINVAL, "clip_grad_norm: NULL pointer");
  if (reinterpret_cast<uintptr_t>(grads) % 16 || reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(SLT_EINVAL, "clip_grad_norm: grads and workspace must be 16-byte aligned");
  return launch_grad_norm(n, grads, kind, max_norm, norm, scale, workspace, as_stream(stream));
}

slt_status slt_gemm(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_kmajor, const void* B,
                    int64_t ldb, int32_t b_kmajor, void* C, int64_t ldc, const void* R, int64_t ldr,
                    int32_t in_dtype, int32_t out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(SLT_EINVAL, "gemm: negative size");
  if (!is_dtype(in_dtype) || !is_dtype(out_dtype)) return fail(SLT_EINVAL, "gemm: bad dtype");
  if (M == 0 || N == 0) return SLT_OK;
  if (!C || (K > 0 && (!A || !B))) return fail(SLT_EINVAL, "gemm: NULL operand");
  if (ldc < N || (R && ldr < N)) return fail(SLT_EINVAL, "gemm: ldc/ldr smaller than N");
  if (K > 0) {
    if (a_kmajor ? lda < K : lda < M) return fail(SLT_EINVAL, "gemm: lda too small");
    if (b_kmajor ? ldb < K : ldb < N) return fail(SLT_EINVAL, "gemm: ldb too small");
  }
  if (workspace_bytes < 0 || (workspace && reinterpret_cast<uintptr_t>(workspace) % 16))
    return fail(SLT_EINVAL, "gemm: workspace must be 16-byte aligned");
  GemmArgs g{M, N, K, A, lda, a_kmajor != 0, B, ldb, b_kmajor != 0, C, ldc, R, ldr, in_dtype, out_dtype,
             static_cast<float*>(workspace), workspace ? workspace_bytes : 0};
  return launch_gemm(g, as_stream(stream));
}

slt_status slt_embedding_fwd(const int32_t* tokens, int32_t B, int32_t T, int64_t ld_tokens, const void* wte,
                             void* x, int32_t V, int32_t C, int32_t dtype, void* stream) {
  if (B < 0 || T < 0 || V <= 0 || C <= 0 || ld_tokens < T || !is_dtype(dtype))
    return fail(SLT_EINVAL, "embedding_fwd: bad sizes");
  if ((int64_t)B * T == 0) return SLT_OK;
  if (!tokens || !wte || !x) return fail(SLT_EINVAL, "embedding_fwd: NULL pointer");
  return launch_embedding_fwd(tokens, B, T, ld_tokens, wte, x, V, C, dtype, as_stream(stream));
}

int64_t slt_embedding_bwd_workspace(int64_t N, int32_t V) { return embedding_bwd_ws(N, V); }

slt_status slt_embedding_bwd(const int32_t* tokens, int32_t B, int32_t T, int64_t ld_tokens, const void* dx,
                             float* dwte, int32_t V, int32_t C, int32_t dtype, void* workspace, void* stream) {
  if (B < 0 || T < 0 || V <= 0 || C <= 0 || C > 4096 || ld_tokens < T || !is_dtype(dtype))
    return fail(SLT_EINVAL, "embedding_bwd: bad sizes");
  if (!dwte || !workspace || ((int64_t)B * T > 0 && (!tokens || !dx)))
    return fail(SLT_EINVAL, "embedding_bwd: NULL pointer");
  if ((int64_t)B * T == 0) return launch_fill_f32(dwte, 0.f, (int64_t)V * C, as_stream(stream));
  return launch_embedding_bwd(tokens, B, T, ld_tokens, dx, dwte, V, C, dtype, workspace, as_stream(stream));
}

slt_status slt_rmsnorm_fwd(const void* x, const void* g, void* y, float* rstd, int32_t rows, int32_t C, float eps,
                           int32_t dtype, void* stream) {
  if (rows < 0 || C <= 0 || !is_dtype(dtype)) return fail(SLT_EINVAL, "rmsnorm_fwd: bad sizes");
  if (rows == 0) return SLT_OK;
  if (!x || !g || !y || !rstd) return fail(SLT_EINVAL, "rmsnorm_fwd: NULL pointer");
  return launch_rmsnorm_fwd(x, g, y, rstd, rows, C, eps, dtype, as_stream(stream));
}

int64_t slt_norm_bwd_workspace(int32_t rows, int32_t C) { return norm_bwd_ws(rows, C); }

slt_status slt_rmsnorm_bwd(const void* x, const void* g, const float* rstd, const void* dy, const void* dres,
                           void* dx, float* dg, int32_t rows, int32_t C, int32_t dtype, void* workspace,
                           void* stream) {
  if (rows < 0 || C <= 0 || !is_dtype(dtype)) return fail(SLT_EINVAL, "rmsnorm_bwd: bad sizes");
  if (!dg || !workspace) return fail(SLT_EINVAL, "rmsnorm_bwd: NULL pointer");
  if (rows == 0) return launch_fill_f32(dg, 0.f, C, as_stream(stream));
  if (!x || !g || !rstd || !dy || !dx) return fail(SLT_EINVAL, "rmsnorm_bwd: NULL pointer");
  return launch_rmsnorm_bwd(x, g, rstd, dy, dres, dx, dg, rows, C, dtype, workspace, as_stream(stream));
}

slt_status slt_layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                             int32_t rows, int32_t C, float eps, int32_t dtype, void* stream) {
  if (rows < 0 || C <= 0 || !is_dtype(dtype)) return fail(SLT_EINVAL, "layernorm_fwd: bad sizes");
  if (rows == 0) return SLT_OK;
  if (!x || !gamma || !beta || !y || !mean || !rstd) return fail(SLT_EINVAL, "layernorm_fwd: NULL pointer");
  return launch_layernorm_fwd(x, gamma, beta, y, mean, rstd, rows, C, eps, dtype, as_stream(stream));
}

slt_status slt_layernorm_bwd(const void* x, const void* gamma, const float* mean, const float* rstd,
                             const void* dy, const void* dres, void* dx, float* dgamma, float* dbeta, int32_t rows,
                             int32_t C, int32_t dtype, void* workspace, void* stream) {
  if (rows < 0 || C <= 0 || !is_dtype(dtype)) return fail(SLT_EINVAL, "layernorm_bwd: bad sizes");
  if (!dgamma || !dbeta || !workspace) return fail(SLT_EINVAL, "layernorm_bwd: NULL pointer");
  if (rows == 0) {
    SLT_TRY(launch_fill_f32(dgamma, 0.f, C, as_stream(stream)));
    return launch_fill_f32(dbeta, 0.f, C, as_stream(stream));
  }
  if (!x || !gamma || !mean || !rstd || !dy || !dx) return fail(SLT_EINVAL, "layernorm_bwd: NULL pointer");
  return launch_layernorm_bwd(x, gamma, mean, rstd, dy, dres, dx, dgamma, dbeta, rows, C, dtype, workspace,
                              as_stream(stream));
}

slt_status slt_rope_table(int32_t T, int32_t R, float base, float* cs, void* stream) {
  if (T < 0 || R < 0 || (R & 1) || !(base > 0.f)) return fail(SLT_EINVAL, "rope_table: bad arguments");
  if (T == 0 || R == 0) return SLT_OK;
  if (!cs) return fail(SLT_EINVAL, "rope_table: NULL pointer");
  return launch_rope_table(T, R, base, cs, as_stream(stream));
}

static slt_status rope_call(const char* what, const void* x, int64_t ldx, void* y, int64_t ldy, int32_t B, int32_t T,
                            int32_t nheads, int32_t d, int32_t R, int32_t mode, const float* cs, int32_t dtype,
                            float sign, void* stream) {
  if (B < 0 || T < 0 || nheads < 0 || d <= 0 || R < 0 || R > d || (R & 1) || !is_dtype(dtype))
    return fail(SLT_EINVAL, std::string(what) + ": bad sizes (R must be even and <= d)");
  if (mode != SLT_ROPE_HALF && mode != SLT_ROPE_PAIRS) return fail(SLT_EINVAL, std::string(what) + ": bad rope_mode");
  if ((int64_t)B * T * nheads == 0) return SLT_OK;
  if (ldx < (int64_t)nheads * d || ldy < (int64_t)nheads * d)
    return fail(SLT_EINVAL, std::string(what) + ": row stride smaller than the heads it holds");
  if (!x || !y || (R > 0 && !cs)) return fail(SLT_EINVAL, std::string(what) + ": NULL pointer");
  if (x == y && ldx != ldy) return fail(SLT_EINVAL, std::string(what) + ": in place needs equal row strides");
  if (R == 0 && x == y) return SLT_OK;
  return launch_rope(x, ldx, y, ldy, (int64_t)B * T, T, nheads, d, R, mode, cs, sign, dtype, as_stream(stream));
}

slt_status slt_rope_fwd(const void* x, int64_t ldx, void* y, int64_t ldy, int32_t B, int32_t T, int32_t nheads,
                        int32_t d, int32_t R, int32_t rope_mode, const float* cs, int32_t dtype, void* stream) {
  return rope_call("rope_fwd", x, ldx, y, ldy, B, T, nheads, d, R, rope_mode, cs, dtype, 1.0f, stream);
}

slt_status slt_rope_bwd(const void* dy, int64_t lddy, void* dx, int64_t lddx, int32_t B, int32_t T, int32_t nheads,
                        int32_t d, int32_t R, int32_t rope_mode, const float* cs, int32_t dtype, void* stream) {
  return rope_call("rope_bwd", dy, lddy, dx, lddx, B, T, nheads, d, R, rope_mode, cs, dtype, -1.0f, stream);
}

static slt_status attn_check(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t R, int32_t mode,
                             int32_t dtype, const float* cs) {
  if (B < 0 || T < 0 || H <= 0 || Hkv <= 0 || d <= 0 || H % Hkv || !is_dtype(dtype))
    return fail(SLT_EINVAL, "attention: bad sizes");
  if (d > 64) return fail(SLT_EUNSUPPORTED, "attention: head dim above 64");
  if (R < 0 || R > d || (R & 1)) return fail(SLT_EINVAL, "attention: R must be even and <= d");
  if (mode != SLT_ROPE_HALF && mode != SLT_ROPE_PAIRS) return fail(SLT_EINVAL, "attention: bad rope_mode");
  if (R > 0 && !cs) return fail(SLT_EINVAL, "attention: RoPE table is NULL");
  return SLT_OK;
}

static int64_t attn_rot_bytes(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || Hkv <= 0 || !flash_eligible(dtype, d)) return 0;
  return a256(flash_rot_elems(B, T, H, Hkv, d) * 2);
}

int64_t slt_attention_fwd_workspace(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t dtype) {
  return attn_rot_bytes(B, T, H, Hkv, d, dtype);
}

slt_status slt_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* o_res, int64_t ldq,
                             int64_t ldk, int64_t ldv, int64_t ldo, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                             int32_t d, int32_t R, int32_t rope_mode, const float* cs, int32_t dtype,
                             void* workspace, void* stream) {
  SLT_TRY(attn_check(B, T, H, Hkv, d, R, rope_mode, dtype, cs));
  if ((int64_t)B * T == 0) return SLT_OK;
  if (!q || !k || !v || !o || !lse) return fail(SLT_EINVAL, "attention_fwd: NULL pointer");
  if (ldq < (int64_t)H * d || ldk < (int64_t)Hkv * d || ldv < (int64_t)Hkv * d || ldo < (int64_t)H * d)
    return fail(SLT_EINVAL, "attention_fwd: row stride smaller than the heads it holds");
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = o; a.lse = lse; a.ores_out = o_res;
  a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo;
  a.B = B; a.T = T; a.H = H; a.Hkv = Hkv; a.d = d; a.R = R; a.rope_mode = rope_mode; a.dtype = dtype; a.cs = cs;
  if (attn_rot_bytes(B, T, H, Hkv, d, dtype) > 0 && !workspace)
    return fail(SLT_EINVAL, "attention_fwd: workspace is NULL (slt_attention_fwd_workspace is non-zero)");
  a.qk_rotated = false;
  a.rot = workspace;
  return launch_attention_fwd(a, as_stream(stream));
}

int64_t slt_attention_bwd_workspace(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t dtype) {
  if (B <= 0 || T <= 0 || H <= 0) return 0;
  return a256(attention_bwd_ws(B, H, T)) + attn_rot_bytes(B, T, H, Hkv, d, dtype);
}

slt_status slt_attention_bwd(const void* q, const void* k, const void* v, const void* o, const void* o_res,
                             const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, int64_t ldq, int64_t ldk, int64_t ldv,
                             int64_t ldo, int64_t lddo, int64_t lddq, int64_t lddk, int64_t lddv, int32_t B,
                             int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t R, int32_t rope_mode,
                             const float* cs, int32_t dtype, void* workspace, void* stream) {
  SLT_TRY(attn_check(B, T, H, Hkv, d, R, rope_mode, dtype, cs));
  if ((int64_t)B * T == 0) return SLT_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return fail(SLT_EINVAL, "attention_bwd: NULL pointer");
  const int64_t hd = (int64_t)H * d, kvd = (int64_t)Hkv * d;
  if (ldq < hd || ldo < hd || lddo < hd || lddq < hd || ldk < kvd || ldv < kvd || lddk < kvd || lddv < kvd)
    return fail(SLT_EINVAL, "attention_bwd: row stride smaller than the heads it holds");
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.ores_in = o_res; a.dout = dout; a.lse_in = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo; a.lddo = lddo; a.lddq = lddq; a.lddk = lddk; a.lddv = lddv;
  a.B = B; a.T = T; a.H = H; a.Hkv = Hkv; a.d = d; a.R = R; a.rope_mode = rope_mode; a.dtype = dtype; a.cs = cs;
  a.delta = static_cast<float*>(workspace);
  a.rot = attn_rot_bytes(B, T, H, Hkv, d, dtype) > 0 ? static_cast<char*>(workspace) + a256(attention_bwd_ws(B, H, T))
                                                      : nullptr;
  a.qk_rotated = false;
  return launch_attention_bwd(a, as_stream(stream));
}

slt_status slt_swiglu_fwd(const void* a, const void* b, void* h, int32_t rows, int32_t F, int64_t lda, int64_t ldb,
                          int64_t ldh, int32_t dtype, void* stream) {
  if (rows < 0 || F < 0 || lda < F || ldb < F || ldh < F || !is_dtype(dtype))
    return fail(SLT_EINVAL, "swiglu_fwd: bad sizes");
  if ((int64_t)rows * F == 0) return SLT_OK;
  if (!a || !b || !h) return fail(SLT_EINVAL, "swiglu_fwd: NULL pointer");
  return launch_swiglu_fwd(a, b, h, rows, F, lda, ldb, ldh, dtype, as_stream(stream));
}

slt_status slt_swiglu_bwd(const void* a, const void* b, const void* dh, void* da, void* db, int32_t rows, int32_t F,
                          int64_t lda, int64_t ldb, int64_t lddh, int64_t ldda, int64_t lddb, int32_t dtype,
                          void* stream) {
  if (rows < 0 || F < 0 || lda < F || ldb < F || lddh < F || ldda < F || lddb < F || !is_dtype(dtype))
    return fail(SLT_EINVAL, "swiglu_bwd: bad sizes");
  if ((int64_t)rows * F == 0) return SLT_OK;
  if (!a || !b || !dh || !da || !db) return fail(SLT_EINVAL, "swiglu_bwd: NULL pointer");
  return launch_swiglu_bwd(a, b, dh, da, db, rows, F, lda, ldb, lddh, ldda, lddb, dtype, as_stream(stream));
}

slt_status slt_gelu_fwd(const void* a, void* u, int32_t rows, int32_t F, int64_t lda, int64_t ldu, int32_t dtype,
                        void* stream) {
  if (rows < 0 || F < 0 || lda < F || ldu < F || !is_dtype(dtype)) return fail(SLT_EINVAL, "gelu_fwd: bad sizes");
  if ((int64_t)rows * F == 0) return SLT_OK;
  if (!a || !u) return fail(SLT_EINVAL, "gelu_fwd: NULL pointer");
  return launch_gelu_fwd(a, u, rows, F, lda, ldu, dtype, as_stream(stream));
}

slt_status slt_gelu_bwd(const void* a, const void* du, void* da, int32_t rows, int32_t F, int64_t lda, int64_t lddu,
                        int64_t ldda, int32_t dtype, void* stream) {
  if (rows < 0 || F < 0 || lda < F || lddu < F || ldda < F || !is_dtype(dtype))
    return fail(SLT_EINVAL, "gelu_bwd: bad sizes");
  if ((int64_t)rows * F == 0) return SLT_OK;
  if (!a || !du || !da) return fail(SLT_EINVAL, "gelu_bwd: NULL pointer");
  return launch_gelu_bwd(a, du, da, rows, F, lda, lddu, ldda, dtype, as_stream(stream));
}

slt_status slt_softmax_xent(void* z, int64_t ldz, const int32_t* tokens, int32_t B, int32_t T, int64_t ld_tokens,
                            int32_t V, float* loss, float* lse, int32_t dtype, void* workspace, void* stream) {
  if (B <= 0 || T <= 0 || V <= 0 || ldz < V || ld_tokens < T + 1 || !is_dtype(dtype))
    return fail(SLT_EINVAL, "softmax_xent: bad sizes");
  if (!z || !tokens || !loss || !workspace) return fail(SLT_EINVAL, "softmax_xent: NULL pointer");
  return launch_softmax_xent(z, ldz, tokens, B, T, ld_tokens, V, loss, lse, dtype, workspace, as_stream(stream));
}

slt_status slt_mlp_swiglu_fwd(int32_t M, int32_t F, int32_t C, const void* x, const void* w13, void* ab, void* h,
                              int32_t dtype, void* stream) {
  if (M < 0 || F <= 0 || C <= 0) return fail(SLT_EINVAL, "mlp_swiglu_fwd: bad sizes");
  if (!is_dtype(dtype)) return fail(SLT_EINVAL, "mlp_swiglu_fwd: bad dtype");
  if (M == 0) return SLT_OK;
  if (!x || !w13 || !ab || !h) return fail(SLT_EINVAL, "mlp_swiglu_fwd: NULL pointer");
  return mlp_in(M, F, C, x, w13, static_cast<char*>(ab), h, dtype, as_stream(stream));
}

slt_status slt_proj_gelu_fwd(int32_t M, int32_t N, int32_t K, const void* x, const void* w, void* y, int64_t ldy,
                             int32_t col0, void* u, int64_t ldu, int32_t dtype, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || col0 < 0 || col0 >= N || ldy < N || ldu < N - col0)
    return fail(SLT_EINVAL, "proj_gelu_fwd: bad sizes");
  if (!is_dtype(dtype)) return fail(SLT_EINVAL, "proj_gelu_fwd: bad dtype");
  if (M == 0) return SLT_OK;
  if (!x || !w || !y || !u) return fail(SLT_EINVAL, "proj_gelu_fwd: NULL pointer");
  return proj_gelu(M, N, K, x, w, static_cast<char*>(y), ldy, col0, static_cast<char*>(u), ldu, dtype,
                   as_stream(stream));
}

slt_status slt_qkv_rope_fwd(int32_t M, int32_t N, int32_t K, const void* x, const void* w, void* y, int64_t ldy,
                            int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t R, int32_t rope_mode, const float* cs,
                            int32_t dtype, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || T <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || ldy < N)
    return fail(SLT_EINVAL, "qkv_rope_fwd: bad sizes");
  if ((int64_t)(H + Hkv) * d > N) return fail(SLT_EINVAL, "qkv_rope_fwd: (H + Hkv) d exceeds N");
  if (R < 0 || R > d || (R & 1)) return fail(SLT_EINVAL, "qkv_rope_fwd: R must be even and <= d");
  if (rope_mode != SLT_ROPE_HALF && rope_mode != SLT_ROPE_PAIRS) return fail(SLT_EINVAL, "qkv_rope_fwd: bad rope_mode");
  if (!is_dtype(dtype)) return fail(SLT_EINVAL, "qkv_rope_fwd: bad dtype");
  if (M == 0) return SLT_OK;
  if (!x || !w || !y || (R > 0 && !cs)) return fail(SLT_EINVAL, "qkv_rope_fwd: NULL pointer");
  return rope_proj(M, N, K, x, w, static_cast<char*>(y), ldy, T, H, Hkv, d, R, rope_mode, cs, dtype,
                   as_stream(stream));
}

slt_status slt_mlp_swiglu_bwd(int32_t M, int32_t F, int32_t C, const void* dy, const void* w2, const void* ab,
                              void* dab, void* dh_workspace, int32_t dtype, void* stream) {
  if (M < 0 || F <= 0 || C <= 0) return fail(SLT_EINVAL, "mlp_swiglu_bwd: bad sizes");
  if (!is_dtype(dtype)) return fail(SLT_EINVAL, "mlp_swiglu_bwd: bad dtype");
  if (M == 0) return SLT_OK;
  if (!dy || !w2 || !ab || !dab || !dh_workspace) return fail(SLT_EINVAL, "mlp_swiglu_bwd: NULL pointer");
  return mlp_in_bwd(M, F, C, dy, w2, static_cast<const char*>(ab), static_cast<char*>(dab), dh_workspace, dtype,
                    as_stream(stream));
}

slt_status slt_gemm_dw_group(const slt_gemm_group_item* items, int32_t n, int32_t K, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  if (!items || n < 1 || n > 6) return fail(SLT_EINVAL, "gemm group: 1 to 6 items required");
  if (K <= 0) return fail(SLT_EINVAL, "gemm group: K must be positive");
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
    return fail(SLT_EINVAL, "gemm group: bad workspace");
  GroupItem g[6];
  for (int i = 0; i < n; ++i) {
    const slt_gemm_group_item& t = items[i];
    if (!t.A || !t.B || !t.C) return fail(SLT_EINVAL, "gemm group: NULL operand");
    g[i] = GroupItem{t.M, t.N, t.A, t.lda, t.B, t.ldb, t.C, t.ldc, t.alpha, t.accumulate != 0};
    if (!gemm_group_ok(g[i], K)) return fail(SLT_EUNSUPPORTED, "gemm group: shape or alignment");
  }
  return launch_gemm_group(g, n, K, static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                           as_stream(stream));
}

slt_status slt_kv_cache_bytes(const slt_config* cfg, int32_t B, int32_t Tq, int32_t Tmax, int64_t* cache_bytes,
                              int64_t* workspace_bytes) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (B <= 0 || Tq <= 0 || Tmax <= 0 || Tq > Tmax) return fail(SLT_EINVAL, "kv cache: need B, Tq > 0 and Tq <= Tmax");
  if (!cache_bytes || !workspace_bytes) return fail(SLT_EINVAL, "kv cache: output pointers must not be NULL");
  const CachePlan q = cache_plan(p, B, Tq, Tmax);
  *cache_bytes = q.bytes;
  *workspace_bytes = q.ws_bytes;
  return SLT_OK;
}

slt_status slt_forward_cached(const slt_config* cfg, const void* params, const int32_t* tokens, int32_t B, int32_t Tq,
                              int64_t ld_tokens, int32_t pos0, void* cache, int32_t Tmax, void* workspace,
                              int32_t last_only, void* logits, int64_t ld_logits, void* stream) {
  Plan p;
  SLT_TRY(make_plan(cfg, p));
  if (B <= 0 || Tq <= 0 || pos0 < 0 || Tmax <= 0 || (int64_t)pos0 + Tq > Tmax)
    return fail(SLT_EINVAL, "forward_cached: need B, Tq > 0, pos0 >= 0 and pos0 + Tq <= Tmax");
  if (ld_tokens < Tq || ld_logits < cfg->V) return fail(SLT_EINVAL, "forward_cached: ld_tokens < Tq or ld_logits < V");
  if ((int64_t)B * Tq > (1 << 30)) return fail(SLT_EUNSUPPORTED, "forward_cached: too many rows");
  if (!params || !tokens || !cache || !workspace || !logits) return fail(SLT_EINVAL, "forward_cached: NULL pointer");
  Ctx x{p, as_stream(stream), (char*)workspace, nullptr, (const char*)params, cfg->act};
  return forward_cached(p, x, cache_plan(p, B, Tq, Tmax), tokens, B, Tq, ld_tokens, pos0, (char*)cache, Tmax,
                        last_only != 0, logits, ld_logits);
}

}  // extern "C"
