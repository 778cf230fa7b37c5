// Causal attention forward and backward with RoPE fused into the q/k loads
// (Hephaistos, "Architecture at a glance": RoPE applied to q and k inside
// attention, causal multi-head attention with a numerically stable softmax;
// strata: flash-style attention with online softmax, forward and backward,
// no T x T score matrix, one op for MHA/GQA/MQA through independent n_head and
// n_kv_head).
//
// MFMA building block: 16x16 output tiles with a k-depth of 16, where lane l
// supplies the operand values at row/column l%16 and depth 4*(l/16)+i,
// i = 0..3, for both operands, and receives output rows 4*(l/16)+r, column
// l%16.  bf16 operands use one v_mfma_f32_16x16x16_bf16; fp32 operands use
// four v_mfma_f32_16x16x4_f32 (depth slot l/16 taken as 4*(l/16)+i at step i).
// Because a lane's four output values lie along the output rows, computing
// S^T = K Q^T leaves each lane with four consecutive keys of one query row:
// exactly the operand layout of the next product (O^T = V^T P^T), so the
// probabilities never leave registers.  The backward uses the same trick for
// every product (choosing which side of each product is transposed).
//
// Tiling: 64 queries (or keys) per workgroup, 16 per wave; key (or query)
// tiles of 64 staged in LDS; head dimension padded to a multiple of 16.
#include "slt_internal.h"

#include <math.h>

namespace slt {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TQ = 64;        // rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int N>
struct alignas(sizeof(T) * N) Pk {
  T e[N];
};

template <typename T> __device__ __forceinline__ T zero_v();
template <> __device__ __forceinline__ bf16 zero_v<bf16>() { return bf16{0}; }
template <> __device__ __forceinline__ float zero_v<float>() { return 0.f; }

__device__ __forceinline__ f32x4 mma16(const Pk<bf16, 4>& a, const Pk<bf16, 4>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a), __builtin_bit_cast(bf16x4_t, b),
                                                    c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Pk<float, 4>& a, const Pk<float, 4>& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[0], b.e[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[1], b.e[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[2], b.e[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[3], b.e[3], c, 0, 0, 0);
  return c;
}

template <typename T>
__device__ __forceinline__ Pk<T, 4> pack4(float a, float b, float c, float d) {
  Pk<T, 4> p;
  p.e[0] = from_f32<T>(a); p.e[1] = from_f32<T>(b); p.e[2] = from_f32<T>(c); p.e[3] = from_f32<T>(d);
  return p;
}

// Second term of a two-term bf16 expansion v ~ hi + lo (zero for fp32).  The
// probability-gradient dS sums to zero along each row, so one bf16 rounding
// per element would leave an error proportional to the mean key or query;
// feeding hi and lo to the MFMA keeps ~16 significant bits.
template <typename T>
__device__ __forceinline__ Pk<T, 4> low_part(const Pk<T, 4>& hi, const float (&v)[4]) {
  return pack4<T>(v[0] - to_f32(hi.e[0]), v[1] - to_f32(hi.e[1]), v[2] - to_f32(hi.e[2]), v[3] - to_f32(hi.e[3]));
}

template <typename T>
__device__ __forceinline__ Pk<T, 4> lds4(const T* p) {
  return *reinterpret_cast<const Pk<T, 4>*>(p);
}

// Value of dim j of a row u at position t after RoPE (sign = +1) or after the
// transposed rotation (sign = -1, the backward of RoPE).  Dims >= R pass
// through.  cs: [T][R] with (cos, sin) of angle t * theta_i at 2i, 2i+1.
template <typename T>
__device__ __forceinline__ float rope_elem(const T* u, int j, int t, int R, int mode, const float* cs, float sign) {
  const float x = to_f32(u[j]);
  if (j >= R) return x;
  int i, p;
  bool first;
  if (mode == SLT_ROPE_HALF) {
    const int h = R >> 1;
    first = j < h;
    i = first ? j : j - h;
    p = first ? j + h : j - h;
  } else {
    first = (j & 1) == 0;
    i = j >> 1;
    p = j ^ 1;
  }
  const float c = cs[(int64_t)t * R + 2 * i];
  const float s = sign * cs[(int64_t)t * R + 2 * i + 1];
  const float y = to_f32(u[p]);
  return first ? x * c - y * s : x * c + y * s;
}

// Same for an fp32 row held in LDS.
__device__ __forceinline__ float rope_elem_f(const float* u, int j, int t, int R, int mode, const float* cs,
                                             float sign) {
  const float x = u[j];
  if (j >= R) return x;
  int i, p;
  bool first;
  if (mode == SLT_ROPE_HALF) {
    const int h = R >> 1;
    first = j < h;
    i = first ? j : j - h;
    p = first ? j + h : j - h;
  } else {
    first = (j & 1) == 0;
    i = j >> 1;
    p = j ^ 1;
  }
  const float c = cs[(int64_t)t * R + 2 * i];
  const float s = sign * cs[(int64_t)t * R + 2 * i + 1];
  const float y = u[p];
  return first ? x * c - y * s : x * c + y * s;
}

// Stage a 64-row tile of a [rows of the sequence] x d operand into LDS, padded
// to DP columns, optionally rotated, into a row-major copy X[r][j] (row stride
// XS) and/or a transposed copy Xt[j][r] (row stride XTS).  Rows >= T and
// columns >= d are zero.
// Xlo / Xtlo (optional, strides XS / XTS) receive the bf16 rounding residual
// of the rotated value, for products that need it beyond bf16.
template <typename T, int DP, bool ROT>
__device__ __forceinline__ void stage_tile(const T* base, int64_t ld, int col0, int row0, int T_, int d, int R,
                                           int mode, const float* cs, T* X, int XS, T* Xt, int XTS,
                                           T* Xlo = nullptr, T* Xtlo = nullptr) {
  for (int idx = threadIdx.x; idx < TQ * DP; idx += blockDim.x) {
    const int r = idx / DP, j = idx % DP;
    const int t = row0 + r;
    T val = zero_v<T>(), lo = zero_v<T>();
    if (t < T_ && j < d) {
      const T* row = base + (int64_t)t * ld + col0;
      if (ROT && R > 0) {
        const float f = rope_elem<T>(row, j, t, R, mode, cs, 1.0f);
        val = from_f32<T>(f);
        lo = from_f32<T>(f - to_f32(val));
      } else {
        val = row[j];
      }
    }
    if (X) X[r * XS + j] = val;
    if (Xt) Xt[j * XTS + r] = val;
    if (Xlo) Xlo[r * XS + j] = lo;
    if (Xtlo) Xtlo[j * XTS + r] = lo;
  }
}

constexpr int kPad = 4;

// ---------------------------------------------------------------------------
// Forward.  grid (ceil(T/64), H, B); wave w owns queries q0 + 16w + l%16.
// ---------------------------------------------------------------------------
template <typename T, int NC>
__global__ __launch_bounds__(256) void attn_fwd_k(AttnArgs a) {
  constexpr int DP = NC * 16;
  constexpr int KS = DP + kPad;      // Ks row stride
  constexpr int VS = TQ + kPad;      // Vt row stride
  __shared__ __attribute__((aligned(16))) T Ks[TQ * KS];
  __shared__ __attribute__((aligned(16))) T Ksl[sizeof(T) == 2 ? TQ * KS : 4];  // rotated k, low part
  __shared__ __attribute__((aligned(16))) T Vt[DP * VS];

  const int b = blockIdx.z, h = blockIdx.y, q0 = blockIdx.x * TQ;
  const int T_ = a.T, d = a.d;
  const int kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qi = q0 + wave * 16 + (lane & 15);   // this lane's query
  const int g4 = (lane >> 4) * 4;
  const float scale2 = kLog2e / sqrtf((float)d);

  const T* qb = static_cast<const T*>(a.q) + (int64_t)b * T_ * a.ldq + h * d;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * T_ * a.ldk + kvh * d;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * T_ * a.ldv + kvh * d;

  // Q fragments (rotated): lane holds Q[qi][16c + g4 + i] as hi + lo
  Pk<T, 4> qf[NC], qfl[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * c + g4 + i;
      f[i] = 0.f;
      if (qi < T_ && j < d) {
        const T* row = qb + (int64_t)qi * a.ldq;
        f[i] = a.R > 0 ? rope_elem<T>(row, j, qi, a.R, a.rope_mode, a.cs, 1.0f) : to_f32(row[j]);
      }
    }
    qf[c] = pack4<T>(f[0], f[1], f[2], f[3]);
    qfl[c] = low_part<T>(qf[c], f);
  }

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int last_q = min(T_, q0 + TQ) - 1;
  const int ntiles = last_q / TQ + 1;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * TQ;
    __syncthreads();
    stage_tile<T, DP, true>(kb, a.ldk, 0, k0, T_, d, a.R, a.rope_mode, a.cs, Ks, KS, nullptr, 0,
                            sizeof(T) == 2 ? Ksl : nullptr);
    stage_tile<T, DP, false>(vb, a.ldv, 0, k0, T_, d, 0, 0, nullptr, nullptr, 0, Vt, VS);
    __syncthreads();

    float s[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const Pk<T, 4> k4 = lds4(&Ks[(ks * 16 + (lane & 15)) * KS + 16 * c + g4]);
        acc = mma16(k4, qf[c], acc);
        if constexpr (sizeof(T) == 2) {
          acc = mma16(k4, qfl[c], acc);
          acc = mma16(lds4(&Ksl[(ks * 16 + (lane & 15)) * KS + 16 * c + g4]), qf[c], acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + ks * 16 + g4 + r;
        const float v = (key <= qi && key < T_) ? acc[r] * scale2 : -INFINITY;
        s[ks][r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float alpha = exp2f(m - mn);  // m = -inf on the first tile gives 0
    float rs = 0.f;
    Pk<T, 4> pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = exp2f(s[ks][r] - mn);
        rs += p[r];
      }
      pf[ks] = pack4<T>(p[0], p[1], p[2], p[3]);
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l = l * alpha + rs;
    m = mn;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      oacc[c] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        oacc[c] = mma16(lds4(&Vt[(16 * c + (lane & 15)) * VS + ks * 16 + g4]), pf[ks], oacc[c]);
    }
  }

  if (qi < T_) {
    const float inv = 1.0f / l;
    T* ob = static_cast<T*>(a.out) + ((int64_t)b * T_ + qi) * a.ldo + h * d;
    T* rb = a.ores_out ? static_cast<T*>(a.ores_out) + ((int64_t)b * T_ + qi) * ((int64_t)a.H * d) + h * d
                       : nullptr;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * c + g4 + r;
        if (j < d) {
          const float val = oacc[c][r] * inv;
          const T hi = from_f32<T>(val);
          ob[j] = hi;
          if (rb) rb[j] = from_f32<T>(val - to_f32(hi));
        }
      }
    if (lane < 16) a.lse[((int64_t)b * a.H + h) * T_ + qi] = (m + log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// dQ.  grid (ceil(T/64), H, B); wave w owns queries q0 + 16w + l%16.
//   D = dO . O (written for the dK/dV kernel, which runs after this one),
//   S^T = K Q^T, P = exp(S/sqrt(d) - lse), dP^T = V dO^T,
//   dS = P (dP - D), dQ^T += K^T dS^T, then dq = rotate^T(dQ) / sqrt(d).
// ---------------------------------------------------------------------------
template <typename T, int NC>
__global__ __launch_bounds__(256) void attn_bwd_dq_k(AttnArgs a) {
  constexpr int DP = NC * 16;
  constexpr int KS = DP + kPad;
  constexpr int TS = TQ + kPad;
  __shared__ __attribute__((aligned(16))) T Ks[TQ * KS];
  __shared__ __attribute__((aligned(16))) T Ksl[sizeof(T) == 2 ? TQ * KS : 4];  // rotated k, low part
  __shared__ __attribute__((aligned(16))) T Vs[TQ * KS];
  __shared__ __attribute__((aligned(16))) T Kt[DP * TS];
  __shared__ __attribute__((aligned(16))) T Ktl[sizeof(T) == 2 ? DP * TS : 4];  // rotated k, low part
  __shared__ float dqs[TQ * (DP + 1)];

  const int b = blockIdx.z, h = blockIdx.y, q0 = blockIdx.x * TQ;
  const int T_ = a.T, d = a.d;
  const int kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qi = q0 + wave * 16 + (lane & 15);
  const int g4 = (lane >> 4) * 4;
  const float scale = 1.0f / sqrtf((float)d);
  const float scale2 = kLog2e * scale;

  const T* qb = static_cast<const T*>(a.q) + (int64_t)b * T_ * a.ldq + h * d;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * T_ * a.ldk + kvh * d;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * T_ * a.ldv + kvh * d;
  const T* gb = static_cast<const T*>(a.dout) + (int64_t)b * T_ * a.lddo + h * d;

  // Q (rotated, hi + lo) and dO fragments; D = dO . O for this lane's query,
  // with O taken with its bf16 rounding residual (D multiplies the weighted
  // mean key, so its error is not averaged away over the keys).
  Pk<T, 4> qf[NC], qfl[NC], gf[NC];
  const T* ob = static_cast<const T*>(a.o) + (int64_t)b * T_ * a.ldo + h * d;
  const T* rbase = a.ores_in ? static_cast<const T*>(a.ores_in) + (int64_t)b * T_ * ((int64_t)a.H * d) + h * d
                             : nullptr;
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float f[4], g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * c + g4 + i;
      f[i] = g[i] = 0.f;
      if (qi < T_ && j < d) {
        const T* row = qb + (int64_t)qi * a.ldq;
        f[i] = a.R > 0 ? rope_elem<T>(row, j, qi, a.R, a.rope_mode, a.cs, 1.0f) : to_f32(row[j]);
        g[i] = to_f32(gb[(int64_t)qi * a.lddo + j]);
        float ov = to_f32(ob[(int64_t)qi * a.ldo + j]);
        if (rbase) ov += to_f32(rbase[(int64_t)qi * ((int64_t)a.H * d) + j]);
        dpart += ov * g[i];
      }
    }
    qf[c] = pack4<T>(f[0], f[1], f[2], f[3]);
    qfl[c] = low_part<T>(qf[c], f);
    gf[c] = pack4<T>(g[0], g[1], g[2], g[3]);
  }
  dpart += __shfl_xor(dpart, 16, 64);
  dpart += __shfl_xor(dpart, 32, 64);
  const float Dq = dpart;
  const int64_t srow = ((int64_t)b * a.H + h) * T_;
  if (qi < T_ && lane < 16) a.delta[srow + qi] = Dq;   // read by the dK/dV kernel
  const float lse2 = qi < T_ ? a.lse_in[srow + qi] * kLog2e : 0.f;

  f32x4 dqacc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dqacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int last_q = min(T_, q0 + TQ) - 1;
  const int ntiles = last_q / TQ + 1;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * TQ;
    __syncthreads();
    stage_tile<T, DP, true>(kb, a.ldk, 0, k0, T_, d, a.R, a.rope_mode, a.cs, Ks, KS, Kt, TS,
                            sizeof(T) == 2 ? Ksl : nullptr, sizeof(T) == 2 ? Ktl : nullptr);
    stage_tile<T, DP, false>(vb, a.ldv, 0, k0, T_, d, 0, 0, nullptr, Vs, KS, nullptr, 0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const Pk<T, 4> k4 = lds4(&Ks[(ks * 16 + (lane & 15)) * KS + 16 * c + g4]);
        sacc = mma16(k4, qf[c], sacc);
        if constexpr (sizeof(T) == 2) {
          sacc = mma16(k4, qfl[c], sacc);
          sacc = mma16(lds4(&Ksl[(ks * 16 + (lane & 15)) * KS + 16 * c + g4]), qf[c], sacc);
        }
        pacc = mma16(lds4(&Vs[(ks * 16 + (lane & 15)) * KS + 16 * c + g4]), gf[c], pacc);
      }
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + ks * 16 + g4 + r;
        const bool ok = key <= qi && key < T_ && qi < T_;
        const float p = ok ? exp2f(sacc[r] * scale2 - lse2) : 0.f;
        ds[r] = p * (pacc[r] - Dq);
      }
      const Pk<T, 4> dsf = pack4<T>(ds[0], ds[1], ds[2], ds[3]);
      const Pk<T, 4> dsl = low_part<T>(dsf, ds);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const Pk<T, 4> kt4 = lds4(&Kt[(16 * c + (lane & 15)) * TS + ks * 16 + g4]);
        dqacc[c] = mma16(kt4, dsf, dqacc[c]);
        if constexpr (sizeof(T) == 2) {
          dqacc[c] = mma16(kt4, dsl, dqacc[c]);
          dqacc[c] = mma16(lds4(&Ktl[(16 * c + (lane & 15)) * TS + ks * 16 + g4]), dsf, dqacc[c]);
        }
      }
    }
  }
  // dq~ (rotated frame) -> LDS, then rotate back and store.
  __syncthreads();
  constexpr int QS = DP + 1;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) dqs[(wave * 16 + (lane & 15)) * QS + 16 * c + g4 + r] = dqacc[c][r] * scale;
  __syncthreads();
  T* db = static_cast<T*>(a.dq) + (int64_t)b * T_ * a.lddq + h * d;
  for (int idx = threadIdx.x; idx < TQ * d; idx += blockDim.x) {
    const int r = idx / d, j = idx % d;
    const int t = q0 + r;
    if (t >= T_) continue;
    const float v = a.R > 0 ? rope_elem_f(&dqs[r * QS], j, t, a.R, a.rope_mode, a.cs, -1.0f) : dqs[r * QS + j];
    db[(int64_t)t * a.lddq + j] = from_f32<T>(v);
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  grid (ceil(T/64), Hkv, B); wave w owns keys k0 + 16w + l%16 and
// loops over the query heads of its KV head and the query tiles at or after
// its key tile:  S = Q K^T, P = exp(S/sqrt(d) - lse), dP = dO V^T,
// dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <typename T, int NC>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_k(AttnArgs a) {
  constexpr int DP = NC * 16;
  constexpr int XS = DP + kPad;
  constexpr int TS = TQ + kPad;
  __shared__ __attribute__((aligned(16))) T Qs[TQ * XS];
  __shared__ __attribute__((aligned(16))) T Qsl[sizeof(T) == 2 ? TQ * XS : 4];  // rotated q, low part
  __shared__ __attribute__((aligned(16))) T Gs[TQ * XS];
  __shared__ __attribute__((aligned(16))) T Qt[DP * TS];
  __shared__ __attribute__((aligned(16))) T Qtl[sizeof(T) == 2 ? DP * TS : 4];  // rotated q^T, low part
  __shared__ __attribute__((aligned(16))) T Gt[DP * TS];
  __shared__ float lse2s[TQ], Ds[TQ];

  const int b = blockIdx.z, kvh = blockIdx.y, k0 = blockIdx.x * TQ;
  const int T_ = a.T, d = a.d;
  const int rep = a.H / a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ki = k0 + wave * 16 + (lane & 15);   // this lane's key
  const int g4 = (lane >> 4) * 4;
  const float scale = 1.0f / sqrtf((float)d);
  const float scale2 = kLog2e * scale;

  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * T_ * a.ldk + kvh * d;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * T_ * a.ldv + kvh * d;

  Pk<T, 4> kf[NC], kfl[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float f[4], g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * c + g4 + i;
      f[i] = g[i] = 0.f;
      if (ki < T_ && j < d) {
        const T* row = kb + (int64_t)ki * a.ldk;
        f[i] = a.R > 0 ? rope_elem<T>(row, j, ki, a.R, a.rope_mode, a.cs, 1.0f) : to_f32(row[j]);
        g[i] = to_f32(vb[(int64_t)ki * a.ldv + j]);
      }
    }
    kf[c] = pack4<T>(f[0], f[1], f[2], f[3]);
    kfl[c] = low_part<T>(kf[c], f);
    vf[c] = pack4<T>(g[0], g[1], g[2], g[3]);
  }

  f32x4 dk[NC], dv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dk[c] = dv[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nqt = (T_ + TQ - 1) / TQ;
  for (int hh = 0; hh < rep; ++hh) {
    const int h = kvh * rep + hh;
    const T* qb = static_cast<const T*>(a.q) + (int64_t)b * T_ * a.ldq + h * d;
    const T* gb = static_cast<const T*>(a.dout) + (int64_t)b * T_ * a.lddo + h * d;
    const int64_t srow = ((int64_t)b * a.H + h) * T_;
    for (int qt = blockIdx.x; qt < nqt; ++qt) {
      const int q0 = qt * TQ;
      __syncthreads();
      stage_tile<T, DP, true>(qb, a.ldq, 0, q0, T_, d, a.R, a.rope_mode, a.cs, Qs, XS, Qt, TS,
                              sizeof(T) == 2 ? Qsl : nullptr, sizeof(T) == 2 ? Qtl : nullptr);
      stage_tile<T, DP, false>(gb, a.lddo, 0, q0, T_, d, 0, 0, nullptr, Gs, XS, Gt, TS);
      if (threadIdx.x < TQ) {
        const int t = q0 + threadIdx.x;
        lse2s[threadIdx.x] = t < T_ ? a.lse_in[srow + t] * kLog2e : 0.f;
        Ds[threadIdx.x] = t < T_ ? a.delta[srow + t] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const Pk<T, 4> q4 = lds4(&Qs[(qs * 16 + (lane & 15)) * XS + 16 * c + g4]);
          sacc = mma16(q4, kf[c], sacc);
          if constexpr (sizeof(T) == 2) {
            sacc = mma16(lds4(&Qsl[(qs * 16 + (lane & 15)) * XS + 16 * c + g4]), kf[c], sacc);
            sacc = mma16(q4, kfl[c], sacc);
          }
          pacc = mma16(lds4(&Gs[(qs * 16 + (lane & 15)) * XS + 16 * c + g4]), vf[c], pacc);
        }
        float p[4], ds[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = qs * 16 + g4 + r;
          const int q = q0 + ql;
          const bool ok = ki <= q && q < T_ && ki < T_;
          p[r] = ok ? exp2f(sacc[r] * scale2 - lse2s[ql]) : 0.f;
          ds[r] = p[r] * (pacc[r] - Ds[ql]);
        }
        const Pk<T, 4> pf = pack4<T>(p[0], p[1], p[2], p[3]);
        const Pk<T, 4> dsf = pack4<T>(ds[0], ds[1], ds[2], ds[3]);
        const Pk<T, 4> dsl = low_part<T>(dsf, ds);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          dv[c] = mma16(lds4(&Gt[(16 * c + (lane & 15)) * TS + qs * 16 + g4]), pf, dv[c]);
          const Pk<T, 4> qt4 = lds4(&Qt[(16 * c + (lane & 15)) * TS + qs * 16 + g4]);
          dk[c] = mma16(qt4, dsf, dk[c]);
          if constexpr (sizeof(T) == 2) {
            dk[c] = mma16(qt4, dsl, dk[c]);
            dk[c] = mma16(lds4(&Qtl[(16 * c + (lane & 15)) * TS + qs * 16 + g4]), dsf, dk[c]);
          }
        }
      }
    }
  }

  // dv: lane holds dV[ki][16c + g4 + r]
  if (ki < T_) {
    T* dvb = static_cast<T*>(a.dv) + ((int64_t)b * T_ + ki) * a.lddv + kvh * d;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * c + g4 + r;
        if (j < d) dvb[j] = from_f32<T>(dv[c][r]);
      }
  }
  // dk~ -> LDS (reusing Qs/Gs space as fp32), rotate back, store.
  __syncthreads();
  constexpr int QS2 = DP + 1;
  __shared__ float dkbuf[TQ * QS2];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) dkbuf[(wave * 16 + (lane & 15)) * QS2 + 16 * c + g4 + r] = dk[c][r] * scale;
  __syncthreads();
  T* dkb = static_cast<T*>(a.dk) + (int64_t)b * T_ * a.lddk + kvh * d;
  for (int idx = threadIdx.x; idx < TQ * d; idx += blockDim.x) {
    const int r = idx / d, j = idx % d;
    const int t = k0 + r;
    if (t >= T_) continue;
    const float v = a.R > 0 ? rope_elem_f(&dkbuf[r * QS2], j, t, a.R, a.rope_mode, a.cs, -1.0f) : dkbuf[r * QS2 + j];
    dkb[(int64_t)t * a.lddk + j] = from_f32<T>(v);
  }
}

}  // namespace

int64_t attention_bwd_ws(int B, int H, int T) { return (int64_t)B * H * T * 4; }

template <typename T>
static slt_status attn_fwd_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.T + TQ - 1) / TQ, a.H, a.B);
  const int nc = (a.d + 15) / 16;
  switch (nc) {
    case 1: attn_fwd_k<T, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: attn_fwd_k<T, 2><<<grid, 256, 0, s>>>(a); break;
    case 3: attn_fwd_k<T, 3><<<grid, 256, 0, s>>>(a); break;
    case 4: attn_fwd_k<T, 4><<<grid, 256, 0, s>>>(a); break;
    default: return fail(SLT_EUNSUPPORTED, "attention: head dim above 64");
  }
  return check_launch("attention_fwd");
}

template <typename T>
static slt_status attn_bwd_t(const AttnArgs& a, hipStream_t s) {
  dim3 gq((a.T + TQ - 1) / TQ, a.H, a.B);
  dim3 gk((a.T + TQ - 1) / TQ, a.Hkv, a.B);
  const int nc = (a.d + 15) / 16;
  switch (nc) {
#define SLT_ATT_BWD(NCv)                                  \
  case NCv:                                               \
    attn_bwd_dq_k<T, NCv><<<gq, 256, 0, s>>>(a);          \
    attn_bwd_dkdv_k<T, NCv><<<gk, 256, 0, s>>>(a);        \
    break;
    SLT_ATT_BWD(1) SLT_ATT_BWD(2) SLT_ATT_BWD(3) SLT_ATT_BWD(4)
#undef SLT_ATT_BWD
    default: return fail(SLT_EUNSUPPORTED, "attention: head dim above 64");
  }
  return check_launch("attention_bwd");
}

slt_status launch_attention_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return SLT_OK;
  return a.dtype == SLT_BF16 ? attn_fwd_t<bf16>(a, s) : attn_fwd_t<float>(a, s);
}

slt_status launch_attention_bwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return SLT_OK;
  return a.dtype == SLT_BF16 ? attn_bwd_t<bf16>(a, s) : attn_bwd_t<float>(a, s);
}

}  // namespace slt
