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
//
// Staging: RoPE is applied while a tile is copied from HBM to LDS.  On the
// vector path a thread takes 4 rows x 16 bytes of dims, loads the partner
// dims of each pair and the (cos, sin) table entries as vectors, rotates in
// fp32, and writes the rows (16-byte stores) and, for operands needed
// transposed, the 4-row columns (8-byte stores).  Shapes whose pairs do not
// fall on 16-byte groups take the element-wise path.
//
// Precision (bf16): the rotated q and k are rounded once to bf16, as the
// step stores them (the low parts of their two-term expansions are zero
// here); the probability gradient dS enters its products as a bf16 hi + lo
// pair (dS sums to zero along a row).  D = dO.O uses O with its bf16 rounding
// residual (see the forward).
#include "slt_internal.h"

#include <math.h>

namespace slt {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TQ = 64;  // rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int N>
struct alignas(sizeof(T) * N) Pk {
  T e[N];
};

template <typename T> __device__ __forceinline__ T zero_v();
template <> __device__ __forceinline__ bf16 zero_v<bf16>() { return bf16{0}; }
template <> __device__ __forceinline__ float zero_v<float>() { return 0.f; }

template <typename T> constexpr bool kBf = sizeof(T) == 2;
template <typename T> constexpr int kG = 16 / (int)sizeof(T);  // elements per 16 bytes

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
__device__ __forceinline__ Pk<T, 4> pack4(const float (&v)[4]) {
  Pk<T, 4> p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p.e[i] = from_f32<T>(v[i]);
  return p;
}

// Second term of a two-term bf16 expansion v ~ hi + lo.
template <typename T>
__device__ __forceinline__ Pk<T, 4> low_part(const Pk<T, 4>& hi, const float (&v)[4]) {
  Pk<T, 4> p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p.e[i] = from_f32<T>(v[i] - to_f32(hi.e[i]));
  return p;
}

template <typename T>
__device__ __forceinline__ Pk<T, 4> lds4(const T* p) {
  return *reinterpret_cast<const Pk<T, 4>*>(p);
}

// Dim j of row u at position t after RoPE (sign +1) or after the transposed
// rotation (sign -1, the backward of RoPE); dims >= R pass through.
// cs: [T][R] with (cos, sin) of angle t * theta_i at 2i, 2i+1.
template <typename U>
__device__ __forceinline__ float rope_elem(const U* u, int j, int t, int R, int mode, const float* cs, float sign) {
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

// G consecutive dims j0..j0+G-1 of row u at position t, rotated (sign +1) or
// rotated back (sign -1).  Requires j0 % G == 0 and pairs aligned to G
// (half mode: (R/2) % G == 0; pairs mode: R % G == 0 with G even), which the
// host checks before choosing the vector path.
template <int G, typename U>
__device__ __forceinline__ void rope_group(const U* u, int j0, int t, int R, int mode, const float* cs, float sign,
                                           float (&out)[G]) {
  Pk<U, G> own = *reinterpret_cast<const Pk<U, G>*>(u + j0);
#pragma unroll
  for (int e = 0; e < G; ++e) out[e] = to_f32(own.e[e]);
  if (R == 0 || j0 >= R) return;
  const float2* tb = reinterpret_cast<const float2*>(cs + (int64_t)t * R);
  if (mode == SLT_ROPE_HALF) {
    const int h = R >> 1;
    const bool first = j0 < h;
    const int i0 = first ? j0 : j0 - h;
    Pk<U, G> par = *reinterpret_cast<const Pk<U, G>*>(u + (first ? j0 + h : j0 - h));
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const float2 c = tb[i0 + e];
      const float x = out[e], y = to_f32(par.e[e]);
      out[e] = first ? x * c.x - y * (sign * c.y) : x * c.x + y * (sign * c.y);
    }
  } else {
#pragma unroll
    for (int e = 0; e < G; e += 2) {
      const float2 c = tb[(j0 + e) >> 1];
      const float x = out[e], y = out[e + 1];
      out[e] = x * c.x - y * (sign * c.y);
      out[e + 1] = y * c.x + x * (sign * c.y);
    }
  }
}

// The 4 dims j0 .. j0+3 of row `row` at position t (zero when not valid or
// beyond d), rotated when ROT.
template <typename T, bool VEC, bool ROT>
__device__ __forceinline__ void frag_load(const T* row, bool valid, int j0, int d, int t, int R, int mode,
                                          const float* cs, float (&f)[4]) {
  if (VEC) {
    if (valid && j0 < d) {
      if (ROT) {
        rope_group<4>(row, j0, t, R, mode, cs, 1.0f, f);
      } else {
        Pk<T, 4> p = *reinterpret_cast<const Pk<T, 4>*>(row + j0);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = to_f32(p.e[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      f[i] = (valid && j < d) ? (ROT && R > 0 ? rope_elem(row, j, t, R, mode, cs, 1.0f) : to_f32(row[j])) : 0.f;
    }
  }
}

// Stage rows [row0, row0 + 64) of a [T, d] operand (row stride ld) into LDS,
// dims padded to DP, rows >= T and dims >= d zero.  Outputs, each optional:
// X[r*XS + j] (bf16-rounded value), Xl (its rounding residual, rotated
// operands only), Xt[j*XTS + r] and Xtl (the same transposed).
template <typename T, int DP, bool ROT, bool VEC>
__device__ __forceinline__ void stage(const T* base, int64_t ld, int row0, int T_, int d, int R, int mode,
                                      const float* cs, T* X, T* Xl, int XS, T* Xt, T* Xtl, int XTS) {
  if constexpr (VEC) {
    constexpr int G = kG<T>;
    constexpr int NCH = DP / G;
    for (int item = threadIdx.x; item < (TQ / 4) * NCH; item += blockDim.x) {
      const int rg = item / NCH, j0 = (item % NCH) * G;
      float v[4][G];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = row0 + 4 * rg + rr;
        if (t < T_ && j0 < d) {
          const T* row = base + (int64_t)t * ld;
          if (ROT) {
            rope_group<G>(row, j0, t, R, mode, cs, 1.0f, v[rr]);
          } else {
            Pk<T, G> p = *reinterpret_cast<const Pk<T, G>*>(row + j0);
#pragma unroll
            for (int e = 0; e < G; ++e) v[rr][e] = to_f32(p.e[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < G; ++e) v[rr][e] = 0.f;
        }
      }
      Pk<T, G> hi[4], lo[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int e = 0; e < G; ++e) {
          hi[rr].e[e] = from_f32<T>(v[rr][e]);
          lo[rr].e[e] = zero_v<T>();  // rotated operands are rounded once
        }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        if (X) *reinterpret_cast<Pk<T, G>*>(X + (4 * rg + rr) * XS + j0) = hi[rr];
        if (Xl) *reinterpret_cast<Pk<T, G>*>(Xl + (4 * rg + rr) * XS + j0) = lo[rr];
      }
#pragma unroll
      for (int e = 0; e < G; ++e) {
        if (Xt) {
          Pk<T, 4> col;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) col.e[rr] = hi[rr].e[e];
          *reinterpret_cast<Pk<T, 4>*>(Xt + (j0 + e) * XTS + 4 * rg) = col;
        }
        if (Xtl) {
          Pk<T, 4> col;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) col.e[rr] = lo[rr].e[e];
          *reinterpret_cast<Pk<T, 4>*>(Xtl + (j0 + e) * XTS + 4 * rg) = col;
        }
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < TQ * DP; idx += blockDim.x) {
      const int r = idx / DP, j = idx % DP;
      const int t = row0 + r;
      float f = 0.f;
      if (t < T_ && j < d) {
        const T* row = base + (int64_t)t * ld;
        f = (ROT && R > 0) ? rope_elem(row, j, t, R, mode, cs, 1.0f) : to_f32(row[j]);
      }
      const T hv = from_f32<T>(f);
      const T lv = zero_v<T>();  // rotated operands are rounded once
      if (X) X[r * XS + j] = hv;
      if (Xl) Xl[r * XS + j] = lv;
      if (Xt) Xt[j * XTS + r] = hv;
      if (Xtl) Xtl[j * XTS + r] = lv;
    }
  }
}

// Rotate back rows held in LDS as fp32 (F[r*FS + j], r < 64) and store them
// to out[(row0 + r) * ld + j] for rows < T.
template <typename T, bool VEC>
__device__ __forceinline__ void store_unrotated(const float* F, int FS, T* out, int64_t ld, int row0, int T_, int d,
                                                int R, int mode, const float* cs) {
  if (VEC) {
    const int ng = d / 4;
    for (int idx = threadIdx.x; idx < TQ * ng; idx += blockDim.x) {
      const int r = idx / ng, j0 = (idx % ng) * 4;
      const int t = row0 + r;
      if (t >= T_) continue;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = F[r * FS + j0 + i];
      if (R > 0 && j0 < R) {
        // the partner dims of this group, read from the fp32 row in LDS
        const float2* tb = reinterpret_cast<const float2*>(cs + (int64_t)t * R);
        if (mode == SLT_ROPE_HALF) {
          const int h = R >> 1;
          const bool first = j0 < h;
          const int i0 = first ? j0 : j0 - h, p0 = first ? j0 + h : j0 - h;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float2 c = tb[i0 + i];
            const float x = v[i], y = F[r * FS + p0 + i];
            v[i] = first ? x * c.x + y * c.y : x * c.x - y * c.y;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float2 c = tb[(j0 + i) >> 1];
            const float x = v[i], y = v[i + 1];
            v[i] = x * c.x + y * c.y;
            v[i + 1] = y * c.x - x * c.y;
          }
        }
      }
      *reinterpret_cast<Pk<T, 4>*>(out + (int64_t)t * ld + j0) = pack4<T>(v);
    }
  } else {
    for (int idx = threadIdx.x; idx < TQ * d; idx += blockDim.x) {
      const int r = idx / d, j = idx % d;
      const int t = row0 + r;
      if (t >= T_) continue;
      const float v = R > 0 ? rope_elem(&F[r * FS], j, t, R, mode, cs, -1.0f) : F[r * FS + j];
      out[(int64_t)t * ld + j] = from_f32<T>(v);
    }
  }
}

template <typename T, int NC>
struct Geo {
  static constexpr int DP = NC * 16;
  static constexpr int XS = DP + kG<T>;   // row stride of row-major tiles (16-byte aligned rows)
  static constexpr int TS = TQ + kG<T>;   // row stride of transposed tiles
  static constexpr int TILE = TQ * XS;    // elements of a row-major tile
  static constexpr int TTILE = DP * TS;   // elements of a transposed tile
  static constexpr int FS = DP + 1;       // fp32 scratch row stride
};

// ---------------------------------------------------------------------------
// Forward.  grid (ceil(T/64), H, B); wave w owns queries q0 + 16w + l%16.
// ---------------------------------------------------------------------------
template <typename T, int NC, bool VEC, bool DROP>
__global__ __launch_bounds__(256) void attn_fwd_k(AttnArgs a) {
  using Gm = Geo<T, NC>;
  constexpr int DP = Gm::DP, XS = Gm::XS, TS = Gm::TS;
  __shared__ __attribute__((aligned(16))) T smem[2 * Gm::TILE + Gm::TTILE];
  T* Ks = smem;                 // rotated k (bf16-rounded)
  T* Ksl = smem + Gm::TILE;     // its residual (bf16 only)
  T* Vt = smem + 2 * Gm::TILE;  // v transposed

  const int b = blockIdx.z, h = blockIdx.y, q0 = blockIdx.x * TQ;
  const int T_ = a.T, d = a.d;
  const int kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qi = q0 + wave * 16 + (lane & 15);
  const int g4 = (lane >> 4) * 4;
  const float scale2 = kLog2e / sqrtf((float)d);

  const T* qb = static_cast<const T*>(a.q) + (int64_t)b * T_ * a.ldq + h * d;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * T_ * a.ldk + kvh * d;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * T_ * a.ldv + kvh * d;

  Pk<T, 4> qf[NC], qfl[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float f[4];
    frag_load<T, VEC, true>(qb + (int64_t)qi * a.ldq, qi < T_, 16 * c + g4, d, qi, a.R, a.rope_mode, a.cs, f);
    qf[c] = pack4<T>(f);
    qfl[c] = Pk<T, 4>{};  // rotated q rounded once
  }

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (min(T_, q0 + TQ) - 1) / TQ + 1;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * TQ;
    __syncthreads();
    stage<T, DP, true, VEC>(kb, a.ldk, k0, T_, d, a.R, a.rope_mode, a.cs, Ks, kBf<T> ? Ksl : nullptr, XS, nullptr,
                            nullptr, TS);
    stage<T, DP, false, VEC>(vb, a.ldv, k0, T_, d, 0, 0, nullptr, nullptr, nullptr, XS, Vt, nullptr, TS);
    __syncthreads();

    float s[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (ks * 16 + (lane & 15)) * XS + 16 * c + g4;
        const Pk<T, 4> k4 = lds4(&Ks[off]);
        acc = mma16(k4, qf[c], acc);
        if constexpr (kBf<T>) {
          acc = mma16(k4, qfl[c], acc);
          acc = mma16(lds4(&Ksl[off]), qf[c], acc);
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
      if (DROP) {  // the normaliser keeps every weight; the values see the dropped ones
        float dm[4];
        drop_mults<4>(a.drop, att_elem(b, a.H, h, T_, qi, k0 + ks * 16 + g4), dm);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] *= dm[r];
      }
      pf[ks] = pack4<T>(p);
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
        oacc[c] = mma16(lds4(&Vt[(16 * c + (lane & 15)) * TS + ks * 16 + g4]), pf[ks], oacc[c]);
    }
  }

  // o: lane holds O[qi][16c + g4 + r]; the residual o - bf16(o) goes to ores_out.
  if (qi < T_) {
    const float inv = 1.0f / l;
    T* ob = static_cast<T*>(a.out) + ((int64_t)b * T_ + qi) * a.ldo + h * d;
    T* rb = a.ores_out ? static_cast<T*>(a.ores_out) + ((int64_t)b * T_ + qi) * ((int64_t)a.H * d) + h * d
                       : nullptr;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j0 = 16 * c + g4;
      if (j0 >= d) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = oacc[c][r] * inv;
      const Pk<T, 4> hi = pack4<T>(v);
      const Pk<T, 4> lo = low_part<T>(hi, v);
      if (VEC) {
        *reinterpret_cast<Pk<T, 4>*>(ob + j0) = hi;
        if (rb) *reinterpret_cast<Pk<T, 4>*>(rb + j0) = lo;
      } else {
        for (int r = 0; r < 4 && j0 + r < d; ++r) {
          ob[j0 + r] = hi.e[r];
          if (rb) rb[j0 + r] = lo.e[r];
        }
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
template <typename T, int NC, bool VEC, bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dq_k(AttnArgs a) {
  using Gm = Geo<T, NC>;
  constexpr int DP = Gm::DP, XS = Gm::XS, TS = Gm::TS, FS = Gm::FS;
  constexpr int TILES = 3 * Gm::TILE + 2 * Gm::TTILE;
  constexpr int FBYTES = TQ * FS * 4;
  constexpr int SBYTES = TILES * (int)sizeof(T) > FBYTES ? TILES * (int)sizeof(T) : FBYTES;
  __shared__ __attribute__((aligned(16))) char smem[SBYTES];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Ksl = Ks + Gm::TILE;
  T* Vs = Ks + 2 * Gm::TILE;
  T* Kt = Ks + 3 * Gm::TILE;
  T* Ktl = Kt + Gm::TTILE;
  float* dqs = reinterpret_cast<float*>(smem);  // reused after the last tile

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
  const T* ob = static_cast<const T*>(a.o) + (int64_t)b * T_ * a.ldo + h * d;
  const T* rbase = a.ores_in ? static_cast<const T*>(a.ores_in) + (int64_t)b * T_ * ((int64_t)a.H * d) + h * d
                             : nullptr;

  Pk<T, 4> qf[NC], qfl[NC], gf[NC];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j0 = 16 * c + g4;
    float f[4], g[4], o[4], r4[4];
    frag_load<T, VEC, true>(qb + (int64_t)qi * a.ldq, qi < T_, j0, d, qi, a.R, a.rope_mode, a.cs, f);
    frag_load<T, VEC, false>(gb + (int64_t)qi * a.lddo, qi < T_, j0, d, qi, 0, 0, nullptr, g);
    frag_load<T, VEC, false>(ob + (int64_t)qi * a.ldo, qi < T_, j0, d, qi, 0, 0, nullptr, o);
    if (rbase) {
      frag_load<T, VEC, false>(rbase + (int64_t)qi * ((int64_t)a.H * d), qi < T_, j0, d, qi, 0, 0, nullptr, r4);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) r4[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dpart += (o[i] + r4[i]) * g[i];
    qf[c] = pack4<T>(f);
    qfl[c] = Pk<T, 4>{};  // rotated q rounded once
    gf[c] = pack4<T>(g);
  }
  dpart += __shfl_xor(dpart, 16, 64);
  dpart += __shfl_xor(dpart, 32, 64);
  const float Dq = dpart;
  const int64_t srow = ((int64_t)b * a.H + h) * T_;
  if (qi < T_ && lane < 16) a.delta[srow + qi] = Dq;  // read by the dK/dV kernel
  const float lse2 = qi < T_ ? a.lse_in[srow + qi] * kLog2e : 0.f;

  f32x4 dqacc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dqacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (min(T_, q0 + TQ) - 1) / TQ + 1;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * TQ;
    __syncthreads();
    stage<T, DP, true, VEC>(kb, a.ldk, k0, T_, d, a.R, a.rope_mode, a.cs, Ks, kBf<T> ? Ksl : nullptr, XS, Kt,
                            kBf<T> ? Ktl : nullptr, TS);
    stage<T, DP, false, VEC>(vb, a.ldv, k0, T_, d, 0, 0, nullptr, Vs, nullptr, XS, nullptr, nullptr, TS);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (ks * 16 + (lane & 15)) * XS + 16 * c + g4;
        const Pk<T, 4> k4 = lds4(&Ks[off]);
        sacc = mma16(k4, qf[c], sacc);
        if constexpr (kBf<T>) {
          sacc = mma16(k4, qfl[c], sacc);
          sacc = mma16(lds4(&Ksl[off]), qf[c], sacc);
        }
        pacc = mma16(lds4(&Vs[off]), gf[c], pacc);
      }
      float ds[4], dm[4] = {1.f, 1.f, 1.f, 1.f};
      if (DROP) drop_mults<4>(a.drop, att_elem(b, a.H, h, T_, qi, k0 + ks * 16 + g4), dm);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + ks * 16 + g4 + r;
        const bool ok = key <= qi && key < T_ && qi < T_;
        const float p = ok ? exp2f(sacc[r] * scale2 - lse2) : 0.f;
        ds[r] = DROP ? p * (dm[r] * pacc[r] - Dq) : p * (pacc[r] - Dq);
      }
      const Pk<T, 4> dsf = pack4<T>(ds);
      const Pk<T, 4> dsl = low_part<T>(dsf, ds);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int toff = (16 * c + (lane & 15)) * TS + ks * 16 + g4;
        const Pk<T, 4> kt4 = lds4(&Kt[toff]);
        dqacc[c] = mma16(kt4, dsf, dqacc[c]);
        if constexpr (kBf<T>) {
          dqacc[c] = mma16(kt4, dsl, dqacc[c]);
          dqacc[c] = mma16(lds4(&Ktl[toff]), dsf, dqacc[c]);
        }
      }
    }
  }
  // dq~ (rotated frame) -> LDS, then rotate back and store.
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) dqs[(wave * 16 + (lane & 15)) * FS + 16 * c + g4 + r] = dqacc[c][r] * scale;
  __syncthreads();
  T* dqb = static_cast<T*>(a.dq) + (int64_t)b * T_ * a.lddq + h * d;
  store_unrotated<T, VEC>(dqs, FS, dqb, a.lddq, q0, T_, d, a.R, a.rope_mode, a.cs);
}

// ---------------------------------------------------------------------------
// dK, dV.  grid (ceil(T/64), Hkv, B); wave w owns keys k0 + 16w + l%16 and
// loops over the query heads of its KV head and the query tiles at or after
// its key tile:  S = Q K^T, P = exp(S/sqrt(d) - lse), dP = dO V^T,
// dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <typename T, int NC, bool VEC, bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_k(AttnArgs a) {
  using Gm = Geo<T, NC>;
  constexpr int DP = Gm::DP, XS = Gm::XS, TS = Gm::TS, FS = Gm::FS;
  constexpr int TILES = 3 * Gm::TILE + 3 * Gm::TTILE;
  constexpr int FBYTES = TQ * FS * 4;
  constexpr int SBYTES = TILES * (int)sizeof(T) > FBYTES ? TILES * (int)sizeof(T) : FBYTES;
  __shared__ __attribute__((aligned(16))) char smem[SBYTES];
  __shared__ float lse2s[TQ], Ds[TQ];
  T* Qs = reinterpret_cast<T*>(smem);
  T* Qsl = Qs + Gm::TILE;
  T* Gs = Qs + 2 * Gm::TILE;
  T* Qt = Qs + 3 * Gm::TILE;
  T* Qtl = Qt + Gm::TTILE;
  T* Gt = Qt + 2 * Gm::TTILE;
  float* dks = reinterpret_cast<float*>(smem);  // reused after the last tile

  const int b = blockIdx.z, kvh = blockIdx.y, k0 = blockIdx.x * TQ;
  const int T_ = a.T, d = a.d;
  const int rep = a.H / a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ki = k0 + wave * 16 + (lane & 15);  // this lane's key
  const int g4 = (lane >> 4) * 4;
  const float scale = 1.0f / sqrtf((float)d);
  const float scale2 = kLog2e * scale;

  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * T_ * a.ldk + kvh * d;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * T_ * a.ldv + kvh * d;

  Pk<T, 4> kf[NC], kfl[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float f[4], g[4];
    frag_load<T, VEC, true>(kb + (int64_t)ki * a.ldk, ki < T_, 16 * c + g4, d, ki, a.R, a.rope_mode, a.cs, f);
    frag_load<T, VEC, false>(vb + (int64_t)ki * a.ldv, ki < T_, 16 * c + g4, d, ki, 0, 0, nullptr, g);
    kf[c] = pack4<T>(f);
    kfl[c] = Pk<T, 4>{};  // rotated k rounded once
    vf[c] = pack4<T>(g);
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
      stage<T, DP, true, VEC>(qb, a.ldq, q0, T_, d, a.R, a.rope_mode, a.cs, Qs, kBf<T> ? Qsl : nullptr, XS, Qt,
                              kBf<T> ? Qtl : nullptr, TS);
      stage<T, DP, false, VEC>(gb, a.lddo, q0, T_, d, 0, 0, nullptr, Gs, nullptr, XS, Gt, nullptr, TS);
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
          const int off = (qs * 16 + (lane & 15)) * XS + 16 * c + g4;
          const Pk<T, 4> q4 = lds4(&Qs[off]);
          sacc = mma16(q4, kf[c], sacc);
          if constexpr (kBf<T>) {
            sacc = mma16(lds4(&Qsl[off]), kf[c], sacc);
            sacc = mma16(q4, kfl[c], sacc);
          }
          pacc = mma16(lds4(&Gs[off]), vf[c], pacc);
        }
        float p[4], ds[4], dm[4] = {1.f, 1.f, 1.f, 1.f};
        if (DROP) drop_mults_strided<4>(a.drop, att_elem(b, a.H, h, T_, q0 + qs * 16 + g4, ki), (uint64_t)T_, dm);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = qs * 16 + g4 + r;
          const int q = q0 + ql;
          const bool ok = ki <= q && q < T_ && ki < T_;
          p[r] = ok ? exp2f(sacc[r] * scale2 - lse2s[ql]) : 0.f;
          if (DROP) {  // dS takes the dropped dP, dV the dropped weights
            ds[r] = p[r] * (dm[r] * pacc[r] - Ds[ql]);
            p[r] *= dm[r];
          } else {
            ds[r] = p[r] * (pacc[r] - Ds[ql]);
          }
        }
        const Pk<T, 4> pf = pack4<T>(p);
        const Pk<T, 4> pfl = low_part<T>(pf, p);  // dV sums over the whole group: P as hi + lo
        const Pk<T, 4> dsf = pack4<T>(ds);
        const Pk<T, 4> dsl = low_part<T>(dsf, ds);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int toff = (16 * c + (lane & 15)) * TS + qs * 16 + g4;
          const Pk<T, 4> gt4 = lds4(&Gt[toff]);
          dv[c] = mma16(gt4, pf, dv[c]);
          if constexpr (kBf<T>) dv[c] = mma16(gt4, pfl, dv[c]);
          const Pk<T, 4> qt4 = lds4(&Qt[toff]);
          dk[c] = mma16(qt4, dsf, dk[c]);
          if constexpr (kBf<T>) {
            dk[c] = mma16(qt4, dsl, dk[c]);
            dk[c] = mma16(lds4(&Qtl[toff]), dsf, dk[c]);
          }
        }
      }
    }
  }

  // dv: lane holds dV[ki][16c + g4 + r]
  if (ki < T_) {
    T* dvb = static_cast<T*>(a.dv) + ((int64_t)b * T_ + ki) * a.lddv + kvh * d;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j0 = 16 * c + g4;
      if (j0 >= d) continue;
      float v[4] = {dv[c][0], dv[c][1], dv[c][2], dv[c][3]};
      const Pk<T, 4> pk = pack4<T>(v);
      if (VEC) {
        *reinterpret_cast<Pk<T, 4>*>(dvb + j0) = pk;
      } else {
        for (int r = 0; r < 4 && j0 + r < d; ++r) dvb[j0 + r] = pk.e[r];
      }
    }
  }
  // dk~ -> LDS (reusing the tile space), rotate back, store.
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) dks[(wave * 16 + (lane & 15)) * FS + 16 * c + g4 + r] = dk[c][r] * scale;
  __syncthreads();
  T* dkb = static_cast<T*>(a.dk) + (int64_t)b * T_ * a.lddk + kvh * d;
  store_unrotated<T, VEC>(dks, FS, dkb, a.lddk, k0, T_, d, a.R, a.rope_mode, a.cs);
}

// The vector path needs every row group of 16 bytes (and the fragment groups
// of 4) to be aligned and the RoPE pairs not to straddle a group.
template <typename T>
bool vec_path_ok(const AttnArgs& a, bool bwd) {
  constexpr int G = kG<T>;
  auto al = [](const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (a.d % G) return false;
  if (a.R > 0 && (a.rope_mode == SLT_ROPE_HALF ? (a.R / 2) % G : a.R % G)) return false;
  for (int64_t ld : {a.ldq, a.ldk, a.ldv, a.ldo})
    if (ld % G) return false;
  if (!al(a.q) || !al(a.k) || !al(a.v) || !al(a.out) || !al(a.ores_out) || !al(a.cs)) return false;
  if (bwd) {
    for (int64_t ld : {a.lddo, a.lddq, a.lddk, a.lddv})
      if (ld % G) return false;
    if (!al(a.o) || !al(a.dout) || !al(a.dq) || !al(a.dk) || !al(a.dv) || !al(a.ores_in)) return false;
  }
  return true;
}

}  // namespace

int64_t attention_bwd_ws(int B, int H, int T) { return (int64_t)B * H * T * 4; }

template <typename T, bool VEC, bool DROP>
static slt_status attn_fwd_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.T + TQ - 1) / TQ, a.H, a.B);
  switch ((a.d + 15) / 16) {
    case 1: attn_fwd_k<T, 1, VEC, DROP><<<grid, 256, 0, s>>>(a); break;
    case 2: attn_fwd_k<T, 2, VEC, DROP><<<grid, 256, 0, s>>>(a); break;
    case 3: attn_fwd_k<T, 3, VEC, DROP><<<grid, 256, 0, s>>>(a); break;
    case 4: attn_fwd_k<T, 4, VEC, DROP><<<grid, 256, 0, s>>>(a); break;
    default: return fail(SLT_EUNSUPPORTED, "attention: head dim above 64");
  }
  return check_launch("attention_fwd");
}

template <typename T, bool VEC>
static slt_status attn_fwd_t(const AttnArgs& a, hipStream_t s) {
  return a.drop.on ? attn_fwd_t<T, VEC, true>(a, s) : attn_fwd_t<T, VEC, false>(a, s);
}

template <typename T, bool VEC, bool DROP>
static slt_status attn_bwd_t(const AttnArgs& a, hipStream_t s) {
  dim3 gq((a.T + TQ - 1) / TQ, a.H, a.B);
  dim3 gk((a.T + TQ - 1) / TQ, a.Hkv, a.B);
  switch ((a.d + 15) / 16) {
#define SLT_ATT_BWD(NCv)                                         \
  case NCv:                                                      \
    attn_bwd_dq_k<T, NCv, VEC, DROP><<<gq, 256, 0, s>>>(a);      \
    attn_bwd_dkdv_k<T, NCv, VEC, DROP><<<gk, 256, 0, s>>>(a);    \
    break;
    SLT_ATT_BWD(1) SLT_ATT_BWD(2) SLT_ATT_BWD(3) SLT_ATT_BWD(4)
#undef SLT_ATT_BWD
    default: return fail(SLT_EUNSUPPORTED, "attention: head dim above 64");
  }
  return check_launch("attention_bwd");
}

template <typename T, bool VEC>
static slt_status attn_bwd_t(const AttnArgs& a, hipStream_t s) {
  return a.drop.on ? attn_bwd_t<T, VEC, true>(a, s) : attn_bwd_t<T, VEC, false>(a, s);
}

slt_status launch_attention_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return SLT_OK;
  if (flash_ok(a, false)) return flash_fwd(a, s);
  if (a.qk_rotated) return fail(SLT_EUNSUPPORTED, "attention: pre-rotated q/k need the bf16 tiled kernels");
  if (a.dtype == SLT_BF16)
    return vec_path_ok<bf16>(a, false) ? attn_fwd_t<bf16, true>(a, s) : attn_fwd_t<bf16, false>(a, s);
  return vec_path_ok<float>(a, false) ? attn_fwd_t<float, true>(a, s) : attn_fwd_t<float, false>(a, s);
}

slt_status launch_attention_bwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return SLT_OK;
  if (flash_ok(a, true)) return flash_bwd(a, s);
  if (a.qk_rotated) return fail(SLT_EUNSUPPORTED, "attention: pre-rotated q/k need the bf16 tiled kernels");
  if (a.dtype == SLT_BF16)
    return vec_path_ok<bf16>(a, true) ? attn_bwd_t<bf16, true>(a, s) : attn_bwd_t<bf16, false>(a, s);
  return vec_path_ok<float>(a, true) ? attn_bwd_t<float, true>(a, s) : attn_bwd_t<float, false>(a, s);
}

}  // namespace slt
