// Key/value-cache forward pieces: appending rotated keys and values to the
// cache, and attention of a few new queries over every cached position
// (randyGPT, "Features": prefill once, then one single-token forward per new
// token; Transformer in Rust, "CodeGen Inference Pipeline": each new token's
// keys and values are appended to the cache; strata, model table: the cache
// holds pre-rotated keys).
//
// Cache layout per layer: K then V, each [B, Hkv, Tmax, d] in the activation
// type, keys after RoPE at their absolute position.
//
// Attention over the cache (flash-decoding): a workgroup takes one sequence,
// one KV head, up to 8 of the query heads that share it, one query row and
// one chunk of cached positions.  Each of its 4 waves walks 64-key tiles:
// lane j scores key j against the heads (fp32 dot products, queries
// broadcast from LDS), the wave keeps an online softmax per head (max by a
// wave reduction, sums per lane), writes the probabilities to LDS and then
// accumulates P V with lanes spread over (key phase, 4-dim group) so that
// value rows are read as contiguous vectors.  Waves merge through LDS at the
// end; with several chunks per query, a second kernel merges the chunks'
// (max, sum, output) triples.  Work and traffic: every cached key and value
// row of the sequence's KV head is read once per group of 8 query heads.
#include "slt_internal.h"

namespace slt {
namespace {

constexpr int KT = 64;  // keys per wave tile
constexpr int DG = 8;   // query heads per workgroup
constexpr float kLog2e = 1.4426950408889634f;

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Rotated value of dim j of the head row u at table row t (cs: [*, R] with
// (cos, sin) of pair i at 2i, 2i+1); dims >= R pass through.
template <typename T>
__device__ __forceinline__ float rot_dim(const T* u, int j, const float* cst, int R, int mode) {
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
  const float c = cst[2 * i], s = cst[2 * i + 1], y = to_f32(u[p]);
  return first ? x * c - y * s : x * c + y * s;
}

// One workgroup per new token row (b, i) at position pos0 + i: rotated q to
// qrot (fp32 [rows, H d]), rotated k and v into the cache.
template <typename T>
__global__ __launch_bounds__(256) void kv_append_k(const T* qkv, int64_t ld, float* qrot, int Tq, int pos0, int H,
                                                   int Hkv, int d, int R, int mode, const float* cs, T* Kc, T* Vc,
                                                   int Tmax) {
  const int row = blockIdx.x;
  const int b = row / Tq, t = pos0 + row % Tq;
  const T* u = qkv + (int64_t)row * ld;
  const float* cst = cs + (int64_t)t * R;
  const int qd = H * d, kd = Hkv * d;
  for (int e = threadIdx.x; e < qd + 2 * kd; e += blockDim.x) {
    if (e < qd) {
      const int h = e / d;
      qrot[(int64_t)row * qd + e] = rot_dim(u + h * d, e - h * d, cst, R, mode);
    } else if (e < qd + kd) {
      const int g = (e - qd) / d, j = e - qd - g * d;
      Kc[(((int64_t)b * Hkv + g) * Tmax + t) * d + j] = from_f32<T>(rot_dim(u + qd + g * d, j, cst, R, mode));
    } else {
      const int g = (e - qd - kd) / d, j = e - qd - kd - g * d;
      Vc[(((int64_t)b * Hkv + g) * Tmax + t) * d + j] = u[e];
    }
  }
}

struct DecArgs {
  const float* q;      // rotated queries [B Tq, H d]
  const void* K;       // cache of this layer [B, Hkv, Tmax, d]
  const void* V;
  void* out;           // [B Tq, ldo], head h at column h d
  int64_t ldo;
  float* part;         // per (row, head, chunk): m, l, o[d]   (nsplit > 1)
  int Tq, pos0, Tmax, H, Hkv, d, G, ngh, nsplit, chunk, ncg_log2;
  float qscale;        // log2(e) / sqrt(d)
};

// Orders LDS writes and reads between the lanes of one wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* p, float (&x)[VEC]) {
  if constexpr (VEC == 4 && sizeof(T) == 2) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(r.x << 16);
    x[1] = __uint_as_float(r.x & 0xffff0000u);
    x[2] = __uint_as_float(r.y << 16);
    x[3] = __uint_as_float(r.y & 0xffff0000u);
  } else if constexpr (VEC == 4) {
    const float4 r = *reinterpret_cast<const float4*>(p);
    x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) x[v] = to_f32(p[v]);
  }
}

template <typename T, int VEC>
__global__ __launch_bounds__(256) void attn_decode_k(DecArgs a) {
  __shared__ float qs[DG][64];
  __shared__ float ps[4][DG][KT];
  __shared__ float wm[4][DG], wl[4][DG];
  __shared__ float wo[4][DG][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gh = blockIdx.x % a.ngh;
  const int bk = blockIdx.x / a.ngh;  // b * Hkv + kv head
  const int kvh = bk % a.Hkv, b = bk / a.Hkv;
  const int i = blockIdx.y, s = blockIdx.z;
  const int row = b * a.Tq + i;
  const int h0 = kvh * a.G + gh * DG;
  const int ng = min(DG, a.G - gh * DG);
  const int d = a.d;
  const int klo = s * a.chunk;
  const int khi = min(klo + a.chunk, a.pos0 + i + 1);

  for (int e = threadIdx.x; e < DG * 64; e += 256) {
    const int gg = e >> 6, c = e & 63;
    qs[gg][c] = (gg < ng && c < d) ? a.q[(int64_t)row * a.H * d + (int64_t)(h0 + gg) * d + c] * a.qscale : 0.f;
  }
  __syncthreads();

  const T* Kb = static_cast<const T*>(a.K) + (int64_t)bk * a.Tmax * d;
  const T* Vb = static_cast<const T*>(a.V) + (int64_t)bk * a.Tmax * d;
  const int ncg = 1 << a.ncg_log2;
  const int cq = lane & (ncg - 1), kq = lane >> a.ncg_log2, nkq = 64 >> a.ncg_log2;
  const int c0 = cq * VEC;

  float m[DG], l[DG], o[DG][VEC];
#pragma unroll
  for (int g = 0; g < DG; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[g][v] = 0.f;
  }

  for (int kb = klo + wave * KT; kb < khi; kb += 4 * KT) {
    // scores: lane j takes key kb + j
    const int key = kb + lane;
    const bool valid = key < khi;
    float sc[DG];
#pragma unroll
    for (int g = 0; g < DG; ++g) sc[g] = 0.f;
    if (valid) {
      const T* kr = Kb + (int64_t)key * d;
      for (int c = 0; c < d; c += VEC) {
        float kx[VEC];
        load_vec<T, VEC>(kr + c, kx);
#pragma unroll
        for (int g = 0; g < DG; ++g)
#pragma unroll
          for (int v = 0; v < VEC; ++v) sc[g] += qs[g][c + v] * kx[v];
      }
    }
    wave_sync();  // the previous tile's probabilities have been read
    float alpha[DG];
#pragma unroll
    for (int g = 0; g < DG; ++g) {
      const float mt = wave_max(valid ? sc[g] : -INFINITY);
      const float mn = fmaxf(m[g], mt);
      alpha[g] = exp2f(m[g] - mn);
      const float p = valid ? exp2f(sc[g] - mn) : 0.f;
      l[g] = l[g] * alpha[g] + p;
      m[g] = mn;
      ps[wave][g][lane] = p;
    }
    wave_sync();
    // P V: lane (kq, cq) takes keys kb + kq, kb + kq + nkq, ... and dims c0 .. c0 + VEC - 1
#pragma unroll
    for (int g = 0; g < DG; ++g)
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[g][v] *= alpha[g];
    if (c0 < d) {
      const int jend = min(KT, khi - kb);
      for (int j = kq; j < jend; j += nkq) {
        float vx[VEC];
        load_vec<T, VEC>(Vb + (int64_t)(kb + j) * d + c0, vx);
#pragma unroll
        for (int g = 0; g < DG; ++g) {
          const float p = ps[wave][g][j];
#pragma unroll
          for (int v = 0; v < VEC; ++v) o[g][v] += p * vx[v];
        }
      }
    }
  }

  // wave totals: sums over lanes, outputs over the key phases
#pragma unroll
  for (int g = 0; g < DG; ++g) {
    l[g] = wave_sum(l[g]);
    for (int off = ncg; off < 64; off <<= 1)
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[g][v] += __shfl_xor(o[g][v], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < DG; ++g) {
      wm[wave][g] = m[g];
      wl[wave][g] = l[g];
    }
  }
  if (kq == 0 && c0 < d) {
#pragma unroll
    for (int g = 0; g < DG; ++g)
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        if (c0 + v < d) wo[wave][g][c0 + v] = o[g][v];
  }
  __syncthreads();

  // merge the 4 waves: thread (g, c)
  for (int e = threadIdx.x; e < DG * 64; e += 256) {
    const int g = e >> 6, c = e & 63;
    if (g >= ng || c >= d) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(wm[w][g] - M);
        L += f * wl[w][g];
        O += f * wo[w][g][c];
      }
    }
    const int h = h0 + g;
    if (a.nsplit == 1) {
      static_cast<T*>(a.out)[(int64_t)row * a.ldo + (int64_t)h * d + c] = from_f32<T>(O / L);
    } else {
      float* pp = a.part + (((int64_t)row * a.H + h) * a.nsplit + s) * (d + 2);
      if (c == 0) {
        pp[0] = M;
        pp[1] = L;
      }
      pp[2 + c] = O;
    }
  }
}

// Merge the chunks of one (row, head): thread c of a 64-thread workgroup.
template <typename T>
__global__ __launch_bounds__(64) void attn_decode_merge_k(DecArgs a) {
  const int rh = blockIdx.x;  // row * H + h
  const int c = threadIdx.x;
  if (c >= a.d) return;
  const float* pp = a.part + (int64_t)rh * a.nsplit * (a.d + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pp[s * (a.d + 2)]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = pp[s * (a.d + 2)];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - M);
    L += f * pp[s * (a.d + 2) + 1];
    O += f * pp[s * (a.d + 2) + 2 + c];
  }
  const int row = rh / a.H, h = rh % a.H;
  static_cast<T*>(a.out)[(int64_t)row * a.ldo + (int64_t)h * a.d + c] = from_f32<T>(O / L);
}

int decode_splits(int B, int Hkv, int G, int Tq, int Lmax) {
  const int64_t base = (int64_t)B * Hkv * cdiv(G, DG) * Tq;
  const int most = cdiv(Lmax, 4 * KT);
  const int want = (int)std::max<int64_t>(1, (1024 + base - 1) / base);
  return std::max(1, std::min(most, want));
}

}  // namespace

// Partials of every (row, head, chunk): with base = B Hkv ceil(G/8) Tq
// workgroups per chunk, chunks <= ceil(1024 / base), so rows x heads x chunks
// <= H (B Tq + 1024 / (Hkv ceil(G/8))): a bound that grows with B and Tq, so
// a workspace sized for some (B, Tq) serves every smaller call.
int64_t decode_attention_ws(int B, int Tq, int H, int Hkv, int d, int Tmax) {
  if (Tmax <= 4 * KT) return 0;  // one chunk
  const int64_t per = (int64_t)cdiv(1024, (int64_t)Hkv * cdiv(H / Hkv, DG));
  return ((int64_t)B * Tq + per) * H * (d + 2) * 4;
}

slt_status launch_kv_append(const void* qkv, int64_t ld, float* qrot, int B, int Tq, int pos0, int H, int Hkv, int d,
                            int R, int mode, const float* cs, void* Kc, void* Vc, int Tmax, int dtype,
                            hipStream_t s) {
  if (B == 0 || Tq == 0) return SLT_OK;
  if (dtype == SLT_BF16)
    kv_append_k<bf16><<<B * Tq, 256, 0, s>>>(static_cast<const bf16*>(qkv), ld, qrot, Tq, pos0, H, Hkv, d, R, mode, cs,
                                             static_cast<bf16*>(Kc), static_cast<bf16*>(Vc), Tmax);
  else
    kv_append_k<float><<<B * Tq, 256, 0, s>>>(static_cast<const float*>(qkv), ld, qrot, Tq, pos0, H, Hkv, d, R, mode,
                                              cs, static_cast<float*>(Kc), static_cast<float*>(Vc), Tmax);
  return check_launch("kv_append");
}

slt_status launch_attention_decode(const float* qrot, const void* Kc, const void* Vc, void* out, int64_t ldo, int B,
                                   int Tq, int pos0, int H, int Hkv, int d, int Tmax, int dtype, float* ws,
                                   hipStream_t s) {
  if (B == 0 || Tq == 0) return SLT_OK;
  if (d > 64 || H % Hkv) return fail(SLT_EUNSUPPORTED, "decode attention: head dimension above 64 or H % Hkv != 0");
  DecArgs a{};
  a.q = qrot; a.K = Kc; a.V = Vc; a.out = out; a.ldo = ldo; a.part = ws;
  a.Tq = Tq; a.pos0 = pos0; a.Tmax = Tmax; a.H = H; a.Hkv = Hkv; a.d = d;
  a.G = H / Hkv;
  a.ngh = cdiv(a.G, DG);
  const int Lmax = pos0 + Tq;
  a.nsplit = decode_splits(B, Hkv, a.G, Tq, Lmax);
  a.chunk = cdiv(cdiv(Lmax, a.nsplit), KT) * KT;
  a.nsplit = cdiv(Lmax, a.chunk);
  if (a.nsplit > 1 && !ws) return fail(SLT_EINVAL, "decode attention: workspace required");
  a.qscale = kLog2e / sqrtf((float)d);
  const bool v4 = d % 4 == 0;
  const int ncg = v4 ? cdiv(d, 4) : d;
  int lg = 0;
  while ((1 << lg) < ncg) ++lg;
  a.ncg_log2 = lg;
  const dim3 grid(B * Hkv * a.ngh, Tq, a.nsplit);
  if (dtype == SLT_BF16) {
    if (v4) attn_decode_k<bf16, 4><<<grid, 256, 0, s>>>(a);
    else attn_decode_k<bf16, 1><<<grid, 256, 0, s>>>(a);
    if (a.nsplit > 1) attn_decode_merge_k<bf16><<<B * Tq * H, 64, 0, s>>>(a);
  } else {
    if (v4) attn_decode_k<float, 4><<<grid, 256, 0, s>>>(a);
    else attn_decode_k<float, 1><<<grid, 256, 0, s>>>(a);
    if (a.nsplit > 1) attn_decode_merge_k<float><<<B * Tq * H, 64, 0, s>>>(a);
  }
  return check_launch("attention over the cache");
}

}  // namespace slt
