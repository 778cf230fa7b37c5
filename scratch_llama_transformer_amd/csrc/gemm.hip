// MFMA GEMM for the three forms of the matmul family (strata, "A.B, A.B^T,
// A^T.B"): C[m, n] = sum_k A(m, k) B(n, k) (+ R), each operand either
// k-contiguous ("k-major") or m/n-contiguous in memory.
//
// Design (gfx950, 64-wide wavefronts):
//  * 256 threads = 4 waves per workgroup, 128 x 128 output tile, each wave a
//    64 x 64 quadrant made of 4 x 4 MFMA 16x16 tiles.
//  * bf16 operands: v_mfma_f32_16x16x32_bf16, k-step 32; fp32 operands:
//    v_mfma_f32_16x16x4_f32 four times per k-step of 16.  In both cases one
//    lane's operand fragment is 16 contiguous bytes of a k-contiguous LDS row,
//    so LDS tiles are always stored k-contiguous: a k-major operand is copied
//    as is, an m/n-major one is transposed on its way from registers to LDS
//    (each thread loads 4 m/n x KV k values and stores 4 rows of KV k values).
//  * The MFMA is issued with the operands swapped (B tile as "A"), so each
//    lane ends up holding 4 consecutive output columns of one row and the
//    epilogue stores 8 or 16 bytes per lane.
//  * Two LDS buffers: global loads of tile k+1 are in flight while tile k is
//    multiplied; one barrier per k-step.
//  * Split-K for small output grids (the weight gradients, whose K is the
//    token count): partial tiles go to a fp32 workspace and a second kernel
//    adds them in split order, so the result is deterministic.
#include "slt_internal.h"

#include <algorithm>

namespace slt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, NT = 256;

template <typename T> struct Tr;
template <> struct Tr<bf16> { static constexpr int BK = 32, EPV = 8, KV = 4; };
template <> struct Tr<float> { static constexpr int BK = 16, EPV = 4, KV = 2; };

template <typename T> constexpr int kStride = Tr<T>::BK + Tr<T>::EPV;  // padded LDS row (80 bytes)

template <typename T, int N>
struct alignas(sizeof(T) * N) Pk {
  T e[N];
};

__device__ __forceinline__ f32x4 mfma(const uint4& a, const uint4& b, f32x4 c, bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma(const uint4& a, const uint4& b, f32x4 c, float) {
  // lane l supplies k = 4*(l/16) + i at step i for both operands
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

template <typename T> __device__ __forceinline__ T zero_v();
template <> __device__ __forceinline__ bf16 zero_v<bf16>() { return bf16{0}; }
template <> __device__ __forceinline__ float zero_v<float>() { return 0.f; }

// Register staging for one operand tile (128 rows x BK).
template <typename T, bool KMAJOR> struct Stage;

template <typename T> struct Stage<T, true> {
  static constexpr int EPV = Tr<T>::EPV;
  Pk<T, EPV> r[2];
  template <bool VEC>
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows, int K, int row0, int k0, int tid) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = tid + v * NT;
      const int row = row0 + (idx >> 2);
      const int k = k0 + (idx & 3) * EPV;
      if (VEC) {
        if (row < rows && k < K) {
          r[v] = *reinterpret_cast<const Pk<T, EPV>*>(g + (int64_t)row * ld + k);
        } else {
#pragma unroll
          for (int e = 0; e < EPV; ++e) r[v].e[e] = zero_v<T>();
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e)
          r[v].e[e] = (row < rows && k + e < K) ? g[(int64_t)row * ld + k + e] : zero_v<T>();
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = tid + v * NT;
      *reinterpret_cast<Pk<T, EPV>*>(s + (idx >> 2) * kStride<T> + (idx & 3) * EPV) = r[v];
    }
  }
};

template <typename T> struct Stage<T, false> {
  static constexpr int KV = Tr<T>::KV;
  Pk<T, 4> r[KV];  // r[kk] = 4 consecutive m/n values at k = kg + kk
  template <bool VEC>
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows, int K, int row0, int k0, int tid) {
    const int mn = row0 + 4 * (tid >> 3);
    const int kg = k0 + (tid & 7) * KV;
#pragma unroll
    for (int kk = 0; kk < KV; ++kk) {
      const int k = kg + kk;
      if (VEC) {
        if (k < K && mn < rows) {
          r[kk] = *reinterpret_cast<const Pk<T, 4>*>(g + (int64_t)k * ld + mn);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) r[kk].e[e] = zero_v<T>();
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[kk].e[e] = (k < K && mn + e < rows) ? g[(int64_t)k * ld + mn + e] : zero_v<T>();
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
    const int mn = 4 * (tid >> 3);
    const int kg = (tid & 7) * KV;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Pk<T, KV> p;
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) p.e[kk] = r[kk].e[e];
      *reinterpret_cast<Pk<T, KV>*>(s + (mn + e) * kStride<T> + kg) = p;
    }
  }
};

struct KArgs {
  int M, N, K;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  void* C; int64_t ldc;
  const void* R; int64_t ldr;
  float* ws;          // split-K partials [splits][M][N]
  int kchunk;         // k range per split (multiple of BK)
  int tiles_n;
  bool evec;          // 4-wide epilogue stores allowed
};

template <typename TO>
__device__ __forceinline__ void store4(TO* p, const float (&v)[4]) {
  Pk<TO, 4> pk;
#pragma unroll
  for (int r = 0; r < 4; ++r) pk.e[r] = from_f32<TO>(v[r]);
  *reinterpret_cast<Pk<TO, 4>*>(p) = pk;
}

template <typename TO>
__device__ __forceinline__ void load4(const TO* p, float (&v)[4]) {
  Pk<TO, 4> pk = *reinterpret_cast<const Pk<TO, 4>*>(p);
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = to_f32(pk.e[r]);
}

template <typename T, typename TO, bool AK, bool BKM, bool VEC, bool SPLIT>
__global__ __launch_bounds__(NT) void gemm_k(KArgs a) {
  constexpr int BK = Tr<T>::BK, EPV = Tr<T>::EPV, STR = kStride<T>;
  __shared__ __attribute__((aligned(16))) T As[2][BM * STR];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * STR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = blockIdx.x / a.tiles_n, tn = blockIdx.x % a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = SPLIT ? blockIdx.z * a.kchunk : 0;
  const int kend = SPLIT ? min(a.K, kbeg + a.kchunk) : a.K;
  const int nk = (kend - kbeg + BK - 1) / BK;

  const T* A = static_cast<const T*>(a.A);
  const T* B = static_cast<const T*>(a.B);
  Stage<T, AK> sa;
  Stage<T, BKM> sb;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    sa.template load<VEC>(A, a.lda, a.M, a.K, m0, kbeg, tid);
    sb.template load<VEC>(B, a.ldb, a.N, a.K, n0, kbeg, tid);
    sa.store(As[0], tid);
    sb.store(Bs[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      const int k = kbeg + (it + 1) * BK;
      sa.template load<VEC>(A, a.lda, a.M, a.K, m0, k, tid);
      sb.template load<VEC>(B, a.ldb, a.N, a.K, n0, k, tid);
    }
    uint4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const uint4*>(&As[cur][(wm * 64 + i * 16 + (lane & 15)) * STR + (lane >> 4) * EPV]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = *reinterpret_cast<const uint4*>(&Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * STR + (lane >> 4) * EPV]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma(bfr[j], af[i], acc[i][j], T{});
    if (more) {
      sa.store(As[cur ^ 1], tid);
      sb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue: lane holds C[m][n .. n+3].
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + i * 16 + (lane & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
      if (n >= a.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (SPLIT) {
        float* dst = a.ws + ((int64_t)blockIdx.z * a.M + m) * a.N + n;
        if (a.evec && n + 3 < a.N) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int r = 0; r < 4 && n + r < a.N; ++r) dst[r] = v[r];
        }
      } else {
        TO* dst = static_cast<TO*>(a.C) + (int64_t)m * a.ldc + n;
        const TO* res = a.R ? static_cast<const TO*>(a.R) + (int64_t)m * a.ldr + n : nullptr;
        if (a.evec && n + 3 < a.N) {
          if (res) {
            float rv[4];
            load4<TO>(res, rv);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += rv[r];
          }
          store4<TO>(dst, v);
        } else {
          for (int r = 0; r < 4 && n + r < a.N; ++r) {
            float x = v[r];
            if (res) x += to_f32(res[r]);
            dst[r] = from_f32<TO>(x);
          }
        }
      }
    }
  }
}

// out[m, n] = sum_z ws[z][m][n] (+ R[m, n]), z in increasing order.
template <typename TO>
__global__ __launch_bounds__(256) void splitk_reduce_k(const float* __restrict__ ws, int splits, int M, int N,
                                                       TO* C, int64_t ldc, const TO* R, int64_t ldr) {
  const int64_t total = (int64_t)M * N;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / N, n = idx % N;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += ws[(int64_t)z * total + idx];
    if (R) s += to_f32(R[m * ldr + n]);
    C[m * ldc + n] = from_f32<TO>(s);
  }
}

inline bool al(const void* p, int b) { return (reinterpret_cast<uintptr_t>(p) % b) == 0; }

template <typename T, typename TO, bool AK, bool BKM, bool VEC, bool SPLIT>
void launch_one(const KArgs& ka, dim3 grid, hipStream_t s) {
  gemm_k<T, TO, AK, BKM, VEC, SPLIT><<<grid, NT, 0, s>>>(ka);
}

template <typename T, typename TO>
slt_status run(const GemmArgs& g, hipStream_t s) {
  constexpr int BK = Tr<T>::BK, EPV = Tr<T>::EPV;
  KArgs ka{};
  ka.M = g.M; ka.N = g.N; ka.K = g.K;
  ka.A = g.A; ka.lda = g.lda; ka.B = g.B; ka.ldb = g.ldb;
  ka.C = g.C; ka.ldc = g.ldc; ka.R = g.R; ka.ldr = g.ldr;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  ka.tiles_n = tiles_n;
  const int tiles = tiles_m * tiles_n;

  // Vector loads need every vector wholly inside or outside the operand.
  auto op_ok = [&](const void* p, int64_t ld, bool kmajor, int rows) {
    if (kmajor) return g.K % EPV == 0 && ld % EPV == 0 && al(p, 16);
    return rows % 4 == 0 && ld % 4 == 0 && al(p, 4 * (int)sizeof(T));
  };
  const bool vec = op_ok(g.A, g.lda, g.a_kmajor, g.M) && op_ok(g.B, g.ldb, g.b_kmajor, g.N);

  // Split K when the output grid cannot fill the 256 compute units and K is
  // long; the partials must fit the workspace.
  int splits = 1;
  if (g.workspace && tiles < 256) {
    const int kt = (g.K + BK - 1) / BK;
    int want = std::min((512 + tiles - 1) / tiles, kt / 8);
    const int64_t per = (int64_t)g.M * g.N * 4;
    while (want > 1 && per * want > g.workspace_bytes) --want;
    splits = std::max(1, want);
  }
  bool split = splits > 1;
  if (split) {
    const int kt = (g.K + BK - 1) / BK;
    const int chunk_t = (kt + splits - 1) / splits;
    ka.kchunk = chunk_t * BK;
    splits = (g.K + ka.kchunk - 1) / ka.kchunk;
    ka.ws = g.workspace;
    ka.evec = g.N % 4 == 0 && al(g.workspace, 16);
  } else {
    ka.kchunk = g.K;
    ka.evec = g.N % 4 == 0 && g.ldc % 4 == 0 && al(g.C, 4 * (int)sizeof(TO)) &&
              (g.R == nullptr || (g.ldr % 4 == 0 && al(g.R, 4 * (int)sizeof(TO))));
  }
  dim3 grid(tiles, 1, split ? splits : 1);

#define SLT_GEMM_GO(AKv, BKv)                                                     \
  do {                                                                            \
    if (split) {                                                                  \
      if (vec) launch_one<T, float, AKv, BKv, true, true>(ka, grid, s);           \
      else launch_one<T, float, AKv, BKv, false, true>(ka, grid, s);              \
    } else {                                                                      \
      if (vec) launch_one<T, TO, AKv, BKv, true, false>(ka, grid, s);             \
      else launch_one<T, TO, AKv, BKv, false, false>(ka, grid, s);                \
    }                                                                             \
  } while (0)

  if (g.a_kmajor && g.b_kmajor) SLT_GEMM_GO(true, true);
  else if (g.a_kmajor) SLT_GEMM_GO(true, false);
  else if (g.b_kmajor) SLT_GEMM_GO(false, true);
  else SLT_GEMM_GO(false, false);
#undef SLT_GEMM_GO

  if (split) {
    const int64_t total = (int64_t)g.M * g.N;
    int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
    splitk_reduce_k<TO><<<blocks, 256, 0, s>>>(g.workspace, splits, g.M, g.N, static_cast<TO*>(g.C), g.ldc,
                                               static_cast<const TO*>(g.R), g.ldr);
  }
  return check_launch("gemm");
}

}  // namespace

slt_status launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return SLT_OK;
  if (g.in_dtype == SLT_BF16) {
    return g.out_dtype == SLT_BF16 ? run<bf16, bf16>(g, s) : run<bf16, float>(g, s);
  }
  if (g.out_dtype == SLT_BF16) return fail(SLT_EUNSUPPORTED, "gemm: fp32 inputs with bf16 output");
  return run<float, float>(g, s);
}

}  // namespace slt
