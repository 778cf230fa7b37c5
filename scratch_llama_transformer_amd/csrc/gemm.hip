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
//  * XCD-aware tile order: workgroups are dispatched round-robin over the 8
//    XCDs, each with its own L2, so workgroup i is given tile
//    (i % 8) * (tiles / 8) + i / 8: every XCD works on a contiguous band of
//    output rows and reads each A row-block into its L2 once.
#include "slt_internal.h"

#include <algorithm>

// k-step depth as a multiple of one MFMA depth (32 bf16 / 16 fp32 elements)
#ifndef SLT_GEMM_BKX
#define SLT_GEMM_BKX 2
#endif
#ifndef SLT_GEMM_XCD
#define SLT_GEMM_XCD 1
#endif

namespace slt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, NT = 256;

template <typename T> struct Tr;
template <> struct Tr<bf16> { static constexpr int EPV = 8, BK = 32 * SLT_GEMM_BKX, KV = BK / 8; };
template <> struct Tr<float> { static constexpr int EPV = 4, BK = 16 * SLT_GEMM_BKX, KV = BK / 8; };

// MFMA depth steps per k-step; padded LDS row (one extra 16-byte group)
template <typename T> constexpr int kSub = Tr<T>::BK / (4 * Tr<T>::EPV);
template <typename T> constexpr int kStride = Tr<T>::BK + Tr<T>::EPV;

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
  static constexpr int VPR = Tr<T>::BK / EPV;      // 16-byte vectors per tile row
  static constexpr int NV = BM * VPR / NT;         // vectors per thread
  Pk<T, EPV> r[NV];
  template <bool VEC>
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows, int K, int row0, int k0, int tid) {
    if (VEC && row0 + BM <= rows && k0 + Tr<T>::BK <= K) {  // whole tile inside: no bounds checks
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int idx = tid + v * NT;
        r[v] = *reinterpret_cast<const Pk<T, EPV>*>(g + (int64_t)(row0 + idx / VPR) * ld + k0 + (idx % VPR) * EPV);
      }
      return;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * NT;
      const int row = row0 + idx / VPR;
      const int k = k0 + (idx % VPR) * EPV;
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
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * NT;
      *reinterpret_cast<Pk<T, EPV>*>(s + (idx / VPR) * kStride<T> + (idx % VPR) * EPV) = r[v];
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
    if (VEC && row0 + BM <= rows && k0 + Tr<T>::BK <= K) {  // whole tile inside: no bounds checks
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) r[kk] = *reinterpret_cast<const Pk<T, 4>*>(g + (int64_t)(kg + kk) * ld + mn);
      return;
    }
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
  int tiles_n, tiles;
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
  int tile = blockIdx.x;
  if (SLT_GEMM_XCD) {
    const int q = a.tiles >> 3, r = a.tiles & 7, x = tile & 7;
    tile = x * q + min(x, r) + (tile >> 3);
  }
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
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
#pragma unroll
    for (int ks = 0; ks < kSub<T>; ++ks) {
      uint4 af[4], bfr[4];
      const int ko = ks * 4 * EPV + (lane >> 4) * EPV;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(&As[cur][(wm * 64 + i * 16 + (lane & 15)) * STR + ko]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(&Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * STR + ko]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(bfr[j], af[i], acc[i][j], T{});
    }
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

// ---------------------------------------------------------------------------
// Direct-to-LDS variant for bf16 operands that are both k-major (C = A B^T):
// tiles are copied from HBM/L2 into LDS by global_load_lds_dwordx4 (lane i of
// an instruction lands at LDS base + 16 i), so no registers stage them; three
// LDS stages keep two k-steps of loads in flight while one is multiplied,
// which the register-staged kernel cannot afford without losing occupancy.
// LDS tile: 128 rows x 4 chunks of 16 bytes (32 bf16); the chunk position is
// XOR-swizzled with (row >> 2) & 3 so that the 16 rows one MFMA fragment read
// touches fall in distinct banks.  Rows past M (N) are read from the last
// valid row: they only feed output rows (columns) that are never stored.
// ---------------------------------------------------------------------------
constexpr int DL_BK = 32;
constexpr int DL_S = 3;
constexpr int DL_TILE = BM * DL_BK;  // elements per operand tile

__device__ __forceinline__ int dl_swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void dl_issue(const bf16* g, int64_t ld, int rows, int row0, int k0, bf16* tile, int wave,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = (wave * 2 + i) * 64 + lane;  // 16-byte chunk index in the tile
    const int r = p >> 2;
    const int lc = (p & 3) ^ dl_swz(r);
    const int row = min(row0 + r, rows - 1);
    const bf16* src = g + (int64_t)row * ld + k0 + lc * 8;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)(tile + (wave * 2 + i) * 512), 16,
                                     0, 0);
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// LDS byte offset of a pointer into a __shared__ array: the generic address
// is the LDS aperture (upper 32 bits) plus the offset.
__device__ __forceinline__ unsigned lds_off(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>(p));
}

// The 4 A and 4 B fragments of one k-step (rows 16 apart = 1 KiB apart).
// Written as one asm block that also waits for its own reads: the compiler
// cannot tell which LDS stage a global_load_lds copy targets and would
// otherwise wait for every copy in flight before any LDS read.
__device__ __forceinline__ void dl_read(unsigned a_addr, unsigned b_addr, u32x4 (&af)[4], u32x4 (&bf)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:1024\n\t"
      "ds_read_b128 %6, %9 offset:2048\n\t"
      "ds_read_b128 %7, %9 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]),
        "=&v"(bf[3])
      : "v"(a_addr), "v"(b_addr)
      : "memory");
}

// Workgroup barrier that orders LDS accesses only: global_load_lds writes
// are waited for explicitly (vmcnt) by each wave before it arrives.
__device__ __forceinline__ void dl_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One k-step: wait for this wave's part of tile `it`, barrier, read the
// current stage, refill the stage freed in step it-1 with tile it+2, multiply.
__device__ __forceinline__ void dl_step(const KArgs& a, const bf16* A, const bf16* B, int m0, int n0, int nk, int it,
                                        const bf16* As, const bf16* Bs, bf16* An, bf16* Bn, int wave, int lane,
                                        f32x4 (&acc)[4][4]) {
  __builtin_amdgcn_s_waitcnt(0xF74);  // vmcnt(4): only the 4 loads of tile it+1 may still fly
  dl_barrier();
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 15, fch = lane >> 4;
  // fragment i (j) of this wave starts 16 rows after fragment i-1, and the
  // swizzle depends on (row >> 2) & 3 only, so it is one address + 1 KiB steps
  const int ra = wm * 64 + frow, rb = wn * 64 + frow;
  u32x4 af[4], bfr[4];
  dl_read(lds_off(As) + (ra * 4 + (fch ^ dl_swz(ra))) * 16, lds_off(Bs) + (rb * 4 + (fch ^ dl_swz(rb))) * 16, af, bfr);
  // past the end the last tile is copied again into the free stage, which
  // keeps exactly 4 copies in flight per step; that stage is never read
  const int kn = min(it + 2, nk - 1) * DL_BK;
  dl_issue(A, a.lda, a.M, m0, kn, An, wave, lane);
  dl_issue(B, a.ldb, a.N, n0, kn, Bn, wave, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[j]),
                                                          __builtin_bit_cast(bf16x8_t, af[i]), acc[i][j], 0, 0, 0);
}

template <typename TO>
__global__ __launch_bounds__(NT) void gemm_dl_k(KArgs a) {
  // three stages as distinct LDS objects, so that reads of one stage need not
  // wait for copies still landing in another
  __shared__ __attribute__((aligned(16))) bf16 A0[DL_TILE], A1[DL_TILE], A2[DL_TILE];
  __shared__ __attribute__((aligned(16))) bf16 B0[DL_TILE], B1[DL_TILE], B2[DL_TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  int tile = blockIdx.x;
  if (SLT_GEMM_XCD) {
    const int q = a.tiles >> 3, r = a.tiles & 7, x = tile & 7;
    tile = x * q + min(x, r) + (tile >> 3);
  }
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = a.K / DL_BK;
  const bf16* A = static_cast<const bf16*>(a.A);
  const bf16* B = static_cast<const bf16*>(a.B);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  dl_issue(A, a.lda, a.M, m0, 0, A0, wave, lane);
  dl_issue(B, a.ldb, a.N, n0, 0, B0, wave, lane);
  dl_issue(A, a.lda, a.M, m0, min(1, nk - 1) * DL_BK, A1, wave, lane);
  dl_issue(B, a.ldb, a.N, n0, min(1, nk - 1) * DL_BK, B1, wave, lane);
  for (int it = 0; it < nk; it += 3) {
    dl_step(a, A, B, m0, n0, nk, it, A0, B0, A2, B2, wave, lane, acc);
    if (it + 1 < nk) dl_step(a, A, B, m0, n0, nk, it + 1, A1, B1, A0, B0, wave, lane, acc);
    if (it + 2 < nk) dl_step(a, A, B, m0, n0, nk, it + 2, A2, B2, A1, B1, wave, lane, acc);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): no copy may land after the block ends

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + i * 16 + (lane & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
      if (n >= a.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
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
  ka.tiles = tiles;

  // Vector loads need every vector wholly inside or outside the operand.
  auto op_ok = [&](const void* p, int64_t ld, bool kmajor, int rows) {
    if (kmajor) return g.K % EPV == 0 && ld % EPV == 0 && al(p, 16);
    return rows % 4 == 0 && ld % 4 == 0 && al(p, 4 * (int)sizeof(T));
  };
  const bool vec = op_ok(g.A, g.lda, g.a_kmajor, g.M) && op_ok(g.B, g.ldb, g.b_kmajor, g.N);

  // Direct-to-LDS path: bf16, both operands k-major, K a multiple of 32,
  // 16-byte aligned rows, and enough tiles to fill the chip without split-K.
  if constexpr (sizeof(T) == 2) {
    if (g.a_kmajor && g.b_kmajor && g.K > 0 && g.K % DL_BK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
        al(g.A, 16) && al(g.B, 16) && (tiles >= 256 || g.workspace == nullptr)) {
      ka.evec = g.N % 4 == 0 && g.ldc % 4 == 0 && al(g.C, 4 * (int)sizeof(TO)) &&
                (g.R == nullptr || (g.ldr % 4 == 0 && al(g.R, 4 * (int)sizeof(TO))));
      gemm_dl_k<TO><<<tiles, NT, 0, s>>>(ka);
      return check_launch("gemm");
    }
  }

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
