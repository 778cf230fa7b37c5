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
#ifndef SLT_SPLIT_TARGET
#define SLT_SPLIT_TARGET 384  // blocks a split-K grid aims for
#endif
#ifndef SLT_GROUP_TARGET
#define SLT_GROUP_TARGET 512  // blocks a grouped weight-gradient grid aims for
#endif
#ifndef SLT_GROUP_W8_MIN
#define SLT_GROUP_W8_MIN 160  // fewest 256 x 256 tiles for the 8-wave grouped kernel
#endif
#ifndef SLT_SPLIT_MINK
#define SLT_SPLIT_MINK 8  // fewest k-steps per split
#endif
#ifndef SLT_GEMM_D64
#define SLT_GEMM_D64 1  // 64-deep two-stage kernel for k-major x k-major 128 x 128 tiles
#endif
#ifndef SLT_GEMM_BIG
#define SLT_GEMM_BIG 1
#endif
#ifndef SLT_GEMM_W8
#define SLT_GEMM_W8 1
#endif
#ifndef SLT_W8_MIN
#define SLT_W8_MIN 256  // fewest 256 x 256 tiles for the 8-wave kernel
#endif
#ifndef SLT_NT_STORE
#define SLT_NT_STORE 1  // non-temporal output stores in the 256 x 256 kernel's staged epilogues
#endif
#ifndef SLT_FUSED_SWIGLU
#define SLT_FUSED_SWIGLU 1  // SwiGLU in the epilogue of the 256 x 256 kernel
#endif
#ifndef SLT_GEMM_BAND
#define SLT_GEMM_BAND 8  // tile rows per band of the 256 x 256 tile order
#endif
#ifndef SLT_GEMM_XCD
#define SLT_GEMM_XCD 1
#endif
#ifndef SLT_ROPE_PRELOAD
#define SLT_ROPE_PRELOAD 1  // the 64-deep kernel loads its RoPE table entries before the k-loop
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

// Load width of the register-staged copies: whole 16-byte groups (k-major) or
// 4-wide m/n groups, element pairs (for an odd number of pairs along the
// vector dimension, e.g. an MLP width of 682), or single elements.
constexpr int kVecFull = 2, kVecPair = 1, kVecOne = 0;

template <typename T, int N>
__device__ __forceinline__ void ld_group(const T* g, bool ok, T* out) {
  Pk<T, N> x;
  if (ok) {
    x = *reinterpret_cast<const Pk<T, N>*>(g);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) x.e[e] = zero_v<T>();
  }
#pragma unroll
  for (int e = 0; e < N; ++e) out[e] = x.e[e];
}

template <typename T> struct Stage<T, true> {
  static constexpr int EPV = Tr<T>::EPV;
  static constexpr int VPR = Tr<T>::BK / EPV;      // 16-byte vectors per tile row
  static constexpr int NV = BM * VPR / NT;         // vectors per thread
  Pk<T, EPV> r[NV];
  template <int VL>
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows, int K, int row0, int k0, int tid) {
    const bool inside = row0 + BM <= rows && k0 + Tr<T>::BK <= K;  // whole tile inside: no bounds checks
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * NT;
      const int row = row0 + idx / VPR;
      const int k = k0 + (idx % VPR) * EPV;
      const T* src = g + (int64_t)row * ld + k;
      if constexpr (VL == kVecFull) {
        ld_group<T, EPV>(src, inside || (row < rows && k < K), r[v].e);
      } else {
        constexpr int W = VL == kVecPair ? 2 : 1;  // K a multiple of W: a group is wholly in or out
#pragma unroll
        for (int e = 0; e < EPV; e += W) ld_group<T, W>(src + e, inside || (row < rows && k + e < K), r[v].e + e);
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
  template <int VL>
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows, int K, int row0, int k0, int tid) {
    const int mn = row0 + 4 * (tid >> 3);
    const int kg = k0 + (tid & 7) * KV;
    const bool inside = row0 + BM <= rows && k0 + Tr<T>::BK <= K;  // whole tile inside: no bounds checks
#pragma unroll
    for (int kk = 0; kk < KV; ++kk) {
      const int k = kg + kk;
      const T* src = g + (int64_t)k * ld + mn;
      if constexpr (VL == kVecFull) {
        ld_group<T, 4>(src, inside || (k < K && mn < rows), r[kk].e);
      } else {
        constexpr int W = VL == kVecPair ? 2 : 1;  // rows a multiple of W: a group is wholly in or out
#pragma unroll
        for (int e = 0; e < 4; e += W) ld_group<T, W>(src + e, inside || (k < K && mn + e < rows), r[kk].e + e);
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
  float alpha;        // C = alpha A B (+ R)
  void* C2;           // fused SwiGLU epilogues: h (forward)
  int64_t ldc2;
  int F;              // fused SwiGLU epilogues: MLP width (b at column F + f)
  Drop drop;          // C = drop(alpha A B) + R, element (m, n) = e m N + n
  RopeEpi rope;       // RoPE epilogue (kernels instantiated with it only)
};

// B-operand row (output column) whose weights a tile column holds under the
// RoPE epilogue: for rotate-half pairs (j, j + R/2) of a head, tile columns
// 2i and 2i + 1 hold output dims i and i + R/2, so that each pair lands in
// one lane's four consecutive accumulator columns; other columns map to
// themselves (the even-odd pairing is already adjacent).
__device__ __forceinline__ int rope_row(const RopeEpi& r, int n) {
  if (!r.half || n >= r.end) return n;
  const int c = n % r.d;
  if (c >= r.R) return n;
  return n - c + ((c & 1) ? (r.R >> 1) + (c >> 1) : (c >> 1));
}

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

template <typename T, typename TO, bool AK, bool BKM, int VL, bool SPLIT>
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
    sa.template load<VL>(A, a.lda, a.M, a.K, m0, kbeg, tid);
    sb.template load<VL>(B, a.ldb, a.N, a.K, n0, kbeg, tid);
    sa.store(As[0], tid);
    sb.store(Bs[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      const int k = kbeg + (it + 1) * BK;
      sa.template load<VL>(A, a.lda, a.M, a.K, m0, k, tid);
      sb.template load<VL>(B, a.ldb, a.N, a.K, n0, k, tid);
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
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] *= a.alpha;
        if (a.drop.on) {
          float dm[4];
          drop_mults<4>(a.drop, (uint64_t)m * a.N + n, dm);
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] *= dm[r];
        }
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
                                                       TO* C, int64_t ldc, const TO* R, int64_t ldr, float alpha) {
  const int64_t total = (int64_t)M * N;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / N, n = idx % N;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += ws[(int64_t)z * total + idx];
    s *= alpha;
    if (R) s += to_f32(R[m * ldr + n]);
    C[m * ldc + n] = from_f32<TO>(s);
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel for bf16 operands in any layout.  Operand tiles are
// copied HBM/L2 -> LDS by global_load_lds_dwordx4 (lane i of an instruction
// lands at LDS base + 16 i, so the LDS layout is fixed by which global chunk
// each lane fetches); no registers stage them, and three LDS stages keep two
// k-steps of copies in flight while one is multiplied.
//
// k-major operand (rows of K contiguous): LDS tile of 128 rows x 4 chunks of
// 16 bytes (32 k), chunk position XOR (row >> 2) & 3; a fragment is one
// ds_read_b128 per lane (row l%16, k 8(l/16)..+7).
// m/n-major operand (rows of M or N contiguous): LDS tile of 32 k-rows x 16
// chunks (8 m each), chunk position XOR f(k-row); a fragment is two
// ds_read_b64_tr_b16.  That instruction hands lane 16g+i element j of the
// 8-byte row supplied by lane 16g+4j+i/4, at position i%4; so lane 16g+4j+q
// supplies (k = 8g+j, m = 4q..4q+3) and receives k = 8g..8g+3 at its own m,
// the MFMA operand layout (the second read covers k + 4).  The rows one read
// touches are k = 8g+j (+4); f spreads the chunk pairs of those rows over the
// banks.
// Rows (columns) past M (N) are read from a valid row: they only feed outputs
// that are never stored.
// ---------------------------------------------------------------------------
constexpr int DL_BK = 32;
constexpr int DL_TILE = BM * DL_BK;  // elements per operand tile (8 KiB)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// k-major tile: chunk position XOR (r >> 1) & 3.  A fragment read takes rows
// r0..r0+15 (r0 a multiple of 16) at one logical chunk per 16-lane group;
// measured with the SQ_LDS_BANK_CONFLICT counter on gfx950, this swizzle
// reads them conflict-free where (r >> 2) & 3 costs 4 extra cycles per read.
__device__ __forceinline__ int dl_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int dl_swz_mn(int kr) { return 2 * ((kr & 3) | (((kr >> 3) & 1) << 2)); }


// Tile coordinates of list position `idx` in bands of G tile rows, each band
// walked column by column: the tiles an XCD runs together (a contiguous range
// of positions) then share both A row-blocks and B column-blocks in its L2,
// where a row-major walk shares only A and streams B from memory.
__device__ __forceinline__ void band_coords(int idx, int tiles, int tiles_n, int G, int& tm, int& tn) {
  const int tiles_m = tiles / tiles_n;
  const int band = idx / (G * tiles_n), within = idx - band * G * tiles_n;
  const int gm = min(G, tiles_m - band * G);
  tm = band * G + within % gm;
  tn = within / gm;
}

// Copy the 128 x 32 tile at (row0, k0) of an operand into `tile`: 2 copies per
// wave (512 chunks of 16 bytes over 4 waves).
template <bool KM, bool MAP = false>
__device__ __forceinline__ void dl_issue(const bf16* g, int64_t ld, int rows, int row0, int k0, bf16* tile, int wave,
                                         int lane, const int* rmap = nullptr) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = (wave * 2 + i) * 64 + lane;  // 16-byte chunk position in the tile
    const bf16* src;
    if constexpr (KM) {
      const int r = p >> 2;
      const int lc = (p & 3) ^ dl_swz(r);
      const int row = MAP ? rmap[i] : min(row0 + r, rows - 1);
      src = g + (int64_t)row * ld + k0 + lc * 8;
    } else {
      const int kr = p >> 4;
      const int c = (p & 15) ^ dl_swz_mn(kr);
      src = g + (int64_t)(k0 + kr) * ld + min(row0 + c * 8, rows - 8);
    }
    lds_copy16(src, tile + (wave * 2 + i) * 512);
  }
}

// Per-lane LDS byte addresses of a wave's F fragments (16 rows or columns
// each) starting at row w0 of an operand tile made of 128-row sub-tiles
// (8 KiB each): k-major: one address, fragments 1 KiB apart; m/n-major: one
// address per fragment, the second read of each at +1 KiB (4 k-rows of 256
// bytes further).  w0 is a multiple of 16 F, so the fragments stay inside
// one sub-tile.
template <bool KM, int F> struct DlAddr;
template <int F> struct DlAddr<true, F> {
  unsigned a;
  __device__ __forceinline__ DlAddr(int w0, int lane) {
    const int i = lane & 15;
    a = (w0 >> 7) * 8192 + ((w0 & 127) + i) * 64 + ((lane >> 4) ^ dl_swz(i)) * 16;
  }
  __device__ __forceinline__ DlAddr at(unsigned base) const {
    DlAddr x = *this;
    x.a += base;
    return x;
  }
};
template <int F> struct DlAddr<false, F> {
  unsigned a[F];
  __device__ __forceinline__ DlAddr(int w0, int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
    const int kr = 8 * g + j;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int c = ((w0 & 127) + 16 * f) / 8 + (q >> 1);
      a[f] = (w0 >> 7) * 8192 + (kr * 16 + (c ^ dl_swz_mn(kr))) * 16 + (q & 1) * 8;
    }
  }
  __device__ __forceinline__ DlAddr at(unsigned base) const {
    DlAddr x = *this;
#pragma unroll
    for (int f = 0; f < F; ++f) x.a[f] += base;
    return x;
  }
};

#define DL_R128(X, f, off) "ds_read_b128 %[" #X #f "], %[" #X "p] offset:" #off "\n\t"
#define DL_KM4(X) DL_R128(X, 0, 0) DL_R128(X, 1, 1024) DL_R128(X, 2, 2048) DL_R128(X, 3, 3072)
#define DL_KM8(X) DL_KM4(X) DL_R128(X, 4, 4096) DL_R128(X, 5, 5120) DL_R128(X, 6, 6144) DL_R128(X, 7, 7168)
#define DL_RTR(X, f)                                                  \
  "ds_read_b64_tr_b16 %[" #X #f "l], %[" #X "p" #f "]\n\t"            \
  "ds_read_b64_tr_b16 %[" #X #f "h], %[" #X "p" #f "] offset:1024\n\t"
#define DL_MN4(X) DL_RTR(X, 0) DL_RTR(X, 1) DL_RTR(X, 2) DL_RTR(X, 3)
#define DL_OKM(X, f, v) [X##f] "=&v"(v[f])
#define DL_OUT_KM4(X, v) DL_OKM(X, 0, v), DL_OKM(X, 1, v), DL_OKM(X, 2, v), DL_OKM(X, 3, v)
#define DL_OUT_KM8(X, v) DL_OUT_KM4(X, v), DL_OKM(X, 4, v), DL_OKM(X, 5, v), DL_OKM(X, 6, v), DL_OKM(X, 7, v)
#define DL_OMN(X, f, lo, hi) [X##f##l] "=&v"(lo[f]), [X##f##h] "=&v"(hi[f])
#define DL_OUT_MN4(X, lo, hi) DL_OMN(X, 0, lo, hi), DL_OMN(X, 1, lo, hi), DL_OMN(X, 2, lo, hi), DL_OMN(X, 3, lo, hi)
#define DL_IN_KM(X, d) [X##p] "v"(d.a)
#define DL_IN_MN4(X, d) [X##p0] "v"(d.a[0]), [X##p1] "v"(d.a[1]), [X##p2] "v"(d.a[2]), [X##p3] "v"(d.a[3])

// The A and B fragments of one k-step, as one asm block that also waits for
// its own reads: the compiler cannot tell which LDS stage a global_load_lds
// copy targets and would otherwise wait for every copy in flight before any
// LDS read.  Supported shapes: 4 fragments per side, and 8 on the side of a
// k-major operand whose partner has 4.
template <bool AK, bool BK, int FA, int FB>
__device__ __forceinline__ void dl_read(const DlAddr<AK, FA>& da, const DlAddr<BK, FB>& db, u32x4 (&af)[FA],
                                        u32x4 (&bf)[FB]) {
  u32x2 al[FA], ah[FA], bl[FB], bh[FB];
  if constexpr (AK && BK && FA == 4 && FB == 4) {
    asm volatile(DL_KM4(a) DL_KM4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_KM4(a, af), DL_OUT_KM4(b, bf) : DL_IN_KM(a, da), DL_IN_KM(b, db) : "memory");
  } else if constexpr (AK && BK && FA == 8 && FB == 4) {
    asm volatile(DL_KM8(a) DL_KM4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_KM8(a, af), DL_OUT_KM4(b, bf) : DL_IN_KM(a, da), DL_IN_KM(b, db) : "memory");
  } else if constexpr (AK && BK && FA == 4 && FB == 8) {
    asm volatile(DL_KM4(a) DL_KM8(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_KM4(a, af), DL_OUT_KM8(b, bf) : DL_IN_KM(a, da), DL_IN_KM(b, db) : "memory");
  } else if constexpr (AK && !BK && FA == 4 && FB == 4) {
    asm volatile(DL_KM4(a) DL_MN4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_KM4(a, af), DL_OUT_MN4(b, bl, bh) : DL_IN_KM(a, da), DL_IN_MN4(b, db) : "memory");
  } else if constexpr (AK && !BK && FA == 8 && FB == 4) {
    asm volatile(DL_KM8(a) DL_MN4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_KM8(a, af), DL_OUT_MN4(b, bl, bh) : DL_IN_KM(a, da), DL_IN_MN4(b, db) : "memory");
  } else if constexpr (!AK && BK && FA == 4 && FB == 4) {
    asm volatile(DL_MN4(a) DL_KM4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_MN4(a, al, ah), DL_OUT_KM4(b, bf) : DL_IN_MN4(a, da), DL_IN_KM(b, db) : "memory");
  } else if constexpr (!AK && !BK && FA == 8 && FB == 4) {
    // two blocks (operand count): A fragments 0..3 with B, then A 4..7
    asm volatile(DL_MN4(a) DL_MN4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_MN4(a, al, ah), DL_OUT_MN4(b, bl, bh) : DL_IN_MN4(a, da), DL_IN_MN4(b, db) : "memory");
    u32x2* al4 = al + 4;
    u32x2* ah4 = ah + 4;
    asm volatile(DL_MN4(c) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_MN4(c, al4, ah4)
                 : [cp0] "v"(da.a[4]), [cp1] "v"(da.a[5]), [cp2] "v"(da.a[6]), [cp3] "v"(da.a[7])
                 : "memory");
  } else if constexpr (!AK && !BK && FA == 4 && FB == 4) {
    asm volatile(DL_MN4(a) DL_MN4(b) "s_waitcnt lgkmcnt(0)"
                 : DL_OUT_MN4(a, al, ah), DL_OUT_MN4(b, bl, bh) : DL_IN_MN4(a, da), DL_IN_MN4(b, db) : "memory");
  } else {
    static_assert(AK && BK && FA == 4 && FB == 4, "unsupported fragment shape");
  }
  if constexpr (!AK) {
#pragma unroll
    for (int i = 0; i < FA; ++i) af[i] = u32x4{al[i][0], al[i][1], ah[i][0], ah[i][1]};
  }
  if constexpr (!BK) {
#pragma unroll
    for (int i = 0; i < FB; ++i) bf[i] = u32x4{bl[i][0], bl[i][1], bh[i][0], bh[i][1]};
  }
}
#undef DL_R128
#undef DL_KM4
#undef DL_KM8
#undef DL_RTR
#undef DL_MN4
#undef DL_OKM
#undef DL_OUT_KM4
#undef DL_OUT_KM8
#undef DL_OMN
#undef DL_OUT_MN4
#undef DL_IN_KM
#undef DL_IN_MN4

struct DlCtx {
  const bf16* A;
  const bf16* B;
  int64_t lda, ldb;
  int M, N, m0, n0, kbeg, nk, wave, lane;
  int brow[4];  // B rows this lane copies under the RoPE epilogue's row map (sub-tile s, copy i at 2 s + i)
};

// The B rows (output columns) a lane copies for the (NS x 128)-row tile at
// n0 under the RoPE epilogue's row map, computed once per block.
template <int NS>
__device__ __forceinline__ void dl_rope_rows(const RopeEpi& r, int N, int n0, int wave, int lane, int (&out)[4]) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      out[2 * s + i] = rope_row(r, min(n0 + 128 * s + (((wave * 2 + i) * 64 + lane) >> 2), N - 1));
}

// Copy the (NS x 128) x 32 operand tile at (row0, k0) into NS sub-tiles.
template <bool KM, int NS, bool MAP = false>
__device__ __forceinline__ void dl_issue_tile(const bf16* g, int64_t ld, int rows, int row0, int k0, bf16* tile,
                                              int wave, int lane, const int* rmap = nullptr) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
    dl_issue<KM, MAP>(g, ld, rows, row0 + 128 * s, k0, tile + s * DL_TILE, wave, lane, MAP ? rmap + 2 * s : nullptr);
}

// One k-step: wait for this wave's part of tile `it`, barrier, read the
// current stage, refill the stage freed in step it-1 with tile it+2 (past the
// end: the last tile again, into a stage nobody reads, so that the same
// number of copies per wave is in flight at every wait), multiply.
template <bool AK, bool BK, int FM, int FN, bool MAP = false>
__device__ __forceinline__ void dl_step(const DlCtx& c, int it, const DlAddr<AK, FM>& da, const DlAddr<BK, FN>& db,
                                        unsigned as, unsigned bs, bf16* An, bf16* Bn, f32x4 (&acc)[FM][FN]) {
  constexpr int NSA = FM / 4, NSB = FN / 4;
  SLT_WAIT_VMCNT(2 * (NSA + NSB));  // only the copies of tile it+1 may still fly
  lds_barrier();
  u32x4 af[FM], bfr[FN];
  dl_read<AK, BK, FM, FN>(da.at(as), db.at(bs), af, bfr);
  const int kn = c.kbeg + min(it + 2, c.nk - 1) * DL_BK;
  dl_issue_tile<AK, NSA>(c.A, c.lda, c.M, c.m0, kn, An, c.wave, c.lane);
  dl_issue_tile<BK, NSB, MAP>(c.B, c.ldb, c.N, c.n0, kn, Bn, c.wave, c.lane, c.brow);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[j]),
                                                          __builtin_bit_cast(bf16x8_t, af[i]), acc[i][j], 0, 0, 0);
}

// RoPE epilogue (RP), first phase: accumulator columns n .. n+3 of a rotated
// head hold two pairs (output dims i, i + R/2, i + 1, i + 1 + R/2 for
// rotate-half, by the B-row map; dims c .. c+3 for even-odd), rotated in
// place in fp32 by the angle of row m's position t = m % T.  No store runs
// in this phase, so every table read may be issued ahead of the others (a
// store to C between them would have to be assumed to alias the table).
template <int FM, int FN>
__device__ __forceinline__ void rope_rotate_acc(const KArgs& a, f32x4 (&acc)[FM][FN], int m0, int n0, int wm, int wn,
                                                int lane) {
  const RopeEpi& r = a.rope;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = min(m0 + wm * 16 * FM + i * 16 + (lane & 15), a.M - 1);
    const float* tb = r.cs + (int64_t)(m % r.T) * r.R;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * 16 * FN + j * 16 + 4 * (lane >> 4);
      const int c = n % r.d;
      if (n < r.end && c < r.R) {
        const float4 cs = *reinterpret_cast<const float4*>(tb + c);  // pairs c/2 and c/2 + 1
        const f32x4 v = acc[i][j];
        acc[i][j] = f32x4{v[0] * cs.x - v[1] * cs.y, v[0] * cs.y + v[1] * cs.x, v[2] * cs.z - v[3] * cs.w,
                          v[2] * cs.w + v[3] * cs.z};
      }
    }
  }
}

// The same rotation with the table entries loaded ahead (rope_load_cs, before
// the k-loop, so that their latency overlaps it): cs[i][j] holds the
// (cos, sin) pairs of fragment (i, j), unused where no pair is rotated.
template <int FM, int FN>
__device__ __forceinline__ void rope_load_cs(const KArgs& a, float4 (&cs)[FM][FN], int m0, int n0, int wm, int wn,
                                             int lane) {
  const RopeEpi& r = a.rope;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = min(m0 + wm * 16 * FM + i * 16 + (lane & 15), a.M - 1);
    const float* tb = r.cs + (int64_t)(m % r.T) * r.R;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * 16 * FN + j * 16 + 4 * (lane >> 4);
      const int c = n % r.d;
      cs[i][j] = (n < r.end && c < r.R) ? *reinterpret_cast<const float4*>(tb + c) : make_float4(1.f, 0.f, 1.f, 0.f);
    }
  }
}
template <int FM, int FN>
__device__ __forceinline__ void rope_rotate_pre(const KArgs& a, f32x4 (&acc)[FM][FN], const float4 (&cs)[FM][FN],
                                                int n0, int wn, int lane) {
  const RopeEpi& r = a.rope;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * 16 * FN + j * 16 + 4 * (lane >> 4);
      const int c = n % r.d;
      if (n < r.end && c < r.R) {
        const float4 t = cs[i][j];
        const f32x4 v = acc[i][j];
        acc[i][j] = f32x4{v[0] * t.x - v[1] * t.y, v[0] * t.y + v[1] * t.x, v[2] * t.z - v[3] * t.w,
                          v[2] * t.w + v[3] * t.z};
      }
    }
}

// Block epilogue: lane holds C[m][n .. n+3] of each 16 x 16 fragment; split-K
// blocks write fp32 partials, the others alpha C (+ R) in the output type.
// RP: the accumulators were rotated by rope_rotate_acc; a rotated
// rotate-half group (y0, y1, y2, y3) = dims (i, i + R/2, i + 1, i + 1 + R/2)
// is stored as two pairs.
template <typename TO, bool SPLIT, int FM, int FN, bool RP = false>
__device__ __forceinline__ void dl_epilogue(const KArgs& a, const f32x4 (&acc)[FM][FN], int m0, int n0, int wm, int wn,
                                            int lane) {
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * 16 * FM + i * 16 + (lane & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * 16 * FN + j * 16 + 4 * (lane >> 4);
      if (n >= a.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if constexpr (RP) {
        const int c = n % a.rope.d;
        if (a.rope.half && n < a.rope.end && c < a.rope.R) {
          TO* row = static_cast<TO*>(a.C) + (int64_t)m * a.ldc + (n - c) + (c >> 1);
          Pk<TO, 2> lo, hi;
          lo.e[0] = from_f32<TO>(v[0]); lo.e[1] = from_f32<TO>(v[2]);
          hi.e[0] = from_f32<TO>(v[1]); hi.e[1] = from_f32<TO>(v[3]);
          *reinterpret_cast<Pk<TO, 2>*>(row) = lo;
          *reinterpret_cast<Pk<TO, 2>*>(row + (a.rope.R >> 1)) = hi;
          continue;
        }
      }
      if (SPLIT) {
        float* dst = a.ws + ((int64_t)blockIdx.z * a.M + m) * a.N + n;
        if (a.evec && n + 3 < a.N) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int r = 0; r < 4 && n + r < a.N; ++r) dst[r] = v[r];
        }
        continue;
      }
      TO* dst = static_cast<TO*>(a.C) + (int64_t)m * a.ldc + n;
      const TO* res = a.R ? static_cast<const TO*>(a.R) + (int64_t)m * a.ldr + n : nullptr;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] *= a.alpha;
      if (a.drop.on) {
        float dm[4];
        drop_mults<4>(a.drop, (uint64_t)m * a.N + n, dm);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] *= dm[r];
      }
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

// Block tile (32 FM) x (32 FN): 2 x 2 waves, each 16 FM x 16 FN.
template <typename TO, bool AK, bool BK, bool SPLIT, int FM, int FN, bool RP = false>
__global__ __launch_bounds__(NT, (FM * FN > 16) ? 2 : 1) void gemm_dl_k(KArgs a) {
  constexpr int NSA = FM / 4, NSB = FN / 4;
  constexpr int TBM = 32 * FM, TBN = 32 * FN;
  // three stages as distinct LDS objects
  __shared__ __attribute__((aligned(16))) bf16 A0[NSA * DL_TILE], A1[NSA * DL_TILE], A2[NSA * DL_TILE];
  __shared__ __attribute__((aligned(16))) bf16 B0[NSB * DL_TILE], B1[NSB * DL_TILE], B2[NSB * DL_TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  int tile = blockIdx.x;
  if (SLT_GEMM_XCD) {
    const int q = a.tiles >> 3, r = a.tiles & 7, x = tile & 7;
    tile = x * q + min(x, r) + (tile >> 3);
  }
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  DlCtx c;
  c.A = static_cast<const bf16*>(a.A);
  c.B = static_cast<const bf16*>(a.B);
  c.lda = a.lda;
  c.ldb = a.ldb;
  c.M = a.M;
  c.N = a.N;
  c.m0 = tm * TBM;
  c.n0 = tn * TBN;
  c.kbeg = SPLIT ? blockIdx.z * a.kchunk : 0;
  c.nk = (min(a.K, c.kbeg + a.kchunk) - c.kbeg) / DL_BK;
  c.wave = wave;
  c.lane = lane;
  if constexpr (RP) dl_rope_rows<NSB>(a.rope, a.N, c.n0, wave, lane, c.brow);
  const DlAddr<AK, FM> da(wm * 16 * FM, lane);
  const DlAddr<BK, FN> db(wn * 16 * FN, lane);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  dl_issue_tile<AK, NSA>(c.A, c.lda, c.M, c.m0, c.kbeg, A0, wave, lane);
  dl_issue_tile<BK, NSB, RP>(c.B, c.ldb, c.N, c.n0, c.kbeg, B0, wave, lane, c.brow);
  dl_issue_tile<AK, NSA>(c.A, c.lda, c.M, c.m0, c.kbeg + min(1, c.nk - 1) * DL_BK, A1, wave, lane);
  dl_issue_tile<BK, NSB, RP>(c.B, c.ldb, c.N, c.n0, c.kbeg + min(1, c.nk - 1) * DL_BK, B1, wave, lane, c.brow);
  const unsigned a0 = lds_off(A0), a1 = lds_off(A1), a2 = lds_off(A2);
  const unsigned b0 = lds_off(B0), b1 = lds_off(B1), b2 = lds_off(B2);
  for (int it = 0; it < c.nk; it += 3) {
    dl_step<AK, BK, FM, FN, RP>(c, it, da, db, a0, b0, A2, B2, acc);
    if (it + 1 < c.nk) dl_step<AK, BK, FM, FN, RP>(c, it + 1, da, db, a1, b1, A0, B0, acc);
    if (it + 2 < c.nk) dl_step<AK, BK, FM, FN, RP>(c, it + 2, da, db, a2, b2, A1, B1, acc);
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends
  if constexpr (RP) rope_rotate_acc<FM, FN>(a, acc, c.m0, c.n0, wm, wn, lane);
  dl_epilogue<TO, SPLIT, FM, FN, RP>(a, acc, c.m0, c.n0, wm, wn, lane);
}


// ---------------------------------------------------------------------------
// 256 x 256 block tile, 8 waves (512 threads) as 2 x 4, each wave 128 x 64
// (EPI 0: plain; EPI 1: the fused SwiGLU projection; EPI 2: the RoPE epilogue)
// (8 x 4 MFMA tiles).  Per 32-deep k-step a block copies 32 KiB for 4 MFLOP
// -- half the bytes per FLOP of the 128 x 128 tile, whose copy path is the
// limit -- and two waves per SIMD let one wave's LDS reads overlap the
// other's MFMAs.  Three-stage LDS ring of 32 KiB stages (one block per CU).
// Each 128-row operand sub-tile takes one copy per lane.  Tiles are taken in
// bands of SLT_GEMM_BAND tile rows (band_coords).  Measured on gfx950 against
// a persistent form (one block per CU walking its XCD's tiles as one stream
// of k-steps) and a 64-deep two-stage form, this one was fastest.
// ---------------------------------------------------------------------------
constexpr int W8_NT = 512;

template <bool KM, bool MAP = false>
__device__ __forceinline__ void w8_issue(const bf16* g, int64_t ld, int rows, int row0, int k0, bf16* tile, int wave,
                                         int lane, const int* rmap = nullptr) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int p = wave * 64 + lane;  // 16-byte chunk position in the 128 x 32 sub-tile
    const int r0 = row0 + 128 * s;
    const bf16* src;
    if constexpr (KM) {
      const int r = p >> 2;
      const int lc = (p & 3) ^ dl_swz(r);
      const int row = MAP ? rmap[s] : min(r0 + r, rows - 1);
      src = g + (int64_t)row * ld + k0 + lc * 8;
    } else {
      const int kr = p >> 4;
      const int c = (p & 15) ^ dl_swz_mn(kr);
      src = g + (int64_t)(k0 + kr) * ld + min(r0 + c * 8, rows - 8);
    }
    lds_copy16(src, tile + s * DL_TILE + wave * 512);
  }
}

// B sub-tiles of the fused [W1; W3] projection: tile rows 64 w .. 64 w + 31
// are W1 rows f0 + 32 w + (0..31) and rows 64 w + 32 .. 64 w + 63 the W3 rows
// F + f0 + 32 w + (0..31), so that wave w's fragments 0, 1 (a) and 2, 3 (b)
// hold the same 32 output columns f.  F % 128 == 0.
__device__ __forceinline__ void w8_issue_pair(const bf16* g, int64_t ld, int F, int f0, int k0, bf16* tile, int wave,
                                              int lane) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int p = wave * 64 + lane;
    const int r = p >> 2;
    const int lc = (p & 3) ^ dl_swz(r);
    const int n = 128 * s + r, w = n & 63;
    const int grow = (w < 32 ? f0 : F + f0 - 32) + 32 * (n >> 6) + w;
    lds_copy16(g + (int64_t)grow * ld + k0 + lc * 8, tile + s * DL_TILE + wave * 512);
  }
}

template <bool AK, bool BK, int EPI = 0>
__device__ __forceinline__ void w8_step(const DlCtx& c, int it, const DlAddr<AK, 8>& da, const DlAddr<BK, 4>& db,
                                        unsigned as, unsigned bs, bf16* An, bf16* Bn, f32x4 (&acc)[8][4]) {
  SLT_WAIT_VMCNT(4);  // only the copies of tile it+1 may still fly
  lds_barrier();
  u32x4 af[8], bfr[4];
  dl_read<AK, BK, 8, 4>(da.at(as), db.at(bs), af, bfr);
  const int kn = c.kbeg + min(it + 2, c.nk - 1) * DL_BK;
  w8_issue<AK>(c.A, c.lda, c.M, c.m0, kn, An, c.wave, c.lane);
  if constexpr (EPI == 1) w8_issue_pair(c.B, c.ldb, c.N, c.n0, kn, Bn, c.wave, c.lane);
  else w8_issue<BK, EPI == 2>(c.B, c.ldb, c.N, c.n0, kn, Bn, c.wave, c.lane, c.brow);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[j]),
                                                          __builtin_bit_cast(bf16x8_t, af[i]), acc[i][j], 0, 0, 0);
}

// Fused SwiGLU epilogue of the 256 x 256 kernel (bf16, EPI 1): the tile
// covers f0 .. f0 + 127 of a and of b (w8_issue_pair); writes a, b and h.
// Measured alternatives that were not kept: the backward counterpart (dh's
// product with SwiGLU's backward in the epilogue) was slower than the GEMM
// plus the element kernel -- with one block per CU its 256 KiB of a/b reads
// per tile are not overlapped -- and GELU in the parallel block's projection
// epilogue was no faster than the separate element kernel (its extra stores
// cost what the saved read gained).
__device__ __forceinline__ void w8_epilogue_swiglu_fwd(const KArgs& a, const f32x4 (&acc)[8][4], int m0, int f0,
                                                       int wm, int wn, int lane) {
  bf16* ab = static_cast<bf16*>(a.C);
  bf16* hb = static_cast<bf16*>(a.C2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + wm * 128 + i * 16 + (lane & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int f = f0 + wn * 32 + j * 16 + 4 * (lane >> 4);
      float av[4], bv[4], hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        av[r] = to_f32(from_f32<bf16>(acc[i][j][r]));
        bv[r] = to_f32(from_f32<bf16>(acc[i][j + 2][r]));
        hv[r] = swiglu_h(av[r], bv[r]);
      }
      store4<bf16>(ab + (int64_t)m * a.ldc + f, av);
      store4<bf16>(ab + (int64_t)m * a.ldc + a.F + f, bv);
      store4<bf16>(hb + (int64_t)m * a.ldc2 + f, hv);
    }
  }
}

// LDS-staged epilogues of the 256 x 256 kernel.  Measured at the d=1024
// workloads, the output writes took 23-31 % of a forward projection's time
// (all CUs end their tiles together and write 128 KiB each).  Staged through
// LDS (the ring is free once the k-loop ends), each store instruction writes
// whole 16-byte chunks along rows, a wave covering full 128-byte lines, and
// the stores are non-temporal, so the outputs do not displace the operand
// panels from L2: the d=1024 lm_head projection went from 1.91 to 1.59 ms
// and the steps 1-3 % faster (the same stores in the 128 x 128 kernels and
// the weight-gradient kernels, whose smaller outputs the next kernel reads
// soon after, made the d=384 step slower and are not used there).  Same
// arithmetic as the direct stores: the fp32 accumulators are staged, and
// alpha, the dropout multipliers and the residual are applied before the
// one rounding to the output type.
constexpr int W8_CS = 256 + 4;                     // fp32 row stride of a staged 128-row half tile
constexpr int W8_HALF_BYTES = 128 * W8_CS * 4;     // 133,120 bytes
constexpr int W8_SWS = 128 + 8;                    // bf16 row stride of the staged SwiGLU a and b tiles
constexpr int W8_SW_BYTES = 2 * 256 * W8_SWS * 2;  // 139,264 bytes
constexpr int W8_RING_BYTES = 6 * 2 * DL_TILE * 2;  // three stages of A and B sub-tile pairs (96 KiB)
constexpr int W8_SMEM = W8_SW_BYTES > W8_HALF_BYTES ? W8_SW_BYTES : W8_HALF_BYTES;
static_assert(W8_SMEM >= W8_RING_BYTES, "staging area covers the ring");

// Eight consecutive outputs at (m, n): alpha v, dropout, residual, one rounding.
template <typename TO, bool NTS = SLT_NT_STORE>
__device__ __forceinline__ void w8_store8(const KArgs& a, int m, int n, const float (&vin)[8], bool vec) {
  float v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = vin[r] * a.alpha;
  if (a.drop.on) {
    float dm[8];
    drop_mults<8>(a.drop, (uint64_t)m * a.N + n, dm);
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] *= dm[r];
  }
  TO* dst = static_cast<TO*>(a.C) + (int64_t)m * a.ldc + n;
  const TO* res = a.R ? static_cast<const TO*>(a.R) + (int64_t)m * a.ldr + n : nullptr;
  if (vec && n + 7 < a.N) {
    if (res) {
      float r0[4], r1[4];
      load4<TO>(res, r0);
      load4<TO>(res + 4, r1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] += r0[r];
        v[4 + r] += r1[r];
      }
    }
    if constexpr (sizeof(TO) == 2) {
      Pk<TO, 8> pk;
#pragma unroll
      for (int r = 0; r < 8; ++r) pk.e[r] = from_f32<TO>(v[r]);
      if constexpr (NTS) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pk), reinterpret_cast<u32x4*>(dst));
      else *reinterpret_cast<Pk<TO, 8>*>(dst) = pk;
    } else {
      const float lo[4] = {v[0], v[1], v[2], v[3]}, hi[4] = {v[4], v[5], v[6], v[7]};
      store4<TO>(dst, lo);
      store4<TO>(dst + 4, hi);
    }
  } else {
    for (int r = 0; r < 8 && n + r < a.N; ++r) {
      float x = v[r];
      if (res) x += to_f32(res[r]);
      dst[r] = from_f32<TO>(x);
    }
  }
}

// Plain and RoPE (EPI 2) outputs: two passes of 128 rows; in pass h the
// waves of rows h write their fp32 accumulators into the LDS tile (RoPE
// pairs at their output columns, after the rotation: the launch takes this
// form for RoPE only when the head dim divides 256, so that every rotated
// head lies inside its tile), then all 512 threads store 8 columns at a
// time.
template <typename TO, int EPI>
__device__ __forceinline__ void w8_epilogue_staged(const KArgs& a, const f32x4 (&acc)[8][4], int m0, int n0, int wm,
                                                   int wn, int lane, float* F) {
  const bool vec = a.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(a.C) % (8 * sizeof(TO))) == 0 &&
                   (a.R == nullptr ||
                    (a.ldr % 8 == 0 && (reinterpret_cast<uintptr_t>(a.R) % (8 * sizeof(TO))) == 0));
  for (int h = 0; h < 2; ++h) {
    __syncthreads();  // the ring (pass 0) or the previous pass's tile is no longer read
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rl = i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cl = wn * 64 + j * 16 + 4 * (lane >> 4);
          const f32x4 v = acc[i][j];
          if constexpr (EPI == 2) {
            const int n = n0 + cl, c = n % a.rope.d;
            if (a.rope.half && n < a.rope.end && c < a.rope.R) {
              const int lo = n - c + (c >> 1) - n0, hi = lo + (a.rope.R >> 1);
              // four 4-byte stores: 8-byte pair stores push this kernel past
              // 256 VGPRs into scratch spills
              F[rl * W8_CS + lo] = v[0];
              F[rl * W8_CS + lo + 1] = v[2];
              F[rl * W8_CS + hi] = v[1];
              F[rl * W8_CS + hi + 1] = v[3];
              continue;
            }
          }
          *reinterpret_cast<float4*>(F + rl * W8_CS + cl) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = threadIdx.x + W8_NT * k;  // 4096 chunks of 8 columns
      const int rl = idx >> 5, cl = (idx & 31) * 8;
      const int m = m0 + h * 128 + rl, n = n0 + cl;
      if (m >= a.M || n >= a.N) continue;
      const float4 x0 = *reinterpret_cast<const float4*>(F + rl * W8_CS + cl);
      const float4 x1 = *reinterpret_cast<const float4*>(F + rl * W8_CS + cl + 4);
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      w8_store8<TO>(a, m, n, v, vec);
    }
  }
}

// Fused SwiGLU outputs (EPI 1): the bf16-rounded a and b of the whole tile
// go to LDS (256 rows x 128 columns each), then all 512 threads form h and
// store a, b and h 8 columns at a time.
__device__ __forceinline__ void w8_epilogue_swiglu_staged(const KArgs& a, const f32x4 (&acc)[8][4], int m0, int f0,
                                                          int wm, int wn, int lane, bf16* S) {
  bf16* SA = S;
  bf16* SB = S + 256 * W8_SWS;
  __syncthreads();  // the ring is no longer read
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = wm * 128 + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int fl = wn * 32 + j * 16 + 4 * (lane >> 4);
      Pk<bf16, 4> pa, pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pa.e[r] = from_f32<bf16>(acc[i][j][r]);
        pb.e[r] = from_f32<bf16>(acc[i][j + 2][r]);
      }
      *reinterpret_cast<Pk<bf16, 4>*>(SA + rl * W8_SWS + fl) = pa;
      *reinterpret_cast<Pk<bf16, 4>*>(SB + rl * W8_SWS + fl) = pb;
    }
  }
  __syncthreads();
  bf16* ab = static_cast<bf16*>(a.C);
  bf16* hb = static_cast<bf16*>(a.C2);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int idx = threadIdx.x + W8_NT * k;  // 4096 chunks of 8 columns
    const int rl = idx >> 4, fl = (idx & 15) * 8;
    const int m = m0 + rl, f = f0 + fl;
    if (m >= a.M) continue;
    const Pk<bf16, 8> pa = *reinterpret_cast<const Pk<bf16, 8>*>(SA + rl * W8_SWS + fl);
    const Pk<bf16, 8> pb = *reinterpret_cast<const Pk<bf16, 8>*>(SB + rl * W8_SWS + fl);
    Pk<bf16, 8> ph;
#pragma unroll
    for (int r = 0; r < 8; ++r) ph.e[r] = from_f32<bf16>(swiglu_h(to_f32(pa.e[r]), to_f32(pb.e[r])));
#if SLT_NT_STORE
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pa), reinterpret_cast<u32x4*>(ab + (int64_t)m * a.ldc + f));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pb),
                                reinterpret_cast<u32x4*>(ab + (int64_t)m * a.ldc + a.F + f));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ph), reinterpret_cast<u32x4*>(hb + (int64_t)m * a.ldc2 + f));
#else
    *reinterpret_cast<Pk<bf16, 8>*>(ab + (int64_t)m * a.ldc + f) = pa;
    *reinterpret_cast<Pk<bf16, 8>*>(ab + (int64_t)m * a.ldc + a.F + f) = pb;
    *reinterpret_cast<Pk<bf16, 8>*>(hb + (int64_t)m * a.ldc2 + f) = ph;
#endif
  }
}

// ST: LDS-staged epilogue (w8_epilogue_staged / w8_epilogue_swiglu_staged),
// else the direct stores of dl_epilogue / w8_epilogue_swiglu_fwd.
template <typename TO, bool AK, bool BK, int EPI = 0, bool ST = true>
__global__ __launch_bounds__(W8_NT, 1) void gemm_w8_k(KArgs a) {
  // the k-loop's three-stage ring, overlaid by the staged epilogue's tile
  __shared__ __attribute__((aligned(16))) char smem[ST ? W8_SMEM : W8_RING_BYTES];
  bf16* const A0 = reinterpret_cast<bf16*>(smem);
  bf16* const A1 = A0 + 2 * DL_TILE;
  bf16* const A2 = A1 + 2 * DL_TILE;
  bf16* const B0 = A2 + 2 * DL_TILE;
  bf16* const B1 = B0 + 2 * DL_TILE;
  bf16* const B2 = B1 + 2 * DL_TILE;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  int tile = blockIdx.x;
  if (SLT_GEMM_XCD) {
    const int q = a.tiles >> 3, r = a.tiles & 7, x = tile & 7;
    tile = x * q + min(x, r) + (tile >> 3);
  }
  int tm, tn;
  band_coords(tile, a.tiles, a.tiles_n, SLT_GEMM_BAND, tm, tn);
  DlCtx c;
  c.A = static_cast<const bf16*>(a.A);
  c.B = static_cast<const bf16*>(a.B);
  c.lda = a.lda;
  c.ldb = a.ldb;
  c.M = a.M;
  c.N = a.N;
  c.m0 = tm * 256;
  c.n0 = EPI == 1 ? tn * 128 : tn * 256;  // EPI 1: first f of the tile (B rows gathered by w8_issue_pair)
  if (EPI == 1) c.N = a.F;
  c.kbeg = 0;
  c.nk = a.K / DL_BK;
  c.wave = wave;
  c.lane = lane;
  if constexpr (EPI == 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) c.brow[s] = rope_row(a.rope, min(c.n0 + 128 * s + ((wave * 64 + lane) >> 2), a.N - 1));
  }
  const DlAddr<AK, 8> da(wm * 128, lane);
  const DlAddr<BK, 4> db(wn * 64, lane);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile 0's copies (A then B), then tile 1's: the first step's vmcnt wait
  // counts on that order
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int k0 = min(t, c.nk - 1) * DL_BK;
    w8_issue<AK>(c.A, c.lda, c.M, c.m0, k0, t ? A1 : A0, wave, lane);
    if constexpr (EPI == 1) w8_issue_pair(c.B, c.ldb, c.N, c.n0, k0, t ? B1 : B0, wave, lane);
    else w8_issue<BK, EPI == 2>(c.B, c.ldb, c.N, c.n0, k0, t ? B1 : B0, wave, lane, c.brow);
  }
  const unsigned a0 = lds_off(A0), a1 = lds_off(A1), a2 = lds_off(A2);
  const unsigned b0 = lds_off(B0), b1 = lds_off(B1), b2 = lds_off(B2);
  for (int it = 0; it < c.nk; it += 3) {
    w8_step<AK, BK, EPI>(c, it, da, db, a0, b0, A2, B2, acc);
    if (it + 1 < c.nk) w8_step<AK, BK, EPI>(c, it + 1, da, db, a1, b1, A0, B0, acc);
    if (it + 2 < c.nk) w8_step<AK, BK, EPI>(c, it + 2, da, db, a2, b2, A1, B1, acc);
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends
  if constexpr (EPI == 2) rope_rotate_acc<8, 4>(a, acc, c.m0, c.n0, wm, wn, lane);
  if constexpr (ST) {
    if constexpr (EPI == 1) w8_epilogue_swiglu_staged(a, acc, c.m0, c.n0, wm, wn, lane, reinterpret_cast<bf16*>(smem));
    else w8_epilogue_staged<TO, EPI>(a, acc, c.m0, c.n0, wm, wn, lane, reinterpret_cast<float*>(smem));
  } else {
    if constexpr (EPI == 1) w8_epilogue_swiglu_fwd(a, acc, c.m0, c.n0, wm, wn, lane);
    else dl_epilogue<TO, false, 8, 4, EPI == 2>(a, acc, c.m0, c.n0, wm, wn, lane);
  }
}

// ---------------------------------------------------------------------------
// Both operands k-major, 128 x 128 block tile: 64-deep k-steps in two stages.
// A tile row is then a whole 128-byte line (8 chunks of 16 bytes at position
// chunk XOR 2 ((row >> 1) & 3), conflict-free for the 16-row fragment reads),
// so each copy instruction fetches 8 full lines where the 32-deep ring's
// fetches 16 half lines.  Per k-step: one wait and barrier, the next tile's
// copies, then two 32-deep halves of reads and MFMAs.  Measured on gfx950 it
// beats the 32-deep ring on the forward projections with 384 to 1152 output
// columns; it loses on the m/n-major layouts and, as a 256 x 128 tile, on the
// wider forward projections, where it is not used.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int d64_swz(int r) { return 2 * ((r >> 1) & 3); }

// Copy the (32 F) x 64 tile at (row0, k0): F copies per lane.
template <int F, bool MAP = false>
__device__ __forceinline__ void d64_issue(const bf16* g, int64_t ld, int rows, int row0, int k0, bf16* tile, int wave,
                                          int lane, const int* rmap = nullptr) {
#pragma unroll
  for (int i = 0; i < F; ++i) {
    const int p = (wave * F + i) * 64 + lane;  // 16-byte chunk position in the tile
    const int r = p >> 3;
    const int lc = (p & 7) ^ d64_swz(r);
    const int row = MAP ? rmap[i] : min(row0 + r, rows - 1);
    lds_copy16(g + (int64_t)row * ld + k0 + lc * 8, tile + (wave * F + i) * 512);
  }
}

#define D64_R128(X, f, off) "ds_read_b128 %[" #X #f "], %[" #X "p] offset:" #off "\n\t"
#define D64_KM4(X) D64_R128(X, 0, 0) D64_R128(X, 1, 2048) D64_R128(X, 2, 4096) D64_R128(X, 3, 6144)
#define D64_OKM(X, f, v) [X##f] "=&v"(v[f])
#define D64_OUT_KM4(X, v) D64_OKM(X, 0, v), D64_OKM(X, 1, v), D64_OKM(X, 2, v), D64_OKM(X, 3, v)

// Fragments f = 0..3 of both operands (16 rows of 128 bytes each, 2 KiB
// apart) from LDS byte addresses pa and pb.
__device__ __forceinline__ void d64_read(unsigned pa, unsigned pb, u32x4 (&af)[4], u32x4 (&bf)[4]) {
  asm volatile(D64_KM4(a) D64_KM4(b) "s_waitcnt lgkmcnt(0)"
               : D64_OUT_KM4(a, af), D64_OUT_KM4(b, bf) : [ap] "v"(pa), [bp] "v"(pb) : "memory");
}
// Fragments 0..3 of A and 0..2 of B (the 64 x 192 tile's waves).
__device__ __forceinline__ void d64_read43(unsigned pa, unsigned pb, u32x4 (&af)[4], u32x4 (&bf)[3]) {
  asm volatile(D64_KM4(a) D64_R128(b, 0, 0) D64_R128(b, 1, 2048) D64_R128(b, 2, 4096) "s_waitcnt lgkmcnt(0)"
               : D64_OUT_KM4(a, af), D64_OKM(b, 0, bf), D64_OKM(b, 1, bf), D64_OKM(b, 2, bf)
               : [ap] "v"(pa), [bp] "v"(pb)
               : "memory");
}
#undef D64_R128
#undef D64_KM4
#undef D64_OKM
#undef D64_OUT_KM4

#ifndef SLT_D64_STAGED
#define SLT_D64_STAGED 1  // LDS-staged epilogue in the 64-deep kernel
#endif
#ifndef SLT_D64_NT
#define SLT_D64_NT 0  // ... with non-temporal stores
#endif

// Staged epilogue of the 64-deep kernel: in passes of 64 rows (two for the
// 128 x 128 tile, one for 64 x 192) the waves holding those rows write their
// fp32 accumulators into LDS (rotated RoPE pairs at their output columns:
// taken for rotate-half only when the head dim divides the tile width, so
// that every head lies inside one tile), then all 256 threads store 8
// consecutive columns at a time, each 64-thread wave covering whole rows.
// Same arithmetic as the direct stores: alpha, dropout and the residual are
// applied to the fp32 value before its one rounding.
template <typename TO, int LAY, bool RP>
__device__ __forceinline__ void d64_epilogue_staged(const KArgs& a, const f32x4 (&acc)[4][LAY ? 3 : 4], int m0,
                                                    int n0, int wm, int wn, int lane, float* F) {
  constexpr int FN = LAY ? 3 : 4, TBN = LAY ? 192 : 128, CS = TBN + 4, PASSES = LAY ? 1 : 2;
  const bool vec = a.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(a.C) % (8 * sizeof(TO))) == 0 &&
                   (a.R == nullptr ||
                    (a.ldr % 8 == 0 && (reinterpret_cast<uintptr_t>(a.R) % (8 * sizeof(TO))) == 0));
  for (int h = 0; h < PASSES; ++h) {
    __syncthreads();  // the ring (first pass) or the previous pass's rows are no longer read
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int cl = wn * 16 * FN + j * 16 + 4 * (lane >> 4);
          const f32x4 v = acc[i][j];
          if constexpr (RP) {
            const int n = n0 + cl, c = n % a.rope.d;
            if (a.rope.half && n < a.rope.end && c < a.rope.R) {
              const int lo = n - c + (c >> 1) - n0, hi = lo + (a.rope.R >> 1);
              // lo and hi are even (head starts, R / 2 and the tile origin
              // are), so each pair is one 8-byte store
              *reinterpret_cast<float2*>(F + rl * CS + lo) = make_float2(v[0], v[2]);
              *reinterpret_cast<float2*>(F + rl * CS + hi) = make_float2(v[1], v[3]);
              continue;
            }
          }
          *reinterpret_cast<float4*>(F + rl * CS + cl) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 64 * TBN / 8 / NT; ++k) {
      const int idx = threadIdx.x + NT * k;
      const int rl = idx / (TBN / 8), cl = (idx % (TBN / 8)) * 8;
      const int m = m0 + h * 64 + rl, n = n0 + cl;
      if (m >= a.M || n >= a.N) continue;
      const float4 x0 = *reinterpret_cast<const float4*>(F + rl * CS + cl);
      const float4 x1 = *reinterpret_cast<const float4*>(F + rl * CS + cl + 4);
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      w8_store8<TO, SLT_D64_NT>(a, m, n, v, vec);
    }
  }
}

// LAY 0: 128 x 128 block tile, 2 x 2 waves of 64 x 64.  LAY 1: 64 x 192,
// 1 x 4 waves of 64 x 48 (4 x 3 MFMA tiles): a 16384 x 384 output is 512
// such tiles, one full round of two blocks per CU, where 384 square tiles
// leave a quarter of the block slots idle.
// ST: the staged epilogue (d64_epilogue_staged), else dl_epilogue's direct
// stores (split-K partials always take those).
template <typename TO, bool SPLIT, bool RP = false, int LAY = 0, bool ST = false>
__global__ __launch_bounds__(NT) void gemm_d64_k(KArgs a) {
  constexpr int FM = 4, FN = LAY ? 3 : 4;
  constexpr int TBM = LAY ? 64 : 128, TBN = LAY ? 192 : 128;
  constexpr int FA = TBM / 32, FB = TBN / 32;  // copies per lane of an A and a B tile
  // the two stages of A and B (64 KiB), overlaid by the staged epilogue's rows
  static_assert(64 * (TBN + 4) * 4 <= 2 * (TBM + TBN) * 64 * 2, "staged rows fit in the ring");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (TBM + TBN) * 64];
  bf16* const A0 = smem;
  bf16* const A1 = A0 + TBM * 64;
  bf16* const B0 = A1 + TBM * 64;
  bf16* const B1 = B0 + TBN * 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = LAY ? 0 : wave >> 1, wn = LAY ? wave : wave & 1;
  int tile = blockIdx.x;
  if (SLT_GEMM_XCD) {
    const int q = a.tiles >> 3, r = a.tiles & 7, x = tile & 7;
    tile = x * q + min(x, r) + (tile >> 3);
  }
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  const bf16* A = static_cast<const bf16*>(a.A);
  const bf16* B = static_cast<const bf16*>(a.B);
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int kbeg = SPLIT ? blockIdx.z * a.kchunk : 0;
  const int nk = (min(a.K, kbeg + a.kchunk) - kbeg) / 64;
  // lane (g, i) reads row i of a fragment, k chunk 4 s + g of half s
  const int i = lane & 15, g = lane >> 4;
  unsigned ra[2], rb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    ra[s] = (wm * 16 * FM + i) * 128 + ((4 * s + g) ^ d64_swz(i)) * 16;
    rb[s] = (wn * 16 * FN + i) * 128 + ((4 * s + g) ^ d64_swz(i)) * 16;
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int x = 0; x < FM; ++x)
#pragma unroll
    for (int y = 0; y < FN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  int brow[FB];  // B rows this lane copies under the RoPE epilogue's row map
#pragma unroll
  for (int i = 0; i < FB; ++i) brow[i] = 0;
  if constexpr (RP) {
#pragma unroll
    for (int i = 0; i < FB; ++i) brow[i] = rope_row(a.rope, min(n0 + (((wave * FB + i) * 64 + lane) >> 3), a.N - 1));
  }
  d64_issue<FA>(A, a.lda, a.M, m0, kbeg, A0, wave, lane);
  d64_issue<FB, RP>(B, a.ldb, a.N, n0, kbeg, B0, wave, lane, brow);
  float4 csv[RP && SLT_ROPE_PRELOAD ? FM : 1][RP && SLT_ROPE_PRELOAD ? FN : 1];
  if constexpr (RP && SLT_ROPE_PRELOAD) rope_load_cs<FM, FN>(a, csv, m0, n0, wm, wn, lane);
  for (int it = 0; it < nk; ++it) {
    SLT_WAIT_VMCNT(0);  // this wave's copies of tile it have landed
    lds_barrier();      // ... everyone's have, and the other stage is free
    if (it + 1 < nk) {
      const int kn = kbeg + (it + 1) * 64;
      d64_issue<FA>(A, a.lda, a.M, m0, kn, (it & 1) ? A0 : A1, wave, lane);
      d64_issue<FB, RP>(B, a.ldb, a.N, n0, kn, (it & 1) ? B0 : B1, wave, lane, brow);
    }
    const unsigned as = lds_off((it & 1) ? A1 : A0), bs = lds_off((it & 1) ? B1 : B0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 af[FM], bfr[FN];
      if constexpr (FN == 4) d64_read(as + ra[s], bs + rb[s], af, bfr);
      else d64_read43(as + ra[s], bs + rb[s], af, bfr);
#pragma unroll
      for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[y]),
                                                              __builtin_bit_cast(bf16x8_t, af[x]), acc[x][y], 0, 0, 0);
    }
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends
  if constexpr (RP && SLT_ROPE_PRELOAD) rope_rotate_pre<FM, FN>(a, acc, csv, n0, wn, lane);
  else if constexpr (RP) rope_rotate_acc<FM, FN>(a, acc, m0, n0, wm, wn, lane);
  if constexpr (ST && !SPLIT) d64_epilogue_staged<TO, LAY, RP>(a, acc, m0, n0, wm, wn, lane, reinterpret_cast<float*>(smem));
  else dl_epilogue<TO, SPLIT, FM, FN, RP>(a, acc, m0, n0, wm, wn, lane);
}

#ifndef SLT_D64_ROPE192
#define SLT_D64_ROPE192 1  // RoPE projections whose rotate-half heads fit 192-wide tiles only: 64 x 192 tiles
#endif
#ifndef SLT_D64_NARROW
#define SLT_D64_NARROW 1  // the 64-deep kernel's 64 x 192 layout where it fills the chip better
#endif
// Layout of the 64-deep kernel for an M x N output: the 64 x 192 tile when N
// is a multiple of 192 and its estimated time is lower.  The estimate is
// tile area x tiles, counted as at least one full round of 512 blocks (two
// per CU), times 7/6 for the narrow tile (its k-steps stage 256 rows for
// 3/4 of the MFMA work of a 128 x 128 tile; measured: 16384 x 384 outputs
// are 13% faster as 512 narrow tiles than as 384 square ones, 16384 x 1152
// outputs 10% slower as 1536 narrow tiles than as 1152 square ones).
inline bool d64_narrow(int M, int N) {
  if (!SLT_D64_NARROW || N % 192 != 0) return false;
  const int64_t t0 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  const int64_t t1 = (int64_t)((M + 63) / 64) * (N / 192);
  return std::max<int64_t>(t1, 512) * (64 * 192) * 7 < std::max<int64_t>(t0, 512) * (128 * 128) * 6;
}

// ---------------------------------------------------------------------------
// Grouped weight gradients: several products dW_i = alpha_i A_i^T B_i with
// the same K (the token count) and both operands m/n-major (rows of tokens),
// in one launch.  The tiles of all products form one list, so a layer's
// weight gradients together fill the chip with few K splits (long k-ranges
// per block, few partials) where each alone needs many.  Blocks run the
// direct-to-LDS main loop of gemm_dl_k; with splits, partial tiles go to
// ws[split][tile][128 x 128] and gemm_group_reduce_k adds them in split
// order (deterministic); without, the block writes alpha C (+ C).
// ---------------------------------------------------------------------------
constexpr int kGroupMax = 6;

struct GProb {
  const bf16* A;  // A(m, k) = A[k lda + m]
  const bf16* B;  // B(n, k) = B[k ldb + n]
  float* C;
  int64_t lda, ldb, ldc;
  int M, N, tiles_n, tile0;  // first tile of this product in the group's list
  float alpha;
  int accumulate;  // C = alpha A B + C
};

struct GArgs {
  GProb p[kGroupMax];
  int np, tiles, kchunk;
  float* ws;
};

__device__ __forceinline__ int group_find(const GArgs& a, int tile) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kGroupMax; ++j)
    if (j < a.np && tile >= a.p[j].tile0) i = j;
  return i;
}

template <bool SPLIT>
__global__ __launch_bounds__(NT) void gemm_group_k(GArgs a) {
  constexpr int FM = 4, FN = 4;
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
  const GProb& P = a.p[group_find(a, tile)];
  const int lt = tile - P.tile0;
  const int tm = lt / P.tiles_n, tn = lt % P.tiles_n;
  DlCtx c;
  c.A = P.A;
  c.B = P.B;
  c.lda = P.lda;
  c.ldb = P.ldb;
  c.M = P.M;
  c.N = P.N;
  c.m0 = tm * 128;
  c.n0 = tn * 128;
  c.kbeg = SPLIT ? blockIdx.z * a.kchunk : 0;
  c.nk = a.kchunk / DL_BK;
  c.wave = wave;
  c.lane = lane;
  const DlAddr<false, FM> da(wm * 64, lane);
  const DlAddr<false, FN> db(wn * 64, lane);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  dl_issue_tile<false, 1>(c.A, c.lda, c.M, c.m0, c.kbeg, A0, wave, lane);
  dl_issue_tile<false, 1>(c.B, c.ldb, c.N, c.n0, c.kbeg, B0, wave, lane);
  dl_issue_tile<false, 1>(c.A, c.lda, c.M, c.m0, c.kbeg + min(1, c.nk - 1) * DL_BK, A1, wave, lane);
  dl_issue_tile<false, 1>(c.B, c.ldb, c.N, c.n0, c.kbeg + min(1, c.nk - 1) * DL_BK, B1, wave, lane);
  const unsigned a0 = lds_off(A0), a1 = lds_off(A1), a2 = lds_off(A2);
  const unsigned b0 = lds_off(B0), b1 = lds_off(B1), b2 = lds_off(B2);
  for (int it = 0; it < c.nk; it += 3) {
    dl_step<false, false, FM, FN>(c, it, da, db, a0, b0, A2, B2, acc);
    if (it + 1 < c.nk) dl_step<false, false, FM, FN>(c, it + 1, da, db, a1, b1, A0, B0, acc);
    if (it + 2 < c.nk) dl_step<false, false, FM, FN>(c, it + 2, da, db, a2, b2, A1, B1, acc);
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends

  // lane holds C[m][n .. n+3] of each 16 x 16 fragment
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int ml = wm * 64 + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nl = wn * 64 + j * 16 + 4 * (lane >> 4);
      const f32x4 v = acc[i][j];
      if (SPLIT) {
        float* dst = a.ws + ((int64_t)blockIdx.z * a.tiles + tile) * (128 * 128) + ml * 128 + nl;
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        const int m = c.m0 + ml, n = c.n0 + nl;
        if (m >= P.M || n >= P.N) continue;  // N % 8 == 0: the 4 columns are all inside
        float* dst = P.C + (int64_t)m * P.ldc + n;
        float4 o = make_float4(P.alpha * v[0], P.alpha * v[1], P.alpha * v[2], P.alpha * v[3]);
        if (P.accumulate) {
          const float4 r = *reinterpret_cast<const float4*>(dst);
          o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
        }
        *reinterpret_cast<float4*>(dst) = o;
      }
    }
  }
}

// Large groups: 256 x 256 tiles, 8 waves of 128 x 64 (the gemm_w8_k main
// loop), whole K per block, alpha C (+ C) written directly.
__global__ __launch_bounds__(W8_NT, 1) void gemm_group_w8_k(GArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 A0[2 * DL_TILE], A1[2 * DL_TILE], A2[2 * DL_TILE];
  __shared__ __attribute__((aligned(16))) bf16 B0[2 * DL_TILE], B1[2 * DL_TILE], B2[2 * DL_TILE];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  int tile = blockIdx.x;
  if (SLT_GEMM_XCD) {
    const int q = a.tiles >> 3, r = a.tiles & 7, x = tile & 7;
    tile = x * q + min(x, r) + (tile >> 3);
  }
  const GProb& P = a.p[group_find(a, tile)];
  const int lt = tile - P.tile0;
  DlCtx c;
  c.A = P.A;
  c.B = P.B;
  c.lda = P.lda;
  c.ldb = P.ldb;
  c.M = P.M;
  c.N = P.N;
  c.m0 = (lt / P.tiles_n) * 256;
  c.n0 = (lt % P.tiles_n) * 256;
  c.kbeg = 0;
  c.nk = a.kchunk / DL_BK;
  c.wave = wave;
  c.lane = lane;
  const DlAddr<false, 8> da(wm * 128, lane);
  const DlAddr<false, 4> db(wn * 64, lane);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  w8_issue<false>(c.A, c.lda, c.M, c.m0, 0, A0, wave, lane);
  w8_issue<false>(c.B, c.ldb, c.N, c.n0, 0, B0, wave, lane);
  w8_issue<false>(c.A, c.lda, c.M, c.m0, min(1, c.nk - 1) * DL_BK, A1, wave, lane);
  w8_issue<false>(c.B, c.ldb, c.N, c.n0, min(1, c.nk - 1) * DL_BK, B1, wave, lane);
  const unsigned a0 = lds_off(A0), a1 = lds_off(A1), a2 = lds_off(A2);
  const unsigned b0 = lds_off(B0), b1 = lds_off(B1), b2 = lds_off(B2);
  for (int it = 0; it < c.nk; it += 3) {
    w8_step<false, false>(c, it, da, db, a0, b0, A2, B2, acc);
    if (it + 1 < c.nk) w8_step<false, false>(c, it + 1, da, db, a1, b1, A0, B0, acc);
    if (it + 2 < c.nk) w8_step<false, false>(c, it + 2, da, db, a2, b2, A1, B1, acc);
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = c.m0 + wm * 128 + i * 16 + (lane & 15);
    if (m >= P.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = c.n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
      if (n >= P.N) continue;  // N % 8 == 0: the 4 columns are all inside
      const f32x4 v = acc[i][j];
      float* dst = P.C + (int64_t)m * P.ldc + n;
      float4 o = make_float4(P.alpha * v[0], P.alpha * v[1], P.alpha * v[2], P.alpha * v[3]);
      if (P.accumulate) {
        const float4 r = *reinterpret_cast<const float4*>(dst);
        o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
      }
      *reinterpret_cast<float4*>(dst) = o;
    }
  }
}

// C[m, n] = alpha sum_z ws[z][tile][m, n] (+ C) over the group's tiles; four
// consecutive columns per thread, splits added in increasing order.
__global__ __launch_bounds__(256) void gemm_group_reduce_k(GArgs a, int splits) {
  const int64_t total = (int64_t)a.tiles * (128 * 128 / 4);
  const int64_t tstride = (int64_t)a.tiles * (128 * 128);
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int tile = (int)(idx >> 12);
    const int e = (int)(idx & 4095) * 4;
    const GProb& P = a.p[group_find(a, tile)];
    const int lt = tile - P.tile0;
    const int m = (lt / P.tiles_n) * 128 + (e >> 7), n = (lt % P.tiles_n) * 128 + (e & 127);
    if (m >= P.M || n >= P.N) continue;
    const float* src = a.ws + (int64_t)tile * (128 * 128) + e;
    float4 s = *reinterpret_cast<const float4*>(src);
    for (int z = 1; z < splits; ++z) {
      const float4 t = *reinterpret_cast<const float4*>(src + z * tstride);
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    float* dst = P.C + (int64_t)m * P.ldc + n;
    float4 o = make_float4(P.alpha * s.x, P.alpha * s.y, P.alpha * s.z, P.alpha * s.w);
    if (P.accumulate) {
      const float4 r = *reinterpret_cast<const float4*>(dst);
      o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
    }
    *reinterpret_cast<float4*>(dst) = o;
  }
}

inline bool al(const void* p, int b) { return (reinterpret_cast<uintptr_t>(p) % b) == 0; }

template <typename T, typename TO, bool AK, bool BKM, int VL, bool SPLIT>
void launch_one(const KArgs& ka, dim3 grid, hipStream_t s) {
  gemm_k<T, TO, AK, BKM, VL, SPLIT><<<grid, NT, 0, s>>>(ka);
}

// After the main kernel: the fixed-order sum of split-K partials, if any.
template <typename TO>
slt_status finish(const GemmArgs& g, bool split, int splits, hipStream_t s) {
  if (slt_status st = check_launch("gemm"); st != SLT_OK) return st;
  if (split) {
    const int64_t total = (int64_t)g.M * g.N;
    int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
    splitk_reduce_k<TO><<<blocks, 256, 0, s>>>(g.workspace, splits, g.M, g.N, static_cast<TO*>(g.C), g.ldc,
                                               static_cast<const TO*>(g.R), g.ldr, g.alpha);
  }
  return check_launch("gemm split-K reduction");
}

template <typename T, typename TO>
slt_status run(const GemmArgs& g, hipStream_t s) {
  constexpr int BK = Tr<T>::BK, EPV = Tr<T>::EPV;
  KArgs ka{};
  ka.M = g.M; ka.N = g.N; ka.K = g.K;
  ka.A = g.A; ka.lda = g.lda; ka.B = g.B; ka.ldb = g.ldb;
  ka.C = g.C; ka.ldc = g.ldc; ka.R = g.R; ka.ldr = g.ldr;
  ka.alpha = g.alpha;
  ka.drop = g.drop;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  ka.tiles_n = tiles_n;
  const int tiles = tiles_m * tiles_n;
  ka.tiles = tiles;

  // Vector loads need every vector wholly inside or outside the operand:
  // whole groups where the vector dimension (K for a k-major operand, its
  // rows otherwise) and the row stride are multiples of the group, else
  // element pairs (fp32) where they are even, else single elements.
  auto op_vl = [&](const void* p, int64_t ld, bool kmajor, int rows) {
    const int full = kmajor ? EPV : 4;
    const int64_t q = kmajor ? g.K : rows;
    if (q % full == 0 && ld % full == 0 && al(p, full * (int)sizeof(T))) return kVecFull;
    if (sizeof(T) == 4 && q % 2 == 0 && ld % 2 == 0 && al(p, 2 * (int)sizeof(T))) return kVecPair;
    return kVecOne;
  };
  const int vl = std::min(op_vl(g.A, g.lda, g.a_kmajor, g.M), op_vl(g.B, g.ldb, g.b_kmajor, g.N));

  // Split K when the output grid cannot fill the 256 compute units and K is
  // long; the partials must fit the workspace.
  int splits = 1;
  if (g.workspace && tiles < 256 && !g.drop.on) {
    const int kt = (g.K + BK - 1) / BK;
    int want = std::min((SLT_SPLIT_TARGET + tiles - 1) / tiles, kt / SLT_SPLIT_MINK);
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

  // Direct-to-LDS path (bf16): K a multiple of 32 (and of each split's
  // range), 16-byte aligned rows, m/n-major operands at least 8 wide in
  // whole 16-byte chunks.
  if constexpr (sizeof(T) == 2) {
    auto dl_ok = [&](const void* p, int64_t ld, bool kmajor, int rows) {
      return al(p, 16) && ld % 8 == 0 && (kmajor || (rows % 8 == 0 && rows >= 8));
    };
    if (g.K > 0 && g.K % DL_BK == 0 && ka.kchunk % DL_BK == 0 && dl_ok(g.A, g.lda, g.a_kmajor, g.M) &&
        dl_ok(g.B, g.ldb, g.b_kmajor, g.N)) {
#define SLT_DL_GO(AKv, BKv, FMv, FNv)                                                          \
  do {                                                                                         \
    if (split) gemm_dl_k<float, AKv, BKv, true, FMv, FNv><<<grid, NT, 0, s>>>(ka);             \
    else gemm_dl_k<TO, AKv, BKv, false, FMv, FNv><<<grid, NT, 0, s>>>(ka);                     \
  } while (0)
      // Larger block tiles stage fewer bytes per FLOP (the copies feeding LDS
      // are the limit at 128 x 128): 256 x 128 (or 128 x 256) when the grid
      // holds at least 1.5 rounds of two such blocks per CU and K is not split
      // (at fewer tiles the last round leaves CUs idle and 128 x 128 is faster).
      // 256 x 256 tiles (one 8-wave block per CU) for grids of at least
      // SLT_W8_MIN such tiles whose edges waste little and whose last round
      // of 256 blocks is mostly full (measured: 1.25 or 1.5 rounds lose to
      // the smaller tiles)
      if (!split && g.a_kmajor && SLT_GEMM_W8) {
        const int t8m = (g.M + 255) / 256, t8n = (g.N + 255) / 256, t8 = t8m * t8n;
        const bool edges = (int64_t)t8 * 256 * 256 <= (int64_t)g.M * g.N * 9 / 8;
        const bool rounds = t8 * 20 >= ((t8 + 255) / 256) * 256 * 17;
        if (t8 >= SLT_W8_MIN && edges && rounds) {
          ka.tiles_n = t8n;
          ka.tiles = t8m * t8n;
          if (g.b_kmajor) gemm_w8_k<TO, true, true><<<ka.tiles, W8_NT, 0, s>>>(ka);
          else gemm_w8_k<TO, true, false><<<ka.tiles, W8_NT, 0, s>>>(ka);
          return finish<TO>(g, false, 1, s);
        }
      }
      int fm = 4, fn = 4;
      if (!split && g.a_kmajor && SLT_GEMM_BIG) {
        auto ntiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn); };
        if (g.M >= g.N && ntiles(256, 128) >= 768) fm = 8;
        else if (g.b_kmajor && ntiles(128, 256) >= 768) fn = 8;
      }
      if (fm != 4 || fn != 4) {
        ka.tiles_n = (g.N + 32 * fn - 1) / (32 * fn);
        ka.tiles = ((g.M + 32 * fm - 1) / (32 * fm)) * ka.tiles_n;
        grid = dim3(ka.tiles, 1, 1);
      }
      if (SLT_GEMM_D64 && g.a_kmajor && g.b_kmajor && fm == 4 && fn == 4 && g.K % 64 == 0 && ka.kchunk % 64 == 0) {
        if (split) {
          gemm_d64_k<float, true><<<grid, NT, 0, s>>>(ka);
        } else if (d64_narrow(g.M, g.N)) {
          ka.tiles_n = g.N / 192;
          ka.tiles = ((g.M + 63) / 64) * ka.tiles_n;
          gemm_d64_k<TO, false, false, 1, SLT_D64_STAGED><<<ka.tiles, NT, 0, s>>>(ka);
        } else {
          gemm_d64_k<TO, false, false, 0, SLT_D64_STAGED><<<grid, NT, 0, s>>>(ka);
        }
      } else if (g.a_kmajor && g.b_kmajor) {
        if (fm == 8) SLT_DL_GO(true, true, 8, 4);
        else if (fn == 8) SLT_DL_GO(true, true, 4, 8);
        else SLT_DL_GO(true, true, 4, 4);
      } else if (g.a_kmajor) {
        if (fm == 8) SLT_DL_GO(true, false, 8, 4);
        else SLT_DL_GO(true, false, 4, 4);
      } else if (g.b_kmajor) {
        SLT_DL_GO(false, true, 4, 4);
      } else {
        SLT_DL_GO(false, false, 4, 4);
      }
#undef SLT_DL_GO
      return finish<TO>(g, split, splits, s);
    }
  }

#define SLT_GEMM_VL(TOv, AKv, BKv, SPv)                                                   \
  do {                                                                                    \
    if (vl == kVecFull) launch_one<T, TOv, AKv, BKv, kVecFull, SPv>(ka, grid, s);         \
    else if (vl == kVecOne) launch_one<T, TOv, AKv, BKv, kVecOne, SPv>(ka, grid, s);      \
    else if constexpr (sizeof(T) == 4) launch_one<T, TOv, AKv, BKv, kVecPair, SPv>(ka, grid, s); \
  } while (0)
#define SLT_GEMM_GO(AKv, BKv)                  \
  do {                                         \
    if (split) SLT_GEMM_VL(float, AKv, BKv, true); \
    else SLT_GEMM_VL(TO, AKv, BKv, false);     \
  } while (0)

  if (g.a_kmajor && g.b_kmajor) SLT_GEMM_GO(true, true);
  else if (g.a_kmajor) SLT_GEMM_GO(true, false);
  else if (g.b_kmajor) SLT_GEMM_GO(false, true);
  else SLT_GEMM_GO(false, false);
#undef SLT_GEMM_GO
#undef SLT_GEMM_VL
  return finish<TO>(g, split, splits, s);
}

}  // namespace

// The 256 x 256 kernel's selection rule (see run()) for an M x N grid.
static bool w8_fits(int M, int N) {
  const int t8m = (M + 255) / 256, t8n = (N + 255) / 256, t8 = t8m * t8n;
  const bool edges = (int64_t)t8 * 256 * 256 <= (int64_t)M * N * 9 / 8;
  const bool rounds = t8 * 20 >= ((t8 + 255) / 256) * 256 * 17;
  return SLT_GEMM_W8 && t8 >= SLT_W8_MIN && edges && rounds;
}

slt_status launch_gemm_rope(const GemmArgs& g, const RopeEpi& r, hipStream_t s) {
  const bool ok = g.in_dtype == SLT_BF16 && g.out_dtype == SLT_BF16 && g.a_kmajor && g.b_kmajor && g.M > 0 &&
                  g.N > 0 && g.K > 0 && g.K % DL_BK == 0 && al(g.A, 16) && g.lda % 8 == 0 && al(g.B, 16) &&
                  g.ldb % 8 == 0 && g.N % 4 == 0 && g.ldc % 4 == 0 && al(g.C, 8) && g.R == nullptr &&
                  g.alpha == 1.0f && !g.drop.on && r.cs && al(r.cs, 16) && r.T > 0 && r.d > 0 && r.d % 4 == 0 &&
                  r.R > 0 && r.R % 4 == 0 && r.R <= r.d && r.end > 0 && r.end % r.d == 0 && r.end <= g.N;
  if (!ok) return fail(SLT_EUNSUPPORTED, "projection with RoPE epilogue: shape or alignment");
  KArgs ka{};
  ka.M = g.M; ka.N = g.N; ka.K = g.K;
  ka.A = g.A; ka.lda = g.lda; ka.B = g.B; ka.ldb = g.ldb;
  ka.C = g.C; ka.ldc = g.ldc;
  ka.alpha = 1.0f;
  ka.kchunk = g.K;
  ka.evec = true;
  ka.rope = r;
  if (w8_fits(g.M, g.N)) {
    ka.tiles_n = (g.N + 255) / 256;
    ka.tiles = ((g.M + 255) / 256) * ka.tiles_n;
    // the staged epilogue keeps each rotated head inside its 256-column tile
    if (256 % r.d == 0) gemm_w8_k<bf16, true, true, 2, true><<<ka.tiles, W8_NT, 0, s>>>(ka);
    else gemm_w8_k<bf16, true, true, 2, false><<<ka.tiles, W8_NT, 0, s>>>(ka);
    return check_launch("gemm with RoPE epilogue");
  }
  auto ntiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn); };
  int fm = 4, fn = 4;
  if (SLT_GEMM_BIG) {
    if (g.M >= g.N && ntiles(256, 128) >= 768) fm = 8;
    else if (ntiles(128, 256) >= 768) fn = 8;
  }
  // the staged epilogue keeps each rotated head inside its tile: for
  // rotate-half, the head dim must divide the tile width
  const bool st128 = SLT_D64_STAGED && (!r.half || 128 % r.d == 0);
  const bool st192 = SLT_D64_STAGED && (!r.half || 192 % r.d == 0);
  if (fm == 4 && fn == 4 && SLT_GEMM_D64 && g.K % 64 == 0 &&
      (d64_narrow(g.M, g.N) || (SLT_D64_ROPE192 && g.N % 192 == 0 && st192 && !st128))) {
    ka.tiles_n = g.N / 192;
    ka.tiles = ((g.M + 63) / 64) * ka.tiles_n;
    if (st192) gemm_d64_k<bf16, false, true, 1, true><<<ka.tiles, NT, 0, s>>>(ka);
    else gemm_d64_k<bf16, false, true, 1, false><<<ka.tiles, NT, 0, s>>>(ka);
    return check_launch("gemm with RoPE epilogue");
  }
  ka.tiles_n = (g.N + 32 * fn - 1) / (32 * fn);
  ka.tiles = ((g.M + 32 * fm - 1) / (32 * fm)) * ka.tiles_n;
  const dim3 grid(ka.tiles, 1, 1);
  if (fm == 8) gemm_dl_k<bf16, true, true, false, 8, 4, true><<<grid, NT, 0, s>>>(ka);
  else if (fn == 8) gemm_dl_k<bf16, true, true, false, 4, 8, true><<<grid, NT, 0, s>>>(ka);
  else if (SLT_GEMM_D64 && g.K % 64 == 0 && st128) gemm_d64_k<bf16, false, true, 0, true><<<grid, NT, 0, s>>>(ka);
  else if (SLT_GEMM_D64 && g.K % 64 == 0) gemm_d64_k<bf16, false, true, 0, false><<<grid, NT, 0, s>>>(ka);
  else gemm_dl_k<bf16, true, true, false, 4, 4, true><<<grid, NT, 0, s>>>(ka);
  return check_launch("gemm with RoPE epilogue");
}

slt_status launch_gemm_swiglu_fwd(int M, int F, int K, const void* X, int64_t ldx, const void* W13, void* ab,
                                  int64_t ldab, void* h, int64_t ldh, hipStream_t s) {
  if (!(SLT_FUSED_SWIGLU && M > 0 && F > 0 && F % 128 == 0 && K > 0 && K % DL_BK == 0 && al(X, 16) && ldx % 8 == 0 && al(W13, 16) &&
        al(ab, 8) && ldab % 4 == 0 && al(h, 8) && ldh % 4 == 0 && w8_fits(M, 2 * F)))
    return fail(SLT_EUNSUPPORTED, "fused SwiGLU projection: shape or alignment");
  KArgs ka{};
  ka.M = M; ka.N = 2 * F; ka.K = K;
  ka.A = X; ka.lda = ldx; ka.B = W13; ka.ldb = K;
  ka.C = ab; ka.ldc = ldab; ka.C2 = h; ka.ldc2 = ldh; ka.F = F;
  ka.alpha = 1.f;
  ka.tiles_n = F / 128;
  ka.tiles = ((M + 255) / 256) * ka.tiles_n;
  // the staged epilogue stores 16-byte groups
  if (al(ab, 16) && ldab % 8 == 0 && al(h, 16) && ldh % 8 == 0)
    gemm_w8_k<bf16, true, true, 1, true><<<ka.tiles, W8_NT, 0, s>>>(ka);
  else
    gemm_w8_k<bf16, true, true, 1, false><<<ka.tiles, W8_NT, 0, s>>>(ka);
  return check_launch("fused SwiGLU projection");
}

bool gemm_group_ok(const GroupItem& it, int K) {
  auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return K > 0 && K % DL_BK == 0 && it.M >= 8 && it.N >= 8 && it.M % 8 == 0 && it.N % 8 == 0 && it.lda % 8 == 0 &&
         it.ldb % 8 == 0 && it.ldc % 4 == 0 && al16(it.A) && al16(it.B) && al16(it.C);
}

slt_status launch_gemm_group(const GroupItem* items, int n, int K, float* ws, int64_t ws_bytes, hipStream_t s) {
  if (n <= 0) return SLT_OK;
  if (n > kGroupMax) return fail(SLT_EUNSUPPORTED, "gemm group: too many products");
  GArgs a{};
  a.np = n;
  int tiles = 0;
  for (int i = 0; i < n; ++i) {
    const GroupItem& it = items[i];
    if (!gemm_group_ok(it, K)) return fail(SLT_EUNSUPPORTED, "gemm group: shape or alignment");
    GProb& P = a.p[i];
    P.A = static_cast<const bf16*>(it.A);
    P.B = static_cast<const bf16*>(it.B);
    P.C = it.C;
    P.lda = it.lda;
    P.ldb = it.ldb;
    P.ldc = it.ldc;
    P.M = it.M;
    P.N = it.N;
    P.tiles_n = (it.N + 127) / 128;
    P.tile0 = tiles;
    P.alpha = it.alpha;
    P.accumulate = it.accumulate ? 1 : 0;
    tiles += ((it.M + 127) / 128) * P.tiles_n;
  }
  a.tiles = tiles;
  // 256 x 256 tiles when the group has at least SLT_GROUP_W8_MIN of them and
  // their edges waste little
  {
    int64_t t8 = 0, area = 0;
    for (int i = 0; i < n; ++i) {
      t8 += (int64_t)((items[i].M + 255) / 256) * ((items[i].N + 255) / 256);
      area += (int64_t)items[i].M * items[i].N;
    }
    if (SLT_GEMM_W8 && t8 >= SLT_GROUP_W8_MIN && t8 * 256 * 256 <= area * 9 / 8) {
      GArgs b = a;
      int t = 0;
      for (int i = 0; i < n; ++i) {
        b.p[i].tiles_n = (items[i].N + 255) / 256;
        b.p[i].tile0 = t;
        t += ((items[i].M + 255) / 256) * b.p[i].tiles_n;
      }
      b.tiles = t;
      b.kchunk = K;
      gemm_group_w8_k<<<t, W8_NT, 0, s>>>(b);
      return check_launch("gemm group (256 x 256)");
    }
  }
  // splits: aim for SLT_GROUP_TARGET blocks, at least SLT_SPLIT_MINK k-steps
  // each, K divided evenly in whole k-steps, partials inside the workspace
  const int kt = K / DL_BK;
  int splits = std::max(1, std::min((SLT_GROUP_TARGET + tiles - 1) / tiles, kt / SLT_SPLIT_MINK));
  const int64_t per = (int64_t)tiles * 128 * 128 * 4;
  while (splits > 1 && (kt % splits || !ws || per * splits > ws_bytes)) --splits;
  a.kchunk = (kt / splits) * DL_BK;
  a.ws = ws;
  const dim3 grid(tiles, 1, splits);
  if (splits > 1) {
    gemm_group_k<true><<<grid, NT, 0, s>>>(a);
    if (slt_status st = check_launch("gemm group"); st != SLT_OK) return st;
    const int64_t total = (int64_t)tiles * 4096;
    const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
    gemm_group_reduce_k<<<blocks, 256, 0, s>>>(a, splits);
    return check_launch("gemm group reduction");
  }
  gemm_group_k<false><<<grid, NT, 0, s>>>(a);
  return check_launch("gemm group");
}

slt_status launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return SLT_OK;
  if (g.in_dtype == SLT_BF16) {
    return g.out_dtype == SLT_BF16 ? run<bf16, bf16>(g, s) : run<bf16, float>(g, s);
  }
  if (g.out_dtype == SLT_BF16) return fail(SLT_EUNSUPPORTED, "gemm: fp32 inputs with bf16 output");
  return run<float, float>(g, s);
}

}  // namespace slt
