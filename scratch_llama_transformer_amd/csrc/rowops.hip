// Bandwidth-bound kernels of the training step: embedding, norms, MLP
// activations, fused softmax cross-entropy, AdamW, casts and the RoPE table.
//
// Layout rules: one 64-lane wavefront per row for the norms (rows are at most
// a few KB, so a row is read with 16-byte vector loads by one wave and reduced
// with cross-lane shuffles); flat vectorised grid-stride loops for the
// elementwise kernels; one 256-thread block per row for the loss, whose rows
// are up to 100 KB.  Every reduction runs in a fixed order, so results do not
// depend on scheduling (Hephaistos, "Design notes": results independent of the
// thread count).
#include "slt_internal.h"

#include <math.h>

#include <algorithm>
#include <initializer_list>
#include <type_traits>

namespace slt {

namespace {

constexpr int kWave = 64;

template <typename T, int VEC>
struct alignas(sizeof(T) * VEC) Pack {
  T e[VEC];
};

template <typename T, int VEC>
__device__ __forceinline__ void load_f(const T* p, float (&f)[VEC]) {
  Pack<T, VEC> pk = *reinterpret_cast<const Pack<T, VEC>*>(p);
#pragma unroll
  for (int i = 0; i < VEC; ++i) f[i] = to_f32(pk.e[i]);
}

template <typename T, int VEC>
__device__ __forceinline__ void store_f(T* p, const float (&f)[VEC]) {
  Pack<T, VEC> pk;
#pragma unroll
  for (int i = 0; i < VEC; ++i) pk.e[i] = from_f32<T>(f[i]);
  *reinterpret_cast<Pack<T, VEC>*>(p) = pk;
}

// Streaming (non-temporal) forms, for operands read or written once per step
// that no later kernel of the step reads soon: the lines are not kept in the
// caches, which measured on gfx950 raises a read stream from 6.3 to 7.1 TB/s
// and a copy from 5.5 to 5.8 TB/s (2 GiB buffers).
typedef unsigned ew_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned ew_u32x2 __attribute__((ext_vector_type(2)));
template <typename W> __device__ __forceinline__ W ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const W*>(p));
}
template <typename W> __device__ __forceinline__ void st_nt(void* p, W w) {
  __builtin_nontemporal_store(w, reinterpret_cast<W*>(p));
}
template <typename T, int VEC>
__device__ __forceinline__ Pack<T, VEC> ld_pack_nt(const T* p) {
  constexpr int B = VEC * (int)sizeof(T);
  if constexpr (B == 16) return __builtin_bit_cast(Pack<T, VEC>, ld_nt<ew_u32x4>(p));
  else if constexpr (B == 8) return __builtin_bit_cast(Pack<T, VEC>, ld_nt<ew_u32x2>(p));
  else if constexpr (B == 4) return __builtin_bit_cast(Pack<T, VEC>, ld_nt<unsigned>(p));
  else return *reinterpret_cast<const Pack<T, VEC>*>(p);
}
template <typename T, int VEC>
__device__ __forceinline__ void load_f_nt(const T* p, float (&f)[VEC]) {
  const Pack<T, VEC> pk = ld_pack_nt<T, VEC>(p);
#pragma unroll
  for (int i = 0; i < VEC; ++i) f[i] = to_f32(pk.e[i]);
}
__device__ __forceinline__ float4 ld_f4_nt(const float* p) {
  return __builtin_bit_cast(float4, ld_nt<ew_u32x4>(p));
}
__device__ __forceinline__ void st_f4_nt(float* p, float4 v) { st_nt<ew_u32x4>(p, __builtin_bit_cast(ew_u32x4, v)); }

#ifndef SLT_EW_THREADS
#define SLT_EW_THREADS 256  // block size of the streaming element kernels (1024 measured: faster alone, slower in the step)
#endif
constexpr int kEw = SLT_EW_THREADS;


inline bool aligned(const void* p, int bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// Embedding forward: x[i, :] = wte[id_i, :].  An id outside [0, V) yields a
// NaN row instead of an out-of-bounds read.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ __launch_bounds__(256) void embedding_fwd_k(const int32_t* __restrict__ tok, int T_, int64_t ld,
                                                       const T* __restrict__ wte, T* __restrict__ x, int N,
                                                       int V, int C, Drop drop) {
  const int cv = C / VEC;
  const int64_t total = (int64_t)N * cv;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx / cv);
    const int c = (int)(idx % cv) * VEC;
    const int id = tok[(int64_t)(i / T_) * ld + (i % T_)];
    float f[VEC];
    if (id >= 0 && id < V) {
      load_f<T, VEC>(wte + (int64_t)id * C + c, f);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = __builtin_nanf("");
    }
    if (drop.on) {  // inverted dropout of the embedding output (site 0)
      float m[VEC];
      drop_mults<VEC>(drop, (uint64_t)i * C + c, m);
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] *= m[e];
    }
    store_f<T, VEC>(x + (int64_t)i * C + c, f);
  }
}

// ---------------------------------------------------------------------------
// Embedding backward, deterministic:
//  1. per chunk of 256 positions: rank of each position among earlier equal
//     ids of the chunk, and the count of each id in the chunk;
//  2. per id: exclusive prefix of the chunk counts (in chunk order) and total;
//  3. exclusive scan of the totals -> start of each id in the sorted order;
//  4. scatter: position i goes to start[id] + prefix[chunk][id] + rank
//     (a stable counting sort by id, so positions of an id are increasing);
//     with it goes the slot's id and what its tile does at the slot (the run
//     goes on, or ends there as a head partial, a tail partial or a final
//     row), so that step 5 gathers rows with no lookups in between;
//  5. tiles of 16 sorted entries, one wave per tile and 64-lane column slab:
//     all 16 rows are loaded at once, then each run of equal ids is summed in
//     order; runs wholly inside a tile are final, the others leave a head or
//     tail partial;
//  6. per id: zero if absent; for ids spanning tiles, tail + heads in tile
//     order.
// ---------------------------------------------------------------------------
constexpr int kEmbChunk = 256;
constexpr int kEmbTile = 16;

struct EmbWs {
  int32_t* cnt;     // [nchunk][V]
  int32_t* rank;    // [N]
  int32_t* start;   // [V + 1]
  int32_t* total;   // [V]
  int32_t* sorted;  // [N]
  int32_t* skind;   // [N]: id << 2 | what the tile does at the slot (0 go on, 1 head, 2 tail, 3 final row)
  float* head;      // [ntile][C]
  float* tail;      // [ntile][C]
};

inline int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

EmbWs emb_ws_layout(void* base, int64_t N, int V, int C) {
  char* p = static_cast<char*>(base);
  const int64_t nchunk = (N + kEmbChunk - 1) / kEmbChunk;
  const int64_t ntile = (N + kEmbTile - 1) / kEmbTile;
  EmbWs w;
  w.cnt = reinterpret_cast<int32_t*>(p); p += align256(nchunk * V * 4);
  w.rank = reinterpret_cast<int32_t*>(p); p += align256(N * 4);
  w.start = reinterpret_cast<int32_t*>(p); p += align256((int64_t)(V + 1) * 4);
  w.total = reinterpret_cast<int32_t*>(p); p += align256((int64_t)V * 4);
  w.sorted = reinterpret_cast<int32_t*>(p); p += align256(N * 4);
  w.skind = reinterpret_cast<int32_t*>(p); p += align256(N * 4);
  w.head = reinterpret_cast<float*>(p); p += align256(ntile * C * 4);
  w.tail = reinterpret_cast<float*>(p); p += align256(ntile * C * 4);
  return w;
}

int64_t emb_ws_bytes(int64_t N, int V, int C) {
  const int64_t nchunk = (N + kEmbChunk - 1) / kEmbChunk;
  const int64_t ntile = (N + kEmbTile - 1) / kEmbTile;
  return align256(nchunk * V * 4) + 3 * align256(N * 4) + align256((int64_t)(V + 1) * 4) +
         align256((int64_t)V * 4) + 2 * align256(ntile * C * 4);
}

__global__ void fill_i32_k(int32_t* p, int32_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(kEmbChunk) void emb_chunk_rank_k(const int32_t* __restrict__ tok, int T_,
                                                               int64_t ld, int N, int V, EmbWs w) {
  __shared__ int32_t ids[kEmbChunk];
  const int t = threadIdx.x;
  const int i = blockIdx.x * kEmbChunk + t;
  int id = -1;
  if (i < N) {
    id = tok[(int64_t)(i / T_) * ld + (i % T_)];
    if (id < 0 || id >= V) id = -1;
  }
  ids[t] = id;
  __syncthreads();
  if (id < 0) return;
  int before = 0, after = 0;
  for (int j = 0; j < kEmbChunk; ++j) {
    const int o = ids[j];
    before += (o == id) & (j < t);
    after += (o == id) & (j > t);
  }
  w.rank[i] = before;
  if (after == 0) w.cnt[(int64_t)blockIdx.x * V + id] = before + 1;
}

__global__ void emb_col_prefix_k(int V, int nchunk, EmbWs w) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= V) return;
  constexpr int G = 16;  // counts loaded per batch (independent loads in flight)
  int run = 0;
  for (int c0 = 0; c0 < nchunk; c0 += G) {
    int x[G];
#pragma unroll
    for (int j = 0; j < G; ++j) x[j] = c0 + j < nchunk ? w.cnt[(int64_t)(c0 + j) * V + v] : 0;
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (c0 + j < nchunk) {
        w.cnt[(int64_t)(c0 + j) * V + v] = run;
        run += x[j];
      }
  }
  w.total[v] = run;
}

// Exclusive scan of total[0..V) into start[0..V] by one 1024-thread block.
__global__ __launch_bounds__(1024) void emb_scan_k(int V, EmbWs w) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int per = (V + 1023) / 1024;
  const int b = t * per, e = min(V, b + per);
  constexpr int G = 16;  // totals loaded per batch (independent loads in flight)
  int s = 0;
  for (int k0 = b; k0 < e; k0 += G) {
    int x[G];
#pragma unroll
    for (int j = 0; j < G; ++j) x[j] = k0 + j < e ? w.total[k0 + j] : 0;
#pragma unroll
    for (int j = 0; j < G; ++j) s += x[j];
  }
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
    const int add = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int run = t == 0 ? 0 : part[t - 1];
  for (int k0 = b; k0 < e; k0 += G) {
    int x[G];
#pragma unroll
    for (int j = 0; j < G; ++j) x[j] = k0 + j < e ? w.total[k0 + j] : 0;
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (k0 + j < e) {
        w.start[k0 + j] = run;
        run += x[j];
      }
  }
  if (t == 1023) w.start[V] = part[1023];
}

__global__ void emb_scatter_k(const int32_t* __restrict__ tok, int T_, int64_t ld, int N, int V, EmbWs w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const int id = tok[(int64_t)(i / T_) * ld + (i % T_)];
  if (id < 0 || id >= V) return;
  const int chunk = i / kEmbChunk;
  const int rs = w.start[id], re = w.start[id + 1], nvalid = w.start[V];
  const int j = rs + w.cnt[(int64_t)chunk * V + id] + w.rank[i];
  w.sorted[j] = i;
  // the slot's tile [ts, te): does the run end here, and where does its sum go
  const int ts = j / kEmbTile * kEmbTile, te = min(nvalid, ts + kEmbTile);
  const bool last = j == re - 1 || j == te - 1;
  const int kind = !last ? 0 : rs < ts ? 1 : re > te ? 2 : 3;
  w.skind[j] = (id << 2) | kind;
}

// One wave per (tile of kEmbTile sorted entries, slab of 64 VEC columns):
// the tile's slot records are uniform loads, its 16 rows are loaded at once,
// then runs are summed in order and stored where the slot record says.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void emb_tile_sum_k(const T* __restrict__ dx, float* __restrict__ dwte, int N,
                                                      int V_, int C, int nslab, EmbWs w, GradW gw, Drop drop) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int item = blockIdx.x * 4 + wave;
  const int tile = item / nslab, slab = item % nslab;
  const int s = tile * kEmbTile;
  const int nvalid = min(N, w.start[V_]);  // ids outside [0, V) are not sorted
  if (s >= nvalid) return;
  const int e = min(nvalid, s + kEmbTile);
  const int c0 = (slab * kWave + lane) * VEC;
  const int32_t* __restrict__ srt = w.sorted;
  const int32_t* __restrict__ skd = w.skind;
  int pos[kEmbTile], sk[kEmbTile];
#pragma unroll
  for (int k = 0; k < kEmbTile; ++k) {
    pos[k] = s + k < e ? srt[s + k] : 0;
    sk[k] = s + k < e ? skd[s + k] : 0;
  }
  if (c0 >= C) return;
  using P = Pack<T, VEC>;
  P fr[kEmbTile];
#pragma unroll
  for (int k = 0; k < kEmbTile; ++k)
    if (s + k < e) fr[k] = *reinterpret_cast<const P*>(dx + (int64_t)pos[k] * C + c0);
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
#pragma unroll
  for (int k = 0; k < kEmbTile; ++k) {
    if (s + k >= e) continue;
    float f[VEC];
#pragma unroll
    for (int q = 0; q < VEC; ++q) f[q] = to_f32(fr[k].e[q]);
    if (drop.on) {  // the embedding output's dropout mask (site 0), regenerated
      float m[VEC];
      drop_mults<VEC>(drop, (uint64_t)pos[k] * C + c0, m);
#pragma unroll
      for (int q = 0; q < VEC; ++q) f[q] *= m[q];
    }
#pragma unroll
    for (int q = 0; q < VEC; ++q) acc[q] += f[q];
    const int kind = sk[k] & 3;
    if (kind != 0) {
      float* dst;
      if (kind == 1) dst = w.head + (int64_t)tile * C + c0;       // continues from an earlier tile
      else if (kind == 2) dst = w.tail + (int64_t)tile * C + c0;  // continues into a later tile
      else dst = dwte + (int64_t)(sk[k] >> 2) * C + c0;           // complete inside this tile
      float o[VEC];
#pragma unroll
      for (int q = 0; q < VEC; ++q) {
        o[q] = kind == 3 ? gw.alpha * acc[q] + (gw.accumulate ? dst[q] : 0.f) : acc[q];
        acc[q] = 0.f;
      }
      if constexpr (VEC == 4 || VEC == 8) {
#pragma unroll
        for (int q = 0; q < VEC; q += 4)
          *reinterpret_cast<float4*>(dst + q) = make_float4(o[q], o[q + 1], o[q + 2], o[q + 3]);
      } else {
#pragma unroll
        for (int q = 0; q < VEC; ++q) dst[q] = o[q];
      }
    }
  }
}

// One 256-thread block per vocabulary row: zero rows, and rows spanning
// several tiles.  For the latter the 4 waves take contiguous quarters of the
// pieces (tail of the first tile, then heads in tile order); a lane owns 8
// columns of a 512-column pass (two 16-byte groups when the row width allows)
// and sums 8 pieces per step into 8 interleaved accumulators, so that 16
// 16-byte loads are in flight per lane (a frequent id of a skewed token mix
// spans a tenth of all tiles: its row is the critical path); the quarters are
// added in order.
template <bool V4>
__global__ __launch_bounds__(256) void emb_row_finish_k(float* __restrict__ dwte, int V, int C, EmbWs w,
                                                        GradW gw) {
  constexpr int QN = 8;  // columns per lane per pass
  constexpr int P = 8;   // pieces per step
  __shared__ __attribute__((aligned(16))) float part[4][kWave * QN];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int v = blockIdx.x;
  const int rs = w.start[v], re = w.start[v + 1];
  float* row = dwte + (int64_t)v * C;
  if (re == rs) {  // unseen id: exactly zero (or unchanged when accumulating)
    if (!gw.accumulate)
      for (int c = threadIdx.x; c < C; c += blockDim.x) row[c] = 0.f;
    return;
  }
  const int t0 = rs / kEmbTile, t1 = (re - 1) / kEmbTile;
  if (t0 == t1) return;
  // pieces: index 0 = tail[t0], index k >= 1 = head[t0 + k]
  const int np = t1 - t0 + 1;
  const int per = (np + 3) / 4;
  const int pb = min(np, wave * per), pe = min(np, pb + per);
  // column of a lane's value q in a pass: 4-wide groups at 4 lane + 256 (q / 4)
  // (V4), else single columns at lane + 64 q
  auto col = [&](int q) { return V4 ? 4 * lane + 256 * (q / 4) + (q % 4) : lane + kWave * q; };
  for (int c0 = 0; c0 < C; c0 += kWave * QN) {
    float acc[P][QN];
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
      for (int q = 0; q < QN; ++q) acc[u][q] = 0.f;
    for (int k = pb; k < pe; k += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int kk = k + u;
        if (kk < pe) {
          const float* src = (kk == 0 ? w.tail + (int64_t)t0 * C : w.head + (int64_t)(t0 + kk) * C) + c0;
          if (V4) {
#pragma unroll
            for (int g = 0; g < QN / 4; ++g) {
              const int c = col(4 * g);
              if (c0 + c < C) {
                const float4 f = *reinterpret_cast<const float4*>(src + c);
                acc[u][4 * g] += f.x;
                acc[u][4 * g + 1] += f.y;
                acc[u][4 * g + 2] += f.z;
                acc[u][4 * g + 3] += f.w;
              }
            }
          } else {
#pragma unroll
            for (int q = 0; q < QN; ++q)
              if (c0 + col(q) < C) acc[u][q] += src[col(q)];
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < QN; ++q)
      part[wave][col(q)] = ((acc[0][q] + acc[1][q]) + (acc[2][q] + acc[3][q])) +
                           ((acc[4][q] + acc[5][q]) + (acc[6][q] + acc[7][q]));
    __syncthreads();
    for (int c = threadIdx.x; c < kWave * QN; c += blockDim.x)
      if (c0 + c < C) {
        const float sum = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
        row[c0 + c] = gw.alpha * sum + (gw.accumulate ? row[c0 + c] : 0.f);
      }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// RMSNorm and LayerNorm: one wave per row.  VEC-wide groups of columns; lane
// l owns groups l, l+64, ... (at most NCH of them).
// ---------------------------------------------------------------------------
template <typename T, int VEC, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_fwd_k(const T* __restrict__ x, const T* __restrict__ g,
                                                     T* __restrict__ y, float* __restrict__ rstd,
                                                     int rows, int C, float eps) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const T* xr = x + (int64_t)row * C;
  float xv[NCH][VEC], gv[NCH][VEC];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {  // the gain is loaded with x, not after the reduction
    const int c = (lane + j * kWave) * VEC;
    if (c < C) {
      load_f<T, VEC>(xr + c, xv[j]);
      load_f<T, VEC>(g + c, gv[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + j * kWave) * VEC;
    if (c < C) {
#pragma unroll
      for (int q = 0; q < VEC; ++q) ss += xv[j][q] * xv[j][q];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)C + eps);
  if (lane == 0) rstd[row] = r;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + j * kWave) * VEC;
    if (c < C) {
      float out[VEC];
#pragma unroll
      for (int q = 0; q < VEC; ++q) out[q] = xv[j][q] * r * gv[j][q];
      store_f<T, VEC>(y + (int64_t)row * C + c, out);
    }
  }
}

template <typename T, int VEC, int NCH>
__global__ __launch_bounds__(256) void layernorm_fwd_k(const T* __restrict__ x, const T* __restrict__ gm,
                                                       const T* __restrict__ bt, T* __restrict__ y,
                                                       float* __restrict__ mean, float* __restrict__ rstd,
                                                       int rows, int C, float eps) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const T* xr = x + (int64_t)row * C;
  float xv[NCH][VEC];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + j * kWave) * VEC;
    if (c < C) {
      load_f<T, VEC>(xr + c, xv[j]);
#pragma unroll
      for (int q = 0; q < VEC; ++q) s += xv[j][q];
    }
  }
  const float mu = wave_sum(s) / (float)C;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + j * kWave) * VEC;
    if (c < C) {
#pragma unroll
      for (int q = 0; q < VEC; ++q) {
        const float d = xv[j][q] - mu;
        ss += d * d;
      }
    }
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) / (float)C + eps);
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = r;
  }
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + j * kWave) * VEC;
    if (c < C) {
      float gv[VEC], bv[VEC], out[VEC];
      load_f<T, VEC>(gm + c, gv);
      load_f<T, VEC>(bt + c, bv);
#pragma unroll
      for (int q = 0; q < VEC; ++q) out[q] = (xv[j][q] - mu) * r * gv[q] + bv[q];
      store_f<T, VEC>(y + (int64_t)row * C + c, out);
    }
  }
}

// Norm backward.  Block b (NWV waves) handles rows b*NWV + wave + k*gridDim*NWV
// and leaves per-column partial sums of dy*xh (and dy for LayerNorm) in
// part[b][C] (and part[nb + b][C]); norm_colsum_k adds the partials in block
// order.
template <typename T, int VEC, int NCH, bool LN, int NWV>
__global__ __launch_bounds__(64 * NWV) void norm_bwd_k(const T* __restrict__ x, const T* __restrict__ g,
                                                  const float* __restrict__ mean, const float* __restrict__ rstd,
                                                  const T* __restrict__ dy, const T* dres, T* dx,
                                                  float* __restrict__ part, int rows, int C) {
  extern __shared__ float red[];  // [C] (x2 for LayerNorm)
  using P = Pack<T, VEC>;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  float pg[NCH][VEC], pb[NCH][VEC];
  P gp[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + j * kWave) * VEC;
#pragma unroll
    for (int q = 0; q < VEC; ++q) pg[j][q] = pb[j][q] = 0.f;
    gp[j] = c < C ? *reinterpret_cast<const P*>(g + c) : P{};
  }

  // RP rows per iteration, every load of them issued before any use, so that
  // each wave keeps RP rows of x, dy and the incoming gradient in flight (the
  // grid is small: its block count sets the number of dg partials).  The rows
  // stay in registers as loaded (bf16 where T is bf16) and are widened where
  // used, so that wide rows do not push the kernel to one wave per SIMD.  A
  // wave visits rows blockIdx*4 + wave + m*step in increasing m whatever RP is,
  // so the partial sums do not depend on it.
  constexpr int RP = NCH >= 4 ? 1 : 4 / NCH;
  const int step = gridDim.x * NWV;
  for (int row0 = blockIdx.x * NWV + wave; row0 < rows; row0 += RP * step) {
    P xr[RP][NCH], dr[RP][NCH], rr[RP][NCH];
    float r[RP], mu[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int row = row0 + k * step;
      const bool ok = row < rows;
      const int64_t base = (int64_t)(ok ? row : row0) * C;
      r[k] = ok ? rstd[row] : 0.f;
      mu[k] = (LN && ok) ? mean[row] : 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = (lane + j * kWave) * VEC;
        xr[k][j] = dr[k][j] = rr[k][j] = P{};
        if (c < C && ok) {
          xr[k][j] = *reinterpret_cast<const P*>(x + base + c);
          dr[k][j] = *reinterpret_cast<const P*>(dy + base + c);
          if (dres != nullptr) rr[k][j] = *reinterpret_cast<const P*>(dres + base + c);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int row = row0 + k * step;
      if (row >= rows) break;
      const int64_t base = (int64_t)row * C;
      float s1 = 0.f, s2 = 0.f;  // sum dxh, sum dxh*xh
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = (lane + j * kWave) * VEC;
        if (c < C) {
#pragma unroll
          for (int q = 0; q < VEC; ++q) {
            const float xh = (to_f32(xr[k][j].e[q]) - mu[k]) * r[k];
            const float dyv = to_f32(dr[k][j].e[q]);
            const float dxh = dyv * to_f32(gp[j].e[q]);
            pg[j][q] += dyv * xh;
            pb[j][q] += dyv;
            s1 += dxh;
            s2 += dxh * xh;
          }
        }
      }
      const float m2 = wave_sum(s2) / (float)C;
      const float m1 = LN ? wave_sum(s1) / (float)C : 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = (lane + j * kWave) * VEC;
        if (c < C) {
          float out[VEC];
#pragma unroll
          for (int q = 0; q < VEC; ++q) {
            const float xh = (to_f32(xr[k][j].e[q]) - mu[k]) * r[k];
            const float dxh = to_f32(dr[k][j].e[q]) * to_f32(gp[j].e[q]);
            out[q] = to_f32(rr[k][j].e[q]) + r[k] * (dxh - m1 - xh * m2);
          }
          store_f<T, VEC>(dx + base + c, out);
        }
      }
    }
  }
  // Combine the waves' column partials in wave order, then write this
  // block's partial row.
  for (int w = 0; w < NWV; ++w) {
    if (wave == w) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = (lane + j * kWave) * VEC;
        if (c < C) {
#pragma unroll
          for (int q = 0; q < VEC; ++q) {
            red[c + q] = (w == 0 ? 0.f : red[c + q]) + pg[j][q];
            if (LN) red[C + c + q] = (w == 0 ? 0.f : red[C + c + q]) + pb[j][q];
          }
        }
      }
    }
    __syncthreads();
  }
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    part[(int64_t)blockIdx.x * C + c] = red[c];
    if (LN) part[(int64_t)(gridDim.x + blockIdx.x) * C + c] = red[C + c];
  }
}

// out[c] = sum_b part[b][c].  A 1024-thread block owns 32 columns: thread
// (g, c) adds partials g, g+32, ... in order, then the 32 group sums are added
// in a fixed tree.
__global__ __launch_bounds__(1024) void norm_colsum_k(const float* __restrict__ part, int nb, int C,
                                                       float* __restrict__ out, GradW gw) {
  __shared__ float red[32][33];
  const int tc = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int c = blockIdx.x * 32 + tc;
  float s = 0.f;
  if (c < C) {
#pragma unroll 8
    for (int b = g; b < nb; b += 32) s += part[(int64_t)b * C + c];
  }
  red[g][tc] = s;
  __syncthreads();
  for (int off = 16; off > 0; off >>= 1) {
    if (g < off) red[g][tc] += red[g + off][tc];
    __syncthreads();
  }
  if (g == 0 && c < C) out[c] = gw.alpha * red[0][tc] + (gw.accumulate ? out[c] : 0.f);
}

#ifndef SLT_NORM_BLOCKS
#define SLT_NORM_BLOCKS 512
#endif
constexpr int kNormBwdBlocks = SLT_NORM_BLOCKS;
#ifndef SLT_NORM_BWD_WAVES
#define SLT_NORM_BWD_WAVES 4  // waves per block of the norm backward
#endif
constexpr int kNormBwdWaves = SLT_NORM_BWD_WAVES;

// ---------------------------------------------------------------------------
// SwiGLU and GELU on [rows, F] with row strides.
// ---------------------------------------------------------------------------

template <typename T, int VEC>
__global__ __launch_bounds__(kEw) void swiglu_fwd_k(const T* __restrict__ a, const T* __restrict__ b,
                                                    T* __restrict__ h, int rows, int F, int64_t lda,
                                                    int64_t ldb, int64_t ldh) {
  const int fv = F / VEC;
  const int64_t total = (int64_t)rows * fv;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / fv;
    const int c = (int)(idx % fv) * VEC;
    float av[VEC], bv[VEC], out[VEC];
    load_f<T, VEC>(a + r * lda + c, av);
    load_f<T, VEC>(b + r * ldb + c, bv);
#pragma unroll
    for (int q = 0; q < VEC; ++q) out[q] = swiglu_h(av[q], bv[q]);
    store_f<T, VEC>(h + r * ldh + c, out);
  }
}

template <typename T, int VEC>
__global__ __launch_bounds__(kEw) void swiglu_bwd_k(const T* __restrict__ a, const T* __restrict__ b,
                                                    const T* __restrict__ dh, T* __restrict__ da,
                                                    T* __restrict__ db, int rows, int F, int64_t lda,
                                                    int64_t ldb, int64_t lddh, int64_t ldda, int64_t lddb) {
  const int fv = F / VEC;
  const int64_t total = (int64_t)rows * fv;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / fv;
    const int c = (int)(idx % fv) * VEC;
    float av[VEC], bv[VEC], hv[VEC], oa[VEC], ob[VEC];
    load_f_nt<T, VEC>(a + r * lda + c, av);
    load_f_nt<T, VEC>(b + r * ldb + c, bv);
    load_f<T, VEC>(dh + r * lddh + c, hv);
#pragma unroll
    for (int q = 0; q < VEC; ++q) swiglu_grad(av[q], bv[q], hv[q], oa[q], ob[q]);
    store_f<T, VEC>(da + r * ldda + c, oa);
    store_f<T, VEC>(db + r * lddb + c, ob);
  }
}


template <typename T, int VEC>
__global__ __launch_bounds__(kEw) void gelu_fwd_k(const T* __restrict__ a, T* __restrict__ u, int rows, int F,
                                                  int64_t lda, int64_t ldu) {
  const int fv = F / VEC;
  const int64_t total = (int64_t)rows * fv;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / fv;
    const int c = (int)(idx % fv) * VEC;
    float av[VEC], out[VEC];
    load_f<T, VEC>(a + r * lda + c, av);
#pragma unroll
    for (int q = 0; q < VEC; ++q) out[q] = gelu_tanh(av[q]);
    store_f<T, VEC>(u + r * ldu + c, out);
  }
}

template <typename T, int VEC>
__global__ __launch_bounds__(kEw) void gelu_bwd_k(const T* __restrict__ a, const T* __restrict__ du,
                                                  T* __restrict__ da, int rows, int F, int64_t lda,
                                                  int64_t lddu, int64_t ldda) {
  const int fv = F / VEC;
  const int64_t total = (int64_t)rows * fv;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / fv;
    const int c = (int)(idx % fv) * VEC;
    float av[VEC], gv[VEC], out[VEC];
    load_f_nt<T, VEC>(a + r * lda + c, av);
    load_f<T, VEC>(du + r * lddu + c, gv);
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      out[q] = gv[q] * gelu_tanh_grad(av[q]);
    }
    store_f<T, VEC>(da + r * ldda + c, out);
  }
}

// ---------------------------------------------------------------------------
// Fused softmax cross-entropy: one 256-thread block per row.  Pass 1 keeps a
// running (max, sum of exp) per thread and merges them across the block;
// pass 2 overwrites the logits with (softmax - onehot) / rows.  The row loss
// lse - z[y] goes to rowloss[]; xent_mean_k adds those in index order.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ __launch_bounds__(256) void xent_rows_k(T* z, int64_t ldz, const int32_t* __restrict__ tok, int T_,
                                                   int64_t ld, int V, int rows, float* __restrict__ rowloss,
                                                   float* lse_out) {
  __shared__ float sm[8], ss[8];
  __shared__ float zy_s;
  const int row = blockIdx.x;
  T* zr = z + (int64_t)row * ldz;
  const int y = tok[(int64_t)(row / T_) * ld + (row % T_) + 1];
  const int t = threadIdx.x;
  if (t == 0) zy_s = (y >= 0 && y < V) ? to_f32(zr[y]) : __builtin_nanf("");
  float m = -INFINITY, s = 0.f;
  for (int c = t * VEC; c < V; c += 256 * VEC) {
    float f[VEC];
    load_f<T, VEC>(zr + c, f);
    float mx = f[0];
#pragma unroll
    for (int q = 1; q < VEC; ++q) mx = fmaxf(mx, f[q]);
    const float mn = fmaxf(m, mx);
    float add = 0.f;
#pragma unroll
    for (int q = 0; q < VEC; ++q) add += __expf(f[q] - mn);
    s = s * __expf(m - mn) + add;
    m = mn;
  }
  // merge (m, s) over the wave, then over the 4 waves
  const float wm = wave_max(m);
  float wsum = wave_sum(m == -INFINITY ? 0.f : s * __expf(m - wm));
  const int wave = t / kWave, lane = t % kWave;
  if (lane == 0) {
    sm[wave] = wm;
    ss[wave] = wsum;
  }
  __syncthreads();
  float M = sm[0];
  for (int w = 1; w < 4; ++w) M = fmaxf(M, sm[w]);
  float S = 0.f;
  for (int w = 0; w < 4; ++w) S += ss[w] * __expf(sm[w] - M);
  const float lse = M + logf(S);
  const float inv_rows = 1.0f / (float)rows;
  if (t == 0) {
    rowloss[row] = lse - zy_s;
    if (lse_out) lse_out[row] = lse;
  }
  for (int c = t * VEC; c < V; c += 256 * VEC) {
    float f[VEC];
    load_f<T, VEC>(zr + c, f);
#pragma unroll
    for (int q = 0; q < VEC; ++q) f[q] = (__expf(f[q] - lse) - (c + q == y ? 1.0f : 0.0f)) * inv_rows;
    store_f<T, VEC>(zr + c, f);
  }
}

// The same row operation for bf16 rows of at most NIT x 2048 logits, the row
// held in registers as loaded (NIT 16-byte groups per thread): one read of
// the logits from HBM instead of two (measured: the two-pass form ran at
// 3.9 TB/s of algorithmic bytes on 51200-wide rows).  Max over the row,
// the sum of exp(z - max), then dz = exp(z - max) / sum - onehot, all over
// 1 / rows.  The bf16 -> fp32 widening is an asm statement at each use so
// that the widened row is never kept in registers (it would not fit).
__device__ __forceinline__ float bf_lo(uint32_t u) {
  float f;
  asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(f) : "v"(u));
  return f;
}
__device__ __forceinline__ float bf_hi(uint32_t u) {
  float f;
  asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(f) : "v"(u));
  return f;
}

template <int NIT>
__global__ __launch_bounds__(256) void xent_rows_reg_k(bf16* z, int64_t ldz, const int32_t* __restrict__ tok, int T_,
                                                       int64_t ld, int V, int rows, float* __restrict__ rowloss,
                                                       float* lse_out) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ float sm[4], ss[4];
  const int row = blockIdx.x;
  bf16* zr = z + (int64_t)row * ldz;
  const int y = tok[(int64_t)(row / T_) * ld + (row % T_) + 1];
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  u32x4_t x[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int c = (t + 256 * k) * 8;
    x[k] = c < V ? *reinterpret_cast<const u32x4_t*>(zr + c) : u32x4_t{0u, 0u, 0u, 0u};
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NIT; ++k)
    if ((t + 256 * k) * 8 < V)
#pragma unroll
      for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(bf_lo(x[k][q]), bf_hi(x[k][q])));
  m = wave_max(m);
  if (lane == 0) sm[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NIT; ++k)
    if ((t + 256 * k) * 8 < V)
#pragma unroll
      for (int q = 0; q < 4; ++q) s += __expf(bf_lo(x[k][q]) - M) + __expf(bf_hi(x[k][q]) - M);
  s = wave_sum(s);
  if (lane == 0) ss[wave] = s;
  __syncthreads();
  const float S = (ss[0] + ss[1]) + (ss[2] + ss[3]);
  const float lse = M + logf(S);
  const float inv_rows = 1.0f / (float)rows, scale = inv_rows / S;
  if (t == 0) {
    rowloss[row] = (y >= 0 && y < V) ? lse - to_f32(zr[y]) : __builtin_nanf("");
    if (lse_out) lse_out[row] = lse;
  }
  __syncthreads();  // the target logit is read before its row is overwritten
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int c = (t + 256 * k) * 8;
    if (c < V) {
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __expf(bf_lo(x[k][q]) - M) * scale;
        f[2 * q + 1] = __expf(bf_hi(x[k][q]) - M) * scale;
      }
      if (y >= c && y < c + 8) f[y - c] -= inv_rows;
      store_f<bf16, 8>(zr + c, f);
    }
  }
}

__global__ __launch_bounds__(1024) void xent_mean_k(const float* __restrict__ rowloss, int rows,
                                                    float* __restrict__ loss) {
  __shared__ float part[1024];
  const int t = threadIdx.x;
  float s = 0.f;
  for (int i = t; i < rows; i += 1024) s += rowloss[i];
  part[t] = s;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (t < off) part[t] += part[t + off];
    __syncthreads();
  }
  if (t == 0) *loss = part[0] / (float)rows;
}

// ---------------------------------------------------------------------------
// AdamW over a flat fp32 buffer, 4 elements per thread per step.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void adamw_one(float& th, float g, float& m, float& v, float b1, float b2,
                                          float ib1, float ib2, float lr, float eps, float wd) {
  m = b1 * m + (1.0f - b1) * g;
  v = b2 * v + (1.0f - b2) * g * g;
  const float mh = m * ib1;
  const float vh = v * ib2;
  th = th - lr * (mh / (sqrtf(vh) + eps) + wd * th);
}

__global__ __launch_bounds__(kEw) void adamw_k(int64_t n, float* __restrict__ th, uint16_t* __restrict__ shadow,
                                               const float* __restrict__ g, float* __restrict__ m,
                                               float* __restrict__ v, float b1, float b2, float ib1, float ib2,
                                               float lr, float eps, float wd, const uint8_t* __restrict__ mask,
                                               const float* __restrict__ gscale) {
  const float gs = gscale ? *gscale : 1.0f;  // gradient clipping factor (1: none)
  const int64_t n4 = n / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float4 t4 = ld_f4_nt(th + 4 * i);
    float4 g4 = ld_f4_nt(g + 4 * i);
    g4.x *= gs; g4.y *= gs; g4.z *= gs; g4.w *= gs;
    float4 m4 = ld_f4_nt(m + 4 * i);
    float4 v4 = ld_f4_nt(v + 4 * i);
    float w[4] = {wd, wd, wd, wd};
    if (mask) {
      const uchar4 k = __builtin_bit_cast(uchar4, ld_nt<unsigned>(mask + 4 * i));
      w[0] = k.x ? wd : 0.f; w[1] = k.y ? wd : 0.f; w[2] = k.z ? wd : 0.f; w[3] = k.w ? wd : 0.f;
    }
    adamw_one(t4.x, g4.x, m4.x, v4.x, b1, b2, ib1, ib2, lr, eps, w[0]);
    adamw_one(t4.y, g4.y, m4.y, v4.y, b1, b2, ib1, ib2, lr, eps, w[1]);
    adamw_one(t4.z, g4.z, m4.z, v4.z, b1, b2, ib1, ib2, lr, eps, w[2]);
    adamw_one(t4.w, g4.w, m4.w, v4.w, b1, b2, ib1, ib2, lr, eps, w[3]);
    st_f4_nt(th + 4 * i, t4);
    st_f4_nt(m + 4 * i, m4);
    st_f4_nt(v + 4 * i, v4);
    if (shadow) {
      const ew_u32x2 s2 = {(unsigned)f32_to_bf16_bits(t4.x) | ((unsigned)f32_to_bf16_bits(t4.y) << 16),
                           (unsigned)f32_to_bf16_bits(t4.z) | ((unsigned)f32_to_bf16_bits(t4.w) << 16)};
      st_nt<ew_u32x2>(shadow + 4 * i, s2);
    }
  }
  // tail elements
  const int64_t i = n4 * 4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && i < n) {
    float t1 = th[i], m1 = m[i], v1 = v[i];
    adamw_one(t1, g[i] * gs, m1, v1, b1, b2, ib1, ib2, lr, eps, (mask && !mask[i]) ? 0.f : wd);
    th[i] = t1; m[i] = m1; v[i] = v1;
    if (shadow) shadow[i] = f32_to_bf16_bits(t1);
  }
}

// Global gradient norm, two deterministic stages: a fixed grid of
// kGnBlocks blocks each reduces a fixed strided share in double precision
// (sum of squares, or max |g|) and writes one partial; one block reduces the
// partials in a fixed tree and writes the norm and the clipping factor
// (MicroGPT in Rust, "Gradient Clipping": max_norm / norm above max_norm,
// else 1).
constexpr int kGnBlocks = 1024;

template <bool LINF>
__global__ __launch_bounds__(256) void gnorm_partial_k(int64_t n, const float* __restrict__ g,
                                                       double* __restrict__ part) {
  double acc = 0.0;
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 x = ld_f4_nt(g + 4 * i);
    if (LINF) {
      acc = fmax(acc, (double)fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    } else {
      acc += (double)x.x * x.x + (double)x.y * x.y + (double)x.z * x.z + (double)x.w * x.w;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (int)(n - n4 * 4)) {
    const double x = g[n4 * 4 + threadIdx.x];
    acc = LINF ? fmax(acc, fabs(x)) : acc + x * x;
  }
  __shared__ double red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = LINF ? fmax(red[threadIdx.x], red[threadIdx.x + w])
                                                 : red[threadIdx.x] + red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

template <bool LINF>
__global__ __launch_bounds__(1024) void gnorm_final_k(const double* __restrict__ part, float max_norm,
                                                      float* norm_out, float* scale_out) {
  __shared__ double red[1024];
  red[threadIdx.x] = part[threadIdx.x];
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = LINF ? fmax(red[threadIdx.x], red[threadIdx.x + w])
                                                 : red[threadIdx.x] + red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double nrm = LINF ? red[0] : sqrt(red[0]);
    if (norm_out) *norm_out = (float)nrm;
    if (scale_out) *scale_out = nrm > (double)max_norm ? (float)((double)max_norm / nrm) : 1.0f;
  }
}

__global__ __launch_bounds__(256) void cast_bf16_k(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                   int64_t n) {
  const int64_t n4 = n / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 f = reinterpret_cast<const float4*>(src)[i];
    ushort4 s;
    s.x = f32_to_bf16_bits(f.x); s.y = f32_to_bf16_bits(f.y);
    s.z = f32_to_bf16_bits(f.z); s.w = f32_to_bf16_bits(f.w);
    reinterpret_cast<ushort4*>(dst)[i] = s;
  }
  const int64_t i = n4 * 4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && i < n) dst[i] = f32_to_bf16_bits(src[i]);
}

__global__ void fill_f32_k(float* p, float v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// RoPE table from float64 angles: cs[t*R + 2j] = cos, cs[t*R + 2j + 1] = sin.
__global__ void rope_table_k(int T_, int R, double base, float* cs) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = R / 2;
  if (idx >= T_ * h) return;
  const int t = idx / h, j = idx % h;
  const double theta = pow(base, -2.0 * (double)j / (double)R);
  const double ang = (double)t * theta;
  cs[(int64_t)t * R + 2 * j] = (float)cos(ang);
  cs[(int64_t)t * R + 2 * j + 1] = (float)sin(ang);
}

// *dst += a * (*x): the running mean loss of gradient accumulation.
__global__ void scalar_axpy_k(float* dst, float a, const float* x) { *dst += a * *x; }

// RoPE (Hephaistos, "Architecture at a glance"; Transformer in Rust, "Key
// Features": even-odd pairs): one thread per rotated pair (a, b) of one head
// of one row, (a, b) -> (a c - b s, a s + b c) with s times `sign` (-1: the
// transposed rotation, RoPE's backward); both values read before either is
// written, so y may equal x.  Then, when y is another buffer, the dims >= R
// are copied.
template <typename T>
__global__ void rope_apply_k(const T* x, int64_t ldx, T* y, int64_t ldy, int64_t rows, int T_, int nh, int d, int R,
                             int mode, const float* cs, float sign) {
  const int hr = R >> 1;
  const int64_t npair = rows * nh * hr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < npair; idx += stride) {
    const int j = (int)(idx % hr);
    const int64_t rh = idx / hr;
    const int h = (int)(rh % nh);
    const int64_t r = rh / nh;
    const int t = (int)(r % T_);
    const int ia = mode == SLT_ROPE_HALF ? j : 2 * j, ib = mode == SLT_ROPE_HALF ? j + hr : 2 * j + 1;
    const T* xr = x + r * ldx + (int64_t)h * d;
    T* yr = y + r * ldy + (int64_t)h * d;
    const float a = to_f32(xr[ia]), b = to_f32(xr[ib]);
    const float c = cs[(int64_t)t * R + 2 * j], sn = sign * cs[(int64_t)t * R + 2 * j + 1];
    yr[ia] = from_f32<T>(a * c - b * sn);
    yr[ib] = from_f32<T>(a * sn + b * c);
  }
  if (x == y || R >= d) return;
  const int rest = d - R;
  const int64_t ncopy = rows * nh * rest;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < ncopy; idx += stride) {
    const int j = R + (int)(idx % rest);
    const int64_t rh = idx / rest;
    const int h = (int)(rh % nh);
    const int64_t r = rh / nh;
    y[r * ldy + (int64_t)h * d + j] = x[r * ldx + (int64_t)h * d + j];
  }
}

}  // namespace

namespace {
// kind 0: N(0, std^2) by Box-Muller on the first two Philox outputs of
// counter (index, 0, 0, 0); kind 1: constant std (used for ones and zeros).
__global__ void model_init_k(float* dst, int64_t n, int64_t index0, uint32_t k0, uint32_t k1, float std,
                             int kind) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (kind == 1) {
      dst[i] = std;
      continue;
    }
    const uint64_t idx = (uint64_t)(index0 + i);
    const uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), 0u, 0u};
    const uint32_t key[2] = {k0, k1};
    uint32_t r[4];
    philox4x32_10(ctr, key, r);
    const float u1 = ((float)r[0] + 0.5f) * 2.3283064365386963e-10f;  // (0, 1)
    const float u2 = ((float)r[1] + 0.5f) * 2.3283064365386963e-10f;
    const float z = sqrtf(-2.0f * logf(u1)) * cosf(6.283185307179586f * u2);
    dst[i] = z * std;
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static int grid_for(int64_t work, int per_block = 256, int cap = 65536) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

template <typename T>
static constexpr int full_vec() { return 16 / (int)sizeof(T); }

slt_status launch_embedding_fwd(const int32_t* tok, int B, int T_, int64_t ld, const void* wte, void* x, int V,
                                int C, int dtype, hipStream_t s, Drop drop) {
  const int N = B * T_;
  auto go = [&](auto tag) {
    using T = decltype(tag);
    constexpr int VEC = full_vec<T>();
    if (C % VEC == 0 && aligned(wte, 16) && aligned(x, 16))
      embedding_fwd_k<T, VEC><<<grid_for((int64_t)N * C / VEC), 256, 0, s>>>(
          tok, T_, ld, (const T*)wte, (T*)x, N, V, C, drop);
    else
      embedding_fwd_k<T, 1><<<grid_for((int64_t)N * C), 256, 0, s>>>(tok, T_, ld, (const T*)wte, (T*)x, N, V, C,
                                                                     drop);
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  return check_launch("embedding_fwd");
}

int64_t embedding_bwd_ws(int64_t N, int V) {
  // head/tail partials are sized for C up to 4096
  return emb_ws_bytes(N, V, 4096);
}

slt_status launch_embedding_sort(const int32_t* tok, int B, int T_, int64_t ld, int V, void* ws, hipStream_t s) {
  const int N = B * T_;
  EmbWs w = emb_ws_layout(ws, N, V, 4096);
  const int nchunk = cdiv(N, kEmbChunk);
  fill_i32_k<<<grid_for((int64_t)nchunk * V), 256, 0, s>>>(w.cnt, 0, (int64_t)nchunk * V);
  emb_chunk_rank_k<<<nchunk, kEmbChunk, 0, s>>>(tok, T_, ld, N, V, w);
  emb_col_prefix_k<<<cdiv(V, 256), 256, 0, s>>>(V, nchunk, w);
  emb_scan_k<<<1, 1024, 0, s>>>(V, w);
  emb_scatter_k<<<cdiv(N, 256), 256, 0, s>>>(tok, T_, ld, N, V, w);
  return check_launch("embedding_bwd (sort)");
}

slt_status launch_embedding_bwd(const int32_t* tok, int B, int T_, int64_t ld, const void* dx, float* dwte, int V,
                                int C, int dtype, void* ws, hipStream_t s, GradW gw, Drop drop, bool sorted) {
  const int N = B * T_;
  EmbWs w = emb_ws_layout(ws, N, V, 4096);
  const int ntile = cdiv(N, kEmbTile);
  if (!sorted) {  // else launch_embedding_sort ran on this workspace, ordered before this call
    const slt_status st = launch_embedding_sort(tok, B, T_, ld, V, ws, s);
    if (st != SLT_OK) return st;
  }
  auto go = [&](auto tag) {
    using T = decltype(tag);
    constexpr int VEC = full_vec<T>();
    // float4 stores of the partials and rows need 16-byte aligned rows of
    // dwte and of the workspace's partials (at 256-byte offsets)
    if (C % VEC == 0 && aligned(dx, 16) && aligned(dwte, 16) && aligned(ws, 16) && C % 4 == 0) {
      const int nslab = cdiv(C, kWave * VEC);
      emb_tile_sum_k<T, VEC><<<cdiv(ntile * nslab, 4), 256, 0, s>>>((const T*)dx, dwte, N, V, C, nslab, w, gw, drop);
    } else {
      const int nslab = cdiv(C, kWave);
      emb_tile_sum_k<T, 1><<<cdiv(ntile * nslab, 4), 256, 0, s>>>((const T*)dx, dwte, N, V, C, nslab, w, gw, drop);
    }
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  if (C % 4 == 0 && aligned(dwte, 16) && aligned(ws, 16))  // the partials sit at 256-byte offsets in ws
    emb_row_finish_k<true><<<V, 256, 0, s>>>(dwte, V, C, w, gw);
  else
    emb_row_finish_k<false><<<V, 256, 0, s>>>(dwte, V, C, w, gw);
  return check_launch("embedding_bwd");
}

// out[r, c] = g[r, c] * (dropout multiplier of element r C + c): the
// gradient of a dropped site's pre-dropout value (stored in the activation
// type, as the GEMMs that consume it read it).
template <typename T, int VEC>
__global__ __launch_bounds__(256) void drop_apply_k(const T* __restrict__ g, T* __restrict__ out, int rows, int C,
                                                    Drop drop) {
  const int cv = C / VEC;
  const int64_t total = (int64_t)rows * cv;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / cv;
    const int c = (int)(idx % cv) * VEC;
    float f[VEC], m[VEC];
    load_f<T, VEC>(g + r * C + c, f);
    drop_mults<VEC>(drop, (uint64_t)r * C + c, m);
#pragma unroll
    for (int q = 0; q < VEC; ++q) f[q] *= m[q];
    store_f<T, VEC>(out + r * C + c, f);
  }
}

slt_status launch_drop_apply(const void* g, void* out, int rows, int C, int dtype, Drop drop, hipStream_t s) {
  auto go = [&](auto tag) {
    using T = decltype(tag);
    constexpr int VEC = full_vec<T>();
    if (C % VEC == 0 && aligned(g, 16) && aligned(out, 16))
      drop_apply_k<T, VEC><<<grid_for((int64_t)rows * C / VEC), 256, 0, s>>>((const T*)g, (T*)out, rows, C, drop);
    else
      drop_apply_k<T, 1><<<grid_for((int64_t)rows * C), 256, 0, s>>>((const T*)g, (T*)out, rows, C, drop);
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  return check_launch("dropout (backward)");
}

// Picks VEC (16-byte groups when C allows) and NCH = groups per lane.
template <typename T, typename F>
static slt_status norm_dispatch(int C, bool vec_ok, F&& f) {
  constexpr int FV = full_vec<T>();
  if (vec_ok && C % FV == 0) {
    const int nch = cdiv(C, 64 * FV);
    if (nch <= 1) return f(std::integral_constant<int, FV>{}, std::integral_constant<int, 1>{});
    if (nch <= 2) return f(std::integral_constant<int, FV>{}, std::integral_constant<int, 2>{});
    if (nch <= 4) return f(std::integral_constant<int, FV>{}, std::integral_constant<int, 4>{});
    if (nch <= 8) return f(std::integral_constant<int, FV>{}, std::integral_constant<int, 8>{});
    return fail(SLT_EUNSUPPORTED, "norm: C too large");
  }
  const int nch = cdiv(C, 64);
  if (nch <= 1) return f(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
  if (nch <= 2) return f(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
  if (nch <= 4) return f(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{});
  if (nch <= 8) return f(std::integral_constant<int, 1>{}, std::integral_constant<int, 8>{});
  return fail(SLT_EUNSUPPORTED, "norm: C too large for an unaligned row");
}

slt_status launch_rmsnorm_fwd(const void* x, const void* g, void* y, float* rstd, int rows, int C, float eps,
                              int dtype, hipStream_t s) {
  auto go = [&](auto tag) -> slt_status {
    using T = decltype(tag);
    const bool ok = aligned(x, 16) && aligned(g, 16) && aligned(y, 16);
    return norm_dispatch<T>(C, ok, [&](auto vec, auto nch) -> slt_status {
      rmsnorm_fwd_k<T, decltype(vec)::value, decltype(nch)::value><<<cdiv(rows, 4), 256, 0, s>>>(
          (const T*)x, (const T*)g, (T*)y, rstd, rows, C, eps);
      return check_launch("rmsnorm_fwd");
    });
  };
  return dtype == SLT_BF16 ? go(bf16{}) : go(float{});
}

slt_status launch_layernorm_fwd(const void* x, const void* gm, const void* bt, void* y, float* mean, float* rstd,
                                int rows, int C, float eps, int dtype, hipStream_t s) {
  auto go = [&](auto tag) -> slt_status {
    using T = decltype(tag);
    const bool ok = aligned(x, 16) && aligned(gm, 16) && aligned(bt, 16) && aligned(y, 16);
    return norm_dispatch<T>(C, ok, [&](auto vec, auto nch) -> slt_status {
      layernorm_fwd_k<T, decltype(vec)::value, decltype(nch)::value><<<cdiv(rows, 4), 256, 0, s>>>(
          (const T*)x, (const T*)gm, (const T*)bt, (T*)y, mean, rstd, rows, C, eps);
      return check_launch("layernorm_fwd");
    });
  };
  return dtype == SLT_BF16 ? go(bf16{}) : go(float{});
}

// Blocks of the norm backward for `rows` rows: one partial row of column
// sums per block (the workspace, the backward and the column sums all use it).
static int norm_bwd_blocks(int rows) { return std::max(1, std::min(kNormBwdBlocks, cdiv(rows, kNormBwdWaves))); }

int64_t norm_bwd_ws(int rows, int C) { return (int64_t)2 * norm_bwd_blocks(rows) * C * 4; }

slt_status launch_norm_colsum(const void* ws, int rows, int C, float* dg, float* db, hipStream_t s, GradW gw) {
  const int nb = norm_bwd_blocks(rows);
  const float* part = static_cast<const float*>(ws);
  norm_colsum_k<<<cdiv(C, 32), 1024, 0, s>>>(part, nb, C, dg, gw);
  if (db) norm_colsum_k<<<cdiv(C, 32), 1024, 0, s>>>(part + (int64_t)nb * C, nb, C, db, gw);
  return check_launch("norm_colsum");
}

template <bool LN>
static slt_status norm_bwd_common(const void* x, const void* g, const float* mean, const float* rstd,
                                  const void* dy, const void* dres, void* dx, float* dg, float* db, int rows,
                                  int C, int dtype, void* ws, hipStream_t s, GradW gw, bool defer_sums) {
  const int nb = norm_bwd_blocks(rows);
  float* part = static_cast<float*>(ws);
  const size_t smem = (size_t)(LN ? 2 : 1) * C * sizeof(float);
  auto go = [&](auto tag) -> slt_status {
    using T = decltype(tag);
    const bool ok = aligned(x, 16) && aligned(g, 16) && aligned(dy, 16) && aligned(dres, 16) && aligned(dx, 16);
    return norm_dispatch<T>(C, ok, [&](auto vec, auto nch) -> slt_status {
      norm_bwd_k<T, decltype(vec)::value, decltype(nch)::value, LN, kNormBwdWaves><<<nb, 64 * kNormBwdWaves, smem, s>>>(
          (const T*)x, (const T*)g, mean, rstd, (const T*)dy, (const T*)dres, (T*)dx, part, rows, C);
      return check_launch("norm_bwd");
    });
  };
  slt_status st = dtype == SLT_BF16 ? go(bf16{}) : go(float{});
  if (st != SLT_OK || defer_sums) return st;
  return launch_norm_colsum(ws, rows, C, dg, LN ? db : nullptr, s, gw);
}

slt_status launch_rmsnorm_bwd(const void* x, const void* g, const float* rstd, const void* dy, const void* dres,
                              void* dx, float* dg, int rows, int C, int dtype, void* ws, hipStream_t s, GradW gw,
                              bool defer_sums) {
  return norm_bwd_common<false>(x, g, nullptr, rstd, dy, dres, dx, dg, nullptr, rows, C, dtype, ws, s, gw,
                                defer_sums);
}

slt_status launch_layernorm_bwd(const void* x, const void* gm, const float* mean, const float* rstd,
                                const void* dy, const void* dres, void* dx, float* dgm, float* dbt, int rows,
                                int C, int dtype, void* ws, hipStream_t s, GradW gw, bool defer_sums) {
  return norm_bwd_common<true>(x, gm, mean, rstd, dy, dres, dx, dgm, dbt, rows, C, dtype, ws, s, gw, defer_sums);
}

slt_status launch_rope(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int T_, int nh, int d, int R,
                       int mode, const float* cs, float sign, int dtype, hipStream_t s) {
  if (rows == 0 || nh == 0 || d == 0) return SLT_OK;
  const int64_t work = rows * nh * std::max(R / 2, d - R);
  const int blocks = (int)std::min<int64_t>(cdiv(work, 256), 65536);
  if (dtype == SLT_BF16)
    rope_apply_k<bf16><<<blocks, 256, 0, s>>>(static_cast<const bf16*>(x), ldx, static_cast<bf16*>(y), ldy, rows, T_,
                                              nh, d, R, mode, cs, sign);
  else
    rope_apply_k<float><<<blocks, 256, 0, s>>>(static_cast<const float*>(x), ldx, static_cast<float*>(y), ldy, rows,
                                               T_, nh, d, R, mode, cs, sign);
  return check_launch("rope");
}

slt_status launch_scalar_axpy(float* dst, float a, const float* x, hipStream_t s) {
  scalar_axpy_k<<<1, 1, 0, s>>>(dst, a, x);
  return check_launch("scalar axpy");
}

slt_status launch_rope_table(int T_, int R, float base, float* cs, hipStream_t s) {
  const int n = T_ * (R / 2);
  if (n == 0) return SLT_OK;
  rope_table_k<<<cdiv(n, 256), 256, 0, s>>>(T_, R, (double)base, cs);
  return check_launch("rope_table");
}

// Widest vector (in elements) for the element kernels: 16 bytes, else 8, else
// 4, else single elements -- the first width that divides F and every row
// stride, with every pointer aligned to it.
template <typename T>
static int ew_vec(int F, std::initializer_list<int64_t> lds, std::initializer_list<const void*> ptrs) {
  for (int v = full_vec<T>(); v >= 2; v /= 2) {
    bool ok = F % v == 0;
    for (auto l : lds) ok = ok && l % v == 0;
    for (auto p : ptrs) ok = ok && aligned(p, v * (int)sizeof(T));
    if (ok) return v;
  }
  return 1;
}

// Calls f(std::integral_constant<int, v>) for the width ew_vec chose.
template <typename T, typename Fn>
static void ew_dispatch(int v, Fn&& f) {
  constexpr int FV = full_vec<T>();
  if (v == FV) f(std::integral_constant<int, FV>{});
  else if (v == FV / 2) f(std::integral_constant<int, FV / 2>{});
  else if (FV >= 8 && v == FV / 4) f(std::integral_constant<int, (FV >= 8 ? FV / 4 : 1)>{});
  else f(std::integral_constant<int, 1>{});
}

slt_status launch_swiglu_fwd(const void* a, const void* b, void* h, int rows, int F, int64_t lda, int64_t ldb,
                             int64_t ldh, int dtype, hipStream_t s) {
  auto go = [&](auto tag) {
    using T = decltype(tag);
    ew_dispatch<T>(ew_vec<T>(F, {lda, ldb, ldh}, {a, b, h}), [&](auto vec) {
      constexpr int V = decltype(vec)::value;
      swiglu_fwd_k<T, V><<<grid_for((int64_t)rows * F / V, kEw, 1 << 20), kEw, 0, s>>>((const T*)a, (const T*)b, (T*)h, rows, F,
                                                                         lda, ldb, ldh);
    });
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  return check_launch("swiglu_fwd");
}

slt_status launch_swiglu_bwd(const void* a, const void* b, const void* dh, void* da, void* db, int rows, int F,
                             int64_t lda, int64_t ldb, int64_t lddh, int64_t ldda, int64_t lddb, int dtype,
                             hipStream_t s) {
  auto go = [&](auto tag) {
    using T = decltype(tag);
    ew_dispatch<T>(ew_vec<T>(F, {lda, ldb, lddh, ldda, lddb}, {a, b, dh, da, db}), [&](auto vec) {
      constexpr int V = decltype(vec)::value;
      swiglu_bwd_k<T, V><<<grid_for((int64_t)rows * F / V, kEw, 1 << 20), kEw, 0, s>>>(
          (const T*)a, (const T*)b, (const T*)dh, (T*)da, (T*)db, rows, F, lda, ldb, lddh, ldda, lddb);
    });
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  return check_launch("swiglu_bwd");
}

slt_status launch_gelu_fwd(const void* a, void* u, int rows, int F, int64_t lda, int64_t ldu, int dtype,
                           hipStream_t s) {
  auto go = [&](auto tag) {
    using T = decltype(tag);
    ew_dispatch<T>(ew_vec<T>(F, {lda, ldu}, {a, u}), [&](auto vec) {
      constexpr int V = decltype(vec)::value;
      gelu_fwd_k<T, V><<<grid_for((int64_t)rows * F / V, kEw, 1 << 20), kEw, 0, s>>>((const T*)a, (T*)u, rows, F, lda, ldu);
    });
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  return check_launch("gelu_fwd");
}

slt_status launch_gelu_bwd(const void* a, const void* du, void* da, int rows, int F, int64_t lda, int64_t lddu,
                           int64_t ldda, int dtype, hipStream_t s) {
  auto go = [&](auto tag) {
    using T = decltype(tag);
    ew_dispatch<T>(ew_vec<T>(F, {lda, lddu, ldda}, {a, du, da}), [&](auto vec) {
      constexpr int V = decltype(vec)::value;
      gelu_bwd_k<T, V><<<grid_for((int64_t)rows * F / V, kEw, 1 << 20), kEw, 0, s>>>((const T*)a, (const T*)du, (T*)da, rows, F,
                                                                       lda, lddu, ldda);
    });
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  return check_launch("gelu_bwd");
}

slt_status launch_softmax_xent(void* z, int64_t ldz, const int32_t* tok, int B, int T_, int64_t ld, int V,
                               float* loss, float* lse, int dtype, void* ws, hipStream_t s) {
  const int rows = B * T_;
  float* rowloss = static_cast<float*>(ws);
  auto go = [&](auto tag) {
    using T = decltype(tag);
    constexpr int FV = full_vec<T>();
    const bool vec = V % FV == 0 && ldz % FV == 0 && aligned(z, 16);
    if constexpr (sizeof(T) == 2) {
      const int nit = cdiv(V, 2048);  // 16-byte groups per thread
      auto reg = [&](auto n) {
        xent_rows_reg_k<decltype(n)::value><<<rows, 256, 0, s>>>((bf16*)z, ldz, tok, T_, ld, V, rows, rowloss, lse);
      };
      // register footprint follows the row length (occupancy 8 .. 2)
      if (vec && nit > 2 && nit <= 8) return reg(std::integral_constant<int, 8>{});
      if (vec && nit > 8 && nit <= 16) return reg(std::integral_constant<int, 16>{});
      if (vec && nit > 16 && nit <= 20) return reg(std::integral_constant<int, 20>{});
      if (vec && nit > 20 && nit <= 26) return reg(std::integral_constant<int, 26>{});
      if (vec && nit > 26 && nit <= 32) return reg(std::integral_constant<int, 32>{});
    }
    if (vec)
      xent_rows_k<T, FV><<<rows, 256, 0, s>>>((T*)z, ldz, tok, T_, ld, V, rows, rowloss, lse);
    else
      xent_rows_k<T, 1><<<rows, 256, 0, s>>>((T*)z, ldz, tok, T_, ld, V, rows, rowloss, lse);
  };
  if (dtype == SLT_BF16) go(bf16{}); else go(float{});
  xent_mean_k<<<1, 1024, 0, s>>>(rowloss, rows, loss);
  return check_launch("softmax_xent");
}

slt_status launch_adamw(int64_t n, float* master, uint16_t* shadow, const float* g, float* m, float* v, int64_t t,
                        float lr, float b1, float b2, float eps, float wd, const uint8_t* mask, const float* gscale,
                        hipStream_t s) {
  const double bc1 = 1.0 - pow((double)b1, (double)t);
  const double bc2 = 1.0 - pow((double)b2, (double)t);
  adamw_k<<<grid_for(n / 4 + 1, kEw, 1 << 20), kEw, 0, s>>>(n, master, shadow, g, m, v, b1, b2, (float)(1.0 / bc1),
                                                           (float)(1.0 / bc2), lr, eps, wd, mask, gscale);
  return check_launch("adamw");
}

int64_t grad_norm_ws() { return kGnBlocks * (int64_t)sizeof(double); }

slt_status launch_grad_norm(int64_t n, const float* g, int kind, float max_norm, float* norm, float* scale, void* ws,
                            hipStream_t s) {
  double* part = static_cast<double*>(ws);
  if (kind == SLT_NORM_LINF) {
    gnorm_partial_k<true><<<kGnBlocks, 256, 0, s>>>(n, g, part);
    gnorm_final_k<true><<<1, 1024, 0, s>>>(part, max_norm, norm, scale);
  } else {
    gnorm_partial_k<false><<<kGnBlocks, 256, 0, s>>>(n, g, part);
    gnorm_final_k<false><<<1, 1024, 0, s>>>(part, max_norm, norm, scale);
  }
  return check_launch("grad_norm");
}

slt_status launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  cast_bf16_k<<<grid_for(n / 4 + 1, 256, 8192), 256, 0, s>>>(src, dst, n);
  return check_launch("cast_bf16");
}

slt_status launch_fill_f32(float* dst, float value, int64_t n, hipStream_t s) {
  fill_f32_k<<<grid_for(n, 256, 8192), 256, 0, s>>>(dst, value, n);
  return check_launch("fill_f32");
}

slt_status launch_model_init_range(float* dst, int64_t n, int64_t index0, uint64_t seed, float std, int kind,
                                   hipStream_t s) {
  model_init_k<<<grid_for(n, 256, 8192), 256, 0, s>>>(dst, n, index0, (uint32_t)seed, (uint32_t)(seed >> 32), std,
                                                      kind);
  return check_launch("model_init");
}

}  // namespace slt

extern "C" void slt_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  slt::philox4x32_10(ctr, key, out);
}
