// Causal attention for bf16 activations, head dim d <= 64 with d % 16 == 0
// (Hephaistos, "Architecture at a glance": RoPE applied to q and k inside
// attention, causal multi-head attention with a numerically stable softmax;
// strata: flash-style attention with online softmax, forward and backward,
// no T x T score matrix, MHA/GQA through independent n_head and n_kv_head).
//
// Work split:
//  * fl_prep_k rotates q and k once (RoPE, fp32) and stores each rotated
//    value as a bf16 pair hi + lo (lo = bf16(x - hi)) in head-major copies
//    [B][heads][T][d] (tiles zero-pad them to 64 dims); the query copy also carries
//    the factor log2(e)/sqrt(d), so that q.k comes out as the score in base-2
//    units the softmax exponentiates.  The attention kernels then
//    only copy tiles: every tile (64 rows x 64 dims, 8 KiB) goes HBM -> LDS
//    with global_load_lds_dwordx4, double-buffered, no register staging.
//  * MFMA v_mfma_f32_16x16x32_bf16: operand A lane (g = l/16, i = l%16)
//    holds A[row i][k 8g..8g+7], B holds B[k 8g..8g+7][col i], the result
//    lane holds C[row 4g+r][col i], r = 0..3.  Computing S^T = K Q^T leaves
//    each lane four consecutive keys of one query; two neighbouring 16-key
//    results give the 8 k-values a lane supplies to the next product, in the
//    order (keys 4g..4g+3 of the first, then of the second) -- a fixed
//    permutation of k that the other operand follows by reading its rows in
//    the same order.  That other operand is the transpose of a staged tile
//    (V^T, K^T, Q^T, dO^T): ds_read_b64_tr_b16 gives lane 16g+i element j
//    of the 8-byte row addressed by lane 16g+4j+i/4, at position i%4, so
//    lane 16g+4j+q addresses (row 4g+j, dims 4q..4q+3) of the tile.
//  * Precision: the rotated q and k and the score gradient dS enter their
//    products as hi + lo pairs (three MFMAs: hi*hi + hi*lo + lo*hi), since a
//    single bf16 rounding of either leaves errors proportional to the mean
//    key (query) instead of the result; P enters P V once and P^T dO (a sum
//    over every query of a KV head's group) as hi + lo.
//    D = dO.O uses O plus its stored bf16 rounding residual.
//  * Tiles: 64 queries (or keys) per workgroup, 16 per wave; LDS tile rows
//    are 8 chunks of 16 bytes with chunk position XOR 2((row >> 1) & 3), so
//    both the row-fragment reads (ds_read_b128) and the transposing reads
//    spread over all banks.  LDS reads are asm blocks that wait for their
//    own results: the compiler cannot tell which buffer an in-flight
//    global_load_lds targets and would otherwise wait for all of them.
#include "slt_internal.h"

#include <math.h>

#include <type_traits>

namespace slt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int FD = 64;                // padded head dim of LDS tiles
constexpr int FR = 64;                // rows per tile and per workgroup
constexpr int FTB = FR * FD * 2;      // bytes per LDS tile (8 KiB)
constexpr int FS = FD + 4;            // fp32 row stride of the epilogue staging tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16 zero bytes in device memory: the copy source of padding chunks.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ u32x4 cat(const u32x2& lo, const u32x2& hi) { return u32x4{lo[0], lo[1], hi[0], hi[1]}; }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf_hi(float x) { return __uint_as_float((uint32_t)f32_to_bf16_bits(x) << 16); }

// Maximum and sum over the four lanes l, l^16, l^32, l^48 (the lanes holding
// one query's keys) with gfx950's v_permlane32_swap / v_permlane16_swap: with
// both operands equal, the swap leaves each lane its own value in one result
// and its partner's in the other, so no LDS round trip is needed.
__device__ __forceinline__ float max4lanes(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum4lanes(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Work item of this block: consecutive block ids go round-robin to the 8
// XCDs, so the id is remapped to give each XCD one contiguous range of work
// items -- the tiles of one (batch, head) then share that XCD's L2.
__device__ __forceinline__ int fl_work_item() {
  const int n = gridDim.x, id = blockIdx.x;
  const int q = n >> 3, r = n & 7, x = id & 7;
  return x * q + min(x, r) + (id >> 3);
}

// chunk position of logical chunk c in row r of a tile
__device__ __forceinline__ int fsw(int r) { return 2 * ((r >> 1) & 3); }

// Copy rows row0..row0+63 (rows >= nrows read row nrows-1) of a bf16 array
// whose row t starts at g + t*ld into an LDS tile; chunks >= nch are zero.
// Two copies per lane (512 chunks over 256 lanes).
__device__ __forceinline__ void fl_issue(const bf16* g, int64_t ld, int row0, int nrows, int nch, char* tile,
                                         int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = (wave * 2 + i) * 64 + lane;
    const int r = p >> 3;
    const int c = (p & 7) ^ fsw(r);
    const void* src = c < nch ? static_cast<const void*>(g + (int64_t)min(row0 + r, nrows - 1) * ld + c * 8)
                              : static_cast<const void*>(g_zero16);
    lds_copy16(src, tile + (wave * 2 + i) * 1024);
  }
}

// Lane byte offsets inside a tile.  Row fragments (ds_read_b128): row i,
// dims 32s + 8g..+7 (s = 0, 1); the 16-row subtile t adds 2048 t.
// Column fragments (ds_read_b64_tr_b16) of dims 16 dt..16 dt+15: lane
// 16g+4j+q addresses row 4g+j, dims 16 dt + 4q..+3; rows +16 add 2048,
// rows +32 add 4096.
struct FlOff {
  unsigned row[2], col[4];
  __device__ __forceinline__ FlOff(int lane) {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int s = 0; s < 2; ++s) row[s] = i * 128 + (((4 * s + g) ^ fsw(i)) * 16);
    const int j = (lane >> 2) & 3, q = lane & 3;
    const int r = 4 * g + j;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) col[dt] = r * 128 + (((2 * dt + (q >> 1)) ^ fsw(r)) * 16) + (q & 1) * 8;
  }
};

#define FL_R128(o, a, off) "ds_read_b128 %[" #o "], %[" #a "] offset:" #off "\n\t"
#define FL_RTR(o, a, off) "ds_read_b64_tr_b16 %[" #o "], %[" #a "] offset:" #off "\n\t"
#define FL_O(n, x) [n] "=&v"(x)

// Row fragments of one tile at byte address t0: f[t][s], t = 0..3.
__device__ __forceinline__ void rd_rows8(unsigned a0, unsigned a1, u32x4 (&f)[4][2]) {
  asm volatile(FL_R128(f00, a0, 0) FL_R128(f01, a1, 0) FL_R128(f10, a0, 2048) FL_R128(f11, a1, 2048)
                   FL_R128(f20, a0, 4096) FL_R128(f21, a1, 4096) FL_R128(f30, a0, 6144) FL_R128(f31, a1, 6144)
               "s_waitcnt lgkmcnt(0)"
               : FL_O(f00, f[0][0]), FL_O(f01, f[0][1]), FL_O(f10, f[1][0]), FL_O(f11, f[1][1]), FL_O(f20, f[2][0]),
                 FL_O(f21, f[2][1]), FL_O(f30, f[3][0]), FL_O(f31, f[3][1])
               : [a0] "v"(a0), [a1] "v"(a1)
               : "memory");
}

// Row fragments of two tiles 8 KiB apart (hi at a, lo at a + 8192): f[hl][t][s].
__device__ __forceinline__ void rd_rows16(unsigned a0, unsigned a1, u32x4 (&f)[2][4][2]) {
  asm volatile(FL_R128(h00, a0, 0) FL_R128(h01, a1, 0) FL_R128(h10, a0, 2048) FL_R128(h11, a1, 2048)
                   FL_R128(h20, a0, 4096) FL_R128(h21, a1, 4096) FL_R128(h30, a0, 6144) FL_R128(h31, a1, 6144)
                       FL_R128(l00, a0, 8192) FL_R128(l01, a1, 8192) FL_R128(l10, a0, 10240)
                           FL_R128(l11, a1, 10240) FL_R128(l20, a0, 12288) FL_R128(l21, a1, 12288)
                               FL_R128(l30, a0, 14336) FL_R128(l31, a1, 14336) "s_waitcnt lgkmcnt(0)"
               : FL_O(h00, f[0][0][0]), FL_O(h01, f[0][0][1]), FL_O(h10, f[0][1][0]), FL_O(h11, f[0][1][1]),
                 FL_O(h20, f[0][2][0]), FL_O(h21, f[0][2][1]), FL_O(h30, f[0][3][0]), FL_O(h31, f[0][3][1]),
                 FL_O(l00, f[1][0][0]), FL_O(l01, f[1][0][1]), FL_O(l10, f[1][1][0]), FL_O(l11, f[1][1][1]),
                 FL_O(l20, f[1][2][0]), FL_O(l21, f[1][2][1]), FL_O(l30, f[1][3][0]), FL_O(l31, f[1][3][1])
               : [a0] "v"(a0), [a1] "v"(a1)
               : "memory");
}

// Column fragments of one tile: f[dt][c] = rows 32c + (4g..4g+3, then
// 16 + 4g..4g+3) at dims 16 dt + i, dt = 0..3, c = 0..1.  cK = address of
// the tile plus the lane's col[dt].
__device__ __forceinline__ void rd_cols16(unsigned c0, unsigned c1, unsigned c2, unsigned c3, u32x4 (&f)[4][2]) {
  u32x2 x[4][2][2];
  asm volatile(FL_RTR(x000, c0, 0) FL_RTR(x001, c0, 2048) FL_RTR(x010, c0, 4096) FL_RTR(x011, c0, 6144)
                   FL_RTR(x100, c1, 0) FL_RTR(x101, c1, 2048) FL_RTR(x110, c1, 4096) FL_RTR(x111, c1, 6144)
                       FL_RTR(x200, c2, 0) FL_RTR(x201, c2, 2048) FL_RTR(x210, c2, 4096) FL_RTR(x211, c2, 6144)
                           FL_RTR(x300, c3, 0) FL_RTR(x301, c3, 2048) FL_RTR(x310, c3, 4096)
                               FL_RTR(x311, c3, 6144) "s_waitcnt lgkmcnt(0)"
               : FL_O(x000, x[0][0][0]), FL_O(x001, x[0][0][1]), FL_O(x010, x[0][1][0]), FL_O(x011, x[0][1][1]),
                 FL_O(x100, x[1][0][0]), FL_O(x101, x[1][0][1]), FL_O(x110, x[1][1][0]), FL_O(x111, x[1][1][1]),
                 FL_O(x200, x[2][0][0]), FL_O(x201, x[2][0][1]), FL_O(x210, x[2][1][0]), FL_O(x211, x[2][1][1]),
                 FL_O(x300, x[3][0][0]), FL_O(x301, x[3][0][1]), FL_O(x310, x[3][1][0]), FL_O(x311, x[3][1][1])
               : [c0] "v"(c0), [c1] "v"(c1), [c2] "v"(c2), [c3] "v"(c3)
               : "memory");
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) f[dt][c] = cat(x[dt][c][0], x[dt][c][1]);
}
// K row fragments of one 32-key half (16-key groups tt = 0, 1) of a hi tile
// and of the lo tile 8 KiB after it: f[hl][tt][s].  a0 / a1 = tile address
// plus the lane's row[0] / row[1] plus 4096 per half.
__device__ __forceinline__ void rd_khalf(unsigned a0, unsigned a1, u32x4 (&f)[2][2][2]) {
  asm volatile(FL_R128(h00, a0, 0) FL_R128(h01, a1, 0) FL_R128(h10, a0, 2048) FL_R128(h11, a1, 2048)
                   FL_R128(l00, a0, 8192) FL_R128(l01, a1, 8192) FL_R128(l10, a0, 10240)
                       FL_R128(l11, a1, 10240) "s_waitcnt lgkmcnt(0)"
               : FL_O(h00, f[0][0][0]), FL_O(h01, f[0][0][1]), FL_O(h10, f[0][1][0]), FL_O(h11, f[0][1][1]),
                 FL_O(l00, f[1][0][0]), FL_O(l01, f[1][0][1]), FL_O(l10, f[1][1][0]), FL_O(l11, f[1][1][1])
               : [a0] "v"(a0), [a1] "v"(a1)
               : "memory");
}

// Row fragments of one 32-row half of one tile: f[tt][s] (a0 / a1 as for
// rd_khalf).
__device__ __forceinline__ void rd_rows4(unsigned a0, unsigned a1, u32x4 (&f)[2][2]) {
  asm volatile(FL_R128(f00, a0, 0) FL_R128(f01, a1, 0) FL_R128(f10, a0, 2048) FL_R128(f11, a1, 2048)
               "s_waitcnt lgkmcnt(0)"
               : FL_O(f00, f[0][0]), FL_O(f01, f[0][1]), FL_O(f10, f[1][0]), FL_O(f11, f[1][1])
               : [a0] "v"(a0), [a1] "v"(a1)
               : "memory");
}

// Column fragments of one 32-row half of a tile: f[dt] = rows 32 hf +
// (4g..4g+3, then 16 + 4g..4g+3) at dims 16 dt + i.  cK = tile address plus
// the lane's col[dt] plus 4096 hf.
__device__ __forceinline__ void rd_chalf(unsigned c0, unsigned c1, unsigned c2, unsigned c3, u32x4 (&f)[4]) {
  u32x2 x[4][2];
  asm volatile(FL_RTR(x00, c0, 0) FL_RTR(x01, c0, 2048) FL_RTR(x10, c1, 0) FL_RTR(x11, c1, 2048)
                   FL_RTR(x20, c2, 0) FL_RTR(x21, c2, 2048) FL_RTR(x30, c3, 0) FL_RTR(x31, c3, 2048)
                       "s_waitcnt lgkmcnt(0)"
               : FL_O(x00, x[0][0]), FL_O(x01, x[0][1]), FL_O(x10, x[1][0]), FL_O(x11, x[1][1]),
                 FL_O(x20, x[2][0]), FL_O(x21, x[2][1]), FL_O(x30, x[3][0]), FL_O(x31, x[3][1])
               : [c0] "v"(c0), [c1] "v"(c1), [c2] "v"(c2), [c3] "v"(c3)
               : "memory");
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) f[dt] = cat(x[dt][0], x[dt][1]);
}
#undef FL_R128
#undef FL_RTR
#undef FL_O

__device__ __forceinline__ void rd_cols(unsigned base, const FlOff& o, u32x4 (&f)[4][2]) {
  rd_cols16(base + o.col[0], base + o.col[1], base + o.col[2], base + o.col[3], f);
}

// (x, y) -> bf16 pairs hi = (bf16(x), bf16(y)) and lo = (bf16(x - hi.x),
// bf16(y - hi.y)): two conversions, two subtractions.
__device__ __forceinline__ void split2(float x, float y, uint32_t& hi, uint32_t& lo) {
  hi = f32x2_to_bf16x2_bits(x, y);
  lo = f32x2_to_bf16x2_bits(x - __uint_as_float(hi << 16), y - __uint_as_float(hi & 0xffff0000u));
}

// Four probabilities (or gradients) of two neighbouring 16-row results in
// the k order the transposed reads use.
__device__ __forceinline__ u32x4 pack_k(const float (&x)[4], const float (&y)[4]) {
  return u32x4{f32x2_to_bf16x2_bits(x[0], x[1]), f32x2_to_bf16x2_bits(x[2], x[3]), f32x2_to_bf16x2_bits(y[0], y[1]),
               f32x2_to_bf16x2_bits(y[2], y[3])};
}
__device__ __forceinline__ void pack_k_hilo(const float (&x)[4], const float (&y)[4], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
  split2(x[0], x[1], h[0], l[0]);
  split2(x[2], x[3], h[1], l[1]);
  split2(y[0], y[1], h[2], l[2]);
  split2(y[2], y[3], h[3], l[3]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

struct FlArgs {
  const bf16 *qh, *ql, *kh, *kl;  // rotated copies [B][H | Hkv][T][64]
  const bf16* v;                  // row (b, t) at v + (b T + t) ldv, head kvh at + kvh d
  const bf16 *o, *ores, *dout;    // [B T] rows: o (ldo), ores (ldores), dout (lddo)
  bf16 *out, *ores_out, *dq, *dk, *dv;
  float* lse;
  const float* lse_in;
  float* delta;
  const float* cs;
  int64_t ldv, ldo, ldores, lddo, lddq, lddk, lddv;
  int B, T, H, Hkv, d, R, rope_mode;
  Drop drop;                      // dropout of the attention weights (att_elem)
};

// ---------------------------------------------------------------------------
// RoPE once: q and k heads -> hi/lo rotated copies.  Item = (b, t, head
// slot, 8-dim chunk); slots 0..H-1 are query heads, H..H+Hkv-1 key heads.
// VEC: every chunk is wholly rotated or wholly past R and its partner chunk
// is 16-byte aligned ((R/2) % 8 == 0 for rotate-half, R % 8 == 0 for
// pairs), so a chunk is three 16-byte loads (own, partner, table) and two
// 16-byte stores; otherwise element by element.
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(128) void fl_prep_k(const bf16* __restrict__ q, int64_t ldq, const bf16* __restrict__ k,
                                                 int64_t ldk, bf16* qh, bf16* ql, bf16* kh, bf16* kl, int B, int T,
                                                 int H, int Hkv, int d, int R, int mode, const float* cs,
                                                 float qscale) {
  // grid (B T, ceil(d/8 (H + Hkv) / 128)): one token per block row, one
  // (head slot, 8-dim chunk) per thread
  const int slots = H + Hkv, nch = d / 8;
  const int j = blockIdx.y * blockDim.x + threadIdx.x;
  if (j < slots * nch) {
    const int c = j % nch;
    const int slot = j / nch;
    const int64_t bt = blockIdx.x;
    const int t = (int)(bt % T), b = (int)(bt / T);
    const bool isq = slot < H;
    const int hd = isq ? slot : slot - H;
    const int64_t drow = ((int64_t)(b * (isq ? H : Hkv) + hd) * T + t) * d + c * 8;
    bf16* dh = (isq ? qh : kh) + drow;
    bf16* dl = (isq ? ql : kl) + drow;
    uint32_t hw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
    const int j0 = c * 8;
    if (j0 < d) {
      const bf16* u = isq ? q + bt * ldq + (int64_t)hd * d : k + bt * ldk + (int64_t)hd * d;
      float x[8];
      if (VEC) {
        const uint4 own = *reinterpret_cast<const uint4*>(u + j0);
        const uint32_t ow[4] = {own.x, own.y, own.z, own.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(ow[e] << 16);
          x[2 * e + 1] = __uint_as_float(ow[e] & 0xffff0000u);
        }
        if (j0 < R) {
          const float* tb = cs + (int64_t)t * R;
          if (mode == SLT_ROPE_HALF) {
            const int hr = R >> 1;
            const bool first = j0 < hr;
            const int i0 = first ? j0 : j0 - hr;
            const uint4 par = *reinterpret_cast<const uint4*>(u + (first ? j0 + hr : j0 - hr));
            const uint32_t pw[4] = {par.x, par.y, par.z, par.w};
            const float4* t4 = reinterpret_cast<const float4*>(tb + 2 * i0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float4 cs2 = t4[e];  // (cos, sin) of dims i0 + 2e, i0 + 2e + 1
              const float y0 = __uint_as_float(pw[e] << 16), y1 = __uint_as_float(pw[e] & 0xffff0000u);
              const float x0 = x[2 * e], x1 = x[2 * e + 1];
              x[2 * e] = first ? x0 * cs2.x - y0 * cs2.y : x0 * cs2.x + y0 * cs2.y;
              x[2 * e + 1] = first ? x1 * cs2.z - y1 * cs2.w : x1 * cs2.z + y1 * cs2.w;
            }
          } else {
            const float4* t4 = reinterpret_cast<const float4*>(tb + j0);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float4 cs2 = t4[e];  // pairs (j0 + 4e, +1) and (j0 + 4e + 2, +3)
              const float a0 = x[4 * e], a1 = x[4 * e + 1], b0 = x[4 * e + 2], b1 = x[4 * e + 3];
              x[4 * e] = a0 * cs2.x - a1 * cs2.y;
              x[4 * e + 1] = a1 * cs2.x + a0 * cs2.y;
              x[4 * e + 2] = b0 * cs2.z - b1 * cs2.w;
              x[4 * e + 3] = b1 * cs2.z + b0 * cs2.w;
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e;
          float v = to_f32(u[j]);
          if (j < R) {
            int ii, p;
            bool first;
            if (mode == SLT_ROPE_HALF) {
              const int hr = R >> 1;
              first = j < hr;
              ii = first ? j : j - hr;
              p = first ? j + hr : j - hr;
            } else {
              first = (j & 1) == 0;
              ii = j >> 1;
              p = j ^ 1;
            }
            const float cth = cs[(int64_t)t * R + 2 * ii], sth = cs[(int64_t)t * R + 2 * ii + 1];
            const float y = to_f32(u[p]);
            v = first ? v * cth - y * sth : v * cth + y * sth;
          }
          x[e] = v;
        }
      }
      if (isq) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= qscale;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], hw[e], lw[e]);
    }
    *reinterpret_cast<uint4*>(dh) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(dl) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// ---------------------------------------------------------------------------
// Forward, one workgroup per (64 FNS-query chunk, head, batch), longest
// chunks first.  Wave w owns the 16-query subtiles u = w, w+4, .., w+4(FNS-1)
// of the chunk, their rotated queries held as MFMA fragments in registers.  Key /
// value tiles of 64 rows stream through a three-stage LDS ring ([K hi | K lo
// | V] per stage, two tiles in flight while one is used); each 32-key half
// is read from LDS once per wave and applied to all of the wave's subtiles
// that reach it, so a tile is fetched once per chunk and its fragments once
// per wave.  Per subtile and half: S^T = K Q^T (hi/lo), online softmax in
// base 2, O^T += V^T P^T.  Subtile u needs key tile j iff 64 j <= 16 u + 15
// (chunk-relative), i.e. subtile i of a wave from tile i on, so every wave
// does the same work.
// ---------------------------------------------------------------------------

template <bool DROP, int FNS>
__global__ __launch_bounds__(256, 2) void fl_fwd2_k(FlArgs a) {
  constexpr int FC = 64 * FNS;  // queries per chunk
  __shared__ __attribute__((aligned(16))) char lds[3][3 * FTB];
  const int T = a.T, nck = (T + FC - 1) / FC;
  const int w = fl_work_item();
  const int ck = nck - 1 - w % nck, h = (w / nck) % a.H, b = w / (nck * a.H);
  const int c0 = ck * FC, kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int nch = a.d / 8;
  const FlOff off(lane);

  // subtile i of this wave: queries c0 + 16 (wave + 4 i) + li
  u32x4 qh[FNS][2], ql[FNS][2];
  const int64_t qb = (int64_t)(b * a.H + h) * T;
#pragma unroll
  for (int i = 0; i < FNS; ++i) {
    const int qc = min(c0 + 16 * (wave + 4 * i) + li, T - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int j0 = 32 * s + 8 * g;
      qh[i][s] = ql[i][s] = u32x4{0u, 0u, 0u, 0u};
      if (j0 < a.d) {
        qh[i][s] = *reinterpret_cast<const u32x4*>(a.qh + (qb + qc) * a.d + j0);
        ql[i][s] = *reinterpret_cast<const u32x4*>(a.ql + (qb + qc) * a.d + j0);
      }
    }
  }
  const int64_t kbase = (int64_t)(b * a.Hkv + kvh) * T * a.d;
  const bf16* kh = a.kh + kbase;
  const bf16* kl = a.kl + kbase;
  const bf16* vb = a.v + (int64_t)b * T * a.ldv + (int64_t)kvh * a.d;

  f32x4 oacc[FNS][4];
  float m[FNS], l[FNS];
#pragma unroll
  for (int i = 0; i < FNS; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // key tiles 0 .. nt-1 cover keys up to the chunk's last query
  const int nt = (min(T, c0 + FC) + FR - 1) / FR;
  auto issue = [&](int j, char* st) {
    fl_issue(kh, a.d, j * FR, T, nch, st, wave, lane);
    fl_issue(kl, a.d, j * FR, T, nch, st + FTB, wave, lane);
    fl_issue(vb, a.ldv, j * FR, T, nch, st + 2 * FTB, wave, lane);
  };
  issue(0, lds[0]);
  issue(min(1, nt - 1), lds[1]);  // past the end: tile 0 again, into a stage nobody reads
  for (int j = 0; j < nt; ++j) {
    SLT_WAIT_VMCNT(6);  // only the copies of tile j+1 may still fly
    lds_barrier();
    issue(min(j + 2, nt - 1), lds[(j + 2) % 3]);
    const unsigned base = lds_off(lds[j % 3]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int k0 = j * FR + 32 * hf;  // first key of this half
      // subtiles whose last query reaches this half (uniform over the wave)
      if (k0 > c0 + 16 * (wave + 4 * (FNS - 1)) + 15 || k0 >= T) break;
      u32x4 kf[2][2][2], vf[4];
      rd_khalf(base + off.row[0] + 4096 * hf, base + off.row[1] + 4096 * hf, kf);
      rd_chalf(base + 2 * FTB + off.col[0] + 4096 * hf, base + 2 * FTB + off.col[1] + 4096 * hf,
               base + 2 * FTB + off.col[2] + 4096 * hf, base + 2 * FTB + off.col[3] + 4096 * hf, vf);
#pragma unroll
      for (int i = 0; i < FNS; ++i) {
        const int u0 = c0 + 16 * (wave + 4 * i);  // first query of subtile i
        if (k0 > u0 + 15 || u0 >= T) continue;
        const int qi = u0 + li;
        float sv[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            st = mma(kf[0][tt][s], qh[i][s], st);
            st = mma(kf[0][tt][s], ql[i][s], st);
            st = mma(kf[1][tt][s], qh[i][s], st);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[tt][r] = st[r];
          if (k0 + 31 > u0) {  // keys after a query of the subtile are masked
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (k0 + 16 * tt + 4 * g + r > qi) sv[tt][r] = -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sv[tt][r]);
        }
        // The running maximum moves only where a row's new maximum exceeds it
        // by more than 8 (base 2), so the weights stay below 2^8; a wave whose
        // rows all keep theirs skips rescaling its accumulators.  (The first
        // half processed holds key 0, which no query masks, so m is finite
        // from then on.)
        const float mt = max4lanes(tmax);
        const bool grow = mt > m[i] + 8.f;
        if (__ballot(grow) != 0) {
          const float mn = grow ? mt : m[i];
          const float alpha = ex2(m[i] - mn);  // 1 where the maximum stays, 0 on the first half
          l[i] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[i][dt] *= alpha;
          m[i] = mn;
        }
        float rs = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sv[tt][r] = ex2(sv[tt][r] - m[i]);
            rs += sv[tt][r];
          }
        l[i] += rs;  // this lane's keys only; the four lanes are summed at the end
        if (DROP) {  // the normaliser keeps every weight; the values see the dropped ones
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            float dm[4];
            drop_mults<4>(a.drop, att_elem(b, a.H, h, T, qi, k0 + 16 * tt + 4 * g), dm);
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[tt][r] *= dm[r];
          }
        }
        const u32x4 pb = pack_k(sv[0], sv[1]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[i][dt] = mma(vf[dt], pb, oacc[i][dt]);
      }
    }
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends

#pragma unroll
  for (int i = 0; i < FNS; ++i) l[i] = sum4lanes(l[i]);
#pragma unroll
  for (int i = 0; i < FNS; ++i) {
    const int qi = c0 + 16 * (wave + 4 * i) + li;
    if (qi >= T) continue;
    const float inv = 1.0f / l[i];
    bf16* ob = a.out + ((int64_t)b * T + qi) * a.ldo + (int64_t)h * a.d;
    bf16* rb = a.ores_out ? a.ores_out + ((int64_t)b * T + qi) * a.ldores + (int64_t)h * a.d : nullptr;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int j0 = 16 * dt + 4 * g;
      if (j0 >= a.d) continue;
      float v[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = oacc[i][dt][r] * inv;
        lo[r] = v[r] - bf_hi(v[r]);
      }
      *reinterpret_cast<u32x2*>(ob + j0) = u32x2{f32x2_to_bf16x2_bits(v[0], v[1]), f32x2_to_bf16x2_bits(v[2], v[3])};
      if (rb)
        *reinterpret_cast<u32x2*>(rb + j0) =
            u32x2{f32x2_to_bf16x2_bits(lo[0], lo[1]), f32x2_to_bf16x2_bits(lo[2], lo[3])};
    }
    if (g == 0) a.lse[((int64_t)b * a.H + h) * T + qi] = (m[i] + log2f(l[i])) * kLn2;
  }
}

// fp32 [64][FS] tile in LDS -> bf16 rows row0.. of out (row t at out + t ld),
// scaled, rotated back by RoPE when R > 0 (the transpose of the forward
// rotation: the gradient of the rotated copy is the rotated-back gradient).
__device__ __forceinline__ void fl_store_rows(const float* F, float scale, bf16* out, int64_t ld, int row0, int T,
                                              int d, int R, int mode, const float* cs, int nrows = FR) {
  const int ng = d / 4;
  for (int idx = threadIdx.x; idx < nrows * ng; idx += blockDim.x) {
    const int r = idx / ng, j0 = (idx % ng) * 4;
    const int t = row0 + r;
    if (t >= T) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = F[r * FS + j0 + e];
    const int hr = R >> 1;
    if (j0 < R && !(j0 + 4 <= R && (mode != SLT_ROPE_HALF || j0 + 4 <= hr || j0 >= hr))) {
      // the group straddles R or (rotate-half) the middle of the rotated
      // dims: one element at a time
      const float* tb = cs + (int64_t)t * R;
      float w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + e;
        w[e] = v[e];
        if (j >= R) continue;
        if (mode == SLT_ROPE_HALF) {
          const bool first = j < hr;
          const int i = first ? j : j - hr;
          const float c = tb[2 * i], s = tb[2 * i + 1], y = F[r * FS + (first ? j + hr : j - hr)];
          w[e] = first ? v[e] * c + y * s : v[e] * c - y * s;
        } else {
          const float c = tb[j & ~1], s = tb[(j & ~1) + 1];
          w[e] = (j & 1) == 0 ? v[e] * c + F[r * FS + j + 1] * s : v[e] * c - F[r * FS + j - 1] * s;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = w[e];
    } else if (j0 < R) {
      const float* tb = cs + (int64_t)t * R;
      if (mode == SLT_ROPE_HALF) {
        const bool first = j0 < hr;
        const int i0 = first ? j0 : j0 - hr, p0 = first ? j0 + hr : j0 - hr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = tb[2 * (i0 + e)], s = tb[2 * (i0 + e) + 1];
          const float x = v[e], y = F[r * FS + p0 + e];
          v[e] = first ? x * c + y * s : x * c - y * s;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float c = tb[j0 + e], s = tb[j0 + e + 1];
          const float x = v[e], y = v[e + 1];
          v[e] = x * c + y * s;
          v[e + 1] = y * c - x * s;
        }
      }
    }
    *reinterpret_cast<u32x2*>(out + (int64_t)t * ld + j0) =
        u32x2{f32x2_to_bf16x2_bits(v[0] * scale, v[1] * scale), f32x2_to_bf16x2_bits(v[2] * scale, v[3] * scale)};
  }
}

// Accumulators acc[dt] (lane: dims 16 dt + 4g + r of row `row`) -> F[row][dims].
__device__ __forceinline__ void fl_stage_acc(float* F, int row, int g, const f32x4 (&acc)[4]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    *reinterpret_cast<float4*>(F + row * FS + 16 * dt + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2],
                                                                             acc[dt][3]);
}

// ---------------------------------------------------------------------------
// dQ (and D).  One workgroup per (query tile, head, batch).  Wave w owns queries q0 + 16w + i:
// D = dO.(O + ores); per key tile: S^T = K Q^T, P^T = exp2(S^T - lse),
// dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (hi/lo).
// LDS stage: [K hi | K lo | V], two stages.
// ---------------------------------------------------------------------------
template <bool DROP>
__global__ __launch_bounds__(256) void fl_dq_k(FlArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2][3 * FTB];
  const int T = a.T, ntq = (T + FR - 1) / FR;
  const int w = fl_work_item();
  const int qt = ntq - 1 - w % ntq, h = (w / ntq) % a.H, b = w / (ntq * a.H);
  const int q0 = qt * FR, kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int qi = q0 + wave * 16 + (lane & 15);
  const int qc = min(qi, T - 1);
  const int nch = a.d / 8;
  const FlOff off(lane);

  const int64_t qrow = ((int64_t)(b * a.H + h) * T + qc) * a.d;
  u32x4 qh[2], ql[2], gf[2];
  float D = 0.f;
  const int64_t tok = (int64_t)b * T + qc;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j0 = 32 * s + 8 * g;
    qh[s] = ql[s] = u32x4{0u, 0u, 0u, 0u};
    if (j0 < a.d) {
      qh[s] = *reinterpret_cast<const u32x4*>(a.qh + qrow + j0);
      ql[s] = *reinterpret_cast<const u32x4*>(a.ql + qrow + j0);
    }
    gf[s] = u32x4{0u, 0u, 0u, 0u};
    if (j0 < a.d) {
      const int64_t col = (int64_t)h * a.d + j0;
      gf[s] = *reinterpret_cast<const u32x4*>(a.dout + tok * a.lddo + col);
      const u32x4 ov = *reinterpret_cast<const u32x4*>(a.o + tok * a.ldo + col);
      u32x4 rv = u32x4{0u, 0u, 0u, 0u};
      if (a.ores) rv = *reinterpret_cast<const u32x4*>(a.ores + tok * a.ldores + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g0 = __uint_as_float(gf[s][e] << 16), g1 = __uint_as_float(gf[s][e] & 0xffff0000u);
        const float o0 = __uint_as_float(ov[e] << 16) + __uint_as_float(rv[e] << 16);
        const float o1 = __uint_as_float(ov[e] & 0xffff0000u) + __uint_as_float(rv[e] & 0xffff0000u);
        D += g0 * o0 + g1 * o1;
      }
    }
  }
  D = sum4lanes(D);
  const float lse2 = a.lse_in[((int64_t)b * a.H + h) * T + qc] * kLog2e;
  if (g == 0 && qi < T) a.delta[((int64_t)b * a.H + h) * T + qi] = D;

  const int64_t kbase = (int64_t)(b * a.Hkv + kvh) * T * a.d;
  const bf16* kh = a.kh + kbase;
  const bf16* kl = a.kl + kbase;
  const bf16* vb = a.v + (int64_t)b * T * a.ldv + (int64_t)kvh * a.d;

  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nt = qt + 1;
  fl_issue(kh, a.d, 0, T, nch, lds[0], wave, lane);
  fl_issue(kl, a.d, 0, T, nch, lds[0] + FTB, wave, lane);
  fl_issue(vb, a.ldv, 0, T, nch, lds[0] + 2 * FTB, wave, lane);
  for (int kt = 0; kt < nt; ++kt) {
    SLT_WAIT_VMCNT(0);
    lds_barrier();
    if (kt + 1 < nt) {
      char* nx = lds[(kt + 1) & 1];
      const int r0 = (kt + 1) * FR;
      fl_issue(kh, a.d, r0, T, nch, nx, wave, lane);
      fl_issue(kl, a.d, r0, T, nch, nx + FTB, wave, lane);
      fl_issue(vb, a.ldv, r0, T, nch, nx + 2 * FTB, wave, lane);
    }
    const unsigned base = lds_off(lds[kt & 1]);
    const int k0 = kt * FR;
    float p[4][4];
    {
      u32x4 kf[2][4][2];
      rd_rows16(base + off.row[0], base + off.row[1], kf);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          st = mma(kf[0][t][s], qh[s], st);
          st = mma(kf[0][t][s], ql[s], st);
          st = mma(kf[1][t][s], qh[s], st);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) p[t][r] = ex2(st[r] - lse2);
        if (kt == qt) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + 16 * t + 4 * g + r > qi) p[t][r] = 0.f;
        }
      }
    }
    float ds[4][4];
    {
      u32x4 vf[4][2];
      rd_rows8(base + 2 * FTB + off.row[0], base + 2 * FTB + off.row[1], vf);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) dp = mma(vf[t][s], gf[s], dp);
        if (DROP) {  // dS takes the dropped dP
          float dm[4];
          drop_mults<4>(a.drop, att_elem(b, a.H, h, T, qi, k0 + 16 * t + 4 * g), dm);
#pragma unroll
          for (int r = 0; r < 4; ++r) dp[r] *= dm[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[t][r] = p[t][r] * (dp[r] - D);
      }
    }
    u32x4 dh[2], dl[2];
    pack_k_hilo(ds[0], ds[1], dh[0], dl[0]);
    pack_k_hilo(ds[2], ds[3], dh[1], dl[1]);
    {
      u32x4 kt_[4][2];
      rd_cols(base, off, kt_);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[dt] = mma(kt_[dt][c], dh[c], acc[dt]);
          acc[dt] = mma(kt_[dt][c], dl[c], acc[dt]);
        }
      rd_cols(base + FTB, off, kt_);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[dt] = mma(kt_[dt][c], dh[c], acc[dt]);
    }
  }

  // acc[dt] lane: dQ^T[dims 16dt + 4g + r][query i]
  lds_barrier();
  float* F = reinterpret_cast<float*>(&lds[0][0]);
  fl_stage_acc(F, wave * 16 + (lane & 15), g, acc);
  lds_barrier();
  fl_store_rows(F, 1.0f / sqrtf((float)a.d), a.dq + (int64_t)b * T * a.lddq + (int64_t)h * a.d, a.lddq, q0, T, a.d,
                a.R, a.rope_mode, a.cs);
}

// ---------------------------------------------------------------------------
// dK, dV.  One workgroup per (key tile, KV head, batch).  Wave w owns keys k0 + 16w + i and
// loops over the query heads of its KV head and the query tiles at or after
// its key tile: S = Q K^T (hi/lo), P = exp2(S - lse), dP = dO V^T,
// dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS (hi/lo).
// LDS stage: [Q hi | Q lo | dO], two stages.
// ---------------------------------------------------------------------------
template <bool DROP>
__global__ __launch_bounds__(256) void fl_dkdv_k(FlArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2][3 * FTB];
  const int T = a.T, G = a.H / a.Hkv, ntk = (T + FR - 1) / FR;
  const int w = fl_work_item();
  const int kt = w % ntk, kvh = (w / ntk) % a.Hkv, b = w / (ntk * a.Hkv);  // earliest keys (most queries) first
  const int k0 = kt * FR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int ki = k0 + wave * 16 + (lane & 15);
  const int kc = min(ki, T - 1);
  const int nch = a.d / 8;
  const FlOff off(lane);

  const int64_t krow = ((int64_t)(b * a.Hkv + kvh) * T + kc) * a.d;
  u32x4 kh[2], kl[2], vf[2];
  const bf16* vrow = a.v + ((int64_t)b * T + kc) * a.ldv + (int64_t)kvh * a.d;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j0 = 32 * s + 8 * g;
    kh[s] = kl[s] = vf[s] = u32x4{0u, 0u, 0u, 0u};
    if (j0 < a.d) {
      kh[s] = *reinterpret_cast<const u32x4*>(a.kh + krow + j0);
      kl[s] = *reinterpret_cast<const u32x4*>(a.kl + krow + j0);
      vf[s] = *reinterpret_cast<const u32x4*>(vrow + j0);
    }
  }

  f32x4 dva[4], dka[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int ntq = (T + FR - 1) / FR;
  const int per = ntq - kt;  // query tiles kt..ntq-1 per head
  const int nsteps = G * per;
  auto issue = [&](int n, char* st) {
    const int hh = kvh * G + n / per, qt = kt + n % per;
    const int64_t hb = (int64_t)(b * a.H + hh) * T * a.d;
    fl_issue(a.qh + hb, a.d, qt * FR, T, nch, st, wave, lane);
    fl_issue(a.ql + hb, a.d, qt * FR, T, nch, st + FTB, wave, lane);
    fl_issue(a.dout + (int64_t)b * T * a.lddo + (int64_t)hh * a.d, a.lddo, qt * FR, T, nch, st + 2 * FTB, wave,
             lane);
  };
  // lse (times log2 e) and D of the 16 query rows 16t + 4g + r a lane
  // needs, loaded one step ahead (before that step's tile copies, so that
  // waiting for them never waits for the copies issued after them)
  float ln[4][4], dn[4][4];
  // rows (b, h) of lse and D start 16-byte aligned when T % 4 == 0
  const bool vec4 = (T & 3) == 0 && (reinterpret_cast<uintptr_t>(a.lse_in) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.delta) & 15) == 0;
  auto rows_of = [&](int n) {
    const int hh = kvh * G + n / per, qt = kt + n % per;
    const int64_t sb = ((int64_t)b * a.H + hh) * T;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int q4 = qt * FR + 16 * t + 4 * g;
      if (vec4 && q4 + 3 < T) {
        const float4 l4 = *reinterpret_cast<const float4*>(a.lse_in + sb + q4);
        const float4 d4 = *reinterpret_cast<const float4*>(a.delta + sb + q4);
        ln[t][0] = l4.x * kLog2e; ln[t][1] = l4.y * kLog2e; ln[t][2] = l4.z * kLog2e; ln[t][3] = l4.w * kLog2e;
        dn[t][0] = d4.x; dn[t][1] = d4.y; dn[t][2] = d4.z; dn[t][3] = d4.w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qq = min(q4 + r, T - 1);
          ln[t][r] = a.lse_in[sb + qq] * kLog2e;
          dn[t][r] = a.delta[sb + qq];
        }
      }
    }
  };
  rows_of(0);
  issue(0, lds[0]);
  for (int n = 0; n < nsteps; ++n) {
    SLT_WAIT_VMCNT(0);
    lds_barrier();
    float lc[4][4], dc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lc[t][r] = ln[t][r];
        dc[t][r] = dn[t][r];
      }
    if (n + 1 < nsteps) {
      rows_of(n + 1);
      asm volatile("" ::: "memory");
      issue(n + 1, lds[(n + 1) & 1]);
    }
    const int qt = kt + n % per;
    const int q0 = qt * FR;
    const unsigned base = lds_off(lds[n & 1]);

    float p[4][4];
    {
      u32x4 qf[2][4][2];
      rd_rows16(base + off.row[0], base + off.row[1], qf);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          st = mma(qf[0][t][s], kh[s], st);
          st = mma(qf[0][t][s], kl[s], st);
          st = mma(qf[1][t][s], kh[s], st);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) p[t][r] = ex2(st[r] - lc[t][r]);
        if (qt == kt || q0 + FR > T) {  // the diagonal tile, or rows past T
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int qq = q0 + 16 * t + 4 * g + r;
            if (qq >= T || ki > qq) p[t][r] = 0.f;
          }
        }
      }
    }
    float ds[4][4];
    {
      u32x4 gr[4][2];
      rd_rows8(base + 2 * FTB + off.row[0], base + 2 * FTB + off.row[1], gr);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) dp = mma(gr[t][s], vf[s], dp);
        if (DROP) {  // dS takes the dropped dP, dV the dropped weights
          float dm[4];
          drop_mults_strided<4>(a.drop, att_elem(b, a.H, kvh * G + n / per, T, q0 + 16 * t + 4 * g, ki),
                                (uint64_t)T, dm);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ds[t][r] = p[t][r] * (dm[r] * dp[r] - dc[t][r]);
            p[t][r] *= dm[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) ds[t][r] = p[t][r] * (dp[r] - dc[t][r]);
        }
      }
    }
    {
      // dV sums P dO over every query of the group's heads: P as hi + lo
      u32x4 ph[2], pl[2];
      pack_k_hilo(p[0], p[1], ph[0], pl[0]);
      pack_k_hilo(p[2], p[3], ph[1], pl[1]);
      u32x4 gt[4][2];
      rd_cols(base + 2 * FTB, off, gt);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          dva[dt] = mma(gt[dt][c], ph[c], dva[dt]);
          dva[dt] = mma(gt[dt][c], pl[c], dva[dt]);
        }
    }
    {
      u32x4 dh[2], dl[2];
      pack_k_hilo(ds[0], ds[1], dh[0], dl[0]);
      pack_k_hilo(ds[2], ds[3], dh[1], dl[1]);
      u32x4 qt_[4][2];
      rd_cols(base, off, qt_);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          dka[dt] = mma(qt_[dt][c], dh[c], dka[dt]);
          dka[dt] = mma(qt_[dt][c], dl[c], dka[dt]);
        }
      rd_cols(base + FTB, off, qt_);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) dka[dt] = mma(qt_[dt][c], dh[c], dka[dt]);
    }
  }

  lds_barrier();
  float* F = reinterpret_cast<float*>(&lds[0][0]);
  float* F2 = reinterpret_cast<float*>(&lds[1][0]);
  const int row = wave * 16 + (lane & 15);
  fl_stage_acc(F, row, g, dka);
  fl_stage_acc(F2, row, g, dva);
  lds_barrier();
  // the query copy carries log2(e) / sqrt(d): dK = dS^T Q / sqrt(d) = ln(2) dS^T Q'
  fl_store_rows(F, kLn2, a.dk + (int64_t)b * T * a.lddk + (int64_t)kvh * a.d, a.lddk, k0, T, a.d, a.R, a.rope_mode,
                a.cs);
  fl_store_rows(F2, 1.0f, a.dv + (int64_t)b * T * a.lddv + (int64_t)kvh * a.d, a.lddv, k0, T, a.d, 0, 0, nullptr);
}

// Copy rows row0..row0+63 of a bf16 array into an LDS tile with 512 threads:
// one copy per lane (as fl_issue).
__device__ __forceinline__ void fl_issue8(const bf16* g, int64_t ld, int row0, int nrows, int nch, char* tile,
                                          int wave, int lane) {
  const int p = wave * 64 + lane;
  const int r = p >> 3;
  const int c = (p & 7) ^ fsw(r);
  const void* src = c < nch ? static_cast<const void*>(g + (int64_t)min(row0 + r, nrows - 1) * ld + c * 8)
                            : static_cast<const void*>(g_zero16);
  lds_copy16(src, tile + wave * 1024);
}

// ---------------------------------------------------------------------------
// dK, dV over 256-key chunks.  One 8-wave workgroup per (key chunk, KV head,
// batch), chunks with the most queries first; wave w owns the key subtiles
// u = w and w + 8 (16 keys each) of the chunk, their rotated keys, values and
// dK / dV accumulators held in registers.  Query tiles of 64 rows of every
// query head of the group stream through a three-stage LDS ring ([Q hi | Q lo
// | dO | lse, D] per stage); each 32-query half is read from LDS once per
// wave and applied to both subtiles: S = Q K^T (hi/lo), P = exp2(S - lse),
// dP = dO V^T, dS = P (dP - D), then dV^T += dO^T P (P as hi/lo) and
// dK^T += Q^T dS (hi/lo).  Needs T % 4 == 0 (16-byte lse / D rows).
// ---------------------------------------------------------------------------
constexpr int KC = 256;                 // keys per chunk
constexpr int STB = 3 * FTB + 1024;     // stage bytes: Q hi, Q lo, dO, then lse (256 B), D (256 B), pad


template <bool DROP>
__global__ __launch_bounds__(512, 1) void fl_dkdv2_k(FlArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[3][STB];
  const int T = a.T, G = a.H / a.Hkv, nkc = (T + KC - 1) / KC;
  const int w = fl_work_item();
  const int kc = w % nkc, kvh = (w / nkc) % a.Hkv, b = w / (nkc * a.Hkv);  // earliest keys (most queries) first
  const int k0 = kc * KC;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int nch = a.d / 8;
  const FlOff off(lane);

  // subtile i: keys k0 + 16 (wave + 8 i) + li
  u32x4 kh[2][2], kl[2][2], vf[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kc_ = min(k0 + 16 * (wave + 8 * i) + li, T - 1);
    const int64_t krow = ((int64_t)(b * a.Hkv + kvh) * T + kc_) * a.d;
    const bf16* vrow = a.v + ((int64_t)b * T + kc_) * a.ldv + (int64_t)kvh * a.d;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int j0 = 32 * s + 8 * g;
      kh[i][s] = kl[i][s] = vf[i][s] = u32x4{0u, 0u, 0u, 0u};
      if (j0 < a.d) {
        kh[i][s] = *reinterpret_cast<const u32x4*>(a.kh + krow + j0);
        kl[i][s] = *reinterpret_cast<const u32x4*>(a.kl + krow + j0);
        vf[i][s] = *reinterpret_cast<const u32x4*>(vrow + j0);
      }
    }
  }
  f32x4 dva[2][4], dka[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      dva[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dka[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int ntq = (T + FR - 1) / FR;
  const int qt0 = k0 / FR;         // first query tile a key of the chunk needs
  const int per = ntq - qt0;       // query tiles per head
  const int nsteps = G * per;
  auto issue = [&](int n, char* st) {
    const int hh = kvh * G + n / per, qt = qt0 + n % per;
    const int64_t hb = (int64_t)(b * a.H + hh) * T;
    fl_issue8(a.qh + hb * a.d, a.d, qt * FR, T, nch, st, wave, lane);
    fl_issue8(a.ql + hb * a.d, a.d, qt * FR, T, nch, st + FTB, wave, lane);
    fl_issue8(a.dout + (int64_t)b * T * a.lddo + (int64_t)hh * a.d, a.lddo, qt * FR, T, nch, st + 2 * FTB, wave,
              lane);
    if (wave == 0) {  // lse then D of the 64 rows: 16 + 16 chunks (lanes 32..63 repeat into the pad)
      const int c = lane & 15;
      const int q = min(qt * FR + 4 * c, T - 4);
      const float* src = (lane & 16) ? a.delta + hb + q : a.lse_in + hb + q;
      lds_copy16(src, st + 3 * FTB);
    }
  };
  issue(0, lds[0]);
  issue(min(1, nsteps - 1), lds[1]);
  for (int n = 0; n < nsteps; ++n) {
    SLT_WAIT_VMCNT(3);  // only the next step's copies may still fly (wave 0 waits for one more)
    lds_barrier();
    issue(min(n + 2, nsteps - 1), lds[(n + 2) % 3]);
    const int qt = qt0 + n % per;
    const int q0 = qt * FR;
    char* stg = lds[n % 3];
    const unsigned base = lds_off(stg);
    const float* lsd = reinterpret_cast<const float*>(stg + 3 * FTB);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int qh0 = q0 + 32 * hf;  // first query of this half
      if (qh0 >= T || qh0 + 31 < k0 + 16 * wave) continue;  // past T, or before every key of the wave
      u32x4 qf[2][2][2], gr[2][2];
      rd_khalf(base + off.row[0] + 4096 * hf, base + off.row[1] + 4096 * hf, qf);
      rd_rows4(base + 2 * FTB + off.row[0] + 4096 * hf, base + 2 * FTB + off.row[1] + 4096 * hf, gr);
      u32x4 ph[2], pl[2], dh[2], dl[2];
      bool act[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kf = k0 + 16 * (wave + 8 * i);  // first key of subtile i
        act[i] = qh0 + 31 >= kf;
        if (!act[i]) continue;
        const int ki = kf + li;
        float p[2][4], ds[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            st = mma(qf[0][tt][s], kh[i][s], st);
            st = mma(qf[0][tt][s], kl[i][s], st);
            st = mma(qf[1][tt][s], kh[i][s], st);
            dp = mma(gr[tt][s], vf[i][s], dp);
          }
          // lse (to base 2) and D of the lane's 4 query rows, read where used
          const float4 l4 = *reinterpret_cast<const float4*>(lsd + 32 * hf + 16 * tt + 4 * g);
          const float4 d4 = *reinterpret_cast<const float4*>(lsd + 64 + 32 * hf + 16 * tt + 4 * g);
          p[tt][0] = ex2(st[0] - l4.x * kLog2e);
          p[tt][1] = ex2(st[1] - l4.y * kLog2e);
          p[tt][2] = ex2(st[2] - l4.z * kLog2e);
          p[tt][3] = ex2(st[3] - l4.w * kLog2e);
          const float dn[4] = {d4.x, d4.y, d4.z, d4.w};
          if (qh0 < kf + 15 || qh0 + 31 >= T) {  // the diagonal, or rows past T
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int qq = qh0 + 16 * tt + 4 * g + r;
              if (qq >= T || ki > qq) p[tt][r] = 0.f;
            }
          }
          if (DROP) {  // dS takes the dropped dP, dV the dropped weights
            float dm[4];
            drop_mults_strided<4>(a.drop, att_elem(b, a.H, kvh * G + n / per, T, qh0 + 16 * tt + 4 * g, ki),
                                  (uint64_t)T, dm);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              ds[tt][r] = p[tt][r] * (dm[r] * dp[r] - dn[r]);
              p[tt][r] *= dm[r];
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) ds[tt][r] = p[tt][r] * (dp[r] - dn[r]);
          }
        }
        pack_k_hilo(p[0], p[1], ph[i], pl[i]);
        pack_k_hilo(ds[0], ds[1], dh[i], dl[i]);
      }
      {
        u32x4 gt[4];
        rd_chalf(base + 2 * FTB + off.col[0] + 4096 * hf, base + 2 * FTB + off.col[1] + 4096 * hf,
                 base + 2 * FTB + off.col[2] + 4096 * hf, base + 2 * FTB + off.col[3] + 4096 * hf, gt);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            dva[i][dt] = mma(gt[dt], ph[i], dva[i][dt]);
            dva[i][dt] = mma(gt[dt], pl[i], dva[i][dt]);
          }
        }
      }
      {
        u32x4 qc[4];
        rd_chalf(base + off.col[0] + 4096 * hf, base + off.col[1] + 4096 * hf, base + off.col[2] + 4096 * hf,
                 base + off.col[3] + 4096 * hf, qc);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            dka[i][dt] = mma(qc[dt], dh[i], dka[i][dt]);
            dka[i][dt] = mma(qc[dt], dl[i], dka[i][dt]);
          }
        }
        rd_chalf(base + FTB + off.col[0] + 4096 * hf, base + FTB + off.col[1] + 4096 * hf,
                 base + FTB + off.col[2] + 4096 * hf, base + FTB + off.col[3] + 4096 * hf, qc);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) dka[i][dt] = mma(qc[dt], dh[i], dka[i][dt]);
        }
      }
    }
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends

  // stage the chunk's 256 rows of dK (then dV) as fp32 and store them
  lds_barrier();
  float* F = reinterpret_cast<float*>(&lds[0][0]);
#pragma unroll
  for (int i = 0; i < 2; ++i) fl_stage_acc(F, 16 * (wave + 8 * i) + li, g, dka[i]);
  lds_barrier();
  // the query copy carries log2(e) / sqrt(d): dK = dS^T Q / sqrt(d) = ln(2) dS^T Q'
  fl_store_rows(F, kLn2, a.dk + (int64_t)b * T * a.lddk + (int64_t)kvh * a.d, a.lddk, k0, T, a.d, a.R, a.rope_mode,
                a.cs, KC);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < 2; ++i) fl_stage_acc(F, 16 * (wave + 8 * i) + li, g, dva[i]);
  lds_barrier();
  fl_store_rows(F, 1.0f, a.dv + (int64_t)b * T * a.lddv + (int64_t)kvh * a.d, a.lddv, k0, T, a.d, 0, 0, nullptr, KC);
}

inline bool al(const void* p, int n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

FlArgs to_fl(const AttnArgs& a) {
  FlArgs f{};
  const int64_t nq = (int64_t)a.B * a.H * a.T * a.d, nk = (int64_t)a.B * a.Hkv * a.T * a.d;
  bf16* rot = static_cast<bf16*>(a.rot);
  f.qh = rot;
  f.ql = rot + nq;
  f.kh = rot + 2 * nq;
  f.kl = rot + 2 * nq + nk;
  f.v = static_cast<const bf16*>(a.v);
  f.o = static_cast<const bf16*>(a.o);
  f.ores = static_cast<const bf16*>(a.ores_in);
  f.dout = static_cast<const bf16*>(a.dout);
  f.out = static_cast<bf16*>(a.out);
  f.ores_out = static_cast<bf16*>(a.ores_out);
  f.dq = static_cast<bf16*>(a.dq);
  f.dk = static_cast<bf16*>(a.dk);
  f.dv = static_cast<bf16*>(a.dv);
  f.lse = a.lse;
  f.lse_in = a.lse_in;
  f.delta = a.delta;
  f.cs = a.cs;
  f.ldv = a.ldv;
  f.ldo = a.ldo;
  f.ldores = (int64_t)a.H * a.d;
  f.lddo = a.lddo;
  f.lddq = a.lddq;
  f.lddk = a.lddk;
  f.lddv = a.lddv;
  f.B = a.B;
  f.T = a.T;
  f.H = a.H;
  f.Hkv = a.Hkv;
  f.d = a.d;
  f.R = a.R;
  f.rope_mode = a.rope_mode;
  f.drop = a.drop;
  return f;
}

slt_status prep(const AttnArgs& a, const FlArgs& f, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.T), (unsigned)(((a.H + a.Hkv) * (a.d / 8) + 127) / 128));
  const bool vec = al(a.q, 16) && al(a.k, 16) && a.ldq % 8 == 0 && a.ldk % 8 == 0 && (a.R == 0 || a.cs != nullptr) &&
                   (a.R == 0 || (a.rope_mode == SLT_ROPE_HALF ? (a.R / 2) % 8 == 0 : a.R % 8 == 0));
  auto* kern = vec ? fl_prep_k<true> : fl_prep_k<false>;
  kern<<<grid, 128, 0, s>>>(static_cast<const bf16*>(a.q), a.ldq, static_cast<const bf16*>(a.k), a.ldk,
                                   const_cast<bf16*>(f.qh), const_cast<bf16*>(f.ql), const_cast<bf16*>(f.kh),
                                   const_cast<bf16*>(f.kl), a.B, a.T, a.H, a.Hkv, a.d, a.R, a.rope_mode, a.cs,
                                   kLog2e / sqrtf((float)a.d));
  return check_launch("attention rope prep");
}

}  // namespace

int64_t flash_rot_elems(int B, int T, int H, int Hkv, int d) { return 2 * (int64_t)B * (H + Hkv) * T * d; }

bool flash_eligible(int dtype, int d) { return dtype == SLT_BF16 && d > 0 && d % 16 == 0 && d <= FD; }

bool flash_ok(const AttnArgs& a, bool bwd) {
  if (!flash_eligible(a.dtype, a.d) || !a.rot || !al(a.rot, 16)) return false;
  if (!al(a.v, 16) || a.ldv % 8) return false;
  if (!bwd) return al(a.out, 8) && a.ldo % 4 == 0 && (!a.ores_out || al(a.ores_out, 8));
  return al(a.o, 16) && a.ldo % 8 == 0 && al(a.dout, 16) && a.lddo % 8 == 0 && (!a.ores_in || al(a.ores_in, 16)) &&
         al(a.dq, 8) && al(a.dk, 8) && al(a.dv, 8) && a.lddq % 4 == 0 && a.lddk % 4 == 0 && a.lddv % 4 == 0 &&
         (a.H * a.d) % 8 == 0;
}

slt_status flash_fwd(const AttnArgs& a, hipStream_t s) {
  const FlArgs f = to_fl(a);
  if (!a.rot_ready) {
    const slt_status st = prep(a, f, s);
    if (st != SLT_OK) return st;
  }
  // 128-query chunks (two subtiles per wave) from T = 2048 on: the longest
  // chunks there hold 32 key tiles, and halving them evens out the last round
  // of the grid (measured: 11 % faster at T = 2048, 2 % slower at T = 1024
  // and 14 % slower at T = 256)
  auto go = [&](auto ns) {
    constexpr int NS = decltype(ns)::value;
    const int nck = (a.T + 64 * NS - 1) / (64 * NS);
    if (a.drop.on) fl_fwd2_k<true, NS><<<nck * a.H * a.B, 256, 0, s>>>(f);
    else fl_fwd2_k<false, NS><<<nck * a.H * a.B, 256, 0, s>>>(f);
  };
  if (a.T >= 2048) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 4>{});
  return check_launch("attention forward");
}

slt_status flash_bwd(const AttnArgs& a, hipStream_t s) {
  const FlArgs f = to_fl(a);
  if (!a.rot_ready) {
    const slt_status st = prep(a, f, s);
    if (st != SLT_OK) return st;
  }
  const int nt = (a.T + FR - 1) / FR;
  if (a.drop.on) fl_dq_k<true><<<nt * a.H * a.B, 256, 0, s>>>(f);
  else fl_dq_k<false><<<nt * a.H * a.B, 256, 0, s>>>(f);
  slt_status st = check_launch("attention backward (dq)");
  if (st != SLT_OK) return st;
  if (a.T % 4 == 0 && al(a.lse_in, 16) && al(a.delta, 16)) {
    const int nkc = (a.T + KC - 1) / KC;
    if (a.drop.on) fl_dkdv2_k<true><<<nkc * a.Hkv * a.B, 512, 0, s>>>(f);
    else fl_dkdv2_k<false><<<nkc * a.Hkv * a.B, 512, 0, s>>>(f);
  } else {
    if (a.drop.on) fl_dkdv_k<true><<<nt * a.Hkv * a.B, 256, 0, s>>>(f);
    else fl_dkdv_k<false><<<nt * a.Hkv * a.B, 256, 0, s>>>(f);
  }
  return check_launch("attention backward (dk, dv)");
}

}  // namespace slt
