// Causal attention for bf16 activations, head dim d <= 64 with d % 16 == 0
// (Hephaistos, "Architecture at a glance": RoPE applied to q and k inside
// attention, causal multi-head attention with a numerically stable softmax;
// strata: flash-style attention with online softmax, forward and backward,
// no T x T score matrix, MHA/GQA through independent n_head and n_kv_head).
//
// Operands: q and k arrive rotated by RoPE and rounded once to bf16 (the
// training forward's QKV projection rotates them in its epilogue; the per-op
// entry points rotate them into a workspace first), v as projected; all three
// are read in place as strided rows (row (b, t) at base + (b T + t) ld, head h
// at + h d), so no copies are made.  Every tile (64 rows x 64 dims, 8 KiB,
// dims >= d zero-filled) goes HBM -> LDS with global_load_lds_dwordx4, no
// register staging.  The softmax scale log2(e)/sqrt(d) is applied to the fp32
// scores, so the exponentials run in base 2.
//
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
//  * Output dims run over ND = d/16 tiles of 16 (3 at d = 48, 4 at d = 64):
//    the products whose outputs are head dims (O, dQ, dK, dV) skip the
//    zero-padded dims; the score products contract over 64 padded dims.
//  * Precision: one bf16 operand per product.  The probabilities P (into
//    P V and dV) and the score gradient dS (into dQ and dK) are rounded to
//    bf16 in registers (at d = 64 the forward's softmax denominators are the
//    sums of those rounded P); D = dO.O uses O plus its stored bf16 rounding
//    residual, so that sum_j dS_ij stays zero to fp32 accuracy.
//  * Tiles: LDS tile rows are 8 chunks of 16 bytes with chunk position XOR
//    2((row >> 1) & 3), so both the row-fragment reads (ds_read_b128) and the
//    transposing reads spread over all banks.  LDS reads are asm blocks that
//    wait for their own results: the compiler cannot tell which buffer an
//    in-flight global_load_lds targets and would otherwise wait for all of
//    them.
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
constexpr int FSB = FR * FS * 4;      // bytes of one 64-row fp32 staging tile
constexpr float kLog2e = 1.4426950408889634f;

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
// fmax: IEEE maximum (NaN-propagating; the scores hold no NaN), which gfx950
// runs as v_maximum3_f32 with no canonicalising step per operand.
__device__ __forceinline__ float fmx(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max4lanes(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmx(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmx(__uint_as_float(q[0]), __uint_as_float(q[1]));
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

// Row fragments of one tile at byte address t0: f[t][s], t = 0..3 (16-row
// groups), s = 0..1 (32-dim halves).
__device__ __forceinline__ void rd_rows8(unsigned a0, unsigned a1, u32x4 (&f)[4][2]) {
  asm volatile(FL_R128(f00, a0, 0) FL_R128(f01, a1, 0) FL_R128(f10, a0, 2048) FL_R128(f11, a1, 2048)
                   FL_R128(f20, a0, 4096) FL_R128(f21, a1, 4096) FL_R128(f30, a0, 6144) FL_R128(f31, a1, 6144)
               "s_waitcnt lgkmcnt(0)"
               : FL_O(f00, f[0][0]), FL_O(f01, f[0][1]), FL_O(f10, f[1][0]), FL_O(f11, f[1][1]), FL_O(f20, f[2][0]),
                 FL_O(f21, f[2][1]), FL_O(f30, f[3][0]), FL_O(f31, f[3][1])
               : [a0] "v"(a0), [a1] "v"(a1)
               : "memory");
}

// Row fragments of one 32-row half of one tile: f[tt][s].  a0 / a1 = tile
// address plus the lane's row[0] / row[1] plus 4096 per half.
__device__ __forceinline__ void rd_rows4(unsigned a0, unsigned a1, u32x4 (&f)[2][2]) {
  asm volatile(FL_R128(f00, a0, 0) FL_R128(f01, a1, 0) FL_R128(f10, a0, 2048) FL_R128(f11, a1, 2048)
               "s_waitcnt lgkmcnt(0)"
               : FL_O(f00, f[0][0]), FL_O(f01, f[0][1]), FL_O(f10, f[1][0]), FL_O(f11, f[1][1])
               : [a0] "v"(a0), [a1] "v"(a1)
               : "memory");
}

// Column fragments of one tile: f[dt][c] = rows 32c + (4g..4g+3, then
// 16 + 4g..4g+3) at dims 16 dt + i, dt < ND (3 or 4), c = 0..1.  cK = address
// of the tile plus the lane's col[dt].
template <int ND>
__device__ __forceinline__ void rd_cols_t(unsigned c0, unsigned c1, unsigned c2, unsigned c3, u32x4 (&f)[4][2]) {
  u32x2 x[4][2][2];
  if constexpr (ND == 4) {
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
  } else {
    static_assert(ND == 3, "3 or 4 dim tiles");
    asm volatile(FL_RTR(x000, c0, 0) FL_RTR(x001, c0, 2048) FL_RTR(x010, c0, 4096) FL_RTR(x011, c0, 6144)
                     FL_RTR(x100, c1, 0) FL_RTR(x101, c1, 2048) FL_RTR(x110, c1, 4096) FL_RTR(x111, c1, 6144)
                         FL_RTR(x200, c2, 0) FL_RTR(x201, c2, 2048) FL_RTR(x210, c2, 4096) FL_RTR(x211, c2, 6144)
                             "s_waitcnt lgkmcnt(0)"
                 : FL_O(x000, x[0][0][0]), FL_O(x001, x[0][0][1]), FL_O(x010, x[0][1][0]), FL_O(x011, x[0][1][1]),
                   FL_O(x100, x[1][0][0]), FL_O(x101, x[1][0][1]), FL_O(x110, x[1][1][0]), FL_O(x111, x[1][1][1]),
                   FL_O(x200, x[2][0][0]), FL_O(x201, x[2][0][1]), FL_O(x210, x[2][1][0]), FL_O(x211, x[2][1][1])
                 : [c0] "v"(c0), [c1] "v"(c1), [c2] "v"(c2)
                 : "memory");
    (void)c3;
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) f[dt][c] = cat(x[dt][c][0], x[dt][c][1]);
}

// Column fragments of one 32-row half of a tile: f[dt] = rows 32 hf +
// (4g..4g+3, then 16 + 4g..4g+3) at dims 16 dt + i, dt < ND.  cK = tile
// address plus the lane's col[dt] plus 4096 hf.
template <int ND>
__device__ __forceinline__ void rd_chalf_t(unsigned c0, unsigned c1, unsigned c2, unsigned c3, u32x4 (&f)[4]) {
  u32x2 x[4][2];
  if constexpr (ND == 4) {
    asm volatile(FL_RTR(x00, c0, 0) FL_RTR(x01, c0, 2048) FL_RTR(x10, c1, 0) FL_RTR(x11, c1, 2048)
                     FL_RTR(x20, c2, 0) FL_RTR(x21, c2, 2048) FL_RTR(x30, c3, 0) FL_RTR(x31, c3, 2048)
                         "s_waitcnt lgkmcnt(0)"
                 : FL_O(x00, x[0][0]), FL_O(x01, x[0][1]), FL_O(x10, x[1][0]), FL_O(x11, x[1][1]),
                   FL_O(x20, x[2][0]), FL_O(x21, x[2][1]), FL_O(x30, x[3][0]), FL_O(x31, x[3][1])
                 : [c0] "v"(c0), [c1] "v"(c1), [c2] "v"(c2), [c3] "v"(c3)
                 : "memory");
  } else {
    static_assert(ND == 3, "3 or 4 dim tiles");
    asm volatile(FL_RTR(x00, c0, 0) FL_RTR(x01, c0, 2048) FL_RTR(x10, c1, 0) FL_RTR(x11, c1, 2048)
                     FL_RTR(x20, c2, 0) FL_RTR(x21, c2, 2048) "s_waitcnt lgkmcnt(0)"
                 : FL_O(x00, x[0][0]), FL_O(x01, x[0][1]), FL_O(x10, x[1][0]), FL_O(x11, x[1][1]),
                   FL_O(x20, x[2][0]), FL_O(x21, x[2][1])
                 : [c0] "v"(c0), [c1] "v"(c1), [c2] "v"(c2)
                 : "memory");
    (void)c3;
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) f[dt] = cat(x[dt][0], x[dt][1]);
}
#undef FL_R128
#undef FL_RTR
#undef FL_O

template <int ND>
__device__ __forceinline__ void rd_cols(unsigned base, const FlOff& o, u32x4 (&f)[4][2]) {
  rd_cols_t<ND>(base + o.col[0], base + o.col[1], base + o.col[2], base + o.col[3], f);
}
template <int ND>
__device__ __forceinline__ void rd_chalf(unsigned base, const FlOff& o, u32x4 (&f)[4]) {
  rd_chalf_t<ND>(base + o.col[0], base + o.col[1], base + o.col[2], base + o.col[3], f);
}

// The log-sum-exp and D values of a lane's query rows in a 32-query half,
// from the stage's [lse | D] rows at byte address a (the half's first row
// plus the lane's 4 g): v[0], v[1] = lse of rows +0..3 and +16..19, v[2],
// v[3] = D of the same rows.  One asm block that waits for its own reads: a
// plain load would make the compiler first wait for every copy in flight
// into the ring, the next two steps' tiles included.
__device__ __forceinline__ void rd_lsd(unsigned a, u32x4 (&v)[4]) {
  asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:64\n\t"
               "ds_read_b128 %2, %4 offset:256\n\tds_read_b128 %3, %4 offset:320\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
               : "v"(a)
               : "memory");
}

// Four probabilities (or gradients) of two neighbouring 16-row results in
// the k order the transposed reads use, rounded to bf16.
__device__ __forceinline__ u32x4 pack_k(const float (&x)[4], const float (&y)[4]) {
  return u32x4{f32x2_to_bf16x2_bits(x[0], x[1]), f32x2_to_bf16x2_bits(x[2], x[3]), f32x2_to_bf16x2_bits(y[0], y[1]),
               f32x2_to_bf16x2_bits(y[2], y[3])};
}

// A row fragment (dims 32 s + 8 g .. + 7) of a strided bf16 row, zero past d.
__device__ __forceinline__ u32x4 ld_frag(const bf16* row, int s, int g, int d) {
  const int j0 = 32 * s + 8 * g;
  return j0 < d ? *reinterpret_cast<const u32x4*>(row + j0) : u32x4{0u, 0u, 0u, 0u};
}

struct FlArgs {
  const bf16 *q, *k, *v;          // rotated q, rotated k, v: row (b, t) at base + (b T + t) ld, head h at + h d
  const bf16 *o, *ores, *dout;    // [B T] rows: o (ldo), ores (ldores), dout (lddo)
  bf16 *out, *ores_out, *dq, *dk, *dv;
  float* lse;
  const float* lse_in;
  float* delta;
  const float* cs;
  int64_t ldq, ldk, ldv, ldo, ldores, lddo, lddq, lddk, lddv;
  int B, T, H, Hkv, d, R, rope_mode;
  float c2;                       // log2(e) / sqrt(d): scores in base-2 units
  Drop drop;                      // dropout of the attention weights (att_elem)
};

// ---------------------------------------------------------------------------
// Forward, one workgroup per (64 FNS-query chunk, head, batch), longest
// chunks first.  Wave w owns the 16-query subtiles u = w, w+4, .., w+4(FNS-1)
// of the chunk, their queries held as MFMA fragments in registers.  Key /
// value tiles of 64 rows stream through a three-stage LDS ring ([K | V] per
// stage, two tiles in flight while one is used); each 32-key half is read
// from LDS once per wave and applied to all of the wave's subtiles that reach
// it, so a tile is fetched once per chunk and its fragments once per wave.
// Per subtile and half: S^T = K Q^T, online softmax in base 2, O^T += V^T
// P^T.  Subtile u needs key tile j iff 64 j <= 16 u + 15 (chunk-relative),
// i.e. subtile i of a wave from tile i on, so every wave does the same work.
// ---------------------------------------------------------------------------
template <bool DROP, int FNS, int ND>
__global__ __launch_bounds__(256, 2) void fl_fwd_k(FlArgs a) {
  constexpr int FC = 64 * FNS;  // queries per chunk
  __shared__ __attribute__((aligned(16))) char lds[3][2 * FTB];
  const int T = a.T, nck = (T + FC - 1) / FC;
  const int w = fl_work_item();
  const int ck = nck - 1 - w % nck, h = (w / nck) % a.H, b = w / (nck * a.H);
  const int c0 = ck * FC, kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int nch = a.d / 8;
  const float c2 = a.c2;
  const FlOff off(lane);

  // subtile i of this wave: queries c0 + 16 (wave + 4 i) + li
  u32x4 qf[FNS][2];
#pragma unroll
  for (int i = 0; i < FNS; ++i) {
    const int qc = min(c0 + 16 * (wave + 4 * i) + li, T - 1);
    const bf16* qrow = a.q + ((int64_t)b * T + qc) * a.ldq + (int64_t)h * a.d;
#pragma unroll
    for (int s = 0; s < 2; ++s) qf[i][s] = ld_frag(qrow, s, g, a.d);
  }
  const bf16* kb = a.k + (int64_t)b * T * a.ldk + (int64_t)kvh * a.d;
  const bf16* vb = a.v + (int64_t)b * T * a.ldv + (int64_t)kvh * a.d;

  // At d = 64 without dropout the row sums l come from the matrix cores: a
  // product of P with an all-ones "V" tile leaves each lane the sum over the
  // half's keys of its query's bf16 probabilities -- the weights P V uses --
  // in every element of lacc (measured: no slower than the lanes' adds at
  // d = 64, slower at d = 48, where P V is one MFMA shorter).  Otherwise the
  // lanes add the weights (l; with dropout, the weights before the mask, as
  // the normaliser must see them) and combine them at the end.
  constexpr bool MSUM = !DROP && ND == 4;
  f32x4 oacc[FNS][4], lacc[FNS];
  float m[FNS], l[FNS];
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int i = 0; i < FNS; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
    lacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // key tiles 0 .. nt-1 cover keys up to the chunk's last query
  const int nt = (min(T, c0 + FC) + FR - 1) / FR;
  auto issue = [&](int j, char* st) {
    fl_issue(kb, a.ldk, j * FR, T, nch, st, wave, lane);
    fl_issue(vb, a.ldv, j * FR, T, nch, st + FTB, wave, lane);
  };
  issue(0, lds[0]);
  issue(min(1, nt - 1), lds[1]);  // past the end: tile 0 again, into a stage nobody reads
  for (int j = 0; j < nt; ++j) {
    SLT_WAIT_VMCNT(4);  // only the copies of tile j+1 may still fly
    lds_barrier();
    issue(min(j + 2, nt - 1), lds[(j + 2) % 3]);
    const unsigned base = lds_off(lds[j % 3]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int k0 = j * FR + 32 * hf;  // first key of this half
      // subtiles whose last query reaches this half (uniform over the wave)
      if (k0 > c0 + 16 * (wave + 4 * (FNS - 1)) + 15 || k0 >= T) break;
      u32x4 kf[2][2], vf[4];
      rd_rows4(base + off.row[0] + 4096 * hf, base + off.row[1] + 4096 * hf, kf);
      rd_chalf<ND>(base + FTB + 4096 * hf, off, vf);
      if (k0 + 31 < c0 + 16 * wave) {
        // Every query of every subtile of the wave comes after the half's
        // last key: no mask and no subtile to skip, so the subtiles' steps
        // run side by side (all scores, all maxima, all probabilities, all
        // products), giving each dependent step independent work from the
        // other subtiles.  Same arithmetic as the masked path below.
        float sv[FNS][2][4];
#pragma unroll
        for (int i = 0; i < FNS; ++i)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
            st = mma(kf[tt][0], qf[i][0], st);
            st = mma(kf[tt][1], qf[i][1], st);
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[i][tt][r] = st[r];
          }
        float mt[FNS];
        bool grow[FNS], any = false;
#pragma unroll
        for (int i = 0; i < FNS; ++i) {
          float tmax = sv[i][0][0];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) tmax = fmx(tmax, sv[i][tt][r]);
          mt[i] = max4lanes(tmax) * c2;
          grow[i] = mt[i] > m[i] + 8.f;
          any |= grow[i];
        }
        if (__ballot(any) != 0) {
#pragma unroll
          for (int i = 0; i < FNS; ++i) {
            const float mn = grow[i] ? mt[i] : m[i];
            const float alpha = grow[i] ? ex2(m[i] - mn) : 1.f;
            if (MSUM) lacc[i] *= alpha;
            else l[i] *= alpha;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) oacc[i][dt] *= alpha;
            m[i] = mn;
          }
        }
        u32x4 pb[FNS];
#pragma unroll
        for (int i = 0; i < FNS; ++i) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[i][tt][r] = ex2(fmaf(sv[i][tt][r], c2, -m[i]));
          if (!MSUM) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int r = 0; r < 4; ++r) l[i] += sv[i][tt][r];
          }
          if (DROP) {
            const int qi = c0 + 16 * (wave + 4 * i) + li;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              float dm[4];
              drop_mults<4>(a.drop, att_elem(b, a.H, h, T, qi, k0 + 16 * tt + 4 * g), dm);
#pragma unroll
              for (int r = 0; r < 4; ++r) sv[i][tt][r] *= dm[r];
            }
          }
          pb[i] = pack_k(sv[i][0], sv[i][1]);
        }
#pragma unroll
        for (int i = 0; i < FNS; ++i) {
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) oacc[i][dt] = mma(vf[dt], pb[i], oacc[i][dt]);
          if (MSUM) lacc[i] = mma(ones, pb[i], lacc[i]);
        }
        continue;
      }
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
          st = mma(kf[tt][0], qf[i][0], st);
          st = mma(kf[tt][1], qf[i][1], st);
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[tt][r] = st[r];
          if (k0 + 31 > u0) {  // keys after a query of the subtile are masked
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (k0 + 16 * tt + 4 * g + r > qi) sv[tt][r] = -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) tmax = fmx(tmax, sv[tt][r]);
        }
        // The running maximum (base-2 units) moves only where a row's new
        // maximum exceeds it by more than 8, so the weights stay below 2^8;
        // a wave whose rows all keep theirs skips rescaling its
        // accumulators.  (The first half processed holds key 0, which no
        // query masks, so m is finite from then on.)
        const float mt = max4lanes(tmax) * c2;
        const bool grow = mt > m[i] + 8.f;
        if (__ballot(grow) != 0) {
          const float mn = grow ? mt : m[i];
          const float alpha = ex2(m[i] - mn);  // 1 where the maximum stays, 0 on the first half
          if (MSUM) lacc[i] *= alpha;
          else l[i] *= alpha;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) oacc[i][dt] *= alpha;
          m[i] = mn;
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[tt][r] = ex2(fmaf(sv[tt][r], c2, -m[i]));
        if (!MSUM) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) l[i] += sv[tt][r];  // this lane's keys; the four lanes are summed at the end
        }
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
        for (int dt = 0; dt < ND; ++dt) oacc[i][dt] = mma(vf[dt], pb, oacc[i][dt]);
        if (MSUM) lacc[i] = mma(ones, pb, lacc[i]);
      }
    }
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends

#pragma unroll
  for (int i = 0; i < FNS; ++i) l[i] = MSUM ? lacc[i][0] : sum4lanes(l[i]);
#pragma unroll
  for (int i = 0; i < FNS; ++i) {
    const int qi = c0 + 16 * (wave + 4 * i) + li;
    if (qi >= T) continue;
    const float inv = 1.0f / l[i];
    bf16* ob = a.out + ((int64_t)b * T + qi) * a.ldo + (int64_t)h * a.d;
    bf16* rb = a.ores_out ? a.ores_out + ((int64_t)b * T + qi) * a.ldores + (int64_t)h * a.d : nullptr;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
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
    // lse in natural-log units: (m + log2 l) ln 2 = max s / sqrt(d) + ln l
    if (g == 0) a.lse[((int64_t)b * a.H + h) * T + qi] = (m[i] + log2f(l[i])) / kLog2e;
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

// Accumulators acc[dt] (lane: dims 16 dt + 4g + r of row `row`) -> F[row][dims].
template <int ND>
__device__ __forceinline__ void fl_stage_acc(float* F, int row, int g, const f32x4 (&acc)[4]) {
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
    *reinterpret_cast<float4*>(F + row * FS + 16 * dt + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2],
                                                                             acc[dt][3]);
}

// ---------------------------------------------------------------------------
// dQ (and D).  One workgroup per (query tile, head, batch).  Wave w owns
// queries q0 + 16w + i: D = dO.(O + ores); per key tile: S^T = K Q^T,
// P^T = exp2(c2 S^T - lse2), dP^T = V dO^T, dS^T = P^T (dP^T - D),
// dQ^T += K^T dS^T.  LDS stage: [K | V], two stages.
// ---------------------------------------------------------------------------
template <bool DROP, int ND>
__global__ __launch_bounds__(256) void fl_dq_k(FlArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2][2 * FTB];  // also the 64-row fp32 staging tile (FSB bytes)
  static_assert(2 * 2 * FTB >= FSB, "staging tile fits");
  const int T = a.T, ntq = (T + FR - 1) / FR;
  const int w = fl_work_item();
  const int qt = ntq - 1 - w % ntq, h = (w / ntq) % a.H, b = w / (ntq * a.H);
  const int q0 = qt * FR, kvh = h / (a.H / a.Hkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int qi = q0 + wave * 16 + (lane & 15);
  const int qc = min(qi, T - 1);
  const int nch = a.d / 8;
  const float c2 = a.c2;
  const FlOff off(lane);

  const int64_t tok = (int64_t)b * T + qc;
  const bf16* qrow = a.q + tok * a.ldq + (int64_t)h * a.d;
  u32x4 qf[2], gf[2];
  float D = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j0 = 32 * s + 8 * g;
    qf[s] = ld_frag(qrow, s, g, a.d);
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

  const bf16* kb = a.k + (int64_t)b * T * a.ldk + (int64_t)kvh * a.d;
  const bf16* vb = a.v + (int64_t)b * T * a.ldv + (int64_t)kvh * a.d;

  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nt = qt + 1;
  fl_issue(kb, a.ldk, 0, T, nch, lds[0], wave, lane);
  fl_issue(vb, a.ldv, 0, T, nch, lds[0] + FTB, wave, lane);
  for (int kt = 0; kt < nt; ++kt) {
    SLT_WAIT_VMCNT(0);
    lds_barrier();
    if (kt + 1 < nt) {
      char* nx = lds[(kt + 1) & 1];
      const int r0 = (kt + 1) * FR;
      fl_issue(kb, a.ldk, r0, T, nch, nx, wave, lane);
      fl_issue(vb, a.ldv, r0, T, nch, nx + FTB, wave, lane);
    }
    const unsigned base = lds_off(lds[kt & 1]);
    const int k0 = kt * FR;
    float p[4][4];
    {
      u32x4 kf[4][2];
      rd_rows8(base + off.row[0], base + off.row[1], kf);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
        st = mma(kf[t][0], qf[0], st);
        st = mma(kf[t][1], qf[1], st);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[t][r] = ex2(fmaf(st[r], c2, -lse2));
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
      rd_rows8(base + FTB + off.row[0], base + FTB + off.row[1], vf);
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
    const u32x4 dsb[2] = {pack_k(ds[0], ds[1]), pack_k(ds[2], ds[3])};
    {
      u32x4 kt_[4][2];
      rd_cols<ND>(base, off, kt_);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[dt] = mma(kt_[dt][c], dsb[c], acc[dt]);
    }
  }

  // acc[dt] lane: dQ^T[dims 16dt + 4g + r][query i]
  lds_barrier();
  float* F = reinterpret_cast<float*>(&lds[0][0]);
  fl_stage_acc<ND>(F, wave * 16 + (lane & 15), g, acc);
  lds_barrier();
  fl_store_rows(F, 1.0f / sqrtf((float)a.d), a.dq + (int64_t)b * T * a.lddq + (int64_t)h * a.d, a.lddq, q0, T, a.d,
                a.R, a.rope_mode, a.cs);
}

// ---------------------------------------------------------------------------
// dK, dV.  One workgroup per (key tile, KV head, batch).  Wave w owns keys
// k0 + 16w + i and loops over the query heads of its KV head and the query
// tiles at or after its key tile: S = Q K^T, P = exp2(c2 S - lse2), dP =
// dO V^T, dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
// LDS stage: [Q | dO], two stages (the fp32 staging tiles of dK and dV
// overlay them at the end).
// ---------------------------------------------------------------------------
template <bool DROP, int ND>
__global__ __launch_bounds__(256) void fl_dkdv_k(FlArgs a) {
  constexpr int SB = 2 * FTB;  // stage bytes
  __shared__ __attribute__((aligned(16))) char lds[2 * FSB > 2 * SB ? 2 * FSB : 2 * SB];
  const int T = a.T, G = a.H / a.Hkv, ntk = (T + FR - 1) / FR;
  const int w = fl_work_item();
  const int kt = w % ntk, kvh = (w / ntk) % a.Hkv, b = w / (ntk * a.Hkv);  // earliest keys (most queries) first
  const int k0 = kt * FR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int ki = k0 + wave * 16 + (lane & 15);
  const int kc = min(ki, T - 1);
  const int nch = a.d / 8;
  const float c2 = a.c2;
  const FlOff off(lane);

  u32x4 kf[2], vf[2];
  const bf16* krow = a.k + ((int64_t)b * T + kc) * a.ldk + (int64_t)kvh * a.d;
  const bf16* vrow = a.v + ((int64_t)b * T + kc) * a.ldv + (int64_t)kvh * a.d;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    kf[s] = ld_frag(krow, s, g, a.d);
    vf[s] = ld_frag(vrow, s, g, a.d);
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
    fl_issue(a.q + (int64_t)b * T * a.ldq + (int64_t)hh * a.d, a.ldq, qt * FR, T, nch, st, wave, lane);
    fl_issue(a.dout + (int64_t)b * T * a.lddo + (int64_t)hh * a.d, a.lddo, qt * FR, T, nch, st + FTB, wave, lane);
  };
  // lse (times log2 e) and D of the 16 query rows 16t + 4g + r a lane
  // needs, loaded one step ahead (before that step's tile copies, so that
  // waiting for them never waits for the copies issued after them)
  float ln[4][4], dn[4][4];
  auto rows_of = [&](int n) {
    const int hh = kvh * G + n / per, qt = kt + n % per;
    const int64_t sb = ((int64_t)b * a.H + hh) * T;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = min(qt * FR + 16 * t + 4 * g + r, T - 1);
        ln[t][r] = a.lse_in[sb + qq] * kLog2e;
        dn[t][r] = a.delta[sb + qq];
      }
  };
  rows_of(0);
  issue(0, lds);
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
      issue(n + 1, lds + ((n + 1) & 1) * SB);
    }
    const int qt = kt + n % per;
    const int q0 = qt * FR;
    const unsigned base = lds_off(lds + (n & 1) * SB);

    float p[4][4];
    {
      u32x4 qf[4][2];
      rd_rows8(base + off.row[0], base + off.row[1], qf);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
        st = mma(qf[t][0], kf[0], st);
        st = mma(qf[t][1], kf[1], st);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[t][r] = ex2(fmaf(st[r], c2, -lc[t][r]));
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
      rd_rows8(base + FTB + off.row[0], base + FTB + off.row[1], gr);
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
      const u32x4 pb[2] = {pack_k(p[0], p[1]), pack_k(p[2], p[3])};
      u32x4 gt[4][2];
      rd_cols<ND>(base + FTB, off, gt);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) dva[dt] = mma(gt[dt][c], pb[c], dva[dt]);
    }
    {
      const u32x4 db[2] = {pack_k(ds[0], ds[1]), pack_k(ds[2], ds[3])};
      u32x4 qt_[4][2];
      rd_cols<ND>(base, off, qt_);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) dka[dt] = mma(qt_[dt][c], db[c], dka[dt]);
    }
  }

  lds_barrier();
  float* F = reinterpret_cast<float*>(lds);
  float* F2 = reinterpret_cast<float*>(lds + FSB);
  const int row = wave * 16 + (lane & 15);
  fl_stage_acc<ND>(F, row, g, dka);
  fl_stage_acc<ND>(F2, row, g, dva);
  lds_barrier();
  // dK = dS^T Q / sqrt(d), rotated back by RoPE
  fl_store_rows(F, 1.0f / sqrtf((float)a.d), a.dk + (int64_t)b * T * a.lddk + (int64_t)kvh * a.d, a.lddk, k0, T,
                a.d, a.R, a.rope_mode, a.cs);
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
// u = w and w + 8 (16 keys each) of the chunk, their keys, values and
// dK / dV accumulators held in registers.  Query tiles of 64 rows of every
// query head of the group stream through a three-stage LDS ring ([Q | dO |
// lse, D] per stage); each 32-query half is read from LDS once per wave and
// applied to both subtiles: S = Q K^T, P = exp2(c2 S - lse2), dP = dO V^T,
// dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS.  Needs T % 4 == 0
// (16-byte lse / D rows).
// ---------------------------------------------------------------------------
constexpr int KC = 256;               // keys per chunk
constexpr int STB = 2 * FTB + 1024;   // stage bytes: Q, dO, then lse (256 B), D (256 B), pad
constexpr int KC_LDS = 3 * STB > (KC / FR) * FSB ? 3 * STB : (KC / FR) * FSB;  // ring, or the 256-row staging tile

template <bool DROP, int ND>
__global__ __launch_bounds__(512, 1) void fl_dkdv2_k(FlArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[KC_LDS];
  const int T = a.T, G = a.H / a.Hkv, nkc = (T + KC - 1) / KC;
  const int w = fl_work_item();
  const int kc = w % nkc, kvh = (w / nkc) % a.Hkv, b = w / (nkc * a.Hkv);  // earliest keys (most queries) first
  const int k0 = kc * KC;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int nch = a.d / 8;
  const float c2 = a.c2;
  const FlOff off(lane);

  // subtile i: keys k0 + 16 (wave + 8 i) + li
  u32x4 kf[2][2], vf[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kc_ = min(k0 + 16 * (wave + 8 * i) + li, T - 1);
    const bf16* krow = a.k + ((int64_t)b * T + kc_) * a.ldk + (int64_t)kvh * a.d;
    const bf16* vrow = a.v + ((int64_t)b * T + kc_) * a.ldv + (int64_t)kvh * a.d;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      kf[i][s] = ld_frag(krow, s, g, a.d);
      vf[i][s] = ld_frag(vrow, s, g, a.d);
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
    fl_issue8(a.q + (int64_t)b * T * a.ldq + (int64_t)hh * a.d, a.ldq, qt * FR, T, nch, st, wave, lane);
    fl_issue8(a.dout + (int64_t)b * T * a.lddo + (int64_t)hh * a.d, a.lddo, qt * FR, T, nch, st + FTB, wave, lane);
    if (wave == 0) {  // lse then D of the 64 rows: 16 + 16 chunks (lanes 32..63 repeat into the pad)
      const int c = lane & 15;
      const int q = min(qt * FR + 4 * c, T - 4);
      const int64_t hb = (int64_t)(b * a.H + hh) * T;
      const float* src = (lane & 16) ? a.delta + hb + q : a.lse_in + hb + q;
      lds_copy16(src, st + 2 * FTB);
    }
  };
  issue(0, lds);
  issue(min(1, nsteps - 1), lds + STB);
  for (int n = 0; n < nsteps; ++n) {
    SLT_WAIT_VMCNT(2);  // only the next step's copies may still fly (wave 0 waits for one more)
    lds_barrier();
    issue(min(n + 2, nsteps - 1), lds + ((n + 2) % 3) * STB);
    const int qt = qt0 + n % per;
    const int q0 = qt * FR;
    char* stg = lds + (n % 3) * STB;
    const unsigned base = lds_off(stg);
    const unsigned lsd = base + 2 * FTB;  // the stage's lse row (64 floats), then D
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int qh0 = q0 + 32 * hf;  // first query of this half
      if (qh0 >= T || qh0 + 31 < k0 + 16 * wave) continue;  // past T, or before every key of the wave
      u32x4 qf[2][2], gr[2][2];
      rd_rows4(base + off.row[0] + 4096 * hf, base + off.row[1] + 4096 * hf, qf);
      rd_rows4(base + FTB + off.row[0] + 4096 * hf, base + FTB + off.row[1] + 4096 * hf, gr);
      u32x4 pb[2], db[2];
      bool act[2];
      if (qh0 >= k0 + 16 * (wave + 8) + 15 && qh0 + 31 < T) {
        // Every query of the half comes after every key of both subtiles and
        // before T: no mask and both subtiles active, so their steps run
        // side by side (all products, then all probabilities and score
        // gradients).  Same arithmetic as the general path below.
        f32x4 st[2][2], dp[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            st[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              st[i][tt] = mma(qf[tt][s], kf[i][s], st[i][tt]);
              dp[i][tt] = mma(gr[tt][s], vf[i][s], dp[i][tt]);
            }
          }
        float l2[2][4], dn[2][4];
        u32x4 ld4[4];
        rd_lsd(lsd + 4 * (32 * hf + 4 * g), ld4);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            l2[tt][r] = __uint_as_float(ld4[tt][r]) * kLog2e;
            dn[tt][r] = __uint_as_float(ld4[2 + tt][r]);
          }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ki = k0 + 16 * (wave + 8 * i) + li;
          float p[2][4], ds[2][4];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) p[tt][r] = ex2(fmaf(st[i][tt][r], c2, -l2[tt][r]));
            if (DROP) {
              float dm[4];
              drop_mults_strided<4>(a.drop, att_elem(b, a.H, kvh * G + n / per, T, qh0 + 16 * tt + 4 * g, ki),
                                    (uint64_t)T, dm);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                ds[tt][r] = p[tt][r] * (dm[r] * dp[i][tt][r] - dn[tt][r]);
                p[tt][r] *= dm[r];
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) ds[tt][r] = p[tt][r] * (dp[i][tt][r] - dn[tt][r]);
            }
          }
          pb[i] = pack_k(p[0], p[1]);
          db[i] = pack_k(ds[0], ds[1]);
          act[i] = true;
        }
      } else {
      u32x4 ld4[4];
      rd_lsd(lsd + 4 * (32 * hf + 4 * g), ld4);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kf0 = k0 + 16 * (wave + 8 * i);  // first key of subtile i
        act[i] = qh0 + 31 >= kf0;
        if (!act[i]) continue;
        const int ki = kf0 + li;
        float p[2][4], ds[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            st = mma(qf[tt][s], kf[i][s], st);
            dp = mma(gr[tt][s], vf[i][s], dp);
          }
          // lse (to base 2) and D of the lane's 4 query rows
#pragma unroll
          for (int r = 0; r < 4; ++r) p[tt][r] = ex2(fmaf(st[r], c2, -__uint_as_float(ld4[tt][r]) * kLog2e));
          const float dn[4] = {__uint_as_float(ld4[2 + tt][0]), __uint_as_float(ld4[2 + tt][1]),
                               __uint_as_float(ld4[2 + tt][2]), __uint_as_float(ld4[2 + tt][3])};
          if (qh0 < kf0 + 15 || qh0 + 31 >= T) {  // the diagonal, or rows past T
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
        pb[i] = pack_k(p[0], p[1]);
        db[i] = pack_k(ds[0], ds[1]);
      }
      }
      {
        u32x4 gt[4];
        rd_chalf<ND>(base + FTB + 4096 * hf, off, gt);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) dva[i][dt] = mma(gt[dt], pb[i], dva[i][dt]);
        }
      }
      {
        u32x4 qc[4];
        rd_chalf<ND>(base + 4096 * hf, off, qc);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) dka[i][dt] = mma(qc[dt], db[i], dka[i][dt]);
        }
      }
    }
  }
  SLT_WAIT_VMCNT(0);  // no copy may land after the block ends

  // stage the chunk's 256 rows of dK (then dV) as fp32 and store them
  lds_barrier();
  float* F = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i) fl_stage_acc<ND>(F, 16 * (wave + 8 * i) + li, g, dka[i]);
  lds_barrier();
  // dK = dS^T Q / sqrt(d), rotated back by RoPE
  fl_store_rows(F, 1.0f / sqrtf((float)a.d), a.dk + (int64_t)b * T * a.lddk + (int64_t)kvh * a.d, a.lddk, k0, T,
                a.d, a.R, a.rope_mode, a.cs, KC);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < 2; ++i) fl_stage_acc<ND>(F, 16 * (wave + 8 * i) + li, g, dva[i]);
  lds_barrier();
  fl_store_rows(F, 1.0f, a.dv + (int64_t)b * T * a.lddv + (int64_t)kvh * a.d, a.lddv, k0, T, a.d, 0, 0, nullptr, KC);
}

inline bool al(const void* p, int n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

FlArgs to_fl(const AttnArgs& a, const void* q, int64_t ldq, const void* k, int64_t ldk) {
  FlArgs f{};
  f.q = static_cast<const bf16*>(q);
  f.k = static_cast<const bf16*>(k);
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
  f.ldq = ldq;
  f.ldk = ldk;
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
  f.c2 = kLog2e / sqrtf((float)a.d);
  f.drop = a.drop;
  return f;
}

// The rotated q and k the kernels read: in place when the caller's q and k
// already are (or R = 0), else RoPE'd once into the workspace a.rot as
// [B T, H d] then [B T, Hkv d] bf16 rows.
slt_status operands(const AttnArgs& a, hipStream_t s, FlArgs& f) {
  if (a.qk_rotated || a.R == 0) {
    f = to_fl(a, a.q, a.ldq, a.k, a.ldk);
    return SLT_OK;
  }
  const int64_t rows = (int64_t)a.B * a.T, qd = (int64_t)a.H * a.d, kd = (int64_t)a.Hkv * a.d;
  bf16* rq = static_cast<bf16*>(a.rot);
  bf16* rk = rq + rows * qd;
  slt_status st = launch_rope(a.q, a.ldq, rq, qd, rows, a.T, a.H, a.d, a.R, a.rope_mode, a.cs, 1.0f, SLT_BF16, s);
  if (st == SLT_OK) st = launch_rope(a.k, a.ldk, rk, kd, rows, a.T, a.Hkv, a.d, a.R, a.rope_mode, a.cs, 1.0f, SLT_BF16, s);
  f = to_fl(a, rq, qd, rk, kd);
  return st;
}

}  // namespace

int64_t flash_rot_elems(int B, int T, int H, int Hkv, int d) { return (int64_t)B * (H + Hkv) * T * d; }

bool flash_eligible(int dtype, int d) { return dtype == SLT_BF16 && d > 0 && d % 16 == 0 && d <= FD; }

bool flash_ok(const AttnArgs& a, bool bwd) {
  if (!flash_eligible(a.dtype, a.d)) return false;
  const bool need_rot = !a.qk_rotated && a.R > 0;
  if (need_rot && (!a.rot || !al(a.rot, 16))) return false;
  if (!need_rot && (!al(a.q, 16) || !al(a.k, 16) || a.ldq % 8 || a.ldk % 8)) return false;
  if (!al(a.v, 16) || a.ldv % 8) return false;
  if (!bwd) return al(a.out, 8) && a.ldo % 4 == 0 && (!a.ores_out || al(a.ores_out, 8));
  return al(a.o, 16) && a.ldo % 8 == 0 && al(a.dout, 16) && a.lddo % 8 == 0 && (!a.ores_in || al(a.ores_in, 16)) &&
         al(a.dq, 8) && al(a.dk, 8) && al(a.dv, 8) && a.lddq % 4 == 0 && a.lddk % 4 == 0 && a.lddv % 4 == 0 &&
         (a.H * a.d) % 8 == 0;
}

slt_status flash_fwd(const AttnArgs& a, hipStream_t s) {
  FlArgs f;
  if (slt_status st = operands(a, s, f); st != SLT_OK) return st;
  // 128-query chunks (two subtiles per wave) from T = 2048 on: the longest
  // chunks there hold 32 key tiles, and halving them evens out the last round
  // of the grid (measured: 11 % faster at T = 2048, 2 % slower at T = 1024
  // and 14 % slower at T = 256)
  auto go = [&](auto ns, auto nd) {
    constexpr int NS = decltype(ns)::value, ND = decltype(nd)::value;
    const int nck = (a.T + 64 * NS - 1) / (64 * NS);
    if (a.drop.on) fl_fwd_k<true, NS, ND><<<nck * a.H * a.B, 256, 0, s>>>(f);
    else fl_fwd_k<false, NS, ND><<<nck * a.H * a.B, 256, 0, s>>>(f);
  };
  auto go_nd = [&](auto ns) {
    if (a.d <= 48) go(ns, std::integral_constant<int, 3>{});
    else go(ns, std::integral_constant<int, 4>{});
  };
  if (a.T >= 2048) go_nd(std::integral_constant<int, 2>{});
  else go_nd(std::integral_constant<int, 4>{});
  return check_launch("attention forward");
}

slt_status flash_bwd(const AttnArgs& a, hipStream_t s) {
  FlArgs f;
  if (slt_status st = operands(a, s, f); st != SLT_OK) return st;
  const int nt = (a.T + FR - 1) / FR;
  auto go = [&](auto nd) {
    constexpr int ND = decltype(nd)::value;
    if (a.drop.on) fl_dq_k<true, ND><<<nt * a.H * a.B, 256, 0, s>>>(f);
    else fl_dq_k<false, ND><<<nt * a.H * a.B, 256, 0, s>>>(f);
    slt_status st = check_launch("attention backward (dq)");
    if (st != SLT_OK) return st;
    if (a.T % 4 == 0 && al(a.lse_in, 16) && al(a.delta, 16)) {
      const int nkc = (a.T + KC - 1) / KC;
      if (a.drop.on) fl_dkdv2_k<true, ND><<<nkc * a.Hkv * a.B, 512, 0, s>>>(f);
      else fl_dkdv2_k<false, ND><<<nkc * a.Hkv * a.B, 512, 0, s>>>(f);
    } else {
      if (a.drop.on) fl_dkdv_k<true, ND><<<nt * a.Hkv * a.B, 256, 0, s>>>(f);
      else fl_dkdv_k<false, ND><<<nt * a.Hkv * a.B, 256, 0, s>>>(f);
    }
    return check_launch("attention backward (dk, dv)");
  };
  if (a.d <= 48) return go(std::integral_constant<int, 3>{});
  return go(std::integral_constant<int, 4>{});
}

}  // namespace slt
