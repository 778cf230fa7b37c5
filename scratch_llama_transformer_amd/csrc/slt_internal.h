// Internal declarations shared by the HIP translation units of libslt.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/slt.h"

namespace slt {

// ---------------------------------------------------------------------------
// Storage types.  bf16 is the upper half of an IEEE binary32.
// ---------------------------------------------------------------------------
struct bf16 {
  uint16_t u;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(((uint32_t)x.u) << 16); }

// Round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32 (what clang
// emits for a float -> __bf16 conversion) rounds in the IEEE default mode,
// keeps binary32 subnormals (the default f32 denormal mode preserves them)
// and turns NaNs into quiet NaNs.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two values in one conversion: a in the low half, b in the high half.
typedef __bf16 slt_bf16x2 __attribute__((ext_vector_type(2)));
typedef float slt_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(slt_f32x2{a, b}, slt_bf16x2));
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes) without LDS: DPP row_mirror, row_half_mirror
// and two quad permutations sum each 16-lane row, v_permlane16_swap and
// v_permlane32_swap (gfx950) then combine the four rows.  Every step adds a
// value to its partner's with both orders giving the same float, so all 64
// lanes end with bitwise the same result.  (A __shfl_xor ladder compiles to
// six ds_bpermute LDS round trips.)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0x140>(v);  // row_mirror: lane i with 15 - i
  v += dpp_mov<0x141>(v);  // row_half_mirror: lane i with 7 - i in each half row
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0x140>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0xB1>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---------------------------------------------------------------------------
// Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64 multiplies with the
// key bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
__host__ __device__ inline void philox4x32_10(const uint32_t in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// Inverted dropout of one site (Hephaistos, "Architecture at a glance";
// randyGPT, "Architecture Details"): element e of the site's [rows, C] tensor
// (e = row C + column) is kept iff word e % 4 of Philox-4x32-10 at counter
// (e / 4 low, e / 4 high, site, layer) under the seed is >= thr = floor(p
// 2^32); a kept value is multiplied by scale = float(1 / (1 - p)).  The
// backward regenerates the same words.
struct Drop {
  bool on = false;
  uint32_t thr = 0, k0 = 0, k1 = 0;
  int site = 0, layer = 0;
  float scale = 1.f;
};

// Multiplier (0 or scale) of element e.
__device__ __forceinline__ float drop_mult(const Drop& d, uint64_t e) {
  const uint64_t q = e >> 2;
  const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), (uint32_t)d.site, (uint32_t)d.layer};
  const uint32_t key[2] = {d.k0, d.k1};
  uint32_t w[4];
  philox4x32_10(ctr, key, w);
  const uint32_t r = (e & 3) == 0 ? w[0] : (e & 3) == 1 ? w[1] : (e & 3) == 2 ? w[2] : w[3];
  return r >= d.thr ? d.scale : 0.f;
}

// Multipliers of elements e0 .. e0 + N - 1 (one generator call per aligned
// group of four).
template <int N>
__device__ __forceinline__ void drop_mults(const Drop& d, uint64_t e0, float (&m)[N]) {
  if ((e0 & 3) == 0 && N % 4 == 0) {
#pragma unroll
    for (int g = 0; g < N / 4; ++g) {
      const uint64_t q = (e0 >> 2) + g;
      const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), (uint32_t)d.site, (uint32_t)d.layer};
      const uint32_t key[2] = {d.k0, d.k1};
      uint32_t w[4];
      philox4x32_10(ctr, key, w);
#pragma unroll
      for (int r = 0; r < 4; ++r) m[4 * g + r] = w[r] >= d.thr ? d.scale : 0.f;
    }
  } else {
#pragma unroll
    for (int r = 0; r < N; ++r) m[r] = drop_mult(d, e0 + r);
  }
}

// Multipliers of elements e0, e0 + stride, ... (one generator call each).
template <int N>
__device__ __forceinline__ void drop_mults_strided(const Drop& d, uint64_t e0, uint64_t stride, float (&m)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) m[r] = drop_mult(d, e0 + r * stride);
}

// Element of attention weight (query i, key j) of head h of sequence b: the
// weights of one head form a T x T block, the blocks ordered by (b, h).
__device__ __forceinline__ uint64_t att_elem(int b, int H, int h, int T, int i, int j) {
  return (uint64_t)(((int64_t)b * H + h) * T + i) * (uint64_t)T + (uint64_t)j;
}

// SwiGLU (Hephaistos, "Architecture at a glance": silu(x W1) * (x W3)), shared
// by the element kernels and the fused GEMM epilogues so both compute the
// same expression: h = a sigmoid(a) b; db = dh a sigmoid(a),
// da = dh b sigmoid(a) (1 + a (1 - sigmoid(a))).
__device__ __forceinline__ float slt_sigmoid(float a) { return 1.0f / (1.0f + __expf(-a)); }
__device__ __forceinline__ float swiglu_h(float a, float b) { return a * slt_sigmoid(a) * b; }
__device__ __forceinline__ void swiglu_grad(float a, float b, float dh, float& da, float& db) {
  const float sg = slt_sigmoid(a);
  db = dh * a * sg;
  da = dh * b * sg * (1.0f + a * (1.0f - sg));
}

// GELU, tanh form (the GPT-2 / CodeGen family's): 0.5 x (1 + tanh(y)),
// y = sqrt(2/pi) (x + 0.044715 x^3), evaluated as x sigmoid(2y) -- the same
// function with one exponential and one reciprocal instead of a tanh (the
// element kernels are otherwise bound by its instruction count).  Derivative:
// s + x s (1 - s) 2 sqrt(2/pi) (1 + 3 * 0.044715 x^2), s = sigmoid(2y).
__device__ __forceinline__ float gelu_sig(float x) {
  const float y2 = 1.5957691216057308f * (x + 0.044715f * x * x * x);
  return __builtin_amdgcn_rcpf(1.0f + __expf(-y2));
}
__device__ __forceinline__ float gelu_tanh(float x) { return x * gelu_sig(x); }
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  const float s = gelu_sig(x);
  return s + 1.5957691216057308f * x * (1.0f + 0.134145f * x * x) * s * (1.0f - s);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return bf16{f32_to_bf16_bits(x)}; }

// ---------------------------------------------------------------------------
// Direct HBM -> LDS copies (gfx950 global_load_lds_dwordx4).  Lane i of one
// instruction writes the 16 bytes it fetched to LDS at (dst of lane 0) + 16 i:
// the LDS layout is decided by which global chunk each lane fetches.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_copy16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
}

// LDS byte offset of a pointer into a __shared__ array: the generic address
// is the LDS aperture (upper 32 bits) plus the offset.
__device__ __forceinline__ unsigned lds_off(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>(p));
}

// Workgroup barrier that orders LDS accesses only; copies into LDS are
// waited for explicitly (vmcnt) by each wave before it arrives.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
#define SLT_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt((((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14)))

// ---------------------------------------------------------------------------
// Error reporting (thread-local message)
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
slt_status fail(slt_status code, const std::string& msg);
slt_status check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// Kernel launchers (return hipSuccess or the launch error)
// ---------------------------------------------------------------------------
// RoPE applied in a projection's epilogue: output columns [0, end) are heads
// of d dims whose first R dims are rotated by the angle of row m's position
// m % T (cs: the [T][R] table of (cos, sin) pairs), in fp32 before the
// rounding to bf16.  half: rotate-half pairs (j, j + R/2), else even-odd.
struct RopeEpi {
  const float* cs = nullptr;
  int T = 1, d = 1, R = 0, end = 0;
  int half = 0;
};

struct GemmArgs {
  int M, N, K;
  const void* A; int64_t lda; bool a_kmajor;
  const void* B; int64_t ldb; bool b_kmajor;
  void* C; int64_t ldc;
  const void* R; int64_t ldr;
  int in_dtype, out_dtype;
  float* workspace; int64_t workspace_bytes;
  float alpha = 1.0f;  // C = alpha A B (+ R)
  Drop drop{};         // C = drop(alpha A B) + R: element (m, n) is e = m N + n of the site
};

// How a parameter-gradient kernel writes its result g: out = alpha g, or
// out += alpha g when accumulating over micro-batches.
struct GradW {
  float alpha = 1.0f;
  bool accumulate = false;
};
slt_status launch_gemm(const GemmArgs& g, hipStream_t s);
// y = x W^T with the RoPE epilogue (bf16, both operands k-major, no residual,
// alpha 1); SLT_EUNSUPPORTED, nothing enqueued, where it does not apply.
slt_status launch_gemm_rope(const GemmArgs& g, const RopeEpi& r, hipStream_t s);
// RoPE on the first R dims of each of nh heads (d dims, head h at column h d)
// of rows r = b T + t, position t = r % T: y = rotate(x) (sign 1) or the
// transposed rotation (sign -1, RoPE's backward); dims >= R are copied.
// y may equal x (in place).
slt_status launch_rope(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int T, int nh, int d, int R,
                       int mode, const float* cs, float sign, int dtype, hipStream_t s);

// [W1; W3] projection fused with SwiGLU: ab[M, 2F] = X[M, K] W13[2F, K]^T
// (a | b, bf16, row stride ldab) and h[M, F] = swiglu(bf16(a), bf16(b)).
// SLT_EUNSUPPORTED (nothing enqueued) where the fused kernel does not apply.
slt_status launch_gemm_swiglu_fwd(int M, int F, int K, const void* X, int64_t ldx, const void* W13, void* ab,
                                  int64_t ldab, void* h, int64_t ldh, hipStream_t s);

// One product of a grouped weight-gradient launch: C[M, N] (fp32, row stride
// ldc) = alpha sum_k A[k lda + m] B[k ldb + n] (+ C when accumulate), bf16
// operands with rows of tokens.  All products of a group share K.
struct GroupItem {
  int M, N;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  float* C; int64_t ldc;
  float alpha;
  bool accumulate;
};
bool gemm_group_ok(const GroupItem& it, int K);
slt_status launch_gemm_group(const GroupItem* items, int n, int K, float* ws, int64_t ws_bytes, hipStream_t s);

slt_status launch_embedding_fwd(const int32_t* tok, int B, int T, int64_t ld, const void* wte,
                                void* x, int V, int C, int dtype, hipStream_t s, Drop drop = {});
int64_t embedding_bwd_ws(int64_t N, int V);
// The embedding gradient in two phases: the stable sort of token positions
// by id (tokens only), then the per-id sums of dx rows; launch_embedding_bwd
// runs the sort itself unless `sorted` says it already ran on ws.
slt_status launch_embedding_sort(const int32_t* tok, int B, int T, int64_t ld, int V, void* ws, hipStream_t s);
slt_status launch_embedding_bwd(const int32_t* tok, int B, int T, int64_t ld, const void* dx,
                                float* dwte, int V, int C, int dtype, void* ws, hipStream_t s, GradW gw = {},
                                Drop drop = {}, bool sorted = false);
slt_status launch_drop_apply(const void* g, void* out, int rows, int C, int dtype, Drop drop, hipStream_t s);
int64_t norm_bwd_ws(int rows, int C);
slt_status launch_rmsnorm_fwd(const void* x, const void* g, void* y, float* rstd, int rows, int C,
                              float eps, int dtype, hipStream_t s);
// Norm backward: the row kernel writes dx and per-block partials of the gain
// (and bias) gradients into ws; launch_norm_colsum reduces them, which the
// launch does itself unless defer_sums (the caller then runs it, on any
// stream ordered after this launch, before ws is reused).
slt_status launch_norm_colsum(const void* ws, int rows, int C, float* dg, float* db, hipStream_t s, GradW gw);
slt_status launch_rmsnorm_bwd(const void* x, const void* g, const float* rstd, const void* dy,
                              const void* dres, void* dx, float* dg, int rows, int C, int dtype,
                              void* ws, hipStream_t s, GradW gw = {}, bool defer_sums = false);
slt_status launch_layernorm_fwd(const void* x, const void* gm, const void* bt, void* y, float* mean,
                                float* rstd, int rows, int C, float eps, int dtype, hipStream_t s);
slt_status launch_layernorm_bwd(const void* x, const void* gm, const float* mean, const float* rstd,
                                const void* dy, const void* dres, void* dx, float* dgm, float* dbt,
                                int rows, int C, int dtype, void* ws, hipStream_t s, GradW gw = {},
                                bool defer_sums = false);
slt_status launch_rope_table(int T, int R, float base, float* cs, hipStream_t s);
slt_status launch_swiglu_fwd(const void* a, const void* b, void* h, int rows, int F, int64_t lda,
                             int64_t ldb, int64_t ldh, int dtype, hipStream_t s);
slt_status launch_swiglu_bwd(const void* a, const void* b, const void* dh, void* da, void* db,
                             int rows, int F, int64_t lda, int64_t ldb, int64_t lddh, int64_t ldda,
                             int64_t lddb, int dtype, hipStream_t s);
slt_status launch_gelu_fwd(const void* a, void* u, int rows, int F, int64_t lda, int64_t ldu,
                           int dtype, hipStream_t s);
slt_status launch_gelu_bwd(const void* a, const void* du, void* da, int rows, int F, int64_t lda,
                           int64_t lddu, int64_t ldda, int dtype, hipStream_t s);
slt_status launch_softmax_xent(void* z, int64_t ldz, const int32_t* tok, int B, int T, int64_t ld,
                               int V, float* loss, float* lse, int dtype, void* ws, hipStream_t s);
slt_status launch_adamw(int64_t n, float* master, uint16_t* shadow, const float* g, float* m,
                        float* v, int64_t t, float lr, float b1, float b2, float eps, float wd,
                        const uint8_t* mask, const float* gscale, hipStream_t s);
int64_t grad_norm_ws();
slt_status launch_grad_norm(int64_t n, const float* g, int kind, float max_norm, float* norm, float* scale,
                            void* ws, hipStream_t s);
slt_status launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
slt_status launch_fill_f32(float* dst, float value, int64_t n, hipStream_t s);
// *dst += a * (*x) on the device (one value)
slt_status launch_scalar_axpy(float* dst, float a, const float* x, hipStream_t s);
slt_status launch_model_init_range(float* dst, int64_t n, int64_t index0, uint64_t seed, float std,
                                   int kind, hipStream_t s);

struct AttnArgs {
  const void *q, *k, *v, *o, *dout;
  void *dq, *dk, *dv, *out;
  float* lse;
  const float* lse_in;
  int64_t ldq, ldk, ldv, ldo, lddo, lddq, lddk, lddv;
  int B, T, H, Hkv, d, R, rope_mode, dtype;
  const float* cs;
  float* delta;        // workspace [B, H, T] for the backward
  void* ores_out;      // forward: optional o - bf16(o), dense [B*T, H*d]
  const void* ores_in; // backward: that residual (NULL: treat as 0)
  bool qk_rotated;     // q and k already carry RoPE (the projection's epilogue applied it; bf16 path only):
                       // no rotation on load, but dq and dk are still rotated back
  void* rot;           // bf16 path with q, k not yet rotated: workspace for their rotated copies
                       // (flash_rot_elems bf16 values)
  Drop drop{};         // dropout of the attention weights: element ((b H + h) T + i) T + j
};
slt_status launch_attention_fwd(const AttnArgs& a, hipStream_t s);
slt_status launch_attention_bwd(const AttnArgs& a, hipStream_t s);
int64_t attention_bwd_ws(int B, int H, int T);
// bf16 attention on rotated bf16 q/k with LDS tiles copied straight from HBM
// (flash.hip)
int64_t flash_rot_elems(int B, int T, int H, int Hkv, int d);
bool flash_eligible(int dtype, int d);
bool flash_ok(const AttnArgs& a, bool bwd);
slt_status flash_fwd(const AttnArgs& a, hipStream_t s);
slt_status flash_bwd(const AttnArgs& a, hipStream_t s);

// Key/value cache (decode.hip): append rotated keys and values of Tq new rows
// per sequence at positions pos0.., and attend those rows over the cache.
slt_status launch_kv_append(const void* qkv, int64_t ld, float* qrot, int B, int Tq, int pos0, int H, int Hkv, int d,
                            int R, int mode, const float* cs, void* Kc, void* Vc, int Tmax, int dtype, hipStream_t s);
int64_t decode_attention_ws(int B, int Tq, int H, int Hkv, int d, int Tmax);
slt_status launch_attention_decode(const float* qrot, const void* Kc, const void* Vc, void* out, int64_t ldo, int B,
                                   int Tq, int pos0, int H, int Hkv, int d, int Tmax, int dtype, float* ws,
                                   hipStream_t s);

}  // namespace slt
