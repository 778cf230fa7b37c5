// Machine bounds measured with the library's own code: a streaming copy (the
// HBM read + write rate a bandwidth-bound kernel can reach) and a loop of
// independent bf16 MFMAs (the matrix-core rate).  strata's benchmark reports
// kernels as a fraction of a measured machine bound; these two kernels give
// that bound on the GPU the library runs on.
#include "slt_internal.h"

#include <algorithm>

namespace slt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// dst[i] = src[i] over n 16-byte words: each thread moves U words per
// iteration (all loads issued before the stores; a wave's U loads cover U
// whole KiB), grid-stride.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT = true, int NTH = 256>
__global__ __launch_bounds__(NTH) void stream_copy_k(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (NT) __builtin_nontemporal_store(v[u], dst + i + u * stride);
      else dst[i + u * stride] = v[u];
    }
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave runs `iters` rounds of CH independent MFMAs on register operands
// -- v_mfma_f32_16x16x32_bf16 (16384 FLOP) or, with BIG,
// v_mfma_f32_32x32x16_bf16 (32768 FLOP) -- then writes its accumulators so
// that none of the work is dead.
template <bool BIG, int CH>
__global__ __launch_bounds__(256) void mfma_loop_k(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  unsigned av[4], bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    av[i] = 0x3f803f80u ^ (lane + i);  // bf16 pairs near 1
    bv[i] = 0x3f803f80u ^ (lane * 3 + i);
  }
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
  float s = 0.f;
  if constexpr (BIG) {
    f32x16 acc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) acc[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < CH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
  } else {
    f32x4 acc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < CH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace slt

using namespace slt;

extern "C" {

slt_status slt_stream_copy(const void* src, void* dst, int64_t bytes, int32_t variant, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(SLT_EINVAL, "stream_copy: bytes must be a non-negative multiple of 16");
  if (variant < 0 || variant > 4) return fail(SLT_EINVAL, "stream_copy: variant must be 0, 1, 2, 3 or 4");
  if (bytes == 0) return SLT_OK;
  if (!src || !dst || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return fail(SLT_EINVAL, "stream_copy: NULL or misaligned buffer");
  const int64_t n = bytes / 16;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  hipStream_t st = as_stream(stream);
  // variant 0: 4 words per thread per iteration on 8192 blocks; 1: 8 words on
  // 4096 blocks; 2: one pass, 4 words per thread, as many blocks as that
  // needs; 3: as 2 with ordinary (cached) loads and stores; 4: as 2 with
  // 1024-thread blocks (a quarter of the workgroups to dispatch)
  const int one_pass = (int)std::min<int64_t>((n + 1023) / 1024, 1 << 20);
  if (variant == 0) stream_copy_k<4><<<(int)std::min<int64_t>((n + 1023) / 1024, 8192), 256, 0, st>>>(s, d, n);
  else if (variant == 1) stream_copy_k<8><<<(int)std::min<int64_t>((n + 2047) / 2048, 4096), 256, 0, st>>>(s, d, n);
  else if (variant == 2) stream_copy_k<4><<<one_pass, 256, 0, st>>>(s, d, n);
  else if (variant == 3) stream_copy_k<4, false><<<one_pass, 256, 0, st>>>(s, d, n);
  else stream_copy_k<4, true, 1024><<<(int)std::min<int64_t>((n + 4095) / 4096, 1 << 20), 1024, 0, st>>>(s, d, n);
  return check_launch("stream_copy");
}

int64_t slt_mfma_loop_flops(int32_t blocks, int32_t iters, int32_t variant) {
  const int64_t per = variant == 1 ? 8 * 32768 : variant == 2 ? 16 * 16384 : 8 * 16384;
  return (int64_t)blocks * 4 * iters * per;
}

slt_status slt_mfma_loop(int32_t blocks, int32_t iters, int32_t variant, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out || variant < 0 || variant > 2)
    return fail(SLT_EINVAL, "mfma_loop: bad arguments");
  hipStream_t s = as_stream(stream);
  if (variant == 0) mfma_loop_k<false, 8><<<blocks, 256, 0, s>>>(iters, out);
  else if (variant == 1) mfma_loop_k<true, 8><<<blocks, 256, 0, s>>>(iters, out);
  else mfma_loop_k<false, 16><<<blocks, 256, 0, s>>>(iters, out);
  return check_launch("mfma_loop");
}

}  // extern "C"
