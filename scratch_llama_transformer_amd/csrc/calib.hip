// Machine bounds measured with the library's own code: a streaming copy (the
// HBM read + write rate a bandwidth-bound kernel can reach) and a loop of
// independent bf16 MFMAs (the matrix-core rate).  strata's benchmark reports
// kernels as a fraction of a measured machine bound; these two kernels give
// that bound on the GPU the library runs on.
#include "slt_internal.h"

namespace slt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// dst[i] = src[i] over n 16-byte words: each thread moves 4 words per
// iteration (all loads issued before the stores), grid-stride.
__global__ __launch_bounds__(256) void stream_copy_k(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// Each wave runs `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16
// (16384 FLOP each) on register operands, then writes its accumulators so
// that none of the work is dead.
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
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace slt

using namespace slt;

extern "C" {

slt_status slt_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(SLT_EINVAL, "stream_copy: bytes must be a non-negative multiple of 16");
  if (bytes == 0) return SLT_OK;
  if (!src || !dst || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return fail(SLT_EINVAL, "stream_copy: NULL or misaligned buffer");
  const int64_t n = bytes / 16;
  const int blocks = (int)std::min<int64_t>((n + 1023) / 1024, 256 * 16);
  stream_copy_k<<<blocks, 256, 0, as_stream(stream)>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return check_launch("stream_copy");
}

int64_t slt_mfma_loop_flops(int32_t blocks, int32_t iters) {
  return (int64_t)blocks * 4 * iters * 8 * 16384;
}

slt_status slt_mfma_loop(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return fail(SLT_EINVAL, "mfma_loop: bad arguments");
  mfma_loop_k<<<blocks, 256, 0, as_stream(stream)>>>(iters, out);
  return check_launch("mfma_loop");
}

}  // extern "C"
