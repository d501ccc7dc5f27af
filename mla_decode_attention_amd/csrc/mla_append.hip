// Latent-KV append for gfx950: store each sequence's newest latent rows in
// their cache pages, the step before attention in a decode step. The 8-bit
// cache form (C8 among the cache precisions of PaddleNLP issue #10157's
// overview) is OCP E4M3FN codes with one fp32 scale per token.
//
// One wave per new token. bf16 cache: a 1152-byte copy (16 bytes per lane).
// fp8 cache: lane l holds dims 9l..9l+8; the wave reduces max|x|, every lane
// derives the same scale = max|x| / 448 (1 for an all-zero row), divides its
// values by it (IEEE fp32 division), clamps to +-448 and converts with
// v_cvt_pk_fp8_f32 (OCP E4M3FN on gfx950, round to nearest even).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTokensPerBlock = 4;   // one wave each
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}

__global__ __launch_bounds__(64 * kTokensPerBlock) void append_kernel(
    const uint16_t* __restrict__ latent, int batch, int new_tokens, const int32_t* __restrict__ block_table,
    int max_pages, const int32_t* __restrict__ seqlens, uint8_t* __restrict__ kv, float* __restrict__ kv_scale,
    int fp8, int num_pages) {
  const int lane = threadIdx.x & 63;
  const long long g = (long long)blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
  if (g >= (long long)batch * new_tokens) return;
  const int b = (int)(g / new_tokens), i = (int)(g % new_tokens);
  const int j = seqlens[b] - new_tokens + i;
  if (j < 0) return;
  const int page_idx = j / kPage;
  if (page_idx >= max_pages) return;
  const int page = block_table[(size_t)b * max_pages + page_idx];
  if (page < 0 || page >= num_pages) return;
  const size_t row = (size_t)page * kPage + (j % kPage);
  const uint16_t* src = latent + (size_t)g * kDqk;

  if (!fp8) {
    // 72 chunks of 16 bytes
    const uint4* s4 = (const uint4*)src;
    uint4* d4 = (uint4*)(kv + row * kDqk * 2);
    for (int c = lane; c < kDqk / 8; c += 64) d4[c] = s4[c];
    return;
  }

  float x[9];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 9; ++e) {
    const uint32_t bits = (uint32_t)src[9 * lane + e] << 16;
    x[e] = __builtin_bit_cast(float, bits);
    amax = fmaxf(amax, fabsf(x[e]));
  }
  amax = wave_max(amax);
  const float scale = amax > 0.f ? amax / kE4m3Max : 1.0f;
  uint8_t* dst = kv + row * kDqk + 9 * lane;
  auto clamp448 = [](float v) { return fminf(fmaxf(v, -kE4m3Max), kE4m3Max); };
#pragma unroll
  for (int e = 0; e < 9; e += 2) {
    const float y0 = clamp448(x[e] / scale);
    const float y1 = e + 1 < 9 ? clamp448(x[e + 1] / scale) : 0.f;
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    dst[e] = (uint8_t)(packed & 0xFF);
    if (e + 1 < 9) dst[e + 1] = (uint8_t)((packed >> 8) & 0xFF);
  }
  if (lane == 0) kv_scale[row] = scale;
}

}  // namespace

hipError_t launch_append(const uint16_t* latent, int batch, int new_tokens, const int32_t* block_table,
                         int max_pages, const int32_t* seqlens, uint8_t* kv, float* kv_scale, int fp8,
                         int num_pages, hipStream_t s) {
  const long long tokens = (long long)batch * new_tokens;
  const unsigned blocks = (unsigned)((tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(64 * kTokensPerBlock), 0, s, latent, batch, new_tokens,
                     block_table, max_pages, seqlens, kv, kv_scale, fp8, num_pages);
  return hipGetLastError();
}

}  // namespace mla
