// Quantised prefill / extend attention: INT8 Q.K^T, FP8 P.V (gfx950).
//
// The method of PaddleNLP issue #10157's quantization section (SageAttention
// for DeepSeek, head dim 192): Q and K are quantised on the fly to INT8 and V
// to FP8; the INT32 products Q.K^T are turned into FP32 and dequantised for an
// online softmax whose P is quantised to FP8 and multiplied with the FP8 V;
// the product is dequantised once.
//
// Formats (block sizes and scale rules are not fixed by the pages):
//   Q: INT8, one scale per (query token, head) = max|q| / 127 over 192 features;
//   K: INT8, one scale per (sequence, 64-key tile, head) over the tile's valid
//      keys x 192 features;
//   V: E4M3FN, one power-of-two scale 2^e per (32-key block, feature), e the
//      smallest integer with max|v| <= 448 * 2^e, kept as its E8M0 byte
//      127 + e so that the FP8 MFMA applies it itself;
//   P: E4M3FN of P * 2^8 (P <= 1: the running max is always raised to the
//      tile's max), unit MFMA scale; the row sum l adds the unquantised P * 2^8.
//
// quant_kv_kernel (one workgroup per (64-key tile, head)) writes K and V in the
// order the attention kernel's MFMA operands take them; prefill_q8_kernel has
// the bf16 prefill kernel's shape (128 query rows of one (sequence, head) per
// workgroup, 4 waves x 32 rows, 64-key tiles through LDS, double buffered,
// direct global->LDS loads; three workgroups per CU) with
//   the query rows quantised in registers at the start (B operand of
//       S^T = K Q^T: k-step c holds features 32c + 16h .. +15 of row n);
//   QK on v_mfma_i32_32x32x32_i8, 12 per tile and wave, dequantised by one
//       multiply per score (q scale x k scale x softmax scale x log2 e);
//   PV on v_mfma_scale_f32_32x32x64_f8f6f4, 4 per tile and wave: O^T[32
//       features, 32 rows] += V^T P^T, where P^T is the score accumulator
//       converted to E4M3 in place (bytes 0-15 of a lane are its 16 registers
//       of key block 0, bytes 16-31 those of block 1) and V^T is stored by the
//       quantiser with the matching key order.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <math.h>

#include "mla_device.h"

namespace mla {
namespace q8 {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;

constexpr int kTile = 64, kDNope = 128, kDRope = 64, kDK = 192, kDV = 128;
constexpr int kKBytes = kTile * kDK;      // 12288: 12 fragments of 1 KiB
constexpr int kVBytes = kTile * kDV;      // 8192: 8 fragments of 1 KiB
constexpr int kVsBytes = 256;             // E8M0 bytes: 64 lanes x 4 feature blocks
constexpr int kStage = kKBytes + kVBytes + kVsBytes;
static_assert(kKBytes == 12288 && kVBytes == 8192 && kVsBytes == 256, "record sizes of qkv_layout");
constexpr int kRowsWg = 128;
constexpr int kThreads = 256;
constexpr int kPShift = 8;                // P is stored as P * 2^8
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// INT8 code of x: rint(x * inv) clamped to +-127, as a byte
__device__ __forceinline__ uint32_t i8code(float x, float inv) {
  const float r = fminf(fmaxf(rintf(x * inv), -127.f), 127.f);
  return (uint32_t)((int)r & 0xFF);
}

// Tile index of (sequence b, tile t): cu_k[b] / 64 + b + t. These bases grow by
// at least 1 + (tiles of b) from one sequence to the next, so the tiles of
// all sequences get distinct indices below total_k / 64 + batch.
__device__ __forceinline__ int tile_base(const int32_t* cu_k, int b) { return cu_k[b] / kTile + b; }

// K and V of one (64-key tile, head) -> the quantised layout:
//   k8[T][h] byte f*1024 + l*16 + i: code of K[key 32(f/6) + l%32][feature
//       32(f%6) + 16(l/32) + i] (features 0-127: the head's k_nope, 128-191:
//       k_rope); ks[T][h]: its fp32 scale;
//   v8[T][h] byte (2fb + q)*1024 + l*16 + i: code of V[key 32q + 8(i/4) +
//       4(l/32) + i%4][feature 32fb + l%32];
//   vs[T][h] byte 4l + fb: E8M0 byte of (feature 32fb + l%32, key block l/32).
// Keys past the sequence's end get code 0.
__global__ __launch_bounds__(kThreads) void quant_kv_kernel(const uint16_t* __restrict__ k_nope,
                                                           const uint16_t* __restrict__ k_rope,
                                                           const uint16_t* __restrict__ v,
                                                           const int32_t* __restrict__ cu_k, int batch, int H,
                                                           uint8_t* __restrict__ k8, uint8_t* __restrict__ v8,
                                                           uint8_t* __restrict__ vs, float* __restrict__ ks) {
  __shared__ float s_red[4];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kTile * kDV];
  __shared__ int s_e[2][kDV];
  const int T = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  // the sequence whose tiles cover T: the largest b with tile_base(b) <= T
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_base(cu_k, mid) <= T) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int k0 = cu_k[b], L = cu_k[b + 1] - k0;
  const int t = T - tile_base(cu_k, b);
  if (t < 0 || t * kTile >= L) return;   // an index between two sequences' tiles
  const int nvalid = min(kTile, L - t * kTile);
  const size_t key0 = (size_t)k0 + (size_t)t * kTile;
  const size_t rec = (size_t)T * H + head;

  // ---- K: 768 chunks of 16 codes, 3 per thread
  u32x4 raw[3][2];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int ch = tid + kThreads * r, f = ch >> 6, l = ch & 63;
    const int key = 32 * (f / 6) + (l & 31), feat = 32 * (f % 6) + 16 * (l >> 5);
    if (key < nvalid) {
      const uint16_t* src = feat < kDNope ? k_nope + ((key0 + key) * H + head) * kDNope + feat
                                          : k_rope + (key0 + key) * kDRope + (feat - kDNope);
      raw[r][0] = *(const u32x4*)src;
      raw[r][1] = *(const u32x4*)(src + 8);
    } else {
      raw[r][0] = raw[r][1] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t u = raw[r][w >> 2][w & 3];
      amax = fmaxf(amax, fmaxf(fabsf(bf16f(u & 0xFFFF)), fabsf(bf16f(u >> 16))));
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) s_red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float inv = amax > 0.f ? 127.f / amax : 0.f;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int ch = tid + kThreads * r;
    uint32_t w4[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t u0 = raw[r][w >> 1][2 * (w & 1)], u1 = raw[r][w >> 1][2 * (w & 1) + 1];
      w4[w] = i8code(bf16f(u0 & 0xFFFF), inv) | (i8code(bf16f(u0 >> 16), inv) << 8) |
              (i8code(bf16f(u1 & 0xFFFF), inv) << 16) | (i8code(bf16f(u1 >> 16), inv) << 24);
    }
    *(uint4*)(k8 + rec * kKBytes + (size_t)ch * 16) = uint4{w4[0], w4[1], w4[2], w4[3]};
  }
  if (tid == 0) ks[rec] = amax > 0.f ? amax / 127.f : 1.f;

  // ---- V: stage the tile's rows (bf16) in LDS, tail keys zero
  for (int i = tid; i < kTile * (kDV / 8); i += kThreads) {
    const int key = i >> 4, pc = i & 15;
    const uint4 val = key < nvalid ? *(const uint4*)(v + ((key0 + key) * H + head) * kDV + pc * 8) : uint4{0, 0, 0, 0};
    *(uint4*)&s_v[key * kDV + pc * 8] = val;
  }
  __syncthreads();
  {
    // exponent of (key block q, feature d)
    const int d = tid & (kDV - 1), q = tid >> 7;
    float am = 0.f;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) am = fmaxf(am, fabsf(bf16f(s_v[(32 * q + k) * kDV + d])));
    int e = 0;
    if (am > 0.f) {
      int E;
      const float m = frexpf(am, &E);
      e = m <= 0.875f ? E - 9 : E - 8;
      e = min(127, max(-127, e));
    }
    s_e[q][d] = e;
    vs[rec * kVsBytes + ((d & 31) + 32 * q) * 4 + (d >> 5)] = (uint8_t)(127 + e);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int ch = tid + kThreads * r, g = ch >> 6, l = ch & 63;
    const int q = g & 1, d = 32 * (g >> 1) + (l & 31), hh = l >> 5;
    const int e = s_e[q][d];
    uint32_t w4[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 32 * q + 8 * w + 4 * hh + j;     // byte 4w + j of the chunk
        y[j] = fminf(fmaxf(ldexpf(bf16f(s_v[key * kDV + d]), -e), -kE4m3Max), kE4m3Max);
      }
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
      w4[w] = (uint32_t)pk;
    }
    *(uint4*)(v8 + rec * kVBytes + (size_t)ch * 16) = uint4{w4[0], w4[1], w4[2], w4[3]};
  }
}

struct Args {
  const uint16_t* q;        // [Tq, H, 192] bf16
  const uint8_t* k8;        // quantised K, V, V scales, K scales (layout above)
  const uint8_t* v8;
  const uint8_t* vs;
  const float* ks;
  const int32_t* cu_q;
  const int32_t* cu_k;
  float* out;               // [Tq, H, 128]
  float* lse;               // [Tq, H]
  int H, nblk;
  float scale_log2;
};

// K/V stages in LDS: the loads of tile t + kStages - 1 go out during tile t.
// Two stages (41.5 KiB) leave room for three workgroups per CU, which
// measured faster than three stages at two workgroups per CU.
#ifndef Q8_STAGES
#define Q8_STAGES 2
#endif
constexpr int kStages = Q8_STAGES;
static_assert(kStages == 2 || kStages == 3, "waits below cover up to one younger tile");

// Wait until this wave's loads of the current tile have landed (younger: the
// loads of the one later tile issued after them, 0 or nload of them; the
// hardware counts vector memory operations in issue order), then make every
// wave's loads visible.
__device__ __forceinline__ void wait_tile(bool younger, bool wave0) {
  if (!younger) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (wave0) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  lds_barrier();
}
#define CONST_AS __attribute__((address_space(4)))
__device__ __forceinline__ float sldf(const float* p, size_t i) { return ((const CONST_AS float*)p)[i]; }
__device__ __forceinline__ i32x4 ld128i(const LDS_AS uint8_t* p) { return *(const LDS_AS i32x4*)p; }
__device__ __forceinline__ int max_xor32_i(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r[0], (int)r[1]);
}

#ifndef Q8_WAVES
#define Q8_WAVES 3     // waves per SIMD: three workgroups of four waves per CU (<= 168 VGPRs)
#endif
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(Q8_WAVES, Q8_WAVES)))
void prefill_q8_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];
  LDS_AS uint8_t* const stage0 = (LDS_AS uint8_t*)smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // longest query blocks first across the grid (as the bf16 prefill kernel)
  const int nseq = (int)gridDim.x / a.nblk;
  const int lin = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
  const int rank = lin / (nseq * a.H), rem = lin - rank * (nseq * a.H);
  const int head = uniform(rem % a.H);
  const int b = uniform(rem / a.H);
  const int qb = uniform(a.nblk - 1 - rank);
  const int q0 = uniform(a.cu_q[b]), N = uniform(a.cu_q[b + 1] - q0);
  const int k0 = uniform(a.cu_k[b]), L = uniform(a.cu_k[b + 1] - k0);
  const int i0 = qb * kRowsWg;
  if (i0 >= N) return;
  const int H = a.H;
  const int off = L - N;                       // query i sees keys j <= off + i
  const int last_key = off + min(N, i0 + kRowsWg) - 1;
  const int ntiles = last_key >= 0 ? last_key / kTile + 1 : 0;
  const int tbase = uniform(k0 / kTile + b);   // tile index of the sequence's first tile
  const int qi = i0 + 32 * wave + n;
  const bool row_live = qi < N;

  // ---- this lane's query row -> INT8 (features 32c + 16h .. +15, c < 6)
  i32x4 q8[6];
  float rowc;                                  // q scale * softmax scale * log2 e
  {
    const uint16_t* qrow = a.q + ((size_t)(q0 + min(qi, N - 1)) * H + head) * kDK + 16 * h;
    u32x4 raw[6][2];
    float am = 0.f;
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      raw[c][0] = *(const u32x4*)(qrow + 32 * c);
      raw[c][1] = *(const u32x4*)(qrow + 32 * c + 8);
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint32_t u = raw[c][w >> 2][w & 3];
        am = fmaxf(am, fmaxf(fabsf(bf16f(u & 0xFFFF)), fabsf(bf16f(u >> 16))));
      }
    }
    am = max_xor32(am);
    // codes of -q for a negative softmax scale (rint and the clamp are odd
    // functions, so these are exactly the negated codes of q), so that the
    // score scale c below is positive and the row max can be taken on the dots
    const float inv = (am > 0.f ? 127.f / am : 0.f) * (a.scale_log2 < 0.f ? -1.f : 1.f);
    const float sq = am > 0.f ? am / 127.f : 1.f;
#pragma unroll
    for (int c = 0; c < 6; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u0 = raw[c][w >> 1][2 * (w & 1)], u1 = raw[c][w >> 1][2 * (w & 1) + 1];
        const uint32_t word = i8code(bf16f(u0 & 0xFFFF), inv) | (i8code(bf16f(u0 >> 16), inv) << 8) |
                              (i8code(bf16f(u1 & 0xFFFF), inv) << 16) | (i8code(bf16f(u1 >> 16), inv) << 24);
        q8[c][w] = row_live ? (int)word : 0;
      }
    rowc = sq * fabsf(a.scale_log2);
  }

  // ---- loads of one tile: K fragments wave + 4i (i < 3), V fragments wave +
  //      4(i - 3) (i = 3, 4), and on wave 0 the 256 E8M0 bytes (i = 5)
  const uint32_t lds0 = (uint32_t)uniform((int)(uintptr_t)stage0);
  const int nload = wave == 0 ? 6 : 5;
  auto issue = [&](int t, int stage, int i) {
    const size_t rec = (size_t)(tbase + t) * H + head;
    const uint32_t st = lds0 + stage * kStage;
    if (i < 3) {
      const int f = wave + 4 * i;
      dma16(lane * 16, a.k8 + rec * kKBytes + f * 1024, st + f * 1024);
    } else if (i < 5) {
      const int g = wave + 4 * (i - 3);
      dma16(lane * 16, a.v8 + rec * kVBytes + g * 1024, st + kKBytes + g * 1024);
    } else {
      dma4(lane * 4, a.vs + rec * kVsBytes, st + kKBytes + kVBytes);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) o[fb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = 0; t0 < kStages - 1 && t0 < ntiles; ++t0)
    for (int i = 0; i < nload; ++i) issue(t0, t0, i);
  int st_cur = 0;                              // stage of tile t
  for (int t = 0; t < ntiles; ++t) {
    LDS_AS uint8_t* const cur = stage0 + st_cur * kStage;
    const float kscale = sldf(a.ks, (size_t)(tbase + t) * H + head);
    wait_tile(kStages == 3 && t + 1 < ntiles, wave == 0);
    const int t_load = t + kStages - 1;        // its stage held tile t - 1, read by every wave before the barrier
    const bool load_next = t_load < ntiles;
    const int st_load = st_cur == 0 ? kStages - 1 : st_cur - 1;

    // ---- QK: S^T[64 keys, 32 rows] = K Q^T, k-step i: features 32(i/2).., key block i%2
    i32x16 sacc[2];
    sacc[0] = sacc[1] = i32x16{};
    {
      constexpr int NQ = 12, D = 4;
      auto kaddr = [&](int i) { return cur + ((i & 1) * 6 + (i >> 1)) * 1024 + lane * 16; };
      i32x4 ring[D];
#pragma unroll
      for (int i = 0; i < D; ++i) ring[i] = ld128i(kaddr(i));
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const i32x4 av = ring[i % D];
        if (i + D < NQ) ring[i % D] = ld128i(kaddr(i + D));
        sacc[i & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, q8[i >> 1], sacc[i & 1], 0, 0, 0);
        if ((i & 1) == 0 && (i >> 1) < nload && load_next) issue(t_load, st_load, i >> 1);
      }
    }

    // ---- mask (tiles that reach past the block's first row's last key): lane
    //      (n, h) register r of block kb is key 64t + 32kb + 8(r/4) + 4h + r%4
    //      of row qi; a masked dot becomes INT_MIN, below every real one
    //      (|dot| <= 192 * 127^2)
    const int kt0 = t * kTile;
    const bool diag = kt0 + kTile - 1 > off + i0;
    if (diag) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3) > off + qi) sacc[kb][r] = INT_MIN;
    }
    // ---- online softmax on S * log2 e = dot * c (c > 0: the query codes carry
    //      the sign of the softmax scale), the row max taken on the integer
    //      dots; the running max is raised to every tile's max
    const float c = rowc * kscale;
    int mi = INT_MIN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mi = max(mi, sacc[kb][r]);
    mi = max_xor32_i(mi);
    const float mx = mi == INT_MIN ? -INFINITY : (float)mi * c;
    const float m_new = fmaxf(m_run, mx);
    const bool raise = m_new > m_run;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? exp2_fast(m_run - m_new) : 1.0f;   // 0 while m_run is -inf
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) o[fb] *= alpha;
      l_run *= alpha;
    }
    m_run = m_new;
    const float mo = (m_run == -INFINITY ? 0.f : m_run) - (float)kPShift;   // exp2(dot * c - mo) = P * 2^8
    float x[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kb][r] = __builtin_fmaf((float)sacc[kb][r], c, -mo);
    if (diag) {   // masked scores to -inf (their INT_MIN dots need not give exp2 = 0)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3) > off + qi) x[kb][r] = -INFINITY;
    }
    i32x8 p8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[j] = exp2_fast(x[kb][4 * w + j]);
          l_run += y[j];
        }
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
        p8[4 * kb + w] = pk;
      }

    // ---- PV: O^T[32fb + .., 32 rows] += V^T P^T, the E8M0 byte fb of this
    //      lane's word scales (feature 32fb + n, key block h)
    const uint32_t vsw = *(const LDS_AS uint32_t*)(cur + kKBytes + kVBytes + lane * 4);
    const LDS_AS uint8_t* vbase = cur + kKBytes + lane * 16;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const i32x4 v0 = ld128i(vbase + (2 * fb) * 1024), v1 = ld128i(vbase + (2 * fb + 1) * 1024);
      const i32x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      switch (fb) {
        case 0: o[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, p8, o[0], 0, 0, 0, (int)vsw, 0, 127); break;
        case 1: o[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, p8, o[1], 0, 0, 1, (int)vsw, 0, 127); break;
        case 2: o[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, p8, o[2], 0, 0, 2, (int)vsw, 0, 127); break;
        default: o[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, p8, o[3], 0, 0, 3, (int)vsw, 0, 127); break;
      }
    }
    st_cur = st_cur + 1 == kStages ? 0 : st_cur + 1;
  }

  // ---- epilogue: O / l, LSE = (m + log2 l - 8) ln 2
  const float l_row = sum_xor32(l_run);
  if (!row_live) return;
  const bool live = l_row > 0.f;
  const float inv = live ? 1.0f / l_row : 0.f;
  const size_t row = (size_t)(q0 + qi) * H + head;
  float* dst = a.out + row * kDV;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 v = {o[fb][4 * jj], o[fb][4 * jj + 1], o[fb][4 * jj + 2], o[fb][4 * jj + 3]};
      *(f32x4*)(dst + 32 * fb + 8 * jj + 4 * h) = v * inv;
    }
  if (h == 0) a.lse[row] = live ? (m_run + log2_fast(l_row) - (float)kPShift) * kLn2 : -INFINITY;
}

}  // namespace q8

hipError_t launch_quant_kv(const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v, const int32_t* cu_k,
                           int batch, long long total_k, int num_heads, uint8_t* qkv, hipStream_t s,
                           hipEvent_t ev_start, hipEvent_t ev_stop) {
  const QkvLayout l = qkv_layout(batch, total_k, num_heads);
  dim3 grid((unsigned)(total_k / q8::kTile + batch), num_heads);
  hipExtLaunchKernelGGL(q8::quant_kv_kernel, grid, dim3(q8::kThreads), 0, s, ev_start, ev_stop, 0, k_nope, k_rope,
                        v, cu_k, batch, num_heads, qkv + l.k8, qkv + l.v8, qkv + l.vs, (float*)(qkv + l.ks));
  return hipGetLastError();
}

int prefill_q8_rows_per_block() { return q8::kRowsWg; }

hipError_t launch_prefill_q8(const uint16_t* q, const uint8_t* qkv, const int32_t* cu_q, const int32_t* cu_k,
                             int batch, int max_q_len, long long total_k, int num_heads, float softmax_scale,
                             float* out, float* lse, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const QkvLayout l = qkv_layout(batch, total_k, num_heads);
  q8::Args a;
  a.q = q;
  a.k8 = qkv + l.k8;
  a.v8 = qkv + l.v8;
  a.vs = qkv + l.vs;
  a.ks = (const float*)(qkv + l.ks);
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.out = out;
  a.lse = lse;
  a.H = num_heads;
  a.nblk = (max_q_len + q8::kRowsWg - 1) / q8::kRowsWg;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  dim3 grid(batch * a.nblk, num_heads);
  hipExtLaunchKernelGGL(q8::prefill_q8_kernel, grid, dim3(q8::kThreads), 0, s, ev_start, ev_stop, 0, a);
  return hipGetLastError();
}

}  // namespace mla
