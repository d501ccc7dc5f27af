// MLA decode kernels for gfx950 (MI355X / CDNA4).
//
// One pass follows the four steps the pages give for their MLA operator
// (PaddleNLP issue #10157, "Multi-head Latent Attention (MLA) operator",
// overview): data load, QK GEMM, online softmax update, PV GEMM. The Hopper
// warp-group pipelines described there are prior art only; this is the
// CDNA4 mapping:
//
//  * Data load: one tile = one 64-token page (64 x 576 bf16 = 72 KiB) moved
//    by direct global->LDS 16-byte loads (no register staging) into one of
//    two LDS buffers, so the next page streams in while the current one is
//    computed. Rows are XOR-swizzled in 16-byte chunks so both MFMA operand
//    reads below are free of LDS bank conflicts.
//  * QK GEMM: S^T[key, row] = K . Q^T with v_mfma_f32_16x16x32_bf16. Each
//    wave keeps its 16 query rows (16 x 576 bf16) in registers for the whole
//    KV loop; K comes from LDS. Every head of a sequence shares each tile.
//  * Softmax: base-2 online softmax per row, reduced across the 4 lane groups
//    that hold a row; causal/tail masking only on tiles that need it; the
//    running max is raised lazily (only when it grows by more than 2^8), so
//    the O accumulators are rarely rescaled.
//  * PV GEMM: O^T[feature, row] += V^T . P^T. V is the first 512 columns of
//    the same LDS tile, read transposed with ds_read_b64_tr_b16; P^T comes
//    straight out of the QK accumulators in the layout the MFMA B operand
//    wants, so P never goes through LDS.
//
// Split-KV: work units of equal tile count over the flattened
// (sequence, tile) space; sequences cut across units write partial (O, LSE)
// that the combine kernel merges by log-sum-exp.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "mla_internal.h"

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowBytes = kDqk * 2;                  // 1152
constexpr int kTileBytes = kPage * kRowBytes;        // 73728
constexpr int kGroupBytes = 4096;                    // 32 features x 64 keys, bf16
constexpr int kLoadsPerThread = kTileBytes / (kThreads * 16);  // 18
constexpr int kQChunks = kDqk / 32;                  // 18 k-steps of 32
constexpr int kFeatBlocks = kDv / 16;                // 32 output blocks of 16
constexpr float kRescaleThreshold = 8.0f;            // log2 units
constexpr float kLn2 = 0.6931471805599453f;
// s_waitcnt immediate for vmcnt(0), expcnt/lgkmcnt untouched (gfx9 encoding)
constexpr int kVmcntZero = 0x0F70;

static_assert(kLoadsPerThread * kThreads * 16 == kTileBytes, "tile must split evenly");

// LDS tile layout (bf16). Feature f of key k is at byte
//   (f / 32) * 4096 + (k / 16) * 1024 + ((f / 8) % 4) * 256 + (k % 16) * 16 + (f % 8) * 2
// i.e. [32-feature group][16-key block][16-byte chunk of the group][key][8 values].
// A QK operand fetch (16 keys x one 16-byte chunk per lane group) is then one
// contiguous KiB in lane order, every address below is a per-lane constant plus
// a compile-time offset, and one load instruction fills one contiguous KiB.

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct-to-LDS 16-byte load per lane: global address sbase + voff, LDS
// destination lds_addr + 16 * lane (lds_addr wave-uniform, in M0). Written as
// inline asm so the compiler does not treat it as an LDS store it must wait on:
// the kernel orders these loads itself with explicit vmcnt waits + barriers.
__device__ __forceinline__ void dma16(uint32_t voff, const uint8_t* sbase, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Issue the 18 direct-to-LDS loads of one page (each lane: 16 bytes per load;
// load i fills feature group i). Keys at or past `nvalid` re-read the last
// valid key, so tail slots hold finite values (their probabilities are exactly
// 0) and every wave issues exactly 18 loads.
__device__ __forceinline__ void load_tile(const uint8_t* page, int nvalid, LDS_AS uint8_t* buf,
                                          int tid) {
  const int key = (tid >> 6) * 16 + (tid & 15);
  const int src_key = key < nvalid ? key : nvalid - 1;
  const uint32_t voff = src_key * kRowBytes + ((tid >> 4) & 3) * 16;
  const uint32_t lds0 = (uint32_t)uniform((int)(uintptr_t)(buf + (tid & ~63) * 16));
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) dma16(voff + 64 * i, page, lds0 + i * kGroupBytes);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x4 tr_read(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
}
__device__ __forceinline__ bf16x8 ld128(const LDS_AS uint8_t* p) { return *(const LDS_AS bf16x8*)p; }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
template <int VAR>
struct Cfg;
template <>
struct Cfg<VAR_NARROW16> {
  static constexpr int kKeysPerWave = 16;
  static constexpr int kRowsWg = 16;
};
template <>
struct Cfg<VAR_WIDE64> {
  static constexpr int kKeysPerWave = 64;
  static constexpr int kRowsWg = 64;
};

constexpr int kQkDepth = 6;   // LDS operand fetches in flight ahead of the QK MFMAs
constexpr int kPvDepth = 4;   // ... ahead of the PV MFMAs

template <int VAR>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeParams p, const int32_t* __restrict__ md, const int32_t* __restrict__ prefix,
                   const int32_t* __restrict__ split_off, const int32_t* __restrict__ seqlens,
                   const int32_t* __restrict__ block_table, const uint16_t* __restrict__ qptr,
                   const uint8_t* __restrict__ kv) {
  constexpr int KPW = Cfg<VAR>::kKeysPerWave;
  constexpr int NKB = KPW / 16;              // 16-key blocks per wave
  constexpr int ROWS_WG = Cfg<VAR>::kRowsWg;
  constexpr bool NARROW = (VAR == VAR_NARROW16);

  __shared__ __attribute__((aligned(1024))) uint8_t smem0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[kTileBytes];
  __shared__ float mrg[2][4][16];
  LDS_AS uint8_t* const buf0 = (LDS_AS uint8_t*)(smem0);
  LDS_AS uint8_t* const buf1 = (LDS_AS uint8_t*)(smem1);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int R = p.rows;
  const int row = blockIdx.y * ROWS_WG + (NARROW ? 0 : wave * 16) + li;
  const int key_blk = NARROW ? wave : 0;     // first 16-key block of this wave
  const int u = blockIdx.x;

  // ---- this unit's flattened tile range and first sequence
  int f_begin, f_end, b;
  int payload = 1;
  if (md) {
    const int B = p.batch;
    payload = md[MD_PAYLOAD];
    const int T = prefix[B];
    f_begin = u * payload;
    if (f_begin >= T) return;
    f_end = min(f_begin + payload, T);
    b = split_off[B + 1 + u];
  } else {
    b = u;
    const int L = max(seqlens[b], 0);
    f_begin = 0;
    f_end = (L + kPage - 1) / kPage;
    if (f_end == 0) {
      // nothing cached: O = 0, LSE = -inf for this workgroup's rows
      const int r0 = blockIdx.y * ROWS_WG;
      for (int r = r0 + wave; r < min(r0 + ROWS_WG, R); r += 4) {
        float* o = p.out + ((size_t)b * R + r) * kDv;
        for (int d = lane * 4; d < kDv; d += 256) *(f32x4*)(o + d) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (lane == 0) p.lse[(size_t)b * R + r] = -INFINITY;
      }
      return;
    }
  }
  f_begin = uniform(f_begin);
  f_end = uniform(f_end);
  b = uniform(b);
  auto seq_first = [&](int bb) { return md ? prefix[bb] : 0; };
  auto seq_last = [&](int bb) { return md ? prefix[bb + 1] : f_end; };

  // Scalar facts of a tile, read when its load is issued (one iteration ahead)
  // so nothing between the barrier and the MFMAs waits on a scalar load.
  struct TileInfo {
    int b, t, L;
    bool first, last;
  };
  int bp = b;  // sequence cursor of the prefetch stream
  auto issue = [&](int f, LDS_AS uint8_t* dst) {
    while (f >= seq_last(bp)) ++bp;
    bp = uniform(bp);
    TileInfo ti;
    ti.b = bp;
    ti.t = uniform(f - seq_first(bp));
    ti.L = uniform(seqlens[bp]);
    ti.first = (f == f_begin) || (ti.t == 0);
    ti.last = (f + 1 == f_end) || (f + 1 == seq_last(bp));
    const int page = uniform(block_table[(size_t)bp * p.max_pages + ti.t]);
    const int nvalid = min(kPage, ti.L - ti.t * kPage);
    load_tile(kv + (size_t)page * kTileBytes, nvalid, dst, tid);
    return ti;
  };

  // ---- per-lane constant LDS offsets
  // QK operand fetch: (16-key block kb, 16-byte chunk g of the feature group, key li)
  const int qk_lane = key_blk * 1024 + lane * 16;
  // V transposed fetch: keys 4g + li/4 of a 16-key block, features 16fb + 4(li%4)
  const int v_lane = key_blk * 1024 + ((li & 3) >> 1) * 256 + (4 * g + (li >> 2)) * 16 + 8 * (li & 1);

  bf16x8 qreg[kQChunks];
  f32x4 o[kFeatBlocks];
  float m_run = -INFINITY, l_run = 0.f;

  TileInfo next = issue(f_begin, buf0);

  auto step = [&](const int f, LDS_AS uint8_t* const cur, LDS_AS uint8_t* const nxt) {
    const TileInfo ti = next;
    const int bc = ti.b, t = ti.t, L = ti.L;

    if (ti.first) {
      // new sequence: its query rows into registers, fresh softmax state
      const int rr = row < R ? row : R - 1;
      const bf16x8* qrow = (const bf16x8*)(qptr + ((size_t)bc * R + rr) * kDqk);
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) {
        bf16x8 v = qrow[4 * c + g];
        qreg[c] = row < R ? v : bf16x8{};
      }
#pragma unroll
      for (int fb = 0; fb < kFeatBlocks; ++fb) o[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
      // Drain here, once per sequence, before the next page's loads are
      // issued: the query rows (and the current page) are then known to be in
      // place and the compiler needs no wait at their first use.
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
    }

    // epilogue destination (scalar loads, done before the barrier)
    bool final_out = true;
    int slot = 0;
    if (ti.last && md) {
      const int ns = split_off[bc + 1] - split_off[bc];
      final_out = (ns == 1);
      slot = split_off[bc] + (u - prefix[bc] / payload);
    }
    final_out = uniform(final_out);
    slot = uniform(slot);

    if (f + 1 < f_end) {
      next = issue(f + 1, nxt);
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();

    // ---- QK GEMM: S^T (keys x rows) for this wave's keys, K from LDS, Q^T in registers
    constexpr int NACC = NKB == 1 ? 2 : NKB;      // split a lone chain in two
    constexpr int NQK = kQChunks * NKB;
    f32x4 s[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) s[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const LDS_AS uint8_t* kp = cur + qk_lane;
      bf16x8 ring[kQkDepth];
#pragma unroll
      for (int i = 0; i < kQkDepth; ++i) ring[i] = ld128(kp + (i / NKB) * kGroupBytes + (i % NKB) * 1024);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        const int c = i / NKB, kb = i % NKB;
        const bf16x8 a = ring[i % kQkDepth];
        if (i + kQkDepth < NQK) {
          const int j = i + kQkDepth;
          ring[i % kQkDepth] = ld128(kp + (j / NKB) * kGroupBytes + (j % NKB) * 1024);
        }
        const int acc = NKB == 1 ? (c & 1) : kb;
        s[acc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[c], s[acc], 0, 0, 0);
        sched_fence();
      }
    }
    if constexpr (NKB == 1) s[0] += s[1];

    // ---- online softmax (base 2)
    const int key0 = t * kPage + key_blk * 16;
    const int vis = L - p.q_len + (row < R ? row : R - 1) / p.num_heads + 1;
    const bool need_mask = (t * kPage + kPage) > (L - p.q_len + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = s[kb][r] * p.scale_log2;
        if (need_mask && (key0 + kb * 16 + 4 * g + r) >= vis) v = -INFINITY;
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool raise = m_new > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? exp2_fast(m_run - m_new) : 1.0f;
      if (raise) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int fb = 0; fb < kFeatBlocks; ++fb) o[fb] *= alpha;
    }
    const float m_eff = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = exp2_fast(s[kb][r] - m_eff);
        s[kb][r] = pr;
        l_run += pr;
      }
    }

    // ---- PV GEMM: O^T (features x rows) += V^T . P^T, V^T read transposed from LDS
    {
      const LDS_AS uint8_t* vp = cur + v_lane;
      if constexpr (NARROW) {
        bf16x4 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[r] = (__bf16)s[0][r];
        const i16x4 pbs = __builtin_bit_cast(i16x4, pb);
        bf16x4 ring[kPvDepth];
#pragma unroll
        for (int i = 0; i < kPvDepth; ++i) ring[i] = tr_read(vp + (i >> 1) * kGroupBytes + (i & 1) * 512);
#pragma unroll
        for (int fb = 0; fb < kFeatBlocks; ++fb) {
          const bf16x4 v = ring[fb % kPvDepth];
          if (fb + kPvDepth < kFeatBlocks) {
            const int j = fb + kPvDepth;
            ring[fb % kPvDepth] = tr_read(vp + (j >> 1) * kGroupBytes + (j & 1) * 512);
          }
          o[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, v), pbs, o[fb],
                                                            0, 0, 0);
          sched_fence();
        }
      } else {
        bf16x8 pb[2];
#pragma unroll
        for (int c32 = 0; c32 < 2; ++c32) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pb[c32][r] = (__bf16)s[2 * c32][r];
            pb[c32][4 + r] = (__bf16)s[2 * c32 + 1][r];
          }
        }
        constexpr int NPV = 2 * kFeatBlocks;
        auto vaddr = [&](int i, int second) {
          const int c32 = i / kFeatBlocks, fb = i % kFeatBlocks;
          return vp + (fb >> 1) * kGroupBytes + (fb & 1) * 512 + (2 * c32 + second) * 1024;
        };
        bf16x4 r0[kPvDepth], r1[kPvDepth];
#pragma unroll
        for (int i = 0; i < kPvDepth; ++i) {
          r0[i] = tr_read(vaddr(i, 0));
          r1[i] = tr_read(vaddr(i, 1));
        }
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int c32 = i / kFeatBlocks, fb = i % kFeatBlocks;
          const bf16x8 a = __builtin_shufflevector(r0[i % kPvDepth], r1[i % kPvDepth], 0, 1, 2, 3, 4, 5, 6, 7);
          if (i + kPvDepth < NPV) {
            r0[i % kPvDepth] = tr_read(vaddr(i + kPvDepth, 0));
            r1[i % kPvDepth] = tr_read(vaddr(i + kPvDepth, 1));
          }
          o[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[c32], o[fb], 0, 0, 0);
          sched_fence();
        }
      }
    }

    lds_barrier();  // every wave is done with `cur`

    if (!ti.last) return;

    // ---- epilogue for sequence bc
    float l_row = l_run + __shfl_xor(l_run, 16);
    l_row += __shfl_xor(l_row, 32);
    float m_row = m_run;

    if constexpr (NARROW) {
      // merge the 4 waves' key quarters of the same 16 rows (fixed order)
      if (g == 0) {
        mrg[0][wave][li] = m_run;
        mrg[1][wave][li] = l_row;
      }
      lds_barrier();
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[0][w][li]);
      float Ltot = 0.f, mine = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = mrg[0][w][li];
        const float cw = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
        Ltot += cw * mrg[1][w][li];
        if (w == wave) mine = cw;
      }
      const float scl = Ltot > 0.f ? mine : 0.f;
#pragma unroll
      for (int fb = 0; fb < kFeatBlocks; ++fb) o[fb] *= scl;
      LDS_AS f32x4* region = (LDS_AS f32x4*)cur;   // 2 x (32 x 64) f32x4 = 64 KiB
      if (wave >= 2) {
#pragma unroll
        for (int fb = 0; fb < kFeatBlocks; ++fb) region[(wave - 2) * 2048 + fb * 64 + lane] = o[fb];
      }
      lds_barrier();
      if (wave < 2) {
#pragma unroll
        for (int fb = 0; fb < kFeatBlocks; ++fb) o[fb] += region[wave * 2048 + fb * 64 + lane];
      }
      lds_barrier();
      if (wave == 1) {
#pragma unroll
        for (int fb = 0; fb < kFeatBlocks; ++fb) region[2048 + fb * 64 + lane] = o[fb];
      }
      lds_barrier();
      if (wave == 0) {
#pragma unroll
        for (int fb = 0; fb < kFeatBlocks; ++fb) o[fb] += region[2048 + fb * 64 + lane];
      }
      l_row = Ltot;
      m_row = M;
    }

    if (!NARROW || wave == 0) {
      const bool live = l_row > 0.f;
      const float inv = live ? 1.0f / l_row : 0.f;
      const float lse_v = live ? (m_row + log2_fast(l_row)) * kLn2 : -INFINITY;
      if (row < R) {
        float* dst_o;
        float* dst_l;
        if (final_out) {
          dst_o = p.out + ((size_t)bc * R + row) * kDv;
          dst_l = p.lse + (size_t)bc * R + row;
        } else {
          dst_o = p.ws_out + ((size_t)slot * R + row) * kDv;
          dst_l = p.ws_lse + (size_t)slot * R + row;
        }
#pragma unroll
        for (int fb = 0; fb < kFeatBlocks; ++fb) *(f32x4*)(dst_o + 16 * fb + 4 * g) = o[fb] * inv;
        if (g == 0) *dst_l = lse_v;
      }
    }
    if constexpr (NARROW) lds_barrier();  // `cur` is the next prefetch target
  };

  // Two copies of the step with the buffers fixed at compile time, so the
  // compiler sees that LDS reads of one buffer never wait on the direct-to-LDS
  // loads still landing in the other.
  for (int f = f_begin; f < f_end; f += 2) {
    step(f, buf0, buf1);
    if (f + 1 < f_end) step(f + 1, buf1, buf0);
  }
}

// ---------------------------------------------------------------------------
// Split schedule (one workgroup). Integer only; matches the definition in the
// header: equal tile counts per unit over the flattened (sequence, tile) space.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void metadata_kernel(const int32_t* seqlens, int B, int units,
                                                        int min_tiles, int32_t* md) {
  __shared__ int part[1024];
  __shared__ int s_total, s_payload;
  const int tid = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int lo = min(tid * per, B), hi = min(lo + per, B);
  int32_t* prefix = md + MD_HEADER;
  int32_t* split_off = prefix + B + 1;
  int32_t* unit_seq = split_off + B + 1;

  auto tiles = [&](int bb) { return (max(seqlens[bb], 0) + kPage - 1) / kPage; };

  int acc = 0;
  for (int bb = lo; bb < hi; ++bb) acc += tiles(bb);
  part[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
    s_total = run;
    const int T = run;
    const int by_units = (T + units - 1) / units;
    s_payload = max(max(by_units, min_tiles), 1);
  }
  __syncthreads();
  const int T = s_total, payload = s_payload;
  int run = part[tid];
  for (int bb = lo; bb < hi; ++bb) {
    prefix[bb] = run;
    run += tiles(bb);
  }
  if (tid == 0) prefix[B] = T;
  __syncthreads();

  acc = 0;
  for (int bb = lo; bb < hi; ++bb) {
    const int tb = tiles(bb);
    const int pb = prefix[bb];
    acc += tb ? ((pb + tb - 1) / payload - pb / payload + 1) : 0;
  }
  part[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    int r = 0;
    for (int i = 0; i < 1024; ++i) {
      const int v = part[i];
      part[i] = r;
      r += v;
    }
    s_total = r;
  }
  __syncthreads();
  run = part[tid];
  for (int bb = lo; bb < hi; ++bb) {
    split_off[bb] = run;
    const int tb = tiles(bb);
    const int pb = prefix[bb];
    run += tb ? ((pb + tb - 1) / payload - pb / payload + 1) : 0;
  }
  if (tid == 0) split_off[B] = s_total;
  __syncthreads();

  for (int uu = tid; uu < units; uu += 1024) {
    const long long f = (long long)uu * payload;
    int res = B;
    if (f < T) {
      int lo2 = 0, hi2 = B;  // last bb with prefix[bb] <= f
      while (hi2 - lo2 > 1) {
        const int mid = (lo2 + hi2) >> 1;
        if (prefix[mid] <= f) lo2 = mid; else hi2 = mid;
      }
      res = lo2;
    }
    unit_seq[uu] = res;
  }
  if (tid == 0) {
    md[MD_MAGIC] = kMdMagic;
    md[MD_BATCH] = B;
    md[MD_UNITS] = units;
    md[MD_PAYLOAD] = payload;
    md[MD_TOTAL_PARTIALS] = s_total;
    md[MD_UNITS_USED] = T ? (T + payload - 1) / payload : 0;
    md[6] = 0;
    md[7] = 0;
  }
}

// ---------------------------------------------------------------------------
// LSE merge of partials. 256 threads = 2 rows x 128 threads x 4 features.
// ---------------------------------------------------------------------------
constexpr int kCombineRowsPerBlock = 16;

__global__ __launch_bounds__(256) void combine_kernel(const float* part_out, const float* part_lse,
                                                      const int32_t* offsets, int B, int R,
                                                      float* out, float* lse, int skip_single) {
  const int b = blockIdx.x;
  const int k0 = offsets[b];
  const int n = offsets[b + 1] - k0;
  if (skip_single && n == 1) return;
  const int half = threadIdx.x >> 7;
  const int d = (threadIdx.x & 127) * 4;
  const int r_end = min((int)(blockIdx.y + 1) * kCombineRowsPerBlock, R);
  for (int r = blockIdx.y * kCombineRowsPerBlock + half; r < r_end; r += 2) {
    float M = -INFINITY;
    for (int k = 0; k < n; ++k) M = fmaxf(M, part_lse[(size_t)(k0 + k) * R + r]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lse_v = -INFINITY;
    if (M != -INFINITY) {
      float tot = 0.f;
      for (int k = 0; k < n; ++k) {
        const float lk = part_lse[(size_t)(k0 + k) * R + r];
        tot += (lk == -INFINITY) ? 0.f : expf(lk - M);
      }
      lse_v = M + logf(tot);
      const float inv = 1.0f / tot;
      for (int k = 0; k < n; ++k) {
        const float lk = part_lse[(size_t)(k0 + k) * R + r];
        if (lk == -INFINITY) continue;
        const float w = expf(lk - M) * inv;
        const f32x4 v = *(const f32x4*)(part_out + ((size_t)(k0 + k) * R + r) * kDv + d);
        acc += w * v;
      }
    }
    *(f32x4*)(out + ((size_t)b * R + r) * kDv + d) = acc;
    if (d == 0) lse[(size_t)b * R + r] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int variant_for(int rows) { return rows <= 16 ? VAR_NARROW16 : VAR_WIDE64; }
int variant_rows(int variant) { return variant == VAR_NARROW16 ? 16 : 64; }

hipError_t launch_decode(const DecodeParams& p, int variant, int grid_units, hipStream_t s) {
  const int rb = (p.rows + variant_rows(variant) - 1) / variant_rows(variant);
  dim3 grid(grid_units, rb);
  const int32_t* prefix = p.md ? p.md + MD_HEADER : nullptr;
  const int32_t* split_off = p.md ? prefix + p.batch + 1 : nullptr;
  if (variant == VAR_NARROW16)
    hipLaunchKernelGGL(decode_kernel<VAR_NARROW16>, grid, dim3(kThreads), 0, s, p, p.md, prefix, split_off,
                       p.seqlens, p.block_table, p.q, p.kv);
  else
    hipLaunchKernelGGL(decode_kernel<VAR_WIDE64>, grid, dim3(kThreads), 0, s, p, p.md, prefix, split_off,
                       p.seqlens, p.block_table, p.q, p.kv);
  return hipGetLastError();
}

hipError_t launch_metadata(const int32_t* seqlens, int batch, int units, int min_tiles, int32_t* md,
                           hipStream_t s) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(1024), 0, s, seqlens, batch, units, min_tiles, md);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_out, const float* part_lse, const int32_t* offsets,
                          int /*unused*/, int batch, int rows, float* out, float* lse, int skip_single,
                          hipStream_t s) {
  dim3 grid(batch, (rows + kCombineRowsPerBlock - 1) / kCombineRowsPerBlock);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, part_out, part_lse, offsets, batch, rows,
                     out, lse, skip_single);
  return hipGetLastError();
}

}  // namespace mla
