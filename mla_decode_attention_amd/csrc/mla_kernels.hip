// MLA decode kernels for gfx950 (MI355X / CDNA4).
//
// One pass follows the four steps the pages give for their MLA operator
// (PaddleNLP issue #10157, "Multi-head Latent Attention (MLA) operator",
// overview): data load, QK GEMM, online softmax update, PV GEMM. The Hopper
// warp-group pipelines described there are prior art only; this is the
// CDNA4 mapping:
//
//  * Data load: one tile = one 64-token page (64 x 576 bf16 = 72 KiB) in one
//    of two LDS buffers, so the next page streams in while the current one is
//    computed. The 16-row kernel streams pages through the registers of
//    dedicated producer waves; the 64-row kernels use direct global->LDS
//    16-byte loads issued between MFMAs. The LDS layout (below) makes every
//    MFMA operand fetch a per-lane constant address plus a compile-time
//    offset, free of bank conflicts.
//  * QK GEMM: S^T[key, row] = K . Q^T on bf16 MFMA with fp32 accumulation.
//    Each wave keeps its query rows (or a feature half of them) in registers
//    for the whole KV loop; K comes from LDS. Every head of a sequence shares
//    each tile.
//  * Softmax: base-2 online softmax per row, reduced across the lanes that
//    hold a row; causal/tail masking only on tiles that need it; the running
//    max is raised lazily (only when it grows by more than 2^8), so the O
//    accumulators are rarely rescaled.
//  * PV GEMM: O^T[feature, row] += V^T . P^T. V is the first 512 columns of
//    the same LDS tile, read transposed with ds_read_b64_tr_b16; P^T leaves
//    the QK accumulators in the layout the MFMA B operand wants (the key
//    order inside each MFMA k-step is permuted to match), and is exchanged
//    through LDS between the waves that own keys and the waves that own
//    output features.
//
// Variants by rows per sequence (R = q_len * heads):
//   NARROW16PC (R <= 16, bf16): 8 waves, 4 producers + 4 consumers; the
//                        consumers split the keys for QK and the output
//                        features for PV (16x16 MFMA).
//   NARROW16PC8 (R <= 16, fp8): the same roles over E4M3 pages kept in LDS,
//                        the operands widened in registers.
//   WIDE64X    (R > 16): 64 rows, 8 waves, score waves (QK, softmax) and
//                        output waves (PV, page loads); bf16 and fp8 cache,
//                        one query count for all sequences or per-sequence
//                        counts (decode_kernel_so in mla_decode_so.hip).
//   Q8         (fp8 cache, mla_decode_fwd_fp8mma): queries and P in E4M3 on
//                        fp8 MFMA, 64 rows, score and output waves
//                        (decode_kernel_so8 in mla_decode_so.hip).
// (The prefill / extend kernel is in mla_prefill.hip.)
//
// Split-KV: work units of equal tile count over the flattened
// (sequence, tile) space; sequences cut across units write partial (O, LSE)
// that the combine kernel merges by log-sum-exp.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <math.h>
#include <algorithm>
#include <utility>

#include "mla_device.h"

namespace mla {

// LDS operand fetches in flight ahead of the MFMAs of the 16-row kernel
constexpr int kQkDepth = 6;   // QK
constexpr int kPvDepth = 4;   // PV

// Register-staged page stream (producer waves of NARROW16PC, 256 threads).
// Two register stages of one page each (18 x 16-byte loads per lane) keep two
// pages in flight per workgroup while the consumers compute a third from LDS:
// with two LDS buffers, direct-to-LDS loads could only ever have one page in
// flight. Right after barrier B0 of tile f the producers write the stage
// holding tile f+1 into the free LDS buffer and refill that stage with tile
// f+3. Each refill is exactly 18 loads (a single cache line, never used, when
// the unit has no such tile), so the wait before every LDS write is the static
// "all but the 18 newest loads" the compiler derives. Barrier count per tile
// matches the consumers' (B0, B1, B2).
struct TileRegs {
  static constexpr int kLoads = kLoadsPerThread;
  const uint8_t* page;
  uint32_t voff[2];
  __device__ __forceinline__ void plan(const uint8_t* kv, const float* /*kv_scale*/, int page_id,
                                       int nvalid, LDS_AS uint8_t* /*buf*/, LDS_AS float* /*sbuf*/,
                                       int ptid) {
    page = kv + (size_t)page_id * kTileBytes;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int key = 32 * par + (ptid >> 3);
      const int src_key = key < nvalid ? key : nvalid - 1;
      voff[par] = src_key * kRowBytes + 16 * ((ptid & 7) ^ swz3(key));
    }
  }
  __device__ __forceinline__ void idle(const uint8_t* kv) {
    page = kv;
    voff[0] = voff[1] = 0;
  }
  __device__ __forceinline__ void load(u32x4 (&st)[kLoads]) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) st[i] = *(const u32x4*)(page + voff[i & 1] + 128 * (i >> 1));
  }
};

__device__ __forceinline__ void store_page(const u32x4 (&st)[kLoadsPerThread], LDS_AS uint8_t* buf,
                                           int ptid) {
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) *(LDS_AS u32x4*)(buf + i * 4096 + ptid * 16) = st[i];
}

__device__ __forceinline__ void produce_pages(const KernelArgs& a, Unit& unit, LDS_AS uint8_t* buf0,
                                              LDS_AS uint8_t* buf1, LDS_AS int* info_ring, int ptid) {
  const int f0 = unit.f_begin, fe = unit.f_end;
  TileRegs r;
  // plan the loads of tile f and publish its facts in info_ring[f % 4] (read
  // by the consumers after a barrier that follows this write)
  auto plan = [&](int f) {
    if (f < fe) {
      const TileInfo ti = unit.prepare(a, f, buf0, nullptr, ptid, r);
      if (ptid == 0) put_info(info_ring + 8 * (f & 3), ti);
    } else {
      r.idle(a.kv);
    }
  };
  u32x4 st0[kLoadsPerThread], st1[kLoadsPerThread];
  plan(f0);
  r.load(st0);
  plan(f0 + 1);
  r.load(st1);
  store_page(st0, buf0, ptid);
  plan(f0 + 2);
  r.load(st0);
  for (int f = f0; f < fe; f += 2) {
    lds_barrier();   // B0 of tile f (in buf0)
    if (f + 1 < fe) store_page(st1, buf1, ptid);
    plan(f + 3);
    r.load(st1);
    lds_barrier();   // B1
    lds_barrier();   // B2
    if (f + 1 >= fe) break;
    lds_barrier();   // B0 of tile f + 1 (in buf1)
    if (f + 2 < fe) store_page(st0, buf0, ptid);
    plan(f + 4);
    r.load(st0);
    lds_barrier();   // B1
    lds_barrier();   // B2
  }
}

// ---------------------------------------------------------------------------
// NARROW16PC (bf16 cache, up to 16 rows): 8 waves per workgroup, 2 per SIMD.
//   Waves 4-7 are producers: they only stream the next page into LDS (their
//   vector-memory issue stalls never hold up an MFMA wave).
//   Waves 0-3 are consumers: wave c computes S^T for keys 16c..16c+15 of the
//   tile (16x16x32 MFMA, Q^T of the 16 rows in registers), the 4 half-tile row
//   maxima are exchanged in LDS, and each consumer writes its P values into LDS
//   in the PV B-operand layout; then wave c accumulates O^T for output
//   features 128c..128c+127 of all 16 rows (O: 32 registers), so no merge of
//   per-wave outputs is needed at the end.
//   PV k-step ks (keys 32ks..32ks+31): k-slot 8g + e is key 32ks + 4g + e
//   (e < 4, from consumer 2ks) or 32ks + 16 + 4g + (e - 4) (from 2ks + 1).
//   Three workgroup barriers per tile: B0 (tile in LDS, other buffer free),
//   B1 (row maxima published), B2 (P and, on a sequence's last tile, the row
//   sums published). The producers keep two pages in flight in registers
//   (produce_pages).
// ---------------------------------------------------------------------------
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void decode_kernel_pc(DecodeParams p_, const int32_t* __restrict__ md_, const int32_t* __restrict__ prefix_,
    const int32_t* __restrict__ split_off_, const int32_t* __restrict__ seqlens_,
    const int32_t* __restrict__ block_table_, const uint16_t* __restrict__ qptr_,
    const uint8_t* __restrict__ kv_) {
  const KernelArgs a{p_, md_, prefix_, split_off_, seqlens_, block_table_, qptr_, kv_};
  constexpr int kQChunks = kDqk / 32;        // 18 k-steps of 32 features
  constexpr int kFb = 8;                     // 16-feature output blocks per consumer

  __shared__ __attribute__((aligned(1024))) uint8_t smem0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 p_lds[2][64];   // [k-step][lane]
  __shared__ float smax[4][16];
  __shared__ float ssum[4][16];
  __shared__ int info_lds[4][8];                                  // tile facts, ring of 4
  LDS_AS uint8_t* const buf0 = (LDS_AS uint8_t*)(smem0);
  LDS_AS uint8_t* const buf1 = (LDS_AS uint8_t*)(smem1);
  LDS_AS int* const info_ring = (LDS_AS int*)(&info_lds[0][0]);

  const DecodeParams& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool producer = wave >= 4;
  const int cw = wave & 3;
  const int g = lane >> 4, li = lane & 15;
  const int R = p.rows;
  const int row = li;
  const int u = blockIdx.x;

  Unit unit;
  if (!unit.init(a, u)) {
    if (!a.md && !producer) write_empty(p, unit.b0, 0, 16, 4);
    return;
  }

  // consumer LDS offsets: QK operand of key 16cw + li,
  // chunk 4c + g; transposed V operand of keys 4g + li/4 (+ 16 per key block)
  int qk_lane[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) qk_lane[par] = lds_byte(16 * cw + li, 4 * par + g);
  int v_lane[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    v_lane[q4] = lds_byte(4 * g + (li >> 2), 2 * q4 + ((li & 3) >> 1)) + 8 * (li & 1);

  bf16x8 qreg[kQChunks];
  f32x4 o[kFb];
  float m_run = -INFINITY, l_run = 0.f;

  if (producer) {
    produce_pages(a, unit, buf0, buf1, info_ring, tid - 256);
    return;
  }

  // Query rows of a sequence into registers, issued ahead of their first tile
  // (no wait here). Rows past the sequence's own read its last row: finite
  // values whose results are never stored, so no select waits on the loads.
  auto fetch_q = [&](const TileInfo& nt) {
    const int rr = row < nt.rows ? row : max(nt.rows - 1, 0);
    const bf16x8* qrow = (const bf16x8*)(a.qptr + (size_t)min(nt.qrow0 + rr, p.q_rows - 1) * kDqk);
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) qreg[c] = qrow[4 * c + g];
  };
  {
    TileFacts plan_only;   // the first tile's facts, to fetch its query rows early
    fetch_q(unit.prepare(a, unit.f_begin, buf0, nullptr, tid & 255, plan_only));
  }

  for (int f = unit.f_begin; f < unit.f_end; ++f) {
    const bool odd = ((f - unit.f_begin) & 1) != 0;
    LDS_AS uint8_t* const cur = odd ? buf1 : buf0;
    const bool more = f + 1 < unit.f_end;

    lds_barrier();   // B0: tile f is in `cur`, everyone is done with the other buffer
    const TileInfo ti = get_info(info_ring + 8 * (f & 3));

    const int bc = ti.b, t = ti.t, L = ti.L;
    if (ti.first) {
#pragma unroll
      for (int fb = 0; fb < kFb; ++fb) o[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
      __builtin_amdgcn_s_waitcnt(kVmcntZero);   // its query rows (fetched a tile ahead)
    }

    // QK: S^T[keys 16cw.., 16 rows]
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
    {
      auto kaddr = [&](int c) { return cur + qk_lane[c & 1] + (c >> 1) * kLineGroupBytes; };
      bf16x8 ring[kQkDepth];
#pragma unroll
      for (int i = 0; i < kQkDepth; ++i) ring[i] = ld128(kaddr(i));
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) {
        const bf16x8 av = ring[c % kQkDepth];
        if (c + kQkDepth < kQChunks) ring[c % kQkDepth] = ld128(kaddr(c + kQkDepth));
        if (c & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[c], sb, 0, 0, 0);
        else sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[c], sa, 0, 0, 0);
        sched_fence();
      }
    }
    f32x4 sv = sa + sb;
    if (more) {
      // the next tile starts a sequence: its query rows now (qreg is free)
      const TileInfo nt = get_info(info_ring + 8 * ((f + 1) & 3));
      if (nt.first) fetch_q(nt);
    }

    const int key0 = t * kPage + 16 * cw + 4 * g;
    const int vis = L - ti.qlen + (row < ti.rows ? row : max(ti.rows - 1, 0)) / p.num_heads + 1;
    const bool need_mask = (t * kPage + kPage) > (L - ti.qlen + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = sv[r] * p.scale_log2;
      if (need_mask && (key0 + r) >= vis) v = -INFINITY;
      sv[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_xor32(max_xor16(mx));
    if (g == 0) smax[cw][li] = mx;
    lds_barrier();   // B1

    const float tmax = fmaxf(fmaxf(smax[0][li], smax[1][li]), fmaxf(smax[2][li], smax[3][li]));
    const float m_new = fmaxf(m_run, tmax);
    const bool raise = m_new > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? exp2_fast(m_run - m_new) : 1.0f;
      if (raise) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int fb = 0; fb < kFb; ++fb) o[fb] *= alpha;
    }
    const float m_eff = (m_run == -INFINITY) ? 0.0f : m_run;
    bf16x4 pq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = exp2_fast(sv[r] - m_eff);
      l_run += pr;
      pq[r] = (__bf16)pr;
    }
    *(LDS_AS bf16x4*)((LDS_AS uint8_t*)&p_lds[cw >> 1][lane] + 8 * (cw & 1)) = pq;
    if (ti.last) {
      const float ls = sum_xor32(sum_xor16(l_run));
      if (g == 0) ssum[cw][li] = ls;
    }
    lds_barrier();   // B2

    // PV: O^T[features 128cw.., 16 rows] += V^T . P^T
    {
      auto vaddr = [&](int i, int second) {
        const int ks = i / kFb, fb = 8 * cw + (i % kFb);
        return cur + v_lane[fb & 3] + (fb >> 2) * kLineGroupBytes + (2 * ks + second) * 2048;
      };
      constexpr int NPV = 2 * kFb;
      bf16x4 r0[kPvDepth], r1[kPvDepth];
#pragma unroll
      for (int i = 0; i < kPvDepth; ++i) {
        r0[i] = tr_read(vaddr(i, 0));
        r1[i] = tr_read(vaddr(i, 1));
      }
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int ks = i / kFb, fb = i % kFb;
        if (fb == 0) pb = p_lds[ks][lane];
        const bf16x8 av = __builtin_shufflevector(r0[i % kPvDepth], r1[i % kPvDepth], 0, 1, 2, 3, 4, 5, 6, 7);
        if (i + kPvDepth < NPV) {
          r0[i % kPvDepth] = tr_read(vaddr(i + kPvDepth, 0));
          r1[i % kPvDepth] = tr_read(vaddr(i + kPvDepth, 1));
        }
        o[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[fb], 0, 0, 0);
        sched_fence();
      }
    }

    if (ti.last) {
      const float l_row = ssum[0][li] + ssum[1][li] + ssum[2][li] + ssum[3][li];
      const bool live = l_row > 0.f;
      const float inv = live ? 1.0f / l_row : 0.f;
      if (row < ti.rows) {
        float* dst_o;
        float* dst_l;
        if (ti.final_out) {
          dst_o = p.out + ((size_t)ti.qrow0 + row) * kDv;
          dst_l = p.lse + (size_t)ti.qrow0 + row;
        } else {
          dst_o = p.ws_out + ((size_t)ti.slot * R + row) * kDv;
          dst_l = p.ws_lse + (size_t)ti.slot * R + row;
        }
#pragma unroll
        for (int fb = 0; fb < kFb; ++fb) *(f32x4*)(dst_o + 128 * cw + 16 * fb + 4 * g) = o[fb] * inv;
        if (cw == 0 && g == 0) *dst_l = live ? (m_run + log2_fast(l_row)) * kLn2 : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NARROW16PC8 (fp8 cache, up to 16 rows): the roles of decode_kernel_pc over
// E4M3 pages, which stay E4M3 in LDS (the K and V^T operands are widened to
// bf16 in registers, exactly, as in the 64-row fp8 kernel).
//   Waves 4-7 are producers: direct-to-LDS loads of whole pages (codes and
//   the page's 64 token scales) into a ring of three buffers, two pages in
//   flight while the consumers compute the third (a fourth buffer, three
//   pages in flight, measured slower).
//   Waves 0-3 are consumers: wave c computes S^T for keys 16c..16c+15
//   (v_mfma_f32_16x16x32_bf16; one 16-byte LDS read of 16 codes serves two
//   k-steps, the query registers follow that feature order), scales each
//   score by its token's scale, exchanges the row maxima, writes
//   P_j s_j (bf16) into LDS as the PV B operand with k-slot 8g + e = key
//   8g + e of the k-step, and accumulates O^T for output features
//   128c..128c+127 with V^T from ds_read_b64_tr_b8 (8 consecutive keys of one
//   feature per lane); the row sums take the unscaled P.
//   Three workgroup barriers per tile, as in decode_kernel_pc.
// Tile layout: chunk c (16 codes) of key k at ((c/4) * 64 + k) * 64 +
// ((c%4) ^ swz8p(k)) * 16 (64-byte line groups of 4 KiB), swz8p(k) = (k3, k2):
// every 16 consecutive keys at one chunk (QK operand) and 16 consecutive keys
// x 2 halves of one chunk (V^T operand) cover 16 distinct 16-byte bank groups.
// The 64 scales (256 bytes) follow the codes.
// ---------------------------------------------------------------------------
constexpr int kPc8BufBytes = kFp8TileBytes + 1024;   // 37888: codes, scales, padding to 1 KiB
constexpr int kPc8Bufs = 3;
constexpr int kPc8Loads = 9;                         // code loads per producer lane and page
__device__ __forceinline__ int swz8p(int key) { return (((key >> 3) & 1) << 1) | ((key >> 2) & 1); }
__device__ __forceinline__ int byte8p(int key, int chunk) {
  return ((chunk >> 2) * 64 + key) * 64 + (((chunk & 3) ^ swz8p(key)) << 4);
}

// Load i < 9 of producer lane t fills line group i, key t / 4, 16-byte unit
// t % 4 (the lane fetches the chunk that belongs there); load 9, issued by
// lanes 0-15 of wave 4 only, brings the page's 64 scales. Keys at or past
// `nvalid` re-read the last valid key.
struct TileDmaPc8 {
  static constexpr int kLoads = kPc8Loads + 1;
  const uint8_t* page;
  const uint8_t* scales;
  uint32_t voff, lds0;
  __device__ __forceinline__ void plan(const uint8_t* kv, const float* kv_scale, int page_id, int nvalid,
                                       LDS_AS uint8_t* buf, LDS_AS float* /*sbuf*/, int ptid) {
    page = kv + (size_t)page_id * kFp8TileBytes;
    scales = (const uint8_t*)(kv_scale + (size_t)page_id * kPage);
    const int key = ptid >> 2, pos = ptid & 3;
    const int src_key = min(key, nvalid - 1);
    voff = src_key * kFp8RowBytes + 16 * (pos ^ swz8p(key));
    lds0 = (uint32_t)uniform((int)(uintptr_t)(buf + (ptid & ~63) * 16));
  }
  __device__ __forceinline__ void load(int i) const {
    if (i < 9) {
      dma16(voff + 64 * i, page, lds0 + i * 4096);
    } else if (threadIdx.x < 256 + 16) {
      // (wave 4 only, a wave-uniform choice; within it lanes 0-15)
      dma16(16 * (threadIdx.x & 15), scales, lds0 + 9 * 4096);
    }
  }
};

// vmcnt(n) with expcnt and lgkmcnt untouched (gfx9 encoding)
constexpr int vm_imm_n(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void decode_kernel_pc8(DecodeParams p_, const int32_t* __restrict__ md_, const int32_t* __restrict__ prefix_,
    const int32_t* __restrict__ split_off_, const int32_t* __restrict__ seqlens_,
    const int32_t* __restrict__ block_table_, const uint16_t* __restrict__ qptr_,
    const uint8_t* __restrict__ kv_) {
  const KernelArgs a{p_, md_, prefix_, split_off_, seqlens_, block_table_, qptr_, kv_};
  constexpr int kQChunks = kDqk / 32;        // 18 k-steps of 32 features
  constexpr int kFb = 8;                     // 16-feature output blocks per consumer

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPc8Bufs * kPc8BufBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 p_lds[2][64];   // [k-step][lane]
  __shared__ float smax[4][16];
  __shared__ float ssum[4][16];
  __shared__ int info_lds[4][8];                                  // tile facts, ring of 4
  LDS_AS uint8_t* const bufs = (LDS_AS uint8_t*)(smem);
  LDS_AS int* const info_ring = (LDS_AS int*)(&info_lds[0][0]);
  auto buf = [&](int f) { return bufs + (f % kPc8Bufs) * kPc8BufBytes; };

  const DecodeParams& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool producer = wave >= 4;
  const int cw = wave & 3;
  const int g = lane >> 4, li = lane & 15;
  const int R = p.rows;
  const int row = li;
  const int u = blockIdx.x;

  Unit unit;
  if (!unit.init(a, u)) {
    if (!a.md && !producer) write_empty(p, unit.b0, 0, 16, 4);
    return;
  }
  const int f0 = unit.f_begin, fe = unit.f_end;

  if (producer) {
    // ---- page stream: tiles f0 .. f0 + 2 ahead, then f + 3 after barrier B0
    //      of tile f (the buffer of tile f - 1 is free by then)
    const int ptid = tid - 256;
    constexpr int AHEAD = kPc8Bufs - 1;
    TileDmaPc8 dma;
    auto issue = [&](int f) {
      const TileInfo ti = unit.prepare(a, f, buf(f), nullptr, ptid, dma);
      if (ptid == 0) put_info(info_ring + 8 * (f & 3), ti);
#pragma unroll
      for (int i = 0; i < TileDmaPc8::kLoads; ++i) dma.load(i);
    };
    // tile f has landed when at most the loads of the tiles issued after it
    // are outstanding (wave 4 issues one more load per tile than the others)
    auto wait_landed = [&](int f, int last_issued) {
      const int after = last_issued - f;
      if (wave == 4) {
        if (after >= 2) __builtin_amdgcn_s_waitcnt(vm_imm_n(2 * (kPc8Loads + 1)));
        else if (after == 1) __builtin_amdgcn_s_waitcnt(vm_imm_n(kPc8Loads + 1));
        else __builtin_amdgcn_s_waitcnt(kVmcntZero);
      } else {
        if (after >= 2) __builtin_amdgcn_s_waitcnt(vm_imm_n(2 * kPc8Loads));
        else if (after == 1) __builtin_amdgcn_s_waitcnt(vm_imm_n(kPc8Loads));
        else __builtin_amdgcn_s_waitcnt(kVmcntZero);
      }
    };
    static_assert(AHEAD <= 3 && 2 * (kPc8Loads + 1) <= 63, "wait counts");
    for (int j = 0; j < AHEAD && f0 + j < fe; ++j) issue(f0 + j);
    wait_landed(f0, min(f0 + AHEAD - 1, fe - 1));
    for (int f = f0; f < fe; ++f) {
      lds_barrier();   // B0: tile f and its facts are in LDS
      if (f + AHEAD < fe) issue(f + AHEAD);
      lds_barrier();   // B1
      lds_barrier();   // B2
      if (f + 1 < fe) wait_landed(f + 1, min(f + AHEAD, fe - 1));
    }
    return;
  }

  // ---- consumer operand offsets: K of key 16 cw + li at chunk g of each line
  //      group (16 codes: features 64 r + 16 g .. + 15 of read r); V^T of
  //      keys 8 g + li / 2 (+ 32 per k-step), feature chunk 8 cw + fb, half li % 2
  const int k_lane = byte8p(16 * cw + li, g);
  int v_lane[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) v_lane[q4] = byte8p(8 * g + (li >> 1), 8 * cw + q4) + 8 * (li & 1);

  bf16x8 qreg[kQChunks];   // k-step j: features 64 (j / 2) + 16 g + 8 (j % 2) .. + 7 of this lane's row
  f32x4 o[kFb];
  float m_run = -INFINITY, l_run = 0.f;

  auto fetch_q = [&](const TileInfo& nt) {
    const int rr = row < nt.rows ? row : max(nt.rows - 1, 0);
    const bf16x8* qrow = (const bf16x8*)(a.qptr + (size_t)min(nt.qrow0 + rr, p.q_rows - 1) * kDqk);
#pragma unroll
    for (int j = 0; j < kQChunks; ++j) qreg[j] = qrow[8 * (j >> 1) + 2 * g + (j & 1)];
  };
  {
    TileFacts plan_only;   // the first tile's facts, to fetch its query rows early
    fetch_q(unit.prepare(a, f0, bufs, nullptr, tid & 255, plan_only));
  }

  for (int f = f0; f < fe; ++f) {
    const LDS_AS uint8_t* const cur = buf(f);
    const bool more = f + 1 < fe;

    lds_barrier();   // B0
    const TileInfo ti = get_info(info_ring + 8 * (f & 3));
    const int t = ti.t, L = ti.L;
    if (ti.first) {
#pragma unroll
      for (int fb = 0; fb < kFb; ++fb) o[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
      __builtin_amdgcn_s_waitcnt(kVmcntZero);   // its query rows (fetched a tile ahead)
    }

    // QK: S^T[keys 16cw.., 16 rows]; read r feeds k-steps 2r and 2r + 1
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
    {
      constexpr int NR = kQChunks / 2, D = 4;
      u32x4 ring[D];
#pragma unroll
      for (int i = 0; i < D; ++i) ring[i] = *(const LDS_AS u32x4*)(cur + k_lane + i * 4096);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4 w = ring[r % D];
        if (r + D < NR) ring[r % D] = *(const LDS_AS u32x4*)(cur + k_lane + (r + D) * 4096);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(w[0], w[1]), qreg[2 * r], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(w[2], w[3]), qreg[2 * r + 1], sb, 0, 0, 0);
        sched_fence();
      }
    }
    f32x4 sv = sa + sb;
    if (more) {
      const TileInfo nt = get_info(info_ring + 8 * ((f + 1) & 3));
      if (nt.first) fetch_q(nt);
    }

    const f32x4 ksc = *(const LDS_AS f32x4*)(cur + kFp8TileBytes + (16 * cw + 4 * g) * 4);
    const int key0 = t * kPage + 16 * cw + 4 * g;
    const int vis = L - ti.qlen + (row < ti.rows ? row : max(ti.rows - 1, 0)) / p.num_heads + 1;
    const bool need_mask = (t * kPage + kPage) > (L - ti.qlen + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = sv[r] * (ksc[r] * p.scale_log2);
      if (need_mask && (key0 + r) >= vis) v = -INFINITY;
      sv[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_xor32(max_xor16(mx));
    if (g == 0) smax[cw][li] = mx;
    lds_barrier();   // B1

    const float tmax = fmaxf(fmaxf(smax[0][li], smax[1][li]), fmaxf(smax[2][li], smax[3][li]));
    const float m_new = fmaxf(m_run, tmax);
    const bool raise = m_new > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? exp2_fast(m_run - m_new) : 1.0f;
      if (raise) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int fb = 0; fb < kFb; ++fb) o[fb] *= alpha;
    }
    const float m_eff = (m_run == -INFINITY) ? 0.0f : m_run;
    bf16x4 pq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = exp2_fast(sv[r] - m_eff);
      l_run += pr;
      // masked keys may carry any scale (NaN in a page's unused tail)
      pq[r] = (__bf16)(sv[r] == -INFINITY ? 0.f : pr * ksc[r]);
    }
    // key 16 (cw % 2) + 4 g + r of k-step cw / 2 is k-slot 8 g' + e, g' = 2 (cw % 2) + g / 2
    *(LDS_AS bf16x4*)((LDS_AS uint8_t*)&p_lds[cw >> 1][li + 16 * (2 * (cw & 1) + (g >> 1))] + 8 * (g & 1)) = pq;
    if (ti.last) {
      const float ls = sum_xor32(sum_xor16(l_run));
      if (g == 0) ssum[cw][li] = ls;
    }
    lds_barrier();   // B2

    // PV: O^T[features 128cw.., 16 rows] += V^T . P^T, V^T widened from the codes
    {
      constexpr int NPV = 2 * kFb, D = 4;
      auto vaddr = [&](int i) {
        const int ks = i / kFb, fb = i % kFb;
        return cur + v_lane[fb & 3] + (fb >> 2) * 4096 + ks * 2048;
      };
      i32x2 ring[D];
#pragma unroll
      for (int i = 0; i < D; ++i) ring[i] = tr8_read(vaddr(i));
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int ks = i / kFb, fb = i % kFb;
        if (fb == 0) pb = p_lds[ks][lane];
        const i32x2 x = ring[i % D];
        if (i + D < NPV) ring[i % D] = tr8_read(vaddr(i + D));
        o[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8((unsigned)x[0], (unsigned)x[1]), pb, o[fb], 0, 0, 0);
        sched_fence();
      }
    }

    if (ti.last) {
      const float l_row = ssum[0][li] + ssum[1][li] + ssum[2][li] + ssum[3][li];
      const bool live = l_row > 0.f;
      const float inv = live ? 1.0f / l_row : 0.f;
      if (row < ti.rows) {
        float* dst_o;
        float* dst_l;
        if (ti.final_out) {
          dst_o = p.out + ((size_t)ti.qrow0 + row) * kDv;
          dst_l = p.lse + (size_t)ti.qrow0 + row;
        } else {
          dst_o = p.ws_out + ((size_t)ti.slot * R + row) * kDv;
          dst_l = p.ws_lse + (size_t)ti.slot * R + row;
        }
#pragma unroll
        for (int fb = 0; fb < kFb; ++fb) *(f32x4*)(dst_o + 128 * cw + 16 * fb + 4 * g) = o[fb] * inv;
        if (cw == 0 && g == 0) *dst_l = live ? (m_run + log2_fast(l_row)) * kLn2 : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split schedule (one workgroup). Integer only; matches the definition in the
// header: equal tile counts per unit over the flattened (sequence, tile) space.
// ---------------------------------------------------------------------------

// Exclusive prefix sums of two values over the 1024 threads of the block;
// *total gets the sums. It communicates through LDS only.
__device__ __forceinline__ int2 block_exclusive_scan2(int2 v, int* wave_tot, int2* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int2 x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int yx = __shfl_up(x.x, d), yy = __shfl_up(x.y, d);
    if (lane >= d) {
      x.x += yx;
      x.y += yy;
    }
  }
  if (lane == 63) {
    wave_tot[wave] = x.x;
    wave_tot[16 + wave] = x.y;
  }
  lds_barrier();
  if (wave == 0) {
    int tx = lane < 16 ? wave_tot[lane] : 0, ty = lane < 16 ? wave_tot[16 + lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int yx = __shfl_up(tx, d), yy = __shfl_up(ty, d);
      if (lane >= d) {
        tx += yx;
        ty += yy;
      }
    }
    if (lane < 16) {
      wave_tot[32 + lane] = tx;   // inclusive per-wave offsets
      wave_tot[48 + lane] = ty;
    }
  }
  lds_barrier();
  const int2 base = wave ? make_int2(wave_tot[32 + wave - 1], wave_tot[48 + wave - 1]) : make_int2(0, 0);
  if (total) *total = make_int2(wave_tot[47], wave_tot[63]);
  const int2 r = make_int2(base.x + x.x - v.x, base.y + x.y - v.y);
  lds_barrier();
  return r;
}

// The split schedule in closed form. On the weighted line a sequence with
// tiles occupies [wpre_b, wpre_b + c + T_b): c start positions, then its
// tiles. The line is cut at floor(u * W / U') for u = 0..U', U' =
// max(1, min(units, floor(W / min_tiles))) (units past U' are empty), so the
// tile at position p belongs to unit owner(p) = floor(((p + 1) U' - 1) / W).
// A sequence's pieces are the units owner(wpre_b + c) .. owner(wpre_b + c +
// T_b - 1); the units starting inside its range start at its first tile or at
// the tile their cut names; and it shares its first unit with the previous
// sequence with tiles iff owner(wpre_b - 1) (that sequence's last tile) is the
// same unit. One workgroup; sequences are split evenly over the threads.
__global__ __launch_bounds__(1024) void metadata_kernel(const int32_t* seqlens, int B, int units,
                                                        int min_tiles, int c, int32_t* md) {
  constexpr int kLdsSeqs = 4096;   // batches up to this size place units by a search in LDS
  __shared__ int wave_tot[64];
  __shared__ int s_wpre[kLdsSeqs + 1], s_prefix[kLdsSeqs + 1];
  __shared__ int s_max_pieces;
  const int tid = threadIdx.x;
  if (tid == 0) s_max_pieces = 0;   // published by the first scan's barriers
  const int per = (B + 1023) / 1024;
  const int lo = min(tid * per, B), hi = min(lo + per, B);
  int32_t* prefix = md + MD_HEADER;
  int32_t* split_off = prefix + B + 1;
  int32_t* unit_seq = split_off + B + 1;
  int32_t* unit_begin = md + md_unit_begin(B, units);
  int32_t* first_unit = md + md_seq_first_unit(B, units);

  auto tiles = [&](int bb) { return (max(seqlens[bb], 0) + kPage - 1) / kPage; };

  // tile prefix and weighted prefix
  int2 acc = make_int2(0, 0);
  for (int bb = lo; bb < hi; ++bb) {
    const int t = tiles(bb);
    acc.x += t;
    acc.y += t ? t + c : 0;
  }
  int2 tot;
  const int2 run = block_exclusive_scan2(acc, wave_tot, &tot);
  const int T = tot.x, W = tot.y;
  const int ucut = max(1, min(units, W / max(min_tiles, 1)));
  const long long Wl = W, Ul = ucut;
  // 32-bit arithmetic when every product fits (W * U' < 2^31); 64-bit integer
  // division is a long software routine
  const bool fits32 = Wl * Ul < (1LL << 31);
  auto owner = [&](long long pos) {
    return fits32 ? (int)(((unsigned)(pos + 1) * (unsigned)ucut - 1u) / (unsigned)W)
                  : (int)(((pos + 1) * Ul - 1) / Wl);
  };
  auto cut = [&](long long u) {
    return fits32 ? (long long)((unsigned)u * (unsigned)W / (unsigned)ucut) : u * Wl / Ul;
  };
  const long long wq = W / ucut, wr = W % ucut;

  // pieces of each sequence, the units starting in it, and the first units
  // shared with the previous sequence
  auto pieces = [&](int wp, int t) { return t ? owner(wp + c + t - 1) - owner(wp + c) + 1 : 0; };
  const bool lds_search = B <= kLdsSeqs;
  int2 acc2 = make_int2(0, 0);
  int max_pieces = 0;
  {
    int tp = run.x, wp = run.y;
    for (int bb = lo; bb < hi; ++bb) {
      const int t = tiles(bb);
      prefix[bb] = tp;
      if (lds_search) {
        s_prefix[bb] = tp;
        s_wpre[bb] = wp;
      }
      first_unit[bb] = t ? owner(wp + c) : 0;
      if (t) {
        max_pieces = max(max_pieces, pieces(wp, t));
        acc2.x += pieces(wp, t);
        acc2.y += (wp > 0 && owner(wp - 1) == owner(wp + c)) ? 1 : 0;
      }
      if (t && !lds_search) {
        // units u with wp <= cut(u) < wp + c + t
        // cut(u + 1) = cut(u) + W / U' + (1 when the remainder wraps): one
        // division for the first unit, then adds
        const long long u0 = fits32 ? (long long)(((unsigned)wp * (unsigned)ucut + (unsigned)W - 1u) / (unsigned)W)
                                    : ((long long)wp * Ul + Wl - 1) / Wl;
        long long cu = cut(u0);
        long long rem = u0 * Wl - cu * Ul;
        for (long long u = u0; cu < (long long)wp + c + t; ++u) {
          unit_begin[u] = tp + (int)max(0LL, cu - wp - c);
          unit_seq[u] = bb;
          cu += wq;
          rem += wr;
          if (rem >= Ul) {
            rem -= Ul;
            ++cu;
          }
        }
      }
      tp += t;
      wp += t ? t + c : 0;
    }
  }
  // the largest count: a wave maximum first (one LDS atomic per wave, not one
  // per thread on a single word)
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) max_pieces = max(max_pieces, __shfl_xor(max_pieces, d));
  if ((tid & 63) == 0) atomicMax(&s_max_pieces, max_pieces);
  int2 tot2;
  const int2 run2 = block_exclusive_scan2(acc2, wave_tot, &tot2);   // its barriers also publish s_wpre, s_prefix, s_max_pieces
  if (lds_search) {
    // one unit per thread: the sequence holding position cut(u) is the last
    // one whose weighted prefix is at or below it
    for (int uu = tid; uu < ucut && W > 0; uu += 1024) {
      const long long cu = cut(uu);
      int lo2 = 0, hi2 = B;
      while (hi2 - lo2 > 1) {
        const int mid = (lo2 + hi2) >> 1;
        if (s_wpre[mid] <= cu) lo2 = mid; else hi2 = mid;
      }
      unit_begin[uu] = s_prefix[lo2] + (int)max(0LL, cu - s_wpre[lo2] - c);
      unit_seq[uu] = lo2;
    }
  }
  {
    int so = run2.x, wp = run.y;
    for (int bb = lo; bb < hi; ++bb) {
      const int t = tiles(bb);
      split_off[bb] = so;
      so += pieces(wp, t);
      wp += t ? t + c : 0;
    }
  }
  // units from the last cut on start at T and hold no tile
  for (int uu = tid; uu <= units; uu += 1024) {
    if (W == 0 || uu >= ucut) {
      unit_begin[uu] = T;
      if (uu < units) unit_seq[uu] = B;
    }
  }
  if (tid == 0) {
    prefix[B] = T;
    split_off[B] = tot2.x;
    md[MD_MAGIC] = kMdMagic;
    md[MD_BATCH] = B;
    md[MD_UNITS] = units;
    md[MD_UNITS_CUT] = ucut;
    md[MD_TOTAL_PARTIALS] = tot2.x;
    md[MD_UNITS_USED] = tot2.x - tot2.y;
    md[MD_SEQ_COST] = c;
    md[MD_MAX_PIECES] = s_max_pieces;
  }
}

// ---------------------------------------------------------------------------
// LSE merge of partials. A partial with LSE -inf weighs nothing and its values
// are not used (they may be anything, NaN included). Each thread holds 8
// features of a row (d..d+3 and 256+d..256+d+3, so each load of a wave covers
// 1 KiB contiguous) and merges partials in an online pass (running max,
// rescaled sum and output; the loads of four partials issued together).
// Two shapes of workgroup (4 waves):
//   light: four rows of one sequence, one wave per row, every partial of the
//          row in that wave (sequences of at most 16 partials, one or a few
//          passes);
//   heavy: one row, the four waves each taking every fourth partial, merged
//          through LDS (sequences of more than 16 partials: a long context
//          over many units; a quarter of the memory round trips).
// Heavy workgroups exist only when the decode's metadata says some sequence
// has more than 16 partials and the batch has at most kCombineOrderMaxB
// sequences: every workgroup then ranks the sequences (heavy first, each
// class in index order) and the heavy sequences' rows take the first ids, so
// they start in the first round instead of wherever their index puts them.
// Otherwise every workgroup is light. The grid has room for the light
// workgroups of the whole batch plus the extra ones of as many heavy
// sequences as the unit count allows (each has at least 16 partials beyond
// its first, and there are fewer than `units` of those in all); workgroups
// past the need return at once. When the metadata shows every sequence in
// exactly one partial (largest count 1, total equal to the batch), the decode
// has written every output itself and each workgroup returns after reading
// the header.
// md (nullable): the decode's metadata; the merge does nothing unless it was
// built for this batch and num_units (as the decode kernels check). The
// header is read before the offsets, which sit in the metadata at positions
// this call's batch sets (metadata built for a smaller batch is shorter).
// ---------------------------------------------------------------------------
constexpr int kCombineGroups = 4;    // waves per workgroup: partial groups of a heavy row, rows of a light one
constexpr int kCombineInFlight = 4;  // partials per wave whose loads are issued together
constexpr int kCombineThreads = kCombineGroups * 64;
constexpr int kCombinePass = kCombineGroups * kCombineInFlight;   // partials a heavy row takes per pass
constexpr int kCombineOrderMaxB = kCombineThreads;                // one thread per sequence ranks them

__device__ __forceinline__ int combine_light_blocks(int R) { return (R + kCombineGroups - 1) / kCombineGroups; }

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ part_out,
                                                      const float* __restrict__ part_lse,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ cu_q, int num_heads,
                                                      int B, int R, float* __restrict__ out,
                                                      float* __restrict__ lse, int skip_single,
                                                      const int32_t* __restrict__ md, int units) {
  __shared__ float s_ms[kCombineGroups][2];               // (max, sum)
  __shared__ f32x4 s_acc[kCombineGroups - 1][2][64];       // groups 1.., two halves
  __shared__ int s_count[kCombineThreads / 64];
  __shared__ int s_seq[kCombineOrderMaxB];                 // place -> sequence
  int max_pieces = 0, total_partials = -1;
  if (md) {
    // the header words are read together (one round trip)
    const int h_magic = md[MD_MAGIC], h_batch = md[MD_BATCH], h_units = md[MD_UNITS];
    max_pieces = md[MD_MAX_PIECES];
    total_partials = md[MD_TOTAL_PARTIALS];
    if ((h_magic != kMdMagic) | (h_batch != B) | (h_units != units)) return;
  }
  if (skip_single && max_pieces <= 1 && total_partials == B) return;
  const int RL = combine_light_blocks(R);
  const int id = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  bool heavy_wg = false;
  int b, r0;
  if (B <= kCombineOrderMaxB && max_pieces > kCombinePass) {
    // the order: heavy sequences first, each class in index order
    const int t = threadIdx.x;
    const int nt = t < B ? offsets[t + 1] - offsets[t] : 0;
    const bool heavy = nt > kCombinePass;
    const uint64_t hb = __builtin_amdgcn_ballot_w64(heavy);
    if (lane == 0) s_count[wave] = __builtin_popcountll(hb);
    __syncthreads();
    int heavy_before = 0, heavy_all = 0;
#pragma unroll
    for (int v = 0; v < kCombineThreads / 64; ++v) {
      heavy_before += v < wave ? s_count[v] : 0;
      heavy_all += s_count[v];
    }
    const int hr = heavy_before + __builtin_popcountll(hb & ((1ull << lane) - 1));
    if (t < B) s_seq[heavy ? hr : heavy_all + (t - hr)] = t;
    __syncthreads();
    // ids: one per row of the heavy sequences, then one per four rows of the
    // others, the place running fastest within each class
    const int hitems = heavy_all * R, light = B - heavy_all;
    if (id < hitems) {
      heavy_wg = true;
      b = s_seq[id % heavy_all];
      r0 = id / heavy_all;
    } else {
      const int j = id - hitems;
      if (j >= light * RL) return;
      b = s_seq[heavy_all + j % light];
      r0 = kCombineGroups * (j / light);
    }
  } else {
    if (id >= B * RL) return;
    b = id % B;
    r0 = kCombineGroups * (id / B);
  }
  const int k0 = offsets[b];
  const int n = offsets[b + 1] - k0;
  if (skip_single && n == 1) return;
  // partial slots hold R rows; sequence b owns the first rows_b of them
  const int rows_b = cu_q ? (cu_q[b + 1] - cu_q[b]) * num_heads : R;
  const size_t out_row0 = cu_q ? (size_t)cu_q[b] * num_heads : (size_t)b * R;
  const int d = lane * 4;
  const size_t lstride = R, ostride = (size_t)R * kDv;
  constexpr int kU = kCombineInFlight;

  // online pass of this wave over partials k0 + first, + step, ... of row r
  float M = -INFINITY, S = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  auto pass = [&](int r, int first, int step) {
    const float* pl = part_lse + (size_t)k0 * R + r;
    const float* po = part_out + ((size_t)k0 * R + r) * kDv + d;
    for (int k = first; k < n; k += step * kU) {
      float v[kU];
      f32x4 o0[kU], o1[kU];
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int kk = k + j * step;
        const bool in = kk < n;
        v[j] = in ? pl[kk * lstride] : -INFINITY;
        o0[j] = in ? *(const f32x4*)(po + kk * ostride) : f32x4{0.f, 0.f, 0.f, 0.f};
        o1[j] = in ? *(const f32x4*)(po + kk * ostride + 256) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        if (v[j] == -INFINITY) continue;
        if (v[j] > M) {
          const float c = expf(M - v[j]);   // 0 while M is -inf
          S = S * c + 1.f;
          acc0 = acc0 * c + o0[j];
          acc1 = acc1 * c + o1[j];
          M = v[j];
        } else {
          const float w = expf(v[j] - M);
          S += w;
          acc0 += w * o0[j];
          acc1 += w * o1[j];
        }
      }
    }
  };
  auto store = [&](int r, float Mt, float St, f32x4 a0, f32x4 a1) {
    const bool live = Mt != -INFINITY;
    const float inv = live ? 1.f / St : 0.f;
    float* dst = out + (out_row0 + r) * kDv + d;
    *(f32x4*)dst = a0 * inv;
    *(f32x4*)(dst + 256) = a1 * inv;
    if (lane == 0) lse[out_row0 + r] = live ? Mt + logf(St) : -INFINITY;
  };

  if (!heavy_wg) {
    const int r = r0 + wave;
    if (r >= rows_b) return;
    pass(r, 0, 1);
    store(r, M, S, acc0, acc1);
    return;
  }

  // heavy: one row, wave g takes partials g, g + 4, ...; states merged through LDS
  const int r = r0;
  const bool row_ok = r < rows_b;
  if (row_ok) pass(r, wave, kCombineGroups);
  if (lane == 0) {
    s_ms[wave][0] = M;
    s_ms[wave][1] = S;
  }
  if (wave > 0) {
    s_acc[wave - 1][0][lane] = acc0;
    s_acc[wave - 1][1][lane] = acc1;
  }
  __syncthreads();
  if (wave != 0 || !row_ok) return;
  float Mt = M;
#pragma unroll
  for (int g = 1; g < kCombineGroups; ++g) Mt = fmaxf(Mt, s_ms[g][0]);
  float St = 0.f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  if (Mt != -INFINITY) {
    const float c0 = M == -INFINITY ? 0.f : expf(M - Mt);
    St = S * c0;
    a0 = acc0 * c0;
    a1 = acc1 * c0;
#pragma unroll
    for (int g = 1; g < kCombineGroups; ++g) {
      const float mg = s_ms[g][0];
      const float cg = mg == -INFINITY ? 0.f : expf(mg - Mt);
      St += s_ms[g][1] * cg;
      a0 += cg * s_acc[g - 1][0][lane];
      a1 += cg * s_acc[g - 1][1][lane];
    }
  }
  store(r, Mt, St, a0, a1);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int variant_for(int rows) { return rows <= 16 ? VAR_NARROW16 : VAR_WIDE64X; }
int variant_rows(int variant) { return variant == VAR_NARROW16 ? 16 : 64; }   // VAR_WIDE64X, VAR_Q8: 64

hipError_t launch_decode(const DecodeParams& p, int variant, int grid_units, hipStream_t s,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  // over 16 rows: the 64-row kernels with score and output waves
  if (variant == VAR_WIDE64X) return launch_decode_so(p, grid_units, s, ev_start, ev_stop);
  // the fp8 cache on fp8 MFMA (uniform q_len only)
  if (variant == VAR_Q8) return p.cu_q ? hipErrorInvalidValue : launch_decode_so(p, grid_units, s, ev_start, ev_stop, true);
  // up to 16 rows: the producer/consumer kernels
  const int rb = (p.rows + variant_rows(variant) - 1) / variant_rows(variant);
  dim3 grid(grid_units, rb);
  KernelArgs a;
  a.p = p;
  a.p.grid_units = grid_units;
  a.md = p.md;
  a.prefix = p.md ? p.md + MD_HEADER : nullptr;
  a.split_off = p.md ? a.prefix + p.batch + 1 : nullptr;
  a.seqlens = p.seqlens;
  a.block_table = p.block_table;
  a.qptr = p.q;
  a.kv = p.kv;
  // The events (may be null) are recorded by the dispatch itself, so their
  // interval is the kernel's execution alone. Without events a plain launch
  // (what a captured graph records).
#define MLA_LAUNCH(kernel, threads)                                                                      \
  do {                                                                                                  \
    if (ev_start || ev_stop)                                                                            \
      hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, ev_start, ev_stop, 0, a.p, a.md, a.prefix, \
                            a.split_off, a.seqlens, a.block_table, a.qptr, a.kv);                        \
    else                                                                                                \
      hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, a.p, a.md, a.prefix, a.split_off, a.seqlens, \
                         a.block_table, a.qptr, a.kv);                                                   \
  } while (0)
  const bool fp8 = p.kv_scale != nullptr;
  if (fp8) MLA_LAUNCH(decode_kernel_pc8, 2 * kThreads);
  else MLA_LAUNCH(decode_kernel_pc, 2 * kThreads);
#undef MLA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_metadata(const int32_t* seqlens, int batch, int units, int min_tiles, int seq_cost,
                           int32_t* md, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(metadata_kernel, dim3(1), dim3(1024), 0, s, ev_start, ev_stop, 0, seqlens, batch,
                          units, min_tiles, seq_cost, md);
  else
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(1024), 0, s, seqlens, batch, units, min_tiles, seq_cost,
                       md);
  return hipGetLastError();
}

MLA_PAGE_VIOLATIONS_ACCESSOR(page_violations_kernels)

hipError_t launch_combine(const float* part_out, const float* part_lse, const int32_t* offsets,
                          const int32_t* cu_q, int num_heads, int batch, int rows, float* out,
                          float* lse, int skip_single, hipStream_t s, const int32_t* md, int units,
                          hipEvent_t ev_start, hipEvent_t ev_stop) {
  // light workgroups for the whole batch, plus the extra rows of as many heavy
  // sequences as there can be: each has more than kCombinePass partials, and
  // the extra partials of all sequences number fewer than `units`
  const long long light = (long long)batch * ((rows + kCombineGroups - 1) / kCombineGroups);
  const long long heavy_max = md ? std::min<long long>(batch, std::max(units - 1, 0) / kCombinePass) : 0;
  const long long wgs = light + heavy_max * (rows - (rows + kCombineGroups - 1) / kCombineGroups);
  if (wgs < 1 || wgs > INT32_MAX) return hipErrorInvalidValue;   // ids are 32-bit
  dim3 grid((unsigned)wgs);
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, s, ev_start, ev_stop, 0, part_out, part_lse,
                          offsets, cu_q, num_heads, batch, rows, out, lse, skip_single, md, units);
  else
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, s, part_out, part_lse, offsets, cu_q, num_heads,
                       batch, rows, out, lse, skip_single, md, units);
  return hipGetLastError();
}

}  // namespace mla
