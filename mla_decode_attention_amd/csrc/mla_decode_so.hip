// 64-row MLA decode kernel with score waves and output waves (gfx950).
//
// The four steps of one MLA pass -- data load, QK GEMM, online softmax update
// with the probabilities staged from registers to shared memory, PV GEMM
// (PaddleNLP issue #10157, "Multi-head Latent Attention (MLA) operator",
// overview) -- split over two kinds of wave, so that on every SIMD one wave's
// softmax runs under the other wave's matrix work (the overlap of PV with the
// softmax update that the pages' second scheme aims at, done here with one
// wave of each kind per SIMD):
//
//   score waves 0-3   S^T = K . Q^T for the wave's key half x 32 rows over
//                     all 576 features, the 32 query rows of the wave in
//                     registers (bf16 cache: 16 keys on
//                     v_mfma_f32_16x16x32_bf16; fp8 cache: 32 keys on
//                     v_mfma_scale_f32_32x32x64_f8f6f4 straight from the
//                     E4M3 codes, the query row split exactly into two E4M3
//                     parts, one row per lane pair), then the softmax of
//                     those scores, and the probabilities P (bf16) into LDS
//                     in the B-operand layout of the PV GEMM.
//   output waves 4-7  O^T[128 features, 64 rows] += V^T . P^T
//                     (v_mfma_f32_32x32x16_bf16, V^T read transposed from the
//                     same LDS tile), and the page loads.
//
// A step is half a page (32 keys) for the bf16 cache and a whole page (64
// keys) for the fp8 cache. In iteration k the score waves work on step k while
// the output waves work on step k - 1, and one workgroup barrier ends the
// iteration: it publishes step k's P and row references to the output waves
// and frees step k - 2's buffer for the loads of a later step. Steps land in a
// ring of LDS buffers (4 x 36 KiB for the bf16 cache, 3 x 40 KiB for the fp8
// cache), so the loads of a step are issued two iterations (bf16) or one
// iteration (fp8, at its start) before it is used.
//
// Online softmax without a per-step agreement. Each score wave keeps its own
// running row maximum m (base 2) and partial row sum l over its half of the
// keys of every step, raised lazily (only when a step's maximum exceeds m by more than
// 2^8, so P <= 2^8) and, one step later, raised to its partner's maximum (the
// other key half of the same rows), so the two halves agree again after a
// raise. With each step's P the wave publishes the reference m it used. The
// output waves keep their own reference M per row: when the two halves'
// references equal M (nearly every step) the PV GEMM runs as is; otherwise O is
// rescaled to the largest reference and the lower half's P is scaled down in
// registers before its MFMAs. At a sequence's end the row sum is
// l_0 2^(m_0 - M) + l_1 2^(m_1 - M), so O / l and LSE = M + log2 l are exact
// for any interleaving of raises.
//
// fp8 cache: the E4M3 codes stay in LDS and are the A operand of the QK MFMAs
// as they are; V^T comes from the transposed byte read and is widened to bf16
// in registers for the PV MFMAs; the token's scale multiplies its score and
// its probability (P_j s_j goes into the PV GEMM, P_j into the row sum). The per-token scales past a page's valid
// keys repeat the last valid one, so every scale in LDS is finite.
//
// Used for q_len * heads > 16 rows, with one query count for all sequences or
// per-sequence counts (a workgroup passes over sequences with no row in its
// 64-row block).
#include "mla_device.h"

namespace mla {
namespace so {

// LDS operand reads in flight ahead of the MFMAs: K in the score waves, V^T
// in the output waves
#ifndef SO_KD
#define SO_KD 8
#endif
#ifndef SO_VD
#define SO_VD 4
#endif
constexpr int kThreadsSo = 512;
constexpr int kRowsSo = 64;
constexpr int kNq = kDqk / 32;     // 18 k-steps of 32 features in the QK GEMM

template <bool FP8>
struct Cfg;

// bf16: steps of 32 keys. Chunk c (8 features) of key k (0..31) at byte
// ((c / 8) * 256 + k * 8 + ((c ^ swz3(k)) % 8)) * 16: line groups of 4 KiB
// (one 128-byte line of all 32 keys), conflict-free for 16 consecutive keys at
// one chunk (K operand) and for 4 keys x 4 chunks (transposed V read).
template <>
struct Cfg<false> {
  static constexpr int kKeys = 32;
  static constexpr int kBufBytes = kKeys * kRowBytes;      // 36864
  static constexpr int kBufs = 4;
  static constexpr int kLoads = kBufBytes / (256 * 16);    // 9 per output-wave lane
  static constexpr int kLineGroup = kKeys * 128;           // 4096
  __device__ static int byte(int key, int chunk) {
    return ((chunk >> 3) * 256 + key * 8 + ((chunk ^ swz3(key)) & 7)) * 16;
  }
};

// fp8: steps of 64 keys (a page). Chunk c (16 codes) of key k at
// lds8q_byte(k, c) = ((c / 4) * 64 + k) * 64 + ((c % 4) ^ swz2q(k)) * 16
// (64-byte line groups of 4 KiB, the layout of the fp8 matrix-core kernel);
// the 64 per-token scales follow the codes, then padding up to 10 loads x 256
// lanes x 16 bytes. Of the two-bit swizzles tried, (k2, k2^k3) is one of
// those under which this kernel's operand reads -- 32 consecutive keys x 2
// chunks (K, 16-byte reads) and 8 keys x 2 chunks x 2 halves (V^T,
// transposed 8-byte reads) -- measure least LDS bank conflicts on gfx950.
template <>
struct Cfg<true> {
  static constexpr int kKeys = 64;
  static constexpr int kCodeBytes = kKeys * kFp8RowBytes;  // 36864
  static constexpr int kBufBytes = 10 * 256 * 16;          // 40960
  static constexpr int kBufs = 3;
  static constexpr int kLoads = 10;
  static constexpr int kLineGroup = kKeys * 64;            // 4096
  __device__ static int byte(int key, int chunk) { return lds8q_byte(key, chunk); }
};

// Exchange area after the buffers: P [parity][k-step][row half][lane] x 16 B
// (k-steps of 16 keys), the references M [parity][key half][row] and row sums
// L [parity][key half][row] of the score waves.
constexpr int kMBytes = 2 * 2 * 64 * 4;        // 1024

// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt untouched (gfx9
// encoding: vmcnt bits 3:0 and 15:14).
constexpr int vm_imm(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

// Wait until at most `steps` steps' worth of page loads (L per lane each) are
// in flight: the loads of older steps have landed.
template <int L>
__device__ __forceinline__ void wait_steps_in_flight(int steps) {
  if (steps <= 0) __builtin_amdgcn_s_waitcnt(vm_imm(0));
  else if (steps == 1) __builtin_amdgcn_s_waitcnt(vm_imm(L));
  else __builtin_amdgcn_s_waitcnt(vm_imm(2 * L));
}

// Scalar load (s_load) of a word the kernel never writes, at a uniform index.
#define CONST_AS __attribute__((address_space(4)))
__device__ __forceinline__ int sld(const int32_t* p, size_t i) { return ((const CONST_AS int32_t*)p)[i]; }

// Page walk of one work unit: the flattened tiles [f_begin, f_end) of the
// unit, one page record at a time, every fact in scalar registers (read with
// scalar loads on a sequence change). With per-sequence query counts
// (cu_seqlens_q) a sequence with no row at the workgroup's first row row0 is
// passed over: its pages are neither loaded nor computed. PAGES: also the page
// ids, from a vector register of 64 cached ids (lane i = tile pc_t0 + i). Each
// role of wave walks the unit at its own pace: the page loads ahead, the score
// waves at their step, the output waves one step behind.
template <bool PAGES>
struct Walk {
  int u, f, f_begin, f_end, n_pages;   // n_pages: the unit's pages this workgroup computes
  int b, bfirst, blast, L;   // sequence of page f, its first flattened tile, the next sequence's, its length
  int final_out, slot;
  int qlen, rows, qrow0;     // query tokens of sequence b, its rows, its first q / out row
  int row0;
  int pc_t0, page_cache;     // lane i of page_cache: the page of tile pc_t0 + i of sequence b

  // page ids of tiles t0 .. t0 + 63 of sequence b into page_cache (a vector
  // load, waited for here: on a sequence change and every 64 pages)
  __device__ __forceinline__ void load_pages(const KernelArgs& a, int t0) {
    if (!PAGES) return;
    const DecodeParams& p = a.p;
    pc_t0 = t0;
    const int t = t0 + (int)(threadIdx.x & 63);
    const int tiles = (L + kPage - 1) / kPage;
    page_cache = table_page(p.block_table + (size_t)b * p.max_pages, t, tiles, p.max_pages);
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  __device__ __forceinline__ int seq_rows(const DecodeParams& p, int bb) const {
    return p.cu_q ? (sld(p.cu_q, bb + 1) - sld(p.cu_q, bb)) * p.num_heads : p.rows;
  }

  // false if the unit has no pages for this workgroup (or the metadata was
  // not built for this call)
  __device__ __forceinline__ bool init(const KernelArgs& a, int unit, int r0) {
    u = unit;
    row0 = r0;
    const DecodeParams& p = a.p;
    if (a.md) {
      const int B = p.batch;
      if (sld(a.md, MD_MAGIC) != kMdMagic || sld(a.md, MD_BATCH) != B || sld(a.md, MD_UNITS) != p.grid_units)
        return false;
      const size_t ub = md_unit_begin(B, p.grid_units);
      f_begin = sld(a.md, ub + u);
      f_end = sld(a.md, ub + u + 1);
      if (f_begin >= f_end) return false;
      f = f_begin;
      enter(a, sld(a.split_off, B + 1 + u));   // the sequence holding the unit's first tile
    } else {
      f_begin = f = 0;
      f_end = (max(sld(p.seqlens, u), 0) + kPage - 1) / kPage;
      if (f_end <= 0) return false;
      enter(a, u);
    }
    n_pages = f_end - f_begin;
    if (p.cu_q) {
      // the pages of the unit's sequences that have rows at row0
      n_pages = 0;
      int ff = f, bb = b, bl = blast;
      while (true) {
        const int e = min(bl, f_end);
        if (seq_rows(p, bb) > row0) n_pages += e - ff;
        if (e >= f_end) break;
        ff = e;
        ++bb;
        while (sld(a.prefix, bb + 1) <= ff) ++bb;   // sequences without tiles in between
        bl = sld(a.prefix, bb + 1);
      }
      pass_over(a);
    }
    return n_pages > 0;
  }
  __device__ __forceinline__ void enter(const KernelArgs& a, int bb) {
    const DecodeParams& p = a.p;
    b = bb;
    L = max(sld(p.seqlens, b), 0);
    if (p.cu_q) {
      const int c0 = sld(p.cu_q, b);
      qlen = sld(p.cu_q, b + 1) - c0;
      qrow0 = c0 * p.num_heads;
    } else {
      qlen = p.q_len;
      qrow0 = b * p.rows;
    }
    rows = qlen * p.num_heads;
    if (a.md) {
      bfirst = sld(a.prefix, b);
      blast = sld(a.prefix, b + 1);
      const int so0 = sld(a.split_off, b), so1 = sld(a.split_off, b + 1);
      final_out = so1 - so0 == 1;
      slot = so0 + (u - sld(a.md, md_seq_first_unit(p.batch, p.grid_units) + b));
    } else {
      bfirst = 0;
      blast = f_end;
      final_out = 1;
      slot = 0;
    }
    if (rows > row0) load_pages(a, f - bfirst);
  }
  // past the pages of sequences with no row at row0 (per-sequence q_len)
  __device__ __forceinline__ void pass_over(const KernelArgs& a) {
    while (rows <= row0 && blast < f_end) {
      f = blast;
      int bb = b + 1;
      while (sld(a.prefix, bb + 1) <= f) ++bb;
      enter(a, bb);
    }
  }
  // the record of page f (and with PAGES its page id and valid tokens); then
  // the next page
  __device__ __forceinline__ TileInfo next(const KernelArgs& a) {
    int page, nvalid;
    return next(a, page, nvalid);
  }
  __device__ __forceinline__ TileInfo next(const KernelArgs& a, int& page, int& nvalid) {
    const DecodeParams& p = a.p;
    if (f >= blast) {
      int bb = b + 1;
      while (sld(a.prefix, bb + 1) <= f) ++bb;   // sequences without tiles in between
      enter(a, bb);
      if (p.cu_q) pass_over(a);
    }
    TileInfo ti;
    ti.b = b;
    ti.t = f - bfirst;
    ti.L = L;
    ti.first = f == f_begin || ti.t == 0;
    ti.last = f + 1 == f_end || f + 1 == blast;
    ti.final_out = final_out != 0;
    ti.slot = slot;
    ti.qlen = qlen;
    ti.rows = rows;
    ti.qrow0 = qrow0;
    page = 0;
    if (PAGES) {
      if (ti.t - pc_t0 >= 64) load_pages(a, ti.t);
      page = checked_page(uniform(__builtin_amdgcn_readlane(page_cache, ti.t - pc_t0)), p.num_pages);
    }
    nvalid = min(kPage, L - ti.t * kPage);
    ++f;
    return ti;
  }
};

template <bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void decode_kernel_so(DecodeParams p_, const int32_t* __restrict__ md_, const int32_t* __restrict__ prefix_,
                      const int32_t* __restrict__ split_off_, const int32_t* __restrict__ seqlens_,
                      const int32_t* __restrict__ block_table_, const uint16_t* __restrict__ qptr_,
                      const uint8_t* __restrict__ kv_) {
  using C = Cfg<FP8>;
  constexpr int NB = C::kBufs;
  constexpr int SPP = kPage / C::kKeys;     // steps per page
  constexpr int KB = C::kKeys / 32;         // 16-key blocks of a score wave per step
  constexpr int NKS = C::kKeys / 16;        // PV k-steps (16 keys) per step
  constexpr int kPBytes = 2 * NKS * 2 * 64 * 16;
  const KernelArgs a{p_, md_, prefix_, split_off_, seqlens_, block_table_, qptr_, kv_};
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NB * C::kBufBytes + kPBytes + 2 * kMBytes];
  LDS_AS uint8_t* const bufs = (LDS_AS uint8_t*)smem;
  LDS_AS uint8_t* const pbuf = bufs + NB * C::kBufBytes;
  LDS_AS float* const mpub = (LDS_AS float*)(pbuf + kPBytes);
  LDS_AS float* const lpub = mpub + kMBytes / 4;

  const DecodeParams& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  const int R = p.rows;
  const WgCoord wc = wg_coord((R + kRowsSo - 1) / kRowsSo);
  if (wc.unit >= p.grid_units) return;
  const int row0 = wc.rb * kRowsSo;
  const int u = wc.unit;

  Walk<false> walk;   // this wave's own step (score waves) or the step behind (output waves)
  if (!walk.init(a, u, row0)) {
    if (!a.md) write_empty(p, u, row0, row0 + kRowsSo, kThreadsSo / 64);
    return;
  }
  const int n_steps = SPP * walk.n_pages;
  auto buf = [&](int k) { return bufs + (k % NB) * C::kBufBytes; };

  if (wave >= 4) {
    // ======================================================== output waves
    const int ow = wave - 4;                 // features 128 ow .. 128 ow + 127
    const int tt = tid - 256;                // 0..255: lane of the page loads
    const int n = lane & 31, h = lane >> 5;

    // ---- page loads. Step j (page f_begin + j / SPP, part j % SPP) goes to
    // buf(j); load i of lane tt fills LDS slot 256 i + tt (one KiB per wave
    // and load).
    Walk<true> wload;   // the page loads' walk, ahead of every other
    wload.init(a, u, row0);
    int plan_page = 0, plan_nvalid = 1, plan_hh = 0;
    uint32_t voff = 0;
    const uint8_t* src = nullptr;
    auto plan_step = [&](int j) {
      plan_hh = j % SPP;
      if (plan_hh == 0) wload.next(a, plan_page, plan_nvalid);
      if constexpr (!FP8) {
        // line group i, key tt / 8, position tt % 8
        const int key = tt >> 3, pos = tt & 7;
        const int src_key = min(32 * plan_hh + key, plan_nvalid - 1);
        src = a.kv + (size_t)plan_page * kTileBytes;
        voff = src_key * kRowBytes + 16 * (pos ^ swz3(key));
      } else {
        // line group i, key tt / 4, position tt % 4
        const int key = tt >> 2, pos = tt & 3;
        const int src_key = min(key, plan_nvalid - 1);
        src = a.kv + (size_t)plan_page * kFp8TileBytes;
        voff = src_key * kFp8RowBytes + 16 * (pos ^ swz2q(key));
      }
    };
    auto load = [&](int j, int i) {
      const uint32_t dst = (uint32_t)uniform((int)(uintptr_t)(buf(j) + (4 * i + ow) * 1024));
      if constexpr (!FP8) {
        dma16(voff + 128 * i, src, dst);
      } else {
        if (i < 9) {
          dma16(voff + 64 * i, src, dst);
        } else {
          // the page's 64 per-token scales (wave 4; the others re-read them
          // into the padding), those past the valid keys repeating the last
          // valid one, so that every scale in LDS is finite
          const uint8_t* sc = (const uint8_t*)(p.kv_scale + (size_t)plan_page * kPage);
          dma4(4 * min(lane, plan_nvalid - 1), sc, dst);
        }
      }
    };
    auto load_all = [&](int j) {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) load(j, i);
    };

    static_assert(NB - 3 <= 2 && 2 * C::kLoads <= 63, "wait counts");
    // prologue: steps 0 .. NB-3 in flight, step 0 landed
    for (int j = 0; j < NB - 2 && j < n_steps; ++j) {
      plan_step(j);
      load_all(j);
    }
    wait_steps_in_flight<C::kLoads>(min(NB - 3, n_steps - 1));
    lds_barrier();

    // ---- V^T operand addresses (32x32x16 A operand, keys in natural order:
    // k-slot 8h + e of k-step ks is key 16 ks + 8h + e)
    int v_lane[2][2];    // bf16: [second][fb & 1]
    int v8_lane[4];      // fp8: [fb]
    {
      const int q = lane >> 4, j = lane & 15;
      if constexpr (!FP8) {
#pragma unroll
        for (int second = 0; second < 2; ++second)
#pragma unroll
          for (int fb1 = 0; fb1 < 2; ++fb1)
            v_lane[second][fb1] = C::byte(8 * h + 4 * second + (j >> 2), 4 * fb1 + 2 * (q & 1) + ((j & 3) >> 1)) +
                                  8 * (j & 1);
      } else {
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
          v8_lane[fb] = C::byte(8 * h + (j >> 1), 8 * ow + 2 * fb + (q & 1)) + 8 * (j & 1);
      }
    }

    f32x16 o[4][2];   // [feature block][row half]
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) o[fb][0] = o[fb][1] = f32x16{};
    float M[2] = {-INFINITY, -INFINITY};
    // epilogue of a finished sequence, stored at the start of the next
    // iteration (before that iteration's page loads)
    bool pend = false;
    float pend_inv[2] = {0.f, 0.f}, pend_lse[2] = {0.f, 0.f};
    TileInfo pend_ti{};

    auto flush = [&]() {
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        const int row = row0 + 32 * rh + n;
        if (row < pend_ti.rows) {
          float* dst_o;
          float* dst_l;
          if (pend_ti.final_out) {
            dst_o = p.out + ((size_t)pend_ti.qrow0 + row) * kDv;
            dst_l = p.lse + (size_t)pend_ti.qrow0 + row;
          } else {
            dst_o = p.ws_out + ((size_t)pend_ti.slot * R + row) * kDv;
            dst_l = p.ws_lse + (size_t)pend_ti.slot * R + row;
          }
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const f32x4 v = {o[fb][rh][4 * jj], o[fb][rh][4 * jj + 1], o[fb][rh][4 * jj + 2],
                               o[fb][rh][4 * jj + 3]};
              *(f32x4*)(dst_o + 128 * ow + 32 * fb + 8 * jj + 4 * h) = v * pend_inv[rh];
            }
          if (ow == 0 && h == 0) *dst_l = pend_lse[rh];
        }
      }
      // O restarts through the rescale of the next sequence's first step
      // (alpha = 0 while M is -inf), so O itself is not touched here
      M[0] = M[1] = -INFINITY;
      pend = false;
    };

    // iteration 0: the score waves take step 0, the output waves only load
    if (NB - 2 < n_steps) {
      plan_step(NB - 2);
      load_all(NB - 2);
    }
    wait_steps_in_flight<C::kLoads>(min(NB - 2, n_steps - 1) - 1);
    lds_barrier();
    TileInfo ti{};
    for (int k = 1; k <= n_steps; ++k) {
      const int t = k - 1;   // the step computed here
      const int par = t & 1;
      const LDS_AS uint8_t* cur = buf(t);
      const int j_load = k + NB - 2;
      const bool do_load = j_load < n_steps;
      // with three buffers a step's loads have one iteration to land: all of
      // them go out first
      constexpr bool kLoadsFirst = NB == 3;
      if (do_load) plan_step(j_load);
      if (kLoadsFirst && do_load) load_all(j_load);
      // LDS reads that depend on nothing else, issued first: the references
      // of the two key halves for this lane's rows, the P operands, and the
      // first V^T operands
      float r[2][2];   // [key half][row half]
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) r[kh][rh] = mpub[(par * 2 + kh) * 64 + 32 * rh + n];
      bf16x8 pb[NKS][2];   // [k-step][row half]
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int rh = 0; rh < 2; ++rh)
          pb[ks][rh] = *(const LDS_AS bf16x8*)(pbuf + (((par * NKS + ks) * 2 + rh) * 64 + lane) * 16);
      // V^T operand of (k-step, feature block) pair i = 4 ks + fb
      constexpr int NPAIRS = 4 * NKS;
      constexpr int D = SO_VD < NPAIRS ? SO_VD : NPAIRS;
      using VOp = typename std::conditional<FP8, i32x2, bf16x8>::type;
      auto vread = [&](int i) -> VOp {
        const int ks = i >> 2, fb = i & 3;
        if constexpr (!FP8) {
          const LDS_AS uint8_t* vb = cur + (2 * ow + (fb >> 1)) * C::kLineGroup + ks * 2048;
          const bf16x4 x0 = tr_read(vb + v_lane[0][fb & 1]);
          const bf16x4 x1 = tr_read(vb + v_lane[1][fb & 1]);
          return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          return tr8_read(cur + v8_lane[fb] + ks * 1024);
        }
      };
      VOp vr[D];
#pragma unroll
      for (int i = 0; i < D; ++i) vr[i] = vread(i);

      if (pend) flush();
      if (t % SPP == 0) ti = walk.next(a);
      const bool last_step = ti.last && (t % SPP == SPP - 1);

      // (a row whose reference is still -inf takes the rescale path, which
      // zeroes O until the row has a visible key: a sequence's restart)
      const bool odd = (r[0][0] != M[0]) | (r[1][0] != M[0]) | (r[0][1] != M[1]) | (r[1][1] != M[1]) |
                       (M[0] == -INFINITY) | (M[1] == -INFINITY);
      if (__builtin_amdgcn_ballot_w64(odd) != 0) {
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const float mn = fmaxf(M[rh], fmaxf(r[0][rh], r[1][rh]));
          const float alpha = M[rh] == -INFINITY ? 0.f : exp2_fast(M[rh] - mn);
#pragma unroll
          for (int fb = 0; fb < 4; ++fb) o[fb][rh] *= alpha;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            // P of key half ks / KB down to the new reference
            const int kh = ks / KB;
            const float fk = mn == -INFINITY ? 1.f : exp2_fast(r[kh][rh] - mn);
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[ks][rh][e] = (__bf16)((float)pb[ks][rh][e] * fk);
          }
          M[rh] = mn;
        }
      }

      // ---- PV GEMM; the loads of step j_load (when not issued above) go
      //      after MFMA pairs floor(i * pairs / loads)
#pragma unroll
      for (int i = 0; i < NPAIRS; ++i) {
        const int ks = i >> 2, fb = i & 3;
        bf16x8 av;
        if constexpr (!FP8) av = vr[i % D];
        else av = widen8((unsigned)vr[i % D][0], (unsigned)vr[i % D][1]);
        if (i + D < NPAIRS) vr[i % D] = vread(i + D);
        o[fb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks][0], o[fb][0], 0, 0, 0);
        o[fb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks][1], o[fb][1], 0, 0, 0);
        if constexpr (!kLoadsFirst) {
#pragma unroll
          for (int l = 0; l < C::kLoads; ++l)
            if ((l * NPAIRS) / C::kLoads == i && do_load) load(j_load, l);
        }
        sched_fence();
      }

      if (last_step) {
        // row sums of the two key halves, in this lane's reference
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          float l = 0.f;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const float lk = lpub[(par * 2 + kh) * 64 + 32 * rh + n];
            if (r[kh][rh] != -INFINITY) l += lk * exp2_fast(r[kh][rh] - M[rh]);
          }
          const bool live = l > 0.f;
          pend_inv[rh] = live ? 1.0f / l : 0.f;
          pend_lse[rh] = live ? (M[rh] + log2_fast(l)) * kLn2 : -INFINITY;
        }
        pend_ti = ti;
        pend = true;
      }
      // step k + 1 has landed: the loads issued after its own (steps k + 2
      // .. k + NB - 2 that exist) may still be in flight
      wait_steps_in_flight<C::kLoads>(min(k + NB - 2, n_steps - 1) - (k + 1));
      lds_barrier();
    }
    if (pend) flush();
    return;
  }

  // ========================================================== score waves
  if constexpr (FP8) {
    // fp8 cache: S^T[32 keys of half kh, 32 rows of half rh] on
    // v_mfma_scale_f32_32x32x64_f8f6f4 straight from the cache's E4M3 codes,
    // one row per lane pair (lane (n, h): row 32 rh + n, keys
    // 32 kh + 8 jj + 4 h + e), so a row's reductions take one cross-lane step.
    // The query row enters as two E4M3 parts, q = hi 2^k + lo 2^(k-4), k the
    // smallest with max|q| <= 448 2^k: a bf16 value has 8 significant bits,
    // hi takes the leading 4 (nearest even) and the remainder, a multiple of
    // 2^(e-7) of at most 2^(e-4) in size, is exact in lo (for every element
    // at or above 2^-6 of 448 2^k; below that, lo rounds). The powers of two
    // are the B-operand block scales of two MFMAs per k-step, so QK runs on the
    // fp8 matrix core with no conversion of the page (lane (n, h) holds
    // features 64 cc + 16 h .. + 15 and 64 cc + 32 + 16 h .. + 15 of k-step
    // cc: chunks 4 cc + h and 4 cc + 2 + h).
    const int rh = wave & 1, kh = wave >> 1;
    const int n = lane & 31, h = lane >> 5;
    const int row = 32 * rh + n;
    int k_lane[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) k_lane[e] = C::byte(32 * kh + n, 2 * e + h);
    constexpr int NK = kDqk / 64;   // 9 k-steps of 64 features
    i32x8 qhi[NK], qlo[NK];
    int sc_hi = 127, sc_lo = 127;   // their E8M0 scale bytes: 2^k, 2^(k-4)
    float m_run = -INFINITY, l_run = 0.f;
    int row_tok = 0;
    // the query row of a sequence: its maximum from one pass over the row
    // (the lane's half, then the partner lane's), then a second pass (cache
    // hits), one k-step at a time, to the two parts
    auto quant_q = [&](const TileInfo& tq) {
      const int rr = min(row0 + row, max(tq.rows - 1, 0));
      const u32x4* qrow = (const u32x4*)(a.qptr + (size_t)min(tq.qrow0 + rr, p.q_rows - 1) * kDqk);
      // part 0-3: features 64 cc + 16 h + 0..7, + 8..15, 64 cc + 32 + 16 h + 0..7, + 8..15
      auto qword = [&](int cc, int part) { return qrow[8 * cc + 4 * (part >> 1) + 2 * h + (part & 1)]; };
      float amax = 0.f;
#pragma unroll
      for (int cc = 0; cc < NK; ++cc)
#pragma unroll
        for (int part = 0; part < 4; ++part) {
          const u32x4 w = qword(cc, part);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, w[e] << 16)),
                                     fabsf(__builtin_bit_cast(float, w[e] & 0xFFFF0000u))));
        }
      amax = max_xor32(amax);
      // amax = 1.f * 2^E: 448 * 2^(E - 8) = 1.75 * 2^E covers it unless f > .75
      const unsigned ab = __builtin_bit_cast(unsigned, amax);
      int kq = amax > 0.f ? (int)(ab >> 23) - 127 - 8 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0) : 0;
      kq = min(max(kq, -122), 126);
      const float down_hi = __builtin_bit_cast(float, (unsigned)(127 - kq) << 23);       // 2^-k
      const float down_lo = __builtin_bit_cast(float, (unsigned)(127 - kq + 4) << 23);   // 2^(4-k)
      const float up_hi = __builtin_bit_cast(float, (unsigned)(127 + kq) << 23);         // 2^k
      sc_hi = 127 + kq;
      sc_lo = 127 + kq - 4;
      sched_fence();
#pragma unroll
      for (int cc = 0; cc < NK; ++cc) {
#pragma unroll
        for (int part = 0; part < 4; ++part) {
          const u32x4 x = qword(cc, part);
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            float v[4];
            v[0] = __builtin_bit_cast(float, x[2 * e2] << 16);
            v[1] = __builtin_bit_cast(float, x[2 * e2] & 0xFFFF0000u);
            v[2] = __builtin_bit_cast(float, x[2 * e2 + 1] << 16);
            v[3] = __builtin_bit_cast(float, x[2 * e2 + 1] & 0xFFFF0000u);
            const int hi4 = pack_fp8x4(v[0] * down_hi, v[1] * down_hi, v[2] * down_hi, v[3] * down_hi);
            typedef __attribute__((ext_vector_type(2))) float f32x2_t;
            const f32x2_t d01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi4, false);
            const f32x2_t d23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi4, true);
            // the remainders are exact: both terms are multiples of 2^(e-7)
            qhi[cc][2 * part + e2] = hi4;
            qlo[cc][2 * part + e2] =
                pack_fp8x4((v[0] - d01[0] * up_hi) * down_lo, (v[1] - d01[1] * up_hi) * down_lo,
                           (v[2] - d23[0] * up_hi) * down_lo, (v[3] - d23[1] * up_hi) * down_lo);
          }
        }
        sched_fence();   // keeps the second pass's loads from piling up in registers
      }
    };

    TileInfo ti = walk.next(a);   // page of step 0
    quant_q(ti);
    lds_barrier();   // the prologue's loads of step 0 have landed
    for (int k = 0; k <= n_steps; ++k) {
      if (k < n_steps) {
        const int par = k & 1;
        const LDS_AS uint8_t* cur = buf(k);
        if (ti.first) {
          // another sequence of this unit: its query row
          if (k > 0) quant_q(ti);
          m_run = -INFINITY;
          l_run = 0.f;
          row_tok = min(row0 + row, max(ti.rows - 1, 0)) / p.num_heads;
        }
        // the partner's reference of the previous step, read ahead of its use
        const float pm = ti.first ? -INFINITY : mpub[((par ^ 1) * 2 + (kh ^ 1)) * 64 + row];
        // ---- QK GEMM: two fp8 MFMAs per k-step, read i is half i % 2 of
        //      k-step i / 2
        f32x16 sacc = f32x16{};
        {
          constexpr int NR = 2 * NK;
          constexpr int D = 6;   // three k-steps (six 64-cycle MFMAs) ahead
          auto kread = [&](int i) { return ld128u(cur + k_lane[i & 1] + (i >> 1) * C::kLineGroup); };
          u32x4 kr[D];
#pragma unroll
          for (int i = 0; i < D; ++i) kr[i] = kread(i);
#pragma unroll
          for (int cc = 0; cc < NK; ++cc) {
            const i32x8 kf = cat8(kr[(2 * cc) % D], kr[(2 * cc + 1) % D]);
            if (2 * cc + D < NR) kr[(2 * cc) % D] = kread(2 * cc + D);
            if (2 * cc + 1 + D < NR) kr[(2 * cc + 1) % D] = kread(2 * cc + 1 + D);
            sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qhi[cc], sacc, 0, 0, 0, 127, 0, sc_hi);
            sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qlo[cc], sacc, 0, 0, 0, 127, 0, sc_lo);
            sched_fence();
          }
        }
        // the record of the next page
        TileInfo nti = ti;
        if (k + 1 < n_steps) nti = walk.next(a);
        // ---- softmax of this wave's keys; the per-token scales past a
        //      page's valid keys repeat the last valid one, so all are finite
        const int step_key0 = ti.t * kPage;
        f32x4 ksc[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ksc[jj] = *(const LDS_AS f32x4*)(cur + C::kCodeBytes + (32 * kh + 8 * jj + 4 * h) * 4);
        float sv[16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[4 * jj + e] = sacc[4 * jj + e] * (ksc[jj][e] * p.scale_log2);
        if (__builtin_expect((step_key0 + kPage) > (ti.L - ti.qlen + 1), 0)) {
          const int vis = ti.L - ti.qlen + row_tok + 1;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (step_key0 + 32 * kh + 8 * jj + 4 * h + e >= vis) sv[4 * jj + e] = -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
        mx = max_xor32(mx);
        // adopt the partner's reference of the previous step (same sequence)
        const float base = fmaxf(m_run, pm);
        const float m_new = (mx > base + kRescaleThreshold) ? mx : base;
        if (m_new != m_run) {
          l_run = m_run == -INFINITY ? 0.f : l_run * exp2_fast(m_run - m_new);
          m_run = m_new;
        }
        const float m_ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 pq;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = exp2_fast(sv[4 * jj + e] - m_ref);
            l_run += pr;
            pq[e] = (__bf16)(pr * ksc[jj][e]);
          }
          // PV k-step 2 kh + jj / 2, B-operand lane n + 32 (jj % 2), keys 4h..
          *(LDS_AS bf16x4*)(pbuf + ((par * NKS + 2 * kh + (jj >> 1)) * 2 + rh) * 1024 + (n + 32 * (jj & 1)) * 16 +
                            8 * h) = pq;
        }
        if (h == 0) mpub[(par * 2 + kh) * 64 + row] = m_run;
        if (ti.last) {
          const float lt = sum_xor32(l_run);
          if (h == 0) lpub[(par * 2 + kh) * 64 + row] = lt;
        }
        ti = nti;
      }
      lds_barrier();
    }
  } else {
    // ================================================== score waves (bf16)
    static_assert(KB == 1 && NKS == 2, "bf16 steps: 32 keys, 16 per score wave");
    const int rh = wave & 1, kh = wave >> 1;
    const int c = lane & 15, g = lane >> 4;
    // K operand offsets (16x16x32 A operand: lane (c, g) holds key 16 kh + c,
    // features 8g..8g+7 of the k-step; k-step j is chunk 4j + g = line group
    // j/2, chunk-in-line 4(j%2) + g)
    int k_lane[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) k_lane[e] = C::byte(16 * kh + c, 4 * e + g);
    bf16x8 q[2][kNq];         // [row block][k-step]
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    int row_tok[2] = {0, 0};

    auto load_q = [&](const TileInfo& tq) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int rr = min(row0 + 32 * rh + 16 * rb + c, max(tq.rows - 1, 0));
        const bf16x8* qrow = (const bf16x8*)(a.qptr + (size_t)min(tq.qrow0 + rr, p.q_rows - 1) * kDqk);
#pragma unroll
        for (int j = 0; j < kNq; ++j) q[rb][j] = qrow[4 * j + g];
      }
    };

    TileInfo ti = walk.next(a);   // page of step 0
    load_q(ti);
    lds_barrier();   // the prologue's loads of step 0 have landed
    for (int k = 0; k <= n_steps; ++k) {
      if (k < n_steps) {
        const int par = k & 1;
        const int hh = k % SPP;
        const bool first_step = ti.first && hh == 0;
        const bool last_step = ti.last && hh == SPP - 1;
        const LDS_AS uint8_t* cur = buf(k);
        if (first_step) {
          // its query rows were loaded before the loop or after the previous
          // step's QK
          m_run[0] = m_run[1] = -INFINITY;
          l_run[0] = l_run[1] = 0.f;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            row_tok[rb] = min(row0 + 32 * rh + 16 * rb + c, max(ti.rows - 1, 0)) / p.num_heads;
          __builtin_amdgcn_s_waitcnt(kVmcntZero);
        }
        // the partner's reference of the previous step, read ahead of its use
        float pm[2] = {-INFINITY, -INFINITY};
        if (!first_step) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) pm[rb] = mpub[((par ^ 1) * 2 + (kh ^ 1)) * 64 + 32 * rh + 16 * rb + c];
        }
        // ---- QK GEMM: S^T[16 keys of half kh, 32 rows of half rh], one
        //      16-byte read per k-step
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        {
          constexpr int NR = kNq;
          constexpr int D = SO_KD < NR ? SO_KD : NR;
          auto kaddr = [&](int j) { return cur + k_lane[j & 1] + (j >> 1) * C::kLineGroup; };
          bf16x8 kr[D];
#pragma unroll
          for (int i = 0; i < D; ++i) kr[i] = ld128(kaddr(i));
#pragma unroll
          for (int j = 0; j < NR; ++j) {
            const bf16x8 av = kr[j % D];
            if (j + D < NR) kr[j % D] = ld128(kaddr(j + D));
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, q[0][j], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, q[1][j], s[1], 0, 0, 0);
            sched_fence();
          }
        }
        // the next step starts another sequence of this unit: its query rows
        // now (the registers are free once the MFMAs above have read them)
        TileInfo nti = ti;
        if (hh == SPP - 1 && k + 1 < n_steps) {
          nti = walk.next(a);   // the next page
          if (last_step) load_q(nti);
        }

        // ---- softmax of this wave's keys (lane (c, g): keys 16 kh + 4g + i)
        const int step_key0 = ti.t * kPage + C::kKeys * hh;
        float sv[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[rb][i] = s[rb][i] * p.scale_log2;
        if (__builtin_expect((step_key0 + C::kKeys) > (ti.L - ti.qlen + 1), 0)) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int vis = ti.L - ti.qlen + row_tok[rb] + 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (step_key0 + 16 * kh + 4 * g + i >= vis) sv[rb][i] = -INFINITY;
          }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float mx = fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3]));
          mx = max_xor32(max_xor16(mx));
          const int row = 32 * rh + 16 * rb + c;
          // adopt the partner's reference of the previous step (same sequence)
          const float base = fmaxf(m_run[rb], pm[rb]);
          const float m_new = (mx > base + kRescaleThreshold) ? mx : base;
          if (m_new != m_run[rb]) {
            l_run[rb] = m_run[rb] == -INFINITY ? 0.f : l_run[rb] * exp2_fast(m_run[rb] - m_new);
            m_run[rb] = m_new;
          }
          const float m_ref = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
          bf16x4 pq;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = exp2_fast(sv[rb][i] - m_ref);
            l_run[rb] += pr;
            pq[i] = (__bf16)pr;
          }
          // PV k-step kh, B-operand lane 16 rb + c + 32 (g / 2), keys 4 (g % 2)..
          *(LDS_AS bf16x4*)(pbuf + ((par * NKS + kh) * 2 + rh) * 1024 + (16 * rb + c + 32 * (g >> 1)) * 16 +
                            8 * (g & 1)) = pq;
          if (g == 0) mpub[(par * 2 + kh) * 64 + row] = m_run[rb];
          if (last_step) {
            const float lt = sum_xor32(sum_xor16(l_run[rb]));
            if (g == 0) lpub[(par * 2 + kh) * 64 + row] = lt;
          }
        }
        ti = nti;
      }
      lds_barrier();
    }
  }
}


// ---------------------------------------------------------------------------
// fp8 cache on fp8 MFMA with score and output waves (uniform q_len): the
// approximation of the fp8 matrix-core path -- query rows in E4M3 with a
// power-of-two scale per row (the smallest 2^k with max|q| <= 448 * 2^k),
// P'_j = P_j s_j in E4M3 with a power-of-two scale per (row, 32-key half of
// the page) whose block maximum lands in [128, 256), both contractions on
// E4M3 operands and fp32 accumulation (PaddleNLP issue #10157, quantization
// section, SageAttention2) -- on the wave split above, one page per step:
//   score wave (rh, kh)  S^T[32 keys of half kh, 32 rows of half rh] on
//                        v_mfma_scale_f32_32x32x64_f8f6f4, nine k-steps of 64
//                        features (one row per lane pair: a row's reductions
//                        take one cross-lane step); the softmax of those
//                        scores, P' into the P8 buffer and its E8M0 byte.
//   output wave ow       O^T[128 features, 64 rows] += V^T . P'^T on
//                        v_mfma_scale_f32_32x32x64_f8f6f4: one MFMA per 32
//                        features and row half takes the page's 64 keys, the
//                        B-operand block scales being the two key halves'
//                        E8M0 bytes; V^T comes transposed from the tile
//                        (ds_read_b64_tr_b8), no widening anywhere.
// The references are whole numbers (a raise rounds the new maximum up), so
// every rescale factor is a power of two: where a key half's reference is
// below the output wave's, its factor goes into that half's E8M0 block scale,
// exactly, and P itself is never touched. Otherwise the exchange, the lazy
// raise and the epilogue are those of the kernel above.
// fp8 tile in LDS: chunk c (16 codes) of key k at lds8q_byte(k, c); the 64
// per-token scales after the codes, then padding, 10 loads x 256 lanes x 16 B.
// ---------------------------------------------------------------------------
constexpr int kBufBytes8 = 10 * 256 * 16;   // 40960
constexpr int kBufs8 = 3;
constexpr int kLoads8 = 10;
constexpr int kNk8 = kDqk / 64;              // 9 k-steps of 64 features in the QK GEMM
constexpr int kPStride8 = 80;                // bytes per row of the P8 buffer: 64 keys + pad
constexpr int kP8Bytes = kRowsSo * kPStride8;

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void decode_kernel_so8(DecodeParams p_, const int32_t* __restrict__ md_, const int32_t* __restrict__ prefix_,
                       const int32_t* __restrict__ split_off_, const int32_t* __restrict__ seqlens_,
                       const int32_t* __restrict__ block_table_, const uint16_t* __restrict__ qptr_,
                       const uint8_t* __restrict__ kv_) {
  constexpr int NB = kBufs8;
  const KernelArgs a{p_, md_, prefix_, split_off_, seqlens_, block_table_, qptr_, kv_};
  // buffers | P8 [parity][row][key] | E8M0 [parity][row][key half] | M | L
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NB * kBufBytes8 + 2 * kP8Bytes + 2 * kRowsSo * 2 +
                                                         2 * kMBytes];
  LDS_AS uint8_t* const bufs = (LDS_AS uint8_t*)smem;
  LDS_AS uint8_t* const p8 = bufs + NB * kBufBytes8;
  LDS_AS uint8_t* const psc = p8 + 2 * kP8Bytes;
  LDS_AS float* const mpub = (LDS_AS float*)(psc + 2 * kRowsSo * 2);
  LDS_AS float* const lpub = mpub + kMBytes / 4;

  const DecodeParams& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  const int R = p.rows;
  const WgCoord wc = wg_coord((R + kRowsSo - 1) / kRowsSo);
  if (wc.unit >= p.grid_units) return;
  const int row0 = wc.rb * kRowsSo;
  const int u = wc.unit;

  Walk<false> walk;
  if (!walk.init(a, u, row0)) {
    if (!a.md) write_empty(p, u, row0, row0 + kRowsSo, kThreadsSo / 64);
    return;
  }
  const int n_steps = walk.n_pages;   // one page per step
  auto buf = [&](int k) { return bufs + (k % NB) * kBufBytes8; };

  if (wave >= 4) {
    // ======================================================== output waves
    const int ow = wave - 4;                 // features 128 ow .. 128 ow + 127
    const int tt = tid - 256;                // 0..255: lane of the page loads
    const int n = lane & 31, h = lane >> 5;

    // ---- page loads: load i of lane tt fills LDS slot 256 i + tt = line
    // group i, key tt / 4, position tt % 4; the tenth brings the page's 64
    // per-token scales (wave 4; the others re-read them into the padding),
    // those past the valid keys repeating the last valid one
    Walk<true> wload;
    wload.init(a, u, row0);
    int plan_page = 0, plan_nvalid = 1;
    uint32_t voff = 0;
    const uint8_t* src = nullptr;
    auto plan_step = [&](int /*j*/) {
      wload.next(a, plan_page, plan_nvalid);
      const int key = tt >> 2, pos = tt & 3;
      const int src_key = min(key, plan_nvalid - 1);
      src = a.kv + (size_t)plan_page * kFp8TileBytes;
      voff = src_key * kFp8RowBytes + 16 * (pos ^ swz2q(key));
    };
    auto load_all = [&](int j) {
      LDS_AS uint8_t* const b = buf(j);
#pragma unroll
      for (int i = 0; i < kLoads8 - 1; ++i)
        dma16(voff + 64 * i, src, (uint32_t)uniform((int)(uintptr_t)(b + (4 * i + ow) * 1024)));
      const uint8_t* sc = (const uint8_t*)(p.kv_scale + (size_t)plan_page * kPage);
      dma4(4 * min(lane, plan_nvalid - 1), sc, (uint32_t)uniform((int)(uintptr_t)(b + (4 * (kLoads8 - 1) + ow) * 1024)));
    };

    // prologue: step 0 landed
    plan_step(0);
    load_all(0);
    __builtin_amdgcn_s_waitcnt(vm_imm(0));
    lds_barrier();

    // ---- V^T operand offsets (32x32x64 A operand): 16-lane group gi covers
    // features 32 fb + 16 (gi % 2) + 0..15 of this wave's 128 and key half
    // gi / 2 of each 32-key block; as a source, lane i reads key
    // 16 (gi / 2) + 8 r1 + i / 2 at byte 8 (i % 2) of chunk 8 ow + 2 fb + gi % 2.
    // Read r of a feature block: r1 = r % 2, plus 32 keys (2048 bytes) for r / 2.
    int v_lane[4][2];
    {
      const int gi = lane >> 4, i = lane & 15;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int r1 = 0; r1 < 2; ++r1)
          v_lane[fb][r1] = lds8q_byte(16 * (gi >> 1) + 8 * r1 + (i >> 1), 8 * ow + 2 * fb + (gi & 1)) + 8 * (i & 1);
    }

    f32x16 o[4][2];   // [feature block][row half]
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) o[fb][0] = o[fb][1] = f32x16{};
    float M[2] = {-INFINITY, -INFINITY};
    float pend_inv[2] = {0.f, 0.f}, pend_lse[2] = {0.f, 0.f};
    TileInfo pend_ti{};

    auto flush = [&]() {
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        const int row = row0 + 32 * rh + n;
        if (row < pend_ti.rows) {
          float* dst_o;
          float* dst_l;
          if (pend_ti.final_out) {
            dst_o = p.out + ((size_t)pend_ti.qrow0 + row) * kDv;
            dst_l = p.lse + (size_t)pend_ti.qrow0 + row;
          } else {
            dst_o = p.ws_out + ((size_t)pend_ti.slot * R + row) * kDv;
            dst_l = p.ws_lse + (size_t)pend_ti.slot * R + row;
          }
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const f32x4 v = {o[fb][rh][4 * jj], o[fb][rh][4 * jj + 1], o[fb][rh][4 * jj + 2],
                               o[fb][rh][4 * jj + 3]};
              *(f32x4*)(dst_o + 128 * ow + 32 * fb + 8 * jj + 4 * h) = v * pend_inv[rh];
            }
          if (ow == 0 && h == 0) *dst_l = pend_lse[rh];
        }
      }
      M[0] = M[1] = -INFINITY;
    };

    // iteration 0: the score waves take step 0, the output waves load step 1
    if (n_steps > 1) {
      plan_step(1);
      load_all(1);
    }
    bool pend = false;   // a finished sequence's results are still to be stored
    TileInfo ti{};
    for (int k = 1; k <= n_steps + 1; ++k) {
      // the end of iteration k - 1, at the top of this one (so that no code
      // motion puts the PV MFMAs of iteration k - 1 behind the wait): step k
      // has landed; then a finished sequence's results go out, and have this
      // iteration to complete
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
      if (pend) {
        flush();
        pend = false;
      }
      lds_barrier();
      if (k > n_steps) break;
      const int t = k - 1;   // the step computed here
      const int par = t & 1;
      const LDS_AS uint8_t* cur = buf(t);
      // step k + 1's loads go out first: they have this iteration to land
      if (k + 1 < n_steps) {
        plan_step(k + 1);
        load_all(k + 1);
      }
      // the references of the two key halves for this lane's rows, P'^T and
      // its block scales, and every V^T operand of the step
      float r[2][2];   // [key half][row half]
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) r[kh][rh] = mpub[(par * 2 + kh) * 64 + 32 * rh + n];
      i32x8 pf[2];
      int psb[2];
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        const LDS_AS uint8_t* prow = p8 + par * kP8Bytes + (32 * rh + n) * kPStride8 + 16 * h;
        pf[rh] = cat8(ld128u(prow), ld128u(prow + 32));
        psb[rh] = psc[par * 2 * kRowsSo + (32 * rh + n) * 2 + h];
      }
      i32x2 vr[4][4];   // [feature block][read]
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int rd = 0; rd < 4; ++rd) vr[fb][rd] = tr8_read(cur + v_lane[fb][rd & 1] + (rd >> 1) * 2048);

      ti = walk.next(a);

      const bool odd = (r[0][0] != M[0]) | (r[1][0] != M[0]) | (r[0][1] != M[1]) | (r[1][1] != M[1]) |
                       (M[0] == -INFINITY) | (M[1] == -INFINITY);
      if (__builtin_amdgcn_ballot_w64(odd) != 0) {
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const float mn = fmaxf(M[rh], fmaxf(r[0][rh], r[1][rh]));
          // whole-number references: the factors are exact powers of two
          const float alpha = M[rh] == -INFINITY ? 0.f : ldexpf(1.f, (int)(M[rh] - mn));
#pragma unroll
          for (int fb = 0; fb < 4; ++fb) o[fb][rh] *= alpha;
          // this lane supplies the block scale of key half h: lowered by the
          // distance of that half's reference from the new one (a half still
          // at -inf has P' = 0)
          const float rk = h ? r[1][rh] : r[0][rh];
          if (rk != -INFINITY && mn != -INFINITY) psb[rh] = max(psb[rh] + (int)(rk - mn), 0);
          M[rh] = mn;
        }
      }

      // ---- PV GEMM: 4 feature blocks x 2 row halves, 64 keys each
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const i32x8 vf = {vr[fb][0][0], vr[fb][0][1], vr[fb][1][0], vr[fb][1][1],
                          vr[fb][2][0], vr[fb][2][1], vr[fb][3][0], vr[fb][3][1]};
        o[fb][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf[0], o[fb][0], 0, 0, 0, 127, 0, psb[0]);
        o[fb][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf[1], o[fb][1], 0, 0, 0, 127, 0, psb[1]);
      }

      // row sums of the two key halves in this lane's reference (read every
      // step, used at a sequence's end)
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        float l = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const float lk = lpub[(par * 2 + kh) * 64 + 32 * rh + n];
          l += r[kh][rh] != -INFINITY ? lk * ldexpf(1.f, (int)(r[kh][rh] - M[rh])) : 0.f;
        }
        const bool live = l > 0.f;
        pend_inv[rh] = live ? 1.0f / l : 0.f;
        pend_lse[rh] = live ? (M[rh] + log2_fast(l)) * kLn2 : -INFINITY;
      }
      if (ti.last) {
        pend_ti = ti;
        pend = true;
      }
    }
    return;
  }

  // ========================================================== score waves
  const int rh = wave & 1, kh = wave >> 1;
  const int n = lane & 31, h = lane >> 5;
  // K operand (32x32x64 A operand): lane (n, h) holds key 32 kh + n, features
  // 16 h .. 16 h + 15 (bytes 0-15) and 32 + 16 h .. (bytes 16-31) of the
  // k-step = chunks 4 cc + h and 4 cc + 2 + h (one line group per k-step)
  int k_lane[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) k_lane[e] = lds8q_byte(32 * kh + n, 2 * e + h);
  i32x8 q8[kNk8];              // E4M3 codes of row 32 rh + n, same feature order
  float qsc = 0.f;             // 2^kq * softmax scale * log2(e)
  float m_run = -INFINITY;     // reference (base 2) of the row over this key half
  float l_run = 0.f;           // partial row sum (this lane's keys)
  int row_tok = 0;

  // the query row of a sequence to E4M3 with a power-of-two scale 2^kq, the
  // smallest with max|row| <= 448 * 2^kq (not below 2^-126): the maximum from
  // one pass over the row (the lane's half, then the partner lane's), then a
  // second pass (cache hits) to the codes of the exact products q * 2^-kq
  auto quant_q = [&](const TileInfo& tq) {
    const int rr = min(row0 + 32 * rh + n, max(tq.rows - 1, 0));
    const u32x4* qrow = (const u32x4*)(a.qptr + (size_t)min(tq.qrow0 + rr, p.q_rows - 1) * kDqk);
    // part 0-3: features 64 cc + 16 h + 0..7, + 8..15, 64 cc + 32 + 16 h + 0..7, + 8..15
    auto qword = [&](int cc, int part) { return qrow[8 * cc + 4 * (part >> 1) + 2 * h + (part & 1)]; };
    float amax = 0.f;
#pragma unroll
    for (int cc = 0; cc < kNk8; ++cc)
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        const u32x4 w = qword(cc, part);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, w[e] << 16)),
                                   fabsf(__builtin_bit_cast(float, w[e] & 0xFFFF0000u))));
      }
    amax = max_xor32(amax);
    // amax = 1.f * 2^E: 448 * 2^(E - 8) = 1.75 * 2^E covers it unless f > .75
    const unsigned ab = __builtin_bit_cast(unsigned, amax);
    int kq = amax > 0.f ? (int)(ab >> 23) - 127 - 8 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0) : 0;
    kq = max(kq, -126);
    const float down = __builtin_bit_cast(float, (unsigned)(127 - kq) << 23);
    qsc = __builtin_bit_cast(float, (unsigned)(127 + kq) << 23) * p.scale_log2;
    auto qv = [&](unsigned bits) { return __builtin_bit_cast(float, bits) * down; };
#pragma unroll
    for (int cc = 0; cc < kNk8; ++cc) {
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        const u32x4 x = qword(cc, part);
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2)
          q8[cc][2 * part + e2] = pack_fp8x4(qv(x[2 * e2] << 16), qv(x[2 * e2] & 0xFFFF0000u),
                                             qv(x[2 * e2 + 1] << 16), qv(x[2 * e2 + 1] & 0xFFFF0000u));
      }
      sched_fence();   // keeps the second pass's loads from piling up in registers
    }
  };

  TileInfo ti = walk.next(a);   // page of step 0
  quant_q(ti);
  lds_barrier();   // the prologue's loads of step 0 have landed
  const int row = 32 * rh + n;
  for (int k = 0; k <= n_steps; ++k) {
    if (k < n_steps) {
      const int par = k & 1;
      const LDS_AS uint8_t* cur = buf(k);
      if (ti.first) {
        // another sequence of this unit: its query row (a reload in the
        // middle of the step, once the MFMAs have read the registers, spills)
        if (k > 0) quant_q(ti);
        m_run = -INFINITY;
        l_run = 0.f;
        row_tok = min(row0 + row, max(ti.rows - 1, 0)) / p.num_heads;
      }
      // the partner's reference of the previous step, read ahead of its use
      const float pm = ti.first ? -INFINITY : mpub[((par ^ 1) * 2 + (kh ^ 1)) * 64 + row];
      // ---- QK GEMM: S^T[32 keys of half kh, 32 rows of half rh], 9 k-steps
      f32x16 s = f32x16{};
      {
        constexpr int NR = 2 * kNk8;   // read i: k-step i / 2, half i % 2
        constexpr int D = SO_KD < NR ? SO_KD : NR;
        auto kread = [&](int i) { return ld128u(cur + k_lane[i & 1] + (i >> 1) * 4096); };
        u32x4 kr[D];
#pragma unroll
        for (int i = 0; i < D; ++i) kr[i] = kread(i);
#pragma unroll
        for (int cc = 0; cc < kNk8; ++cc) {
          const i32x8 kf = cat8(kr[(2 * cc) % D], kr[(2 * cc + 1) % D]);
          if (2 * cc + D < NR) kr[(2 * cc) % D] = kread(2 * cc + D);
          if (2 * cc + 1 + D < NR) kr[(2 * cc + 1) % D] = kread(2 * cc + 1 + D);
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, q8[cc], s, 0, 0, 0, 127, 0, 127);
          sched_fence();
        }
      }
      // ---- scores (lane (n, h): keys 32 kh + 8 jj + 4 h + e of row 32 rh + n);
      //      the per-token scales past a page's valid keys repeat the last
      //      valid one, so every scale is finite
      f32x4 ksc[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        ksc[jj] = *(const LDS_AS f32x4*)(cur + kFp8TileBytes + (32 * kh + 8 * jj + 4 * h) * 4);
      float sv[16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * jj + e] = s[4 * jj + e] * (qsc * ksc[jj][e]);

      // the record of the next page
      TileInfo nti = ti;
      if (k + 1 < n_steps) nti = walk.next(a);

      const int step_key0 = ti.t * kPage;
      if (__builtin_expect((step_key0 + kPage) > (ti.L - ti.qlen + 1), 0)) {
        const int vis = ti.L - ti.qlen + row_tok + 1;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (step_key0 + 32 * kh + 8 * jj + 4 * h + e >= vis) sv[4 * jj + e] = -INFINITY;
      }
      // ---- softmax, P' to E4M3
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
      mx = max_xor32(mx);
      // adopt the partner's reference of the previous step; a raise goes to
      // the new maximum rounded up to a whole number
      const float base = fmaxf(m_run, pm);
      const float m_new = (mx > base + kRescaleThreshold) ? ceilf(mx) : base;
      if (m_new != m_run) {
        l_run = m_run == -INFINITY ? 0.f : l_run * ldexpf(1.f, (int)(m_run - m_new));
        m_run = m_new;
      }
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
      float pp[16];
      float pmax = 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pr = exp2_fast(sv[4 * jj + e] - m_ref);
          l_run += pr;
          pp[4 * jj + e] = pr * ksc[jj][e];
          pmax = fmaxf(pmax, pp[4 * jj + e]);
        }
      pmax = max_xor32(pmax);
      // block scale 2^e with pmax / 2^e in [128, 256)
      int ex = pmax > 0.f ? (int)((__builtin_bit_cast(unsigned, pmax) >> 23) & 255u) - 126 - 8 : 0;
      ex = min(max(ex, -126), 126);
      const float inv = __builtin_bit_cast(float, (unsigned)(127 - ex) << 23);
      LDS_AS uint8_t* const prow = p8 + par * kP8Bytes + row * kPStride8 + 32 * kh + 4 * h;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *(LDS_AS int*)(prow + 8 * jj) =
            pack_fp8x4(pp[4 * jj] * inv, pp[4 * jj + 1] * inv, pp[4 * jj + 2] * inv, pp[4 * jj + 3] * inv);
      if (h == 0) {
        psc[par * 2 * kRowsSo + row * 2 + kh] = (uint8_t)(127 + ex);
        mpub[(par * 2 + kh) * 64 + row] = m_run;
      }
      if (ti.last) {
        const float lt = sum_xor32(l_run);
        if (h == 0) lpub[(par * 2 + kh) * 64 + row] = lt;
      }
      ti = nti;
    }
    lds_barrier();
  }
}

}  // namespace so

MLA_PAGE_VIOLATIONS_ACCESSOR(page_violations_so)

hipError_t launch_decode_so(const DecodeParams& p, int grid_units, hipStream_t s, hipEvent_t ev_start,
                            hipEvent_t ev_stop, bool fp8_mma) {
  const int rb = (p.rows + so::kRowsSo - 1) / so::kRowsSo;
  dim3 grid(((grid_units + 7) / 8) * 8 * rb);
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
  const bool fp8 = p.kv_scale != nullptr;
  auto kern = fp8_mma ? so::decode_kernel_so8 : fp8 ? so::decode_kernel_so<true> : so::decode_kernel_so<false>;
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(kern, grid, dim3(so::kThreadsSo), 0, s, ev_start, ev_stop, 0, a.p, a.md, a.prefix,
                          a.split_off, a.seqlens, a.block_table, a.qptr, a.kv);
  else
    hipLaunchKernelGGL(kern, grid, dim3(so::kThreadsSo), 0, s, a.p, a.md, a.prefix, a.split_off, a.seqlens,
                       a.block_table, a.qptr, a.kv);
  return hipGetLastError();
}

}  // namespace mla
