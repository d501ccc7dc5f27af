// Device helpers shared by the decode kernels (mla_kernels.hip,
// mla_decode_so.hip): vector types, the LDS tile layouts and their
// direct-to-LDS page loads, cross-lane reductions, and the work-unit tile
// stream over the split schedule. Internal; device code only.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <math.h>
#include <utility>

#include "mla_internal.h"

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowBytes = kDqk * 2;                  // 1152
constexpr int kTileBytes = kPage * kRowBytes;        // 73728
constexpr int kLoadsPerThread = kTileBytes / (kThreads * 16);  // 18
constexpr float kRescaleThreshold = 8.0f;            // log2 units
constexpr float kLn2 = 0.6931471805599453f;
// s_waitcnt immediate for vmcnt(0), expcnt/lgkmcnt untouched (gfx9 encoding)
constexpr int kVmcntZero = 0x0F70;

static_assert(kLoadsPerThread * kThreads * 16 == kTileBytes, "tile must split evenly");


// LDS tile layout (bf16). Chunk c (16 bytes = features 8c..8c+7) of key k
// sits at byte
//   lds_byte(k, c) = ((c / 8) * 512 + k * 8 + ((c ^ swz3(k)) % 8)) * 16
// i.e. [128-byte line group of the row][key][chunk within the line, permuted
// by a 3-bit function of the key]. One 1 KiB load instruction fills 8 keys x
// one 128-byte line each (every 8 lanes read one whole cache line). With key
// bits k0..k3, swz3 = (k1, k0^k2, k0) (high to low bit). The LDS (64 banks of
// 4 bytes) itself flips the lowest bit of a 16-byte unit's bank group with
// address bit 10 -- key bit 3 here, rows being 128 bytes apart (measured with
// the bank-conflict counter on gfx950) -- so the unit a key's chunk lands in
// is permuted by (k1, k0^k2, k0^k3) in effect. That keeps every operand fetch
// of the kernels free of bank conflicts: 16 consecutive keys at one chunk (QK
// operand, 16 lanes per 16-byte-read cycle) and 8 consecutive keys x 2
// adjacent chunks or 4 keys x 4 chunks (transposed V operand, 32 lanes per
// 8-byte-read cycle) all land on distinct banks. (Adding the k3 term in the
// layout too would cancel the hardware's and pair keys 8 apart.)
__device__ __forceinline__ int swz3(int key) {
  return (((key >> 1) & 1) << 2) | (((key ^ (key >> 2)) & 1) << 1) | (key & 1);
}
__device__ __forceinline__ int lds_byte(int key, int chunk) {
  return ((chunk >> 3) * 512 + key * 8 + ((chunk ^ swz3(key)) & 7)) * 16;
}
constexpr int kLineGroupBytes = 8192;   // one 128-byte line of all 64 keys

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct-to-LDS 16-byte load per lane: global address sbase + voff, LDS
// destination lds_addr + 16 * lane (lds_addr wave-uniform, in M0). Written as
// inline asm so the compiler does not treat it as an LDS store it must wait on:
// the kernel orders these loads itself with explicit vmcnt waits + barriers.
// The LDS address is an M0 operand, so the compiler writes M0 itself and knows
// it is in use; the s_nop is the wait state the hardware needs between an M0
// write and a load into LDS, which the compiler cannot see inside the asm.
__device__ __forceinline__ void dma16(uint32_t voff, const uint8_t* sbase, uint32_t lds_addr) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "{m0}"(lds_addr)
      : "memory");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Page ids come from the caller's block table, which release builds trust (a
// documented caller contract). A MLA_DEBUG_BOUNDS build checks each page id
// the decode kernels use against [0, num_pages): an id outside is counted in
// this translation unit's counter and replaced by page 0, so the kernel still
// reads only pool memory. `page` is wave-uniform.
#ifdef MLA_DEBUG_BOUNDS
static __device__ unsigned int g_page_violations;
__device__ __forceinline__ int checked_page(int page, int num_pages) {
  const bool bad = (unsigned)page >= (unsigned)num_pages;
  if (bad && (threadIdx.x & 63) == 0) atomicAdd(&g_page_violations, 1u);
  return uniform(bad ? 0 : page);   // stays a scalar (the loads take it as a base)
}
// block-table entry t of a sequence with tiles entries: beyond the table's
// row (max_pages) it is an id of -1, which the check above counts
__device__ __forceinline__ int table_page(const int32_t* row, int t, int tiles, int max_pages) {
  return t < tiles ? (t < max_pages ? row[t] : -1) : 0;
}
#define MLA_PAGE_VIOLATIONS_ACCESSOR(name)                                              \
  hipError_t name(unsigned* count, bool reset) {                                        \
    hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_page_violations), sizeof(unsigned), 0, \
                                       hipMemcpyDeviceToHost);                          \
    if (e == hipSuccess && reset) {                                                     \
      const unsigned zero = 0;                                                          \
      e = hipMemcpyToSymbol(HIP_SYMBOL(g_page_violations), &zero, sizeof(unsigned), 0,  \
                            hipMemcpyHostToDevice);                                     \
    }                                                                                   \
    return e;                                                                           \
  }
#else
__device__ __forceinline__ int checked_page(int page, int) { return page; }
__device__ __forceinline__ int table_page(const int32_t* row, int t, int tiles, int) {
  return t < tiles ? row[t] : 0;
}
#define MLA_PAGE_VIOLATIONS_ACCESSOR(name) \
  hipError_t name(unsigned* count, bool) { *count = 0; return hipErrorNotSupported; }
#endif

// 64-row kernels: (unit, row block) of this workgroup. Workgroups are handed
// to the 8 XCDs round-robin by their linear id, so the row blocks of one unit
// (which read the same pages) take ids that are equal mod 8 and share that
// XCD's L2. The grid is padded to a multiple of 8 units; padding workgroups
// get a unit past the last and exit.
struct WgCoord {
  int unit, rb;
};
__device__ __forceinline__ WgCoord wg_coord(int row_blocks) {
  const int l = blockIdx.x, xcd = l & 7, k = l >> 3;
  return WgCoord{(k / row_blocks) * 8 + xcd, k % row_blocks};
}

// The 18 direct-to-LDS loads of one page. Load i of thread t fills slot
// i*256 + t: line group i/2, key 32(i%2) + t/8, in-line position t%8; the
// lane fetches the chunk that belongs there, so the 8 lanes of an octet read
// one whole 128-byte line of one key row. Keys at or past `nvalid` re-read the
// last valid key, so tail slots hold finite values (their probabilities are
// exactly 0). The loads are issued one at a time in between the MFMAs of the
// previous tile.
// 4-byte direct-to-LDS load per lane (used for the fp8 per-token scales).
__device__ __forceinline__ void dma4(uint32_t voff, const uint8_t* sbase, uint32_t lds_addr) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(sbase), "{m0}"(lds_addr)
      : "memory");
}

// The plan argument of the tile stream for callers that take only a tile's
// record (the 16-row kernels stream their pages themselves).
struct TileFacts {
  __device__ __forceinline__ void plan(const uint8_t*, const float*, int, int, LDS_AS uint8_t*, LDS_AS float*,
                                       int) {}
};

// fp8 page: 64 rows of 576 E4M3 codes, plus 64 fp32 token scales elsewhere
constexpr int kFp8RowBytes = kDqk;                        // 576
constexpr int kFp8TileBytes = kPage * kFp8RowBytes;       // 36864

// Pairwise reductions across lanes l and l ^ 32 (l ^ 16) on the VALU
// (v_permlane32_swap / v_permlane16_swap), with no LDS round trip. Both lanes
// of a pair combine the same two values in the same order, so they agree
// bit for bit.
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x4 tr_read(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
}
__device__ __forceinline__ bf16x8 ld128(const LDS_AS uint8_t* p) { return *(const LDS_AS bf16x8*)p; }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---------------------------------------------------------------------------
// Work unit and tile stream shared by the variants.
// ---------------------------------------------------------------------------
struct TileInfo {
  int b, t, L;
  bool first, last;
  bool final_out;   // epilogue writes the output (false: a partial slot)
  int slot;         // partial slot when !final_out
  int qlen;         // query tokens of sequence b
  int rows;         // its rows (qlen * heads)
  int qrow0;        // row of q / out holding its row 0
};

// TileInfo through LDS (8 ints): the producers of the narrow kernel publish
// the facts of the tiles they stream, so the compute waves never wait on the
// metadata loads of a sequence change.
__device__ __forceinline__ void put_info(LDS_AS int* d, const TileInfo& ti) {
  d[0] = ti.b;
  d[1] = ti.t;
  d[2] = ti.L;
  d[3] = (ti.first ? 1 : 0) | (ti.last ? 2 : 0) | (ti.final_out ? 4 : 0);
  d[4] = ti.slot;
  d[5] = ti.qlen;
  d[6] = ti.rows;
  d[7] = ti.qrow0;
}
__device__ __forceinline__ TileInfo get_info(const LDS_AS int* d) {
  TileInfo ti;
  ti.b = __builtin_amdgcn_readfirstlane(d[0]);
  ti.t = __builtin_amdgcn_readfirstlane(d[1]);
  ti.L = __builtin_amdgcn_readfirstlane(d[2]);
  const int fl = __builtin_amdgcn_readfirstlane(d[3]);
  ti.first = (fl & 1) != 0;
  ti.last = (fl & 2) != 0;
  ti.final_out = (fl & 4) != 0;
  ti.slot = __builtin_amdgcn_readfirstlane(d[4]);
  ti.qlen = __builtin_amdgcn_readfirstlane(d[5]);
  ti.rows = __builtin_amdgcn_readfirstlane(d[6]);
  ti.qrow0 = __builtin_amdgcn_readfirstlane(d[7]);
  return ti;
}

struct KernelArgs {
  DecodeParams p;
  const int32_t* md;
  const int32_t* prefix;
  const int32_t* split_off;
  const int32_t* seqlens;
  const int32_t* block_table;
  const uint16_t* qptr;
  const uint8_t* kv;
};

// Query tokens of sequence b and the q / out row holding its row 0: uniform
// q_len (rows = q_len * heads per sequence, sequences back to back) or the
// per-sequence offsets cu_q (q_len_b = cu_q[b+1] - cu_q[b]).
__device__ __forceinline__ int seq_qlen(const DecodeParams& p, int b) {
  return p.cu_q ? uniform(p.cu_q[b + 1] - p.cu_q[b]) : p.q_len;
}
__device__ __forceinline__ int seq_qrow0(const DecodeParams& p, int b) {
  return p.cu_q ? uniform(p.cu_q[b]) * p.num_heads : b * p.rows;
}

// Metadata built for this launch's batch and unit count. A mismatch is a
// caller error; the kernels then read no further metadata and write nothing
// (a unit index past the metadata's units would read past its arrays).
__device__ __forceinline__ bool md_matches(const DecodeParams& p) {
  return uniform(p.md[MD_MAGIC]) == kMdMagic && uniform(p.md[MD_BATCH]) == p.batch &&
         uniform(p.md[MD_UNITS]) == p.grid_units;
}

// Flattened tile range [f_begin, f_end) of unit u and the prefetch cursor.
// Everything the tile stream needs per tile is held in scalar registers or in
// one VGPR of cached page ids (lane i = page of tile pc_t0 + i), so loading a
// tile performs no metadata load; sequence changes (and every 64 tiles) reload
// the cache.
// NX: load the next sequence's facts ahead (two more registers; off in the
// kernels that have none to spare).
template <bool NX>
struct UnitT {
  int u, f_begin, f_end, b0;
  const int32_t* seq_first_unit;               // metadata: unit holding each sequence's first tile
  int bp, bp_first, bp_last, bp_L, bp_tiles;  // sequence of the prefetch cursor
  bool bp_final;
  int bp_slot;
  int bp_qlen, bp_qrow0;                       // query tokens and first q/out row
  int pc_t0, page_cache;
  // facts of sequence nx_b = bp + 1, loaded when bp is entered so that the
  // switch to it needs no memory round trip: lane 0 its length, lanes 1-2 its
  // tile prefix, lanes 3-4 its partial offsets, lanes 5-6 its query offsets,
  // lane 7 the unit holding its first tile;
  // nx_pages lane i = its page of tile i (i < max_pages)
  int nx_b, nx_facts, nx_pages;

  // false if the unit has no tiles
  __device__ __forceinline__ bool init(const KernelArgs& a, int unit) {
    u = unit;
    seq_first_unit = nullptr;
    if (a.md) {
      const int B = a.p.batch;
      if (!md_matches(a.p)) return false;
      const int32_t* ub = a.md + md_unit_begin(B, a.p.grid_units);
      seq_first_unit = a.md + md_seq_first_unit(B, a.p.grid_units);
      f_begin = ub[u];
      f_end = ub[u + 1];
      if (f_begin >= f_end) return false;
      b0 = a.split_off[B + 1 + u];
    } else {
      b0 = u;
      const int L = max(a.seqlens[b0], 0);
      f_begin = 0;
      f_end = (L + kPage - 1) / kPage;
    }
    f_begin = uniform(f_begin);
    f_end = uniform(f_end);
    b0 = uniform(b0);
    if (f_end <= f_begin) return false;
    nx_b = -1;
    enter(a, b0, f_begin);
    return true;
  }
  __device__ __forceinline__ void load_pages(const KernelArgs& a, int t0) {
    pc_t0 = t0;
    const int lane = threadIdx.x & 63;
    const int t = t0 + lane;
    page_cache = table_page(a.block_table + (size_t)bp * a.p.max_pages, t, bp_tiles, a.p.max_pages);
    // drain here (rare path) so the per-tile readlane below needs no wait
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  // Load the facts of sequence bp + 1 (split mode only: in unsplit mode a
  // unit is one sequence). Nothing waits here; the first use waits.
  __device__ __forceinline__ void prefetch_next(const KernelArgs& a) {
    nx_b = -1;
    if (!NX || !a.md || bp + 1 >= a.p.batch) return;
    nx_b = bp + 1;
    const int lane = threadIdx.x & 63;
    const int32_t* src = a.seqlens + nx_b;
    if (lane == 1 || lane == 2) src = a.prefix + nx_b + (lane - 1);
    if (lane == 3 || lane == 4) src = a.split_off + nx_b + (lane - 3);
    if (a.p.cu_q && (lane == 5 || lane == 6)) src = a.p.cu_q + nx_b + (lane - 5);
    if (lane == 7) src = seq_first_unit + nx_b;
    nx_facts = *src;
    nx_pages = lane < a.p.max_pages ? a.block_table[(size_t)nx_b * a.p.max_pages + lane] : 0;
  }
  // Make sequence bb (holding flattened tile f) the prefetch sequence.
  __device__ __forceinline__ void enter(const KernelArgs& a, int bb, int f) {
    bb = uniform(bb);
    if (NX && bb == nx_b && f == uniform(__builtin_amdgcn_readlane(nx_facts, 1))) {
      // entered at its first tile with its facts already loaded
      bp = bb;
      bp_L = max(uniform(__builtin_amdgcn_readlane(nx_facts, 0)), 0);
      bp_tiles = (bp_L + kPage - 1) / kPage;
      bp_first = f;
      bp_last = uniform(__builtin_amdgcn_readlane(nx_facts, 2));
      const int so0 = uniform(__builtin_amdgcn_readlane(nx_facts, 3));
      const int so1 = uniform(__builtin_amdgcn_readlane(nx_facts, 4));
      bp_final = so1 - so0 == 1;
      bp_slot = so0 + (u - uniform(__builtin_amdgcn_readlane(nx_facts, 7)));
      if (a.p.cu_q) {
        const int c0 = uniform(__builtin_amdgcn_readlane(nx_facts, 5));
        bp_qlen = uniform(__builtin_amdgcn_readlane(nx_facts, 6)) - c0;
        bp_qrow0 = c0 * a.p.num_heads;
      } else {
        bp_qlen = a.p.q_len;
        bp_qrow0 = bp * a.p.rows;
      }
      pc_t0 = 0;
      page_cache = (int)(threadIdx.x & 63) < bp_tiles ? nx_pages : 0;
    } else {
      bp = bb;
      bp_L = uniform(max(a.seqlens[bp], 0));
      bp_tiles = (bp_L + kPage - 1) / kPage;
      bp_qlen = seq_qlen(a.p, bp);
      bp_qrow0 = seq_qrow0(a.p, bp);
      bp_final = true;
      bp_slot = 0;
      if (a.md) {
        bp_first = uniform(a.prefix[bp]);
        bp_last = uniform(a.prefix[bp + 1]);
        bp_final = uniform(a.split_off[bp + 1] - a.split_off[bp]) == 1;
        bp_slot = uniform(a.split_off[bp] + (u - seq_first_unit[bp]));
      } else {
        bp_first = 0;
        bp_last = f_end;
      }
      load_pages(a, f - bp_first);
    }
    if (bp_last < f_end) prefetch_next(a);
  }
  // Scalar facts of flattened tile f and the plan of its loads into `dst`.
  template <class Dma>
  __device__ __forceinline__ TileInfo prepare(const KernelArgs& a, int f, LDS_AS uint8_t* dst,
                                              LDS_AS float* sdst, int tid, Dma& dma) {
    if (f >= bp_last) {
      int bb = bp + 1;
      // the prefetched sequence holds tile f unless sequences without tiles
      // come between: then walk the prefix
      if (!(NX && bb == nx_b && uniform(__builtin_amdgcn_readlane(nx_facts, 2)) > f))
        while (a.prefix[bb + 1] <= f) ++bb;
      enter(a, bb, f);
    }
    TileInfo ti;
    ti.b = bp;
    ti.t = f - bp_first;
    ti.L = bp_L;
    ti.first = (f == f_begin) || (ti.t == 0);
    ti.last = (f + 1 == f_end) || (f + 1 == bp_last);
    ti.final_out = bp_final;
    ti.slot = bp_slot;
    ti.qlen = bp_qlen;
    ti.rows = bp_qlen * a.p.num_heads;
    ti.qrow0 = bp_qrow0;
    if (ti.t - pc_t0 >= 64) load_pages(a, ti.t);
    const int page = checked_page(uniform(__builtin_amdgcn_readlane(page_cache, ti.t - pc_t0)), a.p.num_pages);
    const int nvalid = min(kPage, ti.L - ti.t * kPage);
    dma.plan(a.kv, a.p.kv_scale, page, nvalid, dst, sdst, tid);
    return ti;
  }
};
using Unit = UnitT<true>;

// O = 0, LSE = -inf for rows [r0, r1) of an empty sequence (unsplit mode).
// Called by waves 0..nwaves-1 of the block.
__device__ __forceinline__ void write_empty(const DecodeParams& p, int b, int r0, int r1, int nwaves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = seq_qlen(p, b) * p.num_heads, base = seq_qrow0(p, b);
  for (int r = r0 + wave; r < min(r1, rows); r += nwaves) {
    float* o = p.out + ((size_t)base + r) * kDv;
    for (int d = lane * 4; d < kDv; d += 256) *(f32x4*)(o + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0) p.lse[(size_t)base + r] = -INFINITY;
  }
}

// Wait for this wave's loads of the current tile (issued during the previous
// tile), then make every wave's loads visible.
__device__ __forceinline__ void wait_tile() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
}

// ---------------------------------------------------------------------------
// E4M3 tile layouts (fp8 cache): 64-byte line groups of all keys of the tile;
// chunk c (16 codes = features 16c..16c+15) of key k sits in line group c/4
// at position (c % 4) ^ swz(k), a two-bit swizzle of the key.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) int i32x2;

// The fp8 matrix-core kernels' tile: the E4M3 layout with swizzle
// (k2, k2^k3) (high to low bit), under which both of their operand reads -- 16
// consecutive keys x 4 chunk pairs (K, 16-byte reads) and 8 key pairs x 2
// chunks (V^T, transposed 8-byte reads) -- measure free of LDS bank conflicts
// on gfx950, where the swizzle (k2, k3) conflicts on the K reads.
__device__ __forceinline__ int swz2q(int key) { return (((key >> 2) & 1) << 1) | (((key >> 2) ^ (key >> 3)) & 1); }
__device__ __forceinline__ int lds8q_byte(int key, int chunk) {
  return ((chunk >> 2) * 64 + key) * 64 + (((chunk & 3) ^ swz2q(key)) << 4);
}

// 32 bytes of fp8 operand from two 16-byte halves; four floats -> four E4M3
// codes (RNE; the caller keeps them within +-448)
typedef __attribute__((ext_vector_type(8))) int i32x8;
__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ __forceinline__ u32x4 ld128u(const LDS_AS uint8_t* p) { return *(const LDS_AS u32x4*)p; }
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}
__device__ __forceinline__ i32x2 tr8_read(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)p);
}

// Eight E4M3 codes (two words) -> eight bf16 values (exact).
__device__ __forceinline__ bf16x8 widen8(unsigned lo, unsigned hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

}  // namespace mla
