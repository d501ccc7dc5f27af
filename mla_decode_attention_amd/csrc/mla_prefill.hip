// Prefill / extend attention in the un-absorbed MLA form, gfx950.
//
// The second workload: new tokens attend causally over their sequence. Per
// head the key is [k_nope_h (128), k_rope (64, shared by all heads)] -- head
// dim 192, the DeepSeek head dim PaddleNLP issue #10157 names for its long
// prefill attention (quantization section, SageAttention) -- and the value is
// v_h (128). Query i of the N new tokens of a sequence of L sees keys
// j <= L - N + i.
//
// One workgroup = 128 query rows of one (sequence, head): 4 waves of 32 rows,
// two workgroups per CU. Keys stream in tiles of 64 through LDS (double
// buffered, direct global->LDS 16-byte loads): K from k_nope and k_rope, V
// from v, in the swizzled chunk layout of the decode kernels (conflict-free
// MFMA operand fetches). Per tile and wave:
//   QK: S^T[64 keys, 32 rows] on v_mfma_f32_32x32x16_bf16, K from LDS, Q^T
//       (12 k-steps of 16 dims, 48 registers) from registers;
//   softmax: each lane owns one row (column of S^T) and 32 of its scores, so
//       the row max and sum need one cross-lane step (lane ^ 32) and no LDS;
//       base-2 online softmax with the lazy rescale (threshold 2^8);
//   PV: O^T[128, 32 rows] += V^T . P^T. The S^T accumulator registers of a
//       16-key half block are already the B operand of that PV k-step (the
//       key order inside the k-step is permuted to match, and V^T is read
//       with the same permutation through ds_read_b64_tr_b16), so P never
//       leaves the registers.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <math.h>

#include "mla_internal.h"

namespace mla {
namespace prefill {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDNope = 128, kDRope = 64, kDK = kDNope + kDRope, kDVh = 128;
constexpr int kTile = 64;                    // keys per tile
constexpr int kRB = 1;                        // row blocks of 32 per wave (RB = 2 measured slower: 1 wave per SIMD, AGPR copies, coarser causal blocks)
constexpr int kRowsWg = 4 * 32 * kRB;          // query rows per workgroup
constexpr int kThreads = 256;
constexpr int kLineGroup = 8192;             // one 128-byte line of 64 keys
constexpr int kKBytes = kTile * kDK * 2;     // 24576
constexpr int kVBytes = kTile * kDVh * 2;    // 16384
constexpr int kStage = kKBytes + kVBytes;    // 40960
constexpr float kRescaleThreshold = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

// chunk c (8 bf16) of key k: [line group c/8][key][c%8 permuted by the key]
__device__ __forceinline__ int swz3(int key) {
  // (k1, k0^k2, k0^k3): with this kernel's operand reads (32 consecutive keys
  // at one chunk per half-wave) the LDS measures free of bank conflicts with
  // the k3 term, unlike the decode kernels' reads of 16 keys x 4 chunks
  return (((key >> 1) & 1) << 2) | (((key ^ (key >> 2)) & 1) << 1) | ((key ^ (key >> 3)) & 1);
}
__device__ __forceinline__ int lds_byte(int key, int chunk) {
  return ((chunk >> 3) * 512 + key * 8 + ((chunk ^ swz3(key)) & 7)) * 16;
}

__device__ __forceinline__ void dma16(uint32_t voff, const uint8_t* sbase, uint32_t lds_addr) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "{m0}"(lds_addr)
      : "memory");
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  barrier_lds();
}
__device__ __forceinline__ float xor32_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ bf16x8 ld128(const LDS_AS uint8_t* p) { return *(const LDS_AS bf16x8*)p; }
__device__ __forceinline__ bf16x4 tr_read(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
}

struct Args {
  const uint16_t* q;        // [Tq, H, 192]
  const uint8_t* k_nope;    // [Tk, H, 128] bf16
  const uint8_t* k_rope;    // [Tk, 64] bf16
  const uint8_t* v;         // [Tk, H, 128] bf16
  const int32_t* cu_q;
  const int32_t* cu_k;
  float* out;               // [Tq, H, 128]
  float* lse;               // [Tq, H]
  int H, nblk;
  float scale_log2;         // |softmax_scale| * log2 e
  uint32_t q_sign;          // 0x80008000 when softmax_scale < 0: q enters negated
};

// RB = query row blocks of 32 per wave: RB = 1 gives 128 rows per workgroup
// and two workgroups per CU; RB = 2 gives 256 rows per workgroup, one per CU,
// and halves the LDS bytes per MFMA (each K or V fragment feeds two MFMAs).
template <int RB>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3 - RB, 3 - RB)))
void prefill_kernel(Args a) {
  constexpr int ROWS_WG = 4 * 32 * RB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];
  LDS_AS uint8_t* const stage0 = (LDS_AS uint8_t*)smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // Longest query blocks first (causal work grows with the block index),
  // across the whole grid: workgroups are dispatched in linear-id order, so
  // the linear id runs over (query block, descending) x sequence x head and
  // every sequence's and head's longest blocks start in the first round.
  const int nseq = (int)gridDim.x / a.nblk;
  const int lin = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
  const int rank = lin / (nseq * a.H), rem = lin - rank * (nseq * a.H);
  const int head = uniform(rem % a.H);
  const int b = uniform(rem / a.H);
  const int qb = uniform(a.nblk - 1 - rank);
  const int q0 = uniform(a.cu_q[b]), N = uniform(a.cu_q[b + 1] - q0);
  const int k0 = uniform(a.cu_k[b]), L = uniform(a.cu_k[b + 1] - k0);
  const int i0 = qb * ROWS_WG;               // first query index of the block
  if (i0 >= N) return;
  const int H = a.H;
  const int off = L - N;                     // query i sees keys j <= off + i
  const int last_key = off + min(N, i0 + ROWS_WG) - 1;
  const int ntiles = last_key >= 0 ? last_key / kTile + 1 : 0;
  int qi[RB];                                // this lane's queries (row n of each row block)
  bool row_live[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qi[rb] = i0 + 32 * (RB * wave + rb) + n;
    row_live[rb] = qi[rb] < N;
  }

  // ---- query rows: B operand of S^T = K Q^T, k-step c holds dims 16c + 8h..+7
  bf16x8 qreg[RB][12];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bf16x8* qrow = (const bf16x8*)(a.q + ((size_t)(q0 + min(qi[rb], N - 1)) * H + head) * kDK);
#pragma unroll
    for (int c = 0; c < 12; ++c) {
      // with a negative softmax scale the scores use -q and |scale|, so that
      // the row max below can be taken on the raw dot products
      typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;
      const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4v, qrow[2 * c + h]) ^ a.q_sign);
      qreg[rb][c] = row_live[rb] ? v : bf16x8{};
    }
  }

  // ---- loads of one key tile
  const size_t rowK = (size_t)H * kDNope * 2;   // bytes between keys in k_nope / v
  const uint32_t lds_k0 = (uint32_t)uniform((int)(uintptr_t)(stage0 + (tid & ~63) * 16));
  // Load i (0..9) of key tile t into a stage. K load i (0-5) of thread t
  // fills slot 256i + t of the K region: line group i/2, key 32(i%2) + t/8,
  // in-line position t%8 -- loads 0-3 from k_nope (chunks 0..15), 4-5 from
  // k_rope (chunks 16..23); V loads 6-9 fill the V region the same way. Keys
  // at or past the sequence end re-read the last key.
  auto issue_one = [&](int t, int stage, int i) {
    const int kt0 = t * kTile;
    const int nvalid = min(kTile, L - kt0);
    const uint32_t lds = lds_k0 + stage * kStage;
    const int ii = i < 6 ? i : i - 6;
    const int key = 32 * (ii & 1) + (tid >> 3);
    const int src = key < nvalid ? key : nvalid - 1;
    const int c = 8 * (ii >> 1) + ((tid & 7) ^ swz3(key));
    if (i < 4)
      dma16((uint32_t)(src * rowK + c * 16), a.k_nope + ((size_t)(k0 + kt0) * H + head) * (kDNope * 2),
            lds + i * 4096);
    else if (i < 6)
      dma16((uint32_t)(src * (kDRope * 2) + (c - 16) * 16), a.k_rope + (size_t)(k0 + kt0) * (kDRope * 2),
            lds + i * 4096);
    else
      dma16((uint32_t)(src * rowK + c * 16), a.v + ((size_t)(k0 + kt0) * H + head) * (kDVh * 2),
            lds + kKBytes + ii * 4096);
  };

  // per-lane LDS offsets: K operand (key 32kb + n, chunk 2c + h), V^T reads
  int k_lane[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) k_lane[kb][q4] = lds_byte(32 * kb + n, 2 * q4 + h);
  int v_lane[2][2];   // [second][fb % 2]
  {
    const int qq = lane >> 4, j = lane & 15;
#pragma unroll
    for (int second = 0; second < 2; ++second)
#pragma unroll
      for (int par = 0; par < 2; ++par)
        v_lane[second][par] = kKBytes + lds_byte(4 * h + (j >> 2) + 8 * second, 4 * par + 2 * (qq & 1) + ((j & 3) >> 1)) +
                              8 * (j & 1);
  }

  f32x16 o[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) o[rb][fb] = f32x16{};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }
  bool first = true;

  if (ntiles > 0)
#pragma unroll
    for (int i = 0; i < 10; ++i) issue_one(0, 0, i);
  for (int t = 0; t < ntiles; ++t) {
    LDS_AS uint8_t* const cur = stage0 + (t & 1) * kStage;
    wait_loads();
    // the next tile's 10 loads go out one per even QK slot (not as a burst)
    const bool load_next = t + 1 < ntiles;

    // ---- QK: S^T[64 keys, 32 rows] per row block; each K fragment feeds RB MFMAs
    f32x16 sacc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb][0] = sacc[rb][1] = f32x16{};
    {
      auto kaddr = [&](int i) {
        const int c = i >> 1, kb = i & 1;
        return cur + k_lane[kb][c & 3] + (c >> 2) * kLineGroup;
      };
      constexpr int NQ = 24, D = 6;
      bf16x8 ring[D];
#pragma unroll
      for (int i = 0; i < D; ++i) ring[i] = ld128(kaddr(i));
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const bf16x8 av = ring[i % D];
        if (i + D < NQ) ring[i % D] = ld128(kaddr(i + D));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[rb][i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[rb][i >> 1], sacc[rb][i & 1], 0, 0, 0);
        if ((i & 1) == 0 && i < 20 && load_next) issue_one(t + 1, (t + 1) & 1, i >> 1);
      }
    }

    // ---- softmax: row qi[rb], keys 64t + 32kb + 8(r/4) + 4h + r%4. The max is
    //      taken on the raw scores (the scale c is positive; q carries its
    //      sign), and the scale is folded into the exponent: P = 2^(s * c - m).
    const int kt0 = t * kTile;
    if (kt0 + kTile - 1 > off + i0) {          // tile reaches past the block's first row's last key
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kt0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3) > off + qi[rb]) sacc[rb][kb][r] = -INFINITY;
    }
    float alpha[RB];
    bool any_raise = first;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rb][kb][r]);
      mx = xor32_max(mx) * a.scale_log2;
      const float m_new = fmaxf(m_run[rb], mx);
      const bool raise = first || m_new > m_run[rb] + kRescaleThreshold;
      alpha[rb] = first ? 0.0f : raise ? __builtin_amdgcn_exp2f(m_run[rb] - m_new) : 1.0f;
      if (raise) m_run[rb] = m_new;
      any_raise |= raise;
    }
    if (__builtin_amdgcn_ballot_w64(any_raise)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) o[rb][fb] *= alpha[rb];
        l_run[rb] *= alpha[rb];
      }
    }
    first = false;

    // ---- PV: O^T[128 dims, 32 rows] += V^T . P^T; P for k-step ks = 2kb + s is
    //      the S registers 8s..8s+7 of block kb; each V fragment feeds RB MFMAs
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 pb[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m_eff = m_run[rb] == -INFINITY ? 0.0f : m_run[rb];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr =
              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rb][ks >> 1][8 * (ks & 1) + e], a.scale_log2, -m_eff));
          l_run[rb] += pr;
          pb[rb][e] = (__bf16)pr;
        }
      }
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const LDS_AS uint8_t* base = cur + (fb >> 1) * kLineGroup + ks * 2048;
        const bf16x4 r0 = tr_read(base + v_lane[0][fb & 1]);
        const bf16x4 r1 = tr_read(base + v_lane[1][fb & 1]);
        const bf16x8 av = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[rb], o[rb][fb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l, LSE = (m + log2 l) ln 2
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_row = xor32_sum(l_run[rb]);
    if (!row_live[rb]) continue;
    const bool live = l_row > 0.f;
    const float inv = live ? 1.0f / l_row : 0.f;
    const size_t row = (size_t)(q0 + qi[rb]) * H + head;
    float* dst = a.out + row * kDVh;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 v = {o[rb][fb][4 * jj], o[rb][fb][4 * jj + 1], o[rb][fb][4 * jj + 2], o[rb][fb][4 * jj + 3]};
        *(f32x4*)(dst + 32 * fb + 8 * jj + 4 * h) = v * inv;
      }
    if (h == 0) a.lse[row] = live ? (m_run[rb] + __builtin_amdgcn_logf(l_row)) * kLn2 : -INFINITY;
  }
}

}  // namespace prefill

int prefill_rows_per_block() { return prefill::kRowsWg; }

hipError_t launch_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v,
                          const int32_t* cu_q, const int32_t* cu_k, int batch, int max_q_len, int num_heads,
                          float softmax_scale, float* out, float* lse, hipStream_t s, hipEvent_t ev_start,
                          hipEvent_t ev_stop) {
  prefill::Args a;
  a.q = q;
  a.k_nope = (const uint8_t*)k_nope;
  a.k_rope = (const uint8_t*)k_rope;
  a.v = (const uint8_t*)v;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.out = out;
  a.lse = lse;
  a.H = num_heads;
  a.nblk = (max_q_len + prefill::kRowsWg - 1) / prefill::kRowsWg;
  a.scale_log2 = fabsf(softmax_scale) * 1.4426950408889634f;
  a.q_sign = softmax_scale < 0.f ? 0x80008000u : 0u;
  dim3 grid(batch * a.nblk, num_heads);
  // the events (may be null) are recorded by the dispatch itself
  hipExtLaunchKernelGGL(prefill::prefill_kernel<prefill::kRB>, grid, dim3(prefill::kThreads), 0, s, ev_start, ev_stop, 0, a);
  return hipGetLastError();
}

}  // namespace mla
