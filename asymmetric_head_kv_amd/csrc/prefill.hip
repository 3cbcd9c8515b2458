// Chunked causal prefill of DiffQKV attention on the bf16 matrix cores.
//
// t_new new query rows per sequence attend the cache (which already holds
// them): new row r of sequence b sits at position p = ctx_len[b] - t_new + r
// and attends key rows 0..p.  Query head i reads K head floor(i n_k / n_q)
// and V head floor(i n_v / n_q) (Sigma architecture page, section 3.4 Steps
// 3-5); each query row is the decode formula with its own causal length.
//
// Work split: a workgroup = 4 waves = 128 consecutive query rows of one query
// head; each wave owns 32 rows.  The workgroup walks the visible keys in
// tiles of 64 through two LDS stages, software-pipelined so that the matrix
// products of one tile overlap the softmax of another inside each wave (see
// the key loop).  Tiles travel from HBM straight into LDS (16-byte
// global_load_lds through lds_dma.h, no register staging; the key loop's
// own vmcnt waits and barriers order them): K and V row-major, their 16-byte
// slots XOR-swizzled by row against bank conflicts.  The V^T operand
// is read with ds_read_b64_tr_b16, which hands each lane one value column for
// four consecutive keys, so V needs no rearranging.  Everything is computed
// transposed so that each lane owns one query row:
//   S^T[key][q]  = K . Q^T   (v_mfma_f32_32x32x16_bf16: A = K from LDS,
//                             B = Q^T held in registers for the whole walk)
//   P^T          = 2^(S^T * scale * log2 e - m), row sums per lane (over
//                  the bf16-rounded weights, v_dot2_f32_bf16), the two lane
//                  halves of a query row joined by one v_permlane32_swap;
//                  m is the row max of the split's first key tile and is
//                  then kept, so later weights may exceed 1; a 32-key block
//                  whose weights pass 2^64 moves m to that block's max
//                  first (exact: O and l always share one m)
//   O^T[d][q]   += V^T . P^T (A = V^T from LDS, B = P^T straight from the
//                             S^T accumulators, rounded to bf16)
// In the 32x32 accumulator layout lane l holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for register r; the keys a lane holds for a
// 16-key step are therefore {4h..4h+3, 8+4h..8+4h+3} (h = l/32), and the two
// transposed V reads of an operand fetch exactly those two key quads.
//
// Workgroups are renumbered so that the q-tiles of a head, and the heads of
// a K group, are dispatched to the same XCD and share its L2.

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace dqkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kPfWaves = 4;
constexpr int kPfRowsPerWave = 32;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // query rows per workgroup
constexpr int kPfKeys = 64;                          // keys per tile

// LDS tile layout: rows of 16-byte slots; logical slot c of key row j sits at
// physical slot c ^ swizzle(j).  The gfx950 LDS serves 256 bytes (64 banks)
// per cycle: a 16-byte read serves 16 lanes at a time, an 8-byte read 32, and
// lanes served together conflict when their addresses meet modulo 256 bytes
// (measured with the bank-conflict counter).  K is read 16 bytes per lane,
// 16 consecutive key rows per cycle at one logical slot: the swizzle spreads
// them over the 16 slots of a 256-byte window.  V is read 8 bytes per lane
// (transposed), 4 key rows x 4 logical slots per cycle: the swizzle moves
// each of the 4 rows to its own group of 4 slots.
template <int DK, int DV>
struct PfLds {
  static constexpr int K16 = DK / 8;                 // 16-byte slots per K row
  static constexpr int V16 = DV / 8;                 // per V row
  static constexpr int KR256 = 16 / K16;             // K rows per 256 bytes
  static constexpr int VR256 = 16 / V16;             // V rows per 256 bytes
  static constexpr int kKBytes = kPfKeys * DK * 2;
  static constexpr int kVBytes = kPfKeys * DV * 2;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kTotal = 2 * kStage;
  __device__ static int kswz(int j) { return (j / KR256) & (K16 - 1); }
  __device__ static int vswz(int j) { return 4 * ((j / VR256) & (V16 / 4 - 1)); }
};

// The two lane halves of a query row joined: v_permlane32_swap hands lanes
// 0-31 the upper half's values and lanes 32-63 the lower half's.
// (Issued as inline asm: through the builtin the compiler has dropped the
// second result and returned the first one twice.  The s_nop gives the two
// wait states a swap needs after a VALU write of its operands.)
__device__ __forceinline__ f32x2 halves(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return f32x2{a, b};
}
__device__ __forceinline__ float halves_max(float v) {
  const f32x2 h = halves(v);
  return fmaxf(h[0], h[1]);
}
__device__ __forceinline__ float halves_sum(float v) {
  const f32x2 h = halves(v);
  return h[0] + h[1];
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// kExactSum: the row sums l add the fp32 weights (needed for an accurate
// lse); otherwise they add the bf16-rounded weights that the P.V product
// multiplies, two per v_dot2_f32_bf16, which normalises O by exactly the
// weights it used.
//
// PAGED: kc / vc are page pools ([num_pages][n_k][page_rows][d_k] and
// [num_pages][n_v][page_rows][d_v]) and key row j of sequence b sits in page
// pm.table[b][j / page_rows]; pages hold a power-of-two multiple of 64 rows,
// so each 64-row tile lies in one page and costs one table read.  l_cap is
// then the table's row capacity.
template <int DK, int DV, bool kExactSum, bool PAGED>
__global__ __launch_bounds__(256) void prefill_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, bf16* __restrict__ out, float* __restrict__ lse,
    int n_q, int n_k, int n_v, int t_new, int l_cap, int n_qtiles, float qscale,
    int n_split, float* __restrict__ part_o, float* __restrict__ part_ml, PageMap pm) {
  using Lds = PfLds<DK, DV>;
  constexpr int KS = DK / 16;       // 16-wide d_k steps of S^T
  constexpr int NB = DV / 32;       // 32-wide d_v blocks of O^T
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  // Renumber workgroups: linear id -> (head, key split, q-tile) so that
  // consecutive logical ids -- the q-tiles of one head and split, which walk
  // the same K and V tiles -- land on one XCD (dispatch is round-robin over
  // 8 XCDs).
  const int nwg = gridDim.x;
  const int id = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (id % 8) * (nwg / 8) + id / 8 : id;
  const int qt = logical % n_qtiles;  // query tile
  const int hs = logical / n_qtiles;
  const int split = hs % n_split;     // key split
  const int i = hs / n_split;         // query head
  const int b = blockIdx.y;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int hk = (i * n_k) / n_q, hv = (i * n_v) / n_q;
  int L = ctx_len[b];
  L = min(L, l_cap);
  const int r0 = qt * kPfRows;                 // first query row of the workgroup
  const int base = L - t_new;                  // position of new row 0
  const int r_last = min(r0 + kPfRows, t_new) - 1;
  // (Workgroup-uniform values pinned to scalar registers with readfirstlane,
  // so that the tile bookkeeping below compiles to scalar branches.)
  const int n_keys = __builtin_amdgcn_readfirstlane(max(0, min(L, base + r_last + 1)));
  // This workgroup's share of the key tiles: split s of n_split.
  const int all_tiles = (n_keys + kPfKeys - 1) / kPfKeys;
  const int per_split = (all_tiles + n_split - 1) / n_split;
  const int t_begin = __builtin_amdgcn_readfirstlane(min(all_tiles, split * per_split));
  const int t_end = __builtin_amdgcn_readfirstlane(min(all_tiles, t_begin + per_split));

  // This lane's query row and its Q^T operands (B operand: lane = q column
  // col, 8 consecutive d_k elements 8h..8h+7 of each 16-wide step).
  const int rq = r0 + wave * kPfRowsPerWave + col;
  const int p_q = base + rq;                   // its position; sees keys <= p_q
  const bool q_ok = rq < t_new;
  bf16x8 qb[KS];
  {
    const bf16* qp = q + (((size_t)b * t_new + (q_ok ? rq : 0)) * n_q + i) * DK + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qb[s] = as_bf16x8(q_ok ? load16(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u});
    // vmcnt(0) as a compiler-visible wait: Q is in registers before the key
    // loop, so the compiler adds no wait for it inside the loop (where it
    // would also wait for the in-flight tile transfers).
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // Row j of this head's K (V) is at k_head(j) + (j % rows_per_base) * DK.
  // Contiguous: one base for the sequence; paged: the base of j's page.
  auto k_head = [&](int j0) -> const bf16* {
    if constexpr (PAGED) {
      const int blk = pm.table[(size_t)b * pm.max_blocks + (j0 >> pm.page_shift)];
      const size_t page = (size_t)min(max(blk, 0), pm.num_pages - 1);
      return kc + ((page * n_k + hk) << pm.page_shift) * DK;
    }
    return kc + ((size_t)b * n_k + hk) * l_cap * DK;
  };
  auto v_head = [&](int j0) -> const bf16* {
    if constexpr (PAGED) {
      const int blk = pm.table[(size_t)b * pm.max_blocks + (j0 >> pm.page_shift)];
      const size_t page = (size_t)min(max(blk, 0), pm.num_pages - 1);
      return vc + ((page * n_v + hv) << pm.page_shift) * DV;
    }
    return vc + ((size_t)b * n_v + hv) * l_cap * DV;
  };
  const int row_mask = PAGED ? (1 << pm.page_shift) - 1 : 0x7fffffff;

  // Tile loads, HBM -> LDS: per round the workgroup's 256 lanes fill 256
  // consecutive 16-byte slots (wave w: slots 64w .. 64w+63, in lane order).
  // Lane-constant parts: the key row of this lane's slot and the element
  // offset of its logical chunk within the row.
  constexpr int KR = kPfKeys * Lds::K16 / 256;   // K rounds per tile
  constexpr int VR = kPfKeys * Lds::V16 / 256;   // V rounds per tile
  static_assert(KR >= 1 && VR >= 1, "tile");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Slot r of this lane: key row slot / row16 of the tile, logical chunk
  // (slot % row16) ^ swizzle(row) of that row (element offset).
  auto k_row = [&](int r) { return (r * 256 + tid) / Lds::K16; };
  auto k_off = [&](int r) { return (((r * 256 + tid) % Lds::K16) ^ Lds::kswz(k_row(r))) * 8; };
  auto v_row = [&](int r) { return (r * 256 + tid) / Lds::V16; };
  auto v_off = [&](int r) { return (((r * 256 + tid) % Lds::V16) ^ Lds::vswz(v_row(r))) * 8; };
  // Byte offsets of this lane's slots from the tile's first row (full tiles).
  uint32_t k_vo[KR], v_vo[VR];
#pragma unroll
  for (int r = 0; r < KR; ++r) k_vo[r] = (uint32_t)(k_row(r) * DK + k_off(r)) * 2u;
#pragma unroll
  for (int r = 0; r < VR; ++r) v_vo[r] = (uint32_t)(v_row(r) * DV + v_off(r)) * 2u;
  // A full tile goes from its first row's address (scalar) plus the lane
  // offsets; in the last, partial tile rows past n_keys are clamped to the
  // last visible row: the loads stay in bounds and every score they feed is
  // masked.
  auto issue_k = [&](int t, int stage) {
    const int j0 = t * kPfKeys;
    const bf16* kbase = k_head(j0);
    unsigned char* kl = lds + stage * Lds::kStage + wave_u * 1024;
    if (j0 + kPfKeys <= n_keys) {
      const bf16* tb = kbase + (size_t)(j0 & row_mask) * DK;
#pragma unroll
      for (int r = 0; r < KR; ++r) dma16s(tb, k_vo[r], (lds_dma_t*)(kl + r * 4096));
    } else {
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const int j = min(j0 + k_row(r), n_keys - 1);
        dma16(kbase + (size_t)(j & row_mask) * DK + k_off(r), (lds_dma_t*)(kl + r * 4096));
      }
    }
  };
  auto issue_v = [&](int t, int stage) {
    const int j0 = t * kPfKeys;
    const bf16* vbase = v_head(j0);
    unsigned char* vl = lds + stage * Lds::kStage + Lds::kKBytes + wave_u * 1024;
    if (j0 + kPfKeys <= n_keys) {
      const bf16* tb = vbase + (size_t)(j0 & row_mask) * DV;
#pragma unroll
      for (int r = 0; r < VR; ++r) dma16s(tb, v_vo[r], (lds_dma_t*)(vl + r * 4096));
    } else {
#pragma unroll
      for (int r = 0; r < VR; ++r) {
        const int j = min(j0 + v_row(r), n_keys - 1);
        dma16(vbase + (size_t)(j & row_mask) * DV + v_off(r), (lds_dma_t*)(vl + r * 4096));
      }
    }
  };

  // Operand addresses within a stage (bytes).  K (A of S^T, 16 bytes): key
  // row kb * 32 + col, logical slot 2 ks + h.
  int k_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_rd[ks] = (col * Lds::K16 + ((2 * ks + h) ^ Lds::kswz(col))) * 16;
  // V^T (A of O^T), two transposed 8-byte reads per operand: in 16-lane
  // group g, lane j points at key row 16 st + 4 (g / 2) + j / 4 (+ 8 for the
  // second read) and value columns 32 n + 16 (g % 2) + 4 (j % 4) .. +3; lane i
  // of the group then holds column 32 n + 16 (g % 2) + i for the four rows.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_key = 4 * (g16 >> 1) + (j16 >> 2);          // + 16 st (+ 8)
  const int v_col = 16 * (g16 & 1) + 4 * (j16 & 3);        // + 32 n
  auto v_rd = [&](int st, int n, int second) -> int {
    const int key = 16 * st + v_key + 8 * second;
    const int d = 32 * n + v_col;
    return (key * Lds::V16 + ((d >> 3) ^ Lds::vswz(key))) * 16 + (d & 7) * 2;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x16{};

  const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
  // K operands of one tile (A of S^T, 16 bytes per lane), all 2 KS reads
  // issued together so that the S^T products never wait on one read each.
  auto kread = [&](const unsigned char* kl, bf16x8 (&ka)[2 * KS]) {
#pragma unroll
    for (int u = 0; u < 2 * KS; ++u)
      ka[u] = as_bf16x8(*reinterpret_cast<const u32x4*>(
          kl + (u / KS) * 32 * Lds::K16 * 16 + k_rd[u % KS]));
  };
  // S^T of one tile from its K operands into sx: two 32-key blocks.
  auto qk2 = [&](const bf16x8 (&ka)[2 * KS], f32x16 (&sx)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sx[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sx[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb * KS + ks], qb[ks], sx[kb], 0, 0, 0);
    }
  };
  auto qk = [&](const unsigned char* kl, f32x16 (&sx)[2]) {
    bf16x8 ka[2 * KS];
    kread(kl, ka);
    qk2(ka, sx);
  };
  // A tile's row maximum of the scaled scores (the two lane halves of a
  // query row joined by one shuffle).
  auto tile_max = [&](const f32x16 (&sx)[2]) -> float {
    float smax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) smax = fmaxf(fmaxf(smax, sx[kb][r]), sx[kb][r + 1]);
    }
    smax = halves_max(smax);
    return smax * qscale;
  };
  // Row maximum of one 32-key block of the scaled scores.
  auto block_max = [&](const f32x16 (&sx)[2], int kb) -> float {
    float smax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) smax = fmaxf(fmaxf(smax, sx[kb][r]), sx[kb][r + 1]);
    return halves_max(smax) * qscale;
  };
  // Overflow guard: the running max m_run is taken from the split's first
  // tile and then kept; later tiles' weights 2^(s - m_run) may exceed 1.  A
  // 32-key block whose weights pass 2^64 (inf included) is caught through
  // its row sums before its P.V product; the running max then moves to that
  // block's own max, O, l and the tile's earlier row sums are rescaled, and
  // the block's weights are recomputed (no weight then exceeds 1).
  constexpr float kPLimit = 18446744073709551616.f;  // 2^64
  auto overflowed = [&](const float (&ps)[2]) {
    return __builtin_amdgcn_ballot_w64(!(ps[0] + ps[1] <= kPLimit)) != 0;
  };
  auto rescale_to = [&](float m_tile, float (&ps_prev)[2]) {
    const float m_new = fmaxf(m_run, m_tile);
    if (m_new > m_run) {
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
      ps_prev[0] *= alpha;
      ps_prev[1] *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= alpha;
      m_run = m_new;
    }
  };
  // Causal mask of tile t (only tiles that reach past this wave's first
  // row): key j is visible to this row iff j <= p_q.
  auto mask = [&](f32x16 (&sx)[2], int t) {
    const int j0 = t * kPfKeys;
    if (j0 + kPfKeys - 1 > base + r0 + wave * kPfRowsPerWave) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + kb * 32 + (r >> 2) * 8 + 4 * h + (r & 3);
          sx[kb][r] = j <= p_q ? sx[kb][r] : -INFINITY;
        }
      }
    }
  };
  // P for one 32-key block: exponentials, row sums, bf16 operands.
  auto make_p = [&](const f32x16 (&sx)[2], int kb, bf16x8 (&pb)[4], float (&psum)[2],
                    float m_use) {
    psum[0] = 0.f;
    psum[1] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(sx[kb][r], qscale, -m_use));
      const float p1 = fast_exp2(fmaf(sx[kb][r + 1], qscale, -m_use));
      const bf16x2 pk = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
      if constexpr (kExactSum) psum[(r >> 1) & 1] += p0 + p1;
      else psum[(r >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes, psum[(r >> 1) & 1], false);
      pb[kb * 2 + (r >> 3)][r & 7] = pk[0];
      pb[kb * 2 + (r >> 3)][(r & 7) + 1] = pk[1];
    }
  };
  // O^T += V^T P^T for one 16-key step (V in LDS at vl).
  auto pv = [&](const unsigned char* vl, int st, const bf16x8 (&pb)[4]) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vl + v_rd(st, n, 0)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vl + v_rd(st, n, 1)));
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[n], 0, 0, 0);
    }
  };
  auto stage_k = [&](int st) -> const unsigned char* { return lds + st * Lds::kStage; };
  auto stage_v = [&](int st) -> const unsigned char* {
    return lds + st * Lds::kStage + Lds::kKBytes;
  };

  // Software pipeline over key tiles, K one tile ahead of V: iteration t
  // finds K(t + 1) and V(t) in LDS and S^T(t) in registers, requests K(t + 2)
  // and V(t + 1), and runs three phases that each pair matrix-core work with
  // independent VALU work of the same wave:
  //   A: S^T(t + 1) = K(t + 1) Q^T      with  P(t) for keys 0-31
  //   B: O^T += V^T(t) P^T, keys 0-31   with  P(t) for keys 32-63
  //   C: O^T += V^T(t) P^T, keys 32-63  with  the causal mask of S^T(t + 1)
  // LDS stage s holds K of tiles t_begin + s, + s + 2, ... and V of the same
  // tiles, each loaded one iteration apart.  (On the last iteration phase A
  // multiplies a stale K stage; its result is never used.)
  f32x16 sa0[2], sa1[2];
  if (t_begin < t_end) {
    issue_k(t_begin, 0);
    issue_v(t_begin, 0);
    if (t_begin + 1 < t_end) issue_k(t_begin + 1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    qk(stage_k(0), sa0);
    mask(sa0, t_begin);
    m_run = tile_max(sa0);
  }
  auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], int t, const int cur) {
    const int nxt = cur ^ 1;
    // K(t + 1) and V(t) have landed for every wave; every wave is done with
    // K(t) and V(t - 1), whose places receive K(t + 2) and V(t + 1).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < t_end) issue_k(t + 2, cur);
    if (t + 1 < t_end) issue_v(t + 1, nxt);
    float m_use = m_run == -INFINITY ? 0.f : m_run;  // rows with nothing visible
    float psA[2], psB[2];  // row sums of keys 0-31 and 32-63, two chains each
    bf16x8 pb[4];
    // The three phases run at raised wave priority (back to normal before
    // the next tile's wait): measured 2.5% faster than without.
    __builtin_amdgcn_s_setprio(1);
    bf16x8 ka[2 * KS];
    {
      const unsigned char* kl = stage_k(nxt);
#pragma unroll
      for (int u = 0; u < KS; ++u)
        ka[u] = as_bf16x8(*reinterpret_cast<const u32x4*>(kl + k_rd[u]));
      __builtin_amdgcn_sched_barrier(0);  // the first key block's reads go out first
#pragma unroll
      for (int u = KS; u < 2 * KS; ++u)
        ka[u] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            kl + 32 * Lds::K16 * 16 + k_rd[u - KS]));
    }
    qk2(ka, sn);
    make_p(sc, 0, pb, psA, m_use);
#pragma unroll
    for (int k = 0; k < 2 * KS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read for a later MFMA
    }
    if (overflowed(psA)) {
      float none[2] = {0.f, 0.f};
      rescale_to(block_max(sc, 0), none);
      m_use = m_run == -INFINITY ? 0.f : m_run;
      make_p(sc, 0, pb, psA, m_use);
    }
    pv(stage_v(cur), 0, pb);
    pv(stage_v(cur), 1, pb);
    make_p(sc, 1, pb, psB, m_use);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads for a later MFMA
    }
    if (overflowed(psB)) {
      rescale_to(block_max(sc, 1), psA);
      m_use = m_run == -INFINITY ? 0.f : m_run;
      make_p(sc, 1, pb, psB, m_use);
    }
    const float ps = halves_sum((psA[0] + psA[1]) + (psB[0] + psB[1]));
    l_run += ps;
    mask(sn, t + 1);
    pv(stage_v(cur), 2, pb);
    pv(stage_v(cur), 3, pb);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads for a later MFMA
    }
    __builtin_amdgcn_s_setprio(0);
  };
  int t = t_begin;
  for (; t + 1 < t_end; t += 2) {
    step(sa0, sa1, t, 0);
    step(sa1, sa0, t + 1, 1);
  }
  if (t < t_end) step(sa0, sa1, t, 0);

  // Store this lane's query row: rows 8*(r/4)+4h+r%4 of each 32-column block
  // of O^T are value columns.  One split: normalise and write bf16 out / lse.
  // Several: write the split's normalised fp32 partial and (m, l) for the
  // merge kernel.
  if (q_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const size_t row = ((size_t)b * t_new + rq) * n_q + i;
    if (n_split == 1) {
      bf16* op = out + row * DV;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = n * 32 + g * 8 + 4 * h;
          const uint32_t w0 = (uint32_t)f32_to_bf16(o[n][4 * g] * inv) |
                              ((uint32_t)f32_to_bf16(o[n][4 * g + 1] * inv) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16(o[n][4 * g + 2] * inv) |
                              ((uint32_t)f32_to_bf16(o[n][4 * g + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
        }
      }
      if (lse != nullptr && h == 0)
        lse[row] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
    } else {
      const size_t rows_total = (size_t)gridDim.y * t_new * n_q;
      float* po = part_o + ((size_t)split * rows_total + row) * DV;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = n * 32 + g * 8 + 4 * h;
          *reinterpret_cast<f32x4*>(po + d) =
              f32x4{o[n][4 * g] * inv, o[n][4 * g + 1] * inv, o[n][4 * g + 2] * inv,
                    o[n][4 * g + 3] * inv};
        }
      }
      if (h == 0) {
        // Split lse in log2 units (-inf when this split saw no key of the row).
        part_ml[split * rows_total + row] =
            l_run > 0.f ? m_run + fast_log2(l_run) : -INFINITY;
      }
    }
  }
}

// Merge of the key splits of one prefill: for every (sequence, row, head),
// o = sum_s 2^(lse_s - LSE) o_s with LSE = log2 sum_s 2^(lse_s), exact in real
// arithmetic.  One thread per 4 value columns of a row.
template <int DV>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    bf16* __restrict__ out, float* __restrict__ lse, size_t rows_total, int n_split) {
  constexpr int TPR = DV / 4;  // threads per row
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / TPR;
  const int c4 = gid % TPR;
  if (row >= rows_total) return;
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, part_ml[s * rows_total + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float w = fast_exp2(part_ml[s * rows_total + row] - mx);
      wsum += w;
      acc += w * *reinterpret_cast<const f32x4*>(part_o + (s * rows_total + row) * DV + c4 * 4);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const uint32_t w0 = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
  const uint32_t w1 = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(out + row * DV + c4 * 4) = make_uint2(w0, w1);
  if (lse != nullptr && c4 == 0)
    lse[row] = wsum > 0.f ? (mx + fast_log2(wsum)) * kLn2 : -INFINITY;
}

template <int DK, int DV, bool kExact, bool PAGED>
static void launch_prefill_kernel(const PrefillArgs& a, int n_qtiles) {
  dim3 grid(n_qtiles * a.n_q * a.n_split, a.batch);
  constexpr size_t lds = PfLds<DK, DV>::kTotal;
  static_assert(lds <= 65536, "dynamic LDS above 64 KiB is not launched");
  hipLaunchKernelGGL((prefill_kernel<DK, DV, kExact, PAGED>), grid, dim3(256), lds, a.stream,
                     (const bf16*)a.q,
                     (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.ctx_len, (bf16*)a.out,
                     a.lse, a.n_q, a.n_k, a.n_v, a.t_new, a.l_cap, n_qtiles,
                     a.scale * kLog2e, a.n_split, a.part_o, a.part_ml, a.pages);
}

template <int DK, int DV, bool kExact>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  const int n_qtiles = (a.t_new + kPfRows - 1) / kPfRows;
  if (a.pages.table != nullptr) launch_prefill_kernel<DK, DV, kExact, true>(a, n_qtiles);
  else launch_prefill_kernel<DK, DV, kExact, false>(a, n_qtiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.n_split == 1) return err;
  const size_t rows_total = (size_t)a.batch * a.t_new * a.n_q;
  const size_t threads = rows_total * (DV / 4);
  hipLaunchKernelGGL((prefill_merge_kernel<DV>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, a.stream, a.part_o, a.part_ml, (bf16*)a.out, a.lse,
                     rows_total, a.n_split);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_prefill_dd(const PrefillArgs& a) {
  // An exact fp32 row sum whenever lse is returned.  Without lse the split
  // merge weights carry the rounded sums' ~2^-9 relative error, far below
  // the bf16 output's own rounding.
  if (a.lse != nullptr) return launch_prefill_t<DK, DV, true>(a);
  return launch_prefill_t<DK, DV, false>(a);
}

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_prefill_dd<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_prefill_dd<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_prefill_dd<128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return launch_prefill_dd<128, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace dqkv
