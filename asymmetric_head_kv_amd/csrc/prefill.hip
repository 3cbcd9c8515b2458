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
// tiles of 64, double-buffered in LDS: the K tile row-major (rows padded by
// 16 bytes against bank conflicts) and the V tile rearranged so that every
// lane's 8 matrix-core operands for one value column are 16 contiguous
// bytes.  Everything is computed transposed so that each lane owns one query
// row:
//   S^T[key][q]  = K . Q^T   (v_mfma_f32_32x32x16_bf16: A = K from LDS,
//                             B = Q^T held in registers for the whole walk)
//   P^T          = 2^(S^T * scale * log2 e - m), online max / sum per lane
//                  (the sum over the bf16-rounded weights, v_dot2_f32_bf16),
//                  the two lane halves of a query row joined by one shuffle;
//                  the running max m is moved (and O rescaled) only when it
//                  grows by more than 2^8 (exact: O and l share the stale m)
//   O^T[d][q]   += V^T . P^T (A = V^T from LDS, B = P^T straight from the
//                             S^T accumulators, rounded to bf16)
// In the 32x32 accumulator layout lane l holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for register r; the keys a lane holds for a
// 16-key step are therefore {4h..4h+3, 8+4h..8+4h+3} (h = l/32), and the V
// tile is stored with exactly that key order so that A and B agree.
//
// Workgroups are renumbered so that the q-tiles of a head, and the heads of
// a K group, are dispatched to the same XCD and share its L2.

#include "device_common.h"
#include "launch.h"

namespace dqkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 4;
constexpr int kPfRowsPerWave = 32;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // query rows per workgroup
constexpr int kPfKeys = 64;                          // keys per tile

template <int DK, int DV>
struct PfLds {
  static constexpr int kPitch = DK * 2 + 16;               // K row pitch (bytes)
  static constexpr int kKBytes = kPfKeys * kPitch;
  static constexpr int kVBytes = kPfKeys * DV * 2;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kTotal = 2 * kStage;
};

// V tile in LDS: for 16-key step s, lane half h and value column d, the 16
// bytes at slot (s * 2 + h) * d_v + vswz(d) hold that column's 8 keys of the
// half, so the 32 lanes of a half read one contiguous run (no bank
// conflicts).  vswz XORs a column's low three bits with bits 3-5: each group
// of 8 columns stays in place for the reads while the cooperative stores,
// whose lanes are 8 columns apart, spread over the banks.
__device__ __forceinline__ int vswz(int d) { return d ^ ((d >> 3) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// kExactSum: the row sums l add the fp32 weights (needed for an accurate
// lse); otherwise they add the bf16-rounded weights that the P.V product
// multiplies, two per v_dot2_f32_bf16, which normalises O by exactly the
// weights it used.
template <int DK, int DV, bool kExactSum>
__global__ __launch_bounds__(256) void prefill_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, bf16* __restrict__ out, float* __restrict__ lse,
    int n_q, int n_k, int n_v, int t_new, int l_cap, int n_qtiles, float qscale,
    int n_split, float* __restrict__ part_o, float* __restrict__ part_ml) {
  using Lds = PfLds<DK, DV>;
  constexpr int KS = DK / 16;       // 16-wide d_k steps of S^T
  constexpr int NB = DV / 32;       // 32-wide d_v blocks of O^T
  constexpr int K16 = DK / 8;       // 16-byte chunks per K row
  constexpr int KCH = kPfKeys * K16 / 256;  // K chunks per thread per tile
  constexpr int VD8 = DV / 8;       // 8-column chunks per V row
  static_assert(KCH >= 1, "K tile");
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
  const int n_keys = max(0, min(L, base + r_last + 1));  // keys any row here sees
  // This workgroup's share of the key tiles: split s of n_split.
  const int all_tiles = (n_keys + kPfKeys - 1) / kPfKeys;
  const int per_split = (all_tiles + n_split - 1) / n_split;
  const int t_begin = min(all_tiles, split * per_split);
  const int t_end = min(all_tiles, t_begin + per_split);

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
  }

  const bf16* kbase = kc + ((size_t)b * n_k + hk) * l_cap * DK;
  const bf16* vbase = vc + ((size_t)b * n_v + hv) * l_cap * DV;

  // Cooperative tile loads.  K: KCH 16-byte chunks per thread.  V: each
  // thread owns 4 consecutive keys x 8 consecutive columns.
  const int v_dc = tid % VD8;            // column chunk
  const int v_kq = tid / VD8;            // key quad (0..15 when active)
  const bool v_act = VD8 * (kPfKeys / 4) >= 256 || v_kq < kPfKeys / 4;
  u32x4 kreg[KCH];
  u32x4 vreg[4];

  // Per-thread base pointers of the cooperative loads; a tile adds j0 rows.
  // Rows past n_keys (only in the last tile) are clamped to the last
  // visible row: the loads stay in bounds and every score they feed is
  // masked.
  const bf16* kthr[KCH];
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int e = tid + c * 256;
    kthr[c] = kbase + (size_t)(e / K16) * DK + (e % K16) * 8;
  }
  const bf16* vthr = vbase + (size_t)(v_kq * 4) * DV + v_dc * 8;
  auto load_tile = [&](int t) {
    const int j0 = t * kPfKeys;
    if (j0 + kPfKeys <= n_keys) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) kreg[c] = load16(kthr[c] + (size_t)j0 * DK);
      if (v_act) {
#pragma unroll
        for (int k = 0; k < 4; ++k) vreg[k] = load16(vthr + (size_t)(j0 + k) * DV);
      }
    } else {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int e = tid + c * 256;
        const int j = min(j0 + e / K16, n_keys - 1);
        kreg[c] = load16(kbase + (size_t)j * DK + (e % K16) * 8);
      }
      if (v_act) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = min(j0 + v_kq * 4 + k, n_keys - 1);
          vreg[k] = load16(vbase + (size_t)j * DV + v_dc * 8);
        }
      }
    }
  };

  auto store_tile = [&](int stage) {
    unsigned char* kl = lds + stage * Lds::kStage;
    unsigned char* vl = kl + Lds::kKBytes;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int e = tid + c * 256;
      const int key = e / K16, ch = e % K16;
      *reinterpret_cast<u32x4*>(kl + key * Lds::kPitch + ch * 16) = kreg[c];
    }
    if (v_act) {
      // Keys 4*v_kq .. +3 lie in 16-key step s = v_kq / 4, quad qq = v_kq % 4:
      // quads 0,1 fill bytes 0-7 of halves h = 0,1; quads 2,3 bytes 8-15.
      const int s = v_kq >> 2, qq = v_kq & 3;
      const int hh = qq & 1, off = (qq >> 1) * 8;
      // Transpose the 4 keys x 8 columns block: column d gets 4 keys (8 bytes).
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {       // word dw holds columns 2dw, 2dw+1
        const uint32_t w0 = vreg[0][dw], w1 = vreg[1][dw], w2 = vreg[2][dw], w3 = vreg[3][dw];
        // low halves (column 2dw) of keys 0..3, then high halves (column 2dw+1)
        const uint32_t lo01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
        const int d0 = v_dc * 8 + 2 * dw;
        uint2* p0 = reinterpret_cast<uint2*>(vl + ((s * 2 + hh) * DV + vswz(d0)) * 16 + off);
        uint2* p1 = reinterpret_cast<uint2*>(vl + ((s * 2 + hh) * DV + vswz(d0 + 1)) * 16 + off);
        *p0 = make_uint2(lo01, lo23);
        *p1 = make_uint2(hi01, hi23);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x16{};

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int stage = (t - t_begin) & 1;
    load_tile(t + 1);  // past the last tile: clamped rows, stored but never read
    const unsigned char* kl = lds + stage * Lds::kStage;
    const unsigned char* vl = kl + Lds::kKBytes;
    const int j0 = t * kPfKeys;

    // S^T for two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            kl + (kb * 32 + col) * Lds::kPitch + (ks * 16 + 8 * h) * 2));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s[kb], 0, 0, 0);
      }
    }

    // Causal mask (only on tiles that reach past this wave's first row):
    // key j is visible to this row iff j <= p_q.
    const bool diag = j0 + kPfKeys - 1 > base + r0 + wave * kPfRowsPerWave;
    if (diag) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + kb * 32 + (r >> 2) * 8 + 4 * h + (r & 3);
          s[kb][r] = j <= p_q ? s[kb][r] : -INFINITY;
        }
      }
    }
    float smax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) smax = fmaxf(fmaxf(smax, s[kb][r]), s[kb][r + 1]);
    }
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    // Lazy rescaling: the running max only moves (and O, l are rescaled)
    // when some row's max grows by more than 2^8; otherwise the stale max is
    // kept, probabilities stay <= 256, and the final O / l is unchanged.
    const float m_tile = smax * qscale;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // rows with nothing visible yet
    float psum = 0.f;
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 pb[4];
    // P for one 32-key block: exponentials, row sums, bf16 operands.
    auto make_p = [&](int kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[kb][r], qscale, -m_use));
        const float p1 = fast_exp2(fmaf(s[kb][r + 1], qscale, -m_use));
        const bf16x2 pk = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
        if constexpr (kExactSum) psum += p0 + p1;
        else psum = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes, psum, false);
        pb[kb * 2 + (r >> 3)][r & 7] = pk[0];
        pb[kb * 2 + (r >> 3)][(r & 7) + 1] = pk[1];
      }
    };
    // O^T += V^T P^T for one 16-key step.
    auto pv = [&](int st) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            vl + ((st * 2 + h) * DV + vswz(n * 32 + col)) * 16));
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[n], 0, 0, 0);
      }
    };
    // Software overlap inside the tile: the matrix products of keys 0-31
    // run while the VALU computes P for keys 32-63, and those of keys 32-63
    // while it rearranges the next tile into LDS.
    make_p(0);
    pv(0);
    pv(1);
    make_p(1);
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
    psum += __shfl_xor(psum, 32);
    l_run += psum;
    pv(2);
    pv(3);
    store_tile(stage ^ 1);  // the last tile stores a clamped copy no one reads
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
    }
    __syncthreads();
  }

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

template <int DK, int DV, bool kExact>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  const int n_qtiles = (a.t_new + kPfRows - 1) / kPfRows;
  dim3 grid(n_qtiles * a.n_q * a.n_split, a.batch);
  const size_t lds = PfLds<DK, DV>::kTotal;
  if (lds > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&prefill_kernel<DK, DV, kExact>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((prefill_kernel<DK, DV, kExact>), grid, dim3(256), lds, a.stream,
                     (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                     a.ctx_len, (bf16*)a.out, a.lse, a.n_q, a.n_k, a.n_v, a.t_new, a.l_cap,
                     n_qtiles, a.scale * kLog2e, a.n_split, a.part_o, a.part_ml);
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
