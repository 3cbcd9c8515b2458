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
//   P^T          = 2^(S^T * scale * log2 e - m), online max / sum per lane,
//                  the two lane halves of a query row joined by one shuffle
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

// Position of value column d inside a 16-key step of the V tile.  The XOR
// of its low three bits with bits 3-5 keeps each group of 8 columns in place
// (reads stay conflict-free) while the cooperative stores, whose lanes are 8
// columns apart, spread over the LDS banks.
__device__ __forceinline__ int vswz(int d) { return d ^ ((d >> 3) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void prefill_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, bf16* __restrict__ out, float* __restrict__ lse,
    int n_q, int n_k, int n_v, int t_new, int l_cap, int n_qtiles, float qscale) {
  using Lds = PfLds<DK, DV>;
  constexpr int KS = DK / 16;       // 16-wide d_k steps of S^T
  constexpr int NB = DV / 32;       // 32-wide d_v blocks of O^T
  constexpr int K16 = DK / 8;       // 16-byte chunks per K row
  constexpr int KCH = kPfKeys * K16 / 256;  // K chunks per thread per tile
  constexpr int VD8 = DV / 8;       // 8-column chunks per V row
  static_assert(KCH >= 1, "K tile");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  // Renumber workgroups: linear id -> (head, q-tile) so that consecutive
  // logical tiles land on one XCD (dispatch is round-robin over 8 XCDs).
  const int nwg = gridDim.x;
  const int id = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (id % 8) * (nwg / 8) + id / 8 : id;
  const int i = logical / n_qtiles;   // query head
  const int qt = logical % n_qtiles;  // query tile
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
  const int n_tiles = (n_keys + kPfKeys - 1) / kPfKeys;

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
  const bool v_act = v_kq < kPfKeys / 4;
  u32x4 kreg[KCH];
  u32x4 vreg[4];

  auto load_tile = [&](int t) {
    const int j0 = t * kPfKeys;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int e = tid + c * 256;
      const int key = e / K16, ch = e % K16;
      const int j = j0 + key;
      kreg[c] = j < n_keys ? load16(kbase + (size_t)j * DK + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (v_act) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = j0 + v_kq * 4 + k;
        vreg[k] = j < n_keys ? load16(vbase + (size_t)j * DV + v_dc * 8) : u32x4{0u, 0u, 0u, 0u};
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
        uint2* p0 = reinterpret_cast<uint2*>(vl + ((s * DV + vswz(d0)) * 2 + hh) * 16 + off);
        uint2* p1 = reinterpret_cast<uint2*>(vl + ((s * DV + vswz(d0 + 1)) * 2 + hh) * 16 + off);
        *p0 = make_uint2(lo01, lo23);
        *p1 = make_uint2(hi01, hi23);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x16{};

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
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

    // Causal mask: key j is visible to this row iff j <= p_q.
    const bool diag = j0 + kPfKeys - 1 > base + r0 + wave * kPfRowsPerWave;
    float smax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r];
        if (diag) {
          const int j = j0 + kb * 32 + (r >> 2) * 8 + 4 * h + (r & 3);
          x = j <= p_q ? x : -INFINITY;
          s[kb][r] = x;
        }
        smax = fmaxf(smax, x);
      }
    }
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    const float m_new = fmaxf(m_run, smax * qscale);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // rows with nothing visible yet
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], qscale, -m_use));
        psum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NB; ++n) o[n] *= alpha;

    // O^T += V^T P^T over four 16-key steps.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            vl + ((st * DV + vswz(n * 32 + col)) * 2 + h) * 16));
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[n], 0, 0, 0);
      }
    }

    if (t + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Normalise and store this lane's query row (rows 8*(r/4)+4h+r%4 of each
  // 32-column block of O^T are value columns).
  if (q_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16* op = out + (((size_t)b * t_new + rq) * n_q + i) * DV;
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
      lse[((size_t)b * t_new + rq) * n_q + i] =
          l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
  }
}

template <int DK, int DV>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  const int n_qtiles = (a.t_new + kPfRows - 1) / kPfRows;
  dim3 grid(n_qtiles * a.n_q, a.batch);
  const size_t lds = PfLds<DK, DV>::kTotal;
  if (lds > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&prefill_kernel<DK, DV>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((prefill_kernel<DK, DV>), grid, dim3(256), lds, a.stream,
                     (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                     a.ctx_len, (bf16*)a.out, a.lse, a.n_q, a.n_k, a.n_v, a.t_new, a.l_cap,
                     n_qtiles, a.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_prefill_t<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_prefill_t<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_prefill_t<128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return launch_prefill_t<128, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace dqkv
