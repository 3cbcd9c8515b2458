// Split-KV decode attention with asymmetric K / V heads, and the exact
// log-sum-exp combine of its per-chunk partial results.
//
// Computes, for every sequence b and query head i (Sigma architecture page,
// section 3.4 Steps 3-5; FlexHeadFA section for the split/combine structure):
//   s_j = scale * q_i . K[floor(i n_k / n_q)][j],     j < ctx_len[b]
//   o_i = sum_j softmax(s)_j V[floor(i n_v / n_q)][j]
//
// Split kernel: one wavefront per (sequence, query head -- or pair of query
// heads that share their K and V heads --, context chunk); a workgroup holds
// four consecutive waves of one chunk, so when n_q / n_k >= 4 its waves read
// the same K rows (the first wave to touch a row brings it from HBM, the
// others hit the CU's L1 / the XCD's L2).  Each wave walks its chunk in tiles
// of 64 rows:
//   * all V loads of the tile are issued at once (16-byte lane loads, 1 KiB
//     contiguous per wave instruction), K either with them or one tile
//     ahead, during the previous tile's V work (bf16 contiguous caches with
//     d_k <= 64 or chunks of at most 1024 rows; see the launcher);
//   * scores: each lane multiplies its 16-byte slice of a K row with the
//     matching slice of q (bf16: packed two-element dot products), DPP sums
//     over the lanes of a row; each lane keeps the score of exactly one row
//     of the tile;
//   * online softmax over tiles (running max m, running sum l, rescaled
//     accumulator) with base-2 exponentials, log2(e) folded into the query
//     scale; m moves only when a score passes it by more than 8 (log2
//     units), so most tiles skip the wave max, and l is summed per lane and
//     reduced once per chunk;
//   * V rows are accumulated in fp32 with each lane owning a 16-byte column
//     slice; the row's probability arrives by ds_bpermute from the lane that
//     owns it (bf16: two rows per step, their probabilities packed as a bf16
//     pair and each column's two values paired by v_perm, then one packed
//     dot product per column).
// The chunk's (m, l, acc[d_v]) goes to the workspace.
//
// Combine kernel: one workgroup per (query head, sequence, 16 value columns)
// merges the chunks
//   M = max_c m_c, w_c = 2^(m_c - M), Lambda = sum_c w_c l_c,
//   o = sum_c w_c acc_c / Lambda, lse = (M + log2 Lambda) ln 2,
// which is exact in real arithmetic.  Chunks past the sequence's length never
// enter the sums.

#include "device_common.h"
#include "launch.h"

namespace dqkv {

constexpr int kTile = 64;  // rows per wave iteration: one score per lane

// H = query heads per wave.  With H = 2 the wave takes two consecutive query
// heads that share one K head and one V head (n_q = 2 n_v): each K and V row
// it loads serves both, halving the per-CU load traffic of such layouts.
//
// PAGED: kc / vc are page pools and row j of sequence b sits in page
// pm.table[b][j / page_rows] (see PageMap).  Pages hold a multiple of 64 rows
// and chunks start at multiples of 64, so a 64-row tile never straddles two
// pages: one table entry per tile, read one tile ahead.
template <typename T, int DK, int DV, int H, bool PAGED, bool NEXT_K>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T* __restrict__ q, const T* kc, const T* vc,
    const int32_t* __restrict__ ctx_len, float* __restrict__ part_ml,
    float* __restrict__ part_acc, int n_q, int n_k, int n_v, int l_cap,
    int max_ctx, int S, int C, float qscale, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* kc_w, T* vc_w, PageMap pm) {
  // kc / kc_w (and vc / vc_w) are the same cache: the kernel reads rows
  // other than the appended one through the first and writes only that row
  // through the second.
  constexpr int EPL = Elem<T>::kPer16;       // elements per 16-byte lane load
  constexpr int LPR_K = DK / EPL;            // lanes per K row
  constexpr int RPL_K = 64 / LPR_K;          // K rows per wave load
  constexpr int NK = kTile / RPL_K;          // K wave loads per tile (= LPR_K)
  constexpr int LPR_V = DV / EPL;            // lanes per V row
  constexpr int RPL_V = 64 / LPR_V;          // V rows per wave load
  constexpr int NV = kTile / RPL_V;          // V wave loads per tile
  constexpr int VB = NV < 16 ? NV : 16;      // V loads held in registers at once
  static_assert(LPR_K >= 1 && LPR_K <= 32 && LPR_V >= 1 && LPR_V <= 64, "head dim");
  // bf16: scores and the V accumulation use packed two-element dot products
  // (v_dot2_f32_bf16, fp32 accumulation), the latter over pairs of rows
  // RPL_V apart, with the probabilities rounded to bf16.
  constexpr bool kDot = sizeof(T) == 2;
  static_assert(VB % 2 == 0, "V loads are consumed in pairs");

  const int c = blockIdx.x, quad = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = (quad * 4 + wave) * H;   // this wave's first query head
  if (i0 >= n_q) return;
  const int L_raw = ctx_len[b];
  const int L = max(0, min(L_raw, min(max_ctx, l_cap)));
  const int j0 = c * S;
  if (j0 >= L) return;
  const int rows = min(S, L - j0);
  const int hk = (i0 * n_k) / n_q;        // shared by the wave's H heads
  const int hv = (i0 * n_v) / n_q;

  // This lane's slice of q for each head: fp32 scaled by scale * log2 e, or
  // for bf16 the raw pairs (the scale is applied to the finished dot).
  const int kl = lane % LPR_K, kr = lane / LPR_K;
  float qf[H][EPL];
  u32x4 qp[H];
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
    qp[hh] = load16(q + ((size_t)b * n_q + i0 + hh) * DK + kl * EPL);
    if constexpr (!kDot) {
      Elem<T>::unpack(qp[hh], qf[hh]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[hh][e] *= qscale;
    }
  }

  const int vl = lane % LPR_V, vr = lane / LPR_V;
  // Page of the tile at chunk row t0: the raw table entry, and the entry
  // clamped into [0, num_pages) that reads use.
  auto page_raw = [&](int t0) -> int {
    return pm.table[(size_t)b * pm.max_blocks + ((j0 + t0) >> pm.page_shift)];
  };
  auto page_of = [&](int t0) -> size_t {
    return (size_t)min(max(page_raw(t0), 0), pm.num_pages - 1);
  };
  // Address of row 0 of the 64-row tile that starts at chunk row t0 (this
  // lane's slice of it), for K and for V.
  auto k_tile = [&](auto* base, int t0, size_t page) {
    if constexpr (PAGED)
      return base + ((page * n_k + hk) * ((size_t)1 << pm.page_shift) +
                     ((j0 + t0) & ((1 << pm.page_shift) - 1))) * DK + kl * EPL;
    return base + (((size_t)b * n_k + hk) * l_cap + j0 + t0) * DK + kl * EPL;
  };
  auto v_tile = [&](auto* base, int t0, size_t page) {
    if constexpr (PAGED)
      return base + ((page * n_v + hv) * ((size_t)1 << pm.page_shift) +
                     ((j0 + t0) & ((1 << pm.page_shift) - 1))) * DV + vl * EPL;
    return base + (((size_t)b * n_v + hv) * l_cap + j0 + t0) * DV + vl * EPL;
  };

  // Fused append: the sequence's newest row (L - 1) is the last row of the
  // chunk that owns it.  Every wave of that chunk stores the row of its own K
  // head and V head into the cache (waves sharing a head store identical
  // bytes) and then reads it back like any other row.  The lanes that store
  // a 16-byte slice are exactly the lanes that later load it (the row's lane
  // group in the K and V load patterns), so each lane reads back its own
  // store: program order, with kc / kc_w and vc / vc_w possibly aliasing as
  // far as the compiler knows.  Only this chunk touches row L - 1.
  // Nothing is stored when the length lies outside [1, min(max_ctx, l_cap)]
  // (it is clamped for reading, and row L - 1 then holds history that must
  // survive) or, paged, when the row's table entry names no page: such rows
  // are skipped, as kv_append skips them.
  if (k_new != nullptr && L_raw == L && L - 1 - j0 < rows) {
    const int r_new = L - 1 - j0;
    const int t_new0 = r_new & ~63;  // tile holding the new row
    const int blk = PAGED ? page_raw(t_new0) : 0;
    if (!PAGED || (blk >= 0 && blk < pm.num_pages)) {
      const size_t pg = (size_t)blk;
      const int in_tile = r_new - t_new0;
      if (kr == in_tile % RPL_K)
        *reinterpret_cast<u32x4*>(k_tile(kc_w, t_new0, pg) + (size_t)in_tile * DK) =
            load16(k_new + ((size_t)b * n_k + hk) * DK + kl * EPL);
      if (vr == in_tile % RPL_V)
        *reinterpret_cast<u32x4*>(v_tile(vc_w, t_new0, pg) + (size_t)in_tile * DV) =
            load16(v_new + ((size_t)b * n_v + hv) * DV + vl * EPL);
    }
  }

  // The lane keeps the score of tile row my_row = kl * RPL_K + kr (K load kl,
  // row kr of that load); row r's score therefore sits in lane
  // (r % RPL_K) * LPR_K + r / RPL_K.
  const int my_row = kl * RPL_K + kr;

  float m_run[H], l_run[H], acc[H][EPL];
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }

  // r: row within the chunk; kt / vt: the tile's row-0 addresses.  Loads of
  // the chunk's last tile: rows past the chunk's end read as zeros.  Every
  // other tile takes plain loads at constant offsets from the tile's address.
  auto load_k = [&](int r, const T* kt, int t0) -> u32x4 {
    if (r >= rows) return u32x4{0u, 0u, 0u, 0u};
    return load16(kt + (size_t)(r - t0) * DK);
  };
  auto load_v = [&](int r, const T* vt, int t0) -> u32x4 {
    if (r >= rows) return u32x4{0u, 0u, 0u, 0u};
    return load16_nt(vt + (size_t)(r - t0) * DV);
  };
  size_t page_next = PAGED ? page_of(0) : 0;

  // One tile of 64 rows per iteration: its V loads go out at the top and the
  // scores use K rows requested earlier.  With NEXT_K (bf16 contiguous
  // caches, chosen by the launcher) the next tile's K rows are requested
  // right after this tile's scores, while the softmax and the V products run;
  // otherwise K goes out together with V (paged caches read the tile's page
  // one tile ahead).  (Keeping a whole second tile in flight -- double
  // buffers, or re-filling each register right after use -- measured slower:
  // more bytes in flight per wave lower the achieved HBM rate here.)
  static_assert(!NEXT_K || (!PAGED && kDot), "K look-ahead: bf16, contiguous");
  constexpr bool kNextK = NEXT_K;
  u32x4 kv[NK];
  auto issue_k = [&](int t0, const T* kt) {
    if (t0 + kTile <= rows) {
#pragma unroll
      for (int u = 0; u < NK; ++u) kv[u] = load16(kt + (size_t)(u * RPL_K + kr) * DK);
    } else {
#pragma unroll
      for (int u = 0; u < NK; ++u) kv[u] = load_k(t0 + u * RPL_K + kr, kt, t0);
    }
  };
  if constexpr (kNextK) issue_k(0, k_tile(kc, 0, 0));
  // Per-lane row sums: the wave sum is taken once, after the last tile.
  float l_lane[H];
#pragma unroll
  for (int hh = 0; hh < H; ++hh) l_lane[hh] = 0.f;

  for (int t0 = 0; t0 < rows; t0 += kTile) {
    const size_t page = page_next;
    if constexpr (PAGED) page_next = t0 + kTile < rows ? page_of(t0 + kTile) : 0;
    const T* kt = k_tile(kc, t0, page);
    const T* vt = v_tile(vc, t0, page);
    u32x4 vv[VB];
    if constexpr (!kNextK) issue_k(t0, kt);
    if (t0 + kTile <= rows) {
#pragma unroll
      for (int u = 0; u < VB; ++u) vv[u] = load16_nt(vt + (size_t)(u * RPL_V + vr) * DV);
    } else {
#pragma unroll
      for (int u = 0; u < VB; ++u) vv[u] = load_v(t0 + u * RPL_V + vr, vt, t0);
    }
    // Every load of the tile is issued before any arithmetic: left alone, the
    // scheduler sinks each K load to its dot product and waits for it there.
    __builtin_amdgcn_sched_barrier(0);

    // Scores (one row per lane per head) and the online-softmax update.
    float s_mine[H];
#pragma unroll
    for (int hh = 0; hh < H; ++hh) s_mine[hh] = 0.f;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      float kf[EPL];
      if constexpr (!kDot) Elem<T>::unpack(kv[u], kf);
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        float s = 0.f;
        if constexpr (kDot) {
#pragma unroll
          for (int w = 0; w < 4; ++w) s = dot2_bf16(kv[u][w], qp[hh][w], s);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s = fmaf(qf[hh][e], kf[e], s);
        }
        s = group_sum<LPR_K>(s);
        s_mine[hh] = (u == kl) ? s : s_mine[hh];
      }
    }
    if constexpr (kNextK) {
      if (t0 + kTile < rows) issue_k(t0 + kTile, k_tile(kc, t0 + kTile, 0));
    }
    if constexpr (kDot) {
#pragma unroll
      for (int hh = 0; hh < H; ++hh) s_mine[hh] *= qscale;
    }
    // Online softmax with a lazily moved reference: the running max m_run is
    // raised (and l, acc rescaled) only when some score of the tile exceeds
    // it by more than 8 in log2 units, so the weights 2^(s - m_run) stay
    // below 2^8 and most tiles need no wave reduction.  The partial's m is
    // then at most 8 below the chunk's true max; the combine's merge is exact
    // for any such reference.  The first tile always sets it (m_run = -inf).
    float p[H];
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      if (t0 + my_row >= rows) s_mine[hh] = -INFINITY;
      if (__any(s_mine[hh] > m_run[hh] + 8.f)) {
        const float m_new = fmaxf(m_run[hh], wave_max(s_mine[hh]));
        const float alpha = fast_exp2(m_run[hh] - m_new);
        l_lane[hh] *= alpha;
        m_run[hh] = m_new;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
      }
      p[hh] = fast_exp2(s_mine[hh] - m_run[hh]);
      l_lane[hh] += p[hh];
    }

    // bf16: pack this lane's probability with that of row my_row ^ RPL_V
    // (row my_row + RPL_V where my_row % (2 RPL_V) < RPL_V, the only lanes
    // whose pair is used).
    uint32_t pp[H];
    if constexpr (kDot) {
      const int partner = my_row ^ RPL_V;
      const int psrc = (partner % RPL_K) * LPR_K + partner / RPL_K;
#pragma unroll
      for (int hh = 0; hh < H; ++hh) pp[hh] = pack_bf16x2(p[hh], __shfl(p[hh], psrc));
    }

    // acc_h += p_h(row) * V_row for every head of the wave.
#pragma unroll
    for (int vb = 0; vb < NV; vb += VB) {
      if (vb > 0) {  // only for fp32 with wide V rows: next batch of loads
#pragma unroll
        for (int u = 0; u < VB; ++u) vv[u] = load_v(t0 + (vb + u) * RPL_V + vr, vt, t0);
      }
      if constexpr (kDot) {
        // Loads u and u + 1 hold rows r and r + RPL_V of the same columns;
        // the lane owning row r holds (p[r], p[r + RPL_V]) packed in pp.
#pragma unroll
        for (int u = 0; u < VB; u += 2) {
          const int r = (vb + u) * RPL_V + vr;
          const int src = (r % RPL_K) * LPR_K + r / RPL_K;
          uint32_t pr[H];
#pragma unroll
          for (int hh = 0; hh < H; ++hh) pr[hh] = (uint32_t)__shfl((int)pp[hh], src);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = __builtin_amdgcn_perm(vv[u + 1][w], vv[u][w], 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(vv[u + 1][w], vv[u][w], 0x07060302u);
#pragma unroll
            for (int hh = 0; hh < H; ++hh) {
              acc[hh][2 * w] = dot2_bf16(lo, pr[hh], acc[hh][2 * w]);
              acc[hh][2 * w + 1] = dot2_bf16(hi, pr[hh], acc[hh][2 * w + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const int r = (vb + u) * RPL_V + vr;  // row within the tile
          const int src = (r % RPL_K) * LPR_K + r / RPL_K;
          float vf[EPL];
          Elem<T>::unpack(vv[u], vf);
#pragma unroll
          for (int hh = 0; hh < H; ++hh) {
            const float pr = __shfl(p[hh], src);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
          }
        }
      }
    }
  }

  // Sum the row groups of the wave (lanes with equal vl) and write each
  // head's partial.
#pragma unroll
  for (int hh = 0; hh < H; ++hh) l_run[hh] = wave_sum(l_lane[hh]);
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
#pragma unroll
    for (int off = LPR_V; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], off);
    }
    const size_t pidx = ((size_t)b * n_q + i0 + hh) * C + c;
    if (vr == 0) {
      f32x4* dst = reinterpret_cast<f32x4*>(part_acc + pidx * DV + vl * EPL);
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        dst[e / 4] = f32x4{acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]};
    }
    if (lane == 0) {
      part_ml[2 * pidx] = m_run[hh];
      part_ml[2 * pidx + 1] = l_run[hh];
    }
  }
}

constexpr int kCombineThreads = 256;
// Value columns per combine workgroup: 16 (32k step 29.27 against 29.04 us
// at 32 columns, 29.68 at 64; 8 as 16).
constexpr int kCombineCols = 16;

// One workgroup per (query head, sequence, 16-column slice of d_v).  The
// partial slots are requested together with the sequence length (all C
// slots of the head exist in the workspace; those past the sequence's
// chunk count are loaded but never used), so the merge costs one memory
// round trip.  Each thread merges its own partials around its local max;
// after one barrier wave 0 merges the threads' results with the same
// rescaling, lane shuffles doing the cross-thread steps.
template <typename T, int DV>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_acc,
    const int32_t* __restrict__ ctx_len, T* __restrict__ out,
    float* __restrict__ lse, int n_q, int l_cap, int max_ctx, int S, int C) {
  constexpr int COLS = DV < kCombineCols ? DV : kCombineCols;
  constexpr int LPR = COLS / 4;               // lanes per partial row slice (float4)
  constexpr int CPP = kCombineThreads / LPR;  // partials per pass
  constexpr int G = 64 / LPR;                 // partial groups per wave-0 lane column
  constexpr int U = 4;                        // passes loaded up front
  static_assert(CPP % G == 0, "combine shape");
  __shared__ f32x4 part[CPP][LPR];
  __shared__ float pm[CPP], pl[CPP];

  const int i = blockIdx.x, b = blockIdx.y, slice = blockIdx.z;
  const int tid = threadIdx.x;
  const int cl = tid % LPR, cr = tid / LPR;
  const size_t base = ((size_t)b * n_q + i) * C;
  const float* src = part_acc + base * DV + slice * COLS + cl * 4;

  const int L_raw = ctx_len[b];
  f32x4 a[U];
  float mc[U], lc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = cr + u * CPP;
    if (c < C) {
      a[u] = *reinterpret_cast<const f32x4*>(src + (size_t)c * DV);
      mc[u] = part_ml[2 * (base + c)];
      lc[u] = part_ml[2 * (base + c) + 1];
    }
  }
  const int L = max(0, min(L_raw, min(max_ctx, l_cap)));
  const int nc = min(C, (L + S - 1) / S);

  // This thread's partials c = cr, cr + CPP, ... below nc.
  float m_t = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (cr + u * CPP < nc) m_t = fmaxf(m_t, mc[u]);
  for (int c = cr + U * CPP; c < nc; c += CPP) m_t = fmaxf(m_t, part_ml[2 * (base + c)]);
  float l_t = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (cr + u * CPP < nc) {
      const float w = fast_exp2(mc[u] - m_t);
      l_t += w * lc[u];
      o += w * a[u];
    }
  }
  for (int c = cr + U * CPP; c < nc; c += CPP) {
    const float w = fast_exp2(part_ml[2 * (base + c)] - m_t);
    l_t += w * part_ml[2 * (base + c) + 1];
    o += w * *reinterpret_cast<const f32x4*>(src + (size_t)c * DV);
  }
  part[cr][cl] = o;
  if (cl == 0) {
    pm[cr] = m_t;
    pl[cr] = l_t;
  }
  __syncthreads();
  if (tid >= 64) return;

  // Wave 0: lane = g * LPR + col; group g takes thread rows g, g + G, ...
  const int col = tid % LPR, g = tid / LPR;
  float M = -INFINITY;
#pragma unroll
  for (int k = g; k < CPP; k += G) M = fmaxf(M, pm[k]);
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
  float lam = 0.f;
#pragma unroll
  for (int k = g; k < CPP; k += G) {
    const float mk = pm[k];
    if (mk > -INFINITY) {  // rows with no partial hold (-inf, 0, 0)
      const float w = fast_exp2(mk - M);
      t += w * part[k][col];
      lam += w * pl[k];
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    t.x += __shfl_xor(t.x, off);
    t.y += __shfl_xor(t.y, off);
    t.z += __shfl_xor(t.z, off);
    t.w += __shfl_xor(t.w, off);
    lam += __shfl_xor(lam, off);
  }
  if (g == 0) {
    const float inv = nc > 0 ? 1.f / lam : 0.f;
    T* dst = out + ((size_t)b * n_q + i) * DV + slice * COLS + col * 4;
    dst[0] = Elem<T>::from_f32(t.x * inv);
    dst[1] = Elem<T>::from_f32(t.y * inv);
    dst[2] = Elem<T>::from_f32(t.z * inv);
    dst[3] = Elem<T>::from_f32(t.w * inv);
  }
  if (tid == 0 && slice == 0 && lse != nullptr)
    lse[(size_t)b * n_q + i] = nc > 0 ? (M + fast_log2(lam)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ launch

// Query heads per wave: two when consecutive pairs of query heads share both
// their K head and their V head (n_q = 2 n_v and n_q / n_k even).
static int heads_per_wave(const DecodeArgs& a) {
  return (a.n_q == 2 * a.n_v && (a.n_q / a.n_k) % 2 == 0) ? 2 : 1;
}

template <typename T, int DK, int DV, int H, bool PAGED, bool NEXT_K = false>
static void launch_split_hp(const DecodeArgs& a) {
  dim3 grid(a.C, (a.n_q + 4 * H - 1) / (4 * H), a.batch);
  hipLaunchKernelGGL((decode_split_kernel<T, DK, DV, H, PAGED, NEXT_K>), grid, dim3(256), 0,
                     a.stream,
                     (const T*)a.q, (const T*)a.k_cache, (const T*)a.v_cache, a.ctx_len,
                     a.part_ml, a.part_acc, a.n_q, a.n_k, a.n_v, a.l_cap, a.max_ctx, a.S, a.C,
                     a.scale * kLog2e, (const T*)a.k_new, (const T*)a.v_new, (T*)a.k_cache,
                     (T*)a.v_cache, a.pages);
}

// Contiguous bf16 caches with the K look-ahead (same-process A/B, µs per
// step, without -> with): at d_k <= 64 always (32k 28.9 -> 28.2, 16 ragged
// sequences 235.2 -> 233.9; 4 x 64k 181.0 -> 175.6 against the form without
// it -- 174.5 before the lazy reference), at larger d_k for chunks of up to
// 1024 rows (32k symmetric d = 128: 50.3 -> 48.3) but not for longer ones
// (4 x 64k, d_k = 128: 198.3 against 202.4; symmetric 64k alike).
template <typename T, int DK, int DV, int H>
static void launch_split_contig(const DecodeArgs& a) {
  if constexpr (sizeof(T) == 2 && DK <= 64) {
    launch_split_hp<T, DK, DV, H, false, true>(a);
  } else if constexpr (sizeof(T) == 2) {
    if (a.S <= 1024) launch_split_hp<T, DK, DV, H, false, true>(a);
    else launch_split_hp<T, DK, DV, H, false>(a);
  } else {
    launch_split_hp<T, DK, DV, H, false>(a);
  }
}

template <typename T, int DK, int DV>
static hipError_t launch_split_t(const DecodeArgs& a) {
  const bool paged = a.pages.table != nullptr;
  if (heads_per_wave(a) == 2) {
    if (paged) launch_split_hp<T, DK, DV, 2, true>(a);
    else launch_split_contig<T, DK, DV, 2>(a);
  } else {
    if (paged) launch_split_hp<T, DK, DV, 1, true>(a);
    else launch_split_contig<T, DK, DV, 1>(a);
  }
  return hipGetLastError();
}

template <typename T, int DV>
static hipError_t launch_combine_t(const DecodeArgs& a) {
  constexpr int COLS = DV < kCombineCols ? DV : kCombineCols;
  dim3 grid(a.n_q, a.batch, DV / COLS);
  hipLaunchKernelGGL((decode_combine_kernel<T, DV>), grid, dim3(kCombineThreads), 0, a.stream,
                     a.part_ml, a.part_acc, a.ctx_len, (T*)a.out, a.lse, a.n_q, a.l_cap,
                     a.max_ctx, a.S, a.C);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t split_dv(const DecodeArgs& a) {
  switch (a.d_v) {
    case 32: return launch_split_t<T, DK, 32>(a);
    case 64: return launch_split_t<T, DK, 64>(a);
    case 128: return launch_split_t<T, DK, 128>(a);
    case 256: return launch_split_t<T, DK, 256>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t split_dk(const DecodeArgs& a) {
  switch (a.d_k) {
    case 32: return split_dv<T, 32>(a);
    case 64: return split_dv<T, 64>(a);
    case 128: return split_dv<T, 128>(a);
    case 256:
      if constexpr (sizeof(T) == 2) return split_dv<T, 256>(a);
      break;
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t combine_dv(const DecodeArgs& a) {
  switch (a.d_v) {
    case 32: return launch_combine_t<T, 32>(a);
    case 64: return launch_combine_t<T, 64>(a);
    case 128: return launch_combine_t<T, 128>(a);
    case 256: return launch_combine_t<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_split(const DecodeArgs& a) {
  return a.bf16 ? split_dk<bf16>(a) : split_dk<float>(a);
}

hipError_t launch_decode_combine(const DecodeArgs& a) {
  return a.bf16 ? combine_dv<bf16>(a) : combine_dv<float>(a);
}

}  // namespace dqkv
