// Selective V fetching for decode (Sigma architecture page, section
// "Selective V Cache Fetching"): the attention weights alpha_i of every query
// head are computed over the whole K cache, but only the V rows of the top_k
// largest weights are read, and the output is their alpha-weighted sum
//   o_i ~= sum_{j in TopK(alpha_i)} alpha_ij V[floor(i n_v / n_q)][j]
// with alpha the full softmax (no renormalisation over the selected rows).
// Equal weights are ordered by row index, lower first.
//
// Three kernels, each one pass:
//   1. score:  s_ij = (scale log2 e) q_i . K_j for every visible row, written
//              to the workspace (fp32, base-2 logits).  A wave takes one
//              64-row tile of a K head and all the query heads that share it
//              (up to 16), so every K row is read once; bf16 products run on
//              the matrix cores, fp32 ones on the vector ALUs.
//   2. local:  per (query head, range of 2048 or 4096 rows): the range's max and
//              sum of 2^(s - max), and its own top_k rows (a row in the
//              global top_k is in its range's top_k), kept in index order.
//   3. gather: per query head: merge the ranges' (max, sum) into the full
//              softmax normaliser, select the top_k among the candidates,
//              read only those V rows and sum them with their weights.
// Selection is an exact radix select on order-preserving 32-bit keys of the
// fp32 logits (three digit passes of 11, 11 and 10 bits over a 2048-bin LDS
// histogram) followed by an index-ordered compaction, so the chosen set is
// the top_k by (logit, -row index) in the kernel's fp32 logits.

#include "device_common.h"
#include "launch.h"

namespace dqkv {

constexpr int kSelThreads = 256;
constexpr int kBins = 2048;

// Monotone map from fp32 to uint32 (a < b  <=>  key(a) < key(b)); -0 and +0
// share the key of +0.  Logits here are always finite.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Row j of head h of sequence b: in a contiguous [B][H][l_cap][D] cache, or
// (pm.table set) in a page pool [num_pages][H][page_rows][D] through the
// page table, entries outside [0, num_pages) clamped.  A 64-row tile that
// starts at a multiple of 64 lies in one page, so rows j .. j + 63 follow
// the returned address contiguously.
template <typename T, int D>
__device__ __forceinline__ T* cache_row(T* c, const PageMap& pm, int b, int H, int h,
                                        int l_cap, int j) {
  if (pm.table != nullptr) {
    const int blk = pm.table[(size_t)b * pm.max_blocks + (j >> pm.page_shift)];
    const size_t page = (size_t)min(max(blk, 0), pm.num_pages - 1);
    return c + (((page * H + h) << pm.page_shift) + (j & ((1 << pm.page_shift) - 1))) * D;
  }
  return c + (((size_t)b * H + h) * l_cap + j) * D;
}

// Row j as a store destination: as cache_row, but a page-table entry outside
// [0, num_pages) gives nullptr and the row is not written (a read may clamp;
// a write there would land in another sequence's page).
template <typename T, int D>
__device__ __forceinline__ T* cache_row_store(T* c, const PageMap& pm, int b, int H, int h,
                                              int l_cap, int j) {
  if (pm.table != nullptr) {
    const int blk = pm.table[(size_t)b * pm.max_blocks + (j >> pm.page_shift)];
    if (blk < 0 || blk >= pm.num_pages) return nullptr;
  }
  return cache_row<T, D>(c, pm, b, H, h, l_cap, j);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive prefix sum of v over the NT threads of the block, in thread
// order; *total receives the block's sum.  Uses red[0 .. NT/64 - 1]; ends
// synchronised.
template <int NT = kSelThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = red[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

struct Threshold {
  uint32_t key;  // keys above it are taken (the k-th largest key, or one below a whole bin)
  int need_eq;   // rows with this key to take as well (the lowest-indexed ones)
};

// k-th largest of the n keys key(0..n-1), 1 <= k <= n, by radix select from
// the most significant digit.  Invariant before each pass: the keys that
// match the digits fixed so far number at least krem, and the keys above
// that prefix number k - krem.  A pass whose chosen bin holds exactly krem
// keys ends the search: every key with that prefix is taken, so the
// threshold is the prefix's lowest key minus one with no equal keys taken
// (the same set as the remaining passes would give).  NT threads; hist: kBins
// LDS words; red: 2 NT/64 LDS ints (the digit search uses red[NT/64 ..
// NT/64 + 2]).
template <int NT = kSelThreads, class KeyF>
__device__ Threshold block_select_threshold(KeyF key, int n, int k, uint32_t* hist, int* red) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int d = tid; d < kBins; d += NT) hist[d] = 0u;
    __syncthreads();
    for (int x = tid; x < n; x += NT) {
      const uint32_t kk = key(x);
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1u);
    }
    __syncthreads();
    // Thread t owns bins kBins-1-BPT t down to kBins-BPT-BPT t: bins in
    // descending order across the block, so the exclusive scan counts the
    // keys in higher bins.
    constexpr int BPT = kBins / NT;
    int cnt[BPT], own = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      cnt[e] = (int)hist[kBins - 1 - BPT * tid - e];
      own += cnt[e];
    }
    int total;
    const int above = block_exclusive_scan<NT>(own, red, &total);
    if (above < krem && krem <= above + own) {  // exactly one thread
      int run = above;
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        if (run + cnt[e] >= krem) {
          red[NW] = kBins - 1 - BPT * tid - e;
          red[NW + 1] = krem - run;
          red[NW + 2] = cnt[e] == krem - run;
          break;
        }
        run += cnt[e];
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)red[NW];
    krem = red[NW + 1];
    prefix |= digit << shift;
    pmask |= dmask << shift;
    if (red[NW + 2] != 0 && prefix != 0u) {  // the whole bin is taken
      __syncthreads();  // red[NW .. NW + 2] are rewritten by the next caller
      return Threshold{prefix - 1u, 0};
    }
  }
  __syncthreads();  // red[NW .. NW + 2] are rewritten by the next caller
  return Threshold{prefix, krem};
}

// Calls emit(pos, x) for the k selected positions x (key above the
// threshold, or equal to it and among the first need_eq such in index
// order), with pos = rank of x among the selected in index order.  Each of
// the NT/64 waves walks one contiguous segment of [0, n) in 64-element
// steps; red: 2 NT/64 ints.
template <int NT = kSelThreads, class KeyF, class EmitF>
__device__ void block_compact(KeyF key, int n, Threshold th, int* red, EmitF emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = ((n + NW * 64 - 1) / (NW * 64)) * 64;
  const int lo = min(n, wave * seg), hi = min(n, lo + seg);
  int gt = 0, eq = 0;
  for (int x0 = lo; x0 < hi; x0 += 64) {
    const int x = x0 + lane;
    const uint32_t kk = x < hi ? key(x) : 0u;
    gt += __popcll(__builtin_amdgcn_ballot_w64(x < hi && kk > th.key));
    eq += __popcll(__builtin_amdgcn_ballot_w64(x < hi && kk == th.key));
  }
  if (lane == 0) {
    red[wave] = gt;
    red[NW + wave] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += red[w];
    eq_before += red[NW + w];
  }
  __syncthreads();
  int pos0 = gt_before + min(eq_before, th.need_eq);
  const uint64_t below = lanes_below();
  for (int x0 = lo; x0 < hi; x0 += 64) {
    const int x = x0 + lane;
    const uint32_t kk = x < hi ? key(x) : 0u;
    const bool is_gt = x < hi && kk > th.key;
    const bool is_eq = x < hi && kk == th.key;
    const uint64_t emask = __builtin_amdgcn_ballot_w64(is_eq);
    const bool take = is_gt || (is_eq && eq_before + __popcll(emask & below) < th.need_eq);
    const uint64_t smask = __builtin_amdgcn_ballot_w64(take);
    if (take) emit(pos0 + __popcll(smask & below), x);
    pos0 += __popcll(smask);
    eq_before += __popcll(emask);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes within each row of 16 (lanes without a source add 0), then lane 15
// of each row added to the next row and lane 31 to rows 2 and 3.  All lanes
// must be active.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Register-resident variants for up to NT * E keys (NT threads): wave w,
// lane l holds elements w * 64 E + 64 e + l (e < E) in its registers, so
// each wave owns a contiguous segment and every load of a wave is 64
// consecutive elements.  One round of loads, then every pass works from
// registers.

template <int E>
__device__ __forceinline__ int reg_index(int e) {
  return (threadIdx.x >> 6) * 64 * E + 64 * e + (threadIdx.x & 63);
}

// hist: three kBins-word histograms (one per digit pass), zeroed and made
// visible by a barrier before the call; red: NT/64 ints, which other waves
// may still read when a wave returns (the caller syncs before rewriting
// them).  Two barriers per pass: after the histogram, and after the waves'
// bin totals; every wave then finds the digit itself from the totals and
// the bins of the wave that holds the krem-th key, so all waves take the
// same exits.  Ends early as the block variant.
template <int E, int NT = kSelThreads>
__device__ Threshold reg_select_threshold(const uint32_t (&key)[E], int n, int k,
                                          uint32_t* hist, int* red) {
  constexpr int NW = NT / 64, BPT = kBins / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    uint32_t* h = hist + pass * kBins;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (reg_index<E>(e) < n && (key[e] & pmask) == prefix)
        atomicAdd(&h[(key[e] >> shift) & dmask], 1u);
    __syncthreads();
    // Thread t owns bins kBins-1-BPT t down to kBins-BPT-BPT t (descending
    // across the block); a wave's total goes to red[wave].
    int own = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) own += (int)h[kBins - 1 - BPT * tid - e];
    own = wave_inclusive_scan(own);
    if (lane == 63) red[wave] = own;
    __syncthreads();
    int tot[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[w] = red[w];
    // The wave ws whose bins hold the krem-th key from the top, and the
    // keys in higher waves' bins.
    int ws = NW - 1, above = 0, run = 0;
    bool found = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const bool here = !found && run + tot[w] >= krem;
      ws = here ? w : ws;
      above = here ? run : above;
      found = found || here;
      run += tot[w];
    }
    // Lane l takes the bins of thread 64 ws + l.
    const int t2 = 64 * ws + lane;
    int cnt[BPT], mine = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      cnt[e] = (int)h[kBins - 1 - BPT * t2 - e];
      mine += cnt[e];
    }
    const int before = above + wave_inclusive_scan(mine) - mine;
    const bool holds = before < krem && krem <= before + mine;
    int digit = 0, kr = 0, whole = 0;
    if (holds) {
      int r = before;
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        if (r + cnt[e] >= krem) {
          digit = kBins - 1 - BPT * t2 - e;
          kr = krem - r;
          whole = cnt[e] == kr;
          break;
        }
        r += cnt[e];
      }
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(holds);
    const int src = bal != 0ull ? (int)__builtin_ctzll(bal) : 0;
    digit = __builtin_amdgcn_readlane(digit, src);
    kr = __builtin_amdgcn_readlane(kr, src);
    whole = __builtin_amdgcn_readlane(whole, src);
    prefix |= (uint32_t)digit << shift;
    pmask |= dmask << shift;
    krem = kr;
    if (whole != 0 && prefix != 0u) return Threshold{prefix - 1u, 0};  // whole bin taken
  }
  return Threshold{prefix, krem};
}

template <int NT = kSelThreads>
__device__ __forceinline__ void clear_hists(uint32_t* hist) {
  u32x4* h = reinterpret_cast<u32x4*>(hist);
  for (int x = threadIdx.x; x < 3 * kBins / 4; x += NT) h[x] = u32x4{0u, 0u, 0u, 0u};
}

// emit(pos, e) for every selected register slot e, pos = rank in index order
// (NT threads; red: 2 NT/64 ints not used by the threshold search that
// gave th, and not rewritten before the caller's next barrier).
template <int E, int NT = kSelThreads, class EmitF>
__device__ __forceinline__ void reg_compact(const uint32_t (&key)[E], int n, Threshold th,
                                            int* red, EmitF emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool ok = reg_index<E>(e) < n;
    gt += __popcll(__builtin_amdgcn_ballot_w64(ok && key[e] > th.key));
    eq += __popcll(__builtin_amdgcn_ballot_w64(ok && key[e] == th.key));
  }
  if (lane == 0) {
    red[wave] = gt;
    red[NW + wave] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += red[w];
    eq_before += red[NW + w];
  }
  int pos0 = gt_before + min(eq_before, th.need_eq);
  const uint64_t below = lanes_below();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool ok = reg_index<E>(e) < n;
    const bool is_gt = ok && key[e] > th.key;
    const bool is_eq = ok && key[e] == th.key;
    const uint64_t emask = __builtin_amdgcn_ballot_w64(is_eq);
    const bool take = is_gt || (is_eq && eq_before + __popcll(emask & below) < th.need_eq);
    const uint64_t smask = __builtin_amdgcn_ballot_w64(take);
    if (take) emit(pos0 + __popcll(smask & below), e);
    pos0 += __popcll(smask);
    eq_before += __popcll(emask);
  }
}


// ------------------------------------------------------------ 1. scores

// fp32 logits on the vector ALUs (fp32 caches).  One wave per 64-row tile
// and HW query heads that share one K head: each K row the wave loads serves
// all HW heads, and the four waves of a workgroup take different tiles, so
// all their loads are distinct.
template <typename T, int DK, int HW>
__global__ __launch_bounds__(256) void sel_score_kernel(
    const T* __restrict__ q, const T* kc, const int32_t* __restrict__ ctx_len,
    float* __restrict__ scores, int n_q, int n_k, int l_cap, int max_ctx, int ld_s, int S,
    float qscale, const T* __restrict__ k_new, T* kc_w, PageMap pm) {
  constexpr int EPL = Elem<T>::kPer16;
  constexpr int LPR_K = DK / EPL;   // lanes per K row
  constexpr int RPL_K = 64 / LPR_K; // K rows per wave load
  constexpr int NK = 64 / RPL_K;    // wave loads per 64-row tile
  static_assert(LPR_K >= 1 && LPR_K <= 32, "head dim");

  const int c = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = n_q / n_k, slices = G / HW;
  const int hk = blockIdx.y / slices, slice = blockIdx.y % slices;
  const int i0 = hk * G + slice * HW;
  const int L_raw = ctx_len[b];
  const int L = max(0, min(L_raw, min(max_ctx, l_cap)));
  const int j0 = c * S;
  if (j0 >= L) return;
  const int rows = min(S, L - j0);

  const int kl = lane % LPR_K, kr = lane / LPR_K;
  float qf[HW][EPL];
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    Elem<T>::unpack(load16(q + ((size_t)b * n_q + i0 + h) * DK + kl * EPL), qf[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= qscale;
  }

  // Fused append only for a length inside [1, min(max_ctx, l_cap)] (a longer
  // one is clamped for reading and row L - 1 keeps its history).
  const bool fused = k_new != nullptr && L_raw == L;
  const int r_new = fused ? L - 1 - j0 : -1;  // in [0, rows) iff this chunk owns it
  const T* kn = fused ? k_new + ((size_t)b * n_k + hk) * DK + kl * EPL : nullptr;
  if (fused && r_new < rows && slice == 0 && wave == (r_new / 64) % 4 && lane < LPR_K) {
    if (T* dst = cache_row_store<T, DK>(kc_w, pm, b, n_k, hk, l_cap, L - 1))
      *reinterpret_cast<u32x4*>(dst + kl * EPL) = load16(kn);
  }

  float* out = scores + ((size_t)b * n_q + i0) * ld_s + j0;
  const int my_row = kl * RPL_K + kr;
  for (int t0 = wave * 64; t0 < rows; t0 += 256) {
    const T* kt = cache_row<const T, DK>(kc, pm, b, n_k, hk, l_cap, j0 + t0) + kl * EPL;
    u32x4 kv[NK];
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int r = t0 + u * RPL_K + kr;
      kv[u] = r >= rows ? u32x4{0u, 0u, 0u, 0u}
                        : load16(r == r_new ? kn : kt + (size_t)(r - t0) * DK);
    }
    float s_mine[HW];
#pragma unroll
    for (int h = 0; h < HW; ++h) s_mine[h] = 0.f;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      float kf[EPL];
      Elem<T>::unpack(kv[u], kf);
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qf[h][e], kf[e], s);
        s = group_sum<LPR_K>(s);
        s_mine[h] = (u == kl) ? s : s_mine[h];
      }
    }
    if (t0 + my_row < rows) {
#pragma unroll
      for (int h = 0; h < HW; ++h) out[(size_t)h * ld_s + t0 + my_row] = s_mine[h];
    }
  }
}

typedef __bf16 sel_bf16x8 __attribute__((ext_vector_type(8)));

// bf16 logits on the matrix cores.  For each 16-row block of a 64-row tile,
// S^T[16 rows][16 heads] = K[16 rows][DK] . Q^T[DK][16 heads], in DK / 32
// v_mfma_f32_16x16x32_bf16 steps.  Operand layouts: A lane l = K row l % 16,
// elements 8 (l / 16) .. +7 of a 32-wide k block (one 16-byte load straight
// from memory); B lane l = query head l % 16, the same k elements; D lane l
// = head l % 16, rows 4 (l / 16) .. +3 of the block.  Up to 16 query heads
// that share the K head ride on one product; the four waves of a workgroup
// take different tiles.  The logits are the exact bf16 products summed in
// fp32 by the matrix core, then scaled by scale * log2 e.
template <int DK>
__global__ __launch_bounds__(256) void sel_score_mfma_kernel(
    const bf16* __restrict__ q, const bf16* kc, const int32_t* __restrict__ ctx_len,
    float* __restrict__ scores, int n_q, int n_k, int l_cap, int max_ctx, int ld_s, int S,
    float qscale, const bf16* __restrict__ k_new, bf16* kc_w, PageMap pm) {
  constexpr int KB = DK / 32;  // k blocks per row
  const int c = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = n_q / n_k, slices = (G + 15) / 16;
  const int hk = blockIdx.y / slices, slice = blockIdx.y % slices;
  const int h0 = slice * 16, nh = min(16, G - h0);
  const int i0 = hk * G + h0;
  const int L_raw = ctx_len[b];
  const int L = max(0, min(L_raw, min(max_ctx, l_cap)));
  const int j0 = c * S;
  if (j0 >= L) return;
  const int rows = min(S, L - j0);

  const int l16 = lane & 15, kg = lane >> 4;
  sel_bf16x8 qb[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qb[kb] = __builtin_bit_cast(
        sel_bf16x8, l16 < nh ? load16(q + ((size_t)b * n_q + i0 + l16) * DK + kb * 32 + 8 * kg)
                             : u32x4{0u, 0u, 0u, 0u});

  // Fused append only for a length inside [1, min(max_ctx, l_cap)].
  const bool fused = k_new != nullptr && L_raw == L;
  const int r_new = fused ? L - 1 - j0 : -1;  // in [0, rows) iff this chunk owns it
  const bf16* kn = fused ? k_new + ((size_t)b * n_k + hk) * DK + 8 * kg : nullptr;
  if (fused && r_new < rows && slice == 0 && wave == (r_new / 64) % 4 && lane < DK / 8) {
    if (bf16* dst = cache_row_store<bf16, DK>(kc_w, pm, b, n_k, hk, l_cap, L - 1))
      *reinterpret_cast<u32x4*>(dst + 8 * lane) =
          load16(k_new + ((size_t)b * n_k + hk) * DK + 8 * lane);
  }

  float* out = scores + ((size_t)b * n_q + i0 + l16) * ld_s + j0;
  for (int t0 = wave * 64; t0 < rows; t0 += 256) {
    const bf16* kt = cache_row<const bf16, DK>(kc, pm, b, n_k, hk, l_cap, j0 + t0) + 8 * kg;
    u32x4 kv[4][KB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = t0 + rb * 16 + l16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        kv[rb][kb] = r >= rows ? u32x4{0u, 0u, 0u, 0u}
                               : load16((r == r_new ? kn : kt + (size_t)(r - t0) * DK) + kb * 32);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sel_bf16x8, kv[rb][kb]),
                                                      qb[kb], acc, 0, 0, 0);
      const int r = t0 + rb * 16 + 4 * kg;
      if (l16 < nh) {
        if (r + 3 < rows) {
          *reinterpret_cast<f32x4*>(out + r) = acc * qscale;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r + e < rows) out[r + e] = acc[e] * qscale;
        }
      }
    }
  }
}

// ------------------------------------------------- 2. per-range selection

// One workgroup per (query head, range of RS rows); candidates of range rg
// are written at [rg * top_k, rg * top_k + min(top_k, rows)), so a head's
// candidate list is contiguous and in ascending row order.
template <int RS, int NT>
__global__ __launch_bounds__(NT) void sel_local_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_len,
    float* __restrict__ range_ml, float* __restrict__ cand_s, int32_t* __restrict__ cand_i,
    int n_q, int l_cap, int max_ctx, int ld_s, int n_ranges, int top_k) {
  constexpr int E = RS / NT;  // keys per thread
  constexpr int NW = NT / 64;
  __shared__ __align__(16) uint32_t hist[3 * kBins];
  __shared__ int red[4 * NW];
  __shared__ float wm[NW], wl[NW];
  const int rg = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int L = ctx_len[b];
  // The range's logits are requested together with the sequence length
  // (every one of the ld_s columns of the head's logit row exists; those at
  // or past the length are masked once it arrives), so the two loads cost
  // one memory round trip.
  const int j0 = rg * RS;
  const int avail = min(RS, ld_s - j0);
  const float* sc = scores + ((size_t)b * n_q + i) * ld_s + j0;
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = reg_index<E>(e);
    s[e] = x < avail ? sc[x] : -INFINITY;
  }
  L = max(0, min(L, min(max_ctx, l_cap)));
  if (j0 >= L) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no wave ends with loads in flight
    return;
  }
  const int rows = min(RS, L - j0);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (reg_index<E>(e) >= rows) s[e] = -INFINITY;
  clear_hists<NT>(hist);
  // The range's max and sum of 2^(s - max): per wave, then over the waves.
  float m = s[0];
#pragma unroll
  for (int e = 1; e < E; ++e) m = fmaxf(m, s[e]);
  m = wave_max(m);
  float l = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) l += reg_index<E>(e) < rows ? fast_exp2(s[e] - m) : 0.f;
  l = wave_sum(l);
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = l;
  }
  __syncthreads();
  const size_t slot = ((size_t)b * n_q + i) * n_ranges + rg;
  if (threadIdx.x == 0) {
    float M = wm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, wm[w]);
    float Z = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Z += wl[w] > 0.f ? wl[w] * fast_exp2(wm[w] - M) : 0.f;
    range_ml[2 * slot] = M;
    range_ml[2 * slot + 1] = Z;
  }

  float* cs = cand_s + slot * top_k;
  int32_t* ci = cand_i + slot * top_k;
  if (rows <= top_k) {  // the whole range is a candidate
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = reg_index<E>(e);
      if (x < rows) {
        cs[x] = s[e];
        ci[x] = j0 + x;
      }
    }
    return;
  }
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = order_key(s[e]);
  const Threshold th = reg_select_threshold<E, NT>(key, rows, top_k, hist, red);
  reg_compact<E, NT>(key, rows, th, red + 2 * NW, [&](int pos, int e) {
    if (pos < top_k) {
      cs[pos] = s[e];
      ci[pos] = j0 + reg_index<E>(e);
    }
  });
}

// ------------------------------------------ 3. final selection and gather

// E: candidate keys per thread held in registers (E * NT of them), NT threads.
template <typename T, int DV, int E, int NT>
__global__ __launch_bounds__(NT) void sel_gather_kernel(
    const T* vc, const int32_t* __restrict__ ctx_len, const float* __restrict__ range_ml,
    const float* __restrict__ cand_s, const int32_t* __restrict__ cand_i, T* __restrict__ out,
    float* __restrict__ lse, int32_t* __restrict__ sel_idx, int n_q, int n_v, int l_cap,
    int max_ctx, int n_ranges, int range_rows, int top_k, const T* __restrict__ v_new, T* vc_w,
    PageMap pm) {
  constexpr int EPL = Elem<T>::kPer16;
  constexpr int LPR = DV / EPL;               // lanes per V row
  constexpr int RPP = NT / LPR;               // V rows per pass of the block
  constexpr int U = 128 / RPP < 1 ? 1 : (128 / RPP > 8 ? 8 : 128 / RPP);  // passes in flight
  __shared__ __align__(16) uint32_t hist[3 * kBins];
  __shared__ int red[4 * (NT / 64)];
  __shared__ int32_t sel_j[kMaxTopK];
  __shared__ float sel_w[kMaxTopK];
  __shared__ float part[RPP][DV + 4];

  const int i = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int L_raw = ctx_len[b];
  int L;
  const size_t head = (size_t)b * n_q + i;
  // The candidate slots and the ranges' (max, sum) are requested together
  // with the sequence length (all n_ranges slots of the head exist in the
  // workspace; those past the length's ranges are masked once it arrives),
  // so these loads cost one memory round trip.
  const float* cs = cand_s + head * n_ranges * top_k;
  const int32_t* ci = cand_i + head * n_ranges * top_k;
  const float* ml = range_ml + head * n_ranges * 2;
  const int n_slots = n_ranges * top_k;
  float s[E];
  int32_t idx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = reg_index<E>(e);
    s[e] = p < n_slots ? cs[p] : -INFINITY;
    idx[e] = p < n_slots ? ci[p] : 0;
  }
  const float ml_m = lane < n_ranges ? ml[2 * lane] : -INFINITY;
  const float ml_l = lane < n_ranges ? ml[2 * lane + 1] : 0.f;
  L = max(0, min(L_raw, min(max_ctx, l_cap)));
  const int hv = (i * n_v) / n_q;
  // Fused append only for a length inside [1, min(max_ctx, l_cap)].
  const bool fused = v_new != nullptr && L_raw == L && L > 0;
  const T* vn = fused ? v_new + ((size_t)b * n_v + hv) * DV : nullptr;
  if (fused && i % (n_q / n_v) == 0 && tid < LPR) {
    if (T* dst = cache_row_store<T, DV>(vc_w, pm, b, n_v, hv, l_cap, L - 1))
      *reinterpret_cast<u32x4*>(dst + tid * EPL) = load16(vn + tid * EPL);
  }

  // Candidates: range r contributed min(top_k, rows of r) entries at
  // [r * top_k, ...); all ranges but the last are full, so the n_c entries
  // are contiguous and in ascending row order.
  const int nr = (L + range_rows - 1) / range_rows;
  const int n_c = nr == 0 ? 0 : (nr - 1) * top_k + min(top_k, L - (nr - 1) * range_rows);
  const int kk = min(top_k, L);
  const bool in_regs = n_c <= E * NT;
  if (in_regs) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (reg_index<E>(e) >= n_c) {
        s[e] = -INFINITY;
        idx[e] = 0;
      }
    }
  }

  clear_hists<NT>(hist);
  // Softmax normaliser over all L rows from the ranges' (max, sum); every
  // wave computes it alike, so no barrier is needed.
  float M = lane < nr ? ml_m : -INFINITY;
  for (int r = lane + 64; r < nr; r += 64) M = fmaxf(M, ml[2 * r]);
  M = wave_max(M);
  float Z = lane < nr ? fast_exp2(ml_m - M) * ml_l : 0.f;
  for (int r = lane + 64; r < nr; r += 64) Z += fast_exp2(ml[2 * r] - M) * ml[2 * r + 1];
  Z = wave_sum(Z);
  const float invZ = L > 0 ? 1.f / Z : 0.f;
  __syncthreads();  // histograms cleared

  if (in_regs) {
    auto take = [&](int pos, int e) {
      if (pos < kk) {
        sel_j[pos] = idx[e];
        sel_w[pos] = fast_exp2(s[e] - M) * invZ;
      }
    };
    if (n_c <= kk) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (reg_index<E>(e) < n_c) take(reg_index<E>(e), e);
    } else {
      uint32_t key[E];
#pragma unroll
      for (int e = 0; e < E; ++e) key[e] = order_key(s[e]);
      const Threshold th = reg_select_threshold<E, NT>(key, n_c, kk, hist, red);
      reg_compact<E, NT>(key, n_c, th, red + 2 * (NT / 64), take);
    }
  } else {  // more candidates than registers hold: passes over global memory
    auto take = [&](int pos, int p) {
      if (pos < kk) {
        sel_j[pos] = ci[p];
        sel_w[pos] = fast_exp2(cs[p] - M) * invZ;
      }
    };
    auto key = [&](int p) { return order_key(cs[p]); };
    const Threshold th = block_select_threshold<NT>(key, n_c, kk, hist, red);
    block_compact<NT>(key, n_c, th, red, take);
  }
  __syncthreads();
  if (sel_idx != nullptr)
    for (int p = tid; p < top_k; p += NT)
      sel_idx[head * top_k + p] = p < kk ? sel_j[p] : -1;

  // o = sum over the selected rows of w_j V_j: LPR lanes per row, RPP rows
  // per pass, the loads of U passes issued before their use.
  const int vl = tid % LPR, vr = tid / LPR;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int r0 = vr; r0 < kk; r0 += U * RPP) {
    u32x4 v[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPP;
      w[u] = 0.f;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (r < kk) {
        const int j = min(max(sel_j[r], 0), L - 1);  // a chosen row is always in [0, L)
        w[u] = sel_w[r];
        v[u] = (fused && j == L - 1)
                   ? load16(vn + vl * EPL)
                   : load16(cache_row<const T, DV>(vc, pm, b, n_v, hv, l_cap, j) + vl * EPL);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      Elem<T>::unpack(v[u], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w[u], vf[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[vr][vl * EPL + e] = acc[e];
  __syncthreads();
  for (int d = tid; d < DV; d += NT) {
    float o = 0.f;
    for (int r = 0; r < RPP; ++r) o += part[r][d];
    out[head * DV + d] = Elem<T>::from_f32(o);
  }
  if (tid == 0 && lse != nullptr) lse[head] = L > 0 ? (M + fast_log2(Z)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ launch

// Query heads per score wave: the largest of 8, 4, 2, 1 dividing n_q / n_k
// (at most 2 when a tile's K loads already take 32 registers per lane).
static int score_heads_per_wave(const SelectiveArgs& a, int nk_loads) {
  const int G = a.n_q / a.n_k;
  const int cap = nk_loads >= 32 ? 2 : 8;
  for (int hw = cap; hw > 1; hw >>= 1)
    if (G % hw == 0) return hw;
  return 1;
}

template <typename T, int DK, int HW>
static hipError_t launch_score_hw(const SelectiveArgs& a) {
  dim3 grid(a.C, a.n_k * (a.n_q / a.n_k / HW), a.batch);
  hipLaunchKernelGGL((sel_score_kernel<T, DK, HW>), grid, dim3(256), 0, a.stream, (const T*)a.q,
                     (const T*)a.k_cache, a.ctx_len, a.scores, a.n_q, a.n_k, a.l_cap,
                     a.max_ctx, a.ld_s, a.S, a.scale * kLog2e, (const T*)a.k_new,
                     (T*)a.k_cache, a.pages);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_score_t(const SelectiveArgs& a) {
  constexpr int NK = DK / Elem<T>::kPer16;
  switch (score_heads_per_wave(a, NK)) {
    case 8:
      if constexpr (NK < 32) return launch_score_hw<T, DK, 8>(a);
      break;
    case 4:
      if constexpr (NK < 32) return launch_score_hw<T, DK, 4>(a);
      break;
    case 2: return launch_score_hw<T, DK, 2>(a);
    case 1: return launch_score_hw<T, DK, 1>(a);
  }
  return hipErrorInvalidValue;
}

// Threads of a range-selection workgroup: 512 for the short ranges (planned
// when the long ones leave CUs idle; 32k step 21.2 -> 20.7 us), 256 for the
// long ones, where more workgroups share each CU (4 x 64k 54.8 against 56.0
// at 512; 16 sequences of 4k..32k 70.5 against 72.1).
constexpr int kLocalThreadsShort = 512, kLocalThreadsLong = 256;

// Threads of the final selection and gather workgroup (selective step,
// same process: 32k 22.5 / 21.4 / 22.0 us at 256 / 512 / 1024 threads,
// 4 x 64k 56.3 / 54.9 / 55.8, 16 sequences of 4k..32k 71.3 / 70.1 / 71.1).
constexpr int kGatherThreads = 512;

template <typename T, int DV, int E>
static void launch_gather_e(const SelectiveArgs& a) {
  hipLaunchKernelGGL((sel_gather_kernel<T, DV, E, kGatherThreads>), dim3(a.n_q, a.batch),
                     dim3(kGatherThreads), 0, a.stream, (const T*)a.v_cache, a.ctx_len,
                     a.range_ml, a.cand_s, a.cand_i, (T*)a.out, a.lse, a.sel_idx, a.n_q, a.n_v,
                     a.l_cap, a.max_ctx, a.n_ranges, a.range_rows, a.top_k, (const T*)a.v_new,
                     (T*)a.v_cache, a.pages);
}

template <typename T, int DV>
static hipError_t launch_gather_t(const SelectiveArgs& a) {
  // Half the registers when every candidate fits in 2048 slots.
  constexpr int E_SMALL = 2048 / kGatherThreads, E_LARGE = 4096 / kGatherThreads;
  if ((long long)a.n_ranges * a.top_k <= 2048) launch_gather_e<T, DV, E_SMALL>(a);
  else launch_gather_e<T, DV, E_LARGE>(a);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_score_mfma(const SelectiveArgs& a) {
  const int slices = (a.n_q / a.n_k + 15) / 16;
  dim3 grid(a.C, a.n_k * slices, a.batch);
  hipLaunchKernelGGL((sel_score_mfma_kernel<DK>), grid, dim3(256), 0, a.stream, (const bf16*)a.q,
                     (const bf16*)a.k_cache, a.ctx_len, a.scores, a.n_q, a.n_k, a.l_cap,
                     a.max_ctx, a.ld_s, a.S, a.scale * kLog2e, (const bf16*)a.k_new,
                     (bf16*)a.k_cache, a.pages);
  return hipGetLastError();
}

template <typename T>
static hipError_t score_dk(const SelectiveArgs& a) {
  if constexpr (sizeof(T) == 2) {
    switch (a.d_k) {
      case 32: return launch_score_mfma<32>(a);
      case 64: return launch_score_mfma<64>(a);
      case 128: return launch_score_mfma<128>(a);
      case 256: return launch_score_mfma<256>(a);
    }
    return hipErrorInvalidValue;
  } else {
    switch (a.d_k) {
      case 32: return launch_score_t<T, 32>(a);
      case 64: return launch_score_t<T, 64>(a);
      case 128: return launch_score_t<T, 128>(a);
    }
    return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t gather_dv(const SelectiveArgs& a) {
  switch (a.d_v) {
    case 32: return launch_gather_t<T, 32>(a);
    case 64: return launch_gather_t<T, 64>(a);
    case 128: return launch_gather_t<T, 128>(a);
    case 256: return launch_gather_t<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_selective(const SelectiveArgs& a) {
  hipError_t e = a.bf16 ? score_dk<bf16>(a) : score_dk<float>(a);
  if (e != hipSuccess) return e;
  if (a.range_rows == kSelRowsShort)
    hipLaunchKernelGGL((sel_local_kernel<kSelRowsShort, kLocalThreadsShort>),
                       dim3(a.n_ranges, a.n_q, a.batch), dim3(kLocalThreadsShort), 0, a.stream,
                       a.scores, a.ctx_len, a.range_ml, a.cand_s, a.cand_i, a.n_q, a.l_cap,
                       a.max_ctx, a.ld_s, a.n_ranges, a.top_k);
  else
    hipLaunchKernelGGL((sel_local_kernel<kSelRows, kLocalThreadsLong>),
                       dim3(a.n_ranges, a.n_q, a.batch), dim3(kLocalThreadsLong), 0, a.stream,
                       a.scores, a.ctx_len, a.range_ml, a.cand_s, a.cand_i, a.n_q, a.l_cap,
                       a.max_ctx, a.ld_s, a.n_ranges, a.top_k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.bf16 ? gather_dv<bf16>(a) : gather_dv<float>(a);
}

}  // namespace dqkv
