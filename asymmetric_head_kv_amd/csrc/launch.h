// Host-side launch descriptors shared by the C ABI (api.hip) and the kernel
// translation units.  Sizes are validated by the ABI layer before a launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dqkv {

// Paged cache: row j of sequence b lives in page table[b * max_blocks +
// j / page_rows], slot j % page_rows; K pages [num_pages][n_k][page_rows][d_k],
// V pages [num_pages][n_v][page_rows][d_v].  table == nullptr: contiguous.
struct PageMap {
  const int32_t* table = nullptr;
  int max_blocks = 0;
  int page_shift = 0;  // log2(page_rows); page_rows is a multiple of 64
  int num_pages = 0;
};

struct DecodeArgs {
  bool bf16;
  int n_q, n_k, n_v, d_k, d_v;
  int batch, l_cap, max_ctx;
  int S, C;  // chunk rows, chunks per sequence
  float scale;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* ctx_len;
  void* out;
  float* lse;
  float* part_ml;   // [B][n_q][C][2]
  float* part_acc;  // [B][n_q][C][d_v]
  const void* k_new;  // fused append: newest row per sequence, or null
  const void* v_new;
  PageMap pages;
  hipStream_t stream;
};

struct AppendArgs {
  int elem_bytes;
  int n_k, n_v, d_k, d_v;
  int batch, t_new, l_cap;
  const void* k_new;
  const void* v_new;
  const int32_t* pos;
  void* k_cache;
  void* v_cache;
  PageMap pages;
  hipStream_t stream;
};

// kv_group_sharing: copy of a head-major cache [B][n_src][l_cap][d] to
// [B][n_dst][l_cap][d], destination head h reading source head
// floor(h * n_src / n_dst).
struct ExpandArgs {
  int n_src, n_dst;
  size_t head_bytes;  // l_cap * d * element size, a multiple of 16
  int batch;
  const void* src;
  void* dst;
  hipStream_t stream;
};

struct PrefillArgs {
  int n_q, n_k, n_v, d_k, d_v;
  int batch, t_new, l_cap;
  float scale;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* ctx_len;
  void* out;
  float* lse;
  int n_split;      // key splits (1: no merge, no workspace)
  float* part_o;    // [n_split][B][t_new][n_q][d_v] fp32
  float* part_ml;   // [n_split][B][t_new][n_q] split lse, log2 units
  PageMap pages;    // table == nullptr: contiguous caches
  hipStream_t stream;
};

// Selective-V decode: rows per local-selection range (planned: the longer
// one unless that leaves fewer workgroups than compute units), and the
// largest top_k.
constexpr int kSelRows = 4096;
constexpr int kSelRowsShort = 2048;
constexpr int kMaxTopK = 1024;

struct SelectiveArgs {
  bool bf16;
  int n_q, n_k, n_v, d_k, d_v;
  int batch, l_cap, max_ctx;
  int S, C;       // score-kernel chunk rows, chunks per sequence
  int ld_s;       // row stride of the logit buffer (max_ctx rounded up to 64)
  int range_rows; // rows per local-selection range: kSelRows or kSelRowsShort
  int n_ranges;   // ceil(max_ctx / range_rows)
  int top_k;
  float scale;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* ctx_len;
  void* out;
  float* lse;
  int32_t* sel_idx;   // [B][n_q][top_k] or null
  float* scores;      // [B][n_q][ld_s]      base-2 logits
  float* range_ml;    // [B][n_q][n_ranges][2]
  float* cand_s;      // [B][n_q][n_ranges][top_k]
  int32_t* cand_i;    // [B][n_q][n_ranges][top_k]
  const void* k_new;  // fused append, or null
  const void* v_new;
  PageMap pages;    // table == nullptr: contiguous caches
  hipStream_t stream;
};

// Augmented-Q projection (bf16): h [M][d_m]; w_gate, w_up [d_i][d_m];
// w_down [d_out][d_i], all three packed (launch_augq_pack); act [M][d_i]
// (the gated intermediate); q [M][d_out].
struct AugQArgs {
  int M, d_m, d_i, d_out;
  const void* h;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* act;
  void* q;
  hipStream_t stream;
};

hipError_t launch_decode_split(const DecodeArgs& a);
hipError_t launch_decode_combine(const DecodeArgs& a);
hipError_t launch_kv_append(const AppendArgs& a);
hipError_t launch_expand_heads(const ExpandArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_decode_selective(const SelectiveArgs& a);
hipError_t launch_augq(const AugQArgs& a);
hipError_t launch_augq_pack(const void* w, void* wp, int N, int K, hipStream_t stream);

}  // namespace dqkv
