// C ABI of the DiffQKV attention library (declarations and contracts in
// include/diffqkv.h): argument validation, launch planning and workspace
// layout.  No entry point allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "diffqkv.h"
#include "launch.h"

namespace {

constexpr int kCUs = 256;             // MI355X compute units
// Split waves to aim for per CU.  Contiguous caches: one four-wave
// workgroup per CU in one round (32k x 1 sequence: 512-row chunks, 29.5 us
// per step against 30.5 at 256-row chunks with two per CU; a fraction of a
// second round, e.g. 448-row chunks, costs 25%).  Paged caches keep two per
// CU: each 64-row tile sits in its own page, and the second wave per SIMD
// hides that latency (512-row chunks: 33.2 us against 30.8).
constexpr int kWavesPerCUContig = 4;
constexpr int kWavesPerCUPaged = 8;
// A contiguous layout whose workgroup loads fewer than kSmallTileElems
// elements per 64-row tile (the rows of its distinct K heads plus those of
// its distinct V heads; 48 KiB in bf16) also plans two workgroups per CU, for
// enough loads in flight: the pages' SIGMA-1.5B attention (32 / 4 / 16 heads,
// d 64: one K head and four V heads per workgroup, 40 KiB in bf16) takes
// 21.5 us per 32k step at 256-row chunks against 22.2 at 512, and 14.5
// against 15.4 at 16k; the 16 / 4 / 16 d_k 64 / d_v 128 layout (72 KiB)
// loses 2% that way.  Counted in elements, not bytes, so that the plan does
// not depend on the dtype (the chunk and workspace queries take none).
constexpr long long kSmallTileElems = 24 << 10;
constexpr int kMaxChunks = 8192;      // bounds the workspace and the combine's loop
// Batches of at least kRaggedBatch sequences plan kRaggedOversub times more
// split workgroups: the host cannot see the lengths (they stay on the
// device), and when they differ the chunks past a short sequence's end are
// empty, so with one planned round many CU slots would sit idle.  With more,
// smaller chunks the dispatcher refills them (16 sequences of 4k..32k rows:
// 276 us at one round, 254 us at 8x (512-row chunks), 238 us at 7x (640-row
// chunks; 448 and 768 rows time alike, 512 and 1024 slower); uniform
// 4 x 64k loses 3% at such chunk lengths, so small batches keep one round).
constexpr int kRaggedBatch = 8;
constexpr int kRaggedOversub = 7;
constexpr int kMinChunk = 64;
// Contiguous layouts with d_k <= 64 (split kernel with the K look-ahead)
// whose one-round plan gives chunks of kLongChunk rows or more aim at 15/16
// of the CUs instead, chunks rounded up to kLongRound rows: fewer, longer
// streams run faster there (4 x 64k, 16 / 4 / 16 heads: 4096-row chunks
// 175.8 us per step, 4416 173.5, 4608 171.9 -- the rule's choice, 15 chunks
// per sequence -- and 5120 172.4; same process, three boxes).  Without the
// look-ahead fewer workgroups were slower (d_k 128: 5120-row chunks 227 us
// against 198.6 at 4096; the symmetric layout 322.6 against 319.8).
constexpr int kLongChunk = 4096;
constexpr int kLongRound = 512;

bool is_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

int check_heads(int n_q, int n_k, int n_v, int d_k, int d_v) {
  if (n_q <= 0 || n_k <= 0 || n_v <= 0 || d_k <= 0 || d_v <= 0) return DQKV_ERR_SHAPE;
  if (n_k > n_q || n_v > n_q || n_q % n_k != 0 || n_q % n_v != 0) return DQKV_ERR_SHAPE;
  return DQKV_OK;
}

int check_dtype_dims(int dtype, int d_k, int d_v) {
  if (dtype != DQKV_F32 && dtype != DQKV_BF16) return DQKV_ERR_UNSUPPORTED;
  if (!is_dim(d_k) || !is_dim(d_v)) return DQKV_ERR_UNSUPPORTED;
  if (dtype == DQKV_F32 && d_k == 256) return DQKV_ERR_UNSUPPORTED;
  return DQKV_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int to_status(hipError_t e) { return e == hipSuccess ? DQKV_OK : DQKV_ERR_HIP; }

// Rows per context chunk: enough (sequence, head-quad, chunk) workgroups to
// give every CU about the planned waves (times kRaggedOversub for large
// batches), in multiples of 64 rows.  H = query heads per wave; small =
// fewer than kSmallTileElems per workgroup tile.
int plan_chunk_h(int n_q, int H, int batch, int max_ctx, bool paged, bool small,
                 bool look_ahead) {
  long long quads = (long long)batch * ((n_q / H + 3) / 4);
  if (quads < 1) quads = 1;  // an empty batch launches nothing
  const bool one_round = !(paged || small || batch >= kRaggedBatch);
  const int waves = one_round ? kWavesPerCUContig : kWavesPerCUPaged;
  const long long want_wg = (long long)kCUs * waves / 4 *
                            (batch >= kRaggedBatch ? kRaggedOversub : 1);
  long long chunks_per_seq = (want_wg + quads - 1) / quads;
  if (chunks_per_seq < 1) chunks_per_seq = 1;
  long long S = (max_ctx + chunks_per_seq - 1) / chunks_per_seq;
  S = (S + kMinChunk - 1) / kMinChunk * kMinChunk;
  if (one_round && look_ahead && S >= kLongChunk) {
    long long cps = (want_wg * 15 / 16 + quads - 1) / quads;
    if (cps < 1) cps = 1;
    S = (max_ctx + cps - 1) / cps;
    S = (S + kLongRound - 1) / kLongRound * kLongRound;
  }
  if (S < kMinChunk) S = kMinChunk;
  const long long s_floor = ((long long)max_ctx + kMaxChunks - 1) / kMaxChunks;
  if (S < s_floor) S = (s_floor + kMinChunk - 1) / kMinChunk * kMinChunk;
  if (S > (1 << 30)) S = 1 << 30;
  return (int)S;
}

int plan_chunk(int n_q, int n_k, int n_v, int d_k, int d_v, int batch, int max_ctx,
               bool paged) {
  // Waves per (sequence, chunk): one per query head, or per pair of query
  // heads that share their K and V heads (see the split kernel).
  const int H = (n_q == 2 * n_v && (n_q / n_k) % 2 == 0) ? 2 : 1;
  // Elements of one 64-row tile of a four-wave workgroup: the distinct K and
  // V heads of its 4 H consecutive query heads.
  const long long heads = 4LL * H, G = n_q / n_k, Gv = n_q / n_v;
  const long long k_heads = (heads + G - 1) / G, v_heads = (heads + Gv - 1) / Gv;
  const long long tile = 64LL * (k_heads * d_k + v_heads * d_v);
  return plan_chunk_h(n_q, H, batch, max_ctx, paged, tile < kSmallTileElems, d_k <= 64);
}

int chunks_for(int max_ctx, int S) {
  const int c = (int)(((long long)max_ctx + S - 1) / S);
  return c < 1 ? 1 : c;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The softmax scale a call uses: 0 selects the default 1/sqrt(d_k), the
// divisor of the attention scores in section 3.4 Step 4 of the Sigma
// architecture page; any other value must be positive and finite.  Returns
// false for a rejected value.
bool resolve_scale(float scale, int d_k, float* out) {
  if (scale == 0.f) {
    *out = 1.f / sqrtf((float)d_k);
    return true;
  }
  if (!(scale > 0.f) || !isfinite(scale)) return false;
  *out = scale;
  return true;
}

constexpr int kPrefillRows = 128;  // query rows per prefill workgroup

// Key splits for a prefill: enough workgroups for two per CU (the kernel's
// registers allow two waves per SIMD), at most 4.
int plan_prefill_split(int n_q, int batch, int t_new) {
  const long long wg = (long long)batch * n_q * ((t_new + kPrefillRows - 1) / kPrefillRows);
  if (wg <= 0) return 1;
  long long ns = (2LL * kCUs + wg - 1) / wg;
  if (ns < 1) ns = 1;
  if (ns > 4) ns = 4;
  return (int)ns;
}

size_t prefill_workspace_bytes(int ns, int n_q, int d_v, int batch, int t_new) {
  if (ns <= 1) return 0;
  const size_t rows = (size_t)batch * t_new * n_q;
  return align256((size_t)ns * rows * d_v * sizeof(float)) + (size_t)ns * rows * sizeof(float);
}

size_t workspace_bytes(int n_q, int d_v, int batch, int C) {
  const size_t parts = (size_t)batch * n_q * C;
  return align256(parts * 2 * sizeof(float)) + parts * d_v * sizeof(float);
}

int resolve_chunk(int n_q, int n_k, int n_v, int d_k, int d_v, int batch, int max_ctx,
                  int chunk_tokens, int* S, bool paged = false) {
  if (chunk_tokens < 0 || chunk_tokens % kMinChunk != 0) return DQKV_ERR_SHAPE;
  *S = chunk_tokens ? chunk_tokens : plan_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx, paged);
  if (chunks_for(max_ctx, *S) > kMaxChunks) return DQKV_ERR_UNSUPPORTED;
  return DQKV_OK;
}

// Workspace of a selective-V decode: logits, per-range (max, sum), and the
// per-range candidates (logit, row).
struct SelLayout {
  int S, C, ld_s, range_rows, n_ranges;
  size_t off_ml, off_cs, off_ci, total;
};

// Rows per logit-kernel workgroup (four waves, one 64-row tile each per
// step): one tile per wave while that needs at most 4096 waves, more beyond;
// batches of kRaggedBatch or more sequences aim at 16384 waves, since chunks
// past a short sequence's end are empty (4 x 64k: 51.7 -> 50.4 us per
// selective step at 1024-row chunks; 16 sequences of 4k..32k rows:
// 80.7 -> 74.5 us at 512-row chunks).
int plan_score_chunk(int n_k, int batch, int max_ctx) {
  const long long tiles = ((long long)max_ctx + 63) / 64 * n_k * batch;
  const long long target = batch >= kRaggedBatch ? 16384 : 4096;
  long long tpw = (tiles + target - 1) / target;
  if (tpw < 1) tpw = 1;
  if (tpw > (1 << 20)) tpw = 1 << 20;
  return (int)(256 * tpw);
}

int selective_layout(int n_q, int n_k, int batch, int max_ctx, int top_k, SelLayout* o) {
  if (top_k < 1) return DQKV_ERR_SHAPE;
  if (top_k > dqkv::kMaxTopK) return DQKV_ERR_UNSUPPORTED;
  o->S = plan_score_chunk(n_k, batch, max_ctx);
  o->C = chunks_for(max_ctx, o->S);
  if (o->C > kMaxChunks) return DQKV_ERR_UNSUPPORTED;
  o->ld_s = (int)(((long long)max_ctx + 63) / 64 * 64);
  if (o->ld_s < 64) o->ld_s = 64;
  // Shorter ranges when the longer ones would leave CUs without a local
  // selection (32k x 1 sequence x 16 heads: 8 ranges each -> 128 workgroups;
  // 2048-row ranges: 26.9 -> 23.0 us per step; with enough workgroups the
  // longer ranges win, as the final selection then merges half the
  // candidates: 4 x 64k, 53.9 against 67.0 us).
  const long long long_ranges = ((long long)max_ctx + dqkv::kSelRows - 1) / dqkv::kSelRows;
  o->range_rows = (long long)batch * n_q * long_ranges < kCUs ? dqkv::kSelRowsShort
                                                               : dqkv::kSelRows;
  o->n_ranges = (int)(((long long)max_ctx + o->range_rows - 1) / o->range_rows);
  if (o->n_ranges < 1) o->n_ranges = 1;
  const size_t heads = (size_t)batch * n_q;
  o->off_ml = align256(heads * o->ld_s * sizeof(float));
  o->off_cs = o->off_ml + align256(heads * o->n_ranges * 2 * sizeof(float));
  const size_t cand = heads * o->n_ranges * (size_t)top_k;
  o->off_ci = o->off_cs + align256(cand * sizeof(float));
  o->total = o->off_ci + cand * sizeof(int32_t);
  return DQKV_OK;
}

}  // namespace

// ------------------------------------------------- static decode scratch
//
// diffqkv_decode_append_noalloc keeps the split kernel's partial results in
// this file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy (kScratchBytes, from module load until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// device memory: the device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is passed to
// kernels.
namespace {
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of scratch, per device

// The current device's scratch address (looked up on the first call on that
// device).  Returns DQKV_OK or DQKV_ERR_HIP.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DQKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return DQKV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DQKV_OK;
}
}  // namespace

extern "C" {

const char* dqkv_status_str(int32_t status) {
  switch (status) {
    case DQKV_OK: return "DQKV_OK";
    case DQKV_ERR_NULL: return "DQKV_ERR_NULL: a required pointer is NULL";
    case DQKV_ERR_SHAPE: return "DQKV_ERR_SHAPE: sizes violate the head / length rules";
    case DQKV_ERR_UNSUPPORTED: return "DQKV_ERR_UNSUPPORTED: size or dtype not built";
    case DQKV_ERR_WORKSPACE: return "DQKV_ERR_WORKSPACE: workspace too small";
    case DQKV_ERR_HIP: return "DQKV_ERR_HIP: the HIP runtime refused a launch";
    case DQKV_ERR_ALIGN: return "DQKV_ERR_ALIGN: a device pointer is not 16-byte aligned";
  }
  return "unknown dqkv status";
}

int32_t diffqkv_decode_chunk(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                             int32_t d_v, int32_t batch, int32_t max_ctx,
                             int32_t* chunk_tokens) {
  if (!chunk_tokens) return DQKV_ERR_NULL;
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  if (batch < 0 || max_ctx < 0) return DQKV_ERR_SHAPE;
  return resolve_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx, 0, chunk_tokens);
}

int32_t diffqkv_decode_workspace(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                                 int32_t d_v, int32_t batch, int32_t max_ctx,
                                 int32_t chunk_tokens, size_t* bytes) {
  if (!bytes) return DQKV_ERR_NULL;
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  if (batch < 0 || max_ctx < 0) return DQKV_ERR_SHAPE;
  // With the automatic choice: enough for the contiguous and the paged plan
  // (the paged one never has fewer chunks).
  int S = 0, Sp = 0;
  st = resolve_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx, chunk_tokens, &S);
  if (st) return st;
  st = resolve_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx, chunk_tokens, &Sp, true);
  if (st) return st;
  *bytes = workspace_bytes(n_q, d_v, batch, chunks_for(max_ctx, S < Sp ? S : Sp));
  return DQKV_OK;
}

int32_t kv_append(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                  int32_t dtype, int32_t batch, int32_t t_new, int32_t l_cap,
                  const void* k_new, const void* v_new, const int32_t* pos,
                  void* k_cache, void* v_cache, void* stream) {
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  st = check_dtype_dims(dtype, d_k, d_v);
  if (st) return st;
  if (batch < 0 || t_new < 0 || l_cap < 0 || batch > 65535) return DQKV_ERR_SHAPE;
  if (batch == 0 || t_new == 0) return DQKV_OK;
  if (!k_new || !v_new || !pos || !k_cache || !v_cache) return DQKV_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return DQKV_ERR_ALIGN;
  dqkv::AppendArgs a;
  a.elem_bytes = dtype == DQKV_BF16 ? 2 : 4;
  a.n_k = n_k; a.n_v = n_v; a.d_k = d_k; a.d_v = d_v;
  a.batch = batch; a.t_new = t_new; a.l_cap = l_cap;
  a.k_new = k_new; a.v_new = v_new; a.pos = pos;
  a.k_cache = k_cache; a.v_cache = v_cache;
  a.stream = (hipStream_t)stream;
  return to_status(dqkv::launch_kv_append(a));
}

// Points the descriptor's partial-result arrays into a decode workspace:
// (m, l) pairs first, then the weighted V sums from the next 256-byte
// boundary.
static void bind_decode_workspace(dqkv::DecodeArgs* a, void* workspace) {
  const size_t parts = (size_t)a->batch * a->n_q * a->C;
  a->part_ml = (float*)workspace;
  a->part_acc = workspace ? (float*)((char*)workspace + align256(parts * 2 * sizeof(float)))
                          : nullptr;
}

// Validates a decode call and fills the launch descriptor.  need_qkv /
// need_out select which buffers the caller's entry point uses.
static int prepare_decode(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                          int32_t dtype, int32_t batch, int32_t l_cap, int32_t max_ctx,
                          float scale, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* ctx_len, void* out,
                          float* lse, int32_t chunk_tokens, void* workspace,
                          size_t workspace_bytes_given, void* stream, bool need_qkv,
                          bool need_out, dqkv::DecodeArgs* a, bool paged = false,
                          bool check_ws_ptr = true) {
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  st = check_dtype_dims(dtype, d_k, d_v);
  if (st) return st;
  if (batch < 0 || l_cap < 0 || max_ctx < 0 || max_ctx > l_cap || batch > 65535)
    return DQKV_ERR_SHAPE;
  if (need_qkv && !resolve_scale(scale, d_k, &scale)) return DQKV_ERR_SHAPE;
  if (need_qkv && (!q || !k_cache || !v_cache)) return DQKV_ERR_NULL;
  if (need_out && !out) return DQKV_ERR_NULL;
  if (!ctx_len || (check_ws_ptr && !workspace)) return DQKV_ERR_NULL;
  if ((need_qkv && (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))) ||
      (need_out && !aligned16(out)) || (check_ws_ptr && !aligned16(workspace)))
    return DQKV_ERR_ALIGN;
  int S = 0;
  st = resolve_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx, chunk_tokens, &S, paged);
  if (st) return st;
  const int C = chunks_for(max_ctx, S);
  if ((long long)(n_q + 3) / 4 > 65535) return DQKV_ERR_UNSUPPORTED;
  const size_t need = workspace_bytes(n_q, d_v, batch, C);
  if (workspace_bytes_given < need) return DQKV_ERR_WORKSPACE;

  a->bf16 = dtype == DQKV_BF16;
  a->n_q = n_q; a->n_k = n_k; a->n_v = n_v; a->d_k = d_k; a->d_v = d_v;
  a->batch = batch; a->l_cap = l_cap; a->max_ctx = max_ctx;
  a->S = S; a->C = C; a->scale = scale;
  a->q = q; a->k_cache = k_cache; a->v_cache = v_cache; a->ctx_len = ctx_len;
  a->out = out; a->lse = lse;
  a->k_new = nullptr; a->v_new = nullptr;
  bind_decode_workspace(a, workspace);
  a->stream = (hipStream_t)stream;
  return DQKV_OK;
}

int32_t diffqkv_decode(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                       int32_t dtype, int32_t batch, int32_t l_cap, int32_t max_ctx,
                       float scale, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* ctx_len, void* out,
                       float* lse, int32_t chunk_tokens, void* workspace,
                       size_t workspace_bytes_given, void* stream) {
  if (batch == 0 && n_q > 0) {
    int st = check_heads(n_q, n_k, n_v, d_k, d_v);
    return st ? st : check_dtype_dims(dtype, d_k, d_v);
  }
  dqkv::DecodeArgs a;
  int st = prepare_decode(n_q, n_k, n_v, d_k, d_v, dtype, batch, l_cap, max_ctx, scale, q,
                          k_cache, v_cache, ctx_len, out, lse, chunk_tokens, workspace,
                          workspace_bytes_given, stream, true, true, &a);
  if (st) return st;
  st = to_status(dqkv::launch_decode_split(a));
  if (st) return st;
  return to_status(dqkv::launch_decode_combine(a));
}

int32_t diffqkv_decode_split(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                             int32_t dtype, int32_t batch, int32_t l_cap, int32_t max_ctx,
                             float scale, const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* ctx_len, int32_t chunk_tokens, void* workspace,
                             size_t workspace_bytes_given, void* stream) {
  if (batch == 0 && n_q > 0) {
    int st = check_heads(n_q, n_k, n_v, d_k, d_v);
    return st ? st : check_dtype_dims(dtype, d_k, d_v);
  }
  if ((k_new == nullptr) != (v_new == nullptr)) return DQKV_ERR_NULL;
  dqkv::DecodeArgs a;
  int st = prepare_decode(n_q, n_k, n_v, d_k, d_v, dtype, batch, l_cap, max_ctx, scale, q,
                          k_cache, v_cache, ctx_len, nullptr, nullptr, chunk_tokens,
                          workspace, workspace_bytes_given, stream, true, false, &a);
  if (st) return st;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return DQKV_ERR_ALIGN;
  a.k_new = k_new;
  a.v_new = v_new;
  return to_status(dqkv::launch_decode_split(a));
}

int32_t diffqkv_decode_append(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                              int32_t d_v, int32_t dtype, int32_t batch, int32_t l_cap,
                              int32_t max_ctx, float scale, const void* q,
                              const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, const int32_t* ctx_len, void* out, float* lse,
                              int32_t chunk_tokens, void* workspace,
                              size_t workspace_bytes_given, void* stream) {
  if (batch == 0 && n_q > 0) {
    int st = check_heads(n_q, n_k, n_v, d_k, d_v);
    return st ? st : check_dtype_dims(dtype, d_k, d_v);
  }
  dqkv::DecodeArgs a;
  int st = prepare_decode(n_q, n_k, n_v, d_k, d_v, dtype, batch, l_cap, max_ctx, scale, q,
                          k_cache, v_cache, ctx_len, out, lse, chunk_tokens, workspace,
                          workspace_bytes_given, stream, true, true, &a);
  if (st) return st;
  if (!k_new || !v_new) return DQKV_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return DQKV_ERR_ALIGN;
  a.k_new = k_new;
  a.v_new = v_new;
  st = to_status(dqkv::launch_decode_split(a));
  if (st) return st;
  return to_status(dqkv::launch_decode_combine(a));
}

int32_t diffqkv_decode_append_noalloc(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                                      int32_t d_v, int32_t dtype, int32_t batch,
                                      int32_t l_cap, int32_t max_ctx, float scale,
                                      const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* ctx_len,
                                      void* out, float* lse, int32_t chunk_tokens,
                                      void* stream) {
  if (batch == 0 && n_q > 0) {
    int st = check_heads(n_q, n_k, n_v, d_k, d_v);
    return st ? st : check_dtype_dims(dtype, d_k, d_v);
  }
  if ((k_new == nullptr) != (v_new == nullptr)) return DQKV_ERR_NULL;
  // Host-side checks first; the size check rejects calls whose partials do
  // not fit the static scratch (DQKV_ERR_WORKSPACE).
  dqkv::DecodeArgs a;
  int st = prepare_decode(n_q, n_k, n_v, d_k, d_v, dtype, batch, l_cap, max_ctx, scale, q,
                          k_cache, v_cache, ctx_len, out, lse, chunk_tokens, nullptr,
                          kScratchBytes, stream, true, true, &a, false, false);
  if (st) return st;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return DQKV_ERR_ALIGN;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st) return st;
  bind_decode_workspace(&a, ws);
  a.k_new = k_new;
  a.v_new = v_new;
  st = to_status(dqkv::launch_decode_split(a));
  if (st) return st;
  return to_status(dqkv::launch_decode_combine(a));
}

int32_t diffqkv_decode_combine(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                               int32_t d_v, int32_t dtype, int32_t batch, int32_t l_cap,
                               int32_t max_ctx, const int32_t* ctx_len, void* out,
                               float* lse, int32_t chunk_tokens, void* workspace,
                               size_t workspace_bytes_given, void* stream) {
  if (batch == 0 && n_q > 0) {
    int st = check_heads(n_q, n_k, n_v, d_k, d_v);
    return st ? st : check_dtype_dims(dtype, d_k, d_v);
  }
  dqkv::DecodeArgs a;
  int st = prepare_decode(n_q, n_k, n_v, d_k, d_v, dtype, batch, l_cap, max_ctx, 1.f,
                          nullptr, nullptr, nullptr, ctx_len, out, lse, chunk_tokens,
                          workspace, workspace_bytes_given, stream, false, true, &a);
  if (st) return st;
  return to_status(dqkv::launch_decode_combine(a));
}

int32_t diffqkv_prefill_workspace(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                                  int32_t d_v, int32_t batch, int32_t t_new, size_t* bytes) {
  if (!bytes) return DQKV_ERR_NULL;
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  if (batch < 0 || t_new < 0) return DQKV_ERR_SHAPE;
  const int ns = plan_prefill_split(n_q, batch, t_new);
  *bytes = prefill_workspace_bytes(ns, n_q, d_v, batch, t_new);
  return DQKV_OK;
}

static int check_pages(int32_t page_rows, int32_t num_pages, int32_t max_blocks,
                       const int32_t* table, dqkv::PageMap* pm, int* cap);

// Shared by diffqkv_prefill and diffqkv_prefill_paged: validates the call
// and launches the prefill (and, when split, its merge).  pm.table == NULL
// means contiguous caches of l_cap rows.
static int run_prefill(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                       int32_t dtype, int32_t batch, int32_t t_new, int32_t l_cap, float scale,
                       const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* ctx_len, void* out, float* lse, void* workspace,
                       size_t workspace_bytes_given, void* stream, const dqkv::PageMap& pm) {
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  if (dtype != DQKV_BF16) return DQKV_ERR_UNSUPPORTED;
  if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return DQKV_ERR_UNSUPPORTED;
  if (batch < 0 || t_new < 0 || l_cap < 0 || batch > 65535) return DQKV_ERR_SHAPE;
  if (!resolve_scale(scale, d_k, &scale)) return DQKV_ERR_SHAPE;
  if (batch == 0 || t_new == 0) return DQKV_OK;
  if (!q || !k_cache || !v_cache || !ctx_len || !out) return DQKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (workspace && !aligned16(workspace)))
    return DQKV_ERR_ALIGN;
  const long long n_qtiles = ((long long)t_new + kPrefillRows - 1) / kPrefillRows;
  int ns = plan_prefill_split(n_q, batch, t_new);
  const size_t need = prefill_workspace_bytes(ns, n_q, d_v, batch, t_new);
  if (ns > 1 && (!workspace || workspace_bytes_given < need)) ns = 1;  // run unsplit
  if (n_qtiles * n_q * ns > 0x7fffffffLL) return DQKV_ERR_UNSUPPORTED;
  dqkv::PrefillArgs a;
  a.n_q = n_q; a.n_k = n_k; a.n_v = n_v; a.d_k = d_k; a.d_v = d_v;
  a.batch = batch; a.t_new = t_new; a.l_cap = l_cap; a.scale = scale;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.ctx_len = ctx_len;
  a.out = out; a.lse = lse;
  a.n_split = ns;
  const size_t rows = (size_t)batch * t_new * n_q;
  a.part_o = ns > 1 ? (float*)workspace : nullptr;
  a.part_ml = ns > 1 ? (float*)((char*)workspace + align256((size_t)ns * rows * d_v * sizeof(float)))
                     : nullptr;
  a.pages = pm;
  a.stream = (hipStream_t)stream;
  return to_status(dqkv::launch_prefill(a));
}

int32_t diffqkv_prefill(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                        int32_t dtype, int32_t batch, int32_t t_new, int32_t l_cap,
                        float scale, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* ctx_len, void* out,
                        float* lse, void* workspace, size_t workspace_bytes_given,
                        void* stream) {
  return run_prefill(n_q, n_k, n_v, d_k, d_v, dtype, batch, t_new, l_cap, scale, q, k_cache,
                     v_cache, ctx_len, out, lse, workspace, workspace_bytes_given, stream,
                     dqkv::PageMap{});
}

int32_t diffqkv_prefill_paged(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                              int32_t dtype, int32_t batch, int32_t t_new, int32_t page_rows,
                              int32_t num_pages, int32_t max_blocks, float scale,
                              const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* ctx_len, void* out,
                              float* lse, void* workspace, size_t workspace_bytes_given,
                              void* stream) {
  dqkv::PageMap pm;
  int cap = 0;
  int st = check_pages(page_rows, num_pages, max_blocks, block_table, &pm, &cap);
  if (st) return st;
  if (batch > 0 && t_new > 0 && !block_table) return DQKV_ERR_NULL;
  return run_prefill(n_q, n_k, n_v, d_k, d_v, dtype, batch, t_new, cap, scale, q, k_pages,
                     v_pages, ctx_len, out, lse, workspace, workspace_bytes_given, stream, pm);
}

int32_t diffqkv_decode_selective_workspace(int32_t n_q, int32_t n_k, int32_t n_v,
                                           int32_t d_k, int32_t d_v, int32_t batch,
                                           int32_t max_ctx, int32_t top_k, size_t* bytes) {
  if (!bytes) return DQKV_ERR_NULL;
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  if (batch < 0 || max_ctx < 0) return DQKV_ERR_SHAPE;
  SelLayout lay;
  st = selective_layout(n_q, n_k, batch, max_ctx, top_k, &lay);
  if (st) return st;
  *bytes = lay.total;
  return DQKV_OK;
}

// Shared by diffqkv_decode_selective and its paged form (pm.table != NULL:
// k_cache / v_cache are page pools and l_cap their table's row capacity).
static int run_selective(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                         int32_t dtype, int32_t batch, int32_t l_cap, int32_t max_ctx,
                         float scale, int32_t top_k, const void* q, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* ctx_len, void* out, float* lse, int32_t* sel_idx,
                         void* workspace, size_t workspace_bytes_given, void* stream,
                         const dqkv::PageMap& pm) {
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  st = check_dtype_dims(dtype, d_k, d_v);
  if (st) return st;
  if (batch < 0 || l_cap < 0 || max_ctx < 0 || max_ctx > l_cap || batch > 65535 ||
      n_q > 65535)
    return DQKV_ERR_SHAPE;
  if (!resolve_scale(scale, d_k, &scale)) return DQKV_ERR_SHAPE;
  SelLayout lay;
  st = selective_layout(n_q, n_k, batch, max_ctx, top_k, &lay);
  if (st) return st;
  if (batch == 0) return DQKV_OK;
  if ((k_new == nullptr) != (v_new == nullptr)) return DQKV_ERR_NULL;
  if (!q || !k_cache || !v_cache || !ctx_len || !out || !workspace) return DQKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace) || (k_new && (!aligned16(k_new) || !aligned16(v_new))))
    return DQKV_ERR_ALIGN;
  if (workspace_bytes_given < lay.total) return DQKV_ERR_WORKSPACE;
  dqkv::SelectiveArgs a;
  a.bf16 = dtype == DQKV_BF16;
  a.n_q = n_q; a.n_k = n_k; a.n_v = n_v; a.d_k = d_k; a.d_v = d_v;
  a.batch = batch; a.l_cap = l_cap; a.max_ctx = max_ctx;
  a.S = lay.S; a.C = lay.C; a.ld_s = lay.ld_s; a.n_ranges = lay.n_ranges;
  a.range_rows = lay.range_rows;
  a.top_k = top_k; a.scale = scale;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.ctx_len = ctx_len;
  a.out = out; a.lse = lse; a.sel_idx = sel_idx;
  char* ws = (char*)workspace;
  a.scores = (float*)ws;
  a.range_ml = (float*)(ws + lay.off_ml);
  a.cand_s = (float*)(ws + lay.off_cs);
  a.cand_i = (int32_t*)(ws + lay.off_ci);
  a.k_new = k_new; a.v_new = v_new;
  a.pages = pm;
  a.stream = (hipStream_t)stream;
  return to_status(dqkv::launch_decode_selective(a));
}

int32_t diffqkv_decode_selective(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                                 int32_t d_v, int32_t dtype, int32_t batch, int32_t l_cap,
                                 int32_t max_ctx, float scale, int32_t top_k, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const int32_t* ctx_len, void* out, float* lse,
                                 int32_t* sel_idx, void* workspace,
                                 size_t workspace_bytes_given, void* stream) {
  return run_selective(n_q, n_k, n_v, d_k, d_v, dtype, batch, l_cap, max_ctx, scale, top_k, q,
                       k_new, v_new, k_cache, v_cache, ctx_len, out, lse, sel_idx, workspace,
                       workspace_bytes_given, stream, dqkv::PageMap{});
}

int32_t diffqkv_decode_selective_paged(
    int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v, int32_t dtype,
    int32_t batch, int32_t page_rows, int32_t num_pages, int32_t max_blocks, int32_t max_ctx,
    float scale, int32_t top_k, const void* q, const void* k_new, const void* v_new,
    void* k_pages, void* v_pages, const int32_t* block_table, const int32_t* ctx_len,
    void* out, float* lse, int32_t* sel_idx, void* workspace, size_t workspace_bytes_given,
    void* stream) {
  dqkv::PageMap pm;
  int cap = 0;
  int st = check_pages(page_rows, num_pages, max_blocks, block_table, &pm, &cap);
  if (st) return st;
  if (batch > 0 && !block_table) return DQKV_ERR_NULL;
  return run_selective(n_q, n_k, n_v, d_k, d_v, dtype, batch, cap, max_ctx, scale, top_k, q,
                       k_new, v_new, k_pages, v_pages, ctx_len, out, lse, sel_idx, workspace,
                       workspace_bytes_given, stream, pm);
}

// ---------------------------------------------------------------- paged cache

// Validates a page geometry; fills *pm and the row capacity it implies.
static int check_pages(int32_t page_rows, int32_t num_pages, int32_t max_blocks,
                       const int32_t* table, dqkv::PageMap* pm, int* cap) {
  if (page_rows < 64 || page_rows > (1 << 20) || (page_rows & (page_rows - 1)) != 0)
    return DQKV_ERR_SHAPE;
  if (num_pages < 1 || max_blocks < 1) return DQKV_ERR_SHAPE;
  int shift = 0;
  while ((1 << shift) < page_rows) ++shift;
  const long long c = (long long)max_blocks * page_rows;
  if (c > 0x7fffffffLL) return DQKV_ERR_UNSUPPORTED;
  pm->table = table;
  pm->max_blocks = max_blocks;
  pm->page_shift = shift;
  pm->num_pages = num_pages;
  *cap = (int)c;
  return DQKV_OK;
}

int32_t kv_append_paged(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                        int32_t dtype, int32_t batch, int32_t t_new, int32_t page_rows,
                        int32_t num_pages, int32_t max_blocks, const void* k_new,
                        const void* v_new, const int32_t* pos, const int32_t* block_table,
                        void* k_pages, void* v_pages, void* stream) {
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  st = check_dtype_dims(dtype, d_k, d_v);
  if (st) return st;
  if (batch < 0 || t_new < 0 || batch > 65535) return DQKV_ERR_SHAPE;
  dqkv::PageMap pm;
  int cap = 0;
  st = check_pages(page_rows, num_pages, max_blocks, block_table, &pm, &cap);
  if (st) return st;
  if (batch == 0 || t_new == 0) return DQKV_OK;
  if (!k_new || !v_new || !pos || !block_table || !k_pages || !v_pages) return DQKV_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages))
    return DQKV_ERR_ALIGN;
  dqkv::AppendArgs a;
  a.elem_bytes = dtype == DQKV_BF16 ? 2 : 4;
  a.n_k = n_k; a.n_v = n_v; a.d_k = d_k; a.d_v = d_v;
  a.batch = batch; a.t_new = t_new; a.l_cap = cap;
  a.k_new = k_new; a.v_new = v_new; a.pos = pos;
  a.k_cache = k_pages; a.v_cache = v_pages;
  a.pages = pm;
  a.stream = (hipStream_t)stream;
  return to_status(dqkv::launch_kv_append(a));
}

int32_t diffqkv_decode_paged(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                             int32_t dtype, int32_t batch, int32_t page_rows,
                             int32_t num_pages, int32_t max_blocks, int32_t max_ctx,
                             float scale, const void* q, const void* k_new, const void* v_new,
                             void* k_pages, void* v_pages, const int32_t* block_table,
                             const int32_t* ctx_len, void* out, float* lse,
                             int32_t chunk_tokens, void* workspace,
                             size_t workspace_bytes_given, void* stream) {
  dqkv::PageMap pm;
  int cap = 0;
  int st = check_pages(page_rows, num_pages, max_blocks, block_table, &pm, &cap);
  if (st) return st;
  if (batch == 0 && n_q > 0) {
    st = check_heads(n_q, n_k, n_v, d_k, d_v);
    return st ? st : check_dtype_dims(dtype, d_k, d_v);
  }
  if ((k_new == nullptr) != (v_new == nullptr)) return DQKV_ERR_NULL;
  if (!block_table) return DQKV_ERR_NULL;
  dqkv::DecodeArgs a;
  st = prepare_decode(n_q, n_k, n_v, d_k, d_v, dtype, batch, cap, max_ctx, scale, q, k_pages,
                      v_pages, ctx_len, out, lse, chunk_tokens, workspace,
                      workspace_bytes_given, stream, true, true, &a, true);
  if (st) return st;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return DQKV_ERR_ALIGN;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pages = pm;
  st = to_status(dqkv::launch_decode_split(a));
  if (st) return st;
  return to_status(dqkv::launch_decode_combine(a));
}

// ------------------------------------------------------ kv_group_sharing

int32_t kv_group_sharing(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v,
                         int32_t dtype, int32_t batch, int32_t l_cap, const void* k_cache,
                         const void* v_cache, void* k_out, void* v_out, void* stream) {
  int st = check_heads(n_q, n_k, n_v, d_k, d_v);
  if (st) return st;
  st = check_dtype_dims(dtype, d_k, d_v);
  if (st) return st;
  if (batch < 0 || l_cap < 0 || batch > 65535) return DQKV_ERR_SHAPE;
  const int n_h = n_k > n_v ? n_k : n_v;
  if (n_h > 65535) return DQKV_ERR_UNSUPPORTED;
  if (batch == 0 || l_cap == 0) return DQKV_OK;
  if (!k_cache || !v_cache || !k_out || !v_out) return DQKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out))
    return DQKV_ERR_ALIGN;
  const size_t e = dtype == DQKV_BF16 ? 2 : 4;
  dqkv::ExpandArgs a;
  a.batch = batch;
  a.stream = (hipStream_t)stream;
  a.n_src = n_k; a.n_dst = n_h; a.head_bytes = (size_t)l_cap * d_k * e;
  a.src = k_cache; a.dst = k_out;
  st = to_status(dqkv::launch_expand_heads(a));
  if (st) return st;
  a.n_src = n_v; a.n_dst = n_h; a.head_bytes = (size_t)l_cap * d_v * e;
  a.src = v_cache; a.dst = v_out;
  return to_status(dqkv::launch_expand_heads(a));
}

// ------------------------------------------------------- augmented Q

int32_t augq_workspace(int32_t M, int32_t d_m, int32_t d_i, int32_t d_out, size_t* bytes) {
  if (!bytes) return DQKV_ERR_NULL;
  if (M < 0 || d_m <= 0 || d_i <= 0 || d_out <= 0) return DQKV_ERR_SHAPE;
  *bytes = (size_t)M * d_i * 2;
  return DQKV_OK;
}

int32_t augq_forward(int32_t M, int32_t d_m, int32_t d_i, int32_t d_out, const void* h,
                     const void* w_gate, const void* w_up, const void* w_down, void* q,
                     void* workspace, size_t workspace_bytes_given, void* stream) {
  if (M < 0 || d_m <= 0 || d_i <= 0 || d_out <= 0) return DQKV_ERR_SHAPE;
  // Reductions split up to sixteen ways in 32-wide steps; outputs in
  // 16-column tiles.
  if (d_m % 1024 != 0 || d_i % 1024 != 0 || d_i % 16 != 0 || d_out % 16 != 0)
    return DQKV_ERR_UNSUPPORTED;
  if ((long long)d_i / 16 > 0x7fffffffLL || (M + 15) / 16 > 65535) return DQKV_ERR_UNSUPPORTED;
  if (M == 0) return DQKV_OK;
  if (!h || !w_gate || !w_up || !w_down || !q || !workspace) return DQKV_ERR_NULL;
  if (!aligned16(h) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(q) || !aligned16(workspace))
    return DQKV_ERR_ALIGN;
  if (workspace_bytes_given < (size_t)M * d_i * 2) return DQKV_ERR_WORKSPACE;
  dqkv::AugQArgs a;
  a.M = M; a.d_m = d_m; a.d_i = d_i; a.d_out = d_out;
  a.h = h; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down;
  a.act = workspace; a.q = q;
  a.stream = (hipStream_t)stream;
  return to_status(dqkv::launch_augq(a));
}

int32_t augq_pack(int32_t n_out, int32_t n_in, const void* w, void* w_packed, void* stream) {
  if (n_out < 0 || n_in < 0) return DQKV_ERR_SHAPE;
  if (n_out % 16 != 0 || n_in % 32 != 0) return DQKV_ERR_UNSUPPORTED;
  if (n_out == 0 || n_in == 0) return DQKV_OK;
  if (!w || !w_packed) return DQKV_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_packed)) return DQKV_ERR_ALIGN;
  return to_status(dqkv::launch_augq_pack(w, w_packed, n_out, n_in, (hipStream_t)stream));
}

}  // extern "C"
