// kv_append: Step 2 of the Sigma architecture page's section 3.4,
// K_t = [K_{t-1}; k_t] and V_t = [V_{t-1}; v_t], into the separate K and V
// caches (section 3.2 item 3), each with its own head count and head
// dimension.  Token-major new rows [B][t_new][n_h][d] are scattered to the
// head-major caches [B][n_h][l_cap][d] at row pos[b] + t, or into a paged
// cache through its page table.  Also the kv_group_sharing head expansion.
// Pure copies in 16-byte units: bit-exact by construction.
#include "device_common.h"
#include "launch.h"

namespace dqkv {

// One workgroup per (token, sequence); its threads copy the token's K row
// (n_k * d_k elements) and V row (n_v * d_v elements).  With a page table the
// row goes to its page and slot; rows whose page index falls outside the
// table, or whose table entry is not a page, are skipped like rows past
// l_cap.
__global__ __launch_bounds__(256) void kv_append_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    const int32_t* __restrict__ pos, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int n_k, int n_v, int k16, int v16, int t_new,
    int l_cap, PageMap pm) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int p0 = pos[b];
  const long long row = (long long)p0 + t;
  if (p0 < 0 || row >= l_cap) return;  // destination outside the cache
  long long base_row;  // row index in units of head rows within the head's plane
  int plane;           // rows per head plane: l_cap, or the page size
  size_t unit;         // sequence (contiguous) or page (paged) holding the row
  if (pm.table != nullptr) {
    const long long blk_i = row >> pm.page_shift;
    if (blk_i >= pm.max_blocks) return;
    const int page = pm.table[(size_t)b * pm.max_blocks + blk_i];
    if (page < 0 || page >= pm.num_pages) return;
    unit = (size_t)page;
    plane = 1 << pm.page_shift;
    base_row = row & (plane - 1);
  } else {
    unit = (size_t)b;
    plane = l_cap;
    base_row = row;
  }
  const int kn = n_k * k16, vn = n_v * v16;
  const u32x4* ks = k_new + ((size_t)b * t_new + t) * kn;
  const u32x4* vs = v_new + ((size_t)b * t_new + t) * vn;
  for (int e = threadIdx.x; e < kn; e += blockDim.x) {
    const int h = e / k16, x = e - h * k16;
    k_cache[((unit * n_k + h) * plane + base_row) * k16 + x] = ks[e];
  }
  for (int e = threadIdx.x; e < vn; e += blockDim.x) {
    const int h = e / v16, x = e - h * v16;
    v_cache[((unit * n_v + h) * plane + base_row) * v16 + x] = vs[e];
  }
}

hipError_t launch_kv_append(const AppendArgs& a) {
  if (a.batch == 0 || a.t_new == 0) return hipSuccess;
  const int k16 = a.d_k * a.elem_bytes / 16, v16 = a.d_v * a.elem_bytes / 16;
  dim3 grid(a.t_new, a.batch);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(256), 0, a.stream,
                     (const u32x4*)a.k_new, (const u32x4*)a.v_new, a.pos,
                     (u32x4*)a.k_cache, (u32x4*)a.v_cache, a.n_k, a.n_v, k16, v16,
                     a.t_new, a.l_cap, a.pages);
  return hipGetLastError();
}

// kv_group_sharing (architecture page, FlexHeadFA section): destination head
// h of sequence b copies source head floor(h * n_src / n_dst), 16 bytes per
// thread, grid-stride over the head's bytes.
__global__ __launch_bounds__(256) void expand_heads_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int n_src,
                                                          int n_dst, size_t head16) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int hs = (int)(((long long)h * n_src) / n_dst);
  const u32x4* s = src + ((size_t)b * n_src + hs) * head16;
  u32x4* d = dst + ((size_t)b * n_dst + h) * head16;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < head16;
       x += (size_t)gridDim.x * blockDim.x)
    d[x] = s[x];
}

hipError_t launch_expand_heads(const ExpandArgs& a) {
  if (a.batch == 0 || a.head_bytes == 0) return hipSuccess;
  const size_t head16 = a.head_bytes / 16;
  size_t gx = (head16 + 255) / 256;
  if (gx > 1024) gx = 1024;
  dim3 grid((unsigned)gx, a.n_dst, a.batch);
  hipLaunchKernelGGL(expand_heads_kernel, grid, dim3(256), 0, a.stream, (const u32x4*)a.src,
                     (u32x4*)a.dst, a.n_src, a.n_dst, head16);
  return hipGetLastError();
}

}  // namespace dqkv
