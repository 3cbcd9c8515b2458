// kv_append: Step 2 of the Sigma architecture page's section 3.4,
// K_t = [K_{t-1}; k_t] and V_t = [V_{t-1}; v_t], into the separate K and V
// caches (section 3.2 item 3), each with its own head count and head
// dimension.  Token-major new rows [B][t_new][n_h][d] are scattered to the
// head-major caches [B][n_h][l_cap][d] at row pos[b] + t.  A pure copy in
// 16-byte units: bit-exact by construction.
#include "device_common.h"
#include "launch.h"

namespace dqkv {

// One workgroup per (token, sequence); its threads copy the token's K row
// (n_k * d_k elements) and V row (n_v * d_v elements).
__global__ __launch_bounds__(256) void kv_append_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    const int32_t* __restrict__ pos, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int n_k, int n_v, int k16, int v16, int t_new,
    int l_cap) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int p0 = pos[b];
  const long long row = (long long)p0 + t;
  if (p0 < 0 || row >= l_cap) return;  // destination outside the cache
  const int kn = n_k * k16, vn = n_v * v16;
  const u32x4* ks = k_new + ((size_t)b * t_new + t) * kn;
  const u32x4* vs = v_new + ((size_t)b * t_new + t) * vn;
  for (int e = threadIdx.x; e < kn; e += blockDim.x) {
    const int h = e / k16, x = e - h * k16;
    k_cache[(((size_t)b * n_k + h) * l_cap + row) * k16 + x] = ks[e];
  }
  for (int e = threadIdx.x; e < vn; e += blockDim.x) {
    const int h = e / v16, x = e - h * v16;
    v_cache[(((size_t)b * n_v + h) * l_cap + row) * v16 + x] = vs[e];
  }
}

hipError_t launch_kv_append(const AppendArgs& a) {
  if (a.batch == 0 || a.t_new == 0) return hipSuccess;
  const int k16 = a.d_k * a.elem_bytes / 16, v16 = a.d_v * a.elem_bytes / 16;
  dim3 grid(a.t_new, a.batch);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(256), 0, a.stream,
                     (const u32x4*)a.k_new, (const u32x4*)a.v_new, a.pos,
                     (u32x4*)a.k_cache, (u32x4*)a.v_cache, a.n_k, a.n_v, k16, v16,
                     a.t_new, a.l_cap);
  return hipGetLastError();
}

}  // namespace dqkv
