// Augmented-Q projection (Sigma architecture page, section 3.2 item 4:
// Augmented Q with SwiGLU gating):
//   a = silu(h W_gate^T) * (h W_up^T)      [M][d_i]   (bf16, rounded once)
//   q = a W_down^T                          [M][d_out]
// with weights in (out, in) layout, so both operands of every product are
// contiguous along the reduction dimension.
//
// Weights are packed once (augq_pack_kernel) into matrix-core fragment order:
// Wp[N / 16][K / 32][64 lanes][8], lane l of fragment (nb, kb) holding
// W[16 nb + l % 16][32 kb + 8 (l / 16) .. +7] -- exactly the B operand of
// v_mfma_f32_16x16x32_bf16.  A wave then loads a fragment as 1 KiB of
// contiguous memory (eight full cache lines) instead of 64-byte pieces of
// sixteen rows, which is what lets the weight stream reach HBM speed.
//
// One kernel template, C[M][N] = A[M][K] . B[N][K]^T on the matrix cores: the
// 16-byte loads of A rows (lane l = row l % 16, elements 8 (l / 16) .. +7 of
// a 32-wide step) and of packed B fragments are the MFMA operands as they
// arrive, so nothing is staged through LDS.  A workgroup owns 16 output
// columns and 16 * MT rows; its waves split the reduction and meet in LDS,
// where wave 0 adds the parts and applies the epilogue.  For the gate/up
// product the workgroup computes the gate and up tiles of the same columns
// and writes silu(g) * u.  At decode sizes (M = a few tokens) the kernel
// streams the weights once, each wave with all loads of its slice in flight.

#include "device_common.h"
#include "launch.h"

namespace dqkv {

typedef __bf16 aq_bf16x8 __attribute__((ext_vector_type(8)));

// W = waves splitting the reduction; STEPS = 32-wide reduction steps whose
// loads are issued together (a wave's whole slice at decode sizes).
template <int MT, bool SWIGLU, int W, int STEPS>
__global__ __launch_bounds__(64 * W) void augq_gemm_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B0, const bf16* __restrict__ B1,
    bf16* __restrict__ C, int M, int N, int K) {
  constexpr int NP = SWIGLU ? 2 : 1;  // products per tile
  __shared__ f32x4 part[W - 1][MT][NP][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16 * MT;
  const int l16 = lane & 15, kg = lane >> 4;
  const int kq = K / W;  // a multiple of 32 (checked on the host)
  const int kbeg = wave * kq, kend = kbeg + kq;

  // Packed fragments of this workgroup's 16 columns: fragment kb at
  // (blockIdx.x * (K / 32) + kb) * 512 elements, this lane's 8 at lane * 8.
  const size_t frag0 = (size_t)blockIdx.x * (K / 32) * 512 + lane * 8;
  const bf16* b0p = B0 + frag0;
  const bf16* b1p = SWIGLU ? B1 + frag0 : nullptr;
  const bf16* ap[MT];
  bool arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = m0 + mt * 16 + l16;
    arow[mt] = row < M;
    ap[mt] = A + (size_t)(arow[mt] ? row : 0) * K + 8 * kg;
  }

  f32x4 acc[MT][NP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[mt][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kend; k0 += 32 * STEPS) {
    u32x4 bv[NP][STEPS], av[MT][STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const bool ok = k0 + 32 * s < kend;
      const size_t fo = (size_t)((k0 >> 5) + s) * 512;  // fragment (k0 / 32 + s)
      bv[0][s] = ok ? load16_nt(b0p + fo) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (SWIGLU)
        bv[NP - 1][s] = ok ? load16_nt(b1p + fo) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        av[mt][s] = ok && arow[mt] ? load16(ap[mt] + k0 + 32 * s) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          acc[mt][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(aq_bf16x8, av[mt][s]), __builtin_bit_cast(aq_bf16x8, bv[p][s]),
              acc[mt][p], 0, 0, 0);
  }

  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p = 0; p < NP; ++p) part[wave - 1][mt][p][lane] = acc[mt][p];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < W - 1; ++w)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p = 0; p < NP; ++p) acc[mt][p] += part[w][mt][p][lane];

  // D layout: lane l holds output column n0 + l % 16, rows 4 (l / 16) .. +3.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + mt * 16 + 4 * kg + e;
      if (row >= M) continue;
      float v;
      if constexpr (SWIGLU) {
        const float g = acc[mt][0][e];
        v = g / (1.f + fast_exp2(-g * kLog2e)) * acc[mt][1][e];
      } else {
        v = acc[mt][0][e];
      }
      C[(size_t)row * N + n0 + l16] = Elem<bf16>::from_f32(v);
    }
  }
}

template <int MT, bool SWIGLU, int W, int STEPS>
static hipError_t launch_gemm(const bf16* A, const bf16* B0, const bf16* B1, bf16* C, int M,
                              int N, int K, hipStream_t stream) {
  dim3 grid(N / 16, (M + 16 * MT - 1) / (16 * MT));
  hipLaunchKernelGGL((augq_gemm_kernel<MT, SWIGLU, W, STEPS>), grid, dim3(64 * W), 0, stream, A,
                     B0, B1, C, M, N, K);
  return hipGetLastError();
}

// Decode sizes (M <= 16): 16 rows per workgroup and sixteen waves on the
// reduction, each issuing all loads of its slice (up to 8 steps) at once, so
// the weights stream in about one memory round trip.  Larger M: 64 rows per
// workgroup (each weight load feeds four products), eight waves, four steps
// per round.
template <bool SWIGLU>
static hipError_t gemm(const bf16* A, const bf16* B0, const bf16* B1, bf16* C, int M, int N,
                       int K, hipStream_t stream) {
  if (M <= 16) return launch_gemm<1, SWIGLU, 16, 8>(A, B0, B1, C, M, N, K, stream);
  return launch_gemm<4, SWIGLU, 8, 4>(A, B0, B1, C, M, N, K, stream);
}

// W [N][K] -> Wp [N / 16][K / 32][64][8]: one 16-byte lane slice per
// thread, grid-stride.
__global__ __launch_bounds__(256) void augq_pack_kernel(const u32x4* __restrict__ w,
                                                        u32x4* __restrict__ wp, int N, int K) {
  const size_t total = (size_t)N * K / 8;
  const int kb_n = K / 32;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
       x += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(x & 63);
    const size_t frag = x >> 6;
    const int kb = (int)(frag % kb_n);
    const int nb = (int)(frag / kb_n);
    const int row = nb * 16 + (lane & 15), k = kb * 32 + 8 * (lane >> 4);
    wp[x] = w[((size_t)row * K + k) / 8];
  }
}

hipError_t launch_augq_pack(const void* w, void* wp, int N, int K, hipStream_t stream) {
  const size_t total = (size_t)N * K / 8;
  if (total == 0) return hipSuccess;
  size_t g = (total + 255) / 256;
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(augq_pack_kernel, dim3((unsigned)g), dim3(256), 0, stream,
                     (const u32x4*)w, (u32x4*)wp, N, K);
  return hipGetLastError();
}

hipError_t launch_augq(const AugQArgs& a) {
  if (a.M == 0) return hipSuccess;
  hipError_t e = gemm<true>((const bf16*)a.h, (const bf16*)a.w_gate, (const bf16*)a.w_up,
                            (bf16*)a.act, a.M, a.d_i, a.d_m, a.stream);
  if (e != hipSuccess) return e;
  return gemm<false>((const bf16*)a.act, (const bf16*)a.w_down, nullptr, (bf16*)a.q, a.M,
                     a.d_out, a.d_i, a.stream);
}

}  // namespace dqkv
