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
// Two kernel templates compute C[M][N] = A[M][K] . B[N][K]^T on the matrix
// cores.  For a few rows (decode sizes) the streaming kernel: the 16-byte
// loads of A rows (lane l = row l % 16, elements 8 (l / 16) .. +7 of a
// 32-wide step) and of packed B fragments are the MFMA operands as they
// arrive, so nothing is staged through LDS.  A workgroup owns 16 output
// columns and 16 * MT rows; its waves split the reduction and meet in LDS,
// where wave 0 adds the parts and applies the epilogue.  For the gate/up
// product the workgroup computes the gate and up tiles of the same columns
// and writes silu(g) * u.  At decode sizes (M = a few tokens) the kernel
// streams the weights once, each wave with all loads of its slice in flight.
// For more rows the LDS-tiled kernel below.

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace dqkv {

typedef __bf16 aq_bf16x8 __attribute__((ext_vector_type(8)));

// W = waves splitting the reduction; STEPS = 32-wide reduction steps whose
// loads are issued together (a wave's whole slice at decode sizes).
// CHUNKED_IN / CHUNKED_OUT (MT = 1 only, so M <= 16): A, resp. C, is stored
// chunk-major, [cols / 8][M][8] -- element (r, c) at ((c / 8) M + r) 8 + c % 8
// -- so that the 16 x 32 A operand of one step is M x 64 contiguous bytes (a
// row-major A gives 16-byte pieces of rows K elements apart, and every load
// touches a cache line per row).  The gate/up product writes the gated
// intermediate this way for the down product.  STAGE_A (MT = 1, row-major A,
// slices of at most 128 columns in one round; chosen for more than 8 rows):
// each wave loads its 16 x kq slice of A as whole 2 kq-byte row pieces, four
// rows per load, into its own LDS rows and reads the operands from there (16
// tokens: 14.7 -> 14.2 us per call; up to 8 rows the direct loads are
// 0.1-0.2 us faster).
template <int MT, bool SWIGLU, int W, int STEPS, bool CHUNKED_IN = false,
          bool CHUNKED_OUT = false, bool STAGE_A = false>
__global__ __launch_bounds__(64 * W) void augq_gemm_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B0, const bf16* __restrict__ B1,
    bf16* __restrict__ C, int M, int N, int K) {
  static_assert(MT == 1 || !(CHUNKED_IN || CHUNKED_OUT), "chunked layout: one row tile");
  static_assert(!STAGE_A || (MT == 1 && !CHUNKED_IN), "staging: one row tile, row-major A");
  constexpr int NP = SWIGLU ? 2 : 1;  // products per tile
  __shared__ f32x4 part[W - 1][MT][NP][64];
  constexpr int kSC = 128, kSP = kSC + 8;  // staged columns per row, row pitch (bf16)
  __shared__ __align__(16) __bf16 astage[STAGE_A ? W : 1][16][kSP];

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
    ap[mt] = CHUNKED_IN ? A + ((size_t)kg * M + (arow[mt] ? row : 0)) * 8
                        : A + (size_t)(arow[mt] ? row : 0) * K + 8 * kg;
  }

  f32x4 acc[MT][NP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[mt][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool staged = STAGE_A && kq <= kSC && kq <= 32 * STEPS;  // checked on the host too
  for (int k0 = kbeg; k0 < kend; k0 += 32 * STEPS) {
    u32x4 bv[NP][STEPS], av[MT][STEPS];
    u32x4 sv[4];
    const int ncr = kq / 8;  // 16-byte chunks per staged row
    if (staged) {  // one round (kq <= 32 STEPS): the wave's whole A slice
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = i * 64 + lane, row = idx / ncr, c = idx % ncr;
        sv[i] = idx < 16 * ncr && m0 + row < M ? load16(A + (size_t)(m0 + row) * K + kbeg + 8 * c)
                                                : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const bool ok = k0 + 32 * s < kend;
      const size_t fo = (size_t)((k0 >> 5) + s) * 512;  // fragment (k0 / 32 + s)
      bv[0][s] = ok ? load16_nt(b0p + fo) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (SWIGLU)
        bv[NP - 1][s] = ok ? load16_nt(b1p + fo) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const size_t ao = CHUNKED_IN ? (size_t)((k0 + 32 * s) / 8) * M * 8 : (size_t)(k0 + 32 * s);
        av[mt][s] = !staged && ok && arow[mt] ? load16(ap[mt] + ao) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (staged) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = i * 64 + lane, row = idx / ncr, c = idx % ncr;
        if (idx < 16 * ncr)
          *reinterpret_cast<u32x4*>(&astage[STAGE_A ? wave : 0][row][8 * c]) = sv[i];
      }
#pragma unroll
      for (int s = 0; s < STEPS; ++s)
        if (32 * s < kq)
          av[0][s] =
              *reinterpret_cast<const u32x4*>(&astage[STAGE_A ? wave : 0][l16][32 * s + 8 * kg]);
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
      const int col = n0 + l16;
      if constexpr (CHUNKED_OUT)
        C[((size_t)(col >> 3) * M + row) * 8 + (col & 7)] = Elem<bf16>::from_f32(v);
      else
        C[(size_t)row * N + col] = Elem<bf16>::from_f32(v);
    }
  }
}

template <int MT, bool SWIGLU, int W, int STEPS, bool CHUNKED_IN = false,
          bool CHUNKED_OUT = false, bool STAGE_A = false>
static hipError_t launch_gemm(const bf16* A, const bf16* B0, const bf16* B1, bf16* C, int M,
                              int N, int K, hipStream_t stream) {
  dim3 grid(N / 16, (M + 16 * MT - 1) / (16 * MT));
  hipLaunchKernelGGL((augq_gemm_kernel<MT, SWIGLU, W, STEPS, CHUNKED_IN, CHUNKED_OUT, STAGE_A>),
                     grid, dim3(64 * W), 0, stream, A, B0, B1, C, M, N, K);
  return hipGetLastError();
}

// ------------------------------------------------------------ tiled product
// Larger M: C[M][N] = A[M][K] . B[N][K]^T with both operands staged in LDS.
// A workgroup (4 or 8 waves) owns BN weight rows x BM activation rows and
// walks the reduction in 64-wide stages through S LDS buffers, every load
// going from HBM straight into LDS (16-byte global_load_lds, issued through
// asm so that only the kernel's own waits order them: lane l of a wave
// instruction fills bytes 16 l .. 16 l + 15 of a 1 KiB block).
//   * Weights: one instruction = one packed 1 KiB fragment (16 rows x 32
//     reduction elements, contiguous in the packed weights); in LDS a
//     16-lane group reads 256 contiguous bytes per operand.
//   * Activations: one instruction = 8 rows x 128 bytes (full cache lines);
//     LDS holds the rows row-major, logical 16-byte slot c of row r at
//     physical slot c ^ ((r / 2) & 7) (the loads permute their sources), so
//     the 16 rows an operand read serves at once meet 16 different 16-byte
//     positions of the 64-bank LDS.
// The matrix cores compute D = W_tile . A_tile^T, so lane l holds output
// row m = l % 16 and four consecutive output columns 4 (l / 16) .. +3, stored
// as 8 bytes.  For the gate/up product a wave's NF weight blocks are NF / 2
// gate blocks followed by the up blocks of the same output columns, so
// silu(g) * u pairs accumulators of the same lane and register.
// s_waitcnt encoding (gfx9 family): vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their maxima (no wait).
template <int N>
struct VmWait {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  static constexpr int kImm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
};

// BK = reduction elements per stage (64: one cache line per activation row),
// S = LDS stages; the loads of stage k + S - 1 are issued while stage k is
// multiplied.
template <bool SWIGLU, int BN, int BM, int WN, int WM, int BK, int S>
__global__ __launch_bounds__(64 * WN * WM) void augq_tiled_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B0, const bf16* __restrict__ B1,
    bf16* __restrict__ C, int M, int N, int K, int n_mtiles) {
  constexpr int NW = WN * WM;               // waves per workgroup
  static_assert((NW == 4 || NW == 8) && BK == 64 && S >= 2, "tile shape");
  constexpr int KB = BK / 32;               // 32-wide blocks per stage
  constexpr int NF = BN / WN / 16;          // weight blocks per wave
  constexpr int MF = BM / WM / 16;          // activation blocks per wave
  constexpr int BFR = BN / 16 * KB;         // weight fragments per stage
  constexpr int AFR = BM / 16 * KB;         // activation fragments per stage
  constexpr int FR = BFR + AFR;
  constexpr int STAGE = FR * 1024;          // bytes
  constexpr int LPW = FR / NW;              // fragment loads per wave per stage
  static_assert(FR % NW == 0 && (!SWIGLU || NF % 2 == 0), "tile shape");
  __shared__ __attribute__((aligned(16))) unsigned char lds[S * STAGE];

  // Consecutive logical tiles share a weight stripe; the renumbering puts
  // them on one XCD (dispatch is round-robin over 8 XCDs) to share its L2.
  const int nwg = gridDim.x, id = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (id % 8) * (nwg / 8) + id / 8 : id;
  const int mt = logical % n_mtiles, nt = logical / n_mtiles;
  const int m0 = mt * BM;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int kb_n = K / 32;

  // Sources of this wave's fragment loads (fragments wave, wave + NW, ...) at
  // stage 0; a stage advances weights by KB fragments (512 elements each)
  // and activations by BK elements.
  const bf16* src[LPW];
  bool is_w[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int f = wave + NW * u;
    if (f < BFR) {
      const int nbl = f / KB, kbl = f % KB;  // local 16-row weight block, k block
      const bf16* Bsrc = B0;
      int nb;
      if constexpr (SWIGLU) {
        const int g = nbl / NF, j = nbl % NF;   // wave-n group, block within it
        Bsrc = j < NF / 2 ? B0 : B1;
        nb = nt * (BN / 32) + g * (NF / 2) + j % (NF / 2);
      } else {
        nb = nt * (BN / 16) + nbl;
      }
      src[u] = Bsrc + ((size_t)nb * kb_n + kbl) * 512 + lane * 8;
      is_w[u] = true;
    } else {
      // Activation load a: rows 8a .. 8a + 7 of the tile, 128 bytes each;
      // lane l fills LDS slot l % 8 of row r = 8a + l / 8, which holds the
      // row's logical 16-byte slot (l % 8) ^ ((r / 2) & 7).
      const int a = f - BFR;
      const int r = 8 * a + (lane >> 3);
      const int row = min(m0 + r, M - 1);
      src[u] = A + (size_t)row * K + 8 * ((lane & 7) ^ ((r >> 1) & 7));
      is_w[u] = false;
    }
  }
  auto issue = [&](int kt, int stage) {
    unsigned char* dst = lds + stage * STAGE;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const size_t adv = is_w[u] ? (size_t)kt * KB * 512 : (size_t)kt * BK;
      dma16(src[u] + adv, (lds_dma_t*)(dst + (wave + NW * u) * 1024));
    }
  };

  f32x4 acc[NF][MF];
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int j = 0; j < MF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  // A wave's operands of stage kt (16-byte LDS reads into registers).
  auto read_ops = [&](int kt, aq_bf16x8 (&wf)[KB][NF], aq_bf16x8 (&af)[KB][MF]) {
    const int st = kt % S;
    const unsigned char* base = lds + st * STAGE + lane * 16;
#pragma unroll
    for (int s = 0; s < KB; ++s) {
#pragma unroll
      for (int i = 0; i < NF; ++i)
        wf[s][i] = *reinterpret_cast<const aq_bf16x8*>(base + ((wn * NF + i) * KB + s) * 1024);
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        const int r = (wm * MF + j) * 16 + (lane & 15), c = 4 * s + (lane >> 4);
        af[s][j] = *reinterpret_cast<const aq_bf16x8*>(lds + st * STAGE + BFR * 1024 + r * 128 +
                                                      ((c ^ ((r >> 1) & 7)) << 4));
      }
    }
  };
  auto mul = [&](const aq_bf16x8 (&wf)[KB][NF], const aq_bf16x8 (&af)[KB][MF]) {
#pragma unroll
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < MF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s][i], af[s][j], acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
    if (k < nk) issue(k, k);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed for this wave (the loads of the S - 2 later
    // stages may still be in flight; near the end wait for everything),
    // then for every wave, and every wave is done with the buffer that
    // receives stage kt + S - 1.
    if (kt + S - 2 < nk) __builtin_amdgcn_s_waitcnt(VmWait<(S - 2) * LPW>::kImm);
    else __builtin_amdgcn_s_waitcnt(VmWait<0>::kImm);
    __syncthreads();
    if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
    // All operands of the stage are read first, then multiplied.
    aq_bf16x8 wf[KB][NF], af[KB][MF];
    read_ops(kt, wf, af);
    __builtin_amdgcn_sched_barrier(0);
    mul(wf, af);
  }

  // D[n][m]: lane l holds m = l % 16 and n = 4 (l / 16) .. +3 of its block.
  const int l16 = lane & 15, q4 = 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < MF; ++j) {
    const int m = m0 + (wm * MF + j) * 16 + l16;
    if (m >= M) continue;
    constexpr int NO = SWIGLU ? NF / 2 : NF;  // output blocks per wave
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (SWIGLU) {
          const float g = acc[i][j][e];
          v[e] = g / (1.f + fast_exp2(-g * kLog2e)) * acc[i + NF / 2][j][e];
        } else {
          v[e] = acc[i][j][e];
        }
      }
      const int n = SWIGLU ? nt * (BN / 2) + (wn * NO + i) * 16 + q4
                           : nt * BN + (wn * NF + i) * 16 + q4;
      const uint32_t w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(C + (size_t)m * N + n) = make_uint2(w0, w1);
    }
  }
}

template <bool SWIGLU, int BN, int BM, int WN, int WM, int BK, int S>
static hipError_t launch_tiled(const bf16* A, const bf16* B0, const bf16* B1, bf16* C, int M,
                               int N, int K, hipStream_t stream) {
  constexpr int OUT_N = SWIGLU ? BN / 2 : BN;  // output columns per tile
  const int n_mtiles = (M + BM - 1) / BM;
  const long long tiles = (long long)n_mtiles * (N / OUT_N);
  hipLaunchKernelGGL((augq_tiled_kernel<SWIGLU, BN, BM, WN, WM, BK, S>), dim3((unsigned)tiles),
                     dim3(64 * WN * WM), 0, stream, A, B0, B1, C, M, N, K, n_mtiles);
  return hipGetLastError();
}

// Decode sizes (M <= 16): 16 rows per workgroup and sixteen waves on the
// reduction, each issuing all loads of its slice (up to 8 steps) at once, so
// the weights stream in about one memory round trip; the gated intermediate
// passes between the two products chunk-major (at 16 tokens: 15.8 -> 14.9 us
// per call, same process).  Up to 64 rows: 64 rows
// per workgroup (each weight load feeds four products), eight waves, four
// steps per round.  Beyond that the LDS-tiled product: from 1024 rows eight
// waves per workgroup on 192 x 256 gate/up tiles (96 output columns) and
// 128 x 128 down tiles with four stages; below, four waves on 128 x 128
// gate/up tiles (64 output columns) and 64 x 128 down tiles.  Widths that
// do not divide into whole tiles take the 64-row kernel.
template <bool SWIGLU>
static hipError_t gemm(const bf16* A, const bf16* B0, const bf16* B1, bf16* C, int M, int N,
                       int K, hipStream_t stream) {
  if (M <= 16) {
    // The staged gate/up product takes 4 steps per round (d_m = 2048: one
    // round, registers left for the staging).
    if constexpr (SWIGLU) {
      if (M > 8 && K / 16 <= 128)
        return launch_gemm<1, true, 16, 4, false, true, true>(A, B0, B1, C, M, N, K, stream);
    }
    return launch_gemm<1, SWIGLU, 16, 8, !SWIGLU, SWIGLU>(A, B0, B1, C, M, N, K, stream);
  }
  if (M > 64 && K % 64 == 0) {
    const bool big = M >= 1024;
    if constexpr (SWIGLU) {
      if (big && N % 96 == 0)
        return launch_tiled<true, 192, 256, 2, 4, 64, 2>(A, B0, B1, C, M, N, K, stream);
      if (N % 64 == 0)
        return launch_tiled<true, 128, 128, 2, 2, 64, 2>(A, B0, B1, C, M, N, K, stream);
    } else {
      if (big && N % 128 == 0)
        return launch_tiled<false, 128, 128, 2, 4, 64, 4>(A, B0, B1, C, M, N, K, stream);
      if (N % 64 == 0)
        return launch_tiled<false, 64, 128, 1, 4, 64, 2>(A, B0, B1, C, M, N, K, stream);
    }
  }
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
