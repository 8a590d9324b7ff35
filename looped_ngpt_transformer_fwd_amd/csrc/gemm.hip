// bf16 GEMM on gfx950 MFMA (v_mfma_f32_32x32x16_bf16) for the dense
// projections of the forward pass: fused q/k/v/gate, attention output,
// SwiGLU up/gate (with the activation fused into the epilogue), MLP down
// projection and the LM head (with the logit scale fused).
//
// C[m, n] = sum_k A[m, k] * B[n, k]. A is the activation (row-major,
// K-contiguous), B the weight in [out, in] layout (also K-contiguous), so
// both operand tiles are loaded along K with 16-byte vector loads.
//
// Tiling: BM x BN output tile per workgroup, BK = 64, waves arranged
// (BM/WM) x (BN/WN), each wave owning a WM x WN sub-tile of 32x32 MFMA
// blocks. Operand tiles are staged through LDS with a 16-byte row pad
// (row stride 144 B) so that the 16-byte fragment reads of 8 consecutive
// rows hit distinct banks. Two LDS stages: the global loads of tile t+1 are
// issued before the MFMAs of tile t and written to the other stage after
// them, one barrier per K step.
#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

constexpr int BK = 64;
constexpr int ROW_BYTES = BK * 2 + 16;  // padded LDS row

template <int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(64 * (BM / WM) * (BN / WN))
gemm_nt_kernel(GemmArgs g) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NT = 64 * (BM / WM) * WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_LD = BM * 8 / NT;  // 16-byte chunks per thread
  constexpr int B_LD = BN * 8 / NT;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the block");
  static_assert(EPI != EPI_SWIGLU || (FN % 2) == 0, "swiglu pairs 32-col blocks");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * ROW_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int ntn = (g.N + BN - 1) / BN;
  const int tile = blockIdx.x;
  const int tm = tile / ntn, tn = tile % ntn;
  const int m0 = tm * BM, n0 = tn * BN;

  // K range of this split
  const int ksteps = g.K / BK;
  const int per = (ksteps + g.nsplit - 1) / g.nsplit;
  const int ks0 = blockIdx.z * per;
  const int ks1 = min(ksteps, ks0 + per);

  // per-thread global source rows
  const int kc = tid & 7;  // 16-byte chunk within the 128-byte K slice
  const uint16_t* a_src[A_LD];
  const uint16_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    int r = (tid >> 3) + i * (NT / 8);
    int gm = min(m0 + r, g.M - 1);
    a_src[i] = g.A + (int64_t)gm * g.lda + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    int r = (tid >> 3) + i * (NT / 8);
    int v = min(n0 + r, g.N - 1);
    int row = v;
    if (EPI == EPI_SWIGLU) {
      // 32-column blocks alternate up / gate for the same 32 features
      int f = ((v >> 6) << 5) | (v & 31);
      row = (v & 32) ? g.F + f : f;
    }
    b_src[i] = g.B + (int64_t)row * g.ldb + kc * 8;
  }

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint4 ra[A_LD], rb[B_LD];
  auto gload = [&](int ks) {
    const int koff = ks * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + koff);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + koff);
  };
  auto sstore = [&](int stage) {
    uint8_t* sa = smem + stage * (BM + BN) * ROW_BYTES;
    uint8_t* sb = sa + BM * ROW_BYTES;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      int r = (tid >> 3) + i * (NT / 8);
      *reinterpret_cast<uint4*>(sa + r * ROW_BYTES + kc * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      int r = (tid >> 3) + i * (NT / 8);
      *reinterpret_cast<uint4*>(sb + r * ROW_BYTES + kc * 16) = rb[i];
    }
  };

  const int frow = lane & 31;   // fragment row (A) / column (B)
  const int fk = lane >> 5;     // which 8-element half of the 16-wide k step

  if (ks0 < ks1) {
    gload(ks0);
    sstore(0);
    __syncthreads();
    for (int ks = ks0; ks < ks1; ++ks) {
      const int stage = (ks - ks0) & 1;
      const bool more = ks + 1 < ks1;
      if (more) gload(ks + 1);
      const uint8_t* sa = smem + stage * (BM + BN) * ROW_BYTES;
      const uint8_t* sb = sa + BM * ROW_BYTES;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[FM], bfr[FN];
        const int cb = (kk * 2 + fk) * 16;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(sa + (wm * WM + i * 32 + frow) * ROW_BYTES + cb);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (wn * WN + j * 32 + frow) * ROW_BYTES + cb);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (more) sstore(stage ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue. Output layout of a 32x32 block: lane holds column
  // (lane & 31) and rows (e/4)*8 + (lane/32)*4 + (e%4), e = 0..15.
  const int rbase = m0 + wm * WM + (lane >> 5) * 4;
  const int cbase = n0 + wn * WN + (lane & 31);
  if (EPI == EPI_F32 || EPI == EPI_LOGITS) {
    float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = cbase + j * 32;
      if (col >= g.N) continue;
      const float sc = (EPI == EPI_LOGITS) ? g.s1[col] : 1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + (e >> 2) * 8 + (e & 3);
          if (row < g.M) C[(int64_t)row * g.ldc + col] = acc[i][j][e] * sc;
        }
    }
  } else {
#pragma unroll
    for (int jp = 0; jp < FN / 2; ++jp) {
      const int v = cbase + jp * 64;  // virtual column of the up half
      if (v >= g.N) continue;
      const int f = ((v >> 6) << 5) | (v & 31);
      const float su = g.s1[f], sv = g.s2[f];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + (e >> 2) * 8 + (e & 3);
          if (row < g.M) {
            const float up = acc[i][2 * jp][e] * su;
            const float gt = acc[i][2 * jp + 1][e] * sv;
            const float act = gt / (1.f + __expf(-gt));
            g.C16[(int64_t)row * g.ldc16 + f] = f2bf(act * up);
          }
        }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, int epi, hipStream_t st) {
  constexpr int NT = 64 * (BM / WM) * (BN / WN);
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(tiles, 1, a.nsplit), block(NT);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WM, WN, EPI_F32>), grid, block, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WM, WN, EPI_SWIGLU>), grid, block, 0, st, a); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WM, WN, EPI_LOGITS>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr int kLargeM = 1024;

}  // namespace

int gemm_pick_split(int M, int N, int K, int max_split) {
  if (M >= kLargeM) return 1;
  const int tiles = ((M + 63) / 64) * ((N + 127) / 128);
  const int ksteps = K / BK;
  int s = 1;
  while (s * 2 <= max_split && tiles * s < 512 && ksteps / (s * 2) >= 4) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  if (a.K % BK != 0 || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
  if (epi != EPI_F32 && a.nsplit != 1) return hipErrorInvalidValue;
  if (a.M >= kLargeM) return launch_cfg<256, 256, 64, 128>(a, epi, st);
  return launch_cfg<64, 128, 32, 64>(a, epi, st);
}

}  // namespace dory
