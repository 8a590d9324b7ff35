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

// ---------------------------------------------------------------------------
// Large-M kernel: 256 x 256 x 64 tiles, 8 waves (4 x 2, each 64 x 128), two
// LDS stages filled by direct global->LDS DMA (global_load_lds_dwordx4), so
// no VGPRs stage the operands. Each 1 KiB DMA block holds 8 rows x 128 B;
// lane l of a block writes LDS bytes [16 l, 16 l + 16) and fetches logical
// 16-byte chunk (l % 8) ^ ((row / 2) % 8) of its row, i.e. the tile is
// stored XOR-swizzled. The LDS serves a 16-byte read for 16 lanes per cycle
// from its 64 banks (256 B); fragment reads of 16 consecutive rows then hit
// 16 distinct 16-byte bank groups (rows 2j and 2j + 1 differ by 128 B, rows
// 2j and 2j + 2 in their chunk). One barrier per K step: after it, the loads of step k+1 are issued
// into the other stage and stay in flight during the MFMAs of step k. The
// loop has a single body (stage chosen at run time): a body unrolled per
// stage with an exit between the copies doubles the live accumulators.
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives
// each XCD a contiguous range of tiles, traversed in groups of 8 row panels,
// so concurrently running tiles of one XCD share A and B panels in its L2.
constexpr int BIG_BM = 256, BIG_BN = 256;
constexpr int BIG_TILE_BYTES = 256 * 128;  // one operand tile of one stage

__device__ __forceinline__ void big_tile_coords(int bid, int ntm, int ntn, int* tm, int* tn) {
  const int ntiles = ntm * ntn;
  int t = bid;
  if ((ntiles & 7) == 0) t = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int per_group = G * ntn;
  const int grp = t / per_group;
  const int first = grp * G;
  const int gsz = min(ntm - first, G);
  const int r = t - grp * per_group;
  *tm = first + r % gsz;
  *tn = r / gsz;
}

// Buffer resource over [base, base + bytes): raw (stride 0) buffer loads
// with 32-bit per-lane byte offsets; bytes past the end read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc + voff + soff into LDS at lds_block + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      uint8_t* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block, 16,
                                           voff, soff, 0, 0);
}

// vmcnt(0), expcnt/lgkmcnt untouched
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int FM, int FN>
__device__ __forceinline__ void big_compute(const uint8_t* sa, const uint8_t* sb,
                                            const int (&loff)[4], floatx16 (&acc)[FM][FN]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(sa + i * 32 * 128 + loff[kk]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(sb + j * 32 * 128 + loff[kk]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

template <int EPI, int WAVES_M, int WAVES_N>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1)
gemm_big_kernel(GemmArgs g) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BIG_WM = BIG_BM / WAVES_M, BIG_WN = BIG_BN / WAVES_N;
  constexpr int FM = BIG_WM / 32, FN = BIG_WN / 32;
  constexpr int BPW = 32 / NW;               // DMA blocks per wave per operand
  static_assert(BIG_WN == 128, "epilogues assume 128 columns per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BIG_TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BIG_TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BIG_TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BIG_TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int ntm = (g.M + BIG_BM - 1) / BIG_BM, ntn = (g.N + BIG_BN - 1) / BIG_BN;
  int tm, tn;
  big_tile_coords(blockIdx.x, ntm, ntn, &tm, &tn);
  const int m0 = tm * BIG_BM, n0 = tn * BIG_BN;
  const int ksteps = g.K / BK;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)(g.M - 1) * g.lda * 2 + g.K * 2));
  const int brows = EPI == EPI_SWIGLU ? 2 * g.F : g.N;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)(brows - 1) * g.ldb * 2 + g.K * 2));

  // DMA sources: wave w fills blocks w, w+NW, w+2NW, ... of each operand tile
  const int lr = lane >> 3;                 // row within the block
  uint32_t aoff[BPW], boff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int r = (wave + NW * i) * 8 + lr;
    const int lc = (lane & 7) ^ ((r >> 1) & 7);  // logical chunk fetched by this lane
    aoff[i] = (uint32_t)((int64_t)min(m0 + r, g.M - 1) * g.lda * 2 + lc * 16);
    int v = min(n0 + r, g.N - 1);
    int row = v;
    if (EPI == EPI_SWIGLU) {
      const int f = ((v >> 6) << 5) | (v & 31);
      row = (v & 32) ? g.F + f : f;
    }
    boff[i] = (uint32_t)((int64_t)row * g.ldb * 2 + lc * 16);
  }
  // LDS lane offsets of the fragment reads for the 4 k-steps of 16; rows of
  // every fragment are multiples of 32 apart, so the swizzle of a lane's row
  // depends on lane & 31 only
  const int fr = lane & 31, fh = lane >> 5;
  int loff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) loff[kk] = fr * 128 + (((2 * kk + fh) ^ ((fr >> 1) & 7)) << 4);
  const int a_wave = wm * BIG_WM * 128, b_wave = wn * BIG_WN * 128;

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#define DORY_ISSUE(KS, SA, SB)                                              \
  do {                                                                      \
    const uint32_t ko_ = (uint32_t)(KS) * (BK * 2);                         \
    _Pragma("unroll") for (int i_ = 0; i_ < BPW; ++i_) {                    \
      dma16(ra, aoff[i_], ko_, (SA) + (wave + NW * i_) * 1024);             \
      dma16(rb, boff[i_], ko_, (SB) + (wave + NW * i_) * 1024);             \
    }                                                                       \
  } while (0)

  DORY_ISSUE(0, sA0, sB0);
  for (int ks = 0; ks < ksteps; ++ks) {
    wait_vm0();
    __syncthreads();
    const bool odd = ks & 1;
    if (ks + 1 < ksteps) {
      if (odd) DORY_ISSUE(ks + 1, sA0, sB0);
      else DORY_ISSUE(ks + 1, sA1, sB1);
    }
    big_compute((odd ? sA1 : sA0) + a_wave, (odd ? sB1 : sB0) + b_wave, loff, acc);
  }
#undef DORY_ISSUE

  const int rbase = m0 + wm * BIG_WM + (lane >> 5) * 4;
  const int cbase = n0 + wn * BIG_WN + (lane & 31);
  if (EPI == EPI_QKV) {
    // Each wave's 128 columns are one head of q, k, v or the gate. Lane holds
    // head dims d = 32 j + (lane & 31), j = 0..3, for 32 rows; RoPE pairs
    // (d, d + 64) are (j, j + 2) of the same lane; the per-head norm sums the
    // lane's 4 values and reduces over the 32 lanes that share its rows.
    const QkvEpi& q = g.qkv;
    const int dq = q.nq * 128, dkv = q.nkv * 128;
    const int c0 = n0 + wn * BIG_WN;
    const int dl = lane & 31;
    int kind, hh;
    if (c0 < dq) { kind = 0; hh = c0 >> 7; }
    else if (c0 < dq + dkv) { kind = 1; hh = (c0 - dq) >> 7; }
    else if (c0 < dq + 2 * dkv) { kind = 2; hh = (c0 - dq - dkv) >> 7; }
    else { kind = 3; hh = (c0 - dq - 2 * dkv) >> 7; }
    if (c0 >= g.N) kind = 4;
    float sq0 = 0.f, sq1 = 0.f;
    if (kind <= 1) { sq0 = q.s_qk[dl]; sq1 = q.s_qk[dl + 32]; }
    float sq2 = kind <= 1 ? q.s_qk[dl + 64] : 0.f, sq3 = kind <= 1 ? q.s_qk[dl + 96] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = rbase + i * 32 + (e >> 2) * 8 + (e & 3);
        const bool ok = row < g.M;
        const int b = row / q.T, t = row - b * q.T;
        float x0 = acc[i][0][e], x1 = acc[i][1][e], x2 = acc[i][2][e], x3 = acc[i][3][e];
        if (kind <= 1) {
          const int tr = ok ? t : 0;
          const float c0f = q.cs[tr * 64 + dl], s0f = q.sn[tr * 64 + dl];
          const float c1f = q.cs[tr * 64 + 32 + dl], s1f = q.sn[tr * 64 + 32 + dl];
          const float r0 = x0 * c0f - x2 * s0f, r2 = x2 * c0f + x0 * s0f;
          const float r1 = x1 * c1f - x3 * s1f, r3 = x3 * c1f + x1 * s1f;
          float ss = r0 * r0 + r1 * r1 + r2 * r2 + r3 * r3;
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
          const float inv = 1.0f / sqrtf(ss);
          x0 = r0 * inv * sq0; x1 = r1 * inv * sq1; x2 = r2 * inv * sq2; x3 = r3 * inv * sq3;
          if (ok) {
            uint16_t* dst = kind == 0
                ? q.qh + (((int64_t)b * q.nq + hh) * q.T + t) * 128
                : q.kf + (((int64_t)b * q.nkv + hh) * q.f_rows + t + q.row_off) * 128;
            dst[dl] = f2bf(x0); dst[dl + 32] = f2bf(x1); dst[dl + 64] = f2bf(x2); dst[dl + 96] = f2bf(x3);
          }
        } else if (kind == 2) {
          if (ok) {
            uint16_t* dst = q.vf + (((int64_t)b * q.nkv + hh) * 128 + dl) * q.f_rows + t + q.row_off;
            const int64_t cstep = 32 * q.f_rows;
            dst[0] = f2bf(x0); dst[cstep] = f2bf(x1); dst[2 * cstep] = f2bf(x2); dst[3 * cstep] = f2bf(x3);
          }
        } else if (kind == 3) {
          if (ok) {
            uint16_t* dst = q.gate + (int64_t)row * dq + hh * 128;
            dst[dl] = f2bf(1.f / (1.f + __expf(-x0)));
            dst[dl + 32] = f2bf(1.f / (1.f + __expf(-x1)));
            dst[dl + 64] = f2bf(1.f / (1.f + __expf(-x2)));
            dst[dl + 96] = f2bf(1.f / (1.f + __expf(-x3)));
          }
        }
      }
  } else if (EPI == EPI_F32 || EPI == EPI_LOGITS) {
    float* C = g.C;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
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
    for (int jp = 0; jp < 2; ++jp) {
      const int v = cbase + jp * 64;
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

// Tile shape of the large-M kernel: 8 waves of 64 x 128 (two waves per SIMD)
// or 4 waves of 128 x 128 (one wave per SIMD, accumulators in AGPRs, a
// third less LDS fragment traffic per MFMA).
constexpr int BIG_WAVES_M = 4, BIG_WAVES_N = 2;

hipError_t launch_big(const GemmArgs& a, int epi, hipStream_t st) {
  const int tiles = ((a.M + BIG_BM - 1) / BIG_BM) * ((a.N + BIG_BN - 1) / BIG_BN);
  dim3 grid(tiles), block(64 * BIG_WAVES_M * BIG_WAVES_N);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_big_kernel<EPI_F32, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_big_kernel<EPI_SWIGLU, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_big_kernel<EPI_LOGITS, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_big_kernel<EPI_QKV, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny kernel for M <= 64 (decode, the LM head of a prefill): the weight
// stream dominates, so the goal is bytes in flight. 64 x 64 x 64 tiles, 4
// waves of 32 x 32, two LDS stages filled by buffer DMA (the same XOR-
// swizzled 128-byte rows as the large kernel), 32 KiB of LDS so that four
// workgroups share a CU, and split-K for enough workgroups.
template <int EPI>
__global__ void __launch_bounds__(256)
gemm_skinny_kernel(GemmArgs g) {
  constexpr int SB = 64 * 128;  // one operand tile of one stage
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * 64;
  const int ksteps = g.K / BK;
  const int per = (ksteps + g.nsplit - 1) / g.nsplit;
  const int ks0 = blockIdx.z * per;
  const int ks1 = min(ksteps, ks0 + per);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)(g.M - 1) * g.lda * 2 + g.K * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)(g.N - 1) * g.ldb * 2 + g.K * 2));
  const int lr = lane >> 3;
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave + 4 * i) * 8 + lr;
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = (uint32_t)((int64_t)min(r, g.M - 1) * g.lda * 2 + lc * 16);
    boff[i] = (uint32_t)((int64_t)min(n0 + r, g.N - 1) * g.ldb * 2 + lc * 16);
  }
  const int fr = lane & 31, fh = lane >> 5;
  int loff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) loff[kk] = fr * 128 + (((2 * kk + fh) ^ ((fr >> 1) & 7)) << 4);

  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

#define DORY_SISSUE(KS, SA, SB_)                                            \
  do {                                                                      \
    const uint32_t ko_ = (uint32_t)(KS) * (BK * 2);                         \
    _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_) {                      \
      dma16(ra, aoff[i_], ko_, (SA) + (wave + 4 * i_) * 1024);              \
      dma16(rb, boff[i_], ko_, (SB_) + (wave + 4 * i_) * 1024);             \
    }                                                                       \
  } while (0)

  if (ks0 < ks1) DORY_SISSUE(ks0, sA0, sB0);
  for (int ks = ks0; ks < ks1; ++ks) {
    wait_vm0();
    __syncthreads();
    const bool odd = (ks - ks0) & 1;
    if (ks + 1 < ks1) {
      if (odd) DORY_SISSUE(ks + 1, sA0, sB0);
      else DORY_SISSUE(ks + 1, sA1, sB1);
    }
    const uint8_t* sa = (odd ? sA1 : sA0) + wm * 32 * 128;
    const uint8_t* sb = (odd ? sB1 : sB0) + wn * 32 * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(sa + loff[kk]);
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(sb + loff[kk]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
  }
#undef DORY_SISSUE

  const int col = n0 + wn * 32 + (lane & 31);
  if (col < g.N) {
    const float sc = (EPI == EPI_LOGITS) ? g.s1[col] : 1.f;
    float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
    const int rbase = wm * 32 + (lane >> 5) * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rbase + (e >> 2) * 8 + (e & 3);
      if (row < g.M) C[(int64_t)row * g.ldc + col] = acc[e] * sc;
    }
  }
}

hipError_t launch_skinny(const GemmArgs& a, int epi, hipStream_t st) {
  dim3 grid((a.N + 63) / 64, 1, a.nsplit), block(256);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_skinny_kernel<EPI_F32>), grid, block, 0, st, a); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_skinny_kernel<EPI_LOGITS>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  const int ksteps = K / BK;
  if (M <= 64) {
    // skinny path: aim for about four workgroups per CU, >= 2 K steps each
    const int tiles = (N + 63) / 64;
    int s = 1;
    while (s * 2 <= max_split && tiles * s < 1024 && ksteps / (s * 2) >= 2) s *= 2;
    return s;
  }
  const int tiles = ((M + 63) / 64) * ((N + 127) / 128);
  int s = 1;
  while (s * 2 <= max_split && tiles * s < 512 && ksteps / (s * 2) >= 4) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  if (a.K % BK != 0 || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
  if (epi != EPI_F32 && a.nsplit != 1) return hipErrorInvalidValue;
  if (a.M >= kLargeM) return launch_big(a, epi, st);
  if (epi == EPI_QKV) return hipErrorInvalidValue;
  if (a.M <= 64 && (epi == EPI_F32 || epi == EPI_LOGITS)) return launch_skinny(a, epi, st);
  return launch_cfg<64, 128, 32, 64>(a, epi, st);
}

}  // namespace dory
