// bf16 GEMM on gfx950 MFMA (v_mfma_f32_32x32x16_bf16) for the dense
// projections of the forward pass: fused q/k/v/gate, attention output,
// SwiGLU up/gate (with the activation fused into the epilogue), MLP down
// projection and the LM head (with the logit scale fused).
//
// C[m, n] = sum_k A[m, k] * B[n, k]. A is the activation (row-major,
// K-contiguous), B the weight in [out, in] layout (also K-contiguous), so
// both operand tiles are loaded along K with 16-byte vector loads.
//
// Three bf16 kernels cover every row count: the large-M kernel (M >= 1024,
// prefill; 256 x 256 tiles on four DMA-fed LDS stages, fused epilogues), the
// skinny kernel (64 < M < 1024: verification chunks and short prefills;
// 64 x 64 tiles, split-K) and its wide form for decode (M <= 64: 64 x 128
// tiles, split-K, weight streaming), plus an MXFP8-weight variant (M <= 64).
#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

constexpr int BK = 64;

// ---------------------------------------------------------------------------
// Large-M kernel: 256 x 256 output tiles (256 x 288 for bf16 outputs 2,304
// wide: 8 column tiles fill whole rounds of 256 CUs where 9 leave the last
// round half empty), 8 waves (4 x 2, each 64 x 128 or 64 x 144), K
// in steps of 32 through four LDS stages filled by direct global->LDS DMA
// (buffer_load ... lds, 16 bytes per lane), so no VGPRs stage the operands
// and the loads of step k+3 are in flight while step k computes: a distance
// of three steps (about 3000 cycles) covers the global-load latency under
// full load, which one step of 64 (about 2000 cycles) did not.
// A stage holds the A tile (256 rows x 64 B) and then the B tile. Each 1 KiB
// DMA block holds 16 rows; lane l writes LDS bytes [16 l, 16 l + 16) and
// fetches logical 16-byte chunk (l % 4) ^ ((row / 2) % 4) of its row, i.e.
// the tile is stored XOR-swizzled. With this XOR the 16-byte fragment reads
// (16 consecutive rows, one chunk each) run free of bank conflicts on this
// part; the XOR by (row / 4) % 4, which keeps the 16 rows in 16 distinct
// 16-byte bank groups, still conflicted on half of the LDS cycles (measured
// with the LDS bank-conflict counters).
// One LDS-only barrier per step; the four stages are separate arrays and the
// loop body is unrolled over them, so that the compiler sees which stage a
// DMA writes and waits for in-flight DMA only through the explicit counts.
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives
// each XCD a contiguous range of tiles, traversed in groups of 8 row panels,
// so concurrently running tiles of one XCD share A and B panels in its L2.
constexpr int BIG_BM = 256, BIG_BN = 256;
constexpr int BIG_BK = 32;
constexpr int BIG_OP_BYTES = 256 * BIG_BK * 2;  // one operand tile of one stage

// Tile order: workgroups are dispatched round-robin over the 8 XCDs, so
// t = (bid % 8) * (tiles / 8) + bid / 8 gives each XCD a contiguous range of
// tiles; the range is walked in groups of `grp` row panels (or column panels
// if `by_cols`), so that the tiles running at once on one XCD share A and B
// panels in its L2.
__device__ __forceinline__ void big_tile_coords(int bid, int ntm, int ntn, int grp, bool by_cols,
                                                int* tm, int* tn) {
  const int ntiles = ntm * ntn;
  int t = bid;
  if ((ntiles & 7) == 0) t = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int na = by_cols ? ntn : ntm, nb = by_cols ? ntm : ntn;
  const int per_group = grp * nb;
  const int gi = t / per_group;
  const int first = gi * grp;
  const int gsz = min(na - first, grp);
  const int r = t - gi * per_group;
  const int a = first + r % gsz, b = r / gsz;
  *tm = by_cols ? b : a;
  *tn = by_cols ? a : b;
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

// Fragments of one k-step of 32 for a wave's tile: 16-row A blocks and
// 16-column B blocks; lane l holds row (l % 16) and k = 8 (l / 16) .. + 7.
template <int FM, int FN>
__device__ __forceinline__ void big_read(const uint8_t* sa, const uint8_t* sb, int loff,
                                         bf16x8 (&af)[FM], bf16x8 (&bfr)[FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(sa + i * 16 * 64 + loff);
#pragma unroll
  for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(sb + j * 16 * 64 + loff);
}

// v_mfma_f32_16x16x32_bf16: on random bf16 data it sustains about 14% more
// throughput on this part than the 32x32x16 form (measured, register-only).
// TR: the operands swapped, so that block (i, j) holds the transpose (lane
// holds row (lane % 16) and columns 4 (lane / 16) + e).
template <bool TR, int FM, int FN>
__device__ __forceinline__ void big_mfma(const bf16x8 (&af)[FM], const bf16x8 (&bfr)[FN],
                                         floatx4 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = TR ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

// Phase boundary of the ping-pong schedule: an LDS-only barrier that the
// scheduler may not move instructions across.
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  barrier_lds();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_vm8() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F78);
  __builtin_amdgcn_sched_barrier(0);
}

template <int EPI, int WAVES_M, int WAVES_N, int BN = BIG_BN>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1)
gemm_big_kernel(GemmArgs g) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BIG_WM = BIG_BM / WAVES_M, BIG_WN = BN / WAVES_N;
  constexpr int FM = BIG_WM / 16, FN = BIG_WN / 16;
  constexpr int BPW = 16 / NW;               // A DMA blocks per wave (B: BN / 16 blocks in all)
  constexpr int NBB = BN / 16;               // B DMA blocks of a stage
  constexpr int BPWB = (NBB + NW - 1) / NW;  // B DMA blocks per wave, at most
  static_assert(BIG_WN == 128 || (BN == 288 && EPI == EPI_BF16 && NW == 8),
                "epilogues assume 128 columns per wave; 288-column tiles have the bf16 one only");
  static_assert(NW == 8 || BN == BIG_BN, "one wave per SIMD: 256 columns");
  // A stage holds the A tile (16 KiB) and the B tile (BN x 64 B)
  constexpr int STAGE = BIG_OP_BYTES + BN * BIG_BK * 2;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int ntm = (g.M + BIG_BM - 1) / BIG_BM, ntn = (g.N + BN - 1) / BN;
  int tm, tn;
  big_tile_coords(blockIdx.x, ntm, ntn, g.order & 0xFF, (g.order >> 8) & 1, &tm, &tn);
  if (EPI == EPI_QKV) {
    // column tiles in the order s * tn mod ntn (s coprime to ntn): the tiles
    // that run at once on an XCD (neighbouring columns) mix q, k, v and gate
    // heads instead of all fetching RoPE rows and normalizing at the same
    // moment (B panels of neighbouring columns share nothing, so L2 reuse
    // is unchanged)
    const int sp = ntn % 3 != 0 ? 3 : ntn % 7 != 0 ? 7 : 1;
    tn = (tn * sp) % ntn;
  }
  const int m0 = tm * BIG_BM, n0 = tn * BN;
  const int ksteps = g.K / BIG_BK;           // even: K is a multiple of 64

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)(g.M - 1) * g.lda * 2 + g.K * 2));
  const int brows = EPI == EPI_SWIGLU ? 2 * g.F : g.N;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)(brows - 1) * g.ldb * 2 + g.K * 2));

  // DMA sources: wave w fills blocks w, w + NW of each operand tile
  const int lr = lane >> 2;                  // row within the block
  const int lc = (lane & 3) ^ ((lr >> 1) & 3);  // logical chunk (block rows are 16-aligned)
  uint32_t aoff[BPW], boff[BPWB];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int r = (wave + NW * i) * 16 + lr;
    aoff[i] = (uint32_t)((int64_t)min(m0 + r, g.M - 1) * g.lda * 2 + lc * 16);
  }
#pragma unroll
  for (int i = 0; i < BPWB; ++i) {
    const int r = (wave + NW * i) * 16 + lr;  // (rows past the tile: never loaded)
    int v = min(n0 + r, g.N - 1);
    int row = v;
    if (EPI == EPI_SWIGLU) {
      const int f = ((v >> 6) << 5) | (v & 31);
      row = (v & 32) ? g.F + f : f;
    }
    boff[i] = (uint32_t)((int64_t)row * g.ldb * 2 + lc * 16);
  }
  // LDS lane offset of the fragment reads; fragment rows are multiples of 16
  // apart, so the swizzle of a lane's row depends on lane & 15 only
  const int fr = lane & 15, fc = lane >> 4;
  const int loff = fr * 64 + ((fc ^ ((fr >> 1) & 3)) << 4);
  const int a_wave = wm * BIG_WM * 64, b_wave = BIG_OP_BYTES + wn * BIG_WN * 64;

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  // the B blocks of a 288-wide tile do not divide by the waves: waves
  // 0 .. NBB % NW - 1 load one more, and wait for two more per step
  const bool extra_b = NBB % NW != 0 && wave < NBB % NW;
  auto issue = [&](int ks, uint8_t* stg) {
    const uint32_t ko = (uint32_t)ks * (BIG_BK * 2);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      dma16(ra, aoff[i], ko, stg + (wave + NW * i) * 1024);
      dma16(rb, boff[i], ko, stg + BIG_OP_BYTES + (wave + NW * i) * 1024);
    }
    if (BPWB > BPW && extra_b) dma16(rb, boff[BPWB - 1], ko, stg + BIG_OP_BYTES + (wave + NW * BPW) * 1024);
  };
  // two younger steps stay in flight
  auto wait_two = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    if (BPWB > BPW && extra_b) __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
    else __builtin_amdgcn_s_waitcnt(0x0F78);                        // vmcnt(8)
    __builtin_amdgcn_sched_barrier(0);
  };
  bf16x8 af[FM], bfr[FN];
  if constexpr (NW == 8) {
    // Ping-pong schedule. Waves 0-3 (group A) and 4-7 (group B) hold one wave
    // on each SIMD. Time is cut into phases separated by workgroup barriers; in
    // every phase one group runs the memory part of a step (fragment reads
    // from the stage into registers, then its share of the DMA of step + 3)
    // while the other group runs the 16 MFMAs of the step whose fragments it
    // read in the phase before, so each SIMD's matrix pipe is fed by one wave
    // while the other waits on the LDS. Group A: M(s) in phase 2s, C(s) in 2s+1;
    // group B one phase later.
    // Stage (s + 3) % 4 is last read by B's M(s - 1) in phase 2s - 1, so both
    // groups' M(s) may load it. The DMA of step t must be complete in every
    // wave before the barrier that opens phase 2t (A's M(t)): A waits at the
    // end of C(t - 1), B at the end of M(t - 1). Each M issues exactly 4 DMA
    // (the last steps reload the final step into a stage no one reads again),
    // so both waits are vmcnt(8) (the two younger steps stay in flight).
    auto mem = [&](int ks, const uint8_t* cur, uint8_t* nxt) {
      big_read(cur + a_wave, cur + b_wave, loff, af, bfr);
      issue(min(ks + 3, ksteps - 1), nxt);
    };

    issue(0, st0);
    issue(1, st1);
    issue(min(2, ksteps - 1), st2);
    wait_two();
    pp_barrier();
    if (wave < NW / 2) {
  #define DORY_PP_A(KS, CUR, NXT)                                             \
      mem(KS, CUR, NXT); pp_barrier();                                        \
      big_mfma<EPI == EPI_QKV || EPI == EPI_BF16>(af, bfr, acc); wait_two(); pp_barrier();
      int ks = 0;
      for (; ks + 4 <= ksteps; ks += 4) {
        DORY_PP_A(ks, st0, st3)
        DORY_PP_A(ks + 1, st1, st0)
        DORY_PP_A(ks + 2, st2, st1)
        DORY_PP_A(ks + 3, st3, st2)
      }
      if (ks < ksteps) {  // ksteps % 4 == 2
        DORY_PP_A(ks, st0, st3)
        DORY_PP_A(ks + 1, st1, st0)
      }
  #undef DORY_PP_A
      pp_barrier();
    } else {
  #define DORY_PP_B(KS, CUR, NXT)                                             \
      mem(KS, CUR, NXT); wait_two(); pp_barrier();                            \
      big_mfma<EPI == EPI_QKV || EPI == EPI_BF16>(af, bfr, acc); pp_barrier();
      pp_barrier();
      int ks = 0;
      for (; ks + 4 <= ksteps; ks += 4) {
        DORY_PP_B(ks, st0, st3)
        DORY_PP_B(ks + 1, st1, st0)
        DORY_PP_B(ks + 2, st2, st1)
        DORY_PP_B(ks + 3, st3, st2)
      }
      if (ks < ksteps) {
        DORY_PP_B(ks, st0, st3)
        DORY_PP_B(ks + 1, st1, st0)
      }
  #undef DORY_PP_B
    }

  } else {
    // One wave per SIMD: every wave waits for its loads of step ks (the
    // loads of the two younger steps stay in flight), the barrier makes all
    // parts visible and frees stage (ks + 3) % 4 (read in step ks - 1), then
    // the wave loads step ks + 3 (clamped, as above) and computes step ks.
    auto step = [&](int ks, const uint8_t* cur, uint8_t* nxt) {
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): two younger steps of 8
      barrier_lds();
      issue(min(ks + 3, ksteps - 1), nxt);
      big_read(cur + a_wave, cur + b_wave, loff, af, bfr);
      big_mfma<EPI == EPI_QKV || EPI == EPI_BF16>(af, bfr, acc);
    };
    issue(0, st0);
    issue(1, st1);
    issue(min(2, ksteps - 1), st2);
    int ks = 0;
    for (; ks + 4 <= ksteps; ks += 4) {
      step(ks, st0, st3);
      step(ks + 1, st1, st0);
      step(ks + 2, st2, st1);
      step(ks + 3, st3, st2);
    }
    if (ks < ksteps) {
      step(ks, st0, st3);
      step(ks + 1, st1, st0);
    }
  }
  wait_vm0();  // no DMA may outlive the workgroup's LDS

  // Output layout of a 16x16 block: lane holds column (lane % 16) and rows
  // 4 (lane / 16) + e, e = 0..3.
  const int rbase = m0 + wm * BIG_WM + (lane >> 4) * 4;
  const int cbase = n0 + wn * BIG_WN + (lane & 15);
  if (EPI == EPI_QKV) {
    // Each wave's 128 columns are one head of q, k, v or the gate. The
    // accumulators are transposed (the MFMA operands are swapped for this
    // epilogue): lane l holds token row wm * 64 + 16 i + (l % 16) of the tile
    // and head dims d = 16 j + 4 (l / 16) + e, e = 0..3, so q, k and gate
    // rows leave as 8-byte pieces (4 consecutive dims) and V^T columns as
    // runs of 16 consecutive tokens. RoPE pairs (d, d + 64) are blocks (j,
    // j + 4) of the same lane; the per-head norm sums the lane's 32 values
    // and reduces over the 4 lanes that hold the same token.
    const QkvEpi& q = g.qkv;
    const int dq = q.nq * 128, dkv = q.nkv * 128;
    const int c0 = n0 + wn * BIG_WN;
    const int tl = lane & 15, dg = (lane >> 4) * 4;
    int kind, hh;
    if (c0 < dq) { kind = 0; hh = c0 >> 7; }
    else if (c0 < dq + dkv) { kind = 1; hh = (c0 - dq) >> 7; }
    else if (c0 < dq + 2 * dkv) { kind = 2; hh = (c0 - dq - dkv) >> 7; }
    else { kind = 3; hh = (c0 - dq - 2 * dkv) >> 7; }
    if (c0 >= g.N) kind = 4;
    float4 sq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sq[j] = kind <= 1 ? make_float4(q.s_qk[16 * j + dg], q.s_qk[16 * j + dg + 1], q.s_qk[16 * j + dg + 2],
                                      q.s_qk[16 * j + dg + 3])
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    // s_qk becomes plain register values before any store: a global load
    // consumed between the stores would make each wait for all earlier
    // stores (one counter).
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(sq[j].x), "+v"(sq[j].y), "+v"(sq[j].z), "+v"(sq[j].w));
    // The RoPE table rows of the tile's 256 token rows go to the (now free)
    // stages by direct global->LDS DMA, all 128 KiB in flight at once (the
    // table is evicted from L2 by the operand stream, so a load costs a
    // memory round trip): cos in st0/st1, sin in st2/st3, 256 B per row,
    // 16-byte chunk c of row r stored at c ^ (r % 16) so that the 16 rows
    // one fragment read covers fall in distinct bank groups. 1 KiB block
    // k holds rows 4 k' .. 4 k' + 3 of its table (k' = k % 64), lane l
    // chunk l % 16 of row 4 k' + l / 16.
    if (n0 < dq + dkv) {
      __syncthreads();  // every wave is done with the stages
#pragma unroll
      for (int kb = 0; kb < 128 / NW; ++kb) {
        const int blk = wave * (128 / NW) + kb;  // 0-63 cos, 64-127 sin
        const int r0 = (blk & 63) * 4;
        const int rr = r0 + (lane >> 4);
        const int row = m0 + rr;
        const int t = row < g.M ? row % q.T : 0;
        const int c = (lane & 15) ^ (rr & 15);
        const float* src = (blk < 64 ? q.cs : q.sn) + (int64_t)t * 64 + c * 4;
        uint8_t* dst = (blk < 64 ? (r0 < 128 ? st0 : st1) : (r0 < 128 ? st2 : st3)) + (r0 & 127) * 256;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
      wait_vm0();
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rl = wm * BIG_WM + 16 * i + tl;  // token row within the tile
      const int row = m0 + rl;
      const bool ok = row < g.M;
      const int b = row / q.T, t = row - b * q.T;
      if (kind <= 1) {
        const uint8_t* lcs = (rl < 128 ? st0 : st1) + (rl & 127) * 256;
        const uint8_t* lsn = (rl < 128 ? st2 : st3) + (rl & 127) * 256;
        float4 c4[4], s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int po = ((4 * j + (lane >> 4)) ^ tl) << 4;  // chunk of dims 16 j + dg .. + 3
          c4[j] = *reinterpret_cast<const float4*>(lcs + po);
          s4[j] = *reinterpret_cast<const float4*>(lsn + po);
        }
        float r[8][4];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float cv[4] = {c4[j].x, c4[j].y, c4[j].z, c4[j].w};
          const float sv[4] = {s4[j].x, s4[j].y, s4[j].z, s4[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = acc[i][j][e], x1 = acc[i][j + 4][e];
            r[j][e] = x0 * cv[e] - x1 * sv[e];
            r[j + 4][e] = x1 * cv[e] + x0 * sv[e];
            ss += r[j][e] * r[j][e] + r[j + 4][e] * r[j + 4][e];
          }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float inv = __builtin_amdgcn_rsqf(ss);  // bf16 outputs: 1 ulp is ample
        if (ok) {
          uint16_t* dst = kind == 0
              ? q.qh + (((int64_t)b * q.nq + hh) * q.T + t) * 128
              : q.kf + (((int64_t)b * q.nkv + hh) * q.f_rows + t + q.row_off) * 128;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float sj[4] = {sq[j].x, sq[j].y, sq[j].z, sq[j].w};
            ushort4 o;
            o.x = f2bf_hw(r[j][0] * inv * sj[0]);
            o.y = f2bf_hw(r[j][1] * inv * sj[1]);
            o.z = f2bf_hw(r[j][2] * inv * sj[2]);
            o.w = f2bf_hw(r[j][3] * inv * sj[3]);
            *reinterpret_cast<ushort4*>(dst + 16 * j + dg) = o;
          }
        }
      } else if (kind == 2) {
        if (ok) {
          uint16_t* dst = q.vf + ((int64_t)b * q.nkv + hh) * 128 * q.f_rows + t + q.row_off;
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(int64_t)(16 * j + dg + e) * q.f_rows] = f2bf_hw(acc[i][j][e]);
        }
      } else if (kind == 3) {
        if (ok) {
          uint16_t* dst = q.gate + (int64_t)row * dq + hh * 128;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            ushort4 o;
            o.x = f2bf_hw(__builtin_amdgcn_rcpf(1.f + __expf(-acc[i][j][0])));
            o.y = f2bf_hw(__builtin_amdgcn_rcpf(1.f + __expf(-acc[i][j][1])));
            o.z = f2bf_hw(__builtin_amdgcn_rcpf(1.f + __expf(-acc[i][j][2])));
            o.w = f2bf_hw(__builtin_amdgcn_rcpf(1.f + __expf(-acc[i][j][3])));
            *reinterpret_cast<ushort4*>(dst + 16 * j + dg) = o;
          }
        }
      }
    }
  } else if (EPI == EPI_F32 || EPI == EPI_LOGITS) {
    float* C = g.C;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = cbase + j * 16;
      if (col >= g.N) continue;
      const float sc = (EPI == EPI_LOGITS) ? g.s1[col] : 1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + i * 16 + e;
          if (row < g.M) C[(int64_t)row * g.ldc + col] = acc[i][j][e] * sc;
        }
    }
  } else if (EPI == EPI_BF16) {
    // Accumulators transposed (the MFMA operands are swapped for this
    // epilogue): lane l holds row 16 i + (l % 16) of the wave's 64 rows and
    // columns 16 j + 4 (l / 16) + e, e = 0..3, i.e. four consecutive
    // outputs of one row, rounded to bf16 and stored as one 8-byte piece
    // (no staging through LDS, no workgroup barrier).
    const int cl = n0 + wn * BIG_WN + 4 * (lane >> 4);
    const bool vec_ok = g.ldc16 % 4 == 0 && (reinterpret_cast<uintptr_t>(g.C16) & 7) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = m0 + wm * BIG_WM + 16 * i + (lane & 15);
      if (row < g.M) {
        uint16_t* dst = g.C16 + (int64_t)row * g.ldc16;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = cl + 16 * j;
          ushort4 o;
          o.x = f2bf_hw(acc[i][j][0]);
          o.y = f2bf_hw(acc[i][j][1]);
          o.z = f2bf_hw(acc[i][j][2]);
          o.w = f2bf_hw(acc[i][j][3]);
          if (vec_ok && col + 4 <= g.N) {
            *reinterpret_cast<ushort4*>(dst + col) = o;
          } else {
            const uint16_t oe[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (col + k < g.N) dst[col + k] = oe[k];
          }
        }
      }
    }
  } else {
    // 64-column groups: blocks 0, 1 are up, blocks 2, 3 the gate of the same
    // 32 features (see the B-row interleave of the DMA sources). The scales
    // are loaded and every output computed before the first store: a load
    // consumed between stores makes the compiler wait for all earlier stores
    // (one vector-memory counter), which serialized the epilogue.
    constexpr int NJP = FN / 4;
    float su[NJP][2], sv[NJP][2];
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int v = cbase + jp * 64 + h * 16;
        const int f = min(((v >> 6) << 5) | (v & 31), g.F - 1);
        su[jp][h] = g.s1[f];
        sv[jp][h] = g.s2[f];
      }
    // the loaded scales become plain register values here (one wait for
    // the loads), so that the guarded stores below depend on no load
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(su[jp][h]), "+v"(sv[jp][h]));
    // The wave's outputs (64 rows x 64 features, bf16) are staged through
    // LDS, free after the main loop, and written as whole 128-byte row
    // pieces, 16 bytes per lane (in the accumulator layout a lane's values
    // of one row are 16 features apart: 2-byte stores of 32-byte pieces).
    static_assert(NJP * 32 == 64 && BIG_WM == 64, "one 64-feature group per wave");
    constexpr int SROW = 64 * 2 + 16;  // padded LDS row of the staging tile
    __syncthreads();                   // every wave is done with the stages
    uint8_t* stg = wave < 3 ? st0 + wave * 64 * SROW
                 : wave < 6 ? st1 + (wave - 3) * 64 * SROW : st2 + (wave - 6) * 64 * SROW;
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float up = acc[i][4 * jp + h][e] * su[jp][h];
            const float gt = acc[i][4 * jp + 2 + h][e] * sv[jp][h];
            const float act = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt));
            const int r = (lane >> 4) * 4 + i * 16 + e;
            const int lf = jp * 32 + h * 16 + (lane & 15);
            *reinterpret_cast<uint16_t*>(stg + r * SROW + lf * 2) = f2bf(act * up);
          }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's staging writes are done
    __builtin_amdgcn_wave_barrier();
    const int fbase = (n0 + wn * BIG_WN) / 2;  // first feature of the wave's group
    if (fbase < g.F) {
#pragma unroll
      for (int pass = 0; pass < 8; ++pass) {
        const int r = pass * 8 + (lane >> 3);
        const int row = m0 + wm * BIG_WM + r;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * SROW + (lane & 7) * 16);
        if (row < g.M)
          *reinterpret_cast<uint4*>(g.C16 + (int64_t)row * g.ldc16 + fbase + (lane & 7) * 8) = v;
      }
    }
  }
}

// Tile shape of the large-M kernel: 8 waves of 64 x 128 (two waves per SIMD)
// or 4 waves of 128 x 128 (one wave per SIMD, accumulators in AGPRs, a
// third less LDS fragment traffic per MFMA).
constexpr int BIG_WAVES_M = 4, BIG_WAVES_N = 2;

// Panel grouping per shape, measured at M = 32768 on MI355X: wide outputs
// (>= 16 column tiles: the q/k/v/gate and up/gate projections) run best in
// groups of 4 row panels; narrow ones (the d-wide outputs) in groups of 2,
// by rows for long K (down projection, K = 6144) and by columns for short K
// (attention output, K = 2048). Against groups of 8 rows: -17% time for
// up/gate, -13% q/k/v/gate, -9% down, -4% attention output.
int big_order(int N, int K) {
  const int ntn = (N + BIG_BN - 1) / BIG_BN;
  if (ntn >= 16) return 4;
  return K >= 4096 ? 2 : (0x100 | 2);
}

hipError_t launch_big(const GemmArgs& a0, int epi, hipStream_t st) {
  GemmArgs a = a0;
  if (epi == EPI_BF16 && a.N % 288 == 0 && (a.N / 288) % 8 == 0 &&
      !(a.N % BIG_BN == 0 && (a.N / BIG_BN) % 8 == 0)) {
    // e.g. N = 2,304: 8 columns of 288-wide tiles fill whole rounds (256
    // CUs) where 9 of 256 leave the last round half empty
    a.order = big_order(a.N, a.K);
    const int tiles = ((a.M + BIG_BM - 1) / BIG_BM) * (a.N / 288);
    hipLaunchKernelGGL((gemm_big_kernel<EPI_BF16, BIG_WAVES_M, BIG_WAVES_N, 288>), dim3(tiles),
                       dim3(64 * BIG_WAVES_M * BIG_WAVES_N), 0, st, a);
    return hipGetLastError();
  }
  a.order = big_order(a.N, a.K);
  const int tiles = ((a.M + BIG_BM - 1) / BIG_BM) * ((a.N + BIG_BN - 1) / BIG_BN);
  dim3 grid(tiles), block(64 * BIG_WAVES_M * BIG_WAVES_N);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_big_kernel<EPI_F32, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_big_kernel<EPI_SWIGLU, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_big_kernel<EPI_LOGITS, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_big_kernel<EPI_QKV, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    case EPI_BF16: hipLaunchKernelGGL((gemm_big_kernel<EPI_BF16, BIG_WAVES_M, BIG_WAVES_N>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny kernel for small M (decode, the LM head of a prefill, short
// verification chunks of a batch): the weight stream dominates, so the goal
// is bytes in flight. A ring of four LDS stages (one K step of 64 each, the
// same XOR-swizzled 128-byte rows as the large kernel) filled by DMA three
// steps ahead; every step issues exactly four DMA per wave (the last steps
// reload the final step into a stage no one reads again), so the wait
// before each step is vmcnt(8). 64 x 64 output tiles, 4 waves of 32 x 32,
// split-K; above 64 rows one workgroup per 64-row block, grouped by XCD.
constexpr int SK_MAX = 4;

template <int EPI>
__global__ void __launch_bounds__(256)
gemm_skinny_kernel(GemmArgs g) {
  constexpr int SB = 64 * 128;  // one operand tile of one stage
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA3[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB3[SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // work item: (64-column tile, split) pair and 64-row block. Up to 64 rows:
  // blockIdx.x = tile, blockIdx.z = split. More rows (1-D grid): workgroups
  // are dispatched round-robin over the 8 XCDs, so XCD x takes pairs x,
  // x + 8, ... and runs the row blocks of one pair back to back; the pair's
  // weight tile then comes from that XCD's L2 after the first row block.
  int tile, split, m0 = 0;
  if (g.M > 64) {
    const int nmb = (g.M + 63) / 64;
    const int lin = blockIdx.x, j = lin >> 3;
    const int pair = (lin & 7) + 8 * (j / nmb);
    const int ntile = (g.N + 63) / 64;
    if (pair >= ntile * g.nsplit) return;  // padding of the last round of pairs
    tile = pair % ntile;
    split = pair / ntile;
    m0 = (j % nmb) * 64;
  } else {
    tile = blockIdx.x;
    split = blockIdx.z;
  }
  const int n0 = tile * 64;
  const int ksteps = g.K / BK;
  const int per = (ksteps + g.nsplit - 1) / g.nsplit;
  const int ks0 = split * per;
  const int n = max(0, min(ksteps, ks0 + per) - ks0);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)(g.M - 1) * g.lda * 2 + g.K * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)(g.N - 1) * g.ldb * 2 + g.K * 2));
  const int lr = lane >> 3;
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave + 4 * i) * 8 + lr;
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = (uint32_t)((int64_t)min(m0 + r, g.M - 1) * g.lda * 2 + lc * 16);
    boff[i] = (uint32_t)((int64_t)min(n0 + r, g.N - 1) * g.ldb * 2 + lc * 16);
  }
  const int fr = lane & 31, fh = lane >> 5;
  int loff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) loff[kk] = fr * 128 + (((2 * kk + fh) ^ ((fr >> 1) & 7)) << 4);

  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  // 2 + na DMA instructions per wave per step: the A blocks (8 rows each)
  // past the last row are not loaded (with few rows, as in decode, the
  // clamped rows would only repeat the last one); the MFMA rows they feed
  // are never stored
  const int mrows = g.M - m0;
  const bool a0 = wave * 8 < mrows, a1 = (wave + 4) * 8 < mrows;
  auto issue = [&](int ks, uint8_t* sa, uint8_t* sb) {
    const uint32_t ko = (uint32_t)ks * (BK * 2);
    if (a0) dma16(ra, aoff[0], ko, sa + wave * 1024);
    if (a1) dma16(ra, aoff[1], ko, sa + (wave + 4) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rb, boff[i], ko, sb + (wave + 4 * i) * 1024);
  };
  const int na = (a0 ? 1 : 0) + (a1 ? 1 : 0);
  auto compute = [&](const uint8_t* sa0, const uint8_t* sb0) {
    const uint8_t* sa = sa0 + wm * 32 * 128;
    const uint8_t* sb = sb0 + wn * 32 * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(sa + loff[kk]);
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(sb + loff[kk]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
  };
  if (n > 0) {
    issue(ks0, sA0, sB0);
    issue(ks0 + min(1, n - 1), sA1, sB1);
    issue(ks0 + min(2, n - 1), sA2, sB2);
    // the ring runs a multiple of 4 steps; steps past n only keep the wait
    // and load pattern uniform (no branch around the DMA) and compute nothing
    auto step = [&](int i, const uint8_t* ca, const uint8_t* cb, uint8_t* sna, uint8_t* snb) {
      // steps i + 1, i + 2 stay in flight: vmcnt(2 (2 + na))
      if (na == 2) __builtin_amdgcn_s_waitcnt(0x0F78);
      else if (na == 1) __builtin_amdgcn_s_waitcnt(0x0F76);
      else __builtin_amdgcn_s_waitcnt(0x0F74);
      barrier_lds();                        // all parts of step i landed; stage (i + 3) % 4 is free
      issue(ks0 + min(i + 3, n - 1), sna, snb);
      if (i < n) compute(ca, cb);
    };
    for (int i = 0; i < n; i += 4) {
      step(i, sA0, sB0, sA3, sB3);
      step(i + 1, sA1, sB1, sA0, sB0);
      step(i + 2, sA2, sB2, sA1, sB1);
      step(i + 3, sA3, sB3, sA2, sB2);
    }
    wait_vm0();  // no DMA may outlive the workgroup's LDS
  }

  const int col = n0 + wn * 32 + (lane & 31);
  if (col < g.N) {
    const float sc = (EPI == EPI_LOGITS) ? g.s1[col] : 1.f;
    float* C = g.C + (int64_t)split * g.split_stride;
    const int rbase = m0 + wm * 32 + (lane >> 5) * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rbase + (e >> 2) * 8 + (e & 3);
      if (row < g.M) C[(int64_t)row * g.ldc + col] = acc[e] * sc;
    }
  }
}

// Small-M kernel with MXFP8 weights (W8A16): the same 64 x 64 tiles, four
// waves of 32 x 32 and four-stage DMA ring as the bf16 kernel, with the
// weight tile held as E4M3 codes (64 columns x 64 bytes per step, half the
// bytes) and converted to bf16 in registers by the hardware conversion
// (v_cvt_scalef32_pk_bf16_fp8: two codes times the block scale per
// instruction) just before the MFMA; the product is then the bf16 product
// with the dequantized weights, which are exact in bf16. The block scales of
// the workgroup's 64 columns and K range (two per step and column) are read
// into LDS once, before the DMA stream starts. Every step issues exactly
// three DMA per wave (two activation blocks, one code block), so the wait
// before each step is vmcnt(6).
constexpr int MX_MAX_STEPS = 96;  // K steps of 64 per workgroup (scale table size)

template <int EPI>
__global__ void __launch_bounds__(256)
gemm_skinny_fp8_kernel(GemmArgs g) {
  constexpr int SA = 64 * 128;  // activation tile of one stage: 64 rows x 64 k
  constexpr int SB = 64 * 64;   // code tile: 64 columns x 64 k
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sA3[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB3[SB];
  __shared__ __attribute__((aligned(16))) uint8_t ssc[64 * 2 * MX_MAX_STEPS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * 64;
  const int ksteps = g.K / BK;
  const int per = (ksteps + g.nsplit - 1) / g.nsplit;
  const int ks0 = blockIdx.z * per;
  const int n = max(0, min(ksteps, ks0 + per) - ks0);

  // block scales: column c, block j of this workgroup's K range at c * 2n + j
  {
    const int nb = g.K / 32, w2 = 2 * n;
    for (int idx = tid; idx < 64 * w2; idx += 256) {
      const int c = idx / w2, j = idx - c * w2;
      ssc[idx] = g.Bs[(int64_t)min(n0 + c, g.N - 1) * nb + 2 * ks0 + j];
    }
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)(g.M - 1) * g.lda * 2 + g.K * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.Bq, (uint32_t)((int64_t)(g.N - 1) * g.K + g.K));
  const int lr = lane >> 3;
  uint32_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave + 4 * i) * 8 + lr;
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = (uint32_t)((int64_t)min(r, g.M - 1) * g.lda * 2 + lc * 16);
  }
  // code block `wave`: 16 columns x 64 bytes; lane l writes LDS bytes
  // [16 l, 16 l + 16) = chunk l % 4 of column l / 4, fetching logical chunk
  // (l % 4) ^ ((column / 2) % 4)
  uint32_t boff;
  {
    const int r = wave * 16 + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 1) & 3);
    boff = (uint32_t)((int64_t)min(n0 + r, g.N - 1) * g.K + lc * 16);
  }
  const int fr = lane & 31, fh = lane >> 5;
  int aloff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) aloff[kk] = fr * 128 + (((2 * kk + fh) ^ ((fr >> 1) & 7)) << 4);
  const int bcol = wn * 32 + fr;  // column of this lane's weight fragment within the tile
  int bloff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) bloff[kk] = bcol * 64 + ((kk ^ ((bcol >> 1) & 3)) << 4) + fh * 8;
  const uint8_t* sc_col = ssc + bcol * 2 * n;

  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  auto issue = [&](int ks, uint8_t* sa, uint8_t* sb) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(ra, aoff[i], (uint32_t)ks * (BK * 2), sa + (wave + 4 * i) * 1024);
    dma16(rb, boff, (uint32_t)ks * BK, sb + wave * 1024);
  };
  auto compute = [&](int i, const uint8_t* sa0, const uint8_t* sb) {
    const uint8_t* sa = sa0 + wm * 32 * 128;
    const float s0 = __uint_as_float((uint32_t)sc_col[2 * i] << 23);
    const float s1 = __uint_as_float((uint32_t)sc_col[2 * i + 1] << 23);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(sa + aloff[kk]);
      const uint2 cw = *reinterpret_cast<const uint2*>(sb + bloff[kk]);
      const float sc = kk < 2 ? s0 : s1;
      const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.x, sc, false);
      const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.x, sc, true);
      const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.y, sc, false);
      const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw.y, sc, true);
      bf16x8 bf;
      bf[0] = b0[0]; bf[1] = b0[1]; bf[2] = b1[0]; bf[3] = b1[1];
      bf[4] = b2[0]; bf[5] = b2[1]; bf[6] = b3[0]; bf[7] = b3[1];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
  };
  if (n > 0) {
    issue(ks0, sA0, sB0);
    issue(ks0 + min(1, n - 1), sA1, sB1);
    issue(ks0 + min(2, n - 1), sA2, sB2);
    // the ring runs a multiple of 4 steps; steps past n only keep the wait
    // and load pattern uniform (no branch around the DMA) and compute nothing
    auto step = [&](int i, const uint8_t* ca, const uint8_t* cb, uint8_t* na, uint8_t* nb) {
      __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6): steps i + 1, i + 2 stay in flight
      barrier_lds();                        // all parts of step i landed; stage (i + 3) % 4 is free
      issue(ks0 + min(i + 3, n - 1), na, nb);
      if (i < n) compute(i, ca, cb);
    };
    for (int i = 0; i < n; i += 4) {
      step(i, sA0, sB0, sA3, sB3);
      step(i + 1, sA1, sB1, sA0, sB0);
      step(i + 2, sA2, sB2, sA1, sB1);
      step(i + 3, sA3, sB3, sA2, sB2);
    }
    wait_vm0();  // no DMA may outlive the workgroup's LDS
  }

  const int col = n0 + wn * 32 + (lane & 31);
  if (col < g.N) {
    float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
    const int rbase = wm * 32 + (lane >> 5) * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rbase + (e >> 2) * 8 + (e & 3);
      if (row < g.M) C[(int64_t)row * g.ldc + col] = acc[e];
    }
  }
}

// Up to 64 rows (decode): 64 x 128 output tiles, 8 waves of 32 x 32 (2 row x
// 4 column), K in steps of 64 through four LDS stages (A 8 KB + B 16 KB:
// one workgroup of 8 waves per CU). The activation tile, which every
// column tile reads again, is half the DMA of a 64 x 64 tile; here a third.
template <int EPI>
__global__ void __launch_bounds__(512)
gemm_skinny_wide_kernel(GemmArgs g) {
  constexpr int SA = 64 * 128, SBW = 128 * 128;
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[SBW];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[SBW];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[SBW];
  __shared__ __attribute__((aligned(1024))) uint8_t sA3[SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB3[SBW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int tile = blockIdx.x, split = blockIdx.z;
  const int n0 = tile * 128;
  const int ksteps = g.K / BK;
  const int per = (ksteps + g.nsplit - 1) / g.nsplit;
  const int ks0 = split * per;
  const int n = max(0, min(ksteps, ks0 + per) - ks0);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)((int64_t)(g.M - 1) * g.lda * 2 + g.K * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)((int64_t)(g.N - 1) * g.ldb * 2 + g.K * 2));
  const int lr = lane >> 3;
  // DMA: A block `wave` (rows 8 wave ..), B blocks wave and wave + 8
  const int ra_row = wave * 8 + lr;
  const uint32_t aoff = (uint32_t)((int64_t)min(ra_row, g.M - 1) * g.lda * 2 +
                                   (((lane & 7) ^ ((ra_row >> 1) & 7)) << 4));
  uint32_t boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave + 8 * i) * 8 + lr;
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    boff[i] = (uint32_t)((int64_t)min(n0 + r, g.N - 1) * g.ldb * 2 + lc * 16);
  }
  const int fr = lane & 31, fh = lane >> 5;
  int loff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) loff[kk] = fr * 128 + (((2 * kk + fh) ^ ((fr >> 1) & 7)) << 4);

  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  // A blocks past the last row are not loaded (their MFMA rows are never
  // stored): 2 or 3 DMA per wave per step
  const bool has_a = wave * 8 < g.M;
  auto issue = [&](int ks, uint8_t* sa, uint8_t* sb) {
    const uint32_t ko = (uint32_t)ks * (BK * 2);
    if (has_a) dma16(ra, aoff, ko, sa + wave * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rb, boff[i], ko, sb + (wave + 8 * i) * 1024);
  };
  auto compute = [&](const uint8_t* sa0, const uint8_t* sb0) {
    const uint8_t* sa = sa0 + wm * 32 * 128;
    const uint8_t* sb = sb0 + wn * 32 * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(sa + loff[kk]);
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(sb + loff[kk]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
  };
  if (n > 0) {
    issue(ks0, sA0, sB0);
    issue(ks0 + min(1, n - 1), sA1, sB1);
    issue(ks0 + min(2, n - 1), sA2, sB2);
    auto step = [&](int i, const uint8_t* ca, const uint8_t* cb, uint8_t* sna, uint8_t* snb) {
      // steps i + 1, i + 2 stay in flight
      if (has_a) __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
      else __builtin_amdgcn_s_waitcnt(0x0F74);        // vmcnt(4)
      barrier_lds();
      issue(ks0 + min(i + 3, n - 1), sna, snb);
      if (i < n) compute(ca, cb);
    };
    for (int i = 0; i < n; i += 4) {
      step(i, sA0, sB0, sA3, sB3);
      step(i + 1, sA1, sB1, sA0, sB0);
      step(i + 2, sA2, sB2, sA1, sB1);
      step(i + 3, sA3, sB3, sA2, sB2);
    }
    wait_vm0();
  }

  const int col = n0 + wn * 32 + (lane & 31);
  if (col < g.N) {
    const float sc = (EPI == EPI_LOGITS) ? g.s1[col] : 1.f;
    float* C = g.C + (int64_t)split * g.split_stride;
    const int rbase = wm * 32 + (lane >> 5) * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rbase + (e >> 2) * 8 + (e & 3);
      if (row < g.M) C[(int64_t)row * g.ldc + col] = acc[e] * sc;
    }
  }
}


hipError_t launch_skinny(const GemmArgs& a, int epi, hipStream_t st) {
  if (a.M <= 64) {
    // the same split as 64-column tiles gives (N a multiple of 128: tiles x
    // split <= 256, one workgroup per CU)
    dim3 gw((a.N + 127) / 128, 1, a.nsplit);
    switch (epi) {
      case EPI_F32: hipLaunchKernelGGL((gemm_skinny_wide_kernel<EPI_F32>), gw, dim3(512), 0, st, a); break;
      case EPI_LOGITS: hipLaunchKernelGGL((gemm_skinny_wide_kernel<EPI_LOGITS>), gw, dim3(512), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid((a.N + 63) / 64, 1, a.nsplit), block(256);
  if (a.M > 64) {
    // 1-D grid: 8 pairs per round, every row block of each
    const int pairs = ((a.N + 63) / 64) * a.nsplit;
    grid = dim3((unsigned)(8 * ((a.M + 63) / 64) * ((pairs + 7) / 8)), 1, 1);
  }
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_skinny_kernel<EPI_F32>), grid, block, 0, st, a); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_skinny_kernel<EPI_LOGITS>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr int kLargeM = 1024;
static_assert(kGemmSkinnyMaxM < kLargeM, "the skinny range ends below the large-M kernel");

}  // namespace

int gemm_pick_split(int M, int N, int K, int max_split) {
  if (M >= kLargeM) return 1;
  const int ksteps = K / BK;
  if (M <= kGemmSkinnyMaxM) {
    // skinny path: the most workgroups that fit one round (2 per CU, 512),
    // at least SK_MAX K steps each, within max_split
    const int tiles = ((N + 63) / 64) * ((M + 63) / 64);
    int s = 1;
    while (s < max_split && tiles * (s + 1) <= 512 && ksteps / (s + 1) >= SK_MAX) ++s;
    return s;
  }
  return 1;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  if (a.K % BK != 0 || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
  if (epi != EPI_F32 && a.nsplit != 1) return hipErrorInvalidValue;
  if (a.Bq) {
    // MXFP8 weights: the small-M kernel with an fp32 output only
    const int ksteps = a.K / BK;
    if (a.M > 64 || epi != EPI_F32 || !a.Bs || a.nsplit < 1 ||
        (ksteps + a.nsplit - 1) / a.nsplit > MX_MAX_STEPS)
      return hipErrorInvalidValue;
    dim3 grid((a.N + 63) / 64, 1, a.nsplit), block(256);
    hipLaunchKernelGGL((gemm_skinny_fp8_kernel<EPI_F32>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  if (a.M >= kLargeM) return launch_big(a, epi, st);
  // below the large-M kernel only the fp32 and logit outputs exist
  if (epi != EPI_F32 && epi != EPI_LOGITS) return hipErrorInvalidValue;
  return launch_skinny(a, epi, st);
}

}  // namespace dory
