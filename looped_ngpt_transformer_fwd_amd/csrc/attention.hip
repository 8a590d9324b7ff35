// Gated grouped-query attention for gfx950.
//
// Prefill: flash attention on MFMA. One workgroup = one (batch row, KV head,
// query tile); its 8 waves cover the n_q/n_kv query heads of that KV group
// times 32-query blocks, so every K/V tile staged in LDS is reused by all
// query heads of the group. Scores are computed transposed,
// S^T = K Q^T (v_mfma_f32_32x32x16_bf16 with K as the A operand), so that in
// the accumulator layout each lane owns one query column: the softmax state
// needs a single lane-pair exchange per tile (none with the fixed reference:
// when the layer's s_qk bounds every score tightly enough, the bound is the
// softmax reference and no running maximum is kept). The
// output is likewise accumulated transposed, O^T += V^T P^T, with P^T taken
// straight from the score registers (converted to bf16) and V^T read from an
// LDS tile stored [head_dim][keys]. Keys come from two sources: the cache
// (positions below f_origin, ring-indexed for sliding-window layers) and the
// fresh K/V of the current step. Tiles wholly outside the causal or
// sliding-window band are skipped. The sigmoid gate is applied in the
// epilogue; the concatenation norm is left to the output projection's
// consumer (it cancels under N(y)).
//
// Decode: one query per sequence, the query/key transform of the token
// fused in; both contractions on MFMA with the KV group's query heads as the
// padded 16-wide side. Small batches split the keys (partial (max, sum, o)
// per split and a combine kernel that merges them and applies the gate);
// large batches take one workgroup per (sequence, KV head) that writes the
// gated output itself.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

constexpr int PF_WAVES = 8;
constexpr int PF_BN = 64;

__device__ __forceinline__ void dma16_flat(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_block, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm0_attn() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A pointer held in scalar registers (the value is the same in every lane).
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

// K/V tiles are staged by direct global->LDS DMA into two stages (the next
// tile's loads are in flight during the current tile's MFMAs). Both tiles are
// stored XOR-swizzled by row so that the MFMA fragment reads of consecutive
// rows hit distinct bank groups:
//   K tile   [BN keys][DH]   row = DH*2 bytes, chunk c of row r stored at c ^ kswz(r)
//   V^T tile [DH][BN keys]   row = BN*2 = 128 bytes, chunk c of row d at c ^ ((d / 2) & 7)
// The LDS serves a 16-byte read for 16 lanes per cycle from 64 banks (256
// bytes): the 16 key rows of one K fragment read must fall in 16 distinct
// 16-byte bank groups, so rows at the same offset within 256 bytes get
// distinct chunk XORs. The 8-byte V^T fragment reads conflict least with
// the chunk XORed by (d / 2) & 7 (measured with the LDS conflict counters:
// half the LDS cycles of the (d & 7) swizzle).
template <int DH>
__device__ __forceinline__ int kswz(int r) {
  constexpr int KCH = DH / 8;         // 16-byte chunks per row
  constexpr int RP = 256 / (DH * 2);  // rows per 256 bytes
  return (r / RP) & (KCH - 1);
}

template <int DH, int GRP, bool FRESH>
__global__ void __launch_bounds__(PF_WAVES * 64)
attn_prefill_kernel(AttnArgs a) {
  constexpr int QB = PF_WAVES / GRP;   // 32-query blocks per workgroup
  constexpr int BQ = QB * 32;          // queries per workgroup
  constexpr int BN = PF_BN;
  constexpr int KT_BYTES = BN * DH * 2;
  constexpr int VT_BYTES = DH * BN * 2;
  constexpr int KCH = DH / 8;
  constexpr int K_BLOCKS = KT_BYTES / 1024, V_BLOCKS = VT_BYTES / 1024;
  constexpr int KRPB = 1024 / (DH * 2);  // key rows per DMA block

  // Software pipeline over key tiles: iteration j computes the scores of
  // tile j + 1 on the matrix pipe while the softmax of tile j runs on the
  // VALU (the two are independent, so the compiler interleaves them), then
  // the P V product of tile j; the other wave of the SIMD fills the matrix
  // pipe meanwhile. K tiles are needed one iteration before their V tiles,
  // so each has its own ring of three LDS stages, filled by DMA: iteration j
  // loads K of tile j + 3 and V of tile j + 2, and waits for the loads of
  // iteration j - 2. Every stage is a separate array so that each LDS read
  // names its stage statically and the compiler does not drain DMA still
  // landing elsewhere.
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks2[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[VT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[VT_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs2[VT_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work order: heaviest query tiles (most keys under the causal mask) first.
  // Workgroups are dispatched round-robin over the 8 XCDs; when the (batch,
  // KV head) pairs split evenly, XCD x serves pairs x, x+8, ... only, so the
  // K/V of a pair is shared through one XCD's L2.
  const int ntq = gridDim.x, npairs = gridDim.y * gridDim.z;
  int qt, g, b;
  {
    const int lin = blockIdx.x + ntq * (blockIdx.y + gridDim.y * blockIdx.z);
    if ((npairs & 7) == 0) {
      const int x = lin & 7, j = lin >> 3;
      const int ppx = npairs >> 3;
      const int pair = x + 8 * (j % ppx);
      qt = ntq - 1 - j / ppx;
      g = pair % gridDim.y;
      b = pair / gridDim.y;
    } else {
      qt = ntq - 1 - blockIdx.x;
      g = blockIdx.y;
      b = blockIdx.z;
    }
  }
  // a sequence that has left the loop needs no attention output (its state
  // is not updated); the whole workgroup leaves before any barrier
  if (a.rl.k_rows && a.rl.loop >= a.rl.k_rows[b]) return;
  const int qb = wave / GRP, head = g * GRP + (wave % GRP);
  const int C = a.C;
  const int t0 = qt * BQ + qb * 32;
  const int tq = t0 + (lane & 31);
  const int hl = lane >> 5;
  const int64_t bg = (int64_t)b * a.n_kv + g;
  const int pq = (int)a.p0 + tq;  // positions fit 31 bits (at most 2^24)

  // |s_qk| for the fixed softmax reference (loaded first: the waits for the
  // DMA below count only younger loads)
  float sqk_m = 0.f;
  if (a.ref_s_qk) {
#pragma unroll
    for (int d = lane; d < DH; d += 64) sqk_m = fmaxf(sqk_m, fabsf(a.ref_s_qk[d]));
  }

  bf16x8 qf[DH / 16];
  {
    const int tc = min(tq, C - 1);
    const uint16_t* qrow = a.q + (((int64_t)b * a.n_q + head) * C + tc) * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 16 + hl * 8);
  }

  floatx16 o[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  const int tw0 = qt * BQ;
  const int tw1 = min(C, tw0 + BQ) - 1;
  const int64_t p_lo = a.p0 + tw0, p_hi = a.p0 + tw1;
  int64_t k_lo = 0;
  if (a.window > 0) k_lo = max((int64_t)0, p_lo - a.window + 1);
  const int64_t kt_first = (k_lo / BN) * BN;
  const int ntiles = (int)((p_hi - kt_first) / BN) + 1;

  // per-wave query extent
  const bool wave_live = t0 < C;
  const int wq_lo = (int)a.p0 + t0, wq_hi = (int)a.p0 + min(t0 + 31, C - 1);

  // Fragment read offsets (lane parts). Row r of the S^T product's A operand
  // is key row perm(r) of the K tile, perm swapping bits 2 and 3 of r: in the
  // 32x32 accumulator layout lane l then holds, in elements 8 h .. 8 h + 7,
  // the scores of keys 16 h + 8 (l / 32) + 0 .. 7 of each 32-key block,
  // which is exactly the k-slice lane l supplies to the P V product. So the
  // V^T operand of a lane is 8 consecutive keys of one head dimension: one
  // 16-byte LDS read, and P needs no shuffle.
  int koff[DH / 16];
#pragma unroll
  for (int s = 0; s < DH / 16; ++s) {
    const int r0 = lane & 31;
    const int r = (r0 & 0x13) | ((r0 & 4) << 1) | ((r0 & 8) >> 1);
    koff[s] = r * DH * 2 + (((2 * s + hl) ^ kswz<DH>(r)) << 4);
  }
  int voff[BN / 32][2];
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int d = lane & 31;
      const int c = kb * 4 + kc * 2 + hl;  // keys 8 c .. 8 c + 7 of the tile
      voff[kb][kc] = d * (BN * 2) + ((c ^ ((d >> 1) & 7)) << 4);
    }

  // Source rows are chosen with selects, not branches: a branch between the
  // DMA and the LDS reads makes the compiler drain the DMA in flight before
  // the reads. Positions, rows and element offsets fit 31 bits (positions
  // are checked on the host: at most 2^24), so the per-lane arithmetic is
  // 32-bit: a key at offset rel + r from the fresh buffer's origin (rel the
  // uniform tile start minus f_origin) is a cache row when that is negative,
  // else a fresh row. A lane's row (K) or 8-key column group (V) within a
  // tile is the same in every tile, so its remainder modulo the ring is taken
  // once; per tile only the (uniform) remainder of the tile start is added,
  // with one conditional subtraction. A layer without a ring uses a divisor
  // above every position.
  const uint32_t ring_div = a.ring > 0 ? (uint32_t)a.ring : 0x7FFFFFFFu;
  // the four base pointers as uniform values (a select between two fields of
  // the argument block would become a per-lane load of the selected field)
  const uint16_t* const kcb = uniform_ptr(a.kc + bg * a.c_rows * DH);
  const uint16_t* const kfb = uniform_ptr(a.kf + bg * a.f_rows * DH);
  const uint16_t* const vcb = uniform_ptr(a.vc + bg * DH * a.c_rows);
  const uint16_t* const vfb = uniform_ptr(a.vf + bg * DH * a.f_rows);
  const int f_org = (int)a.f_origin;
  const int k_last = (int)a.f_rows - 1;
  // V^T columns from the last 8-key group holding step keys or zeros on:
  // groups at or past the step's end read that group instead (finite values
  // that meet probabilities of exactly 0)
  const int v_last = (int)((a.p0 + C - a.f_origin + 7) / 8 * 8) - 8;
  const int kt_first32 = (int)kt_first;
  constexpr int KJ = (K_BLOCKS + PF_WAVES - 1) / PF_WAVES;
  constexpr int VJ = (V_BLOCKS + PF_WAVES - 1) / PF_WAVES;
  uint32_t k_rm[KJ], v_cm[VJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) k_rm[j] = (uint32_t)((wave + j * PF_WAVES) * KRPB + lane / KCH) % ring_div;
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int d = (wave + j * PF_WAVES) * 8 + (lane >> 3);
    v_cm[j] = (uint32_t)(((lane & 7) ^ ((d >> 1) & 7)) * 8) % ring_div;
  }
  const uint32_t c_rows32 = (uint32_t)a.c_rows, f_rows32 = (uint32_t)a.f_rows;
  auto issue_k = [&](int it, uint8_t* kst) __attribute__((always_inline)) {
    const int kt = kt_first32 + min(it, ntiles - 1) * BN;
    const int rel = kt - f_org;
    const uint32_t km = (uint32_t)kt % ring_div;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int blk = wave + j * PF_WAVES;
      if (K_BLOCKS % PF_WAVES != 0 && blk >= K_BLOCKS) break;
      const int r = blk * KRPB + lane / KCH;
      const int c = (lane % KCH) ^ kswz<DH>(r);
      const int ur = rel + r;
      uint32_t ci = km + k_rm[j];
      ci = min(ci, ci - ring_div);
      if constexpr (FRESH) {
        // every key of the launch is a step key (no cache rows below it)
        dma16_flat(kfb + ((uint32_t)min(ur, k_last) * DH + c * 8), kst + blk * 1024);
      } else {
        const bool in_cache = ur < 0;
        const uint32_t row = in_cache ? ci : (uint32_t)min(ur, k_last);
        dma16_flat((in_cache ? kcb : kfb) + (row * DH + c * 8), kst + blk * 1024);
      }
    }
  };
  auto issue_v = [&](int it, uint8_t* vst) __attribute__((always_inline)) {
    const int kt = kt_first32 + min(it, ntiles - 1) * BN;
    const int rel = kt - f_org;
    const uint32_t km = (uint32_t)kt % ring_div;
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      const int blk = wave + j * PF_WAVES;
      if (V_BLOCKS % PF_WAVES != 0 && blk >= V_BLOCKS) break;
      const int d = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((d >> 1) & 7);
      const int ur = rel + c * 8;
      uint32_t ci = km + v_cm[j];
      ci = min(ci, ci - ring_div);
      if constexpr (FRESH) {
        dma16_flat(vfb + ((uint32_t)d * f_rows32 + (uint32_t)min(ur, v_last)), vst + blk * 1024);
      } else {
        const bool in_cache = ur < 0;
        // both offsets, then a bitwise select (a plain select of the two sums
        // is turned into a divergent branch)
        const uint32_t sel = (uint32_t)(ur >> 31);
        const uint32_t off = (((uint32_t)d * c_rows32 + ci) & sel) |
                             (((uint32_t)d * f_rows32 + (uint32_t)min(ur, v_last)) & ~sel);
        dma16_flat((in_cache ? vcb : vfb) + off, vst + blk * 1024);
      }
    }
  };
  // DMA instructions this wave issues per K tile and per V tile
  const int kpw = K_BLOCKS > wave ? (K_BLOCKS - wave + PF_WAVES - 1) / PF_WAVES : 0;
  const int vpw = V_BLOCKS > wave ? (V_BLOCKS - wave + PF_WAVES - 1) / PF_WAVES : 0;
  // s_waitcnt vmcnt(n) (expcnt and lgkmcnt not waited). The count must be a
  // compile-time constant wherever it can be (every wave issues the same
  // number of DMA when the blocks divide evenly): with a count chosen at run
  // time the compiler cannot tell which DMA an LDS read depends on and
  // drains them all before it.
  constexpr bool kEven = K_BLOCKS % PF_WAVES == 0 && V_BLOCKS % PF_WAVES == 0;
  constexpr int kPW = K_BLOCKS / PF_WAVES, vPW = V_BLOCKS / PF_WAVES;
  auto wait_vm = [](int n) __attribute__((always_inline)) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
      case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    }
  };

  // S^T of one tile: 32 keys x 32 queries per accumulator, two per tile
  auto scores = [&](const uint8_t* kst, floatx16 (&sacc)[BN / 32]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(kst + kb * 32 * DH * 2 + koff[s]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qf[s], sacc[kb], 0, 0, 0);
      }
    }
  };
  // O^T += V^T P^T of one tile
  auto pv = [&](const uint8_t* vst, const bf16x8 (&pf)[BN / 32][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) {
      const uint8_t* vrow = vst + db * 32 * (BN * 2);
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 vfr = *reinterpret_cast<const bf16x8*>(vrow + voff[kb][kc]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr, pf[kb][kc], o[db], 0, 0, 0);
        }
    }
  };
  // the maximum score of each query over a tile (the two lanes holding a
  // query's keys exchange theirs)
  auto tile_max = [&](const floatx16 (&sacc)[BN / 32]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    return fmaxf(mx, __shfl_xor(mx, 32, 64));
  };
  // masks of an edge (or dead) tile, applied to its scores; the tile's
  // maximum (taken before masking) is then taken again
  auto mask = [&](auto fixed, int it, floatx16 (&sacc)[BN / 32], float& mx) __attribute__((always_inline)) {
    const int kt = kt_first32 + it * BN;
    const bool interior = wave_live && kt + BN - 1 <= wq_lo &&
                          (a.window == 0 || wq_hi - kt < a.window);
    if (interior) return;
    const int rel0 = pq - kt - hl * 8;  // pq - (key index within tile)
    const bool qok = tq < C;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int dist = rel0 - (kb * 32 + (e >> 3) * 16 + (e & 7));  // pq - u
        const bool vis = qok && dist >= 0 && (a.window == 0 || dist < a.window);
        if (!vis) sacc[kb][e] = -INFINITY;
      }
    if constexpr (!decltype(fixed)::value) mx = tile_max(sacc);
  };
  // Online softmax in base 2 with lazy rescaling: the reference maximum
  // m_run moves only when a tile's maximum exceeds it by more than 8 in
  // base-2 units, so probabilities stay below 2^8 and o and l are rescaled
  // rarely; the final o / l is the same softmax either way. From m_run =
  // -inf the first visible score always moves it (exp2(-inf) = 0 rescales
  // the empty o and l), and all-masked queries keep -inf and get
  // probabilities of 0. reference() returns the factor by which o and l
  // must be rescaled (1 if the reference did not move).
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float nm = 0.f;  // -m_run in base-2 units (0 while m_run = -inf)
  auto reference = [&](float mx) __attribute__((always_inline)) {
    const bool grow = (mx - m_run) * sl2 > 8.f;
    const float m_new = grow ? mx : m_run;
    // branch-free: exp2(0) = 1 when the reference stays, exp2(-inf) = 0 when
    // it leaves -inf
    const float corr = __builtin_amdgcn_exp2f(grow ? (m_run - m_new) * sl2 : 0.f);
    m_run = m_new;
    nm = -(m_run == -INFINITY ? 0.f : m_run) * sl2;
    return corr;
  };
  // bf16 probabilities of one tile under the current reference
  auto probs = [&](const floatx16 (&sacc)[BN / 32], bf16x8 (&pf)[BN / 32][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[kb][h][e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * h + e], sl2, nm)));
  };
  // l sums the same bf16 probabilities that enter the P V product
  auto prob_sum = [&](const bf16x8 (&pf)[BN / 32][2]) __attribute__((always_inline)) {
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pp;
          pp[0] = pf[kb][h][e];
          pp[1] = pf[kb][h][e + 1];
          if (e & 2) lb = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lb, false);
          else la = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, la, false);
        }
    return la + lb;
  };
  auto rescale = [&](float corr) __attribute__((always_inline)) {
    if (__ballot(corr != 1.f)) {
#pragma unroll
      for (int i = 0; i < DH / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= corr;
    }
  };

  // the DMA stream starts while the query fragments are in flight: they were
  // issued first, so every vmcnt wait below (which counts the most recent
  // DMA) also covers them
  issue_k(0, ks0);
  issue_k(1, ks1);
  issue_v(0, vs0);
  issue_k(2, ks2);
  issue_v(1, vs1);
  if constexpr (kEven) {
    static_assert(2 * kPW + 2 * vPW <= 15, "wait count");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kPW + 2 * vPW));  // tile 0's K has landed
  } else {
    wait_vm(2 * kpw + 2 * vpw);
  }
  barrier_lds();
  floatx16 sc[BN / 32], sn[BN / 32];
  bf16x8 pf[BN / 32][2];
  scores(ks0, sc);

  // Fixed softmax reference. q and k heads are s_qk times unit vectors, so
  // every raw score lies in [-B, B] with B = max |s_qk|^2 (times 1 + 2^-6
  // for the bf16 rounding of q and k). When 2 B scale log2(e) <= 120 the
  // probabilities exp2((s - B) scale log2(e)) are normal fp32 and bf16
  // numbers in (2^-120, 1] for every possible score, so B serves as the
  // reference itself: no running maximum, no rescaling, no per-tile lane
  // exchange. Otherwise (or without s_qk) the running maximum below. The
  // normalized result o / l is the same softmax either way.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sqk_m = fmaxf(sqk_m, __shfl_xor(sqk_m, o, 64));
  const float ref_b = sqk_m * sqk_m * (1.f + 1.f / 64.f);
  const bool fixed_ref =
      __builtin_amdgcn_readfirstlane((int)(a.ref_s_qk != nullptr && ref_b * sl2 <= 60.f)) != 0;

  // Iteration j: K read from stage (j + 1) % 3 and K of tile j + 3 loaded
  // into stage j % 3; V read from stage j % 3 and V of tile j + 2 loaded
  // into stage (j + 2) % 3. Loads past the last tile reload it (uniform
  // counts, no branch around the DMA); the scores computed from such a
  // reload after the last tile are discarded. s_cur holds the scores of tile
  // j on entry and mx their maximum (as computed before masking); s_next
  // receives the scores of tile j + 1 and mx their maximum. After the
  // reference update (and the rare rescale) one block runs the scores of
  // tile j + 1 and the P V product of tile j on the matrix pipe, with the
  // probabilities of tile j, their sum and the maximum of tile j + 1 on the
  // VALU in between. With the fixed reference the maxima and the reference
  // update are left out.
  auto run = [&](auto fixed) __attribute__((always_inline)) {
    constexpr bool FIX = decltype(fixed)::value;
    float mx = 0.f;
    if constexpr (FIX) nm = -ref_b * sl2;
    else mx = tile_max(sc);
    auto iter = [&](int j, const uint8_t* kr, uint8_t* kw, const uint8_t* vr, uint8_t* vw,
                    floatx16 (&s_cur)[BN / 32], floatx16 (&s_next)[BN / 32])
        __attribute__((always_inline)) {
      // the loads of iteration j - 2 (K of j + 1, V of j) have landed
      if constexpr (kEven) __builtin_amdgcn_s_waitcnt(0x0F70 | (kPW + vPW));
      else wait_vm(kpw + vpw);
      barrier_lds();
      issue_k(j + 3, kw);
      issue_v(j + 2, vw);
      mask(fixed, j, s_cur, mx);
      if constexpr (!FIX) {
        const float corr = reference(mx);
        l_run *= corr;
        rescale(corr);
      }
      scores(kr, s_next);
      probs(s_cur, pf);
      pv(vr, pf);
      l_run += prob_sum(pf);
      if constexpr (!FIX) mx = tile_max(s_next);
      // interleave: per MFMA (the next tile's scores, then this tile's
      // product) one LDS fragment read and a share of the VALU work
      constexpr int NMF = 2 * (BN / 32) * (DH / 16);
      constexpr int AHEAD = 4;  // fragment reads in flight ahead of their MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS read
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i + AHEAD < NMF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
    };
    for (int j = 0;; j += 6) {
      iter(j, ks1, ks0, vs0, vs2, sc, sn);
      if (j + 1 >= ntiles) break;
      iter(j + 1, ks2, ks1, vs1, vs0, sn, sc);
      if (j + 2 >= ntiles) break;
      iter(j + 2, ks0, ks2, vs2, vs1, sc, sn);
      if (j + 3 >= ntiles) break;
      iter(j + 3, ks1, ks0, vs0, vs2, sn, sc);
      if (j + 4 >= ntiles) break;
      iter(j + 4, ks2, ks1, vs1, vs0, sc, sn);
      if (j + 5 >= ntiles) break;
      iter(j + 5, ks0, ks2, vs2, vs1, sn, sc);
      if (j + 6 >= ntiles) break;
    }
  };
  if (fixed_ref) run(std::true_type{});
  else run(std::false_type{});
  // ---- epilogue: normalize, gate, store z[b*C + t][head*DH + d]. The O^T
  // registers hold one query per lane, so the 32 x DH tile of a wave is
  // transposed through LDS (the stage buffers, free after the loop; two
  // waves per K stage and the first V stage, rows of DH * 2 bytes with the
  // 16-byte chunk c of row q stored at c ^ (q mod chunks per row)) and
  // written as contiguous 16-byte pieces of each query row. The gate loads
  // are issued first, so their latency overlaps the wait for the last
  // (clamped) K/V loads and the staging.
  constexpr int CPR = DH / 8;            // 16-byte chunks per query row
  constexpr int EPJ = 32 * CPR / 64;     // chunks per lane
  static_assert(2 * 32 * DH * 2 <= KT_BYTES, "epilogue staging");
  const int dq = a.n_q * DH;
  // the lane index afresh (mbcnt), so that nothing derived from it has to be
  // kept through the tile loop
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  uint4 gv[EPJ];
#pragma unroll
  for (int j = 0; j < EPJ; ++j) {
    const int c = ln + 64 * j;
    // unconditional (rows past the step read its last row, unused) so that
    // the loads stay in flight together
    const int t = min(t0 + c / CPR, C - 1);
    gv[j] = *reinterpret_cast<const uint4*>(a.gate + ((int64_t)b * C + t) * dq + head * DH + (c % CPR) * 8);
  }
  l_run += __shfl_xor(l_run, 32, 64);
  const float il = l_run > 0.f ? 1.0f / l_run : 0.f;
  wait_vm0_attn();  // the clamped reloads have landed before the stages are reused
  __syncthreads();  // and every wave has finished reading them
  uint8_t* const buf = (wave < 2 ? ks0 : wave < 4 ? ks1 : wave < 6 ? ks2 : vs0) + (wave & 1) * (32 * DH * 2);
  {
    const int q = ln & 31;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int eq = 0; eq < 4; ++eq) {
        const int c = db * 4 + eq;  // 16-byte chunk of dims 8 c .. 8 c + 7
        bf16x4 v4;
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = static_cast<__bf16>(o[db][eq * 4 + j] * il);
        *reinterpret_cast<bf16x4*>(buf + q * (DH * 2) + ((c ^ (q % CPR)) << 4) + (ln >> 5) * 8) = v4;
      }
  }
  // each wave reads back only what it wrote (LDS operations of a wave are
  // processed in order)
#pragma unroll
  for (int j = 0; j < EPJ; ++j) {
    const int c = ln + 64 * j;
    const int q = c / CPR, cc = c % CPR;
    const int t = t0 + q;
    if (t < C) {
      const uint4 ov = *reinterpret_cast<const uint4*>(buf + q * (DH * 2) + ((cc ^ (q % CPR)) << 4));
      const uint16_t* oe = reinterpret_cast<const uint16_t*>(&ov);
      const uint16_t* ge = reinterpret_cast<const uint16_t*>(&gv[j]);
      uint4 zv;
      uint16_t* ze = reinterpret_cast<uint16_t*>(&zv);
#pragma unroll
      for (int k = 0; k < 8; ++k) ze[k] = f2bf(bf2f(oe[k]) * bf2f(ge[k]));
      *reinterpret_cast<uint4*>(a.z + ((int64_t)b * C + t) * dq + head * DH + cc * 8) = zv;
    }
  }
}

// ------------------------------------------------------------------ decode
constexpr int DEC_NT = 256;
// Keys per split (multiples of 64): sliding-window layers and contexts up to
// DEC_LONG keys use DEC_SWAK / DEC_MAXK (more workgroups in flight); longer
// full-attention contexts use DEC_LONGK, which halves the partials that the
// combine kernel merges per (sequence, head).
constexpr int DEC_MAXK = 256;
constexpr int DEC_SWAK = 256;
constexpr int DEC_LONGK = 512;
constexpr int64_t DEC_LONG = 65536;

__device__ __forceinline__ bf16x8 load16_or_zero(const uint16_t* p, bool ok) {
  bf16x8 v;
  if (ok) {
    v = *reinterpret_cast<const bf16x8*>(p);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (__bf16)0.f;
  }
  return v;
}

// One workgroup per (split, KV head, sequence); the keys of the query at
// position p are [lo, p] (lo = p - W + 1 for sliding-window layers), splits
// are windows of SPLITK keys (DEC_MAXK for full attention, DEC_SWAK for the
// short sliding-window ranges) aligned to 64 starting at floor(lo / 64) * 64,
// and each wave takes SPLITK / 4 consecutive keys of its split in blocks of 32.
// Both contractions run on v_mfma_f32_16x16x32_bf16 with the GRP query heads
// of the KV group as the (zero-padded) 16-wide dimension:
//   S^T block = K Q^T: A = 16 key rows (lane l: row l % 16, dims 8 (l / 16)
//     .. + 7 of each 32-dim slice), B = Q^T (lane l: head l % 16). Tile t of
//     a 32-key block puts key u0 + 8 (r / 4) + 4 t + r % 4 in row r, so the
//     output lane (G = l / 16, head l % 16) holds the scores of keys
//     u0 + 8 G + j, j = 0..7: exactly the A operand of the P V product.
//   O += P V: A = P (lane: head l % 16, keys 8 (l / 16) .. + 7), B = V^T rows
//     (lane: dim l % 16 of a 16-dim block, the same 8 keys, one 16-byte read).
// Online softmax per wave in base 2; P is rounded to bf16 for the product.
// Keys outside [lo, p] are never read (cache rows past p may not be written)
// and enter as zero K/V rows with probability 0. The four waves merge their
// (max, sum, o) in LDS into the split's partial.
// DIRECT (batches with at least one workgroup per CU per (sequence, KV
// head)): one workgroup of NT threads takes every key of its (sequence, KV
// head), wave w the 32-key blocks w, w + NT / 64, ..., and the merge writes
// the gated output z itself (no partials, no combine launch).
template <int DH, int GRP, int SPLITK, bool DIRECT = false, int NT = DEC_NT>
__global__ void __launch_bounds__(NT, 2)  // two waves per SIMD
attn_decode_kernel(AttnArgs a, int nsplit, float* part) {
  constexpr int NWV = NT / 64;
  constexpr int DEC_WKEYS = DIRECT ? 64 : SPLITK / NWV;  // keys per wave (split form)
  constexpr int NS = DH / 32;   // 32-dim slices of the q.k contraction
  constexpr int NB = DH / 16;   // 16-dim blocks of the output
  static_assert(GRP <= 16, "query heads per KV head must fit the 16-wide MFMA side");
  __shared__ float wmax[NWV][GRP];
  __shared__ float wsum[NWV][GRP];
  __shared__ float wout[NWV][GRP][DH];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.rl.k_rows && a.rl.loop >= a.rl.k_rows[b]) {  // left the loop
    if (DIRECT)  // (the split form's combine writes the zeros)
      for (int i = tid; i < GRP * DH; i += NT) a.z[((int64_t)b * a.n_q + g * GRP) * DH + i] = 0;
    return;
  }
  const int G = lane >> 4, r = lane & 15;
  const int64_t bg = (int64_t)b * a.n_kv + g;
  const int64_t p = a.p0_dev ? *a.p0_dev : a.p0;
  int64_t lo = 0;
  if (a.window > 0) lo = max((int64_t)0, p - a.window + 1);
  const int64_t A = (lo / 64) * 64 + (int64_t)split * SPLITK;
  if (A > p) return;  // a split past the query's last key (launched for longer contexts)
  const int64_t ua = max(lo, A), ub = DIRECT ? p + 1 : min(p + 1, A + SPLITK);
  const int64_t w0 = A + (int64_t)wave * DEC_WKEYS;

  const bool holds_p = DIRECT || p < A + SPLITK;  // this workgroup's keys include p
  __shared__ __attribute__((aligned(16))) uint16_t qs[GRP][DH];
  bf16x8 qb[NS];
  floatx4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[nb][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  // buffer resources over this (sequence, KV head)'s K rows and V^T rows:
  // 32-bit offsets, and an offset past the end reads zeros
  const uint32_t kbytes = (uint32_t)(a.c_rows * DH * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.kc + bg * a.c_rows * DH), (short)0, (int)kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.vc + bg * DH * a.c_rows), (short)0, (int)kbytes, 0x00020000);
  const uint32_t OOB = 0xFFFFFFF0u;

  // loads of the 32-key block from key u0 into (kf, vf): keys outside
  // [lo, p] read as zeros
  auto load = [&](int64_t u0, bf16x8 (&kf)[2][NS], bf16x8 (&vf)[NB]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t u = u0 + 8 * (r >> 2) + 4 * t + (r & 3);
      const int64_t row = cache_row(u, a.ring);
      const uint32_t off = (u >= ua && u < ub) ? (uint32_t)(row * DH + 8 * G) * 2u : OOB;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 64 * s, 0);
        kf[t][s] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // V^T chunks of 8 keys are aligned to 8 and lie inside the slot whenever
    // their first key is a cached position
    const int64_t uv = u0 + 8 * G;
    const bool vany = uv + 7 >= ua && uv < ub;
    const uint32_t voff = vany ? (uint32_t)(cache_row(uv, a.ring) * 2 + r * a.c_rows * 2) : OOB;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, (int)(16 * nb * a.c_rows * 2), 0);
      vf[nb] = __builtin_bit_cast(bf16x8, v);
    }
  };
  auto compute = [&](int64_t u0, const bf16x8 (&kf)[2][NS], bf16x8 (&vf)[NB]) {
    if (u0 + 31 < ua || u0 >= ub) return;  // the whole block is outside [lo, p]
    const int64_t uv = u0 + 8 * G;
    if (!(uv >= ua && uv + 7 < ub)) {
      // keys outside [lo, p] in this lane's V chunk are zeroed
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t u = uv + j;
        if (u < ua || u >= ub) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) vf[nb][j] = (__bf16)0.f;
        }
      }
    }
    floatx4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[t][e] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][s], qb[s], sacc[t], 0, 0, 0);
    }
    float sv[8];
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t u = uv + 4 * t + e;
        const float x = (u >= ua && u < ub) ? sacc[t][e] * sl2 : -INFINITY;
        sv[4 * t + e] = x;
        mb = fmaxf(mb, x);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m_run, mb);      // finite: the block holds a key
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    bf16x8 pf;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pj = __builtin_amdgcn_exp2f(sv[j] - m_new);
      ps += pj;
      pf[j] = (__bf16)pj;
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // o rows are heads 4 (l / 16) + e; their rescale factors sit in lanes 0..15
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ae = __shfl(alpha, 4 * G + e, 64);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb][e] *= ae;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf[nb], o[nb], 0, 0, 0);
  };

  auto prep = [&]() {
    // Fused query/key transform: the group's query heads from the projection
    // partials (RoPE, per-head L2 norm, s_qk) into LDS; the workgroup whose
    // keys include p also computes the token's key and value and stores them
    // in the cache before its key loads (the only workgroup that reads them).
    if (a.qkv_part) {
      constexpr int HALF = DH / 2;
      const int64_t N = 2 * (int64_t)a.n_q * DH + 2 * (int64_t)a.n_kv * DH;
      const float* row = a.qkv_part + (int64_t)b * N;
      const int64_t prow = cache_row(p, a.ring);
      const int nh = GRP + (holds_p ? 1 : 0);
      for (int hh = wave; hh < nh; hh += NWV) {  // head GRP: the KV head's key
        const int col = hh < GRP ? (g * GRP + hh) * DH : a.n_q * DH + g * DH;
        float r1 = 0.f, r2 = 0.f;
        if (lane < HALF) {
          const float x1 = sum_splits(row + col + lane, a.qkv_nsplit, a.qkv_ss);
          const float x2 = sum_splits(row + col + lane + HALF, a.qkv_nsplit, a.qkv_ss);
          const float c = a.cs[lane], sn = a.sn[lane];
          r1 = x1 * c - x2 * sn;
          r2 = x2 * c + x1 * sn;
        }
        const float inv = 1.0f / sqrtf(wave_sum(r1 * r1 + r2 * r2));
        if (lane < HALF) {
          const uint16_t v1 = f2bf(a.s_qk[lane] * r1 * inv), v2 = f2bf(a.s_qk[lane + HALF] * r2 * inv);
          if (hh < GRP) {
            qs[hh][lane] = v1;
            qs[hh][lane + HALF] = v2;
          } else {
            uint16_t* kr = const_cast<uint16_t*>(a.kc) + (bg * a.c_rows + prow) * DH;
            kr[lane] = v1;
            kr[lane + HALF] = v2;
          }
        }
      }
      if (holds_p) {
        for (int d = tid; d < DH; d += NT) {
          const float v = sum_splits(row + (int64_t)a.n_q * DH + (int64_t)a.n_kv * DH + g * DH + d,
                                     a.qkv_nsplit, a.qkv_ss);
          const_cast<uint16_t*>(a.vc)[(bg * DH + d) * a.c_rows + prow] = f2bf(v);
        }
        __threadfence_block();  // the token's K/V stores complete before the key loads
      }
      __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (a.qkv_part) {
        qb[s] = *reinterpret_cast<const bf16x8*>(&qs[r < GRP ? r : 0][32 * s + 8 * G]);
        if (r >= GRP) {
#pragma unroll
          for (int j = 0; j < 8; ++j) qb[s][j] = (__bf16)0.f;
        }
      } else {
        qb[s] = load16_or_zero(a.q + ((int64_t)b * a.n_q + g * GRP + (r < GRP ? r : 0)) * DH + 32 * s + 8 * G,
                               r < GRP);
      }
    }
  };

  // two register sets: the loads of the next block are in flight while a
  // block computes
  bf16x8 kfa[2][NS], vfa[NB], kfb[2][NS], vfb[NB];
  // a block may be loaded before the transform unless it holds key p (whose
  // K/V the transform stores), so its loads overlap the transform's
  auto early_ok = [&](int64_t u0) { return !(a.qkv_part && holds_p) || u0 + 31 < p; };
  if constexpr (DIRECT) {
    // this wave's blocks: keys A + 32 (wave + NWV i), i < nbw
    const int64_t nblk = (p + 1 - A + 31) / 32;
    const int nbw = (int)((nblk - wave + NWV - 1) / NWV);
    auto ub0 = [&](int i) { return A + 32 * ((int64_t)wave + (int64_t)NWV * i); };
    const bool e0 = nbw > 0 && early_ok(ub0(0)), e1 = nbw > 1 && early_ok(ub0(1));
    if (e0) load(ub0(0), kfa, vfa);
    if (e1) load(ub0(1), kfb, vfb);
    prep();
    if (nbw > 0 && !e0) load(ub0(0), kfa, vfa);
    if (nbw > 1 && !e1) load(ub0(1), kfb, vfb);
    for (int i = 0; i < nbw; i += 2) {
      compute(ub0(i), kfa, vfa);
      if (i + 2 < nbw) load(ub0(i + 2), kfa, vfa);
      if (i + 1 < nbw) {
        compute(ub0(i + 1), kfb, vfb);
        if (i + 3 < nbw) load(ub0(i + 3), kfb, vfb);
      }
    }
  } else {
    constexpr int NBLK = DEC_WKEYS / 32;
    static_assert(NBLK % 2 == 0, "blocks per wave come in pairs");
    const bool e0 = early_ok(w0), e1 = early_ok(w0 + 32);
    if (e0) load(w0, kfa, vfa);
    if (e1) load(w0 + 32, kfb, vfb);
    prep();
    if (!e0) load(w0, kfa, vfa);
    if (!e1) load(w0 + 32, kfb, vfb);
#pragma unroll
    for (int blk = 0; blk < NBLK; blk += 2) {
      compute(w0 + 32 * blk, kfa, vfa);
      if (blk + 2 < NBLK) load(w0 + 32 * (blk + 2), kfa, vfa);
      compute(w0 + 32 * (blk + 1), kfb, vfb);
      if (blk + 3 < NBLK) load(w0 + 32 * (blk + 3), kfb, vfb);
    }
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (G == 0 && r < GRP) {
    wmax[wave][r] = m_run;
    wsum[wave][r] = l_run;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * G + e;
    if (h < GRP) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wout[wave][h][16 * nb + r] = o[nb][e];
    }
  }
  __syncthreads();
  for (int i = tid; i < GRP * DH; i += NT) {
    const int h = i / DH, d = i % DH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, wmax[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float f = __builtin_amdgcn_exp2f(wmax[w][h] - M);
        L += wsum[w][h] * f;
        O += wout[w][h][d] * f;
      }
    }
    if constexpr (DIRECT) {
      const int64_t zi = ((int64_t)b * a.n_q + g * GRP + h) * DH + d;
      float gv;
      if (a.qkv_part) {
        const int64_t N = 2 * (int64_t)a.n_q * DH + 2 * (int64_t)a.n_kv * DH;
        const float x = sum_splits(a.qkv_part + (int64_t)b * N + (int64_t)a.n_q * DH +
                                       2 * (int64_t)a.n_kv * DH + (g * GRP + h) * DH + d,
                                   a.qkv_nsplit, a.qkv_ss);
        gv = bf2f(f2bf(1.0f / (1.0f + __expf(-x))));
      } else {
        gv = bf2f(a.gate[zi]);
      }
      a.z[zi] = f2bf(O / L * gv);
      continue;
    }
    float* dst = part + (((int64_t)b * a.n_q + g * GRP + h) * nsplit + split) * (DH + 2);
    dst[2 + d] = O;
    if (d == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// grid B * n_q * (dh / dc), block G groups of dc threads: a workgroup
// takes dc output dims of one (sequence, head), thread i of a group dim i.
// Group j merges splits j, j + G, ... online (running maximum, rescaled sum
// and output), loading eight splits at a time, so a long context (hundreds
// of splits) costs a few round trips; the G group results are merged
// through LDS.
constexpr int COMB_NT = 1024;
__global__ void __launch_bounds__(COMB_NT)
attn_decode_combine_kernel(const float* part, int nsplit, int n_q, int dh, int dc,
                           const uint16_t* gate, uint16_t* z, RowLoops rl, int sk, int window,
                           int64_t p0, const int64_t* p0_dev, const float* qkv_part, int qkv_nsplit,
                           int64_t qkv_ss, int n_kv) {
  __shared__ float gm[COMB_NT / 32], gl[COMB_NT / 32];
  __shared__ float go[COMB_NT];
  const int nch = dh / dc;
  const int bh = blockIdx.x / nch, ch = blockIdx.x - bh * nch;
  const int b = bh / n_q, h = bh % n_q;
  const int G = blockDim.x / dc, grp = threadIdx.x / dc, dl = threadIdx.x - grp * dc;
  const int d = ch * dc + dl;
  const int64_t idx = (int64_t)b * n_q * dh + h * dh + d;
  if (rl.k_rows && rl.loop >= rl.k_rows[b]) {  // left the loop: no partials were written
    if (grp == 0) z[idx] = 0;
    return;
  }
  const int64_t stride = dh + 2;
  const float* pp = part + (int64_t)bh * nsplit * stride;
  {
    // the splits that hold keys of the query at position p (the first
    // nsplit of the launch when the position is known on the host)
    const int64_t p = p0_dev ? *p0_dev : p0;
    const int64_t lo = window > 0 ? max((int64_t)0, p - window + 1) : 0;
    const int64_t ns = (p + 1 - lo / 64 * 64 + sk - 1) / sk;
    nsplit = (int)min((int64_t)nsplit, max((int64_t)1, ns));
  }
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int s0 = grp; s0 < nsplit; s0 += 8 * G) {
    float mm[8], ll[8], oo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sp = s0 + j * G;
      const bool ok = sp < nsplit;
      mm[j] = ok ? pp[sp * stride] : -INFINITY;
      ll[j] = ok ? pp[sp * stride + 1] : 0.f;
      oo[j] = ok ? pp[sp * stride + 2 + d] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (mm[j] == -INFINITY) continue;  // no split, or a split without keys
      const float mn = fmaxf(M, mm[j]);
      const float fa = exp2f(M - mn), fb = exp2f(mm[j] - mn);
      L = L * fa + ll[j] * fb;
      O = O * fa + oo[j] * fb;
      M = mn;
    }
  }
  if (dl == 0) {
    gm[grp] = M;
    gl[grp] = L;
  }
  go[threadIdx.x] = O;
  __syncthreads();
  if (grp != 0) return;
  float Mx = -INFINITY;
  for (int j = 0; j < G; ++j) Mx = fmaxf(Mx, gm[j]);
  float Lt = 0.f, Ot = 0.f;
  for (int j = 0; j < G; ++j) {
    if (gm[j] == -INFINITY) continue;
    const float w = exp2f(gm[j] - Mx);
    Lt += gl[j] * w;
    Ot += go[j * dc + dl] * w;
  }
  float gv;
  if (qkv_part) {  // sigma(gate) from the projection partials, rounded as stored
    const int64_t N = 2 * (int64_t)n_q * dh + 2 * (int64_t)n_kv * dh;
    const float x = sum_splits(qkv_part + (int64_t)b * N + (int64_t)n_q * dh + 2 * (int64_t)n_kv * dh +
                                   h * dh + d, qkv_nsplit, qkv_ss);
    gv = bf2f(f2bf(1.0f / (1.0f + __expf(-x))));
  } else {
    gv = bf2f(gate[idx]);
  }
  z[idx] = f2bf(Ot / Lt * gv);
}

template <int DH, int GRP>
hipError_t prefill_cfg(const AttnArgs& a, hipStream_t st) {
  constexpr int BQ = (PF_WAVES / GRP) * 32;
  dim3 grid((a.C + BQ - 1) / BQ, a.n_kv, a.B);
  // a step from position 0 (no positions below the fresh buffer's origin)
  // reads step keys only: the DMA addressing without the cache rows
  if (DH == 128 && a.f_origin == 0)
    hipLaunchKernelGGL((attn_prefill_kernel<DH, GRP, DH == 128>), grid, dim3(PF_WAVES * 64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<DH, GRP, false>), grid, dim3(PF_WAVES * 64), 0, st, a);
  return hipGetLastError();
}


int decode_split_keys(int64_t lo, int64_t p, bool window) {
  if (window) return DEC_SWAK;
  return p + 1 - lo / 64 * 64 > DEC_LONG ? DEC_LONGK : DEC_MAXK;
}

// Batches with at least 256 (sequence, KV head) pairs take the direct form:
// every CU holds one of them, without split partials or a combine launch.
constexpr int DEC_DIRECT_MIN = 256;
constexpr int DEC_DIRECT_NT = 512;

template <int DH, int GRP>
hipError_t decode_cfg(const AttnArgs& a, int nsplit, float* part, hipStream_t st) {
  if (a.B * a.n_kv >= DEC_DIRECT_MIN) {
    hipLaunchKernelGGL((attn_decode_kernel<DH, GRP, 0, true, DEC_DIRECT_NT>), dim3(1, a.n_kv, a.B),
                       dim3(DEC_DIRECT_NT), 0, st, a, 1, part);
    return hipGetLastError();
  }
  dim3 grid(nsplit, a.n_kv, a.B);
  const int64_t lo = a.window > 0 ? std::max<int64_t>(0, a.p0 - a.window + 1) : 0;
  const int sk = decode_split_keys(lo, a.p0, a.window > 0);
  if (sk == DEC_LONGK)
    hipLaunchKernelGGL((attn_decode_kernel<DH, GRP, DEC_LONGK>), grid, dim3(DEC_NT), 0, st, a, nsplit, part);
  else if (a.window > 0)
    hipLaunchKernelGGL((attn_decode_kernel<DH, GRP, DEC_SWAK>), grid, dim3(DEC_NT), 0, st, a, nsplit, part);
  else
    hipLaunchKernelGGL((attn_decode_kernel<DH, GRP, DEC_MAXK>), grid, dim3(DEC_NT), 0, st, a, nsplit, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // few splits: one group per head; up to 64: groups of DH threads;
  // more (long contexts): 32-dim chunks of a head per workgroup, 32 groups
  const int dc = nsplit > 64 ? 32 : DH;
  const int nt = nsplit <= 8 ? DH : COMB_NT;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.n_q * (DH / dc)), dim3(nt), 0, st, part,
                     nsplit, a.n_q, DH, dc, a.gate, a.z, a.rl, sk, a.window, a.p0, a.p0_dev, a.qkv_part,
                     a.qkv_nsplit, a.qkv_ss, a.n_kv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t st) {
  const int grp = a.n_q / a.n_kv;
#define DORY_PF(DHV, G) if (a.dh == DHV && grp == G) return prefill_cfg<DHV, G>(a, st);
  DORY_PF(128, 1) DORY_PF(128, 2) DORY_PF(128, 4) DORY_PF(128, 8)
  DORY_PF(64, 1) DORY_PF(64, 2) DORY_PF(64, 4) DORY_PF(64, 8)
  DORY_PF(32, 1) DORY_PF(32, 2) DORY_PF(32, 4) DORY_PF(32, 8)
#undef DORY_PF
  return hipErrorInvalidValue;
}

int64_t decode_attn_part_floats(int B, int n_q, int dh, int nsplit) {
  return (int64_t)B * n_q * nsplit * (dh + 2);
}

int decode_attn_split_keys(int64_t lo, int64_t p, bool window) {
  return decode_split_keys(lo, p, window);
}

int decode_attn_pick_split(int64_t lo, int64_t p, bool window) {
  const int64_t base = lo / 64 * 64;
  const int64_t sk = decode_split_keys(lo, p, window);
  const int64_t s = (p + 1 - base + sk - 1) / sk;
  return (int)(s < 1 ? 1 : s);
}

hipError_t launch_attn_decode(const AttnArgs& a, int nsplit, float* part, hipStream_t st) {
  const int grp = a.n_q / a.n_kv;
#define DORY_DC(DHV, G) if (a.dh == DHV && grp == G) return decode_cfg<DHV, G>(a, nsplit, part, st);
  DORY_DC(128, 1) DORY_DC(128, 2) DORY_DC(128, 4) DORY_DC(128, 8)
  DORY_DC(64, 1) DORY_DC(64, 2) DORY_DC(64, 4) DORY_DC(64, 8)
  DORY_DC(32, 1) DORY_DC(32, 2) DORY_DC(32, 4) DORY_DC(32, 8)
#undef DORY_DC
  return hipErrorInvalidValue;
}

}  // namespace dory
