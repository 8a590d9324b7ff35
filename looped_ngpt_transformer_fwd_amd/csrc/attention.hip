// Gated grouped-query attention for gfx950.
//
// Prefill: flash attention on MFMA. One workgroup = one (batch row, KV head,
// query tile); its 8 waves cover the n_q/n_kv query heads of that KV group
// times 32-query blocks, so every K/V tile staged in LDS is reused by all
// query heads of the group. Scores are computed transposed,
// S^T = K Q^T (v_mfma_f32_32x32x16_bf16 with K as the A operand), so that in
// the accumulator layout each lane owns one query column: the running max and
// sum of the online softmax need a single lane-pair exchange per tile. The
// output is likewise accumulated transposed, O^T += V^T P^T, with P^T taken
// straight from the score registers (converted to bf16) and V^T read from an
// LDS tile stored [head_dim][keys]. Keys come from two sources: the cache
// (positions below f_origin, ring-indexed for sliding-window layers) and the
// fresh K/V of the current step. Tiles wholly outside the causal or
// sliding-window band are skipped. The sigmoid gate is applied in the
// epilogue; the concatenation norm is left to the output projection's
// consumer (it cancels under N(y)).
//
// Decode: one query per sequence; split over keys, VALU dot products with
// 16 lanes per 256-byte key row, partial (max, sum, o) per split, and a
// combine kernel that merges the splits and applies the gate.
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

template <int DH, int GRP>
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
  constexpr int NT = PF_WAVES * 64;

  // Three LDS stages (two tiles in flight), as separate arrays: every LDS
  // read below names its stage statically, so the compiler can tell it
  // apart from the DMA still landing in the other stages and does not drain
  // that DMA before the read.
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
  const int64_t pq = a.p0 + tq;

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
  const int64_t k_end = a.p0 + C;
  int64_t k_lo = 0;
  if (a.window > 0) k_lo = max((int64_t)0, p_lo - a.window + 1);
  const int64_t kt_first = (k_lo / BN) * BN;
  const int ntiles = (int)((p_hi - kt_first) / BN) + 1;

  // per-wave query extent
  const bool wave_live = t0 < C;
  const int64_t wq_lo = a.p0 + t0, wq_hi = a.p0 + min(t0 + 31, C - 1);

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
  // the reads. A lane's row (K) or 8-key column group (V) within a tile is
  // the same in every tile, so its remainder modulo the ring is taken once;
  // per tile only the (uniform) remainder of the tile start is added, with
  // one conditional subtraction. Positions fit 31 bits (checked on the
  // host: at most 2^24); a layer without a ring uses a divisor above every
  // position.
  const uint32_t ring_div = a.ring > 0 ? (uint32_t)a.ring : 0x7FFFFFFFu;
  // the four base pointers as uniform values (a select between two fields of
  // the argument block would become a per-lane load of the selected field)
  const uint16_t* const kcb = uniform_ptr(a.kc + bg * a.c_rows * DH);
  const uint16_t* const kfb = uniform_ptr(a.kf + bg * a.f_rows * DH);
  const uint16_t* const vcb = uniform_ptr(a.vc + bg * DH * a.c_rows);
  const uint16_t* const vfb = uniform_ptr(a.vf + bg * DH * a.f_rows);
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
  auto issue = [&](int64_t kt, uint8_t* kst, uint8_t* vst) __attribute__((always_inline)) {
    const uint32_t km = (uint32_t)kt % ring_div;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int blk = wave + j * PF_WAVES;
      if (K_BLOCKS % PF_WAVES != 0 && blk >= K_BLOCKS) break;
      const int r = blk * KRPB + lane / KCH;
      const int c = (lane % KCH) ^ kswz<DH>(r);
      const int64_t u = kt + r;
      uint32_t ci = km + k_rm[j];
      ci = ci >= ring_div ? ci - ring_div : ci;
      const bool in_cache = u < a.f_origin;
      // per-lane parts in 32 bits (rows * DH stay below 2^31)
      const uint32_t fr = (uint32_t)min(u - a.f_origin, a.f_rows - 1);
      const uint32_t off = (in_cache ? ci : fr) * DH + c * 8;
      dma16_flat((in_cache ? kcb : kfb) + off, kst + blk * 1024);
    }
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      const int blk = wave + j * PF_WAVES;
      if (V_BLOCKS % PF_WAVES != 0 && blk >= V_BLOCKS) break;
      const int d = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((d >> 1) & 7);
      // chunks at or past the last key load the row's first chunk instead:
      // finite values that meet probabilities of exactly 0 (the loads stay
      // unconditional so every wave issues a fixed number per tile)
      const int64_t u = kt + c * 8;
      uint32_t ci = km + v_cm[j];
      ci = ci >= ring_div ? ci - ring_div : ci;
      // every candidate offset is computed, then selected (no branch);
      // per-lane parts in 32 bits (DH * rows stays below 2^31)
      const bool past = u >= k_end, in_cache = u < a.f_origin;
      const bool use_c = past ? a.f_origin > 0 : in_cache;
      const uint32_t col = past ? 0u : in_cache ? ci : (uint32_t)(u - a.f_origin);
      const uint32_t off = (uint32_t)d * (use_c ? (uint32_t)a.c_rows : (uint32_t)a.f_rows) + col;
      dma16_flat((use_c ? vcb : vfb) + off, vst + blk * 1024);
    }
  };
  // DMA instructions issued per tile by this wave
  const int per_tile = (K_BLOCKS > wave ? (K_BLOCKS - wave + PF_WAVES - 1) / PF_WAVES : 0) +
                       (V_BLOCKS > wave ? (V_BLOCKS - wave + PF_WAVES - 1) / PF_WAVES : 0);

  // the query fragments must have landed before the DMA stream starts: the
  // vmcnt waits in the loop count DMA only
  wait_vm0_attn();
  issue(kt_first, ks0, vs0);
  issue(kt_first + (int64_t)min(1, ntiles - 1) * BN, ks1, vs1);

  // Every tile issues the loads of the tile two ahead, clamped to the last
  // tile (a reload into a stage no one reads again), so the wait count is
  // the same in every tile and no branch surrounds the DMA.
  auto tile = [&](int it, const uint8_t* kst, const uint8_t* vst, uint8_t* kn, uint8_t* vn) {
    const int64_t kt = kt_first + (int64_t)it * BN;
    // this wave's loads of tile `it` are done once at most the next tile's
    // loads are outstanding
    if constexpr (K_BLOCKS % PF_WAVES == 0 && V_BLOCKS % PF_WAVES == 0) {
      constexpr int pt = K_BLOCKS / PF_WAVES + V_BLOCKS / PF_WAVES;
      static_assert(pt == 1 || pt == 2 || pt == 4, "wait counts");
      __builtin_amdgcn_s_waitcnt(pt == 4 ? 0x0F74 : pt == 2 ? 0x0F72 : 0x0F71);
    } else {
      if (per_tile == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
      else if (per_tile == 2) __builtin_amdgcn_s_waitcnt(0x0F72);
      else if (per_tile == 1) __builtin_amdgcn_s_waitcnt(0x0F71);
      else wait_vm0_attn();
    }
    barrier_lds();
    issue(kt_first + (int64_t)min(it + 2, ntiles - 1) * BN, kn, vn);

    // tile class for this wave
    const bool dead = !wave_live || kt > wq_hi ||
                      (a.window > 0 && wq_lo - (kt + BN - 1) >= a.window);
    if (dead) return;
    const bool interior = kt + BN - 1 <= wq_lo && (a.window == 0 || wq_hi - kt < a.window);

    floatx16 sacc[BN / 32];
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
    if (!interior) {
      // relative positions fit 32 bits: |pq - u| < C + 64
      const int rel0 = (int)(pq - kt) - hl * 8;  // pq - (key index within tile)
      const bool qok = tq < C;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dist = rel0 - (kb * 32 + (e >> 3) * 16 + (e & 7));  // pq - u
          const bool vis = qok && dist >= 0 && (a.window == 0 || dist < a.window);
          if (!vis) sacc[kb][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescaling: the reference maximum m_run (that of the exponentials
    // accumulated so far) moves only when a score exceeds it by more than 8
    // in base-2 units, so probabilities stay below 2^8 and o and l are
    // rescaled rarely; the final o / l is the same softmax either way. (From
    // m_run = -inf the first visible score always moves it; all-masked
    // queries keep -inf and contribute probabilities of 0.)
    if (__ballot((mx - m_run) * sl2 > 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * sl2);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < DH / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= corr;
    }
    const float nm = -(m_run == -INFINITY ? 0.f : m_run) * sl2;
    bf16x8 pf[BN / 32][2];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], sl2, nm));
        l_run += p;
        pf[kb][e >> 3][e & 7] = static_cast<__bf16>(p);
      }
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

  // stage of tile t is t % 3; the tile two ahead goes into stage (t + 2) % 3
  for (int it = 0;; it += 6) {
    tile(it, ks0, vs0, ks2, vs2);
    if (it + 1 >= ntiles) break;
    tile(it + 1, ks1, vs1, ks0, vs0);
    if (it + 2 >= ntiles) break;
    tile(it + 2, ks2, vs2, ks1, vs1);
    if (it + 3 >= ntiles) break;
    tile(it + 3, ks0, vs0, ks2, vs2);
    if (it + 4 >= ntiles) break;
    tile(it + 4, ks1, vs1, ks0, vs0);
    if (it + 5 >= ntiles) break;
    tile(it + 5, ks2, vs2, ks1, vs1);
    if (it + 6 >= ntiles) break;
  }
  wait_vm0_attn();  // the clamped reloads have landed before the stages are reused

  // ---- epilogue: normalize, gate, store z[b*C + t][head*DH + d]. The O^T
  // registers hold one query per lane, so the 32 x DH tile of a wave is
  // transposed through LDS (the stage buffers, free after the loop) and
  // written as contiguous 16-byte pieces of each query row. Waves 0-5 use
  // one stage buffer each, then waves 6-7.
  l_run += __shfl_xor(l_run, 32, 64);
  const float il = l_run > 0.f ? 1.0f / l_run : 0.f;
  constexpr int EP_ROW = DH * 2 + 16;   // padded LDS row (16-byte aligned)
  constexpr int CPR = DH / 8;           // 16-byte chunks per query row
  static_assert(32 * EP_ROW <= KT_BYTES && 32 * EP_ROW <= VT_BYTES, "epilogue staging");
  const int dq = a.n_q * DH;
  __syncthreads();
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const bool active = round == 0 ? wave < 6 : wave >= 6;
    const int slot = wave % 6;
    uint8_t* buf = slot == 0 ? ks0 : slot == 1 ? ks1 : slot == 2 ? ks2 : slot == 3 ? vs0 : slot == 4 ? vs1 : vs2;
    if (active) {
      const int q = lane & 31;
#pragma unroll
      for (int db = 0; db < DH / 32; ++db)
#pragma unroll
        for (int eq = 0; eq < 4; ++eq) {
          const int d0 = db * 32 + eq * 8 + hl * 4;
          bf16x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = static_cast<__bf16>(o[db][eq * 4 + j] * il);
          *reinterpret_cast<bf16x4*>(buf + q * EP_ROW + d0 * 2) = v4;
        }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int j = 0; j < 32 * CPR / 64; ++j) {
        const int c = lane + 64 * j;
        const int q = c / CPR, cc = c % CPR;
        const int t = t0 + q;
        if (t < C) {
          const uint4 ov = *reinterpret_cast<const uint4*>(buf + q * EP_ROW + cc * 16);
          const int64_t off = ((int64_t)b * C + t) * dq + head * DH + cc * 8;
          const uint4 gv = *reinterpret_cast<const uint4*>(a.gate + off);
          const uint16_t* oe = reinterpret_cast<const uint16_t*>(&ov);
          const uint16_t* ge = reinterpret_cast<const uint16_t*>(&gv);
          uint4 zv;
          uint16_t* ze = reinterpret_cast<uint16_t*>(&zv);
#pragma unroll
          for (int k = 0; k < 8; ++k) ze[k] = f2bf(bf2f(oe[k]) * bf2f(ge[k]));
          *reinterpret_cast<uint4*>(a.z + off) = zv;
        }
      }
    }
    __syncthreads();
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
template <int DH, int GRP, int SPLITK>
__global__ void __launch_bounds__(DEC_NT)
attn_decode_kernel(AttnArgs a, int nsplit, float* part) {
  constexpr int DEC_WKEYS = SPLITK / (DEC_NT / 64);  // keys per wave
  constexpr int NS = DH / 32;   // 32-dim slices of the q.k contraction
  constexpr int NB = DH / 16;   // 16-dim blocks of the output
  static_assert(GRP <= 16, "query heads per KV head must fit the 16-wide MFMA side");
  __shared__ float wmax[DEC_NT / 64][GRP];
  __shared__ float wsum[DEC_NT / 64][GRP];
  __shared__ float wout[DEC_NT / 64][GRP][DH];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (a.rl.k_rows && a.rl.loop >= a.rl.k_rows[b]) return;  // left the loop (merge writes zeros)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 4, r = lane & 15;
  const int64_t bg = (int64_t)b * a.n_kv + g;
  const int64_t p = a.p0;
  int64_t lo = 0;
  if (a.window > 0) lo = max((int64_t)0, p - a.window + 1);
  const int64_t A = (lo / 64) * 64 + (int64_t)split * SPLITK;
  const int64_t ua = max(lo, A), ub = min(p + 1, A + SPLITK);
  const int64_t w0 = A + (int64_t)wave * DEC_WKEYS;

  bf16x8 qb[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qb[s] = load16_or_zero(a.q + ((int64_t)b * a.n_q + g * GRP + (r < GRP ? r : 0)) * DH + 32 * s + 8 * G,
                           r < GRP);
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

  // loads of block blk into (kf, vf): keys outside [lo, p] read as zeros
  auto load = [&](int blk, bf16x8 (&kf)[2][NS], bf16x8 (&vf)[NB]) {
    const int64_t u0 = w0 + 32 * blk;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t u = u0 + 8 * (r >> 2) + 4 * t + (r & 3);
      const int64_t row = a.ring > 0 ? u % a.ring : u;
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
    const uint32_t voff = vany ? (uint32_t)((a.ring > 0 ? uv % a.ring : uv) * 2 + r * a.c_rows * 2) : OOB;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, (int)(16 * nb * a.c_rows * 2), 0);
      vf[nb] = __builtin_bit_cast(bf16x8, v);
    }
  };
  auto compute = [&](int blk, const bf16x8 (&kf)[2][NS], bf16x8 (&vf)[NB]) {
    const int64_t u0 = w0 + 32 * blk;
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

  // two register sets: the loads of block blk + 1 are in flight while block
  // blk computes
  constexpr int NBLK = DEC_WKEYS / 32;
  static_assert(NBLK % 2 == 0, "blocks per wave come in pairs");
  bf16x8 kfa[2][NS], vfa[NB], kfb[2][NS], vfb[NB];
  load(0, kfa, vfa);
  load(1, kfb, vfb);
#pragma unroll
  for (int blk = 0; blk < NBLK; blk += 2) {
    compute(blk, kfa, vfa);
    if (blk + 2 < NBLK) load(blk + 2, kfa, vfa);
    compute(blk + 1, kfb, vfb);
    if (blk + 3 < NBLK) load(blk + 3, kfb, vfb);
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
  for (int i = tid; i < GRP * DH; i += DEC_NT) {
    const int h = i / DH, d = i % DH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_NT / 64; ++w) M = fmaxf(M, wmax[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < DEC_NT / 64; ++w) {
        const float f = __builtin_amdgcn_exp2f(wmax[w][h] - M);
        L += wsum[w][h] * f;
        O += wout[w][h][d] * f;
      }
    }
    float* dst = part + (((int64_t)b * a.n_q + g * GRP + h) * nsplit + split) * (DH + 2);
    dst[2 + d] = O;
    if (d == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// grid B * n_q, block DH. The split maxima go through LDS once; the weighted
// sums keep eight splits' loads in flight per thread.
__global__ void __launch_bounds__(128)
attn_decode_combine_kernel(const float* part, int nsplit, int n_q, int dh, const uint16_t* gate,
                           uint16_t* z, RowLoops rl) {
  __shared__ float wsc[2048];  // 2^(m_s - M) per split (nsplit <= 2048)
  __shared__ float pm[128];    // per-thread partial maxima (blockDim = dh <= 128)
  const int bh = blockIdx.x, d = threadIdx.x;
  const int b = bh / n_q, h = bh % n_q;
  if (rl.k_rows && rl.loop >= rl.k_rows[b]) {  // left the loop: no partials were written
    z[(int64_t)b * n_q * dh + h * dh + d] = 0;
    return;
  }
  const int64_t stride = dh + 2;
  const float* pp = part + (int64_t)bh * nsplit * stride;
  float M = -INFINITY;
  for (int s = d; s < nsplit; s += blockDim.x) M = fmaxf(M, pp[s * stride]);
  pm[d] = M;
  __syncthreads();
  M = -INFINITY;
  for (int t = 0; t < (int)blockDim.x; ++t) M = fmaxf(M, pm[t]);
  float L = 0.f;
  for (int s = d; s < nsplit; s += blockDim.x) {
    const float m = pp[s * stride];
    const float w = m == -INFINITY ? 0.f : exp2f(m - M);
    wsc[s] = w;
  }
  __syncthreads();
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    float o[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      o[j] = pp[(s + j) * stride + 2 + d];
      l[j] = pp[(s + j) * stride + 1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc += o[j] * wsc[s + j];
      L += l[j] * wsc[s + j];
    }
  }
  for (; s < nsplit; ++s) {
    acc += pp[s * stride + 2 + d] * wsc[s];
    L += pp[s * stride + 1] * wsc[s];
  }
  const int64_t idx = (int64_t)b * n_q * dh + h * dh + d;
  z[idx] = f2bf(acc / L * bf2f(gate[idx]));
}

template <int DH, int GRP>
hipError_t prefill_cfg(const AttnArgs& a, hipStream_t st) {
  constexpr int BQ = (PF_WAVES / GRP) * 32;
  dim3 grid((a.C + BQ - 1) / BQ, a.n_kv, a.B);
  hipLaunchKernelGGL((attn_prefill_kernel<DH, GRP>), grid, dim3(PF_WAVES * 64), 0, st, a);
  return hipGetLastError();
}

int decode_split_keys(int64_t lo, int64_t p, bool window) {
  if (window) return DEC_SWAK;
  return p + 1 - lo / 64 * 64 > DEC_LONG ? DEC_LONGK : DEC_MAXK;
}

template <int DH, int GRP>
hipError_t decode_cfg(const AttnArgs& a, int nsplit, float* part, hipStream_t st) {
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
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.n_q), dim3(DH), 0, st, part, nsplit,
                     a.n_q, DH, a.gate, a.z, a.rl);
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
