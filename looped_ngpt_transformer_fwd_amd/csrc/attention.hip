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

template <int DH, int GRP>
__global__ void __launch_bounds__(PF_WAVES * 64)
attn_prefill_kernel(AttnArgs a) {
  constexpr int QB = PF_WAVES / GRP;   // 32-query blocks per workgroup
  constexpr int BQ = QB * 32;          // queries per workgroup
  constexpr int BN = PF_BN;
  constexpr int KROW = DH * 2 + 16;    // padded LDS bytes per key row
  constexpr int VROW = BN * 2 + 8;     // padded LDS bytes per V^T row
  constexpr int NT = PF_WAVES * 64;
  constexpr int K_CHUNKS = BN * DH / 8;
  constexpr int V_CHUNKS = DH * BN / 8;
  static_assert(K_CHUNKS % NT == 0 || K_CHUNKS < NT, "");

  __shared__ __attribute__((aligned(16))) uint8_t ks[BN * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t vs[DH * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int qb = wave / GRP, head = g * GRP + (wave % GRP);
  const int C = a.C;
  const int t0 = qt * BQ + qb * 32;
  const int tq = t0 + (lane & 31);           // this lane's query row
  const int64_t pq = a.p0 + tq;              // its position
  const int hl = lane >> 5;                  // lane half
  const int64_t bg = (int64_t)b * a.n_kv + g;

  // query fragments (B operand of S^T): column = query, k = head dims
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

  // key range of the workgroup
  const int tw0 = qt * BQ;
  const int tw1 = min(C, tw0 + BQ) - 1;
  const int64_t p_lo = a.p0 + tw0, p_hi = a.p0 + tw1;
  const int64_t k_end = a.p0 + C;            // keys [0, k_end) exist
  int64_t k_lo = 0;
  if (a.window > 0) k_lo = max((int64_t)0, p_lo - a.window + 1);
  const int64_t kt_first = (k_lo / BN) * BN;

  for (int64_t kt = kt_first; kt <= p_hi; kt += BN) {
    // ---- stage K tile [BN][DH]
    for (int c = tid; c < K_CHUNKS; c += NT) {
      const int r = c / (DH / 8), cc = c % (DH / 8);
      const int64_t u = kt + r;
      const uint16_t* src;
      if (u < a.f_origin) {
        const int64_t row = a.ring > 0 ? u % a.ring : u;
        src = a.kc + (bg * a.c_rows + row) * DH;
      } else {
        const int64_t row = min(u - a.f_origin, a.f_rows - 1);
        src = a.kf + (bg * a.f_rows + row) * DH;
      }
      *reinterpret_cast<uint4*>(ks + r * KROW + cc * 16) =
          *reinterpret_cast<const uint4*>(src + cc * 8);
    }
    // ---- stage V^T tile [DH][BN]; keys at or beyond k_end read as zero
    for (int c = tid; c < V_CHUNKS; c += NT) {
      const int d = c / (BN / 8), cc = c % (BN / 8);
      const int64_t u = kt + cc * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (u < k_end) {
        const uint16_t* src;
        if (u < a.f_origin) {
          const int64_t col = a.ring > 0 ? u % a.ring : u;
          src = a.vc + (bg * DH + d) * a.c_rows + col;
        } else {
          src = a.vf + (bg * DH + d) * a.f_rows + (u - a.f_origin);
        }
        v = *reinterpret_cast<const uint4*>(src);
        if (u + 8 > k_end) {
          const int keep = (int)(k_end - u);
          uint16_t* e = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j >= keep) e[j] = 0;
        }
      }
      uint2* dst = reinterpret_cast<uint2*>(vs + d * VROW + cc * 16);
      dst[0] = make_uint2(v.x, v.y);
      dst[1] = make_uint2(v.z, v.w);
    }
    __syncthreads();

    // ---- S^T = K Q^T for BN/32 key blocks
    floatx16 sacc[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            ks + (kb * 32 + (lane & 31)) * KROW + (s * 2 + hl) * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
      }
    }
    // ---- mask, scale (log2 domain), online softmax
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t u = kt + kb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
        const bool vis = tq < C && key_visible(pq, u, a.window);
        const float sv = vis ? sacc[kb][e] * sl2 : -INFINITY;
        sacc[kb][e] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float corr = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] *= corr;
    bf16x8 pf[BN / 32][2];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(sacc[kb][e] - m_use);
        l_run += p;
        pf[kb][e >> 3][e & 7] = static_cast<__bf16>(p);
      }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) {
      const uint8_t* vrow = vs + (db * 32 + (lane & 31)) * VROW;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int k0 = kb * 32 + kc * 16 + hl * 4;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + k0 * 2);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + (k0 + 8) * 2);
          bf16x8 vf;
#pragma unroll
          for (int j = 0; j < 4; ++j) { vf[j] = lo[j]; vf[j + 4] = hi[j]; }
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][kc], o[db], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // ---- epilogue: normalize, gate, store z[b*C + t][head*DH + d]
  l_run += __shfl_xor(l_run, 32, 64);
  if (tq < C) {
    const float il = 1.0f / l_run;
    const int dq = a.n_q * DH;
    const int64_t zrow = ((int64_t)b * C + tq) * dq + head * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = db * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
        const float gv = bf2f(a.gate[zrow + d]);
        a.z[zrow + d] = f2bf(o[db][e] * il * gv);
      }
  }
}

// ------------------------------------------------------------------ decode
constexpr int DEC_NT = 256;
constexpr int DEC_MAXK = 512;  // keys per split

template <int DH, int GRP>
__global__ void __launch_bounds__(DEC_NT)
attn_decode_kernel(AttnArgs a, int nsplit, float* part) {
  __shared__ float qs[GRP][DH];
  __shared__ float sc[GRP][DEC_MAXK];
  __shared__ float red[GRP][DEC_NT / 64];
  constexpr int HALVES = DEC_NT / DH;   // threads per head dim in the V pass
  __shared__ float ostage[HALVES][GRP][DH];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bg = (int64_t)b * a.n_kv + g;
  const int64_t p = a.p0;  // query position; cache rows hold keys 0..p
  int64_t lo = 0;
  if (a.window > 0) lo = max((int64_t)0, p - a.window + 1);
  const int64_t nkeys = p - lo + 1;
  const int64_t per = (nkeys + nsplit - 1) / nsplit;
  const int64_t ka = lo + split * per;
  const int64_t kb_ = min(p + 1, ka + per);
  const int nk = (int)max((int64_t)0, kb_ - ka);

  for (int i = tid; i < GRP * DH; i += DEC_NT) {
    const int h = i / DH, d = i % DH;
    qs[h][d] = bf2f(a.q[((int64_t)b * a.n_q + g * GRP + h) * DH + d]);
  }
  __syncthreads();

  // ---- scores: 16 lanes per key row (8 dims each), 4 keys per wave pass
  constexpr int LPK = DH / 8;            // lanes per key
  constexpr int KPW = 64 / LPK;          // keys per wave pass
  const int sub = lane % LPK, kl = lane / LPK;
  float qreg[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) qreg[h][j] = qs[h][sub * 8 + j];
  for (int k0 = wave * KPW; k0 < nk; k0 += (DEC_NT / 64) * KPW) {
    const int kk = k0 + kl;
    float acc[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) acc[h] = 0.f;
    if (kk < nk) {
      const int64_t u = ka + kk;
      const int64_t row = a.ring > 0 ? u % a.ring : u;
      const uint4 raw = *reinterpret_cast<const uint4*>(a.kc + (bg * a.c_rows + row) * DH + sub * 8);
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kv = bf2f(e[j]);
#pragma unroll
        for (int h = 0; h < GRP; ++h) acc[h] += qreg[h][j] * kv;
      }
    }
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1) acc[h] += __shfl_xor(acc[h], o, 64);
    }
    if (sub == 0 && kk < nk) {
#pragma unroll
      for (int h = 0; h < GRP; ++h) sc[h][kk] = acc[h] * a.scale * kLog2e;
    }
  }
  __syncthreads();

  // ---- softmax pieces per head
  float mh[GRP], lh[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    float m = -INFINITY;
    for (int i = tid; i < nk; i += DEC_NT) m = fmaxf(m, sc[h][i]);
    m = wave_max(m);
    if (lane == 0) red[h][wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    float m = red[h][0];
    for (int w = 1; w < DEC_NT / 64; ++w) m = fmaxf(m, red[h][w]);
    mh[h] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const float mu = mh[h] == -INFINITY ? 0.f : mh[h];
    float l = 0.f;
    for (int i = tid; i < nk; i += DEC_NT) {
      const float e = exp2f(sc[h][i] - mu);
      sc[h][i] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) red[h][wave] = l;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    float l = 0.f;
    for (int w = 0; w < DEC_NT / 64; ++w) l += red[h][w];
    lh[h] = l;
  }

  // ---- o[h][d] = sum_u p[h][u] V^T[d][u]; thread = (d, key slice)
  {
    const int d = tid % DH;
    const int half = tid / DH;
    float acc[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) acc[h] = 0.f;
    const uint16_t* vrow = a.vc + (bg * DH + d) * a.c_rows;
    for (int kk = half; kk < nk; kk += HALVES) {
      const int64_t u = ka + kk;
      const int64_t col = a.ring > 0 ? u % a.ring : u;
      const float v = bf2f(vrow[col]);
#pragma unroll
      for (int h = 0; h < GRP; ++h) acc[h] += sc[h][kk] * v;
    }
#pragma unroll
    for (int h = 0; h < GRP; ++h) ostage[half][h][d] = acc[h];
  }
  __syncthreads();
  for (int i = tid; i < GRP * DH; i += DEC_NT) {
    const int h = i / DH, d = i % DH;
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < HALVES; ++j) v += ostage[j][h][d];
    float* dst = part + (((int64_t)b * a.n_q + g * GRP + h) * nsplit + split) * (DH + 2);
    dst[2 + d] = v;
    if (d == 0) {
      dst[0] = mh[h];
      dst[1] = lh[h];
    }
  }
}

// grid B * n_q, block DH
__global__ void attn_decode_combine_kernel(const float* part, int nsplit, int n_q, int dh,
                                           const uint16_t* gate, uint16_t* z) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const int b = bh / n_q, h = bh % n_q;
  const float* pp = part + (int64_t)bh * nsplit * (dh + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pp[s * (dh + 2)]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float m = pp[s * (dh + 2)];
    if (m == -INFINITY) continue;
    const float w = exp2f(m - M);
    L += pp[s * (dh + 2) + 1] * w;
    acc += pp[s * (dh + 2) + 2 + d] * w;
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

template <int DH, int GRP>
hipError_t decode_cfg(const AttnArgs& a, int nsplit, float* part, hipStream_t st) {
  dim3 grid(nsplit, a.n_kv, a.B);
  hipLaunchKernelGGL((attn_decode_kernel<DH, GRP>), grid, dim3(DEC_NT), 0, st, a, nsplit, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.n_q), dim3(DH), 0, st, part, nsplit,
                     a.n_q, DH, a.gate, a.z);
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

int decode_attn_pick_split(int B, int n_kv, int64_t keys) {
  int64_t s = (keys + DEC_MAXK - 1) / DEC_MAXK;
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
