// Bandwidth-bound row kernels of the forward pass: embedding gather, the
// fused nGPT normalize-and-update (optionally with the loop-boundary
// re-injection fused in), the query/key transform (RoPE, per-head L2 norm,
// s_qk) with the K/V placement, KV-cache copies, SwiGLU over split partials,
// greedy argmax, and the probe kernels of the debug dumps (fills, K/V
// placement, one-hot mask probes, slot rows).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

constexpr int NT_ROW = 256;
constexpr int MAXV = 4;  // float4 per thread: d <= 4 * 4 * 256 = 4096

__global__ void __launch_bounds__(NT_ROW)
embed_kernel(const int32_t* tok, const uint16_t* E, int vocab, int d, float* h32,
             uint16_t* h16, float* x32) {
  const int m = blockIdx.x;
  const int id = tok[m];
  const bool ok = id >= 0 && id < vocab;
  const uint16_t* src = E + (int64_t)(ok ? id : 0) * d;
  const float nanv = __uint_as_float(0x7fc00000u);
  for (int i = threadIdx.x; i < d; i += NT_ROW) {
    const uint16_t v = src[i];
    const float f = ok ? bf2f(v) : nanv;
    h32[(int64_t)m * d + i] = f;
    h16[(int64_t)m * d + i] = ok ? v : (uint16_t)0x7fc0;
    if (x32) x32[(int64_t)m * d + i] = f;
  }
}

// h <- N(h + alpha (N(y) - h)); optional aux copy of the result, optional
// boundary h <- N(result + x). Y16: y is one bf16 matrix (the large-M
// projections' output), else nsplit fp32 split-K partials. One workgroup
// per row, NT threads, each holding d / (4 NT) float4 columns; every load
// of the row (h, alpha, x, the partials) is issued up front.
template <bool Y16, int NT>
__global__ void __launch_bounds__(NT)
update_kernel(float* h32, uint16_t* h16, const float* y, int nsplit, int64_t ss, int64_t ldy,
              const float* alpha, int d, const float* x, float* aux, RowLoops rl) {
  constexpr int MV = 4 * MAXV * NT_ROW / (4 * NT);  // float4 per thread for d <= 4096
  __shared__ float red[NT / 64];
  const int m = blockIdx.x;
  if (rl.k_rows) {
    const int kb = rl.k_rows[m / rl.T];
    if (rl.loop >= kb) return;           // the sequence has left the loop: keep its state
    if (rl.loop == kb - 1) x = nullptr;  // its last loop: no boundary into another one
  }
  const int nv = d >> 2;
  float4 hv[MV], yv[MV], av[MV], xv[MV];
  float syy = 0.f;
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      hv[i] = reinterpret_cast<const float4*>(h32 + (int64_t)m * d)[c];
      av[i] = reinterpret_cast<const float4*>(alpha)[c];
      if (x) xv[i] = reinterpret_cast<const float4*>(x + (int64_t)m * d)[c];
      if (Y16) {
        const ushort4 t = reinterpret_cast<const ushort4*>(reinterpret_cast<const uint16_t*>(y) +
                                                           (int64_t)m * ldy)[c];
        yv[i] = make_float4(bf2f(t.x), bf2f(t.y), bf2f(t.z), bf2f(t.w));
      } else {
        yv[i] = sum_splits4(y + (int64_t)m * ldy + 4 * c, nsplit, ss);
      }
      syy += yv[i].x * yv[i].x + yv[i].y * yv[i].y + yv[i].z * yv[i].z + yv[i].w * yv[i].w;
    }
  }
  const float iy = 1.0f / sqrtf(block_sum<NT>(syy, red));
  float stt = 0.f;
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      const float4 a = av[i];
      float4 t;
      t.x = hv[i].x + a.x * (yv[i].x * iy - hv[i].x);
      t.y = hv[i].y + a.y * (yv[i].y * iy - hv[i].y);
      t.z = hv[i].z + a.z * (yv[i].z * iy - hv[i].z);
      t.w = hv[i].w + a.w * (yv[i].w * iy - hv[i].w);
      hv[i] = t;
      stt += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
    }
  }
  float it = 1.0f / sqrtf(block_sum<NT>(stt, red));
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      hv[i].x *= it; hv[i].y *= it; hv[i].z *= it; hv[i].w *= it;
      if (aux) reinterpret_cast<float4*>(aux + (int64_t)m * d)[c] = hv[i];
    }
  }
  if (x) {
    float suu = 0.f;
#pragma unroll
    for (int i = 0; i < MV; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < nv) {
        hv[i].x += xv[i].x; hv[i].y += xv[i].y; hv[i].z += xv[i].z; hv[i].w += xv[i].w;
        suu += hv[i].x * hv[i].x + hv[i].y * hv[i].y + hv[i].z * hv[i].z + hv[i].w * hv[i].w;
      }
    }
    it = 1.0f / sqrtf(block_sum<NT>(suu, red));
#pragma unroll
    for (int i = 0; i < MV; ++i) {
      hv[i].x *= it; hv[i].y *= it; hv[i].z *= it; hv[i].w *= it;
    }
  }
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      reinterpret_cast<float4*>(h32 + (int64_t)m * d)[c] = hv[i];
      if (h16) {  // no bf16 shadow in the fp32 build
        ushort4 o;
        o.x = f2bf(hv[i].x); o.y = f2bf(hv[i].y); o.z = f2bf(hv[i].z); o.w = f2bf(hv[i].w);
        reinterpret_cast<ushort4*>(h16 + (int64_t)m * d)[c] = o;
      }
    }
  }
}

__global__ void __launch_bounds__(NT_ROW)
boundary_kernel(float* h32, uint16_t* h16, const float* x, int d) {
  __shared__ float red[NT_ROW / 64];
  const int m = blockIdx.x;
  const int nv = d >> 2;
  float4 v[MAXV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + i * NT_ROW;
    if (c < nv) {
      const float4 a = reinterpret_cast<const float4*>(h32 + (int64_t)m * d)[c];
      const float4 b = reinterpret_cast<const float4*>(x + (int64_t)m * d)[c];
      v[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
      s += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  }
  const float it = 1.0f / sqrtf(block_sum<NT_ROW>(s, red));
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + i * NT_ROW;
    if (c < nv) {
      float4 r = make_float4(v[i].x * it, v[i].y * it, v[i].z * it, v[i].w * it);
      reinterpret_cast<float4*>(h32 + (int64_t)m * d)[c] = r;
      if (h16) {  // no bf16 shadow in the fp32 build
        ushort4 o;
        o.x = f2bf(r.x); o.y = f2bf(r.y); o.z = f2bf(r.z); o.w = f2bf(r.w);
        reinterpret_cast<ushort4*>(h16 + (int64_t)m * d)[c] = o;
      }
    }
  }
}

__global__ void copy_rows_kernel(const float* src, int64_t lds, float* dst, int d) {
  const int m = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[(int64_t)m * d + i] = src[(int64_t)m * lds + i];
}

__global__ void swiglu_partials_kernel(const float* p, int nsplit, int64_t ss, int M, int F,
                                       const float* s_u, const float* s_v, uint16_t* a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * F) return;
  const int64_t m = idx / F;
  const int f = (int)(idx - m * F);
  float up = sum_splits(p + m * 2 * F + f, nsplit, ss);
  float gt = sum_splits(p + m * 2 * F + F + f, nsplit, ss);
  up *= s_u[f];
  gt *= s_v[f];
  a[idx] = f2bf(gt / (1.f + __expf(-gt)) * up);
}

// Grid (token rows, head groups + v/gate groups). Blocks y < n_groups rotate,
// normalize and scale `heads_per_block` q/k heads (dh/2 threads per head, dh
// in {32, 64, 128}); the remaining blocks write v (as V^T) and sigma(gate),
// NT_ROW columns each. cos/sin of the row's angles come from the step's RoPE
// table ([C][dh/2]).
__global__ void __launch_bounds__(NT_ROW)
qk_prep_kernel(const float* P, int nsplit, int64_t ss, int C, int64_t p0, int nq, int nkv,
               int dh, const float* cs_tab, const float* sn_tab, const float* s_qk, uint16_t* qh,
               QkDest kv, uint16_t* gate, RowLoops rl, const int64_t* p0_dev) {
  if (p0_dev) p0 = *p0_dev;
  const int m = blockIdx.x;
  const int b = m / C, t = m - b * C;
  const int64_t pos = p0 + t;
  const int half = dh >> 1;
  const int dq = nq * dh, dkv = nkv * dh;
  const int N = 2 * dq + 2 * dkv;
  const float* row = P + (int64_t)m * N;
  const int64_t krow = cache_row(pos - kv.pos_origin, kv.ring);
  const int per_block = NT_ROW / half;
  const int ngroups = (nq + nkv + per_block - 1) / per_block;
  if ((int)blockIdx.y < ngroups) {
    const int i = threadIdx.x % half;
    const int hh = blockIdx.y * per_block + threadIdx.x / half;
    if (hh >= nq + nkv) return;  // whole head groups exit together
    const float c = cs_tab[(int64_t)t * half + i], sn = sn_tab[(int64_t)t * half + i];
    const int col = hh < nq ? hh * dh : dq + (hh - nq) * dh;
    const float x1 = sum_splits(row + col + i, nsplit, ss);
    const float x2 = sum_splits(row + col + i + half, nsplit, ss);
    const float r1 = x1 * c - x2 * sn;
    const float r2 = x2 * c + x1 * sn;
    float sq = r1 * r1 + r2 * r2;
    for (int o = half >> 1; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    const float inv = 1.0f / sqrtf(sq);
    uint16_t* dst;
    if (hh < nq) {
      dst = qh + (((int64_t)b * nq + hh) * C + t) * dh;
    } else {
      if (rl.k_rows && rl.loop >= rl.k_rows[b]) return;  // left the loop: no K/V store
      dst = kv.kbase + (((int64_t)b * nkv + (hh - nq)) * kv.k_rows + krow) * dh;
    }
    dst[i] = f2bf(s_qk[i] * r1 * inv);
    dst[i + half] = f2bf(s_qk[i + half] * r2 * inv);
    return;
  }
  // v and gate columns: NT_ROW consecutive columns per block
  const int idx = ((int)blockIdx.y - ngroups) * NT_ROW + threadIdx.x;
  if (idx >= dkv + dq) return;
  const float v = sum_splits(row + dq + dkv + idx, nsplit, ss);
  if (idx < dkv) {
    if (rl.k_rows && rl.loop >= rl.k_rows[b]) return;  // left the loop: no K/V store
    const int g = idx / dh, d = idx - g * dh;
    kv.vbase[(((int64_t)b * nkv + g) * dh + d) * kv.v_cols + krow] = f2bf(v);
  } else {
    gate[(int64_t)m * dq + (idx - dkv)] = f2bf(1.0f / (1.0f + __expf(-v)));
  }
}

// grid (npos, n_kv, B), block dh
__global__ void prefix_copy_kernel(const uint16_t* kc, const uint16_t* vc, int64_t c_rows,
                                   int64_t ring, int nkv, int dh, int64_t pos_a, uint16_t* kf,
                                   uint16_t* vf, int64_t f_rows) {
  const int64_t pos = pos_a + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int64_t bg = (int64_t)b * nkv + g;
  const int64_t crow = cache_row(pos, ring);
  const int64_t frow = blockIdx.x;
  kf[(bg * f_rows + frow) * dh + d] = kc[(bg * c_rows + crow) * dh + d];
  vf[(bg * dh + d) * f_rows + frow] = vc[(bg * dh + d) * c_rows + crow];
}

__global__ void kv_write_kernel(const uint16_t* kf, const uint16_t* vf, int64_t f_rows,
                                int64_t f_origin, int nkv, int dh, int64_t pos_a, uint16_t* kc,
                                uint16_t* vc, int64_t c_rows, int64_t ring, RowLoops rl) {
  const int64_t pos = pos_a + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  if (rl.k_rows && rl.k_rows[b] != rl.loop + 1) return;  // not this sequence's last loop
  const int64_t bg = (int64_t)b * nkv + g;
  const int64_t crow = cache_row(pos, ring);
  const int64_t frow = pos - f_origin;
  kc[(bg * c_rows + crow) * dh + d] = kf[(bg * f_rows + frow) * dh + d];
  vc[(bg * dh + d) * c_rows + crow] = vf[(bg * dh + d) * f_rows + frow];
}

// The same copy in 64-position tiles (blockIdx.x counted from pos_a rounded
// down to a multiple of 8; blockIdx.y = group, blockIdx.z = sequence): K rows
// move as 16-byte pieces, V^T columns as 16-byte groups of 8 aligned
// positions, which occupy 8 consecutive columns on both sides (f_origin,
// f_rows, c_rows and the ring are multiples of 8). The one-position form
// above writes a V^T element per thread into a different row each, i.e. 2
// bytes per cache line per store.
__global__ void kv_write_tiled_kernel(const uint16_t* kf, const uint16_t* vf, int64_t f_rows,
                                      int64_t f_origin, int nkv, int dh, int64_t pos_a,
                                      int64_t pos_b, uint16_t* kc, uint16_t* vc, int64_t c_rows,
                                      int64_t ring, RowLoops rl) {
  const int g = blockIdx.y, b = blockIdx.z;
  if (rl.k_rows && rl.k_rows[b] != rl.loop + 1) return;  // not this sequence's last loop
  const int64_t bg = (int64_t)b * nkv + g;
  const int64_t base = (pos_a & ~(int64_t)7) + (int64_t)blockIdx.x * 64;
  const int cpr = dh / 8;  // 16-byte pieces per K row
  for (int i = threadIdx.x; i < 64 * cpr; i += blockDim.x) {
    const int64_t pos = base + i / cpr;
    if (pos < pos_a || pos >= pos_b) continue;
    const int c = i % cpr;
    *reinterpret_cast<uint4*>(kc + (bg * c_rows + cache_row(pos, ring)) * dh + c * 8) =
        *reinterpret_cast<const uint4*>(kf + (bg * f_rows + pos - f_origin) * dh + c * 8);
  }
  for (int i = threadIdx.x; i < 8 * dh; i += blockDim.x) {
    const int d = i >> 3;
    const int64_t p0 = base + (i & 7) * 8;
    const uint16_t* srow = vf + (bg * dh + d) * f_rows;  // column pos - f_origin (pos >= f_origin)
    uint16_t* drow = vc + (bg * dh + d) * c_rows;
    if (p0 >= pos_a && p0 + 8 <= pos_b) {
      *reinterpret_cast<uint4*>(drow + cache_row(p0, ring)) =
          *reinterpret_cast<const uint4*>(srow + (p0 - f_origin));
    } else {
      for (int e = 0; e < 8; ++e) {
        const int64_t pos = p0 + e;
        if (pos < pos_a || pos >= pos_b) continue;
        drow[cache_row(pos, ring)] = srow[pos - f_origin];
      }
    }
  }
}

// Cache-to-cache copy of positions [pos_a, pos_b) of one sequence's K rows
// and V^T columns. blockIdx.x = 64-position tile counted from pos_a rounded
// down to a multiple of 8, blockIdx.y = group. Rows and rings are multiples
// of 8, so an aligned group of 8 positions occupies 8 consecutive, 16-byte
// aligned V^T columns on both sides and moves as one 16-byte vector; K rows
// move in 16-byte pieces (dh a multiple of 8). Positions outside the range
// are never written: in a ring they share rows with positions inside it.
__global__ void kv_copy_kernel(const uint16_t* sk, const uint16_t* sv, int64_t s_rows,
                               int64_t s_ring, int64_t s_bg, uint16_t* dk, uint16_t* dv,
                               int64_t d_rows, int64_t d_ring, int64_t d_bg, int dh,
                               int64_t pos_a, int64_t pos_b) {
  const int64_t base = (pos_a & ~(int64_t)7) + (int64_t)blockIdx.x * 64;
  const int64_t sbg = s_bg + blockIdx.y, dbg = d_bg + blockIdx.y;
  const int cpr = dh / 8;  // 16-byte pieces per K row
  for (int i = threadIdx.x; i < 64 * cpr; i += blockDim.x) {
    const int64_t pos = base + i / cpr;
    if (pos < pos_a || pos >= pos_b) continue;
    const int c = i % cpr;
    const int64_t sr = cache_row(pos, s_ring);
    const int64_t dr = cache_row(pos, d_ring);
    *reinterpret_cast<uint4*>(dk + (dbg * d_rows + dr) * dh + c * 8) =
        *reinterpret_cast<const uint4*>(sk + (sbg * s_rows + sr) * dh + c * 8);
  }
  for (int i = threadIdx.x; i < 8 * dh; i += blockDim.x) {
    const int d = i >> 3;
    const int64_t p0 = base + (i & 7) * 8;
    const uint16_t* srow = sv + (sbg * dh + d) * s_rows;
    uint16_t* drow = dv + (dbg * dh + d) * d_rows;
    if (p0 >= pos_a && p0 + 8 <= pos_b) {
      const int64_t sr = cache_row(p0, s_ring);
      const int64_t dr = cache_row(p0, d_ring);
      *reinterpret_cast<uint4*>(drow + dr) = *reinterpret_cast<const uint4*>(srow + sr);
    } else {
      for (int e = 0; e < 8; ++e) {
        const int64_t pos = p0 + e;
        if (pos < pos_a || pos >= pos_b) continue;
        drow[cache_row(pos, d_ring)] = srow[cache_row(pos, s_ring)];
      }
    }
  }
}

__global__ void rope_table_kernel(int64_t p0, int T, int half, int dh, double base, float* cs,
                                  float* sn, const int64_t* p0_dev) {
  if (p0_dev) p0 = *p0_dev;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * half) return;
  const int t = (int)(idx / half), i = (int)(idx % half);
  const double invf = pow(base, -2.0 * (double)i / (double)dh);
  double s, c;
  sincos((double)(p0 + t) * invf, &s, &c);
  cs[idx] = (float)c;
  sn[idx] = (float)s;
}

// Zero V^T columns [c0, c1) of every (b, g, d) row of the fresh buffer.
__global__ void vt_zero_cols_kernel(uint16_t* vf, int64_t f_rows, int nkv, int dh, int64_t c0,
                                    int64_t c1) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int64_t bg = (int64_t)b * nkv + g;
  for (int d = threadIdx.x; d < dh; d += blockDim.x)
    for (int64_t c = c0; c < c1; ++c) vf[(bg * dh + d) * f_rows + c] = 0;
}

constexpr int NT_ARG = 1024;

__global__ void __launch_bounds__(NT_ARG) argmax_kernel(const float* x, int n, int32_t* out) {
  __shared__ float bv[NT_ARG / 64];
  __shared__ int bi[NT_ARG / 64];
  const float* row = x + (int64_t)blockIdx.x * n;
  float best = -INFINITY;
  int idx = n;  // sentinel above every index
  for (int i = threadIdx.x; i < n; i += NT_ARG) {
    const float v = row[i];
    if (v > best) { best = v; idx = i; }  // strided scan: first hit is the lowest index
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ov > best || (ov == best && oi < idx)) { best = ov; idx = oi; }
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { bv[w] = best; bi[w] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int j = 1; j < NT_ARG / 64; ++j)
      if (bv[j] > best || (bv[j] == best && bi[j] < idx)) { best = bv[j]; idx = bi[j]; }
    out[blockIdx.x] = idx < n ? idx : 0;
  }
}

__global__ void fill_u16_kernel(uint16_t* p, int64_t n, uint16_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// K and V of positions p0 .. p0 + T - 1 given as [B][n_kv][T][dh] go to the
// places the query/key transform stores them (K rows and V^T columns of
// QkDest, row cache_row(p0 + t - pos_origin, ring)). grid (T, n_kv, B),
// block dh.
__global__ void kv_place_kernel(const uint16_t* k, const uint16_t* v, int T, int nkv, int dh,
                                int64_t p0, QkDest dst) {
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int64_t bg = (int64_t)b * nkv + g;
  const int64_t row = cache_row(p0 + t - dst.pos_origin, dst.ring);
  const int64_t src = (bg * T + t) * dh + d;
  dst.kbase[(bg * dst.k_rows + row) * dh + d] = k[src];
  dst.vbase[(bg * dh + d) * dst.v_cols + row] = v[src];
}

// Mask probe values: for positions u in [ua, ub), V entries become one-hot,
// 1.0 at head dimension u - first (when that lies in [0, dh)) and 0
// elsewhere. Cached positions (u < p0, and u >= p0 - ring for a ring) are
// written to the V^T column of their cache row; positions p0 .. p0 + T - 1 to
// vnew [B][n_kv][T][dh]. grid (ub - ua, n_kv, B), block dh.
__global__ void mask_probe_v_kernel(uint16_t* vc, int64_t c_rows, int64_t ring, uint16_t* vnew,
                                    int T, int nkv, int dh, int64_t p0, int64_t ua, int64_t first) {
  const int64_t u = ua + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int64_t bg = (int64_t)b * nkv + g;
  const uint16_t val = (u - first == d) ? (uint16_t)0x3F80 : (uint16_t)0;
  if (u < p0) {
    if (ring > 0 && u < p0 - ring) return;  // no longer held by the ring
    vc[(bg * dh + d) * c_rows + cache_row(u, ring)] = val;
  } else if (u < p0 + T) {
    vnew[(bg * T + (u - p0)) * dh + d] = val;
  }
}

// out[((b * nq + h) * T + t) * L + first + d] = z[b * T + t][h * dh + d] (the
// bf16 weight of key first + d) for first + d < L. grid (B * T, nq), block dh.
__global__ void mask_extract_kernel(const uint16_t* z, int T, int nq, int dh, int64_t L,
                                    int64_t first, uint16_t* out) {
  const int bt = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int b = bt / T, t = bt - b * T;
  if (first + d >= L) return;
  out[(((int64_t)b * nq + h) * T + t) * L + first + d] = z[(int64_t)bt * nq * dh + h * dh + d];
}

__global__ void slot_rows_kernel(int64_t pos_a, int64_t n, int64_t ring, int64_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = cache_row(pos_a + i, ring);
}

}  // namespace

hipError_t launch_embed(const int32_t* tok, const uint16_t* E, int vocab, int M, int d,
                        float* h32, uint16_t* h16, float* x32, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(NT_ROW), 0, st, tok, E, vocab, d, h32, h16, x32);
  return hipGetLastError();
}

hipError_t launch_update(float* h32, uint16_t* h16, const float* y, int nsplit,
                         int64_t split_stride, int64_t ldy, const float* alpha, int M, int d,
                         const float* x, float* state_out, float* copy_out, hipStream_t st,
                         RowLoops rl, bool y_bf16) {
  if (d % 4 != 0 || d > 4 * MAXV * NT_ROW) return hipErrorInvalidValue;
  float* aux = state_out ? state_out : copy_out;
  if (state_out && copy_out) return hipErrorInvalidValue;
  if (y_bf16) {
    if (nsplit != 1 || ldy % 4 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((update_kernel<true, NT_ROW>), dim3(M), dim3(NT_ROW), 0, st, h32, h16, y, nsplit,
                       split_stride, ldy, alpha, d, x, aux, rl);
  } else {
    // split partials (short launches: decode, verification, chunks): one
    // float4 column per thread, all partial loads in flight at once
    if (nsplit < 1 || nsplit > 32) return hipErrorInvalidValue;
    hipLaunchKernelGGL((update_kernel<false, 1024>), dim3(M), dim3(1024), 0, st, h32, h16, y, nsplit,
                       split_stride, ldy, alpha, d, x, aux, rl);
  }
  return hipGetLastError();
}

namespace {
__global__ void transpose_i32_kernel(const int32_t* src, int rows, int cols, int32_t* dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * cols) return;
  const int r = i / cols, c = i - r * cols;
  dst[(int64_t)c * rows + r] = src[i];
}
}  // namespace

hipError_t launch_transpose_i32(const int32_t* src, int rows, int cols, int32_t* dst, hipStream_t st) {
  if (rows < 1 || cols < 1) return hipErrorInvalidValue;
  const int n = rows * cols;
  hipLaunchKernelGGL(transpose_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, src, rows, cols, dst);
  return hipGetLastError();
}

hipError_t launch_boundary(float* h32, uint16_t* h16, const float* x, int M, int d,
                           hipStream_t st) {
  if (d % 4 != 0 || d > 4 * MAXV * NT_ROW) return hipErrorInvalidValue;
  hipLaunchKernelGGL(boundary_kernel, dim3(M), dim3(NT_ROW), 0, st, h32, h16, x, d);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const float* src, int64_t ld_src, float* dst, int rows, int d,
                            hipStream_t st) {
  hipLaunchKernelGGL(copy_rows_kernel, dim3(rows), dim3(256), 0, st, src, ld_src, dst, d);
  return hipGetLastError();
}

hipError_t launch_swiglu_partials(const float* p, int nsplit, int64_t split_stride, int M, int F,
                                  const float* s_u, const float* s_v, uint16_t* a, hipStream_t st) {
  const int64_t n = (int64_t)M * F;
  hipLaunchKernelGGL(swiglu_partials_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     p, nsplit, split_stride, M, F, s_u, s_v, a);
  return hipGetLastError();
}

hipError_t launch_qk_prep(const float* P, int nsplit, int64_t split_stride, int B, int C,
                          int64_t p0, int n_q, int n_kv, int dh, const float* cs, const float* sn,
                          const float* s_qk, uint16_t* q_hat, QkDest kv, uint16_t* gate,
                          hipStream_t st, RowLoops rl, const int64_t* p0_dev) {
  if (dh != 32 && dh != 64 && dh != 128) return hipErrorInvalidValue;
  const int per_block = NT_ROW / (dh / 2);
  const int ngroups = (n_q + n_kv + per_block - 1) / per_block;
  const int nvg = (n_kv * dh + n_q * dh + NT_ROW - 1) / NT_ROW;
  hipLaunchKernelGGL(qk_prep_kernel, dim3(B * C, ngroups + nvg), dim3(NT_ROW), 0, st, P, nsplit,
                     split_stride, C, p0, n_q, n_kv, dh, cs, sn, s_qk, q_hat, kv, gate, rl, p0_dev);
  return hipGetLastError();
}

hipError_t launch_prefix_copy(const uint16_t* kc, const uint16_t* vc, int64_t c_rows,
                              int64_t ring, int B, int n_kv, int dh, int64_t pos_a,
                              int64_t pos_b, uint16_t* kf, uint16_t* vf, int64_t f_rows,
                              hipStream_t st) {
  if (pos_b <= pos_a) return hipSuccess;
  hipLaunchKernelGGL(prefix_copy_kernel, dim3((unsigned)(pos_b - pos_a), n_kv, B), dim3(dh), 0, st,
                     kc, vc, c_rows, ring, n_kv, dh, pos_a, kf, vf, f_rows);
  return hipGetLastError();
}

hipError_t launch_kv_write(const uint16_t* kf, const uint16_t* vf, int64_t f_rows,
                           int64_t f_origin, int B, int n_kv, int dh, int64_t pos_a,
                           int64_t pos_b, uint16_t* kc, uint16_t* vc, int64_t c_rows,
                           int64_t ring, hipStream_t st, RowLoops rl) {
  if (pos_b <= pos_a) return hipSuccess;
  const bool aligned = dh % 8 == 0 && f_rows % 8 == 0 && f_origin % 8 == 0 && c_rows % 8 == 0 &&
                       ring % 8 == 0 && (reinterpret_cast<uintptr_t>(kf) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(vf) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(kc) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(vc) & 15) == 0;
  if (aligned) {
    const int64_t span = pos_b - (pos_a & ~(int64_t)7);
    hipLaunchKernelGGL(kv_write_tiled_kernel, dim3((unsigned)((span + 63) / 64), n_kv, B), dim3(256), 0,
                       st, kf, vf, f_rows, f_origin, n_kv, dh, pos_a, pos_b, kc, vc, c_rows, ring, rl);
  } else {
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)(pos_b - pos_a), n_kv, B), dim3(dh), 0, st,
                       kf, vf, f_rows, f_origin, n_kv, dh, pos_a, kc, vc, c_rows, ring, rl);
  }
  return hipGetLastError();
}

hipError_t launch_kv_copy(const uint16_t* sk, const uint16_t* sv, int64_t s_rows, int64_t s_ring,
                          int s_seq, uint16_t* dk, uint16_t* dv, int64_t d_rows, int64_t d_ring,
                          int d_seq, int n_kv, int dh, int64_t pos_a, int64_t pos_b,
                          hipStream_t st) {
  if (pos_b <= pos_a) return hipSuccess;
  if (dh % 8 != 0 || s_rows % 8 != 0 || d_rows % 8 != 0 || s_ring % 8 != 0 || d_ring % 8 != 0)
    return hipErrorInvalidValue;
  const int64_t span = pos_b - (pos_a & ~(int64_t)7);
  hipLaunchKernelGGL(kv_copy_kernel, dim3((unsigned)((span + 63) / 64), n_kv), dim3(256), 0, st,
                     sk, sv, s_rows, s_ring, (int64_t)s_seq * n_kv, dk, dv, d_rows, d_ring,
                     (int64_t)d_seq * n_kv, dh, pos_a, pos_b);
  return hipGetLastError();
}

hipError_t launch_rope_table(int64_t p0, int T, int dh, double base, float* cs, float* sn,
                             hipStream_t st, const int64_t* p0_dev) {
  const int half = dh / 2;
  const int64_t n = (int64_t)T * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p0, T,
                     half, dh, base, cs, sn, p0_dev);
  return hipGetLastError();
}

namespace {
__global__ void set_i64_kernel(int64_t* dst, int64_t v) { *dst = v; }
}  // namespace

hipError_t launch_set_i64(int64_t* dst, int64_t v, hipStream_t st) {
  hipLaunchKernelGGL(set_i64_kernel, dim3(1), dim3(1), 0, st, dst, v);
  return hipGetLastError();
}

hipError_t launch_vt_zero_cols(uint16_t* vf, int64_t f_rows, int B, int n_kv, int dh, int64_t c0,
                               int64_t c1, hipStream_t st) {
  if (c1 <= c0) return hipSuccess;
  hipLaunchKernelGGL(vt_zero_cols_kernel, dim3(n_kv, B), dim3(dh), 0, st, vf, f_rows, n_kv, dh, c0, c1);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* x, int rows, int n, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(NT_ARG), 0, st, x, n, out);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* p, int64_t n, uint16_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_kv_place(const uint16_t* k, const uint16_t* v, int B, int n_kv, int T, int dh,
                           int64_t p0, QkDest dst, hipStream_t st) {
  hipLaunchKernelGGL(kv_place_kernel, dim3(T, n_kv, B), dim3(dh), 0, st, k, v, T, n_kv, dh, p0, dst);
  return hipGetLastError();
}

hipError_t launch_mask_probe_v(uint16_t* vc, int64_t c_rows, int64_t ring, uint16_t* vnew, int B,
                               int T, int n_kv, int dh, int64_t p0, int64_t ua, int64_t ub,
                               int64_t first, hipStream_t st) {
  if (ub <= ua) return hipSuccess;
  hipLaunchKernelGGL(mask_probe_v_kernel, dim3((unsigned)(ub - ua), n_kv, B), dim3(dh), 0, st, vc,
                     c_rows, ring, vnew, T, n_kv, dh, p0, ua, first);
  return hipGetLastError();
}

hipError_t launch_mask_extract(const uint16_t* z, int B, int T, int n_q, int dh, int64_t L,
                               int64_t first, uint16_t* out, hipStream_t st) {
  hipLaunchKernelGGL(mask_extract_kernel, dim3(B * T, n_q), dim3(dh), 0, st, z, T, n_q, dh, L, first,
                     out);
  return hipGetLastError();
}

hipError_t launch_slot_rows(int64_t pos_a, int64_t n, int64_t ring, int64_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(slot_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pos_a, n,
                     ring, out);
  return hipGetLastError();
}

}  // namespace dory
