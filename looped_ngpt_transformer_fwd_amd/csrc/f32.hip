// fp32 debug build of the forward pass: the same step as the bf16 path (same
// runtime control flow, schedule, cache policies and layouts, with every
// tensor in fp32), on plain fp32 arithmetic. It exists to check the method at
// a tighter tolerance than bf16 allows; the kernels favour simplicity over
// speed and are meant for small models.
//
//   embed_f32      h = E[tok] (fp32 table)
//   sgemm_kernel   C = A B^T on 64 x 64 tiles staged through LDS, 4 x 4
//                  outputs per thread, fp32 FMA (optional logit scale)
//   qk_prep_f32    RoPE, per-head L2 norm and s_qk on q and k, v and sigma(g),
//                  K/V placed in the fresh buffers or the cache slot
//   attn_f32       one wave per (sequence, query head, query): online softmax
//                  over the visible keys, from the cache below the step's
//                  first position and from the fresh buffers within it
//   swiglu_f32     SiLU(s_v gate) s_u up from the projection output
//   kv_write_f32   fresh K/V of the step into the cache slot
#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

__global__ void embed_f32_kernel(const int32_t* tok, const float* E, int vocab, int d, float* h32,
                                 float* x32) {
  const int m = blockIdx.x;
  const int id = tok[m];
  const bool ok = id >= 0 && id < vocab;
  const float* src = E + (int64_t)(ok ? id : 0) * d;
  const float nanv = __uint_as_float(0x7fc00000u);
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float f = ok ? src[i] : nanv;
    h32[(int64_t)m * d + i] = f;
    if (x32) x32[(int64_t)m * d + i] = f;
  }
}

// C[m, n] (* scale[n]) = sum_k A[m, k] B[n, k]; 256 threads, 64 x 64 tile,
// K in steps of 16 through LDS (stored transposed, padded against bank
// conflicts); thread (ty, tx) computes rows ty + 16 i and columns tx + 16 j.
constexpr int SG_T = 64, SG_K = 16;
__global__ void __launch_bounds__(256)
sgemm_kernel(const float* A, int64_t lda, const float* B, int64_t ldb, int M, int N, int K,
             float* C, int64_t ldc, const float* scale) {
  __shared__ float As[SG_K][SG_T + 1];
  __shared__ float Bs[SG_K][SG_T + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * SG_T, n0 = blockIdx.x * SG_T;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += SG_K) {
    for (int i = threadIdx.x; i < SG_T * SG_K; i += 256) {
      const int r = i / SG_K, kk = i % SG_K;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.f;
      Bs[kk][r] = (gn < N && gk < K) ? B[(int64_t)gn * ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SG_K; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) C[(int64_t)m * ldc + n] = acc[i][j] * (scale ? scale[n] : 1.f);
    }
}

// heads = true: grid (token rows, n_q + n_kv), one wave per q or k head,
// lane i < dh / 2 rotating the pair (i, i + dh / 2). heads = false: grid
// (token rows), 256 threads over the v and gate columns.
// P: [M][2 d_q + 2 d_kv] projections, rows m = b * C + t at position p0 + t.
__global__ void qk_prep_f32_kernel(bool heads, const float* P, int C, int64_t p0, int nq, int nkv,
                                   int dh, const float* cs_tab, const float* sn_tab,
                                   const float* s_qk, float* qh, float* kdst, float* vdst,
                                   int64_t k_rows, int64_t v_cols, int64_t pos_origin, int64_t ring,
                                   float* gate, RowLoops rl) {
  const int m = blockIdx.x;
  const int b = m / C, t = m - b * C;
  const int64_t pos = p0 + t;
  const int half = dh >> 1;
  const int dq = nq * dh, dkv = nkv * dh;
  const float* row = P + (int64_t)m * (2 * dq + 2 * dkv);
  const int64_t krow = cache_row(pos - pos_origin, ring);
  const bool stores_kv = !(rl.k_rows && rl.loop >= rl.k_rows[b]);
  if (heads) {
    const int hh = blockIdx.y, i = threadIdx.x;
    const bool act = i < half;
    const int col = hh < nq ? hh * dh : dq + (hh - nq) * dh;
    float r1 = 0.f, r2 = 0.f;
    if (act) {
      const float c = cs_tab[(int64_t)t * half + i], sn = sn_tab[(int64_t)t * half + i];
      const float x1 = row[col + i], x2 = row[col + i + half];
      r1 = x1 * c - x2 * sn;
      r2 = x2 * c + x1 * sn;
    }
    const float inv = 1.0f / sqrtf(wave_sum(r1 * r1 + r2 * r2));
    if (!act) return;
    float* dst;
    if (hh < nq) {
      dst = qh + (((int64_t)b * nq + hh) * C + t) * dh;
    } else {
      if (!stores_kv) return;
      dst = kdst + (((int64_t)b * nkv + (hh - nq)) * k_rows + krow) * dh;
    }
    dst[i] = s_qk[i] * r1 * inv;
    dst[i + half] = s_qk[i + half] * r2 * inv;
    return;
  }
  for (int idx = threadIdx.x; idx < dkv + dq; idx += blockDim.x) {
    const float v = row[dq + dkv + idx];
    if (idx < dkv) {
      if (!stores_kv) continue;
      const int g = idx / dh, d = idx - g * dh;
      vdst[(((int64_t)b * nkv + g) * dh + d) * v_cols + krow] = v;
    } else {
      gate[(int64_t)m * dq + (idx - dkv)] = 1.0f / (1.0f + expf(-v));
    }
  }
}

// One wave per (query t, query head h, sequence b): keys u <= p (and
// p - u < window for a sliding-window layer); u below f_origin come from
// the cache slot (row cache_row(u, ring)), the rest from the fresh buffers
// (row u - f_origin). Lane d holds head dimensions d and d + 64.
__global__ void __launch_bounds__(64)
attn_f32_kernel(const float* q, const float* kc, const float* vc, int64_t c_rows, int64_t ring,
                const float* kf, const float* vf, int64_t f_rows, int64_t f_origin,
                const float* gate, float* z, int C, int nq, int nkv, int dh, int64_t p0,
                int window, float scale, RowLoops rl) {
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  if (rl.k_rows && rl.loop >= rl.k_rows[b]) return;  // left the loop: its row is not updated
  const int g = h / (nq / nkv);
  const int64_t bg = (int64_t)b * nkv + g;
  const int64_t p = p0 + t;
  const int64_t lo = window > 0 ? max((int64_t)0, p - window + 1) : 0;
  const float* qr = q + (((int64_t)b * nq + h) * C + t) * dh;
  float qv[2], ov[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) qv[j] = lane + 64 * j < dh ? qr[lane + 64 * j] : 0.f;
  float m = -INFINITY, l = 0.f;
  for (int64_t u = lo; u <= p; ++u) {
    const bool cached = u < f_origin;
    const int64_t r = cached ? cache_row(u, ring) : u - f_origin;
    const float* kr = cached ? kc + (bg * c_rows + r) * dh : kf + (bg * f_rows + r) * dh;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (lane + 64 * j < dh) s += qv[j] * kr[lane + 64 * j];
    s = wave_sum(s) * scale;
    const float m_new = fmaxf(m, s);
    const float corr = expf(m - m_new);
    const float pr = expf(s - m_new);
    l = l * corr + pr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = lane + 64 * j;
      if (d < dh) {
        const float v = cached ? vc[(bg * dh + d) * c_rows + r] : vf[(bg * dh + d) * f_rows + r];
        ov[j] = ov[j] * corr + pr * v;
      }
    }
    m = m_new;
  }
  const int64_t zr = ((int64_t)b * C + t) * nq * dh + (int64_t)h * dh;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int d = lane + 64 * j;
    if (d < dh) z[zr + d] = ov[j] / l * gate[zr + d];
  }
}

__global__ void swiglu_f32_kernel(const float* p, int M, int F, const float* s_u, const float* s_v,
                                  float* a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * F) return;
  const int64_t m = idx / F;
  const int f = (int)(idx - m * F);
  const float up = p[m * 2 * F + f] * s_u[f];
  const float gt = p[m * 2 * F + F + f] * s_v[f];
  a[idx] = gt / (1.f + expf(-gt)) * up;
}

// grid (npos, n_kv, B), block dh
__global__ void kv_write_f32_kernel(const float* kf, const float* vf, int64_t f_rows,
                                    int64_t f_origin, int nkv, int dh, int64_t pos_a, float* kc,
                                    float* vc, int64_t c_rows, int64_t ring, RowLoops rl) {
  const int64_t pos = pos_a + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  if (rl.k_rows && rl.k_rows[b] != rl.loop + 1) return;  // not this sequence's last loop
  const int64_t bg = (int64_t)b * nkv + g;
  const int64_t crow = cache_row(pos, ring);
  const int64_t frow = pos - f_origin;
  kc[(bg * c_rows + crow) * dh + d] = kf[(bg * f_rows + frow) * dh + d];
  vc[(bg * dh + d) * c_rows + crow] = vf[(bg * dh + d) * f_rows + frow];
}

}  // namespace

hipError_t launch_embed_f32(const int32_t* tok, const float* E, int vocab, int M, int d,
                            float* h32, float* x32, hipStream_t st) {
  hipLaunchKernelGGL(embed_f32_kernel, dim3(M), dim3(256), 0, st, tok, E, vocab, d, h32, x32);
  return hipGetLastError();
}

hipError_t launch_sgemm(const float* A, int64_t lda, const float* B, int64_t ldb, int M, int N,
                        int K, float* C, int64_t ldc, const float* scale, hipStream_t st) {
  if (M <= 0 || N <= 0 || K <= 0) return hipErrorInvalidValue;
  dim3 grid((N + SG_T - 1) / SG_T, (M + SG_T - 1) / SG_T);
  hipLaunchKernelGGL(sgemm_kernel, grid, dim3(256), 0, st, A, lda, B, ldb, M, N, K, C, ldc, scale);
  return hipGetLastError();
}

hipError_t launch_qk_prep_f32(const float* P, int B, int C, int64_t p0, int n_q, int n_kv, int dh,
                              const float* cs, const float* sn, const float* s_qk, float* q_hat,
                              float* kdst, float* vdst, int64_t k_rows, int64_t v_cols,
                              int64_t pos_origin, int64_t ring, float* gate, hipStream_t st,
                              RowLoops rl) {
  if (dh % 2 || dh > 128 || dh < 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qk_prep_f32_kernel, dim3(B * C, n_q + n_kv), dim3(64), 0, st, true, P, C, p0,
                     n_q, n_kv, dh, cs, sn, s_qk, q_hat, kdst, vdst, k_rows, v_cols, pos_origin,
                     ring, gate, rl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qk_prep_f32_kernel, dim3(B * C), dim3(256), 0, st, false, P, C, p0, n_q, n_kv,
                     dh, cs, sn, s_qk, q_hat, kdst, vdst, k_rows, v_cols, pos_origin, ring, gate, rl);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const float* q, const float* kc, const float* vc, int64_t c_rows,
                           int64_t ring, const float* kf, const float* vf, int64_t f_rows,
                           int64_t f_origin, const float* gate, float* z, int B, int C, int n_q,
                           int n_kv, int dh, int64_t p0, int window, float scale, RowLoops rl,
                           hipStream_t st) {
  if (dh > 128 || n_q % n_kv) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(C, n_q, B), dim3(64), 0, st, q, kc, vc, c_rows, ring, kf,
                     vf, f_rows, f_origin, gate, z, C, n_q, n_kv, dh, p0, window, scale, rl);
  return hipGetLastError();
}

hipError_t launch_swiglu_f32(const float* p, int M, int F, const float* s_u, const float* s_v,
                             float* a, hipStream_t st) {
  const int64_t n = (int64_t)M * F;
  hipLaunchKernelGGL(swiglu_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, M, F,
                     s_u, s_v, a);
  return hipGetLastError();
}

hipError_t launch_kv_write_f32(const float* kf, const float* vf, int64_t f_rows, int64_t f_origin,
                               int B, int n_kv, int dh, int64_t pos_a, int64_t pos_b, float* kc,
                               float* vc, int64_t c_rows, int64_t ring, hipStream_t st,
                               RowLoops rl) {
  if (pos_b <= pos_a) return hipSuccess;
  hipLaunchKernelGGL(kv_write_f32_kernel, dim3((unsigned)(pos_b - pos_a), n_kv, B), dim3(dh), 0, st,
                     kf, vf, f_rows, f_origin, n_kv, dh, pos_a, kc, vc, c_rows, ring, rl);
  return hipGetLastError();
}

}  // namespace dory
