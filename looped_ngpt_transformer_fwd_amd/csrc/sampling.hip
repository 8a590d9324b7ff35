// Sampled decoding for self-speculative rounds (section Self-Speculative
// Decoding): sampling by inversion from softmax(logits / T), and the
// rejection rule that accepts drafted tokens with probability
// min(1, p / q) and corrects the first rejection from the residual
// max(0, p - q), which keeps the verifier's sampling distribution. The
// uniforms are inputs: the kernels draw no random numbers.
//
// One workgroup of 1024 threads per row: each thread owns a contiguous chunk
// of the vocabulary, so a block-wide exclusive scan of the chunk sums tells
// which thread's chunk holds the inverse-CDF target, and that thread walks
// its chunk in index order.
#include "common.h"
#include "kernels.h"

namespace dory {

namespace {

constexpr int NT_S = 1024;

__device__ __forceinline__ float block_max_1024(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT_S / 64; ++i) t = fmaxf(t, red[i]);
  __syncthreads();
  return t;
}

// Prefix sums of v over the block in thread order: *lo = sum over the
// threads before this one, *hi = *lo + v, computed so that *hi of a thread
// is bit for bit the *lo of the next (the intervals [lo, hi) of the threads
// tile [0, total) exactly, whatever the rounding); returns the total.
__device__ __forceinline__ float block_scan_1024(float v, float* red, float* lo, float* hi) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  float prev = __shfl_up(incl, 1, 64);
  if (lane == 0) prev = 0.f;
  if (lane == 63) red[w] = incl;
  __syncthreads();
  // the same additions in the same order in every thread, so that the total
  // (and u * total) is one value block-wide and equals the last thread's hi
  float base = 0.f, tot = 0.f;
  for (int i = 0; i < NT_S / 64; ++i) {
    if (i == w) base = tot;
    tot += red[i];
  }
  __syncthreads();
  *lo = base + prev;
  *hi = base + incl;
  return tot;
}

// Inversion over the weights w(i) of one row (a functor of the index): the
// smallest i whose cumulative weight exceeds u * total. A target at or past
// the end of the claimed ranges (rounding) takes the last index of nonzero
// weight; a row without positive weight gives -1.
template <class Wt>
__device__ __forceinline__ int invert_row(const Wt& weight, int V, float u, float* red,
                                          int* pick) {
  const int chunk = (V + NT_S - 1) / NT_S;
  const int i0 = min(V, (int)threadIdx.x * chunk), i1 = min(V, i0 + chunk);
  float s = 0.f;
  int last_nz = -1;
  for (int i = i0; i < i1; ++i) {
    const float wi = weight(i);
    s += wi;
    if (wi > 0.f) last_nz = i;
  }
  float lo, hi;
  const float total = block_scan_1024(s, red, &lo, &hi);
  if (threadIdx.x == 0) *pick = -1;
  __syncthreads();
  const float target = u * total;
  if (lo <= target && target < hi) {  // exactly one thread when 0 <= target < total
    float c = lo;
    int found = last_nz;
    for (int i = i0; i < i1; ++i) {
      c += weight(i);
      if (c > target) { found = i; break; }
    }
    *pick = found;
  }
  __syncthreads();
  if (*pick < 0 && last_nz >= 0) atomicMax(pick, last_nz);
  __syncthreads();
  const int r = *pick;
  __syncthreads();  // *pick may be reused by the caller
  return r;
}

// max and normalizer of softmax(row / T)
__device__ __forceinline__ void row_softmax_stats(const float* row, int V, float it, float* red,
                                                  float* mx, float* z) {
  float m = -INFINITY;
  for (int i = threadIdx.x; i < V; i += NT_S) m = fmaxf(m, row[i]);
  m = block_max_1024(m, red);
  float s = 0.f;
  for (int i = threadIdx.x; i < V; i += NT_S) s += expf((row[i] - m) * it);
  float lo, hi;
  *mx = m;
  *z = block_scan_1024(s, red, &lo, &hi);
}

__global__ void __launch_bounds__(NT_S)
sample_kernel(const float* logits, int V, float temperature, const float* u, int32_t* out) {
  __shared__ float red[NT_S / 64];
  __shared__ int pick;
  const float* row = logits + (int64_t)blockIdx.x * V;
  const float it = 1.0f / temperature;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < V; i += NT_S) m = fmaxf(m, row[i]);
  m = block_max_1024(m, red);
  auto w = [&](int i) { return expf((row[i] - m) * it); };
  const int r = invert_row(w, V, u[blockIdx.x], red, &pick);
  if (threadIdx.x == 0) out[blockIdx.x] = max(r, 0);  // (no finite logit: token 0)
}

// One workgroup per sequence b. draft_logits [gamma][B][V], verify_logits
// [gamma + 1][B][V], drafts [gamma][B], u [gamma + 1][B]; out [gamma + 1][B]:
// the accepted drafts, then the next token, then -1.
__global__ void __launch_bounds__(NT_S)
spec_accept_kernel(const float* draft_logits, const float* verify_logits, const int32_t* drafts,
                   const float* u, int B, int V, int gamma, float temperature, int32_t* n_out,
                   int32_t* out) {
  __shared__ float red[NT_S / 64];
  __shared__ int pick;
  const int b = blockIdx.x;
  const float it = 1.0f / temperature;
  int j = 0;
  float mq = 0.f, zq = 1.f, mp = 0.f, zp = 1.f;
  for (; j < gamma; ++j) {
    const float* qrow = draft_logits + ((int64_t)j * B + b) * V;
    const float* prow = verify_logits + ((int64_t)j * B + b) * V;
    row_softmax_stats(qrow, V, it, red, &mq, &zq);
    row_softmax_stats(prow, V, it, red, &mp, &zp);
    const int x = min(max(drafts[(int64_t)j * B + b], 0), V - 1);
    const float qx = expf((qrow[x] - mq) * it) / zq;
    const float px = expf((prow[x] - mp) * it) / zp;
    if (!(u[(int64_t)j * B + b] < px / qx)) break;  // (uniform across the block)
  }
  int nxt;
  if (j < gamma) {
    // first rejection at draft j: the residual max(0, p_j - q_j)
    const float* qrow = draft_logits + ((int64_t)j * B + b) * V;
    const float* prow = verify_logits + ((int64_t)j * B + b) * V;
    auto w = [&](int i) {
      return fmaxf(expf((prow[i] - mp) * it) / zp - expf((qrow[i] - mq) * it) / zq, 0.f);
    };
    nxt = invert_row(w, V, u[(int64_t)gamma * B + b], red, &pick);
    if (nxt < 0) {
      // no residual mass (p <= q everywhere in fp32, so p and q agree up to
      // rounding): the verifier's own distribution
      auto wp = [&](int i) { return expf((prow[i] - mp) * it); };
      nxt = max(invert_row(wp, V, u[(int64_t)gamma * B + b], red, &pick), 0);
    }
  } else {
    const float* prow = verify_logits + ((int64_t)gamma * B + b) * V;
    float m = -INFINITY;
    for (int i = threadIdx.x; i < V; i += NT_S) m = fmaxf(m, prow[i]);
    m = block_max_1024(m, red);
    auto w = [&](int i) { return expf((prow[i] - m) * it); };
    nxt = max(invert_row(w, V, u[(int64_t)gamma * B + b], red, &pick), 0);
  }
  if (threadIdx.x <= gamma) {
    const int r = threadIdx.x;
    out[(int64_t)r * B + b] = r < j ? drafts[(int64_t)r * B + b] : (r == j ? nxt : -1);
  }
  if (threadIdx.x == 0) n_out[b] = j;
}

}  // namespace

hipError_t launch_sample(const float* logits, int rows, int V, float temperature, const float* u,
                         int32_t* out, hipStream_t st) {
  if (rows < 1 || V < 1 || !(temperature > 0.f)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_kernel, dim3(rows), dim3(NT_S), 0, st, logits, V, temperature, u, out);
  return hipGetLastError();
}

hipError_t launch_spec_accept(const float* draft_logits, const float* verify_logits,
                              const int32_t* drafts, const float* u, int B, int V, int gamma,
                              float temperature, int32_t* n_out, int32_t* out, hipStream_t st) {
  if (B < 1 || V < 1 || gamma < 1 || gamma >= NT_S || !(temperature > 0.f))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(spec_accept_kernel, dim3(B), dim3(NT_S), 0, st, draft_logits, verify_logits,
                     drafts, u, B, V, gamma, temperature, n_out, out);
  return hipGetLastError();
}

}  // namespace dory
