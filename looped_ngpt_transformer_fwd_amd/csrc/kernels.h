// Host-side launchers of the gfx950 kernels. Each returns the HIP error of
// its launch. All pointers are device pointers; bf16 values are passed as
// their 16-bit patterns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dory {

// ---------------------------------------------------------------- GEMM
// C[m, n] = sum_k A[m, k] * B[n, k]  (both operands K-contiguous, bf16;
// accumulation in fp32 on MFMA). K must be a multiple of 64.
enum GemmEpi {
  EPI_F32 = 0,     // C (+ split * split_stride) = partial sum of split z
  EPI_SWIGLU = 1,  // B = [W_up; W_gate] (2F rows); C16[m, f] =
                   //   bf16(SiLU(s2[f] * gate) * s1[f] * up); N = 2F; no split;
                   //   large-M path only
  EPI_LOGITS = 2,  // C[m, n] = s1[n] * acc; no split
  EPI_QKV = 3,     // fused query/key transform (large-M path, head_dim 128):
                   // columns of B = w_qkvg; writes q_hat, fresh K, fresh V^T
                   // and sigma(gate) as qk_prep does (see QkvEpi)
  EPI_BF16 = 4,    // C16[m, n] = bf16(acc) (ldc16); large-M path only, no split
};

// Destinations of the fused q/k/v/gate epilogue. Row m = b * T + t is the
// token at position p0 + t; cs/sn hold cos/sin of RoPE angle (p0 + t) *
// theta_i as [T][64].
struct QkvEpi {
  uint16_t* qh = nullptr;     // [B][n_q][T][128]
  uint16_t* kf = nullptr;     // [B][n_kv][f_rows][128], row t + row_off
  uint16_t* vf = nullptr;     // [B][n_kv][128][f_rows], column t + row_off
  uint16_t* gate = nullptr;   // [B*T][n_q*128]
  const float* cs = nullptr;
  const float* sn = nullptr;
  const float* s_qk = nullptr;
  int T = 0, nq = 0, nkv = 0;
  int64_t f_rows = 0, row_off = 0;
};

struct GemmArgs {
  const uint16_t* A = nullptr;
  int64_t lda = 0;
  const uint16_t* B = nullptr;
  int64_t ldb = 0;
  int M = 0, N = 0, K = 0;
  int nsplit = 1;
  float* C = nullptr;
  int64_t ldc = 0;
  int64_t split_stride = 0;
  uint16_t* C16 = nullptr;
  int64_t ldc16 = 0;
  const float* s1 = nullptr;
  const float* s2 = nullptr;
  int F = 0;
  int order = 0;  // large-M tile order, set by the launcher
  QkvEpi qkv;
  // MXFP8 weights (M <= 64, fp32 output): E4M3 codes [N][K] replace B, block
  // scale codes [N][K / 32]
  const uint8_t* Bq = nullptr;
  const uint8_t* Bs = nullptr;
};

// GEMMs with at most this many rows (every M below the large-M kernel's
// 1024) and an fp32 or logits output stream the weights through the skinny
// kernel (no fused SwiGLU epilogue there).
constexpr int kGemmSkinnyMaxM = 1023;

// Picks a tile configuration and split factor; `max_split` bounds the split
// (the workspace holds that many partial outputs).
int gemm_pick_split(int M, int N, int K, int max_split);
hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st);

// MXFP8 quantization of a bf16 matrix [rows][cols] (cols a multiple of 32):
// E4M3 codes [rows][cols], scale codes [rows][cols / 32] and, if deq is not
// null, the dequantized values as bf16 [rows][cols]. 16-byte aligned rows.
hipError_t launch_mx_quantize(const uint16_t* w, int64_t rows, int cols, uint8_t* codes,
                              uint8_t* scales, uint16_t* deq, hipStream_t st);

// Loop counts per sequence for a step whose sequences run different k (the
// loop-count-per-request property of the looped model). k_rows == nullptr:
// every sequence runs every loop. Token row m belongs to sequence m / T; in
// recurrent loop `loop` a sequence is active iff loop < k_rows[b].
struct RowLoops {
  const int32_t* k_rows = nullptr;  // device [B]
  int loop = 0;
  int T = 1;
};

// ---------------------------------------------------------------- row ops
// h32/h16[m, :] = E[tok[m], :]; out-of-range ids give NaN rows.
hipError_t launch_embed(const int32_t* tok, const uint16_t* E, int vocab, int M, int d,
                        float* h32, uint16_t* h16, float* x32, hipStream_t st);

// nGPT update h <- N(h + alpha (N(y) - h)), y = sum of nsplit partials.
// If x != null, additionally applies the loop boundary to the result:
//   state_out (optional) = result; h <- N(result + x).
// With rl.k_rows: rows of sequences that have left the loop are untouched,
// and a sequence in its last loop gets no boundary.
hipError_t launch_update(float* h32, uint16_t* h16, const float* y, int nsplit,
                         int64_t split_stride, int64_t ldy, const float* alpha, int M, int d,
                         const float* x, float* state_out, float* copy_out, hipStream_t st,
                         RowLoops rl = RowLoops(), bool y_bf16 = false);

// dst [cols][rows] = transpose of src [rows][cols] (int32).
hipError_t launch_transpose_i32(const int32_t* src, int rows, int cols, int32_t* dst, hipStream_t st);

// Loop boundary h <- N(h + x) (also writes the bf16 shadow).
hipError_t launch_boundary(float* h32, uint16_t* h16, const float* x, int M, int d,
                           hipStream_t st);

// Copy fp32 rows (row stride `ld_src`) into `dst` [rows, d].
hipError_t launch_copy_rows(const float* src, int64_t ld_src, float* dst, int rows, int d,
                            hipStream_t st);

// Split-sum of [nsplit][M][2F] partials and SwiGLU -> a [M, F] bf16.
hipError_t launch_swiglu_partials(const float* p, int nsplit, int64_t split_stride, int M, int F,
                                  const float* s_u, const float* s_v, uint16_t* a, hipStream_t st);

// Query/key transform. P = [nsplit][M][d_q + 2 d_kv + d_q] projections
// (rows m = b * C + t, position p0 + t); cs/sn: RoPE table of the layer's
// base for the step's positions ([C][dh/2], see launch_rope_table). Writes
//   q_hat [B][n_q][C][dh] bf16 = s_qk * N(RoPE(q))
//   k_hat to kdst, v to vdst (see QkDest), sigma(g) [M][d_q] bf16.
struct QkDest {
  // Key rows: kbase + ((b * n_kv + g) * k_rows + row(t)) * dh
  // V^T:      vbase + ((b * n_kv + g) * dh + d) * v_cols + row(t)
  // row(t) = (p0 + t - pos_origin) mod ring  (ring = 0: no modulo)
  uint16_t* kbase;
  uint16_t* vbase;
  int64_t k_rows;
  int64_t v_cols;
  int64_t pos_origin;
  int64_t ring;
};
// With rl.k_rows, sequences that have left the loop store no K/V.
// p0_dev (optional): the position is read from device memory instead.
hipError_t launch_qk_prep(const float* P, int nsplit, int64_t split_stride, int B, int C,
                          int64_t p0, int n_q, int n_kv, int dh, const float* cs, const float* sn,
                          const float* s_qk, uint16_t* q_hat, QkDest kv, uint16_t* gate,
                          hipStream_t st, RowLoops rl = RowLoops(),
                          const int64_t* p0_dev = nullptr);

// RoPE table for positions p0 .. p0 + T - 1: cs/sn [T][dh/2] fp32 from fp64
// angles (p0 + t) * base^(-2i/dh).
hipError_t launch_rope_table(int64_t p0, int T, int dh, double base, float* cs, float* sn,
                             hipStream_t st, const int64_t* p0_dev = nullptr);

// *dst = v (one thread): the step position of a replayed decode graph.
hipError_t launch_set_i64(int64_t* dst, int64_t v, hipStream_t st);

// Copy cached K / V^T entries of positions [pos_a, pos_b) into the fresh
// buffers (layout as QkDest with pos_origin = pos_a, no ring).
hipError_t launch_prefix_copy(const uint16_t* kc, const uint16_t* vc, int64_t c_rows,
                              int64_t ring, int B, int n_kv, int dh, int64_t pos_a,
                              int64_t pos_b, uint16_t* kf, uint16_t* vf, int64_t f_rows,
                              hipStream_t st);

// Persistent-cache store of positions [pos_a, pos_b) from fresh buffers
// (origin f_origin) into the cache (ring slots if ring > 0). With
// rl.k_rows, only sequences in their last loop (rl.loop == k_rows[b] - 1)
// store.
hipError_t launch_kv_write(const uint16_t* kf, const uint16_t* vf, int64_t f_rows,
                           int64_t f_origin, int B, int n_kv, int dh, int64_t pos_a,
                           int64_t pos_b, uint16_t* kc, uint16_t* vc, int64_t c_rows,
                           int64_t ring, hipStream_t st, RowLoops rl = RowLoops());

// Copy the entries of positions [pos_a, pos_b) of sequence s_seq of one
// cache slot into sequence d_seq of another (layouts as QkDest: K rows
// [batch][n_kv][rows][dh], V^T [batch][n_kv][dh][rows]; row = pos mod ring
// when ring > 0). The two ranges must not overlap in memory unless identical.
hipError_t launch_kv_copy(const uint16_t* sk, const uint16_t* sv, int64_t s_rows, int64_t s_ring,
                          int s_seq, uint16_t* dk, uint16_t* dv, int64_t d_rows, int64_t d_ring,
                          int d_seq, int n_kv, int dh, int64_t pos_a, int64_t pos_b,
                          hipStream_t st);

// Zero columns [c0, c1) of every row of a fresh V^T buffer
// ([B][n_kv][dh][f_rows]); the prefill attention reads whole 8-key chunks.
hipError_t launch_vt_zero_cols(uint16_t* vf, int64_t f_rows, int B, int n_kv, int dh, int64_t c0,
                               int64_t c1, hipStream_t st);

// Greedy argmax over rows of [rows, n] fp32, lowest index on ties.
hipError_t launch_argmax(const float* x, int rows, int n, int32_t* out, hipStream_t st);

// ------------------------------------------------------------ debug dumps
// n 16-bit values set to v.
hipError_t launch_fill_u16(uint16_t* p, int64_t n, uint16_t v, hipStream_t st);
// K and V of positions p0 .. p0 + T - 1 ([B][n_kv][T][dh] bf16) stored where
// the query/key transform stores them (see QkDest).
hipError_t launch_kv_place(const uint16_t* k, const uint16_t* v, int B, int n_kv, int T, int dh,
                           int64_t p0, QkDest dst, hipStream_t st);
// One-hot V probe values for positions [ua, ub): 1.0 at head dimension
// u - first, 0 elsewhere; cached positions (below p0, and held by the ring)
// into the cache slot's V^T, the step's positions into vnew [B][n_kv][T][dh].
hipError_t launch_mask_probe_v(uint16_t* vc, int64_t c_rows, int64_t ring, uint16_t* vnew, int B,
                               int T, int n_kv, int dh, int64_t p0, int64_t ua, int64_t ub,
                               int64_t first, hipStream_t st);
// out [B][n_q][T][L] at key columns first .. first + dh - 1: the bf16 z values.
hipError_t launch_mask_extract(const uint16_t* z, int B, int T, int n_q, int dh, int64_t L,
                               int64_t first, uint16_t* out, hipStream_t st);
// out[i] = cache row of position pos_a + i in a slot with this ring.
hipError_t launch_slot_rows(int64_t pos_a, int64_t n, int64_t ring, int64_t* out, hipStream_t st);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const uint16_t* q;     // [B][n_q][C][dh]
  const uint16_t* kc;    // cache K [B][n_kv][c_rows][dh] (nullptr if no prefix)
  const uint16_t* vc;    // cache V^T [B][n_kv][dh][c_rows]
  int64_t c_rows;        // rows per (b, g) in the cache
  int64_t ring;          // 0: linear (row = pos), else row = pos mod ring
  const uint16_t* kf;    // fresh K [B][n_kv][f_rows][dh]; row = pos - f_origin
  const uint16_t* vf;    // fresh V^T [B][n_kv][dh][f_rows]
  int64_t f_rows;
  int64_t f_origin;      // position of fresh row 0 (multiple of 8, <= p0)
  const uint16_t* gate;  // sigma(g) [B*C][n_q*dh] bf16
  uint16_t* z;           // out [B*C][n_q*dh] bf16 (gated, un-normalized)
  int B, C, n_q, n_kv, dh;
  int64_t p0;            // position of query row 0
  int window;            // 0 = full (causal) else sliding window
  float scale;           // logit scale (sqrt(dh))
  RowLoops rl;           // sequences past their loop count are skipped (z rows
                         // left as they are in prefill, zero in decode)
  const int64_t* p0_dev = nullptr;  // decode: position read from device memory
                                    // (replayed graphs), else p0
  // decode with the query/key transform fused in (else q and gate are read
  // from q / gate): split-K partials of the q/k/v/gate projection, row b =
  // sequence b ([qkv_nsplit][B][2 dq + 2 dkv], split stride qkv_ss), the
  // RoPE cos/sin of the step's position ([dh / 2] each) and s_qk. The
  // workgroup holding key p also stores the token's k and v in the cache.
  const float* qkv_part = nullptr;
  int qkv_nsplit = 0;
  int64_t qkv_ss = 0;
  const float* cs = nullptr;
  const float* sn = nullptr;
  const float* s_qk = nullptr;
  // prefill: the layer's s_qk ([dh]), from which the kernel bounds every
  // score and, when the bound allows, uses it as a fixed softmax reference;
  // null: running maximum (inputs not made by the layer, e.g. probes)
  const float* ref_s_qk = nullptr;
};
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t st);

// Decode attention over cache rows only (current token already stored);
// split over keys with `part` scratch of decode_attn_part_floats() floats.
int64_t decode_attn_part_floats(int B, int n_q, int dh, int nsplit);
// Splits for a decode query at position p whose keys are [lo, p]; window:
// a sliding-window layer (shorter splits).
int decode_attn_pick_split(int64_t lo, int64_t p, bool window);
// Keys per split for that query (the split size changes above 65,536 keys).
int decode_attn_split_keys(int64_t lo, int64_t p, bool window);
// nsplit: the launched split count (the partials' stride). With a.p0_dev the
// kernels read the position from device memory, splits past the query's
// last key exit, and the merge takes the splits that hold keys; the split
// size is the one a.p0 selects (a replayed graph is captured per size).
hipError_t launch_attn_decode(const AttnArgs& a, int nsplit, float* part, hipStream_t st);

// ------------------------------------------------------- sampled decoding
// Sampling by inversion from softmax(logits / T): out[r] = the smallest i
// whose cumulative weight exceeds u[r] * total.
hipError_t launch_sample(const float* logits, int rows, int V, float temperature, const float* u,
                         int32_t* out, hipStream_t st);
// Self-speculative rejection rule over draft_logits [gamma][B][V],
// verify_logits [gamma + 1][B][V], drafts [gamma][B] and uniforms
// u [gamma + 1][B]: n_out [B] accepted drafts, out [gamma + 1][B] the accepted
// drafts then the next token then -1.
hipError_t launch_spec_accept(const float* draft_logits, const float* verify_logits,
                              const int32_t* drafts, const float* u, int B, int V, int gamma,
                              float temperature, int32_t* n_out, int32_t* out, hipStream_t st);

// ------------------------------------------------------- fp32 debug build
// The same steps on fp32 tensors (weights, K/V, activations): embedding,
// C = A B^T (optionally times scale[n]), the query/key transform into q_hat
// [B][n_q][C][dh], K rows / V^T columns at cache_row(p0 + t - pos_origin,
// ring) and sigma(gate), attention with keys below f_origin from the cache
// and the rest from the fresh buffers (row u - f_origin), SwiGLU, and the
// persistent store of fresh K/V.
hipError_t launch_embed_f32(const int32_t* tok, const float* E, int vocab, int M, int d,
                            float* h32, float* x32, hipStream_t st);
hipError_t launch_sgemm(const float* A, int64_t lda, const float* B, int64_t ldb, int M, int N,
                        int K, float* C, int64_t ldc, const float* scale, hipStream_t st);
hipError_t launch_qk_prep_f32(const float* P, int B, int C, int64_t p0, int n_q, int n_kv, int dh,
                              const float* cs, const float* sn, const float* s_qk, float* q_hat,
                              float* kdst, float* vdst, int64_t k_rows, int64_t v_cols,
                              int64_t pos_origin, int64_t ring, float* gate, hipStream_t st,
                              RowLoops rl);
hipError_t launch_attn_f32(const float* q, const float* kc, const float* vc, int64_t c_rows,
                           int64_t ring, const float* kf, const float* vf, int64_t f_rows,
                           int64_t f_origin, const float* gate, float* z, int B, int C, int n_q,
                           int n_kv, int dh, int64_t p0, int window, float scale, RowLoops rl,
                           hipStream_t st);
hipError_t launch_swiglu_f32(const float* p, int M, int F, const float* s_u, const float* s_v,
                             float* a, hipStream_t st);
hipError_t launch_kv_write_f32(const float* kf, const float* vf, int64_t f_rows, int64_t f_origin,
                               int B, int n_kv, int dh, int64_t pos_a, int64_t pos_b, float* kc,
                               float* vc, int64_t c_rows, int64_t ring, hipStream_t st,
                               RowLoops rl);

}  // namespace dory
