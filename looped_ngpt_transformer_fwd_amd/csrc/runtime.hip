// Host runtime behind include/dory.h: argument validation, the sublayer
// schedule, KV-cache layout, workspace planning and the forward executor
// that enqueues the kernels of one prefill or decode step on a stream.
//
// Model structure followed here ("Dory1.0-4B: A Looped Normalized-GPT"):
// section Training with Loops (input block once, shared recurrent block k
// times with the input-block output re-injected and the state normalized at
// both loop boundaries, output block once) and section Last-Loop KV Caching
// (per-loop versus last-loop cache slots).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <array>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dory.h"
#include "kernels.h"

using namespace dory;

namespace {

thread_local std::string g_last_error;

dory_status fail(dory_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

int64_t round8(int64_t x) { return (x + 7) / 8 * 8; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

constexpr int kMaxDecodeSplits = 2048;
constexpr int kMaxGemmSplit = 16;   // split-K partials for 64 < M < kLargeM
constexpr int kMaxSkinnySplit = 32; // and for M <= 64 (weight-streaming path)

constexpr int64_t kLargeM = 1024;  // GEMMs at or above this many rows run unsplit
// Split-K bound of a projection with M token rows (1: no split).
int max_split_for(int64_t M) {
  return M <= 64 ? kMaxSkinnySplit : (M < kLargeM ? kMaxGemmSplit : 1);
}

struct Shape {
  int d, nq, nkv, dh, F, V, nin, nrec, nout, W, full_every, lm;
  double base_swa, base_full, scale;
  bool f32 = false;  // fp32 debug build: weights, K/V and activations in fp32
  int eb() const { return f32 ? 4 : 2; }  // bytes per weight / K / V / activation element
  int dq() const { return nq * dh; }
  int dkv() const { return nkv * dh; }
  int nsub() const { return nin + nrec + nout; }
  int nqkvg() const { return 2 * dq() + 2 * dkv(); }
};

dory_status read_shape(const dory_config* c, Shape* s) {
  if (!c) return fail(DORY_ERR_ARG, "config is NULL");
  s->d = c->d_model; s->nq = c->n_q_heads; s->nkv = c->n_kv_heads; s->dh = c->head_dim;
  s->F = c->d_ff; s->V = c->vocab; s->nin = c->n_input; s->nrec = c->n_recurrent;
  s->nout = c->n_output; s->W = c->window; s->full_every = c->full_every;
  s->lm = c->has_lm_head ? 1 : 0;
  s->base_swa = c->rope_base_swa; s->base_full = c->rope_base_full;
  s->scale = c->softmax_scale > 0 ? c->softmax_scale : std::sqrt((double)c->head_dim);
  if (c->precision != DORY_PRECISION_BF16 && c->precision != DORY_PRECISION_FP32)
    return fail(DORY_ERR_ARG, "unknown precision");
  s->f32 = c->precision == DORY_PRECISION_FP32;
  if (s->d <= 0 || s->nq <= 0 || s->nkv <= 0 || s->dh <= 0 || s->F <= 0 || s->V <= 0 ||
      s->nin < 0 || s->nrec < 0 || s->nout < 0 || s->nsub() <= 0 || s->W <= 0)
    return fail(DORY_ERR_ARG, "non-positive dimension in config");
  if (s->nq % s->nkv != 0) return fail(DORY_ERR_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (!c->layer_kinds && s->full_every <= 0) return fail(DORY_ERR_ARG, "full_every must be >= 1");
  if (!(s->base_swa > 0) || !(s->base_full > 0)) return fail(DORY_ERR_ARG, "RoPE bases must be > 0");
  const int grp = s->nq / s->nkv;
  if (s->dh != 32 && s->dh != 64 && s->dh != 128)
    return fail(DORY_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(DORY_ERR_UNSUPPORTED, "n_q/n_kv must be 1, 2, 4 or 8");
  if (s->d % 64 || s->dq() % 64 || s->F % 64)
    return fail(DORY_ERR_UNSUPPORTED, "d_model, n_q*head_dim and d_ff must be multiples of 64");
  if (s->d > 4096) return fail(DORY_ERR_UNSUPPORTED, "d_model above 4096");
  return DORY_OK;
}

dory_status build_schedule(const dory_config* c, const Shape& s, std::vector<int>* kinds) {
  kinds->assign(s.nsub(), DORY_LAYER_MLP);
  if (c->layer_kinds) {
    for (int i = 0; i < s.nsub(); ++i) {
      const int k = c->layer_kinds[i];
      if (k != DORY_LAYER_ATTN_SWA && k != DORY_LAYER_ATTN_FULL && k != DORY_LAYER_MLP)
        return fail(DORY_ERR_ARG, "invalid layer kind");
      (*kinds)[i] = k;
    }
    return DORY_OK;
  }
  // alternate attention / MLP starting with attention; every full_every-th
  // attention sublayer (1-based) is full attention
  int j = 0;
  for (int i = 0; i < s.nsub(); ++i) {
    if (i % 2 == 0) {
      (*kinds)[i] = (j % s.full_every == s.full_every - 1) ? DORY_LAYER_ATTN_FULL : DORY_LAYER_ATTN_SWA;
      ++j;
    }
  }
  return DORY_OK;
}

bool is_recurrent(const Shape& s, int i) { return i >= s.nin && i < s.nin + s.nrec; }

// Longest cache: the attention kernels take positions in 31 bits and
// address one (sequence, KV head) slab of K rows or V^T columns with 32-bit
// byte offsets (the decode kernel's buffer resources span the whole slab), so
// rows x head_dim x 2 bytes must stay below 2^32 as well.
constexpr int64_t kMaxSeq = int64_t(1) << 24;

int64_t max_seq_limit(const Shape& s) {
  const int64_t by_bytes = ((((int64_t)1 << 32) - 1) / ((int64_t)s.dh * 2)) / 8 * 8;
  return std::min(kMaxSeq, by_bytes);
}

int64_t slot_rows(const Shape& s, int kind, int64_t max_seq) {
  // a sliding-window ring keeps DORY_KV_ROLLBACK positions beyond the
  // window, so that the cache can be shortened by up to DORY_KV_ROLLBACK
  // positions (rejected speculative tokens) with every key the next step's
  // window needs still in place
  if (kind == DORY_LAYER_ATTN_SWA) return round8(std::min<int64_t>(max_seq, s.W + DORY_KV_ROLLBACK));
  return round8(max_seq);
}

size_t slot_bytes(const Shape& s, int kind, int batch, int64_t max_seq) {
  return (size_t)2 * batch * s.nkv * slot_rows(s, kind, max_seq) * s.dh * s.eb();
}

// Workspace layout for B sequences of T tokens.
struct WsLayout {
  size_t h32, h16, x32, qh, kf, vf, gate, z, a, P, part, logits, rope, krows, state, total;
  int64_t f_rows;
};

// exact_p0 >= 0 (a decode step at that position): the split-K partials and
// the decode-attention partials are sized for that step (the splits its
// GEMMs and attention launches pick) instead of for the most any step needs.
WsLayout plan_ws(const Shape& s, int B, int T, int64_t exact_p0 = -1) {
  WsLayout L{};
  const int64_t M = (int64_t)B * T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.f_rows = round8(T + 7);
  L.h32 = take(M * s.d * 4);
  L.h16 = take(M * s.d * 2);
  L.x32 = take(M * s.d * 4);
  const int eb = s.eb();
  L.qh = take(M * s.dq() * eb);
  L.kf = take((size_t)B * s.nkv * L.f_rows * s.dh * eb);
  L.vf = take((size_t)B * s.nkv * L.f_rows * s.dh * eb);
  L.gate = take(M * s.dq() * eb);
  L.z = take(M * s.dq() * eb);
  L.a = take(M * s.F * eb);
  if (exact_p0 >= 0 && T == 1) {
    // the projections of a decode step: (N, K) of q/k/v/gate, attention
    // output, up/gate and down
    const int shapes[4][2] = {{s.nqkvg(), s.d}, {s.d, s.dq()}, {2 * s.F, s.d}, {s.d, s.F}};
    size_t pbytes = 0;
    for (const auto& nk : shapes)
      pbytes = std::max(pbytes, (size_t)gemm_pick_split((int)M, nk[0], nk[1], max_split_for(M)) *
                                    M * nk[0] * 4);
    L.P = take(pbytes);
    const int64_t lo_w = std::max<int64_t>(0, exact_p0 - s.W + 1);
    const int ns = std::max(decode_attn_pick_split(0, exact_p0, false),
                            decode_attn_pick_split(lo_w, exact_p0, true));
    L.part = take((size_t)decode_attn_part_floats(B, s.nq, s.dh, ns) * 4);
  } else {
    int64_t ncols = std::max<int64_t>(s.nqkvg(), s.d);
    const int64_t nsplit = max_split_for(M);
    if (M < kLargeM) ncols = std::max<int64_t>(ncols, 2 * (int64_t)s.F);
    L.P = take((size_t)nsplit * M * ncols * 4);
    L.part = take((size_t)decode_attn_part_floats(B, s.nq, s.dh, kMaxDecodeSplits) * 4);
  }
  L.logits = s.lm ? take((size_t)B * s.V * 4) : 0;
  // cos / sin tables of the step's positions for the two RoPE bases
  L.rope = take((size_t)4 * T * (s.dh / 2) * 4);
  // per-sequence loop counts of a mixed-k step
  L.krows = take((size_t)B * 4);
  // the step position, read by the kernels of a replayed decode graph
  L.state = take(8);
  L.total = off;
  return L;
}

// Event pairs around kernel launches, for the measurement hooks.
struct Profiler {
  bool on = false;
  int max = 0;
  std::vector<hipEvent_t> ev;  // 2 per launch
  std::vector<int> cls;        // class of each recorded launch
  void clear() {
    for (hipEvent_t e : ev) hipEventDestroy(e);
    ev.clear();
    cls.clear();
    on = false;
    max = 0;
  }
};

struct ProfScope {
  Profiler* p;
  hipStream_t st;
  int idx = -1;
  ProfScope(Profiler* p_, hipStream_t st_, int c) : p(p_), st(st_) {
    if (p->on && (int)p->cls.size() < p->max) {
      idx = (int)p->cls.size();
      p->cls.push_back(c);
      hipEventRecord(p->ev[2 * idx], st);
    }
  }
  ~ProfScope() {
    if (idx >= 0) hipEventRecord(p->ev[2 * idx + 1], st);
  }
};

}  // namespace

// MXFP8 copy of one projection matrix [N][K]: E4M3 codes, block scale codes
// and the dequantized values in bf16 (exact).
struct MxMat {
  const uint8_t* q = nullptr;
  const uint8_t* sc = nullptr;
  const uint16_t* deq = nullptr;
};

// A captured decode step, replayed for every later step with the same
// cache, batch, loop count, policy, weight format, buffers and split size;
// only the node that writes the step position changes between replays.
// graphs kept per model (one per cache, batch, loop count, policy, weight
// format, buffers and split size); the oldest is dropped beyond this
constexpr size_t kMaxDecodeGraphs = 32;

struct DecodeGraph {
  const dory_kv* kv;
  int B, k, mode;
  bool long_ctx, mx;
  const void *tokens, *logits, *next, *hidden, *states, *ws;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipGraphNode_t pos_node = nullptr;
  hipKernelNodeParams pos_params{};
};

struct dory_model {
  Shape s;
  Profiler prof;
  std::vector<int> kinds;
  std::vector<dory_sublayer_weights> sub;
  const uint16_t* embed;
  const uint16_t* lm_head;
  const float* s_z;
  // per sublayer: [0] w_qkvg or w_upgate, [1] w_o or w_down
  std::vector<std::array<MxMat, 2>> mx;
  bool mx_ready = false;
  bool use_mx = false;
  // decode-step graphs (section Training with Loops: 32 + 40k sublayer
  // applications per token make a decode step hundreds of short launches)
  bool graphs_on = true;
  std::vector<DecodeGraph> graphs;
  hipStream_t cap_stream = nullptr;  // capture only; replays go to the caller's stream
  std::mutex graph_mu;
  void drop_graphs(const dory_kv* kv) {
    std::lock_guard<std::mutex> lock(graph_mu);
    for (auto it = graphs.begin(); it != graphs.end();) {
      if (kv && it->kv != kv) { ++it; continue; }
      if (it->exec) hipGraphExecDestroy(it->exec);
      if (it->graph) hipGraphDestroy(it->graph);
      it = graphs.erase(it);
    }
  }
  ~dory_model() {
    prof.clear();
    drop_graphs(nullptr);
    if (cap_stream) hipStreamDestroy(cap_stream);
  }
};

struct dory_kv {
  const dory_model* m;
  uint8_t* base;
  size_t bytes;
  dory_cache_mode mode;
  int k_max, batch;
  int64_t max_seq;
  int64_t len;
  // highest length written since the last reset: rows of a sliding-window
  // ring hold positions up to hi - 1, so shortening is bounded by it
  int64_t hi = 0;
  bool wraps = false;  // some sliding-window ring is shorter than max_seq
  // per-loop caching: filled[j] (j = 1 .. k_max) = number of leading
  // positions whose loop-j entries are written (non-increasing in j)
  std::vector<int64_t> filled;
  bool invalid;
  // per sublayer: offset of slot 0 (or SIZE_MAX for MLP), rows and ring
  std::vector<size_t> off;
  std::vector<int> nslots;
  std::vector<int64_t> rows, ring;
};

namespace {

struct SlotPtr {
  uint16_t* k;
  uint16_t* v;
  int64_t rows, ring;
};

SlotPtr slot_ptr(const dory_kv* kv, int sub, int slot) {
  const Shape& s = kv->m->s;
  const size_t half = (size_t)kv->batch * s.nkv * kv->rows[sub] * s.dh * s.eb();
  uint8_t* p = kv->base + kv->off[sub] + (size_t)slot * 2 * half;
  return SlotPtr{reinterpret_cast<uint16_t*>(p), reinterpret_cast<uint16_t*>(p + half),
                 kv->rows[sub], kv->ring[sub]};
}

struct Ctx {
  dory_model* m;
  dory_kv* kv;
  const Shape& s;
  int B, T;
  int64_t M, p0;
  uint8_t* ws;
  WsLayout L;
  hipStream_t st;
  float* h32() const { return reinterpret_cast<float*>(ws + L.h32); }
  uint16_t* h16() const { return reinterpret_cast<uint16_t*>(ws + L.h16); }
  float* x32() const { return reinterpret_cast<float*>(ws + L.x32); }
  uint16_t* qh() const { return reinterpret_cast<uint16_t*>(ws + L.qh); }
  uint16_t* kf() const { return reinterpret_cast<uint16_t*>(ws + L.kf); }
  uint16_t* vf() const { return reinterpret_cast<uint16_t*>(ws + L.vf); }
  uint16_t* gate() const { return reinterpret_cast<uint16_t*>(ws + L.gate); }
  uint16_t* z() const { return reinterpret_cast<uint16_t*>(ws + L.z); }
  uint16_t* a() const { return reinterpret_cast<uint16_t*>(ws + L.a); }
  float* P() const { return reinterpret_cast<float*>(ws + L.P); }
  float* part() const { return reinterpret_cast<float*>(ws + L.part); }
  float* logits_scratch() const { return reinterpret_cast<float*>(ws + L.logits); }
  // table 0 = sliding-window base, 1 = full-attention base
  float* rope_cs(int full) const {
    return reinterpret_cast<float*>(ws + L.rope) + (size_t)(2 * full) * T * (s.dh / 2);
  }
  float* rope_sn(int full) const { return rope_cs(full) + (size_t)T * (s.dh / 2); }
  // prefill projections take the fused q/k/v/gate epilogue
  bool fused_qkv() const { return T > 1 && M >= kLargeM && s.dh == 128; }
  Profiler* prof() const { return &m->prof; }
  int32_t* krows() const { return reinterpret_cast<int32_t*>(ws + L.krows); }
  bool mixed = false;  // sequences run different loop counts (krows on the device)
  // replayed decode graphs: the position is read from device memory (p0 is
  // that of the capture), and the decode attention is launched for the
  // highest position the graph serves (p_hi), its extra splits exiting
  const int64_t* p0_dev = nullptr;
  int64_t p_hi = -1;
  int64_t* state() const { return reinterpret_cast<int64_t*>(ws + L.state); }
  RowLoops rl;         // loop masks while in the recurrent block of a mixed step
};

#define PROF(c, cls) ProfScope prof_scope_##__LINE__((c).prof(), (c).st, (cls))

#define HIPCHK(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      g_last_error = std::string(#expr) + ": " + hipGetErrorString(e_);           \
      return DORY_ERR_HIP;                                                        \
    }                                                                             \
  } while (0)

// The weights a projection reads: the bf16 matrix, or with MXFP8 enabled its
// quantized copy (E4M3 codes streamed by the small-M kernel, the exact bf16
// dequantization elsewhere).
struct WSel {
  const uint16_t* b = nullptr;
  const uint8_t* q = nullptr;
  const uint8_t* sc = nullptr;
};

WSel wsel(const Ctx& c, int sub, int which, const void* w_bf16) {
  WSel r;
  r.b = reinterpret_cast<const uint16_t*>(w_bf16);
  if (c.m->use_mx) {
    const MxMat& x = c.m->mx[sub][which];
    r.b = x.deq;
    if (c.M <= 64) { r.q = x.q; r.sc = x.sc; }
  }
  return r;
}

// y = A W^T into P (split partials), returns the split used. With y16 given
// (a consumer that reads bf16), large-M calls write y once in bf16 instead
// (half the bytes of the fp32 output, which is written in one burst at the
// end of every round of tiles); *y16 tells which form was written.
dory_status gemm_f32(Ctx& c, const uint16_t* A, int64_t lda, const WSel& W, int N, int K,
                     int64_t M, int* nsplit_out, int cls, bool* y16 = nullptr) {
  PROF(c, cls);
  GemmArgs g;
  g.A = A; g.lda = lda;
  g.B = W.b; g.ldb = K; g.Bq = W.q; g.Bs = W.sc;
  g.M = (int)M; g.N = N; g.K = K;
  g.nsplit = gemm_pick_split((int)M, N, K, max_split_for(M));
  const bool half = y16 && M >= kLargeM && !W.q && g.nsplit == 1;
  if (y16) *y16 = half;
  if (half) {
    g.C16 = reinterpret_cast<uint16_t*>(c.P()); g.ldc16 = N;
    HIPCHK(launch_gemm(g, EPI_BF16, c.st));
  } else {
    g.C = c.P(); g.ldc = N; g.split_stride = M * N;
    HIPCHK(launch_gemm(g, EPI_F32, c.st));
  }
  *nsplit_out = g.nsplit;
  return DORY_OK;
}

// The update after a sublayer, with the loop-boundary fusion options.
struct UpdateOpts {
  const float* x = nullptr;  // apply boundary N(r + x) after the update
  float* aux = nullptr;      // copy of the post-update value
};

// The attention of one sublayer over the step's q_hat (grouped-query,
// sliding-window or causal by `full`), gated into z. Prefill reads the step's
// own K/V from the fresh buffers, rows counted from f_origin (the step's first
// position rounded down to 8), after copying the cached positions
// [f_origin, p0) in front of them and zeroing the V^T columns past the step's
// last key up to the next multiple of 8 (the kernel reads whole 8-key
// chunks); keys below f_origin come from the cache slot. Decode reads the
// cache slot only: the token's K/V are stored there first.
// Decode with the query/key transform fused into the attention (the
// projection's split partials instead of q / gate).
struct FusedQk {
  const float* part = nullptr;
  int nsplit = 0;
  int64_t ss = 0;
  const float *cs = nullptr, *sn = nullptr, *s_qk = nullptr;
};

// ref_s_qk: the layer's s_qk when q and the keys were made by the layer (the
// prefill kernel bounds the scores with it); null for caller-made inputs.
dory_status attend(Ctx& c, const SlotPtr& sp, bool full, const uint16_t* q, const uint16_t* gate,
                   uint16_t* z, const FusedQk* fq = nullptr, const float* ref_s_qk = nullptr) {
  const Shape& s = c.s;
  AttnArgs aa{};
  if (fq) {
    aa.qkv_part = fq->part; aa.qkv_nsplit = fq->nsplit; aa.qkv_ss = fq->ss;
    aa.cs = fq->cs; aa.sn = fq->sn; aa.s_qk = fq->s_qk;
  }
  aa.q = q;
  aa.kc = sp.k; aa.vc = sp.v; aa.c_rows = sp.rows; aa.ring = sp.ring;
  aa.gate = gate; aa.z = z;
  aa.B = c.B; aa.C = c.T; aa.n_q = s.nq; aa.n_kv = s.nkv; aa.dh = s.dh;
  aa.p0 = c.p0; aa.window = full ? 0 : s.W; aa.scale = (float)s.scale;
  aa.rl = c.rl;
  aa.p0_dev = c.p0_dev;
  if (c.T == 1) {
    const int64_t lo = full ? 0 : std::max<int64_t>(0, c.p0 - s.W + 1);
    int nsd = decode_attn_pick_split(lo, c.p0, !full);  // <= kMaxDecodeSplits (checked up front)
    if (c.p0_dev) {
      // a replayed graph serves positions up to p_hi with the split size of
      // its capture: launch the splits the highest of them needs
      const int sk = decode_attn_split_keys(lo, c.p0, !full);
      nsd = full ? (int)((c.p_hi + sk) / sk) : (int)((s.W + 63 + sk - 1) / sk);
      nsd = std::max(nsd, 1);
    }
    PROF(c, DORY_K_ATTN);
    HIPCHK(launch_attn_decode(aa, nsd, c.part(), c.st));
    return DORY_OK;
  }
  const int64_t f_origin = c.p0 / 8 * 8;
  {
    const int64_t vend = c.p0 + c.T - f_origin;
    PROF(c, DORY_K_KV_WRITE);
    HIPCHK(launch_vt_zero_cols(c.vf(), c.L.f_rows, c.B, s.nkv, s.dh, vend, (vend + 7) / 8 * 8, c.st));
  }
  if (c.p0 > f_origin) {
    PROF(c, DORY_K_KV_WRITE);
    HIPCHK(launch_prefix_copy(sp.k, sp.v, sp.rows, sp.ring, c.B, s.nkv, s.dh, f_origin, c.p0,
                              c.kf(), c.vf(), c.L.f_rows, c.st));
  }
  aa.kf = c.kf(); aa.vf = c.vf(); aa.f_rows = c.L.f_rows; aa.f_origin = f_origin;
  aa.ref_s_qk = ref_s_qk;
  PROF(c, DORY_K_ATTN);
  HIPCHK(launch_attn_prefill(aa, c.st));
  return DORY_OK;
}

dory_status attention_sublayer(Ctx& c, int i, int slot, bool write, const UpdateOpts& uo) {
  const Shape& s = c.s;
  const dory_sublayer_weights& w = c.m->sub[i];
  const int kind = c.m->kinds[i];
  const bool full = kind == DORY_LAYER_ATTN_FULL;
  const SlotPtr sp = slot_ptr(c.kv, i, slot);
  int ns = 1;
  dory_status st = DORY_OK;
  const int64_t f_origin = c.p0 / 8 * 8;
  FusedQk fq;
  if (c.fused_qkv()) {
    // projections with RoPE / per-head norm / s_qk / K-V placement / gate in
    // the GEMM epilogue
    PROF(c, DORY_K_GEMM_QKVG);
    GemmArgs g;
    g.A = c.h16(); g.lda = s.d;
    g.B = wsel(c, i, 0, w.w_qkvg).b; g.ldb = s.d;
    g.M = (int)c.M; g.N = s.nqkvg(); g.K = s.d; g.nsplit = 1;
    g.qkv.qh = c.qh(); g.qkv.kf = c.kf(); g.qkv.vf = c.vf(); g.qkv.gate = c.gate();
    g.qkv.cs = c.rope_cs(full ? 1 : 0); g.qkv.sn = c.rope_sn(full ? 1 : 0);
    g.qkv.s_qk = w.s_qk; g.qkv.T = c.T; g.qkv.nq = s.nq; g.qkv.nkv = s.nkv;
    g.qkv.f_rows = c.L.f_rows; g.qkv.row_off = c.p0 - f_origin;
    HIPCHK(launch_gemm(g, EPI_QKV, c.st));
  } else {
    st = gemm_f32(c, c.h16(), s.d, wsel(c, i, 0, w.w_qkvg), s.nqkvg(), s.d, c.M, &ns,
                  DORY_K_GEMM_QKVG);
    if (st != DORY_OK) return st;
    const int64_t split_stride = c.M * s.nqkvg();
    if (c.T == 1) {
      // decode: the attention kernel transforms q and k from the partials
      // and stores the token's K/V straight into the cache slot (the
      // last-loop rule read literally: overwrite at every loop) before it
      // reads the cache
      fq.part = c.P(); fq.nsplit = ns; fq.ss = split_stride;
      fq.cs = c.rope_cs(full ? 1 : 0); fq.sn = c.rope_sn(full ? 1 : 0); fq.s_qk = w.s_qk;
    } else {
      // prefill: the step's K/V go to the fresh buffers
      const QkDest kd{c.kf(), c.vf(), c.L.f_rows, c.L.f_rows, f_origin, 0};
      PROF(c, DORY_K_QK);
      HIPCHK(launch_qk_prep(c.P(), ns, split_stride, c.B, c.T, c.p0, s.nq, s.nkv, s.dh,
                            c.rope_cs(full ? 1 : 0), c.rope_sn(full ? 1 : 0), w.s_qk, c.qh(), kd,
                            c.gate(), c.st, RowLoops(), c.p0_dev));
    }
  }
  st = attend(c, sp, full, c.qh(), c.gate(), c.z(), fq.part ? &fq : nullptr, w.s_qk);
  if (st != DORY_OK) return st;
  if (c.T > 1 && write) {
    PROF(c, DORY_K_KV_WRITE);
    // persistent store after the step's attention; a ring keeps only the
    // newest `ring` positions
    int64_t pa = c.p0;
    if (sp.ring > 0) pa = std::max<int64_t>(pa, c.p0 + c.T - sp.ring);
    HIPCHK(launch_kv_write(c.kf(), c.vf(), c.L.f_rows, f_origin, c.B, s.nkv, s.dh, pa,
                           c.p0 + c.T, sp.k, sp.v, sp.rows, sp.ring, c.st, c.rl));
  }
  bool y16 = false;
  st = gemm_f32(c, c.z(), s.dq(), wsel(c, i, 1, w.w_o), s.d, s.dq(), c.M, &ns, DORY_K_GEMM_O, &y16);
  if (st != DORY_OK) return st;
  PROF(c, DORY_K_UPDATE);
  HIPCHK(launch_update(c.h32(), c.h16(), c.P(), ns, c.M * s.d, s.d, w.alpha, (int)c.M, s.d, uo.x,
                       uo.aux, nullptr, c.st, c.rl, y16));
  return DORY_OK;
}

dory_status mlp_sublayer(Ctx& c, int i, const UpdateOpts& uo) {
  const Shape& s = c.s;
  const dory_sublayer_weights& w = c.m->sub[i];
  const int ns_up = gemm_pick_split((int)c.M, 2 * s.F, s.d, max_split_for(c.M));
  const WSel wug = wsel(c, i, 0, w.w_upgate);
  // the fused SwiGLU epilogue reads bf16 weights and runs on the tiled
  // kernels; MXFP8 codes and the skinny kernel go through fp32 outputs
  if (ns_up == 1 && !wug.q && c.M > kGemmSkinnyMaxM) {
    PROF(c, DORY_K_GEMM_UPGATE);
    GemmArgs g;
    g.A = c.h16(); g.lda = s.d;
    g.B = wug.b; g.ldb = s.d;
    g.M = (int)c.M; g.N = 2 * s.F; g.K = s.d; g.nsplit = 1;
    g.C16 = c.a(); g.ldc16 = s.F; g.s1 = w.s_u; g.s2 = w.s_v; g.F = s.F;
    HIPCHK(launch_gemm(g, EPI_SWIGLU, c.st));
  } else {
    int ns = 1;
    dory_status st = gemm_f32(c, c.h16(), s.d, wug, 2 * s.F, s.d, c.M, &ns, DORY_K_GEMM_UPGATE);
    if (st != DORY_OK) return st;
    PROF(c, DORY_K_OTHER);
    HIPCHK(launch_swiglu_partials(c.P(), ns, c.M * 2 * s.F, (int)c.M, s.F, w.s_u, w.s_v, c.a(),
                                  c.st));
  }
  int ns = 1;
  bool y16 = false;
  dory_status st = gemm_f32(c, c.a(), s.F, wsel(c, i, 1, w.w_down), s.d, s.F, c.M, &ns,
                            DORY_K_GEMM_DOWN, &y16);
  if (st != DORY_OK) return st;
  PROF(c, DORY_K_UPDATE);
  HIPCHK(launch_update(c.h32(), c.h16(), c.P(), ns, c.M * s.d, s.d, w.alpha, (int)c.M, s.d, uo.x,
                       uo.aux, nullptr, c.st, c.rl, y16));
  return DORY_OK;
}

// fp32 debug build: the same sublayer steps on fp32 tensors. The step's own
// K/V sit in the fresh buffers from row 0 (f_origin = p0) in prefill; decode
// stores them in the cache slot and reads every key from there.
dory_status attention_sublayer_f32(Ctx& c, int i, int slot, bool write, const UpdateOpts& uo) {
  const Shape& s = c.s;
  const dory_sublayer_weights& w = c.m->sub[i];
  const bool full = c.m->kinds[i] == DORY_LAYER_ATTN_FULL;
  const SlotPtr sp = slot_ptr(c.kv, i, slot);
  float* kc = reinterpret_cast<float*>(sp.k);
  float* vc = reinterpret_cast<float*>(sp.v);
  float* qh = reinterpret_cast<float*>(c.qh());
  float* kf = reinterpret_cast<float*>(c.kf());
  float* vf = reinterpret_cast<float*>(c.vf());
  float* gate = reinterpret_cast<float*>(c.gate());
  float* z = reinterpret_cast<float*>(c.z());
  const bool dec = c.T == 1;
  {
    PROF(c, DORY_K_GEMM_QKVG);
    HIPCHK(launch_sgemm(c.h32(), s.d, reinterpret_cast<const float*>(w.w_qkvg), s.d, (int)c.M,
                        s.nqkvg(), s.d, c.P(), s.nqkvg(), nullptr, c.st));
  }
  {
    PROF(c, DORY_K_QK);
    if (dec)
      HIPCHK(launch_qk_prep_f32(c.P(), c.B, 1, c.p0, s.nq, s.nkv, s.dh, c.rope_cs(full ? 1 : 0),
                                c.rope_sn(full ? 1 : 0), w.s_qk, qh, kc, vc, sp.rows, sp.rows, 0,
                                sp.ring, gate, c.st, c.rl));
    else
      HIPCHK(launch_qk_prep_f32(c.P(), c.B, c.T, c.p0, s.nq, s.nkv, s.dh, c.rope_cs(full ? 1 : 0),
                                c.rope_sn(full ? 1 : 0), w.s_qk, qh, kf, vf, c.L.f_rows, c.L.f_rows,
                                c.p0, 0, gate, c.st, RowLoops()));
  }
  {
    PROF(c, DORY_K_ATTN);
    HIPCHK(launch_attn_f32(qh, kc, vc, sp.rows, sp.ring, kf, vf, c.L.f_rows, dec ? c.p0 + 1 : c.p0,
                           gate, z, c.B, c.T, s.nq, s.nkv, s.dh, c.p0, full ? 0 : s.W,
                           (float)s.scale, c.rl, c.st));
  }
  if (!dec && write) {
    PROF(c, DORY_K_KV_WRITE);
    int64_t pa = c.p0;
    if (sp.ring > 0) pa = std::max<int64_t>(pa, c.p0 + c.T - sp.ring);
    HIPCHK(launch_kv_write_f32(kf, vf, c.L.f_rows, c.p0, c.B, s.nkv, s.dh, pa, c.p0 + c.T, kc, vc,
                               sp.rows, sp.ring, c.st, c.rl));
  }
  {
    PROF(c, DORY_K_GEMM_O);
    HIPCHK(launch_sgemm(z, s.dq(), reinterpret_cast<const float*>(w.w_o), s.dq(), (int)c.M, s.d,
                        s.dq(), c.P(), s.d, nullptr, c.st));
  }
  PROF(c, DORY_K_UPDATE);
  HIPCHK(launch_update(c.h32(), nullptr, c.P(), 1, c.M * s.d, s.d, w.alpha, (int)c.M, s.d, uo.x,
                       uo.aux, nullptr, c.st, c.rl, false));
  return DORY_OK;
}

dory_status mlp_sublayer_f32(Ctx& c, int i, const UpdateOpts& uo) {
  const Shape& s = c.s;
  const dory_sublayer_weights& w = c.m->sub[i];
  float* a = reinterpret_cast<float*>(c.a());
  {
    PROF(c, DORY_K_GEMM_UPGATE);
    HIPCHK(launch_sgemm(c.h32(), s.d, reinterpret_cast<const float*>(w.w_upgate), s.d, (int)c.M,
                        2 * s.F, s.d, c.P(), 2 * s.F, nullptr, c.st));
  }
  {
    PROF(c, DORY_K_OTHER);
    HIPCHK(launch_swiglu_f32(c.P(), (int)c.M, s.F, w.s_u, w.s_v, a, c.st));
  }
  {
    PROF(c, DORY_K_GEMM_DOWN);
    HIPCHK(launch_sgemm(a, s.F, reinterpret_cast<const float*>(w.w_down), s.F, (int)c.M, s.d, s.F,
                        c.P(), s.d, nullptr, c.st));
  }
  PROF(c, DORY_K_UPDATE);
  HIPCHK(launch_update(c.h32(), nullptr, c.P(), 1, c.M * s.d, s.d, w.alpha, (int)c.M, s.d, uo.x,
                       uo.aux, nullptr, c.st, c.rl, false));
  return DORY_OK;
}

dory_status run_sublayer(Ctx& c, int i, int slot, bool write, const UpdateOpts& uo) {
  if (c.s.f32) {
    if (c.m->kinds[i] == DORY_LAYER_MLP) return mlp_sublayer_f32(c, i, uo);
    return attention_sublayer_f32(c, i, slot, write, uo);
  }
  if (c.m->kinds[i] == DORY_LAYER_MLP) return mlp_sublayer(c, i, uo);
  return attention_sublayer(c, i, slot, write, uo);
}

// next_all (device int32 [T][B], or null): greedy token after every position;
// logits_all (device fp32 [T][B][V], or null): the logits after every position
// of the step, one LM-head call of B rows per position.
dory_status run_step(Ctx& c, const int32_t* tokens, int k, float* logits, int32_t* next,
                     float* hidden, float* states, int32_t* next_all = nullptr,
                     float* logits_all = nullptr) {
  const Shape& s = c.s;
  const int64_t Md = c.M * s.d;
  const bool per_loop = c.kv->mode == DORY_CACHE_PER_LOOP;
  {
    // cos / sin of the step's positions for both RoPE bases
    PROF(c, DORY_K_QK);
    HIPCHK(launch_rope_table(c.p0, c.T, s.dh, s.base_swa, c.rope_cs(0), c.rope_sn(0), c.st, c.p0_dev));
    HIPCHK(launch_rope_table(c.p0, c.T, s.dh, s.base_full, c.rope_cs(1), c.rope_sn(1), c.st, c.p0_dev));
  }
  {
    PROF(c, DORY_K_OTHER);
    if (s.f32)
      HIPCHK(launch_embed_f32(tokens, reinterpret_cast<const float*>(c.m->embed), s.V, (int)c.M, s.d,
                              c.h32(), s.nin == 0 ? c.x32() : nullptr, c.st));
    else
      HIPCHK(launch_embed(tokens, c.m->embed, s.V, (int)c.M, s.d, c.h32(), c.h16(),
                          s.nin == 0 ? c.x32() : nullptr, c.st));
  }
  for (int i = 0; i < s.nin; ++i) {
    UpdateOpts uo;
    if (i == s.nin - 1) uo.aux = c.x32();  // x: output of the input block
    dory_status st = run_sublayer(c, i, 0, true, uo);
    if (st != DORY_OK) return st;
  }
  // loop 1 starts from N(x + x) = N(x): x is already unit-norm when it comes
  // out of an update; a bare embedding is normalized here
  if (s.nin == 0) {
    PROF(c, DORY_K_UPDATE);
    HIPCHK(launch_boundary(c.h32(), s.f32 ? nullptr : c.h16(), c.x32(), (int)c.M, s.d, c.st));
  }
  for (int it = 0; it < k; ++it) {
    const int slot = per_loop ? it : 0;
    // a mixed step stores each sequence's K/V at its own last loop
    const bool write = per_loop || it == k - 1 || c.mixed;
    if (c.mixed) {
      c.rl.k_rows = c.krows();
      c.rl.loop = it;
      c.rl.T = c.T;
    }
    float* st_out = states ? states + (int64_t)it * Md : nullptr;
    if (s.nrec == 0) {
      if (it > 0) HIPCHK(launch_boundary(c.h32(), s.f32 ? nullptr : c.h16(), c.x32(), (int)c.M, s.d, c.st));
      if (st_out) HIPCHK(hipMemcpyAsync(st_out, c.h32(), Md * 4, hipMemcpyDeviceToDevice, c.st));
      continue;
    }
    for (int i = s.nin; i < s.nin + s.nrec; ++i) {
      UpdateOpts uo;
      if (i == s.nin + s.nrec - 1) {
        uo.aux = st_out;                        // s_{it+1}
        if (it < k - 1) uo.x = c.x32();         // boundary into the next loop
      }
      dory_status st = run_sublayer(c, i, slot, write, uo);
      if (st != DORY_OK) return st;
    }
  }
  c.rl = RowLoops();
  for (int i = s.nin + s.nrec; i < s.nsub(); ++i) {
    dory_status st = run_sublayer(c, i, 0, true, UpdateOpts());
    if (st != DORY_OK) return st;
  }
  if (hidden) HIPCHK(hipMemcpyAsync(hidden, c.h32(), Md * 4, hipMemcpyDeviceToDevice, c.st));
  if ((logits || next) && s.f32) {
    float* out = logits ? logits : c.logits_scratch();
    {
      PROF(c, DORY_K_GEMM_LM);
      HIPCHK(launch_sgemm(c.h32() + (int64_t)(c.T - 1) * s.d, (int64_t)c.T * s.d,
                          reinterpret_cast<const float*>(c.m->lm_head), s.d, c.B, s.V, s.d, out, s.V,
                          c.m->s_z, c.st));
    }
    if (next) {
      PROF(c, DORY_K_OTHER);
      HIPCHK(launch_argmax(out, c.B, s.V, next, c.st));
    }
  } else if (logits || next) {
    float* out = logits ? logits : c.logits_scratch();
    GemmArgs g;
    g.A = c.h16() + (int64_t)(c.T - 1) * s.d; g.lda = (int64_t)c.T * s.d;
    g.B = c.m->lm_head; g.ldb = s.d;
    g.M = c.B; g.N = s.V; g.K = s.d; g.nsplit = 1;
    g.C = out; g.ldc = s.V; g.s1 = c.m->s_z;
    {
      PROF(c, DORY_K_GEMM_LM);
      HIPCHK(launch_gemm(g, EPI_LOGITS, c.st));
    }
    if (next) {
      PROF(c, DORY_K_OTHER);
      HIPCHK(launch_argmax(out, c.B, s.V, next, c.st));
    }
  }
  if (next_all || logits_all) {
    // the LM head after every position of the step (B rows each)
    for (int t = 0; t < c.T; ++t) {
      float* out = logits_all ? logits_all + (int64_t)t * c.B * s.V : c.logits_scratch();
      {
        PROF(c, DORY_K_GEMM_LM);
        if (s.f32) {
          HIPCHK(launch_sgemm(c.h32() + (int64_t)t * s.d, (int64_t)c.T * s.d,
                              reinterpret_cast<const float*>(c.m->lm_head), s.d, c.B, s.V, s.d, out,
                              s.V, c.m->s_z, c.st));
        } else {
          GemmArgs g;
          g.A = c.h16() + (int64_t)t * s.d; g.lda = (int64_t)c.T * s.d;
          g.B = c.m->lm_head; g.ldb = s.d;
          g.M = c.B; g.N = s.V; g.K = s.d; g.nsplit = 1;
          g.C = out; g.ldc = s.V; g.s1 = c.m->s_z;
          HIPCHK(launch_gemm(g, EPI_LOGITS, c.st));
        }
      }
      if (next_all) {
        PROF(c, DORY_K_OTHER);
        HIPCHK(launch_argmax(out, c.B, s.V, next_all + (int64_t)t * c.B, c.st));
      }
    }
  }
  return DORY_OK;
}

// Decode step through a captured graph. *ran tells whether the graph ran;
// when capture is not possible the caller runs the step directly.
dory_status decode_graph_step(Ctx& c, const int32_t* tokens, int k, float* logits, int32_t* next,
                              float* hidden, float* states, bool* ran) {
  *ran = false;
  dory_model* m = c.m;
  // the split size of the full-attention decode changes above 65,536 keys;
  // a graph serves the positions of one split size
  const bool long_ctx = c.p0 + 1 > 65536;
  const int64_t p_hi = std::min<int64_t>(c.kv->max_seq - 1, long_ctx ? 1048575 : 65535);
  std::lock_guard<std::mutex> lock(m->graph_mu);
  DecodeGraph* gph = nullptr;
  for (auto& g : m->graphs)
    if (g.kv == c.kv && g.B == c.B && g.k == k && g.mode == (int)c.kv->mode && g.long_ctx == long_ctx &&
        g.mx == m->use_mx && g.tokens == tokens && g.logits == logits && g.next == next &&
        g.hidden == hidden && g.states == states && g.ws == c.ws) {
      gph = &g;
      break;
    }
  if (!gph) {
    if (m->graphs.size() >= kMaxDecodeGraphs) {
      // the oldest graph goes; its replays are finished first
      HIPCHK(hipStreamSynchronize(c.st));
      DecodeGraph& old = m->graphs.front();
      if (old.exec) hipGraphExecDestroy(old.exec);
      if (old.graph) hipGraphDestroy(old.graph);
      m->graphs.erase(m->graphs.begin());
    }
    if (!m->cap_stream && hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess) {
      m->cap_stream = nullptr;
      return DORY_OK;
    }
    Ctx cc = c;
    cc.st = m->cap_stream;
    cc.p0_dev = c.state();
    cc.p_hi = p_hi;
    if (hipStreamBeginCapture(cc.st, hipStreamCaptureModeThreadLocal) != hipSuccess) return DORY_OK;
    dory_status st = DORY_OK;
    if (launch_set_i64(c.state(), c.p0, cc.st) != hipSuccess) st = DORY_ERR_HIP;
    if (st == DORY_OK) st = run_step(cc, tokens, k, logits, next, hidden, states);
    hipGraph_t graph = nullptr;
    const hipError_t e_end = hipStreamEndCapture(cc.st, &graph);
    DecodeGraph g{c.kv, c.B, k, (int)c.kv->mode, long_ctx, m->use_mx,
                  tokens, logits, next, hidden, states, c.ws};
    g.graph = graph;
    bool ok = st == DORY_OK && e_end == hipSuccess && graph;
    size_t nroots = 0;
    if (ok) ok = hipGraphGetRootNodes(graph, nullptr, &nroots) == hipSuccess && nroots == 1;
    if (ok) ok = hipGraphGetRootNodes(graph, &g.pos_node, &nroots) == hipSuccess;
    hipGraphNodeType type;
    if (ok) ok = hipGraphNodeGetType(g.pos_node, &type) == hipSuccess && type == hipGraphNodeTypeKernel;
    if (ok) ok = hipGraphKernelNodeGetParams(g.pos_node, &g.pos_params) == hipSuccess;
    if (ok) ok = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0) == hipSuccess;
    hipGetLastError();  // a failed capture leaves no sticky error behind
    if (!ok) {
      if (g.exec) hipGraphExecDestroy(g.exec);
      if (graph) hipGraphDestroy(graph);
      return DORY_OK;  // run the step directly
    }
    m->graphs.push_back(g);
    gph = &m->graphs.back();
  }
  int64_t* dst = c.state();
  int64_t pos = c.p0;
  void* args[2] = {&dst, &pos};
  hipKernelNodeParams kp = gph->pos_params;
  kp.kernelParams = args;
  kp.extra = nullptr;
  HIPCHK(hipGraphExecKernelNodeSetParams(gph->exec, gph->pos_node, &kp));
  HIPCHK(hipGraphLaunch(gph->exec, c.st));
  *ran = true;
  return DORY_OK;
}

// exact_ws: the workspace is laid out for exactly this step (plan_ws with the
// step's position); otherwise for any step of B x T tokens.
dory_status step_common(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                        int32_t k, const int32_t* k_rows, dory_cache_mode mode, void* ws,
                        size_t ws_bytes, float* logits, int32_t* next, float* hidden,
                        float* states, void* stream, int32_t* next_all = nullptr,
                        bool exact_ws = false, float* logits_all = nullptr,
                        bool allow_graph = true) {
  if (!m || !kv || !tokens) return fail(DORY_ERR_ARG, "model, cache and tokens must be non-NULL");
  if (kv->m != m) return fail(DORY_ERR_ARG, "cache bound to another model");
  if (B <= 0 || T <= 0) return fail(DORY_ERR_ARG, "B and T must be >= 1");
  if (k_rows) {
    // per-sequence loop counts: the step runs max k_b loops
    k = 0;
    for (int b = 0; b < B; ++b) {
      if (k_rows[b] < 1) return fail(DORY_ERR_ARG, "every per-sequence loop count must be >= 1");
      k = std::max(k, k_rows[b]);
    }
    if (mode != DORY_CACHE_LAST_LOOP)
      return fail(DORY_ERR_MODE, "per-sequence loop counts need the last-loop cache");
    if (m->s.nrec == 0) return fail(DORY_ERR_UNSUPPORTED, "per-sequence loop counts need a recurrent block");
  }
  if (k < 1) return fail(DORY_ERR_ARG, "loop count k must be >= 1");
  if (kv->invalid) return fail(DORY_ERR_STATE, "cache invalid after a HIP failure; call dory_kv_reset");
  if (mode != kv->mode) return fail(DORY_ERR_MODE, "cache mode differs from the bound mode");
  if (mode == DORY_CACHE_PER_LOOP) {
    if (k > kv->k_max) return fail(DORY_ERR_MODE, "per-loop cache: k exceeds k_max");
    // a loop-j query reads the loop-j entries of every earlier position
    if (kv->filled[k] < kv->len)
      return fail(DORY_ERR_MODE, "per-loop cache: earlier positions lack loop-k entries");
  }
  if (B > kv->batch) return fail(DORY_ERR_CAPACITY, "B exceeds the bound batch");
  if (B < kv->batch) return fail(DORY_ERR_ARG, "B must equal the bound batch");
  if (kv->len + T > kv->max_seq) return fail(DORY_ERR_CAPACITY, "cache capacity exceeded");
  if (T == 1) {
    const int64_t lo_w = std::max<int64_t>(0, kv->len - m->s.W + 1);
    if (decode_attn_pick_split(0, kv->len, false) > kMaxDecodeSplits ||
        decode_attn_pick_split(lo_w, kv->len, true) > kMaxDecodeSplits)
      return fail(DORY_ERR_UNSUPPORTED, "context too long for decode attention splits");
  }
  if (!ws) return fail(DORY_ERR_ARG, "workspace is NULL");
  const Shape& s = m->s;
  WsLayout L = exact_ws ? plan_ws(s, B, T, kv->len) : plan_ws(s, B, T);
  if (ws_bytes < L.total)
    return fail(DORY_ERR_WORKSPACE, exact_ws ? "the step needs more scratch than the static "
                                               "array holds (DORY_NOALLOC_SCRATCH_BYTES)"
                                             : "workspace smaller than dory_workspace_bytes()");
  if ((logits || next) && !s.lm) return fail(DORY_ERR_ARG, "model has no LM head");
  Ctx c{m, kv, s, B, T, (int64_t)B * T, kv->len, reinterpret_cast<uint8_t*>(ws), L,
        reinterpret_cast<hipStream_t>(stream)};
  if (k_rows) {
    c.mixed = true;
    if (hipMemcpyAsync(c.krows(), k_rows, (size_t)B * 4, hipMemcpyHostToDevice, c.st) != hipSuccess)
      return fail(DORY_ERR_HIP, "copy of the per-sequence loop counts failed");
  }
  dory_status st = DORY_OK;
  bool ran = false;
  if (T == 1 && !k_rows && !next_all && !logits_all && !exact_ws && allow_graph && m->graphs_on &&
      !m->prof.on && !m->s.f32) {
    // replay a captured decode step unless the caller's stream is itself
    // being captured (then its capture records the kernels)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(c.st, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
      st = decode_graph_step(c, tokens, k, logits, next, hidden, states, &ran);
    hipGetLastError();
  }
  if (st == DORY_OK && !ran)
    st = run_step(c, tokens, k, logits, next, hidden, states, next_all, logits_all);
  if (st != DORY_OK) {
    if (st == DORY_ERR_HIP) kv->invalid = true;
    return st;
  }
  kv->len += T;
  kv->hi = std::max(kv->hi, kv->len);
  if (mode == DORY_CACHE_PER_LOOP)
    for (int j = 1; j <= k; ++j) kv->filled[j] = kv->len;
  return DORY_OK;
}

}  // namespace

extern "C" {

dory_status dory_schedule(const dory_config* cfg, int32_t* kinds_out, int32_t capacity) {
  Shape s;
  dory_status st = read_shape(cfg, &s);
  if (st != DORY_OK) return st;
  if (!kinds_out || capacity < s.nsub()) return fail(DORY_ERR_ARG, "kinds_out too small");
  std::vector<int> kinds;
  st = build_schedule(cfg, s, &kinds);
  if (st != DORY_OK) return st;
  for (int i = 0; i < s.nsub(); ++i) kinds_out[i] = kinds[i];
  return DORY_OK;
}

dory_status dory_model_create(const dory_config* cfg, const dory_weights* w, dory_model** out) {
  if (!out) return fail(DORY_ERR_ARG, "out is NULL");
  *out = nullptr;
  Shape s;
  dory_status st = read_shape(cfg, &s);
  if (st != DORY_OK) return st;
  if (!w || !w->embed || !w->sublayers) return fail(DORY_ERR_ARG, "weights incomplete");
  if (s.lm && (!w->lm_head || !w->s_z)) return fail(DORY_ERR_ARG, "LM head weights missing");
  std::vector<int> kinds;
  st = build_schedule(cfg, s, &kinds);
  if (st != DORY_OK) return st;
  for (int i = 0; i < s.nsub(); ++i) {
    const dory_sublayer_weights& sw = w->sublayers[i];
    if (!sw.alpha) return fail(DORY_ERR_ARG, "sublayer " + std::to_string(i) + ": alpha missing");
    if (kinds[i] == DORY_LAYER_MLP) {
      if (!sw.w_upgate || !sw.w_down || !sw.s_u || !sw.s_v)
        return fail(DORY_ERR_ARG, "sublayer " + std::to_string(i) + ": MLP weights missing");
    } else if (!sw.w_qkvg || !sw.w_o || !sw.s_qk) {
      return fail(DORY_ERR_ARG, "sublayer " + std::to_string(i) + ": attention weights missing");
    }
  }
  dory_model* m = new dory_model();
  m->s = s;
  m->kinds = kinds;
  m->sub.assign(w->sublayers, w->sublayers + s.nsub());
  m->embed = reinterpret_cast<const uint16_t*>(w->embed);
  m->lm_head = reinterpret_cast<const uint16_t*>(w->lm_head);
  m->s_z = w->s_z;
  *out = m;
  return DORY_OK;
}

void dory_model_destroy(dory_model* m) { delete m; }

namespace {

// Rows and columns of the two projection matrices of sublayer kind `kind`.
void mx_dims(const Shape& s, int kind, int which, int64_t* rows, int* cols) {
  if (kind == DORY_LAYER_MLP) {
    *rows = which == 0 ? 2 * (int64_t)s.F : s.d;
    *cols = which == 0 ? s.d : s.F;
  } else {
    *rows = which == 0 ? s.nqkvg() : s.d;
    *cols = which == 0 ? s.d : s.dq();
  }
}

// Byte offsets of the codes, scales and dequantized copy of one matrix
// within its region, and the region size.
void mx_region(int64_t rows, int cols, size_t* off_sc, size_t* off_deq, size_t* total) {
  const size_t n = (size_t)rows * cols;
  *off_sc = align256(n);
  *off_deq = *off_sc + align256(n / 32);
  *total = *off_deq + align256(2 * n);
}

}  // namespace

size_t dory_mxfp8_bytes(const dory_config* cfg) {
  Shape s;
  if (read_shape(cfg, &s) != DORY_OK || s.f32) return 0;
  std::vector<int> kinds;
  if (build_schedule(cfg, s, &kinds) != DORY_OK) return 0;
  size_t total = 0;
  for (int i = 0; i < s.nsub(); ++i)
    for (int which = 0; which < 2; ++which) {
      int64_t rows; int cols; size_t a, b, t;
      mx_dims(s, kinds[i], which, &rows, &cols);
      mx_region(rows, cols, &a, &b, &t);
      total += t;
    }
  return total;
}

dory_status dory_mxfp8_quantize(const void* w, int64_t rows, int32_t cols, void* codes,
                                void* scales, void* deq, void* stream) {
  if (!w || !codes || !scales) return fail(DORY_ERR_ARG, "matrix, codes and scales must be non-NULL");
  if (rows < 1 || cols < 32 || cols % 32 != 0) return fail(DORY_ERR_ARG, "cols must be a positive multiple of 32");
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(codes) |
       reinterpret_cast<uintptr_t>(deq)) % 16 != 0)
    return fail(DORY_ERR_ARG, "matrix, codes and dequantized copy must be 16-byte aligned");
  hipError_t e = launch_mx_quantize(reinterpret_cast<const uint16_t*>(w), rows, cols,
                                    reinterpret_cast<uint8_t*>(codes), reinterpret_cast<uint8_t*>(scales),
                                    reinterpret_cast<uint16_t*>(deq), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DORY_ERR_HIP, hipGetErrorString(e));
  return DORY_OK;
}

dory_status dory_model_quantize_mxfp8(dory_model* m, void* buf, size_t bytes, void* stream) {
  if (!m || !buf) return fail(DORY_ERR_ARG, "model and buffer must be non-NULL");
  if (m->s.f32) return fail(DORY_ERR_UNSUPPORTED, "MXFP8 weights need the bf16 build");
  if (reinterpret_cast<uintptr_t>(buf) % 256 != 0) return fail(DORY_ERR_ARG, "buffer must be 256-byte aligned");
  const Shape& s = m->s;
  // everything is checked before the first launch
  size_t need = 0;
  for (int i = 0; i < s.nsub(); ++i)
    for (int which = 0; which < 2; ++which) {
      int64_t rows; int cols; size_t o_sc, o_deq, t;
      mx_dims(s, m->kinds[i], which, &rows, &cols);
      mx_region(rows, cols, &o_sc, &o_deq, &t);
      if (cols % 64 != 0) return fail(DORY_ERR_UNSUPPORTED, "MXFP8 needs reduction widths that are multiples of 64");
      const dory_sublayer_weights& w = m->sub[i];
      const void* src = m->kinds[i] == DORY_LAYER_MLP ? (which == 0 ? w.w_upgate : w.w_down)
                                                       : (which == 0 ? w.w_qkvg : w.w_o);
      if (reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return fail(DORY_ERR_ARG, "weight matrices must be 16-byte aligned");
      need += t;
    }
  if (need > bytes) return fail(DORY_ERR_CAPACITY, "buffer smaller than dory_mxfp8_bytes()");
  std::vector<std::array<MxMat, 2>> mx(s.nsub());
  size_t off = 0;
  for (int i = 0; i < s.nsub(); ++i)
    for (int which = 0; which < 2; ++which) {
      int64_t rows; int cols; size_t o_sc, o_deq, t;
      mx_dims(s, m->kinds[i], which, &rows, &cols);
      mx_region(rows, cols, &o_sc, &o_deq, &t);
      const dory_sublayer_weights& w = m->sub[i];
      const void* src = m->kinds[i] == DORY_LAYER_MLP ? (which == 0 ? w.w_upgate : w.w_down)
                                                       : (which == 0 ? w.w_qkvg : w.w_o);
      uint8_t* base = reinterpret_cast<uint8_t*>(buf) + off;
      dory_status st = dory_mxfp8_quantize(src, rows, cols, base, base + o_sc, base + o_deq, stream);
      if (st != DORY_OK) return st;
      mx[i][which] = MxMat{base, base + o_sc, reinterpret_cast<const uint16_t*>(base + o_deq)};
      off += t;
    }
  m->drop_graphs(nullptr);  // graphs captured with an earlier copy name its buffers
  m->mx = mx;
  m->mx_ready = true;
  m->use_mx = true;
  return DORY_OK;
}

dory_status dory_model_set_decode_graphs(dory_model* m, int32_t on) {
  if (!m) return fail(DORY_ERR_ARG, "model is NULL");
  m->graphs_on = on != 0;
  if (!m->graphs_on) m->drop_graphs(nullptr);
  return DORY_OK;
}

dory_status dory_model_use_mxfp8(dory_model* m, int32_t on) {
  if (!m) return fail(DORY_ERR_ARG, "model is NULL");
  if (on && !m->mx_ready) return fail(DORY_ERR_ARG, "no MXFP8 copy: call dory_model_quantize_mxfp8 first");
  m->use_mx = on != 0;
  return DORY_OK;
}

size_t dory_kv_bytes(const dory_config* cfg, dory_cache_mode mode, int32_t k_max, int32_t batch,
                     int64_t max_seq) {
  Shape s;
  if (read_shape(cfg, &s) != DORY_OK) return 0;
  if (k_max < 1 || batch < 1 || max_seq < 1 || max_seq > max_seq_limit(s)) return 0;
  if (mode != DORY_CACHE_LAST_LOOP && mode != DORY_CACHE_PER_LOOP) return 0;
  std::vector<int> kinds;
  if (build_schedule(cfg, s, &kinds) != DORY_OK) return 0;
  size_t total = 0;
  for (int i = 0; i < s.nsub(); ++i) {
    if (kinds[i] == DORY_LAYER_MLP) continue;
    const int slots = (mode == DORY_CACHE_PER_LOOP && is_recurrent(s, i)) ? k_max : 1;
    total += slots * slot_bytes(s, kinds[i], batch, max_seq);
  }
  return total;
}

size_t dory_workspace_bytes(const dory_config* cfg, int32_t batch, int32_t tokens) {
  Shape s;
  if (read_shape(cfg, &s) != DORY_OK) return 0;
  if (batch < 1 || tokens < 1) return 0;
  return plan_ws(s, batch, tokens).total;
}

dory_status dory_kv_bind(const dory_model* m, void* kv_dev, size_t kv_bytes, dory_cache_mode mode,
                         int32_t k_max, int32_t batch, int64_t max_seq, dory_kv** out) {
  if (!out) return fail(DORY_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!m || !kv_dev) return fail(DORY_ERR_ARG, "model and buffer must be non-NULL");
  if (mode != DORY_CACHE_LAST_LOOP && mode != DORY_CACHE_PER_LOOP)
    return fail(DORY_ERR_MODE, "unknown cache mode");
  if (k_max < 1 || batch < 1 || max_seq < 1) return fail(DORY_ERR_ARG, "k_max, batch, max_seq must be >= 1");
  const Shape& s = m->s;
  if (max_seq > max_seq_limit(s))
    return fail(DORY_ERR_ARG, "max_seq above the longest cache (2^24 positions, and a slab of "
                              "rows x head_dim x 2 bytes below 2^32)");
  dory_kv* kv = new dory_kv();
  kv->m = m; kv->base = reinterpret_cast<uint8_t*>(kv_dev); kv->bytes = kv_bytes;
  kv->mode = mode; kv->k_max = k_max; kv->batch = batch; kv->max_seq = max_seq;
  kv->len = 0; kv->hi = 0; kv->invalid = false;
  kv->filled.assign(k_max + 1, 0);
  kv->off.assign(s.nsub(), (size_t)-1);
  kv->nslots.assign(s.nsub(), 0);
  kv->rows.assign(s.nsub(), 0);
  kv->ring.assign(s.nsub(), 0);
  size_t off = 0;
  for (int i = 0; i < s.nsub(); ++i) {
    const int kind = m->kinds[i];
    if (kind == DORY_LAYER_MLP) continue;
    const int slots = (mode == DORY_CACHE_PER_LOOP && is_recurrent(s, i)) ? k_max : 1;
    kv->off[i] = off;
    kv->nslots[i] = slots;
    kv->rows[i] = slot_rows(s, kind, max_seq);
    kv->ring[i] = kind == DORY_LAYER_ATTN_SWA ? kv->rows[i] : 0;
    if (kv->ring[i] > 0 && kv->ring[i] < max_seq) kv->wraps = true;
    off += slots * slot_bytes(s, kind, batch, max_seq);
  }
  if (kv_bytes < off) {
    delete kv;
    return fail(DORY_ERR_CAPACITY, "KV buffer smaller than dory_kv_bytes()");
  }
  *out = kv;
  return DORY_OK;
}

void dory_kv_destroy(dory_kv* kv) {
  if (!kv) return;
  const_cast<dory_model*>(kv->m)->drop_graphs(kv);  // graphs name its slots
  delete kv;
}

dory_status dory_kv_reset(dory_kv* kv) {
  if (!kv) return fail(DORY_ERR_ARG, "cache is NULL");
  kv->len = 0;
  kv->hi = 0;
  std::fill(kv->filled.begin(), kv->filled.end(), 0);
  kv->invalid = false;
  return DORY_OK;
}

int64_t dory_kv_length(const dory_kv* kv) { return kv ? kv->len : -1; }

dory_status dory_kv_slot(const dory_kv* kv, int32_t sublayer, int32_t loop, dory_kv_slot_info* out) {
  if (!kv || !out) return fail(DORY_ERR_ARG, "NULL argument");
  const Shape& s = kv->m->s;
  if (sublayer < 0 || sublayer >= s.nsub() || kv->m->kinds[sublayer] == DORY_LAYER_MLP)
    return fail(DORY_ERR_ARG, "not an attention sublayer");
  int slot = 0;
  if (kv->nslots[sublayer] > 1) {
    if (loop < 0 || loop >= kv->nslots[sublayer]) return fail(DORY_ERR_ARG, "loop out of range");
    slot = loop;
  }
  SlotPtr p = slot_ptr(kv, sublayer, slot);
  out->k = p.k; out->v = p.v; out->rows = p.rows; out->ring = p.ring;
  return DORY_OK;
}

dory_status dory_prefill(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                         int32_t k, dory_cache_mode mode, void* ws, size_t ws_bytes,
                         float* logits, int32_t* next, float* hidden, float* states,
                         void* stream) {
  return step_common(m, kv, tokens, B, T, k, nullptr, mode, ws, ws_bytes, logits, next, hidden, states,
                     stream);
}

dory_status dory_decode_step(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                             int32_t k, dory_cache_mode mode, void* ws, size_t ws_bytes,
                             float* logits, int32_t* next, float* hidden, float* states,
                             void* stream) {
  return step_common(m, kv, tokens, B, 1, k, nullptr, mode, ws, ws_bytes, logits, next, hidden, states,
                     stream);
}

}  // extern "C"

namespace {

// Workspace of dory_decode_step_noalloc: one static array per GPU, held
// until the process ends. In host code `scratch` only names the symbol; its
// device address (one per GPU) comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratch = DORY_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array (looked up once per GPU).
dory_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DORY_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DORY_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DORY_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DORY_OK;
}

}  // namespace

extern "C" {

dory_status dory_decode_step_noalloc(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                                     int32_t k, dory_cache_mode mode, float* logits, int32_t* next,
                                     float* hidden, float* states, void* stream) {
  if (!m || !kv) return fail(DORY_ERR_ARG, "model and cache must be non-NULL");
  if (kv->m != m) return fail(DORY_ERR_ARG, "cache bound to another model");
  if (B <= 0) return fail(DORY_ERR_ARG, "B must be >= 1");
  // the size check comes first: a step that does not fit is refused before
  // any HIP call
  const size_t need = plan_ws(m->s, B, 1, kv->len).total;
  if (need > kNoAllocScratch)
    return fail(DORY_ERR_WORKSPACE, "the step needs " + std::to_string(need) +
                                        " bytes of scratch, more than the static array holds (" +
                                        std::to_string(kNoAllocScratch) + ")");
  void* ws = nullptr;
  dory_status st = scratch_for_current_device(&ws);
  if (st != DORY_OK) return st;
  return step_common(m, kv, tokens, B, 1, k, nullptr, mode, ws, kNoAllocScratch, logits, next,
                     hidden, states, stream, nullptr, true);
}

dory_status dory_prefill_rows(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                              int32_t T, const int32_t* k_rows, dory_cache_mode mode, void* ws,
                              size_t ws_bytes, float* logits, int32_t* next, float* hidden,
                              float* states, void* stream) {
  if (!k_rows) return fail(DORY_ERR_ARG, "k_rows is NULL");
  return step_common(m, kv, tokens, B, T, 0, k_rows, mode, ws, ws_bytes, logits, next, hidden,
                     states, stream);
}

dory_status dory_decode_step_rows(dory_model* m, dory_kv* kv, const int32_t* tokens, int32_t B,
                                  const int32_t* k_rows, dory_cache_mode mode, void* ws,
                                  size_t ws_bytes, float* logits, int32_t* next, float* hidden,
                                  float* states, void* stream) {
  if (!k_rows) return fail(DORY_ERR_ARG, "k_rows is NULL");
  return step_common(m, kv, tokens, B, 1, 0, k_rows, mode, ws, ws_bytes, logits, next, hidden,
                     states, stream);
}

dory_status dory_selfspec_step(dory_model* m, dory_kv* kv, const int32_t* last, int32_t B,
                               int32_t gamma, int32_t k_draft, int32_t k_verify, dory_cache_mode mode,
                               void* ws, size_t ws_bytes, int32_t* scratch, int32_t* out,
                               int32_t* n_accepted, void* stream) {
  if (!m || !kv || !last || !scratch || !out || !n_accepted)
    return fail(DORY_ERR_ARG, "model, cache, tokens, scratch, out and n_accepted must be non-NULL");
  if (kv->m != m) return fail(DORY_ERR_ARG, "cache bound to another model");
  if (gamma < 1 || gamma > DORY_KV_ROLLBACK) return fail(DORY_ERR_ARG, "need 1 <= gamma <= DORY_KV_ROLLBACK");
  if (k_draft < 1 || k_verify < k_draft) return fail(DORY_ERR_ARG, "need 1 <= k_draft <= k_verify");
  if (!m->s.lm) return fail(DORY_ERR_ARG, "model has no LM head");
  if (B != kv->batch) return fail(DORY_ERR_ARG, "B must equal the bound batch");
  if (mode != kv->mode) return fail(DORY_ERR_MODE, "cache mode differs from the bound mode");
  // under last-loop caching a verification chunk reads its own tokens'
  // current-loop entries where step-by-step decoding reads final-loop ones,
  // so the verifier would not reproduce plain decoding
  if (mode != DORY_CACHE_PER_LOOP) return fail(DORY_ERR_MODE, "self-speculative decoding needs the per-loop cache");
  if (kv->invalid) return fail(DORY_ERR_STATE, "cache invalid after a HIP failure; call dory_kv_reset");
  const int64_t L0 = kv->len;
  if (L0 + gamma + 1 > kv->max_seq) return fail(DORY_ERR_CAPACITY, "cache capacity exceeded");
  if (mode == DORY_CACHE_PER_LOOP) {
    if (k_verify > kv->k_max) return fail(DORY_ERR_MODE, "per-loop cache: k_verify exceeds k_max");
    if (kv->filled[k_verify] < L0)
      return fail(DORY_ERR_MODE, "per-loop cache: earlier positions lack loop-k_verify entries");
  }
  const size_t need = std::max(plan_ws(m->s, B, 1).total, plan_ws(m->s, B, gamma + 1).total);
  if (!ws || ws_bytes < need) return fail(DORY_ERR_WORKSPACE, "workspace smaller than dory_workspace_bytes(B, gamma + 1)");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int G = gamma + 1;
  // scratch rows 0 .. gamma: the token fed to draft step j (row 0: `last`)
  // and, in row j, the draft of step j; then the same as [B][gamma + 1]
  if (hipMemcpyAsync(scratch, last, (size_t)B * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return fail(DORY_ERR_HIP, "copy of the last tokens failed");
  for (int j = 1; j <= gamma; ++j) {
    dory_status s1 = step_common(m, kv, scratch + (int64_t)(j - 1) * B, B, 1, k_draft, nullptr, mode,
                                 ws, ws_bytes, nullptr, scratch + (int64_t)j * B, nullptr, nullptr,
                                 stream, nullptr, false, nullptr, false);
    if (s1 != DORY_OK) {
      dory_kv_set_length(kv, L0);
      return s1;
    }
  }
  dory_kv_set_length(kv, L0);  // roll back the drafts' positions
  int32_t* bt = scratch + (int64_t)G * B;
  if (launch_transpose_i32(scratch, G, B, bt, st) != hipSuccess)
    return fail(DORY_ERR_HIP, "token transpose failed");
  dory_status s2 = step_common(m, kv, bt, B, G, k_verify, nullptr, mode, ws, ws_bytes, nullptr,
                               nullptr, nullptr, nullptr, stream, out);
  if (s2 != DORY_OK) {
    dory_kv_set_length(kv, L0);
    return s2;
  }
  std::vector<int32_t> drafts((size_t)G * B), greedy((size_t)G * B);
  if (hipMemcpyAsync(drafts.data(), scratch, drafts.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(greedy.data(), out, greedy.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    dory_kv_set_length(kv, L0);
    kv->invalid = true;
    return fail(DORY_ERR_HIP, "copy of the drafted and verified tokens failed");
  }
  // draft j is accepted while it equals the verifier's greedy token after
  // position L0 + j - 1; the batch keeps the prefix accepted by every row
  int n = gamma;
  for (int b = 0; b < B; ++b) {
    int nb = 0;
    while (nb < gamma && drafts[(size_t)(nb + 1) * B + b] == greedy[(size_t)nb * B + b]) ++nb;
    n = std::min(n, nb);
  }
  dory_kv_set_length(kv, L0 + n + 1);
  *n_accepted = n;
  return DORY_OK;
}

dory_status dory_sample(const float* logits, int32_t rows, int32_t V, float temperature,
                        const float* u, int32_t* out, void* stream) {
  if (!logits || !u || !out) return fail(DORY_ERR_ARG, "logits, u and out must be non-NULL");
  if (rows < 1 || V < 1) return fail(DORY_ERR_ARG, "rows and V must be >= 1");
  if (!(temperature > 0.f)) return fail(DORY_ERR_ARG, "temperature must be > 0");
  hipError_t e = launch_sample(logits, rows, V, temperature, u, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DORY_ERR_HIP, hipGetErrorString(e));
  return DORY_OK;
}

dory_status dory_speculative_accept(const float* draft_logits, const float* verify_logits,
                                    const int32_t* drafts, const float* u, int32_t B, int32_t V,
                                    int32_t gamma, float temperature, int32_t* n_accepted,
                                    int32_t* out, void* stream) {
  if (!draft_logits || !verify_logits || !drafts || !u || !n_accepted || !out)
    return fail(DORY_ERR_ARG, "pointer arguments must be non-NULL");
  if (B < 1 || V < 1 || gamma < 1 || gamma > 1000) return fail(DORY_ERR_ARG, "need B, V >= 1 and 1 <= gamma <= 1000");
  if (!(temperature > 0.f)) return fail(DORY_ERR_ARG, "temperature must be > 0");
  hipError_t e = launch_spec_accept(draft_logits, verify_logits, drafts, u, B, V, gamma, temperature,
                                    n_accepted, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DORY_ERR_HIP, hipGetErrorString(e));
  return DORY_OK;
}

dory_status dory_selfspec_step_sampled(dory_model* m, dory_kv* kv, const int32_t* last, int32_t B,
                                       int32_t gamma, int32_t k_draft, int32_t k_verify,
                                       dory_cache_mode mode, float temperature, const float* u,
                                       void* ws, size_t ws_bytes, int32_t* scratch,
                                       float* logits_buf, int32_t* out, int32_t* n_accepted,
                                       void* stream) {
  if (!m || !kv || !last || !u || !scratch || !logits_buf || !out || !n_accepted)
    return fail(DORY_ERR_ARG, "pointer arguments must be non-NULL");
  if (kv->m != m) return fail(DORY_ERR_ARG, "cache bound to another model");
  if (gamma < 1 || gamma > DORY_KV_ROLLBACK) return fail(DORY_ERR_ARG, "need 1 <= gamma <= DORY_KV_ROLLBACK");
  if (k_draft < 1 || k_verify < k_draft) return fail(DORY_ERR_ARG, "need 1 <= k_draft <= k_verify");
  if (!(temperature > 0.f)) return fail(DORY_ERR_ARG, "temperature must be > 0");
  if (!m->s.lm) return fail(DORY_ERR_ARG, "model has no LM head");
  if (B != kv->batch) return fail(DORY_ERR_ARG, "B must equal the bound batch");
  if (mode != kv->mode) return fail(DORY_ERR_MODE, "cache mode differs from the bound mode");
  if (mode != DORY_CACHE_PER_LOOP) return fail(DORY_ERR_MODE, "self-speculative decoding needs the per-loop cache");
  if (kv->invalid) return fail(DORY_ERR_STATE, "cache invalid after a HIP failure; call dory_kv_reset");
  const int64_t L0 = kv->len;
  if (L0 + gamma + 1 > kv->max_seq) return fail(DORY_ERR_CAPACITY, "cache capacity exceeded");
  if (k_verify > kv->k_max) return fail(DORY_ERR_MODE, "per-loop cache: k_verify exceeds k_max");
  if (kv->filled[k_verify] < L0)
    return fail(DORY_ERR_MODE, "per-loop cache: earlier positions lack loop-k_verify entries");
  const size_t need = std::max(plan_ws(m->s, B, 1).total, plan_ws(m->s, B, gamma + 1).total);
  if (!ws || ws_bytes < need) return fail(DORY_ERR_WORKSPACE, "workspace smaller than dory_workspace_bytes(B, gamma + 1)");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int G = gamma + 1, V = m->s.V;
  const int64_t BV = (int64_t)B * V;
  // scratch rows 0 .. gamma: the token fed to draft step j (row 0: `last`),
  // row j the draft of step j; then the same as [B][gamma + 1], whose space
  // receives the accepted counts after the verification pass
  if (hipMemcpyAsync(scratch, last, (size_t)B * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return fail(DORY_ERR_HIP, "copy of the last tokens failed");
  for (int j = 1; j <= gamma; ++j) {
    float* dl = logits_buf + (int64_t)(j - 1) * BV;
    dory_status s1 = step_common(m, kv, scratch + (int64_t)(j - 1) * B, B, 1, k_draft, nullptr, mode,
                                 ws, ws_bytes, dl, nullptr, nullptr, nullptr, stream, nullptr, false,
                                 nullptr, false);
    if (s1 == DORY_OK && launch_sample(dl, B, V, temperature, u + (int64_t)(j - 1) * B,
                                       scratch + (int64_t)j * B, st) != hipSuccess) {
      kv->invalid = true;
      s1 = fail(DORY_ERR_HIP, "draft sampling launch failed");
    }
    if (s1 != DORY_OK) {
      dory_kv_set_length(kv, L0);
      return s1;
    }
  }
  dory_kv_set_length(kv, L0);  // roll back the drafts' positions
  int32_t* bt = scratch + (int64_t)G * B;
  if (launch_transpose_i32(scratch, G, B, bt, st) != hipSuccess)
    return fail(DORY_ERR_HIP, "token transpose failed");
  dory_status s2 = step_common(m, kv, bt, B, G, k_verify, nullptr, mode, ws, ws_bytes, nullptr,
                               nullptr, nullptr, nullptr, stream, nullptr, false,
                               logits_buf + (int64_t)gamma * BV);
  if (s2 != DORY_OK) {
    dory_kv_set_length(kv, L0);
    return s2;
  }
  int32_t* n_dev = bt;  // the verification input is consumed
  if (launch_spec_accept(logits_buf, logits_buf + (int64_t)gamma * BV, scratch + B, u + (int64_t)gamma * B,
                         B, V, gamma, temperature, n_dev, out, st) != hipSuccess) {
    dory_kv_set_length(kv, L0);
    kv->invalid = true;
    return fail(DORY_ERR_HIP, "acceptance launch failed");
  }
  std::vector<int32_t> nb(B);
  if (hipMemcpyAsync(nb.data(), n_dev, (size_t)B * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    dory_kv_set_length(kv, L0);
    kv->invalid = true;
    return fail(DORY_ERR_HIP, "copy of the accepted counts failed");
  }
  int n = gamma;
  for (int b = 0; b < B; ++b) n = std::min(n, nb[b]);
  dory_kv_set_length(kv, L0 + n + 1);
  *n_accepted = n;
  return DORY_OK;
}

dory_status dory_kv_copy_prefix(const dory_kv* src, int32_t src_seq, dory_kv* dst, int32_t dst_seq,
                                int64_t n, void* stream) {
  if (!src || !dst) return fail(DORY_ERR_ARG, "caches must be non-NULL");
  if (src->m != dst->m) return fail(DORY_ERR_ARG, "caches bound to different models");
  if (src->mode != dst->mode) return fail(DORY_ERR_MODE, "caches use different policies");
  if (src_seq < 0 || src_seq >= src->batch || dst_seq < 0 || dst_seq >= dst->batch)
    return fail(DORY_ERR_ARG, "sequence index outside the bound batch");
  if (n < 1 || n > src->len) return fail(DORY_ERR_ARG, "n must be in [1, source length]");
  if (n > dst->max_seq) return fail(DORY_ERR_CAPACITY, "n exceeds the destination's max_seq");
  if (dst->len != 0 && dst->len != n)
    return fail(DORY_ERR_STATE, "destination length must be 0 or n");
  if (src->invalid || dst->invalid) return fail(DORY_ERR_STATE, "cache invalid after a HIP failure");
  if (src->m->s.f32) return fail(DORY_ERR_UNSUPPORTED, "prefix copies run on the bf16 cache layout");
  if (src == dst && src_seq == dst_seq) return DORY_OK;
  const Shape& s = src->m->s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // loops whose first n positions the source holds (per-loop); slot j is loop j + 1
  int loops = 1;
  if (src->mode == DORY_CACHE_PER_LOOP) {
    loops = 0;
    while (loops < std::min(src->k_max, dst->k_max) && src->filled[loops + 1] >= n) ++loops;
  }
  for (int i = 0; i < s.nsub(); ++i) {
    if (src->m->kinds[i] == DORY_LAYER_MLP) continue;
    const int slots = src->nslots[i] > 1 ? loops : 1;
    // a ring keeps its last `ring` positions: copy what both rings hold
    int64_t keep = n;
    if (src->ring[i] > 0) keep = std::min(keep, src->ring[i]);
    if (dst->ring[i] > 0) keep = std::min(keep, dst->ring[i]);
    for (int j = 0; j < slots; ++j) {
      SlotPtr a = slot_ptr(src, i, j), b = slot_ptr(dst, i, j);
      if (launch_kv_copy(a.k, a.v, a.rows, a.ring, src_seq, b.k, b.v, b.rows, b.ring, dst_seq, s.nkv,
                         s.dh, n - keep, n, st) != hipSuccess) {
        dst->invalid = true;
        return fail(DORY_ERR_HIP, "KV copy launch failed");
      }
    }
  }
  if (dst->len == 0) {
    dst->len = n;
    dst->hi = n;
    for (int j = 0; j <= dst->k_max; ++j) dst->filled[j] = (j == 0 || j <= loops) ? n : 0;
  } else {
    // the other sequences' loops stay as they are; loops this one lacks are not held
    for (int j = loops + 1; j <= dst->k_max; ++j) dst->filled[j] = 0;
  }
  return DORY_OK;
}

dory_status dory_kv_set_length(dory_kv* kv, int64_t length) {
  if (!kv) return fail(DORY_ERR_ARG, "cache is NULL");
  if (length < 0 || length > kv->max_seq) return fail(DORY_ERR_CAPACITY, "length outside [0, max_seq]");
  if (length < kv->len && kv->wraps && kv->hi - length > DORY_KV_ROLLBACK)
    return fail(DORY_ERR_ARG, "a sliding-window cache can be shortened by at most DORY_KV_ROLLBACK "
                              "positions below the longest length written");
  if (length <= kv->len) {
    // roll back: positions at or past `length` are forgotten
    for (auto& f : kv->filled) f = std::min(f, length);
  } else {
    // extend: the caller declares every loop's entries of the new positions
    for (auto& f : kv->filled) f = length;
    kv->hi = std::max(kv->hi, length);
  }
  kv->len = length;
  return DORY_OK;
}

dory_status dory_profile_begin(dory_model* m, int32_t max_launches) {
  if (!m || max_launches < 1) return fail(DORY_ERR_ARG, "bad profile arguments");
  m->prof.clear();
  m->prof.ev.resize(2 * (size_t)max_launches);
  for (auto& e : m->prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      m->prof.ev.resize(&e - m->prof.ev.data());
      m->prof.clear();
      return fail(DORY_ERR_HIP, hipGetErrorString(r));
    }
  }
  m->prof.max = max_launches;
  m->prof.on = true;
  return DORY_OK;
}

dory_status dory_profile_end(dory_model* m, int64_t* counts, double* ms) {
  if (!m || !counts || !ms) return fail(DORY_ERR_ARG, "bad profile arguments");
  for (int i = 0; i < DORY_K_NUM_CLASSES; ++i) { counts[i] = 0; ms[i] = 0.0; }
  Profiler& p = m->prof;
  dory_status st = DORY_OK;
  for (size_t i = 0; i < p.cls.size(); ++i) {
    if (hipEventSynchronize(p.ev[2 * i + 1]) != hipSuccess) { st = fail(DORY_ERR_HIP, "event sync"); break; }
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) { st = fail(DORY_ERR_HIP, "event time"); break; }
    counts[p.cls[i]] += 1;
    ms[p.cls[i]] += t;
  }
  p.clear();
  return st;
}

dory_status dory_greedy(const float* logits, int32_t rows, int32_t n, int32_t* out, void* stream) {
  if (!logits || !out) return fail(DORY_ERR_ARG, "logits and out must be non-NULL");
  if (rows < 1 || n < 1) return fail(DORY_ERR_ARG, "rows and n must be >= 1");
  hipError_t e = launch_argmax(logits, rows, n, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DORY_ERR_HIP, hipGetErrorString(e));
  return DORY_OK;
}

dory_status dory_debug_kv_slots(const dory_kv* kv, int32_t sublayer, int64_t pos_a, int64_t n,
                                int64_t* rows_out, void* stream) {
  if (!kv || !rows_out) return fail(DORY_ERR_ARG, "cache and rows_out must be non-NULL");
  const Shape& s = kv->m->s;
  if (sublayer < 0 || sublayer >= s.nsub() || kv->m->kinds[sublayer] == DORY_LAYER_MLP)
    return fail(DORY_ERR_ARG, "not an attention sublayer");
  if (pos_a < 0 || n < 1 || pos_a + n > kv->max_seq)
    return fail(DORY_ERR_ARG, "positions outside [0, max_seq)");
  hipError_t e = launch_slot_rows(pos_a, n, kv->ring[sublayer], rows_out,
                                  reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DORY_ERR_HIP, hipGetErrorString(e));
  return DORY_OK;
}

namespace {

// Shared checks of the attention probes: an attention sublayer's slot of a
// valid cache, the step's positions within max_seq, a large enough
// workspace, and a decode context within the split limit.
dory_status probe_check(const dory_model* m, const dory_kv* kv, int32_t sublayer, int32_t loop,
                        int64_t p0, int32_t T, void* ws, size_t ws_bytes, SlotPtr* sp, bool* full) {
  if (!m || !kv || !ws) return fail(DORY_ERR_ARG, "model, cache and workspace must be non-NULL");
  if (kv->m != m) return fail(DORY_ERR_ARG, "cache bound to another model");
  if (kv->invalid) return fail(DORY_ERR_STATE, "cache invalid after a HIP failure; call dory_kv_reset");
  const Shape& s = m->s;
  if (s.f32) return fail(DORY_ERR_UNSUPPORTED, "the attention probes run the bf16 kernels");
  if (sublayer < 0 || sublayer >= s.nsub() || m->kinds[sublayer] == DORY_LAYER_MLP)
    return fail(DORY_ERR_ARG, "not an attention sublayer");
  int slot = 0;
  if (kv->nslots[sublayer] > 1) {
    if (loop < 0 || loop >= kv->nslots[sublayer]) return fail(DORY_ERR_ARG, "loop out of range");
    slot = loop;
  }
  if (T < 1 || p0 < 0) return fail(DORY_ERR_ARG, "need T >= 1 and p0 >= 0");
  if (p0 + T > kv->max_seq) return fail(DORY_ERR_CAPACITY, "p0 + T exceeds max_seq");
  if (ws_bytes < plan_ws(s, kv->batch, T).total)
    return fail(DORY_ERR_WORKSPACE, "workspace smaller than dory_workspace_bytes(batch, T)");
  *full = m->kinds[sublayer] == DORY_LAYER_ATTN_FULL;
  if (T == 1) {
    const int64_t lo = *full ? 0 : std::max<int64_t>(0, p0 - s.W + 1);
    if (decode_attn_pick_split(lo, p0, !*full) > kMaxDecodeSplits)
      return fail(DORY_ERR_UNSUPPORTED, "context too long for decode attention splits");
  }
  *sp = slot_ptr(kv, sublayer, slot);
  return DORY_OK;
}

// Where the step's own K/V go before the attention: the cache row of p0 for
// decode (as the decode step stores them), the fresh buffers for prefill.
QkDest probe_dest(const Ctx& c, const SlotPtr& sp) {
  if (c.T == 1) return QkDest{sp.k, sp.v, sp.rows, sp.rows, 0, sp.ring};
  return QkDest{c.kf(), c.vf(), c.L.f_rows, c.L.f_rows, c.p0 / 8 * 8, 0};
}

}  // namespace

dory_status dory_debug_attention(dory_model* m, dory_kv* kv, int32_t sublayer, int32_t loop,
                                 int64_t p0, int32_t T, const void* q_hat, const void* k_new,
                                 const void* v_new, const void* gate, void* z, void* ws,
                                 size_t ws_bytes, void* stream) {
  SlotPtr sp;
  bool full = false;
  dory_status st = probe_check(m, kv, sublayer, loop, p0, T, ws, ws_bytes, &sp, &full);
  if (st != DORY_OK) return st;
  if (!q_hat || !k_new || !v_new || !gate || !z)
    return fail(DORY_ERR_ARG, "q_hat, k_new, v_new, gate and z must be non-NULL");
  const int B = kv->batch;
  Ctx c{m, kv, m->s, B, T, (int64_t)B * T, p0, reinterpret_cast<uint8_t*>(ws),
        plan_ws(m->s, B, T), reinterpret_cast<hipStream_t>(stream)};
  const Shape& s = m->s;
  hipError_t e = launch_kv_place(reinterpret_cast<const uint16_t*>(k_new),
                                 reinterpret_cast<const uint16_t*>(v_new), B, s.nkv, T, s.dh, p0,
                                 probe_dest(c, sp), c.st);
  if (e != hipSuccess) {
    kv->invalid = true;
    return fail(DORY_ERR_HIP, hipGetErrorString(e));
  }
  st = attend(c, sp, full, reinterpret_cast<const uint16_t*>(q_hat),
              reinterpret_cast<const uint16_t*>(gate), reinterpret_cast<uint16_t*>(z));
  if (st == DORY_ERR_HIP) kv->invalid = true;
  return st;
}

dory_status dory_debug_mask(dory_model* m, dory_kv* kv, int32_t sublayer, int32_t loop, int64_t p0,
                            int32_t T, void* ws, size_t ws_bytes, uint16_t* out, void* stream) {
  SlotPtr sp;
  bool full = false;
  dory_status st = probe_check(m, kv, sublayer, loop, p0, T, ws, ws_bytes, &sp, &full);
  if (st != DORY_OK) return st;
  if (!out) return fail(DORY_ERR_ARG, "out must be non-NULL");
  const int B = kv->batch;
  const Shape& s = m->s;
  Ctx c{m, kv, s, B, T, (int64_t)B * T, p0, reinterpret_cast<uint8_t*>(ws), plan_ws(s, B, T),
        reinterpret_cast<hipStream_t>(stream)};
  // probe inputs in the workspace: q_hat = 0 and K = 0 give every key the
  // score 0, so a visible key has probability 1 / (number of visible keys)
  // and a masked one exactly 0; gate = 1, and with one-hot values the output
  // column of a key is its weight. The step's own K/V sit in the
  // projection-output region until they are placed.
  const int64_t nkv_el = (int64_t)B * s.nkv * T * s.dh;
  uint16_t* knew = reinterpret_cast<uint16_t*>(c.P());
  uint16_t* vnew = knew + nkv_el;
  const int64_t slot_el = (int64_t)B * s.nkv * sp.rows * s.dh;
  const int64_t L = p0 + T;
  const QkDest dst = probe_dest(c, sp);
  auto run = [&]() -> dory_status {
    HIPCHK(launch_fill_u16(c.qh(), c.M * s.dq(), 0, c.st));
    HIPCHK(launch_fill_u16(c.gate(), c.M * s.dq(), 0x3F80, c.st));
    HIPCHK(launch_fill_u16(knew, 2 * nkv_el, 0, c.st));
    HIPCHK(launch_fill_u16(sp.k, slot_el, 0, c.st));
    HIPCHK(launch_fill_u16(sp.v, slot_el, 0, c.st));
    // Pass r puts one-hot values on the keys [r dh, (r + 1) dh): output
    // column d of every query head is the weight of key r dh + d. Each pass
    // rewrites the keys of the previous pass (back to 0) and of its own.
    for (int64_t first = 0; first < L; first += s.dh) {
      const int64_t ua = std::max<int64_t>(0, first - s.dh), ub = std::min<int64_t>(L, first + s.dh);
      HIPCHK(launch_mask_probe_v(sp.v, sp.rows, sp.ring, vnew, B, T, s.nkv, s.dh, p0, ua, ub, first,
                                 c.st));
      HIPCHK(launch_kv_place(knew, vnew, B, s.nkv, T, s.dh, p0, dst, c.st));
      dory_status r = attend(c, sp, full, c.qh(), c.gate(), c.z());
      if (r != DORY_OK) return r;
      HIPCHK(launch_mask_extract(c.z(), B, T, s.nq, s.dh, L, first, out, c.st));
    }
    return DORY_OK;
  };
  st = run();
  if (st == DORY_ERR_HIP) kv->invalid = true;
  return st;
}

const char* dory_status_string(dory_status s) {
  switch (s) {
    case DORY_OK: return "ok";
    case DORY_ERR_ARG: return "invalid argument";
    case DORY_ERR_MODE: return "cache mode / loop count mismatch";
    case DORY_ERR_CAPACITY: return "cache capacity exceeded";
    case DORY_ERR_WORKSPACE: return "workspace too small";
    case DORY_ERR_UNSUPPORTED: return "unsupported shape";
    case DORY_ERR_HIP: return "HIP launch failure";
    case DORY_ERR_STATE: return "cache invalid";
  }
  return "unknown status";
}

const char* dory_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
