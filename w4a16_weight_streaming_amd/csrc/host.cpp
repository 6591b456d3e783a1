// Host side of libe2b: configuration, layer table and K/V share map, device
// arena plan, weight upload, K/V binding and the orchestration of one decode
// step (or a prefill pass) as a sequence of HIP kernel launches on the
// caller's stream.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "e2b.h"
#include "e2b_internal.h"

using e2b::Lin;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(E2B_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int kMaxCtlRows = 4096;  // rows per call the control words cover (batch, prefill pass)
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct LayerInfo {
  int full = 0, hd = 0, I = 0, src = 0;
  double theta = 0;
};

struct LinOff {  // a linear layer as offsets into the arena
  int quant = 0;  // E2B_QUANT_*
  size_t w = 0, q = 0, s = 0;
  bool tiled = false;   // a copy tiled for the matrix cores: tw (bf16) or tq, ts (W4A16)
  size_t tw = 0, tq = 0, ts = 0;
  int N = 0, K = 0;
};

struct Copy {  // one canonical tensor -> arena offset
  std::string name;
  int dtype = 0;
  int ndim = 0;
  int64_t d0 = 0, d1 = 0;
  size_t dst = 0;
};

struct LayerOff {
  LinOff qkv, o, gu, down, pg, pp;
  size_t g_in = 0, g_q = 0, g_k = 0, g_pa = 0, g_pf = 0, g_ff = 0, g_pple = 0, scalar = 0;
};

struct LayerDev {
  Lin qkv, o, gu, down, pg, pp;
  const uint16_t *g_in = nullptr, *g_q = nullptr, *g_k = nullptr, *g_pa = nullptr,
                 *g_pf = nullptr, *g_ff = nullptr, *g_pple = nullptr, *scalar = nullptr;
};

}  // namespace

struct e2b_model {
  e2b_config c{};
  int L = 0, H = 0, P = 0, V = 0, nq = 0, first = 0, quant = 0;
  int equant = 0;  // format of the two vocabulary tables (E2B_QUANT_*)
  int kv_quant = 0;  // format of the K/V cache (E2B_KV_*)
  std::vector<LayerInfo> li;
  // arena plan
  std::vector<Copy> plan;
  size_t arena_bytes = 0, weight_bytes = 0;
  size_t off_plpn = 0, off_final = 0, off_invf[2] = {0, 0};
  // the vocabulary tables as linears [V, H] and [V, L*P] (the tied embedding
  // also tiled for the batched lm_head)
  LinOff embed_off, ple_off;
  LinOff plmp_off;
  std::vector<LayerOff> lo;
  // device views (valid after load)
  char* arena = nullptr;
  bool loaded = false;
  const uint16_t *g_plpn = nullptr, *g_final = nullptr;
  Lin embed, ple;  // the vocabulary tables (bf16 w, or W4A16 q + s)
  const double* invf[2] = {nullptr, nullptr};
  Lin plmp;
  std::vector<LayerDev> ld;
  // K/V binding
  char* kv = nullptr;
  int max_batch = 0, max_ctx = 0;
  int kvq = 0;                // cache format: E2B_KV_BF16 / E2B_KV_INT8
  std::vector<char*> kc, vc;  // per layer: the K / V rows it reads (its source's)
  std::vector<float*> ks, vs; // int8: the row scales
  // paged cache: n_pages pages of kPageSize positions per K/V-owning layer; the
  // device page table [max_batch][page_stride] (caller-owned) and its host
  // mirror; pages per slot and the free list (the allocator)
  int n_pages = 0, page_stride = 0;
  int32_t* d_pages = nullptr;
  std::vector<int32_t> h_pages;
  std::vector<int> slot_pages;
  std::vector<int32_t> free_pages;
  // per-kernel timing
  int prof_kind = 0;
  struct Mark {
    hipEvent_t a, b;
    double bytes;
  };
  std::vector<Mark> marks;
};

struct e2b_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

bool is_full(const e2b_config& c, int l) {
  return (l % c.layer_pattern_period) == c.layer_pattern_period - 1;
}

// Source layer of layer l's K/V: itself below the first shared layer; above
// it the last non-shared layer of the same attention type; a shared layer
// with no such layer keeps its own K/V.
int kv_src(const e2b_config& c, int l) {
  const int first = c.num_hidden_layers - c.num_kv_shared_layers;
  if (l < first) return l;
  int s = -1;
  for (int i = 0; i < first; ++i)
    if (is_full(c, i) == is_full(c, l)) s = i;
  return s < 0 ? l : s;
}

bool supported_k(int K) { return e2b::gemv_supported(K); }

struct Planner {
  e2b_model* m;
  size_t cur = 0;
  size_t alloc(size_t bytes) {
    size_t o = cur;
    cur = align_up(cur + bytes);
    return o;
  }
  void copy(const std::string& name, int dtype, int ndim, int64_t d0, int64_t d1, size_t dst,
            size_t bytes) {
    m->plan.push_back(Copy{name, dtype, ndim, d0, d1, dst});
    m->weight_bytes += bytes;
  }
  size_t vec(const std::string& name, int64_t n) {  // bf16 1-D
    size_t o = alloc(n * 2);
    copy(name, E2B_DTYPE_BF16, 1, n, 0, o, n * 2);
    return o;
  }
  size_t mat(const std::string& name, int64_t r, int64_t c) {  // bf16 2-D
    size_t o = alloc(r * c * 2);
    copy(name, E2B_DTYPE_BF16, 2, r, c, o, r * c * 2);
    return o;
  }
  // linears stacked along N into one matrix [sum N, K]; tiled: also keep a
  // copy in the matrix-core fragment order (batched passes)
  LinOff lin(const std::vector<std::string>& names, const std::vector<int>& Ns, int K,
             bool tiled = true, int quant = -1) {
    LinOff L;
    int N = 0;
    for (int n : Ns) N += n;
    L.N = N;
    L.K = K;
    L.quant = quant < 0 ? m->quant : quant;
    if (L.quant == E2B_QUANT_BF16) {
      L.w = alloc((size_t)N * K * 2);
      if (tiled && N % 16 == 0) {
        L.tiled = true;
        L.tw = alloc((size_t)N * K * 2);
      }
      size_t r = 0;
      for (size_t i = 0; i < names.size(); ++i) {
        copy(names[i], E2B_DTYPE_BF16, 2, Ns[i], K, L.w + r * K * 2, (size_t)Ns[i] * K * 2);
        r += Ns[i];
      }
    } else {
      L.q = alloc((size_t)N * K / 2);
      L.s = alloc((size_t)N * (K / 32) * 2);
      if (tiled && N % 16 == 0 && K % 128 == 0) {
        L.tiled = true;
        L.tq = alloc((size_t)N * K / 2);
        L.ts = alloc((size_t)N * (K / 32) * 2);
      }
      size_t r = 0;
      for (size_t i = 0; i < names.size(); ++i) {
        copy(names[i] + "_packed", E2B_DTYPE_INT32, 2, Ns[i], K / 8, L.q + r * K / 2,
             (size_t)Ns[i] * K / 2);
        copy(names[i] + "_scale", E2B_DTYPE_BF16, 2, Ns[i], K / 32, L.s + r * (K / 32) * 2,
             (size_t)Ns[i] * (K / 32) * 2);
        r += Ns[i];
      }
    }
    return L;
  }
};

int build_plan(e2b_model* m) {
  Planner p{m};
  const int L = m->L, H = m->H, P = m->P, V = m->V, nq = m->nq;
  m->embed_off = p.lin({"model.embed_tokens.weight"}, {V}, H, true, m->equant);
  m->ple_off = p.lin({"model.embed_tokens_per_layer.weight"}, {V}, L * P, false, m->equant);
  m->plmp_off = p.lin({"model.per_layer_model_projection.weight"}, {L * P}, H);
  m->off_plpn = p.vec("model.per_layer_projection_norm.weight", P);
  m->off_final = p.vec("model.norm.weight", H);
  m->lo.resize(L);
  for (int l = 0; l < L; ++l) {
    const LayerInfo& y = m->li[l];
    LayerOff& o = m->lo[l];
    const std::string pre = "model.layers." + std::to_string(l) + ".";
    o.g_in = p.vec(pre + "input_layernorm.weight", H);
    if (y.src == l)
      o.qkv = p.lin({pre + "self_attn.q_proj.weight", pre + "self_attn.k_proj.weight",
                     pre + "self_attn.v_proj.weight"},
                    {nq * y.hd, y.hd, y.hd}, H);
    else
      o.qkv = p.lin({pre + "self_attn.q_proj.weight"}, {nq * y.hd}, H);
    o.o = p.lin({pre + "self_attn.o_proj.weight"}, {H}, nq * y.hd);
    o.g_q = p.vec(pre + "self_attn.q_norm.weight", y.hd);
    if (y.src == l) o.g_k = p.vec(pre + "self_attn.k_norm.weight", y.hd);
    o.g_pa = p.vec(pre + "post_attention_layernorm.weight", H);
    o.g_pf = p.vec(pre + "pre_feedforward_layernorm.weight", H);
    o.gu = p.lin({pre + "mlp.gate_proj.weight", pre + "mlp.up_proj.weight"}, {y.I, y.I}, H);
    o.down = p.lin({pre + "mlp.down_proj.weight"}, {H}, y.I);
    o.g_ff = p.vec(pre + "post_feedforward_layernorm.weight", H);
    // (the per-layer input gate and projection always run on the matvec kernel)
    o.pg = p.lin({pre + "per_layer_input_gate.weight"}, {P}, H, false);
    o.pp = p.lin({pre + "per_layer_projection.weight"}, {H}, P, false);
    o.g_pple = p.vec(pre + "post_per_layer_input_norm.weight", H);
    o.scalar = p.vec(pre + "layer_scalar", 1);
  }
  // RoPE inverse frequencies theta^(-2i/hd), double, per attention type
  m->off_invf[0] = p.alloc(sizeof(double) * m->c.head_dim / 2);
  m->off_invf[1] = p.alloc(sizeof(double) * m->c.global_head_dim / 2);
  m->arena_bytes = p.cur;
  return E2B_OK;
}

// K-side tensors of layers that read another layer's K/V: accepted and ignored
bool ignorable(const e2b_model* m, const char* name) {
  int l = -1;
  char rest[128];
  if (sscanf(name, "model.layers.%d.%127s", &l, rest) != 2) return false;
  if (l < 0 || l >= m->L || m->li[l].src == l) return false;
  return strncmp(rest, "self_attn.k_proj.", 17) == 0 || strncmp(rest, "self_attn.v_proj.", 17) == 0 ||
         strcmp(rest, "self_attn.k_norm.weight") == 0;
}

Lin resolve(const e2b_model* m, const LinOff& o) {
  Lin L;
  L.N = o.N;
  L.K = o.K;
  if (o.quant == E2B_QUANT_BF16) {
    L.w = reinterpret_cast<const uint16_t*>(m->arena + o.w);
    if (o.tiled) L.tw = reinterpret_cast<const uint16_t*>(m->arena + o.tw);
  } else {
    L.q = reinterpret_cast<const uint32_t*>(m->arena + o.q);
    L.s = reinterpret_cast<const uint16_t*>(m->arena + o.s);
    if (o.tiled) {
      L.tq = reinterpret_cast<const uint32_t*>(m->arena + o.tq);
      L.ts = reinterpret_cast<const uint16_t*>(m->arena + o.ts);
    }
  }
  return L;
}

// ---- workspace layout ------------------------------------------------------
struct Ws {
  size_t err, rope, h0, h1, tokple, u, pli, qkv, part, attn, oo, gu, dn, pgy, ppo, cv, ci, xh, xl, xg,
      xh2, xl2, xg2, total;
  int ncand;  // argmax candidates per row
};

Ws ws_layout(const e2b_model* m, int R) {
  Ws w{};
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    size_t o = cur;
    cur = align_up(cur + bytes);
    return o;
  };
  const size_t f = sizeof(float);
  const int hdm = std::max(m->c.head_dim, m->c.global_head_dim);
  // K-slice partials a product can write (matvec or matrix-core plan)
  auto parts = [&](int N, int K) {
    return std::max(e2b::gemv_splits(K), e2b::gemm_plan(m->quant, N, K, true).nks);
  };
  const int H = m->H, P = m->P, LPn = m->L * m->P;
  int Kmax = std::max(H, P), Imax = 0;
  size_t qkv_f = 0, gu_f = 0, oo_f = 0, dn_f = 0, pgy_f = 0, ppo_f = 0;
  for (const LayerInfo& y : m->li) {
    const int nqkv = (m->nq + (y.src == &y - &m->li[0] ? 2 : 0)) * y.hd;
    Kmax = std::max(Kmax, std::max(y.I, m->nq * y.hd));
    Imax = std::max(Imax, y.I);
    qkv_f = std::max(qkv_f, (size_t)parts(nqkv, H) * nqkv);
    gu_f = std::max(gu_f, (size_t)parts(2 * y.I, H) * 2 * y.I);
    oo_f = std::max(oo_f, (size_t)parts(H, m->nq * y.hd) * H);
    dn_f = std::max(dn_f, (size_t)parts(H, y.I) * H);
    pgy_f = std::max(pgy_f, (size_t)parts(P, H) * P);
    ppo_f = std::max(ppo_f, (size_t)parts(H, P) * H);
  }
  // the one-row O product writes one partial per head
  oo_f = std::max(oo_f, (size_t)m->nq * H);
  const size_t u_f = (size_t)parts(LPn, H) * LPn;
  w.ncand = std::max(e2b::kLmBlocks, (m->V + 63) / 64);
  const size_t LP = (size_t)m->L * m->P;
  w.err = take(64);
  w.rope = take(f * R * (m->c.head_dim + m->c.global_head_dim));
  w.h0 = take(f * R * m->H);
  w.h1 = take(f * R * m->H);
  w.tokple = take(f * R * LP);
  w.u = take(f * R * u_f);
  w.pli = take(f * R * LP);
  w.qkv = take(f * R * qkv_f);
  w.part = take(f * R * m->nq * e2b::kMaxChunks * (hdm + 2));
  w.attn = take(f * R * m->nq * hdm);
  w.oo = take(f * R * oo_f);
  w.gu = take(f * R * gu_f);
  w.dn = take(f * R * dn_f);
  w.pgy = take(f * R * pgy_f);
  w.ppo = take(f * R * ppo_f);
  w.cv = take(f * R * w.ncand);
  w.ci = take(sizeof(int32_t) * R * w.ncand);
  if (R > 1) {  // batched rows go through the MFMA path
    w.xh = take(2 * (size_t)R * Kmax);
    w.xl = take(2 * (size_t)R * Kmax);
    w.xg = take(f * (size_t)R * (Kmax / 32));
    // the down product's input, written by the gate/up product's epilogue
    // while that product still reads its own input from xh / xl / xg
    w.xh2 = take(2 * (size_t)R * Imax);
    w.xl2 = take(2 * (size_t)R * Imax);
    w.xg2 = take(f * (size_t)R * (Imax / 32));
  } else {
    w.xh = w.xl = w.xg = w.xh2 = w.xl2 = w.xg2 = 0;
  }
  w.total = cur;
  return w;
}

// Attention blocks per (row, layer) and the fewest keys per block: 16 for a
// single row (each wave then takes one group of 4 keys: the shortest chain,
// and the chip has room for the blocks), 32 for a few rows, 64 from 32 rows
// on (measured: B = 8 at context 500 is fastest with 32, B = 64 at context
// 140 with 64; 128 is slower for both).  The grid covers the longest span max_ctx allows (at most
// kMaxChunks blocks); each row splits its live span over those blocks on the
// device, so a short context is not left to a few long blocks.
//
// A prefill pass on the matrix-core kernel takes 16 queries (RW = 16 / nq
// rows) per block, and at least kPrefillMinChunk keys (whole 32-key tiles)
// per block: the group's span is at most max_ctx (full) or the window plus
// RW - 1 positions (sliding).
void attn_chunks(const e2b_model* m, bool full, int rows, bool mfma, int* chunk, int* nchunk) {
  if (mfma) {
    const int rw = 16 / m->nq;
    const int span = full ? m->max_ctx : std::min(m->c.sliding_window + rw - 1, m->max_ctx);
    int n = (span + e2b::kPrefillMinChunk - 1) / e2b::kPrefillMinChunk;
    *nchunk = std::max(1, std::min(n, e2b::kMaxChunks));
    *chunk = e2b::kPrefillMinChunk;
    return;
  }
  const int span = full ? m->max_ctx : std::min(m->c.sliding_window, m->max_ctx);
  const int w = rows == 1 ? 16 : rows < 32 ? 32 : 64;
  int n = (span + w - 1) / w;
  if (n > e2b::kMaxChunks) n = e2b::kMaxChunks;
  if (n < 1) n = 1;
  *nchunk = n;
  *chunk = w;
}

// One product of a linear layer with `rows` input rows built by `pr`:
// a one-row pass streams through the matvec kernel, a batched pass (even
// where only one of its rows reaches this product, as the last-row lm_head of
// prefill does) through the x-prep + MFMA kernels, so that a row's result
// does not depend on the other rows of its pass.  *nd receives the number of K-slice partials written
// (only where partial_ok: the consumer sums them).  Bracketed by events when
// this kind is being profiled.
hipError_t matmul(e2b_model* m, int quant, int tag, const Lin& W, int rows, bool batched,
                  const e2b::Prologue& pr, const e2b::Epilogue& ep, bool partial_ok, int* nd,
                  int* nblk, char* ws, const struct Ws& L, hipStream_t st);

#define CK(call, what)                         \
  do {                                         \
    hipError_t e_ = (call);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

hipError_t matmul(e2b_model* m, int quant, int tag, const Lin& W, int rows, bool batched,
                  const e2b::Prologue& pr, const e2b::Epilogue& ep, bool partial_ok, int* nd,
                  int* nblk, char* ws, const Ws& L, hipStream_t st) {
  const bool prof = m->prof_kind == tag;
  e2b_model::Mark mk{};
  hipError_t e = hipSuccess;
  if (prof) {  // the product kernel itself records them (dispatch timestamps)
    e = hipEventCreate(&mk.a);
    if (e == hipSuccess) e = hipEventCreate(&mk.b);
    if (e != hipSuccess) return e;
  }
  int splits = 1;
  // The per-layer input gate and projection (256 x H and H x 256, under 1 MB)
  // run through the matvec kernel for any number of rows: each row re-reads
  // the weights from L2, which costs less than the input-prep kernel and the
  // fixed cost of a matrix-core pass; a row's result still does not depend on
  // the other rows of its pass.
  int gemv_tag = tag;
  if (tag == e2b::kTagPleGate || tag == e2b::kTagPleProj) {
    if (batched && tag == e2b::kTagPleGate) gemv_tag = e2b::kTagPleGateRows;
    batched = false;
  }
  if (!batched) {
    // the merged attention input comes one head (K slice) at a time
    splits = pr.kind == e2b::kAttnMerge ? (pr.slice > 0 ? W.K / pr.slice : -1) : e2b::gemv_splits(W.K);
    // the matvec prologue reads one copy of a; it splits only K > 2048
    if (pr.na != 1 || (splits > 1 && !partial_ok)) return hipErrorInvalidValue;
    if (prof) e2b::set_launch_events(mk.a, mk.b);
    e = e2b::launch_gemv(quant, gemv_tag, W, rows, pr, ep, 0, nblk, st);
  } else {
    e2b::GemmPlan plan = ep.gh ? e2b::gemm_plan_geglu(quant, W.N / 2, W.K, rows)
                               : e2b::gemm_plan(quant, W.N, W.K, partial_ok);
    // Rows per block and column tiles (neither changes an output's
    // arithmetic): W4A16 q/k/v, O and down in 16-row blocks (the row blocks
    // re-read the small int4 weights from L2); bf16 q/k/v and O above 32
    // rows in 32-row blocks of two tiles per wave.  Measured at 64 rows:
    // W4A16 +8%, bf16 +2% per step.
    if (!ep.gh && (tag == e2b::kTagQkv || tag == e2b::kTagO || (quant && tag == e2b::kTagDown))) {
      if (quant) {
        plan.mt = 1;
      } else if (rows > 32) {
        plan.mt = 2;
        plan.nt = 2;
      }
    }
    splits = plan.nks;
    e2b::GemmA A;
    if (pr.kind == e2b::kPlain && pr.na == 1 && plan.nt <= 2) {  // read fp32 rows directly
      A.a = pr.a;
      A.kind = pr.kind;
      A.lda = pr.lda;
    } else if (pr.kind == e2b::kPrepared) {  // written in prepared form by the producer
      A.xh = reinterpret_cast<uint16_t*>(ws + (pr.alt ? L.xh2 : L.xh));
      A.xl = reinterpret_cast<uint16_t*>(ws + (pr.alt ? L.xl2 : L.xl));
      A.xg = reinterpret_cast<float*>(ws + (pr.alt ? L.xg2 : L.xg));
    } else {
      A.xh = reinterpret_cast<uint16_t*>(ws + L.xh);
      A.xl = reinterpret_cast<uint16_t*>(ws + L.xl);
      A.xg = reinterpret_cast<float*>(ws + L.xg);
      e = e2b::launch_xprep(pr, rows, W.K, const_cast<uint16_t*>(A.xh),
                            const_cast<uint16_t*>(A.xl), const_cast<float*>(A.xg), st);
    }
    if (e == hipSuccess && prof) e2b::set_launch_events(mk.a, mk.b);
    if (e == hipSuccess) e = e2b::launch_gemm(quant, tag, W, rows, A, plan, ep, nblk, st);
  }
  if (nd) *nd = splits;
  if (e != hipSuccess) return e;
  if (prof) {
    const double wb = quant ? (double)W.N * W.K / 2 + (double)W.N * (W.K / 32) * 2
                            : (double)W.N * W.K * 2;
    mk.bytes = wb + (double)rows * (W.K + W.N) * sizeof(float);
    m->marks.push_back(mk);
  }
  return hipSuccess;
}

// One pass over R.n rows: all layers, then (if head) the final norm, lm_head
// and argmax for every row (head_row < 0) or for row head_row only.
int run_rows(e2b_model* m, const e2b::Rows& R, bool head, int head_row, float* d_logits,
             int32_t* d_argmax, char* ws, const Ws& W, hipStream_t st, int32_t* adv_pos = nullptr) {
  using namespace e2b;
  const int n = R.n, H = m->H, P = m->P, L = m->L, LP = L * P, q = m->quant;
  const float eps = m->c.rms_eps;
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  int* err = reinterpret_cast<int*>(ws + W.err);

  const bool bat = n > 1;  // batched pass: matrix-core products
  int nd_u = 1;            // K-slice partials of the per-layer model projection
  RopeTable rt;
  rt.out = F(W.rope);
  rt.inv_s = m->invf[0];
  rt.inv_f = m->invf[1];
  rt.hd_s = m->c.head_dim;
  rt.hd_f = m->c.global_head_dim;
  CK(launch_embed(R, m->embed, m->ple, std::sqrt((float)H), std::sqrt((float)P), F(W.h0),
                  F(W.tokple), err, rt, st),
     "embed");
  {
    Prologue pr;
    pr.kind = kPlain;
    pr.a = F(W.h0);
    pr.lda = H;
    Epilogue ep;
    ep.y = F(W.u);
    CK(matmul(m, q, kTagPleModel, m->plmp, n, bat, pr, ep, true, &nd_u, nullptr, ws, W, st),
       "per-layer model projection");
  }
  CK(launch_ple_finish(R, F(W.u), nd_u, (size_t)n * LP, F(W.tokple), m->g_plpn, L, P,
                       1.0f / std::sqrt((float)H), eps, F(W.pli), st),
     "per-layer inputs");

  float* cur = F(W.h0);
  float* oth = F(W.h1);
  const float* pend = nullptr;  // per-layer projection output not yet added
  int pend_n = 1;               // ... as this many K-slice partials
  const uint16_t *pend_g = nullptr, *pend_s = nullptr;
  for (int l = 0; l < L; ++l) {
    const LayerInfo& y = m->li[l];
    // batched: the GeGLU runs in the gate/up product's epilogue
    const bool geglu_fold = bat && gemm_plan_geglu(q, y.I, H, n).nt > 0;
    const LayerDev& d = m->ld[l];
    const bool owns = y.src == l;
    int nd_qkv = 1, nd_o = 1, nd_gu = 1, nd_dn = 1, nd_pg = 1;  // K-slice partials written
    int nchunk = 0;                                             // attention chunks per head
    {  // QKV with the residual update of the previous layer fused in front
      Prologue pr;
      pr.kind = kResNorm;
      pr.a = cur;
      pr.d = pend;
      pr.nd = pend_n;
      pr.d_pstride = (size_t)n * H;
      pr.gd = pend_g;
      pr.scalar = pend_s;
      pr.gx = d.g_in;
      pr.h_out = oth;
      pr.eps = eps;
      Epilogue ep;
      ep.y = F(W.qkv);
      CK(matmul(m, q, kTagQkv, d.qkv, n, bat, pr, ep, true, &nd_qkv, nullptr, ws, W, st),
         "qkv projection");
      if (pend) std::swap(cur, oth);
    }
    // decode rows are distinct sequences: the attention kernel writes the new
    // K/V itself; prefill rows attend to each other's K/V, written first
    const bool mfma_attn = R.seq_stride == 0 && attn_prefill_supported(y.hd, m->nq);
    const bool fused_kv = R.seq_stride != 0 && !mfma_attn;
    if (owns && !fused_kv) {
      QkvPostArgs a;
      a.qkv = F(W.qkv);
      a.gq = d.g_q;
      a.gk = d.g_k;
      a.rope = F(W.rope);
      a.rope_ld = m->c.head_dim + m->c.global_head_dim;
      a.rope_off = y.full ? m->c.head_dim : 0;
      a.kc = m->kc[l];
      a.vc = m->vc[l];
      a.ks = m->ks[l];
      a.vs = m->vs[l];
      a.kvq = m->kv_quant;
      a.nq = m->nq;
      a.hd = y.hd;
      a.qkv_parts = nd_qkv;
      a.qkv_pstride = (size_t)n * d.qkv.N;
      a.eps = eps;
      CK(launch_qkv_post(R, a, st), "k/v write");
    }
    {
      AttnArgs a;
      a.qkv = F(W.qkv);
      a.gq = d.g_q;
      a.gk = d.g_k;
      a.rope = F(W.rope);
      a.rope_ld = m->c.head_dim + m->c.global_head_dim;
      a.rope_off = y.full ? m->c.head_dim : 0;
      a.kc = m->kc[y.src];
      a.vc = m->vc[y.src];
      a.ks = m->ks[y.src];
      a.vs = m->vs[y.src];
      a.kvq = m->kv_quant;
      a.kc_own = (owns && fused_kv) ? m->kc[l] : nullptr;
      a.vc_own = (owns && fused_kv) ? m->vc[l] : nullptr;
      a.ks_own = (owns && fused_kv) ? m->ks[l] : nullptr;
      a.vs_own = (owns && fused_kv) ? m->vs[l] : nullptr;
      a.owns = owns;
      a.part = F(W.part);
      a.out = F(W.attn);
      a.nq = m->nq;
      a.hd = y.hd;
      a.window = y.full ? 0 : m->c.sliding_window;
      a.qkv_parts = nd_qkv;
      a.qkv_pstride = (size_t)n * d.qkv.N;
      a.eps = eps;
      a.mfma = mfma_attn;
      attn_chunks(m, y.full, n, mfma_attn, &a.chunk, &a.nchunk);
      // one row: the O product merges the chunk partials itself; batched: the
      // merge writes the O product's prepared input
      a.combine = bat ? 1 : 0;
      if (bat) {
        a.xh = reinterpret_cast<uint16_t*>(ws + W.xh);
        a.xl = reinterpret_cast<uint16_t*>(ws + W.xl);
        a.xg = F(W.xg);
      }
      nchunk = a.nchunk;
      e2b_model::Mark mk{};
      const bool prof = m->prof_kind == E2B_KIND_ATTN;
      if (prof) {  // the attention kernel's own dispatch timestamps (bytes: the caller's)
        CK(hipEventCreate(&mk.a), "profile event");
        CK(hipEventCreate(&mk.b), "profile event");
        set_launch_events(mk.a, mk.b);
      }
      CK(launch_attention(R, a, st), "attention");
      if (prof) m->marks.push_back(mk);
    }
    {
      Prologue pr;
      if (bat) {
        pr.kind = kPrepared;
      } else {
        pr.kind = kAttnMerge;
        pr.a = F(W.part);
        pr.nchunk = nchunk;
        pr.slice = y.hd;
      }
      Epilogue ep;
      ep.y = F(W.oo);
      CK(matmul(m, q, kTagO, d.o, n, bat, pr, ep, true, &nd_o, nullptr, ws, W, st), "o projection");
    }
    {  // post-attention norm + residual, pre-FFN norm, gate/up
      Prologue pr;
      pr.kind = kResNorm;
      pr.a = cur;
      pr.d = F(W.oo);
      pr.nd = nd_o;
      pr.d_pstride = (size_t)n * H;
      pr.gd = d.g_pa;
      pr.gx = d.g_pf;
      pr.h_out = oth;
      pr.eps = eps;
      Epilogue ep;
      ep.y = F(W.gu);
      if (geglu_fold) {  // the product writes the down product's input itself
        ep.gh = reinterpret_cast<uint16_t*>(ws + W.xh2);
        ep.gl = reinterpret_cast<uint16_t*>(ws + W.xl2);
        ep.gg = F(W.xg2);
        ep.gi = y.I;
      }
      CK(matmul(m, q, kTagGateUp, d.gu, n, bat, pr, ep, true, &nd_gu, nullptr, ws, W, st),
         "gate/up projection");
      std::swap(cur, oth);
    }
    {  // GeGLU then down
      Prologue pr;
      pr.kind = kGeglu;
      pr.a = F(W.gu);
      pr.lda = 2 * y.I;
      pr.na = nd_gu;
      pr.a_pstride = (size_t)n * 2 * y.I;
      if (geglu_fold) {
        pr = Prologue();
        pr.kind = kPrepared;
        pr.alt = 1;
      }
      Epilogue ep;
      ep.y = F(W.dn);
      CK(matmul(m, q, kTagDown, d.down, n, bat, pr, ep, true, &nd_dn, nullptr, ws, W, st),
         "down projection");
    }
    {  // post-FFN norm + residual, per-layer input gate
      Prologue pr;
      pr.kind = kRes;
      pr.a = cur;
      pr.d = F(W.dn);
      pr.nd = nd_dn;
      pr.d_pstride = (size_t)n * H;
      pr.gd = d.g_ff;
      pr.h_out = oth;
      pr.eps = eps;
      Epilogue ep;
      ep.y = F(W.pgy);
      CK(matmul(m, q, kTagPleGate, d.pg, n, bat, pr, ep, true, &nd_pg, nullptr, ws, W, st),
         "per-layer input gate");
      std::swap(cur, oth);
    }
    {  // gelu(gate) * pli[l], per-layer projection
      Prologue pr;
      pr.kind = kPleGate;
      pr.a = F(W.pgy);
      pr.lda = P;
      pr.na = nd_pg;
      pr.a_pstride = (size_t)n * P;
      pr.pli = F(W.pli) + (size_t)l * P;
      pr.pli_ld = LP;
      Epilogue ep;
      ep.y = F(W.ppo);
      CK(matmul(m, q, kTagPleProj, d.pp, n, bat, pr, ep, true, &pend_n, nullptr, ws, W, st),
         "per-layer projection");
    }
    pend = F(W.ppo);
    pend_g = d.g_pple;
    pend_s = d.scalar;
  }
  if (!head) return E2B_OK;
  const int hr = head_row < 0 ? 0 : head_row;
  const int nh = head_row < 0 ? n : 1;
  const Lin& E = m->embed;  // the tied lm_head
  Prologue pr;
  pr.kind = kResNorm;
  pr.a = cur + (size_t)hr * H;
  pr.d = pend + (size_t)hr * H;
  pr.nd = pend_n;
  pr.d_pstride = (size_t)n * H;
  pr.gd = pend_g;
  pr.scalar = pend_s;
  pr.gx = m->g_final;
  pr.h_out = oth + (size_t)hr * H;
  pr.eps = eps;
  Epilogue ep;
  ep.argmax = 1;
  ep.logits = d_logits;
  ep.cand_val = F(W.cv);
  ep.cand_idx = reinterpret_cast<int32_t*>(ws + W.ci);
  int nblk = 0;
  CK(matmul(m, m->equant, kTagLmHead, E, nh, bat, pr, ep, false, nullptr, &nblk, ws, W, st),
     "lm_head");
  if (nblk > W.ncand) return fail(E2B_EINVAL, "lm_head: %d candidate blocks", nblk);
  CK(launch_argmax_final(nh, nblk, ep.cand_val, ep.cand_idx, d_argmax, adv_pos, st), "argmax");
  return E2B_OK;
}

}  // namespace

// ============================================================== public ABI
extern "C" {

const char* e2b_last_error(void) { return g_err.c_str(); }

int e2b_config_preset(const char* name, e2b_config* out) {
  if (!name || !out) return fail(E2B_EINVAL, "null argument");
  e2b_config c{};
  c.num_key_value_heads = 1;
  c.layer_pattern_period = 5;
  c.use_double_wide_mlp = 1;
  c.quant = E2B_QUANT_BF16;
  c.embed_quant = E2B_QUANT_BF16;
  c.kv_quant = E2B_KV_BF16;
  c.group_size = 32;
  c.rms_eps = 1e-6f;
  c.rope_theta_sliding = 1.0e4f;
  c.rope_theta_full = 1.0e6f;
  if (!strcmp(name, "e2b")) {
    c.num_hidden_layers = 35;
    c.num_kv_shared_layers = 20;
    c.hidden_size = 1536;
    c.num_attention_heads = 8;
    c.head_dim = 256;
    c.global_head_dim = 512;
    c.sliding_window = 512;
    c.intermediate_size = 6144;
    c.hidden_size_per_layer_input = 256;
    c.vocab_size = 262144;
  } else if (!strcmp(name, "toy") || !strcmp(name, "toy10")) {
    const bool ten = !strcmp(name, "toy10");
    c.num_hidden_layers = ten ? 10 : 5;
    c.num_kv_shared_layers = ten ? 5 : 2;
    c.hidden_size = 256;
    c.num_attention_heads = 2;
    c.head_dim = 64;
    c.global_head_dim = 128;
    c.sliding_window = 16;
    c.intermediate_size = 512;
    c.hidden_size_per_layer_input = 32;
    c.vocab_size = 4096;
  } else {
    return fail(E2B_EINVAL, "unknown preset '%s'", name);
  }
  *out = c;
  return E2B_OK;
}

int e2b_create(const e2b_config* cfg, e2b_model** out) {
  if (!cfg || !out) return fail(E2B_EINVAL, "null argument");
  *out = nullptr;
  const e2b_config& c = *cfg;
  auto hd_ok = [](int h) { return h == 64 || h == 128 || h == 256 || h == 512; };
  if (c.num_key_value_heads != 1) return fail(E2B_EINVAL, "num_key_value_heads must be 1");
  if (c.num_hidden_layers < 1 || c.num_hidden_layers > 256)
    return fail(E2B_EINVAL, "num_hidden_layers out of range");
  if (c.num_kv_shared_layers < 0 || c.num_kv_shared_layers >= c.num_hidden_layers)
    return fail(E2B_EINVAL, "num_kv_shared_layers out of range");
  if (!hd_ok(c.head_dim) || !hd_ok(c.global_head_dim))
    return fail(E2B_EINVAL, "head dims must be 64, 128, 256 or 512");
  if (c.num_attention_heads < 1 || c.num_attention_heads > 8)
    return fail(E2B_EINVAL, "num_attention_heads must be 1..8");
  if (c.group_size != 32) return fail(E2B_EINVAL, "group_size must be 32");
  if (c.layer_pattern_period < 1) return fail(E2B_EINVAL, "layer_pattern_period < 1");
  if (c.sliding_window < 1) return fail(E2B_EINVAL, "sliding_window < 1");
  if (c.vocab_size < 1 || c.hidden_size_per_layer_input < 1 ||
      c.hidden_size_per_layer_input > 256)
    return fail(E2B_EINVAL, "vocab_size / hidden_size_per_layer_input out of range");
  if (c.quant != E2B_QUANT_BF16 && c.quant != E2B_QUANT_W4A16)
    return fail(E2B_EINVAL, "unknown quant mode %d", c.quant);
  if (c.embed_quant != E2B_QUANT_BF16 && c.embed_quant != E2B_QUANT_W4A16)
    return fail(E2B_EINVAL, "unknown vocabulary-table format %d", c.embed_quant);
  if (c.kv_quant != E2B_KV_BF16 && c.kv_quant != E2B_KV_INT8)
    return fail(E2B_EINVAL, "unknown K/V cache format %d", c.kv_quant);
  if (c.embed_quant == E2B_QUANT_W4A16 &&
      (c.hidden_size % 32 || (c.num_hidden_layers * c.hidden_size_per_layer_input) % 32))
    return fail(E2B_EINVAL, "int4 vocabulary tables need rows in whole 32-groups");
  if (!(c.rms_eps > 0) || !(c.rope_theta_sliding > 1) || !(c.rope_theta_full > 1))
    return fail(E2B_EINVAL, "rms_eps / rope thetas out of range");
  e2b_model* m = new e2b_model();
  m->c = c;
  m->L = c.num_hidden_layers;
  m->H = c.hidden_size;
  m->P = c.hidden_size_per_layer_input;
  m->V = c.vocab_size;
  m->nq = c.num_attention_heads;
  m->first = c.num_hidden_layers - c.num_kv_shared_layers;
  m->quant = c.quant;
  m->equant = c.embed_quant;
  m->kv_quant = c.kv_quant;
  m->li.resize(m->L);
  for (int l = 0; l < m->L; ++l) {
    LayerInfo& y = m->li[l];
    y.full = is_full(c, l);
    y.hd = y.full ? c.global_head_dim : c.head_dim;
    y.theta = y.full ? c.rope_theta_full : c.rope_theta_sliding;
    y.I = c.intermediate_size * ((c.use_double_wide_mlp && l >= m->first) ? 2 : 1);
    y.src = kv_src(c, l);
  }
  // every matrix-vector product must have a supported K and widths in 32-groups
  std::vector<int> Ks = {m->H, m->P};
  for (const LayerInfo& y : m->li) {
    Ks.push_back(m->nq * y.hd);
    Ks.push_back(y.I);
  }
  for (int K : Ks)
    if (K % 32 || !supported_k(K)) {
      delete m;
      return fail(E2B_EINVAL, "unsupported reduction width %d", K);
    }
  if (e2b::gemv_splits(m->H) != 1) {
    delete m;
    return fail(E2B_EINVAL, "hidden_size %d must be a single slice (<=512, 1536 or 2048)", m->H);
  }
  build_plan(m);
  *out = m;
  return E2B_OK;
}

void e2b_destroy(e2b_model* m) { delete m; }

int e2b_kv_share_map(const e2b_model* m, int32_t* out) {
  if (!m || !out) return fail(E2B_EINVAL, "null argument");
  for (int l = 0; l < m->L; ++l) out[l] = m->li[l].src;
  return E2B_OK;
}

size_t e2b_weight_bytes(const e2b_model* m) { return m ? m->weight_bytes : 0; }
size_t e2b_arena_bytes(const e2b_model* m) { return m ? m->arena_bytes : 0; }

}  // extern "C"

namespace {
// bytes of a K/V pool of `rows` cached rows per K/V-owning layer
size_t kv_pool_bytes(const e2b_model* m, size_t rows) {
  size_t b = 0;
  for (int l = 0; l < m->L; ++l) {
    if (m->li[l].src != l) continue;
    if (m->kv_quant == E2B_KV_INT8)  // int8 codes, then one fp32 scale per row, for K and V
      b += 2 * (rows * m->li[l].hd + align_up(rows * sizeof(float)));
    else
      b += 2 * rows * m->li[l].hd * sizeof(uint16_t);
  }
  return b;
}

// bind d_kv as a pool of `rows` rows per K/V-owning layer: K rows, V rows
// (bf16 or int8 codes), then for int8 the K and V row scales
void bind_pool(e2b_model* m, char* kv, size_t rows) {
  m->kv = kv;
  m->kc.assign(m->L, nullptr);
  m->vc.assign(m->L, nullptr);
  m->ks.assign(m->L, nullptr);
  m->vs.assign(m->L, nullptr);
  const bool i8 = m->kv_quant == E2B_KV_INT8;
  size_t off = 0;
  for (int l = 0; l < m->L; ++l) {
    if (m->li[l].src != l) continue;
    const size_t one = rows * m->li[l].hd * (i8 ? 1 : sizeof(uint16_t));
    m->kc[l] = m->kv + off;
    m->vc[l] = m->kv + off + one;
    off += 2 * one;
    if (i8) {
      const size_t sb = align_up(rows * sizeof(float));
      m->ks[l] = reinterpret_cast<float*>(m->kv + off);
      m->vs[l] = reinterpret_cast<float*>(m->kv + off + sb);
      off += 2 * sb;
    }
  }
  for (int l = 0; l < m->L; ++l)  // sharing layers read their source's region
    if (m->li[l].src != l) {
      const int s = m->li[l].src;
      m->kc[l] = m->kc[s];
      m->vc[l] = m->vc[s];
      m->ks[l] = m->ks[s];
      m->vs[l] = m->vs[s];
    }
}

// upload one slot's row of the page table (synchronous: the host mirror may
// change right after)
int upload_page_row(e2b_model* m, int slot, hipStream_t st) {
  const size_t n = m->page_stride;
  CK(hipMemcpyAsync(m->d_pages + slot * n, m->h_pages.data() + slot * n, n * sizeof(int32_t),
                    hipMemcpyHostToDevice, st),
     "page table upload");
  CK(hipStreamSynchronize(st), "page table upload sync");
  return E2B_OK;
}
}  // namespace

extern "C" {

size_t e2b_kv_bytes(const e2b_model* m, int max_batch, int max_ctx) {
  if (!m || max_batch < 1 || max_ctx < 1) return 0;
  return kv_pool_bytes(m, (size_t)max_batch * max_ctx);
}

size_t e2b_kv_paged_bytes(const e2b_model* m, int n_pages) {
  if (!m || n_pages < 1) return 0;
  // one spare page past the pool: where a position with no reserved page goes
  return kv_pool_bytes(m, (size_t)(n_pages + 1) * e2b::kPageSize);
}

size_t e2b_workspace_bytes(const e2b_model* m, int max_rows) {
  if (!m || max_rows < 1) return 0;
  return ws_layout(m, max_rows).total;
}

int e2b_load_weights(e2b_model* m, const e2b_tensor* t, int n, void* d_arena, size_t arena_bytes,
                     void* stream) {
  if (!m || (!t && n) || !d_arena) return fail(E2B_EINVAL, "null argument");
  if (arena_bytes < m->arena_bytes)
    return fail(E2B_ENOMEM, "arena of %zu bytes < %zu required", arena_bytes, m->arena_bytes);
  if (reinterpret_cast<uintptr_t>(d_arena) % kAlign)
    return fail(E2B_EINVAL, "arena must be %zu-byte aligned", kAlign);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // match every planned copy to exactly one tensor; reject strays
  std::vector<int> used(n, 0);
  std::vector<int> src(m->plan.size(), -1);
  for (size_t i = 0; i < m->plan.size(); ++i) {
    const Copy& cp = m->plan[i];
    for (int j = 0; j < n; ++j) {
      if (!t[j].name || strcmp(t[j].name, cp.name.c_str())) continue;
      if (src[i] >= 0) return fail(E2B_EINVAL, "duplicate tensor %s", cp.name.c_str());
      src[i] = j;
    }
    if (src[i] < 0) return fail(E2B_EINVAL, "missing tensor %s", cp.name.c_str());
    const e2b_tensor& x = t[src[i]];
    const bool shape_ok = x.ndim == cp.ndim && x.shape[0] == cp.d0 && (cp.ndim == 1 || x.shape[1] == cp.d1);
    if (x.dtype != cp.dtype || !shape_ok || !x.data)
      return fail(E2B_EINVAL, "tensor %s: expected dtype %d shape [%lld%s%lld], got dtype %d ndim %d [%lld, %lld]",
                  cp.name.c_str(), cp.dtype, (long long)cp.d0, cp.ndim == 2 ? ", " : "",
                  cp.ndim == 2 ? (long long)cp.d1 : 0LL, x.dtype, x.ndim,
                  (long long)x.shape[0], (long long)(x.ndim > 1 ? x.shape[1] : 0));
    used[src[i]] = 1;
  }
  for (int j = 0; j < n; ++j)
    if (!used[j] && !(t[j].name && ignorable(m, t[j].name)))
      return fail(E2B_EINVAL, "unexpected tensor %s", t[j].name ? t[j].name : "(null)");
  char* A = reinterpret_cast<char*>(d_arena);
  for (size_t i = 0; i < m->plan.size(); ++i) {
    const Copy& cp = m->plan[i];
    const size_t esz = cp.dtype == E2B_DTYPE_INT32 ? 4 : 2;
    const size_t bytes = esz * cp.d0 * (cp.ndim == 2 ? cp.d1 : 1);
    CK(hipMemcpyAsync(A + cp.dst, t[src[i]].data, bytes, hipMemcpyHostToDevice, st),
       "weight upload");
  }
  for (int k = 0; k < 2; ++k) {
    const int hd = k ? m->c.global_head_dim : m->c.head_dim;
    const double theta = k ? m->c.rope_theta_full : m->c.rope_theta_sliding;
    std::vector<double> f(hd / 2);
    for (int i = 0; i < hd / 2; ++i) f[i] = std::pow(theta, -2.0 * i / hd);
    CK(hipMemcpyAsync(A + m->off_invf[k], f.data(), f.size() * sizeof(double),
                      hipMemcpyHostToDevice, st),
       "rope table upload");
    CK(hipStreamSynchronize(st), "weight upload sync");  // f must outlive the copy
  }
  m->arena = A;
  auto U = [&](size_t off) { return reinterpret_cast<const uint16_t*>(A + off); };
  m->embed = resolve(m, m->embed_off);
  m->ple = resolve(m, m->ple_off);
  m->g_plpn = U(m->off_plpn);
  m->g_final = U(m->off_final);
  m->invf[0] = reinterpret_cast<const double*>(A + m->off_invf[0]);
  m->invf[1] = reinterpret_cast<const double*>(A + m->off_invf[1]);
  m->plmp = resolve(m, m->plmp_off);
  m->ld.assign(m->L, LayerDev());
  for (int l = 0; l < m->L; ++l) {
    const LayerOff& o = m->lo[l];
    LayerDev& d = m->ld[l];
    d.qkv = resolve(m, o.qkv);
    d.o = resolve(m, o.o);
    d.gu = resolve(m, o.gu);
    d.down = resolve(m, o.down);
    d.pg = resolve(m, o.pg);
    d.pp = resolve(m, o.pp);
    d.g_in = U(o.g_in);
    d.g_q = U(o.g_q);
    d.g_k = m->li[l].src == l ? U(o.g_k) : nullptr;
    d.g_pa = U(o.g_pa);
    d.g_pf = U(o.g_pf);
    d.g_ff = U(o.g_ff);
    d.g_pple = U(o.g_pple);
    d.scalar = U(o.scalar);
  }
  // the matrix-core copies of the linears (and of the tied embedding, for the
  // batched lm_head), tiled on the device
  auto tile = [&](const LinOff& o) -> hipError_t {
    if (!o.tiled) return hipSuccess;
    const Lin W = resolve(m, o);
    if (o.quant == E2B_QUANT_BF16) return e2b::launch_tile_bf16(W, reinterpret_cast<uint16_t*>(A + o.tw), st);
    return e2b::launch_tile_w4(W, reinterpret_cast<uint32_t*>(A + o.tq),
                               reinterpret_cast<uint16_t*>(A + o.ts), st);
  };
  CK(tile(m->plmp_off), "weight tiling");
  CK(tile(m->embed_off), "embedding tiling");
  for (int l = 0; l < m->L; ++l) {
    const LayerOff& o = m->lo[l];
    for (const LinOff* x : {&o.qkv, &o.o, &o.gu, &o.down, &o.pg, &o.pp}) CK(tile(*x), "weight tiling");
  }
  CK(hipStreamSynchronize(st), "weight tiling sync");
  m->loaded = true;
  return E2B_OK;
}

int e2b_kv_alloc(e2b_model* m, void* d_kv, size_t bytes, int max_batch, int max_ctx) {
  if (!m || !d_kv) return fail(E2B_EINVAL, "null argument");
  if (max_batch < 1 || max_ctx < 1) return fail(E2B_EINVAL, "max_batch and max_ctx must be >= 1");
  if (max_batch > kMaxCtlRows) return fail(E2B_EINVAL, "max_batch above %d", kMaxCtlRows);
  const size_t need = e2b_kv_bytes(m, max_batch, max_ctx);
  if (bytes < need) return fail(E2B_ENOMEM, "kv buffer of %zu bytes < %zu required", bytes, need);
  if (reinterpret_cast<uintptr_t>(d_kv) % 16) return fail(E2B_EINVAL, "kv buffer must be 16-byte aligned");
  m->max_batch = max_batch;
  m->max_ctx = max_ctx;
  m->n_pages = 0;
  m->d_pages = nullptr;
  bind_pool(m, reinterpret_cast<char*>(d_kv), (size_t)max_batch * max_ctx);
  return E2B_OK;
}

int e2b_kv_alloc_paged(e2b_model* m, void* d_kv, size_t bytes, int n_pages, int32_t* d_page_table,
                       int max_batch, int max_ctx, void* stream) {
  if (!m || !d_kv || !d_page_table) return fail(E2B_EINVAL, "null argument");
  if (n_pages < 1 || max_batch < 1 || max_ctx < 1)
    return fail(E2B_EINVAL, "n_pages, max_batch and max_ctx must be >= 1");
  if (max_batch > kMaxCtlRows) return fail(E2B_EINVAL, "max_batch above %d", kMaxCtlRows);
  const size_t need = e2b_kv_paged_bytes(m, n_pages);
  if (bytes < need) return fail(E2B_ENOMEM, "kv buffer of %zu bytes < %zu required", bytes, need);
  if (reinterpret_cast<uintptr_t>(d_kv) % 16 || reinterpret_cast<uintptr_t>(d_page_table) % 4)
    return fail(E2B_EINVAL, "kv buffer must be 16-byte aligned, page table 4-byte aligned");
  m->max_batch = max_batch;
  m->max_ctx = max_ctx;
  m->n_pages = n_pages;
  m->page_stride = (max_ctx + e2b::kPageSize - 1) / e2b::kPageSize;
  m->d_pages = d_page_table;
  m->h_pages.assign((size_t)max_batch * m->page_stride, -1);
  m->slot_pages.assign(max_batch, 0);
  m->free_pages.clear();
  for (int p = n_pages - 1; p >= 0; --p) m->free_pages.push_back(p);  // page 0 handed out first
  bind_pool(m, reinterpret_cast<char*>(d_kv), (size_t)(n_pages + 1) * e2b::kPageSize);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CK(hipMemcpyAsync(m->d_pages, m->h_pages.data(), m->h_pages.size() * sizeof(int32_t),
                    hipMemcpyHostToDevice, st),
     "page table upload");
  CK(hipStreamSynchronize(st), "page table upload sync");
  return E2B_OK;
}

int e2b_seq_reserve(e2b_model* m, int slot, int n_positions, void* stream) {
  if (!m) return fail(E2B_EINVAL, "null argument");
  if (!m->d_pages) return fail(E2B_ESTATE, "the cache is not paged");
  if (slot < 0 || slot >= m->max_batch) return fail(E2B_ERANGE, "slot %d outside [0, %d)", slot, m->max_batch);
  if (n_positions < 0 || n_positions > m->max_ctx)
    return fail(E2B_ERANGE, "positions %d outside [0, %d]", n_positions, m->max_ctx);
  const int need = (n_positions + e2b::kPageSize - 1) / e2b::kPageSize;
  const int more = need - m->slot_pages[slot];
  if (more <= 0) return E2B_OK;
  if (more > (int)m->free_pages.size())
    return fail(E2B_ENOMEM, "%d more pages needed, %zu free", more, m->free_pages.size());
  for (int k = m->slot_pages[slot]; k < need; ++k) {
    m->h_pages[(size_t)slot * m->page_stride + k] = m->free_pages.back();
    m->free_pages.pop_back();
  }
  m->slot_pages[slot] = need;
  return upload_page_row(m, slot, reinterpret_cast<hipStream_t>(stream));
}

int e2b_seq_release(e2b_model* m, int slot, void* stream) {
  if (!m) return fail(E2B_EINVAL, "null argument");
  if (!m->d_pages) return fail(E2B_ESTATE, "the cache is not paged");
  if (slot < 0 || slot >= m->max_batch) return fail(E2B_ERANGE, "slot %d outside [0, %d)", slot, m->max_batch);
  for (int k = m->slot_pages[slot] - 1; k >= 0; --k) {
    int32_t& e = m->h_pages[(size_t)slot * m->page_stride + k];
    m->free_pages.push_back(e);
    e = -1;
  }
  m->slot_pages[slot] = 0;
  return upload_page_row(m, slot, reinterpret_cast<hipStream_t>(stream));
}

int e2b_seq_move(e2b_model* m, int from, int to, void* stream) {
  if (!m) return fail(E2B_EINVAL, "null argument");
  if (!m->d_pages) return fail(E2B_ESTATE, "the cache is not paged");
  if (from < 0 || from >= m->max_batch || to < 0 || to >= m->max_batch)
    return fail(E2B_ERANGE, "slots %d, %d outside [0, %d)", from, to, m->max_batch);
  if (from == to) return E2B_OK;
  if (m->slot_pages[to]) return fail(E2B_ESTATE, "slot %d still holds pages", to);
  const size_t n = m->page_stride;
  std::copy(m->h_pages.begin() + from * n, m->h_pages.begin() + (from + 1) * n, m->h_pages.begin() + to * n);
  std::fill(m->h_pages.begin() + from * n, m->h_pages.begin() + (from + 1) * n, -1);
  m->slot_pages[to] = m->slot_pages[from];
  m->slot_pages[from] = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rc = upload_page_row(m, to, st);
  return rc ? rc : upload_page_row(m, from, st);
}

int e2b_pages_free(const e2b_model* m) { return m && m->d_pages ? (int)m->free_pages.size() : 0; }

}  // extern "C"

namespace {
void set_paging(const e2b_model* m, e2b::Rows& R, void* d_ws) {
  R.pages = m->d_pages;
  R.page_stride = m->page_stride;
  R.n_pages = m->n_pages;
  R.err = reinterpret_cast<int*>(d_ws);
}

// adv_pos (graph capture): also advance the positions, by the final argmax
// kernel of the per-phase path (*advanced set) or not at all
int decode_impl(e2b_model* m, const int32_t* d_tokens, const int32_t* d_positions, int batch,
                float* d_logits, int32_t* d_argmax, void* d_ws, size_t ws_bytes, void* stream,
                int32_t* adv_pos, bool* advanced) {
  if (advanced) *advanced = false;
  if (!m || !d_tokens || !d_positions || !d_argmax || !d_ws)
    return fail(E2B_EINVAL, "null argument");
  if (!m->loaded) return fail(E2B_ESTATE, "weights not loaded");
  if (!m->kv) return fail(E2B_ESTATE, "kv cache not bound");
  if (batch < 1 || batch > m->max_batch)
    return fail(E2B_ERANGE, "batch %d outside [1, %d]", batch, m->max_batch);
  const Ws W = ws_layout(m, batch);
  if (ws_bytes < W.total)
    return fail(E2B_ENOMEM, "workspace of %zu bytes < %zu required", ws_bytes, W.total);
  if (reinterpret_cast<uintptr_t>(d_ws) % kAlign)
    return fail(E2B_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  e2b::Rows R;
  R.tokens = d_tokens;
  R.positions = d_positions;
  R.seq0 = 0;
  R.seq_stride = 1;
  R.n = batch;
  R.max_ctx = m->max_ctx;
  R.vocab = m->V;
  set_paging(m, R, d_ws);
  const int rc = run_rows(m, R, true, -1, d_logits, d_argmax, reinterpret_cast<char*>(d_ws), W,
                         reinterpret_cast<hipStream_t>(stream), adv_pos);
  if (rc == E2B_OK && advanced) *advanced = adv_pos != nullptr;
  return rc;
}
}  // namespace

extern "C" {
int e2b_decode_step(e2b_model* m, const int32_t* d_tokens, const int32_t* d_positions, int batch,
                    float* d_logits, int32_t* d_argmax, void* d_ws, size_t ws_bytes,
                    void* stream) {
  return decode_impl(m, d_tokens, d_positions, batch, d_logits, d_argmax, d_ws, ws_bytes, stream,
                     nullptr, nullptr);
}

int e2b_prefill(e2b_model* m, int seq, const int32_t* d_tokens, int n_tokens, int pos0,
                float* d_logits_last, int32_t* d_argmax_last, void* d_ws, size_t ws_bytes,
                void* stream) {
  if (!m || !d_tokens || !d_argmax_last || !d_ws) return fail(E2B_EINVAL, "null argument");
  if (!m->loaded) return fail(E2B_ESTATE, "weights not loaded");
  if (!m->kv) return fail(E2B_ESTATE, "kv cache not bound");
  if (seq < 0 || seq >= m->max_batch) return fail(E2B_ERANGE, "sequence %d outside [0, %d)", seq, m->max_batch);
  if (n_tokens < 1 || pos0 < 0 || (int64_t)pos0 + n_tokens > m->max_ctx)
    return fail(E2B_ERANGE, "positions [%d, %lld) outside [0, %d)", pos0,
                (long long)pos0 + n_tokens, m->max_ctx);
  if (reinterpret_cast<uintptr_t>(d_ws) % kAlign)
    return fail(E2B_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  int cap = std::min(n_tokens, 128);
  while (cap > 0 && ws_layout(m, cap).total > ws_bytes) --cap;
  if (cap < 1)
    return fail(E2B_ENOMEM, "workspace of %zu bytes < %zu required for one row", ws_bytes,
                ws_layout(m, 1).total);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int off = 0; off < n_tokens; off += cap) {
    const int r = std::min(cap, n_tokens - off);
    e2b::Rows R;
    R.tokens = d_tokens + off;
    R.positions = nullptr;
    R.pos0 = pos0 + off;
    R.seq0 = seq;
    R.seq_stride = 0;
    R.n = r;
    R.max_ctx = m->max_ctx;
    R.vocab = m->V;
    set_paging(m, R, d_ws);
    const bool last = off + r == n_tokens;
    int rc = run_rows(m, R, last, r - 1, d_logits_last, d_argmax_last,
                      reinterpret_cast<char*>(d_ws), ws_layout(m, r), st);
    if (rc) return rc;
  }
  return E2B_OK;
}

int e2b_kv_view(const e2b_model* m, int layer, int which, void** out) {
  if (!m || !out) return fail(E2B_EINVAL, "null argument");
  if (!m->kv) return fail(E2B_ESTATE, "kv cache not bound");
  const int nwhich = m->kv_quant == E2B_KV_INT8 ? 4 : 2;
  if (layer < 0 || layer >= m->L || which < 0 || which >= nwhich)
    return fail(E2B_EINVAL, "bad layer %d / which %d", layer, which);
  const int s = m->li[layer].src;
  void* v[4] = {m->kc[s], m->vc[s], m->ks[s], m->vs[s]};
  *out = v[which];
  return E2B_OK;
}

namespace {
// Workspace of e2b_matvec: the K-slice partials of the one-row matvec kernel
// or of the several-row matrix-core product (none when unsplit), then, for
// several rows with N % 16 == 0, the copy of the weights tiled in the
// matrix-core fragment order that batched decode reads (the arena holds one
// per linear; here it is built in the workspace).
struct MvWs {
  size_t part, tq, ts, total;
  int nks;
  bool tiled;
};
MvWs matvec_ws(int quant, int N, int K, int rows) {
  MvWs w{};
  w.nks = rows == 1 ? e2b::gemv_splits(K) : e2b::gemm_plan(quant, N, K, true).nks;
  size_t cur = 0;
  w.part = 0;
  if (w.nks > 1) cur = align_up((size_t)w.nks * rows * N * sizeof(float));
  w.tiled = rows > 1 && N % 16 == 0 && (quant == E2B_QUANT_BF16 || K % 128 == 0);
  if (w.tiled) {
    w.tq = cur;
    cur = align_up(cur + (quant ? (size_t)N * K / 2 : (size_t)N * K * 2));
    if (quant) {
      w.ts = cur;
      cur = align_up(cur + (size_t)N * (K / 32) * 2);
    }
  }
  w.total = cur;
  return w;
}
}  // namespace

size_t e2b_matvec_workspace_bytes(int quant, int N, int K, int rows) {
  if (quant != E2B_QUANT_BF16 && quant != E2B_QUANT_W4A16) return 0;
  if (N < 1 || rows < 1 || K < 32 || K % 32 || !supported_k(K)) return 0;
  return matvec_ws(quant, N, K, rows).total;
}

int e2b_matvec(int quant, const void* d_w, const uint16_t* d_scale, int N, int K,
               const float* d_x, int rows, float* d_y, void* d_ws, size_t ws_bytes,
               void* stream) {
  if (!d_w || !d_x || !d_y || (quant == E2B_QUANT_W4A16 && !d_scale))
    return fail(E2B_EINVAL, "null argument");
  if (quant != E2B_QUANT_BF16 && quant != E2B_QUANT_W4A16)
    return fail(E2B_EINVAL, "unknown quant mode %d", quant);
  if (N < 1 || rows < 1 || rows > 65535 || K % 32 || !supported_k(K))
    return fail(E2B_EINVAL, "unsupported shape N=%d K=%d rows=%d", N, K, rows);
  if (reinterpret_cast<uintptr_t>(d_w) % 16) return fail(E2B_EINVAL, "weights must be 16-byte aligned");
  if (rows > 1 && reinterpret_cast<uintptr_t>(d_x) % 16)
    return fail(E2B_EINVAL, "x must be 16-byte aligned for several rows");
  const MvWs L = matvec_ws(quant, N, K, rows);
  if (L.total && (!d_ws || ws_bytes < L.total))
    return fail(E2B_ENOMEM, "workspace of %zu bytes < %zu required", ws_bytes, L.total);
  if (L.total && reinterpret_cast<uintptr_t>(d_ws) % 256)
    return fail(E2B_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(d_ws);
  Lin W;
  W.N = N;
  W.K = K;
  if (quant == E2B_QUANT_BF16) {
    W.w = reinterpret_cast<const uint16_t*>(d_w);
  } else {
    W.q = reinterpret_cast<const uint32_t*>(d_w);
    W.s = d_scale;
  }
  if (L.tiled) {
    if (quant == E2B_QUANT_BF16) {
      uint16_t* tw = reinterpret_cast<uint16_t*>(ws + L.tq);
      CK(e2b::launch_tile_bf16(W, tw, st), "matvec tiling");
      W.tw = tw;
    } else {
      uint32_t* tq = reinterpret_cast<uint32_t*>(ws + L.tq);
      uint16_t* ts = reinterpret_cast<uint16_t*>(ws + L.ts);
      CK(e2b::launch_tile_w4(W, tq, ts, st), "matvec tiling");
      W.tq = tq;
      W.ts = ts;
    }
  }
  e2b::Prologue pr;
  pr.kind = e2b::kPlain;
  pr.a = d_x;
  pr.lda = K;
  e2b::Epilogue ep;
  ep.y = L.nks > 1 ? reinterpret_cast<float*>(ws + L.part) : d_y;
  if (rows == 1) {
    CK(e2b::launch_gemv(quant, e2b::kTagOther, W, rows, pr, ep, 0, nullptr, st), "matvec");
  } else {
    e2b::GemmA A;
    A.a = d_x;
    A.kind = e2b::kPlain;
    A.lda = K;
    CK(e2b::launch_gemm(quant, e2b::kTagOther, W, rows, A, e2b::gemm_plan(quant, N, K, true), ep,
                        nullptr, st),
       "matvec mfma");
  }
  if (L.nks > 1) CK(e2b::launch_sum_partials(L.nks, (size_t)rows * N, ep.y, d_y, st), "matvec sum");
  return E2B_OK;
}

}  // extern "C"

// ---- allocation-free matrix-vector product --------------------------------
// The K-slice partials of e2b_matvec_noalloc live in this array, one copy per
// device, held until the process ends.  In host code `scratch` is only a
// host-side stand-in for the symbol: its device address on each device comes
// from hipGetSymbolAddress (resolved once per device, with that device
// current) and only that address is handed to kernels.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
}
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_dev;  // device address of `scratch`, by device ordinal

int scratch_address(void** out) {
  int dev = -1;
  CK(hipGetDevice(&dev), "noalloc: current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_dev.size() <= dev) g_scratch_dev.resize(dev + 1, nullptr);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    CK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "noalloc: scratch address");
    if (!p) return fail(E2B_EHIP, "noalloc: scratch address is null");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return E2B_OK;
}
}  // namespace

extern "C" {

size_t e2b_matvec_noalloc_max_bytes(void) { return kScratchBytes; }

int e2b_matvec_noalloc(int quant, const void* d_w, const uint16_t* d_scale, int N, int K,
                       const float* d_x, int rows, float* d_y, void* stream) {
  if (!d_w || !d_x || !d_y || (quant == E2B_QUANT_W4A16 && !d_scale))
    return fail(E2B_EINVAL, "null argument");
  if (quant != E2B_QUANT_BF16 && quant != E2B_QUANT_W4A16)
    return fail(E2B_EINVAL, "unknown quant mode %d", quant);
  if (N < 1 || rows < 1 || rows > 65535 || K % 32 || !supported_k(K))
    return fail(E2B_EINVAL, "unsupported shape N=%d K=%d rows=%d", N, K, rows);
  if (reinterpret_cast<uintptr_t>(d_w) % 16) return fail(E2B_EINVAL, "weights must be 16-byte aligned");
  if (rows > 1 && reinterpret_cast<uintptr_t>(d_x) % 16)
    return fail(E2B_EINVAL, "x must be 16-byte aligned for several rows");
  // the same product plan as e2b_matvec; only its K-slice partials need room
  const int nks = rows == 1 ? e2b::gemv_splits(K) : e2b::gemm_plan(quant, N, K, true).nks;
  const size_t need = nks > 1 ? (size_t)nks * rows * N * sizeof(float) : 0;
  if (need > kScratchBytes)
    return fail(E2B_ENOMEM, "noalloc: %zu bytes of K-slice partials exceed the %zu-byte scratch", need,
                kScratchBytes);
  void* sp = nullptr;
  if (need) {
    const int rc = scratch_address(&sp);
    if (rc) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Lin W;
  W.N = N;
  W.K = K;
  if (quant == E2B_QUANT_BF16) {
    W.w = reinterpret_cast<const uint16_t*>(d_w);
  } else {
    W.q = reinterpret_cast<const uint32_t*>(d_w);
    W.s = d_scale;
  }
  e2b::Prologue pr;
  pr.kind = e2b::kPlain;
  pr.a = d_x;
  pr.lda = K;
  e2b::Epilogue ep;
  ep.y = need ? reinterpret_cast<float*>(sp) : d_y;
  if (rows == 1) {
    CK(e2b::launch_gemv(quant, e2b::kTagOther, W, rows, pr, ep, 0, nullptr, st), "matvec");
  } else {
    e2b::GemmA A;
    A.a = d_x;
    A.kind = e2b::kPlain;
    A.lda = K;
    CK(e2b::launch_gemm(quant, e2b::kTagOther, W, rows, A, e2b::gemm_plan(quant, N, K, true), ep,
                        nullptr, st),
       "matvec mfma");
  }
  if (need) CK(e2b::launch_sum_partials(nks, (size_t)rows * N, ep.y, d_y, st), "matvec sum");
  return E2B_OK;
}

int e2b_stream_reduce(const void* d_buf, size_t bytes, float* d_out, void* stream) {
  if (!d_buf || !d_out) return fail(E2B_EINVAL, "null argument");
  if (bytes % 16 || reinterpret_cast<uintptr_t>(d_buf) % 16)
    return fail(E2B_EINVAL, "buffer and byte count must be multiples of 16");
  CK(e2b::launch_stream_reduce(d_buf, bytes, d_out, reinterpret_cast<hipStream_t>(stream)),
     "stream reduce");
  return E2B_OK;
}

int e2b_stream_reduce_blocks(void) { return e2b::kStreamBlocks; }

int e2b_embed(e2b_model* m, const int32_t* d_tokens, int n, float* d_h, float* d_tokple, void* d_ws,
              size_t ws_bytes, void* stream) {
  if (!m || !d_tokens || !d_h || !d_tokple || !d_ws) return fail(E2B_EINVAL, "null argument");
  if (!m->loaded) return fail(E2B_ESTATE, "weights not loaded");
  if (n < 1 || n > kMaxCtlRows) return fail(E2B_ERANGE, "n %d outside [1, %d]", n, kMaxCtlRows);
  const Ws W = ws_layout(m, n);
  if (ws_bytes < W.total)
    return fail(E2B_ENOMEM, "workspace of %zu bytes < %zu required", ws_bytes, W.total);
  if (reinterpret_cast<uintptr_t>(d_ws) % kAlign)
    return fail(E2B_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  if (reinterpret_cast<uintptr_t>(d_h) % 16 || reinterpret_cast<uintptr_t>(d_tokple) % 16)
    return fail(E2B_EINVAL, "outputs must be 16-byte aligned");
  char* ws = reinterpret_cast<char*>(d_ws);
  e2b::Rows R;
  R.tokens = d_tokens;
  R.positions = nullptr;  // rows at positions 0..n-1 (the RoPE angles go to the workspace)
  R.pos0 = 0;
  R.n = n;
  R.max_ctx = n;
  R.vocab = m->V;
  e2b::RopeTable rt;
  rt.out = reinterpret_cast<float*>(ws + W.rope);
  rt.inv_s = m->invf[0];
  rt.inv_f = m->invf[1];
  rt.hd_s = m->c.head_dim;
  rt.hd_f = m->c.global_head_dim;
  CK(e2b::launch_embed(R, m->embed, m->ple, std::sqrt((float)m->H),
                       std::sqrt((float)m->P), d_h, d_tokple, reinterpret_cast<int*>(ws + W.err), rt,
                       reinterpret_cast<hipStream_t>(stream)),
     "embed");
  return E2B_OK;
}

int e2b_graph_capture(e2b_model* m, const int32_t* d_tokens, int32_t* d_positions, int batch,
                      float* d_logits, int32_t* d_argmax, void* d_ws, size_t ws_bytes,
                      int advance_positions, void* stream, e2b_graph** out) {
  if (!out) return fail(E2B_EINVAL, "null argument");
  *out = nullptr;
  if (!stream) return fail(E2B_EINVAL, "graph capture needs a non-null stream");
  if (m && m->prof_kind) return fail(E2B_ESTATE, "cannot capture while profiling");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  e2b_graph* g = new e2b_graph();
  hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    delete g;
    return hip_fail(e, "begin capture");
  }
  bool advanced = false;
  int rc = decode_impl(m, d_tokens, d_positions, batch, d_logits, d_argmax, d_ws, ws_bytes, stream,
                       advance_positions ? d_positions : nullptr, &advanced);
  if (rc == E2B_OK && advance_positions && !advanced) {
    hipError_t ea = e2b::launch_advance(d_positions, batch, st);
    if (ea != hipSuccess) rc = hip_fail(ea, "advance positions");
  }
  const std::string saved = g_err;
  e = hipStreamEndCapture(st, &g->graph);
  if (rc != E2B_OK) {
    if (g->graph) (void)hipGraphDestroy(g->graph);
    delete g;
    g_err = saved;
    return rc;
  }
  if (e != hipSuccess) {
    delete g;
    return hip_fail(e, "end capture");
  }
  e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g->graph);
    delete g;
    return hip_fail(e, "graph instantiate");
  }
  *out = g;
  return E2B_OK;
}

int e2b_graph_replay(e2b_graph* g, void* stream) {
  if (!g || !g->exec) return fail(E2B_EINVAL, "null graph");
  CK(hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream)), "graph launch");
  return E2B_OK;
}

void e2b_graph_destroy(e2b_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

static void drop_marks(e2b_model* m) {
  for (auto& mk : m->marks) {
    (void)hipEventDestroy(mk.a);
    (void)hipEventDestroy(mk.b);
  }
  m->marks.clear();
}

int e2b_profile_begin(e2b_model* m, int kind) {
  if (!m) return fail(E2B_EINVAL, "null argument");
  if (kind < E2B_KIND_NONE || kind > E2B_KIND_ATTN) return fail(E2B_EINVAL, "bad kind %d", kind);
  drop_marks(m);
  m->prof_kind = kind;
  return E2B_OK;
}

int e2b_profile_read(e2b_model* m, int* launches, double* total_ms, double* total_bytes) {
  if (!m || !launches || !total_ms || !total_bytes) return fail(E2B_EINVAL, "null argument");
  *launches = 0;
  *total_ms = 0;
  *total_bytes = 0;
  for (auto& mk : m->marks) {
    hipError_t e = hipEventSynchronize(mk.b);
    float ms = 0;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, mk.a, mk.b);
    if (e != hipSuccess) {
      drop_marks(m);
      m->prof_kind = 0;
      return hip_fail(e, "profile read");
    }
    *launches += 1;
    *total_ms += ms;
    *total_bytes += mk.bytes;
  }
  drop_marks(m);
  m->prof_kind = 0;
  return E2B_OK;
}

int e2b_check(e2b_model* m, void* d_ws, void* stream) {
  if (!m || !d_ws) return fail(E2B_EINVAL, "null argument");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CK(hipStreamSynchronize(st), "check: stream sync");
  int w[4] = {0, 0, 0, 0};
  CK(hipMemcpy(w, d_ws, sizeof w, hipMemcpyDeviceToHost), "check: read error word");
  if (!w[0]) return E2B_OK;
  const int zero[4] = {0, 0, 0, 0};
  CK(hipMemcpy(d_ws, zero, sizeof zero, hipMemcpyHostToDevice), "check: clear error word");
  return fail(E2B_EDEVICE, "device flagged%s%s%s (token %d, position %d, row %d)",
              (w[0] & e2b::kErrToken) ? " a token outside the vocabulary" : "",
              (w[0] & e2b::kErrPos) ? " a position outside [0, max_ctx)" : "",
              (w[0] & e2b::kErrPage) ? " a cached position on no reserved page" : "", w[1], w[2], w[3]);
}

}  // extern "C"
