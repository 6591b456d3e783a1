// Persistent one-row decode step for CDNA4 (gfx950, wave64).
//
// The same computation as the per-phase kernels (pages: "Porting Gemma 4 E2B
// to SGLang-JAX", Steps 1, 3-5; "One TPU chip, eight agents", The engine) for
// a single sequence, as ONE kernel per step: one block per compute unit runs
// every phase (embedding, per-layer inputs, per layer: QKV, attention,
// combine, O, gate/up, down, PLE gate, PLE projection; lm_head and argmax),
// phases separated by a grid barrier.  At batch 1 each product streams a few
// MB to a few tens of MB, so the step is dominated by per-launch and
// per-phase latency; here a block issues the first weight loads of its next
// product before it waits at the barrier, so the weight stream overlaps the
// synchronisation instead of following it.
//
// Coherence inside one launch: every region another block reads later is
// written once per launch (a per-layer slab) with agent-coherent stores, and
// read only after the barrier that follows all its writes, so no cache can
// hold a stale copy.  The barrier waits for the block's stores to complete,
// then counts arrivals on 64-bit monotonic tickets (per group of blocks, then
// overall); a wait that does not finish within a bound flags the device
// error word and every block leaves the kernel, so a missing block cannot
// hang the device.
#include "dev_common.h"

#include <hip/hip_ext.h>

#include <type_traits>

namespace e2b {

constexpr int kStepThreads = 256;
constexpr long kSpinLimit = 1L << 20;  // barrier polls before giving up (about a second)
constexpr int kPF = 12;                // prefetched weight fragments per lane

__device__ __forceinline__ unsigned long long ld_c64(unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier; false (error word flagged) if the grid did not arrive in time.
__device__ bool grid_sync(unsigned long long* bar, int* err) {
  __shared__ int ok;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    ok = 1;
    const int G = gridDim.x, ng = G < 8 ? G : 8, grp = blockIdx.x % ng;
    const unsigned long long gsize = (G - grp + ng - 1) / ng;
    unsigned long long* gc = bar + 8 * (1 + grp);  // one 64-byte line per counter
    const unsigned long long tk =
        __hip_atomic_fetch_add(gc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long inst = tk / gsize;  // which barrier (since the counters started)
    if (tk % gsize == gsize - 1)
      __hip_atomic_fetch_add(bar, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long target = (inst + 1) * (unsigned long long)ng;
    long s = 0;
    while (ld_c64(bar) < target) {
      if (++s > kSpinLimit) {
        atomicOr(err, kErrSync);
        ok = 0;
        break;
      }
    }
  }
  __syncthreads();
  return ok != 0;
}

// ------------------------------------------------------------ products
// rows per unit (U) as the per-phase matvec kernels choose them
template <int WQ, int KS>
struct UOf {
  static constexpr int v = KS == 2048 ? 2 : (KS == 1536 ? (WQ ? 2 : 4) : 4);
};

struct PF {
  uint4 w[kPF];
  float s[kPF];
};

// The product's virtual blocks (column block, K slice) on the grid: nks
// slices of G / nks column blocks each; blocks past them sit out.
struct VB {
  int bxi, bx, ks, active;
};
__device__ __forceinline__ VB vblock(int K, int KS) {
  const int nks = K / KS, G = gridDim.x;
  VB v;
  v.bx = G / nks < 1 ? 1 : G / nks;
  v.active = blockIdx.x < v.bx * nks;
  v.bxi = blockIdx.x % v.bx;
  v.ks = blockIdx.x / v.bx;
  return v;
}

// The first batch of the block's weight fragments for a product (the loads
// the product itself would issue first), into pf.
template <int WQ, int KS>
__device__ __forceinline__ void gemv_prefetch(const Lin& W, const VB& v, PF& pf) {
  using Y = Lay<WQ, KS>;
  constexpr int U = UOf<WQ, KS>::v;
  static_assert(U * Y::C <= kPF, "prefetch slots");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ls = lane % Y::S, rsub = lane / Y::S;
  const int NU = (W.N + Y::RPL - 1) / Y::RPL, stride = v.bx * 4;
  const int u0 = v.bxi * 4 + wave;
  const size_t ldq = (size_t)W.K / 8, lds = (size_t)W.K / 32;
#pragma unroll
  for (int uu = 0; uu < U; ++uu) {
    const int u = u0 + uu * stride, n = u * Y::RPL + rsub;
    const bool ok = v.active && u < NU && n < W.N;
#pragma unroll
    for (int c = 0; c < Y::C; ++c) {
      uint4 w = make_uint4(0, 0, 0, 0);
      float sc = 0.f;
      if (ok) {
        if (WQ) {
          const int g = ls + Y::S * c;
          w = *reinterpret_cast<const uint4*>(W.q + (size_t)n * ldq + (size_t)v.ks * (KS / 8) + 4 * g);
          sc = bf2f(W.s[(size_t)n * lds + (size_t)v.ks * Y::G + g]);
        } else {
          w = *reinterpret_cast<const uint4*>(W.w + (size_t)n * W.K + (size_t)v.ks * KS + 512 * c +
                                              8 * ls);
        }
      }
      pf.w[uu * Y::C + c] = w;
      pf.s[uu * Y::C + c] = sc;
    }
  }
}

// The block's share of y = W x (one row): the matvec kernel's arithmetic,
// with its first batch of weights taken from pf, outputs stored coherently
// (y[ks][N]) or, with ARGMAX, per-block (max, lowest index) candidates.
template <int WQ, int KS, bool ARGMAX>
__device__ void gemv_step(const Lin& W, const Prologue& pro, const VB& v, const PF& pf, float* y,
                          float* cand_v, int* cand_i, float* logits, float* smem) {
  if (!v.active) return;
  using Y = Lay<WQ, KS>;
  constexpr int U = UOf<WQ, KS>::v;
  float* xs = smem;
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem + KS);
  float* red = smem + KS + Packed<WQ, KS>::words;
  const int ks = v.ks, K = W.K, N = W.N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ls = lane % Y::S, rsub = lane / Y::S;
  const int NU = (N + Y::RPL - 1) / Y::RPL;
  const int stride = v.bx * 4;
  const size_t ldq = (size_t)K / 8, lds = (size_t)K / 32;

  struct Batch {
    uint4 wv[U][Y::C];
    float sc[U][Y::C];
    int n[U];
  };
  auto load_batch = [&](Batch& B, int u0) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int u = u0 + uu * stride;
      B.n[uu] = u * Y::RPL + rsub;
      const bool ok = (u < NU) && (B.n[uu] < N);
#pragma unroll
      for (int c = 0; c < Y::C; ++c) {
        B.wv[uu][c] = make_uint4(0, 0, 0, 0);
        B.sc[uu][c] = 0.f;
        if (ok) {
          if (WQ) {
            const int g = ls + Y::S * c;
            B.wv[uu][c] = *reinterpret_cast<const uint4*>(W.q + (size_t)B.n[uu] * ldq +
                                                          (size_t)ks * (KS / 8) + 4 * g);
            B.sc[uu][c] = bf2f(W.s[(size_t)B.n[uu] * lds + (size_t)ks * Y::G + g]);
          } else {
            B.wv[uu][c] = *reinterpret_cast<const uint4*>(W.w + (size_t)B.n[uu] * K +
                                                          (size_t)ks * KS + 512 * c + 8 * ls);
          }
        }
      }
    }
  };

  PrologueRegs<KS> pr;
  pr.template load<true>(pro, 1, 0, ks * KS, K);
  int u0 = v.bxi * 4 + wave;
  Batch A, Bq;
#pragma unroll
  for (int uu = 0; uu < U; ++uu) {
    A.n[uu] = (u0 + uu * stride) * Y::RPL + rsub;
#pragma unroll
    for (int c = 0; c < Y::C; ++c) {
      A.wv[uu][c] = pf.w[uu * Y::C + c];
      A.sc[uu][c] = pf.s[uu * Y::C + c];
    }
  }
  pr.template finish<true>(pro, 0, K, xs, red, v.bxi == 0 && v.ks == 0);
  pack_x<WQ, KS>(xs, xp);

  uint32_t xh[Y::NP], xl[Y::NP];
  float gsum[Y::C];
#pragma unroll
  for (int c = 0; c < Y::C; ++c) {
    if (WQ) {
      const uint4* src = reinterpret_cast<const uint4*>(xp + (ls + Y::S * c) * Packed<WQ, KS>::kWordsW4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 h4 = src[q], l4 = src[4 + q];
        xh[c * 16 + 4 * q + 0] = h4.x; xh[c * 16 + 4 * q + 1] = h4.y;
        xh[c * 16 + 4 * q + 2] = h4.z; xh[c * 16 + 4 * q + 3] = h4.w;
        xl[c * 16 + 4 * q + 0] = l4.x; xl[c * 16 + 4 * q + 1] = l4.y;
        xl[c * 16 + 4 * q + 2] = l4.z; xl[c * 16 + 4 * q + 3] = l4.w;
      }
      gsum[c] = __uint_as_float(xp[(ls + Y::S * c) * Packed<WQ, KS>::kWordsW4 + 32]);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(xp + (c * Y::S + ls) * 8);
      const uint4 h4 = src[0], l4 = src[1];
      xh[c * 4 + 0] = h4.x; xh[c * 4 + 1] = h4.y; xh[c * 4 + 2] = h4.z; xh[c * 4 + 3] = h4.w;
      xl[c * 4 + 0] = l4.x; xl[c * 4 + 1] = l4.y; xl[c * 4 + 2] = l4.z; xl[c * 4 + 3] = l4.w;
      gsum[c] = 0.f;
    }
  }

  float best = -FLT_MAX;
  int bidx = 0x7FFFFFFF;
  auto reduce_batch = [&](const Batch& B, int ub) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < Y::C; ++c) {
        const uint32_t w4[4] = {B.wv[uu][c].x, B.wv[uu][c].y, B.wv[uu][c].z, B.wv[uu][c].w};
        if (WQ) {
          float s_ = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = w4[j] & 0x0F0F0F0Fu, hi = (w4[j] >> 4) & 0x0F0F0F0Fu;
            const uint32_t p0 = __builtin_amdgcn_perm(0x43434343u, lo, 0x04020400u);  // codes 0, 4
            const uint32_t p1 = __builtin_amdgcn_perm(0x43434343u, hi, 0x04020400u);  // codes 1, 5
            const uint32_t p2 = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030401u);  // codes 2, 6
            const uint32_t p3 = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030401u);  // codes 3, 7
            s_ = dot2(p0, xh[c * 16 + j * 4 + 0], s_);
            s_ = dot2(p0, xl[c * 16 + j * 4 + 0], s_);
            s_ = dot2(p1, xh[c * 16 + j * 4 + 1], s_);
            s_ = dot2(p1, xl[c * 16 + j * 4 + 1], s_);
            s_ = dot2(p2, xh[c * 16 + j * 4 + 2], s_);
            s_ = dot2(p2, xl[c * 16 + j * 4 + 2], s_);
            s_ = dot2(p3, xh[c * 16 + j * 4 + 3], s_);
            s_ = dot2(p3, xl[c * 16 + j * 4 + 3], s_);
          }
          acc = fmaf(B.sc[uu][c], fmaf(-136.0f, gsum[c], s_), acc);  // as the per-phase kernel
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc = dot2(w4[j], xh[c * 4 + j], acc);
            acc = dot2(w4[j], xl[c * 4 + j], acc);
          }
        }
      }
      acc = lanes_sum<Y::S>(acc);
      const int u = ub + uu * stride;
      const int nn = B.n[uu];
      if (ls == 0 && u < NU && nn < N) {
        if (ARGMAX) {
          if (logits) logits[nn] = acc;
          if (acc > best || (acc == best && nn < bidx)) {
            best = acc;
            bidx = nn;
          }
        } else {
          st32<true>(y + (size_t)ks * N + nn, acc);
        }
      }
    }
  };
  while (u0 < NU) {
    const int u1 = u0 + stride * U;
    if (u1 < NU) load_batch(Bq, u1);
    reduce_batch(A, u0);
    if (u1 >= NU) break;
    const int u2 = u1 + stride * U;
    if (u2 < NU) load_batch(A, u2);
    reduce_batch(Bq, u1);
    u0 = u2;
  }

  if (ARGMAX) {
    argmax_lanes<64>(best, bidx);
    int* redi = reinterpret_cast<int*>(red + 8);
    __syncthreads();
    if (lane == 0) {
      red[wave] = best;
      redi[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = red[0];
      int bi = redi[0];
      for (int w = 1; w < 4; ++w)
        if (red[w] > bv || (red[w] == bv && redi[w] < bi)) {
          bv = red[w];
          bi = redi[w];
        }
      st32<true>(cand_v + v.bxi, bv);
      st32i<true>(cand_i + v.bxi, bi);
    }
  }
}

template <int WQ, int KS>
__device__ __forceinline__ void prefetch(const Lin& W, PF& pf) {
  gemv_prefetch<WQ, KS>(W, vblock(W.K, KS), pf);
}
template <int WQ, int KS, bool ARGMAX = false>
__device__ __forceinline__ void product(const Lin& W, const Prologue& pr, const PF& pf, float* y,
                                        float* smem, float* cv = nullptr, int* ci = nullptr,
                                        float* logits = nullptr) {
  gemv_step<WQ, KS, ARGMAX>(W, pr, vblock(W.K, KS), pf, y, cv, ci, logits, smem);
}

// ------------------------------------------------------------ the step
// KH: K slice of the products over the hidden size (= H); KOS / KOF: of the
// O product in sliding / full layers; KD: of the down product; KP: of the
// per-layer projection (= P).
template <int WQ, int KH, int KOS, int KOF, int KD, int KP, int HDS, int HDF>
__global__ __launch_bounds__(kStepThreads) void k_step1(StepArgs a) {
  extern __shared__ float smem[];
  const int t = threadIdx.x, b = blockIdx.x, G = gridDim.x;
  float* S = a.slab;
  const int H = a.H, P = a.P, L = a.L, LP = L * P;
  PF pf;
  int ntr = 0;
  auto mark = [&]() {
    if (a.trace && b == 0 && t == 0) a.trace[ntr] = __builtin_amdgcn_s_memrealtime();
    ++ntr;
  };
  mark();

  // ---- token / position checks, embedding, per-layer table row, RoPE angles
  int tok = a.tokens[0];
  const int pos_raw = a.positions[0];
  if (tok < 0 || tok >= a.V) {
    if (b == 0 && t == 0) {
      atomicOr(a.err, kErrToken);
      atomicExch(a.err + 1, tok);
      atomicExch(a.err + 3, 0);
    }
    tok = 0;
  }
  if ((pos_raw < 0 || pos_raw >= a.max_ctx) && b == 0 && t == 0) {
    atomicOr(a.err, kErrPos);
    atomicExch(a.err + 2, pos_raw);
    atomicExch(a.err + 3, 0);
  }
  const int pos = pos_raw < 0 ? 0 : (pos_raw >= a.max_ctx ? a.max_ctx - 1 : pos_raw);
  {
    const int nr = a.hd_s / 2 + a.hd_f / 2;
    for (int i = b * kStepThreads + t; i < H + LP + nr; i += G * kStepThreads) {
      if (i < H) {
        st32<true>(S + a.e + i, bf2f(a.embed[(size_t)tok * H + i]) * a.sqrtH);
      } else if (i < H + LP) {
        const int k = i - H;
        st32<true>(S + a.tokple + k, bf2f(a.ple[(size_t)tok * LP + k]) * a.sqrtP);
      } else {  // cos then sin, hd/2 each; sliding first, then full (from fp64)
        const int k0 = i - H - LP;
        const bool full = k0 >= a.hd_s / 2;
        const int k = full ? k0 - a.hd_s / 2 : k0;
        const int half = full ? a.hd_f / 2 : a.hd_s / 2;
        float* base = S + a.rope + (full ? a.hd_s : 0);
        double sd, cd;
        sincos((double)pos * (full ? a.inv_f : a.inv_s)[k], &sd, &cd);
        st32<true>(base + k, (float)cd);
        st32<true>(base + half + k, (float)sd);
      }
    }
  }
  prefetch<WQ, KH>(a.plmp, pf);
  if (!grid_sync(a.bar, a.err)) return;
    mark();

  // ---- per-layer model projection u = W_plmp e
  {
    Prologue pr;
    pr.kind = kPlain;
    pr.a = S + a.e;
    pr.lda = H;
    product<WQ, KH>(a.plmp, pr, pf, S + a.u, smem);
  }
  prefetch<WQ, KH>(a.layers[0].qkv, pf);
  if (!grid_sync(a.bar, a.err)) return;
    mark();

  Rows R;
  R.tokens = a.tokens;
  R.positions = a.positions;
  R.n = 1;
  R.max_ctx = a.max_ctx;
  R.vocab = a.V;
  for (int l = 0; l < L; ++l) {
    const StepLayer& y = a.layers[l];
    const StepLayer* prev = l ? &a.layers[l - 1] : nullptr;
    const size_t hcur = l ? y.hq : a.e;  // residual stream entering the layer
    {  // QKV: the previous layer's per-layer-input residual and scalar, input norm
      Prologue pr;
      pr.kind = kResNorm;
      pr.a = S + (l ? prev->h2 : a.e);
      pr.d = l ? S + prev->ppo : nullptr;
      pr.nd = 1;
      pr.d_pstride = H;
      pr.gd = l ? prev->g_pple : nullptr;
      pr.scalar = l ? prev->scalar : nullptr;
      pr.gx = y.g_in;
      pr.h_out = S + y.hq;
      pr.eps = a.eps;
      product<WQ, KH>(y.qkv, pr, pf, S + y.qkv_out, smem);
    }
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    AttnArgs aa;
    aa.qkv = S + y.qkv_out;
    aa.gq = y.g_q;
    aa.gk = y.g_k;
    aa.kc = y.kc;
    aa.vc = y.vc;
    aa.kc_own = y.kc_own;
    aa.vc_own = y.vc_own;
    aa.part = S + y.part;
    aa.out = S + y.attn;
    aa.nq = a.nq;
    aa.hd = y.hd;
    aa.window = y.full ? 0 : a.window;
    aa.chunk = y.chunk;
    aa.nchunk = y.nchunk;
    aa.owns = y.owns;
    aa.rope = S + a.rope;
    aa.rope_ld = a.hd_s + a.hd_f;
    aa.rope_off = y.full ? a.hd_s : 0;
    aa.eps = a.eps;
    if (b < y.nchunk) {
      if (y.full) attn_chunk<HDF, true>(R, aa, b, 0);
      else attn_chunk<HDS, true>(R, aa, b, 0);
    } else if (l == 0 && b < y.nchunk + L) {  // per-layer inputs, one layer slice per block
      __shared__ float sh[4];
      const int ls = b - y.nchunk;
      float v = 0.f;
      if (t < P) v = ld32<true>(S + a.u + (size_t)ls * P + t) * a.inv_sqrtH;
      const float rr = rsqrtf(block_sum<kStepThreads>(v * v, sh) / (float)P + a.eps);
      if (t < P)
        st32<true>(S + a.pli + (size_t)ls * P + t,
                   fmaf(v * rr, bf2f(a.g_plpn[t]), ld32<true>(S + a.tokple + (size_t)ls * P + t)) *
                       0.70710678118654752f);
    }
    if (y.full) prefetch<WQ, KOF>(y.o, pf);
    else prefetch<WQ, KOS>(y.o, pf);
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    if (b < a.nq) attn_combine<true>(aa, 0, b);
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    {  // O
      Prologue pr;
      pr.kind = kPlain;
      pr.a = S + y.attn;
      pr.lda = a.nq * y.hd;
      if (y.full) product<WQ, KOF>(y.o, pr, pf, S + y.oo, smem);
      else product<WQ, KOS>(y.o, pr, pf, S + y.oo, smem);
    }
    prefetch<WQ, KH>(y.gu, pf);
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    {  // post-attention norm + residual, pre-FFN norm, gate/up
      Prologue pr;
      pr.kind = kResNorm;
      pr.a = S + hcur;
      pr.d = S + y.oo;
      pr.nd = y.o.K / (y.full ? KOF : KOS);
      pr.d_pstride = H;
      pr.gd = y.g_pa;
      pr.gx = y.g_pf;
      pr.h_out = S + y.h1;
      pr.eps = a.eps;
      product<WQ, KH>(y.gu, pr, pf, S + y.gu_out, smem);
    }
    prefetch<WQ, KD>(y.down, pf);
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    {  // GeGLU, down
      Prologue pr;
      pr.kind = kGeglu;
      pr.a = S + y.gu_out;
      pr.lda = 2 * y.I;
      product<WQ, KD>(y.down, pr, pf, S + y.dn, smem);
    }
    prefetch<WQ, KH>(y.pg, pf);
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    {  // post-FFN norm + residual, per-layer input gate
      Prologue pr;
      pr.kind = kRes;
      pr.a = S + y.h1;
      pr.d = S + y.dn;
      pr.nd = y.I / KD;
      pr.d_pstride = H;
      pr.gd = y.g_ff;
      pr.h_out = S + y.h2;
      pr.eps = a.eps;
      product<WQ, KH>(y.pg, pr, pf, S + y.pg_out, smem);
    }
    prefetch<WQ, KP>(y.pp, pf);
    if (!grid_sync(a.bar, a.err)) return;
    mark();

    {  // gelu(gate) * pli[l], per-layer projection
      Prologue pr;
      pr.kind = kPleGate;
      pr.a = S + y.pg_out;
      pr.lda = P;
      pr.pli = S + a.pli + (size_t)l * P;
      pr.pli_ld = LP;
      product<WQ, KP>(y.pp, pr, pf, S + y.ppo, smem);
    }
    if (l + 1 < L) prefetch<WQ, KH>(a.layers[l + 1].qkv, pf);
    else prefetch<0, KH>(a.lm, pf);
    if (!grid_sync(a.bar, a.err)) return;
    mark();
  }

  {  // final norm (after the last layer's per-layer-input residual), tied lm_head, argmax candidates
    const StepLayer& y = a.layers[L - 1];
    Prologue pr;
    pr.kind = kResNorm;
    pr.a = S + y.h2;
    pr.d = S + y.ppo;
    pr.nd = 1;
    pr.d_pstride = H;
    pr.gd = y.g_pple;
    pr.scalar = y.scalar;
    pr.gx = a.g_final;
    pr.h_out = S + a.hfin;
    pr.eps = a.eps;
    product<0, KH, true>(a.lm, pr, pf, nullptr, smem, S + a.cand_v,
                         reinterpret_cast<int*>(S + a.cand_i), a.logits);
  }
  if (!grid_sync(a.bar, a.err)) return;
    mark();
  if (b == 0) {  // argmax over the blocks' candidates (lowest index on ties)
    __shared__ float sv[4];
    __shared__ int si[4];
    const VB v = vblock(a.lm.K, KH);
    const float* cv = S + a.cand_v;
    const int* ci = reinterpret_cast<const int*>(S + a.cand_i);
    float best = -FLT_MAX;
    int bi = 0x7FFFFFFF;
    for (int i = t; i < v.bx; i += kStepThreads) {
      const float x = ld32<true>(cv + i);
      const int xi = ld32i<true>(ci + i);
      if (x > best || (x == best && xi < bi)) {
        best = x;
        bi = xi;
      }
    }
    argmax_lanes<64>(best, bi);
    if ((t & 63) == 0) {
      sv[t >> 6] = best;
      si[t >> 6] = bi;
    }
    __syncthreads();
    if (t == 0) {
      for (int w = 1; w < 4; ++w)
        if (sv[w] > best || (sv[w] == best && si[w] < bi)) {
          best = sv[w];
          bi = si[w];
        }
      a.argmax[0] = bi == 0x7FFFFFFF ? 0 : bi;
    }
  }
}

// ------------------------------------------------------------ host side
namespace {
template <int WQ, int KS>
constexpr int gemv_smem_floats() {
  return KS + Packed<WQ, KS>::words + 32;
}
template <int WQ, int KH, int KOS, int KOF, int KD, int KP>
constexpr size_t step_smem() {
  const int v[6] = {gemv_smem_floats<WQ, KH>(), gemv_smem_floats<WQ, KOS>(),
                    gemv_smem_floats<WQ, KOF>(), gemv_smem_floats<WQ, KD>(),
                    gemv_smem_floats<WQ, KP>(), gemv_smem_floats<0, KH>()};
  int m = 0;
  for (int i = 0; i < 6; ++i) m = v[i] > m ? v[i] : m;
  return (size_t)m * sizeof(float);
}

// variant 0: E2B widths; variant 1: the toy models' widths
template <int WQ, int V>
struct StepK;
template <int WQ>
struct StepK<WQ, 0> {
  static constexpr auto fn = k_step1<WQ, 1536, 2048, 2048, 2048, 256, 256, 512>;
  static constexpr size_t smem = step_smem<WQ, 1536, 2048, 2048, 2048, 256>();
};
template <int WQ>
struct StepK<WQ, 1> {
  static constexpr auto fn = k_step1<WQ, 256, 128, 256, 512, 32, 64, 128>;
  static constexpr size_t smem = step_smem<WQ, 256, 128, 256, 512, 32>();
};

template <int WQ, int V>
int grid_of() {
  int dev = 0, cus = 0, nb = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(StepK<WQ, V>::fn),
                                                   kStepThreads, StepK<WQ, V>::smem) != hipSuccess)
    return 0;
  return nb >= 1 ? cus : 0;
}
}  // namespace

int step1_variant(int H, int P, int nq, int hd_s, int hd_f, int I0, int I1) {
  if (nq > kMaxHeads) return -1;
  if (H == 1536 && P == 256 && nq * hd_s == 2048 && nq * hd_f == 4096 && hd_s == 256 && hd_f == 512 &&
      I0 % 2048 == 0 && I1 % 2048 == 0)
    return 0;
  if (H == 256 && P == 32 && nq * hd_s == 128 && nq * hd_f == 256 && hd_s == 64 && hd_f == 128 &&
      I0 % 512 == 0 && I1 % 512 == 0 && I0 <= 2048 * 8 && I1 <= 2048 * 8)
    return 1;
  return -1;
}

int step1_grid(int variant, int quant) {
  if (variant == 0) return quant ? grid_of<1, 0>() : grid_of<0, 0>();
  if (variant == 1) return quant ? grid_of<1, 1>() : grid_of<0, 1>();
  return 0;
}

size_t step1_barrier_bytes() { return 9 * 64; }

namespace {
template <int WQ, int V>
hipError_t launch_v(const StepArgs& a, int grid, hipStream_t st) {
  auto fn = StepK<WQ, V>::fn;
  const size_t sm = StepK<WQ, V>::smem;
  hipEvent_t ea = nullptr, eb = nullptr;
  if (take_launch_events(&ea, &eb))
    hipExtLaunchKernelGGL(fn, dim3(grid), dim3(kStepThreads), sm, st, ea, eb, 0, a);
  else
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kStepThreads), sm, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_step1(int variant, int quant, const StepArgs& a, int grid, hipStream_t st) {
  if (grid < 1) return hipErrorInvalidValue;
  if (variant == 0) return quant ? launch_v<1, 0>(a, grid, st) : launch_v<0, 0>(a, grid, st);
  if (variant == 1) return quant ? launch_v<1, 1>(a, grid, st) : launch_v<0, 1>(a, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace e2b
