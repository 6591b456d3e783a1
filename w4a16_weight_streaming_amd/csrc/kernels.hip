// HIP kernels of the decode step for CDNA4 (gfx950, wave64).
//
// Step structure (pages: "Porting Gemma 4 E2B to SGLang-JAX", Steps 1, 3-5;
// "One TPU chip, eight agents", The engine): embedding and per-layer inputs,
// then per layer a QKV product, head norms + RoPE + in-place K/V write,
// decode attention over the source layer's cache, O product, GeGLU MLP,
// per-layer-input mixing; finally the tied lm_head with greedy argmax.
//
// Matrix-vector products stream each weight byte from HBM once.  The fp32
// input row is split into a bf16 high part and a bf16 low part (x = hi + lo to
// ~17 significant bits) held in registers; products use v_dot2_f32_bf16 with
// fp32 accumulation.  W4A16 codes are unpacked in registers by OR-ing a nibble
// into the mantissa of bf16 128.0 (giving 128 + c exactly), so one group of 32
// contributes  s * (sum (128 + c_k) x_k - 136 * sum x_k) = s * sum (c_k - 8) x_k,
// with the group scale s applied in fp32 (exact decode: (c - 8) * s needs at
// most 12 significant bits).
#include "e2b_internal.h"

#include <float.h>
#include <math.h>

namespace e2b {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float((b & 0xFFFFu) << 16); }

__device__ __forceinline__ uint32_t f2bf(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a block of NT threads, same value returned to every thread.
// `sh` needs NT/64 floats; the leading barrier makes back-to-back calls safe.
template <int NT>
__device__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += sh[i];
  return s;
}

__device__ __forceinline__ int row_pos(const Rows& R, int r) {
  return R.positions ? R.positions[r] : R.pos0 + r;
}
__device__ __forceinline__ int clamp_pos(const Rows& R, int p) {
  return p < 0 ? 0 : (p >= R.max_ctx ? R.max_ctx - 1 : p);
}
__device__ __forceinline__ int row_seq(const Rows& R, int r) { return R.seq0 + r * R.seq_stride; }

// ---------------------------------------------------------------- embedding
// h[r] = E[tok] * sqrt(H);  tokple[r] = E_ple[tok] * sqrt(P)
__global__ __launch_bounds__(256) void k_embed(Rows R, const uint16_t* __restrict__ E,
                                               const uint16_t* __restrict__ Eple, int H, int LP,
                                               float sqrtH, float sqrtP, float* __restrict__ h,
                                               float* __restrict__ tokple, int* err) {
  const int r = blockIdx.x;
  int tok = R.tokens[r];
  if (tok < 0 || tok >= R.vocab) {
    if (threadIdx.x == 0) {
      atomicOr(err, kErrToken);
      atomicExch(err + 1, tok);
      atomicExch(err + 3, r);
    }
    tok = 0;
  }
  const int pos = row_pos(R, r);
  if ((pos < 0 || pos >= R.max_ctx) && threadIdx.x == 0) {
    atomicOr(err, kErrPos);
    atomicExch(err + 2, pos);
    atomicExch(err + 3, r);
  }
  const uint16_t* e = E + (size_t)tok * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) h[(size_t)r * H + i] = bf2f(e[i]) * sqrtH;
  const uint16_t* t = Eple + (size_t)tok * LP;
  for (int i = threadIdx.x; i < LP; i += blockDim.x)
    tokple[(size_t)r * LP + i] = bf2f(t[i]) * sqrtP;
}

hipError_t launch_embed(const Rows& R, const uint16_t* E, const uint16_t* Eple, int H, int LP,
                        float sqrtH, float sqrtP, float* h, float* tokple, int* err,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_embed, dim3(R.n), dim3(256), 0, st, R, E, Eple, H, LP, sqrtH, sqrtP, h,
                     tokple, err);
  return hipGetLastError();
}

// ------------------------------------------------------ per-layer input finish
// pli[r][l] = (rms(u[r][l] * H^-1/2) * g + tokple[r][l]) * 2^-1/2
__global__ __launch_bounds__(256) void k_ple_finish(int LP, int P, const float* __restrict__ u,
                                                    const float* __restrict__ tokple,
                                                    const uint16_t* __restrict__ g, float inv_sqrtH,
                                                    float eps, float* __restrict__ pli) {
  __shared__ float sh[4];
  const int r = blockIdx.x, l = blockIdx.y, i = threadIdx.x;
  const size_t base = (size_t)r * LP + (size_t)l * P;
  float v = (i < P) ? u[base + i] * inv_sqrtH : 0.f;
  const float ss = block_sum<256>(v * v, sh);
  const float rr = rsqrtf(ss / (float)P + eps);
  if (i < P) pli[base + i] = (v * rr * bf2f(g[i]) + tokple[base + i]) * 0.70710678118654752f;
}

hipError_t launch_ple_finish(const Rows& R, const float* u, const float* tokple,
                             const uint16_t* g, int L, int P, float inv_sqrtH, float eps,
                             float* pli, hipStream_t st) {
  if (P > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_ple_finish, dim3(R.n, L), dim3(256), 0, st, L * P, P, u, tokple, g,
                     inv_sqrtH, eps, pli);
  return hipGetLastError();
}

// ------------------------------------------------------- matrix-vector product
// Lane layout for one K slice of KS elements (a 16-byte load per lane):
//  bf16  : a lane covers 8 consecutive k per 512-wide chunk; S lanes per row.
//  W4A16 : a lane covers whole 32-groups (16 bytes = one group); S lanes per row.
// RPL = 64 / S rows are covered by one wave-wide load ("unit"); C loads per unit.
template <int WQ, int KS>
struct Lay {
  static constexpr int G = KS / 32;
  static constexpr int S =
      WQ ? ((G % 64 == 0) ? 64 : ((G % 16 == 0) ? 16 : G)) : (KS / 8 < 64 ? KS / 8 : 64);
  static constexpr int RPL = 64 / S;
  static constexpr int C = WQ ? G / S : (KS >= 512 ? KS / 512 : 1);
  static constexpr int NP = WQ ? C * 16 : C * 4;  // bf16 pairs of x per lane
  static_assert(64 % S == 0, "lanes per row must divide the wave");
};

// Build the block's fp32 input slice xs[0..KS) for row b (slice k0..k0+KS).
template <int KS>
__device__ void build_x(const Prologue& p, int rows, int b, int k0, int K, float* xs,
                        float* red) {
  const int t = threadIdx.x;
  if (p.kind == kPlain) {
    for (int i = t; i < KS; i += kGemvThreads) xs[i] = p.a[(size_t)b * p.lda + k0 + i];
  } else if (p.kind == kGeglu) {
    for (int i = t; i < KS; i += kGemvThreads) {
      const float g = p.a[(size_t)b * p.lda + k0 + i];
      const float u = p.a[(size_t)b * p.lda + K + k0 + i];
      xs[i] = gelu_tanh(g) * u;
    }
  } else if (p.kind == kPleGate) {
    for (int i = t; i < KS; i += kGemvThreads)
      xs[i] = gelu_tanh(p.a[(size_t)b * p.lda + k0 + i]) * p.pli[(size_t)b * p.pli_ld + k0 + i];
  } else {  // kRes / kResNorm: KS == K == hidden size (host guarantees)
    constexpr int PT = (KS + kGemvThreads - 1) / kGemvThreads;
    float dv[PT];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = t + j * kGemvThreads;
      float s = 0.f;
      if (i < KS && p.d)
        for (int q = 0; q < p.nd; ++q) s += p.d[((size_t)q * rows + b) * K + i];
      dv[j] = s;
      ss += s * s;
    }
    float rd = 0.f;
    if (p.d) rd = rsqrtf(block_sum<kGemvThreads>(ss, red) / (float)K + p.eps);
    const float sc = p.scalar ? bf2f(p.scalar[0]) : 1.0f;
    const bool store = p.d && p.h_out && blockIdx.x == 0 && blockIdx.y == 0;
    float hs = 0.f;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = t + j * kGemvThreads;
      if (i < KS) {
        float hn = p.a[(size_t)b * K + i];
        if (p.d) hn = (hn + dv[j] * rd * bf2f(p.gd[i])) * sc;
        xs[i] = hn;
        hs += hn * hn;
        if (store) p.h_out[(size_t)b * K + i] = hn;
      }
    }
    if (p.kind == kResNorm) {
      const float rh = rsqrtf(block_sum<kGemvThreads>(hs, red) / (float)K + p.eps);
      for (int i = t; i < KS; i += kGemvThreads) xs[i] = xs[i] * rh * bf2f(p.gx[i]);
    }
  }
  __syncthreads();
}

// split an fp32 pair into bf16 hi pair and bf16 lo pair
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo,
                                           float& sum) {
  const uint32_t ha = f2bf(a), hb = f2bf(b);
  const float ra = a - bf2f(ha), rb = b - bf2f(hb);
  const uint32_t la = f2bf(ra), lb = f2bf(rb);
  hi = ha | (hb << 16);
  lo = la | (lb << 16);
  sum += (bf2f(ha) + bf2f(la)) + (bf2f(hb) + bf2f(lb));
}

// TAG only names the kernel after the matrix it streams (QKV, O, gate/up, ...)
// so that per-kernel profiles separate them; the code is identical.
template <int WQ, int KS, int U, int TAG>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(Lin W, int rows, Prologue pro,
                                                       Epilogue epi) {
  using Y = Lay<WQ, KS>;
  extern __shared__ float smem[];
  float* xs = smem;       // KS
  float* red = smem + KS; // 8 floats of reduction scratch + 16 for argmax
  const int ks = blockIdx.y, b = blockIdx.z;
  const int K = W.K, N = W.N;
  build_x<KS>(pro, rows, b, ks * KS, K, xs, red);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ls = lane % Y::S, rsub = lane / Y::S;

  // x of this lane as bf16 hi/lo pairs (and group sums for W4A16)
  uint32_t xh[Y::NP], xl[Y::NP];
  float gsum[Y::C];
#pragma unroll
  for (int c = 0; c < Y::C; ++c) {
    gsum[c] = 0.f;
    if (WQ) {
      const int g = ls + Y::S * c;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = 32 * g + 8 * j + i;  // pair (k, k + 4): matches the nibble unpack
          split_pair(xs[k], xs[k + 4], xh[c * 16 + j * 4 + i], xl[c * 16 + j * 4 + i], gsum[c]);
        }
    } else {
      const int k0 = 512 * c + 8 * ls;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float dummy = 0.f;
        split_pair(xs[k0 + 2 * j], xs[k0 + 2 * j + 1], xh[c * 4 + j], xl[c * 4 + j], dummy);
      }
    }
  }

  const int NU = (N + Y::RPL - 1) / Y::RPL;
  const int stride = gridDim.x * 4;
  float best = -FLT_MAX;
  int bidx = 0x7FFFFFFF;
  const size_t ldq = (size_t)K / 8, lds = (size_t)K / 32;

  for (int u0 = blockIdx.x * 4 + wave; u0 < NU; u0 += stride * U) {
    uint4 wv[U][Y::C];
    float sc[U][Y::C];
    int n[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int u = u0 + uu * stride;
      n[uu] = u * Y::RPL + rsub;
      const bool ok = (u < NU) && (n[uu] < N);
#pragma unroll
      for (int c = 0; c < Y::C; ++c) {
        if (ok) {
          if (WQ) {
            const int g = ls + Y::S * c;
            const uint32_t* src = W.q + (size_t)n[uu] * ldq + (size_t)ks * (KS / 8) + 4 * g;
            wv[uu][c] = *reinterpret_cast<const uint4*>(src);
            sc[uu][c] = bf2f(W.s[(size_t)n[uu] * lds + (size_t)ks * Y::G + g]);
          } else {
            const uint16_t* src = W.w + (size_t)n[uu] * K + (size_t)ks * KS + 512 * c + 8 * ls;
            wv[uu][c] = *reinterpret_cast<const uint4*>(src);
            sc[uu][c] = 0.f;
          }
        } else {
          wv[uu][c] = make_uint4(0, 0, 0, 0);
          sc[uu][c] = 0.f;
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < Y::C; ++c) {
        const uint32_t w4[4] = {wv[uu][c].x, wv[uu][c].y, wv[uu][c].z, wv[uu][c].w};
        if (WQ) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t p = ((w4[j] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
              a = dot2(p, xh[c * 16 + j * 4 + i], a);
              a = dot2(p, xl[c * 16 + j * 4 + i], a);
            }
          }
          acc += sc[uu][c] * (a - 136.0f * gsum[c]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc = dot2(w4[j], xh[c * 4 + j], acc);
            acc = dot2(w4[j], xl[c * 4 + j], acc);
          }
        }
      }
#pragma unroll
      for (int o = Y::S / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      const int u = u0 + uu * stride;
      if (ls == 0 && u < NU && n[uu] < N) {
        if (epi.argmax) {
          if (epi.logits) epi.logits[(size_t)b * N + n[uu]] = acc;
          if (acc > best || (acc == best && n[uu] < bidx)) {
            best = acc;
            bidx = n[uu];
          }
        } else {
          epi.y[((size_t)ks * rows + b) * N + n[uu]] = acc;
        }
      }
    }
  }

  if (epi.argmax) {
    // wave reduce (max value, lowest index), then across the 4 waves
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bidx, o, 64);
      if (ov > best || (ov == best && oi < bidx)) {
        best = ov;
        bidx = oi;
      }
    }
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
      epi.cand_val[(size_t)b * gridDim.x + blockIdx.x] = bv;
      epi.cand_idx[(size_t)b * gridDim.x + blockIdx.x] = bi;
    }
  }
}

int gemv_splits(int K) {
  if (K % 2048 == 0) return K / 2048;
  if (K % 1536 == 0) return K / 1536;
  if (K <= 512) return 1;
  if (K % 512 == 0) return K / 512;
  return -1;
}

static int gemv_slice(int K) {
  const int n = gemv_splits(K);
  return n > 0 ? K / n : -1;
}

template <int WQ, int KS, int U, int TAG>
static hipError_t run_gemv(const Lin& W, int rows, const Prologue& pro, const Epilogue& epi,
                           int blocks_hint, int* blocks_out, hipStream_t st) {
  using Y = Lay<WQ, KS>;
  const int nks = W.K / KS;
  const int NU = (W.N + Y::RPL - 1) / Y::RPL;
  int bx = blocks_hint > 0 ? blocks_hint : (NU + 4 * U - 1) / (4 * U);
  if (bx > 1024) bx = 1024;
  if (bx < 1) bx = 1;
  if (blocks_out) *blocks_out = bx;
  const size_t shm = (size_t)KS * sizeof(float) + 32 * sizeof(float);
  hipLaunchKernelGGL((k_gemv<WQ, KS, U, TAG>), dim3(bx, nks, rows), dim3(kGemvThreads), shm, st,
                     W, rows, pro, epi);
  return hipGetLastError();
}

template <int WQ, int TAG>
static hipError_t dispatch_gemv(const Lin& W, int rows, const Prologue& pro,
                                const Epilogue& epi, int blocks_hint, int* bo, hipStream_t st) {
  switch (gemv_slice(W.K)) {
    case 32: return run_gemv<WQ, 32, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 128: return run_gemv<WQ, 128, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 256: return run_gemv<WQ, 256, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 512: return run_gemv<WQ, 512, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 1536: return run_gemv<WQ, 1536, WQ ? 2 : 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 2048: return run_gemv<WQ, 2048, 2, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    default: return hipErrorInvalidValue;
  }
}

template <int WQ>
static hipError_t dispatch_tag(int tag, const Lin& W, int rows, const Prologue& pro,
                               const Epilogue& epi, int blocks_hint, int* bo, hipStream_t st) {
  switch (tag) {
    case kTagQkv: return dispatch_gemv<WQ, kTagQkv>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagO: return dispatch_gemv<WQ, kTagO>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagGateUp: return dispatch_gemv<WQ, kTagGateUp>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagDown: return dispatch_gemv<WQ, kTagDown>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagPleGate: return dispatch_gemv<WQ, kTagPleGate>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagPleProj: return dispatch_gemv<WQ, kTagPleProj>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagPleModel: return dispatch_gemv<WQ, kTagPleModel>(W, rows, pro, epi, blocks_hint, bo, st);
    case kTagLmHead: return dispatch_gemv<WQ, kTagLmHead>(W, rows, pro, epi, blocks_hint, bo, st);
    default: return dispatch_gemv<WQ, kTagOther>(W, rows, pro, epi, blocks_hint, bo, st);
  }
}

hipError_t launch_gemv(int quant, int tag, const Lin& W, int rows, const Prologue& pro,
                       const Epilogue& epi, int blocks_hint, int* blocks_out, hipStream_t st) {
  if (rows < 1 || rows > 65535) return hipErrorInvalidValue;
  if ((pro.kind == kRes || pro.kind == kResNorm) && gemv_slice(W.K) != W.K)
    return hipErrorInvalidValue;
  if (epi.argmax && gemv_splits(W.K) != 1) return hipErrorInvalidValue;
  if (epi.argmax && quant) return hipErrorInvalidValue;  // the tied lm_head is bf16
  if (epi.argmax) return dispatch_gemv<0, kTagLmHead>(W, rows, pro, epi, blocks_hint, blocks_out, st);
  return quant ? dispatch_tag<1>(tag, W, rows, pro, epi, blocks_hint, blocks_out, st)
               : dispatch_tag<0>(tag, W, rows, pro, epi, blocks_hint, blocks_out, st);
}

// ------------------------------------------------ head norms, RoPE, K/V write
// One block per (row, head).  Heads 0..nq-1 are queries; when the layer owns
// its K/V, head nq is the key and nq+1 the value.  Keys and queries: RMS norm
// with gain, then rotate-half RoPE at the logical position; values: RMS norm
// without gain.  K/V go to the cache slot = position, as bf16.
__global__ __launch_bounds__(256) void k_qkv_post(Rows R, QkvPostArgs a) {
  __shared__ float sh[4];
  const int r = blockIdx.x, hh = blockIdx.y, hd = a.hd, half = hd / 2;
  const int pos = clamp_pos(R, row_pos(R, r));
  const int seq = row_seq(R, r);
  const int nh = a.nq + (a.kc ? 2 : 0);
  const float* src = a.qkv + (size_t)r * nh * hd + (size_t)hh * hd;
  const int i = threadIdx.x;
  const bool act = i < half;
  const float x0 = act ? src[i] : 0.f, x1 = act ? src[i + half] : 0.f;
  const float ss = block_sum<256>(x0 * x0 + x1 * x1, sh);
  const float rr = rsqrtf(ss / (float)hd + a.eps);
  if (!act) return;
  const bool is_v = hh == a.nq + 1;
  const uint16_t* g = hh < a.nq ? a.gq : a.gk;
  float y0 = x0 * rr, y1 = x1 * rr;
  if (!is_v) {
    y0 *= bf2f(g[i]);
    y1 *= bf2f(g[i + half]);
    double sn, cs;
    sincos((double)pos * a.inv_freq[i], &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float z0 = y0 * c - y1 * s, z1 = y0 * s + y1 * c;
    y0 = z0;
    y1 = z1;
  }
  if (hh < a.nq) {
    float* q = a.q_out + ((size_t)r * a.nq + hh) * hd;
    q[i] = y0;
    q[i + half] = y1;
  } else {
    uint16_t* dst = (is_v ? a.vc : a.kc) + ((size_t)seq * R.max_ctx + pos) * hd;
    dst[i] = (uint16_t)f2bf(y0);
    dst[i + half] = (uint16_t)f2bf(y1);
  }
}

hipError_t launch_qkv_post(const Rows& R, const QkvPostArgs& a, hipStream_t st) {
  if (a.hd > 512 || a.hd % 2) return hipErrorInvalidValue;
  const int nh = a.nq + (a.kc ? 2 : 0);
  hipLaunchKernelGGL(k_qkv_post, dim3(R.n, nh), dim3(256), 0, st, R, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ decode attention
// Block (chunk c, row r): keys j0..j1-1 of the row's window, all query heads
// against one K/V head.  Key tiles of TK rows are staged in LDS (bf16); an
// online softmax keeps (max, sum, o) per head.  Partial results per chunk go to
// `part`; k_attn_combine merges the chunks of a (row, head).
constexpr int kTK = 16;
constexpr int kMaxHeads = 8;

template <int HD>
__global__ __launch_bounds__(256) void k_attn(Rows R, AttnArgs a) {
  __shared__ float qs[kMaxHeads * HD];
  __shared__ uint16_t ks[kTK * (HD + 2)];
  __shared__ uint16_t vs[kTK * HD];
  __shared__ float p[kMaxHeads * kTK];
  __shared__ float mh[kMaxHeads], lh[kMaxHeads], corr[kMaxHeads];
  constexpr int NO = (kMaxHeads * HD + 255) / 256;
  const int c = blockIdx.x, r = blockIdx.y, t = threadIdx.x, nq = a.nq;
  const int pos = clamp_pos(R, row_pos(R, r));
  const int seq = row_seq(R, r);
  const int lo = a.window ? max(0, pos - a.window + 1) : 0;
  const int j0 = lo + c * a.chunk;
  const int j1 = min(j0 + a.chunk, pos + 1);
  float* part = a.part + ((size_t)r * nq * kMaxChunks + c) * (HD + 2);
  const size_t hstride = (size_t)kMaxChunks * (HD + 2);
  if (j0 >= j1) {
    if (t < nq) {
      part[t * hstride + HD] = -INFINITY;
      part[t * hstride + HD + 1] = 0.f;
    }
    return;
  }
  for (int i = t; i < nq * HD; i += 256) qs[i] = a.q[(size_t)r * nq * HD + i];
  if (t < nq) {
    mh[t] = -INFINITY;
    lh[t] = 0.f;
  }
  float acc[NO];
#pragma unroll
  for (int j = 0; j < NO; ++j) acc[j] = 0.f;
  const uint16_t* kb = a.kc + (size_t)seq * R.max_ctx * HD;
  const uint16_t* vb = a.vc + (size_t)seq * R.max_ctx * HD;
  const float scale = rsqrtf((float)HD);
  for (int jt = j0; jt < j1; jt += kTK) {
    const int nk = min(kTK, j1 - jt);
    __syncthreads();
    for (int i = t; i < nk * HD; i += 256) {
      const int kk = i / HD, d = i % HD;
      ks[kk * (HD + 2) + d] = kb[(size_t)(jt + kk) * HD + d];
      vs[kk * HD + d] = vb[(size_t)(jt + kk) * HD + d];
    }
    __syncthreads();
    for (int idx = t; idx < nq * kTK; idx += 256) {
      const int h = idx / kTK, kk = idx % kTK;
      float s = -INFINITY;
      if (kk < nk) {
        float d0 = 0.f;
        const float* qh = qs + h * HD;
        const uint16_t* kr = ks + kk * (HD + 2);
        for (int d = 0; d < HD; ++d) d0 += qh[d] * bf2f(kr[d]);
        s = d0 * scale;
      }
      p[idx] = s;
    }
    __syncthreads();
    if (t < nq) {
      float mt = -INFINITY;
      for (int kk = 0; kk < nk; ++kk) mt = fmaxf(mt, p[t * kTK + kk]);
      const float mn = fmaxf(mh[t], mt);
      const float cr = (mh[t] == -INFINITY) ? 0.f : expf(mh[t] - mn);
      float sum = 0.f;
      for (int kk = 0; kk < kTK; ++kk) {
        const float e = (kk < nk) ? expf(p[t * kTK + kk] - mn) : 0.f;
        p[t * kTK + kk] = e;
        sum += e;
      }
      lh[t] = lh[t] * cr + sum;
      mh[t] = mn;
      corr[t] = cr;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int o = t + 256 * j;
      if (o < nq * HD) {
        const int h = o / HD, d = o % HD;
        float s = acc[j] * corr[h];
        for (int kk = 0; kk < nk; ++kk) s += p[h * kTK + kk] * bf2f(vs[kk * HD + d]);
        acc[j] = s;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NO; ++j) {
    const int o = t + 256 * j;
    if (o < nq * HD) {
      const int h = o / HD, d = o % HD;
      part[h * hstride + d] = acc[j];
    }
  }
  if (t < nq) {
    part[t * hstride + HD] = mh[t];
    part[t * hstride + HD + 1] = lh[t];
  }
}

// out[r][h*hd + d] = sum_c e^(m_c - M) o_c[d] / sum_c e^(m_c - M) l_c
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, hd = a.hd;
  const size_t hstride = (size_t)kMaxChunks * (hd + 2);
  const float* part = a.part + ((size_t)r * a.nq + h) * hstride;
  float M = -INFINITY;
  for (int c = 0; c < a.nchunk; ++c) {
    const float* pc = part + (size_t)c * (hd + 2);
    if (pc[hd + 1] > 0.f) M = fmaxf(M, pc[hd]);
  }
  float L = 0.f;
  for (int c = 0; c < a.nchunk; ++c) {
    const float* pc = part + (size_t)c * (hd + 2);
    if (pc[hd + 1] > 0.f) L += pc[hd + 1] * expf(pc[hd] - M);
  }
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float o = 0.f;
    for (int c = 0; c < a.nchunk; ++c) {
      const float* pc = part + (size_t)c * (hd + 2);
      if (pc[hd + 1] > 0.f) o += pc[d] * expf(pc[hd] - M);
    }
    a.out[(size_t)r * a.nq * hd + (size_t)h * hd + d] = o / L;
  }
}

hipError_t launch_attention(const Rows& R, const AttnArgs& a, hipStream_t st) {
  if (a.nq > kMaxHeads || a.nchunk > kMaxChunks || a.nchunk < 1 || a.chunk < 1)
    return hipErrorInvalidValue;
  dim3 grid(a.nchunk, R.n);
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(k_attn<64>, grid, dim3(256), 0, st, R, a); break;
    case 128: hipLaunchKernelGGL(k_attn<128>, grid, dim3(256), 0, st, R, a); break;
    case 256: hipLaunchKernelGGL(k_attn<256>, grid, dim3(256), 0, st, R, a); break;
    case 512: hipLaunchKernelGGL(k_attn<512>, grid, dim3(256), 0, st, R, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(R.n, a.nq), dim3(256), 0, st, a);
  return hipGetLastError();
}

// positions[r] += 1 (graph-replayed decode loops advance on the device)
__global__ void k_advance(int32_t* pos, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[i] += 1;
}

hipError_t launch_advance(int32_t* pos, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_advance, dim3((n + 255) / 256), dim3(256), 0, st, pos, n);
  return hipGetLastError();
}

// out[i] = sum_p parts[p][i]
__global__ __launch_bounds__(256) void k_sum_partials(int nparts, size_t n,
                                                      const float* __restrict__ parts,
                                                      float* __restrict__ out) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int p = 0; p < nparts; ++p) s += parts[(size_t)p * n + i];
    out[i] = s;
  }
}

hipError_t launch_sum_partials(int nparts, size_t n, const float* parts, float* out,
                               hipStream_t st) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)blocks), dim3(256), 0, st, nparts, n, parts,
                     out);
  return hipGetLastError();
}

// ------------------------------------------------------------- argmax, pass 2
__global__ __launch_bounds__(256) void k_argmax_final(int nblk, const float* __restrict__ cv,
                                                      const int32_t* __restrict__ ci,
                                                      int32_t* __restrict__ out) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int r = blockIdx.x, t = threadIdx.x;
  float best = -FLT_MAX;
  int bi = 0x7FFFFFFF;
  for (int i = t; i < nblk; i += 256) {
    const float v = cv[(size_t)r * nblk + i];
    const int x = ci[(size_t)r * nblk + i];
    if (v > best || (v == best && x < bi)) {
      best = v;
      bi = x;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
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
    out[r] = bi == 0x7FFFFFFF ? 0 : bi;
  }
}

hipError_t launch_argmax_final(int rows, int nblk, const float* cand_val,
                               const int32_t* cand_idx, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax_final, dim3(rows), dim3(256), 0, st, nblk, cand_val, cand_idx, out);
  return hipGetLastError();
}

}  // namespace e2b
