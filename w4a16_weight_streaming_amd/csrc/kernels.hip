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
#include "dev_common.h"

#include <hip/hip_ext.h>

#include <float.h>
#include <stdlib.h>
#include <type_traits>
#include <math.h>

namespace e2b {

// Timestamps of the next matrix product launch (per host thread): when set,
// that launch records them at its own start and end (the dispatch's
// timestamps, not a marker queued before it), then they are cleared.
namespace {
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
}
void set_launch_events(hipEvent_t start, hipEvent_t stop) {
  g_ev_start = start;
  g_ev_stop = stop;
}
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_ev_start;
  *stop = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
  return *start != nullptr;
}

// ---------------------------------------------------------------- embedding
// h[r] = E[tok] * sqrt(H);  tokple[r] = E_ple[tok] * sqrt(P).  bf16 tables
// (EQ = 0) are widened; int4 tables (EQ = 1) decode (c - 8) * s, exact in
// fp32, first.  Either way the one rounding is the product with the fp32
// constant.
template <int EQ>
__global__ __launch_bounds__(256) void k_embed(Rows R, Lin E, Lin Ep, float sqrtH, float sqrtP,
                                               float* __restrict__ h, float* __restrict__ tokple,
                                               int* err, RopeTable rt) {
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
  const int H = E.K, LP = Ep.K;
  // 8 values per item (H and LP are multiples of 8; of 32 for int4), the
  // loads of up to 8 items per thread issued before any store
  const int nh = H / 8, nw = nh + LP / 8;
  for (int b0 = 0; b0 < nw; b0 += 8 * 256) {
    uint4 v[8];
    uint32_t sc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int w = b0 + threadIdx.x + 256 * k;
      w = w < nw ? w : nw - 1;
      if constexpr (EQ) {  // one packed word (8 codes) and its group scale
        const bool is_h = w < nh;
        const int ww = is_h ? w : w - nh;
        const uint32_t* q = is_h ? E.q + (size_t)tok * (H / 8) : Ep.q + (size_t)tok * (LP / 8);
        const uint16_t* gs = is_h ? E.s + (size_t)tok * (H / 32) : Ep.s + (size_t)tok * (LP / 32);
        v[k].x = q[ww];
        sc[k] = gs[ww / 4];
      } else {
        v[k] = *reinterpret_cast<const uint4*>(w < nh ? E.w + (size_t)tok * H + 8 * w
                                                      : Ep.w + (size_t)tok * LP + 8 * (w - nh));
        sc[k] = 0u;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int w = b0 + threadIdx.x + 256 * k;
      if (w >= nw) break;
      const bool is_h = w < nh;
      const float c = is_h ? sqrtH : sqrtP;
      float* dst = is_h ? h + (size_t)r * H + 8 * w : tokple + (size_t)r * LP + 8 * (w - nh);
      float x[8];
      if constexpr (EQ) {
        const float gsv = bf2f(sc[k]);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)((int)((v[k].x >> (4 * i)) & 15u) - 8) * gsv;
      } else {
        const uint32_t q[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf2f(q[i]);
          x[2 * i + 1] = bf2f(q[i] >> 16);
        }
      }
      reinterpret_cast<float4*>(dst)[0] = make_float4(x[0] * c, x[1] * c, x[2] * c, x[3] * c);
      reinterpret_cast<float4*>(dst)[1] = make_float4(x[4] * c, x[5] * c, x[6] * c, x[7] * c);
    }
  }
  // RoPE angles of this row's position for both layer types, from fp64
  // (cos then sin, hd/2 each; sliding first, then full)
  const int p = clamp_pos(R, pos);
  float* o = rt.out + (size_t)r * (rt.hd_s + rt.hd_f);
  for (int i = threadIdx.x; i < rt.hd_s / 2 + rt.hd_f / 2; i += blockDim.x) {
    const bool full = i >= rt.hd_s / 2;
    const int k = full ? i - rt.hd_s / 2 : i;
    const int half = full ? rt.hd_f / 2 : rt.hd_s / 2;
    float* base = full ? o + rt.hd_s : o;
    double sd, cd;
    sincos((double)p * (full ? rt.inv_f : rt.inv_s)[k], &sd, &cd);
    base[k] = (float)cd;
    base[half + k] = (float)sd;
  }
}

hipError_t launch_embed(const Rows& R, const Lin& E, const Lin& Eple, float sqrtH, float sqrtP,
                        float* h, float* tokple, int* err, const RopeTable& rt, hipStream_t st) {
  if (!rt.out || !rt.inv_s || !rt.inv_f) return hipErrorInvalidValue;
  const bool q = E.q != nullptr;
  if (q != (Eple.q != nullptr) || (q && (!E.s || !Eple.s)) || (!q && (!E.w || !Eple.w)))
    return hipErrorInvalidValue;
  const int g = q ? 32 : 8;
  if (E.K % g || Eple.K % g || E.K < 8) return hipErrorInvalidValue;
  if (q)
    hipLaunchKernelGGL(k_embed<1>, dim3(R.n), dim3(256), 0, st, R, E, Eple, sqrtH, sqrtP, h, tokple, err, rt);
  else
    hipLaunchKernelGGL(k_embed<0>, dim3(R.n), dim3(256), 0, st, R, E, Eple, sqrtH, sqrtP, h, tokple, err, rt);
  return hipGetLastError();
}

// ------------------------------------------------------ per-layer input finish
// pli[r][l] = (rms(u[r][l] * H^-1/2) * g + tokple[r][l]) * 2^-1/2
__global__ __launch_bounds__(256) void k_ple_finish(int LP, int P, const float* __restrict__ u,
                                                    int u_parts, size_t u_pstride,
                                                    const float* __restrict__ tokple,
                                                    const uint16_t* __restrict__ g, float inv_sqrtH,
                                                    float eps, float* __restrict__ pli) {
  __shared__ float sh[4];
  const int r = blockIdx.x, l = blockIdx.y, i = threadIdx.x;
  const size_t base = (size_t)r * LP + (size_t)l * P;
  const int ic = i < P ? i : 0;
  const uint32_t gi = g[ic];          // read with u, used after the reduction
  const float tp = tokple[base + ic];
  float v = 0.f;
  for (int q = 0; q < u_parts; ++q) v += u[(size_t)q * u_pstride + base + ic];
  v = i < P ? v * inv_sqrtH : 0.f;
  const float ss = block_sum<256>(v * v, sh);
  const float rr = rsqrtf(ss / (float)P + eps);
  if (i < P) pli[base + i] = fmaf(v * rr, bf2f(gi), tp) * 0.70710678118654752f;
}

hipError_t launch_ple_finish(const Rows& R, const float* u, int u_parts, size_t u_pstride,
                             const float* tokple, const uint16_t* g, int L, int P,
                             float inv_sqrtH, float eps, float* pli, hipStream_t st) {
  if (P > 256 || u_parts < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_ple_finish, dim3(R.n, L), dim3(256), 0, st, L * P, P, u, u_parts, u_pstride,
                     tokple, g, inv_sqrtH, eps, pli);
  return hipGetLastError();
}

// ------------------------------------------------------- matrix-vector product
template <int WQ, int KS, int U, int TAG>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(Lin W, int rows, Prologue pro,
                                                       Epilogue epi) {
  using Y = Lay<WQ, KS>;
  extern __shared__ float smem[];
  float* xs = smem;                                              // KS floats
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem + KS);         // packed pairs
  float* red = smem + KS + Packed<WQ, KS>::words;                // reduction scratch
  // (the per-layer input gate of a batched pass: blockIdx.x is the row, so a
  // row's blocks run on one XCD and its partial inputs are fetched into that
  // L2 once instead of once per block)
  constexpr bool kRowMajor = TAG == kTagPleGateRows;
  const int ks = blockIdx.y, b = kRowMajor ? blockIdx.x : blockIdx.z;
  const int bxi = kRowMajor ? blockIdx.z : blockIdx.x, gxn = kRowMajor ? gridDim.z : gridDim.x;
  const int K = W.K, N = W.N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ls = lane % Y::S, rsub = lane / Y::S;
  const int NU = (N + Y::RPL - 1) / Y::RPL;
  const int stride = gxn * 4;
  const size_t ldq = (size_t)K / 8, lds = (size_t)K / 32;

  // A batch is U units (RPL rows each) of this wave; batches are double
  // buffered: batch i+1 is requested before batch i is reduced.
  struct Batch {
    uint4 wv[U][Y::C];
    uint32_t sc[U][Y::C];  // W4A16 scales, raw bf16 (converted when used)
    int n[U];
  };
  // every load is unconditional (units past the end read row 0 and are never
  // stored), so no value is touched before the batch is reduced
  auto load_batch = [&](Batch& B, int u0) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int u = u0 + uu * stride;
      B.n[uu] = u * Y::RPL + rsub;
      const size_t row = (u < NU) && (B.n[uu] < N) ? (size_t)B.n[uu] : 0;
#pragma unroll
      for (int c = 0; c < Y::C; ++c) {
        if (WQ) {
          const int g = ls + Y::S * c;
          B.wv[uu][c] = *reinterpret_cast<const uint4*>(W.q + row * ldq + (size_t)ks * (KS / 8) + 4 * g);
          B.sc[uu][c] = W.s[row * lds + (size_t)ks * Y::G + g];
        } else {
          B.wv[uu][c] = *reinterpret_cast<const uint4*>(W.w + row * K + (size_t)ks * KS + 512 * c + 8 * ls);
          B.sc[uu][c] = 0u;
        }
      }
    }
  };

  typename std::conditional<tag_kind(TAG) == kAttnMerge, MergeRegs<KS>,
                            PrologueRegs<KS, tag_kind(TAG), tag_nd(TAG)>>::type pr;
  pr.load(pro, rows, b, ks * KS, K);  // input reads first: they gate the compute
  // every wave's input reads enter the memory pipeline before the block's
  // weight reads (otherwise they queue behind the other waves' weights)
  __syncthreads();
  int u0 = bxi * 4 + wave;
  Batch A, Bq;
  load_batch(A, u0);                  // then the weights (independent of x)
  // (no arithmetic on the inputs may move above the weight loads: it would
  // wait for the inputs before the weights are requested)
  __builtin_amdgcn_sched_barrier(0);
  pr.finish(pro, b, K, xs, red, bxi == 0 && blockIdx.y == 0);
  pack_x<WQ, KS>(xs, xp);

  // this lane's x pairs (and group sums for W4A16), read once
  uint32_t xh[Y::NP], xl[Y::NP];
  float gsum[Y::C];
#pragma unroll
  for (int c = 0; c < Y::C; ++c) {
    if (WQ) {
      const uint4* src = reinterpret_cast<const uint4*>(xp + (ls + Y::S * c) * Packed<WQ, KS>::kWordsW4);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 h4 = src[v], l4 = src[4 + v];
        xh[c * 16 + 4 * v + 0] = h4.x; xh[c * 16 + 4 * v + 1] = h4.y;
        xh[c * 16 + 4 * v + 2] = h4.z; xh[c * 16 + 4 * v + 3] = h4.w;
        xl[c * 16 + 4 * v + 0] = l4.x; xl[c * 16 + 4 * v + 1] = l4.y;
        xl[c * 16 + 4 * v + 2] = l4.z; xl[c * 16 + 4 * v + 3] = l4.w;
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
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // bytes of lo: codes 6,4,2,0 of the word; bytes of hi: codes 7,5,3,1.
            // v_perm puts two codes under the bf16 exponent byte 0x43 (128 + c).
            const uint32_t lo = w4[j] & 0x0F0F0F0Fu, hi = (w4[j] >> 4) & 0x0F0F0F0Fu;
            const uint32_t p0 = __builtin_amdgcn_perm(0x43434343u, lo, 0x04020400u);  // codes 0, 4
            const uint32_t p1 = __builtin_amdgcn_perm(0x43434343u, hi, 0x04020400u);  // codes 1, 5
            const uint32_t p2 = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030401u);  // codes 2, 6
            const uint32_t p3 = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030401u);  // codes 3, 7
            a = dot2(p0, xh[c * 16 + j * 4 + 0], a);
            a = dot2(p0, xl[c * 16 + j * 4 + 0], a);
            a = dot2(p1, xh[c * 16 + j * 4 + 1], a);
            a = dot2(p1, xl[c * 16 + j * 4 + 1], a);
            a = dot2(p2, xh[c * 16 + j * 4 + 2], a);
            a = dot2(p2, xl[c * 16 + j * 4 + 2], a);
            a = dot2(p3, xh[c * 16 + j * 4 + 3], a);
            a = dot2(p3, xl[c * 16 + j * 4 + 3], a);
          }
          acc = fmaf(bf2f(B.sc[uu][c]), fmaf(-136.0f, gsum[c], a), acc);  // (fmas written out)
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
        if (epi.argmax) {
          if (epi.logits) epi.logits[(size_t)b * N + nn] = acc;
          if (acc > best || (acc == best && nn < bidx)) {
            best = acc;
            bidx = nn;
          }
        } else {
          epi.y[((size_t)ks * rows + b) * N + nn] = acc;
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

  if (epi.argmax) {
    // wave reduce (max value, lowest index), then across the 4 waves
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
      epi.cand_val[(size_t)b * gxn + bxi] = bv;
      epi.cand_idx[(size_t)b * gxn + bxi] = bi;
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

// the slice widths the matvec kernel is instantiated for (dispatch_gemv)
bool gemv_supported(int K) {
  const int n = gemv_splits(K), ks = gemv_slice(K);
  return n >= 1 && n <= kMaxSplitK &&
         (ks == 32 || ks == 128 || ks == 256 || ks == 512 || ks == 1536 || ks == 2048);
}

template <int WQ, int KS, int U, int TAG>
static hipError_t run_gemv(const Lin& W, int rows, const Prologue& pro, const Epilogue& epi,
                           int blocks_hint, int* blocks_out, hipStream_t st) {
  using Y = Lay<WQ, KS>;
  const int nks = W.K / KS;
  const int NU = (W.N + Y::RPL - 1) / Y::RPL;
  // one unit per wave when N is small (latency); at most ~512 blocks in all
  // (two per CU, K slices and rows included) so that every block is resident
  // and waves of large matrices stream many units back to back
  int cap = 512 / (nks * rows);
  if (cap < 1) cap = 1;
  int bx = blocks_hint > 0 ? blocks_hint : (NU + 3) / 4;
  if (bx > cap) bx = cap;
  if (bx < 1) bx = 1;
  if (blocks_out) *blocks_out = bx;
  const size_t shm = ((size_t)KS + Packed<WQ, KS>::words + 32) * sizeof(float);
  const dim3 grid = TAG == kTagPleGateRows ? dim3(rows, nks, bx) : dim3(bx, nks, rows);
  E2B_TIMED_LAUNCH((k_gemv<WQ, KS, U, TAG>), grid, dim3(kGemvThreads), shm, st, W, rows, pro, epi);
  return hipGetLastError();
}

template <int WQ, int TAG>
static hipError_t dispatch_gemv(const Lin& W, int rows, const Prologue& pro,
                                const Epilogue& epi, int blocks_hint, int* bo, hipStream_t st) {
  // the merged attention input comes one head per K slice
  switch (pro.kind == kAttnMerge ? pro.slice : gemv_slice(W.K)) {
    case 64:
      if (pro.kind != kAttnMerge) return hipErrorInvalidValue;
      return run_gemv<WQ, 64, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 32: return run_gemv<WQ, 32, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 128: return run_gemv<WQ, 128, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 256: return run_gemv<WQ, 256, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    case 512: return run_gemv<WQ, 512, 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
    // (W4A16 gate/up: the double-width layers give each wave three units, one
    // batch of three instead of two dependent round trips)
    case 1536: return run_gemv<WQ, 1536, WQ ? (TAG == kTagGateUp ? 3 : 2) : 4, TAG>(W, rows, pro, epi, blocks_hint, bo, st);
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
    case kTagPleGateRows: return dispatch_gemv<WQ, kTagPleGateRows>(W, rows, pro, epi, blocks_hint, bo, st);
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
  if (pro.kind == kAttnMerge &&
      (tag != kTagO || !pro.a || pro.slice < 64 || W.K % pro.slice != 0 || W.K / pro.slice > kMaxHeads ||
       pro.nchunk < 1 || pro.nchunk > kMaxChunks))
    return hipErrorInvalidValue;
  if (epi.argmax && gemv_splits(W.K) != 1) return hipErrorInvalidValue;
  // the kernel is specialised on the product's prologue (argmax: the lm_head's)
  const int tk = epi.argmax ? kTagLmHead : tag;
  if (tag_kind(tk) >= 0 && pro.kind != tag_kind(tk)) return hipErrorInvalidValue;
  if ((pro.kind == kRes || pro.kind == kResNorm) && pro.d) {
    const int ndmax = tag_kind(tk) >= 0 ? tag_nd(tk) : kMaxSplitK;
    if (pro.nd < 1 || pro.nd > ndmax) return hipErrorInvalidValue;
  }
  if (epi.argmax)  // the tied lm_head: bf16 or int4 vocabulary table
    return quant ? dispatch_gemv<1, kTagLmHead>(W, rows, pro, epi, blocks_hint, blocks_out, st)
                 : dispatch_gemv<0, kTagLmHead>(W, rows, pro, epi, blocks_hint, blocks_out, st);
  return quant ? dispatch_tag<1>(tag, W, rows, pro, epi, blocks_hint, blocks_out, st)
               : dispatch_tag<0>(tag, W, rows, pro, epi, blocks_hint, blocks_out, st);
}

// ------------------------------------------------------------ prefill K/V write
// Prefill rows of one sequence attend to each other's keys, so every row's
// K/V is written before attention: block per row, wave 0 the key (norm with
// gain + RoPE), wave 1 the value (norm), bf16 at slot = position.
// ------------------------------------------------------------ decode attention
// (grid: rows x chunks, so a row's chunks are dispatched R.n apart and, for
// R.n a multiple of 8, run on one XCD: the row's query partials are fetched
// into one L2, where the merge of its chunk partials finds them)
template <int HD, int KQ>
__global__ __launch_bounds__(256) void k_attn_dec(Rows R, AttnArgs a) {
  attn_chunk<HD, KQ>(R, a, blockIdx.y, blockIdx.x);
}

__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  attn_combine(a, blockIdx.x, blockIdx.y);
}

// Prefill: K/V of every row written before attention.  Block per row, wave 0
// the key (norm with gain + RoPE), wave 1 the value (norm), bf16 at slot =
// position (the same arithmetic as the decode path's own-K/V write).
template <int HD, int KQ>
__global__ __launch_bounds__(128) void k_kv_write(Rows R, QkvPostArgs a) {
  constexpr int DPL = HD / 64;
  const int r = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pos = clamp_pos(R, row_pos(R, r));
  const int seq = row_seq(R, r);
  const float* cs = a.rope + (size_t)r * a.rope_ld + a.rope_off;
  const float* sn = cs + HD / 2;
  const float* raw = a.qkv + (size_t)r * (a.nq + 2) * HD + (size_t)(a.nq + wave) * HD;
  const bool is_v = wave == 1;
  float y[DPL];
  head_vec<HD>(raw, a.qkv_parts, a.qkv_pstride, is_v ? nullptr : a.gk, !is_v, cs, sn, lane, a.eps, y);
  const size_t slot = cache_row(R, seq, pos);
  if constexpr (KQ) {
    float deq[DPL];
    store_int8_row<DPL>(y, static_cast<int8_t*>(is_v ? a.vc : a.kc) + slot * HD, (is_v ? a.vs : a.ks) + slot,
                        lane, deq);
  } else {
    uint16_t* dst = static_cast<uint16_t*>(is_v ? a.vc : a.kc) + slot * HD;
#pragma unroll
    for (int i = 0; i < DPL; ++i) dst[lane * DPL + i] = (uint16_t)f2bf(y[i]);
  }
}

template <int KQ>
static hipError_t kv_write_q(const Rows& R, const QkvPostArgs& a, hipStream_t st) {
  switch (a.hd) {
    case 64: hipLaunchKernelGGL((k_kv_write<64, KQ>), dim3(R.n), dim3(128), 0, st, R, a); break;
    case 128: hipLaunchKernelGGL((k_kv_write<128, KQ>), dim3(R.n), dim3(128), 0, st, R, a); break;
    case 256: hipLaunchKernelGGL((k_kv_write<256, KQ>), dim3(R.n), dim3(128), 0, st, R, a); break;
    case 512: hipLaunchKernelGGL((k_kv_write<512, KQ>), dim3(R.n), dim3(128), 0, st, R, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qkv_post(const Rows& R, const QkvPostArgs& a, hipStream_t st) {
  if (!a.kc || !a.vc || !a.rope || (a.kvq && (!a.ks || !a.vs))) return hipErrorInvalidValue;
  return a.kvq ? kv_write_q<1>(R, a, st) : kv_write_q<0>(R, a, st);
}

template <int KQ>
static hipError_t attn_q(const Rows& R, const AttnArgs& a, hipStream_t st) {
  dim3 grid(R.n, a.nchunk);
  switch (a.hd) {
    case 64: E2B_TIMED_LAUNCH((k_attn_dec<64, KQ>), grid, dim3(256), 0, st, R, a); break;
    case 128: E2B_TIMED_LAUNCH((k_attn_dec<128, KQ>), grid, dim3(256), 0, st, R, a); break;
    case 256: E2B_TIMED_LAUNCH((k_attn_dec<256, KQ>), grid, dim3(256), 0, st, R, a); break;
    case 512: E2B_TIMED_LAUNCH((k_attn_dec<512, KQ>), grid, dim3(256), 0, st, R, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const Rows& R, const AttnArgs& a, hipStream_t st) {
  if (a.nq > kMaxHeads || a.nchunk > kMaxChunks || a.nchunk < 1 || a.chunk < 1 || !a.rope)
    return hipErrorInvalidValue;
  if (a.kvq && (!a.ks || !a.vs || (a.kc_own && (!a.ks_own || !a.vs_own)))) return hipErrorInvalidValue;
  hipError_t e = a.mfma ? launch_attn_prefill(R, a, st) : a.kvq ? attn_q<1>(R, a, st) : attn_q<0>(R, a, st);
  if (e != hipSuccess || !a.combine) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(R.n, a.nq), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The matrix-core copy of a W4A16 matrix, per 16-row tile t and 128-k block
// b: for each lane l its four code words (row 16t + l%16, groups 4b..4b+3,
// quarter l/16 of each group) in 16 contiguous bytes, then per row of the
// tile its four group scales in 8.  (K a multiple of 128.)
__global__ __launch_bounds__(256) void k_tile_w4(const uint32_t* __restrict__ q,
                                                 const uint16_t* __restrict__ s, int N, int K,
                                                 uint32_t* __restrict__ tq, uint16_t* __restrict__ ts) {
  const size_t G = K / 32, NB = K / 128, n_words = (size_t)N * K / 8;
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n_words; i += (size_t)gridDim.x * 256) {
    const size_t st = i % 4, l = (i / 4) % 64, tb = i / 256, t = tb / NB, g = 4 * (tb % NB) + st;
    tq[i] = q[(16 * t + l % 16) * (K / 8) + 4 * g + l / 16];
    if (l < 16) ts[(tb * 16 + l) * 4 + st] = s[(16 * t + l) * G + g];
  }
}

__global__ __launch_bounds__(256) void k_tile_bf16(const uint4* __restrict__ w, int N, int K,
                                                   uint4* __restrict__ tw) {
  const size_t G = K / 32, n = (size_t)N * K / 8;  // 16-byte pieces
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t l = i % 64, tg = i / 64, t = tg / G, g = tg % G;
    tw[i] = w[(16 * t + l % 16) * (K / 8) + 4 * g + l / 16];
  }
}

hipError_t launch_tile_bf16(const Lin& W, uint16_t* tw, hipStream_t st) {
  if (!W.w || !tw || W.N % 16 || W.K % 32 || W.N < 16) return hipErrorInvalidValue;
  const size_t n = (size_t)W.N * W.K / 8;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_tile_bf16, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(W.w), W.N, W.K, reinterpret_cast<uint4*>(tw));
  return hipGetLastError();
}

hipError_t launch_tile_w4(const Lin& W, uint32_t* tq, uint16_t* ts, hipStream_t st) {
  if (!W.q || !W.s || !tq || !ts || W.N % 16 || W.K % 128 || W.N < 16) return hipErrorInvalidValue;
  const size_t n_words = (size_t)W.N * W.K / 8;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_tile_w4, dim3((unsigned)blocks), dim3(256), 0, st, W.q, W.s, W.N, W.K, tq, ts);
  return hipGetLastError();
}

// ===================================================== batched rows: MFMA path
// For rows >= 2 (batched decode, prefill) the input rows are prepared once by
// k_xprep (the same prologue arithmetic as the single-row matvec, K-slice
// partials of the producer summed) as bf16 hi/lo pairs [rows][K] plus per-32
// group sums of hi+lo, and k_gemm streams each weight row once for up to 64
// rows with v_mfma_f32_16x16x32_bf16:
//   D[m][n] += A_hi[m][k] W[n][k] + A_lo[m][k] W[n][k]
// A (16 rows x 32 k): lane l holds row l%16, k = 8(l/16)..8(l/16)+7.
// B (32 k x 16 cols): lane l holds col l%16, the same k range.
// D (16 x 16): lane l holds rows 4(l/16)..4(l/16)+3 of col l%16.
// W4A16: the B operand holds 128 + c (code c under the bf16 exponent byte
// 0x43); each 32-wide k step is one scale group, so per group
//   acc += s[n][g] * (D_group - 136 * sum_k (A_hi + A_lo)[m][k]).

__device__ __forceinline__ void ld8_bf(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf2f(w[i]); v[2 * i + 1] = bf2f(w[i] >> 16); }
}
// sum of n partial rows (stride floats apart), 8 consecutive elements; the
// loads of up to B partials are issued together, the sum runs in order
template <int B = 8>
__device__ __forceinline__ void ld8_parts(const float* p, int n, size_t stride, float (&v)[8]) {
  // the first 4 partials are read unconditionally (the zero row past n),
  // with no use in between: a loop entered with a read pending would wait
  // for it first
  float t0[4][8];
#pragma unroll
  for (int k = 0; k < 4; ++k) ld8(k < n ? p + (size_t)k * stride : zero_f(), t0[k]);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = t0[0][j];
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (k < n)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] += t0[k][j];
  for (int q0 = 4; q0 < n; q0 += B) {
    float t[B][8];
#pragma unroll
    for (int u = 0; u < B; ++u) ld8(q0 + u < n ? p + (size_t)(q0 + u) * stride : zero_f(), t[u]);
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (q0 + u < n)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += t[u][j];
  }
}

// Two operands (the second optional) with their partials, all reads in
// flight together (the first 4 partials of each unconditionally, as above)
__device__ __forceinline__ void ld8_parts2(const float* p0, const float* p1, bool two, int n,
                                           size_t stride, float (&v)[8], float (&u)[8]) {
  if (!two) {
    ld8_parts(p0, n, stride, v);
    return;
  }
  float t0[4][8], t1[4][8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ld8(k < n ? p0 + (size_t)k * stride : zero_f(), t0[k]);
    ld8(k < n ? p1 + (size_t)k * stride : zero_f(), t1[k]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = t0[0][j];
    u[j] = t1[0][j];
  }
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (k < n)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] += t0[k][j];
        u[j] += t1[k][j];
      }
  for (int q0 = 4; q0 < n; q0 += 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ld8(q0 + k < n ? p0 + (size_t)(q0 + k) * stride : zero_f(), t0[k]);
      ld8(q0 + k < n ? p1 + (size_t)(q0 + k) * stride : zero_f(), t1[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (q0 + k < n)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[j] += t0[k][j];
          u[j] += t1[k][j];
        }
  }
}

__device__ __forceinline__ void unpack8(uint4 w, float (&v)[8]) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf2f(q[i]); v[2 * i + 1] = bf2f(q[i] >> 16); }
}

// Thread t handles elements 8t.. of the row's slice.  kRes / kResNorm: block
// per row (K <= 2048, row reductions); the other kinds: block per (row,
// 2048-slice).  Every read is issued before the first value is used (absent
// gains read the zero row); bf16 gains stay packed until then.
__global__ __launch_bounds__(256) void k_xprep(Prologue p, int rows, int K, uint16_t* __restrict__ xh,
                                               uint16_t* __restrict__ xl, float* __restrict__ xg) {
  __shared__ float red[8];
  const int b = blockIdx.x, t = threadIdx.x;
  uint16_t* oh = xh + (size_t)b * K;
  uint16_t* ol = xl + (size_t)b * K;
  float* og = xg + (size_t)b * (K / 32);
  if (p.kind == kRes || p.kind == kResNorm) {
    const int i0 = 8 * t;
    const bool on = i0 < K;
    const int ic = on ? i0 : 0;
    const uint16_t* gdp = p.d ? p.gd : kZeroRow;
    const uint16_t* gxp = p.kind == kResNorm ? p.gx : kZeroRow;
    const uint4 gdw = *reinterpret_cast<const uint4*>(gdp + ic);
    const uint4 gxw = *reinterpret_cast<const uint4*>(gxp + ic);
    const uint32_t scw = *(p.scalar ? p.scalar : kZeroRow);
    float av[8], dv[8];
    ld8(p.a + (size_t)b * K + ic, av);
#pragma unroll
    for (int j = 0; j < 8; ++j) dv[j] = 0.f;
    if (p.d) ld8_parts<8>(p.d + (size_t)b * K + ic, p.nd, p.d_pstride, dv);
    float ss = 0.f;
    if (on)
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(dv[j], dv[j], ss);
    float rd = 0.f;
    if (p.d) rd = rsqrtf(block_sum<256>(ss, red) / (float)K + p.eps);
    const float sc = p.scalar ? bf2f(scw) : 1.0f;
    float gdv[8], gxv[8];
    unpack8(gdw, gdv);
    unpack8(gxw, gxv);
    float hs = 0.f;
    if (p.d) {
#pragma unroll
      for (int j = 0; j < 8; ++j) av[j] = fmaf(dv[j] * rd, gdv[j], av[j]) * sc;
      if (p.h_out && on) {
        float* ho = p.h_out + (size_t)b * K + i0;
        *reinterpret_cast<float4*>(ho) = make_float4(av[0], av[1], av[2], av[3]);
        *reinterpret_cast<float4*>(ho + 4) = make_float4(av[4], av[5], av[6], av[7]);
      }
    }
    if (on)
#pragma unroll
      for (int j = 0; j < 8; ++j) hs = fmaf(av[j], av[j], hs);
    if (p.kind == kResNorm) {
      const float rh = rsqrtf(block_sum<256>(hs, red) / (float)K + p.eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) av[j] = av[j] * rh * gxv[j];
    }
    if (on) emit8(av, oh, ol, og, i0);
  } else {
    const int i0 = blockIdx.y * 2048 + 8 * t;
    if (i0 >= K) return;  // whole 32-groups: the four threads of a group go together
    const float* src = p.a + (size_t)b * p.lda + i0;
    float v[8], u[8];
    const bool two = p.kind == kGeglu;
    if (p.kind == kPleGate) ld8(p.pli + (size_t)b * p.pli_ld + i0, u);
    ld8_parts2(src, src + K, two, p.na, p.a_pstride, v, u);
    if (p.kind == kGeglu || p.kind == kPleGate)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = gelu_tanh(v[j]) * u[j];
    emit8(v, oh, ol, og, i0);
  }
}

hipError_t launch_xprep(const Prologue& p, int rows, int K, uint16_t* xh, uint16_t* xl, float* xg,
                        hipStream_t st) {
  const bool res = p.kind == kRes || p.kind == kResNorm;
  if (K % 32 || (res && K > 2048)) return hipErrorInvalidValue;
  if (p.na < 1 || (p.d && p.nd < 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_xprep, dim3(rows, res ? 1 : (K + 2047) / 2048), dim3(256), 0, st, p, rows, K,
                     xh, xl, xg);
  return hipGetLastError();
}

// Column tile and K slices of a batched product (independent of the row
// count, so a row's result does not depend on how many rows share the pass).
// Enough blocks to cover the chip: narrower column tiles first, then (where
// the consumer sums partials) K slices of >= 256.
GemmPlan gemm_plan(int quant, int N, int K, bool partial_ok) {
  constexpr int kTarget = 256;  // (512 or 1024 target blocks: no better)
  GemmPlan p;
  auto cols = [&](int nt) { return (N + 64 * nt - 1) / (64 * nt); };
  // Two column tiles per wave where the product still fills the chip with
  // its K split (each activation fragment read from LDS then feeds two
  // products, half the LDS traffic per weight byte); bf16 products too narrow
  // for that (q/k/v, the sliding layers' O) keep one.
  // (a W4A16 matrix with K a multiple of 128 has a tiled copy, read in
  // whole 128-k blocks: its K slices are whole blocks)
  const int kq = quant && K % 128 == 0 ? 128 : 32;
  int kmax = 1;
  for (int c : {2, 3, 4, 6, 8, 12, 16})
    if (K % (kq * c) == 0 && K / c >= 256) kmax = c;
  p.nt = quant ? 4 : 2;
  const int nt_min = quant || cols(2) * (partial_ok ? kmax : 1) >= 192 ? 2 : 1;
  while (p.nt > nt_min && cols(p.nt) < kTarget) p.nt >>= 1;
  p.nks = 1;
  if (partial_ok) {
    static const int cand[] = {2, 3, 4, 6, 8, 12, 16};
    for (int c : cand) {
      if (cols(p.nt) * p.nks >= kTarget) break;
      if (K % (kq * c) == 0 && K / c >= 256) p.nks = c;
    }
  }
  return p;
}

// No K slices (the epilogue needs whole sums), for every row count, so a
// row's result still does not depend on its pass.  Narrow column tiles and
// few rows per block keep the block count up (measured at K = 1536: bf16 at
// most 32 rows per block, one tile of 16 columns per wave up to 32 rows and
// two beyond; W4A16 16 rows per block, one tile up to 16 rows and two from
// 17, whose weights re-read by the row blocks come from L2).  Tiles and rows
// per block do not change the arithmetic of an output.
GemmPlan gemm_plan_geglu(int quant, int I, int K, int rows) {
  GemmPlan p;
  p.nks = 1;
  p.nt = rows > (quant ? 16 : 32) ? 2 : 1;
  p.mt = quant ? 1 : 2;
  // (whole blocks for every tile width the row count may pick: the fold is
  // taken or not for all passes alike)
  if (I % 64 || K % 128) p.nt = 0;
  return p;
}

hipError_t launch_gemm(int quant, int tag, const Lin& W, int rows, const GemmA& A,
                       const GemmPlan& plan, const Epilogue& epi, int* nblk, hipStream_t st) {
  const int nks = plan.nks;
  if (rows < 1 || nks < 1 || nks > kMaxGemmSplit || W.K % nks || (W.K / nks) % 32)
    return hipErrorInvalidValue;
  if (epi.argmax && nks != 1) return hipErrorInvalidValue;
  if (epi.gh && (tag != kTagGateUp || epi.argmax || nks != 1 || plan.nt < 1 || !epi.gl || !epi.gg ||
                 (quant && !W.tq) ||  // (the untiled W4A16 kernel has no GeGLU epilogue)
                 epi.gi < 1 || W.N != 2 * epi.gi || epi.gi % (32 * plan.nt)))
    return hipErrorInvalidValue;
  if (quant && W.tq && (!W.ts || (W.K / nks) % 128)) return hipErrorInvalidValue;
  if (A.a ? A.kind != kPlain || A.na != 1 || A.lda % 8
          : (!A.xh || !A.xl || (quant && !A.xg)))
    return hipErrorInvalidValue;
  return quant ? launch_gemm_w4(tag, W, rows, A, plan, epi, nblk, st)
               : launch_gemm_bf16(tag, W, rows, A, plan, epi, nblk, st);
}

// ------------------------------------------------- calibration: streaming read
// out[block] = sum of the buffer's 32-bit words (as fp32) that the block
// read: every byte read once, 16 bytes per lane per load, four loads in
// flight per lane.  Its rate is the read bandwidth a plain stream sustains.
__global__ __launch_bounds__(256) void k_stream_reduce(const uint4* __restrict__ p, size_t n16,
                                                       float* __restrict__ out) {
  __shared__ float sh[4];
  float acc = 0.f;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = p[i + k * stride];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc += (__uint_as_float(v[k].x) + __uint_as_float(v[k].y)) +
             (__uint_as_float(v[k].z) + __uint_as_float(v[k].w));
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc += (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
  }
  acc = block_sum<256>(acc, sh);
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

hipError_t launch_stream_reduce(const void* buf, size_t bytes, float* out, hipStream_t st) {
  if (!buf || !out || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_reduce, dim3(kStreamBlocks), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

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
// adv (optional): the row's position, advanced by one once the token is out
// (a captured step that advances its positions needs no kernel of its own)
__global__ __launch_bounds__(256) void k_argmax_final(int nblk, const float* __restrict__ cv,
                                                      const int32_t* __restrict__ ci,
                                                      int32_t* __restrict__ out,
                                                      int32_t* __restrict__ adv) {
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
    out[r] = bi == 0x7FFFFFFF ? 0 : bi;
    if (adv) adv[r] += 1;
  }
}

hipError_t launch_argmax_final(int rows, int nblk, const float* cand_val,
                               const int32_t* cand_idx, int32_t* out, int32_t* adv,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_argmax_final, dim3(rows), dim3(256), 0, st, nblk, cand_val, cand_idx, out,
                     adv);
  return hipGetLastError();
}

}  // namespace e2b
