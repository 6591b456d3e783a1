// Device helpers of the kernels of libe2b (kernels.hip: one kernel per phase
// of the step).
#pragma once

#include "e2b_internal.h"

#include <hip/hip_ext.h>

#include <float.h>
#include <math.h>

namespace e2b {

// Launch a kernel; when the host thread has pending profiling events (see
// set_launch_events), the launch records them at its own start and end.
#define E2B_TIMED_LAUNCH(kernel, grid, block, shm, st, ...)                                       \
  do {                                                                                            \
    hipEvent_t ev_a_, ev_b_;                                                                      \
    if (take_launch_events(&ev_a_, &ev_b_))                                                       \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, st, ev_a_, ev_b_, 0, __VA_ARGS__);           \
    else                                                                                          \
      hipLaunchKernelGGL(kernel, grid, block, shm, st, __VA_ARGS__);                              \
  } while (0)

// Plain accessors (one place to change how activations cross kernels).
__device__ __forceinline__ void st32(float* p, float v) { *p = v; }
__device__ __forceinline__ float ld32(const float* p) { return *p; }
__device__ __forceinline__ void st16(uint16_t* p, uint16_t v) { *p = v; }

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
  // (fused multiply-adds written out: the same rounding wherever it is inlined)
  return 0.5f * x * (1.0f + tanhf(c * fmaf(0.044715f * x * x, x, x)));
}

// Cross-lane exchange.  A shuffle through the LDS crossbar (ds_bpermute)
// costs a round trip per step; inside a row of 16 lanes the partner lane^o,
// o = 1, 2, 4, 8, is reached by DPP moves (VALU): quad permutes for 1 and 2,
// half-row mirror then quad reverse for 4, row mirror then half-row mirror
// for 8.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int O>
__device__ __forceinline__ float xor_lane(float v) {  // v of lane ^ O, O < 16
  static_assert(O == 1 || O == 2 || O == 4 || O == 8, "DPP xor partner within a row");
  if constexpr (O == 1) return dpp_mov<0xB1>(v);                  // quad_perm [1,0,3,2]
  else if constexpr (O == 2) return dpp_mov<0x4E>(v);             // quad_perm [2,3,0,1]
  else if constexpr (O == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));  // half mirror, quad reverse
  else return dpp_mov<0x141>(dpp_mov<0x140>(v));                  // row mirror, half mirror
}

// Sum over aligned groups of S lanes (S <= 16): every lane of a group gets
// the group's sum, the same value (and rounding) as the xor butterfly.  Once
// a quad (8-group) holds one value, a mirror pairs it with the neighbouring
// quad (8-group) exactly as xor 4 (8) would.
template <int S>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16, "group of at most one row");
  if constexpr (S >= 2) v += dpp_mov<0xB1>(v);
  if constexpr (S >= 4) v += dpp_mov<0x4E>(v);
  if constexpr (S >= 8) v += dpp_mov<0x141>(v);
  if constexpr (S >= 16) v += dpp_mov<0x140>(v);
  return v;
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over groups of S lanes for any S up to 64 (S = 32: two halves): the
// row sums by DPP, then the xor-16 / xor-32 steps on the four row sums read
// out of lanes 0, 16, 32, 48 ((r0 + r1) + (r2 + r3), the butterfly's order).
template <int S>
__device__ __forceinline__ float lanes_sum(float v) {
  if constexpr (S <= 16) {
    return group_sum<S>(v);
  } else {
    v = group_sum<16>(v);
    const float a = lane_value(v, 0) + lane_value(v, 16), b = lane_value(v, 32) + lane_value(v, 48);
    if constexpr (S == 64) return a + b;
    else return (threadIdx.x & 32) ? b : a;
  }
}

__device__ __forceinline__ float wave_sum(float v) { return lanes_sum<64>(v); }

template <int O>
__device__ __forceinline__ int xor_lane_i(int v) {
  return __builtin_bit_cast(int, xor_lane<O>(__builtin_bit_cast(float, v)));
}

// Maximum over the wave, every lane gets it (row maxima by DPP, then the
// four rows read out)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, xor_lane_i<1>(v));
  v = max(v, xor_lane_i<2>(v));
  v = max(v, __builtin_bit_cast(int, dpp_mov<0x141>(__builtin_bit_cast(float, v))));
  v = max(v, __builtin_bit_cast(int, dpp_mov<0x140>(__builtin_bit_cast(float, v))));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// (value, index) maximum with the lowest index among equal values; the
// result does not depend on the order of the comparisons
__device__ __forceinline__ void arg_better(float ov, int oi, float& v, int& i) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
template <int O>
__device__ __forceinline__ void argmax_xor(float& v, int& i) {
  arg_better(xor_lane<O>(v), xor_lane_i<O>(i), v, i);
}
// over groups of S lanes (S <= 16) by DPP, or the whole wave (S = 64)
template <int S>
__device__ __forceinline__ void argmax_lanes(float& v, int& i) {
  if constexpr (S >= 2) argmax_xor<1>(v, i);
  if constexpr (S >= 4) argmax_xor<2>(v, i);
  if constexpr (S >= 8) argmax_xor<4>(v, i);
  if constexpr (S >= 16) argmax_xor<8>(v, i);
  if constexpr (S == 64) {  // each lane folds in the four row results
    const float v0 = v;
    const int i0 = i;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      arg_better(lane_value(v0, 16 * r), __builtin_amdgcn_readlane(i0, 16 * r), v, i);
  }
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

// Cache row of (sequence slot, position): contiguous, or through the page
// table.  A page entry outside the pool flags the error word and maps to the
// pool's spare page (index n_pages), which no sequence owns.
__device__ __forceinline__ size_t cache_row(const Rows& R, int seq, int pos) {
  if (!R.pages) return (size_t)seq * R.max_ctx + pos;
  int pg = R.pages[(size_t)seq * R.page_stride + (pos >> kPageShift)];
  if ((unsigned)pg >= (unsigned)R.n_pages) {
    if (R.err) atomicOr(R.err, kErrPage);
    pg = R.n_pages;
  }
  return (size_t)pg * kPageSize + (pos & (kPageSize - 1));
}

// eight consecutive fp32 values (16-byte aligned)
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
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

// The block's fp32 input slice xs[0..KS) for row b (K slice k0..k0+KS), in two
// halves: load() issues every global read the prologue needs at once (one
// round trip; the weight prefetch is issued after it), finish() does the
// arithmetic and writes xs.
// A never-written row of zeros: what an unconditional load of an absent
// operand reads.  (Repeating a real operand's address would not do: the
// compiler then copies that load's register, which waits for it.)  4096 bf16
// = 2048 floats,
// the widest row such a load covers.
static __device__ __align__(16) uint16_t kZeroRow[4096];
__device__ __forceinline__ const float* zero_f() { return reinterpret_cast<const float*>(kZeroRow); }

template <int KS, int PK = -1, int ND = kMaxSplitK>
struct PrologueRegs {
  static constexpr int PT = (KS + kGemvThreads - 1) / kGemvThreads;
  static constexpr int NDX = PK >= 0 ? (ND > 0 ? ND : 1) : kMaxSplitK;
  // PK >= 0: the kind is known at compile time and every load is
  // unconditional (absent operands read from stand-ins and are dropped by
  // selects later).  bf16 gains and the layer scalar stay raw until finish():
  // a conversion next to its load (which the compiler makes out of a
  // conditional load) waits for every load in flight, one memory round trip
  // each.
  float a0[PT], a1[PT];
  uint32_t g0[PT], g1[PT], sc;
  float dq[PT][NDX];
  int nd;

  __device__ __forceinline__ int kind(const Prologue& p) const { return PK >= 0 ? PK : p.kind; }

  __device__ __forceinline__ void load(const Prologue& p, int rows, int b, int k0, int K) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      a0[j] = a1[j] = 0.f;
      g0[j] = g1[j] = 0u;
#pragma unroll
      for (int q = 0; q < NDX; ++q) dq[j][q] = 0.f;
    }
    sc = 0u;
    nd = 0;
    auto ok = [&](int j) { return KS % kGemvThreads == 0 || t + j * kGemvThreads < KS; };
    const int kd = kind(p);
    if (kd == kPlain || kd == kGeglu || kd == kPleGate) {
      const float* s0 = p.a + (size_t)b * p.lda + k0;
      const float* s1 = kd == kGeglu ? s0 + K
                        : kd == kPleGate ? p.pli + (size_t)b * p.pli_ld + k0
                                         : nullptr;
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (ok(j)) a0[j] = ld32(s0 + t + j * kGemvThreads);
      if (PK == kGeglu || PK == kPleGate || (PK < 0 && s1))
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (ok(j)) a1[j] = ld32(s1 + t + j * kGemvThreads);
      return;
    }
    // kRes / kResNorm: KS == K == hidden size.  Gains absent here read the
    // zero row and are not used
    const float* hrow = p.a + (size_t)b * K;
    const uint16_t* stand_in = kZeroRow;
    const uint16_t* gx = kd == kResNorm ? p.gx : stand_in;
    const uint16_t* gd = p.d ? p.gd : stand_in;
#pragma unroll
    for (int j = 0; j < PT; ++j)
      if (ok(j)) {
        const int i = t + j * kGemvThreads;
        a0[j] = ld32(hrow + i);
        g1[j] = gx[i];
        g0[j] = gd[i];
      }
    nd = p.d ? p.nd : 0;
    if constexpr (PK >= 0) {
      // partial q, or the zero row past nd
      const float* dp = p.d ? p.d + (size_t)b * K : zero_f();
#pragma unroll
      for (int q = 0; q < NDX; ++q) {
        const float* src = q < nd ? dp + (size_t)q * p.d_pstride : zero_f();
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (ok(j)) dq[j][q] = ld32(src + t + j * kGemvThreads);
      }
    } else if (p.d) {
#pragma unroll
      for (int q = 0; q < NDX; ++q)
        if (q < nd)
#pragma unroll
          for (int j = 0; j < PT; ++j)
            if (ok(j)) dq[j][q] = ld32(p.d + (size_t)q * p.d_pstride + (size_t)b * K + t + j * kGemvThreads);
    }
    sc = *(p.scalar ? p.scalar : stand_in);  // (1 when there is no scalar)
  }

  // store_h: this block writes the updated residual h' (one block per
  // product)
  __device__ __forceinline__ void finish(const Prologue& p, int b, int K, float* xs, float* red,
                                         bool store_h) {
    const int t = threadIdx.x;
    const int kd = kind(p);
    if (kd == kPlain) {
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (t + j * kGemvThreads < KS) xs[t + j * kGemvThreads] = a0[j];
    } else if (kd == kGeglu || kd == kPleGate) {
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (t + j * kGemvThreads < KS) xs[t + j * kGemvThreads] = gelu_tanh(a0[j]) * a1[j];
    } else {
      float dv[PT], ss = 0.f;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < NDX; ++q) s += q < nd ? dq[j][q] : 0.f;
        dv[j] = s;
        ss = fmaf(s, s, ss);
      }
      float rd = 0.f;
      if (p.d) rd = rsqrtf(block_sum<kGemvThreads>(ss, red) / (float)K + p.eps);
      const float scv = p.scalar ? bf2f(sc) : 1.0f;
      const bool store = p.d && p.h_out && store_h;
      float hv[PT], hs = 0.f;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int i = t + j * kGemvThreads;
        float hn = a0[j];
        if (p.d) hn = fmaf(dv[j] * rd, bf2f(g0[j]), hn) * scv;
        hv[j] = hn;
        if (i < KS) {
          hs = fmaf(hn, hn, hs);
          if (store) st32(p.h_out + (size_t)b * K + i, hn);
        }
      }
      if (kd == kResNorm) {
        const float rh = rsqrtf(block_sum<kGemvThreads>(hs, red) / (float)K + p.eps);
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (t + j * kGemvThreads < KS) xs[t + j * kGemvThreads] = hv[j] * rh * bf2f(g1[j]);
      } else {
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (t + j * kGemvThreads < KS) xs[t + j * kGemvThreads] = hv[j];
      }
    }
    __syncthreads();
  }
};

// Input slice of the one-row O product: the attention output of one head.
// The block's K slice is head h = k0 / KS (KS = hd, K = nq * hd), and its
// input is merged here from the (max m_c, sum l_c, unnormalised o_c) partials
// that the attention chunks wrote for (row b, head h), instead of in a kernel
// of its own: o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c over the chunks
// that hold keys (M their largest m_c).  Lane c of every wave reads chunk c's
// (m_c, l_c), so each wave forms M, the sum and the weights itself; the o
// values of the first CB chunks are requested together with them.  Chunks
// without keys (l_c = 0) and slots past nchunk hold stale values: they get no
// weight and are skipped by a select, never multiplied.
template <int KS>
struct MergeRegs {
  static constexpr int PT = (KS + kGemvThreads - 1) / kGemvThreads;
  static constexpr int CB = 32 / PT;  // chunks per batch of reads
  static_assert(kMaxChunks <= 64, "one chunk per lane");
  float v[CB][PT];
  float mc, lc;
  const float* base;
  int nchunk;

  __device__ __forceinline__ void issue(int c0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int d = t + j * kGemvThreads < KS ? t + j * kGemvThreads : 0;
        v[c][j] = c0 + c < nchunk ? base[(size_t)(c0 + c) * (KS + 2) + d] : zero_f()[d];
      }
  }

  __device__ __forceinline__ void load(const Prologue& p, int rows, int b, int k0, int K) {
    const int lane = threadIdx.x & 63, nq = K / KS, h = k0 / KS;
    nchunk = p.nchunk;
    base = p.a + (size_t)(b * nq + h) * kMaxChunks * (KS + 2);
    const float* ml = lane < nchunk ? base + (size_t)lane * (KS + 2) + KS : zero_f();
    mc = ml[0];
    lc = ml[1];
    issue(0);
  }

  __device__ __forceinline__ void finish(const Prologue&, int, int, float* xs, float*, bool) {
    const int t = threadIdx.x, lane = t & 63;
    const bool act = lane < nchunk && lc > 0.f;
    const float M = wave_max(act ? mc : -INFINITY);
    const float w = act ? expf(mc - M) : 0.f;
    const float L = wave_sum(w * lc);
    const float wn = L > 0.f ? w / L : 0.f;  // this lane's chunk weight
    float o[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) o[j] = 0.f;
    for (int c0 = 0; c0 < nchunk; c0 += CB) {
      if (c0 > 0) issue(c0);
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float wc = lane_value(wn, (c0 + c) & 63);  // 0 past nchunk (lane >= nchunk)
#pragma unroll
        for (int j = 0; j < PT; ++j) o[j] = wc != 0.f ? fmaf(wc, v[c][j], o[j]) : o[j];
      }
    }
#pragma unroll
    for (int j = 0; j < PT; ++j)
      if (t + j * kGemvThreads < KS) xs[t + j * kGemvThreads] = o[j];
    __syncthreads();
  }
};

// split an fp32 pair into a bf16 hi pair and a bf16 lo pair (x = hi + lo)
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t ha = f2bf(a), hb = f2bf(b);
  const uint32_t la = f2bf(a - bf2f(ha)), lb = f2bf(b - bf2f(hb));
  hi = ha | (hb << 16);
  lo = la | (lb << 16);
}

// Writes x[i0 .. i0+7] as bf16 hi/lo and, from the four threads that cover
// one 32-group (consecutive threads, all active together), its group sum.
__device__ __forceinline__ void emit8(const float (&v)[8], uint16_t* xh, uint16_t* xl, float* xg,
                                      int i0) {
  uint32_t h[4], l[4];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    split_pair(v[2 * j], v[2 * j + 1], h[j], l[j]);
    s += (bf2f(h[j]) + bf2f(l[j])) + (bf2f(h[j] >> 16) + bf2f(l[j] >> 16));
  }
  *reinterpret_cast<uint4*>(xh + i0) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4*>(xl + i0) = make_uint4(l[0], l[1], l[2], l[3]);
  s = group_sum<4>(s);
  if ((threadIdx.x & 3) == 0) xg[i0 / 32] = s;
}

// LDS words of the packed input: bf16 layout 8 words per (chunk, lane slot)
// [4 hi pairs | 4 lo pairs]; W4A16 layout 36 words per 32-group
// [16 hi pairs | 16 lo pairs | group sum | pad].
template <int WQ, int KS>
struct Packed {
  static constexpr int kWordsW4 = 36;
  static constexpr int words = WQ ? (KS / 32) * kWordsW4 : KS;
};

// xs (fp32, KS) -> xp (packed pairs in the order lanes consume them)
template <int WQ, int KS>
__device__ void pack_x(const float* xs, uint32_t* xp) {
  using Y = Lay<WQ, KS>;
  for (int p = threadIdx.x; p < KS / 2; p += kGemvThreads) {
    uint32_t hi, lo;
    if (WQ) {
      // 16 consecutive threads hold the 16 pairs of group g: its sum of
      // hi + lo is a 16-lane butterfly
      const int g = p / 16, q = p % 16, j = q / 4, i = q % 4;
      const int k = 32 * g + 8 * j + i;  // pair (k, k + 4) matches the nibble unpack
      split_pair(xs[k], xs[k + 4], hi, lo);
      xp[g * Packed<WQ, KS>::kWordsW4 + q] = hi;
      xp[g * Packed<WQ, KS>::kWordsW4 + 16 + q] = lo;
      const float s = group_sum<16>((bf2f(hi) + bf2f(lo)) + (bf2f(hi >> 16) + bf2f(lo >> 16)));
      if (q == 0) xp[g * Packed<WQ, KS>::kWordsW4 + 32] = __float_as_uint(s);
    } else {
      const int k = 2 * p, c = k / 512, o = k % 512, ls = o / 8, j = (o % 8) / 2;
      split_pair(xs[k], xs[k + 1], hi, lo);
      xp[(c * Y::S + ls) * 8 + j] = hi;
      xp[(c * Y::S + ls) * 8 + 4 + j] = lo;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------ decode attention
constexpr int kMaxHeads = 8;

// One butterfly step of a transposing reduction: lanes whose bit `o` is set
// keep the upper half of their values, the others the lower half; each adds
// its partner's copy of the half it keeps.
template <int H>
__device__ __forceinline__ void tr_step(float* cur, int lane, int o) {
  const bool upper = (lane & o) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = upper ? cur[i] : cur[i + H];
    const float keep = upper ? cur[i + H] : cur[i];
    cur[i] = keep + __shfl_xor(send, o, 64);
  }
}

template <int H, int O>
__device__ __forceinline__ void tr_step_dpp(float* cur, int lane) {
  const bool upper = (lane & O) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = upper ? cur[i] : cur[i + H];
    const float keep = upper ? cur[i + H] : cur[i];
    cur[i] = keep + xor_lane<O>(send);
  }
}

// 32 values per lane -> every lane ends with the full 64-lane sum of value
// tr_index(lane).  The wide steps (16 exchanges, then 8, 4, 2) run on the
// DPP partners 1, 2, 4, 8; only the last two (16, then the pair sum over 32)
// go through the crossbar.  Each step's partner decides one index bit, so
// value bit 4 - i comes from lane bit i (i < 5).
__device__ __forceinline__ int tr_index(int lane) {
  return ((lane & 1) << 4) | ((lane & 2) << 2) | (lane & 4) | ((lane & 8) >> 2) | ((lane & 16) >> 4);
}
__device__ __forceinline__ float transpose_reduce32(float (&v)[32], int lane) {
  tr_step_dpp<16, 1>(v, lane);
  tr_step_dpp<8, 2>(v, lane);
  tr_step_dpp<4, 4>(v, lane);
  tr_step_dpp<2, 8>(v, lane);
  tr_step<1>(v, lane, 16);
  return v[0] + __shfl_xor(v[0], 32, 64);
}

template <int DPL>
__device__ __forceinline__ void load_row(const uint16_t* p, float (&out)[DPL]) {
  if constexpr (DPL == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[2 * i] = bf2f(w[i]); out[2 * i + 1] = bf2f(w[i] >> 16); }
  } else if constexpr (DPL == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = bf2f(v.x); out[1] = bf2f(v.x >> 16); out[2] = bf2f(v.y); out[3] = bf2f(v.y >> 16);
  } else if constexpr (DPL == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    out[0] = bf2f(v); out[1] = bf2f(v >> 16);
  } else {
    out[0] = bf2f(*p);
  }
}

// One head vector of a row: RMS norm over hd (gain optional), then (rope)
// rotate-half RoPE with the position's angles cs/sn [hd/2].  Lane l holds dims
// l*DPL .. l*DPL+DPL-1; the rotation partner of dim d < hd/2 is d + hd/2, held
// by lane l ^ 32.  Used for queries, and for the keys and values written to
// the cache, by both the decode and the prefill path (identical arithmetic).
// Split in two so that a wave issues the reads of all its heads (and the gains
// and angles) before it waits for any: head_raw sums the K-slice partials of
// the projection, head_side reads gain and angles, head_finish does the rest.
template <int HD>
__device__ __forceinline__ void head_raw(const float* raw, int nparts, size_t pstride, int lane,
                                         float (&y)[HD / 64]) {
  constexpr int DPL = HD / 64;
#pragma unroll
  for (int i = 0; i < DPL; ++i) y[i] = ld32(raw + lane * DPL + i);
  for (int q0 = 1; q0 < nparts; q0 += 4) {  // further partials, 4 in flight
    float v[4][DPL];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float* src = q0 + k < nparts ? raw + (size_t)(q0 + k) * pstride : zero_f();
#pragma unroll
      for (int i = 0; i < DPL; ++i) v[k][i] = ld32(src + lane * DPL + i);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < DPL; ++i) y[i] += q0 + k < nparts ? v[k][i] : 0.f;
  }
}

// head_raw for NH heads at once: where the partials number at most MP
// (registers: NH * MP * HD / 64 floats), every read of every head is issued
// before the first sum (one memory round trip instead of one or more per
// head); the sums run in the same order.
template <int HD, int NH, int MP>
__device__ __forceinline__ void heads_raw(const float* const (&raw)[NH], int nparts, size_t pstride,
                                          int lane, float (&y)[NH][HD / 64]) {
  constexpr int DPL = HD / 64;
  if (nparts == 1) {  // (a product not split along K: one read per value)
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < DPL; ++i) y[h][i] = ld32(raw[h] + lane * DPL + i);
    return;
  }
  if (nparts > MP) {
#pragma unroll
    for (int h = 0; h < NH; ++h) head_raw<HD>(raw[h], nparts, pstride, lane, y[h]);
    return;
  }
  float v[NH][MP][DPL];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const float* src = k < nparts ? raw[h] + (size_t)k * pstride : zero_f();
#pragma unroll
      for (int i = 0; i < DPL; ++i) v[h][k][i] = ld32(src + lane * DPL + i);
    }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) y[h][i] = v[h][0][i];
#pragma unroll
    for (int k = 1; k < MP; ++k)
      if (k < nparts)
#pragma unroll
        for (int i = 0; i < DPL; ++i) y[h][i] += v[h][k][i];
  }
}

template <int HD>
struct HeadSide {
  static constexpr int DPL = HD / 64;
  static constexpr int GW = DPL >= 2 ? DPL / 2 : 1;
  uint32_t g[GW];  // gain, raw bf16 pairs (split when used)
  float c[DPL], s[DPL];
  __device__ __forceinline__ float gain(int i) const {
    return DPL == 1 ? bf2f(g[0]) : bf2f((i & 1) ? g[i / 2] >> 16 : g[i / 2]);
  }
};

// gain: may be null (values: no gain); cs/sn: null when there is no rotation.
// Absent operands read the zero row and are not used.
template <int HD>
__device__ __forceinline__ void head_side(const uint16_t* gain, const float* cs, const float* sn,
                                          int lane, HeadSide<HD>& hs) {
  constexpr int DPL = HD / 64;
  const float* zf = reinterpret_cast<const float*>(kZeroRow);
  const uint16_t* gp = gain ? gain : kZeroRow;
  const float* cp = cs ? cs : zf;
  const float* sp = sn ? sn : zf;
  if constexpr (DPL == 1) {
    hs.g[0] = gp[lane];
  } else {
#pragma unroll
    for (int w = 0; w < DPL / 2; ++w) hs.g[w] = reinterpret_cast<const uint32_t*>(gp + lane * DPL)[w];
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int ii = (lane & 31) * DPL + i;
    hs.c[i] = ld32(cp + ii);
    hs.s[i] = ld32(sp + ii);
  }
}

template <int HD>
__device__ __forceinline__ void head_finish(float (&y)[HD / 64], const HeadSide<HD>& hs, bool gain,
                                            bool rope, int lane, float eps) {
  constexpr int DPL = HD / 64;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) ss = fmaf(y[i], y[i], ss);
  const float rr = rsqrtf(wave_sum(ss) / (float)HD + eps);
#pragma unroll
  for (int i = 0; i < DPL; ++i) y[i] = y[i] * rr * (gain ? hs.gain(i) : 1.0f);
  if (rope) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const float other = __shfl_xor(y[i], 32, 64);
      const float os = other * hs.s[i];
      y[i] = fmaf(y[i], hs.c[i], lane < 32 ? -os : os);
    }
  }
}

template <int HD>
__device__ __forceinline__ void head_vec(const float* raw, int nparts, size_t pstride,
                                         const uint16_t* gain, bool rope, const float* cs,
                                         const float* sn, int lane, float eps,
                                         float (&y)[HD / 64]) {
  HeadSide<HD> hs;
  head_side<HD>(gain, rope ? cs : nullptr, rope ? sn : nullptr, lane, hs);
  head_raw<HD>(raw, nparts, pstride, lane, y);
  head_finish<HD>(y, hs, gain != nullptr, rope, lane, eps);
}

// One wave's K/V rows for a group of 4 keys, kept packed until used: bf16
// (KQ = 0), or int8 codes with each key's row scale (KQ = 1).
template <int DPL, int KQ = 0>
struct KvGroup {
  // 32-bit words per lane per row
  static constexpr int W = KQ ? (DPL >= 4 ? DPL / 4 : 1) : (DPL >= 2 ? DPL / 2 : 1);
  uint32_t k[4][W], v[4][W];
  float ks[4], vs[4];  // int8: the keys' row scales
};

template <int DPL>
__device__ __forceinline__ void load_packed(const uint16_t* p, uint32_t (&w)[KvGroup<DPL>::W]) {
  if constexpr (DPL == 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  } else if constexpr (DPL == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    w[0] = u.x; w[1] = u.y;
  } else if constexpr (DPL == 2) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    w[0] = *p;
  }
}

template <int DPL>
__device__ __forceinline__ void unpack(const uint32_t (&w)[KvGroup<DPL>::W], float (&out)[DPL]) {
  if constexpr (DPL == 1) {
    out[0] = bf2f(w[0]);
  } else {
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i) { out[2 * i] = bf2f(w[i]); out[2 * i + 1] = bf2f(w[i] >> 16); }
  }
}

// int8 rows: a lane's DPL codes (DPL bytes)
template <int DPL>
__device__ __forceinline__ void load_codes(const int8_t* p, uint32_t (&w)[KvGroup<DPL, 1>::W]) {
  if constexpr (DPL == 8) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    w[0] = u.x; w[1] = u.y;
  } else if constexpr (DPL == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (DPL == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    w[0] = *reinterpret_cast<const uint8_t*>(p);
  }
}

// code * row scale, as fp32 (one rounding)
template <int DPL>
__device__ __forceinline__ void unpack_i8(const uint32_t (&w)[KvGroup<DPL, 1>::W], float s, float (&out)[DPL]) {
#pragma unroll
  for (int i = 0; i < DPL; ++i) out[i] = (float)(int8_t)((w[i / 4] >> (8 * (i % 4))) & 0xFFu) * s;
}

// One cached row held by a wave (lane l: values l*DPL ..) stored as int8:
// scale s = max |y| / 127, code = nearest-even(y / s) (0 for a row of
// zeros), decided in fp32; deq receives code * s, what a read of the cache
// gives back.  The whole wave must be active.
template <int DPL>
__device__ __forceinline__ void store_int8_row(const float (&y)[DPL], int8_t* codes, float* scale, int lane,
                                               float (&deq)[DPL]) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) am = fmaxf(am, fabsf(y[i]));
  am = wave_max(am);
  const float s = am / 127.0f;
  uint32_t w[KvGroup<DPL, 1>::W];
#pragma unroll
  for (int j = 0; j < KvGroup<DPL, 1>::W; ++j) w[j] = 0u;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    float c = s > 0.f ? rintf(y[i] / s) : 0.f;
    c = fminf(fmaxf(c, -127.f), 127.f);
    w[i / 4] |= ((uint32_t)(int)c & 0xFFu) << (8 * (i % 4));
    deq[i] = c * s;
  }
  int8_t* dst = codes + lane * DPL;
  if constexpr (DPL == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  else if constexpr (DPL == 4) *reinterpret_cast<uint32_t*>(dst) = w[0];
  else if constexpr (DPL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0];
  else *reinterpret_cast<uint8_t*>(dst) = (uint8_t)w[0];
  if (lane == 0) *scale = s;
}

// Block (chunk c, row r): the keys j0..j1-1 of chunk c of the row's window,
// all query heads against the single K/V head.  The block normalises and
// rotates the row's queries itself (q_norm with gain, rotate-half RoPE at the
// logical position).  With own_kv (decode: every row is its own sequence) the
// block whose chunk holds the row's position also norms, rotates and stores
// that position's key and value (bf16) before attending, so no separate pass
// is needed; for prefill the cache is written by k_kv_write first.
// Lanes own hd/64 consecutive dims; each wave takes groups of 4 keys, reduces
// the 32 (key, head) dot products with a transposing butterfly (31 shuffles),
// and keeps an online softmax (max, sum, o) per head.  The 4 waves merge in
// LDS and write one (max, sum, o) partial per (row, head, chunk).
// Block (chunk c, row r): the keys j0..j1-1 of chunk c of the row's window,
// all query heads against the single K/V head; 4 waves take groups of 4 keys,
// the next group's K/V rows loaded while the current one is used.  Queries
// are normed and rotated in the block (angles from the per-row table).  With
// own K/V (decode, the layer computes K/V) the block holding the position
// norms, rotates and stores that position's key and value (bf16) and uses
// them from LDS.  Every block writes a (max, sum, o) partial per head;
// k_attn_combine merges them.  (Merging in the row's last block instead needs
// a device-scope fence per block, which writes back the L2 and costs more
// than the extra launch.)
template <int HD, int KQ>
__device__ void attn_chunk(const Rows& R, const AttnArgs& a, int c, int r) {
  constexpr int DPL = HD / 64;
  constexpr int NH = kMaxHeads;
  using G = KvGroup<DPL, KQ>;
  __shared__ float qs[NH * HD];
  __shared__ float kv_own[2][HD];
  __shared__ float pw[4][32];
  __shared__ float cw[4][NH];
  __shared__ float wm[4][NH], wl[4][NH];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6, nq = a.nq;
  const int pos = clamp_pos(R, row_pos(R, r));
  const int seq = row_seq(R, r);
  const int lo = a.window ? max(0, pos - a.window + 1) : 0;
  // the row's live span split over the grid's chunks, at least a.chunk keys
  // each: the chunks that hold keys are a prefix of the grid
  const int span = pos + 1 - lo;
  const int chunk = max(a.chunk, (span + a.nchunk - 1) / a.nchunk);
  const int j0 = lo + c * chunk;
  const int j1 = min(j0 + chunk, pos + 1);
  const size_t hstride = (size_t)kMaxChunks * (HD + 2);
  float* part = a.part + ((size_t)r * nq * kMaxChunks + c) * (HD + 2);

  if (j0 < j1) {
    const bool own = a.kc_own != nullptr && j1 == pos + 1;
    // bf16 rows, or int8 rows plus one scale per key; row of a key: cache_row
    const uint16_t* kb = static_cast<const uint16_t*>(a.kc) + lane * DPL;
    const uint16_t* vb = static_cast<const uint16_t*>(a.vc) + lane * DPL;
    const int8_t* kb8 = static_cast<const int8_t*>(a.kc) + lane * DPL;
    const int8_t* vb8 = static_cast<const int8_t*>(a.vc) + lane * DPL;
    const int ngroups = (j1 - j0 + 3) / 4;
    // K/V rows of a group.  Keys past the chunk, and the own position (which
    // this block writes), read the zero row instead (loads are unconditional:
    // a select right after a load would wait for it); row_of takes the own
    // position from the block's own K/V
    auto load_group = [&](int gi, G& g) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int key = j0 + 4 * gi + k;
        const bool ok = gi < ngroups && key < j1 && !(own && key == pos);
        const size_t row = cache_row(R, seq, ok ? key : lo);
        if constexpr (KQ) {
          const int8_t* z = reinterpret_cast<const int8_t*>(kZeroRow) + lane * DPL;
          load_codes<DPL>(ok ? kb8 + row * HD : z, g.k[k]);
          load_codes<DPL>(ok ? vb8 + row * HD : z, g.v[k]);
          g.ks[k] = *(ok ? a.ks + row : zero_f());
          g.vs[k] = *(ok ? a.vs + row : zero_f());
        } else {
          const uint16_t* kr = ok ? kb + row * HD : kZeroRow + lane * DPL;
          const uint16_t* vr = ok ? vb + row * HD : kZeroRow + lane * DPL;
          load_packed<DPL>(kr, g.k[k]);
          load_packed<DPL>(vr, g.v[k]);
        }
      }
    };
    G cur;
    load_group(wave, cur);  // issued before the query work: independent of it

    const int nraw = nq + (a.owns ? 2 : 0);
    const float* raw = a.qkv + (size_t)r * nraw * HD;
    const float* cs = a.rope + (size_t)r * a.rope_ld + a.rope_off;
    const float* sn = cs + HD / 2;
    // reads first (every head of this wave, its own K/V, gains, angles), then
    // the arithmetic: one round trip instead of one per head
    constexpr int HW = (kMaxHeads + 3) / 4;  // query heads per wave
    const bool own_kv = own && wave < 2;
    // (all unconditional: heads past nq and K/V rows a block does not own read
    // head 0 and are not used)
    HeadSide<HD> sq, sk;
    head_side<HD>(a.gq, cs, sn, lane, sq);
    head_side<HD>(own_kv && wave == 0 ? a.gk : nullptr, cs, sn, lane, sk);
    float yq[HW][DPL], yk[DPL];  // this wave's query heads, its own K or V row
    if constexpr (HD >= 512 && KQ) {  // (too few registers left for all reads at once)
#pragma unroll
      for (int x = 0; x < HW; ++x)
        head_raw<HD>(raw + (wave + 4 * x < nq ? wave + 4 * x : 0) * HD, a.qkv_parts, a.qkv_pstride,
                     lane, yq[x]);
      head_raw<HD>(raw + (own_kv ? nq + wave : 0) * HD, a.qkv_parts, a.qkv_pstride, lane, yk);
    } else {
      const float* srcs[HW + 1];
#pragma unroll
      for (int x = 0; x < HW; ++x) srcs[x] = raw + (wave + 4 * x < nq ? wave + 4 * x : 0) * HD;
      srcs[HW] = raw + (own_kv ? nq + wave : 0) * HD;
      float yy[HW + 1][DPL];
      heads_raw<HD, HW + 1, HD >= 512 ? 4 : 8>(srcs, a.qkv_parts, a.qkv_pstride, lane, yy);
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
#pragma unroll
        for (int x = 0; x < HW; ++x) yq[x][i] = yy[x][i];
        yk[i] = yy[HW][i];
      }
    }
#pragma unroll
    for (int x = 0; x < HW; ++x) {
      const int h = wave + 4 * x;
      if (h < nq) {
        head_finish<HD>(yq[x], sq, a.gq != nullptr, true, lane, a.eps);
#pragma unroll
        for (int i = 0; i < DPL; ++i) qs[h * HD + lane * DPL + i] = yq[x][i];
      }
    }
    if (own_kv) {
      const bool is_v = wave == 1;
      head_finish<HD>(yk, sk, !is_v && a.gk != nullptr, !is_v, lane, a.eps);
      const size_t slot = cache_row(R, seq, pos);
      if constexpr (KQ) {
        float deq[DPL];
        store_int8_row<DPL>(yk, static_cast<int8_t*>(is_v ? a.vc_own : a.kc_own) + slot * HD,
                            (is_v ? a.vs_own : a.ks_own) + slot, lane, deq);
#pragma unroll
        for (int i = 0; i < DPL; ++i) kv_own[wave][lane * DPL + i] = deq[i];
      } else {
        uint16_t* dst = static_cast<uint16_t*>(is_v ? a.vc_own : a.kc_own) + slot * HD;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const uint32_t b = f2bf(yk[i]);
          st16(dst + lane * DPL + i, (uint16_t)b);
          kv_own[wave][lane * DPL + i] = bf2f(b);
        }
      }
    }
    __syncthreads();

    // this lane's query dims for every head
    float qr[NH][DPL];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < DPL; ++i) qr[h][i] = h < nq ? qs[h * HD + lane * DPL + i] : 0.f;

    const float scale = rsqrtf((float)HD);
    // value index k * 8 + h of this lane after the transposing reduction: the
    // 4 keys of a head sit in lane bits 0-1 (DPP partners 1 and 2)
    const int vidx = tr_index(lane), myh = vidx & 7, myk = vidx >> 3;
    float m_run = -INFINITY, l_run = 0.f;
    float o[NH][DPL];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[h][i] = 0.f;

    for (int gi = wave; gi < ngroups; gi += 4) {
      // the next group's reads, if this wave has one (a wave's last group
      // must not wait for reads that nothing uses)
      const bool more = gi + 4 < ngroups;
      G nxt;
      if constexpr (DPL < 8)
        if (more) load_group(gi + 4, nxt);  // hd 512: registers too tight
      const int key0 = j0 + 4 * gi;
      // key / value row k of the group as fp32 (unpacked when used)
      auto row_of = [&](int k, int which, float (&x)[DPL]) {
        if (own && key0 + k == pos) {
#pragma unroll
          for (int i = 0; i < DPL; ++i) x[i] = kv_own[which][lane * DPL + i];
        } else if constexpr (KQ) {
          unpack_i8<DPL>(which ? cur.v[k] : cur.k[k], which ? cur.vs[k] : cur.ks[k], x);
        } else {
          unpack<DPL>(which ? cur.v[k] : cur.k[k], x);
        }
      };
      float part32[32];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float kr[DPL];
        row_of(k, 0, kr);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < DPL; ++i) d = fmaf(qr[h][i], kr[i], d);
          part32[k * NH + h] = d;
        }
      }
      float sc_ = transpose_reduce32(part32, lane) * scale;
      if (key0 + myk >= j1 || myh >= nq) sc_ = -INFINITY;
      float mx = fmaxf(sc_, xor_lane<1>(sc_));
      mx = fmaxf(mx, xor_lane<2>(mx));
      const float m_new = fmaxf(m_run, mx);
      const float pr = (m_new == -INFINITY || sc_ == -INFINITY) ? 0.f : expf(sc_ - m_new);
      const float corr = (m_new == -INFINITY || m_run == -INFINITY)
                             ? (m_run == -INFINITY ? 0.f : 1.f)
                             : expf(m_run - m_new);
      float ps = pr + xor_lane<1>(pr);
      ps += xor_lane<2>(ps);
      l_run = fmaf(l_run, corr, ps);
      m_run = m_new;
      if (lane < 32) pw[wave][vidx] = pr;
      if (lane < 32 && myk == 0) cw[wave][myh] = corr;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float cf = cw[wave][h];
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[h][i] *= cf;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float vr[DPL];
        row_of(k, 1, vr);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const float pk = pw[wave][k * NH + h];
#pragma unroll
          for (int i = 0; i < DPL; ++i) o[h][i] = fmaf(pk, vr[i], o[h][i]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (more) {
        if constexpr (DPL < 8) cur = nxt;
        else load_group(gi + 4, cur);
      }
    }
    // merge the four waves: per head max M, then rescale and sum.  Each wave
    // parks its o in LDS (wave 0 in qs, whose queries are in registers); the
    // factors are formed once per (wave, head); every element then sums the
    // four in wave order (the same arithmetic as folding them in one by one)
    __shared__ float op[3][NH * HD];
    __shared__ float fw[4][NH];
    if (lane < 32 && myk == 0) {
      wm[wave][myh] = m_run;
      wl[wave][myh] = l_run;
    }
    float* mine = wave == 0 ? qs : op[wave - 1];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < DPL; ++i) mine[h * HD + lane * DPL + i] = o[h][i];
    __syncthreads();
    if (t < 4 * NH) {
      const int w = t / NH, h = t % NH;
      float M = wm[0][h];
      for (int x = 1; x < 4; ++x) M = fmaxf(M, wm[x][h]);
      fw[w][h] = (wm[w][h] == -INFINITY) ? 0.f : expf(wm[w][h] - M);
    }
    if (t < nq) {
      float M = wm[0][t];
      for (int x = 1; x < 4; ++x) M = fmaxf(M, wm[x][t]);
      float L = 0.f;
      for (int x = 0; x < 4; ++x)
        if (wm[x][t] != -INFINITY) L = fmaf(wl[x][t], expf(wm[x][t] - M), L);
      st32(part + t * hstride + HD, M);
      st32(part + t * hstride + HD + 1, L);
    }
    __syncthreads();
    for (int idx = t; idx < nq * HD; idx += 256) {
      const int h = idx / HD, d = idx % HD;
      float a_ = qs[idx] * fw[0][h];
      a_ = fmaf(op[0][idx], fw[1][h], a_);
      a_ = fmaf(op[1][idx], fw[2][h], a_);
      a_ = fmaf(op[2][idx], fw[3][h], a_);
      st32(part + h * hstride + d, a_);
    }
  } else if (t < nq) {  // no keys in this chunk
    st32(part + t * hstride + HD, -INFINITY);
    st32(part + t * hstride + HD + 1, 0.f);
  }
}

// out[r][h*hd + d] = sum_c e^(m_c - M) o_c[d] / sum_c e^(m_c - M) l_c over the
// chunks holding keys.  Those are a prefix of the chunk list (keys are split in
// order); empty chunks leave o unwritten, so they are never read.
__device__ void attn_combine(const AttnArgs& a, int r, int h) {
  __shared__ float wn[kMaxChunks];
  __shared__ float sh[8];
  __shared__ int na[4];
  const int hd = a.hd, t = threadIdx.x;
  const size_t hstride = (size_t)kMaxChunks * (hd + 2);
  const float* part = a.part + ((size_t)r * a.nq + h) * hstride;
  // the o values of the first kPre chunks are read together with (m, l), before
  // the weights are known (slots past the last written chunk hold stale
  // values, and chunks past nchunk read the zero row: dropped by a select,
  // never multiplied)
  constexpr int kPre = 32, kDt = 2;  // hd <= 512 = kDt * 256
  float pv[kDt][kPre];
#pragma unroll
  for (int it = 0; it < kDt; ++it) {
    const int d = t + 256 * it < hd ? t + 256 * it : 0;
#pragma unroll
    for (int c = 0; c < kPre; ++c)
      pv[it][c] = c < a.nchunk ? ld32(part + (size_t)c * (hd + 2) + d) : ld32(zero_f() + d);
  }
  float mc = -INFINITY, lc = 0.f;
  if (t < a.nchunk) {
    mc = ld32(part + (size_t)t * (hd + 2) + hd);
    lc = ld32(part + (size_t)t * (hd + 2) + hd + 1);
  }
  const bool act = lc > 0.f;
  float M = act ? mc : -INFINITY;
  int nact = act ? t + 1 : 0;
  M = wave_max(M);
  nact = wave_max_i(nact);
  if ((t & 63) == 0) {
    sh[t >> 6] = M;
    na[t >> 6] = nact;
  }
  __syncthreads();
  M = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  nact = max(max(na[0], na[1]), max(na[2], na[3]));
  const float w = act ? expf(mc - M) : 0.f;
  const float L = block_sum<256>(w * lc, sh + 4);
  if (t < kMaxChunks) wn[t] = w / L;
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kDt; ++it) {
    const int d = t + 256 * it;
    if (d >= hd) break;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    // (explicit fma: the same rounding in every instantiation)
    for (int c = 0; c < kPre; c += 4) {
      o0 = c < nact ? fmaf(wn[c], pv[it][c], o0) : o0;
      o1 = c + 1 < nact ? fmaf(wn[c + 1], pv[it][c + 1], o1) : o1;
      o2 = c + 2 < nact ? fmaf(wn[c + 2], pv[it][c + 2], o2) : o2;
      o3 = c + 3 < nact ? fmaf(wn[c + 3], pv[it][c + 3], o3) : o3;
    }
    int cc = kPre;
    for (; cc + 4 <= nact; cc += 4) {
      o0 = fmaf(wn[cc], ld32(part + (size_t)cc * (hd + 2) + d), o0);
      o1 = fmaf(wn[cc + 1], ld32(part + (size_t)(cc + 1) * (hd + 2) + d), o1);
      o2 = fmaf(wn[cc + 2], ld32(part + (size_t)(cc + 2) * (hd + 2) + d), o2);
      o3 = fmaf(wn[cc + 3], ld32(part + (size_t)(cc + 3) * (hd + 2) + d), o3);
    }
    for (; cc < nact; ++cc) o0 = fmaf(wn[cc], ld32(part + (size_t)cc * (hd + 2) + d), o0);
    const float v = (o0 + o1) + (o2 + o3);
    if (a.xh) {  // the O product's prepared input: hi + lo = v, group sums of 32
      const size_t K = (size_t)a.nq * hd, i = (size_t)r * K + (size_t)h * hd + d;
      const uint32_t hb = f2bf(v), lb = f2bf(v - bf2f(hb));
      a.xh[i] = (uint16_t)hb;
      a.xl[i] = (uint16_t)lb;
      // (32 consecutive d are the lanes of one half wave: hd is a multiple of
      // 64, so a wave is either whole in this loop or has left it)
      const float gs = lanes_sum<32>(bf2f(hb) + bf2f(lb));
      if ((d & 31) == 0) a.xg[i / 32] = gs;
    } else {
      st32(a.out + (size_t)r * a.nq * hd + (size_t)h * hd + d, v);
    }
  }
}

}  // namespace e2b
