// The batched (matrix-core) product of libe2b for CDNA4 (gfx950): the kernel
// template and its launch dispatch, compiled once per weight format
// (gemm_bf16.hip, gemm_w4.hip) so the two sets of instantiations build in
// parallel.
#pragma once

#include "dev_common.h"

#include <float.h>
#include <type_traits>

namespace e2b {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16- and 8-byte loads into registers, built from scalars (a plain struct
// copy of a load into a register array can become a memory copy that keeps
// the array in scratch memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8u(const void* p) {
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
  return make_uint2(v.x, v.y);
}

// eight int4 codes (one packed word) -> eight bf16 values 128 + c
__device__ __forceinline__ uint4 w4_to_bf16(uint32_t word) {
  const uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
  const uint32_t u = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // codes 0,1,2,3 as bytes
  const uint32_t v = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // codes 4,5,6,7
  uint4 r;
  r.x = __builtin_amdgcn_perm(0x43434343u, u, 0x04010400u);
  r.y = __builtin_amdgcn_perm(0x43434343u, u, 0x04030402u);
  r.z = __builtin_amdgcn_perm(0x43434343u, v, 0x04010400u);
  r.w = __builtin_amdgcn_perm(0x43434343u, v, 0x04030402u);
  return r;
}

// input rows per block: 16 * MT (MT m-tiles of 16 rows; 1, 2 or 4, chosen
// from the row count so that 2-16 rows do not pay for 64)
constexpr int kKC = 128;        // k per LDS stage (4 k-steps of 32)
constexpr int kAP = kKC + 8;    // padded LDS row of bf16: 16-byte reads conflict-free

// Block = 4 waves side by side along N; wave w owns NT column tiles of 16
// (block covers 64*NT columns) for all 16*MT rows, over one K slice of KS.
// A chunks (16*MT rows x 128 k, hi and lo) are double-buffered in LDS, one
// barrier per chunk; each wave's weight fragments for the next chunk are
// loaded into registers while the current chunk is multiplied.
template <int WQ, int NT, int MT, int FA, int TAG, int TQ>
__global__ __launch_bounds__(256, 2) void k_gemm(Lin W, int rows, GemmA A, int KS, Epilogue epi) {
  constexpr int MB = 16 * MT;
  const uint16_t* __restrict__ xh = A.xh;
  const uint16_t* __restrict__ xl = A.xl;
  const float* __restrict__ xg = A.xg;
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][2][MB][kAP];
  __shared__ __attribute__((aligned(16))) float sg[2][kKC / 32][MB];  // 136 * group sums
  __shared__ float rv[4][MB];
  __shared__ int ri[4][MB];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, kq = lane >> 4;
  const int ks = blockIdx.y, m0 = blockIdx.z * MB;
  const int K = W.K, N = W.N;
  const int mrows = min(MB, rows - m0);
  int ncol[NT];
  // (GeGLU epilogue: waves 0-1 take gate columns c0 .. c0 + 32 NT - 1, waves
  // 2-3 the matching up columns gi + c0 ..)
  const bool geglu = TAG == kTagGateUp && epi.gh != nullptr;
#pragma unroll
  for (int j = 0; j < NT; ++j)
    ncol[j] = geglu ? (wave >> 1) * epi.gi + blockIdx.x * 32 * NT + (wave & 1) * 16 * NT + 16 * j + (lane & 15)
                    : blockIdx.x * 64 * NT + wave * 16 * NT + 16 * j + (lane & 15);

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // weight fragments of one chunk (4 k-steps)
  // weight fragments: a ring of D chunks, D - 1 of them in flight ahead
  constexpr int D = WQ ? (NT >= 4 ? 2 : 4) : (NT >= 2 ? 3 : 4);
  // (loaded values are kept raw until the multiply: an operation on a loaded
  // value right after the load would wait for it, and with it for every load
  // issued before it)
  uint4 bw[D][WQ ? 1 : 4][WQ ? 1 : NT];
  uint32_t bq[D][WQ ? 4 : 1][WQ ? NT : 1];
  uint32_t bs[D][WQ ? 2 : 1][WQ ? NT : 1];  // W4A16 scales: bf16 pairs (groups 2i, 2i + 1)
  // A chunk staged through registers
  uint4 rah[MT], ral[MT];
  float rg = 0.f, rgs[MT];  // (rg: the raw group sum, scaled when staged)
#pragma unroll
  for (int j = 0; j < MT; ++j) rgs[j] = 0.f;
  float raf[FA ? MT : 1][8];  // fp32 input slots (FA)
#pragma unroll
  for (int x = 0; x < D; ++x) {
#pragma unroll
    for (int s = 0; s < (WQ ? 1 : 4); ++s)
#pragma unroll
      for (int j = 0; j < (WQ ? 1 : NT); ++j) bw[x][s][j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < (WQ ? 4 : 1); ++s)
#pragma unroll
      for (int j = 0; j < (WQ ? NT : 1); ++j) bq[x][s][j] = 0x88888888u;
#pragma unroll
    for (int s = 0; s < (WQ ? 2 : 1); ++s)
#pragma unroll
      for (int j = 0; j < (WQ ? NT : 1); ++j) bs[x][s][j] = 0u;
  }

  const int kbeg = ks * KS, kend = kbeg + KS;
  // (buffer indices are compile-time constants so the fragments stay in registers)
  // Out-of-range operands are read at a valid address and never zeroed: a
  // column past N (row 0 read) or a row past the pass (element 0 read) only
  // reaches its own output column or row, which is never stored, and k past
  // the slice is never multiplied (the k-steps stop at kcn, a multiple of 32).
  auto load_b = [&](auto BUF, int kc, int kcn) {
    constexpr int buf = decltype(BUF)::value;
    if constexpr (WQ && TQ) {
      {
        // the tiled copy: a lane's four code words of the chunk (k-steps
        // 0..3) in 16 bytes, its column's four group scales in 8 (the chunk
        // is one 128-k block: slices are whole blocks on this path)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const size_t row = ncol[j] < N ? (size_t)ncol[j] : 0;
          const size_t blk = (row / 16) * (K / 128) + (size_t)kc / 128;
          const uint4 qv = ld16(W.tq + (blk * 64 + lane) * 4);
          const uint2 sv = ld8u(W.ts + (blk * 16 + (lane & 15)) * 4);
          bq[buf][0][j] = qv.x;
          bq[buf][1][j] = qv.y;
          bq[buf][2][j] = qv.z;
          bq[buf][3][j] = qv.w;
          bs[buf][0][j] = sv.x;
          bs[buf][1][j] = sv.y;
        }
        return;
      }
    }
    // (every k-step is read, a k-step past kcn at the chunk's first group:
    // the same loads on every path keep the compiler's wait counts exact)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const size_t row = ncol[j] < N ? (size_t)ncol[j] : 0;
        const size_t g = (size_t)(kc + (32 * s < kcn ? 32 * s : 0)) / 32;
        if constexpr (WQ) {  // (no tiled copy: one word and one scale per k-step)
          bq[buf][s][j] = W.q[row * (K / 8) + 4 * g + kq];
          const uint32_t sv = W.s[row * (K / 32) + g];
          bs[buf][s >> 1][j] = (s & 1) ? (bs[buf][s >> 1][j] | (sv << 16)) : sv;
        } else {
          // (the tiled copy when there is one: one contiguous kilobyte per wave)
          const uint16_t* wp = W.tw ? W.tw + (((row / 16) * (K / 32) + g) * 64 + lane) * 8
                                    : W.w + row * K + 32 * g + 8 * kq;
          bw[buf][s][j] = ld16(wp);
        }
      }
    }
  };
  auto load_a = [&](int kc, int kcn) {
    if constexpr (FA) {  // fp32 rows: loaded now, split when stored (after the multiply)
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int idx = t + 256 * j, m = idx >> 4, k8 = idx & 15;
        const bool ok = m < mrows && 8 * k8 < kcn;
        ld8(A.a + (ok ? (size_t)(m0 + m) * A.lda + kc + 8 * k8 : 0), raf[j]);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int idx = t + 256 * j, m = idx >> 4, k8 = idx & 15;
      const bool ok = m < mrows && 8 * k8 < kcn;
      const size_t o = ok ? (size_t)(m0 + m) * K + kc + 8 * k8 : 0;
      rah[j] = ld16(xh + o);
      ral[j] = ld16(xl + o);
    }
    if (WQ) {
      const int m = t >> 2, g = t & 3;
      const bool ok = m < mrows && 32 * g < kcn;
      rg = xg[ok ? (size_t)(m0 + m) * (K / 32) + kc / 32 + g : 0];
    }
  };
  auto store_a = [&](int st) {
    if constexpr (FA) {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        uint32_t h[4], l[4];
        float gs = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          split_pair(raf[j][2 * x], raf[j][2 * x + 1], h[x], l[x]);
          gs += (bf2f(h[x]) + bf2f(l[x])) + (bf2f(h[x] >> 16) + bf2f(l[x] >> 16));
        }
        rah[j] = make_uint4(h[0], h[1], h[2], h[3]);
        ral[j] = make_uint4(l[0], l[1], l[2], l[3]);
        if (WQ) {  // group of 32 = the 4 consecutive lanes with the same row
          gs = group_sum<4>(gs);
          rgs[j] = 136.0f * gs;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int idx = t + 256 * j, m = idx >> 4, k8 = idx & 15;
      *reinterpret_cast<uint4*>(&sa[st][0][m][8 * k8]) = rah[j];
      *reinterpret_cast<uint4*>(&sa[st][1][m][8 * k8]) = ral[j];
    }
    if constexpr (WQ && FA) {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int idx = t + 256 * j, m = idx >> 4, k8 = idx & 15;
        if ((k8 & 3) == 0) sg[st][k8 >> 2][m] = rgs[j];
      }
    } else if (WQ) {
      if ((t >> 2) < MB) sg[st][t & 3][t >> 2] = 136.0f * rg;
    }
  };

  const int nch = (KS + kKC - 1) / kKC;
  // one chunk: issue the weight loads of chunk c + D - 1 and the activation
  // loads of chunk c + 1, multiply chunk c, stage chunk c + 1 in LDS
  auto chunk = [&](auto BUF, int c) {
    constexpr int buf = decltype(BUF)::value;
    // A chunk past the slice (the ring's tail) multiplies nothing, but it
    // issues the same loads, at the last chunk's addresses: every path then
    // has the same loads in flight, so the compiler waits only for the ones
    // the multiply uses
    const bool live = c < nch;
    const int cl = live ? c : nch - 1;
    const int kc = kbeg + cl * kKC, kcn = min(kKC, kend - kc), st = cl & 1;
    const bool more = c + 1 < nch;
    // (activation loads first: loads complete in issue order, and staging
    // chunk c + 1 must not wait for the weight loads issued after it)
    const int ka = more ? kc + kKC : kc;
    load_a(ka, min(kKC, kend - ka));
    __builtin_amdgcn_sched_barrier(0);  // (keep every activation load ahead of the weights)
    {
      const int cf = min(c + D - 1, nch - 1), kf = kbeg + cf * kKC;
      load_b(std::integral_constant<int, (buf + D - 1) % D>(), kf, min(kKC, kend - kf));
    }
    if (!live) return;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (32 * s >= kcn) break;
      bf16x8_t B[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if constexpr (WQ) B[j] = as_bf16x8(w4_to_bf16(bq[buf][s][j]));
        else B[j] = as_bf16x8(bw[buf][s][j]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int mr = 16 * mt + (lane & 15);
        const bf16x8_t Ah = as_bf16x8(*reinterpret_cast<const uint4*>(&sa[st][0][mr][32 * s + 8 * kq]));
        const bf16x8_t Al = as_bf16x8(*reinterpret_cast<const uint4*>(&sa[st][1][mr][32 * s + 8 * kq]));
        if constexpr (WQ) {
          const float4 g4 = *reinterpret_cast<const float4*>(&sg[st][s][16 * mt + 4 * kq]);
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            f32x4_t d = f32x4_t{0.f, 0.f, 0.f, 0.f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B[j], d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B[j], d, 0, 0, 0);
            const float sc = bf2f((s & 1) ? bs[buf][s >> 1][j] >> 16 : bs[buf][s >> 1][j]);
            acc[mt][j][0] = fmaf(sc, d[0] - g4.x, acc[mt][j][0]);
            acc[mt][j][1] = fmaf(sc, d[1] - g4.y, acc[mt][j][1]);
            acc[mt][j][2] = fmaf(sc, d[2] - g4.z, acc[mt][j][2]);
            acc[mt][j][3] = fmaf(sc, d[3] - g4.w, acc[mt][j][3]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B[j], acc[mt][j], 0, 0, 0);
            acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B[j], acc[mt][j], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_a(st ^ 1);
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;

  load_a(kbeg, min(kKC, KS));
  load_b(C0(), kbeg, min(kKC, KS));
  if constexpr (D > 2) {
    const int k1 = kbeg + min(1, nch - 1) * kKC;
    load_b(C1(), k1, min(kKC, kend - k1));
  }
  if constexpr (D > 3) {
    const int k2 = kbeg + min(2, nch - 1) * kKC;
    load_b(C2(), k2, min(kKC, kend - k2));
  }
  store_a(0);
  __syncthreads();
  for (int c = 0; c < nch; c += D) {
    chunk(C0(), c);
    chunk(C1(), c + 1);
    if constexpr (D > 2) chunk(C2(), c + 2);
    if constexpr (D > 3) chunk(C3(), c + 3);
  }

  if constexpr (TAG == kTagGateUp) {
    if (geglu) {
      // gate and up tiles side by side in LDS (the A stages are free: every
      // wave has passed the last chunk's barrier), then gelu_tanh(gate) * up
      // for 8 consecutive columns per thread, emitted as the down product's
      // prepared input (four consecutive threads cover one 32-column group)
      constexpr int SP = 64 * NT + 4;
      static_assert(sizeof(sa) >= sizeof(float) * MB * SP, "GeGLU tile fits in the A stages");
      float* ep = reinterpret_cast<float*>(&sa[0][0][0][0]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            ep[(16 * mt + 4 * kq + i) * SP + (wave >> 1) * 32 * NT + (wave & 1) * 16 * NT + 16 * j + (lane & 15)] =
                acc[mt][j][i];
      __syncthreads();
      const int c0 = blockIdx.x * 32 * NT, I = epi.gi;
      for (int it = t; it < MB * 4 * NT; it += 256) {
        const int m = it / (4 * NT), c8 = it % (4 * NT);
        if (m >= mrows) continue;  // (the four threads of a group share m)
        const float* g = ep + m * SP + 8 * c8;
        float v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = gelu_tanh(g[x]) * g[32 * NT + x];
        const size_t r = (size_t)(m0 + m);
        emit8(v, epi.gh + r * I, epi.gl + r * I, epi.gg + r * (I / 32), c0 + 8 * c8);
      }
      return;
    }
  }
  if (!epi.argmax) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * kq + i;
        if (m < mrows)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            if (ncol[j] < N) epi.y[((size_t)ks * rows + m0 + m) * N + ncol[j]] = acc[mt][j][i];
      }
    return;
  }
  // argmax: per row, best (value, lowest index) over this block's columns
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * mt + 4 * kq + i;
      float v = -FLT_MAX;
      int x = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (ncol[j] < N) {
          const float a_ = acc[mt][j][i];
          if (epi.logits && m < mrows) epi.logits[(size_t)(m0 + m) * N + ncol[j]] = a_;
          if (a_ > v || (a_ == v && ncol[j] < x)) {
            v = a_;
            x = ncol[j];
          }
        }
      argmax_lanes<16>(v, x);
      if ((lane & 15) == 0) {
        rv[wave][m] = v;
        ri[wave][m] = x;
      }
    }
  __syncthreads();
  if (t < mrows) {
    float v = rv[0][t];
    int x = ri[0][t];
    for (int w = 1; w < 4; ++w)
      if (rv[w][t] > v || (rv[w][t] == v && ri[w][t] < x)) {
        v = rv[w][t];
        x = ri[w][t];
      }
    epi.cand_val[(size_t)(m0 + t) * gridDim.x + blockIdx.x] = v;
    epi.cand_idx[(size_t)(m0 + t) * gridDim.x + blockIdx.x] = x;
  }
}

template <int WQ, int NT, int FA, int TAG>
static hipError_t run_gemm(const Lin& W, int rows, const GemmA& A, int nks, int mtmax, const Epilogue& epi,
                           int* nblk, hipStream_t st) {
  const int nbx = (W.N + 64 * NT - 1) / (64 * NT);
  if (nblk) *nblk = nbx;
  // m-tiles per block from the row count, at most mtmax where the plan sets
  // it (a row's arithmetic does not depend on which rows share its block)
  int mt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  if (mtmax > 0 && mt > mtmax) mt = mtmax >= 4 ? 4 : (mtmax >= 2 ? 2 : 1);
  dim3 grid(nbx, nks, (rows + 16 * mt - 1) / (16 * mt));
  // a W4A16 matrix without the tiled copy (a shape the copy does not cover,
  // through the matvec entry point) takes the one-word-per-k-step loads
  if (WQ && !W.tq) {
    if (mt == 1)
      E2B_TIMED_LAUNCH((k_gemm<WQ, NT, 1, FA, kTagOther, 0>), grid, dim3(256), 0, st, W, rows, A, W.K / nks, epi);
    else if (mt == 2)
      E2B_TIMED_LAUNCH((k_gemm<WQ, NT, 2, FA, kTagOther, 0>), grid, dim3(256), 0, st, W, rows, A, W.K / nks, epi);
    else
      E2B_TIMED_LAUNCH((k_gemm<WQ, NT, 4, FA, kTagOther, 0>), grid, dim3(256), 0, st, W, rows, A, W.K / nks, epi);
    return hipGetLastError();
  }
  if (mt == 1)
    E2B_TIMED_LAUNCH((k_gemm<WQ, NT, 1, FA, TAG, 1>), grid, dim3(256), 0, st, W, rows, A, W.K / nks, epi);
  else if (mt == 2)
    E2B_TIMED_LAUNCH((k_gemm<WQ, NT, 2, FA, TAG, 1>), grid, dim3(256), 0, st, W, rows, A, W.K / nks, epi);
  else
    E2B_TIMED_LAUNCH((k_gemm<WQ, NT, 4, FA, TAG, 1>), grid, dim3(256), 0, st, W, rows, A, W.K / nks, epi);
  return hipGetLastError();
}

template <int WQ, int NT>
static hipError_t gemm_tag(int tag, const Lin& W, int rows, const GemmA& A, int nks, int mtmax,
                           const Epilogue& epi, int* nblk, hipStream_t st) {
  if (A.a) {  // fp32 input rows: the products whose input is a plain copy
    switch (tag) {
      case kTagO: return run_gemm<WQ, NT, 1, kTagO>(W, rows, A, nks, mtmax, epi, nblk, st);
      case kTagPleModel: return run_gemm<WQ, NT, 1, kTagPleModel>(W, rows, A, nks, mtmax, epi, nblk, st);
      default: return run_gemm<WQ, NT, 1, kTagOther>(W, rows, A, nks, mtmax, epi, nblk, st);
    }
  }
  switch (tag) {
    case kTagO: return run_gemm<WQ, NT, 0, kTagO>(W, rows, A, nks, mtmax, epi, nblk, st);
    case kTagQkv: return run_gemm<WQ, NT, 0, kTagQkv>(W, rows, A, nks, mtmax, epi, nblk, st);
    case kTagGateUp: return run_gemm<WQ, NT, 0, kTagGateUp>(W, rows, A, nks, mtmax, epi, nblk, st);
    case kTagDown: return run_gemm<WQ, NT, 0, kTagDown>(W, rows, A, nks, mtmax, epi, nblk, st);
    case kTagPleGate: return run_gemm<WQ, NT, 0, kTagPleGate>(W, rows, A, nks, mtmax, epi, nblk, st);
    case kTagPleProj: return run_gemm<WQ, NT, 0, kTagPleProj>(W, rows, A, nks, mtmax, epi, nblk, st);
    case kTagLmHead: return run_gemm<WQ, NT, 0, kTagLmHead>(W, rows, A, nks, mtmax, epi, nblk, st);
    default: return run_gemm<WQ, NT, 0, kTagOther>(W, rows, A, nks, mtmax, epi, nblk, st);
  }
}

template <int WQ>
hipError_t launch_gemm_q(int tag, const Lin& W, int rows, const GemmA& A, const GemmPlan& plan,
                         const Epilogue& epi, int* nblk, hipStream_t st) {
  const int nks = plan.nks;
  if constexpr (WQ) {
    if (plan.nt == 4) return gemm_tag<1, 4>(tag, W, rows, A, nks, plan.mt, epi, nblk, st);
    if (plan.nt == 2) return gemm_tag<1, 2>(tag, W, rows, A, nks, plan.mt, epi, nblk, st);
    // (one tile per wave: the gate/up product with the GeGLU epilogue only)
    if (plan.nt == 1 && tag == kTagGateUp && !A.a)
      return run_gemm<1, 1, 0, kTagGateUp>(W, rows, A, nks, plan.mt, epi, nblk, st);
  } else {
    if (plan.nt == 2) return gemm_tag<0, 2>(tag, W, rows, A, nks, plan.mt, epi, nblk, st);
    if (plan.nt == 1) return gemm_tag<0, 1>(tag, W, rows, A, nks, plan.mt, epi, nblk, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace e2b
