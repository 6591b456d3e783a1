// Prefill attention on the matrix cores (CDNA4 gfx950, wave64), head dims 256
// and 512.
//
// A prefill pass holds R consecutive positions of one sequence, whose K/V
// are already in the cache ("Gemma 4 E2B in JAX on One TPU v5e", Step 2:
// jitted prefill against a static cache; "Porting Gemma 4 E2B to SGLang-JAX",
// Step 4: shared K/V, queries rotated at their logical positions).  The
// decode kernel would run once per row and re-read the same keys for every
// row; here one block takes the 16 queries of RW = 16 / nq consecutive rows
// (all nq heads of each: GQA, one K/V head) as one 16-row MFMA tile and a
// chunk of keys, so every key tile read serves them all:
//
//   scores S = Q K^T   v_mfma_f32_16x16x32_bf16, the 4 waves each over a
//                      quarter of the head dimension, summed through LDS;
//   online softmax     per query over its causal window (every wave keeps the
//                      same running max and sum);
//   O += P V           each wave for its quarter of the head dimension, V
//                      staged in LDS once per key tile.
//
// Queries and probabilities are carried as bf16 hi/lo pairs (q = hi + lo to
// ~2^-17), so the products keep fp32-class precision; K and V are exact bf16
// (or int8 codes, exact in bf16, with the row scale applied to the score
// column and folded into the probability).  The block writes the (max, sum,
// unnormalised o) partial of its chunk for each (row, head), the layout the
// decode kernel writes, and k_attn_combine merges the chunks.
#include "dev_common.h"

#include <type_traits>

namespace e2b {

namespace {

typedef __bf16 bf16x8_pf __attribute__((ext_vector_type(8)));
typedef float f32x4_pf __attribute__((ext_vector_type(4)));

constexpr int kKT = 32;  // keys per tile

__device__ __forceinline__ bf16x8_pf as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8_pf, v); }

// maximum over each aligned group of 16 lanes (a DPP row), every lane gets it
__device__ __forceinline__ float group_max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return v;
}

// eight int8 codes (two words) as eight bf16 values, exact (|code| <= 127)
__device__ __forceinline__ uint4 codes_to_bf16(uint2 w) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = i < 2 ? w.x : w.y;
    const int c0 = (int8_t)((word >> (16 * (i & 1))) & 0xFFu);
    const int c1 = (int8_t)((word >> (16 * (i & 1) + 8)) & 0xFFu);
    o[i] = f2bf((float)c0) | (f2bf((float)c1) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

template <int HD, int KQ>
__global__ __launch_bounds__(256, 2) void k_attn_prefill(Rows R, AttnArgs a) {
  constexpr int HDW = HD / 4;    // each wave's quarter of the head dimension
  constexpr int KSW = HDW / 32;  // its k-steps of the score product
  constexpr int DTW = HDW / 16;  // its 16-wide output tiles
  constexpr int VP = HD + 8;     // padded V row in LDS (bf16)
  constexpr int VPT = HD / 64;   // 16-byte pieces of the V tile per thread
  constexpr int QB = 16 * HD * 4, VB = kKT * VP * 2;
  // the normed queries (only before the key loop) share room with the V tile
  __shared__ __align__(16) unsigned char smem[QB > VB ? QB : VB];
  __shared__ float sp[4][16][kKT];                      // partial scores per wave, [query][key]
  __shared__ __align__(16) uint16_t pw[4][2][16][kKT + 8];  // P hi / lo per wave, [query][key]
  __shared__ float vsc[kKT];                            // int8: the V row scales of the tile
  float* qs = reinterpret_cast<float*>(smem);           // [16][HD]
  uint16_t* vt = reinterpret_cast<uint16_t*>(smem);     // [kKT][VP]

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, col = lane & 15, grp = lane >> 4;
  const int nq = a.nq, RW = 16 / nq;
  // (grid: query tiles x chunks, a tile's chunks dispatched a row of tiles
  // apart)
  const int r0 = blockIdx.x * RW, c = blockIdx.y;
  const int rlast = min(r0 + RW, R.n) - 1;
  const int seq = row_seq(R, r0);  // every row of a prefill pass is one sequence
  // keys of this chunk: the group's span (the window start of its earliest
  // position to its latest position) split over the grid's chunks, whole
  // tiles each
  int p_first = R.max_ctx, p_last = 0;
  for (int r = r0; r <= rlast; ++r) {
    const int p = clamp_pos(R, row_pos(R, r));
    p_first = min(p_first, p);
    p_last = max(p_last, p);
  }
  const int lo_min = a.window ? max(0, p_first - a.window + 1) : 0;
  const int span = p_last + 1 - lo_min;
  int chunk = (span + a.nchunk - 1) / a.nchunk;
  chunk = max(a.chunk, (chunk + kKT - 1) / kKT * kKT);
  const int k0 = lo_min + c * chunk, k1 = min(k0 + chunk, p_last + 1);

  // ---- the 16 queries: q = row * nq + head; wave w norms and rotates q = w, w+4, ..
  {
    constexpr int DPL = HD / 64;
    const int nraw = nq + (a.owns ? 2 : 0);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int q = wave + 4 * x, rr = q / nq, h = q % nq;
      const int r = min(r0 + rr, R.n - 1);  // (rows past the pass: computed, not used)
      const float* raw = a.qkv + ((size_t)r * nraw + h) * HD;
      const float* cs = a.rope + (size_t)r * a.rope_ld + a.rope_off;
      HeadSide<HD> hs;
      head_side<HD>(a.gq, cs, cs + HD / 2, lane, hs);
      float y[DPL];
      head_raw<HD>(raw, a.qkv_parts, a.qkv_pstride, lane, y);
      head_finish<HD>(y, hs, a.gq != nullptr, true, lane, a.eps);
      const bool live = r0 + rr < R.n;
#pragma unroll
      for (int i = 0; i < DPL; ++i) qs[q * HD + lane * DPL + i] = live ? y[i] : 0.f;
    }
  }
  __syncthreads();
  // this wave's A fragments of the queries (its quarter of d), bf16 hi / lo
  uint4 qh[KSW], ql[KSW];
#pragma unroll
  for (int s = 0; s < KSW; ++s) {
    const float* src = qs + col * HD + HDW * wave + 32 * s + 8 * grp;
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split_pair(src[2 * j], src[2 * j + 1], h[j], l[j]);
    qh[s] = make_uint4(h[0], h[1], h[2], h[3]);
    ql[s] = make_uint4(l[0], l[1], l[2], l[3]);
  }
  __syncthreads();  // the query region becomes the V tile

  // ---- the lane's 4 queries (4 grp + i): their rows' causal windows
  int qlo[4], qhi[4];
  float m[4], lsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * grp + i, r = r0 + q / nq;
    const int p = r < R.n ? clamp_pos(R, row_pos(R, r)) : -1;
    qhi[i] = p;  // (-1: no keys)
    qlo[i] = a.window ? max(0, p - a.window + 1) : 0;
    m[i] = -INFINITY;
    lsum[i] = 0.f;
  }
  f32x4_pf acc[DTW];
#pragma unroll
  for (int d = 0; d < DTW; ++d) acc[d] = f32x4_pf{0.f, 0.f, 0.f, 0.f};
  const float scale = rsqrtf((float)HD);
  const uint16_t* kc16 = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vc16 = static_cast<const uint16_t*>(a.vc);
  const int8_t* kc8 = static_cast<const int8_t*>(a.kc);
  const int8_t* vc8 = static_cast<const int8_t*>(a.vc);

  // One key tile's cache reads, kept raw (int8 codes are widened when used):
  // V: thread t takes key t / 8 and the 16-byte (int8: 8-byte) pieces
  // t % 8 + 8 i; K: this wave's quarter of d for keys 16 half + col.  Keys
  // past the chunk read the zero row.
  using VW = typename std::conditional<KQ != 0, uint2, uint4>::type;
  struct Tile {
    VW v[VPT];
    VW k[2][KSW];
    float vs, ks[2];
  };
  auto load_tile = [&](int kt, Tile& T) {
    {
      const int j = t >> 3, key = kt + j;
      const bool ok = key < k1;
      const size_t row = cache_row(R, seq, ok ? key : lo_min);
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int d = 8 * ((t & 7) + 8 * i);
        if constexpr (KQ) {
          const int8_t* p = ok ? vc8 + row * HD + d : reinterpret_cast<const int8_t*>(kZeroRow);
          T.v[i] = *reinterpret_cast<const uint2*>(p);
        } else {
          const uint16_t* p = ok ? vc16 + row * HD + d : kZeroRow;
          T.v[i] = *reinterpret_cast<const uint4*>(p);
        }
      }
      T.vs = KQ ? *(ok ? a.vs + row : zero_f()) : 0.f;
    }
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
      const int key = kt + 16 * jh + col;
      const bool ok = key < k1;
      const size_t row = cache_row(R, seq, ok ? key : lo_min);
#pragma unroll
      for (int s = 0; s < KSW; ++s) {
        const int d = HDW * wave + 32 * s + 8 * grp;
        if constexpr (KQ) {
          const int8_t* p = ok ? kc8 + row * HD + d : reinterpret_cast<const int8_t*>(kZeroRow);
          T.k[jh][s] = *reinterpret_cast<const uint2*>(p);
        } else {
          const uint16_t* p = ok ? kc16 + row * HD + d : kZeroRow;
          T.k[jh][s] = *reinterpret_cast<const uint4*>(p);
        }
      }
      T.ks[jh] = KQ ? *(ok ? a.ks + row : zero_f()) : 1.f;
    }
  };
  auto widen = [](VW w) -> uint4 {
    if constexpr (KQ) return codes_to_bf16(w);
    else return w;
  };

  // the next tile's reads are issued before this tile's arithmetic
  Tile cur, nxt;
  if (k0 < k1) load_tile(k0, cur);
  for (int kt = k0; kt < k1; kt += kKT) {
    if (kt + kKT < k1) load_tile(kt + kKT, nxt);
    uint4 kb[2][KSW];
    float ksc[2];
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
#pragma unroll
      for (int s = 0; s < KSW; ++s) kb[jh][s] = widen(cur.k[jh][s]);
      ksc[jh] = cur.ks[jh];
    }
    // partial scores over this wave's quarter of d
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
      f32x4_pf sacc = f32x4_pf{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSW; ++s) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(qh[s]), as_bf8(kb[jh][s]), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ql[s]), as_bf8(kb[jh][s]), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[wave][4 * grp + i][16 * jh + col] = sacc[i];
    }
    {
      const int j = t >> 3;
#pragma unroll
      for (int i = 0; i < VPT; ++i) *reinterpret_cast<uint4*>(vt + j * VP + 8 * ((t & 7) + 8 * i)) = widen(cur.v[i]);
      if (KQ && (t & 7) == 0) vsc[j] = cur.vs;
    }
    __syncthreads();

    // scores (the four quarters summed in wave order), online softmax update
    float pv[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 4 * grp + i;
      float sv[2];
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int kk = 16 * jh + col, key = kt + kk;
        float s = ((sp[0][q][kk] + sp[1][q][kk]) + sp[2][q][kk]) + sp[3][q][kk];
        s = s * ksc[jh] * scale;
        const bool ok = key < k1 && key >= qlo[i] && key <= qhi[i];
        sv[jh] = ok ? s : -INFINITY;
      }
      const float mx = group_max16(fmaxf(sv[0], sv[1]));
      const float m_new = fmaxf(m[i], mx);
      float corr = 1.f;
      if (m_new == -INFINITY) {
        pv[i][0] = pv[i][1] = 0.f;
      } else {
        pv[i][0] = sv[0] == -INFINITY ? 0.f : expf(sv[0] - m_new);
        pv[i][1] = sv[1] == -INFINITY ? 0.f : expf(sv[1] - m_new);
        corr = m[i] == -INFINITY ? 0.f : expf(m[i] - m_new);
      }
      lsum[i] = fmaf(lsum[i], corr, group_sum<16>(pv[i][0] + pv[i][1]));
      m[i] = m_new;
#pragma unroll
      for (int d = 0; d < DTW; ++d) acc[d][i] *= corr;
    }
    // P (times the V row scale for int8) as bf16 hi / lo, [query][key]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int kk = 16 * jh + col;
        const float p = KQ ? pv[i][jh] * vsc[kk] : pv[i][jh];
        const uint32_t h = f2bf(p), l = f2bf(p - bf2f(h));
        pw[wave][0][4 * grp + i][kk] = (uint16_t)h;
        pw[wave][1][4 * grp + i][kk] = (uint16_t)l;
      }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // O += P V over this wave's quarter of d
    const uint4 ph = *reinterpret_cast<const uint4*>(&pw[wave][0][col][8 * grp]);
    const uint4 pl = *reinterpret_cast<const uint4*>(&pw[wave][1][col][8 * grp]);
#pragma unroll
    for (int d = 0; d < DTW; ++d) {
      const int dc = HDW * wave + 16 * d + col;
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        b[e] = (uint32_t)vt[(8 * grp + 2 * e) * VP + dc] | ((uint32_t)vt[(8 * grp + 2 * e + 1) * VP + dc] << 16);
      const bf16x8_pf vb = as_bf8(make_uint4(b[0], b[1], b[2], b[3]));
      acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ph), vb, acc[d], 0, 0, 0);
      acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(pl), vb, acc[d], 0, 0, 0);
    }
    __syncthreads();  // the next tile overwrites the V tile and the scores
    cur = nxt;
  }

  // the chunk's partial for each (row, head): unnormalised o, running max, sum
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * grp + i, rr = q / nq, h = q % nq, r = r0 + rr;
    if (r >= R.n) continue;
    float* part = a.part + (((size_t)r * nq + h) * kMaxChunks + c) * (HD + 2);
#pragma unroll
    for (int d = 0; d < DTW; ++d) part[HDW * wave + 16 * d + col] = acc[d][i];
    if (wave == 0 && col == 0) {
      part[HD] = m[i];
      part[HD + 1] = lsum[i];
    }
  }
}

bool attn_prefill_supported(int hd, int nq) {
  return (hd == 256 || hd == 512) && (nq == 1 || nq == 2 || nq == 4 || nq == 8);
}

hipError_t launch_attn_prefill(const Rows& R, const AttnArgs& a, hipStream_t st) {
  if (!attn_prefill_supported(a.hd, a.nq) || R.seq_stride != 0 || R.n < 1 || a.chunk < kKT ||
      a.chunk % kKT || a.nchunk < 1 || a.nchunk > kMaxChunks || !a.part || !a.rope || a.kc_own)
    return hipErrorInvalidValue;
  if (a.kvq && (!a.ks || !a.vs)) return hipErrorInvalidValue;
  const int rw = 16 / a.nq;
  dim3 grid((R.n + rw - 1) / rw, a.nchunk);
  if (a.hd == 256) {
    if (a.kvq) E2B_TIMED_LAUNCH((k_attn_prefill<256, 1>), grid, dim3(256), 0, st, R, a);
    else E2B_TIMED_LAUNCH((k_attn_prefill<256, 0>), grid, dim3(256), 0, st, R, a);
  } else {
    if (a.kvq) E2B_TIMED_LAUNCH((k_attn_prefill<512, 1>), grid, dim3(256), 0, st, R, a);
    else E2B_TIMED_LAUNCH((k_attn_prefill<512, 0>), grid, dim3(256), 0, st, R, a);
  }
  return hipGetLastError();
}

}  // namespace e2b
