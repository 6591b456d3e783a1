// Internal declarations shared by the host side (host.cpp) and the HIP
// kernels (kernels.hip) of libe2b.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e2b {

constexpr int kMaxChunks = 64;   // attention key chunks per (row, layer)
constexpr int kMaxSplitK = 8;    // K slices of one matrix-vector product
constexpr int kMaxGemmSplit = 16;  // K slices of one batched (matrix-core) product
constexpr int kGemvThreads = 256;
constexpr int kLmBlocks = 1024;  // blocks of the lm_head pass (argmax candidates)
constexpr int kStreamBlocks = 1024;  // blocks of the streaming-read calibration
constexpr int kPageShift = 7;        // paged K/V cache: 128 positions per page
constexpr int kPageSize = 1 << kPageShift;

// Matrix kinds; each gets its own kernel symbol so profiles tell them apart.
enum : int {
  kTagOther = 0, kTagQkv, kTagO, kTagGateUp, kTagDown, kTagPleGate, kTagPleProj, kTagPleModel,
  kTagLmHead,
  kTagPleGateRows = 10  // the PLE gate of a batched pass (matvec per row; more input partials)
};

// Device error word bits (first 16 bytes of the workspace).
enum : int { kErrToken = 1, kErrPos = 2, kErrPage = 4 };

// One linear layer resident in the weight arena.  bf16: w [N, K].
// W4A16: q [N, K/8] packed int4 codes, s [N, K/32] bf16 group scales.  Both
// optionally also in matrix-core fragment order (tw, or tq and ts: see
// launch_tile_bf16 / launch_tile_w4), which the batched products read.
struct Lin {
  const uint16_t* w = nullptr;
  const uint16_t* tw = nullptr;
  const uint32_t* q = nullptr;
  const uint16_t* s = nullptr;
  const uint32_t* tq = nullptr;
  const uint16_t* ts = nullptr;
  int N = 0, K = 0;
};

// Which sequence / position / token each processed row is.
// Decode: row b is sequence b at positions[b].  Prefill: every row is the
// same sequence, at positions pos0 + row.
struct Rows {
  const int32_t* tokens = nullptr;
  const int32_t* positions = nullptr;  // null: pos0 + row
  int pos0 = 0, seq0 = 0, seq_stride = 1, n = 0;
  int max_ctx = 0, vocab = 0;
  // paged cache (pages != null): the cache row of (sequence slot s, position
  // p) is pages[s * page_stride + p / kPageSize] * kPageSize + p % kPageSize
  // (the pool holds n_pages + 1 pages, the last a spare); else s * max_ctx + p
  const int32_t* pages = nullptr;
  int page_stride = 0, n_pages = 0;
  int* err = nullptr;  // device error word (a page entry outside the pool)
};

// How a matrix-vector product builds its fp32 input x for one row.
enum PrologueKind : int {
  kPlain = 0,    // x = a[row][k]
  kResNorm = 1,  // h' = (a + rms(sum_s d[s]) * gd) * scalar; x = rms(h') * gx; block 0 stores h'
  kRes = 2,      // same h', x = h'
  kGeglu = 3,    // x = gelu_tanh(a[row][k]) * a[row][I + k]   (I = K)
  kPleGate = 4,  // x = gelu_tanh(a[row][k]) * pli[row][k]
  kAttnMerge = 5, // x = attention output of head k0 / K-slice, merged from the
                  // per-chunk partials a = AttnArgs::part (one-row O product)
  kPrepared = 6   // batched products only: the input rows are already in the
                  // workspace's prepared form (bf16 hi/lo + group sums)
};

// The prologue of each product of the decode step is fixed by its kind
// (tag): the matrix-vector kernel is specialised on it.  -1: read at run time.
// tag_nd: most K-slice partials of the residual delta that prologue sums.
__host__ __device__ constexpr int tag_kind(int tag) {
  return tag == kTagQkv || tag == kTagGateUp || tag == kTagLmHead ? kResNorm
         : tag == kTagPleGate || tag == kTagPleGateRows         ? kRes
         : tag == kTagO                                         ? kAttnMerge
         : tag == kTagPleModel                                  ? kPlain
         : tag == kTagDown                                      ? kGeglu
         : tag == kTagPleProj                                   ? kPleGate
                                                                : -1;
}
__host__ __device__ constexpr int tag_nd(int tag) {
  // (gate/up: the one-row O product writes one partial per query head; the
  // PLE gate of a batched pass: the matrix-core down product's partials.  A
  // specialised prologue reads every slot, so each kind gets only as many as
  // its producer writes)
  return tag == kTagPleGateRows ? kMaxGemmSplit
         : tag == kTagPleGate || tag == kTagGateUp ? kMaxSplitK
         : tag == kTagQkv || tag == kTagLmHead ? 2 : 0;
}

struct Prologue {
  int kind = kPlain;
  const float* a = nullptr;   // kPlain: x [rows, lda]; kRes*: h [rows, K]; kGeglu: [rows, 2K]; kPleGate: [rows, K]
  int lda = 0;                // row stride of a (elements)
  const float* d = nullptr;   // delta partials: nd of them, d_pstride floats apart, each [rows][K]
  int nd = 0;
  size_t d_pstride = 0;
  int na = 1;                 // batched prep only: a is the sum of na partials a_pstride apart
  size_t a_pstride = 0;
  const uint16_t* gd = nullptr;      // gain of rms(delta)
  const uint16_t* scalar = nullptr;  // layer scalar (bf16[1]) or null
  const uint16_t* gx = nullptr;      // gain of rms(h') (kResNorm)
  float* h_out = nullptr;            // [rows, K] (kRes*), written when d != null
  const float* pli = nullptr;        // kPleGate: row stride pli_ld
  int pli_ld = 0;
  int nchunk = 0;                    // kAttnMerge: attention chunks written per head
  int slice = 0;                     // kAttnMerge: head dim (the K slice of one head)
  float eps = 1e-6f;
  int alt = 0;                       // kPrepared: the second prepared buffer (a product's epilogue wrote it)
};

// Output of a matrix-vector product: y [nks][rows][N] fp32 partial sums over
// K slices, or (argmax mode) per-block best (value, index) candidates.
struct Epilogue {
  float* y = nullptr;
  int argmax = 0;
  float* logits = nullptr;      // argmax mode: optional fp32 [rows, N]
  float* cand_val = nullptr;    // [rows][gridDim.x]
  int32_t* cand_idx = nullptr;  // [rows][gridDim.x]
  // batched gate/up product ([W_g; W_u], N = 2 * gi): each block pairs gate
  // and up columns and writes gelu_tanh(gate) * up, the down product's input,
  // in prepared form (bf16 hi/lo [rows][gi], group sums [rows][gi / 32])
  // instead of y
  uint16_t* gh = nullptr;
  uint16_t* gl = nullptr;
  float* gg = nullptr;
  int gi = 0;
};

// Per-row RoPE cos/sin for both layer types, built once per pass by the
// embedding kernel: row r holds [cos_s | sin_s] (hd_s/2 each) then
// [cos_f | sin_f] (hd_f/2 each).
struct RopeTable {
  float* out = nullptr;
  const double* inv_s = nullptr;  // sliding inverse frequencies [hd_s/2]
  const double* inv_f = nullptr;  // full [hd_f/2]
  int hd_s = 0, hd_f = 0;
};

struct AttnArgs {
  const float* qkv = nullptr;   // raw projections [rows][(nq + 2 * (kc_own != null)) * hd]
  const uint16_t* gq = nullptr; // q_norm gain
  const uint16_t* gk = nullptr; // k_norm gain (own K/V)
  const void* kc = nullptr;     // K cache read (the source layer's) [max_batch][max_ctx][hd],
  const void* vc = nullptr;     // bf16, or int8 codes (kvq) with one fp32 scale per row (ks, vs)
  const float* ks = nullptr;    // [max_batch][max_ctx] (int8)
  const float* vs = nullptr;
  void* kc_own = nullptr;       // decode: cache to write this position's K/V into (layer owns
  void* vc_own = nullptr;       // K/V); null when the layer shares or the K/V are already written
  float* ks_own = nullptr;      // (int8: the row scales)
  float* vs_own = nullptr;
  int kvq = 0;                  // cache format: 0 bf16, 1 int8
  float* part = nullptr;        // [rows][nq][kMaxChunks][hd + 2]
  float* out = nullptr;         // [rows][nq * hd]
  uint16_t* xh = nullptr;       // non-null: the merge writes its output as the O product's
  uint16_t* xl = nullptr;       // prepared input instead (bf16 hi/lo [rows][nq * hd],
  float* xg = nullptr;          // sums of hi + lo per 32-group [rows][nq * hd / 32])
  const float* rope = nullptr;  // RoPE table rows (rope_ld floats each), this type at rope_off
  int rope_ld = 0, rope_off = 0;
  int nq = 0, hd = 0, window = 0 /* 0: full */;
  int chunk = 0;   // fewest keys per block; a row's live span is split over
  int nchunk = 0;  // nchunk blocks of max(chunk, ceil(span / nchunk)) keys
  int owns = 0;                 // the layer computes K/V (raw rows hold q, k, v)
  int combine = 1;              // merge the chunk partials into out (else the O product does)
  int mfma = 0;                 // the matrix-core kernel (launch_attn_prefill): a prefill pass
                                // whose K/V are all written, chunk plan for it
  int qkv_parts = 1;            // qkv is the sum of this many partials
  size_t qkv_pstride = 0;       // floats between partials
  float eps = 1e-6f;
};

struct QkvPostArgs {
  const float* qkv = nullptr;   // [rows][(nq + 2*owns) * hd] raw projections
  const uint16_t* gq = nullptr;
  const uint16_t* gk = nullptr;
  const float* rope = nullptr;  // RoPE table (see AttnArgs)
  int rope_ld = 0, rope_off = 0;
  void* kc = nullptr;           // this layer's cache when it owns K/V, else null (bf16 or int8)
  void* vc = nullptr;
  float* ks = nullptr;          // int8: the row scales
  float* vs = nullptr;
  int kvq = 0;                  // cache format: 0 bf16, 1 int8
  int nq = 0, hd = 0;
  int qkv_parts = 1;
  size_t qkv_pstride = 0;
  float eps = 1e-6f;
};

// ---- launchers (kernels.hip) ----------------------------------------------
// E [V, H] and Eple [V, L*P]: both bf16 (w) or both int4 (q + s)
hipError_t launch_embed(const Rows& R, const Lin& E, const Lin& Eple, float sqrtH, float sqrtP,
                        float* h, float* tokple, int* err, const RopeTable& rt, hipStream_t st);
// u: u_parts partials u_pstride floats apart, each [rows][L*P]
hipError_t launch_ple_finish(const Rows& R, const float* u, int u_parts, size_t u_pstride,
                             const float* tokple, const uint16_t* g, int L, int P,
                             float inv_sqrtH, float eps, float* pli, hipStream_t st);
// blocks_hint > 0 fixes the number of blocks along N (else chosen from N);
// *blocks_out (nullable) receives it -- the argmax candidate count per row.
hipError_t launch_gemv(int quant, int tag, const Lin& W, int rows, const Prologue& pro,
                       const Epilogue& epi, int blocks_hint, int* blocks_out, hipStream_t st);
int gemv_splits(int K);
bool gemv_supported(int K);  // K is one of the widths the matvec kernel handles
// W4A16 words and scales in the order the matrix-core product consumes
// them (N % 16 == 0): for column tile t (columns 16t .. 16t+15) and 32-group
// g, the 64 words tq[(t * K/32 + g) * 64 + l] = q[16t + l % 16][4g + l / 16]
// (the B fragment of one MFMA step, lane l) and the 16 scales
// ts[(t * K/32 + g) * 16 + c] = s[16t + c][g].  A wave's weight reads are
// then 256 contiguous bytes per step instead of 16 pieces of 16 bytes.
hipError_t launch_tile_w4(const Lin& W, uint32_t* tq, uint16_t* ts, hipStream_t st);
// The same for bf16 weights (N % 16 == 0): for column tile t and 32-step g,
// the 64 lanes' 16-byte B fragments tw[((t * K/32 + g) * 64 + l) * 8 + e] =
// w[16t + l % 16][32g + 8 (l / 16) + e], one contiguous kilobyte per step.
hipError_t launch_tile_bf16(const Lin& W, uint16_t* tw, hipStream_t st);
hipError_t launch_qkv_post(const Rows& R, const QkvPostArgs& a, hipStream_t st);
hipError_t launch_attention(const Rows& R, const AttnArgs& a, hipStream_t st);
// Prefill attention on the matrix cores: rows of one sequence (seq_stride 0),
// head dims 256 / 512, nq in {1, 2, 4, 8}, K/V already in the cache; chunk a
// multiple of 32.  Writes the chunk partials; the merge is launch_attention's.
bool attn_prefill_supported(int hd, int nq);
hipError_t launch_attn_prefill(const Rows& R, const AttnArgs& a, hipStream_t st);
constexpr int kPrefillMinChunk = 128;
hipError_t launch_advance(int32_t* pos, int n, hipStream_t st);
hipError_t launch_stream_reduce(const void* buf, size_t bytes, float* out, hipStream_t st);
// batched rows (>= 2): prologue into bf16 hi/lo rows + group sums, then MFMA
hipError_t launch_xprep(const Prologue& p, int rows, int K, uint16_t* xh, uint16_t* xl, float* xg,
                        hipStream_t st);
struct GemmPlan {
  int nt = 1;   // 16-column tiles per wave (block covers 64 * nt columns)
  int nks = 1;  // K slices (partials written [nks][rows][N])
  int mt = 0;   // 16-row tiles per block at most (0: from the row count alone)
};
GemmPlan gemm_plan(int quant, int N, int K, bool partial_ok);
// The gate/up product with the GeGLU in its epilogue (I gate and I up rows)
// for a pass of `rows` rows: no K slices; nt = 0 where I does not split into
// whole blocks.
GemmPlan gemm_plan_geglu(int quant, int I, int K, int rows);
// Input rows of a batched product: either prepared by k_xprep (bf16 hi/lo
// [rows][K] + fp32 group sums [rows][K/32]) or, for a plain input (kPlain,
// one partial), fp32 rows [rows][lda] read and split by the product itself.
struct GemmA {
  const uint16_t* xh = nullptr;
  const uint16_t* xl = nullptr;
  const float* xg = nullptr;
  const float* a = nullptr;  // non-null: fp32 rows
  int kind = kPlain, lda = 0, na = 1;
};
// *nblk receives the number of column blocks (argmax candidates per row)
hipError_t launch_gemm(int quant, int tag, const Lin& W, int rows, const GemmA& A,
                       const GemmPlan& plan, const Epilogue& epi, int* nblk, hipStream_t st);
// (launch_gemm, by weight format: gemm_bf16.hip, gemm_w4.hip)
hipError_t launch_gemm_bf16(int tag, const Lin& W, int rows, const GemmA& A, const GemmPlan& plan,
                            const Epilogue& epi, int* nblk, hipStream_t st);
hipError_t launch_gemm_w4(int tag, const Lin& W, int rows, const GemmA& A, const GemmPlan& plan,
                          const Epilogue& epi, int* nblk, hipStream_t st);
// The next launch_gemv / launch_gemm on this host thread records these
// events at its kernel's start and end.
void set_launch_events(hipEvent_t start, hipEvent_t stop);
// (launchers) the pending events, cleared; false if none are set
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop);
hipError_t launch_sum_partials(int nparts, size_t n, const float* parts, float* out,
                               hipStream_t st);
hipError_t launch_argmax_final(int rows, int nblk, const float* cand_val,
                               const int32_t* cand_idx, int32_t* out, int32_t* adv,
                               hipStream_t st);

}  // namespace e2b
