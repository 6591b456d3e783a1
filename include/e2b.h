/*
 * e2b.h -- C ABI of libe2b: one decode step (and the prefill that fills its
 * cache) of a Gemma-4-E2B-shaped decoder on one MI355X (gfx950).
 *
 * What the step computes is defined on the pages
 *   [P1] "Gemma 4 E2B in JAX on One TPU v5e: bf16 or 4-Bit, Python or Rust"
 *   [P2] "Six Serving Engines on One Cloud TPU v5e Chip"
 *   [P3] "Porting Gemma 4 E2B to SGLang-JAX on One Cloud TPU v5e"
 *   [P4] "Gemma 4 E2B in Pure JAX on a Colab TPU: Google's 4-Bit Export
 *        Against an Exact Repack"
 *   [P5] "One TPU chip, eight agents: serving small agent workloads with raw JAX"
 * and cited per call below.
 *
 * Conventions for every call:
 *  - Device pointers ("d_" prefix) are owned by the caller (the Python binding
 *    allocates them with PyTorch); the library never allocates or frees
 *    device memory.  Host pointers are only read during the call.
 *  - `stream` is a hipStream_t passed as void*; work is enqueued on it and the
 *    call returns without synchronising unless stated.
 *  - Return value: E2B_OK or an error code; on error nothing was enqueued and
 *    e2b_last_error() (thread-local) holds a message.  There is no fallback
 *    path of any kind.
 *  - bf16 data is raw IEEE bfloat16 bit patterns (uint16).
 */
#ifndef E2B_H
#define E2B_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  E2B_OK = 0,
  E2B_EINVAL = 1,  /* bad argument, shape or configuration */
  E2B_ERANGE = 2,  /* batch / position / sequence outside the bound state */
  E2B_ENOMEM = 3,  /* caller-provided buffer too small */
  E2B_EHIP = 4,    /* a HIP runtime call failed (message carries its string) */
  E2B_EDEVICE = 5, /* a kernel flagged an out-of-range token or position */
  E2B_ESTATE = 6   /* call order violated (e.g. decode before load) */
};

enum { E2B_QUANT_BF16 = 0, E2B_QUANT_W4A16 = 1 };
enum { E2B_KV_BF16 = 0, E2B_KV_INT8 = 1 };
enum { E2B_DTYPE_BF16 = 0, E2B_DTYPE_INT32 = 1 };

/* Model configuration.  Field names follow the checkpoint config fields
 * listed in [P3] Step 1 (num_hidden_layers, num_kv_shared_layers,
 * hidden_size_per_layer_input, num_key_value_heads, head_dim /
 * global_head_dim, layer_types "4 sliding, 1 full, repeating") and Step 5
 * (use_double_wide_mlp).  Layer l is a full-attention layer iff
 * l % layer_pattern_period == layer_pattern_period - 1.  quant selects how
 * every linear layer is stored: bf16 [N, K], or W4A16 = int4 codes eight per
 * int32 with one bf16 scale per group_size (32) consecutive K ([P5] The
 * engine; [P4] intro table).  embed_quant selects the same for the two
 * vocabulary tables: bf16, or W4A16 (the int4 vocabulary tables and int4
 * lm_head of [P2] "Six Serving Engines on One Cloud TPU v5e Chip", What
 * Changes and What Stays and Step 3), decoded exactly for the gathers and
 * streamed as int4 by the tied lm_head.  kv_quant selects the K/V cache
 * format: bf16, or int8 ([P5] Measured: int8 KV with donation; KV memory
 * math: one byte per element) with one fp32 scale per cached row (a token's
 * K or V of one layer): s = max |x| / 127, code = nearest-even(x / s), read
 * back as code * s. */
typedef struct {
  int32_t num_hidden_layers;
  int32_t num_kv_shared_layers;
  int32_t hidden_size;
  int32_t num_attention_heads;
  int32_t num_key_value_heads;  /* must be 1 */
  int32_t head_dim;             /* sliding layers */
  int32_t global_head_dim;      /* full layers */
  int32_t sliding_window;       /* keys p-W+1 .. p */
  int32_t layer_pattern_period; /* 5: four sliding then one full */
  int32_t intermediate_size;    /* layers below the first shared layer */
  int32_t use_double_wide_mlp;  /* 2x width from the first shared layer on */
  int32_t hidden_size_per_layer_input;
  int32_t vocab_size;
  int32_t quant;       /* E2B_QUANT_*: every linear layer */
  int32_t embed_quant; /* E2B_QUANT_*: the two vocabulary tables (the tied token
                          embedding / lm_head and the per-layer table) */
  int32_t kv_quant;    /* E2B_KV_*: the K/V cache */
  int32_t group_size;  /* 32 */
  float rms_eps;
  float rope_theta_sliding;
  float rope_theta_full;
} e2b_config;

/* One host tensor handed to e2b_load_weights.  Names are the canonical
 * parameter names of [P3] Step 5 and [P5] "#3225" ("model.embed_tokens.weight",
 * "model.embed_tokens_per_layer.weight", "model.per_layer_model_projection.weight",
 * "model.per_layer_projection_norm.weight", "model.norm.weight",
 * "model.layers.{l}.{input_layernorm, post_attention_layernorm,
 *  pre_feedforward_layernorm, post_feedforward_layernorm,
 *  post_per_layer_input_norm}.weight", "...self_attn.{q,k,v,o}_proj.weight",
 * "...self_attn.{q,k}_norm.weight", "...mlp.{gate,up,down}_proj.weight",
 * "...per_layer_input_gate.weight", "...per_layer_projection.weight",
 * "...layer_scalar").  Under W4A16 a linear "X.weight" (and, with
 * embed_quant W4A16, each vocabulary table) is given as
 * "X.weight_packed" (int32 [N, K/8]; word j holds K-elements 8j..8j+7, element
 * 8j+i in bits [4i, 4i+4) as the code q+8, q in -8..7) and "X.weight_scale"
 * (bf16 [N, K/32]).  Row-major, C-contiguous. */
typedef struct {
  const char* name;
  int32_t dtype; /* E2B_DTYPE_* */
  int32_t ndim;  /* 1 or 2 */
  int64_t shape[2];
  const void* data; /* host pointer */
} e2b_tensor;

typedef struct e2b_model e2b_model;

/* Fill *out with a preset: "toy" (5 layers, hidden 256), "toy10" (10 layers,
 * 2 full, last 5 shared) or "e2b" (35 layers, hidden 1536, 8 query heads,
 * head dims 256/512, window 512, MLP 6144/12288, per-layer input 256, vocab
 * 262144).  quant and embed_quant are set to bf16; change them before
 * e2b_create.
 * E2B_EINVAL for an unknown name. */
int e2b_config_preset(const char* name, e2b_config* out);

/* Validate the config and build the host descriptor (layer table, K/V share
 * map).  E2B_EINVAL if num_key_value_heads != 1, a head dim is not one of
 * 64/128/256/512, hidden_size or a width is not a multiple of group_size, or
 * a count is out of range.  The caller frees with e2b_destroy. */
int e2b_create(const e2b_config* cfg, e2b_model** out);
void e2b_destroy(e2b_model* model);

/* out[l] = layer whose K/V layer l reads ([P5] The engine, kv_share_map:
 * itself below first_shared = L - num_kv_shared_layers, else the last
 * non-shared layer of its own type; a shared layer with no such layer keeps
 * its own K/V).  out has num_hidden_layers entries. */
int e2b_kv_share_map(const e2b_model* model, int32_t* out);

/* Parameter bytes of the model as stored on the device by this library (the
 * checkpoint view, K-side tensors only on layers that own K/V), i.e. what
 * [P1] Steps 3-4 report as "weights 9.257 GB" (bf16) / "6.559 GB" (W4A16). */
size_t e2b_weight_bytes(const e2b_model* model);

/* Device bytes e2b_load_weights needs in its arena: the parameters plus
 * alignment padding, small derived tables (RoPE frequencies) and a second
 * copy of every matrix the batched (matrix-core) products read, in their
 * fragment order (bf16 weights or W4A16 words and scales; for bf16 also the
 * tied embedding), built on the device at load time. */
size_t e2b_arena_bytes(const e2b_model* model);

/* K/V cache bytes for max_batch sequences of max_ctx positions: K and V of
 * every layer that owns K/V, one KV head; bf16: 18,432 B per token per
 * sequence at E2B ([P5] Feasibility part 1: 9,216 elements per token); int8:
 * 9,216 B of codes plus 2 x 15 fp32 row scales (each scale array padded to
 * 256 bytes). */
size_t e2b_kv_bytes(const e2b_model* model, int max_batch, int max_ctx);

/* Workspace bytes for calls that process up to max_rows rows (decode batch,
 * or prefill rows per pass).  The workspace (256-byte aligned) is scratch
 * except its first 256 bytes, the device error word: zero them once before
 * the first call; e2b_check reads and re-zeroes it.  Calls that overlap in
 * time must not share a workspace. */
size_t e2b_workspace_bytes(const e2b_model* model, int max_rows);

/* Copy the tensors to the caller's device arena (d_arena, arena_bytes >=
 * e2b_arena_bytes) on `stream`, then synchronise it.  Every tensor the model
 * reads must be present exactly once with the expected dtype and shape;
 * missing, duplicate or mis-shaped tensors give E2B_EINVAL naming the tensor.
 * K-side tensors of layers that read shared K/V are ignored ([P5] "#3225":
 * such layers hold no K-side parameters).  The arena must stay alive and
 * unmodified while the model is used. */
int e2b_load_weights(e2b_model* model, const e2b_tensor* tensors, int n, void* d_arena,
                     size_t arena_bytes, void* stream);

/* Bind caller-owned device memory as the K/V cache: bytes >=
 * e2b_kv_bytes(model, max_batch, max_ctx), else E2B_ENOMEM.  Layout per
 * owning layer: K [max_batch][max_ctx][hd] then V, bf16 or int8; for int8
 * then the K and V row scales, fp32 [max_batch][max_ctx] each.  Slot = position
 * ([P5] The engine: RoPE follows the logical position).  Contents need no
 * initialisation: a position is always written before it is read. */
int e2b_kv_alloc(e2b_model* model, void* d_kv, size_t bytes, int max_batch, int max_ctx);

/* ---- paged K/V cache ------------------------------------------------------
 * The cache as a pool of pages of E2B_PAGE (128) positions ([P3] Step 7 and
 * [P2] Step 3: page size 128, with which a server keeps 64 requests running
 * where page size 1 held 8), so that sequences of uneven length share one
 * pool and a finished sequence's pages go straight to a new one: the
 * continuous batching that [P5] Feasibility part 2 contrasts with lockstep
 * batches.  Every K/V-owning layer has its own pool of n_pages * 128 rows
 * (layout as e2b_kv_alloc with max_batch * max_ctx replaced by (n_pages +
 * 1) * 128: the pool, then the spare page); one page id covers the same 128
 * positions in every layer.  The
 * decode step's row b and a prefill's `seq` name a sequence slot whose row of
 * the page table maps position p to page table[slot][p / 128], row p % 128.
 * The library's allocator (e2b_seq_reserve / release / move) owns the table;
 * a cached position outside the slot's reserved pages is never read or
 * written through a stale entry: the kernels flag it on the device error
 * word (e2b_check) and use a spare page past the pool that no sequence owns. */
enum { E2B_PAGE = 128 };
size_t e2b_kv_paged_bytes(const e2b_model* model, int n_pages);
/* Bind d_kv (>= e2b_kv_paged_bytes) as a pool of n_pages pages and
 * d_page_table (caller-owned device int32 [max_batch][ceil(max_ctx / 128)])
 * as its page table, all entries free.  Synchronises `stream`. */
int e2b_kv_alloc_paged(e2b_model* model, void* d_kv, size_t bytes, int n_pages, int32_t* d_page_table,
                       int max_batch, int max_ctx, void* stream);
/* Give slot `slot` pages for positions [0, n_positions) (it keeps the ones it
 * has; E2B_ENOMEM, nothing changed, if the pool is short).  Synchronises. */
int e2b_seq_reserve(e2b_model* model, int slot, int n_positions, void* stream);
/* Return slot `slot`'s pages to the pool.  Synchronises. */
int e2b_seq_release(e2b_model* model, int slot, void* stream);
/* Move a sequence from slot `from` to the empty slot `to` (its page-table row;
 * no K/V is copied), e.g. to keep a batch's live sequences in rows 0..B-1.
 * E2B_ESTATE if `to` holds pages.  Synchronises. */
int e2b_seq_move(e2b_model* model, int from, int to, void* stream);
/* Pages left in the pool (0 for a contiguous cache). */
int e2b_pages_free(const e2b_model* model);

/* One greedy decode step for `batch` sequences b = 0..batch-1 (sequence b
 * uses cache slot row b): token d_tokens[b] at position d_positions[b]
 * (int32 device arrays).  The step is the decoder pass the pages define:
 * embedding and per-layer inputs, then per layer the attention block over the
 * cache of the layer's K/V source, the GeGLU MLP (double width from the first
 * shared layer on) and the per-layer-input mix, then the final norm, the tied
 * lm_head and the greedy choice ([P3] Steps 1 and 3-5; [P5] The engine:
 * kv_share_map, RoPE at the logical position, the cache updated in place).
 * Writes K/V of position d_positions[b] in place, attends over positions <= it
 * (window on sliding layers), and writes the greedy next token to d_argmax[b]
 * (lowest index on ties) and, if d_logits is not NULL, fp32 logits [batch,
 * vocab].  d_argmax may alias d_tokens.  Allocates nothing and does not
 * synchronise.  E2B_ERANGE if batch exceeds the bound max_batch or the
 * workspace rows; E2B_ENOMEM if ws_bytes < e2b_workspace_bytes(model, batch).
 * Tokens >= vocab or positions outside [0, max_ctx) are not read or written;
 * they set the device error word reported by e2b_check. */
int e2b_decode_step(e2b_model* model, const int32_t* d_tokens, const int32_t* d_positions,
                    int batch, float* d_logits, int32_t* d_argmax, void* d_ws, size_t ws_bytes,
                    void* stream);

/* Prefill of one sequence: tokens d_tokens[0..n_tokens) at positions
 * pos0..pos0+n_tokens-1 of cache row `seq`, in order; equivalent to n_tokens
 * decode steps of that sequence ([P1] Step 2: jitted prefill plus one decode
 * step per token against a static cache).  All K/V of a layer are written
 * before its attention reads them.  Writes the logits (nullable) and greedy
 * token of the last position.  E2B_ERANGE if seq >= max_batch or pos0 +
 * n_tokens > max_ctx.  The workspace must hold e2b_workspace_bytes(model, r)
 * for some r >= 1; longer prompts are processed r rows per pass. */
int e2b_prefill(e2b_model* model, int seq, const int32_t* d_tokens, int n_tokens, int pos0,
                float* d_logits_last, int32_t* d_argmax_last, void* d_ws, size_t ws_bytes,
                void* stream);

/* Device address of the K (which 0) or V (which 1) cache region that layer
 * `layer` reads, [max_batch][max_ctx][hd] bf16 or int8 ([(n_pages + 1) * 128]
 * [hd] for a paged cache), or (int8 cache) its K (2) or V (3) row scales,
 * fp32 [max_batch][max_ctx] ([(n_pages + 1) * 128]): the layer's own region if it
 * owns K/V, else its source layer's region (the same address, so shared
 * layers see bit-identical K/V; [P3] Step 1, [P5] The engine).  Requires
 * e2b_kv_alloc.  E2B_EINVAL for a bad layer or which. */
int e2b_kv_view(const e2b_model* model, int layer, int which, void** out);

/* Weight-streaming matrix-vector product, the kernel every linear layer of
 * the step uses: y[r][n] = sum_k W[n][k] x[r][k] for r < rows, n < N, fp32
 * accumulation.  quant E2B_QUANT_BF16: d_w is bf16 [N, K], d_scale NULL.
 * E2B_QUANT_W4A16: d_w is the packed int32 [N, K/8] (format of e2b_tensor)
 * and d_scale the bf16 [N, K/32] group scales; each code is decoded exactly
 * as (c - 8) * scale in fp32 ([P4] cell 3.1).  x: fp32 [rows, K]; y: fp32
 * [rows, N].  K must be one of the widths the library supports: K split into
 * at most 8 equal slices of width 32, 128, 256, 512, 1536 or 2048 (the first
 * that divides K among 2048, 1536; else K itself when K <= 512; else 512);
 * other K -> E2B_EINVAL.  d_ws (256-byte aligned) must hold
 * e2b_matvec_workspace_bytes(quant, N, K, rows) bytes: the K-slice partial
 * sums (none when the product is not split) and, for two or more rows with
 * N % 16 == 0, a copy of the weights tiled in the matrix-core fragment order
 * that batched decode reads (built by the call).  One row streams the
 * weights through the matvec kernel; two or more rows (x 16-byte aligned)
 * share one pass over the weights on the matrix cores.  Asynchronous. */
size_t e2b_matvec_workspace_bytes(int quant, int N, int K, int rows);
int e2b_matvec(int quant, const void* d_w, const uint16_t* d_scale, int N, int K,
               const float* d_x, int rows, float* d_y, void* d_ws, size_t ws_bytes,
               void* stream);

/* e2b_matvec for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, arithmetic and results as
 * e2b_matvec, without d_ws: the K-slice partial sums go to a scratch array
 * of e2b_matvec_noalloc_max_bytes() bytes (16 MiB) that the library holds on
 * each device it runs on until the process ends; several rows read the
 * row-major weights directly (no tiled copy is built).  E2B_ENOMEM if the
 * product's partials (slices x rows x N x 4 bytes, the plan e2b_matvec uses)
 * exceed the scratch.  Calls no allocating routine.  Every call on a device
 * shares that device's scratch, so calls that overlap in time on one device
 * (on different streams or threads) race and must be serialised by the
 * caller; nothing in the scratch needs to start at zero (each call writes
 * every partial it reads).  Asynchronous. */
size_t e2b_matvec_noalloc_max_bytes(void);
int e2b_matvec_noalloc(int quant, const void* d_w, const uint16_t* d_scale, int N, int K,
                       const float* d_x, int rows, float* d_y, void* stream);

/* The embedding gathers of the step for n tokens, on their own: d_h[r][i] =
 * E[t_r][i] * sqrt(H) (the tied table, [P4] cell 2.2) and d_tokple[r][j] =
 * E_ple[t_r][j] * sqrt(P) for j < L * P (the per-layer table, [P3] Step 3),
 * fp32 row-major, each a widened bf16 table value times the fp32-rounded
 * constant (one rounding), exactly what the decode step consumes.  The
 * workspace must hold e2b_workspace_bytes(model, n).  Tokens outside the
 * vocabulary read row 0 and set the device error word.  Asynchronous. */
int e2b_embed(e2b_model* model, const int32_t* d_tokens, int n, float* d_h, float* d_tokple,
              void* d_ws, size_t ws_bytes, void* stream);

/* ---- HIP graph of one decode step -------------------------------------
 * Capture exactly what e2b_decode_step enqueues for these arguments into a
 * HIP graph, followed (if advance_positions) by d_positions[b] += 1 for every
 * b.  With d_argmax == d_tokens, replaying the graph runs a greedy decode
 * loop entirely on the device with one launch per step ([P1] Step 2: one
 * decode step per token against a static cache, the cache written in
 * place -- [P5] Measured: donated buffers).  `stream` must not be the null
 * stream.  All pointers are baked into the graph and must stay valid.  The
 * model must not be profiling.  Free with e2b_graph_destroy. */
typedef struct e2b_graph e2b_graph;
int e2b_graph_capture(e2b_model* model, const int32_t* d_tokens, int32_t* d_positions, int batch,
                      float* d_logits, int32_t* d_argmax, void* d_ws, size_t ws_bytes,
                      int advance_positions, void* stream, e2b_graph** out);
int e2b_graph_replay(e2b_graph* graph, void* stream);
void e2b_graph_destroy(e2b_graph* graph);

/* ---- per-kernel timing ----------------------------------------------------
 * While profiling a kind, every eager launch of that kind's product kernel
 * records HIP events at its own start and end (the dispatch's timestamps,
 * hipExtLaunchKernel; a batched product's input-prep kernel is not included);
 * e2b_profile_read synchronises them and returns the launch count, summed
 * duration (ms) and summed algorithmic bytes (weights streamed once plus input
 * and output vectors), then stops profiling.  kind 0 stops without reading. */
enum {
  E2B_KIND_NONE = 0, E2B_KIND_QKV = 1, E2B_KIND_O = 2, E2B_KIND_GATE_UP = 3, E2B_KIND_DOWN = 4,
  E2B_KIND_PLE_GATE = 5, E2B_KIND_PLE_PROJ = 6, E2B_KIND_PLE_MODEL = 7, E2B_KIND_LM_HEAD = 8,
  E2B_KIND_ATTN = 9 /* the decode attention kernel (bytes reported as 0: the K/V
                       span it reads depends on device-side positions) */
};
int e2b_profile_begin(e2b_model* model, int kind);
int e2b_profile_read(e2b_model* model, int* launches, double* total_ms, double* total_bytes);

/* ---- bandwidth calibration -------------------------------------------------
 * A plain streaming reduction over `bytes` of device memory (every byte read
 * once, 16 bytes per lane per load): d_out (fp32, e2b_stream_reduce_blocks()
 * entries) receives one partial sum per block of the buffer's 32-bit words
 * read as fp32.  Timed by the caller, its rate is the read bandwidth a plain
 * stream sustains on this device, the denominator of a calibrated roofline
 * ([P5] Measured: the calibrated streaming reduction the decode step's KV
 * read is compared with).  bytes and d_buf must be multiples of 16.
 * Asynchronous. */
int e2b_stream_reduce(const void* d_buf, size_t bytes, float* d_out, void* stream);
int e2b_stream_reduce_blocks(void);

/* Synchronise `stream`, then read and clear the device error word in d_ws.
 * E2B_EDEVICE (message names the first bad token or position) if a kernel
 * flagged one since the last check, else E2B_OK. */
int e2b_check(e2b_model* model, void* d_ws, void* stream);

/* Thread-local message of the last failing call on this thread. */
const char* e2b_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* E2B_H */
