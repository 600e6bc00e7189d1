/*
 * mi_prefill.h - C ABI of the gfx950 (MI355X) Q8_0 prefill library.
 *
 * One call runs the prefill forward of a Qwen2/Qwen3-style decoder over all prompt
 * tokens together, writes every token's K/V row into persistent per-layer KV regions
 * at the row its position names, and returns the logits of the last token only.
 * Sources for what each call computes (the "minfer Inference E2E Walkthrough"
 * pages):
 *   - "09 - Prefill: the first forward": the prefill call, positions as data
 *     (section 2.2), last-token logits (2.4), KV regions sized by n_ctx (2.5),
 *     one owned copy of the logits (2.6), the position check (3.4);
 *   - "05 - Graph build - the IR and the builder": the layer node by node (2.5),
 *     GQA (2.5), the tail rows (2.8), inline matmul bias and the KV store (3.2);
 *   - the walkthrough index, stages 10 and 11: Q8_0 activations quantized on the
 *     fly against quantized weights; RMSNorm, RoPE, softmax, SiLU, GQA attention.
 *
 * Conventions for every entry point
 *   - All functions return an mi_status (0 = MI_OK).  On error nothing has been
 *     enqueued or written, except for MI_ERR_HIP (a runtime failure after launch);
 *     mi_last_error() then describes the failure (thread-local, valid until the
 *     next call on the same thread).
 *   - Pointers marked "device" are HIP device memory owned by the caller; the
 *     library never allocates, frees or retains them.  "host" pointers are read
 *     before the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is asynchronous on that stream; the caller synchronizes before reading.
 *   - Matrices are row-major.  A Q8_0 matrix [rows][cols] is stored as two
 *     planes: int8 codes [rows][cols] and fp16 scales [rows][cols/32] (bits in a
 *     uint16).  Value (r, c) = scale[r][c/32] * code[r][c].  cols % 32 == 0.
 *     Weights use rows = output features, cols = input features ([out][in]).
 *   - Activations are token-major f32: [n_tokens][features].
 *   - Numerics: every node computes to f64 accuracy from its f32 inputs and
 *     rounds its result once to f32 (round to nearest even); the Q8_0 quantizer
 *     runs in f32 exactly as specified below.
 */
#ifndef MI_PREFILL_H
#define MI_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MI_OK = 0,
  MI_ERR_INVALID_ARG = 1,     /* null pointer, bad size, dims not multiples of 32, ... */
  MI_ERR_POSITION_RANGE = 2,  /* a position < 0 or >= n_ctx ("09", section 3.4)       */
  MI_ERR_DUP_POSITION = 3,    /* two tokens of one call name the same KV row           */
  MI_ERR_KV_MISMATCH = 4,     /* KV descriptor disagrees with the model or the call   */
  MI_ERR_WORKSPACE = 5,       /* workspace too small                                   */
  MI_ERR_HIP = 6,             /* HIP runtime error                                     */
  MI_ERR_UNSUPPORTED = 7      /* shape outside what the kernels implement              */
} mi_status;

/* Model shape.  n_head % n_head_kv == 0; head_dim 64 or 128; hidden, ffn, n_head*head_dim
 * multiples of 32; hidden at most 4096, n_head*head_dim and ffn at most 49152 (MI_ERR_UNSUPPORTED
 * otherwise).
 * rms_eps is used for every RMSNorm (and the Qwen3 per-head QK norm); rope_theta is the NeoX
 * RoPE base. */
typedef struct {
  int32_t n_layers, hidden, n_head, n_head_kv, head_dim, ffn, vocab;
  float rms_eps, rope_theta;
  int32_t qkv_bias;  /* 1: Q/K/V matmuls add a bias (Qwen2)            */
  int32_t qk_norm;   /* 1: per-head RMSNorm of Q and K before RoPE (Qwen3) */
  int32_t tied;      /* 1: lm_head reuses token_embd                      */
} mi_hparams;

/* A Q8_0 matrix in device memory (layout above). */
typedef struct {
  const int8_t* codes;     /* device [rows][cols]      */
  const uint16_t* scales;  /* device [rows][cols / 32] */
  int32_t rows, cols;
} mi_q8_matrix;

/* One decoder layer, in the library's weight layout (the binding builds it once at load):
 *   wqkv      rows of Wq, then Wk, then Wv stacked: [nh*hd + 2*nkv*hd][hidden].  One matmul
 *             computes Q, K and V; each output element is the same dot product as in three
 *             separate matmuls.
 *   bqkv      device f32 [nh*hd + 2*nkv*hd] (bq, bk, bv stacked), NULL unless hp.qkv_bias.
 *   wo        [hidden][nh*hd].
 *   w_gate_up gate and up rows interleaved in groups of 32: rows 64p..64p+31 are gate rows
 *             32p..32p+31, rows 64p+32..64p+63 are up rows 32p..32p+31; [2*ffn][hidden], so
 *             one tile of the matmul holds matching gate and up columns and SwiGLU plus the
 *             Q8_0 of its result run in the matmul epilogue.
 *   w_down    [hidden][ffn].
 *   attn_norm, ffn_norm device f32 [hidden]; q_norm, k_norm device f32 [head_dim] (NULL unless
 *   hp.qk_norm). */
typedef struct {
  mi_q8_matrix wqkv, wo, w_gate_up, w_down;
  const float* bqkv;
  const float *attn_norm, *ffn_norm;
  const float *q_norm, *k_norm;
} mi_layer_weights;

/* Pinned host staging of the host arrays a forward call reads: its token ids and positions (and,
 * for several sequences, the attention tile table and region pointers).  The prefill page takes
 * token ids and positions as host slices that are only read during the call ("09", section 2.2,
 * the forward signature), so the call copies them into pinned host memory before it returns and
 * the transfer to the device runs asynchronously from there: a small kernel, first on the call's
 * stream, reads the pinned buffer (mapped, coherent) into the workspace.  The stage is a ring of
 * MI_STAGE_RING pinned buffers, each guarded by a HIP event: a buffer is rewritten only after the
 * transfer that last read it has completed, so back-to-back calls never wait for the GPU unless they are
 * MI_STAGE_RING calls ahead of it.  Created once per model (it allocates pinned host memory and
 * events; nothing on the device); not thread-safe, like the mi_model that refers to it.
 *   mi_stage_create   hp and max_tokens as for mi_prefill_workspace_bytes; *out NULL on error
 *   mi_stage_destroy  waits for the transfers still reading the stage, then frees it (NULL: no-op) */
#define MI_STAGE_RING 4
typedef struct mi_stage mi_stage;
int mi_stage_create(const mi_hparams* hp, int32_t max_tokens, mi_stage** out);
void mi_stage_destroy(mi_stage* stage);

/* A loaded model plus the per-model buffers one forward uses.  Not thread-safe:
 * calls that share one mi_model (its workspace) must be serialized. */
typedef struct {
  mi_hparams hp;
  mi_q8_matrix token_embd;          /* [vocab][hidden]                       */
  mi_q8_matrix output;              /* [vocab][hidden]; ignored when tied    */
  const float* output_norm;         /* device [hidden]                       */
  const mi_layer_weights* layers;   /* host array [n_layers]                 */
  const double* rope_table;         /* device, filled by mi_rope_table_init  */
  int32_t rope_rows;                /* positions the table covers (>= n_ctx) */
  void* workspace;                  /* device scratch                        */
  size_t workspace_bytes;           /* >= mi_prefill_workspace_bytes(...)    */
  int32_t max_tokens;               /* largest n_tokens the workspace serves */
  void* stream;                     /* hipStream_t                           */
  mi_stage* stage;                  /* from mi_stage_create with >= max_tokens and these hparams */
} mi_model;

/* Persistent KV regions ("09", section 2.5): for each layer one K and one V
 * region, device f32 [n_ctx][n_head_kv*head_dim]; row p holds the position-p
 * token (K after RoPE, and after the QK norm for Qwen3; V raw plus bias).  The
 * caller owns them; they persist across calls so a later call can continue at
 * later positions. */
typedef struct {
  float* const* k;   /* host array [n_layers] of device pointers */
  float* const* v;
  int32_t n_layers, n_ctx, n_kv_embd;
} mi_kv_regions;

/* ------------------------------------------------------------------ forward */

/* Bytes of workspace one forward needs for up to max_tokens tokens. */
size_t mi_prefill_workspace_bytes(const mi_hparams* hp, int32_t max_tokens);

/* Bytes of the RoPE table for positions [0, rows): rows x (head_dim/2) x {cos, sin} f64. */
size_t mi_rope_table_bytes(const mi_hparams* hp, int32_t rows);

/* Fill a device RoPE table: entry (p, i) = cos/sin(p * theta^(-2i/head_dim)), computed
 * on the host in f64 and copied to `table` (device) on `stream` (synchronously). */
int mi_rope_table_init(const mi_hparams* hp, int32_t rows, double* table, void* stream);

/* The prefill forward ("09", sections 2.2-2.6; "05", sections 2.5 and 2.8).
 *   token_ids  host int32 [n_tokens], each in [0, vocab)
 *   positions  host int32 [n_tokens]: the KV row each token writes, the causal
 *              limit (token t sees rows 0..=positions[t]) and the RoPE angle
 *   n_ctx      rows of every KV region; must equal kv->n_ctx
 *   kv         the persistent regions; rows named by `positions` are overwritten;
 *              rows <= max(positions) not written by this call must hold earlier
 *              calls' rows (the caller's contract)
 *   logits_out device f32 [vocab]: logits of token n_tokens-1
 * Checks before enqueueing: every position in [0, n_ctx) (MI_ERR_POSITION_RANGE),
 * no position repeated (MI_ERR_DUP_POSITION), descriptor shapes
 * (MI_ERR_KV_MISMATCH), n_tokens <= model->max_tokens and workspace size
 * (MI_ERR_WORKSPACE), rope table rows >= n_ctx, the KV regions of all layers pairwise
 * disjoint (MI_ERR_INVALID_ARG), model->stage present and sized for max_tokens
 * (MI_ERR_INVALID_ARG / MI_ERR_WORKSPACE), and every activation offset of the kernels
 * (max_tokens times the widest row) below 2^31 (MI_ERR_UNSUPPORTED).
 * token_ids and positions are copied into model->stage before the call returns. */
int mi_prefill_forward(const mi_model* model, const int32_t* token_ids, const int32_t* positions,
                       int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv, float* logits_out);

/* The same forward with the logits of the last n_out tokens ("09", section 2.4: the tail rows
 * [n_tokens - n_out, n_tokens) continue past the last layer's output projection; "05",
 * section 2.8).  1 <= n_out <= n_tokens (MI_ERR_INVALID_ARG otherwise); n_out = n_tokens gives
 * the logits of every token.
 *   logits_out device f32 [n_out][vocab], row r = token n_tokens - n_out + r
 * mi_prefill_forward is this call with n_out = 1. */
int mi_prefill_forward_n(const mi_model* model, const int32_t* token_ids, const int32_t* positions,
                         int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv, int32_t n_out,
                         float* logits_out);

/* Several independent sequences ("slots") in one prefill call, each with its own KV regions and
 * positions ("09", section 2.2: positions need not count the tokens before them in the call, and a
 * server keeps one cache per slot; section 3.2: the slot-scoped cache entry).  One slot is
 * mi_prefill_forward.  The call computes, for every slot, exactly what mi_prefill_forward computes
 * for that slot's tokens alone over that slot's regions: the matmuls run over all slots' rows
 * together, the Q|K|V epilogue stores each row's K/V into its own slot's regions, and one
 * attention launch per layer covers every slot's query tiles (up to 16 rows of one slot each).
 *   slot_tokens  host int32 [n_slots]: the token count of each slot (>= 1); the slots' tokens are
 *                consecutive runs of token_ids / positions, in slot order
 *   kv           host array [n_slots] of region descriptors (each as for mi_prefill_forward)
 *   logits_out   device f32 [n_slots][vocab]: the last token of each slot
 * 1 <= n_slots <= MI_MAX_SLOTS; the total token count <= model->max_tokens; positions must not
 * repeat within a slot.  No two regions of any slots may overlap (two slots writing one region
 * would race): MI_ERR_INVALID_ARG.  Errors as mi_prefill_forward (nothing written).  The host
 * arrays are copied into model->stage before the call returns; the work is asynchronous. */
#define MI_MAX_SLOTS 64
int mi_prefill_forward_slots(const mi_model* model, const int32_t* token_ids, const int32_t* positions,
                             const int32_t* slot_tokens, int32_t n_slots, int32_t n_ctx, const mi_kv_regions* kv,
                             float* logits_out);

/* Decode step: one token `token_id` at `position`, through the same layers and KV regions as the
 * prefill (the second act of the walkthrough index's two-act engine; the prefill page, section
 * 2.2, for attention over region rows 0..=position).  Computes exactly what mi_prefill_forward
 * computes for n_tokens = 1 -- which runs the same one-row kernels: HBM-bound exact Q8_0
 * matrix-vector products with the RMSNorms in their prologues and the bias / residual / SwiGLU
 * work in their epilogues, and a single-query attention split over fixed key ranges (which also
 * applies the per-head QK norm and RoPE and stores the new K/V rows), whose ranges one more kernel
 * merges.
 *   token_id, position  host values, 0 <= token_id < vocab, 0 <= position < n_ctx
 *   logits_out          device f32 [vocab]
 * Writes K/V row `position` of every layer.  Errors as mi_prefill_forward (nothing written).
 * A captured graph (mi_prefill_graph_create with n_tokens = 1) replays decode steps at any
 * position. */
int mi_decode_step(const mi_model* model, int32_t token_id, int32_t position, int32_t n_ctx,
                   const mi_kv_regions* kv, float* logits_out);

/* ---- sampler: one next token from last-token logits (the sampler row of the walkthrough index:
 * penalties over the last-64 window -> top-k -> top-p -> temperature -> seeded sample).
 *   penalties   for token t seen c_t > 0 times in the window, in f64 from its f32 logit:
 *               l = l / repeat_penalty if l > 0 else l * repeat_penalty; then
 *               l - c_t * frequency_penalty - presence_penalty
 *   top-k       the top_k largest penalized logits, ties by the smaller token id
 *   top-p       softmax of those candidates at temperature 1 (temperature is the next step);
 *               the shortest prefix whose cumulative probability reaches top_p (at least one)
 *   temperature kept logits / temperature; temperature 0 picks the first candidate (greedy)
 *   sample      u = (SplitMix64 output number step+1 of the generator seeded with `seed`) >> 11,
 *               times 2^-53; weights e^(l_i - l_0); the first candidate whose running weight sum
 *               exceeds u times the total */
#define MI_SAMPLER_MAX_K 64
typedef struct mi_sampler_params {
  float repeat_penalty;     /* > 0; 1 = off */
  float frequency_penalty;  /* 0 = off */
  float presence_penalty;   /* 0 = off */
  int32_t top_k;            /* 1 .. MI_SAMPLER_MAX_K */
  float top_p;              /* (0, 1]; 1 = off */
  float temperature;        /* >= 0; 0 = greedy */
} mi_sampler_params;

/* Device workspace bytes mi_sample needs (caller-owned, any alignment of 256). */
size_t mi_sampler_workspace_bytes(void);

/* One token.
 *   logits     device f32 [vocab], finite or -inf; 1 <= vocab <= 262144
 *   window     host int32 [n_window], the recent token ids (only the last 64 count), each in
 *              [0, vocab); may be NULL when n_window is 0
 *   seed, step the draw's counter (step = the number of tokens sampled before in this sequence)
 *   token_out  device int32 [1]
 * Errors (MI_ERR_INVALID_ARG): bad sizes or parameters, window ids out of range; nothing is
 * written.  Enqueued on `stream`; the window is read before the call returns (it goes to the first
 * kernel as an argument), so the caller may reuse it at once. */
int mi_sample(const float* logits, int32_t vocab, const int32_t* window, int32_t n_window,
              const mi_sampler_params* params, uint64_t seed, uint64_t step, void* workspace,
              size_t workspace_bytes, int32_t* token_out, void* stream);

/* Graph replay of the forward for callers that repeat one shape (HIP graphs).
 * mi_prefill_graph_create validates the shapes like mi_prefill_forward_n, then captures the
 * forward's kernel sequence on model->stream (which must be a non-default stream) into a graph;
 * nothing runs and nothing is allocated on the device.  The graph keeps the pointers of `model`
 * (weights, workspace, RoPE table, stage), of `kv` and of `logits_out` as they are now: the caller
 * keeps them alive and unchanged until mi_prefill_graph_destroy.
 * mi_prefill_graph_launch validates token ids and positions (as mi_prefill_forward_n: errors leave
 * everything untouched), copies them into the model's pinned stage, enqueues their transfer to the
 * workspace and replays the graph on the captured stream; it computes exactly what
 * mi_prefill_forward_n computes for the same arguments.
 * Launches of one graph run in stream order; different graphs sharing a workspace must not
 * overlap.  *out is set to NULL on error. */
typedef struct mi_prefill_graph mi_prefill_graph;
int mi_prefill_graph_create(const mi_model* model, int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv,
                            int32_t n_out, float* logits_out, mi_prefill_graph** out);
int mi_prefill_graph_launch(mi_prefill_graph* graph, const int32_t* token_ids, const int32_t* positions);
/* The number of nodes (kernel launches) in the captured forward, into *n_nodes. */
int mi_prefill_graph_nodes(const mi_prefill_graph* graph, int32_t* n_nodes);
void mi_prefill_graph_destroy(mi_prefill_graph* graph);

/* ------------------------------------------------------------------ per-op calls */

/* Q8_0 quantize rows of f32 ("CPU matmul kernels" stage of the walkthrough index;
 * format as the workload defines it): for each block of 32 values
 * amax = max|x|, d = f32(amax/127), id = d ? f32(1/d) : 0,
 * code = round-half-away(f32(x*id)) clamped to [-127,127], stored scale fp16(d) RNE.
 *   x      device f32 [rows][cols], cols % 32 == 0
 *   codes  device int8 [rows][cols]; scales device uint16 (fp16 bits) [rows][cols/32] */
int mi_quantize_q8_0(const float* x, int64_t rows, int32_t cols, int8_t* codes, uint16_t* scales,
                     void* stream);

/* Q8_0 blocks in their canonical byte layout -> the library's two planes (the walkthrough index,
 * stage 10: quantized weights are fixed-layout C blocks).  A canonical block is 34 bytes: the fp16
 * scale (little-endian bits) followed by the 32 int8 codes; a row of cols values is cols/32 blocks
 * back to back, rows follow each other.  The planes receive exactly those bytes:
 * scales[r][b] = bytes 0..1 of block (r, b), codes[r][32b + i] = byte 2 + i of it.
 *   blocks  device, rows * (cols/32) * 34 bytes, 2-byte aligned
 *   codes   device int8 [rows][cols], 16-byte aligned; scales device uint16 [rows][cols/32]
 * cols % 32 == 0 and rows, cols > 0 (MI_ERR_INVALID_ARG otherwise). */
int mi_pack_q8_0(const void* blocks, int64_t rows, int32_t cols, int8_t* codes, uint16_t* scales, void* stream);

/* Q8_0 x Q8_0 matmul with inline bias and optional residual ("05", sections 2.5, 3.2):
 *   out[t][n] = residual[t][n] + f32( sum_kb da[t][kb] dw[n][kb] sum_32 qa qw + bias[n] )
 * a_codes/a_scales: device, the activations already in Q8_0 [m][k];
 * w: the weight [n][k]; bias device f32 [n] or NULL; residual device f32 [m][n] or
 * NULL (may alias out); out device f32 [m][n].  The block sums are exact (int8
 * MFMA, int32) and the scaled sum is accumulated in f64.  The kernels address operands with
 * 32-bit offsets: m*k, n*k and m*n must be below 2^31 (MI_ERR_UNSUPPORTED otherwise). */
int mi_gemm_q8_0(const int8_t* a_codes, const uint16_t* a_scales, int32_t m, const mi_q8_matrix* w,
                 const float* bias, const float* residual, float* out, void* stream);

/* The same matmul with a caller workspace for split-K partials (f64 [split][m][n], reduced in
 * a fixed order afterwards).  split_k = 0 lets the library choose; the split is lowered when the
 * workspace is too small.  mi_gemm_q8_0_workspace_bytes gives the bytes for its own choice. */
int mi_gemm_q8_0_ws(const int8_t* a_codes, const uint16_t* a_scales, int32_t m, const mi_q8_matrix* w,
                    const float* bias, const float* residual, float* out, void* workspace,
                    size_t workspace_bytes, int32_t split_k, void* stream);
size_t mi_gemm_q8_0_workspace_bytes(int32_t m, int32_t n, int32_t k);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): mi_gemm_q8_0_ws with the split-K partials in a static device
 * array of the library, MI_STATIC_SCRATCH_BYTES per GPU, held from the library's first use on that
 * GPU until the process ends.  Calls allocate nothing.  split_k = 0 lets the library choose and
 * lowers the split to what the array holds; an explicit split_k > 1 whose partials
 * (split_k * m * n * 8 bytes) exceed the array fails with MI_ERR_WORKSPACE.  All calls on one GPU
 * share the array: calls that may overlap on one GPU (other streams, other threads) race, so the
 * caller serializes them.  Results are those of mi_gemm_q8_0_ws with the same split. */
#define MI_STATIC_SCRATCH_BYTES (64u << 20)
int mi_gemm_q8_0_static(const int8_t* a_codes, const uint16_t* a_scales, int32_t m, const mi_q8_matrix* w,
                        const float* bias, const float* residual, float* out, int32_t split_k, void* stream);

/* gate|up matmul with SwiGLU and Q8_0 in the epilogue ("05", section 2.5 gate, up, SwiGLU):
 *   g = f32(x.Wgate), u = f32(x.Wup), s = f32(silu(g) * u), then s -> Q8_0.
 *   w_gate_up in the interleaved layout of mi_layer_weights ([2*ffn][k], rows % 64 == 0);
 *   s_codes device int8 [m][ffn], s_scales device uint16 [m][ffn/32]; workspace as above.
 *   32-bit offsets as for mi_gemm_q8_0. */
int mi_gemm_swiglu_q8_0(const int8_t* a_codes, const uint16_t* a_scales, int32_t m,
                        const mi_q8_matrix* w_gate_up, int8_t* s_codes, uint16_t* s_scales,
                        void* workspace, size_t workspace_bytes, void* stream);

/* RMSNorm then Q8_0 ("05", section 2.5 attn_norm / ffn_norm / output_norm):
 * y = f32(x / sqrt(mean(x^2) + eps) * gamma) per row, then quantized as above.
 *   x device f32 [rows][cols]; gamma device f32 [cols]; codes/scales as above.
 *   y_out optional device f32 [rows][cols] (NULL to skip). */
int mi_rmsnorm_quant(const float* x, const float* gamma, int64_t rows, int32_t cols, float eps,
                     int8_t* codes, uint16_t* scales, float* y_out, void* stream);

/* Per-head RMSNorm of Q and K over head_dim (Qwen3 QkNorm, "05", sections 2.3, 2.6),
 * in place.  x device f32 [rows][n_heads*head_dim]; gamma device f32 [head_dim]. */
int mi_qk_norm(float* x, const float* gamma, int64_t rows, int32_t n_heads, int32_t head_dim,
               float eps, void* stream);

/* NeoX RoPE of Q (in place) and K, then the KV store ("09", section 2.2: row p of the
 * layer's K and V regions <- the position-p token; "05", section 3.2: rotated K, raw V):
 *   q device f32 [n_tokens][n_head*head_dim], rotated in place
 *   k, v device f32 [n_tokens][n_head_kv*head_dim] (k is not modified)
 *   positions device int32 [n_tokens] (validated by the caller; see mi_prefill_forward)
 *   rope_table from mi_rope_table_init with rope_rows > max position
 *   k_region, v_region device f32 [n_ctx][n_head_kv*head_dim] */
int mi_rope_kvstore(float* q, const float* k, const float* v, const int32_t* positions,
                    int32_t n_tokens, int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                    const double* rope_table, int32_t rope_rows, float* k_region, float* v_region,
                    int32_t n_ctx, void* stream);

/* Causal GQA attention over a layer's regions ("09", section 2.2; "05", section 2.5):
 *   out[t][h] = sum_{j<=pos[t]} softmax_j(q[t][h].K[j][g] / sqrt(hd)) V[j][g],
 *   g = h / (n_head/n_head_kv).  q device f32 [n_tokens][n_head*head_dim];
 *   positions device int32 [n_tokens], each < n_ctx; out device f32 like q.
 *   max_pos: host copy of max(positions) (bounds the rows read). */
int mi_attention_gqa(const float* q, const float* k_region, const float* v_region,
                     const int32_t* positions, int32_t n_tokens, int32_t max_pos, int32_t n_head,
                     int32_t n_head_kv, int32_t head_dim, int32_t n_ctx, float* out, void* stream);

/* SwiGLU then Q8_0 ("05", section 2.5): s = f32(silu(g) * u), silu(x) = x*sigmoid(x),
 * quantized as above.  gate, up device f32 [rows][cols]. */
int mi_swiglu_quant(const float* gate, const float* up, int64_t rows, int32_t cols, int8_t* codes,
                    uint16_t* scales, void* stream);

/* Embedding rows: out[t] = dequant(table row ids[t]) ("05", section 2.5, GetRows).
 *   ids device int32 [n_tokens] in [0, table->rows); out device f32 [n_tokens][cols]. */
int mi_embed_q8_0(const mi_q8_matrix* table, const int32_t* ids, int32_t n_tokens, float* out,
                  void* stream);

/* Last-row lm_head ("09", section 2.4): RMSNorm of one hidden row, Q8_0, then the
 * matvec against the head matrix: logits[v] = f32(sum_kb dx dw sum qx qw).
 *   x device f32 [cols] (the last token's hidden state); gamma device f32 [cols];
 *   head [vocab][cols]; logits device f32 [vocab]; scratch device >= cols + 2*cols/32 bytes. */
int mi_lm_head_row(const float* x, const float* gamma, float eps, const mi_q8_matrix* head,
                   float* logits, void* scratch, void* stream);

/* Description of the last error on this thread ("" if none). */
const char* mi_last_error(void);

/* Library version string. */
const char* mi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MI_PREFILL_H */
