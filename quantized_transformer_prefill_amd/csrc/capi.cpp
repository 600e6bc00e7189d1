// C ABI: argument validation, the per-op entry points and the prefill forward.
//
// The forward is the Qwen2/Qwen3 layer sequence of the graph-build page (section 2.5):
// embedding -> per layer [attn RMSNorm+Q8_0 -> fused Q|K|V matmul (+bias) -> (Qwen3) per-head QK
// norm -> RoPE + KV store at positions -> causal GQA attention -> Q8_0 -> output projection +
// residual -> ffn RMSNorm+Q8_0 -> gate|up matmul with SwiGLU+Q8_0 fused in its epilogue -> down
// projection + residual] -> final RMSNorm+Q8_0 -> lm_head on the last row.  In the last layer only
// the last token's row continues after the attention output projection (the tail rows of the
// prefill page, section 2.4): its FFN, the final norm and the lm_head run on one row.
//
// Everything is validated on the host before anything is enqueued; nothing is allocated.
#include <cstdarg>
#include <cstring>
#include <vector>
#include <algorithm>
#include <cmath>

#include "common.h"

namespace mi {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_check(hipError_t e, const char* what) {
  return set_error(MI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool q8_ok(const mi_q8_matrix& w, int rows, int cols) {
  return w.codes && w.scales && w.rows == rows && w.cols == cols && cols % QK == 0;
}

// ---------------------------------------------------------------- workspace layout
struct Ws {
  // the staged part, contiguous at the start: one host-to-device copy from the pinned stage
  // (mi_stage) fills it with the same layout
  int32_t* ids; int32_t* pos;
  int32_t* maxpos;   // [1] largest position of the call
  float* h;          // [T][hidden]
  int8_t* xq;        // [T][max(hidden, nq, ffn)]
  uint16_t* xs;      // [T][max(...)/32]
  float* qkv;        // [T][nq + 2 nkv]
  float* attn;       // [T][nq]
  int8_t* sq;        // [T][ffn] SwiGLU output codes
  uint16_t* ss;      // [T][ffn/32]
  double* attn_part; // decode: partial attention states [n_head][AD_MAX_RANGES][head_dim + 2]
  // several sequences: one staging area copied in one transfer per call, holding the attention
  // query tiles [n_layers][n_tiles], region pointers [2][n_layers][MI_MAX_SLOTS] (K, V), the slot
  // of each row [T] and the last row of each slot [MI_MAX_SLOTS]
  char* slot_stage;
  size_t slot_stage_bytes;
  size_t staged_bytes;   // ids .. end of slot_stage
  int slot_tiles_max;    // per layer: T/16 + MI_MAX_SLOTS
  float* slot_h;         // several sequences: the slots' last rows gathered [MI_MAX_SLOTS][hidden]
  void* gemm_ws; size_t gemm_ws_bytes;
  size_t total;
};

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

static Ws carve(const mi_hparams& hp, int T, char* base) {
  Ws w{};
  const size_t nq = (size_t)hp.n_head * hp.head_dim, nkv = (size_t)hp.n_head_kv * hp.head_dim;
  const size_t wide = std::max({(size_t)hp.hidden, nq, (size_t)hp.ffn});
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += align_up(bytes); return p; };
  w.ids = (int32_t*)take(sizeof(int32_t) * T);
  w.pos = (int32_t*)take(sizeof(int32_t) * T);
  w.maxpos = (int32_t*)take(sizeof(int32_t));
  w.slot_tiles_max = T / 16 + MI_MAX_SLOTS;
  {
    const size_t L = (size_t)std::max(hp.n_layers, 1);
    w.slot_stage_bytes = align_up(sizeof(AttnSlotTile) * L * w.slot_tiles_max) +
                         align_up(sizeof(float*) * 2 * L * MI_MAX_SLOTS) + align_up(sizeof(int32_t) * (size_t)T) +
                         align_up(sizeof(int32_t) * MI_MAX_SLOTS);
    w.slot_stage = take(w.slot_stage_bytes);
  }
  w.staged_bytes = off;
  w.h = (float*)take(sizeof(float) * T * (size_t)hp.hidden);
  w.xq = (int8_t*)take((size_t)T * wide);
  w.xs = (uint16_t*)take(sizeof(uint16_t) * (size_t)T * (wide / QK));
  w.qkv = (float*)take(sizeof(float) * (size_t)T * (nq + 2 * nkv));
  w.attn = (float*)take(sizeof(float) * (size_t)T * nq);
  w.sq = (int8_t*)take((size_t)T * hp.ffn);
  w.ss = (uint16_t*)take(sizeof(uint16_t) * (size_t)T * (hp.ffn / QK));
  w.attn_part = (double*)take(sizeof(double) * (size_t)hp.n_head * AD_MAX_RANGES * (hp.head_dim + 2));
  w.slot_h = (float*)take(sizeof(float) * MI_MAX_SLOTS * (size_t)hp.hidden);
  size_t g = 0;
  g = std::max(g, gemm_workspace_bytes(T, (int)(nq + 2 * nkv), hp.hidden));
  g = std::max(g, gemm_workspace_bytes(T, hp.hidden, (int)nq));
  g = std::max(g, gemm_workspace_bytes(T, 2 * hp.ffn, hp.hidden));
  g = std::max(g, gemm_workspace_bytes(T, hp.hidden, hp.ffn));
  g = std::max(g, gemm_workspace_bytes(1, hp.hidden, (int)nq));
  g = std::max(g, gemm_workspace_bytes(1, 2 * hp.ffn, hp.hidden));
  g = std::max(g, gemm_workspace_bytes(1, hp.hidden, hp.ffn));
  w.gemm_ws = take(g);
  w.gemm_ws_bytes = g;
  w.total = off;
  return w;
}

static int check_hparams(const mi_hparams* hp) {
  if (!hp) return set_error(MI_ERR_INVALID_ARG, "hparams is NULL");
  if (hp->n_layers < 0 || hp->hidden <= 0 || hp->n_head <= 0 || hp->n_head_kv <= 0 || hp->head_dim <= 0 ||
      hp->ffn <= 0 || hp->vocab <= 0)
    return set_error(MI_ERR_INVALID_ARG, "hparams: sizes must be positive");
  if (hp->n_head % hp->n_head_kv) return set_error(MI_ERR_INVALID_ARG, "n_head %% n_head_kv != 0");
  if (hp->hidden % QK || hp->ffn % QK || (hp->n_head * hp->head_dim) % QK)
    return set_error(MI_ERR_INVALID_ARG, "hidden, ffn and n_head*head_dim must be multiples of 32");
  if (hp->head_dim != 64 && hp->head_dim != 128)
    return set_error(MI_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", hp->head_dim);
  if (hp->hidden > 4096) return set_error(MI_ERR_UNSUPPORTED, "hidden %d > 4096", hp->hidden);
  // the one-row matrix-vector kernels (the last layer's tail row, decode) stage a whole Q8_0 input
  // row in LDS: the attention output (n_head * head_dim values) and the SwiGLU row (ffn values)
  if ((int64_t)hp->n_head * hp->head_dim > GV_MAX_K || hp->ffn > GV_MAX_K)
    return set_error(MI_ERR_UNSUPPORTED, "n_head * head_dim %d or ffn %d above %d", hp->n_head * hp->head_dim,
                     hp->ffn, GV_MAX_K);
  if (hp->ffn % 32) return set_error(MI_ERR_INVALID_ARG, "ffn %% 32 != 0");
  return MI_OK;
}

}  // namespace mi

// ---------------------------------------------------------------- pinned host staging
// A ring of pinned host buffers, each a mirror of the workspace's staged part (ids, positions,
// largest position, the several-sequence tables) with the same offsets, so one call fills a buffer
// and a small kernel on the call's stream reads it into the workspace (zero-copy: no copy-engine
// transfer in front of the forward's first kernel).  The event recorded after that kernel tells when
// the buffer may be written again.
struct mi_stage {
  mi_hparams hp{};
  int32_t max_tokens = 0;
  size_t bytes = 0;  // per buffer
  char* host[MI_STAGE_RING] = {};
  const char* dev[MI_STAGE_RING] = {};  // the same buffers' device addresses
  hipEvent_t ev[MI_STAGE_RING] = {};
  bool pending[MI_STAGE_RING] = {};
  int next = 0;
};

namespace mi {

static void stage_free(mi_stage* st) {
  for (int i = 0; i < MI_STAGE_RING; ++i) {
    if (st->ev[i]) {
      if (st->pending[i]) (void)hipEventSynchronize(st->ev[i]);
      (void)hipEventDestroy(st->ev[i]);
    }
    if (st->host[i]) (void)hipHostFree(st->host[i]);
  }
  delete st;
}

// The staged part of workspace `w` (the carve of the model's max_tokens) must fit one buffer.
static int check_stage(const mi_model* md, const Ws& w) {
  if (!md->stage) return set_error(MI_ERR_INVALID_ARG, "forward: model->stage is NULL (mi_stage_create)");
  if (md->stage->bytes < w.staged_bytes)
    return set_error(MI_ERR_WORKSPACE, "forward: stage made for fewer tokens or layers than the model's max_tokens");
  return MI_OK;
}

// Take the next ring buffer (waiting for the copy that last read it), let fill() write it, and send
// its first n bytes to dev (the workspace's staged part) on stream s.
template <class F>
static int stage_send(mi_stage* st, void* dev, size_t n, hipStream_t s, F fill) {
  const int i = st->next;
  if (st->pending[i]) {
    MI_HIP(hipEventSynchronize(st->ev[i]));
    st->pending[i] = false;
  }
  st->next = (i + 1) % MI_STAGE_RING;
  fill(st->host[i]);
  if (int rc = launch_stage_in(dev, st->dev[i], n, s)) return rc;
  MI_HIP(hipEventRecord(st->ev[i], s));
  st->pending[i] = true;
  return MI_OK;
}

}  // namespace mi

using namespace mi;

extern "C" int mi_stage_create(const mi_hparams* hp, int32_t max_tokens, mi_stage** out) {
  if (!out) return set_error(MI_ERR_INVALID_ARG, "mi_stage_create: NULL output handle");
  *out = nullptr;
  int rc = check_hparams(hp);
  if (rc) return rc;
  if (max_tokens < 1) return set_error(MI_ERR_INVALID_ARG, "mi_stage_create: max_tokens must be >= 1");
  mi_stage* st = new mi_stage();
  st->hp = *hp;
  st->max_tokens = max_tokens;
  st->bytes = carve(*hp, max_tokens, nullptr).staged_bytes;
  for (int i = 0; i < MI_STAGE_RING; ++i) {
    // mapped and coherent: a kernel reads it over the bus (launch_stage_in)
    hipError_t e = hipHostMalloc((void**)&st->host[i], st->bytes, hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) e = hipHostGetDevicePointer((void**)&st->dev[i], st->host[i], 0);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      stage_free(st);
      return hip_check(e, "mi_stage_create");
    }
  }
  *out = st;
  return MI_OK;
}

extern "C" void mi_stage_destroy(mi_stage* st) {
  if (st) stage_free(st);
}

extern "C" const char* mi_last_error(void) { return g_err; }
extern "C" const char* mi_version(void) { return "mi_prefill 0.1 gfx950"; }

extern "C" size_t mi_prefill_workspace_bytes(const mi_hparams* hp, int32_t max_tokens) {
  if (check_hparams(hp) != MI_OK || max_tokens <= 0) return 0;
  return carve(*hp, max_tokens, nullptr).total;
}

// ---------------------------------------------------------------- per-op entry points
extern "C" int mi_quantize_q8_0(const float* x, int64_t rows, int32_t cols, int8_t* codes, uint16_t* scales,
                                void* stream) {
  if (!x || !codes || !scales || rows < 0 || cols <= 0 || cols % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_quantize_q8_0: bad arguments (cols must be a positive multiple of 32)");
  return launch_quantize(x, rows, cols, cols, codes, scales, as_stream(stream));
}

extern "C" int mi_pack_q8_0(const void* blocks, int64_t rows, int32_t cols, int8_t* codes, uint16_t* scales,
                            void* stream) {
  if (!blocks || !codes || !scales || rows <= 0 || cols <= 0 || cols % QK || ((uintptr_t)blocks & 1) ||
      ((uintptr_t)codes & 15) || ((uintptr_t)scales & 1))
    return set_error(MI_ERR_INVALID_ARG, "mi_pack_q8_0: bad arguments (cols a positive multiple of 32, blocks and "
                     "scales 2-byte aligned, codes 16-byte aligned)");
  return launch_pack_q8_0(blocks, rows, cols, codes, scales, as_stream(stream));
}

// The matmul kernels address their operands with 32-bit offsets (row * K and row * N)
static int check_gemm_offsets(const char* who, int64_t m, int64_t n, int64_t k) {
  if (m * k >= ((int64_t)1 << 31) || n * k >= ((int64_t)1 << 31) || m * n >= ((int64_t)1 << 31))
    return set_error(MI_ERR_UNSUPPORTED, "%s: m*k, n*k and m*n must be below 2^31 (m %lld, n %lld, k %lld)", who,
                     (long long)m, (long long)n, (long long)k);
  return MI_OK;
}

extern "C" int mi_gemm_q8_0(const int8_t* a_codes, const uint16_t* a_scales, int32_t m, const mi_q8_matrix* w,
                            const float* bias, const float* residual, float* out, void* stream) {
  if (!a_codes || !a_scales || !w || !w->codes || !w->scales || !out || m < 0 || w->rows <= 0 || w->cols <= 0 ||
      w->cols % QK || w->rows % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_gemm_q8_0: bad arguments (k and n multiples of 32)");
  if (int rc = check_gemm_offsets("mi_gemm_q8_0", m, w->rows, w->cols)) return rc;
  GemmArgs g{};
  g.a_codes = a_codes; g.a_scales = a_scales; g.m = m;
  g.w_codes = w->codes; g.w_scales = w->scales; g.n = w->rows; g.k = w->cols;
  g.bias = bias; g.residual = residual; g.out = out; g.ld_out = w->rows;
  g.split_k = 1;
  return launch_gemm_q8(g, as_stream(stream));
}

extern "C" int mi_gemm_q8_0_ws(const int8_t* a_codes, const uint16_t* a_scales, int32_t m, const mi_q8_matrix* w,
                               const float* bias, const float* residual, float* out, void* workspace,
                               size_t workspace_bytes, int32_t split_k, void* stream) {
  if (!a_codes || !a_scales || !w || !w->codes || !w->scales || !out || m < 0 || w->rows <= 0 || w->cols <= 0 ||
      w->cols % QK || w->rows % QK || split_k < 0)
    return set_error(MI_ERR_INVALID_ARG, "mi_gemm_q8_0_ws: bad arguments");
  if (int rc = check_gemm_offsets("mi_gemm_q8_0_ws", m, w->rows, w->cols)) return rc;
  GemmArgs g{};
  g.a_codes = a_codes; g.a_scales = a_scales; g.m = m;
  g.w_codes = w->codes; g.w_scales = w->scales; g.n = w->rows; g.k = w->cols;
  g.bias = bias; g.residual = residual; g.out = out; g.ld_out = w->rows;
  g.workspace = workspace; g.workspace_bytes = workspace_bytes; g.split_k = split_k;
  return launch_gemm_q8(g, as_stream(stream));
}

extern "C" int mi_gemm_q8_0_static(const int8_t* a_codes, const uint16_t* a_scales, int32_t m,
                                   const mi_q8_matrix* w, const float* bias, const float* residual, float* out,
                                   int32_t split_k, void* stream) {
  if (!a_codes || !a_scales || !w || !w->codes || !w->scales || !out || m < 0 || w->rows <= 0 || w->cols <= 0 ||
      w->cols % QK || w->rows % QK || split_k < 0)
    return set_error(MI_ERR_INVALID_ARG, "mi_gemm_q8_0_static: bad arguments");
  if (int rc = check_gemm_offsets("mi_gemm_q8_0_static", m, w->rows, w->cols)) return rc;
  if (split_k > 1 && (uint64_t)split_k * (uint64_t)m * (uint64_t)w->rows * sizeof(double) > MI_STATIC_SCRATCH_BYTES)
    return set_error(MI_ERR_WORKSPACE, "mi_gemm_q8_0_static: split %d x %d x %d f64 partials exceed the %u-byte "
                     "static scratch", split_k, m, w->rows, (unsigned)MI_STATIC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (int rc = static_scratch(&scratch)) return rc;
  GemmArgs g{};
  g.a_codes = a_codes; g.a_scales = a_scales; g.m = m;
  g.w_codes = w->codes; g.w_scales = w->scales; g.n = w->rows; g.k = w->cols;
  g.bias = bias; g.residual = residual; g.out = out; g.ld_out = w->rows;
  g.workspace = scratch; g.workspace_bytes = MI_STATIC_SCRATCH_BYTES; g.split_k = split_k;
  return launch_gemm_q8(g, as_stream(stream));
}

extern "C" size_t mi_gemm_q8_0_workspace_bytes(int32_t m, int32_t n, int32_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  return gemm_workspace_bytes(m, n, k);
}

extern "C" int mi_gemm_swiglu_q8_0(const int8_t* a_codes, const uint16_t* a_scales, int32_t m,
                                   const mi_q8_matrix* w_gate_up, int8_t* s_codes, uint16_t* s_scales,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!a_codes || !a_scales || !w_gate_up || !w_gate_up->codes || !w_gate_up->scales || !s_codes || !s_scales ||
      m < 0 || w_gate_up->rows <= 0 || w_gate_up->rows % 64 || w_gate_up->cols % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_gemm_swiglu_q8_0: bad arguments (rows a multiple of 64)");
  if (int rc = check_gemm_offsets("mi_gemm_swiglu_q8_0", m, w_gate_up->rows, w_gate_up->cols)) return rc;
  GemmArgs g{};
  g.a_codes = a_codes; g.a_scales = a_scales; g.m = m;
  g.w_codes = w_gate_up->codes; g.w_scales = w_gate_up->scales; g.n = w_gate_up->rows; g.k = w_gate_up->cols;
  g.q_codes = s_codes; g.q_scales = s_scales;
  g.workspace = workspace; g.workspace_bytes = workspace_bytes;
  return launch_gemm_q8(g, as_stream(stream));
}

extern "C" int mi_rmsnorm_quant(const float* x, const float* gamma, int64_t rows, int32_t cols, float eps,
                                int8_t* codes, uint16_t* scales, float* y_out, void* stream) {
  if (!x || !gamma || !codes || !scales || rows < 0 || cols <= 0 || cols % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_rmsnorm_quant: bad arguments");
  // no pending partials: x is only read
  return launch_rmsnorm_quant(const_cast<float*>(x), gamma, rows, cols, eps, codes, scales, y_out, as_stream(stream));
}

extern "C" int mi_qk_norm(float* x, const float* gamma, int64_t rows, int32_t n_heads, int32_t head_dim, float eps,
                          void* stream) {
  if (!x || !gamma || rows < 0 || n_heads <= 0 || head_dim <= 0 || head_dim > 128)
    return set_error(MI_ERR_INVALID_ARG, "mi_qk_norm: bad arguments (head_dim <= 128)");
  return launch_qk_norm(x, (int64_t)n_heads * head_dim, gamma, rows, n_heads, head_dim, eps, as_stream(stream));
}

extern "C" int mi_rope_kvstore(float* q, const float* k, const float* v, const int32_t* positions, int32_t n_tokens,
                               int32_t n_head, int32_t n_head_kv, int32_t head_dim, const double* rope_table,
                               int32_t rope_rows, float* k_region, float* v_region, int32_t n_ctx, void* stream) {
  if (!q || !k || !v || !positions || !rope_table || !k_region || !v_region || n_tokens < 0 || n_head <= 0 ||
      n_head_kv <= 0 || head_dim <= 0 || (head_dim & 1) || n_ctx <= 0 || rope_rows < n_ctx)
    return set_error(MI_ERR_INVALID_ARG, "mi_rope_kvstore: bad arguments (rope_rows must cover n_ctx)");
  return launch_rope_kvstore(q, (int64_t)n_head * head_dim, k, v, (int64_t)n_head_kv * head_dim, positions, n_tokens,
                             n_head, n_head_kv, head_dim, rope_table, k_region, v_region, as_stream(stream));
}

extern "C" int mi_attention_gqa(const float* q, const float* k_region, const float* v_region,
                                const int32_t* positions, int32_t n_tokens, int32_t max_pos, int32_t n_head,
                                int32_t n_head_kv, int32_t head_dim, int32_t n_ctx, float* out, void* stream) {
  if (!q || !k_region || !v_region || !positions || !out || n_tokens < 0 || n_head <= 0 || n_head_kv <= 0 ||
      n_head % n_head_kv || n_ctx <= 0)
    return set_error(MI_ERR_INVALID_ARG, "mi_attention_gqa: bad arguments");
  if (max_pos < 0 || max_pos >= n_ctx) return set_error(MI_ERR_POSITION_RANGE, "max_pos %d outside [0, %d)", max_pos, n_ctx);
  if ((int64_t)n_ctx * n_head_kv * head_dim > INT32_MAX)
    return set_error(MI_ERR_INVALID_ARG, "mi_attention_gqa: n_ctx * n_head_kv * head_dim exceeds 2^31 elements");
  return launch_attention(q, (int64_t)n_head * head_dim, k_region, v_region, positions, n_tokens, nullptr, max_pos,
                          n_head, n_head_kv, head_dim, out, (int64_t)n_head * head_dim, as_stream(stream));
}

extern "C" int mi_swiglu_quant(const float* gate, const float* up, int64_t rows, int32_t cols, int8_t* codes,
                               uint16_t* scales, void* stream) {
  if (!gate || !up || !codes || !scales || rows < 0 || cols <= 0 || cols % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_swiglu_quant: bad arguments");
  return launch_swiglu_quant(gate, up, rows, cols, cols, codes, scales, as_stream(stream));
}

extern "C" int mi_embed_q8_0(const mi_q8_matrix* table, const int32_t* ids, int32_t n_tokens, float* out,
                             void* stream) {
  if (!table || !table->codes || !table->scales || !ids || !out || n_tokens < 0 || table->cols % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_embed_q8_0: bad arguments");
  return launch_embed(table->codes, table->scales, table->cols, ids, n_tokens, out, as_stream(stream));
}

extern "C" int mi_lm_head_row(const float* x, const float* gamma, float eps, const mi_q8_matrix* head, float* logits,
                              void* scratch, void* stream) {
  if (!x || !gamma || !head || !head->codes || !head->scales || !logits || !scratch || head->cols % QK)
    return set_error(MI_ERR_INVALID_ARG, "mi_lm_head_row: bad arguments");
  int8_t* xq = (int8_t*)scratch;
  uint16_t* xs = (uint16_t*)((char*)scratch + align_up(head->cols));
  hipStream_t s = as_stream(stream);
  int rc = launch_rmsnorm_quant(const_cast<float*>(x), gamma, 1, head->cols, eps, xq, xs, nullptr, s);
  if (rc) return rc;
  return launch_lm_head(xq, xs, head->cols, head->codes, head->scales, head->rows, logits, s);
}

// ---------------------------------------------------------------- sampler
extern "C" size_t mi_sampler_workspace_bytes(void) { return sampler_workspace_bytes(); }

extern "C" int mi_sample(const float* logits, int32_t vocab, const int32_t* window, int32_t n_window,
                         const mi_sampler_params* p, uint64_t seed, uint64_t step, void* workspace,
                         size_t workspace_bytes, int32_t* token_out, void* stream) {
  if (!logits || !p || !token_out || !workspace || vocab < 1 || vocab > 256 * 1024 || n_window < 0 ||
      (n_window > 0 && !window))
    return set_error(MI_ERR_INVALID_ARG, "mi_sample: bad arguments (1 <= vocab <= 262144)");
  if (workspace_bytes < sampler_workspace_bytes())
    return set_error(MI_ERR_WORKSPACE, "mi_sample: workspace smaller than mi_sampler_workspace_bytes()");
  if (p->top_k < 1 || p->top_k > MI_SAMPLER_MAX_K || !(p->top_p > 0.0f && p->top_p <= 1.0f) ||
      !(p->temperature >= 0.0f) || !(p->repeat_penalty > 0.0f) || !std::isfinite(p->temperature) ||
      !std::isfinite(p->repeat_penalty) || !std::isfinite(p->frequency_penalty) || !std::isfinite(p->presence_penalty))
    return set_error(MI_ERR_INVALID_ARG, "mi_sample: parameters out of range (top_k 1..%d, top_p in (0, 1], "
                     "temperature >= 0, repeat_penalty > 0, all finite)", MI_SAMPLER_MAX_K);
  const int nw = std::min(n_window, 64);
  const int32_t* w = window + (n_window - nw);  // the last 64 count
  for (int i = 0; i < nw; ++i)
    if (w[i] < 0 || w[i] >= vocab) return set_error(MI_ERR_INVALID_ARG, "mi_sample: window id %d outside [0, %d)", w[i], vocab);
  return launch_sample(logits, vocab, w, nw, *p, seed, step, workspace, token_out, as_stream(stream));
}

// ---------------------------------------------------------------- the forward
static int validate_kv(const mi_hparams& hp, const mi_kv_regions* kv, int32_t n_ctx) {
  if (!kv) return set_error(MI_ERR_INVALID_ARG, "forward: NULL kv descriptor");
  if (kv->n_ctx != n_ctx) return set_error(MI_ERR_KV_MISMATCH, "forward: kv n_ctx %d != call n_ctx %d", kv->n_ctx, n_ctx);
  if (kv->n_layers != hp.n_layers || kv->n_kv_embd != hp.n_head_kv * hp.head_dim || !kv->k || !kv->v)
    return set_error(MI_ERR_KV_MISMATCH, "forward: kv descriptor does not match the model");
  for (int l = 0; l < hp.n_layers; ++l)
    if (!kv->k[l] || !kv->v[l]) return set_error(MI_ERR_KV_MISMATCH, "forward: kv region of layer %d is NULL", l);
  if ((int64_t)n_ctx * kv->n_kv_embd > INT32_MAX)  // the kernels address a region with 32-bit element offsets
    return set_error(MI_ERR_INVALID_ARG, "forward: n_ctx * n_kv_embd exceeds 2^31 elements");
  return MI_OK;
}

// No two KV regions of the descriptors overlap (two regions sharing memory would make the stores of
// one call race, or one sequence overwrite another's rows).
static int validate_kv_disjoint(const mi_kv_regions* kv, int n_sets) {
  std::vector<std::pair<uintptr_t, uintptr_t>> iv;
  for (int sl = 0; sl < n_sets; ++sl) {
    const size_t bytes = sizeof(float) * (size_t)kv[sl].n_ctx * kv[sl].n_kv_embd;
    for (int l = 0; l < kv[sl].n_layers; ++l) {
      iv.emplace_back((uintptr_t)kv[sl].k[l], (uintptr_t)kv[sl].k[l] + bytes);
      iv.emplace_back((uintptr_t)kv[sl].v[l], (uintptr_t)kv[sl].v[l] + bytes);
    }
  }
  std::sort(iv.begin(), iv.end());
  for (size_t i = 1; i < iv.size(); ++i)
    if (iv[i].first < iv[i - 1].second)
      return set_error(MI_ERR_INVALID_ARG, "forward: two KV regions overlap (each layer's K and V region, and each "
                       "sequence's, must be distinct memory)");
  return MI_OK;
}

static int validate_static(const mi_model* md, int32_t nt, int32_t n_ctx, const mi_kv_regions* kv,
                           const float* logits, int32_t n_out) {
  if (!md || !kv || !logits) return set_error(MI_ERR_INVALID_ARG, "forward: NULL argument");
  int rc = check_hparams(&md->hp);
  if (rc) return rc;
  const mi_hparams& hp = md->hp;
  if (nt < 1) return set_error(MI_ERR_INVALID_ARG, "forward: n_tokens must be >= 1");
  if (n_out < 1 || n_out > nt) return set_error(MI_ERR_INVALID_ARG, "forward: n_out %d outside [1, n_tokens = %d]", n_out, nt);
  if (n_ctx < 1) return set_error(MI_ERR_INVALID_ARG, "forward: n_ctx must be >= 1");
  if ((rc = validate_kv(hp, kv, n_ctx))) return rc;
  if ((rc = validate_kv_disjoint(kv, 1))) return rc;
  if (nt > md->max_tokens) return set_error(MI_ERR_WORKSPACE, "forward: n_tokens %d > max_tokens %d", nt, md->max_tokens);
  if (!md->workspace || md->workspace_bytes < carve(hp, md->max_tokens, nullptr).total)
    return set_error(MI_ERR_WORKSPACE, "forward: workspace smaller than mi_prefill_workspace_bytes(max_tokens)");
  if (!md->rope_table || md->rope_rows < n_ctx) return set_error(MI_ERR_INVALID_ARG, "forward: rope table rows < n_ctx");
  const int nq = hp.n_head * hp.head_dim, nkv = hp.n_head_kv * hp.head_dim;
  if (!q8_ok(md->token_embd, hp.vocab, hp.hidden)) return set_error(MI_ERR_INVALID_ARG, "forward: token_embd shape");
  if (!hp.tied && !q8_ok(md->output, hp.vocab, hp.hidden)) return set_error(MI_ERR_INVALID_ARG, "forward: output shape");
  if (!md->output_norm || (hp.n_layers && !md->layers)) return set_error(MI_ERR_INVALID_ARG, "forward: missing tensors");
  for (int l = 0; l < hp.n_layers; ++l) {
    const mi_layer_weights& L = md->layers[l];
    if (!q8_ok(L.wqkv, nq + 2 * nkv, hp.hidden) || !q8_ok(L.wo, hp.hidden, nq) ||
        !q8_ok(L.w_gate_up, 2 * hp.ffn, hp.hidden) || !q8_ok(L.w_down, hp.hidden, hp.ffn) || !L.attn_norm ||
        !L.ffn_norm || (hp.qkv_bias && !L.bqkv) || (hp.qk_norm && (!L.q_norm || !L.k_norm)))
      return set_error(MI_ERR_INVALID_ARG, "forward: layer %d tensors missing or mis-shaped", l);
  }
  if (hp.ffn % 32) return set_error(MI_ERR_INVALID_ARG, "forward: ffn %% 32");
  // 32-bit offsets of the kernels: activation rows (max_tokens of them) and weight rows
  const int64_t wide = std::max({(int64_t)hp.hidden, (int64_t)nq + 2 * nkv, (int64_t)2 * hp.ffn});
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)md->max_tokens * wide >= lim || ((int64_t)nq + 2 * nkv) * hp.hidden >= lim ||
      (int64_t)2 * hp.ffn * hp.hidden >= lim || (int64_t)hp.vocab * hp.hidden >= lim)
    return set_error(MI_ERR_UNSUPPORTED, "forward: max_tokens %d x row width %lld (or a weight matrix) reaches 2^31 "
                     "elements, beyond the kernels' 32-bit offsets", md->max_tokens, (long long)wide);
  return MI_OK;
}

// token ids and positions: ranges, no repeated position; returns the largest position
static int validate_tokens(const mi_hparams& hp, const int32_t* ids, const int32_t* pos, int32_t nt, int32_t n_ctx,
                           int* max_pos) {
  if (!ids || !pos) return set_error(MI_ERR_INVALID_ARG, "forward: NULL token ids or positions");
  int mp = 0;
  for (int t = 0; t < nt; ++t) {
    if (pos[t] < 0 || pos[t] >= n_ctx)
      return set_error(MI_ERR_POSITION_RANGE, "forward: position %d of token %d outside [0, %d)", pos[t], t, n_ctx);
    if (ids[t] < 0 || ids[t] >= hp.vocab)
      return set_error(MI_ERR_INVALID_ARG, "forward: token id %d of token %d outside [0, %d)", ids[t], t, hp.vocab);
    mp = std::max(mp, pos[t]);
  }
  std::vector<int32_t> sorted(pos, pos + nt);
  std::sort(sorted.begin(), sorted.end());
  for (int t = 1; t < nt; ++t)
    if (sorted[t] == sorted[t - 1]) return set_error(MI_ERR_DUP_POSITION, "forward: position %d repeated", sorted[t]);
  *max_pos = mp;
  return MI_OK;
}

// boundary staging: token ids, positions and the largest position copied into the next pinned
// buffer of the stage (before the call returns), then read into the workspace by one small kernel
static int stage_tokens(mi_stage* st, const Ws& w, const int32_t* ids, const int32_t* pos, int32_t nt, int32_t max_pos,
                        hipStream_t s) {
  char* base = reinterpret_cast<char*>(w.ids);
  const size_t o_pos = (char*)w.pos - base, o_max = (char*)w.maxpos - base;
  return stage_send(st, base, o_max + sizeof(int32_t), s, [&](char* h) {
    std::memcpy(h, ids, sizeof(int32_t) * nt);
    std::memcpy(h + o_pos, pos, sizeof(int32_t) * nt);
    std::memcpy(h + o_max, &max_pos, sizeof(int32_t));
  });
}

// The decode step: one token through the same layers and regions, with the one-row kernels
// (decode.hip).  Per layer: Q|K|V matrix-vector product with the attention RMSNorm in its prologue
// and the bias in its epilogue; single-query attention over ranges of keys 0..pos, which also applies
// the QK norm and RoPE and stores the new K/V rows; the ranges merged into a Q8_0 row; output projection + residual;
// gate|up with the ffn RMSNorm in its prologue and SwiGLU + Q8_0 in its epilogue; down projection
// + residual.  Then the lm_head with the final RMSNorm in its prologue.
static int enqueue_decode(const mi_model* md, const Ws& w, int32_t n_ctx, const mi_kv_regions* kv, float* logits_out,
                          hipStream_t s) {
  const mi_hparams& hp = md->hp;
  const int H = hp.hidden, F = hp.ffn;
  const int nq = hp.n_head * hp.head_dim, nkv = hp.n_head_kv * hp.head_dim, nqkv = nq + 2 * nkv;
  const float eps = hp.rms_eps;
  int rc;
  if ((rc = launch_embed(md->token_embd.codes, md->token_embd.scales, H, w.ids, 1, w.h, s))) return rc;
  for (int l = 0; l < hp.n_layers; ++l) {
    const mi_layer_weights& L = md->layers[l];
    GemvArgs g{};
    g.x = w.h; g.gamma = L.attn_norm; g.eps = eps; g.k = H;
    g.w_codes = L.wqkv.codes; g.w_scales = L.wqkv.scales; g.n = nqkv;
    g.bias = hp.qkv_bias ? L.bqkv : nullptr; g.out = w.qkv; g.epi = GV_F32;
    if ((rc = launch_gemv_q8(g, s))) return rc;
    const AttnFinish fin{md->rope_table, hp.qk_norm ? L.q_norm : nullptr, hp.qk_norm ? L.k_norm : nullptr, eps};
    if ((rc = launch_attn_decode(w.qkv, kv->k[l], kv->v[l], w.pos, n_ctx, hp.n_head, hp.n_head_kv, hp.head_dim,
                                 w.attn_part, &fin, s)))
      return rc;
    if ((rc = launch_attn_merge(w.attn_part, n_ctx, w.pos, hp.n_head, hp.head_dim, w.xq, w.xs, s))) return rc;
    GemvArgs go{};  // input: the merged attention row
    go.xq = w.xq; go.xs = w.xs; go.k = nq;
    go.w_codes = L.wo.codes; go.w_scales = L.wo.scales; go.n = H;
    go.residual = w.h; go.out = w.h; go.epi = GV_RES;
    if ((rc = launch_gemv_q8(go, s))) return rc;
    GemvArgs gg{};
    gg.x = w.h; gg.gamma = L.ffn_norm; gg.eps = eps; gg.k = H;
    gg.w_codes = L.w_gate_up.codes; gg.w_scales = L.w_gate_up.scales; gg.n = 2 * F;
    gg.q_codes = w.sq; gg.q_scales = w.ss; gg.epi = GV_SWIGLU;
    if ((rc = launch_gemv_q8(gg, s))) return rc;
    GemvArgs gd{};
    gd.xq = w.sq; gd.xs = w.ss; gd.k = F;
    gd.w_codes = L.w_down.codes; gd.w_scales = L.w_down.scales; gd.n = H;
    gd.residual = w.h; gd.out = w.h; gd.epi = GV_RES;
    if ((rc = launch_gemv_q8(gd, s))) return rc;
  }
  const mi_q8_matrix& head = hp.tied ? md->token_embd : md->output;
  GemvArgs gl{};
  gl.x = w.h; gl.gamma = md->output_norm; gl.eps = eps; gl.k = H;
  gl.w_codes = head.codes; gl.w_scales = head.scales; gl.n = head.rows;
  gl.out = logits_out; gl.epi = GV_F32;
  return launch_gemv_q8(gl, s);
}

// Every kernel of one forward, in order, on stream s.  Reads the staged ids, positions and largest
// position from the workspace; the sequence depends only on the shapes, so it can be captured
// once into a HIP graph and replayed.
static int enqueue_forward(const mi_model* md, const Ws& w, int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv,
                           int32_t n_out, float* logits_out, hipStream_t s) {
  const mi_hparams& hp = md->hp;
  const int nt = n_tokens, H = hp.hidden, F = hp.ffn;
  const int nq = hp.n_head * hp.head_dim, nkv = hp.n_head_kv * hp.head_dim, nqkv = nq + 2 * nkv;
  const float eps = hp.rms_eps;
  if (nt == 1) return enqueue_decode(md, w, n_ctx, kv, logits_out, s);  // one token: the decode kernels
  int rc;
  if ((rc = launch_embed(md->token_embd.codes, md->token_embd.scales, H, w.ids, nt, w.h, s))) return rc;
  float* h_tail = w.h + (size_t)(nt - n_out) * H;  // the tail rows [nt - n_out, nt)
  // the down projection's split-K partials, reduced (with its residual add) by the next RMSNorm
  int pending = 1;
  for (int l = 0; l < hp.n_layers; ++l) {
    const mi_layer_weights& L = md->layers[l];
    const bool last = l == hp.n_layers - 1;
    if ((rc = launch_rmsnorm_quant(w.h, L.attn_norm, nt, H, eps, w.xq, w.xs, nullptr, s, (const double*)w.gemm_ws,
                                   pending)))
      return rc;
    // Q|K|V matmul; its epilogue applies the QK norm (Qwen3) and RoPE, writes Q, and stores the
    // rotated K and the raw V into the layer's regions at the tokens' positions
    GemmArgs g{};
    g.a_codes = w.xq; g.a_scales = w.xs; g.m = nt;
    g.w_codes = L.wqkv.codes; g.w_scales = L.wqkv.scales; g.n = nqkv; g.k = H;
    g.bias = hp.qkv_bias ? L.bqkv : nullptr; g.out = w.qkv; g.ld_out = nqkv;
    g.workspace = w.gemm_ws; g.workspace_bytes = w.gemm_ws_bytes;
    g.qkv.pos = w.pos; g.qkv.rope = md->rope_table; g.qkv.n_q = nq; g.qkv.n_kv = nkv; g.qkv.head_dim = hp.head_dim;
    g.qkv.k_region = kv->k[l]; g.qkv.v_region = kv->v[l];
    g.qkv.q_norm = hp.qk_norm ? L.q_norm : nullptr; g.qkv.k_norm = hp.qk_norm ? L.k_norm : nullptr; g.qkv.eps = eps;
    if ((rc = launch_gemm_q8(g, s))) return rc;
    float* q = w.qkv;
    if (last && n_out == 1) {
      // From here on only the last token continues, through the one-token kernels of the decode
      // step: single-query attention over key ranges (reading the regions after the store above),
      // the ranges merged into a Q8_0 row, then matrix-vector products whose prologues apply the
      // RMSNorm and whose epilogues add the residual or apply SwiGLU + Q8_0; the final RMSNorm is
      // the lm_head's prologue.  The previous layer's deferred partials were reduced by this
      // layer's RMSNorm.
      const int32_t* pos1 = w.pos + (nt - 1);
      if ((rc = launch_attn_decode(q + (size_t)(nt - 1) * nqkv, kv->k[l], kv->v[l], pos1, n_ctx, hp.n_head,
                                   hp.n_head_kv, hp.head_dim, w.attn_part, nullptr, s)))
        return rc;
      if ((rc = launch_attn_merge(w.attn_part, n_ctx, pos1, hp.n_head, hp.head_dim, w.xq, w.xs, s))) return rc;
      GemvArgs go{};
      go.xq = w.xq; go.xs = w.xs; go.k = nq;
      go.w_codes = L.wo.codes; go.w_scales = L.wo.scales; go.n = H;
      go.residual = h_tail; go.out = h_tail; go.epi = GV_RES;
      if ((rc = launch_gemv_q8(go, s))) return rc;
      GemvArgs gg{};
      gg.x = h_tail; gg.gamma = L.ffn_norm; gg.eps = eps; gg.k = H;
      gg.w_codes = L.w_gate_up.codes; gg.w_scales = L.w_gate_up.scales; gg.n = 2 * F;
      gg.q_codes = w.sq; gg.q_scales = w.ss; gg.epi = GV_SWIGLU;
      if ((rc = launch_gemv_q8(gg, s))) return rc;
      GemvArgs gd{};
      gd.xq = w.sq; gd.xs = w.ss; gd.k = F;
      gd.w_codes = L.w_down.codes; gd.w_scales = L.w_down.scales; gd.n = H;
      gd.residual = h_tail; gd.out = h_tail; gd.epi = GV_RES;
      if ((rc = launch_gemv_q8(gd, s))) return rc;
      const mi_q8_matrix& head1 = hp.tied ? md->token_embd : md->output;
      GemvArgs gl{};
      gl.x = h_tail; gl.gamma = md->output_norm; gl.eps = eps; gl.k = H;
      gl.w_codes = head1.codes; gl.w_scales = head1.scales; gl.n = head1.rows;
      gl.out = logits_out; gl.epi = GV_F32;
      return launch_gemv_q8(gl, s);
    }
    // attention, its output rows quantized to Q8_0 in the same kernel.  In the last layer only the
    // last n_out tokens continue past the output projection, so only their rows are computed (the
    // KV store above covered every token).
    const int rows = last ? n_out : nt;
    const int t0 = nt - rows;
    float* h_rows = last ? h_tail : w.h;
    if ((rc = launch_attention(q + (size_t)t0 * nqkv, nqkv, kv->k[l], kv->v[l], w.pos + t0, rows, w.maxpos, 0,
                               hp.n_head, hp.n_head_kv, hp.head_dim, nullptr, nq, s, w.xq, w.xs)))
      return rc;
    GemmArgs go{};
    go.a_codes = w.xq; go.a_scales = w.xs; go.m = rows;
    go.w_codes = L.wo.codes; go.w_scales = L.wo.scales; go.n = H; go.k = nq;
    go.residual = h_rows; go.out = h_rows; go.ld_out = H;
    go.workspace = w.gemm_ws; go.workspace_bytes = w.gemm_ws_bytes;
    // split-K partials of the output projection (short reductions included), reduced with its
    // residual add by the FFN RMSNorm
    int pending_o = 1;
    go.split_out = &pending_o;
    if ((rc = launch_gemm_q8(go, s))) return rc;
    if ((rc = launch_rmsnorm_quant(h_rows, L.ffn_norm, rows, H, eps, w.xq, w.xs, nullptr, s, (const double*)w.gemm_ws,
                                   pending_o)))
      return rc;
    GemmArgs gg{};
    gg.a_codes = w.xq; gg.a_scales = w.xs; gg.m = rows;
    gg.w_codes = L.w_gate_up.codes; gg.w_scales = L.w_gate_up.scales; gg.n = 2 * F; gg.k = H;
    int8_t* s_codes = w.sq;
    uint16_t* s_scales = w.ss;
    gg.q_codes = s_codes; gg.q_scales = s_scales;
    gg.workspace = w.gemm_ws; gg.workspace_bytes = w.gemm_ws_bytes;
    if ((rc = launch_gemm_q8(gg, s))) return rc;
    GemmArgs gd{};
    gd.a_codes = s_codes; gd.a_scales = s_scales; gd.m = rows;
    gd.w_codes = L.w_down.codes; gd.w_scales = L.w_down.scales; gd.n = H; gd.k = F;
    gd.residual = h_rows; gd.out = h_rows; gd.ld_out = H;
    gd.workspace = w.gemm_ws; gd.workspace_bytes = w.gemm_ws_bytes;
    gd.split_out = &pending;
    if ((rc = launch_gemm_q8(gd, s))) return rc;
  }
  // several rows (n_out > 1; one row returned inside the last layer): the MFMA matmul, logits
  // [n_out][vocab]
  const mi_q8_matrix& head = hp.tied ? md->token_embd : md->output;
  if ((rc = launch_rmsnorm_quant(h_tail, md->output_norm, n_out, H, eps, w.xq, w.xs, nullptr, s,
                                 (const double*)w.gemm_ws, pending)))
    return rc;
  GemmArgs gl{};
  gl.a_codes = w.xq; gl.a_scales = w.xs; gl.m = n_out;
  gl.w_codes = head.codes; gl.w_scales = head.scales; gl.n = head.rows; gl.k = H;
  gl.out = logits_out; gl.ld_out = head.rows;
  gl.split_k = 1;
  return launch_gemm_q8(gl, s);
}

extern "C" int mi_prefill_forward(const mi_model* md, const int32_t* token_ids, const int32_t* positions,
                                  int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv, float* logits_out) {
  return mi_prefill_forward_n(md, token_ids, positions, n_tokens, n_ctx, kv, 1, logits_out);
}

extern "C" int mi_decode_step(const mi_model* md, int32_t token_id, int32_t position, int32_t n_ctx,
                              const mi_kv_regions* kv, float* logits_out) {
  return mi_prefill_forward_n(md, &token_id, &position, 1, n_ctx, kv, 1, logits_out);
}

extern "C" int mi_prefill_forward_n(const mi_model* md, const int32_t* token_ids, const int32_t* positions,
                                    int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv, int32_t n_out,
                                    float* logits_out) {
  int rc = validate_static(md, n_tokens, n_ctx, kv, logits_out, n_out);
  if (rc) return rc;
  int max_pos = 0;
  if ((rc = validate_tokens(md->hp, token_ids, positions, n_tokens, n_ctx, &max_pos))) return rc;
  hipStream_t s = as_stream(md->stream);
  const Ws w = carve(md->hp, md->max_tokens, (char*)md->workspace);
  if ((rc = check_stage(md, w))) return rc;
  if ((rc = stage_tokens(md->stage, w, token_ids, positions, n_tokens, max_pos, s))) return rc;
  return enqueue_forward(md, w, n_tokens, n_ctx, kv, n_out, logits_out, s);
}

// ---------------------------------------------------------------- several sequences in one call
// Rows of all slots go through the matmuls, norms and activations together; the Q|K|V epilogue
// stores each row's K/V into its slot's regions; attention runs per slot over that slot's regions;
// the last layer keeps every row (the tail rows of different slots are not contiguous), and each
// slot's last row goes through the final norm and the lm_head.
// device views of the staging area of a call with several sequences
struct SlotStage {
  const AttnSlotTile* tiles;  // [n_layers][n_tiles]
  float* const* regions;      // [2][n_layers][MI_MAX_SLOTS]
  const int32_t* slot_of_row; // [nt]
  const int32_t* last;        // [n_slots]
  int n_tiles;
};

static int enqueue_slots(const mi_model* md, const Ws& w, const SlotStage& st, int nt, int n_slots,
                         const mi_kv_regions* kv, float* logits_out, hipStream_t s) {
  const mi_hparams& hp = md->hp;
  const int H = hp.hidden, F = hp.ffn;
  const int nq = hp.n_head * hp.head_dim, nkv = hp.n_head_kv * hp.head_dim, nqkv = nq + 2 * nkv;
  const float eps = hp.rms_eps;
  const int L = std::max(hp.n_layers, 1);
  int rc;
  if ((rc = launch_embed(md->token_embd.codes, md->token_embd.scales, H, w.ids, nt, w.h, s))) return rc;
  int pending = 1;
  for (int l = 0; l < hp.n_layers; ++l) {
    const mi_layer_weights& Lw = md->layers[l];
    const bool last = l == hp.n_layers - 1;
    if ((rc = launch_rmsnorm_quant(w.h, Lw.attn_norm, nt, H, eps, w.xq, w.xs, nullptr, s, (const double*)w.gemm_ws,
                                   pending)))
      return rc;
    GemmArgs g{};
    g.a_codes = w.xq; g.a_scales = w.xs; g.m = nt;
    g.w_codes = Lw.wqkv.codes; g.w_scales = Lw.wqkv.scales; g.n = nqkv; g.k = H;
    g.bias = hp.qkv_bias ? Lw.bqkv : nullptr; g.out = w.qkv; g.ld_out = nqkv;
    g.workspace = w.gemm_ws; g.workspace_bytes = w.gemm_ws_bytes;
    g.qkv.pos = w.pos; g.qkv.rope = md->rope_table; g.qkv.n_q = nq; g.qkv.n_kv = nkv; g.qkv.head_dim = hp.head_dim;
    g.qkv.k_region = kv[0].k[l]; g.qkv.v_region = kv[0].v[l];
    g.qkv.slot_of_row = st.slot_of_row;
    g.qkv.k_slots = st.regions + (size_t)l * MI_MAX_SLOTS;
    g.qkv.v_slots = st.regions + ((size_t)L + l) * MI_MAX_SLOTS;
    g.qkv.q_norm = hp.qk_norm ? Lw.q_norm : nullptr; g.qkv.k_norm = hp.qk_norm ? Lw.k_norm : nullptr; g.qkv.eps = eps;
    if ((rc = launch_gemm_q8(g, s))) return rc;
    // one launch for every slot: the query tiles of this layer's table
    if ((rc = launch_attention(w.qkv, nqkv, kv[0].k[l], kv[0].v[l], w.pos, nt, nullptr, 0, hp.n_head, hp.n_head_kv,
                               hp.head_dim, nullptr, nq, s, w.xq, w.xs, st.tiles + (size_t)l * st.n_tiles,
                               st.n_tiles)))
      return rc;
    GemmArgs go{};
    go.a_codes = w.xq; go.a_scales = w.xs; go.m = nt;
    go.w_codes = Lw.wo.codes; go.w_scales = Lw.wo.scales; go.n = H; go.k = nq;
    go.residual = w.h; go.out = w.h; go.ld_out = H;
    go.workspace = w.gemm_ws; go.workspace_bytes = w.gemm_ws_bytes;
    if ((rc = launch_gemm_q8(go, s))) return rc;
    if ((rc = launch_rmsnorm_quant(w.h, Lw.ffn_norm, nt, H, eps, w.xq, w.xs, nullptr, s))) return rc;
    GemmArgs gg{};
    gg.a_codes = w.xq; gg.a_scales = w.xs; gg.m = nt;
    gg.w_codes = Lw.w_gate_up.codes; gg.w_scales = Lw.w_gate_up.scales; gg.n = 2 * F; gg.k = H;
    gg.q_codes = w.sq; gg.q_scales = w.ss;
    gg.workspace = w.gemm_ws; gg.workspace_bytes = w.gemm_ws_bytes;
    if ((rc = launch_gemm_q8(gg, s))) return rc;
    GemmArgs gd{};
    gd.a_codes = w.sq; gd.a_scales = w.ss; gd.m = nt;
    gd.w_codes = Lw.w_down.codes; gd.w_scales = Lw.w_down.scales; gd.n = H; gd.k = F;
    gd.residual = w.h; gd.out = w.h; gd.ld_out = H;
    gd.workspace = w.gemm_ws; gd.workspace_bytes = w.gemm_ws_bytes;
    pending = 1;
    gd.split_out = last ? nullptr : &pending;  // the last layer reduces its own partials
    if ((rc = launch_gemm_q8(gd, s))) return rc;
  }
  // the slots' last rows, gathered; final norm and the lm_head as one matmul over them
  const mi_q8_matrix& head = hp.tied ? md->token_embd : md->output;
  if ((rc = launch_gather_rows(w.h, H, st.last, n_slots, w.slot_h, s))) return rc;
  if ((rc = launch_rmsnorm_quant(w.slot_h, md->output_norm, n_slots, H, eps, w.xq, w.xs, nullptr, s))) return rc;
  if (n_slots == 1) return launch_lm_head(w.xq, w.xs, H, head.codes, head.scales, head.rows, logits_out, s);
  GemmArgs gl{};
  gl.a_codes = w.xq; gl.a_scales = w.xs; gl.m = n_slots;
  gl.w_codes = head.codes; gl.w_scales = head.scales; gl.n = head.rows; gl.k = H;
  gl.out = logits_out; gl.ld_out = head.rows;
  gl.split_k = 1;
  return launch_gemm_q8(gl, s);
}

extern "C" int mi_prefill_forward_slots(const mi_model* md, const int32_t* token_ids, const int32_t* positions,
                                        const int32_t* slot_tokens, int32_t n_slots, int32_t n_ctx,
                                        const mi_kv_regions* kv, float* logits_out) {
  if (!slot_tokens || !kv || n_slots < 1 || n_slots > MI_MAX_SLOTS)
    return set_error(MI_ERR_INVALID_ARG, "forward_slots: 1 <= n_slots <= %d and non-NULL descriptors", MI_MAX_SLOTS);
  int32_t off[MI_MAX_SLOTS], maxpos[MI_MAX_SLOTS];
  int nt = 0;
  for (int sl = 0; sl < n_slots; ++sl) {
    if (slot_tokens[sl] < 1) return set_error(MI_ERR_INVALID_ARG, "forward_slots: slot %d has no tokens", sl);
    off[sl] = nt;
    nt += slot_tokens[sl];
  }
  int rc = validate_static(md, nt, n_ctx, &kv[0], logits_out, 1);
  if (rc) return rc;
  for (int sl = 1; sl < n_slots; ++sl)
    if ((rc = validate_kv(md->hp, &kv[sl], n_ctx))) return rc;
  if ((rc = validate_kv_disjoint(kv, n_slots))) return rc;
  for (int sl = 0; sl < n_slots; ++sl)  // positions: ranges; no repeat within a slot
    if ((rc = validate_tokens(md->hp, token_ids + off[sl], positions + off[sl], slot_tokens[sl], n_ctx, &maxpos[sl])))
      return rc;
  hipStream_t s = as_stream(md->stream);
  const Ws w = carve(md->hp, md->max_tokens, (char*)md->workspace);
  if ((rc = check_stage(md, w))) return rc;
  const int L = std::max(md->hp.n_layers, 1);
  // attention query tiles: up to 16 rows of one slot each
  int n_tiles = 0;
  for (int sl = 0; sl < n_slots; ++sl) n_tiles += (slot_tokens[sl] + 15) / 16;
  if (n_tiles > w.slot_tiles_max) return set_error(MI_ERR_WORKSPACE, "forward_slots: too many attention tiles");
  // the staging area, built on the host in the device layout and sent in one copy
  const size_t o_tiles = 0, o_regions = o_tiles + align_up(sizeof(AttnSlotTile) * (size_t)L * n_tiles),
               o_rows = o_regions + align_up(sizeof(float*) * 2 * (size_t)L * MI_MAX_SLOTS),
               o_last = o_rows + align_up(sizeof(int32_t) * (size_t)nt),
               bytes = o_last + sizeof(int32_t) * MI_MAX_SLOTS;
  if (bytes > w.slot_stage_bytes) return set_error(MI_ERR_WORKSPACE, "forward_slots: staging area too small");
  int32_t mp_all = 0;
  for (int sl = 0; sl < n_slots; ++sl) mp_all = std::max(mp_all, maxpos[sl]);
  // ids, positions, the largest position and the tables, written into the next pinned buffer of the
  // stage in the workspace's layout and sent in one copy
  char* base = reinterpret_cast<char*>(w.ids);
  const size_t o_pos = (char*)w.pos - base, o_max = (char*)w.maxpos - base, o_blob = w.slot_stage - base;
  rc = stage_send(md->stage, base, o_blob + bytes, s, [&](char* h) {
    std::memcpy(h, token_ids, sizeof(int32_t) * nt);
    std::memcpy(h + o_pos, positions, sizeof(int32_t) * nt);
    std::memcpy(h + o_max, &mp_all, sizeof(int32_t));
    char* blob = h + o_blob;
    std::memset(blob, 0, bytes);
    AttnSlotTile* tiles = reinterpret_cast<AttnSlotTile*>(blob + o_tiles);
    float** regions = reinterpret_cast<float**>(blob + o_regions);
    int32_t* slot_of_row = reinterpret_cast<int32_t*>(blob + o_rows);
    int32_t* last = reinterpret_cast<int32_t*>(blob + o_last);
    for (int l = 0; l < md->hp.n_layers; ++l) {
      int i = 0;
      for (int sl = 0; sl < n_slots; ++sl) {
        regions[(size_t)l * MI_MAX_SLOTS + sl] = kv[sl].k[l];
        regions[((size_t)L + l) * MI_MAX_SLOTS + sl] = kv[sl].v[l];
        for (int t = 0; t < slot_tokens[sl]; t += 16)
          tiles[(size_t)l * n_tiles + i++] =
              AttnSlotTile{kv[sl].k[l], kv[sl].v[l], off[sl] + t, std::min(16, slot_tokens[sl] - t), maxpos[sl], 0};
      }
    }
    for (int sl = 0; sl < n_slots; ++sl) {
      for (int t = 0; t < slot_tokens[sl]; ++t) slot_of_row[off[sl] + t] = sl;
      last[sl] = off[sl] + slot_tokens[sl] - 1;
    }
  });
  if (rc) return rc;
  const SlotStage st{reinterpret_cast<const AttnSlotTile*>(w.slot_stage + o_tiles),
                     reinterpret_cast<float* const*>(w.slot_stage + o_regions),
                     reinterpret_cast<const int32_t*>(w.slot_stage + o_rows),
                     reinterpret_cast<const int32_t*>(w.slot_stage + o_last), n_tiles};
  return enqueue_slots(md, w, st, nt, n_slots, kv, logits_out, s);
}

// ---------------------------------------------------------------- graph replay
struct mi_prefill_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipStream_t stream = nullptr;
  mi_stage* stage = nullptr;  // the model's stage: ids and positions of each launch go through it
  mi_hparams hp{};
  Ws w{};
  int32_t n_tokens = 0, n_ctx = 0;
  int32_t max_pos = 0;  // host copy staged to the device on every launch
};

extern "C" int mi_prefill_graph_create(const mi_model* md, int32_t n_tokens, int32_t n_ctx, const mi_kv_regions* kv,
                                       int32_t n_out, float* logits_out, mi_prefill_graph** out) {
  if (!out) return set_error(MI_ERR_INVALID_ARG, "graph: NULL output handle");
  *out = nullptr;
  int rc = validate_static(md, n_tokens, n_ctx, kv, logits_out, n_out);
  if (rc) return rc;
  hipStream_t s = as_stream(md->stream);
  if (!s) return set_error(MI_ERR_INVALID_ARG, "graph: capture needs a non-default stream in model->stream");
  mi_prefill_graph* g = new mi_prefill_graph();
  g->stream = s;
  g->hp = md->hp;
  g->w = carve(md->hp, md->max_tokens, (char*)md->workspace);
  if ((rc = check_stage(md, g->w))) {
    delete g;
    return rc;
  }
  g->stage = md->stage;
  g->n_tokens = n_tokens;
  g->n_ctx = n_ctx;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    delete g;
    return hip_check(e, "hipStreamBeginCapture");
  }
  rc = enqueue_forward(md, g->w, n_tokens, n_ctx, kv, n_out, logits_out, s);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(s, &graph);
  if (rc || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    delete g;
    return rc ? rc : hip_check(e, "hipStreamEndCapture");
  }
  g->graph = graph;
  e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    delete g;
    return hip_check(e, "hipGraphInstantiate");
  }
  *out = g;
  return MI_OK;
}

extern "C" int mi_prefill_graph_launch(mi_prefill_graph* g, const int32_t* token_ids, const int32_t* positions) {
  if (!g || !g->exec) return set_error(MI_ERR_INVALID_ARG, "graph: NULL handle");
  int rc = validate_tokens(g->hp, token_ids, positions, g->n_tokens, g->n_ctx, &g->max_pos);
  if (rc) return rc;
  if ((rc = stage_tokens(g->stage, g->w, token_ids, positions, g->n_tokens, g->max_pos, g->stream))) return rc;
  MI_HIP(hipGraphLaunch(g->exec, g->stream));
  return MI_OK;
}

extern "C" int mi_prefill_graph_nodes(const mi_prefill_graph* g, int32_t* n_nodes) {
  if (!g || !g->graph || !n_nodes) return set_error(MI_ERR_INVALID_ARG, "graph: NULL handle or output");
  size_t n = 0;
  MI_HIP(hipGraphGetNodes(g->graph, nullptr, &n));
  *n_nodes = (int32_t)n;
  return MI_OK;
}

extern "C" void mi_prefill_graph_destroy(mi_prefill_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}
