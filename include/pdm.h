/*
 * pdm.h - C ABI of the batch-1 persistent decode engine for MI355X (gfx950).
 *
 * The engine runs one autoregressive decode step of a DeepSeek-V3 style
 * MLA + MoE transformer as a single persistent HIP kernel: one workgroup per
 * compute unit walks a fixed list of stages (GEMV tiles, MLA attention,
 * routing, LM head) and orders them with dependency counters in device
 * memory instead of kernel boundaries. This is the execution model of the
 * TileRT engine kernel (SemiAnalysis, "Ultra-High Interactivity on NVIDIA
 * GPUs? - TileRT InferenceX", section on how TileRT works: the whole decode
 * graph compiled into one persistent kernel, operators split into tile tasks,
 * no per-operator launch), re-designed for one MI355X.
 *
 * Lifecycle (the pages' "What is TileRT" section 6.1 lists prepare resources /
 * run inference / reset sequence / clean up):
 *   pdm_query_sizes -> caller allocates device buffers -> pdm_create ->
 *   pdm_bind -> pdm_load_fp8 / pdm_load_raw (or pdm_load_packed_weights) ->
 *   pdm_reset_cache -> pdm_import_kv -> pdm_decode_step ... -> pdm_destroy.
 *
 * Conventions
 *   - Every function returns PDM_OK (0) or a negative PDM_ERR_* code; no
 *     exception crosses the ABI and nothing aborts.
 *   - All device memory is allocated and owned by the caller. The engine
 *     borrows the bound pointers until pdm_destroy or the next pdm_bind and
 *     never frees them.
 *   - Calls taking a hipStream_t only enqueue work on that stream and return
 *     without waiting, except pdm_sync_status which synchronises the stream.
 *   - One engine serves one sequence; calls on one engine must not overlap.
 *     An engine is not thread-safe; distinct engines are independent.
 *   - Pointers named *_dev are device pointers; every other pointer is host.
 */
#ifndef PDM_H
#define PDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pdm_stream_t; /* a hipStream_t; 0 is the null stream */

#define PDM_MAX_LAYERS 128
#define PDM_ABI_VERSION 1

/* Error codes */
enum {
  PDM_OK = 0,
  PDM_ERR_ARG = -1,      /* null pointer or out-of-range argument */
  PDM_ERR_CONFIG = -2,   /* shape not supported (see pdm_dims) */
  PDM_ERR_DEVICE = -3,   /* no such device, not gfx950, or too few resources */
  PDM_ERR_OOM = -4,      /* host allocation failed */
  PDM_ERR_ALIGN = -5,    /* a bound buffer is not 256-byte aligned */
  PDM_ERR_SIZE = -6,     /* a bound buffer or blob is smaller than required */
  PDM_ERR_FORMAT = -7,   /* packed blob header does not match this engine */
  PDM_ERR_POS = -8,      /* decode position is not the current cache length */
  PDM_ERR_TOKEN = -9,    /* token id outside [0, vocab) or input missing */
  PDM_ERR_CTX = -10,     /* position would exceed max_ctx */
  PDM_ERR_LAUNCH = -11,  /* the HIP runtime rejected a launch or copy */
  PDM_ERR_WATCHDOG = -12,/* a device-side dependency wait exceeded its spin limit */
  PDM_ERR_UNBOUND = -13  /* buffers not bound yet */
};

/*
 * Model shape. Shapes follow the DeepSeek-V3 layout the pages describe
 * ("What is TileRT", section 5.2: MLA attention, 256 routed experts with 8
 * active, hidden 7168, vocabulary 129,280, dense layers then MoE layers).
 * Requirements checked by every call that takes dims:
 *   hidden, q_lora, kv_lora, ffn, moe_ffn are multiples of 64;
 *   qk_nope, rope, v_head are even multiples of 16 with rope <= 64*2;
 *   every FP8 matrix row count is a multiple of 8;
 *   n_heads * kv_lora and n_heads * v_head multiples of 8;
 *   top_k <= n_experts <= 1024, top_k + n_shared <= 16;
 *   vocab == 0 means a bare layer stack whose input is a hidden vector.
 */
typedef struct pdm_dims {
  int32_t hidden;     /* D */
  int32_t n_heads;    /* H */
  int32_t q_lora;     /* d_q */
  int32_t kv_lora;    /* d_c */
  int32_t qk_nope;    /* d_n */
  int32_t rope;       /* d_r */
  int32_t v_head;     /* d_v */
  int32_t ffn;        /* dense SwiGLU intermediate */
  int32_t n_experts;  /* routed experts per MoE layer */
  int32_t moe_ffn;    /* per-expert SwiGLU intermediate */
  int32_t top_k;      /* routed experts per token */
  int32_t n_shared;   /* shared experts per MoE layer */
  int32_t vocab;      /* 0: bare layer stack */
  int32_t n_layers;
  uint8_t layer_moe[PDM_MAX_LAYERS]; /* 0 dense, 1 MoE, per layer in order */
  float rms_eps;      /* RMSNorm epsilon */
  float rope_base;    /* rotary base */
} pdm_dims;

/* Device buffer sizes (bytes) the caller must allocate before pdm_bind. */
typedef struct pdm_sizes {
  uint64_t weight_bytes;   /* packed weight arena (= the packed blob) */
  uint64_t kv_bytes;       /* latent KV cache, n_layers x max_ctx x (kv_lora+rope) bf16 */
  uint64_t scratch_bytes;  /* plan, counters, activations, taps */
  uint64_t trace_bytes;    /* optional per-stage timestamps, 64 B per stage and workgroup */
  uint64_t alignment;      /* required alignment of every buffer (256) */
  int32_t n_stages;        /* stages of one decode step */
  int32_t n_workgroups;    /* persistent workgroups the sizes were computed for */
} pdm_sizes;

/* Weight tensors, in their logical (checkpoint) form. */
enum pdm_tensor {
  PDM_T_EMBED = 0,       /* bf16 [vocab, hidden] (global) */
  PDM_T_FINAL_NORM = 1,  /* f32 [hidden] (global) */
  PDM_T_LM_HEAD = 2,     /* bf16 [vocab, hidden] (global) */
  PDM_T_ATTN_NORM = 3,   /* f32 [hidden] */
  PDM_T_WQ_A = 4,        /* fp8 [q_lora, hidden] */
  PDM_T_Q_NORM = 5,      /* f32 [q_lora] */
  PDM_T_WQ_B = 6,        /* fp8 [n_heads*(qk_nope+rope), q_lora]; per head [nope ; rope] rows */
  PDM_T_WKV_A = 7,       /* fp8 [kv_lora+rope, hidden]; [latent ; rotary key] rows */
  PDM_T_KV_NORM = 8,     /* f32 [kv_lora] */
  PDM_T_WKV_B = 9,       /* fp8 [n_heads*(qk_nope+v_head), kv_lora]; per head [key ; value] rows */
  PDM_T_WO = 10,         /* fp8 [hidden, n_heads*v_head] */
  PDM_T_FFN_NORM = 11,   /* f32 [hidden] */
  PDM_T_W_GATE = 12,     /* fp8 [ffn or moe_ffn, hidden] */
  PDM_T_W_UP = 13,       /* fp8 [ffn or moe_ffn, hidden] */
  PDM_T_W_DOWN = 14,     /* fp8 [hidden, ffn or moe_ffn] */
  PDM_T_ROUTER = 15,     /* bf16 [n_experts, hidden] */
  PDM_T_COUNT = 16
};

/* Device-side status of the last decode step (pdm_sync_status). */
typedef struct pdm_status {
  int32_t code;          /* PDM_OK or PDM_ERR_WATCHDOG */
  int32_t stage;         /* stage whose wait timed out, -1 if none */
  int32_t workgroup;     /* workgroup that timed out first */
  int32_t observed;      /* counter value it observed */
  uint32_t epoch;        /* epoch of the step that set the status */
  int32_t pad[3];
} pdm_status;

/* Device pointers to the last step's taps (views into the scratch buffer). */
typedef struct pdm_taps {
  const float* hidden_dev;       /* [n_layers, hidden] layer outputs (bf16 values) */
  const float* hidden_attn_dev;  /* [n_layers, hidden] residual after attention */
  const int32_t* router_idx_dev; /* [n_layers, top_k]; rows of dense layers unused */
  const float* router_w_dev;     /* [n_layers, top_k] normalised routing weights */
  const float* logits_dev;       /* [vocab] when no logits buffer was passed */
  const uint64_t* trace_dev;     /* [n_stages, n_workgroups, 8] or null when unbound */
  int32_t n_stages, n_workgroups;
  uint32_t epoch;                /* epoch of the last launched step */
} pdm_taps;

/* One stage of the step, for inspection (pdm_describe_plan). */
typedef struct pdm_stage_info {
  int32_t type;          /* PDM_ST_* */
  int32_t layer;         /* -1 for the LM head */
  int32_t wait_stage;    /* stage that must be complete before this one reads inputs, -1 none */
  int32_t rows;          /* output rows (GEMV) or work units (attention) */
  int32_t k;             /* reduction length in elements */
  int32_t reads[4];      /* activation buffer ids read, -1 padded (PDM_BUF_*) */
  int32_t writes[2];     /* activation buffer ids written, -1 padded */
  uint64_t weight_bytes; /* weight + scale bytes one step streams in this stage (active experts only) */
} pdm_stage_info;

enum pdm_stage_type {
  PDM_ST_QKV = 0,      /* [W_DQ ; W_DKV] * RMSNorm(x): query and key/value latents */
  PDM_ST_QB = 1,       /* W_UQ * RMSNorm(c_q), RoPE on the rotary rows; cache row append */
  PDM_ST_ABSORB = 2,   /* q_lat[h] = W_UK[h]^T q_nope[h] */
  PDM_ST_ATTN = 3,     /* split-KV MLA attention partials over the latent cache */
  PDM_ST_UV = 4,       /* merge partials, o[h] = W_UV[h] o_lat[h] */
  PDM_ST_WO = 5,       /* x += W_O o */
  PDM_ST_ROUTER = 6,   /* router logits W_r * RMSNorm(x) */
  PDM_ST_GU = 7,       /* SwiGLU gate/up of the dense FFN */
  PDM_ST_GU_ROUTED = 8,/* top-k routing, SwiGLU gate/up of the shared and the routed experts */
  PDM_ST_DOWN = 9,     /* x += sum of down projections (weighted), bf16 layer output */
  PDM_ST_LM = 10       /* logits = W_lm * RMSNorm(x), argmax */
};

enum pdm_buffer_id {
  PDM_BUF_INPUT = 0, PDM_BUF_QKV = 1, PDM_BUF_Q = 2, PDM_BUF_QLAT = 3, PDM_BUF_ATTN = 4,
  PDM_BUF_O = 5, PDM_BUF_XATTN = 6, PDM_BUF_ROUTER = 7, PDM_BUF_ACT = 8, PDM_BUF_XOUT = 9,
  PDM_BUF_LOGITS = 10, PDM_BUF_KV = 11
};
/* Buffer ids are per layer: id + 16 * layer (the LM head uses layer n_layers). */

typedef struct pdm_engine pdm_engine;

/* Sizes of the device buffers for dims and max_ctx positions, planned for
 * n_workgroups persistent workgroups (0: 256, the MI355X CU count). Pure: no
 * GPU needed. */
int pdm_query_sizes(const pdm_dims* dims, int32_t max_ctx, int32_t n_workgroups, pdm_sizes* out);

/* The stage list of one decode step (the compile-time task DAG). Pure.
 * Writes min(cap, n) entries to out (may be null) and n to *n_out. */
int pdm_describe_plan(const pdm_dims* dims, int32_t max_ctx, int32_t n_workgroups,
                      pdm_stage_info* out, int32_t cap, int32_t* n_out);

/* Create an engine on HIP device `hip_device` (must be gfx950). The number of
 * persistent workgroups is the device's CU count. */
int pdm_create(const pdm_dims* dims, int32_t max_ctx, int hip_device, pdm_engine** out);

/* Sizes for this engine (as pdm_query_sizes with its workgroup count). */
int pdm_get_sizes(const pdm_engine* e, pdm_sizes* out);

/* Bind caller-owned device buffers of at least the queried sizes, 256-byte
 * aligned. trace_dev may be null (no tracing). Writes the packed-blob header
 * into the weight buffer and the stage plan into the scratch buffer
 * (synchronously). Rebinding replaces the previous buffers. */
int pdm_bind(pdm_engine* e, void* weights_dev, uint64_t weight_bytes, void* kv_dev, uint64_t kv_bytes,
             void* scratch_dev, uint64_t scratch_bytes, void* trace_dev, uint64_t trace_bytes);

/* Offline packer for one FP8 matrix: reads its logical form (row-major e4m3
 * codes [N, K] and bf16 block scales [ceil(N/128), ceil(K/128)], device
 * memory) and writes the engine's tile layout into the bound weight arena
 * (the compile-time weight preprocessing of "What is TileRT" section 6.2).
 * layer = -1 for global tensors; expert = -1 for dense FFN / attention,
 * 0..n_experts-1 routed, n_experts + j for shared expert j. */
int pdm_load_fp8(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert,
                 const uint8_t* codes_dev, const uint16_t* scales_dev, pdm_stream_t stream);

/* Copy a bf16 (embedding, LM head, router) or f32 (norm gains) tensor from
 * device memory into the arena. bytes must equal the tensor's size. */
int pdm_load_raw(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert,
                 const void* src_dev, uint64_t bytes, pdm_stream_t stream);

/* Replace the whole weight arena with a previously packed blob (the contents
 * of a weight buffer of an engine with the same dims). The 256-byte header is
 * checked for magic, ABI version and dims. */
int pdm_load_packed_weights(pdm_engine* e, const void* blob, uint64_t bytes, int blob_on_device,
                            pdm_stream_t stream);

/* Start a new sequence: cache length 0 ("What is TileRT" section 6.1, reset). */
int pdm_reset_cache(pdm_engine* e, pdm_stream_t stream);

/* Write n latent rows (bf16, [n, kv_lora + rope], device memory) at positions
 * pos0.. of one layer's cache. Every layer must be imported with the same
 * pos0 and n; the cache length becomes pos0 + n. pos0 must not exceed the
 * current length. */
int pdm_import_kv(pdm_engine* e, int32_t layer, int32_t pos0, int32_t n, const uint16_t* rows_dev,
                  pdm_stream_t stream);

/* Copy n cache rows of one layer out to rows_dev ([n, kv_lora + rope] bf16). */
int pdm_export_kv(const pdm_engine* e, int32_t layer, int32_t pos0, int32_t n, uint16_t* rows_dev,
                  pdm_stream_t stream);

/* Enqueue one decode step: one persistent kernel launch on `stream`.
 * token: input token id (configs with a vocabulary), else ignored;
 * x_in_dev: bf16 [hidden] input of a bare layer stack, else ignored;
 * pos: must equal the cache length and be < max_ctx; the step appends row pos.
 * logits_dev: optional f32 [vocab] output; argmax_dev: optional int32 output
 * (lowest index among equal maxima). Both written before the kernel ends. */
int pdm_decode_step(pdm_engine* e, int32_t token, int32_t pos, const uint16_t* x_in_dev,
                    float* logits_dev, int32_t* argmax_dev, pdm_stream_t stream);

/* Synchronise `stream` and read the device status word. Returns PDM_OK or
 * PDM_ERR_WATCHDOG (details in *out, which may be null). */
int pdm_sync_status(pdm_engine* e, pdm_stream_t stream, pdm_status* out);

int pdm_get_taps(const pdm_engine* e, pdm_taps* out);

/* Current cache length. */
int pdm_cache_length(const pdm_engine* e, int32_t* out);

/* Debug controls: spin_limit > 0 bounds every dependency wait to that many
 * polls (0 restores the default); skip_signal_stage >= 0 makes workgroup 0
 * skip signalling that stage, which must trip the watchdog. */
int pdm_set_debug(pdm_engine* e, int32_t spin_limit, int32_t skip_signal_stage);

/* Record per-stage timestamps (wall clock, 100 MHz on MI355X) of the
 * following steps into the bound trace buffer: on != 0 enables, 0 disables.
 * Requires a trace buffer at bind time. Records: [stage][workgroup] x
 * {entered, dependency satisfied, signalled, epoch, input staged, weights
 * consumed, epilogue done, 0}; a mark a stage does not pass through is 0. */
int pdm_set_trace(pdm_engine* e, int32_t on);

int pdm_destroy(pdm_engine* e);

const char* pdm_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* PDM_H */
