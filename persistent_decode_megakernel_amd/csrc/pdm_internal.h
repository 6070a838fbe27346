// Internal plan structures shared by the host planner and the device engine.
//
// The plan is the compile-time part of the engine: where every packed weight
// matrix, cache and activation lives, and the ordered stage list each
// persistent workgroup walks. It is built once on the host (planner.cpp),
// patched with absolute device addresses at bind time and copied into the
// scratch buffer, where the kernel reads it through scalar loads.
#pragma once

#include <cstdint>

#include "../../include/pdm.h"

namespace pdm {

constexpr int kThreads = 512;         // 8 waves of 64 lanes per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kStripes = 32;          // arrival counters per stage (power of two, < 64)
constexpr int kCounterStride = 32;    // ints between counters (128 B)
constexpr int kRowChunk = 256;        // rows combined per LDS pass
constexpr int kXMax = 32768;          // floats of staged activation per workgroup (128 KB)
constexpr int kMaxSlots = 16;         // expert slots of one MoE stage
constexpr int kMaxStages = PDM_MAX_LAYERS * 12 + 4;
constexpr int kHeadGroup = 16;        // attention heads per work unit (at most)
constexpr int kMaxChunks = 64;        // attention position chunks per head (one per lane when merged)
constexpr uint32_t kMagic = 0x57444d50u;  // "PDMW"
constexpr int kHeaderBytes = 256;
constexpr int kTraceWords = 8;        // u64 words per (stage, workgroup) trace record

// Packed FP8 matrix: e4m3 codes [rows][K] row-major, then bf16 scales
// [rows / 8][nkb] with nkb = ceil(K / 128). A scale entry covers 8 packed rows
// by 128 columns; the packer guarantees each such tile lies inside a single
// 128x128 block of the logical matrix.
struct Fp8Mat {
  uint64_t codes;
  uint64_t scales;
  int32_t rows;
  int32_t K;
  int32_t nkb;
  int32_t pad;
};

struct LayerPlan {
  int32_t is_moe;
  int32_t pad0;
  // weights (arena)
  uint64_t attn_norm, q_norm, kv_norm, ffn_norm;  // f32 gains
  Fp8Mat qkv;    // [W_DQ ; W_DKV]                     rows d_q + d_c + d_r, K = D
  Fp8Mat qb;     // W_UQ                               rows H*(d_n+d_r),     K = d_q
  Fp8Mat ukT;    // W_UK transposed per head [h][c][n] rows H*d_c,           K = d_n
  Fp8Mat uv;     // W_UV per head [h][v][c]            rows H*d_v,           K = d_c
  Fp8Mat wo;     // W_O                                rows D,               K = H*d_v
  Fp8Mat gu;     // dense gate/up, 8-row interleaved   rows 2F,              K = D
  Fp8Mat down;   // dense down                         rows D,               K = F
  uint64_t router;         // bf16 [E][D]
  uint64_t expert_base;    // expert block e at expert_base + e * expert_stride
  uint64_t expert_stride;
  Fp8Mat egu;              // offsets relative to an expert block: gate/up rows 2F_e, K = D
  Fp8Mat edown;            //                                      down rows D, K = F_e
  // latent cache [max_ctx][d_c + d_r] bf16
  uint64_t kv;
  // activations (scratch), f32 unless noted
  uint64_t qkv_raw;    // [d_q + d_c + d_r]
  uint64_t q;          // [H][d_n + d_r], rotary part rotated
  uint64_t ql;         // attention-ready queries: bf16 [n_hg][high, residual][kHeadGroup][d_c + d_r + 8]
  uint64_t attn_part;  // [H][chunks][d_c + 2]: acc, max, sum (chunks <= nch, chosen per step)
  uint64_t o;          // [H * d_v]
  uint64_t xa;         // [D] residual after attention
  uint64_t act;        // [slots * F_e] or [F]: weighted SwiGLU activations
  uint64_t router_logits;  // [E]
  uint64_t xo;         // [D] layer output (bf16 values)
  uint64_t topk_idx;   // int32 [top_k]
  uint64_t topk_w;     // f32 [top_k]
};

struct StagePlan {
  int32_t type;    // PDM_ST_*
  int32_t layer;
  int32_t wait;    // stage index to wait for, -1 none
  int32_t rows;
  int32_t K;
  int32_t gran;    // row-split granularity
  int32_t flags;   // kSt* bits below
  int32_t pad;
};

// StagePlan flags. Consecutive stages of one workgroup share LDS:
constexpr int kStXStaged = 1;  // the input the previous stage staged in LDS is this stage's input

struct Plan {
  pdm_dims dims;
  int32_t G;          // persistent workgroups
  int32_t n_stages;
  int32_t max_ctx;
  int32_t nch;        // most attention position chunks per head group (the count is chosen per step)
  int32_t hg;         // heads per attention unit
  int32_t n_hg;       // head groups
  int32_t pad[2];
  uint64_t embed, final_norm, lm_head;  // arena
  uint64_t rope_tab;                    // scratch: f32 [max_ctx][rope/2][2] (cos, sin)
  uint64_t counters;                    // scratch: int [n_stages + 1][kStripes][kCounterStride]
  uint64_t status;                      // scratch: u64
  uint64_t lm_best;                     // scratch: [G] x {f32 value, i32 index}
  uint64_t logits_internal;             // scratch: f32 [vocab]
  uint64_t x0;                          // scratch: f32 [D] step input (tap)
  uint64_t trace;                       // trace buffer or 0
  LayerPlan layers[PDM_MAX_LAYERS];
  StagePlan stages[kMaxStages];
};

// Byte layout of the three caller-owned buffers.
struct Layout {
  uint64_t weight_bytes = 0, kv_bytes = 0, scratch_bytes = 0, trace_bytes = 0;
  uint64_t plan_off = 0;  // scratch offset of the Plan copy
};

// Host planner (planner.cpp). Offsets in the returned plan are relative to
// the start of their buffer; bind adds the base addresses.
int validate_dims(const pdm_dims& d, int32_t max_ctx);
int build_plan(const pdm_dims& d, int32_t max_ctx, int32_t G, Plan* plan, Layout* lay);
void stage_info(const Plan& p, int s, pdm_stage_info* out);
uint64_t dims_hash(const pdm_dims& d);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int64_t v) { int r = 0; while ((int64_t(1) << r) < v) ++r; return r; }

}  // namespace pdm
