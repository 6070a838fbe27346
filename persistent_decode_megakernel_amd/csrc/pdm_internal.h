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

// Functions shared by the host planner and the device code.
#if defined(__HIPCC__)
#define PDM_HD __host__ __device__
#else
#define PDM_HD
#endif

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
constexpr int kMaxHeads = 256;        // attention heads
constexpr uint32_t kMagic = 0x57444d50u;  // "PDMW"
constexpr int kHeaderBytes = 256;
constexpr int kTraceWords = 8;        // u64 words per (stage, workgroup) trace record

// Packed FP8 matrix: e4m3 codes [rows][K] row-major, then bf16 scales
// [rows / 8][nkb] with nkb = ceil(K / 128). A scale entry covers 8 packed rows
// by 128 columns; the packer guarantees each such tile lies inside a single
// 128x128 block of the logical matrix.
// A packed weight matrix. FP8 (fmt PDM_FMT_FP8): e4m3 codes [rows][K] and
// bf16 scales [rows / 8][nkb], nkb = ceil(K / 128). MXFP4 (PDM_FMT_MXFP4):
// e2m1 codes [rows][K] bytes (2 elements each) and e8m0 scales [rows][nkb]
// bytes, nkb = K / 16 (one per 32 elements). K is bytes per row in both.
struct Fp8Mat {
  uint64_t codes;
  uint64_t scales;
  int32_t rows;
  int32_t K;
  int32_t nkb;
  int32_t fmt;
};

struct LayerPlan {
  int32_t is_moe;
  int32_t pad0;
  // weights (arena)
  uint64_t attn_norm, q_norm, kv_norm, ffn_norm;  // f32 gains
  Fp8Mat qkv;    // [W_DQ ; W_DKV]                     rows d_q + d_c + d_r, K = D
  Fp8Mat qb;     // W_UQ                               rows H*(d_n+d_r),     K = d_q
  Fp8Mat uk;     // W_UK per head [h][n][c]            rows H*d_n,           K = d_c
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
  uint64_t qlat_part;  // [H][qb_maxparts][d_c]: per-workgroup partials of W_UK[h]^T q_nope[h]
  uint64_t qrope;      // bf16 [n_hg][high, residual][hg][d_r]: rotated rotary queries * tau
  uint64_t attn_part;  // [H][chunks][d_c + 4]: acc, max, sum, 2 zeros (chunks <= nch, chosen per step)
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
constexpr int kStMx = 2;       // the stage's expert matrices are MXFP4

struct Plan {
  pdm_dims dims;
  int32_t G;          // persistent workgroups
  int32_t n_stages;
  int32_t max_ctx;
  int32_t nch;        // most attention position chunks per head group (the count is chosen per step)
  int32_t hg;         // heads per attention unit
  int32_t n_hg;       // head groups
  int32_t qb_gran;    // row-split granularity of the q_b stage
  int32_t qb_maxparts;  // most q_b workgroups holding query rows of one head
  uint64_t embed, final_norm, lm_head;  // arena
  uint64_t rope_tab;                    // scratch: f32 [max_ctx][rope/2][2] (cos, sin)
  uint64_t counters;                    // scratch: int [n_stages + 1][kStripes][kCounterStride]
  uint64_t flags;                       // scratch: u32 [n_stages][G] epoch of each workgroup's last finished stage
  uint64_t status;                      // scratch: u64
  uint64_t lm_best;                     // scratch: [G] x {f32 value, i32 index}
  uint64_t logits_internal;             // scratch: f32 [vocab]
  uint64_t x0;                          // scratch: f32 [D] step input (tap)
  uint64_t trace;                       // trace buffer or 0
  // per head: bit k set when q_b workgroup qb_first(h) + k owns rows (wrote partial slot k)
  uint64_t qb_mask[kMaxHeads];
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

// Balanced contiguous share of `rows` (whole groups of `gran` rows) for
// workgroup wg of G: rows [ra, rb). Requires (rows / gran) * G < 2^31.
// Packed FP8 matrix from a logical one (codes [N][K] row-major, bf16 block
// scales [ceil(N/128)][ceil(K/128)]): packed codes [rows][Kp] (Kp = K) and
// scales [rows / 8][nkb], one per 8 packed rows and 128 columns (the scale of
// the logical block holding that tile's first element). Packed row r takes
// logical row sr (columns unchanged) by mode:
//   0: sr = r - row0 for r in [row0, row0 + N) (row concatenation; the rest
//      of the packed rows come from other tensors)
//   1: W_UK rows out of W_UKV: r = h * dn + n <- h * (dn + dv) + n
//   2: W_UV rows out of W_UKV: r = h * dv + v <- h * (dn + dv) + dn + v
//   3: gate/up interleave in groups of 8: r = 16 i + j <- gate row 8 i + j
//      (j < 8, which = 0) or up row 8 i + (j - 8) (j >= 8, which = 1)
struct PackMap {
  int mode, N, K, rows, Kp, nkb, row0, dn, dv, dc, which;
};
PDM_HD inline bool pack_src(const PackMap& m, int r, int k, int& sr, int& sc) {
  sc = k;
  switch (m.mode) {
    case 0:
      if (r < m.row0 || r >= m.row0 + m.N) return false;
      sr = r - m.row0;
      return true;
    case 1:
      sr = r / m.dn * (m.dn + m.dv) + r % m.dn;
      return true;
    case 2:
      sr = r / m.dv * (m.dn + m.dv) + m.dn + r % m.dv;
      return true;
    default: {
      const int i = r >> 4, j = r & 15;
      if ((j >= 8) != (m.which == 1)) return false;
      sr = 8 * i + (j & 7);
      return true;
    }
  }
}

PDM_HD inline void split_rows(int rows, int gran, int G, int wg, int& ra, int& rb) {
  const int ng = rows / gran;
  ra = ng * wg / G * gran;
  rb = ng * (wg + 1) / G * gran;
}
// The workgroup whose share (split_rows) holds row r, 0 <= r < rows.
// floor(ng * w / G) <= r / gran < floor(ng * (w + 1) / G) solves to
// w = ceil((r / gran + 1) * G / ng) - 1.
PDM_HD inline int split_owner(int rows, int gran, int G, int r) {
  const int ng = rows / gran, g = r / gran;
  return ((g + 1) * G + ng - 1) / ng - 1;
}

// The q_b stage splits the rows of W_UQ ([head][d_n nope ; d_r rotary]) over
// the workgroups; each workgroup also multiplies the nope rows it produced by
// the matching rows of W_UK. Partial `slot` of head h comes from workgroup
// qb_first(h) + slot; there are qb_parts(h) of them.
PDM_HD inline int qb_first(const pdm_dims& d, int gran, int G, int h) {
  return split_owner(d.n_heads * (d.qk_nope + d.rope), gran, G, h * (d.qk_nope + d.rope));
}
PDM_HD inline int qb_parts(const pdm_dims& d, int gran, int G, int h) {
  const int rows = d.n_heads * (d.qk_nope + d.rope);
  return split_owner(rows, gran, G, h * (d.qk_nope + d.rope) + d.qk_nope - 1) - qb_first(d, gran, G, h) + 1;
}
// W_UK rows [u0, u1) (row h * d_n + n) whose q_nope values q_b rows [ra, rb) produce.
PDM_HD inline void qb_nope_rows(const pdm_dims& d, int ra, int rb, int& u0, int& u1) {
  const int qkh = d.qk_nope + d.rope;
  if (ra >= rb) { u0 = u1 = 0; return; }
  const int ha = ra / qkh, ja = ra - ha * qkh, hb = (rb - 1) / qkh, jb = rb - 1 - hb * qkh;
  u0 = ha * d.qk_nope + (ja < d.qk_nope ? ja : d.qk_nope);
  u1 = hb * d.qk_nope + (jb + 1 < d.qk_nope ? jb + 1 : d.qk_nope);
  if (u1 < u0) u1 = u0;
}
inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int64_t v) { int r = 0; while ((int64_t(1) << r) < v) ++r; return r; }

}  // namespace pdm
