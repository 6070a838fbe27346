// Kernel launch interface between the C ABI (api.cpp) and the device code.
#pragma once

#include <hip/hip_runtime.h>

#include "pdm_internal.h"

namespace pdm {

// Per-step arguments of the persistent kernel (passed by value).
// A launch runs n_steps decode steps; step j has epoch epoch + j and
// position pos + j.
struct LaunchArgs {
  uint32_t epoch;        // epoch of the first step (steps since bind); counters target epoch * arrivals
  int32_t token;         // input token of a single step (tokens == null)
  int32_t pos;           // position of the first step's token == cache length
  int32_t spin_limit;    // polls before a dependency wait gives up
  int32_t skip_stage;    // debug: workgroup 0 does not signal this stage (-1 none)
  int32_t n_steps;       // decode steps in this launch (>= 1)
  int32_t greedy;        // step j > 0 takes the argmax of step j - 1 as its token
  int32_t pad;
  const int32_t* tokens; // tokens of the steps (step 0 only when greedy), or null
  const uint16_t* x_in;  // bf16 hidden input of a bare layer stack
  float* logits;         // optional logits output (the last step's)
  int32_t* argmax;       // optional argmax output, one per step
  uint64_t* trace;       // optional trace records (the last step's)
};

// Row/column map of the offline packer (see engine.hip, pack_codes_kernel).

// One persistent launch; expert_format (PDM_FMT_*) picks the kernel instance.
hipError_t launch_engine(const Plan* plan_dev, const LaunchArgs& a, int G, int expert_format, hipStream_t stream,
                         bool cooperative);
hipError_t launch_rope_table(float* tab, int max_ctx, int rope, double base, hipStream_t stream);
hipError_t launch_pack(const uint8_t* src_codes, const uint16_t* src_scales, uint8_t* dst_codes,
                       uint16_t* dst_scales, const PackMap& m, hipStream_t stream);
// Whole-row copy by the pack map (MXFP4 codes or scales): row_bytes per row.
hipError_t launch_pack_rows(const uint8_t* src, uint8_t* dst, const PackMap& m, int row_bytes, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
// ---- batched products (batch.hip)
constexpr int kBatchMax = 16;                    // tokens per batched call (MFMA columns)
constexpr int kMaxExpertsU = 1024;               // routed experts per layer (the dims limit)
constexpr int kMaxUnion = kBatchMax * 16 + 16;   // union slots: B * top_k routed + shared (top_k + n_shared <= 16)

typedef uint32_t bu32x4 __attribute__((ext_vector_type(4)));

// One batched product. base: the matrix (mode 0) or expert block 0 (modes
// 1, 2, slot s at base + u_list[s] * stride); codes_off / scales_off: the
// packed FP8 matrix inside it. xg: the staged activations (whole K slabs;
// mode 2: one run of slabs per slot, xg_slot u32x4 apart). The geometry
// fields are set by batch_gemm_grid.
struct BatchGemm {
  const uint8_t* base;
  uint64_t stride;
  uint64_t codes_off, scales_off;
  int32_t rows, K, nkb, B;
  const int32_t* u_count;  // modes 1, 2: slots in use
  const int32_t* u_list;   // modes 1, 2: expert of each slot
  const bu32x4* xg;
  int64_t xg_slot;
  float* y;                // mode 0, 2: [B][ldy]; mode 1: [slot][B][ldy]
  int32_t ldy;
  int32_t tiles, slabs, groups;  // 16-row tiles, 512-column K slabs, 8-tile row groups
  int32_t spw, splits;           // K slabs per workgroup, K splits per row group
  int32_t fmt;                   // PDM_FMT_FP8 (K code bytes per row), PDM_FMT_MXFP4 (K / 2; nkb = K / 32
                                 // e8m0 scale bytes per row) or kFmtBf16 (2 K bytes, no scales, mode 0);
                                 // K counts columns either way
};
constexpr int kFmtBf16 = 2;      // BatchGemm::fmt of a bf16 matrix (router, LM head)
// Geometry of a launch over n_slots slot matrices (1 for mode 0).
void batch_gemm_grid(BatchGemm& g, int n_slots);
hipError_t launch_batch_gemm(const BatchGemm& g, int mode, int n_slots, hipStream_t st);

// A staging pass: x [B][ldx] over K columns (or, act, the SwiGLU activations
// of every slot in use from gate/up outputs x [slot][B][ldx] with weights
// uw), written to xg over nwin windows (per slot); it also zeroes n0 floats
// at z0 (times *c0 when c0 is set) and n1 floats at z1.
struct BatchStage {
  const float* x;
  const float* uw;
  const int32_t* u_count;
  bu32x4* xg;
  int32_t ldx, B, K, nwin;
  float* z0;
  const int32_t* c0;
  float* z1;
  size_t n0, n1;
  int32_t mx;  // column order of an MXFP4 product (window pairs interleaved)
};
hipError_t launch_batch_stage(const BatchStage& a, bool act, int max_jobs, hipStream_t st);
hipError_t launch_batch_union(const int32_t* idx, const float* wts, int B, int top_k, int E, int n_shared,
                              int* u_count, int* u_list, float* uw, hipStream_t st);
hipError_t launch_batch_dense_slot(int* u_count, int* u_list, float* uw, hipStream_t st);

// ---- per-token kernels of a batched decode step (batch_step.hip)
struct BatchTokens {
  int32_t token[kBatchMax];  // input token of each sequence (vocabulary models)
  int32_t pos[kBatchMax];    // its position == its cache length before the step
};
hipError_t bs_input(const uint16_t* embed, const uint16_t* x_in, const BatchTokens& tk, int B, int D, float* x,
                    hipStream_t st);
hipError_t bs_norm(float* x, const float* add, bool round, const float* gain, float eps, int B, int D, float* h,
                   hipStream_t st);
// rope_tab: the engine's RoPE table, f32 [max_ctx][rope / 2][2] (cos, sin)
hipError_t bs_latent(const float* qkv, int ldq, int dq, int dc, int dr, const float* q_norm, const float* kv_norm,
                     float eps, const float* rope_tab, const BatchTokens& tk, int B, uint16_t* cache,
                     int64_t seq_stride, float* cq, hipStream_t st);
hipError_t bs_absorb(const float* q, const uint8_t* codes, const uint16_t* scales, int nkb, int H, int dn, int dr,
                     int dc, int B, const float* rope_tab, const BatchTokens& tk, float* qlat, float* qpe,
                     hipStream_t st);
constexpr int kAttnChunksMax = 32;  // position chunks per (sequence, head group) of the batched attention
// part: f32 [B][H][kAttnChunksMax][kv_lora + 2] chunk partials. With sel set,
// attention position t of sequence b is cache row sel[b * sel_stride + t]
// (clamped to [0, sel_rows)) and tk.pos[b] + 1 is the number of positions.
hipError_t bs_attn(const float* qlat, const float* qpe, const uint16_t* cache, int64_t seq_stride, int H, int dc,
                   int dr, float tau, const BatchTokens& tk, int B, float* part, float* olat, hipStream_t st,
                   const int32_t* sel = nullptr, int sel_stride = 0, int sel_rows = 0);
// Sparse attention's indexer scores and top-k selection (dsa.hip).
// scores[s] = sum_j w[j] * max(0, q[j] . k[s]); q f32 [HI][dI], w f32 [HI],
// k bf16 [n][dI]; HI a multiple of 16 up to 64, dI a multiple of 32 up to 256.
hipError_t dsa_scores(const float* q, const float* w, const uint16_t* k, int n, int HI, int dI, float* scores,
                      hipStream_t st);
// idx: the min(kk, n) positions of largest score (ties: lower position) in
// ascending order. work: dsa_topk_work_bytes(n) bytes of device scratch (used
// only for lists longer than one workgroup's register-resident size).
size_t dsa_topk_work_bytes(int n);
hipError_t dsa_topk(const float* scores, int n, int kk, int32_t* idx, uint32_t* work, hipStream_t st);
hipError_t bs_uv(const float* olat, const uint8_t* codes, const uint16_t* scales, int nkb, int H, int dv, int dc,
                 int B, float* o, hipStream_t st);
hipError_t bs_bf16_rows(const float* h, const uint16_t* M, int N, int K, int B, float* out, hipStream_t st);
hipError_t bs_topk(const float* logits, int B, int E, int top_k, int32_t* idx, float* wts, hipStream_t st);
constexpr int kArgPartsMax = 64;    // argmax parts per token
// part_v, part_i: [B][kArgPartsMax] scratch
hipError_t bs_argmax(const float* logits, int B, int V, float* part_v, int32_t* part_i, int32_t* out,
                     hipStream_t st);

// Device address of the library's static scratch array on `device`
// (PDM_STATIC_SCRATCH_BYTES), looked up once per device.
hipError_t static_scratch(int device, void** ptr);

}  // namespace pdm
