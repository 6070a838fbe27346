// Batched weight products for gfx950: B decode tokens (1 <= B <= 16) share
// every weight byte.
//
// At batch 1 every weight product of a decode step is a matrix-vector product
// and the persistent engine streams it through the vector ALUs. Batching B
// sequences turns each into a skinny matrix product Y[B][N] = X[B][K] W^T: the
// weight bytes per step stay the same while the useful work grows B-fold,
// which is how the pages trade per-user speed for total throughput (SemiAnalysis
// "Ultra-High Interactivity on NVIDIA GPUs? - TileRT InferenceX", the section
// on next steps: batch 2, 4 and 8). At B = 4 and above the multiply-adds no
// longer fit in the vector ALU time that streaming a weight byte from HBM
// leaves, so these kernels run on the matrix cores instead.
//
// Weights are the engine's packed FP8 matrices, read in place: e4m3 codes
// [rows][K] row-major and bf16 scales [rows / 8][ceil(K / 128)]. One 16 x 16 x
// 32 bf16 MFMA multiplies 16 packed rows by the (up to) 16 token columns:
//   A = weights: lane l (g = l / 16) holds row l % 16, and the 16 code bytes it
//       loads (columns 16 g .. 16 g + 15 of a 64-column window) feed two MFMAs,
//       bytes 0-7 then bytes 8-15. e4m3 values are exact in bf16.
//   B = activations: lane l holds token l % 16 at the same 8 columns, as a bf16
//       high part plus a bf16 residual (two MFMAs), so the product keeps about
//       2^-17 relative accuracy, as fp32 activations would.
//   C: lane l holds rows 4 g .. 4 g + 3 of the tile for token l % 16.
// A scale covers 8 packed rows and 128 columns, so the eight MFMAs of one
// 128-column block accumulate apart and are scaled per lane before they join
// the running sum. MXFP4 expert matrices (codes [rows][K / 2], element 2j in
// the low nibble of byte j, one e8m0 scale per row and 32 columns) take the
// same operand layout: a lane's 16 columns of a window are 8 code bytes under
// one scale, converted straight to bf16 with the scale applied (e2m1 times a
// power of two is exact in bf16), so their MFMAs join the sum unscaled. For
// MXFP4 products the columns of a window pair are interleaved so that one
// 16-byte load of a lane is the 32 columns (one scale block) it needs for
// both windows: window 2p + h, lane group g holds columns 128 p + 32 g + 16 h
// .. + 15 (the activations are staged in the same order). bf16 matrices (the
// router and the LM head, kFmtBf16) need no conversion at all: a lane's 16
// columns of a window are two 16-byte loads, A1 and A2 as they are.
//
// Work split: a workgroup (4 waves) owns 8 row tiles (128 rows) and a run of
// K slabs (8 windows = 512 columns each). Per slab, each wave issues its two
// row tiles' codes (16 KB in flight) before the slab's activations are staged
// in LDS in operand order; the tiles' sums stay in registers across the run
// and are then added into the fp32 output with device-scope atomics (the
// output is zeroed first). The runs of different workgroups therefore sum in
// no fixed order: results agree with a fixed order to fp32 rounding, not bit
// for bit. The host sizes the runs so that a launch has about 1024
// workgroups.
//
// Mixture of experts at batch B ("union of experts"): the tokens' top-k
// choices are merged into one list of distinct experts, each with a weight
// per token (0 for tokens that did not choose it); shared experts join with
// weight 1. Every listed expert's gate/up rows and down rows are then read
// once for all tokens:
//   h[u][b]   = W_gu[u] x[b]                          (row slots: expert u)
//   y[b]     += W_down[u] (w[u][b] silu(gate) * up)   (K slots: expert u)
// The SwiGLU and the routing weight are applied while the down product stages
// its activations, so the intermediate never makes a separate pass.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "engine.h"

namespace pdm {
namespace {

constexpr int kBT = 256;         // threads per workgroup
constexpr int kBWaves = kBT / 64;
constexpr int kSlabW = 8;        // 64-column windows per K slab
constexpr int kGroupT = 8;       // 16-row tiles per workgroup
constexpr int kTilesPerWave = kGroupT / kBWaves;
constexpr uint32_t kBufWord3 = 0x00020000;  // raw buffer descriptor, gfx9
constexpr uint32_t kOob = 0xFFFFFFF0u;      // buffer offset past any matrix: loads 0

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// v = hi + lo: hi the nearest bf16, lo the nearest bf16 of the remainder
__device__ __forceinline__ void split2(float v, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne_bits(v);
  lo = bf16_rne_bits(v - __builtin_bit_cast(float, hi << 16));
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// four e4m3 codes (one dword) -> four bf16 (two dwords), exact: the gfx950
// conversion straight to packed bf16, with a unit scale. (Taking the high
// halves of v_cvt_pk_f32_fp8's two floats instead is miscompiled by this
// hipcc: both halves come from the first float.)
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t& d0, uint32_t& d1) {
  d0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  d1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
// 2^(e - 127) as an fp32 bit pattern (e = 0: the subnormal 2^-127)
__device__ __forceinline__ float e8m0_f32(uint32_t e) { return __builtin_bit_cast(float, e ? e << 23 : 0x00400000u); }
// eight e2m1 codes (one dword, element 2j in the low nibble of byte j) times
// the block scale -> eight bf16 (four dwords), exact
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, float sc, uint32_t& d0, uint32_t& d1, uint32_t& d2,
                                              uint32_t& d3) {
  d0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  d1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  d2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  d3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
}
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace

// Staged activations: for every 64-column window, the B-operand pieces of
// the 64 lanes (hi 0-7, hi 8-15, lo 0-7, lo 8-15: 4 x 64 x 16 bytes), zero
// for tokens >= B and columns >= K, over whole slabs. Written once per
// product by a staging pass, copied into LDS per slab by the product kernel.
constexpr int kWinU4 = 4 * 64;             // u32x4 per window
constexpr int kSlabU4 = kSlabW * kWinU4;   // u32x4 per slab (32 KB)

// first column of a staged piece: window win, lane jl, half (columns 0-7 or
// 8-15 of the lane's 16); MXFP4 products interleave window pairs
__device__ __forceinline__ int stage_col(int win, int jl, int half, int mx) {
  return mx ? (win >> 1) * 128 + (jl >> 4) * 32 + (win & 1) * 16 + half * 8 : win * 64 + (jl >> 4) * 16 + half * 8;
}

__device__ __forceinline__ void stage_piece(u32x4_t* xw, int jl, int half, const float (&v)[8]) {
  uint32_t hb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split2(v[e], hb[e], lb[e]);
  u32x4_t hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = hb[2 * e] | (hb[2 * e + 1] << 16);
    lo[e] = lb[2 * e] | (lb[2 * e + 1] << 16);
  }
  xw[half * 64 + jl] = hi;
  xw[(2 + half) * 64 + jl] = lo;
}

// Zero n0 floats at z0 (times *c0 when c0 is set) and n1 floats at z1: the
// outputs the following product adds into.
__device__ __forceinline__ void zero_outputs(const BatchStage& a) {
  const size_t stride = (size_t)gridDim.x * blockDim.x, t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n0 = a.c0 ? (size_t)*a.c0 * a.n0 : a.n0;
  for (size_t i = t0; i < n0; i += stride) a.z0[i] = 0.f;
  for (size_t i = t0; i < a.n1; i += stride) a.z1[i] = 0.f;
}

// x [B][ldx] (f32) staged for a product over K columns; one thread per
// (window, half, lane), grid-stride.
__global__ void __launch_bounds__(kBT) batch_stage_x_kernel(BatchStage a) {
  zero_outputs(a);
  const int total = a.nwin * 2 * 64;
  for (int j = blockIdx.x * kBT + threadIdx.x; j < total; j += gridDim.x * kBT) {
    const int jl = j & 63, half = (j >> 6) & 1, win = j >> 7;
    const int n = jl & 15, k = stage_col(win, jl, half, a.mx);
    float v[8];
    if (n < a.B && k < a.K) {
      const float* xr = a.x + (size_t)n * a.ldx + k;
      const float4 p = *reinterpret_cast<const float4*>(xr), q = *reinterpret_cast<const float4*>(xr + 4);
      v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w; v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    stage_piece(a.xg + (size_t)win * kWinU4, jl, half, v);
  }
}

// The down product's activations of every expert slot in use:
// w[s][b] * silu(gate) * up from the gate/up outputs h [slot][B][ldx] (in
// every 16 values, 8 gate then 8 up), staged per slot at xg + s * nwin windows.
__global__ void __launch_bounds__(kBT) batch_stage_act_kernel(BatchStage a) {
  zero_outputs(a);
  const int per = a.nwin * 2 * 64, total = *a.u_count * per;
  for (int j = blockIdx.x * kBT + threadIdx.x; j < total; j += gridDim.x * kBT) {
    const int slot = j / per, r = j - slot * per;
    const int jl = r & 63, half = (r >> 6) & 1, win = r >> 7;
    const int n = jl & 15, k = stage_col(win, jl, half, a.mx);
    float v[8];
    if (n < a.B && k < a.K) {
      const float* hr = a.x + ((size_t)slot * a.B + n) * a.ldx + (k >> 3) * 16;
      const float4 g0 = *reinterpret_cast<const float4*>(hr), g1 = *reinterpret_cast<const float4*>(hr + 4);
      const float4 u0 = *reinterpret_cast<const float4*>(hr + 8), u1 = *reinterpret_cast<const float4*>(hr + 12);
      const float wt = a.uw[slot * kBatchMax + n];
      v[0] = wt * silu_f(g0.x) * u0.x; v[1] = wt * silu_f(g0.y) * u0.y;
      v[2] = wt * silu_f(g0.z) * u0.z; v[3] = wt * silu_f(g0.w) * u0.w;
      v[4] = wt * silu_f(g1.x) * u1.x; v[5] = wt * silu_f(g1.y) * u1.y;
      v[6] = wt * silu_f(g1.z) * u1.z; v[7] = wt * silu_f(g1.w) * u1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    stage_piece(a.xg + ((size_t)slot * a.nwin + win) * kWinU4, jl, half, v);
  }
}

// MODE 0: one matrix. MODE 1: row slots, slot s the gate/up matrix of expert
// u_list[s], output y + s * B * ldy ([slot][B][rows]). MODE 2: K slots, slot
// s the down matrix of expert u_list[s], its staged activations at xg + s *
// xg_slot (u32x4). Activations come staged (xg, whole slabs).
template <int MODE, int FMT>  // FMT: PDM_FMT_FP8 or PDM_FMT_MXFP4 codes, or kFmtBf16 weights
__global__ void __launch_bounds__(kBT) batch_gemm_kernel(BatchGemm g) {
  constexpr bool kMx = FMT == PDM_FMT_MXFP4;
  constexpr bool kBf = FMT == kFmtBf16;
  __shared__ u32x4_t xs[kSlabU4];  // [window][piece][lane]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per = g.splits * g.groups;
  const int slot = MODE == 0 ? 0 : (int)blockIdx.x / per;
  if (MODE != 0 && slot >= *g.u_count) return;  // workgroup-uniform
  const int rem = (int)blockIdx.x - slot * per;
  const int split = rem / g.groups, q = rem - split * g.groups;
  const int s0 = split * g.spw, s1 = min(g.slabs, s0 + g.spw);
  const uint8_t* blk = g.base + (MODE == 0 ? 0 : (uint64_t)g.u_list[slot] * g.stride);
  const uint8_t* codes = blk + g.codes_off;
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(blk + g.scales_off);
  const u32x4_t* xg = g.xg + (MODE == 2 ? (size_t)slot * g.xg_slot : 0);
  const int rows = g.rows, K = g.K, B = g.B, nkb = g.nkb, nsc = rows >> 3;
  const int rowb = kBf ? 2 * K : kMx ? K / 2 : K;  // weight bytes per row
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes), 0, (int)((uint64_t)rows * rowb), kBufWord3);
  // MXFP4: e8m0 scale bytes [rows][nkb], nkb = K / 32
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales), 0, kMx ? (int)((uint64_t)rows * nkb) : 0, kBufWord3);
  const int r16 = lane & 15, lg = lane >> 4;
  f32x4 acc[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int s = s0; s < s1; ++s) {
    if (s > s0) __syncthreads();  // every wave is done reading the previous slab's activations
    // ---- the slab's staged activations into LDS (1 KB per instruction, no registers)
    const u32x4_t* src = xg + (size_t)s * kSlabU4;
#pragma unroll
    for (int i = 0; i < kSlabU4 / 64 / kBWaves; ++i) {
      const int piece = (i * kBWaves + w) * 64;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + piece + lane),
                                       (__attribute__((address_space(3))) void*)(xs + piece), 16, 0, 0);
    }
    // ---- this slab's weight codes (and MXFP4 scales) for the wave's row tiles:
    // FP8, one 16-byte load per window; MXFP4, one per window pair (32 columns)
    constexpr int kLd = kMx ? kSlabW / 2 : kBf ? 2 * kSlabW : kSlabW;
    u32x4_t wv[kTilesPerWave][kLd];
    uint32_t ws[kMx ? kTilesPerWave : 1][kMx ? kLd : 1];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int rt = q * kGroupT + w + t * kBWaves;
      const int row = rt * 16 + r16;
#pragma unroll
      for (int i = 0; i < kLd; ++i) {
        if constexpr (kMx) {
          const int k = (s * kLd + i) * 128 + lg * 32;
          const bool in = rt < g.tiles && row < rows && k < K;
          wv[t][i] = __builtin_amdgcn_raw_buffer_load_b128(rc, in ? (uint32_t)(row * rowb + k / 2) : kOob, 0, 0);
          ws[t][i] = __builtin_amdgcn_raw_buffer_load_b8(rs, in ? (uint32_t)(row * nkb + k / 32) : kOob, 0, 0);
        } else if constexpr (kBf) {  // window i / 2, columns 8 (i & 1) .. of the lane's 16
          const int k = (s * kSlabW + (i >> 1)) * 64 + lg * 16 + (i & 1) * 8;
          const bool in = rt < g.tiles && row < rows && k < K;
          wv[t][i] = __builtin_amdgcn_raw_buffer_load_b128(rc, in ? (uint32_t)(row * rowb + 2 * k) : kOob, 0, 0);
        } else {
          const int k = (s * kSlabW + i) * 64 + lg * 16;
          const bool in = rt < g.tiles && row < rows && k < K;
          wv[t][i] = __builtin_amdgcn_raw_buffer_load_b128(rc, in ? (uint32_t)(row * K + k) : kOob, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the copies (and the codes) have landed
    __syncthreads();

    // ---- products of the slab
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int rt = q * kGroupT + w + t * kBWaves;
      if (rt >= g.tiles) break;  // wave-uniform
      const int srow = rt * 2 + (lg >> 1);  // scale row of this lane's 4 output rows
#pragma unroll
      for (int kb = 0; kb < kSlabW / 2; ++kb) {
        const int kbg = s * (kSlabW / 2) + kb;
        if (kbg * 128 >= K) break;  // uniform
        f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const int win = kb * 2 + i2;
          uint32_t p[8];
          if constexpr (kBf) {
            const u32x4_t c0 = wv[t][2 * win], c1 = wv[t][2 * win + 1];
            p[0] = c0[0]; p[1] = c0[1]; p[2] = c0[2]; p[3] = c0[3];
            p[4] = c1[0]; p[5] = c1[1]; p[6] = c1[2]; p[7] = c1[3];
          } else if constexpr (kMx) {  // window pair kb: bytes 8 i2 .. 8 i2 + 7 of its load
            const u32x4_t c = wv[t][kb];
            const float sc4 = e8m0_f32(ws[t][kb]);
            fp4x8_to_bf16(c[2 * i2], sc4, p[0], p[1], p[2], p[3]);
            fp4x8_to_bf16(c[2 * i2 + 1], sc4, p[4], p[5], p[6], p[7]);
          } else {
            const u32x4_t c = wv[t][win];
            fp8x4_to_bf16(c[0], p[0], p[1]);
            fp8x4_to_bf16(c[1], p[2], p[3]);
            fp8x4_to_bf16(c[2], p[4], p[5]);
            fp8x4_to_bf16(c[3], p[6], p[7]);
          }
          const u32x4_t a1 = {p[0], p[1], p[2], p[3]}, a2 = {p[4], p[5], p[6], p[7]};
          const bf16x8 A1 = __builtin_bit_cast(bf16x8, a1), A2 = __builtin_bit_cast(bf16x8, a2);
          const bf16x8 H1 = __builtin_bit_cast(bf16x8, xs[win * kWinU4 + 0 * 64 + lane]);
          const bf16x8 H2 = __builtin_bit_cast(bf16x8, xs[win * kWinU4 + 1 * 64 + lane]);
          const bf16x8 L1 = __builtin_bit_cast(bf16x8, xs[win * kWinU4 + 2 * 64 + lane]);
          const bf16x8 L2 = __builtin_bit_cast(bf16x8, xs[win * kWinU4 + 3 * 64 + lane]);
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, H1, tmp, 0, 0, 0);
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, L1, tmp, 0, 0, 0);
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, H2, tmp, 0, 0, 0);
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, L2, tmp, 0, 0, 0);
        }
        const float sc = kMx || kBf ? 1.f  // (MXFP4: applied in the conversion; bf16: none)
                         : srow < nsc ? __builtin_bit_cast(float, (uint32_t)scales[(size_t)srow * nkb + kbg] << 16)
                                      : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] += sc * tmp[i];
      }
    }
  }

  // ---- this workgroup's K range adds into the output
  const int n = r16;
  if (n < B) {
    float* yb = g.y + (MODE == 1 ? (size_t)slot * B * g.ldy : 0) + (size_t)n * g.ldy;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int rt = q * kGroupT + w + t * kBWaves;
      if (rt >= g.tiles) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + lg * 4 + i;
        if (row < rows) unsafeAtomicAdd(yb + row, acc[t][i]);
      }
    }
  }
}

// Union of the batch's experts (one workgroup). Experts any token chose get
// slots in increasing expert order, then the shared experts (ids E .. E +
// n_shared - 1) with weight 1 for every token. uw[s][b] is the routing weight
// token b gave slot s's expert (0 if it did not choose it). Indices outside
// [0, E) are skipped.
__global__ void __launch_bounds__(kBT) batch_union_kernel(const int32_t* idx, const float* wts, int B, int top_k,
                                                          int E, int n_shared, int* u_count, int* u_list,
                                                          float* uw) {
  __shared__ int slot_of[kMaxExpertsU];
  __shared__ int wsum[kBWaves];
  __shared__ float uws[kMaxUnion * kBatchMax];
  for (int e = threadIdx.x; e < kMaxExpertsU; e += kBT) slot_of[e] = 0;
  for (int i = threadIdx.x; i < kMaxUnion * kBatchMax; i += kBT) uws[i] = 0.f;
  __syncthreads();
  for (int i = threadIdx.x; i < B * top_k; i += kBT) {
    const int e = idx[i];
    if (e >= 0 && e < E) slot_of[e] = 1;
  }
  __syncthreads();
  // exclusive prefix count over experts: thread t owns experts 4t .. 4t + 3
  constexpr int kPer = kMaxExpertsU / kBT;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) cnt += slot_of[threadIdx.x * kPer + j];
  int incl = cnt;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int base = incl - cnt;
  for (int i = 0; i < wv; ++i) base += wsum[i];
  int n_routed = 0;
  for (int i = 0; i < kBWaves; ++i) n_routed += wsum[i];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = threadIdx.x * kPer + j;
    if (slot_of[e]) {
      u_list[base] = e;
      slot_of[e] = base;
      ++base;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B * top_k; i += kBT) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&uws[slot_of[e] * kBatchMax + i / top_k], wts[i]);
  }
  for (int i = threadIdx.x; i < n_shared * kBatchMax; i += kBT) {
    const int s = i / kBatchMax, b = i - s * kBatchMax;
    uws[(n_routed + s) * kBatchMax + b] = b < B ? 1.f : 0.f;
    if (b == 0) u_list[n_routed + s] = E + s;
  }
  __syncthreads();
  const int n_u = n_routed + n_shared;
  for (int i = threadIdx.x; i < n_u * kBatchMax; i += kBT) uw[i] = uws[i];
  if (threadIdx.x == 0) *u_count = n_u;
}

// A dense layer's SwiGLU as a one-slot union: slot 0, weight 1 per token.
__global__ void batch_dense_slot_kernel(int* u_count, int* u_list, float* uw) {
  if (threadIdx.x < kBatchMax) uw[threadIdx.x] = 1.f;
  if (threadIdx.x == 0) { *u_count = 1; u_list[0] = 0; }
}

// Workgroups per launch the K split aims for: 4 per compute unit, enough
// loads in flight to cover HBM latency. Beyond that a workgroup takes more K
// slabs (fewer output atomics) rather than the launch more workgroups.
constexpr int kTargetGroups = 1024;

void batch_gemm_grid(BatchGemm& g, int n_slots) {
  g.tiles = (g.rows + 15) / 16;
  g.slabs = (g.K + kSlabW * 64 - 1) / (kSlabW * 64);
  g.groups = (g.tiles + kGroupT - 1) / kGroupT;
  const int base = std::max(1, n_slots * g.groups);
  const int want = std::min(g.slabs, std::max(1, (kTargetGroups + base - 1) / base));
  g.spw = (g.slabs + want - 1) / want;
  g.splits = (g.slabs + g.spw - 1) / g.spw;
  g.xg_slot = (int64_t)g.slabs * kSlabU4;
}

hipError_t launch_batch_gemm(const BatchGemm& g, int mode, int n_slots, hipStream_t st) {
  const int per = g.splits * g.groups;
  const int grid = per * (mode == 0 ? 1 : n_slots);
  if (grid <= 0) return hipSuccess;
  const bool mx = g.fmt == PDM_FMT_MXFP4;
  if (mode == 0 && g.fmt == kFmtBf16)
    hipLaunchKernelGGL((batch_gemm_kernel<0, kFmtBf16>), dim3(grid), dim3(kBT), 0, st, g);
  else if (mode == 0 && !mx) hipLaunchKernelGGL((batch_gemm_kernel<0, PDM_FMT_FP8>), dim3(grid), dim3(kBT), 0, st, g);
  else if (mode == 0) hipLaunchKernelGGL((batch_gemm_kernel<0, PDM_FMT_MXFP4>), dim3(grid), dim3(kBT), 0, st, g);
  else if (mode == 1 && !mx) hipLaunchKernelGGL((batch_gemm_kernel<1, PDM_FMT_FP8>), dim3(grid), dim3(kBT), 0, st, g);
  else if (mode == 1) hipLaunchKernelGGL((batch_gemm_kernel<1, PDM_FMT_MXFP4>), dim3(grid), dim3(kBT), 0, st, g);
  else if (!mx) hipLaunchKernelGGL((batch_gemm_kernel<2, PDM_FMT_FP8>), dim3(grid), dim3(kBT), 0, st, g);
  else hipLaunchKernelGGL((batch_gemm_kernel<2, PDM_FMT_MXFP4>), dim3(grid), dim3(kBT), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_batch_union(const int32_t* idx, const float* wts, int B, int top_k, int E, int n_shared,
                              int* u_count, int* u_list, float* uw, hipStream_t st) {
  hipLaunchKernelGGL(batch_union_kernel, dim3(1), dim3(kBT), 0, st, idx, wts, B, top_k, E, n_shared, u_count,
                     u_list, uw);
  return hipGetLastError();
}

hipError_t launch_batch_dense_slot(int* u_count, int* u_list, float* uw, hipStream_t st) {
  hipLaunchKernelGGL(batch_dense_slot_kernel, dim3(1), dim3(64), 0, st, u_count, u_list, uw);
  return hipGetLastError();
}

hipError_t launch_batch_stage(const BatchStage& a, bool act, int max_jobs, hipStream_t st) {
  const int blocks = std::max(1, std::min(2048, (max_jobs + kBT - 1) / kBT));
  if (act) hipLaunchKernelGGL(batch_stage_act_kernel, dim3(blocks), dim3(kBT), 0, st, a);
  else hipLaunchKernelGGL(batch_stage_x_kernel, dim3(blocks), dim3(kBT), 0, st, a);
  return hipGetLastError();
}

}  // namespace pdm
