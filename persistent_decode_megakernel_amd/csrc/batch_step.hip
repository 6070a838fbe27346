// The per-token parts of a batched decode step for gfx950: B sequences, each
// at its own position with its own latent cache, step through the layers
// together. The weight products run as batched products (batch.hip: every
// weight byte read once for all B tokens); the kernels here do what is per
// sequence or per token: embedding rows, RMSNorms and residuals, the latent
// norms, RoPE and cache append, the absorbed key projection, MLA attention
// over each sequence's own cache, the per-head value projection, the router
// and top-k, and the LM head's argmax. The layer computation is the batch-1
// step of the pages' DeepSeek-V3 layer ("What is TileRT" section 5.2: MLA
// attention and a routed + shared expert FFN) per token; the batching is the
// next-step benchmark of the SemiAnalysis TileRT page (batch 2, 4 and 8).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "engine.h"

namespace pdm {
namespace {

constexpr int kST = 256;  // threads of most kernels here
typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));
typedef float sf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t su32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bfv(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ __forceinline__ uint16_t bf_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf_round(float v) { return bfv(bf_rne(v)); }

// dst[i] = src(i) for i < n, by the NT threads of the workgroup, 8 loads per
// thread in flight: the loads are unconditional (indices past n repeat the
// last element), so no load waits for the one before it.
template <int NT, class F>
__device__ __forceinline__ void copy_in(float* dst, int n, F src) {
  for (int i0 = 0; i0 < n; i0 += 8 * NT) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src(min(i0 + j * NT + (int)threadIdx.x, n - 1));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * NT + (int)threadIdx.x;
      if (i < n) dst[i] = v[j];
    }
  }
}

// sum over the workgroup (blockDim.x a multiple of 64, <= 1024); red holds 16 floats
__device__ __forceinline__ float wg_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// FP8 weight of a packed matrix (codes [rows][K], bf16 scales [rows / 8][nkb])
__device__ __forceinline__ float fp8w(const uint8_t* codes, const uint16_t* scales, int K, int nkb, int r, int c) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[(size_t)r * K + c], false);
  return f[0] * bfv(scales[(size_t)(r >> 3) * nkb + (c >> 7)]);
}

// rotate the pair (2i, 2i + 1) by pos * base^(-2i / d): tab_row is row pos
// of the engine's RoPE table, (cos, sin) of each pair's angle (computed in
// float64 when the engine was bound)
__device__ __forceinline__ void rope_pair(float& a, float& b, const float* tab_row, int i) {
  const float cs = tab_row[2 * i], sn = tab_row[2 * i + 1];
  const float x = a, y = b;
  a = x * cs - y * sn;
  b = x * sn + y * cs;
}

}  // namespace

// x[b] = embedding row tokens[b] (bf16 -> f32), or the bf16 input rows.
__global__ void __launch_bounds__(kST) bs_input_kernel(const uint16_t* embed, const uint16_t* x_in, BatchTokens tk,
                                                      int D, float* x) {
  const int b = blockIdx.x;
  const uint16_t* src = x_in ? x_in + (size_t)b * D : embed + (size_t)tk.token[b] * D;
  for (int i = threadIdx.x; i < D; i += kST) x[(size_t)b * D + i] = bfv(src[i]);
}

// x[b] += add[b] (if add), rounded to bf16 (if round), then h[b] =
// RMSNorm(x[b]) * gain (if h). D a multiple of 4, rows 16-byte aligned.
constexpr int kNT = 1024;
__global__ void __launch_bounds__(kNT) bs_norm_kernel(float* x, const float* add, int round, const float* gain,
                                                     float eps, int D, float* h) {
  __shared__ float red[16];
  const int b = blockIdx.x, n4 = D / 4;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)b * D);
  const float4* ar = add ? reinterpret_cast<const float4*>(add + (size_t)b * D) : nullptr;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += kNT) {
    float4 v = xr[i];
    if (ar) {
      const float4 a = ar[i];
      v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
    }
    if (round) {
      v.x = bf_round(v.x); v.y = bf_round(v.y); v.z = bf_round(v.z); v.w = bf_round(v.w);
    }
    xr[i] = v;
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  if (!h) return;  // uniform
  const float r = 1.0f / sqrtf(wg_sum(ss, red) / D + eps);
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  float4* h4 = reinterpret_cast<float4*>(h + (size_t)b * D);
  for (int i = threadIdx.x; i < n4; i += kNT) {
    const float4 v = xr[i], g = g4[i];
    h4[i] = make_float4(v.x * r * g.x, v.y * r * g.y, v.z * r * g.z, v.w * r * g.w);
  }
}

// From [c_q ; c_kv ; k_pe] of token b: RMSNorm(c_q) * q_norm for the query
// product, and the new cache row [RMSNorm(c_kv) * kv_norm ; RoPE(k_pe)]
// rounded to bf16 at position pos[b] of sequence b's cache of this layer.
__global__ void __launch_bounds__(kST) bs_latent_kernel(const float* qkv, int ldq, int dq, int dc, int dr,
                                                       const float* q_norm, const float* kv_norm, float eps,
                                                       const float* rope_tab, BatchTokens tk, uint16_t* cache,
                                                       int64_t seq_stride, float* cq) {
  __shared__ float red[16];
  const int b = blockIdx.x;
  const float* in = qkv + (size_t)b * ldq;
  float s1 = 0.f, s2 = 0.f;
  for (int i = threadIdx.x; i < dq; i += kST) s1 += in[i] * in[i];
  for (int i = threadIdx.x; i < dc; i += kST) s2 += in[dq + i] * in[dq + i];
  const float r1 = 1.0f / sqrtf(wg_sum(s1, red) / dq + eps);
  const float r2 = 1.0f / sqrtf(wg_sum(s2, red) / dc + eps);
  for (int i = threadIdx.x; i < dq; i += kST) cq[(size_t)b * dq + i] = in[i] * r1 * q_norm[i];
  uint16_t* row = cache + (size_t)b * seq_stride + (size_t)tk.pos[b] * (dc + dr);
  for (int i = threadIdx.x; i < dc; i += kST) row[i] = bf_rne(in[dq + i] * r2 * kv_norm[i]);
  for (int i = threadIdx.x; i < dr / 2; i += kST) {
    float a = in[dq + dc + 2 * i], c = in[dq + dc + 2 * i + 1];
    rope_pair(a, c, rope_tab + (size_t)tk.pos[b] * dr, i);
    row[dc + 2 * i] = bf_rne(a);
    row[dc + 2 * i + 1] = bf_rne(c);
  }
}

// Head h: q_lat[b][h][c] = sum_n W_UK[h * dn + n][c] * q_nope[b][h][n] (the
// key projection folded into the query) and the rotated rotary query
// q_pe[b][h] = RoPE(q[b][h][dn ..], pos[b]). q: [B][H][dn + dr]. A workgroup
// takes the columns of one column part (256 columns, or all of a narrower
// latent) of one head: thread t handles 4 columns (t mod column threads) of
// one group of rows (t / column threads), with every row's codes and scale of
// its group loaded at once (one memory round trip), and the groups' sums meet
// in LDS.
constexpr int kAbT = 512;     // threads per absorb workgroup
constexpr int kAbRows = 32;   // rows per thread and load batch
__host__ __device__ __forceinline__ int ab_col_parts(int dc) { return dc >= 256 ? dc / 256 : 1; }
__global__ void __launch_bounds__(kAbT) bs_absorb_kernel(const float* q, const uint8_t* codes, const uint16_t* scales,
                                                        int nkb, int H, int dn, int dr, int dc, int B,
                                                        const float* rope_tab, BatchTokens tk, float* qlat, float* qpe) {
  extern __shared__ float ab_lds[];  // q_nope [B][dn], column sums [B][wcols]
  const int cps = ab_col_parts(dc), h = blockIdx.x / cps, cpart = blockIdx.x % cps, qkh = dn + dr;
  const int wcols = dc / cps, nct = wcols / 4, ng = kAbT / nct;
  const int ct = threadIdx.x % nct, rg = threadIdx.x / nct;
  float* qn = ab_lds;
  float* red = ab_lds + B * dn;
  const int rpg = (dn + ng - 1) / ng, n_beg = min(dn, rg * rpg), n_end = min(dn, n_beg + rpg);
  const int c0 = cpart * wcols + ct * 4;
  // the group's codes and scales first: they do not depend on the queries
  uint32_t cw[kAbRows];
  float sc[kAbRows];
#pragma unroll
  for (int i = 0; i < kAbRows; ++i) {  // unconditional loads (past the group: its first row, unused)
    const int n = n_beg + i;
    const int r = h * dn + (n < n_end ? n : min(n_beg, dn - 1));
    cw[i] = *reinterpret_cast<const uint32_t*>(codes + (size_t)r * dc + c0);
    sc[i] = bfv(scales[(size_t)(r >> 3) * nkb + (c0 >> 7)]);
  }
  copy_in<kAbT>(qn, B * dn, [&](int i) { return q[((size_t)(i / dn) * H + h) * qkh + i % dn]; });
  for (int i = threadIdx.x; i < B * wcols; i += kAbT) red[i] = 0.f;
  if (cpart == 0) {
    for (int i = threadIdx.x; i < B * dr / 2; i += kAbT) {
      const int b = i / (dr / 2), j = i % (dr / 2);
      const float* src = q + ((size_t)b * H + h) * qkh + dn;
      float a = src[2 * j], c = src[2 * j + 1];
      rope_pair(a, c, rope_tab + (size_t)tk.pos[b] * dr, j);
      qpe[((size_t)b * H + h) * dr + 2 * j] = a;
      qpe[((size_t)b * H + h) * dr + 2 * j + 1] = c;
    }
  }
  __syncthreads();
  float acc[4][kBatchMax];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int b = 0; b < kBatchMax; ++b) acc[e][b] = 0.f;
  for (int n0 = n_beg; n0 < n_end; n0 += kAbRows) {
    if (n0 > n_beg) {  // rows past the first batch (a row group longer than kAbRows)
#pragma unroll
      for (int i = 0; i < kAbRows; ++i) {
        const int n = n0 + i;
        const int r = h * dn + (n < n_end ? n : n0);
        cw[i] = *reinterpret_cast<const uint32_t*>(codes + (size_t)r * dc + c0);
        sc[i] = bfv(scales[(size_t)(r >> 3) * nkb + (c0 >> 7)]);
      }
    }
#pragma unroll
    for (int i = 0; i < kAbRows; ++i) {
      if (n0 + i < n_end) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i], true);
        const float wv[4] = {lo[0] * sc[i], lo[1] * sc[i], hi[0] * sc[i], hi[1] * sc[i]};
#pragma unroll
        for (int b = 0; b < kBatchMax; ++b) {
          if (b < B) {
            const float qv = qn[b * dn + n0 + i];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e][b] = fmaf(wv[e], qv, acc[e][b]);
          }
        }
      }
    }
  }
  if (n_beg < n_end) {
#pragma unroll
    for (int b = 0; b < kBatchMax; ++b) {
      if (b < B) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_fetch_add(&red[b * wcols + ct * 4 + e], acc[e][b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B * wcols; i += kAbT)
    qlat[((size_t)(i / wcols) * H + h) * dc + cpart * wcols + i % wcols] = red[i];
}

// MLA attention of sequence b over its cache positions 0 .. pos[b] for a group
// of 16 heads (one workgroup of 8 waves): scores S[t][h] = tau * ([q_lat ;
// q_pe][h] . row t) and values O[h] = sum_t softmax(S)[t][h] * c_t on the
// matrix cores (v_mfma_f32_16x16x32_bf16: cache rows are bf16 already, the
// fp32 queries and probabilities enter as a bf16 high part plus a bf16
// residual), online softmax over blocks of 64 positions. Operand layout
// (lane l, g = l / 16): A holds A[l % 16][8 g .. 8 g + 7], B holds B[8 g ..
// 8 g + 7][l % 16], C holds C[4 g .. 4 g + 3][l % 16]. Scores: waves 0-3
// take the block's four 16-position tiles over the first half of the latent
// k-blocks, waves 4-7 the same tiles over the second half (two partial score
// arrays, added by the softmax); values: wave w takes NT / 2 tiles of 16
// latent dims.
constexpr int kBlk = 64;
constexpr int kAT = 512;                                    // threads of an attention workgroup
constexpr int kAtMaxRow = 640;                              // kv_lora + rope, at most 512 + 128
constexpr int kAtLd = (kBlk * (kAtMaxRow / 8) + kAT - 1) / kAT;  // 16-byte cache pieces per thread and block
constexpr int kAtQ = (16 * kAtMaxRow + kAT - 1) / kAT;           // query values per thread
// SP: sparse attention over a position list. Attention position t of
// sequence b is then cache row sel[b * sel_stride + t] (clamped to
// [0, sel_rows)), and tk.pos[b] + 1 is the list's length.
template <int NT, bool SP>  // NT: value tiles of 16 latent dims per pair of waves: dc / 64 (2, 4 or 8)
__global__ void __launch_bounds__(kAT) bs_attn_kernel(const float* qlat, const float* qpe, const uint16_t* cache,
                                                     int64_t seq_stride, int H, int dc, int dr, float tau,
                                                     BatchTokens tk, int nch, int chunk, float* part,
                                                     const int32_t* sel, int sel_stride, int sel_rows) {
  static_assert(NT % 2 == 0, "value tiles split over two waves");
  constexpr int kVT = NT / 2;  // value tiles per wave
  extern __shared__ __align__(16) unsigned char lds[];
  const int kvr = dc + dr, rs = kvr + 8;  // cache-row stride in LDS (bf16), padded
  const int ngrp = (H + 15) / 16;
  const int ch = blockIdx.x % nch, bh = blockIdx.x / nch;
  const int b = bh / ngrp, hg = bh % ngrp, h0 = hg * 16;
  const int ctx = tk.pos[b] + 1, t0 = ch * chunk, t1 = min(ctx, t0 + chunk);
  if (t0 >= ctx) return;  // no positions in this chunk for this sequence (workgroup-uniform)
  __bf16* qh = reinterpret_cast<__bf16*>(lds);                 // [16][rs]
  __bf16* ql = qh + 16 * rs;                                   // [16][rs]
  uint16_t* kv = reinterpret_cast<uint16_t*>(ql + 16 * rs);    // [kBlk][rs]
  float* S = reinterpret_cast<float*>(kv + kBlk * rs);         // [2][16][kBlk] score partials
  float* hm = S + 2 * 16 * kBlk;                               // running max, sum, rescale per head
  float* hl = hm + 16;
  float* ha = hl + 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
  const uint16_t* seq = cache + (size_t)b * seq_stride;
  const int q8 = kvr / 8;  // 16-byte pieces per row
  // A block's cache rows: every piece a thread copies is loaded at once into
  // registers (one memory round trip), then stored to LDS. The loads are
  // unconditional (pieces past the block read its first row and are zeroed
  // when stored): no branch around them, so none waits for another.
  su32x4 kvr_regs[kAtLd];
  auto load_block = [&](int tb) {
    const int nb = min(kBlk, t1 - tb);
#pragma unroll
    for (int j = 0; j < kAtLd; ++j) {
      const int i = (int)threadIdx.x + j * kAT, r = i / q8, p = i - r * q8;
      const bool ok = i < kBlk * q8 && r < nb;
      const int t = tb + (ok ? r : 0);
      const int row = SP ? min(max(sel[(size_t)b * sel_stride + t], 0), sel_rows - 1) : t;
      kvr_regs[j] = *reinterpret_cast<const su32x4*>(seq + (size_t)row * kvr + (ok ? p : 0) * 8);
    }
  };
  load_block(t0);
  // queries of the group, scaled by tau, split hi / lo (heads past H are zero):
  // all of a thread's values are loaded before any is stored
  {
    float qv[kAtQ];
#pragma unroll
    for (int j = 0; j < kAtQ; ++j) {
      const int i = (int)threadIdx.x + j * kAT, hh = i / kvr, d = i - hh * kvr, hd = h0 + hh;
      const bool ok = i < 16 * kvr && hd < H;
      const int hq = ok ? hd : h0, dq = ok ? d : 0;
      const float* src = dq < dc ? qlat + ((size_t)b * H + hq) * dc + dq : qpe + ((size_t)b * H + hq) * dr + dq - dc;
      qv[j] = *src;
    }
#pragma unroll
    for (int j = 0; j < kAtQ; ++j) {
      const int i = (int)threadIdx.x + j * kAT, hh = i / kvr, d = i - hh * kvr;
      if (i < 16 * kvr) {
        const float v = h0 + hh < H ? tau * qv[j] : 0.f, hi = bf_round(v);
        qh[hh * rs + d] = __builtin_bit_cast(__bf16, bf_rne(v));
        ql[hh * rs + d] = __builtin_bit_cast(__bf16, bf_rne(v - hi));
      }
    }
  }
  if (threadIdx.x < 16) { hm[threadIdx.x] = -INFINITY; hl[threadIdx.x] = 0.f; }
  sf32x4 acc[kVT];
#pragma unroll
  for (int i = 0; i < kVT; ++i) acc[i] = (sf32x4){0.f, 0.f, 0.f, 0.f};
  const int nkb = kvr / 32;  // MFMA k-blocks of a score
  for (int tb = t0; tb < t1; tb += kBlk) {
    const int nb = min(kBlk, t1 - tb);
    if (tb > t0) load_block(tb);
    __syncthreads();  // previous block's rows and probabilities are consumed
#pragma unroll
    for (int j = 0; j < kAtLd; ++j) {
      const int i = (int)threadIdx.x + j * kAT, r = i / q8, p = i - r * q8;
      if (i < kBlk * q8)
        *reinterpret_cast<su32x4*>(kv + r * rs + p * 8) = r < nb ? kvr_regs[j] : (su32x4){0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // scores: wave w takes positions 16 (w & 3) .. + 15 over half (w >> 2) of the k-blocks
    {
      const int tile = w & 3, half = w >> 2;
      const int kb0 = half ? nkb / 2 : 0, kb1 = half ? nkb : nkb / 2;
      sf32x4 sc = {0.f, 0.f, 0.f, 0.f};
      if (16 * tile < nb) {
        for (int kb = kb0; kb < kb1; ++kb) {
          const sbf16x8 a = *reinterpret_cast<const sbf16x8*>(kv + (16 * tile + lr) * rs + kb * 32 + lg * 8);
          const sbf16x8 b1 = *reinterpret_cast<const sbf16x8*>(qh + lr * rs + kb * 32 + lg * 8);
          const sbf16x8 b2 = *reinterpret_cast<const sbf16x8*>(ql + lr * rs + kb * 32 + lg * 8);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, sc, 0, 0, 0);
        }
      }
      // sc[i] = partial S[position 16 tile + 4 lg + i][head lr]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tile + 4 * lg + i;
        S[(half * 16 + lr) * kBlk + t] = sc[i];
      }
    }
    __syncthreads();
    // online softmax: 32 threads per head, 2 positions each; the probabilities
    // replace the first score partial
    {
      const int hh = threadIdx.x >> 5, sub = threadIdx.x & 31;
      float* s0 = S + hh * kBlk + sub * 2;
      const float* s1 = S + (16 + hh) * kBlk + sub * 2;
      const float v0 = sub * 2 < nb ? s0[0] + s1[0] : -INFINITY;
      const float v1 = sub * 2 + 1 < nb ? s0[1] + s1[1] : -INFINITY;
      float mx = fmaxf(v0, v1);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
      const float mold = hm[hh], mn = fmaxf(mold, mx);
      const float p0 = v0 == -INFINITY ? 0.f : __expf(v0 - mn), p1 = v1 == -INFINITY ? 0.f : __expf(v1 - mn);
      s0[0] = p0;
      s0[1] = p1;
      float ps = p0 + p1;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) ps += __shfl_xor(ps, o, 32);
      __syncthreads();  // every thread has read hm before it changes
      if (sub == 0) {
        const float alpha = mold == -INFINITY ? 0.f : __expf(mold - mn);
        ha[hh] = alpha;
        hl[hh] = hl[hh] * alpha + ps;
        hm[hh] = mn;
      }
    }
    __syncthreads();
    // values: wave w takes dims [w * kVT * 16, (w + 1) * kVT * 16)
#pragma unroll
    for (int i = 0; i < kVT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] *= ha[4 * lg + r];
    for (int pb = 0; pb < kBlk / 32; ++pb) {
      if (pb * 32 >= nb) break;  // uniform
      const float* prow = S + lr * kBlk + pb * 32 + 8 * lg;
      sbf16x8 ah, al;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = prow[e], hi = bf_round(v);
        ah[e] = __builtin_bit_cast(__bf16, bf_rne(v));
        al[e] = __builtin_bit_cast(__bf16, bf_rne(v - hi));
      }
      // B of tile i = V[pb*32 + 8*lg + e][dim w*kVT*16 + kVT*lr + i]: a lane's
      // kVT dims of one row are adjacent and come in one LDS read
      const uint16_t* vrow = kv + (pb * 32 + 8 * lg) * rs + w * kVT * 16 + kVT * lr;
      uint32_t vw[8][(kVT + 1) / 2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (kVT == 4) {
          const uint2 t = *reinterpret_cast<const uint2*>(vrow + e * rs);
          vw[e][0] = t.x;
          vw[e][1] = t.y;
        } else if constexpr (kVT == 2) {
          vw[e][0] = *reinterpret_cast<const uint32_t*>(vrow + e * rs);
        } else {
          vw[e][0] = vrow[e * rs];
        }
      }
#pragma unroll
      for (int i = 0; i < kVT; ++i) {
        su32x4 bu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = vw[2 * k][i / 2], hi = vw[2 * k + 1][i / 2];
          bu[k] = (i & 1) ? (lo >> 16) | (hi & 0xffff0000u) : (lo & 0xffffu) | (hi << 16);
        }
        const sbf16x8 bv = __builtin_bit_cast(sbf16x8, bu);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc[i], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  // the chunk's partial per head: [acc (dc) ; max ; sum] at part[b][h][ch];
  // acc[i][r] = O[head 4 lg + r][dim w kVT 16 + kVT lr + i]
  const int ps = dc + 2;
#pragma unroll
  for (int i = 0; i < kVT; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = h0 + 4 * lg + r;
      if (hd < H) part[(((size_t)b * H + hd) * nch + ch) * ps + w * kVT * 16 + kVT * lr + i] = acc[i][r];
    }
  }
  if (threadIdx.x < 16 && h0 + (int)threadIdx.x < H) {
    float* pm = part + (((size_t)b * H + h0 + threadIdx.x) * nch + ch) * ps + dc;
    pm[0] = hm[threadIdx.x];
    pm[1] = hl[threadIdx.x];
  }
}

// Merge of sequence b's chunk partials for head h: o_lat = sum_i acc_i
// e^(m_i - m) / sum_i l_i e^(m_i - m), m the largest m_i. One wave reduces
// the chunks' (m_i, l_i) (one chunk per lane), then every thread adds its
// columns over the chunks.
__global__ void __launch_bounds__(kST) bs_attn_merge_kernel(const float* part, int H, int dc, int nch, int chunk,
                                                           BatchTokens tk, float* olat) {
  static_assert(kAttnChunksMax <= 64, "one lane per chunk");
  __shared__ float wch[kAttnChunksMax];
  __shared__ float linv;
  const int b = blockIdx.x / H, h = blockIdx.x % H, ps = dc + 2;
  const int n = (tk.pos[b] + 1 + chunk - 1) / chunk;  // chunks with positions (<= nch <= 64)
  const float* pb = part + ((size_t)b * H + h) * nch * ps;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const float mi = lane < n ? pb[lane * ps + dc] : -INFINITY;
    const float li = lane < n ? pb[lane * ps + dc + 1] : 0.f;
    float m = mi;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float wi = lane < n ? __expf(mi - m) : 0.f;
    float l = li * wi;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane < n) wch[lane] = wi;
    if (lane == 0) linv = 1.0f / l;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < dc; c += kST) {
    float v[kAttnChunksMax];
#pragma unroll
    for (int i = 0; i < kAttnChunksMax; ++i) v[i] = pb[min(i, n - 1) * ps + c];  // unconditional loads
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < kAttnChunksMax; ++i)
      if (i < n) o += v[i] * wch[i];
    olat[((size_t)b * H + h) * dc + c] = o * linv;
  }
}

// Head h: o[b][h * dv + v] = sum_c W_UV[h * dv + v][c] * o_lat[b][h][c]. A
// workgroup takes 32 rows of one head (all of a narrower head), each of its 4
// waves a quarter of them: a row's codes are 16-byte loads of dc / 16 lanes,
// so one wave load covers 64 / (dc / 16) rows, and all of a wave's loads are
// issued at once (one memory round trip). A row's per-token sums are added
// across its lanes.
constexpr int kUvRows = 32;  // rows per workgroup
constexpr int kUvLd = 4;     // wave loads of codes: rows per wave (<= 8) / rows per load (>= 2)
__host__ __device__ __forceinline__ int uv_row_parts(int dv) { return dv > kUvRows ? dv / kUvRows : 1; }
__global__ void __launch_bounds__(kST) bs_uv_kernel(const float* olat, const uint8_t* codes, const uint16_t* scales,
                                                   int nkb, int H, int dv, int dc, int B, float* o) {
  extern __shared__ float ol[];  // [B][dc]
  const int rps = uv_row_parts(dv), h = blockIdx.x / rps, part = blockIdx.x % rps;
  const int rw = dv / rps, rpw = rw / (kST / 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lpr = dc / 16, rpl = 64 / lpr, sub = lane / lpr, cl = lane % lpr, c0 = cl * 16;
  const int r_w = h * dv + part * rw + w * rpw;  // first row of this wave
  bu32x4 wv[kUvLd];
  float sc[kUvLd];
#pragma unroll
  for (int j = 0; j < kUvLd; ++j) {
    // unconditional loads: rows past the wave's read its first row, unused
    const int ro = j * rpl + sub;
    const int r = r_w + (ro < rpw ? ro : 0);
    wv[j] = *reinterpret_cast<const bu32x4*>(codes + (size_t)r * dc + c0);
    sc[j] = bfv(scales[(size_t)(r >> 3) * nkb + (c0 >> 7)]);
  }
  copy_in<kST>(ol, B * dc, [&](int i) { return olat[((size_t)(i / dc) * H + h) * dc + i % dc]; });
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kUvLd; ++j) {
    if (j * rpl >= rpw) break;  // wave-uniform
    const int ro = j * rpl + sub;
    float f[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[j][e], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[j][e], true);
      f[4 * e + 0] = lo[0] * sc[j];
      f[4 * e + 1] = lo[1] * sc[j];
      f[4 * e + 2] = hi[0] * sc[j];
      f[4 * e + 3] = hi[1] * sc[j];
    }
#pragma unroll
    for (int b = 0; b < kBatchMax; ++b) {
      if (b < B) {
        const float4* x4 = reinterpret_cast<const float4*>(ol + b * dc + c0);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 x = x4[e];
          d = fmaf(f[4 * e + 0], x.x, d);
          d = fmaf(f[4 * e + 1], x.y, d);
          d = fmaf(f[4 * e + 2], x.z, d);
          d = fmaf(f[4 * e + 3], x.w, d);
        }
        for (int off = lpr / 2; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
        if (cl == 0 && ro < rpw) o[(size_t)b * H * dv + r_w + ro] = d;
      }
    }
  }
}

// out[b][r] = sum_k M[r][k] * h[b][k] for a bf16 matrix M [N][K] (router, LM
// head): one wave per kBrR consecutive rows, 16-byte loads of 8 values, K a
// multiple of 8. A lane's loads of kBrP pieces of each of its rows go out
// together, and every activation piece it loads serves all kBrR rows. BM (a
// power of two >= B) bounds the tokens: activations are loaded 4 tokens at a
// time, unconditionally (tokens past B repeat token B - 1, unused), so the
// loads of a group do not wait for each other.
constexpr int kBrR = 4;  // rows per wave
constexpr int kBrP = 4;  // 16-byte pieces per lane and row in flight
template <int BM>
__global__ void __launch_bounds__(kST) bs_bf16_rows_kernel(const float* h, const uint16_t* M, int N, int K, int B,
                                                          float* out) {
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * (kST / 64) + (threadIdx.x >> 6)) * kBrR;
  if (r0 >= N) return;  // wave-uniform
  const int np = K / 8;
  float acc[kBrR][BM];
#pragma unroll
  for (int rr = 0; rr < kBrR; ++rr)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[rr][b] = 0.f;
  for (int p0 = 0; p0 < np; p0 += 64 * kBrP) {
    su32x4 v[kBrR][kBrP];
#pragma unroll
    for (int rr = 0; rr < kBrR; ++rr) {
      const int r = min(r0 + rr, N - 1);
#pragma unroll
      for (int j = 0; j < kBrP; ++j) {
        const int k8 = min(p0 + 64 * j + lane, np - 1);  // unconditional; pieces past the row unused
        v[rr][j] = *reinterpret_cast<const su32x4*>(M + (size_t)r * K + (size_t)k8 * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kBrP; ++j) {
      const int k8 = min(p0 + 64 * j + lane, np - 1);
      const bool kin = p0 + 64 * j + lane < np;
      float m[kBrR][8];
#pragma unroll
      for (int rr = 0; rr < kBrR; ++rr)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          m[rr][2 * e] = kin ? __builtin_bit_cast(float, v[rr][j][e] << 16) : 0.f;
          m[rr][2 * e + 1] = kin ? __builtin_bit_cast(float, v[rr][j][e] & 0xFFFF0000u) : 0.f;
        }
#pragma unroll
      for (int b0 = 0; b0 < BM; b0 += 4) {
        float4 x[4][2];
#pragma unroll
        for (int i = 0; i < 4 && b0 + i < BM; ++i) {
          const int bb = min(b0 + i, B - 1);
          x[i][0] = *reinterpret_cast<const float4*>(h + (size_t)bb * K + k8 * 8);
          x[i][1] = *reinterpret_cast<const float4*>(h + (size_t)bb * K + k8 * 8 + 4);
        }
#pragma unroll
        for (int i = 0; i < 4 && b0 + i < BM; ++i) {
          const float4 x0 = x[i][0], x1 = x[i][1];
#pragma unroll
          for (int rr = 0; rr < kBrR; ++rr)
            acc[rr][b0 + i] += m[rr][0] * x0.x + m[rr][1] * x0.y + m[rr][2] * x0.z + m[rr][3] * x0.w +
                               m[rr][4] * x1.x + m[rr][5] * x1.y + m[rr][6] * x1.z + m[rr][7] * x1.w;
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < kBrR; ++rr) {
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      if (b < B) {
        float s = acc[rr][b];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (lane == 0 && r0 + rr < N) out[(size_t)b * N + r0 + rr] = s;
      }
    }
  }
}

// Token b's routing: sigmoid scores of its E router logits, the top_k (larger
// first, lower index on ties) and their weights normalised to sum 1. One wave.
__global__ void __launch_bounds__(64) bs_topk_kernel(const float* logits, int E, int top_k, int32_t* idx, float* wts) {
  __shared__ float sg[kMaxExpertsU];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) sg[e] = 1.0f / (1.0f + __expf(-logits[(size_t)b * E + e]));
  __syncthreads();
  float total = 0.f;
  for (int j = 0; j < top_k; ++j) {
    float bv = -1.f;
    int bi = 0x7fffffff;
    for (int e = lane; e < E; e += 64) {
      const float v = sg[e];
      if (v > bv || (v == bv && e < bi)) { bv = v; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) {
      idx[b * top_k + j] = bi;
      wts[b * top_k + j] = bv;
      sg[bi] = -2.f;  // taken
    }
    total += bv;
    __syncthreads();
  }
  if (lane < top_k) wts[b * top_k + lane] /= total;
}

// argmax over V logits of token b (lowest index on ties), in two stages:
// kArgParts workgroups per token each reduce a range, then one wave per token
// reduces the parts.
constexpr int kArgParts = kArgPartsMax;
__device__ __forceinline__ void arg_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}
__global__ void __launch_bounds__(kST) bs_argmax_part_kernel(const float* logits, int V, float* pv, int32_t* pi) {
  __shared__ float bvs[kST / 64];
  __shared__ int bis[kST / 64];
  const int b = blockIdx.x / kArgParts, part = blockIdx.x % kArgParts;
  const int per = (V + kArgParts - 1) / kArgParts, i0 = part * per, i1 = min(V, i0 + per);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = i0 + threadIdx.x; i < i1; i += kST) arg_better(bv, bi, logits[(size_t)b * V + i], i);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) arg_better(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
  if ((threadIdx.x & 63) == 0) { bvs[threadIdx.x >> 6] = bv; bis[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {  // holds wave 0's result already
    for (int i = 1; i < kST / 64; ++i) arg_better(bv, bi, bvs[i], bis[i]);
    pv[blockIdx.x] = bv;
    pi[blockIdx.x] = bi;
  }
}
__global__ void __launch_bounds__(64) bs_argmax_final_kernel(const float* pv, const int32_t* pi, int32_t* out) {
  const int b = blockIdx.x, lane = threadIdx.x;
  float bv = pv[b * kArgParts + lane];
  int bi = pi[b * kArgParts + lane];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) arg_better(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
  if (lane == 0) out[b] = bi;
}

// ------------------------------------------------------------------ launchers

hipError_t bs_input(const uint16_t* embed, const uint16_t* x_in, const BatchTokens& tk, int B, int D, float* x,
                    hipStream_t st) {
  hipLaunchKernelGGL(bs_input_kernel, dim3(B), dim3(kST), 0, st, embed, x_in, tk, D, x);
  return hipGetLastError();
}
hipError_t bs_norm(float* x, const float* add, bool round, const float* gain, float eps, int B, int D, float* h,
                   hipStream_t st) {
  hipLaunchKernelGGL(bs_norm_kernel, dim3(B), dim3(kNT), 0, st, x, add, round ? 1 : 0, gain, eps, D, h);
  return hipGetLastError();
}
hipError_t bs_latent(const float* qkv, int ldq, int dq, int dc, int dr, const float* q_norm, const float* kv_norm,
                     float eps, const float* rope_tab, const BatchTokens& tk, int B, uint16_t* cache,
                     int64_t seq_stride, float* cq, hipStream_t st) {
  hipLaunchKernelGGL(bs_latent_kernel, dim3(B), dim3(kST), 0, st, qkv, ldq, dq, dc, dr, q_norm, kv_norm, eps,
                     rope_tab, tk, cache, seq_stride, cq);
  return hipGetLastError();
}
hipError_t bs_absorb(const float* q, const uint8_t* codes, const uint16_t* scales, int nkb, int H, int dn, int dr,
                     int dc, int B, const float* rope_tab, const BatchTokens& tk, float* qlat, float* qpe,
                     hipStream_t st) {
  const int cps = ab_col_parts(dc);
  hipLaunchKernelGGL(bs_absorb_kernel, dim3(H * cps), dim3(kAbT), (size_t)B * (dn + dc / cps) * 4, st, q, codes,
                     scales, nkb, H, dn, dr, dc, B, rope_tab, tk, qlat, qpe);
  return hipGetLastError();
}
size_t bs_attn_lds(int dc, int dr) {
  const int rs = dc + dr + 8;
  return (size_t)2 * 16 * rs * 2 + (size_t)kBlk * rs * 2 + 2 * 16 * kBlk * 4 + 48 * 4;
}
// Position chunk of the attention workgroups for a longest context of ctx:
// at least one block of kBlk positions, at most kAttnChunksMax chunks.
int bs_attn_chunk(int ctx) {
  const int c = std::max(kBlk, (ctx + kAttnChunksMax - 1) / kAttnChunksMax);
  return (c + kBlk - 1) / kBlk * kBlk;
}
template <int NT, bool SP>
static hipError_t launch_attn(dim3 grid, size_t lds, hipStream_t st, const float* qlat, const float* qpe,
                              const uint16_t* cache, int64_t seq_stride, int H, int dc, int dr, float tau,
                              const BatchTokens& tk, int nch, int chunk, float* part, const int32_t* sel,
                              int sel_stride, int sel_rows) {
  static bool raised = false;  // more dynamic LDS than the default 64 KB (gfx950 has 160 KB)
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bs_attn_kernel<NT, SP>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL((bs_attn_kernel<NT, SP>), grid, dim3(kAT), lds, st, qlat, qpe, cache, seq_stride, H, dc, dr,
                     tau, tk, nch, chunk, part, sel, sel_stride, sel_rows);
  return hipGetLastError();
}
template <bool SP>
static hipError_t launch_attn_nt(dim3 grid, size_t lds, hipStream_t st, const float* qlat, const float* qpe,
                                 const uint16_t* cache, int64_t seq_stride, int H, int dc, int dr, float tau,
                                 const BatchTokens& tk, int nch, int chunk, float* part, const int32_t* sel,
                                 int sel_stride, int sel_rows) {
  if (dc == 512)
    return launch_attn<8, SP>(grid, lds, st, qlat, qpe, cache, seq_stride, H, dc, dr, tau, tk, nch, chunk, part, sel,
                              sel_stride, sel_rows);
  if (dc == 256)
    return launch_attn<4, SP>(grid, lds, st, qlat, qpe, cache, seq_stride, H, dc, dr, tau, tk, nch, chunk, part, sel,
                              sel_stride, sel_rows);
  return launch_attn<2, SP>(grid, lds, st, qlat, qpe, cache, seq_stride, H, dc, dr, tau, tk, nch, chunk, part, sel,
                            sel_stride, sel_rows);
}
hipError_t bs_attn(const float* qlat, const float* qpe, const uint16_t* cache, int64_t seq_stride, int H, int dc,
                   int dr, float tau, const BatchTokens& tk, int B, float* part, float* olat, hipStream_t st,
                   const int32_t* sel, int sel_stride, int sel_rows) {
  const size_t lds = bs_attn_lds(dc, dr);
  int ctx = 1;
  for (int b = 0; b < B; ++b) ctx = std::max(ctx, tk.pos[b] + 1);
  const int chunk = bs_attn_chunk(ctx), nch = (ctx + chunk - 1) / chunk;
  const dim3 grid(B * ((H + 15) / 16) * nch);
  const hipError_t e =
      sel ? launch_attn_nt<true>(grid, lds, st, qlat, qpe, cache, seq_stride, H, dc, dr, tau, tk, nch, chunk, part,
                                 sel, sel_stride, sel_rows)
          : launch_attn_nt<false>(grid, lds, st, qlat, qpe, cache, seq_stride, H, dc, dr, tau, tk, nch, chunk, part,
                                  nullptr, 0, 0);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bs_attn_merge_kernel, dim3(B * H), dim3(kST), 0, st, part, H, dc, nch, chunk, tk, olat);
  return hipGetLastError();
}
hipError_t bs_uv(const float* olat, const uint8_t* codes, const uint16_t* scales, int nkb, int H, int dv, int dc,
                 int B, float* o, hipStream_t st) {
  hipLaunchKernelGGL(bs_uv_kernel, dim3(H * uv_row_parts(dv)), dim3(kST), (size_t)B * dc * 4, st, olat, codes, scales,
                     nkb, H, dv, dc, B, o);
  return hipGetLastError();
}
hipError_t bs_bf16_rows(const float* h, const uint16_t* M, int N, int K, int B, float* out, hipStream_t st) {
  const int rows_per_wg = kBrR * (kST / 64);
  const dim3 grid((N + rows_per_wg - 1) / rows_per_wg);
  if (B <= 1) hipLaunchKernelGGL(bs_bf16_rows_kernel<1>, grid, dim3(kST), 0, st, h, M, N, K, B, out);
  else if (B <= 2) hipLaunchKernelGGL(bs_bf16_rows_kernel<2>, grid, dim3(kST), 0, st, h, M, N, K, B, out);
  else if (B <= 4) hipLaunchKernelGGL(bs_bf16_rows_kernel<4>, grid, dim3(kST), 0, st, h, M, N, K, B, out);
  else if (B <= 8) hipLaunchKernelGGL(bs_bf16_rows_kernel<8>, grid, dim3(kST), 0, st, h, M, N, K, B, out);
  else hipLaunchKernelGGL(bs_bf16_rows_kernel<kBatchMax>, grid, dim3(kST), 0, st, h, M, N, K, B, out);
  return hipGetLastError();
}
hipError_t bs_topk(const float* logits, int B, int E, int top_k, int32_t* idx, float* wts, hipStream_t st) {
  hipLaunchKernelGGL(bs_topk_kernel, dim3(B), dim3(64), 0, st, logits, E, top_k, idx, wts);
  return hipGetLastError();
}
hipError_t bs_argmax(const float* logits, int B, int V, float* part_v, int32_t* part_i, int32_t* out,
                     hipStream_t st) {
  hipLaunchKernelGGL(bs_argmax_part_kernel, dim3(B * kArgParts), dim3(kST), 0, st, logits, V, part_v, part_i);
  hipLaunchKernelGGL(bs_argmax_final_kernel, dim3(B), dim3(64), 0, st, part_v, part_i, out);
  return hipGetLastError();
}

}  // namespace pdm
