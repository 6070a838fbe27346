// Host planner: buffer layouts and the ordered stage list of one decode step.
//
// The stage list is the compile-time tile-task DAG of the engine. TileRT
// moves orchestration to compile time and keeps only minimal scheduling at
// run time ("What is TileRT", section 6.2; SemiAnalysis TileRT page, section
// on dataflow ideas: ahead-of-time scheduling, persistent execution). Here a
// stage is one operator split over all persistent workgroups; the workgroup's
// share of a stage is fixed by its index, and the only run-time scheduling is
// waiting on the arrival counters of the stage a stage depends on.
#include <cstring>
#include <algorithm>

#include "pdm_internal.h"

namespace pdm {

int validate_dims(const pdm_dims& d, int32_t max_ctx) {
  if (d.n_layers < 1 || d.n_layers > PDM_MAX_LAYERS) return PDM_ERR_CONFIG;
  if (max_ctx < 1 || max_ctx > (1 << 22)) return PDM_ERR_ARG;
  auto m16 = [](int v) { return v > 0 && v % 16 == 0; };
  if (!m16(d.hidden) || !m16(d.q_lora) || !m16(d.qk_nope) || !m16(d.v_head)) return PDM_ERR_CONFIG;
  if (d.rope <= 0 || d.rope % 16 != 0 || d.rope > 128) return PDM_ERR_CONFIG;
  if (!(d.kv_lora == 128 || d.kv_lora == 256 || d.kv_lora == 512)) return PDM_ERR_CONFIG;
  if (!is_pow2(d.v_head)) return PDM_ERR_CONFIG;
  if (d.n_heads <= 0 || d.n_heads % 8 != 0 || d.n_heads > kMaxHeads) return PDM_ERR_CONFIG;
  if (d.hidden > kXMax || d.q_lora > kXMax || d.n_heads * d.v_head > kXMax) return PDM_ERR_CONFIG;
  bool any_dense = false, any_moe = false;
  for (int l = 0; l < d.n_layers; ++l) {
    if (d.layer_moe[l] > 1) return PDM_ERR_CONFIG;
    (d.layer_moe[l] ? any_moe : any_dense) = true;
  }
  if (any_dense && (!m16(d.ffn) || d.ffn > kXMax)) return PDM_ERR_CONFIG;
  if (any_moe) {
    if (!is_pow2(d.moe_ffn) || d.moe_ffn < 16) return PDM_ERR_CONFIG;
    if (d.n_experts < 1 || d.n_experts > 1024 || d.top_k < 1 || d.top_k > d.n_experts) return PDM_ERR_CONFIG;
    if (d.n_shared < 0 || d.top_k + d.n_shared > kMaxSlots) return PDM_ERR_CONFIG;
    if ((int64_t)(d.top_k + d.n_shared) * d.moe_ffn > kXMax) return PDM_ERR_CONFIG;
  }
  if (d.vocab < 0) return PDM_ERR_CONFIG;
  // small-K GEMV units must not straddle a per-head input vector
  if (d.qk_nope < 1024 && (!is_pow2(d.qk_nope) || 1024 / d.qk_nope > d.kv_lora)) return PDM_ERR_CONFIG;
  if (d.kv_lora < 1024 && 1024 / d.kv_lora > d.v_head) return PDM_ERR_CONFIG;
  if (!(d.rms_eps >= 0.f) || !(d.rope_base > 1.f)) return PDM_ERR_CONFIG;
  if (d.expert_format != PDM_FMT_FP8 && d.expert_format != PDM_FMT_MXFP4) return PDM_ERR_CONFIG;
  if (any_moe && d.expert_format == PDM_FMT_MXFP4 && (d.moe_ffn < 64 || d.hidden % 32 != 0)) return PDM_ERR_CONFIG;
  return PDM_OK;
}

uint64_t dims_hash(const pdm_dims& d) {
  // FNV-1a over the bytes of the shape fields
  const unsigned char* p = reinterpret_cast<const unsigned char*>(&d);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < sizeof(pdm_dims); ++i) { h ^= p[i]; h *= 1099511628211ull; }
  return h;
}

namespace {

struct Cursor {
  uint64_t off = 0;
  uint64_t take(uint64_t bytes) {
    uint64_t o = align_up(off, 256);
    off = o + bytes;
    return o;
  }
};

Fp8Mat fp8_mat(Cursor& c, int rows, int K) {
  Fp8Mat m{};
  m.rows = rows;
  m.K = K;
  m.nkb = (int)ceil_div(K, 128);
  m.fmt = PDM_FMT_FP8;
  m.codes = c.take((uint64_t)rows * K);
  m.scales = c.take((uint64_t)(rows / 8) * m.nkb * 2);
  return m;
}

// K elements per row (a multiple of 32): K / 2 code bytes and K / 32 scale bytes per row
Fp8Mat mxfp4_mat(Cursor& c, int rows, int K) {
  Fp8Mat m{};
  m.rows = rows;
  m.K = K / 2;
  m.nkb = K / 32;
  m.fmt = PDM_FMT_MXFP4;
  m.codes = c.take((uint64_t)rows * m.K);
  m.scales = c.take((uint64_t)rows * m.nkb);
  return m;
}

uint64_t mat_bytes(const Fp8Mat& m) {
  return (uint64_t)m.rows * m.K + (m.fmt == PDM_FMT_MXFP4 ? (uint64_t)m.rows * m.nkb : (uint64_t)(m.rows / 8) * m.nkb * 2);
}

// rows covered by one 1 KB GEMV unit when a row is shorter than 1 KB
int unit_rows(int K, int ebytes) {
  int kb = K * ebytes;
  return (kb < 1024 && is_pow2(kb)) ? 1024 / kb : 1;
}

}  // namespace

int build_plan(const pdm_dims& d, int32_t max_ctx, int32_t G, Plan* p, Layout* lay) {
  int rc = validate_dims(d, max_ctx);
  if (rc) return rc;
  if (G < 1 || G > 4096) return PDM_ERR_ARG;
  std::memset(p, 0, sizeof(Plan));
  p->dims = d;
  p->G = G;
  p->max_ctx = max_ctx;
  const int H = d.n_heads, D = d.hidden, qkh = d.qk_nope + d.rope, kvr = d.kv_lora + d.rope;
  p->hg = (H % kHeadGroup == 0) ? kHeadGroup : 8;
  p->n_hg = H / p->hg;
  // every head group needs at least one attention unit (one workgroup)
  if (p->n_hg > G) return PDM_ERR_CONFIG;
  {
    int by_wg = G / p->n_hg;
    int by_ctx = (int)std::max<int64_t>(1, ceil_div(max_ctx, 16));
    p->nch = std::min(by_wg, by_ctx);
  }
  p->nch = std::min(p->nch, kMaxChunks);
  if (kvr % 32 != 0 || p->hg > 16) return PDM_ERR_CONFIG;
  // q_b row split and the number of q_lat partials per head
  p->qb_gran = std::max(2, unit_rows(d.q_lora, 1));
  if (((int64_t)H * qkh / p->qb_gran) * G >= (1LL << 31)) return PDM_ERR_CONFIG;
  p->qb_maxparts = 1;
  for (int h = 0; h < H; ++h) p->qb_maxparts = std::max(p->qb_maxparts, qb_parts(d, p->qb_gran, G, h));
  if (p->qb_maxparts > 64) return PDM_ERR_CONFIG;  // the attention stage keeps a 64-bit slot mask per head
  for (int h = 0; h < H; ++h) {
    const int first = qb_first(d, p->qb_gran, G, h), np = qb_parts(d, p->qb_gran, G, h);
    uint64_t m = 0;
    for (int k = 0; k < np; ++k) {
      int ra, rb;
      split_rows(H * qkh, p->qb_gran, G, first + k, ra, rb);
      if (rb > ra) m |= 1ull << k;
    }
    p->qb_mask[h] = m;
  }
  {
    // q_b LDS: staged c_q, the workgroup's q_nope values, its W_UK rows and
    // their scales (each DMA'd with 1 KB of slack), the absorb reduction
    int64_t most = 0;
    for (int w = 0; w < G; ++w) {
      int ra, rb, u0, u1;
      split_rows(H * qkh, p->qb_gran, G, w, ra, rb);
      qb_nope_rows(d, ra, rb, u0, u1);
      most = std::max<int64_t>(most, u1 - u0);
    }
    const int64_t bytes = align_up(d.q_lora, 1024) * 4 + align_up(most, 4) * 4 + most * d.kv_lora + 1024 +
                          (most / 8 + 2) * (d.kv_lora / 128) * 2 + 32 + 1024 + (int64_t)kThreads * 16 * 4;
    if (bytes > (int64_t)kXMax * 4) return PDM_ERR_CONFIG;
  }
  {
    // attention LDS: query hi/lo rows [16][kvr + 8] bf16, 64 staged cache
    // rows [64][kvr / 2 + 4] u32, two score partials [2][16][68] f32, 48 head
    // scalars, the current cache row [kvr / 2] u32. Before the first block is
    // staged, the space after the queries holds the DMA'd q_lat partials,
    // rotary queries and key/value latent (each with 1 KB of slack).
    const int64_t qbytes = 2LL * 16 * (kvr + 8) * 2;
    const int64_t end = (int64_t)kXMax * 4 - kvr * 2 - 48 * 4;  // head scalars and the new row at the end
    if (qbytes + 64LL * (kvr / 2 + 4) * 4 + 2LL * 16 * 68 * 4 > end) return PDM_ERR_CONFIG;
    const int64_t tmp = (int64_t)p->hg * p->qb_maxparts * d.kv_lora * 4 + 1024 + 2LL * p->hg * d.rope * 2 + 1024 +
                        (int64_t)kvr * 4 + 1024;
    if (qbytes + tmp > end) return PDM_ERR_CONFIG;
  }
  // every packed 8-row x 128-column scale tile of W_UK and W_UV must lie in one logical block
  for (int h = 0; h < H; ++h) {
    const int base = h * (d.qk_nope + d.v_head);
    for (int n0 = 0; n0 < d.qk_nope; n0 += 8)
      if ((base + n0) / 128 != (base + n0 + 7) / 128) return PDM_ERR_CONFIG;
    for (int v0 = 0; v0 < d.v_head; v0 += 8)
      if ((base + d.qk_nope + v0) / 128 != (base + d.qk_nope + v0 + 7) / 128) return PDM_ERR_CONFIG;
  }

  // ---------------- weight arena
  Cursor w;
  w.off = kHeaderBytes;
  if (d.vocab > 0) {
    p->embed = w.take((uint64_t)d.vocab * D * 2);
    p->final_norm = w.take((uint64_t)D * 4);
    p->lm_head = w.take((uint64_t)d.vocab * D * 2);
  }
  for (int l = 0; l < d.n_layers; ++l) {
    LayerPlan& L = p->layers[l];
    L.is_moe = d.layer_moe[l];
    L.attn_norm = w.take((uint64_t)D * 4);
    L.q_norm = w.take((uint64_t)d.q_lora * 4);
    L.kv_norm = w.take((uint64_t)d.kv_lora * 4);
    L.ffn_norm = w.take((uint64_t)D * 4);
    L.qkv = fp8_mat(w, d.q_lora + kvr, D);
    L.qb = fp8_mat(w, H * qkh, d.q_lora);
    L.uk = fp8_mat(w, H * d.qk_nope, d.kv_lora);
    L.uv = fp8_mat(w, H * d.v_head, d.kv_lora);
    L.wo = fp8_mat(w, D, H * d.v_head);
    if (!L.is_moe) {
      L.gu = fp8_mat(w, 2 * d.ffn, D);
      L.down = fp8_mat(w, D, d.ffn);
    } else {
      L.router = w.take((uint64_t)d.n_experts * D * 2);
      Cursor e;  // layout inside one expert block
      auto emat = d.expert_format == PDM_FMT_MXFP4 ? mxfp4_mat : fp8_mat;
      L.egu = emat(e, 2 * d.moe_ffn, D);
      L.edown = emat(e, D, d.moe_ffn);
      L.expert_stride = align_up(e.off, 256);
      L.expert_base = w.take(L.expert_stride * (uint64_t)(d.n_experts + d.n_shared));
    }
  }
  lay->weight_bytes = align_up(w.off, 256);

  // ---------------- KV cache
  Cursor kv;
  for (int l = 0; l < d.n_layers; ++l) p->layers[l].kv = kv.take((uint64_t)max_ctx * kvr * 2);
  lay->kv_bytes = align_up(std::max<uint64_t>(kv.off, 256), 256);

  // ---------------- stages
  int ns = 0;
  auto add = [&](int type, int layer, int wait, int rows, int K, int gran) {
    StagePlan& s = p->stages[ns];
    s.type = type; s.layer = layer; s.wait = wait; s.rows = rows; s.K = K; s.gran = gran;
    return ns++;
  };
  int last = -1;
  for (int l = 0; l < d.n_layers; ++l) {
    const LayerPlan& L = p->layers[l];
    int s_qkv = add(PDM_ST_QKV, l, last, L.qkv.rows, D, unit_rows(D, 1));
    int s_qb = add(PDM_ST_QB, l, s_qkv, L.qb.rows, d.q_lora, p->qb_gran);
    // attention units wait only for the q_b workgroups of their head group,
    // W_UV workgroups only for the attention units of their heads
    int s_att = add(PDM_ST_ATTN, l, s_qb, p->n_hg * p->nch, kvr, 1);
    int s_uv = add(PDM_ST_UV, l, s_att, L.uv.rows, d.kv_lora, unit_rows(d.kv_lora, 1));
    int s_wo = add(PDM_ST_WO, l, s_uv, D, H * d.v_head, unit_rows(H * d.v_head, 1));
    if (!L.is_moe) {
      int s_gu = add(PDM_ST_GU, l, s_wo, 2 * d.ffn, D, std::max(16, unit_rows(D, 1)));
      last = add(PDM_ST_DOWN, l, s_gu, D, d.ffn, unit_rows(d.ffn, 1));
    } else {
      // Router and gate/up both read RMSNorm(x_attn): the router stage stages
      // it and the gate/up stage (shared and routed experts) reuses it from LDS.
      int s_rt = add(PDM_ST_ROUTER, l, s_wo, d.n_experts, D, unit_rows(D, 2));
      // expert rows hold K bytes (FP8) or K / 2 bytes (MXFP4)
      const bool fp4 = d.expert_format == PDM_FMT_MXFP4;
      int s_gr = add(PDM_ST_GU_ROUTED, l, s_rt, 2 * d.moe_ffn * (d.n_shared + d.top_k), D,
                     std::max(16, unit_rows(fp4 ? D / 2 : D, 1)));
      // (the MXFP4 stage stages its input in its own order)
      p->stages[s_gr].flags = fp4 ? kStMx : kStXStaged;
      int kslots = (d.top_k + d.n_shared) * d.moe_ffn;
      last = add(PDM_ST_DOWN, l, s_gr, D, kslots, unit_rows(fp4 ? kslots / 2 : kslots, 1));
      if (fp4) p->stages[last].flags = kStMx;
    }
    if (ns > kMaxStages - 2) return PDM_ERR_CONFIG;
  }
  if (d.vocab > 0) add(PDM_ST_LM, -1, last, d.vocab, D, unit_rows(D, 2));
  p->n_stages = ns;

  // per-workgroup staged-input limit for the per-head GEMVs
  for (int s = 0; s < ns; ++s) {
    const StagePlan& st = p->stages[s];
    int rpv = st.type == PDM_ST_UV ? d.v_head : 0;
    if (!rpv) continue;
    int64_t ng = st.rows / st.gran;
    int64_t per = ceil_div(ng, G) * st.gran;
    int64_t heads = ceil_div(per, rpv) + 1;
    // staged vectors occupy whole 1024-float blocks of the permuted LDS layout
    if (align_up((uint64_t)(heads * st.K), 1024) > (uint64_t)kXMax) return PDM_ERR_CONFIG;
  }

  // ---------------- scratch
  Cursor s;
  lay->plan_off = s.take(sizeof(Plan));
  p->rope_tab = s.take((uint64_t)max_ctx * (d.rope / 2) * 2 * 4);
  p->counters = s.take((uint64_t)(ns + 1) * kStripes * kCounterStride * 4);
  p->flags = s.take((uint64_t)ns * G * 4);
  p->status = s.take(256);
  p->lm_best = s.take((uint64_t)G * 8);
  p->logits_internal = s.take((uint64_t)std::max(d.vocab, 1) * 4);
  p->x0 = s.take((uint64_t)D * 4);
  // per-layer taps are contiguous across layers: [n_layers][...]
  const uint64_t xo_all = s.take((uint64_t)d.n_layers * D * 4);
  const uint64_t xa_all = s.take((uint64_t)d.n_layers * D * 4);
  const int kk = std::max(d.top_k, 1);
  const uint64_t ti_all = s.take((uint64_t)d.n_layers * kk * 4);
  const uint64_t tw_all = s.take((uint64_t)d.n_layers * kk * 4);
  // Working activations are shared by all layers: a layer's buffers are
  // written again only after full barriers that every reader of the previous
  // layer has passed (the next q_a/kv_a stage waits for all workgroups' last
  // stage, the W_O stage for all W_UV workgroups).
  int64_t act = 1;
  for (int l = 0; l < d.n_layers; ++l)
    act = std::max<int64_t>(act, d.layer_moe[l] ? (int64_t)(d.top_k + d.n_shared) * d.moe_ffn : d.ffn);
  const uint64_t qkv_raw = s.take((uint64_t)(d.q_lora + kvr) * 4);
  const uint64_t qlat_part = s.take((uint64_t)H * p->qb_maxparts * d.kv_lora * 4);
  const uint64_t qrope = s.take((uint64_t)p->n_hg * 2 * p->hg * d.rope * 2);
  const uint64_t attn_part = s.take((uint64_t)H * p->nch * (d.kv_lora + 4) * 4);
  const uint64_t o = s.take((uint64_t)H * d.v_head * 4);
  const uint64_t act_buf = s.take((uint64_t)act * 4);
  const uint64_t router_logits = s.take((uint64_t)std::max(d.n_experts, 1) * 4);
  for (int l = 0; l < d.n_layers; ++l) {
    LayerPlan& L = p->layers[l];
    L.xo = xo_all + (uint64_t)l * D * 4;
    L.xa = xa_all + (uint64_t)l * D * 4;
    L.topk_idx = ti_all + (uint64_t)l * kk * 4;
    L.topk_w = tw_all + (uint64_t)l * kk * 4;
    L.qkv_raw = qkv_raw;
    L.qlat_part = qlat_part;
    L.qrope = qrope;
    L.attn_part = attn_part;
    L.o = o;
    L.act = act_buf;
    L.router_logits = router_logits;
  }
  lay->scratch_bytes = align_up(s.off, 256);
  lay->trace_bytes = (uint64_t)ns * G * kTraceWords * 8;
  return PDM_OK;
}

void stage_info(const Plan& p, int s, pdm_stage_info* o) {
  const pdm_dims& d = p.dims;
  const StagePlan& st = p.stages[s];
  std::memset(o, 0, sizeof(*o));
  for (int i = 0; i < 4; ++i) o->reads[i] = -1;
  for (int i = 0; i < 2; ++i) o->writes[i] = -1;
  o->type = st.type;
  o->layer = st.layer;
  o->wait_stage = st.wait;
  o->rows = st.rows;
  o->k = st.K;
  const int l = st.layer;
  auto id = [&](int buf, int layer) { return buf + 16 * layer; };
  auto input = [&]() { return l == 0 ? id(PDM_BUF_INPUT, 0) : id(PDM_BUF_XOUT, l - 1); };
  auto fp8b = [](const Fp8Mat& m) { return mat_bytes(m); };
  if (st.type == PDM_ST_LM) {
    o->reads[0] = id(PDM_BUF_XOUT, d.n_layers - 1);
    o->writes[0] = id(PDM_BUF_LOGITS, d.n_layers);
    o->weight_bytes = (uint64_t)d.vocab * d.hidden * 2 + (uint64_t)d.hidden * 4;
    return;
  }
  const LayerPlan& L = p.layers[l];
  switch (st.type) {
    case PDM_ST_QKV:
      o->reads[0] = input(); o->writes[0] = id(PDM_BUF_QKV, l);
      o->weight_bytes = fp8b(L.qkv) + (uint64_t)d.hidden * 4; break;
    case PDM_ST_QB:
      o->reads[0] = id(PDM_BUF_QKV, l); o->writes[0] = id(PDM_BUF_QLAT, l);
      o->weight_bytes = fp8b(L.qb) + fp8b(L.uk) + (uint64_t)d.q_lora * 4; break;
    case PDM_ST_ATTN:
      o->reads[0] = id(PDM_BUF_QLAT, l); o->reads[1] = id(PDM_BUF_QKV, l); o->reads[2] = id(PDM_BUF_KV, l);
      o->writes[0] = id(PDM_BUF_ATTN, l); o->writes[1] = id(PDM_BUF_KV, l);
      o->weight_bytes = (uint64_t)d.kv_lora * 4; break;
    case PDM_ST_UV:
      o->reads[0] = id(PDM_BUF_ATTN, l); o->writes[0] = id(PDM_BUF_O, l);
      o->weight_bytes = fp8b(L.uv); break;
    case PDM_ST_WO:
      o->reads[0] = id(PDM_BUF_O, l); o->reads[1] = input(); o->writes[0] = id(PDM_BUF_XATTN, l);
      o->weight_bytes = fp8b(L.wo); break;
    case PDM_ST_ROUTER:
      o->reads[0] = id(PDM_BUF_XATTN, l); o->writes[0] = id(PDM_BUF_ROUTER, l);
      o->weight_bytes = (uint64_t)d.n_experts * d.hidden * 2 + (uint64_t)d.hidden * 4; break;
    case PDM_ST_GU:
      o->reads[0] = id(PDM_BUF_XATTN, l); o->writes[0] = id(PDM_BUF_ACT, l);
      o->weight_bytes = fp8b(L.gu); break;
    case PDM_ST_GU_ROUTED:
      o->reads[0] = id(PDM_BUF_XATTN, l); o->reads[1] = id(PDM_BUF_ROUTER, l); o->writes[0] = id(PDM_BUF_ACT, l);
      o->weight_bytes = fp8b(L.egu) * (d.top_k + d.n_shared); break;
    case PDM_ST_DOWN:
      o->reads[0] = id(PDM_BUF_ACT, l); o->reads[1] = id(PDM_BUF_XATTN, l); o->writes[0] = id(PDM_BUF_XOUT, l);
      if (L.is_moe) o->reads[2] = id(PDM_BUF_ROUTER, l);
      o->weight_bytes = L.is_moe ? fp8b(L.edown) * (d.top_k + d.n_shared) : fp8b(L.down); break;
    default: break;
  }
}

}  // namespace pdm
