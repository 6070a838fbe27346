// C ABI of the persistent decode engine (declared in include/pdm.h).
//
// Host side only: argument validation, buffer binding, the offline packer
// entry points and one kernel launch per decode step. No compute of the step
// happens here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "engine.h"
#include "pdm_internal.h"

using namespace pdm;

struct pdm_engine {
  pdm_dims dims;
  int32_t max_ctx = 0;
  int device = 0;
  int G = 0;
  Plan plan;   // relative offsets
  Layout lay;
  bool bound = false;
  uint8_t* w = nullptr;
  uint8_t* kv = nullptr;
  uint8_t* scratch = nullptr;
  uint64_t* trace = nullptr;
  Plan* plan_dev = nullptr;
  Plan abs;    // absolute addresses (as copied to the device)
  uint32_t epoch = 0;
  std::vector<int32_t> layer_len;
  int32_t spin_limit = 1 << 22;
  int32_t skip_stage = -1;
  bool cooperative = false;
  bool trace_on = true;
  uint8_t* batch_ws = nullptr;  // workspace of the batched feed-forward call (allocated on first use)
  uint8_t* step_ws = nullptr;   // activations of the batched decode step (allocated on first use)
};

namespace {

constexpr int32_t kDefaultSpin = 1 << 22;

struct Header {
  uint32_t magic;
  uint32_t abi;
  uint64_t dims_hash;
  uint64_t weight_bytes;
  uint64_t pad[29];
};
static_assert(sizeof(Header) == kHeaderBytes, "header is 256 bytes");

int hip_fail(hipError_t e) { return e == hipSuccess ? PDM_OK : PDM_ERR_LAUNCH; }

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

void fill_sizes(const Plan& p, const Layout& lay, pdm_sizes* out) {
  out->weight_bytes = lay.weight_bytes;
  out->kv_bytes = lay.kv_bytes;
  out->scratch_bytes = lay.scratch_bytes;
  out->trace_bytes = lay.trace_bytes;
  out->alignment = 256;
  out->n_stages = p.n_stages;
  out->n_workgroups = p.G;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Absolute-address copy of the plan for the bound buffers.
void absolutize(const pdm_engine& e, Plan* a) {
  *a = e.plan;
  const uint64_t W = reinterpret_cast<uint64_t>(e.w), K = reinterpret_cast<uint64_t>(e.kv),
                 S = reinterpret_cast<uint64_t>(e.scratch);
  auto fw = [&](uint64_t& v) { v += W; };
  auto fm = [&](Fp8Mat& m) { m.codes += W; m.scales += W; };
  auto fs = [&](uint64_t& v) { v += S; };
  if (e.dims.vocab > 0) { fw(a->embed); fw(a->final_norm); fw(a->lm_head); }
  fs(a->rope_tab); fs(a->counters); fs(a->flags); fs(a->status); fs(a->lm_best); fs(a->logits_internal); fs(a->x0);
  a->trace = reinterpret_cast<uint64_t>(e.trace);
  for (int l = 0; l < e.dims.n_layers; ++l) {
    LayerPlan& L = a->layers[l];
    fw(L.attn_norm); fw(L.q_norm); fw(L.kv_norm); fw(L.ffn_norm);
    fm(L.qkv); fm(L.qb); fm(L.uk); fm(L.uv); fm(L.wo);
    if (!L.is_moe) { fm(L.gu); fm(L.down); }
    else { fw(L.router); fw(L.expert_base); }  // egu / edown stay relative to an expert block
    L.kv += K;
    fs(L.qkv_raw); fs(L.qlat_part); fs(L.qrope); fs(L.attn_part); fs(L.o); fs(L.xa); fs(L.act);
    fs(L.router_logits); fs(L.xo); fs(L.topk_idx); fs(L.topk_w);
  }
}

int check_engine(const pdm_engine* e, bool need_bound) {
  if (!e) return PDM_ERR_ARG;
  if (need_bound && !e->bound) return PDM_ERR_UNBOUND;
  return PDM_OK;
}

int bind_buffers(pdm_engine* e, void* weights_dev, uint64_t weight_bytes, void* kv_dev, uint64_t kv_bytes,
                 void* scratch_dev, uint64_t scratch_bytes, void* trace_dev, uint64_t trace_bytes);

// Where an FP8 tensor goes in the weight arena: one packed matrix, or two for
// W_UKV (its key rows to W_UK, its value rows to W_UV). Offsets are relative
// to the arena start (plan with relative addresses).
struct PackTarget {
  PackMap m;
  uint64_t codes, scales;
  int fmt;  // PDM_FMT_* of the packed matrix
};
int pack_targets(const pdm_dims& d, const Plan& p, int32_t tensor, int32_t layer, int32_t expert, PackTarget* t,
                 int* n) {
  if (layer < 0 || layer >= d.n_layers) return PDM_ERR_ARG;
  const LayerPlan& L = p.layers[layer];
  const int H = d.n_heads, D = d.hidden, qkh = d.qk_nope + d.rope, kvr = d.kv_lora + d.rope;
  const bool moe = L.is_moe != 0;
  *n = 1;
  auto set = [&](PackTarget& x, int mode, int N, int K, const Fp8Mat& dst, uint64_t base, int row0, int which) {
    x.m = PackMap{};
    x.m.mode = mode; x.m.N = N; x.m.K = K; x.m.rows = dst.rows; x.m.Kp = dst.K; x.m.nkb = dst.nkb;
    x.m.row0 = row0; x.m.which = which; x.m.dn = d.qk_nope; x.m.dv = d.v_head; x.m.dc = d.kv_lora;
    x.codes = base + dst.codes;
    x.scales = base + dst.scales;
    x.fmt = dst.fmt;
  };
  if (expert >= 0) {
    if (!moe || expert >= d.n_experts + d.n_shared) return PDM_ERR_ARG;
    const uint64_t blk = L.expert_base + (uint64_t)expert * L.expert_stride;
    switch (tensor) {
      case PDM_T_W_GATE: set(t[0], 3, d.moe_ffn, D, L.egu, blk, 0, 0); return PDM_OK;
      case PDM_T_W_UP: set(t[0], 3, d.moe_ffn, D, L.egu, blk, 0, 1); return PDM_OK;
      case PDM_T_W_DOWN: set(t[0], 0, D, d.moe_ffn, L.edown, blk, 0, 0); return PDM_OK;
      default: return PDM_ERR_ARG;
    }
  }
  switch (tensor) {
    case PDM_T_WQ_A: set(t[0], 0, d.q_lora, D, L.qkv, 0, 0, 0); return PDM_OK;
    case PDM_T_WKV_A: set(t[0], 0, kvr, D, L.qkv, 0, d.q_lora, 0); return PDM_OK;
    case PDM_T_WQ_B: set(t[0], 0, H * qkh, d.q_lora, L.qb, 0, 0, 0); return PDM_OK;
    case PDM_T_WKV_B:
      set(t[0], 1, H * (d.qk_nope + d.v_head), d.kv_lora, L.uk, 0, 0, 0);
      set(t[1], 2, H * (d.qk_nope + d.v_head), d.kv_lora, L.uv, 0, 0, 0);
      *n = 2;
      return PDM_OK;
    case PDM_T_WO: set(t[0], 0, D, H * d.v_head, L.wo, 0, 0, 0); return PDM_OK;
    case PDM_T_W_GATE: if (moe) return PDM_ERR_ARG; set(t[0], 3, d.ffn, D, L.gu, 0, 0, 0); return PDM_OK;
    case PDM_T_W_UP: if (moe) return PDM_ERR_ARG; set(t[0], 3, d.ffn, D, L.gu, 0, 0, 1); return PDM_OK;
    case PDM_T_W_DOWN: if (moe) return PDM_ERR_ARG; set(t[0], 0, D, d.ffn, L.down, 0, 0, 0); return PDM_OK;
    default: return PDM_ERR_ARG;
  }
}

// Arena offset and byte size of a bf16 or f32 tensor.
int raw_target(const pdm_dims& d, const Plan& p, int32_t tensor, int32_t layer, int32_t expert, uint64_t* off,
               uint64_t* need) {
  if (expert >= 0) return PDM_ERR_ARG;
  if (tensor == PDM_T_EMBED || tensor == PDM_T_LM_HEAD || tensor == PDM_T_FINAL_NORM) {
    if (d.vocab <= 0) return PDM_ERR_ARG;
    if (tensor == PDM_T_EMBED) { *off = p.embed; *need = (uint64_t)d.vocab * d.hidden * 2; }
    else if (tensor == PDM_T_LM_HEAD) { *off = p.lm_head; *need = (uint64_t)d.vocab * d.hidden * 2; }
    else { *off = p.final_norm; *need = (uint64_t)d.hidden * 4; }
    return PDM_OK;
  }
  if (layer < 0 || layer >= d.n_layers) return PDM_ERR_ARG;
  const LayerPlan& L = p.layers[layer];
  switch (tensor) {
    case PDM_T_ATTN_NORM: *off = L.attn_norm; *need = (uint64_t)d.hidden * 4; return PDM_OK;
    case PDM_T_Q_NORM: *off = L.q_norm; *need = (uint64_t)d.q_lora * 4; return PDM_OK;
    case PDM_T_KV_NORM: *off = L.kv_norm; *need = (uint64_t)d.kv_lora * 4; return PDM_OK;
    case PDM_T_FFN_NORM: *off = L.ffn_norm; *need = (uint64_t)d.hidden * 4; return PDM_OK;
    case PDM_T_ROUTER:
      if (!L.is_moe) return PDM_ERR_ARG;
      *off = L.router; *need = (uint64_t)d.n_experts * d.hidden * 2;
      return PDM_OK;
    default: return PDM_ERR_ARG;
  }
}

Header blob_header(const pdm_dims& d, uint64_t weight_bytes) {
  Header h{};
  h.magic = kMagic;
  h.abi = PDM_ABI_VERSION;
  h.dims_hash = dims_hash(d);
  h.weight_bytes = weight_bytes;
  return h;
}

// Relative plan of a model shape for the host packer (the weight arena
// layout depends on neither the context length nor the workgroup count).
struct HostPlan {
  Plan* p = nullptr;
  Layout lay;
  int rc = PDM_OK;
  explicit HostPlan(const pdm_dims* d) {
    if (!d) { rc = PDM_ERR_ARG; return; }
    p = new (std::nothrow) Plan;
    if (!p) { rc = PDM_ERR_OOM; return; }
    rc = build_plan(*d, 1, 256, p, &lay);
  }
  ~HostPlan() { delete p; }
};

}  // namespace

extern "C" {

const char* pdm_strerror(int code) {
  switch (code) {
    case PDM_OK: return "ok";
    case PDM_ERR_ARG: return "invalid argument";
    case PDM_ERR_CONFIG: return "unsupported model shape";
    case PDM_ERR_DEVICE: return "device is not a usable gfx950 GPU";
    case PDM_ERR_OOM: return "host allocation failed";
    case PDM_ERR_ALIGN: return "buffer not 256-byte aligned";
    case PDM_ERR_SIZE: return "buffer or blob too small";
    case PDM_ERR_FORMAT: return "packed blob header mismatch";
    case PDM_ERR_POS: return "position is not the cache length";
    case PDM_ERR_TOKEN: return "token out of range or input missing";
    case PDM_ERR_CTX: return "position exceeds max_ctx";
    case PDM_ERR_LAUNCH: return "HIP runtime error";
    case PDM_ERR_WATCHDOG: return "device dependency wait timed out";
    case PDM_ERR_UNBOUND: return "buffers not bound";
    default: return "unknown error";
  }
}

int pdm_query_sizes(const pdm_dims* dims, int32_t max_ctx, int32_t n_workgroups, pdm_sizes* out) {
  if (!dims || !out) return PDM_ERR_ARG;
  Plan* p = new (std::nothrow) Plan;
  if (!p) return PDM_ERR_OOM;
  Layout lay;
  int rc = build_plan(*dims, max_ctx, n_workgroups > 0 ? n_workgroups : 256, p, &lay);
  if (rc == PDM_OK) fill_sizes(*p, lay, out);
  delete p;
  return rc;
}

int pdm_describe_plan(const pdm_dims* dims, int32_t max_ctx, int32_t n_workgroups, pdm_stage_info* out,
                      int32_t cap, int32_t* n_out) {
  if (!dims || !n_out || cap < 0 || (cap > 0 && !out)) return PDM_ERR_ARG;
  Plan* p = new (std::nothrow) Plan;
  if (!p) return PDM_ERR_OOM;
  Layout lay;
  int rc = build_plan(*dims, max_ctx, n_workgroups > 0 ? n_workgroups : 256, p, &lay);
  if (rc == PDM_OK) {
    *n_out = p->n_stages;
    for (int s = 0; s < p->n_stages && s < cap; ++s) stage_info(*p, s, out + s);
  }
  delete p;
  return rc;
}

int pdm_create(const pdm_dims* dims, int32_t max_ctx, int hip_device, pdm_engine** out) {
  if (!dims || !out) return PDM_ERR_ARG;
  *out = nullptr;
  int rc = validate_dims(*dims, max_ctx);
  if (rc) return rc;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || hip_device < 0 || hip_device >= ndev) return PDM_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) return PDM_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return PDM_ERR_DEVICE;
  pdm_engine* e = new (std::nothrow) pdm_engine;
  if (!e) return PDM_ERR_OOM;
  e->dims = *dims;
  e->max_ctx = max_ctx;
  e->device = hip_device;
  e->G = prop.multiProcessorCount;
  rc = build_plan(*dims, max_ctx, e->G, &e->plan, &e->lay);
  if (rc) { delete e; return rc; }
  e->layer_len.assign(dims->n_layers, 0);
  const char* coop = std::getenv("PDM_COOPERATIVE");
  e->cooperative = coop && coop[0] == '1';
  *out = e;
  return PDM_OK;
}

int pdm_get_sizes(const pdm_engine* e, pdm_sizes* out) {
  if (!e || !out) return PDM_ERR_ARG;
  fill_sizes(e->plan, e->lay, out);
  return PDM_OK;
}

int pdm_bind(pdm_engine* e, void* weights_dev, uint64_t weight_bytes, void* kv_dev, uint64_t kv_bytes,
             void* scratch_dev, uint64_t scratch_bytes, void* trace_dev, uint64_t trace_bytes) {
  return bind_buffers(e, weights_dev, weight_bytes, kv_dev, kv_bytes, scratch_dev, scratch_bytes, trace_dev,
                      trace_bytes);
}

int pdm_bind_static(pdm_engine* e, void* weights_dev, uint64_t weight_bytes, void* kv_dev, uint64_t kv_bytes) {
  if (!e) return PDM_ERR_ARG;
  if (e->lay.scratch_bytes > PDM_STATIC_SCRATCH_BYTES) return PDM_ERR_SIZE;
  void* ws = nullptr;
  if (static_scratch(e->device, &ws) != hipSuccess || !ws) return PDM_ERR_DEVICE;
  return bind_buffers(e, weights_dev, weight_bytes, kv_dev, kv_bytes, ws, PDM_STATIC_SCRATCH_BYTES, nullptr, 0);
}

}  // extern "C"

namespace {

int bind_buffers(pdm_engine* e, void* weights_dev, uint64_t weight_bytes, void* kv_dev, uint64_t kv_bytes,
                 void* scratch_dev, uint64_t scratch_bytes, void* trace_dev, uint64_t trace_bytes) {
  if (!e || !weights_dev || !kv_dev || !scratch_dev) return PDM_ERR_ARG;
  if (!aligned(weights_dev) || !aligned(kv_dev) || !aligned(scratch_dev) || (trace_dev && !aligned(trace_dev)))
    return PDM_ERR_ALIGN;
  if (weight_bytes < e->lay.weight_bytes || kv_bytes < e->lay.kv_bytes || scratch_bytes < e->lay.scratch_bytes ||
      (trace_dev && trace_bytes < e->lay.trace_bytes))
    return PDM_ERR_SIZE;
  DeviceGuard g(e->device);
  e->w = static_cast<uint8_t*>(weights_dev);
  e->kv = static_cast<uint8_t*>(kv_dev);
  e->scratch = static_cast<uint8_t*>(scratch_dev);
  e->trace = static_cast<uint64_t*>(trace_dev);
  e->plan_dev = reinterpret_cast<Plan*>(e->scratch + e->lay.plan_off);
  absolutize(*e, &e->abs);
  const Header h = blob_header(e->dims, e->lay.weight_bytes);
  hipError_t err = hipMemcpy(e->w, &h, sizeof(h), hipMemcpyHostToDevice);
  if (err == hipSuccess) err = hipMemcpy(e->plan_dev, &e->abs, sizeof(Plan), hipMemcpyHostToDevice);
  if (err == hipSuccess) {
    // counters, status, argmax slots start at zero; epoch restarts
    uint64_t z0 = e->plan.counters, z1 = e->plan.logits_internal;
    err = hipMemset(e->scratch + z0, 0, z1 - z0);
  }
  if (err == hipSuccess)
    err = launch_rope_table(reinterpret_cast<float*>(e->abs.rope_tab), e->max_ctx, e->dims.rope, (double)e->dims.rope_base, 0);
  if (err == hipSuccess) err = hipDeviceSynchronize();
  if (err != hipSuccess) { e->bound = false; return PDM_ERR_LAUNCH; }
  e->epoch = 0;
  std::fill(e->layer_len.begin(), e->layer_len.end(), 0);
  e->bound = true;
  return PDM_OK;
}

}  // namespace

extern "C" {

int pdm_load_fp8(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert, const uint8_t* codes_dev,
                 const uint16_t* scales_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!codes_dev || !scales_dev) return PDM_ERR_ARG;
  PackTarget t[2];
  int n = 0;
  rc = pack_targets(e->dims, e->plan, tensor, layer, expert, t, &n);
  if (rc) return rc;
  if (t[0].fmt != PDM_FMT_FP8) return PDM_ERR_ARG;
  DeviceGuard g(e->device);
  for (int i = 0; i < n; ++i) {
    rc = hip_fail(launch_pack(codes_dev, scales_dev, e->w + t[i].codes, reinterpret_cast<uint16_t*>(e->w + t[i].scales),
                              t[i].m, (hipStream_t)stream));
    if (rc) return rc;
  }
  return PDM_OK;
}

int pdm_load_mxfp4(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert, const uint8_t* codes_dev,
                   const uint8_t* scales_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!codes_dev || !scales_dev) return PDM_ERR_ARG;
  PackTarget t[2];
  int n = 0;
  rc = pack_targets(e->dims, e->plan, tensor, layer, expert, t, &n);
  if (rc) return rc;
  if (t[0].fmt != PDM_FMT_MXFP4) return PDM_ERR_ARG;
  DeviceGuard g(e->device);
  const PackMap& m = t[0].m;
  rc = hip_fail(launch_pack_rows(codes_dev, e->w + t[0].codes, m, m.Kp, (hipStream_t)stream));
  if (!rc) rc = hip_fail(launch_pack_rows(scales_dev, e->w + t[0].scales, m, m.nkb, (hipStream_t)stream));
  return rc;
}

int pdm_load_raw(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert, const void* src_dev, uint64_t bytes,
                 pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!src_dev) return PDM_ERR_ARG;
  uint64_t off = 0, need = 0;
  rc = raw_target(e->dims, e->plan, tensor, layer, expert, &off, &need);
  if (rc) return rc;
  if (bytes != need) return PDM_ERR_SIZE;
  DeviceGuard g(e->device);
  return hip_fail(hipMemcpyAsync(e->w + off, src_dev, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream));
}

int pdm_load_packed_weights(pdm_engine* e, const void* blob, uint64_t bytes, int blob_on_device, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!blob) return PDM_ERR_ARG;
  if (bytes < e->lay.weight_bytes) return PDM_ERR_SIZE;
  DeviceGuard g(e->device);
  Header h{};
  if (blob_on_device) {
    if (hipMemcpy(&h, blob, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return PDM_ERR_LAUNCH;
  } else {
    std::memcpy(&h, blob, sizeof(h));
  }
  if (h.magic != kMagic || h.abi != PDM_ABI_VERSION || h.dims_hash != dims_hash(e->dims) ||
      h.weight_bytes != e->lay.weight_bytes)
    return PDM_ERR_FORMAT;
  return hip_fail(hipMemcpyAsync(e->w, blob, e->lay.weight_bytes,
                                 blob_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, (hipStream_t)stream));
}

int pdm_pack_header(const pdm_dims* dims, void* arena, uint64_t arena_bytes) {
  HostPlan hp(dims);
  if (hp.rc) return hp.rc;
  if (!arena) return PDM_ERR_ARG;
  if (arena_bytes < hp.lay.weight_bytes) return PDM_ERR_SIZE;
  const Header h = blob_header(*dims, hp.lay.weight_bytes);
  std::memcpy(arena, &h, sizeof(h));
  return PDM_OK;
}

int pdm_pack_fp8(const pdm_dims* dims, int32_t tensor, int32_t layer, int32_t expert, const uint8_t* codes,
                 const uint16_t* scales, void* arena, uint64_t arena_bytes) {
  HostPlan hp(dims);
  if (hp.rc) return hp.rc;
  if (!codes || !scales || !arena) return PDM_ERR_ARG;
  if (arena_bytes < hp.lay.weight_bytes) return PDM_ERR_SIZE;
  PackTarget t[2];
  int n = 0;
  int rc = pack_targets(*dims, *hp.p, tensor, layer, expert, t, &n);
  if (rc) return rc;
  if (t[0].fmt != PDM_FMT_FP8) return PDM_ERR_ARG;
  uint8_t* a = static_cast<uint8_t*>(arena);
  for (int i = 0; i < n; ++i) {
    const PackMap& m = t[i].m;
    uint8_t* dc = a + t[i].codes;
    uint16_t* ds = reinterpret_cast<uint16_t*>(a + t[i].scales);
    int sr = 0, sc = 0;
    // pack_src keeps columns (sc = k): a packed row is one logical row
    for (int r = 0; r < m.rows; ++r)
      if (pack_src(m, r, 0, sr, sc)) std::memcpy(dc + (size_t)r * m.Kp, codes + (size_t)sr * m.K, (size_t)m.Kp);
    const int skb = (m.K + 127) / 128;
    for (int rg = 0; rg < m.rows / 8; ++rg)
      for (int kb = 0; kb < m.nkb; ++kb)
        if (pack_src(m, rg * 8, kb * 128, sr, sc)) ds[(size_t)rg * m.nkb + kb] = scales[(size_t)(sr / 128) * skb + sc / 128];
  }
  return PDM_OK;
}

int pdm_pack_mxfp4(const pdm_dims* dims, int32_t tensor, int32_t layer, int32_t expert, const uint8_t* codes,
                   const uint8_t* scales, void* arena, uint64_t arena_bytes) {
  HostPlan hp(dims);
  if (hp.rc) return hp.rc;
  if (!codes || !scales || !arena) return PDM_ERR_ARG;
  if (arena_bytes < hp.lay.weight_bytes) return PDM_ERR_SIZE;
  PackTarget t[2];
  int n = 0;
  int rc = pack_targets(*dims, *hp.p, tensor, layer, expert, t, &n);
  if (rc) return rc;
  if (t[0].fmt != PDM_FMT_MXFP4) return PDM_ERR_ARG;
  const PackMap& m = t[0].m;
  uint8_t* a = static_cast<uint8_t*>(arena);
  int sr = 0, sc = 0;
  // whole rows: K / 2 code bytes and K / 32 scale bytes per row
  for (int r = 0; r < m.rows; ++r)
    if (pack_src(m, r, 0, sr, sc)) {
      std::memcpy(a + t[0].codes + (size_t)r * m.Kp, codes + (size_t)sr * m.Kp, (size_t)m.Kp);
      std::memcpy(a + t[0].scales + (size_t)r * m.nkb, scales + (size_t)sr * m.nkb, (size_t)m.nkb);
    }
  return PDM_OK;
}

int pdm_pack_raw(const pdm_dims* dims, int32_t tensor, int32_t layer, int32_t expert, const void* src,
                 uint64_t bytes, void* arena, uint64_t arena_bytes) {
  HostPlan hp(dims);
  if (hp.rc) return hp.rc;
  if (!src || !arena) return PDM_ERR_ARG;
  if (arena_bytes < hp.lay.weight_bytes) return PDM_ERR_SIZE;
  uint64_t off = 0, need = 0;
  int rc = raw_target(*dims, *hp.p, tensor, layer, expert, &off, &need);
  if (rc) return rc;
  if (bytes != need) return PDM_ERR_SIZE;
  std::memcpy(static_cast<uint8_t*>(arena) + off, src, bytes);
  return PDM_OK;
}

int pdm_packed_layout(const pdm_dims* dims, int32_t tensor, int32_t layer, int32_t expert, int32_t part,
                      pdm_packed_matrix* out) {
  HostPlan hp(dims);
  if (hp.rc) return hp.rc;
  if (!out) return PDM_ERR_ARG;
  PackTarget t[2];
  int n = 0;
  int rc = pack_targets(*dims, *hp.p, tensor, layer, expert, t, &n);
  if (rc) return rc;
  if (part < 0 || part >= n) return PDM_ERR_ARG;
  out->codes_offset = t[part].codes;
  out->scales_offset = t[part].scales;
  out->rows = t[part].m.rows;
  out->K = t[part].m.Kp;
  out->n_kblocks = t[part].m.nkb;
  out->parts = n;
  out->format = t[part].fmt;
  return PDM_OK;
}

int pdm_reset_cache(pdm_engine* e, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  // a new sequence also restarts the device scheduler: counters, status and
  // the argmax arrival slot go back to zero (stream-ordered, no memset node)
  DeviceGuard g(e->device);
  uint64_t z0 = e->plan.counters, z1 = e->plan.logits_internal;
  rc = hip_fail(launch_zero(e->scratch + z0, z1 - z0, (hipStream_t)stream));
  if (rc) return rc;
  e->epoch = 0;
  std::fill(e->layer_len.begin(), e->layer_len.end(), 0);
  return PDM_OK;
}

int pdm_import_kv(pdm_engine* e, int32_t layer, int32_t pos0, int32_t n, const uint16_t* rows_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  const pdm_dims& d = e->dims;
  if (layer < 0 || layer >= d.n_layers || n < 0 || (n > 0 && !rows_dev)) return PDM_ERR_ARG;
  if (pos0 < 0 || pos0 > e->layer_len[layer]) return PDM_ERR_POS;
  if ((int64_t)pos0 + n > e->max_ctx) return PDM_ERR_CTX;
  const int kvr = d.kv_lora + d.rope;
  DeviceGuard g(e->device);
  if (n > 0) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(e->abs.layers[layer].kv) + (size_t)pos0 * kvr;
    rc = hip_fail(hipMemcpyAsync(dst, rows_dev, (size_t)n * kvr * 2, hipMemcpyDeviceToDevice, (hipStream_t)stream));
    if (rc) return rc;
  }
  e->layer_len[layer] = pos0 + n;
  return PDM_OK;
}

int pdm_export_kv(const pdm_engine* e, int32_t layer, int32_t pos0, int32_t n, uint16_t* rows_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  const pdm_dims& d = e->dims;
  if (layer < 0 || layer >= d.n_layers || n < 0 || pos0 < 0 || (n > 0 && !rows_dev)) return PDM_ERR_ARG;
  if ((int64_t)pos0 + n > e->max_ctx) return PDM_ERR_CTX;
  const int kvr = d.kv_lora + d.rope;
  if (n == 0) return PDM_OK;
  DeviceGuard g(e->device);
  const uint16_t* src = reinterpret_cast<const uint16_t*>(e->abs.layers[layer].kv) + (size_t)pos0 * kvr;
  return hip_fail(hipMemcpyAsync(rows_dev, src, (size_t)n * kvr * 2, hipMemcpyDeviceToDevice, (hipStream_t)stream));
}

int pdm_decode_step(pdm_engine* e, int32_t token, int32_t pos, const uint16_t* x_in_dev, float* logits_dev,
                    int32_t* argmax_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  const pdm_dims& d = e->dims;
  if (d.vocab > 0) {
    if (token < 0 || token >= d.vocab) return PDM_ERR_TOKEN;
  } else if (!x_in_dev) {
    return PDM_ERR_TOKEN;
  } else if (reinterpret_cast<uintptr_t>(x_in_dev) & 15u) {
    return PDM_ERR_ALIGN;  // the first stage reads it in 16-byte pieces
  }
  if (pos < 0) return PDM_ERR_POS;
  if (pos >= e->max_ctx) return PDM_ERR_CTX;
  for (int l = 0; l < d.n_layers; ++l)
    if (e->layer_len[l] != pos) return PDM_ERR_POS;
  LaunchArgs a{};
  a.epoch = e->epoch + 1;
  a.token = token;
  a.pos = pos;
  a.spin_limit = e->spin_limit > 0 ? e->spin_limit : kDefaultSpin;
  a.skip_stage = e->skip_stage;
  a.n_steps = 1;
  a.x_in = x_in_dev;
  a.logits = d.vocab > 0 ? logits_dev : nullptr;
  a.argmax = d.vocab > 0 ? argmax_dev : nullptr;
  a.trace = e->trace_on ? e->trace : nullptr;
  DeviceGuard g(e->device);
  hipError_t err = launch_engine(e->plan_dev, a, e->G, e->dims.expert_format, (hipStream_t)stream, e->cooperative);
  if (err != hipSuccess) return PDM_ERR_LAUNCH;
  e->epoch = a.epoch;
  for (int l = 0; l < d.n_layers; ++l) e->layer_len[l] = pos + 1;
  return PDM_OK;
}

int pdm_decode_steps(pdm_engine* e, int32_t pos0, int32_t n_steps, const int32_t* tokens_dev, int greedy,
                     float* logits_dev, int32_t* argmax_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  const pdm_dims& d = e->dims;
  if (d.vocab <= 0 || !tokens_dev) return PDM_ERR_TOKEN;
  if (n_steps < 1 || (greedy && !argmax_dev)) return PDM_ERR_ARG;
  if (pos0 < 0) return PDM_ERR_POS;
  if ((int64_t)pos0 + n_steps > e->max_ctx) return PDM_ERR_CTX;
  for (int l = 0; l < d.n_layers; ++l)
    if (e->layer_len[l] != pos0) return PDM_ERR_POS;
  LaunchArgs a{};
  a.epoch = e->epoch + 1;
  a.pos = pos0;
  a.spin_limit = e->spin_limit > 0 ? e->spin_limit : kDefaultSpin;
  a.skip_stage = e->skip_stage;
  a.n_steps = n_steps;
  a.greedy = greedy ? 1 : 0;
  a.tokens = tokens_dev;
  a.logits = logits_dev;
  a.argmax = argmax_dev;
  a.trace = e->trace_on ? e->trace : nullptr;
  DeviceGuard g(e->device);
  hipError_t err = launch_engine(e->plan_dev, a, e->G, e->dims.expert_format, (hipStream_t)stream, e->cooperative);
  if (err != hipSuccess) return PDM_ERR_LAUNCH;
  e->epoch += (uint32_t)n_steps;
  for (int l = 0; l < d.n_layers; ++l) e->layer_len[l] = pos0 + n_steps;
  return PDM_OK;
}

int pdm_sync_status(pdm_engine* e, pdm_stream_t stream, pdm_status* out) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  DeviceGuard g(e->device);
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return PDM_ERR_LAUNCH;
  int32_t raw[8] = {0};
  if (hipMemcpy(raw, reinterpret_cast<void*>(e->abs.status), sizeof(raw), hipMemcpyDeviceToHost) != hipSuccess)
    return PDM_ERR_LAUNCH;
  const uint32_t code = (uint32_t)raw[0];
  const uint32_t ep = (uint32_t)raw[1];
  pdm_status st{};
  st.code = code ? -(int32_t)code : PDM_OK;
  st.stage = code ? raw[4] : -1;
  st.workgroup = code ? raw[5] : -1;
  st.observed = code ? raw[6] : 0;
  st.epoch = ep;
  if (out) *out = st;
  return code ? -(int32_t)code : PDM_OK;
}

int pdm_get_taps(const pdm_engine* e, pdm_taps* out) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!out) return PDM_ERR_ARG;
  std::memset(out, 0, sizeof(*out));
  const Plan& a = e->abs;
  out->hidden_dev = reinterpret_cast<const float*>(a.layers[0].xo);       // [n_layers][hidden]
  out->hidden_attn_dev = reinterpret_cast<const float*>(a.layers[0].xa);  // [n_layers][hidden]
  out->router_idx_dev = reinterpret_cast<const int32_t*>(a.layers[0].topk_idx);
  out->router_w_dev = reinterpret_cast<const float*>(a.layers[0].topk_w);
  out->logits_dev = reinterpret_cast<const float*>(a.logits_internal);
  out->trace_dev = e->trace;
  out->n_stages = a.n_stages;
  out->n_workgroups = a.G;
  out->epoch = e->epoch;
  return PDM_OK;
}

int pdm_cache_length(const pdm_engine* e, int32_t* out) {
  if (!e || !out) return PDM_ERR_ARG;
  int32_t v = e->layer_len.empty() ? 0 : e->layer_len[0];
  for (int32_t x : e->layer_len) v = x < v ? x : v;
  *out = v;
  return PDM_OK;
}

int pdm_set_debug(pdm_engine* e, int32_t spin_limit, int32_t skip_signal_stage) {
  if (!e || spin_limit < 0) return PDM_ERR_ARG;
  e->spin_limit = spin_limit > 0 ? spin_limit : kDefaultSpin;
  e->skip_stage = skip_signal_stage >= 0 ? skip_signal_stage : -1;
  return PDM_OK;
}

int pdm_set_trace(pdm_engine* e, int32_t on) {
  if (!e) return PDM_ERR_ARG;
  if (on && !e->trace) return PDM_ERR_UNBOUND;
  e->trace_on = on != 0;
  return PDM_OK;
}

// ---- batched products

namespace {

constexpr size_t kWsList = 16;                                             // int32 [kMaxUnion] slot experts
constexpr size_t kWsUw = 1280;                                             // f32 [kMaxUnion][kBatchMax]
constexpr size_t kWsH = kWsUw + (size_t)kMaxUnion * kBatchMax * 4 + 256;   // f32 [slot][B][2 F]
constexpr size_t kSlabBytes = 8 * 4 * 64 * 16;                             // staged activations of 512 columns
static_assert(kWsList + kMaxUnion * 4 <= kWsUw, "workspace regions do not overlap");

int64_t slabs_of(int64_t K) { return (K + 511) / 512; }

// Most expert slots a batched MoE call can use.
int batch_slots(const pdm_dims& d, int32_t B, bool moe) {
  return moe ? std::min(B * d.top_k, d.n_experts) + d.n_shared : 1;
}

// Bytes of the gate/up output region and of the staged-activation region,
// sized for the largest call (kBatchMax tokens, every matrix and layer kind).
void ws_sizes(const pdm_dims& d, size_t* h_bytes, size_t* xg_bytes) {
  const bool any_moe = std::any_of(d.layer_moe, d.layer_moe + d.n_layers, [](uint8_t m) { return m != 0; });
  const int n_max = any_moe ? batch_slots(d, kBatchMax, true) : 1;
  const size_t moe_h = any_moe ? (size_t)n_max * kBatchMax * 2 * d.moe_ffn : 0;
  *h_bytes = 4 * std::max(moe_h, (size_t)kBatchMax * 2 * d.ffn);
  const int64_t kmax = std::max({(int64_t)d.hidden, (int64_t)d.q_lora, (int64_t)d.kv_lora, (int64_t)d.ffn,
                                 (int64_t)d.n_heads * d.v_head, (int64_t)d.moe_ffn});
  *xg_bytes = kSlabBytes * std::max<size_t>(slabs_of(kmax), any_moe ? (size_t)n_max * slabs_of(d.moe_ffn) : 0);
}

int ensure_ws(pdm_engine* e) {
  if (e->batch_ws) return PDM_OK;
  size_t hb, xg;
  ws_sizes(e->dims, &hb, &xg);
  if (hipMalloc(&e->batch_ws, kWsH + ((hb + 255) & ~(size_t)255) + xg) != hipSuccess) {
    e->batch_ws = nullptr;
    return PDM_ERR_OOM;
  }
  return PDM_OK;
}
float* ws_h(pdm_engine* e) { return reinterpret_cast<float*>(e->batch_ws + kWsH); }
bu32x4* ws_xg(pdm_engine* e) {
  size_t hb, xg;
  ws_sizes(e->dims, &hb, &xg);
  return reinterpret_cast<bu32x4*>(e->batch_ws + kWsH + ((hb + 255) & ~(size_t)255));
}

int batch_args(const pdm_engine* e, int32_t B, const float* x_dev, const float* y_dev) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (B < 1 || B > kBatchMax || !x_dev || !y_dev) return PDM_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(x_dev) & 15u) return PDM_ERR_ALIGN;  // read in 16-byte pieces
  return PDM_OK;
}

}  // namespace

int pdm_batch_gemm(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert, int32_t part,
                   const float* x_dev, int32_t B, float* y_dev, pdm_stream_t stream) {
  int rc = batch_args(e, B, x_dev, y_dev);
  if (rc) return rc;
  PackTarget t[2];
  int n = 0;
  rc = pack_targets(e->dims, e->plan, tensor, layer, expert, t, &n);
  if (rc) return rc;
  if (part < 0 || part >= n) return PDM_ERR_ARG;
  const bool mx = t[part].fmt == PDM_FMT_MXFP4;
  DeviceGuard dg(e->device);
  if ((rc = ensure_ws(e))) return rc;
  BatchGemm g{};
  g.base = e->w;
  g.codes_off = t[part].codes;
  g.scales_off = t[part].scales;
  g.rows = t[part].m.rows;
  g.K = mx ? 2 * t[part].m.Kp : t[part].m.Kp;  // columns (MXFP4 rows hold two per byte)
  g.nkb = t[part].m.nkb;
  g.fmt = t[part].fmt;
  g.B = B;
  g.xg = ws_xg(e);
  g.y = y_dev;
  g.ldy = g.rows;
  batch_gemm_grid(g, 1);
  BatchStage sa{};
  sa.x = x_dev;
  sa.xg = ws_xg(e);
  sa.ldx = g.K;
  sa.B = B;
  sa.K = g.K;
  sa.nwin = g.slabs * 8;
  sa.z0 = y_dev;
  sa.n0 = (size_t)B * g.rows;
  sa.mx = mx ? 1 : 0;
  const hipStream_t st = (hipStream_t)stream;
  if (launch_batch_stage(sa, false, sa.nwin * 128, st) != hipSuccess) return PDM_ERR_LAUNCH;
  return launch_batch_gemm(g, 0, 1, st) == hipSuccess ? PDM_OK : PDM_ERR_LAUNCH;
}

int pdm_batch_ffn(pdm_engine* e, int32_t layer, const float* h_dev, int32_t B, const int32_t* idx_dev,
                  const float* w_dev, float* y_dev, pdm_stream_t stream) {
  int rc = batch_args(e, B, h_dev, y_dev);
  if (rc) return rc;
  const pdm_dims& d = e->dims;
  if (layer < 0 || layer >= d.n_layers) return PDM_ERR_ARG;
  const LayerPlan& L = e->plan.layers[layer];
  const bool moe = L.is_moe != 0;
  if (moe && (!idx_dev || !w_dev)) return PDM_ERR_ARG;
  DeviceGuard dg(e->device);
  if ((rc = ensure_ws(e))) return rc;
  int32_t* cnt = reinterpret_cast<int32_t*>(e->batch_ws);
  int32_t* list = reinterpret_cast<int32_t*>(e->batch_ws + kWsList);
  float* uw = reinterpret_cast<float*>(e->batch_ws + kWsUw);
  float* hb = ws_h(e);
  bu32x4* xg = ws_xg(e);
  const hipStream_t st = (hipStream_t)stream;
  const int n_slots = batch_slots(d, B, moe);
  hipError_t err = moe ? launch_batch_union(idx_dev, w_dev, B, d.top_k, d.n_experts, d.n_shared, cnt, list, uw, st)
                       : launch_batch_dense_slot(cnt, list, uw, st);
  if (err != hipSuccess) return PDM_ERR_LAUNCH;
  const Fp8Mat& gum = moe ? L.egu : L.gu;
  const Fp8Mat& dnm = moe ? L.edown : L.down;
  BatchGemm gu{};
  gu.base = e->w + (moe ? L.expert_base : 0);
  gu.stride = moe ? L.expert_stride : 0;
  // columns per row: MXFP4 expert rows hold two per code byte
  auto cols = [](const Fp8Mat& m) { return m.fmt == PDM_FMT_MXFP4 ? 2 * m.K : m.K; };
  gu.codes_off = gum.codes;
  gu.scales_off = gum.scales;
  gu.rows = gum.rows;
  gu.K = cols(gum);
  gu.nkb = gum.nkb;
  gu.fmt = gum.fmt;
  gu.B = B;
  gu.u_count = cnt;
  gu.u_list = list;
  gu.xg = xg;
  gu.y = hb;
  gu.ldy = gum.rows;
  batch_gemm_grid(gu, n_slots);
  BatchGemm dn = gu;
  dn.codes_off = dnm.codes;
  dn.scales_off = dnm.scales;
  dn.rows = dnm.rows;
  dn.K = cols(dnm);
  dn.nkb = dnm.nkb;
  dn.fmt = dnm.fmt;
  dn.y = y_dev;
  dn.ldy = d.hidden;
  batch_gemm_grid(dn, n_slots);
  // stage the input, zero the gate/up outputs of the slots in use and y
  BatchStage sx{};
  sx.x = h_dev;
  sx.xg = xg;
  sx.ldx = d.hidden;
  sx.B = B;
  sx.K = gu.K;
  sx.nwin = gu.slabs * 8;
  sx.z0 = hb;
  sx.c0 = cnt;
  sx.n0 = (size_t)B * gum.rows;
  sx.z1 = y_dev;
  sx.n1 = (size_t)B * d.hidden;
  sx.mx = gu.fmt == PDM_FMT_MXFP4 ? 1 : 0;
  if (launch_batch_stage(sx, false, sx.nwin * 128, st) != hipSuccess) return PDM_ERR_LAUNCH;
  if (launch_batch_gemm(gu, 1, n_slots, st) != hipSuccess) return PDM_ERR_LAUNCH;
  // stage the weighted SwiGLU activations of every slot for the down product
  BatchStage sa{};
  sa.x = hb;
  sa.uw = uw;
  sa.u_count = cnt;
  sa.xg = xg;
  sa.ldx = gum.rows;
  sa.B = B;
  sa.K = dn.K;
  sa.nwin = dn.slabs * 8;
  sa.mx = dn.fmt == PDM_FMT_MXFP4 ? 1 : 0;
  if (launch_batch_stage(sa, true, n_slots * sa.nwin * 128, st) != hipSuccess) return PDM_ERR_LAUNCH;
  return launch_batch_gemm(dn, 2, n_slots, st) == hipSuccess ? PDM_OK : PDM_ERR_LAUNCH;
}

// ---- batched decode step

namespace {

// Activations of a batched step for kBatchMax tokens: offsets (bytes) of each
// region in the step workspace.
struct StepWs {
  size_t x, h, t, qkv, cq, q, qlat, qpe, olat, o, rlog, idx, w, part, argv, argi, total;
};
StepWs step_ws_layout(const pdm_dims& d) {
  StepWs o{};
  size_t at = 0;
  auto take = [&](size_t floats) {
    const size_t r = at;
    at += (floats * 4 + 255) & ~(size_t)255;
    return r;
  };
  const size_t B = kBatchMax, H = d.n_heads;
  o.x = take(B * d.hidden);
  o.h = take(B * d.hidden);
  o.t = take(B * d.hidden);
  o.qkv = take(B * (d.q_lora + d.kv_lora + d.rope));
  o.cq = take(B * d.q_lora);
  o.q = take(B * H * (d.qk_nope + d.rope));
  o.qlat = take(B * H * d.kv_lora);
  o.qpe = take(B * H * d.rope);
  o.olat = take(B * H * d.kv_lora);
  o.o = take(B * H * d.v_head);
  o.rlog = take(B * std::max(1, d.n_experts));
  o.idx = take(B * 16);
  o.w = take(B * 16);
  o.part = take(B * H * kAttnChunksMax * (d.kv_lora + 2));
  o.argv = take(B * kArgPartsMax);
  o.argi = take(B * kArgPartsMax);
  o.total = at;
  return o;
}

// One batched product over a packed FP8 matrix of the plan (relative offsets).
int step_gemm(pdm_engine* e, const Fp8Mat& m, const float* x, int B, float* y, hipStream_t st) {
  BatchGemm g{};
  g.base = e->w;
  g.codes_off = m.codes;
  g.scales_off = m.scales;
  g.rows = m.rows;
  g.K = m.K;
  g.nkb = m.nkb;
  g.B = B;
  g.xg = ws_xg(e);
  g.y = y;
  g.ldy = g.rows;
  batch_gemm_grid(g, 1);
  BatchStage sa{};
  sa.x = x;
  sa.xg = ws_xg(e);
  sa.ldx = g.K;
  sa.B = B;
  sa.K = g.K;
  sa.nwin = g.slabs * 8;
  sa.z0 = y;
  sa.n0 = (size_t)B * g.rows;
  if (launch_batch_stage(sa, false, sa.nwin * 128, st) != hipSuccess) return PDM_ERR_LAUNCH;
  return launch_batch_gemm(g, 0, 1, st) == hipSuccess ? PDM_OK : PDM_ERR_LAUNCH;
}

// y[b] = M x[b] for a bf16 matrix M [rows][K] at arena offset off (router, LM
// head): on the matrix cores from kBf16MfmaMinB tokens on (no conversion of
// the weights at all), else one wave per 4 rows on the vector ALUs. The
// matrix cores' buffer addressing covers matrices below 2 GiB.
constexpr int kBf16MfmaMinB = 2;
int step_bf16(pdm_engine* e, uint64_t off, int rows, int K, const float* x, int B, float* y, hipStream_t st) {
  if (B < kBf16MfmaMinB || (uint64_t)rows * K * 2 > 0x7FFFFFFFull)
    return bs_bf16_rows(x, reinterpret_cast<const uint16_t*>(e->w + off), rows, K, B, y, st) == hipSuccess
               ? PDM_OK
               : PDM_ERR_LAUNCH;
  BatchGemm g{};
  g.base = e->w;
  g.codes_off = off;
  g.rows = rows;
  g.K = K;
  g.B = B;
  g.fmt = kFmtBf16;
  g.xg = ws_xg(e);
  g.y = y;
  g.ldy = rows;
  batch_gemm_grid(g, 1);
  BatchStage sa{};
  sa.x = x;
  sa.xg = ws_xg(e);
  sa.ldx = K;
  sa.B = B;
  sa.K = K;
  sa.nwin = g.slabs * 8;
  sa.z0 = y;
  sa.n0 = (size_t)B * rows;
  if (launch_batch_stage(sa, false, sa.nwin * 128, st) != hipSuccess) return PDM_ERR_LAUNCH;
  return launch_batch_gemm(g, 0, 1, st) == hipSuccess ? PDM_OK : PDM_ERR_LAUNCH;
}

}  // namespace

int pdm_batch_decode_step(pdm_engine* e, int32_t B, const int32_t* tokens, const int32_t* positions,
                          const uint16_t* x_in_dev, uint16_t* caches_dev, float* logits_dev, int32_t* argmax_dev,
                          float* hidden_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  const pdm_dims& d = e->dims;
  if (B < 1 || B > kBatchMax || !positions || !caches_dev) return PDM_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(caches_dev) & 15u) return PDM_ERR_ALIGN;
  BatchTokens tk{};
  for (int b = 0; b < B; ++b) {
    if (positions[b] < 0) return PDM_ERR_POS;
    if (positions[b] >= e->max_ctx) return PDM_ERR_CTX;
    tk.pos[b] = positions[b];
    if (d.vocab > 0) {
      if (!tokens || tokens[b] < 0 || tokens[b] >= d.vocab) return PDM_ERR_TOKEN;
      tk.token[b] = tokens[b];
    }
  }
  if (d.vocab > 0 && !logits_dev) return PDM_ERR_ARG;
  if (d.vocab <= 0 && !x_in_dev) return PDM_ERR_TOKEN;
  DeviceGuard dg(e->device);
  if ((rc = ensure_ws(e))) return rc;
  const StepWs L0 = step_ws_layout(d);
  if (!e->step_ws) {
    if (hipMalloc(&e->step_ws, L0.total) != hipSuccess) {
      e->step_ws = nullptr;
      return PDM_ERR_OOM;
    }
  }
  auto F = [&](size_t off) { return reinterpret_cast<float*>(e->step_ws + off); };
  float *x = F(L0.x), *h = F(L0.h), *t = F(L0.t), *qkv = F(L0.qkv), *cq = F(L0.cq), *q = F(L0.q);
  float *qlat = F(L0.qlat), *qpe = F(L0.qpe), *olat = F(L0.olat), *o = F(L0.o), *rlog = F(L0.rlog);
  int32_t* idx = reinterpret_cast<int32_t*>(e->step_ws + L0.idx);
  float* part = F(L0.part);
  float* wts = F(L0.w);
  const hipStream_t st = (hipStream_t)stream;
  const uint8_t* W = e->w;
  auto gain = [&](uint64_t off) { return reinterpret_cast<const float*>(W + off); };
  const int D = d.hidden, H = d.n_heads, dc = d.kv_lora, dr = d.rope, kvr = dc + dr;
  const int64_t seq_stride = (int64_t)d.n_layers * e->max_ctx * kvr;
  const float tau = (float)(1.0 / std::sqrt((double)(d.qk_nope + d.rope)));
  const Plan& P = e->plan;
  const float* rope_tab = reinterpret_cast<const float*>(e->abs.rope_tab);
  auto ok = [](hipError_t x2) { return x2 == hipSuccess; };
  if (!ok(bs_input(reinterpret_cast<const uint16_t*>(W + P.embed), d.vocab > 0 ? nullptr : x_in_dev, tk, B, D, x, st)))
    return PDM_ERR_LAUNCH;
  if (!ok(bs_norm(x, nullptr, false, gain(P.layers[0].attn_norm), d.rms_eps, B, D, h, st))) return PDM_ERR_LAUNCH;
  for (int l = 0; l < d.n_layers; ++l) {
    const LayerPlan& Lp = P.layers[l];
    uint16_t* cache = caches_dev + (size_t)l * e->max_ctx * kvr;
    if ((rc = step_gemm(e, Lp.qkv, h, B, qkv, st))) return rc;
    if (!ok(bs_latent(qkv, Lp.qkv.rows, d.q_lora, dc, dr, gain(Lp.q_norm), gain(Lp.kv_norm), d.rms_eps, rope_tab, tk,
                      B, cache, seq_stride, cq, st)))
      return PDM_ERR_LAUNCH;
    if ((rc = step_gemm(e, Lp.qb, cq, B, q, st))) return rc;
    if (!ok(bs_absorb(q, W + Lp.uk.codes, reinterpret_cast<const uint16_t*>(W + Lp.uk.scales), Lp.uk.nkb, H,
                      d.qk_nope, dr, dc, B, rope_tab, tk, qlat, qpe, st)))
      return PDM_ERR_LAUNCH;
    if (!ok(bs_attn(qlat, qpe, cache, seq_stride, H, dc, dr, tau, tk, B, part, olat, st))) return PDM_ERR_LAUNCH;
    if (!ok(bs_uv(olat, W + Lp.uv.codes, reinterpret_cast<const uint16_t*>(W + Lp.uv.scales), Lp.uv.nkb, H,
                  d.v_head, dc, B, o, st)))
      return PDM_ERR_LAUNCH;
    if ((rc = step_gemm(e, Lp.wo, o, B, t, st))) return rc;
    if (!ok(bs_norm(x, t, false, gain(Lp.ffn_norm), d.rms_eps, B, D, h, st))) return PDM_ERR_LAUNCH;
    if (Lp.is_moe) {
      if ((rc = step_bf16(e, Lp.router, d.n_experts, D, h, B, rlog, st))) return rc;
      if (!ok(bs_topk(rlog, B, d.n_experts, d.top_k, idx, wts, st))) return PDM_ERR_LAUNCH;
    }
    if ((rc = pdm_batch_ffn(e, l, h, B, Lp.is_moe ? idx : nullptr, Lp.is_moe ? wts : nullptr, t, stream))) return rc;
    const float* next = l + 1 < d.n_layers ? gain(P.layers[l + 1].attn_norm) : (d.vocab > 0 ? gain(P.final_norm) : nullptr);
    if (!ok(bs_norm(x, t, true, next, d.rms_eps, B, D, next ? h : nullptr, st))) return PDM_ERR_LAUNCH;
    if (hidden_dev && !ok(hipMemcpyAsync(hidden_dev + (size_t)l * B * D, x, (size_t)B * D * 4,
                                         hipMemcpyDeviceToDevice, st)))
      return PDM_ERR_LAUNCH;
  }
  if (d.vocab > 0) {
    if ((rc = step_bf16(e, P.lm_head, d.vocab, D, h, B, logits_dev, st))) return rc;
    if (argmax_dev && !ok(bs_argmax(logits_dev, B, d.vocab, F(L0.argv), reinterpret_cast<int32_t*>(e->step_ws + L0.argi),
                                    argmax_dev, st)))
      return PDM_ERR_LAUNCH;
  }
  return PDM_OK;
}

int pdm_dsa_index_scores(const float* q_dev, const float* w_dev, const uint16_t* k_dev, int32_t n, int32_t HI,
                         int32_t dI, float* scores_dev, pdm_stream_t stream) {
  if (!q_dev || !w_dev || !k_dev || !scores_dev || n < 0) return PDM_ERR_ARG;
  if (HI < 16 || HI > 64 || HI % 16 || dI < 32 || dI > 256 || dI % 32) return PDM_ERR_CONFIG;
  if (reinterpret_cast<uintptr_t>(k_dev) & 15) return PDM_ERR_ALIGN;
  return dsa_scores(q_dev, w_dev, k_dev, n, HI, dI, scores_dev, (hipStream_t)stream) == hipSuccess ? PDM_OK : PDM_ERR_LAUNCH;
}

uint64_t pdm_dsa_topk_work_bytes(int32_t n) { return dsa_topk_work_bytes(n); }

int pdm_dsa_topk(const float* scores_dev, int32_t n, int32_t k, int32_t* idx_dev, void* work_dev,
                 uint64_t work_bytes, pdm_stream_t stream) {
  if (!scores_dev || !idx_dev || !work_dev || n < 0 || k < 0) return PDM_ERR_ARG;
  if (work_bytes < dsa_topk_work_bytes(n)) return PDM_ERR_SIZE;
  return dsa_topk(scores_dev, n, k, idx_dev, static_cast<uint32_t*>(work_dev), (hipStream_t)stream) == hipSuccess
             ? PDM_OK
             : PDM_ERR_LAUNCH;
}

uint64_t pdm_dsa_attention_work_bytes(int32_t H, int32_t kv_lora) {
  if (H < 1 || kv_lora < 1) return 0;
  return (uint64_t)H * kAttnChunksMax * (kv_lora + 2) * 4;
}

int pdm_dsa_attention(const float* q_lat_dev, const float* q_pe_dev, const uint16_t* cache_dev, int32_t cache_rows,
                      const int32_t* sel_dev, int32_t n_sel, int32_t H, int32_t kv_lora, int32_t rope, float tau,
                      float* work_dev, uint64_t work_bytes, float* o_lat_dev, pdm_stream_t stream) {
  if (!q_lat_dev || !q_pe_dev || !cache_dev || !sel_dev || !work_dev || !o_lat_dev) return PDM_ERR_ARG;
  if (n_sel < 1 || H < 1 || cache_rows < 1) return PDM_ERR_ARG;
  if (kv_lora != 128 && kv_lora != 256 && kv_lora != 512) return PDM_ERR_CONFIG;
  const int kvr = kv_lora + rope;
  if (rope < 0 || kvr % 32 || kvr > 640) return PDM_ERR_CONFIG;
  if (reinterpret_cast<uintptr_t>(cache_dev) & 15) return PDM_ERR_ALIGN;
  if (work_bytes < pdm_dsa_attention_work_bytes(H, kv_lora)) return PDM_ERR_SIZE;
  BatchTokens tk{};
  tk.pos[0] = n_sel - 1;  // the attention's positions are the list's entries
  return bs_attn(q_lat_dev, q_pe_dev, cache_dev, 0, H, kv_lora, rope, tau, tk, 1, work_dev, o_lat_dev,
                 (hipStream_t)stream, sel_dev, 0, cache_rows) == hipSuccess
             ? PDM_OK
             : PDM_ERR_LAUNCH;
}

int pdm_destroy(pdm_engine* e) {
  if (!e) return PDM_ERR_ARG;
  if (e->batch_ws || e->step_ws) {
    DeviceGuard g(e->device);
    if (e->batch_ws) (void)hipFree(e->batch_ws);
    if (e->step_ws) (void)hipFree(e->step_ws);
  }
  delete e;
  return PDM_OK;
}

}  // extern "C"
