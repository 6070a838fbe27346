// C ABI of the persistent decode engine (declared in include/pdm.h).
//
// Host side only: argument validation, buffer binding, the offline packer
// entry points and one kernel launch per decode step. No compute of the step
// happens here.
#include <hip/hip_runtime.h>

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
  fs(a->rope_tab); fs(a->counters); fs(a->status); fs(a->lm_best); fs(a->logits_internal); fs(a->x0);
  a->trace = reinterpret_cast<uint64_t>(e.trace);
  for (int l = 0; l < e.dims.n_layers; ++l) {
    LayerPlan& L = a->layers[l];
    fw(L.attn_norm); fw(L.q_norm); fw(L.kv_norm); fw(L.ffn_norm);
    fm(L.qkv); fm(L.qb); fm(L.ukT); fm(L.uv); fm(L.wo);
    if (!L.is_moe) { fm(L.gu); fm(L.down); }
    else { fw(L.router); fw(L.expert_base); }  // egu / edown stay relative to an expert block
    L.kv += K;
    fs(L.qkv_raw); fs(L.q); fs(L.ql); fs(L.attn_part); fs(L.o); fs(L.xa); fs(L.act);
    fs(L.router_logits); fs(L.xo); fs(L.topk_idx); fs(L.topk_w);
  }
}

int check_engine(const pdm_engine* e, bool need_bound) {
  if (!e) return PDM_ERR_ARG;
  if (need_bound && !e->bound) return PDM_ERR_UNBOUND;
  return PDM_OK;
}

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
  Header h{};
  h.magic = kMagic;
  h.abi = PDM_ABI_VERSION;
  h.dims_hash = dims_hash(e->dims);
  h.weight_bytes = e->lay.weight_bytes;
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

int pdm_load_fp8(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert, const uint8_t* codes_dev,
                 const uint16_t* scales_dev, pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!codes_dev || !scales_dev) return PDM_ERR_ARG;
  const pdm_dims& d = e->dims;
  if (layer < 0 || layer >= d.n_layers) return PDM_ERR_ARG;
  const LayerPlan& L = e->abs.layers[layer];
  const int H = d.n_heads, D = d.hidden, qkh = d.qk_nope + d.rope, kvr = d.kv_lora + d.rope;
  const bool moe = L.is_moe != 0;
  PackMap m{};
  m.dn = d.qk_nope; m.dv = d.v_head; m.dc = d.kv_lora;
  // dst offsets are absolute addresses (base 0) or relative to an expert block
  auto into = [&](const Fp8Mat& dst, uint64_t base) {
    return hip_fail(launch_pack(codes_dev, scales_dev, reinterpret_cast<uint8_t*>(base + dst.codes),
                                reinterpret_cast<uint16_t*>(base + dst.scales), m, (hipStream_t)stream));
  };
  auto set = [&](int mode, int N, int K, const Fp8Mat& dst, int row0, int which) {
    m.mode = mode; m.N = N; m.K = K; m.rows = dst.rows; m.Kp = dst.K; m.nkb = dst.nkb; m.row0 = row0; m.which = which;
  };
  DeviceGuard g(e->device);
  const uint64_t zero = 0;
  if (expert >= 0) {
    if (!moe || expert >= d.n_experts + d.n_shared) return PDM_ERR_ARG;
    const uint64_t blk = L.expert_base + (uint64_t)expert * L.expert_stride;
    switch (tensor) {
      case PDM_T_W_GATE: set(3, d.moe_ffn, D, L.egu, 0, 0); return into(L.egu, blk);
      case PDM_T_W_UP: set(3, d.moe_ffn, D, L.egu, 0, 1); return into(L.egu, blk);
      case PDM_T_W_DOWN: set(0, D, d.moe_ffn, L.edown, 0, 0); return into(L.edown, blk);
      default: return PDM_ERR_ARG;
    }
  }
  switch (tensor) {
    case PDM_T_WQ_A: set(0, d.q_lora, D, L.qkv, 0, 0); return into(L.qkv, zero);
    case PDM_T_WKV_A: set(0, kvr, D, L.qkv, d.q_lora, 0); return into(L.qkv, zero);
    case PDM_T_WQ_B: set(0, H * qkh, d.q_lora, L.qb, 0, 0); return into(L.qb, zero);
    case PDM_T_WKV_B: {
      set(1, H * (d.qk_nope + d.v_head), d.kv_lora, L.ukT, 0, 0);
      rc = into(L.ukT, zero);
      if (rc) return rc;
      set(2, H * (d.qk_nope + d.v_head), d.kv_lora, L.uv, 0, 0);
      return into(L.uv, zero);
    }
    case PDM_T_WO: set(0, D, H * d.v_head, L.wo, 0, 0); return into(L.wo, zero);
    case PDM_T_W_GATE: if (moe) return PDM_ERR_ARG; set(3, d.ffn, D, L.gu, 0, 0); return into(L.gu, zero);
    case PDM_T_W_UP: if (moe) return PDM_ERR_ARG; set(3, d.ffn, D, L.gu, 0, 1); return into(L.gu, zero);
    case PDM_T_W_DOWN: if (moe) return PDM_ERR_ARG; set(0, D, d.ffn, L.down, 0, 0); return into(L.down, zero);
    default: return PDM_ERR_ARG;
  }
}

int pdm_load_raw(pdm_engine* e, int32_t tensor, int32_t layer, int32_t expert, const void* src_dev, uint64_t bytes,
                 pdm_stream_t stream) {
  int rc = check_engine(e, true);
  if (rc) return rc;
  if (!src_dev || expert >= 0) return PDM_ERR_ARG;
  const pdm_dims& d = e->dims;
  uint64_t dst = 0, need = 0;
  if (tensor == PDM_T_EMBED || tensor == PDM_T_LM_HEAD || tensor == PDM_T_FINAL_NORM) {
    if (d.vocab <= 0) return PDM_ERR_ARG;
    if (tensor == PDM_T_EMBED) { dst = e->abs.embed; need = (uint64_t)d.vocab * d.hidden * 2; }
    else if (tensor == PDM_T_LM_HEAD) { dst = e->abs.lm_head; need = (uint64_t)d.vocab * d.hidden * 2; }
    else { dst = e->abs.final_norm; need = (uint64_t)d.hidden * 4; }
  } else {
    if (layer < 0 || layer >= d.n_layers) return PDM_ERR_ARG;
    const LayerPlan& L = e->abs.layers[layer];
    switch (tensor) {
      case PDM_T_ATTN_NORM: dst = L.attn_norm; need = (uint64_t)d.hidden * 4; break;
      case PDM_T_Q_NORM: dst = L.q_norm; need = (uint64_t)d.q_lora * 4; break;
      case PDM_T_KV_NORM: dst = L.kv_norm; need = (uint64_t)d.kv_lora * 4; break;
      case PDM_T_FFN_NORM: dst = L.ffn_norm; need = (uint64_t)d.hidden * 4; break;
      case PDM_T_ROUTER:
        if (!L.is_moe) return PDM_ERR_ARG;
        dst = L.router; need = (uint64_t)d.n_experts * d.hidden * 2; break;
      default: return PDM_ERR_ARG;
    }
  }
  if (bytes != need) return PDM_ERR_SIZE;
  DeviceGuard g(e->device);
  return hip_fail(hipMemcpyAsync(reinterpret_cast<void*>(dst), src_dev, bytes, hipMemcpyDeviceToDevice,
                                 (hipStream_t)stream));
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
  a.x_in = x_in_dev;
  a.logits = d.vocab > 0 ? logits_dev : nullptr;
  a.argmax = d.vocab > 0 ? argmax_dev : nullptr;
  a.trace = e->trace_on ? e->trace : nullptr;
  DeviceGuard g(e->device);
  hipError_t err = launch_engine(e->plan_dev, a, e->G, (hipStream_t)stream, e->cooperative);
  if (err != hipSuccess) return PDM_ERR_LAUNCH;
  e->epoch = a.epoch;
  for (int l = 0; l < d.n_layers; ++l) e->layer_len[l] = pos + 1;
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
  return code ? PDM_ERR_WATCHDOG : PDM_OK;
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

int pdm_destroy(pdm_engine* e) {
  if (!e) return PDM_ERR_ARG;
  delete e;
  return PDM_OK;
}

}  // extern "C"
