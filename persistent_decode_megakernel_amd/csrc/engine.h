// Kernel launch interface between the C ABI (api.cpp) and the device code.
#pragma once

#include <hip/hip_runtime.h>

#include "pdm_internal.h"

namespace pdm {

// Per-step arguments of the persistent kernel (passed by value).
struct LaunchArgs {
  uint32_t epoch;        // step counter since bind; counters target epoch * arrivals
  int32_t token;         // input token (configs with a vocabulary)
  int32_t pos;           // position of the new token == cache length
  int32_t spin_limit;    // polls before a dependency wait gives up
  int32_t skip_stage;    // debug: workgroup 0 does not signal this stage (-1 none)
  int32_t pad;
  const uint16_t* x_in;  // bf16 hidden input of a bare layer stack
  float* logits;         // optional logits output
  int32_t* argmax;       // optional argmax output
  uint64_t* trace;       // optional trace records
};

// Row/column map of the offline packer (see engine.hip, pack_codes_kernel).
struct PackMap {
  int mode, N, K, rows, Kp, nkb, row0, dn, dv, dc, which;
};

hipError_t launch_engine(const Plan* plan_dev, const LaunchArgs& a, int G, hipStream_t stream, bool cooperative);
hipError_t launch_rope_table(float* tab, int max_ctx, int rope, double base, hipStream_t stream);
hipError_t launch_pack(const uint8_t* src_codes, const uint16_t* src_scales, uint8_t* dst_codes,
                       uint16_t* dst_scales, const PackMap& m, hipStream_t stream);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace pdm
