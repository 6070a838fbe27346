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
// Device address of the library's static scratch array on `device`
// (PDM_STATIC_SCRATCH_BYTES), looked up once per device.
hipError_t static_scratch(int device, void** ptr);

}  // namespace pdm
