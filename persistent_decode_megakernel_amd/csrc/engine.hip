// Persistent decode engine kernel for gfx950.
//
// One launch runs one batch-1 decode step of the MLA + MoE stack. The grid is
// one 512-thread workgroup per compute unit; every workgroup walks the same
// ordered stage list (the plan) and takes a fixed share of each stage. Stages
// are ordered by striped arrival counters in device memory: a workgroup
// finishing a stage bumps one counter, a workgroup starting a stage that reads
// another stage's output spins until that stage's counters reach epoch * count.
// This replaces kernel boundaries between operators, the central idea of the
// TileRT engine kernel (SemiAnalysis, "Ultra-High Interactivity on NVIDIA
// GPUs? - TileRT InferenceX", how-it-works section: one persistent kernel,
// operators as tile tasks, no per-operator launch or teardown).
//
// Cross-workgroup data (activations, the new cache row, counters) moves only
// through agent-coherent loads and stores (sc1: they bypass the per-XCD L2s'
// non-coherent copies), so no L2 writeback or invalidate is needed per stage.
// Weights and older cache rows are immutable during a launch and use ordinary
// cached loads.
//
// GEMV stages (every weight product at batch 1 is a matrix-vector product)
// stream FP8 e4m3 weights with 16-byte loads per lane, convert them in
// registers with the hardware OCP-FP8 conversion, multiply by fp32
// activations staged in LDS and reduce with DPP cross-lane adds. M = 1 is not
// a dense contraction, so MFMA is not used there.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pdm_internal.h"
#include "engine.h"

namespace pdm {
namespace {

constexpr int kUnroll = 5;  // 1 KB units in flight per wave and buffer (FP8, bf16 and MXFP4 alike)
constexpr int kEarlyBatches = 1;       // unit batches per wave issued before a stage's dependency wait
// The last wave of a workgroup polls the dependency counters and issues no
// load before the wait: loads complete in order per wave, so a poll issued
// behind a batch of weight loads would only return after them.
constexpr int kPollWave = kWaves - 1;
constexpr int kPreThreads = kPollWave * 64;  // threads that may issue loads before a wait
static_assert((512 + 128) / 2 <= kPreThreads, "cache-row pairs fit the loading threads");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache-policy operand of loads: sc1, the policy of a relaxed agent-scope
// atomic load, for data written this step by other workgroups.
constexpr unsigned kCpolSc1 = 16;

// Every device pointer of the plan is global memory. Accessing it through an
// address_space(1) pointer makes the compiler emit global (not flat) memory
// instructions, which only count against vmcnt; flat ones also count against
// lgkmcnt and would make every LDS read wait for all weight loads in flight.
#define GLOBAL_AS __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const GLOBAL_AS T* gp(const T* p) { return (const GLOBAL_AS T*)p; }
template <class T>
__device__ __forceinline__ GLOBAL_AS T* gpw(T* p) { return (GLOBAL_AS T*)p; }
template <class T>
__device__ __forceinline__ T gld(const T* p) { return *gp(p); }
// Copy a plan struct out of global memory word by word (C++ copy constructors
// cannot bind address-space-qualified objects); unused words are dropped.
template <class T>
__device__ __forceinline__ T load_plan(const GLOBAL_AS T* p) {
  static_assert(sizeof(T) % 4 == 0, "plan structs are word-sized");
  T v;
  const GLOBAL_AS uint32_t* src = reinterpret_cast<const GLOBAL_AS uint32_t*>(p);
  uint32_t* dst = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) dst[i] = src[i];
  return v;
}
template <class T>
__device__ __forceinline__ void gst(T* p, T v) { *gpw(p) = v; }

// Weight matrix of one expert slot: FP8 codes and their block scales.
struct __align__(16) SlotRef {
  const uint8_t* codes;
  const uint8_t* scales;  // bf16 block scales (FP8) or e8m0 bytes (MXFP4)
};

struct __align__(16) Smem {
  float x[kXMax];                 // staged input vector(s) of the current stage
  float part[kWaves][kRowChunk];  // per-wave row partial sums
  SlotRef slot[kMaxSlots];        // weight matrices of the expert slots (one 16-byte LDS read each)
  float slot_w[kMaxSlots];
  int slot_act[kMaxSlots];        // act offset of each slot
  int route_idx[kMaxSlots];       // top-k experts of the current MoE layer
  float route_w[kMaxSlots];       // their normalised weights
  float red[2 * kWaves];
  float nred[kWaves];             // per-wave sums of squares of the last normalised staging
  int ired[2 * kWaves];
  uint64_t t_entry, t_enter, t_ready;  // stage entered, dependency wait entered, wait done
  uint64_t t_mark[3];             // input staged, weights consumed, epilogue done
  int abort;
  int claim;                      // next free unit batch of the current GEMV row chunk
  int slots_ready;                // the routed slot tables of the current MoE gate/up stage are set
  int last;                       // this workgroup arrived last at the LM head
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The thread and lane index as values the compiler cannot see through (an
// empty asm that claims to change them): the MXFP4 stage code uses them so
// that what it derives from them is computed in the stage, not hoisted out of
// the step loop to the kernel entry, where each value would hold a register
// for the whole kernel (the hoisting pays for the FP8 stages; for the two
// MXFP4 stages it made the kernel run out of registers).
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int opaque_lane() { return opaque_tid() & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh_i(const int* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh_u(const uint32_t* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(gpw(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_i(int* p, int v) {
  __hip_atomic_store(gpw(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(gpw(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this thread issued has completed.
__device__ __forceinline__ void mem_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// v as a bf16 high part plus the bf16 of the remainder
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}
__device__ __forceinline__ uint32_t pack_bf16x2(__bf16 a, __bf16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

constexpr int kMH = kHeadGroup;  // heads per MFMA tile (unit heads padded to kMH)

// Round an fp32 value to the nearest bf16 value (ties to even), kept in fp32.
__device__ __forceinline__ float round_bf16(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  return __builtin_bit_cast(float, u);
}
__device__ __forceinline__ uint16_t bf16_bits(float v) {
  return (uint16_t)(__builtin_bit_cast(uint32_t, round_bf16(v)) >> 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// xor 1, xor 2 (quad_perm), then mirror within 8 and within 16 lanes
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}
// sum over the 64 lanes, returned uniform
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
// minimum over the 64 lanes of an int, returned uniform
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppXor1, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppXor2, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// sum within aligned groups of `gs` lanes (gs a power of two <= 64); every lane gets its group sum
__device__ __forceinline__ float group_sum(float v, int gs) {
  if (gs >= 2) v += dpp<kDppXor1>(v);
  if (gs >= 4) v += dpp<kDppXor2>(v);
  if (gs >= 8) v += dpp<kDppHalfMirror>(v);
  if (gs >= 16) v += dpp<kDppMirror>(v);
  if (gs >= 32) v += __shfl_xor(v, 16);
  if (gs >= 64) v += __shfl_xor(v, 32);
  return v;
}

// block-wide sum (all 512 threads participate); result in every thread

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// ------------------------------------------------------------------ sync

struct Ctx {
  const GLOBAL_AS Plan* P;  // plan in global memory: uniform reads become scalar loads
  LaunchArgs A;             // with the current step's epoch, position, token and outputs
  uint32_t epoch0;          // epoch of the launch's first step
  int G;
  int wg;
};

// The status word holds (epoch << 32) | -code of the first failure; a
// failure of any step of this launch (epoch >= epoch0) aborts every wait.
__device__ __forceinline__ bool status_aborts(const Ctx& c, unsigned long long v) {
  return (uint32_t)v != 0u && (int)((uint32_t)(v >> 32) - c.epoch0) >= 0;
}

__device__ __forceinline__ int* counter_ptr(const Ctx& c, int stage, int stripe) {
  return reinterpret_cast<int*>(c.P->counters) + ((size_t)stage * kStripes + stripe) * kCounterStride;
}
__device__ __forceinline__ int stripe_count(int G, int stripe) { return (G - stripe + kStripes - 1) / kStripes; }

// Record a failure (a dependency-wait timeout, or a bad token) in the status
// word (first one wins). Scalar arguments only: a by-reference argument of a
// non-inlined call would force the caller's structs into scratch memory.
__device__ __noinline__ void set_status(uint64_t status, uint32_t epoch, int code, int wg, int stage, int observed) {
  GLOBAL_AS unsigned long long* st = (GLOBAL_AS unsigned long long*)status;
  unsigned long long mine = ((unsigned long long)epoch << 32) | (unsigned)(-code);
  unsigned long long cur = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)(cur >> 32) != epoch || (uint32_t)cur == 0u) {
    if (__hip_atomic_compare_exchange_strong(st, &cur, mine, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
      int* det = reinterpret_cast<int*>(status) + 4;
      st_coh_i(det + 0, stage);
      st_coh_i(det + 1, wg);
      st_coh_i(det + 2, observed);
    }
  }
}

// Wait until stage `s` is complete in every workgroup. Returns false when the
// step was aborted (watchdog). All threads of the workgroup must call it.
__device__ __forceinline__ bool wait_stage(const Ctx& c, Smem& sm, int s, int my_stage) {
  if (threadIdx.x == 0) {
    sm.abort = 0;
    if (c.A.trace) {
      sm.t_enter = wall_clock64();
      sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = 0;
    }
  }
  if (s >= 0 && wave_id() == kPollWave) {
    const int lane = lane_id();
    const int* ctr = counter_ptr(c, s, lane & (kStripes - 1));
    // counters grow by stripe_count per step: compare modulo 2^32
    const uint32_t target = c.A.epoch * (uint32_t)stripe_count(c.G, lane & (kStripes - 1));
    const GLOBAL_AS unsigned long long* st = gp(reinterpret_cast<const unsigned long long*>(c.P->status));
    const bool poll_ctr = lane < kStripes && lane < c.G;
    int spins = 0;
    while (true) {
      bool ok = true;
      int seen = 0;
      if (poll_ctr) { seen = ld_coh_i(ctr); ok = (int)((uint32_t)seen - target) >= 0; }
      bool abort = false;
      if (lane == kStripes) {
        unsigned long long v = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        abort = status_aborts(c, v);
      }
      if (__any(abort)) { if (lane == 0) sm.abort = 1; break; }
      if (__all(ok)) break;
      if (++spins > c.A.spin_limit) {
        if (!ok) set_status(c.P->status, c.A.epoch, PDM_ERR_WATCHDOG, c.wg, my_stage, seen);
        if (lane == 0) sm.abort = 1;
        break;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && c.A.trace) sm.t_ready = wall_clock64();
  return sm.abort == 0;
}

// Wait until workgroups [w0, w1] of G have finished stage `s` this step: each
// workgroup's completion flag holds the epoch of the last step in which it
// finished the stage. The polling wave samples up to 256 flags per round (4
// per lane, loaded together) and the status word. An empty range (w0 > w1)
// or s < 0 waits for nothing. All threads of the workgroup must call it.
__device__ __forceinline__ bool wait_flags(const Ctx& c, Smem& sm, int s, int w0, int w1, int my_stage) {
  if (threadIdx.x == 0) {
    sm.abort = 0;
    if (c.A.trace) {
      sm.t_enter = wall_clock64();
      sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = 0;
    }
  }
  if (s >= 0 && w0 <= w1 && wave_id() == kPollWave) {
    const int lane = lane_id();
    const int n = w1 - w0 + 1;
    const uint32_t* f = reinterpret_cast<const uint32_t*>(c.P->flags) + (size_t)s * c.G + w0;
    const GLOBAL_AS unsigned long long* st = gp(reinterpret_cast<const unsigned long long*>(c.P->status));
    int spins = 0;
    while (true) {
      uint32_t v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = lane + 64 * k < n ? ld_coh_u(f + lane + 64 * k) : c.A.epoch;
      unsigned long long sv = lane == 0 ? __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
      bool ok = true;
      uint32_t seen = c.A.epoch;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((int)(v[k] - c.A.epoch) < 0) { ok = false; seen = v[k]; }
      for (int i = lane + 256; i < n; i += 64) {  // ranges beyond 256 workgroups
        const uint32_t x = ld_coh_u(f + i);
        if ((int)(x - c.A.epoch) < 0) { ok = false; seen = x; }
      }
      const bool abort = lane == 0 && status_aborts(c, sv);
      if (__any(abort)) { if (lane == 0) sm.abort = 1; break; }
      if (__all(ok)) break;
      if (++spins > c.A.spin_limit) {
        if (!ok) set_status(c.P->status, c.A.epoch, PDM_ERR_WATCHDOG, c.wg, my_stage, (int)seen);
        if (lane == 0) sm.abort = 1;
        break;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && c.A.trace) sm.t_ready = wall_clock64();
  return sm.abort == 0;
}

// Intra-stage trace mark i (0 input staged, 1 weights consumed (attention:
// blocks done), 2 epilogue done). GEMV stages carry the staged time in a
// register and write it with mark 1.
__device__ __forceinline__ void mark(const Ctx& c, Smem& sm, int i) {
  if (c.A.trace && threadIdx.x == 0) sm.t_mark[i] = wall_clock64();
}

__device__ __forceinline__ void signal_stage(const Ctx& c, Smem& sm, int s) {
  mem_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!(s == c.A.skip_stage && c.wg == 0)) {
      __hip_atomic_fetch_add(gpw(counter_ptr(c, s, c.wg & (kStripes - 1))), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      st_coh_u(reinterpret_cast<uint32_t*>(c.P->flags) + (size_t)s * c.G + c.wg, c.A.epoch);
    }
    if (c.A.trace) {
      GLOBAL_AS uint64_t* t = gpw(reinterpret_cast<uint64_t*>(c.A.trace) + ((size_t)s * c.G + c.wg) * kTraceWords);
      t[0] = sm.t_enter;
      t[1] = sm.t_ready;
      t[2] = wall_clock64();
      t[3] = c.A.epoch;
      t[4] = sm.t_mark[0];
      t[5] = sm.t_mark[1];
      t[6] = sm.t_mark[2];
      t[7] = sm.t_entry;
    }
  }
}

// ------------------------------------------------------------------ GEMV core

// Addressing of one GEMV stage. A "matrix" may be split into slots: row slots
// (rows [j << lg, (j+1) << lg) come from slot j's matrix) or K slots (bytes
// [j << lg, (j+1) << lg) of every row come from slot j's matrix).
struct Gemv {
  const uint8_t* codes;     // slot-less matrix
  const uint16_t* scales;
  int Kb;                   // bytes per logical row (all slots concatenated for K slots)
  int nkb;                  // scale blocks per row of one (slot) matrix
  int slot_mode;            // 0 none, 1 row slots, 2 K slots
  int lg_slot;
  int slot_Kb;              // bytes per row of one slot matrix
  int lg_rpv;               // rows per input vector = 1 << lg_rpv (31: one shared vector)
  int vbase;                // first staged vector
  int xK;                   // floats per staged vector
  // two-segment row map (SLOT 3): local rows [0, seg_n1) are row slot rows
  // seg_p1 + r, the rest seg_p2 + (r - seg_n1); with `split` only the first
  // segment's addresses are known before prep
  int seg_n1, seg_p1, seg_p2;
  int split;
};

// Address of the 16 bytes a lane reads for (row, byte offset b) and of its
// scale: FP8 (EB 1) a bf16 block scale, one per 8 rows and 128 bytes; MXFP4
// (EB 0, slot matrices only) the e8m0 byte of its 32 elements (its 16 bytes).
template <int EB>
__device__ __forceinline__ const uint8_t* scale_ptr(const uint8_t* scales, int nkb, int row, int b) {
  if constexpr (EB == 0) return scales + (size_t)row * nkb + (b >> 4);
  return reinterpret_cast<const uint8_t*>(reinterpret_cast<const uint16_t*>(scales) + (size_t)(row >> 3) * nkb +
                                          (b >> 7));
}
template <int EB, int SLOT>
__device__ __forceinline__ void unit_ptr_t(const Gemv& g, const Smem& sm, int row, int b,
                                           const uint8_t*& cp, const uint8_t*& sp) {
  static_assert(EB != 0 || SLOT != 0, "MXFP4 matrices are expert slots");
  if constexpr (SLOT == 0) {
    cp = g.codes + (size_t)row * g.Kb + b;
    if (EB == 1) sp = scale_ptr<1>(reinterpret_cast<const uint8_t*>(g.scales), g.nkb, row, b);
  } else if constexpr (SLOT == 1 || SLOT == 3) {
    int pr = row;
    if constexpr (SLOT == 3) pr = row < g.seg_n1 ? g.seg_p1 + row : g.seg_p2 + (row - g.seg_n1);
    int j = pr >> g.lg_slot;
    int rr = pr & ((1 << g.lg_slot) - 1);
    const SlotRef sr = sm.slot[j];
    cp = sr.codes + (size_t)rr * g.slot_Kb + b;
    if (EB != 2) sp = scale_ptr<EB>(sr.scales, g.nkb, rr, b);
  } else {
    int j = b >> g.lg_slot;
    int bb = b & ((1 << g.lg_slot) - 1);
    const SlotRef sr = sm.slot[j];
    cp = sr.codes + (size_t)row * g.slot_Kb + bb;
    if (EB != 2) sp = scale_ptr<EB>(sr.scales, g.nkb, row, bb);
  }
}

// A staged input vector sits in LDS permuted within each block of 1024
// floats: float k (k = 16 l + 4 i + e in its block) is stored at float
// 256 i + 4 l + e. The 16 floats a lane multiplies with its 16 FP8 weight
// bytes are then four float4 reads 1 KB apart, and the lanes of a wave read
// consecutive float4s (no LDS bank conflicts; with the plain order the lanes'
// float4s were 64 bytes apart). Vectors of K floats occupy K rounded up to a
// multiple of 1024; groups of 16 (FP8) or 8 (bf16) floats stay together.
static_assert(kXMax % 1024 == 0, "staged vectors occupy whole 1024-float blocks");
__device__ __forceinline__ int xperm(int k) {
  return (k & ~1023) | (((k >> 2) & 3) << 8) | (((k >> 4) & 63) << 2) | (k & 3);
}
// MXFP4 stages stage their input in blocks of 2048 floats instead (a lane's
// 16 code bytes hold 32 elements): float k = 32 l + 4 i + e of a block at
// float 256 i + 4 l + e, so the lane's eight float4 reads are again 1 KB apart
// and the lanes of a wave read consecutive float4s.
static_assert(kXMax % 2048 == 0, "MXFP4-staged vectors occupy whole 2048-float blocks");
__device__ __forceinline__ int xperm4(int k) {
  return (k & ~2047) | (((k >> 2) & 7) << 8) | (((k >> 5) & 63) << 2) | (k & 3);
}
// xperm (xperm4 for EB 0) of a group start: k a multiple of 16 (FP8 units),
// of 8 (bf16 units) or of 32 (MXFP4 units)
template <int EB>
__device__ __forceinline__ int xperm_group(int k) {
  if constexpr (EB == 0) return (k & ~2047) | ((k >> 3) & 252);
  else if constexpr (EB == 1) return (k & ~1023) | ((k >> 2) & 252);
  else return (k & ~1023) | ((k & 8) << 6) | ((k >> 2) & 252);
}

// dot of one lane's 16 bytes with the staged input; xs = sm.x + xperm(k0)
// for the lane's first input float k0
template <int EB>
__device__ __forceinline__ float unit_dot(const u32x4& w, const float* xs) {
  const float4* x4 = reinterpret_cast<const float4*>(xs);
  float acc = 0.f;
  if constexpr (EB == 1) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      float4 xv = x4[64 * i];
      acc = fmaf(lo[0], xv.x, acc);
      acc = fmaf(lo[1], xv.y, acc);
      acc = fmaf(hi[0], xv.z, acc);
      acc = fmaf(hi[1], xv.w, acc);
    }
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float4 xv = x4[64 * i];
      acc = fmaf(bf16_lo(ws[2 * i]), xv.x, acc);
      acc = fmaf(bf16_hi(ws[2 * i]), xv.y, acc);
      acc = fmaf(bf16_lo(ws[2 * i + 1]), xv.z, acc);
      acc = fmaf(bf16_hi(ws[2 * i + 1]), xv.w, acc);
    }
  }
  return acc;
}


// dot of one lane's 16 MXFP4 code bytes (32 elements of one scale block,
// element 2j in the low nibble of byte j) with the staged input (xperm4
// order; xs = sm.x + xperm_group<0>(k0)). The hardware conversion applies the
// block scale: each converted value is exactly e2m1 * 2^(s - 127).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  // 2^(s - 127) as an fp32 bit pattern; s = 0 is the subnormal 2^-127
  return __builtin_bit_cast(float, s ? s << 23 : 0x00400000u);
}
__device__ __forceinline__ float unit_dot_mx(const u32x4& w, const float* xs, float scale) {
  const float4* x4 = reinterpret_cast<const float4*>(xs);
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  // two accumulators: 32 products per lane would otherwise be one chain of
  // dependent FMAs
  float acc0 = 0.f, acc1 = 0.f;
  // word q holds elements 8q .. 8q+7, two per byte (the byte index is an
  // immediate of the conversion); they meet float4s 2q and 2q + 1
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)ws[q], scale, 0);
    const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)ws[q], scale, 1);
    const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)ws[q], scale, 2);
    const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((int)ws[q], scale, 3);
    const float4 xa = x4[64 * (2 * q)], xb = x4[64 * (2 * q + 1)];
    acc0 = fmaf(e0[0], xa.x, acc0);
    acc0 = fmaf(e0[1], xa.y, acc0);
    acc0 = fmaf(e1[0], xa.z, acc0);
    acc0 = fmaf(e1[1], xa.w, acc0);
    acc1 = fmaf(e2[0], xb.x, acc1);
    acc1 = fmaf(e2[1], xb.y, acc1);
    acc1 = fmaf(e3[0], xb.z, acc1);
    acc1 = fmaf(e3[1], xb.w, acc1);
  }
  return acc0 + acc1;
}

// Sum within aligned groups of 2^lg lanes (lg <= 6) without branches.
__device__ __forceinline__ float group_sum_lg(float v, int lg) {
  v += lg >= 1 ? dpp<kDppXor1>(v) : 0.f;
  v += lg >= 2 ? dpp<kDppXor2>(v) : 0.f;
  v += lg >= 3 ? dpp<kDppHalfMirror>(v) : 0.f;
  v += lg >= 4 ? dpp<kDppMirror>(v) : 0.f;
  v += lg >= 5 ? __shfl_xor(v, 16) : 0.f;
  v += lg >= 6 ? __shfl_xor(v, 32) : 0.f;
  return v;
}

// Runs the units of rows [ra, rb) of a GEMV (ra, rb multiples of the unit
// row count) split over the 8 waves; writes per-wave row partials to
// sm.part[w][row - ra]. A unit is one 16-byte load per lane: 1 KB of one row
// (LONG: rows of 1 KB or more) or 1024 / Kb whole rows (short power-of-two
// rows). `prep` is called once by every thread after the scale loads and the
// first batch of weight loads have been issued (when `early`) and before any
// input is used; it must end with a workgroup barrier. Returns false on abort.
//
// Every unit of an unrolled batch issues its load unconditionally (units past
// the wave's range read a valid address and are dropped): with no branch
// around the loads the compiler waits only for the batch being consumed, so
// the next batch stays in flight.
// Work that only the polling wave does after prep (none by default).
struct NoLate {
  __device__ __forceinline__ void operator()() const {}
};

// FULL (LONG only): rows are whole KB (K a multiple of 1024) and there is one
// input vector, so a unit's validity is the same for all lanes and its input
// floats are at a lane-fixed LDS offset: every per-unit address term but the
// lane's own is uniform (scalar arithmetic).
//
// PAIR (MXFP4 only; rows of whole 512-byte pieces, an even row count, one
// input vector): a unit is 512 bytes of each of two consecutive rows, lanes
// 0-31 on the first and 32-63 on the second, at the same columns. Every lane
// is valid for any such row length (MXFP4 gate/up rows of 3584 bytes are not
// whole KB) and the two halves of a wave read the same staged inputs.
template <int EB, bool LONG, int SLOT, bool FULL, bool PAIR, class Prep, class Late>
__device__ __forceinline__ bool gemv_rows_t(const Gemv& g, Smem& sm, int ra, int rb, bool early, Prep&& prep,
                                            Late&& late) {
  static_assert(LONG || !FULL, "whole-KB rows are long rows");
  static_assert(!PAIR || (EB == 0 && LONG && !FULL), "row pairs are an MXFP4 long-row mode");
  constexpr int U = kUnroll;  // units per batch
  const int lane = EB == 0 ? opaque_lane() : lane_id();
  const int w = wave_id();
  const int kb = g.Kb;
  int S = 1, m = 1, lg_lpr = 0;
  int nunits;
  if constexpr (!LONG) {
    m = 1024 / kb;
    lg_lpr = 31 - __builtin_clz(kb >> 4);
    nunits = (rb - ra) / m;
  } else if constexpr (PAIR) {
    S = kb >> 9;  // 512-byte pieces per row
    nunits = ((rb - ra) >> 1) * S;
  } else {
    S = (kb + 1023) >> 10;
    nunits = (rb - ra) * S;
  }
  // Units go out in batches of U. Wave w takes batch w first (issued
  // before the dependency wait when early); later batches are claimed from an
  // LDS counter, so waves whose loads return sooner stream more of the rows.
  const int nbat = (nunits + U - 1) / U;
  const int lpr_mask = (1 << lg_lpr) - 1;
  // u / S by multiply-high (exact for u < 2^32 / S)
  const uint32_t magic = S == 1 ? 0u : 0xFFFFFFFFu / (uint32_t)S + 1u;
  auto div_s = [&](int u) { return S == 1 ? u : (int)__umulhi((uint32_t)u, magic); };
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(&sm.claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readlane(v, 0);
  };

  // A batch: each lane's 16 code bytes of U units and, for FP8, the
  // block scale each 16 bytes belong to, loaded alongside (the scale lines of
  // a row group are shared by its 8 rows and come from cache after the first).
  u32x4 wa[U], wb[U];
  uint32_t sa[U], sb[U];
  auto issue = [&](u32x4* W, uint32_t* SC, int bt) {
    const int ub = bt * U;
    int i_row = 0, i_seg = 0;
    if constexpr (LONG) { i_row = div_s(ub); i_seg = ub - i_row * S; }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = ub + j;
      int row, b;
      if constexpr (PAIR) {
        row = ra + 2 * i_row + (lane >> 5);
        b = (i_seg << 9) + ((lane & 31) << 4);
        const bool wrap = i_seg + 1 == S;
        i_row += wrap ? 1 : 0;
        i_seg = wrap ? 0 : i_seg + 1;
      } else if constexpr (LONG) {
        row = ra + i_row;
        b = (i_seg << 10) + (lane << 4);
        const bool wrap = i_seg + 1 == S;
        i_row += wrap ? 1 : 0;
        i_seg = wrap ? 0 : i_seg + 1;
      } else {
        row = ra + u * m + (lane >> lg_lpr);
        b = (lane & lpr_mask) << 4;
      }
      const bool ok = u < nunits && (FULL || PAIR || b < kb);
      const uint8_t* cp;
      const uint8_t* sp = nullptr;
      unit_ptr_t<EB, SLOT>(g, sm, ok ? row : ra, ok ? b : 0, cp, sp);
      W[j] = __builtin_nontemporal_load(gp(reinterpret_cast<const u32x4*>(cp)));
      if constexpr (EB == 1) SC[j] = gld(reinterpret_cast<const uint16_t*>(sp));
      if constexpr (EB == 0) SC[j] = gld(sp);
    }
  };

  // LONG rows span several units and possibly several batches (and waves):
  // each wave adds its share of a row into its own partial.
  auto compute = [&](const u32x4* W, const uint32_t* SC, int bt) {
    const int ub = bt * U;
    int c_row = 0, c_seg = 0;
    if constexpr (LONG) { c_row = div_s(ub); c_seg = ub - c_row * S; }
    int cur_row = ra + (PAIR ? 2 * c_row : c_row);  // PAIR: the pair's first row
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = ub + j;
      const bool uok = u < nunits;
      int row, b;
      const int seg = c_seg;
      if constexpr (PAIR) {
        row = ra + 2 * c_row;
        b = (c_seg << 9) + ((lane & 31) << 4);
        const bool wrap = c_seg + 1 == S;
        c_row += wrap ? 1 : 0;
        c_seg = wrap ? 0 : c_seg + 1;
      } else if constexpr (LONG) {
        row = ra + c_row;
        b = (c_seg << 10) + (lane << 4);
        const bool wrap = c_seg + 1 == S;
        c_row += wrap ? 1 : 0;
        c_seg = wrap ? 0 : c_seg + 1;
      } else {
        row = ra + u * m + (lane >> lg_lpr);
        b = (lane & lpr_mask) << 4;
      }
      const bool ok = uok && (FULL || PAIR || b < kb);
      const float* xs;
      if constexpr (PAIR) {
        // xperm4 of element 1024 seg + 32 (lane & 31)
        xs = sm.x + ((seg >> 1) << 11) + ((((seg & 1) << 5) | (lane & 31)) << 2);
      } else if constexpr (FULL) {
        // xperm_group of (seg * 1024 + 16 * lane) (FP8), (seg * 512 + 8 * lane)
        // (bf16) or xperm4 of (seg * 2048 + 32 * lane) (MXFP4)
        xs = sm.x + (EB == 1 ? (seg << 10) + (lane << 2)
                     : EB == 0 ? (seg << 11) + (lane << 2)
                               : ((seg >> 1) << 10) + ((lane & 1) << 9) + ((seg & 1) << 7) + ((lane >> 1) << 2));
      } else {
        const int bq = ok ? b : 0;
        const int rq = ok ? row : ra;
        const int k0 = (EB == 1) ? bq : (EB == 2) ? (bq >> 1) : (bq << 1);
        const int xoff = (g.lg_rpv >= 31) ? 0 : ((rq >> g.lg_rpv) - g.vbase) * g.xK;
        xs = sm.x + xperm_group<EB>(xoff + k0);
      }
      float d;
      if constexpr (EB == 0) d = unit_dot_mx(W[j], xs, e8m0_value(SC[j]));
      else d = unit_dot<EB>(W[j], xs);
      if constexpr (EB == 1) d *= bf16_val((uint16_t)SC[j]);
      d = ok ? d : 0.f;
      if constexpr (LONG) {
        // rows change at most once per unit; flushing is a uniform branch.
        // A flush adds the four 16-lane row sums into the wave's partial
        // with LDS atomics (no read-back wait; a wave's adds to one row stay
        // in program order)
        if (uok && row != cur_row) {
          const float t = row16_sum(acc);
          if ((lane & 15) == 0)
            __hip_atomic_fetch_add(&sm.part[w][cur_row - ra + (PAIR ? lane >> 5 : 0)], t, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
          acc = 0.f;
          cur_row = row;
        }
        acc += d;
      } else {
        float t = group_sum_lg(d, lg_lpr);
        if (uok && (lane & lpr_mask) == 0) sm.part[w][row - ra] = t;
      }
    }
    if constexpr (LONG) {
      const float t = row16_sum(acc);
      if ((lane & 15) == 0)
        __hip_atomic_fetch_add(&sm.part[w][cur_row - ra + (PAIR ? lane >> 5 : 0)], t, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };

  // With `early`, weight and scale addresses do not depend on this step's
  // data: each static wave's first batch is in flight before prep (the
  // dependency wait). Without it (slot tables set inside prep) everything
  // follows prep. With g.split only the batches inside the first row segment
  // go out before prep.
  constexpr int kStat = kWaves - 1;  // waves with static batches (not the polling wave)
  int bA = w < kStat ? w : nbat, bB = kEarlyBatches == 2 && w < kStat ? w + kStat : nbat;
  // (first-segment units: S per row, S per row pair, or one per m rows)
  const int ebat = !early ? 0 : !g.split ? nbat
                 : min(nbat, (PAIR ? (g.seg_n1 >> 1) * S : LONG ? g.seg_n1 * S : g.seg_n1 / m) / U);
  if (bA < ebat) issue(wa, sa, bA);
  if (kEarlyBatches == 2 && bB < ebat) issue(wb, sb, bB);
  if (!prep()) return false;
  // With g.split the polling wave sets up the second segment (late) while the
  // other waves stream the first; a batch beyond the first segment waits for
  // its LDS flag. The flag stays set for later row chunks of the stage.
  bool ready = !g.split;
  if (w == kPollWave) {
    late();
    if (g.split) {
      __hip_atomic_store(&sm.slots_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      ready = true;
    }
  }
  auto gate = [&](int bt) {
    if (ready || bt < ebat || bt >= nbat) return;
    while (__hip_atomic_load(&sm.slots_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(1);
    ready = true;
  };
  gate(bA);
  if (bA >= ebat && bA < nbat) issue(wa, sa, bA);
  gate(bB);
  if (kEarlyBatches == 2 && bB >= ebat && bB < nbat) issue(wb, sb, bB);
  if (w == kPollWave) {  // no static batch: claim the first one too
    bA = claim();
    if (bA < nbat) issue(wa, sa, bA);
  }
  if (kEarlyBatches == 1 || w == kPollWave) {
    bB = claim();
    gate(bB);
    if (bB < nbat) issue(wb, sb, bB);
  }
  // Claims increase monotonically, so the batch in A is always older than the
  // one in B and a failed claim means every later claim fails too.
  while (bA < nbat) {
    compute(wa, sa, bA);
    bA = claim();
    gate(bA);
    if (bA < nbat) issue(wa, sa, bA);
    if (bB >= nbat) break;
    compute(wb, sb, bB);
    bB = claim();
    gate(bB);
    if (bB < nbat) issue(wb, sb, bB);
  }
  return true;
}

template <int EB, int SLOT, class Prep, class Late>
__device__ __forceinline__ bool gemv_rows(const Gemv& g, Smem& sm, int ra, int rb, bool early, Prep&& prep,
                                          Late&& late) {
  const bool small = g.Kb < 1024 && (1024 % g.Kb) == 0;
  if (small) return gemv_rows_t<EB, false, SLOT, false, false>(g, sm, ra, rb, early, prep, late);
  if ((g.Kb & 1023) == 0 && g.lg_rpv >= 31)
    return gemv_rows_t<EB, true, SLOT, true, false>(g, sm, ra, rb, early, prep, late);
  if constexpr (EB == 0) {
    // MXFP4 rows of whole 512-byte pieces (the gate/up rows): row pairs
    if ((g.Kb & 511) == 0 && g.lg_rpv >= 31 && ((rb - ra) & 1) == 0 && (SLOT != 2 || (g.slot_Kb & 511) == 0))
      return gemv_rows_t<EB, true, SLOT, false, true>(g, sm, ra, rb, early, prep, late);
  }
  return gemv_rows_t<EB, true, SLOT, false, false>(g, sm, ra, rb, early, prep, late);
}

// Balanced contiguous share of `rows` (in groups of `gran`) for workgroup wg.
__device__ __forceinline__ void my_rows(int rows, int gran, int G, int wg, int& ra, int& rb) {
  const int ng = rows / gran;  // ng * G < 2^31 for every plan shape
  ra = ng * wg / G * gran;
  rb = ng * (wg + 1) / G * gran;
}

// A chunk row's result: the sum of the waves' partials (each wave adds only
// the units it claimed; the others' entries stay zero).
__device__ __forceinline__ float part_sum(const Smem& sm, int t) {
  float y = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) y += sm.part[w][t];
  return y;
}

// Zero the per-wave partials and reset the batch counter (the first
// kEarlyBatches batches of every wave but the polling wave are static).
__device__ __forceinline__ void zero_part(Smem& sm) {
  float* p = &sm.part[0][0];
  for (int i = threadIdx.x; i < kWaves * kRowChunk; i += kThreads) p[i] = 0.f;
  if (threadIdx.x == 0) sm.claim = kEarlyBatches * (kWaves - 1);
}

// Contiguous fp32 vectors written this step by other workgroups (K a multiple
// of 4) are staged with 16-byte buffer loads under the sc1 policy, so every
// vector of up to kStageVec * 4 * kThreads floats costs one round trip. The
// buffer descriptor's bound makes loads past the end read zero.
constexpr int kBufDword3 = 0x00020000;  // raw (untyped) buffer descriptor, gfx9
constexpr int kStageVec = 10;           // 16-byte loads per thread in flight

__device__ __forceinline__ __amdgpu_buffer_rsrc_t vec_rsrc(const float* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, n * 4, kBufDword3);
}
template <unsigned CPOL>
__device__ __forceinline__ float4 ld_vec4(__amdgpu_buffer_rsrc_t r, int i4) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, i4 * 16, 0, CPOL));
}

// x_lds = v (gain null) or v * gain, v = src[0, K) loaded coherently. Returns
// this thread's sum of squares of v. Whether a batch slot has any element is
// the same for the whole workgroup, so only the loads a vector needs are issued.
template <bool MX = false>  // MX: xperm4 order (MXFP4 stages)
__device__ __forceinline__ float stage_vec(Smem& sm, int K, const float* src, const float* gain) {
  const __amdgpu_buffer_rsrc_t rv = vec_rsrc(src, K);
  const __amdgpu_buffer_rsrc_t rg = vec_rsrc(gain ? gain : src, K);
  const int n4 = K / 4;
  const int tid = MX ? opaque_tid() : (int)threadIdx.x;
  float ss = 0.f;
  for (int b0 = 0; b0 < n4; b0 += kStageVec * kThreads) {
    float4 v[kStageVec], g[kStageVec];
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      v[i] = g[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b0 + i * kThreads < n4) {
        v[i] = ld_vec4<kCpolSc1>(rv, b0 + i * kThreads + tid);
        if (gain) g[i] = ld_vec4<0>(rg, b0 + i * kThreads + tid);
      }
    }
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const int i4 = b0 + i * kThreads + tid;
      float4 y = v[i];
      if (gain) { y.x *= g[i].x; y.y *= g[i].y; y.z *= g[i].z; y.w *= g[i].w; }
      if (i4 < n4) *reinterpret_cast<float4*>(sm.x + (MX ? xperm4(4 * i4) : xperm(4 * i4))) = y;
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  }
  return ss;
}

// Fused RMSNorm of a contiguous coherent vector, applied to the product: the
// stage holds gain * v in LDS and multiplies its rows' results by 1 / rms (the
// GEMV is linear in its input), so the staging needs one barrier and no
// second pass over LDS. The per-wave sums of squares stay in sm.nred for
// rms_scale(), also in the next stage when it reuses the staged input.
template <bool MX = false>
__device__ __forceinline__ void stage_norm_vec(Smem& sm, int K, const float* gain, const float* src) {
  const float w = wave_sum(stage_vec<MX>(sm, K, src, gain));
  if (lane_id() == 0) sm.nred[wave_id()] = w;
  __syncthreads();
}
// The same for a bf16 vector (the embedding row or a bare stack's input; K a
// multiple of 8, src 16-byte aligned, not written this step): 16-byte loads
// of 8 values, gain * v staged in xperm order, sums of squares to sm.nred.
constexpr int kStageVecBf16 = 2;      // 8 values per load: 8192 per pass
__device__ __forceinline__ void stage_norm_bf16(Smem& sm, int K, const float* gain, const uint16_t* src) {
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t rg = vec_rsrc(gain, K);
  const int n8 = K / 8;
  float ss = 0.f;
  for (int b0 = 0; b0 < n8; b0 += kStageVecBf16 * kThreads) {
    u32x4 v[kStageVecBf16];
    float4 g0[kStageVecBf16], g1[kStageVecBf16];
#pragma unroll
    for (int i = 0; i < kStageVecBf16; ++i) {
      const int i8 = b0 + i * kThreads + (int)threadIdx.x;
      v[i] = (u32x4){0u, 0u, 0u, 0u};
      g0[i] = g1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b0 + i * kThreads < n8) {
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, i8 * 16, 0, 0);
        g0[i] = ld_vec4<0>(rg, 2 * i8);
        g1[i] = ld_vec4<0>(rg, 2 * i8 + 1);
      }
    }
#pragma unroll
    for (int i = 0; i < kStageVecBf16; ++i) {
      const int i8 = b0 + i * kThreads + (int)threadIdx.x;
      const float a0 = bf16_lo(v[i].x), a1 = bf16_hi(v[i].x), a2 = bf16_lo(v[i].y), a3 = bf16_hi(v[i].y);
      const float a4 = bf16_lo(v[i].z), a5 = bf16_hi(v[i].z), a6 = bf16_lo(v[i].w), a7 = bf16_hi(v[i].w);
      if (i8 < n8) {
        *reinterpret_cast<float4*>(sm.x + xperm(8 * i8)) =
            make_float4(a0 * g0[i].x, a1 * g0[i].y, a2 * g0[i].z, a3 * g0[i].w);
        *reinterpret_cast<float4*>(sm.x + xperm(8 * i8 + 4)) =
            make_float4(a4 * g1[i].x, a5 * g1[i].y, a6 * g1[i].z, a7 * g1[i].w);
      }
      ss += a0 * a0 + a1 * a1 + a2 * a2 + a3 * a3 + a4 * a4 + a5 * a5 + a6 * a6 + a7 * a7;
    }
  }
  const float w = wave_sum(ss);
  if (lane_id() == 0) sm.nred[wave_id()] = w;
  __syncthreads();
}

__device__ __forceinline__ float rms_scale(const Smem& sm, int K, float eps) {
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += sm.nred[i];
  return 1.0f / sqrtf(t / (float)K + eps);
}
// stage_plain of a contiguous coherent vector
template <bool MX = false>
__device__ __forceinline__ void stage_plain_vec(Smem& sm, int K, const float* src) {
  stage_vec<MX>(sm, K, src, nullptr);
  __syncthreads();
}

// LDS DMA copy by the calling wave of `nbytes` (a multiple of 16) from a
// 16-byte aligned global address into LDS: 16 bytes per lane and 1 KB per
// instruction, no registers held. Lanes past the end re-read the last 16
// bytes and write up to 1 KB - 16 bytes past the end of `dst` (callers leave
// that much LDS slack). A coherent copy uses the sc1 cache policy, as a
// relaxed agent-scope atomic load does, for data written this step by other
// workgroups. The caller waits for completion (vmcnt) before using the data.

template <unsigned CPOL = kCpolSc1>
__device__ __forceinline__ void dma_to_lds(void* dst, const void* src, int nbytes) {
  const int lane = lane_id();
  const char* sb = reinterpret_cast<const char*>(src);
  char* db = reinterpret_cast<char*>(dst);
  for (int off = 0; off < nbytes; off += 1024) {
    const int o = min(off + lane * 16, nbytes - 16);
    __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(sb + o),
                                     (__attribute__((address_space(3))) void*)(db + off), 16, 0, CPOL);
  }
}

// The same copy spread over all waves of the workgroup (1 KB pieces round
// robin), for copies too large for one wave's loads in flight. Every wave
// then waits for its own pieces (mem_done) before the barrier that publishes
// the data; `dst` needs the same 1 KB of slack.
template <unsigned CPOL = kCpolSc1>
__device__ __forceinline__ void dma_to_lds_wg(void* dst, const void* src, int nbytes) {
  const int lane = lane_id();
  const char* sb = reinterpret_cast<const char*>(src);
  char* db = reinterpret_cast<char*>(dst);
  for (int off = wave_id() * 1024; off < nbytes; off += kWaves * 1024) {
    const int o = min(off + lane * 16, nbytes - 16);
    __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(sb + o),
                                     (__attribute__((address_space(3))) void*)(db + off), 16, 0, CPOL);
  }
}

// ------------------------------------------------------------------ stage bodies

struct StageEnv {
  Ctx c;
  StagePlan st;
  int s;
};

__device__ __forceinline__ LayerPlan layer_of(const Ctx& c, int l) { return load_plan(&c.P->layers[l]); }


// Input of layer l: the embedding row or external hidden vector for l == 0,
// else the previous layer's output (written this step: coherent loads).
struct LayerInput {
  const float* prev;     // previous layer output, or null
  const uint16_t* bf16;  // embedding row / x_in
  __device__ __forceinline__ float operator()(int k) const {
    return prev ? ld_coh(prev + k) : bf16_val(gld(bf16 + k));
  }
};

__device__ __forceinline__ LayerInput layer_input(const Ctx& c, int l) {
  LayerInput in{nullptr, nullptr};
  if (l > 0) {
    in.prev = reinterpret_cast<const float*>(c.P->layers[l - 1].xo);
  } else if (c.P->dims.vocab > 0) {
    in.bf16 = reinterpret_cast<const uint16_t*>(c.P->embed) + (size_t)c.A.token * c.P->dims.hidden;
  } else {
    in.bf16 = c.A.x_in;
  }
  return in;
}

__device__ __forceinline__ Gemv gemv_of(const Fp8Mat& m, const char* base_unused = nullptr) {
  (void)base_unused;
  Gemv g{};
  g.codes = reinterpret_cast<const uint8_t*>(m.codes);
  g.scales = reinterpret_cast<const uint16_t*>(m.scales);
  g.Kb = m.K;
  g.nkb = m.nkb;
  g.slot_mode = 0;
  g.lg_rpv = 31;
  return g;
}

// Generic single-chunk-loop driver: processes the workgroup's rows in chunks;
// `prep` (wait + staging) runs before the first chunk; `epi(ra_chunk, n)`
// reads the chunk's row results through part_sum.
// `late` runs on the polling wave once, after prep (with g.split: while the
// other waves already stream the first row segment).
template <int EB, int SLOT, class Prep, class Epi, class Late = NoLate>
__device__ __forceinline__ bool run_gemv(const StageEnv& E, Smem& sm, const Gemv& g, int ra, int rb, bool early,
                                         Prep&& prep, Epi&& epi, Late&& late = Late{}) {
  if (ra >= rb) {
    // no rows: still take part in the dependency wait so barriers match
    const bool r = prep();
    if (r && wave_id() == kPollWave) late();
    return r;
  }
  bool first = true;
  uint64_t t_staged = 0;
  for (int ca = ra; ca < rb; ca += kRowChunk) {
    int cb = min(rb, ca + kRowChunk);
    bool ok;
    if (first) {
      ok = gemv_rows<EB, SLOT>(g, sm, ca, cb, early, [&]() {
        zero_part(sm);
        const bool r = prep();
        if (E.c.A.trace) t_staged = wall_clock64();
        return r;
      }, late);
    } else {
      zero_part(sm);
      // later chunks need the zeroed partials and batch counter visible
      // before their first claim
      ok = gemv_rows<EB, SLOT>(g, sm, ca, cb, true, [&]() {
        __syncthreads();
        return true;
      }, NoLate{});
    }
    if (!ok) return false;
    first = false;
    mark(E.c, sm, 1);
    if (E.c.A.trace && threadIdx.x == 0 && t_staged) sm.t_mark[0] = t_staged;
    __syncthreads();
    epi(ca, cb - ca);
    // The next chunk reuses the partials; after the last chunk the stage's
    // signal (a workgroup barrier) orders the epilogue before any later LDS use.
    if (cb < rb) __syncthreads();
    mark(E.c, sm, 2);
  }
  return true;
}

// --- QKV: [W_DQ ; W_DKV] * RMSNorm(x)
__device__ __forceinline__ bool stage_qkv(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const int l = E.st.layer;
  const LayerPlan L = layer_of(c, l);
  const int D = c.P->dims.hidden;
  Gemv g = gemv_of(L.qkv);
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  float* out = reinterpret_cast<float*>(L.qkv_raw);
  float rs = 1.f;  // 1 / rms of the input when the staging leaves it to the product
  // The step input tap (layer 0): every workgroup copies its slice, loaded
  // before the dependency wait (the input does not depend on this step's work).
  const LayerInput in = layer_input(c, l);
  const int tk0 = D * c.wg / c.G, tn = D * (c.wg + 1) / c.G - tk0;
  const bool tapper = l == 0 && (int)threadIdx.x < tn;
  const float tap = tapper ? in(tk0 + threadIdx.x) : 0.f;
  return run_gemv<1, 0>(E, sm, g, ra, rb, true,
      [&]() {
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        if (in.prev) {
          stage_norm_vec(sm, D, reinterpret_cast<const float*>(L.attn_norm), in.prev);
          rs = rms_scale(sm, D, c.P->dims.rms_eps);
        } else {
          stage_norm_bf16(sm, D, reinterpret_cast<const float*>(L.attn_norm), in.bf16);
          rs = rms_scale(sm, D, c.P->dims.rms_eps);
        }
        if (tapper) st_coh(reinterpret_cast<float*>(c.P->x0) + tk0 + threadIdx.x, tap);
        return true;
      },
      [&](int ca, int n) {
        for (int t = threadIdx.x; t < n; t += kThreads) st_coh(out + ca + t, part_sum(sm, t) * rs);
      });
}

// --- QB: q = W_UQ * RMSNorm(c_q), with the absorbed key projection fused in.
//
// Rotary query pairs are rotated and stored (scaled by tau = 1 / sqrt(d_qk),
// split into a bf16 high part and a bf16 residual) for the attention stage.
// The q_nope values the workgroup computed stay in LDS and are multiplied by
// the matching rows of W_UK: q_lat[h] = W_UK[h]^T q_nope[h] = sum over n of
// q_nope[h][n] * W_UK[h][n][:], so the rows n this workgroup holds give a
// partial sum of q_lat[h] (one per head and workgroup; the attention stage
// adds a head's partials in a fixed order). No workgroup waits for another
// between the query projection and the absorbed product, and the W_UK rows
// (static weights) are copied into LDS by the polling wave while the other
// waves stream W_UQ.
__device__ __forceinline__ void store_qrope(uint32_t* qr, int h, int col, int hg, int dr, float tau, float a,
                                            float b) {
  const int grp = h / hg, hh = h - grp * hg;
  __bf16 ah, al, bh, bl;
  split_bf16(a * tau, ah, al);
  split_bf16(b * tau, bh, bl);
  st_coh_u(qr + ((((size_t)grp * 2 + 0) * hg + hh) * dr + col) / 2, pack_bf16x2(ah, bh));
  st_coh_u(qr + ((((size_t)grp * 2 + 1) * hg + hh) * dr + col) / 2, pack_bf16x2(al, bl));
}

// LDS layout of the q_b stage (byte offsets into sm.x): the staged c_q, the
// workgroup's q_nope values, its W_UK rows and their scale entries (both
// copied by DMA, each followed by 1 KB of slack), the absorb reduction.
struct QbLds {
  int qn, wk, wsc, red, sc_pre, sc_bytes, gA;
  __device__ __forceinline__ QbLds(int q_lora, int nq, int dc, int u0, int u1, const uint16_t* scales) {
    const int nkb = dc / 128;
    qn = ((q_lora + 1023) & ~1023) * 4;
    wk = qn + ((nq + 3) & ~3) * 4;
    gA = u0 >> 3;
    const int gB = nq > 0 ? (u1 - 1) >> 3 : gA;
    const uintptr_t src = reinterpret_cast<uintptr_t>(scales + (size_t)gA * nkb);
    sc_pre = (int)(src & 15);
    sc_bytes = ((gB - gA + 1) * nkb * 2 + sc_pre + 15) & ~15;
    wsc = wk + nq * dc + 1024;
    red = wsc + sc_bytes + 1024;
  }
};

__device__ __forceinline__ bool stage_qb(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const int l = E.st.layer;
  const LayerPlan L = layer_of(c, l);
  const float* raw = reinterpret_cast<const float*>(L.qkv_raw);
  const float* tab = reinterpret_cast<const float*>(c.P->rope_tab) + (size_t)c.A.pos * d.rope;  // (cos, sin) pairs
  const int qkh = d.qk_nope + d.rope, dn = d.qk_nope, dc = d.kv_lora, dr = d.rope;
  Gemv g = gemv_of(L.qb);
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  int u0, u1;
  qb_nope_rows(d, ra, rb, u0, u1);
  const int nq = u1 - u0;
  const QbLds lay(d.q_lora, nq, dc, u0, u1, reinterpret_cast<const uint16_t*>(L.uk.scales));
  char* xb = reinterpret_cast<char*>(sm.x);
  float* qn = reinterpret_cast<float*>(xb + lay.qn);
  const uint8_t* wk = reinterpret_cast<const uint8_t*>(xb + lay.wk);
  const uint8_t* wsc = reinterpret_cast<const uint8_t*>(xb + lay.wsc);
  float* red = reinterpret_cast<float*>(xb + lay.red);
  uint32_t* qr = reinterpret_cast<uint32_t*>(L.qrope);
  const int hg = c.P->hg;
  const float tau = 1.0f / sqrtf((float)qkh);
  float rs = 1.f;  // 1 / rms of c_q, applied to the product
  const bool ok = run_gemv<1, 0>(E, sm, g, ra, rb, true,
      [&]() {
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        stage_norm_vec(sm, d.q_lora, reinterpret_cast<const float*>(L.q_norm), raw);
        rs = rms_scale(sm, d.q_lora, d.rms_eps);
        return true;
      },
      [&](int ca, int n) {
        // q_nope rows into LDS (W_UK row index h * d_n + j); rotary pairs
        // (adjacent rows, starting even) rotated into the query store
        for (int t = threadIdx.x; t < n; t += kThreads) {
          const int r = ca + t;
          const int h = r / qkh, j = r - h * qkh;
          if (j < dn) {
            qn[h * dn + j - u0] = part_sum(sm, t) * rs;
          } else if (((j - dn) & 1) == 0) {
            const int i = (j - dn) >> 1;
            const float cs = gld(tab + 2 * i), sn = gld(tab + 2 * i + 1);
            const float x0 = part_sum(sm, t) * rs, x1 = part_sum(sm, t + 1) * rs;
            store_qrope(qr, h, j - dn, hg, dr, tau, x0 * cs - x1 * sn, x0 * sn + x1 * cs);
          }
        }
      },
      [&]() {
        // polling wave, after the wait: the W_UK rows and scales of this
        // workgroup's q_nope rows into LDS (static weights, default policy)
        if (nq > 0) {
          dma_to_lds<0>(xb + lay.wk, reinterpret_cast<const uint8_t*>(L.uk.codes) + (size_t)u0 * dc, nq * dc);
          const uintptr_t sa = reinterpret_cast<uintptr_t>(reinterpret_cast<const uint16_t*>(L.uk.scales) +
                                                           (size_t)lay.gA * (dc / 128));
          dma_to_lds<0>(xb + lay.wsc, reinterpret_cast<const void*>(sa - lay.sc_pre), lay.sc_bytes);
        }
      });
  if (!ok) return false;
  if (nq <= 0) return true;
  if (wave_id() == kPollWave) mem_done();
  __syncthreads();  // q_nope values and the copied W_UK rows are in LDS
  // Absorbed product: thread t takes the 16 latent columns of 16-byte unit
  // cb = t mod (d_c / 16) of every (threads per column block)-th row and
  // keeps 16 sums; the per-thread sums of a column are then added in LDS.
  const int cpr = dc >> 4;              // 16-byte units per W_UK row
  const int slots = kThreads / cpr;     // threads per column block
  const int cb = threadIdx.x & (cpr - 1), sl = threadIdx.x / cpr;
  const int nkb = dc / 128;
  const int maxp = c.P->qb_maxparts, gran = c.P->qb_gran;
  float* part = reinterpret_cast<float*>(L.qlat_part);
  const int hA = u0 / dn, hB = (u1 - 1) / dn;
  for (int h = hA; h <= hB; ++h) {
    const int a = max(u0, h * dn) - u0, b = min(u1, (h + 1) * dn) - u0;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int r = a + sl; r < b; r += slots) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(wk + (size_t)r * dc + cb * 16);
      const int u = u0 + r;
      const uint16_t sb = *reinterpret_cast<const uint16_t*>(wsc + lay.sc_pre + (((u >> 3) - lay.gA) * nkb + (cb >> 3)) * 2);
      const float q = qn[r] * bf16_val(sb);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
        acc[4 * i + 0] = fmaf(lo[0], q, acc[4 * i + 0]);
        acc[4 * i + 1] = fmaf(lo[1], q, acc[4 * i + 1]);
        acc[4 * i + 2] = fmaf(hi[0], q, acc[4 * i + 2]);
        acc[4 * i + 3] = fmaf(hi[1], q, acc[4 * i + 3]);
      }
    }
    float4* rd = reinterpret_cast<float4*>(red + sl * dc + cb * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) rd[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    __syncthreads();
    const int slot = c.wg - qb_first(d, gran, c.G, h);
    float* dst = part + ((size_t)h * maxp + slot) * dc;
    for (int cc = threadIdx.x; cc < dc; cc += kThreads) {
      float sum = 0.f;
      for (int k = 0; k < slots; ++k) sum += red[k * dc + cc];
      st_coh(dst + cc, sum);
    }
    __syncthreads();
  }
  return true;
}

// Position chunks per head group this step: at least kChunkPos positions
// per attention unit and at most the planned count (one unit per workgroup
// when the context allows it), which also sizes the partial buffer. The
// attention and W_UV stages derive the same count from the position.
constexpr int kChunkPos = 64;
__device__ __forceinline__ int attn_chunks(const Ctx& c, int ctx) {
  return min(c.P->nch, max(1, (ctx + kChunkPos - 1) / kChunkPos));
}

// --- ATTN: split-KV MLA attention partials (m, l, acc) per (head, position chunk)
//
// Attention is the one dense contraction of the step: 16 heads share every
// latent cache row, so a work unit (16 heads x a chunk of positions) runs its
// two products on the matrix cores with v_mfma_f32_16x16x32_bf16:
//   scores  S^T[t][h] = sum_d K[t][d] Q[h][d]   (A = cache rows, B = queries)
//   values  O[h][c]   = sum_t P[h][t] V[t][c]   (A = probabilities, B = cache rows)
// K and V are the bf16 cache rows themselves. The fp32 operands (the scaled
// queries and the probabilities) enter as a bf16 high part plus a bf16
// residual, two MFMAs each, which keeps both products accurate to about
// 2^-16 relative: the result matches fp32 arithmetic, not bf16 rounding.
// Operand layout (lane l, g = l / 16): A holds A[l % 16][8g .. 8g + 7],
// B holds B[8g .. 8g + 7][l % 16], C holds C[4g .. 4g + 3][l % 16].
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kAttnBlock = 64;    // positions staged per round


__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int DTILES>  // latent dim tiles of 16 per wave: kv_lora / 128
__device__ __forceinline__ bool stage_attn(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const LayerPlan L = layer_of(c, E.st.layer);
  const int nch = attn_chunks(c, c.A.pos + 1), hg = c.P->hg;
  const int units = c.P->n_hg * nch;
  if (c.wg >= units) return wait_flags(c, sm, -1, 0, -1, E.s);  // no share of this stage
  const int grp = c.wg / nch, ch = c.wg % nch;
  const int pos = c.A.pos, ctx = pos + 1;
  const int chunk = (ctx + nch - 1) / nch;
  const int t0 = min(ctx, ch * chunk), t1 = min(ctx, t0 + chunk);
  const int dc = d.kv_lora, dr = d.rope, kvr = dc + dr, qkh = d.qk_nope + dr;
  const int q8n = kvr / 8;              // 16-byte pieces per cache row
  const int nkb = kvr / 32;             // MFMA k-blocks of a score
  const int kstr = kvr / 2 + 4;         // LDS cache-row stride in u32 (padded)
  const int qstr = kvr + 8;             // LDS query-row stride in bf16 (padded)
  constexpr int pstr = kAttnBlock + 4;  // LDS probability-row stride in floats
  const uint16_t* cache = reinterpret_cast<const uint16_t*>(L.kv);
  // The unit whose chunk holds position pos builds this step's cache row
  // [RMSNorm(latent) ; RoPE(rotary key)] itself from the key/value latent of
  // the q_a/kv_a stage (bf16, rounding point R1); the unit of head group 0
  // also appends it to the cache. Thread p owns the value pair (2p, 2p + 1):
  // its gains or rotation are static and loaded before the wait.
  const bool has_cur = pos >= t0 && pos < t1;
  const int npairs = kvr / 2;  // <= kPreThreads
  const int p = threadIdx.x;
  const bool own = has_cur && p < npairs;
  const bool is_lat = 2 * p < dc;
  float ga = 0.f, gb = 0.f;  // gains (latent pairs) or (cos, sin) (rotary pairs)
  if (own) {
    if (is_lat) {
      const float* gk = reinterpret_cast<const float*>(L.kv_norm) + 2 * p;
      ga = gld(gk);
      gb = gld(gk + 1);
    } else {
      const float* tab = reinterpret_cast<const float*>(c.P->rope_tab) + (size_t)pos * dr + 2 * (p - dc / 2);
      ga = gld(tab);
      gb = gld(tab + 1);
    }
  }

  // Cache rows of a block before pos were written by earlier steps: their
  // loads need no dependency, so the first block is issued before the wait
  // and each later block while the previous one is being computed.
  // (threads of the polling wave load none of them)
  constexpr int kPer = (kAttnBlock * 80 + kPreThreads - 1) / kPreThreads;
  u32x4 v[kPer];
  const bool loader = (int)threadIdx.x < kPreThreads;
  // piece i of a block is 16-byte piece i of the block's contiguous rows
  auto issue_block = [&](int tb) {
    if (!loader) return;
    const int nb = min(kAttnBlock, t1 - tb);
    const int nmain = max(0, min(nb, pos - tb)) * q8n;
    const u32x4* src = reinterpret_cast<const u32x4*>(cache + (size_t)tb * kvr);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + r * kPreThreads;
      v[r] = gld(src + (i < nmain ? i : 0));
    }
  };
  // LDS position of piece i: (row, col) = (i / q8n, i % q8n), stepped per r
  // from the thread's first piece without a division per piece
  const int row0 = (int)threadIdx.x / q8n, col0 = (int)threadIdx.x - row0 * q8n;
  const int drow = kPreThreads / q8n, dcol = kPreThreads - drow * q8n;
  if (t0 < t1) issue_block(t0);
  // wait for the q_b workgroups that produced this head group's queries
  const int gran = c.P->qb_gran, qrows = d.n_heads * qkh;
  const int wlo = split_owner(qrows, gran, c.G, grp * hg * qkh);
  const int whi = split_owner(qrows, gran, c.G, (grp + 1) * hg * qkh - 1);
  if (!wait_flags(c, sm, E.st.wait, wlo, whi, E.s)) return false;

  // LDS: query hi/lo [16][qstr] bf16, cache rows [64][kstr] u32, two score
  // partials [2][16][pstr] f32; at the end of the staging area the per-head
  // max / sum / rescale and the new cache row [kvr / 2] u32
  __bf16* qh = reinterpret_cast<__bf16*>(sm.x);
  __bf16* ql = qh + kMH * qstr;
  uint32_t* kvs = reinterpret_cast<uint32_t*>(ql + kMH * qstr);
  float* sp = reinterpret_cast<float*>(kvs + kAttnBlock * kstr);
  uint32_t* crow = reinterpret_cast<uint32_t*>(sm.x + kXMax) - npairs;
  float* hm = reinterpret_cast<float*>(crow) - 3 * kMH;  // running max per head
  float* hl = hm + kMH;                                   // running sum per head
  float* ha = hl + kMH;                                   // rescale of the accumulators this round

  {
    // All waves copy the head group's q_lat partials, the polling wave (no
    // cache-row loads queued ahead of it) the rotary queries and (for the
    // unit holding pos) the key/value latent, into the space the cache rows
    // use later. Then the queries are assembled: latent columns = tau * the
    // sum of the head's partials in slot order, split into bf16 high and
    // residual parts; rotary columns as stored; rows of heads >= hg zero.
    const int maxp = c.P->qb_maxparts;
    float* tpart = reinterpret_cast<float*>(kvs);                    // [hg][maxp][dc]
    uint32_t* trope = reinterpret_cast<uint32_t*>(tpart + hg * maxp * dc + 256);  // [2][hg][dr / 2]
    float* tkv = reinterpret_cast<float*>(trope + hg * dr + 256);    // [kvr]
    const float* raw = reinterpret_cast<const float*>(L.qkv_raw);
    // slot k of head h holds a partial only if q_b workgroup qb_first(h) + k
    // owns rows (with fewer row groups than workgroups some own none): the
    // planner's per-head slot mask
    uint64_t* qmask = reinterpret_cast<uint64_t*>(&sm.part[0][0]);
    if ((int)threadIdx.x < hg) {
      const int t = opaque_lane();  // threads < hg <= 64 are lanes of wave 0
      qmask[t] = gld(&c.P->qb_mask[grp * hg + t]);
    }
    dma_to_lds_wg(tpart, reinterpret_cast<const float*>(L.qlat_part) + (size_t)grp * hg * maxp * dc, hg * maxp * dc * 4);
    if (wave_id() == kPollWave) {
      dma_to_lds(trope, reinterpret_cast<const uint16_t*>(L.qrope) + (size_t)grp * 2 * hg * dr, 2 * hg * dr * 2);
      if (has_cur) dma_to_lds(tkv, raw + d.q_lora, kvr * 4);
    }
    mem_done();
    __syncthreads();
    const float tau = 1.0f / sqrtf((float)qkh);
    const int lgdc = 31 - __builtin_clz(dc);
    for (int i = threadIdx.x; i < hg * dc / 4; i += kThreads) {
      const int hh = (4 * i) >> lgdc, col = (4 * i) & (dc - 1);
      const uint64_t m = qmask[hh];
      const float4* pp = reinterpret_cast<const float4*>(tpart + (size_t)hh * maxp * dc + col);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < maxp; ++k)
        if ((m >> k) & 1) {
          const float4 v = pp[k * (dc / 4)];
          sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
      __bf16 h0, l0, h1, l1, h2, l2, h3, l3;
      split_bf16(sum.x * tau, h0, l0);
      split_bf16(sum.y * tau, h1, l1);
      split_bf16(sum.z * tau, h2, l2);
      split_bf16(sum.w * tau, h3, l3);
      uint32_t* qh2 = reinterpret_cast<uint32_t*>(qh + hh * qstr + col);
      uint32_t* ql2 = reinterpret_cast<uint32_t*>(ql + hh * qstr + col);
      qh2[0] = pack_bf16x2(h0, h1);
      qh2[1] = pack_bf16x2(h2, h3);
      ql2[0] = pack_bf16x2(l0, l1);
      ql2[1] = pack_bf16x2(l2, l3);
    }
    for (int i = threadIdx.x; i < hg * (dr / 2); i += kThreads) {
      const int hh = i / (dr / 2), cp = i - hh * (dr / 2);
      reinterpret_cast<uint32_t*>(qh + hh * qstr + dc)[cp] = trope[i];
      reinterpret_cast<uint32_t*>(ql + hh * qstr + dc)[cp] = trope[hg * (dr / 2) + i];
    }
    for (int i = threadIdx.x; i < (kMH - hg) * qstr; i += kThreads) {
      qh[hg * qstr + i] = (__bf16)0.f;
      ql[hg * qstr + i] = (__bf16)0.f;
    }
    if (threadIdx.x < kMH) { hm[threadIdx.x] = -INFINITY; hl[threadIdx.x] = 0.f; }
    if (has_cur) {
      // every wave forms the latent's sum of squares itself (no barrier)
      float ss = 0.f;
      for (int k = lane_id(); k < dc; k += 64) ss += tkv[k] * tkv[k];
      const float rsk = 1.0f / sqrtf(wave_sum(ss) / (float)dc + d.rms_eps);
      if (own) {
        const float x0 = tkv[2 * p], x1 = tkv[2 * p + 1];
        float a, b;
        if (is_lat) {
          a = x0 * rsk * ga;
          b = x1 * rsk * gb;
        } else {
          a = x0 * ga - x1 * gb;
          b = x0 * gb + x1 * ga;
        }
        const uint32_t pr = (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
        crow[p] = pr;
        if (grp == 0)
          st_coh_u(reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(cache) + (size_t)pos * kvr) + p, pr);
      }
    }
    mark(c, sm, 0);
  }

  const int lane = lane_id();
  const int w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  f32x4 acc[DTILES];
#pragma unroll
  for (int i = 0; i < DTILES; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int tb = t0; tb < t1; tb += kAttnBlock) {
    const int nb = min(kAttnBlock, t1 - tb);
    // ---- stage rows [tb, tb + nb) (zeros beyond nb); the row of pos was
    // written this step by another workgroup and is read coherently
    {
      const int nmain = max(0, min(nb, pos - tb)) * q8n;
      const bool cur_here = pos >= tb && pos < tb + nb;
      __syncthreads();  // the previous round's readers are done with kvs and sp
      int row = row0, col = col0;
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = threadIdx.x + r * kPreThreads;
        if (loader && i < kAttnBlock * q8n) {
          u32x4 z = {0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(kvs + row * kstr + col * 4) = i < nmain ? v[r] : z;
        }
        col += dcol;
        row += drow;
        if (col >= q8n) { col -= q8n; ++row; }
      }
      if (tb + kAttnBlock < t1) issue_block(tb + kAttnBlock);
      __syncthreads();
      if (cur_here && threadIdx.x < kvr / 2) kvs[(pos - tb) * kstr + threadIdx.x] = crow[threadIdx.x];
      __syncthreads();
    }
    // ---- scores: waves 0-3 take position tiles 0-3 over the first half of
    // the k-blocks, waves 4-7 the same tiles over the second half
    {
      const int tile = w & 3, half = w >> 2;
      const int kb0 = half ? nkb / 2 : 0, kb1 = half ? nkb : nkb / 2;
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      if (tile * 16 < nb) {
        const uint32_t* arow = kvs + (tile * 16 + lr) * kstr + lg * 4;
        const __bf16* bh = qh + lr * qstr + lg * 8;
        const __bf16* bl = ql + lr * qstr + lg * 8;
        for (int kb = kb0; kb < kb1; ++kb) {
          bf16x8 a = u32x4_as_bf16x8(*reinterpret_cast<const u32x4*>(arow + kb * 16));
          bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bh + kb * 32);
          bf16x8 b2 = *reinterpret_cast<const bf16x8*>(bl + kb * 32);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, sc, 0, 0, 0);
        }
      }
      // sc[r] = S^T[tile*16 + 4*lg + r][lr] = score of head lr at that position
      float* dst = sp + half * kMH * pstr + lr * pstr + tile * 16 + 4 * lg;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = sc[r];
    }
    __syncthreads();
    // ---- online softmax: wave w owns heads 2w and 2w+1, lanes are positions
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int h = 2 * w + q;
      const bool valid = lane < nb;
      float sv = valid ? sp[h * pstr + lane] + sp[kMH * pstr + h * pstr + lane] : -INFINITY;
      float mold = hm[h];
      float mn = fmaxf(mold, wave_max(sv));
      float alpha = __expf(mold - mn);  // 0 on the first round (mold = -inf)
      float pv = valid ? __expf(sv - mn) : 0.f;
      float ps = wave_sum(pv);
      sp[h * pstr + lane] = pv;          // probabilities replace the first partial
      if (lane == 0) { hm[h] = mn; hl[h] = hl[h] * alpha + ps; ha[h] = alpha; }
    }
    __syncthreads();
    // ---- values: wave w owns latent dim tiles [w * DTILES, w * DTILES + DTILES)
    {
#pragma unroll
      for (int i = 0; i < DTILES; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][r] *= ha[4 * lg + r];
      }
      for (int pb = 0; pb < (nb + 31) / 32; ++pb) {
        // A = P[head lr][pb*32 + 8*lg + 0..7], split hi / lo
        const float* prow = sp + lr * pstr + pb * 32 + 8 * lg;
        bf16x8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 hi, lo;
          split_bf16(prow[e], hi, lo);
          ah[e] = hi;
          al[e] = lo;
        }
        // B of tile i = V[pb*32 + 8*lg + e][dim w*DTILES*16 + DTILES*lr + i]:
        // the DTILES dims a lane needs from one row are adjacent, so one LDS
        // read of 2*DTILES bytes per row serves every tile of the wave
        const uint16_t* vrow =
            reinterpret_cast<const uint16_t*>(kvs) + (pb * 32 + 8 * lg) * (2 * kstr) + w * DTILES * 16 + DTILES * lr;
        uint32_t vw[8][(DTILES + 1) / 2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (DTILES == 4) {
            const uint2 t = *reinterpret_cast<const uint2*>(vrow + e * 2 * kstr);
            vw[e][0] = t.x;
            vw[e][1] = t.y;
          } else if constexpr (DTILES == 2) {
            vw[e][0] = *reinterpret_cast<const uint32_t*>(vrow + e * 2 * kstr);
          } else {
            vw[e][0] = vrow[e * 2 * kstr];
          }
        }
#pragma unroll
        for (int i = 0; i < DTILES; ++i) {
          u32x4 bu;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t lo = vw[2 * k][i / 2], hi = vw[2 * k + 1][i / 2];
            bu[k] = (i & 1) ? (lo >> 16) | (hi & 0xffff0000u) : (lo & 0xffffu) | (hi << 16);
          }
          const bf16x8 b = u32x4_as_bf16x8(bu);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[i], 0, 0, 0);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[i], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();
  mark(c, sm, 1);
  // ---- partials: acc[i][r] = O[head 4*lg + r][dim w*DTILES*16 + DTILES*lr + i].
  // A head's partial row is [acc (d_c) ; max ; sum ; 0 ; 0] (a 16-byte
  // multiple); the rows are transposed through LDS (the cache-row space is
  // free now) so that every lane stores whole 16-byte pieces.
  const int ps = dc + 4;
  float* tout = reinterpret_cast<float*>(kvs);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * lg + r;
#pragma unroll
    for (int i = 0; i < DTILES; ++i) tout[hh * ps + w * DTILES * 16 + DTILES * lr + i] = acc[i][r];
  }
  if (threadIdx.x < kMH) {
    float* t = tout + threadIdx.x * ps + dc;
    t[0] = hm[threadIdx.x];
    t[1] = hl[threadIdx.x];
    t[2] = t[3] = 0.f;
  }
  __syncthreads();
  {
    float* part = reinterpret_cast<float*>(L.attn_part) + ((size_t)grp * hg * nch + ch) * ps;
    const int p4 = ps / 4;  // 16-byte pieces per head row
    const __amdgpu_buffer_rsrc_t rp = vec_rsrc(part, (hg - 1) * nch * ps + ps);
    for (int q = threadIdx.x; q < hg * p4; q += kThreads) {
      const int hh = q / p4, c4 = q - hh * p4;
      const float4 v = *reinterpret_cast<const float4*>(tout + hh * ps + 4 * c4);
      // head hh's row of this chunk lies hh * nch rows further on
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, ((hh * nch) * ps + 4 * c4) * 4, 0,
                                             kCpolSc1);
    }
  }
  mark(c, sm, 2);
  return true;
}

// --- UV: merge the attention partials of each head, o[h] = W_UV[h] o_lat[h]
constexpr int kMergeBatch = 32;  // chunk accumulators in flight per thread
__device__ __forceinline__ bool stage_uv(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const LayerPlan L = layer_of(c, E.st.layer);
  const int nch = attn_chunks(c, c.A.pos + 1), dc = d.kv_lora;
  const float* part = reinterpret_cast<const float*>(L.attn_part);
  Gemv g = gemv_of(L.uv);
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  g.lg_rpv = 31 - __builtin_clz(d.v_head);
  g.vbase = ra / d.v_head;
  g.xK = dc;
  float* out = reinterpret_cast<float*>(L.o);
  return run_gemv<1, 0>(E, sm, g, ra, rb, true,
      [&]() {
        // wait for the attention units of this workgroup's heads only
        const int h0 = ra / d.v_head, h1 = (rb - 1) / d.v_head;
        const int hg = c.P->hg;
        if (ra >= rb) return wait_flags(c, sm, -1, 0, -1, E.s);
        if (!wait_flags(c, sm, E.st.wait, h0 / hg * nch, (h1 / hg + 1) * nch - 1, E.s)) return false;
        const int lane = lane_id();
        const int ps = dc + 4;                   // partial row: acc, max, sum, padding
        const int hbytes = nch * ps * 4;         // partials of one head
        if (h0 == h1 && (hbytes & 15) == 0 && 4096 + hbytes + 1024 <= kXMax * 4) {
          // One head: all waves copy its partials into LDS with coherent
          // DMA; thread k then merges latent column k from LDS (chunk i's
          // maximum and sum in lane i of every wave).
          const float* ph = part + (size_t)h0 * nch * ps;
          float* pr = sm.x + 1024;
          dma_to_lds_wg(pr, ph, hbytes);
          mem_done();
          __syncthreads();
          const bool lane_ch = lane < nch;
          const float m = lane_ch ? pr[lane * ps + dc] : -INFINITY;
          const float sv = lane_ch ? pr[lane * ps + dc + 1] : 0.f;
          const float mx = wave_max(m);
          const float e = m == -INFINITY ? 0.f : __expf(m - mx);
          const float fac = e / wave_sum(e * sv);
          if ((int)threadIdx.x < dc) {
            float num = 0.f;
            for (int i = 0; i < nch; ++i)
              num += pr[i * ps + threadIdx.x] *
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fac), i));
            sm.x[xperm(threadIdx.x)] = num;
          }
          __syncthreads();
          return true;
        }
        // Several heads: thread k merges latent column k of each head, with
        // the chunk maxima and sums (chunk i in lane i of every wave) and the
        // chunk accumulators of its column all loaded before any is used.
        const int k = min((int)threadIdx.x, dc - 1);
        const bool lane_ch = lane < nch;
        for (int h = h0; h <= h1; ++h) {
          const float* ph = part + (size_t)h * nch * ps;
          const float* pl = ph + (size_t)(lane_ch ? lane : 0) * ps + dc;
          const float mi = ld_coh(pl), si = ld_coh(pl + 1);
          float fac = 0.f, num = 0.f;
          for (int i0 = 0; i0 < nch; i0 += kMergeBatch) {
            float v[kMergeBatch];
#pragma unroll
            for (int b = 0; b < kMergeBatch; ++b) v[b] = ld_coh(ph + (size_t)min(i0 + b, nch - 1) * ps + k);
            if (i0 == 0) {
              const float m = lane_ch ? mi : -INFINITY;
              const float mx = wave_max(m);
              const float e = m == -INFINITY ? 0.f : __expf(m - mx);
              fac = e / wave_sum(e * (lane_ch ? si : 0.f));
            }
#pragma unroll
            for (int b = 0; b < kMergeBatch; ++b) {
              const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fac), (i0 + b) & 63));
              num += i0 + b < nch ? v[b] * f : 0.f;
            }
          }
          if ((int)threadIdx.x < dc) sm.x[xperm((h - h0) * dc + threadIdx.x)] = num;
        }
        __syncthreads();
        return true;
      },
      [&](int ca, int n) {
        for (int t = threadIdx.x; t < n; t += kThreads) st_coh(out + ca + t, part_sum(sm, t));
      });
}

// --- WO: x_attn = x + W_O o
__device__ __forceinline__ bool stage_wo(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const int l = E.st.layer;
  const LayerPlan L = layer_of(c, l);
  const float* o = reinterpret_cast<const float*>(L.o);
  Gemv g = gemv_of(L.wo);
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  float* out = reinterpret_cast<float*>(L.xa);
  const LayerInput in = layer_input(c, l);
  // the residual (this layer's input) is complete before this stage's
  // dependency: load the workgroup's share before waiting
  float res = 0.f;
  const bool res_pre = rb - ra <= kRowChunk;  // one chunk: thread t holds row ra + t
  return run_gemv<1, 0>(E, sm, g, ra, rb, true,
      [&]() {
        if (res_pre && (int)threadIdx.x < rb - ra) res = in(ra + threadIdx.x);
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        stage_plain_vec(sm, d.n_heads * d.v_head, o);
        return true;
      },
      [&](int ca, int n) {
        for (int t = threadIdx.x; t < n; t += kThreads)
          st_coh(out + ca + t, (res_pre ? res : in(ca + t)) + part_sum(sm, t));
      });
}

// --- ROUTER: z = W_r * RMSNorm(x_attn)   (bf16 weights)
__device__ __forceinline__ bool stage_router(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const LayerPlan L = layer_of(c, E.st.layer);
  const float* xa = reinterpret_cast<const float*>(L.xa);
  Gemv g{};
  g.codes = reinterpret_cast<const uint8_t*>(L.router);
  g.Kb = d.hidden * 2;
  g.lg_rpv = 31;
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  float* out = reinterpret_cast<float*>(L.router_logits);
  float rs = 1.f;  // 1 / rms of x_attn, applied to the product
  return run_gemv<2, 0>(E, sm, g, ra, rb, true,
      [&]() {
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        stage_norm_vec(sm, d.hidden, reinterpret_cast<const float*>(L.ffn_norm), xa);
        rs = rms_scale(sm, d.hidden, d.rms_eps);
        return true;
      },
      [&](int ca, int n) {
        for (int t = threadIdx.x; t < n; t += kThreads) st_coh(out + ca + t, part_sum(sm, t) * rs);
      });
}

// Top-k of the router logits by the calling wave (ties to the lower index),
// with sigmoid weights normalised over the chosen experts: into LDS, and the
// routed slot tables of the gate/up stage (slots n_shared + j) set from them.
// Lane j keeps the j-th choice, so nothing is read back from LDS.
template <int NV>  // logits per lane: experts lane + 64 i, i < NV (NV * 64 >= n_experts)
__device__ __forceinline__ void route_wave_t(const pdm_dims& d, Smem& sm, const LayerPlan& L, bool write_tap) {
  const float* z = reinterpret_cast<const float*>(L.router_logits);
  const int E = d.n_experts, k = d.top_k;
  const int lane = lane_id();
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? ld_coh(z + e) : -INFINITY;
  }
  float wsum = 0.f;
  int my_e = 0;
  float my_w = 0.f;
  for (int j = 0; j < k; ++j) {
    // lane-local best: scanning in increasing index order with a strict
    // compare keeps the lowest index among equal values
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int e = lane + 64 * i;
      if (e < E && v[i] > bv) { bv = v[i]; bi = e; }
    }
    // wave maximum, then the lowest index holding it (DPP reductions)
    const float gm = wave_max(bv);
    int bw = wave_min_i(bv == gm ? bi : 0x7fffffff);
    if (bw >= E) bw = 0;  // only when no finite logit is left (never for finite inputs)
    // remove it
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i == bw) v[i] = -INFINITY;
    const float sg = 1.0f / (1.0f + __expf(-gm));
    if (lane == j) { my_e = bw; my_w = sg; }
    wsum += sg;
  }
  if (lane < k) {
    my_w /= wsum;
    sm.route_idx[lane] = my_e;
    sm.route_w[lane] = my_w;
    if (write_tap) {
      gst(reinterpret_cast<int*>(L.topk_idx) + lane, my_e);
      gst(reinterpret_cast<float*>(L.topk_w) + lane, my_w);
    }
    const int t = d.n_shared + lane;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(L.expert_base) + (size_t)my_e * L.expert_stride;
    sm.slot[t] = SlotRef{base + L.egu.codes, base + L.egu.scales};
    sm.slot_w[t] = my_w;
    sm.slot_act[t] = lane * d.moe_ffn;
  }
}

__device__ __forceinline__ void route_wave(const pdm_dims& d, Smem& sm, const LayerPlan& L, bool write_tap) {
  if (d.n_experts <= 256) route_wave_t<4>(d, sm, L, write_tap);
  else route_wave_t<16>(d, sm, L, write_tap);
}

// Slot tables of a MoE stage: expert matrix pointers, gate weights and act
// offsets. Gate/up (row slots): shared experts in slots [0, n_shared) (which
// need no routing), routed experts in [n_shared, n_shared + top_k). Down
// (K slots, in act order): routed experts first, then the shared ones. Routed
// slots use the layer's top-k in LDS.
__device__ __forceinline__ void set_slots(const pdm_dims& d, const LayerPlan& L, Smem& sm, bool shared, bool routed,
                                          bool down) {
  const int t = threadIdx.x;
  const int ns = d.n_shared, k = d.top_k;
  if (t < ns + k) {
    const bool is_shared = down ? t >= k : t < ns;
    if (is_shared ? !shared : !routed) return;
    const int i = down ? (is_shared ? t - k : t) : (is_shared ? t : t - ns);  // index among its kind
    const int e = is_shared ? d.n_experts + i : sm.route_idx[i];
    const uint8_t* base = reinterpret_cast<const uint8_t*>(L.expert_base) + (size_t)e * L.expert_stride;
    const Fp8Mat& m = down ? L.edown : L.egu;
    sm.slot[t] = SlotRef{base + m.codes, base + m.scales};
    sm.slot_w[t] = down || is_shared ? 1.f : sm.route_w[i];
    sm.slot_act[t] = (is_shared ? k + i : i) * d.moe_ffn;
  }
}

// --- GU: SwiGLU gate/up of the dense FFN (rows gate/up interleaved in groups of 8)
__device__ __forceinline__ bool stage_gu(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const LayerPlan L = layer_of(c, E.st.layer);
  const float* xa = reinterpret_cast<const float*>(L.xa);
  float* act = reinterpret_cast<float*>(L.act);
  Gemv g = gemv_of(L.gu);
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  float rs = 1.f;  // 1 / rms of x_attn, applied to the product
  return run_gemv<1, 0>(E, sm, g, ra, rb, true,
      [&]() {
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        stage_norm_vec(sm, d.hidden, reinterpret_cast<const float*>(L.ffn_norm), xa);
        rs = rms_scale(sm, d.hidden, d.rms_eps);
        return true;
      },
      [&](int ca, int n) {
        // rows [gate 8 ; up 8] per group of 16: pair row (ca >> 1) + t
        for (int t = threadIdx.x; t < n / 2; t += kThreads) {
          int grp = t >> 3, r = t & 7;
          float gt = part_sum(sm, grp * 16 + r) * rs;
          float up = part_sum(sm, grp * 16 + 8 + r) * rs;
          st_coh(act + (ca >> 1) + t, silu(gt) * up);
        }
      });
}

// --- GU (MoE): SwiGLU gate/up of the shared and the top-k routed experts in
// one stage. Each workgroup takes a share of the shared-expert rows and a
// share of the routed rows; the shared rows come first, so their weight loads
// go out before the wait for the router logits and stream while this
// workgroup computes the top-k. The router stage this workgroup ran last
// already staged RMSNorm(x_attn) in LDS (kStXStaged).
// EB: 1 FP8 experts, 0 MXFP4 experts (input staged in xperm4 order).
template <int EB>
__device__ __forceinline__ bool stage_gu_moe_t(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const LayerPlan L = layer_of(c, E.st.layer);
  const float* xa = reinterpret_cast<const float*>(L.xa);
  float* act = reinterpret_cast<float*>(L.act);
  const int F = d.moe_ffn;
  const int rows_sh = 2 * F * d.n_shared;  // row slots [0, n_shared) hold the shared experts
  Gemv g{};
  g.lg_rpv = 31;
  g.Kb = EB == 0 ? d.hidden / 2 : d.hidden;
  g.slot_mode = 1;
  g.lg_slot = 31 - __builtin_clz(2 * F);
  g.slot_Kb = g.Kb;
  g.nkb = L.egu.nkb;
  int p1, e1, p2, e2;
  my_rows(rows_sh, E.st.gran, c.G, c.wg, p1, e1);
  my_rows(2 * F * d.top_k, E.st.gran, c.G, c.wg, p2, e2);
  g.seg_n1 = e1 - p1;
  g.seg_p1 = p1;
  g.seg_p2 = rows_sh + p2;
  g.split = 1;
  const int n = (e1 - p1) + (e2 - p2);
  const bool reuse = (E.st.flags & kStXStaged) != 0;
  set_slots(d, L, sm, true, false, false);
  if (threadIdx.x == 0) sm.slots_ready = 0;
  __syncthreads();
  float rs = 1.f;  // 1 / rms of x_attn, applied to the product
  return run_gemv<EB, 3>(E, sm, g, 0, n, true,
      [&]() {
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        if (!reuse) stage_norm_vec<EB == 0>(sm, d.hidden, reinterpret_cast<const float*>(L.ffn_norm), xa);
        rs = rms_scale(sm, d.hidden, d.rms_eps);  // with reuse: the router stage's sums
        return true;
      },
      [&](int ca, int nr) {
        for (int t = threadIdx.x; t < nr / 2; t += kThreads) {
          int grp = t >> 3, r = t & 7;
          float gt = part_sum(sm, grp * 16 + r) * rs;
          float up = part_sum(sm, grp * 16 + 8 + r) * rs;
          // local gate row -> row-slot row -> pair row across all slots
          const int lr = ca + grp * 16 + r;
          const int pr = lr < g.seg_n1 ? g.seg_p1 + lr : g.seg_p2 + (lr - g.seg_n1);
          const int pair = (pr >> 4) * 8 + (pr & 7);
          const int j = pair / F, f = pair - j * F;
          st_coh(act + sm.slot_act[j] + f, silu(gt) * up * sm.slot_w[j]);
        }
      },
      [&]() { route_wave(d, sm, L, c.wg == 0); });
}


// --- DOWN: x_out = bf16(x_attn + sum_slots W_down[slot] act[slot])
// EB 0: the MoE layer's experts are MXFP4 (input staged in xperm4 order)
template <int EB>
__device__ __forceinline__ bool stage_down_t(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const LayerPlan L = layer_of(c, E.st.layer);
  const float* xa = reinterpret_cast<const float*>(L.xa);
  const float* act = reinterpret_cast<const float*>(L.act);
  float* out = reinterpret_cast<float*>(L.xo);
  Gemv g{};
  int K;
  if (!L.is_moe) {
    g = gemv_of(L.down);
    K = d.ffn;
  } else {
    K = (d.top_k + d.n_shared) * d.moe_ffn;
    g.Kb = EB == 0 ? K / 2 : K;
    g.slot_mode = 2;
    g.slot_Kb = EB == 0 ? d.moe_ffn / 2 : d.moe_ffn;
    g.lg_slot = 31 - __builtin_clz(g.slot_Kb);
    g.nkb = L.edown.nkb;
    g.lg_rpv = 31;
  }
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  // the layer's routing is already in LDS (computed by the gate/up stage)
  if (L.is_moe) {
    set_slots(d, L, sm, true, true, true);
    __syncthreads();
  }
  // the residual x_attn is complete before this stage's dependency (the
  // gate/up stage this workgroup already passed waited for it)
  float res = 0.f;
  const bool res_pre = rb - ra <= kRowChunk;  // one chunk: thread t holds row ra + t
  auto prep = [&]() {
        if (res_pre && (int)threadIdx.x < rb - ra) res = ld_coh(xa + ra + threadIdx.x);
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        if (EB == 0 && L.is_moe) stage_plain_vec<true>(sm, K, act);
        else stage_plain_vec(sm, K, act);
        return true;
      };
  auto epi = [&](int ca, int n) {
        for (int t = threadIdx.x; t < n; t += kThreads)
          st_coh(out + ca + t, round_bf16((res_pre ? res : ld_coh(xa + ca + t)) + part_sum(sm, t)));
      };
  if constexpr (EB == 0) return run_gemv<0, 2>(E, sm, g, ra, rb, true, prep, epi);
  if (L.is_moe) return run_gemv<1, 2>(E, sm, g, ra, rb, true, prep, epi);
  return run_gemv<1, 0>(E, sm, g, ra, rb, true, prep, epi);
}


// --- LM: logits = W_lm * RMSNorm(x), argmax over the vocabulary
__device__ __forceinline__ bool stage_lm(const StageEnv& E, Smem& sm) {
  const Ctx& c = E.c;
  const pdm_dims d = load_plan(&c.P->dims);
  const float* x = reinterpret_cast<const float*>(layer_of(c, d.n_layers - 1).xo);
  float* logits = c.A.logits ? c.A.logits : reinterpret_cast<float*>(c.P->logits_internal);
  Gemv g{};
  g.codes = reinterpret_cast<const uint8_t*>(c.P->lm_head);
  g.Kb = d.hidden * 2;
  g.lg_rpv = 31;
  int ra, rb;
  my_rows(E.st.rows, E.st.gran, c.G, c.wg, ra, rb);
  float bestv = -INFINITY;
  int besti = 0x7fffffff;
  float rs = 1.f;  // 1 / rms of the final hidden state, applied to the product
  bool ok = run_gemv<2, 0>(E, sm, g, ra, rb, true,
      [&]() {
        if (!wait_stage(c, sm, E.st.wait, E.s)) return false;
        stage_norm_vec(sm, d.hidden, reinterpret_cast<const float*>(c.P->final_norm), x);
        rs = rms_scale(sm, d.hidden, d.rms_eps);
        return true;
      },
      [&](int ca, int n) {
        for (int t = threadIdx.x; t < n; t += kThreads) {
          float v = part_sum(sm, t) * rs;
          gst(logits + ca + t, v);
          if (v > bestv || (v == bestv && ca + t < besti)) { bestv = v; besti = ca + t; }
        }
      });
  if (!ok) return false;
  // workgroup argmax
  for (int off = 1; off < 64; off <<= 1) {
    float ov = __shfl_xor(bestv, off);
    int oi = __shfl_xor(besti, off);
    if (ov > bestv || (ov == bestv && oi < besti)) { bestv = ov; besti = oi; }
  }
  if (lane_id() == 0) { sm.red[wave_id()] = bestv; sm.ired[wave_id()] = besti; }
  __syncthreads();
  // workgroup result, then the last workgroup to arrive reduces all of them
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w)
      if (sm.red[w] > bestv || (sm.red[w] == bestv && sm.ired[w] < besti)) { bestv = sm.red[w]; besti = sm.ired[w]; }
    float* best = reinterpret_cast<float*>(c.P->lm_best) + 2 * c.wg;
    st_coh(best, bestv);
    st_coh_i(reinterpret_cast<int*>(best + 1), besti);
    mem_done();
    int* done = counter_ptr(c, c.P->n_stages, 0);
    int old = __hip_atomic_fetch_add(gpw(done), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (uint32_t)old == c.A.epoch * (uint32_t)c.G - 1u;
  }
  __syncthreads();
  if (sm.last && threadIdx.x < 64) {
    // one wave: every lane loads its share of the per-workgroup maxima at once
    const int lane = threadIdx.x;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int w0 = 0; w0 < c.G; w0 += 64 * 4) {
      float v[4];
      int ix[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int wg = w0 + r * 64 + lane;
        const float* bw = reinterpret_cast<const float*>(c.P->lm_best) + 2 * (wg < c.G ? wg : 0);
        v[r] = wg < c.G ? ld_coh(bw) : -INFINITY;
        ix[r] = wg < c.G ? ld_coh_i(reinterpret_cast<const int*>(bw + 1)) : 0x7fffffff;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (v[r] > bv || (v[r] == bv && ix[r] < bi)) { bv = v[r]; bi = ix[r]; }
    }
    for (int off = 1; off < 64; off <<= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0 && c.A.argmax) st_coh_i(c.A.argmax, bi);  // read back by the next step in greedy mode
  }
  return true;
}

// All stages of one decode step, in plan order. Returns false when the step
// was aborted (every workgroup leaves at its next wait).
// XF: the expert format (PDM_FMT_*) the kernel is built for. The MXFP4 stage
// code lives only in that kernel's instance: kernel-wide register allocation
// and instruction-cache footprint of the FP8 kernel stay as they are.
template <int XF>
__device__ __forceinline__ bool run_step(const Ctx& c, Smem& sm, int n, int dpl) {
  for (int s = 0; s < n; ++s) {
    if (c.A.trace && threadIdx.x == 0) sm.t_entry = wall_clock64();
    StageEnv E{c, load_plan(&c.P->stages[s]), s};
    bool ok;
    switch (E.st.type) {
      case PDM_ST_QKV: ok = stage_qkv(E, sm); break;
      case PDM_ST_QB: ok = stage_qb(E, sm); break;
      case PDM_ST_ATTN:
        ok = dpl == 8 ? stage_attn<4>(E, sm) : dpl == 4 ? stage_attn<2>(E, sm) : stage_attn<1>(E, sm);
        break;
      case PDM_ST_UV: ok = stage_uv(E, sm); break;
      case PDM_ST_WO: ok = stage_wo(E, sm); break;
      case PDM_ST_ROUTER: ok = stage_router(E, sm); break;
      case PDM_ST_GU: ok = stage_gu(E, sm); break;
      case PDM_ST_GU_ROUTED:
        ok = XF == PDM_FMT_MXFP4 ? stage_gu_moe_t<0>(E, sm) : stage_gu_moe_t<1>(E, sm);
        break;
      case PDM_ST_DOWN:
        // (dense layers keep FP8 in either kernel)
        ok = XF == PDM_FMT_MXFP4 && (E.st.flags & kStMx) ? stage_down_t<0>(E, sm) : stage_down_t<1>(E, sm);
        break;
      case PDM_ST_LM: ok = stage_lm(E, sm); break;
      default: ok = false; break;
    }
    if (!ok) {
      mem_done();
      return false;
    }
    signal_stage(c, sm, s);
  }
  return true;
}

}  // namespace


// One launch runs A.n_steps decode steps, so the engine can stay resident
// for a whole request (SemiAnalysis TileRT page, how-it-works section: the
// host launches once and execution stays on the device for the decode
// lifecycle). Step j > 0 starts once every workgroup has finished step j - 1
// (the counters of its last stage); its token comes from the token array, or
// in greedy mode is the argmax step j - 1 wrote.
template <int XF>
__global__ void __launch_bounds__(kThreads, 1) engine_kernel(const Plan* __restrict__ P, LaunchArgs A) {
  __shared__ Smem sm;
  Ctx c;
  c.P = (const GLOBAL_AS Plan*)P;
  c.A = A;
  c.epoch0 = A.epoch;
  c.G = c.P->G;
  c.wg = blockIdx.x;
  const int n = c.P->n_stages;
  const int dpl = c.P->dims.kv_lora / 64;
  const int vocab = c.P->dims.vocab;
  for (int step = 0; step < A.n_steps; ++step) {
    if (step > 0) {
      c.A.epoch = A.epoch + step - 1;  // the previous step's last stage, everywhere
      if (!wait_stage(c, sm, n - 1, n - 1)) return;
    }
    c.A.epoch = A.epoch + step;
    c.A.pos = A.pos + step;
    if (A.tokens) {
      const int t = step > 0 && A.greedy ? ld_coh_i(A.argmax + step - 1) : gld(A.tokens + step);
      c.A.token = __builtin_amdgcn_readfirstlane(t);
    }
    if (vocab > 0 && (c.A.token < 0 || c.A.token >= vocab)) {
      // every workgroup sees the same token and leaves; workgroup 0 reports it
      if (c.wg == 0 && threadIdx.x == 0) set_status(c.P->status, c.A.epoch, PDM_ERR_TOKEN, 0, -1, c.A.token);
      return;
    }
    c.A.argmax = A.argmax ? A.argmax + step : nullptr;
    c.A.logits = step + 1 == A.n_steps ? A.logits : nullptr;
    if (!run_step<XF>(c, sm, n, dpl)) return;
  }
}

// ------------------------------------------------------------------ setup kernels

// cos/sin table for RoPE: tab[t][i] = (cos, sin) of t * base^(-2i/d), computed in float64.
__global__ void rope_table_kernel(float* tab, int max_ctx, int rope, double base) {
  const int half = rope / 2;
  const size_t n = (size_t)max_ctx * half;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    int t = (int)(i / half), j = (int)(i % half);
    double inv = pow(base, -2.0 * j / rope);
    double a = (double)t * inv;
    tab[2 * i] = (float)cos(a);
    tab[2 * i + 1] = (float)sin(a);
  }
}

// Offline packer on the device: the logical-to-packed map of pack_src
// (pdm_internal.h), one byte or scale per thread.

__global__ void pack_codes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, PackMap m) {
  const size_t n = (size_t)m.rows * m.Kp;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    int r = (int)(i / m.Kp), k = (int)(i % m.Kp);
    int sr, sc;
    if (pack_src(m, r, k, sr, sc)) dst[i] = src[(size_t)sr * m.K + sc];
  }
}

// Whole packed rows (MXFP4 codes or scales): packed row r is logical row sr
// of the map, row_bytes bytes each.
__global__ void pack_rows_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, PackMap m,
                                 int row_bytes) {
  const size_t n = (size_t)m.rows * row_bytes;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    int r = (int)(i / row_bytes), c = (int)(i % row_bytes);
    int sr, sc;
    if (pack_src(m, r, 0, sr, sc)) dst[i] = src[(size_t)sr * row_bytes + c];
  }
}

// One scale per (8 packed rows, 128 packed columns): the logical block holding
// the tile's first element. The host checks at plan time that every tile lies
// inside one logical 128x128 block.
__global__ void pack_scales_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, PackMap m) {
  const int skb = (m.K + 127) / 128;
  const size_t n = (size_t)(m.rows / 8) * m.nkb;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    int rg = (int)(i / m.nkb), kb = (int)(i % m.nkb);
    int sr, sc;
    if (!pack_src(m, rg * 8, kb * 128, sr, sc)) continue;
    dst[i] = src[(size_t)(sr / 128) * skb + (sc / 128)];
  }
}

}  // namespace pdm

namespace pdm {

// Scratch workspace for callers that cannot allocate device memory: one
// static array per device the library runs on, held until the process ends.
// Host code must not use its name as a device address; its address on a
// device comes from hipGetSymbolAddress with that device current, taken once
// per device and kept.
static __device__ __align__(256) uint8_t scratch[PDM_STATIC_SCRATCH_BYTES];

hipError_t static_scratch(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != device) (void)hipSetDevice(prev);
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t launch_engine(const Plan* plan_dev, const LaunchArgs& a, int G, int expert_format, hipStream_t stream,
                         bool cooperative) {
  const void* k = expert_format == PDM_FMT_MXFP4 ? (const void*)engine_kernel<PDM_FMT_MXFP4>
                                                 : (const void*)engine_kernel<PDM_FMT_FP8>;
  if (cooperative) {
    const Plan* p = plan_dev;
    LaunchArgs args = a;
    void* kargs[] = {(void*)&p, (void*)&args};
    return hipLaunchCooperativeKernel(k, dim3(G), dim3(kThreads), kargs, 0, stream);
  }
  if (expert_format == PDM_FMT_MXFP4)
    hipLaunchKernelGGL(engine_kernel<PDM_FMT_MXFP4>, dim3(G), dim3(kThreads), 0, stream, plan_dev, a);
  else
    hipLaunchKernelGGL(engine_kernel<PDM_FMT_FP8>, dim3(G), dim3(kThreads), 0, stream, plan_dev, a);
  return hipGetLastError();
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  size_t n = bytes / 4;
  int blocks = (int)std::min<size_t>(1024, (n + 255) / 256);
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* tab, int max_ctx, int rope, double base, hipStream_t stream) {
  size_t n = (size_t)max_ctx * (rope / 2);
  int blocks = (int)std::min<size_t>(4096, (n + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, stream, tab, max_ctx, rope, base);
  return hipGetLastError();
}

hipError_t launch_pack_rows(const uint8_t* src, uint8_t* dst, const PackMap& m, int row_bytes, hipStream_t stream) {
  size_t n = (size_t)m.rows * row_bytes;
  int blocks = (int)std::min<size_t>(8192, (n + 255) / 256);
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(pack_rows_kernel, dim3(blocks), dim3(256), 0, stream, src, dst, m, row_bytes);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* src_codes, const uint16_t* src_scales, uint8_t* dst_codes,
                       uint16_t* dst_scales, const PackMap& m, hipStream_t stream) {
  size_t n = (size_t)m.rows * m.Kp;
  int blocks = (int)std::min<size_t>(8192, (n + 255) / 256);
  hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks), dim3(256), 0, stream, src_codes, dst_codes, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t ns = (size_t)(m.rows / 8) * m.nkb;
  int sblocks = (int)std::min<size_t>(4096, (ns + 255) / 256);
  hipLaunchKernelGGL(pack_scales_kernel, dim3(sblocks), dim3(256), 0, stream, src_scales, dst_scales, m);
  return hipGetLastError();
}

}  // namespace pdm
