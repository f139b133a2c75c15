// Device-wide maximum of one non-negative float per workgroup, returned to
// every workgroup of the grid (a grid barrier that carries the maximum).
//
// Every workgroup of the grid must be resident at once; the host sizes the
// grid from the kernel's occupancy.  Wave 0 of each workgroup takes part;
// the other waves wait at the workgroup barrier that follows.
//
// Same-address device-scope atomics serialize at the memory side (about
// 40 ns each on gfx950 with every workgroup polling the same word: a flat
// counter costs 11 us at 256 workgroups and 31 us at 768), so the barrier is
// a two-level tree of fan-in kGroup with the polling spread over the groups:
//  * each workgroup stores its maximum to its own partial slot, waits for
//    the store to complete, and counts itself in its group's counter;
//  * the last arrival of a group reduces the group's partials into the
//    group's slot and counts the group in the top counter;
//  * the last group reduces the group maxima, publishes the result, clears
//    every counter (all have arrived, none is touched again in this call)
//    and bumps every group's release flag;
//  * each workgroup polls its own group's flag, whose value it read before
//    arriving, so the flags never need clearing.
// All accesses are relaxed device-scope atomics performed at the coherence
// point; their order comes from waiting for completion (s_waitcnt) between
// dependent steps.  The wait is bounded: a grid that cannot become resident
// gets a NaN after about a second instead of hanging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

constexpr int kGroup = 32;                  // workgroups per first-level group
constexpr int kMaxGroups = 64;              // groups (one per lane of wave 0)
constexpr int kGridMaxWgs = kGroup * kMaxGroups;
constexpr unsigned kGridSpinLimit = 1u << 21;

// One barrier's state; every counter and flag on its own 128-byte line.
struct GridMaxSlot {
  unsigned cnt[kMaxGroups][32];    // group arrival counters (word 0 of each line)
  unsigned flag[kMaxGroups][32];   // group release flags (word 0 of each line)
  unsigned top[32];                // group counter (word 0)
  float result[32];                // the maximum (word 0)
  float part[kGridMaxWgs];         // per-workgroup maxima
  float gpart[kMaxGroups];         // per-group maxima
};

__device__ __forceinline__ void grid_wait_mem() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T gm_load(T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void gm_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned gm_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Called by all 64 lanes of wave 0 with the workgroup's maximum m (the same
// value in every lane); returns the grid's maximum (NaN on a timeout).
__device__ __forceinline__ float grid_max_wave0(GridMaxSlot* s, float m) {
  const int lane = threadIdx.x & 63;
  const unsigned nwg = gridDim.x, b = blockIdx.x, k = b / kGroup;
  const unsigned ngroups = (nwg + kGroup - 1) / kGroup;
  const unsigned gsize = min((unsigned)kGroup, nwg - k * kGroup);
  unsigned f0 = 0, last_wg = 0;
  if (lane == 0) {
    f0 = gm_load(&s->flag[k][0]);
    gm_store(&s->part[b], m);
    grid_wait_mem();   // the flag is read and the partial stored before arriving
    last_wg = gm_add(&s->cnt[k][0], 1u) == gsize - 1;
  }
  f0 = __shfl(f0, 0);
  if (__shfl(last_wg, 0)) {
    // every partial of the group was stored before its counter moved
    const float gm = wave_max(lane < (int)gsize ? gm_load(&s->part[k * kGroup + lane]) : 0.f);
    unsigned last_grp = 0;
    if (lane == 0) {
      gm_store(&s->gpart[k], gm);
      grid_wait_mem();
      last_grp = gm_add(&s->top[0], 1u) == ngroups - 1;
    }
    if (__shfl(last_grp, 0)) {
      const float a = wave_max(lane < (int)ngroups ? gm_load(&s->gpart[lane]) : 0.f);
      if (lane == 0) gm_store(&s->result[0], a);
      if (lane < (int)ngroups) gm_store(&s->cnt[lane][0], 0u);
      if (lane == 0) gm_store(&s->top[0], 0u);
      grid_wait_mem();   // result and cleared counters land before any release
      if (lane < (int)ngroups) gm_add(&s->flag[lane][0], 1u);
    }
  }
  bool ok = true;
  if (lane == 0) {
    for (unsigned it = 0; gm_load(&s->flag[k][0]) == f0;) {
      if (++it > kGridSpinLimit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  ok = __shfl((int)ok, 0) != 0;
  const float r = gm_load(&s->result[0]);
  return ok ? r : __builtin_nanf("");
}

}  // namespace mxq
