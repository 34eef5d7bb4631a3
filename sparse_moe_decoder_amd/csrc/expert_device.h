// Device helper shared by the weight-streaming expert kernels (BF16 and MXFP4).
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

// The expert of workgroup slot `slot` of a streaming launch (grid sized for the
// largest possible number of active experts), its first row and row count; -1 if
// fewer experts are active.
__device__ __forceinline__ int expert_of_block(const ExpertArgs& a, int slot, int& row0,
                                               int& cnt) {
  // slot < E, so active[slot] is in bounds: both loads are issued before either is used
  const int na = *a.n_active, e = a.active[slot];
  asm volatile("" ::"s"(na), "s"(e));
  if (slot >= na) return -1;
  row0 = a.offsets[e];
  cnt = a.offsets[e + 1] - row0;
  return e;
}

}  // namespace beam
