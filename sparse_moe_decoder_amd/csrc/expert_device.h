// Device helper shared by the weight-streaming expert kernels (BF16 and MXFP4).
#pragma once
#include "common.h"
#include "kernels.h"
#include "gemm_device.h"

namespace beam {

// The expert of workgroup slot `slot` of a streaming launch (grid sized for the
// largest possible number of active experts); -1 if fewer experts are active.
__device__ __forceinline__ int active_expert(const ExpertArgs& a, int slot) {
  // slot < E, so active[slot] is in bounds: both loads are issued before either is used
  const int na = *a.n_active, e = a.active[slot];
  asm volatile("" ::"s"(na), "s"(e));
  return slot < na ? e : -1;
}

// First row and row count of active expert e. Scalar loads (constant address space): the
// offsets are written only by earlier launches, and a scalar load is counted apart from
// the vector loads, so waiting for it never waits for weights already in flight.
__device__ __forceinline__ void expert_rows(const ExpertArgs& a, int e, int& row0, int& cnt) {
  const auto* off = (const __attribute__((address_space(4))) int*)a.offsets;
  row0 = off[e];
  cnt = off[e + 1] - row0;
}

__device__ __forceinline__ int expert_of_block(const ExpertArgs& a, int slot, int& row0,
                                               int& cnt) {
  const int e = active_expert(a, slot);
  if (e >= 0) expert_rows(a, e, row0, cnt);
  return e;
}

// Single-token passes (T = 1): every active expert holds the one token row, so each wave
// stages its K quarter of that row into LDS once (nc 16-byte chunks, chunk c = values
// 8c .. 8c + 7 of the quarter, at xs[c]) and reads the MFMA A operand from there, leaving
// the register ring to the weights alone. The row arrives by direct global-to-LDS copies
// (lds_dma16), which the compiler does not count: one_row_wait<N>, with N the number of
// vector loads issued after the copies, waits for them. Both passes issue them before their
// weight rings (N = the ring's loads, so the ring stays in flight; down first loads the
// expert's offset, a scalar load, for the row address: measured faster than issuing its ring
// first and waiting for all of it with the row), so the loop's own waits name exactly the
// ring's oldest slot. Lanes past the last chunk
// re-read it into positions past nc (xs holds kOneRowChunks * 64 chunks): every lane issues
// the same copies, with no branch.
constexpr int kOneRowChunks = 4;  // chunks per lane: a K quarter of at most 2048 values

__device__ __forceinline__ void one_row_load(u32x4* xs, const uint16_t* src, int nc, int lane) {
#pragma unroll
  for (int i = 0; i < kOneRowChunks; ++i)
    lds_dma16(src + min(i * 64 + lane, nc - 1) * 8, lds_addr(xs + i * 64));
}

template <int N>
__device__ __forceinline__ void one_row_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace beam
