// Fused sublayer boundary: post-RMSNorm -> depth-scaled residual -> next pre-RMSNorm.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §MoE und Residual-Stream]
//   sandwich norm; the n-th residual add is h <- sqrt((n-1)/n) h + x / sqrt(n).
// [same page, §Agentengetriebene Optimierung, change 1] post-norm, scaled add and
//   next pre-norm as one kernel with FP32 math and BF16 rounding points.
// [SGLang "SGLang 支撑编程模型 Beam 生产部署", §三明治归一化与深度缩放残差]
//   both scaled operands are rounded to BF16 before the add.
//
// A row of d BF16 values is read as 16-byte chunks (consecutive lanes read
// consecutive 16 bytes) and stays in registers between the three phases (sum of
// squares of x; scaled add and sum of squares of h'; pre-norm), so each row costs
// 2 reads and 2 writes of d BF16 values. Rows up to 8192 wide get a workgroup
// each (one chunk per lane); wider rows one wavefront each.
#include "boundary_device.h"
#include "combine_device.h"

namespace beam {

// One workgroup per row (rows up to kBoundaryWgMaxD wide): one 16-byte chunk per lane, W =
// ceil(d / 512) waves. Each sum of squares is a per-lane sum of its chunk, a wave
// sum, then the W wave sums added in wave order through LDS; every lane forms the
// same total. The whole row is in flight after one round of loads.
// COMBINE: x is the weighted combine of the token's expert rows (combine_chunk), formed
// in place of the load of x (and written to c.y when that is not null): the MoE
// output crosses into the next sublayer's boundary without a round trip through HBM.
template <bool COMBINE>
__global__ __launch_bounds__(1024) void boundary_row_wg_kernel(BoundaryArgs a, CombineArgs cb) {
  __shared__ float red[2][16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int64_t t = blockIdx.x;
  const int nch = a.d >> 3;
  const int idx = threadIdx.x;
  const bool ok = idx < nch;
  const int li = ok ? idx : 0;
  // h and the norm weights first: with COMBINE their loads run under the combine's
  // dependent loads (ids, then the expert rows)
  u32x4 hv = ld_u32x4((const u32x4*)(a.h + t * a.d) + li);
  const u32x4 wo = ld_u32x4((const u32x4*)a.w_post + li);
  const u32x4 wr = ld_u32x4((const u32x4*)a.w_pre + li);
  u32x4 xv;
  if constexpr (COMBINE) {
    xv = combine_chunk(t, li, cb.k, a.d, cb.E, cb.ids, cb.yk);
    if (cb.y && ok) st_u32x4((u32x4*)(cb.y + t * a.d) + idx, xv);
  } else {
    xv = ld_u32x4((const u32x4*)(a.x + t * a.d) + li);
  }
  float ss = wave_sum(ok ? sumsq8(xv) : 0.0f);
  if (lane == 0) red[0][wv] = ss;
  __syncthreads();
  ss = 0.0f;
  for (int w = 0; w < nw; ++w) ss += red[0][w];
  const float r = rms_scale(ss, a.d, a.eps);
  float ss2 = 0.0f;
  const u32x4 xn = norm8(xv, r, wo);
  hv = residual8(hv, xn, a.c1, a.c2, ss2);
  if (ok) st_u32x4((u32x4*)(a.h_out + t * a.d) + idx, hv);
  ss2 = wave_sum(ok ? ss2 : 0.0f);
  if (lane == 0) red[1][wv] = ss2;
  __syncthreads();
  ss2 = 0.0f;
  for (int w = 0; w < nw; ++w) ss2 += red[1][w];
  const float r2 = rms_scale(ss2, a.d, a.eps);
  if (ok) st_u32x4((u32x4*)(a.z_out + t * a.d) + idx, norm8(hv, r2, wr));
}

// Wider rows: one wavefront per row, re-reading x and h' instead of keeping the row
// in registers.
__global__ __launch_bounds__(256) void boundary_rows_wide_kernel(BoundaryArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int nch = a.d >> 3;
  const u32x4* xr = (const u32x4*)(a.x + t * a.d);
  const u32x4* hr = (const u32x4*)(a.h + t * a.d);
  const u32x4* wpo = (const u32x4*)a.w_post;
  const u32x4* wpr = (const u32x4*)a.w_pre;
  u32x4* ho = (u32x4*)(a.h_out + t * a.d);
  u32x4* zo = (u32x4*)(a.z_out + t * a.d);
  float ss = 0.0f;
  for (int idx = lane; idx < nch; idx += 64) ss += sumsq8(ld_u32x4(xr + idx));
  const float r = rms_scale(wave_sum(ss), a.d, a.eps);
  float ss2 = 0.0f;
  for (int idx = lane; idx < nch; idx += 64) {
    u32x4 xn = norm8(ld_u32x4(xr + idx), r, ld_u32x4(wpo + idx));
    st_u32x4(ho + idx, residual8(ld_u32x4(hr + idx), xn, a.c1, a.c2, ss2));
  }
  const float r2 = rms_scale(wave_sum(ss2), a.d, a.eps);
  // each lane re-reads only the chunks it wrote itself
  for (int idx = lane; idx < nch; idx += 64)
    st_u32x4(zo + idx, norm8(ld_u32x4(ho + idx), r2, ld_u32x4(wpr + idx)));
}

hipError_t launch_boundary(const BoundaryArgs& a, hipStream_t s) {
  // the choice depends on d only, so a row's result does not depend on T
  if (a.d <= kBoundaryWgMaxD) {
    const int nv = ((a.d >> 3) + 63) / 64;
    hipLaunchKernelGGL(boundary_row_wg_kernel<false>, dim3((unsigned)a.T), dim3(64 * nv), 0, s, a,
                       CombineArgs{});
  } else {
    hipLaunchKernelGGL(boundary_rows_wide_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine_boundary(const BoundaryArgs& b, const CombineArgs& c, hipStream_t s) {
  const int nv = ((b.d >> 3) + 63) / 64;
  hipLaunchKernelGGL(boundary_row_wg_kernel<true>, dim3((unsigned)b.T), dim3(64 * nv), 0, s, b, c);
  return hipGetLastError();
}

}  // namespace beam
