// Seeded, counter-based input generator (device side).
//
// Input plumbing only: none of the MoE sublayer's arithmetic is here. This is
// the device twin of synth.c, written from the same definition (SplitMix64,
// Steele/Lea/Flood 2014; Box-Muller for normals): element i of a tensor is the
// (i+1)-th output of a SplitMix64 stream whose state starts at
// mix(mix(seed) + tensor). Values are formed in double, rounded once to float
// and, for BF16 outputs, that float is rounded to BF16 (round to nearest even).
// Multiply-add contraction is off so the double arithmetic matches the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__host__ uint64_t host_mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ uint64_t draw(uint64_t base, uint64_t i) {
  return mix64(base + (i + 1ull) * kGolden);
}

__device__ __forceinline__ double uniform_at(uint64_t base, uint64_t i) {
  return (double)(draw(base, i) >> 11) * 0x1.0p-53;
}

__device__ __forceinline__ double normal_at(uint64_t base, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = (double)((draw(base, 2 * p) >> 11) + 1ull) * 0x1.0p-53;
  double u2 = (double)(draw(base, 2 * p + 1) >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u)
    return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// kind: 0 normal -> f32, 1 normal -> bf16, 2 uniform -> f32, 3 uniform -> bf16
__global__ void fill_kernel(void* out, uint64_t base, uint64_t start, int64_t n, double a,
                            double b, int kind) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    uint64_t i = start + (uint64_t)j;
    double v;
    if (kind < 2)
      v = a + b * normal_at(base, i);
    else
      v = a + (b - a) * uniform_at(base, i);
    float fv = (float)v;
    if (kind & 1)
      ((uint16_t*)out)[j] = f32_to_bf16(fv);
    else
      ((float*)out)[j] = fv;
  }
}

int launch(void* out, uint64_t seed, uint64_t tensor, uint64_t start, int64_t n, double a,
           double b, int kind, void* stream) {
  if (n <= 0) return 0;
  if (out == nullptr) return -1;
  uint64_t base = host_mix64(host_mix64(seed) + tensor);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out,
                     base, start, n, a, b, kind);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

extern "C" {
// a = mean, b = std for normals; a = lo, b = hi for uniforms. out is device memory.
int synth_gpu_normal_f32(void* out, uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                         double mean, double stdv, void* stream) {
  return launch(out, seed, tensor, start, n, mean, stdv, 0, stream);
}
int synth_gpu_normal_bf16(void* out, uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                          double mean, double stdv, void* stream) {
  return launch(out, seed, tensor, start, n, mean, stdv, 1, stream);
}
int synth_gpu_uniform_f32(void* out, uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                          double lo, double hi, void* stream) {
  return launch(out, seed, tensor, start, n, lo, hi, 2, stream);
}
int synth_gpu_uniform_bf16(void* out, uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                           double lo, double hi, void* stream) {
  return launch(out, seed, tensor, start, n, lo, hi, 3, stream);
}
}
