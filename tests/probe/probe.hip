// probe.hip — test-only checks of gfx950 builtins used by the library:
// the lane layouts of v_mfma_f32_16x16x32_f16 and v_mfma_f32_16x16x4_f32, and
// the single rounding of the packed binary16 fused multiply-add.  Every access
// is within the fixed-size buffers documented per entry point; one wave each.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// a, b: 64 lanes x 8 binary16; d: 64 lanes x 4 floats
__global__ void __launch_bounds__(64) k_mfma32(const f16x8* a, const f16x8* b, f32x4* d) {
  int l = threadIdx.x;
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  d[l] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[l], b[l], c, 0, 0, 0);
}

// a, b: 64 floats; d: 64 lanes x 4 floats
__global__ void __launch_bounds__(64) k_mfma4(const float* a, const float* b, f32x4* d) {
  int l = threadIdx.x;
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  d[l] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[l], b[l], c, 0, 0, 0);
}

// n pairs: out[i] = fma(a[i], b[i], c[i]) on binary16 pairs
__global__ void __launch_bounds__(256) k_pkfma(const f16x2* a, const f16x2* b, const f16x2* c, f16x2* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = __builtin_elementwise_fma(a[i], b[i], c[i]);
}

extern "C" {
int probe_mfma_16x16x32_f16(const void* a, const void* b, float* d) {
  hipLaunchKernelGGL(k_mfma32, dim3(1), dim3(64), 0, 0, (const f16x8*)a, (const f16x8*)b, (f32x4*)d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
int probe_mfma_16x16x4_f32(const float* a, const float* b, float* d) {
  hipLaunchKernelGGL(k_mfma4, dim3(1), dim3(64), 0, 0, a, b, (f32x4*)d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
int probe_pk_fma_f16(const void* a, const void* b, const void* c, void* out, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_pkfma, dim3((n + 255) / 256), dim3(256), 0, 0, (const f16x2*)a, (const f16x2*)b,
                     (const f16x2*)c, (f16x2*)out, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
}
