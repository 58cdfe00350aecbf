// synth_dev.hip -- device fill kernels of the seeded synthetic input generator.
//
// Input generation only (no routed-MoE arithmetic).  The kernels evaluate the
// same counter-based definitions as the host generator (synth_core.h), so a
// buffer filled here holds exactly the bytes that synth_host.c would write; this
// is what lets the large weight stacks be generated in device memory directly.
// Built with -ffp-contract=off so the double multiply and add of the scale and
// uniform draws stay separately rounded, as on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_FN static inline __host__ __device__
#include "synth_core.h"

namespace {

__global__ void k_fill_codes(uint32_t* __restrict__ dst, uint64_t nw, uint64_t key) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nw; j += stride)
    dst[j] = syn_code_word(key, j);
}

__global__ void k_fill_scales(uint16_t* __restrict__ dst, uint64_t n, uint64_t key, double lo,
                              double width, int is_f16) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = syn_scale(key, j, lo, width, is_f16);
}

__global__ void k_fill_uniform_bf16(uint16_t* __restrict__ dst, uint64_t n, uint64_t key,
                                    double a) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = syn_uniform_bf16(key, j, a);
}

unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  if (g == 0) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

// Each returns a hipError_t value (0 = success).  dst must be device memory
// holding at least the bytes written; nbytes is a multiple of 4.
int syn_dev_fill_codes(void* dst, uint64_t nbytes, uint64_t seed, uint64_t layer, uint64_t expert,
                       uint64_t matrix, hipStream_t stream) {
  if (nbytes % 4) return (int)hipErrorInvalidValue;
  uint64_t key = syn_key(seed, layer, SYN_CODES, expert, matrix);
  uint64_t nw = nbytes / 4;
  hipLaunchKernelGGL(k_fill_codes, dim3(grid_for(nw)), dim3(256), 0, stream, (uint32_t*)dst, nw,
                     key);
  return (int)hipGetLastError();
}

int syn_dev_fill_scales(void* dst, uint64_t n, uint64_t seed, uint64_t layer, uint64_t expert,
                        uint64_t matrix, double lo, double width, int is_f16, hipStream_t stream) {
  uint64_t key = syn_key(seed, layer, SYN_SCALES, expert, matrix);
  hipLaunchKernelGGL(k_fill_scales, dim3(grid_for(n)), dim3(256), 0, stream, (uint16_t*)dst, n,
                     key, lo, width, is_f16);
  return (int)hipGetLastError();
}

int syn_dev_fill_uniform_bf16(void* dst, uint64_t n, uint64_t seed, uint64_t layer, uint64_t field,
                              uint64_t expert, uint64_t matrix, double a, hipStream_t stream) {
  uint64_t key = syn_key(seed, layer, field, expert, matrix);
  hipLaunchKernelGGL(k_fill_uniform_bf16, dim3(grid_for(n)), dim3(256), 0, stream,
                     (uint16_t*)dst, n, key, a);
  return (int)hipGetLastError();
}

}  // extern "C"
