// Device filler for the seeded synthetic inputs: the same definitions as the
// host filler (both include synth_core.h), used to fill multi-gigabyte weight
// sets in device memory without a host round trip. Launch-only C ABI; every
// call is asynchronous on the given stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "synth_core.h"

namespace {

__global__ void fill_f32_kernel(float* out, int64_t n, uint64_t base, float c, int64_t idx0) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = msk_syn_normal(base, (uint64_t)(idx0 + i), c);
}

__global__ void fill_bf16_kernel(uint16_t* out, int64_t n, uint64_t base, float c, int64_t idx0) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = msk_syn_bf16(msk_syn_normal(base, (uint64_t)(idx0 + i), c));
}

__global__ void fill_nvfp4_kernel(uint8_t* codes, uint8_t* scales, int64_t nblk, uint64_t base,
                                  float c, float s_tensor) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    uint8_t c8[8];
    scales[b] = msk_syn_nvfp4_block(base, (uint64_t)b * 16u, c, s_tensor, c8);
    uint2 v;
    v.x = (uint32_t)c8[0] | ((uint32_t)c8[1] << 8) | ((uint32_t)c8[2] << 16) | ((uint32_t)c8[3] << 24);
    v.y = (uint32_t)c8[4] | ((uint32_t)c8[5] << 8) | ((uint32_t)c8[6] << 16) | ((uint32_t)c8[7] << 24);
    *reinterpret_cast<uint2*>(codes + b * 8) = v;
  }
}

float normal_const(float std) { return (float)((double)std * sqrt(3.0) / 65536.0); }

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" int msk_synth_gpu_fill_f32(float* out, int64_t n, uint64_t seed, uint64_t stream,
                                      float std, int64_t idx0, hipStream_t s) {
  if (n <= 0) return 0;
  fill_f32_kernel<<<grid_for(n), 256, 0, s>>>(out, n, msk_syn_base(seed, stream), normal_const(std), idx0);
  return (int)hipGetLastError();
}

extern "C" int msk_synth_gpu_fill_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream,
                                       float std, int64_t idx0, hipStream_t s) {
  if (n <= 0) return 0;
  fill_bf16_kernel<<<grid_for(n), 256, 0, s>>>(out, n, msk_syn_base(seed, stream), normal_const(std), idx0);
  return (int)hipGetLastError();
}

extern "C" int msk_synth_gpu_fill_nvfp4(uint8_t* codes, uint8_t* scales, int64_t rows, int64_t cols,
                                        uint64_t seed, uint64_t stream, float std, float s_tensor,
                                        hipStream_t s) {
  if (cols % 16 != 0) return 1;
  int64_t nblk = rows * (cols / 16);
  if (nblk <= 0) return 0;
  if (((uintptr_t)codes & 7u) != 0) return 1;
  fill_nvfp4_kernel<<<grid_for(nblk), 256, 0, s>>>(codes, scales, nblk, msk_syn_base(seed, stream),
                                                   normal_const(std), s_tensor);
  return (int)hipGetLastError();
}
