// Roof probes for the benchmark (built into libchunkattn_roofs.so, not part
// of the chunk-attention ABI): the bf16 matrix-core peak and the HBM read
// bandwidth this GPU reaches, to put the attention kernels' rates next to
// measured denominators as well as the datasheet's.
//
// roof_mfma_kernel: every wave keeps four independent v_mfma_f32_32x32x16_bf16
// accumulator chains busy for `iters` rounds (4 MFMAs = 131072 FLOP per wave
// and round); operands stay in registers, so nothing but the matrix cores is
// exercised.  The accumulators are stored only when `sink` is non-zero (the
// caller passes 0), which keeps the compiler from dropping the work.
//
// roof_read_kernel: streams `n16` 16-byte words with fully coalesced loads
// (each wave reads 1 KB per instruction, four instructions in flight) and
// folds them into a register that is stored only when `sink` is non-zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__global__ __launch_bounds__(256) void roof_mfma_kernel(int iters, int sink, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  if (sink) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  }
}

__global__ __launch_bounds__(256) void roof_read_kernel(const u32x4_t* __restrict__ x, int64_t n16,
                                                        int sink, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t v0 = x[i], v1 = x[i + stride], v2 = x[i + 2 * stride], v3 = x[i + 3 * stride];
    acc ^= v0[0] ^ v0[3] ^ v1[1] ^ v1[2] ^ v2[0] ^ v2[3] ^ v3[1] ^ v3[2];
  }
  for (; i < n16; i += stride) acc ^= x[i][0];
  if (sink) out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// FLOPs the MFMA probe performs: grid x 4 waves x iters x 4 x 32768.
int ca_roof_mfma(int grid, int iters, float* sink_buf, void* stream) {
  if (grid <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(roof_mfma_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, 0, sink_buf);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int ca_roof_read(const void* x, int64_t bytes, int grid, uint32_t* sink_buf, void* stream) {
  if (grid <= 0 || bytes < 16 || (reinterpret_cast<uintptr_t>(x) & 15)) return 1;
  hipLaunchKernelGGL(roof_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(x), bytes / 16, 0, sink_buf);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
