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
// roof_mix_kernel: the instruction mix of the attention tile loop without its
// memory traffic, barriers or data dependencies.  Per round a wave issues
// what one eighth of a 64-key tile step costs it: 4 v_mfma_f32_32x32x16_bf16
// whose A operands come from LDS (2 ds_read_b128 as for K and 4
// ds_read_b64_tr_b16 as for V^T, read one round ahead) and about 16 VALU
// operations (4 v_exp_f32 with their FMAs, 4 adds, 2 max, 2 bf16 packs), the
// packed exponentials feeding the next round's V-side MFMAs as P does.  With
// no memory traffic, barriers or waits on matrix results, its MFMA rate is
// what the tile loop could reach at best on this chip.
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
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

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

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

struct MixOps {
  bf16x8_t k0, k1, va, vb;
};

__device__ __forceinline__ MixOps mix_load(const char* lds, int wbase, int lane, int it) {
  constexpr int kLdsBytes = 16384;
  const int rot = (it & 3) * 1024;
  const int ko = (wbase + rot + 16 * lane) & (kLdsBytes - 16);
  const int vo = (wbase + rot + 8 * lane) & (kLdsBytes - 8);
  MixOps o;
  o.k0 = *reinterpret_cast<const bf16x8_t*>(lds + ko);
  o.k1 = *reinterpret_cast<const bf16x8_t*>(lds + (ko ^ 2048));
  auto tr = [&](int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<char*>(lds + off)));
  };
  const s16x4_t v0 = tr(vo), v1 = tr(vo ^ 512), v2 = tr(vo ^ 1024), v3 = tr(vo ^ 1536);
  o.va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  o.vb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v2, v3, 0, 1, 2, 3, 4, 5, 6, 7));
  return o;
}

// The operands of round it + 1 are read during round it (as the tile loop
// reads ahead; iters is taken as even), the bf16 P operand of the two V-side MFMAs is the previous
// round's packed exponentials, and the issue order is pinned per quarter.
__global__ __launch_bounds__(256) void roof_mix_kernel(int iters, int sink, float* out) {
  constexpr int kLdsBytes = 16384;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += 256)
    reinterpret_cast<u32x4_t*>(lds)[i] = u32x4_t{(uint32_t)i * 0x00010001u, 0x3F803F80u, 0u, 1u};
  __syncthreads();
  bf16x8_t b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(0.002f * (float)(lane - i));
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float e[4], g[4], h0 = -1.f, h1 = -1.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = -0.001f * (float)(lane + i);
    g[i] = 0.f;
  }
  bf16x8_t pb = b;
  const int wbase = (threadIdx.x >> 6) * 4096;   // each address is aligned and inside lds
  auto round = [&](const MixOps& o) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.k0, b, c0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      e[i] = __builtin_amdgcn_exp2f(fmaf(e[i], 0.999f, -0.0001f));
      g[i] += e[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.k1, b, c1, 0, 0, 0);
    h0 = fmaxf(h0, fmaxf(e[0], e[1]));
    const bf16x2_t p01 = __builtin_convertvector((f32x2_t){e[0], e[1]}, bf16x2_t);
    __builtin_amdgcn_sched_barrier(0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.va, pb, c2, 0, 0, 0);
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      e[i] = __builtin_amdgcn_exp2f(fmaf(e[i], 0.999f, -0.0001f));
      g[i] += e[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.vb, pb, c3, 0, 0, 0);
    h1 = fmaxf(h1, fmaxf(e[2], e[3]));
    const bf16x2_t p23 = __builtin_convertvector((f32x2_t){e[2], e[3]}, bf16x2_t);
    const bf16x8_t p8 = __builtin_shufflevector(p01, p23, 0, 1, 2, 3, -1, -1, -1, -1);
    pb = __builtin_shufflevector(pb, p8, 4, 5, 6, 7, 8, 9, 10, 11);
    __builtin_amdgcn_sched_barrier(0);
  };
  // two operand sets alternate: set y is read during round x and vice versa
  MixOps x = mix_load(lds, wbase, lane, 0);
  for (int it = 0; it < iters; it += 2) {
    const MixOps y = mix_load(lds, wbase, lane, it + 1);
    round(x);
    x = mix_load(lds, wbase, lane, it + 2);
    round(y);
  }
  if (sink) {
    float s = h0 + h1 + (float)pb[0];
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) s += e[i] + g[i];
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

// The instruction-mix roof (roof_mix_kernel): FLOPs = grid x 4 waves x iters
// x 4 x 32768 (iters rounded up to even).  grid = 512 puts two waves on every SIMD, as the attention
// kernels run.
int ca_roof_mix(int grid, int iters, float* sink_buf, void* stream) {
  if (grid <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(roof_mix_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
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
