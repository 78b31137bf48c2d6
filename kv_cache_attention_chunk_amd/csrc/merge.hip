// LSE merge of a local and a history attention branch (ISPA page, section 2
// item 1: the branches' LSE states let them be recombined after the fact).
// Elementwise and HBM-bound: each thread handles 8 consecutive d-values of
// one (b, n, h) row with 16- or 32-byte loads; the row's LSE is written by
// the thread holding its first 8 values.
#include "common.h"

namespace chunkattn {

namespace {

constexpr int kMergeThreads = 256;

template <bool IN_F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float v[8]) {
  if (IN_F32) {
    const float* p = reinterpret_cast<const float*>(base) + off;
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + off;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(a[e] << 16);
      v[2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
    }
  }
}

template <bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const void* o1, const float* l1, const void* o2, const float* l2, void* o, float* l,
    int H, int N, int d, int64_t total, int64_t s1b, int64_t s1n, int64_t s1h, int64_t s2b,
    int64_t s2n, int64_t s2h, int64_t sob, int64_t son, int64_t soh) {
  const int cpr = d / 8;
  for (int64_t t = blockIdx.x * (int64_t)kMergeThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kMergeThreads) {
    const int64_t row = t / cpr;           // row = (b*N + n)*H + h
    const int c = (int)(t - row * cpr);
    const int h = (int)(row % H);
    const int64_t bn = row / H;
    const int n = (int)(bn % N);
    const int b = (int)(bn / N);
    const int64_t li = ((int64_t)b * H + h) * N + n;
    const float a1 = l1[li], a2 = l2[li];
    const float M = fmaxf(a1, a2);
    float w1 = 0.f, w2 = 0.f, lo = -INFINITY;
    if (M != -INFINITY) {
      w1 = expf(a1 - M);
      w2 = expf(a2 - M);
      lo = M + logf(w1 + w2);
      const float inv = 1.f / (w1 + w2);
      w1 *= inv;
      w2 *= inv;
    }
    float x1[8], x2[8], y[8];
    load8<IN_F32>(o1, b * s1b + n * s1n + h * s1h + 8 * c, x1);
    load8<IN_F32>(o2, b * s2b + n * s2n + h * s2h + 8 * c, x2);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = w1 * x1[e] + w2 * x2[e];
    const int64_t oo = b * sob + n * son + h * soh + 8 * c;
    if (OUT_F32) {
      float* p = reinterpret_cast<float*>(o) + oo;
      *reinterpret_cast<f32x4_t*>(p) = f32x4_t{y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{y[4], y[5], y[6], y[7]};
    } else {
      const f32x8_t yv = {y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7]};
      *reinterpret_cast<bf16x8_t*>(reinterpret_cast<uint16_t*>(o) + oo) =
          __builtin_convertvector(yv, bf16x8_t);
    }
    // o may alias o1 and l may alias l1: the d/8 threads of a row sit in one
    // wavefront (the host requires d/8 to divide 64), and every lane's loads
    // of the row feed the values stored, so all reads precede the writes.
    if (c == 0) l[li] = lo;
  }
}

template <bool I, bool O>
void launch_t(const void* o1, const float* l1, const void* o2, const float* l2, void* o,
              float* l, int B, int H, int N, int d, const int64_t* s1, const int64_t* s2,
              const int64_t* so, hipStream_t stream) {
  const int64_t total = (int64_t)B * N * H * (d / 8);
  int64_t blocks = (total + kMergeThreads - 1) / kMergeThreads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((lse_merge_kernel<I, O>), dim3((unsigned)blocks), dim3(kMergeThreads), 0,
                     stream, o1, l1, o2, l2, o, l, H, N, d, total, s1[0], s1[1], s1[2], s2[0],
                     s2[1], s2[2], so[0], so[1], so[2]);
}

}  // namespace

hipError_t launch_lse_merge(const void* o1, const float* l1, const void* o2, const float* l2,
                            int in_f32, void* o, float* l, int out_f32, int B, int H, int N,
                            int d, const int64_t* s1, const int64_t* s2, const int64_t* so,
                            hipStream_t stream) {
  if ((int64_t)B * H * N == 0) return hipSuccess;
  if (in_f32 && out_f32) launch_t<true, true>(o1, l1, o2, l2, o, l, B, H, N, d, s1, s2, so, stream);
  else if (in_f32) launch_t<true, false>(o1, l1, o2, l2, o, l, B, H, N, d, s1, s2, so, stream);
  else if (out_f32) launch_t<false, true>(o1, l1, o2, l2, o, l, B, H, N, d, s1, s2, so, stream);
  else launch_t<false, false>(o1, l1, o2, l2, o, l, B, H, N, d, s1, s2, so, stream);
  return hipGetLastError();
}

}  // namespace chunkattn
