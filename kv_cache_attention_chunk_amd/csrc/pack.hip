// Ragged cache packing (Pyramid Forcing page, section 2: per-head cache
// policies keep different frame subsets -- stride or periodic samples, or
// adjacent frames merged into one -- and section 3: variable-length caches
// are stored flat with boundary indices, packed in one vectorized pass).
//
// Output frame j of the flat K/V buffers (head bh owns frames
// [frame_ptr[bh], frame_ptr[bh+1])) copies source frame a = src[2j] of its
// head from the dense cache, or, with c = src[2j+1] != -1, merges frames a
// and c: each element is the float32 sum of the two bf16 values times 1/2,
// rounded to bf16 (nearest, ties to even).  Source frames outside the cache
// contribute zeros.  An HBM-bound stream: each thread moves 16-byte chunks
// (8 bf16) of K and of V, with all of its loads issued before its stores.
#include "common.h"

namespace chunkattn {

namespace {

constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 4;            // 16-byte chunks per thread and tensor

typedef __attribute__((ext_vector_type(8))) float f32x8v_t;

__device__ __forceinline__ f32x8v_t unpack8(const u32x4_t x) {
  f32x8v_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[2 * e] = __uint_as_float(x[e] << 16);
    r[2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
  }
  return r;
}

__global__ __launch_bounds__(kPackThreads) void pack_ragged_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int H, int n_frames,
    int64_t sb, int64_t sn, int64_t sh, int T, int d, const int32_t* __restrict__ frame_ptr,
    int BH, int F, const int32_t* __restrict__ src, uint16_t* __restrict__ kf,
    uint16_t* __restrict__ vf, int64_t fs, int32_t* __restrict__ cu) {
  const int j = blockIdx.y;                                  // output frame
  if (blockIdx.x == 0 && j == 0)
    for (int i = threadIdx.x; i <= BH; i += kPackThreads) cu[i] = frame_ptr[i] * T;
  if (j >= F) return;
  // head of frame j: the last bh with frame_ptr[bh] <= j
  int lo = 0, hi = BH - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (frame_ptr[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int bh = lo;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int a = src[2 * j], c = src[2 * j + 1];
  const bool a_ok = a >= 0 && a < n_frames;
  const bool merge = c != -1;
  const bool c_ok = merge && c >= 0 && c < n_frames;
  const int cpr = d / 8;                                     // chunks per token row
  const int total = T * cpr;
  const int64_t head_off = b * sb + h * sh;
  u32x4_t ka[kPackUnroll], va[kPackUnroll], kc[kPackUnroll], vc[kPackUnroll];
  const int base = (blockIdx.x * kPackThreads * kPackUnroll) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const int ch = base + u * kPackThreads;
    const int t = ch / cpr, col = ch - (ch / cpr) * cpr;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    ka[u] = va[u] = kc[u] = vc[u] = z;
    if (ch < total) {
      if (a_ok) {
        const int64_t o = head_off + ((int64_t)a * T + t) * sn + 8 * col;
        ka[u] = *reinterpret_cast<const u32x4_t*>(k + o);
        va[u] = *reinterpret_cast<const u32x4_t*>(v + o);
      }
      if (c_ok) {
        const int64_t o = head_off + ((int64_t)c * T + t) * sn + 8 * col;
        kc[u] = *reinterpret_cast<const u32x4_t*>(k + o);
        vc[u] = *reinterpret_cast<const u32x4_t*>(v + o);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const int ch = base + u * kPackThreads;
    if (ch >= total) continue;
    const int t = ch / cpr, col = ch - (ch / cpr) * cpr;
    const int64_t o = ((int64_t)j * T + t) * fs + 8 * col;
    u32x4_t ko = ka[u], vo = va[u];
    if (merge) {
      // float32 sums (one rounding), exact halving, bf16 round to nearest even
      const bf16x8_t kb = __builtin_convertvector((unpack8(ka[u]) + unpack8(kc[u])) * 0.5f, bf16x8_t);
      const bf16x8_t vb = __builtin_convertvector((unpack8(va[u]) + unpack8(vc[u])) * 0.5f, bf16x8_t);
      ko = __builtin_bit_cast(u32x4_t, kb);
      vo = __builtin_bit_cast(u32x4_t, vb);
    }
    *reinterpret_cast<u32x4_t*>(kf + o) = ko;
    *reinterpret_cast<u32x4_t*>(vf + o) = vo;
  }
}

}  // namespace

hipError_t launch_pack_ragged(const uint16_t* k, const uint16_t* v, int B, int N, int H, int d,
                              const int64_t* ks, int T, const int32_t* frame_ptr,
                              int total_frames, const int32_t* src, uint16_t* kf, uint16_t* vf,
                              int64_t fs, int32_t* cu, hipStream_t stream) {
  const int BH = B * H;
  const int per_block = kPackThreads * kPackUnroll;
  const int gx = (T * (d / 8) + per_block - 1) / per_block;
  const dim3 grid(gx > 0 ? gx : 1, total_frames > 0 ? total_frames : 1);
  // with no frames one workgroup still writes the boundary indices
  hipLaunchKernelGGL(pack_ragged_kernel, grid, dim3(kPackThreads), 0, stream, k, v, H, N / T,
                     ks[0], ks[1], ks[2], T, d, frame_ptr, BH, total_frames, src, kf, vf, fs, cu);
  return hipGetLastError();
}

}  // namespace chunkattn
