// Block selection kernels for the block-sparse cache mode (Sparse Forcing
// page, section 2): block representatives (mean of each block's tokens),
// coarse scores against those representatives with per-query-block top-K,
// and assembly of the PBSA block lists (sink + persistent + top-K local).
#include "common.h"

namespace chunkattn {

namespace {

// ---------------------------------------------------------------------------
// Block mean.  One workgroup per (b*H + h, block).  d/8 threads cover a row
// with 16-byte loads; 256/(d/8) rows are summed in parallel in float32 and
// the row groups are reduced through LDS.  HBM-bound stream of x.
// ---------------------------------------------------------------------------
constexpr int kMeanThreads = 256;

__global__ __launch_bounds__(kMeanThreads) void block_mean_kernel(
    const uint16_t* __restrict__ x, int N, int H, int d, int64_t sb, int64_t sn, int64_t sh,
    int block, int seg, int bps, int nb, float* __restrict__ out) {
  __shared__ float red[kMeanThreads * 8];
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - (bh / H) * H;
  int start, len;
  block_span(blk, N, block, seg, bps, start, len);
  const int tpr = d / 8;                    // threads per row
  const int rpp = kMeanThreads / tpr;       // rows in parallel
  const int tid = threadIdx.x;
  const int rg = tid / tpr;
  const int c = tid - rg * tpr;
  float accv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (rg < rpp) {
    const uint16_t* base = x + b * sb + h * sh + (int64_t)start * sn + c * 8;
    for (int r = rg; r < len; r += rpp) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + (int64_t)r * sn);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        accv[2 * e] += __uint_as_float(v[e] << 16);
        accv[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tid * 8 + e] = accv[e];
  __syncthreads();
  // thread j < d sums element j over the row groups (fixed order)
  for (int j = tid; j < d; j += kMeanThreads) {
    const int cc = j / 8, e = j - (j / 8) * 8;
    float s = 0.f;
    for (int g = 0; g < rpp; ++g) s += red[(g * tpr + cc) * 8 + e];
    out[((int64_t)bh * nb + blk) * d + j] = len > 0 ? s / (float)len : 0.f;
  }
}

// Mean over all N tokens of each (b, h) from its block means: sum over blocks
// of len_j * mean_j (block order, float32) divided by N.  One workgroup per
// (b, h), one thread per d-element.
__global__ __launch_bounds__(kMeanThreads) void total_mean_kernel(
    const float* __restrict__ means, int N, int block, int seg, int bps, int nb, int d,
    float* __restrict__ out) {
  const int bh = blockIdx.x;
  for (int j = threadIdx.x; j < d; j += kMeanThreads) {
    float s = 0.f;
    for (int blk = 0; blk < nb; ++blk) {
      int start, len;
      block_span(blk, N, block, seg, bps, start, len);
      s = fmaf((float)len, means[((int64_t)bh * nb + blk) * d + j], s);
    }
    out[(int64_t)bh * d + j] = N > 0 ? s / (float)N : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Coarse scores + top-K.  One workgroup per (b*H + h, query block): every
// thread scores candidates with a float32 dot product over d (sequential
// fused multiply-adds in index order), then a bitonic sort in LDS orders the
// padded list by (score descending, block id ascending) and a second bitonic
// sort puts the first K ids in ascending order.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 256;
constexpr int kTopkMaxCand = 4096;

__device__ __forceinline__ bool before(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

__global__ __launch_bounds__(kTopkThreads) void score_topk_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, int NQB, int NKB, int d,
    int cand_begin, int cand_count, int K, int npad, int kpad, int32_t* __restrict__ out_idx,
    float* __restrict__ out_score) {
  __shared__ float qs[512];
  __shared__ float ss[kTopkMaxCand];
  __shared__ int is[kTopkMaxCand];
  const int qb = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const float* q = qm + ((int64_t)bh * NQB + qb) * d;
  for (int j = tid; j < d; j += kTopkThreads) qs[j] = q[j];
  __syncthreads();
  for (int j = tid; j < npad; j += kTopkThreads) {
    if (j < cand_count) {
      const float* kr = km + ((int64_t)bh * NKB + cand_begin + j) * d;
      float acc = 0.f;
      for (int c = 0; c < d; c += 4) {
        const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kr + c);
        acc = fmaf(qs[c], kv[0], acc);
        acc = fmaf(qs[c + 1], kv[1], acc);
        acc = fmaf(qs[c + 2], kv[2], acc);
        acc = fmaf(qs[c + 3], kv[3], acc);
      }
      ss[j] = acc;
      is[j] = cand_begin + j;
    } else {
      ss[j] = -INFINITY;
      is[j] = 0x7FFFFFFF;
    }
  }
  __syncthreads();
  // bitonic sort of npad entries: (score desc, id asc)
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < npad; i += kTopkThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;   // this run ascends in "before" order
          const float si = ss[i], sj = ss[j];
          const int ii = is[i], ij = is[j];
          const bool swap = up ? before(sj, ij, si, ii) : before(si, ii, sj, ij);
          if (swap) {
            ss[i] = sj; ss[j] = si;
            is[i] = ij; is[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  // keep the first K, pad to kpad, sort by id ascending
  for (int i = tid; i < kpad; i += kTopkThreads) {
    if (i >= K) {
      ss[i] = 0.f;
      is[i] = 0x7FFFFFFF;
    }
  }
  __syncthreads();
  for (int size = 2; size <= kpad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < kpad; i += kTopkThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const int ii = is[i], ij = is[j];
          const bool swap = up ? (ij < ii) : (ii < ij);
          if (swap) {
            const float t = ss[i];
            ss[i] = ss[j]; ss[j] = t;
            is[i] = ij; is[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  const int64_t o = ((int64_t)bh * NQB + qb) * K;
  for (int i = tid; i < K; i += kTopkThreads) {
    out_idx[o + i] = is[i];
    if (out_score) out_score[o + i] = ss[i];
  }
}

// ---------------------------------------------------------------------------
// PBSA block lists.  One workgroup of 1024 threads; each thread owns a
// contiguous range of CSR rows.  Row = sorted merge, duplicates dropped, of
// the sink id range, the head's persistent ids and the query block's top-K
// ids (+ offset); all three inputs ascending.  Pass 1 counts, a workgroup
// exclusive scan gives row offsets, pass 2 writes.
// ---------------------------------------------------------------------------
constexpr int kIndexThreads = 1024;

struct Merge3 {
  int s_lo, s_hi;            // sink range [s_lo, s_hi)
  const int32_t* pp; int pc;  // persistent ids
  const int32_t* tp; int tc; int toff;  // top-K ids + offset

  template <bool WRITE>
  __device__ int run(int32_t* dst) const {
    int i = 0, j = 0, n = 0, a = s_lo, last = -2147483647 - 1;
    bool any = false;
    while (a < s_hi || i < pc || j < tc) {
      int v = 0x7FFFFFFF;
      if (a < s_hi) v = a;
      if (i < pc && pp[i] < v) v = pp[i];
      if (j < tc && tp[j] + toff < v) v = tp[j] + toff;
      if (a < s_hi && a == v) ++a;
      if (i < pc && pp[i] == v) ++i;
      if (j < tc && tp[j] + toff == v) ++j;
      if (!any || v != last) {
        if (WRITE) dst[n] = v;
        ++n;
        last = v;
        any = true;
      }
    }
    return n;
  }
};

__global__ __launch_bounds__(kIndexThreads) void build_index_kernel(
    int rows, int sink_begin, int sink_count, const int32_t* __restrict__ pers, int C, int NQB,
    const int32_t* __restrict__ topk, int K, int toff, int32_t* __restrict__ indptr,
    int32_t* __restrict__ indices) {
  __shared__ int scan[kIndexThreads];
  const int tid = threadIdx.x;
  const int per = (rows + kIndexThreads - 1) / kIndexThreads;
  const int r0 = tid * per;
  const int r1 = r0 + per < rows ? r0 + per : rows;
  auto make = [&](int r) {
    Merge3 m;
    m.s_lo = sink_begin;
    m.s_hi = sink_begin + sink_count;
    const int bh = r / NQB;
    m.pp = pers ? pers + (int64_t)bh * C : nullptr;
    m.pc = pers ? C : 0;
    m.tp = topk ? topk + (int64_t)r * K : nullptr;
    m.tc = topk ? K : 0;
    m.toff = toff;
    return m;
  };
  int cnt = 0;
  for (int r = r0; r < r1; ++r) cnt += make(r).template run<false>(nullptr);
  scan[tid] = cnt;
  __syncthreads();
  // Hillis-Steele inclusive scan
  for (int off = 1; off < kIndexThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int pos = scan[tid] - cnt;
  for (int r = r0; r < r1; ++r) {
    indptr[r] = pos;
    pos += make(r).template run<true>(indices + pos);
  }
  if (tid == kIndexThreads - 1) indptr[rows] = scan[tid];
}

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace

hipError_t launch_block_mean(const uint16_t* x, int B, int N, int H, int d, const int64_t* xs,
                             int block, int seg, int bps, int nb, float* out, float* out_total,
                             hipStream_t stream) {
  if (B * H == 0) return hipSuccess;
  if (nb > 0)
    hipLaunchKernelGGL(block_mean_kernel, dim3(nb, B * H), dim3(kMeanThreads), 0, stream, x, N,
                       H, d, xs[0], xs[1], xs[2], block, seg, bps, nb, out);
  if (out_total)
    hipLaunchKernelGGL(total_mean_kernel, dim3(B * H), dim3(kMeanThreads), 0, stream, out, N,
                       block, seg, bps, nb, d, out_total);
  return hipGetLastError();
}

hipError_t launch_score_topk(const float* qm, const float* km, int B, int H, int NQB, int NKB,
                             int d, int cand_begin, int cand_count, int K, int32_t* out_idx,
                             float* out_score, hipStream_t stream) {
  if (B * H == 0 || NQB == 0) return hipSuccess;
  const int npad = next_pow2(cand_count);
  const int kpad = next_pow2(K);
  hipLaunchKernelGGL(score_topk_kernel, dim3(NQB, B * H), dim3(kTopkThreads), 0, stream, qm,
                     km, NQB, NKB, d, cand_begin, cand_count, K, npad, kpad, out_idx,
                     out_score);
  return hipGetLastError();
}

hipError_t launch_build_kv_index(int rows, int sink_begin, int sink_count,
                                 const int32_t* persistent, int C, int NQB, const int32_t* topk,
                                 int K, int topk_offset, int32_t* indptr, int32_t* indices,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(build_index_kernel, dim3(1), dim3(kIndexThreads), 0, stream, rows,
                     sink_begin, sink_count, persistent, C, NQB, topk, K, topk_offset, indptr,
                     indices);
  return hipGetLastError();
}

}  // namespace chunkattn
