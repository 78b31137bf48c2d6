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

// One or two tensors of the same shape and tiling (blockIdx.z picks one):
// the query and the key block means of the block-sparse path in one launch.
struct MeanSrc {
  const uint16_t* x;
  int64_t sb, sn, sh;
  float* out;
};
struct MeanSrcs {
  MeanSrc s[2];
};

__global__ __launch_bounds__(kMeanThreads) void block_mean_kernel(
    const MeanSrcs srcs, int N, int H, int d, int block, int seg, int bps, int nb) {
  const bool second = blockIdx.z != 0;
  const uint16_t* __restrict__ x = second ? srcs.s[1].x : srcs.s[0].x;
  const int64_t sb = second ? srcs.s[1].sb : srcs.s[0].sb;
  const int64_t sn = second ? srcs.s[1].sn : srcs.s[0].sn;
  const int64_t sh = second ? srcs.s[1].sh : srcs.s[0].sh;
  float* __restrict__ out = second ? srcs.s[1].out : srcs.s[0].out;
  // Partial sums, 8 floats per thread, as two 16-byte halves.  Threads with
  // bit 2 set store their halves swapped, so the 16-byte stores of 8
  // consecutive threads land in 8 different bank groups; a column read of
  // 64 consecutive elements still covers 64 consecutive words.
  __shared__ __attribute__((aligned(16))) float red[kMeanThreads * 8];
  auto red_at = [](int row, int e) { return row * 8 + (e ^ (((row >> 2) & 1) << 2)); };
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
  {
    const int sw = ((tid >> 2) & 1) << 2;
    *reinterpret_cast<f32x4_t*>(red + tid * 8 + sw) = f32x4_t{accv[0], accv[1], accv[2], accv[3]};
    *reinterpret_cast<f32x4_t*>(red + tid * 8 + (4 ^ sw)) = f32x4_t{accv[4], accv[5], accv[6], accv[7]};
  }
  __syncthreads();
  // thread j < d sums element j over the row groups (fixed order)
  for (int j = tid; j < d; j += kMeanThreads) {
    const int cc = j / 8, e = j - (j / 8) * 8;
    float s = 0.f;
    for (int g = 0; g < rpp; ++g) s += red[red_at(g * tpr + cc, e)];
    out[((int64_t)bh * nb + blk) * d + j] = len > 0 ? s / (float)len : 0.f;
  }
}

// Mean over all N tokens of each (b, h) from its block means: sum over blocks
// of len_j * mean_j divided by N.  The arithmetic is fixed by G = 1024 / d
// thread groups whatever the workgroup size: group g sums blocks g, g + G,
// ... in float32 (independent loads, so many are in flight; the block's frame
// and position are stepped along instead of divided out per block), then the
// G partial sums of each column are added in group order.  A workgroup of
// THREADS threads covers the G * d (group, column) slots in THREADS-strided
// passes; `red` is 1024 floats of LDS.  Writes the d means to out (global)
// and, if given, to out_lds.
constexpr int kTotThreads = 1024;

template <int THREADS>
__device__ __forceinline__ void total_mean_row(const float* __restrict__ m, int N, int block,
                                               int seg, int bps, int nb, int d, float* red,
                                               float* __restrict__ out, float* out_lds) {
  const int G = kTotThreads / d;
  for (int slot = threadIdx.x; slot < G * d; slot += THREADS) {
    const int g = slot / d, j = slot - (slot / d) * d;
    int fs = g / bps, fj = g - (g / bps) * bps;       // frame and position of block g
    float s = 0.f;
#pragma unroll 4
    for (int blk = g; blk < nb; blk += G) {
      int seg_len = N - fs * seg;
      seg_len = seg_len < seg ? seg_len : seg;
      int len = seg_len - fj * block;
      len = len < block ? len : block;
      len = len < 0 ? 0 : len;
      s = fmaf((float)len, m[(int64_t)blk * d + j], s);
      fj += G;
      while (fj >= bps) {
        fj -= bps;
        ++fs;
      }
    }
    red[slot] = s;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < d; j += THREADS) {
    float t = 0.f;
    for (int g = 0; g < G; ++g) t += red[g * d + j];
    t = N > 0 ? t / (float)N : 0.f;
    out[j] = t;
    if (out_lds) out_lds[j] = t;
  }
}

// One workgroup of 1024 threads per (b, h).
__global__ __launch_bounds__(kTotThreads) void total_mean_kernel(
    const float* __restrict__ means, int N, int block, int seg, int bps, int nb, int d,
    float* __restrict__ out) {
  __shared__ float red[kTotThreads];
  const int bh = blockIdx.x;
  total_mean_row<kTotThreads>(means + (int64_t)bh * nb * d, N, block, seg, bps, nb, d, red,
                              out + (int64_t)bh * d, nullptr);
}

// ---------------------------------------------------------------------------
// Coarse scores + top-K.  One workgroup per (b*H + h, query block).
//   * scores: float32 dot products.  For d/4 a power of two up to 64, d/4
//     lanes share one candidate (a 16-byte slice each, then a butterfly sum)
//     and the loads of a batch of candidates are all issued before any is
//     used; otherwise each thread scores whole candidates sequentially.
//     A NaN score ranks as -inf.
//   * selection: the K candidates first in (score descending, block id
//     ascending) order, i.e. rank(i) = #{j : s_j > s_i} + #{j < i : s_j =
//     s_i} below K.  Up to kRankMaxCand candidates the ranks are counted
//     directly: F threads share one candidate, each counting a slice of j
//     four scores at a time; the second term is counted only when s_i has a
//     tie.  Above that (the count grows as n^2), a radix select finds the
//     K-th largest score T in four 8-bit digit passes over an order-
//     preserving integer image of the scores, together with the number of
//     T-valued candidates to take (need = K - #{s > T}); the selection is
//     then {s > T} and the first `need` candidates with s = T, the same set.
//     The selected candidates are written in index order, i.e. ascending
//     block id.
// Scores live in dynamic LDS, padded with -inf to a multiple of 4.
// Optionally the kernel also writes each row's PBSA block list (CSR row
// r = (b*H + h)*NQB + qb of W = prefix_count + K entries): the prefix range
// [prefix_begin, prefix_begin + prefix_count) followed by id_offset + the
// selected ids.  The caller guarantees the prefix lies below every selected
// id, so the row is sorted and free of duplicates as written.
// ---------------------------------------------------------------------------
struct TopkLists {
  int32_t* indptr;           // nullptr: no block lists
  int32_t* indices;
  int prefix_begin, prefix_count, id_offset, rows;
};

// With `cm_src`, the job's query (NQB = 1) is the chunk mean, computed by the
// job's own workgroup from the head's query block means cm_src [BH, cm_nb, d]
// (tiling cm_block / cm_seg over cm_N tokens) and also written to qm.
struct TopkJob {
  const float* qm;
  const float* km;
  int NQB, NKB, d, cand_begin, n, K, wg_begin;
  int32_t* out_idx;
  float* out_score;
  TopkLists lists;
  const float* cm_src;
  int cm_N, cm_block, cm_seg, cm_nb;
};
constexpr int kTopkMaxJobs = 4;
constexpr int kTopkBatchThreads = 512;
struct TopkJobs {
  TopkJob j[kTopkMaxJobs];
  int n_jobs;
};

constexpr int kTopkMaxCand = 4096;
constexpr int kTopkBatch = 16;
constexpr int kRankMaxCand = 128;    // larger candidate sets use the radix select

__host__ __device__ constexpr int topk_lds_bytes(int n, int threads) {
  return 4 * (4 * ((n + 3) / 4)) + 4 * n + 8 * (threads / 64);
}

// Order-preserving image of a float score (no NaN) as an unsigned integer:
// -0 is first mapped to +0 so that equal scores have equal images.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// K-th largest of the n scores ss[0..n) (1 <= K <= n) by radix select, most
// significant digit first: each pass histograms the digit of the candidates
// that match the digits chosen so far, and wave 0 finds the digit whose bin
// holds the K-th largest (bins scanned from the top).  Returns T and need =
// its position among the T-valued candidates (1 <= need <= #{s = T}), so
// #{s > T} = K - need.  hist: 256 ints; state: 2 ints (LDS).
template <int THREADS>
__device__ void kth_largest(const float* ss, int n, int K, int* hist, int* state, float& thr,
                            int& need) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, mask = 0;
  int k = K;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += THREADS) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += THREADS) {
      const uint32_t u = order_key(ss[i]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 255 - 4l .. 252 - 4l (descending)
      int c[4], tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * lane - e];
        tot += c[e];
      }
      int incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      int cum = incl - tot;
      if (cum < k && k <= incl) {       // exactly one lane
        bool found = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (!found && cum + c[e] >= k) {
            found = true;
            state[0] = 255 - 4 * lane - e;
            state[1] = k - cum;
          }
          cum += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)state[0] << shift;
    mask |= 0xFFu << shift;
    k = state[1];
  }
  thr = order_key_inv(prefix);
  need = k;
}

// Coarse scores ss[c] = <q, row(c)> for c in [0, n) (a NaN score as -inf),
// and -inf in ss[n .. n_pad); n >= 1 whenever n_pad > 0.  For d/4 a power of two up to 64, d/4 lanes
// share one candidate (a 16-byte slice each, then a butterfly sum) and the
// loads of a batch of candidates are all issued before any is used;
// otherwise each thread scores whole candidates sequentially.
template <int THREADS, class Row>
__device__ __forceinline__ void coarse_scores(const float* q, int d, int n, int n_pad, Row row,
                                              float* ss) {
  const int tid = threadIdx.x;
  auto key = [](float x) { return x != x ? -INFINITY : x; };
  const int lpc = d / 4;                       // lanes per candidate
  if ((lpc & (lpc - 1)) == 0 && lpc <= 64) {
    const int sub = tid & (lpc - 1);
    const int slot = tid / lpc;
    const int per_pass = THREADS / lpc;
    const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(q + 4 * sub);
    for (int c0 = 0; c0 < n_pad; c0 += kTopkBatch * per_pass) {
      f32x4_t kv[kTopkBatch];
      // rows past n load row n - 1 (no branch per load, so the batch's
      // loads all go out together); their scores are replaced below
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u) {
        const int c = c0 + u * per_pass + slot;
        kv[u] = *reinterpret_cast<const f32x4_t*>(row(c < n ? c : n - 1) + 4 * sub);
      }
      float part[kTopkBatch];
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u)
        part[u] = fmaf(qv[3], kv[u][3], fmaf(qv[2], kv[u][2], fmaf(qv[1], kv[u][1], qv[0] * kv[u][0])));
      // butterfly over the lpc lanes of each candidate, the batch's exchanges
      // issued together
      for (int o = lpc >> 1; o > 0; o >>= 1) {
#pragma unroll
        for (int u = 0; u < kTopkBatch; ++u) part[u] += __shfl_xor(part[u], o);
      }
#pragma unroll
      for (int u = 0; u < kTopkBatch; ++u) {
        const int c = c0 + u * per_pass + slot;
        if (sub == 0 && c < n_pad) ss[c] = c < n ? key(part[u]) : -INFINITY;
      }
    }
  } else {
    for (int j = tid; j < n_pad; j += THREADS) {
      float acc = -INFINITY;
      if (j < n) {
        const float* kr = row(j);
        acc = 0.f;
        for (int c = 0; c < d; ++c) acc = fmaf(q[c], kr[c], acc);
        acc = key(acc);
      }
      ss[j] = acc;
    }
  }
}

// One selection row (b*H + h = bh, query block qb) on a whole workgroup;
// topk_lds is the dynamic LDS (topk_lds_bytes(n, THREADS)), hist and rstate
// static LDS.
template <int THREADS>
__device__ void topk_row(const float* __restrict__ qm, const float* __restrict__ km, int NQB,
                         int NKB, int d, int cand_begin, int n, int K,
                         int32_t* __restrict__ out_idx, float* __restrict__ out_score,
                         const TopkLists& lists, int qb, int bh, float* topk_lds, int* hist,
                         int* rstate, const float* q_given = nullptr) {
  const int n4 = (n + 3) >> 2;
  float* ss = topk_lds;                                          // [4 n4] scores
  int* rk = reinterpret_cast<int*>(ss + 4 * n4);                 // [n] ranks
  int* wcount = rk + n;                                          // [2 THREADS / 64]
  const int tid = threadIdx.x;
  const float* q = q_given ? q_given : qm + ((int64_t)bh * NQB + qb) * d;
  const float* kbase = km + ((int64_t)bh * NKB + cand_begin) * d;
  coarse_scores<THREADS>(q, d, n, 4 * n4, [&](int c) { return kbase + (int64_t)c * d; }, ss);
  __syncthreads();

  // selection: the threshold score T and how many T-valued candidates to
  // take, or the ranks themselves for small candidate sets
  const bool radix = n > kRankMaxCand;
  float thr = 0.f;
  int need = 0;
  if (radix) kth_largest<THREADS>(ss, n, K, hist, rstate, thr, need);
  // ranks (padding entries sit above every index, compare as -inf and so
  // never count)
  int F = 1;
  while (F < 64 && n * (2 * F) <= THREADS) F *= 2;
  const int chunk4 = (n4 + F - 1) / F;
  const f32x4_t* ss4 = reinterpret_cast<const f32x4_t*>(ss);
  for (int base = 0; base < (radix ? 0 : n); base += THREADS / F) {
    const int i = base + tid / F;
    const int part = tid & (F - 1);
    int gt = 0, eq = 0;
    float si = 0.f;
    if (i < n) {
      si = ss[i];
      const int b0 = part * chunk4;
      const int b1 = b0 + chunk4 < n4 ? b0 + chunk4 : n4;
#pragma unroll 4
      for (int b = b0; b < b1; ++b) {
        const f32x4_t v = ss4[b];
        gt += (int)(v[0] > si) + (int)(v[1] > si) + (int)(v[2] > si) + (int)(v[3] > si);
        eq += (int)(v[0] == si) + (int)(v[1] == si) + (int)(v[2] == si) + (int)(v[3] == si);
      }
    }
    for (int o = F >> 1; o > 0; o >>= 1) {
      gt += __shfl_xor(gt, o);
      eq += __shfl_xor(eq, o);
    }
    if (i < n && part == 0) {
      if (eq > 1)                              // s_i is tied: lower ids rank first
        for (int j = 0; j < i; ++j) gt += ss[j] == si;
      rk[i] = gt;
    }
  }
  __syncthreads();

  // the K candidates of rank < K, compacted in index order
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t o = ((int64_t)bh * NQB + qb) * K;
  const int W = lists.prefix_count + K;
  const int64_t row = (int64_t)bh * NQB + qb;
  if (lists.indptr) {
    for (int j = tid; j < lists.prefix_count; j += THREADS)
      lists.indices[row * W + j] = lists.prefix_begin + j;
    if (tid == 0) {
      lists.indptr[row] = (int32_t)(row * W);
      if (row == lists.rows - 1) lists.indptr[lists.rows] = lists.rows * W;
    }
  }
  // position of a selected candidate = #{selected j < i} = #{j < i : s_j > T}
  // + min(#{j < i : s_j = T}, need) (with ranks: #{j < i : rank_j < K})
  int carry_gt = 0, carry_eq = 0;
  const unsigned long long below = (1ull << lane) - 1;
  for (int c0 = 0; c0 < n; c0 += THREADS) {
    const int i = c0 + tid;
    bool gt = false, eq = false;
    if (i < n) {
      if (radix) {
        gt = ss[i] > thr;
        eq = ss[i] == thr;
      } else {
        gt = rk[i] < K;
      }
    }
    const unsigned long long mg = __ballot(gt), me = __ballot(eq);
    if (lane == 0) {
      wcount[wave] = __popcll(mg);
      wcount[THREADS / 64 + wave] = __popcll(me);
    }
    __syncthreads();
    int gpre = 0, gtot = 0, epre = 0, etot = 0;
    for (int w = 0; w < THREADS / 64; ++w) {
      const int cg = wcount[w], ce = wcount[THREADS / 64 + w];
      gpre += w < wave ? cg : 0;
      epre += w < wave ? ce : 0;
      gtot += cg;
      etot += ce;
    }
    const int before_eq = carry_eq + epre + __popcll(me & below);
    if (gt || (eq && before_eq < need)) {
      const int before_gt = carry_gt + gpre + __popcll(mg & below);
      const int pos = before_gt + (before_eq < need ? before_eq : need);
      if (pos < K) {
        out_idx[o + pos] = cand_begin + i;
        if (out_score) out_score[o + pos] = ss[i];
        if (lists.indptr) lists.indices[row * W + lists.prefix_count + pos] = lists.id_offset + cand_begin + i;
      }
    }
    carry_gt += gtot;
    carry_eq += etot;
    __syncthreads();
  }
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void score_topk_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, int NQB, int NKB, int d,
    int cand_begin, int n, int K, int32_t* __restrict__ out_idx, float* __restrict__ out_score,
    const TopkLists lists) {
  extern __shared__ __attribute__((aligned(16))) float topk_lds[];
  __shared__ int hist[256];
  __shared__ int rstate[2];
  topk_row<THREADS>(qm, km, NQB, NKB, d, cand_begin, n, K, out_idx, out_score, lists, blockIdx.x,
                    blockIdx.y, topk_lds, hist, rstate);
}

// Several independent selections in one launch (the persistent top-C and
// the local top-K of the block-sparse path run side by side): workgroups
// [wg_begin_j, wg_begin_j + BH_j * NQB_j) serve job j.
__global__ __launch_bounds__(kTopkBatchThreads) void score_topk_batch_kernel(const TopkJobs jobs) {
  extern __shared__ __attribute__((aligned(16))) float topk_lds[];
  __shared__ int hist[256];
  __shared__ int rstate[2];
  int j = 0;
  while (j + 1 < jobs.n_jobs && (int)blockIdx.x >= jobs.j[j + 1].wg_begin) ++j;
  const TopkJob& jb = jobs.j[j];
  const int local = (int)blockIdx.x - jb.wg_begin;
  const int bh = local / jb.NQB;
  const int qb = local - bh * jb.NQB;
  const float* q_given = nullptr;
  if (jb.cm_src) {
    // the chunk-mean query of this head, from its query block means
    __shared__ float red[kTotThreads];
    __shared__ __attribute__((aligned(16))) float cmq[kTotThreads];   // d <= 1024
    const int bps = (jb.cm_seg + jb.cm_block - 1) / jb.cm_block;
    total_mean_row<kTopkBatchThreads>(jb.cm_src + (int64_t)bh * jb.cm_nb * jb.d, jb.cm_N,
                                      jb.cm_block, jb.cm_seg, bps, jb.cm_nb, jb.d, red,
                                      const_cast<float*>(jb.qm) + (int64_t)bh * jb.d, cmq);
    __syncthreads();
    q_given = cmq;
  }
  topk_row<kTopkBatchThreads>(jb.qm, jb.km, jb.NQB, jb.NKB, jb.d, jb.cand_begin, jb.n, jb.K,
                              jb.out_idx, jb.out_score, jb.lists, qb, bh, topk_lds, hist, rstate,
                              q_given);
}

// ---------------------------------------------------------------------------
// PBSA block lists.  One workgroup of 1024 threads.  Row r (head h = r / NQB)
// = sorted union, duplicates dropped, of the sink range S = [s_lo, s_hi),
// the head's persistent ids P_h and the row's top-K ids T_r (+ offset); P and
// T are ascending.
//
// The inputs are staged in LDS when they fit.  With many rows, one thread
// merges whole rows (count pass, workgroup scan, write pass).  With few rows
// (each long), every output element is placed independently:
// an id is kept if no earlier list (S, then P, then T) and no earlier index
// of its own list holds it, and its position in the row is the number of
// distinct ids below it,
//   |S below v| + kept P ids below v + kept T ids below v,
// the last two read from per-list prefix counts of kept flags at the list's
// lower bound of v.  Inputs too large for LDS are merged row by row straight
// from global memory.
// ---------------------------------------------------------------------------
constexpr int kIndexThreads = 1024;
constexpr int kIndexLds = 32768;       // int32 words of LDS (128 KB)

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

// first index in a[0, n) whose value is >= v (a ascending)
__device__ __forceinline__ int lower_bound(const int32_t* a, int n, int v) {
  int lo = 0;
  while (n > 0) {
    const int half = n >> 1;
    if (a[lo + half] < v) {
      lo += half + 1;
      n -= half + 1;
    } else {
      n = half;
    }
  }
  return lo;
}

// Workgroup exclusive scan of per-thread counts; returns this thread's offset
// and writes the total to *total.
__device__ int block_exclusive_scan(int cnt, int* scan, int* total) {
  const int tid = threadIdx.x;
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kIndexThreads; off <<= 1) {   // Hillis-Steele inclusive scan
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  *total = scan[kIndexThreads - 1];
  const int r = scan[tid] - cnt;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kIndexThreads) void build_index_kernel(
    int rows, int sink_begin, int sink_count, const int32_t* __restrict__ pers, int C, int NQB,
    const int32_t* __restrict__ topk, int K, int toff, int32_t* __restrict__ indptr,
    int32_t* __restrict__ indices) {
  __shared__ int scan[kIndexThreads];
  __shared__ int32_t lds[kIndexLds];
  const int tid = threadIdx.x;
  const int per = (rows + kIndexThreads - 1) / kIndexThreads;
  const int r0 = tid * per;
  const int r1 = r0 + per < rows ? r0 + per : rows;
  const int BH = NQB > 0 ? rows / NQB : 0;
  const int nc = pers ? C : 0;
  const int nk = topk ? K : 0;
  const int s_lo = sink_begin, s_hi = sink_begin + sink_count;

  // one thread merges whole rows: count pass, workgroup scan, write pass
  auto merge_rows = [&](const int32_t* P, const int32_t* T, int t_off) {
    auto make = [&](int r) {
      Merge3 m;
      m.s_lo = s_lo;
      m.s_hi = s_hi;
      m.pp = nc ? P + (r / NQB) * nc : nullptr;
      m.pc = nc;
      m.tp = nk ? T + r * nk : nullptr;
      m.tc = nk;
      m.toff = t_off;
      return m;
    };
    int cnt = 0, total;
    for (int r = r0; r < r1; ++r) cnt += make(r).template run<false>(nullptr);
    int pos = block_exclusive_scan(cnt, scan, &total);
    for (int r = r0; r < r1; ++r) {
      indptr[r] = pos;
      pos += make(r).template run<true>(indices + pos);
    }
    if (tid == 0) indptr[rows] = total;
  };

  const int64_t need = (int64_t)BH * (2 * nc + 1) + (int64_t)rows * (2 * nk + 2);
  if (need > kIndexLds) {
    merge_rows(pers, topk, toff);
    return;
  }

  // LDS layout: P [BH][nc], prefP [BH][nc + 1], T [rows][nk] (offset added),
  // prefT [rows][nk + 1], row offsets [rows]
  int32_t* P = lds;
  int* prefP = P + BH * nc;
  int32_t* T = prefP + BH * (nc + 1);
  int* prefT = T + rows * nk;
  int* rowoff = prefT + rows * (nk + 1);
  for (int i = tid; i < BH * nc; i += kIndexThreads) P[i] = pers[i];
  for (int i = tid; i < rows * nk; i += kIndexThreads) T[i] = topk[i] + toff;
  __syncthreads();
  if (rows >= kIndexThreads / 4) {
    // many rows: a thread per row already fills the workgroup
    merge_rows(P, T, 0);
    return;
  }

  // few (long) rows: every output id is placed by its own thread
  auto in_s = [&](int v) { return v >= s_lo && v < s_hi; };
  for (int hh = tid; hh < BH; hh += kIndexThreads) {
    const int32_t* p = P + hh * nc;
    int* pp = prefP + hh * (nc + 1);
    int c = 0;
    pp[0] = 0;
    for (int i = 0; i < nc; ++i) {
      const int v = p[i];
      c += !in_s(v) && (i == 0 || p[i - 1] != v);
      pp[i + 1] = c;
    }
  }
  __syncthreads();
  for (int r = tid; r < rows; r += kIndexThreads) {
    const int32_t* t = T + r * nk;
    const int32_t* p = P + (r / NQB) * nc;
    int* pt = prefT + r * (nk + 1);
    int c = 0;
    pt[0] = 0;
    for (int j = 0; j < nk; ++j) {
      const int v = t[j];
      const int lb = lower_bound(p, nc, v);
      c += !in_s(v) && (j == 0 || t[j - 1] != v) && !(lb < nc && p[lb] == v);
      pt[j + 1] = c;
    }
  }
  __syncthreads();
  auto row_count = [&](int r) {
    return sink_count + prefP[(r / NQB) * (nc + 1) + nc] + prefT[r * (nk + 1) + nk];
  };
  int cnt = 0, total;
  for (int r = r0; r < r1; ++r) cnt += row_count(r);
  int pos = block_exclusive_scan(cnt, scan, &total);
  for (int r = r0; r < r1; ++r) {
    indptr[r] = pos;
    rowoff[r] = pos;
    pos += row_count(r);
  }
  if (tid == 0) indptr[rows] = total;
  __syncthreads();
  const int width = sink_count + nc + nk;          // rows * width < 2^31 (checked by the caller)
  for (int e = tid; e < rows * width; e += kIndexThreads) {
    const int r = e / width;
    const int slot = e - r * width;
    const int hh = r / NQB;
    const int32_t* p = P + hh * nc;
    const int* pp = prefP + hh * (nc + 1);
    const int32_t* t = T + r * nk;
    const int* pt = prefT + r * (nk + 1);
    int v;
    bool keep;
    if (slot < sink_count) {
      v = s_lo + slot;
      keep = true;
    } else if (slot < sink_count + nc) {
      const int i = slot - sink_count;
      v = p[i];
      keep = pp[i + 1] > pp[i];
    } else {
      const int j = slot - sink_count - nc;
      v = t[j];
      keep = pt[j + 1] > pt[j];
    }
    if (!keep) continue;
    const int below_s = v <= s_lo ? 0 : (v >= s_hi ? sink_count : v - s_lo);
    const int at = below_s + pp[lower_bound(p, nc, v)] + pt[lower_bound(t, nk, v)];
    if (at < row_count(r)) indices[rowoff[r] + at] = v;   // always, for ascending inputs
  }
}

// ---------------------------------------------------------------------------
// Persistent-memory update (Sparse Forcing page, section 2 item 1, memory
// management): when the local window slides, its evicted blocks [eb, eb + ne)
// join the head's persistent blocks as candidates and the C best by coarse
// score <q_mean, k_mean[id]> stay.  One workgroup per (b, h):
//   * candidates in LDS: the evicted range, then the persistent ids that lie
//     in [0, NKB) and outside the evicted range (a set union; persistent ids
//     are distinct by contract);
//   * float32 scores, d/4 lanes per candidate as in the top-K kernel (a NaN
//     score ranks as -inf);
//   * rank(i) = #{j : s_j > s_i} + #{j : s_j = s_i, id_j < id_i}, i.e. the
//     position in (score descending, block id ascending) order, counted
//     directly up to kRankMaxCand candidates; above that, the radix select
//     gives the C-th largest score T and the candidates are those above T
//     plus the T-valued ones of lowest id (ties are counted among those
//     only);
//   * the rank < C candidates are written at their position in ascending id
//     order; slots past the candidate count get id -1 and score -inf.
// The persistent row is read into LDS before anything is written, so the
// output may overwrite it in place (same C).
// ---------------------------------------------------------------------------
constexpr int kUpdThreads = 256;

__global__ __launch_bounds__(kUpdThreads) void persistent_update_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, int NKB, int d,
    const int32_t* pers, int C_in, int eb, int ne, int C, int32_t* out,
    float* __restrict__ out_score) {
  // candidates padded to a multiple of 4 (score -inf, id INT_MAX, not kept),
  // so that the comparison loops read 4 at a time
  __shared__ __attribute__((aligned(16))) int ids[kTopkMaxCand];
  __shared__ __attribute__((aligned(16))) float sc[kTopkMaxCand];
  __shared__ __attribute__((aligned(16))) int rk[kTopkMaxCand];
  __shared__ int wcount[kUpdThreads / 64];
  __shared__ int hist[256];
  __shared__ int rstate[2];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < ne; i += kUpdThreads) ids[i] = eb + i;
  // compact the kept persistent ids behind the evicted range
  int n = ne;
  for (int c0 = 0; c0 < C_in; c0 += kUpdThreads) {
    const int i = c0 + tid;
    const int id = i < C_in ? pers[(int64_t)bh * C_in + i] : -1;
    const bool keep = i < C_in && id >= 0 && id < NKB && !(id >= eb && id < eb + ne);
    const unsigned long long m = __ballot(keep);
    if (lane == 0) wcount[wave] = __popcll(m);
    __syncthreads();
    int wpre = 0, tot = 0;
    for (int w = 0; w < kUpdThreads / 64; ++w) {
      wpre += w < wave ? wcount[w] : 0;
      tot += wcount[w];
    }
    if (keep) ids[n + wpre + __popcll(m & ((1ull << lane) - 1))] = id;
    n += tot;
    __syncthreads();
  }
  // The evicted-range fill above is read by other waves below; with no
  // persistent ids (C_in = 0) the compaction loop, whose barriers would
  // otherwise order it, does not run.
  __syncthreads();
  const int n4 = (n + 3) >> 2;
  for (int i = n + tid; i < 4 * n4; i += kUpdThreads) {
    ids[i] = 0x7FFFFFFF;
    rk[i] = C;
  }
  // scores
  const float* q = qm + (int64_t)bh * d;
  const float* kb = km + (int64_t)bh * NKB * d;
  coarse_scores<kUpdThreads>(q, d, n, 4 * n4, [&](int c) { return kb + (int64_t)ids[c] * d; }, sc);
  __syncthreads();
  const f32x4_t* sc4 = reinterpret_cast<const f32x4_t*>(sc);
  const i32x4_t* ids4 = reinterpret_cast<const i32x4_t*>(ids);
  const i32x4_t* rk4 = reinterpret_cast<const i32x4_t*>(rk);
  if (n > kRankMaxCand) {
    // rk = 0 for a kept candidate, C otherwise
    float thr;
    int need;
    kth_largest<kUpdThreads>(sc, n, C < n ? C : n, hist, rstate, thr, need);
    for (int i = tid; i < n; i += kUpdThreads) {
      const float si = sc[i];
      int r = C;
      if (si > thr) {
        r = 0;
      } else if (si == thr) {
        const int idi = ids[i];
        int t = 0;
#pragma unroll 4
        for (int j4 = 0; j4 < n4; ++j4) {
          const f32x4_t s4 = sc4[j4];
          const i32x4_t d4 = ids4[j4];
#pragma unroll
          for (int e = 0; e < 4; ++e) t += (int)(s4[e] == thr) & (int)(d4[e] < idi);
        }
        r = t < need ? 0 : C;
      }
      rk[i] = r;
    }
  } else {
    for (int i = tid; i < n; i += kUpdThreads) {
      const float si = sc[i];
      const int idi = ids[i];
      int r = 0;
#pragma unroll 4
      for (int j4 = 0; j4 < n4; ++j4) {
        const f32x4_t s4 = sc4[j4];
        const i32x4_t d4 = ids4[j4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r += (int)(s4[e] > si) + ((int)(s4[e] == si) & (int)(d4[e] < idi));
      }
      rk[i] = r;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += kUpdThreads) {
    if (rk[i] >= C) continue;
    const int idi = ids[i];
    int pos = 0;
#pragma unroll 4
    for (int j4 = 0; j4 < n4; ++j4) {
      const i32x4_t r4 = rk4[j4];
      const i32x4_t d4 = ids4[j4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pos += (int)(r4[e] < C) & (int)(d4[e] < idi);
    }
    out[(int64_t)bh * C + pos] = idi;
    if (out_score) out_score[(int64_t)bh * C + pos] = sc[i];
  }
  for (int pos = n + tid; pos < C; pos += kUpdThreads) {
    out[(int64_t)bh * C + pos] = -1;
    if (out_score) out_score[(int64_t)bh * C + pos] = -INFINITY;
  }
}

}  // namespace

hipError_t launch_block_mean(const uint16_t* x, int B, int N, int H, int d, const int64_t* xs,
                             int block, int seg, int bps, int nb, float* out, float* out_total,
                             hipStream_t stream, const uint16_t* x2, const int64_t* xs2,
                             float* out2) {
  if (B * H == 0) return hipSuccess;
  MeanSrcs srcs{};
  srcs.s[0] = MeanSrc{x, xs[0], xs[1], xs[2], out};
  if (x2) srcs.s[1] = MeanSrc{x2, xs2[0], xs2[1], xs2[2], out2};
  if (nb > 0)
    hipLaunchKernelGGL(block_mean_kernel, dim3(nb, B * H, x2 ? 2 : 1), dim3(kMeanThreads), 0,
                       stream, srcs, N, H, d, block, seg, bps, nb);
  if (out_total)
    hipLaunchKernelGGL(total_mean_kernel, dim3(B * H), dim3(kTotThreads), 0, stream, out, N,
                       block, seg, bps, nb, d, out_total);
  return hipGetLastError();
}

hipError_t launch_score_topk(const float* qm, const float* km, int B, int H, int NQB, int NKB,
                             int d, int cand_begin, int cand_count, int K, int32_t* out_idx,
                             float* out_score, hipStream_t stream, int32_t* indptr,
                             int32_t* indices, int prefix_begin, int prefix_count, int id_offset) {
  if (B * H == 0 || NQB == 0) return hipSuccess;
  const TopkLists lists{indptr, indices, prefix_begin, prefix_count, id_offset, B * H * NQB};
  // small candidate sets: 256-thread workgroups, several resident per CU
  const dim3 grid(NQB, B * H);
  if (cand_count <= 256)
    hipLaunchKernelGGL(score_topk_kernel<256>, grid, dim3(256), topk_lds_bytes(cand_count, 256),
                       stream, qm, km, NQB, NKB, d, cand_begin, cand_count, K, out_idx, out_score,
                       lists);
  else
    hipLaunchKernelGGL(score_topk_kernel<1024>, grid, dim3(1024), topk_lds_bytes(cand_count, 1024),
                       stream, qm, km, NQB, NKB, d, cand_begin, cand_count, K, out_idx, out_score,
                       lists);
  return hipGetLastError();
}

hipError_t launch_score_topk_batch(const TopkJobDesc* jobs, int n_jobs, hipStream_t stream) {
  TopkJobs tj{};
  int wgs = 0, n_max = 1;
  for (int i = 0; i < n_jobs; ++i) {
    const TopkJobDesc& a = jobs[i];
    const int rows = a.B * a.H * a.NQB;
    tj.j[i] = TopkJob{a.qm, a.km, a.NQB, a.NKB, a.d, a.cand_begin, a.cand_count, a.K, wgs,
                      a.out_idx, a.out_score,
                      TopkLists{a.indptr, a.indices, a.prefix_begin, a.prefix_count, a.id_offset, rows},
                      a.cm_src, a.cm_N, a.cm_block, a.cm_seg, a.cm_nb};
    wgs += rows;
    n_max = a.cand_count > n_max ? a.cand_count : n_max;
  }
  tj.n_jobs = n_jobs;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(score_topk_batch_kernel, dim3(wgs), dim3(kTopkBatchThreads),
                     topk_lds_bytes(n_max, kTopkBatchThreads), stream, tj);
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

hipError_t launch_persistent_update(const float* qm, const float* km, int B, int H, int NKB,
                                   int d, const int32_t* pers, int C_in, int evict_begin,
                                   int evict_count, int C, int32_t* out, float* out_score,
                                   hipStream_t stream) {
  if (B * H == 0) return hipSuccess;
  hipLaunchKernelGGL(persistent_update_kernel, dim3(B * H), dim3(kUpdThreads), 0, stream, qm, km,
                     NKB, d, pers, C_in, evict_begin, evict_count, C, out, out_score);
  return hipGetLastError();
}

}  // namespace chunkattn
