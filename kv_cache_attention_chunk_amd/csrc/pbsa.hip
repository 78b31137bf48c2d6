// Persistent + block-sparse attention (PBSA) in one pass for gfx950.
//
// The Sparse Forcing page (section 2 item 3) attends densely to a head's
// persistent blocks and sparsely to the top-K blocks of the local window that
// each query block selected.  Here every query block qb of head bh attends to
// the union of two block lists: the head's shared list (the sink frame and
// the persistent blocks, the same for all its query blocks) and the query
// block's own local list (its top-K window blocks).  One workgroup serves
// four query blocks of one head with 8 waves, a pair of waves (64 rows) per
// query block, and keeps their softmax state in registers across both lists:
//   phase 1  the shared list, as 64-key tiles streamed through one LDS ring
//            of four K and four V stages by all 8 waves (each K/V tile goes
//            from L2 to LDS once for the four query blocks);
//   phase 2  each pair's local list, as 32-key tiles (two per block) through
//            a ring of two K and two V stages of its own, in the same LDS,
//            all four pairs stepping together (the loop's
//            barriers are workgroup-wide, so a shorter list is padded with
//            empty tiles up to the longest of the four).
// Both phases run the tile loop of attn_tile.h.  Nothing is written between
// the phases: no float32 branch output, no second pass resuming from it.
#include "attn_tile.h"

namespace chunkattn {

namespace {

using tile::kLn2;

constexpr int kPbsaWaves = 8;
constexpr int kPbsaPairs = kPbsaWaves / 2;   // query blocks per workgroup

template <int D, bool OF32>
__global__ __launch_bounds__(kPbsaWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void pbsa_fwd_kernel(const PbsaParams p) {
  constexpr int NDT = D / 32;
  using G1 = tile::Geom<D, kTileKeys>;   // phase 1: 64-key tiles, all 8 waves
  using G2 = tile::Geom<D, 32>;          // phase 2: 32-key tiles, per pair
  // K stages and V stages as two LDS objects (as in attn_fwd_kernel), so that
  // the reads of each carry the object they come from; each object holds the
  // phase-1 ring's four stages or, in phase 2, every pair's two stages
  constexpr int NS1 = 4;
  constexpr int HALF1 = NS1 * G1::TILEB;
  constexpr int HALF2 = kPbsaPairs * tile::kStages * G2::TILEB;
  constexpr int HALFB = HALF1 > HALF2 ? HALF1 : HALF2;
  __shared__ __attribute__((aligned(1024))) char kst[HALFB];
  __shared__ __attribute__((aligned(1024))) char vst[HALFB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hg = lane >> 5;
  const int pair = wave >> 1;

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= p.n_items) return;
  const int hi = item / p.groups;
  const int grp = item - hi * p.groups;
  const int bh = p.use_list ? (int)p.heads[hi] : hi;
  const int b = bh / p.H;
  const int h = bh - b * p.H;

  // rows of this wave: half (wave & 1) of query block 4 grp + pair
  const int qb = kPbsaPairs * grp + pair;
  int qs = 0, ql = 0;
  if (qb < p.nqb) block_span(qb, p.Nq, p.q_block, p.q_seg, p.q_bps, qs, ql);
  const int row0 = qs + 32 * (wave & 1);
  const int nrows = ql - 32 * (wave & 1);
  const bool qvalid = col < nrows;
  const int qrow = row0 + col;

  tile::Rows<D> rs;
  rs.load_q(p.q + b * p.qs_b + (int64_t)qrow * p.qs_n + h * p.qs_h, qvalid, hg);
  rs.init_offsets(lane);
  rs.clear();

  const uint16_t* kh = p.k + b * p.ks_b + h * p.ks_h;
  const uint16_t* vh = p.v + b * p.ks_b + h * p.ks_h;
  const uint32_t stride_bytes = (uint32_t)(p.ks_n * 2);
  auto span = [&](const int32_t* ptr, int nnz, int row, int& lo, int& n) {
    int a = ptr[row], e = ptr[row + 1];
    a = a < 0 ? 0 : (a > nnz ? nnz : a);
    e = e < a ? a : (e > nnz ? nnz : e);
    lo = a;
    n = e - a;
  };
  // block id -> (element offset, valid rows); ids outside the tiling give an
  // empty tile
  auto block_tile = [&](int id, int64_t& off, int& len) {
    int s0 = 0, l0 = 0;
    if (id >= 0 && id < p.nkb)
      block_span(id, p.Nkv, p.kv_block, p.kv_seg, p.kv_bps, s0, l0, p.kv_bps_magic);
    off = (int64_t)s0 * p.ks_n;
    len = l0;
  };

  // ---- phase 1: the head's shared list, 64-key tiles, all 8 waves --------
  {
    int lo1, n1;
    span(p.sh_ptr, p.sh_nnz, bh, lo1, n1);
    // entry t + 1's id is fetched one tile ahead (scalar loads)
    int id_next = n1 > 0 ? tile::ld_uniform(p.sh_idx, lo1) : 0;
    auto src1 = [&](int t, int64_t& off, int& len) {
      const int id = id_next;
      if (t + 1 < n1) id_next = tile::ld_uniform(p.sh_idx, lo1 + t + 1);
      block_tile(id, off, len);
    };
    tile::Loader<D, kTileKeys, kPbsaWaves> ldr1;
    ldr1.init(lane, wave, stride_bytes);
    tile::run<D, kTileKeys, kPbsaWaves, NS1>(rs, ldr1, kst, vst, kh, vh, stride_bytes, n1,
                                        p.scale_log2, hg, src1, [](int) {});
  }

  // ---- phase 2: each pair's local list, 32-key tiles, per-pair rings -----
  {
    // the four lists' lengths (every wave reads all four: the step count is
    // the longest, so that all waves meet the same barriers)
    int nmax = 0, lo2 = 0, n2 = 0;
#pragma unroll
    for (int pp = 0; pp < kPbsaPairs; ++pp) {
      const int qbp = kPbsaPairs * grp + pp;
      int a = 0, n = 0;
      if (qbp < p.nqb) span(p.lo_ptr, p.lo_nnz, bh * p.nqb + qbp, a, n);
      nmax = n > nmax ? n : nmax;
      if (pp == pair) {
        lo2 = a;
        n2 = n;
      }
    }
    int id_next = n2 > 0 ? tile::ld_uniform(p.lo_idx, lo2) : 0;
    int id_hold = 0;
    auto src2 = [&](int t, int64_t& off, int& len) {
      const int e = t >> 1, half = t & 1;
      if (half == 0) {
        id_hold = e < n2 ? id_next : -1;
        if (e + 1 < n2) id_next = tile::ld_uniform(p.lo_idx, lo2 + e + 1);
      }
      block_tile(id_hold, off, len);
      off += (int64_t)(32 * half) * p.ks_n;
      len -= 32 * half;
      len = len < 0 ? 0 : (len > 32 ? 32 : len);
    };
    tile::Loader<D, 32, 2> ldr2;
    ldr2.init(lane, wave & 1, stride_bytes);
    const int pr = pair * tile::kStages * G2::TILEB;
    tile::run<D, 32, 2>(rs, ldr2, kst + pr, vst + pr, kh, vh, stride_bytes, 2 * nmax,
                        p.scale_log2, hg, src2, [](int) {});
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 (m + log2 l) ----------------------
  const float lt = tile::half_sum(rs.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!qvalid) return;
  const int64_t obase = b * p.os_b + (int64_t)qrow * p.os_n + h * p.os_h;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d0 = 32 * dt + 8 * r + 4 * hg;
      f32x4_t v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = rs.acc[dt][4 * r + e] * inv;
      if (OF32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.o) + obase + d0) = v4;
      } else {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
        *reinterpret_cast<bf16x4_t*>(reinterpret_cast<uint16_t*>(p.o) + obase + d0) =
            __builtin_convertvector(v4, bf16x4_t);
      }
    }
  }
  if (hg == 0) p.lse[(int64_t)bh * p.Nq + qrow] = lt > 0.f ? (rs.m + log2f(lt)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(bool of32, const PbsaParams& p, hipStream_t stream) {
  const dim3 grid(p.n_items), block(kPbsaWaves * 64);
  if (of32)
    hipLaunchKernelGGL((pbsa_fwd_kernel<D, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((pbsa_fwd_kernel<D, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pbsa(int d, bool out_f32, const PbsaParams& p, hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  return d == 64 ? launch_d<64>(out_f32, p, stream) : launch_d<128>(out_f32, p, stream);
}

}  // namespace chunkattn
