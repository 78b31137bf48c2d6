// Fused chunk-attention forward for gfx950 (MI355X).
//
// One workgroup owns NW*32 query rows of one (b, h) and streams that head's
// key set in 64-token tiles (32-token tiles for 2-wave workgroups) through
// the tile loop of attn_tile.h: buffer->LDS loads into a swizzled ring of
// K and V stages, S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16,
// online softmax in the log2 domain, software-pipelined so that the softmax of
// tile t overlaps the QK MFMAs of tile t+1.  Epilogue: O = acc / l, LSE =
// ln2 * (m + log2 l); an empty key set gives O = 0, LSE = -inf.
// The three cache modes differ only in where tile t's keys come from: the
// dense cache, the t-th block of a CSR row (the PBSA block lists of the
// Sparse Forcing page, section 2 item 3) or the t-th 64-row slice of a
// head's span of a flat ragged buffer (Pyramid Forcing page, section 3).
#include "attn_tile.h"

#include <type_traits>

namespace chunkattn {

namespace {

using tile::kLn2;

// LDS ring of K and V tile stages.  An 8-wave workgroup (256 query rows)
// holds a CU's 8 waves, so each K/V tile goes from L2 to LDS once per CU for
// 256 rows; it keeps four K and four V stages (128 KB at d = 128) and meets
// the workgroup barrier every second tile.  Smaller workgroups share a CU and
// keep two of each.  The stage of every read is a compile-time constant in
// the loop unrolled by the stage count.
//
// 2-wave workgroups (64-row query blocks, the per-query-block lists) stream
// 32-key tiles instead: each list entry (a block of up to 64 tokens) becomes
// two tiles, and the 32 KB ring lets four such workgroups, i.e. two waves
// per SIMD, share a CU (a 64 KB ring held them to one wave per SIMD).
template <int NW>
constexpr int tile_keys() { return NW == 2 ? 32 : kTileKeys; }

// Two waves per SIMD: caps VGPR + AGPR at 256 per lane, so a CU holds at most
// 8 waves: one 8-wave workgroup; smaller workgroups are held to two per CU by
// their 64 KB of LDS (d = 128).
template <int D, int NW, int MODE, bool OF32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const AttnParams p) {
  constexpr int BM = NW * 32;
  constexpr int NDT = D / 32;     // 32-row d tiles of O^T
  constexpr int TK = tile_keys<NW>();   // keys per tile
  using G = tile::Geom<D, TK>;
  constexpr int TPE = kTileKeys / TK;   // tiles per list entry (block mode)
  static_assert(MODE == MODE_BLOCKS || TK == kTileKeys, "range mode streams 64-key tiles");
  // Ring stages: four for the 8-wave workgroups (one per CU), whose loop then
  // meets the workgroup barrier every second tile; two for the smaller ones,
  // which share a CU.  K and V stages are two LDS objects, so that the reads
  // of each carry the object they come from.
  constexpr int NS = NW == 8 ? 4 : 2;
  __shared__ __attribute__((aligned(1024))) char kst[NS * G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vst[NS * G::TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;      // query column (B/C operands) or A-operand row
  const int hg = lane >> 5;       // lane half: selects k sub-range / row quad

  // ---- work decomposition ----------------------------------------------------
  // Each pass of the loop below runs one segment: query rows [row0, row0 +
  // nrows) of launch-local head `sel` against key tiles [kt0, kt1) of its key
  // set (range mode; kt1 < 0 = every tile) or its CSR row (block mode).
  // slot < 0 writes the final O and LSE; slot >= 0 the float32 partial state
  // into workspace slot `slot`.  Block mode and the plain grid run one
  // segment per workgroup; the balanced schedule runs the workgroup's unit
  // range as consecutive segments.
  //
  // Segment order under the balanced schedule: every segment of a range
  // starts at key tile 0 except possibly the first, which continues a query
  // tile begun by the previous workgroup.  That one runs last, so that each
  // workgroup walks its head's keys in ascending order: the workgroups
  // sharing a head then read the same few key tiles at any moment (shared
  // through L2) instead of tiles spread over the whole cache.
  int u_cur = 0, u_end = 0, u_first = 0, first_end = 0, head_i = 0, head_first = 0, g_self = 0;
  int deferred = 0;     // 1: the first segment is still to run, at the end
  if (MODE == MODE_RANGE && p.sched) {
    g_self = xcd_remap(blockIdx.x, gridDim.x);
    u_first = sched_real(p, unit_begin(g_self, p.n_vunits, p.n_wgs));
    u_end = sched_real(p, unit_begin(g_self + 1, p.n_vunits, p.n_wgs));
    // head holding u_first (binary search over the prefix)
    int lo = 0, hi = p.n_heads - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.n_qtiles * p.tprefix[mid + 1] <= u_first) lo = mid + 1; else hi = mid;
    }
    const int nt = p.tprefix[lo + 1] - p.tprefix[lo];
    const int rel = u_first - p.n_qtiles * p.tprefix[lo];
    const int k0 = rel % nt;
    first_end = u_first + (nt - k0 < u_end - u_first ? nt - k0 : u_end - u_first);
    // a first segment that starts mid-tile and is not the whole range runs last
    deferred = k0 != 0 && first_end < u_end;
    u_cur = deferred ? first_end : u_first;
    head_i = head_first = lo;
  }
  for (;;) {
  int sel, row0, nrows, csr_row = 0, kt0 = 0, kt1 = -1, slot = -1;
  if (MODE == MODE_BLOCKS) {
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= p.n_items) return;
    const int per_head = p.nqb * p.q_sub;
    sel = item / per_head;
    const int rem = item - sel * per_head;
    const int qb = rem / p.q_sub;
    const int st = rem - qb * p.q_sub;
    int qs, ql;
    block_span(qb, p.Nq, p.q_block, p.q_seg, p.q_bps, qs, ql);
    row0 = qs + st * BM;
    nrows = ql - st * BM;
    if (nrows <= 0) return;
    if (nrows > BM) nrows = BM;
    const int bh_ = (p.use_list ? p.heads[sel] : sel) & 0x7FFF;
    csr_row = bh_ * p.nqb + qb;
  } else if (!p.sched) {
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= p.n_items) return;
    sel = item / p.n_qtiles;
    const int qt = item - sel * p.n_qtiles;
    row0 = qt * BM;
    nrows = p.Nq - row0;
    if (nrows > BM) nrows = BM;
  } else {
    if (u_cur >= u_end) {
      if (!deferred) return;
      deferred = 0;
      u_cur = u_first;
      u_end = first_end;
      head_i = head_first;
    }
    while (p.n_qtiles * p.tprefix[head_i + 1] <= u_cur) ++head_i;
    sel = head_i;
    const int nt = p.tprefix[head_i + 1] - p.tprefix[head_i];
    const int rel = u_cur - p.n_qtiles * p.tprefix[head_i];
    const int qt = rel / nt;
    kt0 = rel - qt * nt;
    kt1 = nt - kt0 < u_end - u_cur ? nt : kt0 + (u_end - u_cur);
    u_cur += kt1 - kt0;
    if (kt0 != 0 || kt1 != nt) slot = u_cur - (kt1 - kt0) == u_first ? 2 * g_self : 2 * g_self + 1;
    row0 = qt * BM;
    nrows = p.Nq - row0;
    if (nrows > BM) nrows = BM;
  }
  const int hword = p.use_list ? p.heads[sel] : sel;
  const int bh = hword & 0x7FFF;
  const bool flat = p.use_list ? (hword & kFlatHead) != 0 : p.all_flat != 0;
  const int b = bh / p.H;
  const int h = bh - b * p.H;

  // ---- key set -------------------------------------------------------------
  int ntiles;
  int kv_lo = 0, kv_len = 0, list0 = 0;
  int64_t kstride;
  const uint16_t* kh;
  const uint16_t* vh;
  if (MODE == MODE_RANGE) {
    if (flat) {
      int lo = p.cu[bh], hi = p.cu[bh + 1];
      lo = lo < 0 ? 0 : (lo > p.total_kv ? p.total_kv : lo);
      hi = hi < lo ? lo : (hi > p.total_kv ? p.total_kv : hi);
      kv_lo = lo;
      kv_len = hi - lo;
      kh = p.kf;
      vh = p.vf;
      kstride = p.kfs_n;
    } else {
      kv_len = p.Nkv;
      kh = p.k + b * p.ks_b + h * p.ks_h;
      vh = p.v + b * p.ks_b + h * p.ks_h;
      kstride = p.ks_n;
    }
    if (kt1 < 0) kt1 = (kv_len + kTileKeys - 1) / kTileKeys;
    ntiles = kt1 - kt0;
  } else {
    int lo = p.indptr[csr_row], hi = p.indptr[csr_row + 1];
    lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
    hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
    list0 = lo;
    ntiles = (hi - lo) * TPE;
    kh = p.k + b * p.ks_b + h * p.ks_h;
    vh = p.v + b * p.ks_b + h * p.ks_h;
    kstride = p.ks_n;
  }

  // tile t -> (element offset of its row 0, number of valid rows).  Called
  // for t = 0, 1, 2, ... in order; in block mode each call also fetches the
  // next list entry's block id, so that its latency overlaps one iteration
  // (with 32-key tiles, entry t / 2 gives tile t its half t % 2; the second
  // half of a short block has no valid rows).  In range mode tile t covers
  // keys [(kt0 + t) 64, +64) of the key set; a tile past its end (possible
  // only when the schedule's tile count exceeds the device-side span) has no
  // valid rows.
  int id_next = (MODE == MODE_BLOCKS && ntiles > 0) ? tile::ld_uniform(p.indices, list0) : 0;
  int id_hold = 0;
  auto tile_src = [&](int t, int64_t& off, int& len) {
    if (MODE == MODE_BLOCKS) {
      const int half = TPE == 2 ? (t & 1) : 0;
      const int e = TPE == 2 ? (t >> 1) : t;
      if (half == 0) {
        id_hold = id_next;
        if (e + 1 < ntiles / TPE) id_next = tile::ld_uniform(p.indices, list0 + e + 1);
      }
      const int id = id_hold;
      int s0 = 0, l0 = 0;
      if (id >= 0 && id < p.nkb)
        block_span(id, p.Nkv, p.kv_block, p.kv_seg, p.kv_bps, s0, l0, p.kv_bps_magic);
      if (TPE == 2) {
        s0 += TK * half;
        l0 -= TK * half;
        l0 = l0 < 0 ? 0 : (l0 > TK ? TK : l0);
      }
      off = (int64_t)s0 * kstride;
      len = l0;
    } else {
      int s0 = (kt0 + t) * kTileKeys;
      s0 = s0 < kv_len ? s0 : kv_len;
      const int rest = kv_len - s0;
      off = (int64_t)(kv_lo + s0) * kstride;
      len = rest < kTileKeys ? rest : kTileKeys;
    }
  };

  const uint32_t stride_bytes = (uint32_t)(kstride * 2);
  tile::Loader<D, TK, NW> ldr;
  ldr.init(lane, wave, stride_bytes);

  // ---- Q^T operands in registers (query row row0 + 32 wave + col) ----------
  const int qr = wave * 32 + col;
  const bool qvalid = qr < nrows;
  const int qrow = row0 + qr;
  tile::Rows<D> rs;
  rs.load_q(p.q + b * p.qs_b + (int64_t)qrow * p.qs_n + h * p.qs_h, qvalid, hg);
  rs.init_offsets(lane);
  rs.clear();
  if (p.o_init && qvalid) {
    // Resume from a previous branch (O1, LSE1): the state (m, l, acc) =
    // (LSE1 * log2 e, 1, O1) has acc / l = O1 and m + log2 l = LSE1 / ln 2,
    // i.e. it is that branch's softmax state up to a common scale.
    rs.m = p.lse_init[(int64_t)bh * p.Nq + qrow] * 1.4426950408889634f;
    rs.l = hg == 0 ? 1.f : 0.f;
    const float* oi = p.o_init + b * p.is_b + (int64_t)qrow * p.is_n + h * p.is_h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(oi + 32 * dt + 8 * r + 4 * hg);
#pragma unroll
        for (int e = 0; e < 4; ++e) rs.acc[dt][4 * r + e] = x[e];
      }
  }

  // Writes the softmax state of the tiles processed so far: O = acc / l and
  // LSE = ln 2 (m + log2 l) (empty key set: O = 0, LSE = -inf), to the
  // snapshot outputs (to_snap), else to the float32 partial slot of a split
  // query tile or to the final outputs.
  auto emit_state = [&](bool to_snap) {
    const float lt = tile::half_sum(rs.l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_row = lt > 0.f ? (rs.m + log2f(lt)) * kLn2 : -INFINITY;
    if (!qvalid) return;
    if (!to_snap && slot >= 0) {
      // partial state of a split query tile: O / l and LSE, float32
      float* part = p.ws + (int64_t)slot * BM * (D + 1);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = 32 * dt + 8 * r + 4 * hg;
          f32x4_t v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = rs.acc[dt][4 * r + e] * inv;
          *reinterpret_cast<f32x4_t*>(part + qr * D + d0) = v4;
        }
      }
      if (hg == 0) part[BM * D + qr] = lse_row;
      return;
    }
    void* const obuf = to_snap ? p.o_snap : p.o;
    float* const lbuf = to_snap ? p.lse_snap : p.lse;
    const int64_t obase = to_snap ? b * p.ss_b + (int64_t)qrow * p.ss_n + h * p.ss_h
                                  : b * p.os_b + (int64_t)qrow * p.os_n + h * p.os_h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * dt + 8 * r + 4 * hg;
        f32x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = rs.acc[dt][4 * r + e] * inv;
        if (OF32) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(obuf) + obase + d0) = v4;
        } else {
          typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
          const bf16x4_t bv = __builtin_convertvector(v4, bf16x4_t);
          *reinterpret_cast<bf16x4_t*>(reinterpret_cast<uint16_t*>(obuf) + obase + d0) = bv;
        }
      }
    }
    if (hg == 0) lbuf[(int64_t)bh * p.Nq + qrow] = lse_row;
  };
  // Dual output (block mode): after the first `snap` tiles of the list the
  // state is also written to the snapshot outputs.
  const int snap = (MODE == MODE_BLOCKS && p.snap >= 0)
                       ? (p.snap * TPE < ntiles ? p.snap * TPE : ntiles) : -1;
  if (MODE == MODE_BLOCKS && snap == 0) emit_state(true);
  tile::run<D, TK, NW, NS>(rs, ldr, kst, vst, kh, vh, stride_bytes, ntiles, p.scale_log2, hg,
                       tile_src, [&](int t) {
                         if (MODE == MODE_BLOCKS && t == snap - 1) emit_state(true);
                       });

  // ---- epilogue --------------------------------------------------------------
  emit_state(false);
  if (MODE == MODE_BLOCKS || !p.sched) return;
  }   // segment loop
}

// Final O and LSE of the query tiles that the balanced schedule split across
// workgroups: the LSE merge of their partial states (the decomposition of
// the ISPA page, section 2 item 1, over consecutive key ranges):
// M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum_s w_s O_s / sum_s w_s,
// LSE = M + ln sum_s w_s; every part empty -> O = 0, LSE = -inf.
// One workgroup per (query tile, group of 1024/D rows), one thread per
// 4-float chunk of a row; tiles written whole by one workgroup exit at once.
// The parts' LSE values and O chunks are all loaded before they are used
// (up to kMergeFast parts; more parts take a second, looped pass).
constexpr int kMergeFast = 4;

template <int D, bool OF32>
__global__ __launch_bounds__(256) void split_merge_kernel(const AttnParams p) {
  constexpr int BM = kRangeRows;
  constexpr int C4 = D / 4;                  // float4 chunks per row
  constexpr int RPW = 256 / C4;              // rows per workgroup
  constexpr int GPT = BM / RPW;              // row groups per query tile
  const int item = blockIdx.x / GPT;         // launch-local head * n_qtiles + query tile
  const int rg = blockIdx.x - item * GPT;
  const int sel = item / p.n_qtiles;
  const int qt = item - sel * p.n_qtiles;
  const int nt = p.tprefix[sel + 1] - p.tprefix[sel];
  const int u0 = p.n_qtiles * p.tprefix[sel] + qt * nt;
  const int g0 = g_of_unit(sched_virtual(p, u0), p.n_vunits, p.n_wgs);
  const int g1 = g_of_unit(sched_virtual(p, u0 + nt - 1), p.n_vunits, p.n_wgs);
  if (g0 == g1) return;
  const int row0 = qt * BM;
  const int r = rg * RPW + (int)threadIdx.x / C4;
  const int c = (int)threadIdx.x % C4;
  if (row0 + r >= p.Nq) return;
  const int hword = p.use_list ? p.heads[sel] : sel;
  const int bh = hword & 0x7FFF;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  // the tile is the last segment of g0 when g0's range starts before it,
  // else g0's first; it is the first segment of every later workgroup
  const int slot0 = sched_real(p, unit_begin(g0, p.n_vunits, p.n_wgs)) < u0 ? 2 * g0 + 1 : 2 * g0;
  const int np = g1 - g0 + 1;
  auto part = [&](int j) {
    return p.ws + (int64_t)(j == 0 ? slot0 : 2 * (g0 + j)) * BM * (D + 1);
  };
  float ls[kMergeFast];
  f32x4_t xs[kMergeFast];
#pragma unroll
  for (int j = 0; j < kMergeFast; ++j) {
    if (j < np) {
      const float* pp = part(j);
      ls[j] = pp[BM * D + r];
      xs[j] = *reinterpret_cast<const f32x4_t*>(pp + r * D + 4 * c);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMergeFast; ++j)
    if (j < np) M = fmaxf(M, ls[j]);
  for (int j = kMergeFast; j < np; ++j) M = fmaxf(M, part(j)[BM * D + r]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kMergeFast; ++j) {
      if (j < np) {
        const float w = expf(ls[j] - M);
        wsum += w;
        acc += w * xs[j];
      }
    }
    for (int j = kMergeFast; j < np; ++j) {
      const float* pp = part(j);
      const float w = expf(pp[BM * D + r] - M);
      wsum += w;
      acc += w * *reinterpret_cast<const f32x4_t*>(pp + r * D + 4 * c);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  acc *= inv;
  const int64_t obase = b * p.os_b + (int64_t)(row0 + r) * p.os_n + h * p.os_h + 4 * c;
  if (OF32) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.o) + obase) = acc;
  } else {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
    *reinterpret_cast<bf16x4_t*>(reinterpret_cast<uint16_t*>(p.o) + obase) =
        __builtin_convertvector(acc, bf16x4_t);
  }
  if (c == 0) p.lse[(int64_t)bh * p.Nq + row0 + r] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

template <int D, int NW, int MODE>
hipError_t launch_t(bool of32, const AttnParams& p, hipStream_t stream) {
  const dim3 grid(MODE == MODE_RANGE && p.sched ? p.n_wgs : p.n_items), block(NW * 64);
  if (of32)
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, MODE, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, MODE, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int mode, int nwaves, bool of32, const AttnParams& p, hipStream_t stream) {
  if (mode == MODE_RANGE) return launch_t<D, 8, MODE_RANGE>(of32, p, stream);
  return nwaves == 2 ? launch_t<D, 2, MODE_BLOCKS>(of32, p, stream)
       : nwaves == 4 ? launch_t<D, 4, MODE_BLOCKS>(of32, p, stream)
                     : launch_t<D, 8, MODE_BLOCKS>(of32, p, stream);
}

template <int D>
int slots_d() {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per, reinterpret_cast<const void*>(&attn_fwd_kernel<D, 8, MODE_RANGE, false>),
          8 * 64, 0) != hipSuccess)
    return 0;
  return cus * per;
}

}  // namespace

hipError_t launch_attention(int mode, int d, int nwaves, bool out_f32, const AttnParams& p,
                            hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  return d == 64 ? launch_d<64>(mode, nwaves, out_f32, p, stream)
                 : launch_d<128>(mode, nwaves, out_f32, p, stream);
}

hipError_t launch_split_merge(int d, bool out_f32, const AttnParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_heads * p.n_qtiles;
  if (items <= 0) return hipSuccess;
  const dim3 grid((unsigned)(items * (kRangeRows / (1024 / d)))), block(256);
  if (d == 64) {
    if (out_f32) hipLaunchKernelGGL((split_merge_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_merge_kernel<64, false>), grid, block, 0, stream, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((split_merge_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_merge_kernel<128, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

int attention_slots(int d) {
  // per device and head dim, computed once
  static int cache[2][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int di = d == 64 ? 0 : 1;
  int v = __atomic_load_n(&cache[di][dev], __ATOMIC_RELAXED);
  if (v == 0) {
    v = d == 64 ? slots_d<64>() : slots_d<128>();
    __atomic_store_n(&cache[di][dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

}  // namespace chunkattn
