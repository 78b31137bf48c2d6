// Fused chunk-attention forward for gfx950 (MI355X).
//
// One workgroup owns NW*32 query rows of one (b, h) and streams that head's
// key set in 64-token tiles:
//   * K and V tiles go straight from global memory to LDS with buffer loads
//     (buffer_load_dwordx4 ... lds, 1 KB per wave instruction): no staging
//     registers, and the buffer range check returns zeros for rows past a
//     partial tile.  K and V are double-buffered: K(t+2) and V(t+1) are
//     loaded during iteration t.
//   * LDS rows are unpadded and XOR-swizzled by 16-byte chunk so that every
//     read pattern below is free of bank conflicts: K chunk c of row r sits at
//     c ^ (r & 15) (d = 128) or c ^ ((r >> 1) & 7) (d = 64); V chunk c at
//     c ^ 4(r & 3) (d = 128) or c ^ 4((r >> 1) & 1) (d = 64).
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K tile rows (keys), B =
//     Q^T held in registers for the whole loop (lane = query column).  The
//     accumulator layout puts one query per lane column, so the row max and
//     row sum over keys are in-lane except for one exchange with lane^32.
//   * software pipeline: iteration t issues the QK MFMAs of tile t+1 before
//     the softmax of tile t, so the softmax VALU work overlaps matrix work of
//     the same wave (two score register sets alternate).
//   * online softmax in the log2 domain (scale*log2e folded into one FMA),
//     P rounded to bf16, then O^T += V^T P^T with the same MFMA: B = P^T
//     straight from the S^T accumulator registers (no shuffle), A = V^T read
//     with gfx950's transposing LDS load (ds_read_b64_tr_b16): within each
//     16-lane group, lane i receives element i%4 of the 8-byte chunks
//     addressed by lanes i/4 + 4e (e = 0..3), so pointing the source lanes at
//     4 key rows x 4 column quads yields 4 consecutive keys of one d per lane.
//   * epilogue: O = acc / l, LSE = ln2 * (m + log2 l); an empty key set gives
//     O = 0, LSE = -inf.
// The three cache modes differ only in where tile t's keys come from: the
// dense cache, the t-th block of a CSR row (the PBSA block lists of the
// Sparse Forcing page, section 2 item 3) or the t-th 64-row slice of a
// head's span of a flat ragged buffer (Pyramid Forcing page, section 3).
#include "common.h"

#include <type_traits>

namespace chunkattn {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBufferWord3 = 0x00020000;   // raw buffer resource, gfx9 family

// LDS ring of K and V tile stages: K x2 and V x2 (64 KB at d = 128).  An
// 8-wave workgroup (256 query rows) holds a CU's 8 waves, so each K/V tile
// goes from L2 to LDS once per CU for 256 rows.  With two stages each, the stage of every
// read is a compile-time constant in the two-iteration unrolled loop.
//
// 2-wave workgroups (64-row query blocks, the per-query-block lists) stream
// 32-key tiles instead: each list entry (a block of up to 64 tokens) becomes
// two tiles, and the 32 KB ring lets four such workgroups, i.e. two waves
// per SIMD, share a CU (a 64 KB ring held them to one wave per SIMD).
template <int D, int NW>
struct Layout {
  static constexpr int TK = NW == 2 ? 32 : kTileKeys;  // keys per tile
  static constexpr int ROWB = 2 * D;                    // bytes per K / V row
  static constexpr int TILEB = TK * ROWB;               // bytes per K or V tile
  static constexpr int KSTAGES = 2;
  static constexpr int VSTAGES = 2;
  static constexpr int LDSB = (KSTAGES + VSTAGES) * TILEB;
  // physical 16-byte chunk of logical chunk c in row r
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// max / sum of x over lanes l and l ^ 32 (the two halves of one query
// column), exchanged with v_permlane32_swap instead of an LDS permute.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

// Destination of a buffer->LDS load as a bare wave-uniform LDS address.  The
// kernel orders these loads against its LDS reads itself (s_waitcnt vmcnt +
// barrier at the end of each iteration).  A destination the compiler cannot
// tie to an LDS object keeps it from also placing a vmcnt(0) wait, i.e. a
// wait for every load in flight, in front of the transposing LDS reads.
__device__ __forceinline__ lds_void_t* dma_dst(char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_char_t*)p;
  return (lds_void_t*)(uintptr_t)__builtin_amdgcn_readfirstlane(a);
}

// Workgroup barrier for the load pipeline.  The caller has already waited
// (s_waitcnt) for its own buffer->LDS loads and LDS reads; the empty asm
// statements keep the compiler from moving memory accesses across the
// barrier.  (__syncthreads' release fence would add a vmcnt(0) wait here,
// draining the loads meant to stay in flight.)
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Read-only kernel input read through the scalar cache (s_load): the block
// lists do not change while a launch runs.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int i) {
  return ((const_i32_t*)p)[i];
}

// Transposing LDS read of 4 bf16 (see the header comment for the lane layout).
__device__ __forceinline__ s16x4_t ld_tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<char*>(p)));
}

// Per-lane byte offsets of the buffer->LDS loads of one 64 x D tile: wave w's
// instruction j fills LDS bytes [(NI w + j) KB, +1 KB), lane i the 16 bytes at
// +16 i, i.e. physical row r and chunk pc; it loads logical chunk
// pc ^ swizzle(r) of row r.
template <int D, int NW>
struct TileLoader {
  using L = Layout<D, NW>;
  static constexpr int NI = L::TILEB / (1024 * NW);
  uint32_t koff[NI], voff[NI];
  int wave;

  __device__ __forceinline__ void init(int lane, int wave_, uint32_t stride_bytes) {
    wave = wave_;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int pbyte = (NI * wave + j) * 1024 + 16 * lane;
      const int r = pbyte / L::ROWB;
      const int pc = (pbyte % L::ROWB) / 16;
      koff[j] = r * stride_bytes + 16 * (pc ^ L::swz_k(r));
      voff[j] = r * stride_bytes + 16 * (pc ^ L::swz_v(r));
    }
  }

  // Loads rows [0, len) of the tile whose row 0 is at kb (vb); rows past len
  // (and all rows when len == 0) are written as zeros by the range check.
  __device__ __forceinline__ void issue_k(const uint16_t* kb, int len, uint32_t stride_bytes,
                                          char* lk) const {
    const int nrec = len * (int)stride_bytes;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), (short)0, nrec, kBufferWord3);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dma_dst(lk + (NI * wave + j) * 1024), 16,
                                               (int)koff[j], 0, 0, 0);
  }

  __device__ __forceinline__ void issue_v(const uint16_t* vb, int len, uint32_t stride_bytes,
                                          char* lv) const {
    const int nrec = len * (int)stride_bytes;
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), (short)0, nrec, kBufferWord3);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dma_dst(lv + (NI * wave + j) * 1024), 16,
                                               (int)voff[j], 0, 0, 0);
  }
};

// Two waves per SIMD: caps VGPR + AGPR at 256 per lane, so a CU holds at most
// 8 waves: one 8-wave workgroup; smaller workgroups are held to two per CU by
// their 64 KB of LDS (d = 128).
template <int D, int NW, int MODE, bool OF32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const AttnParams p) {
  using L = Layout<D, NW>;
  constexpr int BM = NW * 32;
  constexpr int NST = D / 16;     // MFMA k-steps over d for S
  constexpr int NDT = D / 32;     // 32-row d tiles of O^T
  constexpr int TK = L::TK;       // keys per tile
  constexpr int KT = TK / 32;     // 32-key halves of a tile (S accumulators)
  constexpr int NG = 2 * KT;      // 16-key P groups of a tile
  constexpr int TPE = kTileKeys / TK;   // tiles per list entry (block mode)
  static_assert(MODE == MODE_BLOCKS || TK == kTileKeys, "range mode streams 64-key tiles");
  // K and V stages as two LDS objects, so that the reads of each carry the
  // object they come from.
  __shared__ __attribute__((aligned(1024))) char kst[L::KSTAGES * L::TILEB];
  __shared__ __attribute__((aligned(1024))) char vst[L::VSTAGES * L::TILEB];

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
    u_first = unit_begin(g_self, p.n_units, p.n_wgs);
    u_end = unit_begin(g_self + 1, p.n_units, p.n_wgs);
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
  int id_next = (MODE == MODE_BLOCKS && ntiles > 0) ? ld_uniform(p.indices, list0) : 0;
  int id_hold = 0;
  auto tile_src = [&](int t, int64_t& off, int& len) {
    if (MODE == MODE_BLOCKS) {
      const int half = TPE == 2 ? (t & 1) : 0;
      const int e = TPE == 2 ? (t >> 1) : t;
      if (half == 0) {
        id_hold = id_next;
        if (e + 1 < ntiles / TPE) id_next = ld_uniform(p.indices, list0 + e + 1);
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
  TileLoader<D, NW> ldr;
  ldr.init(lane, wave, stride_bytes);

  // ---- Q^T operands in registers (query row row0 + 32 wave + col) ----------
  const int qr = wave * 32 + col;
  const bool qvalid = qr < nrows;
  const int qrow = row0 + qr;
  bf16x8_t qreg[NST];
  {
    const uint16_t* qp = p.q + b * p.qs_b + (int64_t)qrow * p.qs_n + h * p.qs_h + 8 * hg;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const u32x4_t x = qvalid ? ld16(qp + 16 * s) : u32x4_t{0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // Per-lane LDS read addresses.  Row base, stage offset and the swizzled
  // chunk occupy disjoint address bits, so each read is (base | swizzle) ^
  // (step * chunk), one v_xor per read.
  //   K rows 32kt + col, chunk 2st + hg: byte 16((2st + hg) ^ kz)
  //     = 32(st ^ (kz >> 1)) + 16(hg ^ (kz & 1)).
  const int kz = L::swz_k(col);
  const int kbx = col * L::ROWB + 16 * (hg ^ (kz & 1)) + 32 * (kz >> 1);
  int kx[NST];                    // per-k-step K read offsets within a stage
#pragma unroll
  for (int st = 0; st < NST; ++st) kx[st] = kbx ^ (32 * st);
  //   V source row 4hg + (lane & 15)/4 (+ 32kt + 16u + 8 half), chunk
  //   4dt + vcol16: byte 16((4dt + vcol16) ^ vz) = 64(dt ^ vz/4) + 16 vcol16.
  const int vz = D == 128 ? ((lane & 15) >> 2) : ((lane >> 3) & 1);
  const int vcol16 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vbx = (4 * hg + ((lane & 15) >> 2)) * L::ROWB + 8 * (lane & 1) + 16 * vcol16 + 64 * vz;
  int vx[NDT];                    // per-d-tile V read offsets within a stage
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) vx[dt] = vbx ^ (64 * dt);

  f32x16_t acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16_t{};
  float m = -INFINITY;   // running max of this lane's query row (log2 domain)
  float l = 0.f;         // this lane's partial row sum (lane halves added at the end)
  if (p.o_init && qvalid) {
    // Resume from a previous branch (O1, LSE1): the state (m, l, acc) =
    // (LSE1 * log2 e, 1, O1) has acc / l = O1 and m + log2 l = LSE1 / ln 2,
    // i.e. it is that branch's softmax state up to a common scale.
    m = p.lse_init[(int64_t)bh * p.Nq + qrow] * 1.4426950408889634f;
    l = hg == 0 ? 1.f : 0.f;
    const float* oi = p.o_init + b * p.is_b + (int64_t)qrow * p.is_n + h * p.is_h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(oi + 32 * dt + 8 * r + 4 * hg);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dt][4 * r + e] = x[e];
      }
  }

  // S^T = K Q^T for the two 32-key halves of the tile in K stage ks.
  auto qk = [&](int ks, f32x16_t (&sc)[2]) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sc[kt] = f32x16_t{};
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            kst + ks * L::TILEB + kx[st] + kt * 32 * L::ROWB);
        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[st], sc[kt], 0, 0, 0);
      }
    }
  };

  // Row max of one tile and the accumulator rescale when a row's max grew.
  // The raw (unscaled) per-lane max of a full tile arrives precomputed in
  // `rawmax`; a partial tile first masks keys past len_cur and takes its max
  // here.  Key of sc[kt][i] = 32kt + 8(i/4) + 4hg + i%4.
  auto prep = [&](f32x16_t (&sc)[2], int len_cur, float rawmax) {
    float mx = rawmax;
    if (len_cur < TK) {
      mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kt + 8 * (i >> 2) + 4 * hg + (i & 3);
          if (key >= len_cur) sc[kt][i] = -INFINITY;
          mx = fmaxf(mx, sc[kt][i]);
        }
    }
    mx = half_max(mx) * p.scale_log2;
    // The exponent base m is the exact running row max, so the largest
    // weight of a row is exactly 1 and survives the bf16 rounding of P
    // unchanged.  The O accumulator is rescaled only when some row of the
    // wave found a new max in this tile.
    const bool grow = mx > m;
    if (__any(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - (m_new == -INFINITY ? 0.f : m_new));
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) acc[i] *= alpha;
    }
  };

  // Segments of the fused iteration body.  Group g (0..3) is the g-th 8-key
  // slice of tile t's P; segment s of group g = s / SEG holds the QK MFMA of
  // K fragment (g, s % SEG) for tile t+1 (if s % SEG < QPG; groups 0-1 build
  // scores 0-31, groups 2-3 scores 32-63) and the PV MFMA of d tile s % SEG
  // for group g - 1 (if g >= 1 and s % SEG < NDT); NDT tail segments finish
  // group 3's PV.
  constexpr int QPG = NST / 2;                      // K fragments per group
  constexpr int SEG = QPG > NDT ? QPG : NDT;        // segments per group
  constexpr int NSEG = NG * SEG + NDT;
  constexpr int EPS = 8 / SEG;                      // exp2 per segment
  constexpr int PD = 2;                             // operand read-ahead, segments
  auto has_qk = [](int s_) { return s_ < NG * SEG && (s_ % SEG) < QPG; };
  auto has_pv = [](int s_) { return s_ >= SEG && (s_ % SEG) < NDT; };
  auto kfrag = [&](int ks, int g, int i) {
    const int st = (g & 1) * QPG + i;
    return *reinterpret_cast<const bf16x8_t*>(kst + ks * L::TILEB + kx[st] + (g >> 1) * 32 * L::ROWB);
  };
  auto vfrag = [&](int vs, int g, int dt) {
    const char* vp = vst + vs * L::TILEB + vx[dt] + (32 * (g >> 1) + 16 * (g & 1)) * L::ROWB;
    const s16x4_t lo = ld_tr4(vp);
    const s16x4_t hi = ld_tr4(vp + 8 * L::ROWB);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // MFMA operands of segment s are read PD segments ahead into ring slot
  // s % (PD + 1), so each LDS read has PD segments of work to land in.
  bf16x8_t kr[PD + 1], vr[PD + 1];
  auto fetch = [&](int s1, int ks, int vs) {
    const int g1 = s1 / SEG, i1 = s1 % SEG;
    if (has_qk(s1)) kr[s1 % (PD + 1)] = kfrag(ks, g1, i1);
    if (has_pv(s1)) vr[s1 % (PD + 1)] = vfrag(vs, g1 - 1, i1);
  };

  // The fused body of one iteration, straight-line and explicitly ordered:
  // P of tile t (exp2, row sum, bf16 pack), the QK MFMAs of tile t+1 (-> nx)
  // and the PV MFMAs of tile t are interleaved segment by segment, so the
  // softmax VALU work issues while the matrix cores run.  The raw row max of
  // nx is taken here too, each half a few segments after its last QK MFMA.
  // The operands of segments 0 .. PD-1 have been fetched by the caller.
  auto fused = [&](f32x16_t (&sc)[2], int ks, int vs, f32x16_t (&nx)[2], float& nmax) {
    const float m_use = m == -INFINITY ? 0.f : m;
    nx[0] = f32x16_t{};
    nx[1] = f32x16_t{};
    float nm0 = -INFINITY, nm1 = -INFINITY;
    // Row max of the next tile: with two halves, nx[0]'s during segments
    // M0 .. M0 + 3 (after its last QK MFMA in group 1) and nx[1]'s in the NDT
    // tail segments; with one half, nx[0]'s in the tail segments.
    constexpr int M0 = 2 * SEG + 1;                 // segments taking nx[0]'s max
    constexpr int M1 = NG * SEG;                    // tail segments: the last half's max
    constexpr int V1 = 16 / NDT;                    // values per tail segment
    bf16x8_t pb = {};
    f32x8_t pf;
#pragma unroll
    for (int s_ = 0; s_ < NSEG; ++s_) {
      const int g = s_ / SEG, i = s_ % SEG;
      if (s_ + PD < NSEG) fetch(s_ + PD, ks, vs);
      // softmax VALU work of group g
      if (g < NG) {
        const int kt = g >> 1, u = g & 1;
#pragma unroll
        for (int e = i * EPS; e < (i + 1) * EPS; ++e) {
          pf[e] = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * u + e], p.scale_log2, -m_use));
          l += pf[e];   // float32 weights: the LSE must not carry bf16 rounding
        }
      }
      if (KT == 2 && s_ >= M0 && s_ < M0 + 4)
#pragma unroll
        for (int e = 4 * (s_ - M0); e < 4 * (s_ - M0 + 1); ++e) nm0 = fmaxf(nm0, nx[0][e]);
      if (s_ >= M1)
#pragma unroll
        for (int e = V1 * (s_ - M1); e < V1 * (s_ - M1 + 1); ++e) nm1 = fmaxf(nm1, nx[KT - 1][e]);
      const int slot = s_ % (PD + 1);
      if (has_pv(s_))
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[slot], pb, acc[i], 0, 0, 0);
      if (has_qk(s_))
        nx[g >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[slot], qreg[(g & 1) * QPG + i],
                                                            nx[g >> 1], 0, 0, 0);
      if (g < NG && i == SEG - 1) pb = __builtin_convertvector(pf, bf16x8_t);
      __builtin_amdgcn_sched_barrier(0);
    }
    nmax = fmaxf(nm0, nm1);
  };
  static_assert((KT == 1 || 2 * SEG + 1 + 4 <= NSEG) && 16 % NDT == 0, "max segments must fit the body");

  // Load pipeline.  K(t) is last read by the QK MFMAs of iteration t-1, so
  // K(t + KSTAGES) goes out at the start of iteration t; V(t) is read in
  // iteration t, so V(t + VSTAGES - 1) goes out at the start of iteration t.
  // Each iteration issues its V load before its K load.  The end-of-iteration
  // wait needs V(t+1) and K(t+2) and leaves every load issued after V(t+1)
  // in flight: vmcnt counts this wave's loads in issue order.
  constexpr int NIK = TileLoader<D, NW>::NI;     // load instructions per wave per tile
  constexpr int KA = L::KSTAGES, VA = L::VSTAGES - 1;   // K / V load lead in tiles
  static_assert(KA >= 2 && VA >= 1, "K(t+2) and V(t+1) must already be on their way");
  auto wait_vm = [&](int groups_after) {
    // s_waitcnt vmcnt(n): vmcnt[3:0] | expcnt 7 << 4 | lgkmcnt 0 << 8 | vmcnt[5:4] << 14
#define CA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14))
    switch (groups_after) {
      case 0: CA_WAIT_VM(0); break;
      case 1: CA_WAIT_VM(NIK); break;
      case 2: CA_WAIT_VM(2 * NIK); break;
      default: CA_WAIT_VM(3 * NIK); break;
    }
#undef CA_WAIT_VM
    block_sync();
  };

  // Tile descriptor ring: (doff[j], dlen[j]) describe tile t + j, j = 0..KA;
  // each is computed once, when the tile's K load is issued.
  int64_t doff[KA + 1];
  int dlen[KA + 1];
#pragma unroll
  for (int j = 0; j <= KA; ++j) {
    doff[j] = 0;
    dlen[j] = 0;
  }

  // Writes the softmax state of the tiles processed so far: O = acc / l and
  // LSE = ln 2 (m + log2 l) (empty key set: O = 0, LSE = -inf), to the
  // snapshot outputs (to_snap), else to the float32 partial slot of a split
  // query tile or to the final outputs.
  auto emit_state = [&](bool to_snap) {
    const float lt = half_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_row = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
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
          for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * r + e] * inv;
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
        for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * r + e] * inv;
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

  // One iteration: the first operand reads of the fused body go out right
  // after the barrier, ahead of the load issue and the rescale.
  float rawmax = -INFINITY;     // raw row max of the tile in `cur`
  // `par` = t % 2 as a compile-time constant (the loop below is unrolled by
  // two), which makes every stage index a constant offset.
  static_assert(L::KSTAGES == 2 && L::VSTAGES == 2, "stage indices below assume two stages");
  auto step = [&](int t, auto par, f32x16_t (&cur)[2], f32x16_t (&nx)[2]) {
    constexpr int P = decltype(par)::value;
    constexpr int ks = (P + 1) % 2, vs = P;
#pragma unroll
    for (int s1 = 0; s1 < PD; ++s1) fetch(s1, ks, vs);
    if (t + VA < ntiles)
      ldr.issue_v(vh + doff[VA], dlen[VA], stride_bytes, vst + ((P + VA) % 2) * L::TILEB);
    if (t + KA < ntiles) {
      tile_src(t + KA, doff[KA], dlen[KA]);
      ldr.issue_k(kh + doff[KA], dlen[KA], stride_bytes, kst + ((P + KA) % 2) * L::TILEB);
    }
    prep(cur, dlen[0], rawmax);
    fused(cur, ks, vs, nx, rawmax);
#pragma unroll
    for (int j = 0; j < KA; ++j) {
      doff[j] = doff[j + 1];
      dlen[j] = dlen[j + 1];
    }
    // Tile loads issued after the later of V(t+1) and K(t+2), which may stay
    // in flight.  V(t+1) went out in iteration t + 1 - VA and K(t+2) in
    // iteration t + 2 - KA (a negative iteration is the prologue, which ended
    // with a full wait); within an iteration V goes out before K.
    const int it_k = t + 2 - KA, it_v = t + 1 - VA;
    const int last_it = it_k > it_v ? it_k : it_v;
    const int last_slot = it_k >= it_v ? 1 : 0;
    int after = 0;
    for (int it = last_it > 0 ? last_it : 0; it <= t; ++it) {
      if ((it > last_it || last_slot < 0) && it + VA < ntiles) ++after;   // V(it + VA)
      if ((it > last_it || last_slot < 1) && it + KA < ntiles) ++after;   // K(it + KA)
    }
    wait_vm(after);
    if (MODE == MODE_BLOCKS && t == snap - 1) emit_state(true);
  };

  f32x16_t sa[2], sb[2];
  if (MODE == MODE_BLOCKS && snap == 0) emit_state(true);
  if (ntiles > 0) {
#pragma unroll
    for (int j = 0; j < KA; ++j)
      if (j < ntiles) {
        tile_src(j, doff[j], dlen[j]);
        ldr.issue_k(kh + doff[j], dlen[j], stride_bytes, kst + j * L::TILEB);
      }
#pragma unroll
    for (int j = 0; j < VA; ++j)
      if (j < ntiles) ldr.issue_v(vh + doff[j], dlen[j], stride_bytes, vst + j * L::TILEB);
    wait_vm(0);
    qk(0, sa);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) rawmax = fmaxf(rawmax, sa[kt][i]);
    // iteration 0 refills K stage 0, which every wave has just read
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    block_sync();
    for (int t = 0; t < ntiles; t += 2) {
      step(t, std::integral_constant<int, 0>{}, sa, sb);
      if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{}, sb, sa);
    }
  }

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
  const int g0 = g_of_unit(u0, p.n_units, p.n_wgs);
  const int g1 = g_of_unit(u0 + nt - 1, p.n_units, p.n_wgs);
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
  const int slot0 = unit_begin(g0, p.n_units, p.n_wgs) < u0 ? 2 * g0 + 1 : 2 * g0;
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
