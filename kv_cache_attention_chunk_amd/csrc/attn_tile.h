// The streaming tile loop of the chunk-attention kernels for gfx950 (internal).
//
// A wave owns 32 query rows and a group of NWL waves streams one key set in
// tiles of TK keys (64, or 32 for the per-query-block lists):
//   * K and V tiles go straight from global memory to LDS with buffer loads
//     (buffer_load_dwordx4 ... lds, 1 KB per wave instruction, the NWL waves
//     of the group each filling their share): no staging registers, and the
//     buffer range check returns zeros for rows past a partial tile.  With
//     two K and two V stages, K(t+2) and V(t+1) are loaded during iteration
//     t; with four, K(t+3) and V(t+2), and the barrier comes every second
//     iteration.
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
// Every wave of the workgroup takes part in the loop's barriers, so all the
// groups of a workgroup run the same number of tiles.
#pragma once

#include "common.h"

#include <type_traits>

namespace chunkattn {
namespace tile {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBufferWord3 = 0x00020000;   // raw buffer resource, gfx9 family
constexpr int kStages = 2;                 // K and V stages of a ring, unless a caller asks for 4

// physical 16-byte chunk of logical chunk c in row r: c ^ swz_k(r) for K,
// c ^ swz_v(r) for V
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int D, int TK>
struct Geom {
  static constexpr int ROWB = 2 * D;                    // bytes per K / V row
  static constexpr int TILEB = TK * ROWB;               // bytes per K or V tile
  static constexpr int RING = 2 * kStages * TILEB;      // K stages + V stages
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

// Per-lane byte offsets of the buffer->LDS loads of one TK x D tile by a
// group of NWL waves: wave w of the group fills LDS bytes [(NI w + j) KB,
// +1 KB) with its instruction j, lane i the 16 bytes at +16 i, i.e. physical
// row r and chunk pc; it loads logical chunk pc ^ swizzle(r) of row r.
template <int D, int TK, int NWL>
struct Loader {
  using G = Geom<D, TK>;
  static constexpr int NI = G::TILEB / (1024 * NWL);
  static_assert(NI >= 1 && NI * 1024 * NWL == G::TILEB, "the group's loads must fill a tile");
  uint32_t koff[NI], voff[NI];
  int wave;

  __device__ __forceinline__ void init(int lane, int wave_, uint32_t stride_bytes) {
    wave = wave_;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int pbyte = (NI * wave + j) * 1024 + 16 * lane;
      const int r = pbyte / G::ROWB;
      const int pc = (pbyte % G::ROWB) / 16;
      koff[j] = r * stride_bytes + 16 * (pc ^ swz_k<D>(r));
      voff[j] = r * stride_bytes + 16 * (pc ^ swz_v<D>(r));
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

// Softmax state of the 32 query rows of a wave: Q^T operands, the O^T
// accumulators (d tiles of 32), the running max m (log2 domain) and this
// lane's partial row sum l (the lane halves are added at the end).
template <int D>
struct Rows {
  static constexpr int NST = D / 16;     // MFMA k-steps over d for S
  static constexpr int NDT = D / 32;     // 32-row d tiles of O^T
  bf16x8_t qreg[NST];
  f32x16_t acc[NDT];
  float m, l;
  // Per-lane LDS read offsets within a stage.  Row base, stage offset and
  // the swizzled chunk occupy disjoint address bits, so each read is
  // (base | swizzle) ^ (step * chunk), one v_xor per read.
  //   K rows 32kt + col, chunk 2st + hg: byte 16((2st + hg) ^ kz)
  //     = 32(st ^ (kz >> 1)) + 16(hg ^ (kz & 1)).
  //   V source row 4hg + (lane & 15)/4 (+ 32kt + 16u + 8 half), chunk
  //   4dt + vcol16: byte 16((4dt + vcol16) ^ vz) = 64(dt ^ vz/4) + 16 vcol16.
  int kx[NST], vx[NDT];

  __device__ __forceinline__ void init_offsets(int lane) {
    constexpr int ROWB = 2 * D;
    const int col = lane & 31, hg = lane >> 5;
    const int kz = swz_k<D>(col);
    const int kbx = col * ROWB + 16 * (hg ^ (kz & 1)) + 32 * (kz >> 1);
#pragma unroll
    for (int st = 0; st < NST; ++st) kx[st] = kbx ^ (32 * st);
    const int vz = D == 128 ? ((lane & 15) >> 2) : ((lane >> 3) & 1);
    const int vcol16 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int vbx = (4 * hg + ((lane & 15) >> 2)) * ROWB + 8 * (lane & 1) + 16 * vcol16 + 64 * vz;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vx[dt] = vbx ^ (64 * dt);
  }

  // Q^T operands of query row `qrow` (zeros when !valid).
  __device__ __forceinline__ void load_q(const uint16_t* qp_row, bool valid, int hg) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const u32x4_t x = valid ? ld16(qp_row + 8 * hg + 16 * s) : u32x4_t{0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < NDT; ++i) acc[i] = f32x16_t{};
    m = -INFINITY;
    l = 0.f;
  }
};

// Streams `ntiles` tiles of TK keys through the ring at kst (K stages) and
// vst (V stages) and folds them into the rows' softmax state.  tile_src(t,
// off, len) gives tile t's element offset from kh / vh and its valid rows; it
// is called for t = 0, 1, 2, ... in order.  after_tile(t) runs in each wave
// once tile t has been folded into its rows.
//
// NS is the number of K stages and of V stages in the ring (2 or 4, each
// TK x D).  With 2, every iteration ends with the workgroup barrier; with 4,
// loads run one tile further ahead and only every second iteration ends with
// one (the ring then holds the two tiles being read and the two being
// loaded).
template <int D, int TK, int NWL, int NS = kStages, class Src, class After>
__device__ __forceinline__ void run(Rows<D>& rs, const Loader<D, TK, NWL>& ldr, char* kst,
                                    char* vst, const uint16_t* kh, const uint16_t* vh,
                                    uint32_t stride_bytes, int ntiles, float scale_log2, int hg,
                                    Src& tile_src, After&& after_tile) {
  using G = Geom<D, TK>;
  constexpr int NST = Rows<D>::NST;
  constexpr int NDT = Rows<D>::NDT;
  constexpr int KT = TK / 32;     // 32-key halves of a tile (S accumulators)
  constexpr int NG = 2 * KT;      // 16-key P groups of a tile
  float& m = rs.m;
  float& l = rs.l;

  // S^T = K Q^T for the 32-key halves of the tile in K stage ks.
  auto qk = [&](int ks, f32x16_t (&sc)[2]) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sc[kt] = f32x16_t{};
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            kst + ks * G::TILEB + rs.kx[st] + kt * 32 * G::ROWB);
        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, rs.qreg[st], sc[kt], 0, 0, 0);
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
    mx = half_max(mx) * scale_log2;
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
      for (int i = 0; i < NDT; ++i) rs.acc[i] *= alpha;
    }
  };

  // Segments of the fused iteration body.  Group g (0..NG-1) is the g-th
  // 16-key slice of tile t's P (8 values per lane); segment s of group
  // g = s / SEG holds the QK MFMA of K fragment (g, s % SEG) for tile t+1
  // (if s % SEG < QPG; groups 0-1 build scores 0-31, groups 2-3 scores
  // 32-63) and the PV MFMA of d tile s % SEG for group g - 1 (if g >= 1 and
  // s % SEG < NDT); NDT tail segments finish the last group's PV.
  constexpr int QPG = NST / 2;                      // K fragments per group
  constexpr int SEG = QPG > NDT ? QPG : NDT;        // segments per group
  constexpr int NSEG = NG * SEG + NDT;
  constexpr int EPS = 8 / SEG;                      // exp2 per segment
  constexpr int PD = 2;                             // operand read-ahead, segments
  auto has_qk = [](int s_) { return s_ < NG * SEG && (s_ % SEG) < QPG; };
  auto has_pv = [](int s_) { return s_ >= SEG && (s_ % SEG) < NDT; };
  auto kfrag = [&](int ks, int g, int i) {
    const int st = (g & 1) * QPG + i;
    return *reinterpret_cast<const bf16x8_t*>(kst + ks * G::TILEB + rs.kx[st] +
                                              (g >> 1) * 32 * G::ROWB);
  };
  auto vfrag = [&](int vs, int g, int dt) {
    const char* vp = vst + vs * G::TILEB + rs.vx[dt] + (32 * (g >> 1) + 16 * (g & 1)) * G::ROWB;
    const s16x4_t lo = ld_tr4(vp);
    const s16x4_t hi = ld_tr4(vp + 8 * G::ROWB);
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
          pf[e] = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * u + e], scale_log2, -m_use));
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
        rs.acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[slot], pb, rs.acc[i], 0, 0, 0);
      if (has_qk(s_))
        nx[g >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[slot], rs.qreg[(g & 1) * QPG + i],
                                                            nx[g >> 1], 0, 0, 0);
      if (g < NG && i == SEG - 1) pb = __builtin_convertvector(pf, bf16x8_t);
      __builtin_amdgcn_sched_barrier(0);
    }
    nmax = fmaxf(nm0, nm1);
  };
  static_assert((KT == 1 || 2 * SEG + 1 + 4 <= NSEG) && 16 % NDT == 0, "max segments must fit the body");

  // Load pipeline.  K(t) is last read by the QK MFMAs of iteration t-1 and
  // V(t) in iteration t.
  //   NS = 2: K(t + 2) and V(t + 1) go out at the start of iteration t, into
  //   the stages of K(t) and V(t - 1), read before the previous barrier.  The
  //   end-of-iteration wait needs V(t+1) and K(t+2) and leaves every load
  //   issued after V(t+1) in flight (vmcnt counts this wave's loads in issue
  //   order; each iteration issues its V load before its K load).
  //   NS = 4: K(t + 3) and V(t + 2) go out at the start of iteration t.  The
  //   barrier follows the odd iterations only: iterations 2u and 2u + 1 read
  //   K(2u+1), K(2u+2), V(2u), V(2u+1), all loaded during iterations 2u-2
  //   and 2u-1, and refill the stages of K(2u-1), K(2u), V(2u-2), V(2u-1),
  //   all read before the barrier that ends iteration 2u-1; that barrier
  //   follows a wait for every load in flight.
  static_assert(NS == 2 || NS == 4, "two or four stages");
  constexpr int NIK = Loader<D, TK, NWL>::NI;    // load instructions per wave per tile
  constexpr int KA = NS == 2 ? 2 : 3, VA = KA - 1;  // K / V load lead in tiles
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

  // One iteration: the first operand reads of the fused body go out right
  // after the barrier, ahead of the load issue and the rescale.
  float rawmax = -INFINITY;     // raw row max of the tile in `cur`
  // `par` = t % NS as a compile-time constant (the loop below is unrolled by
  // NS), which makes every stage index a constant offset.
  auto step = [&](int t, auto par, f32x16_t (&cur)[2], f32x16_t (&nx)[2]) {
    constexpr int P = decltype(par)::value;
    constexpr int ks = (P + 1) % NS, vs = P;
#pragma unroll
    for (int s1 = 0; s1 < PD; ++s1) fetch(s1, ks, vs);
    if (t + VA < ntiles)
      ldr.issue_v(vh + doff[VA], dlen[VA], stride_bytes, vst + ((P + VA) % NS) * G::TILEB);
    if (t + KA < ntiles) {
      tile_src(t + KA, doff[KA], dlen[KA]);
      ldr.issue_k(kh + doff[KA], dlen[KA], stride_bytes, kst + ((P + KA) % NS) * G::TILEB);
    }
    prep(cur, dlen[0], rawmax);
    fused(cur, ks, vs, nx, rawmax);
#pragma unroll
    for (int j = 0; j < KA; ++j) {
      doff[j] = doff[j + 1];
      dlen[j] = dlen[j + 1];
    }
    if (NS == 4) {
      if (P % 2 == 1) wait_vm(0);
      after_tile(t);
      return;
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
    after_tile(t);
  };

  f32x16_t sa[2], sb[2];
  if (ntiles > 0) {
#pragma unroll
    for (int j = 0; j < KA; ++j)
      if (j < ntiles) {
        tile_src(j, doff[j], dlen[j]);
        ldr.issue_k(kh + doff[j], dlen[j], stride_bytes, kst + j * G::TILEB);
      }
#pragma unroll
    for (int j = 0; j < VA; ++j)
      if (j < ntiles) ldr.issue_v(vh + doff[j], dlen[j], stride_bytes, vst + j * G::TILEB);
    wait_vm(0);
    qk(0, sa);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) rawmax = fmaxf(rawmax, sa[kt][i]);
    // iteration 0 (NS = 2) or 1 (NS = 4) refills K stage 0, which every wave
    // has just read
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    block_sync();
    for (int t = 0; t < ntiles; t += NS) {
      step(t, std::integral_constant<int, 0>{}, sa, sb);
      if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{}, sb, sa);
      if (NS == 4) {
        if (t + 2 < ntiles) step(t + 2, std::integral_constant<int, 2 % NS>{}, sa, sb);
        if (t + 3 < ntiles) step(t + 3, std::integral_constant<int, 3 % NS>{}, sb, sa);
      }
    }
    // with four stages an even last iteration ends without the barrier that
    // orders the ring's LDS against whatever the caller does next
    if (NS == 4 && ntiles % 2 == 1) wait_vm(0);
  }
}

}  // namespace tile
}  // namespace chunkattn
