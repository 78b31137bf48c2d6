// Fused chunk-attention forward for gfx950 (MI355X).
//
// One workgroup owns NW*32 query rows of one (b, h) and streams that head's
// key set in 64-token tiles:
//   * K and V tiles go global -> registers -> LDS, double buffered; the next
//     tile's global loads are in flight while the current tile is computed.
//     Both are stored row-major [key][d] with 16-byte row writes; the row
//     pads (16 B for K, 64 B for V) keep every LDS read pattern below free of
//     bank conflicts.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K tile rows (keys), B =
//     Q^T held in registers for the whole loop (lane = query column).  The
//     accumulator layout puts one query per lane column, so the row max and
//     row sum over keys are in-lane except for one exchange with lane^32.
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

namespace chunkattn {

namespace {

constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Layout {
  static constexpr int KROW = D + 8;               // bf16 per K row in LDS (+16 B)
  static constexpr int VROW = D + 32;              // bf16 per V row in LDS (+64 B)
  static constexpr int STAGE = kTileKeys * (KROW + VROW);
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
};

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Global -> register staging of one K/V tile and register -> LDS store.
// Thread c of the workgroup moves 16-byte chunks c, c + NT, ... of each
// 64 x D tile (row = chunk / (D/8)); rows past the tile length are zero.
template <int D, int NT>
struct TileStage {
  using L = Layout<D>;
  static constexpr int N = (kTileKeys * L::CPR) / NT;            // chunks / thread
  u32x4_t kr[N];
  u32x4_t vr[N];

  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb,
                                       int64_t stride, int len, int tid) {
    if (len == kTileKeys) {          // full tile: no per-row predicates
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int c = tid + i * NT;
        const int64_t off = (c / L::CPR) * stride + (c % L::CPR) * 8;
        kr[i] = ld16(kb + off);
        vr[i] = ld16(vb + off);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT;
      const int row = c / L::CPR;
      const int64_t off = row * stride + (c % L::CPR) * 8;
      kr[i] = row < len ? ld16(kb + off) : u32x4_t{0, 0, 0, 0};
      vr[i] = row < len ? ld16(vb + off) : u32x4_t{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(uint16_t* stage, int tid) const {
    uint16_t* ks = stage;
    uint16_t* vs = stage + kTileKeys * L::KROW;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT;
      const int row = c / L::CPR;
      const int col = (c % L::CPR) * 8;
      *reinterpret_cast<u32x4_t*>(ks + row * L::KROW + col) = kr[i];
      *reinterpret_cast<u32x4_t*>(vs + row * L::VROW + col) = vr[i];
    }
  }
};

// max of x over lanes l and l ^ 32 (the two halves of one query column),
// exchanged with v_permlane32_swap instead of an LDS permute.
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

// Transposing LDS read of 4 bf16 (see the header comment for the lane layout).
__device__ __forceinline__ s16x4_t ld_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<uint16_t*>(p)));
}

// Two waves per SIMD: caps VGPR + AGPR at 256 per lane so that two 4-wave
// workgroups share a CU and one wave's softmax overlaps the other's MFMAs.
template <int D, int NW, int MODE, bool OF32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const AttnParams p) {
  using L = Layout<D>;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int NST = D / 16;     // MFMA k-steps over d for S
  constexpr int NDT = D / 32;     // 32-row d tiles of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;      // query column (B/C operands) or A-operand row
  const int hg = lane >> 5;       // lane half: selects k sub-range / row quad

  // ---- work item ---------------------------------------------------------
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= p.n_items) return;
  int sel, row0, nrows, csr_row = 0;
  if (MODE == MODE_BLOCKS) {
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
    const int bh_ = p.use_list ? p.heads[sel] : sel;
    csr_row = bh_ * p.nqb + qb;
  } else {
    sel = item / p.n_qtiles;
    const int qt = item - sel * p.n_qtiles;
    row0 = qt * BM;
    nrows = p.Nq - row0;
    if (nrows > BM) nrows = BM;
  }
  const int bh = p.use_list ? p.heads[sel] : sel;
  const int b = bh / p.H;
  const int h = bh - b * p.H;

  // ---- key set -------------------------------------------------------------
  int ntiles;
  int kv_lo = 0, kv_len = 0, list0 = 0;
  const uint16_t* kh;
  const uint16_t* vh;
  if (MODE == MODE_DENSE) {
    kv_len = p.Nkv;
    ntiles = (kv_len + kTileKeys - 1) / kTileKeys;
    kh = p.k + b * p.ks_b + h * p.ks_h;
    vh = p.v + b * p.ks_b + h * p.ks_h;
  } else if (MODE == MODE_VARLEN) {
    int lo = p.cu[bh], hi = p.cu[bh + 1];
    lo = lo < 0 ? 0 : (lo > p.total_kv ? p.total_kv : lo);
    hi = hi < lo ? lo : (hi > p.total_kv ? p.total_kv : hi);
    kv_lo = lo;
    kv_len = hi - lo;
    ntiles = (kv_len + kTileKeys - 1) / kTileKeys;
    kh = p.k;
    vh = p.v;
  } else {
    int lo = p.indptr[csr_row], hi = p.indptr[csr_row + 1];
    lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
    hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
    list0 = lo;
    ntiles = hi - lo;
    kh = p.k + b * p.ks_b + h * p.ks_h;
    vh = p.v + b * p.ks_b + h * p.ks_h;
  }

  auto tile_src = [&](int t, int64_t& off, int& len) {
    if (MODE == MODE_BLOCKS) {
      const int id = p.indices[list0 + t];
      int s = 0, l = 0;
      if (id >= 0 && id < p.nkb) block_span(id, p.Nkv, p.kv_block, p.kv_seg, p.kv_bps, s, l);
      off = (int64_t)s * p.ks_n;
      len = l;
    } else {
      const int s = t * kTileKeys;
      const int rest = kv_len - s;
      off = (int64_t)(kv_lo + s) * p.ks_n;
      len = rest < kTileKeys ? rest : kTileKeys;
    }
  };

  // ---- Q^T operand in registers ---------------------------------------------
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

  f32x16_t acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16_t{};
  float m = -INFINITY;   // running max, log2 domain
  float l = 0.f;         // this lane's partial row sum

  TileStage<D, NT> stg;
  if (ntiles > 0) {
    int64_t off;
    int len;
    tile_src(0, off, len);
    stg.load(kh + off, vh + off, p.ks_n, len, tid);
    stg.store(smem, tid);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    int64_t off_cur;
    int len_cur;
    tile_src(t, off_cur, len_cur);
    const bool more = t + 1 < ntiles;
    if (more) {
      int64_t off;
      int len;
      tile_src(t + 1, off, len);
      stg.load(kh + off, vh + off, p.ks_n, len, tid);
    }
    const uint16_t* ks = smem + (t & 1) * L::STAGE;
    // this lane's source address for the transposing V reads: key row
    // 4*(lane/32) + (lane%16)/4, column 16*((lane/16)%2) + 4*(lane%4)
    const uint16_t* vtr = ks + kTileKeys * L::KROW +
                          (4 * hg + ((lane & 15) >> 2)) * L::VROW +
                          16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // S^T = K Q^T for two 32-key sub-tiles
    f32x16_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16_t{};
      const uint16_t* kp = ks + (32 * kt + col) * L::KROW + 8 * hg;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + 16 * st);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[st], s[kt], 0, 0, 0);
      }
    }

    // online softmax in the log2 domain; key of s[kt][i] = 32kt + 8(i/4) + 4hg + i%4.
    // Row max of the raw scores (scale > 0 keeps the order), one exchange
    // with lane^32 (the other half of the same query column).
    if (len_cur < kTileKeys) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kt + 8 * (i >> 2) + 4 * hg + (i & 3);
          if (key >= len_cur) s[kt][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    mx = half_max(mx) * p.scale_log2;
    // The exponent base m is the exact running row max, so the largest weight
    // of a row is exactly 1 and survives the bf16 rounding of P unchanged.
    // The O accumulator is rescaled only when some row of the wave found a
    // new max in this tile (a minority of tiles once a few have been seen).
    const bool grow = mx > m;
    if (__any(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - (m_new == -INFINITY ? 0.f : m_new));
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) acc[i] *= alpha;
    }
    const float m_use = m == -INFINITY ? 0.f : m;

#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x8_t pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[e] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * u + e], p.scale_log2, -m_use));
          l += pf[e];    // float32 weights: the LSE must not carry bf16 rounding
        }
        const bf16x8_t pb = __builtin_convertvector(pf, bf16x8_t);
        // A = V^T rows d = 32dt + (lane & 31), keys 32kt + 16u + {4hg..4hg+3,
        // 8+4hg..8+4hg+3}: two transposing reads of 4 keys each.
        const uint16_t* vp = vtr + (32 * kt + 16 * u) * L::VROW;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const s16x4_t lo = ld_tr4(vp + 32 * dt);
          const s16x4_t hi = ld_tr4(vp + 8 * L::VROW + 32 * dt);
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[dt], 0, 0, 0);
        }
      }
    }

    if (more) stg.store(smem + ((t + 1) & 1) * L::STAGE, tid);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
  const float lt = half_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    const int64_t obase = b * p.os_b + (int64_t)qrow * p.os_n + h * p.os_h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * dt + 8 * r + 4 * hg;
        f32x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * r + e] * inv;
        if (OF32) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.o) + obase + d0) = v4;
        } else {
          typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
          const bf16x4_t bv = __builtin_convertvector(v4, bf16x4_t);
          *reinterpret_cast<bf16x4_t*>(reinterpret_cast<uint16_t*>(p.o) + obase + d0) = bv;
        }
      }
    }
    if (hg == 0) {
      p.lse[(int64_t)bh * p.Nq + qrow] =
          lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int NW, int MODE>
hipError_t launch_t(bool of32, const AttnParams& p, hipStream_t stream) {
  const dim3 grid(p.n_items), block(NW * 64);
  if (of32)
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, MODE, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, MODE, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_mode(int mode, bool of32, const AttnParams& p, hipStream_t stream) {
  switch (mode) {
    case MODE_DENSE: return launch_t<D, NW, MODE_DENSE>(of32, p, stream);
    case MODE_BLOCKS: return launch_t<D, NW, MODE_BLOCKS>(of32, p, stream);
    default: return launch_t<D, NW, MODE_VARLEN>(of32, p, stream);
  }
}

}  // namespace

hipError_t launch_attention(int mode, int d, int nwaves, bool out_f32, const AttnParams& p,
                            hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  if (d == 64)
    return nwaves == 2 ? launch_mode<64, 2>(mode, out_f32, p, stream)
                       : launch_mode<64, 4>(mode, out_f32, p, stream);
  return nwaves == 2 ? launch_mode<128, 2>(mode, out_f32, p, stream)
                     : launch_mode<128, 4>(mode, out_f32, p, stream);
}

}  // namespace chunkattn
