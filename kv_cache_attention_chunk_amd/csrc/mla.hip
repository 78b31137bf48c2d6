// Chunk attention over a latent KV cache (VideoMLA page, method): the cache
// keeps per token one content latent c_t (DC = 192 values) and one rotated
// position key k^R_t (DR = 32), shared by all heads; head h's keys and values
// are [W^K_h c_t ; k^R_t] and W^V_h c_t.  Folding W^K_h into the query
// (q~ = (W^K_h)^T q^nope) and W^V_h into the output turns every (query, head)
// pair into a row attending to the same latent rows:
//   s = scale ([q~ ; q^R] . [c_t ; k^R_t]),   o~ = sum_t softmax(s)_t c_t,
//   o_h = W^V_h o~.
// Three kernels: the per-head projections (query absorption, value
// up-projection) and the latent attention.
//
// Latent attention (mla_attn_kernel).  One workgroup = 8 waves x 32 rows of
// one batch entry; rows are (query, head) pairs, so every row of the grid
// streams the same latent rows, 32 at a time.  Such a half-tile [32 x 224]
// serves as K (all 224 values) and as V (the first 192).  The operands are fp16: the absorbed
// query is rounded once to fp16 (11-bit significand; bf16 would put its
// rounding error on every score), the latent cache is kept in fp16 (a bf16
// cache converts exactly in its normal range, see ca_cast_bf16_to_f16), and P
// is rounded to fp16 for the PV product; all accumulation is float32.
// Half-tiles go from global memory to LDS with buffer loads (no staging
// registers) into rows padded to 512 bytes, a ring of four stages loaded three
// steps ahead; each step interleaves the softmax and P V of one half-tile with
// the scores of the next.  Chunk c of row r sits at
// c ^ (4 (r & 3) + ((r >> 2) & 3)): sixteen consecutive rows take sixteen
// distinct chunk slots (the S = K Q^T operand reads) and four consecutive
// rows take four disjoint groups of four slots (the transposing V^T reads),
// so both read patterns are free of bank conflicts.
#include "common.h"

#include <type_traits>

namespace chunkattn {

namespace {

constexpr int kMlaDC = 192;               // content latent
constexpr int kMlaDR = 32;                // position key
constexpr int kMlaDK = kMlaDC + kMlaDR;   // 224 cached values per token
constexpr int kMlaRowB = 512;             // LDS bytes per latent row (448 used)
constexpr int kMlaNW = 8;                 // 256 rows per workgroup, one per CU
constexpr int kMlaQLds = 2;               // Q^T fragments per wave kept in LDS
constexpr float kLn2f = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ int mla_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

__device__ __forceinline__ float mla_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float mla_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kBufWord3 = 0x00020000;      // raw buffer resource, gfx9 family
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

__device__ __forceinline__ lds_void_t* mla_dma_dst(char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_char_t*)p;
  return (lds_void_t*)(uintptr_t)__builtin_amdgcn_readfirstlane(a);
}

struct MlaParams {
  const uint16_t* q;       // fp16 [B, Nq, H, 224] contiguous (absorbed query ; q^R)
  const uint16_t* q_lo;    // optional bf16 [B, Nq, H, 192]: absorbed query - fp16(absorbed query)
  const uint16_t* kv;      // fp16 latent rows, 224 values each
  int64_t kv_bs, kv_rs;    // batch and row strides of kv, elements
  float* o;                // float32 [B, Nq, H, 192] contiguous
  float* lse;              // float32 [B, H, Nq]
  int B, Nq, H, Nkv;
  int rows_per_b;          // Nq * H
  int wg_per_b;
  float scale_log2;
  float scale;
};

// Half-tiles of 32 latent rows flow through a ring of four LDS stages
// (16 KB each): half-tile u sits in stage u % 4 and is loaded three
// iterations ahead.  Iteration u turns the scores of half-tile u (computed in
// iteration u - 1) into P, accumulates O^T += V^T P^T for it and computes the
// scores of half-tile u + 1, the three interleaved segment by segment.
constexpr int kMlaHalf = 32;                         // latent rows per step
constexpr int kMlaStages = 4;
constexpr int kMlaStageB = kMlaHalf * kMlaRowB;      // 16 KB

__global__ __launch_bounds__(kMlaNW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mla_attn_kernel(const MlaParams p) {
  constexpr int BM = kMlaNW * 32;
  constexpr int NST = kMlaDK / 16;        // 14 k-steps of S
  constexpr int NDT = kMlaDC / 32;        // 6 d-tiles of O^T
  constexpr int CPR = kMlaDK / 8;         // 28 16-byte chunks per latent row
  constexpr int NLD = kMlaStageB / (1024 * kMlaNW);  // buffer->LDS loads per wave per half-tile
  static_assert(NLD >= 1 && NLD * 1024 * kMlaNW == kMlaStageB, "the loads must fill a stage");
  static_assert(NST == 14 && NDT == 6, "the segment plan below is laid out for 224 / 192");
  __shared__ __attribute__((aligned(1024))) char lat[kMlaStages * kMlaStageB];
  // the last NQL Q^T fragments (the position part q^R) of each wave, read
  // back from LDS in the segments that use them, when the score and P
  // registers of the step are already free: kept in registers for the whole
  // loop they would push it past 256 VGPRs into scratch spills
  constexpr int NQR = NST - kMlaQLds;
  __shared__ __attribute__((aligned(16))) char qx[kMlaNW * kMlaQLds * 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hg = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int b = item / p.wg_per_b;
  const int r0 = (item - b * p.wg_per_b) * BM;
  const int qr = wave * 32 + col;
  const int rloc = r0 + qr;                          // row within batch entry b
  const bool qvalid = rloc < p.rows_per_b;
  const int64_t rglob = (int64_t)b * p.rows_per_b + rloc;

  // Q^T operands: row rloc, values 16 st + 8 hg .. + 8
  f16x8_t qreg[NQR];
  char* const qxw = qx + (wave * kMlaQLds * 64 + lane) * 16;   // this lane's fragments
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qvalid) x = *reinterpret_cast<const u32x4_t*>(p.q + rglob * kMlaDK + 16 * st + 8 * hg);
    if (st < NQR)
      qreg[st] = __builtin_bit_cast(f16x8_t, x);
    else
      *reinterpret_cast<u32x4_t*>(qxw + (st - NQR) * 1024) = x;
  }
  // (each lane reads back only what it wrote: no barrier needed)
  auto qlds = [&](int st) { return *reinterpret_cast<const f16x8_t*>(qxw + (st - NQR) * 1024); };

  // Loads of half-tile u into stage u % 4: lane i of wave w's instruction j
  // fills physical row pr = 2 (NLD w + j) + i / 32 of the stage, slot i % 32,
  // with logical chunk (i % 32) ^ swz(pr).  Each instruction's buffer starts
  // at its row pair (a uniform base), whose valid bytes bound the range
  // check: rows past the cache and padding slots (logical chunk >= 28, given
  // an out-of-range offset) read as zeros.
  const uint32_t rs_bytes = (uint32_t)(p.kv_rs * 2);
  const uint16_t* kvb = p.kv + b * p.kv_bs;
  const int nh = (p.Nkv + kMlaHalf - 1) / kMlaHalf;
  auto issue = [&](int u) {
    const int valid = p.Nkv - u * kMlaHalf < kMlaHalf ? p.Nkv - u * kMlaHalf : kMlaHalf;
    char* base = lat + (u % kMlaStages) * kMlaStageB;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int pr0 = 2 * (NLD * wave + j);
      const int here = valid - pr0;                     // valid rows from pr0 on
      const int nrec = here >= 2 ? (int)rs_bytes + 2 * kMlaDK : (here == 1 ? 2 * kMlaDK : 0);
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(kvb + ((int64_t)u * kMlaHalf + pr0) * p.kv_rs), (short)0, nrec,
          kBufWord3);
      // (the empty asm keeps this offset at the load instead of a live register)
      int cl = col, h1 = hg;
      asm volatile("" : "+v"(cl), "+v"(h1));
      const int c = cl ^ mla_swz(pr0 + h1);
      const uint32_t voff = c < CPR ? (uint32_t)h1 * rs_bytes + 16u * c : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, mla_dma_dst(base + (NLD * wave + j) * 1024), 16,
                                               (int)voff, 0, 0, 0);
    }
  };
  auto block_sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // MFMA operands.  S^T = K Q^T: A = latent rows (keys) of a stage, row col,
  // chunk (2 s + hg) ^ swz(col) for k-step s.  O^T += V^T P^T: A = V^T read
  // with transposing loads; group g covers keys 16 g .. 16 g + 15 of the
  // half-tile (P values cur[8 g + e], key 16 g + 8 (e / 4) + 4 hg + e % 4):
  // rows vr = 16 g + 4 hg + (lane & 15) / 4 and vr + 8, chunk 4 dt + vcol16
  // swizzled by swz(vr) = 4 ((lane & 15) / 4) + hg and swz(vr + 8) = that + 2.
  // Both swizzles only touch the low four chunk bits, so k-steps s and s + 8
  // (d-tiles dt and dt + 4) differ by 256 bytes and groups by 16 rows: eight
  // per-lane offsets for K and eight for V cover every read, the rest is an
  // immediate.
  const int zk = mla_swz(col);
  const int vcol16 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int r4 = (lane & 15) >> 2;
  int ka[8], va[4], vb[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) ka[s] = col * kMlaRowB + 16 * ((2 * s + hg) ^ zk);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    va[q] = (4 * hg + r4) * kMlaRowB + 16 * ((4 * q + vcol16) ^ (4 * r4 + hg)) + 8 * (lane & 1);
    vb[q] = (4 * hg + r4 + 8) * kMlaRowB + 16 * ((4 * q + vcol16) ^ (4 * r4 + hg + 2)) + 8 * (lane & 1);
  }
  auto kfrag = [&](int stg, int s) {
    return *reinterpret_cast<const f16x8_t*>(lat + stg * kMlaStageB + ka[s & 7] + 256 * (s >> 3));
  };
  auto vfrag = [&](int stg, int g, int dt) {
    const char* sb = lat + stg * kMlaStageB + 16 * g * kMlaRowB + 256 * (dt >> 2);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<char*>(sb + va[dt & 3])));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<char*>(sb + vb[dt & 3])));
    return __builtin_bit_cast(f16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16_t{};
  float m = -INFINITY, l = 0.f;
  float rawmax = -INFINITY;     // raw row max of the half-tile in `cur`

  // Segment plan of one iteration (14 segments):
  //   QK: k-step s of the next half-tile's scores in segment s;
  //   exp2 of P group 0 in segments 0-3, of group 1 in 4-7 (two per segment);
  //   PV: group 0, d-tile s - 4 in segments 4-9; group 1, d-tile s - 8 in 8-13.
  // Operands of segment s + 1 are read during segment s (two register slots).
  auto step = [&](int u, auto par, f32x16_t& cur, f32x16_t& nx) {
    constexpr int P = decltype(par)::value;
    constexpr int vs = P % kMlaStages, ks = (P + 1) % kMlaStages;
    if (u + kMlaStages - 1 < nh) issue(u + kMlaStages - 1);   // stage of half-tile u - 1
    // row max over this half-tile and the accumulator rescale
    const int len = p.Nkv - u * kMlaHalf;
    float mx = rawmax;
    if (len < kMlaHalf) {
      mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hg + (i & 3);
        if (key >= len) cur[i] = -INFINITY;
        mx = fmaxf(mx, cur[i]);
      }
    }
    mx = mla_half_max(mx) * p.scale_log2;
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

    f16x8_t kr[2], v0[2], v1[2], qf[2];
    auto fetch = [&](int s1) {
      if (s1 < NST) kr[s1 & 1] = kfrag(ks, s1);
      if (s1 >= NQR && s1 < NST) qf[s1 & 1] = qlds(s1);
      if (s1 >= 4 && s1 < 10) v0[s1 & 1] = vfrag(vs, 0, s1 - 4);
      if (s1 >= 8 && s1 < 14) v1[s1 & 1] = vfrag(vs, 1, s1 - 8);
    };
    nx = f32x16_t{};
    f32x8_t pf;
    f16x8_t pb0 = {}, pb1 = {};
    fetch(0);
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      if (s + 1 < NST) fetch(s + 1);
      if (s < 8) {
        const int g = s >> 2;
#pragma unroll
        for (int e = 2 * (s & 3); e < 2 * (s & 3) + 2; ++e) {
          pf[e] = __builtin_amdgcn_exp2f(fmaf(cur[8 * g + e], p.scale_log2, -m_use));
          l += pf[e];   // float32 weights: the LSE must not carry the fp16 rounding of P
        }
        if (s == 3) pb0 = __builtin_convertvector(pf, f16x8_t);
        if (s == 7) pb1 = __builtin_convertvector(pf, f16x8_t);
      }
      if (s >= 4 && s < 10) acc[s - 4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0[s & 1], pb0, acc[s - 4], 0, 0, 0);
      if (s >= 8) acc[s - 8] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1[s & 1], pb1, acc[s - 8], 0, 0, 0);
      nx = __builtin_amdgcn_mfma_f32_32x32x16_f16(kr[s & 1], s < NQR ? qreg[s] : qf[s & 1], nx,
                                                  0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    rawmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) rawmax = fmaxf(rawmax, nx[i]);
    // half-tile u + 2 (issued one iteration earlier) must have landed; this
    // iteration's load may stay in flight.  Then every wave's loads are
    // visible and every read of stage u % 4 is done before it is refilled.
    if (u + kMlaStages - 1 < nh) {
#define CA_MLA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (0 << 8) | (((n) >> 4) << 14))
      CA_MLA_WAIT_VM(NLD);
    } else {
      CA_MLA_WAIT_VM(0);
#undef CA_MLA_WAIT_VM
    }
    block_sync();
  };

  if (nh > 0) {
#pragma unroll
    for (int j = 0; j < kMlaStages - 1; ++j)
      if (j < nh) issue(j);
    __builtin_amdgcn_s_waitcnt(0x3F70);     // vmcnt(0)
    block_sync();
    f32x16_t sa = f32x16_t{}, sb;
#pragma unroll
    for (int st = 0; st < NST; ++st)
      sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfrag(0, st), st < NQR ? qreg[st] : qlds(st),
                                                  sa, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) rawmax = fmaxf(rawmax, sa[i]);
    for (int u = 0; u < nh; u += kMlaStages) {
      step(u, std::integral_constant<int, 0>{}, sa, sb);
      if (u + 1 < nh) step(u + 1, std::integral_constant<int, 1>{}, sb, sa);
      if (u + 2 < nh) step(u + 2, std::integral_constant<int, 2>{}, sa, sb);
      if (u + 3 < nh) step(u + 3, std::integral_constant<int, 3>{}, sb, sa);
    }
  }

  const float lt = mla_half_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // First-order correction of the LSE for the fp16 rounding of the absorbed
  // query: with q = fp16(q) + dq, ln sum_t exp(scale (q . kv_t)) =
  // LSE(fp16(q)) + scale dq . kbar + O(dq^2), kbar = sum_t w_t kv_t the
  // softmax-weighted mean latent row.  dq is zero on the position part (a
  // bf16 q^R is exact in fp16), and on the content part kbar is the latent
  // output o~ itself, so the term is a dot product of dq with this row's
  // outputs: the LSE then carries float32-grade error, not 2^-12 relative
  // error on every score.
  float corr = 0.f;
  if (qvalid) {
    float* ob = p.o + rglob * kMlaDC;
    const uint16_t* lo = p.q_lo ? p.q_lo + rglob * kMlaDC : nullptr;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * dt + 8 * r + 4 * hg;
        f32x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * r + e] * inv;
        *reinterpret_cast<f32x4_t*>(ob + d0) = v4;
        if (lo) {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(lo + d0);
          corr = fmaf(__uint_as_float(x[0] << 16), v4[0], corr);
          corr = fmaf(__uint_as_float(x[0] & 0xFFFF0000u), v4[1], corr);
          corr = fmaf(__uint_as_float(x[1] << 16), v4[2], corr);
          corr = fmaf(__uint_as_float(x[1] & 0xFFFF0000u), v4[3], corr);
        }
      }
  }
  corr = mla_half_sum(corr);
  if (qvalid && hg == 0) {
    const int n = rloc / p.H, h = rloc - (rloc / p.H) * p.H;
    p.lse[((int64_t)b * p.H + h) * p.Nq + n] =
        lt > 0.f ? fmaf(p.scale, corr, (m + log2f(lt)) * kLn2f) : -INFINITY;
  }
}

// float32 -> fp16 operand value: finite values beyond fp16's largest finite
// value (65504) saturate to +-65504 instead of becoming infinities (which
// would turn whole rows of scores into NaN); NaN stays NaN.  The conversion
// itself rounds to nearest even.
constexpr float kF16Max = 65504.f;
__device__ __forceinline__ float f16_saturate(float x) {
  return fabsf(x) > kF16Max ? copysignf(kF16Max, x) : x;
}

// bf16 -> fp16, round to nearest even, saturating; 8 values per thread
__global__ __launch_bounds__(256) void cast_bf16_f16_kernel(const uint16_t* __restrict__ x,
                                                            uint16_t* __restrict__ y, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4_t v = reinterpret_cast<const u32x4_t*>(x)[i];
  f32x8_t f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = f16_saturate(__uint_as_float(v[e] << 16));
    f[2 * e + 1] = f16_saturate(__uint_as_float(v[e] & 0xFFFF0000u));
  }
  reinterpret_cast<u32x4_t*>(y)[i] = __builtin_bit_cast(u32x4_t, __builtin_convertvector(f, f16x8_t));
}

// ---------------------------------------------------------------------------
// Per-head projection: out[r, h, j] = sum_i in[r, h, i] * W(h, i, j) for the
// rows r of one batch entry and head h, on the bf16 MFMA with float32
// accumulation.
//   W_IN_MAJOR: W stored [H, K, N] (W(h, i, j) = w[h][i][j]) -- the absorbed
//               query uses (W^K_h)^T, i.e. W^K stored [H, d_nope, d_c]
//   else:       W stored [H, N, K] (W(h, i, j) = w[h][j][i]) -- the value
//               up-projection W^V stored [H, d_v, d_c]
// The product is computed transposed, out^T = W^T in^T with
// v_mfma_f32_32x32x16_bf16: A = W^T (rows j, staged in LDS as bf16 [N][K + 8]
// once per workgroup), B = in^T straight from global memory (lane = row r,
// 8 consecutive i per lane), so each lane ends up holding 4 consecutive
// outputs j of its row per accumulator group.
// TIN: 0 = bf16 input (exact MFMA operand); 1 = float32 input, split as
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) and both halves multiplied
// (2^-17 relative residual, i.e. float32-grade products).
// TOUT: 0 = bf16, 1 = float32, 2 = fp16 (one round-to-nearest-even).
// Optional tail copy: input values [K, K + 32) of each row go to outputs
// [N, N + 32) in the output type (the query's position part next to its
// absorbed content part).
// One workgroup = 4 waves x 32 rows of one head.
// ---------------------------------------------------------------------------
constexpr int kProjWaves = 4;
constexpr int kProjRows = kProjWaves * 32;

struct ProjParams {
  const void* in;
  int64_t is_r, is_h;        // input row and head strides (elements); values contiguous
  const uint16_t* w;         // bf16 weights
  void* out;
  int64_t os_r, os_h;
  int rows, H, tail;
  uint16_t* lo;              // fp16 output only, optional: bf16(x - fp16(x)) of each output
  int64_t ls_r, ls_h;        // its row and head strides (elements)
};

template <int K, int N, bool W_IN_MAJOR, int TIN, int TOUT>
__global__ __launch_bounds__(kProjWaves * 64) void head_proj_kernel(const ProjParams p) {
  constexpr int WR = K + 8;                 // LDS row of W^T, bf16 elements (16 B pad)
  constexpr int NKS = K / 16;               // MFMA k-steps
  constexpr int NJB = N / 32;               // 32-row blocks of out^T
  static_assert(K % 16 == 0 && N % 32 == 0, "projection tiles");
  __shared__ __attribute__((aligned(16))) uint16_t ws[N * WR];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31, hg = lane >> 5;

  // W^T into LDS: ws[j * WR + i] = W(h, i, j)
  if (W_IN_MAJOR) {
    // two consecutive i and eight consecutive j per thread: two 16-byte
    // loads, then eight 4-byte stores of the pairs (W(i, j), W(i + 1, j)).
    // Consecutive lanes take consecutive i pairs, so the stores of a wave
    // for one j fill consecutive LDS words (distinct banks) instead of
    // 2-byte stores 8 rows apart landing in two banks.
    static_assert(K % 2 == 0 && WR % 2 == 0, "i pairs are 4-byte words");
    uint32_t* ws32 = reinterpret_cast<uint32_t*>(ws);
    for (int c = tid; c < K * N / 16; c += kProjWaves * 64) {
      const int ip = c % (K / 2), j0 = 8 * (c / (K / 2));
      const int i = 2 * ip;
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(p.w + ((int64_t)h * K + i) * N + j0);
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(p.w + ((int64_t)h * K + i + 1) * N + j0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ws32[((j0 + 2 * e) * WR + i) / 2] = (x0[e] & 0xFFFFu) | (x1[e] << 16);
        ws32[((j0 + 2 * e + 1) * WR + i) / 2] = (x0[e] >> 16) | (x1[e] & 0xFFFF0000u);
      }
    }
  } else {
    for (int c = tid; c < K * N / 8; c += kProjWaves * 64) {
      const int j = c / (K / 8), i0 = 8 * (c - j * (K / 8));
      *reinterpret_cast<u32x4_t*>(ws + j * WR + i0) =
          *reinterpret_cast<const u32x4_t*>(p.w + ((int64_t)h * N + j) * K + i0);
    }
  }

  // in^T operands of row r (lane column), values 16 ks + 8 hg .. + 8
  const int r = blockIdx.x * kProjRows + wave * 32 + col;
  const bool rvalid = r < p.rows;
  const int64_t ibase = (int64_t)r * p.is_r + (int64_t)h * p.is_h;
  bf16x8_t xb[NKS], xl[TIN == 1 ? NKS : 1];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int i0 = 16 * ks + 8 * hg;
    if (TIN == 0) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (rvalid) x = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p.in) + ibase + i0);
      xb[ks] = __builtin_bit_cast(bf16x8_t, x);
    } else {
      f32x8_t x = {};
      if (rvalid) {
        const float* ip = reinterpret_cast<const float*>(p.in) + ibase + i0;
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(ip);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(ip + 4);
        x = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      const bf16x8_t hi = __builtin_convertvector(x, bf16x8_t);
      xb[ks] = hi;
      xl[(TIN == 1) ? ks : 0] = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8_t), bf16x8_t);
    }
  }
  __syncthreads();

  f32x16_t acc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) acc[jb] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ws + (32 * jb + col) * WR + 16 * ks + 8 * hg);
      acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb[ks], acc[jb], 0, 0, 0);
      if (TIN == 1)
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xl[(TIN == 1) ? ks : 0], acc[jb], 0, 0, 0);
    }
  }
  if (!rvalid) return;

  // out^T block jb, register 4 g + e = output j = 32 jb + 8 g + 4 hg + e of row r
  const int64_t obase = (int64_t)r * p.os_r + (int64_t)h * p.os_h;
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
  typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j0 = 32 * jb + 8 * g + 4 * hg;
      const f32x4_t v = {acc[jb][4 * g], acc[jb][4 * g + 1], acc[jb][4 * g + 2], acc[jb][4 * g + 3]};
      if (TOUT == 1) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.out) + obase + j0) = v;
      } else if (TOUT == 2) {
        f32x4_t vs;
#pragma unroll
        for (int e = 0; e < 4; ++e) vs[e] = f16_saturate(v[e]);
        const f16x4_t h4 = __builtin_convertvector(vs, f16x4_t);
        *reinterpret_cast<f16x4_t*>(reinterpret_cast<_Float16*>(p.out) + obase + j0) = h4;
        if (p.lo) {
          // the rounding residual, exact in float32, kept to bf16 precision
          const f32x4_t res = v - __builtin_convertvector(h4, f32x4_t);
          *reinterpret_cast<bf16x4_t*>(reinterpret_cast<__bf16*>(p.lo) +
                                       (int64_t)r * p.ls_r + (int64_t)h * p.ls_h + j0) =
              __builtin_convertvector(res, bf16x4_t);
        }
      } else
        *reinterpret_cast<bf16x4_t*>(reinterpret_cast<__bf16*>(p.out) + obase + j0) =
            __builtin_convertvector(v, bf16x4_t);
    }
  // tail copy: lane half hg moves values K + 16 hg .. + 16 (bf16 input only)
  if (TIN == 0 && p.tail == 32) {
    const uint16_t* tp = reinterpret_cast<const uint16_t*>(p.in) + ibase + K + 16 * hg;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(tp + 8 * c);
      const f32x8_t f = __builtin_convertvector(__builtin_bit_cast(bf16x8_t, x), f32x8_t);
      const int64_t o = obase + N + 16 * hg + 8 * c;
      if (TOUT == 2) {
        typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_o;
        f32x8_t fs;
#pragma unroll
        for (int e = 0; e < 8; ++e) fs[e] = f16_saturate(f[e]);
        *reinterpret_cast<f16x8_o*>(reinterpret_cast<_Float16*>(p.out) + o) = __builtin_convertvector(fs, f16x8_o);
      } else if (TOUT == 1) {
        *reinterpret_cast<f32x8_t*>(reinterpret_cast<float*>(p.out) + o) = f;
      } else {
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(p.out) + o) = x;
      }
    }
  }
}

}  // namespace

// Absorbed query: q_lat[b, n, h, :] = [(W^K_h)^T q[b, n, h, :96] ; q[b, n, h, 96:128]]
// (fp16), from bf16 q [B, Nq, H, 128] with element strides (qs_b, qs_n, qs_h)
// and bf16 W^K [H, 96, 192].
hipError_t launch_mla_absorb(const uint16_t* q, int B, int Nq, int H, const int64_t* qs,
                             const uint16_t* w_uk, uint16_t* q_lat, uint16_t* q_lat_lo,
                             hipStream_t stream) {
  for (int b = 0; b < B; ++b) {
    ProjParams p{};
    p.in = q + b * qs[0];
    p.is_r = qs[1]; p.is_h = qs[2];
    p.w = w_uk;
    p.out = q_lat + (int64_t)b * Nq * H * kMlaDK;
    p.os_r = (int64_t)H * kMlaDK; p.os_h = kMlaDK;
    p.rows = Nq; p.H = H; p.tail = kMlaDR;
    p.lo = q_lat_lo ? q_lat_lo + (int64_t)b * Nq * H * kMlaDC : nullptr;
    p.ls_r = (int64_t)H * kMlaDC; p.ls_h = kMlaDC;
    const dim3 grid((Nq + kProjRows - 1) / kProjRows, H);
    if (Nq > 0 && H > 0)
      hipLaunchKernelGGL((head_proj_kernel<96, kMlaDC, true, 0, 2>), grid, dim3(kProjWaves * 64), 0,
                         stream, p);
  }
  return hipGetLastError();
}

// Output: o[b, n, h, :] = W^V_h o_lat[b, n, h, :] from float32 o_lat
// [B, Nq, H, 192] and bf16 W^V [H, 128, 192]; o bf16 or float32 with element
// strides (os_b, os_n, os_h).
hipError_t launch_mla_up(const float* o_lat, int B, int Nq, int H, const uint16_t* w_uv,
                         void* o, bool o_f32, const int64_t* os, hipStream_t stream) {
  for (int b = 0; b < B; ++b) {
    ProjParams p{};
    p.in = o_lat + (int64_t)b * Nq * H * kMlaDC;
    p.is_r = (int64_t)H * kMlaDC; p.is_h = kMlaDC;
    p.w = w_uv;
    p.out = o_f32 ? static_cast<void*>(static_cast<float*>(o) + b * os[0])
                  : static_cast<void*>(static_cast<uint16_t*>(o) + b * os[0]);
    p.os_r = os[1]; p.os_h = os[2];
    p.rows = Nq; p.H = H; p.tail = 0;
    const dim3 grid((Nq + kProjRows - 1) / kProjRows, H);
    if (Nq == 0 || H == 0) continue;
    if (o_f32)
      hipLaunchKernelGGL((head_proj_kernel<kMlaDC, 128, false, 1, 1>), grid, dim3(kProjWaves * 64), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((head_proj_kernel<kMlaDC, 128, false, 1, 0>), grid, dim3(kProjWaves * 64), 0,
                         stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_cast_bf16_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 > 0)
    hipLaunchKernelGGL(cast_bf16_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                       stream, x, y, n8);
  return hipGetLastError();
}

hipError_t launch_mla_attn(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* kv,
                           int64_t kv_bs, int64_t kv_rs, int B, int Nq, int H, int Nkv,
                           float scale, float* o_lat, float* lse, hipStream_t stream) {
  MlaParams p{};
  p.q = q_lat; p.q_lo = q_lat_lo; p.kv = kv; p.kv_bs = kv_bs; p.kv_rs = kv_rs;
  p.scale = scale;
  p.o = o_lat; p.lse = lse;
  p.B = B; p.Nq = Nq; p.H = H; p.Nkv = Nkv;
  p.rows_per_b = Nq * H;
  p.wg_per_b = (p.rows_per_b + kMlaNW * 32 - 1) / (kMlaNW * 32);
  p.scale_log2 = scale * 1.4426950408889634f;
  const int grid = B * p.wg_per_b;
  if (grid > 0)
    hipLaunchKernelGGL(mla_attn_kernel, dim3(grid), dim3(kMlaNW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace chunkattn
