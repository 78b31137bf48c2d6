// Internal declarations shared by the chunkattn HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace chunkattn {

// Vector types used with the gfx950 MFMA builtins and 16-byte memory ops.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) float f32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// Key-set modes of the attention kernel.  MODE_RANGE: each head attends to a
// contiguous token range, either all Nkv tokens of the dense cache or its span
// [cu[bh], cu[bh+1]) of the flat ragged buffers.  MODE_BLOCKS: each query
// block attends to the blocks listed in its CSR row.
enum Mode { MODE_RANGE = 0, MODE_BLOCKS = 1 };

constexpr int kMaxHeadsPerLaunch = 1024;
constexpr int kMaxSchedHeads = 256;   // heads of one launch under the balanced schedule
constexpr int kTileKeys = 64;         // keys per KV tile (and max KV block size)
constexpr int kRangeRows = 256;       // query rows per workgroup in range mode (8 waves)
constexpr uint16_t kFlatHead = 0x8000;  // heads[] flag: the head reads the flat buffers

// Kernel arguments of the fused attention kernel (passed by value).
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int64_t qs_b, qs_n, qs_h;
  int64_t ks_b, ks_n, ks_h;   // varlen: ks_n = flat row stride, ks_b = ks_h = 0
  int64_t os_b, os_n, os_h;
  const float* o_init;        // optional starting state (float32 O and LSE)
  const float* lse_init;
  int64_t is_b, is_n, is_h;
  int B, H, Nq, Nkv;
  float scale_log2;           // softmax scale * log2(e)
  // dual output (block mode): after the first `snap` list entries (-1: none)
  // the state is also written to o_snap (dtype of o) and lse_snap
  int snap;
  void* o_snap;
  float* lse_snap;
  int64_t ss_b, ss_n, ss_h;
  // block-list mode
  const int32_t* indptr;
  const int32_t* indices;
  int nnz;                    // entries of indices; row spans are clamped to it
  int kv_block, kv_seg, kv_bps, nkb;
  uint32_t kv_bps_magic;      // floor(2^32 / kv_bps): id / kv_bps by multiply-high
  int q_block, q_seg, q_bps, nqb, q_sub;
  // flat ragged buffers (range mode): head bh owns rows [cu[bh], cu[bh+1])
  const uint16_t* kf;
  const uint16_t* vf;
  int64_t kfs_n;              // row stride of the flat buffers, elements
  const int32_t* cu;
  int total_kv;
  int all_flat;               // use_list == 0: every head reads the flat buffers
  // work decomposition
  int n_qtiles;               // query tiles per head (range mode)
  int n_items;                // logical work items of this launch
  int n_heads;                // heads covered by this launch
  int use_list;               // heads[] maps launch-local head -> b*H + h (| kFlatHead)
  // Balanced schedule (range mode, sched = 1): the launch's work is
  // n_units = n_qtiles * tprefix[n_heads] units of one (query tile, key tile)
  // pair, ordered head, query tile, key tile; head i has tprefix[i+1] -
  // tprefix[i] >= 1 key tiles.  The units are dealt out by cost: every query
  // tile is preceded by seg_cost virtual units, the fixed cost of a segment
  // (loading the query tile, filling and draining the tile ring, writing the
  // state) in key-tile units, so the n_vunits = n_qtiles * (tprefix[n_heads]
  // + seg_cost * n_heads) virtual units are split evenly: workgroup g (of
  // n_wgs) takes virtual units [g*n_vunits/n_wgs, (g+1)*n_vunits/n_wgs) and
  // with them the real units they cover (sched_real / sched_virtual).  A
  // query tile whose units fall to more than one workgroup is written as
  // float32 partials (O / l, LSE) into ws: slot 2g holds a workgroup's first
  // segment, slot 2g+1 its last; each slot is kRangeRows x d floats of O
  // followed by kRangeRows LSE values.
  int sched;
  int n_units;
  int n_vunits;
  int seg_cost;
  int n_wgs;
  float* ws;
  int32_t tprefix[kMaxSchedHeads + 1];
  uint16_t heads[kMaxHeadsPerLaunch];
};

// Kernel arguments of the one-pass PBSA kernel (pbsa.hip): query block qb of
// head bh = b*H + h attends to the blocks of shared CSR row bh and of local
// CSR row bh * nqb + qb; one workgroup per four query blocks of a head.
struct PbsaParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int64_t qs_b, qs_n, qs_h;
  int64_t ks_b, ks_n, ks_h;
  int64_t os_b, os_n, os_h;
  int B, H, Nq, Nkv;
  float scale_log2;           // softmax scale * log2(e)
  const int32_t* sh_ptr;      // shared lists: row bh
  const int32_t* sh_idx;
  int sh_nnz;
  const int32_t* lo_ptr;      // local lists: row bh * nqb + qb
  const int32_t* lo_idx;
  int lo_nnz;
  int kv_block, kv_seg, kv_bps, nkb;
  uint32_t kv_bps_magic;      // floor(2^32 / kv_bps)
  int q_block, q_seg, q_bps, nqb;
  int groups;                 // workgroups per head: ceil(nqb / 4)
  int n_items;                // heads of this launch * groups
  int use_list;               // 0: head i of the launch is b*H + h = i; 1: heads[i]
  uint16_t heads[kMaxHeadsPerLaunch];
};

// First unit of workgroup g under the balanced schedule, and the workgroup
// that owns unit u (exact integer forms: g_of_unit(u) = g iff
// unit_begin(g) <= u < unit_begin(g + 1), for 1 <= n_wgs <= n_units).
__host__ __device__ __forceinline__ int unit_begin(int g, int n_units, int n_wgs) {
  return (int)(((int64_t)g * n_units) / n_wgs);
}
__host__ __device__ __forceinline__ int g_of_unit(int u, int n_units, int n_wgs) {
  return (int)((((int64_t)u + 1) * n_wgs - 1) / n_units);
}

// Real unit at virtual unit v of the balanced schedule: the virtual units of
// a query tile are seg_cost leading ones (mapped to the tile's first unit)
// followed by one per unit; v >= n_vunits maps to n_units.  Monotone, and
// sched_real(v) <= u iff v <= sched_virtual(u), so workgroup g owns unit u
// iff g_of_unit(sched_virtual(u), n_vunits, n_wgs) = g.  A workgroup's range
// is never empty when n_vunits / n_wgs > seg_cost.
__host__ __device__ inline int sched_real(const AttnParams& p, int v) {
  if (v >= p.n_vunits) return p.n_units;
  const int S = p.seg_cost;
  int lo = 0, hi = p.n_heads - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p.n_qtiles * (p.tprefix[mid + 1] + S * (mid + 1)) <= v) lo = mid + 1; else hi = mid;
  }
  const int nt = p.tprefix[lo + 1] - p.tprefix[lo];
  const int rel = v - p.n_qtiles * (p.tprefix[lo] + S * lo);
  const int qt = rel / (nt + S);
  const int o = rel - qt * (nt + S);
  return p.n_qtiles * p.tprefix[lo] + qt * nt + (o > S ? o - S : 0);
}
// Virtual unit of real unit u (0 <= u < n_units): the tile's leading
// seg_cost virtual units come before it.
__host__ __device__ inline int sched_virtual(const AttnParams& p, int u) {
  const int S = p.seg_cost;
  int lo = 0, hi = p.n_heads - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p.n_qtiles * p.tprefix[mid + 1] <= u) lo = mid + 1; else hi = mid;
  }
  const int nt = p.tprefix[lo + 1] - p.tprefix[lo];
  const int rel = u - p.n_qtiles * p.tprefix[lo];
  const int qt = rel / nt;
  return p.n_qtiles * (p.tprefix[lo] + S * lo) + qt * (nt + S) + S + (rel - qt * nt);
}

// Launchers implemented in attn_fwd.hip / select.hip / merge.hip.
hipError_t launch_attention(int mode, int d, int nwaves, bool out_f32,
                            const AttnParams& p, hipStream_t stream);
// The one-pass PBSA kernel (pbsa.hip), d = 64 or 128.
hipError_t launch_pbsa(int d, bool out_f32, const PbsaParams& p, hipStream_t stream);
// Combines the float32 partials of the query tiles the balanced schedule
// split across workgroups (runs after launch_attention on the same stream).
hipError_t launch_split_merge(int d, bool out_f32, const AttnParams& p, hipStream_t stream);
// Workgroups of the range-mode attention kernel resident on the whole device
// at once (0 on failure).
int attention_slots(int d);
// With x2 non-null, the block means of a second tensor of the same shape
// and tiling (strides xs2) go to out2 in the same launch; out_total is the
// first tensor's.
hipError_t launch_block_mean(const uint16_t* x, int B, int N, int H, int d,
                             const int64_t* xs, int block, int seg, int bps, int nb,
                             float* out, float* out_total, hipStream_t stream,
                             const uint16_t* x2 = nullptr, const int64_t* xs2 = nullptr,
                             float* out2 = nullptr);
// One selection of a batched launch (fields as launch_score_topk's).
struct TopkJobDesc {
  const float* qm;
  const float* km;
  int B, H, NQB, NKB, d, cand_begin, cand_count, K;
  int prefix_begin, prefix_count, id_offset;
  int32_t* out_idx;
  float* out_score;
  int32_t* indptr;
  int32_t* indices;
  // optional: the query (NQB = 1) is the chunk mean of these query block
  // means [B*H, cm_nb, d] (tiling cm_block / cm_seg over cm_N tokens),
  // computed in the launch and written to qm
  const float* cm_src;
  int cm_N, cm_block, cm_seg, cm_nb;
};
// Up to 4 independent selections in one launch of 512-thread workgroups.
hipError_t launch_score_topk_batch(const TopkJobDesc* jobs, int n_jobs, hipStream_t stream);
// With indptr non-null the kernel also writes each row's block list: the
// prefix range [prefix_begin, prefix_begin + prefix_count) followed by
// id_offset + the selected ids (W = prefix_count + K entries per row).
hipError_t launch_score_topk(const float* qm, const float* km, int B, int H, int NQB,
                             int NKB, int d, int cand_begin, int cand_count, int K,
                             int32_t* out_idx, float* out_score, hipStream_t stream,
                             int32_t* indptr = nullptr, int32_t* indices = nullptr,
                             int prefix_begin = 0, int prefix_count = 0, int id_offset = 0);
hipError_t launch_persistent_update(const float* qm, const float* km, int B, int H, int NKB,
                                   int d, const int32_t* pers, int C_in, int evict_begin,
                                   int evict_count, int C, int32_t* out, float* out_score,
                                   hipStream_t stream);
hipError_t launch_pack_ragged(const uint16_t* k, const uint16_t* v, int B, int N, int H, int d,
                              const int64_t* ks, int T, const int32_t* frame_ptr,
                              int total_frames, const int32_t* src, uint16_t* kf, uint16_t* vf,
                              int64_t fs, int32_t* cu, hipStream_t stream);
hipError_t launch_mla_absorb(const uint16_t* q, int B, int Nq, int H, const int64_t* qs,
                             const uint16_t* w_uk, uint16_t* q_lat, uint16_t* q_lat_lo,
                             hipStream_t stream);
hipError_t launch_mla_attn(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* kv,
                           int64_t kv_bs, int64_t kv_rs, int B, int Nq, int H, int Nkv,
                           float scale, float* o_lat, float* lse, hipStream_t stream);
hipError_t launch_mla_up(const float* o_lat, int B, int Nq, int H, const uint16_t* w_uv,
                         void* o, bool o_f32, const int64_t* os, hipStream_t stream);
hipError_t launch_cast_bf16_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream);
hipError_t launch_build_kv_index(int rows, int sink_begin, int sink_count,
                                 const int32_t* persistent, int C, int NQB,
                                 const int32_t* topk, int K, int topk_offset,
                                 int32_t* indptr, int32_t* indices, hipStream_t stream);
hipError_t launch_lse_merge(const void* o1, const float* l1, const void* o2,
                            const float* l2, int in_f32, void* o, float* l, int out_f32,
                            int B, int H, int N, int d, const int64_t* s1,
                            const int64_t* s2, const int64_t* so, hipStream_t stream);

// Map a hardware block index to a logical work item so that consecutive
// logical items run on the same XCD (workgroups are dispatched to the 8 XCDs
// round-robin; each XCD has its own L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd;
  const int rem = nblocks % kXcd;
  const int x = bid % kXcd;
  const int j = bid / kXcd;
  return x * per + (x < rem ? x : rem) + j;
}

// id / div for 0 <= id < 2^31 with magic = floor(2^32 / div): the
// multiply-high estimate is low by at most one, fixed by one correction.
__host__ __device__ __forceinline__ int div_magic(int id, int div, uint32_t magic) {
  int q = (int)(((uint64_t)(uint32_t)id * magic) >> 32);
  if (id - q * div >= div) ++q;
  return q;
}

// Start and length of block `id` of the frame-aligned tiling of n tokens
// (segments of `seg` tokens, `bps` blocks of `block` tokens per segment).
__host__ __device__ __forceinline__ void block_span(int id, int n, int block, int seg,
                                                    int bps, int& start, int& len,
                                                    uint32_t magic = 0) {
  const int s = magic ? div_magic(id, bps, magic) : id / bps;
  const int j = id - s * bps;
  const int seg_start = s * seg;
  int seg_len = n - seg_start;
  seg_len = seg_len < seg ? seg_len : seg;
  start = seg_start + j * block;
  const int rest = seg_len - j * block;
  len = rest < block ? rest : block;
  if (len < 0) len = 0;
}

}  // namespace chunkattn
