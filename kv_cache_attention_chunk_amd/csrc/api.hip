// C ABI of chunkattn: argument checks, work decomposition and kernel dispatch.
// Every check runs on the host before any device call; nothing here
// synchronises or allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include "chunkattn.h"
#include "common.h"

using namespace chunkattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return CA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-side block count of the frame-aligned tiling.
int num_blocks(int n, int block, int seg) {
  if (n < 0 || block <= 0 || seg <= 0) return -1;
  const int bps = (seg + block - 1) / block;
  const int full = n / seg;
  const int rest = n - full * seg;
  return full * bps + (rest + block - 1) / block;
}

int check_device() {
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0) return fail(CA_ENODEV, "no HIP device visible");
  return CA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Strides of a bf16/f32 [B, N, H, d] tensor: non-negative, 16-byte row starts.
int check_strides(const char* name, const int64_t* s, int elem_align) {
  if (!s) return fail(CA_EINVAL, "%s_strides is NULL", name);
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(CA_EINVAL, "%s_strides[%d] < 0", name, i);
    if (s[i] % elem_align) return fail(CA_EINVAL, "%s_strides[%d] not a multiple of %d", name, i, elem_align);
  }
  return CA_OK;
}

struct Common {
  int B, H, Nq, d;
  const void* q;
  const int64_t* qs;
  const int64_t* os;
  void* o;
  int o_dtype;
  float* lse;
  float scale;
};

int check_common(const Common& c) {
  if (c.B < 0 || c.H < 0 || c.Nq < 0) return fail(CA_EINVAL, "negative size");
  if ((int64_t)c.B * c.H > 32767) return fail(CA_ERANGE, "B*H above 32767");
  if (c.d != 64 && c.d != 128) return fail(CA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", c.d);
  if (c.o_dtype != CA_BF16 && c.o_dtype != CA_F32) return fail(CA_EUNSUPPORTED, "o_dtype %d", c.o_dtype);
  if (!c.q || !c.o || !c.lse) return fail(CA_EINVAL, "q, o and lse must be non-NULL");
  if (!aligned16(c.q) || !aligned16(c.o) || !aligned16(c.lse)) return fail(CA_EINVAL, "q, o, lse must be 16-byte aligned");
  if (int r = check_strides("q", c.qs, 8)) return r;
  if (int r = check_strides("o", c.os, c.o_dtype == CA_BF16 ? 8 : 4)) return r;
  if (!(std::isfinite(c.scale) && c.scale > 0.f)) return fail(CA_EINVAL, "scale must be finite and > 0");
  return CA_OK;
}

void fill_common(AttnParams& p, const Common& c) {
  p.snap = -1;
  p.q = static_cast<const uint16_t*>(c.q);
  p.o = c.o;
  p.lse = c.lse;
  p.qs_b = c.qs[0]; p.qs_n = c.qs[1]; p.qs_h = c.qs[2];
  p.os_b = c.os[0]; p.os_n = c.os[1]; p.os_h = c.os[2];
  p.B = c.B; p.H = c.H; p.Nq = c.Nq;
  p.scale_log2 = c.scale * 1.4426950408889634f;
}

constexpr int kDenseWaves = 8;            // 256 query rows per workgroup (range mode)
constexpr int kMinUnitsPerWg = 8;         // balanced schedule: key tiles per workgroup, at least
// Balanced schedule: the fixed cost of a segment in key-tile units.  Measured
// on the Wan shapes with per-workgroup timestamps: a segment takes about
// 15 us beyond its ~1.85 us per key tile (loading its query tile, filling and
// draining the tile ring, writing its state), about 8 tiles' worth.
constexpr int kSegmentCost = 8;

// Block mode: one workgroup per query block (or row slice of one), over a
// list of heads (all heads when `heads` is empty), in launches of at most
// kMaxHeadsPerLaunch heads.
int launch_blocks(const Common& c, AttnParams& p, const std::vector<int>& heads,
                  hipStream_t stream) {
  const bool all = heads.empty();
  const int nh = all ? c.B * c.H : (int)heads.size();
  const int maxq = std::min(std::min(p.q_block, p.q_seg), std::max(c.Nq, 1));
  const int nwaves = maxq <= 64 ? 2 : (maxq <= 128 ? 4 : 8);
  p.q_sub = (maxq + nwaves * 32 - 1) / (nwaves * 32);
  for (int h0 = 0; h0 < nh; h0 += kMaxHeadsPerLaunch) {
    const int n = std::min(kMaxHeadsPerLaunch, nh - h0);
    p.n_heads = n;
    p.use_list = (all && h0 == 0) ? 0 : 1;
    if (p.use_list)
      for (int i = 0; i < n; ++i) p.heads[i] = (uint16_t)(all ? h0 + i : heads[h0 + i]);
    const int64_t items = (int64_t)p.nqb * p.q_sub * n;
    if (items > 0x7FFFFFFF) return fail(CA_ERANGE, "too many work items");
    p.n_items = (int)items;
    const hipError_t e = launch_attention(MODE_BLOCKS, c.d, nwaves, c.o_dtype == CA_F32, p, stream);
    if (e != hipSuccess) return launched(e, "chunk attention launch");
  }
  return ok();
}

// Bytes of the balanced schedule's partials for `slots` workgroups.
size_t workspace_bytes(int slots, int d) {
  return (size_t)2 * slots * kRangeRows * (d + 1) * sizeof(float);
}

// Range mode over a list of head words (b*H + h, | kFlatHead for heads that
// read the flat buffers).  tiles[i] (host) is head i's key-tile count when
// known (empty vector: unknown).  With a workspace and known tile counts a
// launch takes the balanced schedule when that shortens it by more than a
// fifth: the plain grid runs one workgroup per (head, query tile), so its
// length is set by the longest head and by how many rounds of workgroups the
// device needs; the balanced grid gives every resident workgroup the same
// number of key tiles.  The margin covers the merge pass and the balanced
// grid's second, phase-shifted stream over each head's keys (roughly double
// the L2 fill traffic), and on a uniform cache the gain from filling idle CUs
// is returned as a lower clock under the power limit (measured: the dense
// Wan layer runs no faster balanced).
int launch_range(const Common& c, AttnParams& p, const std::vector<uint16_t>& words,
                 const std::vector<int>& tiles, int split, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  const int nh = (int)words.size();
  p.n_qtiles = (c.Nq + kRangeRows - 1) / kRangeRows;
  const int slots = (ws && split != CA_SPLIT_NEVER) ? attention_slots(c.d) : 0;
  for (int h0 = 0; h0 < nh;) {
    int n = std::min(kMaxHeadsPerLaunch, nh - h0);
    p.sched = 0;
    if (slots > 0 && !tiles.empty() && !p.o_init) {
      const int ns = std::min(n, kMaxSchedHeads);
      int64_t tsum = 0;
      int max_nt = 0;
      for (int i = 0; i < ns; ++i) {
        tsum += std::max(1, tiles[h0 + i]);
        max_nt = std::max(max_nt, tiles[h0 + i]);
      }
      const int64_t units = tsum * p.n_qtiles;
      const int64_t items = (int64_t)ns * p.n_qtiles;
      const int64_t vunits = units + items * kSegmentCost;
      // (every workgroup's virtual range longer than kSegmentCost: no empty range)
      const int64_t g = std::min<int64_t>(std::min<int64_t>(slots, units / kMinUnitsPerWg),
                                          vunits / (kSegmentCost + 1));
      const int64_t est_plain = (items + slots - 1) / slots * (int64_t)(max_nt + kSegmentCost);
      const int64_t est_bal = g > 0 ? (vunits + g - 1) / g + kSegmentCost + 2 : INT64_MAX;
      // (the merge grid has 32 workgroups per query tile; keep it in range)
      const bool worth = split == CA_SPLIT_ALWAYS || est_bal * 5 < est_plain * 4;
      if (vunits <= 0x7FFFFFFF && items * 32 <= 0x7FFFFFFF && g >= 1 && est_plain >= 64 && worth) {
        if (ws_bytes < workspace_bytes((int)g, c.d))
          return fail(CA_EINVAL, "workspace of %zu bytes is smaller than the %zu required",
                      ws_bytes, workspace_bytes((int)g, c.d));
        n = ns;
        p.sched = 1;
        p.n_units = (int)units;
        p.n_vunits = (int)vunits;
        p.seg_cost = kSegmentCost;
        p.n_wgs = (int)g;
        p.ws = static_cast<float*>(ws);
        p.tprefix[0] = 0;
        for (int i = 0; i < ns; ++i) p.tprefix[i + 1] = p.tprefix[i] + std::max(1, tiles[h0 + i]);
      }
    }
    if ((int64_t)n * p.n_qtiles > 0x7FFFFFFF) return fail(CA_ERANGE, "too many work items");
    p.n_heads = n;
    p.use_list = 1;
    for (int i = 0; i < n; ++i) p.heads[i] = words[h0 + i];
    p.n_items = n * p.n_qtiles;
    hipError_t e = launch_attention(MODE_RANGE, c.d, kDenseWaves, c.o_dtype == CA_F32, p, stream);
    if (e != hipSuccess) return launched(e, "chunk attention launch");
    if (p.sched) {
      e = launch_split_merge(c.d, c.o_dtype == CA_F32, p, stream);
      if (e != hipSuccess) return launched(e, "split merge launch");
    }
    h0 += n;
  }
  return ok();
}

int check_workspace(int split, const void* ws, size_t ws_bytes) {
  if (split < CA_SPLIT_AUTO || split > CA_SPLIT_ALWAYS) return fail(CA_EINVAL, "split policy %d", split);
  if (ws && !aligned16(ws)) return fail(CA_EINVAL, "workspace must be 16-byte aligned");
  if (!ws && ws_bytes) return fail(CA_EINVAL, "workspace_bytes given without a workspace");
  return CA_OK;
}

int check_csr(const int32_t* indptr, const int32_t* indices, int nnz, int kv_block, int kv_seg,
              int q_block, int q_seg) {
  if (!indptr || !indices) return fail(CA_EINVAL, "kv_indptr and kv_indices must both be given");
  if (nnz < 0) return fail(CA_EINVAL, "kv_nnz < 0");
  if (kv_block < 1 || kv_block > kTileKeys) return fail(CA_ERANGE, "kv_block %d outside 1..%d", kv_block, kTileKeys);
  if (kv_seg < 1 || q_block < 1 || q_seg < 1) return fail(CA_EINVAL, "tiling sizes must be >= 1");
  return CA_OK;
}

void fill_blocks(AttnParams& p, int Nq, int Nkv, const int32_t* indptr, const int32_t* indices,
                 int nnz, int kv_block, int kv_seg, int q_block, int q_seg) {
  p.indptr = indptr;
  p.indices = indices;
  p.nnz = nnz;
  p.kv_block = kv_block;
  p.kv_seg = kv_seg;
  p.kv_bps = (kv_seg + kv_block - 1) / kv_block;
  p.kv_bps_magic = (uint32_t)((((uint64_t)1) << 32) / (uint64_t)p.kv_bps);
  p.nkb = num_blocks(Nkv, kv_block, kv_seg);
  p.q_block = q_block;
  p.q_seg = q_seg;
  p.q_bps = (q_seg + q_block - 1) / q_block;
  p.nqb = num_blocks(Nq, q_block, q_seg);
}

// Launch arguments of the one-pass PBSA kernel (checked by the caller).
PbsaParams pbsa_params(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nkv,
                       const int64_t* qs, const int64_t* kvs, const int64_t* os,
                       const int32_t* sh_ptr, const int32_t* sh_idx, int sh_nnz,
                       const int32_t* lo_ptr, const int32_t* lo_idx, int lo_nnz, int kv_block,
                       int kv_seg, int q_block, int q_seg, float scale, void* o, float* lse) {
  PbsaParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.qs_b = qs[0]; p.qs_n = qs[1]; p.qs_h = qs[2];
  p.ks_b = kvs[0]; p.ks_n = kvs[1]; p.ks_h = kvs[2];
  p.os_b = os[0]; p.os_n = os[1]; p.os_h = os[2];
  p.B = B; p.H = H; p.Nq = Nq; p.Nkv = Nkv;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.sh_ptr = sh_ptr; p.sh_idx = sh_idx; p.sh_nnz = sh_nnz;
  p.lo_ptr = lo_ptr; p.lo_idx = lo_idx; p.lo_nnz = lo_nnz;
  p.kv_block = kv_block;
  p.kv_seg = kv_seg;
  p.kv_bps = (kv_seg + kv_block - 1) / kv_block;
  p.kv_bps_magic = (uint32_t)((((uint64_t)1) << 32) / (uint64_t)p.kv_bps);
  p.nkb = num_blocks(Nkv, kv_block, kv_seg);
  p.q_block = q_block;
  p.q_seg = q_seg;
  p.q_bps = (q_seg + q_block - 1) / q_block;
  p.nqb = num_blocks(Nq, q_block, q_seg);
  p.groups = (p.nqb + 3) / 4;
  p.n_items = B * H * p.groups;
  return p;
}

std::vector<int> longest_first(const int32_t* cu_host, const std::vector<int>& heads) {
  std::vector<int> order = heads;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return (cu_host[a + 1] - cu_host[a]) > (cu_host[b + 1] - cu_host[b]);
  });
  return order;
}

}  // namespace

extern "C" {

int ca_abi_version(void) { return CA_ABI_VERSION; }

const char* ca_status_str(int status) {
  switch (status) {
    case CA_OK: return "ok";
    case CA_EINVAL: return "invalid argument";
    case CA_EUNSUPPORTED: return "unsupported configuration";
    case CA_ERANGE: return "value out of range";
    case CA_ENODEV: return "no HIP device";
    case CA_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* ca_last_error(void) { return g_last_error.c_str(); }

int ca_num_blocks(int n_tokens, int block_size, int seg_len) {
  return num_blocks(n_tokens, block_size, seg_len);
}

size_t ca_attn_workspace_bytes(int d) {
  if (d != 64 && d != 128) return 0;
  if (check_device() != CA_OK) return 0;
  return workspace_bytes(attention_slots(d), d);
}

int ca_chunk_attn_fwd(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nkv,
                      int d, const int64_t* q_strides, const int64_t* kv_strides,
                      const int64_t* o_strides, const int32_t* kv_indptr,
                      const int32_t* kv_indices, int kv_nnz, int kv_block, int kv_seg,
                      int q_block, int q_seg, float scale, const float* o_init,
                      const int64_t* o_init_strides, const float* lse_init, void* o,
                      int o_dtype, float* lse, int split, void* workspace,
                      size_t workspace_bytes, void* stream) {
  Common c{B, H, Nq, d, q, q_strides, o_strides, o, o_dtype, lse, scale};
  if (int r = check_common(c)) return r;
  if (int r = check_workspace(split, workspace, workspace_bytes)) return r;
  if ((o_init == nullptr) != (lse_init == nullptr))
    return fail(CA_EINVAL, "o_init and lse_init must be given together");
  if (o_init) {
    if (!aligned16(o_init) || !aligned16(lse_init)) return fail(CA_EINVAL, "o_init, lse_init must be 16-byte aligned");
    if (int r = check_strides("o_init", o_init_strides, 4)) return r;
    if (o == o_init && (o_dtype != CA_F32 || o_init_strides[0] != o_strides[0] ||
                        o_init_strides[1] != o_strides[1] || o_init_strides[2] != o_strides[2]))
      return fail(CA_EINVAL, "o aliases o_init with a different dtype or strides");
  }
  if (Nkv < 0) return fail(CA_EINVAL, "Nkv < 0");
  if (Nkv > 0 && (!k || !v)) return fail(CA_EINVAL, "k and v must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(CA_EINVAL, "k, v must be 16-byte aligned");
  if (int r = check_strides("kv", kv_strides, 8)) return r;
  if (kv_strides[1] < d || kv_strides[1] > (1 << 23)) return fail(CA_ERANGE, "kv row stride outside [d, 2^23]");
  const bool blocks = kv_indptr || kv_indices;
  if (blocks) {
    if (int r = check_csr(kv_indptr, kv_indices, kv_nnz, kv_block, kv_seg, q_block, q_seg)) return r;
  }
  if (int r = check_device()) return r;
  if ((int64_t)B * H * Nq == 0) return ok();
  static thread_local AttnParams p;
  p = AttnParams{};
  fill_common(p, c);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.ks_b = kv_strides[0]; p.ks_n = kv_strides[1]; p.ks_h = kv_strides[2];
  p.Nkv = Nkv;
  if (o_init) {
    p.o_init = o_init;
    p.lse_init = lse_init;
    p.is_b = o_init_strides[0]; p.is_n = o_init_strides[1]; p.is_h = o_init_strides[2];
  }
  if (blocks) {
    fill_blocks(p, Nq, Nkv, kv_indptr, kv_indices, kv_nnz, kv_block, kv_seg, q_block, q_seg);
    return launch_blocks(c, p, {}, static_cast<hipStream_t>(stream));
  }
  std::vector<uint16_t> words(B * H);
  std::iota(words.begin(), words.end(), 0);
  const std::vector<int> tiles(Nkv > 0 ? B * H : 0, (Nkv + kTileKeys - 1) / kTileKeys);
  return launch_range(c, p, words, tiles, split, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream));
}

int ca_chunk_attn_pbsa_fwd(const void* q, const void* k, const void* v, int B, int H, int Nq,
                           int Nkv, int d, const int64_t* q_strides, const int64_t* kv_strides,
                           const int64_t* o_strides, const int32_t* shared_indptr,
                           const int32_t* shared_indices, int shared_nnz,
                           const int32_t* local_indptr, const int32_t* local_indices,
                           int local_nnz, int kv_block, int kv_seg, int q_block, int q_seg,
                           float scale, void* o, int o_dtype, float* lse, void* stream) {
  Common c{B, H, Nq, d, q, q_strides, o_strides, o, o_dtype, lse, scale};
  if (int r = check_common(c)) return r;
  if (Nkv < 0) return fail(CA_EINVAL, "Nkv < 0");
  if (Nkv > 0 && (!k || !v)) return fail(CA_EINVAL, "k and v must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(CA_EINVAL, "k, v must be 16-byte aligned");
  if (int r = check_strides("kv", kv_strides, 8)) return r;
  if (kv_strides[1] < d || kv_strides[1] > (1 << 23)) return fail(CA_ERANGE, "kv row stride outside [d, 2^23]");
  if (int r = check_csr(shared_indptr, shared_indices, shared_nnz, kv_block, kv_seg, q_block, q_seg)) return r;
  if (int r = check_csr(local_indptr, local_indices, local_nnz, kv_block, kv_seg, q_block, q_seg)) return r;
  if (q_block > 64) return fail(CA_ERANGE, "q_block %d above 64 (a query block is served by 64 rows)", q_block);
  if (int r = check_device()) return r;
  const int nqb = num_blocks(Nq, q_block, q_seg);
  if ((int64_t)B * H * ((nqb + 3) / 4) > 0x7FFFFFFF) return fail(CA_ERANGE, "too many work items");
  if ((int64_t)B * H * Nq == 0) return ok();
  const PbsaParams p = pbsa_params(q, k, v, B, H, Nq, Nkv, q_strides, kv_strides, o_strides,
                                   shared_indptr, shared_indices, shared_nnz, local_indptr,
                                   local_indices, local_nnz, kv_block, kv_seg, q_block, q_seg,
                                   scale, o, lse);
  return launched(launch_pbsa(d, o_dtype == CA_F32, p, static_cast<hipStream_t>(stream)),
                  "pbsa launch");
}

int ca_chunk_attn_dual_fwd(const void* q, const void* k, const void* v, int B, int H, int Nq,
                           int Nkv, int d, const int64_t* q_strides, const int64_t* kv_strides,
                           const int32_t* kv_indptr, const int32_t* kv_indices, int kv_nnz,
                           int kv_block, int kv_seg, int q_block, int q_seg, int local_count,
                           float scale, void* o_local, const int64_t* o_local_strides,
                           float* lse_local, void* o, const int64_t* o_strides, int o_dtype,
                           float* lse, void* stream) {
  Common c{B, H, Nq, d, q, q_strides, o_strides, o, o_dtype, lse, scale};
  if (int r = check_common(c)) return r;
  if (local_count < 0) return fail(CA_EINVAL, "local_count < 0");
  if (!o_local || !lse_local) return fail(CA_EINVAL, "o_local and lse_local must be non-NULL");
  if (!aligned16(o_local) || !aligned16(lse_local)) return fail(CA_EINVAL, "o_local, lse_local must be 16-byte aligned");
  if (int r = check_strides("o_local", o_local_strides, o_dtype == CA_BF16 ? 8 : 4)) return r;
  if (o_local == o || lse_local == lse) return fail(CA_EINVAL, "local and full outputs must not alias");
  if (Nkv < 0) return fail(CA_EINVAL, "Nkv < 0");
  if (Nkv > 0 && (!k || !v)) return fail(CA_EINVAL, "k and v must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(CA_EINVAL, "k, v must be 16-byte aligned");
  if (int r = check_strides("kv", kv_strides, 8)) return r;
  if (kv_strides[1] < d || kv_strides[1] > (1 << 23)) return fail(CA_ERANGE, "kv row stride outside [d, 2^23]");
  if (int r = check_csr(kv_indptr, kv_indices, kv_nnz, kv_block, kv_seg, q_block, q_seg)) return r;
  if (int r = check_device()) return r;
  if ((int64_t)B * H * Nq == 0) return ok();
  static thread_local AttnParams p;
  p = AttnParams{};
  fill_common(p, c);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.ks_b = kv_strides[0]; p.ks_n = kv_strides[1]; p.ks_h = kv_strides[2];
  p.Nkv = Nkv;
  p.snap = local_count;
  p.o_snap = o_local;
  p.lse_snap = lse_local;
  p.ss_b = o_local_strides[0]; p.ss_n = o_local_strides[1]; p.ss_h = o_local_strides[2];
  fill_blocks(p, Nq, Nkv, kv_indptr, kv_indices, kv_nnz, kv_block, kv_seg, q_block, q_seg);
  return launch_blocks(c, p, {}, static_cast<hipStream_t>(stream));
}

int ca_chunk_attn_varlen_fwd(const void* q, const void* k_flat, const void* v_flat,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int total_kv, int B, int H, int Nq, int d, const int64_t* q_strides,
                             int64_t kv_row_stride, const int64_t* o_strides, float scale,
                             void* o, int o_dtype, float* lse, int split, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Common c{B, H, Nq, d, q, q_strides, o_strides, o, o_dtype, lse, scale};
  if (int r = check_common(c)) return r;
  if (int r = check_workspace(split, workspace, workspace_bytes)) return r;
  if (!cu_seqlens) return fail(CA_EINVAL, "cu_seqlens must be non-NULL");
  if (total_kv > 0 && (!k_flat || !v_flat)) return fail(CA_EINVAL, "k_flat, v_flat must be non-NULL");
  if (!aligned16(k_flat) || !aligned16(v_flat)) return fail(CA_EINVAL, "k_flat, v_flat must be 16-byte aligned");
  if (total_kv < 0) return fail(CA_EINVAL, "total_kv < 0");
  if (kv_row_stride < d || kv_row_stride % 8 || kv_row_stride > (1 << 23))
    return fail(CA_EINVAL, "kv_row_stride must be in [d, 2^23] and a multiple of 8");
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0) return fail(CA_EINVAL, "cu_seqlens[0] != 0");
    for (int i = 0; i < B * H; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return fail(CA_EINVAL, "cu_seqlens decreasing at %d", i);
    if (cu_seqlens_host[B * H] > total_kv) return fail(CA_ERANGE, "cu_seqlens[B*H] > total_kv");
  }
  if (int r = check_device()) return r;
  if ((int64_t)B * H * Nq == 0) return ok();
  static thread_local AttnParams p;
  p = AttnParams{};
  fill_common(p, c);
  p.kf = static_cast<const uint16_t*>(k_flat);
  p.vf = static_cast<const uint16_t*>(v_flat);
  p.kfs_n = kv_row_stride;
  p.cu = cu_seqlens;
  p.total_kv = total_kv;
  std::vector<int> all(B * H);
  std::iota(all.begin(), all.end(), 0);
  std::vector<uint16_t> words;
  std::vector<int> tiles;
  if (cu_seqlens_host) {
    // longest heads first, so that the plain grid starts the long ones first
    for (int bh : longest_first(cu_seqlens_host, all)) {
      words.push_back((uint16_t)(bh | kFlatHead));
      tiles.push_back((cu_seqlens_host[bh + 1] - cu_seqlens_host[bh] + kTileKeys - 1) / kTileKeys);
    }
  } else {
    for (int bh : all) words.push_back((uint16_t)(bh | kFlatHead));
  }
  return launch_range(c, p, words, tiles, split, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream));
}

int ca_chunk_attn_mixed_fwd(const void* q, const void* k, const void* v, int B, int H, int Nq,
                            int Nkv, int d, const int64_t* q_strides, const int64_t* kv_strides,
                            const int64_t* o_strides, const int32_t* head_mode,
                            const int32_t* kv_indptr, const int32_t* kv_indices, int kv_nnz,
                            const int32_t* kv_shared_indptr, const int32_t* kv_shared_indices,
                            int kv_shared_nnz, int kv_block, int kv_seg, int q_block, int q_seg,
                            const void* k_flat, const void* v_flat, const int32_t* cu_seqlens,
                            const int32_t* cu_seqlens_host, int total_kv, int64_t kv_row_stride,
                            float scale, void* o, int o_dtype, float* lse, int split,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Common c{B, H, Nq, d, q, q_strides, o_strides, o, o_dtype, lse, scale};
  if (int r = check_common(c)) return r;
  if (int r = check_workspace(split, workspace, workspace_bytes)) return r;
  if (!head_mode) return fail(CA_EINVAL, "head_mode is NULL");
  std::vector<int> hd, hb, hv;
  for (int i = 0; i < B * H; ++i) {
    switch (head_mode[i]) {
      case CA_MODE_DENSE: hd.push_back(i); break;
      case CA_MODE_BLOCKS: hb.push_back(i); break;
      case CA_MODE_VARLEN: hv.push_back(i); break;
      default: return fail(CA_EINVAL, "head_mode[%d] = %d", i, head_mode[i]);
    }
  }
  if (!hd.empty() || !hb.empty()) {
    if (!k || !v) return fail(CA_EINVAL, "k and v must be non-NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(CA_EINVAL, "k, v must be 16-byte aligned");
    if (int r = check_strides("kv", kv_strides, 8)) return r;
    if (kv_strides[1] < d || kv_strides[1] > (1 << 23)) return fail(CA_ERANGE, "kv row stride outside [d, 2^23]");
    if (Nkv < 0) return fail(CA_EINVAL, "Nkv < 0");
  }
  if (!hb.empty()) {
    if (int r = check_csr(kv_indptr, kv_indices, kv_nnz, kv_block, kv_seg, q_block, q_seg)) return r;
    if (kv_shared_indptr || kv_shared_indices) {
      if (int r = check_csr(kv_shared_indptr, kv_shared_indices, kv_shared_nnz, kv_block, kv_seg,
                            q_block, q_seg)) return r;
      if (q_block > 64) return fail(CA_ERANGE, "q_block %d above 64 (a query block is served by 64 rows)", q_block);
      const int nqb = num_blocks(Nq, q_block, q_seg);
      if ((int64_t)hb.size() * ((nqb + 3) / 4) > 0x7FFFFFFF) return fail(CA_ERANGE, "too many work items");
    }
  }
  if (!hv.empty()) {
    if (!k_flat || !v_flat || !cu_seqlens) return fail(CA_EINVAL, "k_flat, v_flat, cu_seqlens must be non-NULL");
    if (!aligned16(k_flat) || !aligned16(v_flat)) return fail(CA_EINVAL, "k_flat, v_flat must be 16-byte aligned");
    if (total_kv < 0) return fail(CA_EINVAL, "total_kv < 0");
    if (kv_row_stride < d || kv_row_stride % 8 || kv_row_stride > (1 << 23))
    return fail(CA_EINVAL, "kv_row_stride must be in [d, 2^23] and a multiple of 8");
  }
  if (int r = check_device()) return r;
  if ((int64_t)B * H * Nq == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  static thread_local AttnParams p;
  if (!hd.empty() || !hv.empty()) {
    // dense and ragged heads both attend to one contiguous token range: one
    // range-mode launch covers them, each head reading its own source
    p = AttnParams{};
    fill_common(p, c);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    if (!hd.empty()) {
      p.ks_b = kv_strides[0]; p.ks_n = kv_strides[1]; p.ks_h = kv_strides[2];
    }
    p.Nkv = Nkv;
    p.kf = static_cast<const uint16_t*>(k_flat);
    p.vf = static_cast<const uint16_t*>(v_flat);
    p.kfs_n = kv_row_stride;
    p.cu = cu_seqlens;
    p.total_kv = total_kv;
    std::vector<uint16_t> words;
    std::vector<int> tiles;
    const bool known = hv.empty() || cu_seqlens_host;
    for (int bh : hd) {
      words.push_back((uint16_t)bh);
      if (known) tiles.push_back((Nkv + kTileKeys - 1) / kTileKeys);
    }
    if (cu_seqlens_host) hv = longest_first(cu_seqlens_host, hv);
    for (int bh : hv) {
      words.push_back((uint16_t)(bh | kFlatHead));
      if (known)
        tiles.push_back((cu_seqlens_host[bh + 1] - cu_seqlens_host[bh] + kTileKeys - 1) / kTileKeys);
    }
    if (int r = launch_range(c, p, words, tiles, split, workspace, workspace_bytes, s)) return r;
  }
  if (!hb.empty() && kv_shared_indptr) {
    // one-pass PBSA over the block-list heads, in launches of at most
    // kMaxHeadsPerLaunch heads
    static thread_local PbsaParams pp;
    pp = pbsa_params(q, k, v, B, H, Nq, Nkv, q_strides, kv_strides, o_strides, kv_shared_indptr,
                     kv_shared_indices, kv_shared_nnz, kv_indptr, kv_indices, kv_nnz, kv_block,
                     kv_seg, q_block, q_seg, scale, o, lse);
    const int groups = pp.groups;
    for (size_t h0 = 0; h0 < hb.size(); h0 += kMaxHeadsPerLaunch) {
      const int n = (int)std::min<size_t>(kMaxHeadsPerLaunch, hb.size() - h0);
      pp.use_list = 1;
      for (int i = 0; i < n; ++i) pp.heads[i] = (uint16_t)hb[h0 + i];
      pp.n_items = n * groups;
      if (int r = launched(launch_pbsa(d, o_dtype == CA_F32, pp, s), "pbsa launch")) return r;
    }
  } else if (!hb.empty()) {
    p = AttnParams{};
    fill_common(p, c);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.ks_b = kv_strides[0]; p.ks_n = kv_strides[1]; p.ks_h = kv_strides[2];
    p.Nkv = Nkv;
    fill_blocks(p, Nq, Nkv, kv_indptr, kv_indices, kv_nnz, kv_block, kv_seg, q_block, q_seg);
    if (int r = launch_blocks(c, p, hb, s)) return r;
  }
  return ok();
}

int ca_lse_merge(const void* o1, const float* lse1, const void* o2, const float* lse2,
                 int in_dtype, void* o, float* lse, int out_dtype, int B, int H, int N, int d,
                 const int64_t* o1_strides, const int64_t* o2_strides, const int64_t* o_strides,
                 void* stream) {
  if (B < 0 || H < 0 || N < 0) return fail(CA_EINVAL, "negative size");
  if (d != 8 && d != 16 && d != 32 && d != 64 && d != 128 && d != 256 && d != 512)
    return fail(CA_EUNSUPPORTED, "head dim %d (supported: 8..512, powers of two)", d);
  if ((in_dtype != CA_BF16 && in_dtype != CA_F32) || (out_dtype != CA_BF16 && out_dtype != CA_F32))
    return fail(CA_EUNSUPPORTED, "dtype");
  if (!o1 || !o2 || !lse1 || !lse2 || !o || !lse) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(o1) || !aligned16(o2) || !aligned16(o)) return fail(CA_EINVAL, "o1, o2, o must be 16-byte aligned");
  const int ia = in_dtype == CA_BF16 ? 8 : 4, oa = out_dtype == CA_BF16 ? 8 : 4;
  if (int r = check_strides("o1", o1_strides, ia)) return r;
  if (int r = check_strides("o2", o2_strides, ia)) return r;
  if (int r = check_strides("o", o_strides, oa)) return r;
  if (o == o2 || lse == lse2) return fail(CA_EINVAL, "outputs may alias only o1 / lse1");
  if (o == o1 && (in_dtype != out_dtype || o1_strides[0] != o_strides[0] ||
                  o1_strides[1] != o_strides[1] || o1_strides[2] != o_strides[2]))
    return fail(CA_EINVAL, "o aliases o1 with a different dtype or strides");
  if (int r = check_device()) return r;
  return launched(launch_lse_merge(o1, lse1, o2, lse2, in_dtype == CA_F32, o, lse,
                                   out_dtype == CA_F32, B, H, N, d, o1_strides, o2_strides,
                                   o_strides, static_cast<hipStream_t>(stream)),
                  "lse_merge launch");
}

int ca_block_mean(const void* x, int B, int N, int H, int d, const int64_t* x_strides,
                  int block_size, int seg_len, float* out, float* out_total, void* stream) {
  if (B < 0 || N < 0 || H < 0) return fail(CA_EINVAL, "negative size");
  if (d <= 0 || d % 8 || d > 512) return fail(CA_EUNSUPPORTED, "head dim %d (multiple of 8, <= 512)", d);
  if (block_size < 1 || seg_len < 1) return fail(CA_EINVAL, "block_size and seg_len must be >= 1");
  if (!x || !out) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(x)) return fail(CA_EINVAL, "x must be 16-byte aligned");
  if (int r = check_strides("x", x_strides, 8)) return r;
  if ((int64_t)B * H > 65535) return fail(CA_ERANGE, "B*H above 65535");
  const int nb = num_blocks(N, block_size, seg_len);
  if (int r = check_device()) return r;
  return launched(launch_block_mean(static_cast<const uint16_t*>(x), B, N, H, d, x_strides,
                                    block_size, seg_len, (seg_len + block_size - 1) / block_size,
                                    nb, out, out_total, static_cast<hipStream_t>(stream)),
                  "block_mean launch");
}

int ca_block_mean_pair(const void* x1, const int64_t* x1_strides, float* out1, float* out1_total,
                       const void* x2, const int64_t* x2_strides, float* out2, int B, int N,
                       int H, int d, int block_size, int seg_len, void* stream) {
  if (B < 0 || N < 0 || H < 0) return fail(CA_EINVAL, "negative size");
  if (d <= 0 || d % 8 || d > 512) return fail(CA_EUNSUPPORTED, "head dim %d (multiple of 8, <= 512)", d);
  if (block_size < 1 || seg_len < 1) return fail(CA_EINVAL, "block_size and seg_len must be >= 1");
  if (!x1 || !out1 || !x2 || !out2) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(x1) || !aligned16(x2)) return fail(CA_EINVAL, "x1 and x2 must be 16-byte aligned");
  if (int r = check_strides("x1", x1_strides, 8)) return r;
  if (int r = check_strides("x2", x2_strides, 8)) return r;
  if ((int64_t)B * H > 65535) return fail(CA_ERANGE, "B*H above 65535");
  const int nb = num_blocks(N, block_size, seg_len);
  if (int r = check_device()) return r;
  return launched(launch_block_mean(static_cast<const uint16_t*>(x1), B, N, H, d, x1_strides,
                                    block_size, seg_len, (seg_len + block_size - 1) / block_size,
                                    nb, out1, out1_total, static_cast<hipStream_t>(stream),
                                    static_cast<const uint16_t*>(x2), x2_strides, out2),
                  "block_mean_pair launch");
}

// Argument checks shared by the selection calls (one job of the batched
// call, or the single calls' arguments); `who` prefixes the message.
static int check_topk_job(const ca_topk_job& a, const char* who) {
  if (a.B < 0 || a.H < 0 || a.NQB < 0 || a.NKB < 0) return fail(CA_EINVAL, "%s: negative size", who);
  if (a.d <= 0 || a.d % 4 || a.d > 512)
    return fail(CA_EUNSUPPORTED, "%s: head dim %d (multiple of 4, <= 512)", who, a.d);
  if (!a.q_mean || !a.k_mean || !a.out_idx) return fail(CA_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(a.q_mean) || !aligned16(a.k_mean))
    return fail(CA_EINVAL, "%s: means must be 16-byte aligned", who);
  if (a.cand_count < 1 || a.cand_count > 4096)
    return fail(CA_ERANGE, "%s: cand_count %d outside 1..4096", who, a.cand_count);
  if (a.cand_begin < 0 || a.cand_begin + a.cand_count > a.NKB)
    return fail(CA_ERANGE, "%s: candidate range outside [0, NKB)", who);
  if (a.K < 1 || a.K > a.cand_count) return fail(CA_ERANGE, "%s: K=%d outside 1..cand_count", who, a.K);
  if (!a.indptr) return 0;
  if (!a.indices) return fail(CA_EINVAL, "%s: indices is NULL", who);
  if (a.prefix_begin < 0 || a.prefix_count < 0) return fail(CA_EINVAL, "%s: negative prefix", who);
  if ((int64_t)a.id_offset + a.cand_begin < 0 ||
      (int64_t)a.id_offset + a.cand_begin + a.cand_count > 0x7FFFFFFF)
    return fail(CA_ERANGE, "%s: id_offset out of range", who);
  if ((int64_t)a.prefix_begin + a.prefix_count > (int64_t)a.id_offset + a.cand_begin)
    return fail(CA_EINVAL, "%s: prefix range must lie below every candidate id + id_offset", who);
  if ((int64_t)a.B * a.H * a.NQB * (a.prefix_count + a.K) > 0x7FFFFFFF)
    return fail(CA_ERANGE, "%s: too many entries", who);
  return 0;
}

int ca_block_score_topk(const float* q_mean, const float* k_mean, int B, int H, int NQB, int NKB,
                        int d, int cand_begin, int cand_count, int K, int32_t* out_idx,
                        float* out_score, void* stream) {
  const ca_topk_job a{q_mean, k_mean, B, H, NQB, NKB, d, cand_begin, cand_count, K,
                      0, 0, 0, out_idx, out_score, nullptr, nullptr};
  if (int r = check_topk_job(a, "block_score_topk")) return r;
  if ((int64_t)B * H > 65535) return fail(CA_ERANGE, "grid too large");
  if (int r = check_device()) return r;
  return launched(launch_score_topk(q_mean, k_mean, B, H, NQB, NKB, d, cand_begin, cand_count, K,
                                    out_idx, out_score, static_cast<hipStream_t>(stream)),
                  "block_score_topk launch");
}

int ca_block_score_topk_lists(const float* q_mean, const float* k_mean, int B, int H, int NQB,
                              int NKB, int d, int cand_begin, int cand_count, int K,
                              int prefix_begin, int prefix_count, int id_offset,
                              int32_t* out_idx, int32_t* indptr, int32_t* indices, void* stream) {
  if (!indptr) return fail(CA_EINVAL, "block_score_topk_lists: indptr is NULL");
  const ca_topk_job a{q_mean, k_mean, B, H, NQB, NKB, d, cand_begin, cand_count, K,
                      prefix_begin, prefix_count, id_offset, out_idx, nullptr, indptr, indices};
  if (int r = check_topk_job(a, "block_score_topk_lists")) return r;
  if ((int64_t)B * H > 65535) return fail(CA_ERANGE, "grid too large");
  if (int r = check_device()) return r;
  return launched(launch_score_topk(q_mean, k_mean, B, H, NQB, NKB, d, cand_begin, cand_count, K,
                                    out_idx, nullptr, static_cast<hipStream_t>(stream), indptr,
                                    indices, prefix_begin, prefix_count, id_offset),
                  "block_score_topk_lists launch");
}

int ca_block_score_topk_batch(const ca_topk_job* jobs, int n_jobs, void* stream) {
  if (n_jobs < 1 || n_jobs > 4) return fail(CA_ERANGE, "n_jobs %d outside 1..4", n_jobs);
  if (!jobs) return fail(CA_EINVAL, "jobs is NULL");
  TopkJobDesc desc[4];
  int64_t wgs = 0;
  for (int i = 0; i < n_jobs; ++i) {
    const ca_topk_job& a = jobs[i];
    char who[16];
    snprintf(who, sizeof who, "job %d", i);
    if (int r = check_topk_job(a, who)) return r;
    wgs += (int64_t)a.B * a.H * a.NQB;
    desc[i] = TopkJobDesc{a.q_mean, a.k_mean, a.B, a.H, a.NQB, a.NKB, a.d, a.cand_begin,
                          a.cand_count, a.K, a.prefix_begin, a.prefix_count, a.id_offset,
                          a.out_idx, a.out_score, a.indptr, a.indices};
  }
  if (wgs > 0x7FFFFFFF) return fail(CA_ERANGE, "too many selection rows");
  if (int r = check_device()) return r;
  return launched(launch_score_topk_batch(desc, n_jobs, static_cast<hipStream_t>(stream)),
                  "block_score_topk_batch launch");
}

int ca_persistent_update(const float* q_mean, const float* k_mean, int B, int H, int NKB, int d,
                         const int32_t* persistent, int C_in, int evict_begin, int evict_count,
                         int C, int32_t* out, float* out_score, void* stream) {
  if (B < 0 || H < 0 || NKB < 0 || C_in < 0 || evict_count < 0 || evict_begin < 0)
    return fail(CA_EINVAL, "negative size");
  if (d <= 0 || d % 4 || d > 512) return fail(CA_EUNSUPPORTED, "head dim %d (multiple of 4, <= 512)", d);
  if (!q_mean || !k_mean || !out) return fail(CA_EINVAL, "NULL pointer");
  if (C_in > 0 && !persistent) return fail(CA_EINVAL, "persistent is NULL with C_in > 0");
  if (!aligned16(q_mean) || !aligned16(k_mean)) return fail(CA_EINVAL, "means must be 16-byte aligned");
  if (evict_begin + (int64_t)evict_count > NKB) return fail(CA_ERANGE, "evicted range outside [0, NKB)");
  if (C < 1 || (int64_t)C_in + evict_count > 4096 || C > 4096)
    return fail(CA_ERANGE, "need 1 <= C and C_in + evict_count, C <= 4096");
  if ((const void*)out == (const void*)persistent && C != C_in)
    return fail(CA_EINVAL, "in-place update needs C == C_in");
  if ((int64_t)B * H > 65535) return fail(CA_ERANGE, "B*H above 65535");
  if (int r = check_device()) return r;
  return launched(launch_persistent_update(q_mean, k_mean, B, H, NKB, d, persistent, C_in,
                                           evict_begin, evict_count, C, out, out_score,
                                           static_cast<hipStream_t>(stream)),
                  "persistent_update launch");
}

int ca_pack_ragged(const void* k, const void* v, int B, int N, int H, int d,
                   const int64_t* kv_strides, int frame_tokens, const int32_t* frame_ptr,
                   const int32_t* frame_ptr_host, int total_frames, const int32_t* frame_src,
                   void* k_flat, void* v_flat, int64_t flat_row_stride, int32_t* cu_seqlens,
                   void* stream) {
  if (B < 0 || H < 0 || N < 0 || total_frames < 0) return fail(CA_EINVAL, "negative size");
  if (d <= 0 || d % 8 || d > 512) return fail(CA_EUNSUPPORTED, "head dim %d (multiple of 8, <= 512)", d);
  if (frame_tokens < 1) return fail(CA_EINVAL, "frame_tokens must be >= 1");
  if ((int64_t)B * H < 1 || (int64_t)B * H > 32767) return fail(CA_ERANGE, "B*H outside 1..32767");
  if (!frame_ptr || !cu_seqlens) return fail(CA_EINVAL, "frame_ptr and cu_seqlens must be non-NULL");
  if (total_frames > 0 && (!k || !v || !frame_src || !k_flat || !v_flat))
    return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_flat) || !aligned16(v_flat))
    return fail(CA_EINVAL, "k, v, k_flat, v_flat must be 16-byte aligned");
  if (int r = check_strides("kv", kv_strides, 8)) return r;
  if (flat_row_stride < d || flat_row_stride % 8) return fail(CA_EINVAL, "flat_row_stride must be >= d and a multiple of 8");
  if ((int64_t)total_frames * frame_tokens > 0x7FFFFFFF || total_frames > 65535)
    return fail(CA_ERANGE, "too many output frames (at most 65535)");
  if (frame_ptr_host) {
    if (frame_ptr_host[0] != 0) return fail(CA_EINVAL, "frame_ptr[0] != 0");
    for (int i = 0; i < B * H; ++i)
      if (frame_ptr_host[i + 1] < frame_ptr_host[i]) return fail(CA_EINVAL, "frame_ptr decreasing at %d", i);
    if (frame_ptr_host[B * H] != total_frames) return fail(CA_EINVAL, "frame_ptr[B*H] != total_frames");
  }
  if (int r = check_device()) return r;
  return launched(launch_pack_ragged(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                     B, N, H, d, kv_strides, frame_tokens, frame_ptr, total_frames,
                                     frame_src, static_cast<uint16_t*>(k_flat),
                                     static_cast<uint16_t*>(v_flat), flat_row_stride, cu_seqlens,
                                     static_cast<hipStream_t>(stream)),
                  "pack_ragged launch");
}

// ---- latent KV cache (VideoMLA page, method) --------------------------------
namespace {
constexpr int kMlaNope = 96, kMlaRope = 32, kMlaLat = 192, kMlaVal = 128;

int check_mla_dims(int d_nope, int d_rope, int d_c, int d_v) {
  if (d_nope != kMlaNope || d_rope != kMlaRope || d_c != kMlaLat || d_v != kMlaVal)
    return fail(CA_EUNSUPPORTED, "latent dims (d_nope %d, d_rope %d, d_c %d, d_v %d); supported: 96, 32, 192, 128",
                d_nope, d_rope, d_c, d_v);
  return CA_OK;
}
}  // namespace

int ca_mla_absorb_q(const void* q, int B, int Nq, int H, int d_nope, int d_rope, int d_c,
                    const int64_t* q_strides, const void* w_uk, void* q_lat, void* q_lat_lo,
                    void* stream) {
  if (B < 0 || Nq < 0 || H < 0) return fail(CA_EINVAL, "negative size");
  if (int r = check_mla_dims(d_nope, d_rope, d_c, kMlaVal)) return r;
  if (!q || !w_uk || !q_lat) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(w_uk) || !aligned16(q_lat) || !aligned16(q_lat_lo))
    return fail(CA_EINVAL, "q, w_uk, q_lat, q_lat_lo must be 16-byte aligned");
  if (int r = check_strides("q", q_strides, 8)) return r;
  if ((int64_t)B * Nq * H > 0x7FFFFFFF / 256) return fail(CA_ERANGE, "too many rows");
  if (int r = check_device()) return r;
  return launched(launch_mla_absorb(static_cast<const uint16_t*>(q), B, Nq, H, q_strides,
                                    static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_lat),
                                    static_cast<uint16_t*>(q_lat_lo),
                                    static_cast<hipStream_t>(stream)),
                  "mla absorb launch");
}

int ca_mla_attn_fwd(const void* q_lat, const void* q_lat_lo, const void* kv_lat, int B, int Nq,
                    int H, int Nkv, int d_c, int d_rope, int64_t kv_batch_stride,
                    int64_t kv_row_stride, float scale, float* o_lat, float* lse, void* stream) {
  if (B < 0 || Nq < 0 || H < 0 || Nkv < 0) return fail(CA_EINVAL, "negative size");
  if (int r = check_mla_dims(kMlaNope, d_rope, d_c, kMlaVal)) return r;
  if (!q_lat || !o_lat || !lse || (Nkv > 0 && !kv_lat)) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(q_lat) || !aligned16(kv_lat) || !aligned16(o_lat) || !aligned16(q_lat_lo))
    return fail(CA_EINVAL, "q_lat, q_lat_lo, kv_lat, o_lat must be 16-byte aligned");
  if (kv_row_stride < d_c + d_rope || kv_row_stride % 8 || kv_row_stride > (1 << 22))
    return fail(CA_EINVAL, "kv_row_stride must be a multiple of 8 in [d_c + d_rope, 2^22]");
  if (kv_batch_stride < 0 || kv_batch_stride % 8) return fail(CA_EINVAL, "kv_batch_stride must be a non-negative multiple of 8");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CA_EINVAL, "scale must be finite and > 0");
  if ((int64_t)Nq * H > 0x7FFFFFFF / 2 || (int64_t)B * ((int64_t)Nq * H + 127) / 128 > 0x7FFFFFFF)
    return fail(CA_ERANGE, "too many rows");
  if (int r = check_device()) return r;
  return launched(launch_mla_attn(static_cast<const uint16_t*>(q_lat),
                                  static_cast<const uint16_t*>(q_lat_lo),
                                  static_cast<const uint16_t*>(kv_lat),
                                  kv_batch_stride, kv_row_stride, B, Nq, H, Nkv, scale, o_lat, lse,
                                  static_cast<hipStream_t>(stream)),
                  "mla attention launch");
}

int ca_mla_up_proj(const float* o_lat, const void* w_uv, int B, int Nq, int H, int d_c, int d_v,
                   void* o, int o_dtype, const int64_t* o_strides, void* stream) {
  if (B < 0 || Nq < 0 || H < 0) return fail(CA_EINVAL, "negative size");
  if (int r = check_mla_dims(kMlaNope, kMlaRope, d_c, d_v)) return r;
  if (o_dtype != CA_BF16 && o_dtype != CA_F32) return fail(CA_EUNSUPPORTED, "o_dtype %d", o_dtype);
  if (!o_lat || !w_uv || !o) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(o)) return fail(CA_EINVAL, "o_lat, w_uv, o must be 16-byte aligned");
  if (int r = check_strides("o", o_strides, 4)) return r;
  if ((int64_t)B * Nq * H > 0x7FFFFFFF / 256) return fail(CA_ERANGE, "too many rows");
  if (int r = check_device()) return r;
  return launched(launch_mla_up(o_lat, B, Nq, H, static_cast<const uint16_t*>(w_uv), o, o_dtype == CA_F32,
                                o_strides, static_cast<hipStream_t>(stream)),
                  "mla up-projection launch");
}

int ca_cast_bf16_to_f16(const void* x, void* y, int64_t n, void* stream) {
  if (n < 0 || n % 8) return fail(CA_EINVAL, "n must be a non-negative multiple of 8");
  if (n > 0 && (!x || !y)) return fail(CA_EINVAL, "NULL pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(CA_EINVAL, "x, y must be 16-byte aligned");
  if (int r = check_device()) return r;
  return launched(launch_cast_bf16_f16(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), n,
                                       static_cast<hipStream_t>(stream)),
                  "cast launch");
}

int ca_build_kv_index(int B, int H, int NQB, int sink_begin, int sink_count,
                      const int32_t* persistent, int C, const int32_t* topk, int K,
                      int topk_offset, int32_t* indptr, int32_t* indices, void* stream) {
  if (B < 0 || H < 0 || NQB < 0 || sink_count < 0 || C < 0 || K < 0 || sink_begin < 0)
    return fail(CA_EINVAL, "negative size");
  if ((int64_t)B * H * NQB > 65536) return fail(CA_ERANGE, "more than 65536 rows");
  if (!indptr || !indices) return fail(CA_EINVAL, "indptr and indices must be non-NULL");
  if ((C > 0 && !persistent) || (K > 0 && !topk)) return fail(CA_EINVAL, "persistent/topk NULL with nonzero count");
  if ((int64_t)B * H * NQB * ((int64_t)sink_count + C + K) > 0x7FFFFFFF) return fail(CA_ERANGE, "too many entries");
  if (int r = check_device()) return r;
  return launched(launch_build_kv_index(B * H * NQB, sink_begin, sink_count, C ? persistent : nullptr,
                                        C, NQB, K ? topk : nullptr, K, topk_offset, indptr, indices,
                                        static_cast<hipStream_t>(stream)),
                  "build_kv_index launch");
}

// ---- the block-sparse pipeline (Sparse Forcing page, section 2) -------------
namespace {

struct SparseArgs {
  const void* q;
  const void* k;
  const void* v;
  int B, H, Nq, Nkv, d;
  const int64_t* qs;
  const int64_t* kvs;
  const int64_t* os;
  int block, seg;
  int sink_begin, sink_count, hist_begin, hist_count, C, local_begin, local_count, K;
  const float* k_mean;
  float scale;
  void* o;
  int o_dtype;
  float* lse;
};

constexpr size_t kWsAlign = 256;

size_t ws_take(size_t& at, size_t bytes) {
  const size_t r = at;
  at += (bytes + kWsAlign - 1) / kWsAlign * kWsAlign;
  return r;
}

// Pointer and stride checks of the pipeline's tensors.
int check_sparse_tensors(const SparseArgs& a) {
  Common c{a.B, a.H, a.Nq, a.d, a.q, a.qs, a.os, a.o, a.o_dtype, a.lse, a.scale};
  if (int r = check_common(c)) return r;
  if (a.Nkv > 0 && (!a.k || !a.v)) return fail(CA_EINVAL, "k and v must be non-NULL");
  if (!aligned16(a.k) || !aligned16(a.v) || !aligned16(a.k_mean))
    return fail(CA_EINVAL, "k, v, k_mean must be 16-byte aligned");
  if (int r = check_strides("kv", a.kvs, 8)) return r;
  if (a.kvs[1] < a.d || a.kvs[1] > (1 << 23)) return fail(CA_ERANGE, "kv row stride outside [d, 2^23]");
  return CA_OK;
}

// Checks the sizes and block ranges and lays out the intermediates in a
// workspace (a.k_mean is only tested for NULL here).
int plan_sparse(const SparseArgs& a, ca_block_sparse_ws& w) {
  w = ca_block_sparse_ws{};
  if (a.B < 0 || a.H < 0 || a.Nq < 0 || a.Nkv < 0) return fail(CA_EINVAL, "negative size");
  if (a.d != 64 && a.d != 128) return fail(CA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", a.d);
  if (a.block < 1 || a.block > 64) return fail(CA_ERANGE, "block %d outside 1..64", a.block);
  if (a.seg < 1) return fail(CA_EINVAL, "seg < 1");
  if ((int64_t)a.B * a.H > 65535) return fail(CA_ERANGE, "B*H above 65535");
  const int nkb = num_blocks(a.Nkv, a.block, a.seg);
  const int nqb = num_blocks(a.Nq, a.block, a.seg);
  const int rng[3][2] = {{a.sink_begin, a.sink_count}, {a.hist_begin, a.hist_count},
                         {a.local_begin, a.local_count}};
  for (int i = 0; i < 3; ++i) {
    if (rng[i][0] < 0 || rng[i][1] < 0 || (int64_t)rng[i][0] + rng[i][1] > nkb)
      return fail(CA_ERANGE, "block range %d outside [0, %d)", i, nkb);
    for (int j = 0; j < i; ++j)
      if (rng[i][1] && rng[j][1] && rng[i][0] < rng[j][0] + rng[j][1] &&
          rng[j][0] < rng[i][0] + rng[i][1])
        return fail(CA_EINVAL, "sink, history and local block ranges must be disjoint");
  }
  if (a.C < 0 || a.C > a.hist_count || a.hist_count > 4096)
    return fail(CA_ERANGE, "C=%d outside 0..hist_count (at most 4096 candidates)", a.C);
  if (a.K < 0 || a.K > a.local_count || a.local_count > 4096)
    return fail(CA_ERANGE, "K=%d outside 0..local_count (at most 4096 candidates)", a.K);
  const int64_t BH = (int64_t)a.B * a.H;
  if (BH * nqb > 65536) return fail(CA_ERANGE, "more than 65536 query blocks");
  const int bps = (a.seg + a.block - 1) / a.block;
  // local-window means over the window alone: the window starts on a segment
  // boundary and its own tiling has exactly local_count blocks
  int win_t0 = 0, win_n = 0;
  bool window = false;
  if (a.k_mean && a.K > 0 && a.local_begin % bps == 0) {
    const int last = a.local_begin + a.local_count - 1;
    win_t0 = (a.local_begin / bps) * a.seg;
    const int t1 = std::min(a.Nkv, (last / bps) * a.seg + std::min(a.seg, (last % bps + 1) * a.block));
    win_n = t1 - win_t0;
    window = win_n > 0 && num_blocks(win_n, a.block, a.seg) == a.local_count;
  }
  const bool selects = a.C > 0 || a.K > 0;
  const bool all_k = selects && (!a.k_mean || (a.K > 0 && !window));
  size_t at = 0;
  const size_t f = sizeof(float), i4 = sizeof(int32_t);
  w.q_mean = ws_take(at, selects ? BH * nqb * a.d * f : 0);
  w.k_mean = ws_take(at, all_k ? BH * nkb * a.d * f : 0);
  w.k_mean_local = ws_take(at, window ? BH * a.local_count * a.d * f : 0);
  w.chunk_mean = ws_take(at, BH * a.d * f);
  w.persistent = ws_take(at, BH * std::max(a.C, 1) * i4);
  w.local = ws_take(at, BH * nqb * std::max(a.K, 1) * i4);
  w.shared_indptr = ws_take(at, (BH + 1) * i4);
  w.shared_indices = ws_take(at, (BH * ((int64_t)a.sink_count + a.C) + 1) * i4);
  w.local_indptr = ws_take(at, (BH * nqb + 1) * i4);
  w.local_indices = ws_take(at, (BH * nqb * a.K + 1) * i4);
  w.bytes = at;
  w.window_means = window ? 1 : 0;
  w.window_token0 = window ? win_t0 : 0;
  w.window_tokens = window ? win_n : 0;
  w.local_id_base = window ? a.local_begin : 0;
  w.k_mean_in_ws = all_k ? 1 : 0;
  return CA_OK;
}

// The pipeline on a planned workspace: block means (and the chunk mean),
// persistent top-C and local top-K with their block lists, then one PBSA
// launch.  Every intermediate is written before it is read.
int run_sparse(const SparseArgs& a, const ca_block_sparse_ws& w, char* ws, hipStream_t s) {
  if (int r = check_device()) return r;
  if ((int64_t)a.B * a.H * a.Nq == 0) return ok();
  const int BH = a.B * a.H;
  const int nkb = num_blocks(a.Nkv, a.block, a.seg);
  const int nqb = num_blocks(a.Nq, a.block, a.seg);
  const int bps = (a.seg + a.block - 1) / a.block;
  float* qm = reinterpret_cast<float*>(ws + w.q_mean);
  float* km_ws = reinterpret_cast<float*>(ws + w.k_mean);
  float* km_win = reinterpret_cast<float*>(ws + w.k_mean_local);
  float* cm = reinterpret_cast<float*>(ws + w.chunk_mean);
  int32_t* pers = reinterpret_cast<int32_t*>(ws + w.persistent);
  int32_t* loc = reinterpret_cast<int32_t*>(ws + w.local);
  int32_t* sh_ptr = reinterpret_cast<int32_t*>(ws + w.shared_indptr);
  int32_t* sh_idx = reinterpret_cast<int32_t*>(ws + w.shared_indices);
  int32_t* lo_ptr = reinterpret_cast<int32_t*>(ws + w.local_indptr);
  int32_t* lo_idx = reinterpret_cast<int32_t*>(ws + w.local_indices);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  hipError_t e = hipSuccess;

  // 1. block representatives: the query blocks, the local window's key
  //    blocks (or every key block); the chunk mean is formed from the query
  //    block means inside the selection launch
  if (a.C > 0 || a.K > 0) {
    if (w.window_means && w.window_tokens == a.Nq) {
      // the window holds as many tokens as the chunk: one launch for both
      e = launch_block_mean(q, a.B, a.Nq, a.H, a.d, a.qs, a.block, a.seg, bps, nqb, qm, nullptr, s,
                            k + (int64_t)w.window_token0 * a.kvs[1], a.kvs, km_win);
    } else {
      e = launch_block_mean(q, a.B, a.Nq, a.H, a.d, a.qs, a.block, a.seg, bps, nqb, qm, nullptr, s);
      if (e == hipSuccess && w.window_means)
        e = launch_block_mean(k + (int64_t)w.window_token0 * a.kvs[1], a.B, w.window_tokens, a.H,
                              a.d, a.kvs, a.block, a.seg, bps, a.local_count, km_win, nullptr, s);
      if (e == hipSuccess && w.k_mean_in_ws)
        e = launch_block_mean(k, a.B, a.Nkv, a.H, a.d, a.kvs, a.block, a.seg, bps, nkb, km_ws,
                              nullptr, s);
    }
    if (e != hipSuccess) return launched(e, "block mean launch");
  }

  // 2. selections, writing the block lists where each row is a prefix range
  //    followed by the selected ids
  const float* km_hist = a.k_mean ? a.k_mean : km_ws;
  const bool fused_shared = a.C > 0 && a.sink_begin + a.sink_count <= a.hist_begin;
  TopkJobDesc jobs[2];
  int nj = 0;
  if (a.C > 0)
    jobs[nj++] = TopkJobDesc{cm, km_hist, a.B, a.H, 1, nkb, a.d, a.hist_begin, a.hist_count, a.C,
                             a.sink_begin, a.sink_count, 0, pers, nullptr,
                             fused_shared ? sh_ptr : nullptr, fused_shared ? sh_idx : nullptr,
                             qm, a.Nq, a.block, a.seg, nqb};
  if (a.K > 0) {
    const float* km_loc = w.window_means ? km_win : km_ws;
    const int nkb_loc = w.window_means ? a.local_count : nkb;
    const int cand0 = w.window_means ? 0 : a.local_begin;
    jobs[nj++] = TopkJobDesc{qm, km_loc, a.B, a.H, nqb, nkb_loc, a.d, cand0, a.local_count, a.K,
                             0, 0, w.local_id_base, loc, nullptr, lo_ptr, lo_idx};
  }
  if (nj > 0) {
    e = launch_score_topk_batch(jobs, nj, s);
    if (e != hipSuccess) return launched(e, "selection launch");
  }
  if (!fused_shared) {
    // sink range above the history, or no persistent blocks: a general merge
    e = launch_build_kv_index(BH, a.sink_begin, a.sink_count, a.C > 0 ? pers : nullptr, a.C, 1,
                              nullptr, 0, 0, sh_ptr, sh_idx, s);
    if (e != hipSuccess) return launched(e, "block list launch");
  }
  if (a.K == 0) {
    e = launch_build_kv_index(BH * nqb, 0, 0, nullptr, 0, nqb, nullptr, 0, 0, lo_ptr, lo_idx, s);
    if (e != hipSuccess) return launched(e, "block list launch");
  }

  // 3. attention over the union of each query block's two lists
  const PbsaParams p = pbsa_params(a.q, a.k, a.v, a.B, a.H, a.Nq, a.Nkv, a.qs, a.kvs, a.os, sh_ptr,
                                   sh_idx, BH * (a.sink_count + a.C), lo_ptr, lo_idx,
                                   BH * nqb * a.K, a.block, a.seg, a.block, a.seg, a.scale, a.o,
                                   a.lse);
  return launched(launch_pbsa(a.d, a.o_dtype == CA_F32, p, s), "pbsa launch");
}

// Device scratch of the allocation-free pipeline (one copy per GPU, held
// until the process ends).  Host code never passes the array's name to a
// kernel: it is a host-side stand-in, and the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = CA_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

char* scratch_ptr(int& status) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    status = fail(CA_ENODEV, "no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      status = fail(CA_EHIP, "scratch address: %s", hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = ptr;
  }
  status = CA_OK;
  return static_cast<char*>(ptrs[dev]);
}

}  // namespace

size_t ca_block_sparse_workspace(int B, int H, int Nq, int Nkv, int d, int block, int seg,
                                 int sink_begin, int sink_count, int hist_begin, int hist_count,
                                 int C, int local_begin, int local_count, int K, int have_k_mean,
                                 ca_block_sparse_ws* layout) {
  static const int64_t dummy[3] = {0, 0, 0};
  const SparseArgs a{nullptr, nullptr, nullptr, B, H, Nq, Nkv, d, dummy, dummy, dummy, block, seg,
                     sink_begin, sink_count, hist_begin, hist_count, C, local_begin, local_count,
                     K, have_k_mean ? reinterpret_cast<const float*>(kWsAlign) : nullptr, 1.f,
                     nullptr, CA_BF16, nullptr};
  ca_block_sparse_ws w;
  if (plan_sparse(a, w) != CA_OK) return 0;
  if (layout) *layout = w;
  ok();
  return w.bytes;
}

int ca_block_sparse_fwd(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nkv,
                        int d, const int64_t* q_strides, const int64_t* kv_strides,
                        const int64_t* o_strides, int block, int seg, int sink_begin,
                        int sink_count, int hist_begin, int hist_count, int C, int local_begin,
                        int local_count, int K, const float* k_mean, float scale, void* o,
                        int o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const SparseArgs a{q, k, v, B, H, Nq, Nkv, d, q_strides, kv_strides, o_strides, block, seg,
                     sink_begin, sink_count, hist_begin, hist_count, C, local_begin, local_count,
                     K, k_mean, scale, o, o_dtype, lse};
  if (int r = check_sparse_tensors(a)) return r;
  ca_block_sparse_ws w;
  if (int r = plan_sparse(a, w)) return r;
  if (!workspace || !aligned16(workspace)) return fail(CA_EINVAL, "workspace must be non-NULL and 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign)
    return fail(CA_EINVAL, "workspace must be %zu-byte aligned", kWsAlign);
  if (workspace_bytes < w.bytes)
    return fail(CA_EINVAL, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, w.bytes);
  return run_sparse(a, w, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

int ca_block_sparse_fwd_noalloc(const void* q, const void* k, const void* v, int B, int H, int Nq,
                                int Nkv, int d, const int64_t* q_strides,
                                const int64_t* kv_strides, const int64_t* o_strides, int block,
                                int seg, int sink_begin, int sink_count, int hist_begin,
                                int hist_count, int C, int local_begin, int local_count, int K,
                                const float* k_mean, float scale, void* o, int o_dtype,
                                float* lse, void* stream) {
  const SparseArgs a{q, k, v, B, H, Nq, Nkv, d, q_strides, kv_strides, o_strides, block, seg,
                     sink_begin, sink_count, hist_begin, hist_count, C, local_begin, local_count,
                     K, k_mean, scale, o, o_dtype, lse};
  if (int r = check_sparse_tensors(a)) return r;
  ca_block_sparse_ws w;
  if (int r = plan_sparse(a, w)) return r;
  if (w.bytes > kScratchBytes)
    return fail(CA_ERANGE, "the pipeline needs %zu bytes of scratch; the library holds %zu",
                w.bytes, kScratchBytes);
  if (int r = check_device()) return r;
  int st = CA_OK;
  char* ws = scratch_ptr(st);
  if (!ws) return st;
  return run_sparse(a, w, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
