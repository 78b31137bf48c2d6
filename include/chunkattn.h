/*
 * chunkattn — chunk attention of a streaming video generator's new latent-frame
 * chunk against its KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  Every tensor argument is a DEVICE pointer owned by the caller
 * unless marked "host".  Every call is asynchronous on `stream` (a hipStream_t;
 * NULL = the null stream), never synchronises, never allocates device memory
 * and keeps no state between calls besides the thread-local error text and a
 * per-device count of resident workgroups, queried once.
 *
 * Element types: CA_BF16 = bfloat16 (round-to-nearest-even on output),
 * CA_F32 = IEEE float32.  LSE is always float32, natural log.
 *
 * Layouts.  Q, K, V and O are 4-D [B, N, H, d] described by a host array of
 * three element strides {stride_b, stride_n, stride_h}; the d axis is
 * contiguous (stride 1).  LSE is a contiguous float32 [B, H, Nq] array.
 *
 * Alignment: base pointers 16-byte aligned; every stride must keep each
 * row start 16-byte aligned (a multiple of 8 elements for bf16, of 4 for f32).
 *
 * Errors.  Arguments are checked on the host before any device call; a bad
 * argument returns CA_EINVAL / CA_EUNSUPPORTED / CA_ERANGE and launches
 * nothing.  No visible GPU returns CA_ENODEV.  A failed launch returns CA_EHIP.
 * ca_last_error() then holds a message for the calling thread.  Outputs are
 * undefined after an error.  Contents of device index arrays (CSR ids,
 * cu_seqlens) cannot be checked without synchronising: ids outside the valid
 * range and spans outside the flat buffers are skipped by the kernels (they
 * contribute no keys), they never cause an out-of-bounds access.
 */
#ifndef CHUNKATTN_H
#define CHUNKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CA_ABI_VERSION 4

enum ca_status {
  CA_OK = 0,
  CA_EINVAL = 1,        /* null or misaligned pointer, bad shape or stride */
  CA_EUNSUPPORTED = 2,  /* head dim or dtype the kernels do not cover */
  CA_ERANGE = 3,        /* K larger than the candidates, tiling too large */
  CA_ENODEV = 4,        /* no HIP device visible */
  CA_EHIP = 5           /* a HIP launch failed; see ca_last_error() */
};

enum ca_dtype { CA_BF16 = 0, CA_F32 = 1 };

/* key-range split policy of the dense / ragged launches (see
 * ca_attn_workspace_bytes): taken when it shortens a launch by more than a
 * fifth (AUTO), never, or whenever it applies (ALWAYS: a workspace is given,
 * head lengths are known and there is enough work) */
enum ca_split_policy { CA_SPLIT_AUTO = 0, CA_SPLIT_NEVER = 1, CA_SPLIT_ALWAYS = 2 };

/* per-head cache mode for ca_chunk_attn_mixed_fwd */
enum ca_head_mode { CA_MODE_DENSE = 0, CA_MODE_BLOCKS = 1, CA_MODE_VARLEN = 2 };

int ca_abi_version(void);
const char* ca_status_str(int status);
const char* ca_last_error(void);

/*
 * Number of blocks of the frame-aligned tiling of n_tokens: the token axis is
 * cut into segments of seg_len tokens (the last may be shorter) and each
 * segment into blocks of block_size tokens (the last block of a segment takes
 * the remainder).  Block id j covers tokens [start_j, start_j + len_j).
 * Blocks are the spatio-temporal blocks of the Sparse Forcing page, section 2
 * item 2 (blockified compression); with seg_len = 1560 a latent frame is 24
 * blocks of 64 plus one block of 24.  Host-only; returns -1 on bad sizes.
 */
int ca_num_blocks(int n_tokens, int block_size, int seg_len);

/*
 * Size in bytes of the optional workspace of the chunk-attention calls for
 * head dim d (64 or 128) on the current device; 0 for another d or no device.
 *
 * With a workspace (caller-owned device memory, 16-byte aligned, at least this
 * size) a dense or ragged launch may take the balanced schedule: its grid is
 * the number of workgroups the device holds at once, and each workgroup takes
 * an equal share of the cost of the (query tile, 64-key tile) pairs of all
 * heads, in head order, where every query tile a workgroup touches also
 * costs a fixed charge of 8 key tiles (loading its queries, filling and
 * draining the tile pipeline, writing its state).  A query tile whose key
 * range is split between workgroups is
 * finished by an LSE merge of the float32 partial results (O/l, LSE) that
 * the workgroups leave in the workspace: attention over consecutive key
 * ranges recombined through the LSE state (ISPA page, section 2 item 1).
 * The result is the same attention up to float32 rounding.  The schedule is
 * taken only when it shortens the launch by more than a fifth by that cost
 * (chiefly heads of unequal length); it needs every head's key count on the
 * host (always for the dense cache; for ragged heads only with
 * cu_seqlens_host).  Calls sharing one workspace
 * must be ordered on one stream.  NULL = no workspace: one workgroup per
 * (head, query tile).
 */
size_t ca_attn_workspace_bytes(int d);

/*
 * Chunk attention, dense or block-list cache.  For each (b, h) and query row i
 * over its key set I:
 *   O[b,i,h,:] = sum_{j in I} softmax_j(scale * q_i . k_j) v_j
 *   LSE[b,h,i] = ln sum_{j in I} exp(scale * q_i . k_j)
 * (attention with its LSE state: ISPA page, section 2 item 1, decomposable
 * attention; block lists: Sparse Forcing page, section 2 item 3, PBSA — dense
 * over persistent blocks, top-K blocks of the local window).
 *
 *   q            bf16 [B, Nq, H, d], strides q_strides (host, 3 elements)
 *   k, v         bf16 [B, Nkv, H, d], both with strides kv_strides (host);
 *                may be NULL when Nkv = 0 (every key set empty)
 *   d            64 or 128
 *   kv_indptr,   NULL, NULL  -> dense: I = all Nkv cached tokens.
 *   kv_indices   else CSR over rows (b*H + h)*NQB + qb, NQB =
 *                ca_num_blocks(Nq, q_block, q_seg): row r lists KV block ids
 *                (tiling kv_block, kv_seg of the Nkv axis) whose tokens are the
 *                key set of the rows of query block qb.  int32, device.
 *                kv_indptr has B*H*NQB + 1 entries, nondecreasing from 0.
 *                Ids must be distinct within a row; order is free.
 *   kv_nnz       number of entries of kv_indices; row spans are clamped to it.
 *   kv_block     1..64; kv_seg >= 1; q_block >= 1; q_seg >= 1 (block mode)
 *   scale        softmax scale, finite and > 0 (1/sqrt(d) for the pages' models)
 *   o_init,      NULL, NULL -> plain attention.  Else the float32 O [B, Nq, H, d]
 *   lse_init     (strides o_init_strides) and LSE [B, H, Nq] of attention over
 *                another, disjoint key set: the softmax state starts from it, so
 *                the outputs are the LSE merge of that branch with this call's
 *                key set (ISPA page, section 2 item 1: local and history
 *                branches combined through the LSE), without a separate pass.
 *                o may alias o_init (float32 output, same strides) and lse may
 *                alias lse_init.
 *   o            [B, Nq, H, d] of o_dtype (CA_BF16 or CA_F32), strides o_strides
 *   lse          float32 [B, H, Nq]; an empty key set gives O = 0, LSE = -inf
 *   split        a ca_split_policy value (CA_SPLIT_AUTO unless tuning)
 *   workspace,   optional (NULL, 0 allowed), see ca_attn_workspace_bytes; used
 *   workspace_bytes  by the dense cache only (block lists and o_init ignore
 *                it).  A workspace smaller than the schedule needs is
 *                CA_EINVAL.
 */
int ca_chunk_attn_fwd(const void* q, const void* k, const void* v,
                      int B, int H, int Nq, int Nkv, int d,
                      const int64_t* q_strides, const int64_t* kv_strides,
                      const int64_t* o_strides,
                      const int32_t* kv_indptr, const int32_t* kv_indices, int kv_nnz,
                      int kv_block, int kv_seg, int q_block, int q_seg, float scale,
                      const float* o_init, const int64_t* o_init_strides, const float* lse_init,
                      void* o, int o_dtype, float* lse, int split,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * PBSA in one pass (Sparse Forcing page, section 2 item 3: dense attention
 * over the persistent blocks, sparse attention over the top-K blocks of the
 * local window chosen per query block).  The key set of query block qb of
 * head (b, h) is the union of two block lists:
 *   shared_indptr,   CSR row b*H + h (B*H + 1 entries): blocks every query
 *   shared_indices   block of the head attends to (the sink frame and the
 *                    persistent blocks)
 *   local_indptr,    CSR row (b*H + h)*NQB + qb (B*H*NQB + 1 entries,
 *   local_indices    NQB = ca_num_blocks(Nq, q_block, q_seg)): the query
 *                    block's own blocks (its top-K window blocks)
 * Ids refer to the KV tiling (kv_block, kv_seg), must be distinct within a
 * row, and a block must not appear in both lists of a row (it would count
 * twice); order is free.  Ids outside the tiling contribute no keys.
 *   *_nnz        entries of the indices arrays; row spans are clamped to them
 *   q_block      1..64 (each query block is served by 64 rows of a workgroup)
 * One launch: each workgroup keeps four query blocks' softmax state in
 * registers over the shared list and then their local lists, with no
 * intermediate output.  Other arguments as in ca_chunk_attn_fwd; an empty
 * key set gives O = 0, LSE = -inf.
 */
int ca_chunk_attn_pbsa_fwd(const void* q, const void* k, const void* v,
                           int B, int H, int Nq, int Nkv, int d,
                           const int64_t* q_strides, const int64_t* kv_strides,
                           const int64_t* o_strides,
                           const int32_t* shared_indptr, const int32_t* shared_indices,
                           int shared_nnz, const int32_t* local_indptr,
                           const int32_t* local_indices, int local_nnz,
                           int kv_block, int kv_seg, int q_block, int q_seg, float scale,
                           void* o, int o_dtype, float* lse, void* stream);

/*
 * The block-sparse path in one call (Sparse Forcing page, section 2): block
 * representatives (item 2: the mean of each block's tokens), persistent
 * memory = the C history blocks with the highest coarse score against the
 * chunk-mean query (item 1), the K local-window blocks with the highest
 * coarse score per query block (item 2), and PBSA over the union of the
 * sink blocks, the persistent blocks and the query block's top-K blocks
 * (item 3, one ca_chunk_attn_pbsa_fwd launch).  Coarse scores, ties and id
 * order as in ca_block_score_topk.
 *
 *   q, k, v, strides, scale, o, o_dtype, lse   as in ca_chunk_attn_fwd
 *   block, seg   one frame-aligned tiling for both axes (block 1..64): query
 *                block qb and KV block ids as ca_num_blocks counts them
 *   sink_begin, sink_count   KV blocks every query block attends to
 *   hist_begin, hist_count   candidates of the persistent selection
 *   local_begin, local_count candidates of the top-K selection (the local
 *                            window, at most 4096; so is the history)
 *                The three ranges lie in [0, NKB) and must be disjoint.
 *   C, K         0 <= C <= hist_count, 0 <= K <= local_count
 *   k_mean       optional float32 [B, H, NKB, d]: key-block means kept as
 *                resident state from earlier steps (only the history
 *                entries are read; the local window holds the current chunk,
 *                so its means are recomputed from k).  NULL: every key
 *                block's mean is computed.
 *   workspace    caller-owned device memory of at least the size
 *                ca_block_sparse_workspace returns, 256-byte aligned; it
 *                holds the intermediates at the offsets that call reports
 *                (they can be read back after the call).  Calls sharing a
 *                workspace must be ordered on one stream.
 * Launches: one block-mean launch (two or three when the local window is
 * not the chunk's own size or not frame-aligned), one selection launch
 * (both selections and their block lists; a separate list merge when the
 * sink range lies above the history or C = 0), one attention launch.
 */
typedef struct ca_block_sparse_ws {
  size_t bytes;            /* workspace size */
  size_t q_mean;           /* float32 [B, H, NQB, d] query-block means */
  size_t k_mean;           /* float32 [B, H, NKB, d] every key block's mean (k_mean_in_ws) */
  size_t k_mean_local;     /* float32 [B, H, local_count, d] the window's means (window_means) */
  size_t chunk_mean;       /* float32 [B, H, d] mean of all Nq queries per head (C > 0) */
  size_t persistent;       /* int32 [B, H, C] persistent ids, ascending */
  size_t local;            /* int32 [B, H, NQB, K] top-K ids - local_id_base, ascending */
  size_t shared_indptr;    /* int32 [B*H + 1] ... */
  size_t shared_indices;   /* ... CSR per head: sink + persistent ids */
  size_t local_indptr;     /* int32 [B*H*NQB + 1] ... */
  size_t local_indices;    /* ... CSR per query block: its top-K ids */
  int window_means;        /* 1: the local window's means are computed over the window alone */
  int window_token0;       /* its first token */
  int window_tokens;       /* its token count */
  int local_id_base;       /* absolute KV block id = local id + local_id_base */
  int k_mean_in_ws;        /* 1: k_mean holds every key block's mean */
} ca_block_sparse_ws;

/* Workspace size of ca_block_sparse_fwd for these sizes and ranges
 * (have_k_mean: whether k_mean will be given), 0 on invalid arguments
 * (ca_last_error() says why); `layout` (NULL allowed) receives the offsets. */
size_t ca_block_sparse_workspace(int B, int H, int Nq, int Nkv, int d, int block, int seg,
                                 int sink_begin, int sink_count, int hist_begin, int hist_count,
                                 int C, int local_begin, int local_count, int K, int have_k_mean,
                                 ca_block_sparse_ws* layout);

int ca_block_sparse_fwd(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nkv,
                        int d, const int64_t* q_strides, const int64_t* kv_strides,
                        const int64_t* o_strides, int block, int seg, int sink_begin,
                        int sink_count, int hist_begin, int hist_count, int C, int local_begin,
                        int local_count, int K, const float* k_mean, float scale, void* o,
                        int o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * ca_block_sparse_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results, without the workspace: the
 * intermediates live in a device array the library holds, CA_SCRATCH_BYTES
 * (16 MiB) per GPU, for the lifetime of the process (about 1 MB suffices for
 * the 12-head Wan layer with resident key means, 4.3 MB without).  Sizes
 * whose ca_block_sparse_workspace exceeds it return CA_ERANGE.  No call
 * allocates or frees anything.  Every call on one GPU uses the same array:
 * calls that overlap on a GPU (different streams, or host threads) race and
 * must be ordered by the caller; every intermediate is rewritten by each call
 * before it is read, so nothing carries over between calls.
 */
#define CA_SCRATCH_BYTES ((size_t)16 << 20)
int ca_block_sparse_fwd_noalloc(const void* q, const void* k, const void* v, int B, int H, int Nq,
                                int Nkv, int d, const int64_t* q_strides,
                                const int64_t* kv_strides, const int64_t* o_strides, int block,
                                int seg, int sink_begin, int sink_count, int hist_begin,
                                int hist_count, int C, int local_begin, int local_count, int K,
                                const float* k_mean, float scale, void* o, int o_dtype,
                                float* lse, void* stream);

/*
 * Dual-output chunk attention (ISPA page, section 2 item 1: the dual-stream
 * warmup computes attention over the local tokens — the current frames and
 * the sink — and over the full history side by side).  Block-list mode as in
 * ca_chunk_attn_fwd, where the first local_count ids of every CSR row form
 * the local key set and the whole row the full key set.  One pass over each
 * row writes both:
 *   o_local, lse_local  attention over the row's first local_count blocks
 *                       (all of them when the row is shorter; an empty local
 *                       set gives O = 0, LSE = -inf)
 *   o, lse              attention over the whole row
 *   o_local             [B, Nq, H, d] of o_dtype, strides o_local_strides (host);
 *                       lse_local float32 [B, H, Nq].  Neither may alias o, lse.
 * Other arguments as in ca_chunk_attn_fwd (no o_init, no workspace).
 */
int ca_chunk_attn_dual_fwd(const void* q, const void* k, const void* v,
                           int B, int H, int Nq, int Nkv, int d,
                           const int64_t* q_strides, const int64_t* kv_strides,
                           const int32_t* kv_indptr, const int32_t* kv_indices, int kv_nnz,
                           int kv_block, int kv_seg, int q_block, int q_seg, int local_count,
                           float scale, void* o_local, const int64_t* o_local_strides,
                           float* lse_local, void* o, const int64_t* o_strides, int o_dtype,
                           float* lse, void* stream);

/*
 * Chunk attention over ragged per-head caches (Pyramid Forcing page, section
 * 3, ragged-cache attention): head (b, h) owns rows
 * [cu_seqlens[b*H+h], cu_seqlens[b*H+h+1]) of the flat K/V buffers, no padding.
 *
 *   k_flat, v_flat  bf16 [total_kv, d], row stride kv_row_stride elements;
 *                   may be NULL when total_kv = 0
 *   cu_seqlens      int32 [B*H + 1], device, nondecreasing, cu[0] = 0,
 *                   cu[B*H] <= total_kv
 *   cu_seqlens_host optional host copy (NULL allowed), equal to cu_seqlens:
 *                   when given, the launch can take the balanced schedule
 *                   (with a workspace), else heads are scheduled longest first.
 * Other arguments as in ca_chunk_attn_fwd.
 */
int ca_chunk_attn_varlen_fwd(const void* q, const void* k_flat, const void* v_flat,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int total_kv, int B, int H, int Nq, int d,
                             const int64_t* q_strides, int64_t kv_row_stride,
                             const int64_t* o_strides, float scale,
                             void* o, int o_dtype, float* lse, int split,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged cache packing (Pyramid Forcing page, section 2: per-head cache
 * policies -- adaptive-stride or periodic frame sampling, or merging adjacent
 * frames -- plus the shared sink and forced recent frames; section 3: the
 * variable-length caches are stored flat with boundary indices and packed in
 * one vectorized pass).  Builds the inputs of ca_chunk_attn_varlen_fwd from a
 * dense per-head cache in one launch.
 *
 *   k, v         bf16 dense cache [B, N, H, d], strides kv_strides (host);
 *                frame f of a head is its tokens [f T, (f + 1) T),
 *                T = frame_tokens; only whole frames (f < N / T) are frames
 *   frame_ptr    int32 [B*H + 1], device: head b*H + h owns output frames
 *                [frame_ptr[bh], frame_ptr[bh+1]), nondecreasing from 0 to
 *                total_frames.  frame_ptr_host: optional host copy, checked
 *                when given
 *   frame_src    int32 [total_frames, 2], device: output frame j copies
 *                source frame frame_src[j][0] of its head, or, when
 *                frame_src[j][1] != -1, merges the two source frames: each
 *                element = bf16(round to nearest even of (float32(a + b) /
 *                2)).  Source frames outside [0, N / T) contribute zeros.
 *   k_flat,      bf16 [total_frames * T, d] outputs, row stride
 *   v_flat       flat_row_stride elements (a multiple of 8, >= d)
 *   cu_seqlens   int32 [B*H + 1] output: frame_ptr * T
 *   limits       d a multiple of 8, <= 512; 1 <= B*H <= 32767;
 *                total_frames <= 65535
 */
int ca_pack_ragged(const void* k, const void* v, int B, int N, int H, int d,
                   const int64_t* kv_strides, int frame_tokens, const int32_t* frame_ptr,
                   const int32_t* frame_ptr_host, int total_frames, const int32_t* frame_src,
                   void* k_flat, void* v_flat, int64_t flat_row_stride, int32_t* cu_seqlens,
                   void* stream);

/*
 * Mixed per-head cache modes in one call (Pyramid Forcing page, section 3:
 * heads with different cache layouts served together to cut launches).
 * head_mode (host, int32 [B*H]) picks CA_MODE_DENSE (k, v dense cache),
 * CA_MODE_BLOCKS (k, v + the CSR, as in ca_chunk_attn_fwd; rows of other heads
 * are ignored) or CA_MODE_VARLEN (k_flat, v_flat + cu_seqlens, as in
 * ca_chunk_attn_varlen_fwd; other heads' spans are ignored).  Pointers of a
 * mode no head uses may be NULL.  Dense and ragged heads share one launch
 * (balanced across them when a workspace is given and the ragged lengths are
 * known on the host); block-list heads follow in a second launch.
 * With kv_shared_indptr / kv_shared_indices (device, a CSR of B*H rows, row
 * b*H + h; NULL for none) the block-list heads run one-pass PBSA instead (as
 * ca_chunk_attn_pbsa_fwd, Sparse Forcing page, section 2 item 3): each of
 * their query blocks attends to its head's shared row together with its own
 * row of kv_indptr / kv_indices (its local list); the two lists of a row must
 * be disjoint and q_block at most 64 (CA_ERANGE otherwise).
 */
int ca_chunk_attn_mixed_fwd(const void* q, const void* k, const void* v,
                            int B, int H, int Nq, int Nkv, int d,
                            const int64_t* q_strides, const int64_t* kv_strides,
                            const int64_t* o_strides, const int32_t* head_mode,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            int kv_nnz, const int32_t* kv_shared_indptr,
                            const int32_t* kv_shared_indices, int kv_shared_nnz,
                            int kv_block, int kv_seg, int q_block, int q_seg,
                            const void* k_flat, const void* v_flat,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                            int total_kv, int64_t kv_row_stride, float scale,
                            void* o, int o_dtype, float* lse, int split,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * LSE merge of two attention results over disjoint key sets (ISPA page,
 * section 2 item 1: local and history branches recombined afterwards):
 *   M = max(L1, L2), w_k = exp(L_k - M), LSE = M + ln(w1 + w2),
 *   O = (w1 O1 + w2 O2) / (w1 + w2);  both branches -inf -> O = 0, LSE = -inf.
 *   o1, o2   [B, N, H, d] of in_dtype, strides o1_strides / o2_strides (host)
 *   lse1,2   float32 [B, H, N]
 *   o, lse   outputs, out_dtype / float32.  o may alias o1 (same strides and
 *            dtype) and lse may alias lse1; no other overlap is allowed.
 *   d        8, 16, 32, 64, 128, 256 or 512
 */
int ca_lse_merge(const void* o1, const float* lse1, const void* o2, const float* lse2,
                 int in_dtype, void* o, float* lse, int out_dtype,
                 int B, int H, int N, int d,
                 const int64_t* o1_strides, const int64_t* o2_strides,
                 const int64_t* o_strides, void* stream);

/*
 * Block representatives (Sparse Forcing page, section 2 item 2: each block is
 * compressed to one representative token for coarse scoring): the mean of
 * each block's tokens, accumulated in float32.
 *   x          bf16 [B, N, H, d], strides x_strides (host); d a multiple of 8, <= 512
 *   out        float32 [B, H, NB, d] contiguous, NB = ca_num_blocks(N, block, seg)
 *   out_total  optional (NULL allowed) float32 [B, H, 1, d]: the mean over all N
 *              tokens (the chunk-mean query used to pick persistent blocks),
 *              formed from the block means weighted by block length.
 */
int ca_block_mean(const void* x, int B, int N, int H, int d, const int64_t* x_strides,
                  int block_size, int seg_len, float* out, float* out_total, void* stream);

/*
 * ca_block_mean of two bf16 tensors of the same shape [B, N, H, d] and block
 * tiling in one launch (Sparse Forcing page, section 2 item 2: the query
 * blocks and the local-window key blocks are compressed for the same
 * scoring step): out1 (and optionally out1_total) from x1, out2 from x2, each
 * exactly as ca_block_mean would write them.  Strides are per tensor (host);
 * limits and errors as ca_block_mean.
 */
int ca_block_mean_pair(const void* x1, const int64_t* x1_strides, float* out1, float* out1_total,
                       const void* x2, const int64_t* x2_strides, float* out2,
                       int B, int N, int H, int d, int block_size, int seg_len, void* stream);

/*
 * Coarse block scores and top-K (Sparse Forcing page, section 2 items 1-2:
 * scoring on block representatives, top-C persistent blocks, top-K local
 * blocks).  score(qb, c) = <q_mean[b,h,qb,:], k_mean[b,h,c,:]> in float32 for
 * candidates c in [cand_begin, cand_begin + cand_count); the K highest per
 * (b, h, qb) are kept, equal scores resolved toward the lower block id, and
 * written in ascending id order.
 *   q_mean   float32 [B, H, NQB, d] contiguous; k_mean float32 [B, H, NKB, d]
 *   out_idx  int32 [B, H, NQB, K] (absolute block ids, ascending)
 *   out_score optional float32 [B, H, NQB, K] (score of each out_idx entry)
 *   limits   1 <= K <= cand_count <= 4096, cand range inside [0, NKB), d <= 512
 */
int ca_block_score_topk(const float* q_mean, const float* k_mean,
                        int B, int H, int NQB, int NKB, int d,
                        int cand_begin, int cand_count, int K,
                        int32_t* out_idx, float* out_score, void* stream);

/*
 * ca_block_score_topk that also writes the PBSA block lists (Sparse Forcing
 * page, section 2 item 3) of the selection in the same launch, for the case
 * where the lists are a fixed prefix range followed by the selected ids:
 * CSR row r = (b*H + h)*NQB + qb holds W = prefix_count + K ids,
 *   prefix_begin .. prefix_begin + prefix_count - 1, then
 *   id_offset + out_idx[b,h,qb,0..K-1] (ascending).
 * The result equals ca_build_kv_index with sink range = the prefix and this
 * selection as its persistent ids (NQB = 1) or top-K ids (id_offset as
 * topk_offset), without the separate launch.
 *   out_idx  int32 [B, H, NQB, K] as ca_block_score_topk (required)
 *   indptr   int32 [B*H*NQB + 1] (= r * W); indices int32 [B*H*NQB*W]
 *   limits   as ca_block_score_topk; prefix_begin, prefix_count >= 0 and
 *            prefix_begin + prefix_count <= id_offset + cand_begin (so every
 *            row is sorted and free of duplicates), else CA_EINVAL
 */
int ca_block_score_topk_lists(const float* q_mean, const float* k_mean,
                              int B, int H, int NQB, int NKB, int d,
                              int cand_begin, int cand_count, int K,
                              int prefix_begin, int prefix_count, int id_offset,
                              int32_t* out_idx, int32_t* indptr, int32_t* indices,
                              void* stream);

/*
 * Several independent selections (each as ca_block_score_topk, or as
 * ca_block_score_topk_lists when indptr is non-NULL) in one launch.  The
 * persistent top-C against the chunk-mean query and the local top-K per
 * query block (Sparse Forcing page, section 2 items 1-3) depend only on the
 * block means, so the persistent selection's few workgroups can run beside
 * the local selection's many.  Each job's outputs equal the separate call's.
 *   jobs     host array of n_jobs descriptors, 1 <= n_jobs <= 4; each job has
 *            the arguments and limits of the single call (out_score may be
 *            NULL; indptr NULL = no block lists, else indices, prefix_begin,
 *            prefix_count and id_offset as in ca_block_score_topk_lists)
 */
typedef struct ca_topk_job {
  const float* q_mean;
  const float* k_mean;
  int B, H, NQB, NKB, d;
  int cand_begin, cand_count, K;
  int prefix_begin, prefix_count, id_offset;
  int32_t* out_idx;
  float* out_score;
  int32_t* indptr;
  int32_t* indices;
} ca_topk_job;

int ca_block_score_topk_batch(const ca_topk_job* jobs, int n_jobs, void* stream);

/*
 * Persistent-memory update when the local window slides (Sparse Forcing
 * page, section 2 item 1, memory management: blocks evicted from the local
 * window are candidates, and the top C by coarse score are kept or updated as
 * persistent memory).  Per (b, h), the candidates are the set union of the
 * evicted blocks [evict_begin, evict_begin + evict_count) and the current
 * persistent ids persistent[b,h,:] that lie in [0, NKB); each is scored
 * <q_mean[b,h,0,:], k_mean[b,h,id,:]> in float32 (q_mean: the query
 * representative, e.g. the chunk-mean query from ca_block_mean's out_total)
 * and the C highest are kept, equal scores resolved toward the lower block
 * id, written in ascending id order.  Slots past the number of candidates get
 * id -1 (score -inf).
 *   q_mean     float32 [B, H, 1, d] contiguous; k_mean float32 [B, H, NKB, d]
 *   persistent int32 [B, H, C_in] (distinct ids per head); NULL with C_in = 0
 *   out        int32 [B, H, C]; may be the persistent array itself when
 *              C == C_in (updated in place)
 *   out_score  optional float32 [B, H, C]
 *   limits     d a multiple of 4, <= 512; 1 <= C; C_in + evict_count <= 4096,
 *              C <= 4096; the evicted range inside [0, NKB)
 */
int ca_persistent_update(const float* q_mean, const float* k_mean, int B, int H, int NKB, int d,
                         const int32_t* persistent, int C_in, int evict_begin, int evict_count,
                         int C, int32_t* out, float* out_score, void* stream);

/*
 * Latent KV cache (VideoMLA page, method).  The cache keeps per token one
 * content latent c_t (d_c = 192 values) and one rotated position key k^R_t
 * (d_rope = 32), shared by all heads, stored together as one row [c_t ; k^R_t]
 * of 224 fp16 values; head h's keys and values are [W^K_h c_t ; k^R_t] and
 * W^V_h c_t (d_nope = 96 + d_rope = 32 key values, d_v = 128 value values).
 * Attention runs in the absorbed form: the query's content part is projected
 * into the latent space, all (query, head) rows attend to the same latent
 * rows, and the latent-space output is projected per head:
 *   ca_mla_absorb_q  q_lat = [(W^K_h)^T q^nope ; q^R]          (fp16)
 *   ca_mla_attn_fwd  o_lat = sum_t softmax_t(scale q_lat . kv_t) c_t, LSE
 *   ca_mla_up_proj   o = W^V_h o_lat
 * which equals attention with the reconstructed per-head keys and values
 * (associativity).  The pages' configuration d_c = 192, d_rope = 32 (d_nope =
 * 96, d_v = 128) is the one supported; other sizes are CA_EUNSUPPORTED.
 *
 * ca_mla_absorb_q
 *   q      bf16 [B, Nq, H, 128] (q^nope = first 96 values, q^R = last 32),
 *          element strides q_strides (host, multiples of 8), values contiguous
 *   w_uk   bf16 [H, 96, 192] (W^K_h: latent -> content key), contiguous
 *   q_lat  fp16 [B, Nq, H, 224] contiguous output (exact bf16 products,
 *          float32 accumulation, one rounding to fp16; values beyond fp16's
 *          range saturate to +-65504)
 *   q_lat_lo  optional (NULL allowed) bf16 [B, Nq, H, 192] contiguous output:
 *          the rounding residual x - fp16(x) of each absorbed content value
 * ca_mla_attn_fwd
 *   q_lat  fp16 [B, Nq, H, 224] contiguous (from ca_mla_absorb_q)
 *   q_lat_lo  optional (NULL allowed) residual from ca_mla_absorb_q.  Given,
 *          the LSE gets the first-order correction of the query's fp16
 *          rounding: LSE += scale * (q_lat_lo . o_lat) (the softmax-weighted
 *          mean latent row is o_lat on the content part, and the position
 *          part of the query is exact in fp16), leaving float32-grade LSE
 *          error instead of 2^-12 relative error on every score.  o_lat is
 *          not corrected (its error from the rounding is first order in the
 *          score error times the spread of the values, well inside the O bar)
 *   kv_lat fp16 latent rows [c ; k^R] (224 values): row t of batch entry b at
 *          kv_lat + b kv_batch_stride + t kv_row_stride (elements; the row
 *          stride a multiple of 8 and >= 224); a bf16 cache converts with
 *          ca_cast_bf16_to_f16 (exact for values in fp16's normal range)
 *   scale  softmax scale (1/sqrt(128) for the pages' model)
 *   o_lat  float32 [B, Nq, H, 192] contiguous; lse float32 [B, H, Nq]
 *          (natural log; no keys -> o_lat = 0, LSE = -inf)
 * ca_mla_up_proj
 *   o_lat  as above; w_uv bf16 [H, 128, 192] (W^V_h), contiguous
 *   o      [B, Nq, H, 128] of o_dtype (CA_BF16 or CA_F32), element strides
 *          o_strides (host, multiples of 4); float32 o_lat enters the product
 *          as a sum of two bf16 parts (relative residual 2^-17)
 * All pointers of the three calls are 16-byte aligned (else CA_EINVAL).
 * ca_cast_bf16_to_f16: y[i] = fp16 round-to-nearest-even of bf16 x[i], n a
 *   multiple of 8, both 16-byte aligned.  Exact for |x| in fp16's normal
 *   range [2^-14, 65504]; smaller magnitudes round to fp16's subnormal grid
 *   (absolute error <= 2^-25); larger finite magnitudes saturate to +-65504
 *   (no infinities, which would turn whole rows of scores into NaN); +-inf
 *   maps to +-65504 and NaN stays NaN.  A cache holding values beyond 65504
 *   is therefore not represented exactly and its attention is not exact.
 */
int ca_mla_absorb_q(const void* q, int B, int Nq, int H, int d_nope, int d_rope, int d_c,
                    const int64_t* q_strides, const void* w_uk, void* q_lat, void* q_lat_lo,
                    void* stream);
int ca_mla_attn_fwd(const void* q_lat, const void* q_lat_lo, const void* kv_lat, int B, int Nq,
                    int H, int Nkv, int d_c, int d_rope, int64_t kv_batch_stride,
                    int64_t kv_row_stride, float scale, float* o_lat, float* lse, void* stream);
int ca_mla_up_proj(const float* o_lat, const void* w_uv, int B, int Nq, int H, int d_c, int d_v,
                   void* o, int o_dtype, const int64_t* o_strides, void* stream);
int ca_cast_bf16_to_f16(const void* x, void* y, int64_t n, void* stream);

/*
 * PBSA block lists (Sparse Forcing page, section 2 item 3): CSR row
 * (b*H + h)*NQB + qb = sorted union, duplicates removed, of the sink blocks
 * [sink_begin, sink_begin + sink_count), persistent[b,h,:] (C ids, ascending,
 * may be NULL with C = 0) and topk_offset + topk[b,h,qb,:] (K ids, ascending,
 * may be NULL with K = 0).
 *   indptr   int32 [B*H*NQB + 1]   indices int32, room for
 *            B*H*NQB*(sink_count + C + K) entries.
 * B*H*NQB at most 65536.
 */
int ca_build_kv_index(int B, int H, int NQB, int sink_begin, int sink_count,
                      const int32_t* persistent, int C, const int32_t* topk, int K,
                      int topk_offset, int32_t* indptr, int32_t* indices, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKATTN_H */
