/*
 * bsa.h -- routed block-sparse attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsa.so.  Every operation here is one stage of VSA-style routed
 * block-sparse attention, or of its two alternative index modes:
 *
 *   vsa_tile_index       3D spatio-temporal tiling tables
 *   vsa_pool_route_topk  per-block mean pooling, routing scores, TopK + index table
 *   bsa_forward_qouter   exact sparse attention, one query block (VSA) or one
 *                        query token (NSA) at a time over its selected KV blocks
 *   bsa_forward_kvouter  KV-outer schedule: reverse index, scheduler, K1 partials
 *   bsa_combine          K2: exact log-sum-exp merge of the K1 partials
 *
 * Sources (page title, section):
 *   [VSA]  "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" (maple.link)
 *   [NSA]  "NSA 算子解析（Torch/Tilelang）" (devpress.csdn.net)
 *   [MSA]  "MSA 为什么采用 KV-outer Sparse Attention Forward" (notes.kuangjux.top)
 *   [Spark] "深度解读|Spark-H3：从注意力几何到稀疏内核代码" (jefxiong.cn)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array argument is device memory owned by the caller.  The
 *           library never allocates: calls that need scratch take a
 *           caller-supplied workspace whose size comes from the matching *_ws
 *           query (contents undefined after the call, except the regions
 *           bsa_kvouter_index_layout describes).  Calls that share a
 *           workspace must be ordered on one stream; calls with their own
 *           workspaces may run concurrently on different streams.  The only
 *           state the library keeps is one sticky index-error flag per device
 *           (see Errors).
 * Streams.  `stream` is a hipStream_t (NULL = the legacy default stream).
 *           Every call only enqueues work on that stream and returns; results
 *           are ready when the stream is synchronised.
 * Errors.   Shapes, strides, dtypes, sizes and null pointers are validated on
 *           the host before anything is enqueued; on failure nothing is
 *           written and the status says why (bsa_last_error() gives a message
 *           for the calling thread).  Launch failures map to BSA_ERR_HIP.
 *           Index entries < 0, and entries at positions >= their row count,
 *           are skipped and never dereferenced ([VSA] section 6.2: -1 entries
 *           are not addresses; [NSA] "Tilelang优化实现": negative ids are
 *           skipped).  Entries that name no block (>= the number of blocks J,
 *           or at or beyond the sequence in token mode and KV-outer) are
 *           skipped the same way, and the kernel that meets one sets the
 *           device's index-error flag, which bsa_check() reports as
 *           BSA_ERR_INDEX (and clears).  Nothing aborts, throws or prints.
 * Tensors.  A bsa_tdesc describes a 4-D view [B, N, H, D] (batch, token,
 *           head, channel) with element strides sB, sN, sH and D contiguous
 *           (stride 1).  Both BSHD ([B,N,H,D] contiguous) and BHSD
 *           ([B,H,N,D] contiguous, described with sH = N*D, sN = D) are
 *           accepted: the layout changes the memory order, not the tiling
 *           ([VSA] section 5.4).  Base pointers must be 16-byte aligned and,
 *           for bf16, strides must be multiples of 8 elements.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_ARG = 1,          /* null pointer, negative size, bad enum        */
  BSA_ERR_SHAPE = 2,        /* inconsistent shapes / strides / alignment    */
  BSA_ERR_UNSUPPORTED = 3,  /* valid request outside the supported envelope */
  BSA_ERR_WORKSPACE = 4,    /* workspace null or smaller than required      */
  BSA_ERR_INDEX = 5,        /* index table inconsistent with its shapes     */
  BSA_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed   */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_F32 = 1 } bsa_dtype;

/* Strided 4-D tensor view [B, N, H, D]; strides in elements, D contiguous. */
typedef struct {
  int64_t B, N, H, D;
  int64_t sB, sN, sH;
} bsa_tdesc;

/* Selection modes of bsa_forward_qouter. */
enum { BSA_SEL_BLOCK = 0, BSA_SEL_TOKEN = 1 };

/* Message describing the last non-OK status returned on this thread. */
const char* bsa_last_error(void);

/* Library version string. */
const char* bsa_version(void);

/* Synchronise `stream` and report any asynchronous HIP error as BSA_ERR_HIP;
 * then read the current device's index-error flag: if a kernel (of any
 * stream of this device) met a block id that names no block since the last
 * check, clear the flag and return BSA_ERR_INDEX. */
bsa_status bsa_check(void* stream);

/* ----------------------------------------------------------------------------
 * Tiling ([VSA] sections 1 and 3).
 *
 * bsa_tile_dims (host only): J = ceil(T/bT)*ceil(H/bH)*ceil(W/bW) blocks of
 * capacity M = bT*bH*bW.
 *
 * vsa_tile_index: block b = (bt*JH + by)*JW + bx covers t in
 * [bt*bT, min(T,(bt+1)*bT)) and likewise y, x; its n_b valid members are listed
 * with t slowest and x fastest, token id = t*H*W + y*W + x.
 *   perm      int32 [J*M]  token id held by packed slot b*M + r, or -1 for r >= n_b
 *   block_len int32 [J]    n_b
 *   inv       int32 [N]    packed slot of each token (inv[perm[p]] = p); may be NULL
 * N = T*H*W must be below 2^31.
 * ------------------------------------------------------------------------- */
bsa_status bsa_tile_dims(int T, int H, int W, int bT, int bH, int bW, int* J, int* M);
bsa_status vsa_tile_index(int T, int H, int W, int bT, int bH, int bW,
                          int32_t* perm, int32_t* block_len, int32_t* inv, void* stream);

/* Keep budget R = max(1, min(ceil((1 - s) * J), J)) ([VSA] section 2.2), with
 * 1e-9 subtracted before the ceiling so that (1-0.7)*10 gives 3.  Host only;
 * returns -1 when J < 1 or s lies outside [0, 1]. */
int vsa_budget(double drop_ratio, int J);

/* ----------------------------------------------------------------------------
 * Pool -> route -> TopK ([VSA] sections 2.1, 2.2 and 4).
 *
 * For every batch b, head h and query block i:
 *   qbar_i = (1/n_i) * sum_{r < n_i} Q[b, perm[i*M + r], h, :]   (likewise kbar)
 *   E[i, j] = scale * qbar_i . kbar_j           (scale is normally 1/sqrt(D))
 *   the R largest E[i, :] (ties: lower j first) are written to
 *   q2k_idx[b,h,i,0:R] in increasing order, q2k_idx[b,h,i,R:kmax] = -1, and
 *   q2k_num[b,h,i] = R.
 * Pooled means are accumulated in fp32 and E is formed to fp32 accuracy
 * (a three-product bf16 split on the matrix cores).
 *
 * q, k      strided views (dtype dt) of the same [B, N, H, D] shape
 * perm, block_len   tiling tables of J blocks of capacity M (vsa_tile_index)
 * q2k_idx   int32 [B, H, J, kmax] contiguous, kmax >= R
 * q2k_num   int32 [B, H, J] contiguous
 * qbar, kbar  optional fp32 [B, H, J, D] outputs (NULL: kept in the workspace)
 * E         optional fp32 [B, H, J, J] output of the scores (NULL: none); the
 *           input of vsa_coarse
 * item_order  optional int32 [B, H, J] output (NULL: not computed): for each
 *           (b, h) a permutation of 0..J-1 that places query blocks with
 *           similar kept sets next to each other (ascending Morton code of the
 *           quartile entries q2k_idx[.., (n-1)/4], [(n-1)/2], [3(n-1)/4],
 *           each scaled to 10 bits, ties by block index).  It is a processing
 *           order for bsa_forward_qouter and changes no result.
 * perm_bh_stride  0: perm is one table shared by every (b, h); else each
 *           (b, h) has its own table at perm + (b*H + h) * perm_bh_stride
 *           (>= J*M; per-head layouts such as spark_reblock's), block_len is
 *           shared.
 * Supported: 1 <= R <= J <= 4096, D <= 256, any N.  qbar, kbar and the
 * workspace must be 16-byte aligned.  The workspace holds the pooled means
 * and, for D = 64, 128 or 256, the pooled keys split into bf16 hi/lo planes
 * for the score products: vsa_pool_route_topk_ws() bytes.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* q;
  const void* k;
  bsa_tdesc d;
  bsa_dtype dt;
  const int32_t* perm;
  const int32_t* block_len;
  int J, M;
  int R, kmax;
  float scale;
  int32_t* q2k_idx;
  int32_t* q2k_num;
  float* qbar;
  float* kbar;
  float* E;
  int32_t* item_order;
  int64_t perm_bh_stride;
} vsa_route_args;

bsa_status vsa_pool_route_topk_ws(const vsa_route_args* a, size_t* bytes);
bsa_status vsa_pool_route_topk(const vsa_route_args* a, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * H3 multi-region layout ([VSA] section 5.2) and grouped routing ([VSA]
 * section 5.3, the default "exempt" rule).
 *
 * A packed sequence is a list of segments in their original order: a dense
 * segment (text, reference image, audio; video = 0, T = its token count, may
 * be 0) or a video region (video = 1, a T x H x W grid).  Layout: every dense
 * segment is cut on its own into 1D chunks of M = bT*bH*bW tokens (the last
 * chunk of each segment is short, no chunk mixes segments); all dense chunks
 * come first, in segment order (the prefix, num_prefix blocks); then every
 * video region in order, tiled in 3D exactly as vsa_tile_index tiles one
 * grid.  Tables as for vsa_tile_index: perm [J*M] holds original positions
 * (segment offset + position inside the segment, t slowest, x fastest inside
 * a video), -1 padding; block_len [J]; inv [N] optional.
 *
 * h3_tile_dims (host only): J, M, N (total tokens), num_prefix, the number of
 * video regions and, when spans is not NULL, their half-open block ranges
 * spans[2r], spans[2r+1] (room for 2*BSA_H3_MAX_SEGMENTS ints).
 * Supported: 1 <= nseg <= BSA_H3_MAX_SEGMENTS, N and J*M below 2^31.
 * ------------------------------------------------------------------------- */
#define BSA_H3_MAX_SEGMENTS 16

typedef struct {
  int video;
  int T, H, W;
} bsa_segment;

bsa_status h3_tile_dims(const bsa_segment* seg, int nseg, int bT, int bH, int bW, int* J, int* M, int* N,
                        int* num_prefix, int* nregions, int* spans);
bsa_status h3_tile_index(const bsa_segment* seg, int nseg, int bT, int bH, int bW, int32_t* perm,
                         int32_t* block_len, int32_t* inv, void* stream);

/* Grouped routing over a multi-region layout.  Pooled means and scores as in
 * vsa_pool_route_topk over all J blocks; then for every batch b and head h:
 *   query block i < num_prefix (context): keeps every block 0..J-1;
 *   query block i >= num_prefix (video): keeps blocks 0..num_prefix-1 and, for
 *     every region r = [spans[2r], spans[2r+1]), the budgets[r] largest
 *     E[i, j] over the region's j (ties: lower j first);
 * written ascending to q2k_idx[b,h,i,:] with -1 fill ([VSA] section 5.3: the
 * table is kmax = J wide, so a video row is mostly fill), count in q2k_num.
 * With no_fill set, entries at or past a row's count are left as they are
 * (bsa_forward_qouter and the item order read only the first q2k_num[row]
 * entries of a row); this saves rewriting the fill, most of the table's
 * bytes, on every call.  item_order (optional) is as in vsa_pool_route_topk
 * with the num_prefix context blocks first in every (b, h), so that
 * bsa_forward_qouter with order_long = num_prefix takes them first.  The
 * attention over the union is bsa_forward_qouter in block mode.
 *   spans, budgets   host arrays [2*nregions], [nregions]: the regions must
 *                    tile [num_prefix, J) in order; 1 <= budgets[r] <= size
 *   kmax             >= J when num_prefix > 0, and >= num_prefix + sum budgets
 * Supported as vsa_pool_route_topk (J <= 4096, D <= 256, B*H <= 65535),
 * nregions <= BSA_H3_MAX_SEGMENTS; nregions = 0 only with num_prefix = J.
 * The workspace holds the pooled means and the key planes of the widest
 * region: h3_pool_route_topk_ws() bytes (alignment as vsa_pool_route_topk). */
typedef struct {
  const void* q;
  const void* k;
  bsa_tdesc d;
  bsa_dtype dt;
  const int32_t* perm;
  const int32_t* block_len;
  int J, M;
  int num_prefix;
  int nregions;
  const int32_t* spans;
  const int32_t* budgets;
  int kmax;
  float scale;
  int32_t* q2k_idx;
  int32_t* q2k_num;
  float* qbar;
  float* kbar;
  int32_t* item_order;
  int no_fill;  /* 0: -1 fill past each row's count; nonzero: no fill */
} h3_route_args;

bsa_status h3_pool_route_topk_ws(const h3_route_args* a, size_t* bytes);
bsa_status h3_pool_route_topk(const h3_route_args* a, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Exact sparse attention, query-outer order.
 *
 * mode BSA_SEL_BLOCK (VSA; [VSA] sections 4, 6.2, 6.3, 6.5): every valid query
 *   token a of block i (a = perm[i*M + r], r < n_i) attends, with one softmax,
 *   to the union of the valid tokens of blocks q2k_idx[b,h,i,p] for
 *   p < q2k_num[b,h,i] (entries < 0 skipped).  No causal mask.  Output rows are
 *   written at the tokens' original positions; padding rows are never written.
 *   Requires Hq == Hkv.  Fields: perm, block_len, J, M, q2k_idx [B,H,J,kmax],
 *   q2k_num [B,H,J], kmax; optional item_order int32 [B,H,J] (NULL: blocks in
 *   index order), the order in which the query blocks of each (b, h) are
 *   processed -- a permutation of 0..J-1 (entries outside [0, J) are
 *   skipped); vsa_pool_route_topk can produce one that raises cache reuse.
 *   Results do not depend on it.
 *
 * mode BSA_SEL_TOKEN (NSA; [NSA] "Torch朴素实现"): query head hq of token t
 *   reads KV head hq / G (G = Hq / Hkv) and attends to the tokens
 *   blk*BS + u (u < BS, < N, and <= t when causal) of the blocks
 *   blk_idx[b,t,hkv,p] for p < blk_cnt[b,t,hkv] with blk >= 0.  blk_cnt may be
 *   NULL (all S entries count).  Fields: blk_idx int32 [B,N,Hkv,S] contiguous,
 *   blk_cnt int32 [B,N,Hkv] contiguous, S, BS, causal.
 *
 * Both modes: out = softmax(scale * q k^T) v over the allowed keys, a row with
 * no allowed key gives 0 (and lse = -inf).  lse (optional, NULL: none) is fp32
 * [B, Hq, N] contiguous, natural log.  q/out use dq/dout, k/v use dkv.
 * Supported: D in {64, 128}.  dt = BF16 runs on the matrix cores (bf16
 * products, fp32 accumulation and softmax, bf16 output); dt = F32 (block mode
 * only) is computed entirely in fp32 on the vector ALUs and meant for small
 * problems.  VSA block capacity M in {16, 32, 64, 128}; NSA (bf16 only) block
 * size BS in {16, 32, 64, 128}, S <= 64.  Capacity 128 runs as 64-token
 * halves of every block (the same keys per query, so the same attention; the
 * halves' index tables go in the workspace) and takes no summaries and no
 * coarse branch.  Block mode in bf16 addresses one (batch,
 * head) K/V slice with 32-bit byte offsets: it needs N < 2^24, a token stride
 * (dkv.sN) below 2^23 elements and (N - 1) * dkv.sN + D below 2^31 elements;
 * anything larger returns BSA_ERR_UNSUPPORTED.
 *
 * Workspace: bsa_qouter_ws() bytes (256-byte aligned, caller-owned, contents
 * undefined after the call; 0 bytes in token mode and for fp32 at capacity
 * <= 64).  Block mode in bf16 keeps the work counters of its persistent grid
 * there (cleared by a kernel on `stream` before every launch), so two calls
 * with different workspaces can run concurrently on different streams;
 * capacity 128 adds its half tables (B*H*2J*(2*kmax + 2) + 2J int32), so its
 * size depends on the shapes.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  bsa_tdesc dq, dkv, dout;
  bsa_dtype dt;
  float scale;
  int mode;
  /* BSA_SEL_BLOCK */
  const int32_t* perm;
  const int32_t* block_len;
  int J, M;
  const int32_t* q2k_idx;
  const int32_t* q2k_num;
  int kmax;
  /* BSA_SEL_TOKEN */
  const int32_t* blk_idx;
  const int32_t* blk_cnt;
  int S, BS, causal;
  /* optional */
  float* lse;
  const int32_t* item_order;
  /* optional, BSA_SEL_BLOCK: Spark-Reweight summaries from spark_summaries
   * ([Spark] sections 03 and 08).  When set, every block j of (b, h) that no
   * kept entry of query block i names adds one virtual token to the same
   * softmax: logit scale * q . k_sum[b,h,j,:] + b_sum[b,h,j], value
   * v_sum[b,h,j,:].  k_sum, v_sum bf16 [B, H, J, D] and b_sum fp32 [B, H, J],
   * contiguous; all three or none.  Needs bf16, M = 64 and J <= 4096. */
  const void* k_sum;
  const void* v_sum;
  const float* b_sum;
  /* optional, BSA_SEL_BLOCK: coarse pooled-V branch ([VSA] section 6.7).  When
   * set, every token a of query block i gets, before the bf16 rounding,
   *   out[b, a, h, :] += gate[h, :] * coarse[b, h, i, :]
   * with coarse fp32 [B, H, J, D] from vsa_coarse and gate fp32 [H, D], both
   * contiguous and 16-byte aligned; both or neither. */
  const float* coarse;
  const float* gate;
  /* optional, BSA_SEL_BLOCK: per-(b, h) tables, as in vsa_route_args (0:
   * shared); not with summaries. */
  int64_t perm_bh_stride;
  /* optional, BSA_SEL_BLOCK, 0 <= order_long <= J: the first order_long
   * positions of every (b, h)'s processing order (item_order, or block index
   * order) are processed before every other item, across all (b, h); the rest
   * follow (b, h) by (b, h).  For query blocks with far longer kept lists than
   * the others (the H3 context rows keep every block), so that none of them
   * starts late and runs alone at the end.  0: (b, h) by (b, h).  Results do
   * not depend on it. */
  int order_long;
} bsa_qouter_args;

bsa_status bsa_qouter_ws(const bsa_qouter_args* a, size_t* bytes);
bsa_status bsa_forward_qouter(const bsa_qouter_args* a, void* ws, size_t ws_bytes, void* stream);

/* bsa_forward_qouter for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, kernels and results, with no workspace argument.  The scratch
 * it needs (the persistent grid's work counters, the bsa_qouter_ws() bytes)
 * is a static device array of 256 KiB inside the library, one per device,
 * held until the process ends; the call allocates nothing (no hipMalloc, no
 * allocating library routine).  Every call on a device shares that device's
 * array and clears it on `stream` before use, so calls that overlap on one
 * device race (their work counters mix and outputs may be left unwritten):
 * order such calls on one stream.  A request whose scratch would exceed the
 * static array returns BSA_ERR_UNSUPPORTED. */
bsa_status bsa_forward_qouter_static(const bsa_qouter_args* a, void* stream);

/* ----------------------------------------------------------------------------
 * Coarse pooled-V branch ([VSA] section 6.7, with the pooling of section 2.1).
 *
 * For every batch b, head h and query block i:
 *   vbar_j = (1/n_j) * sum_{r < n_j} V[b, perm[j*M + r], h, :]
 *   C[b,h,i,:] = sum_j softmax_j(E[b,h,i,:]) vbar_j      (over all J blocks)
 * E is the fp32 [B, H, J, J] score matrix of vsa_pool_route_topk (or any
 * finite scores of that layout).  The branch is merged into the attention
 * output by bsa_forward_qouter (fields coarse and gate).
 *   v        strided view (dtype dt: bf16 or fp32) [B, N, H, D]
 *   perm, block_len  tiling tables of J blocks of capacity M
 *   E        fp32 [B, H, J, J] contiguous input
 *   vbar     optional fp32 [B, H, J, D] contiguous output (NULL: workspace)
 *   C        fp32 [B, H, J, D] contiguous output
 * Supported: D in {64, 128}, B*H <= 65535; C, vbar and the workspace 16-byte
 * aligned.  The softmax weights and the sums are fp32; the products weight x
 * vbar take both factors as a bf16 pair hi + lo (hi*hi + hi*lo + lo*hi, within
 * 3 * 2^-18 of each product).  The workspace (always needed: vsa_coarse_ws()
 * bytes, caller-owned, contents undefined after the call) holds vbar when it
 * is not an output and the transposed bf16 hi/lo copy of vbar.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* v;
  bsa_tdesc d;
  bsa_dtype dt;
  const int32_t* perm;
  const int32_t* block_len;
  int J, M;
  const float* E;
  float* vbar;
  float* C;
} vsa_coarse_args;

bsa_status vsa_coarse_ws(const vsa_coarse_args* a, size_t* bytes);
bsa_status vsa_coarse(const vsa_coarse_args* a, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Spark-Reweight block summaries ([Spark] sections 07 and 08).
 *
 * For every batch b and head h, with the representative query
 * a = anchor[b,h,:] (NULL: the mean of q[b,n,h,:] over all N tokens, computed
 * here), and every block j of the tiling (its n_j tokens t = perm[j*M + r]):
 *   s_r = scale * a . k_t,  p_r = exp(s_r) / sum_r exp(s_r),  l_j = log sum_r exp(s_r)
 *   k_sum[b,h,j,:] = bf16(sum_r p_r k_t)      v_sum[b,h,j,:] = bf16(sum_r p_r v_t)
 *   b_sum[b,h,j]   = l_j - scale * a . k_sum[b,h,j,:]   (with the stored bf16 key)
 * so that a query q sees block j through one virtual token with logit
 * scale * q . k_sum + b_sum and value v_sum; at q = a it carries the block's
 * exact exponential mass and content.
 *   q, k, v     bf16 [B, N, H, D] strided views sharing the descriptor d
 *               (q is read only when anchor is NULL)
 *   anchor      optional fp32 [B, H, D] contiguous input
 *   anchor_out  optional fp32 [B, H, D] contiguous output: the anchor used
 *   k_sum, v_sum bf16 [B, H, J, D] contiguous; b_sum fp32 [B, H, J] contiguous
 * Supported: D in {64, 128}, 1 <= M <= 64, 16-byte aligned tensors.  The
 * workspace (only when anchor is NULL) holds the partial sums of the anchor:
 * spark_summaries_ws() bytes.  The anchor is reduced in a fixed order, so
 * results are deterministic.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  bsa_tdesc d;
  bsa_dtype dt;
  const int32_t* perm;
  const int32_t* block_len;
  int J, M;
  float scale;
  const float* anchor;
  float* anchor_out;
  void* k_sum;
  void* v_sum;
  float* b_sum;
} spark_summary_args;

bsa_status spark_summaries_ws(const spark_summary_args* a, size_t* bytes);
bsa_status spark_summaries(const spark_summary_args* a, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Spark-Reblock key layout ([Spark] sections 04, 05, 06).
 *
 * For every batch b and head h (the key layout, reused by the queries):
 *   M_Q = Q^T Q / N (uncentred, fp32), L = chol(M_Q + lam I) with
 *   lam = ridge * tr(M_Q) / D (ridge when the trace is 0; a pivot that fp32
 *   rounding pushes below lam is clamped to lam);
 *   u_j = z_j / |z_j|, z_j = k_j^T L (0 for a zero key), rounded to fp16:
 *   cos(u_i, u_j) is the cosine of keys i and j's score profiles over all
 *   queries;
 *   an equal-capacity binary tree of leaves of M tokens: a node of n tokens
 *   spans c = ceil(n/M) leaves, its first child takes floor(c/2)*M of them;
 *   at each split the node's tokens (in their current order, the root in
 *   token order) give 32 landmarks at ranks floor((2s+1) n / 64), the top
 *   principal direction of the centred landmarks (16 power iterations on
 *   their Gram matrix from the ramp s - 15.5; largest entry positive), and
 *   are stably sorted by u . v (fp32); the first child is the first part.
 *   perm[(b*H + h)*J*M + j*M + r] = token r of leaf j (left to right), -1 past
 *   N; block_len[j] = M except the last leaf's N - (J-1)*M.  Use the tables
 *   with perm_bh_stride = J*M in vsa_pool_route_topk and bsa_forward_qouter.
 *   q, k       bf16 [B, N, H, D] views sharing the descriptor d; D in {64, 128},
 *              strides multiples of 8 elements, 16-byte aligned
 *   M          16, 32 or 64; J = ceil(N / M) <= 65536; B*H <= 65535
 *   ridge      > 0 (1e-4 is the documented default)
 *   moment, factor  optional fp32 [B*H, D, D] outputs (factor lower-triangular)
 *   features        optional fp32 [B*H, N, D] output: the unit features as
 *                   the splits use them (stored in fp16 in the workspace)
 *   levels          optional int32 [nlevels, B*H, N]: the token order after
 *                   every level (level 0 = token order), for checking
 *   dirs            optional fp32 [nlevels - 1, B*H, S, D], S = 2^(nlevels-2):
 *                   the split direction of node (slot) s of every level
 *                   (entries of nodes that do not split are left untouched)
 * spark_reblock_dims (host only): J and the number of levels for N and M.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* q;
  const void* k;
  bsa_tdesc d;
  bsa_dtype dt;
  int M;
  float ridge;
  int32_t* perm;
  int32_t* block_len;
  float* moment;
  float* factor;
  float* features;
  int32_t* levels;
  float* dirs;
} spark_reblock_args;

bsa_status spark_reblock_dims(int N, int M, int* J, int* nlevels);
bsa_status spark_reblock_ws(const spark_reblock_args* a, size_t* bytes);
bsa_status spark_reblock(const spark_reblock_args* a, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * KV-outer schedule ([MSA] sections 5-8).
 *
 * Selections q2k int32 [B, N, Hkv, k_sel] contiguous (entries < 0 skipped;
 * with q2k_cnt int32 [B, N, Hkv], only p < q2k_cnt[...] count).  For query
 * position i and KV head r, the valid entries taken in increasing block order
 * get slots s = 0, 1, ...; nslot[b,i,r] is their number.
 *
 * bsa_forward_kvouter:
 *   1. reverse index: for every (b, r, kv block) the list of (i, s) selecting it
 *      (count, exclusive scan, scatter);
 *   2. scheduler: each list is cut into chunks of at most chunk_cap query
 *      positions (0: 2 * k_sel * BK; any cap above B * N * Hkv * k_sel, the
 *      bound on the number of edges, acts as that bound), so hot blocks
 *      spread over workgroups; results do not depend on the cap;
 *   3. K1: per chunk, the K/V tile of the block is staged once and the gathered
 *      queries (G heads per position) attend to it with a local softmax:
 *        L_s = log sum_{j in J_s} exp S_j,  O_s = sum_{j in J_s} exp(S_j - L_s) v_j,
 *      S_j = scale * q . k_j over the block's keys (<= i when causal).  Results
 *      go to the preassigned slot: o_buf[b,s,i,hq,:] (bf16) and
 *      lse_buf[b,s,i,hq] (fp32), so no accumulation and no atomics touch them.
 *      An empty J_s gives L_s = -inf and O_s = 0.
 *   q [B,N,Hq,D] and k/v [B,N,Hkv,D] strided, bf16, D = 128 or 64, BK in {16, 32, 64, 128}
 *   (16 and 32 run in 64-key tiles with the keys past the block masked).
 *   o_buf bf16 [B, k_sel, N, Hq, D], lse_buf fp32 [B, k_sel, N, Hq] and
 *   nslot int32 [B, N, Hkv], all contiguous, live until bsa_combine.  Slots at
 *   or beyond nslot are left untouched.
 *
 * bsa_combine (K2, [MSA] section 6.2): for every (b, i, hq), over s < nslot:
 *   a = max L_s, L = a + log sum exp(L_s - a), out = sum_s exp(L_s - L) O_s;
 *   out = 0 and L = -inf when there is no slot or all L_s are -inf.
 *   out is a bf16 strided view [B, N, Hq, D]; lse (optional) fp32 [B, Hq, N].
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  bsa_tdesc dq, dkv;
  bsa_dtype dt;
  float scale;
  int causal;
  const int32_t* q2k;
  const int32_t* q2k_cnt;
  int k_sel, BK;
  void* o_buf;
  float* lse_buf;
  int32_t* nslot;
  int chunk_cap;
} bsa_kvouter_args;

bsa_status bsa_kvouter_ws(const bsa_kvouter_args* a, size_t* bytes);
bsa_status bsa_forward_kvouter(const bsa_kvouter_args* a, void* ws, size_t ws_bytes, void* stream);

/* Where bsa_forward_kvouter leaves the reverse index and the schedule of steps
 * 1 and 2 inside its workspace ([MSA] section 5: the q2k -> k2q CSR; section 7:
 * the chunk list).  Unlike the rest of the workspace, these regions hold, after
 * the call and until the workspace is reused, with rows = B * Hkv * NB,
 * NB = ceil(N / BK), reverse rows in (b, r, block) order:
 *   count  int32 [rows]        edges per reverse row;
 *   rowptr int32 [rows + 1]    exclusive prefix sum of count;
 *   nchunk int32 [1]           number of chunks;
 *   chunks int32x4 [nchunk]    {row, begin, end, 0}: a run of at most
 *                              chunk_cap edges of one row, rows in order;
 *   edges  int32x2 [rowptr[rows]]  {query position i, slot s}, each row's
 *                              edges between rowptr[row] and rowptr[row + 1]
 *                              in an unspecified order.
 * A block entirely after position i (block * BK > i) under the causal rule
 * keeps its slot but has no edge.  Offsets are in bytes from the workspace
 * start (each 256-byte aligned); `bytes` equals bsa_kvouter_ws; chunk_cap is
 * the effective cap (the argument's, or its default, bounded by max_edges).
 * Same validation and errors as bsa_kvouter_ws.  For inspection and tests of
 * the schedule; the call reads no device memory. */
typedef struct {
  int64_t rows;        /* reverse-index rows B * Hkv * NB */
  int64_t max_edges;   /* B * N * Hkv * k_sel */
  int64_t max_chunks;  /* bound on nchunk */
  int64_t chunk_cap;
  size_t off_count, off_rowptr, off_nchunk, off_chunks, off_edges;
  size_t bytes;
} bsa_kvouter_layout;

bsa_status bsa_kvouter_index_layout(const bsa_kvouter_args* a, bsa_kvouter_layout* out);

typedef struct {
  const void* o_buf;
  const float* lse_buf;
  const int32_t* nslot;
  int k_sel;
  int Hkv;
  bsa_tdesc dout;
  void* out;
  float* lse;
} bsa_combine_args;

bsa_status bsa_combine(const bsa_combine_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
