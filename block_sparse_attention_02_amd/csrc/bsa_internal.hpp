// Host-side declarations shared between the C-ABI layer (api.hip) and the
// kernel translation units.  Every launcher enqueues on `stream` and returns
// the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// ---- tiling -----------------------------------------------------------------
hipError_t launch_tile_index(int T, int H, int W, int bT, int bH, int bW, int J, int M,
                             int32_t* perm, int32_t* block_len, int32_t* inv, hipStream_t s);

// ---- pool / route / TopK ------------------------------------------------------
struct PoolParams {
  const void* q;
  const void* k;
  int64_t sB, sN, sH;
  int B, H, D, J, M;
  const int32_t* perm;
  const int32_t* block_len;
  float* qbar;  // [B, H, J, D]
  float* kbar;
  int64_t perm_bh_stride;  // elements between the tables of consecutive (b, h); 0: one shared table
};
// `vec`: D, strides and base pointers allow 16-byte vector loads.  ntensors:
// 2 pools q and k, 1 pools q only.
hipError_t launch_pool(const PoolParams& p, bool f32_input, bool vec, hipStream_t s, int ntensors = 2);

// Coarse branch: C[bh, i, :] = sum_j softmax_j(E[bh, i, :]) vbar[bh, j, :].
struct CoarseParams {
  const float* E;     // [BH, J, J]
  const float* vbar;  // [BH, J, D]
  float* C;           // [BH, J, D]
  int BH, J, D;
  __bf16* vt;         // [2, BH, D, coarse_jpad(J)]: V_bar transposed, bf16 hi then lo parts, zero padded
};
__host__ __device__ inline int coarse_jpad(int J) { return (J + 63) / 64 * 64; }
hipError_t launch_coarse(const CoarseParams& p, hipStream_t s);

struct RouteParams {
  const float* qbar;  // [B, H, J, D]
  const float* kbar;
  int B, H, J, D, R, kmax;
  float scale;
  int32_t* q2k_idx;  // [B, H, J, kmax]
  int32_t* q2k_num;  // [B, H, J]
  float* E;          // optional [B, H, J, J]
  // Sub-problem (grouped routing): query blocks [row0, row0 + nrows) against
  // key blocks [col0, col0 + ncols), R of them written (as global ids) to
  // entries [out_off, out_off + R) of each row; `tail` also writes the -1
  // fill and q2k_num = R.  The whole square: 0, J, 0, J, 0, 1.
  int row0, nrows, col0, ncols, out_off, tail;
  // Scratch of route_planes_bytes(B*H, ncols, D) bytes (D = 64, 128, 256):
  // the launch first writes the pooled keys of the column range there as bf16
  // hi/lo planes in matrix-core operand order.
  __bf16* kplanes;
};
// Largest J the fused route + TopK kernel handles.
constexpr int kRouteMaxJ = 4096;
size_t route_planes_bytes(int BH, int ncols, int D);
hipError_t launch_route_topk(const RouteParams& p, hipStream_t s);

// ---- Spark-Reblock ------------------------------------------------------------------
struct ReblockParams {
  const void* q;  // bf16 [B, N, H, D] views sharing strides
  const void* k;
  int64_t sB, sN, sH;
  int B, H, N, D, M;
  float ridge;
  float* part;      // [ceil(N/2048), BH, D, D] partial moments
  float* moment;    // optional [BH, D, D]
  float* factor;    // [BH, D, D]
  _Float16* features;   // [BH, N, D] fp16 unit features
  float* features32;  // optional fp32 copy of the same values
  float* dirs;      // [BH, max slots, D]
  float* dirs_out;  // optional [nlevels - 1, BH, max slots, D]: every level's directions
  uint64_t* keys0;  // [BH*N] each: sort composites (projection key << 32 | position)
  uint64_t* keys1;
  int32_t* order0;
  int32_t* order1;
  int32_t* levels;     // optional [nlevels, BH, N]
  int32_t* perm;       // [BH, J*M]
  int32_t* block_len;  // [J]
};
int reblock_levels(int N, int M);
hipError_t launch_reblock(const ReblockParams& p, hipStream_t s);

// ---- H3 multi-region layout and grouped routing ------------------------------
constexpr int kH3MaxParts = 16;
struct H3Part {
  int video;       // 0: dense chunks, 1: 3D-tiled video
  int tok0;        // first original position of the segment
  int b0, b1;      // its block range in the layout
  int n;           // dense: token count
  int T, H, W, JH, JW;
};
struct H3Layout {
  int nparts, M, bT, bH, bW;
  H3Part part[kH3MaxParts];  // in layout order (dense chunks first)
};
hipError_t launch_h3_tile_index(const H3Layout& L, int J, int32_t* perm, int32_t* block_len, int32_t* inv,
                                hipStream_t s);
// Rows < num_prefix: every block; other rows: blocks [0, num_prefix), the
// region entries already written at [num_prefix, nsel), then -1 when `fill`;
// q2k_num.
hipError_t launch_h3_fill(int32_t* q2k_idx, int32_t* q2k_num, int BH, int J, int kmax, int num_prefix, int nsel,
                          bool fill, hipStream_t s);
// Processing order of the query blocks of every (b, h): Morton order of the
// quartile entries of their kept lists ([B*H, J] int32 output).
hipError_t launch_item_order(const int32_t* q2k_idx, const int32_t* q2k_num, int BH, int J, int kmax, int num_first,
                             int32_t* order, hipStream_t s);

// ---- Spark-Reweight summaries -------------------------------------------------
struct SummaryParams {
  const void* k;
  const void* v;
  int64_t sB, sN, sH;
  int B, H, D, J, M;
  const int32_t* perm;
  const int32_t* block_len;
  const float* anchor;  // [B, H, D]
  float scale;
  void* k_sum;   // bf16 [B, H, J, D]
  void* v_sum;   // bf16 [B, H, J, D]
  float* b_sum;  // [B, H, J]
};
// Partial-sum buffer of the anchor reduction (bytes).
size_t anchor_workspace_bytes(int B, int N, int H, int D);
// anchor[b, h, :] = mean over the N tokens of q[b, :, h, :] (bf16 input).
hipError_t launch_anchor(const void* q, int64_t sB, int64_t sN, int64_t sH, int B, int N, int H, int D, float* part,
                         float* anchor, hipStream_t s);
hipError_t launch_summaries(const SummaryParams& p, hipStream_t s);

// ---- query-outer attention -----------------------------------------------------
struct VsaAttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_sB, q_sN, q_sH;
  int64_t kv_sB, kv_sN, kv_sH;
  int64_t o_sB, o_sN, o_sH;
  const int32_t* perm;
  const int32_t* block_len;
  const int32_t* q2k_idx;
  const int32_t* q2k_num;
  int B, H, J, M, kmax, D;
  int64_t N;
  float scale_log2;  // softmax scale * log2(e)
  float* lse;        // optional [B, H, N]
  const int32_t* order;  // optional [B, H, J] processing order of query blocks
  // optional Spark-Reweight summaries (M = 64, bf16): [B, H, J, D] bf16 and [B, H, J]
  const void* k_sum;
  const void* v_sum;
  const float* b_sum;
  // optional coarse branch (M = 64, bf16): out += gate[h, :] * C[b, h, i, :]
  const float* coarse;  // [B, H, J, D]
  const float* gate;    // [H, D]
  int64_t perm_bh_stride;  // elements between the perm tables of consecutive (b, h); 0: shared
  void* sched;             // scheduler state of the persistent grid (qouter_sched_bytes(), 256-byte aligned)
  uint32_t* err;           // sticky index-error flag of the device (a kept id >= J sets it)
  int order_long;          // leading order positions of every (b, h) taken first, across all (b, h)
};
// Bytes of the persistent-grid scheduler state the block-mode kernels use.
size_t qouter_sched_bytes();
hipError_t launch_vsa_attention(const VsaAttnParams& p, bool f32_io, hipStream_t s);
// Block capacity 128 as pairs of 64-token halves (same tokens, same perm
// table): query block i becomes halves 2i and 2i+1, both with the kept list
// of i, and kept block j becomes halves 2j and 2j+1; half lengths min(n, 64)
// and n - min(n, 64).  Writes q2k2 [BH, 2J, 2*kmax], num2 [BH, 2J],
// blen2 [2J] and, when order is given, order2 [BH, 2J].
hipError_t launch_expand_halves(const int32_t* q2k, const int32_t* num, const int32_t* blen, const int32_t* order,
                                int BH, int J, int kmax, int32_t* q2k2, int32_t* num2, int32_t* blen2,
                                int32_t* order2, hipStream_t s);

struct NsaAttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_sB, q_sN, q_sH;
  int64_t kv_sB, kv_sN, kv_sH;
  int64_t o_sB, o_sN, o_sH;
  const int32_t* blk_idx;  // [B, N, Hkv, S]
  const int32_t* blk_cnt;  // [B, N, Hkv] or null
  int B, Hq, Hkv, S, BS, causal, D;
  int64_t N;
  float scale_log2;
  float* lse;  // optional [B, Hq, N]
  uint32_t* err;  // sticky index-error flag (a block id past the sequence sets it)
};
hipError_t launch_nsa_attention(const NsaAttnParams& p, bool f32_io, hipStream_t s);

// ---- KV-outer schedule -----------------------------------------------------------
struct KvOuterParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sB, q_sN, q_sH;
  int64_t kv_sB, kv_sN, kv_sH;
  const int32_t* q2k;      // [B, N, Hkv, ks]
  const int32_t* q2k_cnt;  // [B, N, Hkv] or null
  int B, Hq, Hkv, ks, BK, D, causal, chunk_cap;
  int64_t N;
  float scale_log2;
  __bf16* o_buf;   // [B, ks, N, Hq, D]
  float* lse_buf;  // [B, ks, N, Hq]
  int32_t* nslot;  // [B, N, Hkv]
  uint32_t* err;   // sticky index-error flag (a block id past the sequence sets it)
};
size_t kvouter_ws_bytes(const KvOuterParams& p);
hipError_t launch_kvouter(const KvOuterParams& p, void* ws, hipStream_t s);

struct CombineParams {
  const __bf16* o_buf;
  const float* lse_buf;
  const int32_t* nslot;
  int B, Hq, Hkv, ks, D;
  int64_t N;
  __bf16* out;
  int64_t o_sB, o_sN, o_sH;
  float* lse;  // optional [B, Hq, N]
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

// ---- index errors ----------------------------------------------------------------
// Records that a kernel met a block id outside its table: the lowest active
// lane of the calling wave sets the flag (lanes may call it divergently); the
// flag only ever goes from 0 to 1 until bsa_check clears it.
__device__ __forceinline__ void flag_index_error(uint32_t* err) {
  const uint64_t active = __builtin_amdgcn_read_exec();
  if (err != nullptr && (int)(threadIdx.x & 63) == __builtin_ctzll(active))
    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace bsa
