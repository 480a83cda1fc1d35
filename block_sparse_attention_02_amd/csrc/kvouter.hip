// KV-outer schedule for gfx950: reverse index, scheduler, K1 partial attention
// and the K2 log-sum-exp combine.
//
// Source: "MSA 为什么采用 KV-outer Sparse Attention Forward" -- section 5 (the
// reverse sparse index: count queries per (KV head, KV block), prefix sum into
// row pointers, scatter query ids), section 7 (hot KV tiles are cut into query
// chunks of bounded size; every (query, block) partial gets a preassigned slot
// s in [0, k) so no atomic accumulation is needed and the result is
// deterministic), section 6.1 (K1: per slot, L_s = log sum_j exp S_j and
// O_s = sum_j exp(S_j - L_s) V_j over the block's visible keys, written to
// O_buf[s, i, h] and LSE_buf[s, i, h]), section 6.2 (K2: a = max_s L_s,
// L = a + log sum_s exp(L_s - a), O = sum_s exp(L_s - L) O_s) and section 4
// (queries selecting the same block are concatenated into 128-row tiles that
// share one K/V tile).
//
// Slot rule (the page leaves it open): slot s of (query i, KV head r) is the
// rank of the block among the row's valid selections in increasing block order
// (ties by position), which also fixes the summation order of the combine.
#include <algorithm>

#include "bsa.h"
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

#define BSA_BARRIER() asm volatile("s_barrier" ::: "memory")

namespace {

struct KvLayout {
  int rows;          // B * Hkv * NB reverse-index rows
  int64_t emax;      // upper bound of edges
  int max_chunks;    // upper bound of K1 work items
  size_t off_count, off_cursor, off_rowptr, off_nchunk, off_chunks, off_edges, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunk capacity: the caller's (0: 2 * k * BK), at most the edge bound, so
// that begin + cap never overflows an int in the scan.
int64_t kv_chunk_cap(const KvOuterParams& p) {
  const int64_t emax = std::max<int64_t>(1, (int64_t)p.B * p.N * p.Hkv * p.ks);
  const int64_t cap = p.chunk_cap > 0 ? p.chunk_cap : 2 * (int64_t)p.ks * p.BK;
  return std::min(cap, emax);
}

KvLayout kv_layout(const KvOuterParams& p) {
  KvLayout L{};
  const int64_t NB = (p.N + p.BK - 1) / p.BK;
  L.rows = (int)(p.B * p.Hkv * NB);
  L.emax = (int64_t)p.B * p.N * p.Hkv * p.ks;
  const int64_t cap = kv_chunk_cap(p);
  L.max_chunks = (int)(L.rows + (L.emax + cap - 1) / cap);
  size_t o = 0;
  L.off_count = o;  o += align256((size_t)L.rows * 4);
  L.off_cursor = o; o += align256((size_t)L.rows * 4);
  L.off_rowptr = o; o += align256((size_t)(L.rows + 1) * 4);
  L.off_nchunk = o; o += align256(4);
  L.off_chunks = o; o += align256((size_t)L.max_chunks * 16);
  L.off_edges = o;  o += align256((size_t)L.emax * 8);
  L.total = o;
  return L;
}

}  // namespace

size_t kvouter_ws_bytes(const KvOuterParams& p) { return kv_layout(p).total; }

// Offsets of the reverse index and chunk list inside the workspace, for
// bsa_kvouter_index_layout.
void kvouter_index_layout(const KvOuterParams& p, bsa_kvouter_layout* out) {
  const KvLayout L = kv_layout(p);
  *out = bsa_kvouter_layout{L.rows,      L.emax,       L.max_chunks, kv_chunk_cap(p), L.off_count,
                            L.off_rowptr, L.off_nchunk, L.off_chunks, L.off_edges,     L.total};
}

// ----------------------------------------------------------------------------
__global__ void kv_clear_kernel(int32_t* __restrict__ a, int32_t* __restrict__ b, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    a[i] = 0;
    b[i] = 0;
  }
}

// Slot of entry p of a selection row: rank among the valid entries in
// increasing block order, ties by position.
__device__ __forceinline__ int kv_slot(const int32_t* row, int cnt, int NB, int p, int blk) {
  int s = 0;
  for (int q = 0; q < cnt; ++q) {
    const int o = row[q];
    if (o < 0 || o >= NB) continue;
    s += (o < blk || (o == blk && q < p)) ? 1 : 0;
  }
  return s;
}

// One thread per (b, i, r): count edges per reverse-index row, write nslot,
// and write the empty partial (L = -inf, O = 0) of blocks that lie entirely
// after the query when causal.
__global__ void kv_count_kernel(KvOuterParams p, int NB, int32_t* __restrict__ count) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.N * p.Hkv;
  if (tid >= total) return;
  const int r = (int)(tid % p.Hkv);
  const int64_t bi = tid / p.Hkv;
  const int64_t i = bi % p.N;
  const int b = (int)(bi / p.N);
  const int32_t* row = p.q2k + tid * p.ks;
  const int cnt = p.q2k_cnt ? min(p.q2k_cnt[tid], p.ks) : p.ks;
  const int G = p.Hq / p.Hkv;
  int nvalid = 0;
  for (int q = 0; q < cnt; ++q) {
    const int blk = row[q];
    if (blk >= NB) flag_index_error(p.err);
    if (blk < 0 || blk >= NB) continue;
    ++nvalid;
    if (p.causal && (int64_t)blk * p.BK > i) {
      const int s = kv_slot(row, cnt, NB, q, blk);
      const int64_t base = (((int64_t)b * p.ks + s) * p.N + i) * p.Hq + (int64_t)r * G;
      for (int h = 0; h < G; ++h) {
        p.lse_buf[base + h] = -INFINITY;
        for (int d = 0; d < p.D; ++d) p.o_buf[(base + h) * p.D + d] = (__bf16)0.f;
      }
    } else {
      atomicAdd(&count[((int64_t)b * p.Hkv + r) * NB + blk], 1);
    }
  }
  p.nslot[tid] = nvalid;
}

// Single workgroup: exclusive scan of the counts into row pointers, then the
// chunk list.  Each row is cut into ceil(count / cap) chunks of at most `cap`
// edges; chunks[c] = {row, begin, end, 0}; nchunk = number of chunks.
__global__ __launch_bounds__(1024) void kv_scan_kernel(const int32_t* __restrict__ count, int rows, int cap,
                                                       int32_t* __restrict__ rowptr, int32_t* __restrict__ nchunk,
                                                       int4* __restrict__ chunks) {
  __shared__ int part[1024];
  __shared__ int cpart[1024];
  const int tid = threadIdx.x;
  const int per = (rows + 1023) / 1024;
  const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int s = 0, sc = 0;
  for (int r = r0; r < r1; ++r) {
    s += count[r];
    sc += count[r] / cap + (count[r] % cap != 0);  // ceil without overflow for any cap
  }
  part[tid] = s;
  cpart[tid] = sc;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = tid >= o ? part[tid - o] : 0;
    const int c = tid >= o ? cpart[tid - o] : 0;
    __syncthreads();
    part[tid] += a;
    cpart[tid] += c;
    __syncthreads();
  }
  int e = part[tid] - s;    // exclusive prefix of this thread's first row
  int ce = cpart[tid] - sc;
  for (int r = r0; r < r1; ++r) {
    rowptr[r] = e;
    const int n = count[r];
    for (int64_t c0 = 0; c0 < n; c0 += cap)
      chunks[ce++] = make_int4(r, e + (int)c0, e + (int)std::min<int64_t>(n, c0 + cap), 0);
    e += n;
  }
  if (tid == 1023) {
    rowptr[rows] = part[1023];
    *nchunk = cpart[1023];
  }
}

// One thread per (b, i, r): scatter (position, slot) edges into the rows.
__global__ void kv_scatter_kernel(KvOuterParams p, int NB, const int32_t* __restrict__ rowptr,
                                  int32_t* __restrict__ cursor, int2* __restrict__ edges) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.N * p.Hkv;
  if (tid >= total) return;
  const int r = (int)(tid % p.Hkv);
  const int64_t bi = tid / p.Hkv;
  const int64_t i = bi % p.N;
  const int b = (int)(bi / p.N);
  const int32_t* row = p.q2k + tid * p.ks;
  const int cnt = p.q2k_cnt ? min(p.q2k_cnt[tid], p.ks) : p.ks;
  for (int q = 0; q < cnt; ++q) {
    const int blk = row[q];
    if (blk < 0 || blk >= NB) continue;
    if (p.causal && (int64_t)blk * p.BK > i) continue;
    const int s = kv_slot(row, cnt, NB, q, blk);
    const int64_t rid = ((int64_t)b * p.Hkv + r) * NB + blk;
    const int at = rowptr[rid] + atomicAdd(&cursor[rid], 1);
    edges[at] = make_int2((int)i, s);
  }
}

// ----------------------------------------------------------------------------
// Reverse index with per-workgroup histograms.  A workgroup of 1024 threads
// takes 1024 consecutive (i, r) selection rows of one batch entry and counts
// their edges per (r, block) bin in LDS; only one global atomic per non-empty
// bin and workgroup follows (instead of one per edge: every row holds the sink
// block and popular blocks collect thousands of edges).  The scatter pass
// recounts, reserves each bin's range with one global atomic and writes its
// edges at the reserved offset plus an LDS rank.  The order of edges inside a
// row then depends on atomic order; K1 results do not (each edge writes its
// own slot).  Used when Hkv * NB fits kIndexBins.
// ----------------------------------------------------------------------------
constexpr int kIndexBins = 8192;
constexpr int kIndexRows = 1024;

template <bool SCATTER>
__global__ __launch_bounds__(1024) void kv_index_kernel(KvOuterParams p, int NB, int32_t* __restrict__ count,
                                                        const int32_t* __restrict__ rowptr,
                                                        int32_t* __restrict__ cursor, int2* __restrict__ edges) {
  __shared__ int hist[kIndexBins];
  __shared__ int rank[SCATTER ? kIndexBins : 1];
  const int nbins = p.Hkv * NB;
  const int64_t rows_b = (int64_t)p.N * p.Hkv;
  const int64_t per_b = (rows_b + kIndexRows - 1) / kIndexRows;
  const int b = (int)(blockIdx.x / per_b);
  const int64_t rr = (blockIdx.x % per_b) * kIndexRows + threadIdx.x;  // row within batch entry b
  for (int x = threadIdx.x; x < nbins; x += blockDim.x) {
    hist[x] = 0;
    if constexpr (SCATTER) rank[x] = 0;
  }
  __syncthreads();
  const bool live = rr < rows_b;
  const int64_t tid = (int64_t)b * rows_b + rr;  // global (b, i, r) row
  const int r = (int)(rr % p.Hkv);
  const int64_t i = rr / p.Hkv;
  const int32_t* row = p.q2k + tid * p.ks;
  const int cnt = live ? (p.q2k_cnt ? min(p.q2k_cnt[tid], p.ks) : p.ks) : 0;
  const int G = p.Hq / p.Hkv;
  int nvalid = 0;
  for (int q = 0; q < cnt; ++q) {
    const int blk = row[q];
    if (!SCATTER && blk >= NB) flag_index_error(p.err);
    if (blk < 0 || blk >= NB) continue;
    ++nvalid;
    if (p.causal && (int64_t)blk * p.BK > i) {
      if constexpr (!SCATTER) {  // empty partial of a block entirely after the query
        const int s = kv_slot(row, cnt, NB, q, blk);
        const int64_t base = (((int64_t)b * p.ks + s) * p.N + i) * p.Hq + (int64_t)r * G;
        for (int h = 0; h < G; ++h) {
          p.lse_buf[base + h] = -INFINITY;
          for (int d = 0; d < p.D; ++d) p.o_buf[(base + h) * p.D + d] = (__bf16)0.f;
        }
      }
      continue;
    }
    atomicAdd(&hist[r * NB + blk], 1);
  }
  if constexpr (!SCATTER) {
    if (live) p.nslot[tid] = nvalid;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < nbins; x += blockDim.x) {
    const int c = hist[x];
    if (c == 0) continue;
    const int64_t rid = ((int64_t)b * p.Hkv + x / NB) * NB + x % NB;
    if constexpr (SCATTER)
      hist[x] = rowptr[rid] + atomicAdd(&cursor[rid], c);
    else
      atomicAdd(&count[rid], c);
  }
  if constexpr (SCATTER) {
    __syncthreads();
    for (int q = 0; q < cnt; ++q) {
      const int blk = row[q];
      if (blk < 0 || blk >= NB) continue;
      if (p.causal && (int64_t)blk * p.BK > i) continue;
      const int x = r * NB + blk;
      const int at = hist[x] + atomicAdd(&rank[x], 1);
      edges[at] = make_int2((int)i, kv_slot(row, cnt, NB, q, blk));
    }
  }
}

// ----------------------------------------------------------------------------
// K1 on 16x16x32 MFMAs.  One workgroup of 8 waves per chunk stages the
// block's K and V tiles (BK x D) in LDS once; every wave then walks its own
// 16-row tiles of the chunk's flat (edge, head) row list -- with G = 16 one
// tile is one edge: one query position and its 16 heads -- with no further
// barrier:
//   S^T (BK keys x 16 rows) = K Q^T     v_mfma_f32_16x16x32_bf16
//   single-pass softmax per row over the block's visible keys
//   O^T (D x 16 rows)       = V^T P^T   v_mfma_f32_16x16x32_bf16
// Lane l owns row l%16 and keys 16kt + 4(l/16) + i of S^T; the 8 weights of
// a 32-key step are the B operand of the PV product as they lie (V rows are
// read in the matching order).  K and V rows are padded in LDS (K by 16
// bytes, V by 32) rather than swizzled: both reads are then bank-conflict
// free and every operand address is a per-lane base plus a constant.  The next tile's query rows are loaded into
// the operand registers right after the QK^T product that frees them, the
// edge list two tiles ahead, so the gathers overlap the softmax and PV.
// ----------------------------------------------------------------------------
template <int D, int BK>
struct K1w {
  static constexpr int NW = 8;                     // waves per workgroup
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int KT = BK / 16;               // 16-key tiles of S^T
  static constexpr int KS = D / 32;                // 32-channel k-steps of QK^T
  static constexpr int DT = D / 16;                // 16-channel tiles of O^T
  static constexpr int US = BK / 32;               // 32-key k-steps of PV
  static constexpr int KSE = D + 8;                // K row stride in LDS (elements)
  static constexpr int VSE = D + 16;               // V row stride in LDS (elements)
  static constexpr int SK = CPR + 1, SV = CPR + 2; // 16-byte slots per padded row
  static constexpr int NIK = BK * SK / 64;         // staging copies (64 slots each)
  static constexpr int NIV = BK * SV / 64;
  static_assert(KT % 2 == 0 && DT % 2 == 0 && (BK * SK) % 64 == 0 && (BK * SV) % 64 == 0, "K1 shape");
};

// Stage a block's rows into an LDS tile of `slots` 16-byte slots per row:
// copy ii (of ni, spread over the waves) fills the 64 consecutive slots
// [64 ii, 64 ii + 64); a slot maps back to (row, chunk), and slots in a row's
// padding copy chunk 0 (never read).
template <int CPR>
__device__ __forceinline__ void k1_stage(const __bf16* src, int64_t row_stride, int64_t k0, int nkeys, __bf16* lds,
                                         int slots, int ni, int w, int nw, int lane) {
  for (int ii = w; ii < ni; ii += nw) {
    const int sl = ii * 64 + lane;
    const int row = sl / slots, c = sl % slots;
    const int64_t pos = k0 + min(row, nkeys - 1);
    global_to_lds16(src + pos * row_stride + (c < CPR ? c : 0) * 8, lds + (size_t)ii * 64 * 8);
  }
}

// Edge and head of flat row f of a chunk (G heads per edge).
struct K1Row {
  int qpos, slot, hq;
};

template <int D, int BK>
__global__ __launch_bounds__(512) void kv_k1w_kernel(KvOuterParams p, int NB, const int32_t* __restrict__ nchunk,
                                                     const int4* __restrict__ chunks, const int2* __restrict__ edges) {
  using SH = K1w<D, BK>;
  constexpr int CPR = SH::CPR;
  __shared__ __align__(1024) __bf16 Ks[BK * SH::KSE];
  __shared__ __align__(1024) __bf16 Vs[BK * SH::VSE];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, jl = lane & 15;
  if ((int)blockIdx.x >= *nchunk) return;
  const int4 ck = chunks[blockIdx.x];
  const int rid = ck.x, e0 = ck.y, e1 = ck.z;
  const int blk = rid % NB;
  const int r = (rid / NB) % p.Hkv;
  const int b = rid / (NB * p.Hkv);
  const int G = p.Hq / p.Hkv;
  // block size p.BK <= BK (16 and 32 run in 64-key tiles with the rest masked)
  const int64_t k0 = (int64_t)blk * p.BK;
  const int nkeys = (int)min((int64_t)p.BK, p.N - k0);

  const __bf16* __restrict__ kg = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_sB + r * p.kv_sH;
  const __bf16* __restrict__ vg = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_sB + r * p.kv_sH;
  k1_stage<CPR>(kg, p.kv_sN, k0, nkeys, Ks, SH::SK, SH::NIK, w, SH::NW, lane);
  k1_stage<CPR>(vg, p.kv_sN, k0, nkeys, Vs, SH::SV, SH::NIV, w, SH::NW, lane);
  wait_vmcnt<0>();
  __syncthreads();

  const int64_t nrows = (int64_t)(e1 - e0) * G;
  const int ntile = (int)((nrows + 15) / 16);
  const __bf16* __restrict__ qbase = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sB;
  // flat row f = edge * G + head; shifts when G is a power of two (uniform)
  const int lg_g = ((G & (G - 1)) == 0) ? __builtin_ctz(G) : -1;
  auto row_of = [&](int t, int2 ed) {
    const int64_t f = min((int64_t)t * 16 + jl, nrows - 1);
    const int head = (lg_g >= 0) ? (int)(f & (G - 1)) : (int)(f % G);
    return K1Row{ed.x, ed.y, r * G + head};
  };
  auto edge_of = [&](int t) {
    const int64_t f = min((int64_t)t * 16 + jl, nrows - 1);
    return edges[e0 + ((lg_g >= 0) ? (f >> lg_g) : f / G)];
  };
  auto load_q = [&](bf16x8* qop, const K1Row& rw) {
    const __bf16* qrow = qbase + (int64_t)rw.qpos * p.q_sN + (int64_t)rw.hq * p.q_sH;
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * g);
  };

  // The query rows of a wave's tiles t, t+NW, ... are gathered two tiles
  // ahead into two register sets used in turn; edge records three ahead.
  int2 ea = edge_of(min(w, ntile - 1));
  int2 eb = edge_of(min(w + SH::NW, ntile - 1));
  int2 ec = edge_of(min(w + 2 * SH::NW, ntile - 1));
  bf16x8 qa[SH::KS], qb[SH::KS];
  load_q(qa, row_of(min(w, ntile - 1), ea));
  __builtin_amdgcn_sched_barrier(0);
  // Output of a tile is written one tile later, right after the next QK^T and
  // before the next query gather, so at every QK^T the gathered rows are the
  // youngest memory operations in flight and the wait for them never waits
  // for stores.  Every load and store is unconditional (a tail row beyond the
  // chunk recomputes the chunk's last row and writes the same values), and the
  // first "pending" output is zeros written to the wave's own first tile,
  // which the real values overwrite later in program order.
  u32x4 pend[SH::DT / 2];
#pragma unroll
  for (int m = 0; m < SH::DT / 2; ++m) pend[m] = u32x4{0u, 0u, 0u, 0u};
  float pend_lse = -INFINITY;
  int64_t pend_obase;
  {
    const K1Row r0w = row_of(min(w, ntile - 1), ea);
    pend_obase = (((int64_t)b * p.ks + r0w.slot) * p.N + r0w.qpos) * p.Hq + r0w.hq;
  }
  auto store_pending = [&]() {
    __bf16* orow = p.o_buf + pend_obase * D;
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int m = 0; m < SH::DT / 2; ++m) {
      const int ch = odd ? 32 * m + 16 + 4 * (g - 1) : 32 * m + 4 * g;
      *reinterpret_cast<u32x4*>(orow + ch) = pend[m];
    }
    p.lse_buf[pend_obase] = pend_lse;  // the four lanes of a row write the same value
  };
  // Same memory-operation history on entry as around the loop: gather,
  // (zero) output of the pending tile, gather of the other register set.
  store_pending();
  load_q(qb, row_of(min(w + SH::NW, ntile - 1), eb));
  __builtin_amdgcn_sched_barrier(0);
  // One tile: t with edge ed_cur and query rows qop; afterwards qop holds the
  // rows of tile t + 2NW (edge ed_two); returns the edge of tile t + 3NW.
  auto tile = [&](const int t, const int2 ed_cur, bf16x8* qop, const int2 ed_two) -> int2 {
    const K1Row rw = row_of(t, ed_cur);

    // ---- S^T over all BK keys (operands read PF products ahead) ----
    constexpr int PF = 2;
    constexpr int NQ = SH::KT * SH::KS;
    f32x4 sacc[SH::KT];
#pragma unroll
    for (int kt = 0; kt < SH::KT; ++kt)
#pragma unroll
      for (int x = 0; x < 4; ++x) sacc[kt][x] = 0.f;
    {
      bf16x8 ka[NQ];
#pragma unroll
      for (int x = 0; x < NQ + PF; ++x) {
        if (x < NQ) {
          const int kt = x / SH::KS, s = x % SH::KS;
          const int krow = 16 * kt + jl;
          ka[x] = *reinterpret_cast<const bf16x8*>(Ks + krow * SH::KSE + (4 * s + g) * 8);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (x >= PF) {
          const int y = x - PF;
          sacc[y / SH::KS] = mfma16(ka[y], qop[y % SH::KS], sacc[y / SH::KS]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
    // ---- next tile's operands: edges two tiles ahead, query rows one ahead ----
    const int2 ed_far = edge_of(min(t + 3 * SH::NW, ntile - 1));
    store_pending();
    load_q(qop, row_of(min(t + 2 * SH::NW, ntile - 1), ed_two));
    __builtin_amdgcn_sched_barrier(0);  // keep the gathers here, ahead of the softmax

    // ---- single-pass softmax (log2 domain) with the causal / tail mask ----
    // keys [0, lim) of the block are visible to this row; the masking pass
    // runs only when some row of the tile does not see the whole block
    const int lim = p.causal ? (int)max((int64_t)0, min((int64_t)nkeys, (int64_t)rw.qpos - k0 + 1)) : nkeys;
    if (__builtin_amdgcn_ballot_w64(lim < BK) != 0) {
#pragma unroll
      for (int kt = 0; kt < SH::KT; ++kt)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int key = 16 * kt + 4 * g + x;
          sacc[kt][x] = (key < lim) ? sacc[kt][x] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < SH::KT; ++kt)
#pragma unroll
      for (int x = 0; x < 4; ++x) mx = fmaxf(mx, sacc[kt][x]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, xor32(mx));
    const float m_use = (mx == -INFINITY) ? 0.f : mx * p.scale_log2;
    float rs = 0.f, rsx = 0.f;
    bf16x8 pop[SH::US];
#pragma unroll
    for (int u = 0; u < SH::US; ++u) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kt = 2 * u + (e >> 1), x = 2 * (e & 1);
        pk[e] = pack2_bf16_sum<true>(fast_exp2(__builtin_fmaf(sacc[kt][x], p.scale_log2, -m_use)),
                                     fast_exp2(__builtin_fmaf(sacc[kt][x + 1], p.scale_log2, -m_use)), &rs, &rsx);
      }
      pop[u] = __builtin_bit_cast(bf16x8, pk);
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += xor32(rs);
    rsx += __shfl_xor(rsx, 16, 64);
    rsx += xor32(rsx);

    // ---- O^T = V^T P^T ----
    f32x4 oacc[SH::DT];
#pragma unroll
    for (int dt = 0; dt < SH::DT; ++dt)
#pragma unroll
      for (int x = 0; x < 4; ++x) oacc[dt][x] = 0.f;
    {
      constexpr int NV = SH::US * SH::DT;
      bf16x8 va[NV];
#pragma unroll
      for (int x = 0; x < NV + PF; ++x) {
        if (x < NV) {
          const int u = x / SH::DT, dt = x % SH::DT;
          const int col = 16 * dt + 4 * (jl & 3);
          const int r0 = 32 * u + 4 * g + (jl >> 2);
          const int r1 = r0 + 16;
          const bf16x4 lo = lds_read_tr16(Vs + r0 * SH::VSE + col);
          const bf16x4 hi = lds_read_tr16(Vs + r1 * SH::VSE + col);
          va[x] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        if (x >= PF) {
          const int y = x - PF;
          oacc[y % SH::DT] = mfma16(va[y], pop[y / SH::DT], oacc[y % SH::DT]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }

    // ---- normalised partial and its log-sum-exp into the edge's slot ----
    // Lanes g and g^1 trade halves so that every lane writes 16 bytes: even g
    // writes channels 32m + 4g .. +7 of tile pair m, odd g channels
    // 32m + 16 + 4(g-1) .. +7.  One row swap (v_permlane16_swap: the odd
    // 16-lane rows of the first operand trade with the even rows of the
    // second) does the exchange: afterwards an even row holds (its v0, the
    // odd row's v0) and an odd row (the even row's v1, its v1).
    const float inv = (rs > 0.f) ? 1.f / rs : 0.f;
    pend_obase = (((int64_t)b * p.ks + rw.slot) * p.N + rw.qpos) * p.Hq + rw.hq;
#pragma unroll
    for (int m = 0; m < SH::DT / 2; ++m) {
      const bf16x4 v0 = {(__bf16)(oacc[2 * m][0] * inv), (__bf16)(oacc[2 * m][1] * inv),
                         (__bf16)(oacc[2 * m][2] * inv), (__bf16)(oacc[2 * m][3] * inv)};
      const bf16x4 v1 = {(__bf16)(oacc[2 * m + 1][0] * inv), (__bf16)(oacc[2 * m + 1][1] * inv),
                         (__bf16)(oacc[2 * m + 1][2] * inv), (__bf16)(oacc[2 * m + 1][3] * inv)};
      const uint2 a = __builtin_bit_cast(uint2, v0), c = __builtin_bit_cast(uint2, v1);
      const auto sx = __builtin_amdgcn_permlane16_swap(a.x, c.x, false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(a.y, c.y, false, false);
      pend[m] = u32x4{sx[0], sy[0], sx[1], sy[1]};
    }
    pend_lse = (rsx > 0.f) ? (m_use + __log2f(rsx)) * kLn2 : -INFINITY;
    return ed_far;
  };
  for (int t = w; t < ntile; t += 2 * SH::NW) {
    const int2 ed3 = tile(t, ea, qa, ec);
    if (t + SH::NW >= ntile) break;
    const int2 ed4 = tile(t + SH::NW, eb, qb, ed3);
    ea = ec;
    eb = ed3;
    ec = ed4;
  }
  if (w < ntile) store_pending();  // the wave's last tile
}

template <int D, int BK>
static hipError_t launch_k1(const KvOuterParams& p, int NB, const KvLayout& L, char* ws, hipStream_t s) {
  kv_k1w_kernel<D, BK><<<dim3(L.max_chunks), dim3(64 * K1w<D, BK>::NW), 0, s>>>(
      p, NB, reinterpret_cast<const int32_t*>(ws + L.off_nchunk), reinterpret_cast<const int4*>(ws + L.off_chunks),
      reinterpret_cast<const int2*>(ws + L.off_edges));
  return hipGetLastError();
}

hipError_t launch_kvouter(const KvOuterParams& p, void* wsv, hipStream_t s) {
  const KvLayout L = kv_layout(p);
  char* ws = static_cast<char*>(wsv);
  const int NB = (int)((p.N + p.BK - 1) / p.BK);
  int32_t* count = reinterpret_cast<int32_t*>(ws + L.off_count);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.off_cursor);
  int32_t* rowptr = reinterpret_cast<int32_t*>(ws + L.off_rowptr);
  int32_t* nchunk = reinterpret_cast<int32_t*>(ws + L.off_nchunk);
  int4* chunks = reinterpret_cast<int4*>(ws + L.off_chunks);
  int2* edges = reinterpret_cast<int2*>(ws + L.off_edges);
  const int cap = (int)kv_chunk_cap(p);

  kv_clear_kernel<<<dim3(min(1024, (L.rows + 255) / 256)), dim3(256), 0, s>>>(count, cursor, L.rows);
  const int64_t threads = (int64_t)p.B * p.N * p.Hkv;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  const bool lds_index = (int64_t)p.Hkv * NB <= kIndexBins;
  const unsigned igrid = (unsigned)(p.B * (((int64_t)p.N * p.Hkv + kIndexRows - 1) / kIndexRows));
  if (lds_index)
    kv_index_kernel<false><<<dim3(igrid), dim3(kIndexRows), 0, s>>>(p, NB, count, nullptr, nullptr, nullptr);
  else
    kv_count_kernel<<<dim3(grid), dim3(256), 0, s>>>(p, NB, count);
  kv_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(count, L.rows, cap, rowptr, nchunk, chunks);
  if (lds_index)
    kv_index_kernel<true><<<dim3(igrid), dim3(kIndexRows), 0, s>>>(p, NB, nullptr, rowptr, cursor, edges);
  else
    kv_scatter_kernel<<<dim3(grid), dim3(256), 0, s>>>(p, NB, rowptr, cursor, edges);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 128) return p.BK == 128 ? launch_k1<128, 128>(p, NB, L, ws, s) : launch_k1<128, 64>(p, NB, L, ws, s);
  return p.BK == 128 ? launch_k1<64, 128>(p, NB, L, ws, s) : launch_k1<64, 64>(p, NB, L, ws, s);
}

// ----------------------------------------------------------------------------
// K2: one workgroup per (b, position); a thread handles 8 channels of one head.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kv_combine_kernel(CombineParams p) {
  constexpr int SB = 8;  // slots per batch: their loads are all in flight together
  const int64_t bi = blockIdx.x;
  const int64_t i = bi % p.N;
  const int b = (int)(bi / p.N);
  const int G = p.Hq / p.Hkv;
  const int cpr = p.D / 8;
  const int64_t sstride = p.N * p.Hq;  // rows between consecutive slots
  for (int c = threadIdx.x; c < p.Hq * cpr; c += blockDim.x) {
    const int hq = c / cpr, dc = c % cpr;
    const int n = min(p.nslot[((int64_t)b * p.N + i) * p.Hkv + hq / G], p.ks);
    const int64_t row0 = ((int64_t)b * p.ks * p.N + i) * p.Hq + hq;
    // One pass over the slots, SB at a time with all their loads in flight:
    // running maximum m, z = sum_s exp(L_s - m), acc = sum_s exp(L_s - m) O_s,
    // rescaled when m grows; then L = m + log z and O = acc / z, which is the
    // section's merge with weights exp(L_s - L).
    float m = -INFINITY, z = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += SB) {
      bf16x8 o[SB];
      float l[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int64_t row = row0 + (int64_t)min(s0 + u, n - 1) * sstride;
        // each partial is read once: a streaming load keeps it from displacing
        // the rows the other workgroups still need
        o[u] = __builtin_bit_cast(
            bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.o_buf + row * p.D + dc * 8)));
        l[u] = p.lse_buf[row];
      }
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (s0 + u >= n) l[u] = -INFINITY;  // the batch's padding slots
      float bm = l[0];
#pragma unroll
      for (int u = 1; u < SB; ++u) bm = fmaxf(bm, l[u]);
      const float m_new = fmaxf(m, bm);
      if (m_new == -INFINITY) continue;  // nothing visible yet
      const float scale = __expf(m - m_new);  // 0 while m is -inf
      z *= scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= scale;
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const float wgt = __expf(l[u] - m_new);
        z += wgt;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)o[u][e];
      }
      m = m_new;
    }
    const float inv = (z > 0.f) ? 1.f / z : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    const float L = (z > 0.f) ? m + __logf(z) : -INFINITY;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)acc[e];
    *reinterpret_cast<bf16x8*>(p.out + b * p.o_sB + i * p.o_sN + hq * p.o_sH + dc * 8) = out;
    if (p.lse && dc == 0) p.lse[((int64_t)b * p.Hq + hq) * p.N + i] = L;
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  // one (head, 8-channel chunk) item per thread when it fits
  const int items = p.Hq * (p.D / 8);
  const int threads = std::min(1024, (items + 63) / 64 * 64);
  kv_combine_kernel<<<dim3((unsigned)(p.B * p.N)), dim3(threads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsa
