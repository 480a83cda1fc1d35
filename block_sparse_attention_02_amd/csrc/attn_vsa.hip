// Exact block-selected attention, query-outer order (VSA mode), for gfx950.
//
// Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" -- section 4 (a
// query block sees every valid key of each kept block, weights per token),
// section 6.3 (per query block, loop over its q2k_num kept blocks, mask keys at
// or beyond the block's true length, one softmax over the union), section 6.5
// (online softmax in exp2 form: alpha = 2^((m - m')g), P = 2^((S - m')g),
// l' = alpha*l + rowsum P, U' = alpha*U + P V, O = U / l; an empty row gives 0)
// and section 3 (outputs go back to the tokens' original positions).
//
// Design (MI355X): one workgroup per (batch, head, query block); MT/32 waves,
// each owning 32 query rows held in registers as the B operand of
//   S^T (keys x queries) = K Q^T        v_mfma_f32_32x32x16_bf16
//   O^T (channels x queries) += V^T P^T v_mfma_f32_32x32x16_bf16
// With S^T in the 32x32 output layout, lane l owns query l%32, so row maxima
// need a single cross-lane step (lanes l, l^32) and the probabilities of 16
// consecutive keys are exactly the B operand of the next product.  K and V
// tiles (MT keys x D) are gathered through the packing table straight into LDS
// with 16-byte asynchronous copies (no register staging); K is read as rows
// (A operand, ds_read_b128) and V through the transposing LDS read.  Row chunks
// are XOR-swizzled per row so both reads are bank-conflict free.  The copy of
// K for the next kept block overlaps the softmax and PV of the current one,
// the copy of V overlaps the next QK^T.
#include <algorithm>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kMaxRounds = 4096;
// Kept-block bitmask words of the summary mode (J <= 32 * kSumMaskWords).
constexpr int kSumMaskWords = 128;
// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Gated coarse term gate[h, d..d+3] * C[b, h, i, d..d+3] of the pooled-V
// branch ("VSA 实现详解" section 6.7), added to the normalised output of every
// token of query block i; zero when the branch is off.
__device__ __forceinline__ f32x4 coarse_term(const VsaAttnParams& p, int64_t bh, int hh, int i, int d) {
  if (!p.coarse) return f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 c = *reinterpret_cast<const f32x4*>(p.coarse + (bh * p.J + i) * p.D + d);
  const f32x4 g = *reinterpret_cast<const f32x4*>(p.gate + (int64_t)hh * p.D + d);
  return f32x4{g[0] * c[0], g[1] * c[1], g[2] * c[2], g[3] * c[3]};
}

// Workgroup barrier that first retires this wave's outstanding LDS reads, so a
// buffer can be refilled right after it.  Asynchronous global->LDS copies are
// ordered separately with wait_vmcnt<>().
// Workgroup barrier that first retires this wave's outstanding LDS reads, so a
// buffer can be refilled right after it.  Asynchronous global->LDS copies are
// ordered separately with wait_vmcnt<>().
#define BSA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

__device__ __forceinline__ int item_of(const VsaAttnParams& p, int64_t wid, int64_t* bh) {
  // Work item wid -> (b * H + h, query block).  The first order_long
  // positions of every (b, h)'s order come first, across all (b, h) (the
  // longest items start first); then the rest, (b, h) by (b, h).  -1: the
  // order names no block.
  const int nl = p.order_long;
  const int64_t nlong = (int64_t)p.B * p.H * nl;
  int64_t pos;
  if (wid < nlong || nl == p.J) {
    *bh = wid / nl;
    pos = wid % nl;
  } else {
    const int64_t w2 = wid - nlong;
    *bh = w2 / (p.J - nl);
    pos = nl + w2 % (p.J - nl);
  }
  if (!p.order) return (int)pos;
  const int i = as_const(p.order)[*bh * p.J + pos];
  return (i >= 0 && i < p.J) ? i : -1;
}

// Kept entry `pos` of a query block's list: the block id, or -1 when the
// entry names no block.  An id at or beyond J is skipped like a negative one;
// `bad` records it, and the item reports it through the device's index-error
// flag when it ends.
template <typename T>
__device__ __forceinline__ int kept_id(T sel, int pos, int J, bool& bad) {
  const int j = sel[pos];
  bad |= j >= J;
  return j < J ? j : -1;
}

// Physical 16-byte chunk of logical chunk c in K tile row r: 16 consecutive
// rows read at the same logical chunk land on 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int k_swz(int r, int c) {
  return c ^ (r & (CPR >= 16 ? 15 : CPR - 1));
}
// V tile: the transposing read takes 4 consecutive rows x 32 bytes per 16-lane
// group (two groups per 64-byte span); rows r%4 = 0..3 get disjoint chunks.
template <int CPR>
__device__ __forceinline__ int v_swz(int r, int c) {
  if constexpr (CPR >= 16) {
    // XOR pattern {0, 6, 10, 12} for r % 4 = 0..3, packed in nibbles
    return c ^ ((0xCA60 >> (4 * (r & 3))) & 15);
  } else {
    return c ^ (2 * (r & 3));
  }
}

// Copy k of wave w covers the 64 chunks [(w*LPT + k)*64, +64) of the row-major
// tile: lane L takes chunk (w*LPT + k)*64 + L, i.e. row (w*LPT + k)*RPI + L/CPR.
// Wave w therefore copies the 32 consecutive rows [32w, 32w + 32).
template <int D, int MT>
struct TileMap {
  static constexpr int NW = MT / 32;
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per copy instruction
  static constexpr int LPT = MT * CPR / (64 * NW);  // copies per lane per tile
  static_assert(LPT * RPI == 32, "each wave copies 32 rows");
  __device__ static int row(int k, int w, int lane) { return (w * LPT + k) * RPI + lane / CPR; }
  __device__ static int pchunk(int lane) { return lane % CPR; }
};

// Buffer resource of one (batch, head) slice: 32-bit byte offsets from `base`;
// offsets at or beyond `bytes` read as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);  // stride 0
  r[2] = (int)bytes;
  r[3] = 0x00020000;                // raw 32-bit buffer
  return r;
}

// The compiler does not see the memory instruction inside these asm
// statements, so it does not pad the hazards that instruction has with what
// precedes it: an SGPR of the buffer resource written by a VALU instruction
// (v_readlane_b32 when the compiler parks SGPRs in VGPR lanes, or
// v_readfirstlane_b32) needs 5 wait states before a VMEM instruction reads
// it, and M0 written by SALU needs 1 before an LDS DMA.  "s_nop 4" provides 5.
#define BSA_VMEM_SGPR_GUARD "s_nop 4\n\t"

// Asynchronous 16-byte buffer -> LDS copy (lane L lands in slot L of the
// wave's 1 KiB LDS window at `lds_byte_offset`); counted by wait_vmcnt<>().
__device__ __forceinline__ void buffer_to_lds16(i32x4 rsrc, uint32_t voffset, uint32_t lds_byte_offset) {
  asm volatile(
      BSA_VMEM_SGPR_GUARD
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "{m0}"(lds_byte_offset)
      : "memory");
}

// Asynchronous copy of one block's token ids into the wave's 256-byte LDS id
// buffer: lane L copies the id of row L.  Rows at or beyond the block capacity
// read the next block's ids, and reads past the table return zero; both only
// name keys that are masked.  Counted by wait_vmcnt<>() like the tile copies.
__device__ __forceinline__ void stage_ids(i32x4 prs, int j, int M, uint32_t ids_lds, int lane) {
  const uint32_t voff = (uint32_t)(j * M + lane) * 4u;
  asm volatile(
      BSA_VMEM_SGPR_GUARD
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(prs), "{m0}"(ids_lds)
      : "memory");
}

// Byte offsets (within the slice) of the LPT tile rows this lane copies (token
// ids and the row stride are below 2^24, so a 24-bit multiply is exact).  Copy
// k of wave w fills LDS row 32w + RPI*k + sub (sub = lane / CPR) with key
// 32w + LPT*sub + k of the block, so a lane's keys are LPT consecutive entries
// of the id buffer.  Padding ids (-1) read token 0; their keys are masked.
template <int D, int MT>
__device__ __forceinline__ void tile_rows(uint32_t* rowoff, const int* ids, int w, int lane, uint32_t row_bytes) {
  using TM = TileMap<D, MT>;
  const int* src = ids + 32 * w + TM::LPT * (lane / TM::CPR);
#pragma unroll
  for (int q = 0; q < TM::LPT / 4; ++q) {
    const i32x4 v = *reinterpret_cast<const i32x4*>(src + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) rowoff[4 * q + e] = __umul24((uint32_t)max(v[e], 0), row_bytes);
  }
}

// Key (position in the block) held by LDS row 32*kt + rr of a tile.
template <int D, int MT>
__device__ __forceinline__ constexpr int tile_key(int kt, int rr) {
  using TM = TileMap<D, MT>;
  return 32 * kt + TM::LPT * (rr % TM::RPI) + rr / TM::RPI;
}

template <int D, int MT>
__device__ __forceinline__ void stage_tile(i32x4 rsrc, uint32_t lds_base, const uint32_t* rowoff,
                                           const uint32_t* chunkoff, int w) {
  using TM = TileMap<D, MT>;
#pragma unroll
  for (int k = 0; k < TM::LPT; ++k)
    buffer_to_lds16(rsrc, rowoff[k] + chunkoff[k], lds_base + (uint32_t)((w * TM::LPT + k) * 1024));
}

// One query block (work item `wid` = (b*H + h)*J + i).  LSE: also keep the
// exact (unrounded) row sum for the log-sum-exp output.
template <int D, int MT, bool LSE>
__device__ __forceinline__ void vsa_attn_item(const VsaAttnParams& p, int wid_in, __bf16* Ks, __bf16* Vs, int* Ids) {
  const int64_t wid = __builtin_amdgcn_readfirstlane(wid_in);  // uniform by construction
  using TM = TileMap<D, MT>;
  constexpr int LPT = TM::LPT;
  constexpr int KT = MT / 32;   // 32-key tiles per KV tile
  constexpr int KS = D / 16;    // k-steps of QK^T
  constexpr int DT = D / 32;    // 32-channel tiles of O
  constexpr int US = MT / 16;   // 16-key steps of PV
  static_assert(LPT >= 4 && LPT <= 16 && LPT % 4 == 0, "tile copy shape");
  constexpr int PF = 2;         // operand prefetch distance (products)

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5;  // which half of the wave
  int64_t bh;
  const int i = item_of(p, wid, &bh);
  if (i < 0) return;  // not a block index (whole workgroup)
  const int hh = (int)(bh % p.H), b = (int)(bh / p.H);
  const int M = p.M;
  const int32_t* __restrict__ perm = p.perm + bh * p.perm_bh_stride;

  const __bf16* __restrict__ qg = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sB + hh * p.q_sH;
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_sB + hh * p.kv_sH;
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_sB + hh * p.kv_sH;
  const uint32_t row_bytes = (uint32_t)(p.kv_sN * 2);
  const uint32_t slice_bytes = (uint32_t)((p.N - 1) * p.kv_sN * 2 + D * 2);
  const i32x4 krs = make_rsrc(kg, slice_bytes), vrs = make_rsrc(vg, slice_bytes);
  const uint32_t ks_lds = lds_offset(Ks), vs_lds = lds_offset(Vs);

  const auto sel = as_const(p.q2k_idx) + (bh * p.J + i) * p.kmax;
  const auto blen = as_const(p.block_len);
  const int num = min(as_const(p.q2k_num)[bh * p.J + i], p.kmax);
  const int ni = blen[i];

  // per-lane swizzled chunk offsets of the copies (fixed for the whole kernel)
  uint32_t koff[LPT], voff[LPT];
#pragma unroll
  for (int k = 0; k < LPT; ++k) {
    const int r = TM::row(k, w, lane), pc = TM::pchunk(lane);
    koff[k] = (uint32_t)k_swz<TM::CPR>(r, pc) * 16;
    voff[k] = (uint32_t)v_swz<TM::CPR>(r, pc) * 16;
  }

  // ---- query rows: B operand of S^T, lane l holds row 32w + l%32 ----
  const int qrow = 32 * w + (lane & 31);
  const int qtok = max(perm[(int64_t)i * M + max(min(qrow, ni - 1), 0)], 0);  // empty block: token 0, no output
  bf16x8 qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qop[s] = load8_bf16<__bf16>(qg + (int64_t)qtok * p.q_sN + 16 * s + 8 * h2);
  // Consume the query registers here so the compiler waits for their loads
  // before the loop; from here on only the tile copies count against vmcnt.
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qop[s]));

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  // running max in log2 units; lane-partial sums of the rounded (and exact) weights
  float m_run = -INFINITY, l_run = 0.f, lx_run = 0.f;

  // Kept blocks are visited in table order; an entry < 0 is an empty tile
  // (copies of block 0, every key masked), which leaves the result unchanged.
  // Copies in flight, oldest first, at the top of iteration pc:
  //   K(pc) [LPT], ids(pc+1) [1], V(pc) [LPT]
  // ids(pc+1) land before K(pc+1) is staged (after QK^T); V(pc) before PV.
  const i32x4 prs = make_rsrc(perm, (uint32_t)p.J * (uint32_t)M * 4u);
  int* ids = Ids + 64 * w;
  const uint32_t ids_lds = lds_offset(ids);
  uint32_t rows[LPT];
  int nj = 0, njn = 0, jn1 = 0;
  bool bad = false;  // a kept id at or beyond J was met
  if (num > 0) {
    const int j0 = kept_id(sel, 0, p.J, bad);
    nj = (j0 >= 0) ? blen[j0] : 0;
    stage_ids(prs, max(j0, 0), M, ids_lds, lane);
    wait_vmcnt<0>();
    tile_rows<D, MT>(rows, ids, w, lane, row_bytes);
    stage_tile<D, MT>(krs, ks_lds, rows, koff, w);
    jn1 = kept_id(sel, min(1, num - 1), p.J, bad);
    stage_ids(prs, max(jn1, 0), M, ids_lds, lane);
    stage_tile<D, MT>(vrs, vs_lds, rows, voff, w);
  }

  for (int pc = 0; pc < num; ++pc) {
    const bool has_next = pc + 1 < num;
    // ---- K(pc) resident; ids(pc+1) and V(pc) may still be in flight ----
    wait_vmcnt<LPT + 1>();
    BSA_BARRIER();

    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
    {
      // K operands are read PF k-steps ahead of the products that use them,
      // so the LDS latency overlaps the matrix ops.
      bf16x8 ka[KS][KT];
#pragma unroll
      for (int s = 0; s < KS + PF; ++s) {
        if (s < KS) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const int krow = 32 * kt + (lane & 31);
            const int pch = k_swz<TM::CPR>(krow, 2 * s + h2);
            ka[s][kt] = *reinterpret_cast<const bf16x8*>(Ks + krow * D + pch * 8);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, KT, 0);
        }
        if (s >= PF) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) sacc[kt] = mfma32(ka[s - PF][kt], qop[s - PF], sacc[kt]);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, KT, 0);
        }
      }
    }
    BSA_BARRIER();  // every wave is done reading Ks
    if (has_next) {
      wait_vmcnt<LPT>();  // ids(pc+1) resident
      tile_rows<D, MT>(rows, ids, w, lane, row_bytes);
      stage_tile<D, MT>(krs, ks_lds, rows, koff, w);
    }

    // Scalar table reads for the coming iterations are issued here, where no
    // LDS result is awaited until the barrier after the softmax: the block
    // after next (the last one again near the end, a harmless repeat) and the
    // true length of the next block.
    __builtin_amdgcn_sched_barrier(0);
    const int jn2 = kept_id(sel, min(pc + 2, num - 1), p.J, bad);
    njn = (jn1 >= 0) ? blen[max(jn1, 0)] : 0;
    __builtin_amdgcn_sched_barrier(0);

    // ---- online softmax (log2 domain); lane owns query 32w + l%32 ----
    if (nj < MT) {  // edge / short block: mask keys at or beyond its true length
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = tile_key<D, MT>(kt, 8 * (r >> 2) + 4 * h2 + (r & 3));
          sacc[kt][r] = (key < nj) ? sacc[kt][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, xor32(mx)) * p.scale_log2;
    // Lazy rescale: keep the old reference unless some row's maximum grew by
    // more than 8 (probabilities then stay below 2^8); the final O = U / l uses
    // the same reference, so the result is unchanged.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);  // 0 on the first kept block
      l_run *= alpha;
      if constexpr (LSE) lx_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    // Weights are rounded to bf16 once; the row sum uses the rounded values the
    // PV product uses, so O = U / l is an exact convex combination of V rows.
    float rs = 0.f, rsx = 0.f;
    bf16x8 pop[US];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * hlf + 2 * e;
          const float a = fast_exp2(__builtin_fmaf(sacc[kt][r], p.scale_log2, -m_use));
          const float c = fast_exp2(__builtin_fmaf(sacc[kt][r + 1], p.scale_log2, -m_use));
          pk[e] = pack2_bf16_sum<LSE>(a, c, &rs, &rsx);
        }
        pop[2 * kt + hlf] = __builtin_bit_cast(bf16x8, pk);
      }
    l_run += rs;
    if constexpr (LSE) lx_run += rsx;

    // ---- V(j) resident (K of the next block may be in flight) ----
    if (has_next)
      wait_vmcnt<LPT>();
    else
      wait_vmcnt<0>();
    BSA_BARRIER();
    {
      // V operands (two transposing reads each) run PF products ahead.
      const int g16 = lane >> 4, jl = lane & 15;
      constexpr int NP = US * DT;
      bf16x8 va[NP];
#pragma unroll
      for (int x = 0; x < NP + PF; ++x) {
        if (x < NP) {
          const int u = x / DT, dt = x % DT;
          const int d = 32 * dt + 16 * (g16 & 1) + 4 * (jl & 3);
          const int c = d >> 3, off = d & 7;
          const int r0 = 16 * u + 4 * h2 + (jl >> 2);
          const int r1 = r0 + 8;
          const bf16x4 lo = lds_read_tr16(Vs + r0 * D + v_swz<TM::CPR>(r0, c) * 8 + off);
          const bf16x4 hi = lds_read_tr16(Vs + r1 * D + v_swz<TM::CPR>(r1, c) * 8 + off);
          va[x] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        if (x >= PF) {
          const int y = x - PF;
          oacc[y % DT] = mfma32(va[y], pop[y / DT], oacc[y % DT]);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
      }
    }
    BSA_BARRIER();  // every wave is done reading Vs

    if (!has_next) break;
    // ---- advance: ids of the block after next, then V of the next block ----
    nj = njn;
    stage_ids(prs, max(jn2, 0), M, ids_lds, lane);
    stage_tile<D, MT>(vrs, vs_lds, rows, voff, w);
    jn1 = jn2;
  }

  if (bad) flag_index_error(p.err);
  // ---- epilogue: O = U / l, written at the tokens' original positions ----
  const float l_tot = l_run + xor32(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qrow < ni) {
    __bf16* __restrict__ og = reinterpret_cast<__bf16*>(p.o) + b * p.o_sB + (int64_t)qtok * p.o_sN + hh * p.o_sH;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * dt + 8 * jj + 4 * h2;
        const f32x4 cg = coarse_term(p, bh, hh, i, d);
        bf16x4 v4 = {(__bf16)fmaf(oacc[dt][4 * jj + 0], inv, cg[0]), (__bf16)fmaf(oacc[dt][4 * jj + 1], inv, cg[1]),
                     (__bf16)fmaf(oacc[dt][4 * jj + 2], inv, cg[2]), (__bf16)fmaf(oacc[dt][4 * jj + 3], inv, cg[3])};
        *reinterpret_cast<bf16x4*>(og + d) = v4;
      }
    if constexpr (LSE) {
      const float lx = lx_run + xor32(lx_run);
      if (h2 == 0) p.lse[bh * p.N + qtok] = (lx > 0.f) ? (m_run + __log2f(lx)) * kLn2 : -INFINITY;
    }
  }
}

// Persistent grid: workgroup g takes items g, g + G, g + 2G, ...  Every item
// visits the same number of kept blocks, so the resident workgroups advance
// through their sorted block lists roughly in step; at any moment they touch a
// narrow window of each head's K/V, which stays in L2 (workgroups are spread
// over the XCDs round-robin, so each XCD serves every 8th query block of the
// same stretch and all eight share the same window in the last-level cache).
//
// All scheduling state lives in the caller's workspace (one SchedState per
// launch, cleared by clear_sched_kernel on the launch's stream), so launches
// on different streams never share counters.
//
// Progress balancing between the two workgroups that share a CU.  The wave
// arbiter favours the older workgroup (by ~18 % here), which would leave the
// younger one behind at every round boundary; instead each workgroup publishes
// how many tiles it has finished and raises its waves' priority while it
// trails its partner.  Slots are found from the hardware CU id, registered
// once per launch.
//
// Work distribution of the four-wave kernel's persistent grid.  Work items
// (in processing order) are cut into chunks of kChunk; chunk c belongs to XCD
// c % kXcds (found from the hardware XCC id), whose workgroups take its items
// in order, so the workgroups of one XCD run consecutive items together; an
// XCD that has used up its chunks takes items of the others', so a faster XCD
// does more of the work.  The workgroups of one XCD also re-align after every
// item with a bounded wait, so they touch the same window of each head's K/V,
// which then stays in that XCD's L2.  Correctness depends only on the
// per-XCD atomic counters: each item is taken exactly once, whatever the waits
// do.
constexpr int kCuKeys = 2048;  // 8 XCDs x 8 SEs x 2 SHs x 16 CUs
constexpr int kXcds = 8;
constexpr int kChunk = 64;  // items per chunk; chunk c belongs to XCD c % kXcds

struct SchedState {
  uint32_t xq[kXcds];                      // items taken from each XCD's chunks
  uint32_t registered;                     // workgroups that joined their cohort
  uint32_t xcd_members[kXcds];
  uint32_t xcd_exited[kXcds];
  uint32_t round_ctr[kMaxRounds];          // two-wave kernel: arrivals per round
  uint32_t cu_slots[kCuKeys];              // workgroups registered per CU
  uint32_t cu_progress[kCuKeys * 2];       // finished tiles per (CU, slot)
  uint32_t xcd_rounds[kXcds * kMaxRounds]; // four-wave kernel: arrivals per (XCD, item)
};

size_t qouter_sched_bytes() { return (sizeof(SchedState) + 255) & ~(size_t)255; }

// Clears the scheduling state before a launch (grid-stride over every word).
__global__ void clear_sched_kernel(SchedState* st) {
  uint32_t* w = reinterpret_cast<uint32_t*>(st);
  constexpr int n = (int)(sizeof(SchedState) / 4);
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < n; r += gridDim.x * blockDim.x) w[r] = 0u;
}

__device__ __forceinline__ uint32_t load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Cohort {
  uint32_t xcc = 0, members = 0;
  int round = 0;
};

// Join this XCD's cohort; waits (bounded) until every workgroup of the grid
// has joined so the member count is final.
__device__ __forceinline__ Cohort cohort_register(SchedState* st, uint32_t* sh) {
  if (threadIdx.x == 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (15 << 11)) & (kXcds - 1);  // XCC_ID
    __hip_atomic_fetch_add(&st->xcd_members[xcc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&st->registered, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int t = 0; t < 4096; ++t) {
      if (load_relaxed(&st->registered) >= gridDim.x) break;
      __builtin_amdgcn_s_sleep(8);
    }
    sh[0] = xcc;
    sh[1] = load_relaxed(&st->xcd_members[xcc]);
  }
  __syncthreads();
  Cohort c;
  c.xcc = __builtin_amdgcn_readfirstlane(sh[0]);
  c.members = __builtin_amdgcn_readfirstlane(sh[1]);
  __syncthreads();
  return c;
}

// Arrive at the end of round c.round and wait (bounded) for the cohort's
// other members, counting those that have already run out of work (called by
// one lane of the workgroup).
__device__ __forceinline__ void cohort_arrive_wait(SchedState* st, const Cohort& c) {
  if (c.round >= kMaxRounds) return;
  uint32_t* ctr = &st->xcd_rounds[c.xcc * kMaxRounds + c.round];
  __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int t = 0; t < 4096; ++t) {
    if (load_relaxed(ctr) + load_relaxed(&st->xcd_exited[c.xcc]) >= c.members) break;
    __builtin_amdgcn_s_sleep(8);
  }
}

// Arrive after a query block and wait for the cohort (whole workgroup).
__device__ __forceinline__ void cohort_sync(SchedState* st, Cohort& c) {
  if (threadIdx.x == 0) cohort_arrive_wait(st, c);
  ++c.round;
  __syncthreads();
}

// The k-th work item of XCD x's chunks (-1 past the end; the valid k form a
// prefix, so a miss means that XCD's chunks are used up).
__device__ __forceinline__ int xcd_item(uint32_t x, uint32_t k, int items) {
  const uint64_t item = ((uint64_t)(k / kChunk) * kXcds + x) * kChunk + (k % kChunk);
  return item < (uint64_t)items ? (int)item : -1;
}

// The next work item for a workgroup of XCD x: from its own chunks in order,
// then from the other XCDs' chunks; -1 when everything is taken.  Every item
// is handed out exactly once (one atomic counter per XCD).
__device__ __forceinline__ int next_item(SchedState* st, uint32_t x, int items, uint32_t* sh) {
  if (threadIdx.x == 0) {
    int it = -1;
    for (uint32_t y = 0; y < (uint32_t)kXcds && it < 0; ++y) {
      const uint32_t xx = (x + y) % kXcds;
      if (xcd_item(xx, load_relaxed(&st->xq[xx]), items) < 0) continue;  // used up already
      it = xcd_item(xx, __hip_atomic_fetch_add(&st->xq[xx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), items);
    }
    sh[0] = (uint32_t)it;
  }
  __syncthreads();
  const int wid = (int)__builtin_amdgcn_readfirstlane(sh[0]);
  __syncthreads();
  return wid;
}

struct Balance {
  uint32_t* mine = nullptr;           // this workgroup's finished-tile count
  const uint32_t* partner = nullptr;  // the other workgroup on the CU
  uint32_t done = 0;
};

// Register this workgroup on its CU (call once, by every thread).
__device__ __forceinline__ Balance balance_register(SchedState* st, uint32_t* slot_sh) {
  Balance bal;
  if (threadIdx.x == 0) {
    const uint32_t hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));   // HW_ID
    const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (15 << 11)) & 7u;  // XCC_ID
    const uint32_t key = (((xcc * 8u + ((hw >> 13) & 7u)) * 2u + ((hw >> 12) & 1u)) * 16u + ((hw >> 8) & 15u));
    const uint32_t slot = __hip_atomic_fetch_add(&st->cu_slots[key], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    slot_sh[0] = key;
    slot_sh[1] = slot;
  }
  __syncthreads();
  const uint32_t key = __builtin_amdgcn_readfirstlane(slot_sh[0]);
  const uint32_t slot = __builtin_amdgcn_readfirstlane(slot_sh[1]);
  if (slot < 2u && key < (uint32_t)kCuKeys) {
    bal.mine = &st->cu_progress[key * 2 + slot];
    bal.partner = &st->cu_progress[key * 2 + (slot ^ 1u)];
  }
  return bal;
}

// Re-align the resident workgroups after each round: arrive, then wait
// (bounded) until every workgroup of the grid has arrived.  The wait only
// affects cache locality, never the result; it gives up after a fixed number
// of polls.
__device__ __forceinline__ void round_sync(SchedState* st, int sync, int wid, int items, int round) {
  if (sync && wid + (int)gridDim.x < items && round < kMaxRounds) {
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(&st->round_ctr[round], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int t = 0; t < 4096; ++t) {
        if (load_relaxed(&st->round_ctr[round]) >= gridDim.x) break;
        __builtin_amdgcn_s_sleep(8);
      }
    }
    __syncthreads();
  }
}

template <int D, int MT, bool LSE>
__global__ __launch_bounds__(2 * MT) __attribute__((amdgpu_waves_per_eu(2, 2))) void vsa_attn_kernel(VsaAttnParams p,
                                                                                                     int items,
                                                                                                     int sync) {
  __shared__ __align__(1024) __bf16 Ks[MT * D];
  __shared__ __align__(1024) __bf16 Vs[MT * D];
  __shared__ __align__(256) int Ids[(MT / 32) * 64];
  int round = 0;
  for (int wid = blockIdx.x; wid < items; wid += gridDim.x, ++round) {
    vsa_attn_item<D, MT, LSE>(p, wid, Ks, Vs, Ids);
    round_sync(reinterpret_cast<SchedState*>(p.sched), sync, wid, items, round);
  }
}


// ============================================================================
// 64-row blocks: four waves per query block.  Wave w = 2*hq + g owns query
// rows [32hq, 32hq + 32) and key half g (keys [32g, 32g + 32) of every kept
// block) with its own online-softmax state; the two key halves are merged
// through LDS once per query block.  K/V tiles are double-buffered: the copies
// of block t+1 are issued right after the single barrier that opens block t,
// so each tile has a whole block of compute to arrive.
// ============================================================================
template <int D>
struct Tile4 {
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per copy instruction
  static constexpr int LPT = 16 / RPI;  // copies per wave per tensor (16 rows)
  static_assert(LPT >= 2 && LPT <= 4 && LPT * RPI == 16, "tile copy shape");
  // LDS row that copy k of wave w fills for this lane
  __device__ static int row(int k, int w, int lane) { return 16 * w + RPI * k + lane / CPR; }
  // Block key held by LDS row rho: copy k of wave w, lane group sub holds key
  // 16w + LPT*sub + k, so a lane's keys are consecutive entries of the ids.
  __device__ static int key_of_row(int rho) {
    const int r = rho & 15;
    return (rho & ~15) + LPT * (r % RPI) + r / RPI;
  }
};

template <int D>
__device__ __forceinline__ void tile_rows4(uint32_t* rowoff, const int* ids, int w, int lane, uint32_t row_bytes) {
  using TM = Tile4<D>;
  const int* src = ids + 16 * w + TM::LPT * (lane / TM::CPR);
  if constexpr (TM::LPT == 4) {
    const i32x4 v = *reinterpret_cast<const i32x4*>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) rowoff[e] = __umul24((uint32_t)max(v[e], 0), row_bytes);
  } else {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 v = *reinterpret_cast<const i32x2*>(src);
#pragma unroll
    for (int e = 0; e < 2; ++e) rowoff[e] = __umul24((uint32_t)max(v[e], 0), row_bytes);
  }
}

template <int D>
__device__ __forceinline__ void stage4(i32x4 rsrc, uint32_t lds_base, const uint32_t* rowoff, const uint32_t* chunkoff,
                                       int w) {
  using TM = Tile4<D>;
#pragma unroll
  for (int k = 0; k < TM::LPT; ++k)
    buffer_to_lds16(rsrc, rowoff[k] + chunkoff[k], lds_base + (uint32_t)((w * TM::LPT + k) * 1024));
}

template <int D, bool LSE, bool SUM>
__device__ __forceinline__ void vsa4_item(const VsaAttnParams& p, int wid_in, __bf16* KV, int* Ids, float* Mx,
                                          Balance& bal, uint32_t* Kept, float* Bsum) {
  using TM = Tile4<D>;
  constexpr int LPT = TM::LPT, CPR = TM::CPR;
  constexpr int KS = D / 16;   // k-steps of QK^T
  constexpr int DT = D / 32;   // 32-channel tiles of O
  constexpr int TILE = 64 * D; // elements of one K or V tile
  constexpr int PF = 2;        // operand prefetch distance (products)
  const int64_t wid = __builtin_amdgcn_readfirstlane(wid_in);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = w >> 1, g = w & 1;  // query half, key half
  const int h2 = lane >> 5;
  int64_t bh;
  const int i = item_of(p, wid, &bh);
  if (i < 0) return;  // not a block index (whole workgroup)
  const int hh = (int)(bh % p.H), b = (int)(bh / p.H);
  constexpr int M = 64;
  const int32_t* __restrict__ perm = p.perm + bh * p.perm_bh_stride;

  const __bf16* __restrict__ qg = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sB + hh * p.q_sH;
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_sB + hh * p.kv_sH;
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_sB + hh * p.kv_sH;
  const uint32_t row_bytes = (uint32_t)(p.kv_sN * 2);
  const uint32_t slice_bytes = (uint32_t)((p.N - 1) * p.kv_sN * 2 + D * 2);
  const i32x4 krs = make_rsrc(kg, slice_bytes), vrs = make_rsrc(vg, slice_bytes);
  const i32x4 prs = make_rsrc(perm, (uint32_t)p.J * (uint32_t)M * 4u);
  const uint32_t kv_lds = lds_offset(KV);
  // buffer x: K tile at kv_lds + x*4*TILE bytes, V tile TILE*2 bytes after it
  auto kbuf = [&](int x) { return kv_lds + (uint32_t)(x * 4 * TILE); };
  auto vbuf = [&](int x) { return kv_lds + (uint32_t)(x * 4 * TILE + 2 * TILE); };

  const auto sel = as_const(p.q2k_idx) + (bh * p.J + i) * p.kmax;
  const auto blen = as_const(p.block_len);
  const int num = min(as_const(p.q2k_num)[bh * p.J + i], p.kmax);
  const int ni = blen[i];

  // Spark-Reweight summaries: after the kept blocks come ceil(J/64) tiles of
  // 64 virtual tokens (summary key, value and bias of blocks 64*tau ..);
  // those of kept blocks and those past J are masked.  Kept holds the kept
  // list as a bitmask, Bsum the biases of the next tile (one 64-entry buffer
  // per wave and parity).
  const int ns = SUM ? (p.J + 63) / 64 : 0;
  const int T = num + ns;
  i32x4 ksrs = krs, vsrs = vrs, bsrs = prs;
  const float bias_mul = 1.4426950408889634f / p.scale_log2;  // 1 / scale
  auto bs_lds = [&](int x) { return lds_offset(Bsum + (x * 4 + w) * 64); };
  if constexpr (SUM) {
    const uint32_t sbytes = (uint32_t)p.J * (uint32_t)(D * 2);
    ksrs = make_rsrc(reinterpret_cast<const __bf16*>(p.k_sum) + bh * p.J * D, sbytes);
    vsrs = make_rsrc(reinterpret_cast<const __bf16*>(p.v_sum) + bh * p.J * D, sbytes);
    bsrs = make_rsrc(p.b_sum + bh * p.J, (uint32_t)p.J * 4u);
    for (int x = threadIdx.x; x < kSumMaskWords; x += blockDim.x) Kept[x] = 0u;
    __syncthreads();
    for (int pp = threadIdx.x; pp < num; pp += blockDim.x) {
      const int j = p.q2k_idx[(bh * p.J + i) * p.kmax + pp];
      if (j >= 0 && j < p.J) atomicOr(&Kept[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }
  // byte offsets of the summary rows this lane copies for summary tile tau
  auto sum_rows = [&](uint32_t* r, int tau) {
#pragma unroll
    for (int k = 0; k < TM::LPT; ++k)
      r[k] = (uint32_t)min(64 * tau + 16 * w + TM::LPT * (lane / TM::CPR) + k, p.J - 1) * (uint32_t)(D * 2);
  };

  // byte offsets (from the LDS base) of this lane's V transposing reads per
  // buffer and 32-channel tile: r0 = 32g + 4h2 + (jl >> 2) (the 16-key step u
  // and the second row group add constants)
  uint32_t vtr[2][DT];
  {
    const int g16 = lane >> 4, jl = lane & 15;
    const int r0 = 32 * g + 4 * h2 + (jl >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + 16 * (g16 & 1) + 4 * (jl & 3);
      const int c = d >> 3, off = d & 7;
      const uint32_t e = (uint32_t)((r0 * D + v_swz<CPR>(r0, c) * 8 + off) * 2);
      vtr[0][dt] = kv_lds + (uint32_t)(2 * TILE) + e;
      vtr[1][dt] = kv_lds + (uint32_t)(4 * TILE + 2 * TILE) + e;
    }
  }
  uint32_t koff[LPT], voff[LPT];
#pragma unroll
  for (int k = 0; k < LPT; ++k) {
    const int r = TM::row(k, w, lane), pc = lane % CPR;
    koff[k] = (uint32_t)k_swz<CPR>(r, pc) * 16;
    voff[k] = (uint32_t)v_swz<CPR>(r, pc) * 16;
  }

  // ---- query rows: B operand of S^T, lane l holds row 32hq + l%32 ----
  const int qrow = 32 * hq + (lane & 31);
  const int qtok = max(perm[(int64_t)i * M + max(min(qrow, ni - 1), 0)], 0);  // empty block: token 0, no output
  bf16x8 qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qop[s] = load8_bf16<__bf16>(qg + (int64_t)qtok * p.q_sN + 16 * s + 8 * h2);
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qop[s]));

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f, lx_run = 0.f;

  // Copies in flight at the top of block t: K(t), V(t) [2*LPT] then ids(t+1) [1].
  int* ids = Ids + 64 * w;
  const uint32_t ids_lds = lds_offset(ids);
  uint32_t rows[LPT];
  int nj = 0, njn = 0, j1 = 0, j2 = 0;
  bool bad = false;  // a kept id at or beyond J was met
  if (num > 0) {
    const int j0 = kept_id(sel, 0, p.J, bad);
    nj = (j0 >= 0) ? blen[j0] : 0;
    stage_ids(prs, max(j0, 0), M, ids_lds, lane);
    wait_vmcnt<0>();
    tile_rows4<D>(rows, ids, w, lane, row_bytes);
    stage4<D>(krs, kbuf(0), rows, koff, w);
    stage4<D>(vrs, vbuf(0), rows, voff, w);
    j1 = kept_id(sel, min(1, num - 1), p.J, bad);
    j2 = kept_id(sel, min(2, num - 1), p.J, bad);
    stage_ids(prs, max(j1, 0), M, ids_lds, lane);
  } else if constexpr (SUM) {
    if (T > 0) {  // no kept block: the first tile is summary tile 0
      sum_rows(rows, 0);
      stage4<D>(ksrs, kbuf(0), rows, koff, w);
      stage4<D>(vsrs, vbuf(0), rows, voff, w);
    }
  }
  if constexpr (SUM) {
    if (T > 0) stage_ids(bsrs, max(-num, 0), 64, bs_lds(0), lane);  // biases of tile 0 if it is a summary tile
  }

  constexpr int NCOPY = 2 * LPT + 1 + (SUM ? 1 : 0);  // K and V of the next tile, ids, biases
  static_assert(NCOPY <= KS + PF, "copies are spread over the QK^T steps");
  uint32_t partner_seen = 0;  // partner count, read one block before it is used
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    wait_vmcnt<0>();  // K(t), V(t) and ids(t+1) resident
    BSA_BARRIER();    // every wave's copies visible; every wave done with t-1
    if (bal.mine != nullptr) {
      // Every 4 blocks: act on the partner count read 1 block ago (that read
      // has completed with the wait above), then publish and re-read.
      if ((t & 3) == 1) {
        if (bal.done + 1 < __builtin_amdgcn_readfirstlane(partner_seen))
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
      if ((t & 3) == 0) {
        if (w == 0 && lane == 0) __hip_atomic_store(bal.mine, bal.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        partner_seen = __hip_atomic_load(bal.partner, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      ++bal.done;
    }
    // Rows of block t+1 (for the last block: the same block again, a
    // harmless extra copy into the idle buffer).
    const bool next_sum = SUM && t + 1 >= num;
    if (next_sum)
      sum_rows(rows, t + 1 - num);
    else
      tile_rows4<D>(rows, ids, w, lane, row_bytes);
    const i32x4 ckr = next_sum ? ksrs : krs, cvr = next_sum ? vsrs : vrs;
    const __bf16* Kc = KV + cur * 2 * TILE;
    const __bf16* Vc = Kc + TILE;

    // ---- S^T (32 keys x 32 queries) = K_g Q^T, with the copies of block t+1
    // issued one per product so the memory pipeline sees a steady stream ----
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    {
      const int krow = 32 * g + (lane & 31);
      bf16x8 ka[KS];
#pragma unroll
      for (int s = 0; s < KS + PF; ++s) {
        if (s < KS) {
          ka[s] = *reinterpret_cast<const bf16x8*>(Kc + krow * D + k_swz<CPR>(krow, 2 * s + h2) * 8);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        if (s >= PF) {
          sacc = mfma32(ka[s - PF], qop[s - PF], sacc);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
        if (s < LPT) {
          buffer_to_lds16(ckr, rows[s] + koff[s], kbuf(cur ^ 1) + (uint32_t)((w * LPT + s) * 1024));
        } else if (s < 2 * LPT) {
          buffer_to_lds16(cvr, rows[s - LPT] + voff[s - LPT], vbuf(cur ^ 1) + (uint32_t)((w * LPT + s - LPT) * 1024));
        } else if (s == 2 * LPT) {
          stage_ids(prs, max(j2, 0), M, ids_lds, lane);  // near the end: a harmless repeat
        } else if (SUM && s == 2 * LPT + 1 && next_sum) {
          stage_ids(bsrs, t + 1 - num, 64, bs_lds(cur ^ 1), lane);
        }
      }
    }

    // scalar table reads for the coming blocks (no LDS result is awaited
    // until the barrier that opens the next block)
    __builtin_amdgcn_sched_barrier(0);
    const int j3 = kept_id(sel, max(0, min(t + 3, num - 1)), p.J, bad);
    njn = (j1 >= 0) ? blen[max(j1, 0)] : 0;
    __builtin_amdgcn_sched_barrier(0);

    // ---- online softmax (log2 domain); lane owns query 32hq + l%32 ----
    if constexpr (SUM) {
      if (t >= num) {  // virtual tokens: add the bias; kept blocks and rows past J get -inf
        const int tau = t - num;
        float* bsm = Bsum + (cur * 4 + w) * 64;
        // this wave's own copy of the tile's biases: lane k marks entry k
        const uint32_t word = Kept[2 * tau + (lane >> 5)];
        if (((word >> (lane & 31)) & 1u) != 0u || 64 * tau + lane >= p.J) bsm[lane] = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = TM::key_of_row(32 * g + 8 * (r >> 2) + 4 * h2 + (r & 3));
          sacc[r] = __builtin_fmaf(bsm[key], bias_mul, sacc[r]);
        }
        nj = M;
      }
    }
    if (nj < M) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = TM::key_of_row(32 * g + 8 * (r >> 2) + 4 * h2 + (r & 3));
        sacc[r] = (key < nj) ? sacc[r] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, xor32(mx)) * p.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      if constexpr (LSE) lx_run *= alpha;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f, rsx = 0.f;
    bf16x8 pop[2];
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * hlf + 2 * e;
        const float a = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -m_use));
        const float c = fast_exp2(__builtin_fmaf(sacc[r + 1], p.scale_log2, -m_use));
        pk[e] = pack2_bf16_sum<LSE>(a, c, &rs, &rsx);
      }
      pop[hlf] = __builtin_bit_cast(bf16x8, pk);
    }
    l_run += rs;
    if constexpr (LSE) lx_run += rsx;

    // ---- O^T (D x 32 queries) += V_g^T P^T ----
    {
      uint32_t vbase[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vbase[dt] = cur ? vtr[1][dt] : vtr[0][dt];
      constexpr int NP = 2 * DT;
      bf16x8 va[NP];
#pragma unroll
      for (int x = 0; x < NP + PF; ++x) {
        if (x < NP) {
          const int u = x / DT, dt = x % DT;
          // rows r0 + 16u and r0 + 16u + 8 keep r0's swizzle (same row % 4)
          const uint32_t a = vbase[dt] + (uint32_t)(16 * u * D * 2);
          const bf16x4 lo = lds_read_tr16_at(a);
          const bf16x4 hi = lds_read_tr16_at(a + (uint32_t)(8 * D * 2));
          va[x] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        if (x >= PF) {
          const int y = x - PF;
          oacc[y % DT] = mfma32(va[y], pop[y / DT], oacc[y % DT]);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
      }
    }
    nj = njn;
    j1 = j2;
    j2 = j3;
  }

  if (bad) flag_index_error(p.err);
  // ---- merge the two key halves of each query row through LDS ----
  // Once every wave is past its last tile and its copies have landed, buffer 1
  // is free (the next query block's first copies go to buffer 0).
  wait_vmcnt<0>();
  BSA_BARRIER();
  float* scr = reinterpret_cast<float*>(KV + 2 * TILE) + hq * (64 * DT * 16);
  float* mx_sh = Mx + hq * 3 * 64;
  if (g == 1) {
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 v = {oacc[d][4 * c4], oacc[d][4 * c4 + 1], oacc[d][4 * c4 + 2], oacc[d][4 * c4 + 3]};
        *reinterpret_cast<f32x4*>(scr + ((d * 4 + c4) * 64 + lane) * 4) = v;
      }
    mx_sh[lane] = m_run;
    mx_sh[64 + lane] = l_run;
    mx_sh[128 + lane] = lx_run;
  }
  BSA_BARRIER();
  if (g == 0) {
    const float mb = mx_sh[lane], lb = mx_sh[64 + lane], lxb = mx_sh[128 + lane];
    const float m = fmaxf(m_run, mb);
    const float fa = (m == -INFINITY) ? 0.f : fast_exp2(m_run - m);
    const float fb = (m == -INFINITY) ? 0.f : fast_exp2(mb - m);
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(scr + ((d * 4 + c4) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[d][4 * c4 + e] = fa * oacc[d][4 * c4 + e] + fb * v[e];
      }
    const float l_part = fa * l_run + fb * lb;
    const float l_tot = l_part + xor32(l_part);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow < ni) {
      __bf16* __restrict__ og =
          reinterpret_cast<__bf16*>(p.o) + b * p.o_sB + (int64_t)qtok * p.o_sN + hh * p.o_sH;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int dd = 32 * d + 8 * jj + 4 * h2;
          const f32x4 cg = coarse_term(p, bh, hh, i, dd);
          bf16x4 v4 = {(__bf16)fmaf(oacc[d][4 * jj + 0], inv, cg[0]), (__bf16)fmaf(oacc[d][4 * jj + 1], inv, cg[1]),
                       (__bf16)fmaf(oacc[d][4 * jj + 2], inv, cg[2]), (__bf16)fmaf(oacc[d][4 * jj + 3], inv, cg[3])};
          *reinterpret_cast<bf16x4*>(og + dd) = v4;
        }
      if constexpr (LSE) {
        const float lx_part = fa * lx_run + fb * lxb;
        const float lx = lx_part + xor32(lx_part);
        if (h2 == 0) p.lse[bh * p.N + qtok] = (lx > 0.f) ? (m + __log2f(lx)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <int D, bool LSE, bool SUM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void vsa4_kernel(VsaAttnParams p,
                                                                                             int items, int sync) {
  __shared__ __align__(1024) __bf16 KV[4 * 64 * D];  // 2 buffers x (K, V)
  __shared__ __align__(256) int Ids[4 * 64];         // token ids, one buffer per wave
  __shared__ float Mx[2 * 3 * 64];                   // merge: max, rounded sum, exact sum
  __shared__ uint32_t slot_sh[2];
  __shared__ uint32_t Kept[SUM ? kSumMaskWords : 1];      // kept blocks of the query block (summaries)
  __shared__ __align__(256) float Bsum[SUM ? 2 * 4 * 64 : 1];  // biases of a summary tile, per parity and wave
  SchedState* st = reinterpret_cast<SchedState*>(p.sched);
  Balance bal;
  Cohort coh;
  if (sync) {
    bal = balance_register(st, slot_sh);
    coh = cohort_register(st, slot_sh);
  }
  int wid = sync ? next_item(st, coh.xcc, items, slot_sh) : (int)blockIdx.x;
  while (wid >= 0 && wid < items) {
    vsa4_item<D, LSE, SUM>(p, wid, KV, Ids, Mx, bal, Kept, Bsum);
    if (sync) {
      cohort_sync(st, coh);
      wid = next_item(st, coh.xcc, items, slot_sh);
    } else {
      wid += gridDim.x;
    }
  }
  if (sync && threadIdx.x == 0)
    __hip_atomic_fetch_add(&st->xcd_exited[coh.xcc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_setprio(0);
}

// ============================================================================
// 64-row blocks, ping-pong schedule.  One 8-wave workgroup per CU works on two
// query blocks at a time, one per group of four waves; inside a group the
// waves take the roles of the four-wave kernel (query half hq, key half g).
// Each step of a group is either a matrix phase M_t (PV of kept block t-1,
// then S^T = K Q^T of kept block t) or a vector phase S_t (the online softmax
// of block t, plus the copies of later blocks).  The two groups run half a
// step apart with one workgroup barrier per phase, so while one group's waves
// run their softmax the other group's waves -- on the same SIMDs -- keep the
// matrix cores busy (the SIMD arbiter issues VALU work of one wave during the
// matrix operations of another).
//
// Phases of one query block with T kept blocks:
//   L0 (S)  take the item, query rows, token ids of blocks 0, 1, 2
//   L1 (M)  copies of K(0), V(0), K(1)
//   L2 (S)  (the first copies land)
//   M_0, S_0, M_1, S_1, ..., M_{T-1}, S_{T-1}, M_T
//   E0 (S)  key half 1 hands its partial state to key half 0 through LDS
//   E1 (M)  key half 0 merges, normalises and stores; the next item is taken
// S_s issues, in this order, the token ids of block s+3 and the copies of
// K(s+2) and V(s+1) (entries past the list repeat its last block: harmless
// copies into free buffers).  K(t) lives in Kbuf[t & 1], V(t) in Vbuf[t & 1],
// the ids of block t in slot t & 3 of the wave's id ring.  Before M_s every
// batch but the last has landed, before S_s the ids at the head of the last.
// ============================================================================
// The next work item of the XCD's chunk queue for one group (called by one
// lane; -1 when everything is taken).
__device__ __forceinline__ int pp_next_item(SchedState* st, uint32_t x, int items) {
  for (uint32_t y = 0; y < (uint32_t)kXcds; ++y) {
    const uint32_t xx = (x + y) % kXcds;
    if (xcd_item(xx, load_relaxed(&st->xq[xx]), items) < 0) continue;
    const int it = xcd_item(xx, __hip_atomic_fetch_add(&st->xq[xx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                            items);
    if (it >= 0) return it;
  }
  return -1;
}

template <int D, bool LSE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void vsa_pp_kernel(VsaAttnParams p,
                                                                                              int items) {
  using TM = Tile4<D>;
  constexpr int LPT = TM::LPT, CPR = TM::CPR;
  constexpr int KS = D / 16;    // k-steps of QK^T
  constexpr int DT = D / 32;    // 32-channel tiles of O
  constexpr int NP = 2 * DT;    // PV products
  constexpr int TILE = 64 * D;  // elements of one K or V tile
  constexpr int M = 64;
  constexpr int PF = 2;         // operand prefetch distance (products)
  // per group: Kbuf[0], Kbuf[1], Vbuf[0], Vbuf[1]
  __shared__ __align__(1024) __bf16 KV[2 * 4 * TILE];
  __shared__ __align__(256) int Ids[8 * 4 * 64];  // per wave: a ring of 4 token-id slots
  __shared__ float Mx[2 * 2 * 3 * 64];            // per group and query half: m, l, lx of key half 1
  __shared__ int item_sh[2];                      // next item of each group
  __shared__ int done_at[2];                      // barrier count at which each group ran out of items
  __shared__ uint32_t coh_sh[2];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wv >> 2, ww = wv & 3;
  const int hq = ww >> 1, g = ww & 1, h2 = lane >> 5;
  const bool lead = ww == 0 && lane == 0;
  SchedState* st = reinterpret_cast<SchedState*>(p.sched);
  const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (15 << 11)) & (kXcds - 1);  // XCC_ID

  __bf16* KVg = KV + grp * 4 * TILE;
  const uint32_t kv_lds = lds_offset(KVg);
  auto kbuf = [&](int x) { return kv_lds + (uint32_t)(x * TILE * 2); };
  auto vbuf = [&](int x) { return kv_lds + (uint32_t)((2 + x) * TILE * 2); };
  int* ring = Ids + wv * 4 * 64;
  auto ring_lds = [&](int slot) { return lds_offset(ring + slot * 64); };
  const int krow = 32 * g + (lane & 31);
  const int qrow = 32 * hq + (lane & 31);
  const uint32_t row_bytes = (uint32_t)(p.kv_sN * 2);
  const uint32_t slice_bytes = (uint32_t)((p.N - 1) * p.kv_sN * 2 + D * 2);
  const auto blen = as_const(p.block_len);

  // per-lane swizzled chunk offsets of the copies
  uint32_t koff[LPT], voff[LPT];
#pragma unroll
  for (int k = 0; k < LPT; ++k) {
    const int r = TM::row(k, ww, lane), pc = lane % CPR;
    koff[k] = (uint32_t)k_swz<CPR>(r, pc) * 16;
    voff[k] = (uint32_t)v_swz<CPR>(r, pc) * 16;
  }
  // byte offset (from Vbuf[0]) of this lane's V transposing reads, per 32-channel tile
  uint32_t vtr[DT];
  {
    const int g16 = lane >> 4, jl = lane & 15;
    const int r0 = 32 * g + 4 * h2 + (jl >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + 16 * (g16 & 1) + 4 * (jl & 3);
      const int c = d >> 3, off = d & 7;
      vtr[dt] = vbuf(0) + (uint32_t)((r0 * D + v_swz<CPR>(r0, c) * 8 + off) * 2);
    }
  }

  // Group 0 of every workgroup of an XCD starts its items together with the
  // others (bounded wait), and group 1 follows its group 0 one phase later, so
  // the XCD's query blocks walk their sorted block lists in step and share
  // the head's K/V window in L2.
  const bool sync = p.sched != nullptr;
  Cohort coh;
  if (sync) coh = cohort_register(st, coh_sh);
  if (threadIdx.x == 0 || threadIdx.x == 256) {
    item_sh[grp] = p.sched ? pp_next_item(st, xcc, items) : (int)(2 * blockIdx.x + grp);
    done_at[grp] = 0x7fffffff;
  }
  __syncthreads();

  // Every phase opens with one workgroup barrier; both groups pass the same
  // number of them, group 1 one phase behind group 0, so that the matrix
  // phases of one group meet the vector phases of the other.
  int q = 0;
  auto phase = [&]() {
    BSA_BARRIER();
    ++q;
  };
  if (grp == 1) phase();

  for (;;) {
    // ---------------- L0: take the item, load the query rows, stage ids ----------------
    phase();
    const int wid = __builtin_amdgcn_readfirstlane(item_sh[grp]);
    if (wid < 0 || wid >= items) {
      if (lead) {
        done_at[grp] = q;
        if (sync && grp == 0)
          __hip_atomic_fetch_add(&st->xcd_exited[coh.xcc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
    int64_t bh;
    int i = item_of(p, wid, &bh);
    const bool out_ok = i >= 0;
    if (!out_ok) i = 0;
    const int hh = (int)(bh % p.H), b = (int)(bh / p.H);
    const int32_t* __restrict__ perm = p.perm + bh * p.perm_bh_stride;
    const __bf16* qg = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sB + hh * p.q_sH;
    const i32x4 krs = make_rsrc(reinterpret_cast<const __bf16*>(p.k) + b * p.kv_sB + hh * p.kv_sH, slice_bytes);
    const i32x4 vrs = make_rsrc(reinterpret_cast<const __bf16*>(p.v) + b * p.kv_sB + hh * p.kv_sH, slice_bytes);
    const i32x4 prs = make_rsrc(perm, (uint32_t)p.J * (uint32_t)M * 4u);
    const auto sel = as_const(p.q2k_idx) + (bh * p.J + i) * p.kmax;
    const int T = out_ok ? min(as_const(p.q2k_num)[bh * p.J + i], p.kmax) : 0;
    const int ni = blen[i];
    const int qtok = max(perm[(int64_t)i * M + max(min(qrow, ni - 1), 0)], 0);  // empty block: token 0, no output
    // a query block of at most 32 tokens leaves query half 1 with no row to
    // write: those waves only copy tiles and pass the barriers
    const bool qidle = hq == 1 && ni <= 32;
    bf16x8 qop[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) qop[k] = load8_bf16<__bf16>(qg + (int64_t)qtok * p.q_sN + 16 * k + 8 * h2);
    bool bad = false;
    int j0 = 0, ja = 0, jb = 0, jc = 0;
    if (T > 0) {
      j0 = kept_id(sel, 0, p.J, bad);
      ja = kept_id(sel, min(1, T - 1), p.J, bad);
      jb = kept_id(sel, min(2, T - 1), p.J, bad);
      jc = kept_id(sel, min(3, T - 1), p.J, bad);
      stage_ids(prs, max(j0, 0), M, ring_lds(0), lane);
      stage_ids(prs, max(ja, 0), M, ring_lds(1), lane);
      stage_ids(prs, max(jb, 0), M, ring_lds(2), lane);
    }

    // ---------------- L1: copies of K(0), V(0), K(1) ----------------
    wait_vmcnt<0>();  // query rows and ids have landed
    phase();
#pragma unroll
    for (int k = 0; k < KS; ++k) asm volatile("" ::"v"(qop[k]));
    uint32_t rows_next[LPT];  // rows of the block whose V copy is next
    int nj = 0;
    if (T > 0) {
      uint32_t rows[LPT];
      nj = (j0 >= 0) ? blen[j0] : 0;
      tile_rows4<D>(rows, ring + 0 * 64, ww, lane, row_bytes);
      stage4<D>(krs, kbuf(0), rows, koff, ww);
      stage4<D>(vrs, vbuf(0), rows, voff, ww);
      tile_rows4<D>(rows_next, ring + 1 * 64, ww, lane, row_bytes);
      stage4<D>(krs, kbuf(1), rows_next, koff, ww);
    }

    // ---------------- L2: the first copies land ----------------
    phase();

    f32x16 oacc[DT];
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f, lx_run = 0.f;
    f32x16 sacc;
    bf16x8 pop[2];
    // S^T = K(s) Q^T for the key half of this wave
    auto qk = [&](int s) {
      const __bf16* Kc = KVg + (s & 1) * TILE;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      bf16x8 ka[KS];
#pragma unroll
      for (int x = 0; x < KS + PF; ++x) {
        if (x < KS) {
          ka[x] = *reinterpret_cast<const bf16x8*>(Kc + krow * D + k_swz<CPR>(krow, 2 * x + h2) * 8);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        if (x >= PF) {
          sacc = mfma32(ka[x - PF], qop[x - PF], sacc);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
      }
    };

    // ---------------- M_0: S^T of block 0 ----------------
    wait_vmcnt<2 * LPT>();  // K(0) of the prologue batch K(0), V(0), K(1)
    phase();
    if (T > 0 && !qidle) qk(0);
    for (int s = 0; s < T; ++s) {
      // ---------------- S_s: copies for later blocks, softmax of block s ----------------
      wait_vmcnt<2 * LPT>();  // the ids at the head of the last batch (own copies only)
      phase();
      // A block of at most 32 tokens leaves key half 1 with masked keys only:
      // its weights are exact zeros, so those waves skip the block's products.
      const bool idle_s = g == 1 && nj <= 32;
      {
        // batch: ids(s+3), K(s+2) with the rows of block s+2, V(s+1) with those of s+1
        stage_ids(prs, max(jc, 0), M, ring_lds((s + 3) & 3), lane);
        uint32_t rows[LPT];
        tile_rows4<D>(rows, ring + ((s + 2) & 3) * 64, ww, lane, row_bytes);
        stage4<D>(krs, kbuf(s & 1), rows, koff, ww);
        stage4<D>(vrs, vbuf((s + 1) & 1), rows_next, voff, ww);
#pragma unroll
        for (int k = 0; k < LPT; ++k) rows_next[k] = rows[k];
      }
      // scalar reads for the coming steps: the block after the ids just staged,
      // and the true length of the next block
      __builtin_amdgcn_sched_barrier(0);
      const int jd = kept_id(sel, min(s + 4, T - 1), p.J, bad);
      const int njn = (ja >= 0) ? blen[max(ja, 0)] : 0;
      __builtin_amdgcn_sched_barrier(0);

      // the softmax of block s: skipped by waves whose rows are never written
      // or whose keys of block s are all masked
      if (!qidle && !idle_s) {
        if (nj < M) {  // edge / short block: mask keys at or beyond its true length
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = TM::key_of_row(32 * g + 8 * (r >> 2) + 4 * h2 + (r & 3));
            sacc[r] = (key < nj) ? sacc[r] : -INFINITY;
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        mx = fmaxf(mx, xor32(mx)) * p.scale_log2;
        // lazy rescale (as in the four-wave kernel): the reference moves only
        // when some row's maximum grew by more than 8 in log2 units
        if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = fast_exp2(m_run - m_new);
          l_run *= alpha;
          if constexpr (LSE) lx_run *= alpha;
#pragma unroll
          for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
          m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float rs = 0.f, rsx = 0.f;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * hlf + 2 * e;
            const float a = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -m_use));
            const float c = fast_exp2(__builtin_fmaf(sacc[r + 1], p.scale_log2, -m_use));
            pk[e] = pack2_bf16_sum<LSE>(a, c, &rs, &rsx);
          }
          pop[hlf] = __builtin_bit_cast(bf16x8, pk);
        }
        l_run += rs;
        if constexpr (LSE) lx_run += rsx;
      }
      nj = njn;
      ja = jb;
      jb = jc;
      jc = jd;

      // The probabilities must be formed in this phase: left to itself the
      // compiler sinks the exponentials past the barrier, next to their use.
      asm volatile("" ::"v"(pop[0]), "v"(pop[1]), "v"(l_run), "v"(lx_run));

      // ---------------- M_{s+1}: PV(s), then S^T of block s+1 ----------------
      wait_vmcnt<2 * LPT + 1>();  // every batch but the last one
      phase();
      if (!idle_s && !qidle) {
        const uint32_t vb = (s & 1) ? (uint32_t)(TILE * 2) : 0u;
        bf16x8 va[NP];
#pragma unroll
        for (int x = 0; x < NP + PF; ++x) {
          if (x < NP) {
            const int u = x / DT, dt = x % DT;
            // rows r0 + 16u and r0 + 16u + 8 keep r0's swizzle (same row % 4)
            const uint32_t a = vtr[dt] + vb + (uint32_t)(16 * u * D * 2);
            const bf16x4 lo = lds_read_tr16_at(a);
            const bf16x4 hi = lds_read_tr16_at(a + (uint32_t)(8 * D * 2));
            va[x] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
          }
          if (x >= PF) {
            const int y = x - PF;
            oacc[y % DT] = mfma32(va[y], pop[y / DT], oacc[y % DT]);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < T && !(g == 1 && nj <= 32) && !qidle) qk(s + 1);  // nj: length of block s+1 here
    }

    // ---------------- E0: key half 1 hands its state to key half 0 ----------------
    wait_vmcnt<0>();  // the last (repeat) copies have landed in this group's buffers
    phase();
    if (bad) flag_index_error(p.err);
    float* scr = reinterpret_cast<float*>(KVg) + hq * (64 * DT * 16);
    float* mxs = Mx + (grp * 2 + hq) * 3 * 64;
    if (g == 1 && out_ok) {
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4 v = {oacc[d][4 * c4], oacc[d][4 * c4 + 1], oacc[d][4 * c4 + 2], oacc[d][4 * c4 + 3]};
          *reinterpret_cast<f32x4*>(scr + ((d * 4 + c4) * 64 + lane) * 4) = v;
        }
      mxs[lane] = m_run;
      mxs[64 + lane] = l_run;
      mxs[128 + lane] = lx_run;
    }

    // ---------------- E1: merge, normalise, store; take the next item ----------------
    phase();
    if (g == 0 && out_ok) {
      const float mb = mxs[lane], lb = mxs[64 + lane], lxb = mxs[128 + lane];
      const float m = fmaxf(m_run, mb);
      const float fa = (m == -INFINITY) ? 0.f : fast_exp2(m_run - m);
      const float fb = (m == -INFINITY) ? 0.f : fast_exp2(mb - m);
      const float l_part = fa * l_run + fb * lb;
      const float l_tot = l_part + xor32(l_part);
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      __bf16* __restrict__ og = reinterpret_cast<__bf16*>(p.o) + b * p.o_sB + (int64_t)qtok * p.o_sN + hh * p.o_sH;
      // one 32-channel tile at a time: merge with key half 1, normalise, store
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(scr + ((d * 4 + c4) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[d][4 * c4 + e] = fa * oacc[d][4 * c4 + e] + fb * v[e];
        }
        if (qrow < ni) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int dd = 32 * d + 8 * jj + 4 * h2;
            const f32x4 cg = coarse_term(p, bh, hh, i, dd);
            bf16x4 v4 = {(__bf16)fmaf(oacc[d][4 * jj + 0], inv, cg[0]), (__bf16)fmaf(oacc[d][4 * jj + 1], inv, cg[1]),
                         (__bf16)fmaf(oacc[d][4 * jj + 2], inv, cg[2]), (__bf16)fmaf(oacc[d][4 * jj + 3], inv, cg[3])};
            *reinterpret_cast<bf16x4*>(og + dd) = v4;
          }
        }
      }
      if constexpr (LSE) {
        const float lx_part = fa * lx_run + fb * lxb;
        const float lx = lx_part + xor32(lx_part);
        if (qrow < ni && h2 == 0) p.lse[bh * p.N + qtok] = (lx > 0.f) ? (m + __log2f(lx)) * kLn2 : -INFINITY;
      }
    }
    if (lead) item_sh[grp] = p.sched ? pp_next_item(st, xcc, items) : item_sh[grp] + 2 * (int)gridDim.x;
    if (sync && grp == 0) {
      if (lead) cohort_arrive_wait(st, coh);
      ++coh.round;
    }
  }

  // Out of items: keep passing barriers until the other group is out too; a
  // count recorded in a phase is read only after the next barrier.
  for (;;) {
    phase();
    if (done_at[0] < q && done_at[1] < q) break;
  }
}

template <int D, bool LSE>
static hipError_t launch_vsa_pp(const VsaAttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    cus = 256;
  const int64_t grid = std::min<int64_t>((items + 1) / 2, cus);
  if (p.sched) clear_sched_kernel<<<64, 256, 0, s>>>(reinterpret_cast<SchedState*>(p.sched));
  vsa_pp_kernel<D, LSE><<<dim3((unsigned)grid), dim3(512), 0, s>>>(p, (int)items);
  return hipGetLastError();
}

// ============================================================================
// float32 inputs: exact fp32 attention on the vector ALUs (teaching-size
// problems).  One workgroup per query block, two lanes per query row, each lane
// owning half of the channels; K and V tiles of the kept block are staged in
// LDS and every key is visited in order with the online-softmax recurrence.
// ============================================================================
template <int D>
__global__ __launch_bounds__(128) void vsa_attn_f32_kernel(VsaAttnParams p) {
  constexpr int HD = D / 2;
  __shared__ float Kt[64 * D];
  __shared__ float Vt[64 * D];
  const int64_t wid = blockIdx.x;
  int64_t bh;
  const int i = item_of(p, wid, &bh);
  if (i < 0) return;  // not a block index (whole workgroup)
  const int hh = (int)(bh % p.H), b = (int)(bh / p.H);
  const int32_t* __restrict__ perm = p.perm + bh * p.perm_bh_stride;
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int ni = p.block_len[i];
  const int num = min(p.q2k_num[bh * p.J + i], p.kmax);
  const int32_t* sel = p.q2k_idx + (bh * p.J + i) * p.kmax;
  const float* qg = reinterpret_cast<const float*>(p.q) + b * p.q_sB + hh * p.q_sH;
  const float* kg = reinterpret_cast<const float*>(p.k) + b * p.kv_sB + hh * p.kv_sH;
  const float* vg = reinterpret_cast<const float*>(p.v) + b * p.kv_sB + hh * p.kv_sH;
  const int qtok = max(perm[(int64_t)i * p.M + max(min(row, ni - 1), 0)], 0);  // empty block: token 0, no output
  float qv[HD], ov[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qv[d] = qg[(int64_t)qtok * p.q_sN + half * HD + d];
    ov[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int pp = 0; pp < num; ++pp) {
    const int j = sel[pp];
    if (j < 0) continue;
    if (j >= p.J) {  // not a block: skipped and reported
      flag_index_error(p.err);
      continue;
    }
    const int nj = p.block_len[j];
    __syncthreads();
    for (int e = threadIdx.x; e < nj * D; e += 128) {
      const int r = e / D, d = e % D;
      const int64_t tok = perm[(int64_t)j * p.M + r];
      Kt[e] = kg[tok * p.kv_sN + d];
      Vt[e] = vg[tok * p.kv_sN + d];
    }
    __syncthreads();
    for (int r = 0; r < nj; ++r) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) part += qv[d] * Kt[r * D + half * HD + d];
      const float s = (part + __shfl_xor(part, 1, 64)) * p.scale_log2;
      const float m_new = fmaxf(m_run, s);
      const float alpha = exp2f(m_run - m_new);
      const float pr = exp2f(s - m_new);
      l_run = l_run * alpha + pr;
#pragma unroll
      for (int d = 0; d < HD; ++d) ov[d] = ov[d] * alpha + pr * Vt[r * D + half * HD + d];
      m_run = m_new;
    }
  }
  if (row < ni) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    float* og = reinterpret_cast<float*>(p.o) + b * p.o_sB + (int64_t)qtok * p.o_sN + hh * p.o_sH + half * HD;
    const float* cr = p.coarse ? p.coarse + (bh * p.J + i) * D + half * HD : nullptr;
    const float* gr = p.gate ? p.gate + (int64_t)hh * D + half * HD : nullptr;
#pragma unroll
    for (int d = 0; d < HD; ++d) og[d] = cr ? fmaf(ov[d], inv, gr[d] * cr[d]) : ov[d] * inv;
    if (p.lse && half == 0) p.lse[bh * p.N + qtok] = (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// Resident workgroups of a kernel on the current device; `cache` is the
// caller's per-device memo for that kernel.
template <typename K>
static int64_t resident_groups(K kernel, int threads, int64_t* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  cache[dev] = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
  return cache[dev];
}

template <int D, int MT, bool LSE>
static hipError_t launch_vsa_lse(const VsaAttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  static int64_t cache[64] = {0};
  const int64_t resident = resident_groups(vsa_attn_kernel<D, MT, LSE>, 2 * MT, cache);
  const int64_t grid = (resident > 0) ? std::min(items, resident) : items;
  const int64_t rounds = (items + grid - 1) / grid;
  const int sync = (rounds > 1 && p.sched != nullptr) ? 1 : 0;
  if (sync) clear_sched_kernel<<<64, 256, 0, s>>>(reinterpret_cast<SchedState*>(p.sched));
  vsa_attn_kernel<D, MT, LSE><<<dim3((unsigned)grid), dim3(2 * MT), 0, s>>>(p, (int)items, sync);
  return hipGetLastError();
}

template <int D, int MT>
static hipError_t launch_vsa_mt(const VsaAttnParams& p, hipStream_t s) {
  return p.lse ? launch_vsa_lse<D, MT, true>(p, s) : launch_vsa_lse<D, MT, false>(p, s);
}

template <int D, bool LSE, bool SUM>
static hipError_t launch_vsa4(const VsaAttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  static int64_t cache[64] = {0};
  const int64_t resident = resident_groups(vsa4_kernel<D, LSE, SUM>, 256, cache);
  const int64_t grid = (resident > 0) ? std::min(items, resident) : items;
  const int64_t rounds = (items + grid - 1) / grid;
  const int sync = (rounds > 1 && p.sched != nullptr) ? 1 : 0;
  if (sync) clear_sched_kernel<<<64, 256, 0, s>>>(reinterpret_cast<SchedState*>(p.sched));
  vsa4_kernel<D, LSE, SUM><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p, (int)items, sync);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_vsa_d(const VsaAttnParams& p, hipStream_t s) {
  if (p.M <= 32) return launch_vsa_mt<D, 32>(p, s);
  if (p.k_sum) return p.lse ? launch_vsa4<D, true, true>(p, s) : launch_vsa4<D, false, true>(p, s);
  return p.lse ? launch_vsa_pp<D, true>(p, s) : launch_vsa_pp<D, false>(p, s);
}

// Index tables of block capacity 128 rewritten for 64-token halves (see
// launch_expand_halves).  One thread per entry of the new kept lists; the
// first threads also write the half lengths and the processing order.  A
// negative kept id stays -1 in both halves, an id at or beyond J becomes 2J
// (still out of range, so the attention kernels skip and report it).
__global__ __launch_bounds__(256) void expand_halves_kernel(const int32_t* __restrict__ q2k,
                                                            const int32_t* __restrict__ num,
                                                            const int32_t* __restrict__ blen,
                                                            const int32_t* __restrict__ order, int BH, int J,
                                                            int kmax, int32_t* __restrict__ q2k2,
                                                            int32_t* __restrict__ num2, int32_t* __restrict__ blen2,
                                                            int32_t* __restrict__ order2) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t J2 = 2 * (int64_t)J, K2 = 2 * (int64_t)kmax;
  if (id < (int64_t)BH * J2 * K2) {
    const int e2 = (int)(id % K2);
    const int64_t row2 = id / K2;  // bh * 2J + i2
    const int64_t bh = row2 / J2;
    const int i = (int)((row2 % J2) >> 1), e = e2 >> 1;
    const int n = max(min(num[bh * J + i], kmax), 0);
    int out = -1;
    if (e < n) {
      const int v = q2k[(bh * J + i) * kmax + e];
      out = v < 0 ? -1 : (v >= J ? (int)J2 : 2 * v + (e2 & 1));
    }
    q2k2[id] = out;
    if (e2 == 0) num2[row2] = 2 * n;
  }
  if (id < J2) {
    const int n = blen[id >> 1], lo = max(min(n, 64), 0);
    blen2[id] = (id & 1) ? max(n - lo, 0) : lo;
  }
  if (order && id < (int64_t)BH * J2) {
    const int64_t bh = id / J2;
    const int o = order[bh * J + ((id % J2) >> 1)];
    order2[id] = (o >= 0 && o < J) ? 2 * o + (int)(id & 1) : -1;
  }
}

hipError_t launch_expand_halves(const int32_t* q2k, const int32_t* num, const int32_t* blen, const int32_t* order,
                                int BH, int J, int kmax, int32_t* q2k2, int32_t* num2, int32_t* blen2,
                                int32_t* order2, hipStream_t s) {
  const int64_t n = std::max<int64_t>((int64_t)BH * 2 * J * 2 * kmax, 2 * (int64_t)J);
  expand_halves_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(q2k, num, blen, order, BH, J, kmax,
                                                                              q2k2, num2, blen2, order2);
  return hipGetLastError();
}

hipError_t launch_vsa_attention(const VsaAttnParams& p, bool f32_io, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  if (f32_io) {
    if (p.D == 128)
      vsa_attn_f32_kernel<128><<<dim3((unsigned)items), dim3(128), 0, s>>>(p);
    else
      vsa_attn_f32_kernel<64><<<dim3((unsigned)items), dim3(128), 0, s>>>(p);
    return hipGetLastError();
  }
  if (p.D == 128) return launch_vsa_d<128>(p, s);
  return launch_vsa_d<64>(p, s);
}

}  // namespace bsa
