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
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

// Workgroup barrier that first retires this wave's outstanding LDS reads, so a
// buffer can be refilled right after it.  Asynchronous global->LDS copies are
// ordered separately with wait_vmcnt<>().
// Workgroup barrier that first retires this wave's outstanding LDS reads, so a
// buffer can be refilled right after it.  Asynchronous global->LDS copies are
// ordered separately with wait_vmcnt<>().
#define BSA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

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

// Asynchronous 16-byte buffer -> LDS copy (lane L lands in slot L of the
// wave's 1 KiB LDS window at `lds_byte_offset`); counted by wait_vmcnt<>().
__device__ __forceinline__ void buffer_to_lds16(i32x4 rsrc, uint32_t voffset, uint32_t lds_byte_offset) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "{m0}"(lds_byte_offset)
      : "memory");
}

// Byte offsets (within the slice) of the tile rows this lane copies.  The 32
// row ids of the wave are read with uniform (scalar) loads from the constant
// address space and each lane picks its own row; padding rows (perm = -1) and
// rows beyond the block capacity repeat the block's first token (their keys
// are masked later).
template <int D, int MT>
__device__ __forceinline__ void tile_rows(uint32_t* rowoff, const int32_t* __restrict__ perm, int j, int M,
                                          int w, int lane, uint32_t row_bytes) {
  using TM = TileMap<D, MT>;
  const auto row0 = as_const(perm) + (int64_t)j * M;
  const int first = row0[0];
  const int sub = lane / TM::CPR;
  // Capacities are 16, 32 or 64 with MT = max(32, M): only M = 16 leaves rows
  // 16..31 of the (single) wave outside the block's table.
  int ids[32];
  const auto rw = row0 + 32 * w;
#pragma unroll
  for (int q = 0; q < 16; ++q) ids[q] = rw[q];
  if (M >= 32) {
#pragma unroll
    for (int q = 16; q < 32; ++q) ids[q] = rw[q];
  } else {
#pragma unroll
    for (int q = 16; q < 32; ++q) ids[q] = -1;
  }
#pragma unroll
  for (int k = 0; k < TM::LPT; ++k) {
    int t = ids[k * TM::RPI];
#pragma unroll
    for (int q = 1; q < TM::RPI; ++q) t = (sub == q) ? ids[k * TM::RPI + q] : t;
    t = (t < 0) ? first : t;
    rowoff[k] = (uint32_t)t * row_bytes;
  }
}

template <int D, int MT>
__device__ __forceinline__ void stage_tile(i32x4 rsrc, uint32_t lds_base, const uint32_t* rowoff,
                                           const uint32_t* chunkoff, int w) {
  using TM = TileMap<D, MT>;
#pragma unroll
  for (int k = 0; k < TM::LPT; ++k)
    buffer_to_lds16(rsrc, rowoff[k] + chunkoff[k], lds_base + (uint32_t)((w * TM::LPT + k) * 1024));
}

// LSE: also keep the exact (unrounded) row sum for the log-sum-exp output.
template <int D, int MT, bool LSE>
__global__ __launch_bounds__(2 * MT) __attribute__((amdgpu_waves_per_eu(2, 2))) void vsa_attn_kernel(VsaAttnParams p) {
  using TM = TileMap<D, MT>;
  constexpr int LPT = TM::LPT;
  constexpr int KT = MT / 32;   // 32-key tiles per KV tile
  constexpr int KS = D / 16;    // k-steps of QK^T
  constexpr int DT = D / 32;    // 32-channel tiles of O
  constexpr int US = MT / 16;   // 16-key steps of PV
  static_assert(LPT >= 1 && LPT <= 16, "tile copy shape");

  __shared__ __align__(1024) __bf16 Ks[MT * D];
  __shared__ __align__(1024) __bf16 Vs[MT * D];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h2 = lane >> 5;  // which half of the wave
  const int64_t wid = blockIdx.x;
  const int i = (int)(wid % p.J);
  const int64_t bh = wid / p.J;
  const int hh = (int)(bh % p.H), b = (int)(bh / p.H);
  const int M = p.M;

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
  const int qtok = p.perm[(int64_t)i * M + min(qrow, ni - 1)];
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
  uint32_t rows[LPT], rowsn[LPT];
  int nj = 0, njn = 0;
  if (num > 0) {
    const int j = sel[0];
    nj = (j >= 0) ? blen[j] : 0;
    tile_rows<D, MT>(rows, p.perm, max(j, 0), M, w, lane, row_bytes);
    stage_tile<D, MT>(krs, ks_lds, rows, koff, w);
    stage_tile<D, MT>(vrs, vs_lds, rows, voff, w);
    if (num > 1) {
      const int jn = sel[1];
      njn = (jn >= 0) ? blen[jn] : 0;
      tile_rows<D, MT>(rowsn, p.perm, max(jn, 0), M, w, lane, row_bytes);
    }
  }

  for (int pc = 0; pc < num; ++pc) {
    const bool has_next = pc + 1 < num;
    // ---- K(j) resident; V(j) may still be in flight ----
    wait_vmcnt<LPT>();
    BSA_BARRIER();

    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int krow = 32 * kt + (lane & 31);
        const int pch = k_swz<TM::CPR>(krow, 2 * s + h2);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + krow * D + pch * 8);
        sacc[kt] = mfma32(a, qop[s], sacc[kt]);
      }
    }
    BSA_BARRIER();  // every wave is done reading Ks
    if (has_next) stage_tile<D, MT>(krs, ks_lds, rowsn, koff, w);

    // ---- online softmax (log2 domain); lane owns query 32w + l%32 ----
    if (nj < MT) {  // edge / short block: mask keys at or beyond its true length
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
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
      const int g16 = lane >> 4, jl = lane & 15;
#pragma unroll
      for (int u = 0; u < US; ++u) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 32 * dt + 16 * (g16 & 1) + 4 * (jl & 3);
          const int c = d >> 3, off = d & 7;
          const int r0 = 16 * u + 4 * h2 + (jl >> 2);
          const int r1 = r0 + 8;
          const bf16x4 lo = lds_read_tr16(Vs + r0 * D + v_swz<TM::CPR>(r0, c) * 8 + off);
          const bf16x4 hi = lds_read_tr16(Vs + r1 * D + v_swz<TM::CPR>(r1, c) * 8 + off);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[dt] = mfma32(a, pop[u], oacc[dt]);
        }
      }
    }
    BSA_BARRIER();  // every wave is done reading Vs

    if (!has_next) break;
    // ---- advance: V of the next block, then the rows of the block after ----
    nj = njn;
#pragma unroll
    for (int k = 0; k < LPT; ++k) rows[k] = rowsn[k];
    stage_tile<D, MT>(vrs, vs_lds, rows, voff, w);
    if (pc + 2 < num) {
      const int jn = sel[pc + 2];
      njn = (jn >= 0) ? blen[jn] : 0;
      tile_rows<D, MT>(rowsn, p.perm, max(jn, 0), M, w, lane, row_bytes);
    }
  }

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
        bf16x4 v4 = {(__bf16)(oacc[dt][4 * jj + 0] * inv), (__bf16)(oacc[dt][4 * jj + 1] * inv),
                     (__bf16)(oacc[dt][4 * jj + 2] * inv), (__bf16)(oacc[dt][4 * jj + 3] * inv)};
        *reinterpret_cast<bf16x4*>(og + d) = v4;
      }
    if constexpr (LSE) {
      const float lx = lx_run + xor32(lx_run);
      if (h2 == 0) p.lse[bh * p.N + qtok] = (lx > 0.f) ? (m_run + __log2f(lx)) * kLn2 : -INFINITY;
    }
  }
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
  const int i = (int)(wid % p.J);
  const int64_t bh = wid / p.J;
  const int hh = (int)(bh % p.H), b = (int)(bh / p.H);
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int ni = p.block_len[i];
  const int num = min(p.q2k_num[bh * p.J + i], p.kmax);
  const int32_t* sel = p.q2k_idx + (bh * p.J + i) * p.kmax;
  const float* qg = reinterpret_cast<const float*>(p.q) + b * p.q_sB + hh * p.q_sH;
  const float* kg = reinterpret_cast<const float*>(p.k) + b * p.kv_sB + hh * p.kv_sH;
  const float* vg = reinterpret_cast<const float*>(p.v) + b * p.kv_sB + hh * p.kv_sH;
  const int qtok = p.perm[(int64_t)i * p.M + min(row, ni - 1)];
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
    const int nj = p.block_len[j];
    __syncthreads();
    for (int e = threadIdx.x; e < nj * D; e += 128) {
      const int r = e / D, d = e % D;
      const int64_t tok = p.perm[(int64_t)j * p.M + r];
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
#pragma unroll
    for (int d = 0; d < HD; ++d) og[d] = ov[d] * inv;
    if (p.lse && half == 0) p.lse[bh * p.N + qtok] = (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, int MT>
static hipError_t launch_vsa_mt(const VsaAttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  if (p.lse)
    vsa_attn_kernel<D, MT, true><<<dim3((unsigned)items), dim3(2 * MT), 0, s>>>(p);
  else
    vsa_attn_kernel<D, MT, false><<<dim3((unsigned)items), dim3(2 * MT), 0, s>>>(p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_vsa_d(const VsaAttnParams& p, hipStream_t s) {
  if (p.M <= 32) return launch_vsa_mt<D, 32>(p, s);
  return launch_vsa_mt<D, 64>(p, s);
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
