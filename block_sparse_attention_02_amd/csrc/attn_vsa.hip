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
#define BSA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// Physical 16-byte chunk of logical chunk c in tile row r.
template <int CPR>
__device__ __forceinline__ int k_swz(int r, int c) {
  return c ^ (r & (CPR >= 8 ? 7 : CPR - 1));
}
template <int CPR>
__device__ __forceinline__ int v_swz(int r, int c) {
  if constexpr (CPR >= 16) {
    // XOR pattern {0, 6, 10, 12} for r % 4 = 0..3, packed in nibbles
    return c ^ ((0xCA60 >> (4 * (r & 3))) & 15);
  } else {
    return c ^ (2 * (r & 3));
  }
}

// Per-thread rows of a tile copy: instruction k of wave w covers the 64 chunks
// [(k*NW + w)*64, +64) of the row-major tile, lane L chunk (k*NW + w)*64 + L.
template <int D, int MT>
struct TileMap {
  static constexpr int NW = MT / 32;
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int LPT = MT * CPR / (64 * NW);  // copies per thread per tile
  __device__ static int row(int k, int w, int lane) { return ((k * NW + w) * 64 + lane) / CPR; }
  __device__ static int pchunk(int k, int w, int lane) { return ((k * NW + w) * 64 + lane) % CPR; }
};

// Copy one K or V tile (rows given by tok[]) into LDS with asynchronous
// 16-byte global->LDS copies (LPT per lane, counted by wait_vmcnt).
template <int D, int MT, bool IS_V>
__device__ __forceinline__ void stage_tile(__bf16* lds, const __bf16* __restrict__ base, int64_t sN,
                                           const int* tok, int w, int lane) {
  using TM = TileMap<D, MT>;
#pragma unroll
  for (int k = 0; k < TM::LPT; ++k) {
    const int r = TM::row(k, w, lane);
    const int pc = TM::pchunk(k, w, lane);
    const int lc = IS_V ? v_swz<TM::CPR>(r, pc) : k_swz<TM::CPR>(r, pc);
    global_to_lds16_async(base + (int64_t)tok[k] * sN + lc * 8, lds_offset(lds + (size_t)(k * TM::NW + w) * 64 * 8));
  }
}

// Token ids of the tile rows this lane copies.  Copy k of wave w covers the
// RPI = 64/CPR consecutive rows starting at (k*NW + w)*RPI; their ids are read
// with uniform (scalar) loads and each lane picks its own row, so these reads
// do not count against the vector-memory counter the copies are tracked with.
template <int D, int MT>
__device__ __forceinline__ void tile_tokens(int* tok, const int32_t* __restrict__ perm, int j, int M,
                                            int nj, int w, int lane) {
  using TM = TileMap<D, MT>;
  constexpr int RPI = 64 / TM::CPR;
  const int sub = lane / TM::CPR;
  const auto row0 = as_const(perm) + (int64_t)j * M;
#pragma unroll
  for (int k = 0; k < TM::LPT; ++k) {
    const int r0 = (k * TM::NW + w) * RPI;
    int t = row0[min(r0, nj - 1)];
#pragma unroll
    for (int q = 1; q < RPI; ++q) {
      const int tq = row0[min(r0 + q, nj - 1)];
      t = (sub == q) ? tq : t;
    }
    tok[k] = t;
  }
}

template <int D, int MT>
__global__ __launch_bounds__(2 * MT) __attribute__((amdgpu_waves_per_eu(2, 2))) void vsa_attn_kernel(VsaAttnParams p) {
  using Tin = __bf16;
  using TM = TileMap<D, MT>;
  constexpr int NW = TM::NW;
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

  const Tin* __restrict__ qg = reinterpret_cast<const Tin*>(p.q) + b * p.q_sB + hh * p.q_sH;
  const Tin* __restrict__ kg = reinterpret_cast<const Tin*>(p.k) + b * p.kv_sB + hh * p.kv_sH;
  const Tin* __restrict__ vg = reinterpret_cast<const Tin*>(p.v) + b * p.kv_sB + hh * p.kv_sH;
  const auto sel = as_const(p.q2k_idx) + (bh * p.J + i) * p.kmax;
  const auto blen = as_const(p.block_len);
  const int num = min(as_const(p.q2k_num)[bh * p.J + i], p.kmax);
  const int ni = blen[i];

  // ---- query rows: B operand of S^T, lane l holds row 32w + l%32 ----
  const int qrow = 32 * w + (lane & 31);
  const int qtok = p.perm[(int64_t)i * M + min(qrow, ni - 1)];
  bf16x8 qop[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qop[s] = load8_bf16<Tin>(qg + (int64_t)qtok * p.q_sN + 16 * s + 8 * h2);
  // Consume the query registers here so the compiler waits for their loads
  // before the loop; from here on only the tile copies count against vmcnt.
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qop[s]));

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  int pc = 0;
  while (pc < num && sel[pc] < 0) ++pc;
  int tok[LPT], tokn[LPT];
  int j = 0, nj = 0, pn = num, jn = 0, njn = 0;
  bool has_next = false;
  if (pc < num) {
    j = sel[pc];
    nj = blen[j];
    tile_tokens<D, MT>(tok, p.perm, j, M, nj, w, lane);
    stage_tile<D, MT, false>(Ks, kg, p.kv_sN, tok, w, lane);
    pn = pc + 1;
    while (pn < num && sel[pn] < 0) ++pn;
    has_next = pn < num;
    if (has_next) {
      jn = sel[pn];
      njn = blen[jn];
      tile_tokens<D, MT>(tokn, p.perm, jn, M, njn, w, lane);
    }
    stage_tile<D, MT, true>(Vs, vg, p.kv_sN, tok, w, lane);
  }

  while (pc < num) {
    // ---- K(j) resident; only V(j) may still be in flight ----
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
    if (has_next) stage_tile<D, MT, false>(Ks, kg, p.kv_sN, tokn, w, lane);

    // ---- online softmax (log2 domain); lane owns query 32w + l%32 ----
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const float x = (key < nj) ? sacc[kt][r] * p.scale_log2 : -INFINITY;
        sacc[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
    bf16x8 pop[US];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(sacc[kt][r] - m_use);
        rs += pr;
        pop[2 * kt + (r >> 3)][r & 7] = (__bf16)pr;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;

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
    // ---- advance: tokens of the block after next, then V of the next block ----
    pc = pn;
    j = jn;
    nj = njn;
#pragma unroll
    for (int k = 0; k < LPT; ++k) tok[k] = tokn[k];
    pn = pc + 1;
    while (pn < num && sel[pn] < 0) ++pn;
    has_next = pn < num;
    if (has_next) {
      jn = sel[pn];
      njn = blen[jn];
      tile_tokens<D, MT>(tokn, p.perm, jn, M, njn, w, lane);
    }
    stage_tile<D, MT, true>(Vs, vg, p.kv_sN, tok, w, lane);
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
    if (p.lse && h2 == 0) {
      p.lse[bh * p.N + qtok] = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
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

template <int D>
static hipError_t launch_vsa_d(const VsaAttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  if (p.M <= 32) {
    vsa_attn_kernel<D, 32><<<dim3((unsigned)items), dim3(64), 0, s>>>(p);
  } else {
    vsa_attn_kernel<D, 64><<<dim3((unsigned)items), dim3(128), 0, s>>>(p);
  }
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
