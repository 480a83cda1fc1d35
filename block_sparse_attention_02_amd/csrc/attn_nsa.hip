// NSA selected-branch attention (token-selection mode of the query-outer
// schedule) for gfx950.
//
// Source: "NSA 算子解析（Torch/Tilelang）", "Torch朴素实现": for every batch, token
// t and query head hq the keys are the tokens blk*BS + u of the selected blocks
// of KV head hq / G (G = HQ / H), a key is dropped when its position exceeds t
// or its block slot is not below the block count, scale = D^-0.5, one softmax
// over the kept keys, weighted sum of V.  The page's TileLang kernel also skips
// negative block ids and blocks that start after t; both rules are kept here
// (negative ids and blocks entirely in the future contribute nothing).
//
// Design (MI355X): one wave per (batch, token, KV head, group of 16 query
// heads).  The 16 query heads of the group form the 16-row dimension of
//   S^T (keys x heads)   = K Q^T          v_mfma_f32_16x16x32_bf16
//   O^T (chans x heads) += V^T P^T        v_mfma_f32_16x16x32_bf16
// so lane l owns head l%16; row maxima and sums reduce over the four lanes
// l%16 + 16g.  K operands are loaded from global memory straight into
// registers (each lane reads 16 contiguous bytes of a key row); V goes to the
// wave's own LDS region with asynchronous 16-byte copies and is read back with
// the transposing LDS read.  Keys are processed in chunks of up to 64.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

template <int D, int KC>
struct NsaShape {
  static constexpr int CPR = D / 8;          // 16-byte chunks per key row
  static constexpr int LPT = KC * CPR / 64;  // V copies per lane per chunk
  static constexpr int KT = KC / 16;         // 16-key tiles of S^T
  static constexpr int KS = D / 32;          // k-steps of QK^T
  static constexpr int US = KC / 32;         // 32-key steps of PV
  static constexpr int DT = D / 16;          // 16-channel tiles of O^T
};

// 16-byte chunk swizzle of the V rows: the 4 rows x 32 bytes read by one
// 16-lane group of the transposing read land on 8 distinct 16-byte bank
// groups, and two neighbouring groups (rows 4 apart) use disjoint halves.
template <int CPR>
__device__ __forceinline__ int nsa_v_swz(int r, int c) {
  return c ^ (2 * (r & 3)) ^ (CPR >= 16 ? 8 * ((r >> 2) & 1) : 0);
}

template <int D, int KC>
__global__ __launch_bounds__(64) void nsa_attn_kernel(NsaAttnParams p) {
  using SH = NsaShape<D, KC>;
  __shared__ __align__(1024) __bf16 Vs[KC * D];

  const int lane = threadIdx.x;
  const int g = lane >> 4, l16 = lane & 15;
  const int G = p.Hq / p.Hkv;
  const int ngroups = (G + 15) / 16;
  // work item: ((b * N + t) * Hkv + r) * ngroups + hg
  int64_t wid = blockIdx.x;
  const int hg = (int)(wid % ngroups);
  wid /= ngroups;
  const int r = (int)(wid % p.Hkv);
  wid /= p.Hkv;
  const int64_t t = wid % p.N;
  const int b = (int)(wid / p.N);

  const int head_in_group = 16 * hg + l16;
  const bool head_ok = head_in_group < G;
  const int hq = r * G + min(head_in_group, G - 1);

  const __bf16* __restrict__ qrow = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sB + t * p.q_sN + hq * p.q_sH;
  const __bf16* __restrict__ kg = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_sB + r * p.kv_sH;
  const __bf16* __restrict__ vg = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_sB + r * p.kv_sH;
  const int64_t row_off = (((int64_t)b * p.N + t) * p.Hkv + r);
  const int32_t* __restrict__ sel = p.blk_idx + row_off * p.S;
  const int cnt = p.blk_cnt ? min(p.blk_cnt[row_off], p.S) : p.S;

  // B operand of S^T: lane l holds Q[head l%16][32s + 8g + e]
  bf16x8 qop[SH::KS];
#pragma unroll
  for (int s = 0; s < SH::KS; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * g);

  f32x4 oacc[SH::DT];
#pragma unroll
  for (int dt = 0; dt < SH::DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f, lx_run = 0.f;  // sums of rounded / exact weights
  const int64_t last = p.causal ? t : p.N - 1;  // last visible key position

  for (int pp = 0; pp < cnt; ++pp) {
    const int blk = sel[pp];
    if (blk < 0) continue;
    const int64_t k0 = (int64_t)blk * p.BS;
    if (k0 >= p.N) {  // not a block of the sequence: skipped and reported
      flag_index_error(p.err);
      continue;
    }
    if (k0 > last) continue;  // the whole block is masked
    for (int c0 = 0; c0 < p.BS; c0 += KC) {
      const int64_t base = k0 + c0;
      if (base > last) break;
      // ---- V chunk -> LDS (asynchronous), rows clamped to valid memory ----
#pragma unroll
      for (int kk = 0; kk < SH::LPT; ++kk) {
        const int chunk = kk * 64 + lane;
        const int vr = chunk / SH::CPR, pc = chunk % SH::CPR;
        const int lc = nsa_v_swz<SH::CPR>(vr, pc);
        const int64_t pos = min(base + vr, (int64_t)p.N - 1);
        global_to_lds16(vg + pos * p.kv_sN + lc * 8, Vs + (size_t)kk * 64 * 8);
      }
      // ---- S^T = K Q^T, K rows read straight from global memory ----
      f32x4 sacc[SH::KT];
#pragma unroll
      for (int kt = 0; kt < SH::KT; ++kt) {
        sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t pos = min(base + 16 * kt + l16, (int64_t)p.N - 1);
        const __bf16* krow = kg + pos * p.kv_sN;
#pragma unroll
        for (int s = 0; s < SH::KS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 32 * s + 8 * g);
          sacc[kt] = mfma16(a, qop[s], sacc[kt]);
        }
      }
      // ---- online softmax; lane owns head l%16, keys 16kt + 4g + i ----
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < SH::KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t pos = base + 16 * kt + 4 * g + i;
          const bool ok = pos <= last && (c0 + 16 * kt + 4 * g + i) < p.BS;
          const float x = ok ? sacc[kt][i] * p.scale_log2 : -INFINITY;
          sacc[kt][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      // weights rounded to bf16 once; the row sum uses the rounded values.
      // k-step u = kt/2 holds keys 32u + 4g + i (e = i) and 32u + 16 + 4g + i (e = 4 + i)
      float rs = 0.f, rsx = 0.f;
      bf16x8 pop[SH::US];
#pragma unroll
      for (int u = 0; u < SH::US; ++u) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kt = 2 * u + (e >> 1), i = 2 * (e & 1);
          pk[e] = pack2_bf16_sum<true>(fast_exp2(sacc[kt][i] - m_use), fast_exp2(sacc[kt][i + 1] - m_use), &rs,
                                       &rsx);
        }
        pop[u] = __builtin_bit_cast(bf16x8, pk);
      }
      l_run = l_run * alpha + rs;
      lx_run = lx_run * alpha + rsx;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < SH::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha;
      // ---- O^T += V^T P^T ----
      wait_vmcnt<0>();
#pragma unroll
      for (int u = 0; u < SH::US; ++u) {
#pragma unroll
        for (int dt = 0; dt < SH::DT; ++dt) {
          const int d = 16 * dt + 4 * (l16 & 3);
          const int c = d >> 3, off = d & 7;
          const int r0 = 32 * u + 4 * g + (l16 >> 2);
          const int r1 = r0 + 16;
          const bf16x4 lo = lds_read_tr16(Vs + r0 * D + nsa_v_swz<SH::CPR>(r0, c) * 8 + off);
          const bf16x4 hi = lds_read_tr16(Vs + r1 * D + nsa_v_swz<SH::CPR>(r1, c) * 8 + off);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[dt] = mfma16(a, pop[u], oacc[dt]);
        }
      }
      // the next chunk's copies overwrite Vs: all reads of this chunk must be done
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }

  // ---- epilogue: the four lanes of a head hold partial row sums ----
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (head_ok) {
    __bf16* __restrict__ og = reinterpret_cast<__bf16*>(p.o) + b * p.o_sB + t * p.o_sN + hq * p.o_sH;
#pragma unroll
    for (int dt = 0; dt < SH::DT; ++dt) {
      const int d = 16 * dt + 4 * g;
      bf16x4 v4 = {(__bf16)(oacc[dt][0] * inv), (__bf16)(oacc[dt][1] * inv), (__bf16)(oacc[dt][2] * inv),
                   (__bf16)(oacc[dt][3] * inv)};
      *reinterpret_cast<bf16x4*>(og + d) = v4;
    }
    if (p.lse) {
      float lx = lx_run + __shfl_xor(lx_run, 16, 64);
      lx += __shfl_xor(lx, 32, 64);
      if (g == 0) p.lse[((int64_t)b * p.Hq + hq) * p.N + t] = (lx > 0.f) ? (m_run + __log2f(lx)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
static hipError_t launch_nsa_d(const NsaAttnParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  const int64_t items = (int64_t)p.B * p.N * p.Hkv * ((G + 15) / 16);
  if (p.BS <= 32)
    nsa_attn_kernel<D, 32><<<dim3((unsigned)items), dim3(64), 0, s>>>(p);
  else
    nsa_attn_kernel<D, 64><<<dim3((unsigned)items), dim3(64), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_nsa_attention(const NsaAttnParams& p, bool f32_io, hipStream_t s) {
  if (f32_io) return hipErrorInvalidValue;
  if (p.D == 128) return launch_nsa_d<128>(p, s);
  return launch_nsa_d<64>(p, s);
}

}  // namespace bsa
