// Spark-Reweight block summaries for gfx950.
//
// Source: "深度解读|Spark-H3：从注意力几何到稀疏内核代码" -- section 07 (the default
// representative query of a head is the mean of all of its video queries)
// and section 08 (in-block weights p = softmax(a.k / sqrt(d)) at the
// representative query a; summary key and value are the p-weighted sums of
// the block's keys and values; the log-mass l = log sum exp; the bias is
// l - a.k~ / sqrt(d)).  The page notes that the bias is formed with the stored
// bf16 summary key, so the key the attention kernel reads and the mass
// correction belong together; that is done here.
//
// Design (MI355X): the anchor is a two-stage reduction (partial sums per
// chunk of 256 tokens, then a fixed-order sum), so it is deterministic.  The
// summaries take one wave per block: lane l covers the 16-byte channel chunk
// l % (D/8) of row l / (D/8) of a step, every row of the block is loaded up
// front (K and V straight into registers), the logits are reduced across the
// lanes of a row, and the weighted sums across the rows.  Memory bound: every
// K and V row is read once.
#include <algorithm>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kAnchorTok = 256;  // tokens per partial sum

__global__ __launch_bounds__(1024) void anchor_partial_kernel(const __bf16* __restrict__ q, int64_t sB, int64_t sN,
                                                             int64_t sH, int N, int H, int D,
                                                             float* __restrict__ part) {
  const int c = blockIdx.x, b = blockIdx.y, nc = gridDim.x;
  const int cpr = D / 8, nch = H * cpr;
  const int t0 = c * kAnchorTok, t1 = min(N, t0 + kAnchorTok);
  for (int ch = threadIdx.x; ch < nch; ch += blockDim.x) {
    const int h = ch / cpr, dc = ch % cpr;
    const __bf16* src = q + b * sB + h * sH + dc * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int t = t0; t < t1; ++t) {
      const bf16x8 v =  // streaming load: every row is read once
          __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)t * sN)));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
    }
    float* dst = part + (((int64_t)b * nc + c) * H + h) * D + dc * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = acc[e];
  }
}

// Anchor, stage 2: one workgroup per (b, h); group gi of 128 threads sums the
// partials c = gi, gi + 8, ... of one channel each, then the 8 group sums are
// added in order (fixed order: deterministic).
__global__ __launch_bounds__(1024) void anchor_final_kernel(const float* __restrict__ part, int nc, int H, int D,
                                                            int N, float* __restrict__ anchor) {
  __shared__ float red[8][128];
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int gi = threadIdx.x / 128, d = threadIdx.x % 128;
  float s = 0.f;
  if (d < D)
    for (int c = gi; c < nc; c += 8) s += part[(((int64_t)b * nc + c) * H + h) * D + d];
  red[gi][d] = s;
  __syncthreads();
  if (gi == 0 && d < D) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += red[k][d];
    anchor[(int64_t)bh * D + d] = t / (float)N;
  }
}

template <int D>
__global__ __launch_bounds__(256) void summary_kernel(SummaryParams p) {
  constexpr int LPR = D / 8;      // lanes per row (16-byte chunks)
  constexpr int RPI = 64 / LPR;   // rows per step
  constexpr int STEPS = 64 / RPI; // steps covering a block of up to 64 rows
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * 4 + w;  // (b*H + h)*J + j
  if (item >= (int64_t)p.B * p.H * p.J) return;      // whole wave
  const int j = (int)(item % p.J);
  const int64_t bh = item / p.J;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int n = p.block_len[j];
  const int sub = lane / LPR, dc = lane % LPR;

  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = p.anchor[bh * D + dc * 8 + e];
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k) + b * p.sB + h * p.sH + dc * 8;
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v) + b * p.sB + h * p.sH + dc * 8;
  const int32_t* members = p.perm + (int64_t)j * p.M;

  bf16x8 kr[STEPS], vr[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int r = st * RPI + sub;
    const int64_t tok = members[min(r, n - 1)];
    // streaming loads: every key and value row is read once
    kr[st] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kg + tok * p.sN)));
    vr[st] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + tok * p.sN)));
  }

  // logits of the rows against the anchor (every lane of a row ends with it)
  float s[STEPS];
  float mx = -INFINITY;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += a[e] * (float)kr[st][e];
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) part += __shfl_xor(part, o, 64);
    s[st] = (st * RPI + sub < n) ? part * p.scale : -INFINITY;
    mx = fmaxf(mx, s[st]);
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));

  // weights, mass and the weighted key / value
  float z = 0.f, ks[8], vs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ks[e] = vs[e] = 0.f;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const float wgt = __expf(s[st] - mx);  // 0 for rows past the block
    z += wgt;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ks[e] += wgt * (float)kr[st][e];
      vs[e] += wgt * (float)vr[st][e];
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
    z += __shfl_xor(z, o, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ks[e] += __shfl_xor(ks[e], o, 64);
      vs[e] += __shfl_xor(vs[e], o, 64);
    }
  }
  const float inv = 1.f / z;
  bf16x8 kb, vb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kb[e] = (__bf16)(ks[e] * inv);
    vb[e] = (__bf16)(vs[e] * inv);
  }
  // bias with the stored (rounded) key
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dot += a[e] * (float)kb[e];
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o, 64);
  const float bias = mx + __logf(z) - p.scale * dot;
  if (sub == 0) {
    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(p.k_sum) + item * D + dc * 8) = kb;
    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(p.v_sum) + item * D + dc * 8) = vb;
  }
  if (lane == 0) p.b_sum[item] = bias;
}

size_t anchor_workspace_bytes(int B, int N, int H, int D) {
  const size_t nc = (size_t)((N + kAnchorTok - 1) / kAnchorTok);
  return nc * (size_t)B * H * D * sizeof(float);
}

hipError_t launch_anchor(const void* q, int64_t sB, int64_t sN, int64_t sH, int B, int N, int H, int D, float* part,
                         float* anchor, hipStream_t s) {
  const int nc = (N + kAnchorTok - 1) / kAnchorTok;
  // the fewest whole waves that give every 8-channel chunk of a token row a thread
  const int nch = H * (D / 8);
  const int threads = std::min(1024, (nch + 63) / 64 * 64);
  anchor_partial_kernel<<<dim3((unsigned)nc, (unsigned)B), dim3(threads), 0, s>>>(
      reinterpret_cast<const __bf16*>(q), sB, sN, sH, N, H, D, part);
  anchor_final_kernel<<<dim3((unsigned)(B * H)), dim3(1024), 0, s>>>(part, nc, H, D, N, anchor);
  return hipGetLastError();
}

hipError_t launch_summaries(const SummaryParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.H * p.J;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (p.D == 128)
    summary_kernel<128><<<grid, dim3(256), 0, s>>>(p);
  else
    summary_kernel<64><<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsa
