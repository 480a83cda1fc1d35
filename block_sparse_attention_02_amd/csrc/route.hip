// Tiling tables, per-block mean pooling and the fused routing-score + TopK
// kernel for gfx950.
//
// Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" -- section 1
// (3D blocks, token numbering, true lengths of edge blocks), section 2.1
// (per-block means of Q and K per batch and head, divided by the true length),
// section 2.2 (E = Q_bar K_bar^T / sqrt(D), per-row TopK on the logits) and
// section 4 (kept block ids in increasing order, -1 fill, separate count).
#include <type_traits>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

// ============================================================================
// Tiling: one thread per packed slot p = b*M + r.
// ============================================================================
__global__ void tile_index_kernel(int T, int H, int W, int bT, int bH, int bW, int JH, int JW, int M,
                                  int J, int32_t* __restrict__ perm, int32_t* __restrict__ block_len,
                                  int32_t* __restrict__ inv) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= (int64_t)J * M) return;
  const int b = (int)(p / M), r = (int)(p % M);
  const int bt = b / (JH * JW), rem = b % (JH * JW), by = rem / JW, bx = rem % JW;
  const int t0 = bt * bT, y0 = by * bH, x0 = bx * bW;
  const int nt = min(bT, T - t0), ny = min(bH, H - y0), nx = min(bW, W - x0);
  const int n = nt * ny * nx;
  if (r == 0) block_len[b] = n;
  if (r < n) {
    // members listed with t slowest and x fastest over the block's valid extent
    const int dt = r / (ny * nx), rr = r % (ny * nx), dy = rr / nx, dx = rr % nx;
    const int tok = ((t0 + dt) * H + (y0 + dy)) * W + (x0 + dx);
    perm[p] = tok;
    if (inv) inv[tok] = (int32_t)p;
  } else {
    perm[p] = -1;
  }
}

hipError_t launch_tile_index(int T, int H, int W, int bT, int bH, int bW, int J, int M, int32_t* perm,
                             int32_t* block_len, int32_t* inv, hipStream_t s) {
  const int JH = (H + bH - 1) / bH, JW = (W + bW - 1) / bW;
  const int64_t total = (int64_t)J * M;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  tile_index_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(T, H, W, bT, bH, bW, JH, JW, M, J,
                                                                      perm, block_len, inv);
  return hipGetLastError();
}

// ============================================================================
// Pool: one workgroup per (block i, batch b, tensor) -- tensor 0 is q (into
// qbar), tensor 1 is k (into kbar); a single-tensor launch pools q only.  Each token row of all
// heads is read with 16-byte loads (VW elements) and accumulated in fp32; the
// sum is divided by the block's true length.  Loads are unconditional (lanes
// past the row read a clamped address and discard it) so that the UT x CPT
// loads of an iteration are all in flight together.
// ============================================================================
template <typename T, int VW, int CPT>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p, int nsplit) {
  constexpr int UT = (CPT <= 2) ? 8 : 4;  // tokens per iteration
  using Vec = typename std::conditional<VW == 1, T, u32x4>::type;
  // blockIdx.z = tensor * nsplit + part: part takes a contiguous share of the
  // (head, chunk) range, so small grids still fill the chip
  const int tsel = blockIdx.z / nsplit, part = blockIdx.z % nsplit;
  const T* __restrict__ x = reinterpret_cast<const T*>(tsel ? p.k : p.q);
  float* __restrict__ out = tsel ? p.kbar : p.qbar;
  const int i = blockIdx.x, b = blockIdx.y;
  const int n = p.block_len[i];
  const int cpr = p.D / VW;  // vector chunks per head row
  const int nch = p.H * cpr;
  const int cw = (nch + nsplit - 1) / nsplit;
  const int cbeg = part * cw, cend = min(nch, cbeg + cw);
  const T* __restrict__ xb = x + (int64_t)b * p.sB;
  for (int c0 = cbeg; c0 < cend; c0 += 256 * CPT) {
    float acc[CPT][VW];
    int64_t off[CPT];
    const int32_t* members[CPT];  // the block's members in this chunk's head (per-head tables)
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = min(c0 + (int)threadIdx.x + 256 * u, cend - 1);
      off[u] = (int64_t)(c / cpr) * p.sH + (int64_t)(c % cpr) * VW;
      members[u] = p.perm + ((int64_t)b * p.H + c / cpr) * p.perm_bh_stride + (int64_t)i * p.M;
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[u][e] = 0.f;
    }
    for (int r = 0; r < n; r += UT) {
      Vec v[UT][CPT];
#pragma unroll
      for (int rr = 0; rr < UT; ++rr) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const T* row = xb + (int64_t)members[u][min(r + rr, n - 1)] * p.sN;
          // streaming loads: every row is read once
          v[rr][u] = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(row + off[u]));
        }
      }
#pragma unroll
      for (int rr = 0; rr < UT; ++rr) {
        const float wgt = (r + rr < n) ? 1.f : 0.f;  // no branch: keeps the loads batched
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          if constexpr (VW == 1) {
            acc[u][0] += wgt * (float)v[rr][u];
          } else {
            const T* e8 = reinterpret_cast<const T*>(&v[rr][u]);
#pragma unroll
            for (int e = 0; e < VW; ++e) acc[u][e] += wgt * (float)e8[e];
          }
        }
      }
    }
    const float fn = (float)n;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = c0 + threadIdx.x + 256 * u;
      if (c < cend) {
        const int hh = c / cpr, dc = c % cpr;
        float* dst = out + (((int64_t)b * p.H + hh) * p.J + i) * p.D + dc * VW;
#pragma unroll
        for (int e = 0; e < VW; ++e) dst[e] = acc[u][e] / fn;
      }
    }
  }
}

template <typename T, int VW>
static hipError_t launch_pool_t(const PoolParams& p, int ntensors, hipStream_t s) {
  const int nch = p.H * (p.D / VW);
  // below 8192 workgroups each block's (head, chunk) range is shared by two
  const int nsplit = ((int64_t)p.J * p.B * ntensors < 8192 && nch > 256) ? 2 : 1;
  const int cpt = ((nch + nsplit - 1) / nsplit + 255) / 256;
  dim3 grid(p.J, p.B, ntensors * nsplit);
  if (cpt <= 1)
    pool_kernel<T, VW, 1><<<grid, 256, 0, s>>>(p, nsplit);
  else if (cpt <= 2)
    pool_kernel<T, VW, 2><<<grid, 256, 0, s>>>(p, nsplit);
  else if (cpt <= 3)
    pool_kernel<T, VW, 3><<<grid, 256, 0, s>>>(p, nsplit);
  else
    pool_kernel<T, VW, 4><<<grid, 256, 0, s>>>(p, nsplit);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolParams& p, bool f32_input, bool vec, hipStream_t s, int ntensors) {
  if (f32_input) {
    if (vec) return launch_pool_t<float, 4>(p, ntensors, s);
    return launch_pool_t<float, 1>(p, ntensors, s);
  }
  if (vec) return launch_pool_t<__bf16, 8>(p, ntensors, s);
  return launch_pool_t<__bf16, 1>(p, ntensors, s);
}

// ============================================================================
// Fused routing scores + TopK.
//
// Workgroup = (batch*head, band of 16*RT query blocks), 8 waves.  Wave w owns
// the 16*NT key-block columns [w*16*NT, (w+1)*16*NT) of the band's score rows
// and keeps them in registers.  Scores E^T = K_bar Q_bar^T come from the
// 16x16x32 bf16 matrix cores with every fp32 operand split as hi + lo bf16
// (hi*hi + hi*lo + lo*hi), which keeps E at fp32 accuracy.  In the output
// layout lane l owns query rows 16*rt + l%16 and columns 4*(l/16) + v of each
// 16-column tile.  For D = 64, 128, 256 the pooled keys are split once per
// launch (route_split_kernel) into hi/lo planes laid out as the operand
// registers of each (16-column tile, 32-channel step): every band then reads
// 1 KiB contiguous per load instead of re-splitting the fp32 means.
//
// TopK per row: an exact search for the R-th largest order-preserving key (a
// radix select over LDS digit histograms for the top 16 bits, then a ballot
// search among the few keys that share them), then every key above the
// threshold is kept plus the lowest-index keys equal to it, and the kept ids
// are emitted in increasing order from per-row bit masks.
// ============================================================================
constexpr int kRouteWaves = 8;
constexpr int kBucket = 64;  // bucket keys gathered per row (more: plain rounds)

__device__ __forceinline__ int wave_excl_scan(int x) {
  const int lane = threadIdx.x & 63;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  return incl - x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Radix-select step over one row's 256-bin digit histogram (whole wave, bins
// 4*lane .. 4*lane+3): the digit d that holds the need-th largest key, so that
// count(digit > d) < need <= count(digit >= d), and count(digit > d).  The
// caller guarantees need <= the histogram's total.
__device__ __forceinline__ void hist_select(const uint32_t* h, int need, int* digit, int* above) {
  const int lane = threadIdx.x & 63;
  const uint4 v = *reinterpret_cast<const uint4*>(h + 4 * lane);
  const int s = (int)(v.x + v.y + v.z + v.w);
  int incl = s;  // keys in this lane's bins and every higher lane's
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += y;
  }
  const int cum = incl - s;  // keys in higher lanes' bins
  int d = -1, ab = 0;
  if (cum < need && incl >= need) {
    const int c3 = cum + (int)v.w, c2 = c3 + (int)v.z, c1 = c2 + (int)v.y;
    if (c3 >= need) { d = 4 * lane + 3; ab = cum; }
    else if (c2 >= need) { d = 4 * lane + 2; ab = c3; }
    else if (c1 >= need) { d = 4 * lane + 1; ab = c2; }
    else { d = 4 * lane; ab = c1; }
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(d >= 0);
  const int src = m ? __ffsll((long long)m) - 1 : 0;
  *digit = max(__shfl(d, src, 64), 0);
  *above = __shfl(ab, src, 64);
}

// KD: D when it is a multiple of 32 (compile-time fast path), else 0.
template <int NT, int RT, int KD>
__global__ __launch_bounds__(512) void route_topk_kernel(RouteParams p) {
  constexpr int BM = 16 * RT;              // query blocks per workgroup
  constexpr int CW = 16 * NT;              // columns per wave
  constexpr int MW = kRouteWaves * CW / 32;  // 32-bit mask words per row
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * BM;  // local query block (global row p.row0 + i)
  const int J = p.ncols, D = p.D;  // local key blocks j < J (global column p.col0 + j)
  const int NR = p.nrows, JT = p.J;
  const int KS = (D + 31) / 32;
  const int DP = KS * 32 + 8;  // padded LDS row (bf16 elements)

  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* qhi = reinterpret_cast<__bf16*>(smem);
  __bf16* qlo = qhi + BM * DP;
  uint32_t* gtm = reinterpret_cast<uint32_t*>(qlo + BM * DP);
  uint32_t* eqm = gtm + BM * MW;
  int* red = reinterpret_cast<int*>(eqm + BM * MW);  // [2][8][BM]
  int* bcnt = red + 2 * kRouteWaves * BM;                  // [BM] bucket sizes
  int* res = bcnt + BM;                                    // [BM] thresholds
  int* flag = res + BM;                                    // [4]: some bucket overflowed
  uint32_t* bkey = reinterpret_cast<uint32_t*>(flag + 4);  // [BM][kBucket]
  uint32_t* hist = bkey + BM * kBucket;                    // [BM][256] digit counts
  int* above = reinterpret_cast<int*>(hist + BM * 256);    // [2][BM] keys above each digit

  const float* __restrict__ qb = p.qbar + ((int64_t)bh * JT + p.row0) * D;
  const float* __restrict__ kb = p.kbar + ((int64_t)bh * JT + p.col0) * D;

  // ---- stage the band's pooled queries as hi/lo bf16 (zero padded) -------------
  for (int e = threadIdx.x; e < BM * KS * 32; e += 512) {
    const int r = e / (KS * 32), d = e % (KS * 32);
    const int i = i0 + r;
    const float x = (i < NR && d < D) ? qb[(int64_t)i * D + d] : 0.f;
    const __bf16 hi = (__bf16)x;
    qhi[r * DP + d] = hi;
    qlo[r * DP + d] = (__bf16)(x - (float)hi);
  }
  for (int e = threadIdx.x; e < 2 * BM * MW; e += 512) gtm[e] = 0u;
  for (int e = threadIdx.x; e < BM * 256; e += 512) hist[e] = 0u;
  for (int e = threadIdx.x; e < BM; e += 512) bcnt[e] = 0;
  if (threadIdx.x == 0) *flag = 0;
  __syncthreads();

  // ---- scores: E^T tiles for this wave's columns -----------------------------
  // order-preserving keys of this lane's scores (padding columns: key 0,
  // below every float)
  uint32_t key[RT][NT][4];
  const int g = lane >> 4, l16 = lane & 15;
  if constexpr (KD > 0) {
    // D = 64, 128, 256: operands from the hi/lo planes (one 16-byte load per
    // lane per plane and 32-channel step, tiles past the last one clamped),
    // the next column tile's fetched before this tile's products.
    constexpr int KS = KD / 32;
    const int nT = (J + 15) / 16;
    const int64_t plane = (int64_t)p.B * p.H * nT * KS * 512;  // bf16 elements per plane
    bf16x8 kh[2][KS], kl[2][KS];
    auto fetch = [&](int b, int t) {
      const int T = min(w * NT + t, nT - 1);
      const __bf16* src = p.kplanes + ((int64_t)bh * nT + T) * KS * 512 + lane * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kh[b][s] = *reinterpret_cast<const bf16x8*>(src + s * 512);
        kl[b][s] = *reinterpret_cast<const bf16x8*>(src + plane + s * 512);
      }
    };
    fetch(0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t + 1 < NT) fetch((t + 1) & 1, t + 1);
      f32x4 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int row = 16 * rt + l16;
          const bf16x8 qh = *reinterpret_cast<const bf16x8*>(qhi + row * DP + 32 * s + 8 * g);
          const bf16x8 ql = *reinterpret_cast<const bf16x8*>(qlo + row * DP + 32 * s + 8 * g);
          acc[rt] = mfma16(kl[t & 1][s], qh, acc[rt]);
          acc[rt] = mfma16(kh[t & 1][s], ql, acc[rt]);
          acc[rt] = mfma16(kh[t & 1][s], qh, acc[rt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float e = acc[rt][v] * p.scale;
          const int j = w * CW + 16 * t + 4 * g + v;
          key[rt][t][v] = (j < J) ? float_key(e) : 0u;
          if (j < J) atomicAdd(&hist[(16 * rt + l16) * 256 + (key[rt][t][v] >> 24)], 1u);
        }
    }
  } else {
    // any D <= 256: element-wise guarded loads (small problems)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int j0 = w * CW + 16 * t;
      const int jr = j0 + l16;
      f32x4 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j0 < J) {
        for (int s = 0; s < KS; ++s) {
          const int d0 = 32 * s + 8 * g;
          float kv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) kv[e] = (jr < J && d0 + e < D) ? kb[(int64_t)jr * D + d0 + e] : 0.f;
          bf16x8 khi, klo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            khi[e] = (__bf16)kv[e];
            klo[e] = (__bf16)(kv[e] - (float)khi[e]);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int row = 16 * rt + l16;
            const bf16x8 qh = *reinterpret_cast<const bf16x8*>(qhi + row * DP + d0);
            const bf16x8 ql = *reinterpret_cast<const bf16x8*>(qlo + row * DP + d0);
            acc[rt] = mfma16(klo, qh, acc[rt]);
            acc[rt] = mfma16(khi, ql, acc[rt]);
            acc[rt] = mfma16(khi, qh, acc[rt]);
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float e = acc[rt][v] * p.scale;
          const int j = w * CW + 16 * t + 4 * g + v;
          key[rt][t][v] = (j < J) ? float_key(e) : 0u;
          if (j < J) atomicAdd(&hist[(16 * rt + l16) * 256 + (key[rt][t][v] >> 24)], 1u);
        }
    }
  }

  if (p.E) {  // optional debug copy of the scores (the key map is a bijection)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = i0 + 16 * rt + l16, j = w * CW + 16 * t + 4 * g + v;
          if (i < NR && j < J) p.E[((int64_t)bh * JT + p.row0 + i) * JT + p.col0 + j] = key_float(key[rt][t][v]);
        }
  }

  // ---- exact threshold: the R-th largest key of every row ------------------------
  // Radix select: the top byte from the histogram built with the scores, then
  // the next byte from a histogram of the keys that share the top byte; that
  // fixes the threshold's top 16 bits.  The keys that share them (the row's
  // "bucket", a handful for continuous scores) are gathered in LDS and one
  // wave finds the exact rank among them with ballots.  When some row's bucket
  // holds more than kBucket keys the workgroup finishes with rounds over bits
  // 15..0 instead (count keys >= candidate across the row); both give the same
  // threshold.
  __syncthreads();
  for (int row = w; row < BM; row += kRouteWaves) {
    int d, ab;
    hist_select(hist + row * 256, p.R, &d, &ab);
    *reinterpret_cast<uint4*>(hist + row * 256 + 4 * lane) = uint4{0u, 0u, 0u, 0u};  // reused below
    if (lane == 0) { res[row] = d; above[row] = ab; }
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * rt + l16;
    const uint32_t d1 = (uint32_t)res[row];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t k = key[rt][t][v];
        if ((k >> 24) == d1 && (w * CW + 16 * t + 4 * g + v) < J)
          atomicAdd(&hist[row * 256 + ((k >> 16) & 255u)], 1u);
      }
  }
  __syncthreads();
  for (int row = w; row < BM; row += kRouteWaves) {
    const int d1 = res[row], ab1 = above[row];
    int d2, ab2;
    hist_select(hist + row * 256, p.R - ab1, &d2, &ab2);
    if (lane == 0) {
      above[BM + row] = ab1 + ab2;
      if (i0 + row < NR && hist[row * 256 + d2] > (uint32_t)kBucket) *flag = 1;  // rows past NR are not emitted
      res[row] = (int)(((uint32_t)d1 << 24) | ((uint32_t)d2 << 16));
    }
  }
  __syncthreads();
  uint32_t thr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) thr[rt] = (uint32_t)res[16 * rt + l16];
  int par = 0;
  auto round_bit = [&](int bit) {
    int cnt[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t cand = thr[rt] | (1u << bit);
      int c = 0;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) c += (key[rt][t][v] >= cand) ? 1 : 0;
      c += __shfl_xor(c, 16, 64);
      c += __shfl_xor(c, 32, 64);
      cnt[rt] = c;
    }
    if (lane < 16) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) red[(par * kRouteWaves + w) * BM + 16 * rt + lane] = cnt[rt];
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      int tot = 0;
#pragma unroll
      for (int ww = 0; ww < kRouteWaves; ++ww) tot += red[(par * kRouteWaves + ww) * BM + 16 * rt + l16];
      if (tot >= p.R) thr[rt] |= (1u << bit);
    }
    par ^= 1;
  };
  if (*flag) {
    for (int bit = 15; bit >= 0; --bit) round_bit(bit);
  } else {
    // bucket of each row: keys whose top 16 bits equal the threshold's
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = 16 * rt + l16;
      const uint32_t hi = thr[rt] >> 16;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t k = key[rt][t][v];
          if ((k >> 16) == hi && (w * CW + 16 * t + 4 * g + v) < J) {
            const int slot = atomicAdd(&bcnt[row], 1);
            if (slot < kBucket) bkey[row * kBucket + slot] = k;
          }
        }
    }
    __syncthreads();
    // the need-th largest bucket key, need = R - #keys above the bucket;
    // one wave per row, one bucket key per lane, ballots over the low 16 bits
    for (int row = w; row < BM; row += kRouteWaves) {
      const int need = p.R - above[BM + row];
      const int nb = bcnt[row];
      const uint32_t mine = lane < nb ? bkey[row * kBucket + lane] : 0u;
      uint32_t t32 = (uint32_t)res[row];
      for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cand = t32 | (1u << bit);
        const int c = __popcll(__builtin_amdgcn_ballot_w64(lane < nb && mine >= cand));
        if (c >= need) t32 = cand;
      }
      if (lane == 0) res[row] = (int)t32;
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) thr[rt] = (uint32_t)res[16 * rt + l16];
  }

  // ---- bit masks of keys above / equal to the threshold ------------------------
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * rt + l16;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t gt = 0u, eq = 0u;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        gt |= (key[rt][t][v] > thr[rt] ? 1u : 0u) << (4 * g + v);
        eq |= (key[rt][t][v] == thr[rt] ? 1u : 0u) << (4 * g + v);
      }
      gt |= __shfl_xor(gt, 16, 64);
      gt |= __shfl_xor(gt, 32, 64);
      eq |= __shfl_xor(eq, 16, 64);
      eq |= __shfl_xor(eq, 32, 64);
      const int j0 = w * CW + 16 * t;
      if (g == 0 && j0 < J) {
        const int word = j0 >> 5, sh = j0 & 31;
        if (gt) atomicOr(&gtm[row * MW + word], gt << sh);
        if (eq) atomicOr(&eqm[row * MW + word], eq << sh);
      }
    }
  }
  __syncthreads();

  // ---- emit kept ids in increasing order, one wave per row ----------------------
  for (int row = w; row < BM; row += kRouteWaves) {
    const int i = i0 + row;
    if (i >= NR) continue;
    int32_t* __restrict__ out = p.q2k_idx + ((int64_t)bh * JT + p.row0 + i) * p.kmax + p.out_off;
    int ngt = 0;
    for (int wb = 0; wb < MW; wb += 64) {
      const int word = wb + lane;
      ngt += wave_sum(word < MW ? __popc(gtm[row * MW + word]) : 0);
    }
    const int need_eq = p.R - ngt;
    int eq_carry = 0, sel_carry = 0;
    for (int wb = 0; wb < MW; wb += 64) {
      const int word = wb + lane;
      const uint32_t gw = word < MW ? gtm[row * MW + word] : 0u;
      uint32_t ew = word < MW ? eqm[row * MW + word] : 0u;
      const int ne = __popc(ew);
      const int eq_before = eq_carry + wave_excl_scan(ne);
      int take = min(max(need_eq - eq_before, 0), ne);
      uint32_t takebits = 0u;
      while (take-- > 0) {
        const uint32_t low = ew & (0u - ew);
        takebits |= low;
        ew ^= low;
      }
      uint32_t sel = gw | takebits;
      const int ns = __popc(sel);
      int pos = sel_carry + wave_excl_scan(ns);
      while (sel) {
        const int bitpos = __ffs(sel) - 1;
        out[pos++] = p.col0 + word * 32 + bitpos;
        sel &= sel - 1u;
      }
      eq_carry += wave_sum(ne);
      sel_carry += wave_sum(ns);
    }
    if (p.tail) {
      for (int q = p.R + lane; q < p.kmax; q += 64) out[q] = -1;
      if (lane == 0) p.q2k_num[(int64_t)bh * JT + p.row0 + i] = p.R;
    }
  }
}

template <int NT, int RT, int KD>
static hipError_t launch_route_k(const RouteParams& p, size_t smem, hipStream_t s) {
  constexpr int BM = 16 * RT;
  dim3 grid((p.nrows + BM - 1) / BM, p.B * p.H);
  route_topk_kernel<NT, RT, KD><<<grid, 512, smem, s>>>(p);
  return hipGetLastError();
}

template <int NT, int RT>
static hipError_t launch_route_t(const RouteParams& p, hipStream_t s) {
  constexpr int BM = 16 * RT;
  constexpr int MW = kRouteWaves * 16 * NT / 32;
  const int KS = (p.D + 31) / 32, DP = KS * 32 + 8;
  const size_t smem = (size_t)2 * BM * DP * sizeof(__bf16) + (size_t)2 * BM * MW * 4 +
                      (size_t)2 * kRouteWaves * BM * 4 + (size_t)(2 * BM + 4) * 4 + (size_t)BM * kBucket * 4 +
                      (size_t)BM * 256 * 4 + (size_t)2 * BM * 4;
  switch (p.D) {
    case 64: return launch_route_k<NT, RT, 64>(p, smem, s);
    case 128: return launch_route_k<NT, RT, 128>(p, smem, s);
    case 256: return launch_route_k<NT, RT, 256>(p, smem, s);
    default: return launch_route_k<NT, RT, 0>(p, smem, s);
  }
}

// ---------------------------------------------------------------------------
// Processing order for the attention kernel.  Query blocks whose kept lists
// have similar quartile entries read overlapping windows of K/V; listing them
// next to each other lets the workgroups that run at the same time share L2.
// One workgroup per (b, h) sorts (Morton code of the three quartiles, 10 bits
// each; block index) keys with a bitonic network: the compare-exchange stages
// between elements less than 64 apart run inside a wave on registers (one
// LDS load and store per element for all of them), the wider ones through LDS
// with a barrier each.  Blocks below num_first (the H3 context rows, whose
// lists hold every block) come first, in index order.  The order changes no
// attention result.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t spread3_10(uint32_t v) {
  v &= 0x3ffu;
  v = (v | (v << 16)) & 0x030000FFu;
  v = (v | (v << 8)) & 0x0300F00Fu;
  v = (v | (v << 4)) & 0x030C30C3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}

__global__ __launch_bounds__(1024) void item_order_kernel(const int32_t* __restrict__ q2k_idx,
                                                          const int32_t* __restrict__ q2k_num, int J, int kmax,
                                                          int num_first, int np, int32_t* __restrict__ order) {
  __shared__ uint64_t key[kRouteMaxJ];
  const int64_t bh = blockIdx.x;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    uint64_t kk = ~0ull;
    if (i < J) {
      const int32_t* row = q2k_idx + (bh * J + i) * (int64_t)kmax;
      const int n = min(q2k_num[bh * J + i], kmax);
      uint32_t code = 0;
      if (n > 0) {
        const int pos[3] = {(n - 1) / 4, (n - 1) / 2, 3 * (n - 1) / 4};
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          const int v = min(max(row[pos[c]], 0), J - 1);
          code |= spread3_10((uint32_t)((int64_t)v * 1024 / J)) << c;
        }
      }
      if (i < num_first) code = 0u;  // key i: below every other block's key
      kk = ((uint64_t)code << 32) | (uint32_t)i;
    }
    key[i] = kk;
  }
  __syncthreads();
  // compare-exchange of elements i and i ^ j, ascending where (i & k) == 0
  auto lds_stage = [&](int k, int j) {
    for (int i = threadIdx.x; i < np; i += blockDim.x) {
      const int l = i ^ j;
      if (l > i) {
        const uint64_t a = key[i], b = key[l];
        if ((a > b) == ((i & k) == 0)) {
          key[i] = b;
          key[l] = a;
        }
      }
    }
    __syncthreads();
  };
  if (np < 64) {
    for (int k = 2; k <= np; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) lds_stage(k, j);
  } else {
    // stages k0..k1 (merge sizes) with j < 64 on 64-element chunks, one per wave
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    auto wave_stages = [&](int k0, int k1) {
      for (int c = threadIdx.x >> 6; c < np / 64; c += nw) {
        const int i = c * 64 + lane;
        uint64_t v = key[i];
        for (int k = k0; k <= k1; k <<= 1) {
          const bool up = (i & k) == 0;
          for (int j = min(k >> 1, 32); j > 0; j >>= 1) {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, j, 64);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), j, 64);
            const uint64_t o = ((uint64_t)hi << 32) | lo;
            const bool take_min = ((lane & j) == 0) == up;
            v = (take_min == (o < v)) ? o : v;
          }
        }
        key[i] = v;
      }
      __syncthreads();
    };
    wave_stages(2, 64);
    for (int k = 128; k <= np; k <<= 1) {
      for (int j = k >> 1; j >= 64; j >>= 1) lds_stage(k, j);
      wave_stages(k, k);
    }
  }
  for (int i = threadIdx.x; i < J; i += blockDim.x) order[bh * J + i] = (int32_t)(uint32_t)key[i];
}

hipError_t launch_item_order(const int32_t* q2k_idx, const int32_t* q2k_num, int BH, int J, int kmax,
                             int num_first, int32_t* order, hipStream_t s) {
  int np = 1;
  while (np < J) np <<= 1;
  if (np > kRouteMaxJ) return hipErrorInvalidValue;
  item_order_kernel<<<dim3((unsigned)BH), dim3(1024), 0, s>>>(q2k_idx, q2k_num, J, kmax, num_first, np, order);
  return hipGetLastError();
}

// ============================================================================
// H3 multi-region layout ("VSA 实现详解" section 5.2): dense segments cut into 1D
// chunks of M tokens (each segment on its own) form the prefix; the video
// regions follow, each tiled in 3D like a single video.  One thread per packed
// slot; the block's part is found by a short scan of the (at most 16) parts.
// ============================================================================
__global__ void h3_tile_index_kernel(H3Layout L, int J, int32_t* __restrict__ perm,
                                     int32_t* __restrict__ block_len, int32_t* __restrict__ inv) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int M = L.M;
  if (p >= (int64_t)J * M) return;
  const int b = (int)(p / M), r = (int)(p % M);
  int k = 0;
  while (k + 1 < L.nparts && b >= L.part[k].b1) ++k;
  const H3Part& P = L.part[k];
  const int lb = b - P.b0;
  int n, tok = -1;
  if (!P.video) {
    n = min(M, P.n - lb * M);
    if (r < n) tok = P.tok0 + lb * M + r;
  } else {
    const int bt = lb / (P.JH * P.JW), rem = lb % (P.JH * P.JW), by = rem / P.JW, bx = rem % P.JW;
    const int t0 = bt * L.bT, y0 = by * L.bH, x0 = bx * L.bW;
    const int nt = min(L.bT, P.T - t0), ny = min(L.bH, P.H - y0), nx = min(L.bW, P.W - x0);
    n = nt * ny * nx;
    if (r < n) {
      const int dt = r / (ny * nx), rr = r % (ny * nx), dy = rr / nx, dx = rr % nx;
      tok = P.tok0 + ((t0 + dt) * P.H + (y0 + dy)) * P.W + (x0 + dx);
    }
  }
  if (r == 0) block_len[b] = n;
  perm[p] = tok;
  if (tok >= 0 && inv) inv[tok] = (int32_t)p;
}

hipError_t launch_h3_tile_index(const H3Layout& L, int J, int32_t* perm, int32_t* block_len, int32_t* inv,
                                hipStream_t s) {
  const int64_t total = (int64_t)J * L.M;
  const int64_t blocks = (total + 255) / 256;
  h3_tile_index_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(L, J, perm, block_len, inv);
  return hipGetLastError();
}

// Grouped routing ("VSA 实现详解" section 5.3, exempt rule): the per-region TopK
// launches write the region entries of every video row; this kernel writes the
// rest -- a context row keeps every block, a video row the prefix blocks in
// front of its region entries -- the -1 fill (when `fill`) and the counts.  One
// wave per row.
__global__ __launch_bounds__(256) void h3_fill_kernel(int32_t* __restrict__ q2k_idx, int32_t* __restrict__ q2k_num,
                                                      int64_t rows, int J, int kmax, int num_prefix, int nsel,
                                                      int fill) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int i = (int)(row % J);
  int32_t* out = q2k_idx + row * kmax;
  const bool context = i < num_prefix;
  const int keep = context ? J : nsel;
  const int end = fill ? kmax : (context ? J : num_prefix);
  for (int q = lane; q < end; q += 64) {
    if (context ? q < J : q < num_prefix)
      out[q] = q;
    else if (q >= keep)
      out[q] = -1;
  }
  if (lane == 0) q2k_num[row] = keep;
}

hipError_t launch_h3_fill(int32_t* q2k_idx, int32_t* q2k_num, int BH, int J, int kmax, int num_prefix, int nsel,
                          bool fill, hipStream_t s) {
  const int64_t rows = (int64_t)BH * J;
  h3_fill_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(q2k_idx, q2k_num, rows, J, kmax, num_prefix,
                                                                       nsel, fill ? 1 : 0);
  return hipGetLastError();
}

// hi/lo planes of the pooled keys of columns [col0, col0 + ncols): for each
// (b*h, 16-column tile T, 32-channel step s) 64 lanes x 8 bf16, lane l holding
// channels 32s + 8(l/16) .. +7 of column 16T + l%16 (zero past ncols), the
// hi plane then the lo plane (lo = x - hi, both rounded to nearest).  One
// thread per lane slot.
__global__ __launch_bounds__(256) void route_split_kernel(const float* __restrict__ kbar, __bf16* __restrict__ out,
                                                          int64_t slots, int JT, int col0, int ncols, int nT, int KS,
                                                          int D) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= slots) return;
  const int lane = (int)(id & 63);
  const int64_t u = id >> 6;
  const int s = (int)(u % KS);
  const int64_t T = (u / KS) % nT, bh = u / KS / nT;
  const int j = (int)(16 * T) + (lane & 15);
  const int d0 = 32 * s + 8 * (lane >> 4);
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, c = a;
  if (j < ncols) {
    const float* src = kbar + (bh * JT + col0 + j) * D + d0;
    a = *reinterpret_cast<const f32x4*>(src);
    c = *reinterpret_cast<const f32x4*>(src + 4);
  }
  const float x[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  bf16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
  *reinterpret_cast<bf16x8*>(out + id * 8) = h;
  *reinterpret_cast<bf16x8*>(out + (slots + id) * 8) = l;
}

static bool route_uses_planes(int D) { return D == 64 || D == 128 || D == 256; }

size_t route_planes_bytes(int BH, int ncols, int D) {
  if (!route_uses_planes(D)) return 0;
  return (size_t)BH * ((ncols + 15) / 16) * (D / 32) * 64 * 8 * sizeof(__bf16) * 2;
}

hipError_t launch_route_topk(const RouteParams& p, hipStream_t s) {
  if (route_uses_planes(p.D)) {
    if (!p.kplanes) return hipErrorInvalidValue;
    const int nT = (p.ncols + 15) / 16, KS = p.D / 32;
    const int64_t slots = (int64_t)p.B * p.H * nT * KS * 64;
    route_split_kernel<<<dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s>>>(p.kbar, p.kplanes, slots, p.J,
                                                                                   p.col0, p.ncols, nT, KS, p.D);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int cols_per_wave = (p.ncols + kRouteWaves - 1) / kRouteWaves;
  if (cols_per_wave <= 16) return launch_route_t<1, 2>(p, s);
  if (cols_per_wave <= 32) return launch_route_t<2, 2>(p, s);
  if (cols_per_wave <= 64) return launch_route_t<4, 1>(p, s);  // 16-row bands measured faster here
  if (cols_per_wave <= 128) return launch_route_t<8, 2>(p, s);
  // 16-row bands here: 64 keys per lane leave room for two workgroups per CU
  if (cols_per_wave <= 256) return launch_route_t<16, 1>(p, s);
  return launch_route_t<32, 1>(p, s);
}

}  // namespace bsa
