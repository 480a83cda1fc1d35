// Spark-Reblock reordering for gfx950.
//
// Source: "深度解读|Spark-H3：从注意力几何到稀疏内核代码" -- section 04 (Q
// permuted, K and V bound to the same key permutation, outputs returned to
// their positions), section 05 (keys are grouped under the query-side
// uncentred second moment M_Q = Q^T Q / N: the cosine of two keys' features
// k^T L, L L^T = M_Q, is the cosine of their score profiles over all queries)
// and section 06 (an equal-capacity hierarchy of 64-token leaves whose split
// directions come from midpoint landmarks; the default layout mode builds the
// key layout and lets the queries reuse it).
//
// Reading of the production heuristic (fanout 16, 32 landmarks): binary
// equal-capacity splits.  A node of n tokens spans c = ceil(n / M) leaves; its
// first child takes floor(c / 2) * M tokens.  The node ranges depend on N and
// M only, so every level is: one direction per node (32 landmarks at ranks
// floor((2s+1) n / 64) of the node's current order, their centred Gram
// matrix, 16 power iterations from the ramp a_s = s - 15.5 (centring puts the
// all-ones vector in the Gram matrix's null space), v = X^T a normalised,
// largest entry positive), one projection key per token, and one stable
// radix sort of (head, node, projection) keys that leaves every node's tokens
// in projection order -- the first child's tokens first, in place.
//
// Design (MI355X): the moment is an fp32 outer-product accumulation over
// 2048-token chunks (each thread an 8 x 8 tile of the D x D matrix), reduced
// in a fixed order, ridged and factored by a one-workgroup Cholesky in LDS;
// the unit features u = z / |z|, z = k^T L, are formed with L resident in LDS.
// Decisions (projections, sort keys) are taken in fp32.
#include <hipcub/hipcub.hpp>

#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kMomentChunk = 2048;  // tokens per partial moment
constexpr int kLandmarks = 32;
constexpr int kPowerIters = 16;
static_assert(kLandmarks == 32, "the ramp start's norm (2728 = sum of (s - 15.5)^2) assumes 32 landmarks");

// ---- tree geometry --------------------------------------------------------------
// Range of slot `slot` at level `level` (start, size, leaves); empty: n = c = 0.
__device__ __forceinline__ void slot_range(int N, int M, int level, int slot, int* start, int* n, int* c) {
  int st = 0, nn = N, cc = (N + M - 1) / M;
  for (int l = level - 1; l >= 0; --l) {
    const int bit = (slot >> l) & 1;
    if (cc <= 1) {
      if (bit == 0) nn = cc = 0;  // a leaf's first child is empty, its second is itself
      continue;
    }
    const int cl = cc / 2, nl = cl * M;
    if (bit == 0) {
      nn = nl, cc = cl;
    } else {
      st += nl, nn -= nl, cc -= cl;
    }
  }
  *start = st, *n = nn, *c = cc;
}

// Slot holding position pos at level `level`, with that slot's leaf count.
__device__ __forceinline__ int slot_of(int N, int M, int level, int pos, int* c) {
  int s = 0, st = 0, cc = (N + M - 1) / M;
  for (int l = 0; l < level; ++l) {
    if (cc <= 1) {
      s = 2 * s + 1;
      continue;
    }
    const int cl = cc / 2, nl = cl * M;
    if (pos < st + nl) {
      s = 2 * s, cc = cl;
    } else {
      s = 2 * s + 1, st += nl, cc -= cl;
    }
  }
  *c = cc;
  return s;
}

int reblock_levels(int N, int M) {
  int c = (N + M - 1) / M, depth = 0;
  while ((1 << depth) < c) ++depth;  // ceil(log2(c)) split levels
  return depth + 1;
}

// ---- second moment -----------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void moment_partial_kernel(const __bf16* __restrict__ q, int64_t sB, int64_t sN,
                                                             int64_t sH, int H, int N, float* __restrict__ part) {
  constexpr int T = D / 16;  // tile edge per thread
  constexpr int TOK = 32;    // tokens staged per step
  __shared__ __align__(16) float xs[TOK][D];
  const int c = blockIdx.x, bh = blockIdx.y, BH = gridDim.y;
  const int b = bh / H, h = bh % H;
  const int t0 = c * kMomentChunk, t1 = min(N, t0 + kMomentChunk);
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
  const __bf16* __restrict__ src = q + b * sB + h * sH;
  float acc[T][T];
#pragma unroll
  for (int i = 0; i < T; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j) acc[i][j] = 0.f;
  for (int base = t0; base < t1; base += TOK) {
    for (int e = threadIdx.x; e < TOK * D / 8; e += 256) {
      const int r = e / (D / 8), cc = e % (D / 8);
      const int tok = base + r;
      f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
      if (tok < t1) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + (int64_t)tok * sN + cc * 8);
        lo = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
        hi = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
      }
      *reinterpret_cast<f32x4*>(&xs[r][cc * 8]) = lo;
      *reinterpret_cast<f32x4*>(&xs[r][cc * 8 + 4]) = hi;
    }
    __syncthreads();
    for (int r = 0; r < TOK; ++r) {
      float a[T], bb[T];
#pragma unroll
      for (int i = 0; i < T; i += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&xs[r][ti * T + i]);
        const f32x4 y = *reinterpret_cast<const f32x4*>(&xs[r][tj * T + i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[i + e] = x[e], bb[i + e] = y[e];
      }
#pragma unroll
      for (int i = 0; i < T; ++i)
#pragma unroll
        for (int j = 0; j < T; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* __restrict__ dst = part + ((int64_t)c * BH + bh) * D * D;
#pragma unroll
  for (int i = 0; i < T; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j) dst[(ti * T + i) * D + tj * T + j] = acc[i][j];
}

// Sum of the partials in chunk order, / N, ridge, Cholesky (right-looking,
// column by column, in LDS).  A pivot that rounding drives below the ridge is
// clamped to it.
template <int D>
__global__ __launch_bounds__(1024) void moment_factor_kernel(const float* __restrict__ part, int nc, int N,
                                                             float ridge, float* __restrict__ moment,
                                                             float* __restrict__ factor) {
  __shared__ float A[D][D + 1];
  __shared__ float lam_sh;
  const int bh = blockIdx.x, BH = gridDim.x;
  for (int e = threadIdx.x; e < D * D; e += 1024) {
    float s = 0.f;
    for (int c = 0; c < nc; ++c) s += part[((int64_t)c * BH + bh) * D * D + e];
    s /= (float)N;
    A[e / D][e % D] = s;
    if (moment) moment[(int64_t)bh * D * D + e] = s;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    float t = 0.f;
    for (int d = threadIdx.x; d < D; d += 64) t += A[d][d];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
    if (threadIdx.x == 0) lam_sh = ridge * ((t > 0.f) ? t / (float)D : 1.f);
  }
  __syncthreads();
  const float lam = lam_sh;
  for (int d = threadIdx.x; d < D; d += 1024) A[d][d] += lam;
  __syncthreads();
  for (int j = 0; j < D; ++j) {
    if (threadIdx.x == 0) A[j][j] = sqrtf(fmaxf(A[j][j], lam));
    __syncthreads();
    const float djj = A[j][j];
    for (int i = j + 1 + threadIdx.x; i < D; i += 1024) A[i][j] /= djj;
    __syncthreads();
    const int m = D - j - 1;
    for (int e = threadIdx.x; e < m * m; e += 1024) {
      const int i = j + 1 + e / m, k = j + 1 + e % m;
      if (k <= i) A[i][k] = fmaf(-A[i][j], A[k][j], A[i][k]);
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < D * D; e += 1024) {
    const int i = e / D, k = e % D;
    factor[(int64_t)bh * D * D + e] = (k <= i) ? A[i][k] : 0.f;
  }
}

// ---- key features: u = z / |z|, z_d = sum_e k_e L[e][d] ----------------------------
template <int D>
__global__ __launch_bounds__(256) void key_feature_kernel(const __bf16* __restrict__ k, int64_t sB, int64_t sN,
                                                          int64_t sH, int H, int N, const float* __restrict__ factor,
                                                          float* __restrict__ u) {
  constexpr int TOKS = 64;   // tokens per workgroup (4 threads each)
  constexpr int QD = D / 4;  // channels per thread
  __shared__ __align__(16) float Ls[D * D];
  __shared__ __align__(16) float ks[TOKS][D + 4];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int tok0 = blockIdx.x * TOKS;
  const float* __restrict__ Lg = factor + (int64_t)bh * D * D;
  for (int e = threadIdx.x; e < D * D / 4; e += 256)
    *reinterpret_cast<f32x4*>(&Ls[4 * e]) = *reinterpret_cast<const f32x4*>(Lg + 4 * e);
  const __bf16* __restrict__ src = k + b * sB + h * sH;
  for (int e = threadIdx.x; e < TOKS * D / 8; e += 256) {
    const int r = e / (D / 8), cc = e % (D / 8);
    const int tok = tok0 + r;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    if (tok < N) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + (int64_t)tok * sN + cc * 8);
      lo = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
      hi = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
    }
    *reinterpret_cast<f32x4*>(&ks[r][cc * 8]) = lo;
    *reinterpret_cast<f32x4*>(&ks[r][cc * 8 + 4]) = hi;
  }
  __syncthreads();
  const int r = threadIdx.x / 4, qd = threadIdx.x % 4;
  float z[QD];
#pragma unroll
  for (int d = 0; d < QD; ++d) z[d] = 0.f;
  for (int e = 0; e < D; ++e) {
    const float ke = ks[r][e];
    const float* Lrow = Ls + e * D + qd * QD;
#pragma unroll
    for (int d = 0; d < QD; d += 4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lrow + d);
#pragma unroll
      for (int x = 0; x < 4; ++x) z[d + x] = fmaf(ke, l4[x], z[d + x]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < QD; ++d) ss = fmaf(z[d], z[d], ss);
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  const float inv = (ss > 0.f) ? 1.f / sqrtf(ss) : 0.f;
  const int tok = tok0 + r;
  if (tok < N) {
    float* __restrict__ dst = u + ((int64_t)bh * N + tok) * D + qd * QD;
#pragma unroll
    for (int d = 0; d < QD; d += 4)
      *reinterpret_cast<f32x4*>(dst + d) = f32x4{z[d] * inv, z[d + 1] * inv, z[d + 2] * inv, z[d + 3] * inv};
  }
}

// ---- one level: split directions --------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void reblock_direction_kernel(const float* __restrict__ u,
                                                                const int32_t* __restrict__ order, int N, int M,
                                                                int level, int max_slots, float* __restrict__ dirs) {
  const int slot = blockIdx.x, bh = blockIdx.y;
  int start, n, c;
  slot_range(N, M, level, slot, &start, &n, &c);
  if (c <= 1) return;  // whole workgroup
  __shared__ float X[kLandmarks][D + 1];
  __shared__ float G[kLandmarks][kLandmarks + 1];
  __shared__ float a_sh[kLandmarks];
  __shared__ float red_v[256];
  __shared__ int red_i[256];
  const int32_t* __restrict__ ord = order + (int64_t)bh * N + start;
  for (int e = threadIdx.x; e < kLandmarks * D; e += 256) {
    const int s = e / D, d = e % D;
    const int tok = ord[(int)(((int64_t)(2 * s + 1) * n) / (2 * kLandmarks))];
    X[s][d] = u[((int64_t)bh * N + tok) * D + d];
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += 256) {
    float m = 0.f;
    for (int s = 0; s < kLandmarks; ++s) m += X[s][d];
    m /= (float)kLandmarks;
    for (int s = 0; s < kLandmarks; ++s) X[s][d] -= m;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kLandmarks * kLandmarks; e += 256) {
    const int s = e / kLandmarks, t = e % kLandmarks;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(X[s][d], X[t][d], acc);
    G[s][t] = acc;
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // power iteration, one wave, lane s < 32 holds a_s
    const int lane = threadIdx.x;
    // ramp start s - 15.5, normalised: |ramp|^2 = sum (s - 15.5)^2 = 2728 for 32 landmarks
    float a = (lane < kLandmarks) ? ((float)lane - 0.5f * (kLandmarks - 1)) * rsqrtf(2728.f) : 0.f;
    for (int it = 0; it < kPowerIters; ++it) {
      float w = 0.f;
      for (int t = 0; t < kLandmarks; ++t) {
        const float at = __shfl(a, t, 64);
        if (lane < kLandmarks) w = fmaf(G[lane][t], at, w);
      }
      float n2 = w * w;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) n2 += __shfl_xor(n2, o, 64);
      if (n2 == 0.f) {  // uniform: the landmarks coincide
        a = w;
        break;
      }
      a = w / sqrtf(n2);
    }
    if (lane < kLandmarks) a_sh[lane] = a;
  }
  __syncthreads();
  float vd = 0.f;
  const int d = threadIdx.x;
  if (d < D)
    for (int s = 0; s < kLandmarks; ++s) vd = fmaf(X[s][d], a_sh[s], vd);
  red_v[threadIdx.x] = vd * vd;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red_v[threadIdx.x] += red_v[threadIdx.x + o];
    __syncthreads();
  }
  const float nrm = sqrtf(red_v[0]);
  __syncthreads();
  // largest |v_d|, lowest d on ties
  red_v[threadIdx.x] = (d < D) ? fabsf(vd) : -1.f;
  red_i[threadIdx.x] = d;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const float x = red_v[threadIdx.x + o];
      const int xi = red_i[threadIdx.x + o];
      if (x > red_v[threadIdx.x] || (x == red_v[threadIdx.x] && xi < red_i[threadIdx.x]))
        red_v[threadIdx.x] = x, red_i[threadIdx.x] = xi;
    }
    __syncthreads();
  }
  __shared__ float sgn_sh;
  if (threadIdx.x == red_i[0]) sgn_sh = (vd < 0.f) ? -1.f : 1.f;
  __syncthreads();
  if (d < D) {
    const float scale = (nrm > 0.f) ? sgn_sh / nrm : sgn_sh;
    dirs[((int64_t)bh * max_slots + slot) * D + d] = vd * scale;
  }
}

// ---- one level: projection keys (16 lanes per position) ------------------------------------
template <int D>
__global__ __launch_bounds__(256) void reblock_key_kernel(const float* __restrict__ u, const int32_t* __restrict__ order,
                                                          const float* __restrict__ dirs, int N, int M, int level,
                                                          int max_slots, int64_t total, uint64_t* __restrict__ keys,
                                                          int32_t* __restrict__ vals) {
  constexpr int PER = D / 16;  // channels per lane
  const int64_t g = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  const int l16 = threadIdx.x % 16;
  if (g >= total) return;  // the 16 lanes of a position leave together
  const int bh = (int)(g / N), pos = (int)(g % N);
  int c;
  const int slot = slot_of(N, M, level, pos, &c);
  const int tok = order[g];
  uint32_t fk = 0u;
  if (c > 1) {
    const float* __restrict__ ur = u + ((int64_t)bh * N + tok) * D + l16 * PER;
    const float* __restrict__ vr = dirs + ((int64_t)bh * max_slots + slot) * D + l16 * PER;
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < PER; x += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(ur + x);
      const f32x4 b = *reinterpret_cast<const f32x4*>(vr + x);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(a[e], b[e], acc);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 16);
    fk = float_key(acc);
  }
  if (l16 == 0) {
    keys[g] = ((uint64_t)bh << 48) | ((uint64_t)slot << 32) | fk;
    vals[g] = tok;
  }
}

__global__ void iota_kernel(int32_t* __restrict__ order, int N, int64_t total) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g < total) order[g] = (int32_t)(g % N);
}

__global__ void reblock_tables_kernel(const int32_t* __restrict__ order, int N, int M, int J, int BH,
                                      int32_t* __restrict__ perm, int32_t* __restrict__ block_len) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)J * M;
  if (g >= per * BH) return;
  const int bh = (int)(g / per), p = (int)(g % per);
  perm[g] = (p < N) ? order[(int64_t)bh * N + p] : -1;
  if (bh == 0 && p % M == 0) block_len[p / M] = min(M, N - p);
}

// ---- host orchestration --------------------------------------------------------------------
static int sort_end_bit(int BH) {
  int bh_bits = 0;
  while ((1 << bh_bits) < BH) ++bh_bits;
  return 48 + bh_bits;
}

size_t reblock_sort_bytes(int64_t total, int BH) {
  size_t bytes = 0;
  hipcub::DeviceRadixSort::SortPairs(nullptr, bytes, (const uint64_t*)nullptr, (uint64_t*)nullptr,
                                     (const int32_t*)nullptr, (int32_t*)nullptr, (int)total, 0, sort_end_bit(BH));
  return bytes;
}

template <int D>
static hipError_t reblock_d(const ReblockParams& p, hipStream_t s) {
  const int BH = p.B * p.H, N = p.N, M = p.M;
  const int64_t total = (int64_t)BH * N;
  const int nc = (N + kMomentChunk - 1) / kMomentChunk;
  moment_partial_kernel<D><<<dim3((unsigned)nc, (unsigned)BH), 256, 0, s>>>(
      reinterpret_cast<const __bf16*>(p.q), p.sB, p.sN, p.sH, p.H, N, p.part);
  moment_factor_kernel<D><<<dim3((unsigned)BH), 1024, 0, s>>>(p.part, nc, N, p.ridge, p.moment, p.factor);
  key_feature_kernel<D><<<dim3((unsigned)((N + 63) / 64), (unsigned)BH), 256, 0, s>>>(
      reinterpret_cast<const __bf16*>(p.k), p.sB, p.sN, p.sH, p.H, N, p.factor, p.features);
  iota_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(p.order0, N, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.levels) {
    e = hipMemcpyAsync(p.levels, p.order0, total * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  int32_t* cur = p.order0;
  int32_t* nxt = p.order1;
  const int end_bit = sort_end_bit(BH);
  const int nlev = reblock_levels(N, M);
  const int max_slots = 1 << (nlev > 1 ? nlev - 2 : 0);
  for (int lev = 0; lev + 1 < nlev; ++lev) {
    const int nslots = 1 << lev;
    // directions of this level: the caller's per-level copy, else the workspace
    float* dirs = p.dirs_out ? p.dirs_out + (int64_t)lev * BH * max_slots * D : p.dirs;
    reblock_direction_kernel<D><<<dim3((unsigned)nslots, (unsigned)BH), 256, 0, s>>>(p.features, cur, N, M, lev,
                                                                                      max_slots, dirs);
    reblock_key_kernel<D><<<dim3((unsigned)((total + 15) / 16)), 256, 0, s>>>(p.features, cur, dirs, N, M, lev,
                                                                             max_slots, total, p.keys0, p.vals0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    size_t bytes = p.sort_bytes;
    e = hipcub::DeviceRadixSort::SortPairs(p.sort_tmp, bytes, p.keys0, p.keys1, p.vals0, nxt, (int)total, 0,
                                           end_bit, s);
    if (e != hipSuccess) return e;
    if (p.levels) {
      e = hipMemcpyAsync(p.levels + (int64_t)(lev + 1) * total, nxt, total * 4, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
    }
    int32_t* t = cur;
    cur = nxt;
    nxt = t;
  }
  const int J = (N + M - 1) / M;
  const int64_t nt = (int64_t)BH * J * M;
  reblock_tables_kernel<<<dim3((unsigned)((nt + 255) / 256)), 256, 0, s>>>(cur, N, M, J, BH, p.perm, p.block_len);
  return hipGetLastError();
}

hipError_t launch_reblock(const ReblockParams& p, hipStream_t s) {
  if (p.D == 128) return reblock_d<128>(p, s);
  return reblock_d<64>(p, s);
}

}  // namespace bsa
