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
// largest entry positive), one projection key per token, and a stable sort of
// every node's tokens by their keys -- the first child's tokens first, in
// place.  Sorts run on unique 64-bit composites (key << 32 | position in the
// node's current order), so any correct sort of them is the stable order:
// nodes of at most 8192 tokens are sorted in LDS by one workgroup (stable
// radix sort), larger ones in 8192-key chunks that merge-path rounds then
// merge.
//
// Design (MI355X): the moment is an fp32 outer-product accumulation over
// 2048-token chunks (each thread an 8 x 8 tile of the D x D matrix), reduced
// in a fixed order, ridged and factored by a one-workgroup Cholesky in LDS;
// the unit features u = z / |z|, z = k^T L, are formed with L resident in LDS.
// Decisions (projections, sort keys) are taken in fp32.

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

// ---- second moment ---------------------------------------------------------------------
// Partial Q^T Q over a 2048-token chunk on the matrix cores: bf16 products are
// exact in fp32, accumulation in fp32.  Tokens are staged row-major (coalesced
// 16-byte loads, 16-byte chunks XOR-swizzled per row, two buffers) and read
// with the transposing LDS read, which gives a lane 8 consecutive tokens of one
// channel: both the A fragment (rows d1) and, for C = Q^T Q, the B fragment
// (columns d2) of a 32 x 32 x 16 product.  The next step's loads are in flight
// during the products.

// Physical 16-byte chunk of logical chunk c in staged row r: the transposing
// read takes 4 consecutive rows x 32 bytes per 16-lane group, so rows r % 4 get
// disjoint chunk sets.
template <int CPR>
__device__ __forceinline__ int tr_swz(int r, int c) {
  if constexpr (CPR >= 16)
    return c ^ ((0xCA60 >> (4 * (r & 3))) & 15);  // XOR 0, 6, 10, 12 for r % 4 = 0..3
  else
    return c ^ (2 * (r & 3));
}

template <int D>
__global__ __launch_bounds__(256) void moment_partial_kernel(const __bf16* __restrict__ q, int64_t sB, int64_t sN,
                                                             int64_t sH, int H, int N, float* __restrict__ part) {
  constexpr int DT = D / 32;       // 32-channel tiles
  constexpr int CPR = D / 8;       // 16-byte chunks per token row
  constexpr int TOK = 64;          // tokens staged per step
  constexpr int LD = TOK * CPR / 256;  // 16-byte loads per thread per step
  constexpr int TILES = DT * DT;   // output tiles, spread over the 4 waves
  constexpr int TPWV = (TILES + 3) / 4;
  __shared__ __align__(16) __bf16 Qs[2][TOK * D];
  const int c = blockIdx.x, bh = blockIdx.y, BH = gridDim.y;
  const int b = bh / H, h = bh % H;
  const int t0 = c * kMomentChunk, t1 = min(N, t0 + kMomentChunk);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __bf16* __restrict__ src = q + b * sB + h * sH;
  f32x16 acc[TPWV];
#pragma unroll
  for (int x = 0; x < TPWV; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[x][r] = 0.f;
  bf16x8 v[LD];
  auto load = [&](int base) {
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int e = threadIdx.x + 256 * u, r = e / CPR, cc = e % CPR;
      v[u] = bf16x8{};
      if (base + r < t1)  // streaming load: every row is read once
        v[u] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(base + r) * sN + cc * 8)));
    }
  };
  // lane's share of the transposing reads: 16-lane group g16, lane jl in it
  const int g16 = lane >> 4, jl = lane & 15, h2 = lane >> 5;
  load(t0);
  int buf = 0;
  for (int base = t0; base < t1; base += TOK, buf ^= 1) {
    __bf16* Qb = Qs[buf];
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int e = threadIdx.x + 256 * u, r = e / CPR, cc = e % CPR;
      *reinterpret_cast<bf16x8*>(Qb + r * D + tr_swz<CPR>(r, cc) * 8) = v[u];
    }
    __syncthreads();  // this buffer was last read two steps ago, before the previous barrier
    if (base + TOK < t1) load(base + TOK);
#pragma unroll
    for (int ks = 0; ks < TOK / 16; ++ks) {
      // fragment of channel tile i over tokens 16ks .. 16ks+15 (runtime i: an
      // address, never an index into a register array)
      auto frag = [&](int i) {
        const int d = 32 * i + 16 * (g16 & 1) + 4 * (jl & 3);
        const int cc = d >> 3, off = d & 7;
        const int r0 = 16 * ks + 4 * h2 + (jl >> 2), r1 = r0 + 8;
        const bf16x4 lo = lds_read_tr16(Qb + r0 * D + tr_swz<CPR>(r0, cc) * 8 + off);
        const bf16x4 hi = lds_read_tr16(Qb + r1 * D + tr_swz<CPR>(r1, cc) * 8 + off);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      if constexpr (TPWV == DT) {  // wave w owns tiles (w, 0 .. DT-1)
        const bf16x8 fa = frag(w);
#pragma unroll
        for (int x = 0; x < DT; ++x) acc[x] = mfma32(fa, frag(x), acc[x]);
      } else {  // one tile per wave: (w / DT, w % DT)
        static_assert(TPWV == 1 && TILES == 4, "tile split");
        acc[0] = mfma32(frag(w / DT), frag(w % DT), acc[0]);
      }
    }
  }
  float* __restrict__ dst = part + ((int64_t)c * BH + bh) * D * D;
#pragma unroll
  for (int x = 0; x < TPWV; ++x) {
    const int tile = w * TPWV + x;
    if (tile >= TILES) continue;
    const int i = tile / DT, j = tile % DT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      dst[row * D + 32 * j + (lane & 31)] = acc[x][r];
    }
  }
}

// Sum of the partials in chunk order, divided by N (one thread per entry).
__global__ void moment_reduce_kernel(const float* __restrict__ part, int nc, int DD, int N, float* __restrict__ moment) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x, bh = blockIdx.y, BH = gridDim.y;
  if (e >= DD) return;
  float sum = 0.f;
  for (int c = 0; c < nc; ++c) sum += part[((int64_t)c * BH + bh) * DD + e];
  moment[(int64_t)bh * DD + e] = sum / (float)N;
}

// Ridge and Cholesky (right-looking, column by column, in LDS; two barriers per
// column, no index division).  A pivot that rounding drives below the ridge is
// clamped to it.
template <int D>
__global__ __launch_bounds__(1024) void moment_factor_kernel(const float* __restrict__ moment, float ridge,
                                                             float* __restrict__ factor) {
  __shared__ float A[D][D + 1];
  __shared__ float lam_sh;
  const int bh = blockIdx.x;
  for (int e = threadIdx.x; e < D * D; e += 1024) A[e / D][e % D] = moment[(int64_t)bh * D * D + e];
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
  // threads as 32 x 32 (row phase, column phase) over the trailing triangle
  const int ti = threadIdx.x >> 5, tk = threadIdx.x & 31;
  for (int j = 0; j < D; ++j) {
    if (threadIdx.x < 64) {  // wave 0: pivot, then the column below it
      const float djj = sqrtf(fmaxf(A[j][j], lam));
      for (int i = j + 1 + threadIdx.x; i < D; i += 64) A[i][j] /= djj;
      if (threadIdx.x == 0) A[j][j] = djj;
    }
    __syncthreads();
    for (int i = j + 1 + ti; i < D; i += 32) {
      const float aij = A[i][j];
      for (int k = j + 1 + tk; k <= i; k += 32) A[i][k] = fmaf(-aij, A[k][j], A[i][k]);
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < D * D; e += 1024) {
    const int i = e / D, k = e % D;
    factor[(int64_t)bh * D * D + e] = (k <= i) ? A[i][k] : 0.f;
  }
}

// ---- key features: u = z / |z|, z_d = sum_e k_e L[e][d] ----------------------------
// On the matrix cores as Z^T = L^T K^T: wave w owns the 32 channels
// 32w .. 32w+31 and keeps its L^T fragments in registers, with L split into
// bf16 hi + lo (two products; the dropped remainder is below 2^-17 of L); K is
// exact in bf16.  Tiles of 32 tokens are staged once per workgroup in LDS
// (coalesced 16-byte loads, 16-byte chunks XOR-swizzled per row, two buffers,
// three tiles' loads in flight in registers) and read as the B fragments.  In
// the output layout lane l holds token l%32, so a token's squared norm is a
// per-lane sum, one swap between the wave halves and one exchange of the
// waves' partials through LDS; the normalised tile goes back through LDS and
// out as whole rows (16-byte stores).  Stored in fp16 (unit vectors:
// |u_d| <= 1), which is what every later decision reads; `u32` (optional)
// receives the same values in fp32.
constexpr int kFeatTokens = 1024;  // tokens per workgroup

template <int D>
__global__ __launch_bounds__(256) void key_feature_kernel(const __bf16* __restrict__ k, int64_t sB, int64_t sN,
                                                          int64_t sH, int H, int N, const float* __restrict__ factor,
                                                          _Float16* __restrict__ u, float* __restrict__ u32) {
  constexpr int DT = D / 32, KS = D / 16, CPR = D / 8;
  constexpr int TT = 32;                // tokens per tile
  constexpr int LDT = TT * CPR / 256;   // 16-byte loads per thread per tile
  static_assert(LDT >= 1 && DT <= 4, "tile shape");
  __shared__ __align__(16) __bf16 Ks[2][TT * D];
  __shared__ __align__(16) _Float16 Os[TT * D];  // normalised tile, rows swizzled like Ks
  __shared__ float Nsq[2][4][TT];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, h2 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool active = w < DT;  // D = 64: waves 2 and 3 only stage
  const int tb = blockIdx.x * kFeatTokens, te = min(N, tb + kFeatTokens);
  // A fragments: lane l holds L[16ks + 8(l/32) + e][32w + l%32], e = 0..7
  bf16x8 lhi[KS], llo[KS];
  if (active) {
    const float* __restrict__ Lg = factor + (int64_t)bh * D * D + 32 * w + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = Lg[(16 * ks + 8 * h2 + e) * D];
        const __bf16 hi = (__bf16)x;
        lhi[ks][e] = hi;
        llo[ks][e] = (__bf16)(x - (float)hi);
      }
  }
  const __bf16* __restrict__ src = k + b * sB + h * sH;
  // three register sets: the loads of tile i + 3 are issued when tile i has
  // been written to LDS, so three tiles are in flight per workgroup
  bf16x8 v0[LDT], v1[LDT], v2[LDT];
  auto load = [&](bf16x8* v, int t0) {
    if (t0 >= te) return;
#pragma unroll
    for (int q = 0; q < LDT; ++q) {
      const int e = threadIdx.x + 256 * q, r = e / CPR, c = e % CPR;
      v[q] = bf16x8{};
      if (t0 + r < te)  // streaming load: every row is read once
        v[q] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(t0 + r) * sN + 8 * c)));
    }
  };
  auto swz = [](int r, int c) { return c ^ (r & (CPR - 1)); };
  // one tile: stage from v, refill v with tile t0 + 3 TT, products, norm, store
  auto tile = [&](bf16x8* v, int t0, int buf) {
    __bf16* Kb = Ks[buf];
#pragma unroll
    for (int q = 0; q < LDT; ++q) {
      const int e = threadIdx.x + 256 * q, r = e / CPR, c = e % CPR;
      *reinterpret_cast<bf16x8*>(Kb + r * D + swz(r, c) * 8) = v[q];
    }
    __syncthreads();  // tile visible; this buffer and Nsq[buf] were last read two tiles ago, Os one tile ago
    load(v, t0 + 3 * TT);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    if (active) {
      const int row = lane & 31;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Kb + row * D + swz(row, 2 * ks + h2) * 8);
        acc = mfma32(lhi[ks], kf, acc);
        acc = mfma32(llo[ks], kf, acc);
      }
      // register 4j + i holds channel 32w + 8j + 4(l/32) + i of token l%32
      float sq = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sq = fmaf(acc[r], acc[r], sq);
      sq += xor32(sq);
      if (h2 == 0) Nsq[buf][w][row] = sq;
    }
    __syncthreads();
    if (active) {
      const int row = lane & 31, tok = t0 + row;
      float tot = 0.f;
#pragma unroll
      for (int x = 0; x < DT; ++x) tot += Nsq[buf][x][row];
      const float inv = (tot > 0.f) ? 1.f / sqrtf(tot) : 0.f;
      typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(acc[4 * j + i] * inv);
        // channels 32w + 8j + 4h2 .. +3: half h2 of logical chunk 4w + j
        *reinterpret_cast<f16x4*>(Os + row * D + swz(row, 4 * w + j) * 8 + 4 * h2) = hv;
        if (u32 && tok < te) {
          const f32x4 fv = {(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
          *reinterpret_cast<f32x4*>(u32 + ((int64_t)bh * N + tok) * D + 32 * w + 8 * j + 4 * h2) = fv;
        }
      }
    }
    __syncthreads();
    // whole rows out: 16-byte stores, consecutive lanes on consecutive chunks
#pragma unroll
    for (int q = 0; q < LDT; ++q) {
      const int e = threadIdx.x + 256 * q, r = e / CPR, c = e % CPR;
      if (t0 + r < te)
        *reinterpret_cast<bf16x8*>(u + ((int64_t)bh * N + t0 + r) * D + 8 * c) =
            *reinterpret_cast<const bf16x8*>(Os + r * D + swz(r, c) * 8);
    }
  };
  load(v0, tb);
  load(v1, tb + TT);
  load(v2, tb + 2 * TT);
  // tile i uses LDS buffer i & 1 (every bound is uniform over the workgroup)
  for (int i = 0, t0 = tb; t0 < te; i += 3, t0 += 3 * TT) {
    tile(v0, t0, i & 1);
    if (t0 + TT >= te) break;
    tile(v1, t0 + TT, (i + 1) & 1);
    if (t0 + 2 * TT >= te) break;
    tile(v2, t0 + 2 * TT, i & 1);
  }
}

// ---- principal axis of the centred landmarks (one wave) ----------------------------------
// X: 32 centred landmark rows in LDS, row stride ldx floats.  The Gram matrix
// G = X X^T runs on the matrix cores (X split into bf16 hi + lo, three
// products, fp32-accurate): lane l holds row l%32, channels 16ks + 8(l/32) + 0..7,
// the A fragment of rows and the B fragment of columns alike.  G is symmetric,
// so the output layout gives lanes l and l+32 the two halves of row l%32; after
// one swap every lane holds its whole row in registers and each of the 16 power
// iterations from the ramp is 32 broadcast-FMAs and a 32-term broadcast sum.
// Returns a_s in lanes s and s + 32.
template <int D>
__device__ __forceinline__ float landmark_axis(const float* X, int ldx, int lane) {
  static_assert(kLandmarks == 32, "one 32 x 32 Gram tile");
  const int h2 = lane >> 5, s = lane & 31;
  f32x16 g;
#pragma unroll
  for (int r = 0; r < 16; ++r) g[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8 hi, lo;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const float xv = X[s * ldx + 16 * ks + 8 * h2 + x];
      hi[x] = (__bf16)xv;
      lo[x] = (__bf16)(xv - (float)hi[x]);
    }
    g = mfma32(lo, hi, g);
    g = mfma32(hi, lo, g);
    g = mfma32(hi, hi, g);
  }
  // g[4j + i] = G[8j + 4 h2 + i][s] = G[s][8j + 4 h2 + i]
  float row[kLandmarks];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float other = xor32(g[r]);
    const int j = r >> 2, i = r & 3;
    row[8 * j + i] = h2 ? other : g[r];
    row[8 * j + 4 + i] = h2 ? g[r] : other;
  }
  auto bcast = [](float x, int t) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), t));
  };
  // ramp start s - 15.5, normalised: |ramp|^2 = sum (s - 15.5)^2 = 2728 for 32 landmarks
  float a = ((float)s - 0.5f * (kLandmarks - 1)) * rsqrtf(2728.f);
  for (int it = 0; it < kPowerIters; ++it) {
    float wv = 0.f;
#pragma unroll
    for (int t = 0; t < kLandmarks; ++t) wv = fmaf(row[t], bcast(a, t), wv);
    const float sq = wv * wv;
    float n2 = 0.f;
#pragma unroll
    for (int t = 0; t < kLandmarks; ++t) n2 += bcast(sq, t);
    if (n2 == 0.f) {  // uniform: the landmarks coincide
      a = wv;
      break;
    }
    a = wv / sqrtf(n2);
  }
  return a;
}

// One wave: centre the 32 landmark rows of X (LDS, row stride ldx), find their
// principal axis a (landmark_axis; a_sh receives it), form v = X^T a, normalise
// it and give its largest-magnitude entry (lowest index on ties) a positive
// sign.  v (LDS, D floats) receives the unit direction.
template <int D>
__device__ __forceinline__ void wave_direction(float* X, int ldx, float* a_sh, float* v, int lane) {
  constexpr int PL = D / 64;  // channels per lane
#pragma unroll
  for (int x = 0; x < PL; ++x) {
    const int d = lane + 64 * x;
    float col[kLandmarks];
    float m = 0.f;
#pragma unroll
    for (int s = 0; s < kLandmarks; ++s) col[s] = X[s * ldx + d], m += col[s];
    m /= (float)kLandmarks;
#pragma unroll
    for (int s = 0; s < kLandmarks; ++s) X[s * ldx + d] = col[s] - m;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const float a = landmark_axis<D>(X, ldx, lane);
  if (lane < kLandmarks) a_sh[lane] = a;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  float vd[PL];
  float n2 = 0.f, best = -1.f;
  int bi = 0;
#pragma unroll
  for (int x = 0; x < PL; ++x) {
    const int d = lane + 64 * x;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < kLandmarks; ++s) acc = fmaf(X[s * ldx + d], a_sh[s], acc);
    vd[x] = acc;
    n2 = fmaf(acc, acc, n2);
    if (fabsf(acc) > best) best = fabsf(acc), bi = d;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n2 += __shfl_xor(n2, o, 64);
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) best = ob, bi = oi;
  }
  float sgn = 1.f;
#pragma unroll
  for (int x = 0; x < PL; ++x)
    if (lane + 64 * x == bi) sgn = (vd[x] < 0.f) ? -1.f : 1.f;
  sgn = __shfl(sgn, bi % 64, 64);
  const float scale = (n2 > 0.f) ? sgn / sqrtf(n2) : sgn;
#pragma unroll
  for (int x = 0; x < PL; ++x) v[lane + 64 * x] = vd[x] * scale;
}

// ---- split direction of one node (all 256 threads of the workgroup) -----------------------
template <int D>
struct DirScratch {
  float X[kLandmarks][D + 1];
  float a[kLandmarks];
};

// ord: the node's tokens in their current order (global or LDS); ub: the
// head's features.  Leaves the unit direction in v (LDS, D floats).  The
// landmark rows are gathered by the whole workgroup (16-byte loads), the rest
// runs in wave 0.
template <int D>
__device__ void node_direction(const _Float16* __restrict__ ub, const int32_t* ord, int n, DirScratch<D>& sh,
                               float* v) {
  for (int e = threadIdx.x; e < kLandmarks * (D / 8); e += blockDim.x) {
    const int s = e / (D / 8), cc = e % (D / 8);
    const int tok = ord[(int)(((int64_t)(2 * s + 1) * n) / (2 * kLandmarks))];
    const half8 h = *reinterpret_cast<const half8*>(ub + (int64_t)tok * D + 8 * cc);
#pragma unroll
    for (int x = 0; x < 8; ++x) sh.X[s][8 * cc + x] = (float)h[x];
  }
  __syncthreads();
  if (threadIdx.x < 64) wave_direction<D>(&sh.X[0][0], D + 1, sh.a, v, threadIdx.x);
  __syncthreads();
}

// Projection u . v of one member by one lane (the whole fp16 row; v in LDS):
// within one wave every lane's row loads are in flight together.
template <int D>
__device__ __forceinline__ float project_row(const _Float16* __restrict__ ur, const float* v) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const half8 h = *reinterpret_cast<const half8*>(ur + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)h[e], v[8 * c + e], acc);
  }
  return acc;
}

// Projections u . v of 16·NB members by one 16-lane group: lane j reads 16
// bytes of every member row (whole rows per group, coalesced; all NB·16 row
// loads in flight together) and keeps one partial sum per member; per batch
// of 16 a butterfly reduce-scatter (8 + 4 + 2 + 1 independent exchanges)
// leaves member `base + 16b + j`'s projection in lane j of out[b].  ord: the
// node's tokens; members at or beyond n read member 0's row (results unused).
template <int D, int NB>
__device__ __forceinline__ void project_batches(const _Float16* __restrict__ ub, const int32_t* ord, int base, int n,
                                                const float* v, int l16, float* out) {
  constexpr int PER = D / 16;  // channels per lane
  using HV = typename std::conditional<PER == 8, half8, half4>::type;
  HV h[NB * 16];
#pragma unroll
  for (int m = 0; m < NB * 16; ++m) {
    const int i = base + m;
    h[m] = *reinterpret_cast<const HV*>(ub + (int64_t)ord[(i < n) ? i : 0] * D + l16 * PER);
  }
  float vr[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) vr[e] = v[l16 * PER + e];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float part[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc = fmaf((float)h[16 * b + m][e], vr[e], acc);
      part[m] = acc;
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      // lanes with bit o clear keep values [0, o), the others [o, 2o)
      const bool hi = (l16 & o) != 0;
#pragma unroll
      for (int m = 0; m < o; ++m) {
        const float send = hi ? part[m] : part[m + o];
        const float keep = hi ? part[m + o] : part[m];
        part[m] = keep + __shfl_xor(send, o, 16);
      }
    }
    out[b] = part[0];
  }
}

template <int D>
__device__ __forceinline__ float project_batch16(const _Float16* __restrict__ ub, const int32_t* ord, int base, int n,
                                                 const float* v, int l16) {
  float r;
  project_batches<D, 1>(ub, ord, base, n, v, l16, &r);
  return r;
}

// ---- one level, large nodes: split directions ----------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void reblock_direction_kernel(const _Float16* __restrict__ u,
                                                                const int32_t* __restrict__ order, int N, int M,
                                                                int level, int max_slots, float* __restrict__ dirs) {
  const int slot = blockIdx.x, bh = blockIdx.y;
  int start, n, c;
  slot_range(N, M, level, slot, &start, &n, &c);
  if (c <= 1) return;  // whole workgroup
  __shared__ DirScratch<D> sh;
  __shared__ float v[D];
  node_direction<D>(u + (int64_t)bh * N * D, order + (int64_t)bh * N + start, n, sh, v);
  for (int d = threadIdx.x; d < D; d += 256) dirs[((int64_t)bh * max_slots + slot) * D + d] = v[d];
}

// ---- one level, large nodes: projection keys (16 positions per 16-lane group) --------------
// Node ranges start at multiples of M (16, 32 or 64), so the 16 aligned
// positions of a batch belong to one node and share its direction.
template <int D>
__global__ __launch_bounds__(256) void reblock_key_kernel(const _Float16* __restrict__ u,
                                                          const int32_t* __restrict__ order,
                                                          const float* __restrict__ dirs, int N, int M, int level,
                                                          int max_slots, uint64_t* __restrict__ keys) {
  const int bh = blockIdx.y;
  const int pos0 = (blockIdx.x * 16 + (int)threadIdx.x / 16) * 16;
  const int l16 = threadIdx.x % 16;
  if (pos0 >= N) return;  // the 16 lanes of a batch leave together
  const int cnt = min(16, N - pos0);
  int c;
  const int slot = slot_of(N, M, level, pos0, &c);
  const int32_t* __restrict__ ord = order + (int64_t)bh * N + pos0;
  uint32_t fk = 0u;
  if (c > 1)
    fk = float_key(project_batch16<D>(u + (int64_t)bh * N * D, ord, 0, cnt,
                                      dirs + ((int64_t)bh * max_slots + slot) * D, l16));
  if (l16 < cnt) {
    int start, n, cc;
    slot_range(N, M, level, slot, &start, &n, &cc);
    keys[(int64_t)bh * N + pos0 + l16] = ((uint64_t)fk << 32) | (uint32_t)(pos0 + l16 - start);
  }
}

// ---- sorts -----------------------------------------------------------------------------
// Stable LSD radix sort of 256 * IPT (key, value) pairs in LDS by 256 threads:
// four passes of 8-bit digits.  Wave w owns the contiguous range
// [w * 64 * IPT, (w + 1) * 64 * IPT) of the current order and takes it in
// rounds of 64 consecutive items, so its lanes meet the items in order.  In a
// round the lanes holding the same digit find each other with 8 ballots; an
// item's rank among the wave's items of its digit is the wave's running count
// of that digit (read before the round's leader adds the round's count) plus
// the number of its peers in lower lanes.  A scan over (digit, wave) then
// gives every (wave, digit) its output offset, and the items are scattered.
// Equal keys keep their order, so sorting (projection key, position) this way
// gives the same order as sorting the unique 64-bit composites.
template <int IPT>
__device__ __forceinline__ void block_radix_sort(uint32_t* keys, uint32_t* vals, uint32_t* hist /* [4 * 256] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int base = w * 64 * IPT;
  for (int shift = 0; shift < 32; shift += 8) {
    for (int x = threadIdx.x; x < 4 * 256; x += 256) hist[x] = 0u;
    __syncthreads();
    uint32_t k[IPT], v[IPT], pre[IPT];
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      k[r] = keys[base + 64 * r + lane];
      v[r] = vals[base + 64 * r + lane];
    }
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      const uint32_t d = (k[r] >> shift) & 255u;
      uint64_t peers = ~0ull;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t bal = __builtin_amdgcn_ballot_w64(((d >> b) & 1u) != 0u);
        peers &= ((d >> b) & 1u) ? bal : ~bal;
      }
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
      uint32_t* h = hist + w * 256 + d;
      pre[r] = *h + below;  // this wave's LDS operations complete in order
      if (below == 0u) *h += (uint32_t)__builtin_popcountll(peers);
    }
    __syncthreads();
    {  // offsets: digit-major, then wave
      const int d = threadIdx.x;
      const uint32_t c0 = hist[d], c1 = hist[256 + d], c2 = hist[512 + d], c3 = hist[768 + d];
      const uint32_t tot = c0 + c1 + c2 + c3;
      // exclusive scan of tot over the 256 digits: within the wave, then across waves
      uint32_t incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      __shared__ uint32_t wsum[4];
      if (lane == 63) wsum[w] = incl;
      __syncthreads();
      uint32_t off = incl - tot;
      for (int ww = 0; ww < w; ++ww) off += wsum[ww];
      hist[d] = off;
      hist[256 + d] = off + c0;
      hist[512 + d] = off + c0 + c1;
      hist[768 + d] = off + c0 + c1 + c2;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      const uint32_t d = (k[r] >> shift) & 255u;
      const uint32_t at = hist[w * 256 + d] + pre[r];
      keys[at] = k[r];
      vals[at] = v[r];
    }
    __syncthreads();
  }
}

// Number of A elements among the first d outputs of merging sorted A (la)
// and B (lb) -- keys are unique.
__device__ __forceinline__ int merge_path(const uint64_t* a, int la, const uint64_t* b, int lb, int d) {
  int lo = max(0, d - lb), hi = min(d, la);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < b[d - 1 - mid])
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// ---- one level, nodes of at most kLocalCap tokens: direction, projections (16
// members per 16-lane group at a time) and a stable radix sort of the
// projection keys with the positions as values, one workgroup per node.
constexpr int kLocalCap = 8192;  // capacities 1024, 4096, 8192 (the largest: one workgroup per CU)

template <int D, int CAP>
__global__ __launch_bounds__(256) void reblock_local_level_kernel(const _Float16* __restrict__ u,
                                                                  const int32_t* __restrict__ cur,
                                                                  int32_t* __restrict__ nxt, int N, int M, int level,
                                                                  int max_slots, float* __restrict__ dirs_out) {
  const int slot = blockIdx.x, bh = blockIdx.y;
  int start, n, c;
  slot_range(N, M, level, slot, &start, &n, &c);
  if (n == 0) return;  // empty slot (whole workgroup)
  const int32_t* __restrict__ src = cur + (int64_t)bh * N + start;
  int32_t* __restrict__ dst = nxt + (int64_t)bh * N + start;
  if (c <= 1) {  // a leaf keeps its order
    for (int i = threadIdx.x; i < n; i += 256) dst[i] = src[i];
    return;
  }
  __shared__ int32_t ord[CAP];
  __shared__ uint32_t keys[CAP];
  __shared__ uint32_t vals[CAP];
  __shared__ uint32_t hist[4 * 256];
  __shared__ DirScratch<D> dsh;
  __shared__ float v[D];
  for (int i = threadIdx.x; i < n; i += 256) ord[i] = src[i];
  __syncthreads();
  const _Float16* __restrict__ ub = u + (int64_t)bh * N * D;
  node_direction<D>(ub, ord, n, dsh, v);
  if (dirs_out)
    for (int d = threadIdx.x; d < D; d += 256) dirs_out[((int64_t)bh * max_slots + slot) * D + d] = v[d];
  const int l16 = threadIdx.x & 15;
  for (int base = 16 * (threadIdx.x >> 4); base < n; base += 256) {  // uniform within each 16-lane group
    const float pr = project_batch16<D>(ub, ord, base, n, v, l16);
    if (base + l16 < n) {
      keys[base + l16] = float_key(pr);
      vals[base + l16] = (uint32_t)(base + l16);
    }
  }
  for (int i = n + (int)threadIdx.x; i < CAP; i += 256) {  // padding sorts last (after every member)
    keys[i] = ~0u;
    vals[i] = (uint32_t)i;
  }
  __syncthreads();
  block_radix_sort<CAP / 256>(keys, vals, hist);
  for (int i = threadIdx.x; i < n; i += 256) dst[i] = ord[vals[i]];
}

// ---- one level, large nodes: sort every 8192-key chunk of every node in LDS ----------------
// (radix sort of the high halves with the low halves -- the positions, unique
// inside a node -- as values; equal keys keep their position order)
constexpr int kChunkKeys = 8192;

__global__ __launch_bounds__(256) void reblock_chunk_sort_kernel(uint64_t* __restrict__ keys, int N, int M,
                                                                 int level) {
  const int slot = blockIdx.y, bh = blockIdx.z;
  int start, n, c;
  slot_range(N, M, level, slot, &start, &n, &c);
  const int c0 = blockIdx.x * kChunkKeys;
  if (c0 >= n) return;  // whole workgroup
  const int m = min(kChunkKeys, n - c0);
  uint64_t* __restrict__ g = keys + (int64_t)bh * N + start + c0;
  __shared__ uint32_t skey[kChunkKeys];
  __shared__ uint32_t sval[kChunkKeys];
  __shared__ uint32_t hist[4 * 256];
  for (int i = threadIdx.x; i < kChunkKeys; i += 256) {  // composites: key << 32 | position
    const uint64_t kv = (i < m) ? g[i] : ~0ull;  // padding sorts last
    skey[i] = (uint32_t)(kv >> 32);
    sval[i] = (uint32_t)kv;
  }
  __syncthreads();
  block_radix_sort<kChunkKeys / 256>(skey, sval, hist);
  for (int i = threadIdx.x; i < m; i += 256) g[i] = ((uint64_t)skey[i] << 32) | sval[i];
}

// ---- one level, large nodes: one merge-path round ------------------------------------------
// Runs of L sorted keys (the last one of a node may be short) are merged in
// pairs into runs of 2L.  Each workgroup writes kMergeTile consecutive outputs
// of one merged pair: it finds where that output range starts and ends in the
// two runs (merge path), stages both pieces in LDS and each thread merges 8
// outputs after its own merge-path search.  The last round (`cur` given)
// writes the tokens themselves: the low half of a composite is the token's
// position in the node's current order.
constexpr int kMergeTile = 2048;

__global__ __launch_bounds__(256) void reblock_merge_kernel(const uint64_t* __restrict__ src,
                                                            uint64_t* __restrict__ dst, int N, int M, int level,
                                                            int L, const int32_t* __restrict__ cur,
                                                            int32_t* __restrict__ nxt) {
  const int slot = blockIdx.y, bh = blockIdx.z;
  int start, n, c;
  slot_range(N, M, level, slot, &start, &n, &c);
  const int t0 = blockIdx.x * kMergeTile;
  if (t0 >= n) return;  // whole workgroup
  const int base = t0 / (2 * L) * (2 * L);  // the merged pair's first output (kMergeTile divides 2L)
  const int la = min(L, n - base), lb = max(0, min(L, n - base - L));
  const int64_t node = (int64_t)bh * N + start;
  const uint64_t* __restrict__ A = src + node + base;
  const uint64_t* __restrict__ B = A + la;
  const int d0 = t0 - base, d1 = min(d0 + kMergeTile, la + lb);
  __shared__ int ends[2];
  __shared__ uint64_t sh[kMergeTile];
  if (threadIdx.x < 64) {  // wave 0: both ends by a 64-way search (3 rounds of loads for 2^16 keys)
    const int lane = threadIdx.x;
    for (int e = 0; e < 2; ++e) {
      const int d = e ? d1 : d0;
      int lo = max(0, d - lb), hi = min(d, la);  // the answer lies in [lo, hi]
      while (lo < hi) {
        // A[i] < B[d - 1 - i] holds exactly for i below the answer; probe 64 points of [lo, hi)
        const int span = hi - lo;
        const int i = lo + (int)(((int64_t)span * lane) >> 6);
        const uint64_t bal = __builtin_amdgcn_ballot_w64(A[i] < B[d - 1 - i]);
        const int t = __builtin_popcountll(bal);  // the true probes are the lowest t lanes
        const int nlo = t > 0 ? lo + (int)(((int64_t)span * (t - 1)) >> 6) + 1 : lo;
        const int nhi = t < 64 ? lo + (int)(((int64_t)span * t) >> 6) : hi;
        lo = nlo;
        hi = nhi;
      }
      if (lane == 0) ends[e] = lo;
    }
  }
  __syncthreads();
  const int i0 = ends[0], i1 = ends[1], j0 = d0 - i0, j1 = d1 - i1;
  const int na = i1 - i0, nb = j1 - j0;
  for (int x = threadIdx.x; x < na + nb; x += 256) sh[x] = (x < na) ? A[i0 + x] : B[j0 + x - na];
  __syncthreads();
  __shared__ uint64_t ob[kMergeTile];  // the merged tile, stored coalesced below
  const int dl = 8 * (int)threadIdx.x;
  if (dl < na + nb) {
    int ia = merge_path(sh, na, sh + na, nb, dl), ib = dl - ia;
    const int cnt = min(8, na + nb - dl);
    for (int q = 0; q < cnt; ++q) {
      const bool take_a = ib >= nb || (ia < na && sh[ia] < sh[na + ib]);
      ob[dl + q] = take_a ? sh[ia++] : sh[na + ib++];
    }
  }
  __syncthreads();
  const int64_t o0 = node + base + d0;
  for (int x = threadIdx.x; x < na + nb; x += 256) {
    if (cur)
      nxt[o0 + x] = cur[node + (int)(uint32_t)ob[x]];
    else
      dst[o0 + x] = ob[x];
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

// ---- one level, nodes of at most 256 tokens: one wave per node, two nodes per workgroup -----
// The same steps as the block-level kernel with wave-level synchronisation; the
// landmark Gram matrix runs on the matrix cores (centred landmarks split into
// bf16 hi + lo, three products, fp32-accurate).
constexpr int kWaveCap = 256;
constexpr int kWaveNodes = 2;  // nodes (waves) per workgroup

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D>
struct WaveNode {
  float X[kLandmarks][D + 4];
  float v[D];
  float a[kLandmarks];
  int32_t ord[kWaveCap];
  uint64_t keys[kWaveCap];
};

template <int D>
__global__ __launch_bounds__(128) void reblock_wave_level_kernel(const _Float16* __restrict__ u,
                                                                 const int32_t* __restrict__ cur,
                                                                 int32_t* __restrict__ nxt, int N, int M, int level,
                                                                 int nslots, int max_slots, float* __restrict__ dirs_out) {
  __shared__ WaveNode<D> wn[kWaveNodes];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int slot = blockIdx.x * kWaveNodes + w, bh = blockIdx.y;
  if (slot >= nslots) return;  // whole wave
  int start, n, c;
  slot_range(N, M, level, slot, &start, &n, &c);
  if (n == 0) return;
  const int32_t* __restrict__ src = cur + (int64_t)bh * N + start;
  int32_t* __restrict__ dst = nxt + (int64_t)bh * N + start;
  if (c <= 1) {
    for (int i = lane; i < n; i += 64) dst[i] = src[i];
    return;
  }
  WaveNode<D>& sh = wn[w];
  const _Float16* __restrict__ ub = u + (int64_t)bh * N * D;
  for (int i = lane; i < n; i += 64) sh.ord[i] = src[i];
  wave_sync();
  // landmarks
  for (int e = lane; e < kLandmarks * (D / 8); e += 64) {
    const int s = e / (D / 8), cc = e % (D / 8);
    const int tok = sh.ord[(int)(((int64_t)(2 * s + 1) * n) / (2 * kLandmarks))];
    const half8 h = *reinterpret_cast<const half8*>(ub + (int64_t)tok * D + 8 * cc);
#pragma unroll
    for (int x = 0; x < 8; ++x) sh.X[s][8 * cc + x] = (float)h[x];
  }
  wave_sync();
  wave_direction<D>(&sh.X[0][0], D + 4, sh.a, sh.v, lane);
  if (dirs_out)
    for (int d = lane; d < D; d += 64) dirs_out[((int64_t)bh * max_slots + slot) * D + d] = sh.v[d];
  wave_sync();
  // projections (one member per lane), then a stable bitonic sort of (key, position)
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = lane; i < P; i += 64) {
    uint64_t key = ~0ull;
    if (i < n) key = ((uint64_t)float_key(project_row<D>(ub + (int64_t)sh.ord[i] * D, sh.v)) << 32) | (uint32_t)i;
    sh.keys[i] = key;
  }
  wave_sync();
  for (int kk = 2; kk <= P; kk <<= 1)
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = lane; i < P; i += 64) {
        const int ij = i ^ j;
        if (ij > i) {
          const uint64_t x = sh.keys[i], y = sh.keys[ij];
          if ((x > y) == ((i & kk) == 0)) sh.keys[i] = y, sh.keys[ij] = x;
        }
      }
      wave_sync();
    }
  for (int i = lane; i < n; i += 64) dst[i] = sh.ord[(int)(sh.keys[i] & 0xffffffffu)];
}

// ---- host orchestration --------------------------------------------------------------------
template <int D>
static hipError_t reblock_d(const ReblockParams& p, hipStream_t s) {
  const int BH = p.B * p.H, N = p.N, M = p.M;
  const int64_t total = (int64_t)BH * N;
  static_assert((2 * kChunkKeys) % kMergeTile == 0, "a merge tile never straddles two merged pairs");
  const int nc = (N + kMomentChunk - 1) / kMomentChunk;
  moment_partial_kernel<D><<<dim3((unsigned)nc, (unsigned)BH), 256, 0, s>>>(
      reinterpret_cast<const __bf16*>(p.q), p.sB, p.sN, p.sH, p.H, N, p.part);
  moment_reduce_kernel<<<dim3((unsigned)((D * D + 255) / 256), (unsigned)BH), 256, 0, s>>>(p.part, nc, D * D, N,
                                                                                         p.moment);
  moment_factor_kernel<D><<<dim3((unsigned)BH), 1024, 0, s>>>(p.moment, p.ridge, p.factor);
  key_feature_kernel<D><<<dim3((unsigned)((N + kFeatTokens - 1) / kFeatTokens), (unsigned)BH), 256, 0, s>>>(
      reinterpret_cast<const __bf16*>(p.k), p.sB, p.sN, p.sH, p.H, N, p.factor, p.features, p.features32);
  iota_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(p.order0, N, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.levels) {
    e = hipMemcpyAsync(p.levels, p.order0, total * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  int32_t* cur = p.order0;
  int32_t* nxt = p.order1;
  const int nlev = reblock_levels(N, M);
  const int max_slots = 1 << (nlev > 1 ? nlev - 2 : 0);
  int cmax = (N + M - 1) / M;  // most leaves of a node at the current level
  for (int lev = 0; lev + 1 < nlev; ++lev, cmax = (cmax + 1) / 2) {
    const int nslots = 1 << lev;
    float* dirs_dbg = p.dirs_out ? p.dirs_out + (int64_t)lev * BH * max_slots * D : nullptr;
    const int64_t nmax = (int64_t)cmax * M;
    if (nmax <= kLocalCap) {
      const dim3 grid((unsigned)nslots, (unsigned)BH);
      if (nmax <= kWaveCap)
        reblock_wave_level_kernel<D><<<dim3((unsigned)((nslots + kWaveNodes - 1) / kWaveNodes), (unsigned)BH),
                                       64 * kWaveNodes, 0, s>>>(
            p.features, cur, nxt, N, M, lev, nslots, max_slots, dirs_dbg);
      else if (nmax <= 1024)
        reblock_local_level_kernel<D, 1024><<<grid, 256, 0, s>>>(p.features, cur, nxt, N, M, lev, max_slots, dirs_dbg);
      else if (nmax <= 4096)
        reblock_local_level_kernel<D, 4096><<<grid, 256, 0, s>>>(p.features, cur, nxt, N, M, lev, max_slots, dirs_dbg);
      else
        reblock_local_level_kernel<D, kLocalCap><<<grid, 256, 0, s>>>(p.features, cur, nxt, N, M, lev, max_slots,
                                                                      dirs_dbg);
      e = hipGetLastError();
    } else {
      // directions of this level: the caller's per-level copy, else the workspace
      float* dirs = dirs_dbg ? dirs_dbg : p.dirs;
      reblock_direction_kernel<D><<<dim3((unsigned)nslots, (unsigned)BH), 256, 0, s>>>(p.features, cur, N, M, lev,
                                                                                        max_slots, dirs);
      const int nbatch = (N + 15) / 16;  // 16 positions per 16-lane group, 16 groups per workgroup
      reblock_key_kernel<D><<<dim3((unsigned)((nbatch + 15) / 16), (unsigned)BH), 256, 0, s>>>(
          p.features, cur, dirs, N, M, lev, max_slots, p.keys0);
      reblock_chunk_sort_kernel<<<dim3((unsigned)((nmax + kChunkKeys - 1) / kChunkKeys), (unsigned)nslots,
                                       (unsigned)BH), 256, 0, s>>>(p.keys0, N, M, lev);
      // merge rounds: runs of 8192, 16384, ... keys until one run holds the
      // largest node; the last round writes the next order itself
      uint64_t* ka = p.keys0;
      uint64_t* kb = p.keys1;
      const dim3 mgrid((unsigned)((nmax + kMergeTile - 1) / kMergeTile), (unsigned)nslots, (unsigned)BH);
      for (int64_t L = kChunkKeys; L < nmax; L *= 2) {
        const bool last = 2 * L >= nmax;
        reblock_merge_kernel<<<mgrid, 256, 0, s>>>(ka, kb, N, M, lev, (int)L, last ? cur : nullptr,
                                                   last ? nxt : nullptr);
        uint64_t* t = ka;
        ka = kb;
        kb = t;
      }
      e = hipGetLastError();
    }
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
