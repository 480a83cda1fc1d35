// Coarse pooled-V branch for gfx950.
//
// Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" -- section 6.7 (coarse
// attention over all logical blocks: C = softmax(E) V_bar, with E the routing
// matrix of section 2.2 and V_bar the per-block means of V; each query block's
// row of C is added to its tokens under a gate, outside the main kernel).
//
// Design (MI355X): one 256-thread workgroup per (batch*head, ROWS query
// blocks), ROWS = 4096 / D, so the C tile is ROWS x D = 4096 values and each
// thread owns a 4 x 4 register tile (4 query blocks x 4 channels).
//   pass 1: each wave reduces ROWS/4 rows of E to max and 1 / sum of exp
//           (wave shuffles), kept in LDS;
//   pass 2: per chunk of KC = 32 columns, the normalised weights (ROWS x KC)
//           and the V_bar rows (KC x D) are staged in LDS, then every thread
//           runs KC steps of one 16-byte weight read (4 rows, a broadcast
//           within the wave), one 16-byte V_bar read (4 channels) and 16 FMAs.
// Weight rows are XOR-swizzled by column so that the 16-byte staging writes of
// 8 consecutive columns cover all banks.  All arithmetic is fp32; E is read
// twice (max/sum, then weights), V_bar once per workgroup from L2.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kCoarseCols = 32;  // columns of E per staged chunk

template <int D>
__global__ __launch_bounds__(256) void coarse_kernel(CoarseParams p) {
  constexpr int ROWS = 4096 / D;  // query blocks per workgroup (32 or 64)
  constexpr int CG = D / 4;       // 4-channel groups
  constexpr int RG = ROWS / 4;    // 4-row groups
  static_assert(CG * RG == 256, "one 4x4 tile per thread");
  constexpr int KC = kCoarseCols;
  __shared__ float mrow[ROWS], zinv[ROWS];
  __shared__ __align__(16) float Wt[KC * ROWS];  // [column][row group ^ (column & 7)][4]
  __shared__ __align__(16) float Vs[KC * D];     // [column][channel]
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * ROWS;
  const int J = p.J;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* __restrict__ Eb = p.E + (int64_t)bh * J * J;
  const float* __restrict__ vb = p.vbar + (int64_t)bh * J * D;

  // ---- pass 1: row maximum and 1 / sum of exp ----
  for (int r = w; r < ROWS; r += 4) {
    const int i = i0 + r;
    float m = -INFINITY, z = 0.f;
    if (i < J) {
      const float* row = Eb + (int64_t)i * J;
      for (int j = lane; j < J; j += 64) m = fmaxf(m, row[j]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      for (int j = lane; j < J; j += 64) z += __expf(row[j] - m);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
    }
    if (lane == 0) {
      mrow[r] = m;
      zinv[r] = (z > 0.f) ? 1.f / z : 0.f;
    }
  }
  __syncthreads();

  // ---- pass 2: C tile = W V_bar ----
  const int cg = tid % CG, rg = tid / CG;
  // staging roles: weights -- column sc, row group sr (4 rows, one 16-byte
  // write); V_bar -- 16-byte chunks e = tid + 256k of the KC x D chunk
  const int sc = tid % KC, sr0 = tid / KC;  // sr = sr0 + (256/KC) * k
  f32x4 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < J; j0 += KC) {
    const int j = j0 + sc;
#pragma unroll
    for (int k = 0; k < RG / (256 / KC); ++k) {
      const int sr = sr0 + (256 / KC) * k;
      f32x4 wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * sr + e, i = i0 + r;
        wv[e] = (i < J && j < J) ? __expf(Eb[(int64_t)i * J + j] - mrow[r]) * zinv[r] : 0.f;
      }
      *reinterpret_cast<f32x4*>(&Wt[sc * ROWS + 4 * (sr ^ (sc & 7))]) = wv;
    }
#pragma unroll
    for (int k = 0; k < KC * D / 4 / 256; ++k) {
      const int e = tid + 256 * k, c = e / CG, dq = e % CG;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j0 + c < J) v = *reinterpret_cast<const f32x4*>(vb + (int64_t)(j0 + c) * D + 4 * dq);
      *reinterpret_cast<f32x4*>(&Vs[c * D + 4 * dq]) = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < KC; ++c) {
      const f32x4 wv = *reinterpret_cast<const f32x4*>(&Wt[c * ROWS + 4 * (rg ^ (c & 7))]);
      const f32x4 v = *reinterpret_cast<const f32x4*>(&Vs[c * D + 4 * cg]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(wv[r], v[e], acc[r][e]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * rg + r;
    if (i < J) *reinterpret_cast<f32x4*>(p.C + ((int64_t)bh * J + i) * D + 4 * cg) = acc[r];
  }
}

hipError_t launch_coarse(const CoarseParams& p, hipStream_t s) {
  const int rows = 4096 / p.D;
  const dim3 grid((unsigned)((p.J + rows - 1) / rows), (unsigned)p.BH);
  if (p.D == 128)
    coarse_kernel<128><<<grid, dim3(256), 0, s>>>(p);
  else
    coarse_kernel<64><<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsa
