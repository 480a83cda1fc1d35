// Coarse pooled-V branch for gfx950.
//
// Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" -- section 6.7 (coarse
// attention over all logical blocks: C = softmax(E) V_bar, with E the routing
// matrix of section 2.2 and V_bar the per-block means of V; each query block's
// row of C is added to its tokens under a gate, outside the main kernel).
//
// Design (MI355X): one 256-thread workgroup per (batch*head, 32 query blocks).
// Pass 1: each wave takes 4 rows of E and reduces max and sum of exp with
// wave shuffles.  Pass 2: the normalised weights of 64 columns at a time are
// staged in LDS ([column][row], so one 16-byte read gives four rows); thread t
// owns channel t % D of rows (t / D) * R0 .. +R0 and accumulates in fp32 while
// V_bar rows stream from L2 (a head's V_bar is J*D*4 bytes).  E is read twice,
// V_bar once per workgroup.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kCoarseRows = 32;  // query blocks per workgroup
constexpr int kCoarseCols = 64;  // columns of E staged per step

template <int D>
__global__ __launch_bounds__(256) void coarse_kernel(CoarseParams p) {
  constexpr int RG = 256 / D;              // row groups
  constexpr int R0 = kCoarseRows / RG;     // rows per thread
  __shared__ float mrow[kCoarseRows], zinv[kCoarseRows];
  __shared__ __align__(16) float wgt[kCoarseCols][kCoarseRows];
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * kCoarseRows;
  const int J = p.J;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* __restrict__ Eb = p.E + (int64_t)bh * J * J;

  // ---- pass 1: row maximum and 1 / sum of exp ----
  for (int r = w; r < kCoarseRows; r += 4) {
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

  // ---- pass 2: C = W V_bar ----
  const int d = threadIdx.x % D, rg = threadIdx.x / D;
  const float* __restrict__ vb = p.vbar + (int64_t)bh * J * D + d;
  float acc[R0];
#pragma unroll
  for (int r = 0; r < R0; ++r) acc[r] = 0.f;
  for (int j0 = 0; j0 < J; j0 += kCoarseCols) {
    // stage the weights of columns j0 .. j0+63 for the 32 rows
    for (int e = threadIdx.x; e < kCoarseCols * kCoarseRows; e += 256) {
      const int r = e / kCoarseCols, c = e % kCoarseCols;
      const int i = i0 + r, j = j0 + c;
      wgt[c][r] = (i < J && j < J) ? __expf(Eb[(int64_t)i * J + j] - mrow[r]) * zinv[r] : 0.f;
    }
    __syncthreads();
    const int nc = min(kCoarseCols, J - j0);
    for (int c = 0; c < nc; ++c) {
      const float v = vb[(int64_t)(j0 + c) * D];
#pragma unroll
      for (int r4 = 0; r4 < R0; r4 += 4) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(&wgt[c][rg * R0 + r4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r4 + e] += wv[e] * v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < R0; ++r) {
    const int i = i0 + rg * R0 + r;
    if (i < J) p.C[((int64_t)bh * J + i) * D + d] = acc[r];
  }
}

hipError_t launch_coarse(const CoarseParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.J + kCoarseRows - 1) / kCoarseRows), (unsigned)p.BH);
  if (p.D == 128)
    coarse_kernel<128><<<grid, dim3(256), 0, s>>>(p);
  else
    coarse_kernel<64><<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsa
