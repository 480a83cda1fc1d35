// Coarse pooled-V branch for gfx950.
//
// Source: "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" -- section 6.7 (coarse
// attention over all logical blocks: C = softmax(E) V_bar, with E the routing
// matrix of section 2.2 and V_bar the per-block means of V; each query block's
// row of C is added to its tokens under a gate, outside the main kernel).
//
// Design (MI355X): a pre-pass writes V_bar transposed ([D][J], zero padded to
// a multiple of 64 columns) as a bf16 pair hi + lo, so the main kernel stages
// it with coalesced 16-byte copies.  The main kernel takes one 256-thread
// workgroup per (batch*head, 32 query blocks) and makes one pass over E with an
// online softmax: per chunk of 64 columns each row's running maximum and sum
// are updated (8 threads per row, shuffles), the accumulated rows are
// rescaled, and C += W V_bar runs on the matrix cores (32 x 32 x 16 products;
// wave w owns channels 32w..32w+31) while the next chunk's global loads are in
// flight.  The weights are split into bf16 hi + lo as well and the products
// taken as hi*hi + hi*lo + lo*hi, which keeps each product within 3 * 2^-18.
// E is read once from HBM; a head's V_bar pair from L2.
#include "bsa_device.hpp"
#include "bsa_internal.hpp"

namespace bsa {

constexpr int kCoarseRows = 32;  // query blocks per workgroup
constexpr int kCoarseCols = 64;  // columns of E per chunk

// V_bar [BH, J, D] fp32 -> vt [2, BH, D, Jp] bf16 (hi, then lo = bf16(v - hi)),
// columns J..Jp-1 zero.  One workgroup per (64 columns, batch*head).
template <int D>
__global__ __launch_bounds__(256) void coarse_split_kernel(const float* __restrict__ vbar, int J, int Jp, int BH,
                                                           __bf16* __restrict__ vt) {
  __shared__ float tile[64][D + 1];
  const int bh = blockIdx.y, j0 = blockIdx.x * 64;
  const float* vb = vbar + (int64_t)bh * J * D;
  for (int t = threadIdx.x; t < 64 * D; t += 256) {
    const int jj = t / D, d = t % D;
    tile[jj][d] = (j0 + jj < J) ? vb[(int64_t)(j0 + jj) * D + d] : 0.f;
  }
  __syncthreads();
  __bf16* hi_out = vt + (int64_t)bh * D * Jp;
  __bf16* lo_out = hi_out + (int64_t)BH * D * Jp;
  for (int t = threadIdx.x; t < D * 8; t += 256) {
    const int d = t / 8, c = t % 8;
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = tile[8 * c + e][d];
      const __bf16 h = (__bf16)x;
      hi[e] = h;
      lo[e] = (__bf16)(x - (float)h);
    }
    *reinterpret_cast<bf16x8*>(hi_out + (int64_t)d * Jp + j0 + 8 * c) = hi;
    *reinterpret_cast<bf16x8*>(lo_out + (int64_t)d * Jp + j0 + 8 * c) = lo;
  }
}

template <int D>
__global__ __launch_bounds__(256) void coarse_kernel(CoarseParams p) {
  constexpr int KC = kCoarseCols, WP = KC + 8;  // padded row of the staged chunks (bf16)
  constexpr int DT = D / 32;
  constexpr int VL = D * (KC / 8) / 256;        // 16-byte loads of each V_bar part per thread per chunk
  __shared__ __align__(16) __bf16 Whi[kCoarseRows * WP], Wlo[kCoarseRows * WP];
  __shared__ __align__(16) __bf16 VThi[D * WP], VTlo[D * WP];
  __shared__ float alpha_sh[kCoarseRows], zinv_sh[kCoarseRows];
  // XCD-aware order: workgroups are dealt round robin over the 8 XCDs, so the
  // tiles of one XCD are made consecutive (one head's row tiles share its L2
  // copy of V_bar) when the grid divides evenly
  const int ntiles = gridDim.x * gridDim.y;
  int lin = blockIdx.y * gridDim.x + blockIdx.x;
  if (ntiles % 8 == 0) lin = (lin % 8) * (ntiles / 8) + lin / 8;
  const int bh = lin / gridDim.x;
  const int i0 = (lin % gridDim.x) * kCoarseRows;
  const int J = p.J, Jp = coarse_jpad(J);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* __restrict__ Eb = p.E + (int64_t)bh * J * J;
  const __bf16* __restrict__ vhi = p.vt + (int64_t)bh * D * Jp;
  const __bf16* __restrict__ vlo = vhi + (int64_t)p.BH * D * Jp;
  // staging role for E: row r, columns 8c .. 8c+7 of the chunk
  const int r = tid / 8, cg = tid % 8;
  const int i = i0 + r;
  const bool row_ok = i < J;
  const bool vec_e = (J & 3) == 0;  // 16-byte aligned rows
  float e[8];
  bf16x8 vh[VL], vl[VL];
  // global loads of chunk j0 into registers (E row piece; V_bar rows d, 8 columns)
  auto load_chunk = [&](int j0) {
    const int jc = j0 + 8 * cg;
    if (row_ok && vec_e && jc + 8 <= J) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(Eb + (int64_t)i * J + jc);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Eb + (int64_t)i * J + jc + 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) e[x] = a[x], e[4 + x] = b[x];
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x) e[x] = (row_ok && jc + x < J) ? Eb[(int64_t)i * J + jc + x] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const int t = tid + 256 * u;
      const int64_t off = (int64_t)(t / 8) * Jp + j0 + 8 * (t % 8);  // inside the zero-padded row
      vh[u] = *reinterpret_cast<const bf16x8*>(vhi + off);
      vl[u] = *reinterpret_cast<const bf16x8*>(vlo + off);
    }
  };
  float m_run = -INFINITY, z_run = 0.f;
  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
  load_chunk(0);
  for (int j0 = 0; j0 < J; j0 += KC) {
    // ---- weights of this chunk, online max / sum (8 threads per row) ----
    float cm = -INFINITY;
#pragma unroll
    for (int x = 0; x < 8; ++x) cm = fmaxf(cm, e[x]);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
    const float m_new = fmaxf(m_run, cm);  // finite for valid rows: every chunk has a valid column
    const float alpha = (m_run == -INFINITY) ? 0.f : __expf(m_run - m_new);
    float zs = 0.f;
    bf16x8 whi, wlo;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const float wv = row_ok ? __expf(e[x] - m_new) : 0.f;
      zs += wv;
      const __bf16 hi = (__bf16)wv;
      whi[x] = hi;
      wlo[x] = (__bf16)(wv - (float)hi);
    }
    *reinterpret_cast<bf16x8*>(&Whi[r * WP + 8 * cg]) = whi;
    *reinterpret_cast<bf16x8*>(&Wlo[r * WP + 8 * cg]) = wlo;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) zs += __shfl_xor(zs, o, 64);
    z_run = z_run * alpha + zs;
    m_run = m_new;
    if (cg == 0) alpha_sh[r] = row_ok ? alpha : 0.f;
    // ---- V_bar chunk: row d of the transposed pair, 8 columns per thread ----
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const int t = tid + 256 * u;
      *reinterpret_cast<bf16x8*>(&VThi[(t / 8) * WP + 8 * (t % 8)]) = vh[u];
      *reinterpret_cast<bf16x8*>(&VTlo[(t / 8) * WP + 8 * (t % 8)]) = vl[u];
    }
    // the next chunk's loads are in flight during the products
    if (j0 + KC < J) load_chunk(j0 + KC);
    __syncthreads();
    if (w < DT) {
      // rescale the accumulated rows: register x holds row 8*(x/4) + 4*(lane/32) + x%4
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[x] *= alpha_sh[8 * (x >> 2) + 4 * (lane >> 5) + (x & 3)];
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        const int ao = (lane & 31) * WP + 16 * ks + 8 * (lane >> 5);
        const int bo = (32 * w + (lane & 31)) * WP + 16 * ks + 8 * (lane >> 5);
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Whi[ao]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Wlo[ao]);
        const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(&VThi[bo]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&VTlo[bo]);
        acc = mfma32(al, bh_, acc);
        acc = mfma32(ah, bl, acc);
        acc = mfma32(ah, bh_, acc);
      }
    }
    __syncthreads();
  }
  if (cg == 0) zinv_sh[r] = (row_ok && z_run > 0.f) ? 1.f / z_run : 0.f;
  __syncthreads();
  if (w < DT) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int row = 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
      if (i0 + row < J) p.C[((int64_t)bh * J + i0 + row) * D + 32 * w + (lane & 31)] = acc[x] * zinv_sh[row];
    }
  }
}

hipError_t launch_coarse(const CoarseParams& p, hipStream_t s) {
  const int Jp = coarse_jpad(p.J);
  const dim3 sgrid((unsigned)(Jp / 64), (unsigned)p.BH);
  const dim3 grid((unsigned)((p.J + kCoarseRows - 1) / kCoarseRows), (unsigned)p.BH);
  if (p.D == 128) {
    coarse_split_kernel<128><<<sgrid, dim3(256), 0, s>>>(p.vbar, p.J, Jp, p.BH, p.vt);
    coarse_kernel<128><<<grid, dim3(256), 0, s>>>(p);
  } else {
    coarse_split_kernel<64><<<sgrid, dim3(256), 0, s>>>(p.vbar, p.J, Jp, p.BH, p.vt);
    coarse_kernel<64><<<grid, dim3(256), 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace bsa
