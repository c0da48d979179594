// Low-rank cache build L = X A on gfx950 MFMA (bf16 products, fp32 sums).
//
// PReCache abstract and Figure 1 caption: each agent's compact low-rank
// cache is precomputed from the hidden states X of a context segment;
// LRAgent abstract: the adapter component is kept in this low-rank form.
// X is [n, hidden] (hidden ~ 4096) and A is [hidden, n_cols] with n_cols
// small (one rank, or the ranks of several adapters side by side: the
// hidden states of a segment build every agent's cache in one pass, PReCache
// Figure 1 caption, A1-A3), so the product is a skinny GEMM bound by reading
// X once. Two launches:
//   1. partial kernel: workgroup = (16-row tile, hidden chunk); each of its 4
//      waves loads its 32-wide k steps of the X rows once, then for every
//      16-column tile of A (A^T of the chunk staged in LDS) runs them on
//      16x16x32 MFMA; the waves' sums are added in LDS and the fp32 partial
//      [16 x n_cols] is written to the workspace.
//   2. finish kernel: workgroup row y = destination group; per output
//      element, the chunk partials are added in a fixed order, rounded once
//      to bf16 and stored densely or through the slot mapping into the
//      group's token-major or rank-major paged pool.
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int kMaxChunk = 1024;

__global__ __launch_bounds__(256) void lr_build_partial_kernel(const BuildArgs a) {
  __shared__ __align__(16) uint16_t sAt[16][kMaxChunk + 8];
  __shared__ float sred[4][16][17];

  const int rt = blockIdx.x / a.ksplit;
  const int ks = blockIdx.x % a.ksplit;
  const int k0 = ks * a.kchunk;
  const int kn = min(a.hidden - k0, a.kchunk);  // > 0 by construction
  const int kpad = (kn + 31) & ~31;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  const int row = rt * 16 + lc;
  const bool row_ok = row < a.n_tokens;
  const uint16_t* xrow = a.X + (size_t)(row_ok ? row : 0) * a.ldx + k0;
  // this wave's k steps of the X rows, read once for all column tiles
  constexpr int kSteps = kMaxChunk / 128;
  bf16x8 xf[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int kk = 32 * wave + 128 * i;
    const bool kok = row_ok && (kk + 8 * lg < kn);
    xf[i] = kok ? as_bf16x8(ld16(xrow + kk + 8 * lg)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  // A rows can be read 8 columns at a time when every row start is 16-byte aligned
  const bool a_vec = ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) && (a.lda % 8 == 0);
  for (int ct = 0; ct < a.col_tiles; ++ct) {
    __syncthreads();
    if (a_vec) {
      // one 16-byte load per (k, 8 columns), transposed into A^T[col][k] in LDS
      for (int e = tid; e < 2 * kpad; e += 256) {
        const int kk = e >> 1, c8 = 8 * (e & 1);
        const int gc = ct * 16 + c8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kk < kn && gc < a.n_cols) v = ld16(a.A + (size_t)(k0 + kk) * a.lda + gc);
        const uint16_t* pv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int j = 0; j < 8; ++j) sAt[c8 + j][kk] = (gc + j < a.n_cols) ? pv[j] : (uint16_t)0;
      }
    } else {
      for (int e = tid; e < 16 * kpad; e += 256) {
        const int kk = e >> 4, col = e & 15;
        const int gc = ct * 16 + col;
        sAt[col][kk] = (kk < kn && gc < a.n_cols) ? a.A[(size_t)(k0 + kk) * a.lda + gc] : (uint16_t)0;
      }
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int kk = 32 * wave + 128 * i;
      if (kk < kpad) {  // uniform
        const bf16x8 ab = as_bf16x8(*reinterpret_cast<const uint4*>(&sAt[lc][kk + 8 * lg]));
        acc = mfma32(xf[i], ab, acc);
      }
    }
    // acc holds D[token 4lg+j][col lc] of this wave's k slice
#pragma unroll
    for (int j = 0; j < 4; ++j) sred[wave][4 * lg + j][lc] = acc[j];
    __syncthreads();
    {
      const int r = tid >> 4, col = tid & 15;
      const int grow = rt * 16 + r, gc = ct * 16 + col;
      if (grow < a.n_tokens && gc < a.n_cols) {
        const float v = sred[0][r][col] + sred[1][r][col] + sred[2][r][col] + sred[3][r][col];
        a.partials[((size_t)ks * a.n_tokens + grow) * a.n_cols + gc] = v;
      }
    }
  }
}

__global__ __launch_bounds__(256) void lr_build_finish_kernel(const BuildArgs a) {
  const int g = blockIdx.y;  // destination group (uniform: its table entries are scalar reads)
  const int c0 = a.group_col[g];
  const int w = a.group_col[g + 1] - c0;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)a.n_tokens * w) return;
  const int i = (int)(e / w), c = (int)(e % w);
  const int col = c0 + c;
  float v = 0.f;
  for (int ks = 0; ks < a.ksplit; ++ks) v += a.partials[((size_t)ks * a.n_tokens + i) * a.n_cols + col];
  const uint16_t b = (uint16_t)(pack_bf16(v, 0.f) & 0xFFFFu);
  uint16_t* L = (uint16_t*)a.group_dst[g];
  const int64_t ld = a.group_ld[g];
  if (!a.slot_mapping) {
    L[(size_t)i * ld + c] = b;
    return;
  }
  const int64_t s = a.slot_mapping[i];
  if (s < 0) return;
  if (a.group_layout[g] == 0)
    L[(size_t)s * ld + c] = b;
  else
    L[((size_t)(s / kBlock) * w + c) * kBlock + (s % kBlock)] = b;
}

}  // namespace

hipError_t launch_lr_build_bf16(const BuildArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(lr_build_partial_kernel, dim3(a.row_tiles * a.ksplit), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)a.max_group_elems;
  hipLaunchKernelGGL(lr_build_finish_kernel, dim3((unsigned)((n + 255) / 256), a.n_groups), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lra
