// Low-rank cache build L = X A on gfx950 MFMA (bf16 products, fp32 sums).
//
// PReCache abstract and Figure 1 caption: each agent's compact low-rank
// cache is precomputed from the hidden states X of a context segment;
// LRAgent abstract: the adapter component is kept in this low-rank form.
// X is [n, hidden] (hidden ~ 4096) and A is [hidden, r] with r small, so the
// product is a skinny GEMM bound by reading X once. Two launches:
//   1. partial kernel: workgroup = (16-row tile, hidden chunk); its 4 waves
//      split the chunk in 32-wide k steps on 16x16x32 MFMA, with A^T of the
//      chunk staged in LDS; the waves' sums are added in LDS and the fp32
//      partial [16 x n_cols] is written to the workspace.
//   2. finish kernel: per output element, the chunk partials are added in a
//      fixed order, rounded once to bf16 and stored densely or through the
//      slot mapping into a token-major or rank-major paged pool.
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

  for (int ct = 0; ct < a.col_tiles; ++ct) {
    __syncthreads();
    for (int e = tid; e < 16 * kpad; e += 256) {
      const int kk = e >> 4, col = e & 15;
      const int gc = ct * 16 + col;
      sAt[col][kk] = (kk < kn && gc < a.n_cols) ? a.A[(size_t)(k0 + kk) * a.lda + gc] : (uint16_t)0;
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kk = 32 * wave; kk < kpad; kk += 128) {
      const bool kok = row_ok && (kk + 8 * lg < kn);
      const bf16x8 xa = kok ? as_bf16x8(ld16(xrow + kk + 8 * lg)) : as_bf16x8(make_uint4(0, 0, 0, 0));
      const bf16x8 ab = as_bf16x8(*reinterpret_cast<const uint4*>(&sAt[lc][kk + 8 * lg]));
      acc = mfma32(xa, ab, acc);
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
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)a.n_tokens * a.n_cols) return;
  const int i = (int)(e / a.n_cols), col = (int)(e % a.n_cols);
  float v = 0.f;
  for (int ks = 0; ks < a.ksplit; ++ks) v += a.partials[((size_t)ks * a.n_tokens + i) * a.n_cols + col];
  const uint16_t b = (uint16_t)(pack_bf16(v, 0.f) & 0xFFFFu);
  uint16_t* L = (uint16_t*)a.L;
  if (!a.slot_mapping) {
    L[(size_t)i * a.ldl + col] = b;
    return;
  }
  const int64_t s = a.slot_mapping[i];
  if (s < 0) return;
  if (a.layout == 0)
    L[(size_t)s * a.ldl + col] = b;
  else
    L[((size_t)(s / kBlock) * a.n_cols + col) * kBlock + (s % kBlock)] = b;
}

}  // namespace

hipError_t launch_lr_build_bf16(const BuildArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(lr_build_partial_kernel, dim3(a.row_tiles * a.ksplit), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)a.n_tokens * a.n_cols;
  hipLaunchKernelGGL(lr_build_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lra
