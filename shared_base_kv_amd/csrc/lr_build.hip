// Low-rank cache build L = X A on gfx950 MFMA (bf16 products, fp32 sums).
//
// PReCache abstract and Figure 1 caption: each agent's compact low-rank
// cache is precomputed from the hidden states X of a context segment;
// LRAgent abstract: the adapter component is kept in this low-rank form.
// X is [n, hidden] (hidden ~ 4096) and A is [hidden, n_cols] with n_cols
// small (one rank, or the ranks of several adapters side by side: the
// hidden states of a segment build every agent's cache in one pass, PReCache
// Figure 1 caption, A1-A3), so the product is a skinny GEMM.
//
// One launch, one workgroup per (16-row tile, 16-column tile): the hidden
// dimension is split over the 16 waves (each runs its 32-wide k steps on a
// 16x16x32 MFMA), the waves' sums are added in LDS, rounded once to bf16 and
// stored densely or through the slot mapping into the destination group's
// token-major or rank-major paged pool. A is row-major [k][column], so each
// chunk of its 16 columns is staged transposed in LDS (A^T [column][k]),
// four k rows at a time per thread (one 8-byte store per column). The column
// tiles of one row tile are consecutive work items dealt to one XCD, so the
// X rows they share are read into that L2 once.
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int kBuildWaves = 16;
constexpr int kBuildThreads = kBuildWaves * 64;
constexpr int kBuildK = 4096;          // hidden values of A^T staged per round
constexpr int kAtPitch = kBuildK + 16;  // bf16; 2056 dwords per row: the 16-byte reads of 16 rows are conflict-free
constexpr int kStepsPerRound = kBuildK / (32 * kBuildWaves);  // k steps of one wave per round
constexpr int kItemsPerThread = (kBuildK / 4) * 2 / kBuildThreads;  // (4 k rows, 8 columns) items

__global__ __launch_bounds__(kBuildThreads) void lr_build_kernel(const BuildArgs a) {
  __shared__ __align__(16) uint16_t sAt[16][kAtPitch];
  __shared__ float sred[kBuildWaves][16][17];

  const int n_items = a.row_tiles * a.col_tiles;
  const int per = (n_items + kNumXcd - 1) / kNumXcd;
  const int logical = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (logical >= n_items) return;
  const int rt = logical / a.col_tiles, ct = logical % a.col_tiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  // one descriptor for the tile's X rows (a per-lane base would put the
  // descriptor in vector registers and turn every load into a loop over
  // lanes); rows past n_tokens lie beyond its range and read zero
  const int rows_valid = min(16, a.n_tokens - rt * 16);
  const auto rx = buf_rsrc(a.X + (size_t)rt * 16 * a.ldx, (uint32_t)(((int64_t)(rows_valid - 1) * a.ldx + a.hidden) * 2));
  const uint32_t a_bytes = (uint32_t)((int64_t)a.hidden * a.lda * 2);  // < 2^31 (checked on the host)
  // A rows can be read 8 columns at a time when every row start is 16-byte aligned
  const bool a_vec = ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) && (a.lda % 8 == 0);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.hidden; k0 += kBuildK) {
    const int kn = min(kBuildK, a.hidden - k0);
    const int kpad = (kn + 31) & ~31;
    // this wave's X operands of the round. No condition around the loads (a
    // uniform one becomes a branch, and each branch waits for the loads in
    // flight): rows past n_tokens and k past the hidden size read zero
    // through the range check.
    bf16x8 xv[kStepsPerRound];
#pragma unroll
    for (int i = 0; i < kStepsPerRound; ++i) {
      const int kk = 32 * wave + 32 * kBuildWaves * i;
      const int k = k0 + kk + 8 * lg;  // k past the hidden size (padding steps) reads zero
      xv[i] = as_bf16x8(bld16(rx, k < a.hidden ? (int)(((int64_t)lc * a.ldx + k) * 2) : kOob));
    }
    __syncthreads();  // the previous round's reads of sAt are done
    if (a_vec) {
      // item = (4 k rows, 8 columns): four 16-byte loads, eight 8-byte
      // stores; every load of the thread is issued before the first store,
      // unconditionally (k rows past the hidden size read zero through the
      // range check; columns past n_cols are zeroed at the store)
      // the descriptor from values marked uniform (built from the argument
      // alone it was kept in vector registers, every load a loop over lanes)
      const uint64_t a_addr = reinterpret_cast<uintptr_t>(a.A);
      const uint64_t a_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a_addr);
      const uint64_t a_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a_addr >> 32));
      const auto ra = buf_rsrc(reinterpret_cast<const void*>(a_lo | (a_hi << 32)),
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)a_bytes));
      uint4 r[kItemsPerThread][4];
#pragma unroll
      for (int it = 0; it < kItemsPerThread; ++it) {
        const int e = tid + it * kBuildThreads;
        const int kq = (e >> 1) * 4, gc = ct * 16 + 8 * (e & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[it][j] = bld16(ra, (int)(((int64_t)(k0 + kq + j) * a.lda + gc) * 2));
      }
#pragma unroll
      for (int it = 0; it < kItemsPerThread; ++it) {
        const int e = tid + it * kBuildThreads;
        const int kq = (e >> 1) * 4, c8 = 8 * (e & 1);
        const int gc = ct * 16 + c8;
        if (kq >= kpad) continue;
        const uint16_t* p0 = reinterpret_cast<const uint16_t*>(&r[it][0]);
        const uint16_t* p1 = reinterpret_cast<const uint16_t*>(&r[it][1]);
        const uint16_t* p2 = reinterpret_cast<const uint16_t*>(&r[it][2]);
        const uint16_t* p3 = reinterpret_cast<const uint16_t*>(&r[it][3]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool on = gc + j < a.n_cols;
          const uint2 v = on ? make_uint2(p0[j] | ((uint32_t)p1[j] << 16), p2[j] | ((uint32_t)p3[j] << 16))
                             : make_uint2(0, 0);
          *reinterpret_cast<uint2*>(&sAt[c8 + j][kq]) = v;
        }
      }
    } else {
      for (int e = tid; e < 16 * kpad; e += kBuildThreads) {
        const int kk = e >> 4, col = e & 15;
        const int gc = ct * 16 + col;
        sAt[col][kk] = (kk < kn && gc < a.n_cols) ? a.A[(size_t)(k0 + kk) * a.lda + gc] : (uint16_t)0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kStepsPerRound; ++i) {
      const int kk = 32 * wave + 32 * kBuildWaves * i;
      if (kk < kpad) {  // uniform
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(&sAt[lc][kk + 8 * lg]));
        acc = mfma32(xv[i], av, acc);
      }
    }
  }
  // acc holds the wave's partial D[token 4lg + j][column lc]
#pragma unroll
  for (int j = 0; j < 4; ++j) sred[wave][4 * lg + j][lc] = acc[j];
  __syncthreads();
  if (tid >= 256) return;
  const int r = tid >> 4, col = tid & 15;
  const int grow = rt * 16 + r, gc = ct * 16 + col;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < kBuildWaves; ++w) v += sred[w][r][col];
  const bool on = grow < a.n_tokens && gc < a.n_cols;
  const uint16_t b = (uint16_t)(pack_bf16(v, 0.f) & 0xFFFFu);
  const int64_t slot = (on && a.slot_mapping) ? a.slot_mapping[grow] : 0;
  // destination group of this column (uniform loop over the groups that
  // overlap the tile: the table entries are scalar reads)
  for (int g = 0; g < a.n_groups; ++g) {
    const int c0 = a.group_col[g], c1 = a.group_col[g + 1];
    if (c1 <= ct * 16 || c0 >= ct * 16 + 16) continue;
    if (!on || gc < c0 || gc >= c1) continue;
    const int w = c1 - c0, c = gc - c0;
    uint16_t* L = (uint16_t*)a.group_dst[g];
    const int64_t ld = a.group_ld[g];
    if (!a.slot_mapping)
      L[(size_t)grow * ld + c] = b;
    else if (slot >= 0) {
      if (a.group_layout[g] == 0)
        L[(size_t)slot * ld + c] = b;
      else
        L[((size_t)(slot / kBlock) * w + c) * kBlock + (slot % kBlock)] = b;
    }
  }
}

}  // namespace

hipError_t launch_lr_build_bf16(const BuildArgs& a, hipStream_t stream) {
  const int n_items = a.row_tiles * a.col_tiles;
  const int per = (n_items + kNumXcd - 1) / kNumXcd;
  hipLaunchKernelGGL(lr_build_kernel, dim3(per * kNumXcd), dim3(kBuildThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lra
