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
// One launch, one workgroup per (16-row tile, 16-column tile, slice of 512
// hidden values): the four waves of a workgroup run their 32-wide k steps of
// the slice on 16x16x32 MFMA and their sums are added in LDS. A is row-major
// [k][column], so the slice's 16 columns are staged transposed in LDS (A^T
// [column][k]), four k rows at a time per thread (one 8-byte store per
// column). With several slices, each workgroup writes its 16x16 fp32 partial
// to the workspace and takes a ticket from the tile's counter; the workgroup
// that arrives last adds the partials in slice order (so the result does not
// depend on the arrival order), rounds once to bf16, stores densely or
// through the slot mapping into the destination group's token-major,
// rank-major or key-chunked paged pool, and puts the counter back to zero. The column tiles
// of one (row tile, slice) are consecutive work items dealt to one XCD, so
// the X rows they share are read into that L2 once.
//
// Visibility across workgroups (the XCDs have separate L2 caches): partials
// are written and read with agent-scope relaxed atomic stores and loads
// (coherent at agent scope without an L2 write-back), and a workgroup waits
// for its partial stores to complete before its ticket is taken.
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int kBuildWaves = 4;
constexpr int kBuildThreads = kBuildWaves * 64;
constexpr int kAtPitch = kBuildSlice + 16;  // bf16; 264 dwords per row: the 16-byte reads of 16 rows are conflict-free
constexpr int kStepsPerWave = kBuildSlice / (32 * kBuildWaves);  // k steps of one wave
constexpr int kItemsPerThread = (kBuildSlice / 4) * 2 / kBuildThreads;  // (4 k rows, 8 columns) items
static_assert(kItemsPerThread >= 1, "whole staging items per thread");

__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// cache-policy operand of a buffer load that is coherent at agent scope (the
// scope bit the compiler sets on a relaxed agent-scope atomic load)
constexpr int kAgentScope = 16;

// One launch covers row tiles rt0 .. rt0 + n_rt - 1 (all their column tiles).
__global__ __launch_bounds__(kBuildThreads) void lr_build_kernel(const BuildArgs a, int rt0, int n_rt) {
  __shared__ __align__(16) uint16_t sAt[16][kAtPitch];
  __shared__ float sred[kBuildWaves][16][17];
  __shared__ int s_ticket;

  const int n_items = n_rt * a.ksplit * a.col_tiles;
  const int per = (n_items + kNumXcd - 1) / kNumXcd;
  const int logical = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (logical >= n_items) return;
  // work item -> (row tile, slice, column tile), column tile fastest
  const int ct = logical % a.col_tiles;
  const int rs = logical / a.col_tiles;
  const int ks = rs % a.ksplit;
  const int rt_local = rs / a.ksplit;
  const int tile_local = rt_local * a.col_tiles + ct;  // tile index within this launch
  const int rt = rt0 + rt_local;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  // output element of this thread (row r, column col of the tile) and its slot,
  // requested first (the store needs it at the very end)
  const int r = tid >> 4, col = tid & 15;
  const int grow = rt * 16 + r, gc = ct * 16 + col;
  const bool on = grow < a.n_tokens && gc < a.n_cols;
  const int64_t slot = (on && a.slot_mapping) ? a.slot_mapping[grow] : 0;

  const int k0 = ks * kBuildSlice;
  const int kn = min(kBuildSlice, a.hidden - k0);
  const int kpad = (kn + 31) & ~31;
  // one descriptor for the tile's X rows (a per-lane base would put the
  // descriptor in vector registers and turn every load into a loop over
  // lanes); rows past n_tokens lie beyond its range and read zero
  const int rows_valid = min(16, a.n_tokens - rt * 16);
  const auto rx = buf_rsrc(a.X + (size_t)rt * 16 * a.ldx, (uint32_t)(((int64_t)(rows_valid - 1) * a.ldx + a.hidden) * 2));
  const uint32_t a_bytes = (uint32_t)((int64_t)a.hidden * a.lda * 2);  // < 2^31 (checked on the host)
  // A rows can be read 8 columns at a time when every row start is 16-byte aligned
  const bool a_vec = ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) && (a.lda % 8 == 0);

  // this wave's X operands. No condition around the loads (a uniform one
  // becomes a branch, and each branch waits for the loads in flight): rows
  // past n_tokens and k past the hidden size read zero through the range check.
  bf16x8 xv[kStepsPerWave];
#pragma unroll
  for (int i = 0; i < kStepsPerWave; ++i) {
    const int k = k0 + 32 * (wave + kBuildWaves * i) + 8 * lg;
    xv[i] = as_bf16x8(bld16(rx, k < a.hidden ? (int)(((int64_t)lc * a.ldx + k) * 2) : kOob));
  }
  if (a_vec) {
    // item = (4 k rows, 8 columns): four 16-byte loads, eight 8-byte stores
    // (every load of the thread issued before its first store);
    // k rows past the hidden size read zero through the range check, columns
    // past n_cols are zeroed at the store. The descriptor from values marked
    // uniform (built from the argument alone it was kept in vector registers,
    // every load a loop over lanes).
    const uint64_t a_addr = reinterpret_cast<uintptr_t>(a.A);
    const uint64_t a_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a_addr);
    const uint64_t a_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a_addr >> 32));
    const auto ra = buf_rsrc(reinterpret_cast<const void*>(a_lo | (a_hi << 32)),
                             (uint32_t)__builtin_amdgcn_readfirstlane((int)a_bytes));
    uint4 rv[kItemsPerThread][4];
#pragma unroll
    for (int it = 0; it < kItemsPerThread; ++it) {
      const int e = tid + it * kBuildThreads;
      const int kq = (e >> 1) * 4, gc8 = ct * 16 + 8 * (e & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rv[it][j] = bld16(ra, k0 + kq + j < a.hidden ? (int)(((int64_t)(k0 + kq + j) * a.lda + gc8) * 2) : kOob);
    }
#pragma unroll
    for (int it = 0; it < kItemsPerThread; ++it) {
      const int e = tid + it * kBuildThreads;
      const int kq = (e >> 1) * 4, c8 = 8 * (e & 1), gc8 = ct * 16 + c8;
      const uint16_t* p0 = reinterpret_cast<const uint16_t*>(&rv[it][0]);
      const uint16_t* p1 = reinterpret_cast<const uint16_t*>(&rv[it][1]);
      const uint16_t* p2 = reinterpret_cast<const uint16_t*>(&rv[it][2]);
      const uint16_t* p3 = reinterpret_cast<const uint16_t*>(&rv[it][3]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool cok = gc8 + j < a.n_cols;
        const uint2 v = cok ? make_uint2(p0[j] | ((uint32_t)p1[j] << 16), p2[j] | ((uint32_t)p3[j] << 16))
                            : make_uint2(0, 0);
        *reinterpret_cast<uint2*>(&sAt[c8 + j][kq]) = v;
      }
    }
  } else {
    for (int e = tid; e < 16 * kBuildSlice; e += kBuildThreads) {
      const int kk = e >> 4, cc = e & 15;
      const int gcc = ct * 16 + cc;
      sAt[cc][kk] = (kk < kn && gcc < a.n_cols) ? a.A[(size_t)(k0 + kk) * a.lda + gcc] : (uint16_t)0;
    }
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kStepsPerWave; ++i) {
    const int kk = 32 * (wave + kBuildWaves * i);
    if (kk < kpad) {  // uniform
      const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(&sAt[lc][kk + 8 * lg]));
      acc = mfma32(xv[i], av, acc);
    }
  }
  // acc holds the wave's partial D[token 4lg + j][column lc]
#pragma unroll
  for (int j = 0; j < 4; ++j) sred[wave][4 * lg + j][lc] = acc[j];
  __syncthreads();
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < kBuildWaves; ++w) v += sred[w][r][col];

  if (a.ksplit > 1) {
    float* part = a.partials + (size_t)tile_local * a.ksplit * kBuildThreads;
    store_agent(part + ks * kBuildThreads + tid, v);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial store has completed
    __syncthreads();                // ... and every other thread's
    if (tid == 0)
      s_ticket = __hip_atomic_fetch_add(a.counters + tile_local, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != a.ksplit - 1) return;  // not the last slice of this tile to arrive
    // every slice's partial is stored: add them in slice order, eight loads in
    // flight at a time (agent-scope loads, as the stores; loads past the last
    // slice read zero through the range check and are not added)
    const auto rp = buf_rsrc(part, (uint32_t)(a.ksplit * kBuildThreads * 4));
    v = 0.f;
    for (int j0 = 0; j0 < a.ksplit; j0 += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        t[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rp, j0 + j < a.ksplit ? ((j0 + j) * kBuildThreads + tid) * 4 : kOob, 0,
                                             kAgentScope));
#pragma unroll
      for (int j = 0; j < 8; ++j) v = j0 + j < a.ksplit ? v + t[j] : v;
    }
    if (tid == 0) __hip_atomic_store(a.counters + tile_local, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const uint16_t b = (uint16_t)(pack_bf16(v, 0.f) & 0xFFFFu);
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
      else if (a.group_layout[g] == 1)
        L[((size_t)(slot / kBlock) * w + c) * kBlock + (slot % kBlock)] = b;
      else
        L[(size_t)(slot / kBlock) * kBlock * w + ((c / 8) * kBlock + slot % kBlock) * 8 + c % 8] = b;
    }
  }
}

}  // namespace

int build_tiles_per_launch(int col_tiles) { return max(1, kBuildCounterSlots / col_tiles) * col_tiles; }

size_t build_workspace_bytes(int n_tokens, int hidden, int n_cols) {
  const int ksplit = (hidden + kBuildSlice - 1) / kBuildSlice;
  if (ksplit <= 1 || n_tokens <= 0) return 0;
  const int col_tiles = (n_cols + 15) / 16;
  const int tiles = min(((n_tokens + 15) / 16) * col_tiles, build_tiles_per_launch(col_tiles));
  return (size_t)kBuildCounterSlots * sizeof(int) + (size_t)tiles * ksplit * kBuildThreads * sizeof(float);
}

// Row tiles in launches of at most kBuildCounterSlots tiles (the counters of
// one launch are reused by the next: the last workgroup of every tile has put
// its counter back to zero when the launch ends).
hipError_t launch_lr_build_bf16(const BuildArgs& a, hipStream_t stream) {
  const int rt_per_launch = a.ksplit > 1 ? build_tiles_per_launch(a.col_tiles) / a.col_tiles : a.row_tiles;
  for (int rt0 = 0; rt0 < a.row_tiles; rt0 += rt_per_launch) {
    const int n_rt = min(rt_per_launch, a.row_tiles - rt0);
    const int n_items = n_rt * a.ksplit * a.col_tiles;
    const int per = (n_items + kNumXcd - 1) / kNumXcd;
    hipLaunchKernelGGL(lr_build_kernel, dim3(per * kNumXcd), dim3(kBuildThreads), 0, stream, a, rt0, n_rt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lra
