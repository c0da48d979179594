// Body of the prefill workgroup (one query tile of one sequence and KV
// head); the kernels that run it are in prefill_bf16.hip (the prefill call)
// and mixed_bf16.hip (decode and prefill in one grid).
//
// Each sequence appends a chunk of q_len new tokens after its context
// (PReCache, Figure 1 caption: an agent's turn is prefilled over its new
// segment on top of the shared context); query i sits at position
// T - q_len + i and sees keys 0..position. Keys and values are the shared
// base plus the agent's low-rank adapter part (LRAgent: Efficient KV Cache
// Sharing for Multi-LoRA LLM Agents, abstract), and the adapter part is never
// written to device memory at full dimension:
//   - per 64-key tile the adapter key rope(L_k B_k) is rebuilt on MFMA,
//     added to the base key and rounded once to bf16 into an LDS key tile;
//   - values stay split: O accumulates P V_base, C accumulates P L_v in rank
//     space, and C B_v is applied once per row after the key loop.
//
// Work decomposition: one workgroup = (sequence s, KV head h, query tile);
// a query tile has 256 rows = 256/G query tokens x G query heads. Each of the
// 8 waves (two per SIMD) consumes 32 query rows (scores, softmax, P V on the
// matrix cores) and also produces part of the next tile: with a key adapter
// every wave loads and rebuilds half of one 16-key cache block (half of the
// rotary pairs and of the V^T rows), so the rebuild's registers fit beside
// the consumer's; without one, waves 0..3 each copy a whole block. Two
// consumers per SIMD let one wave's softmax, rebuild and LDS waits run under
// the other's matrix work. All tiles of one KV head are dealt to one XCD, so
// the keys they share (the common prefix) stream through one L2.
//
// Matrix-core mapping (16x16 tiles):
//   X^T[dim, key]   = B_k^T L_k^T        (per producer: its block's keys, 16x16x16 / 16x16x32)
//   S^T[key, row]   = K_a Q^T            (16x16x32, K_a from LDS)
//   O^T[dim, row]  += V^T P^T            (16x16x32, V^T from LDS, P^T from the S^T accumulators)
//   C^T[rank, row] += L_v^T P^T
//   O^T            += B_v^T C^T          (after the loop; C split into bf16 hi + lo)
//
// Pipeline (one barrier per tile): in step t each wave issues the scores of
// tile t and P V of tile t-1 together, runs the softmax of tile t while the
// matrix cores work through them, then rebuilds its part of tile t+1 into
// the other LDS buffers and issues the loads of tile t+2. Keys are
// double-buffered in LDS and V^T, L_v^T triple-buffered (tile t-1 is read
// while t+1 is written). The rotation of
// the adapter key at position 64t + o is split by angle addition into a
// per-tile part (64t, one table of 64 pairs per tile) and a per-lane part (o,
// fixed for the whole loop), so no transcendental is evaluated per element.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace lra {
namespace pf {
namespace {

constexpr int D = 128;
constexpr int kRows = kPrefillRows;  // query rows per workgroup
constexpr int kTile = 64;      // keys per tile (4 cache blocks)
constexpr int kKPitch = D + 16;         // LDS row pitch of the key tile (bf16; 72 dwords: 16-byte reads conflict-free)
constexpr int kVPitch = kTile + 8;      // LDS row pitch of the V^T / L_v^T tiles (bf16)
constexpr int kKBufs = 2;
constexpr int kVBufs = 3;
constexpr int kThreads = 512;  // 8 waves of 32 query rows
constexpr float kMaxSlack = 8.f;  // log2 of the largest probability kept before a rescale

// V^T and L_v^T tiles keep the 64 keys of a row in the order of the P^T
// operand's k slots: lane group g reads keys 32kp + 4g .. +3 and 32kp + 16 +
// 4g .. +3 as one 16-byte run at 32kp + 8g. kvpos(block, half) is where the
// first of the 4-key runs of keys 8 half .. 8 half + 7 of cache block `block`
// goes; the second run follows 8 halves later.
__device__ __forceinline__ int kvpos(int block, int half) { return 32 * (block >> 1) + 16 * half + 4 * (block & 1); }

// (cos, sin) of one angle given in revolutions, with the revolution count
// reduced exactly in fp64 first.
__device__ __forceinline__ float2 cos_sin_rev(double x) {
  const float f = (float)(x - __builtin_floor(x));
  return make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
}

// One producer wave's share of a 16-key cache block of a tile, on its way
// from HBM: the whole block (NH = 1) or half of it (NH = 2: rotary pairs
// 32 hh .. 32 hh + 31 and the V^T rows of parity hh).
template <int RP, int NH>
struct TileRegs {
  static constexpr int NCB = 4 / NH;  // 16-pair groups cb
  static constexpr int NPAR = 2 / NH; // V^T row parities
  uint2 kbl[NCB], kbh[NCB];    // base keys of key lc: dims 16cb + 4lg .. +3 and +64
  uint4 vv[NPAR][2];           // V^T row 2 lane + parity, keys 8k .. +7 of the block (k = 0, 1)
  uint4 lk[RP == 64 ? 2 : 1];  // L_k row of key lc: ranks 8lg.. (RP 32/64) or 4lg.. (RP 16, .x .y)
  uint4 lvv[NPAR];             // L_v^T item lane + 64 u: rank item/2, keys 8 (item%2) .. +7
};

// LDS arrays of one workgroup (a kernel that runs this workgroup next to
// another kind carves them from one buffer).
template <int RP, bool KAD, bool VAD>
struct Lds {
  alignas(16) uint16_t s_k[kKBufs][kTile * kKPitch];          // rebuilt keys [key][dim]
  alignas(16) uint16_t s_v[kVBufs][D * kVPitch];              // V^T [dim][key]
  alignas(16) uint16_t s_lv[kVBufs][VAD ? RP * kVPitch : 8];  // L_v^T [rank][key]
  alignas(16) uint16_t s_bt[KAD ? D * RP : 8];                // B_k^T [dim][rank]
  alignas(16) uint16_t s_bvt[VAD ? D * RP : 8];               // B_v^T [dim][rank]
  alignas(16) float s_rot[kKBufs][2 * kMaxRopePairs];         // (cos, sin) of 64 t theta_i
  double s_rev[kMaxRopePairs];
};

}  // namespace
}  // namespace pf
}  // namespace lra
