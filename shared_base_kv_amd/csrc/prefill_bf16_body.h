// Body of the prefill workgroup (one query tile of one sequence and KV
// head); the kernel that runs it is in prefill_bf16.hip.
//
// Each sequence appends a chunk of q_len new tokens after its context
// (PReCache, Figure 1 caption: an agent's turn is prefilled over its new
// segment on top of the shared context); query i sits at position
// T - q_len + i and sees keys 0..position. Keys and values are the shared
// base plus the agent's low-rank adapter part (LRAgent: Efficient KV Cache
// Sharing for Multi-LoRA LLM Agents, abstract), and the adapter part is never
// written to device memory at full dimension: per 64-key tile the adapter
// key rope(L_k B_k) and the adapter value L_v B_v are rebuilt on MFMA, added
// to the base key and value and rounded once to bf16 into the LDS tiles.
// (The decode kernel keeps values in rank space, P L_v and then B_v once per
// row. A prefill workgroup has 256 query rows per KV head, twice the head
// dimension, so rebuilding a tile's 64 values takes half the products of
// 256 rows of P L_v, and no rank-space accumulator takes registers.)
//
// Work decomposition: one workgroup = (sequence s, KV head h, query tile);
// a query tile has 256 rows = 256/G query tokens x G query heads. Each of
// the 8 waves (two per SIMD) consumes 32 query rows (scores, softmax, P V on
// the matrix cores) and also produces part of the next tile: with a key
// adapter every wave loads and rebuilds half of one 16-key cache block (half
// of the rotary pairs and of the value dims), so the rebuild's registers fit
// beside the consumer's; without one, waves 0..3 each take a whole block.
// Two consumers per SIMD let one wave's softmax, rebuild and LDS waits run
// under the other's matrix work. All tiles of one KV head are dealt to one
// XCD, so the keys they share (the common prefix) stream through one L2.
//
// Matrix-core mapping (16x16 tiles):
//   X^T[dim, key]   = B_k^T L_k^T        (producer: its block's keys, 16x16x16 / 16x16x32)
//   V_a[key, dim]   = V + L_v B_v        (producer: V in the accumulator; L_v turned to
//                                         [key][rank] through the wave's own LDS rows)
//   S^T[key, row]   = K_a Q^T            (16x16x32, K_a from LDS)
//   O^T[dim, row]  += V_a^T P^T          (16x16x32, V_a^T from LDS, P^T from the S^T accumulators)
//
// Pipeline (one barrier per tile): in step t each wave issues the scores of
// tile t and P V of tile t-1 together, runs the softmax of tile t while the
// matrix cores work through them, then rebuilds its part of tile t+1 into
// the other LDS buffers and issues the loads of tile t+2. Keys are
// double-buffered in LDS and V^T triple-buffered (tile t-1 is read while
// t+1 is written). The rotation of the adapter key at position 64t + o is
// split by angle addition into a per-tile part (64t, one table of 64 pairs
// per tile) and a per-lane part (o, fixed for the whole loop), so no
// transcendental is evaluated per element.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace lra {
namespace pf {
namespace {

constexpr int D = 128;
constexpr int kTile = 64;      // keys per tile (4 cache blocks)
constexpr int kKPitch = D + 16;         // LDS row pitch of the key tile (bf16; 72 dwords: 16-byte reads conflict-free)
constexpr int kVPitch = kTile + 8;      // LDS row pitch of the V^T tile (bf16)
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

// Values: rank space (O accumulates P V_base, C accumulates P L_v, C B_v
// once per row after the key loop) except at rank 64 with both adapters,
// where the two rank-space row tiles of a wave do not fit the registers
// beside the key rebuild: there the producers rebuild the values as
// V + L_v B_v into the V^T tile instead (measured: 0.905 -> 0.612 ms for the
// 4 x 512-token chunk at rank 64; at ranks 16 and 32, and with a value
// adapter alone, the rank-space form is 2-25% faster).
constexpr bool value_rebuild(int rp, bool kad, bool vad) { return rp == 64 && kad && vad; }

// v, made opaque to the compiler when ON (so that values derived from it are
// recomputed where they are used rather than kept in registers).
template <bool ON>
__device__ __forceinline__ int opaque_if(int v) {
  if constexpr (ON) asm volatile("" : "+v"(v));
  return v;
}

// One producer wave's share of a 16-key cache block of a tile, on its way
// from HBM: the whole block (NH = 1) or half of it (NH = 2: rotary pairs
// 32 hh .. 32 hh + 31, and V^T rows (value dims) 64 hh .. 64 hh + 63).
template <int RP, int NH, bool VREB>
struct TileRegs {
  static constexpr int NCB = 4 / NH;  // 16-pair groups cb
  static constexpr int NPAR = 2 / NH; // V^T row parities (rank space)
  static constexpr int NDT = 8 / NH;  // 16-dim value tiles (value rebuild)
  uint2 kbl[NCB], kbh[NCB];     // base keys of key lc as loaded: 16 bytes per lane per pair of 16-dim tiles, and +64
  uint4 vv[VREB ? 1 : NPAR][2]; // rank space: V^T row 64 u + 32k + lane/2, keys 8(lane&1) .. +7 of the block
  uint2 vb[VREB ? NDT : 1];     // value rebuild: base values of dim 16dt + lc, keys 4lg .. +3 of the block
  uint4 lk[RP == 64 ? 2 : 1];   // L_k row of key lc: ranks 8lg.. (RP 32/64) or 4lg.. (RP 16, .x .y)
  uint4 lvv[VREB ? (RP == 64 ? 2 : 1) : NPAR];  // L_v^T item lane + 64 u: rank item/2, keys 8 (item%2) .. +7
};


}  // namespace
}  // namespace pf
}  // namespace lra
