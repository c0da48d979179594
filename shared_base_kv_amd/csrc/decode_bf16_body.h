// Types and helpers of the decode workgroup; its statements are in
// decode_bf16_body.inc, included by the kernels that run it (decode_bf16.hip:
// the decode call; mixed_bf16.hip: decode and prefill in one grid).
//
// What is computed (LRAgent: Efficient KV Cache Sharing for Multi-LoRA LLM
// Agents, abstract): keys and values are a shared base part plus an adapter
// part kept low-rank; the attention is reordered so the adapter part never
// exists at full dimension in device memory:
//   score(n) = q . K_base[n] + q . rope_n(L_k[n] B_k)   (adapter key rebuilt per
//              16-token block in registers, never stored)
//   out      = (sum_n p_n V_base[n] + (sum_n p_n L_v[n]) B_v) / sum_n p_n
//              (value adapter applied once per output row, after the token loop)
//
// Work decomposition. One workgroup = (group g, row tile rt, split c, KV
// head h). A group is a set of sequences sharing one base context; a row
// tile holds up to 16 query rows (up to NA sequences x G query heads of head
// h), so the base K/V of a block is read once for all agents of the tile. A
// split is a contiguous token range; its 8 waves take interleaved 16-token
// cache blocks, two blocks in flight per wave, and keep independent
// online-softmax states, merged in LDS at the end. The merged state of the
// split gets its value adapter term on MFMA and is written as one record per
// row; a second kernel merges the records of all splits.
//
// Matrix-core mapping (16x16 MFMA tiles, tokens on the M side):
//   S^T[token, row]   = K_base[token, :] Q^T            (16x16x32)
//                     + sum_a Y_a[token, :] Qmask_a^T    (16x16x32, Y_a = rotated rebuild)
//   X_a^T[dim, token] = B_k,a^T[dim, :] L_k^T[:, token]  (16x16x16 or 16x16x32 over rank)
//   O^T[dim, row]    += V^T[dim, token] P^T[token, row]  (16x16x16 over the block)
//   C^T[rank, row]   += L_v^T[rank, token] P^T[token, row]
//   O'^T[dim, row]    = O^T + B_v,a^T[dim, rank] C^T[rank, row]  (after the merge; C as bf16 hi + lo)
// The accumulator layout of one product is the operand layout of the next,
// so rebuilt keys and probabilities never leave registers.
//
// Rotation angles: the angle of pair i at position tb + lc (block start tb,
// lane column lc) is split by angle addition into a per-block part (64
// pairs, computed by the wave once per block, one pair per lane) and a
// per-column part (a table of 16 x 64 pairs built once per workgroup), so
// no transcendental is evaluated per element.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace lra {
namespace dec {
namespace {

constexpr int D = 128;
constexpr int kQPitch = D + 8;                    // LDS row pitch of the query tile (bf16)
constexpr float kMaxSlack = 8.f;                  // log2 of the largest probability kept before a rescale
constexpr int kRotPitch = kMaxRopePairs + 4;      // LDS row pitch of the per-column rotation table (f16 pairs)
constexpr int kQpPitch = D + 8;                   // LDS row pitch of the permuted f16 query tile (halves)

struct TileAgent {
  const uint16_t* lk;
  const uint16_t* lv;
  const uint16_t* bk;
  const uint16_t* bv;
  int r;
  int seq;
  int start;  // activation position: tokens before it carry no adapter term
};

__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float2 cos_sin_rev(double x) {
  const float f = (float)(x - __builtin_floor(x));
  return make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
}

// Registers of one 16-token cache block of one wave: base K rows, V^T rows
// and the low-rank rows of the tile's first agent (every agent's, when the
// agents share their low-rank pools).
template <int RP>
struct Blk {
  static constexpr int KC = RP >= 32 ? RP / 32 : 1;
  static constexpr int NRT = RP / 16;
  bf16x8 kr[4];     // K_base[token lc][dims 32ks + 8lg .. +7]
  uint2 vr[8];      // V^T[dim 16cb + lc][tokens 4lg .. +3]
  uint2 lk16;       // L_k[token lc][ranks 4lg .. +3]              (RP 16)
  bf16x8 lk32[KC];  // L_k[token lc][ranks 32kc + 8lg .. +7]       (RP 32, 64)
  uint2 lv[NRT];    // L_v[rank 16rr + lc][tokens 4lg .. +3]
};

// Low-rank rows of agents 1 .. NA-1 of the tile for one block (agent 0's
// travel with the block). Loaded only when the agents keep separate pools;
// otherwise the loads get zero-length ranges.
template <int RP, int NA>
struct AgentRows {
  static constexpr int KC = RP >= 32 ? RP / 32 : 1;
  static constexpr int NRT = RP / 16;
  static constexpr int N = NA > 1 ? NA - 1 : 1;
  uint2 lk16[N];
  bf16x8 lk32[N][KC];
  uint2 lv[N][NRT];
};

struct WorkItem {
  int g, rt, h, c, s_first, s0, ns, T, nact, t_begin, t_end, tile_id;
};

// Logical work item -> (group, row tile, split, KV head). The KV head varies
// fastest, so the heads of one split are consecutive items and share an XCD
// (the low-rank rows of those tokens, shared by every head, reach that L2 once).
// First part: the group's sequences and the row tile's slots (false: the
// tile has no sequences).
__device__ __forceinline__ bool decode_item_rows(const DecodeArgs& a, int logical, WorkItem& w) {
  int rem = logical;
  w.h = rem % a.Hkv;
  rem /= a.Hkv;
  w.c = rem % a.nsplit;
  rem /= a.nsplit;
  w.rt = rem % a.row_tiles;
  w.g = rem / a.row_tiles;
  w.s_first = a.group_offsets ? sload(a.group_offsets + w.g) : w.g;
  const int s_end = a.group_offsets ? sload(a.group_offsets + w.g + 1) : w.g + 1;
  w.s0 = w.s_first + w.rt * a.apt;
  w.ns = min(a.apt, s_end - w.s0);
  w.tile_id = (w.g * a.row_tiles + w.rt) * a.Hkv + w.h;
  return w.ns > 0;
}
// Second part: the group's context length and this split's token range.
__device__ __forceinline__ void decode_item_span(const DecodeArgs& a, WorkItem& w) {
  w.T = sload(a.context_lens + w.s_first);
  w.nact = (w.T + a.split - 1) / a.split;
  w.t_begin = w.c * a.split;
  w.t_end = min(w.T, w.t_begin + a.split);
}

// Compile-time sizes of one workgroup's LDS.
template <int RP, int NA, bool KAD, bool VAD>
struct Cfg {
  static constexpr int PW = D + (VAD ? RP : 0);  // floats per row of a merged state (O, then C)
  // LDS row pitch of the merge buffer: an odd multiple of 8 floats, so the 16
  // rows of a 16-byte access by one wave fall in distinct banks
  static constexpr int PWP = PW + 8;
  static constexpr int HW = kDecodeWaves / 2;
  static constexpr int kBtBytes = KAD ? NA * D * RP * 2 : 0;
  static constexpr int kMergeBytes = HW * 16 * PWP * 4;
  static constexpr int kRegion = kBtBytes > kMergeBytes ? kBtBytes : kMergeBytes;
};

// LDS arrays of one workgroup (a kernel that runs this workgroup next to
// another kind carves them from one buffer).
template <int RP, int NA, bool KAD, bool VAD>
struct Lds {
  using C = Cfg<RP, NA, KAD, VAD>;
  alignas(16) unsigned char s_region[C::kRegion];        // B_k^T [al][dim][k] in the loop, merge buffer after
  alignas(16) uint16_t s_bvt[VAD ? NA * D * RP : 8];     // B_v^T [al][dim][k]
  alignas(16) uint16_t s_q[16 * kQPitch];                // query tile [row][dim]
  alignas(16) uint16_t s_qp[KAD ? 16 * kQpPitch : 8];    // f16 query tile, k slots of the adapter product
  alignas(16) f16x2 s_roff[KAD ? 16 * kRotPitch : 4];    // (cos, sin) of lc theta_i, [lc][i]
  alignas(16) f16x2 s_rbase[KAD ? kDecodeWaves : 1][kMaxRopePairs];  // per wave: (cos, sin) of tb theta_i
  double s_rev[kMaxRopePairs];
  TileAgent s_agent[NA];
  float s_ml[2][C::HW][16];
  int s_shared_l;
  int s_lead;  // first agent slot of the tile with an adapter (its rows travel with the blocks)
  int s_start_min, s_start_max;  // activation positions over the tile's adapted slots
};

}  // namespace
}  // namespace dec
}  // namespace lra
