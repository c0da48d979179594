// Types and helpers of the decode workgroup; its statements are in
// decode_bf16_body.inc, included by the decode kernel (decode_bf16.hip).
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
// LDS row pitches of the tiles that 16 rows read 16 bytes at a time: 72
// dwords. A 16-byte LDS read serves lanes 0-7 with 16-23 (and so on) in one
// pass, so the 8 rows of a pass must start 8 banks apart modulo 64: any odd
// multiple of 8 dwords (measured on MI355X: no bank conflict at 72 dwords,
// about 4 extra cycles per read at 68 and 36).
constexpr int kQPitch = D + 16;                   // query tile (bf16)
constexpr float kMaxSlack = 8.f;                  // log2 of the largest probability kept before a rescale
constexpr int kRotPitch = kMaxRopePairs + 8;      // per-column rotation table (f16 pairs)
constexpr int kQpPitch = D + 16;                  // permuted f16 query tile (halves)


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
  uint2 vr[8];      // V^T[dim 16cb + lc][tokens 4lg .. +3] (RP 16); else as loaded, 16 bytes
                    // per lane per pair of dim tiles (token_rows_to_operands)
  uint2 lk16;       // L_k[token lc][ranks 4lg .. +3]              (RP 16)
  bf16x8 lk32[KC];  // L_k[token lc][ranks 32kc + 8lg .. +7]       (RP 32, 64)
  uint2 lv[NRT];    // L_v rows: RP 16: [rank lc][tokens 4lg .. +3]; else as loaded, like vr
};

// Low-rank rows of the tile's agents for one block: of agents 1 .. NA-1
// (ALL false: agent 0's travel with the block; loaded only when the agents
// keep separate pools), or of every agent slot (ALL true; with shared pools
// slot 0 holds the lead's rows and the others read nothing).
template <int RP, int NA, bool ALL>
struct AgentRows {
  static constexpr int KC = RP >= 32 ? RP / 32 : 1;
  static constexpr int NRT = RP / 16;
  static constexpr int N = ALL ? NA : (NA > 1 ? NA - 1 : 1);
  uint2 lk16[N];
  bf16x8 lk32[N][KC];
  uint2 lv[N][NRT];  // as in Blk
};

// The argument fields the work-item preamble needs first. The kernel takes
// them as leading scalar arguments (fourteen dwords, nsplit, apt and Hkv
// packed in one), which the dispatch preloads into SGPRs when the library is
// built with kernel-argument preloading: the first dependent loads (context
// length, agent ids, block-table entries) then go out without waiting for a
// read of the kernel-argument segment.
struct DecodeHot {
  const int32_t* context_lens;
  const int32_t* block_tables;
  const int32_t* agent_ids;
  const int32_t* group_offsets;
  int n_work, nsplit, apt, Hkv, row_tiles, split, max_blocks, S;
};
// nsplit (< 256), apt (< 256) and Hkv (< 65536) in one dword
__host__ __device__ __forceinline__ int pack_hot_dims(int nsplit, int apt, int Hkv) {
  return nsplit | (apt << 8) | (Hkv << 16);
}
__device__ __forceinline__ DecodeHot make_hot(const int32_t* context_lens, const int32_t* block_tables,
                                              const int32_t* agent_ids, const int32_t* group_offsets, int n_work,
                                              int dims, int row_tiles, int split, int max_blocks, int S) {
  DecodeHot h;
  h.context_lens = context_lens;
  h.block_tables = block_tables;
  h.agent_ids = agent_ids;
  h.group_offsets = group_offsets;
  h.n_work = n_work;
  h.nsplit = dims & 0xff;
  h.apt = (dims >> 8) & 0xff;
  h.Hkv = (int)((unsigned)dims >> 16);
  h.row_tiles = row_tiles;
  h.split = split;
  h.max_blocks = max_blocks;
  h.S = S;
  return h;
}

struct WorkItem {
  int g, rt, h, c, s_first, s0, ns, T, nact, t_begin, t_end, tile_id;
};

// Logical work item -> (group, row tile, split, KV head). The KV head varies
// fastest, then the row tile, so the heads and row tiles of one split are
// consecutive items on one XCD (the low-rank rows of those tokens, shared by
// every head, and the base blocks, shared by the row tiles of a group, reach
// that L2 once).
// First part: the group's sequences and the row tile's slots (false: the
// tile has no sequences).
__device__ __forceinline__ bool decode_item_rows(const DecodeHot& a, int logical, WorkItem& w) {
  int rem = logical;
  w.h = rem % a.Hkv;
  rem /= a.Hkv;
  w.rt = rem % a.row_tiles;
  rem /= a.row_tiles;
  w.c = rem % a.nsplit;
  w.g = rem / a.nsplit;
  // group_offsets rise from 0 to S, so the first group starts at 0 and the
  // last ends at S without a load (one dependent round trip fewer for a call
  // with one group)
  int s_end;
  if (a.group_offsets) {
    w.s_first = 0;
    s_end = a.S;
    if (w.g > 0) w.s_first = sload(a.group_offsets + w.g);
    // not the last group: (g + 1) * items per group < n_work
    if ((w.g + 1) * a.nsplit * a.row_tiles * a.Hkv < a.n_work) s_end = sload(a.group_offsets + w.g + 1);
  } else {
    w.s_first = w.g;
    s_end = w.g + 1;
  }
  w.s0 = w.s_first + w.rt * a.apt;
  w.ns = min(a.apt, s_end - w.s0);
  w.tile_id = (w.g * a.row_tiles + w.rt) * a.Hkv + w.h;
  return w.ns > 0;
}
// Second part: this split's token range, from the group's context length T
// (read by the caller from context_lens[s_first]).
__device__ __forceinline__ void decode_item_span(const DecodeHot& a, WorkItem& w, int T) {
  w.T = T;
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


}  // namespace
}  // namespace dec
}  // namespace lra
