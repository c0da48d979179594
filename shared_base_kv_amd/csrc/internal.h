// Host/device argument blocks and launcher declarations shared by the C-ABI
// layer (lra_api.cpp) and the kernel sources. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lra {

constexpr int kBlock = 16;       // tokens per cache block
constexpr int kNumCU = 256;      // MI355X compute units (8 XCDs x 32)
constexpr int kNumXcd = 8;       // workgroups are dealt round-robin over XCDs
constexpr int kDecodeWaves = 8;  // waves per decode workgroup
constexpr int kWaveBlocks = 2;   // cache blocks per wave in the smallest split
constexpr int kMaxSplits = 64;   // split-K partitions per (group, head, row tile)
constexpr int kMaxTileAgents = 8;  // sequences of one decode row tile
constexpr int kMaxRopePairs = 64;
constexpr int kMaxSplitBlocks = 256;  // cache blocks in one split (split <= 4096 tokens)
// query rows (tokens x query heads of one KV head) per prefill workgroup:
// 8 waves of two 16-row tiles
constexpr int kPrefillRows = 256;

// Decode launch plan: derived on the host from sizes only, so the workspace
// query and the launch agree.
struct DecodePlan {
  int G;            // query heads per KV head
  int apt;          // sequences of a group served by one row tile
  int row_tiles;    // row tiles per group (upper bound)
  int rp;           // rank padded to the MFMA k granule (16, 32, 64)
  int na;           // power-of-two bound on the sequences of one row tile (kernel variant)
  int split;        // tokens per split (multiple of kDecodeWaves * kWaveBlocks * kBlock)
  int nsplit;       // splits for the longest context
  int part_stride;  // floats per partial row record: 4 (m, l, seq, nact) + d
  size_t partial_bytes;
};

struct DecodeArgs {
  const void* q;
  const void* kb;
  const void* vb;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* group_offsets;
  const int32_t* agent_ids;
  const int32_t* act;  // per-sequence activation position, or NULL (0)
  const void* const* lk;
  const void* const* lv;
  const void* const* bk;
  const void* const* bv;
  const int32_t* ranks;
  void* out;
  float* partials;
  int32_t max_blocks;
  int32_t num_groups;
  int32_t S;
  int32_t Hq;
  int32_t Hkv;
  int32_t d;
  int32_t G;
  int32_t apt;
  int32_t row_tiles;
  int32_t split;
  int32_t nsplit;
  int32_t part_stride;
  int32_t n_work;  // num_groups * row_tiles * nsplit * Hkv
  float sm_scale;
  float sm_scale_log2;  // sm_scale * log2(e)
  int32_t rope;             // 1: rotate the adapter key term
  double rope_rev[kMaxRopePairs];  // theta^(-2i/d) / (2 pi): revolutions per position, pair i
};

constexpr int kMaxBuildGroups = 64;  // destination column groups of one cache build
constexpr int kMaxBuildCols = 512;   // columns of A in one cache build
constexpr int kBuildSlice = 512;     // hidden values summed by one cache-build workgroup
constexpr int kBuildCounterSlots = 1024;  // tile counters at the start of the cache-build workspace

// One cache build: L = X A, columns [group_col[g], group_col[g+1]) of the
// product going to destination g (a dense matrix or a paged pool).
struct BuildArgs {
  const uint16_t* X;
  const uint16_t* A;
  const int64_t* slot_mapping;
  int64_t ldx, lda;
  int32_t n_tokens, hidden, n_cols;
  int32_t row_tiles, col_tiles;
  int32_t n_groups;
  int32_t group_col[kMaxBuildGroups + 1];
  int32_t group_layout[kMaxBuildGroups];  // 0 token-major (row stride group_ld), 1 rank-major, 2 key-chunked
  int64_t group_ld[kMaxBuildGroups];
  void* group_dst[kMaxBuildGroups];
  int32_t ksplit;     // slices of the hidden dimension (ceil(hidden / kBuildSlice))
  int* counters;      // [kBuildCounterSlots] tile counters, zero between launches (ksplit > 1)
  float* partials;    // [tiles of a launch][ksplit][256] fp32 partial sums (ksplit > 1)
};

// Cache-build workspace: counters, then the partial sums of one launch.
size_t build_workspace_bytes(int n_tokens, int hidden, int n_cols);
int build_tiles_per_launch(int col_tiles);

struct PrefillArgs {
  const void* q;
  const void* kb;
  const void* vb;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  const int32_t* agent_ids;
  const int32_t* act;  // per-sequence activation position, or NULL (0)
  const void* const* lk;
  const void* const* lv;
  const void* const* bk;
  const void* const* bv;
  const int32_t* ranks;
  void* out;
  int32_t max_blocks;
  int32_t S;
  int32_t Hq;
  int32_t Hkv;
  int32_t d;
  int32_t G;
  int32_t max_q_len;
  int32_t q_tiles;  // query tiles per sequence
  int32_t rp;
  float sm_scale;
  float sm_scale_log2;
  int32_t rope;
  double rope_rev[kMaxRopePairs];
};

hipError_t launch_decode_bf16(const DecodeArgs& a, int rp, int na, hipStream_t stream);
bool launch_decode_bf16_kv(const DecodeArgs& a, int rp, int na, dim3 grid, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_lr_build_bf16(const BuildArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// prefill chunks, then decode rows, on one stream
hipError_t launch_varlen_bf16(const DecodeArgs& d, int rp, int na, const PrefillArgs& p, hipStream_t stream);

}  // namespace lra
