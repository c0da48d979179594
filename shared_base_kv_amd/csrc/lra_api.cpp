// C-ABI layer: host-side argument checks, launch plans and error reporting.
// Every check here runs before the first HIP call of an entry point, so the
// error paths can be exercised on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/lra.h"
#include "internal.h"

namespace lra {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return LRA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// max_rank 0 (a call without adapters) plans as rank 16.
int pad_rank(int max_rank) { return max_rank <= 16 ? 16 : (max_rank <= 32 ? 32 : 64); }

// Launch plan of the decode kernels; depends on host sizes only.
DecodePlan decode_plan(int S, int num_groups, int Hq, int Hkv, int d, int max_rank, int max_ctx, int dtype) {
  DecodePlan p{};
  p.G = Hq / Hkv;
  p.rp = pad_rank(max_rank);
  if (dtype == LRA_F32) {
    // fp32 kernel: one workgroup per (sequence, KV head), no split
    p.apt = 1;
    p.row_tiles = 1;
    p.split = max_ctx;
    p.nsplit = 1;
    p.part_stride = 0;
    p.partial_bytes = 0;
    return p;
  }
  p.apt = 16 / p.G;
  if (p.apt > 256 / p.rp) p.apt = 256 / p.rp;  // staged B_k^T of a tile fits 64 KB of LDS
  if (p.apt > kMaxTileAgents) p.apt = kMaxTileAgents;  // wider tiles would not fit the registers
  const int max_group = S - num_groups + 1;
  p.row_tiles = ceil_div(max_group, p.apt);
  p.na = 1;
  while (p.na < (max_group < p.apt ? max_group : p.apt)) p.na *= 2;
  const long long items = (long long)num_groups * p.row_tiles * Hkv;
  const int granule = kDecodeWaves * kWaveBlocks * kBlock;
  long long split = ((long long)max_ctx * items + kNumCU - 1) / kNumCU;
  split = (long long)round_up((size_t)split, granule);
  if (split < granule) split = granule;
  if (split > 4096) split = 4096;
  if (ceil_div(max_ctx, split) > kMaxSplits) split = (long long)round_up((size_t)ceil_div(max_ctx, kMaxSplits), granule);
  p.split = (int)split;
  p.nsplit = ceil_div(max_ctx, split);
  p.part_stride = 4 + d;  // [m, l, seq, nact, O'[d]] per row
  const size_t tiles = (size_t)num_groups * p.row_tiles * Hkv;
  p.partial_bytes = p.nsplit > 1 ? tiles * p.nsplit * 16 * (size_t)p.part_stride * sizeof(float) : 0;
  return p;
}

int check_decode_sizes(int S, int num_groups, int Hq, int Hkv, int d, int max_rank, int max_ctx, int dtype) {
  if (S < 0) return fail(LRA_ERR_INVALID_ARG, "S must be >= 0 (got %d)", S);
  if (Hq < 1 || Hkv < 1) return fail(LRA_ERR_INVALID_ARG, "Hq and Hkv must be >= 1 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv) return fail(LRA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(LRA_ERR_UNSUPPORTED, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
  if (Hkv > 65535) return fail(LRA_ERR_UNSUPPORTED, "at most 65535 KV heads (got %d)", Hkv);
  if (dtype != LRA_F32 && dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "dtype %d is not LRA_F32 or LRA_BF16", dtype);
  if (dtype == LRA_BF16 && d != 128) return fail(LRA_ERR_UNSUPPORTED, "bf16 kernels are built for d = 128 (got %d)", d);
  if (dtype == LRA_F32 && d != 64 && d != 128) return fail(LRA_ERR_UNSUPPORTED, "fp32 kernel supports d = 64 or 128 (got %d)", d);
  if (max_rank < 0 || max_rank > 64)
    return fail(LRA_ERR_UNSUPPORTED, "max_rank must be in 1..64, or 0 without adapters (got %d)", max_rank);
  if (max_ctx < 1) return fail(LRA_ERR_INVALID_ARG, "max_context_len must be >= 1 (got %d)", max_ctx);
  if (dtype == LRA_BF16 && max_ctx > kMaxSplits * kMaxSplitBlocks * kBlock)
    return fail(LRA_ERR_UNSUPPORTED, "bf16 decode supports contexts up to %d tokens (got %d)",
                kMaxSplits * kMaxSplitBlocks * kBlock, max_ctx);
  if (S > 0 && (num_groups < 1 || num_groups > S))
    return fail(LRA_ERR_INVALID_ARG, "num_groups must be in 1..S (got %d, S=%d)", num_groups, S);
  return LRA_OK;
}

// Adapter arguments: b_k (b_v) NULL means the call has no key (value)
// adapter and its low-rank pool table is not read; with neither, agent ids,
// ranks and N_agents are not read either and max_rank must be 0.
int check_adapters(const int32_t* agent_ids, const void* const* l_k_pools, const void* const* l_v_pools,
                   const void* const* b_k, const void* const* b_v, const int32_t* ranks, int max_rank, int N_agents) {
  if (!b_k && !b_v) {
    if (max_rank != 0) return fail(LRA_ERR_INVALID_ARG, "max_rank must be 0 when b_k and b_v are both NULL (got %d)", max_rank);
    return LRA_OK;
  }
  if (max_rank < 1) return fail(LRA_ERR_INVALID_ARG, "max_rank must be in 1..64 with an adapter (got %d)", max_rank);
  if (N_agents < 1) return fail(LRA_ERR_INVALID_ARG, "N_agents must be >= 1 (got %d)", N_agents);
  if (!agent_ids || !ranks) return fail(LRA_ERR_INVALID_ARG, "agent_ids and ranks must be non-null with an adapter");
  if (b_k && !l_k_pools) return fail(LRA_ERR_INVALID_ARG, "l_k_pools must be non-null when b_k is given");
  if (b_v && !l_v_pools) return fail(LRA_ERR_INVALID_ARG, "l_v_pools must be non-null when b_v is given");
  return LRA_OK;
}

#ifdef LRA_DEBUG_CHECKS
// Debug library only: the device-side data that the release library takes on
// trust is checked on the device before each attention launch (the stream is
// synchronised to read the result). The check kernel reads every table only
// at indices it has bounded first, so bad data yields an error code, never an
// access outside the caller's buffers.
struct CheckArgs {
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* group_offsets;  // NULL: every sequence is its own group
  const int32_t* cu_q_lens;      // NULL for decode
  const int32_t* dec_cu_q_lens;  // varlen decode part: cu_q_lens[s] must be s for s <= S (else NULL)
  const int32_t* agent_ids;      // NULL without adapters
  const int32_t* act;
  const int32_t* ranks;
  const void* const* lk;
  const void* const* lv;
  const void* const* bk;
  const void* const* bv;
  int32_t max_blocks, max_context_len, max_q_len, max_rank, S, num_groups, N_agents;
  int32_t dtype;  // element type of the call
};

// in the order of report priority (per-sequence checks before group checks)
enum : int {
  kChkContext = 1,
  kChkBlock,
  kChkAgent,
  kChkRank,
  kChkPool,
  kChkStart,
  kChkQLen,
  kChkDecodeRows,
  kChkGroups,
  kChkGroupShare,
};

const char* check_message(int code) {
  switch (code) {
    case kChkContext: return "context length outside 1..max_context_len";
    case kChkBlock: return "negative physical block id in a used block-table entry";
    case kChkAgent: return "agent id outside -1..N_agents-1";
    case kChkRank: return "agent rank outside 1..max_rank, or not a multiple of 8";
    case kChkPool: return "null low-rank pool or B pointer for an agent in use";
    case kChkStart: return "negative adapter_start";
    case kChkGroups: return "group_offsets do not rise strictly from 0 to S";
    case kChkGroupShare: return "sequences of one group differ in context length or block-table row";
    case kChkQLen: return "query count outside 0..min(max_q_len, context length)";
    case kChkDecodeRows: return "cu_q_lens[s] != s for a decode sequence s (or for s = S_dec)";
    default: return "unknown check";
  }
}

// the failing check of lowest code, then lowest index, as code << 24 | index
// (index: the sequence, or the group for the group checks); kNoFailure if none
constexpr int kNoFailure = 0x7fffffff;
__device__ int g_check;

__device__ void report(int code, int idx) { atomicMin(&g_check, code << 24 | min(idx, 0xffffff)); }

// one thread per sequence; thread s also checks group s
__global__ void check_inputs_kernel(const CheckArgs c) {
  const int s = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (s >= c.S) return;
  const int T = c.context_lens[s];
  if (T < 1 || T > c.max_context_len) return report(kChkContext, s);
  const int nb = min((T + kBlock - 1) / kBlock, c.max_blocks);
  for (int n = 0; n < nb; ++n)
    if (c.block_tables[(size_t)s * c.max_blocks + n] < 0) return report(kChkBlock, s);
  if (c.agent_ids) {
    const int ag = c.agent_ids[s];
    if (ag < -1 || ag >= c.N_agents) return report(kChkAgent, s);
    if (ag >= 0) {
      const int r = c.ranks[ag];
      if (r < 1 || r > c.max_rank || r % 8 != 0) return report(kChkRank, s);
      if ((c.bk && (!c.bk[ag] || !c.lk[ag])) || (c.bv && (!c.bv[ag] || !c.lv[ag]))) return report(kChkPool, s);
    }
    if (c.act && c.act[s] < 0) return report(kChkStart, s);
  }
  if (c.cu_q_lens) {
    const int ql = c.cu_q_lens[s + 1] - c.cu_q_lens[s];
    if (ql < 0 || ql > c.max_q_len || ql > T) return report(kChkQLen, s);
  }
  if (c.dec_cu_q_lens && (c.dec_cu_q_lens[s] != s || (s == c.S - 1 && c.dec_cu_q_lens[c.S] != c.S)))
    return report(kChkDecodeRows, s);
  if (c.group_offsets && s < c.num_groups) {
    const int g0 = c.group_offsets[s], g1 = c.group_offsets[s + 1];
    if (g0 < 0 || g1 <= g0 || g1 > c.S || (s == 0 && g0 != 0) || (s == c.num_groups - 1 && g1 != c.S))
      return report(kChkGroups, s);
    const int Tg = c.context_lens[g0];
    const int nbg = min((Tg + kBlock - 1) / kBlock, c.max_blocks);
    for (int i = g0 + 1; i < g1; ++i) {
      if (c.context_lens[i] != Tg) return report(kChkGroupShare, s);
      for (int n = 0; n < nbg; ++n)
        if (c.block_tables[(size_t)i * c.max_blocks + n] != c.block_tables[(size_t)g0 * c.max_blocks + n])
          return report(kChkGroupShare, s);
    }
  }
}

int debug_check(const CheckArgs& c, const char* name, hipStream_t stream) {
  if (c.S < 1) return LRA_OK;
  const int none = kNoFailure;
  int got = kNoFailure;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_check), &none, sizeof(none), 0, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(check_inputs_kernel, dim3((c.S + 255) / 256), dim3(256), 0, stream, c);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(&got, HIP_SYMBOL(g_check), sizeof(got), 0, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "%s: input check failed to run: %s", name, hipGetErrorString(e));
  if (got != kNoFailure)
    return fail(LRA_ERR_INVALID_ARG, "%s: %s (index %d)", name, check_message(got >> 24), got & 0xffffff);
  return LRA_OK;
}

// the cache-build workspace's tile counters must all be zero on entry
__global__ void check_build_counters_kernel(const int* counters, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n && counters[i] != 0) atomicMin(&g_check, i);
}

int debug_check_build(const int* counters, const char* name, hipStream_t stream) {
  if (!counters) return LRA_OK;
  const int none = kNoFailure;
  int got = kNoFailure;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_check), &none, sizeof(none), 0, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(check_build_counters_kernel, dim3((kBuildCounterSlots + 255) / 256), dim3(256), 0, stream,
                       counters, kBuildCounterSlots);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(&got, HIP_SYMBOL(g_check), sizeof(got), 0, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "%s: input check failed to run: %s", name, hipGetErrorString(e));
  if (got != kNoFailure)
    return fail(LRA_ERR_WORKSPACE, "%s: workspace tile counter %d is not zero (zero-fill the workspace before first use)",
                name, got);
  return LRA_OK;
}

CheckArgs decode_check_args(const DecodeArgs& a, int max_context_len, int max_rank, int N_agents, int dtype,
                            const int32_t* varlen_cu_q_lens = nullptr) {
  const bool adapted = a.bk || a.bv;
  return CheckArgs{a.block_tables, a.context_lens, a.group_offsets, nullptr, varlen_cu_q_lens,
                   adapted ? a.agent_ids : nullptr, a.act, a.ranks, a.lk, a.lv, a.bk, a.bv, a.max_blocks,
                   max_context_len, 0, max_rank, a.S, a.num_groups, N_agents, dtype};
}

CheckArgs prefill_check_args(const PrefillArgs& a, int max_context_len, int max_rank, int N_agents) {
  const bool adapted = a.bk || a.bv;
  return CheckArgs{a.block_tables, a.context_lens, nullptr, a.cu_q_lens, nullptr, adapted ? a.agent_ids : nullptr,
                   a.act, a.ranks, a.lk, a.lv, a.bk, a.bv, a.max_blocks, max_context_len, a.max_q_len, max_rank,
                   a.S, a.S, N_agents, LRA_BF16};
}
#endif

// Revolutions per position of rotary pair i: theta^(-2i/d) / (2 pi), in fp64.
void rope_table(double* out, float theta, int d) {
  for (int i = 0; i < kMaxRopePairs; ++i)
    out[i] = (theta > 0.f && i < d / 2) ? pow((double)theta, -2.0 * i / d) / (2.0 * M_PI) : 0.0;
}

}  // namespace
}  // namespace lra

using namespace lra;

extern "C" {

int lra_version(void) { return LRA_VERSION; }

const char* lra_last_error(void) { return g_err; }

// --------------------------------------------------------------------------
size_t lr_cache_build_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_cols) {
  if (n_tokens < 0 || hidden < 1 || n_cols < 1 || n_cols > kMaxBuildCols) return 0;
  return build_workspace_bytes(n_tokens, hidden, n_cols);
}

}  // extern "C"

namespace lra {
namespace {

// Checks shared by the cache builds, then the launch. The group table
// (columns, destinations, layouts, row strides) is already in `a`.
int launch_build(BuildArgs& a, const char* name, int32_t dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "%s supports LRA_BF16 only (got %d)", name, dtype);
  if (!a.X || !a.A) return fail(LRA_ERR_INVALID_ARG, "%s: X and A must be non-null", name);
  if (!aligned16(a.X) || a.ldx % 8) return fail(LRA_ERR_INVALID_ARG, "%s: X must be 16-byte aligned with ldx %% 8 == 0", name);
  if (a.ldx < a.hidden || a.lda < a.n_cols)
    return fail(LRA_ERR_INVALID_ARG, "%s: ldx (%lld) < hidden or lda (%lld) < n_cols", name, (long long)a.ldx,
                (long long)a.lda);
  if ((long long)a.hidden * a.lda * 2 > 0x7fffffffLL || (long long)16 * a.ldx * 2 > 0x7fffffffLL)
    return fail(LRA_ERR_UNSUPPORTED, "%s: A spans more than 2 GiB (hidden * lda), or 16 rows of X do (ldx)", name);
  a.row_tiles = ceil_div(a.n_tokens, 16);
  a.col_tiles = ceil_div(a.n_cols, 16);
  a.ksplit = ceil_div(a.hidden, kBuildSlice);
  const size_t need = build_workspace_bytes(a.n_tokens, a.hidden, a.n_cols);
  if (need && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(LRA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned, counters zero-filled) needed (got %zu)",
                name, need, workspace_bytes);
  a.counters = need ? (int*)workspace : nullptr;
  a.partials = need ? (float*)((char*)workspace + (size_t)kBuildCounterSlots * sizeof(int)) : nullptr;
#ifdef LRA_DEBUG_CHECKS
  const int rc = debug_check_build(a.counters, name, (hipStream_t)stream);
  if (rc != LRA_OK) return rc;
#endif
  const hipError_t e = launch_lr_build_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "%s launch failed: %s", name, hipGetErrorString(e));
  return ok();
}

int check_build_sizes(const char* name, int32_t n_tokens, int32_t hidden, int32_t n_cols) {
  if (n_tokens < 0 || hidden < 1 || n_cols < 1)
    return fail(LRA_ERR_INVALID_ARG, "%s: bad sizes n_tokens=%d hidden=%d n_cols=%d", name, n_tokens, hidden, n_cols);
  if (n_cols > kMaxBuildCols) return fail(LRA_ERR_UNSUPPORTED, "%s: n_cols must be <= %d (got %d)", name, kMaxBuildCols, n_cols);
  if (hidden % 8) return fail(LRA_ERR_UNSUPPORTED, "%s: hidden must be a multiple of 8 (got %d)", name, hidden);
  if ((long long)n_tokens * n_cols > (1LL << 30)) return fail(LRA_ERR_UNSUPPORTED, "%s: n_tokens * n_cols too large", name);
  return LRA_OK;
}

// Validation and arguments of the decode kernels (sizes already checked,
// S >= 1); shared by the decode call and the decode part of the varlen call.
int make_decode_args(DecodeArgs& a, DecodePlan& p, const void* q, const void* k_base, const void* v_base,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                     int32_t max_context_len, const int32_t* group_offsets, int32_t num_groups,
                     const int32_t* agent_ids, const int32_t* adapter_start, const void* const* l_k_pools,
                     const void* const* l_v_pools, const void* const* b_k, const void* const* b_v,
                     const int32_t* ranks, int32_t max_rank, int32_t S, int32_t N_agents, int32_t Hq, int32_t Hkv,
                     int32_t d, int32_t block_size, float sm_scale, float rope_theta, int32_t dtype, void* out,
                     void* workspace, size_t workspace_bytes, bool fixed_scratch = false) {
  if (block_size != kBlock) return fail(LRA_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", block_size);
  if (max_blocks < 1 || (long long)max_blocks * kBlock < max_context_len)
    return fail(LRA_ERR_INVALID_ARG, "max_blocks (%d) * 16 must cover max_context_len (%d)", max_blocks, max_context_len);
  if (!q || !k_base || !v_base || !block_tables || !context_lens || !out)
    return fail(LRA_ERR_INVALID_ARG, "a required pointer argument is null");
  int rc = check_adapters(agent_ids, l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, N_agents);
  if (rc != LRA_OK) return rc;
  if (!aligned16(q) || !aligned16(k_base) || !aligned16(v_base) || !aligned16(out))
    return fail(LRA_ERR_INVALID_ARG, "q, k_base, v_base and out must be 16-byte aligned");
  if (!isfinite(sm_scale) || !isfinite(rope_theta) || rope_theta < 0.f)
    return fail(LRA_ERR_INVALID_ARG, "sm_scale must be finite and rope_theta finite and >= 0");
  p = decode_plan(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype);
  const size_t need = p.partial_bytes;
  // fixed_scratch: the records go to the library's fixed array, whose
  // address the caller sets after these checks
  if (need && !fixed_scratch && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(LRA_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed (got %zu)", need, workspace_bytes);
  a.q = q;
  a.kb = k_base;
  a.vb = v_base;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.group_offsets = group_offsets;
  a.agent_ids = agent_ids;
  a.act = (b_k || b_v) ? adapter_start : nullptr;
  a.lk = l_k_pools;
  a.lv = l_v_pools;
  a.bk = b_k;
  a.bv = b_v;
  a.ranks = ranks;
  a.out = out;
  a.partials = need ? (float*)workspace : nullptr;
  a.max_blocks = max_blocks;
  a.num_groups = num_groups;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.G = p.G;
  a.apt = p.apt;
  a.row_tiles = p.row_tiles;
  a.split = p.split;
  a.nsplit = p.nsplit;
  a.part_stride = p.part_stride;
  a.n_work = num_groups * p.row_tiles * p.nsplit * Hkv;
  a.sm_scale = sm_scale;
  a.sm_scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.rope = rope_theta > 0.f;
  rope_table(a.rope_rev, rope_theta, d);
  return LRA_OK;
}

// ---- allocation-free decode: the split records live in a fixed device array ----
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends. In host code the array's name is not a device address: the
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is passed to the kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on the device of `stream` (taken on the first call
// for that device).
int scratch_of_stream(hipStream_t stream, void** out, const char* name) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "%s: no device for the stream: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LRA_ERR_UNSUPPORTED, "%s: device %d beyond %d", name, dev, kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      int cur = -1;
      e = hipGetDevice(&cur);
      if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
      void* q = nullptr;
      if (e == hipSuccess) e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (cur >= 0 && cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess || !q)
        return fail(LRA_ERR_LAUNCH, "%s: address of the fixed scratch on device %d: %s", name, dev,
                    hipGetErrorString(e));
      g_scratch[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return LRA_OK;
}

// The decode call, with a caller workspace or (noalloc) the fixed scratch.
int decode_call(const char* name, const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                const int32_t* group_offsets, int32_t num_groups, const int32_t* agent_ids,
                const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools,
                const void* const* b_k, const void* const* b_v, const int32_t* ranks, int32_t max_rank, int32_t S,
                int32_t N_agents, int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size, float sm_scale,
                float rope_theta, int32_t dtype, void* out, void* workspace, size_t workspace_bytes, bool noalloc,
                void* stream) {
  if (!group_offsets) num_groups = S;
  int rc = check_decode_sizes(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype);
  if (rc != LRA_OK) return rc;
  if (S == 0) return ok();
  if (noalloc) {
    // every host check first; the scratch address only once the call is valid
    const DecodePlan p = decode_plan(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype);
    if (p.partial_bytes > kNoAllocScratchBytes)
      return fail(LRA_ERR_UNSUPPORTED,
                  "%s: the split records of this call need %zu bytes, more than the fixed scratch of %zu bytes "
                  "(use lora_attn_decode with a workspace)",
                  name, p.partial_bytes, kNoAllocScratchBytes);
  }
  DecodeArgs a{};
  DecodePlan p{};
  rc = make_decode_args(a, p, q, k_base, v_base, block_tables, max_blocks, context_lens, max_context_len,
                        group_offsets, num_groups, agent_ids, adapter_start, l_k_pools, l_v_pools, b_k, b_v, ranks,
                        max_rank, S, N_agents, Hq, Hkv, d, block_size, sm_scale, rope_theta, dtype, out, workspace,
                        workspace_bytes, noalloc);
  if (rc != LRA_OK) return rc;
  if (noalloc && p.partial_bytes) {
    void* ptr = nullptr;
    rc = scratch_of_stream((hipStream_t)stream, &ptr, name);
    if (rc != LRA_OK) return rc;
    a.partials = (float*)ptr;
  }
#ifdef LRA_DEBUG_CHECKS
  rc = debug_check(decode_check_args(a, max_context_len, max_rank, N_agents, dtype), name, (hipStream_t)stream);
  if (rc != LRA_OK) return rc;
#endif
  const hipError_t e = dtype == LRA_BF16 ? launch_decode_bf16(a, p.rp, p.na, (hipStream_t)stream)
                                         : launch_decode_f32(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "%s launch failed: %s", name, hipGetErrorString(e));
  return ok();
}

// Validation and arguments of the prefill kernel (sizes already checked,
// S >= 1, bf16); shared by the prefill call and the prefill part of the
// varlen call.
int make_prefill_args(PrefillArgs& a, const void* q, const void* k_base, const void* v_base,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                      int32_t max_context_len, const int32_t* cu_q_lens, int32_t max_q_len, const int32_t* agent_ids,
                      const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools,
                      const void* const* b_k, const void* const* b_v, const int32_t* ranks, int32_t max_rank,
                      int32_t S, int32_t N_agents, int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                      float sm_scale, float rope_theta, void* out) {
  if (block_size != kBlock) return fail(LRA_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", block_size);
  if (max_q_len < 1 || max_q_len > max_context_len)
    return fail(LRA_ERR_INVALID_ARG, "max_q_len must be in 1..max_context_len (got %d)", max_q_len);
  if (max_blocks < 1 || (long long)max_blocks * kBlock < max_context_len)
    return fail(LRA_ERR_INVALID_ARG, "max_blocks (%d) * 16 must cover max_context_len (%d)", max_blocks, max_context_len);
  if (!q || !k_base || !v_base || !block_tables || !context_lens || !cu_q_lens || !out)
    return fail(LRA_ERR_INVALID_ARG, "a required pointer argument is null");
  int rc = check_adapters(agent_ids, l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, N_agents);
  if (rc != LRA_OK) return rc;
  if (!aligned16(q) || !aligned16(k_base) || !aligned16(v_base) || !aligned16(out))
    return fail(LRA_ERR_INVALID_ARG, "q, k_base, v_base and out must be 16-byte aligned");
  if (!isfinite(sm_scale) || !isfinite(rope_theta) || rope_theta < 0.f)
    return fail(LRA_ERR_INVALID_ARG, "sm_scale must be finite and rope_theta finite and >= 0");
  a.q = q;
  a.kb = k_base;
  a.vb = v_base;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_q_lens = cu_q_lens;
  a.agent_ids = agent_ids;
  a.act = (b_k || b_v) ? adapter_start : nullptr;
  a.lk = l_k_pools;
  a.lv = l_v_pools;
  a.bk = b_k;
  a.bv = b_v;
  a.ranks = ranks;
  a.out = out;
  a.max_blocks = max_blocks;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.G = Hq / Hkv;
  a.max_q_len = max_q_len;
  a.rp = pad_rank(max_rank);
  a.q_tiles = ceil_div(max_q_len, kPrefillRows / (Hq / Hkv));
  a.sm_scale = sm_scale;
  a.sm_scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.rope = rope_theta > 0.f;
  rope_table(a.rope_rev, rope_theta, d);
  return LRA_OK;
}

}  // namespace
}  // namespace lra

extern "C" {

int lr_cache_build(const void* X, int64_t ldx, const void* A, int64_t lda, void* L, int64_t ldl,
                   const int64_t* slot_mapping, int32_t l_layout, int32_t n_tokens, int32_t hidden,
                   int32_t n_cols, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "lr_cache_build supports LRA_BF16 only (got %d)", dtype);
  int rc = check_build_sizes("lr_cache_build", n_tokens, hidden, n_cols);
  if (rc != LRA_OK) return rc;
  if (n_tokens == 0) return ok();
  if (!L) return fail(LRA_ERR_INVALID_ARG, "lr_cache_build: L must be non-null");
  if (l_layout != LRA_L_TOKEN_MAJOR && l_layout != LRA_L_RANK_MAJOR && l_layout != LRA_L_KEY_CHUNKED)
    return fail(LRA_ERR_INVALID_ARG, "unknown l_layout %d", l_layout);
  if (!slot_mapping && l_layout != LRA_L_TOKEN_MAJOR)
    return fail(LRA_ERR_INVALID_ARG, "a dense store (no slot mapping) is token-major only");
  if (l_layout == LRA_L_KEY_CHUNKED && n_cols % 8)
    return fail(LRA_ERR_INVALID_ARG, "a key-chunked pool needs n_cols %% 8 == 0 (got %d)", n_cols);
  if (l_layout == LRA_L_TOKEN_MAJOR && ldl < n_cols)
    return fail(LRA_ERR_INVALID_ARG, "ldl (%lld) < n_cols (%d)", (long long)ldl, n_cols);
  BuildArgs a{};
  a.X = (const uint16_t*)X;
  a.A = (const uint16_t*)A;
  a.slot_mapping = slot_mapping;
  a.ldx = ldx;
  a.lda = lda;
  a.n_tokens = n_tokens;
  a.hidden = hidden;
  a.n_cols = n_cols;
  a.n_groups = 1;
  a.group_col[0] = 0;
  a.group_col[1] = n_cols;
  a.group_layout[0] = l_layout;
  a.group_ld[0] = ldl;
  a.group_dst[0] = L;
  return launch_build(a, "lr_cache_build", dtype, workspace, workspace_bytes, stream);
}

int lr_cache_build_multi(const void* X, int64_t ldx, const void* A, int64_t lda, int32_t n_groups,
                         const int32_t* group_cols, void* const* group_pools, const int32_t* group_layouts,
                         const int64_t* slot_mapping, int32_t n_tokens, int32_t hidden, int32_t n_cols,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "lr_cache_build_multi supports LRA_BF16 only (got %d)", dtype);
  int rc = check_build_sizes("lr_cache_build_multi", n_tokens, hidden, n_cols);
  if (rc != LRA_OK) return rc;
  if (n_groups < 1 || n_groups > kMaxBuildGroups)
    return fail(LRA_ERR_UNSUPPORTED, "n_groups must be in 1..%d (got %d)", kMaxBuildGroups, n_groups);
  if (!group_cols || !group_pools || !group_layouts)
    return fail(LRA_ERR_INVALID_ARG, "group_cols, group_pools and group_layouts must be non-null host arrays");
  if (group_cols[0] != 0 || group_cols[n_groups] != n_cols)
    return fail(LRA_ERR_INVALID_ARG, "group_cols must start at 0 and end at n_cols (%d)", n_cols);
  for (int g = 0; g < n_groups; ++g) {
    if (group_cols[g + 1] <= group_cols[g])
      return fail(LRA_ERR_INVALID_ARG, "group %d is empty or group_cols is not increasing", g);
    if (!group_pools[g]) return fail(LRA_ERR_INVALID_ARG, "group_pools[%d] is null", g);
    if (group_layouts[g] != LRA_L_TOKEN_MAJOR && group_layouts[g] != LRA_L_RANK_MAJOR &&
        group_layouts[g] != LRA_L_KEY_CHUNKED)
      return fail(LRA_ERR_INVALID_ARG, "group_layouts[%d] = %d is not a layout", g, group_layouts[g]);
    if (group_layouts[g] == LRA_L_KEY_CHUNKED && (group_cols[g + 1] - group_cols[g]) % 8)
      return fail(LRA_ERR_INVALID_ARG, "group %d: a key-chunked pool needs a width that is a multiple of 8", g);
  }
  if (!slot_mapping) return fail(LRA_ERR_INVALID_ARG, "lr_cache_build_multi needs a slot mapping");
  if (n_tokens == 0) return ok();
  BuildArgs a{};
  a.X = (const uint16_t*)X;
  a.A = (const uint16_t*)A;
  a.slot_mapping = slot_mapping;
  a.ldx = ldx;
  a.lda = lda;
  a.n_tokens = n_tokens;
  a.hidden = hidden;
  a.n_cols = n_cols;
  a.n_groups = n_groups;
  for (int g = 0; g <= n_groups; ++g) a.group_col[g] = group_cols[g];
  for (int g = 0; g < n_groups; ++g) {
    a.group_layout[g] = group_layouts[g];
    a.group_ld[g] = group_cols[g + 1] - group_cols[g];
    a.group_dst[g] = group_pools[g];
  }
  return launch_build(a, "lr_cache_build_multi", dtype, workspace, workspace_bytes, stream);
}

// --------------------------------------------------------------------------
size_t lora_attn_decode_workspace_size(int32_t S, int32_t num_groups, int32_t Hq, int32_t Hkv, int32_t d,
                                       int32_t max_rank, int32_t max_context_len, int32_t dtype) {
  if (S <= 0 || check_decode_sizes(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype) != LRA_OK) return 0;
  return decode_plan(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype).partial_bytes;
}

int lora_attn_decode(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                     int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                     const int32_t* group_offsets, int32_t num_groups, const int32_t* agent_ids,
                     const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools, const void* const* b_k,
                     const void* const* b_v, const int32_t* ranks, int32_t max_rank, int32_t S, int32_t N_agents,
                     int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size, float sm_scale, float rope_theta,
                     int32_t dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call("lora_attn_decode", q, k_base, v_base, block_tables, max_blocks, context_lens, max_context_len,
                     group_offsets, num_groups, agent_ids, adapter_start, l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank,
                     S, N_agents, Hq, Hkv, d, block_size, sm_scale, rope_theta, dtype, out, workspace, workspace_bytes,
                     false, stream);
}

int lora_attn_decode_noalloc(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                             const int32_t* group_offsets, int32_t num_groups, const int32_t* agent_ids,
                             const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools,
                             const void* const* b_k, const void* const* b_v, const int32_t* ranks, int32_t max_rank,
                             int32_t S, int32_t N_agents, int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                             float sm_scale, float rope_theta, int32_t dtype, void* out, void* stream) {
  return decode_call("lora_attn_decode_noalloc", q, k_base, v_base, block_tables, max_blocks, context_lens,
                     max_context_len, group_offsets, num_groups, agent_ids, adapter_start, l_k_pools, l_v_pools, b_k,
                     b_v, ranks, max_rank, S, N_agents, Hq, Hkv, d, block_size, sm_scale, rope_theta, dtype, out, nullptr,
                     0, true, stream);
}

// --------------------------------------------------------------------------
size_t lora_attn_prefill_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t max_rank,
                                        int32_t max_q_len, int32_t max_context_len, int32_t dtype) {
  (void)S; (void)Hq; (void)Hkv; (void)d; (void)max_rank; (void)max_q_len; (void)max_context_len; (void)dtype;
  return 0;
}

int lora_attn_prefill(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                      int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                      const int32_t* cu_q_lens, int32_t max_q_len, const int32_t* agent_ids,
                      const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools, const void* const* b_k,
                      const void* const* b_v, const int32_t* ranks, int32_t max_rank, int32_t S, int32_t N_agents,
                      int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size, float sm_scale, float rope_theta,
                      int32_t dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_decode_sizes(S, S > 0 ? S : 1, Hq, Hkv, d, max_rank, max_context_len, dtype);
  if (rc != LRA_OK) return rc;
  if (dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "prefill supports LRA_BF16 only");
  if (S == 0) return ok();
  (void)workspace;
  (void)workspace_bytes;
  PrefillArgs a{};
  rc = make_prefill_args(a, q, k_base, v_base, block_tables, max_blocks, context_lens, max_context_len, cu_q_lens,
                         max_q_len, agent_ids, adapter_start, l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, S,
                         N_agents, Hq, Hkv, d, block_size, sm_scale, rope_theta, out);
  if (rc != LRA_OK) return rc;
#ifdef LRA_DEBUG_CHECKS
  rc = debug_check(prefill_check_args(a, max_context_len, max_rank, N_agents), "lora_attn_prefill", (hipStream_t)stream);
  if (rc != LRA_OK) return rc;
#endif
  const hipError_t e = launch_prefill_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "lora_attn_prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

// --------------------------------------------------------------------------
size_t lora_attn_varlen_workspace_size(int32_t S, int32_t S_dec, int32_t num_groups, int32_t Hq, int32_t Hkv, int32_t d,
                                       int32_t max_rank, int32_t max_context_len, int32_t dtype) {
  if (S_dec < 0 || S_dec > S || dtype != LRA_BF16) return 0;
  return lora_attn_decode_workspace_size(S_dec, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype);
}

int lora_attn_varlen(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                     int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len, const int32_t* cu_q_lens,
                     int32_t max_q_len, int32_t S, int32_t S_dec, const int32_t* group_offsets, int32_t num_groups,
                     const int32_t* agent_ids, const int32_t* adapter_start, const void* const* l_k_pools,
                     const void* const* l_v_pools, const void* const* b_k, const void* const* b_v, const int32_t* ranks,
                     int32_t max_rank, int32_t N_agents, int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                     float sm_scale, float rope_theta, int32_t dtype, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (S < 0 || S_dec < 0 || S_dec > S)
    return fail(LRA_ERR_INVALID_ARG, "need 0 <= S_dec <= S (got S = %d, S_dec = %d)", S, S_dec);
  if (!group_offsets) num_groups = S_dec;
  int rc = check_decode_sizes(S, S_dec > 0 ? num_groups : 1, Hq, Hkv, d, max_rank, max_context_len, dtype);
  if (rc != LRA_OK) return rc;
  if (dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "lora_attn_varlen supports LRA_BF16 only");
  if (S_dec > 0 && (num_groups < 1 || num_groups > S_dec))
    return fail(LRA_ERR_INVALID_ARG, "num_groups must be in 1..S_dec (got %d)", num_groups);
  if (S == 0) return ok();
  const int S_pre = S - S_dec;
  DecodeArgs da{};
  DecodePlan dp{};
  if (S_dec > 0) {
    rc = make_decode_args(da, dp, q, k_base, v_base, block_tables, max_blocks, context_lens, max_context_len,
                          group_offsets, num_groups, agent_ids, adapter_start, l_k_pools, l_v_pools, b_k, b_v, ranks,
                          max_rank, S_dec, N_agents, Hq, Hkv, d, block_size, sm_scale, rope_theta, dtype, out,
                          workspace, workspace_bytes);
    if (rc != LRA_OK) return rc;
  } else {
    dp.rp = pad_rank(max_rank);
    dp.na = 1;
    da.bk = b_k;
    da.bv = b_v;
  }
  PrefillArgs pa{};
  if (S_pre > 0) {
    // the prefill part: sequences S_dec .. S - 1 (their per-sequence tables
    // offset accordingly); cu_q_lens keeps absolute query row offsets
    if (!block_tables || !context_lens || !cu_q_lens)
      return fail(LRA_ERR_INVALID_ARG, "a required pointer argument is null");
    rc = make_prefill_args(pa, q, k_base, v_base, block_tables + (size_t)S_dec * max_blocks, max_blocks,
                           context_lens + S_dec, max_context_len, cu_q_lens + S_dec, max_q_len,
                           agent_ids ? agent_ids + S_dec : nullptr, adapter_start ? adapter_start + S_dec : nullptr,
                           l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, S_pre, N_agents, Hq, Hkv, d, block_size,
                           sm_scale, rope_theta, out);
    if (rc != LRA_OK) return rc;
  }
#ifdef LRA_DEBUG_CHECKS
  if (S_dec > 0) {
    rc = debug_check(decode_check_args(da, max_context_len, max_rank, N_agents, dtype, cu_q_lens),
                     "lora_attn_varlen (decode part)", (hipStream_t)stream);
    if (rc != LRA_OK) return rc;
  }
  if (S_pre > 0) {
    rc = debug_check(prefill_check_args(pa, max_context_len, max_rank, N_agents), "lora_attn_varlen (prefill part)",
                     (hipStream_t)stream);
    if (rc != LRA_OK) return rc;
  }
#endif
  const hipError_t e = launch_varlen_bf16(da, dp.rp, dp.na, pa, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LRA_ERR_LAUNCH, "lora_attn_varlen launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
