// Decode attention over a shared-base + low-rank KV cache, bf16 in, fp32
// accumulate, on gfx950 MFMA.
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
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace lra {
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
__device__ __forceinline__ bool decode_item(const DecodeArgs& a, int logical, WorkItem& w) {
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
  if (w.ns <= 0) return false;
  w.T = sload(a.context_lens + w.s_first);
  w.nact = (w.T + a.split - 1) / a.split;
  w.t_begin = w.c * a.split;
  w.t_end = min(w.T, w.t_begin + a.split);
  return true;
}

// Main kernel: one workgroup of kDecodeWaves waves per (group, row tile,
// split, KV head). NA is a compile-time bound on the agents of a row tile
// (a tile with fewer runs with zero B_k / L rows for the missing ones).
// KAD / VAD: the call has key / value adapters; without one, that part of
// the work (its low-rank loads, staging and products) is not compiled in.
// ACT: the call passes activation positions (without them no position test
// is compiled in).
// Writes the split's record (m, l, seq, nact, O' per row), or the finished
// rows when the context fits one split.
template <int RP, int NA, bool KAD, bool VAD, bool ACT>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_bf16_kernel(const DecodeArgs a) {
  constexpr int NRT = RP / 16;
  constexpr int KC = RP >= 32 ? RP / 32 : 1;
  constexpr int PW = D + (VAD ? RP : 0);  // floats per row of a merged state (O, then C)
  // LDS row pitch of the merge buffer: an odd multiple of 8 floats, so the 16
  // rows of a 16-byte access by one wave fall in distinct banks
  constexpr int PWP = PW + 8;
  static_assert((PWP / 8) % 2 == 1, "merge row pitch must be an odd multiple of 8 floats");
  constexpr int NT = kDecodeWaves * 64;
  constexpr int HW = kDecodeWaves / 2;
  constexpr int kBtBytes = KAD ? NA * D * RP * 2 : 0;
  constexpr int kMergeBytes = HW * 16 * PWP * 4;
  constexpr int kRegion = kBtBytes > kMergeBytes ? kBtBytes : kMergeBytes;
  static_assert(NA * RP <= 256, "staged B_k^T / B_v^T of a tile exceed their LDS budget");
  constexpr bool ADAPT = KAD || VAD;

  __shared__ __align__(16) unsigned char s_region[kRegion];  // B_k^T [al][dim][k] in the loop, merge buffer after
  __shared__ __align__(16) uint16_t s_bvt[VAD ? NA * D * RP : 8];          // B_v^T [al][dim][k]
  __shared__ __align__(16) uint16_t s_q[16 * kQPitch];                     // query tile [row][dim]
  __shared__ __align__(16) uint16_t s_qp[KAD ? 16 * kQpPitch : 8];         // f16 query tile, k slots of the adapter product
  __shared__ __align__(16) f16x2 s_roff[KAD ? 16 * kRotPitch : 4];         // (cos, sin) of lc theta_i, [lc][i]
  __shared__ __align__(16) f16x2 s_rbase[KAD ? kDecodeWaves : 1][kMaxRopePairs];  // per wave: (cos, sin) of tb theta_i
  __shared__ double s_rev[kMaxRopePairs];
  __shared__ TileAgent s_agent[NA];
  __shared__ float s_ml[2][HW][16];
  __shared__ int s_shared_l;
  __shared__ int s_lead;  // first agent slot of the tile with an adapter (its rows travel with the blocks)
  __shared__ int s_start_min, s_start_max;  // activation positions over the tile's adapted slots

  // ---- work item; consecutive logical items are dealt to one XCD ----
  const int per = (a.n_work + kNumXcd - 1) / kNumXcd;
  const int logical = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (logical >= a.n_work) return;
  WorkItem wi;
  if (!decode_item(a, logical, wi)) {
    // no sequences in this row tile: split 0 marks its rows empty for the combine
    if (a.nsplit > 1 && wi.c == 0 && threadIdx.x < 16)
      *reinterpret_cast<float4*>(a.partials + (((size_t)wi.tile_id * a.nsplit) * 16 + threadIdx.x) * a.part_stride) =
          make_float4(0.f, 0.f, __int_as_float(0), __int_as_float(0));
    return;
  }
  if (wi.c >= wi.nact) return;
  const int h = wi.h, c = wi.c, s0 = wi.s0, ns = wi.ns, t_begin = wi.t_begin, t_end = wi.t_end;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lc = lane & 15;  // accumulator column / operand row
  const int lg = lane >> 4;  // k-group
  const int G = a.G;
  const int HD = a.Hkv * D;
  const int* bt_row = a.block_tables + (size_t)wi.s_first * a.max_blocks;
  const int blk0 = t_begin / kBlock;
  const int nb = (t_end - t_begin + kBlock - 1) / kBlock;  // cache blocks of the split
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;

  // ---- loads of one block; a block past the split gets zero-length ranges
  // (its loads return zero and touch no memory) ----
  auto load_k = [&](Blk<RP>& B, int bi) __attribute__((always_inline)) {
    const bool ok = bi < nb;
    const int phys = sload(bt_row + blk0 + (ok ? bi : 0));
    const auto r = buf_rsrc((const uint16_t*)a.kb + (size_t)phys * blk_elems + (size_t)h * kBlock * D,
                            ok ? kBlock * D * 2 : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) B.kr[ks] = as_bf16x8(bld16(r, (lc * D + 8 * lg + 32 * ks) * 2));
  };
  // low-rank rows of a block are read only when some token of it is at or
  // past the tile's first activation position st_lo
  auto load_lv = [&](Blk<RP>& B, int bi, const uint16_t* lk0, const uint16_t* lv0, int r0, int st_lo)
                     __attribute__((always_inline)) {
    const bool ok = bi < nb;
    const bool lok = ok && (!ACT || t_begin + bi * kBlock + kBlock > st_lo);
    const int phys = sload(bt_row + blk0 + (ok ? bi : 0));
    if constexpr (KAD) {
      const auto rlk = buf_rsrc(lk0 + (size_t)phys * kBlock * r0, lok ? kBlock * r0 * 2 : 0);
      if constexpr (RP == 16) {
        B.lk16 = bld8(rlk, (4 * lg < r0) ? (lc * r0 + 4 * lg) * 2 : kOob);
      } else {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          B.lk32[kc] = as_bf16x8(bld16(rlk, (32 * kc + 8 * lg < r0) ? (lc * r0 + 32 * kc + 8 * lg) * 2 : kOob));
      }
    }
    if constexpr (VAD) {
      const auto rlv = buf_rsrc(lv0 + (size_t)phys * r0 * kBlock, lok ? r0 * kBlock * 2 : 0);
#pragma unroll
      for (int rr = 0; rr < NRT; ++rr)
        B.lv[rr] = bld8(rlv, (16 * rr + lc < r0) ? ((16 * rr + lc) * kBlock + 4 * lg) * 2 : kOob);
    }
    const auto rv = buf_rsrc((const uint16_t*)a.vb + (size_t)phys * blk_elems + (size_t)h * D * kBlock,
                             ok ? D * kBlock * 2 : 0);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) B.vr[cb] = bld8(rv, ((16 * cb + lc) * kBlock + 4 * lg) * 2);
  };

  // ---- (1) loads that need no agent information: the rotary table (kernel
  // arguments), the base keys of this wave's first block and the query
  // tile. No branches around these loads (a load inside a conditional block
  // gets a wait for every load in flight at the block's end); lanes without
  // data read zero through the range check. ----
  double rev_arg = 0.0;
  if (KAD && tid < kMaxRopePairs) rev_arg = a.rope_rev[tid];
  Blk<RP> bufA, bufB;
  load_k(bufA, wave);
  const int qrow = tid / (D / 8), qd8 = (tid % (D / 8)) * 8;
  const bool q_on = tid < 16 * (D / 8) && qrow / G < ns && qrow < a.apt * G;
  const uint4 stq = bld16(buf_rsrc((const uint16_t*)a.q + ((size_t)s0 * a.Hq + h * G) * D, ns * a.Hq * D * 2),
                          q_on ? (((qrow / G) * a.Hq + (qrow % G)) * D + qd8) * 2 : kOob);
  __builtin_amdgcn_sched_barrier(0);

  // ---- (2) agent table, from scalar loads only (which do not wait behind
  // the vector loads in flight). A sequence without an agent (id -1) gets
  // rank 0 and no pointers: its B rows stage as zero, so whatever low-rank
  // rows its slot is given contribute nothing. The lead is the first slot
  // with an adapter; its low-rank rows travel with the blocks, and the
  // tile's pools count as shared when every adapted slot reads the lead's. ----
  if (ADAPT && wave == 0) {
    // Two rounds of scalar loads in flight together (the agent ids, then every
    // table entry of every slot); scheduling barriers keep all uses after all
    // loads of a round. A slot past the tile or without an agent reads entry
    // 0 (an adapter call has at least one agent) and is masked afterwards.
    int ags[NA];
#pragma unroll
    for (int al = 0; al < NA; ++al) ags[al] = sload(a.agent_ids + s0 + min(al, ns - 1));
    __builtin_amdgcn_sched_barrier(0);
    const void* plk[NA];
    const void* pbk[NA];
    const void* plv[NA];
    const void* pbv[NA];
    int pr[NA], pst[NA];
#pragma unroll
    for (int al = 0; al < NA; ++al) {
      const int idx = max(ags[al], 0);
      plk[al] = KAD ? sload(a.lk + idx) : nullptr;
      pbk[al] = KAD ? sload(a.bk + idx) : nullptr;
      plv[al] = VAD ? sload(a.lv + idx) : nullptr;
      pbv[al] = VAD ? sload(a.bv + idx) : nullptr;
      pr[al] = sload(a.ranks + idx);
      pst[al] = ACT ? sload(a.act + s0 + min(al, ns - 1)) : 0;
    }
    // every loaded value is used here, after the last load, so none of the
    // loads moves into the branch of its slot below
#pragma unroll
    for (int al = 0; al < NA; ++al)
      asm volatile("" ::"s"(plk[al]), "s"(pbk[al]), "s"(plv[al]), "s"(pbv[al]), "s"(pr[al]), "s"(pst[al]));
    int sh = 1, lead = -1, st_min = 0x7fffffff, st_max = 0;
    const uint16_t *lk0 = nullptr, *lv0 = nullptr;
    int r0 = 0;
#pragma unroll
    for (int al = 0; al < NA; ++al) {
      const bool adapted = al < ns && ags[al] >= 0;
      TileAgent t{nullptr, nullptr, nullptr, nullptr, 0, s0 + al, 0};
      if (adapted) {
        t.lk = (const uint16_t*)plk[al];
        t.bk = (const uint16_t*)pbk[al];
        t.lv = (const uint16_t*)plv[al];
        t.bv = (const uint16_t*)pbv[al];
        t.r = pr[al];
        t.start = pst[al];
        st_min = min(st_min, t.start);
        st_max = max(st_max, t.start);
        if (lead < 0) {
          lead = al;
          lk0 = t.lk;
          lv0 = t.lv;
          r0 = t.r;
        } else {
          sh &= (t.lk == lk0) & (t.lv == lv0) & (t.r == r0);
        }
      }
      if (lane == 0) s_agent[al] = t;
    }
    if (lane == 0) {
      s_shared_l = sh;
      s_lead = lead < 0 ? 0 : lead;
      s_start_min = st_min;
      s_start_max = st_max;
    }
  }
  if (KAD && tid < kMaxRopePairs) s_rev[tid] = rev_arg;
  __syncthreads();

  // ---- (3) staging loads: B_k, B_v rows of head h per agent (branch-free,
  // as in step 1) ----
  constexpr int kItemsB = ADAPT ? NA * RP * (D / 8) : 0;  // 8-dim chunks of B_k (and of B_v)
  constexpr int kPerB = ADAPT ? (kItemsB + NT - 1) / NT : 1;
  static_assert(!ADAPT || (RP * (D / 8)) % 64 == 0, "one agent slot per wave and staging round");
  uint4 stk[kPerB], stv[kPerB];
#pragma unroll
  for (int i = 0; i < kPerB; ++i) {
    const int e = tid + i * NT;
    const int k = e % RP, d8 = ((e / RP) % (D / 8)) * 8;
    const int al = uniform((e / (RP * (D / 8))) % NA);  // the same for the whole wave
    const int ra = e < kItemsB ? uniform(s_agent[al].r) : 0;
    const int off = k < ra ? (k * HD + h * D + d8) * 2 : kOob;
    stk[i] = make_uint4(0, 0, 0, 0);
    stv[i] = make_uint4(0, 0, 0, 0);
    if constexpr (KAD) stk[i] = bld16(buf_rsrc(uniform_ptr(s_agent[al].bk), ra * HD * 2), off);
    if constexpr (VAD) stv[i] = bld16(buf_rsrc(uniform_ptr(s_agent[al].bv), ra * HD * 2), off);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- (4) the rest of the first block ----
  const int lead = ADAPT ? uniform(s_lead) : 0;
  const uint16_t* lk0 = ADAPT ? uniform_ptr(s_agent[lead].lk) : nullptr;
  const uint16_t* lv0 = ADAPT ? uniform_ptr(s_agent[lead].lv) : nullptr;
  const int r0 = ADAPT ? uniform(s_agent[lead].r) : 0;
  const int st_min = (ADAPT && ACT) ? uniform(s_start_min) : 0;  // blocks wholly before it skip the adapter work
  const int st_max = (ADAPT && ACT) ? uniform(s_start_max) : 0;  // blocks from it on need no per-row mask
  load_lv(bufA, wave, lk0, lv0, r0, st_min);

  // ---- (5) staged values into LDS: waits for the staging loads and what
  // was issued before them (the first block's keys), not for the loads of
  // step 4 ----
  uint16_t* s_bt = reinterpret_cast<uint16_t*>(s_region);
#pragma unroll
  for (int i = 0; i < kPerB; ++i) {
    const int e = tid + i * NT;
    if (e < kItemsB) {
      const int k = e % RP, d8 = ((e / RP) % (D / 8)) * 8, al = e / (RP * (D / 8));
      const uint16_t* pk = reinterpret_cast<const uint16_t*>(&stk[i]);
      const uint16_t* pv = reinterpret_cast<const uint16_t*>(&stv[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (KAD) s_bt[((size_t)al * D + d8 + j) * RP + k] = pk[j];
        if constexpr (VAD) s_bvt[((size_t)al * D + d8 + j) * RP + k] = pv[j];
      }
    }
  }
  if (tid < 16 * (D / 8)) {
    *reinterpret_cast<uint4*>(s_q + qrow * kQPitch + qd8) = stq;
  }
  if constexpr (KAD) {
    if (tid < 16 * (D / 8)) {
      // f16 copy in the k-slot order of the adapter product: for dim tile cb
      // and k-group g, slots 2j and 2j + 1 hold dims 16cb + 4g + j and + 64
      const uint16_t* pq = reinterpret_cast<const uint16_t*>(&stq);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = qd8 + j, dd = d & 63;
        const int slot = (dd >> 4) * 32 + ((dd >> 2) & 3) * 8 + 2 * (dd & 3) + (d >> 6);
        s_qp[qrow * kQpPitch + slot] = __builtin_bit_cast(uint16_t, (_Float16)bf16_to_f32(pq[j]));
      }
    }
    // per-column rotation table: entries (lc, i) for lc < 16, i < 64
    for (int e = tid; e < 16 * kMaxRopePairs; e += NT) {
      const int col = e / kMaxRopePairs, i = e % kMaxRopePairs;
      const float2 cs = cos_sin_rev((double)col * s_rev[i]);
      s_roff[col * kRotPitch + i] = f16x2{(_Float16)cs.x, (_Float16)cs.y};
    }
  }
  __syncthreads();

  const bool shared_l = s_shared_l != 0;
  const int row_al = lc / G;  // agent slot of this lane's query row
  const bool row_ok = row_al < ns && lc < a.apt * G;
  const int row_start = (ADAPT && ACT && row_al < NA) ? s_agent[row_al].start : 0;  // this row's activation position
  const uint16_t* qrow_p = s_q + lc * kQPitch;
  const uint16_t* qp_row = s_qp + lc * kQpPitch;
  const double rev_lane = KAD ? s_rev[lane] : 0.0;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
  f32x4 acl[NRT];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NRT; ++i) acl[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- one block: scores, online softmax, P V and P L_v ----
  // low-rank pools of agents 1 .. NA-1
  const uint16_t* ag_lk[NA];
  const uint16_t* ag_lv[NA];
  int ag_r[NA];
#pragma unroll
  for (int al = 0; al < NA; ++al) {
    ag_lk[al] = ADAPT ? uniform_ptr(s_agent[al].lk) : nullptr;
    ag_lv[al] = ADAPT ? uniform_ptr(s_agent[al].lv) : nullptr;
    ag_r[al] = ADAPT ? uniform(s_agent[al].r) : 0;
  }
  // per-agent low-rank rows of block bi (zero-length ranges past the split):
  // key rows (K) and value rows (V) separately
  auto load_agents = [&](AgentRows<RP, NA>& ar, int bi, bool keys, bool vals) __attribute__((always_inline)) {
    if (shared_l) return;  // every agent reads agent 0's rows, which travel with the block
    const bool ok = bi < nb && (!ACT || t_begin + bi * kBlock + kBlock > st_min);
    const int phys = sload(bt_row + blk0 + (ok ? bi : 0));
#pragma unroll
    for (int al = 1; al < NA; ++al) {
      const int ra = ag_r[al];
      if (KAD && keys) {
        const auto rl = buf_rsrc(ag_lk[al] + (size_t)phys * kBlock * ra, ok ? kBlock * ra * 2 : 0);
        if constexpr (RP == 16) {
          ar.lk16[al - 1] = bld8(rl, (4 * lg < ra) ? (lc * ra + 4 * lg) * 2 : kOob);
        } else {
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            ar.lk32[al - 1][kc] =
                as_bf16x8(bld16(rl, (32 * kc + 8 * lg < ra) ? (lc * ra + 32 * kc + 8 * lg) * 2 : kOob));
        }
      }
      if (VAD && vals) {
        const auto rv = buf_rsrc(ag_lv[al] + (size_t)phys * ra * kBlock, ok ? ra * kBlock * 2 : 0);
#pragma unroll
        for (int rr = 0; rr < NRT; ++rr)
          ar.lv[al - 1][rr] = bld8(rv, (16 * rr + lc < ra) ? ((16 * rr + lc) * kBlock + 4 * lg) * 2 : kOob);
      }
    }
  };

  // Other agents' rows are loaded one block ahead when they fit in 16
  // registers; larger ones are loaded at the start of the block's compute.
  constexpr int kAgentRegs = (KAD ? RP / 8 : 0) + (VAD ? RP / 8 : 0);  // per agent and block
  constexpr bool kAgentAhead = (NA - 1) * kAgentRegs <= 16;
  auto compute = [&](const Blk<RP>& B, const AgentRows<RP, NA>& ar_ahead, int bi) __attribute__((always_inline)) {
    AgentRows<RP, NA> ar_here;
    if constexpr (!kAgentAhead) load_agents(ar_here, bi, true, false);
    const AgentRows<RP, NA>& ar = kAgentAhead ? ar_ahead : ar_here;
    const int tb = t_begin + bi * kBlock;
    bool tv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) tv[jj] = (tb + 4 * lg + jj) < t_end;
    const uint32_t m01 = (tv[0] ? 0xFFFFu : 0u) | (tv[1] ? 0xFFFF0000u : 0u);
    const uint32_t m23 = (tv[2] ? 0xFFFFu : 0u) | (tv[3] ? 0xFFFF0000u : 0u);

    // base scores
    f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sb = mfma32(B.kr[ks], as_bf16x8(*reinterpret_cast<const uint4*>(qrow_p + 32 * ks + 8 * lg)), sb);
    // adapter scores: one accumulator per agent with the full query tile; each
    // row then takes its own agent's accumulator
    f32x4 sa[NA];
#pragma unroll
    for (int al = 0; al < NA; ++al) sa[al] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The rotation runs in packed f16: per pair, (u, w) = (x_i, x_i+64) goes to
    // (u c - w s, w c + u s) in two packed operations, and the rotated pair is
    // already the operand of the f16 adapter product (k slots paired as above).
    // SHARED: every agent's low-rank key rows are agent 0's (no copies, no
    // selects on loaded data in that path)
    auto adapter = [&](auto rope_tag, auto shared_tag) __attribute__((always_inline)) {
      constexpr bool ROPE = decltype(rope_tag)::value;
      constexpr bool SHARED = decltype(shared_tag)::value;
      if constexpr (ROPE) {
        // per-block part of the angles: pair `lane` at position tb
        const float2 cb_ = cos_sin_rev((double)tb * rev_lane);
        s_rbase[wave][lane] = f16x2{(_Float16)cb_.x, (_Float16)cb_.y};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
#pragma unroll 1
      for (int cb = 0; cb < 4; ++cb) {
        const f16x8 qa = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(qp_row + 32 * cb + 8 * lg));
        // angles of pairs 16cb + 4lg + jj at position tb + lc, by angle addition:
        // (cos, sin)(B + O) = (cB, sB) cO + (sB, cB) (-sO, sO)
        f16x2 c2[4], ns2[4];
        if constexpr (ROPE) {
          const uint4 pbv = *reinterpret_cast<const uint4*>(&s_rbase[wave][16 * cb + 4 * lg]);
          const uint4 pov = *reinterpret_cast<const uint4*>(s_roff + lc * kRotPitch + 16 * cb + 4 * lg);
          const uint32_t pbw[4] = {pbv.x, pbv.y, pbv.z, pbv.w};
          const uint32_t pow_[4] = {pov.x, pov.y, pov.z, pov.w};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f16x2 pb = __builtin_bit_cast(f16x2, pbw[jj]);
            const f16x2 po = __builtin_bit_cast(f16x2, pow_[jj]);
            const f16x2 cs = pb * f16x2{po.x, po.x} + f16x2{pb.y, pb.x} * f16x2{-po.y, po.y};
            c2[jj] = f16x2{cs.x, cs.x};
            ns2[jj] = f16x2{-cs.y, cs.y};
          }
        }
#pragma unroll
        for (int al = 0; al < NA; ++al) {
          const uint16_t* btp = s_bt + ((size_t)al * D + lc) * RP;
          f32x4 xl = f32x4{0.f, 0.f, 0.f, 0.f}, xh = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (RP == 16) {
            const uint2 al_ = *reinterpret_cast<const uint2*>(btp + 16 * cb * RP + 4 * lg);
            const uint2 ah_ = *reinterpret_cast<const uint2*>(btp + 16 * (cb + 4) * RP + 4 * lg);
            const uint2 lkop = (SHARED || al == 0) ? B.lk16 : ar.lk16[al > 0 ? al - 1 : 0];
            xl = mfma16(as_i16x4(al_), as_i16x4(lkop), xl);
            xh = mfma16(as_i16x4(ah_), as_i16x4(lkop), xh);
          } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              const uint4 al_ = *reinterpret_cast<const uint4*>(btp + 16 * cb * RP + 32 * kc + 8 * lg);
              const uint4 ah_ = *reinterpret_cast<const uint4*>(btp + 16 * (cb + 4) * RP + 32 * kc + 8 * lg);
              const bf16x8 lkop = (SHARED || al == 0) ? B.lk32[kc] : ar.lk32[al > 0 ? al - 1 : 0][kc];
              xl = mfma32(as_bf16x8(al_), lkop, xl);
              xh = mfma32(as_bf16x8(ah_), lkop, xh);
            }
          }
          f16x2 y[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f16x2 pr = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(xl[jj], xh[jj]));
            if constexpr (ROPE)
              y[jj] = pr * c2[jj] + f16x2{pr.y, pr.x} * ns2[jj];
            else
              y[jj] = pr;
          }
          const f16x8 yop = {y[0].x, y[0].y, y[1].x, y[1].y, y[2].x, y[2].y, y[3].x, y[3].y};
          sa[al] = mfma32h(yop, qa, sa[al]);
        }
      }
    };
    // Activation positions: a block wholly before every row's position skips
    // the adapter products; in a block that some row's position falls inside
    // or after, tokens before that row's position are masked out of its
    // adapter score and of its P L_v.
    const bool blk_ad = !ACT || tb + kBlock > st_min;
    // token jj of this lane carries adapter terms iff jj >= on_from (a block
    // from every row's position on masks nothing: no branch either way)
    const int on_from = (ACT && tb < st_max) ? row_start - tb - 4 * lg : -4;
    if constexpr (KAD) {
      if (blk_ad) {
        if (shared_l) {
          if (a.rope)
            adapter(std::true_type{}, std::true_type{});
          else
            adapter(std::false_type{}, std::true_type{});
        } else {
          if (a.rope)
            adapter(std::true_type{}, std::false_type{});
          else
            adapter(std::false_type{}, std::false_type{});
        }
      }
    }
    if constexpr (!kAgentAhead) load_agents(ar_here, bi, false, true);
    f32x4 sad = sa[0];
#pragma unroll
    for (int al = 1; al < NA; ++al)
      if (row_al == al) sad = sa[al];
    if constexpr (KAD) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sad[jj] = jj >= on_from ? sad[jj] : 0.f;
    }
    // online softmax over the block's 16 tokens (base-2 domain)
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      sv[jj] = tv[jj] ? (KAD ? sb[jj] + sad[jj] : sb[jj]) * a.sm_scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[jj]);
    }
    mx = wave_max_across_groups(mx);
    // The reference max moves only when the block exceeds it by more than
    // kMaxSlack (base 2), so most blocks need no rescale; probabilities stay
    // below 2^kMaxSlack and l, O and C share the reference. Every block holds
    // at least one valid token, so the first block always moves it.
    const float m_cand = fmaxf(m_run, mx);
    const bool move = m_cand > m_run + kMaxSlack;
    const float m_new = move ? m_cand : m_run;
    const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p[jj] = fast_exp2(sv[jj] - m_new);
      psum += p[jj];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      if constexpr (VAD) {
#pragma unroll
        for (int i = 0; i < NRT; ++i) acl[i] *= alpha;
      }
    }
    // P^T operand: k slots 0..3 = tokens 4lg + jj
    const uint2 pop = pack_bf16x4(p[0], p[1], p[2], p[3]);
    // NaN-safe: value rows of positions past the end are selected to zero
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      o[cb] = mfma16(as_i16x4(make_uint2(B.vr[cb].x & m01, B.vr[cb].y & m23)), as_i16x4(pop), o[cb]);
    // C^T += L_v^T P^T (per agent pool; rows of other agents masked out).
    // Blocks wholly before every activation position read zero L_v rows, so
    // the products add exact zeros there.
    if constexpr (VAD) {
      const uint2 popc =
          make_uint2(pop.x & ((0 >= on_from ? 0xFFFFu : 0u) | (1 >= on_from ? 0xFFFF0000u : 0u)),
                     pop.y & ((2 >= on_from ? 0xFFFFu : 0u) | (3 >= on_from ? 0xFFFF0000u : 0u)));
      if (shared_l) {
#pragma unroll
        for (int rr = 0; rr < NRT; ++rr)
          acl[rr] = mfma16(as_i16x4(make_uint2(B.lv[rr].x & m01, B.lv[rr].y & m23)), as_i16x4(popc), acl[rr]);
      } else {
#pragma unroll
        for (int al = 0; al < NA; ++al) {
          const uint2 pm = (row_ok && row_al == al) ? popc : make_uint2(0, 0);
#pragma unroll
          for (int rr = 0; rr < NRT; ++rr) {
            const uint2 lvr = al == 0 ? B.lv[rr] : ar.lv[al > 0 ? al - 1 : 0][rr];
            acl[rr] = mfma16(as_i16x4(make_uint2(lvr.x & m01, lvr.y & m23)), as_i16x4(pm), acl[rr]);
          }
        }
      }
    }
  };

  // ---- main loop over this wave's blocks wave, wave + 8, ...: per block,
  // first its other agents' rows, then the next block's rows, then the
  // compute. All loads are issued on every path (out-of-range ones read
  // nothing), so each wait covers exactly the loads issued before them. ----
  const int nmine = wave < nb ? (nb - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
  AgentRows<RP, NA> ar;
  for (int k = 0; k < nmine; k += 2) {
    const int bi = wave + k * kDecodeWaves;
    if constexpr (kAgentAhead) load_agents(ar, bi, true, true);
    load_k(bufB, bi + kDecodeWaves);
    load_lv(bufB, bi + kDecodeWaves, lk0, lv0, r0, st_min);
    __builtin_amdgcn_sched_barrier(0);  // nothing of the compute moves above these loads
    compute(bufA, ar, bi);
    if (k + 1 >= nmine) break;
    if constexpr (kAgentAhead) load_agents(ar, bi + kDecodeWaves, true, true);
    load_k(bufA, bi + 2 * kDecodeWaves);
    load_lv(bufA, bi + 2 * kDecodeWaves, lk0, lv0, r0, st_min);
    __builtin_amdgcn_sched_barrier(0);
    compute(bufB, ar, bi + kDecodeWaves);
  }

  // ---- merge the waves of this workgroup (two rounds through LDS) ----
  float l_row = wave_sum_across_groups(l_run);
  __syncthreads();  // B_k^T is dead from here on
  float* obuf = reinterpret_cast<float*>(s_region);  // [HW][16][PWP]
  if (wave >= HW) {
    const int slot = wave - HW;
    if (lg == 0) {
      s_ml[0][slot][lc] = m_run;
      s_ml[1][slot][lc] = l_row;
    }
    float* ob = obuf + ((size_t)slot * 16 + lc) * PWP;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) *reinterpret_cast<f32x4*>(ob + 16 * cb + 4 * lg) = o[cb];
    if constexpr (VAD) {
#pragma unroll
      for (int rr = 0; rr < NRT; ++rr) *reinterpret_cast<f32x4*>(ob + D + 16 * rr + 4 * lg) = acl[rr];
    }
  }
  __syncthreads();
  if (wave < HW) {
    const float m2 = s_ml[0][wave][lc], l2 = s_ml[1][wave][lc];
    const float mm = fmaxf(m_run, m2);
    const float w1 = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mm);
    const float w2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mm);
    float* ob = obuf + ((size_t)wave * 16 + lc) * PWP;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(ob + 16 * cb + 4 * lg);
      *reinterpret_cast<f32x4*>(ob + 16 * cb + 4 * lg) = w1 * o[cb] + w2 * v;
    }
    if constexpr (VAD) {
#pragma unroll
      for (int rr = 0; rr < NRT; ++rr) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(ob + D + 16 * rr + 4 * lg);
        *reinterpret_cast<f32x4*>(ob + D + 16 * rr + 4 * lg) = w1 * acl[rr] + w2 * v;
      }
    }
    if (lg == 0) {
      s_ml[0][wave][lc] = mm;
      s_ml[1][wave][lc] = w1 * l_row + w2 * l2;
    }
  }
  __syncthreads();

  // ---- final merge + value adapter: wave w owns dim tiles DTW w .. DTW w +
  // DTW - 1 (16 dims each) of all 16 rows ----
  constexpr int DTW = 8 / kDecodeWaves;
  float wts[HW];
  float M = -INFINITY, L = 0.f;
#pragma unroll
  for (int j = 0; j < HW; ++j) M = fmaxf(M, s_ml[0][j][lc]);
#pragma unroll
  for (int j = 0; j < HW; ++j) {
    const float mj = s_ml[0][j][lc];
    wts[j] = (mj == -INFINITY) ? 0.f : fast_exp2(mj - M);
    L += wts[j] * s_ml[1][j][lc];
  }
  // merged rank-space accumulator C of this lane's row, as bf16 hi + lo, per rank tile
  uint2 chi[NRT], clo[NRT];
#pragma unroll
  for (int rr = 0; rr < (VAD ? NRT : 0); ++rr) {
    f32x4 cm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < HW; ++j)
      cm += wts[j] * *reinterpret_cast<const f32x4*>(obuf + ((size_t)j * 16 + lc) * PWP + D + 16 * rr + 4 * lg);
    float hi[4], lo[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      hi[jj] = bf16_to_f32((uint16_t)(pack_bf16(cm[jj], 0.f) & 0xFFFFu));
      lo[jj] = cm[jj] - hi[jj];
    }
    chi[rr] = pack_bf16x4(hi[0], hi[1], hi[2], hi[3]);
    clo[rr] = pack_bf16x4(lo[0], lo[1], lo[2], lo[3]);
  }
  const bool used = lc < ns * G;
  const int seq = s0 + row_al;
  float* part = a.partials + (((size_t)wi.tile_id * a.nsplit + c) * 16 + lc) * a.part_stride;
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) {
    const int cbt = DTW * wave + dt;  // dim tile 16 cbt .. 16 cbt + 15
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < HW; ++j)
      acc += wts[j] * *reinterpret_cast<const f32x4*>(obuf + ((size_t)j * 16 + lc) * PWP + 16 * cbt + 4 * lg);
#pragma unroll
    for (int rr = 0; rr < (VAD ? NRT : 0); ++rr) {
#pragma unroll
      for (int al = 0; al < NA; ++al) {
        const bool mine = row_ok && row_al == al;
        const uint2 bvt =
            *reinterpret_cast<const uint2*>(s_bvt + ((size_t)al * D + 16 * cbt + lc) * RP + 16 * rr + 4 * lg);
        acc = mfma16(as_i16x4(bvt), as_i16x4(mine ? chi[rr] : make_uint2(0, 0)), acc);
        acc = mfma16(as_i16x4(bvt), as_i16x4(mine ? clo[rr] : make_uint2(0, 0)), acc);
      }
    }
    // this lane holds O'[row lc][dims 16 cbt + 4lg .. +3]
    if (wi.nact > 1) {
      if (used) *reinterpret_cast<f32x4*>(part + 4 + 16 * cbt + 4 * lg) = acc;
    } else if (used) {
      const float inv = 1.f / L;
      *reinterpret_cast<uint2*>((uint16_t*)a.out + ((size_t)seq * a.Hq + h * G + (lc % G)) * D + 16 * cbt + 4 * lg) =
          pack_bf16x4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
  }
  // record header (m, l, seq, nact) of this split; unused rows of split 0 are
  // marked empty (nact = 0), and a context that fits one split marks its
  // rows finished (nact = 1)
  if (wave == 0 && lg == 0) {
    if (wi.nact > 1) {
      if (used)
        *reinterpret_cast<float4*>(part) = make_float4(M, L, __int_as_float(seq), __int_as_float(wi.nact));
      else if (c == 0)
        *reinterpret_cast<float4*>(part) = make_float4(0.f, 0.f, __int_as_float(0), __int_as_float(0));
    } else if (a.nsplit > 1) {
      *reinterpret_cast<float4*>(part) = make_float4(0.f, 0.f, __int_as_float(0), __int_as_float(1));
    }
  }
}

// Combine kernel: one wave per (group, row tile, KV head, row) merges the
// split records of that row with weights 2^(m_c - M) and writes the output.
// The record of split 0 says how many splits the row has (0: no such row;
// 1: finished by the main kernel). Lanes 0..31 take the even splits, lanes
// 32..63 the odd ones, 4 output dims per lane; every load goes out at once
// and loads past the records read zero through the buffer range check.
__global__ __launch_bounds__(64) void decode_bf16_combine(const DecodeArgs a) {
  __shared__ float s_w[kMaxSplits];
  const int lane = threadIdx.x;
  const int gid = blockIdx.x;
  const int n_rows = a.num_groups * a.row_tiles * a.Hkv * 16;
  if (gid >= n_rows) return;
  const int tile_id = gid / 16, row = gid % 16;
  const int h = tile_id % a.Hkv;
  const int cstride = 16 * a.part_stride;  // floats from one split's record of this row to the next
  const float* pb = a.partials + ((size_t)tile_id * a.nsplit * 16 + row) * a.part_stride;
  const auto rs = buf_rsrc(pb, ((a.nsplit - 1) * cstride + a.part_stride) * 4);
  const uint4 hu = bld16(rs, lane < a.nsplit ? lane * cstride * 4 : kOob);
  const int half = lane >> 5, d4 = lane & 31;
  uint4 v[kMaxSplits / 2];
#pragma unroll
  for (int u = 0; u < kMaxSplits / 2; ++u) {
    const int c = 2 * u + half;
    v[u] = bld16(rs, c < a.nsplit ? (c * cstride + 4 + 4 * d4) * 4 : kOob);
  }
  const int nact = __builtin_amdgcn_readfirstlane((int)hu.w);
  const int seq = __builtin_amdgcn_readfirstlane((int)hu.z);
  if (nact <= 1) return;
  const bool okc = lane < nact;
  const float m_c = __uint_as_float(hu.x), l_c = __uint_as_float(hu.y);
  float M = okc ? m_c : -INFINITY;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float w = okc ? fast_exp2(m_c - M) : 0.f;
  float L = okc ? w * l_c : 0.f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  s_w[lane] = w;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMaxSplits / 2; ++u) {
    const int c = 2 * u + half;
    if (2 * u < nact) {  // uniform; records past nact are selected away, never multiplied
      const float wu = c < nact ? s_w[c] : 0.f;
      const uint32_t* vv = reinterpret_cast<const uint32_t*>(&v[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += c < nact ? wu * __uint_as_float(vv[i]) : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i]), __float_as_uint(acc[i]), false, false);
    acc[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (half == 0) {
    const float inv = 1.f / L;
    const uint2 ov = make_uint2(pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv));
    *reinterpret_cast<uint2*>((uint16_t*)a.out + ((size_t)seq * a.Hq + h * a.G + (row % a.G)) * D + 4 * d4) = ov;
  }
}

template <int RP, int NA, bool KAD, bool VAD>
void launch_main(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (a.act)
    hipLaunchKernelGGL((decode_bf16_kernel<RP, NA, KAD, VAD, true>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<RP, NA, KAD, VAD, false>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
}

template <bool KAD, bool VAD>
bool launch_variant(const DecodeArgs& a, int rp, int na, dim3 grid, hipStream_t stream) {
  switch (rp * 100 + na) {
    case 1601: launch_main<16, 1, KAD, VAD>(a, grid, stream); return true;
    case 1602: launch_main<16, 2, KAD, VAD>(a, grid, stream); return true;
    case 1604: launch_main<16, 4, KAD, VAD>(a, grid, stream); return true;
    case 1608: launch_main<16, 8, KAD, VAD>(a, grid, stream); return true;
    case 1616: launch_main<16, 16, KAD, VAD>(a, grid, stream); return true;
    case 3201: launch_main<32, 1, KAD, VAD>(a, grid, stream); return true;
    case 3202: launch_main<32, 2, KAD, VAD>(a, grid, stream); return true;
    case 3204: launch_main<32, 4, KAD, VAD>(a, grid, stream); return true;
    case 3208: launch_main<32, 8, KAD, VAD>(a, grid, stream); return true;
    case 6401: launch_main<64, 1, KAD, VAD>(a, grid, stream); return true;
    case 6402: launch_main<64, 2, KAD, VAD>(a, grid, stream); return true;
    case 6404: launch_main<64, 4, KAD, VAD>(a, grid, stream); return true;
    default: return false;
  }
}

}  // namespace

// The variants with both adapters are built in a translation unit of their
// own (this file compiled with LRA_DECODE_KV_PART), so the two halves of the
// variant set compile in parallel.
#ifdef LRA_DECODE_KV_PART
bool launch_decode_bf16_kv(const DecodeArgs& a, int rp, int na, dim3 grid, hipStream_t stream) {
  return launch_variant<true, true>(a, rp, na, grid, stream);
}
#else
hipError_t launch_decode_bf16(const DecodeArgs& a, int rp, int na, hipStream_t stream) {
  const int per = (a.n_work + kNumXcd - 1) / kNumXcd;
  const dim3 grid(per * kNumXcd);
  const int n_rows = a.num_groups * a.row_tiles * a.Hkv * 16;
  const bool kad = a.bk != nullptr, vad = a.bv != nullptr;
  bool launched;
  if (kad && vad)
    launched = launch_decode_bf16_kv(a, rp, na, grid, stream);
  else if (vad)
    launched = launch_variant<false, true>(a, rp, na, grid, stream);
  else if (kad)
    launched = launch_variant<true, false>(a, rp, na, grid, stream);
  else {  // no adapter: one variant serves every tile width (no per-agent state)
    hipLaunchKernelGGL((decode_bf16_kernel<16, 1, false, false, false>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
    launched = true;
  }
  if (!launched) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit <= 1) return e;
  hipLaunchKernelGGL(decode_bf16_combine, dim3(n_rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}
#endif

}  // namespace lra
