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
// tile holds up to 16 query rows (apt sequences x G query heads of head h),
// so the base K/V of a block is read once for all agents of the tile. A
// split is a contiguous token range; its 4 waves take interleaved 32-token
// steps and keep independent online-softmax states, merged in LDS at the
// end. Each wave loads step i+1 while it computes step i. Splits of one
// (g, rt, h) meet in the last-arriving workgroup, which merges their partial
// states and finishes the rows (adds (P L_v) B_v, divides by the softmax
// sum, rounds to bf16).
//
// Matrix-core mapping (16x16 MFMA tiles, tokens on the M side):
//   S^T[token, row]   = K_base[token, :] Q^T            (16x16x32)
//                     + sum_a Y_a[token, :] Qmask_a^T    (16x16x32, Y_a = rotated rebuild)
//   X_a^T[dim, token] = B_k,a^T[dim, :] L_k^T[:, token]  (16x16x16 or 16x16x32 over rank)
//   O^T[dim, row]    += V^T[dim, token] P^T[token, row]  (16x16x32 over two blocks)
//   C^T[rank, row]   += L_v^T[rank, token] P^T[token, row]
// The accumulator layout of one product is the operand layout of the next,
// so rebuilt keys and probabilities never leave registers.
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int D = 128;
constexpr int kLdsMain = 65536;

struct TileAgent {
  const uint16_t* lk;
  const uint16_t* lv;
  const uint16_t* bk;
  const uint16_t* bv;
  int r;
  int seq;
};

// Registers of one 32-token step of one wave: base K rows, V^T rows and the
// low-rank rows of the tile's first agent (every agent's, when shared).
template <int RP>
struct Step {
  static constexpr int KC = RP >= 32 ? RP / 32 : 1;
  static constexpr bool kLv = RP <= 32;  // at rank 64 L_v rows are read at use (register budget)
  bf16x8 kr[2][4];
  uint2 vr[2][8];
  uint2 lk16[2];
  bf16x8 lk32[2][KC];
  uint2 lv[2][kLv ? RP / 16 : 1];
  int tb;
  int nblk;
  int phys[2];
};

// Loads of one step. Each (block, head) chunk of the pools gets its own
// buffer resource; lanes whose rank slot is past the agent's rank read zero.
template <int RP>
__device__ __forceinline__ void load_step_k(Step<RP>& s, const DecodeArgs& a, int tb, int t_end, int p0, int p1,
                                            int h, int lc, int lg) {
  s.tb = tb;
  s.nblk = (t_end - tb) > kBlock ? 2 : 1;
  s.phys[0] = uniform(p0);
  s.phys[1] = uniform(s.nblk > 1 ? p1 : p0);
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b < s.nblk) {
      const auto r = buf_rsrc((const uint16_t*)a.kb + (size_t)s.phys[b] * blk_elems + (size_t)h * kBlock * D,
                              kBlock * D * 2);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s.kr[b][ks] = as_bf16x8(bld16(r, (lc * D + 8 * lg + 32 * ks) * 2));
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s.kr[b][ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
}

// Values are issued after keys and low-rank rows: loads complete in issue
// order, so the scores of a step can start before its values arrive.
template <int RP>
__device__ __forceinline__ void load_step_v(Step<RP>& s, const DecodeArgs& a, int h, int lc, int lg) {
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b < s.nblk) {
      const auto r = buf_rsrc((const uint16_t*)a.vb + (size_t)s.phys[b] * blk_elems + (size_t)h * D * kBlock,
                              kBlock * D * 2);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) s.vr[b][cb] = bld8(r, ((16 * cb + lc) * kBlock + 4 * lg) * 2);
    } else {
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) s.vr[b][cb] = make_uint2(0, 0);
    }
  }
}

// Low-rank key operand of block b for one agent: L_k[token lc][rank slots].
template <int RP>
__device__ __forceinline__ void load_lk(const TileAgent& ag, int phys, int lc, int lg, uint2& lk16,
                                        bf16x8 (&lk32)[RP >= 32 ? RP / 32 : 1]) {
  const auto r = buf_rsrc(ag.lk + (size_t)phys * kBlock * ag.r, kBlock * ag.r * 2);
  if constexpr (RP == 16) {
    lk16 = bld8(r, (4 * lg < ag.r) ? (lc * ag.r + 4 * lg) * 2 : kOob);
  } else {
#pragma unroll
    for (int kc = 0; kc < RP / 32; ++kc)
      lk32[kc] = as_bf16x8(bld16(r, (32 * kc + 8 * lg < ag.r) ? (lc * ag.r + 32 * kc + 8 * lg) * 2 : kOob));
  }
}

// Low-rank value operand of block b, rank tile rr: L_v[rank 16rr + lc][tokens 4lg..].
__device__ __forceinline__ uint2 load_lv(const TileAgent& ag, int phys, int rr, int lc, int lg) {
  const auto r = buf_rsrc(ag.lv + (size_t)phys * ag.r * kBlock, ag.r * kBlock * 2);
  const int rank = 16 * rr + lc;
  return bld8(r, rank < ag.r ? (rank * kBlock + 4 * lg) * 2 : kOob);
}

template <int RP>
__device__ __forceinline__ void load_step_l(Step<RP>& s, const TileAgent& ag0, int lc, int lg) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b < s.nblk) {
      load_lk<RP>(ag0, s.phys[b], lc, lg, s.lk16[b], s.lk32[b]);
      if constexpr (Step<RP>::kLv) {
#pragma unroll
        for (int rr = 0; rr < RP / 16; ++rr) s.lv[b][rr] = load_lv(ag0, s.phys[b], rr, lc, lg);
      }
    } else {
      s.lk16[b] = make_uint2(0, 0);
#pragma unroll
      for (int kc = 0; kc < Step<RP>::KC; ++kc) s.lk32[b][kc] = as_bf16x8(make_uint4(0, 0, 0, 0));
      if constexpr (Step<RP>::kLv) {
#pragma unroll
        for (int rr = 0; rr < RP / 16; ++rr) s.lv[b][rr] = make_uint2(0, 0);
      }
    }
  }
}

constexpr int kQPitch = D + 8;  // LDS row pitch of the query tile (bf16), breaks bank aliasing

struct Frame {  // per-lane constants of the main loop
  const uint16_t* q;    // LDS query tile [16][kQPitch], this lane's row
  const double* rev;    // LDS table: rotary revolutions per position of pair i
  int row_al;           // sequence (agent slot) of this lane's query row
  bool row_ok;
};

// S^T of one 16-token block: base part plus every agent's rebuilt adapter
// part. The loop runs over rotation pairs (dim blocks cb, cb + 4) outside and
// agents inside, so only one pair's cos/sin is live at a time.
template <int RP>
__device__ __forceinline__ f32x4 block_scores(const Step<RP>& s, const int b, const DecodeArgs& a, const Frame& fr,
                                              const TileAgent* s_agent, const uint16_t* s_bt, int ns, bool shared_l,
                                              int lc, int lg) {
  const bf16x8 zero8 = as_bf16x8(make_uint4(0, 0, 0, 0));
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 qb = as_bf16x8(*reinterpret_cast<const uint4*>(fr.q + 32 * ks + 8 * lg));
    sacc = mfma32(s.kr[b][ks], qb, sacc);
  }
  const double pd = (double)(s.tb + 16 * b + lc);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    float cs[4], sn[4];
    if (a.rope) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const double x = pd * fr.rev[16 * cb + 4 * lg + jj];
        const float f = (float)(x - __builtin_floor(x));
        cs[jj] = __builtin_amdgcn_cosf(f);
        sn[jj] = __builtin_amdgcn_sinf(f);
      }
    }
    const bf16x8 qa = cat8(*reinterpret_cast<const uint2*>(fr.q + 16 * cb + 4 * lg),
                           *reinterpret_cast<const uint2*>(fr.q + 64 + 16 * cb + 4 * lg));
    for (int al = 0; al < ns; ++al) {
      const TileAgent& ag = s_agent[al];
      f32x4 xl = f32x4{0.f, 0.f, 0.f, 0.f}, xh = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* btp = s_bt + ((size_t)al * D + lc) * RP;
      const bool own = al == 0 || shared_l;  // low-rank rows already in registers
      uint2 lko16 = s.lk16[b];
      bf16x8 lko32[Step<RP>::KC];
#pragma unroll
      for (int kc = 0; kc < Step<RP>::KC; ++kc) lko32[kc] = s.lk32[b][kc];
      if (!own) load_lk<RP>(ag, s.phys[b], lc, lg, lko16, lko32);
      if constexpr (RP == 16) {
        const uint2 lk = lko16;
        const uint2 al_ = *reinterpret_cast<const uint2*>(btp + (size_t)16 * cb * RP + 4 * lg);
        const uint2 ah_ = *reinterpret_cast<const uint2*>(btp + (size_t)16 * (cb + 4) * RP + 4 * lg);
        xl = mfma16(as_i16x4(al_), as_i16x4(lk), xl);
        xh = mfma16(as_i16x4(ah_), as_i16x4(lk), xh);
      } else {
#pragma unroll
        for (int kc = 0; kc < RP / 32; ++kc) {
          const bf16x8 lk = lko32[kc];
          const uint4 al_ = *reinterpret_cast<const uint4*>(btp + (size_t)16 * cb * RP + 32 * kc + 8 * lg);
          const uint4 ah_ = *reinterpret_cast<const uint4*>(btp + (size_t)16 * (cb + 4) * RP + 32 * kc + 8 * lg);
          xl = mfma32(as_bf16x8(al_), lk, xl);
          xh = mfma32(as_bf16x8(ah_), lk, xh);
        }
      }
      float y1[4], y2[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (a.rope) {
          y1[jj] = xl[jj] * cs[jj] - xh[jj] * sn[jj];
          y2[jj] = xh[jj] * cs[jj] + xl[jj] * sn[jj];
        } else {
          y1[jj] = xl[jj];
          y2[jj] = xh[jj];
        }
      }
      const bf16x8 yop = cat8(pack_bf16x4(y1[0], y1[1], y1[2], y1[3]), pack_bf16x4(y2[0], y2[1], y2[2], y2[3]));
      const bool mine = fr.row_ok && (fr.row_al == al);
      sacc = mfma32(yop, mine ? qa : zero8, sacc);
    }
  }
  return sacc;
}

template <int RP>
__device__ __forceinline__ void compute_step(const Step<RP>& s, const DecodeArgs& a, const Frame& fr,
                                             const TileAgent* s_agent, const uint16_t* s_bt, int ns, bool shared_l,
                                             int t_end, int lc, int lg, float& m_run, float& l_run, f32x4 (&o)[8],
                                             f32x4 (&acl)[RP / 16]) {
  constexpr int NRT = RP / 16;
  const int tb = s.tb;
  // token validity of this lane's slots: token tb + 16b + 4lg + jj
  bool tv[2][4];
  uint32_t m01[2], m23[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) tv[b][jj] = (tb + 16 * b + 4 * lg + jj) < t_end;
    m01[b] = (tv[b][0] ? 0xFFFFu : 0u) | (tv[b][1] ? 0xFFFF0000u : 0u);
    m23[b] = (tv[b][2] ? 0xFFFFu : 0u) | (tv[b][3] ? 0xFFFF0000u : 0u);
  }
  const bf16x8 zero8 = as_bf16x8(make_uint4(0, 0, 0, 0));

  // ---- scores S^T, one block after the other ----
  f32x4 sacc[2];
  sacc[0] = block_scores<RP>(s, 0, a, fr, s_agent, s_bt, ns, shared_l, lc, lg);
  sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (s.nblk > 1) sacc[1] = block_scores<RP>(s, 1, a, fr, s_agent, s_bt, ns, shared_l, lc, lg);

  // ---- online softmax over this step's 32 tokens (base-2 domain) ----
  float sv[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      sv[b][jj] = tv[b][jj] ? sacc[b][jj] * a.sm_scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[b][jj]);
    }
  mx = wave_max_across_groups(mx);
  const float m_new = fmaxf(m_run, mx);
  const float alpha = fast_exp2(m_run - m_new);
  float p[2][4];
  float psum = 0.f;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p[b][jj] = fast_exp2(sv[b][jj] - m_new);
      psum += p[b][jj];
    }
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
  for (int i = 0; i < NRT; ++i) acl[i] *= alpha;

  // P^T operand: slots 0..3 = block 0 tokens 4lg+jj, slots 4..7 = block 1
  const bf16x8 pop = cat8(pack_bf16x4(p[0][0], p[0][1], p[0][2], p[0][3]), pack_bf16x4(p[1][0], p[1][1], p[1][2], p[1][3]));
  // NaN-safe: value rows of positions past the end are selected to zero
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const uint2 v0 = make_uint2(s.vr[0][cb].x & m01[0], s.vr[0][cb].y & m23[0]);
    const uint2 v1 = make_uint2(s.vr[1][cb].x & m01[1], s.vr[1][cb].y & m23[1]);
    o[cb] = mfma32(cat8(v0, v1), pop, o[cb]);
  }

  // C^T += L_v^T P^T (per agent pool; rows of other agents masked out)
  for (int al = 0; al < ns; ++al) {
    if (shared_l && al > 0) break;
    const TileAgent& ag = s_agent[al];
    const bf16x8 pm = (shared_l || (fr.row_ok && fr.row_al == al)) ? pop : zero8;
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr) {
      uint2 lvr[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (Step<RP>::kLv && al == 0) {
          lvr[b] = s.lv[b][Step<RP>::kLv ? rr : 0];
        } else {
          lvr[b] = b < s.nblk ? load_lv(ag, s.phys[b], rr, lc, lg) : make_uint2(0, 0);
        }
        lvr[b].x &= m01[b];
        lvr[b].y &= m23[b];
      }
      acl[rr] = mfma32(cat8(lvr[0], lvr[1]), pm, acl[rr]);
    }
  }
}

struct WorkItem {
  int g, rt, h, c, s_first, s0, ns, T, nact, t_begin, t_end, tile_id;
};

__device__ __forceinline__ bool decode_item(const DecodeArgs& a, int logical, bool by_head, WorkItem& w) {
  int rem = logical;
  if (by_head) {
    w.c = rem % a.nsplit;
    rem /= a.nsplit;
    w.h = rem % a.Hkv;
    rem /= a.Hkv;
  } else {
    w.h = rem % a.Hkv;
    rem /= a.Hkv;
    w.c = rem % a.nsplit;
    rem /= a.nsplit;
  }
  w.rt = rem % a.row_tiles;
  w.g = rem / a.row_tiles;
  w.s_first = a.group_offsets ? a.group_offsets[w.g] : w.g;
  const int s_end = a.group_offsets ? a.group_offsets[w.g + 1] : w.g + 1;
  w.s0 = w.s_first + w.rt * a.apt;
  w.ns = min(a.apt, s_end - w.s0);
  w.tile_id = (w.g * a.row_tiles + w.rt) * a.Hkv + w.h;
  if (w.ns <= 0) return false;
  w.T = a.context_lens[w.s_first];
  w.nact = (w.T + a.split - 1) / a.split;
  w.t_begin = w.c * a.split;
  w.t_end = min(w.T, w.t_begin + a.split);
  return true;
}

__device__ __forceinline__ TileAgent tile_agent(const DecodeArgs& a, int seq) {
  const int ag = a.agent_ids[seq];
  TileAgent t;
  t.lk = (const uint16_t*)a.lk[ag];
  t.lv = (const uint16_t*)a.lv[ag];
  t.bk = (const uint16_t*)a.bk[ag];
  t.bv = (const uint16_t*)a.bv[ag];
  t.r = a.ranks[ag];
  t.seq = seq;
  return t;
}

// Main kernel: one workgroup of kDecodeWaves waves per (group, row tile,
// split, KV head). Writes the split's partial state (m, l, O, C per row), or
// the finished rows when the context fits one split.
template <int RP>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_bf16_kernel(const DecodeArgs a) {
  constexpr int NRT = RP / 16;  // 16-rank tiles of the value accumulator
  constexpr int PW = D + RP;    // floats per merged row (O then C)
  constexpr int PW4 = PW / 4;
  constexpr int NT = kDecodeWaves * 64;
  constexpr int HW = kDecodeWaves / 2;

  __shared__ __align__(16) unsigned char smem[kLdsMain];
  __shared__ TileAgent s_agent[16];
  __shared__ int s_phys[kMaxSplitBlocks];
  __shared__ double s_rev[kMaxRopePairs];
  __shared__ __align__(16) uint16_t s_q[16 * kQPitch];
  __shared__ __align__(16) uint16_t s_bv[256 * D];  // [al][k][dim], apt * RP <= 256
  __shared__ int s_shared_l;

  // ---- work item; consecutive logical items are dealt to one XCD ----
  const int per = (a.n_work + kNumXcd - 1) / kNumXcd;
  const int logical = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (logical >= a.n_work) return;
  WorkItem wi;
  if (!decode_item(a, logical, a.xcd_by_head, wi)) {
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
  const int nsteps = (t_end - t_begin + kStepTokens - 1) / kStepTokens;

  // the first step's base K/V loads go out before anything else; the agent's
  // pointers (a dependent chain of loads) follow
  Step<RP> buf;
  int st = wave;
  if (st < nsteps) {
    const int tb = t_begin + st * kStepTokens;
    const int bi = tb / kBlock;
    const int p0 = bt_row[bi];
    const int p1 = (tb + kBlock < t_end) ? bt_row[bi + 1] : p0;
    load_step_k(buf, a, tb, t_end, p0, p1, h, lc, lg);
  }
  __builtin_amdgcn_sched_barrier(0);
  const TileAgent ag0 = tile_agent(a, s0);
  if (st < nsteps) {
    load_step_l(buf, ag0, lc, lg);
    load_step_v(buf, a, h, lc, lg);
  }

  // ---- preamble: agent table, block ids of the split, B_k^T in LDS, q ----
  if (tid < ns) s_agent[tid] = tile_agent(a, s0 + tid);
  {
    const int nb = (t_end - t_begin + kBlock - 1) / kBlock;
    for (int i = tid; i < nb; i += NT) s_phys[i] = bt_row[blk0 + i];
  }
  if (tid < kMaxRopePairs) s_rev[tid] = a.rope_rev[tid];
  __syncthreads();
  if (tid == 0) {
    int sh = 1;
    for (int i = 1; i < ns; ++i)
      sh &= (s_agent[i].lk == s_agent[0].lk) & (s_agent[i].lv == s_agent[0].lv) & (s_agent[i].r == s_agent[0].r);
    s_shared_l = sh;
  }
  // s_bt[al][dim][k] = B_k,al[k, h*D + dim] (zero for k >= r); lanes take
  // consecutive k so the 2-byte LDS writes of a wave fall in distinct banks
  uint16_t* s_bt = reinterpret_cast<uint16_t*>(smem);
  for (int e = tid; e < ns * RP * (D / 8); e += NT) {
    const int k = e % RP;
    const int d8 = ((e / RP) % (D / 8)) * 8;
    const int al = e / (RP * (D / 8));
    const TileAgent& t = s_agent[al];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < t.r) v = ld16(t.bk + (size_t)k * HD + h * D + d8);
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) s_bt[((size_t)al * D + d8 + i) * RP + k] = pv[i];
  }

  // B_v rows of head h for every agent of the tile (applied to the rank-space
  // accumulator once per row after the token loop)
  for (int e = tid; e < ns * RP * (D / 8); e += NT) {
    const int al = e / (RP * (D / 8)), k = (e / (D / 8)) % RP, d8 = (e % (D / 8)) * 8;
    const TileAgent& t = s_agent[al];
    const uint4 v = k < t.r ? ld16(t.bv + (size_t)k * HD + h * D + d8) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(s_bv + ((size_t)al * RP + k) * D + d8) = v;
  }
  // query tile: row r = (agent slot r / G, head r % G); rows past the tile are zero
  for (int e = tid; e < 16 * (D / 8); e += NT) {
    const int r = e / (D / 8), d8 = (e % (D / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r / G < ns && r < a.apt * G) v = ld16((const uint16_t*)a.q + ((size_t)(s0 + r / G) * a.Hq + h * G + (r % G)) * D + d8);
    *reinterpret_cast<uint4*>(s_q + r * kQPitch + d8) = v;
  }
  Frame fr;
  fr.rev = s_rev;
  fr.q = s_q + lc * kQPitch;
  fr.row_al = lc / G;
  fr.row_ok = (fr.row_al < ns) && (lc < a.apt * G);
  __syncthreads();

  const bool shared_l = s_shared_l != 0;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
  f32x4 acl[NRT];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NRT; ++i) acl[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- main loop over this wave's steps ----
  for (; st < nsteps; st += kDecodeWaves) {
    if (st != wave) {
      const int tb = t_begin + st * kStepTokens;
      const int bi = tb / kBlock - blk0;
      load_step_k(buf, a, tb, t_end, s_phys[bi], (tb + kBlock < t_end) ? s_phys[bi + 1] : 0, h, lc, lg);
      load_step_l(buf, ag0, lc, lg);
      load_step_v(buf, a, h, lc, lg);
    }
    compute_step(buf, a, fr, s_agent, s_bt, ns, shared_l, t_end, lc, lg, m_run, l_run, o, acl);
  }

  // ---- merge the waves of this workgroup in LDS (two rounds) ----
  float l_row = wave_sum_across_groups(l_run);
  __syncthreads();  // s_bt is dead from here on
  float* f = reinterpret_cast<float*>(smem);
  float* mrow = f;                // [HW][16]
  float* lrow = f + 16 * HW;      // [HW][16]
  float* obuf = f + 32 * HW;      // [HW][16][PW]
  // round 1: the upper half of the waves hands its state to the lower half
  if (wave >= HW) {
    const int slot = wave - HW;
    if (lg == 0) {
      mrow[slot * 16 + lc] = m_run;
      lrow[slot * 16 + lc] = l_row;
    }
    float* ob = obuf + ((size_t)slot * 16 + lc) * PW;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ob[16 * cb + 4 * lg + jj] = o[cb][jj];
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ob[D + 16 * rr + 4 * lg + jj] = acl[rr][jj];
  }
  __syncthreads();
  if (wave < HW) {
    const float m2 = mrow[wave * 16 + lc], l2 = lrow[wave * 16 + lc];
    const float mm = fmaxf(m_run, m2);
    const float w1 = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mm);
    const float w2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mm);
    const float* ob = obuf + ((size_t)wave * 16 + lc) * PW;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o[cb][jj] = w1 * o[cb][jj] + w2 * ob[16 * cb + 4 * lg + jj];
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acl[rr][jj] = w1 * acl[rr][jj] + w2 * ob[D + 16 * rr + 4 * lg + jj];
    m_run = mm;
    l_row = w1 * l_row + w2 * l2;
  }
  __syncthreads();
  // round 2: the lower half writes, then 16 threads per row merge
  if (wave < HW) {
    if (lg == 0) {
      mrow[wave * 16 + lc] = m_run;
      lrow[wave * 16 + lc] = l_row;
    }
    float* ob = obuf + ((size_t)wave * 16 + lc) * PW;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ob[16 * cb + 4 * lg + jj] = o[cb][jj];
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ob[D + 16 * rr + 4 * lg + jj] = acl[rr][jj];
  }
  __syncthreads();
  const int rows_used = ns * G;
  if (tid >= 256) return;  // 16 threads per row from here on
  const int row = tid >> 4;
  const int cl = tid & 15;
  float mw[HW];
  float Mrow = -INFINITY;
#pragma unroll
  for (int w = 0; w < HW; ++w) {
    mw[w] = mrow[w * 16 + row];
    Mrow = fmaxf(Mrow, mw[w]);
  }
  float Lrow = 0.f;
#pragma unroll
  for (int w = 0; w < HW; ++w) {
    mw[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - Mrow);
    Lrow += mw[w] * lrow[w * 16 + row];
  }
  // merged state of row `row`: O (D floats) then C (RP floats)
  __shared__ __align__(16) float s_fin[16][PW];
  for (int col = cl; col < PW; col += 16) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < HW; ++w) v += mw[w] * obuf[((size_t)w * 16 + row) * PW + col];
    s_fin[row][col] = v;
  }
  // 16 threads of a row are consecutive lanes of one wave: a wave barrier suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const int d0 = cl * 8;
  float acc[8];
  int seq = 0;
  if (row < rows_used) {
    // O' = O + C B_v over this thread's 8 dims (B_v of the row's agent, from LDS)
    const int al = row / G;
    const TileAgent& ag = s_agent[al];
    seq = ag.seq;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = s_fin[row][d0 + i];
    for (int k = 0; k < ag.r; ++k) {
      const uint4 bvv = *reinterpret_cast<const uint4*>(s_bv + ((size_t)al * RP + k) * D + d0);
      const uint16_t* pb = reinterpret_cast<const uint16_t*>(&bvv);
      const float ck = s_fin[row][D + k];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += ck * bf16_to_f32(pb[i]);
    }
  }
  if (wi.nact > 1) {
    // partial record of this split: [m, l, seq, nact, O'[D]]; unused rows of
    // split 0 are marked empty (nact = 0)
    float* part = a.partials + (((size_t)wi.tile_id * a.nsplit + c) * 16 + row) * a.part_stride;
    if (row < rows_used) {
      if (cl == 0) *reinterpret_cast<float4*>(part) = make_float4(Mrow, Lrow, __int_as_float(seq), __int_as_float(wi.nact));
      *reinterpret_cast<float4*>(part + 4 + d0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(part + 8 + d0) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else if (c == 0 && cl == 0) {
      *reinterpret_cast<float4*>(part) = make_float4(0.f, 0.f, __int_as_float(0), __int_as_float(0));
    }
    return;
  }
  // single split: finish here (and tell the combine this row is done)
  if (a.nsplit > 1 && cl == 0)
    *reinterpret_cast<float4*>(a.partials + (((size_t)wi.tile_id * a.nsplit) * 16 + row) * a.part_stride) =
        make_float4(0.f, 0.f, __int_as_float(0), __int_as_float(1));
  if (row < rows_used) {
    const float inv = 1.f / Lrow;
    uint4 ov;
    ov.x = pack_bf16(acc[0] * inv, acc[1] * inv);
    ov.y = pack_bf16(acc[2] * inv, acc[3] * inv);
    ov.z = pack_bf16(acc[4] * inv, acc[5] * inv);
    ov.w = pack_bf16(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4*>((uint16_t*)a.out + ((size_t)seq * a.Hq + h * G + (row % G)) * D + d0) = ov;
  }
}

// Combine kernel: one wave per (group, row tile, KV head, row) merges the
// split records of that row with weights 2^(m_c - M) and writes the output.
// Every load goes out at once; the record of split 0 says how many splits
// the row has (0: no such row; 1: finished by the main kernel).
__global__ __launch_bounds__(256) void decode_bf16_combine(const DecodeArgs a) {
  __shared__ __align__(16) float s_w[4][kMaxSplits];
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int gid = blockIdx.x * (blockDim.x >> 6) + wave;
  const int n_tiles = a.num_groups * a.row_tiles * a.Hkv;
  if (gid >= n_tiles * 16) return;
  const int tile_id = gid / 16, row = gid % 16;
  const int h = tile_id % a.Hkv;
  const float* pb = a.partials + ((size_t)tile_id * a.nsplit * 16 + row) * a.part_stride;
  const size_t cstride = (size_t)16 * a.part_stride;
  float4 hd = make_float4(-INFINITY, 0.f, 0.f, 0.f);
  if (lane < a.nsplit) hd = ldf4(pb + lane * cstride);
  float4 v[kMaxSplits];
#pragma unroll
  for (int u = 0; u < kMaxSplits; ++u)
    v[u] = (u < a.nsplit && lane < D / 4) ? ldf4(pb + u * cstride + 4 + 4 * lane) : make_float4(0.f, 0.f, 0.f, 0.f);
  const int nact = __float_as_int(__shfl(hd.w, 0));
  const int seq = __float_as_int(__shfl(hd.z, 0));
  if (nact <= 1) return;
  const bool okc = lane < nact;
  float M = okc ? hd.x : -INFINITY;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float w = okc ? fast_exp2(hd.x - M) : 0.f;
  float L = okc ? w * hd.y : 0.f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  s_w[wave][lane] = w;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kMaxSplits; ++u) {
    if (u < nact) {  // selected, not multiplied: records past nact may hold anything
      const float wu = s_w[wave][u];
      acc.x += wu * v[u].x;
      acc.y += wu * v[u].y;
      acc.z += wu * v[u].z;
      acc.w += wu * v[u].w;
    }
  }
  if (lane < D / 4) {
    const float inv = 1.f / L;
    const uint2 ov = make_uint2(pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv));
    *reinterpret_cast<uint2*>((uint16_t*)a.out + ((size_t)seq * a.Hq + h * a.G + (row % a.G)) * D + 4 * lane) = ov;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int rp, hipStream_t stream) {
  const int per = (a.n_work + kNumXcd - 1) / kNumXcd;
  const dim3 grid(per * kNumXcd), block(kDecodeWaves * 64);
  const int n_rows = a.num_groups * a.row_tiles * a.Hkv * 16;
  const dim3 cgrid((n_rows + 3) / 4), cblock(256);
  switch (rp) {
    case 16: hipLaunchKernelGGL(decode_bf16_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(decode_bf16_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit <= 1) return e;
  hipLaunchKernelGGL(decode_bf16_combine, cgrid, cblock, 0, stream, a);
  return hipGetLastError();
}

}  // namespace lra
