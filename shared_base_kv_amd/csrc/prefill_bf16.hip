// Prefill attention over a shared-base + low-rank KV cache on gfx950 MFMA
// (bf16 inputs, fp32 accumulation).
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
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace lra {
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

// KAD / VAD: the call has key / value adapters; without one, that part of
// the work (low-rank loads, staging, rebuild or rank-space products) is not
// compiled in. A sequence without an agent (id -1) runs with rank 0: its
// low-rank loads read nothing and its staged B rows are zero.
template <int RP, bool KAD, bool VAD>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(const PrefillArgs a) {
  constexpr int NRT = RP / 16;
  constexpr int KC = RP >= 32 ? RP / 32 : 1;
  __shared__ __align__(16) uint16_t s_k[kKBufs][kTile * kKPitch];           // rebuilt keys [key][dim]
  __shared__ __align__(16) uint16_t s_v[kVBufs][D * kVPitch];               // V^T [dim][key]
  __shared__ __align__(16) uint16_t s_lv[kVBufs][VAD ? RP * kVPitch : 8];   // L_v^T [rank][key]
  __shared__ __align__(16) uint16_t s_bt[KAD ? D * RP : 8];                 // B_k^T [dim][rank]
  __shared__ __align__(16) uint16_t s_bvt[VAD ? D * RP : 8];                // B_v^T [dim][rank]
  __shared__ __align__(16) float s_rot[kKBufs][2 * kMaxRopePairs];          // (cos, sin) of 64 t theta_i
  __shared__ double s_rev[kMaxRopePairs];

  const int G = a.G;
  const int TQ = kRows / G;  // query tokens per workgroup
  // ---- work item: all tiles of a KV head are consecutive (one XCD) ----
  const int n_work = a.Hkv * a.S * a.q_tiles;
  const int per = (n_work + kNumXcd - 1) / kNumXcd;
  const int logical = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (logical >= n_work) return;
  const int qt = logical % a.q_tiles;
  const int s = (logical / a.q_tiles) % a.S;
  const int h = logical / (a.q_tiles * a.S);
  const int q0 = a.cu_q_lens[s];
  const int q_len = a.cu_q_lens[s + 1] - q0;
  const int t0 = qt * TQ;  // first query token of the tile
  if (t0 >= q_len) return;
  const int n_tok = min(TQ, q_len - t0);
  const int T = a.context_lens[s];
  const int p0 = T - q_len + t0;        // position of the tile's first query
  const int kv_end = p0 + n_tok;        // keys 0..kv_end-1 are visible to some row
  const int ag = (KAD || VAD) ? a.agent_ids[s] : -1;
  const uint16_t* lk = (KAD && ag >= 0) ? (const uint16_t*)a.lk[ag] : nullptr;
  const uint16_t* lv = (VAD && ag >= 0) ? (const uint16_t*)a.lv[ag] : nullptr;
  const uint16_t* bk = (KAD && ag >= 0) ? (const uint16_t*)a.bk[ag] : nullptr;
  const uint16_t* bv = (VAD && ag >= 0) ? (const uint16_t*)a.bv[ag] : nullptr;
  const int r = ag >= 0 ? a.ranks[ag] : 0;
  // activation position: keys before it keep the base key and value
  const int a_start = (ag >= 0 && a.act) ? a.act[s] : 0;
  const int HD = a.Hkv * D;
  const int* bt_row = a.block_tables + (size_t)s * a.max_blocks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  // Producers: with a key adapter every wave rebuilds half of block pw of
  // each tile (the rebuild's registers then fit beside a consumer's);
  // otherwise waves 0..3 each copy a whole block.
  constexpr int NH = KAD ? 2 : 1;
  const bool producer = NH == 2 || wave < 4;
  const int pw = wave & 3;     // cache block of the tile this wave helps produce
  const int hh = wave >> 2;    // its half (NH = 2)
  const int lc = lane & 15;
  const int lg = lane >> 4;

  // ---- preamble: B_k^T, B_v^T, rotary tables ----
  for (int e = tid; (KAD || VAD) && e < RP * (D / 8); e += kThreads) {
    const int k = e % RP, d8 = (e / RP) * 8;
    uint4 vk = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
    if (k < r) {
      if constexpr (KAD) vk = ld16(bk + (size_t)k * HD + h * D + d8);
      if constexpr (VAD) vw = ld16(bv + (size_t)k * HD + h * D + d8);
    }
    const uint16_t* pk = reinterpret_cast<const uint16_t*>(&vk);
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&vw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KAD) s_bt[(d8 + i) * RP + k] = pk[i];
      if constexpr (VAD) s_bvt[(d8 + i) * RP + k] = pv[i];
    }
  }
  // rotary revolutions per position, staged through LDS (a lane-indexed read
  // of the kernel-argument array would go through scratch)
  if (KAD && tid < kMaxRopePairs) s_rev[tid] = a.rope_rev[tid];
  __syncthreads();
  // per-tile table: every wave computes pair `lane` and writes the same value
  const double rev_lane = KAD ? s_rev[lane] : 0.0;
  auto rot_table = [&](int t) __attribute__((always_inline)) {
    if constexpr (KAD) {
      const float2 cs = cos_sin_rev((double)(t * kTile) * rev_lane);
      *reinterpret_cast<float2*>(&s_rot[t & 1][2 * lane]) = cs;
    }
  };
  rot_table(0);
  rot_table(1);
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;
  const int n_tiles = (kv_end + kTile - 1) / kTile;
  const float csc = a.sm_scale_log2;

  __syncthreads();  // B_k^T, B_v^T and the first rotary tables are in LDS

  // per-lane part (producers): key offset 16 pw + lc within the tile, pairs 16cb + 4lg + jj
  constexpr int NCB = 4 / NH, NPAR = 2 / NH;
  const int cb0 = NH == 2 ? 2 * hh : 0;   // first 16-pair group of this wave
  const int par0 = NH == 2 ? hh : 0;      // first V^T row parity / L_v^T item block of this wave
  float co[NCB][4], so[NCB][4];
  if constexpr (KAD) {
    const double off = (double)(kBlock * pw + lc);
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float2 cs = cos_sin_rev(off * s_rev[16 * (cb0 + c) + 4 * lg + jj]);
        co[c][jj] = cs.x;
        so[c][jj] = cs.y;
      }
  }

  // ---- global -> registers: block `pw` of tile t. Blocks past the
  // visible keys get zero-length buffer ranges, so their loads return 0. ----
  TileRegs<RP, NH> tr;
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * kTile + kBlock * pw;
    const bool valid = key0 < kv_end;
    const int phys = uniform(bt_row[valid ? key0 / kBlock : 0]);
    const int on = valid ? 1 : 0;
    const int lon = (valid && key0 + kBlock > a_start) ? 1 : 0;  // low-rank rows needed
    const auto rk = buf_rsrc((const uint16_t*)a.kb + (size_t)phys * blk_elems + (size_t)h * kBlock * D,
                             on * kBlock * D * 2);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int cb = cb0 + c;
      tr.kbl[c] = bld8(rk, (lc * D + 16 * cb + 4 * lg) * 2);
      tr.kbh[c] = bld8(rk, (lc * D + 64 + 16 * cb + 4 * lg) * 2);
    }
    if constexpr (KAD) {
      const auto rlk = buf_rsrc(lk + (size_t)phys * kBlock * r, lon * kBlock * r * 2);
      // a key before the activation point reads no low-rank row (its
      // rebuilt adapter term is then exactly zero)
      const bool kon = key0 + lc >= a_start;
      if constexpr (RP == 16) {
        const uint2 v = bld8(rlk, (kon && 4 * lg < r) ? (lc * r + 4 * lg) * 2 : kOob);
        tr.lk[0] = make_uint4(v.x, v.y, 0, 0);
      } else {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          tr.lk[kc] = bld16(rlk, (kon && 32 * kc + 8 * lg < r) ? (lc * r + 32 * kc + 8 * lg) * 2 : kOob);
      }
    }
    const auto rv = buf_rsrc((const uint16_t*)a.vb + (size_t)phys * blk_elems + (size_t)h * D * kBlock,
                             on * D * kBlock * 2);
#pragma unroll
    for (int p = 0; p < NPAR; ++p)
#pragma unroll
      for (int k = 0; k < 2; ++k) tr.vv[p][k] = bld16(rv, ((2 * lane + par0 + p) * kBlock + 8 * k) * 2);
    if constexpr (VAD) {
      const auto rlv = buf_rsrc(lv + (size_t)phys * r * kBlock, lon * r * kBlock * 2);
#pragma unroll
      for (int p = 0; p < NPAR; ++p) {
        const int e = lane + 64 * (par0 + p), rank = e >> 1;
        tr.lvv[p] = bld16(rlv, (e < 2 * RP && rank < r) ? (rank * kBlock + 8 * (e & 1)) * 2 : kOob);
      }
    }
  };

  // ---- registers -> LDS: V^T, L_v^T as loaded; keys rebuilt as
  // K_base + rope(B_k^T L_k^T), rounded once to bf16. LAST marks the final
  // tile, the only one that can hold positions >= T (zeroed in V and L_v,
  // whose products with P = 0 must stay finite). Keys before the activation
  // point got zero low-rank rows at load time, so their rebuilt key is the
  // base key; their L_v columns are zeroed here. The rebuild itself has no
  // branch, so it shares one basic block with the next tile's loads. ----
  auto store_tile = [&](int t, auto last_tag) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int key0 = t * kTile + kBlock * pw;
    const bool early = key0 < a_start;  // some key of the block is before the activation point
    uint16_t* sk = s_k[t & 1];
    uint16_t* sv = s_v[t % kVBufs];
    uint16_t* slv = s_lv[t % kVBufs];
#pragma unroll
    for (int pp = 0; pp < NPAR; ++pp)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint4 v = tr.vv[pp][k];
        if constexpr (LAST) {
          const int kk = key0 + 8 * k;
          uint32_t* w32 = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
          for (int p = 0; p < 4; ++p)
            w32[p] &= (kk + 2 * p < T ? 0xFFFFu : 0u) | (kk + 2 * p + 1 < T ? 0xFFFF0000u : 0u);
        }
        // keys 8k .. 8k + 7 of block pw land in the permuted key order (see kvpos)
        uint16_t* row = sv + (2 * lane + par0 + pp) * kVPitch + kvpos(pw, k);
        *reinterpret_cast<uint2*>(row) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(row + 8) = make_uint2(v.z, v.w);
      }
#pragma unroll
    for (int pp = 0; pp < (VAD ? NPAR : 0); ++pp) {
      const int e = lane + 64 * (par0 + pp);
      if (e < 2 * RP) {
        uint4 v = tr.lvv[pp];
        if (LAST || early) {  // keys past the context or before the activation point
          const int kk = key0 + 8 * (e & 1);
          uint32_t* w32 = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int k1 = kk + 2 * p, k2 = k1 + 1;
            w32[p] &= ((k1 >= a_start && (!LAST || k1 < T)) ? 0xFFFFu : 0u) |
                      ((k2 >= a_start && (!LAST || k2 < T)) ? 0xFFFF0000u : 0u);
          }
        }
        uint16_t* row = slv + (e >> 1) * kVPitch + kvpos(pw, e & 1);
        *reinterpret_cast<uint2*>(row) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(row + 8) = make_uint2(v.z, v.w);
      }
    }
    if constexpr (!KAD) {  // no key adapter: the base keys as loaded
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int cb = cb0 + c;
        *reinterpret_cast<uint2*>(sk + (kBlock * pw + lc) * kKPitch + 16 * cb + 4 * lg) = tr.kbl[c];
        *reinterpret_cast<uint2*>(sk + (kBlock * pw + lc) * kKPitch + 64 + 16 * cb + 4 * lg) = tr.kbh[c];
      }
      return;
    }

    const float* rot = s_rot[t & 1];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int cb = cb0 + c;
      f32x4 xl = f32x4{0.f, 0.f, 0.f, 0.f}, xh = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (RP == 16) {
        const uint2 al_ = *reinterpret_cast<const uint2*>(s_bt + (16 * cb + lc) * RP + 4 * lg);
        const uint2 ah_ = *reinterpret_cast<const uint2*>(s_bt + (16 * (cb + 4) + lc) * RP + 4 * lg);
        const uint2 lk2 = make_uint2(tr.lk[0].x, tr.lk[0].y);
        xl = mfma16(as_i16x4(al_), as_i16x4(lk2), xl);
        xh = mfma16(as_i16x4(ah_), as_i16x4(lk2), xh);
      } else {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint4 al_ = *reinterpret_cast<const uint4*>(s_bt + (16 * cb + lc) * RP + 32 * kc + 8 * lg);
          const uint4 ah_ = *reinterpret_cast<const uint4*>(s_bt + (16 * (cb + 4) + lc) * RP + 32 * kc + 8 * lg);
          xl = mfma32(as_bf16x8(al_), as_bf16x8(tr.lk[kc]), xl);
          xh = mfma32(as_bf16x8(ah_), as_bf16x8(tr.lk[kc]), xh);
        }
      }
      const float4 r01 = *reinterpret_cast<const float4*>(rot + 2 * (16 * cb + 4 * lg));
      const float4 r23 = *reinterpret_cast<const float4*>(rot + 2 * (16 * cb + 4 * lg) + 4);
      const float cB[4] = {r01.x, r01.z, r23.x, r23.z};
      const float sB[4] = {r01.y, r01.w, r23.y, r23.w};
      const float kl[4] = {__uint_as_float(tr.kbl[c].x << 16), __uint_as_float(tr.kbl[c].x & 0xFFFF0000u),
                           __uint_as_float(tr.kbl[c].y << 16), __uint_as_float(tr.kbl[c].y & 0xFFFF0000u)};
      const float kh[4] = {__uint_as_float(tr.kbh[c].x << 16), __uint_as_float(tr.kbh[c].x & 0xFFFF0000u),
                           __uint_as_float(tr.kbh[c].y << 16), __uint_as_float(tr.kbh[c].y & 0xFFFF0000u)};
      float y1[4], y2[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // angle of pair 16cb + 4lg + jj at position 64t + 16 pw + lc
        const float cs = cB[jj] * co[c][jj] - sB[jj] * so[c][jj];
        const float sn = sB[jj] * co[c][jj] + cB[jj] * so[c][jj];
        const float u = xl[jj], w = xh[jj];
        y1[jj] = __builtin_fmaf(-w, sn, __builtin_fmaf(u, cs, kl[jj]));
        y2[jj] = __builtin_fmaf(u, sn, __builtin_fmaf(w, cs, kh[jj]));
      }
      *reinterpret_cast<uint2*>(sk + (kBlock * pw + lc) * kKPitch + 16 * cb + 4 * lg) =
          pack_bf16x4(y1[0], y1[1], y1[2], y1[3]);
      *reinterpret_cast<uint2*>(sk + (kBlock * pw + lc) * kKPitch + 64 + 16 * cb + 4 * lg) =
          pack_bf16x4(y2[0], y2[1], y2[2], y2[3]);
    }
  };
  auto store = [&](int t, auto last_tag) __attribute__((always_inline)) { store_tile(t, last_tag); };

  if (producer) {
    load_tile(0);
    if (n_tiles == 1)
      store(0, std::true_type{});
    else
      store(0, std::false_type{});
    if (n_tiles > 1) load_tile(1);
  }
  auto produce = [&](int kt) __attribute__((always_inline)) {
    if (producer) {
      if (kt + 2 < n_tiles) {
        store(kt + 1, std::false_type{});
        load_tile(kt + 2);
        rot_table(kt + 2);
      } else if (kt + 1 < n_tiles) {
        store(kt + 1, std::true_type{});
      }
    }
  };

  // ---- consumers ----
  // ---- query operands (consumers): this wave's rows 32w + 16rt + lc ----
  bf16x8 qb[2][4];
  int rpos[2];    // position of the row's query token
  bool rok[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = 32 * wave + 16 * rt + lc;
    const int t = row / G, j = row % G;
    rok[rt] = (row < TQ * G) && (t < n_tok);
    rpos[rt] = p0 + t;
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(q0 + t0 + t) * a.Hq + h * G + j) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qb[rt][ks] = rok[rt] ? as_bf16x8(ld16(qp + 32 * ks + 8 * lg)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  f32x4 o[2][8];
  f32x4 cacc[2][NRT];
  float m_run[2], l_run[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NRT; ++i) cacc[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // ---- S^T[key, row] for the tile's 4 key blocks x this wave's 2 row tiles ----
  f32x4 sacc[4][2];
  auto scores = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* sk = s_k[t & 1];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kop[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kop[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sk + (kBlock * kb + lc) * kKPitch + 32 * ks + 8 * lg));
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        sacc[kb][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[kb][rt] = mfma32(kop[ks], qb[rt][ks], sacc[kb][rt]);
      }
    }
    // key reads of two blocks ahead of the products that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- O^T += V^T P^T ; C^T += L_v^T P^T for tile t with the P^T operands ----
  bf16x8 pop[2][2];  // [row tile][key pair (blocks 2kp, 2kp+1)]
  auto pv = [&](int t) __attribute__((always_inline)) {
    const uint16_t* sv = s_v[t % kVBufs];
    const uint16_t* slv = s_lv[t % kVBufs];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const bf16x8 vop = as_bf16x8(*reinterpret_cast<const uint4*>(sv + (16 * db + lc) * kVPitch + 32 * kp + 8 * lg));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) o[rt][db] = mfma32(vop, pop[rt][kp], o[rt][db]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < (VAD ? NRT : 0); ++rr) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const bf16x8 lop = as_bf16x8(*reinterpret_cast<const uint4*>(slv + (16 * rr + lc) * kVPitch + 32 * kp + 8 * lg));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) cacc[rt][rr] = mfma32(lop, pop[rt][kp], cacc[rt][rr]);
      }
    }
    // value reads three dim tiles ahead of the products that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, VAD ? 2 * NRT : 0, 1);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12 + (VAD ? 4 * NRT : 0), 1);
  };

  // ---- online softmax (base 2) of tile t; MASK applies causality and the
  // visible-key bound, needed only on tiles that reach past the first row ----
  auto softmax = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kbase = t * kTile;
    float alpha[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if constexpr (MASK) {
            const int key = kbase + kBlock * kb + 4 * lg + jj;
            const bool vis = key <= rpos[rt] && key < kv_end;
            sacc[kb][rt][jj] = vis ? sacc[kb][rt][jj] : -INFINITY;
          }
          mx = fmaxf(mx, sacc[kb][rt][jj]);
        }
      mx = wave_max_across_groups(mx);
      // The reference max of a row moves only when the tile exceeds it by more
      // than kMaxSlack (base 2), so most tiles need no rescale; probabilities
      // stay below 2^kMaxSlack, and l and O use the same reference.
      const float m_cand = fmaxf(m_run[rt], mx * csc);
      const bool move = m_cand > m_run[rt] + kMaxSlack;  // always on a row's first visible key
      const float m_new = move ? m_cand : m_run[rt];
      // with MASK a row may have seen no key yet (m_new = -inf): keep its state
      const bool dead = MASK && m_new == -INFINITY;
      alpha[rt] = move ? fast_exp2(m_run[rt] - m_new) : 1.f;
      const float nm = dead ? 0.f : -m_new;
      float psum = 0.f;
      float pv_[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          pv_[kb][jj] = fast_exp2(__builtin_fmaf(sacc[kb][rt][jj], csc, nm));
          psum += pv_[kb][jj];
        }
      l_run[rt] = l_run[rt] * alpha[rt] + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        pop[rt][kp] = cat8(pack_bf16x4(pv_[2 * kp][0], pv_[2 * kp][1], pv_[2 * kp][2], pv_[2 * kp][3]),
                           pack_bf16x4(pv_[2 * kp + 1][0], pv_[2 * kp + 1][1], pv_[2 * kp + 1][2], pv_[2 * kp + 1][3]));
    }
    // the probabilities and sums are formed here, in the block of the matrix
    // products they can overlap, not sunk past the rescale branch
    asm volatile("" ::"v"(pop[0][0]), "v"(pop[0][1]), "v"(pop[1][0]), "v"(pop[1][1]), "v"(l_run[0]), "v"(l_run[1]));
    // rescale the accumulators only when some row's running max moved
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[rt][i] *= alpha[rt];
#pragma unroll
        for (int i = 0; i < (VAD ? NRT : 0); ++i) cacc[rt][i] *= alpha[rt];
      }
    }
  };
  // tiles wholly at or before the first row's position need no mask; the
  // two loops keep scores, P V and the softmax of one step in one basic
  // block, so the softmax arithmetic can issue between the matrix products
  const int n_plain = (p0 + 1) / kTile;

  __syncthreads();  // tile 0 is in LDS
  scores(0);
  if (n_plain > 0)
    softmax(0, std::false_type{});
  else
    softmax(0, std::true_type{});
  produce(0);
  __syncthreads();  // scores of tile 0 are done and tile 1 is in LDS
  int kt = 1;
  for (; kt < min(n_plain, n_tiles); ++kt) {
    scores(kt);
    pv(kt - 1);
    softmax(kt, std::false_type{});
    produce(kt);
    __syncthreads();  // keys of tile kt and values of tile kt - 1 are consumed; tile kt + 1 is in LDS
  }
  for (; kt < n_tiles; ++kt) {
    scores(kt);
    pv(kt - 1);
    softmax(kt, std::true_type{});
    produce(kt);
    __syncthreads();
  }
  pv(n_tiles - 1);

  // ---- epilogue: O^T += B_v^T C^T (C as bf16 hi + lo), divide by l, store ----
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int rr = 0; rr < (VAD ? NRT : 0); ++rr) {
      float hi[4], lo[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        hi[jj] = bf16_to_f32((uint16_t)(pack_bf16(cacc[rt][rr][jj], 0.f) & 0xFFFFu));
        lo[jj] = cacc[rt][rr][jj] - hi[jj];
      }
      const uint2 chi = pack_bf16x4(hi[0], hi[1], hi[2], hi[3]);
      const uint2 clo = pack_bf16x4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint2 bvt = *reinterpret_cast<const uint2*>(s_bvt + (16 * db + lc) * RP + 16 * rr + 4 * lg);
        o[rt][db] = mfma16(as_i16x4(bvt), as_i16x4(chi), o[rt][db]);
        o[rt][db] = mfma16(as_i16x4(bvt), as_i16x4(clo), o[rt][db]);
      }
    }
    const float l = wave_sum_across_groups(l_run[rt]);
    const int row = 32 * wave + 16 * rt + lc;
    if (rok[rt]) {
      const int t = row / G, j = row % G;
      const float inv = 1.f / l;
      uint16_t* op = (uint16_t*)a.out + ((size_t)(q0 + t0 + t) * a.Hq + h * G + j) * D;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<uint2*>(op + 16 * db + 4 * lg) =
            pack_bf16x4(o[rt][db][0] * inv, o[rt][db][1] * inv, o[rt][db][2] * inv, o[rt][db][3] * inv);
    }
  }
}

}  // namespace

namespace {
template <bool KAD, bool VAD>
bool launch_rank(const PrefillArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  switch (a.rp) {
    case 16: hipLaunchKernelGGL((prefill_bf16_kernel<16, KAD, VAD>), grid, block, 0, stream, a); return true;
    case 32: hipLaunchKernelGGL((prefill_bf16_kernel<32, KAD, VAD>), grid, block, 0, stream, a); return true;
    case 64: hipLaunchKernelGGL((prefill_bf16_kernel<64, KAD, VAD>), grid, block, 0, stream, a); return true;
    default: return false;
  }
}
}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const int n_work = a.Hkv * a.S * a.q_tiles;
  const int per = (n_work + kNumXcd - 1) / kNumXcd;
  const dim3 grid(per * kNumXcd), block(kThreads);
  const bool kad = a.bk != nullptr, vad = a.bv != nullptr;
  bool launched;
  if (kad && vad)
    launched = launch_rank<true, true>(a, grid, block, stream);
  else if (vad)
    launched = launch_rank<false, true>(a, grid, block, stream);
  else if (kad)
    launched = launch_rank<true, false>(a, grid, block, stream);
  else {  // no adapter: rank-free
    hipLaunchKernelGGL((prefill_bf16_kernel<16, false, false>), grid, block, 0, stream, a);
    launched = true;
  }
  if (!launched) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lra
