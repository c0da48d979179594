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
// a query tile has 128 rows = 128/G query tokens x G query heads, 4 waves of
// 32 rows. All tiles of one KV head are dealt to one XCD, so the keys they
// share (the common prefix) stream through one L2.
//
// Matrix-core mapping (16x16 tiles):
//   X^T[dim, key]   = B_k^T L_k^T        (per wave: its 16-key block, 16x16x16 / 16x16x32)
//   S^T[key, row]   = K_a Q^T            (16x16x32, K_a from LDS)
//   O^T[dim, row]  += V^T P^T            (16x16x32, V^T from LDS, P^T from the S^T accumulators)
//   C^T[rank, row] += L_v^T P^T
//   O^T            += B_v^T C^T          (after the loop; C split into bf16 hi + lo)
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int D = 128;
constexpr int kRows = 128;     // query rows per workgroup
constexpr int kTile = 64;      // keys per tile (4 cache blocks)
constexpr int kKPitch = D + 8;          // LDS row pitch of the key tile (bf16)
constexpr int kVPitch = kTile + 8;      // LDS row pitch of the V^T / L_v^T tiles (bf16)

template <int RP>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(const PrefillArgs a) {
  constexpr int NRT = RP / 16;
  constexpr int KC = RP >= 32 ? RP / 32 : 1;
  __shared__ __align__(16) uint16_t s_k[kTile * kKPitch];   // rebuilt keys [key][dim]
  __shared__ __align__(16) uint16_t s_v[D * kVPitch];       // V^T [dim][key]
  __shared__ __align__(16) uint16_t s_lv[RP * kVPitch];     // L_v^T [rank][key]
  __shared__ __align__(16) uint16_t s_bt[D * RP];           // B_k^T [dim][rank]
  __shared__ __align__(16) uint16_t s_bvt[D * RP];          // B_v^T [dim][rank]
  __shared__ double s_rev[kMaxRopePairs];
  __shared__ int s_phys[kTile / kBlock];

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
  const int ag = a.agent_ids[s];
  const uint16_t* lk = (const uint16_t*)a.lk[ag];
  const uint16_t* lv = (const uint16_t*)a.lv[ag];
  const uint16_t* bk = (const uint16_t*)a.bk[ag];
  const uint16_t* bv = (const uint16_t*)a.bv[ag];
  const int r = a.ranks[ag];
  const int HD = a.Hkv * D;
  const int* bt_row = a.block_tables + (size_t)s * a.max_blocks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lc = lane & 15;
  const int lg = lane >> 4;

  // ---- preamble: B_k^T, B_v^T, rotary table ----
  for (int e = tid; e < RP * (D / 8); e += 256) {
    const int k = e % RP, d8 = (e / RP) * 8;
    uint4 vk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (k < r) {
      vk = ld16(bk + (size_t)k * HD + h * D + d8);
      vv = ld16(bv + (size_t)k * HD + h * D + d8);
    }
    const uint16_t* pk = reinterpret_cast<const uint16_t*>(&vk);
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s_bt[(d8 + i) * RP + k] = pk[i];
      s_bvt[(d8 + i) * RP + k] = pv[i];
    }
  }
  if (tid < kMaxRopePairs) s_rev[tid] = a.rope_rev[tid];

  // ---- query operands: this wave's rows 32w + 16rt + lc ----
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
  const bf16x8 zero8 = as_bf16x8(make_uint4(0, 0, 0, 0));
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;
  const int n_tiles = (kv_end + kTile - 1) / kTile;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int kbase = kt * kTile;
    __syncthreads();  // previous tile's LDS reads are done
    if (tid < kTile / kBlock) s_phys[tid] = (kbase + kBlock * tid < kv_end) ? bt_row[kbase / kBlock + tid] : -1;
    __syncthreads();

    // ---- wave w: block w of the tile -> rebuilt keys, V^T and L_v^T into LDS ----
    {
      const int b = wave;
      const int phys = uniform(s_phys[b]);
      const int key0 = kbase + kBlock * b;
      if (phys >= 0) {
        const uint16_t* kp = (const uint16_t*)a.kb + (size_t)phys * blk_elems + (size_t)h * kBlock * D;
        const uint16_t* vp = (const uint16_t*)a.vb + (size_t)phys * blk_elems + (size_t)h * D * kBlock;
        // V^T: 128 dims x 16 keys of this block; keys past the sequence read as zero
        const auto rv = buf_rsrc(vp, D * kBlock * 2);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int dim = 2 * lane + (u >> 1), half = u & 1;  // lane covers dims 2lane, 2lane+1
          uint4 v = bld16(rv, (dim * kBlock + 8 * half) * 2);
          const int kk = key0 + 8 * half;
          uint32_t* w32 = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t m = (kk + 2 * p < T ? 0xFFFFu : 0u) | (kk + 2 * p + 1 < T ? 0xFFFF0000u : 0u);
            w32[p] &= m;
          }
          *reinterpret_cast<uint4*>(s_v + dim * kVPitch + kBlock * b + 8 * half) = v;
        }
        // L_v^T: ranks x 16 keys
        const auto rlv = buf_rsrc(lv + (size_t)phys * r * kBlock, r * kBlock * 2);
        for (int e = lane; e < RP * 2; e += 64) {
          const int rank = e >> 1, half = e & 1;
          uint4 v = bld16(rlv, rank < r ? (rank * kBlock + 8 * half) * 2 : kOob);
          const int kk = key0 + 8 * half;
          uint32_t* w32 = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t m = (kk + 2 * p < T ? 0xFFFFu : 0u) | (kk + 2 * p + 1 < T ? 0xFFFF0000u : 0u);
            w32[p] &= m;
          }
          *reinterpret_cast<uint4*>(s_lv + rank * kVPitch + kBlock * b + 8 * half) = v;
        }
        // rebuilt keys: X^T = B_k^T L_k^T for this block, rotated, plus the base key
        const auto rlk = buf_rsrc(lk + (size_t)phys * kBlock * r, kBlock * r * 2);
        uint2 lk16 = make_uint2(0, 0);
        bf16x8 lk32[KC];
        if constexpr (RP == 16) {
          lk16 = bld8(rlk, (4 * lg < r) ? (lc * r + 4 * lg) * 2 : kOob);
        } else {
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            lk32[kc] = as_bf16x8(bld16(rlk, (32 * kc + 8 * lg < r) ? (lc * r + 32 * kc + 8 * lg) * 2 : kOob));
        }
        const auto rk = buf_rsrc(kp, kBlock * D * 2);
        const double pd = (double)(key0 + lc);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          f32x4 xl = f32x4{0.f, 0.f, 0.f, 0.f}, xh = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (RP == 16) {
            const uint2 al_ = *reinterpret_cast<const uint2*>(s_bt + (16 * cb + lc) * RP + 4 * lg);
            const uint2 ah_ = *reinterpret_cast<const uint2*>(s_bt + (16 * (cb + 4) + lc) * RP + 4 * lg);
            xl = mfma16(as_i16x4(al_), as_i16x4(lk16), xl);
            xh = mfma16(as_i16x4(ah_), as_i16x4(lk16), xh);
          } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              const uint4 al_ = *reinterpret_cast<const uint4*>(s_bt + (16 * cb + lc) * RP + 32 * kc + 8 * lg);
              const uint4 ah_ = *reinterpret_cast<const uint4*>(s_bt + (16 * (cb + 4) + lc) * RP + 32 * kc + 8 * lg);
              xl = mfma32(as_bf16x8(al_), lk32[kc], xl);
              xh = mfma32(as_bf16x8(ah_), lk32[kc], xh);
            }
          }
          // lane: key lc of the block, dims 16cb + 4lg + jj and 64 + 16cb + 4lg + jj
          const uint2 kl = bld8(rk, (lc * D + 16 * cb + 4 * lg) * 2);
          const uint2 kh = bld8(rk, (lc * D + 64 + 16 * cb + 4 * lg) * 2);
          const uint16_t* pkl = reinterpret_cast<const uint16_t*>(&kl);
          const uint16_t* pkh = reinterpret_cast<const uint16_t*>(&kh);
          float y1[4], y2[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float u = xl[jj], w = xh[jj];
            if (a.rope) {
              const double x = pd * s_rev[16 * cb + 4 * lg + jj];
              const float f = (float)(x - __builtin_floor(x));
              const float c = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
              const float u2 = u * c - w * sn;
              w = w * c + u * sn;
              u = u2;
            }
            y1[jj] = bf16_to_f32(pkl[jj]) + u;
            y2[jj] = bf16_to_f32(pkh[jj]) + w;
          }
          *reinterpret_cast<uint2*>(s_k + (kBlock * b + lc) * kKPitch + 16 * cb + 4 * lg) =
              pack_bf16x4(y1[0], y1[1], y1[2], y1[3]);
          *reinterpret_cast<uint2*>(s_k + (kBlock * b + lc) * kKPitch + 64 + 16 * cb + 4 * lg) =
              pack_bf16x4(y2[0], y2[1], y2[2], y2[3]);
        }
      } else {
        // block past the visible keys: zero keys, values and low-rank rows
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int dim = 2 * lane + (u >> 1), half = u & 1;
          *reinterpret_cast<uint4*>(s_v + dim * kVPitch + kBlock * b + 8 * half) = make_uint4(0, 0, 0, 0);
        }
        for (int e = lane; e < RP * 2; e += 64)
          *reinterpret_cast<uint4*>(s_lv + (e >> 1) * kVPitch + kBlock * b + 8 * (e & 1)) = make_uint4(0, 0, 0, 0);
        for (int e = lane; e < kBlock * (D / 8); e += 64)
          *reinterpret_cast<uint4*>(s_k + (kBlock * b + e / (D / 8)) * kKPitch + 8 * (e % (D / 8))) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();

    // ---- scores S^T[key, row] for the 4 key blocks x this wave's 2 row tiles ----
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kop[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kop[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(s_k + (kBlock * kb + lc) * kKPitch + 32 * ks + 8 * lg));
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        sacc[kb][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[kb][rt] = mfma32(kop[ks], qb[rt][ks], sacc[kb][rt]);
      }
    }
    // ---- causal online softmax (base 2) per row ----
    bf16x8 pop[2][2];  // P^T operands: [row tile][key pair (blocks 2kp, 2kp+1)]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float sv[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = kbase + kBlock * kb + 4 * lg + jj;
          const bool vis = key <= rpos[rt] && key < kv_end;
          sv[kb][jj] = vis ? sacc[kb][rt][jj] * a.sm_scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[kb][jj]);
        }
      mx = wave_max_across_groups(mx);
      const float m_new = fmaxf(m_run[rt], mx);
      // a row that sees no key of this tile keeps its state (m_new may be -inf)
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[rt] - m_new);
      float psum = 0.f;
      float pv[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          pv[kb][jj] = (m_new == -INFINITY) ? 0.f : fast_exp2(sv[kb][jj] - m_new);
          psum += pv[kb][jj];
        }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[rt][i] *= alpha;
#pragma unroll
      for (int i = 0; i < NRT; ++i) cacc[rt][i] *= alpha;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        pop[rt][kp] = cat8(pack_bf16x4(pv[2 * kp][0], pv[2 * kp][1], pv[2 * kp][2], pv[2 * kp][3]),
                           pack_bf16x4(pv[2 * kp + 1][0], pv[2 * kp + 1][1], pv[2 * kp + 1][2], pv[2 * kp + 1][3]));
    }
    // ---- O^T += V^T P^T ; C^T += L_v^T P^T ----
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const uint16_t* vr = s_v + (16 * db + lc) * kVPitch + 32 * kp + 4 * lg;
        const bf16x8 vop = cat8(*reinterpret_cast<const uint2*>(vr), *reinterpret_cast<const uint2*>(vr + kBlock));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) o[rt][db] = mfma32(vop, pop[rt][kp], o[rt][db]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const uint16_t* lr = s_lv + (16 * rr + lc) * kVPitch + 32 * kp + 4 * lg;
        const bf16x8 lop = cat8(*reinterpret_cast<const uint2*>(lr), *reinterpret_cast<const uint2*>(lr + kBlock));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) cacc[rt][rr] = mfma32(lop, pop[rt][kp], cacc[rt][rr]);
      }
    }
  }

  // ---- epilogue: O^T += B_v^T C^T (C as bf16 hi + lo), divide by l, store ----
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int rr = 0; rr < NRT; ++rr) {
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

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const int n_work = a.Hkv * a.S * a.q_tiles;
  const int per = (n_work + kNumXcd - 1) / kNumXcd;
  const dim3 grid(per * kNumXcd), block(256);
  switch (a.rp) {
    case 16: hipLaunchKernelGGL(prefill_bf16_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(prefill_bf16_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lra
