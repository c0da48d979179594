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
// end. Splits of one (g, rt, h) meet in the last-arriving workgroup, which
// merges their partial states and finishes the row (adds (P L_v) B_v,
// divides by the softmax sum, rounds to bf16).
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

template <int RP>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const DecodeArgs a) {
  constexpr int NRT = RP / 16;  // 16-rank tiles of the value accumulator
  constexpr int PW = D + RP;    // floats per merged row (O then C)

  __shared__ __align__(16) unsigned char smem[kLdsMain];
  __shared__ TileAgent s_agent[16];
  __shared__ int s_shared_l;
  __shared__ int s_last;

  // ---- work item (XCD-aware: consecutive logical items share an XCD) ----
  const int per = (a.n_work + kNumXcd - 1) / kNumXcd;
  const int logical = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (logical >= a.n_work) return;
  int rem = logical;
  const int h = rem % a.Hkv;
  rem /= a.Hkv;
  const int c = rem % a.nsplit;
  rem /= a.nsplit;
  const int rt = rem % a.row_tiles;
  const int g = rem / a.row_tiles;

  const int s_first = a.group_offsets ? a.group_offsets[g] : g;
  const int s_last_seq = a.group_offsets ? a.group_offsets[g + 1] : g + 1;
  const int s0 = s_first + rt * a.apt;
  const int ns = min(a.apt, s_last_seq - s0);
  if (ns <= 0) return;
  const int T = a.context_lens[s_first];
  const int nact = (T + a.split - 1) / a.split;
  if (c >= nact) return;
  const int t_begin = c * a.split;
  const int t_end = min(T, t_begin + a.split);
  const int tile_id = (g * a.row_tiles + rt) * a.Hkv + h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane & 15;  // accumulator column / operand row
  const int lg = lane >> 4;  // k-group
  const int G = a.G;
  const int HD = a.Hkv * D;

  // ---- per-tile agent table and B_k^T staging ----
  if (tid < ns) {
    const int seq = s0 + tid;
    const int ag = a.agent_ids[seq];
    TileAgent t;
    t.lk = (const uint16_t*)a.lk[ag];
    t.lv = (const uint16_t*)a.lv[ag];
    t.bk = (const uint16_t*)a.bk[ag];
    t.bv = (const uint16_t*)a.bv[ag];
    t.r = a.ranks[ag];
    t.seq = seq;
    s_agent[tid] = t;
  }
  __syncthreads();
  if (tid == 0) {
    int sh = 1;
    for (int i = 1; i < ns; ++i)
      sh &= (s_agent[i].lk == s_agent[0].lk) & (s_agent[i].lv == s_agent[0].lv) & (s_agent[i].r == s_agent[0].r);
    s_shared_l = sh;
  }
  // s_bt[al][dim][k] = B_k,al[k, h*D + dim] (zero for k >= r)
  uint16_t* s_bt = reinterpret_cast<uint16_t*>(smem);
  for (int e = tid; e < ns * RP * (D / 8); e += 256) {
    const int al = e / (RP * (D / 8));
    const int k = (e / (D / 8)) % RP;
    const int d8 = (e % (D / 8)) * 8;
    const TileAgent& t = s_agent[al];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < t.r) v = ld16(t.bk + (size_t)k * HD + h * D + d8);
    const uint16_t* pv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) s_bt[((size_t)al * D + d8 + i) * RP + k] = pv[i];
  }

  // ---- query operands (this lane's column = query row lc of the tile) ----
  const int row_al = lc / G;
  const bool row_ok = (row_al < ns) && (lc < a.apt * G);
  bf16x8 qb[4], qa[4];
  {
    const uint16_t* qp = nullptr;
    if (row_ok) {
      const int seq = s0 + row_al;
      const int qh = h * G + (lc % G);
      qp = (const uint16_t*)a.q + ((size_t)seq * a.Hq + qh) * D;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qb[ks] = row_ok ? as_bf16x8(ld16(qp + 32 * ks + 8 * lg)) : as_bf16x8(make_uint4(0, 0, 0, 0));
      qa[ks] = row_ok ? cat8(ld8(qp + 16 * ks + 4 * lg), ld8(qp + 64 + 16 * ks + 4 * lg))
                      : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }

  // rotary revolutions per position for this lane's 16 pairs i = 16cb + 4lg + jj
  double rev[16];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = 16 * cb + 4 * lg + jj;
      rev[cb * 4 + jj] = a.rope ? exp2(-2.0 * i / D * a.rope_log2_theta) * 0.15915494309189535 : 0.0;
    }
  __syncthreads();

  const bool shared_l = s_shared_l != 0;
  const int* bt_row = a.block_tables + (size_t)s_first * a.max_blocks;
  const size_t head_k = (size_t)h * kBlock * D;  // offset of head h inside a K block
  const size_t head_v = (size_t)h * D * kBlock;
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
  f32x4 acl[NRT];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NRT; ++i) acl[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (t_end - t_begin + kStepTokens - 1) / kStepTokens;
  for (int st = wave; st < nsteps; st += kDecodeWaves) {
    const int tb = t_begin + st * kStepTokens;
    const int nvalid = min(kStepTokens, t_end - tb);
    const int nblk = nvalid > kBlock ? 2 : 1;
    int phys[2];
    phys[0] = bt_row[tb / kBlock];
    phys[1] = nblk > 1 ? bt_row[tb / kBlock + 1] : phys[0];

    // base K (A operand rows = tokens) and V^T (A operand rows = dims)
    bf16x8 kr[2][4];
    uint2 vr[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint16_t* kp = (const uint16_t*)a.kb + (size_t)phys[b] * blk_elems + head_k + lc * D + 8 * lg;
      const uint16_t* vp = (const uint16_t*)a.vb + (size_t)phys[b] * blk_elems + head_v + lc * kBlock + 4 * lg;
      const bool on = b < nblk;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[b][ks] = on ? as_bf16x8(ld16(kp + 32 * ks)) : as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) vr[b][cb] = on ? ld8(vp + cb * 16 * kBlock) : make_uint2(0, 0);
    }
    // token validity of this lane's slots: token tb + 16b + 4lg + jj
    bool tv[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) tv[b][jj] = (tb + 16 * b + 4 * lg + jj) < t_end;
    // NaN-safe: values of positions past the end are selected to zero
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint32_t m01 = (tv[b][0] ? 0xFFFFu : 0u) | (tv[b][1] ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (tv[b][2] ? 0xFFFFu : 0u) | (tv[b][3] ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        vr[b][cb].x &= m01;
        vr[b][cb].y &= m23;
      }
    }

    // ---- scores S^T for each block ----
    f32x4 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (b >= nblk) continue;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[b] = mfma32(kr[b][ks], qb[ks], sacc[b]);

      // rotary cos/sin at this lane's token (tb + 16b + lc) for its 16 pairs
      float cs[16], sn[16];
      if (a.rope) {
        const double pd = (double)(tb + 16 * b + lc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const double x = pd * rev[i];
          const float f = (float)(x - __builtin_floor(x));
          cs[i] = __builtin_amdgcn_cosf(f);
          sn[i] = __builtin_amdgcn_sinf(f);
        }
      }

      const size_t lrow = (size_t)phys[b] * kBlock + lc;  // L_k row of this lane's token
      i16x4 lk16 = as_i16x4(make_uint2(0, 0));
      bf16x8 lk32[RP >= 32 ? RP / 32 : 1];
      for (int al = 0; al < ns; ++al) {
        const TileAgent& ag = s_agent[al];
        if (al == 0 || !shared_l) {
          if constexpr (RP == 16) {
            lk16 = as_i16x4((4 * lg < ag.r) ? ld8(ag.lk + lrow * ag.r + 4 * lg) : make_uint2(0, 0));
          } else {
#pragma unroll
            for (int kc = 0; kc < RP / 32; ++kc)
              lk32[kc] = (32 * kc + 8 * lg < ag.r) ? as_bf16x8(ld16(ag.lk + lrow * ag.r + 32 * kc + 8 * lg))
                                                   : as_bf16x8(make_uint4(0, 0, 0, 0));
          }
        }
        // X^T = B_k^T L_k^T : dims x tokens
        f32x4 x[8];
        const uint16_t* btp = s_bt + ((size_t)al * D + lc) * RP;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          x[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (RP == 16) {
            const uint2 av = *reinterpret_cast<const uint2*>(btp + (size_t)16 * cb * RP + 4 * lg);
            x[cb] = mfma16(as_i16x4(av), lk16, x[cb]);
          } else {
#pragma unroll
            for (int kc = 0; kc < RP / 32; ++kc) {
              const uint4 av = *reinterpret_cast<const uint4*>(btp + (size_t)16 * cb * RP + 32 * kc + 8 * lg);
              x[cb] = mfma32(as_bf16x8(av), lk32[kc], x[cb]);
            }
          }
        }
        // rotate pairs (dim i, dim i + 64) = (x[cb], x[cb+4]) and contract with q
        const bool mine = row_ok && (row_al == al);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          float y1[4], y2[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float u = x[cb][jj], w = x[cb + 4][jj];
            if (a.rope) {
              y1[jj] = u * cs[cb * 4 + jj] - w * sn[cb * 4 + jj];
              y2[jj] = w * cs[cb * 4 + jj] + u * sn[cb * 4 + jj];
            } else {
              y1[jj] = u;
              y2[jj] = w;
            }
          }
          const bf16x8 yop = cat8(pack_bf16x4(y1[0], y1[1], y1[2], y1[3]), pack_bf16x4(y2[0], y2[1], y2[2], y2[3]));
          const bf16x8 qop = mine ? qa[cb] : as_bf16x8(make_uint4(0, 0, 0, 0));
          sacc[b] = mfma32(yop, qop, sacc[b]);
        }
      }
    }

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
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) o[cb] = mfma32(cat8(vr[0][cb], vr[1][cb]), pop, o[cb]);

    // C^T += L_v^T P^T (per agent pool; rows of other agents masked out)
    for (int al = 0; al < ns; ++al) {
      const TileAgent& ag = s_agent[al];
      if (shared_l && al > 0) break;
      const bf16x8 pm = (shared_l || (row_ok && row_al == al)) ? pop : as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int rr = 0; rr < NRT; ++rr) {
        const int rank = 16 * rr + lc;
        uint2 lvr[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          lvr[b] = make_uint2(0, 0);
          if (b < nblk && rank < ag.r) {
            lvr[b] = ld8(ag.lv + ((size_t)phys[b] * ag.r + rank) * kBlock + 4 * lg);
            const uint32_t m01 = (tv[b][0] ? 0xFFFFu : 0u) | (tv[b][1] ? 0xFFFF0000u : 0u);
            const uint32_t m23 = (tv[b][2] ? 0xFFFFu : 0u) | (tv[b][3] ? 0xFFFF0000u : 0u);
            lvr[b].x &= m01;
            lvr[b].y &= m23;
          }
        }
        acl[rr] = mfma32(cat8(lvr[0], lvr[1]), pm, acl[rr]);
      }
    }
  }

  // ---- merge the 4 waves of this workgroup in LDS ----
  const float l_row = wave_sum_across_groups(l_run);
  __syncthreads();  // s_bt is dead from here on
  float* f = reinterpret_cast<float*>(smem);
  float* mrow = f;            // [4][16]
  float* lrow = f + 64;       // [4][16]
  float* obuf = f + 128;      // [4][16][PW]
  if (lg == 0) {
    mrow[wave * 16 + lc] = m_run;
    lrow[wave * 16 + lc] = l_row;
  }
  {
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
  const int row = tid >> 4;  // 16 threads per row
  const int cl = tid & 15;
  float Mrow, Lrow;
  {
    float mw[kDecodeWaves];
    Mrow = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      mw[w] = mrow[w * 16 + row];
      Mrow = fmaxf(Mrow, mw[w]);
    }
    Lrow = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      mw[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - Mrow);
      Lrow += mw[w] * lrow[w * 16 + row];
    }
    for (int col = cl; col < PW; col += 16) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) v += mw[w] * obuf[((size_t)w * 16 + row) * PW + col];
      obuf[(size_t)row * PW + col] = v;  // merged state lives in wave 0's slot
    }
  }
  const int rows_used = ns * G;
  float* merged = obuf;  // [16][PW]

  if (nact > 1) {
    // publish this split's partial state, then count arrivals
    float* part = a.partials + (((size_t)tile_id * a.nsplit + c) * 16 + row) * a.part_stride;
    if (row < rows_used) {
      if (cl == 0) {
        part[0] = Mrow;
        part[1] = Lrow;
      }
      for (int col = cl; col < PW; col += 16) part[4 + col] = merged[(size_t)row * PW + col];
    }
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const unsigned old = atomicAdd(a.counters + tile_id, 1u);
      s_last = (old == (unsigned)(nact - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // last arrival: merge every split's state of this (group, row tile, head)
    float* wts = obuf + 16 * PW;  // [kMaxSplits][16], outside the merged rows
    const float* pbase = a.partials + (size_t)tile_id * a.nsplit * 16 * a.part_stride;
    float mloc = -INFINITY;
    for (int cc = cl; cc < nact; cc += 16) mloc = fmaxf(mloc, pbase[((size_t)cc * 16 + row) * a.part_stride]);
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o2));
    float lloc = 0.f;
    for (int cc = cl; cc < nact; cc += 16) {
      const float* pr = pbase + ((size_t)cc * 16 + row) * a.part_stride;
      const float w = (row < rows_used) ? fast_exp2(pr[0] - mloc) : 0.f;
      wts[cc * 16 + row] = w;
      lloc += w * ((row < rows_used) ? pr[1] : 0.f);
    }
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1) lloc += __shfl_xor(lloc, o2);
    Lrow = lloc;
    __syncthreads();
    if (row < rows_used) {
      for (int col = cl; col < PW; col += 16) {
        float v = 0.f;
        for (int cc = 0; cc < nact; ++cc)
          v += wts[cc * 16 + row] * pbase[((size_t)cc * 16 + row) * a.part_stride + 4 + col];
        merged[(size_t)row * PW + col] = v;
      }
    }
    if (tid == 0) atomicExch(a.counters + tile_id, 0u);
    __syncthreads();
  } else {
    __syncthreads();
  }

  // ---- finish: out = (O + C B_v) / l, one rounding to bf16 ----
  if (row < rows_used) {
    const int al = row / G;
    const TileAgent& ag = s_agent[al];
    const int qh = h * G + (row % G);
    const int d0 = cl * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = merged[(size_t)row * PW + d0 + i];
    const float* cr = merged + (size_t)row * PW + D;
    for (int k = 0; k < ag.r; ++k) {
      const uint4 bvv = ld16(ag.bv + (size_t)k * HD + h * D + d0);
      const uint16_t* pb = reinterpret_cast<const uint16_t*>(&bvv);
      const float ck = cr[k];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += ck * bf16_to_f32(pb[i]);
    }
    const float inv = 1.f / Lrow;
    uint4 ov;
    ov.x = pack_bf16(acc[0] * inv, acc[1] * inv);
    ov.y = pack_bf16(acc[2] * inv, acc[3] * inv);
    ov.z = pack_bf16(acc[4] * inv, acc[5] * inv);
    ov.w = pack_bf16(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4*>((uint16_t*)a.out + ((size_t)ag.seq * a.Hq + qh) * D + d0) = ov;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int rp, hipStream_t stream) {
  const int per = (a.n_work + kNumXcd - 1) / kNumXcd;
  const dim3 grid(per * kNumXcd), block(256);
  switch (rp) {
    case 16: hipLaunchKernelGGL(decode_bf16_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(decode_bf16_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lra
