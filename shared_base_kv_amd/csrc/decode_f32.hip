// Decode attention over a shared-base + low-rank KV cache in fp32 throughout
// (VALU; no matrix cores, since fp32 results must stay within fp32 rounding).
//
// Same operation as the bf16 kernel (LRAgent: Efficient KV Cache Sharing for
// Multi-LoRA LLM Agents, abstract): the adapter key term is rebuilt per
// 64-token chunk in LDS (rotated, added to the base key) and never written
// to device memory; the value adapter is accumulated in rank space,
// C = sum_n p_n L_v[n], and applied once at the end as C B_v.
// One workgroup per (sequence, KV head); the G query heads of that KV head
// share every chunk. Online softmax in the base-2 domain. A call without
// key (value) adapters, or a sequence without an agent, takes rank 0 for
// that part: its loops run zero times and its pools are not read.
//
// Every operand of a chunk is staged in LDS by coalesced 16-byte loads (base
// keys, V^T, the low-rank rows of both pools), and the next chunk's loads are
// in flight in registers while the current chunk is computed, so a chunk
// costs one memory round trip at most; B_k is staged once per workgroup, B_v
// once after the token loop (in the same LDS array).
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int kChunk = 64;  // tokens per chunk: 4 cache blocks
constexpr int kF32Threads = 256;
constexpr int kMaxRankF32 = 64;

template <int D>
__global__ __launch_bounds__(kF32Threads) void decode_f32_kernel(const DecodeArgs a) {
  constexpr int HALF = D / 2;
  constexpr int kQK = kChunk * D / 4 / kF32Threads;            // 16-byte loads per thread: base keys (and values)
  constexpr int kQL = kChunk * kMaxRankF32 / 4 / kF32Threads;  // ... low-rank rows of one pool (at most)
  constexpr int kF4Blk = 4 * D;                                // 16-byte pieces of one block's keys (or values)
  __shared__ float sK[kChunk][D + 1];           // keys of the chunk [token][dim]: base, then + rope(L_k B_k)
  __shared__ float sV[D][kChunk + 1];           // V^T of the chunk [dim][token]
  __shared__ float sLk[kChunk][kMaxRankF32 + 1];  // L_k rows [token][rank]
  __shared__ float sLv[kMaxRankF32][kChunk + 1];  // L_v^T [rank][token]
  __shared__ float sB[kMaxRankF32 * D];         // B_k [rank][dim] of head h; B_v after the token loop
  __shared__ float sQ[16][D];
  __shared__ float sP[16][kChunk];
  __shared__ float sM[16], sL[16], sAlpha[16];
  __shared__ float sC[16][kMaxRankF32];
  __shared__ double sRev[kMaxRopePairs];
  __shared__ float sU[16][kMaxRankF32];         // without rotary: B_k q per query row

  const int s = blockIdx.x / a.Hkv;
  const int h = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.G;
  const int HD = a.Hkv * D;
  const bool kad = a.bk != nullptr, vad = a.bv != nullptr;
  const int ag = (kad || vad) ? a.agent_ids[s] : -1;
  const int r_ag = ag >= 0 ? a.ranks[ag] : 0;
  const int rk = kad ? r_ag : 0;  // rank of the key adapter (0: none)
  const int rv = vad ? r_ag : 0;  // rank of the value adapter (0: none)
  const float* lk = rk ? (const float*)a.lk[ag] : nullptr;
  const float* lv = rv ? (const float*)a.lv[ag] : nullptr;
  const float* bk = rk ? (const float*)a.bk[ag] : nullptr;
  const float* bv = rv ? (const float*)a.bv[ag] : nullptr;
  const int act = (ag >= 0 && a.act) ? a.act[s] : 0;  // tokens before it carry no adapter term
  const float* kb = (const float*)a.kb;
  const float* vb = (const float*)a.vb;
  const int T = a.context_lens[s];
  const int* bt = a.block_tables + (size_t)s * a.max_blocks;

  for (int e = tid; e < G * D; e += kF32Threads) {
    const int row = e / D, i = e % D;
    sQ[row][i] = ((const float*)a.q)[((size_t)s * a.Hq + h * G + row) * D + i];
  }
  for (int e = tid; e < rk * D; e += kF32Threads) sB[e] = bk[(size_t)(e / D) * HD + h * D + e % D];
  if (tid < kMaxRopePairs) sRev[tid] = a.rope_rev[tid];
  if (tid < 16) {
    sM[tid] = -INFINITY;
    sL[tid] = 0.f;
  }

  // ---- the chunk's loads into registers; pieces past the context (or before
  // the activation point, for the low-rank rows) are zero ----
  float4 rK[kQK], rV[kQK], rLk[kQL], rLv[kQL];
  // Physical blocks of a chunk (-1 past the context): lane b of every wave
  // loads entry b with a vector load (a scalar load would share its wait
  // counter with the LDS reads of the compute), read out with readlane when
  // the chunk's loads are issued. They are requested a chunk ahead.
  int ids = -1, ph0, ph1, ph2, ph3;
  auto fetch_ids = [&](int n0) __attribute__((always_inline)) {
    ids = (lane < 4 && n0 + kBlock * lane < T) ? bt[n0 / kBlock + lane] : -1;
  };
  auto take_ids = [&]() __attribute__((always_inline)) {
    ph0 = __builtin_amdgcn_readlane(ids, 0);
    ph1 = __builtin_amdgcn_readlane(ids, 1);
    ph2 = __builtin_amdgcn_readlane(ids, 2);
    ph3 = __builtin_amdgcn_readlane(ids, 3);
  };
  auto block_of = [&](int b) __attribute__((always_inline)) {
    return b == 0 ? ph0 : (b == 1 ? ph1 : (b == 2 ? ph2 : ph3));
  };
  auto fetch = [&](int n0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kQK; ++j) {
      const int q = tid + kF32Threads * j, b = q / kF4Blk, f = 4 * (q % kF4Blk);
      const int p = block_of(b);
      const size_t base = ((size_t)(p < 0 ? 0 : p) * a.Hkv + h) * kBlock * D;
      // keys: f = slot * D + i (one token per piece); values: f = i * 16 + slot (4 tokens)
      rK[j] = (p >= 0 && n0 + kBlock * b + f / D < T) ? *reinterpret_cast<const float4*>(kb + base + f) : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 v = p >= 0 ? *reinterpret_cast<const float4*>(vb + base + f) : make_float4(0.f, 0.f, 0.f, 0.f);
      const int t0 = n0 + kBlock * b + f % kBlock;
      v.x = t0 < T ? v.x : 0.f;
      v.y = t0 + 1 < T ? v.y : 0.f;
      v.z = t0 + 2 < T ? v.z : 0.f;
      v.w = t0 + 3 < T ? v.w : 0.f;
      rV[j] = v;
    }
#pragma unroll
    for (int j = 0; j < kQL; ++j) {
      const int q = tid + kF32Threads * j;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q < kBlock * rk) {  // L_k block: [r/8][16][8], f = (k/8) * 128 + slot * 8 + k % 8
        const int b = q / (4 * rk), f = 4 * (q % (4 * rk));
        const int p = block_of(b), n = n0 + kBlock * b + (f % 128) / 8;
        if (p >= 0 && n < T && n >= act) x = *reinterpret_cast<const float4*>(lk + (size_t)p * kBlock * rk + f);
      }
      if (q < kBlock * rv) {  // L_v block: [r][16], f = k * 16 + slot
        const int b = q / (4 * rv), f = 4 * (q % (4 * rv));
        const int p = block_of(b), t0 = n0 + kBlock * b + f % kBlock;
        if (p >= 0) y = *reinterpret_cast<const float4*>(lv + (size_t)p * kBlock * rv + f);
        y.x = (t0 < T && t0 >= act) ? y.x : 0.f;
        y.y = (t0 + 1 < T && t0 + 1 >= act) ? y.y : 0.f;
        y.z = (t0 + 2 < T && t0 + 2 >= act) ? y.z : 0.f;
        y.w = (t0 + 3 < T && t0 + 3 >= act) ? y.w : 0.f;
      }
      rLk[j] = x;
      rLv[j] = y;
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kQK; ++j) {
      const int q = tid + kF32Threads * j, b = q / kF4Blk, f = 4 * (q % kF4Blk);
      const int t = kBlock * b + f / D, i = f % D;
      sK[t][i] = rK[j].x;
      sK[t][i + 1] = rK[j].y;
      sK[t][i + 2] = rK[j].z;
      sK[t][i + 3] = rK[j].w;
      const int iv = f / kBlock, tv = kBlock * b + f % kBlock;
      sV[iv][tv] = rV[j].x;
      sV[iv][tv + 1] = rV[j].y;
      sV[iv][tv + 2] = rV[j].z;
      sV[iv][tv + 3] = rV[j].w;
    }
#pragma unroll
    for (int j = 0; j < kQL; ++j) {
      const int q = tid + kF32Threads * j;
      if (q < kBlock * rk) {
        const int b = q / (4 * rk), f = 4 * (q % (4 * rk));
        const int t = kBlock * b + (f % 128) / 8, k = 8 * (f / 128) + f % 8;
        sLk[t][k] = rLk[j].x;
        sLk[t][k + 1] = rLk[j].y;
        sLk[t][k + 2] = rLk[j].z;
        sLk[t][k + 3] = rLk[j].w;
      }
      if (q < kBlock * rv) {
        const int b = q / (4 * rv), f = 4 * (q % (4 * rv));
        const int k = f / kBlock, t = kBlock * b + f % kBlock;
        sLv[k][t] = rLv[j].x;
        sLv[k][t + 1] = rLv[j].y;
        sLv[k][t + 2] = rLv[j].z;
        sLv[k][t + 3] = rLv[j].w;
      }
    }
  };

  constexpr int kAccPer = 16 * D / kF32Threads;  // (row, dim) pairs per thread
  float acc[kAccPer];
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) acc[i] = 0.f;
  float accC[4] = {0.f, 0.f, 0.f, 0.f};  // (row, k) pairs: 16 x 64 / 256

  // Without the rotary embedding the adapter score needs no rebuilt key:
  // q . (L_k[n] B_k) = L_k[n] . (B_k q), so u = B_k q is formed once per query
  // row and each token's adapter score is an r-long dot product with its
  // low-rank row (zero for tokens before the activation point).
  const bool fold = rk > 0 && !a.rope;
  fetch_ids(0);
  take_ids();
  fetch(0);
  fetch_ids(kChunk);
  if (fold) {
    __syncthreads();  // sQ and B_k are staged
    for (int e = tid; e < G * rk; e += kF32Threads) {
      const int row = e / rk, k = e % rk;
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D; i += 4)
#pragma unroll
        for (int j = 0; j < 4; ++j) d4[j] = fmaf(sQ[row][i + j], sB[k * D + i + j], d4[j]);
      sU[row][k] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
    }
  }
  for (int n0 = 0; n0 < T; n0 += kChunk) {
    __syncthreads();  // the previous chunk's LDS reads are done
    stage();
    __syncthreads();
    if (n0 + kChunk < T) {  // in flight during this chunk's compute
      take_ids();
      fetch(n0 + kChunk);
      fetch_ids(n0 + 2 * kChunk);
    }
    // rebuilt keys: K = K_base + rope_n(L_k B_k), pair (i, i + D/2) of token t
    if (rk && !fold) {
#pragma unroll 4
      for (int u = 0; u < kChunk * HALF / kF32Threads; ++u) {  // four pairs' reads in flight
        const int e = tid + kF32Threads * u;
        const int t = e / HALF, i = e % HALF;
        const int n = n0 + t;
        if (n >= T || n < act) continue;
        float x1 = 0.f, x2 = 0.f;
        for (int k0 = 0; k0 < rk; k0 += 8) {  // ranks are multiples of 8: eight reads in flight
#pragma unroll
          for (int k = k0; k < k0 + 8; ++k) {
            const float l = sLk[t][k];
            x1 = fmaf(l, sB[k * D + i], x1);
            x2 = fmaf(l, sB[k * D + i + HALF], x2);
          }
        }
        if (a.rope) {
          const double x = (double)n * sRev[i];
          const float f = (float)(x - __builtin_floor(x));
          const float c = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
          const float y1 = x1 * c - x2 * sn, y2 = x2 * c + x1 * sn;
          x1 = y1;
          x2 = y2;
        }
        sK[t][i] += x1;
        sK[t][i + HALF] += x2;
      }
      __syncthreads();
    }
    for (int e = tid; e < G * kChunk; e += kF32Threads) {
      const int row = e / kChunk, t = e % kChunk;
      float sc = -INFINITY;
      if (n0 + t < T) {
        float d4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent sums (short dependency chains)
#pragma unroll
        for (int i = 0; i < D; i += 4)
#pragma unroll
          for (int j = 0; j < 4; ++j) d4[j] = fmaf(sQ[row][i + j], sK[t][i + j], d4[j]);
        float dl = 0.f;
        if (fold)
          for (int k0 = 0; k0 < rk; k0 += 8)
#pragma unroll
            for (int k = k0; k < k0 + 8; ++k) dl = fmaf(sLk[t][k], sU[row][k], dl);
        sc = (((d4[0] + d4[1]) + (d4[2] + d4[3])) + dl) * a.sm_scale_log2;
      }
      sP[row][t] = sc;
    }
    __syncthreads();
    for (int row = wave; row < G; row += 4) {
      const float v = sP[row][lane];
      const float m_old = sM[row];
      const float m_new = fmaxf(m_old, wave_max64(v));
      const float p = exp2f(v - m_new);
      const float ps = wave_sum64(p);
      sP[row][lane] = p;
      if (lane == 0) {
        const float al = exp2f(m_old - m_new);
        sAlpha[row] = al;
        sL[row] = sL[row] * al + ps;
        sM[row] = m_new;
      }
    }
    __syncthreads();
    // O[row, i] += sum_t p V_base ;  C[row, k] += sum_t p L_v (tokens past the
    // context have p = 0 and zero rows)
#pragma unroll
    for (int u = 0; u < kAccPer; ++u) {
      const int e = tid + kF32Threads * u;
      const int row = e / D, i = e % D;
      if (row < G) {
        float v4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kChunk; t += 4)
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = fmaf(sP[row][t + j], sV[i][t + j], v4[j]);
        acc[u] = acc[u] * sAlpha[row] + ((v4[0] + v4[1]) + (v4[2] + v4[3]));
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kF32Threads * u;
      const int row = e / kMaxRankF32, k = e % kMaxRankF32;
      if (row < G && k < rv) {
        float v4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kChunk; t += 4)
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = fmaf(sP[row][t + j], sLv[k][t + j], v4[j]);
        accC[u] = accC[u] * sAlpha[row] + ((v4[0] + v4[1]) + (v4[2] + v4[3]));
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + kF32Threads * u;
    sC[e / kMaxRankF32][e % kMaxRankF32] = accC[u];
  }
  for (int e = tid; e < rv * D; e += kF32Threads) sB[e] = bv[(size_t)(e / D) * HD + h * D + e % D];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kAccPer; ++u) {
    const int e = tid + kF32Threads * u;
    const int row = e / D, i = e % D;
    if (row < G) {
      float v = acc[u];
      for (int k0 = 0; k0 < rv; k0 += 8)
#pragma unroll
        for (int k = k0; k < k0 + 8; ++k) v = fmaf(sC[row][k], sB[k * D + i], v);
      ((float*)a.out)[((size_t)s * a.Hq + h * G + row) * D + i] = v / sL[row];
    }
  }
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.S * a.Hkv), block(kF32Threads);
  if (a.d == 64)
    hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, stream, a);
  else if (a.d == 128)
    hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lra
