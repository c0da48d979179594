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
#include "device_common.h"
#include "internal.h"

namespace lra {
namespace {

constexpr int kChunk = 64;

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(const DecodeArgs a) {
  constexpr int HALF = D / 2;
  __shared__ float sK[kChunk][D + 1];
  __shared__ float sQ[16][D];
  __shared__ float sP[16][kChunk];
  __shared__ float sM[16], sL[16], sAlpha[16];
  __shared__ float sC[16][64];
  __shared__ int sPhys[kChunk / kBlock];
  __shared__ double sRev[kMaxRopePairs];

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
  const size_t blk_elems = (size_t)a.Hkv * kBlock * D;

  for (int e = tid; e < G * D; e += 256) {
    const int row = e / D, i = e % D;
    sQ[row][i] = ((const float*)a.q)[((size_t)s * a.Hq + h * G + row) * D + i];
  }
  if (tid < kMaxRopePairs) sRev[tid] = a.rope_rev[tid];
  if (tid < 16) {
    sM[tid] = -INFINITY;
    sL[tid] = 0.f;
  }
  constexpr int kAccPer = 16 * D / 256;  // (row, dim) pairs per thread
  float acc[kAccPer];
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) acc[i] = 0.f;
  float accC[4] = {0.f, 0.f, 0.f, 0.f};  // (row, k) pairs: 16 x 64 / 256

  for (int n0 = 0; n0 < T; n0 += kChunk) {
    __syncthreads();
    if (tid < kChunk / kBlock) sPhys[tid] = (n0 + tid * kBlock < T) ? bt[n0 / kBlock + tid] : 0;
    __syncthreads();
    // rebuilt keys of this chunk: K = K_base + rope_n(L_k B_k)
    for (int e = tid; e < kChunk * HALF; e += 256) {
      const int t = e / HALF, i = e % HALF;
      const int n = n0 + t;
      float k1 = 0.f, k2 = 0.f;
      if (n < T) {
        const int phys = sPhys[t / kBlock], slot = n % kBlock;
        float x1 = 0.f, x2 = 0.f;
        for (int k = 0; k < (n >= act ? rk : 0); ++k) {
          const float l = lk[(size_t)phys * kBlock * rk + ((k >> 3) * kBlock + slot) * 8 + (k & 7)];
          x1 = fmaf(l, bk[(size_t)k * HD + h * D + i], x1);
          x2 = fmaf(l, bk[(size_t)k * HD + h * D + i + HALF], x2);
        }
        if (a.rope && rk) {
          const double x = (double)n * sRev[i];
          const float f = (float)(x - __builtin_floor(x));
          const float c = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
          const float y1 = x1 * c - x2 * sn, y2 = x2 * c + x1 * sn;
          x1 = y1;
          x2 = y2;
        }
        const float* kp = kb + (size_t)phys * blk_elems + ((size_t)h * kBlock + slot) * D;
        k1 = kp[i] + x1;
        k2 = kp[i + HALF] + x2;
      }
      sK[t][i] = k1;
      sK[t][i + HALF] = k2;
    }
    __syncthreads();
    for (int e = tid; e < G * kChunk; e += 256) {
      const int row = e / kChunk, t = e % kChunk;
      float sc = -INFINITY;
      if (n0 + t < T) {
        float dot = 0.f;
        for (int i = 0; i < D; ++i) dot = fmaf(sQ[row][i], sK[t][i], dot);
        sc = dot * a.sm_scale_log2;
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
    // O[row, i] += sum_t p V_base ;  C[row, k] += sum_t p L_v
#pragma unroll
    for (int u = 0; u < kAccPer; ++u) {
      const int e = tid + 256 * u;
      const int row = e / D, i = e % D;
      if (row < G) {
        float v = acc[u] * sAlpha[row];
        for (int t = 0; t < kChunk && n0 + t < T; ++t) {
          const int phys = sPhys[t / kBlock];
          v = fmaf(sP[row][t], vb[(size_t)phys * blk_elems + ((size_t)h * D + i) * kBlock + t % kBlock], v);
        }
        acc[u] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      const int row = e / 64, k = e % 64;
      if (row < G && k < rv) {
        float v = accC[u] * sAlpha[row];
        for (int t = (act > n0 ? act - n0 : 0); t < kChunk && n0 + t < T; ++t) {
          const int phys = sPhys[t / kBlock];
          v = fmaf(sP[row][t], lv[((size_t)phys * rv + k) * kBlock + t % kBlock], v);
        }
        accC[u] = v;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + 256 * u;
    sC[e / 64][e % 64] = accC[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kAccPer; ++u) {
    const int e = tid + 256 * u;
    const int row = e / D, i = e % D;
    if (row < G) {
      float v = acc[u];
      for (int k = 0; k < rv; ++k) v = fmaf(sC[row][k], bv[(size_t)k * HD + h * D + i], v);
      ((float*)a.out)[((size_t)s * a.Hq + h * G + row) * D + i] = v / sL[row];
    }
  }
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.S * a.Hkv), block(256);
  if (a.d == 64)
    hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, stream, a);
  else if (a.d == 128)
    hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lra
