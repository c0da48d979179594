// Decode attention over a shared-base + low-rank KV cache, bf16 in, fp32
// accumulate, on gfx950 MFMA: the kernels of the decode call (main and
// combine) and their launch. The workgroup's design and citations are in
// decode_bf16_body.h.
#include "decode_bf16_body.h"

namespace lra {
namespace {

using namespace dec;

// Main kernel: one workgroup of kDecodeWaves waves per (group, row tile,
// split, KV head). NA is a compile-time bound on the agents of a row tile
// (a tile with fewer runs with zero B_k / L rows for the missing ones).
// KAD / VAD: the call has key / value adapters; without one, that part of
// the work (its low-rank loads, staging and products) is not compiled in.
// ACT: the call passes activation positions (without them no position test
// is compiled in).
// Writes the split's record (m, l, seq, nact, O' per row), or the finished
// rows when the context fits one split.
// The leading scalar arguments repeat fields of `a` that the preamble reads
// first (DecodeHot), so they can be preloaded into SGPRs.
template <int RP, int NA, bool KAD, bool VAD, bool ACT>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_bf16_kernel(
    const int32_t* context_lens, const int32_t* block_tables, const int32_t* agent_ids, const int32_t* group_offsets,
    int n_work, int dims, int row_tiles, int split, int max_blocks, int S, const DecodeArgs a) {
  const DecodeHot hp =
      make_hot(context_lens, block_tables, agent_ids, group_offsets, n_work, dims, row_tiles, split, max_blocks, S);
  using C = Cfg<RP, NA, KAD, VAD>;
  constexpr int HW = C::HW;
  constexpr int kRegion = C::kRegion;
  // B_k^T [al][dim][k] in the loop (the merge buffer after it), then B_v^T
  // [al][dim][k], in one array: the largest, so it is placed first and the
  // adapter loop's B_k^T reads fit the 16-bit immediate offset of an LDS read
  constexpr int kBvtBytes = (VAD ? NA * D * RP : 8) * 2;
  __shared__ __align__(16) unsigned char s_lds0[kRegion + kBvtBytes];
  unsigned char* const s_region = s_lds0;
  uint16_t* const s_bvt = reinterpret_cast<uint16_t*>(s_lds0 + kRegion);
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

  const unsigned bid = blockIdx.x;
  {  // the included statements define their own compile-time sizes
#include "decode_bf16_body.inc"
  }
}

// Combine kernel: one wave per (group, row tile, KV head, row) merges the
// split records of that row with weights 2^(m_c - M) and writes the output.
// The record of split 0 says how many splits the row has (0: no such row;
// 1: finished by the main kernel). Lanes 0..31 take the even splits, lanes
// 32..63 the odd ones, 4 output dims per lane; every load goes out at once
// and loads past the records read zero through the buffer range check.
// MS: a bound on the split count (32 or 64), so a call with at most 32
// splits issues half the record loads.
template <int MS>
__global__ __launch_bounds__(64) void decode_bf16_combine(const DecodeArgs a) {
  static_assert(MS == 32 || MS == 64, "split bound");
  __shared__ float s_w[64];  // every lane writes its weight (zero past the splits)
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
  uint4 v[MS / 2];
#pragma unroll
  for (int u = 0; u < MS / 2; ++u) {
    const int c = 2 * u + half;
    v[u] = bld16(rs, c < a.nsplit ? (c * cstride + 4 + 4 * d4) * 4 : kOob);
  }
  const int nact = __builtin_amdgcn_readfirstlane((int)hu.w);
  const int seq = __builtin_amdgcn_readfirstlane((int)hu.z);
  if (nact <= 1) return;
  const bool okc = lane < nact;
  const float m_c = __uint_as_float(hu.x), l_c = __uint_as_float(hu.y);
  float M = okc ? m_c : -INFINITY;
  M = wave_max64(M);
  const float w = okc ? fast_exp2(m_c - M) : 0.f;
  float L = okc ? w * l_c : 0.f;
  L = wave_sum64(L);
  s_w[lane] = w;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < MS / 2; ++u) {
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

static_assert(kNumXcd == 8, "the work-item dealing assumes 8 XCDs");
int round_up8(int x) { return (x + 7) & ~7; }

template <int RP, int NA, bool KAD, bool VAD, bool ACT>
void launch_kernel(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_bf16_kernel<RP, NA, KAD, VAD, ACT>), grid, dim3(kDecodeWaves * 64), 0, stream,
                     a.context_lens, a.block_tables, a.agent_ids, a.group_offsets, a.n_work,
                     pack_hot_dims(a.nsplit, a.apt, a.Hkv), a.row_tiles, a.split, a.max_blocks, a.S, a);
}

template <int RP, int NA, bool KAD, bool VAD>
void launch_main(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (a.act)
    launch_kernel<RP, NA, KAD, VAD, true>(a, grid, stream);
  else
    launch_kernel<RP, NA, KAD, VAD, false>(a, grid, stream);
}

template <bool KAD, bool VAD>
bool launch_variant(const DecodeArgs& a, int rp, int na, dim3 grid, hipStream_t stream) {
  switch (rp * 100 + na) {
    case 1601: launch_main<16, 1, KAD, VAD>(a, grid, stream); return true;
    case 1602: launch_main<16, 2, KAD, VAD>(a, grid, stream); return true;
    case 1604: launch_main<16, 4, KAD, VAD>(a, grid, stream); return true;
    case 1608: launch_main<16, 8, KAD, VAD>(a, grid, stream); return true;
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
  // grid: with several groups and 8 or more splits, groups and splits padded
  // to multiples of 8 (dealt over the XCDs by the kernel); else
  // n_work rounded up to 8
  const int usz = a.row_tiles * a.Hkv;
  const int n_grid = (a.nsplit >= kNumXcd && a.num_groups > 1) ? round_up8(a.num_groups) * round_up8(a.nsplit) * usz
                                         : ((a.n_work + kNumXcd - 1) / kNumXcd) * kNumXcd;
  const dim3 grid(n_grid);
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
    launch_kernel<16, 1, false, false, false>(a, grid, stream);
    launched = true;
  }
  if (!launched) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit <= 1) return e;
  static_assert(kMaxSplits == 64, "combine variants cover up to 64 splits");
  if (a.nsplit <= 32)
    hipLaunchKernelGGL(decode_bf16_combine<32>, dim3(n_rows), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_bf16_combine<64>, dim3(n_rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// A serving step with decoding sequences and prefill chunks: the prefill
// kernel, then the decode kernels, on one stream. Each row is computed by the
// same kernel as in the separate calls, so it is bit-identical to them.
hipError_t launch_varlen_bf16(const DecodeArgs& d, int rp, int na, const PrefillArgs& p, hipStream_t stream) {
  if (p.S > 0) {
    const hipError_t e = launch_prefill_bf16(p, stream);
    if (e != hipSuccess) return e;
  }
  if (d.S > 0) return launch_decode_bf16(d, rp, na, stream);
  return hipSuccess;
}
#endif

}  // namespace lra
