// Prefill attention over a shared-base + low-rank KV cache on gfx950 MFMA
// (bf16 inputs, fp32 accumulation): the kernel of the prefill call and its
// launch. The workgroup body, its design and its citations are in
// prefill_bf16_body.h.
#include "prefill_bf16_body.h"

namespace lra {
namespace {

// KAD / VAD: the call has key / value adapters; without one, that part of
// the work (low-rank loads, staging, rebuild or rank-space products) is not
// compiled in. A sequence without an agent (id -1) runs with rank 0: its
// low-rank loads read nothing and its staged B rows are zero.
template <int RP, bool KAD, bool VAD>
__global__ __launch_bounds__(pf::kThreads) void prefill_bf16_kernel(const PrefillArgs a) {
  using namespace pf;
  __shared__ __align__(16) uint16_t s_k[kKBufs][kTile * kKPitch];           // rebuilt keys [key][dim]
  __shared__ __align__(16) uint16_t s_v[kVBufs][D * kVPitch];               // V^T [dim][key]
  // rank space: L_v^T tiles [rank][key]; value rebuild: each wave's L_v rows [key][rank] (s_lvt)
  __shared__ __align__(16) uint16_t s_lv[kVBufs][VAD ? RP * kVPitch : 8];
  uint16_t* const s_lvt = &s_lv[0][0];
  static_assert(!value_rebuild(RP, KAD, VAD) || 8 * kBlock * (RP + 8) <= kVBufs * RP * kVPitch, "L_v rows fit");
  __shared__ __align__(16) uint16_t s_bt[KAD ? D * RP : 8];                 // B_k^T [dim][rank] (see tile_off)
  __shared__ __align__(16) uint16_t s_bvt[VAD ? D * RP : 8];                // B_v^T [dim][rank] (value rebuild: see tile_off)
  __shared__ __align__(16) float s_rot[kKBufs][2 * kMaxRopePairs];          // (cos, sin) of 64 t theta_i
  __shared__ double s_rev[kMaxRopePairs];
  const unsigned bid = blockIdx.x;
#include "prefill_bf16_body.inc"
}

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
  const dim3 grid(per * kNumXcd), block(pf::kThreads);
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
