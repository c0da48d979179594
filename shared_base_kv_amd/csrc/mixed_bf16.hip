// Decode rows and prefill chunks in one grid (bf16, gfx950): workgroups
// 0 .. n_pre - 1 run the prefill workgroup, the rest the decode workgroup,
// over one LDS buffer sized for the larger of the two. A CU holds one
// workgroup of either kind, so the prefill workgroups go first and the short
// decode workgroups fill the CUs that the causal prefill tiles free unevenly
// at the end. Both statement sets are
// the ones the separate calls run (decode_bf16_body.inc,
// prefill_bf16_body.inc), so each row's result is bit-identical to the
// separate call's. The decode rows' split records are merged by the decode
// combine kernel afterwards, as in the decode call.
//
// One launch serves a serving step that mixes decoding sequences with
// prefill chunks (chunked-prefill piggybacking: PReCache, Figure 1 caption,
// and the concurrent agent serving of LRAgent: Efficient KV Cache Sharing
// for Multi-LoRA LLM Agents, abstract); a decode workgroup waiting on its
// latency chains shares the machine with prefill workgroups busy on the
// matrix cores.
//
// The variants are built in three translation units (this file with
// LRA_MIXED_PART 0: both adapters, 1: value adapter only, 2: key adapter only
// and no adapter), so they compile in parallel.
#include "decode_bf16_body.h"
#include "prefill_bf16_body.h"

#ifndef LRA_MIXED_PART
#define LRA_MIXED_PART 0
#endif

namespace lra {
namespace {

template <int RP, int NA, bool KAD, bool VAD, bool ACT>
__global__ __launch_bounds__(kDecodeWaves * 64) void mixed_bf16_kernel(const DecodeArgs a_dec, const PrefillArgs a_pre,
                                                                      int n_pre_blocks) {
  static_assert(kDecodeWaves * 64 == pf::kThreads, "decode and prefill workgroups have the same size");
  using DL = dec::Lds<RP, NA, KAD, VAD>;
  using PL = pf::Lds<RP, KAD, VAD>;
  constexpr size_t kBytes = sizeof(DL) > sizeof(PL) ? sizeof(DL) : sizeof(PL);
  __shared__ __align__(16) unsigned char smem[kBytes];
  if ((int)blockIdx.x >= n_pre_blocks) {  // uniform over the workgroup
    using namespace dec;
    const DecodeArgs& a = a_dec;
    DL& lds = *reinterpret_cast<DL*>(smem);
    auto& s_region = lds.s_region;
    auto& s_bvt = lds.s_bvt;
    auto& s_q = lds.s_q;
    auto& s_qp = lds.s_qp;
    auto& s_roff = lds.s_roff;
    auto& s_rbase = lds.s_rbase;
    auto& s_rev = lds.s_rev;
    auto& s_agent = lds.s_agent;
    auto& s_ml = lds.s_ml;
    auto& s_shared_l = lds.s_shared_l;
    auto& s_lead = lds.s_lead;
    auto& s_start_min = lds.s_start_min;
    auto& s_start_max = lds.s_start_max;
    const unsigned bid = blockIdx.x - (unsigned)n_pre_blocks;
    {
#include "decode_bf16_body.inc"
    }
  } else {
    using namespace pf;
    const PrefillArgs& a = a_pre;
    PL& lds = *reinterpret_cast<PL*>(smem);
    auto& s_k = lds.s_k;
    auto& s_v = lds.s_v;
    auto& s_lv = lds.s_lv;
    auto& s_bt = lds.s_bt;
    auto& s_bvt = lds.s_bvt;
    auto& s_rot = lds.s_rot;
    auto& s_rev = lds.s_rev;
    const unsigned bid = blockIdx.x;
    {
#include "prefill_bf16_body.inc"
    }
  }
}

template <int RP, int NA, bool KAD, bool VAD>
void launch_main(const DecodeArgs& d, const PrefillArgs& p, int n_pre, dim3 grid, hipStream_t stream) {
  const dim3 block(kDecodeWaves * 64);
  if (d.act || p.act)
    hipLaunchKernelGGL((mixed_bf16_kernel<RP, NA, KAD, VAD, true>), grid, block, 0, stream, d, p, n_pre);
  else
    hipLaunchKernelGGL((mixed_bf16_kernel<RP, NA, KAD, VAD, false>), grid, block, 0, stream, d, p, n_pre);
}

template <bool KAD, bool VAD>
bool launch_variant(const DecodeArgs& d, const PrefillArgs& p, int rp, int na, int n_pre, dim3 grid,
                    hipStream_t stream) {
  switch (rp * 100 + na) {
    case 1601: launch_main<16, 1, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 1602: launch_main<16, 2, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 1604: launch_main<16, 4, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 1608: launch_main<16, 8, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 1616: launch_main<16, 16, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 3201: launch_main<32, 1, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 3202: launch_main<32, 2, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 3204: launch_main<32, 4, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 3208: launch_main<32, 8, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 6401: launch_main<64, 1, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 6402: launch_main<64, 2, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    case 6404: launch_main<64, 4, KAD, VAD>(d, p, n_pre, grid, stream); return true;
    default: return false;
  }
}

}  // namespace

#if LRA_MIXED_PART == 0
bool launch_mixed_bf16_kv(const DecodeArgs& d, const PrefillArgs& p, int rp, int na, int n_pre, dim3 grid,
                          hipStream_t stream) {
  return launch_variant<true, true>(d, p, rp, na, n_pre, grid, stream);
}
#elif LRA_MIXED_PART == 1
bool launch_mixed_bf16_v(const DecodeArgs& d, const PrefillArgs& p, int rp, int na, int n_pre, dim3 grid,
                         hipStream_t stream) {
  return launch_variant<false, true>(d, p, rp, na, n_pre, grid, stream);
}
#else
bool launch_mixed_bf16_k(const DecodeArgs& d, const PrefillArgs& p, int rp, int na, int n_pre, dim3 grid,
                         hipStream_t stream) {
  return launch_variant<true, false>(d, p, rp, na, n_pre, grid, stream);
}
bool launch_mixed_bf16_none(const DecodeArgs& d, const PrefillArgs& p, int n_pre, dim3 grid, hipStream_t stream) {
  // no adapter: one variant serves every tile width (no per-agent state)
  launch_main<16, 1, false, false>(d, p, n_pre, grid, stream);
  return true;
}
#endif

}  // namespace lra
