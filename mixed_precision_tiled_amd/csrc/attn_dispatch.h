// Launch and instantiation dispatch of the attention kernels.
#pragma once

#include "attn_kernel.h"

namespace lamp {

template <int D, int NW, bool BF16, bool E4M3, bool AD, bool X8, bool PV8>
hipError_t launch_attn_one(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.Hq * a.n_qt));
  const dim3 block(NW * 64);
  if constexpr (!E4M3) {
    if (a.dbg != nullptr) {
      hipLaunchKernelGGL((attn_fwd_kernel<D, NW, BF16, E4M3, AD, X8, PV8, true>), grid, block, 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, BF16, E4M3, AD, X8, PV8, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

// the 8-bit P V product exists with 8-bit exponentials under mask routing
template <int D, int NW, bool BF16, bool E4M3, bool AD>
hipError_t dispatch_x8(const AttnArgs& a, const AttnConfig& c, hipStream_t s) {
  if (!c.exp8) return launch_attn_one<D, NW, BF16, E4M3, AD, false, false>(a, s);
  if constexpr (!AD) {
    if (c.pv8) return launch_attn_one<D, NW, BF16, E4M3, false, true, true>(a, s);
  }
  return launch_attn_one<D, NW, BF16, E4M3, AD, true, false>(a, s);
}
template <int D, int NW, bool BF16, bool E4M3>
hipError_t dispatch_ad(const AttnArgs& a, const AttnConfig& c, hipStream_t s) {
  return c.adaptive ? dispatch_x8<D, NW, BF16, E4M3, true>(a, c, s)
                    : dispatch_x8<D, NW, BF16, E4M3, false>(a, c, s);
}
template <int D, int NW, bool BF16>
hipError_t dispatch_code(const AttnArgs& a, const AttnConfig& c, hipStream_t s) {
  return c.e4m3 ? dispatch_ad<D, NW, BF16, true>(a, c, s) : dispatch_ad<D, NW, BF16, false>(a, c, s);
}
template <int D, int NW>
hipError_t dispatch_dtype(const AttnArgs& a, const AttnConfig& c, hipStream_t s) {
  return c.bf16 ? dispatch_code<D, NW, true>(a, c, s) : dispatch_code<D, NW, false>(a, c, s);
}

}  // namespace lamp
