// Instantiations of the dual-path attention kernel for head dim 128.
#include "attn_dispatch.h"

namespace lamp {

hipError_t launch_attn_d128(const AttnArgs& a, const AttnConfig& c, hipStream_t s) {
  return c.nw == 2 ? dispatch_dtype<128, 2>(a, c, s) : dispatch_dtype<128, 4>(a, c, s);
}

}  // namespace lamp
