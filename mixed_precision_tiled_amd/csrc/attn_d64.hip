// Instantiations of the dual-path attention kernel for head dim 64.
#include "attn_dispatch.h"

namespace lamp {

hipError_t launch_attn_d64(const AttnArgs& a, const AttnConfig& c, hipStream_t s) {
  return c.nw == 2 ? dispatch_dtype<64, 2>(a, c, s) : dispatch_dtype<64, 4>(a, c, s);
}

}  // namespace lamp
