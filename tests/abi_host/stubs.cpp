// Stand-ins for the kernel launchers and the two HIP runtime calls the C ABI
// layer makes, so that the layer builds and runs on the host alone (under
// AddressSanitizer and UndefinedBehaviorSanitizer).  Each launcher records
// its arguments and reports success.
#include "record.h"

LaunchRecord g_rec;
alignas(256) char g_scratch[256];

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "hip error"; }

namespace lamp {

hipError_t launch_quantize(const QuantArgs& a, hipStream_t) { ++g_rec.n_quant; g_rec.quant = a; return hipSuccess; }
hipError_t launch_quantize_v(const VQuantArgs& a, hipStream_t) { ++g_rec.n_quant_v; g_rec.quant_v = a; return hipSuccess; }
hipError_t launch_exp8_table(uint8_t*, hipStream_t) { ++g_rec.n_exp8; return hipSuccess; }
hipError_t launch_build_mask(const MaskArgs& a, hipStream_t) { ++g_rec.n_mask; g_rec.mask = a; return hipSuccess; }
hipError_t launch_build_mask_template(const TemplateMaskArgs& a, hipStream_t) {
  ++g_rec.n_template;
  g_rec.tmpl = a;
  return hipSuccess;
}
static hipError_t attn(const AttnArgs& a, const AttnConfig& c, int d) {
  ++g_rec.n_attn;
  g_rec.attn = a;
  g_rec.attn_cfg = c;
  g_rec.attn_d = d;
  return hipSuccess;
}
hipError_t launch_attn_d64(const AttnArgs& a, const AttnConfig& c, hipStream_t) { return attn(a, c, 64); }
hipError_t launch_attn_d128(const AttnArgs& a, const AttnConfig& c, hipStream_t) { return attn(a, c, 128); }
hipError_t launch_attn_d256(const AttnArgs& a, const AttnConfig& c, hipStream_t) { return attn(a, c, 256); }
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) { ++g_rec.n_decode; g_rec.decode = a; return hipSuccess; }
hipError_t decode_scratch(void** ptr) {
  ++g_rec.n_scratch;
  *ptr = g_scratch;
  return hipSuccess;
}

}  // namespace lamp
