// C ABI of the mixed-precision tiled attention library: argument validation,
// instantiation choice, launch on the caller's stream.  No allocation, no
// synchronisation; the only state is a thread-local error string.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "../../include/lamp.h"
#include "lamp_internal.h"

namespace {

thread_local char g_err[512] = "";

lamp_status fail(lamp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

lamp_status ok() {
  g_err[0] = '\0';
  return LAMP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool is16(int32_t t) { return t == LAMP_F16 || t == LAMP_BF16; }
bool is8(int32_t t) { return t == LAMP_I8 || t == LAMP_E4M3; }
bool supported_d(int64_t d) { return d == 64 || d == 128 || d == 256; }

constexpr int64_t kMaxSeq = 1 << 20;   // keeps every in-kernel row index in int32
constexpr int64_t kMaxGrid = (1ll << 31) - 1;

// Whether the product of the (non-negative) factors exceeds lim, without
// forming a product that could overflow int64.
bool product_exceeds(std::initializer_list<int64_t> factors, int64_t lim) {
  for (int64_t f : factors)
    if (f == 0) return false;
  int64_t prod = 1;
  for (int64_t f : factors) {
    if (prod > lim / f) return true;
    prod *= f;
  }
  return prod > lim;
}

lamp_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LAMP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* lamp_status_string(lamp_status s) {
  switch (s) {
    case LAMP_OK: return "LAMP_OK";
    case LAMP_ERR_NULL: return "LAMP_ERR_NULL";
    case LAMP_ERR_SHAPE: return "LAMP_ERR_SHAPE";
    case LAMP_ERR_UNSUPPORTED: return "LAMP_ERR_UNSUPPORTED";
    case LAMP_ERR_ALIGN: return "LAMP_ERR_ALIGN";
    case LAMP_ERR_HIP: return "LAMP_ERR_HIP";
  }
  return "LAMP_ERR_UNKNOWN";
}

const char* lamp_last_error(void) { return g_err; }

int32_t lamp_abi_version(void) { return LAMP_ABI_VERSION; }

lamp_status lamp_quantize_blocks(const void* x, int32_t x_dtype, int64_t B, int64_t H, int64_t S,
                                 int64_t D, int64_t sb, int64_t sh, int64_t ss,
                                 int32_t block_rows, int32_t code_dtype, void* codes,
                                 float* scales, void* stream) {
  return lamp_quantize_blocks_varlen(x, x_dtype, B, H, S, D, sb, sh, ss, nullptr, block_rows,
                                     code_dtype, codes, scales, stream);
}

lamp_status lamp_quantize_blocks_varlen(const void* x, int32_t x_dtype, int64_t B, int64_t H,
                                        int64_t S, int64_t D, int64_t sb, int64_t sh,
                                        int64_t ss, const int32_t* seqlens, int32_t block_rows,
                                        int32_t code_dtype, void* codes, float* scales,
                                        void* stream) {
  if (B < 0 || H < 0 || S < 0 || D < 0) return fail(LAMP_ERR_SHAPE, "negative size");
  if (sb < 0 || sh < 0 || ss < 0) return fail(LAMP_ERR_SHAPE, "negative stride");
  if (!is16(x_dtype)) return fail(LAMP_ERR_UNSUPPORTED, "x_dtype must be LAMP_F16 or LAMP_BF16");
  if (!is8(code_dtype)) return fail(LAMP_ERR_UNSUPPORTED, "code_dtype must be LAMP_I8 or LAMP_E4M3");
  if (!supported_d(D)) return fail(LAMP_ERR_UNSUPPORTED, "D=%lld not in {64,128,256}", (long long)D);
  if (block_rows < 1 || block_rows > 256)
    return fail(LAMP_ERR_UNSUPPORTED, "block_rows=%d not in [1, 256]", block_rows);
  if (S > kMaxSeq) return fail(LAMP_ERR_UNSUPPORTED, "S=%lld above %lld", (long long)S, (long long)kMaxSeq);
  if (B == 0 || H == 0 || S == 0) return ok();
  if (!x || !codes || !scales) return fail(LAMP_ERR_NULL, "x, codes and scales are required");
  if (ss < D) return fail(LAMP_ERR_SHAPE, "row stride %lld < D", (long long)ss);
  if (!aligned16(x) || !aligned16(codes) || (ss % 8) || (sh % 8) || (sb % 8))
    return fail(LAMP_ERR_ALIGN, "x, codes need 16-byte alignment and strides a multiple of 8");
  if (reinterpret_cast<uintptr_t>(seqlens) & 3u) return fail(LAMP_ERR_ALIGN, "seqlens needs 4-byte alignment");
  const int64_t nb = cdiv(S, block_rows);
  if (product_exceeds({B, H, nb}, kMaxGrid)) return fail(LAMP_ERR_UNSUPPORTED, "too many blocks");
  lamp::QuantArgs a{};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.sb = sb;
  a.sh = sh;
  a.ss = ss;
  a.B = (int32_t)B;
  a.H = (int32_t)H;
  a.S = (int32_t)S;
  a.D = (int32_t)D;
  a.block_rows = block_rows;
  a.nb = (int32_t)nb;
  a.chunk_shift = D == 64 ? 3 : D == 128 ? 4 : 5;    // log2(D / 8), D in {64, 128, 256}
  a.seqlens = seqlens;
  a.bf16 = x_dtype == LAMP_BF16;
  a.e4m3 = code_dtype == LAMP_E4M3;
  return hip_status(lamp::launch_quantize(a, static_cast<hipStream_t>(stream)), "quantize launch");
}

lamp_status lamp_exp8_table(uint8_t* table, void* stream) {
  if (!table) return fail(LAMP_ERR_NULL, "table is required");
  return hip_status(lamp::launch_exp8_table(table, static_cast<hipStream_t>(stream)), "exp8 table launch");
}

lamp_status lamp_quantize_v_tiles(const void* v, int32_t v_dtype, int64_t B, int64_t H, int64_t S,
                                  int64_t D, int64_t sb, int64_t sh, int64_t ss,
                                  const int32_t* seqlens, void* codes, float* scales,
                                  void* stream) {
  if (B < 0 || H < 0 || S < 0 || D < 0) return fail(LAMP_ERR_SHAPE, "negative size");
  if (sb < 0 || sh < 0 || ss < 0) return fail(LAMP_ERR_SHAPE, "negative stride");
  if (!is16(v_dtype)) return fail(LAMP_ERR_UNSUPPORTED, "v_dtype must be LAMP_F16 or LAMP_BF16");
  if (!supported_d(D)) return fail(LAMP_ERR_UNSUPPORTED, "D=%lld not in {64,128,256}", (long long)D);
  if (S > kMaxSeq) return fail(LAMP_ERR_UNSUPPORTED, "S=%lld above %lld", (long long)S, (long long)kMaxSeq);
  if (B == 0 || H == 0 || S == 0) return ok();
  if (!v || !codes || !scales) return fail(LAMP_ERR_NULL, "v, codes and scales are required");
  if (ss < D) return fail(LAMP_ERR_SHAPE, "row stride %lld < D", (long long)ss);
  if (!aligned16(v) || !aligned16(codes) || (ss % 8) || (sh % 8) || (sb % 8))
    return fail(LAMP_ERR_ALIGN, "v, codes need 16-byte alignment and strides a multiple of 8");
  if (reinterpret_cast<uintptr_t>(seqlens) & 3u) return fail(LAMP_ERR_ALIGN, "seqlens needs 4-byte alignment");
  const int64_t n_kt = cdiv(S, 64);
  if (product_exceeds({B, H, n_kt}, kMaxGrid)) return fail(LAMP_ERR_UNSUPPORTED, "too many tiles");
  lamp::VQuantArgs a{};
  a.v = v;
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = scales;
  a.sb = sb;
  a.sh = sh;
  a.ss = ss;
  a.B = (int32_t)B;
  a.H = (int32_t)H;
  a.S = (int32_t)S;
  a.D = (int32_t)D;
  a.n_kt = (int32_t)n_kt;
  a.seqlens = seqlens;
  a.bf16 = v_dtype == LAMP_BF16;
  return hip_status(lamp::launch_quantize_v(a, static_cast<hipStream_t>(stream)), "V quantize launch");
}

}  // extern "C"

namespace {
// floor(f * 2^32) in double, exact for every double f in [0, 1]
uint64_t frac_threshold(double f) { return (uint64_t)std::floor(f * 4294967296.0); }

lamp_status build_mask_common(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k, int32_t tile_m,
                              int32_t tile_n, int32_t tiles_per_bit, double frac_16bit,
                              const double* frac_per_head, uint64_t seed, uint64_t* mask,
                              int32_t words_per_row, void* stream) {
  if (B < 0 || Hq < 0 || S_q < 0 || S_k < 0) return fail(LAMP_ERR_SHAPE, "negative size");
  if (tile_m <= 0 || tile_n <= 0 || tiles_per_bit <= 0)
    return fail(LAMP_ERR_SHAPE, "tile sizes and tiles_per_bit must be positive");
  if (frac_per_head) {
    if (Hq > lamp::kMaskMaxHeads)
      return fail(LAMP_ERR_UNSUPPORTED, "per-head fractions for Hq=%lld > %d heads", (long long)Hq,
                  lamp::kMaskMaxHeads);
    for (int64_t h = 0; h < Hq; ++h) {
      if (!(frac_per_head[h] >= 0.0 && frac_per_head[h] <= 1.0))
        return fail(LAMP_ERR_SHAPE, "frac_16bit[%lld] must lie in [0, 1]", (long long)h);
    }
  } else if (!(frac_16bit >= 0.0 && frac_16bit <= 1.0)) {
    return fail(LAMP_ERR_SHAPE, "frac_16bit must lie in [0, 1]");
  }
  if (S_q > kMaxSeq || S_k > kMaxSeq) return fail(LAMP_ERR_UNSUPPORTED, "sequence too long");
  const int64_t n_qt = cdiv(S_q, tile_m), n_kt = cdiv(S_k, tile_n);
  const int64_t n_g = cdiv(n_kt, tiles_per_bit);
  if (words_per_row < cdiv(n_g, 64) || words_per_row < 1)
    return fail(LAMP_ERR_UNSUPPORTED, "words_per_row=%d < ceil(n_g/64)=%lld", words_per_row,
                (long long)cdiv(n_g, 64));
  if (B == 0 || Hq == 0 || S_q == 0) return ok();
  if (!mask) return fail(LAMP_ERR_NULL, "mask is required");
  if (reinterpret_cast<uintptr_t>(mask) & 7u) return fail(LAMP_ERR_ALIGN, "mask needs 8-byte alignment");
  if (product_exceeds({B, Hq, n_qt, words_per_row}, kMaxGrid * lamp::kMaskWordsPerBlock))
    return fail(LAMP_ERR_UNSUPPORTED, "mask too large");
  lamp::MaskArgs a{};
  a.mask = mask;
  a.total_words = B * Hq * n_qt * words_per_row;
  a.seed = seed;
  a.threshold = frac_per_head ? 0 : frac_threshold(frac_16bit);
  a.words_per_row = words_per_row;
  a.n_g = (int32_t)n_g;
  a.per_head = frac_per_head ? 1 : 0;
  a.Hq = (int32_t)Hq;
  a.n_qt = (int32_t)n_qt;
  if (frac_per_head) {
    for (int64_t h = 0; h < Hq; ++h) a.head_threshold[h] = frac_threshold(frac_per_head[h]);
  }
  return hip_status(lamp::launch_build_mask(a, static_cast<hipStream_t>(stream)), "mask launch");
}
}  // namespace

extern "C" {

lamp_status lamp_build_mask(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k, int32_t tile_m,
                            int32_t tile_n, int32_t tiles_per_bit, double frac_16bit,
                            uint64_t seed, uint64_t* mask, int32_t words_per_row,
                            void* stream) {
  return build_mask_common(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, frac_16bit, nullptr,
                           seed, mask, words_per_row, stream);
}

lamp_status lamp_build_mask_per_head(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k,
                                     int32_t tile_m, int32_t tile_n, int32_t tiles_per_bit,
                                     const double* frac_16bit, uint64_t seed, uint64_t* mask,
                                     int32_t words_per_row, void* stream) {
  if (!frac_16bit && Hq > 0) return fail(LAMP_ERR_NULL, "frac_16bit is required");
  return build_mask_common(B, Hq, S_q, S_k, tile_m, tile_n, tiles_per_bit, 0.0, frac_16bit, seed,
                           mask, words_per_row, stream);
}

lamp_status lamp_build_mask_template(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k,
                                     int32_t tile_m, int32_t tile_n, int32_t tiles_per_bit,
                                     int32_t sink_groups, int32_t band_groups,
                                     int32_t stride_groups, uint64_t* mask,
                                     int32_t words_per_row, void* stream) {
  if (B < 0 || Hq < 0 || S_q < 0 || S_k < 0) return fail(LAMP_ERR_SHAPE, "negative size");
  if (tile_m <= 0 || tile_n <= 0 || tiles_per_bit <= 0)
    return fail(LAMP_ERR_SHAPE, "tile sizes and tiles_per_bit must be positive");
  if (sink_groups < 0 || band_groups < 0 || stride_groups < 0)
    return fail(LAMP_ERR_SHAPE, "template parameters must be >= 0");
  if ((int64_t)tiles_per_bit * tile_n > INT32_MAX)
    return fail(LAMP_ERR_UNSUPPORTED, "tiles_per_bit * tile_n too large");
  if (S_q > kMaxSeq || S_k > kMaxSeq) return fail(LAMP_ERR_UNSUPPORTED, "sequence too long");
  const int64_t n_qt = cdiv(S_q, tile_m), n_kt = cdiv(S_k, tile_n);
  const int64_t n_g = cdiv(n_kt, tiles_per_bit);
  if (words_per_row < cdiv(n_g, 64) || words_per_row < 1)
    return fail(LAMP_ERR_UNSUPPORTED, "words_per_row=%d < ceil(n_g/64)=%lld", words_per_row,
                (long long)cdiv(n_g, 64));
  if (B == 0 || Hq == 0 || S_q == 0) return ok();
  if (!mask) return fail(LAMP_ERR_NULL, "mask is required");
  if (reinterpret_cast<uintptr_t>(mask) & 7u) return fail(LAMP_ERR_ALIGN, "mask needs 8-byte alignment");
  if (product_exceeds({B, Hq, n_qt, words_per_row}, kMaxGrid * 256))
    return fail(LAMP_ERR_UNSUPPORTED, "mask too large");
  lamp::TemplateMaskArgs a{};
  a.mask = mask;
  a.total_words = B * Hq * n_qt * words_per_row;
  a.words_per_row = words_per_row;
  a.n_g = (int32_t)n_g;
  a.n_qt = (int32_t)n_qt;
  a.tile_m = tile_m;
  a.group_keys = tiles_per_bit * tile_n;
  a.pos_off = S_k - S_q;
  a.sink = sink_groups;
  a.band = band_groups;
  a.stride = stride_groups;
  return hip_status(lamp::launch_build_mask_template(a, static_cast<hipStream_t>(stream)),
                    "template mask launch");
}

lamp_status lamp_attn_fwd(const lamp_attn_params* p, void* stream) {
  if (!p) return fail(LAMP_ERR_NULL, "params is NULL");
  if (p->struct_size != sizeof(lamp_attn_params))
    return fail(LAMP_ERR_UNSUPPORTED, "struct_size %u != %zu (ABI mismatch)", p->struct_size,
                sizeof(lamp_attn_params));
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 0 || p->S_q < 0 || p->S_k < 0 || p->D < 0)
    return fail(LAMP_ERR_SHAPE, "negative size");
  for (int i = 0; i < 3; ++i) {
    if (p->q_str[i] < 0 || p->k_str[i] < 0 || p->v_str[i] < 0 || p->o_str[i] < 0)
      return fail(LAMP_ERR_SHAPE, "negative stride");
  }
  if (p->mode != LAMP_MODE_MASK && p->mode != LAMP_MODE_ADAPTIVE)
    return fail(LAMP_ERR_UNSUPPORTED, "mode %d", p->mode);
  if (!is16(p->in_dtype)) return fail(LAMP_ERR_UNSUPPORTED, "in_dtype must be LAMP_F16 or LAMP_BF16");
  if (!is8(p->code_dtype)) return fail(LAMP_ERR_UNSUPPORTED, "code_dtype must be LAMP_I8 or LAMP_E4M3");
  if (!supported_d(p->D)) return fail(LAMP_ERR_UNSUPPORTED, "D=%lld not in {64,128,256}", (long long)p->D);
  if (p->tile_m != 64 && p->tile_m != 128) return fail(LAMP_ERR_UNSUPPORTED, "tile_m must be 64 or 128");
  if (p->tile_n != 64) return fail(LAMP_ERR_UNSUPPORTED, "tile_n must be 64");
  if (p->tiles_per_bit < 1) return fail(LAMP_ERR_SHAPE, "tiles_per_bit must be >= 1");
  if (p->Hkv == 0 || p->Hq % p->Hkv != 0)
    return fail(LAMP_ERR_UNSUPPORTED, "Hq=%lld must be a positive multiple of Hkv=%lld",
                (long long)p->Hq, (long long)p->Hkv);
  if (p->causal != 0 && p->causal != 1) return fail(LAMP_ERR_SHAPE, "causal must be 0 or 1");
  if (p->causal && p->S_q > p->S_k) return fail(LAMP_ERR_UNSUPPORTED, "causal needs S_q <= S_k");
  if (p->exp8 != 0 && p->exp8 != 1) return fail(LAMP_ERR_SHAPE, "exp8 must be 0 or 1");
  if (p->pv8 != 0 && p->pv8 != 1) return fail(LAMP_ERR_SHAPE, "pv8 must be 0 or 1");
  if (p->pv8 && (!p->exp8 || p->mode != LAMP_MODE_MASK))
    return fail(LAMP_ERR_UNSUPPORTED, "pv8 needs exp8 = 1 and LAMP_MODE_MASK");
  if (p->mode == LAMP_MODE_ADAPTIVE) {
    if (p->sub_rows != 32) return fail(LAMP_ERR_UNSUPPORTED, "sub_rows must be 32");
    if (std::isnan(p->tau)) return fail(LAMP_ERR_SHAPE, "tau is NaN");
  }
  if (std::isnan(p->sm_scale)) return fail(LAMP_ERR_SHAPE, "sm_scale is NaN");
  if (p->S_q > kMaxSeq || p->S_k > kMaxSeq) return fail(LAMP_ERR_UNSUPPORTED, "sequence too long");
  const int64_t n_qt = cdiv(p->S_q, p->tile_m), n_kt = cdiv(p->S_k, p->tile_n);
  const int64_t n_g = cdiv(n_kt, p->tiles_per_bit);
  if (p->words_per_row < cdiv(n_g, 64) || p->words_per_row < 1)
    return fail(LAMP_ERR_UNSUPPORTED, "words_per_row=%d < ceil(n_g/64)=%lld", p->words_per_row,
                (long long)cdiv(n_g, 64));
  if (p->dbg_qk_acc && p->code_dtype != LAMP_I8)
    return fail(LAMP_ERR_UNSUPPORTED, "dbg_qk_acc exists on the int8 path only");
  if (p->B == 0 || p->Hq == 0 || p->S_q == 0) return ok();
  if (p->S_k == 0) return fail(LAMP_ERR_SHAPE, "S_k == 0 with S_q > 0: softmax over no keys");
  if (!p->q || !p->k || !p->v || !p->q8 || !p->k8 || !p->q_scale || !p->k_scale || !p->mask ||
      !p->out)
    return fail(LAMP_ERR_NULL, "q, k, v, q8, k8, q_scale, k_scale, mask and out are required");
  const int64_t D = p->D;
  if (p->q_str[2] < D || p->k_str[2] < D || p->v_str[2] < D || p->o_str[2] < D)
    return fail(LAMP_ERR_SHAPE, "row stride < D");
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->out) ||
      !aligned16(p->q8) || !aligned16(p->k8))
    return fail(LAMP_ERR_ALIGN, "q, k, v, out, q8, k8 need 16-byte alignment");
  for (int i = 0; i < 3; ++i) {
    if ((p->q_str[i] | p->k_str[i] | p->v_str[i] | p->o_str[i]) % 8)
      return fail(LAMP_ERR_ALIGN, "strides must be multiples of 8 elements");
  }
  if (reinterpret_cast<uintptr_t>(p->mask) & 7u) return fail(LAMP_ERR_ALIGN, "mask alignment");
  if ((reinterpret_cast<uintptr_t>(p->seqlens_q) | reinterpret_cast<uintptr_t>(p->seqlens_k)) & 3u)
    return fail(LAMP_ERR_ALIGN, "seqlens need 4-byte alignment");
  if (p->flags_out && (reinterpret_cast<uintptr_t>(p->flags_out) & 7u))
    return fail(LAMP_ERR_ALIGN, "flags_out alignment");
  if (p->pv8) {
    if (!p->v8 || !p->v_scale) return fail(LAMP_ERR_NULL, "pv8 needs v8 and v_scale");
    if (!aligned16(p->v8)) return fail(LAMP_ERR_ALIGN, "v8 needs 16-byte alignment");
    if (reinterpret_cast<uintptr_t>(p->v_scale) & 3u) return fail(LAMP_ERR_ALIGN, "v_scale alignment");
  }
  if (product_exceeds({p->B, p->Hq, n_qt}, kMaxGrid)) return fail(LAMP_ERR_UNSUPPORTED, "grid too large");
  // K and V rows of one head are addressed with 32-bit byte offsets
  if (product_exceeds({2, p->S_k, p->k_str[2]}, kMaxGrid) ||
      product_exceeds({2, p->S_k, p->v_str[2]}, kMaxGrid))
    return fail(LAMP_ERR_UNSUPPORTED, "K/V rows of one head span 2 GiB or more");

  lamp::AttnArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.q8 = static_cast<const uint8_t*>(p->q8);
  a.k8 = static_cast<const uint8_t*>(p->k8);
  a.q_scale = p->q_scale;
  a.k_scale = p->k_scale;
  a.mask = p->mask;
  a.out = p->out;
  a.lse = p->lse;
  a.flags = p->mode == LAMP_MODE_ADAPTIVE ? p->flags_out : nullptr;
  a.dbg = p->dbg_qk_acc;
  a.seqlens_q = p->seqlens_q;
  a.seqlens_k = p->seqlens_k;
  a.v8 = p->pv8 ? static_cast<const uint8_t*>(p->v8) : nullptr;
  a.v_scale = p->pv8 ? p->v_scale : nullptr;
  a.q_sb = p->q_str[0];
  a.q_sh = p->q_str[1];
  a.q_ss = p->q_str[2];
  a.k_sb = p->k_str[0];
  a.k_sh = p->k_str[1];
  a.k_ss = p->k_str[2];
  a.v_sb = p->v_str[0];
  a.v_sh = p->v_str[1];
  a.v_ss = p->v_str[2];
  a.o_sb = p->o_str[0];
  a.o_sh = p->o_str[1];
  a.o_ss = p->o_str[2];
  a.B = (int32_t)p->B;
  a.Hq = (int32_t)p->Hq;
  a.Hkv = (int32_t)p->Hkv;
  a.S_q = (int32_t)p->S_q;
  a.S_k = (int32_t)p->S_k;
  a.n_qt = (int32_t)n_qt;
  a.n_kt = (int32_t)n_kt;
  a.tiles_per_bit = p->tiles_per_bit;
  a.words_per_row = p->words_per_row;
  a.heads_per_group = (int32_t)(p->Hq / p->Hkv);
  a.n_sb = (int32_t)cdiv(p->S_q, 32);
  a.flag_words = (int32_t)cdiv(n_kt, 64);
  a.causal = p->causal;
  a.sm_scale = p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / std::sqrt((double)D));
  a.tau = p->tau;

  lamp::AttnConfig c{};
  c.d = (int)D;
  c.nw = p->tile_m / 32;
  c.bf16 = p->in_dtype == LAMP_BF16;
  c.e4m3 = p->code_dtype == LAMP_E4M3;
  c.adaptive = p->mode == LAMP_MODE_ADAPTIVE;
  c.exp8 = p->exp8 != 0;
  c.pv8 = p->pv8 != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (c.d) {
    case 64: e = lamp::launch_attn_d64(a, c, s); break;
    case 128: e = lamp::launch_attn_d128(a, c, s); break;
    default: e = lamp::launch_attn_d256(a, c, s); break;
  }
  return hip_status(e, "attention launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// decode over an int8 key/value cache
// ---------------------------------------------------------------------------

extern "C" {

size_t lamp_decode_workspace_bytes(int64_t B, int64_t Hkv, int64_t S_k, int64_t D) {
  if (B < 0 || Hkv < 0 || S_k < 0 || D < 0) return 0;
  // sizes no launch accepts: a byte count no workspace can meet
  if (S_k > kMaxSeq || D > 256 || product_exceeds({B, Hkv}, kMaxGrid)) return SIZE_MAX;
  const int64_t n_kt = cdiv(S_k, 64);
  const int64_t n_split = cdiv(n_kt, lamp::decode_tiles_per_split(B, Hkv, n_kt));
  return (size_t)(B * Hkv * n_split * 32 * (D + 2) * (int64_t)sizeof(float));
}

// Validates p and fills a; the partials go to `workspace` (at least
// lamp_decode_workspace_bytes bytes, checked by the callers).  With
// need_ws false the workspace is not checked (the fixed scratch is put in
// place afterwards).
static lamp_status decode_prepare(const lamp_decode_params* p, void* workspace, bool need_ws,
                                  lamp::DecodeArgs* out_args, bool* empty) {
  *empty = false;
  if (!p) return fail(LAMP_ERR_NULL, "params is NULL");
  if (p->struct_size != sizeof(lamp_decode_params))
    return fail(LAMP_ERR_UNSUPPORTED, "struct_size %u != %zu (ABI mismatch)", p->struct_size,
                sizeof(lamp_decode_params));
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 0 || p->S_q < 0 || p->S_k < 0 || p->D < 0)
    return fail(LAMP_ERR_SHAPE, "negative size");
  if (p->causal != 0 && p->causal != 1) return fail(LAMP_ERR_SHAPE, "causal must be 0 or 1");
  if (p->D != 64 && p->D != 128) return fail(LAMP_ERR_UNSUPPORTED, "decode supports D in {64,128}");
  if (!is16(p->out_dtype)) return fail(LAMP_ERR_UNSUPPORTED, "out_dtype must be LAMP_F16 or LAMP_BF16");
  if (p->Hkv == 0 || p->Hq % p->Hkv) return fail(LAMP_ERR_UNSUPPORTED, "Hq must be a multiple of Hkv >= 1");
  if (product_exceeds({p->Hq / p->Hkv, p->S_q}, 32))
    return fail(LAMP_ERR_UNSUPPORTED, "(Hq/Hkv) * S_q above 32");
  if (p->tile_m < 1) return fail(LAMP_ERR_SHAPE, "tile_m must be positive");
  if (p->causal && p->S_q > p->S_k) return fail(LAMP_ERR_UNSUPPORTED, "causal needs S_q <= S_k");
  if (p->S_k > kMaxSeq) return fail(LAMP_ERR_UNSUPPORTED, "S_k above %lld", (long long)kMaxSeq);
  if (p->B == 0 || p->Hq == 0 || p->S_q == 0) {
    *empty = true;
    return ok();
  }
  if (p->S_k == 0) return fail(LAMP_ERR_SHAPE, "S_k == 0 with queries");
  // (before any size is narrowed to 32 bits: B * Hq bounds every one)
  if (product_exceeds({p->B, p->Hq}, kMaxGrid)) return fail(LAMP_ERR_UNSUPPORTED, "grid too large");
  if (!p->q8 || !p->q_scale || !p->k8 || !p->k_scale || !p->v8 || !p->v_scale || !p->out ||
      (need_ws && !workspace))
    return fail(LAMP_ERR_NULL, "q8, k8, v8, their scales, out and workspace are required");
  if (!aligned16(p->q8) || !aligned16(p->k8) || !aligned16(p->v8) || (need_ws && !aligned16(workspace)))
    return fail(LAMP_ERR_ALIGN, "codes and workspace need 16-byte alignment");
  if (((reinterpret_cast<uintptr_t>(p->out)) & 1u) ||
      ((reinterpret_cast<uintptr_t>(p->q_scale) | reinterpret_cast<uintptr_t>(p->k_scale) |
        reinterpret_cast<uintptr_t>(p->v_scale) | reinterpret_cast<uintptr_t>(p->lse)) & 3u))
    return fail(LAMP_ERR_ALIGN, "out, scales and lse need their element alignment");
  for (int i = 0; i < 3; ++i)
    if (p->o_str[i] < 0) return fail(LAMP_ERR_SHAPE, "negative output stride");
  lamp::DecodeArgs a{};
  a.q8 = static_cast<const uint8_t*>(p->q8);
  a.q_scale = p->q_scale;
  a.k8 = static_cast<const uint8_t*>(p->k8);
  a.k_scale = p->k_scale;
  a.v8 = static_cast<const uint8_t*>(p->v8);
  a.v_scale = p->v_scale;
  a.out = p->out;
  a.lse = p->lse;
  a.B = (int32_t)p->B;
  a.Hq = (int32_t)p->Hq;
  a.Hkv = (int32_t)p->Hkv;
  a.S_q = (int32_t)p->S_q;
  a.S_k = (int32_t)p->S_k;
  a.D = (int32_t)p->D;
  a.hpg = (int32_t)(p->Hq / p->Hkv);
  a.cols = a.hpg * a.S_q;
  a.tile_m = p->tile_m;
  a.n_qt = (int32_t)cdiv(p->S_q, p->tile_m);
  a.n_kt = (int32_t)cdiv(p->S_k, 64);
  a.tiles_per_split = lamp::decode_tiles_per_split(a.B, a.Hkv, a.n_kt);
  a.n_split = (int32_t)cdiv(a.n_kt, a.tiles_per_split);
  if ((int64_t)a.B * a.Hkv * a.n_split > kMaxGrid || a.n_split > lamp::kMergeMaxSplit)
    return fail(LAMP_ERR_UNSUPPORTED, "grid too large");
  a.o_sb = p->o_str[0];
  a.o_sh = p->o_str[1];
  a.o_ss = p->o_str[2];
  a.causal = p->causal;
  a.sm_scale = p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / std::sqrt((double)p->D));
  a.bf16 = p->out_dtype == LAMP_BF16;
  if (workspace != nullptr) {
    const int64_t nslot = (int64_t)a.B * a.Hkv * a.n_split * 32;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = a.ws_o + nslot * a.D;
  }
  *out_args = a;
  return ok();
}

lamp_status lamp_decode_fwd_noalloc(const lamp_decode_params* p, void* stream) {
  lamp::DecodeArgs a;
  bool empty = false;
  // validate first with a placeholder workspace; the partials' real home is
  // only looked up for a call that launches
  const lamp_status st = decode_prepare(p, nullptr, false, &a, &empty);
  if (st != LAMP_OK || empty) return st;
  const size_t need = lamp_decode_workspace_bytes(p->B, p->Hkv, p->S_k, p->D);
  if (need > lamp::kDecodeScratchBytes)
    return fail(LAMP_ERR_UNSUPPORTED,
                "these sizes need %zu bytes of split partials; the fixed scratch holds %zu "
                "(use lamp_decode_fwd with a workspace)",
                need, lamp::kDecodeScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = lamp::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "scratch address");
  const int64_t nslot = (int64_t)a.B * a.Hkv * a.n_split * 32;
  a.ws_o = static_cast<float*>(scratch);
  a.ws_ml = a.ws_o + nslot * a.D;
  return hip_status(lamp::launch_decode(a, static_cast<hipStream_t>(stream)), "decode launch");
}

lamp_status lamp_decode_fwd(const lamp_decode_params* p, void* workspace, size_t workspace_bytes,
                            void* stream) {
  lamp::DecodeArgs a;
  bool empty = false;
  const lamp_status st = decode_prepare(p, workspace, true, &a, &empty);
  if (st != LAMP_OK || empty) return st;
  const size_t need = lamp_decode_workspace_bytes(p->B, p->Hkv, p->S_k, p->D);
  if (workspace_bytes < need)
    return fail(LAMP_ERR_SHAPE, "workspace %zu bytes < %zu", workspace_bytes, need);
  return hip_status(lamp::launch_decode(a, static_cast<hipStream_t>(stream)), "decode launch");
}

}  // extern "C"
