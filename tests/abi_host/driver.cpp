// Every C ABI entry point called from the host with valid arguments (the
// stub launcher must see the launch, with the derived sizes the kernels
// rely on) and with each kind of invalid argument (the documented status,
// a message, no launch).  Device pointers are never dereferenced by the
// ABI layer, so aligned fake addresses stand in for them.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/lamp.h"
#include "record.h"

static int g_checks = 0, g_failed = 0;

#define CHECK(cond)                                                                  \
  do {                                                                               \
    ++g_checks;                                                                      \
    if (!(cond)) {                                                                   \
      ++g_failed;                                                                    \
      std::printf("FAILED %s:%d: %s  [last error: %s]\n", __FILE__, __LINE__, #cond, \
                  lamp_last_error());                                                \
    }                                                                                \
  } while (0)

// a status and, for a failure, a message and no launch
#define EXPECT(call, status)                                   \
  do {                                                         \
    const int before_ = g_rec.total();                         \
    const lamp_status st_ = (call);                            \
    CHECK(st_ == (status));                                    \
    if ((status) != LAMP_OK) {                                 \
      CHECK(std::strlen(lamp_last_error()) > 0);               \
      CHECK(g_rec.total() == before_);                         \
    }                                                          \
  } while (0)

static void* dev(uintptr_t a) { return reinterpret_cast<void*>(a); }
static void* const S = nullptr;   // stream

static void quantisers() {
  void* x = dev(0x10000);
  void* c = dev(0x20000);
  float* sc = static_cast<float*>(dev(0x30000));
  const int64_t D = 128, ss = D, sh = 100 * ss, sb = 3 * sh;
  const int n0 = g_rec.n_quant;
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 64, LAMP_I8, c, sc, S), LAMP_OK);
  CHECK(g_rec.n_quant == n0 + 1);
  CHECK(g_rec.quant.nb == 2 && g_rec.quant.chunk_shift == 4 && g_rec.quant.B == 2 && g_rec.quant.H == 3);
  CHECK(g_rec.quant.bf16 && !g_rec.quant.e4m3 && g_rec.quant.seqlens == nullptr);
  EXPECT(lamp_quantize_blocks(x, LAMP_F16, 1, 1, 5, 64, 320, 320, 64, 3, LAMP_E4M3, c, sc, S), LAMP_OK);
  CHECK(g_rec.quant.nb == 2 && g_rec.quant.chunk_shift == 3 && g_rec.quant.e4m3 && !g_rec.quant.bf16);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 1, 1, 64, 256, 0, 0, 256, 64, LAMP_I8, c, sc, S), LAMP_OK);
  CHECK(g_rec.quant.chunk_shift == 5);
  // empty input: no pointer needed, no launch
  const int n1 = g_rec.total();
  EXPECT(lamp_quantize_blocks(nullptr, LAMP_BF16, 2, 3, 0, D, 0, 0, D, 64, LAMP_I8, nullptr, nullptr, S), LAMP_OK);
  CHECK(g_rec.total() == n1);
  CHECK(std::strlen(lamp_last_error()) == 0);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, -1, 3, 100, D, sb, sh, ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, -ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_quantize_blocks(x, LAMP_I8, 2, 3, 100, D, sb, sh, ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 64, LAMP_F16, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, 96, sb, sh, ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 0, LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 257, LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 1, 1, (1 << 20) + 1, D, 0, 0, ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(nullptr, LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_NULL);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 64, LAMP_I8, c, nullptr, S), LAMP_ERR_NULL);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, D - 8, 64, LAMP_I8, c, sc, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_quantize_blocks(dev(0x10008), LAMP_BF16, 2, 3, 100, D, sb, sh, ss, 64, LAMP_I8, c, sc, S), LAMP_ERR_ALIGN);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss + 4, 64, LAMP_I8, c, sc, S), LAMP_ERR_ALIGN);
  EXPECT(lamp_quantize_blocks_varlen(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss,
                                     static_cast<const int32_t*>(dev(0x40002)), 64, LAMP_I8, c, sc, S),
         LAMP_ERR_ALIGN);
  EXPECT(lamp_quantize_blocks_varlen(x, LAMP_BF16, 2, 3, 100, D, sb, sh, ss,
                                     static_cast<const int32_t*>(dev(0x40004)), 64, LAMP_I8, c, sc, S),
         LAMP_OK);
  CHECK(g_rec.quant.seqlens == dev(0x40004));
  // sizes whose block count overflows the grid (and would overflow int64 if
  // multiplied naively)
  const int64_t big = int64_t(1) << 40;
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, big, big, 100, D, 0, 0, ss, 1, LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_blocks(x, LAMP_BF16, std::numeric_limits<int64_t>::max(), 3, 100, D, 0, 0, ss, 1,
                              LAMP_I8, c, sc, S), LAMP_ERR_UNSUPPORTED);

  // V tiles
  EXPECT(lamp_quantize_v_tiles(x, LAMP_BF16, 2, 8, 130, D, sb, sh, ss, nullptr, c, sc, S), LAMP_OK);
  CHECK(g_rec.quant_v.n_kt == 3 && g_rec.quant_v.H == 8 && g_rec.quant_v.bf16);
  EXPECT(lamp_quantize_v_tiles(x, LAMP_BF16, 2, 8, 0, D, sb, sh, ss, nullptr, nullptr, nullptr, S), LAMP_OK);
  EXPECT(lamp_quantize_v_tiles(nullptr, LAMP_BF16, 2, 8, 130, D, sb, sh, ss, nullptr, c, sc, S), LAMP_ERR_NULL);
  EXPECT(lamp_quantize_v_tiles(x, LAMP_E4M3, 2, 8, 130, D, sb, sh, ss, nullptr, c, sc, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_quantize_v_tiles(x, LAMP_BF16, 2, 8, 130, D, sb, sh, ss, nullptr, dev(0x20004), sc, S), LAMP_ERR_ALIGN);
  EXPECT(lamp_quantize_v_tiles(x, LAMP_BF16, big, big, 130, D, 0, 0, ss, nullptr, c, sc, S), LAMP_ERR_UNSUPPORTED);

  // 8-bit exponential table
  EXPECT(lamp_exp8_table(nullptr, S), LAMP_ERR_NULL);
  const int n2 = g_rec.n_exp8;
  EXPECT(lamp_exp8_table(static_cast<uint8_t*>(dev(0x50000)), S), LAMP_OK);
  CHECK(g_rec.n_exp8 == n2 + 1);
}

static void masks() {
  uint64_t* m = static_cast<uint64_t*>(dev(0x60000));
  // 16384 keys / 64 = 256 tiles, 4 per group -> 64 groups, one word per row
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 4, 0.25, 7, m, 1, S), LAMP_OK);
  CHECK(g_rec.mask.n_g == 64 && g_rec.mask.n_qt == 128 && g_rec.mask.threshold == (uint64_t(1) << 30));
  CHECK(g_rec.mask.total_words == 2 * 32 * 128 && g_rec.mask.per_head == 0 && g_rec.mask.seed == 7);
  EXPECT(lamp_build_mask(1, 1, 100, 100, 128, 64, 1, 1.0, 0, m, 1, S), LAMP_OK);
  CHECK(g_rec.mask.threshold == (uint64_t(1) << 32));
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 4, 1.5, 7, m, 1, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 4, std::nan(""), 7, m, 1, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 1, 0.25, 7, m, 3, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 4, 0.25, 7, m, 0, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 0, 64, 4, 0.25, 7, m, 1, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 4, 0.25, 7, nullptr, 1, S), LAMP_ERR_NULL);
  EXPECT(lamp_build_mask(2, 32, 16384, 16384, 128, 64, 4, 0.25, 7, static_cast<uint64_t*>(dev(0x60004)), 1, S),
         LAMP_ERR_ALIGN);
  const int64_t big = int64_t(1) << 40;
  EXPECT(lamp_build_mask(big, big, 16384, 16384, 128, 64, 4, 0.25, 7, m, 1, S), LAMP_ERR_UNSUPPORTED);
  double fr[129];
  for (int h = 0; h < 129; ++h) fr[h] = h / 128.0;
  EXPECT(lamp_build_mask_per_head(1, 128, 256, 256, 128, 64, 1, fr, 3, m, 1, S), LAMP_OK);
  CHECK(g_rec.mask.per_head == 1 && g_rec.mask.head_threshold[64] == (uint64_t(1) << 31) &&
        g_rec.mask.head_threshold[127] == (uint64_t(1) << 32) - (uint64_t(1) << 25) &&
        g_rec.mask.head_threshold[0] == 0);
  EXPECT(lamp_build_mask_per_head(1, 129, 256, 256, 128, 64, 1, fr, 3, m, 1, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_build_mask_per_head(1, 4, 256, 256, 128, 64, 1, nullptr, 3, m, 1, S), LAMP_ERR_NULL);
  fr[2] = -0.5;
  EXPECT(lamp_build_mask_per_head(1, 4, 256, 256, 128, 64, 1, fr, 3, m, 1, S), LAMP_ERR_SHAPE);

  EXPECT(lamp_build_mask_template(1, 2, 1000, 1200, 128, 64, 2, 1, 2, 4, m, 1, S), LAMP_OK);
  CHECK(g_rec.tmpl.group_keys == 128 && g_rec.tmpl.pos_off == 200 && g_rec.tmpl.n_g == 10 &&
        g_rec.tmpl.n_qt == 8 && g_rec.tmpl.sink == 1 && g_rec.tmpl.band == 2 && g_rec.tmpl.stride == 4);
  EXPECT(lamp_build_mask_template(1, 2, 1000, 1200, 128, 64, 2, -1, 2, 4, m, 1, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_build_mask_template(1, 2, 1000, 1200, 128, 1 << 20, 1 << 12, 0, 0, 0, m, 1, S), LAMP_ERR_UNSUPPORTED);
  EXPECT(lamp_build_mask_template(big, big, 1000, 1200, 128, 64, 2, 1, 2, 4, m, 1, S), LAMP_ERR_UNSUPPORTED);
}

static lamp_attn_params attn_ok() {
  lamp_attn_params p;
  std::memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.mode = LAMP_MODE_MASK;
  p.causal = 1;
  p.B = 2; p.Hq = 32; p.Hkv = 8; p.S_q = 1000; p.S_k = 1000; p.D = 128;
  p.q = dev(0x100000); p.k = dev(0x200000); p.v = dev(0x300000); p.out = dev(0x400000);
  p.in_dtype = LAMP_BF16;
  p.code_dtype = LAMP_I8;
  for (int64_t* s : {p.q_str, p.o_str}) { s[2] = 128; s[1] = 1000 * 128; s[0] = 32 * 1000 * 128; }
  for (int64_t* s : {p.k_str, p.v_str}) { s[2] = 128; s[1] = 1000 * 128; s[0] = 8 * 1000 * 128; }
  p.q8 = dev(0x500000); p.k8 = dev(0x600000);
  p.q_scale = static_cast<const float*>(dev(0x700000));
  p.k_scale = static_cast<const float*>(dev(0x710000));
  p.mask = static_cast<const uint64_t*>(dev(0x720000));
  p.words_per_row = 1;
  p.tile_m = 128; p.tile_n = 64; p.tiles_per_bit = 4;
  p.tau = 4.f;
  p.sub_rows = 32;
  return p;
}

static void attention() {
  lamp_attn_params p = attn_ok();
  const int n0 = g_rec.n_attn;
  EXPECT(lamp_attn_fwd(&p, S), LAMP_OK);
  CHECK(g_rec.n_attn == n0 + 1 && g_rec.attn_d == 128);
  CHECK(g_rec.attn.n_qt == 8 && g_rec.attn.n_kt == 16 && g_rec.attn.heads_per_group == 4 &&
        g_rec.attn.n_sb == 32 && g_rec.attn.flag_words == 1);
  CHECK(std::fabs(g_rec.attn.sm_scale - 1.f / std::sqrt(128.f)) < 1e-7f);
  CHECK(g_rec.attn_cfg.nw == 4 && g_rec.attn_cfg.bf16 && !g_rec.attn_cfg.e4m3 && !g_rec.attn_cfg.adaptive);
  CHECK(g_rec.attn.flags == nullptr);
  // adaptive e4m3 exp8 at D 256, tile_m 64, flags kept
  p = attn_ok();
  p.D = 256;
  for (int64_t* s : {p.q_str, p.k_str, p.v_str, p.o_str}) { s[2] = 256; s[1] *= 2; s[0] *= 2; }
  p.mode = LAMP_MODE_ADAPTIVE; p.code_dtype = LAMP_E4M3; p.exp8 = 1; p.tile_m = 64;
  p.flags_out = static_cast<uint64_t*>(dev(0x730000));
  p.sm_scale = 0.5f;
  EXPECT(lamp_attn_fwd(&p, S), LAMP_OK);
  CHECK(g_rec.attn_d == 256 && g_rec.attn_cfg.nw == 2 && g_rec.attn_cfg.adaptive && g_rec.attn_cfg.e4m3 &&
        g_rec.attn_cfg.exp8 && g_rec.attn.flags == p.flags_out && g_rec.attn.sm_scale == 0.5f &&
        g_rec.attn.n_qt == 16);
  // 8-bit P V
  p = attn_ok();
  p.exp8 = 1; p.pv8 = 1; p.code_dtype = LAMP_E4M3;
  p.v8 = dev(0x800000); p.v_scale = static_cast<const float*>(dev(0x810000));
  EXPECT(lamp_attn_fwd(&p, S), LAMP_OK);
  CHECK(g_rec.attn_cfg.pv8 && g_rec.attn.v8 == p.v8);
  p.v8 = nullptr;
  EXPECT(lamp_attn_fwd(&p, S), LAMP_ERR_NULL);
  p.v8 = dev(0x800008);
  EXPECT(lamp_attn_fwd(&p, S), LAMP_ERR_ALIGN);
  // nothing to do
  p = attn_ok(); p.S_q = 0; p.q = nullptr;
  const int n1 = g_rec.total();
  EXPECT(lamp_attn_fwd(&p, S), LAMP_OK);
  CHECK(g_rec.total() == n1);

  struct Case { const char* what; void (*mut)(lamp_attn_params&); lamp_status st; };
  const Case cases[] = {
      {"struct size", [](lamp_attn_params& q) { q.struct_size -= 8; }, LAMP_ERR_UNSUPPORTED},
      {"negative S_k", [](lamp_attn_params& q) { q.S_k = -1; }, LAMP_ERR_SHAPE},
      {"negative stride", [](lamp_attn_params& q) { q.v_str[1] = -8; }, LAMP_ERR_SHAPE},
      {"mode", [](lamp_attn_params& q) { q.mode = 7; }, LAMP_ERR_UNSUPPORTED},
      {"in dtype", [](lamp_attn_params& q) { q.in_dtype = LAMP_I8; }, LAMP_ERR_UNSUPPORTED},
      {"code dtype", [](lamp_attn_params& q) { q.code_dtype = LAMP_BF16; }, LAMP_ERR_UNSUPPORTED},
      {"D", [](lamp_attn_params& q) { q.D = 96; }, LAMP_ERR_UNSUPPORTED},
      {"tile_m", [](lamp_attn_params& q) { q.tile_m = 32; }, LAMP_ERR_UNSUPPORTED},
      {"tile_n", [](lamp_attn_params& q) { q.tile_n = 128; }, LAMP_ERR_UNSUPPORTED},
      {"tiles_per_bit", [](lamp_attn_params& q) { q.tiles_per_bit = 0; }, LAMP_ERR_SHAPE},
      {"Hq % Hkv", [](lamp_attn_params& q) { q.Hkv = 5; }, LAMP_ERR_UNSUPPORTED},
      {"Hkv 0", [](lamp_attn_params& q) { q.Hkv = 0; }, LAMP_ERR_UNSUPPORTED},
      {"causal 2", [](lamp_attn_params& q) { q.causal = 2; }, LAMP_ERR_SHAPE},
      {"causal S_q > S_k", [](lamp_attn_params& q) { q.S_q = 1001; }, LAMP_ERR_UNSUPPORTED},
      {"exp8 2", [](lamp_attn_params& q) { q.exp8 = 2; }, LAMP_ERR_SHAPE},
      {"pv8 without exp8", [](lamp_attn_params& q) { q.pv8 = 1; }, LAMP_ERR_UNSUPPORTED},
      {"pv8 adaptive", [](lamp_attn_params& q) { q.pv8 = 1; q.exp8 = 1; q.mode = LAMP_MODE_ADAPTIVE; },
       LAMP_ERR_UNSUPPORTED},
      {"sub_rows", [](lamp_attn_params& q) { q.mode = LAMP_MODE_ADAPTIVE; q.sub_rows = 16; }, LAMP_ERR_UNSUPPORTED},
      {"tau NaN", [](lamp_attn_params& q) { q.mode = LAMP_MODE_ADAPTIVE; q.tau = std::nanf(""); }, LAMP_ERR_SHAPE},
      {"sm_scale NaN", [](lamp_attn_params& q) { q.sm_scale = std::nanf(""); }, LAMP_ERR_SHAPE},
      {"too long", [](lamp_attn_params& q) { q.S_k = (1 << 20) + 64; q.causal = 0; }, LAMP_ERR_UNSUPPORTED},
      {"words_per_row", [](lamp_attn_params& q) { q.tiles_per_bit = 1; q.S_k = q.S_q = 4160; q.words_per_row = 1; },
       LAMP_ERR_UNSUPPORTED},
      {"dbg on e4m3", [](lamp_attn_params& q) { q.code_dtype = LAMP_E4M3; q.dbg_qk_acc = static_cast<int32_t*>(dev(0x900000)); },
       LAMP_ERR_UNSUPPORTED},
      {"no keys", [](lamp_attn_params& q) { q.S_k = 0; q.causal = 0; }, LAMP_ERR_SHAPE},
      {"null q", [](lamp_attn_params& q) { q.q = nullptr; }, LAMP_ERR_NULL},
      {"null mask", [](lamp_attn_params& q) { q.mask = nullptr; }, LAMP_ERR_NULL},
      {"null out", [](lamp_attn_params& q) { q.out = nullptr; }, LAMP_ERR_NULL},
      {"row stride < D", [](lamp_attn_params& q) { q.k_str[2] = 64; }, LAMP_ERR_SHAPE},
      {"q alignment", [](lamp_attn_params& q) { q.q = dev(0x100008); }, LAMP_ERR_ALIGN},
      {"k8 alignment", [](lamp_attn_params& q) { q.k8 = dev(0x600004); }, LAMP_ERR_ALIGN},
      {"stride multiple", [](lamp_attn_params& q) { q.o_str[1] += 4; }, LAMP_ERR_ALIGN},
      {"mask alignment", [](lamp_attn_params& q) { q.mask = static_cast<const uint64_t*>(dev(0x720004)); }, LAMP_ERR_ALIGN},
      {"seqlens alignment", [](lamp_attn_params& q) { q.seqlens_k = static_cast<const int32_t*>(dev(0x740002)); },
       LAMP_ERR_ALIGN},
      {"flags alignment", [](lamp_attn_params& q) { q.mode = LAMP_MODE_ADAPTIVE; q.flags_out = static_cast<uint64_t*>(dev(0x730004)); },
       LAMP_ERR_ALIGN},
      {"K rows over 2 GiB", [](lamp_attn_params& q) { q.S_q = 64; q.S_k = 1 << 20; q.k_str[2] = 1024; q.words_per_row = 64; },
       LAMP_ERR_UNSUPPORTED},
      {"grid overflow", [](lamp_attn_params& q) { q.B = int64_t(1) << 40; q.Hq = int64_t(1) << 40; q.Hkv = 1; },
       LAMP_ERR_UNSUPPORTED},
      {"K row stride overflow", [](lamp_attn_params& q) { q.k_str[2] = int64_t(1) << 60; }, LAMP_ERR_UNSUPPORTED},
  };
  for (const Case& c : cases) {
    lamp_attn_params q = attn_ok();
    c.mut(q);
    const int before = g_rec.total();
    const lamp_status st = lamp_attn_fwd(&q, S);
    ++g_checks;
    if (st != c.st || std::strlen(lamp_last_error()) == 0 || g_rec.total() != before) {
      ++g_failed;
      std::printf("FAILED attention case '%s': status %s, expected %s [%s]\n", c.what, lamp_status_string(st),
                  lamp_status_string(c.st), lamp_last_error());
    }
  }
  EXPECT(lamp_attn_fwd(nullptr, S), LAMP_ERR_NULL);
}

static lamp_decode_params decode_ok() {
  lamp_decode_params p;
  std::memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.causal = 1;
  p.out_dtype = LAMP_BF16;
  p.B = 8; p.Hq = 32; p.Hkv = 8; p.S_q = 1; p.S_k = 32768; p.D = 128;
  p.q8 = dev(0x100000); p.k8 = dev(0x200000); p.v8 = dev(0x300000);
  p.q_scale = static_cast<const float*>(dev(0x400000));
  p.k_scale = static_cast<const float*>(dev(0x410000));
  p.v_scale = static_cast<const float*>(dev(0x420000));
  p.tile_m = 64;
  p.out = dev(0x500000);
  p.o_str[2] = 128; p.o_str[1] = 128; p.o_str[0] = 32 * 128;
  return p;
}

static void decode() {
  CHECK(lamp_decode_workspace_bytes(8, 8, 32768, 128) == size_t(8) * 8 * 16 * 32 * 130 * 4);
  CHECK(lamp_decode_workspace_bytes(2, 8, 5000, 128) == size_t(2) * 8 * 10 * 32 * 130 * 4);
  CHECK(lamp_decode_workspace_bytes(-1, 8, 5000, 128) == 0);
  CHECK(lamp_decode_workspace_bytes(0, 8, 5000, 128) == 0);
  CHECK(lamp_decode_workspace_bytes(int64_t(1) << 40, int64_t(1) << 40, 5000, 128) == SIZE_MAX);
  CHECK(lamp_decode_workspace_bytes(1, 1, (1 << 20) + 1, 128) == SIZE_MAX);
  CHECK(lamp_decode_workspace_bytes(1, 1, 64, std::numeric_limits<int64_t>::max()) == SIZE_MAX);
  lamp_decode_params p = decode_ok();
  void* ws = dev(0x1000000);
  const size_t need = lamp_decode_workspace_bytes(8, 8, 32768, 128);
  const int n0 = g_rec.n_decode;
  EXPECT(lamp_decode_fwd(&p, ws, need, S), LAMP_OK);
  CHECK(g_rec.n_decode == n0 + 1);
  CHECK(g_rec.decode.tiles_per_split == 32 && g_rec.decode.n_split == 16 && g_rec.decode.n_kt == 512 &&
        g_rec.decode.hpg == 4 && g_rec.decode.cols == 4 && g_rec.decode.ws_o == ws &&
        g_rec.decode.ws_ml == static_cast<float*>(ws) + int64_t(8) * 8 * 16 * 32 * 128);
  EXPECT(lamp_decode_fwd(&p, ws, need - 4, S), LAMP_ERR_SHAPE);
  EXPECT(lamp_decode_fwd(&p, nullptr, need, S), LAMP_ERR_NULL);
  EXPECT(lamp_decode_fwd(&p, dev(0x1000004), need, S), LAMP_ERR_ALIGN);
  const int s0 = g_rec.n_scratch;
  EXPECT(lamp_decode_fwd_noalloc(&p, S), LAMP_OK);
  CHECK(g_rec.n_scratch == s0 + 1 && g_rec.decode.ws_o == reinterpret_cast<float*>(g_scratch));
  // partials beyond the fixed scratch
  p.B = 64;
  EXPECT(lamp_decode_fwd_noalloc(&p, S), LAMP_ERR_UNSUPPORTED);
  p = decode_ok();
  p.S_q = 0; p.q8 = nullptr;
  const int n1 = g_rec.total();
  EXPECT(lamp_decode_fwd(&p, nullptr, 0, S), LAMP_OK);
  CHECK(g_rec.total() == n1);
  struct Case { const char* what; void (*mut)(lamp_decode_params&); lamp_status st; };
  const Case cases[] = {
      {"struct size", [](lamp_decode_params& q) { q.struct_size = 0; }, LAMP_ERR_UNSUPPORTED},
      {"negative", [](lamp_decode_params& q) { q.Hq = -32; }, LAMP_ERR_SHAPE},
      {"D 256", [](lamp_decode_params& q) { q.D = 256; }, LAMP_ERR_UNSUPPORTED},
      {"out dtype", [](lamp_decode_params& q) { q.out_dtype = LAMP_I8; }, LAMP_ERR_UNSUPPORTED},
      {"group too wide", [](lamp_decode_params& q) { q.S_q = 9; }, LAMP_ERR_UNSUPPORTED},
      {"Hq % Hkv", [](lamp_decode_params& q) { q.Hkv = 3; }, LAMP_ERR_UNSUPPORTED},
      {"tile_m", [](lamp_decode_params& q) { q.tile_m = 0; }, LAMP_ERR_SHAPE},
      {"causal S_q > S_k", [](lamp_decode_params& q) { q.S_k = 0; q.S_q = 1; }, LAMP_ERR_UNSUPPORTED},
      {"no keys", [](lamp_decode_params& q) { q.S_k = 0; q.causal = 0; }, LAMP_ERR_SHAPE},
      {"null k8", [](lamp_decode_params& q) { q.k8 = nullptr; }, LAMP_ERR_NULL},
      {"v8 alignment", [](lamp_decode_params& q) { q.v8 = dev(0x300008); }, LAMP_ERR_ALIGN},
      {"out alignment", [](lamp_decode_params& q) { q.out = dev(0x500001); }, LAMP_ERR_ALIGN},
      {"lse alignment", [](lamp_decode_params& q) { q.lse = static_cast<float*>(dev(0x600002)); }, LAMP_ERR_ALIGN},
      {"output stride", [](lamp_decode_params& q) { q.o_str[0] = -1; }, LAMP_ERR_SHAPE},
      {"too long", [](lamp_decode_params& q) { q.S_k = (1 << 20) + 1; }, LAMP_ERR_UNSUPPORTED},
      {"query group overflow", [](lamp_decode_params& q) { q.causal = 0; q.S_q = int64_t(1) << 62; },
       LAMP_ERR_UNSUPPORTED},
      {"grid overflow", [](lamp_decode_params& q) { q.B = int64_t(1) << 40; q.Hkv = int64_t(1) << 40; q.Hq = q.Hkv; },
       LAMP_ERR_UNSUPPORTED},
      {"heads beyond 32 bits", [](lamp_decode_params& q) { q.B = 1; q.Hkv = int64_t(1) << 31; q.Hq = int64_t(1) << 32; },
       LAMP_ERR_UNSUPPORTED},
  };
  for (const Case& c : cases) {
    lamp_decode_params q = decode_ok();
    c.mut(q);
    const int before = g_rec.total();
    const lamp_status st = lamp_decode_fwd(&q, ws, need, S);
    ++g_checks;
    if (st != c.st || std::strlen(lamp_last_error()) == 0 || g_rec.total() != before) {
      ++g_failed;
      std::printf("FAILED decode case '%s': status %s, expected %s [%s]\n", c.what, lamp_status_string(st),
                  lamp_status_string(c.st), lamp_last_error());
    }
  }
  EXPECT(lamp_decode_fwd(nullptr, ws, need, S), LAMP_ERR_NULL);
  EXPECT(lamp_decode_fwd_noalloc(nullptr, S), LAMP_ERR_NULL);
}

int main() {
  quantisers();
  masks();
  attention();
  decode();
  const lamp_status all[] = {LAMP_OK, LAMP_ERR_NULL, LAMP_ERR_SHAPE, LAMP_ERR_UNSUPPORTED, LAMP_ERR_ALIGN,
                             LAMP_ERR_HIP};
  for (lamp_status s : all) CHECK(std::strncmp(lamp_status_string(s), "LAMP_", 5) == 0);
  CHECK(std::strcmp(lamp_status_string(static_cast<lamp_status>(99)), "LAMP_ERR_UNKNOWN") == 0);
  CHECK(lamp_abi_version() == LAMP_ABI_VERSION);
  std::printf("%d checks, %d failed\n", g_checks, g_failed);
  return g_failed == 0 ? 0 : 1;
}
