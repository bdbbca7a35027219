// Internal launch descriptors shared by the C ABI layer and the kernels.
// Arguments reach the kernels by value; every field has been validated by
// the ABI layer before a launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lamp {

struct QuantArgs {
  const void* x;
  void* codes;
  float* scales;
  int64_t sb, sh, ss;          // element strides of x
  int32_t B, H, S, D;
  int32_t block_rows, nb;      // nb = ceil(S / block_rows)
  int32_t chunk_shift;         // log2(D / 8)
  const int32_t* seqlens;      // [B] or nullptr (all S)
  bool bf16, e4m3;
};

struct VQuantArgs {
  const void* v;
  uint8_t* codes;              // [B, H, n_kt, D, 64] tile-packed
  float* scales;               // [B, H, n_kt]
  int64_t sb, sh, ss;          // element strides of v
  int32_t B, H, S, D, n_kt;
  const int32_t* seqlens;      // [B] or nullptr (all S)
  bool bf16;
};

constexpr int kMaskMaxHeads = 128;      // per-head fractions ride in the kernel arguments
constexpr int kMaskWordsPerBlock = 4;    // random-mask builder: one wave per word

struct MaskArgs {
  uint64_t* mask;
  int64_t total_words;         // B * Hq * n_qt * words_per_row
  uint64_t seed;
  uint64_t threshold;          // floor(frac_16bit * 2^32)
  int32_t words_per_row;
  int32_t n_g;
  int32_t per_head;            // 1: threshold of query head h is head_threshold[h]
  int32_t Hq, n_qt;
  uint64_t head_threshold[kMaskMaxHeads];
};

struct TemplateMaskArgs {
  uint64_t* mask;
  int64_t total_words;         // B * Hq * n_qt * words_per_row
  int32_t words_per_row;
  int32_t n_g;
  int32_t n_qt;
  int32_t tile_m;
  int32_t group_keys;          // tiles_per_bit * tile_n
  int32_t sink, band, stride;
  int64_t pos_off;             // S_k - S_q: key position of query row 0
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* q8;
  const uint8_t* k8;
  const float* q_scale;
  const float* k_scale;
  const uint64_t* mask;
  void* out;
  float* lse;
  uint64_t* flags;
  int32_t* dbg;
  const int32_t* seqlens_q;    // [B] or nullptr (all S_q)
  const int32_t* seqlens_k;    // [B] or nullptr (all S_k)
  const uint8_t* v8;           // pv8: [B, Hkv, n_kt, D, 64] tile-packed e4m3 V
  const float* v_scale;        // pv8: [B, Hkv, n_kt] powers of two
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int32_t B, Hq, Hkv, S_q, S_k;
  int32_t n_qt, n_kt, tiles_per_bit, words_per_row;
  int32_t heads_per_group;     // Hq / Hkv
  int32_t n_sb, flag_words;    // ceil(S_q/32), ceil(n_kt/64)
  int32_t causal;
  float sm_scale;              // natural-log units
  float tau;
};

// Decode over an int8 key/value cache: 64-key tiles per split of the keys.
// The split length aims at one wave per SIMD over the whole grid (1024
// SIMDs), within [8, 32] tiles: long enough for the ring of register sets in
// each wave (the next tile's loads in flight) to pay off, short enough to fill
// the chip at small batch.
constexpr int kDecodeMinTilesPerSplit = 8;
constexpr int kDecodeMaxTilesPerSplit = 32;
constexpr int64_t kDecodeTargetWaves = 1024;
inline int decode_tiles_per_split(int64_t B, int64_t Hkv, int64_t n_kt) {
  const int64_t want = (B * Hkv * n_kt + kDecodeTargetWaves - 1) / kDecodeTargetWaves;
  return (int)(want < kDecodeMinTilesPerSplit ? kDecodeMinTilesPerSplit
                                              : want > kDecodeMaxTilesPerSplit ? kDecodeMaxTilesPerSplit : want);
}
constexpr int kMergeMaxSplit = 4096;     // splits of one merge (S_k <= 2^20 keys: at most 2048)

struct DecodeArgs {
  const uint8_t* q8;
  const float* q_scale;        // [B, Hq, n_qt]
  const uint8_t* k8;
  const float* k_scale;        // [B, Hkv, n_kt]
  const uint8_t* v8;
  const float* v_scale;        // [B, Hkv, n_kt]
  void* out;
  float* lse;
  float* ws_o;                 // [B*Hkv, n_split, 32, D] partial O
  float* ws_ml;                // [B*Hkv, n_split, 32, 2] partial (m, l), base 2
  int64_t o_sb, o_sh, o_ss;
  int32_t B, Hq, Hkv, S_q, S_k, D;
  int32_t hpg, cols;           // Hq / Hkv, hpg * S_q (<= 32)
  int32_t tile_m, n_qt, n_kt, n_split, tiles_per_split;
  int32_t causal;
  float sm_scale;
  bool bf16;
};

struct AttnConfig {
  int d;            // 64 | 128 | 256
  int nw;           // waves per workgroup = tile_m / 32
  bool bf16;
  bool e4m3;
  bool adaptive;
  bool exp8;
  bool pv8;
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_quantize_v(const VQuantArgs& a, hipStream_t s);
hipError_t launch_exp8_table(uint8_t* out, hipStream_t s);
hipError_t launch_build_mask(const MaskArgs& a, hipStream_t s);
hipError_t launch_build_mask_template(const TemplateMaskArgs& a, hipStream_t s);
hipError_t launch_attn_d64(const AttnArgs& a, const AttnConfig& c, hipStream_t s);
hipError_t launch_attn_d128(const AttnArgs& a, const AttnConfig& c, hipStream_t s);
hipError_t launch_attn_d256(const AttnArgs& a, const AttnConfig& c, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Size of the fixed device scratch of lamp_decode_fwd_noalloc (one copy per
// GPU, held until the process ends), and the device address of the current
// GPU's copy (looked up once per device, with that device current).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace lamp
