// Dual-path (8-bit / 16-bit) fused attention prefill forward for gfx950.
//
// Sources (pages, by title and section):
//   "TileMix: Mixed-Precision Attention for Faster LLM Prefill", section 2:
//     the score matrix is processed one hardware-aligned tile at a time; the
//     inner loop reads the packed mask bit of the current key-tile group and
//     dispatches the tile's QK^T to a 16-bit product or to an INT8 product
//     rescaled with per-block scales; both update one shared online-softmax
//     state.  Section 4: grouped-query attention.
//   "LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
//     Accelerators", Abstract: 8-bit products and exponentials, sensitive
//     sub-blocks found adaptively and recomputed in 16 bits.
//
// MI355X design (not the pages' A100 / accelerator design):
//   * one workgroup = one query tile of TM = 32*NW rows of one (b, h); each
//     64-lane wave owns 32 query rows;
//   * a wave computes S^T = K Q^T with 32x32 MFMAs (A = K from LDS, B = Q held
//     in registers), so lane l ends up with the 32 logits of query row l%32
//     for its half of the 64-key tile: the row max / row sum need a single
//     cross-half exchange, and alpha rescales only the lane's own rows;
//   * P V is computed as O^T = V^T P^T: the S^T accumulator registers are, once
//     converted to 16 bits, exactly the B operand of the next MFMA (no LDS
//     round trip for P); V stays key-major in LDS and is read with the
//     transposing ds_read_b64_tr_b16, the key order inside each 16-key group
//     permuted to match that register layout;
//   * K (as K16 or K8, whichever the mask selects) and V are double-buffered
//     in LDS through direct-to-LDS buffer loads, one barrier per key tile; a
//     step computes the logits of tile kt and interleaves P V of tile kt-1
//     with the softmax arithmetic of tile kt;
//   * workgroups are mapped so that each XCD processes whole KV-head groups
//     (shared K/V in its L2), longest causal query tiles first;
//   * optional 8-bit P V (with 8-bit exponentials under mask routing): an
//     8-bit tile stages its tile-packed e4m3 V block and multiplies it with
//     the e4m3 weights in fp8 MFMAs, the V tile's power-of-two scale as the
//     operand's block scale.
#pragma once

#include <type_traits>

#include "lamp_device.h"
#include "lamp_internal.h"

namespace lamp {

template <int D, int NW>
struct AttnShape {
  static constexpr int TM = NW * 32;            // query rows per workgroup
  static constexpr int TN = 64;                 // keys per tile
  static constexpr int NT = NW * 64;            // threads
  static constexpr int ND = D / 32;             // O^T blocks of 32 head-dim rows
  static constexpr int NQ16 = D / 16;           // 16-bit MFMAs per 32-key block
  static constexpr int NQ8 = D / 32;            // 16-byte Q8 / K8 fragments per lane
  static constexpr int RB16 = 2 * D;            // bytes per K16 / V row
  static constexpr int RB8 = D;                 // bytes per K8 row
  static constexpr int K16_BYTES = TN * RB16;
  static constexpr int K8_BYTES = TN * RB8;
  static constexpr int V_BYTES = TN * RB16;
  static constexpr int STAGE = K16_BYTES + V_BYTES;   // K region sized for K16
  static constexpr int CH16 = D / 8;            // 16-byte chunks per K16 / V row
  static constexpr int CH8 = D / 16;            // 16-byte chunks per K8 row
  // direct-to-LDS copies: 1 KB per wave instruction, split over the waves
  static constexpr int JK16 = K16_BYTES / 1024 / NW;
  static constexpr int JK8 = K8_BYTES / 1024 / NW;
  static constexpr int JV = V_BYTES / 1024 / NW;
  // 8-bit P V: tile-packed e4m3 V, D rows of 64 keys
  static constexpr int V8_BYTES = D * 64;
  static constexpr int JV8 = V8_BYTES / 1024 / NW;
  static_assert(K8_BYTES % (1024 * NW) == 0, "K8 tile must split evenly over the waves");
  static_assert(V8_BYTES % (1024 * NW) == 0, "V8 tile must split evenly over the waves");
};

// LDS layouts.  Every region is row-major (one key per row) in 16-byte chunks;
// the chunk holding logical chunk lc of row r sits at position lc ^ swz(r).
//  * K16 / K8 rows are read by ds_read_b128 with one row per lane: swz(r)
//    spreads the rows that share a 256-byte bank window over distinct chunk
//    positions, so 16 consecutive rows read the same logical chunk without
//    bank conflicts;
//  * V rows are read by ds_read_b64_tr_b16 with four consecutive rows per
//    16-lane group: swz(r) moves rows r..r+3 to distinct bank quads;
//  * V8 rows (64 bytes, one head-dim column of the tile-packed 8-bit V) are
//    read by ds_read_b128 with one row per lane, like K8.
template <int D>
struct AttnSwizzle {
  static constexpr int RP16 = 256 / (2 * D) > 1 ? 256 / (2 * D) : 1;   // rows per 256 B
  static constexpr int M16 = (D / 8 < 16 ? D / 8 : 16) - 1;
  static constexpr int RP8 = 256 / D > 1 ? 256 / D : 1;
  static constexpr int M8 = (D / 16 < 16 ? D / 16 : 16) - 1;
  __device__ static constexpr int k16(int r) { return (r / RP16) & M16; }
  __device__ static constexpr int k8(int r) { return (r / RP8) & M8; }
  __device__ static constexpr int v(int r) { return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }
  __device__ static constexpr int v8(int r) { return (r >> 2) & 3; }
  // row periods of the swizzles
  static constexpr int P16 = RP16 * (M16 + 1);
  static constexpr int P8 = RP8 * (M8 + 1);
  static constexpr int PV = 4;
};

// Waves per SIMD the register budget is sized for: two for D <= 128 so that
// one wave's MFMAs overlap the other's softmax arithmetic, one for D = 256.
template <int D>
struct AttnOccupancy {
  static constexpr int kWavesPerEU = D <= 128 ? 2 : 1;
};

template <int D, int NW, bool BF16, bool E4M3, bool ADAPTIVE, bool EXP8, bool PV8, bool DBG>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(AttnOccupancy<D>::kWavesPerEU, AttnOccupancy<D>::kWavesPerEU)))
void attn_fwd_kernel(const AttnArgs a) {
  using SH = AttnShape<D, NW>;
  static_assert(!PV8 || (EXP8 && !ADAPTIVE), "8-bit P V needs 8-bit weights and mask routing");
  // base-2 logits with a lazily moved reference maximum (exact in exact
  // arithmetic); used whenever no 8-bit rounding or flag decision depends on
  // the running maximum
  constexpr bool LAZY = !ADAPTIVE && !EXP8;
  constexpr float kLogScale = LAZY ? kLog2e : 1.f;
  // double-buffered K and V tiles as four distinct objects: copies into one
  // buffer and reads of another are then provably disjoint, so reads do not
  // wait for copies in flight
  __shared__ __attribute__((aligned(1024))) char sk0[SH::K16_BYTES];
  __shared__ __attribute__((aligned(1024))) char sk1[SH::K16_BYTES];
  __shared__ __attribute__((aligned(1024))) char sv0[SH::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char sv1[SH::V_BYTES];
  // adaptive mode: an 8-bit tile is staged both as K8 (here) and as K16 (in
  // sk0 / sk1), so that a flagged sub-block recomputes its logits from LDS
  __shared__ __attribute__((aligned(1024))) char sq0[ADAPTIVE ? SH::K8_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char sq1[ADAPTIVE ? SH::K8_BYTES : 16];
  // 8-bit exponentials: E4M3(exp(value(c))) for every e4m3 code c (not at
  // D = 256 in adaptive mode, whose tiles fill the LDS)
  constexpr bool EXP8_TAB = EXP8 && !(ADAPTIVE && D >= 256);
  __shared__ uint8_t exp8_tab[EXP8_TAB ? 256 : 4];

  // ---- workgroup -> (b, h, qt): XCD-contiguous chunks of the logical order
  //      (kv-head group, b) major, query tile descending, head minor.  The
  //      batch index varies fastest among the groups so that the sequences of
  //      a variable-length batch spread over the XCDs instead of loading some
  //      with the long ones. ----
  const int nblk = (int)gridDim.x, bid = (int)blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3, qn = nblk >> 3, rn = nblk & 7;
  const int lin = xcd * qn + min(xcd, rn) + slot;
  const int per_group = a.n_qt * a.heads_per_group;
  const int grp = lin / per_group;
  const int rem = lin - grp * per_group;
  const int qt = a.n_qt - 1 - rem / a.heads_per_group;
  const int hh = rem % a.heads_per_group;
  const int kvh = grp / a.B, b = grp % a.B;
  const int h = kvh * a.heads_per_group + hh;

  // lengths of this batch entry's sequence (a variable-length batch lives in
  // padded tensors); a query tile wholly in the padding has nothing to do
  const int Lq = a.seqlens_q != nullptr ? min(max(ld_uniform(a.seqlens_q + b), 0), a.S_q) : a.S_q;
  const int Lk = a.seqlens_k != nullptr ? min(max(ld_uniform(a.seqlens_k + b), 0), a.S_k) : a.S_k;
  if (qt * SH::TM >= Lq) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if constexpr (EXP8_TAB) {
    // (visible to all waves after the barrier ahead of the main loop)
    for (int c = tid; c < 256; c += SH::NT) exp8_tab[c] = (uint8_t)exp8_code((uint32_t)c);
  }
  // the wave index as a scalar, for the LDS destinations of the tile copies
  // (M0), so that they need no per-copy lane read
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int lr = lane & 31, hf = lane >> 5;
  const int row0 = qt * SH::TM + w * 32;
  const int my_row = row0 + lr;
  const bool wave_live = row0 < Lq;
  const int q_row = min(my_row, Lq - 1);

  // causal: query row i sits at key position i + coff and sees keys up to it
  const int coff = Lk - Lq;
  const int n_kt_seq = (Lk + SH::TN - 1) / SH::TN;
  const int wg_last = min(Lq, (qt + 1) * SH::TM) - 1;
  const int kt_end = a.causal ? min(n_kt_seq, (wg_last + coff) / 64 + 1) : n_kt_seq;
  const int w_last = min(Lq, row0 + 32) - 1;
  const int kt_end_w = !wave_live ? 0 : (a.causal ? min(n_kt_seq, (w_last + coff) / 64 + 1) : n_kt_seq);
  const bool rows_ragged = row0 + 32 > Lq;
  // largest valid key index of this lane's row (-1: padding row)
  const int key_lim = my_row >= Lq ? -1 : (a.causal ? min(my_row + coff, Lk - 1) : Lk - 1);

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop
  const char* qp = reinterpret_cast<const char*>(a.q) +
                   2 * (b * a.q_sb + h * a.q_sh + (int64_t)q_row * a.q_ss);
  u32x4 q16[SH::NQ16];
#pragma unroll
  for (int t = 0; t < SH::NQ16; ++t) q16[t] = ld_global16(qp + 2 * (16 * t + 8 * hf));
  const uint8_t* q8p = a.q8 + (((int64_t)b * a.Hq + h) * a.S_q + q_row) * D;
  u32x4 q8[SH::NQ8];
  if constexpr (E4M3) {
#pragma unroll
    for (int t = 0; t < D / 64; ++t) {
      q8[2 * t] = ld_global16(q8p + 64 * t + 32 * hf);
      q8[2 * t + 1] = ld_global16(q8p + 64 * t + 32 * hf + 16);
    }
  } else {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) q8[t] = ld_global16(q8p + 32 * t + 16 * hf);
  }
  const float sQ = ld_uniform(a.q_scale + ((int64_t)b * a.Hq + h) * a.n_qt + qt);
  const uint64_t* mrow = a.mask + (((int64_t)b * a.Hq + h) * a.n_qt + qt) * a.words_per_row;

  // per-head bases; offsets inside a head fit 32 bits (validated S <= 2^20)
  const char* kbase = reinterpret_cast<const char*>(a.k) + 2 * (b * a.k_sb + kvh * a.k_sh);
  const char* vbase = reinterpret_cast<const char*>(a.v) + 2 * (b * a.v_sb + kvh * a.v_sh);
  const uint8_t* k8base = a.k8 + ((int64_t)b * a.Hkv + kvh) * a.S_k * D;
  const float* sKp = a.k_scale + ((int64_t)b * a.Hkv + kvh) * a.n_kt;
  const uint32_t kss = 2u * (uint32_t)a.k_ss, vss = 2u * (uint32_t)a.v_ss;
  const int key_max = Lk - 1;

  // Mask bits of tiles 0, 1, 2, ... in order: the row's current mask word
  // stays in registers (reloaded when the group index enters the next word)
  // and the group index advances with a counter, so a step needs neither a
  // division nor a memory load to route its next tile.
  int rt_g = 0, rt_r = 0, rt_w = 0;
  uint64_t rt_word = ld_uniform(mrow);
  auto next_tile_is8 = [&]() -> bool {
    if (++rt_r == a.tiles_per_bit) {
      rt_r = 0;
      ++rt_g;
      if ((rt_g >> 6) != rt_w) {
        rt_w = rt_g >> 6;
        rt_word = ld_uniform(mrow + rt_w);
      }
    }
    return (rt_word >> (rt_g & 63)) & 1ull;
  };

  // ---- direct-to-LDS staging of one key tile.  Wave w issues copies
  // n = w + NW*j of each region; copy n fills 16-byte slots 64n .. 64n+63,
  // slot p = (row p / CH, position p % CH) holding logical chunk
  // position ^ swz(row).  Source offsets inside a tile are per-lane
  // constants; a tile adds key0 * row_stride to the (uniform) base. ----
  using SW = AttnSwizzle<D>;
  // Copy j + 1 of a region starts RS rows after copy j.  When RS is a
  // multiple of the region's swizzle period, every copy's per-lane offset is
  // the first copy's plus j * RS rows: one register serves all copies.
  constexpr int RS16 = (64 / SH::CH16) * NW, RS8 = (64 / SH::CH8) * NW;
  constexpr bool K16_1 = RS16 % SW::P16 == 0, K8_1 = RS8 % SW::P8 == 0, V_1 = RS16 % SW::PV == 0;
  uint32_t off_k16[K16_1 ? 1 : SH::JK16], off_k8[K8_1 ? 1 : SH::JK8], off_v[V_1 ? 1 : SH::JV];
#pragma unroll
  for (int j = 0; j < (K16_1 ? 1 : SH::JK16); ++j) {
    const int p = 64 * (w + NW * j) + lane, r = p / SH::CH16;
    off_k16[j] = (uint32_t)r * kss + (uint32_t)(((p % SH::CH16) ^ SW::k16(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < (K8_1 ? 1 : SH::JK8); ++j) {
    const int p = 64 * (w + NW * j) + lane, r = p / SH::CH8;
    off_k8[j] = (uint32_t)(r * D + (((p % SH::CH8) ^ SW::k8(r)) << 4));
  }
#pragma unroll
  for (int j = 0; j < (V_1 ? 1 : SH::JV); ++j) {
    const int p = 64 * (w + NW * j) + lane, r = p / SH::CH16;
    off_v[j] = (uint32_t)r * vss + (uint32_t)(((p % SH::CH16) ^ SW::v(r)) << 4);
  }
  // offset of copy j (the empty asm keeps the sums from being hoisted out
  // of the loop into registers of their own)
  auto copy_off = [](const uint32_t* off, bool one, int j, uint32_t row_step_bytes) -> uint32_t {
    if (!one) return off[j];
    uint32_t o = off[0];
    asm volatile("" : "+v"(o));
    return o + (uint32_t)j * row_step_bytes;
  };
  // tile-packed V8: copy n fills rows 16n .. 16n+15 (4 chunks of 16 bytes
  // each); lane l fills row 16n + l/4, position l%4, and swz of that row is
  // (l/16)%4 for every n, so one per-lane offset serves all copies
  const uint32_t off_v8 = (uint32_t)((lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4));
  const uint8_t* v8base = PV8 ? a.v8 + ((int64_t)b * a.Hkv + kvh) * a.n_kt * SH::V8_BYTES : nullptr;
  const float* sVp = PV8 ? a.v_scale + ((int64_t)b * a.Hkv + kvh) * a.n_kt : nullptr;
  // each tile's copies go through buffer resources that start at the tile's
  // first row and end with the head's last row: per-lane offsets past S_k
  // (ragged last tile) fall outside the resource and read zeros, which are
  // never valid logits
  const uint32_t k16_bytes = Lk > 0 ? (uint32_t)(Lk - 1) * kss + 2u * D : 0u;
  const uint32_t k8_bytes = (uint32_t)Lk * D;
  const uint32_t v_bytes = Lk > 0 ? (uint32_t)(Lk - 1) * vss + 2u * D : 0u;
  // per-step copy of the scalar wave index: the copies' LDS addresses are
  // then a few scalar adds per step instead of registers held (and spilled)
  // across the loop
  auto wave_s = [&]() {
    int v = wu;
    asm volatile("" : "+s"(v));
    return v;
  };
  // kdst: the K region (K16, or K8 outside the adaptive mode); kdst8: the
  // adaptive mode's K8 buffer
  auto issue_k = [&](int kt, bool is8, char* kdst, char* kdst8) {
    const int wu = wave_s();
    const uint32_t key0 = (uint32_t)(kt * SH::TN);
    if (is8) {
      const auto rs = make_rsrc(k8base + key0 * D, k8_bytes - key0 * D);
#pragma unroll
      for (int j = 0; j < SH::JK8; ++j)
        dma16_buf(rs, copy_off(off_k8, K8_1, j, (uint32_t)(RS8 * D)), 0u,
                  (ADAPTIVE ? kdst8 : kdst) + 1024 * (wu + NW * j));
    }
    if (!is8 || ADAPTIVE) {
      const auto rs = make_rsrc(kbase + key0 * kss, k16_bytes - key0 * kss);
#pragma unroll
      for (int j = 0; j < SH::JK16; ++j)
        dma16_buf(rs, copy_off(off_k16, K16_1, j, (uint32_t)RS16 * kss), 0u, kdst + 1024 * (wu + NW * j));
    }
  };
  auto issue_v = [&](int kt, bool is8, char* vdst) {
    const int wu = wave_s();
    if constexpr (PV8) {
      if (is8) {
        // whole tiles, always in bounds (the quantiser zero-fills keys past
        // the sequence)
        const uint8_t* src = v8base + (int64_t)kt * SH::V8_BYTES;
#pragma unroll
        for (int j = 0; j < SH::JV8; ++j)
          dma16(src + 1024 * (wu + NW * j) + off_v8, vdst + 1024 * (wu + NW * j));
        return;
      }
    }
    const uint32_t key0 = (uint32_t)(kt * SH::TN);
    const auto rv = make_rsrc(vbase + key0 * vss, v_bytes - key0 * vss);
#pragma unroll
    for (int j = 0; j < SH::JV; ++j)
      dma16_buf(rv, copy_off(off_v, V_1, j, (uint32_t)RS16 * vss), 0u, vdst + 1024 * (wu + NW * j));
  };

  // ---- per-lane LDS read offsets ----
  // K16 fragment t of key block kb: row kb*32 + lr, logical chunk 2t + hf
  const int s16 = SW::k16(lr), s8 = SW::k8(lr);
  int a16[SH::NQ16], a8[SH::NQ8];
#pragma unroll
  for (int t = 0; t < SH::NQ16; ++t) a16[t] = lr * SH::RB16 + (((2 * t + hf) ^ s16) << 4);
  // K8 fragment i: int8 logical chunk 2i + hf; e4m3 chunks 4(i/2) + 2hf + (i&1)
#pragma unroll
  for (int i = 0; i < SH::NQ8; ++i) {
    const int lc = E4M3 ? 4 * (i >> 1) + 2 * hf + (i & 1) : 2 * i + hf;
    a8[i] = lr * SH::RB8 + ((lc ^ s8) << 4);
  }
  // V through the transposing read: in 16-lane group g, source lane sl reads
  // key (base + 4hf + sl/4), head dims 32db + 16(g%2) + 4(sl%4) .. +3, so that
  // result lane l gets head dim 32db + l%32 and keys base + 4hf + 0..3
  int av[SH::ND];
  {
    const int sl = lane & 15, g1 = (lane >> 4) & 1;
    const int sv = SW::v(4 * hf + (sl >> 2));
#pragma unroll
    for (int db = 0; db < SH::ND; ++db) {
      const int lc = 4 * db + 2 * g1 + ((sl & 3) >> 1);
      av[db] = (4 * hf + (sl >> 2)) * SH::RB16 + ((lc ^ sv) << 4) + 8 * (sl & 1);
    }
  }

  // ---- online-softmax state of row my_row (lane-local; the two lane halves
  //      hold partial sums of l that are combined at the end) ----
  f32x16 O[SH::ND];
#pragma unroll
  for (int db = 0; db < SH::ND; ++db) O[db] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;
  uint64_t fword = 0;

  const int sb_index = qt * NW + w;      // 32-row sub-block of this wave
  uint64_t* frow = (ADAPTIVE && a.flags != nullptr && wave_live)
                       ? a.flags + (((int64_t)b * a.Hq + h) * a.n_sb + sb_index) * a.flag_words
                       : nullptr;
  const float sm = a.sm_scale;

  // element e of x[] (key block e/16, accumulator register e%16) holds key
  // key0 + kofs(e) + 4*hf of query row my_row
  auto kofs = [](int e) { return (e >> 4) * 32 + ((e & 15) >> 2) * 8 + (e & 3); };

  auto qk16_lds = [&](const char* kb, float* x) {
    u32x4 kf0[SH::NQ16], kf1[SH::NQ16];
#pragma unroll
    for (int t = 0; t < SH::NQ16; ++t) kf0[t] = ld_lds16(kb + a16[t]);
#pragma unroll
    for (int t = 0; t < SH::NQ16; ++t) kf1[t] = ld_lds16(kb + 32 * SH::RB16 + a16[t]);
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int t = 0; t < SH::NQ16; ++t) {
      acc0 = mfma16<BF16>(kf0[t], q16[t], acc0);
      acc1 = mfma16<BF16>(kf1[t], q16[t], acc1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = acc0[i];
      x[16 + i] = acc1[i];
    }
  };
  // int8 accumulator start value, kept in registers across the loop
  i32x16 acc_init;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc_init[i] = LAZY ? kMagicBits : 0;
  auto qk8_lds = [&](const char* kb, int key0, float* x) {
    u32x4 kf0[SH::NQ8], kf1[SH::NQ8];
#pragma unroll
    for (int i = 0; i < SH::NQ8; ++i) kf0[i] = ld_lds16(kb + a8[i]);
#pragma unroll
    for (int i = 0; i < SH::NQ8; ++i) kf1[i] = ld_lds16(kb + 32 * SH::RB8 + a8[i]);
    if constexpr (E4M3) {
      f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 64; ++t) {
        acc0 = mfma_e4m3(kf0[2 * t], kf0[2 * t + 1], q8[2 * t], q8[2 * t + 1], acc0);
        acc1 = mfma_e4m3(kf1[2 * t], kf1[2 * t + 1], q8[2 * t], q8[2 * t + 1], acc1);
      }
      xdl16_settle();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = acc0[i];
        x[16 + i] = acc1[i];
      }
    } else {
      // LAZY: the accumulator starts at the bits of the float 1.5 * 2^23, so
      // that its result bits are the float 1.5 * 2^23 + acc (exact: |acc| <=
      // 256 * 127^2 < 2^22), and no int -> float conversion is needed;
      // callers subtract kMagic.  Otherwise plain integers, converted.
      const int init = LAZY ? kMagicBits : 0;
      i32x16 acc[2];
      acc[0] = mfma_i8(kf0[0], q8[0], acc_init);
      acc[1] = mfma_i8(kf1[0], q8[0], acc_init);
#pragma unroll
      for (int t = 1; t < D / 32; ++t) {
        acc[0] = mfma_i8(kf0[t], q8[t], acc[0]);
        acc[1] = mfma_i8(kf1[t], q8[t], acc[1]);
      }
      if constexpr (DBG) {
        if (my_row < Lq) {
          int32_t* dr = a.dbg + (((int64_t)b * a.Hq + h) * a.S_q + my_row) * a.S_k;
#pragma unroll
          for (int e = 0; e < 32; ++e) {
            const int j = key0 + kofs(e) + 4 * hf;
            if (j < Lk) dr[j] = acc[e >> 4][e & 15] - init;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (LAZY) {
          // bit-cast from scalar copies: hipcc mistranslates a bit cast
          // applied directly to a vector-element lvalue (it reads element 0)
          const int v0 = acc[0][i], v1 = acc[1][i];
          x[i] = __builtin_bit_cast(float, v0);
          x[16 + i] = __builtin_bit_cast(float, v1);
        } else {
          x[i] = (float)acc[0][i];
          x[16 + i] = (float)acc[1][i];
        }
      }
    }
  };

  // ---- one key tile, split in three parts so that a wave can overlap the
  //      P V products of tile kt-1 with the softmax of tile kt ----
  // (1) logits of tile kt: x = raw scores, logit = (x - xoff) * c, or the
  //     logits themselves (scaled) with invalid entries -inf
  struct Logits {
    float c, xoff;
    bool is16, scaled;
  };
  // kb: the K region (K16, or K8 outside the adaptive mode); kb8: the
  // adaptive mode's K8 buffer
  auto qk_part = [&](int kt, const char* kb, const char* kb8, bool is8, float sK, float* x) -> Logits {
    const int key0 = kt * SH::TN;
    const bool need_mask = rows_ragged || (key0 + SH::TN > Lk) ||
                           (a.causal && key0 + SH::TN - 1 > row0 + coff);
    // valid(e) <=> kofs(e) <= lim_rel
    const int lim_rel = key_lim - key0 - 4 * hf;
    Logits lg;
    lg.xoff = 0.f;
    lg.is16 = !is8;
    lg.scaled = false;
    auto mask_scale = [&]() {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = kofs(e) <= lim_rel ? (x[e] - lg.xoff) * lg.c : kNegInf;
      lg.xoff = 0.f;
      lg.scaled = true;
    };
    if (is8) {
      qk8_lds(ADAPTIVE ? kb8 : kb, key0, x);
      lg.c = (sQ * sK) * sm * kLogScale;
      if constexpr (LAZY && !E4M3) {
        // 21 significant bits make kMagic * c exact, so that the offset can
        // be folded into the reference without a rounding
        lg.c = round_sig21(lg.c);
        lg.xoff = kMagic;
      }
    } else {
      qk16_lds(kb, x);
      lg.c = sm * kLogScale;
    }
    if (need_mask) mask_scale();
    if constexpr (ADAPTIVE) {
      if (is8) {
        // look-ahead: m' = max(m, rowmax s8); flag the 32-row sub-block if
        // some valid 8-bit logit is within tau of m'
        float mx8 = x[0];
#pragma unroll
        for (int e = 1; e < 32; ++e) mx8 = fmaxf(mx8, x[e]);
        if (!lg.scaled) mx8 *= lg.c;
        mx8 = halves_max(mx8);
        const float mprime = fmaxf(m_run, mx8);
        const bool cond = (mx8 != kNegInf) && (mx8 - mprime >= -a.tau);
        if (wave_any(cond)) {
          lg.is16 = true;
          fword |= 1ull << (kt & 63);
          // recompute the sub-block's logits at 16 bits from the tile's K16
          // copy in LDS
          qk16_lds(kb, x);
          lg.c = sm;
          lg.scaled = false;
          if (need_mask) mask_scale();
        }
      }
    }
    return lg;
  };

  // (2) O^T += V^T P^T for a tile whose 16-bit weights are pk
  auto pv_part = [&](const char* vb, const uint32_t* pk) {
#pragma unroll
    for (int kb_ = 0; kb_ < 2; ++kb_) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int i0 = kb_ * 8 + 4 * cc;
        const u32x4 pb = {pk[i0], pk[i0 + 1], pk[i0 + 2], pk[i0 + 3]};
        const char* vrow = vb + (32 * kb_ + 16 * cc) * SH::RB16;
#pragma unroll
        for (int db = 0; db < SH::ND; ++db) {
          const u32x2 lo = ld_lds_tr16(vrow + av[db]);
          const u32x2 hi = ld_lds_tr16(vrow + 8 * SH::RB16 + av[db]);
          O[db] = mfma16<BF16>(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, O[db]);
        }
      }
    }
  };

  // (2') 8-bit P V: O^T += V8^T P8^T * 2^e for a tile whose e4m3 weights are
  //      pk[0..7] (lane: query row lr, keys in score-register order, which
  //      is the tile-packed V8 key order); one K = 64 fp8 product per 32
  //      head-dim rows, the tile's power-of-two V scale as operand A's E8M0
  //      block scale
  auto pv8_part = [&](const char* vb, const uint32_t* pk, int svc) {
    const u32x4 p0 = {pk[0], pk[1], pk[2], pk[3]}, p1 = {pk[4], pk[5], pk[6], pk[7]};
    const int sw = SW::v8(lr);
#pragma unroll
    for (int db = 0; db < SH::ND; ++db) {
      const char* row = vb + (db * 32 + lr) * 64;
      const u32x4 a0 = ld_lds16(row + (((2 * hf) ^ sw) << 4));
      const u32x4 a1 = ld_lds16(row + (((2 * hf + 1) ^ sw) << 4));
      O[db] = mfma_e4m3_sa(a0, a1, p0, p1, O[db], svc);
    }
  };

  // Instruction order for the block holding P V of tile kt-1 and the
  // softmax of tile kt: a wave issues in order and an MFMA waits for the
  // matrix pipe, so the 16 MFMAs are spread over the softmax arithmetic
  // (V reads a few MFMAs ahead) instead of being issued back to back.
  auto interleave_pv_softmax = [&]() {
    constexpr int NMF = 4 * SH::ND;                        // P V MFMAs per tile
    constexpr int NVALU = D >= 256 ? 4 : (D == 64 ? 16 : 8);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);     // 6 LDS reads
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);   // VALU
    }
  };

  // (3) shared online-softmax update with the logits of tile kt; writes the
  //     weights to pk (16-bit pairs, or with the 8-bit P V on an 8-bit tile
  //     the e4m3 codes in pk[0..7]).  Any rescale of O applies to everything
  //     accumulated so far, P V of the previous tile included.  pvc: whether
  //     the block also holds the (16-bit) P V of the previous tile, whose
  //     products are then spread over the softmax arithmetic.
  auto softmax_part = [&](float* x, const Logits& lg, uint32_t* pk, auto pvc) {
    constexpr bool WITH_PV = decltype(pvc)::value;
    // LAZY after the first tile: the weights are taken against the current
    // reference and the row maximum is only needed when they grow too large
    // (WITH_PV holds exactly on the tiles after a row's first)
    constexpr bool MAXFREE = LAZY && WITH_PV;
    const float cm = lg.scaled ? 1.f : lg.c;
    // offset still in x (cleared when it is subtracted from x in place)
    float xo = lg.xoff;
    auto row_max = [&]() {
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) mx = fmaxf(mx, x[e]);
      mx = (mx - xo) * cm;
      return halves_max(mx);
    };
    // the normaliser sums exactly the rounded weights that feed P V
    auto psum = [&](const uint32_t* w16) {
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        ps0 = sum16x2<BF16>(w16[i], ps0);
        ps1 = sum16x2<BF16>(w16[i + 1], ps1);
      }
      return ps0 + ps1;
    };
    // LAZY, no branch: the weights against mref through the folded offset;
    // `exact` is false on a lane whose folded reference m + xoff * cm was
    // rounded (then these weights are not used: the caller weights again)
    auto weights_folded = [&](float mref, bool& exact) -> float {
      const float mr = (mref == kNegInf) ? 0.f : mref;
      const float t = xo * cm;
      const float msub = mr + t;
      const float bb = msub - mr;
      exact = ((mr - (msub - bb)) + (t - bb)) == 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pk[i] = pack16x2<BF16>(exp2_fast(__builtin_fmaf(x[2 * i], cm, -msub)),
                               exp2_fast(__builtin_fmaf(x[2 * i + 1], cm, -msub)));
      return psum(pk);
    };
    // the weights go to pk (LAZY keeps x; otherwise the fp32 weights
    // overwrite x in place); returns their sum
    auto weights = [&](float mref) -> float {
      if constexpr (LAZY) {
        // exp2((x - xoff) * cm - m) as exp2(x * cm - (m + xoff * cm)), one
        // rounding, when m + xoff * cm is exact in fp32: xoff * cm is exact
        // (cm has 21 significant bits) and the reference m is an integer, so
        // the sum is exact whenever its magnitude stays near xoff * cm's.
        // The rounding error of the sum (TwoSum) says which: otherwise the
        // offset is subtracted from each x first (exact: x = xoff + acc with
        // |acc| < 2^22), again one rounding per weight.
        const float mr = (mref == kNegInf) ? 0.f : mref;
        const float t = xo * cm;
        float msub = mr + t;
        const float bb = msub - mr;
        const float err = (mr - (msub - bb)) + (t - bb);
        if (wave_any(err != 0.f)) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e = 0; e < 32; ++e) x[e] -= xo;
          xo = 0.f;
          msub = mr;
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pk[i] = pack16x2<BF16>(exp2_fast(__builtin_fmaf(x[2 * i], cm, -msub)),
                                 exp2_fast(__builtin_fmaf(x[2 * i + 1], cm, -msub)));
        return psum(pk);
      } else {
        const float msub = (mref == kNegInf) ? 0.f : mref;
        if (EXP8 && !lg.is16) {
          // x = s - m rounded to e4m3, exp, rounded to e4m3 again; four
          // values per code word.  The final codes are the 8-bit P operand,
          // or are converted straight to the 16-bit one.
          // (the sum in the order of psum: even words, odd words)
          float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
          for (int e = 0; e < 32; e += 4) {
            float xs[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // (the table maps what the conversion makes of values below
              // -448 to a zero weight; without it, clamp at -448)
              xs[j] = __builtin_fmaf(x[e + j], cm, -msub);
              if constexpr (!EXP8_TAB) xs[j] = fmaxf(xs[j], -448.f);
            }
            const uint32_t xc = f32x4_to_e4m3(xs[0], xs[1], xs[2], xs[3]);
            uint32_t pc;
            if constexpr (EXP8_TAB) {
              pc = (uint32_t)exp8_tab[xc & 0xFFu] | ((uint32_t)exp8_tab[(xc >> 8) & 0xFFu] << 8) |
                   ((uint32_t)exp8_tab[(xc >> 16) & 0xFFu] << 16) |
                   ((uint32_t)exp8_tab[xc >> 24] << 24);
            } else {
              const f32x2 xlo = e4m3x2_to_f32<false>(xc), xhi = e4m3x2_to_f32<true>(xc);
              pc = f32x4_to_e4m3(exp2_fast(xlo.x * kLog2e), exp2_fast(xlo.y * kLog2e),
                                 exp2_fast(xhi.x * kLog2e), exp2_fast(xhi.y * kLog2e));
            }
            const uint32_t lo16 = e4m3x2_to_16<BF16, false>(pc), hi16 = e4m3x2_to_16<BF16, true>(pc);
            if constexpr (PV8) {
              pk[e >> 2] = pc;
            } else {
              pk[e >> 1] = lo16;
              pk[(e >> 1) + 1] = hi16;
            }
            ps0 = sum16x2<BF16>(lo16, ps0);
            ps1 = sum16x2<BF16>(hi16, ps1);
          }
          if constexpr (PV8) {
            // pk[8..15] are not read by the 8-bit product: let the old
            // 16-bit weights die instead of carrying them through
#pragma unroll
            for (int i = 8; i < 16; ++i) pk[i] = __builtin_nondeterministic_value(pk[i]);
          }
          return ps0 + ps1;
        } else {
          const float c2 = cm * kLog2e, m2 = msub * kLog2e;
#pragma unroll
          for (int e = 0; e < 32; ++e) x[e] = exp2_fast(__builtin_fmaf(x[e], c2, -m2));
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) pk[i] = pack16x2<BF16>(x[2 * i], x[2 * i + 1]);
      return psum(pk);
    };
    // New reference maximum, chosen before the weights (a select, no
    // branch), so that max, weights, packing and the row sum stay in one
    // basic block with the P V products issued before them; the rescale of
    // O and l and the update of m_run follow in a rare branch.  LAZY moves
    // the reference only when a row's max grows by more than 8 (so p <= 2^8
    // in between); the exact modes track the running maximum.
    if constexpr (MAXFREE) {
      // Weights against the current reference first.  A lane's weights are
      // all at most their sum, so a sum up to 2^16 keeps every weight in
      // range; above it (or before any reference exists) the row maximum
      // moves the reference and the tile is weighted again.  The rescale
      // applies to everything accumulated so far, P V of the previous tile
      // included.
      // The folded reference has no branch, so the weights share one block
      // with the P V products and are interleaved with them; a lane whose
      // folded reference was rounded sends the wave to the rare branch too.
      bool exact;
      float l_add = weights_folded(m_run, exact);
      asm volatile("" : "+v"(l_add));
      interleave_pv_softmax();
      if (wave_any((l_add > 65536.f) | (m_run == kNegInf) | !exact)) {
        __builtin_amdgcn_sched_barrier(0);
        const float m_new = ceilf(fmaxf(m_run, row_max()));
        l_add = weights(m_new);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < SH::ND; ++db) O[db] *= alpha;
        m_run = m_new;
      }
      l_run += l_add;
      return;
    }
    const float mx = row_max();
    bool move;
    float m_new;
    if constexpr (LAZY) {
      // the reference stays an integer (base-2 units), which keeps the
      // folded offset exact and makes alpha an exact power of two
      move = wave_any(mx > m_run + 8.f);
      m_new = move ? ceilf(fmaxf(m_run, mx)) : m_run;
    } else {
      m_new = fmaxf(m_run, mx);
      move = wave_any(m_new != m_run);
    }
    float l_add = weights(m_new);
    // the weights must precede the branch (otherwise it is hoisted above
    // them, which splits them off the P V products)
    asm volatile("" : "+v"(l_add));
    if constexpr (WITH_PV) interleave_pv_softmax();
    if (move) {
      __builtin_amdgcn_sched_barrier(0);
      // an 8-bit P V product may have written O shortly before
      if constexpr (PV8) xdl16_settle();
      float alpha;
      if constexpr (LAZY) alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m_run - m_new);
      else alpha = (m_run == kNegInf) ? 0.f : exp2_fast((m_run - m_new) * kLog2e);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < SH::ND; ++db) O[db] *= alpha;
      m_run = m_new;
    }
    l_run += l_add;
  };

  // ---- main loop over key tiles, ascending.  Step kt computes the logits
  // of tile kt (K from one K buffer), P V of tile kt-1 (V from one V
  // buffer) and the softmax of tile kt, while K of tile kt+1 and V of tile
  // kt are copied into the other buffers; the barrier at the end of a step
  // publishes the copies and retires the buffers just read.  The loop is
  // unrolled by two so that every access names its buffer statically. ----
  uint32_t pk[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pk[i] = 0u;
  bool is8_cur = rt_word & 1ull;
  // sK of the current tile and the next one; a step loads the one after
  // that, a step ahead of its use
  float sk_cur = ld_uniform(sKp);
  float sk_n1 = a.n_kt > 1 ? ld_uniform(sKp + 1) : 0.f;
  // route and V scale (E8M0 code) of the tile whose P V is pending
  bool is8_prev = false;
  int svc_cur = 127, svc_prev = 127;
  using True_ = std::integral_constant<bool, true>;
  using False_ = std::integral_constant<bool, false>;
  // P V with no softmax to overlap (ragged waves, the last tile)
  auto pv_tile = [&](const char* vb, bool is8p, int svc) {
    if constexpr (PV8) {
      // one-sided blocks, as in the main step
      int p8 = is8p ? 1 : 0;
      xdl16_settle();
      if (p8) pv8_part(vb, pk, svc);
      xdl16_settle();
      asm volatile("" : "+s"(p8));
      if (!p8) pv_part(vb, pk);
    } else {
      pv_part(vb, pk);
    }
  };
  issue_k(0, is8_cur, sk0, sq0);
  wait_vmem();
  __syncthreads();
  // FIRST: tile 0, which has no previous tile to multiply with V
  auto step = [&](auto first, int kt, const char* kcur, char* knxt, const char* kcur8, char* knxt8,
                  const char* vprev, char* vcur) {
    constexpr bool FIRST = decltype(first)::value;
    bool is8_next = false;
    if (kt + 1 < kt_end) is8_next = next_tile_is8();
    // (after the mask bit, so that a wait for a reloaded mask word does not
    // also wait for this load)
    const float sk_n2 = kt + 2 < kt_end ? ld_uniform(sKp + kt + 2) : 0.f;
    if (kt + 1 < kt_end) issue_k(kt + 1, is8_next, knxt, knxt8);
    if constexpr (PV8) {
      if (is8_cur) svc_cur = (int)((__builtin_bit_cast(uint32_t, ld_uniform(sVp + kt)) >> 23) & 0xFFu);
    }
    issue_v(kt, is8_cur, vcur);
    if (kt < kt_end_w) {
      float x[32];
      const Logits lg = qk_part(kt, kcur, kcur8, is8_cur, sk_cur, x);
      if constexpr (FIRST) {
        softmax_part(x, lg, pk, False_{});
      } else if constexpr (PV8) {
        // P V of the previous tile (8- or 16-bit), then the softmax.  Two
        // one-sided blocks instead of an if/else: with both arms updating O
        // the register allocator gives O different registers in each arm
        // and copies all of it at the join (and then spills); the opaque
        // flag keeps the blocks from being merged back into an if/else.
        int p8 = is8_prev ? 1 : 0;
        if (p8) pv8_part(vprev, pk, svc_prev);
        asm volatile("" : "+s"(p8));
        if (!p8) pv_part(vprev, pk);
        softmax_part(x, lg, pk, False_{});
      } else {
        // a wave in this block (P V products spread over the softmax
        // arithmetic) takes issue priority over the other wave on its SIMD
        // (which runs its own steps, usually for the other workgroup on the
        // CU) while that one computes its logits: the matrix pipe is fed
        // and the other wave's instructions fill the gaps
        __builtin_amdgcn_s_setprio(1);
        pv_part(vprev, pk);
        softmax_part(x, lg, pk, True_{});
        __builtin_amdgcn_s_setprio(0);
      }
    } else if (!FIRST && kt - 1 < kt_end_w) {
      pv_tile(vprev, is8_prev, svc_prev);
    }
    if constexpr (ADAPTIVE) {
      if (((kt & 63) == 63) || kt == kt_end - 1) {
        if (frow != nullptr && lane == 0) frow[kt >> 6] = fword;
        fword = 0;
      }
    }
    wait_vmem();
    __syncthreads();
    is8_prev = is8_cur;
    svc_prev = svc_cur;
    is8_cur = is8_next;
    sk_cur = sk_n1;
    sk_n1 = sk_n2;
  };
  if (kt_end > 0) step(True_{}, 0, sk0, sk1, sq0, sq1, sv1, sv0);
  for (int kt = 1; kt < kt_end; kt += 2) {
    step(False_{}, kt, sk1, sk0, sq1, sq0, sv0, sv1);
    if (kt + 1 < kt_end) step(False_{}, kt + 1, sk0, sk1, sq0, sq1, sv1, sv0);
  }
  // P V of the last tile (its V was copied in the last step)
  if (kt_end_w == kt_end && kt_end > 0) {
    if ((kt_end - 1) & 1) pv_tile(sv1, is8_prev, svc_prev);
    else pv_tile(sv0, is8_prev, svc_prev);
  }
  if constexpr (ADAPTIVE) {
    if (frow != nullptr && lane == 0) {
      for (int wd = ((kt_end - 1) >> 6) + 1; wd < a.flag_words; ++wd) frow[wd] = 0;
    }
  }
  // ---- epilogue: O = acc / l, 16-bit store, optional LSE ----
  const float l_tot = halves_sum(l_run);
  if (wave_live && my_row < Lq) {
    // a row without any valid key (variable-length batch) gets O = 0
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* op = reinterpret_cast<char*>(a.out) +
               2 * (b * a.o_sb + h * a.o_sh + (int64_t)my_row * a.o_ss);
#pragma unroll
    for (int db = 0; db < SH::ND; ++db) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d0 = db * 32 + ii * 8 + hf * 4;
        const u32x2 v2 = {pack16x2<BF16>(O[db][4 * ii] * inv_l, O[db][4 * ii + 1] * inv_l),
                          pack16x2<BF16>(O[db][4 * ii + 2] * inv_l, O[db][4 * ii + 3] * inv_l)};
        *reinterpret_cast<u32x2*>(op + 2 * d0) = v2;
      }
    }
    if (a.lse != nullptr && hf == 0) {
      const float lg = __builtin_amdgcn_logf(l_tot);      // log2
      const float lse = l_tot > 0.f ? (LAZY ? (m_run + lg) * kLn2 : m_run + lg * kLn2) : kNegInf;
      a.lse[((int64_t)b * a.Hq + h) * a.S_q + my_row] = lse;
    }
  }
}

}  // namespace lamp
