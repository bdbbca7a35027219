// Per-block Q/K quantiser, V tile quantiser and mask builders (gfx950).
//
// Quantiser: TileMix page, section 2 "The Dual-Path Engine" (Q and K
// quantised with per-block scale factors); LampAttention abstract (8-bit
// floating point).  One workgroup per (b, h, block) of block_rows x D
// elements; HBM-bound: the block is read once into registers, reduced to its
// absmax, and written back as one byte per element.
//
// Mask builder: TileMix page, section 2 "Packed Bitmasks" (per query row,
// one bit per group of key tiles, 1 = 8-bit).  One thread per uint64 word;
// each bit is a SplitMix64 draw (Steele, Lea & Flood, OOPSLA 2014) compared
// with the 16-bit fraction.
#include "lamp_device.h"
#include "lamp_internal.h"

namespace lamp {

namespace {

constexpr int kQuantThreads = 256;

// Largest of the two 16-bit lanes, each taken as an unsigned integer.
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Byte 0 of each of four words, packed low to high.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return lo | (hi << 16);
}

template <bool BF16, bool E4M3, int CPT>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(QuantArgs a) {
  const int blk = blockIdx.x % a.nb;
  const int bh = blockIdx.x / a.nb;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int r0 = blk * a.block_rows;
  const int rows = min(a.block_rows, a.S - r0);
  // rows at or past the sequence length are padding: not read, zero
  const int len = a.seqlens != nullptr ? min(max(ld_uniform(a.seqlens + b), 0), a.S) : a.S;
  const int rows_live = min(rows, max(len - r0, 0));
  // 8-element chunks: D / 8 per row (a power of two), chunk c = row * D / 8 +
  // column / 8, so the live rows' chunks are exactly c < n_live
  const int cs = a.chunk_shift;
  const int nch = rows << cs;
  const int n_live = rows_live << cs;
  const char* base = reinterpret_cast<const char*>(a.x) +
                     2 * (b * a.sb + h * a.sh + (int64_t)r0 * a.ss);
  const int tid = threadIdx.x;

  // every load is issued unconditionally (a dead chunk reads chunk 0 of the
  // block, which exists, and is zeroed afterwards), so that a thread's loads
  // are in flight together instead of one at a time
  u32x4 cache[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * kQuantThreads;
    const int cl = c < n_live ? c : 0;
    const int r = cl >> cs, col = (cl & ((1 << cs) - 1)) * 8;
    cache[i] = ld_global16(base + 2 * ((int64_t)r * a.ss + col));
  }
  // absmax on the bit patterns: for finite fp16 / bf16 values the magnitude
  // bits (sign cleared) order like the magnitudes themselves
  uint32_t am2 = 0u;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * kQuantThreads;
    if (!(c < n_live)) cache[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) am2 = max_u16x2(am2, cache[i][e] & 0x7FFF7FFFu);
  }
  uint32_t am = max(am2 & 0xFFFFu, am2 >> 16);
  // block absmax: wave butterfly, then across the 4 waves through LDS
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 64));
  __shared__ uint32_t red[kQuantThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  am = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) am = max(am, red[w]);
  const float amax = from16<BF16>(am);

  const float qmax = E4M3 ? 448.f : 127.f;
  const bool nz = amax > 0.f;
  const float scale = nz ? amax / qmax : 0.f;   // IEEE division, RNE
  const float inv = nz ? qmax / amax : 0.f;
  if (tid == 0) a.scales[((int64_t)b * a.H + h) * a.nb + blk] = scale;

  uint8_t* out = reinterpret_cast<uint8_t*>(a.codes) + (((int64_t)b * a.H + h) * a.S + r0) * a.D;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * kQuantThreads;
    if (c < nch) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] = from16<BF16>(cache[i][e] & 0xFFFFu) * inv;
        y[2 * e + 1] = from16<BF16>(cache[i][e] >> 16) * inv;
      }
      u32x2 packed;
      if constexpr (E4M3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(y[e], -448.f), 448.f);
        packed.x = f32x4_to_e4m3(y[0], y[1], y[2], y[3]);
        packed.y = f32x4_to_e4m3(y[4], y[5], y[6], y[7]);
        // an all-zero block encodes as +0 whatever the sign of its zeros
        if (!nz) packed = u32x2{0u, 0u};
      } else {
        // |y| <= 127 (1 + 2^-24)^2 < 127.5, so round-half-even(y) lies in
        // [-127, 127] with no clamp.  y + 1.5 * 2^23 is rounded once, to an
        // integer (the constant is even, so ties go the same way as for y),
        // and its low byte is that integer in two's complement.  The sum
        // must not be fused with the product y = x * inv.
        uint32_t t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma clang fp contract(off)
          t[e] = __builtin_bit_cast(uint32_t, y[e] + 12582912.f);
        }
        packed = u32x2{pack_low_bytes(t[0], t[1], t[2], t[3]), pack_low_bytes(t[4], t[5], t[6], t[7])};
      }
      // (int8: an all-zero block has inv = 0, so every y is +-0, every code 0)
      const int r = c >> cs, col = (c & ((1 << cs) - 1)) * 8;
      *reinterpret_cast<u32x2*>(out + (int64_t)r * a.D + col) = packed;
    }
  }
}

template <bool BF16, bool E4M3>
hipError_t launch_quant_t(const QuantArgs& a, int cpt, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.nb)), block(kQuantThreads);
  switch (cpt) {
    case 4: hipLaunchKernelGGL((quantize_kernel<BF16, E4M3, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((quantize_kernel<BF16, E4M3, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((quantize_kernel<BF16, E4M3, 16>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((quantize_kernel<BF16, E4M3, 32>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// V for the 8-bit P V product: one workgroup per (b, h, 64-key tile), e4m3
// codes with one power-of-two scale 2^e per tile (e the smallest integer with
// absmax <= 448 * 2^e, clamped to [-126, 126]; 0 for an all-zero tile).  The
// output is tile-packed: row d of the tile holds the 64 keys of column d in
// the order of the attention kernel's score registers (position 32 c + p,
// key 32 (p / 16) + 8 ((p % 16) / 4) + p % 4 + 4 c).  Thread t owns the
// half-rows hr = t + 256 i (column hr % D, half hr / D): consecutive threads
// read consecutive columns of one key row, then write 32 contiguous bytes.
template <bool BF16, int D>
__global__ __launch_bounds__(kQuantThreads) void quantize_v_kernel(VQuantArgs a) {
  constexpr int HRT = (2 * D + kQuantThreads - 1) / kQuantThreads;
  const int kt = blockIdx.x % a.n_kt;
  const int bh = blockIdx.x / a.n_kt;
  const int h = bh % a.H;
  const int b = bh / a.H;
  // keys at or past the sequence length are padding: not read, zero
  const int len = a.seqlens != nullptr ? min(max(ld_uniform(a.seqlens + b), 0), a.S) : a.S;
  const char* base = reinterpret_cast<const char*>(a.v) + 2 * (b * a.sb + h * a.sh);
  const int tid = threadIdx.x;

  // every load is issued unconditionally from a clamped key (row S - 1
  // exists) and dead elements are zeroed afterwards, so that a thread's
  // loads are in flight together instead of one at a time
  uint16_t raw[HRT][32];
#pragma unroll
  for (int i = 0; i < HRT; ++i) {
    const int hr = tid + i * kQuantThreads;
    const int d = hr % D, c = hr / D;
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      const int key = kt * 64 + 32 * (p >> 4) + 8 * ((p & 15) >> 2) + (p & 3) + 4 * c;
      raw[i][p] = *reinterpret_cast<const uint16_t*>(base + 2 * ((int64_t)min(key, a.S - 1) * a.ss + d));
    }
  }
  float val[HRT][32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < HRT; ++i) {
    const int hr = tid + i * kQuantThreads;
    const int c = hr / D;
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      const int key = kt * 64 + 32 * (p >> 4) + 8 * ((p & 15) >> 2) + (p & 3) + 4 * c;
      const float x = (hr < 2 * D && key < len) ? from16<BF16>(raw[i][p]) : 0.f;
      val[i][p] = x;
      amax = fmaxf(amax, fabsf(x));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float red[kQuantThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, red[w]);

  // amax = f * 2^k, f in [0.5, 1); 448 = 0.875 * 2^9
  int e = 0;
  if (amax > 0.f) {
    int k;
    const float f = frexpf(amax, &k);
    e = min(max(k - 9 + (f > 0.875f ? 1 : 0), -126), 126);
  }
  const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);   // 2^-e, exact
  if (tid == 0)
    a.scales[((int64_t)b * a.H + h) * a.n_kt + kt] = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);

  uint8_t* out = a.codes + (((int64_t)b * a.H + h) * a.n_kt + kt) * (int64_t)(D * 64);
#pragma unroll
  for (int i = 0; i < HRT; ++i) {
    const int hr = tid + i * kQuantThreads;
    if (hr >= 2 * D) continue;
    const int d = hr % D, c = hr / D;
    uint32_t wd[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // an all-zero tile encodes as +0 whatever the sign of its zeros
      wd[q] = amax > 0.f ? f32x4_to_e4m3(val[i][4 * q] * inv, val[i][4 * q + 1] * inv,
                                         val[i][4 * q + 2] * inv, val[i][4 * q + 3] * inv)
                         : 0u;
    }
    char* dst = reinterpret_cast<char*>(out + d * 64 + 32 * c);
    *reinterpret_cast<u32x4*>(dst) = u32x4{wd[0], wd[1], wd[2], wd[3]};
    *reinterpret_cast<u32x4*>(dst + 16) = u32x4{wd[4], wd[5], wd[6], wd[7]};
  }
}

template <bool BF16>
hipError_t launch_quant_v_t(const VQuantArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)a.B * a.H * a.n_kt)), block(kQuantThreads);
  switch (a.D) {
    case 64: hipLaunchKernelGGL((quantize_v_kernel<BF16, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((quantize_v_kernel<BF16, 128>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((quantize_v_kernel<BF16, 256>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One wave per mask word: lane i hashes group 64 w + i and the wave's ballot
// is the word (groups past n_g give 0 bits).
__global__ __launch_bounds__(64 * kMaskWordsPerBlock) void build_mask_kernel(MaskArgs a) {
  const int64_t wid = (int64_t)blockIdx.x * kMaskWordsPerBlock + (threadIdx.x >> 6);
  if (wid >= a.total_words) return;                 // uniform across the wave
  const int lane = (int)(threadIdx.x & 63u);
  const int64_t row = wid / a.words_per_row;        // (b*Hq + h)*n_qt + qt
  const int w = (int)(wid % a.words_per_row);
  const uint64_t thr = a.per_head ? a.head_threshold[(row / a.n_qt) % a.Hq] : a.threshold;
  const int g = w * 64 + lane;
  bool is8 = false;
  if (g < a.n_g) {
    const uint64_t idx = (uint64_t)row * (uint64_t)a.n_g + (uint64_t)g;
    is8 = !((splitmix64(a.seed, idx) >> 32) < thr);
  }
  const uint64_t word = (uint64_t)__ballot(is8);
  if (lane == 0) a.mask[wid] = word;
}

// Structured template: one thread per mask word; the rule depends only on
// the query tile and the group.
__global__ __launch_bounds__(256) void build_mask_template_kernel(TemplateMaskArgs a) {
  const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wid >= a.total_words) return;
  const int64_t row = wid / a.words_per_row;        // (b*Hq + h)*n_qt + qt
  const int w = (int)(wid % a.words_per_row);
  const int qt = (int)(row % a.n_qt);
  // key position of the tile's last row (floor division: it may be negative)
  const int64_t pos = (int64_t)(qt + 1) * a.tile_m - 1 + a.pos_off;
  const int64_t gpos = pos >= 0 ? pos / a.group_keys : -((-pos + a.group_keys - 1) / a.group_keys);
  const int gq = (int)min((int64_t)a.n_g - 1, max((int64_t)0, gpos));
  uint64_t word = 0;
  const int g0 = w * 64;
  const int gn = min(64, a.n_g - g0);
  for (int i = 0; i < gn; ++i) {
    const int g = g0 + i;
    const int d = gq >= g ? gq - g : g - gq;
    const bool is16 = g < a.sink || d < a.band || (a.stride > 0 && d % a.stride == 0);
    word |= (uint64_t)(!is16) << i;
  }
  a.mask[wid] = word;
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t nch = (int64_t)a.block_rows * (a.D / 8);
  const int need = (int)((nch + kQuantThreads - 1) / kQuantThreads);
  const int cpt = need <= 4 ? 4 : need <= 8 ? 8 : need <= 16 ? 16 : 32;
  if (a.bf16) {
    return a.e4m3 ? launch_quant_t<true, true>(a, cpt, s) : launch_quant_t<true, false>(a, cpt, s);
  }
  return a.e4m3 ? launch_quant_t<false, true>(a, cpt, s) : launch_quant_t<false, false>(a, cpt, s);
}

hipError_t launch_quantize_v(const VQuantArgs& a, hipStream_t s) {
  return a.bf16 ? launch_quant_v_t<true>(a, s) : launch_quant_v_t<false>(a, s);
}

// The attention kernel's 8-bit exponential table, one thread per code.
__global__ __launch_bounds__(256) void exp8_table_kernel(uint8_t* out) {
  out[threadIdx.x] = (uint8_t)exp8_code(threadIdx.x);
}

hipError_t launch_exp8_table(uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(exp8_table_kernel, dim3(1), dim3(256), 0, s, out);
  return hipGetLastError();
}

hipError_t launch_build_mask(const MaskArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.total_words + kMaskWordsPerBlock - 1) / kMaskWordsPerBlock);
  hipLaunchKernelGGL(build_mask_kernel, dim3(blocks), dim3(64 * kMaskWordsPerBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_build_mask_template(const TemplateMaskArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.total_words + 255) / 256);
  hipLaunchKernelGGL(build_mask_template_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lamp
