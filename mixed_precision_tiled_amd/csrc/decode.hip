// Attention over an int8 key/value cache (decode), gfx950.
//
// Source: "TileMix: Mixed-Precision Attention for Faster LLM Prefill",
// section 4: the method supports INT8 key/value caches, which matter for the
// decode phase.  The cache holds K and V as int8 codes with one fp32 scale
// per block of 64 keys (the per-block quantiser's output); the few new
// queries are quantised the same way, so a logit is the 8-bit path's
// (cq . ck) * sQ * sK * sm, and the output uses the dequantised values
// sV * cv.
//
// Decode is bound by reading the cache from HBM (2 D bytes per key, once).
// Split-K over the keys:
//   * decode_split_kernel: one wave per (b, kv head, split of 512 to 2048 keys,
//     sized to give the grid about one wave per SIMD); the
//     group's queries (heads_per_group x S_q <= 32 columns) are the B operand
//     of int8 32x32x32 MFMAs (S^T = K8 Q8^T, K8 straight from global memory
//     into registers, each byte read once, the next tile's codes in flight
//     while one is computed); online softmax per column (the key mask only
//     on tiles that reach past a column's last key, O rescaled only when a
//     column's maximum moves); V
//     codes are converted to 16 bits into LDS in the prefill kernel's layout
//     and multiplied as O^T += V^T P^T, with sV folded into P.  Each wave
//     writes its unnormalised partial (m, l, O) to the caller's workspace;
//   * decode_merge_kernel: one workgroup per (b, KV head, column) combines
//     the splits' partials (log-sum-exp merge) and writes O and LSE.
#include <mutex>

#include "attn_kernel.h"
#include "lamp_internal.h"

// Fixed scratch for the split partials of lamp_decode_fwd_noalloc: a
// file-scope device array, one copy per GPU.  Host code never passes its
// name to a kernel (in host code the name is not a device address); it uses
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[lamp::kDecodeScratchBytes];

namespace lamp {

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

constexpr int kMergeThreads = 128;

template <int D, bool BF16>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using SH = AttnShape<D, 1>;
  using SW = AttnSwizzle<D>;
  __shared__ __attribute__((aligned(1024))) char sv[SH::V_BYTES];   // one V tile, 16-bit

  const int split = (int)(blockIdx.x % (unsigned)a.n_split);
  const int grp = (int)(blockIdx.x / (unsigned)a.n_split);          // b * Hkv + kvh
  const int b = grp / a.Hkv, kvh = grp % a.Hkv;
  const int lane = threadIdx.x, lr = lane & 31, hf = lane >> 5;

  // column of this lane: query row i of head hh of the KV group
  const bool col_live = lr < a.cols;
  const int cc = col_live ? lr : 0;
  const int hh = cc / a.S_q, i = cc % a.S_q;
  const int h = kvh * a.hpg + hh;
  const uint8_t* q8p = a.q8 + (((int64_t)b * a.Hq + h) * a.S_q + i) * D;
  u32x4 q8[SH::NQ8];
#pragma unroll
  for (int t = 0; t < SH::NQ8; ++t) q8[t] = ld_global16(q8p + 32 * t + 16 * hf);
  const float sQ = a.q_scale[((int64_t)b * a.Hq + h) * a.n_qt + i / a.tile_m];
  // largest key this column may see (-1: a padding column)
  const int key_lim = !col_live ? -1 : (a.causal ? min(i + a.S_k - a.S_q, a.S_k - 1) : a.S_k - 1);
  // a tile needs the key mask only if it reaches past a live column's limit
  // (padding columns are never written)
  const int key_lim_m = col_live ? key_lim : 0x7FFFFFFF;

  const uint8_t* k8base = a.k8 + (int64_t)grp * a.S_k * D;
  const uint8_t* v8base = a.v8 + (int64_t)grp * a.S_k * D;
  const float* sKp = a.k_scale + (int64_t)grp * a.n_kt;
  const float* sVp = a.v_scale + (int64_t)grp * a.n_kt;

  // V read offsets (transposing reads), as in the prefill kernel
  int av[SH::ND];
  {
    const int sl = lane & 15, g1 = (lane >> 4) & 1;
    const int svz = SW::v(4 * hf + (sl >> 2));
#pragma unroll
    for (int db = 0; db < SH::ND; ++db) {
      const int lc = 4 * db + 2 * g1 + ((sl & 3) >> 1);
      av[db] = (4 * hf + (sl >> 2)) * SH::RB16 + ((lc ^ svz) << 4) + 8 * (sl & 1);
    }
  }
  auto kofs = [](int e) { return (e >> 4) * 32 + ((e & 15) >> 2) * 8 + (e & 3); };

  f32x16 O[SH::ND];
#pragma unroll
  for (int db = 0; db < SH::ND; ++db) O[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c_log = a.sm_scale * kLog2e * sQ;

  const int kt0 = split * a.tiles_per_split, kt1 = min(a.n_kt, kt0 + a.tiles_per_split);
  // One tile's codes in registers: K as the A operand (rows key0 + 32 kb +
  // lr, clamped; masked below) and V one key row per lane.  The loads of
  // tile kt+1 are issued before tile kt is computed, so a wave always has a
  // tile in flight while it computes.
  struct TileCodes {
    u32x4 kf0[SH::NQ8], kf1[SH::NQ8];
    u32x4 vcode[D / 16];
  };
  auto load_tile = [&](int kt, TileCodes& tc) {
    const int key0 = kt * SH::TN;
    const uint8_t* p0 = k8base + (int64_t)min(key0 + lr, a.S_k - 1) * D + 16 * hf;
    const uint8_t* p1 = k8base + (int64_t)min(key0 + 32 + lr, a.S_k - 1) * D + 16 * hf;
#pragma unroll
    for (int t = 0; t < SH::NQ8; ++t) {
      tc.kf0[t] = ld_global16(p0 + 32 * t);
      tc.kf1[t] = ld_global16(p1 + 32 * t);
    }
    const uint8_t* pv = v8base + (int64_t)min(key0 + lane, a.S_k - 1) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) tc.vcode[c] = ld_global16(pv + 16 * c);
    // keep the loads here, ahead of the computation they overlap
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_tile = [&](int kt, const TileCodes& tc) {
    const int key0 = kt * SH::TN;
    const u32x4* kf0 = tc.kf0;
    const u32x4* kf1 = tc.kf1;
    const u32x4* vcode = tc.vcode;
    const float sK = ld_uniform(sKp + kt), sV = ld_uniform(sVp + kt);

    // logits (base 2) of the 64 keys x 32 columns
    i32x16 acc0 = i32x16{}, acc1 = i32x16{};
#pragma unroll
    for (int t = 0; t < SH::NQ8; ++t) {
      acc0 = mfma_i8(kf0[t], q8[t], acc0);
      acc1 = mfma_i8(kf1[t], q8[t], acc1);
    }
    const float c = c_log * sK;
    float x[32];
    if (wave_any(key0 + SH::TN - 1 > key_lim_m)) {
      const int lim_rel = key_lim - key0 - 4 * hf;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v0 = acc0[e], v1 = acc1[e];
        x[e] = kofs(e) <= lim_rel ? (float)v0 * c : kNegInf;
        x[16 + e] = kofs(16 + e) <= lim_rel ? (float)v1 * c : kNegInf;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[e] = (float)acc0[e] * c;
        x[16 + e] = (float)acc1[e] * c;
      }
    }
    // online softmax with the exact running maximum; the rescale of O and l
    // by alpha = exp2(m_old - m_new) is skipped when no column's maximum
    // moved (alpha would be exactly 1)
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, x[e]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float msub = m_new == kNegInf ? 0.f : m_new;
    float psum = 0.f;
    uint32_t pk[16];
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      const float p0 = exp2_fast(x[e] - msub), p1 = exp2_fast(x[e + 1] - msub);
      psum += p0 + p1;
      pk[e >> 1] = pack16x2<BF16>(p0 * sV, p1 * sV);     // the V scale rides on P
    }
    if (wave_any(m_new != m_run)) {
      const float alpha = m_run == kNegInf ? 0.f : exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < SH::ND; ++db) O[db] *= alpha;
      m_run = m_new;
    }
    l_run += psum;

    // V codes -> 16-bit into LDS: row = key, logical 16-byte chunk lc at
    // position lc ^ swz(row) (the prefill kernel's V layout)
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t word = vcode[c][2 * half + (j >> 1)];
          const int sh = 16 * (j & 1);
          const float f0 = (float)(int)(int8_t)(uint8_t)(word >> sh);
          const float f1 = (float)(int)(int8_t)(uint8_t)(word >> (sh + 8));
          w[j] = pack16x2<BF16>(f0, f1);
        }
        const int lc = 2 * c + half;
        st_lds16(sv + lane * SH::RB16 + ((lc ^ SW::v(lane)) << 4), u32x4{w[0], w[1], w[2], w[3]});
      }
    }
    // O^T += V^T P^T (LDS accesses of one wave complete in order)
#pragma unroll
    for (int kb_ = 0; kb_ < 2; ++kb_) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int i0 = kb_ * 8 + 4 * c2;
        const u32x4 pb = {pk[i0], pk[i0 + 1], pk[i0 + 2], pk[i0 + 3]};
        const char* vrow = sv + (32 * kb_ + 16 * c2) * SH::RB16;
#pragma unroll
        for (int db = 0; db < SH::ND; ++db) {
          const u32x2 lo = ld_lds_tr16(vrow + av[db]);
          const u32x2 hi = ld_lds_tr16(vrow + 8 * SH::RB16 + av[db]);
          O[db] = mfma16<BF16>(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, O[db]);
        }
      }
    }
  };
  // two register sets (unrolled by two so that each names its set
  // statically): one tile in flight while the other is computed.  A deeper
  // ring holds more codes in flight but pushes them through AGPRs (copies
  // on every tile), which costs more than it hides.  The prefetches are
  // unconditional (past the split's last tile they reload
  // that tile, an L2 hit): conditional loads would make the wait for the
  // current set count every load in flight.
  TileCodes t0, t1;
  if (kt0 < kt1) load_tile(kt0, t0);
  for (int kt = kt0; kt < kt1; kt += 2) {
    load_tile(min(kt + 1, kt1 - 1), t1);
    compute_tile(kt, t0);
    load_tile(min(kt + 2, kt1 - 1), t0);
    if (kt + 1 < kt1) compute_tile(kt + 1, t1);
  }

  // partial of this split: O^T block db holds rows d = 32 db + 8 (r / 4) +
  // 4 hf + r % 4 of column lr.  Only live columns are written (the merge
  // reads no others).
  const float l_tot = halves_sum(l_run);
  if (!col_live) return;
  const int64_t slot = ((int64_t)grp * a.n_split + split) * 32 + lr;
  float* wo = a.ws_o + slot * D;
#pragma unroll
  for (int db = 0; db < SH::ND; ++db) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d0 = db * 32 + ii * 8 + hf * 4;
      *reinterpret_cast<f32x4*>(wo + d0) =
          f32x4{O[db][4 * ii], O[db][4 * ii + 1], O[db][4 * ii + 2], O[db][4 * ii + 3]};
    }
  }
  if (hf == 0) *reinterpret_cast<f32x2*>(a.ws_ml + 2 * slot) = f32x2{m_run, l_tot};
}

// One workgroup per (b, KV head, column): the splits' (m, l) go through LDS
// once, every thread then owns one head-dim element and sums the splits'
// partial O with independent loads.
template <bool BF16>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wgt[kMergeMaxSplit];
  __shared__ float red[kMergeThreads / 64];
  const int col = (int)(blockIdx.x % (unsigned)a.cols);
  const int grp = (int)(blockIdx.x / (unsigned)a.cols);
  const int b = grp / a.Hkv, kvh = grp % a.Hkv;
  const int hh = col / a.S_q, i = col % a.S_q;
  const int h = kvh * a.hpg + hh;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)grp * a.n_split * 32 + col;     // slot of split 0
  // maximum of the splits' m over splits that saw a key (l > 0)
  float M = kNegInf;
  for (int s = tid; s < a.n_split; s += kMergeThreads) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ws_ml + 2 * (base + (int64_t)s * 32));
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  // split weights 2^(m - M) (0 for splits without keys) and L
  float Lp = 0.f;
  for (int s = tid; s < a.n_split; s += kMergeThreads) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ws_ml + 2 * (base + (int64_t)s * 32));
    const float w = ml.y > 0.f ? exp2_fast(ml.x - M) : 0.f;
    wgt[s] = w;
    Lp += ml.y * w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Lp += __shfl_xor(Lp, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = Lp;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) L += red[w];
  // O = sum_s w_s O_s / L, one head-dim element per thread
  for (int d = tid; d < a.D; d += kMergeThreads) {
    float acc = 0.f;
    const float* po = a.ws_o + base * a.D + d;
#pragma unroll 8
    for (int s = 0; s < a.n_split; ++s) acc += po[(int64_t)s * 32 * a.D] * wgt[s];
    const float o = L > 0.f ? acc / L : 0.f;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                   (b * a.o_sb + h * a.o_sh + (int64_t)i * a.o_ss + d);
    *op = (uint16_t)(pack16x2<BF16>(o, 0.f) & 0xFFFFu);
  }
  if (tid == 0 && a.lse != nullptr)
    a.lse[((int64_t)b * a.Hq + h) * a.S_q + i] =
        L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : kNegInf;
}

template <int D, bool BF16>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<D, BF16>),
                     dim3((unsigned)((int64_t)a.B * a.Hkv * a.n_split)), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<BF16>), dim3((unsigned)((int64_t)a.B * a.Hkv * a.cols)),
                     dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.D == 64) return a.bf16 ? launch_decode_t<64, true>(a, s) : launch_decode_t<64, false>(a, s);
  return a.bf16 ? launch_decode_t<128, true>(a, s) : launch_decode_t<128, false>(a, s);
}

}  // namespace lamp
