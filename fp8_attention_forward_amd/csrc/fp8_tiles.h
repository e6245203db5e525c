// FP8 tile machinery shared by the attention kernels (gfx950): exponential
// forms of the probabilities, the tile configuration, the LDS swizzles, the
// per-lane MFMA operand offsets and the FP8 MFMA wrappers.
#pragma once

#include "common.h"
#include "attn_internal.h"

namespace attnfp8 {

// Lazy-rescale threshold (log2 units): P <= 2^kTau ~ 445.7, just inside
// e4m3's largest value 448 (and below 464, from where the convert would
// overflow, even with Schraudolph's +2% error).
constexpr float kTau = 8.8f;
// When the reference moves it is set kLift below the tile maximum (log2
// units, a whole number): the key that moved it gets P = 2^kLift, which e4m3
// holds exactly (a fractional lift would round the largest P of the row),
// and the small probabilities sit 2^kLift higher, away from e4m3's subnormal
// range.  The headroom kTau - kLift decides how closely the reference follows
// the running maximum: a larger lift moves it more often (each move costs the
// tile maximum, an O rescale and P formed again) and rounds small P less
// coarsely.  2 moves it on 4% of the steps of outlier inputs against 10% for
// a lift of 4, for a P-rounding error 13% larger.
constexpr float kLift = 2.0f;

// Exponentials of the probabilities P.
//   kExpExact: v_exp_f32 of the scaled score (one FMA + one transcendental).
//   kExpSchraudolph: Schraudolph's approximation (N. N. Schraudolph, "A fast,
//     compact approximation of the exponential function", Neural Computation
//     11(4), 1999), in base 2 for float32: the bit pattern of 2^x is taken to
//     be floor(2^23 (x + 127 - sigma)), i.e. floor(x) lands in the exponent
//     field and the fractional part, linearly, in the mantissa; sigma =
//     60801 / 2^20 is the paper's error-centring constant (relative error
//     within -3.9% .. +2.0%).  One FMA builds 2^23 (x + 127 - sigma) straight
//     from the raw score, one conversion (round toward zero, saturating:
//     negative -> 0) makes the bits.  FLAMIA uses this approximation for
//     inference (4.4 Bit-Level Exponentials at Inference).
enum { kExpExact = 0, kExpSchraudolph = 1 };
constexpr float kSchraudolphSigma = 60801.0f / 1048576.0f;

template <int EXPM>
struct ExpArgs {
  float c, b;   // p = exp(s * c + b)
  __device__ __forceinline__ ExpArgs(float c_log2, float bias_log2) {
    if constexpr (EXPM == kExpExact) {
      c = c_log2;
      b = bias_log2;
    } else {
      c = c_log2 * 8388608.0f;
      b = (bias_log2 + (127.0f - kSchraudolphSigma)) * 8388608.0f;
    }
  }
  __device__ __forceinline__ float operator()(float s) const {
    if constexpr (EXPM == kExpExact) {
      return __builtin_amdgcn_exp2f(__builtin_fmaf(s, c, b));
    } else {
      unsigned bits;
      asm("v_cvt_u32_f32 %0, %1" : "=v"(bits) : "v"(__builtin_fmaf(s, c, b)));
      return __builtin_bit_cast(float, bits);
    }
  }
};
constexpr int kBC = kFp8KeyTile; // keys per tile

// First channel of the 16-byte operand piece `half` that lane half h feeds to
// K-step ks of the score product: channel = the matrix core's k index (plus
// 64 ks), so each 32-channel group is one 32-element scale block of the
// scaled MFMA (lane half h = l / 32).
__device__ __forceinline__ constexpr int op_channel(int ks, int h, int half) { return 64 * ks + 32 * half + 16 * h; }

template <int D>
struct Fp8Cfg {
  static constexpr int KSTEPS = D / 64;      // K-steps of the QK^T contraction
  static constexpr int NSUB = kBC / 32;      // 32-key subtiles of S^T
  static constexpr int NDT = D / 32;         // 32-row (d) tiles of O^T
  static constexpr int TILE = kBC * D;       // bytes per K or V tile
  static constexpr int CHUNKS = TILE / 1024; // 1 KiB direct-load chunks per tile
  static constexpr int CHUNKS_PER_WAVE = CHUNKS / kWaves;
  static_assert(CHUNKS % kWaves == 0, "tile must split evenly over the waves");
  static_assert(kBC == 64, "one PV K-step per tile");
};

// XOR swizzles of the 16-byte column index, per LDS row.  They depend on row
// bits 0..3 only, so moving 16 rows (or more) is a constant address offset.
//   K (ds_read_b128, one row per lane): any 16 consecutive rows at one logical
//     column fall into distinct 16-byte bank groups.
//   V (ds_read_b64_tr_b8): the 8 rows x 2 columns a 32-lane half reads fall
//     into distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return (row & 7) ^ ((row >> 3) & 1);
  else return ((row >> 1) ^ (row >> 2)) & 3;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return (row & 3) | ((row >> 1) & 4);
  else return ((row >> 1) ^ (row >> 2)) & 3;
}

// Per-lane LDS byte offsets of the MFMA operands inside one K / V tile; every
// other operand of the tile is one of these plus a compile-time constant.
template <int D>
struct Fp8LaneOffsets {
  using C = Fp8Cfg<D>;
  int k[C::KSTEPS][2];   // K row (lane % 32), its two 16-byte pieces of k-step ks; + sub * 32 * D
  int v[C::NDT];         // V^T source row for d-tile dt; + 16 rr * D

  __device__ __forceinline__ explicit Fp8LaneOffsets(int lane) {
    const int ql = lane & 31;
    const int h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half) k[ks][half] = ql * D + 16 * ((op_channel(ks, h, half) / 16) ^ swz_k<D>(ql));
    // ds_read_b64_tr_b8 source lane i of 16-lane group g supplies key byte t = i / 2 of
    // the (8 rr + t)-th operand byte; that key is row 8 (j / 4) + 4 h + j % 4, j = 8 rr + t
    const int g = lane >> 4;
    const int i = lane & 15;
    const int gh = g >> 1;
    const int gd = g & 1;
    const int row0 = 8 * (i >> 3) + 4 * gh + ((i >> 1) & 3);   // row for rr = 0
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) v[dt] = row0 * D + 16 * ((2 * dt + gd) ^ swz_v<D>(row0)) + 8 * (i & 1);
  }
};

template <int D>
using STile = v16f[Fp8Cfg<D>::NSUB];

// K operands of one tile (A of S^T = K Q^T): 2 x 16 bytes per lane per MFMA
template <int D>
struct KOps {
  v4i r[Fp8Cfg<D>::NSUB][Fp8Cfg<D>::KSTEPS][2];
};

template <int D>
__device__ __forceinline__ void read_k(const uint8_t* kbuf, const Fp8LaneOffsets<D>& lo, KOps<D>& k) {
  using C = Fp8Cfg<D>;
#pragma unroll
  for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half) k.r[sub][ks][half] = lds_read_b128(kbuf + sub * 32 * D + lo.k[ks][half]);
}

// FP8 MFMA; with MX the E8M0 exponents sa (per row of A) and sb (per column of
// B) scale the products inside the matrix core (127 = 2^0).  Without MX the
// unscaled instruction is used.
template <bool MX>
__device__ __forceinline__ v16f mfma_f8x(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  if constexpr (MX) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  else return mfma_f8(a, b, c);
}

// E8M0 exponent of a power-of-two float (2^-127 is the subnormal 0x00400000)
__device__ __forceinline__ int e8m0_of(float pow2) { return (int)(__builtin_bit_cast(uint32_t, pow2) >> 23) & 0xFF; }

// E8M0 scale operands of the score product, one per K-step of the
// contraction (lane half h of K-step ks covers channels 64 ks + 32 h ..
// + 31: with 32-channel scales they differ per lane half and per K-step)
template <int D>
struct KsScales {
  int v[Fp8Cfg<D>::KSTEPS];
};

template <int D, bool MX>
__device__ __forceinline__ v16f qk_mfma(const KOps<D>& k, const v8i (&qop)[Fp8Cfg<D>::KSTEPS], int sub,
                                        const KsScales<D>& sk, const KsScales<D>& sq) {
  v16f acc = {};
#pragma unroll
  for (int ks = 0; ks < Fp8Cfg<D>::KSTEPS; ++ks) {
    const v4i& a0 = k.r[sub][ks][0];
    const v4i& a1 = k.r[sub][ks][1];
    v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    acc = mfma_f8x<MX>(a, qop[ks], acc, sk.v[ks], sq.v[ks]);
  }
  return acc;
}

}  // namespace attnfp8
