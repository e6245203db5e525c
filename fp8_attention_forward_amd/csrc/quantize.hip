// Fused rotate + per-block scale + e4m3 encode of Q, K and V (gfx950).
//
// Method ("Fused attention kernel", Variants / 8-bit forward pass (FP8)):
// scales are per block, separately for Q, K and V, and Q and K are first
// rotated by a random +-1 diagonal times a Hadamard matrix (incoherent
// processing); the rotation is orthogonal, so Q K^T is unchanged.  FLAMIA (4.3 Ablation Study) fuses the
// quantisation pre-processing into a single launch; here one launch covers
// all three tensors.
//
// Per workgroup: one (tensor, batch*head, block of SB tokens).  The block
// (SB x D float32) is read once with coalesced 16-byte loads and kept in
// registers; each lane holds 4 consecutive channels of a row, D/4 lanes per
// row.  The unnormalised Sylvester Hadamard transform runs as butterfly
// stages h = 1, 2 inside the lane and h = 4 .. D/2 across lanes (ds_swizzle
// xor), always in ascending h so the float32 result is reproducible.  Then
// amax over the block (wave + LDS reduction), inv = 448/a and descale = a/448
// (correctly rounded), and code = e4m3(clamp(y * inv, +-448)) with the
// hardware round-to-nearest-even convert; one 4-byte store per lane per row.
// V's blocks, and with the power-of-two option (the microscaling form, FLAMIA
// 2 Background) every block, take the smallest 2^e that keeps the block's
// amax inside +-448: the attention applies such a scale exactly inside the
// matrix core.
//
// Memory: reads 4 B and writes 1 B per element (HBM bound), both with
// non-temporal accesses (each byte is touched once).
#include "common.h"
#include "attn_internal.h"

namespace attnfp8 {

// Philox4x32-10 (Salmon et al., SC 2011): one block, counter (0,0,0,0), key = seed.
__device__ __forceinline__ void philox_block(uint32_t k0, uint32_t k1, uint32_t out[4]) {
  uint32_t x0 = 0, x1 = 0, x2 = 0, x3 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint32_t lo0 = 0xD2511F53u * x0, hi0 = __umulhi(0xD2511F53u, x0);
    uint32_t lo1 = 0xCD9E8D57u * x2, hi1 = __umulhi(0xCD9E8D57u, x2);
    uint32_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

template <int M>
__device__ __forceinline__ void butterfly_xlane(float (&x)[4], int lane) {
  // stage pairing lanes (lane, lane ^ M): lower lane keeps a + b, upper keeps a - b
  const bool upper = (lane & M) != 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float p = xor_lanes<M>(x[e]);
    x[e] = upper ? (p - x[e]) : (x[e] + p);
  }
}

// Power-of-two block scale (the MX form, E8M0): the smallest 2^e with
// a <= 448 * 2^e, e clamped to [-127, 127], so no code of the block saturates;
// a = 0 -> 2^0.  From the bits of a: a in [2^x, 2^(x+1)) with significand m;
// 448 * 2^(x-8) = 1.75 * 2^x, so e = x - 8, plus one when m > 1.75.
__device__ __forceinline__ int pow2_scale_exponent(float a) {
  if (a == 0.0f) return 0;
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  const int x = (int)(b >> 23) - 127;
  if (x == -127) return -127;                      // subnormal a: below 448 * 2^-127
  int e = x - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as a float32 (e in [-127, 127]; 2^-127 is subnormal)
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __builtin_bit_cast(float, (uint32_t)(e + 127) << 23) : __builtin_bit_cast(float, 0x00400000u);
}

// One scale block: rows [0, nrows) (nrows <= SB) of src, D floats each ->
// e4m3 codes at dst (same row layout) and the block's descale at *dsc, or,
// with GRP = 32, one power-of-two descale per 32 channels at dsc[0 .. D/32)
// (the MX block of 32 elements; pow2 must then be set).
// Called by every thread of the workgroup (it holds a workgroup barrier).
template <int D, int SB, int GRP = 0>
__device__ __forceinline__ void quantize_block(const float* src, uint8_t* dst, int nrows, float* dsc, bool rotate,
                                               bool pow2, uint32_t key0, uint32_t key1) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 4;              // lanes per row
  constexpr int RPI = 256 / LPR;          // rows per iteration (whole workgroup)
  constexpr int ITERS = SB / RPI;
  static_assert(SB % RPI == 0, "block must be a whole number of iterations");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rlane = tid % LPR;            // lane within its row group
  const int c0 = 4 * rlane;               // first channel held by this lane

  float x[ITERS][4];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = it * RPI + tid / LPR;
    if (row < nrows) {
      // (read once and never again: non-temporal, so the stream does not
      // displace reusable lines from the caches)
      v4f t = __builtin_nontemporal_load((const v4f*)(src + (size_t)row * D + c0));
      x[it][0] = t[0]; x[it][1] = t[1]; x[it][2] = t[2]; x[it][3] = t[3];
    } else {
      x[it][0] = x[it][1] = x[it][2] = x[it][3] = 0.0f;
    }
  }

  if (rotate) {
    uint32_t w[4];
    philox_block(key0, key1, w);
    float sg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + e;
      sg[e] = ((w[c >> 5] >> (c & 31)) & 1u) ? -1.0f : 1.0f;
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      float (&y)[4] = x[it];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = y[e] * sg[e];
      // h = 1
      float a0 = y[0] + y[1], a1 = y[0] - y[1], a2 = y[2] + y[3], a3 = y[2] - y[3];
      // h = 2
      y[0] = a0 + a2; y[1] = a1 + a3; y[2] = a0 - a2; y[3] = a1 - a3;
      // h = 4 .. D/2 across lanes
      butterfly_xlane<1>(y, rlane);
      butterfly_xlane<2>(y, rlane);
      butterfly_xlane<4>(y, rlane);
      butterfly_xlane<8>(y, rlane);
      if constexpr (LPR == 32) butterfly_xlane<16>(y, rlane);
    }
  }

  // block amax (rows beyond the block hold zeros and do not raise it)
  float m = 0.0f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(x[it][e]));
  float a;
  if constexpr (GRP == 0) {
    m = wave_max(m);
    __shared__ float red[4];
    if (lane == 0) red[wave] = m;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  } else {
    // the GRP / 4 lanes of a channel group in a row, then the rows of the
    // wave (lanes LPR apart), then the four waves
    static_assert(GRP == 32, "32-channel groups");
    m = fmaxf(m, xor_lanes<1>(m));
    m = fmaxf(m, xor_lanes<2>(m));
    m = fmaxf(m, xor_lanes<4>(m));
    if constexpr (LPR == 16) m = fmaxf(m, xor_lanes<16>(m));
    m = fmaxf(m, swap_halves(m));
    constexpr int NG = D / GRP;
    __shared__ float redg[4][NG];
    if (lane < LPR && (rlane & 7) == 0) redg[wave][rlane >> 3] = m;
    __syncthreads();
    const int g = rlane >> 3;
    a = fmaxf(fmaxf(redg[0][g], redg[1][g]), fmaxf(redg[2][g], redg[3][g]));
  }
  float inv, descale;
  if (pow2) {
    const int e = pow2_scale_exponent(a);
    inv = exp2i(-e);
    descale = exp2i(e);
  } else {
    inv = a == 0.0f ? 1.0f : 448.0f / a;
    descale = a == 0.0f ? 1.0f : a / 448.0f;
  }
  if constexpr (GRP == 0) {
    if (tid == 0) *dsc = descale;
  } else {
    if (tid < LPR && (rlane & 7) == 0) dsc[rlane >> 3] = descale;
  }

#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = it * RPI + tid / LPR;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(x[it][e] * inv, -448.0f), 448.0f);
    int packed = cvt_pk_fp8<false>(v[0], v[1], 0);
    packed = cvt_pk_fp8<true>(v[2], v[3], packed);
    if (row < nrows) __builtin_nontemporal_store(packed, (int*)(dst + (size_t)row * D + c0));
  }
}

// Dense layout: one workgroup per (block, batch*head) and tensor (blockIdx.y).
// GRP = 32: power-of-two descales per 32 channels, [..][nblk][D / 32].
template <int D, int SB, bool POW2, int GRP = 0>
__global__ __launch_bounds__(256) void quantize_qkv_kernel(QuantParams p) {
  const int blk = blockIdx.x % p.nblk;
  const int bh = blockIdx.x / p.nblk;
  const int tensor = blockIdx.y;          // 0 = Q, 1 = K, 2 = V
  const float* src = tensor == 0 ? p.q : (tensor == 1 ? p.k : p.v);
  uint8_t* dst = tensor == 0 ? p.q8 : (tensor == 1 ? p.k8 : p.v8);
  float* dsc = tensor == 0 ? p.qd : (tensor == 1 ? p.kd : p.vd);
  const int row0 = blk * SB;
  const size_t off = ((size_t)bh * p.N + row0) * D;
  const int nrows = p.N - row0 < SB ? p.N - row0 : SB;
  constexpr int NG = GRP == 0 ? 1 : D / GRP;
  quantize_block<D, SB, GRP>(src + off, dst + off, nrows, dsc + ((size_t)bh * p.nblk + blk) * NG,
                             p.hadamard && tensor < 2, POW2 || tensor == 2 || GRP != 0, p.key0, p.key1);
}

// Packed documents ("FLAMIA", Abstract and 4.1 Performance on Packed
// Documents: document-local scaling, no repacking).  Block b of document d
// has descale slot first_slot(d) + b with first_slot(d) = cu[d] / SB + d,
// strictly increasing in d, so a slot g belongs to the last document whose
// first slot is <= g, or to none (the document has fewer blocks).  Entries of
// cu are clamped to [0, T] so that any contents keep every access in bounds.
template <int SB>
__device__ __forceinline__ int doc_first_slot(const int* cu, int d, int T) {
  int c = cu[d];
  c = c < 0 ? 0 : (c > T ? T : c);
  return c / SB + d;
}

// Largest d in [0, ndoc) with doc_first_slot(d) <= g (0 if none): a 64-way
// search, one pivot per lane, the pivots that hold counted by a ballot.  Every
// wave runs it on its own and gets the same answer.
template <int SB>
__device__ __forceinline__ int find_doc(const int* cu, int ndoc, int T, int g) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = ndoc;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool pred = idx < hi && doc_first_slot<SB>(cu, idx, T) <= g;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(pred));
    lo += (cnt > 0 ? cnt - 1 : 0) * step;
    hi = hi < lo + step ? hi : lo + step;
  }
  return lo;
}

template <int D, int SB, bool POW2>
__global__ __launch_bounds__(256) void quantize_qkv_varlen_kernel(QuantVarlenParams p) {
  const int g = blockIdx.x % p.nslot;
  const int h = blockIdx.x / p.nslot;
  const int tensor = blockIdx.y;
  const int d = find_doc<SB>(p.cu, p.ndoc, p.T, g);
  int a = p.cu[d], b = p.cu[d + 1];
  a = a < 0 ? 0 : (a > p.T ? p.T : a);
  b = b < a ? a : (b > p.T ? p.T : b);
  const int r0 = a + (g - (a / SB + d)) * SB;
  if (r0 < a || r0 >= b) return;          // a slot of no block (the same for the whole workgroup)
  const float* src = tensor == 0 ? p.q : (tensor == 1 ? p.k : p.v);
  uint8_t* dst = tensor == 0 ? p.q8 : (tensor == 1 ? p.k8 : p.v8);
  float* dsc = tensor == 0 ? p.qd : (tensor == 1 ? p.kd : p.vd);
  const size_t off = ((size_t)h * p.T + r0) * D;
  const int nrows = b - r0 < SB ? b - r0 : SB;
  quantize_block<D, SB>(src + off, dst + off, nrows, dsc + (size_t)h * p.nslot + g, p.hadamard && tensor < 2,
                        POW2 || tensor == 2, p.key0, p.key1);
}

#define QUANT_INST(D, SB) \
  template __global__ void quantize_qkv_kernel<D, SB, false>(QuantParams); \
  template __global__ void quantize_qkv_kernel<D, SB, true>(QuantParams); \
  template __global__ void quantize_qkv_kernel<D, SB, true, 32>(QuantParams); \
  template __global__ void quantize_qkv_varlen_kernel<D, SB, false>(QuantVarlenParams); \
  template __global__ void quantize_qkv_varlen_kernel<D, SB, true>(QuantVarlenParams);
QUANT_INST(64, 64)
QUANT_INST(64, 128)
QUANT_INST(128, 64)
QUANT_INST(128, 128)

// pow2: 0 amax / 448 for Q and K, 1 power-of-two block scales, 2 power-of-two
// scales per 32 channels
template <int D, int SB>
static void launch_q(const QuantParams& p, int pow2, dim3 grid, hipStream_t stream) {
  if (pow2 == 2) quantize_qkv_kernel<D, SB, true, 32><<<grid, 256, 0, stream>>>(p);
  else if (pow2) quantize_qkv_kernel<D, SB, true><<<grid, 256, 0, stream>>>(p);
  else quantize_qkv_kernel<D, SB, false><<<grid, 256, 0, stream>>>(p);
}

template <int D, int SB>
static void launch_qv(const QuantVarlenParams& p, bool pow2, dim3 grid, hipStream_t stream) {
  if (pow2) quantize_qkv_varlen_kernel<D, SB, true><<<grid, 256, 0, stream>>>(p);
  else quantize_qkv_varlen_kernel<D, SB, false><<<grid, 256, 0, stream>>>(p);
}

hipError_t launch_quantize_varlen(const QuantVarlenParams& p, int D, int SB, int pow2, int H, hipStream_t stream) {
  dim3 grid(p.nslot * H, 3);
  if (D == 64 && SB == 64) launch_qv<64, 64>(p, pow2, grid, stream);
  else if (D == 64 && SB == 128) launch_qv<64, 128>(p, pow2, grid, stream);
  else if (D == 128 && SB == 64) launch_qv<128, 64>(p, pow2, grid, stream);
  else launch_qv<128, 128>(p, pow2, grid, stream);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, int D, int SB, int pow2, int BH, hipStream_t stream) {
  dim3 grid(p.nblk * BH, 3);
  if (D == 64 && SB == 64) launch_q<64, 64>(p, pow2, grid, stream);
  else if (D == 64 && SB == 128) launch_q<64, 128>(p, pow2, grid, stream);
  else if (D == 128 && SB == 64) launch_q<128, 64>(p, pow2, grid, stream);
  else launch_q<128, 128>(p, pow2, grid, stream);
  return hipGetLastError();
}

}  // namespace attnfp8
