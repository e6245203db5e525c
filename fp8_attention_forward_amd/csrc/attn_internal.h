// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfp8 {

struct QuantParams {
  const float* q;
  const float* k;
  const float* v;
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8;
  float* qd;
  float* kd;
  float* vd;
  int N;
  int nblk;        // scale blocks per (batch, head) = ceil(N / scale_block)
  int hadamard;
  uint32_t key0;   // seed, low word
  uint32_t key1;   // seed, high word
};

// Packed documents: Q, K, V, codes and O are [H][T][D]; document d holds
// tokens cu[d] .. cu[d+1]-1 of every head; the descales of its blocks sit at
// slots cu[d] / SB + d + b of a head's row of nslot = T / SB + ndoc entries.
struct QuantVarlenParams {
  const float* q;
  const float* k;
  const float* v;
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8;
  float* qd;
  float* kd;
  float* vd;
  const int* cu;   // [ndoc + 1]
  int ndoc;
  int T;
  int nslot;
  int hadamard;
  uint32_t key0;
  uint32_t key1;
};

// Work list of the packed attention (in the caller's workspace): int32
// count and status words, two unused words, then int2 items (document, query
// tile) from byte 16, in the order the workgroups take them.
constexpr int kWsHeaderInts = 4;
constexpr int kVarlenMaxKeys = 8192;   // cost keys: ceil(T / 128) <= this, so T <= 2^20

struct VarlenSchedParams {
  const int* cu;
  int ndoc;
  int T;
  int natural;     // document-major order instead of longest-first
  int kmax;        // ceil(T / 128)
  int* ws;
};

struct AttnFp8VarlenParams {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qd;
  const float* kd;
  const float* vd;
  uint16_t* o;
  float* lse;
  const int* cu;
  const int* ws;     // work list written by the schedule kernel
  int T;
  int nslot;
  int H;
  float score_scale;
};

// Decode over an FP8 K/V cache: queries [B][Hq][Sq][D] (descales [B][Hq]),
// cache codes [B][Hkv][Ncap][D] (descales [B][Hkv][nblk]), lengths [B].
// Partials per (batch * Hkv, split): O [MQ][D], m [MQ], l [MQ].
struct DecodeParams {
  const uint8_t* q8;
  const float* qd;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* kd;
  const float* vd;
  const int* seqlens;
  float* part_o;
  float* part_m;
  float* part_l;
  uint16_t* o;
  float* lse;
  int B;
  int Hq;
  int Hkv;
  int G;           // query heads per K/V head
  int Sq;          // new tokens per sequence
  int MQ;          // G * Sq <= 32 query rows per K/V head
  int Ncap;
  int nblk;        // ceil(Ncap / scale_block)
  int split;       // fixed ranges: keys per wave range (multiple of 64)
  int nsplit;      // fixed ranges: ceil(Ncap / (4 * split)) partials per (batch, K/V head)
  int nwave;       // balanced schedule: waves sharing the tiles (0: fixed ranges)
  float score_scale;
};

struct AttnFp8Params {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qd;
  const float* kd;
  const float* vd;
  uint16_t* o;
  float* lse;
  int N;
  int nblk;          // scale blocks per head (key tile == scale block)
  int n_qtiles;      // query tiles per head
  float score_scale; // log2(e) / sqrt(D), divided by D when Q and K were rotated
};

struct AttnBf16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N;
  int n_qtiles;
  float score_scale; // log2(e) / sqrt(D)
};

constexpr int kWaves = 4;              // waves per workgroup in the attention kernels
constexpr int kQueriesPerWave = 32;
constexpr int kQueryTile = kWaves * kQueriesPerWave;
constexpr int kFp8KeyTile = 64;      // keys per tile in the FP8 kernel

// pow2: power-of-two (E8M0) block scales instead of amax / 448
hipError_t launch_quantize(const QuantParams& p, int D, int SB, int pow2, int BH, hipStream_t stream);
// exp_mode: 0 exact exponentials, 1 Schraudolph's bit-level approximation
// mx: the block descales are powers of two and the matrix cores apply them
hipError_t launch_attn_fp8(const AttnFp8Params& p, int D, int SB, int causal, int exp_mode, int mx, int BH,
                           hipStream_t stream);
hipError_t launch_quantize_varlen(const QuantVarlenParams& p, int D, int SB, int pow2, int H, hipStream_t stream);
// one workgroup writes the work list (count, status, items) into sp.ws
hipError_t launch_varlen_schedule(const VarlenSchedParams& sp, hipStream_t stream);
// the schedule kernel, then the attention over H * m_cap workgroups (m_cap >= the item count)
hipError_t launch_attn_fp8_varlen(const VarlenSchedParams& sp, const AttnFp8VarlenParams& p, int D, int SB, int causal,
                                  int exp_mode, int mx, int m_cap, hipStream_t stream);
hipError_t launch_attn_fp8_decode(const DecodeParams& p, int D, int SB, int causal, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnBf16Params& p, int D, int causal, int BH, hipStream_t stream);

}  // namespace attnfp8
