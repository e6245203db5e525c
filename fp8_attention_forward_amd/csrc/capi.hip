// C ABI entry points: argument validation, device check, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/attn_fp8.h"
#include "attn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

// Returns ATTN_OK when the current device is a gfx950.
int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_EUNSUPPORTED, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EUNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(ATTN_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (g_dev_state[dev] == 2) return fail(ATTN_EUNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (g_dev_state[dev] != 1) return fail(ATTN_EUNSUPPORTED, "device %d is not gfx950", dev);
  return ATTN_OK;
}

// Scratch memory of attn_fp8_decode_noalloc: the per-range partials that
// attn_fp8_decode keeps in the caller's workspace.  One copy per GPU the
// library runs on, held until the process ends; every call on a GPU shares
// it (calls that overlap on one GPU race).  The host-side name `scratch` is
// only a stand-in: kernels get the device address that hipGetSymbolAddress
// returns for the current device.
constexpr size_t kDecodeScratchBytes = ATTN_FP8_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // device address of `scratch` per device, looked up once

// Device address of this device's `scratch` (the current device must be a
// checked gfx950).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(ATTN_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(ATTN_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return ATTN_OK;
}

int check_sizes(int B, int H, int N, int D) {
  if (B < 1 || H < 1 || N < 1) return fail(ATTN_EINVAL, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (D != 64 && D != 128) return fail(ATTN_EINVAL, "D must be 64 or 128 (got %d)", D);
  const long long tiles = (long long)B * H * ((N + attnfp8::kQueryTile - 1) / attnfp8::kQueryTile);
  if (tiles >= (1LL << 31) || (long long)B * H >= (1LL << 31))
    return fail(ATTN_EINVAL, "B * H * ceil(N / %d) must be < 2^31", attnfp8::kQueryTile);
  // per-head byte offsets (16-bit elements, plus the tiles loaded past the end) stay below 2^31
  if ((long long)N * D * 2 >= (1LL << 31) - (1LL << 20))
    return fail(ATTN_EINVAL, "N * D must be < 2^30 (got N = %d, D = %d)", N, D);
  return ATTN_OK;
}

int check_varlen_sizes(int H, int T, int ndoc, int D) {
  if (H < 1 || T < 1 || ndoc < 1) return fail(ATTN_EINVAL, "H, T, ndoc must be >= 1 (got %d, %d, %d)", H, T, ndoc);
  if (D != 64 && D != 128) return fail(ATTN_EINVAL, "D must be 64 or 128 (got %d)", D);
  if (T > attnfp8::kVarlenMaxKeys * attnfp8::kQueryTile)
    return fail(ATTN_EINVAL, "T must be <= %d (got %d)", attnfp8::kVarlenMaxKeys * attnfp8::kQueryTile, T);
  if (ndoc > (1 << 24)) return fail(ATTN_EINVAL, "ndoc must be <= 2^24 (got %d)", ndoc);
  return ATTN_OK;
}

int check_sb(int sb) {
  if (sb != 64 && sb != 128) return fail(ATTN_EINVAL, "scale_block must be 64 or 128 (got %d)", sb);
  return ATTN_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (p == nullptr) return fail(ATTN_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(ATTN_EINVAL, "%s is not %zu-byte aligned", name, align);
  return ATTN_OK;
}

#define CHECK(expr)              \
  do {                           \
    int _st = (expr);            \
    if (_st != ATTN_OK) return _st; \
  } while (0)

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return ATTN_OK;
}

}  // namespace

extern "C" {

int quantize_qkv_fp8_opts(const float* q, const float* k, const float* v, int B, int H, int N, int D,
                          int scale_block, int hadamard, uint64_t seed, unsigned flags, uint8_t* q8, uint8_t* k8,
                          uint8_t* v8, float* q_descale, float* k_descale, float* v_descale, void* stream) {
  if (flags & ~(unsigned)(ATTN_FP8_MX | ATTN_FP8_MX32)) return fail(ATTN_EINVAL, "unknown flags 0x%x", flags);
  CHECK(check_sizes(B, H, N, D));
  CHECK(check_sb(scale_block));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(q8, 16, "q8"));
  CHECK(check_ptr(k8, 16, "k8"));
  CHECK(check_ptr(v8, 16, "v8"));
  CHECK(check_ptr(q_descale, 4, "q_descale"));
  CHECK(check_ptr(k_descale, 4, "k_descale"));
  CHECK(check_ptr(v_descale, 4, "v_descale"));
  if ((long long)B * H * ((N + scale_block - 1) / scale_block) * ((flags & ATTN_FP8_MX32) ? D / 32 : 1) >= (1LL << 31))
    return fail(ATTN_EINVAL, "the descale count must be < 2^31");
  CHECK(check_device());
  attnfp8::QuantParams p;
  p.q = q; p.k = k; p.v = v;
  p.q8 = q8; p.k8 = k8; p.v8 = v8;
  p.qd = q_descale; p.kd = k_descale; p.vd = v_descale;
  p.N = N;
  p.nblk = (N + scale_block - 1) / scale_block;
  p.hadamard = hadamard ? 1 : 0;
  p.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  p.key1 = (uint32_t)(seed >> 32);
  const int pow2 = (flags & ATTN_FP8_MX32) ? 2 : ((flags & ATTN_FP8_MX) ? 1 : 0);
  return launched(attnfp8::launch_quantize(p, D, scale_block, pow2, B * H,
                                           (hipStream_t)stream),
                  "quantize_qkv_fp8");
}

int quantize_qkv_fp8(const float* q, const float* k, const float* v, int B, int H, int N, int D, int scale_block,
                     int hadamard, uint64_t seed, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_descale,
                     float* k_descale, float* v_descale, void* stream) {
  return quantize_qkv_fp8_opts(q, k, v, B, H, N, D, scale_block, hadamard, seed, 0u, q8, k8, v8, q_descale,
                               k_descale, v_descale, stream);
}

int attn_fp8_fwd_opts(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_descale,
                      const float* k_descale, const float* v_descale, int B, int H, int N, int D, int scale_block,
                      int hadamard, int causal, unsigned flags, uint16_t* o_bf16, float* lse, void* stream) {
  if (flags & ~(unsigned)(ATTN_FP8_EXP2_SCHRAUDOLPH | ATTN_FP8_MX | ATTN_FP8_MX32))
    return fail(ATTN_EINVAL, "unknown flags 0x%x", flags);
  CHECK(check_sizes(B, H, N, D));
  CHECK(check_sb(scale_block));
  CHECK(check_ptr(q8, 16, "q8"));
  CHECK(check_ptr(k8, 16, "k8"));
  CHECK(check_ptr(v8, 16, "v8"));
  CHECK(check_ptr(q_descale, 4, "q_descale"));
  CHECK(check_ptr(k_descale, 4, "k_descale"));
  CHECK(check_ptr(v_descale, 4, "v_descale"));
  CHECK(check_ptr(o_bf16, 16, "o_bf16"));
  CHECK(check_ptr(lse, 4, "lse"));
  CHECK(check_device());
  attnfp8::AttnFp8Params p;
  p.q8 = q8; p.k8 = k8; p.v8 = v8;
  p.qd = q_descale; p.kd = k_descale; p.vd = v_descale;
  p.o = o_bf16; p.lse = lse;
  p.N = N;
  p.nblk = (N + scale_block - 1) / scale_block;
  p.n_qtiles = (N + attnfp8::kQueryTile - 1) / attnfp8::kQueryTile;
  double sc = 1.4426950408889634 / std::sqrt((double)D);
  if (hadamard) sc /= D;
  p.score_scale = (float)sc;
  const int exp_mode = (flags & ATTN_FP8_EXP2_SCHRAUDOLPH) ? 1 : 0;
  const int mx = (flags & ATTN_FP8_MX32) ? 2 : ((flags & ATTN_FP8_MX) ? 1 : 0);
  return launched(attnfp8::launch_attn_fp8(p, D, scale_block, causal ? 1 : 0, exp_mode, mx, B * H,
                                           (hipStream_t)stream),
                  "attn_fp8_fwd");
}

int attn_fp8_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_descale,
                 const float* k_descale, const float* v_descale, int B, int H, int N, int D, int scale_block,
                 int hadamard, int causal, uint16_t* o_bf16, float* lse, void* stream) {
  return attn_fp8_fwd_opts(q8, k8, v8, q_descale, k_descale, v_descale, B, H, N, D, scale_block, hadamard, causal,
                           0u, o_bf16, lse, stream);
}

int attn_bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int H, int N, int D, int causal,
                  uint16_t* o_bf16, float* lse, void* stream) {
  CHECK(check_sizes(B, H, N, D));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(o_bf16, 16, "o_bf16"));
  CHECK(check_ptr(lse, 4, "lse"));
  CHECK(check_device());
  attnfp8::AttnBf16Params p;
  p.q = q; p.k = k; p.v = v;
  p.o = o_bf16; p.lse = lse;
  p.N = N;
  p.n_qtiles = (N + attnfp8::kQueryTile - 1) / attnfp8::kQueryTile;
  p.score_scale = (float)(1.4426950408889634 / std::sqrt((double)D));
  return launched(attnfp8::launch_attn_bf16(p, D, causal ? 1 : 0, B * H, (hipStream_t)stream), "attn_bf16_fwd");
}

size_t attn_fp8_varlen_workspace_bytes(int T, int ndoc) {
  if (T < 1 || ndoc < 1) return 0;
  const long long m_cap = ((long long)T + (long long)(attnfp8::kQueryTile - 1) * ndoc) / attnfp8::kQueryTile;
  return (size_t)(4 * attnfp8::kWsHeaderInts) + 8 * (size_t)m_cap;
}

int quantize_qkv_fp8_varlen(const float* q, const float* k, const float* v, const int32_t* cu_seqlens, int ndoc,
                            int H, int T, int D, int scale_block, int hadamard, uint64_t seed, unsigned flags,
                            uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_descale, float* k_descale,
                            float* v_descale, void* stream) {
  if (flags & ~(unsigned)ATTN_FP8_MX) return fail(ATTN_EINVAL, "unknown flags 0x%x", flags);
  CHECK(check_varlen_sizes(H, T, ndoc, D));
  CHECK(check_sb(scale_block));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(q8, 16, "q8"));
  CHECK(check_ptr(k8, 16, "k8"));
  CHECK(check_ptr(v8, 16, "v8"));
  CHECK(check_ptr(q_descale, 4, "q_descale"));
  CHECK(check_ptr(k_descale, 4, "k_descale"));
  CHECK(check_ptr(v_descale, 4, "v_descale"));
  const long long nslot = (long long)T / scale_block + ndoc;
  if ((long long)H * nslot >= (1LL << 31)) return fail(ATTN_EINVAL, "H * (T / scale_block + ndoc) must be < 2^31");
  CHECK(check_device());
  attnfp8::QuantVarlenParams p;
  p.q = q; p.k = k; p.v = v;
  p.q8 = q8; p.k8 = k8; p.v8 = v8;
  p.qd = q_descale; p.kd = k_descale; p.vd = v_descale;
  p.cu = cu_seqlens;
  p.ndoc = ndoc;
  p.T = T;
  p.nslot = (int)nslot;
  p.hadamard = hadamard ? 1 : 0;
  p.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  p.key1 = (uint32_t)(seed >> 32);
  return launched(attnfp8::launch_quantize_varlen(p, D, scale_block, (flags & ATTN_FP8_MX) ? 1 : 0, H,
                                                  (hipStream_t)stream),
                  "quantize_qkv_fp8_varlen");
}

int attn_fp8_fwd_varlen(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_descale,
                        const float* k_descale, const float* v_descale, const int32_t* cu_seqlens, int ndoc, int H,
                        int T, int D, int scale_block, int hadamard, int causal, unsigned flags, void* workspace,
                        size_t workspace_bytes, uint16_t* o_bf16, float* lse, void* stream) {
  if (flags & ~(unsigned)(ATTN_FP8_EXP2_SCHRAUDOLPH | ATTN_FP8_MX | ATTN_FP8_NATURAL_ORDER))
    return fail(ATTN_EINVAL, "unknown flags 0x%x", flags);
  CHECK(check_varlen_sizes(H, T, ndoc, D));
  CHECK(check_sb(scale_block));
  CHECK(check_ptr(q8, 16, "q8"));
  CHECK(check_ptr(k8, 16, "k8"));
  CHECK(check_ptr(v8, 16, "v8"));
  CHECK(check_ptr(q_descale, 4, "q_descale"));
  CHECK(check_ptr(k_descale, 4, "k_descale"));
  CHECK(check_ptr(v_descale, 4, "v_descale"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(workspace, 16, "workspace"));
  CHECK(check_ptr(o_bf16, 16, "o_bf16"));
  CHECK(check_ptr(lse, 4, "lse"));
  const size_t need = attn_fp8_varlen_workspace_bytes(T, ndoc);
  if (workspace_bytes < need)
    return fail(ATTN_EINVAL, "workspace_bytes %zu < %zu (attn_fp8_varlen_workspace_bytes)", workspace_bytes, need);
  const long long m_cap = ((long long)T + (long long)(attnfp8::kQueryTile - 1) * ndoc) / attnfp8::kQueryTile;
  if ((long long)H * m_cap >= (1LL << 31)) return fail(ATTN_EINVAL, "H * (T + 127 ndoc) / 128 must be < 2^31");
  CHECK(check_device());
  attnfp8::VarlenSchedParams sp;
  sp.cu = cu_seqlens;
  sp.ndoc = ndoc;
  sp.T = T;
  sp.natural = (flags & ATTN_FP8_NATURAL_ORDER) ? 1 : 0;
  sp.kmax = (T + attnfp8::kQueryTile - 1) / attnfp8::kQueryTile;
  sp.ws = (int*)workspace;
  attnfp8::AttnFp8VarlenParams p;
  p.q8 = q8; p.k8 = k8; p.v8 = v8;
  p.qd = q_descale; p.kd = k_descale; p.vd = v_descale;
  p.o = o_bf16; p.lse = lse;
  p.cu = cu_seqlens;
  p.ws = (const int*)workspace;
  p.T = T;
  p.nslot = T / scale_block + ndoc;
  p.H = H;
  double sc = 1.4426950408889634 / std::sqrt((double)D);
  if (hadamard) sc /= D;
  p.score_scale = (float)sc;
  const int exp_mode = (flags & ATTN_FP8_EXP2_SCHRAUDOLPH) ? 1 : 0;
  const int mx = (flags & ATTN_FP8_MX) ? 1 : 0;
  return launched(attnfp8::launch_attn_fp8_varlen(sp, p, D, scale_block, causal ? 1 : 0, exp_mode, mx, (int)m_cap,
                                                  (hipStream_t)stream),
                  "attn_fp8_fwd_varlen");
}

// Balanced schedule of the decode (split 0, B <= 512): the number of waves
// that share the batch's tiles: two workgroups of four waves on each of 256
// compute units, fewer when the cache holds fewer tiles; 0 = fixed ranges.
constexpr int kDecodeWaves = 2048;
constexpr int kDecodeBalancedMaxB = 512;

static int decode_waves(int B, int Hkv, int Ncap, int split) {
  if (split != 0 || B > kDecodeBalancedMaxB) return 0;
  const long long tmax = (long long)B * Hkv * ((Ncap + 63) / 64);
  const long long w = tmax < kDecodeWaves ? tmax : kDecodeWaves;
  return (int)((w + 3) / 4 * 4);
}

// Keys per range of the fixed-range schedule (split > 0, or B above the
// balanced schedule's limit).
static int decode_split(int B, int Hkv, int Ncap, int split) {
  if (split > 0) return split;
  // the largest power of two in [64, 1024] keys per wave that still gives
  // 1024 workgroups over the cache capacity (two rounds of the 512 the chip
  // holds at two per CU when every sequence is full; shorter sequences leave
  // their later splits empty).  Few long-lived workgroups stream best: each
  // wave keeps a tile's loads in flight for its whole range, while every
  // workgroup start and end costs dependent round trips (measured: 16 x 8
  // K/V heads of 32768, lengths 2274..28617: 1024 keys per wave 89 us,
  // 256 keys 97 us, 128 keys 101 us)
  int s = 1024;
  while (s > 64 && (long long)B * Hkv * ((Ncap + 4LL * s - 1) / (4LL * s)) < 1024) s /= 2;
  return s;
}

size_t attn_fp8_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Ncap, int D, int split) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Ncap < 1 || D < 1 || split < 0 || Hq % Hkv) return 0;
  const long long mq = (long long)(Hq / Hkv) * Sq;
  const int nw = decode_waves(B, Hkv, Ncap, split);
  if (nw > 0) return (size_t)(((long long)nw + (long long)B * Hkv) * mq * (D + 2) * 4);
  const int s = decode_split(B, Hkv, Ncap, split);
  const long long nsplit = (Ncap + 4LL * s - 1) / (4LL * s);
  return (size_t)((long long)B * Hkv * nsplit * mq * (D + 2) * 4);
}

}  // extern "C"

// The decode with its partials in `workspace`, or (use_scratch) in the
// library's own scratch array.
static int decode_impl(const uint8_t* q8, const float* q_descale, const uint8_t* k8, const uint8_t* v8,
                       const float* k_descale, const float* v_descale, const int32_t* seqlens, int B, int Hq, int Hkv,
                       int Sq, int Ncap, int D, int scale_block, int hadamard, int causal, int split, void* workspace,
                       size_t workspace_bytes, bool use_scratch, uint16_t* o_bf16, float* lse, void* stream) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Ncap < 1)
    return fail(ATTN_EINVAL, "B, Hq, Hkv, Sq, Ncap must be >= 1 (got %d, %d, %d, %d, %d)", B, Hq, Hkv, Sq, Ncap);
  if (D != 64 && D != 128) return fail(ATTN_EINVAL, "D must be 64 or 128 (got %d)", D);
  CHECK(check_sb(scale_block));
  if (Hq % Hkv) return fail(ATTN_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if ((Hq / Hkv) * Sq > 32) return fail(ATTN_EINVAL, "(Hq / Hkv) * Sq must be <= 32 (got %d)", (Hq / Hkv) * Sq);
  if ((long long)Ncap * D >= (1LL << 30)) return fail(ATTN_EINVAL, "Ncap * D must be < 2^30");
  if ((long long)B * Hkv > 65535) return fail(ATTN_EINVAL, "B * Hkv must be <= 65535");
  if (split < 0 || split % 64 || split > 8192) return fail(ATTN_EINVAL, "split must be 0 or a multiple of 64 up to 8192");
  if (decode_waves(B, Hkv, Ncap, split) == 0 &&
      (Ncap + 4LL * decode_split(B, Hkv, Ncap, split) - 1) / (4LL * decode_split(B, Hkv, Ncap, split)) > 65535)
    return fail(ATTN_EINVAL, "ceil(Ncap / (4 * split)) must be <= 65535");
  if ((long long)B * Hq * Sq >= (1LL << 31)) return fail(ATTN_EINVAL, "B * Hq * Sq must be < 2^31");
  CHECK(check_ptr(q8, 16, "q8"));
  CHECK(check_ptr(q_descale, 4, "q_descale"));
  CHECK(check_ptr(k8, 16, "k8"));
  CHECK(check_ptr(v8, 16, "v8"));
  CHECK(check_ptr(k_descale, 4, "k_descale"));
  CHECK(check_ptr(v_descale, 4, "v_descale"));
  CHECK(check_ptr(seqlens, 4, "seqlens"));
  if (!use_scratch) CHECK(check_ptr(workspace, 16, "workspace"));
  CHECK(check_ptr(o_bf16, 16, "o_bf16"));
  CHECK(check_ptr(lse, 4, "lse"));
  const size_t need = attn_fp8_decode_workspace_bytes(B, Hq, Hkv, Sq, Ncap, D, split);
  if (use_scratch) {
    if (need > kDecodeScratchBytes)
      return fail(ATTN_EINVAL, "these sizes need %zu bytes of partials, more than the %zu bytes of scratch the "
                  "library holds per GPU (attn_fp8_decode takes a workspace of any size)", need, kDecodeScratchBytes);
  } else if (workspace_bytes < need) {
    return fail(ATTN_EINVAL, "workspace_bytes %zu < %zu (attn_fp8_decode_workspace_bytes)", workspace_bytes, need);
  }
  CHECK(check_device());
  if (use_scratch) CHECK(scratch_address(&workspace));
  attnfp8::DecodeParams p;
  p.q8 = q8; p.qd = q_descale;
  p.k8 = k8; p.v8 = v8; p.kd = k_descale; p.vd = v_descale;
  p.seqlens = seqlens;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.Sq = Sq; p.MQ = p.G * Sq;
  p.Ncap = Ncap;
  p.nblk = (Ncap + scale_block - 1) / scale_block;
  p.nwave = decode_waves(B, Hkv, Ncap, split);
  p.split = decode_split(B, Hkv, Ncap, split);
  p.nsplit = (Ncap + 4 * p.split - 1) / (4 * p.split);
  const size_t nparts =
      (p.nwave > 0 ? (size_t)p.nwave + (size_t)B * Hkv : (size_t)B * Hkv * p.nsplit) * (size_t)p.MQ;
  p.part_o = (float*)workspace;
  p.part_m = p.part_o + nparts * D;
  p.part_l = p.part_m + nparts;
  p.o = o_bf16; p.lse = lse;
  double sc = 1.4426950408889634 / std::sqrt((double)D);
  if (hadamard) sc /= D;
  p.score_scale = (float)sc;
  return launched(attnfp8::launch_attn_fp8_decode(p, D, scale_block, causal ? 1 : 0, (hipStream_t)stream),
                  "attn_fp8_decode");
}

extern "C" {

int attn_fp8_decode(const uint8_t* q8, const float* q_descale, const uint8_t* k8, const uint8_t* v8,
                    const float* k_descale, const float* v_descale, const int32_t* seqlens, int B, int Hq, int Hkv,
                    int Sq, int Ncap, int D, int scale_block, int hadamard, int causal, int split, void* workspace,
                    size_t workspace_bytes, uint16_t* o_bf16, float* lse, void* stream) {
  return decode_impl(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, B, Hq, Hkv, Sq, Ncap, D, scale_block,
                     hadamard, causal, split, workspace, workspace_bytes, false, o_bf16, lse, stream);
}

int attn_fp8_decode_noalloc(const uint8_t* q8, const float* q_descale, const uint8_t* k8, const uint8_t* v8,
                            const float* k_descale, const float* v_descale, const int32_t* seqlens, int B, int Hq,
                            int Hkv, int Sq, int Ncap, int D, int scale_block, int hadamard, int causal, int split,
                            uint16_t* o_bf16, float* lse, void* stream) {
  return decode_impl(q8, q_descale, k8, v8, k_descale, v_descale, seqlens, B, Hq, Hkv, Sq, Ncap, D, scale_block,
                     hadamard, causal, split, nullptr, 0, true, o_bf16, lse, stream);
}

int attn_fp8_decode_split(int B, int Hkv, int Ncap, int split) {
  if (B < 1 || Hkv < 1 || Ncap < 1 || split < 0) return 0;
  if (decode_waves(B, Hkv, Ncap, split) > 0) return 0;
  return decode_split(B, Hkv, Ncap, split);
}

const char* attn_fp8_last_error(void) { return g_err; }

int attn_fp8_abi_version(void) { return ATTN_FP8_ABI_VERSION; }

}  // extern "C"
