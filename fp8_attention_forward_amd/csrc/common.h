// Device helpers shared by the gfx950 kernels of this library.
//
// Lane layouts used below (CDNA4 MFMA, wave64):
//   * v_mfma_f32_32x32x64_f8f6f4 (fp8 e4m3 operands): lane l holds, for the A
//     operand, row (l % 32) and 32 k-values in two 16-byte halves: bytes
//     0..15 are k = 16*(l/32) + 0..15, bytes 16..31 are k = 32 + 16*(l/32) +
//     0..15 (measured on the device with per-lane E8M0 scales: the 32-element
//     scale block k = 0..31 is the first half of both lane halves); the B
//     operand likewise with column (l % 32).  The accumulator register r of
//     lane l is element (row 8*(r/4) + 4*(l/32) + r%4, col l%32).  The scale
//     operand of lane l applies to row (column) l % 32 and k-block l / 32.
//   * v_mfma_f32_32x32x16_bf16: the same with 8 bf16 k-values per lane,
//     k = 8*(l/32) .. +7.
//   * ds_read_b64_tr_b8: within each group of 16 lanes, lane i names an 8-byte
//     row R_i; lane j receives byte (j % 8) of rows j/8, j/8+2, ..., j/8+14.
//   * ds_read_b64_tr_b16: lane j receives element (j % 4) of rows j/4, j/4+4,
//     j/4+8, j/4+12 (four 2-byte elements per row).
// Only the relation between A and B matters for a contraction, so every
// permutation of k used here is applied identically to both operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// read-only global data seen through the constant address space: uniform
// indexing then compiles to scalar (s_load) reads
typedef __attribute__((address_space(4))) const float cfloat;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// fp8 e4m3 x fp8 e4m3 -> fp32, 32x32x64 (scale operands 0 select the unscaled form)
__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16(const v4i& a, const v4i& b, const v16f& c) {
  v8bf av = __builtin_bit_cast(v8bf, a);
  v8bf bv = __builtin_bit_cast(v8bf, b);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ v2i lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(v2i, p));
}

__device__ __forceinline__ v2i lds_read_tr16(const uint8_t* p) {
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4s, p));
  return __builtin_bit_cast(v2i, r);
}

__device__ __forceinline__ v4i lds_read_b128(const uint8_t* p) {
  return *LDS_PTR(const v4i, p);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16*l (lds_base must be the same for the whole wave).
__device__ __forceinline__ void global_to_lds16(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, LDS_PTR(void, lds_base), 16, 0, 0);
}

// Buffer resource for raw byte access to [base, base + bytes): loads at or past
// `bytes` return zeros without touching memory (gfx9 descriptor, 32-bit data
// format, no stride, no swizzle).
// The arguments must be wave-uniform; readfirstlane keeps the descriptor in
// scalar registers whatever the compiler's divergence analysis concludes.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (v4i){__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes (buffer
// offset voff) land at lds_addr + 16 * l.  Issued as inline assembly, so the
// compiler neither counts it nor waits for it: the caller owns the vmcnt wait
// and the barrier that make the data visible.  Every address operand is scalar
// except the per-lane offset.
//
// The compiler's hazard checks do not look inside inline assembly, so the
// statement brings its own wait states: on gfx9 a vector-memory instruction
// that reads an SGPR written by a VALU instruction (v_readfirstlane, which
// may well produce the descriptor) needs 5 wait states in between, and an LDS
// DMA needs 1 after M0 is written.  s_nop 4 provides 5.
#define ATTN_LDS_DMA_NOP "s_nop 4\n\t"
__device__ __forceinline__ void buffer_to_lds16(const v4i& rsrc, int voff, uint32_t lds_addr) {
  asm volatile(ATTN_LDS_DMA_NOP "buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// byte address of an LDS object as the hardware sees it
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)LDS_PTR(const uint8_t, p);
}

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier without the memory fence of __syncthreads (which would wait
// for every outstanding global load, including prefetches still in flight).
// The LDS tiles a step reads were completed by an explicit vmcnt wait before it.
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N): all but the N most recent vector-memory operations done.
// Written as inline assembly so that it stays exactly where it is placed (the
// compiler's own waits are added around it as needed).
template <int N>
__device__ __forceinline__ void wait_vmem_prev_step() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// value of lane (l ^ 32)
__device__ __forceinline__ float swap_halves(float x) {
  int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, x)));
}

// value of lane (l ^ m) for m < 32 (ds_swizzle bit mode: and 0x1f, xor m)
template <int M>
__device__ __forceinline__ float xor_lanes(float x) {
  static_assert(M > 0 && M < 32, "swizzle xor covers lanes within 32");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), (M << 10) | 0x1F));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, xor_lanes<1>(x));
  x = fmaxf(x, xor_lanes<2>(x));
  x = fmaxf(x, xor_lanes<4>(x));
  x = fmaxf(x, xor_lanes<8>(x));
  x = fmaxf(x, xor_lanes<16>(x));
  x = fmaxf(x, swap_halves(x));
  return x;
}

// two fp32 -> two e4m3 codes (round to nearest even; inputs must lie in [-448, 448])
// packed into the low 16 bits (word_sel = false) or high 16 bits of `old`
template <bool HI>
__device__ __forceinline__ int cvt_pk_fp8(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Workgroup order: the dispatcher hands consecutive workgroup ids to the 8
// XCDs in turn.  Remap so that each XCD receives one contiguous range of
// logical tiles (so the query tiles of a head share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  if (total % 8 != 0) return pid;
  return (pid % 8) * (total / 8) + pid / 8;
}

}  // namespace attnfp8
