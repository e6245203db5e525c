// BF16 fused attention forward for gfx950: the 16-bit twin of the FP8 kernel.
//
// It runs the same running-softmax loop ("Fused attention kernel", Overview
// and Implementation sketch) on BF16 Q, K, V with v_mfma_f32_32x32x16_bf16,
// FP32 statistics and P in BF16, with no rotation and no quantisation.  It
// is the accuracy yardstick that the problem statement measures FP8 error
// against ("FP8 attention that keeps FlashAttention-3 throughput at
// BF16-level accuracy", What is asked).
//
// The loop has the FP8 kernel's structure, with 32-key tiles (one tile is
// 32 x 2D bytes: 8 KiB at D = 128, the size of an FP8 64-key tile):
//   * one workgroup = 4 waves x 32 queries of one head; S^T = K Q^T, so each
//     lane of the accumulator owns one query and 16 keys (max and sum
//     in-lane up to one exchange of the lane halves); Q resident in
//     registers as the B operand;
//   * P^T in BF16 is directly the B operand of O^T += V^T P^T; the V^T
//     operand comes from the row-major V tile through ds_read_b64_tr_b16;
//   * K and V stream through three-slot LDS rings, two tiles ahead, by
//     buffer loads that write LDS (scalar addresses plus one per-lane offset;
//     rows past the end read as zeros); each step waits only for the loads
//     issued two steps earlier;
//   * step t: phase A forms P_t (exponentials, row sum, BF16 pack) with the
//     lazy reference max; a barrier; phase B adds V_t^T P_t^T to O and
//     computes S_{t+1}.  P_t is formed against the current reference first,
//     and the tile maximum is taken only when some lane's row sum shows that
//     the reference may have to move (the decisions of taking it on every
//     tile: the reference moves when a tile's largest scaled score exceeds
//     it by more than kTauBf16);
//   * an unrolled main loop over tiles that are complete and visible to every
//     query of the workgroup (ring slots as constants, no masks), then the
//     diagonal and ragged tiles in a tail with run-time slots.
#include "common.h"
#include "attn_internal.h"

namespace attnfp8 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> two BF16 values (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32 for the pair
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

constexpr float kTauBf16 = 8.0f;
constexpr int kBf16Ring = 3;
constexpr int kBf16KeyTile = 32;

template <int D>
struct Bf16Cfg {
  static constexpr int BC = kBf16KeyTile;    // keys per tile
  static constexpr int KSTEPS = D / 16;      // 32x32x16 K-steps of S^T = K Q^T
  static constexpr int NKG = BC / 16;        // 16-key steps of P V
  static constexpr int NDT = D / 32;         // 32-row (d) tiles of O^T
  static constexpr int ROWB = 2 * D;         // bytes per row
  static constexpr int TILE = BC * ROWB;
  static constexpr int CHUNKS = TILE / 1024; // 1 KiB direct-load chunks per tile
  static constexpr int CPW = CHUNKS / kWaves;
  static_assert(CHUNKS % kWaves == 0, "tile must split evenly over the waves");
};

// XOR swizzles of the 16-byte column slot per LDS row, for 64 banks of 4 bytes
// (256 bytes per bank cycle; a D = 128 row is one full cycle, a D = 64 row half
// of one).  They keep every slot inside its row, and the loader applies the
// same function, so a read of logical slot s at slot s ^ swz(row) finds it.
//   K (ds_read_b128, 16 lanes per cycle, one row per lane): any 16 consecutive
//     rows at one logical slot land in 16 distinct 16-byte bank groups.
//   V (ds_read_b64_tr_b16, 32 lanes per cycle: 4 consecutive rows x 4 slots of
//     one d-tile): the 4 rows' slot groups are disjoint.  It depends on row % 4
//     only.
template <int D>
__device__ __forceinline__ int swz_k16(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v16(int row) {
  if constexpr (D == 128) return 4 * (row & 3);
  else return 2 * (row & 3);
}

// Per-lane constants: LDS byte offsets (inside a tile) of the MFMA operands and
// of the 16-byte pieces this lane moves in the tile loads.
template <int D>
struct Bf16Lane {
  using C = Bf16Cfg<D>;
  int k[C::KSTEPS];          // K row (lane % 32), slot 2 ks + h
  int v[C::NDT];             // V^T source of d-tile dt at key step 0; + (16 kg + 8 rr) rows
  int koff[C::CPW];          // tile-load source offsets (K, V swizzles)
  int voff[C::CPW];
  uint32_t lds0;             // LDS address of this wave's first chunk in slot 0

  __device__ __forceinline__ Bf16Lane(int wave, int lane, uint32_t smem_addr) {
    const int ql = lane & 31;
    const int h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) k[ks] = ql * C::ROWB + 16 * ((2 * ks + h) ^ swz_k16<D>(ql));
    // ds_read_b64_tr_b16: lane j of each 16-lane group receives element j % 4 of
    // the rows named by lanes j / 4, j / 4 + 4, ...; source lane i of group g names
    // key row 4 (g / 2) + i / 4 (+ 8 for the second read, + 16 per key step) and
    // columns 32 dt + 16 (g % 2) + 4 (i % 4) .. + 3.  The other rows differ by
    // multiples of 4, so the V swizzle of row0 holds for all of them.
    const int g = lane >> 4;
    const int i = lane & 15;
    const int row0 = 4 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int slot = 4 * dt + 2 * (g & 1) + ((i & 3) >> 1);
      v[dt] = row0 * C::ROWB + 16 * (slot ^ swz_v16<D>(row0)) + 8 * (i & 1);
    }
#pragma unroll
    for (int c = 0; c < C::CPW; ++c) {
      const int pos = (wave * C::CPW + c) * 1024 + lane * 16;
      const int prow = pos / C::ROWB;
      const int pslot = (pos % C::ROWB) / 16;
      koff[c] = prow * C::ROWB + 16 * (pslot ^ swz_k16<D>(prow));
      voff[c] = prow * C::ROWB + 16 * (pslot ^ swz_v16<D>(prow));
    }
    lds0 = smem_addr + wave * C::CPW * 1024;
  }
};

// This wave's share of key tile kt of one head into the LDS slot at byte offset
// slot_off.  Bytes at or past lim_bytes read as zeros.
template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile16(const uint8_t* head, uint32_t lim_bytes, int kt, uint32_t slot_off,
                                             const Bf16Lane<D>& ln) {
  using C = Bf16Cfg<D>;
  // (64-bit: the prefetches run up to three tiles past the end of a head whose
  // size may come close to 2^31 bytes)
  const long long off = (long long)kt * C::TILE;
  const long long rem = (long long)lim_bytes - off;
  const v4i rsrc = make_rsrc(head + off, (uint32_t)(rem > 0 ? rem : 0));
#pragma unroll
  for (int c = 0; c < C::CPW; ++c)
    buffer_to_lds16(rsrc, IS_V ? ln.voff[c] : ln.koff[c], ln.lds0 + slot_off + c * 1024);
}

template <int D>
struct Bf16State {
  v16f o[Bf16Cfg<D>::NDT];
  float m_ref;                // reference max (log2 units)
  float l_acc;                // this lane's half of the row sum
  v4i pop[Bf16Cfg<D>::NKG];   // P^T of the last tile in BF16
};

// S^T of a tile: 32 keys x 32 queries
template <int D>
__device__ __forceinline__ v16f qk16(const uint8_t* kbuf, const Bf16Lane<D>& ln,
                                     const v4i (&qop)[Bf16Cfg<D>::KSTEPS]) {
  v16f acc = {};
#pragma unroll
  for (int ks = 0; ks < Bf16Cfg<D>::KSTEPS; ++ks) acc = mfma_bf16(lds_read_b128(kbuf + ln.k[ks]), qop[ks], acc);
  return acc;
}

// keys past the sequence, and (causal) past each query's position -> -inf
template <bool CAUSAL>
__device__ __forceinline__ void mask16(v16f& s, int t, int N, int lane, int iw, int my_q) {
  const int k0 = t * kBf16KeyTile;
  if ((k0 + kBf16KeyTile > N) || (CAUSAL && k0 + kBf16KeyTile - 1 > iw)) {
    const int lim = (CAUSAL ? (my_q < N - 1 ? my_q : N - 1) : N - 1) - k0 - 4 * (lane >> 5);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
  }
}

// P = 2^(s c - m) in BF16 into pop (key step kg: accumulator entries
// r = 8 kg .. 8 kg + 7); returns this lane's share of the row sum
template <int D>
__device__ __forceinline__ float p16(const v16f& s, Bf16State<D>& st, float c) {
  const float b = -st.m_ref;
  float rs = 0.0f;
#pragma unroll
  for (int kg = 0; kg < Bf16Cfg<D>::NKG; ++kg)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r = 8 * kg + 2 * a;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, b));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, b));
      rs += p0 + p1;
      st.pop[kg][a] = (int)pk_bf16(p0, p1);
    }
  return rs;
}

// Phase A of a step: P of the tile in s, with the lazy reference update
template <int D>
__device__ __forceinline__ void bf16_phaseA(const v16f& s, Bf16State<D>& st, float c) {
  float alpha = 1.0f;
  float rs = p16<D>(s, st, c);
  // every P is at most the row sum: while no lane's sum reaches 2^tau (less a
  // margin for the rounding of the exponent argument), no P exceeds it and the
  // reference stays (written so that a NaN sum counts as reaching it)
  if (__builtin_amdgcn_ballot_w64(!(rs <= 256.0f * (1.0f - 1.0f / 64.0f)))) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    float tmax = mx * c;            // c > 0: the max commutes with the scale
    tmax = fmaxf(tmax, swap_halves(tmax));
    const bool upd = tmax > st.m_ref + kTauBf16;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float m_new = upd ? tmax : st.m_ref;
      alpha = upd ? __builtin_amdgcn_exp2f(st.m_ref - m_new) : 1.0f;
      st.m_ref = m_new;
#pragma unroll
      for (int dt = 0; dt < Bf16Cfg<D>::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[dt][r] *= alpha;
      rs = p16<D>(s, st, c);
    }
  }
  st.l_acc = alpha * st.l_acc + rs;
}

// Phase B: O^T += V_t^T P_t^T, then S_{t+1} (when the wave computes it)
template <int D, bool CAUSAL, bool MASK_NEXT>
__device__ __forceinline__ void bf16_phaseB(v16f& s, const uint8_t* vcur, const uint8_t* knext, const Bf16Lane<D>& ln,
                                            const v4i (&qop)[Bf16Cfg<D>::KSTEPS], Bf16State<D>& st, int t, int N,
                                            int lane, int iw, int my_q, bool pv_active, bool next_valid) {
  using C = Bf16Cfg<D>;
  if (!MASK_NEXT || pv_active) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int kg = 0; kg < C::NKG; ++kg) {
        const v2i lo = lds_read_tr16(vcur + (16 * kg) * C::ROWB + ln.v[dt]);
        const v2i hi = lds_read_tr16(vcur + (16 * kg + 8) * C::ROWB + ln.v[dt]);
        const v4i a = {lo[0], lo[1], hi[0], hi[1]};
        st.o[dt] = mfma_bf16(a, st.pop[kg], st.o[dt]);
      }
  }
  // (a tile this wave will not visit must not move the reference max)
  if (!MASK_NEXT || next_valid) {
    s = qk16<D>(knext, ln, qop);
    if (MASK_NEXT) mask16<CAUSAL>(s, t + 1, N, lane, iw, my_q);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 3) void attn_bf16_kernel(AttnBf16Params p) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kBf16Ring * C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // (uniform results of a division on the vector ALU: back to scalar registers)
  const int bh = __builtin_amdgcn_readfirstlane(logical / p.n_qtiles);
  int qt = __builtin_amdgcn_readfirstlane(logical - bh * p.n_qtiles);
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;            // longest tiles first
  const int i0 = qt * kQueryTile;
  const int iw = i0 + wave * kQueriesPerWave;
  const int my_q = iw + (lane & 31);
  const int h = lane >> 5;

  const size_t head = (size_t)bh * N * D;
  const uint8_t* kh = (const uint8_t*)(p.k + head);
  const uint8_t* vh = (const uint8_t*)(p.v + head);

  // queries of this lane as the B operand: Q[q][16 ks + 8 h .. + 7]
  v4i qop[C::KSTEPS];
  {
    const int qrow = my_q < N ? my_q : N - 1;
    const uint16_t* qp = p.q + head + (size_t)qrow * D;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qop[ks] = *(const v4i*)(qp + 16 * ks + 8 * h);
  }

  const int n_kt = (N + C::BC - 1) / C::BC;
  int n_kt_wg = n_kt;              // key tiles the workgroup steps through
  int kt_w = n_kt - 1;             // last key tile this wave computes
  int n_clean = N / C::BC;         // leading tiles complete and visible to every query here
  if (CAUSAL) {
    const int last_wg = (i0 + kQueryTile - 1 < N - 1) ? i0 + kQueryTile - 1 : N - 1;
    n_kt_wg = last_wg / C::BC + 1;
    const int last_w = (iw + kQueriesPerWave - 1 < N - 1) ? iw + kQueriesPerWave - 1 : N - 1;
    kt_w = last_w / C::BC;
    n_clean = n_clean < i0 / C::BC ? n_clean : i0 / C::BC;
  }
  // bytes of K / V this workgroup reads; loads past them return zeros
  const int rows_wg = N < n_kt_wg * C::BC ? N : n_kt_wg * C::BC;
  const uint32_t lim = (uint32_t)rows_wg * C::ROWB;

  const Bf16Lane<D> ln(wave, lane, lds_addr_of(smem));
  Bf16State<D> st;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) st.o[dt] = (v16f){};
  st.m_ref = -1e30f;
  st.l_acc = 0.0f;
#pragma unroll
  for (int kg = 0; kg < C::NKG; ++kg) st.pop[kg] = (v4i){};
  const float c = p.score_scale;
  constexpr uint32_t KS = 0, VS = kBf16Ring * C::TILE;   // ring bases (byte offsets in smem)

  // prologue: K0, K1, K2, V0, V1 resident; S_0 (masked)
  issue_tile16<D, false>(kh, lim, 0, KS + 0 * C::TILE, ln);
  issue_tile16<D, false>(kh, lim, 1, KS + 1 * C::TILE, ln);
  issue_tile16<D, false>(kh, lim, 2, KS + 2 * C::TILE, ln);
  issue_tile16<D, true>(vh, lim, 0, VS + 0 * C::TILE, ln);
  issue_tile16<D, true>(vh, lim, 1, VS + 1 * C::TILE, ln);
  wait_vmem_all();
  __syncthreads();
  v16f s = qk16<D>(smem + KS, ln, qop);
  mask16<CAUSAL>(s, 0, N, lane, iw, my_q);

  // Step t: phase A (P_t), then wait until only the previous step's loads are
  // outstanding and barrier: K_{t+1} and V_t (issued two steps earlier) are
  // resident for every wave, and every wave has finished reading K_t and
  // V_{t-1}.  The step issues K_{t+3} (into K_t's slot) and V_{t+2} (into
  // V_{t-1}'s slot), then runs phase B.  Tile j lives in ring slot j % 3.
  const int t_main = n_clean - 1;
  int t = 0;
#define BF16_STEP(I, KN, KF, VC, VF)                                                                        \
  {                                                                                                       \
    const int tt = t + (I);                                                                               \
    if (tt >= t_main) {                                                                                   \
      t = tt;                                                                                             \
      break;                                                                                              \
    }                                                                                                     \
    bf16_phaseA<D>(s, st, c);                                                                             \
    wait_vmem_prev_step<2 * C::CPW>();                                                                    \
    workgroup_barrier();                                                                                  \
    issue_tile16<D, false>(kh, lim, tt + 3, KS + (KF) * C::TILE, ln);                                    \
    issue_tile16<D, true>(vh, lim, tt + 2, VS + (VF) * C::TILE, ln);                                     \
    bf16_phaseB<D, CAUSAL, false>(s, smem + VS + (VC) * C::TILE, smem + KS + (KN) * C::TILE, ln, qop, st, tt, N, \
                                  lane, iw, my_q, true, true);                                            \
  }
  for (;; t += 3) {
    BF16_STEP(0, 1, 0, 0, 2)
    BF16_STEP(1, 2, 1, 1, 0)
    BF16_STEP(2, 0, 2, 2, 1)
  }
#undef BF16_STEP

  // Tail: diagonal and ragged tiles, waves that stop early; run-time slots and
  // the main loop's partial wait (every step issues the same loads, so the
  // count still names the previous step's).
  for (; t < n_kt_wg; ++t) {
    const bool active = t <= kt_w;
    if (active) bf16_phaseA<D>(s, st, c);
    wait_vmem_prev_step<2 * C::CPW>();
    workgroup_barrier();
    issue_tile16<D, false>(kh, lim, t + 3, KS + (t % kBf16Ring) * C::TILE, ln);
    issue_tile16<D, true>(vh, lim, t + 2, VS + ((t + 2) % kBf16Ring) * C::TILE, ln);
    bf16_phaseB<D, CAUSAL, true>(s, smem + VS + (t % kBf16Ring) * C::TILE,
                                 smem + KS + ((t + 1) % kBf16Ring) * C::TILE, ln, qop, st, t, N, lane, iw, my_q,
                                 active, t + 1 <= kt_w);
  }
  wait_vmem_all();   // no tile load may still be writing LDS when the workgroup ends

  // ---- epilogue: O = O_acc / l ; LSE = ln 2 * (m + log2 l)
  // (the lane's half is recomputed here rather than kept live through the
  // tail, which runs at the register limit of three waves per SIMD)
  const int h_out = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
  const float l_tot = st.l_acc + swap_halves(st.l_acc);
  const float inv_l = 1.0f / l_tot;
  if (my_q < N) {
    uint16_t* orow = p.o + head + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * dt + 8 * a + 4 * h_out;
        uint32_t w0 = pk_bf16(st.o[dt][4 * a + 0] * inv_l, st.o[dt][4 * a + 1] * inv_l);
        uint32_t w1 = pk_bf16(st.o[dt][4 * a + 2] * inv_l, st.o[dt][4 * a + 3] * inv_l);
        *(v2i*)(orow + d) = (v2i){(int)w0, (int)w1};
      }
    if (h_out == 0) p.lse[(size_t)bh * N + my_q] = kLn2 * (st.m_ref + __builtin_amdgcn_logf(l_tot));
  }
}

template __global__ void attn_bf16_kernel<64, false>(AttnBf16Params);
template __global__ void attn_bf16_kernel<64, true>(AttnBf16Params);
template __global__ void attn_bf16_kernel<128, false>(AttnBf16Params);
template __global__ void attn_bf16_kernel<128, true>(AttnBf16Params);

hipError_t launch_attn_bf16(const AttnBf16Params& p, int D, int causal, int BH, hipStream_t stream) {
  dim3 grid(BH * p.n_qtiles);
  if (D == 64) {
    if (causal) attn_bf16_kernel<64, true><<<grid, 256, 0, stream>>>(p);
    else attn_bf16_kernel<64, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (causal) attn_bf16_kernel<128, true><<<grid, 256, 0, stream>>>(p);
    else attn_bf16_kernel<128, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace attnfp8
