// FP8 (e4m3) fused attention forward for gfx950.
//
// Method: the running-softmax loop of "Fused attention kernel" (Overview and
// Implementation sketch): per key block S = Q K_j^T, running row max and row
// sum, rescale of the old state by exp(old max - new max), O += P V_j, and a
// final O / l and logsumexp; every key block is scored, the scores and
// probabilities never leave the chip.  The 8-bit inputs come from the
// block-scaled e4m3 quantiser (Variants / 8-bit forward pass); V keeps its
// token-major layout in HBM and is transposed on chip while it is read from
// LDS (the page rejects a separate global transpose for its bandwidth).
// FLAMIA (4.3 Ablation Study) folds the score scales into one multiplier.
//
// gfx950 design (one workgroup = 4 waves = 128 queries of one head; key
// tiles of 64 keys):
//   * S^T = K_j Q^T on v_mfma_f32_32x32x64_f8f6f4: A = K tile rows from LDS,
//     B = the wave's 32 queries, held in registers for the whole loop.  In the
//     accumulator each lane owns ONE query and 16 keys per 32-key subtile, so
//     the row max / row sum are in-lane except for one exchange between the
//     two lane halves.
//   * P is converted to e4m3 in registers and is directly the B operand of
//     O^T += V_j^T P^T (same instruction); the V^T operand comes from the
//     row-major V tile in LDS through ds_read_b64_tr_b8, in the key order the
//     S accumulator produced.  O^T keeps one query per lane too, so the
//     rescale factor is lane-local.
//   * Software pipeline across tiles: the MFMAs of S_{j+1} are issued in the
//     same basic block as the exponentials of tile j, so the matrix cores and
//     the vector ALU work at the same time (the page's two-stage overlap of
//     the score product of block j+1 with the softmax of block j, done here
//     inside one wave).  K and V stream through three-slot LDS rings, two
//     tiles ahead of use, by buffer loads that write LDS directly; all their
//     address operands are scalar except one fixed per-lane offset, and rows
//     past the end read as zeros.  16-byte columns are XOR-swizzled per row
//     against bank conflicts.
//   * Loop split: an unrolled main loop over the tiles that are complete and
//     visible to every query of the workgroup (no mask code, ring slots as
//     constants), then at most three tail steps for the diagonal and ragged
//     tiles.
//   * Scale folding: t = s * (dq * dk_j * score_scale) in log2 units, one FMA
//     per score with the reference max.  V's block scale is a power of two
//     (the quantiser writes it so) and is applied exactly inside the matrix
//     core: its E8M0 exponent is the A-operand scale of the P V product, so P
//     carries no V factor and keeps e4m3's full range.
//   * Lazy rescale: the reference max only moves when a tile's max exceeds it
//     by more than kTau (log2 units), so most tiles skip the O rescale; P is
//     then <= 2^kTau, inside e4m3's range.  With exact exponentials P is
//     formed first and the tile max is only taken when the row sum shows that
//     the reference might have to move (the same decisions, without the max
//     on most tiles).
//   * Causal: key tiles past the workgroup's last query are not loaded, tiles
//     past a wave's last query are not computed, masks only on diagonal and
//     tail tiles; query tiles are scheduled longest first.
#include <type_traits>

#include "common.h"
#include "attn_internal.h"
#include "fp8_tiles.h"

namespace attnfp8 {

constexpr int kRing = 3;         // LDS slots per operand ring

// Per-lane constants of the tile loads: the buffer offset (inside one tile) of
// each 16-byte piece this lane moves, already permuted by the LDS swizzle, and
// the LDS address of the wave's first 1 KiB chunk in ring slot 0.
template <int D>
struct Fp8Dma {
  using C = Fp8Cfg<D>;
  int koff[C::CHUNKS_PER_WAVE];
  int voff[C::CHUNKS_PER_WAVE];
  uint32_t lds0;

  __device__ __forceinline__ Fp8Dma(int wave, int lane, uint32_t smem_addr) {
#pragma unroll
    for (int i = 0; i < C::CHUNKS_PER_WAVE; ++i) {
      const int pos = (wave * C::CHUNKS_PER_WAVE + i) * 1024 + lane * 16;
      const int prow = pos / D;
      const int pslot = (pos % D) / 16;
      koff[i] = prow * D + 16 * (pslot ^ swz_k<D>(prow));
      voff[i] = prow * D + 16 * (pslot ^ swz_v<D>(prow));
    }
    lds0 = smem_addr + wave * C::CHUNKS_PER_WAVE * 1024;
  }
};

// Issue this wave's share of key tile kt (rows kt*kBC ..) of one head into the
// LDS slot at byte offset slot_off.  Rows at or past `lim_bytes / D` read as
// zeros, so every step issues the same number of loads.
template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile(const uint8_t* head, uint32_t lim_bytes, int kt, uint32_t slot_off,
                                           const Fp8Dma<D>& dma) {
  using C = Fp8Cfg<D>;
  const int off = kt * C::TILE;
  const int rem = (int)lim_bytes - off;
  const v4i rsrc = make_rsrc(head + off, (uint32_t)(rem > 0 ? rem : 0));
#pragma unroll
  for (int i = 0; i < C::CHUNKS_PER_WAVE; ++i)
    buffer_to_lds16(rsrc, IS_V ? dma.voff[i] : dma.koff[i], dma.lds0 + slot_off + i * 1024);
}

// S^T of one tile: 32 keys x 32 queries per subtile
template <int D, bool MX>
__device__ __forceinline__ void qk_tile(const uint8_t* kbuf, const Fp8LaneOffsets<D>& lo,
                                        const v8i (&qop)[Fp8Cfg<D>::KSTEPS], STile<D>& s, const KsScales<D>& sk,
                                        const KsScales<D>& sq) {
  KOps<D> k;
  read_k<D>(kbuf, lo, k);
#pragma unroll
  for (int sub = 0; sub < Fp8Cfg<D>::NSUB; ++sub) s[sub] = qk_mfma<D, MX>(k, qop, sub, sk, sq);
}

// Per-wave running state of the loop.
template <int D>
struct Fp8State {
  v16f o[Fp8Cfg<D>::NDT];
  float m_ref;     // reference max (log2 units)
  float l_acc;     // this lane's half of the row sum
  v8i pop;         // P^T of the last tile in e4m3 (B operand of the P V product)
  int move_run;    // (wave-uniform) consecutive tiles that moved the reference
};

// The rows of one attention sequence as the loop sees them.
struct Fp8SeqView {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qd;     // block descales of this sequence (block 0 first)
  const float* kd;
  const float* vd;
  uint16_t* o;
  float* lse;
  int N;               // tokens
  float score_scale;
};

// Mask of a freshly computed score tile: keys past the sequence, and (causal)
// past each query's position, get -inf.  MASK = false: the tile is known to
// be complete and visible to every query of the workgroup, and no code is
// emitted.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void tile_mask(STile<D>& s, int t, int N, int lane, int iw, int my_q) {
  using C = Fp8Cfg<D>;
  const int h = lane >> 5;
  const int k0 = t * kBC;
  const bool need_mask = MASK && ((k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > iw));
  if (need_mask) {
    const int lim = (CAUSAL ? (my_q < N - 1 ? my_q : N - 1) : N - 1) - k0 - 4 * h;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (sub * 32 + 8 * (r >> 2) + (r & 3) > lim) s[sub][r] = -INFINITY;
  }
}

// P of one score tile against the reference: P = 2^(t - m) in e4m3 into pop
// (the B operand of the P V product).  Returns this lane's share of the row
// sum; *q4max gets the largest sum of 4 of its P (the exponentials come in
// fours anyway): when that stays below kMoveBound no single P can exceed
// 2^kTau, so the reference need not move.
template <int D, int EXPM>
__device__ __forceinline__ float p_tile(const STile<D>& s, v8i& pop, float c, float bias, float* q4max) {
  using C = Fp8Cfg<D>;
  const ExpArgs<EXPM> ex(c, bias);
  float rs = 0.0f;
  float qm = 0.0f;
#pragma unroll
  for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float p0 = ex(s[sub][4 * a + 0]);
      float p1 = ex(s[sub][4 * a + 1]);
      float p2 = ex(s[sub][4 * a + 2]);
      float p3 = ex(s[sub][4 * a + 3]);
      const float q4 = (p0 + p1) + (p2 + p3);
      rs += q4;
      // (fmaxf drops a NaN operand: test for it on the sum instead)
      qm = fmaxf(qm, q4);
      // (the conversion keeps the other half of its destination: start from
      // the previous tile's word, which is dead by now)
      int w = cvt_pk_fp8<false>(p0, p1, pop[4 * sub + a]);
      w = cvt_pk_fp8<true>(p2, p3, w);
      pop[4 * sub + a] = w;
    }
  *q4max = rs == rs ? qm : rs;
  return rs;
}

// Lazy reference update from the tile maximum: the reference m moves only
// when the tile's largest scaled score exceeds it by more than tau, and then
// to kLift below that maximum; O is rescaled by alpha = 2^(m_old - m_new) (1
// for lanes that keep theirs).
// Returns whether any lane of the wave moved.
template <int D>
__device__ __forceinline__ bool move_reference(const STile<D>& s, Fp8State<D>& st, float c, float& alpha) {
  using C = Fp8Cfg<D>;
  float mx = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
  float tmax = mx * c;              // c > 0: the max commutes with the scale
  tmax = fmaxf(tmax, swap_halves(tmax));
  const bool upd = tmax > st.m_ref + kTau;
  if (!__builtin_amdgcn_ballot_w64(upd)) return false;
  const float m_new = upd ? tmax - kLift : st.m_ref;
  alpha = upd ? __builtin_amdgcn_exp2f(st.m_ref - m_new) : 1.0f;
  st.m_ref = m_new;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[dt][r] *= alpha;
  return true;
}

// Tiles in a row that moved the reference after which the next tile's
// maximum is taken before its exponentials
constexpr int kMaxFirstRun = 2;

// Largest P (<= 2^kTau) the reference allows without moving, less a margin
// for the rounding of the exponent argument (|m| < 2^14).
constexpr float kMoveBound = 445.7218f * (1.0f - 1.0f / 64.0f);

// One pipelined step in two phases with the workgroup barrier between them.
// On entry S_t (masked) is ready.  Phase A turns S_t into P_t (exponentials,
// row sum, e4m3) with the lazy reference update that tile t asks for.
// Phase B (after the barrier) adds V_t^T P_t^T to O and computes S_{t+1} =
// K_{t+1} Q^T; V and K operands are read from LDS right before their MFMAs.
// One score buffer serves both phases (S_t is dead once P_t is packed),
// which keeps the registers low enough for three waves per SIMD: the latency
// one wave waits on, the others fill.
//
// Exact exponentials: the reference moves only when some P_t would exceed
// 2^tau against it, and a sum of four P bounds each of them.  So P_t is
// formed against the current reference first, and the tile maximum is taken
// only when one of some lane's sums of four reaches kMoveBound (rarely once
// the reference has settled; always on the first tile, whose reference is
// -1e30 and whose P overflow to +inf).  When the reference does move, P_t is
// formed again, and each P is then at most 2^kLift.  The decisions are those of taking
// the maximum of every tile.  Moves come in runs on some inputs (scores that
// keep growing along the keys): after two steps in a row that moved, the
// wave takes the maximum first and forms P once, which makes the same
// decisions (a move needs a P above 2^tau, and such a P trips the test) at
// the cost of one maximum when the run has ended.  Schraudolph's exponential cannot be
// formed first: past 2^128 its bits run into the sign field instead of
// saturating, so there the maximum is taken before the exponentials, on
// every tile.
template <int D, int EXPM>
__device__ __forceinline__ void fp8_phaseA(const STile<D>& s, Fp8State<D>& st, float c) {
  float alpha = 1.0f;
  float rs, q4;
  if constexpr (EXPM == kExpExact) {
    bool take_max = st.move_run >= kMaxFirstRun;
    bool have_p = false;
    if (!take_max) {
      rs = p_tile<D, EXPM>(s, st.pop, c, -st.m_ref, &q4);
      have_p = true;
      // (written so that a NaN also counts)
      take_max = __builtin_amdgcn_ballot_w64(!(q4 <= kMoveBound)) != 0;
    }
    bool moved = false;
    if (take_max) {
      moved = move_reference<D>(s, st, c, alpha);
      if (moved) have_p = false;
    }
    st.move_run = moved ? st.move_run + 1 : 0;
    if (!have_p) rs = p_tile<D, EXPM>(s, st.pop, c, -st.m_ref, &q4);
  } else {
    move_reference<D>(s, st, c, alpha);
    rs = p_tile<D, EXPM>(s, st.pop, c, -st.m_ref, &q4);
  }
  st.l_acc = alpha * st.l_acc + rs;
}

// V's scale operands of the P V product, one per 32-row d-tile (E8M0)
template <int D>
struct DtScales {
  int v[Fp8Cfg<D>::NDT];
};

template <int D, bool CAUSAL, bool MASK_NEXT, bool MX>
__device__ __forceinline__ void fp8_phaseB(STile<D>& s, const uint8_t* vcur, const uint8_t* knext,
                                           const Fp8LaneOffsets<D>& lo, const v8i (&qop)[Fp8Cfg<D>::KSTEPS],
                                           Fp8State<D>& st, int t, int N, int lane, int iw, int my_q,
                                           bool pv_active, bool next_valid, const DtScales<D>& sv,
                                           const KsScales<D>& sk_next, const KsScales<D>& sq) {
  using C = Fp8Cfg<D>;
  if (!MASK_NEXT || pv_active) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      v2i part[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part[rr] = lds_read_tr8(vcur + 16 * rr * D + lo.v[dt]);
      const v8i a = {part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
      st.o[dt] = mfma_f8x<true>(a, st.pop, st.o[dt], sv.v[dt], 127);
    }
  }
  // (a tile this wave will not visit must not move the reference max)
  if (!MASK_NEXT || next_valid) {
    // K operands one 32-key subtile at a time (16 registers in flight)
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      v16f acc = {};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        const v4i a0 = lds_read_b128(knext + sub * 32 * D + lo.k[ks][0]);
        const v4i a1 = lds_read_b128(knext + sub * 32 * D + lo.k[ks][1]);
        const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        acc = mfma_f8x<MX>(a, qop[ks], acc, sk_next.v[ks], sq.v[ks]);
      }
      s[sub] = acc;
    }
    tile_mask<D, CAUSAL, MASK_NEXT>(s, t + 1, N, lane, iw, my_q);
  }
}

// One query tile (128 queries) of one sequence: the whole loop.  The view
// holds the sequence's rows (a head of the dense layout, or one document of a
// packed head), its block descales and its output rows.
// GRP = 32 (with MX): one power-of-two scale per 32 channels of a block, the
// descales of block b at [b * D / 32, (b + 1) * D / 32).
template <int D, int SB, bool CAUSAL, int EXPM, bool MX, int GRP = 0>
__device__ __forceinline__ void attn_fp8_seq(const Fp8SeqView& seq, int qt) {
  static_assert(GRP == 0 || (GRP == 32 && MX), "32-channel scales are power-of-two scales");
  constexpr int NG = GRP == 0 ? 1 : D / GRP;   // descales per block
  using C = Fp8Cfg<D>;
  constexpr int TPB = SB / kBC;   // key tiles per scale block
  // three-slot rings for K (slots 0..2) and V (slots 3..5): a tile arrives two
  // steps after its loads are issued
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kRing * C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = seq.N;
  const int i0 = qt * kQueryTile;
  const int iw = i0 + wave * kQueriesPerWave;
  const int my_q = iw + (lane & 31);
  const int h = lane >> 5;

  const uint8_t* kh8 = seq.k8;
  const uint8_t* vh8 = seq.v8;
  // block descales are read-only for the whole launch: scalar loads
  const cfloat* kd = (const cfloat*)seq.kd;
  const cfloat* vd = (const cfloat*)seq.vd;

  // queries of this lane as the B operand: Q[q][op_channel(ks, h, 0..1) .. +15]
  v8i qop[C::KSTEPS];
  {
    const int qrow = my_q < N ? my_q : N - 1;
    const uint8_t* qp = seq.q8 + (size_t)qrow * D;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      v4i lo = *(const v4i*)(qp + op_channel(ks, h, 0));
      v4i hi = *(const v4i*)(qp + op_channel(ks, h, 1));
      qop[ks] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  // (a wave's 32 queries lie in one scale block: SB is a multiple of 64 and
  // iw of 32, and the clamp to N - 1 stays in the last block)
  const int qblk = __builtin_amdgcn_readfirstlane((my_q < N ? my_q : N - 1) / SB);
  // MX: the matrix cores apply the power-of-two block scales (E8M0 exponents
  // sq, sk, sv), so the score scale is the constant score_scale and V needs no
  // fold into P
  const float c_q = MX ? seq.score_scale : seq.qd[qblk] * seq.score_scale;
  KsScales<D> sq;
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) {
    if constexpr (GRP == 0) {
      sq.v[ks] = MX ? e8m0_of(seq.qd[qblk]) : 0;
    } else {
      // the scale of lane half h covers k-block h of K-step ks: channels
      // 64 ks + 32 h .. + 31, group 2 ks + h (op_channel puts them there)
      const int lo_e = e8m0_of(seq.qd[qblk * NG + 2 * ks]);
      const int hi_e = e8m0_of(seq.qd[qblk * NG + 2 * ks + 1]);
      sq.v[ks] = h ? hi_e : lo_e;
    }
  }

  const int n_kt = (N + kBC - 1) / kBC;
  int n_kt_wg = n_kt;              // key tiles the workgroup steps through
  int kt_w = n_kt - 1;             // last key tile this wave computes
  int n_clean = N / kBC;           // leading tiles complete and visible to every query here
  if (CAUSAL) {
    const int last_wg = (i0 + kQueryTile - 1 < N - 1) ? i0 + kQueryTile - 1 : N - 1;
    n_kt_wg = last_wg / kBC + 1;
    const int last_w = (iw + kQueriesPerWave - 1 < N - 1) ? iw + kQueriesPerWave - 1 : N - 1;
    kt_w = last_w / kBC;
    n_clean = n_clean < i0 / kBC ? n_clean : i0 / kBC;
  } else {
    // (kept a run-time value: folded to n_kt - 1, it lets the compiler merge
    // the tail into a form that no longer fits three waves per SIMD)
    asm volatile("" : "+s"(kt_w));
  }
  // bytes of K / V this workgroup reads; loads past them return zeros
  const int rows_wg = N < n_kt_wg * kBC ? N : n_kt_wg * kBC;
  const uint32_t lim = (uint32_t)rows_wg * D;

  const Fp8LaneOffsets<D> lo(lane);
  const Fp8Dma<D> dma(wave, lane, lds_addr_of(smem));
  Fp8State<D> st;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) st.o[dt] = (v16f){};
  st.m_ref = -1e30f;
  st.l_acc = 0.0f;
  st.pop = (v8i){};
  st.move_run = kMaxFirstRun;      // (the first tile always moves the reference)

  // per-tile score scale
  auto c_of = [&](int t) { return MX ? c_q : c_q * kd[(t < n_kt ? t : n_kt - 1) / TPB]; };
  // E8M0 exponents of a tile's K block scale (MX only) and V block scale (a
  // power of two in every mode)
  auto sk_of = [&](int t) {
    KsScales<D> r;
    const int b = (t < n_kt ? t : n_kt - 1) / TPB;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      if constexpr (GRP == 0) {
        r.v[ks] = MX ? e8m0_of(kd[b]) : 0;
      } else {
        const int lo_e = e8m0_of(kd[b * NG + 2 * ks]);
        const int hi_e = e8m0_of(kd[b * NG + 2 * ks + 1]);
        r.v[ks] = h ? hi_e : lo_e;
      }
    }
    return r;
  };
  auto sv_of = [&](int t) {
    DtScales<D> r;
    const int b = (t < n_kt ? t : n_kt - 1) / TPB;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) r.v[dt] = e8m0_of(vd[b * NG + (GRP == 0 ? 0 : dt)]);
    return r;
  };
  constexpr uint32_t KS = 0, VS = kRing * C::TILE;   // ring bases (byte offsets in smem)

  // prologue: K0, K1, K2, V0, V1 resident; S_0 (masked)
  issue_tile<D, false>(kh8, lim, 0, KS + 0 * C::TILE, dma);
  issue_tile<D, false>(kh8, lim, 1, KS + 1 * C::TILE, dma);
  issue_tile<D, false>(kh8, lim, 2, KS + 2 * C::TILE, dma);
  issue_tile<D, true>(vh8, lim, 0, VS + 0 * C::TILE, dma);
  issue_tile<D, true>(vh8, lim, 1, VS + 1 * C::TILE, dma);
  wait_vmem_all();
  __syncthreads();
  STile<D> s;
  qk_tile<D, MX>(smem + KS, lo, qop, s, sk_of(0), sq);
  tile_mask<D, CAUSAL, true>(s, 0, N, lane, iw, my_q);

  // Step t: phase A (P_t), then wait until only the previous step's loads are
  // outstanding and barrier: K_{t+1} and V_t (issued two steps earlier) are
  // now resident for every wave, and every wave has finished reading K_t and
  // V_{t-1}.  The step issues K_{t+3} (into K_t's slot) and V_{t+2} (into
  // V_{t-1}'s slot), then runs phase B.  Tile j lives in ring slot j % 3.
  //
  // Main loop: steps whose next tile needs no mask and is computed by every
  // wave; ring slots are compile-time constants (unrolled over the 3 slots).
  const int t_main = n_clean - 1;
  int t = 0;
#define FP8_STEP(I, KN, KF, VC, VF)                                                                   \
  {                                                                                                  \
    const int tt = t + (I);                                                                          \
    if (tt >= t_main) {                                                                              \
      t = tt;                                                                                        \
      break;                                                                                         \
    }                                                                                                \
    fp8_phaseA<D, EXPM>(s, st, c_of(tt));                                                            \
    wait_vmem_prev_step<2 * C::CHUNKS_PER_WAVE>();                                                   \
    workgroup_barrier();                                                                             \
    issue_tile<D, false>(kh8, lim, tt + 3, KS + (KF) * C::TILE, dma);                                \
    issue_tile<D, true>(vh8, lim, tt + 2, VS + (VF) * C::TILE, dma);                                 \
    fp8_phaseB<D, CAUSAL, false, MX>(s, smem + VS + (VC) * C::TILE, smem + KS + (KN) * C::TILE, lo, qop, st,   \
                                     tt, N, lane, iw, my_q, true, true, sv_of(tt), sk_of(tt + 1), sq);       \
  }
  for (;; t += 3) {
    FP8_STEP(0, 1, 0, 0, 2)
    FP8_STEP(1, 2, 1, 1, 0)
    FP8_STEP(2, 0, 2, 2, 1)
  }
#undef FP8_STEP

  // Tail: diagonal and ragged tiles, masks, and waves that stop early; ring
  // slots computed at run time.  The loads are waited for in full here
  // (vmcnt(0)), so the wait stays correct whatever other memory operations the
  // compiler schedules in this part.
  for (; t < n_kt_wg; ++t) {
    const bool active = t <= kt_w;
    if (active) fp8_phaseA<D, EXPM>(s, st, c_of(t));
    wait_vmem_all();
    workgroup_barrier();
    issue_tile<D, false>(kh8, lim, t + 3, KS + (t % kRing) * C::TILE, dma);
    issue_tile<D, true>(vh8, lim, t + 2, VS + ((t + 2) % kRing) * C::TILE, dma);
    fp8_phaseB<D, CAUSAL, true, MX>(s, smem + VS + (t % kRing) * C::TILE, smem + KS + ((t + 1) % kRing) * C::TILE,
                                    lo, qop, st, t, N, lane, iw, my_q, active, t + 1 <= kt_w, sv_of(t), sk_of(t + 1),
                                    sq);
  }
  wait_vmem_all();   // no tile load may still be writing LDS when the workgroup ends

  // ---- epilogue: O = O_acc / l ; LSE = ln 2 * (m + log2 l)
  const float l_tot = st.l_acc + swap_halves(st.l_acc);
  const float inv_l = 1.0f / l_tot;
  if (my_q < N) {
    uint16_t* orow = seq.o + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * dt + 8 * a + 4 * h;
        uint32_t w0 = pack_bf16x2(st.o[dt][4 * a + 0] * inv_l, st.o[dt][4 * a + 1] * inv_l);
        uint32_t w1 = pack_bf16x2(st.o[dt][4 * a + 2] * inv_l, st.o[dt][4 * a + 3] * inv_l);
        *(v2i*)(orow + d) = (v2i){(int)w0, (int)w1};
      }
    if (h == 0) seq.lse[my_q] = kLn2 * (st.m_ref + __builtin_amdgcn_logf(l_tot));
  }
}

// Dense layout: one workgroup per (batch x head, query tile).
template <int D, int SB, bool CAUSAL, int EXPM, bool MX, int GRP = 0>
__global__ __launch_bounds__(256, 3) void attn_fp8_kernel(AttnFp8Params p) {
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  // (the division runs on the vector ALU: bring the uniform results back to
  // scalar registers, so that every address derived from them stays scalar)
  const int bh = __builtin_amdgcn_readfirstlane(logical / p.n_qtiles);
  int qt = __builtin_amdgcn_readfirstlane(logical - bh * p.n_qtiles);
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;            // longest tiles first
  const size_t head = (size_t)bh * p.N * D;
  Fp8SeqView seq;
  seq.q8 = p.q8 + head;
  seq.k8 = p.k8 + head;
  seq.v8 = p.v8 + head;
  constexpr int NG = GRP == 0 ? 1 : D / GRP;
  seq.qd = p.qd + (size_t)bh * p.nblk * NG;
  seq.kd = p.kd + (size_t)bh * p.nblk * NG;
  seq.vd = p.vd + (size_t)bh * p.nblk * NG;
  seq.o = p.o + head;
  seq.lse = p.lse + (size_t)bh * p.N;
  seq.N = p.N;
  seq.score_scale = p.score_scale;
  attn_fp8_seq<D, SB, CAUSAL, EXPM, MX, GRP>(seq, qt);
}

// Packed documents ("FLAMIA", Abstract and 4.1 Performance on Packed
// Documents: documents packed without repacking, document-local scales).
// Workgroup w takes item w / H of the work list (document, query tile),
// head w % H: heads of one item are neighbours, and the dispatcher's turn over
// the 8 XCDs sends every item of a head to the same XCD when H is a multiple
// of 8.  Workgroups past the item count leave before any barrier.
template <int D, int SB, bool CAUSAL, int EXPM, bool MX>
__global__ __launch_bounds__(256, 3) void attn_fp8_varlen_kernel(AttnFp8VarlenParams p) {
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x / p.H);   // (uniform: scalar loads below)
  const int h = blockIdx.x - e * p.H;
  if (e >= p.ws[0]) return;
  const int2 item = ((const int2*)(p.ws + kWsHeaderInts))[e];
  const int d = item.x;
  const int a = p.cu[d];                  // checked by the schedule kernel: 0 <= a <= cu[d+1] <= T
  const size_t row0 = (size_t)h * p.T + a;
  const size_t slot0 = (size_t)h * p.nslot + a / SB + d;
  Fp8SeqView seq;
  seq.q8 = p.q8 + row0 * D;
  seq.k8 = p.k8 + row0 * D;
  seq.v8 = p.v8 + row0 * D;
  seq.qd = p.qd + slot0;
  seq.kd = p.kd + slot0;
  seq.vd = p.vd + slot0;
  seq.o = p.o + row0 * D;
  seq.lse = p.lse + row0;
  seq.N = p.cu[d + 1] - a;
  seq.score_scale = p.score_scale;
  attn_fp8_seq<D, SB, CAUSAL, EXPM, MX>(seq, item.y);
}

#define FP8_INST(D, SB, CA, E, MX)                                                  \
  template __global__ void attn_fp8_kernel<D, SB, CA, E, MX>(AttnFp8Params);        \
  template __global__ void attn_fp8_varlen_kernel<D, SB, CA, E, MX>(AttnFp8VarlenParams);
#define FP8_INST_E(D, SB, CA)                                                                 \
  FP8_INST(D, SB, CA, kExpExact, false) FP8_INST(D, SB, CA, kExpSchraudolph, false)           \
  FP8_INST(D, SB, CA, kExpExact, true) FP8_INST(D, SB, CA, kExpSchraudolph, true)             \
  template __global__ void attn_fp8_kernel<D, SB, CA, kExpExact, true, 32>(AttnFp8Params);    \
  template __global__ void attn_fp8_kernel<D, SB, CA, kExpSchraudolph, true, 32>(AttnFp8Params);
FP8_INST_E(64, 64, false)
FP8_INST_E(64, 64, true)
FP8_INST_E(64, 128, false)
FP8_INST_E(64, 128, true)
FP8_INST_E(128, 64, false)
FP8_INST_E(128, 64, true)
FP8_INST_E(128, 128, false)
FP8_INST_E(128, 128, true)

template <int D, int SB, int E, bool MX, class P>
static void launch_dcem(const P& p, int causal, int grp, dim3 grid, hipStream_t stream) {
  if constexpr (std::is_same<P, AttnFp8Params>::value) {
    if (MX && grp == 32) {
      if (causal) attn_fp8_kernel<D, SB, true, E, true, 32><<<grid, 256, 0, stream>>>(p);
      else attn_fp8_kernel<D, SB, false, E, true, 32><<<grid, 256, 0, stream>>>(p);
    } else if (causal) {
      attn_fp8_kernel<D, SB, true, E, MX><<<grid, 256, 0, stream>>>(p);
    } else {
      attn_fp8_kernel<D, SB, false, E, MX><<<grid, 256, 0, stream>>>(p);
    }
  } else {
    if (causal) attn_fp8_varlen_kernel<D, SB, true, E, MX><<<grid, 256, 0, stream>>>(p);
    else attn_fp8_varlen_kernel<D, SB, false, E, MX><<<grid, 256, 0, stream>>>(p);
  }
}

// mx: 0 scales folded into the score scale (V's on the matrix core), 1
// power-of-two block scales on the matrix core, 2 the same per 32 channels
template <int D, int SB, class P>
static void launch_dc(const P& p, int causal, int exp_mode, int mx, dim3 grid, hipStream_t stream) {
  const int grp = mx == 2 ? 32 : 0;
  if (exp_mode == kExpSchraudolph) {
    if (mx) launch_dcem<D, SB, kExpSchraudolph, true>(p, causal, grp, grid, stream);
    else launch_dcem<D, SB, kExpSchraudolph, false>(p, causal, grp, grid, stream);
  } else {
    if (mx) launch_dcem<D, SB, kExpExact, true>(p, causal, grp, grid, stream);
    else launch_dcem<D, SB, kExpExact, false>(p, causal, grp, grid, stream);
  }
}

template <class P>
static void launch_any(const P& p, int D, int SB, int causal, int exp_mode, int mx, dim3 grid, hipStream_t stream) {
  if (D == 64 && SB == 64) launch_dc<64, 64>(p, causal, exp_mode, mx, grid, stream);
  else if (D == 64 && SB == 128) launch_dc<64, 128>(p, causal, exp_mode, mx, grid, stream);
  else if (D == 128 && SB == 64) launch_dc<128, 64>(p, causal, exp_mode, mx, grid, stream);
  else launch_dc<128, 128>(p, causal, exp_mode, mx, grid, stream);
}

hipError_t launch_attn_fp8(const AttnFp8Params& p, int D, int SB, int causal, int exp_mode, int mx, int BH,
                           hipStream_t stream) {
  launch_any(p, D, SB, causal, exp_mode, mx, dim3(BH * p.n_qtiles), stream);
  return hipGetLastError();
}

hipError_t launch_attn_fp8_varlen(const VarlenSchedParams& sp, const AttnFp8VarlenParams& p, int D, int SB, int causal,
                                  int exp_mode, int mx, int m_cap, hipStream_t stream) {
  hipError_t e = launch_varlen_schedule(sp, stream);
  if (e != hipSuccess) return e;
  launch_any(p, D, SB, causal, exp_mode, mx, dim3(p.H * m_cap), stream);
  return hipGetLastError();
}

}  // namespace attnfp8
