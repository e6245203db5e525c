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
// gfx950 design (one workgroup = 4 waves = 128 queries of one head):
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
//   * K_j / V_j tiles (BC keys = one scale block) stream into a two-slot LDS
//     ring by direct global->LDS 16-byte loads, the next tile in flight while
//     the current one is consumed; 16-byte columns are XOR-swizzled per row
//     against LDS bank conflicts.
//   * Scale folding: t = s * (dq * dk_j * score_scale) in log2 units, one FMA
//     per score with the running max; V's block scale dv_j enters as the
//     factor r_j = dv_j / (max dv over the tiles the wave visits) inside the
//     exponent (so P stays <= 256),
//     and the row sum divides it back out.
//   * Lazy rescale: the reference max only moves when a tile's max exceeds it
//     by more than kTau (log2 units), so most tiles skip the O rescale; P is
//     then <= 2^kTau, inside e4m3's range.
//   * Causal: key tiles past the workgroup's last query are not loaded, tiles
//     past a wave's last query are not computed, masks only on diagonal and
//     tail tiles; query tiles are scheduled longest first.
#include "common.h"
#include "attn_internal.h"

namespace attnfp8 {

constexpr float kTau = 8.0f;   // lazy-rescale threshold (log2 units): P <= 2^8

template <int D, int BC>
struct Fp8Cfg {
  static constexpr int KSTEPS = D / 64;      // K-steps of the QK^T contraction
  static constexpr int NSUB = BC / 32;       // 32-key subtiles of S^T
  static constexpr int NKH = BC / 64;        // 64-key steps of the PV contraction
  static constexpr int NDT = D / 32;         // 32-row (d) tiles of O^T
  static constexpr int SLOTS = D / 16;       // 16-byte columns per row
  static constexpr int TILE = BC * D;        // bytes per K or V tile
  static constexpr int CHUNKS = TILE / 1024; // 1 KiB direct-load chunks per tile
  static constexpr int CHUNKS_PER_WAVE = CHUNKS / kWaves;
  static_assert(CHUNKS % kWaves == 0, "tile must split evenly over the waves");
};

// XOR swizzles of the 16-byte column index, per LDS row
template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (D / 16 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return (row & 3) | ((row >> 1) & 4);
  else return row & 3;
}

// Issue this wave's share of one K or V tile (rows kt*BC ..) into `buf`.
template <int D, int BC, bool IS_V>
__device__ __forceinline__ void load_tile(const uint8_t* __restrict__ src, uint8_t* buf, int kt, int N,
                                          int wave, int lane) {
  using C = Fp8Cfg<D, BC>;
#pragma unroll
  for (int i = 0; i < C::CHUNKS_PER_WAVE; ++i) {
    const int c = wave * C::CHUNKS_PER_WAVE + i;
    const int pos = c * 1024 + lane * 16;
    const int prow = pos / D;
    const int pslot = (pos % D) / 16;
    const int lslot = pslot ^ (IS_V ? swz_v<D>(prow) : swz_k<D>(prow));
    int grow = kt * BC + prow;
    grow = grow < N ? grow : N - 1;
    global_to_lds16(src + (size_t)grow * D + lslot * 16, buf + c * 1024);
  }
}

template <int D, int BC, bool CAUSAL>
struct Fp8Tile {
  using C = Fp8Cfg<D, BC>;

  // one key tile: S^T, softmax update, O^T += V^T P^T
  static __device__ __forceinline__ void run(const uint8_t* kbuf, const uint8_t* vbuf, int kt, int N,
                                             int lane, int iw, int my_q, const v8i (&qop)[C::KSTEPS],
                                             float c_q, float dk, float inv_rv, float log2_rv,
                                             v16f (&o)[C::NDT], float& m_ref, float& l_acc) {
    const int ql = lane & 31;
    const int h = lane >> 5;

    // ---- S^T = K_j Q^T  (32 keys x 32 queries per subtile)
    v16f s[C::NSUB];
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int row = sub * 32 + ql;
      const uint8_t* rp = kbuf + row * D;
      const int sw = swz_k<D>(row);
      v16f acc = {};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        const int s0 = 4 * ks + 2 * h;
        v4i lo = lds_read_b128(rp + 16 * (s0 ^ sw));
        v4i hi = lds_read_b128(rp + 16 * ((s0 + 1) ^ sw));
        v8i a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc = mfma_f8(a, qop[ks], acc);
      }
      s[sub] = acc;
    }

    // ---- masks (causal diagonal tiles, ragged last tile)
    const int k0 = kt * BC;
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > iw);
    if (need_mask) {
      const int lim = CAUSAL ? (my_q < N - 1 ? my_q : N - 1) : N - 1;
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + sub * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > lim) s[sub][r] = -INFINITY;
        }
    }

    // ---- tile max in log2 units (c > 0, so max commutes with the scale)
    const float c = c_q * dk;
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
    float tmax = mx * c;
    tmax = fmaxf(tmax, swap_halves(tmax));

    // ---- lazy reference-max update
    const bool upd = tmax > m_ref + kTau;
    const float m_new = upd ? tmax : m_ref;
    const float alpha = upd ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
    m_ref = m_new;

    // ---- P = 2^(t - m + log2 r_j), row sum, e4m3 packing (B operand layout)
    const float bias = log2_rv - m_ref;
    float rs = 0.0f;
    v8i pop[C::NKH];
#pragma unroll
    for (int kh = 0; kh < C::NKH; ++kh) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int sub = 2 * kh + s2;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][4 * a + 0], c, bias));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][4 * a + 1], c, bias));
          float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][4 * a + 2], c, bias));
          float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][4 * a + 3], c, bias));
          rs += (p0 + p1) + (p2 + p3);
          int w = cvt_pk_fp8<false>(p0, p1, 0);
          w = cvt_pk_fp8<true>(p2, p3, w);
          pop[kh][4 * s2 + a] = w;
        }
      }
    }
    l_acc = alpha * l_acc + rs * inv_rv;

    // ---- rescale O only when some lane moved its reference max
    if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }

    // ---- O^T += V_j^T P^T ; V^T operand via transposing LDS reads
    const int g = lane >> 4;          // 16-lane group
    const int i = lane & 15;
    const int gh = g >> 1;            // k-chunk of this lane (== h)
    const int gd = g & 1;             // which 16 d-rows of the 32
#pragma unroll
    for (int kh = 0; kh < C::NKH; ++kh) {
      int rows[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = i >> 1;                          // key byte this source lane supplies
        const int j = 8 * rr + t;                       // byte index in the 32-byte operand
        rows[rr] = 64 * kh + 8 * (j >> 2) + 4 * gh + (j & 3);
      }
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const int slot = 2 * dt + gd;
        v2i part[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = rows[rr];
          part[rr] = lds_read_tr8(vbuf + row * D + 16 * (slot ^ swz_v<D>(row)) + 8 * (i & 1));
        }
        v8i a = {part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
        o[dt] = mfma_f8(a, pop[kh], o[dt]);
      }
    }
  }
};

template <int D, int BC, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(AttnFp8Params p) {
  using C = Fp8Cfg<D, BC>;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / p.n_qtiles;
  int qt = logical % p.n_qtiles;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;            // longest tiles first
  const int i0 = qt * kQueryTile;
  const int iw = i0 + wave * kQueriesPerWave;
  const int my_q = iw + (lane & 31);
  const int h = lane >> 5;

  const size_t head = (size_t)bh * N * D;
  const uint8_t* __restrict__ kh8 = p.k8 + head;
  const uint8_t* __restrict__ vh8 = p.v8 + head;
  const float* kd = p.kd + (size_t)bh * p.nblk;
  const float* vd = p.vd + (size_t)bh * p.nblk;

  // queries of this lane as the B operand: Q[q][64ks + 32h .. +31]
  v8i qop[C::KSTEPS];
  {
    const int qrow = my_q < N ? my_q : N - 1;
    const uint8_t* qp = p.q8 + head + (size_t)qrow * D;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      v4i lo = *(const v4i*)(qp + 64 * ks + 32 * h);
      v4i hi = *(const v4i*)(qp + 64 * ks + 32 * h + 16);
      qop[ks] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  const int qblk = (my_q < N ? my_q : N - 1) / BC;
  const float c_q = p.qd[(size_t)bh * p.nblk + qblk] * p.score_scale;

  const int n_kt = (N + BC - 1) / BC;
  int n_kt_wg = n_kt;
  int kt_w = n_kt - 1;
  if (CAUSAL) {
    const int last_wg = (i0 + kQueryTile - 1 < N - 1) ? i0 + kQueryTile - 1 : N - 1;
    n_kt_wg = last_wg / BC + 1;
    const int last_w = (iw + kQueriesPerWave - 1 < N - 1) ? iw + kQueriesPerWave - 1 : N - 1;
    kt_w = last_w / BC;
  }

  // largest V block scale over the key tiles this wave visits (for causal calls
  // only blocks up to the wave's own, so no output depends on a later block)
  float dvm = 0.0f;
  for (int b = lane; b <= kt_w; b += 64) dvm = fmaxf(dvm, vd[b]);
  dvm = wave_max(dvm);

  v16f o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] = (v16f){};
  float m_ref = -1e30f;
  float l_acc = 0.0f;

  load_tile<D, BC, false>(kh8, kbuf0, 0, N, wave, lane);
  load_tile<D, BC, true>(vh8, vbuf0, 0, N, wave, lane);

  for (int kt = 0; kt < n_kt_wg; kt += 2) {
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < n_kt_wg) {
      load_tile<D, BC, false>(kh8, kbuf1, kt + 1, N, wave, lane);
      load_tile<D, BC, true>(vh8, vbuf1, kt + 1, N, wave, lane);
    }
    if (kt <= kt_w) {
      const float dv = vd[kt];
      Fp8Tile<D, BC, CAUSAL>::run(kbuf0, vbuf0, kt, N, lane, iw, my_q, qop, c_q, kd[kt], dvm / dv,
                                  __builtin_amdgcn_logf(dv / dvm), o, m_ref, l_acc);
    }
    if (kt + 1 >= n_kt_wg) break;
    wait_vmem_all();
    __syncthreads();
    if (kt + 2 < n_kt_wg) {
      load_tile<D, BC, false>(kh8, kbuf0, kt + 2, N, wave, lane);
      load_tile<D, BC, true>(vh8, vbuf0, kt + 2, N, wave, lane);
    }
    if (kt + 1 <= kt_w) {
      const float dv = vd[kt + 1];
      Fp8Tile<D, BC, CAUSAL>::run(kbuf1, vbuf1, kt + 1, N, lane, iw, my_q, qop, c_q, kd[kt + 1], dvm / dv,
                                  __builtin_amdgcn_logf(dv / dvm), o, m_ref, l_acc);
    }
  }

  // ---- epilogue: O = dvm * O_acc / l ; LSE = ln 2 * (m + log2 l)
  const float l_tot = l_acc + swap_halves(l_acc);
  const float inv_l = dvm / l_tot;
  if (my_q < N) {
    uint16_t* orow = p.o + head + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * dt + 8 * a + 4 * h;
        uint32_t w0 = pack_bf16x2(o[dt][4 * a + 0] * inv_l, o[dt][4 * a + 1] * inv_l);
        uint32_t w1 = pack_bf16x2(o[dt][4 * a + 2] * inv_l, o[dt][4 * a + 3] * inv_l);
        *(v2i*)(orow + d) = (v2i){(int)w0, (int)w1};
      }
    if (h == 0) p.lse[(size_t)bh * N + my_q] = kLn2 * (m_ref + __builtin_amdgcn_logf(l_tot));
  }
}

#define FP8_INST(D, BC, CA) template __global__ void attn_fp8_kernel<D, BC, CA>(AttnFp8Params);
FP8_INST(64, 64, false)
FP8_INST(64, 64, true)
FP8_INST(64, 128, false)
FP8_INST(64, 128, true)
FP8_INST(128, 64, false)
FP8_INST(128, 64, true)
FP8_INST(128, 128, false)
FP8_INST(128, 128, true)

template <int D, int BC>
static void launch_dc(const AttnFp8Params& p, int causal, dim3 grid, hipStream_t stream) {
  if (causal) attn_fp8_kernel<D, BC, true><<<grid, 256, 0, stream>>>(p);
  else attn_fp8_kernel<D, BC, false><<<grid, 256, 0, stream>>>(p);
}

hipError_t launch_attn_fp8(const AttnFp8Params& p, int D, int SB, int causal, int BH, hipStream_t stream) {
  dim3 grid(BH * p.n_qtiles);
  if (D == 64 && SB == 64) launch_dc<64, 64>(p, causal, grid, stream);
  else if (D == 64 && SB == 128) launch_dc<64, 128>(p, causal, grid, stream);
  else if (D == 128 && SB == 64) launch_dc<128, 64>(p, causal, grid, stream);
  else launch_dc<128, 128>(p, causal, grid, stream);
  return hipGetLastError();
}

}  // namespace attnfp8
