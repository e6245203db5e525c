// BF16 fused attention forward for gfx950: the 16-bit twin of the FP8 kernel.
//
// It runs the same running-softmax loop ("Fused attention kernel", Overview
// and Implementation sketch) on BF16 Q, K, V with v_mfma_f32_32x32x16_bf16,
// FP32 statistics and P in BF16, with no rotation and no quantisation.  It
// is the accuracy yardstick that the problem statement measures FP8 error
// against ("FP8 attention that keeps FlashAttention-3 throughput at
// BF16-level accuracy", What is asked).
//
// Same structure as the FP8 kernel: 4 waves x 32 queries, S^T = K Q^T so each
// lane owns one query, P^T in registers as the B operand of O^T += V^T P^T,
// V^T via ds_read_b64_tr_b16 from a row-major V tile, two-slot LDS ring fed
// by direct global->LDS loads, lazy rescale.  Key tile: 64 keys (a 16 KB tile
// at D = 128).
#include "common.h"
#include "attn_internal.h"

namespace attnfp8 {

constexpr float kTauBf16 = 8.0f;

template <int D>
struct Bf16Cfg {
  static constexpr int BC = 64;
  static constexpr int KSTEPS = D / 16;      // 32x32x16 K-steps of QK^T
  static constexpr int NSUB = BC / 32;
  static constexpr int NKG = BC / 16;        // 16-key steps of PV
  static constexpr int NDT = D / 32;
  static constexpr int ROWB = 2 * D;         // bytes per row
  static constexpr int SLOTS = ROWB / 16;
  static constexpr int TILE = BC * ROWB;
  static constexpr int CHUNKS = TILE / 1024;
  static constexpr int CHUNKS_PER_WAVE = CHUNKS / kWaves;
  static_assert(CHUNKS % kWaves == 0, "tile must split evenly over the waves");
};

// XOR swizzles of the 16-byte column slot per LDS row, for 64 banks of 4 bytes
// (256 bytes per bank cycle; a D = 128 row is one full cycle, a D = 64 row half
// of one).  They keep every slot inside its row, and the loader applies the
// same function, so a read of logical slot s at slot s ^ swz(row) finds it.
//   K (ds_read_b128, 16 lanes per cycle, one row per lane): any 16 consecutive
//     rows at one logical slot land in 16 distinct 16-byte bank groups.
//   V (ds_read_b64_tr_b16, 32 lanes per cycle: 4 consecutive rows x 4 slots of
//     one d-tile): the 4 rows' slot groups are disjoint.
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

template <int D, bool IS_V>
__device__ __forceinline__ void load_tile16(const uint16_t* __restrict__ src, uint8_t* buf, int kt, int N,
                                            int wave, int lane) {
  using C = Bf16Cfg<D>;
  const uint8_t* s8 = (const uint8_t*)src;
#pragma unroll
  for (int i = 0; i < C::CHUNKS_PER_WAVE; ++i) {
    const int c = wave * C::CHUNKS_PER_WAVE + i;
    const int pos = c * 1024 + lane * 16;
    const int prow = pos / C::ROWB;
    const int pslot = (pos % C::ROWB) / 16;
    const int lslot = pslot ^ (IS_V ? swz_v16<D>(prow) : swz_k16<D>(prow));
    int grow = kt * C::BC + prow;
    grow = grow < N ? grow : N - 1;
    global_to_lds16(s8 + (size_t)grow * C::ROWB + lslot * 16, buf + c * 1024);
  }
}

template <int D, bool CAUSAL>
struct Bf16Tile {
  using C = Bf16Cfg<D>;

  static __device__ __forceinline__ void run(const uint8_t* kbuf, const uint8_t* vbuf, int kt, int N, int lane,
                                             int iw, int my_q, const v4i (&qop)[C::KSTEPS], float c,
                                             v16f (&o)[C::NDT], float& m_ref, float& l_acc) {
    const int ql = lane & 31;
    const int h = lane >> 5;

    v16f s[C::NSUB];
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int row = sub * 32 + ql;
      const uint8_t* rp = kbuf + row * C::ROWB;
      const int sw = swz_k16<D>(row);
      v16f acc = {};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        v4i a = lds_read_b128(rp + 16 * ((2 * ks + h) ^ sw));
        acc = mfma_bf16(a, qop[ks], acc);
      }
      s[sub] = acc;
    }

    const int k0 = kt * C::BC;
    const bool need_mask = (k0 + C::BC > N) || (CAUSAL && k0 + C::BC - 1 > iw);
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

    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
    float tmax = mx * c;
    tmax = fmaxf(tmax, swap_halves(tmax));
    const bool upd = tmax > m_ref + kTauBf16;
    const float m_new = upd ? tmax : m_ref;
    const float alpha = upd ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
    m_ref = m_new;

    // P (bf16) as the B operand: per 16-key step, 8 keys per lane
    const float bias = -m_ref;
    float rs = 0.0f;
    v4i pop[C::NKG];
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int r = 8 * kg + 2 * a;
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][r], c, bias));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][r + 1], c, bias));
          rs += p0 + p1;
          pop[2 * sub + kg][a] = (int)pack_bf16x2(p0, p1);
        }
    l_acc = alpha * l_acc + rs;

    if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }

    // V^T operand: lane (d = l%32, half gh) needs V[key(j)][d] for j = 0..7 of each
    // 16-key step; two ds_read_b64_tr_b16, source lane i supplies key j = 4*rr + i/4
    // at columns d0 + 4*(i%4) .. +3.
    const int g = lane >> 4;
    const int i = lane & 15;
    const int gh = g >> 1;
    const int gd = g & 1;
#pragma unroll
    for (int kg = 0; kg < C::NKG; ++kg) {
      int rows[2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int j = 4 * rr + (i >> 2);
        rows[rr] = 16 * kg + 8 * (j >> 2) + 4 * gh + (j & 3);
      }
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const int col = 32 * dt + 16 * gd + 4 * (i & 3);   // first element
        const int slot = col / 8;                          // 16-byte column
        const int within = (col % 8) * 2;                  // byte offset inside it
        v2i part[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int row = rows[rr];
          part[rr] = lds_read_tr16(vbuf + row * C::ROWB + 16 * (slot ^ swz_v16<D>(row)) + within);
        }
        v4i a = {part[0][0], part[0][1], part[1][0], part[1][1]};
        o[dt] = mfma_bf16(a, pop[kg], o[dt]);
      }
    }
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnBf16Params p) {
  using C = Bf16Cfg<D>;
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
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int i0 = qt * kQueryTile;
  const int iw = i0 + wave * kQueriesPerWave;
  const int my_q = iw + (lane & 31);
  const int h = lane >> 5;

  const size_t head = (size_t)bh * N * D;
  const uint16_t* __restrict__ kh = p.k + head;
  const uint16_t* __restrict__ vh = p.v + head;

  v4i qop[C::KSTEPS];
  {
    const int qrow = my_q < N ? my_q : N - 1;
    const uint16_t* qp = p.q + head + (size_t)qrow * D;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qop[ks] = *(const v4i*)(qp + 16 * ks + 8 * h);
  }

  const int n_kt = (N + C::BC - 1) / C::BC;
  int n_kt_wg = n_kt;
  int kt_w = n_kt - 1;
  if (CAUSAL) {
    const int last_wg = (i0 + kQueryTile - 1 < N - 1) ? i0 + kQueryTile - 1 : N - 1;
    n_kt_wg = last_wg / C::BC + 1;
    const int last_w = (iw + kQueriesPerWave - 1 < N - 1) ? iw + kQueriesPerWave - 1 : N - 1;
    kt_w = last_w / C::BC;
  }

  v16f o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] = (v16f){};
  float m_ref = -1e30f;
  float l_acc = 0.0f;

  load_tile16<D, false>(kh, kbuf0, 0, N, wave, lane);
  load_tile16<D, true>(vh, vbuf0, 0, N, wave, lane);

  for (int kt = 0; kt < n_kt_wg; kt += 2) {
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < n_kt_wg) {
      load_tile16<D, false>(kh, kbuf1, kt + 1, N, wave, lane);
      load_tile16<D, true>(vh, vbuf1, kt + 1, N, wave, lane);
    }
    if (kt <= kt_w)
      Bf16Tile<D, CAUSAL>::run(kbuf0, vbuf0, kt, N, lane, iw, my_q, qop, p.score_scale, o, m_ref, l_acc);
    if (kt + 1 >= n_kt_wg) break;
    wait_vmem_all();
    __syncthreads();
    if (kt + 2 < n_kt_wg) {
      load_tile16<D, false>(kh, kbuf0, kt + 2, N, wave, lane);
      load_tile16<D, true>(vh, vbuf0, kt + 2, N, wave, lane);
    }
    if (kt + 1 <= kt_w)
      Bf16Tile<D, CAUSAL>::run(kbuf1, vbuf1, kt + 1, N, lane, iw, my_q, qop, p.score_scale, o, m_ref, l_acc);
  }

  const float l_tot = l_acc + swap_halves(l_acc);
  const float inv_l = 1.0f / l_tot;
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
