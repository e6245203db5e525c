// Decode over an FP8 K/V cache (gfx950).
//
// "FP8 attention that keeps FlashAttention-3 throughput at BF16-level
// accuracy", Realistic applications: storing K and V in FP8 relieves the
// bandwidth of the KV cache.  A decode step reads every cached K and V byte
// once for a handful of query rows (the Sq new tokens of the G query heads
// that share one K/V head), so it is bound by HBM, not by the matrix cores:
// at MQ = G * Sq <= 32 rows it does 4 * D * MQ FLOP per 2 * D bytes, a tenth
// of the FP8 MFMA's FLOP-per-byte balance on MI355X.  The design therefore
// goes for bytes in flight and full occupancy rather than for MFMA rate:
//
//   attn_fp8_decode_kernel: grid (B * Hkv, splits), 4 waves per workgroup.
//     Wave w of split x owns the keys [(4 x + w) split, +split) of its
//     sequence and runs the running-softmax loop of the dense kernel on them
//     for all MQ rows (one 32-query MFMA column block; rows past MQ repeat
//     row 0 and are dropped): K tiles go straight from HBM into the MFMA A
//     layout (16-byte buffer loads; rows past the sequence read as zeros), V
//     tiles straight into one of two 8 KiB LDS buffers of the wave (buffer
//     loads that write LDS) so that the transpose read (ds_read_b64_tr_b8)
//     can feed O^T += V^T P^T.  Tile t+1's loads are in flight while tile t
//     is computed; no workgroup barrier inside the loop: every wave streams
//     on its own.  At the end the four waves merge in LDS by their
//     log-sum-exp, in wave order, and write one partial (m, l, O
//     unnormalised) per split.  The split index is the slow grid dimension:
//     lengths are known on the device only, so the grid covers the cache
//     capacity, and the splits past the shorter sequences' ends, dispatched
//     last, leave at once.
//   attn_fp8_decode_combine: one wave per output row merges the splits
//     (M = max m, w = 2^(m - M), O = sum w O / sum w l), writes O in BF16 and
//     LSE = ln 2 (M + log2 l).  Maxima and weights are taken one split per
//     lane; the O rows are then read with independent loads (no chain of
//     dependent round trips through the splits).
//
// Numerics per key range are those of the dense kernel (scale folds, lazy
// reference, P = e4m3(2^(t - m)), V's power-of-two block scale applied inside
// the matrix core, FP32 statistics).
#include "common.h"
#include "attn_internal.h"
#include "fp8_tiles.h"

namespace attnfp8 {

// The running-softmax loop of one wave over the keys [k0, k1) of sequence b
// (length L) and K/V head hk, for all MQ query rows: O unnormalised, the
// reference maximum m and this lane's half of the row sum l.  vbuf0: the
// wave's two V tile buffers in LDS.
template <int D>
struct DecodeState {
  v16f o[Fp8Cfg<D>::NDT];
  float m_ref;
  float l_acc;
};

template <int D, int SB, bool CAUSAL>
__device__ __forceinline__ void decode_range(const DecodeParams& p, int b, int hk, int L, int k0, int k1,
                                             uint8_t* vbuf0, DecodeState<D>& st) {
  using C = Fp8Cfg<D>;
  static_assert(SB % kBC == 0, "a key tile lies in one scale block");
  const int lane = threadIdx.x & 63;
  const int ql = lane & 31;
  const int h = lane >> 5;
  const int bk = b * p.Hkv + hk;

  // this lane's query row: r = g * Sq + i (query head hk * G + g, new token i)
  const int r = ql < p.MQ ? ql : 0;
  const int g = r / p.Sq;
  const int i = r - g * p.Sq;
  const int hq = hk * p.G + g;
  const size_t qrow = ((size_t)b * p.Hq + hq) * p.Sq + i;
  v8i qop[C::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) {
    const v4i lo4 = *(const v4i*)(p.q8 + qrow * D + op_channel(ks, h, 0));
    const v4i hi4 = *(const v4i*)(p.q8 + qrow * D + op_channel(ks, h, 1));
    qop[ks] = (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  }
  const float c_q = p.qd[(size_t)b * p.Hq + hq] * p.score_scale;
  const int qpos = L - p.Sq + i;               // position of this query in its sequence

  const size_t kvh = (size_t)bk * p.Ncap * D;
  const cfloat* kd = (const cfloat*)(p.kd + (size_t)bk * p.nblk);
  const cfloat* vd = (const cfloat*)(p.vd + (size_t)bk * p.nblk);   // (scalar loads in the loop)
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k8 + kvh), 0, L * D, 0x00020000);
  const uint32_t vlds = lds_addr_of(vbuf0);
  const v4i rsv = make_rsrc(p.v8 + kvh, (uint32_t)(L * D));
  // buffer offset of the 16 bytes lane l moves into LDS chunk j: LDS (row,
  // column slot c) holds source (row, c ^ swz_v(row)), as the transpose reads expect
  int voff[C::CHUNKS];
#pragma unroll
  for (int j = 0; j < C::CHUNKS; ++j) {
    const int pos = j * 1024 + lane * 16;
    const int prow = pos / D;
    voff[j] = prow * D + 16 * (((pos % D) / 16) ^ swz_v<D>(prow));
  }
  // K of a tile straight into the MFMA A layout (compiler-tracked buffer
  // loads; rows past the sequence read as zeros), V into one of the wave's
  // LDS buffers (buffer loads that write LDS, inline assembly: no registers)
  KOps<D> kc;
  auto load_k = [&](int t) {
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
        for (int half = 0; half < 2; ++half)
          kc.r[sub][ks][half] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, (t + sub * 32 + ql) * D + op_channel(ks, h, half),
                                                         0, 0));
  };
  auto load_v = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < C::CHUNKS; ++j) buffer_to_lds16(rsv, t * D + voff[j], vlds + buf * C::TILE + j * 1024);
  };
  if (k0 < k1) {
    load_k(k0);
    load_v(k0, 0);
  }

  const Fp8LaneOffsets<D> lo(lane);
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) st.o[dt] = (v16f){};
  st.m_ref = -1e30f;
  st.l_acc = 0.0f;
  v8i pop = (v8i){};

  // Per tile t: one wait (tile t resident, and every transpose read of the
  // other V buffer done), then V of tile t+1 into that buffer; the score
  // products of tile t, then K of tile t+1 into the registers they have just
  // read; then the softmax and the P V products of tile t.  A tile's loads
  // thus overlap the whole previous tile, and no workgroup barrier is needed:
  // every wave streams on its own.
  for (int t = k0; t < k1; t += kBC) {
    // the builtin wait (vmcnt(0) lgkmcnt(0)) is seen by the compiler's own
    // wait bookkeeping; the empty asm keeps memory operations on their side
    __builtin_amdgcn_s_waitcnt(0x0070);
    __asm__ volatile("" ::: "memory");
    const int par = ((t - k0) / kBC) & 1;
    if (t + kBC < k1) load_v(t + kBC, par ^ 1);
    const uint8_t* vcur = vbuf0 + par * C::TILE;
    // S^T = K Q^T
    STile<D> s;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) s[sub] = qk_mfma<D, false>(kc, qop, sub, KsScales<D>{}, KsScales<D>{});
    if (t + kBC < k1) load_k(t + kBC);
    const int blk = t / SB;
    const float c = c_q * kd[blk];
    // keys past the range, and (causal) past this query's position
    if (t + kBC > k1 || (CAUSAL && t + kBC - 1 > L - p.Sq)) {
      const int lim = (CAUSAL ? (qpos < k1 - 1 ? qpos : k1 - 1) : k1 - 1) - t - 4 * h;
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (sub * 32 + 8 * (rr >> 2) + (rr & 3) > lim) s[sub][rr] = -INFINITY;
    }
    // statistics: lazy reference max
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[sub][rr]);
    float tmax = mx * c;
    tmax = fmaxf(tmax, swap_halves(tmax));
    const bool upd = tmax > st.m_ref + kTau;
    const float m_new = upd ? tmax - kLift : st.m_ref;
    const float alpha = upd ? __builtin_amdgcn_exp2f(st.m_ref - m_new) : 1.0f;
    st.m_ref = m_new;
    if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) st.o[dt][rr] *= alpha;
    }
    // P = 2^(t - m) in e4m3 (B operand of the P V product) and its row sum;
    // V's power-of-two block scale is applied inside the matrix core
    const int sv = e8m0_of(vd[blk]);
    const ExpArgs<kExpExact> ex(c, -st.m_ref);
    float rs = 0.0f;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float p0 = ex(s[sub][4 * a + 0]);
        const float p1 = ex(s[sub][4 * a + 1]);
        const float p2 = ex(s[sub][4 * a + 2]);
        const float p3 = ex(s[sub][4 * a + 3]);
        rs += (p0 + p1) + (p2 + p3);
        int w = cvt_pk_fp8<false>(p0, p1, pop[4 * sub + a]);
        w = cvt_pk_fp8<true>(p2, p3, w);
        pop[4 * sub + a] = w;
      }
    st.l_acc = alpha * st.l_acc + rs;
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      v2i part[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part[rr] = lds_read_tr8(vcur + 16 * rr * D + lo.v[dt]);
      const v8i av = {part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
      st.o[dt] = mfma_f8x<true>(av, pop, st.o[dt], sv, 127);
    }
  }
}

template <int D, int SB, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fp8_decode_kernel(DecodeParams p) {
  using C = Fp8Cfg<D>;
  // two V buffers per wave during the loop, the merge after it (dynamic
  // size: decode_lds_bytes)
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31;
  const int h = lane >> 5;
  // (the split index is the slow grid dimension: every sequence's first
  // splits are dispatched before any later ones, so the splits past the
  // shorter sequences' ends come last and leave while the others finish)
  const int bk = blockIdx.x;                   // batch * Hkv + K/V head
  const int xs = blockIdx.y;                   // split
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  int L = p.seqlens[b];
  L = L < 0 ? 0 : (L > p.Ncap ? p.Ncap : L);
  // splits past the sequence's end hold no key: nothing to write (the merge
  // reads only the splits below ceil(L / (4 split)))
  if (xs * kWaves * p.split >= L) return;
  const int k0 = (xs * kWaves + wave) * p.split;
  const int k1 = L < k0 + p.split ? L : k0 + p.split;
  DecodeState<D> st;
  decode_range<D, SB, CAUSAL>(p, b, hk, L, k0, k1, smem + wave * 2 * C::TILE, st);
  const float m_ref = st.m_ref;
  const v16f (&o)[C::NDT] = st.o;
  const float l_acc = st.l_acc;

  // ---- merge the four waves by their log-sum-exp: waves 1..3 write their
  // rows, scaled to the common maximum, into slabs of their own; wave 0 adds
  // them to its own rows in wave order and writes the split's partial
  const float l_tot = l_acc + swap_halves(l_acc);
  __syncthreads();                                   // every wave is done with its V buffer
  float* mm = (float*)smem;                          // [4][32] reference max of each wave
  float* ml = mm + kWaves * 32;                      // [4][32] row sum of each wave
  float* slab = ml + kWaves * 32;                    // [3][MQ][D] scaled O of waves 1..3
  if (h == 0) {
    mm[wave * 32 + ql] = m_ref;
    ml[wave * 32 + ql] = l_tot;
  }
  __syncthreads();
  float M = mm[ql];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mm[w * 32 + ql]);
  const float f = __builtin_amdgcn_exp2f(m_ref - M);
  if (wave > 0 && ql < p.MQ) {
    float* mine = slab + ((size_t)(wave - 1) * p.MQ + ql) * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(v4f*)(mine + 32 * dt + 8 * a + 4 * h) =
            (v4f){f * o[dt][4 * a + 0], f * o[dt][4 * a + 1], f * o[dt][4 * a + 2], f * o[dt][4 * a + 3]};
  }
  __syncthreads();
  if (wave == 0) {
    const size_t part = (size_t)bk * p.nsplit + xs;
    if (ql < p.MQ) {
      float* po = p.part_o + (part * p.MQ + ql) * D;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * dt + 8 * a + 4 * h;
          v4f acc = {f * o[dt][4 * a + 0], f * o[dt][4 * a + 1], f * o[dt][4 * a + 2], f * o[dt][4 * a + 3]};
#pragma unroll
          for (int w = 1; w < kWaves; ++w) {
            const v4f x = *(const v4f*)(slab + ((size_t)(w - 1) * p.MQ + ql) * D + d);
            acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
          }
          *(v4f*)(po + d) = acc;
        }
      if (h == 0) {
        float Lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Lsum += __builtin_amdgcn_exp2f(mm[w * 32 + ql] - M) * ml[w * 32 + ql];
        p.part_m[part * p.MQ + ql] = M;
        p.part_l[part * p.MQ + ql] = Lsum;
      }
    }
  }
}

// Tiles of kBC keys per sequence over the batch (B <= 64 * kMaxSeqPerLane),
// spread over the lanes of a wave: lane j holds sequences [per j, per j + per)
// and the number of tiles of the sequences before them (one K/V head).  One
// round of independent loads of the lengths, then a scan over the lanes.
constexpr int kMaxSeqPerLane = 8;

struct BatchTiles {
  int per;
  int nt[kMaxSeqPerLane];
  int before;      // tiles of the sequences before this lane's
  int total;       // tiles of the whole batch (one K/V head)

  __device__ __forceinline__ BatchTiles(const int* seqlens, int B, int Ncap) {
    const int lane = threadIdx.x & 63;
    per = (B + 63) / 64;
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxSeqPerLane; ++i) {
      const int b = lane * per + i;
      int L = (i < per && b < B) ? seqlens[b] : 0;
      L = L < 0 ? 0 : (L > Ncap ? Ncap : L);
      nt[i] = (L + kBC - 1) / kBC;
      sum += nt[i];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d, 64);
      if (lane >= d) incl += u;
    }
    before = incl - sum;
    total = __builtin_amdgcn_readlane(incl, 63);
  }
  // tiles of sequence b, and of the sequences before it (wave-uniform b)
  __device__ __forceinline__ void of(int b, int& nt_b, int& before_b) const {
    const int j = b / per;
    int acc = __builtin_amdgcn_readlane(before, j);
    int n = 0;
#pragma unroll
    for (int i = 0; i < kMaxSeqPerLane; ++i) {
      const int v = __builtin_amdgcn_readlane(nt[i], j);
      if (i < b - j * per) acc += v;
      if (i == b - j * per) n = v;
    }
    nt_b = n;
    before_b = acc;
  }
  // the (sequence, K/V head, tile) of flat tile x < Hkv * total; the flat
  // order is sequence, then K/V head, then tile
  __device__ __forceinline__ void locate(long long x, int Hkv, int& b, int& hk, int& tile) const {
    const unsigned long long mask = __builtin_amdgcn_ballot_w64((long long)Hkv * before <= x);
    const int j = 63 - __builtin_clzll(mask);            // lane 0 always qualifies
    long long rem = x - (long long)Hkv * __builtin_amdgcn_readlane(before, j);
    long long frem = 0;
    int fn = 1;
    b = j * per;
#pragma unroll
    for (int i = 0; i < kMaxSeqPerLane; ++i) {
      const int n = __builtin_amdgcn_readlane(nt[i], j);
      const long long seg = (long long)Hkv * n;
      if (rem >= 0 && i < per) {
        if (rem < seg) {
          b = j * per + i;
          frem = rem;
          fn = n;
        }
        rem -= seg;
      }
    }
    hk = (int)(frem / fn);
    tile = (int)(frem - (long long)hk * fn);
  }
};

// The wave whose share of the flat tile range holds tile x (shares are
// [floor(w T / W), floor((w + 1) T / W))): the largest w with
// floor(w T / W) <= x, i.e. ceil((x + 1) W / T) - 1.
__device__ __forceinline__ int wave_of_tile(long long x, long long T, int W) {
  return (int)(((x + 1) * W + T - 1) / T) - 1;
}

// Partial (m, l, O unnormalised) of one wave's piece for the MQ rows.
template <int D>
__device__ __forceinline__ void write_partial(const DecodeParams& p, size_t slot, const DecodeState<D>& st) {
  const int lane = threadIdx.x & 63;
  const int ql = lane & 31;
  const int h = lane >> 5;
  const float l_tot = st.l_acc + swap_halves(st.l_acc);
  if (ql < p.MQ) {
    float* po = p.part_o + (slot * p.MQ + ql) * D;
#pragma unroll
    for (int dt = 0; dt < Fp8Cfg<D>::NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(v4f*)(po + 32 * dt + 8 * a + 4 * h) =
            (v4f){st.o[dt][4 * a + 0], st.o[dt][4 * a + 1], st.o[dt][4 * a + 2], st.o[dt][4 * a + 3]};
    if (h == 0) {
      p.part_m[slot * p.MQ + ql] = st.m_ref;
      p.part_l[slot * p.MQ + ql] = l_tot;
    }
  }
}

// Balanced schedule: the tiles of every (sequence, K/V head) in one flat
// order, cut into W equal shares, one per wave (W = 4 x the grid, or the
// number of tiles T if that is smaller).  A share
// may span several (sequence, K/V head) segments: each piece runs the loop on
// its own and writes its partial to slot w + s (s = b Hkv + hk).  Along the
// shares, w and s never decrease, so w + s is distinct for every piece and
// the pieces of one segment sit in consecutive slots.
template <int D, int SB, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fp8_decode_balanced_kernel(DecodeParams p) {
  using C = Fp8Cfg<D>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * kWaves + wave;
  const BatchTiles bt(p.seqlens, p.B, p.Ncap);
  const long long T = (long long)p.Hkv * bt.total;
  // (no more shares than tiles: every share then holds a tile, so the slots
  // of a segment's pieces are consecutive with no unwritten one between)
  const int W = T < p.nwave ? (int)T : p.nwave;
  if (w >= W) return;
  long long x = T * w / W;
  const long long x1 = T * (w + 1) / W;
  int b, hk, tile;
  bt.locate(x, p.Hkv, b, hk, tile);
  int nt, dummy;
  bt.of(b, nt, dummy);
  for (;;) {
    // (all of it is wave-uniform; said so, so that the buffer descriptors
    // built from it stay in scalar registers)
    b = __builtin_amdgcn_readfirstlane(b);
    hk = __builtin_amdgcn_readfirstlane(hk);
    tile = __builtin_amdgcn_readfirstlane(tile);
    nt = __builtin_amdgcn_readfirstlane(nt);
    int L = __builtin_amdgcn_readfirstlane(p.seqlens[b]);
    L = L < 0 ? 0 : (L > p.Ncap ? p.Ncap : L);
    const long long left = x1 - x;
    const int n = left < (long long)(nt - tile) ? (int)left : nt - tile;
    const int k0 = tile * kBC;
    const int k1 = L < (tile + n) * kBC ? L : (tile + n) * kBC;
    DecodeState<D> st;
    decode_range<D, SB, CAUSAL>(p, b, hk, L, k0, k1, smem + wave * 2 * C::TILE, st);
    write_partial<D>(p, (size_t)w + (size_t)b * p.Hkv + hk, st);
    x += n;
    if (x >= x1) break;
    // the next segment that holds a tile (one exists: x < x1 <= T)
    tile = 0;
    if (++hk == p.Hkv) {
      hk = 0;
      do {
        if (++b >= p.B) return;
        bt.of(b, nt, dummy);
      } while (nt == 0);
    }
  }
}

// Partials the merge loads in one round trip.
constexpr int kCombineBatch = 32;

template <int D>
__global__ __launch_bounds__(256) void attn_fp8_decode_combine(DecodeParams p) {
  constexpr int PER = D / 64;                        // channels per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= p.B * p.Hkv * p.MQ) return;             // (no barrier in this kernel)
  const int bk = row / p.MQ;
  const int r = row - bk * p.MQ;
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  const int g = r / p.Sq;
  const int i = r - g * p.Sq;
  size_t base;
  int nx;                                            // partials that hold keys
  if (p.nwave > 0) {
    // balanced schedule: the waves whose shares meet this segment's tiles
    const BatchTiles bt(p.seqlens, p.B, p.Ncap);
    int nt_b, before_b;
    bt.of(b, nt_b, before_b);
    const long long T = (long long)p.Hkv * bt.total;
    const long long x0 = (long long)p.Hkv * before_b + (long long)hk * nt_b;
    nx = 0;
    base = 0;
    if (nt_b > 0) {
      const int W = T < p.nwave ? (int)T : p.nwave;
      const int wf = wave_of_tile(x0, T, W);
      const int wl = wave_of_tile(x0 + nt_b - 1, T, W);
      base = (size_t)wf + bk;
      nx = wl - wf + 1;
    }
  } else {
    base = (size_t)bk * p.nsplit;
    int L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.Ncap ? p.Ncap : L);
    nx = (L + kWaves * p.split - 1) / (kWaves * p.split);
  }
  // kCombineBatch partials at a time: every load of a batch (this lane's (m, l)
  // for partial x0 + lane, and the O rows of all the batch's partials) goes
  // out before any arithmetic needs one, so a batch costs one round trip;
  // the batches merge with a running maximum.
  float M = -INFINITY;
  float lsum = 0.0f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int x0 = 0; x0 < nx; x0 += kCombineBatch) {
    const int n = nx - x0 < kCombineBatch ? nx - x0 : kCombineBatch;
    float mi = -INFINITY, li = 0.0f;
    if (lane < n) {
      mi = p.part_m[(base + x0 + lane) * p.MQ + r];
      li = p.part_l[(base + x0 + lane) * p.MQ + r];
    }
    float vals[kCombineBatch][PER];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const size_t x = base + x0 + (u < n ? u : n - 1);      // (past the batch: a repeat, weight 0)
#pragma unroll
      for (int e = 0; e < PER; ++e) vals[u][e] = p.part_o[(x * p.MQ + r) * D + lane + 64 * e];
    }
    const float Mn = fmaxf(M, wave_max(mi));
    const float f = __builtin_amdgcn_exp2f(M - Mn);          // 0 on the first batch
    lsum *= f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= f;
    const float w = lane < n ? __builtin_amdgcn_exp2f(mi - Mn) : 0.0f;
    lsum += w * li;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += wu * vals[u][e];
    }
    M = Mn;
  }
  // row sum over the lanes
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) lsum += __shfl_xor(lsum, m, 64);
  lsum += swap_halves(lsum);
  const size_t orow = ((size_t)b * p.Hq + hk * p.G + g) * p.Sq + i;
  const float inv_l = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const __bf16 v = (__bf16)(acc[e] * inv_l);
    p.o[orow * D + lane + 64 * e] = __builtin_bit_cast(uint16_t, v);
  }
  if (lane == 0) p.lse[orow] = kLn2 * (M + __builtin_amdgcn_logf(lsum));
}

// LDS of the split kernel: the eight V buffers, or the merge's maxima, sums
// and three slabs, whichever is larger (at most 64 KiB)
static size_t decode_lds_bytes(int D, int MQ) {
  const size_t vbufs = (size_t)2 * kWaves * kBC * D;
  const size_t merge = (size_t)(2 * kWaves * 32 + (kWaves - 1) * MQ * D) * 4;
  return vbufs > merge ? vbufs : merge;
}

template <int D, int SB>
static void launch_dec(const DecodeParams& p, int causal, hipStream_t stream) {
  if (p.nwave > 0) {
    const dim3 grid(p.nwave / kWaves);
    const size_t lds = (size_t)2 * kWaves * kBC * D;   // the waves' V buffers
    if (causal) attn_fp8_decode_balanced_kernel<D, SB, true><<<grid, 256, lds, stream>>>(p);
    else attn_fp8_decode_balanced_kernel<D, SB, false><<<grid, 256, lds, stream>>>(p);
    return;
  }
  dim3 grid(p.B * p.Hkv, p.nsplit);
  const size_t lds = decode_lds_bytes(D, p.MQ);
  if (causal) attn_fp8_decode_kernel<D, SB, true><<<grid, 256, lds, stream>>>(p);
  else attn_fp8_decode_kernel<D, SB, false><<<grid, 256, lds, stream>>>(p);
}

hipError_t launch_attn_fp8_decode(const DecodeParams& p, int D, int SB, int causal, hipStream_t stream) {
  if (D == 64 && SB == 64) launch_dec<64, 64>(p, causal, stream);
  else if (D == 64 && SB == 128) launch_dec<64, 128>(p, causal, stream);
  else if (D == 128 && SB == 64) launch_dec<128, 64>(p, causal, stream);
  else launch_dec<128, 128>(p, causal, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.Hkv * p.MQ;
  dim3 cgrid((rows + kWaves - 1) / kWaves);
  if (D == 64) attn_fp8_decode_combine<64><<<cgrid, 256, 0, stream>>>(p);
  else attn_fp8_decode_combine<128><<<cgrid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace attnfp8
