// Work list of the packed-document FP8 attention (gfx950).
//
// "FLAMIA" (4.3 Ablation Study) runs the work of causal packed workloads
// longest first, and (F. System Integration) keeps its work lists on the GPU,
// so that a call needs no host synchronisation and can be captured in a
// graph.  Here one workgroup of 1024 threads builds the list before the
// attention launch:
//   1. it checks cu_seqlens (starts at 0, never decreases, ends at T) and
//      counts the documents by their number of query tiles nt;
//   2. longest first: documents in non-increasing nt (an exclusive suffix
//      scan of nt * count over nt gives the first position of each length);
//      every document takes one contiguous range of the list (an LDS atomic
//      per document; the order among documents of equal nt is free and no
//      result depends on it) and fills it with its query tiles from the last
//      to the first, the last one seeing the most keys under a causal mask.
//      A document's tiles thus run together, and with them the reuse of its
//      K and V in the L2 of the XCD its head is on; ordering single tiles by
//      their cost across documents loses that reuse and measured slower.
// The natural order (document-major, tiles ascending: the baseline of the
// ablation) is a prefix sum of nt over the documents instead.
// Invalid cu_seqlens: count 0 and status 1, and the attention writes nothing.
#include "common.h"
#include "attn_internal.h"

namespace attnfp8 {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;

// Exclusive prefix sum of one value per thread, in thread order; *total gets
// the sum over the workgroup.  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int x, int* wsum, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSchedWaves; ++w) {
    const int s = wsum[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();   // wsum is free again for the next call
  *total = tot;
  return base + v - x;
}

// In place over a[0 .. n): a[i] <- sum of a[j] over j > i (exclusive) or
// j >= i (inclusive).  Thread t owns a chunk, thread 0 the highest indices.
__device__ __forceinline__ void suffix_scan(int* a, int n, bool inclusive, int* wsum) {
  const int t = threadIdx.x;
  const int per = (n + kSchedThreads - 1) / kSchedThreads;
  const int hi = n - t * per > 0 ? n - t * per : 0;
  const int lo = n - (t + 1) * per > 0 ? n - (t + 1) * per : 0;
  int s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  int total;
  int run = block_exclusive_scan(s, wsum, &total);
  for (int i = hi - 1; i >= lo; --i) {
    const int v = a[i];
    if (inclusive) {
      run += v;
      a[i] = run;
    } else {
      a[i] = run;
      run += v;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int doc_tiles(const int* cu, int d) {
  return (cu[d + 1] - cu[d] + kQueryTile - 1) / kQueryTile;
}

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(VarlenSchedParams p) {
  __shared__ int key_pos[kVarlenMaxKeys];   // per tile count (index nt - 1): documents, then positions
  __shared__ int wsum[kSchedWaves];
  __shared__ int s_bad;
  __shared__ int s_items;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;

  for (int i = t; i < p.kmax; i += kSchedThreads) key_pos[i] = 0;
  if (t == 0) {
    s_bad = 0;
    s_items = 0;
  }
  __syncthreads();
  int mine = 0;
  for (int d = t; d < p.ndoc; d += kSchedThreads) {
    const int a = p.cu[d], b = p.cu[d + 1];
    const bool ok = a >= 0 && a <= b && b <= p.T && (d > 0 || a == 0) && (d < p.ndoc - 1 || b == p.T);
    if (!ok) {
      atomicOr(&s_bad, 1);
      continue;
    }
    const int nt = (b - a + kQueryTile - 1) / kQueryTile;   // <= ceil(T / 128) = kmax
    if (nt > 0) atomicAdd(&key_pos[nt - 1], 1);
    mine += nt;
  }
  atomicAdd(&s_items, mine);
  __syncthreads();
  if (s_bad) {
    if (t == 0) {
      p.ws[0] = 0;
      p.ws[1] = 1;
    }
    return;
  }
  int2* items = (int2*)(p.ws + kWsHeaderInts);

  if (!p.natural) {
    // the nt tiles of every document with nt = c: first position of each c
    for (int i = t; i < p.kmax; i += kSchedThreads) key_pos[i] *= i + 1;
    __syncthreads();
    suffix_scan(key_pos, p.kmax, false, wsum);
    for (int d = wave; d < p.ndoc; d += kSchedWaves) {
      const int nt = doc_tiles(p.cu, d);
      if (nt == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&key_pos[nt - 1], nt);
      base = __shfl(base, 0, 64);
      for (int r = lane; r < nt; r += 64) items[base + (nt - 1 - r)] = make_int2(d, r);
    }
  } else {
    int carry = 0;
    for (int d0 = 0; d0 < p.ndoc; d0 += kSchedThreads) {
      const int d = d0 + t;
      const int nt = d < p.ndoc ? doc_tiles(p.cu, d) : 0;
      int total;
      const int base = carry + block_exclusive_scan(nt, wsum, &total);
      for (int r = 0; r < nt; ++r) items[base + r] = make_int2(d, r);
      carry += total;
    }
  }
  if (t == 0) {
    p.ws[0] = s_items;
    p.ws[1] = 0;
  }
}

hipError_t launch_varlen_schedule(const VarlenSchedParams& sp, hipStream_t stream) {
  varlen_schedule_kernel<<<1, kSchedThreads, 0, stream>>>(sp);
  return hipGetLastError();
}

}  // namespace attnfp8
