// Top-k selection from indexer scores for gfx950.
//
// What is computed (podcast transcript, DeepSeek Sparse Attention passage:
// an indexer scores the prefix and a top-k subset of positions is kept;
// "A Hundred Messages" blog, section 4, the hierarchical indexer: a deeper
// indexer chooses only among the positions of a candidate pool of 8-position
// blocks): for each row (sequence b, index head j) the K positions t < n_b
// with the highest scores, equal scores taken by lower position first,
// written in ascending position order and padded with -1.
//
// One workgroup of 1024 threads per row.  The K-th largest score is found
// exactly by a three-pass radix select on order-preserving 32-bit keys (11,
// 11 and 10 key bits per pass, a 2048-bin histogram in LDS per pass, each
// pass counting only the keys that match the digits fixed so far).  A last
// pass walks the row in position order, 16384 positions at a time, and writes
// every position whose key is above the threshold plus the first `take`
// positions equal to it; wave ballots and one scan of packed (above, equal)
// counts give each thread its output slots.  No sort, no global atomics: the
// result is deterministic.

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;
// Positions each thread handles per step: its loads are all issued before
// any is used, so a row streams with 64 KB in flight per workgroup.
constexpr int kSelUnroll = 16;
constexpr int kSelStep = kSelThreads * kSelUnroll;
// Histogram copies (waves 2c and 2c + 1 count into copy c), so that the
// LDS atomics of different waves rarely meet on one address.
constexpr int kHistCopies = 8;

// Larger score -> larger key; -0 and +0 give the same key.  Every finite or
// infinite score maps above 0, which marks non-candidates.
__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelLds {
  uint32_t hist[kBins];
  int wsum[kSelWaves];
  int found_digit;
  int found_above;
  int pre[kSelUnroll][kSelWaves][2];   // write-out: (above, equal) counts per (step slice, wave)
};

// Exclusive scan of one int per thread over the workgroup; returns the
// exclusive prefix and sets `total`.  Uses wsum (wave totals).
__device__ inline int block_exclusive_scan(int x, SelLds& L, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) L.wsum[wave] = v;
  __syncthreads();
  int wprefix = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = L.wsum[w];
    wprefix += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return wprefix + v - x;
}

}  // namespace

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectParams p) {
  __shared__ SelLds L;
  // dynamic LDS: kHistCopies histograms, then (pool mode) one bit per block
  extern __shared__ uint32_t dyn[];
  uint32_t* hcopy = dyn;
  uint32_t* pool_bits = dyn + kHistCopies * kBins;
  const int row = blockIdx.x;
  const int b = row / p.R;
  const int tid = threadIdx.x;
  const int n = min(max(p.seq_lens[b], 0), p.L_max);
  const float* sc = p.scores + (size_t)row * p.L_max;
  int32_t* out = p.out + (size_t)row * p.K;

  if (p.pool) {
    for (int w = tid; w < p.pool_words; w += kSelThreads) pool_bits[w] = 0u;
    __syncthreads();
    const int32_t* pr = p.pool + (size_t)row * p.P;
    const int nblk = p.pool_words * 32;
    for (int e = tid; e < p.P; e += kSelThreads) {
      const int blk = pr[e];
      if (blk >= 0 && blk < nblk) atomicOr(&pool_bits[blk >> 5], 1u << (blk & 31));
    }
    __syncthreads();
  }
  auto key_at = [&](int t) -> uint32_t {
    if (t >= n) return 0u;
    if (p.pool) {
      const int blk = t / p.pool_block;
      if (!((pool_bits[blk >> 5] >> (blk & 31)) & 1u)) return 0u;
    }
    return score_key(sc[t]);
  };

  // radix select of the K-th largest key
  uint32_t prefix = 0, pmask = 0;
  int remaining = p.K;
  bool all = false;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = tid; i < kHistCopies * kBins; i += kSelThreads) hcopy[i] = 0u;
    __syncthreads();
    uint32_t* myhist = hcopy + (tid >> 7) * kBins;
    for (int base = 0; base < n; base += kSelStep) {
      uint32_t k[kSelUnroll];
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) k[u] = key_at(base + u * kSelThreads + tid);
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u)
        if (k[u] != 0u && (k[u] & pmask) == prefix) atomicAdd(&myhist[(k[u] >> sh) & dmask], 1u);
    }
    __syncthreads();
    for (int i = tid; i < kBins; i += kSelThreads) {
      uint32_t c = 0;
#pragma unroll
      for (int h = 0; h < kHistCopies; ++h) c += hcopy[h * kBins + i];
      L.hist[i] = c;
    }
    __syncthreads();
    // thread tid owns bins hi = 2047 - 2 tid and lo = hi - 1 (descending)
    const int hi = kBins - 1 - 2 * tid;
    const int c_hi = (int)L.hist[hi], c_lo = (int)L.hist[hi - 1];
    int total = 0;
    const int above = block_exclusive_scan(c_hi + c_lo, L, total);
    if (pass == 0 && total <= p.K) {   // every candidate is kept
      all = true;
      break;
    }
    if (above < remaining && remaining <= above + c_hi) {
      L.found_digit = hi;
      L.found_above = above;
    } else if (above + c_hi < remaining && remaining <= above + c_hi + c_lo) {
      L.found_digit = hi - 1;
      L.found_above = above + c_hi;
    }
    __syncthreads();
    const uint32_t d = (uint32_t)L.found_digit;
    remaining -= L.found_above;
    prefix |= d << sh;
    pmask |= dmask << sh;
    __syncthreads();
  }
  const uint32_t thr = all ? 0u : prefix;   // keys above thr are kept
  const int take = all ? 0 : remaining;     // and the first `take` equal to it

  // ordered write-out, kSelStep positions per step: position base + u*1024 +
  // tid (u < kSelUnroll), so ascending positions are ordered by (u, wave,
  // lane).  Per (u, wave) the above/equal counts come from ballots; one
  // scan over the kSelUnroll x 16 (u, wave) pairs gives every pair its
  // prefix, and a lane adds the count of its wave's lower lanes.
  int written = 0, eq_seen = 0;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n; base += kSelStep) {
    uint32_t k[kSelUnroll];
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u) k[u] = key_at(base + u * kSelThreads + tid);
    uint64_t bg[kSelUnroll], be[kSelUnroll];
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u) {
      bg[u] = __ballot(k[u] != 0u && k[u] > thr);
      be[u] = __ballot(!all && k[u] != 0u && k[u] == thr);
      if (lane == 0) {
        L.pre[u][wave][0] = __popcll(bg[u]);
        L.pre[u][wave][1] = __popcll(be[u]);
      }
    }
    __syncthreads();
    // pair i = (u, w) in position order; threads 0..255 scan the pairs
    const int np = kSelUnroll * kSelWaves;
    int c = 0;
    if (tid < np) c = L.pre[tid >> 4][tid & 15][0] | (L.pre[tid >> 4][tid & 15][1] << 16);
    int total = 0;
    const int pre = block_exclusive_scan(c, L, total);
    if (tid < np) {
      L.pre[tid >> 4][tid & 15][0] = pre & 0xFFFF;
      L.pre[tid >> 4][tid & 15][1] = pre >> 16;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u) {
      const int t = base + u * kSelThreads + tid;
      const int gt_before = written + L.pre[u][wave][0] + __popcll(bg[u] & below);
      const int eq_before = eq_seen + L.pre[u][wave][1] + __popcll(be[u] & below);
      if ((bg[u] >> lane) & 1ull) out[gt_before + min(eq_before, take)] = t;
      else if (((be[u] >> lane) & 1ull) && eq_before < take) out[gt_before + eq_before] = t;
    }
    written += total & 0xFFFF;
    eq_seen += total >> 16;
    __syncthreads();
  }
  const int kept = written + min(eq_seen, take);
  for (int i = kept + tid; i < p.K; i += kSelThreads) out[i] = -1;
}

hipError_t launch_topk_select(const SelectParams& p, hipStream_t s) {
  const size_t dyn = (size_t)kHistCopies * kBins * 4 + (p.pool ? (size_t)p.pool_words * 4 : 0);
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(kHistCopies * kBins * 4 + kSelectPoolWords * 4));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)((size_t)p.B * p.R)), dim3(kSelThreads),
                     dyn, s, p);
  return hipGetLastError();
}

}  // namespace kvc
