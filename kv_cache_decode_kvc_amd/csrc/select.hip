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
// One workgroup of 1024 threads per row, scores mapped to order-preserving
// 32-bit keys.  A first pass over the row builds a 2048-bin histogram of the
// top 11 key bits and finds the bin d1 that holds the K-th largest key.
//
// Rows of at most 2^18 positions then take a second pass over the row:
// positions with a higher top digit go straight into a one-bit-per-position
// selection map in LDS (one wave ballot per 64 positions), positions in bin
// d1 are appended to a (key, position) list in LDS (each wave its own
// region, so no shared counter).  The exact threshold is
// found on that list (radix select over the remaining 21 key bits), equal
// keys are cut by a radix select over their positions, the chosen list
// entries are added to the map, and one scan of the map's popcounts writes
// the positions in ascending order.  The row is read twice; everything else
// runs on LDS.
//
// A longer row, or a list that would overflow (a wave region of the bin
// holding more than 512 positions, e.g. massive ties), continues with two more histogram passes
// over the row for the remaining key bits and an ordered write-out that
// walks the row in position order (wave ballots and one scan of packed
// (above, equal) counts per 16384 positions).
//
// Every pass over the row prefetches the next 16384 scores while it works on
// the current ones.  No sort, no global atomics: the result is
// deterministic.

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;
// Positions each thread handles per step (all loaded before any is used).
constexpr int kSelUnroll = 16;
constexpr int kSelStep = kSelThreads * kSelUnroll;
// Histogram copies (waves 2c and 2c + 1 count into copy c), so that the
// LDS atomics of different waves rarely meet on one address.
constexpr int kHistCopies = 8;
// (key, position) list of the threshold's top-digit bin; it reuses the
// histogram copies once the first pass is done.  Each wave fills its own
// region of kWaveCand entries (a running count, no shared counter).
constexpr int kSelCand = kHistCopies * kBins / 2;
constexpr int kWaveCand = kSelCand / kSelWaves;

// Larger score -> larger key; -0 and +0 give the same key.  Every finite or
// infinite score maps above 0, which marks non-candidates.
__device__ inline uint32_t score_key(float f) {
  // adding +0 turns -0 into +0 and leaves every other value as it is
  const uint32_t u = __float_as_uint(f + 0.0f);
  // negative: all bits flipped; positive: sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

struct SelLds {
  uint32_t hist[kBins];
  int wsum[kSelWaves];
  int found_digit;
  int found_above;
  int found_count;
  int wcnt[kSelWaves];                 // list entries per wave region
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

// The bin of L.hist, counting from the top, that holds the r-th largest
// entry: L.found_digit, L.found_above (entries in higher bins) and
// L.found_count (entries in it), valid after the call when r <= the
// returned total.  Thread t owns bins 2047 - 2t and 2046 - 2t.
__device__ inline int find_bin(SelLds& L, int r) {
  const int hi = kBins - 1 - 2 * (int)threadIdx.x;
  const int c_hi = (int)L.hist[hi], c_lo = (int)L.hist[hi - 1];
  int total = 0;
  const int above = block_exclusive_scan(c_hi + c_lo, L, total);
  if (above < r && r <= above + c_hi) {
    L.found_digit = hi;
    L.found_above = above;
    L.found_count = c_hi;
  } else if (above + c_hi < r && r <= above + c_hi + c_lo) {
    L.found_digit = hi - 1;
    L.found_above = above + c_hi;
    L.found_count = c_lo;
  }
  __syncthreads();
  return total;
}

// r-th largest (1 <= r <= entries matching prefix under pmask) of the list
// values; each(f) calls f(value) once for every entry (spread over the
// workgroup's threads).  Refined digit by digit over the passes (sh, dm),
// which must cover every bit outside pmask.  Returns the value; gt and eq
// count the matching entries above it and equal to it.
template <int NP, typename Each>
__device__ uint32_t list_select(Each each, int r, uint32_t prefix, uint32_t pmask,
                                const int (&sh)[NP], const uint32_t (&dm)[NP], SelLds& L,
                                int& gt, int& eq) {
  gt = 0;
  eq = 0;
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    for (int i = threadIdx.x; i < kBins; i += kSelThreads) L.hist[i] = 0u;
    __syncthreads();
    each([&](uint32_t x) {
      if ((x & pmask) == prefix) atomicAdd(&L.hist[(x >> sh[pass]) & dm[pass]], 1u);
    });
    __syncthreads();
    find_bin(L, r);
    const uint32_t d = (uint32_t)L.found_digit;
    const int a = L.found_above, c = L.found_count;
    __syncthreads();
    r -= a;
    gt += a;
    eq = c;
    prefix |= d << sh[pass];
    pmask |= dm[pass] << sh[pass];
  }
  return prefix;
}

// Streams the row's scores 16384 positions at a time, the next step's loads
// in flight while f(v, base) works on the current ones (v[u] is the score of
// position base + u * 1024 + threadIdx.x; past n it reads 0).
template <typename F>
__device__ inline void stream_row(__amdgpu_buffer_rsrc_t sr, int n, F&& f) {
  float cur[kSelUnroll], nxt[kSelUnroll];
  const uint32_t t0 = threadIdx.x * 4u;
  auto load = [&](float (&v)[kSelUnroll], int base) {
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u)   // (uniform part in the scalar offset)
      v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          sr, t0, (uint32_t)(base + u * kSelThreads) * 4u, 0));
  };
  // Two buffers used in turn (copying one into the other would wait for
  // the loads in flight); the loads are unconditional: past the row they
  // read zeros without touching memory, and a load under a branch would
  // leave its registers undefined on the other path, which lets the
  // register allocator reuse them and wait for every load in flight.
  if (n <= 0) return;
  load(cur, 0);
  for (int base = 0;; base += 2 * kSelStep) {
    load(nxt, base + kSelStep);
    __builtin_amdgcn_sched_barrier(0);   // the next step's loads go out first
    f(cur, base);
    if (base + kSelStep >= n) break;
    load(cur, base + 2 * kSelStep);
    __builtin_amdgcn_sched_barrier(0);
    f(nxt, base + kSelStep);
    if (base + 2 * kSelStep >= n) break;
  }
}

}  // namespace

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectParams p) {
  __shared__ SelLds L;
  // dynamic LDS: kHistCopies histograms (later the candidate list), the
  // selection map (sel_words), then (pool mode) one bit per block
  extern __shared__ uint32_t dyn[];
  uint32_t* hcopy = dyn;
  uint32_t* ckey = dyn;
  uint32_t* cpos = dyn + kSelCand;
  uint32_t* sel = dyn + kHistCopies * kBins;
  uint32_t* pool_bits = sel + p.sel_words;
  const int row = blockIdx.x;
  const int b = row / p.R;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // (uniform: scalar addressing)
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int n = min(max(p.seq_lens[b], 0), p.L_max);
  const float* sc = p.scores + (size_t)row * p.L_max;
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc, (uint32_t)n * 4u);
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
  // key of position t with score v (0: not a candidate)
  auto key_of = [&](int t, float v) -> uint32_t {
    if (t >= n) return 0u;
    if (p.pool) {
      const int blk = t / p.pool_block;
      if (!((pool_bits[blk >> 5] >> (blk & 31)) & 1u)) return 0u;
    }
    return score_key(v);
  };

  uint32_t prefix = 0, pmask = 0;
  int remaining = p.K;
  bool all = false;
  auto merge_copies = [&]() {
    for (int i = tid; i < kBins; i += kSelThreads) {
      uint32_t c = 0;
#pragma unroll
      for (int h = 0; h < kHistCopies; ++h) c += hcopy[h * kBins + i];
      L.hist[i] = c;
    }
    __syncthreads();
  };
  // Histogram pass over the row: digit (key >> sh) & dmask of the keys
  // matching the digits fixed so far.  The first pass (bound) stops
  // counting keys below a lower bound of the answer's top digit: the K-th
  // largest key of the first 16384 positions is at most the row's, so a
  // lower digit can neither be selected nor sit above the threshold bin.
  // (For N(0,1) scores this drops most of the LDS atomics, which pile up
  // on the few busiest bins.)
  uint32_t dlb = 0;
  auto hist_pass = [&](int sh, uint32_t dmask, bool bound) {
    for (int i = tid; i < kHistCopies * kBins; i += kSelThreads) hcopy[i] = 0u;
    __syncthreads();
    uint32_t* myhist = hcopy + (tid >> 7) * kBins;
    stream_row(sr, n, [&](const float (&v)[kSelUnroll], int base) {
      if (bound && !p.pool && base + kSelStep <= n) {
        // first pass over a whole step without a pool: every position
        // counts, so one compare per key (the per-key instruction count is
        // what bounds these passes: one busy workgroup per compute unit)
        const uint32_t klb = dlb << 21;
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
          const uint32_t k = score_key(v[u]);
          if (k >= klb) atomicAdd(&myhist[k >> 21], 1u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
          const uint32_t k = key_of(base + u * kSelThreads + tid, v[u]);
          if (k != 0u && (k & pmask) == prefix && (k >> 21) >= dlb)
            atomicAdd(&myhist[(k >> sh) & dmask], 1u);
        }
      }
      if (bound && base == 0 && n > kSelStep) {
        __syncthreads();
        merge_copies();
        if (find_bin(L, p.K) >= p.K) dlb = (uint32_t)L.found_digit;
        __syncthreads();
      }
    });
    __syncthreads();
    merge_copies();
  };

  // first pass: top 11 key bits
  hist_pass(21, 0x7FFu, true);
  // (with a bound in force at least K keys were counted, so "keep every
  // candidate" only applies without one)
  if (find_bin(L, remaining) <= p.K && dlb == 0) {
    all = true;                       // every candidate is kept
  } else {
    const uint32_t d = (uint32_t)L.found_digit;
    remaining -= L.found_above;
    prefix = d << 21;
    pmask = 0x7FFu << 21;
  }
  __syncthreads();

  if (p.sel_words > 0) {
    // second pass: the map takes every key above bin d1 (every key when
    // all are kept), the list every key in it
    const uint32_t d1 = prefix >> 21;
    uint32_t* const wkey = ckey + wave * kWaveCand;
    uint32_t* const wpos = cpos + wave * kWaveCand;
    int wc = 0;                       // this wave's list entries so far
    // above: key > ka; in bin d1: key - kb < span (both empty tests when
    // every candidate is kept)
    const uint32_t ka = all ? 0u : ((d1 << 21) | 0x1FFFFFu);
    const uint32_t kb = d1 << 21;
    const uint32_t span = all ? 0u : (1u << 21);
    stream_row(sr, n, [&](const float (&v)[kSelUnroll], int base) {
      if (!p.pool && base + kSelStep <= n) {
        // whole step without a pool: every position is a candidate
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
          const uint32_t k = score_key(v[u]);
          const uint64_t ba = __ballot(k > ka);
          const bool cand = k - kb < span;
          const uint64_t bc = __ballot(cand);
          const int t0 = base + u * kSelThreads + wave * 64;
          if (lane == 0) *reinterpret_cast<uint64_t*>(sel + (t0 >> 5)) = ba;
          if (cand) {
            const int s = wc + __popcll(bc & below);
            if (s < kWaveCand) {
              wkey[s] = k;
              wpos[s] = (uint32_t)(t0 + lane);
            }
          }
          wc += __popcll(bc);
        }
        return;
      }
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int t = base + u * kSelThreads + tid;
        const uint32_t k = key_of(t, v[u]);
        const bool above = k != 0u && (all || (k >> 21) > d1);
        const bool cand = !all && k != 0u && (k >> 21) == d1;
        const uint64_t ba = __ballot(above);
        // the wave's 64 positions start at t - lane, a multiple of 64
        if (lane < 2) sel[((t - lane) >> 5) + lane] = lane ? (uint32_t)(ba >> 32) : (uint32_t)ba;
        const uint64_t bc = __ballot(cand);
        if (cand) {
          const int s = wc + __popcll(bc & below);
          if (s < kWaveCand) {
            wkey[s] = k;
            wpos[s] = (uint32_t)t;
          }
        }
        wc += __popcll(bc);
      }
    });
    if (lane == 0) L.wcnt[wave] = wc;
    __syncthreads();
    bool fits = true;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) fits = fits && L.wcnt[w] <= kWaveCand;
    // every wave walks the entries of its own list region
    const int wn = min(L.wcnt[wave], kWaveCand);
    auto each_key = [&](auto&& f) {
      for (int i = lane; i < wn; i += 64) f(wkey[i]);
    };
    if (fits) {
      if (!all) {
        // exact threshold among the list, then the first `take` of the keys
        // equal to it by position (largest ~position = lowest position)
        int gt, eq;
        const int shk[2] = {10, 0};
        const uint32_t dmk[2] = {0x7FFu, 0x3FFu};
        const uint32_t thr = list_select<2>(each_key, remaining, prefix, pmask, shk, dmk, L, gt, eq);
        const int take = remaining - gt;
        uint32_t pthr = 0u;
        if (take < eq) {
          int g2, e2;
          const int shp[2] = {9, 0};
          const uint32_t dmp[2] = {0x1FFu, 0x1FFu};
          pthr = list_select<2>(
              [&](auto&& f) {
                for (int i = lane; i < wn; i += 64) f(wkey[i] == thr ? ~wpos[i] : 0u);
              },
              take, 0xFFFC0000u, 0xFFFC0000u, shp, dmp, L, g2, e2);
        }
        for (int i = lane; i < wn; i += 64) {
          const uint32_t k = wkey[i], t = wpos[i];
          if (k > thr || (k == thr && ~t >= pthr)) atomicOr(&sel[t >> 5], 1u << (t & 31));
        }
        __syncthreads();
      }
      // ordered write-out from the map: thread t takes consecutive words
      const int W = (n + 31) >> 5;
      const int wpt = (W + kSelThreads - 1) / kSelThreads;
      const int w0 = tid * wpt;
      int cnt = 0;
      for (int w = w0; w < w0 + wpt && w < W; ++w) cnt += __popc(sel[w]);
      int kept = 0;
      int off = block_exclusive_scan(cnt, L, kept);
      for (int w = w0; w < w0 + wpt && w < W; ++w) {
        uint32_t bits = sel[w];
        while (bits) {
          out[off++] = w * 32 + __builtin_ctz(bits);
          bits &= bits - 1u;
        }
      }
      for (int i = kept + tid; i < p.K; i += kSelThreads) out[i] = -1;
      return;
    }
    // the list overflowed: the list area is the histograms again below
  }

  // remaining key bits over the row: 11, then 10
  if (!all) {
#pragma unroll
    for (int pass = 1; pass < 3; ++pass) {
      const int sh = pass == 1 ? 10 : 0;
      const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
      hist_pass(sh, dmask, false);
      find_bin(L, remaining);
      const uint32_t d = (uint32_t)L.found_digit;
      remaining -= L.found_above;
      prefix |= d << sh;
      pmask |= dmask << sh;
      __syncthreads();
    }
  }
  const uint32_t thr = all ? 0u : prefix;   // keys above thr are kept
  const int take = all ? 0 : remaining;     // and the first `take` equal to it

  // ordered write-out, kSelStep positions per step: position base + u*1024 +
  // tid (u < kSelUnroll), so ascending positions are ordered by (u, wave,
  // lane).  Per (u, wave) the above/equal counts come from ballots; one
  // scan over the kSelUnroll x 16 (u, wave) pairs gives every pair its
  // prefix, and a lane adds the count of its wave's lower lanes.
  int written = 0, eq_seen = 0;
  stream_row(sr, n, [&](const float (&v)[kSelUnroll], int base) {
    uint64_t bg[kSelUnroll], be[kSelUnroll];
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u) {
      const uint32_t k = key_of(base + u * kSelThreads + tid, v[u]);
      bg[u] = __ballot(k != 0u && k > thr);
      be[u] = __ballot(!all && k != 0u && k == thr);
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
  });
  const int kept = written + min(eq_seen, take);
  for (int i = kept + tid; i < p.K; i += kSelThreads) out[i] = -1;
}

hipError_t launch_topk_select(const SelectParams& p, hipStream_t s) {
  const size_t dyn = ((size_t)kHistCopies * kBins + p.sel_words +
                      (p.pool ? (size_t)p.pool_words : 0)) * 4;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        (const void*)topk_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)((kHistCopies * kBins + kSelectMapMax / 32 + kSelectPoolWords) * 4));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)((size_t)p.B * p.R)), dim3(kSelThreads),
                     dyn, s, p);
  return hipGetLastError();
}

}  // namespace kvc
