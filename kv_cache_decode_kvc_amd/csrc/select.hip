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
//
// Segmented form (a workspace given, no pool, rows of at most 2^18
// positions): one workgroup per row leaves most compute units idle when
// there are few rows, so each row is cut into segments of whole
// 16384-position steps, about 256 workgroups in all, one kernel:
//  - every workgroup of a row reads the same 1/32 sample of it (64
//    positions of every 2048) and takes a lower bound of the row's K-th
//    largest key that leaves, in expectation, about K + 4 standard
//    deviations' worth of keys above it;
//  - each of its waves writes the keys of its own contiguous part of the
//    segment at or above the bound, with positions, to its candidate list
//    (no atomics), so the lists in (segment, wave) order run in ascending
//    position order;
//  - the last workgroup of the row to finish (a ticket) gathers all the
//    candidates into LDS in that order, finds the exact K-th largest among
//    them (two 11-bit digit passes over its distance from the bound, three
//    over whole keys when it lies 2^22 or more above it; one wave scanning
//    each 2048-bin histogram), breaks ties by position, and writes the
//    chosen ones out by a prefix count.  A row whose lists overflowed, or
//    whose bound left fewer than K keys above it, is finished by the
//    one-workgroup algorithm above instead.
// The chosen set is the same as the one-workgroup algorithm's (the
// selection is defined uniquely), so the output is too.

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

// hist[bin] += 1 for every lane with `on` (lanes that do not reach the
// call do not count).  LDS atomics on one address are served one lane at a
// time, and candidate lists often share a few leading digits: the lanes
// whose bin equals the first lane's add their count in one atomic, the
// others one each (a second and third such round measured slower: 26.0
// against 26.4 us per 2048-of-131072 selection over 64 rows).
__device__ inline void hist_add(uint32_t* hist, uint32_t bin, bool on) {
  const int lane = threadIdx.x & 63;
  bool left = on;
#pragma unroll
  for (int round = 0; round < 1; ++round) {
    const uint64_t act = __ballot(left);
    if (act == 0) return;
    const int first = __ffsll((long long)act) - 1;
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
    const bool same = left && bin == b0;
    const uint64_t group = __ballot(same);
    if (lane == first) atomicAdd(&hist[b0], (uint32_t)__popcll(group));
    left = left && !same;
  }
  if (left) atomicAdd(&hist[bin], 1u);
}

struct SelLds {
  alignas(16) uint32_t hist[kBins];   // (16-byte reads in find_bin_wave)
  int wsum[kSelWaves];
  int found_digit;
  int found_above;
  int found_count;
  int wcnt[kSelWaves];                 // list entries per wave region
  int pre[kSelUnroll][kSelWaves][2];   // write-out: (above, equal) counts per (step slice, wave)
};

// Inclusive scan over the 64 lanes of a wave with data-parallel-primitive
// moves (vector ALU, no LDS round trips): prefix within each row of 16
// lanes by shifts of 1, 2, 4, 8 (lanes whose source falls before the row
// start add 0), then row 15's total into rows 1 and 3 and lane 31's into
// rows 2 and 3.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive scan of one int per thread over the workgroup; returns the
// exclusive prefix and sets `total`.  Uses wsum (wave totals).
__device__ inline int block_exclusive_scan(int x, SelLds& L, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v = wave_incl_scan(x);
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
__device__ __forceinline__ uint32_t list_select(Each each, int r, uint32_t prefix,
                                                uint32_t pmask, const int (&sh)[NP],
                                                const uint32_t (&dm)[NP], SelLds& L, int& gt,
                                                int& eq) {
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

// Ordered write-out from a one-bit-per-position map of the row's first n
// positions: thread t takes consecutive words, one scan gives its offset;
// slots past the kept count are -1.
__device__ inline void write_out_map(const uint32_t* sel, int n, int32_t* out, int K,
                                     SelLds& L) {
  const int tid = threadIdx.x;
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
  for (int i = kept + tid; i < K; i += kSelThreads) out[i] = -1;
}

// The one-workgroup algorithm for one row (dyn: the dynamic LDS of
// launch_topk_select's one-workgroup kernel).
__device__ __forceinline__ void select_row(const SelectParams& p, const int row, SelLds& L,
                                           uint32_t* dyn) {
  // dynamic LDS: kHistCopies histograms (later the candidate list), the
  // selection map (sel_words), then (pool mode) one bit per block
  uint32_t* hcopy = dyn;
  uint32_t* ckey = dyn;
  uint32_t* cpos = dyn + kSelCand;
  uint32_t* sel = dyn + kHistCopies * kBins;
  uint32_t* pool_bits = sel + p.sel_words;
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
      // ordered write-out from the map
      write_out_map(sel, n, out, p.K, L);
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

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectParams p) {
  __shared__ SelLds L;
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  select_row(p, blockIdx.x, L, dyn);
}

// ---------------------------------------------------------------- segmented
// Segment `seg` of row `row`: positions [s0, s0 + sn) of the row (sn may be
// 0 past the row's length).
struct SegPos {
  int row, seg, b, n, s0, sn;
};

__device__ inline SegPos seg_pos(const SelectParams& p) {
  SegPos q;
  q.row = blockIdx.x / p.S;
  q.seg = blockIdx.x - q.row * p.S;
  q.b = q.row / p.R;
  q.n = min(max(p.seq_lens[q.b], 0), p.L_max);
  q.s0 = q.seg * p.seg_len;
  q.sn = min(max(q.n - q.s0, 0), p.seg_len);
  return q;
}

// Sampled positions: 64 consecutive positions at the start of every
// 2048-position block of the row (1/32 of it, spread over the whole row).
constexpr int kSampleRun = 64;
constexpr int kSampleEvery = 2048;
// (key, position) pairs the finishing workgroup holds in LDS
constexpr int kFinCand = kHistCopies * kBins / 2;
constexpr int kFinPer = kFinCand / kSelThreads;

// r-th largest digit of a 2048-bin histogram h (16-byte aligned): wave 0
// scans the bins from the top, 32 per lane (eight 16-byte reads), one wave
// prefix sum, then the lane holding the r-th entry walks its 32 bins; the
// digit and the counts above it and in it go to L.found_*; one barrier.
// Valid when r <= the histogram's total.
__device__ inline void find_bin_wave(const uint32_t* h, SelLds& L, int r) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int lo = kBins - 32 * (lane + 1);        // this lane's bins lo .. lo + 31
    int qs[8], sum = 0;                            // sums of its eight groups of four
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 c = *reinterpret_cast<const u32x4*>(h + lo + 4 * i);
      qs[i] = (int)(c[0] + c[1] + c[2] + c[3]);
      sum += qs[i];
    }
    const int incl = wave_incl_scan(sum);
    int above = incl - sum;
    if (above < r && r <= incl) {
      int g = 0;                                   // the group holding the r-th entry, from the top
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        if (g == 0 && r <= above + qs[i]) g = i + 1;
        else if (g == 0) above += qs[i];
      }
      const u32x4 c = *reinterpret_cast<const u32x4*>(h + lo + 4 * (g - 1));
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const int cnt = (int)c[j];
        if (above < r && r <= above + cnt) {
          L.found_digit = lo + 4 * (g - 1) + j;
          L.found_above = above;
          L.found_count = cnt;
        }
        above += cnt;
      }
    }
  }
  __syncthreads();
}

// r-th largest of the values get(i) (i < nv, at most kFinPer, uniform;
// counted where ok(i)) matching prefix under pmask, refined digit by digit
// at the shifts sh and masks dm (which must cover every bit outside pmask;
// digits below 2048).  Two 2048-bin histograms h0, h1 alternate: each pass
// counts into one while the other is cleared for the next; the caller
// clears h0 (with a barrier after).  Two barriers per pass.  The first pass
// aggregates lanes that share a bin (candidates above a bound share a few
// leading digits); later passes, whose digits are spread, add one atomic
// per lane.  Returns the value; gt and eq count the matching values above
// it and equal to it.
template <int NP, typename Get, typename Ok>
__device__ __forceinline__ uint32_t reg_select(Get get, Ok ok, int r, uint32_t prefix,
                                               uint32_t pmask, const int (&sh)[NP],
                                               const uint32_t (&dm)[NP], uint32_t* h0,
                                               uint32_t* h1, SelLds& L, int& gt, int& eq,
                                               int nv = kFinPer) {
  gt = 0;
  eq = 0;
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    uint32_t* h = (pass & 1) ? h1 : h0;
    uint32_t* hn = (pass & 1) ? h0 : h1;
#pragma unroll
    for (int i = 0; i < kFinPer; ++i) {
      if (i >= nv) break;
      const uint32_t x = get(i);
      const bool on = ok(i) && (x & pmask) == prefix;
      const uint32_t bin = (x >> sh[pass]) & dm[pass];
      if (pass == 0) hist_add(h, bin, on);
      else if (on) atomicAdd(&h[bin], 1u);
    }
    if (pass + 1 < NP)
      for (int i = threadIdx.x; i < kBins; i += kSelThreads) hn[i] = 0u;
    __syncthreads();
    find_bin_wave(h, L, r);
    const uint32_t d = (uint32_t)L.found_digit;
    const int a = L.found_above, c = L.found_count;
    r -= a;
    gt += a;
    eq = c;
    prefix |= d << sh[pass];
    pmask |= dm[pass] << sh[pass];
  }
  return prefix;
}

// The row's sample as each lane loads it: block c = wave + 16 u (u < 8) of
// the row, position 2048 c + lane (rows of at most 2^18 positions have at
// most 128 blocks).  Loads past the row read zeros.
constexpr int kSampleLoads = kSelectMapMax / kSampleEvery / kSelWaves;

__device__ inline void sample_load(const SelectParams& p, int row, int n,
                                   uint32_t (&v)[kSampleLoads]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.scores + (size_t)row * p.L_max, (uint32_t)n * 4u);
#pragma unroll
  for (int u = 0; u < kSampleLoads; ++u)
    v[u] = __builtin_amdgcn_raw_buffer_load_b32(
        sr, (uint32_t)(((wave + u * kSelWaves) * kSampleEvery + lane) * 4), 0, 0);
}

// Lower bound of the row's K-th largest key from its sample (every
// workgroup of the row computes the same one): the lower edge of the
// top-digit bin holding the sample's r-th largest key, r = K / 32 plus four
// standard deviations of a binomial count of that size, so that in
// expectation comfortably more than K keys of the row lie at or above it,
// but not many more.  0 when the sample has fewer than r keys (every valid
// key is then a candidate).  Whether the bound really leaves K keys above it
// is checked once the candidates are counted.
__device__ inline uint32_t row_bound(const SelectParams& p, int n, const uint32_t (&v)[kSampleLoads],
                                     SelLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kBins; i += kSelThreads) L.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kSampleLoads; ++u) {
    const int t = (wave + u * kSelWaves) * kSampleEvery + lane;
    hist_add(L.hist, score_key(__uint_as_float(v[u])) >> 21, t < n);
  }
  __syncthreads();
  const float mean = (float)p.K / (float)(kSampleEvery / kSampleRun);
  const int r = (int)ceilf(mean + 4.f * sqrtf(mean)) + 1;
  const int total = find_bin(L, r);
  const uint32_t lb = total >= r ? ((uint32_t)L.found_digit << 21) : 0u;
  __syncthreads();
  return lb;
}

// The workgroup of (row, segment): the row's bound (every workgroup of the
// row computes the same one from the row's sample, while its own segment's
// first loads are in flight), then every valid key of the segment at or
// above it, with its position, into this wave's candidate list (collected
// in LDS, then written out whole with device-coherent stores; no atomics).
// The last of the row's workgroups to finish (a device-scope ticket)
// selects among all of them.
__global__ __launch_bounds__(kSelThreads) void seg_select_kernel(SelectParams p) {
  __shared__ SelLds L;
  __shared__ int s_last, s_over;
  __shared__ int s_off[kSelSegWaves * 32 + 1];   // list offsets per (segment, wave); S <= 32
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  const SegPos q = seg_pos(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the row's sample, then the segment's first two steps in flight; the
  // bound is computed from the sample while the steps arrive
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(p.scores + (size_t)q.row * p.L_max + q.s0, (uint32_t)q.sn * 4u);
  // Wave w takes positions [w R, (w + 1) R) of the segment (R = seg_len /
  // 16, whole 1024-position steps), so that its list, and the lists taken
  // in (segment, wave) order, run in ascending position order.  Step k of
  // the wave: v[i][j] is position w R + 1024 k + 256 i + 4 lane + j.
  constexpr int kQ = kSelUnroll / 4;       // 16-byte loads per lane and step
  constexpr int kWStep = 64 * kSelUnroll;  // positions per wave and step
  const int R = p.seg_len / kSelWaves;
  const int wsteps = R / kWStep;
  u32x4 st0[kQ], st1[kQ];
  auto load_step = [&](u32x4 (&v)[kQ], int k) {
#pragma unroll
    for (int i = 0; i < kQ; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(
          sr, lane * 16u, (uint32_t)(wave * R + k * kWStep + i * 256) * 4u, 0);
  };
  uint32_t smp[kSampleLoads];
  sample_load(p, q.row, q.n, smp);
  __builtin_amdgcn_sched_barrier(0);
  load_step(st0, 0);
  load_step(st1, 1);
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t lb = row_bound(p, q.n, smp, L);

  const __amdgpu_buffer_rsrc_t wc_r = make_rsrc(p.ws_cand, kWsRecords);
  const __amdgpu_buffer_rsrc_t wn_r = make_rsrc(p.ws_ccnt, kWsRecords);
  const int nreg = p.S * kSelSegWaves;
  const uint32_t row_cand = (uint32_t)((size_t)q.row * nreg * kSelSegCapw * 8);
  {
    const int region = q.seg * kSelSegWaves + wave;       // within the row
    const uint32_t cbase = row_cand + (uint32_t)(region * kSelSegCapw * 8);
    u32x2* stage = reinterpret_cast<u32x2*>(dyn) + wave * kSelSegCapw;   // this wave's list
    int wc = 0;
    // key >= lb as a float compare (one instruction per position; the key
    // is formed only for the candidates): lb's score, or -inf when every
    // score qualifies
    float lbf = -__builtin_huge_valf();
    if (lb & 0x80000000u) lbf = __uint_as_float(lb & 0x7FFFFFFFu);          // >= +0
    else if (lb != 0u && ((~lb >> 23) & 0xFFu) != 0xFFu) lbf = __uint_as_float(~lb);
    // a lane's candidates among its four positions of each 256, placed
    // after those of the lanes below it (one wave scan per 256 positions)
    auto process = [&](const u32x4 (&v)[kQ], int k) {
      const int base = wave * R + k * kWStep;
      const bool whole = base + kWStep <= q.sn;
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = base + 256 * i + 4 * lane + j;
          const bool c = __uint_as_float(v[i][j]) >= lbf && (whole || t < q.sn);
          m |= (c ? 1u : 0u) << j;
        }
        const int cnt = __popc(m);
        const int incl = wave_incl_scan(cnt);
        int slot = wc + incl - cnt;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if ((m >> j) & 1u) {
            if (slot < kSelSegCapw)
              stage[slot] = u32x2{score_key(__uint_as_float(v[i][j])),
                                  (uint32_t)(q.s0 + base + 256 * i + 4 * lane + j)};
            ++slot;
          }
        wc += __builtin_amdgcn_readlane(incl, 63);
      }
    };
    process(st0, 0);
    if (wsteps > 1) process(st1, 1);
    // longer segments: the remaining steps, each loaded while the previous
    // one is processed
    for (int k = 2; k < wsteps; k += 2) {
      load_step(st0, k);
      load_step(st1, k + 1);
      process(st0, k);
      if (k + 1 < wsteps) process(st1, k + 1);
    }
    // (the wave's own LDS writes are complete for its own reads below)
    const int kept = wc < kSelSegCapw ? wc : kSelSegCapw;
    for (int i = lane; i < kept; i += 64)
      __builtin_amdgcn_raw_buffer_store_b64(stage[i], wc_r, cbase + (uint32_t)(i * 8), 0,
                                            kCoherent);
    if (lane == 0)
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)wc, wn_r,
                                            (uint32_t)(((size_t)q.row * nreg + region) * 4), 0,
                                            kCoherent);
  }
  wait_vm_all();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&p.ws_cnt[q.row], 1) == p.S - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- the row's last workgroup: select among all the candidates
  if (tid == 0) p.ws_cnt[q.row] = 0;
  const int c = tid < nreg ? (int)__builtin_amdgcn_raw_buffer_load_b32(
                                 wn_r, (uint32_t)(((size_t)q.row * nreg + tid) * 4), 0, kCoherent)
                           : 0;
  // Wave w copies lists w, w + 16, ... (kSelSegCapw slots each: two per
  // lane).  Its first batch (four lists) is loaded whole together with the
  // counts, before they are known, so the gather costs no second round trip;
  // slots past a list's count are loaded but not used.
  auto load_batch = [&](u32x2 (&v)[8], int r0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = r0 + (j >> 1) * kSelWaves, i = lane + (j & 1) * 64;
      v[j] = __builtin_amdgcn_raw_buffer_load_b64(
          wc_r, row_cand + (uint32_t)(((r < nreg ? r : 0) * kSelSegCapw + i) * 8), 0, kCoherent);
    }
  };
  u32x2 v[8];
  load_batch(v, wave);
  // list offsets into s_off (the total at s_off[nreg]) and whether a list
  // overflowed; with at most 64 lists wave 0 alone scans them, and one
  // barrier (the one after the clearing below) publishes the result
  if (nreg <= 64) {
    if (wave == 0) {
      const int incl = wave_incl_scan(c);
      const bool ov = __ballot(c > kSelSegCapw) != 0ull;
      if (tid < nreg) s_off[tid] = incl - c;
      if (lane == 63) {
        s_off[nreg] = incl;
        s_over = ov;
      }
    }
  } else {
    const int ov = __syncthreads_or(c > kSelSegCapw);
    int tot = 0;
    const int off = block_exclusive_scan(c, L, tot);
    if (tid < nreg) s_off[tid] = off;
    if (tid == 0) {
      s_off[nreg] = tot;
      s_over = ov;
    }
  }
  uint32_t* ck = dyn;
  uint32_t* cp = dyn + kFinCand;
  // the digit passes' two histograms lie outside the candidate area (the
  // sample's, free since the bound, and one past the map area), so h0 is
  // cleared here and the passes start as soon as the candidates are in
  // registers
  uint32_t* h0 = L.hist;
  uint32_t* h1 = dyn + kHistCopies * kBins + p.sel_words;
  for (int i = tid; i < kBins; i += kSelThreads) h0[i] = 0u;
  __syncthreads();
  const int total = s_off[nreg];
  // every valid key was collected when the bound is 0
  const bool all = lb == 0u && total <= p.K;
  if (s_over || total > kFinCand || (total < p.K && lb != 0u)) {
    // a list overflowed, too many candidates for the LDS, or the bound left
    // fewer than K keys above it: the one-workgroup algorithm
    select_row(p, q.row, L, dyn);
    return;
  }
  // gather: list r's entries go to s_off[r] onwards (lists in (segment,
  // wave) order: the candidates in ascending position order)
  {
    for (int r0 = wave; r0 < nreg; r0 += kSelWaves * 4) {
      if (r0 != wave) load_batch(v, r0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = r0 + (j >> 1) * kSelWaves, i = lane + (j & 1) * 64;
        if (r < nreg && i < s_off[r + 1] - s_off[r]) {
          ck[s_off[r] + i] = v[j][0];
          cp[s_off[r] + i] = v[j][1];
        }
      }
    }
  }
  __syncthreads();
  // each thread's candidates in registers: entries nv tid .. nv tid + nv - 1
  const int nv = (total + kSelThreads - 1) / kSelThreads;   // entries per thread, at most
  uint32_t rk[kFinPer], rp[kFinPer];
#pragma unroll
  for (int i = 0; i < kFinPer; ++i) {
    const int e = tid * nv + i;
    const bool ok = i < nv && e < total;
    rk[i] = ok ? ck[e] : 0u;
    rp[i] = ok ? cp[e] : 0u;
  }
  auto valid = [&](int i) { return i < nv && tid * nv + i < total; };
  uint32_t thr = 0u, pthr = 0u;
  if (!all) {
    int gt = 0, eq = 0;
    bool found = false;
    if (lb != 0u) {
      // Every candidate is at least lb and the K-th largest lies close
      // above it: two 11-bit passes over y = min(key - lb, 2^22 - 1) find
      // it exactly unless it is 2^22 - 1 or more above lb (then the three
      // passes over whole keys).
      constexpr uint32_t kTop = (1u << 22) - 1u;
      const int shy[2] = {11, 0};
      const uint32_t dmy[2] = {0x7FFu, 0x7FFu};
      const uint32_t y = reg_select<2>(
          [&](int i) {
            const uint32_t dk = rk[i] - lb;
            return dk < kTop ? dk : kTop;
          },
          valid, p.K, 0u, 0u, shy, dmy, h0, h1, L, gt, eq, nv);
      if (y != kTop) {
        thr = lb + y;
        found = true;
      } else {
        for (int i = tid; i < kBins; i += kSelThreads) h0[i] = 0u;
        __syncthreads();
      }
    }
    if (!found) {
      const int shk[3] = {21, 10, 0};
      const uint32_t dmk[3] = {0x7FFu, 0x7FFu, 0x3FFu};
      thr = reg_select<3>([&](int i) { return rk[i]; }, valid, p.K, 0u, 0u, shk, dmk, h0, h1, L,
                          gt, eq, nv);
    }
    const int take = p.K - gt;
    if (take < eq) {
      // equal keys: the lowest positions (largest ~position; positions are
      // below 2^18, so ~position starts with 14 one bits)
      for (int i = tid; i < kBins; i += kSelThreads) h0[i] = 0u;
      __syncthreads();
      int g2, e2;
      const int shp[2] = {7, 0};
      const uint32_t dmp[2] = {0x7FFu, 0x7Fu};
      pthr = reg_select<2>([&](int i) { return rk[i] == thr ? ~rp[i] : 0u; }, valid, take,
                           0xFFFC0000u, 0xFFFC0000u, shp, dmp, h0, h1, L, g2, e2, nv);
    }
  }
  // the chosen entries, already in position order: each thread's go after
  // those of the threads below it; the rest of the row's K slots get -1
  uint32_t chosen = 0u;
#pragma unroll
  for (int i = 0; i < kFinPer; ++i)
    if (valid(i) && (all || rk[i] > thr || (rk[i] == thr && ~rp[i] >= pthr))) chosen |= 1u << i;
  int kept = 0;
  int o = block_exclusive_scan(__popc(chosen), L, kept);
  int32_t* out = p.out + (size_t)q.row * p.K;
#pragma unroll
  for (int i = 0; i < kFinPer; ++i)
    if ((chosen >> i) & 1u) out[o++] = (int32_t)rp[i];
  for (int i = kept + tid; i < p.K; i += kSelThreads) out[i] = -1;
}

}  // namespace

SelectSegPlan select_seg_plan(int64_t rows, int L_max) {
  SelectSegPlan sp;
  if (rows < 1 || L_max > kSelectMapMax) return sp;
  const int64_t steps = (L_max + kSelStep - 1) / kSelStep;
  int64_t want = (kSelSegTargetWgs + rows - 1) / rows;
  if (want > steps) want = steps;
  if (want > 32) want = 32;
  if (want < 2) return sp;
  const int64_t seg_steps = (steps + want - 1) / want;
  sp.seg_len = (int)(seg_steps * kSelStep);
  sp.S = (int)((L_max + sp.seg_len - 1) / sp.seg_len);
  if (sp.S < 2) { sp = SelectSegPlan{}; return sp; }
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += round_up(bytes, 256); return o; };
  sp.cnt_off = take((size_t)rows * 4);          // arrival counters (zeroed once, kept zero)
  sp.cand_off = take((size_t)rows * sp.S * kSelSegWaves * kSelSegCapw * 8);
  sp.ccnt_off = take((size_t)rows * sp.S * kSelSegWaves * 4);
  sp.bytes = off;
  return sp;
}

hipError_t launch_topk_select(const SelectParams& p, hipStream_t s) {
  const size_t dyn = ((size_t)kHistCopies * kBins + p.sel_words +
                      (p.pool ? (size_t)p.pool_words : 0) + (p.S >= 2 ? (size_t)kBins : 0)) * 4;
  static bool attr_set = false;
  if (!attr_set) {
    const int most = (int)((kHistCopies * kBins + kSelectMapMax / 32 + kSelectPoolWords) * 4);
    hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, most);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)seg_select_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, most);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned rows = (unsigned)((size_t)p.B * p.R);
  if (p.S >= 2) {
    const unsigned segs = rows * (unsigned)p.S;
    hipLaunchKernelGGL(seg_select_kernel, dim3(segs), dim3(kSelThreads), dyn, s, p);
  } else {
    hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSelThreads), dyn, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
