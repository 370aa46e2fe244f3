// Decode attention over a latent (MLA) cache for gfx950.
//
// What is computed ("KV cache" guide, this.guide, "Caching a compressed
// latent" and the memory footnote): with the key up-projection folded into
// the query, head i scores position t as
//     s = scale * (<q_lat[i], c[t]> + <q_rope[i], k_rope[t]>)
// against the cached row c[t] || k_rope[t] (512 + 64 wide), and the output
// is the softmax-weighted sum of the latents c[t] (512 wide).
//
// This is the one place in decode attention where the contraction is really
// dense: every head reads the same 1152-byte row, so a row carries
// n_h * (576 + 512) multiply-adds.  One workgroup covers 128 heads (64 when
// n_h is not a multiple of 128) of one (sequence, split): every compute unit
// streams rows no other compute unit reads.  Each wave owns 32 heads with the
// full row (no exchange between waves) and runs alone on its SIMD with the
// whole register file: 256 accumulators, 144 query registers (the whole
// 576-wide query of its 32 heads stays in registers).
//
// Per wave (lane l: r = l % 32, g = l / 32) and 32-position chunk, with
// v_mfma_f32_32x32x16_bf16:
//  scores  S^T[t][h], 36 k-steps: A = latent rows from LDS (lane row r is
//          position pi(r), r with bits 2 and 3 swapped; columns 16ks + 8g ..
//          +8), B = the 32 heads' queries in registers.  The row order makes
//          accumulator i of lane (r, g) hold head r at position
//          16(i / 8) + 8g + i % 8, i.e. the B operand of the value product.
//  weights softmax numerators 2^(s - m_ref) in log2 units against a fixed
//          per-head reference (see the pass loop below).
//  values  O^T[c][h] += C^T[c][t] P^T[t][h]: 16 column tiles x 2 k-steps.
//          The A operand (8 positions of one column per lane) is read from
//          LDS already transposed by ds_read_b64_tr_b16 (in each 16-lane
//          group, lane i receives element i % 4 of the 8-byte pieces
//          addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4), two
//          reads per MFMA.  The addressing makes row m of tile ct column
//          32ct + 16((m / 4) % 2) + 4(m / 8) + m % 4, so accumulator k of lane
//          (r, g) holds head r at column 32ct + 16g + k: 16 consecutive
//          columns per lane and tile.  These reads are issued from inline
//          assembly with explicit LDS counter waits: through the builtin the
//          compiler, lacking alias information, would wait for every tile
//          copy in flight before each of them.
//
// Latent tiles go HBM -> LDS directly (buffer_load ... lds), four stages
// (three tiles in flight while one is read), with 16-byte piece k of row rho stored
// at k ^ key(rho), key = bit-reverse of (rho >> 1) & 7: conflict-free for
// the 16-byte score and value reads on the 64-bank LDS.  Rows at or past the sequence length read as zeros (buffer range
// check) and are masked.  Splits of one sequence publish normalised partials
// and a second kernel, spread over every compute unit, merges them by
// log-sum-exp.

#include <utility>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kD = kMlaDc + kMlaDr;          // 576
constexpr int kRowB = kD * 2;                // 1152 bytes per row
constexpr int kTileB = kMlaChunk * kRowB;    // 36864 bytes per chunk
constexpr int kStages = 4;
constexpr int kKSteps = kD / 16;             // 36
constexpr int kColTiles = kMlaDc / 32;       // 16
// The last kQPark query k-steps may wait in LDS (per wave and lane, 1 KB per
// k-step) if the wave would not fit the register file; the four stages leave
// room for at most 3.
constexpr int kQPark = 0;
constexpr int kQRegs = kKSteps - kQPark;
constexpr size_t kParkOff = (size_t)kStages * kTileB;
constexpr size_t kMlaLds = kParkOff + 4 * kQPark * 1024;
// Weights may reach 2^kMlaRefMargin against the reference (bf16 and fp32
// hold that with room to spare: 8193 * 2^64 * |c| stays far below 2^128).
constexpr float kMlaRefMargin = 64.0f;
// LDS reads in flight ahead of the MFMA that consumes them (hides the LDS
// latency behind earlier MFMAs of the same wave).
constexpr int kQkAhead = 4;
// Value product: 32 MFMAs per chunk (k-step J / 16, column tile J % 16); the
// two transposed reads of each are issued kPvAhead MFMAs ahead into one of
// kPvBuf register pairs (one more than in flight, so a read never targets
// the registers of the MFMA issued just before it).
constexpr int kPvSteps = 2 * kColTiles;
constexpr int kPvAhead = 4;
constexpr int kPvBuf = kPvAhead + 1;

typedef __attribute__((address_space(3))) void lds_void;

__device__ constexpr int swz_key(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}

__device__ constexpr int pi_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Copy one tile (32 rows from position cs) into a stage: load k of this wave
// fills LDS byte (blk0 + k)*1024 + lane*16, i.e. row rho, physical piece pc,
// which holds logical piece pc ^ key(rho).
template <int NB>
__device__ inline void issue_tile(char* stage, __amdgpu_buffer_rsrc_t cr, int cs,
                                  int blk0, int lane) {
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int byte = (blk0 + k) * 1024 + lane * 16;
    const int rho = byte / kRowB;
    const int pc = (byte - rho * kRowB) >> 4;
    const uint32_t goff = (uint32_t)(rho * kRowB + ((pc ^ swz_key(rho)) << 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        cr, (lds_void*)(stage + (blk0 + k) * 1024), 16, goff, cs * kRowB, 0, kStream);
  }
}

// One 1-KB block of a tile (block index blk of the 36).
__device__ inline void issue_block(char* stage, __amdgpu_buffer_rsrc_t cr, int cs,
                                   int blk, int lane) {
  const int byte = blk * 1024 + lane * 16;
  const int rho = byte / kRowB;
  const int pc = (byte - rho * kRowB) >> 4;
  const uint32_t goff = (uint32_t)(rho * kRowB + ((pc ^ swz_key(rho)) << 4));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      cr, (lds_void*)(stage + blk * 1024), 16, goff, cs * kRowB, 0, kStream);
}

__device__ inline u32x4 lds_load16(const char* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}


// s_waitcnt vmcnt(N) for N < 64 (gfx9 encoding: vmcnt bits 3:0 and 15:14;
// expcnt and lgkmcnt left at maximum).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, then s_barrier.  __syncthreads() would also drain the vector
// memory counter, i.e. wait for the tiles still being prefetched into LDS.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Any of the NW waves' votes set (slots of the waves of this workgroup only).
template <int NW>
__device__ inline bool any_vote(const int* v) {
  int x = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) x |= v[w];
  return x != 0;
}


template <int NW>
__device__ inline bool any_vote4(u32x4 v) {
  uint32_t x = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) x |= v[w];
  return x != 0;
}

// Transposed reads of value MFMA J: tile ct = J % 16, k-step J / 16 (16 rows
// further), bases tb[half][ct % 2] plus 128 (ct / 2) bytes.
template <int J>
__device__ __forceinline__ void pv_issue(u32x2 (&lo)[kPvBuf], u32x2 (&hi)[kPvBuf],
                                         const uint32_t (&tb)[2][2]) {
  constexpr int ct = J % kColTiles;
  constexpr int off = (J / kColTiles) * 16 * kRowB + 128 * (ct >> 1);
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
               : "=v"(lo[J % kPvBuf]) : "v"(tb[0][ct & 1]), "n"(off));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
               : "=v"(hi[J % kPvBuf]) : "v"(tb[1][ct & 1]), "n"(off));
}

// Value MFMA J: wait until its two reads have landed (LDS operations complete
// in order, so at most the reads issued after them may still be pending;
// the wait is tied to the registers so the MFMA cannot move above it), then
// accumulate and issue the reads kPvAhead MFMAs ahead.
template <int J>
__device__ __forceinline__ void pv_step(f32x16 (&acc)[kColTiles], const bf16x8 (&pop)[2],
                                        u32x2 (&lo)[kPvBuf], u32x2 (&hi)[kPvBuf],
                                        const uint32_t (&tb)[2][2]) {
  constexpr int later = (kPvSteps - 1 - J) < (kPvAhead - 1) ? (kPvSteps - 1 - J) : (kPvAhead - 1);
  asm volatile("s_waitcnt lgkmcnt(%2)"
               : "+v"(lo[J % kPvBuf]), "+v"(hi[J % kPvBuf]) : "n"(2 * later));
  const u32x4 a = {lo[J % kPvBuf][0], lo[J % kPvBuf][1], hi[J % kPvBuf][0], hi[J % kPvBuf][1]};
  acc[J % kColTiles] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      as_bf16x8(a), pop[J / kColTiles], acc[J % kColTiles], 0, 0, 0);
  if constexpr (J + kPvAhead < kPvSteps) pv_issue<J + kPvAhead>(lo, hi, tb);
  __builtin_amdgcn_sched_barrier(0);
}

template <int... Js>
__device__ __forceinline__ void pv_head(std::integer_sequence<int, Js...>, u32x2 (&lo)[kPvBuf],
                                        u32x2 (&hi)[kPvBuf], const uint32_t (&tb)[2][2]) {
  (pv_issue<Js>(lo, hi, tb), ...);
}

// Value MFMA J, then (J = 0, 2, .., 10) piece J / 2 of the softmax's
// remaining vector work, which issues while the matrix unit is busy.
template <int J, class F>
__device__ __forceinline__ void pv_step_w(f32x16 (&acc)[kColTiles], const bf16x8 (&pop)[2],
                                          u32x2 (&lo)[kPvBuf], u32x2 (&hi)[kPvBuf],
                                          const uint32_t (&tb)[2][2], F&& w) {
  pv_step<J>(acc, pop, lo, hi, tb);
  if constexpr (J <= 10 && J % 2 == 0) {
    w(J / 2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// (pieces 1..4 complete pop[1] before MFMA kColTiles, the first to read it)
template <int... Js, class F>
__device__ __forceinline__ void pv_all(std::integer_sequence<int, Js...>,
                                       f32x16 (&acc)[kColTiles], const bf16x8 (&pop)[2],
                                       u32x2 (&lo)[kPvBuf], u32x2 (&hi)[kPvBuf],
                                       const uint32_t (&tb)[2][2], F&& w) {
  static_assert(kColTiles > 10, "pop[1] is complete before its first reader");
  (pv_step_w<Js>(acc, pop, lo, hi, tb, w), ...);
}

}  // namespace

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void mla_kernel(MlaParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ __attribute__((aligned(16))) int s_vote[2][4];         // per chunk parity: wave needs a restart
  constexpr int kHpw = 32 * NW;        // heads per workgroup
  constexpr int kLpt = 36 / NW;        // 1-KB blocks each wave copies per tile

  // Block id -> (sequence b, split, head group).  Consecutive block ids go
  // to the 8 XCDs in turn.  When B is a multiple of 8, every block of
  // sequence b runs on XCD b % 8, so the splits of a sequence share one L2
  // (its query comes from HBM once, and the merge kernel finds the partials
  // there); otherwise that would give some XCDs one more sequence than
  // others (B = 12: twice the work on half of them), so blocks are numbered
  // plainly and every sequence spreads over the XCDs.
  const int groups = p.n_h / kHpw;
  int id = blockIdx.x;
  int b, split, hg;
  if ((p.B & 7) == 0) {
    const int xcd = id & 7;
    id >>= 3;
    hg = id % groups;
    id /= groups;
    split = id % p.P_max;
    b = (id / p.P_max) * 8 + xcd;
  } else {
    hg = id % groups;
    id /= groups;
    split = id % p.P_max;
    b = id / p.P_max;
  }
  if (b >= p.B) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, g = lane >> 5;
  const int h = hg * kHpw + wave * 32 + r;
  const size_t bh = (size_t)b * p.n_h + h;

  const int n = min(max(p.seq_lens[b], 0), p.L_max);
  const int start = split * p.S;
  if (start >= n) {
    if (split == 0) {
      // nothing to attend: zero row, lse = -inf
      uint16_t* o = (uint16_t*)p.out + bh * kMlaDc;
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int c = g * 8; c < kMlaDc; c += 16) *reinterpret_cast<u32x4*>(o + c) = z;
      if (p.lse && g == 0) p.lse[bh] = kNegInf;
    }
    return;
  }
  const int end = min(n, start + p.S);
  const int nsplit = (n + p.S - 1) / p.S;
  const int nchunks = (end - start + kMlaChunk - 1) / kMlaChunk;

  const __amdgpu_buffer_rsrc_t cr = make_rsrc(
      (const char*)p.ckv + (size_t)b * p.L_max * kRowB, (uint32_t)n * kRowB);

  const int blk0 = wave * kLpt;

  // LDS read bases (within a stage).
  // Scores, k-step ks: row pi(r), logical piece 2ks + g, stored at
  // 8(ks / 4) + ((2(ks % 4) + g) ^ key): base by ks % 4, plus 128(ks / 4).
  uint32_t wqk[4];
  {
    const int row = pi_row(r);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      wqk[m] = (uint32_t)(row * kRowB + (((2 * m + g) ^ swz_key(row)) << 4));
  }
  // Values, k-step s2, half t, column tile ct: lane L = lane % 16 of 16-lane
  // group q16 (g = q16 / 2) addresses row 16 s2 + 8g + 4t + L / 4, columns
  // 32ct + 16(L % 2) + 8(q16 % 2) + 4((L / 2) % 2) .. +4, i.e. logical piece
  // 4ct + 2(L % 2) + q16 % 2, half (L / 2) % 2.  The key does not depend on
  // s2 and only flips piece bits 0..2: base by (t, ct % 2), plus 16 s2 rows
  // and 128 (ct / 2) bytes.
  // (the reads are issued from inline assembly, which takes the LDS byte
  // address itself: the low 32 bits of the generic address of smem)
  uint32_t wtr[2][2];
  {
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    const int q16 = lane >> 4, L = lane & 15;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 8 * g + 4 * t + (L >> 2);
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        wtr[t][cp] = lds0 + (uint32_t)(row * kRowB +
                                (((4 * cp + 2 * (L & 1) + (q16 & 1)) ^ swz_key(row)) << 4) +
                                8 * ((L >> 1) & 1));
    }
  }

  // The first two tiles go out right after the query loads, so the two
  // latencies overlap; the query loads come first so that waiting for a tile
  // also covers them.  Tiles 2 and 3 follow during the first chunk's scores:
  // with every workgroup starting at once, a smaller first burst lets the
  // first tile (and the query) land sooner.
  auto issue_first = [&]() {
    issue_tile<kLpt>(smem, cr, start, blk0, lane);
    if (nchunks > 1) issue_tile<kLpt>(smem + kTileB, cr, start + kMlaChunk, blk0, lane);
  };

  bf16x8 qop[kQRegs];
  const uint32_t qpark = (uint32_t)(kParkOff + (wave * kQPark * 64 + lane) * 16);
  {
    const uint16_t* qrow = (const uint16_t*)p.q + bh * kD;
#pragma unroll
    for (int k = 0; k < kQRegs; ++k)
      qop[k] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + k * 16 + g * 8));
#pragma unroll
    for (int k = kQRegs; k < kKSteps; ++k)
      *reinterpret_cast<u32x4*>(smem + qpark + (k - kQRegs) * 1024) =
          *reinterpret_cast<const u32x4*>(qrow + k * 16 + g * 8);
  }
  issue_first();

  // Scores of one chunk (stage offset toff).  The LDS reads run kQkAhead
  // k-steps ahead of the MFMAs; the scheduling barriers keep that order.
  // The copy of a later tile (when dma) is issued one block every NW
  // k-steps (kLpt = 36 / NW blocks per wave): each block occupies the address unit for a while, and spread
  // out its issue hides behind the MFMAs instead of stalling the wave.
  auto scores = [&](uint32_t toff, bool dma, char* dstage, int dcs, bool dma2) {
    uint32_t qb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qb[m] = toff + wqk[m];
      asm volatile("" : "+v"(qb[m]));
    }
    // The scores accumulate in vector registers (the accumulation registers
    // all hold the value product), so the chain is written as inline
    // assembly with a VGPR accumulator: back-to-back accumulation into the
    // same registers needs no wait states.
    f32x16 s;
    // A: latent rows; Bq: parked query k-steps (k >= kQRegs)
    u32x4 A[kQkAhead], Bq[kQkAhead];
#pragma unroll
    for (int k = 0; k < kQkAhead; ++k) {
      A[k] = lds_load16(smem, qb[k & 3] + (k >> 2) * 128);
      if (k >= kQRegs) Bq[k] = lds_load16(smem, qpark + (k - kQRegs) * 1024);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      const bf16x8 bop = k < kQRegs ? qop[k < kQRegs ? k : 0] : as_bf16x8(Bq[k % kQkAhead]);
      const bf16x8 aop = as_bf16x8(A[k % kQkAhead]);
      if (k == 0)
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(aop), "v"(bop));
      else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(aop), "v"(bop));
      if (dma2) {
        // two tiles (the first chunk): all of the first before any of the
        // second, so that the in-order vector memory counter waits below
        // still mean "these tiles landed"
        constexpr int h = NW / 2;
        if (k % h == h - 1)
          issue_block(dstage + (k < kKSteps / 2 ? 0 : kTileB), cr,
                      dcs + (k < kKSteps / 2 ? 0 : kMlaChunk), blk0 + (k % (kKSteps / 2)) / h, lane);
      } else if (k % NW == 1 && dma) {
        issue_block(dstage, cr, dcs, blk0 + k / NW, lane);
      }
      const int kn = k + kQkAhead;
      if (kn < kKSteps) {
        A[k % kQkAhead] = lds_load16(smem, qb[kn & 3] + (kn >> 2) * 128);
        if (kn >= kQRegs) Bq[k % kQkAhead] = lds_load16(smem, qpark + (kn - kQRegs) * 1024);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // vector ALU reads of the chain's result need 11 wait states after an
    // 8-pass matrix instruction; give 21
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s));
    return s;
  };

  f32x16 acc[kColTiles];
  float m_ref = kNegInf, l_run = 0.f;
  const float scale_log2 = p.scale_log2;

  // The pass over the split's chunks.  Weights are 2^(s - m_ref) against a
  // reference fixed by the head's first valid chunk, so the accumulators are
  // never rescaled.  A later score more than kMlaRefMargin above it (never
  // with ordinary data: 2^64) makes the whole workgroup drop the pass, scan
  // the split once for each head's largest score (scores only), and
  // accumulate again against that without further votes: at most three
  // passes.
  bool scan = false, scanned = false, first_pass = true;
  for (;;) {
#pragma unroll
    for (int m = 0; m < kColTiles; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
    l_run = 0.f;
    if (!first_pass) issue_first();
    first_pass = false;
    // (tiles 2 and 3 are issued during the scores of chunk 0, tile k >= 4
    // during those of chunk k - 3, into the stage of chunk k - 4)

    float m_seen = m_ref;     // largest score of this head in this pass
    bool restart = false;
    for (int c = 0; c < nchunks; ++c) {
      const int cs = start + c * kMlaChunk;
      // Tile c landed (tiles issued after it: c + 1 and c + 2, only c + 1 on
      // the first chunk, may still be in flight); every wave is done with the
      // stage of chunk c - 1 and has cast its vote on it.
      const int after = c == 0 ? min(1, nchunks - 1) : min(kStages - 2, nchunks - 1 - c);
      if (after >= 3) wait_vmcnt<3 * kLpt>();
      else if (after == 2) wait_vmcnt<2 * kLpt>();
      else if (after == 1) wait_vmcnt<kLpt>();
      else wait_vmcnt<0>();
      lds_barrier();
      // (the votes on chunk c - 1 are read here and tested after this
      // chunk's scores, so the read's latency hides behind the MFMAs)
      const u32x4 vw = *reinterpret_cast<const u32x4*>(s_vote[(c - 1) & 1]);
      const uint32_t toff = (uint32_t)((c % kStages) * kTileB);
      const bool first = c == 0;
      const f32x16 S = scores(toff, first ? nchunks > 2 : c + kStages - 1 < nchunks,
                              smem + ((first ? 2 : c + kStages - 1) % kStages) * kTileB,
                              cs + (first ? 2 : kStages - 1) * kMlaChunk, first && nchunks > 3);
      if (c > 0 && !scan && !scanned && any_vote4<NW>(vw)) { restart = true; break; }

      // weights of this lane's 16 positions of head r
      float sv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = S[i] * scale_log2;
      if (cs + kMlaChunk > end) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (cs + 16 * (i >> 3) + 8 * g + (i & 7) >= end) sv[i] = kNegInf;
      }
      // This lane's max over its 16 positions.  The two lanes of a head
      // (g = 0, 1) agree on the reference only through the first valid
      // chunk's exchange; afterwards each tests its own half against it, so
      // no cross-lane (LDS-pipe) operation sits in the steady-state loop.
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[i]);
      m_seen = fmaxf(m_seen, mx);
      if (scan) continue;

      // the first value MFMAs' reads go out ahead of the rest of the softmax
      // (only on a pass that uses them: a read left in flight into registers
      // the compiler takes as free could overwrite them)
      uint32_t tb[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
          tb[t][cp] = toff + wtr[t][cp];
          asm volatile("" : "+v"(tb[t][cp]));
        }
      u32x2 trlo[kPvBuf], trhi[kPvBuf];
      pv_head(std::make_integer_sequence<int, kPvAhead>{}, trlo, trhi, tb);

      if (__builtin_amdgcn_readfirstlane(__float_as_int(m_ref)) == __float_as_int(kNegInf)) {
        // first valid chunk (nothing accumulated yet); the empty asm keeps
        // the exchange inside this branch
        asm volatile("" ::: "memory");
        m_ref = fmaxf(mx, __shfl_xor(mx, 32));
      }
      const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
      // Weights of this lane's positions of k-step s2 of the value product,
      // in pairs.  Only k-step 0's are computed before the value product;
      // the rest of the softmax's vector work (k-step 1's weights, the sums
      // of the rounded weights in order, the vote) issues between k-step
      // 0's matrix instructions, which read only pop[0].
      bf16x8 pop[2];
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float psum = 0.f;
      uint32_t pp[2][4];
      auto weights = [&](int s2, int e) {
        pp[s2][e] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[8 * s2 + 2 * e] - m_use),
                                __builtin_amdgcn_exp2f(sv[8 * s2 + 2 * e + 1] - m_use));
        if (e == 3) {
          const u32x4 pv = {pp[s2][0], pp[s2][1], pp[s2][2], pp[s2][3]};
          pop[s2] = as_bf16x8(pv);
        }
      };
      auto sums = [&](int s2) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp[s2][e]), ones, psum,
                                                 false);
      };
#pragma unroll
      for (int e = 0; e < 4; ++e) weights(0, e);

      // weighted sum of the latents of chunk c
      __builtin_amdgcn_sched_barrier(0);
      pv_all(std::make_integer_sequence<int, kPvSteps>{}, acc, pop, trlo, trhi, tb,
             [&](int step) {
               if (step == 0) {
                 sums(0);
               } else if (step <= 4) {
                 weights(1, step - 1);
               } else {
                 sums(1);
                 // (every lane writes the wave's vote; a score this far
                 // above the reference may overflow the weights, and the
                 // vote discards the pass)
                 const int vote = __any(mx > m_ref + kMlaRefMargin) ? 1 : 0;
                 s_vote[c & 1][wave] = vote;
               }
             });
      l_run += psum;      // the rounded weights' sum (bf16 dot with ones)
    }
    if (scan) {
      scan = false;
      scanned = true;
      m_ref = fmaxf(m_seen, __shfl_xor(m_seen, 32));
    } else {
      if (!restart && !scanned) {
        // votes on the last chunk
        lds_barrier();
        restart = any_vote<NW>(s_vote[(nchunks - 1) & 1]);
      }
      if (!restart) break;
      scan = true;
    }
    // Start again: let every tile copy of this pass land before the stages
    // are refilled.
    wait_vmcnt<0>();
    lds_barrier();
  }

  // This split's result for head h: lane (r, g) holds column 32ct + 16g + k
  // in acc[ct][k].
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_ref + __log2f(l_tot) : kNegInf;

  if (nsplit == 1) {
    uint16_t* o = (uint16_t*)p.out + bh * kMlaDc;
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = pack_bf16x2(acc[ct][8 * hf + 2 * e] * inv, acc[ct][8 * hf + 2 * e + 1] * inv);
        *reinterpret_cast<u32x4*>(o + 32 * ct + 16 * g + 8 * hf) = v;
      }
    if (p.lse && g == 0) p.lse[bh] = lse2 * kLn2;
    return;
  }

  // Several splits: publish this one; mla_merge_kernel (launched next on
  // the same stream, so the kernel boundary makes the stores visible to every
  // XCD) combines them.  The normalised partial is stored in bf16 (one more
  // rounding of the same size as the output's; the merge sums in float32),
  // which halves the partial traffic both ways.  A split's partial block is
  // in register order: slot k of lane l of wave w (k = 4 * tile + quad, 64
  // slots of 4 values) is at ((w * 64 + k) * 64 + l) * 4 values, so every
  // store moves 512 bytes contiguous per wave.
  {
    const size_t unit_hg = (size_t)b * groups + hg;
    constexpr size_t kBlock = (size_t)NW * 64 * 256;     // values per split block
    u32x2* blk = reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.ws_o) +
                                          (unit_hg * p.P_max + split) * kBlock) +
                 wave * 64 * 64 + lane;
#pragma unroll
    for (int t = 0; t < kColTiles; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        blk[(4 * t + q4) * 64] = u32x2{pack_bf16x2(acc[t][4 * q4] * inv, acc[t][4 * q4 + 1] * inv),
                                       pack_bf16x2(acc[t][4 * q4 + 2] * inv, acc[t][4 * q4 + 3] * inv)};
    if (g == 0) p.ws_lse[(unit_hg * p.P_max + split) * kHpw + wave * 32 + r] = lse2;
  }
}

// Split merge: one workgroup (NW waves, the main kernel's lane layout) per
// (sequence, head group, tile pair tp).  Every lane combines the same 8 slots
// (tiles 2tp and 2tp + 1, quads 0..3) of all the splits' blocks by
// log-sum-exp weights, with the loads of up to 4 splits in flight together.
// Sequences that needed one split (or none) were finished by the main kernel.
// (Register budget for two waves per SIMD, so that all 32 slot loads of a
// batch stay in flight together.)
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void mla_merge_kernel(MlaParams p) {
  constexpr int kHpw = 32 * NW;
  constexpr size_t kBlock = (size_t)NW * 64 * 256;
  const int groups = p.n_h / kHpw;
  int id = blockIdx.x;
  const int xcd = id & 7;     // sequence b runs on XCD b % 8, as in the main kernel
  id >>= 3;
  const int part = id & 7;    // tile pair: tiles 2 part, 2 part + 1
  id >>= 3;
  const int hg = id % groups;
  const int b = (id / groups) * 8 + xcd;
  if (b >= p.B) return;
  const int n = min(max(p.seq_lens[b], 0), p.L_max);
  const int nsplit = (n + p.S - 1) / p.S;
  if (nsplit <= 1) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, g = lane >> 5;
  const int h = hg * kHpw + wave * 32 + r;
  const size_t bh = (size_t)b * p.n_h + h;
  const size_t unit_hg = (size_t)b * groups + hg;

  // Two round trips for 4 splits: the partial lse values (8 at a time, for
  // the max), then each batch of 4 splits' slots with their lse.
  const float* lse_p = p.ws_lse + unit_hg * p.P_max * kHpw + wave * 32 + r;
  float M = kNegInf;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = lse_p[(size_t)min(s0 + u, nsplit - 1) * kHpw];
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, t[u]);
  }
  const float Mu = (M == kNegInf) ? 0.f : M;

  const u32x2* base = reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(p.ws_o) +
                                                     unit_hg * p.P_max * kBlock) +
                      wave * 64 * 64 + lane;
  f32x4 sum[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) sum[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float Z = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 4) {
    u32x2 v[4][8];
    float ls[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int su = min(s0 + u, nsplit - 1);
      ls[u] = lse_p[(size_t)su * kHpw];
      const u32x2* blk = base + (size_t)su * (kBlock / 4);
#pragma unroll
      for (int m = 0; m < 8; ++m) v[u][m] = blk[(8 * part + m) * 64];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = (s0 + u >= nsplit || ls[u] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ls[u] - Mu);
      Z += w;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        sum[m] += w * f32x4{bf16_lo(v[u][m][0]), bf16_hi(v[u][m][0]),
                            bf16_lo(v[u][m][1]), bf16_hi(v[u][m][1])};
    }
  }
  const float zi = Z > 0.f ? 1.f / Z : 0.f;
  // slot m = 4tt + q4 (tile 2 part + tt, quad q4) element e is column
  // 32(2 part + tt) + 16g + 4q4 + e: eight consecutive columns per pair of
  // slots
  uint16_t* orow = (uint16_t*)p.out + bh * kMlaDc;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      o[e] = pack_bf16x2(sum[2 * j][2 * e] * zi, sum[2 * j][2 * e + 1] * zi);
      o[2 + e] = pack_bf16x2(sum[2 * j + 1][2 * e] * zi, sum[2 * j + 1][2 * e + 1] * zi);
    }
    *reinterpret_cast<u32x4*>(orow + 64 * part + 32 * (j >> 1) + 16 * g + 8 * (j & 1)) = o;
  }
  if (part == 0 && p.lse && g == 0) p.lse[bh] = Z > 0.f ? (M + __log2f(Z)) * kLn2 : kNegInf;
}

template <int NW>
static hipError_t launch_mla_t(const MlaParams& p, hipStream_t s) {
  const int groups = p.n_h / (32 * NW);
  const size_t bq = ((size_t)p.B + 7) / 8;     // sequences per XCD
  const size_t blocks = 8 * bq * p.P_max * groups;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_kernel<NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMlaLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(mla_kernel<NW>, dim3((unsigned)blocks), dim3(NW * 64), kMlaLds, s, p);
  if (p.P_max > 1)
    hipLaunchKernelGGL(mla_merge_kernel<NW>, dim3((unsigned)(8 * bq * groups * 8)),
                       dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mla(const MlaParams& p, hipStream_t s) {
  return mla_heads_per_wg(p.n_h) == 128 ? launch_mla_t<4>(p, s) : launch_mla_t<2>(p, s);
}

}  // namespace kvc
