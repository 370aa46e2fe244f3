// Dense (MHA / GQA / MQA) and top-k decode attention kernels for gfx950.
//
// What is computed: for each sequence b and query head i with KV head
// j = i / G, softmax(scale * q K^T) V over the positions [0, seq_lens[b])
// (or over the listed positions for top-k) - the "KV cache" guide
// (this.guide), first section and "Fewer KV heads"; the podcast transcript's
// DeepSeek Sparse Attention passage for the listed-position variant.
//
// Work decomposition (same for both kernels): one workgroup of 4 waves per
// (b, j, split), where a split is S consecutive positions (or list slots).
// The G query heads of one KV head share every K/V row the workgroup reads,
// so each cache byte crosses HBM once per step.  Waves keep an online
// softmax (running max, running sum, rescaled accumulators) in log2 units.
// A workgroup merges its waves through LDS; when a sequence needs several
// splits, each writes a normalised partial (o_p, lse_p) to the workspace
// and the last workgroup to finish (a device-scope ticket) merges them by
// log-sum-exp and resets the ticket.

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// ---------------------------------------------------------------------------
// shared epilogue
// ---------------------------------------------------------------------------
template <int D>
struct MergeLds {
  float o[4][kMaxGroup][D];            // per-wave accumulators
  float m[4][kMaxGroup];
  float l[4][kMaxGroup];
  int last;
};

template <typename OutT, int CPT>
__device__ inline void store_row(OutT* dst, const float* o);

template <>
__device__ inline void store_row<uint16_t, 8>(uint16_t* dst, const float* o) {
  u32x4 v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
             pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
  *reinterpret_cast<u32x4*>(dst) = v;
}
template <>
__device__ inline void store_row<uint16_t, 4>(uint16_t* dst, const float* o) {
  uint2 v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  *reinterpret_cast<uint2*>(dst) = v;
}
template <>
__device__ inline void store_row<float, 8>(float* dst, const float* o) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(o[4], o[5], o[6], o[7]);
}
template <>
__device__ inline void store_row<float, 4>(float* dst, const float* o) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
}

// Thread t of the workgroup owns local head t/16 and columns
// (t%16)*D/16 .. +D/16 in every epilogue step.
template <typename OutT, int D>
__device__ inline void write_final(const DenseParams& p, size_t bh,
                                   const float* o, float lse2) {
  constexpr int CPT = D / 16;
  const int c0 = (threadIdx.x & 15) * CPT;
  float os[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) os[c] = o[c] * p.out_scale;
  store_row<OutT, CPT>(reinterpret_cast<OutT*>(p.out) + bh * D + c0, os);
  if (p.lse && (threadIdx.x & 15) == 0) p.lse[bh] = lse2 * kLn2;
}

template <typename OutT, int D>
__device__ void write_empty(const DenseParams& p, int b, int j) {
  constexpr int CPT = D / 16;
  const int hl = threadIdx.x >> 4;
  if (hl >= p.G) return;
  float o[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = 0.f;
  write_final<OutT, D>(p, (size_t)b * p.n_h + j * p.G + hl, o, kNegInf);
}

template <typename OutT, int D>
__device__ void finish_split(const DenseParams& p, int b, int j, int split,
                             int nsplit, MergeLds<D>& L) {
  constexpr int CPT = D / 16;
  const int t = threadIdx.x;
  const int hl = t >> 4;
  const int c0 = (t & 15) * CPT;
  const bool active = hl < p.G;
  const size_t bh = (size_t)b * p.n_h + j * p.G + hl;

  float o[CPT];
  float lse2 = kNegInf;
  if (active) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, L.m[w][hl]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float Z = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = __builtin_amdgcn_exp2f(L.m[w][hl] - Mu);
      Z += e * L.l[w][hl];
#pragma unroll
      for (int c = 0; c < CPT; ++c) o[c] += e * L.o[w][hl][c0 + c];
    }
    const float inv = Z > 0.f ? 1.f / Z : 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] *= inv;
    lse2 = Z > 0.f ? M + __log2f(Z) : kNegInf;
  }

  if (nsplit == 1) {
    if (active) write_final<OutT, D>(p, bh, o, lse2);
    return;
  }

  // Several splits: publish this one (device-coherent stores), then the
  // last workgroup to take a ticket merges all of them.
  const __amdgpu_buffer_rsrc_t wo = make_rsrc(p.ws_o, kWsRecords);
  const __amdgpu_buffer_rsrc_t wl = make_rsrc(p.ws_lse, kWsRecords);
  const size_t slot = bh * p.P_max + split;
  if (active) {
#pragma unroll
    for (int c = 0; c < CPT; c += 4)
      store_coherent(wo, (uint32_t)((slot * D + c0 + c) * 4),
                     f32x4{o[c], o[c + 1], o[c + 2], o[c + 3]});
    if ((t & 15) == 0) store_coherent(wl, (uint32_t)(slot * 4), lse2);
  }
  wait_vm_all();
  __syncthreads();
  int32_t* ticket = p.ws_cnt + (size_t)b * p.n_kv + j;
  if (t == 0) L.last = (atomicAdd(ticket, 1) == nsplit - 1);
  __syncthreads();
  if (!L.last) return;

  // Last workgroup.  Thread row hr (16 rows of 16 threads, CPT columns
  // each) serves head hr / R and takes every R-th split from hr % R, where
  // R = 16 / G rows per head when G divides 16 (else 1).  A thread's lse
  // values and partial rows go out together, eight splits per batch, so a
  // sequence of up to 8 * R splits is merged in one round trip; the R rows
  // of a head are then combined through LDS.
  const int G = p.G;
  const int R = (16 % G == 0) ? 16 / G : 1;
  const int hm = hl / R, sg = hl - hm * R;
  const bool mact = hm < G;
  const size_t bhm = (size_t)b * p.n_h + (size_t)j * G + hm;
  float M = kNegInf, Z = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = 0.f;
  if (mact) {
    const size_t base = bhm * p.P_max;
    for (int s0 = sg; s0 < nsplit; s0 += 8 * R) {
      float lv[8];
      f32x4 v[8][CPT / 4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int su = min(s0 + u * R, nsplit - 1);
        lv[u] = load_coherent1(wl, (uint32_t)((base + su) * 4));
#pragma unroll
        for (int c = 0; c < CPT / 4; ++c)
          v[u][c] = load_coherent4(wo, (uint32_t)(((base + su) * D + c0 + 4 * c) * 4));
      }
      float bm = kNegInf;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u * R < nsplit) bm = fmaxf(bm, lv[u]);
      const float Mn = fmaxf(M, bm);
      const float Mu = (Mn == kNegInf) ? 0.f : Mn;
      const float a = __builtin_amdgcn_exp2f(M - Mu);
      Z *= a;
#pragma unroll
      for (int c = 0; c < CPT; ++c) o[c] *= a;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float e = (s0 + u * R < nsplit) ? __builtin_amdgcn_exp2f(lv[u] - Mu) : 0.f;
        Z += e;
#pragma unroll
        for (int c = 0; c < CPT / 4; ++c)
#pragma unroll
          for (int k = 0; k < 4; ++k) o[4 * c + k] += e * v[u][c][k];
      }
      M = Mn;
    }
  }
  if (R > 1) {
    // (L.o[0] is free: the waves' rows were consumed before the ticket)
    if (mact) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) L.o[0][hl][c0 + c] = o[c];
      if ((t & 15) == 0) {
        L.m[0][hl] = M;
        L.l[0][hl] = Z;
      }
    }
    __syncthreads();
    if (mact && sg == 0) {
      float Mt = kNegInf;
      for (int rr = 0; rr < R; ++rr) Mt = fmaxf(Mt, L.m[0][hl + rr]);
      const float Mu = (Mt == kNegInf) ? 0.f : Mt;
      Z = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) o[c] = 0.f;
      for (int rr = 0; rr < R; ++rr) {
        const float e = __builtin_amdgcn_exp2f(L.m[0][hl + rr] - Mu);
        Z += e * L.l[0][hl + rr];
#pragma unroll
        for (int c = 0; c < CPT; ++c) o[c] += e * L.o[0][hl + rr][c0 + c];
      }
      M = Mt;
    }
  }
  if (mact && sg == 0) {
    const float inv = Z > 0.f ? 1.f / Z : 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] *= inv;
    write_final<OutT, D>(p, bhm, o, Z > 0.f ? M + __log2f(Z) : kNegInf);
  }
  if (t == 0) *ticket = 0;
}

// Length attended by this workgroup.  Plain decode: seq_lens[b] (the caller
// appended already).  Fused append-and-attend: n = seq_lens[b] is the slot
// of the new token and the attended length is n + 1.  With WAIT_WRITE the
// split that owns slot n writes the new K/V row here and waits for it before
// any of its waves reads it back; otherwise (the MFMA kernel) that row is
// never read from the cache: the splits cover the n cached rows, and the
// last of them attends the new row from the k_new/v_new registers and
// stores it to the cache from the same registers.  A full cache
// (n outside [0, L_max)) writes nothing, attends the stored positions and
// sets flag bit 0.
//
// The length itself is bumped once every workgroup of sequence b has read
// the old value: thread 0 of each workgroup arrives on its unit's counter
// (issued here, result checked in complete_length after the main work), the
// last arrival of a unit arrives on the sequence's counter, and the last of
// those writes seq_lens[b] = n + 1.  Every workgroup arrives, including ones
// with no positions.
struct LengthState {
  int n_raw;
  bool ok;
  int unit_prev;   // thread 0: value returned by the unit arrival
};

template <bool APPEND, int D, typename T, bool WAIT_WRITE = true>
__device__ inline int attended_length(const DenseParams& p, int b, int j, int split,
                                      LengthState& ls) {
  // One read; the empty asm keeps the compiler from reading it again later
  // (in the fused kernel the last workgroup of the sequence rewrites it).
  int n_raw = p.seq_lens[b];
  asm volatile("" : "+s"(n_raw));
  if constexpr (!APPEND) {
    return min(max(n_raw, 0), p.L_max);
  } else {
    const bool ok = n_raw >= 0 && n_raw < p.L_max;
    ls.n_raw = n_raw;
    ls.ok = ok;
    ls.unit_prev = 0;
    if (threadIdx.x == 0)
      ls.unit_prev = atomicAdd(p.ws_ucnt + (size_t)b * p.n_kv + j, 1);
    // The writer is the last split of the n_raw + 1 attended rows.  Without
    // WAIT_WRITE the kernel writes the row itself, after its loads are out
    // (a store of data still being loaded would hold back every later load
    // of the wave).
    const int rows = n_raw + 1;
    if (WAIT_WRITE && ok &&
        split == dense_num_splits(rows, dense_split_size(rows, p.S, p.P_max, p.even)) - 1) {
      constexpr int U = D * (int)sizeof(T) / 16;    // 16-byte pieces per row
      const size_t unit = (size_t)b * p.n_kv + j;
      const size_t dst = (unit * p.L_max + n_raw) * U;
      const int t = threadIdx.x;
      if (t < U)
        reinterpret_cast<u32x4*>(p.k)[dst + t] = reinterpret_cast<const u32x4*>(p.k_new)[unit * U + t];
      else if (t < 2 * U)
        reinterpret_cast<u32x4*>(p.v)[dst + t - U] = reinterpret_cast<const u32x4*>(p.v_new)[unit * U + t - U];
      wait_vm_all();
      __syncthreads();
    }
    if (!ok && j == 0 && split == 0 && threadIdx.x == 0 && p.flag) atomicOr(p.flag, 1);
    return ok ? n_raw + 1 : min(max(n_raw, 0), p.L_max);
  }
}

template <bool APPEND>
__device__ inline void complete_length(const DenseParams& p, int b, int j,
                                       const LengthState& ls) {
  if constexpr (APPEND) {
    if (threadIdx.x == 0 && ls.unit_prev == p.P_max - 1) {
      p.ws_ucnt[(size_t)b * p.n_kv + j] = 0;
      if (atomicAdd(p.ws_bcnt + b, 1) == p.n_kv - 1) {
        p.ws_bcnt[b] = 0;
        if (ls.ok) p.seq_lens_rw[b] = ls.n_raw + 1;
      }
    }
  }
}

// Workgroup -> (sequence b, KV head j, split).  Workgroups go to the 8 XCDs
// in turn (workgroup w to XCD w mod 8) and a unit's P_max splits are
// numbered consecutively.  With P_max even, plain numbering puts split s of
// every unit on the XCDs s + P_max * u (mod 8), a few fixed ones: with
// ragged lengths the low splits (present in every sequence) then pile onto
// them.  Measured on the 32-sequence GQA layer: 536 us at 16 splits per
// unit against 347 us at 17.  For even P_max each unit's splits are rotated
// by the unit index, which measured 354 us at 16; for odd P_max the plain
// numbering already spreads them and the rotation measured worse (443 us
// at 17), so it is not applied there.
__device__ inline void decode_unit(const DenseParams& p, int& b, int& j,
                                   int& split) {
  int wg = blockIdx.x;
  const int r = wg % p.P_max;
  wg /= p.P_max;
  split = (p.P_max & 1) ? r : (r + wg) % p.P_max;
  j = wg % p.n_kv;
  b = wg / p.n_kv;
}

// ---------------------------------------------------------------------------
// MFMA kernel: bf16, d = 128, G <= 16.
//
// Per wave and 32-position chunk (lane = 16*g + r):
//  scores  S^T[t][h] = K[t,:] . q[h,:] as two 16x16x32 MFMA tiles x 4 k-steps;
//          A = K rows straight from HBM (lane r reads row pi(a,r), 16 B at
//          column kk*32 + g*8), B = q (16 heads, heads >= G are zero).
//          The row order pi(a, r) = (r/4)*8 + a*4 + r%4 makes the output land
//          as: lane (r, g) holds head r at positions g*8 + 0..7.
//  weights those 8 scores are exactly the B operand of the value product
//          (P[h = r][slot j = position g*8 + j]), after an online softmax.
//  values  O^T[c][h] += V^T[c][t] P^T[t][h]: 8 tiles of 16 columns; lane
//          (r, g) reads rows g*8 + 0..7 at columns r*8..r*8+7 (each load
//          instruction covers 4 whole 256-B rows) and transposes 8x8 bf16 in
//          registers with v_perm so that tile m row r is column r*8 + m.
//  result  lane (r, g) ends with head r, columns 32g .. 32g+31.
// ---------------------------------------------------------------------------
struct Chunk {
  u32x4 k[2][4];
  u32x4 v[8];
  uint32_t vmask;   // top-k: slot g*8+e valid
};

// Loads are issued unconditionally; a chunk past the end of the split
// (cs >= end) gets offsets beyond the buffer, which read zeros without
// touching memory.  Keeping the loads out of branches lets the compiler
// wait for exactly the chunk being computed while the next one is in flight.
__device__ inline void load_chunk(Chunk& c, int cs, int end,
                                  __amdgpu_buffer_rsrc_t kr,
                                  __amdgpu_buffer_rsrc_t vr, int r, int g) {
  constexpr uint32_t kRow = 256;
  {
    const bool live = cs < end;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t row = cs + (r >> 2) * 8 + a * 4 + (r & 3);
      const uint32_t kb = live ? row * kRow + g * 16 : kOobOffset;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        c.k[a][kk] = buf_load16_stream(kr, kb + kk * 64);
    }
    const uint32_t vb = live ? (uint32_t)(cs + g * 8) * kRow + r * 16 : kOobOffset;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      c.v[e] = buf_load16_stream(vr, vb + e * kRow);
    c.vmask = 0xFF;
  }
}

// Top-k: the list entries a chunk needs, loaded one chunk ahead of the rows
// they address (entries past K read as zero and are masked).  Lane (r, g)
// takes the slots of its V rows, cs + g*8 + 0..7, and of its K rows,
// cs + pi(a, r).
// A chunk's list entries as lane group g loads them: slots g*8 .. g*8 + 7
// (the value rows).  The key rows' entries are among them (lane (r, g)
// scores slots (r/4)*8 + 4a + r%4, held by lane group r/4) and are fetched
// across the wave when used.
struct ChunkIdx {
  u32x4 v0, v1;
};

__device__ inline void load_idx(ChunkIdx& x, int cs, __amdgpu_buffer_rsrc_t ir, int r, int g) {
  (void)r;
  x.v0 = buf_load16(ir, (uint32_t)(cs + g * 8) * 4);
  x.v1 = buf_load16(ir, (uint32_t)(cs + g * 8 + 4) * 4);
}

__device__ inline void load_listed(Chunk& c, const ChunkIdx& x, int cs, int end, int n,
                                   __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                   int r, int g, bool& bad) {
  constexpr uint32_t kRow = 256;
  const uint32_t iv[8] = {x.v0[0], x.v0[1], x.v0[2], x.v0[3], x.v1[0], x.v1[1], x.v1[2], x.v1[3]};
  uint32_t mask = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool in_list = cs + g * 8 + e < end;
    const bool ok = iv[e] < (uint32_t)n;
    if (in_list && !ok) bad = true;
    const bool use = in_list && ok;
    mask |= (use ? 1u : 0u) << e;
    c.v[e] = buf_load16_stream(vr, use ? iv[e] * kRow + r * 16 : kOobOffset);
  }
  c.vmask = mask;
  // key entries: each lane offers entry lane % 4 of its group's slice a,
  // and lane (r, g) takes it from lane 16 (r / 4) + r % 4
  const int lane = threadIdx.x & 63;
  const int src = ((r >> 2) * 16 + (r & 3)) * 4;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const u32x4 va = a ? x.v1 : x.v0;
    const uint32_t own = (lane & 2) ? ((lane & 1) ? va[3] : va[2]) : ((lane & 1) ? va[1] : va[0]);
    const uint32_t ka = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)own);
    const int slot = cs + (r >> 2) * 8 + a * 4 + (r & 3);
    const bool use = slot < end && ka < (uint32_t)n;
    const uint32_t kb = use ? ka * kRow + g * 16 : kOobOffset;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) c.k[a][kk] = buf_load16_stream(kr, kb + kk * 64);
  }
}

// Paged cache: the block ids of a chunk's rows, loaded two chunks ahead of
// the rows.  Lane (r, g) needs the blocks of its two K rows (cs + pi(a, r))
// and of its eight V rows (cs + g*8 + 0..7, one block: beta is a multiple of
// 8).  Entries past the table read as zero; rows past the split's end are
// never loaded, so their (possibly unset) entries are not used.
struct PageIdx {
  uint32_t k[2];
  uint32_t v;
};

// (cs is a multiple of 32 and blocks hold at least 8 positions, so a lane's
// two key rows, 4 apart within one aligned group of 8, share a block: one
// table load serves both)
__device__ inline void load_page_idx(PageIdx& x, int cs, __amdgpu_buffer_rsrc_t tr, int shift,
                                     int r, int g) {
  x.k[0] = __builtin_amdgcn_raw_buffer_load_b32(
      tr, (uint32_t)((cs + (r >> 2) * 8) >> shift) * 4, 0, 0);
  x.k[1] = x.k[0];
  x.v = __builtin_amdgcn_raw_buffer_load_b32(tr, (uint32_t)((cs + g * 8) >> shift) * 4, 0, 0);
}

// Rows through the block table (pool rows of 256 bytes: d = 128 bf16).  A
// row in an invalid block is not loaded, its position is masked like an
// unlisted top-k slot (vmask) and `bad` is set.
__device__ inline void load_paged(Chunk& c, const PageIdx& x, int cs, int end,
                                  const DenseParams& p, int j, __amdgpu_buffer_rsrc_t kr,
                                  __amdgpu_buffer_rsrc_t vr, int r, int g, bool& bad) {
  constexpr uint32_t kRow = 256;
  const int shift = p.page_shift;
  const int in_blk = (1 << shift) - 1;
  const uint32_t nb = (uint32_t)p.num_blocks;
  const int t0 = cs + g * 8;
  const bool vok = x.v < nb;
  if (t0 < end && !vok) bad = true;
  const uint32_t vrow = ((x.v * (uint32_t)p.n_kv + j) << shift) + (t0 & in_blk);
  uint32_t mask = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool use = t0 + e < end && vok;
    mask |= (use ? 1u : 0u) << e;
    c.v[e] = buf_load16_stream(vr, use ? (vrow + e) * kRow + r * 16 : kOobOffset);
  }
  c.vmask = mask;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int t = cs + (r >> 2) * 8 + a * 4 + (r & 3);
    const bool use = t < end && x.k[a] < nb;
    const uint32_t krow = ((x.k[a] * (uint32_t)p.n_kv + j) << shift) + (t & in_blk);
    const uint32_t kb = use ? krow * kRow + g * 16 : kOobOffset;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) c.k[a][kk] = buf_load16_stream(kr, kb + kk * 64);
  }
}

// Fused append: the new token's row is attended from k_new/v_new, never
// read back from the cache (whose copy is being written concurrently).  Lane
// (r, g) holds K rows pi(a, r) at columns kk*32 + g*8 and V rows g*8 + e at
// columns r*8; knr/vnr are its 16-byte pieces of the new rows (loaded once),
// placed at chunk row `pos` with selects.
__device__ inline void patch_new_row(Chunk& c, int pos, const u32x4 (&knr)[4],
                                     const u32x4& vnr, int r, int g) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const bool mk = (r >> 2) * 8 + a * 4 + (r & 3) == pos;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) c.k[a][kk][w] = mk ? knr[kk][w] : c.k[a][kk][w];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool mv = g * 8 + e == pos;
#pragma unroll
    for (int w = 0; w < 4; ++w) c.v[e][w] = mv ? vnr[w] : c.v[e][w];
  }
}

struct WaveState {
  float m;        // running max (log2 units), same in the 4 lanes of a head
  float l;        // this lane's share of the running sum
  f32x4 acc[8];   // O^T tiles
};

// F16: the chunk's rows, the query operand and the weights are f16 (bits
// in the same containers) and both products are f16 MFMAs (the FP4 cache
// path, whose rows widen to f16 at half the vector work of bf16); its value
// rows come already arranged as the value product's operands: c.v[m] is
// MFMA m's (word w: rows 2w and 2w + 1 of channel 8r + m).
// scale_log2 is this lane's head's factor (lane r = head r).
template <bool TOPK, bool F16 = false>
__device__ inline void compute_chunk(const Chunk& c, int cs, int end,
                                     const u32x4 (&qop)[4], float scale_log2,
                                     int g, WaveState& st) {
  auto mma = [](u32x4 a, u32x4 b, f32x4 acc) {
    if constexpr (F16)
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), acc, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
  };
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    s0 = mma(c.k[0][kk], qop[kk], s0);
    s1 = mma(c.k[1][kk], qop[kk], s1);
  }
  float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  float mx = kNegInf;
  if (!TOPK && cs + kDenseChunk <= end) {   // (wave-uniform) no row past the end
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] *= scale_log2;
      mx = fmaxf(mx, sv[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bool valid;
      if constexpr (TOPK) valid = (c.vmask >> e) & 1;
      else valid = cs + g * 8 + e < end;
      sv[e] = valid ? sv[e] * scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[e]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // Lazy reference max: move it (and rescale) only when this chunk would
  // push weights above 2^kRescaleMargin.
  const bool move = mx > st.m + kRescaleMargin;
  const float m_new = move ? mx : st.m;
  const float alpha = (move && st.m != kNegInf) ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  st.m = m_new;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] *= alpha;
  }
  uint32_t pp[4];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float w0 = __builtin_amdgcn_exp2f(sv[2 * e] - m_use);
    const float w1 = __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_use);
    if constexpr (F16) {
      const f16x2 h = {(_Float16)w0, (_Float16)w1};
      pp[e] = __builtin_bit_cast(uint32_t, h);
      psum = __builtin_amdgcn_fdot2(h, f16x2{(_Float16)1.f, (_Float16)1.f}, psum, false);
    } else {
      pp[e] = pack_bf16x2(w0, w1);
      psum += bf16_lo(pp[e]) + bf16_hi(pp[e]);
    }
  }
  st.l = st.l * alpha + psum;
  const u32x4 pv = {pp[0], pp[1], pp[2], pp[3]};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    u32x4 a;
    if constexpr (F16) {
      a = c.v[m];
    } else {
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      const int dw = m >> 1;
      a[0] = __builtin_amdgcn_perm(c.v[1][dw], c.v[0][dw], sel);
      a[1] = __builtin_amdgcn_perm(c.v[3][dw], c.v[2][dw], sel);
      a[2] = __builtin_amdgcn_perm(c.v[5][dw], c.v[4][dw], sel);
      a[3] = __builtin_amdgcn_perm(c.v[7][dw], c.v[6][dw], sel);
    }
    st.acc[m] = mma(a, pv, st.acc[m]);
  }
}

// FP8 E4M3 cache (d = 128, 128-byte rows): the same chunk, loaded as raw
// codes and expanded to bf16 (exactly) just before its MFMAs.  The dot
// product's column order is free as long as q uses the same one, so K k-step
// kk, lane group g covers columns (kk/2)*64 + g*16 + (kk%2)*8 .. +7: one
// 16-byte load per (row, kk/2).  V ends in the bf16 layout (8 bytes per
// row and lane) but is loaded 16 bytes at a time: lanes 2k and 2k + 1 load
// channels 16k .. 16k + 15 of rows 2w and 2w + 1 respectively, then swap
// halves (one adjacent-lane move per dword), so each lane ends with its 8
// channels of both rows: half the value load instructions.
struct ChunkF8 {
  u32x4 k[2][2];
  u32x4 v[4];
};

__device__ inline int fp8_q_col(int kk, int g) { return (kk >> 1) * 64 + g * 16 + (kk & 1) * 8; }

__device__ inline void load_chunk(ChunkF8& c, int cs, int end, __amdgpu_buffer_rsrc_t kr,
                                  __amdgpu_buffer_rsrc_t vr, int r, int g) {
  constexpr uint32_t kRow = 128;
  const bool live = cs < end;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const uint32_t row = cs + (r >> 2) * 8 + a * 4 + (r & 3);
    const uint32_t kb = live ? row * kRow + g * 16 : kOobOffset;
#pragma unroll
    for (int h = 0; h < 2; ++h) c.k[a][h] = buf_load16_stream(kr, kb + h * 64);
  }
  const uint32_t vb =
      live ? (uint32_t)(cs + g * 8 + (r & 1)) * kRow + (r >> 1) * 16 : kOobOffset;
#pragma unroll
  for (int w = 0; w < 4; ++w) c.v[w] = buf_load16_stream(vr, vb + 2 * w * kRow);
}

__device__ inline void expand_chunk(const ChunkF8& f, Chunk& c) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 w = f.k[a][kk >> 1];
      const u32x2 h = (kk & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
      c.k[a][kk] = fp8x8_to_bf16x8(h);
    }
  const bool odd = threadIdx.x & 1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4 d = f.v[w];                 // row 2w + odd, channels 16k .. 16k + 15
    const uint32_t s0 = odd ? d[0] : d[2], s1 = odd ? d[1] : d[3];
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, false);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);
    const u32x2 re = odd ? u32x2{t0, t1} : u32x2{d[0], d[1]};   // row 2w, own channels
    const u32x2 ro = odd ? u32x2{d[2], d[3]} : u32x2{t0, t1};   // row 2w + 1
    c.v[2 * w] = fp8x8_to_bf16x8(re);
    c.v[2 * w + 1] = fp8x8_to_bf16x8(ro);
  }
  c.vmask = 0xFF;
}

// FP4 cache (d = 128): rows of 64 code bytes (E2M1, channel 2i in the low
// nibble of byte i) and 8 scale bytes (E4M3, one per 16 channels).  K: lane
// group g loads the 16 code bytes of channels 32g .. 32g + 31, so k-step kk
// covers channels 32g + 8kk .. +7 (q is loaded in that order), and the two
// scale bytes of blocks 2g and 2g + 1.  V ends in the bf16 layout: 4 code
// bytes (channels 8r .. 8r + 7) per row and the scale byte of block r / 2.
// Each stream takes one offset select per chunk; its rows differ by
// immediate offsets (a chunk past the split starts at kOobOffset, past every
// buffer's range, and reads zeros like the rows past the length).
// lane j's value in each quad of lanes (j a constant after unrolling)
__device__ inline uint32_t quad_bcast(int x, int j) {
  switch (j) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xFF, 0xF, 0xF, false);
  }
}

struct ChunkF4 {
  u32x4 k[2];
  uint32_t ks[2];
  u32x2 v[4];       // row 2w + (r & 1), channels 16(r / 2) .. + 15
  uint32_t vs[2];   // scale bytes of rows (r & 3) and 4 + (r & 3), blocks 2(r / 4) .. + 1
};

__device__ inline int fp4_q_col(int kk, int g) { return g * 32 + kk * 8; }

__device__ inline void load_chunk(ChunkF4& c, int cs, int end, __amdgpu_buffer_rsrc_t kr,
                                  __amdgpu_buffer_rsrc_t vr, __amdgpu_buffer_rsrc_t ksr,
                                  __amdgpu_buffer_rsrc_t vsr, int r, int g) {
  constexpr uint32_t kRow = 64, kSRow = 8;
  const bool live = cs < end;
  const uint32_t krow = cs + (r >> 2) * 8 + (r & 3);           // rows krow + 4a
  const uint32_t kb = live ? krow * kRow + g * 16 : kOobOffset;
  const uint32_t ksb = live ? krow * kSRow + g * 2 : kOobOffset;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    c.k[a] = buf_load16_stream(kr, kb + a * 4 * kRow);
    c.ks[a] = __builtin_amdgcn_raw_buffer_load_b16(ksr, ksb + a * 4 * kSRow, 0, kStream);
  }
  const uint32_t row0 = cs + g * 8;                           // rows row0 + e
  // value codes 8 bytes at a time: lanes 2k and 2k + 1 load the 16
  // channels they share of rows 2w and 2w + 1 (swapped into place when
  // widened); value scales 2 bytes at a time: lane 4k + i loads the two
  // blocks its quad shares (2k, 2k + 1) of rows i and 4 + i (broadcast
  // within the quad when widened): 6 value load instructions instead of 16
  const uint32_t vb = live ? (row0 + (r & 1)) * kRow + (r >> 1) * 8 : kOobOffset;
  const uint32_t vsb = live ? (row0 + (r & 3)) * kSRow + (r >> 2) * 2 : kOobOffset;
#pragma unroll
  for (int w = 0; w < 4; ++w) c.v[w] = buf_load8_stream(vr, vb + 2 * w * kRow);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    c.vs[h] = __builtin_amdgcn_raw_buffer_load_b16(vsr, vsb + 4 * h * kSRow, 0, kStream);
}

// Widened to f16 (exactly) for the f16 products; the scales two at a time
// (blocks 2g and 2g + 1 of a K row; the block of V rows e and e + 1).  K as
// fp4x8_to_f16x8 gives it.  V straight into the value product's operand
// layout: the codes of rows 2w and 2w + 1 are first interleaved by nibble
// (byte k of x: channel 2k of each row; of y: channel 2k + 1), so that one
// conversion gives the pair (row 2w, row 2w + 1) of one channel, and one
// packed multiply applies the two rows' scales.
__device__ inline void expand_chunk(const ChunkF4& f, Chunk& c) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const f16x2 s = e4m3x2_to_f16x2(f.ks[a]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) c.k[a][kk] = fp4x8_to_f16x8(f.k[a][kk], kk < 2 ? s[0] : s[1]);
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // this lane's channels of rows 2w and 2w + 1 (one adjacent-lane swap)
    const bool odd = threadIdx.x & 1;
    // rows 2w and 2w + 1 come from quad lanes (2w) % 4 and (2w + 1) % 4;
    // this lane's block is byte (r / 2) % 2 of each
    const int vsrc = (int)f.vs[w >> 1];
    const uint32_t sa = quad_bcast(vsrc, (2 * w) & 3);
    const uint32_t sb = quad_bcast(vsrc, (2 * w + 1) & 3);
    const uint32_t bsel = (threadIdx.x >> 1) & 1;
    const f16x2 s =
        e4m3x2_to_f16x2(__builtin_amdgcn_perm(sb, sa, 0x0C0C0000u | bsel | ((4u + bsel) << 8)));
    const u32x2 d = f.v[w];
    const uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? d[0] : d[1]), 0xB1, 0xF, 0xF,
                                                          false);
    const uint32_t r0 = odd ? t : d[0], r1 = odd ? d[1] : t;
    const uint32_t x = (r0 & 0x0F0F0F0Fu) | ((r1 << 4) & 0xF0F0F0F0u);
    const uint32_t y = ((r0 >> 4) & 0x0F0F0F0Fu) | (r1 & 0xF0F0F0F0u);
    const u32x4 ev = fp4x8_to_f16x8(x, s), od = fp4x8_to_f16x8(y, s);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c.v[2 * k][w] = ev[k];
      c.v[2 * k + 1][w] = od[k];
    }
  }
  c.vmask = 0xFF;
}

template <bool FP8, bool FP4> struct ChunkOf { using T = Chunk; };
template <> struct ChunkOf<true, false> { using T = ChunkF8; };
template <> struct ChunkOf<false, true> { using T = ChunkF4; };

// Persistent form: thread 0 takes the next item index from the device
// counter right before the split merge (whose round trips hide the
// atomic's) and leaves it in LDS; nothing is held through the main loop.
struct NextItem {
  int32_t* counter;   // null: one item per workgroup
  int base;
  int* slot;          // LDS
};

__device__ inline int fetch_next_begin(const NextItem& nx) {
  return (nx.counter && threadIdx.x == 0) ? nx.base + atomicAdd(nx.counter, 1) : 0;
}
__device__ inline void fetch_next_end(const NextItem& nx, int v) {
  if (nx.counter && threadIdx.x == 0) *nx.slot = v;
}

// One item of the MFMA kernels: (sequence b, KV head j, split) once the
// attended length n is known (for the fused call also the length state);
// for top-k the first two chunks' list entries are already in flight in I0
// and I1.  Ends after the split merge; the caller owns the length bump.
//
// LAZY_NEW (persistent form): the new row of a fused append is attended by
// split 0 instead of the last split, and its pieces are loaded only after
// split 0's main loop, so they hold no registers through it.  (Split 0 is
// drawn early, so the extra round trip stays off the end of the launch; the
// one-workgroup-per-split form keeps them prefetched in the last, shortest
// split, where a launch of one round waits for its slowest split.)
template <bool TOPK, bool APPEND, bool FP8, bool PAGED, bool FP4, bool LAZY_NEW = false>
__device__ __forceinline__ void dense_mfma_item(const DenseParams& p, int b, int j, int split,
                                                int n, const LengthState& ls, MergeLds<128>& L,
                                                ChunkIdx& I0, ChunkIdx& I1, const NextItem& nx) {
  static_assert(!FP8 || (!TOPK && !APPEND), "FP8 caches: plain decode only");
  static_assert(!PAGED || (!TOPK && !APPEND && !FP8), "paged caches: plain decode only");
  static_assert(!FP4 || (!TOPK && !APPEND && !FP8 && !PAGED), "FP4 caches: plain decode only");
  const int lo = TOPK ? 0 : window_low(p, b, n);    // window mode only (not fused)
  // Fused append: the new row (slot n - 1) is attended from registers, so
  // the splits cover only the rows already in the cache.  A sequence of 4096
  // cached rows then splits into whole 256-row pieces instead of spilling a
  // one-row chunk into an extra load round.
  const bool reg_new = APPEND && ls.ok;
  const int count = TOPK ? p.K : n - lo - (reg_new ? 1 : 0);
  const int S = dense_split_size(count, p.S, p.P_max, p.even);
  const int nsplit = dense_num_splits(count, S);
  if (split >= nsplit || (count == 0 && !reg_new)) {
    const int nxt = fetch_next_begin(nx);
    if (split == 0) write_empty<uint16_t, 128>(p, b, j);
    fetch_next_end(nx, nxt);
    return;
  }
  int start, end;
  dense_split_range(count, S, split, start, end);
  start += lo;
  end += lo;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const size_t unit = (size_t)b * p.n_kv + j;
  constexpr uint32_t kRowBytes = FP4 ? 64u : FP8 ? 128u : 256u;
  const size_t unit_bytes = (size_t)p.L_max * kRowBytes;
  // (paged: the whole pool, at most 2^31 bytes, checked on the host)
  const uint32_t pool_bytes =
      PAGED ? ((uint32_t)p.num_blocks * (uint32_t)p.n_kv << p.page_shift) * kRowBytes : 0u;
  // Rows a load may touch: the attended ones, less the new row of a fused
  // append (slot n - 1 is never read back; rows past the range read zeros).
  // (read-first-lane: a select on the length state may land in a vector
  // register, and a buffer range in one makes each load a read-first-lane
  // loop)
  const uint32_t n_rows = (uint32_t)__builtin_amdgcn_readfirstlane(n - (reg_new ? 1 : 0));
  const __amdgpu_buffer_rsrc_t kr =
      PAGED ? make_rsrc(p.k, pool_bytes)
            : make_rsrc((const char*)p.k + unit * unit_bytes, n_rows * kRowBytes);
  const __amdgpu_buffer_rsrc_t vr =
      PAGED ? make_rsrc(p.v, pool_bytes)
            : make_rsrc((const char*)p.v + unit * unit_bytes, n_rows * kRowBytes);
  // (FP4: the scale rows, 8 bytes per position)
  const __amdgpu_buffer_rsrc_t ksr =
      FP4 ? make_rsrc((const char*)p.k_scales + unit * (size_t)p.L_max * 8, (uint32_t)n * 8u) : kr;
  const __amdgpu_buffer_rsrc_t vsr =
      FP4 ? make_rsrc((const char*)p.v_scales + unit * (size_t)p.L_max * 8, (uint32_t)n * 8u) : kr;
  const __amdgpu_buffer_rsrc_t ir =
      TOPK ? make_rsrc(p.idx + unit * p.K, (uint32_t)p.K * 4u)
           : PAGED ? make_rsrc(p.block_table + (size_t)b * p.max_blocks, (uint32_t)p.max_blocks * 4u)
                   : kr;

  u32x4 qop[4];
  if (r < p.G) {
    const uint16_t* qrow =
        (const uint16_t*)p.q + ((size_t)b * p.n_h + j * p.G + r) * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qop[kk] = *reinterpret_cast<const u32x4*>(
          qrow + (FP4 ? fp4_q_col(kk, g) : FP8 ? fp8_q_col(kk, g) : kk * 32 + g * 8));
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qop[kk] = u32x4{0u, 0u, 0u, 0u};
  }
  // The FP4 path's f16 products take the query as f16: head r's row times
  // 2^a with a = 14 - (exponent of its largest magnitude), so that the
  // largest lies in [2^14, 2^15) and every bf16 component not 2^29 below it
  // converts exactly; the head's score factor takes 2^-a back (exact).
  float scale_log2 = p.scale_log2;
  if constexpr (FP4) {
    float qm = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        qm = fmaxf(qm, fmaxf(fabsf(bf16_lo(qop[kk][w])), fabsf(bf16_hi(qop[kk][w]))));
    qm = fmaxf(qm, __shfl_xor(qm, 16));
    qm = fmaxf(qm, __shfl_xor(qm, 32));
    int sh = qm > 0.f ? 14 - ((int)((__float_as_uint(qm) >> 23) & 0xFF) - 127) : 0;
    sh = sh < -126 ? -126 : (sh > 126 ? 126 : sh);
    const float up = __uint_as_float((uint32_t)(127 + sh) << 23);
    scale_log2 *= __uint_as_float((uint32_t)(127 - sh) << 23);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f16x2 h = {(_Float16)(bf16_lo(qop[kk][w]) * up), (_Float16)(bf16_hi(qop[kk][w]) * up)};
        qop[kk][w] = __builtin_bit_cast(uint32_t, h);
      }
  }

  WaveState st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool bad = false;
  int cs = start + wave * kDenseChunk;
  constexpr int kStride = kDenseChunk * 4;
  // fused append: slot of the new row (or -1), and its source rows
  const int new_slot = (APPEND && ls.ok) ? ls.n_raw : -1;
  u32x4 knr[4], vnr;
  const u32x4* kn = reinterpret_cast<const u32x4*>(p.k_new) + unit * 16;
  const u32x4* vn = reinterpret_cast<const u32x4*>(p.v_new) + unit * 16;
  if constexpr (APPEND && !LAZY_NEW) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) knr[kk] = kn[kk * 4 + g];
    vnr = vn[r];
  }
  using Raw = typename ChunkOf<FP8, FP4>::T;
  auto load = [&](Raw& c, int at) {
    if constexpr (FP4) load_chunk(c, at, end, kr, vr, ksr, vsr, r, g);
    else load_chunk(c, at, end, kr, vr, r, g);
  };
  auto compute = [&](Raw& c, int at) {
    if constexpr (FP4) {
      Chunk x;
      expand_chunk(c, x);
      compute_chunk<false, true>(x, at, end, qop, scale_log2, g, st);
    } else if constexpr (FP8) {
      Chunk x;
      expand_chunk(c, x);
      compute_chunk<false>(x, at, end, qop, p.scale_log2, g, st);
    } else {
      compute_chunk<TOPK || PAGED>(c, at, end, qop, p.scale_log2, g, st);
    }
  };
  if constexpr (TOPK) {
    if (cs < end) {
      // list entries two chunks ahead (the first two loaded at the start),
      // rows one chunk ahead
      Chunk A, Bc;
      load_listed(A, I0, cs, end, n, kr, vr, r, g, bad);
      while (true) {
        load_idx(I0, cs + 2 * kStride, ir, r, g);
        load_listed(Bc, I1, cs + kStride, end, n, kr, vr, r, g, bad);
        __builtin_amdgcn_sched_barrier(0);
        compute(A, cs);
        cs += kStride;
        if (cs >= end) break;
        load_idx(I1, cs + 2 * kStride, ir, r, g);
        load_listed(A, I0, cs + kStride, end, n, kr, vr, r, g, bad);
        __builtin_amdgcn_sched_barrier(0);
        compute(Bc, cs);
        cs += kStride;
        if (cs >= end) break;
      }
    }
  } else if constexpr (PAGED) {
    if (cs < end) {
      // block ids two chunks ahead, rows one chunk ahead
      Chunk A, Bc;
      PageIdx I0, I1;
      load_page_idx(I0, cs, ir, p.page_shift, r, g);
      load_page_idx(I1, cs + kStride, ir, p.page_shift, r, g);
      load_paged(A, I0, cs, end, p, j, kr, vr, r, g, bad);
      while (true) {
        load_page_idx(I0, cs + 2 * kStride, ir, p.page_shift, r, g);
        load_paged(Bc, I1, cs + kStride, end, p, j, kr, vr, r, g, bad);
        __builtin_amdgcn_sched_barrier(0);
        compute(A, cs);
        cs += kStride;
        if (cs >= end) break;
        load_page_idx(I1, cs + 2 * kStride, ir, p.page_shift, r, g);
        load_paged(A, I0, cs + kStride, end, p, j, kr, vr, r, g, bad);
        __builtin_amdgcn_sched_barrier(0);
        compute(Bc, cs);
        cs += kStride;
        if (cs >= end) break;
      }
    }
  } else if (cs < end) {
    // The split's chunks are visited from a rotated start (chunk `rot`,
    // wrapping round), a hash of the item: workgroups that start together
    // would otherwise stream their splits in step, at the same offsets
    // from split starts that are multiples of the split size, and measured
    // about half the bandwidth of ones out of step (the first round
    // of 2048-row items of a 32-sequence GQA layer: 106 us against 50 us).  Wave w takes the chunks w,
    // w + 4, ... of the visiting order; a chunk past the split reads zeros.
    const int nch = (end - start + kDenseChunk - 1) / kDenseChunk;
    const int rot = (int)((((uint32_t)unit * 0x9E3779B1u) ^ ((uint32_t)split * 0x85EBCA77u)) >> 16) % nch;
    auto at = [&](int i) {
      int c = wave + 4 * i;
      if (c >= nch) return end;
      c += rot;
      if (c >= nch) c -= nch;
      return start + c * kDenseChunk;
    };
    Raw A, Bc;
    int i = 0;
    load(A, at(0));
    while (true) {
      load(Bc, at(i + 1));
      __builtin_amdgcn_sched_barrier(0);   // the next chunk's loads go out first
      compute(A, at(i));
      if (wave + 4 * ++i >= nch) break;
      load(A, at(i + 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(Bc, at(i));
      if (wave + 4 * ++i >= nch) break;
    }
  }
  if constexpr (APPEND) {
    // The last split (split 0 with LAZY_NEW) folds in the new row as a
    // one-row chunk, on the wave with the fewest cached chunks (wave 3 when
    // they are even), and that wave writes the row to the cache: lanes r = 0
    // hold all 16 pieces of the K row, lanes g = 0 all 16 of the V row.
    const int chunks = (end - start + kDenseChunk - 1) / kDenseChunk;
    const int new_wave = (chunks & 3) ? (chunks & 3) : 3;
    if (new_slot >= 0 && split == (LAZY_NEW ? 0 : nsplit - 1) && wave == new_wave) {
      if constexpr (LAZY_NEW) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) knr[kk] = kn[kk * 4 + g];
        vnr = vn[r];
      }
      const size_t dst = (unit * p.L_max + new_slot) * 16;
      if (r == 0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) reinterpret_cast<u32x4*>(p.k)[dst + kk * 4 + g] = knr[kk];
      }
      if (g == 0) reinterpret_cast<u32x4*>(p.v)[dst + r] = vnr;
      Chunk c;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c.k[a][kk] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) c.v[e] = u32x4{0u, 0u, 0u, 0u};
      c.vmask = 0xFF;
      patch_new_row(c, 0, knr, vnr, r, g);
      compute_chunk<false>(c, new_slot, new_slot + 1, qop, p.scale_log2, g, st);
    }
  }
  if constexpr (TOPK || PAGED) {
    if (p.flag && __any(bad) && lane == 0) atomicOr(p.flag, 2);
  }

  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (g == 0) {
    L.m[wave][r] = st.m;
    L.l[wave][r] = l_tot;
  }
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) L.o[wave][r][(4 * g + i) * 8 + m] = st.acc[m][i];
  __syncthreads();
  const int nxt = fetch_next_begin(nx);
  finish_split<uint16_t, 128>(p, b, j, split, nsplit, L);
  fetch_next_end(nx, nxt);
}

// One workgroup per (sequence, KV head, split of the longest possible
// length); splits past a sequence's length write nothing (split 0 of an
// empty sequence writes the zero row).
template <bool TOPK, bool APPEND, bool FP8 = false, bool PAGED = false, bool FP4 = false>
__global__ __launch_bounds__(256, 2) void dense_mfma_kernel(DenseParams p) {
  __shared__ MergeLds<128> L;
  int b, j, split;
  decode_unit(p, b, j, split);
  // Top-k: a split's slots and the list do not depend on the sequence
  // length, so the list entries of the first two chunks go out before the
  // length is read (the two round trips overlap).
  ChunkIdx I0, I1;
  if constexpr (TOPK) {
    const int St = dense_split_size(p.K, p.S, p.P_max, p.even);
    const int l0 = threadIdx.x & 63;
    const int cs0 = split * St + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kDenseChunk;
    const __amdgpu_buffer_rsrc_t ir0 =
        make_rsrc(p.idx + ((size_t)b * p.n_kv + j) * p.K, (uint32_t)p.K * 4u);
    load_idx(I0, cs0, ir0, l0 & 15, l0 >> 4);
    load_idx(I1, cs0 + kDenseChunk * 4, ir0, l0 & 15, l0 >> 4);
  }
  LengthState ls;
  const int n = attended_length<APPEND, 128, uint16_t, false>(p, b, j, split, ls);
  dense_mfma_item<TOPK, APPEND, FP8, PAGED, FP4>(p, b, j, split, n, ls, L, I0, I1,
                                                 NextItem{nullptr, 0, nullptr});
  // (after the merge: its atomic is off the path to the output)
  complete_length<APPEND>(p, b, j, ls);
}

// ---------------------------------------------------------------------------
// Persistent form for large problems (fixed split size S): a grid of about
// two workgroups per compute unit, each taking (sequence, KV head, split)
// items from a device counter until none are left.
//
// Each workgroup first reads every sequence's length (and window start)
// into LDS and derives the item list from them: all units' whole splits of
// S positions first, then every unit's last, shorter split (or its one
// empty item), those in four classes by length, longest first, so the items
// drawn last are the shortest and the final workgroups finish close
// together.  Against one workgroup per (unit,
// split) of the longest possible length, no workgroup is launched for a
// split past its sequence's length, the length is read once per workgroup
// instead of once per item, and the fused call needs no arrival counters:
// every workgroup reads the lengths before it takes its first item and
// counts itself done after its last, so the workgroup that counts last
// (a device-scope counter) knows that every workgroup has read the old
// lengths, writes the new ones and resets the counters.  No workgroup
// waits for another, so correctness does not depend on how many workgroups
// are resident at once.
// ---------------------------------------------------------------------------
__device__ inline int last_at_or_below(const int* a, int n, int k) {
  // largest u in [0, n) with a[u] <= k (a non-decreasing, a[0] <= k)
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// The same over 16-bit field q of packed prefixes.
__device__ inline int last_at_or_below16(const uint64_t* a, int n, int q, int k) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int)((a[mid] >> (16 * q)) & 0xFFFF) <= k) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// Length class of a unit's last item: 3 for a remainder of at least 3S/4
// down to 0 for one under S/4 (and the empty item); -1: no last item.
__device__ inline int last_class(int c, int S) {
  const int rem = c % S;
  if (rem == 0) return c == 0 ? 0 : -1;
  return (int)(((int64_t)rem * 4) / S);
}

template <bool APPEND, bool FP8 = false, bool PAGED = false, bool FP4 = false>
__global__ __launch_bounds__(256, 2) void dense_persist_kernel(DenseParams p) {
  __shared__ MergeLds<128> L;
  __shared__ int s_nraw[kPersistMaxB];          // lengths as read
  __shared__ int s_cnt[kPersistMaxB];           // positions the splits of a unit cover
  __shared__ int s_full[kPersistMaxUnits + 1];  // exclusive prefix over units: whole splits
  // exclusive prefixes over units of the last items of each length class,
  // 16 bits per class
  __shared__ uint64_t s_part[kPersistMaxUnits + 1];
  __shared__ uint32_t s_scan[256];
  __shared__ uint64_t s_scan4[256];
  __shared__ int s_next;

  const int tid = threadIdx.x;
  const int B = p.B, n_kv = p.n_kv, units = p.B * p.n_kv, S = p.S;
  for (int b = tid; b < B; b += 256) {
    const int n_raw = p.seq_lens[b];
    int count;
    if constexpr (APPEND) {
      // the new row is attended from registers: the splits cover the cached rows
      count = (n_raw >= 0 && n_raw < p.L_max) ? n_raw : min(max(n_raw, 0), p.L_max);
    } else {
      const int n = min(max(n_raw, 0), p.L_max);
      count = n - window_low(p, b, n);
    }
    s_nraw[b] = n_raw;
    s_cnt[b] = count;
  }
  __syncthreads();
  // per unit: count / S whole splits and one last item (a shorter split, or
  // the empty item of a unit with nothing cached) in one of four length
  // classes; exclusive prefix sums, each thread a run of units (whole splits
  // in 32 bits; the class counts, at most 2048 each, in 16-bit fields)
  const int per = (units + 255) / 256;
  const int u0 = min(tid * per, units), u1 = min(u0 + per, units);
  uint32_t whole = 0;
  uint64_t packed = 0;
  for (int u = u0; u < u1; ++u) {
    const int c = s_cnt[u / n_kv];
    whole += (uint32_t)(c / S);
    const int q = last_class(c, S);
    if (q >= 0) packed += 1ull << (16 * q);
  }
  s_scan[tid] = whole;
  s_scan4[tid] = packed;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t x = tid >= off ? s_scan[tid - off] : 0u;
    const uint64_t x4 = tid >= off ? s_scan4[tid - off] : 0ull;
    __syncthreads();
    s_scan[tid] += x;
    s_scan4[tid] += x4;
    __syncthreads();
  }
  {
    int sf = tid ? (int)s_scan[tid - 1] : 0;
    uint64_t sp = tid ? s_scan4[tid - 1] : 0ull;
    for (int u = u0; u < u1; ++u) {
      const int c = s_cnt[u / n_kv];
      s_full[u] = sf;
      s_part[u] = sp;
      sf += c / S;
      const int q = last_class(c, S);
      if (q >= 0) sp += 1ull << (16 * q);
    }
    if (tid == 0) {
      s_full[units] = (int)s_scan[255];
      s_part[units] = s_scan4[255];
    }
  }
  __syncthreads();
  const int total_full = s_full[units];
  const uint64_t cls = s_part[units];
  const int n3 = (int)((cls >> 48) & 0xFFFF), n2 = (int)((cls >> 32) & 0xFFFF);
  const int n1 = (int)((cls >> 16) & 0xFFFF), n0 = (int)(cls & 0xFFFF);
  const int total = total_full + n3 + n2 + n1 + n0;

  ChunkIdx I0, I1;    // (top-k only; unused here)
  int k = blockIdx.x;
  const NextItem nx{p.ws_sched, (int)gridDim.x, &s_next};
  // (an unsigned test: a counter left non-zero by a workspace that was not
  // zero-filled for this call's layout gives wrong results, never an item
  // index outside the list)
  while ((unsigned)k < (unsigned)total) {
    int u, split;
    if (k < total_full) {
      u = last_at_or_below(s_full, units, k);
      split = k - s_full[u];
    } else {
      // last items, longest class first
      int r = k - total_full, q = 3;
      if (r >= n3) { r -= n3; q = 2;
        if (r >= n2) { r -= n2; q = 1;
          if (r >= n1) { r -= n1; q = 0; } } }
      u = last_at_or_below16(s_part, units, q, r);
      split = s_cnt[u / n_kv] / S;
    }
    u = __builtin_amdgcn_readfirstlane(u);
    split = __builtin_amdgcn_readfirstlane(split);
    const int b = u / n_kv, j = u - b * n_kv;
    // (uniform values: a length in a vector register would make every
    // buffer descriptor divergent, and each load a read-first-lane loop)
    LengthState ls;
    ls.n_raw = __builtin_amdgcn_readfirstlane(s_nraw[b]);
    ls.ok = ls.n_raw >= 0 && ls.n_raw < p.L_max;
    ls.unit_prev = 0;
    int n;
    if constexpr (APPEND) {
      n = ls.ok ? ls.n_raw + 1 : min(max(ls.n_raw, 0), p.L_max);
      if (!ls.ok && j == 0 && split == 0 && tid == 0 && p.flag) atomicOr(p.flag, 1);
    } else {
      n = min(max(ls.n_raw, 0), p.L_max);
    }
    n = __builtin_amdgcn_readfirstlane(n);
    dense_mfma_item<false, APPEND, FP8, PAGED, FP4, true>(p, b, j, split, n, ls, L, I0, I1, nx);
    __syncthreads();
    k = __builtin_amdgcn_readfirstlane(s_next);
    __syncthreads();   // every wave has read s_next before thread 0 writes it again
  }
  // Done: the workgroup that counts last writes the new lengths (fused
  // call) and resets the counters for the next call.
  if (tid == 0) s_next = atomicAdd(p.ws_sched + 1, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (s_next) {
    if constexpr (APPEND) {
      for (int b = tid; b < B; b += 256) {
        const int n_raw = s_nraw[b];
        if (n_raw >= 0 && n_raw < p.L_max) p.seq_lens_rw[b] = n_raw + 1;
      }
    }
    if (tid == 0) {
      p.ws_sched[0] = 0;
      p.ws_sched[1] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic VALU kernel: float32 or bf16, d in {64, 128}, G <= 16.
// Lane = position for the scores; lane = column for the weighted sum, with
// each position's weight broadcast by readlane.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float ld_f32(const T* p);
template <>
__device__ inline float ld_f32<float>(const float* p) { return *p; }
template <>
__device__ inline float ld_f32<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// Eight consecutive elements as float32.
__device__ inline void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ inline void load8(const uint16_t* p, float (&x)[8]) {
  const u32x4 k = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(k[e]);
    x[2 * e + 1] = bf16_hi(k[e]);
  }
}

template <typename T, int D, bool TOPK, bool APPEND>
__global__ __launch_bounds__(256) void dense_generic_kernel(DenseParams p) {
  __shared__ MergeLds<D> L;
  __shared__ float sq[kMaxGroup][D];
  int b, j, split;
  decode_unit(p, b, j, split);
  LengthState ls;
  const int n = attended_length<APPEND, D, T>(p, b, j, split, ls);
  const int lo = TOPK ? 0 : window_low(p, b, n);    // window mode only (not fused)
  const int count = TOPK ? p.K : n - lo;
  const int S = dense_split_size(count, p.S, p.P_max, p.even);
  const int nsplit = dense_num_splits(count, S);
  if (split >= nsplit || count == 0) {
    if (split == 0) write_empty<T, D>(p, b, j);
    complete_length<APPEND>(p, b, j, ls);
    return;
  }
  int start, end;
  dense_split_range(count, S, split, start, end);
  start += lo;
  end += lo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;

  const T* qg = (const T*)p.q + ((size_t)b * p.n_h + j * G) * D;
  for (int e = tid; e < G * D; e += 256) sq[e / D][e % D] = ld_f32<T>(qg + e);
  __syncthreads();

  const size_t unit = (size_t)b * p.n_kv + j;
  const T* kb = (const T*)p.k + unit * p.L_max * D;
  const T* vb = (const T*)p.v + unit * p.L_max * D;
  constexpr int U = D / 64;

  float m_run[kMaxGroup], l_run[kMaxGroup], o[kMaxGroup][U];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) o[h][u] = 0.f;
  }

  bool bad = false;
  for (int blk = start + wave * 64; blk < end; blk += 256) {
    const int slot = blk + lane;
    bool valid = slot < end;
    int row = slot;
    if constexpr (TOPK) {
      row = valid ? p.idx[unit * p.K + slot] : 0;
      const bool ok = (unsigned)row < (unsigned)n;
      if (valid && !ok) bad = true;
      valid = valid && ok;
    }
    float s[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) s[h] = 0.f;
    if (valid) {
      const T* krow = kb + (size_t)row * D;
#pragma unroll 2
      for (int d0 = 0; d0 < D; d0 += 8) {
        float kv[8];
        load8(krow + d0, kv);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h >= G) continue;
#pragma unroll
          for (int e = 0; e < 8; ++e) s[h] += sq[h][d0 + e] * kv[e];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      s[h] = (valid && h < G) ? s[h] * p.scale_log2 : kNegInf;
    float pw[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) { pw[h] = 0.f; continue; }
      const float mx = wave_max(s[h]);
      const bool move = mx > m_run[h] + kRescaleMargin;
      const float m_new = move ? mx : m_run[h];
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = (move && m_run[h] != kNegInf) ? __builtin_amdgcn_exp2f(m_run[h] - m_new) : 1.f;
      pw[h] = __builtin_amdgcn_exp2f(s[h] - m_use);
      l_run[h] = l_run[h] * alpha + wave_sum(pw[h]);
      m_run[h] = m_new;
#pragma unroll
      for (int u = 0; u < U; ++u) o[h][u] *= alpha;
    }
    // Value rows eight at a time, all eight loads in flight before the
    // multiply-adds (one row per position serialised each load's latency).
    // A slot past the block or not attended loads the split's first row (or
    // row 0 for top-k, which the allocation always holds) and is skipped.
    const int nrows = min(64, end - blk);
    const int safe = TOPK ? 0 : start;
    for (int t0 = 0; t0 < nrows; t0 += 8) {
      float v[8][U];
      bool ok[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = min(t0 + e, nrows - 1);
        ok[e] = t0 + e < nrows && __builtin_amdgcn_readlane((int)valid, tt) != 0;
        const int rt = ok[e] ? __builtin_amdgcn_readlane(row, tt) : safe;
        const T* vrow = vb + (size_t)rt * D;
#pragma unroll
        for (int u = 0; u < U; ++u) v[e][u] = ld_f32<T>(vrow + lane + 64 * u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!ok[e]) continue;
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h >= G) continue;
          const float pt =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw[h]), t0 + e));
#pragma unroll
          for (int u = 0; u < U; ++u) o[h][u] += pt * v[e][u];
        }
      }
    }
  }
  if constexpr (TOPK) {
    if (p.flag && __any(bad) && lane == 0) atomicOr(p.flag, 2);
  }

#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) continue;
    if (lane == 0) {
      L.m[wave][h] = m_run[h];
      L.l[wave][h] = l_run[h];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) L.o[wave][h][lane + 64 * u] = o[h][u];
  }
  __syncthreads();
  finish_split<T, D>(p, b, j, split, nsplit, L);
  // (after the merge: its atomic is off the path to the output)
  complete_length<APPEND>(p, b, j, ls);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static dim3 dense_grid(const DenseParams& p) {
  return dim3((unsigned)((size_t)p.B * p.n_kv * p.P_max));
}

// Persistent grid: two workgroups per compute unit (the kernels'
// occupancy), never more than there can be items.
static dim3 persist_grid(const DenseParams& p) {
  const size_t most = (size_t)p.B * p.n_kv * p.P_max;
  const size_t g = (size_t)kPersistWgs < most ? (size_t)kPersistWgs : most;
  return dim3((unsigned)g);
}

template <bool APPEND, bool FP8, bool PAGED, bool FP4>
static void launch_mfma_t(const DenseParams& p, hipStream_t s) {
  if (p.persist)
    hipLaunchKernelGGL((dense_persist_kernel<APPEND, FP8, PAGED, FP4>), persist_grid(p), dim3(256),
                       0, s, p);
  else
    hipLaunchKernelGGL((dense_mfma_kernel<false, APPEND, FP8, PAGED, FP4>), dense_grid(p),
                       dim3(256), 0, s, p);
}

hipError_t launch_dense_mfma(const DenseParams& p, bool topk, bool append, hipStream_t s) {
  if (topk)
    hipLaunchKernelGGL((dense_mfma_kernel<true, false>), dense_grid(p), dim3(256), 0, s, p);
  else if (append)
    launch_mfma_t<true, false, false, false>(p, s);
  else
    launch_mfma_t<false, false, false, false>(p, s);
  return hipGetLastError();
}

hipError_t launch_dense_paged(const DenseParams& p, hipStream_t s) {
  launch_mfma_t<false, false, true, false>(p, s);
  return hipGetLastError();
}

hipError_t launch_dense_fp8(const DenseParams& p, hipStream_t s) {
  launch_mfma_t<false, true, false, false>(p, s);
  return hipGetLastError();
}

hipError_t launch_dense_fp4(const DenseParams& p, hipStream_t s) {
  launch_mfma_t<false, false, false, true>(p, s);
  return hipGetLastError();
}

template <typename T, int D>
static void launch_generic_t(const DenseParams& p, bool topk, bool append, hipStream_t s) {
  if (topk)
    hipLaunchKernelGGL((dense_generic_kernel<T, D, true, false>), dense_grid(p), dim3(256), 0, s, p);
  else if (append)
    hipLaunchKernelGGL((dense_generic_kernel<T, D, false, true>), dense_grid(p), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((dense_generic_kernel<T, D, false, false>), dense_grid(p), dim3(256), 0, s, p);
}

hipError_t launch_dense_generic(const DenseParams& p, int dtype, bool topk,
                                bool append, hipStream_t s) {
  const bool bf = dtype == 1;
  if (p.d == 64) {
    if (bf) launch_generic_t<uint16_t, 64>(p, topk, append, s);
    else launch_generic_t<float, 64>(p, topk, append, s);
  } else {
    if (bf) launch_generic_t<uint16_t, 128>(p, topk, append, s);
    else launch_generic_t<float, 128>(p, topk, append, s);
  }
  return hipGetLastError();
}

}  // namespace kvc
