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
// n_h * (576 + 512) multiply-adds.  A workgroup of 8 waves (two per SIMD)
// owns 64 heads for one split of the positions; the workgroups of all head
// groups of one (sequence, split) are numbered so they land on the same XCD
// and stream the same rows at the same time, so L2 serves the repeats.
//
// Waves 2p and 2p+1 share heads 16p..16p+15.  Wave half h (0 or 1) computes
// the score contribution of row columns [288h, 288h+288) and, after the two
// halves are added through LDS, the output columns [256h, 256h+256).  Per
// wave (lane l: r = l % 16, g = l / 16) and 32-position chunk:
//  scores  S^T[t][hd]: 2 tiles x 9 k-steps of v_mfma_f32_16x16x32_bf16;
//          A = latent tile rows from LDS (tile a, lane row r is position
//          pi(a, r) = (r/4)*8 + 4a + r%4, columns 32kk + 8g .. +8), B = the
//          16 heads' queries held in registers for the whole split.  The row
//          order makes lane (r, g) receive head r at positions g*8 + 0..7.
//  weights both waves of a pair run the same online softmax (log2 units) on
//          the summed scores; a lane's 8 weights are the B operand of the
//          value product.
//  values  O^T[c][hd] += C^T[c][t] P^T[t][hd]: 16 tiles of 16 columns; lane
//          (r, g) reads rows g*8 + 0..7 x 16 B at columns 256h + 128cg + 8r
//          and transposes 8x8 bf16 in registers (v_perm), so tile (cg, m)
//          row r is column 256h + 128cg + 8r + m.
//
// Latent tiles go HBM -> LDS directly (buffer_load ... lds), three chunks
// deep, with 16-byte chunk k of row rho stored at k ^ key(rho),
// key(rho) = ((rho >> 1) & 1) | (((rho >> 3) & 3) << 1).  The row stride
// (1152 B) puts consecutive rows half a bank set apart on the 64-bank LDS;
// this key gives the 16 lanes of an LDS cycle 16 distinct bank groups in both
// read patterns.  Rows at or past the sequence length read as zeros (buffer
// range check) and are masked.  Splits of one sequence are merged by
// log-sum-exp by the last workgroup to finish.

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kD = kMlaDc + kMlaDr;          // 576
constexpr int kRowB = kD * 2;                // 1152 bytes per row
constexpr int kTileB = kMlaChunk * kRowB;    // 36864 bytes per chunk
constexpr int kStages = 3;
constexpr int kKHalf = kD / 32 / 2;          // 9 k-steps (of 32) per wave
constexpr int kThreads = kMlaWaves * 64;
constexpr int kXsBytes = kMlaWaves * 2 * 64 * 16;          // score exchange
constexpr size_t kMlaLds = (size_t)kStages * kTileB + kXsBytes;

typedef __attribute__((address_space(3))) void lds_void;

__device__ constexpr int swz_key(int row) {
  return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
}

// Waves 0-3 copy five 1-KB blocks of a tile, waves 4-7 four (36 in all).
__device__ constexpr int first_block(int wave) { return wave < 4 ? 5 * wave : 20 + 4 * (wave - 4); }

template <int NB>
__device__ inline void issue_tile(char* stage, __amdgpu_buffer_rsrc_t cr, int cs,
                                  int blk0, const uint32_t (&goff)[5]) {
#pragma unroll
  for (int k = 0; k < NB; ++k)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        cr, (lds_void*)(stage + (blk0 + k) * 1024), 16, goff[k], cs * kRowB, 0, kStream);
}

__device__ inline u32x4 lds_load16(const char* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at maximum).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
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

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void mla_kernel(MlaParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_last;

  // Block id -> (head group, unit = b * P_max + split).  Units are dealt to
  // the 8 XCDs round-robin and every head group of a unit gets the same XCD.
  const int groups = p.n_h / kMlaHeadsPerWg;
  const int units = p.B * p.P_max;
  int id = blockIdx.x;
  const int xcd = id & 7;
  id >>= 3;
  const int hg = id % groups;
  const int u = (id / groups) * 8 + xcd;
  if (u >= units) return;
  const int b = u / p.P_max, split = u % p.P_max;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int half = wave & 1;
  const int h = hg * kMlaHeadsPerWg + (wave >> 1) * kMlaHeadsPerWave + r;
  const size_t bh = (size_t)b * p.n_h + h;
  const int col0 = half * 256;                 // this wave's output columns

  const int n = min(max(p.seq_lens[b], 0), p.L_max);
  const int start = split * p.S;
  if (start >= n) {
    if (split == 0) {
      // nothing to attend: zero row, lse = -inf
      uint16_t* o = (uint16_t*)p.out + bh * kMlaDc + col0;
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int c = g * 8; c < 256; c += 32) *reinterpret_cast<u32x4*>(o + c) = z;
      if (p.lse && half == 0 && g == 0) p.lse[bh] = kNegInf;
    }
    return;
  }
  const int end = min(n, start + p.S);
  const int nsplit = (n + p.S - 1) / p.S;
  const int nchunks = (end - start + kMlaChunk - 1) / kMlaChunk;

  const __amdgpu_buffer_rsrc_t cr = make_rsrc(
      (const char*)p.ckv + (size_t)b * p.L_max * kRowB, (uint32_t)n * kRowB);

  // DMA: load k of this wave fills LDS byte (blk0 + k)*1024 + lane*16 of a
  // stage: row rho, physical chunk pc, holding logical chunk pc ^ key(rho).
  const int blk0 = first_block(wave);
  const bool five = wave < 4;
  uint32_t goff[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int byte = (blk0 + k) * 1024 + lane * 16;
    const int rho = byte / kRowB;
    const int pc = (byte - rho * kRowB) >> 4;
    goff[k] = (uint32_t)(rho * kRowB + ((pc ^ swz_key(rho)) << 4));
  }

  // LDS read bases (all within one stage).  Scores: tile a, lane row
  // rho = pi(a, r), logical chunk 4kk + g with kk = 9h + k; writing
  // k = 2m + v gives chunk index 8*m + 8*((9h + v) >> 1) +
  // ((4*((h + v) & 1) + g) ^ key(rho)), so two bases per tile plus m*128.
  // Values: row g*8 + j has key ((j >> 1) & 1) | (g << 1); this half's chunk
  // 32h + 16cg + r lands at 32h + 16cg + 8*(r >> 3) + ((r & 7) ^ key): two
  // bases (by (j >> 1) & 1) plus j*1152 + cg*256.
  uint32_t wqk[2][2], wpv[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int rho = (r >> 2) * 8 + a * 4 + (r & 3);
#pragma unroll
    for (int v = 0; v < 2; ++v)
      wqk[a][v] = (uint32_t)(rho * kRowB + (((4 * ((half + v) & 1) + g) ^ swz_key(rho)) << 4) +
                             ((9 * half + v) >> 1) * 128);
  }
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
    wpv[jb] = (uint32_t)(g * 8 * kRowB +
                         ((32 * half + 8 * (r >> 3) + ((r & 7) ^ (jb | (g << 1)))) << 4));

  bf16x8 qop[kKHalf];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + bh * kD + half * (kD / 2);
#pragma unroll
    for (int k = 0; k < kKHalf; ++k)
      qop[k] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + k * 32 + g * 8));
  }

  // queries first, so waiting for them does not wait for the tiles
  if (five) {
    issue_tile<5>(smem, cr, start, blk0, goff);
    if (nchunks > 1) issue_tile<5>(smem + kTileB, cr, start + kMlaChunk, blk0, goff);
  } else {
    issue_tile<4>(smem, cr, start, blk0, goff);
    if (nchunks > 1) issue_tile<4>(smem + kTileB, cr, start + kMlaChunk, blk0, goff);
  }

  f32x4 acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  f32x4* xs_mine = reinterpret_cast<f32x4*>(smem + kStages * kTileB) + wave * 128 + lane;
  const f32x4* xs_peer =
      reinterpret_cast<const f32x4*>(smem + kStages * kTileB) + (wave ^ 1) * 128 + lane;

  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) {
      if (five) wait_vmcnt<5>();
      else wait_vmcnt<4>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (c + 2 < nchunks) {
      char* st = smem + ((c + 2) % kStages) * kTileB;
      if (five) issue_tile<5>(st, cr, start + (c + 2) * kMlaChunk, blk0, goff);
      else issue_tile<4>(st, cr, start + (c + 2) * kMlaChunk, blk0, goff);
    }
    const int cs = start + c * kMlaChunk;
    // This chunk's LDS bases, materialised once per chunk so that every read
    // below is base + constant (the constant goes in the instruction).
    const uint32_t toff = (uint32_t)((c % kStages) * kTileB);
    uint32_t qb[2][2], pb[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        qb[a][v] = toff + wqk[a][v];
        asm volatile("" : "+v"(qb[a][v]));
      }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      pb[jb] = toff + wpv[jb];
      asm volatile("" : "+v"(pb[jb]));
    }

    // this half's score contribution; LDS reads run two k-steps ahead
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    u32x4 A[2][2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int a = 0; a < 2; ++a) A[k][a] = lds_load16(smem, qb[a][k & 1] + (k >> 1) * 128);
#pragma unroll
    for (int k = 0; k < kKHalf; ++k) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[k & 1][0]), qop[k], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[k & 1][1]), qop[k], s1, 0, 0, 0);
      if (k + 2 < kKHalf) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
          A[k & 1][a] = lds_load16(smem, qb[a][k & 1] + ((k + 2) >> 1) * 128);
      }
    }
    // value rows of the first column group, read while the scores are exchanged
    u32x4 vr[2][8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      vr[0][jj] = lds_load16(smem, pb[(jj >> 1) & 1] + jj * kRowB);

    // add the other half's contribution
    xs_mine[0] = s0;
    xs_mine[64] = s1;
    lds_barrier();
    {
      const f32x4 o0 = xs_peer[0], o1 = xs_peer[64];
      s0 += o0;
      s1 += o1;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      vr[1][jj] = lds_load16(smem, pb[(jj >> 1) & 1] + jj * kRowB + 256);

    // online softmax over this lane's 8 positions of head r, with a lazy
    // reference max (moved only when weights would exceed 2^kRescaleMargin)
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = (cs + g * 8 + e < end) ? sv[e] * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m_run + kRescaleMargin;
    const float m_new = move ? mx : m_run;
    const float alpha = (move && m_run != kNegInf) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int m = 0; m < 16; ++m) acc[m] *= alpha;
    }
    uint32_t pp[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pp[e] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2 * e] - m_use),
                          __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_use));
      psum += bf16_lo(pp[e]) + bf16_hi(pp[e]);
    }
    l_run = l_run * alpha + psum;
    const u32x4 pv = {pp[0], pp[1], pp[2], pp[3]};
    const bf16x8 pop = as_bf16x8(pv);

    // weighted sum of this half's latent columns
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
        const int dw = m >> 1;
        u32x4 a;
        a[0] = __builtin_amdgcn_perm(vr[cg][1][dw], vr[cg][0][dw], sel);
        a[1] = __builtin_amdgcn_perm(vr[cg][3][dw], vr[cg][2][dw], sel);
        a[2] = __builtin_amdgcn_perm(vr[cg][5][dw], vr[cg][4][dw], sel);
        a[3] = __builtin_amdgcn_perm(vr[cg][7][dw], vr[cg][6][dw], sel);
        acc[cg * 8 + m] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), pop, acc[cg * 8 + m], 0, 0, 0);
      }
    }
  }

  // This split's result for head h: lane (r, g) holds columns
  // col0 + 128cg + 32g + 8i + m in acc[cg*8 + m][i].
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;

  if (nsplit == 1) {
    uint16_t* o = (uint16_t*)p.out + bh * kMlaDc;
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = col0 + 128 * cg + 32 * g + 8 * i;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = pack_bf16x2(acc[cg * 8 + 2 * e][i] * inv, acc[cg * 8 + 2 * e + 1][i] * inv);
        *reinterpret_cast<u32x4*>(o + c0) = v;
      }
    if (p.lse && half == 0 && g == 0) p.lse[bh] = lse2 * kLn2;
    return;
  }

  // Several splits: publish this one with device-coherent stores; the last
  // workgroup of the (sequence, head group) to take a ticket merges them.
  const __amdgpu_buffer_rsrc_t wo = make_rsrc(p.ws_o, kWsRecords);
  const __amdgpu_buffer_rsrc_t wl = make_rsrc(p.ws_lse, kWsRecords);
  {
    const size_t row = (bh * p.P_max + split) * kMlaDc;
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = col0 + 128 * cg + 32 * g + 8 * i;
        f32x4 v0, v1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = acc[cg * 8 + e][i] * inv;
          v1[e] = acc[cg * 8 + 4 + e][i] * inv;
        }
        store_coherent(wo, (uint32_t)((row + c0) * 4), v0);
        store_coherent(wo, (uint32_t)((row + c0 + 4) * 4), v1);
      }
    if (half == 0 && g == 0) store_coherent(wl, (uint32_t)((bh * p.P_max + split) * 4), lse2);
  }
  wait_vm_all();
  __syncthreads();
  int32_t* ticket = p.ws_cnt + (size_t)b * groups + hg;
  if (tid == 0) s_last = (atomicAdd(ticket, 1) == nsplit - 1);
  __syncthreads();
  if (!s_last) return;

  // Last split to finish merges every split of the 64 heads.  The split
  // lse values go to LDS first (the tile stages are free now), all loads in
  // flight together; then thread t sums columns (t % 64) * 8 .. +8 of heads
  // t / 64, t / 64 + 8, ... over the splits in batches of 4.
  float* wsm = reinterpret_cast<float*>(smem);
  const size_t bh0 = (size_t)b * p.n_h + hg * kMlaHeadsPerWg;
  for (int e = tid; e < kMlaHeadsPerWg * nsplit; e += kThreads) {
    const int h2 = e / nsplit, s = e - h2 * nsplit;
    wsm[e] = load_coherent1(wl, (uint32_t)(((bh0 + h2) * p.P_max + s) * 4));
  }
  __syncthreads();
  const int c0 = (tid & 63) * 8;
  for (int hl = tid >> 6; hl < kMlaHeadsPerWg; hl += kMlaWaves) {
    const size_t bhh = bh0 + hl;
    const size_t base = bhh * p.P_max;
    const float* lw = wsm + hl * nsplit;
    float M = kNegInf;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, lw[s]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float Z = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
      f32x4 va[4], vb[4];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int su = min(s0 + uu, nsplit - 1);
        const uint32_t off = (uint32_t)(((base + su) * kMlaDc + c0) * 4);
        va[uu] = load_coherent4(wo, off);
        vb[uu] = load_coherent4(wo, off + 16);
      }
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const float w = (s0 + uu < nsplit) ? __builtin_amdgcn_exp2f(lw[s0 + uu] - Mu) : 0.f;
        Z += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] += w * va[uu][e];
          o[4 + e] += w * vb[uu][e];
        }
      }
    }
    const float zi = Z > 0.f ? 1.f / Z : 0.f;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(o[2 * e] * zi, o[2 * e + 1] * zi);
    *reinterpret_cast<u32x4*>((uint16_t*)p.out + bhh * kMlaDc + c0) = v;
    if (p.lse && (tid & 63) == 0) p.lse[bhh] = Z > 0.f ? (M + __log2f(Z)) * kLn2 : kNegInf;
  }
  if (tid == 0) *ticket = 0;
}

hipError_t launch_mla(const MlaParams& p, hipStream_t s) {
  const int groups = p.n_h / kMlaHeadsPerWg;
  const size_t units = (size_t)p.B * p.P_max;
  const size_t blocks = (units + 7) / 8 * 8 * groups;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMlaLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(mla_kernel, dim3((unsigned)blocks), dim3(kThreads), kMlaLds, s, p);
  return hipGetLastError();
}

}  // namespace kvc
