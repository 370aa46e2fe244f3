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
// n_h * (576 + 512) multiply-adds.  A workgroup (4 waves, one per SIMD) owns
// 64 heads for one split of the positions; the workgroups of all head groups
// of one (sequence, split) are numbered so they land on the same XCD and
// stream the same rows at the same time, so L2 serves the repeats.
//
// Waves 2p and 2p+1 share heads 32p..32p+31.  Wave half h (0 or 1) computes
// the score contribution of row columns [288h, 288h+288) and, after the two
// halves are added through LDS, the output columns [256h, 256h+256).  Per
// wave (lane l: r = l % 32, g = l / 32) and 32-position chunk:
//  scores  S^T[t][hd]: 18 k-steps of v_mfma_f32_32x32x16_bf16; A = latent tile
//          rows from LDS (row r, columns 16kk + 8g .. +8), B = the 32 heads'
//          queries held in registers for the whole split.  Lane (r, g) gets
//          head r at rows 8*(i/4) + 4g + i%4, i = 0..15.
//  weights both waves of a pair run the same online softmax (log2 units) on
//          the summed scores; a lane's 16 weights are the B operand of the
//          value product for two k-steps of 16 positions.
//  values  O^T[c][hd] += C^T[c][t] P^T[t][hd]: per k-step 8 tiles of 32
//          columns; lane (r, g) reads 8 rows x 16 B at column 256h + r*8 and
//          transposes 8x8 bf16 in registers (v_perm), so tile m row r is
//          column 256h + r*8 + m.
//
// Latent tiles go HBM -> LDS directly (buffer_load ... lds), three chunks
// deep, with 16-byte chunk k of row rho stored at k ^ ((rho >> 1) & 7).  The
// row stride (1152 B) puts consecutive rows half a bank set apart on the
// 64-bank LDS, so this key gives 16 distinct bank groups to the 16 lanes an
// LDS cycle serves in both read patterns.  Rows at or past the sequence length read
// as zeros (buffer range check) and are masked.  Splits of one sequence are
// merged by log-sum-exp by the last workgroup to finish.

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kD = kMlaDc + kMlaDr;          // 576
constexpr int kRowB = kD * 2;                // 1152 bytes per row
constexpr int kTileB = kMlaChunk * kRowB;    // 36864 bytes per chunk
constexpr int kStages = 3;
constexpr int kLoadsPerWave = kTileB / 1024 / kMlaWaves;  // 9
constexpr int kKHalf = kD / 16 / 2;          // 18 k-steps per wave
constexpr int kXsBytes = kMlaWaves * 4 * 64 * 16;          // score exchange
constexpr size_t kMlaLds = (size_t)kStages * kTileB + kXsBytes;

typedef __attribute__((address_space(3))) void lds_void;

// This wave's share of one chunk's HBM -> LDS copy.  goff[k] is the lane's
// byte offset inside the tile for load k; the chunk start goes in the
// scalar offset.
__device__ inline void issue_tile(char* stage, __amdgpu_buffer_rsrc_t cr,
                                  int cs, int wave,
                                  const uint32_t (&goff)[kLoadsPerWave]) {
#pragma unroll
  for (int k = 0; k < kLoadsPerWave; ++k) {
    const int blk = wave * kLoadsPerWave + k;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        cr, (lds_void*)(stage + blk * 1024), 16, goff[k], cs * kRowB, 0, kStream);
  }
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

__global__ __launch_bounds__(256, 1) void mla_kernel(MlaParams p) {
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
  const int r = lane & 31, g = lane >> 5;
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
      for (int c = g * 8; c < 256; c += 16) *reinterpret_cast<u32x4*>(o + c) = z;
      if (p.lse && half == 0 && g == 0) p.lse[bh] = kNegInf;
    }
    return;
  }
  const int end = min(n, start + p.S);
  const int nsplit = (n + p.S - 1) / p.S;
  const int nchunks = (end - start + kMlaChunk - 1) / kMlaChunk;

  const __amdgpu_buffer_rsrc_t cr = make_rsrc(
      (const char*)p.ckv + (size_t)b * p.L_max * kRowB, (uint32_t)n * kRowB);

  // Load k of this lane fills LDS byte blk*1024 + lane*16 of a stage: row
  // rho, physical chunk pc, which holds logical chunk pc ^ ((rho >> 1) & 7).
  uint32_t goff[kLoadsPerWave];
#pragma unroll
  for (int k = 0; k < kLoadsPerWave; ++k) {
    const int byte = (wave * kLoadsPerWave + k) * 1024 + lane * 16;
    const int rho = byte / kRowB;
    const int pc = (byte - rho * kRowB) >> 4;
    goff[k] = (uint32_t)(rho * kRowB + ((pc ^ ((rho >> 1) & 7)) << 4));
  }
  // LDS read bases.  Scores: row r, logical chunk q = 2kk + g, stored at
  // 8*(q/8) + ((q & 7) ^ f) with f = (r >> 1) & 7.  This wave's k-steps are
  // kk = 18h + k; writing k = 4a + u and x = 2h + u gives kk & 3 = x & 3 and
  // kk >> 2 = 4h + a + (x >> 2), so four per-wave bases plus a*128 cover
  // every k-step.  Values: row rho = 8*(2ks + jj/4) + 4g + (jj & 3) has key
  // f = (4*(jj/4) + 2g + ((jj >> 1) & 1)) & 7 (ks drops out), and this half's
  // chunk 32h + r sits at 32h + (r ^ f): eight bases (one per jj) plus
  // 16*1152*ks.
  uint32_t wqk[4], pv_base[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int x = 2 * half + v;
    wqk[v] = (uint32_t)(r * kRowB + (((2 * (x & 3) + g) ^ ((r >> 1) & 7)) << 4) +
                        (4 * half + (x >> 2)) * 128);
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int rho0 = 8 * (jj >> 2) + 4 * g + (jj & 3);
    const int f = (rho0 >> 1) & 7;
    pv_base[jj] = (uint32_t)(rho0 * kRowB + ((r ^ f) << 4) + half * 512);
  }

  bf16x8 qop[kKHalf];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + bh * kD + half * (kD / 2);
#pragma unroll
    for (int k = 0; k < kKHalf; ++k)
      qop[k] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + k * 16 + g * 8));
  }

  // queries first, so waiting for them does not wait for the tiles
  issue_tile(smem, cr, start, wave, goff);
  if (nchunks > 1) issue_tile(smem + kTileB, cr, start + kMlaChunk, wave, goff);

  f32x16 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  f32x4* xs_mine = reinterpret_cast<f32x4*>(smem + kStages * kTileB) + wave * 256 + lane;
  const f32x4* xs_peer =
      reinterpret_cast<const f32x4*>(smem + kStages * kTileB) + (wave ^ 1) * 256 + lane;

  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) wait_vmcnt<kLoadsPerWave>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (c + 2 < nchunks)
      issue_tile(smem + ((c + 2) % kStages) * kTileB, cr,
                 start + (c + 2) * kMlaChunk, wave, goff);
    const int cs = start + c * kMlaChunk;
    // This chunk's LDS bases, materialised once per chunk so that every read
    // below is base + constant (the constant goes in the instruction).
    const uint32_t toff = (uint32_t)((c % kStages) * kTileB);
    uint32_t qb[4], pb[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      qb[v] = toff + wqk[v];
      asm volatile("" : "+v"(qb[v]));
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      pb[jj] = toff + pv_base[jj];
      asm volatile("" : "+v"(pb[jj]));
    }

    // this half's score contribution; LDS reads run four k-steps ahead
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    u32x4 A[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) A[k] = lds_load16(smem, qb[k & 3] + (k >> 2) * 128);
#pragma unroll
    for (int k = 0; k < kKHalf; ++k) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[k & 3]), qop[k], sacc, 0, 0, 0);
      if (k + 4 < kKHalf) A[k & 3] = lds_load16(smem, qb[(k + 4) & 3] + ((k + 4) >> 2) * 128);
    }
    // value rows of both k-steps, read while the scores are exchanged
    u32x4 vr[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        vr[ks][jj] = lds_load16(smem, pb[jj] + 16 * ks * kRowB);

    // add the other half's contribution
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      xs_mine[q4 * 64] = f32x4{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
    lds_barrier();
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 o = xs_peer[q4 * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[4 * q4 + e] += o[e];
    }

    // online softmax over this lane's 16 positions of head r, with a lazy
    // reference max (moved only when weights would exceed 2^kRescaleMargin)
    float sv[16];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rho = 8 * (i >> 2) + 4 * g + (i & 3);
      sv[i] = (cs + rho < end) ? sacc[i] * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m_run + kRescaleMargin;
    const float m_new = move ? mx : m_run;
    const float alpha = (move && m_run != kNegInf) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] *= alpha;
    }
    uint32_t pp[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pp[e] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2 * e] - m_use),
                          __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_use));
      psum += bf16_lo(pp[e]) + bf16_hi(pp[e]);
    }
    l_run = l_run * alpha + psum;

    // weighted sum of this half's latent columns
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 pv = {pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]};
      const bf16x8 pop = as_bf16x8(pv);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
        const int dw = m >> 1;
        u32x4 a;
        a[0] = __builtin_amdgcn_perm(vr[ks][1][dw], vr[ks][0][dw], sel);
        a[1] = __builtin_amdgcn_perm(vr[ks][3][dw], vr[ks][2][dw], sel);
        a[2] = __builtin_amdgcn_perm(vr[ks][5][dw], vr[ks][4][dw], sel);
        a[3] = __builtin_amdgcn_perm(vr[ks][7][dw], vr[ks][6][dw], sel);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pop, acc[m], 0, 0, 0);
      }
    }
  }

  // this split's result for head h, columns col0 + rho_i * 8 + m
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;

  if (nsplit == 1) {
    uint16_t* o = (uint16_t*)p.out + bh * kMlaDc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c0 = col0 + (8 * (i >> 2) + 4 * g + (i & 3)) * 8;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = pack_bf16x2(acc[2 * e][i] * inv, acc[2 * e + 1][i] * inv);
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
    for (int i = 0; i < 16; ++i) {
      const int c0 = col0 + (8 * (i >> 2) + 4 * g + (i & 3)) * 8;
      f32x4 v0, v1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = acc[e][i] * inv;
        v1[e] = acc[4 + e][i] * inv;
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
  // t / 64, t / 64 + 4, ... over the splits in batches of 4.
  float* wsm = reinterpret_cast<float*>(smem);
  const size_t bh0 = (size_t)b * p.n_h + hg * kMlaHeadsPerWg;
  for (int e = tid; e < kMlaHeadsPerWg * nsplit; e += blockDim.x) {
    const int h2 = e / nsplit, s = e - h2 * nsplit;
    wsm[e] = load_coherent1(wl, (uint32_t)(((bh0 + h2) * p.P_max + s) * 4));
  }
  __syncthreads();
  const int c0 = (tid & 63) * 8;
  for (int hl = tid >> 6; hl < kMlaHeadsPerWg; hl += 4) {
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
      for (int u = 0; u < 4; ++u) {
        const int su = min(s0 + u, nsplit - 1);
        const uint32_t off = (uint32_t)(((base + su) * kMlaDc + c0) * 4);
        va[u] = load_coherent4(wo, off);
        vb[u] = load_coherent4(wo, off + 16);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = (s0 + u < nsplit) ? __builtin_amdgcn_exp2f(lw[s0 + u] - Mu) : 0.f;
        Z += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] += w * va[u][e];
          o[4 + e] += w * vb[u][e];
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
  hipLaunchKernelGGL(mla_kernel, dim3((unsigned)blocks), dim3(256), kMlaLds, s, p);
  return hipGetLastError();
}

}  // namespace kvc
