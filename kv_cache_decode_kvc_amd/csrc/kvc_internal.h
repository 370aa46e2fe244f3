// Internal declarations shared by the host API and the kernel sources.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kvc {

// Positions one wave consumes per step of the MFMA dense kernel, and the
// dense / top-k decode: positions per wave-chunk.
constexpr int kDenseChunk = 32;
constexpr int kDenseGran = 32;     // split sizes are whole chunks
constexpr int kMaxGroup = 16;        // query heads per KV head a kernel serves
// Upper bound on the splits of one sequence (the merge stages their weights
// in LDS); the split policy raises the split size to respect it.
constexpr int kMaxSplits = 256;
// Online softmax: the reference max moves only when a chunk's max exceeds it
// by this much (log2 units), so weights stay <= 2^8 and rescaling of the
// accumulators is rare.  The result is the same; only rounding differs.
constexpr float kRescaleMargin = 8.0f;
// MLA kernel: positions per step (also the split granularity); a workgroup
// of 8 waves (two per SIMD) covers 64 heads, two waves sharing each 16.
constexpr int kMlaChunk = 32;
constexpr int kMlaHeadsPerWave = 32;
constexpr int kMlaHeadsPerWg = 64;      // n_h must be a multiple of this
// Heads one MLA workgroup covers: 128 (4 waves) when n_h allows, else 64.
inline int mla_heads_per_wg(int n_h) { return n_h % 128 == 0 ? 128 : 64; }
constexpr int kMlaDc = 512;
constexpr int kMlaDr = 64;

struct AppendParams {
  void* k_cache;
  void* v_cache;          // may be null
  int32_t* seq_lens;
  const void* k_new;
  const void* v_new;      // may be null
  int32_t* flag;          // may be null
  int B, n_kv, L_max, d, elem_bytes;
  float k_inv, v_inv;     // FP8 append: 1 / scale of the keys and values
  const int32_t* block_table;   // paged append: [B, max_blocks]
  int max_blocks, num_blocks, page_shift;
  void* k_scales;         // FP4 append: per-16-channel E4M3 scales [B, n_kv, L_max, d/16]
  void* v_scales;
};

// Dense and top-k decode.  Workspace pointers are null when P_max == 1.
struct DenseParams {
  const void* q;
  void* k;                // written only by the fused append-and-attend call
  void* v;
  const void* k_new;      // fused call: the new token's rows [B, n_kv, d]
  const void* v_new;
  int32_t* seq_lens_rw;   // fused call: lengths to bump (same array as seq_lens)
  int32_t* ws_bcnt;       // fused call: [B] per-sequence arrival counters
  int32_t* ws_ucnt;       // fused call: [B * n_kv] per-unit arrival counters
  const int32_t* seq_lens;
  const int32_t* idx;     // top-k only
  void* out;
  float* lse;             // may be null
  int32_t* flag;          // may be null (top-k only)
  int32_t* ws_cnt;        // [B * n_kv] completion tickets
  float* ws_lse;          // [B * n_h * P_max] log2-domain partial lse
  float* ws_o;            // [B * n_h * P_max * d] normalised partial outputs
  int B, n_h, n_kv, G, L_max, d;
  int K;                  // top-k list length (0 for dense)
  int S;                  // positions per split (even mode: the least)
  int P_max;              // splits per (b, kv head) in the grid
  int even;               // 1: spread each sequence over the P_max splits
  float scale_log2;       // scale * log2(e) (times the key scale for FP8 caches)
  float out_scale;        // multiplies the output (the value scale for FP8 caches)
  int window;             // > 0: attend only the newest `window` positions
  const int32_t* win_start;  // window mode, may be null: first present position per sequence
  // paged cache: k/v are pools [num_blocks, n_kv, 1 << page_shift, d];
  // position t of sequence b is in block block_table[b * max_blocks + (t >> page_shift)]
  const int32_t* block_table;
  int max_blocks, num_blocks, page_shift;
  // FP4 cache: k/v hold E2M1 codes [B, n_kv, L_max, d/2]; these the E4M3
  // scale of every 16 channels [B, n_kv, L_max, d/16]
  const void* k_scales;
  const void* v_scales;
  // persistent form (fixed split size, MFMA kernels): [0] next item, [1]
  // workgroups done; both zero between calls
  int persist;
  int32_t* ws_sched;
};

// Persistent dense kernels: lengths and per-unit item counts live in LDS,
// so the form is used up to these sizes (beyond them, one workgroup per
// unit and split).  kPersistWgs workgroups: two per compute unit of a
// 256-CU MI355X.
constexpr int kPersistMaxB = 1024;
constexpr int kPersistMaxUnits = 2048;
constexpr int kPersistWgs = 512;

// Pool bitmap words the selection kernel holds in LDS (one bit per block).
constexpr int kSelectPoolWords = 12288;
// Longest score row the selection kernel reads (positions; its loads use
// 32-bit byte offsets).
constexpr int kSelectMaxRow = 1 << 29;
// Selection map: one bit per position, whole 16384-position steps, for rows
// of at most 2^18 positions (longer rows take the multi-pass path only).
constexpr int kSelectMapMax = 1 << 18;
inline int select_map_words(int L_max) {
  return L_max > kSelectMapMax ? 0 : (L_max + 16383) / 16384 * 512;
}

struct SelectParams {
  const float* scores;      // [B, R, L_max]
  const int32_t* seq_lens;  // [B]
  const int32_t* pool;      // [B, R, P] block ids, or null
  int32_t* out;             // [B, R, K]
  int B, R, L_max, K, P, pool_block, pool_words;
  int sel_words;            // > 0: one-bit-per-position selection map (L_max <= 2^18)
  // Segmented form (S >= 2): each row cut into S segments of seg_len
  // positions, spread over the compute units (workspace pointers below).
  int S, seg_len;
  int32_t* ws_cnt;          // [rows] arrival counters (returned to zero)
  uint32_t* ws_cand;        // [rows, S, 16 waves, kSelSegCapw, 2] (key, position)
  int32_t* ws_ccnt;         // [rows, S, 16 waves] candidates per wave
};

// Segmented selection: with a workspace, no pool and rows of at most
// kSelectMapMax positions, a row is cut into segments of whole
// 16384-position steps so that about kSelSegTargetWgs workgroups share the
// rows (one workgroup per row keeps only `rows` compute units busy).  Each
// wave of a segment keeps up to kSelSegCapw candidates (keys at or above a
// sampled lower bound of the row's threshold); a row with more, or whose
// bound turns out too high, is finished by the one-workgroup algorithm.
constexpr int kSelSegTargetWgs = 256;
constexpr int kSelSegCapw = 128;
constexpr int kSelSegWaves = 16;
struct SelectSegPlan {
  int S = 1, seg_len = 0;
  size_t cnt_off = 0, cand_off = 0, ccnt_off = 0;
  size_t bytes = 0;         // 0: no segmented form
};
SelectSegPlan select_seg_plan(int64_t rows, int L_max);

struct MlaParams {
  const void* q;
  const void* ckv;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  int32_t* ws_cnt;        // [B]
  float* ws_lse;          // [B * n_h * P_max]
  float* ws_o;            // [B * n_h * P_max * d_c] bf16 normalised partial outputs
  int B, n_h, L_max;
  int S, P_max;
  float scale_log2;
};

struct WsLayout {
  size_t cnt_off, lse_off, o_off, bcnt_off, sched_off, total;
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Dense / top-k split geometry: split s holds positions [s*S, min(n, (s+1)*S)).
__host__ __device__ inline int dense_num_splits(int n, int S) {
  return n <= 0 ? 1 : (n + S - 1) / S;
}
// Split size for a sequence of n positions.  Fixed mode: S.  Even mode: the
// least whole-chunk size (not below S) that fits n into P splits.
__host__ __device__ inline int dense_split_size(int n, int S, int P, int even) {
  if (!even) return S;
  int Sn = (n + P - 1) / P;
  Sn = (Sn + 31) / 32 * 32;
  return Sn > S ? Sn : S;
}
// Sliding window: the newest query (position n - 1) attends keys from
// max(s, n - window) (bounded-replay rule, s = first present position).
__device__ inline int window_low(const DenseParams& p, int b, int n) {
  if (p.window <= 0) return 0;
  int lo = n - p.window;
  if (p.win_start) lo = max(lo, p.win_start[b]);
  return min(max(lo, 0), n);
}
__host__ __device__ inline void dense_split_range(int n, int S, int split, int& start, int& end) {
  start = split * S;
  end = start + S < n ? start + S : n;
}

// Workspace: [tickets per unit][partial lse][partial outputs] when a
// sequence can need several splits, then (fused append-and-attend only) one
// arrival counter per sequence followed by one per unit, then (persistent
// form) a 256-byte block holding the two scheduling counters.
inline WsLayout ws_layout(size_t units, size_t B, size_t n_h, size_t P_max,
                          size_t d, bool fused = false, bool persist = false) {
  WsLayout w{};
  size_t end = 0;
  if (P_max > 1) {
    w.cnt_off = 0;
    w.lse_off = round_up(units * sizeof(int32_t), 256);
    w.o_off = w.lse_off + round_up(B * n_h * P_max * sizeof(float), 256);
    end = round_up(w.o_off + B * n_h * P_max * d * sizeof(float), 256);
  }
  if (fused) {
    w.bcnt_off = end;
    end += round_up((B + units) * sizeof(int32_t), 256);
  }
  if (persist) {
    w.sched_off = end;
    end += 256;
  }
  w.total = end;
  return w;
}

// The no-allocation entry point's scratch (static_scratch.hip): one
// library-owned device array per GPU.  Three counter arrays of
// kStaticCounterWords int32 (split tickets, per-sequence arrivals, per-unit
// arrivals), then the split partials (lse, outputs) from kStaticPartialOff.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int kStaticCounterWords = 16384;
// (the two scheduling counters of the persistent form follow the three
// counter arrays, in a 256-byte block of their own)
constexpr size_t kStaticSchedOff = 3 * (size_t)kStaticCounterWords * sizeof(int32_t);
constexpr size_t kStaticPartialOff = kStaticSchedOff + 256;
// Device address of this device's scratch (looked up once per device).
hipError_t static_scratch(void** ptr);
// Zero the counter words a call uses (tickets and unit arrivals [0, units),
// sequence arrivals [0, B)) on the call's stream.
hipError_t launch_clear_static_counters(void* base, int units, int B, hipStream_t s);

// Kernel launchers (defined in the .hip sources).
hipError_t launch_append(const AppendParams& p, hipStream_t s);
hipError_t launch_append_fp8(const AppendParams& p, hipStream_t s);
hipError_t launch_dense_fp8(const DenseParams& p, hipStream_t s);
hipError_t launch_append_fp4(const AppendParams& p, hipStream_t s);
hipError_t launch_dense_fp4(const DenseParams& p, hipStream_t s);
hipError_t launch_dense_paged(const DenseParams& p, hipStream_t s);
hipError_t launch_append_paged(const AppendParams& p, hipStream_t s);
hipError_t launch_dense_mfma(const DenseParams& p, bool topk, bool append, hipStream_t s);
hipError_t launch_dense_generic(const DenseParams& p, int dtype, bool topk,
                                bool append, hipStream_t s);
hipError_t launch_mla(const MlaParams& p, hipStream_t s);
hipError_t launch_topk_select(const SelectParams& p, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, float* sink,
                              hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes,
                       hipStream_t s);
size_t stream_read_blocks(size_t bytes);

}  // namespace kvc
