// Host side of the C ABI declared in include/kvc.h: argument checks (done
// before any HIP runtime call, so they work on a machine with no GPU), the
// split policy, workspace layout and kernel launches on the caller's stream.

#include "kvc.h"

#include <math.h>

#include <atomic>

#include "kvc_internal.h"

using namespace kvc;

namespace {

std::atomic<int> g_split_override{0};

constexpr int64_t kMaxOffset = (int64_t)1 << 31;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_bytes(int dtype) { return dtype == KVC_BF16 ? 2 : 4; }

bool good_dtype(int dtype) { return dtype == KVC_F32 || dtype == KVC_BF16; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Dense/top-k splits.  A small problem (the whole step fits in about one
// round of workgroups: two per compute unit of a 256-CU MI355X, the MFMA
// kernel's occupancy) runs in "even" mode: the grid has P = 512 / units
// splits per (sequence, KV head) and each workgroup cuts its sequence's
// actual length into at most P equal whole-chunk splits (at least 128
// positions), so no workgroup starts late and the merge tail is paid once.
// A large problem uses a fixed split of at least 256 positions (two chunks
// per wave, so each wave keeps a second chunk in flight), doubled until there
// are no more than about 18 workgroups per CU, and relies on the hardware to
// balance the rounds.  Measured on MI355X: the 32-sequence GQA layer is
// fastest at 2048.  The size of a small problem is judged from L_max (the
// lengths live on the device).
constexpr int64_t kDenseTargetWgs = 4608;
constexpr int64_t kDenseMinSplit = 256;
constexpr int64_t kDenseRound = 512;
constexpr int64_t kDenseMinEvenSplit = 128;
constexpr int kCUs = 256;

int64_t dense_splits(int64_t n, int64_t S) { return dense_num_splits((int)n, (int)S); }

struct SplitPlan {
  int S;        // fixed split, or the least split in even mode
  int64_t P;    // grid splits per unit
  int even;
};

SplitPlan plan_splits(int kind, int64_t units, int64_t n_max) {
  const int gran = kind == KVC_KIND_MLA ? kMlaChunk : kDenseGran;
  if (n_max < 1) n_max = 1;
  if (units < 1) units = 1;  // empty batch: any valid split will do
  const int64_t S_cap = round_up((size_t)ceil_div(n_max, kMaxSplits), (size_t)gran);
  const int ov = g_split_override.load();
  if (ov > 0) {
    const int64_t S = round_up((size_t)ov, (size_t)gran);
    const int Sf = (int)(S > S_cap ? S : S_cap);
    return {Sf, kind == KVC_KIND_MLA ? ceil_div(n_max, Sf) : dense_splits(n_max, Sf), 0};
  }
  if (kind == KVC_KIND_MLA) {
    // A workgroup covers 64 or 128 heads and occupies a compute unit; aim
    // for one workgroup per CU.  Each split's partial output costs n_h * d_c
    // floats, so keep splits at least 256 positions long.  `units` counts
    // (sequence, head group) pairs.
    int64_t P = ceil_div(kCUs, units);
    if (P < 1) P = 1;
    int64_t S = round_up((size_t)ceil_div(n_max, P), (size_t)gran);
    if (S < 256) S = 256;
    const int Sf = (int)(S > S_cap ? S : S_cap);
    return {Sf, ceil_div(n_max, Sf), 0};
  }
  if (units * dense_splits(n_max, kDenseMinSplit) <= kDenseRound + kDenseRound / 4) {
    // (top-k: one round of one workgroup per CU, so each wave has four
    // listed chunks to pipeline its index and row loads over; measured on
    // the 2048-of-131072 layer over 64 units: 21.6 us with 4 splits of 512
    // against 23.1 with 8 of 256 and 23.1 with 640)
    const int64_t round = kind == KVC_KIND_TOPK ? kCUs : kDenseRound;
    int64_t P = units >= round ? 1 : round / units;
    if (P > kMaxSplits) P = kMaxSplits;
    // no more splits than n_max has minimum-size pieces
    const int64_t P_fill = dense_splits(n_max, kDenseMinEvenSplit);
    if (P > P_fill) P = P_fill;
    // Every length up to n_max fits in P splits.  P is not trimmed to the
    // splits n_max itself takes: a fused append attends n_max - 1 cached
    // rows, which may need all P (4096 rows: 16 x 256, where 4097 takes
    // 15 x 288).
    return {(int)kDenseMinEvenSplit, P, 1};
  }
  int64_t S = kDenseMinSplit;
  while (units * dense_splits(n_max, S) > kDenseTargetWgs && S < ((int64_t)1 << 24))
    S *= 2;
  const int Sf = (int)(S > S_cap ? S : S_cap);
  return {Sf, dense_splits(n_max, Sf), 0};
}

struct DenseCheck {
  int status;
  int S;
  int64_t P_max;
  int even;
  int persist;
  WsLayout ws;
};

// Cache formats of the dense calls (the persistent form's item size
// depends on it).
enum CacheFmt { kFmtPlain = 0, kFmtFp8 = 1, kFmtFp4 = 2 };

// Persistent form: items of whole 1024-position multiples (the multiple
// nearest n_max / P, P = target / units), about this many per call (3.5 per
// workgroup for bf16 and E4M3 caches, 2 for FP4 ones, whose items are the
// quickest to stream and so pay most for each item's set-up and merge).
// Measured on the 32-sequence GQA layer (lengths 1024..32768, 256 units):
// contiguous bf16 314.7 us at 5120 positions against 326.8 at 2048, paged
// 325 against 333, E4M3 171.7 at 5120 against 177.6 at 3072, 183.0 at 4096
// and 181.4 at 6144 (with 16-byte value loads), FP4 123.7 at 8192 against
// 129.3 at 5120, 128.6 at 6144 and 131.6 at 9216.
constexpr int64_t kPersistItems = 1792;
constexpr int64_t kPersistItemsFp4 = 1024;
constexpr int64_t kPersistGran = 1024;

// window > 0: at most `window` positions are attended, which is what the
// split plan and the workspace are sized for.
DenseCheck check_dense_shape(int B, int n_h, int n_kv, int L_max, int d,
                             int dtype, int K, bool topk, bool fused = false,
                             int window = 0, CacheFmt fmt = kFmtPlain) {
  DenseCheck c{KVC_OK, 0, 1, 0, 0, {}};
  if (!good_dtype(dtype)) { c.status = KVC_ERR_BAD_DTYPE; return c; }
  if (B < 0 || n_h < 1 || n_kv < 1 || L_max < 1 || d < 1) {
    c.status = KVC_ERR_BAD_SHAPE; return c;
  }
  if (n_h % n_kv != 0) { c.status = KVC_ERR_BAD_SHAPE; return c; }
  if (topk && (K < 1 || K > L_max)) { c.status = KVC_ERR_BAD_SHAPE; return c; }
  if ((int64_t)L_max * d * elem_bytes(dtype) >= kMaxOffset) {
    c.status = KVC_ERR_BAD_SHAPE; return c;
  }
  if (d != 64 && d != 128) { c.status = KVC_ERR_UNSUPPORTED; return c; }
  if (n_h / n_kv > kMaxGroup) { c.status = KVC_ERR_UNSUPPORTED; return c; }
  const int64_t units = (int64_t)B * n_kv;
  const int64_t n_max = topk ? K : (window > 0 && window < L_max ? window : L_max);
  const SplitPlan plan = plan_splits(topk ? KVC_KIND_TOPK : KVC_KIND_DENSE, units, n_max);
  c.S = plan.S;
  c.P_max = plan.P;
  c.even = plan.even;
  if (units * c.P_max >= kMaxOffset) { c.status = KVC_ERR_BAD_SHAPE; return c; }
  // Large problems (fixed split size) on the MFMA kernels run in the
  // persistent form when the lengths and per-unit item counts fit its LDS.
  c.persist = !c.even && !topk && dtype == KVC_BF16 && d == 128 && B <= kPersistMaxB &&
              units <= kPersistMaxUnits;
  if (c.persist && g_split_override.load() == 0) {
    const int64_t target = fmt == kFmtFp4 ? kPersistItemsFp4 : kPersistItems;
    const int64_t P_allowed = units < target ? target / units : 1;
    int64_t S = (n_max / P_allowed + kPersistGran / 2) / kPersistGran * kPersistGran;
    if (S < kPersistGran) S = kPersistGran;
    const int64_t S_cap = (int64_t)round_up((size_t)ceil_div(n_max, kMaxSplits), (size_t)kDenseGran);
    if (S < S_cap) S = S_cap;
    if (S < c.S) S = c.S;
    c.S = (int)S;
    c.P_max = dense_splits(n_max, S);
  }
  c.ws = ws_layout((size_t)units, (size_t)B, (size_t)n_h, (size_t)c.P_max, (size_t)d, fused,
                   c.persist != 0);
  if (c.ws.total >= (size_t)kMaxOffset) { c.status = KVC_ERR_UNSUPPORTED; return c; }
  return c;
}

int check_workspace(const WsLayout& ws, void* workspace, size_t ws_bytes) {
  if (ws.total == 0) return KVC_OK;
  if (!workspace) return KVC_ERR_NULL_PTR;
  if (!aligned(workspace, 256)) return KVC_ERR_MISALIGNED;
  if (ws_bytes < ws.total) return KVC_ERR_WORKSPACE;
  return KVC_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

void fill_ws(DenseParams& p, const WsLayout& ws, void* workspace, size_t P_max,
             bool fused) {
  p.ws_cnt = nullptr; p.ws_lse = nullptr; p.ws_o = nullptr; p.ws_bcnt = nullptr;
  p.ws_sched = nullptr;
  char* base = static_cast<char*>(workspace);
  if (p.persist) p.ws_sched = reinterpret_cast<int32_t*>(base + ws.sched_off);
  if (P_max > 1) {
    p.ws_cnt = reinterpret_cast<int32_t*>(base + ws.cnt_off);
    p.ws_lse = reinterpret_cast<float*>(base + ws.lse_off);
    p.ws_o = reinterpret_cast<float*>(base + ws.o_off);
  }
  if (fused) {
    p.ws_bcnt = reinterpret_cast<int32_t*>(base + ws.bcnt_off);
    p.ws_ucnt = p.ws_bcnt + p.B;
  }
}

struct MlaCheck {
  int status;
  int S;
  int64_t P_max;
  WsLayout ws;
};

MlaCheck check_mla_shape(int B, int n_h, int L_max, int d_c, int d_r, int dtype) {
  MlaCheck c{KVC_OK, 0, 1, {}};
  if (!good_dtype(dtype)) { c.status = KVC_ERR_BAD_DTYPE; return c; }
  if (B < 0 || n_h < 1 || L_max < 1 || d_c < 1 || d_r < 0) {
    c.status = KVC_ERR_BAD_SHAPE; return c;
  }
  if ((int64_t)L_max * (d_c + d_r) * elem_bytes(dtype) >= kMaxOffset) {
    c.status = KVC_ERR_BAD_SHAPE; return c;
  }
  if (dtype != KVC_BF16 || d_c != kMlaDc || d_r != kMlaDr ||
      n_h % kMlaHeadsPerWg != 0) {
    c.status = KVC_ERR_UNSUPPORTED; return c;
  }
  const SplitPlan plan = plan_splits(KVC_KIND_MLA, (int64_t)B * (n_h / mla_heads_per_wg(n_h)), L_max);
  c.S = plan.S;
  c.P_max = plan.P;
  const int64_t groups = n_h / mla_heads_per_wg(n_h);
  if ((int64_t)B * groups * c.P_max >= kMaxOffset) { c.status = KVC_ERR_BAD_SHAPE; return c; }
  // (partial outputs are bf16: d_c values take the room of d_c / 2 floats)
  c.ws = ws_layout((size_t)B * groups, (size_t)B, (size_t)n_h, (size_t)c.P_max, (size_t)d_c / 2);
  if (c.ws.total >= (size_t)kMaxOffset) { c.status = KVC_ERR_UNSUPPORTED; return c; }
  return c;
}

}  // namespace

extern "C" {

const char* kvc_status_string(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_ERR_NULL_PTR: return "a required pointer is NULL";
    case KVC_ERR_BAD_SHAPE: return "bad shape (non-positive size, n_h % n_kv != 0, K out of range, or offsets beyond 2^31)";
    case KVC_ERR_BAD_DTYPE: return "dtype must be KVC_F32 or KVC_BF16";
    case KVC_ERR_UNSUPPORTED: return "shape or dtype has no kernel in this build";
    case KVC_ERR_WORKSPACE: return "workspace smaller than the size query returned";
    case KVC_ERR_MISALIGNED: return "pointer alignment rule broken";
    case KVC_ERR_HIP: return "HIP launch error";
    case KVC_ERR_BAD_ARG: return "bad argument (non-finite scale or negative override)";
    case KVC_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int kvc_set_split_override(int positions) {
  if (positions < 0) return KVC_ERR_BAD_ARG;
  g_split_override.store(positions);
  return KVC_OK;
}

int kvc_split_positions(int kind, int B, int units, int n_max) {
  if (kind < KVC_KIND_DENSE || kind > KVC_KIND_MLA || B < 1 || units < 1)
    return KVC_ERR_BAD_ARG;
  const SplitPlan plan = plan_splits(kind, units, n_max);
  return dense_split_size(n_max < 1 ? 1 : n_max, plan.S, (int)plan.P, plan.even);
}

int kvc_append(void* k_cache, void* v_cache, int32_t* seq_lens,
               const void* k_new, const void* v_new, int B, int n_kv,
               int L_max, int d, kvc_dtype dtype, int32_t* flag, void* stream) {
  if (!good_dtype(dtype)) return KVC_ERR_BAD_DTYPE;
  if (B < 0 || n_kv < 1 || L_max < 1 || d < 1) return KVC_ERR_BAD_SHAPE;
  if ((int64_t)n_kv * d >= kMaxOffset) return KVC_ERR_BAD_SHAPE;
  if (!k_cache || !seq_lens || !k_new) return KVC_ERR_NULL_PTR;
  if ((v_cache == nullptr) != (v_new == nullptr)) return KVC_ERR_NULL_PTR;
  if (!aligned(k_cache, 16) || !aligned(k_new, 16) ||
      (v_cache && (!aligned(v_cache, 16) || !aligned(v_new, 16))) ||
      !aligned(seq_lens, 4) || (flag && !aligned(flag, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  AppendParams p{k_cache, v_cache, seq_lens, k_new, v_new, flag,
                 B, n_kv, L_max, d, elem_bytes(dtype), 1.f, 1.f};
  return launch_status(launch_append(p, static_cast<hipStream_t>(stream)));
}

int kvc_append_fp8(void* k_cache, void* v_cache, int32_t* seq_lens,
                   const void* k_new, const void* v_new, int B, int n_kv,
                   int L_max, int d, float k_scale, float v_scale,
                   int32_t* flag, void* stream) {
  if (B < 0 || n_kv < 1 || L_max < 1 || d < 1) return KVC_ERR_BAD_SHAPE;
  if (d % 16 != 0 || (int64_t)n_kv * d >= kMaxOffset) return KVC_ERR_BAD_SHAPE;
  if (!(isfinite(k_scale) && isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return KVC_ERR_BAD_ARG;
  if (!k_cache || !v_cache || !seq_lens || !k_new || !v_new) return KVC_ERR_NULL_PTR;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(seq_lens, 4) || (flag && !aligned(flag, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  AppendParams p{k_cache, v_cache, seq_lens, k_new, v_new, flag,
                 B, n_kv, L_max, d, 1,
                 (float)(1.0 / (double)k_scale), (float)(1.0 / (double)v_scale)};
  return launch_status(launch_append_fp8(p, static_cast<hipStream_t>(stream)));
}

int kvc_append_fp4(void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                   int32_t* seq_lens, const void* k_new, const void* v_new, int B, int n_kv,
                   int L_max, int d, int32_t* flag, void* stream) {
  if (B < 0 || n_kv < 1 || L_max < 1 || d < 1) return KVC_ERR_BAD_SHAPE;
  if (d % 16 != 0 || (int64_t)n_kv * d >= kMaxOffset) return KVC_ERR_BAD_SHAPE;
  if (!k_codes || !k_scales || !v_codes || !v_scales || !seq_lens || !k_new || !v_new)
    return KVC_ERR_NULL_PTR;
  if (!aligned(k_codes, 8) || !aligned(v_codes, 8) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(seq_lens, 4) || (flag && !aligned(flag, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  AppendParams p{k_codes, v_codes, seq_lens, k_new, v_new, flag, B, n_kv, L_max, d, 1};
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  return launch_status(launch_append_fp4(p, static_cast<hipStream_t>(stream)));
}

size_t kvc_decode_attn_workspace_size(int B, int n_h, int n_kv, int L_max,
                                      int d, kvc_dtype dtype) {
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, L_max, d, dtype, 0, false);
  return c.status == KVC_OK ? c.ws.total : 0;
}

size_t kvc_decode_attn_topk_workspace_size(int B, int n_h, int n_kv, int K,
                                           int d, kvc_dtype dtype) {
  // The workspace depends on K, not on L_max; any L_max >= K gives the same.
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, K < 1 ? 1 : K, d, dtype, K, true);
  return c.status == KVC_OK ? c.ws.total : 0;
}

static int dense_common(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, const int32_t* idx, int K,
                        void* out, float* lse, int B, int n_h, int n_kv,
                        int L_max, int d, float scale, kvc_dtype dtype, int32_t* flag,
                        void* workspace, size_t ws_bytes, void* stream,
                        bool topk, const void* k_new = nullptr,
                        const void* v_new = nullptr, bool fused = false,
                        bool fp8 = false, float k_scale = 1.f, float v_scale = 1.f,
                        int window = 0, const int32_t* win_start = nullptr,
                        const int32_t* block_table = nullptr, int max_blocks = 0,
                        int num_blocks = 0, int page_shift = 0,
                        const void* k_scales = nullptr, const void* v_scales = nullptr,
                        bool fp4 = false, bool use_static = false) {
  // FP8 caches: q and out are bf16; the shape rules are those of bf16 with
  // d = 128 (checked by the caller).
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, L_max, d, dtype, K, topk, fused, window,
                                         fp8 ? kFmtFp8 : fp4 ? kFmtFp4 : kFmtPlain);
  if (c.status != KVC_OK) return c.status;
  if (!isfinite(scale)) return KVC_ERR_BAD_ARG;
  if (fp8 && !(isfinite(k_scale) && isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return KVC_ERR_BAD_ARG;
  if (!q || !k_cache || !v_cache || !seq_lens || !out || (topk && !idx) ||
      (fused && (!k_new || !v_new)) || (fp4 && (!k_scales || !v_scales)))
    return KVC_ERR_NULL_PTR;
  if (fp4 && (!aligned(k_scales, 8) || !aligned(v_scales, 8))) return KVC_ERR_MISALIGNED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 16) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)) ||
      (idx && !aligned(idx, 16)) || (flag && !aligned(flag, 4)) ||
      (fused && (!aligned(k_new, 16) || !aligned(v_new, 16))) ||
      (win_start && !aligned(win_start, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  const int64_t units = (int64_t)B * n_kv;
  if (use_static) {
    // the library's scratch replaces the workspace: the call must fit it
    const size_t rows = (size_t)B * n_h * c.P_max;
    const size_t partials = c.P_max > 1 ? round_up(rows * sizeof(float), 256) + rows * d * sizeof(float) : 0;
    if (units > kStaticCounterWords || partials > kStaticScratchBytes - kStaticPartialOff)
      return KVC_ERR_SCRATCH;
  } else {
    const int ws_status = check_workspace(c.ws, workspace, ws_bytes);
    if (ws_status != KVC_OK) return ws_status;
  }

  DenseParams p{};
  p.q = q;
  p.k = const_cast<void*>(k_cache);
  p.v = const_cast<void*>(v_cache);
  p.k_new = k_new; p.v_new = v_new;
  p.seq_lens = seq_lens;
  p.seq_lens_rw = fused ? const_cast<int32_t*>(seq_lens) : nullptr;
  p.idx = topk ? idx : nullptr; p.out = out; p.lse = lse;
  p.flag = (topk || fused) ? flag : nullptr;
  p.B = B; p.n_h = n_h; p.n_kv = n_kv; p.G = n_h / n_kv; p.L_max = L_max;
  p.persist = c.persist;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_static) {
    void* base = nullptr;
    if (static_scratch(&base) != hipSuccess) return KVC_ERR_HIP;
    int32_t* w = static_cast<int32_t*>(base);
    char* part = static_cast<char*>(base) + kStaticPartialOff;
    p.ws_cnt = nullptr; p.ws_lse = nullptr; p.ws_o = nullptr; p.ws_bcnt = nullptr; p.ws_ucnt = nullptr;
    if (c.P_max > 1) {
      p.ws_cnt = w;
      p.ws_lse = reinterpret_cast<float*>(part);
      p.ws_o = reinterpret_cast<float*>(part + round_up((size_t)B * n_h * c.P_max * sizeof(float), 256));
    }
    if (fused) {
      p.ws_bcnt = w + kStaticCounterWords;
      p.ws_ucnt = w + 2 * kStaticCounterWords;
    }
    p.ws_sched = p.persist ? w + kStaticSchedOff / sizeof(int32_t) : nullptr;
    if (launch_clear_static_counters(base, (int)units, B, s) != hipSuccess) return KVC_ERR_HIP;
  } else {
    fill_ws(p, c.ws, workspace, (size_t)c.P_max, fused);
  }
  p.d = d; p.K = topk ? K : 0; p.S = c.S; p.P_max = (int)c.P_max; p.even = c.even;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.out_scale = 1.f;
  p.window = window;
  p.win_start = window > 0 ? win_start : nullptr;
  p.block_table = block_table;
  p.max_blocks = max_blocks;
  p.num_blocks = num_blocks;
  p.page_shift = page_shift;
  if (block_table) {
    p.flag = flag;
    return launch_status(launch_dense_paged(p, s));
  }
  if (fp4) {
    p.k_scales = k_scales;
    p.v_scales = v_scales;
    return launch_status(launch_dense_fp4(p, s));
  }
  if (fp8) {
    p.scale_log2 *= k_scale;
    p.out_scale = v_scale;
    return launch_status(launch_dense_fp8(p, s));
  }
  if (dtype == KVC_BF16 && d == 128) return launch_status(launch_dense_mfma(p, topk, fused, s));
  return launch_status(launch_dense_generic(p, dtype, topk, fused, s));
}

size_t kvc_append_decode_attn_workspace_size(int B, int n_h, int n_kv, int L_max,
                                             int d, kvc_dtype dtype) {
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, L_max, d, dtype, 0, false, true);
  return c.status == KVC_OK ? c.ws.total : 0;
}

int kvc_append_decode_attn(const void* q, void* k_cache, void* v_cache,
                           int32_t* seq_lens, const void* k_new,
                           const void* v_new, void* out, float* lse, int B,
                           int n_h, int n_kv, int L_max, int d, float scale,
                           kvc_dtype dtype, int32_t* flag, void* workspace,
                           size_t ws_bytes, void* stream) {
  return dense_common(q, k_cache, v_cache, seq_lens, nullptr, 0, out, lse, B,
                      n_h, n_kv, L_max, d, scale, dtype, flag, workspace,
                      ws_bytes, stream, false, k_new, v_new, true);
}

int kvc_append_decode_attn_noalloc(const void* q, void* k_cache, void* v_cache,
                                   int32_t* seq_lens, const void* k_new, const void* v_new,
                                   void* out, float* lse, int B, int n_h, int n_kv, int L_max,
                                   int d, float scale, kvc_dtype dtype, int32_t* flag,
                                   void* stream) {
  return dense_common(q, k_cache, v_cache, seq_lens, nullptr, 0, out, lse, B, n_h, n_kv, L_max,
                      d, scale, dtype, flag, nullptr, 0, stream, false, k_new, v_new, true,
                      false, 1.f, 1.f, 0, nullptr, nullptr, 0, 0, 0, nullptr, nullptr, false,
                      /*use_static=*/true);
}

int kvc_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, void* out, float* lse, int B,
                    int n_h, int n_kv, int L_max, int d, float scale, kvc_dtype dtype,
                    void* workspace, size_t ws_bytes, void* stream) {
  return dense_common(q, k_cache, v_cache, seq_lens, nullptr, 0, out, lse, B,
                      n_h, n_kv, L_max, d, scale, dtype, nullptr, workspace,
                      ws_bytes, stream, false);
}

int kvc_decode_attn_topk(const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* seq_lens,
                         const int32_t* idx, int K, void* out, float* lse,
                         int B, int n_h, int n_kv, int L_max, int d,
                         float scale, kvc_dtype dtype, int32_t* flag,
                         void* workspace, size_t ws_bytes, void* stream) {
  return dense_common(q, k_cache, v_cache, seq_lens, idx, K, out, lse, B, n_h,
                      n_kv, L_max, d, scale, dtype, flag, workspace, ws_bytes,
                      stream, true);
}

size_t kvc_decode_attn_window_workspace_size(int B, int n_h, int n_kv, int L_max,
                                             int d, kvc_dtype dtype, int window) {
  if (window < 1) return 0;
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, L_max, d, dtype, 0, false, false, window);
  return c.status == KVC_OK ? c.ws.total : 0;
}

int kvc_decode_attn_window(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, const int32_t* win_start,
                           int window, void* out, float* lse, int B, int n_h,
                           int n_kv, int L_max, int d, float scale, kvc_dtype dtype,
                           void* workspace, size_t ws_bytes, void* stream) {
  if (window < 1) return KVC_ERR_BAD_ARG;
  return dense_common(q, k_cache, v_cache, seq_lens, nullptr, 0, out, lse, B,
                      n_h, n_kv, L_max, d, scale, dtype, nullptr, workspace,
                      ws_bytes, stream, false, nullptr, nullptr, false, false,
                      1.f, 1.f, window, win_start);
}

// Paged caches: block size a power of two in [8, 4096]; pools of at most
// 2^31 bytes (32-bit offsets with an out-of-range marker above them).
static int page_shift_of(int block_size) {
  if (block_size < 8 || block_size > 4096 || (block_size & (block_size - 1))) return -1;
  int sh = 0;
  while ((1 << sh) < block_size) ++sh;
  return sh;
}

static int check_paged(int B, int n_kv, int max_blocks, int num_blocks, int block_size,
                       int d, int elem, int& shift) {
  if (B < 0 || n_kv < 1 || max_blocks < 1 || num_blocks < 1 || d < 1) return KVC_ERR_BAD_SHAPE;
  shift = page_shift_of(block_size);
  if (shift < 0) return KVC_ERR_BAD_SHAPE;
  if ((int64_t)max_blocks * block_size >= kMaxOffset) return KVC_ERR_BAD_SHAPE;
  if ((int64_t)num_blocks * n_kv * block_size * d * elem > kMaxOffset) return KVC_ERR_BAD_SHAPE;
  return KVC_OK;
}

size_t kvc_decode_attn_paged_workspace_size(int B, int n_h, int n_kv, int max_blocks,
                                            int block_size, int d, kvc_dtype dtype) {
  if (page_shift_of(block_size) < 0 || max_blocks < 1 ||
      (int64_t)max_blocks * block_size >= kMaxOffset)
    return 0;
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, max_blocks * block_size, d, dtype, 0, false);
  return c.status == KVC_OK ? c.ws.total : 0;
}

int kvc_decode_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, int max_blocks,
                          const int32_t* seq_lens, void* out, float* lse, int B,
                          int n_h, int n_kv, int num_blocks, int block_size, int d,
                          float scale, kvc_dtype dtype, int32_t* flag, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (!good_dtype(dtype)) return KVC_ERR_BAD_DTYPE;
  int shift = 0;
  const int st = check_paged(B, n_kv, max_blocks, num_blocks, block_size, d, elem_bytes(dtype), shift);
  if (st != KVC_OK) return st;
  if (dtype != KVC_BF16 || d != 128) return KVC_ERR_UNSUPPORTED;
  if (!block_table) return KVC_ERR_NULL_PTR;
  if (!aligned(block_table, 4)) return KVC_ERR_MISALIGNED;
  return dense_common(q, k_pool, v_pool, seq_lens, nullptr, 0, out, lse, B, n_h, n_kv,
                      max_blocks * block_size, d, scale, dtype, flag, workspace, ws_bytes,
                      stream, false, nullptr, nullptr, false, false, 1.f, 1.f, 0, nullptr,
                      block_table, max_blocks, num_blocks, shift);
}

int kvc_append_paged(void* k_pool, void* v_pool, const int32_t* block_table,
                     int max_blocks, int32_t* seq_lens, const void* k_new,
                     const void* v_new, int B, int n_kv, int num_blocks,
                     int block_size, int d, kvc_dtype dtype, int32_t* flag, void* stream) {
  if (!good_dtype(dtype)) return KVC_ERR_BAD_DTYPE;
  int shift = 0;
  const int st = check_paged(B, n_kv, max_blocks, num_blocks, block_size, d, elem_bytes(dtype), shift);
  if (st != KVC_OK) return st;
  if ((d * elem_bytes(dtype)) % 16 != 0) return KVC_ERR_BAD_SHAPE;
  if (!k_pool || !v_pool || !block_table || !seq_lens || !k_new || !v_new) return KVC_ERR_NULL_PTR;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      (flag && !aligned(flag, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  AppendParams p{k_pool, v_pool, seq_lens, k_new, v_new, flag,
                 B, n_kv, max_blocks * block_size, d, elem_bytes(dtype), 1.f, 1.f,
                 block_table, max_blocks, num_blocks, shift};
  return launch_status(launch_append_paged(p, static_cast<hipStream_t>(stream)));
}

size_t kvc_decode_attn_fp8_workspace_size(int B, int n_h, int n_kv, int L_max,
                                          int d) {
  if (d != 128) return 0;
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, L_max, d, KVC_BF16, 0, false, false, 0,
                                         kFmtFp8);
  return c.status == KVC_OK ? c.ws.total : 0;
}

int kvc_decode_attn_fp8(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, void* out, float* lse, int B,
                        int n_h, int n_kv, int L_max, int d, float scale,
                        float k_scale, float v_scale, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (B < 0 || n_h < 1 || n_kv < 1 || L_max < 1 || d < 1) return KVC_ERR_BAD_SHAPE;
  if (d != 128) return KVC_ERR_UNSUPPORTED;
  return dense_common(q, k_cache, v_cache, seq_lens, nullptr, 0, out, lse, B,
                      n_h, n_kv, L_max, d, scale, KVC_BF16, nullptr, workspace,
                      ws_bytes, stream, false, nullptr, nullptr, false, true,
                      k_scale, v_scale);
}

size_t kvc_decode_attn_fp4_workspace_size(int B, int n_h, int n_kv, int L_max,
                                          int d) {
  if (d != 128) return 0;
  const DenseCheck c = check_dense_shape(B, n_h, n_kv, L_max, d, KVC_BF16, 0, false, false, 0,
                                         kFmtFp4);
  return c.status == KVC_OK ? c.ws.total : 0;
}

int kvc_decode_attn_fp4(const void* q, const void* k_codes, const void* k_scales,
                        const void* v_codes, const void* v_scales, const int32_t* seq_lens,
                        void* out, float* lse, int B, int n_h, int n_kv, int L_max, int d,
                        float scale, void* workspace, size_t ws_bytes, void* stream) {
  if (B < 0 || n_h < 1 || n_kv < 1 || L_max < 1 || d < 1) return KVC_ERR_BAD_SHAPE;
  if (d != 128) return KVC_ERR_UNSUPPORTED;
  return dense_common(q, k_codes, v_codes, seq_lens, nullptr, 0, out, lse, B, n_h, n_kv,
                      L_max, d, scale, KVC_BF16, nullptr, workspace, ws_bytes, stream, false,
                      nullptr, nullptr, false, false, 1.f, 1.f, 0, nullptr, nullptr, 0, 0, 0,
                      k_scales, v_scales, true);
}

size_t kvc_decode_attn_mla_workspace_size(int B, int n_h, int L_max, int d_c,
                                          int d_r) {
  // (the latent kernel exists for bf16 only; its workspace does not depend
  // on the element type)
  const MlaCheck c = check_mla_shape(B, n_h, L_max, d_c, d_r, KVC_BF16);
  return c.status == KVC_OK ? c.ws.total : 0;
}

int kvc_decode_attn_mla(const void* q, const void* ckv,
                        const int32_t* seq_lens, void* out, float* lse, int B,
                        int n_h, int L_max, int d_c, int d_r, float scale,
                        kvc_dtype dtype, void* workspace, size_t ws_bytes,
                        void* stream) {
  const MlaCheck c = check_mla_shape(B, n_h, L_max, d_c, d_r, dtype);
  if (c.status != KVC_OK) return c.status;
  if (!isfinite(scale)) return KVC_ERR_BAD_ARG;
  if (!q || !ckv || !seq_lens || !out) return KVC_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(ckv, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  const int ws_status = check_workspace(c.ws, workspace, ws_bytes);
  if (ws_status != KVC_OK) return ws_status;
  MlaParams p{};
  p.q = q; p.ckv = ckv; p.seq_lens = seq_lens; p.out = out; p.lse = lse;
  if (c.ws.total) {
    char* base = static_cast<char*>(workspace);
    p.ws_cnt = reinterpret_cast<int32_t*>(base + c.ws.cnt_off);
    p.ws_lse = reinterpret_cast<float*>(base + c.ws.lse_off);
    p.ws_o = reinterpret_cast<float*>(base + c.ws.o_off);
  }
  p.B = B; p.n_h = n_h; p.L_max = L_max; p.S = c.S; p.P_max = (int)c.P_max;
  p.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(launch_mla(p, static_cast<hipStream_t>(stream)));
}

size_t kvc_topk_select_workspace_size(int B, int R, int L_max, int K) {
  if (B < 1 || R < 1 || L_max < 1 || K < 1 || L_max >= kSelectMaxRow) return 0;
  return select_seg_plan((int64_t)B * R, L_max).bytes;
}

int kvc_topk_select(const float* scores, const int32_t* seq_lens, const int32_t* pool,
                    int P, int pool_block, int32_t* idx_out, int B, int R, int L_max,
                    int K, void* workspace, size_t ws_bytes, void* stream) {
  if (B < 0 || R < 1 || L_max < 1 || K < 1) return KVC_ERR_BAD_SHAPE;
  // rows are read through 32-bit byte offsets (with a step of slack)
  if (L_max >= kSelectMaxRow) return KVC_ERR_UNSUPPORTED;
  int words = 0;
  if (pool) {
    if (P < 1 || pool_block < 1) return KVC_ERR_BAD_SHAPE;
    const int64_t nblk = ((int64_t)L_max + pool_block - 1) / pool_block;
    words = (int)((nblk + 31) / 32);
    if (words > kSelectPoolWords) return KVC_ERR_UNSUPPORTED;
  }
  if (!scores || !seq_lens || !idx_out) return KVC_ERR_NULL_PTR;
  if (!aligned(scores, 4) || !aligned(seq_lens, 4) || !aligned(idx_out, 4) ||
      (pool && !aligned(pool, 4)))
    return KVC_ERR_MISALIGNED;
  if (B == 0) return KVC_OK;
  SelectParams p{};
  p.scores = scores; p.seq_lens = seq_lens; p.pool = pool; p.out = idx_out;
  p.B = B; p.R = R; p.L_max = L_max; p.K = K; p.P = pool ? P : 0;
  p.pool_block = pool ? pool_block : 1; p.pool_words = words;
  p.sel_words = select_map_words(L_max);
  p.S = 1;
  // the segmented form: a workspace of at least the queried size, no pool
  const SelectSegPlan sp = select_seg_plan((int64_t)B * R, L_max);
  if (workspace && !pool && sp.bytes > 0) {
    if (ws_bytes < sp.bytes) return KVC_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KVC_ERR_MISALIGNED;
    char* base = static_cast<char*>(workspace);
    p.S = sp.S; p.seg_len = sp.seg_len;
    p.ws_cnt = reinterpret_cast<int32_t*>(base + sp.cnt_off);
    p.ws_cand = reinterpret_cast<uint32_t*>(base + sp.cand_off);
    p.ws_ccnt = reinterpret_cast<int32_t*>(base + sp.ccnt_off);
  }
  return launch_status(launch_topk_select(p, static_cast<hipStream_t>(stream)));
}

size_t kvc_stream_read_sink_floats(size_t bytes) { return stream_read_blocks(bytes); }

int kvc_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink) return KVC_ERR_NULL_PTR;
  if (bytes % 16 || !aligned(src, 16)) return KVC_ERR_MISALIGNED;
  if (bytes == 0) return KVC_OK;
  return launch_status(launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int kvc_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!src || !dst) return KVC_ERR_NULL_PTR;
  if (bytes % 16 || !aligned(src, 16) || !aligned(dst, 16)) return KVC_ERR_MISALIGNED;
  if (bytes == 0) return KVC_OK;
  return launch_status(launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
