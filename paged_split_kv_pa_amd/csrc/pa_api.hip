// C-ABI front end of libpa_decode.so: argument validation, planning (path,
// partition grid, workspace layout) and kernel dispatch.  Declarations and
// the contract of every entry point are in include/pa_decode.h.
//
// Validation is pure host arithmetic and runs before the first HIP call, so
// every error status can be produced without a GPU.  The only host-side HIP
// calls are hipGetDevice / hipMalloc / hipFree for the library-owned
// workspace of pa_decode, hipGetLastError after launches, and the launches.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "pa_decode.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

// V1/V2 choice.  A value >= 0 is a context-length threshold (V1 iff the planning
// bound is <= it: the rule of project_6 commit a2a5dd8 page, decode paths, where it is
// 8192).  The default -1 selects the rule measured on MI355X (GPU-side step times,
// graph replay, GQA 8, head_dim 128, bf16): V1 iff the bound is at most 256 tokens, or
// the V1 grid (one work-group per sequence and KV head) alone already fills the device;
// otherwise V2.  (At 512 tokens and up to 16 sequences V2 is faster: its work split
// reaches more compute units than V1's S*Hkv work-groups.)
constexpr int64_t kMeasuredRule = -1;
constexpr int64_t kV1FillWorkgroups = 256;  // MI355X compute units
constexpr int64_t kV1MaxShortContext = 256;

std::atomic<int64_t>& v1_threshold() {
  static std::atomic<int64_t> t([] {
    const char* env = std::getenv("PA_V1_MAX_CONTEXT");
    if (env && *env) {
      char* end = nullptr;
      long long v = std::strtoll(env, &end, 10);
      if (end && *end == '\0' && v >= kMeasuredRule) return (int64_t)v;
    }
    return kMeasuredRule;
  }());
  return t;
}

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status_t ok() { return PA_OK; }

pa_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int element_bytes(int dtype) { return dtype == PA_F32 ? 4 : 2; }

// Sizes derived from validated dims.
struct Plan {
  int S, Hq, Hkv, D, G, NB, MB;
  // Strides in elements (block-table entries for bt_ss), zeros of pa_dims_t resolved.
  int64_t q_ss, q_sh, o_ss, o_sh, kv_sb, bt_ss;
  int64_t ctx_bound;  // planning bound on every context length
  int32_t P;          // partition size used by the kernels
  int64_t Pmax;       // partition-grid size
  size_t off_tmp, off_max, off_sum;  // phase-1 partials
  int64_t piece_slots;               // piece partials of a work split (see pa::Split)
  size_t off_pout, off_pmax, off_psum;
  size_t ws_bytes;
};

// Largest piece shift the partition size allows: pieces are whole multiples of four
// cache blocks (64 tokens; smaller pieces cost more in fixed per-work-group and phase-2
// work than they save in balance on MI355X), at most 2^kMaxPieceShift of them.
constexpr int kMinPieceTokens = 4 * pa::kBlockSize;
int max_piece_shift(int32_t P) {
  if (P <= 0 || P % kMinPieceTokens) return 0;
  int m = P / kMinPieceTokens, sh = 0;
  while (sh < pa::kMaxPieceShift && (m & 1) == 0) {
    m >>= 1;
    ++sh;
  }
  return sh;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

pa_status_t check_dims(const pa_dims_t* d) {
  if (!d) return fail(PA_ERR_NULL, "dims is NULL");
  if (d->dtype != PA_F32 && d->dtype != PA_F16 && d->dtype != PA_BF16)
    return fail(PA_ERR_DTYPE, "unknown dtype %d (expected PA_F32, PA_F16 or PA_BF16)", d->dtype);
  if (d->num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d is negative", d->num_seqs);
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
    return fail(PA_ERR_SHAPE, "head counts must be positive (Hq=%d, Hkv=%d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_blocks <= 0 || d->max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "num_blocks (%d) and max_blocks_per_seq (%d) must be positive",
                d->num_blocks, d->max_blocks_per_seq);
  if (d->head_dim <= 0 || d->block_size <= 0)
    return fail(PA_ERR_SHAPE, "head_dim (%d) and block_size (%d) must be positive", d->head_dim,
                d->block_size);
  if (d->head_dim != 128 && d->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (128 or 256)", d->head_dim);
  if (d->block_size != pa::kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (16)", d->block_size);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %d not built (1, 2, 4, 8, 16)", G);
  if ((int64_t)d->max_blocks_per_seq * pa::kBlockSize > (int64_t)0x3fffffff)
    return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq %d exceeds the 2^30-token context limit",
                d->max_blocks_per_seq);
  if (d->num_kv_heads > 65535 || d->num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads and num_seqs must be <= 65535 (grid limits)");
  return ok();
}

// Strides of pa_dims_t (0 = row-major) resolved and checked against what the kernels take:
// innermost stride 1, 16-byte aligned rows and blocks, out rows that do not overlap,
// values the kernels' 32-bit fields hold.
pa_status_t resolve_strides(const pa_dims_t* d, Plan* pl) {
  const int64_t D = d->head_dim, Hq = d->num_q_heads;
  const int64_t esz = element_bytes(d->dtype);
  if ((d->q_stride_dim != 0 && d->q_stride_dim != 1) ||
      (d->out_stride_dim != 0 && d->out_stride_dim != 1))
    return fail(PA_ERR_STRIDE, "the head-dim stride of q and out must be 1 (got %lld and %lld)",
                (long long)d->q_stride_dim, (long long)d->out_stride_dim);
  auto pick = [](int64_t v, int64_t dense) { return v == 0 ? dense : v; };
  pl->q_sh = pick(d->q_stride_head, D);
  pl->q_ss = pick(d->q_stride_seq, Hq * D);
  pl->o_sh = pick(d->out_stride_head, D);
  pl->o_ss = pick(d->out_stride_seq, Hq * D);
  pl->kv_sb = pick(d->kv_stride_block, (int64_t)d->num_kv_heads * pa::kBlockSize * D);
  pl->bt_ss = pick(d->bt_stride_seq, d->max_blocks_per_seq);
  const int64_t lim = 0x7fffffff;
  if (pl->q_sh < 0 || pl->q_ss < 0 || pl->o_sh < 0 || pl->o_ss < 0 || pl->kv_sb < 0 ||
      pl->bt_ss < 0)
    return fail(PA_ERR_STRIDE, "strides must not be negative");
  if (pl->q_sh > lim || pl->q_ss > lim || pl->bt_ss > lim)
    return fail(PA_ERR_UNSUPPORTED, "q strides and the block-table row stride must be below 2^31");
  if (pl->o_sh < D || pl->o_ss < (Hq - 1) * pl->o_sh + D)
    return fail(PA_ERR_STRIDE,
                "out rows overlap (out_stride_head %lld must be >= %lld and out_stride_seq %lld "
                ">= %lld)", (long long)pl->o_sh, (long long)D, (long long)pl->o_ss,
                (long long)((Hq - 1) * pl->o_sh + D));
  if (pl->kv_sb < (int64_t)d->num_kv_heads * pa::kBlockSize * D)
    return fail(PA_ERR_STRIDE, "kv_stride_block %lld is smaller than a block (%lld elements)",
                (long long)pl->kv_sb, (long long)d->num_kv_heads * pa::kBlockSize * D);
  if (pl->bt_ss < d->max_blocks_per_seq)
    return fail(PA_ERR_STRIDE, "bt_stride_seq %lld is smaller than max_blocks_per_seq %d",
                (long long)pl->bt_ss, d->max_blocks_per_seq);
  if ((pl->q_sh * esz) % 16 || (pl->q_ss * esz) % 16 || (pl->o_sh * esz) % 16 ||
      (pl->o_ss * esz) % 16 || (pl->kv_sb * esz) % 16)
    return fail(PA_ERR_ALIGN, "q / out rows and cache blocks must start on 16-byte boundaries "
                "(strides times %lld bytes must be multiples of 16)", (long long)esz);
  return ok();
}

pa_status_t make_plan(const pa_dims_t* d, int64_t max_context_len, int32_t partition_size,
                      bool need_partition, Plan* pl) {
  pa_status_t st = check_dims(d);
  if (st != PA_OK) return st;
  if ((st = resolve_strides(d, pl)) != PA_OK) return st;
  pl->S = d->num_seqs;
  pl->Hq = d->num_q_heads;
  pl->Hkv = d->num_kv_heads;
  pl->D = d->head_dim;
  pl->G = d->num_q_heads / d->num_kv_heads;
  pl->NB = d->num_blocks;
  pl->MB = d->max_blocks_per_seq;
  const int64_t cap = (int64_t)d->max_blocks_per_seq * pa::kBlockSize;
  if (max_context_len > cap)
    return fail(PA_ERR_SHAPE, "max_context_len %lld exceeds the block-table capacity %lld",
                (long long)max_context_len, (long long)cap);
  pl->ctx_bound = max_context_len > 0 ? max_context_len : cap;
  if (need_partition) {
    if (partition_size <= 0 || partition_size % pa::kBlockSize)
      return fail(PA_ERR_PARTITION,
                  "partition_size %d must be a positive multiple of the block size %d",
                  partition_size, pa::kBlockSize);
    pl->P = partition_size;
    pl->Pmax = (pl->ctx_bound + partition_size - 1) / partition_size;
    if (pl->Pmax > pa::kMaxReducePartitions)
      return fail(PA_ERR_UNSUPPORTED, "%lld partitions per sequence exceed the limit %d",
                  (long long)pl->Pmax, pa::kMaxReducePartitions);
  } else {
    // V1: one partition spanning the whole bound, rounded up to whole blocks.
    pl->P = (int32_t)(((pl->ctx_bound + pa::kBlockSize - 1) / pa::kBlockSize) * pa::kBlockSize);
    pl->Pmax = 1;
  }
  const size_t rows = (size_t)pl->S * pl->Hq * (size_t)pl->Pmax;
  pl->off_tmp = 0;
  pl->off_max = align256(rows * pl->D * sizeof(float));
  pl->off_sum = pl->off_max + align256(rows * sizeof(float));
  const size_t end = pl->off_sum + align256(rows * sizeof(float));
  const int msh = need_partition ? max_piece_shift(pl->P) : 0;
  const int64_t items = (int64_t)pl->S * pl->Hkv * pl->Pmax;
  pl->piece_slots = msh > 0 ? std::min<int64_t>(pa::kMaxPieceSlots, items << msh) : 0;
  const size_t prow = (size_t)pl->piece_slots * pl->G;
  pl->off_pout = end;
  pl->off_pmax = pl->off_pout + align256(prow * pl->D * sizeof(float));
  pl->off_psum = pl->off_pmax + align256(prow * sizeof(float));
  pl->ws_bytes = pl->off_psum + align256(prow * sizeof(float));
  return ok();
}

// ---- single-launch V2 (see fused_merge in pa_kernels.hip) --------------------------------
// Setting: 0 (default) two launches; 1 one launch wherever it applies.  Measured on
// MI355X the single launch is slower at 100K tokens (41.8 vs 38.8 us/step: its merge
// waits on a chain of device-scope round trips after the last partition, where the second
// launch reads partials the kernel boundary has already written back) and equal on the
// mixed batch, so it is not the default.  Env PA_FUSED sets the initial value.
std::atomic<int> g_fused{-2};  // -2: not yet read from the environment

// Prefill PV form (see pa_set_prefill_mode): 0 one fp16 part (with the two-part
// recompute for bf16 V beyond fp16's range), 1 always two parts.  Env PA_PREFILL_MODE
// sets the initial value.
std::atomic<int> g_prefill_mode{-2};

// Prefill chunk setting (see pa_set_prefill_split): -1 automatic, 0 the non-planned grid,
// >= pa::kPrefillMinChunk a fixed chunk length in tiles.  Env PA_PREFILL_SPLIT.
std::atomic<int> g_prefill_split{-2};

int prefill_split_setting() {
  int v = g_prefill_split.load(std::memory_order_relaxed);
  if (v == -2) {
    v = -1;
    const char* e = std::getenv("PA_PREFILL_SPLIT");
    if (e && *e) {
      char* end = nullptr;
      const long x = std::strtol(e, &end, 10);
      if (end && *end == '\0' && (x == -1 || x == 0 || (x >= pa::kPrefillMinChunk && x <= (1 << 20))))
        v = (int)x;
    }
    g_prefill_split.store(v, std::memory_order_relaxed);
  }
  return v;
}

int prefill_mode_setting() {
  int v = g_prefill_mode.load(std::memory_order_relaxed);
  if (v == -2) {
    v = 0;
    const char* e = std::getenv("PA_PREFILL_MODE");
    if (e && (e[0] == '0' || e[0] == '1') && e[1] == '\0') v = e[0] - '0';
    g_prefill_mode.store(v, std::memory_order_relaxed);
  }
  return v;
}

int fused_setting() {
  int v = g_fused.load(std::memory_order_relaxed);
  if (v == -2) {
    v = 0;
    const char* e = std::getenv("PA_FUSED");
    if (e && (e[0] == '0' || e[0] == '1') && e[1] == '\0') v = e[0] - '0';
    g_fused.store(v, std::memory_order_relaxed);
  }
  return v;
}

// ---- work split (see pa::Split) --------------------------------------------------------
// Setting: pieces -1 = automatic, 0 = off, 2..16 = cut every item from first_item on.
std::atomic<int32_t> g_split_pieces{-1};
std::atomic<int64_t> g_split_first{0};

// Compute units of the current device (cached per device).
std::atomic<int> g_cu_count[64];

pa_status_t compute_units(int* ncu) {
  int dev = 0;
  pa_status_t st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != PA_OK) return st;
  if (dev < 0 || dev >= 64) return fail(PA_ERR_INTERNAL, "device id %d out of range", dev);
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    st = hip_status(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
                          "hipDeviceGetAttribute(compute units)");
    if (st != PA_OK) return st;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  *ncu = n;
  return ok();
}

int floor_log2(int64_t x) {
  int r = -1;
  while (x > 0) {
    x >>= 1;
    ++r;
  }
  return r;
}

// The split of a V2 phase-1 launch.  Automatic rule, with C compute units and W items
// dispatched round-robin over them (measured on MI355X: a CU's HBM bandwidth is capped
// far below what the whole device can stream, so the time of a launch follows the
// most-loaded CUs):
//   W <  C: every item is cut into the largest 2^s pieces with W * 2^s <= 2C, so that a
//           small grid still reaches every compute unit (two one-wave work-groups per
//           unit measured faster than one two-wave one: 8K tokens x 4 KV heads,
//           10.9 vs 11.3 us/step);
//   W >= C: the last r = W mod C items, if 0 < r <= C/2, are cut into the fewest
//           2^s >= 2 pieces with r * 2^s a multiple of C, so that every CU ends with
//           the same load; failing that, into the most pieces allowed.  (With r > C/2
//           the busy CUs of the last round already draw most of the bandwidth, and a
//           cut measured slower.)
pa_status_t plan_split(const Plan& pl, pa::Split* sp) {
  *sp = pa::Split();
  const int msh = max_piece_shift(pl.P);
  const int64_t items = (int64_t)pl.S * pl.Hkv * pl.Pmax;
  const int32_t mode = g_split_pieces.load(std::memory_order_relaxed);
  if (msh == 0 || mode == 0 || mode == 1 || items == 0) return ok();
  int64_t first = 0;
  int shift = 0;
  if (mode > 1) {
    shift = std::min(floor_log2(mode), msh);
    first = std::min<int64_t>(std::max<int64_t>(g_split_first.load(), 0), items);
  } else {
    int ncu = 0;
    pa_status_t st = compute_units(&ncu);
    if (st != PA_OK) return st;
    if (items < ncu) {
      shift = std::min(floor_log2(2 * (int64_t)ncu / items), msh);
      first = 0;
    } else {
      const int64_t rem = items % ncu;
      if (rem == 0 || 2 * rem > ncu) return ok();
      first = items - rem;
      shift = 0;
      for (int s = 1; s <= msh && (rem << s) <= pl.piece_slots; ++s) {
        shift = s;
        if ((rem << s) % ncu == 0) break;
      }
    }
  }
  if (shift <= 0) return ok();
  // Only as many items as the piece area holds are cut (the last ones).
  first = std::max<int64_t>(first, items - (pl.piece_slots >> shift));
  if (first >= items) return ok();
  if (first + ((items - first) << shift) > pa::kMaxSplitGrid) return ok();
  sp->first = (int32_t)first;
  sp->shift = shift;
  return ok();
}

pa_status_t check_tensors(const void* out, const void* q, const void* k, const void* v,
                          const int32_t* bt, const int32_t* ctx) {
  if (!out || !q || !k || !v || !bt || !ctx)
    return fail(PA_ERR_NULL, "a tensor pointer is NULL (out=%p q=%p k=%p v=%p bt=%p ctx=%p)", out,
                q, k, v, (const void*)bt, (const void*)ctx);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(PA_ERR_ALIGN, "out, q, k_cache and v_cache must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(bt) | reinterpret_cast<uintptr_t>(ctx)) & 3u)
    return fail(PA_ERR_ALIGN, "block_tables and context_lens must be 4-byte aligned");
  return ok();
}

pa_status_t check_scale(float scale) {
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale must be finite");
  return ok();
}

// The split with its piece-area pointers inside workspace ws.
pa::Split split_in(const Plan& pl, const pa::Split& sp, const void* ws) {
  pa::Split r = sp;
  if (r.shift == 0 || !ws) return pa::Split();
  char* base = static_cast<char*>(const_cast<void*>(ws));
  r.piece_out = reinterpret_cast<float*>(base + pl.off_pout);
  r.piece_max = reinterpret_cast<float*>(base + pl.off_pmax);
  r.piece_sum = reinterpret_cast<float*>(base + pl.off_psum);
  return r;
}

pa::AttnArgs attn_args(const Plan& pl, void* out, const void* q, const void* k, const void* v,
                       const int32_t* bt, const int32_t* ctx, float scale, void* ws,
                       const pa::Split& sp) {
  pa::AttnArgs a;
  a.out = out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.bt = bt;
  a.ctx = ctx;
  a.q_ss = (int32_t)pl.q_ss;
  a.q_sh = (int32_t)pl.q_sh;
  a.bt_ss = (int32_t)pl.bt_ss;
  a.o_ss = pl.o_ss;
  a.o_sh = pl.o_sh;
  a.kv_sb = pl.kv_sb;
  char* base = static_cast<char*>(ws);
  a.tmp_out = base ? reinterpret_cast<float*>(base + pl.off_tmp) : nullptr;
  a.max_logits = base ? reinterpret_cast<float*>(base + pl.off_max) : nullptr;
  a.exp_sums = base ? reinterpret_cast<float*>(base + pl.off_sum) : nullptr;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  a.Hq = pl.Hq;
  a.Hkv = pl.Hkv;
  a.NB = pl.NB;
  a.MB = pl.MB;
  a.P = pl.P;
  a.Pmax = (int32_t)pl.Pmax;
  a.split = split_in(pl, sp, ws);
  return a;
}

pa_status_t run_partition(const pa_dims_t* dims, const Plan& pl, void* out, const void* q,
                          const void* k, const void* v, const int32_t* bt, const int32_t* ctx,
                          float scale, void* ws, hipStream_t st, const pa::Split& sp,
                          hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  pa::AttnArgs a = attn_args(pl, out, q, k, v, bt, ctx, scale, ws, sp);
  return hip_status(pa::launch_attention(dims->dtype, pl.D, pl.G, a, pl.S, st, e0, e1),
                    "attention kernel launch");
}

pa_status_t run_reduce(const pa_dims_t* dims, const Plan& pl, void* out, const int32_t* ctx,
                       const void* ws, hipStream_t st, const pa::Split& sp) {
  pa::ReduceArgs r;
  const char* base = static_cast<const char*>(ws);
  r.out = out;
  r.o_ss = pl.o_ss;
  r.o_sh = pl.o_sh;
  r.ctx = ctx;
  r.tmp_out = reinterpret_cast<const float*>(base + pl.off_tmp);
  r.max_logits = reinterpret_cast<const float*>(base + pl.off_max);
  r.exp_sums = reinterpret_cast<const float*>(base + pl.off_sum);
  r.Hq = pl.Hq;
  r.Hkv = pl.Hkv;
  r.MB = pl.MB;
  r.P = pl.P;
  r.Pmax = (int32_t)pl.Pmax;
  r.split = split_in(pl, sp, ws);
  return hip_status(pa::launch_reduce(dims->dtype, pl.D, r, pl.S, st), "phase-2 reduce launch");
}

// Library-owned workspaces, grow-only, one per device for decode and one for prefill
// (so that a decode and a prefill call overlapping on two streams do not share memory).
constexpr int kMaxDevices = 64;
enum WsKind { kWsDecode = 0, kWsPrefill = 1 };
std::mutex g_ws_mutex;
void* g_ws_ptr[2][kMaxDevices] = {};
size_t g_ws_size[2][kMaxDevices] = {};

// Library-managed workspaces (pa_decode's, pa_decode_noalloc's and pa_prefill's) start
// with a counter region (pa::kFusedCounterBytes, zero between launches: the single-launch
// V2's counters and flags, the prefill chunks' arrival counters); the rest follows.  The
// counters are zeroed (by a fill kernel on the caller's stream) whenever the memory is new.
pa_status_t owned_workspace(WsKind kind, size_t bytes, hipStream_t stream, void** out) {
  bytes += pa::kFusedCounterBytes;
  int dev = 0;
  pa_status_t st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != PA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_INTERNAL, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  void*& ptr = g_ws_ptr[kind][dev];
  size_t& size = g_ws_size[kind][dev];
  if (size < bytes) {
    if (ptr) {
      st = hip_status(hipFree(ptr), "hipFree(workspace)");
      ptr = nullptr;
      size = 0;
      if (st != PA_OK) return st;
    }
    void* p = nullptr;
    st = hip_status(hipMalloc(&p, bytes), "hipMalloc(workspace)");
    if (st != PA_OK) return st;
    st = hip_status(pa::launch_zero_words(static_cast<uint32_t*>(p),
                                          pa::kFusedCounterBytes / 4, stream),
                    "workspace counter fill");
    if (st != PA_OK) {
      (void)hipFree(p);
      return st;
    }
    ptr = p;
    size = bytes;
  }
  *out = ptr;
  return ok();
}

// Static scratch of pa_decode_noalloc: the V2 workspace of callers that cannot allocate.
// Each device holds its own copy of the array for the life of the process.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device address comes
// from hipGetSymbolAddress, once per device (with that device current), and only that
// address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch's device address on the current device; on the first call per device the
// counter region at its start is zeroed by a fill kernel on `stream`.
pa_status_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  pa_status_t st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != PA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_INTERNAL, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != PA_OK) return st;
    if (!p) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    st = hip_status(pa::launch_zero_words(static_cast<uint32_t*>(p),
                                          pa::kFusedCounterBytes / 4, stream),
                    "scratch counter fill");
    if (st != PA_OK) return st;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

int32_t choose(const Plan& pl, int32_t partition_size) {
  const int64_t t = v1_threshold().load();
  if (t >= 0) return pl.ctx_bound <= t ? PA_PATH_V1 : PA_PATH_V2;
  (void)partition_size;
  const bool short_context = pl.ctx_bound <= kV1MaxShortContext;
  const bool v1_fills = (int64_t)pl.S * pl.Hkv >= kV1FillWorkgroups;
  return (short_context || v1_fills) ? PA_PATH_V1 : PA_PATH_V2;
}

// Whether a V2 call with this plan and split runs as a single launch (given a
// library-managed workspace): the setting asks for it, the counters cover every (sequence,
// KV head), the merge work-groups fit in the second grid row, the merge's LDS holds every
// partial state of a head, and workspace offsets fit 31 bits.
bool fused_applies(const Plan& pl, const pa::Split& sp) {
  if (fused_setting() != 1) return false;
  pa::AttnArgs a;
  a.Pmax = (int32_t)pl.Pmax;
  a.Hkv = pl.Hkv;
  a.split = sp;
  const long long n1 = pa::phase1_workgroups(a, pl.S);
  const long long m = (long long)pl.S * pl.Hq * pa::kFusedChunks;
  return (long long)pl.S * pl.Hkv <= pa::kFusedMaxGroups && m <= n1 && m <= pa::kFusedMaxMerge &&
         pa::fold_states(a, pl.S) <= pa::kFusedMaxFold && pl.ws_bytes < (size_t(1) << 31);
}

// Where the V2 workspace of a decode call comes from.
enum class Ws { kCaller, kOwned, kStatic };

pa_status_t decode_impl(const pa_dims_t* dims, void* out, const void* q, const void* k,
                        const void* v, const int32_t* bt, const int32_t* ctx, float scale,
                        int32_t partition_size, void* stream, void* workspace,
                        size_t workspace_bytes, Ws wsm, int64_t max_context_len,
                        int32_t path, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  if (path != PA_PATH_AUTO && path != PA_PATH_V1 && path != PA_PATH_V2)
    return fail(PA_ERR_SHAPE, "path %d is not PA_PATH_AUTO, PA_PATH_V1 or PA_PATH_V2", path);
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, partition_size, true, &pl);
  if (st != PA_OK) return st;
  if (pl.S == 0) return ok();
  if ((st = check_tensors(out, q, k, v, bt, ctx)) != PA_OK) return st;
  if ((st = check_scale(scale)) != PA_OK) return st;
  const int32_t take = path == PA_PATH_AUTO ? choose(pl, partition_size) : path;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint32_t* counters = nullptr;  // library-managed workspaces: the counter region
  if (wsm == Ws::kStatic) {
    void* base = nullptr;
    if ((st = scratch_address(hs, &base)) != PA_OK) return st;
    const size_t room = PA_NOALLOC_SCRATCH_BYTES - pa::kFusedCounterBytes;
    if (take == PA_PATH_V2 && pl.ws_bytes > room)
      return fail(PA_ERR_WORKSPACE,
                  "this call needs %zu bytes of workspace; the static scratch of "
                  "pa_decode_noalloc holds %zu (use pa_decode_ex with a caller workspace)",
                  pl.ws_bytes, room);
    counters = static_cast<uint32_t*>(base);
    workspace = static_cast<char*>(base) + pa::kFusedCounterBytes;
    workspace_bytes = room;
  }
  if (take == PA_PATH_V1) {
    Plan p1;
    if ((st = make_plan(dims, max_context_len, 0, false, &p1)) != PA_OK) return st;
    return run_partition(dims, p1, out, q, k, v, bt, ctx, scale, nullptr, hs, pa::Split(), e0,
                         e1);
  }
  if (wsm == Ws::kOwned) {
    void* base = nullptr;
    if ((st = owned_workspace(kWsDecode, pl.ws_bytes, hs, &base)) != PA_OK) return st;
    counters = static_cast<uint32_t*>(base);
    workspace = static_cast<char*>(base) + pa::kFusedCounterBytes;
  } else if (wsm == Ws::kCaller) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL; V2 needs %zu bytes",
                                pl.ws_bytes);
    if (workspace_bytes < pl.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, pl.ws_bytes);
    if (!aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  pa::Split sp;
  if ((st = plan_split(pl, &sp)) != PA_OK) return st;
  if (counters && fused_applies(pl, sp)) {
    // Single launch: phase 1 and the merge in one grid (library-managed workspace only:
    // its counter region is zero between launches).
    pa::AttnArgs a = attn_args(pl, out, q, k, v, bt, ctx, scale, workspace, sp);
    a.fused = 1;
    a.fused_m = (int32_t)((long long)pl.S * pl.Hq * pa::kFusedChunks);
    a.counters = counters;
    return hip_status(pa::launch_attention(dims->dtype, pl.D, pl.G, a, pl.S, hs, e0, e1),
                      "single-launch decode");
  }
  if ((st = run_partition(dims, pl, out, q, k, v, bt, ctx, scale, workspace, hs, sp, e0, e1)) !=
      PA_OK)
    return st;
  return run_reduce(dims, pl, out, ctx, workspace, hs, sp);
}

// Validation of prefill dims (no pointer is looked at); *G receives Hq / Hkv.
pa_status_t check_prefill_dims(const pa_prefill_dims_t* d, int* G_out) {
  if (!d) return fail(PA_ERR_NULL, "dims is NULL");
  if (d->dtype != PA_F32 && d->dtype != PA_F16 && d->dtype != PA_BF16)
    return fail(PA_ERR_DTYPE, "unknown dtype %d", d->dtype);
  if (d->num_seqs < 0 || d->num_tokens < 0)
    return fail(PA_ERR_SHAPE, "num_seqs (%d) and num_tokens (%d) must be non-negative",
                d->num_seqs, d->num_tokens);
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_blocks <= 0 || d->max_blocks_per_seq <= 0 || d->head_dim <= 0 ||
      d->block_size <= 0)
    return fail(PA_ERR_SHAPE, "num_blocks, max_blocks_per_seq, head_dim and block_size must be "
                "positive");
  if (d->max_query_len > d->num_tokens)
    return fail(PA_ERR_SHAPE, "max_query_len %d exceeds num_tokens %d", d->max_query_len,
                d->num_tokens);
  if (d->dtype == PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "prefill is built for fp16 and bf16 (matrix cores)");
  if (d->head_dim != 128 && d->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "prefill is built for head_dim 128 and 256 (got %d)",
                d->head_dim);
  if (d->block_size != pa::kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (16)", d->block_size);
  const int G = d->num_q_heads / d->num_kv_heads;
  *G_out = G;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %d not built (1, 2, 4, 8, 16)", G);
  if ((int64_t)d->max_blocks_per_seq * pa::kBlockSize > (int64_t)0x3fffffff)
    return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq %d exceeds the 2^30-token limit",
                d->max_blocks_per_seq);
  if ((int64_t)d->max_blocks_per_seq * pa::kBlockSize + d->num_tokens > (int64_t)0x7fffffff)
    return fail(PA_ERR_UNSUPPORTED, "prefix bound plus num_tokens exceeds 2^31 - 1 keys");
  if (d->num_kv_heads > 65535 || d->num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads and num_seqs must be <= 65535 (grid limits)");
  return ok();
}

// The planned schedule's needs for these dims under the current settings: fills the plan
// fields of a (bounds, compute units, settings) and *bytes with the workspace bytes the
// call needs, counter region included (0: the grid schedule, no workspace).
pa_status_t prefill_plan(const pa_prefill_dims_t* d, int G, pa::PrefillArgs& a, size_t* bytes) {
  *bytes = 0;
  a.T = d->num_tokens;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.NB = d->num_blocks;
  a.MB = d->max_blocks_per_seq;
  a.precise = prefill_mode_setting();
  a.max_query_len = d->max_query_len > 0 ? d->max_query_len : d->num_tokens;
  a.chunk = prefill_split_setting();
  if (a.precise || a.chunk == 0 || d->num_seqs <= 0 || d->num_seqs > pa::kOrderMaxSeqs ||
      d->num_tokens <= 0)
    return ok();
  // A call that cannot take the planned schedule is told apart without the device.
  a.ncu = 1;
  if (pa::prefill_plan_bytes(d->head_dim, G, d->num_seqs, a) == 0) return ok();
  int ncu = 0;
  pa_status_t st = compute_units(&ncu);
  if (st != PA_OK) return st;
  a.ncu = ncu;
  const size_t b = pa::prefill_plan_bytes(d->head_dim, G, d->num_seqs, a);
  if (b > 0) *bytes = b + pa::kFusedCounterBytes;
  return ok();
}

// Plan, partial-state and counter pointers of a prefill workspace at base (256-byte
// aligned, bytes from prefill_plan).
void prefill_carve(pa::PrefillArgs& a, int head_dim, void* base) {
  a.counters = static_cast<uint32_t*>(base);  // zero between launches
  char* ws = static_cast<char*>(base) + pa::kFusedCounterBytes;
  const size_t rows = (size_t)pa::prefill_rows(head_dim);
  const size_t o_bytes = align256((size_t)a.slot_bound * rows * head_dim * 4);
  const size_t s_bytes = align256((size_t)a.slot_bound * rows * 4);
  a.plan = reinterpret_cast<int32_t*>(ws);
  a.part_o = reinterpret_cast<float*>(ws + pa::prefill_plan_words_bytes(a.item_bound));
  a.part_m = reinterpret_cast<float*>(reinterpret_cast<char*>(a.part_o) + o_bytes);
  a.part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(a.part_m) + s_bytes);
}

pa_status_t prefill_impl(const pa_prefill_dims_t* d, void* out, const void* q, const void* kn,
                         const void* vn, const void* kc, const void* vc, const int32_t* bt,
                         const int32_t* ctx, const int32_t* qs, float scale, Ws wsm,
                         void* workspace, size_t workspace_bytes, void* stream, hipEvent_t e0,
                         hipEvent_t e1) {
  int G = 0;
  pa_status_t st = check_prefill_dims(d, &G);
  if (st != PA_OK) return st;
  if ((st = check_scale(scale)) != PA_OK) return st;
  if (d->num_seqs == 0 || d->num_tokens == 0) return ok();
  if (!out || !q || !kn || !vn || !kc || !vc || !bt || !ctx || !qs)
    return fail(PA_ERR_NULL, "a tensor pointer is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(kn) || !aligned16(vn) || !aligned16(kc) ||
      !aligned16(vc))
    return fail(PA_ERR_ALIGN, "out, q, k_new, v_new and the caches must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(bt) | reinterpret_cast<uintptr_t>(ctx) |
       reinterpret_cast<uintptr_t>(qs)) & 3u)
    return fail(PA_ERR_ALIGN, "block_tables, context_lens and query_start must be 4-byte aligned");
  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_new = kn;
  a.v_new = vn;
  a.k_cache = kc;
  a.v_cache = vc;
  a.bt = bt;
  a.ctx = ctx;
  a.query_start = qs;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  size_t bytes = 0;
  if ((st = prefill_plan(d, G, a, &bytes)) != PA_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (bytes > 0) {
    void* base = nullptr;
    if (wsm == Ws::kOwned) {
      if ((st = owned_workspace(kWsPrefill, bytes - pa::kFusedCounterBytes, hs, &base)) != PA_OK)
        return st;
    } else {
      if (!workspace)
        return fail(PA_ERR_WORKSPACE, "workspace is NULL; this prefill needs %zu bytes", bytes);
      if (workspace_bytes < bytes)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    workspace_bytes, bytes);
      if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PA_ERR_ALIGN, "the prefill workspace must be 256-byte aligned");
      base = workspace;
    }
    prefill_carve(a, d->head_dim, base);
  }
  return hip_status(pa::launch_prefill(d->dtype, G, d->head_dim, a, d->num_seqs, a.max_query_len,
                                       hs, e0, e1),
                    "prefill launch");
}

}  // namespace

extern "C" {

pa_status_t pa_decode(const pa_dims_t* dims, void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, int32_t partition_size,
                      void* stream) {
  try {
    return decode_impl(dims, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       partition_size, stream, nullptr, 0, Ws::kOwned, 0, PA_PATH_AUTO);
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

pa_status_t pa_decode_noalloc(const pa_dims_t* dims, void* out, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, int32_t partition_size, void* stream) {
  try {
    return decode_impl(dims, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       partition_size, stream, nullptr, 0, Ws::kStatic, 0, PA_PATH_AUTO);
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

size_t pa_workspace_bytes(const pa_dims_t* dims, int64_t max_context_len,
                          int32_t partition_size) {
  Plan pl;
  if (make_plan(dims, max_context_len, partition_size, true, &pl) != PA_OK) return 0;
  return pl.ws_bytes;
}

pa_status_t pa_workspace_layout(const pa_dims_t* dims, int64_t max_context_len,
                                int32_t partition_size, int64_t* layout) {
  if (!layout) return fail(PA_ERR_NULL, "layout is NULL");
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, partition_size, true, &pl);
  if (st != PA_OK) return st;
  const int64_t v[PA_LAYOUT_FIELDS] = {pl.Pmax,
                                       (int64_t)pl.off_tmp,
                                       (int64_t)pl.off_max,
                                       (int64_t)pl.off_sum,
                                       pl.piece_slots,
                                       (int64_t)pl.off_pout,
                                       (int64_t)pl.off_pmax,
                                       (int64_t)pl.off_psum,
                                       (int64_t)pl.ws_bytes};
  for (int i = 0; i < PA_LAYOUT_FIELDS; ++i) layout[i] = v[i];
  return ok();
}

pa_status_t pa_decode_ex(const pa_dims_t* dims, void* out, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, int32_t partition_size,
                         void* stream, void* workspace, size_t workspace_bytes,
                         int64_t max_context_len, int32_t path) {
  try {
    return decode_impl(dims, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       partition_size, stream, workspace, workspace_bytes, Ws::kCaller,
                       max_context_len, path);
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

pa_status_t pa_decode_profiled(const pa_dims_t* dims, void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int32_t partition_size, void* stream, void* workspace,
                               size_t workspace_bytes, int64_t max_context_len, int32_t path,
                               void* attn_start_event, void* attn_stop_event) {
  try {
    return decode_impl(dims, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       partition_size, stream, workspace, workspace_bytes,
                       workspace == nullptr ? Ws::kOwned : Ws::kCaller, max_context_len, path,
                       static_cast<hipEvent_t>(attn_start_event),
                       static_cast<hipEvent_t>(attn_stop_event));
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

pa_status_t pa_v2_partition(const pa_dims_t* dims, void* out, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int32_t partition_size, int64_t max_context_len,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, partition_size, true, &pl);
  if (st != PA_OK) return st;
  if (pl.S == 0) return ok();
  if ((st = check_tensors(out, q, k_cache, v_cache, block_tables, context_lens)) != PA_OK)
    return st;
  if ((st = check_scale(scale)) != PA_OK) return st;
  if (!workspace || workspace_bytes < pl.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace %p of %zu bytes; %zu needed", workspace,
                workspace_bytes, pl.ws_bytes);
  if (!aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return run_partition(dims, pl, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       workspace, static_cast<hipStream_t>(stream), pa::Split());
}

pa_status_t pa_v2_reduce(const pa_dims_t* dims, void* out, const int32_t* context_lens,
                         int32_t partition_size, int64_t max_context_len,
                         const void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, partition_size, true, &pl);
  if (st != PA_OK) return st;
  if (pl.S == 0) return ok();
  if (!out || !context_lens) return fail(PA_ERR_NULL, "out or context_lens is NULL");
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return fail(PA_ERR_ALIGN, "out must be 16-byte aligned and context_lens 4-byte aligned");
  if (!workspace || workspace_bytes < pl.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace %p of %zu bytes; %zu needed", workspace,
                workspace_bytes, pl.ws_bytes);
  if (!aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return run_reduce(dims, pl, out, context_lens, workspace, static_cast<hipStream_t>(stream),
                    pa::Split());
}

pa_status_t pa_v1(const pa_dims_t* dims, void* out, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_tables,
                  const int32_t* context_lens, float scale, int64_t max_context_len,
                  void* stream) {
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, 0, false, &pl);
  if (st != PA_OK) return st;
  if (pl.S == 0) return ok();
  if ((st = check_tensors(out, q, k_cache, v_cache, block_tables, context_lens)) != PA_OK)
    return st;
  if ((st = check_scale(scale)) != PA_OK) return st;
  return run_partition(dims, pl, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       nullptr, static_cast<hipStream_t>(stream), pa::Split());
}

int32_t pa_choose_path(const pa_dims_t* dims, int64_t max_context_len, int32_t partition_size) {
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, 0, false, &pl);
  if (st != PA_OK) return st;
  return choose(pl, partition_size);
}

void pa_set_v1_max_context(int64_t tokens) {
  v1_threshold().store(tokens < 0 ? kMeasuredRule : tokens);
}

int64_t pa_get_v1_max_context(void) { return v1_threshold().load(); }

int64_t pa_num_partitions(int64_t n, int32_t partition_size) {
  if (n < 0 || partition_size <= 0) return -1;
  return (n + partition_size - 1) / partition_size;
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

void pa_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = -1;
  bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (int k = 0; k < 2; ++k) {
    for (int d = 0; d < kMaxDevices; ++d) {
      if (!g_ws_ptr[k][d]) continue;
      if (hipSetDevice(d) == hipSuccess) (void)hipFree(g_ws_ptr[k][d]);
      g_ws_ptr[k][d] = nullptr;
      g_ws_size[k][d] = 0;
    }
  }
  if (have_cur) (void)hipSetDevice(cur);
}

const char* pa_version(void) { return "pa_decode 0.1.0 gfx950"; }

pa_status_t pa_set_mfma_variant(int32_t variant) {
  if (pa::set_mfma_variant(variant) != 0)
    return fail(PA_ERR_UNSUPPORTED, "matrix-core variant %d unknown (-1, 0, 1, 2 or 3)", variant);
  return ok();
}

int32_t pa_get_mfma_variant(void) { return pa::get_mfma_variant(); }

pa_status_t pa_copy_blocks(void* k_cache, void* v_cache, int64_t block_bytes, int64_t num_blocks,
                           const int32_t* block_pairs, int64_t num_pairs, void* stream) {
  return pa_copy_blocks_profiled(k_cache, v_cache, block_bytes, num_blocks, block_pairs,
                                 num_pairs, stream, nullptr, nullptr);
}

pa_status_t pa_copy_blocks_profiled(void* k_cache, void* v_cache, int64_t block_bytes,
                                    int64_t num_blocks, const int32_t* block_pairs,
                                    int64_t num_pairs, void* stream, void* start_event,
                                    void* stop_event) {
  try {
    if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs %lld is negative", (long long)num_pairs);
    if (block_bytes <= 0 || block_bytes % 16 || block_bytes > (int64_t)0x7fffffff)
      return fail(PA_ERR_SHAPE, "block_bytes %lld must be a positive multiple of 16 below 2^31",
                  (long long)block_bytes);
    if (num_blocks <= 0 || num_blocks > (int64_t)0x7fffffff)
      return fail(PA_ERR_SHAPE, "num_blocks %lld must be in [1, 2^31)", (long long)num_blocks);
    if (num_pairs == 0) return ok();
    if (!k_cache || !block_pairs)
      return fail(PA_ERR_NULL, "k_cache (%p) and block_pairs (%p) must not be NULL", k_cache,
                  (const void*)block_pairs);
    if (!aligned16(k_cache) || (v_cache && !aligned16(v_cache)))
      return fail(PA_ERR_ALIGN, "k_cache and v_cache must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(block_pairs) & 3u)
      return fail(PA_ERR_ALIGN, "block_pairs must be 4-byte aligned");
    pa::CopyArgs a;
    a.k = k_cache;
    a.v = v_cache;
    a.pairs = block_pairs;
    a.block_bytes = (int32_t)block_bytes;
    a.num_blocks = (int32_t)num_blocks;
    a.chunks = (int32_t)((block_bytes + pa::copy_chunk_bytes() - 1) / pa::copy_chunk_bytes());
    if (num_pairs * a.chunks >= (int64_t)0x7fffffff)
      return fail(PA_ERR_UNSUPPORTED, "%lld pairs of %d chunks exceed the grid limit",
                  (long long)num_pairs, a.chunks);
    return hip_status(pa::launch_copy_blocks(a, num_pairs, v_cache != nullptr,
                                             static_cast<hipStream_t>(stream),
                                             static_cast<hipEvent_t>(start_event),
                                             static_cast<hipEvent_t>(stop_event)),
                      "block-copy launch");
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

pa_status_t pa_prefill(const pa_prefill_dims_t* dims, void* out, const void* q,
                       const void* k_new, const void* v_new, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start, float scale,
                       void* stream) {
  try {
    return prefill_impl(dims, out, q, k_new, v_new, k_cache, v_cache, block_tables,
                        context_lens, query_start, scale, Ws::kOwned, nullptr, 0, stream, nullptr,
                        nullptr);
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

pa_status_t pa_prefill_profiled(const pa_prefill_dims_t* dims, void* out, const void* q,
                                const void* k_new, const void* v_new, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start,
                                float scale, void* stream, void* start_event, void* stop_event) {
  try {
    return prefill_impl(dims, out, q, k_new, v_new, k_cache, v_cache, block_tables,
                        context_lens, query_start, scale, Ws::kOwned, nullptr, 0, stream,
                        static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

pa_status_t pa_prefill_ex(const pa_prefill_dims_t* dims, void* out, const void* q,
                          const void* k_new, const void* v_new, const void* k_cache,
                          const void* v_cache, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start, float scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  try {
    return prefill_impl(dims, out, q, k_new, v_new, k_cache, v_cache, block_tables,
                        context_lens, query_start, scale, Ws::kCaller, workspace,
                        workspace_bytes, stream, nullptr, nullptr);
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

int64_t pa_prefill_workspace_bytes(const pa_prefill_dims_t* dims) {
  try {
    int G = 0;
    pa_status_t st = check_prefill_dims(dims, &G);
    if (st != PA_OK) return st;
    pa::PrefillArgs a;
    size_t bytes = 0;
    if ((st = prefill_plan(dims, G, a, &bytes)) != PA_OK) return st;
    return (int64_t)bytes;
  } catch (...) {
    return fail(PA_ERR_INTERNAL, "unexpected C++ exception");
  }
}

int32_t pa_fused_applies(const pa_dims_t* dims, int32_t partition_size) {
  Plan pl;
  pa_status_t st = make_plan(dims, 0, partition_size, true, &pl);
  if (st != PA_OK) return st;
  pa::Split sp;
  if ((st = plan_split(pl, &sp)) != PA_OK) return st;
  return fused_applies(pl, sp) ? 1 : 0;
}

pa_status_t pa_set_fused(int32_t mode) {
  if (mode < 0 || mode > 1)
    return fail(PA_ERR_UNSUPPORTED, "single-launch mode %d unknown (0 or 1)", mode);
  g_fused.store(mode, std::memory_order_relaxed);
  return ok();
}

int32_t pa_get_fused(void) { return fused_setting(); }

pa_status_t pa_set_prefill_mode(int32_t mode) {
  if (mode < 0 || mode > 1)
    return fail(PA_ERR_UNSUPPORTED, "prefill mode %d unknown (0 or 1)", mode);
  g_prefill_mode.store(mode, std::memory_order_relaxed);
  return ok();
}

int32_t pa_get_prefill_mode(void) { return prefill_mode_setting(); }

pa_status_t pa_set_prefill_split(int32_t chunk_tiles) {
  if (chunk_tiles != -1 && chunk_tiles != 0 &&
      (chunk_tiles < pa::kPrefillMinChunk || chunk_tiles > (1 << 20)))
    return fail(PA_ERR_UNSUPPORTED, "prefill chunk setting %d unknown (-1, 0 or %d..%d tiles)",
                chunk_tiles, pa::kPrefillMinChunk, 1 << 20);
  g_prefill_split.store(chunk_tiles, std::memory_order_relaxed);
  return ok();
}

int32_t pa_get_prefill_split(void) { return prefill_split_setting(); }

pa_status_t pa_set_work_split(int32_t pieces, int64_t first_item) {
  if (pieces != -1 && pieces != 0 && pieces != 1 && pieces != 2 && pieces != 4 && pieces != 8 &&
      pieces != 16)
    return fail(PA_ERR_UNSUPPORTED, "work split of %d pieces unknown (-1, 0, 1, 2, 4, 8, 16)",
                pieces);
  if (first_item < 0) return fail(PA_ERR_SHAPE, "first_item %lld is negative",
                                  (long long)first_item);
  g_split_first.store(first_item);
  g_split_pieces.store(pieces);
  return ok();
}

int32_t pa_get_work_split(int64_t* first_item) {
  if (first_item) *first_item = g_split_first.load();
  return g_split_pieces.load();
}

pa_status_t pa_split_plan(const pa_dims_t* dims, int64_t max_context_len, int32_t partition_size,
                          int64_t* plan) {
  if (!plan) return fail(PA_ERR_NULL, "plan is NULL");
  Plan pl;
  pa_status_t st = make_plan(dims, max_context_len, partition_size, true, &pl);
  if (st != PA_OK) return st;
  pa::Split sp;
  if ((st = plan_split(pl, &sp)) != PA_OK) return st;
  const int64_t items = (int64_t)pl.S * pl.Hkv * pl.Pmax;
  plan[0] = items;
  plan[1] = sp.shift ? sp.first : items;
  plan[2] = (int64_t)1 << sp.shift;
  plan[3] = sp.shift ? sp.first + ((items - sp.first) << sp.shift) : items;
  return ok();
}

}  // extern "C"
