// HIP kernels of the paged split-KV decode path, written for CDNA4 (gfx950).
//
// Phase 1 / V1 ("Phase 1: Per-partition attention", project_6 commit 96f4baf
// page, V2 plan): one work-group per (partition, KV head, sequence).  The
// work-group holds every query head of its GQA group, so each K/V byte is
// read from HBM once for all of them.  Its 4 waves take the partition's
// 16-token cache blocks in turn; each wave keeps a running (max, sum,
// unnormalised output) per head -- the online softmax, i.e. the
// flash-attention tiling the page names -- and the 4 partial states are
// merged through LDS at the end with the same log-sum-exp rule Phase 2 uses.
//
// Two inner loops:
//   * attn_mfma_kernel (fp16 / bf16, G >= 4): QK^T and PV are small dense
//     contractions over the head group, done on the matrix cores.
//     QK^T: v_mfma_f32_16x16x32_{bf16,f16}, A = the 16 keys of a block
//     (rows = tokens), B = the group's queries (columns = heads, padded to
//     16).  The result lands with column = head, rows = tokens, which is
//     exactly the A-operand layout of PV: v_mfma_f32_16x16x32 with
//     A = probabilities (rows = heads, k = tokens; each probability as a
//     16-bit high part and a 16-bit low part in two k-slots) and B = V
//     (k = tokens, each V row in both slots).  Each lane loads V rows as
//     16-byte runs of 8 columns and feeds column j of its run to PV
//     instruction j, so no transpose through LDS is needed: column n of
//     instruction j is head-dim index 8n + j.
//   * attn_valu_kernel (fp32, or G < 4): plain fp32 FMAs; the query group is
//     staged in LDS and the probabilities of a block are exchanged through
//     a per-wave LDS slot.
//
// Phase 2 ("Phase 2: Cross-partition reduction (log-sum-exp)", same page):
// reduce_kernel, one work-group per (sequence, head, 32 columns).
//
// Exponentials use v_exp_f32 (base 2) on logits pre-scaled by
// scale * log2(e); max logits are stored back in natural-log units.  All
// accumulation is fp32.  Tail tokens of the last block are excluded by
// selecting -inf logits and zero V rows (never by multiplying by zero, so
// stale NaN/Inf in unused cache slots cannot leak into the result).

#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "pa_internal.h"
#include "pa_decode.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = kWaves * 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;
// Base-2 headroom a block max may exceed the running reference max by before the
// accumulators are rescaled (probabilities stay below 2^8, far from fp32 limits).
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-lane reductions on the vector ALU ------------------------------------------
// __shfl_xor compiles to ds_bpermute, a round trip through the LDS crossbar per step.
// These run on the VALU instead: lanes l ^ 1 and l ^ 2 through DPP quad permutations,
// the lanes of a 16-lane row four and eight apart through DPP row rotations, and l ^ 16 /
// l ^ 32 through the gfx950 half swaps (v_permlane16_swap / v_permlane32_swap: with both
// operands x, the two results hold x of lanes l and l ^ 16, resp. l and l ^ 32).
template <bool kSum>
__device__ __forceinline__ float combine(float a, float b) {
  return kSum ? a + b : fmaxf(a, b);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
template <bool kSum>
__device__ __forceinline__ float swap_combine16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  uint32_t r0 = r[0], r1 = r[1];
  // Without this the compiler (ROCm 7.2) combined one of the two results with itself.
  asm("" : "+v"(r0), "+v"(r1));
  return combine<kSum>(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
template <bool kSum>
__device__ __forceinline__ float swap_combine32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t r0 = r[0], r1 = r[1];
  asm("" : "+v"(r0), "+v"(r1));
  return combine<kSum>(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
// Sum (kSum) or max over the lanes congruent to this lane modulo kFrom (a power of two
// <= 32): every lane of such a group ends up with the group's result (bitwise the same
// in all of them for the max; for the sum, the result a given lane reads is the same
// from run to run).
template <bool kSum, int kFrom>
__device__ __forceinline__ float lane_reduce(float x) {
  static_assert(kFrom >= 1 && kFrom <= 32 && (kFrom & (kFrom - 1)) == 0, "power of two");
  if constexpr (kFrom <= 1) x = combine<kSum>(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
  if constexpr (kFrom <= 2) x = combine<kSum>(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
  if constexpr (kFrom <= 4) x = combine<kSum>(x, dpp_mov<0x124>(x));  // row_ror:4
  if constexpr (kFrom <= 8) x = combine<kSum>(x, dpp_mov<0x128>(x));  // row_ror:8
  if constexpr (kFrom <= 16) x = swap_combine16<kSum>(x);
  return swap_combine32<kSum>(x);
}
// Sum over the four lanes of a quad (l ^ 1, l ^ 2), bitwise the same in all four.
__device__ __forceinline__ float lane_reduce_quad(float x) {
  x += dpp_mov<0xB1>(x);
  return x + dpp_mov<0x4E>(x);
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 raw-buffer format word).
// A load at an offset >= bytes returns zeros without touching memory, so a
// resource with bytes = 0 turns every load through it into a no-op.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16-byte streaming load through a buffer resource (non-temporal hint: K/V are
// read exactly once per step and must not displace reusable cache lines).
__device__ __forceinline__ u32x4 ld_stream(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

// ---- element conversions -------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float half_lo(uint32_t w) {
  if constexpr (DT == PA_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t w) {
  if constexpr (DT == PA_BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <int DT>
__device__ __forceinline__ uint32_t to_bits16(float x) {
  if constexpr (DT == PA_BF16) return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
  else return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return to_bits16<DT>(lo) | (to_bits16<DT>(hi) << 16);
}

// Store n (4 or 8) consecutive fp32 values as element type DT at element offset idx.
template <int DT, int N>
__device__ __forceinline__ void store_out(void* out, size_t idx, const float* v) {
  static_assert(N == 2 || N == 4 || N == 8, "");
  if constexpr (DT == PA_F32) {
    float* o = static_cast<float*>(out) + idx;
    if constexpr (N == 2) {
      *reinterpret_cast<f32x2*>(o) = f32x2{v[0], v[1]};
    } else {
#pragma unroll
      for (int i = 0; i < N; i += 4)
        *reinterpret_cast<f32x4*>(o + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
    }
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + idx;
    if constexpr (N == 2) {
      *reinterpret_cast<uint32_t*>(o) = pack2<DT>(v[0], v[1]);
    } else if constexpr (N == 4) {
      *reinterpret_cast<u32x2*>(o) = u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
    } else {
      *reinterpret_cast<u32x4*>(o) = u32x4{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]),
                                           pack2<DT>(v[4], v[5]), pack2<DT>(v[6], v[7])};
    }
  }
}

// Partial states use plain stores: they are read back by the next kernel, and
// non-temporal stores measured slower for both kernels (phase 1 37.3 -> 39.7 us at
// 100K tokens).
template <int N>
__device__ __forceinline__ void store_f32(float* dst, const float* v) {
#pragma unroll
  for (int i = 0; i < N; i += 4)
    *reinterpret_cast<f32x4*>(dst + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
}

// ---- matrix-core wrappers -------------------------------------------------------------
template <bool BF>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---- leading kernel arguments ---------------------------------------------------------
// The attention kernels take, ahead of AttnArgs, copies of the fields that a work-group's
// first memory round trip depends on (the context-length, block-id and query addresses
// and the integers of the grid mapping).  pa_kernels.hip is built with kernel-argument
// preloading (gfx950): the hardware places these leading scalar arguments in scalar
// registers at wave launch, so a work-group issues those loads without first waiting for
// a load of its argument block.  A by-value struct argument is never preloaded.
// The hardware preloads at most 14 argument dwords (16 user registers, two of which hold
// the argument-block address): three pointers and eight integers, two of them packed
// (the number of KV heads with the sequence-order count; the split's first cut item with
// its piece shift and, in bit 30, the single-launch flag).
#define PA_ATTN_LEAD_PARAMS                                                                \
  const int32_t *lead_ctx, const int32_t *lead_bt, const void *lead_q, int32_t lead_Pmax, \
      int32_t lead_hkv_order, int32_t lead_MB, int32_t lead_P, int32_t lead_q_sh,         \
      int32_t lead_first_shift, int32_t lead_q_ss, int32_t lead_bt_ss

__device__ __forceinline__ AttnArgs with_lead(AttnArgs a, const int32_t* ctx, const int32_t* bt,
                                              const void* q, int32_t Pmax, int32_t hkv_order,
                                              int32_t MB, int32_t P, int32_t q_sh,
                                              int32_t first_shift, int32_t q_ss,
                                              int32_t bt_ss) {
  a.ctx = ctx;
  a.bt = bt;
  a.q = q;
  a.Pmax = Pmax;
  a.Hkv = hkv_order & 0xffff;
  a.order_seqs = hkv_order >> 16;
  a.MB = MB;
  a.P = P;
  a.q_sh = q_sh;
  a.split.shift = first_shift & 15;
  a.split.first = (first_shift >> 4) & 0x3ffffff;
  a.fused = (first_shift >> 30) & 1;
  a.q_ss = q_ss;
  a.bt_ss = bt_ss;
  return a;
}
#define PA_ATTN_APPLY_LEAD(args)                                                           \
  with_lead(args, lead_ctx, lead_bt, lead_q, lead_Pmax, lead_hkv_order, lead_MB, lead_P,   \
            lead_q_sh, lead_first_shift, lead_q_ss, lead_bt_ss)

// Consumes the context length and one field of each 64-byte line of the argument
// struct (output, K/V bases, pool size and scale), so that their scalar loads are issued
// before the wait for the first memory round trip and complete within it.  Otherwise
// the scheduler issued the context-length load after the query waits, and each struct
// field load only where the field is first used, every one a separate wait.
#define PA_PIN_EARLY_SCALARS(a, n_ctx)                                                   \
  asm volatile("" ::"s"(n_ctx), "s"((a).out), "s"((a).k), "s"((a).v), "s"((a).NB),       \
               "s"((a).scale_log2), "s"((a).kv_sb))

// ---- work-group set-up shared by both attention kernels ------------------------------
// The grid item of this work-group (see Split): partition p of KV head g of sequence b,
// whole (piece < 0) or one of its pieces.
struct Item {
  int p, g, b, piece;
};

__device__ __forceinline__ Item grid_item(const AttnArgs& a) {
  Item it;
  it.piece = -1;
  if (a.split.shift == 0 && !a.fused) {
    it.p = blockIdx.x;
    it.g = blockIdx.y;
    it.b = blockIdx.z;
    return it;
  }
  // linear grid: the work split, or a single-launch V2 (row 0 of its grid)
  int j = blockIdx.x;
  if (a.split.shift > 0 && j >= a.split.first) {
    const int t = j - a.split.first;
    j = a.split.first + (t >> a.split.shift);
    it.piece = t & ((1 << a.split.shift) - 1);
  }
  it.p = j % a.Pmax;
  const int r = j / a.Pmax;
  it.g = r % a.Hkv;
  it.b = r / a.Hkv;
  return it;
}

struct Part {
  int n;       // context length (clamped to the table capacity)
  int nparts;  // partitions of this sequence that exist in the grid
  int tok0;    // first token of this work-group's range
  int ntok;    // tokens in the range (<= 0: an empty piece of the last partition)
  int nblk;    // cache blocks in the range
};

// The token range this work-group covers when its partition is full: first token and
// length.  It depends on the grid item only, not on the context length.
__device__ __forceinline__ void nominal_range(const AttnArgs& a, const Item& it, int& tok0,
                                              int& len) {
  len = a.P;
  tok0 = it.p * a.P;
  if (it.piece >= 0) {
    len = a.P >> a.split.shift;
    tok0 += it.piece * len;
  }
}

// n: the sequence's context length as read from context_lens.
__device__ __forceinline__ Part plan_partition(const AttnArgs& a, const Item& it, int n) {
  Part r;
  const int cap = a.MB * kBlockSize;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  int np = (n + a.P - 1) / a.P;
  r.n = n;
  r.nparts = np > a.Pmax ? a.Pmax : np;
  int len;
  nominal_range(a, it, r.tok0, len);
  r.ntok = min(len, n - r.tok0);
  r.nblk = (r.ntok + kBlockSize - 1) / kBlockSize;
  return r;
}

// Compacted order for V2 with several sequences (no work split): the grid has Pmax
// partition slots per (sequence, KV head), and the slots past a sequence's context are
// empty.  Work-groups are placed on compute units in grid order, so with sequences of
// very different lengths the real items of the long ones pile up on the same units
// (mixed 65536..1-token contexts: up to 6 partitions on one unit, 1.9 on average;
// 256 x U{512..4096}: 32 against 18).  Work-group j (linear grid index) instead takes
// the j-th real item in (sequence, KV head, partition) order, so real items are
// contiguous in dispatch order; work-groups past the last one return.  A sequence with
// no tokens still has one item (partition 0), whose work-group writes its zero output.
// Each wave derives its item from all S context lengths: lane l sums the partition
// counts of sequences 8l .. 8l+7 (S <= 512), a wave scan gives each lane's first item,
// and the lane whose range holds j finds the sequence.
__device__ __forceinline__ bool compact_item(const AttnArgs& a, int S, Item& it) {
  const int j = a.fused ? (int)blockIdx.x
                        : (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int lane = threadIdx.x & 63;
  const int cap = a.MB * kBlockSize;
  int np[8];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 8 * lane + i;
    int n = t < S ? a.ctx[t] : 0;
    n = n < 0 ? 0 : (n > cap ? cap : n);
    int c = (n + a.P - 1) / a.P;
    c = c > a.Pmax ? a.Pmax : (c < 1 ? 1 : c);
    np[i] = t < S ? c : 0;
    tot += np[i];
  }
  int incl = tot;  // inclusive scan of the lane totals
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const int first = (incl - tot) * a.Hkv;  // items are (sequence, KV head, partition)
  const unsigned long long hit = __ballot(j >= first && j < incl * a.Hkv);
  if (hit == 0) return false;
  const int owner = __builtin_ctzll(hit);
  int seq = 0, off = 0, cnt = 1;
  if (lane == owner) {
    int rem = j - first;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int items = np[i] * a.Hkv;
      if (rem >= 0 && rem < items) {
        seq = 8 * lane + i;
        off = rem;
        cnt = np[i];
      }
      rem -= items;
    }
  }
  seq = __builtin_amdgcn_readlane(seq, owner);
  off = __builtin_amdgcn_readlane(off, owner);
  cnt = __builtin_amdgcn_readlane(cnt, owner);
  it.b = seq;
  it.g = off / cnt;
  it.p = off - it.g * cnt;
  it.piece = -1;
  return true;
}

// Longest-first order for V1 (one work-group per (sequence, KV head), the whole context):
// work-groups are dispatched in grid order, so with more of them than fit on the chip at
// once, a long sequence dispatched late runs on after the others have finished; taking
// sequences longest context first shortens that tail (batched 256 x U{512..4096}: a
// fluid model of the dispatch gives ~229 us in grid order and ~206 us longest first).
// The work-group of rank r (blockIdx.z) takes the sequence with exactly r sequences
// before it in the order (longer context, or equal and lower index): every work-group
// reads all S context lengths (one coalesced round trip) and counts.  The rank of each
// sequence is distinct, so exactly one thread writes the pick.  The result of each
// (sequence, head) does not depend on which work-group computes it.
__device__ __forceinline__ int seq_of_length_rank(const int32_t* ctx, int S, int r, int* s_len,
                                                  int* s_pick) {
  for (int t = threadIdx.x; t < ((S + 3) & ~3); t += blockDim.x)
    s_len[t] = t < S ? ctx[t] : INT32_MIN;
  __syncthreads();
  // Lengths are compared four at a time (16-byte LDS reads, the same address in every
  // lane); the padding entries (INT32_MIN, index >= S) are never ordered first.
  for (int c = threadIdx.x; c < S; c += blockDim.x) {
    const int lc = s_len[c];
    int rank = 0;
#pragma unroll 4
    for (int k = 0; k < S; k += 4) {
      const int4 l4 = *reinterpret_cast<const int4*>(s_len + k);
      rank += (l4.x > lc) | ((l4.x == lc) & (k < c));
      rank += (l4.y > lc) | ((l4.y == lc) & (k + 1 < c));
      rank += (l4.z > lc) | ((l4.z == lc) & (k + 2 < c));
      rank += (l4.w > lc) | ((l4.w == lc) & (k + 3 < c));
    }
    if (rank == r) *s_pick = c;
  }
  __syncthreads();
  return *s_pick;
}

// Rows of the partial state of query head h of this work-group's group: the
// partition's row of tmp_out / max_logits / exp_sums, or the piece's slot.
template <int G, int D>
__device__ __forceinline__ void partial_rows(const AttnArgs& a, const Item& it, int h, float*& o,
                                             float*& m, float*& s) {
  size_t row;
  if (it.piece >= 0) {
    row = (size_t)(blockIdx.x - a.split.first) * G + h;
    o = a.split.piece_out + row * D;
    m = a.split.piece_max + row;
    s = a.split.piece_sum + row;
  } else {
    row = ((size_t)it.b * a.Hq + (size_t)it.g * G + h) * a.Pmax + it.p;
    o = a.tmp_out + row * D;
    m = a.max_logits + row;
    s = a.exp_sums + row;
  }
}

// ---- single-launch V2: publication of the phase-1 partials ----------------------------
// In a single-launch V2 the merge work-groups of the same grid read the partials, so they
// are stored with device-scope (sc1) stores -- coherent across the XCDs' L2 caches once
// complete -- and each phase-1 work-group then counts itself in its (sequence, KV head)
// arrival counter (see fused_merge).
constexpr int kScDevice = 16;  // cache-policy bits of a device-scope access (sc1)

// Stores 8 (or 4, 2) fp32 values at dst inside the workspace that starts at ws, with
// device-scope stores.  The buffer resource spans the whole workspace (the host keeps
// fused workspaces below 4 GiB), so it is the same in every lane.
template <int N>
__device__ __forceinline__ void store_f32_dev(const float* ws, float* dst, const float* v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ws), (short)0, -1, 0x00020000);
  const int off = (int)((const char*)dst - (const char*)ws);
  if constexpr (N == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])}, r,
                                          off, 0, kScDevice);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{__float_as_uint(v[i]), __float_as_uint(v[i + 1]), __float_as_uint(v[i + 2]),
                __float_as_uint(v[i + 3])},
          r, off + 4 * i, 0, kScDevice);
  }
}
__device__ __forceinline__ void store_stat_dev(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ int fused_expected(const AttnArgs& a, int b, int g, int n);

// Called by every phase-1 work-group of a single-launch V2 exactly once, from wave 0,
// after its last partial store was issued: waits until this wave's stores are complete,
// then counts the work-group in the (sequence, KV head) arrival counter.  The work-group
// that completes the count (every other one has counted itself, so every partial of the
// group is visible) resets the counter for the next launch and raises the go flag of
// each of the group's G * kFusedChunks merge work-groups, one per lane.  Only the flag
// owners poll them, each its own line: polls never queue the arrivals.
// n: the sequence's context length as read from context_lens.
template <int G>
__device__ __forceinline__ void arrive(const AttnArgs& a, int b, int g, int n) {
  if (!a.fused) return;
  __builtin_amdgcn_s_waitcnt(0);  // every store of this wave performed
  const int lane = threadIdx.x & 63;
  uint32_t* const cnt = a.counters + kFusedCounterStride * ((size_t)b * a.Hkv + g);
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  const int cap = a.MB * kBlockSize;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  if (prev + 1 != (unsigned)fused_expected(a, b, g, n)) return;
  if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int m0 = ((b * a.Hq) + g * G) * kFusedChunks;
#pragma unroll
  for (int k = lane; k < G * kFusedChunks; k += 64)
    __hip_atomic_store(a.counters + kFusedFlagBase + kFusedFlagStride * (m0 + k), 1u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Element offsets of row (sequence b, query head h) of q and of out.
__device__ __forceinline__ size_t q_offset(const AttnArgs& a, int b, int h) {
  return (size_t)b * (uint32_t)a.q_ss + (size_t)h * (uint32_t)a.q_sh;
}
__device__ __forceinline__ size_t out_offset(const AttnArgs& a, int b, int h) {
  return (size_t)b * (size_t)a.o_ss + (size_t)h * (size_t)a.o_sh;
}

// A sequence with no cached tokens attends to nothing: its output is 0.
template <int DT, int D, int G>
__device__ __forceinline__ void write_zero_group(const AttnArgs& a, int b, int g) {
  const float z[4] = {0.f, 0.f, 0.f, 0.f};
  for (int idx = threadIdx.x * 4; idx < G * D; idx += blockDim.x * 4) {
    const int h = idx / D, d = idx - h * D;
    store_out<DT, 4>(a.out, out_offset(a, b, g * G + h) + d, z);
  }
}

// =======================================================================================
// Single-launch V2: the merge work-groups ("Phase 2: Cross-partition reduction
// (log-sum-exp)", project_6 commit 96f4baf page, V2 plan, in the same launch as phase 1).
//
// Row 1 of the grid: work-group m takes sequence b, query head hq and the kFusedChunks-th
// part `chunk` of the head dim (m = (b Hq + hq) kFusedChunks + chunk).  It waits for its
// go flag, which the phase-1 work-group that completes the count of (b, KV head hq / G)
// raises (see arrive): the phase-1 work-groups have lower grid indices and are dispatched
// first, so they are resident or finished while it waits.  It clears the flag for the
// next launch, folds the partial states like reduce_kernel, with device-scope loads, and
// writes its columns of out.  The wait is bounded by a wall-clock limit: a protocol error
// would show as NaN outputs (and a flag raised after the limit would stay raised), never
// as a hang.
// =======================================================================================
constexpr uint64_t kFusedWaitTicks = 1ull << 25;  // s_memrealtime runs at 100 MHz: ~0.34 s


__device__ int fused_expected(const AttnArgs& a, int b, int g, int n) {
  if (a.order_seqs > 0 && a.Pmax > 1) {  // compacted order: the real items only
    int c = (n + a.P - 1) / a.P;
    return c > a.Pmax ? a.Pmax : (c < 1 ? 1 : c);
  }
  if (a.split.shift == 0) return a.Pmax;  // every grid slot of (b, g)
  const long long j0 = (long long)a.Pmax * ((long long)g + (long long)a.Hkv * b);
  long long cut = j0 + a.Pmax - (a.split.first > j0 ? (long long)a.split.first : j0);
  cut = cut < 0 ? 0 : cut;
  return (int)((a.Pmax - cut) + (cut << a.split.shift));
}

template <int DT, int D, int T>
__device__ __forceinline__ void fused_merge(const AttnArgs& a) {
  constexpr int kCols = D / kFusedChunks;
  constexpr int NC4 = kCols / 4;   // float4 column lanes
  constexpr int NPG = T / NC4;     // partial-state lanes
  constexpr int NWV = T / 64;
  static_assert(NC4 >= 1 && NC4 <= 64 && T % NC4 == 0, "");
  extern __shared__ float s_w[];   // one weight per partial state (sized at launch)
  __shared__ float s_red[NWV];
  __shared__ f32x4 s_acc[NWV][NC4];
  __shared__ int s_ok;
  const int m = blockIdx.x;
  if (m >= a.fused_m) return;
  const int chunk = m % kFusedChunks;
  const int bh = m / kFusedChunks;
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const int G = a.Hq / a.Hkv;
  const int g = hq / G, gq = hq - g * G;
  const int tid = threadIdx.x;
  const int d4 = tid % NC4, pg = tid / NC4;
  const int lane = tid & 63, wv = tid >> 6;

  int n = a.ctx[b];
  const int cap = a.MB * kBlockSize;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  int nparts = (n + a.P - 1) / a.P;
  if (nparts > a.Pmax) nparts = a.Pmax;
  // Partial states to fold, as in reduce_kernel: partitions [0, p_split) from their rows,
  // then each cut partition's non-empty pieces from consecutive piece slots.
  const int sh = a.split.shift;
  int p_split = nparts, nfold = nparts, slot0 = 0;
  if (sh > 0) {
    const long long item0 = (long long)a.Pmax * ((long long)g + (long long)a.Hkv * b);
    const long long first = (long long)a.split.first - item0;
    const int nom_split = first <= 0 ? 0 : (first >= a.Pmax ? a.Pmax : (int)first);
    if (nom_split < a.Pmax) slot0 = (int)((item0 + nom_split - a.split.first) << sh);
    p_split = nom_split < nparts ? nom_split : nparts;
    if (p_split < nparts) {
      const int sub = a.P >> sh;
      const int last_tok = min(a.P, n - (nparts - 1) * a.P);
      nfold = p_split + ((nparts - 1 - p_split) << sh) + (last_tok + sub - 1) / sub;
    }
  }
  const bool merge = !(p_split == nparts && nparts <= 1);  // else phase 1 wrote out

  uint32_t* const flag = a.counters + kFusedFlagBase + kFusedFlagStride * (size_t)m;
  if (tid == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    int ok = 1;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (__builtin_amdgcn_s_memrealtime() - t0 > kFusedWaitTicks) {
        ok = 0;
        break;
      }
    }
    if (ok) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ok = ok;
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  const int col = chunk * kCols + d4 * 4;
  const size_t orow = (size_t)b * (size_t)a.o_ss + (size_t)hq * (size_t)a.o_sh;
  if (!ok) {  // the wait ran out: make it visible in the output
    if (tid < NC4) {
      const float nan = __builtin_nanf("");
      const float vals[4] = {nan, nan, nan, nan};
      store_out<DT, 4>(a.out, orow + col, vals);
    }
    return;
  }
  if (merge) {
    // Byte offsets from the workspace base (tmp_out) of a state's row and statistics.
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(a.tmp_out, (short)0, -1, 0x00020000);
    const long long base = (long long)bh * a.Pmax;
    const char* const wsb = (const char*)a.tmp_out;
    const long long o_max = (const char*)a.max_logits - wsb, o_sum = (const char*)a.exp_sums - wsb;
    const long long o_pout = sh ? (const char*)a.split.piece_out - wsb : 0;
    const long long o_pmax = sh ? (const char*)a.split.piece_max - wsb : 0;
    const long long o_psum = sh ? (const char*)a.split.piece_sum - wsb : 0;
    auto prow = [&](int q) { return (long long)(slot0 + q - p_split) * G + gq; };
    auto off_o = [&](int q) -> int {
      return (int)(q < p_split ? ((base + q) * D + col) * 4 : o_pout + (prow(q) * D + col) * 4);
    };
    auto load_ms = [&](int q, float& mv, float& sv) {
      const bool whole = q < p_split;
      const int om = (int)(whole ? o_max + (base + q) * 4 : o_pmax + prow(q) * 4);
      const int os = (int)(whole ? o_sum + (base + q) * 4 : o_psum + prow(q) * 4);
      mv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, om, 0, kScDevice));
      sv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, os, 0, kScDevice));
    };
    // Every load of the first kMS statistics and kMO rows per lane is issued before any is
    // used (indices past the list re-read its last entry), so the fold costs one memory
    // round trip; longer lists finish in loops.
    constexpr int kMS = 8, kMO = 24;
    float sm[kMS], ss[kMS];
    f32x4 so[kMO];
#pragma unroll
    for (int j = 0; j < kMS; ++j) load_ms(min(tid + T * j, nfold - 1), sm[j], ss[j]);
#pragma unroll
    for (int i = 0; i < kMO; ++i)
      so[i] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off_o(min(pg + NPG * i, nfold - 1)), 0,
                                                       kScDevice));
    // Maxima (base 2) into LDS and their block max.
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kMS; ++j) {
      const int q = tid + T * j;
      if (q < nfold) {
        const float m2 = sm[j] * kLog2e;
        s_w[q] = m2;
        s_w[nfold + q] = ss[j];
        mx = fmaxf(mx, m2);
      }
    }
    for (int q = tid + T * kMS; q < nfold; q += T) {
      float mv, sv;
      load_ms(q, mv, sv);
      const float m2 = mv * kLog2e;
      s_w[q] = m2;
      s_w[nfold + q] = sv;
      mx = fmaxf(mx, m2);
    }
    mx = lane_reduce<false, 1>(mx);
    if (lane == 0) s_red[wv] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) M = fmaxf(M, s_red[i]);
    // Weights r_q = exp2(m_q - M) s_q and their sum (each lane its own statistics).
    float wsum = 0.f;
    for (int q = tid; q < nfold; q += T) {
      const float rq = exp2_fast(s_w[q] - M) * s_w[nfold + q];
      s_w[q] = rq;
      wsum += rq;
    }
    wsum = lane_reduce<true, 1>(wsum);
    __syncthreads();  // weights visible; s_red reads of M done
    if (lane == 0) s_red[wv] = wsum;
    // sum_q r_q o_q over this lane's states.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMO; ++i)
      if (pg + NPG * i < nfold) acc += so[i] * s_w[pg + NPG * i];
    for (int q0 = pg + NPG * kMO; q0 < nfold; q0 += 8 * NPG) {
      f32x4 o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = min(q0 + NPG * i, nfold - 1);
        o[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off_o(q), 0,
                                                                               kScDevice));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (q0 + NPG * i < nfold) acc += o[i] * s_w[q0 + NPG * i];
    }
    if constexpr (NC4 < 64) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = lane_reduce<true, NC4>(acc[j]);
    }
    if (lane < NC4) s_acc[wv][d4] = acc;
    __syncthreads();
    if (tid < NC4) {
      float total = s_red[0];
      f32x4 o = s_acc[0][d4];
#pragma unroll
      for (int i = 1; i < NWV; ++i) {
        total += s_red[i];
        o += s_acc[i][d4];
      }
      const float inv = 1.f / total;
      const float vals[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      store_out<DT, 4>(a.out, orow + col, vals);
    }
  }
}

// =======================================================================================
// Matrix-core attention kernel: fp16 / bf16, G in {4, 8, 16}.
//
// NW waves per work-group share one partition (wave w takes blocks w, w+NW, ...).
// Each wave runs an NBUF-deep software pipeline in registers: while it computes
// block k, the loads of blocks k+1 .. k+NBUF-1 are in flight.  At head_dim 128
// the register budget is 2 waves per SIMD (256 VGPRs), which keeps every
// work-group of the 100K-token / 4-KV-head shape (784 of them) resident at once
// for NW <= 2.  At head_dim 256 a block is twice the registers and the budget is
// one wave per SIMD.
// =======================================================================================
template <int DT, int D, int G, int NW, int NBUF>
__global__ void __launch_bounds__(NW * 64, D == 128 ? 2 : 1)
    attn_mfma_kernel(PA_ATTN_LEAD_PARAMS, const AttnArgs args) {
  const AttnArgs a = PA_ATTN_APPLY_LEAD(args);
  static_assert(DT == PA_BF16 || DT == PA_F16, "matrix-core path is 16-bit only");
  static_assert(G >= 1 && G <= 16, "head group must fit the 16 MFMA columns");
  static_assert(NBUF >= 2, "need at least one block in flight");
  constexpr bool kBF = DT == PA_BF16;
  constexpr int NKK = D / 32;    // QK^T instructions per block (k = 32 head-dim columns each)
  constexpr int NC = D / 128;    // 16-byte V runs per lane per row
  constexpr int NMM = D / 16;    // PV instructions per block (16 head-dim columns each)

  constexpr int CPR = D / 8;                     // 16-byte chunks per K/V row
  // K staging through LDS (contiguous global reads, see compute_block) pays at
  // head_dim 256, where a strided K read touches 16 rows of 512 bytes per instruction
  // (mixed_d256: 74.4 -> 60.0 us/step); at head_dim 128 it only adds latency.
  constexpr bool kStageK = D == 256;
  constexpr int kTileBytes = kStageK ? NW * 16 * CPR * 16 : 16;  // one K tile per wave
  constexpr int kMergeBytes = (NW > 1 ? NW - 1 : 1) * NMM * 4 * 64 * 4;
  __shared__ u32x4 s_qf[NKK][64];   // query operand, one 16-byte fragment per lane
  __shared__ float s_mref[NW][16];  // per wave and head: reference max of the sums
  __shared__ float s_mmax[NW][16];  // per wave and head: true max logit
  __shared__ float s_l[NW][16];     // per wave and head: exp-sum relative to the reference
  // During the block loop: each wave's K tile on its way from the contiguous load layout
  // to the MFMA operand layout.  After the loop: the other waves' accumulators.
  __shared__ __attribute__((aligned(16)))
  unsigned char s_un[kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes];
  typedef float MergeRows[NMM * 4][64];
  MergeRows* s_o = reinterpret_cast<MergeRows*>(s_un);
  // Longest-first order (see seq_of_length_rank): built into the four-wave shape only,
  // the one used for partitions long enough for the ordering to pay.
  __shared__ __attribute__((aligned(16))) int s_len[NW == 4 ? kOrderMaxSeqs : 4];
  __shared__ int s_pick;

  if (a.fused && blockIdx.y != 0) {  // single-launch V2: a merge work-group
    fused_merge<DT, D, NW * 64>(a);
    return;
  }
  Item it = grid_item(a);
  if (a.order_seqs > 0) {
    if (a.Pmax > 1) {
      if (!compact_item(a, a.order_seqs, it)) return;  // past the last item
    } else if constexpr (NW == 4) {
      it.b = seq_of_length_rank(a.ctx, a.order_seqs, it.b, s_len, &s_pick);
    }
  }
  const int g = it.g, b = it.b;
  const int w = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;  // token row (K loads), head column (Q, S), V column run
  const int kg = lane >> 4;   // k-group of the MFMA operands

  // The block ids of the range a full partition would cover (clipped to the table
  // width, which bounds every context) and the queries do not depend on the context
  // length: they are requested in the same memory round trip as that length, so the
  // first K/V loads wait for one cold round trip, not two.  Entries past the context
  // are fetched but never used as addresses.
  const int n_ctx = a.ctx[b];
  int tok0n, lenn;
  nominal_range(a, it, tok0n, lenn);
  const int blk0 = tok0n / kBlockSize;
  const int nblk_nom = min(lenn / kBlockSize, a.MB - blk0);
  const int kcount_nom = w < nblk_nom ? (nblk_nom - w + NW - 1) / NW : 0;
  const int32_t* btrow = a.bt + (size_t)b * (uint32_t)a.bt_ss + blk0;
  int btv = lane < min(64, kcount_nom) ? btrow[w + NW * lane] : 0;  // first 64 block ids

  // Query operand: lane (r16, kg) holds head r16, columns 32*kk + 8*kg .. +7 (zero rows
  // pad the group to 16 heads).  Kept in LDS in lane order: conflict-free 16-byte reads.
  // The loads are unconditional (every wave loads, padding lanes read the group's last
  // head; wave 0 stores, zeros for the padding) so that the prologue is straight-line and
  // the compiler can neither sink them behind the context-length test nor put a wait
  // ahead of them.
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + q_offset(a, b, g * G + min(r16, G - 1));
  u32x4 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * kg);
  PA_PIN_EARLY_SCALARS(a, n_ctx);
  if (w == 0) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s_qf[kk][lane] = r16 < G ? qf[kk] : u32x4{0u, 0u, 0u, 0u};
  }

  const Part pt = plan_partition(a, it, n_ctx);
  if (it.p >= pt.nparts) {
    if (it.p == 0 && it.piece <= 0) write_zero_group<DT, D, G>(a, b, g);
    if (threadIdx.x < 64) arrive<G>(a, b, g, n_ctx);
    return;
  }
  if (pt.ntok <= 0) {  // empty piece: phase 2 does not read its slot
    if (threadIdx.x < 64) arrive<G>(a, b, g, n_ctx);
    return;
  }
  // pt.nblk <= nblk_nom: the context never extends past the table, so every block id
  // used below is among those fetched above.
  const int kcount = w < pt.nblk ? (pt.nblk - w + NW - 1) / NW : 0;

  const size_t hstride = (size_t)kBlockSize * D;
  const size_t bstride = (size_t)a.kv_sb;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + (size_t)g * hstride;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + (size_t)g * hstride;

  f32x4 O[NMM];
#pragma unroll
  for (int mm = 0; mm < NMM; ++mm) O[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Online softmax of head r16 in base-2 units.  The sums are kept relative to a
  // reference m_ref that only moves when a block max exceeds it by more than
  // kRescaleSlack, so accumulator rescaling is rare; m_max tracks the true max.
  float m_ref = kNegInf, m_max = kNegInf;
  float l_run = 0.f;  // this lane's share of the exp-sum of head r16

  u32x4 kbuf[NBUF][NKK], vbuf[NBUF][NC][4];

  // Loads of one 16-token block (K and V of KV head g).  `real` is false for the
  // prefetches past the wave's last block: their resources cover 0 bytes, so they
  // return zeros with no memory traffic while keeping the instruction stream (and
  // the compiler's wait counts) identical for every stage.  A block id outside the
  // pool is read the same way, as zeros.
  auto load_block = [&](u32x4 (&kr)[NKK], u32x4 (&vr)[NC][4], int kidx, bool real) {
    const int phys = __builtin_amdgcn_readlane(btv, kidx);
    const int nbytes = (real && (unsigned)phys < (unsigned)a.NB) ? kBlockSize * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase + (size_t)phys * bstride, nbytes);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase + (size_t)phys * bstride, nbytes);
    // K, staged: instruction j reads bytes [1024 j, 1024 j + 1024) of the tile, one
    // 16-byte chunk per lane in order -- whole cache lines per instruction.  K, direct:
    // lane (r16, kg) reads row r16, columns 32 kk + 8 kg .. +7 (the operand layout).
#pragma unroll
    for (int j = 0; j < NKK; ++j)
      kr[j] = kStageK ? ld_stream(rk, (64 * j + lane) * 16)
                      : ld_stream(rk, (r16 * D + 32 * j + 8 * kg) * 2);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[c][i] = ld_stream(rv, ((4 * kg + i) * D + 128 * c + 8 * r16) * 2);
  };

  // QK^T and the online softmax of one block; returns the PV A operand.
  auto qk_softmax = [&](u32x4 (&kr)[NKK], int kidx) -> u32x4 {
    // S^T = K Q^T: lane (r16, kg) gets tokens 4*kg + i of head r16.  The query
    // fragments are re-read from LDS every block rather than pinned in registers;
    // the opaque lane index keeps the compiler from hoisting the reads.
    int ql = lane;
    asm volatile("" : "+v"(ql));
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kStageK) {
      // Re-layout K through this wave's LDS tile: chunk (row r, column c) is stored at
      // slot r*CPR + (c + r) % CPR.  The rotation makes both the contiguous writes and
      // the operand reads (16 rows, one column) hit distinct banks.
      u32x4* tile = reinterpret_cast<u32x4*>(s_un) + w * 16 * CPR;
#pragma unroll
      for (int j = 0; j < NKK; ++j) {
        // Unsigned arithmetic on a power-of-two row length: a few instructions per chunk.
        // The one-wave two-deep shape has the registers to keep the slots (the same for
        // every block) from the lane itself; the deeper or wider shapes, which would then
        // spill, recompute them from the opaque lane index.
        static_assert((CPR & (CPR - 1)) == 0, "K tile rows of a power-of-two chunk count");
        const unsigned cl = 64u * j + (unsigned)(NW == 1 && NBUF == 2 ? lane : ql);
        const unsigned r = cl / CPR, c = cl % CPR;
        tile[r * CPR + ((c + r) & (CPR - 1))] = kr[j];
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 kt = tile[r16 * CPR + (4 * kk + kg + r16) % CPR];
        s = mfma_16x16x32<kBF>(kt, s_qf[kk][ql], s);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s = mfma_16x16x32<kBF>(kr[kk], s_qf[kk][ql], s);
    }
    const int valid = pt.ntok - (w + NW * kidx) * kBlockSize;  // >= 1, wave-uniform
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * kg + i < valid) ? s[i] * a.scale_log2 : kNegInf;
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = lane_reduce<false, 16>(bm);
    m_max = fmaxf(m_max, bm);
    if (__any(bm > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, bm);
      const float alpha = m_ref == kNegInf ? 0.f : exp2_fast(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      // Accumulator rows are heads 4*kg + i; fetch their factors from lanes 0..15.
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kg + i);
#pragma unroll
      for (int mm = 0; mm < NMM; ++mm)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[mm][i] *= al[i];
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = x[i] == kNegInf ? 0.f : exp2_fast(x[i] - m_ref);
    // P enters the PV product as a 16-bit high part plus a 16-bit low part (the rounding
    // residual), stacked in the k dimension of one 16x16x32 instruction: k-slots
    // 8 kg + i hold the high parts of tokens 4 kg + i, slots 8 kg + 4 + i their low parts,
    // and the V operand repeats the same four rows in both halves.  p is thus carried to
    // about 16 significant bits instead of 8 (bf16) or 11 (fp16), and the 16x16x32 form
    // takes the same matrix-core cycles on gfx950 as the 16x16x16 one.  The exp-sum adds
    // exactly the values the product uses (high plus rounded low part).
    u32x4 pa;
    {
      const uint32_t h01 = pack2<DT>(pr[0], pr[1]), h23 = pack2<DT>(pr[2], pr[3]);
      const float hf[4] = {half_lo<DT>(h01), half_hi<DT>(h01), half_lo<DT>(h23),
                           half_hi<DT>(h23)};
      const uint32_t l01 = pack2<DT>(pr[0] - hf[0], pr[1] - hf[1]);
      const uint32_t l23 = pack2<DT>(pr[2] - hf[2], pr[3] - hf[3]);
      l_run += ((hf[0] + half_lo<DT>(l01)) + (hf[1] + half_hi<DT>(l01))) +
               ((hf[2] + half_lo<DT>(l23)) + (hf[3] + half_hi<DT>(l23)));
      pa = u32x4{h01, h23, l01, l23};
    }
    return pa;
  };
  // O += P V for one block (V rows past the context are zeroed first).
  auto pv = [&](u32x4 (&vr)[NC][4], int kidx, const u32x4 pa) {
    const int valid = pt.ntok - (w + NW * kidx) * kBlockSize;  // >= 1, wave-uniform
    if (valid < kBlockSize) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * kg + i >= valid) vr[c][i] = u32x4{0u, 0u, 0u, 0u};
    }
    // O += P V: instruction 8c + j uses column j of every lane's 8-column run.
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t v01 = __builtin_amdgcn_perm(vr[c][1][j >> 1], vr[c][0][j >> 1], sel);
        const uint32_t v23 = __builtin_amdgcn_perm(vr[c][3][j >> 1], vr[c][2][j >> 1], sel);
        O[8 * c + j] = mfma_16x16x32<kBF>(pa, u32x4{v01, v23, v01, v23}, O[8 * c + j]);
      }
  };
  auto compute_block = [&](u32x4 (&kr)[NKK], u32x4 (&vr)[NC][4], int kidx) {
    pv(vr, kidx, qk_softmax(kr, kidx));
  };

  // Blocks are taken 64 at a time (one block id per lane).  Inside a chunk the NBUF
  // register buffers rotate; every stage issues the loads of the block NBUF-1 ahead
  // (past the last block those loads are no-ops, see load_block), so the loads are
  // unconditional, the compiler's wait counts stay exact and the prefetch overlaps
  // the compute.
  // The first chunk's block ids were fetched together with the query (one round
  // trip), and the first chunk's prologue loads are issued before the barrier that
  // publishes the query: only the first block's math has to wait for it.  Every wave
  // reaches this barrier exactly once, with or without blocks.
  // Re-define btv once its load has landed: otherwise the compiler's wait-count
  // pass keeps treating it as an in-flight load inside the block loop and drains
  // every outstanding load before each readlane.
  asm volatile("" : "+v"(btv));
  if (kcount > 0) {
    const int last0 = min(64, kcount) - 1;
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) load_block(kbuf[s], vbuf[s], min(s, last0), s <= last0);
  }
  __syncthreads();
  for (int c0 = 0; c0 < kcount; c0 += 64) {
    const int cnt = min(64, kcount - c0);
    const int last = cnt - 1;
    if (c0 > 0) {
      btv = lane < cnt ? btrow[w + NW * (c0 + lane)] : 0;
      asm volatile("" : "+v"(btv));
#pragma unroll
      for (int s = 0; s < NBUF - 1; ++s) load_block(kbuf[s], vbuf[s], min(s, last), s <= last);
    }
    for (int k = 0; k < cnt; k += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const int nb = (s + NBUF - 1) % NBUF;
        load_block(kbuf[nb], vbuf[nb], min(k + s + NBUF - 1, last), k + s + NBUF - 1 <= last);
        // Keep the scheduler from interleaving the next block's loads with this
        // block's math: that would stretch live ranges past the register budget.
        __builtin_amdgcn_sched_barrier(0);
        if (k + s >= cnt) break;
        compute_block(kbuf[s], vbuf[s], c0 + k + s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- merge the NW waves' states (log-sum-exp) ----
  l_run = lane_reduce<true, 16>(l_run);
  if (kg == 0) {
    s_mref[w][r16] = m_ref;
    s_mmax[w][r16] = m_max;
    s_l[w][r16] = l_run;
  }
  __syncthreads();  // every wave is done with its K tile (if staged); the bytes become s_o
  if (NW > 1 && w > 0) {
#pragma unroll
    for (int mm = 0; mm < NMM; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[w - 1][mm * 4 + i][lane] = O[mm][i];
  }
  __syncthreads();
  if (w != 0) return;

  // Per head h: true partition max Mt, wave factors exp2(m_ref_w - Mt) and the exp-sum
  // L = sum_t exp2(x_t - Mt) of the whole partition.
  auto head_stats = [&](int h, float (&fac)[NW], float& Mt, float& L) {
    Mt = s_mmax[0][h];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) Mt = fmaxf(Mt, s_mmax[ww][h]);
    L = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = s_mref[ww][h];
      fac[ww] = mw == kNegInf ? 0.f : exp2_fast(mw - Mt);
      L += fac[ww] * s_l[ww][h];
    }
  };

  const bool single = pt.nparts == 1 && it.piece < 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kg + i;
    if (h >= G) continue;
    float fac[NW], Mt, L;
    head_stats(h, fac, Mt, L);
    const float linv = 1.f / L;
    const size_t orow = out_offset(a, b, g * G + h);
    float *po, *pm, *ps;
    partial_rows<G, D>(a, it, h, po, pm, ps);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float vals[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = (8 * c + j) * 4 + i;
        float o = fac[0] * O[8 * c + j][i];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) o += fac[ww] * s_o[ww - 1][e][lane];
        vals[j] = o * linv;
      }
      const int d0 = 128 * c + 8 * r16;
      if (single)
        store_out<DT, 8>(a.out, orow + d0, vals);
      else if (a.fused)
        store_f32_dev<8>(a.tmp_out, po + d0, vals);
      else
        store_f32<8>(po + d0, vals);
    }
  }
  if (!single && kg == 0 && r16 < G) {
    float fac[NW], Mt, L;
    head_stats(r16, fac, Mt, L);
    float *po, *pm, *ps;
    partial_rows<G, D>(a, it, r16, po, pm, ps);
    if (a.fused) {
      store_stat_dev(pm, Mt * kLn2);
      store_stat_dev(ps, L);
    } else {
      *pm = Mt * kLn2;
      *ps = L;
    }
  }
  arrive<G>(a, b, g, n_ctx);
}

// =======================================================================================
// Vector-ALU attention kernel: any element type, any supported G.
// =======================================================================================
template <int B> struct Bytes;
template <> struct Bytes<4> { typedef uint32_t T; };
template <> struct Bytes<8> { typedef u32x2 T; };
template <> struct Bytes<16> { typedef u32x4 T; };

// Streaming load of B (4, 8 or 16) bytes through a buffer resource.
template <int B>
__device__ __forceinline__ typename Bytes<B>::T ld_bytes(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (B == 4)
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2);
  else if constexpr (B == 8)
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
  else
    return ld_stream(r, off);
}

// Element e (0-based) of a register run holding elements of type DT.
template <int DT, typename V>
__device__ __forceinline__ float elem(const V& v, int e) {
  if constexpr (DT == PA_F32) {
    if constexpr (sizeof(V) == 4) return __uint_as_float(v);
    else return __uint_as_float(v[e]);
  } else {
    uint32_t word;
    if constexpr (sizeof(V) == 4) word = v;
    else word = v[e >> 1];
    return (e & 1) ? half_hi<DT>(word) : half_lo<DT>(word);
  }
}

template <int DT, int D, int G>
__global__ void __launch_bounds__(kThreads) attn_valu_kernel(PA_ATTN_LEAD_PARAMS,
                                                              const AttnArgs args) {
  const AttnArgs a = PA_ATTN_APPLY_LEAD(args);
  constexpr int ES = DT == PA_F32 ? 4 : 2;
  constexpr int ROWB = D * ES;   // bytes per cache row
  constexpr int KCH = ROWB / 64; // 16-byte K chunks per lane (a row is split over 4 lanes)
  constexpr int EPC = 16 / ES;   // elements per 16-byte chunk
  constexpr int VE = D / 64;     // V columns per lane
  constexpr int VB = VE * ES;    // V bytes per lane per row
  typedef typename Bytes<VB>::T VT;
  constexpr int kQBytes = G * D * 4;
  constexpr int kPBytes = kWaves * 16 * G * 4;
  constexpr int kOBytes = (kWaves - 1) * G * VE * 64 * 4;
  constexpr int kSmem = (kQBytes + kPBytes) > kOBytes ? (kQBytes + kPBytes) : kOBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  __shared__ float s_mref[kWaves][G];
  __shared__ float s_mmax[kWaves][G];
  __shared__ float s_l[kWaves][G];
  float* s_q = reinterpret_cast<float*>(smem);             // [G][D]   during the loop
  float* s_p = reinterpret_cast<float*>(smem + kQBytes);   // [kWaves][16][G]
  float* s_o = reinterpret_cast<float*>(smem);             // [kWaves-1][G*VE][64] after it

  if (a.fused && blockIdx.y != 0) {  // single-launch V2: a merge work-group
    fused_merge<DT, D, kThreads>(a);
    return;
  }
  Item it = grid_item(a);
  if (a.order_seqs > 0 && a.Pmax > 1 && !compact_item(a, a.order_seqs, it)) return;
  const int g = it.g, b = it.b;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int t = lane >> 2, r = lane & 3;

  // Context length, the first 64 block ids of the nominal range and the queries in one
  // memory round trip (see attn_mfma_kernel).
  const int n_ctx = a.ctx[b];
  int tok0n, lenn;
  nominal_range(a, it, tok0n, lenn);
  const int blk0 = tok0n / kBlockSize;
  const int nblk_nom = min(lenn / kBlockSize, a.MB - blk0);
  const int kcount_nom = w < nblk_nom ? (nblk_nom - w + kWaves - 1) / kWaves : 0;
  const int32_t* btrow = a.bt + (size_t)b * (uint32_t)a.bt_ss + blk0;
  int btv = lane < min(64, kcount_nom) ? btrow[w + kWaves * lane] : 0;

  // Stage the head group's queries, pre-multiplied by scale*log2(e), as fp32 (all loads
  // issued before the first store).
  constexpr int kQIter = (G * D + kThreads - 1) / kThreads;
  float qv[kQIter];
#pragma unroll
  for (int i = 0; i < kQIter; ++i) {
    const int idx = min(tid + i * kThreads, G * D - 1);
    const int hh = idx / D;
    const size_t src = q_offset(a, b, g * G + hh) + (idx - hh * D);
    if constexpr (DT == PA_F32) qv[i] = static_cast<const float*>(a.q)[src];
    else qv[i] = half_lo<DT>(static_cast<const uint16_t*>(a.q)[src]);
  }
  PA_PIN_EARLY_SCALARS(a, n_ctx);
#pragma unroll
  for (int i = 0; i < kQIter; ++i)
    if (tid + i * kThreads < G * D) s_q[tid + i * kThreads] = qv[i] * a.scale_log2;

  const Part pt = plan_partition(a, it, n_ctx);
  if (it.p >= pt.nparts) {
    if (it.p == 0 && it.piece <= 0) write_zero_group<DT, D, G>(a, b, g);
    if (threadIdx.x < 64) arrive<G>(a, b, g, n_ctx);
    return;
  }
  if (pt.ntok <= 0) {  // empty piece: phase 2 does not read its slot
    if (threadIdx.x < 64) arrive<G>(a, b, g, n_ctx);
    return;
  }
  // pt.nblk <= nblk_nom, so the first chunk's block ids are all in btv.
  const int kcount = w < pt.nblk ? (pt.nblk - w + kWaves - 1) / kWaves : 0;
  asm volatile("" : "+v"(btv));  // see attn_mfma_kernel
  const size_t hstride = (size_t)kBlockSize * ROWB;   // bytes per (block, head)
  const size_t bstride = (size_t)a.kv_sb * ES;        // bytes per block
  const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + (size_t)g * hstride;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + (size_t)g * hstride;
  __syncthreads();

  float O[G][VE];
  float m_ref[G], m_max[G], l_run[G];  // see attn_mfma_kernel; wave-uniform per head
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_ref[h] = kNegInf;
    m_max[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) O[h][e] = 0.f;
  }

  u32x4 kA[KCH], kB[KCH];
  VT vA[16], vB[16];

  // Same loading scheme as attn_mfma_kernel: buffer loads, no-op past the last block.
  auto load_block = [&](u32x4 (&kr)[KCH], VT (&vr)[16], int kidx, bool real) {
    const int phys = __builtin_amdgcn_readlane(btv, kidx);
    const int nbytes = (real && (unsigned)phys < (unsigned)a.NB) ? kBlockSize * ROWB : 0;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase + (size_t)phys * bstride, nbytes);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase + (size_t)phys * bstride, nbytes);
#pragma unroll
    for (int j = 0; j < KCH; ++j) kr[j] = ld_stream(rk, t * ROWB + (r + 4 * j) * 16);
#pragma unroll
    for (int t2 = 0; t2 < 16; ++t2) vr[t2] = ld_bytes<VB>(rv, t2 * ROWB + lane * VB);
  };

  auto compute_block = [&](u32x4 (&kr)[KCH], VT (&vr)[16], int kidx) {
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int d0 = (r + 4 * j) * EPC;
#pragma unroll
      for (int e4 = 0; e4 < EPC; e4 += 4) {
        float kv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = elem<DT>(kr[j], e4 + e);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(s_q + h * D + d0 + e4);
          acc[h] += qv[0] * kv[0] + qv[1] * kv[1] + qv[2] * kv[2] + qv[3] * kv[3];
        }
      }
    }
    const int valid = pt.ntok - (w + kWaves * kidx) * kBlockSize;  // >= 1, wave-uniform
    bool move = false;
    float x[G], bm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sv = acc[h];
      sv = lane_reduce_quad(sv);
      x[h] = t < valid ? sv : kNegInf;
      float v = x[h];
      v = lane_reduce<false, 4>(v);
      bm[h] = v;
      m_max[h] = fmaxf(m_max[h], v);
      move |= v > m_ref[h] + kRescaleSlack;
    }
    if (move) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m_new = fmaxf(m_ref[h], bm[h]);
        const float alpha = m_ref[h] == kNegInf ? 0.f : exp2_fast(m_ref[h] - m_new);
        m_ref[h] = m_new;
        l_run[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VE; ++e) O[h][e] *= alpha;
      }
    }
    float* pw = s_p + w * 16 * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ph = x[h] == kNegInf ? 0.f : exp2_fast(x[h] - m_ref[h]);
      if (r == 0) {
        l_run[h] += ph;
        pw[t * G + h] = ph;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t2 = 0; t2 < 16; ++t2) {
      if (t2 < valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = pw[t2 * G + h];
#pragma unroll
          for (int e = 0; e < VE; ++e) O[h][e] += ph * elem<DT>(vr[t2], e);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Blocks are taken 64 at a time (one block id per lane).  Inside a chunk two
  // register buffers alternate; the next block's loads are always issued (the index
  // is clamped to the chunk's last block) so the compiler's wait counts stay exact
  // and the prefetch overlaps the FMAs.
  for (int c0 = 0; c0 < kcount; c0 += 64) {
    const int cnt = min(64, kcount - c0);
    if (c0 > 0) {
      btv = lane < cnt ? btrow[w + kWaves * (c0 + lane)] : 0;
      asm volatile("" : "+v"(btv));  // see attn_mfma_kernel
    }
    const int last = cnt - 1;
    load_block(kA, vA, 0, true);
    for (int k = 0; k < cnt; k += 2) {
      load_block(kB, vB, min(k + 1, last), k + 1 <= last);
      compute_block(kA, vA, c0 + k);
      if (k + 1 >= cnt) break;
      load_block(kA, vA, min(k + 2, last), k + 2 <= last);
      compute_block(kB, vB, c0 + k + 1);
    }
  }

  // Full-wave exp-sum per head (only lanes with r == 0 accumulated).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = l_run[h];
    l = lane_reduce<true, 1>(l);
    l_run[h] = l;
  }
  __syncthreads();  // every wave is done with s_q / s_p; their bytes become s_o
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_mref[w][h] = m_ref[h];
      s_mmax[w][h] = m_max[h];
      s_l[w][h] = l_run[h];
    }
  }
  if (w > 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VE; ++e) s_o[((w - 1) * G * VE + h * VE + e) * 64 + lane] = O[h][e];
  }
  __syncthreads();
  if (w != 0) return;

  const bool single = pt.nparts == 1 && it.piece < 0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float Mt = s_mmax[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) Mt = fmaxf(Mt, s_mmax[ww][h]);
    float fac[kWaves], L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = s_mref[ww][h];
      fac[ww] = mw == kNegInf ? 0.f : exp2_fast(mw - Mt);
      L += fac[ww] * s_l[ww][h];
    }
    const float linv = 1.f / L;
    float vals[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float o = fac[0] * O[h][e];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww)
        o += fac[ww] * s_o[((ww - 1) * G * VE + h * VE + e) * 64 + lane];
      vals[e] = o * linv;
    }
    if (single) {
      store_out<DT, VE>(a.out, out_offset(a, b, g * G + h) + lane * VE, vals);
    } else {
      float *po, *pm, *ps;
      partial_rows<G, D>(a, it, h, po, pm, ps);
      float* dst = po + lane * VE;
      if (a.fused) {
        store_f32_dev<VE>(a.tmp_out, dst, vals);
        if (lane == 0) {
          store_stat_dev(pm, Mt * kLn2);
          store_stat_dev(ps, L);
        }
      } else {
        if constexpr (VE == 2) *reinterpret_cast<f32x2*>(dst) = f32x2{vals[0], vals[1]};
        else store_f32<VE>(dst, vals);
        if (lane == 0) {
          *pm = Mt * kLn2;
          *ps = L;
        }
      }
    }
  }
  arrive<G>(a, b, g, n_ctx);
}

// =======================================================================================
// Phase 2: cross-partition log-sum-exp merge.
// Grid (S*Hq, kReduceChunks); 256 threads.  Per (sequence, head): M = max of the partial maxima,
// r_q = exp(m_q - M) * s_q per partial state q, out = sum_q r_q o_q / sum_q r_q.
// =======================================================================================
constexpr int kMaxFold = kMaxReducePartitions + kMaxPieceSlots;  // partial states per head
// Phase 2 splits each head's D columns over CHUNKS work-groups.  With few (sequence,
// head) pairs, 8 chunks (16 columns at head_dim 128: 64 partition lanes x 4 float4
// column lanes): phase 2 is bound by per-CU load issue, so more, narrower work-groups
// finish sooner.  With many pairs (>= kReduceWideHeads), 1 chunk: the grid is already
// large, and every extra work-group pays the fixed start-up latency.
constexpr int kReduceWideHeads = 256;

// Leading scalar arguments of reduce_kernel (preloaded into registers like those of the
// attention kernels): the context-length address, the workspace base (= tmp_out), the
// head counts and partition-grid size, the split packed as first << 4 | shift, and the
// other partial arrays as offsets from the base in 256-byte units (every workspace array
// starts on a 256-byte boundary).  The struct carries the output and the table shape.
#define PA_REDUCE_LEAD_PARAMS                                                              \
  const int32_t *lead_ctx, const float *lead_ws, int32_t lead_Hq, int32_t lead_Hkv,       \
      int32_t lead_Pmax, int32_t lead_split, int32_t u_max, int32_t u_sum, int32_t u_pout, \
      int32_t u_pmax, int32_t u_psum
constexpr int kWsUnitFloats = 64;  // 256-byte units

template <int DT, int D, int CHUNKS>
__global__ void __launch_bounds__(256) reduce_kernel(PA_REDUCE_LEAD_PARAMS,
                                                     const ReduceArgs args) {
  ReduceArgs a = args;
  a.ctx = lead_ctx;
  a.tmp_out = lead_ws;
  a.max_logits = lead_ws + (size_t)u_max * kWsUnitFloats;
  a.exp_sums = lead_ws + (size_t)u_sum * kWsUnitFloats;
  a.Hq = lead_Hq;
  a.Hkv = lead_Hkv;
  a.Pmax = lead_Pmax;
  a.split.first = lead_split >> 4;
  a.split.shift = lead_split & 15;
  a.split.piece_out = const_cast<float*>(lead_ws) + (size_t)u_pout * kWsUnitFloats;
  a.split.piece_max = const_cast<float*>(lead_ws) + (size_t)u_pmax * kWsUnitFloats;
  a.split.piece_sum = const_cast<float*>(lead_ws) + (size_t)u_psum * kWsUnitFloats;
  // The weights r_q live in LDS (one per partial state); thread (pg, d4) then sums
  // r_q o_q over its partial states q = pg, pg+NPG, ... for 4 of the work-group's
  // kReduceCols columns, and the NPG partition lanes are summed in a fixed tree
  // (bitwise deterministic).
  constexpr int kReduceCols = D / CHUNKS;
  constexpr int NC4 = kReduceCols / 4;  // float4 column lanes
  constexpr int NPG = 256 / NC4;        // partition lanes
  extern __shared__ float s_w[];        // one weight per partial state (sized at launch)
  __shared__ float s_red[4];
  __shared__ f32x4 s_acc[4][NC4];
  const int bh = blockIdx.x, chunk = blockIdx.y;
  const int b = bh / a.Hq;
  const int tid = threadIdx.x;
  const int d4 = tid % NC4, pg = tid / NC4;
  const int lane = tid & 63, wv = tid >> 6;

  // Partial states to fold, in order: partitions [0, p_split) from their rows, then, for
  // each cut partition (see Split), its non-empty pieces from consecutive piece slots.
  // The list of any context is a prefix of the nominal list of a context that fills the
  // whole partition grid, and every entry of the nominal list lies inside the workspace.
  // So the first loads are issued together with the context-length load (one memory
  // round trip instead of two) and masked once it is known.
  const int hq = bh - b * a.Hq;
  const int G = a.Hq / a.Hkv;
  const int gq = hq % G;
  const int sh = a.split.shift;
  int nom_split = a.Pmax, nom_fold = a.Pmax, slot0 = 0;
  if (sh > 0) {
    const long long item0 = (long long)a.Pmax * ((long long)(hq / G) + (long long)a.Hkv * b);
    const long long first = (long long)a.split.first - item0;
    nom_split = first <= 0 ? 0 : (first >= a.Pmax ? a.Pmax : (int)first);
    nom_fold = nom_split + ((a.Pmax - nom_split) << sh);
    if (nom_split < a.Pmax) slot0 = (int)((item0 + nom_split - a.split.first) << sh);
  }
  const long long base = (long long)bh * a.Pmax;
  const int col = chunk * kReduceCols + d4 * 4;
  // Piece rows are addressed as element offsets from the partition arrays (both live in
  // one workspace), so an entry selects an integer, not a pointer: a selected pointer
  // argument is fetched from the argument segment by the compiler, a dependent load.
  const float* const mls = a.max_logits;
  const float* const ess = a.exp_sums;
  const float* const tmp = a.tmp_out;
  const long long dm = sh ? (long long)(u_pmax - u_max) * kWsUnitFloats : 0;
  const long long ds = sh ? (long long)(u_psum - u_sum) * kWsUnitFloats : 0;
  const long long dO = sh ? (long long)u_pout * kWsUnitFloats : 0;
  auto prow = [&](int q) { return (long long)(slot0 + q - nom_split) * G + gq; };
  auto load_o = [&](int q) {
    const long long io = q < nom_split ? (base + q) * D : dO + prow(q) * D;
    return *reinterpret_cast<const f32x4*>(tmp + io + col);
  };
  auto load_ms = [&](int q, float& m, float& s) {
    const bool whole = q < nom_split;
    m = mls[whole ? base + q : dm + prow(q)];
    s = ess[whole ? base + q : ds + prow(q)];
  };

  // Unconditional loads (an index past the nominal list re-reads its last entry), and
  // no arithmetic on them before the context length is known: a guarded or consumed
  // load would make the compiler wait for it before issuing the next one.
  // Output rows per thread (states pg + NPG i) loaded up front: 320 states cover the
  // 196 partitions of a 100K-token context plus its cut items' pieces (with one chunk,
  // at most 8 rows per thread).
  constexpr int kSpecO = CHUNKS == 1 ? (320 / NPG < 8 ? 320 / NPG : 8) : 320 / NPG;
  constexpr int kSpecMS = 2;  // statistics per thread: partial states tid + 256 j
  f32x4 so[kSpecO];
  float sm[kSpecMS], ss[kSpecMS];
#pragma unroll
  for (int j = 0; j < kSpecMS; ++j) load_ms(min(tid + 256 * j, nom_fold - 1), sm[j], ss[j]);
#pragma unroll
  for (int i = 0; i < kSpecO; ++i) so[i] = load_o(min(pg + NPG * i, nom_fold - 1));

  int n = a.ctx[b];
  // The output address and the table shape load within the same round trip (they are
  // not used before it ends).
  asm volatile("" ::"s"(n), "s"(a.out), "s"(a.MB), "s"(a.P), "s"(a.o_ss), "s"(a.o_sh));
  const int cap = a.MB * kBlockSize;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  int nparts = (n + a.P - 1) / a.P;
  if (nparts > a.Pmax) nparts = a.Pmax;
  const int p_split = nom_split < nparts ? nom_split : nparts;
  int nfold = nparts;
  if (p_split < nparts) {
    const int sub = a.P >> sh;
    // Tokens of the last partition; a context beyond the planning bound (nparts
    // clamped to Pmax) still has at most P there, hence at most 2^sh pieces.
    const int last_tok = min(a.P, n - (nparts - 1) * a.P);
    nfold = p_split + ((nparts - 1 - p_split) << sh) + (last_tok + sub - 1) / sub;
  }
  if (p_split == nparts && nparts <= 1) return;  // phase 1 wrote the final output (or zeros)

  // Base-2 maxima into LDS; block max M.  The weights below read the maxima back from
  // LDS, so exp2(m_q - M) is exactly 1 for the largest (no fused multiply-add can keep
  // the rounding error of m * log2(e)).
  float mx = kNegInf;
  auto put_max = [&](int q, float m) {
    const float m2 = m * kLog2e;
    s_w[q] = m2;
    mx = fmaxf(mx, m2);
  };
#pragma unroll
  for (int j = 0; j < kSpecMS; ++j)
    if (tid + 256 * j < nfold) put_max(tid + 256 * j, sm[j]);
  for (int q = tid + 256 * kSpecMS; q < nfold; q += 256) {
    float m, s;
    load_ms(q, m, s);
    put_max(q, m);
  }
  mx = lane_reduce<false, 1>(mx);
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

  // Weights r_q = exp2(m_q - M) * s_q, and their sum.
  float wsum = 0.f;
#pragma unroll
  for (int j = 0; j < kSpecMS; ++j) {
    const int q = tid + 256 * j;
    if (q < nfold) {
      const float r = exp2_fast(s_w[q] - M) * ss[j];
      s_w[q] = r;
      wsum += r;
    }
  }
  for (int q = tid + 256 * kSpecMS; q < nfold; q += 256) {
    float m, s;
    load_ms(q, m, s);
    const float r = exp2_fast(s_w[q] - M) * s;
    s_w[q] = r;
    wsum += r;
  }
  wsum = lane_reduce<true, 1>(wsum);
  __syncthreads();  // weights visible; s_red reads of M done
  if (lane == 0) s_red[wv] = wsum;

  // sum_q r_q o_q over this thread's partial states.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kSpecO; ++i)
    if (pg + NPG * i < nfold) acc += so[i] * s_w[pg + NPG * i];
#pragma unroll 4
  for (int q = pg + NPG * kSpecO; q < nfold; q += NPG) acc += load_o(q) * s_w[q];

  // Lanes NC4 apart in a wave hold the same columns: cross-lane steps sum a wave's
  // partition lanes, then the 4 waves meet in LDS.
  if constexpr (NC4 < 64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = lane_reduce<true, NC4>(acc[j]);
  }
  if (lane < NC4) s_acc[wv][d4] = acc;
  __syncthreads();
  if (tid < NC4) {
    const float total = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    const f32x4 o = (s_acc[0][d4] + s_acc[1][d4]) + (s_acc[2][d4] + s_acc[3][d4]);
    const float inv = 1.f / total;
    const float vals[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    store_out<DT, 4>(a.out,
                     (size_t)b * (size_t)a.o_ss + (size_t)hq * (size_t)a.o_sh +
                         chunk * kReduceCols + tid * 4,
                     vals);
  }
}

// ---- dispatch --------------------------------------------------------------------------
// Work-group shape of the matrix-core kernel (see attn_mfma_kernel):
//   0 = 2 waves, pipeline depth 3 (head_dim 128) / 2 (head_dim 256)
//   1 = 1 wave,  pipeline depth 2 (one block in flight while the previous one is used)
//   2 = 4 waves, pipeline depth 2
//   3 = 1 wave,  pipeline depth 5 / 3
//  -1 = automatic (default): 2 when a work-group streams more than 64 blocks (a
//       partition longer than 1024 tokens, i.e. V1 over long contexts: four waves
//       share its blocks; batched 256 x U{512..4096}: 199 us, 224 with two waves); else,
//       for grids of at least two work-groups per compute unit, 1 in phase 1 of V2
//       (cold KV: long_100k 38.9 us/step against 40.2 with the same wave 5 deep and 39.4
//       3 deep, mixed_d256 at partition 512 and 256 likewise; more loads in flight per
//       compute unit measured slower) and 3 in V1 (many short sequences: with cache-warm
//       KV, 256 x 256 tokens took 23 us 5 deep and 48 us 2 deep); else 0 (more waves for
//       small grids: single_8k 11.5 us, 11.9 with one wave).
constexpr int kAutoVariant = -1;
constexpr long long kOrderMinItems = 256;  // longest-first V1 order from this many items
constexpr long long kAutoOneWaveGrid = 512;
constexpr int kAutoFourWaveBlocks = 64;
std::atomic<int> g_mfma_variant{-2};  // -2: not yet read from the environment

int mfma_variant_setting() {
  int v = g_mfma_variant.load(std::memory_order_relaxed);
  if (v == -2) {
    v = kAutoVariant;
    const char* e = std::getenv("PA_MFMA_VARIANT");
    if (e && e[0] >= '0' && e[0] <= '3' && e[1] == '\0') v = e[0] - '0';
    g_mfma_variant.store(v, std::memory_order_relaxed);
  }
  return v;
}

int mfma_variant(const dim3& grid, int partition_tokens, bool single_pass) {
  const int v = mfma_variant_setting();
  if (v != kAutoVariant) return v;
  if (partition_tokens > kAutoFourWaveBlocks * kBlockSize) return 2;
  const long long wgs = (long long)grid.x * grid.y * grid.z;
  if (wgs < kAutoOneWaveGrid) return 0;
  return single_pass ? 3 : 1;
}

struct Launch {
  dim3 grid;        // the launch grid (row 1 of a single-launch V2 included)
  dim3 work;        // the phase-1 part of it (kernel-shape choice)
  size_t lds;       // dynamic LDS bytes (the merge weights of a single-launch V2)
  hipStream_t st;
  hipEvent_t e0, e1;
};

template <typename K>
void launch(K kernel, const Launch& l, int threads, const AttnArgs& a) {
  hipExtLaunchKernelGGL(kernel, l.grid, dim3(threads), l.lds, l.st, l.e0, l.e1, 0, a.ctx, a.bt,
                        a.q, a.Pmax, a.Hkv | (a.order_seqs << 16), a.MB, a.P, a.q_sh,
                        (a.split.first << 4) | a.split.shift | (a.fused ? 1 << 30 : 0), a.q_ss,
                        a.bt_ss, a);
}

template <int DT, int D, int G>
hipError_t launch_attn_t(const AttnArgs& a, const Launch& l) {
  if constexpr ((DT == PA_BF16 || DT == PA_F16) && G >= 4) {
    switch (mfma_variant(l.work, a.P, a.Pmax == 1)) {
      case 0: launch(attn_mfma_kernel<DT, D, G, 2, (D == 128 ? 3 : 2)>, l, 2 * 64, a); break;
      case 1: launch(attn_mfma_kernel<DT, D, G, 1, 2>, l, 64, a); break;
      case 3: launch(attn_mfma_kernel<DT, D, G, 1, (D == 128 ? 5 : 3)>, l, 64, a); break;
      default: launch(attn_mfma_kernel<DT, D, G, 4, 2>, l, 4 * 64, a); break;
    }
  } else {
    launch(attn_valu_kernel<DT, D, G>, l, kThreads, a);
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_attn_g(int G, const AttnArgs& a, const Launch& l) {
  switch (G) {
    case 1: return launch_attn_t<DT, D, 1>(a, l);
    case 2: return launch_attn_t<DT, D, 2>(a, l);
    case 4: return launch_attn_t<DT, D, 4>(a, l);
    case 8: return launch_attn_t<DT, D, 8>(a, l);
    case 16: return launch_attn_t<DT, D, 16>(a, l);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_attn_d(int D, int G, const AttnArgs& a, const Launch& l) {
  if (D == 128) return launch_attn_g<DT, 128>(G, a, l);
  if (D == 256) return launch_attn_g<DT, 256>(G, a, l);
  return hipErrorInvalidValue;
}

template <int DT, int D>
hipError_t launch_reduce_dd(const ReduceArgs& a, int S, hipStream_t st) {
  // LDS: one float per partial state of a head: partitions, plus the pieces of cut ones.
  long long fold = a.Pmax;
  if (a.split.shift > 0) {
    const long long items = (long long)a.Pmax * a.Hkv * S;
    const long long cut = (items - a.split.first) << a.split.shift;
    fold += std::min(cut, (long long)a.Pmax << a.split.shift);
  }
  if (fold > kMaxFold) return hipErrorInvalidValue;
  const size_t lds = (size_t)fold * sizeof(float);
  const long long heads = (long long)S * a.Hq;
  // Workspace offsets in 256-byte units from tmp_out (see PA_REDUCE_LEAD_PARAMS).
  const char* ws = reinterpret_cast<const char*>(a.tmp_out);
  bool ok = true;
  auto units = [&](const void* p) -> int32_t {
    if (!p) return 0;
    const long long d = reinterpret_cast<const char*>(p) - ws;
    if (d < 0 || d % 256 || d / 256 > 0x7fffffffLL) ok = false;
    return (int32_t)(d / 256);
  };
  const int32_t u_max = units(a.max_logits), u_sum = units(a.exp_sums);
  const int32_t u_pout = units(a.split.piece_out), u_pmax = units(a.split.piece_max),
                u_psum = units(a.split.piece_sum);
  if (!ok || a.split.first < 0 || a.split.first >= (1 << 27) || a.split.shift > 15)
    return hipErrorInvalidValue;
  const int32_t split = (a.split.first << 4) | a.split.shift;
  if (heads >= kReduceWideHeads) {
    hipLaunchKernelGGL((reduce_kernel<DT, D, 1>), dim3((unsigned)heads, 1), dim3(256), lds, st,
                       a.ctx, a.tmp_out, a.Hq, a.Hkv, a.Pmax, split, u_max, u_sum, u_pout, u_pmax,
                       u_psum, a);
  } else {
    hipLaunchKernelGGL((reduce_kernel<DT, D, 8>), dim3((unsigned)heads, 8), dim3(256), lds, st,
                       a.ctx, a.tmp_out, a.Hq, a.Hkv, a.Pmax, split, u_max, u_sum, u_pout, u_pmax,
                       u_psum, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_reduce_d(int D, const ReduceArgs& a, int S, hipStream_t st) {
  if (D == 128) return launch_reduce_dd<DT, 128>(a, S, st);
  if (D == 256) return launch_reduce_dd<DT, 256>(a, S, st);
  return hipErrorInvalidValue;
}

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

int set_mfma_variant(int v) {
  if (v < kAutoVariant || v > 3) return -1;
  g_mfma_variant.store(v, std::memory_order_relaxed);
  return 0;
}

int get_mfma_variant() { return mfma_variant_setting(); }

Kernel kernel_for(int dtype, int group) {
  return (dtype != PA_F32 && group >= 4) ? Kernel::kMfma : Kernel::kValu;
}

long long phase1_workgroups(const AttnArgs& a, int num_seqs) {
  const long long items = (long long)a.Pmax * a.Hkv * num_seqs;
  if (a.split.shift == 0) return items;
  return a.split.first + ((items - a.split.first) << a.split.shift);
}

long long fold_states(const AttnArgs& a, int num_seqs) {
  long long fold = a.Pmax;
  if (a.split.shift > 0) {
    const long long items = (long long)a.Pmax * a.Hkv * num_seqs;
    const long long cut = (items - a.split.first) << a.split.shift;
    fold += std::min(cut, (long long)a.Pmax << a.split.shift);
  }
  return fold;
}

hipError_t launch_attention(int dtype, int head_dim, int group, const AttnArgs& a, int num_seqs,
                            hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  dim3 grid(a.Pmax, a.Hkv, num_seqs);
  const long long items = (long long)a.Pmax * a.Hkv * num_seqs;
  const long long wgs = phase1_workgroups(a, num_seqs);
  if (a.split.shift > 0) {
    if (a.split.first < 0 || a.split.first > items || wgs > kMaxSplitGrid)
      return hipErrorInvalidValue;
    grid = dim3((unsigned)wgs, 1, 1);
  }
  Launch l{grid, grid, 0, stream, ev_start, ev_stop};
  if (a.fused) {
    // Row 0: the phase-1 work-groups on a linear index; row 1: the merge work-groups
    // (the first fused_m of its wgs slots).  The host checked fused_m <= wgs, the
    // counters and the workspace size.
    if (wgs > kMaxSplitGrid || a.fused_m > wgs || !a.counters) return hipErrorInvalidValue;
    l.grid = dim3((unsigned)wgs, 2, 1);
    l.work = dim3((unsigned)wgs, 1, 1);
    l.lds = (size_t)2 * fold_states(a, num_seqs) * sizeof(float);
  }
  // Longest-first order for V1 on the matrix-core kernel when the grid has more (sequence,
  // KV head) items than compute units, i.e. runs in more than one wave of work-groups,
  // and a work-group covers more than 1024 tokens (the four-wave shape).  The ordering
  // costs each work-group a few microseconds (the ranking and one more dependent round
  // trip): with 256 sequences of 256 tokens that doubled the step (23 -> 49 us), with
  // 2048 tokens it costs ~7 us when all lengths are equal, and with U{512..4096} lengths
  // it saves ~27 us.
  // With V2 (Pmax > 1), several sequences and no split: the compacted item order (both
  // attention kernels).
  AttnArgs ao = a;
  ao.order_seqs = 0;
  const bool mfma = kernel_for(dtype, group) == Kernel::kMfma;
  if (a.Pmax == 1 && a.split.shift == 0 && mfma && num_seqs <= kOrderMaxSeqs &&
      (long long)num_seqs * a.Hkv >= kOrderMinItems && a.P > kAutoFourWaveBlocks * kBlockSize)
    ao.order_seqs = num_seqs;
  if (a.Pmax > 1 && a.split.shift == 0 && num_seqs >= 2 && num_seqs <= kOrderMaxSeqs)
    ao.order_seqs = num_seqs;
  switch (dtype) {
    case PA_F32: return launch_attn_d<PA_F32>(head_dim, group, ao, l);
    case PA_F16: return launch_attn_d<PA_F16>(head_dim, group, ao, l);
    case PA_BF16: return launch_attn_d<PA_BF16>(head_dim, group, ao, l);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(int dtype, int head_dim, const ReduceArgs& a, int num_seqs,
                         hipStream_t stream) {
  switch (dtype) {
    case PA_F32: return launch_reduce_d<PA_F32>(head_dim, a, num_seqs, stream);
    case PA_F16: return launch_reduce_d<PA_F16>(head_dim, a, num_seqs, stream);
    case PA_BF16: return launch_reduce_d<PA_BF16>(head_dim, a, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
