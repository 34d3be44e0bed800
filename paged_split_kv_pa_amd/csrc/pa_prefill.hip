// Paged prefix-prefill attention for gfx950 (MI355X).
//
// Source: project_6 optimizations/prefix_prefill_patch.py (commit fee8f1b), docstring:
// the prefix_prefill kernel is Flash-Attention style -- a grid of (batch, heads,
// query tiles of BLOCK_M positions), K/V tiles of BLOCK_N tokens staged in on-chip
// memory, fp16/bf16, head_dim 128 (256 less often), GQA.  What it computes (the reading stated with the
// oracle): new token i of sequence b (absolute position c_b + i) attends to the c_b
// prefix tokens in the paged cache and to new tokens 0..i, whose K/V arrive packed.
//
// Work-group: 8 waves, R query rows of one KV head g of one sequence (R = 256 at head_dim
// 128, 128 at 256): positions [p0, p0 + R/G) x the G query heads of g, row r = (position
// p0 + r / G, head g*G + r % G).  Sharing every K/V tile among the G heads and R/G
// positions is what makes the tile traffic small next to the MFMA work.  Wave w owns
// R/8 rows, as column groups of 16 rows (the MFMA's 16 columns): two at head_dim 128,
// one at 256.
//
// Two waves share each SIMD, and they take turns: the work of a wave alternates between
// a matrix phase (O += P V for the previous tile, then S^T = K Q^T for this one) and a
// softmax phase (row max, rescale, P = exp2(...)), and waves 0-3 run their matrix phase
// while waves 4-7 run their softmax phase and the other way round, with a work-group
// barrier between phases.  So the matrix cores of a SIMD are fed by one wave while the
// other one's exponentials run on the VALU.
//
// Per 64-key tile: K and V rows are loaded from the cache (key < c, through the
// block table) or from the packed new tokens (c <= key < c + L), into padded LDS rows.
//   S^T = K Q^T:   v_mfma_f32_16x16x32, A = 16 keys x 32 dims (LDS), B = Q (registers):
//                  lane (r16, kg) gets keys 4kg..4kg+3 of query row r16.
//   online softmax per query row in base 2 (scale * log2 e folded in), causal mask on
//                  the tiles that reach the row's own position, lazy rescale as in decode.
//   O += P V:      v_mfma_f32_16x16x32 over 32 keys = two 16-key row blocks: the S^T
//                  accumulators of the two blocks are exactly the A operand (k-slot e of
//                  lane group kg is key 16(2s + e/4) + 4kg + e%4); the B operand comes
//                  from V in LDS through the gfx950 transposing read, in that key order.
//                  P goes in as one fp16 value (11 significant bits), and V as fp16 too:
//                  bf16 V is converted when it is written to LDS, exactly for every
//                  |v| < 65536 (bf16's 8-bit significand fits fp16's 11; below fp16's
//                  normal range the absolute error is at most 2^-25).  A value that does
//                  not fit is noted, and the call is recomputed by a second launch with P
//                  as a 16-bit high part plus a 16-bit low part in the input type (about
//                  16 significant bits, V unconverted).  bf16 P alone (8 bits) is not
//                  enough: with peaky softmax rows the rounding of P moves outputs near
//                  zero by more than the 2e-3 absolute tolerance.  The row sums of P add
//                  exactly the values the products use (on the VALU).
// K and V have two LDS buffers each; a tile's K is written one phase before its first
// QK^T and its V one phase before its first PV, from loads issued two phases earlier.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>


#include "pa_decode.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;
constexpr int kThreads = 512;  // 8 waves
constexpr int kTile = 64;      // keys per K/V tile

// Work-group shape for head_dim D.  A wave owns CG column groups of 16 query rows: two at
// D = 128, one at D = 256, where the output accumulators of 16 rows already take 64
// registers per lane (two waves per SIMD leave 256 per lane).
template <int D>
struct Shape {
  static constexpr int CG = D == 128 ? 2 : 1;  // 16-row column groups per wave
  static constexpr int ROWS = 8 * 16 * CG;     // query rows per work-group
  static constexpr int KK = D / 32;            // k steps of QK^T
  static constexpr int JD = D / 16;            // 16-column blocks of O
  static constexpr int CH = D / 8;             // 16-byte chunks per K / V row
  static constexpr int ROW = CH + 2;           // LDS row stride, 16-byte units
  static constexpr int XC = CH / 8;            // chunks of a row one thread stages
};

static_assert(Shape<128>::ROWS == prefill_rows(128) && Shape<256>::ROWS == prefill_rows(256),
              "work-group rows as the host sizes the partial states");

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to nearest-even 16-bit values, lo in the low half (one
// v_cvt_pk_{bf16,f16}_f32).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (BF)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Larger of two floats, NaN if either is (IEEE maximum: one v_maximum3_f32 for up to three
// operands, where the NaN-ignoring fmaxf first quiets each operand with a v_max of itself).
__device__ __forceinline__ float fmax_p(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups of one MFMA column),
// with the two gfx950 half-swaps (upper 32 lanes with lower 32, odd 16-lane rows with
// even ones).  The swapped pair is passed through an empty asm: without it the compiler
// (ROCm 7.2) emitted the float max of the two results with the same register twice.
__device__ __forceinline__ float max_over_groups(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t a0 = a[0], a1 = a[1];
  asm("" : "+v"(a0), "+v"(a1));
  u = __builtin_bit_cast(uint32_t, fmax_p(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1)));
  const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  uint32_t b0 = b[0], b1 = b[1];
  asm("" : "+v"(b0), "+v"(b1));
  return fmax_p(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

// sum over lanes l, l ^ 16, l ^ 32, l ^ 48, with the same half-swaps; the result is
// bitwise the same in all four lanes (each adds the same two partial sums).
__device__ __forceinline__ float sum_over_groups(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t a0 = a[0], a1 = a[1];
  asm("" : "+v"(a0), "+v"(a1));
  u = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1));
  const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  uint32_t b0 = b[0], b1 = b[1];
  asm("" : "+v"(b0), "+v"(b1));
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

// The two 16-bit halves of a packed pair, widened to float.
template <bool BF>
__device__ __forceinline__ float unpack_lo(uint32_t w) {
  if constexpr (BF) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <bool BF>
__device__ __forceinline__ float unpack_hi(uint32_t w) {
  if constexpr (BF) return __builtin_bit_cast(float, w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane j
// receives element j % 4 of the 8-byte rows read by lanes 4e + j / 4, e = 0..3 (the
// lane layout was checked on the device with an in-bounds probe).
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// LDS rows of K and V are padded by 32 bytes (288 bytes at head_dim 128, 544 at 256): a
// row stride of 32 bytes modulo 256 leaves both operand reads free of bank conflicts with
// plain linear addresses (measured with the LDS bank-conflict counter: the 16-byte reads
// of 16 rows per K operand, and the 8-byte transposing reads of 8 rows per half-wave for
// V; a 256-byte row conflicts 28 cycles per K read, a 272-byte row 4).

// Most-keys-first order over sequences.  A work-group's work grows with the keys it
// attends to (its sequence's prefix plus the new tokens up to its positions), and
// work-groups start in grid order: a sequence with a long prefix whose work-groups start
// last runs on alone at the end (4 sequences with 4096 / 0 / 1000 / 16384-token prefixes:
// the 16384 one came last).  Work-group z takes the sequence with exactly z sequences
// before it (more keys, or as many and a lower index), from every sequence's prefix plus
// new-token count (one round trip for all of them), and its position blocks run last
// first (the last ones attend to the most keys).  The result of each (sequence, head,
// position) does not depend on which work-group computes it.
__device__ __forceinline__ int seq_of_key_rank(const PrefillArgs& a, int S, int r,
                                               long long* s_key, int* s_pick) {
  for (int t = threadIdx.x; t < S; t += blockDim.x)
    s_key[t] = (long long)a.ctx[t] + ((long long)a.query_start[t + 1] - a.query_start[t]);
  __syncthreads();
  for (int c = threadIdx.x; c < S; c += blockDim.x) {
    const long long kc = s_key[c];
    int rank = 0;
    for (int k = 0; k < S; ++k) {
      const long long kk = s_key[k];
      rank += (kk > kc) | ((kk == kc) & (k < c));
    }
    if (rank == r) *s_pick = c;
  }
  __syncthreads();
  return *s_pick;
}

// ---- planned schedule ----------------------------------------------------------------
// A row block is the work of the non-planned grid's work-group: positions [p0, p0 + kPos)
// of one sequence and one KV head, over keys [0, c + min(L, p0 + kPos)) in t 64-key tiles.
// Work-groups start in grid order and one runs per compute unit, so a launch whose row
// blocks differ in length (a long prefix next to short ones, or a few row blocks over a
// long prefix) ends on its longest row blocks alone.  The planned schedule cuts every
// row block of more than C tiles into nch = ceil(t / C) chunks of consecutive tiles (C =
// max(16, ceil(5W / 4N)) for W tiles in the launch over N compute units: a chunk holds at
// most 1.25 units' fair share, and only row blocks longer than that are cut, since every
// extra chunk costs a partial write and its share of a fold) and lists the items (a
// chunk, or a whole row block, of one KV head) largest first; work-group j takes entry j
// of the list, so the dispatcher hands out the work longest-processing-time first.
//
// prefill_plan_kernel writes the list: a counting sort by item size (tiles, capped at
// kSizeKeys - 1) from largest to smallest; each row block reserves its items' places in
// its size bucket with one LDS atomic (so the order among equal sizes varies from run to
// run; no result depends on it: an item's work, slot and fold order follow from its row
// block, head and chunk alone), its items by KV head, then chunk.  A chunk writes its
// (row max, row sum, unnormalised output) to a slot of the workspace (the chunks of one
// row block and head in consecutive slots); the last chunk
// of a row block and head to finish folds them all with the log-sum-exp rule, in chunk
// order (see the end of prefill_kernel), with one arrival counter per row block and head.
// A row that sees no key of a chunk (when the chunk starts inside the causal part) leaves
// (-inf, 0, 0), which the fold weighs by 0.
//
// Workspace: header {C, chunk items with slots, items, cut (row block, head) pairs}, then
// one entry of kItemWords int32 per item.
constexpr int kItemWords = 16;
enum { kItB = 0, kItG, kItXb, kItK, kItNch, kItSlot, kItCut, kItC, kItR0, kItL, kItTb, kItNt };
constexpr int kSizeKeys = 4096;
constexpr int kScDev = 16;  // cache-policy bits of a device-scope access (sc1)

// Buffer resource over the prefill workspace (offsets below 2 GiB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

__device__ __forceinline__ int plan_tiles(int c, int L, int xb, int kpos) {
  return (c + min(L, (xb + 1) * kpos) + kTile - 1) / kTile;
}

// Chunks of a row block of t tiles for chunk length C (C up to 2^31 - 1: no overflow).
__device__ __forceinline__ int chunks_of(int t, int C) { return t / C + (t % C != 0); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2, 4 and 8
// within each row of 16 lanes, then the last lane of row 0 added to row 1, of row 2 to
// row 3, and of row 1 to rows 2 and 3 (a lane with no source in a step adds 0).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sums over the 512 threads of a work-group of N values per thread
// (0 past the data), one pair of barriers for all N; tot[i] receives the sum of the i-th.
// s_tmp: 8 N words of LDS.
template <int N>
__device__ void block_exclusive_scans(const int (&v)[N], int (&ex)[N], int (&tot)[N], int* s_tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    incl[i] = wave_inclusive_scan(v[i]);
    if (lane == 63) s_tmp[8 * i + w] = incl[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int off = 0, t = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = s_tmp[8 * i + k];
      off += k < w ? x : 0;
      t += x;
    }
    ex[i] = off + incl[i] - v[i];
    tot[i] = t;
  }
  __syncthreads();
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int in[1] = {v};
  int ex[1], tot[1];
  block_exclusive_scans<1>(in, ex, tot, s_tmp);
  *total = tot[0];
  return ex[0];
}

// One work-group of 512 threads; S <= kOrderMaxSeqs sequences; kpos query positions per
// row block.
__global__ void __launch_bounds__(512) prefill_plan_kernel(const PrefillArgs a, int S, int kpos) {
  __shared__ int s_c[kOrderMaxSeqs], s_r0[kOrderMaxSeqs], s_L[kOrderMaxSeqs];
  __shared__ int s_npb[kOrderMaxSeqs], s_order[kOrderMaxSeqs], s_rbpre[kOrderMaxSeqs + 1];
  __shared__ int s_bucket[kSizeKeys];  // items per size key, then the key's next position
  __shared__ int s_tmp[24];
  __shared__ int s_bad;
  __shared__ unsigned long long s_wsum;
  const int tid = threadIdx.x;
  const int cap = a.MB * kBlockSize;
  const int H = a.Hkv;
  if (tid < S) {
    int r1 = a.query_start[tid + 1], r0 = a.query_start[tid];
    r1 = min(r1, a.T);
    r0 = min(max(r0, 0), r1);
    int c = a.ctx[tid];
    c = c < 0 ? 0 : (c > cap ? cap : c);
    s_c[tid] = c;
    s_r0[tid] = r0;
    s_L[tid] = r1 - r0;
    s_npb[tid] = (min(r1 - r0, a.max_query_len) + kpos - 1) / kpos;
  }
  for (int k = tid; k < kSizeKeys; k += blockDim.x) s_bucket[k] = 0;
  if (tid == 0) {
    s_wsum = 0;
    s_bad = 0;
  }
  __syncthreads();
  // Sequences most keys first (prefix plus new tokens; ties by index).
  if (tid < S) {
    const long long kc = (long long)s_c[tid] + s_L[tid];
    int rank = 0;
    for (int k = 0; k < S; ++k) {
      const long long kk = (long long)s_c[k] + s_L[k];
      rank += (kk > kc) | ((kk == kc) & (k < tid));
    }
    s_order[rank] = tid;
  }
  __syncthreads();
  int nrb = 0;
  const int pre = block_exclusive_scan(tid < S ? s_npb[s_order[tid]] : 0, s_tmp, &nrb);
  if (tid < S) s_rbpre[tid] = pre;  // by rank
  // Row block p (fixed order): rank r with s_rbpre[r] <= p, position block last first.
  auto row_block = [&](int p, int& b, int& xb) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_rbpre[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    b = s_order[lo];
    xb = s_npb[b] - 1 - (p - s_rbpre[lo]);
  };
  __syncthreads();
  // Each wave sums its row blocks' tiles (at most 64 x 2^25, below 2^31) and adds that
  // once: with one 64-bit LDS atomic per row block on the one word, this loop took ~2.5 us.
  for (int p0 = 0; p0 < nrb; p0 += blockDim.x) {
    const int p = p0 + tid;
    int t = 0;
    if (p < nrb) {
      int b, xb;
      row_block(p, b, xb);
      t = plan_tiles(s_c[b], s_L[b], xb, kpos);
    }
    t = wave_inclusive_scan(t);
    if ((tid & 63) == 63 && t > 0) atomicAdd(&s_wsum, (unsigned long long)t);
  }
  __syncthreads();
  const unsigned long long W = s_wsum * (unsigned long long)H;
  const unsigned long long per = 4ull * (unsigned long long)max(a.ncu, 1);  // C >= 1.25 W / N
  // Tiles per row block stay below 2^25 (2^30 keys at most), so the per-row-block
  // arithmetic below is 32-bit (64-bit division is a long software sequence).
  int C = a.chunk > 0 ? a.chunk
                      : (int)min(max((unsigned long long)kPrefillAutoMinChunk,
                                     (5 * W + per - 1) / per),
                                 (unsigned long long)0x7fffffff);
  // Pass 1 (twice at most): items per size key and the totals.  A plan beyond the sizes
  // the host provided for (not expected) falls back to whole row blocks, which fit.
  int nitems = 0, nslots = 0, ncut = 0;
  for (int attempt = 0; attempt < 2; ++attempt) {
    int li = 0, ls = 0, lc = 0;
    for (int p = tid; p < nrb; p += blockDim.x) {
      int b, xb;
      row_block(p, b, xb);
      const int t = plan_tiles(s_c[b], s_L[b], xb, kpos);
      const int nch = chunks_of(t, C);
      const int key = min((t + nch - 1) / nch, kSizeKeys - 1);
      atomicAdd(&s_bucket[key], H * nch);
      li += H * nch;
      ls += nch > 1 ? H * nch : 0;
      lc += nch > 1 ? H : 0;
    }
    {
      const int in[3] = {li, ls, lc};
      int ex[3], tot[3];
      block_exclusive_scans<3>(in, ex, tot, s_tmp);
      nitems = tot[0];
      nslots = tot[1];
      ncut = tot[2];
    }
    if (nitems <= a.item_bound && nslots <= a.slot_bound && ncut <= a.cut_bound) break;
    C = 0x7fffffff;
    for (int k = tid; k < kSizeKeys; k += blockDim.x) s_bucket[k] = 0;
    __syncthreads();
  }
  // Whole row blocks always fit for query_start as the interface requires (non-decreasing,
  // so the chunks add up to at most T); otherwise nothing is listed and nothing written.
  if (nitems > a.item_bound || nslots > a.slot_bound || ncut > a.cut_bound) {
    if (tid == 0) {
      a.plan[0] = (int)C;
      a.plan[1] = a.plan[2] = a.plan[3] = 0;
    }
    return;
  }
  // Positions: keys from the largest down (thread t owns keys [8t, 8t + 8)).
  {
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kSizeKeys / 512; ++i) sum += s_bucket[kSizeKeys - 1 - (tid * 8 + i)];
    int tot = 0;
    int off = block_exclusive_scan(sum, s_tmp, &tot);
#pragma unroll
    for (int i = 0; i < kSizeKeys / 512; ++i) {
      const int k = kSizeKeys - 1 - (tid * 8 + i);
      const int n = s_bucket[k];
      s_bucket[k] = off;
      off += n;
    }
  }
  __syncthreads();
  // Pass 2, in rounds of 512 row blocks in the fixed order (sequences most keys first,
  // position blocks last first): places in the size buckets, then slots and counters,
  // which follow the fixed order.
  int* items = a.plan + 8;
  int slot_base = 0, cut_base = 0;
  for (int p0 = 0; p0 < nrb; p0 += blockDim.x) {
    const int p = p0 + tid;
    int b = 0, xb = 0, nch = 0, key = -1;
    int t = 0;
    if (p < nrb) {
      row_block(p, b, xb);
      t = plan_tiles(s_c[b], s_L[b], xb, kpos);
      nch = chunks_of(t, C);
      key = min((t + nch - 1) / nch, kSizeKeys - 1);
    }
    const int in[2] = {nch > 1 ? H * nch : 0, nch > 1 ? H : 0};
    int ex[2], tot[2];
    block_exclusive_scans<2>(in, ex, tot, s_tmp);  // has barriers
    const int sl = ex[0], cu = ex[1], nsl = tot[0], ncu = tot[1];
    if (p < nrb) {
      const int pos = atomicAdd(&s_bucket[key], H * nch);
      // Inside the list, slots and counters by construction (the totals were checked
      // against the bounds); tested here as well, so that no store can leave them (a
      // plan that failed it would list nothing, below).
      const bool fits = pos + H * nch <= nitems &&
                        (nch == 1 || (slot_base + sl + H * nch <= nslots &&
                                      cut_base + cu + H <= ncut));
      if (!fits) s_bad = 1;
      if (fits)
      for (int g = 0; g < H; ++g)
        for (int k = 0; k < nch; ++k) {
          // Words kItB .. kItNt as three 16-byte stores.
          typedef int i32x4 __attribute__((ext_vector_type(4)));
          i32x4* e = reinterpret_cast<i32x4*>(items + (size_t)(pos + g * nch + k) * kItemWords);
          // Balanced cut: the first t mod nch chunks get one tile more.
          const int q = t / nch, r = t - q * nch;
          const int tb = k * q + min(k, r);
          static_assert(kItB == 0 && kItNch == 4 && kItTb == 10 && kItNt == 11, "entry layout");
          e[0] = i32x4{b, g, xb, k};
          e[1] = i32x4{nch, nch > 1 ? slot_base + sl + g * nch + k : 0, nch > 1 ? cut_base + cu + g : 0,
                       s_c[b]};
          e[2] = i32x4{s_r0[b], s_L[b], tb, q + (k < r ? 1 : 0)};
        }
    }
    slot_base += nsl;
    cut_base += ncu;
  }
  __syncthreads();
  if (tid == 0) {
    a.plan[0] = (int)C;
    a.plan[1] = s_bad ? 0 : nslots;
    a.plan[2] = s_bad ? 0 : nitems;
    a.plan[3] = s_bad ? 0 : ncut;
  }
}

// kSched: 0 grid order (grid (position blocks, Hkv, S)); 1 the most-keys-first order
// above over the same grid; 2 the planned schedule (a one-dimensional grid of items, see
// prefill_plan_kernel).  Separate instantiations, so the one-sequence kernel's register
// allocation is untouched by the others.
// kPrec: P as a high plus a low part in the input type (else one fp16 part, see the top
// of the file); with a.flag_check the kernel computes only if this call's overflow word
// is set.
template <int DT, int G, int D, int kSched, bool kPrec>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(const PrefillArgs a) {
  constexpr bool kBF = DT == PA_BF16;
  constexpr bool kPvBF = kBF && kPrec;  // PV operand type: bf16, else fp16
  constexpr bool kCvtV = kBF && !kPrec;  // bf16 V converted to fp16 in LDS
  if constexpr (kPrec) {
    if (a.flag_check && a.flags[a.epoch % kPrefillFlagSlots] != a.epoch) return;
  }
  using Sh = Shape<D>;
  constexpr int CG = Sh::CG, KK = Sh::KK, JD = Sh::JD, ROW = Sh::ROW, XC = Sh::XC;
  constexpr int kPos = Sh::ROWS / G;  // query positions per work-group
  __shared__ u32x4 s_k[2][kTile * ROW];
  __shared__ u32x4 s_v[2][kTile * ROW];
  __shared__ int s_pick;
  // At head_dim 128 the two-part form keeps the query operands in LDS, each wave's in
  // lane order (16-byte reads, conflict-free): its low parts of P need the registers.
  constexpr bool kQLds = kPrec && D == 128;
  // Row sums of P: in the one-part form on the matrix cores (one more product per column
  // group and key step, with an all-ones B operand, leaves sum_k P[row][k] in every
  // column, in O's row layout); in the two-part form on the VALU (high plus low parts).
  constexpr bool kSumMfma = !kPrec && D == 128;  // measured: MFMA at 128, VALU at 256
  __shared__ u32x4 s_q[kQLds ? 8 : 1][kQLds ? CG * KK : 1][64];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;  // 0: matrix phases on even phase numbers, 1: on odd ones
  const int lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;

  int g, b, xb, r0, L, c;
  // Tiles [tb, tb + ntiles) of the row block (all of them unless it is cut), chunk k of
  // nch; a cut row block's chunk writes its partial state to slot `slot`.
  int tb = 0, ntiles, nch = 1, slot = 0, kchunk = 0, cut_ord = 0;
  if constexpr (kSched == 2) {
    // Entry j of the plan's item list (scalar loads: the address is uniform).
    const int j = blockIdx.x;
    const int* e = a.plan + 8 + (size_t)j * kItemWords;
    if (j >= a.plan[2]) return;
    b = e[kItB];
    g = e[kItG];
    xb = e[kItXb];
    kchunk = e[kItK];
    nch = e[kItNch];
    slot = e[kItSlot];
    cut_ord = e[kItCut];
    c = e[kItC];
    r0 = e[kItR0];
    L = e[kItL];
    tb = e[kItTb];
    ntiles = e[kItNt];
  } else {
    g = blockIdx.y;
    b = blockIdx.z;
    xb = blockIdx.x;
    if constexpr (kSched == 1) {
      // The key counts live in the first K tile buffer, which is not written before the
      // barrier that ends the ranking.
      b = seq_of_key_rank(a, a.order_seqs, b, reinterpret_cast<long long*>(s_k[0]), &s_pick);
      xb = gridDim.x - 1 - blockIdx.x;
    }
    int r1 = a.query_start[b + 1];
    r0 = a.query_start[b];
    r1 = min(r1, a.T);
    r0 = min(max(r0, 0), r1);
    L = r1 - r0;
    if (xb * kPos >= L) return;
    c = a.ctx[b];
    const int cap = a.MB * kBlockSize;
    c = c < 0 ? 0 : (c > cap ? cap : c);
  }
  const int p0 = xb * kPos;

  // Keys this work-group needs: the prefix and new tokens up to its last position.
  const int pend = min(L, p0 + kPos);
  const int nkeys = c + pend;
  if (kSched != 2) ntiles = (nkeys + kTile - 1) / kTile;

  // ---- query operands and per-row state ----
  // Column group cg of this wave: rows 16 CG w + 16cg + (0..15); lane column r16.  The
  // softmax works on raw dot products scaled by |scale| log2(e); a negative scale is
  // carried by flipping the sign of q (exact in 16-bit floats), so max(scale * s) is
  // |scale| * max of the flipped products.
  u32x4 qf[CG][KK];  // [cg][kk]: Q[row r16][32kk + 8kg .. +7] (in LDS when kQLds)
  int qpos_col[CG];
  {
    const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      const int row = 16 * CG * w + 16 * cg + r16;
      const int pos = p0 + row / G;
      const int hq = g * G + row % G;
      qpos_col[cg] = pos;
      const bool valid = pos < L;
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                             ((size_t)(r0 + (valid ? pos : 0)) * a.Hq + hq) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qf[cg][kk] = (valid ? *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * kg)
                            : u32x4{0u, 0u, 0u, 0u}) ^ u32x4{flip, flip, flip, flip};
    }
    if constexpr (kQLds) {
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s_q[w][cg * KK + kk][lane] = qf[cg][kk];
    }
  }
  const float sl = fabsf(a.scale_log2);
  f32x4 O[CG][JD];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg)
#pragma unroll
    for (int j = 0; j < JD; ++j) O[cg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums of P: lane (r16, kg) adds up the probabilities of query row r16 over its
  // own keys (4 kg + i of every 16-key row block); the four lane groups are summed at
  // the end.
  float lsum[CG];
  f32x4 Lacc[kSumMfma ? CG : 1];
  const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // fp16 1.0
  float m_ref[CG];
  float negm[CG];  // -m_ref, or 0 while m_ref is -inf
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    m_ref[cg] = kNegInf;
    negm[cg] = 0.f;
    lsum[cg] = 0.f;
    if constexpr (kSumMfma) Lacc[cg] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- tile loads: thread tid moves XC chunks (lc, lc + 8, ...) of K and of V of tile row tid/8 ----
  // The 8 rows of a wave (rows 8 w .. 8 w + 7 of a tile) lie in one 16-token cache block,
  // so the block id is one value per wave, read with one uniform load a tile ahead of its
  // use.  A wave whose 8 rows are all prefix keys, or all new tokens, loads them from a
  // wave-uniform base plus a per-lane offset that is the same for every tile (no vector
  // address arithmetic); the waves that hold the end of the prefix or of the keys load
  // from both sources under complementary lane masks.  A row outside the keys, or a prefix
  // row whose block id is out of range, reads zeros (past the end of its buffer resource).
  // Every phase issues its loads, also past the last tile.
  const int lrow = tid >> 3, lc = tid & 7;  // chunks lc + 8 i of row lrow = 8 w + jrow
  const int jrow = lane >> 3;
  const size_t hstride = (size_t)kBlockSize * D;  // elements per (block, head)
  const char* const kc = static_cast<const char*>(a.k_cache) + (size_t)g * hstride * 2;
  const char* const vc = static_cast<const char*>(a.v_cache) + (size_t)g * hstride * 2;
  const char* const knew = static_cast<const char*>(a.k_new) + (size_t)g * D * 2;
  const char* const vnew = static_cast<const char*>(a.v_new) + (size_t)g * D * 2;
  const size_t bstride = (size_t)a.Hkv * hstride * 2;  // bytes per cache block
  const size_t nstride = (size_t)a.Hkv * D * 2;        // bytes per new token
  const int cmax = c > 0 ? c - 1 : 0;
  // Byte offsets of this lane's first chunk: in the wave's rows of a cache block, and in
  // its rows of the new tokens.
  const uint32_t off_pre = (uint32_t)((((8 * w) % kBlockSize + jrow) * D + 8 * lc) * 2);
  const uint32_t off_new = (uint32_t)(jrow * nstride + 16 * lc);
  // First key of this wave's rows in tile t (tile t of the loop is tile tb + t of the row block).
  auto wave_key = [&](int t) { return (tb + t) * kTile + 8 * w; };
  const __amdgpu_buffer_rsrc_t bt_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.bt + (size_t)b * a.MB), (short)0, a.MB * 4, 0x00020000);
  // Block id of this wave's rows of tile t (any if not prefix), as loaded (every lane
  // holds it).  take_block moves it to a scalar register where it is used, a phase after
  // the load, ahead of the next id's load into the same register; as the builtin, the
  // compiler hoisted that move to the top of the phase, where waiting for the id also
  // waited for the tile loads issued after it.
  auto fetch_block = [&](int t) {
    const int i = min(wave_key(t), cmax) / kBlockSize;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(bt_rs, 0, i * 4, 0);
  };
  auto take_block = [](int v) {
    int r;
    asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(r) : "v"(v));
    return r;
  };
  // Wave-uniform rows: a buffer resource at the wave's base (scalar arithmetic only).
  // (bytes: the resource's size; a load past it returns zeros and touches no memory)
  auto load_uniform = [&](u32x4 (&r)[XC], const char* base, uint32_t off,
                          int bytes = 0x7fffffff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < XC; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 128 * i, 0, 0));
  };
  auto load_rows = [&](u32x4 (&r)[XC], const char* cache, const char* fresh, int t, int blk) {
    const int kb = wave_key(t);
    if (kb + 8 <= c && (unsigned)blk < (unsigned)a.NB) {  // all prefix rows
      load_uniform(r, cache + (size_t)blk * bstride, off_pre);
    } else if (kb >= c && kb + 8 <= nkeys) {  // all new tokens
      load_uniform(r, fresh + (size_t)(r0 + kb - c) * nstride, off_new);
    } else {
      // Rows from both sources: the lanes of new-token rows load those (the new-token base
      // is that of key kb, before the prefix end for the other lanes, which do not use
      // it); the other lanes load from the cache block, through a resource of no bytes if
      // the block id is out of range, and rows outside the keys read past the resource:
      // zeros.  The two loads run under complementary lane masks into the same registers.
      const int key = kb + jrow;
      const bool nw = key >= c && key < nkeys;
      if (nw) {
        load_uniform(r, fresh + (ptrdiff_t)(r0 + kb - c) * (ptrdiff_t)nstride, off_new);
        // keeps the two branches' loads apart: merged into one load, its resource would be
        // a per-lane choice, which the compiler lowers to a loop over lanes
        asm volatile("" ::: "memory");
      } else {
        const bool blk_ok = (unsigned)blk < (unsigned)a.NB;
        const bool pre = key < c && blk_ok;
        load_uniform(r, blk_ok ? cache + (size_t)blk * bstride : cache, pre ? off_pre : 0x40000000u,
                     blk_ok ? (int)bstride : 0);
      }
    }
  };
  u32x4 kr[XC], vr[XC];
  auto load_k = [&](int t, int blk) { load_rows(kr, kc, knew, t, blk); };
  auto load_v = [&](int t, int blk) { load_rows(vr, vc, vnew, t, blk); };
  auto store_rows = [&](u32x4* dst, const u32x4 (&r)[XC]) {
#pragma unroll
    for (int i = 0; i < XC; ++i) dst[lrow * ROW + lc + 8 * i] = r[i];
  };
  // V rows as the PV products take them: bf16 converted to fp16 in the one-part form (a
  // value beyond fp16's range becomes an infinity; see the end of the kernel).
  auto cvt_v = [&](u32x4 (&r)[XC]) {
    if constexpr (kCvtV) {
#pragma unroll
      for (int i = 0; i < XC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = r[i][e];
          r[i][e] = pack2<false>(__builtin_bit_cast(float, wv << 16),
                                 __builtin_bit_cast(float, wv & 0xffff0000u));
        }
    }
  };
  auto store_v = [&](u32x4* dst, u32x4 (&r)[XC]) {
    cvt_v(r);
    store_rows(dst, r);
  };

  {
    const int blk0 = take_block(fetch_block(0));
    load_k(0, blk0);
    load_v(0, blk0);
    store_rows(s_k[0], kr);
    store_v(s_v[0], vr);
  }
  {
    const int blk1 = take_block(fetch_block(1));
    load_k(1, blk1);
    load_v(1, blk1);
  }
  int blk_k = fetch_block(2), blk_v = fetch_block(2);
  __syncthreads();

  f32x4 S[4][CG];  // [row block][cg]: S^T of the tile, keys 16rb + 4kg + i, query row r16
  // [cg][st]: P of the tile as PV A operands (keys of row blocks 2st, 2st+1), as the
  // 16-bit high parts (P) and, in the two-part form, low parts (Pl).
  u32x4 P[CG][2], Pl[kPrec ? CG : 1][2];

  // S^T of tile t.
  auto qk = [&](int t) {
    const u32x4* kb = s_k[t & 1];
    u32x4 ka[KK][4];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) ka[kk][rb] = kb[(16 * rb + r16) * ROW + 4 * kk + kg];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) S[rb][cg] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int QR = kQLds ? CG : 0;  // query operand reads per k step
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 qk_op[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) qk_op[cg] = kQLds ? s_q[w][cg * KK + kk][lane] : qf[cg][kk];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) S[rb][cg] = mfma32<kBF>(ka[kk][rb], qk_op[cg], S[rb][cg]);
    }
    // the K (and query) reads of the next k step run under the current step's products
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + QR, 0);
#pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4 + QR, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * CG, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * CG, 0);
  };
  // O += P V for tile t.  V operand [st][jd]: the 32 keys of step st (in the P k-slot
  // order) x head-dim 16 jd + (0..15); lane (j, kg) reads 8 bytes of key
  // 32 st + 4 kg + j / 4 (+16 for the second read), head-dim 16 jd + 4 (j % 4), and the
  // transposing read hands lane (n, kg) the 4 keys of its k-slots at head-dim 16 jd + n.
  auto pv = [&](int t) {
    const char* vbase = reinterpret_cast<const char*>(s_v[t & 1]);
    u32x4 vb[2][JD];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int jd = 0; jd < JD; ++jd) {
        const int key = 32 * st + 4 * kg + (r16 >> 2);
        const char* src = vbase + key * (ROW * 16) + 32 * jd + 8 * (r16 & 3);
        const u32x2 lo = lds_read_tr(src);
        const u32x2 hi = lds_read_tr(src + 16 * ROW * 16);
        vb[st][jd] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    if constexpr (kPrec) {
      // Per pair of 16-column blocks: the high-part products of both blocks and every
      // column group, then the low-part ones, so a product never waits for the one just
      // issued on the same accumulator.
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int jd = 0; jd < JD; jd += 2) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int cg = 0; cg < CG; ++cg)
              O[cg][jd + jj] = mfma32<kPvBF>(P[cg][st], vb[st][jd + jj], O[cg][jd + jj]);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int cg = 0; cg < CG; ++cg)
              O[cg][jd + jj] = mfma32<kPvBF>(Pl[cg][st], vb[st][jd + jj], O[cg][jd + jj]);
        }
      // V reads (two per operand) run two operands ahead of the products that use them
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < 2 * JD - 2; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * CG, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * CG, 0);
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int jd = 0; jd < JD; ++jd)
#pragma unroll
          for (int cg = 0; cg < CG; ++cg)
            O[cg][jd] = mfma32<false>(P[cg][st], vb[st][jd], O[cg][jd]);
        if constexpr (kSumMfma) {
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) Lacc[cg] = mfma32<false>(P[cg][st], ones, Lacc[cg]);
        }
      }
      // V reads (two per operand) run four operands ahead of the products that use them
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int k = 0; k < 2 * JD - 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, CG, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, (kSumMfma ? 6 : 4) * CG, 0);
    }
  };
  // Softmax of tile t: row max (masked keys become -inf on diagonal tiles, where S then
  // holds scaled logits), the rescale of O when a row max grows past the slack, and P.
  auto softmax = [&](int t) {
    const int kbase = (tb + t) * kTile;
    const bool diag = kbase + kTile - 1 > c + p0;  // some key of the tile may lie after some row
    // The row max only decides whether a row grows past its reference by more than the
    // slack, and it does exactly when the max over some lane's 16 keys does: so each lane
    // compares its own max, and the lanes' maxima are combined only on the (rare) rescale.
    float pm[CG];  // this lane's max over its keys 16 rb + 4 kg + i of the tile
    bool grow = false;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      if (diag) {
        // key kbase + 16 rb + 4 kg + i is visible to this lane's row iff it is at most
        // c + position and below nkeys, i.e. iff 16 rb + i <= lim (one compare with a
        // constant per score)
        const int lim = min(c + qpos_col[cg], nkeys - 1) - kbase - 4 * kg;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[rb][cg][i] = 16 * rb + i <= lim ? S[rb][cg][i] * sl : kNegInf;
      }
      // a chain of three-operand maxima (v_maximum3_f32): 8 instructions for 16 values
      float mx = fmax_p(fmax_p(S[0][cg][0], S[0][cg][1]), S[0][cg][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2)
        mx = fmax_p(fmax_p(mx, S[e / 4][cg][e % 4]), S[(e + 1) / 4][cg][(e + 1) % 4]);
      mx = fmax_p(mx, S[3][cg][3]);
      pm[cg] = mx;
      grow = grow || (diag ? mx : mx * sl) > m_ref[cg] + kRescaleSlack;
    }
    if (__any(grow)) {  // rare
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        const float rmax = max_over_groups(pm[cg]);
        const float m_new = fmaxf(m_ref[cg], diag ? rmax : rmax * sl);
        const float alpha = m_ref[cg] == kNegInf ? 0.f : exp2_fast(m_ref[cg] - m_new);
        m_ref[cg] = m_new;
        negm[cg] = m_new == kNegInf ? 0.f : -m_new;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kg + i);
#pragma unroll
        for (int j = 0; j < JD; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[cg][j][i] *= al[i];
        lsum[cg] *= alpha;  // this lane's sums are of row r16, the row alpha belongs to
        if constexpr (kSumMfma) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Lacc[cg][i] *= al[i];
        }
      }
    }
    // m_ref is finite here except in a chunk of the planned schedule (key 0 is visible to
    // every row and lies in tile 0): a chunk that starts inside the causal part can hold no
    // visible key for some rows yet, and negm = 0 gives them p = 0 until one appears.
    const float fs = diag ? 1.f : sl;  // diagonal tiles hold scaled logits already
    const f16x2 ones2 = {(_Float16)1.f, (_Float16)1.f};  // one-part row sums: p0 + p1 + sum
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      const float nm = negm[cg];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float p[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[4 * h + i] = exp2_fast(fmaf(S[2 * st + h][cg][i], fs, nm));
        uint32_t hw[4], lw[4];
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hw[e] = pack2<kPvBF>(p[2 * e], p[2 * e + 1]);
          if constexpr (kPrec) {
            const float h0 = unpack_lo<kPvBF>(hw[e]), h1 = unpack_hi<kPvBF>(hw[e]);
            lw[e] = pack2<kPvBF>(p[2 * e] - h0, p[2 * e + 1] - h1);
            part += (h0 + unpack_lo<kPvBF>(lw[e])) + (h1 + unpack_hi<kPvBF>(lw[e]));
          } else if constexpr (!kSumMfma) {
            part = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, hw[e]), ones2, part, false);
          }
        }
        if constexpr (!kSumMfma) lsum[cg] += part;
        P[cg][st] = u32x4{hw[0], hw[1], hw[2], hw[3]};
        if constexpr (kPrec) Pl[cg][st] = u32x4{lw[0], lw[1], lw[2], lw[3]};
      }
    }
  };

  // Phases: wave group grp runs the matrix work of tile t in phase 2t + grp and the
  // softmax of tile t in phase 2t + grp + 1; a barrier ends every phase.  Tile traffic,
  // the same in every wave: phase 2u + 1 writes K of tile u + 1 and requests K of tile
  // u + 2; phase 2u + 2 writes V of tile u + 1 and requests V of tile u + 2.  K of tile u
  // is read in phases 2u and 2u + 1, V of tile u in phases 2u + 2 and 2u + 3, so two
  // buffers of each hold.
  // Tile traffic of a phase: write tile u + 1 to LDS, request tile u + 2.  Both happen
  // in every phase, also past the last tile (the buffer written is not read again, the
  // rows requested read as zeros): with no branch around them the compiler's wait counts
  // stay close, and no wait drains the loads still in flight.
  // The next block id is requested before the tile loads, so that the wait for it, a
  // phase later, does not include them.
  auto io_k = [&](int u) {
    store_rows(s_k[(u + 1) & 1], kr);
    const int blk = take_block(blk_k);
    blk_k = fetch_block(u + 3);
    load_k(u + 2, blk);
  };
  // cvt: convert bf16 V here (group 0, in its matrix phase).  Group 1's conversion is
  // written in its matrix phase, a phase before this store; the compiler sinks it to the
  // store (pinning it in the matrix phase made that phase wait for the V loads: 4.5%
  // slower), and the same code with the conversion written at the store measured 1% slower.
  auto io_v = [&](int u, bool cvt) {
    if (cvt)
      store_v(s_v[(u + 1) & 1], vr);
    else
      store_rows(s_v[(u + 1) & 1], vr);
    const int blk = take_block(blk_v);
    blk_v = fetch_block(u + 3);
    load_v(u + 2, blk);
  };
  // One tile t of wave group GRP: the matrix phase 2t + GRP, then the softmax phase
  // 2t + GRP + 1.  Group 0 carries the V traffic in its matrix phase and the K traffic
  // in its softmax phase, group 1 the other way round, so that every phase has the
  // same traffic in all waves; the loop is written once per group.
#define PA_TILE(GRP, T)                                                               \
  do {                                                                                 \
    const int t_ = (T);                                                                \
    if (t_ >= 1) pv(t_ - 1);                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                 \
    if (t_ < ntiles) qk(t_);                                                           \
    _Pragma("unroll") for (int cg = 0; cg < CG; ++cg)                                 \
      _Pragma("unroll") for (int j = 0; j < JD; ++j) asm("" : "+v"(O[cg][j]));         \
    if (GRP == 0) {                                                                    \
      if (t_ >= 1) io_v(t_ - 1, true); /* phase 0 has no traffic */                    \
    } else {                                                                           \
      io_k(t_);                                                                        \
      cvt_v(vr); /* V of tile t + 1, stored in the next phase */                       \
    }                                                                                  \
    __syncthreads();                                                                   \
    if (t_ < ntiles) softmax(t_);                                                      \
    if (GRP == 0)                                                                      \
      io_k(t_);                                                                        \
    else                                                                               \
      io_v(t_, false);                                                                 \
    __syncthreads();                                                                   \
  } while (0)
  if (grp == 0) {
    for (int t = 0; t <= ntiles; ++t) PA_TILE(0, t);
    __syncthreads();  // the last phase: group 1's final PV
  } else {
    __syncthreads();  // phase 0: group 0's first QK^T
    for (int t = 0; t <= ntiles; ++t) PA_TILE(1, t);
  }
#undef PA_TILE

  // A V value fp16 does not hold was staged as an infinity, and the PV products carry it
  // into its head-dim column of O in every row of the work-group (as +-inf, or NaN where
  // p = 0): a non-finite accumulator marks this call for the two-part recompute.  So do
  // non-finite inputs and an fp32 overflow of O, which the recompute then meets as well.
  if constexpr (kCvtV) {
    bool bad = false;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg)
#pragma unroll
      for (int j = 0; j < JD; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad |= !__builtin_isfinite(O[cg][j][i]);
    if (bad)
      __hip_atomic_store(a.flags + a.epoch % kPrefillFlagSlots, a.epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- a chunk of a cut row block: its partial state; the last chunk to finish folds ----
  // O unnormalised (relative to the row's running max), in register order, so that every
  // store and load is 16 bytes per lane and contiguous over a wave.  The stores are
  // device-scope (they reach the memory side, where a work-group on another XCD reads
  // them); each wave waits for its own, then one thread counts the chunk in the row
  // block's arrival counter.  The work-group that completes the count resets it and
  // folds all chunks from memory, in chunk order (so the result does not depend on which
  // chunk came last): out = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k, M = max m_k.
  if (kSched == 2 && nch > 1) {
    const __amdgpu_buffer_rsrc_t rs = ws_rsrc(a.plan);
    const char* const wsb = reinterpret_cast<const char*>(a.plan);
    auto off = [&](const float* p) { return (int)(reinterpret_cast<const char*>(p) - wsb); };
    auto o_at = [&](int sl, int cg, int jd) {
      return a.part_o + ((((size_t)sl * 8 + w) * CG + cg) * JD + jd) * 256 + lane * 4;
    };
    auto st_at = [&](float* base, int sl, int cg) {
      return base + (((size_t)sl * 8 + w) * CG + cg) * 16;
    };
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
#pragma unroll
      for (int jd = 0; jd < JD; ++jd)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, O[cg][jd]), rs,
                                               off(o_at(slot, cg, jd)), 0, kScDev);
      if (kg == 0)  // row r16's running max (base 2)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_ref[cg]), rs,
                                              off(st_at(a.part_m, slot, cg) + r16), 0, kScDev);
      if constexpr (kSumMfma) {
        if (r16 == 0) {  // Lacc[cg][i]: the sum of row 4kg + i, in every column lane
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(Lacc[cg][i]), rs, off(st_at(a.part_l, slot, cg) + 4 * kg + i), 0,
                kScDev);
        }
      } else {
        const float lrow = sum_over_groups(lsum[cg]);
        if (kg == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lrow), rs,
                                                off(st_at(a.part_l, slot, cg) + r16), 0, kScDev);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores performed
    __syncthreads();
    if (tid == 0) {
      uint32_t* const cnt = a.counters + (size_t)kPrefillCounterStride * cut_ord;
      const unsigned prev =
          __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = prev + 1 == (unsigned)nch;
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_pick = last ? 1 : 0;
    }
    __syncthreads();
    if (!s_pick) return;
    const int slot0 = slot - kchunk;
    auto ld4 = [&](const float* p) {
      return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off(p), 0, kScDev));
    };
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      f32x4 M = {kNegInf, kNegInf, kNegInf, kNegInf};
      for (int k = 0; k < nch; ++k) {
        const f32x4 mk = ld4(st_at(a.part_m, slot0 + k, cg) + 4 * kg);  // rows 4kg .. 4kg+3
#pragma unroll
        for (int i = 0; i < 4; ++i) M[i] = fmaxf(M[i], mk[i]);
      }
      f32x4 den = {0.f, 0.f, 0.f, 0.f};
      f32x4 acc[JD];
#pragma unroll
      for (int jd = 0; jd < JD; ++jd) acc[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < nch; ++k) {
        const f32x4 mk = ld4(st_at(a.part_m, slot0 + k, cg) + 4 * kg);
        const f32x4 lk = ld4(st_at(a.part_l, slot0 + k, cg) + 4 * kg);
        f32x4 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = exp2_fast(mk[i] - M[i]);  // 0 for a row that saw no key of chunk k
          den[i] += f[i] * lk[i];
        }
#pragma unroll
        for (int jd = 0; jd < JD; ++jd) {
          const f32x4 o = ld4(o_at(slot0 + k, cg, jd));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[jd][i] += f[i] * o[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * CG * w + 16 * cg + 4 * kg + i;
        const int pos = p0 + row / G;
        if (pos >= L) continue;
        const int hq = g * G + row % G;
        const float inv = 1.f / den[i];
        uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)(r0 + pos) * a.Hq + hq) * D;
#pragma unroll
        for (int jd = 0; jd < JD; jd += 2) {
          const uint32_t two = pack2<kBF>(acc[jd][i] * inv, acc[jd + 1][i] * inv);
          orow[16 * jd + r16] = (uint16_t)two;
          orow[16 * (jd + 1) + r16] = (uint16_t)(two >> 16);
        }
      }
    }
    return;
  }

  // ---- normalise and store: lane (r16, kg) holds rows 4kg+i, head-dim 16 jd + r16 ----
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const float lrow = kSumMfma ? 0.f : sum_over_groups(lsum[cg]);  // row r16's sum
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = kSumMfma ? Lacc[cg][i] : __shfl(lrow, 4 * kg + i);
      const int row = 16 * CG * w + 16 * cg + 4 * kg + i;
      const int pos = p0 + row / G;
      if (pos >= L) continue;
      const int hq = g * G + row % G;
      const float inv = 1.f / li;
      uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)(r0 + pos) * a.Hq + hq) * D;
#pragma unroll
      for (int jd = 0; jd < JD; jd += 2) {
        const uint32_t two = pack2<kBF>(O[cg][jd][i] * inv, O[cg][jd + 1][i] * inv);
        orow[16 * jd + r16] = (uint16_t)two;
        orow[16 * (jd + 1) + r16] = (uint16_t)(two >> 16);
      }
    }
  }
}

template <int DT, int D, int kSched, bool kPrec>
hipError_t launch_gg(int G, const dim3& grid, const PrefillArgs& a, hipStream_t st, hipEvent_t e0,
                     hipEvent_t e1) {
  const dim3 block(kThreads);
  switch (G) {
    case 1: hipExtLaunchKernelGGL((prefill_kernel<DT, 1, D, kSched, kPrec>), grid, block, 0, st, e0, e1, 0, a); break;
    case 2: hipExtLaunchKernelGGL((prefill_kernel<DT, 2, D, kSched, kPrec>), grid, block, 0, st, e0, e1, 0, a); break;
    case 4: hipExtLaunchKernelGGL((prefill_kernel<DT, 4, D, kSched, kPrec>), grid, block, 0, st, e0, e1, 0, a); break;
    case 8: hipExtLaunchKernelGGL((prefill_kernel<DT, 8, D, kSched, kPrec>), grid, block, 0, st, e0, e1, 0, a); break;
    case 16: hipExtLaunchKernelGGL((prefill_kernel<DT, 16, D, kSched, kPrec>), grid, block, 0, st, e0, e1, 0, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Non-planned grid (position blocks, Hkv, S): most keys first with several sequences.
template <int DT, int D, bool kPrec>
hipError_t launch_grid(int G, const PrefillArgs& a, int num_seqs, int max_query_len,
                       hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int per = Shape<D>::ROWS / G;
  const dim3 grid((unsigned)((max_query_len + per - 1) / per), (unsigned)a.Hkv, (unsigned)num_seqs);
  PrefillArgs ao = a;
  ao.order_seqs = num_seqs >= 2 && num_seqs <= kOrderMaxSeqs ? num_seqs : 0;
  if (ao.order_seqs > 0) return launch_gg<DT, D, 1, kPrec>(G, grid, ao, st, e0, e1);
  return launch_gg<DT, D, 0, kPrec>(G, grid, ao, st, e0, e1);
}

template <int DT, int D>
hipError_t launch_g(int G, const PrefillArgs& a, int num_seqs, int max_query_len,
                    hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  PrefillArgs ao = a;
  ao.flag_check = 0;
  if (a.precise) return launch_grid<DT, D, true>(G, ao, num_seqs, max_query_len, st, e0, e1);
  // The one-part form; for bf16 the two-part recompute launch follows and ends the call.
  hipEvent_t last = DT == PA_BF16 ? nullptr : e1;
  hipError_t err;
  if (a.plan) {
    ao.order_seqs = num_seqs;
    const int per = Shape<D>::ROWS / G;
    hipExtLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(512), 0, st, e0, nullptr, 0, ao,
                          num_seqs, per);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = launch_gg<DT, D, 2, false>(G, dim3((unsigned)a.item_bound), ao, st, nullptr, last);
    if (err != hipSuccess) return err;
  } else {
    err = launch_grid<DT, D, false>(G, ao, num_seqs, max_query_len, st, e0, last);
    if (err != hipSuccess) return err;
  }
  if constexpr (DT == PA_BF16) {
    // Runs only if the first launch marked this call's overflow word.
    ao.flag_check = 1;
    return launch_grid<DT, D, true>(G, ao, num_seqs, max_query_len, st, nullptr, e1);
  }
  return hipSuccess;
}

// Overflow words of the one-part bf16 form: call e (a number the host draws from a
// 32-bit counter, never 0) owns word e % kPrefillFlagSlots and marks an overflow by
// storing e there; the recompute launch of the same call compares the word with e.  A
// word that still holds e from an earlier run of the same launches (a replayed graph)
// only makes the recompute run when it was not needed.  A call's overflow can be missed
// only if kPrefillFlagSlots later calls on the same device are issued while it is still
// in flight.  In host code `prefill_flag_words` names a host-side stand-in: the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint32_t prefill_flag_words[kPrefillFlagSlots];

}  // namespace

namespace {
constexpr int kFlagDevices = 64;
std::mutex g_flag_mutex;
uint32_t* g_flag_ptr[kFlagDevices] = {};
std::atomic<uint32_t> g_epoch{0};
}  // namespace

hipError_t prefill_overflow_flags(uint32_t** words, uint32_t* epoch) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kFlagDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(g_flag_mutex);
    if (!g_flag_ptr[dev]) {
      void* p = nullptr;
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(prefill_flag_words));
      if (err != hipSuccess) return err;
      if (!p) return hipErrorInvalidSymbol;
      g_flag_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *words = g_flag_ptr[dev];
  }
  uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  if (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  *epoch = e;
  return hipSuccess;
}

size_t prefill_plan_bytes(int head_dim, int group, int num_seqs, PrefillArgs& a) {
  a.item_bound = a.slot_bound = a.cut_bound = 0;
  if (a.precise || a.chunk == 0 || num_seqs < 1 || num_seqs > kOrderMaxSeqs) return 0;
  if ((head_dim != 128 && head_dim != 256) || group < 1) return 0;
  const long long rows = prefill_rows(head_dim);
  const long long kpos = rows / group;
  const long long S = num_seqs, T = a.T, maxq = a.max_query_len;
  // Row blocks (position blocks of every sequence, times KV heads): sum_b ceil(L_b / kpos)
  // with sum_b L_b <= T and every L_b counted up to max_query_len.
  const long long R =
      std::min((T + kpos - 1) / kpos + S, S * ((maxq + kpos - 1) / kpos)) * a.Hkv;
  const long long tmax = ((long long)a.MB * kBlockSize + maxq + kTile - 1) / kTile;
  const long long cmin = a.chunk > 0 ? a.chunk : kPrefillAutoMinChunk;
  const long long per_rb = (tmax + cmin - 1) / cmin;  // chunks of one row block, at most
  // Automatic chunks and no row block long enough to be cut (at most 16 tiles, a small
  // call): the grid schedule, without the plan kernel's latency.
  if (a.chunk < 0 && per_rb <= 1) return 0;
  const long long N = std::max(a.ncu, 1);
  // Automatic chunks: W / C <= 0.8N, so items <= 0.8N + R, chunks of cut row blocks
  // <= 1.6N, cut row blocks <= 0.8N (the bounds below keep 3N and 6N).  A plan beyond
  // these is dropped on the device for the uncut one.
  long long slots = per_rb > 1 ? R * per_rb : 0, merges = per_rb > 1 ? R : 0;
  if (a.chunk < 0) {
    slots = std::min(slots, 6 * N);
    merges = std::min(merges, 3 * N);
  }
  constexpr long long kMaxSlots = 4096;  // about 0.5 GB of partial states
  static_assert(kItemWords == 16, "item entries of 64 bytes");
  constexpr long long kMaxCut = (long long)(kFusedCounterBytes / (4 * kPrefillCounterStride));
  slots = std::min(slots, kMaxSlots);
  merges = std::min(std::min(merges, slots / 2), kMaxCut);  // one arrival counter each
  long long items = R + slots;
  if (a.chunk < 0) items = std::min(items, 3 * N + R);
  if (items > (1ll << 30)) return 0;
  a.item_bound = (int32_t)items;
  a.slot_bound = (int32_t)slots;
  a.cut_bound = (int32_t)merges;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return prefill_plan_words_bytes(a.item_bound) + al((size_t)slots * rows * head_dim * 4) +
         2 * al((size_t)slots * rows * 4);
}

hipError_t launch_prefill(int dtype, int group, int head_dim, const PrefillArgs& args,
                          int num_seqs, int max_query_len, hipStream_t stream, hipEvent_t e0,
                          hipEvent_t e1) {
  PrefillArgs a = args;
  const hipError_t err = prefill_overflow_flags(&a.flags, &a.epoch);  // valid in every launch
  if (err != hipSuccess) return err;
  if (head_dim == 128)
    return dtype == PA_BF16 ? launch_g<PA_BF16, 128>(group, a, num_seqs, max_query_len, stream, e0, e1)
         : dtype == PA_F16  ? launch_g<PA_F16, 128>(group, a, num_seqs, max_query_len, stream, e0, e1)
                            : hipErrorInvalidValue;
  if (head_dim == 256)
    return dtype == PA_BF16 ? launch_g<PA_BF16, 256>(group, a, num_seqs, max_query_len, stream, e0, e1)
         : dtype == PA_F16  ? launch_g<PA_F16, 256>(group, a, num_seqs, max_query_len, stream, e0, e1)
                            : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace pa
