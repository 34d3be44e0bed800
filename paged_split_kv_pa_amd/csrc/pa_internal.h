// Internal interface between the C-ABI front end (pa_api.hip) and the
// kernels (pa_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;   // tokens per KV-cache block
constexpr int kWaves = 4;        // waves per attention work-group
constexpr int kMaxReducePartitions = 8192;  // partition-grid limit per sequence
constexpr int kMaxPieceShift = 4;           // a split item has at most 16 pieces
constexpr int kMaxPieceSlots = 1024;        // piece partials the workspace holds
constexpr int64_t kMaxSplitGrid = 1 << 24;  // linear (split) grids stay below this

// Work split for load balance.  Grid items are (partition p, KV head g, sequence b)
// with linear index p + Pmax * (g + Hkv * b), the order in which work-groups are
// dispatched.  Items from split_first on are each cut into 2^split_shift pieces of
// P >> split_shift tokens, one work-group per piece, on a one-dimensional grid of
// split_first + (items - split_first) << split_shift work-groups.  A piece writes its
// (max, exp-sum, normalised output) per query head to slot (work-group index -
// split_first) of the piece area; phase 2 folds a split partition's pieces in place
// of its row of the partials.  split_shift == 0: no split, grid (Pmax, Hkv, S).
struct Split {
  int32_t first = 0;
  int32_t shift = 0;
  float* piece_out = nullptr;   // [slots][G][D]
  float* piece_max = nullptr;   // [slots][G], natural-log units like max_logits
  float* piece_sum = nullptr;   // [slots][G]
};

// Arguments of the attention kernel (phase 1 and V1 share it).  Strides are in elements
// (block-table entries for bt_ss); all are validated on the host.
struct AttnArgs {
  void* out;                 // [S, Hq, D] element type of q, strides (o_ss, o_sh, 1)
  const void* q;             // [S, Hq, D], strides (q_ss, q_sh, 1)
  const void* k;             // [NB, Hkv, 16, D], block stride kv_sb, dense within a block
  const void* v;             // [NB, Hkv, 16, D], block stride kv_sb
  const int32_t* bt;         // [S, MB], row stride bt_ss
  const int32_t* ctx;        // [S]
  int32_t q_ss, q_sh, bt_ss;
  int64_t o_ss, o_sh, kv_sb;
  float* tmp_out;            // [S, Hq, Pmax, D] (unused when Pmax == 1)
  float* max_logits;         // [S, Hq, Pmax]
  float* exp_sums;           // [S, Hq, Pmax]
  float scale_log2;          // scale * log2(e)
  int32_t Hq, Hkv, NB, MB;
  int32_t P;                 // tokens per partition (multiple of 16)
  int32_t Pmax;              // partition-grid size
  Split split;
  // > 0 (no split): the number of sequences S, and work-groups do not take their item
  // from the grid position.  V1 (Pmax == 1, four-wave matrix-core shape): work-group z
  // takes the sequence of rank z in longest-context-first order.  V2 (both kernels):
  // work-group j takes the j-th non-empty (sequence, KV head, partition) item (see
  // compact_item).
  int32_t order_seqs = 0;
  // Single-launch V2 (see fused_merge): grid (n1, 2); row 0 runs the phase-1 items on
  // a linear index, row 1 the merge work-groups, fused_m of them (one per sequence,
  // query head and kFusedChunks-th of the head dim).  counters: the arrival counter of
  // each (sequence, KV head), then the go flag of each merge work-group (see arrive);
  // all zero before the launch and zero again after it.
  int32_t fused = 0;
  int32_t fused_m = 0;
  uint32_t* counters = nullptr;
};
constexpr int kFusedChunks = 8;              // merge work-groups per query head
// Arrival counter of (sequence, KV head) i at word kFusedCounterStride * i; go flag of
// merge work-group m at word kFusedFlagBase + kFusedFlagStride * m.  Every counter and
// flag has a line of its own.
constexpr int kFusedCounterStride = 64;      // uint32 words (256 bytes)
constexpr int kFusedMaxGroups = 256;         // (sequence, KV head) pairs
constexpr int kFusedFlagBase = kFusedCounterStride * kFusedMaxGroups;
constexpr int kFusedFlagStride = 16;         // uint32 words (64 bytes)
constexpr int kFusedMaxMerge = 4096;         // merge work-groups
constexpr size_t kFusedCounterBytes =
    4 * ((size_t)kFusedFlagBase + (size_t)kFusedFlagStride * kFusedMaxMerge);  // 320 KiB
constexpr int kFusedMaxFold = 4096;          // partial states per head a merge holds in LDS
constexpr int kOrderMaxSeqs = 512;  // longest-first orders (V1, prefill): at most this many sequences

// Arguments of the phase-2 (cross-partition) kernel.
struct ReduceArgs {
  void* out;                 // [S, Hq, D], strides (o_ss, o_sh, 1)
  int64_t o_ss, o_sh;
  const int32_t* ctx;
  const float* tmp_out;
  const float* max_logits;
  const float* exp_sums;
  int32_t Hq, Hkv, MB, P, Pmax;
  Split split;
};

// Work-group shape of the matrix-core kernel (-1 automatic, 0, 1 or 2; see
// pa_kernels.hip).  set_mfma_variant returns -1 for an unknown variant.
int set_mfma_variant(int v);
int get_mfma_variant();

// Kernel family chosen for a (dtype, G) pair.
enum class Kernel { kMfma, kValu };
Kernel kernel_for(int dtype, int group);

// Launch the attention kernel on grid (Pmax, Hkv, S), or on the linear grid of a split
// (see Split).  Returns the launch status.
// ev_start / ev_stop (may be null) are recorded when the kernel starts / ends.
hipError_t launch_attention(int dtype, int head_dim, int group, const AttnArgs& a, int num_seqs,
                            hipStream_t stream, hipEvent_t ev_start = nullptr,
                            hipEvent_t ev_stop = nullptr);
// Zero n uint32 words at p (a fill kernel: graph-capture safe, unlike hipMemsetAsync).
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream);
// Work-groups phase 1 of V2 runs for this launch (grid slots of the item order, or the
// work split's linear grid).
long long phase1_workgroups(const AttnArgs& a, int num_seqs);
// Partial states (partitions plus pieces of cut ones) phase 2 folds per head, at most.
long long fold_states(const AttnArgs& a, int num_seqs);
// Launch the phase-2 kernel on grid (S*Hq, 8), or (S*Hq, 1) for many heads.
hipError_t launch_reduce(int dtype, int head_dim, const ReduceArgs& a, int num_seqs,
                         hipStream_t stream);

// ---- KV block copy (pa_copy.hip) ------------------------------------------------------
struct CopyArgs {
  void* k;                   // K pool: num_blocks blocks of block_bytes bytes
  void* v;                   // V pool (same shape), or null for a K-only copy
  const int32_t* pairs;      // [num_pairs][2] (src, dst) block ids
  int32_t block_bytes;       // bytes of one block of one pool (multiple of 16)
  int32_t num_blocks;
  int32_t chunks;            // work-groups per block: ceil(block_bytes / copy_chunk_bytes())
};
int copy_chunk_bytes();
// Grid (num_pairs * chunks, 1 or 2 pools).
// ev_start / ev_stop (may be null) are recorded when the kernel starts / ends.
hipError_t launch_copy_blocks(const CopyArgs& a, long long num_pairs, bool with_v,
                              hipStream_t stream, hipEvent_t ev_start = nullptr,
                              hipEvent_t ev_stop = nullptr);

// ---- paged prefix prefill (pa_prefill.hip) ---------------------------------------------
struct PrefillArgs {
  void* out;                 // [T, Hq, D]
  const void* q;             // [T, Hq, D]
  const void* k_new;         // [T, Hkv, D]
  const void* v_new;         // [T, Hkv, D]
  const void* k_cache;       // [NB, Hkv, 16, D]
  const void* v_cache;
  const int32_t* bt;         // [S, MB]
  const int32_t* ctx;        // [S] prefix lengths
  const int32_t* query_start;  // [S + 1]
  float scale_log2;          // scale * log2(e)
  int32_t T, Hq, Hkv, NB, MB;
  // > 0: the number of sequences S; work-group z then takes the sequence of rank z in
  // most-keys-first order (prefix plus new tokens), and position blocks run last first.
  int32_t order_seqs = 0;
  // 1: P enters the PV products as a 16-bit high part plus a 16-bit low part (in the
  // input type).  0: as one fp16 part, with V in fp16 too (bf16 V converted when it is
  // written to LDS); for bf16 a second launch then recomputes the call in the two-part
  // form if some V value did not fit fp16 (see prefill_overflow_flags).
  int32_t precise = 0;
  // Set by launch_prefill: the overflow word of this call (flags[epoch % kPrefillFlagSlots]
  // == epoch after an overflow) and, in the recompute launch, flag_check = 1.
  uint32_t* flags = nullptr;
  uint32_t epoch = 0;
  int32_t flag_check = 0;
  // Planned schedule (see prefill_plan_kernel; one-part form, 1..kOrderMaxSeqs sequences):
  // the item list and the partial states of cut row blocks in a workspace (below
  // 2 GiB: addressed by 32-bit offsets from plan), the bounds the host sized them for,
  // the compute-unit count and the chunk setting (-1 automatic, >= kPrefillMinChunk a
  // fixed chunk length in 64-key tiles; 0: no planned schedule).
  int32_t* plan = nullptr;
  // Arrival counters of cut row blocks (word 16 m for the m-th one): zero before the
  // launch and again after it (the library-owned workspace's zeroed counter region).
  uint32_t* counters = nullptr;
  float* part_o = nullptr;   // [slot][8 waves][CG][JD][64 lanes] f32x4
  float* part_m = nullptr;   // [slot][8 waves][CG][16 rows]
  float* part_l = nullptr;   // [slot][8 waves][CG][16 rows]
  int32_t max_query_len = 0;
  int32_t ncu = 0;
  int32_t chunk = 0;
  int32_t item_bound = 0, slot_bound = 0;
  int32_t cut_bound = 0;     // cut (row block, KV head) pairs, each with an arrival counter
};
constexpr int kPrefillFlagSlots = 1024;
constexpr int kPrefillMinChunk = 4;       // tiles; a chunk then spans at least 2 tiles
constexpr int kPrefillAutoMinChunk = 16;  // tiles; the automatic chunk length's floor
// Bytes of the plan (a header of 8 words and 16 words per item), 256-byte aligned.
constexpr size_t prefill_plan_words_bytes(long long items) {
  return ((size_t)4 * (8 + 16 * (size_t)items) + 255) & ~(size_t)255;
}
constexpr int kPrefillCounterStride = 16;  // words: one 64-byte line per counter
// Query rows (position, head) of one prefill work-group.
constexpr int prefill_rows(int head_dim) { return head_dim == 128 ? 256 : 128; }
// Grid (ceil(max_query_len / positions per work-group), Hkv, S); head_dim 128 or 256,
// fp16/bf16.  e0 / e1 (may be null) are recorded when the first kernel starts / the last
// one ends (bf16 one-part form: the prefill kernel, then the recompute launch).
hipError_t launch_prefill(int dtype, int group, int head_dim, const PrefillArgs& a, int num_seqs,
                          int max_query_len, hipStream_t stream, hipEvent_t e0, hipEvent_t e1);
// The current device's overflow words (kPrefillFlagSlots of them, in static device memory)
// and a fresh call number (never 0) for the one-part bf16 prefill.
hipError_t prefill_overflow_flags(uint32_t** words, uint32_t* epoch);
// Whether a prefill launch takes the planned schedule, and the workspace bytes it needs
// (0 if it does not); fills the bounds in a (item_bound, slot_bound, cut_bound).
size_t prefill_plan_bytes(int head_dim, int group, int num_seqs, PrefillArgs& a);

}  // namespace pa
