// Paged prefix-prefill attention for gfx950 (MI355X).
//
// Source: project_6 optimizations/prefix_prefill_patch.py (commit fee8f1b), docstring:
// the prefix_prefill kernel is Flash-Attention style -- a grid of (batch, heads,
// query tiles of BLOCK_M positions), K/V tiles of BLOCK_N tokens staged in on-chip
// memory, fp16/bf16, head_dim 128, GQA.  What it computes (the reading stated with the
// oracle): new token i of sequence b (absolute position c_b + i) attends to the c_b
// prefix tokens in the paged cache and to new tokens 0..i, whose K/V arrive packed.
//
// Work-group: 4 waves, 256 query rows of one KV head g of one sequence: positions
// [p0, p0 + 256/G) x the G query heads of g, row r = (position p0 + r / G, head
// g*G + r % G).  Sharing every K/V tile among the G heads and 256/G positions is what
// makes the tile traffic small next to the MFMA work.  Wave w owns rows 64w..64w+63,
// as four column groups of 16 rows (the MFMA's 16 columns).
//
// Per 64-key tile: K and V rows are loaded from the cache (key < c, through the
// block table) or from the packed new tokens (c <= key < c + L), into LDS rows of
// 256 bytes whose 16-byte chunks are XOR-swizzled with the row index, so that both
// operand reads below hit 16 distinct chunk positions per 16 lanes.
//   S^T = K Q^T:   v_mfma_f32_16x16x32, A = 16 keys x 32 dims (LDS), B = Q (registers):
//                  lane (r16, kg) gets keys 4kg..4kg+3 of query row r16.
//   online softmax per query row in base 2 (scale * log2 e folded in), causal mask on
//                  the tiles that reach the row's own position, lazy rescale as in decode.
//   O += P V:      v_mfma_f32_16x16x32 over 32 keys = two 16-key row blocks: the S^T
//                  accumulators of the two blocks are exactly the A operand (k-slot e of
//                  lane group kg is key 16(2s + e/4) + 4kg + e%4), and the B operand
//                  takes column j of the 16-byte V runs of those 8 keys (v_perm pairs),
//                  so instruction j produces head-dim indices 8n + j.
// The next tile's global loads are issued before the current tile's math.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>


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
constexpr int kD = 128;          // head_dim built
constexpr int kRows = 256;       // query rows per work-group
constexpr int kTile = 64;        // keys per K/V tile
constexpr int kChunks = kD / 8;  // 16-byte chunks per row

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

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups of one MFMA column),
// with the two gfx950 half-swaps (upper 32 lanes with lower 32, odd 16-lane rows with
// even ones).  The swapped pair is passed through an empty asm: without it the compiler
// (ROCm 7.2) emitted the float max of the two results with the same register twice.
__device__ __forceinline__ float max_over_groups(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t a0 = a[0], a1 = a[1];
  asm("" : "+v"(a0), "+v"(a1));
  u = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1)));
  const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  uint32_t b0 = b[0], b1 = b[1];
  asm("" : "+v"(b0), "+v"(b1));
  return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
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

// LDS slot (in 16-byte units) of chunk `c` of tile row `r`.
__device__ __forceinline__ int swz(int r, int c) { return r * kChunks + (c ^ (r & 15)); }

template <int DT, int G>
__global__ void __launch_bounds__(256, 1) prefill_kernel(const PrefillArgs a) {
  constexpr bool kBF = DT == PA_BF16;
  constexpr int kPos = kRows / G;  // query positions per work-group
  __shared__ u32x4 s_k[kTile * kChunks];
  __shared__ u32x4 s_v[kTile * kChunks];

  const int g = blockIdx.y, b = blockIdx.z;
  const int p0 = blockIdx.x * kPos;
  int r1 = a.query_start[b + 1], r0 = a.query_start[b];
  r1 = min(r1, a.T);
  r0 = min(max(r0, 0), r1);
  const int L = r1 - r0;
  if (p0 >= L) return;
  int c = a.ctx[b];
  const int cap = a.MB * kBlockSize;
  c = c < 0 ? 0 : (c > cap ? cap : c);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;

  // Keys this work-group needs: the prefix and new tokens up to its last position.
  const int pend = min(L, p0 + kPos);
  const int nkeys = c + pend;
  const int ntiles = (nkeys + kTile - 1) / kTile;

  // ---- query operands and per-row state ----
  // Column group cg of this wave: rows 64w + 16cg + (0..15); lane column r16.
  u32x4 qf[4][4];  // [cg][kk]: Q[row r16][32kk + 8kg .. +7]
  int qpos_col[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const int row = 64 * w + 16 * cg + r16;
    const int pos = p0 + row / G;
    const int hq = g * G + row % G;
    qpos_col[cg] = pos;
    const bool valid = pos < L;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((size_t)(r0 + (valid ? pos : 0)) * a.Hq + hq) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[cg][kk] = valid ? *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * kg)
                         : u32x4{0u, 0u, 0u, 0u};
  }
  // The softmax works on raw dot products scaled by |scale| log2(e); a negative scale is
  // carried by flipping the sign of q (exact in 16-bit floats), so max(scale * s) is
  // |scale| * max of the flipped products.
  const float sl = fabsf(a.scale_log2);
  if (a.scale_log2 < 0.f) {
    const uint32_t flip = 0x80008000u;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[cg][kk] ^= u32x4{flip, flip, flip, flip};
  }
  // Register classes, pinned with empty asm constraints: the output and score
  // accumulators live in VGPRs (the softmax and the rare rescale work on them there),
  // while MFMA input operands (queries, K rows) and the staged tile loads live in AGPRs.
  // Left to itself the compiler kept the output accumulators in AGPRs and copied all
  // 128 of them to VGPRs and back on every tile.
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) asm("" : "+a"(qf[cg][kk]));
  f32x4 O[4][8];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int j = 0; j < 8; ++j) O[cg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums of P come from the matrix cores too: one more PV product per column group
  // with an all-ones B operand leaves sum_k P[row][k] in every column, in the same
  // row layout as O (and from the same bf16-rounded P as O).
  f32x4 Lacc[4];
  float m_ref[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    m_ref[cg] = kNegInf;
    Lacc[cg] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = kBF ? 0x3F803F80u : 0x3C003C00u;  // two 16-bit 1.0
  const u32x4 ones = {one2, one2, one2, one2};

  // ---- tile loads: thread tid moves 64 bytes (4 chunks) of K and of V of tile row tid/4 ----
  // Loads are unconditional (a row outside the keys reads a valid dummy row and is
  // zeroed when written to LDS), so no branch or wait sits between them.  The block id
  // of a prefix row is read two tiles ahead, behind the K/V loads of the next tile:
  // consuming it never drains loads that are still useful in flight.
  const int lrow = tid >> 2, lc0 = (tid & 3) * 4;
  const size_t hstride = (size_t)kBlockSize * kD;  // elements per (block, head)
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + (size_t)g * hstride;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + (size_t)g * hstride;
  const uint16_t* knew = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vnew = static_cast<const uint16_t*>(a.v_new);
  const size_t bstride = (size_t)a.Hkv * hstride;
  const int32_t* btrow = a.bt + (size_t)b * a.MB;
  const int cmax = c > 0 ? c - 1 : 0;
  auto fetch_block = [&](int t) {  // block id of this thread's row of tile t (any if not prefix)
    return btrow[min(t * kTile + lrow, cmax) / kBlockSize];
  };
  u32x4 kr[4], vr[4];
  bool row_ok = false;
  auto load_tile = [&](int t, int blk) {
    const int key = t * kTile + lrow;
    const bool pre = key < c && (unsigned)blk < (unsigned)a.NB;
    const bool fresh = key >= c && key < nkeys;
    row_ok = pre || fresh;
    const size_t off = pre ? (size_t)blk * bstride + (size_t)(key % kBlockSize) * kD
                           : (fresh ? ((size_t)(r0 + key - c) * a.Hkv + g) * kD : (size_t)r0 * a.Hkv * kD);
    const uint16_t* ks = (pre ? kc : knew) + off;
    const uint16_t* vs = (pre ? vc : vnew) + off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = *reinterpret_cast<const u32x4*>(ks + 8 * (lc0 + i));
      vr[i] = *reinterpret_cast<const u32x4*>(vs + 8 * (lc0 + i));
    }
  };

  int blk_next = fetch_block(1);
  load_tile(0, fetch_block(0));
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // the previous tile's LDS reads are done
    if (__all(row_ok)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_k[swz(lrow, lc0 + i)] = kr[i];
        s_v[swz(lrow, lc0 + i)] = vr[i];
      }
    } else {  // tail tile, or a prefix row with an out-of-range block id
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_k[swz(lrow, lc0 + i)] = row_ok ? kr[i] : z;
        s_v[swz(lrow, lc0 + i)] = row_ok ? vr[i] : z;
      }
    }
    __syncthreads();
    if (t + 1 < ntiles) {  // in flight during this tile's math
      load_tile(t + 1, blk_next);
      blk_next = fetch_block(t + 2);
    }

    // Per tile, the four column groups run as two independent pairs so that the matrix
    // cores and the VALU overlap: the exponentials of pair 0 are interleaved with the
    // QK^T products of pair 1, and the PV products of pair 0 with the exponentials of
    // pair 1 (scheduling groups).  Each pair takes one row max over the whole 64-key tile
    // and one rescale decision.
    const int kbase = t * kTile;
    const bool diag = kbase + kTile - 1 > c + p0;  // some key of the tile may lie after some row
    u32x4 ka[4][4];  // [row block][k step]: the tile's K operands, shared by both pairs
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        ka[rb][kk] = s_k[swz(16 * rb + r16, 4 * kk + kg)];
        asm("" : "+a"(ka[rb][kk]));
      }
    auto qk = [&](int pr, f32x4 (&S)[4][2]) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          S[rb][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            S[rb][q] = mfma32<kBF>(ka[rb][kk], qf[2 * pr + q][kk], S[rb][q]);
        }
    };
    // Row max over the tile and the rescale for pair pr; masked keys become -inf on
    // diagonal tiles, where S then holds scaled logits (exp2 of -inf - m is 0).
    auto pair_max = [&](int pr, f32x4 (&S)[4][2]) {
      float bm[2];
      bool grow = false;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int cg = 2 * pr + q;
        float mx = kNegInf;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (diag) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kbase + 16 * rb + 4 * kg + i;
              const bool vis = key <= c + qpos_col[cg] && key < nkeys;
              S[rb][q][i] = vis ? S[rb][q][i] * sl : kNegInf;
            }
          }
          mx = fmaxf(mx, fmaxf(fmaxf(S[rb][q][0], S[rb][q][1]), fmaxf(S[rb][q][2], S[rb][q][3])));
        }
        mx = max_over_groups(mx);
        bm[q] = diag ? mx : mx * sl;
        grow = grow || bm[q] > m_ref[cg] + kRescaleSlack;
      }
      if (__any(grow)) {  // rare
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int cg = 2 * pr + q;
          const float m_new = fmaxf(m_ref[cg], bm[q]);
          const float alpha = m_ref[cg] == kNegInf ? 0.f : exp2_fast(m_ref[cg] - m_new);
          m_ref[cg] = m_new;
          float al[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kg + i);
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[cg][j][i] *= al[i];
#pragma unroll
          for (int i = 0; i < 4; ++i) Lacc[cg][i] *= al[i];
        }
      }
    };
    // m_ref is finite here: key 0 is visible to every row and lies in tile 0.
    const float fs = diag ? 1.f : sl;  // diagonal tiles hold scaled logits already
    // P of pair pr as PV A operands: Pa[q][s] covers keys of row blocks 2s, 2s+1.
    auto probs = [&](int pr, const f32x4 (&S)[4][2], u32x4 (&Pa)[2][2]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float nm = -m_ref[2 * pr + q];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float p[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[h][i] = exp2_fast(fmaf(S[2 * st + h][q][i], fs, nm));
          Pa[q][st] = u32x4{pack2<kBF>(p[0][0], p[0][1]), pack2<kBF>(p[0][2], p[0][3]),
                            pack2<kBF>(p[1][0], p[1][1]), pack2<kBF>(p[1][2], p[1][3])};
        }
      }
    };
    // V operands of the tile: vb[st][jd] = B of the 32 keys of step st (in the P k-slot
    // order) x head-dim 16 jd + (0..15).  Lane (j, kg) reads 8 bytes of key
    // 32 st + 4 kg + j / 4 (+16 for the second read), head-dim 16 jd + 4 (j % 4), and the
    // transposing read hands lane (n, kg) the 4 keys of its k-slots at head-dim 16 jd + n.
    u32x4 vb[2][8];
    auto load_v = [&]() {
      const char* vbase = reinterpret_cast<const char*>(s_v);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) {
          const int key = 32 * st + 4 * kg + (r16 >> 2);
          const int c = 2 * jd + ((r16 & 3) >> 1), half = r16 & 1;
          const u32x2 lo = lds_read_tr(vbase + swz(key, c) * 16 + half * 8);
          const u32x2 hi = lds_read_tr(vbase + swz(key + 16, c) * 16 + half * 8);
          vb[st][jd] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          asm("" : "+a"(vb[st][jd]));
        }
    };
    auto pv = [&](int pr, const u32x4 (&Pa)[2][2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int jd = 0; jd < 8; ++jd)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            O[2 * pr + q][jd] = mfma32<kBF>(Pa[q][st], vb[st][jd], O[2 * pr + q][jd]);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          Lacc[2 * pr + q] = mfma32<kBF>(Pa[q][st], ones, Lacc[2 * pr + q]);
      }
    };

    f32x4 S0[4][2], S1[4][2];
    u32x4 P0[2][2], P1[2][2];
    qk(0, S0);
    pair_max(0, S0);
    probs(0, S0, P0);
    qk(1, S1);
    // pair 1's 32 QK^T products against pair 0's exponentials and packing
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    load_v();
    pair_max(1, S1);
    pv(0, P0);
    probs(1, S1, P1);
    // pair 0's 36 PV products against pair 1's exponentials and the V operand shuffles
#pragma unroll
    for (int k = 0; k < 36; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);
    }
    pv(1, P1);
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm("" : "+v"(O[cg][j]));
  }

  // ---- normalise and store: lane (r16, kg) holds rows 4kg+i, head-dim 16 jd + r16 ----
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = Lacc[cg][i];
      const int row = 64 * w + 16 * cg + 4 * kg + i;
      const int pos = p0 + row / G;
      if (pos >= L) continue;
      const int hq = g * G + row % G;
      const float inv = 1.f / li;
      uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)(r0 + pos) * a.Hq + hq) * kD;
#pragma unroll
      for (int jd = 0; jd < 8; jd += 2) {
        const uint32_t two = pack2<kBF>(O[cg][jd][i] * inv, O[cg][jd + 1][i] * inv);
        orow[16 * jd + r16] = (uint16_t)two;
        orow[16 * (jd + 1) + r16] = (uint16_t)(two >> 16);
      }
    }
  }
}

template <int DT>
hipError_t launch_g(int G, const PrefillArgs& a, dim3 grid, hipStream_t st, hipEvent_t e0,
                    hipEvent_t e1) {
  const dim3 block(256);
  switch (G) {
    case 1: hipExtLaunchKernelGGL((prefill_kernel<DT, 1>), grid, block, 0, st, e0, e1, 0, a); break;
    case 2: hipExtLaunchKernelGGL((prefill_kernel<DT, 2>), grid, block, 0, st, e0, e1, 0, a); break;
    case 4: hipExtLaunchKernelGGL((prefill_kernel<DT, 4>), grid, block, 0, st, e0, e1, 0, a); break;
    case 8: hipExtLaunchKernelGGL((prefill_kernel<DT, 8>), grid, block, 0, st, e0, e1, 0, a); break;
    case 16: hipExtLaunchKernelGGL((prefill_kernel<DT, 16>), grid, block, 0, st, e0, e1, 0, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int prefill_positions_per_workgroup(int group) { return kRows / group; }

hipError_t launch_prefill(int dtype, int group, const PrefillArgs& a, int num_seqs,
                          int max_query_len, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int per = kRows / group;
  const dim3 grid((unsigned)((max_query_len + per - 1) / per), (unsigned)a.Hkv, (unsigned)num_seqs);
  return dtype == PA_BF16 ? launch_g<PA_BF16>(group, a, grid, stream, e0, e1)
       : dtype == PA_F16  ? launch_g<PA_F16>(group, a, grid, stream, e0, e1)
                          : hipErrorInvalidValue;
}

}  // namespace pa
