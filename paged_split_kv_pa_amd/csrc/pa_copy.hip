// KV-cache block copy for prefix caching (copy-on-write of shared blocks).
//
// Source: project_6_baseline5 GROUND_TRUTH_STATUS_v2.md, section "路径 3": prefix
// caching is on and its cache copy kernel is named as not optimised.  What it
// computes is read as: for every (src, dst) pair of block ids, block dst of the K
// pool and of the V pool becomes a bitwise copy of block src.
//
// A block of one pool is `block_bytes` contiguous bytes (Hkv x 16 x D elements in
// the [num_blocks, Hkv, 16, D] layout).  Work-group (chunk c of pair i, pool z)
// moves bytes [16 KiB c, 16 KiB (c+1)) of that block: 256 threads x 4 x 16 bytes,
// all four loads issued before the stores.  Both sides go through buffer
// resources bounded to the block, so the last, shorter chunk needs no branches:
// loads past the end return 0 and stores past the end are dropped.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyVec = 4;  // 16-byte accesses per thread

__device__ __forceinline__ __amdgpu_buffer_rsrc_t copy_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__global__ void __launch_bounds__(kCopyThreads) copy_blocks_kernel(const CopyArgs a) {
  // The host keeps num_pairs * chunks below 2^31: 32-bit unsigned arithmetic.
  const unsigned wg = blockIdx.x;
  const unsigned pair = wg / (unsigned)a.chunks;
  const int chunk = (int)(wg - pair * (unsigned)a.chunks);
  const int src = a.pairs[2 * (size_t)pair], dst = a.pairs[2 * (size_t)pair + 1];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks) return;
  unsigned char* pool = static_cast<unsigned char*>(blockIdx.y == 0 ? a.k : a.v);
  const __amdgpu_buffer_rsrc_t rs = copy_rsrc(pool + (size_t)src * a.block_bytes, a.block_bytes);
  const __amdgpu_buffer_rsrc_t rd = copy_rsrc(pool + (size_t)dst * a.block_bytes, a.block_bytes);
  const int off0 = chunk * (kCopyThreads * kCopyVec * 16) + threadIdx.x * 16;
  u32x4 r[kCopyVec];
#pragma unroll
  for (int j = 0; j < kCopyVec; ++j)
    r[j] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + j * kCopyThreads * 16, 0, 2));
#pragma unroll
  for (int j = 0; j < kCopyVec; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(r[j], rd, off0 + j * kCopyThreads * 16, 0, 2);
}

}  // namespace

int copy_chunk_bytes() { return kCopyThreads * kCopyVec * 16; }

hipError_t launch_copy_blocks(const CopyArgs& a, long long num_pairs, bool with_v,
                              hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const long long wgs = num_pairs * a.chunks;
  const dim3 grid((unsigned)wgs, with_v ? 2 : 1, 1);
  hipExtLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, e0, e1, 0, a);
  return hipGetLastError();
}

}  // namespace pa
