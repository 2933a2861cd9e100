// Snapshot / restore of whole per-sequence states between the live state and
// a slot pool ("Kimi K3: From Day-0 Availability to Optimized Inference",
// paragraph on prefix caching: the recurrent-state checkpoint sits at the
// token boundary shared with the attention cache, so its position travels
// with it).  A bitwise, bandwidth-bound copy: 16-byte loads and stores, a
// grid of (blocks per sequence) x (pairs in this launch).

#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// The copies stream (each byte is read and written once per call), so the
// loads and stores carry the non-temporal hint.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kCopyThreads)
    copy_states_kernel(const f32x4* __restrict__ src, const int64_t* __restrict__ src_pos, f32x4* __restrict__ dst,
                       int64_t* __restrict__ dst_pos, size_t n_vec, CopyPairs pairs) {
  const int pair = blockIdx.y;
  const size_t s = (size_t)pairs.src[pair], d = (size_t)pairs.dst[pair];
  const f32x4* sp = src + s * n_vec;
  f32x4* dp = dst + d * n_vec;
  const size_t stride = (size_t)gridDim.x * kCopyThreads;
  size_t i = (size_t)blockIdx.x * kCopyThreads + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * stride < n_vec; i += kCopyUnroll * stride) {
    f32x4 x[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) x[u] = __builtin_nontemporal_load(sp + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(x[u], dp + i + u * stride);
  }
  for (; i < n_vec; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(sp + i), dp + i);
  if (blockIdx.x == 0 && threadIdx.x == 0) dst_pos[d] = src_pos[s];
}

}  // namespace

hipError_t launch_copy_states(const float* src, const int64_t* src_pos, float* dst, int64_t* dst_pos,
                              size_t n_floats, const CopyPairs& pairs, hipStream_t st) {
  const size_t n_vec = n_floats / 4;
  // About 16 KiB per block and pass; at least one block per pair.
  size_t blocks = (n_vec + (size_t)kCopyThreads * kCopyUnroll - 1) / ((size_t)kCopyThreads * kCopyUnroll);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_states_kernel, dim3((unsigned)blocks, (unsigned)pairs.n), dim3(kCopyThreads), 0, st,
                     reinterpret_cast<const f32x4*>(src), src_pos, reinterpret_cast<f32x4*>(dst), dst_pos, n_vec,
                     pairs);
  return hipGetLastError();
}

}  // namespace kda
