// Plain-transfer rates of the drift kernels' access patterns (measurement only; no part of
// the method). read_rows: one block of NT threads per row pair; lane `tid` reads the 16-byte
// vectors tid, tid + NT, ... of both rows with nontemporal loads, U per array in flight, as
// the scoring kernels do, and XOR-folds them so that the loads stay live. copy_rows: one
// block per row; active rows are copied with nontemporal loads and stores, U in flight per
// lane, other rows written as zeros, as the gradient pass moves its rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drift_ceiling.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
static_assert(kThreads / 64 == DRIFT_CEILING_SINK_WORDS, "one sink word per wave");

__device__ __forceinline__ uint32_t fold(const v4u& v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int NT, int U>
__global__ void __launch_bounds__(NT) read_rows(const char* a, const char* b, int64_t nvec,
                                                int64_t stride, uint32_t* sink) {
  const size_t off = (size_t)blockIdx.x * (size_t)stride;
  const v4u* va = (const v4u*)(a + off);
  const v4u* vb = (const v4u*)(b + off);
  uint32_t acc = 0;
  int64_t v = threadIdx.x;
  for (; v + (int64_t)(U - 1) * NT < nvec; v += (int64_t)NT * U) {
    v4u x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      x[u] = __builtin_nontemporal_load(va + v + u * NT);
      y[u] = __builtin_nontemporal_load(vb + v + u * NT);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(x[u]) ^ fold(y[u]);
  }
  for (; v < nvec; v += NT)
    acc ^= fold(__builtin_nontemporal_load(va + v)) ^ fold(__builtin_nontemporal_load(vb + v));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0)
    sink[(size_t)blockIdx.x * (NT / 64) + threadIdx.x / 64] = acc;
}

template <int NT, int U>
__global__ void __launch_bounds__(NT) copy_rows(const char* src, char* dst, int64_t nvec,
                                                int64_t sstride, int64_t dstride,
                                                const uint8_t* active) {
  const v4u* vs = (const v4u*)(src + (size_t)blockIdx.x * (size_t)sstride);
  v4u* vd = (v4u*)(dst + (size_t)blockIdx.x * (size_t)dstride);
  int64_t v = threadIdx.x;
  if (!active || active[blockIdx.x]) {
    for (; v + (int64_t)(U - 1) * NT < nvec; v += (int64_t)NT * U) {
      v4u x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(vs + v + u * NT);
#pragma unroll
      for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], vd + v + u * NT);
    }
    for (; v < nvec; v += NT) __builtin_nontemporal_store(__builtin_nontemporal_load(vs + v), vd + v);
  } else {
    const v4u z = {0u, 0u, 0u, 0u};
    for (; v < nvec; v += NT) __builtin_nontemporal_store(z, vd + v);
  }
}

}  // namespace

extern "C" int drift_copy_ceiling(const void* src, void* dst, int64_t rows, int64_t row_bytes,
                                  int64_t src_stride, int64_t dst_stride, const uint8_t* active,
                                  int unroll, void* stream) {
  if (rows < 0 || rows > INT32_MAX || row_bytes <= 0 || (row_bytes & 15) != 0 ||
      src_stride < row_bytes || (src_stride & 15) != 0 || dst_stride < row_bytes ||
      (dst_stride & 15) != 0 || (unroll != 4 && unroll != 8))
    return DRIFT_CEILING_EINVAL;
  if (rows == 0) return DRIFT_CEILING_OK;
  if (!src || !dst || (((uintptr_t)src | (uintptr_t)dst) & 15) != 0) return DRIFT_CEILING_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  if (unroll == 8)
    hipLaunchKernelGGL((copy_rows<kThreads, 8>), dim3((unsigned)rows), dim3(kThreads), 0, s,
                       (const char*)src, (char*)dst, row_bytes / 16, src_stride, dst_stride,
                       active);
  else
    hipLaunchKernelGGL((copy_rows<kThreads, 4>), dim3((unsigned)rows), dim3(kThreads), 0, s,
                       (const char*)src, (char*)dst, row_bytes / 16, src_stride, dst_stride,
                       active);
  return hipGetLastError() == hipSuccess ? DRIFT_CEILING_OK : DRIFT_CEILING_EHIP;
}

extern "C" int drift_read_ceiling(const void* a, const void* b, int64_t rows, int64_t row_bytes,
                                  int64_t stride_bytes, uint32_t* sink, void* stream) {
  if (rows < 0 || rows > INT32_MAX || row_bytes <= 0 || (row_bytes & 15) != 0 ||
      stride_bytes < row_bytes || (stride_bytes & 15) != 0)
    return DRIFT_CEILING_EINVAL;
  if (rows == 0) return DRIFT_CEILING_OK;
  if (!a || !b || !sink || (((uintptr_t)a | (uintptr_t)b) & 15) != 0 ||
      ((uintptr_t)sink & 3) != 0)
    return DRIFT_CEILING_EINVAL;
  hipLaunchKernelGGL((read_rows<kThreads, kUnroll>), dim3((unsigned)rows), dim3(kThreads), 0,
                     (hipStream_t)stream, (const char*)a, (const char*)b, row_bytes / 16,
                     stride_bytes, sink);
  return hipGetLastError() == hipSuccess ? DRIFT_CEILING_OK : DRIFT_CEILING_EHIP;
}
