// Measurement helpers for the bench and the GPU tests (not part of libkvx's
// transfer path): a synthetic ALU-bound compute kernel standing in for a
// model layer (it writes a canary into the layer's source KV blocks when it
// finishes, so a push that does not wait for it is caught), a plain
// contiguous copy (the practical HBM ceiling and the counter calibration
// reference) and a cache-flush fill.
//
// All entry points enqueue on `stream` and return a hipError_t value (0 on
// success).

#include <hip/hip_runtime.h>

#include <cstdint>

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float spin(int iters, float x) {
  float a = x, b = x * 0.5f + 1.0f, c = x * 0.25f + 2.0f, d = x * 0.125f + 3.0f;
  for (int i = 0; i < iters; ++i) {
    a = __builtin_fmaf(a, 0.999f, 0.001f);
    b = __builtin_fmaf(b, 0.999f, 0.002f);
    c = __builtin_fmaf(c, 0.999f, 0.003f);
    d = __builtin_fmaf(d, 0.999f, 0.004f);
  }
  return a + b + c + d;
}

// Spin, then write a 16-byte canary at the start of each listed block of the
// K and V regions (block b of region r starts at r + b * block_bytes).
__global__ __launch_bounds__(kThreads) void layer_compute_kernel(float* sink, int iters,
                                                                 uint8_t* k_region, uint8_t* v_region,
                                                                 const int32_t* blocks, int nblocks,
                                                                 int64_t block_bytes, uint32_t canary) {
  const int gt = blockIdx.x * kThreads + threadIdx.x;
  const float r = spin(iters, float(threadIdx.x) * 1e-3f);
  sink[gt] = r;
  if (!k_region) return;
  __syncthreads();
  const v4u c = {canary, canary ^ 0x5a5a5a5au, canary + 1u, ~canary};
  for (int i = gt; i < nblocks; i += gridDim.x * kThreads) {
    const int64_t off = int64_t(blocks[i]) * block_bytes;
    *reinterpret_cast<v4u*>(k_region + off) = c;
    *reinterpret_cast<v4u*>(v_region + off) = c;
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(v4u* __restrict__ d, const v4u* __restrict__ s,
                                                        int64_t nvec) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const v4u a = __builtin_nontemporal_load(s + i);
    const v4u b = __builtin_nontemporal_load(s + i + stride);
    const v4u c = __builtin_nontemporal_load(s + i + 2 * stride);
    const v4u e = __builtin_nontemporal_load(s + i + 3 * stride);
    __builtin_nontemporal_store(a, d + i);
    __builtin_nontemporal_store(b, d + i + stride);
    __builtin_nontemporal_store(c, d + i + 2 * stride);
    __builtin_nontemporal_store(e, d + i + 3 * stride);
  }
  for (; i < nvec; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

__global__ __launch_bounds__(kThreads) void fill_kernel(v4u* d, int64_t nvec, uint32_t value) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  const v4u v = {value, value, value, value};
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride) d[i] = v;
}

}  // namespace

extern "C" {

// Synthetic layer compute: `grid` workgroups of 256 lanes each run `iters`
// FMA rounds; sink must hold grid*256 floats.  With k_region == NULL no
// canary is written.
int kvxb_layer_compute(float* sink, int32_t iters, int32_t grid, void* k_region, void* v_region,
                       const int32_t* blocks, int32_t nblocks, int64_t block_bytes, uint32_t canary,
                       hipStream_t stream) {
  if (grid < 1 || iters < 0 || !sink) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(layer_compute_kernel, dim3(grid), dim3(kThreads), 0, stream, sink, iters,
                     static_cast<uint8_t*>(k_region), static_cast<uint8_t*>(v_region), blocks, nblocks,
                     block_bytes, canary);
  return int(hipGetLastError());
}

// dst[0, bytes) = src[0, bytes); bytes a multiple of 16, both 16-B aligned.
int kvxb_copy(void* dst, const void* src, int64_t bytes, int32_t grid, hipStream_t stream) {
  if ((bytes & 15) || ((uintptr_t(dst) | uintptr_t(src)) & 15) || grid < 1) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<v4u*>(dst),
                     static_cast<const v4u*>(src), bytes / 16);
  return int(hipGetLastError());
}

// Fill dst[0, bytes) with a 32-bit pattern (used to flush L2 and MALL).
int kvxb_fill(void* dst, int64_t bytes, uint32_t value, hipStream_t stream) {
  if ((bytes & 15) || (uintptr_t(dst) & 15)) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(kThreads), 0, stream, static_cast<v4u*>(dst), bytes / 16,
                     value);
  return int(hipGetLastError());
}

}  // extern "C"
