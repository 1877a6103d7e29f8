// Measurement helpers for the bench and the GPU tests (not part of libkvx's
// transfer path): a synthetic ALU-bound compute kernel standing in for a
// model layer (it writes a canary into the layer's source KV blocks when it
// finishes, so a push that does not wait for it is caught), a plain
// contiguous copy (the counter calibration reference), a plain segment copy
// in the push kernel's shapes (the practical ceiling of the same bytes
// without a block table) and a cache-flush fill.
//
// All entry points enqueue on `stream` and return a hipError_t value (0 on
// success).

#include <hip/hip_ext.h>
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

// Plain copy of `nseg` segments of seg_bytes each, segment i from src[i] to
// dst[i], in the push kernel's workgroup shapes: T lanes keeping V 16-byte
// vectors each in flight, one T x V x 16-byte chunk per workgroup, all of a
// lane's loads issued before its first store, stores with the push kernel's
// cache policy for that shape (SA: nt for one-wave chunks, nt sc0 sc1 for
// four-wave ones).  The practical ceiling of the same bytes moved without
// any block table.
typedef const __attribute__((address_space(4))) uint64_t* ConstU64;
template <int T, int V, int SA>
__global__ __launch_bounds__(T) void segment_copy_kernel(const uint64_t* src, const uint64_t* dst, int64_t seg_bytes,
                                                         int64_t chunks_per_seg) {
  constexpr int kChunk = T * V * 16;
  const int64_t x = blockIdx.x;
  const int64_t seg = x / chunks_per_seg;
  const int64_t off = (x - seg * chunks_per_seg) * kChunk;
  const int64_t rest = seg_bytes - off;
  const int len = rest < kChunk ? int(rest) : kChunk;
  const uint64_t s = ((ConstU64)src)[seg], d = ((ConstU64)dst)[seg];
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(s + uint64_t(off)), (short)0, len, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(d + uint64_t(off)), (short)0, len, 0x00020000);
  v4u r[V];
#pragma unroll
  for (int k = 0; k < V; ++k) r[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (threadIdx.x + k * T) * 16, 0, 2);
#pragma unroll
  for (int k = 0; k < V; ++k) __builtin_amdgcn_raw_buffer_store_b128(r[k], rd, (threadIdx.x + k * T) * 16, 0, SA);
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

// Plain copy of nseg segments: segment i copies seg_bytes from src_ptrs[i]
// to dst_ptrs[i] (device arrays of nseg device addresses, 16-B aligned;
// seg_bytes a multiple of 16).  shape 0: one-wave workgroups of 32 KiB
// chunks; shape 1: four-wave workgroups of 4 KiB chunks.
int kvxb_copy_segments(const uint64_t* src_ptrs, const uint64_t* dst_ptrs, int32_t nseg, int64_t seg_bytes,
                       int32_t shape, hipStream_t stream) {
  if (nseg < 1 || seg_bytes < 16 || (seg_bytes & 15) || !src_ptrs || !dst_ptrs || shape < 0 || shape > 1)
    return int(hipErrorInvalidValue);
  const int64_t chunk = shape == 0 ? 32768 : 4096;
  const int64_t per = (seg_bytes + chunk - 1) / chunk;
  if (per * nseg > (int64_t(1) << 31) - 1) return int(hipErrorInvalidValue);
  const dim3 grid(unsigned(per * nseg));
  if (shape == 0)
    hipLaunchKernelGGL((segment_copy_kernel<64, 32, 2>), grid, dim3(64), 0, stream, src_ptrs, dst_ptrs, seg_bytes,
                       per);
  else
    hipLaunchKernelGGL((segment_copy_kernel<256, 1, 19>), grid, dim3(256), 0, stream, src_ptrs, dst_ptrs,
                       seg_bytes, per);
  return int(hipGetLastError());
}

// A stream at the default priority restricted to the compute units whose bits
// are set in mask[0..words) (bit i of word w = CU 32 w + i), for splitting
// the chip between the compute stand-in and the push.
int kvxb_stream_create_cu_mask(const uint32_t* mask, int32_t words, hipStream_t* out) {
  if (!mask || words < 1 || !out) return int(hipErrorInvalidValue);
  return int(hipExtStreamCreateWithCUMask(out, uint32_t(words), mask));
}

int kvxb_stream_destroy(hipStream_t s) { return int(hipStreamDestroy(s)); }

// Fill dst[0, bytes) with a 32-bit pattern (used to flush L2 and MALL).
int kvxb_fill(void* dst, int64_t bytes, uint32_t value, hipStream_t stream) {
  if ((bytes & 15) || (uintptr_t(dst) & 15)) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(kThreads), 0, stream, static_cast<v4u*>(dst), bytes / 16,
                     value);
  return int(hipGetLastError());
}

}  // extern "C"
