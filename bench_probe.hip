// bench_probe.hip -- measurement code for bench.py (not part of the library):
// the dense bf16 (or FP8) MFMA throughput this GPU sustains right now, and the
// shader clock it runs at while doing so.
//
// A grid of one 512-thread workgroup per compute unit (two waves per SIMD)
// issues v_mfma_f32_32x32x16_bf16 (or v_mfma_f32_32x32x64_f8f6f4 on E4M3
// operands) back to back into four independent accumulators per wave,
// cycling through eight A and four B fragments of random data so that
// consecutive MFMAs see different operands (as the attention loops' do).
// Throughput = 32768 (FP8: 131072) FLOP per MFMA / elapsed time; the clock
// comes from each workgroup's shader-cycle counter (s_memtime) against the
// 100 MHz real-time counter (s_memrealtime).
//
//   int fa2_probe_mfma(int iters, hipStream_t stream, double* tflops, double* ghz)
//   int fa2_probe_mfma_fp8(int iters, hipStream_t stream, double* tflops, double* ghz)
//
// iters: loop trips per wave (16 MFMAs each); stream: where the probe runs
// (0 = default).  Allocates and frees its own small buffers, synchronises the
// stream, returns 0 on success or the HIP error code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// two bf16 values in [-2, 2) with random mantissas
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) {
  const uint32_t lo = 0x3F80u | (h & 0x7Fu) | (((h >> 7) & 1u) << 15) | (((h >> 8) & 1u) << 7);
  const uint32_t hi = 0x3F80u | ((h >> 9) & 0x7Fu) | (((h >> 16) & 1u) << 15) | (((h >> 17) & 1u) << 7);
  return lo | (hi << 16);
}

// four E4M3 values in [-2^3, 2^3] with random mantissas (exponent fields 4..10)
__device__ __forceinline__ uint32_t rand_fp8x4(uint32_t h) {
  uint32_t w = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = h >> (8 * i);
    w |= ((b & 0x87u) | ((4u + (b >> 3) % 7u) << 3)) << (8 * i);
  }
  return w;
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void mfma_probe_fp8_kernel(int iters, float* sink, unsigned long long* clk) {
  const uint32_t tid = threadIdx.x;
  uint32_t h = mix(tid * 7919u + blockIdx.x * 104729u + 1u);
  i32x8 a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h = mix(h + 0x9E3779B9u);
      a[i][e] = (int)rand_fp8x4(h);
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h = mix(h + 0x9E3779B9u);
      b[i][e] = (int)rand_fp8x4(h);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[2 * i], b[i], c0, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[2 * i + 1], b[i], c1, 0, 0, 0, 0x7f7f7f7f, 0,
                                                          0x7f7f7f7f);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(2 * i + 2) & 7], b[(i + 1) & 3], c2, 0, 0, 0,
                                                          0x7f7f7f7f, 0, 0x7f7f7f7f);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(2 * i + 3) & 7], b[(i + 1) & 3], c3, 0, 0, 0,
                                                          0x7f7f7f7f, 0, 0x7f7f7f7f);
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * 512 + tid] = s;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void mfma_probe_kernel(int iters, float* sink, unsigned long long* clk) {
  const uint32_t tid = threadIdx.x;
  uint32_t h = mix(tid * 7919u + blockIdx.x * 104729u + 1u);
  u32x4 a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h = mix(h + 0x9E3779B9u);
      a[i][e] = rand_bf16x2(h);
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h = mix(h + 0x9E3779B9u);
      b[i][e] = rand_bf16x2(h);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[2 * i]),
                                                   __builtin_bit_cast(bf16x8, b[i]), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[2 * i + 1]),
                                                   __builtin_bit_cast(bf16x8, b[i]), c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[(2 * i + 2) & 7]),
                                                   __builtin_bit_cast(bf16x8, b[(i + 1) & 3]), c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[(2 * i + 3) & 7]),
                                                   __builtin_bit_cast(bf16x8, b[(i + 1) & 3]), c3, 0, 0, 0);
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * 512 + tid] = s;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

typedef void (*probe_fn)(int, float*, unsigned long long*);

int run_probe(probe_fn fn, double flop_per_mfma, int iters, hipStream_t stream, double* tflops, double* ghz) {
  if (iters < 1 || !tflops || !ghz) return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  float* sink = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipMalloc(&sink, (size_t)cus * 512 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&clk, (size_t)cus * 2 * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(fn, dim3(cus), dim3(512), 0, stream, 16, sink, clk);   // code load, clocks up
    e = hipEventRecord(e0, stream);
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(fn, dim3(cus), dim3(512), 0, stream, iters, sink, clk);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  unsigned long long* h = nullptr;
  if (e == hipSuccess) {
    h = new unsigned long long[(size_t)cus * 2];
    e = hipMemcpy(h, clk, (size_t)cus * 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  }
  if (e == hipSuccess) {
    double cyc = 0.0, ticks = 0.0;
    for (int i = 0; i < cus; ++i) {
      cyc += (double)h[2 * i];
      ticks += (double)h[2 * i + 1];
    }
    const double flops = (double)cus * 8.0 * (double)iters * 16.0 * flop_per_mfma;   // 8 waves per workgroup
    *tflops = flops / ((double)ms * 1e-3) / 1e12;
    *ghz = ticks > 0.0 ? cyc / (ticks / 100e6) / 1e9 : 0.0;
  }
  delete[] h;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (clk) (void)hipFree(clk);
  return (int)e;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int fa2_probe_mfma(int iters, hipStream_t stream, double* tflops,
                                                                    double* ghz) {
  return run_probe(mfma_probe_kernel, 32768.0, iters, stream, tflops, ghz);
}

extern "C" __attribute__((visibility("default"))) int fa2_probe_mfma_fp8(int iters, hipStream_t stream,
                                                                        double* tflops, double* ghz) {
  return run_probe(mfma_probe_fp8_kernel, 131072.0, iters, stream, tflops, ghz);
}
