// Calibration kernels: the practical ceilings of this device for the bounds
// the library's kernels meet (a streaming read of HBM, the bf16 matrix
// cores, fp32 FMA issue).  They share nothing with the product kernels.
#include "../../include/wq.h"
#include "../../include/wq_peaks.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int RD_THREADS = 1024;
constexpr int RD_DEPTH = 4;               // 16-byte loads in flight per lane
constexpr int RD_MAX_GRID = 4096;
constexpr int64_t RD_SINK_WORDS = int64_t(RD_MAX_GRID) * (RD_THREADS / 64);

// Workgroup b reads the contiguous share [b q + min(b, r), ...) of the n16
// 16-byte units; every lane folds what it reads, each wave stores the XOR
// of its lanes.
__global__ __launch_bounds__(RD_THREADS) void k_peak_read(const uint4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t q = n16 / gridDim.x, r = n16 % gridDim.x;
  const int64_t b = blockIdx.x;
  const int64_t b0 = b * q + (b < r ? b : r), cnt = q + (b < r ? 1 : 0);
  uint32_t acc = 0;
  int64_t i = threadIdx.x;
  for (; i + (RD_DEPTH - 1) * RD_THREADS < cnt; i += RD_DEPTH * RD_THREADS) {
    uint4 v[RD_DEPTH];
#pragma unroll
    for (int d = 0; d < RD_DEPTH; ++d) v[d] = p[b0 + i + d * RD_THREADS];
#pragma unroll
    for (int d = 0; d < RD_DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  for (; i < cnt; i += RD_THREADS) {
    const uint4 v = p[b0 + i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0) sink[b * (RD_THREADS / 64) + (threadIdx.x >> 6)] = acc;
}

// NB independent 32x32x16 bf16 products per round on fixed register operands.
template <int NB>
__global__ __launch_bounds__(256) void k_peak_mfma(float* __restrict__ sink, int iters, uint32_t seed) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  f32x16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  // bf16 bit patterns below 0x4000: finite values in [0, 2)
  const u32x4 ra = u32x4{seed ^ threadIdx.x, seed * 3u, seed + 7u, seed ^ 0x3F803F80u} & 0x3FFF3FFFu;
  const u32x4 rb = u32x4{seed + threadIdx.x, seed * 5u, seed + 9u, seed ^ 0x3F003F00u} & 0x3FFF3FFFu;
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), bv = __builtin_bit_cast(bf16x8, rb);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// 8 independent chains of v_fma_f32 per lane.
__global__ __launch_bounds__(256) void k_peak_fma(float* __restrict__ sink, int iters, uint32_t seed) {
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (float)(threadIdx.x + j) * 1e-3f;
  const uint32_t u = seed ^ threadIdx.x;
  const float f0 = __uint_as_float((u & 0x7FFFFFu) | 0x3F000000u), f1 = f0 * 0.5f;  // f0 in [0.5, 1)
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __builtin_fmaf(f0, a[j], f1);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

int device_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return -1;
  return v;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int loop_args(int workgroups, int iters, const float* sink, int64_t sink_words) {
  if (workgroups < 0 || iters < 0 || sink_words < 0) return WQ_EINVAL;
  if (workgroups == 0) return WQ_OK;
  if (!sink) return WQ_EINVAL;
  if (!aligned(sink, 4)) return WQ_EALIGN;
  if (workgroups > (1 << 20) || iters < 1 || iters > (1 << 20) || sink_words < int64_t(workgroups) * 256)
    return WQ_ESHAPE;
  return 1;  // valid, work to do
}

}  // namespace

extern "C" {

int64_t wq_peak_read_sink_words(void) { return RD_SINK_WORDS; }

int wq_peak_read(const void* buf, int64_t nbytes, uint32_t* sink, int64_t sink_words, void* stream) {
  if (nbytes < 0 || sink_words < 0) return WQ_EINVAL;
  if (nbytes == 0) return WQ_OK;
  if (!buf || !sink) return WQ_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return WQ_EALIGN;
  if (nbytes % 16 != 0 || nbytes >= (int64_t(1) << 40) || sink_words < RD_SINK_WORDS) return WQ_ESHAPE;
  const int cus = device_cus();
  if (cus < 0) return WQ_EHIP;
  const int64_t n16 = nbytes / 16;
  const int grid = (int)(n16 < cus ? n16 : (cus < RD_MAX_GRID ? cus : RD_MAX_GRID));
  hipLaunchKernelGGL(k_peak_read, dim3((unsigned)grid), dim3(RD_THREADS), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_EHIP;
}

int wq_peak_mfma_bf16(int workgroups, int iters, float* sink, int64_t sink_words, void* stream) {
  const int v = loop_args(workgroups, iters, sink, sink_words);
  if (v != 1) return v;
  hipLaunchKernelGGL(k_peak_mfma<8>, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, sink,
                     iters, 12345u);
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_EHIP;
}

int wq_peak_valu_fma(int workgroups, int iters, float* sink, int64_t sink_words, void* stream) {
  const int v = loop_args(workgroups, iters, sink, sink_words);
  if (v != 1) return v;
  hipLaunchKernelGGL(k_peak_fma, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, sink, iters,
                     777u);
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_EHIP;
}

}  // extern "C"
