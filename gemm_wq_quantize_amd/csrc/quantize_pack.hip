// int4 packing and fp16 -> int4 weight-only quantisation (gfx950).
//
// Packing follows the Vulkan post (section 1, packing strategy: eight codes
// per little-endian 32-bit word, element 0 lowest) and the Paddle PR
// ("int4量化kernel": two codes per byte along K).  The gfx950 layout keeps
// words in place and reorders the nibbles inside each word as 0 2 4 6 1 3 5
// 7 -- the fast-dequant order of the Paddle PR's "int4 permute kernel"
// section -- so the GEMV/GEMM inner loops turn (word >> 4j) & 0x000F000F
// into a pair of neighbouring codes with no further moves.
#include "wq_internal.h"

namespace wq {
namespace {

// Eight codes c[0..7] (k order, one per byte of lo/hi) -> one packed word.
__device__ __forceinline__ uint32_t pack_word(uint32_t lo, uint32_t hi, int layout) {
  uint32_t c0 = lo & 15u, c1 = (lo >> 8) & 15u, c2 = (lo >> 16) & 15u, c3 = (lo >> 24) & 15u;
  uint32_t c4 = hi & 15u, c5 = (hi >> 8) & 15u, c6 = (hi >> 16) & 15u, c7 = (hi >> 24) & 15u;
  if (layout == 0)
    return c0 | c1 << 4 | c2 << 8 | c3 << 12 | c4 << 16 | c5 << 20 | c6 << 24 | c7 << 28;
  // nibble p holds element {0,2,4,6,1,3,5,7}[p]
  return c0 | c2 << 4 | c4 << 8 | c6 << 12 | c1 << 16 | c3 << 20 | c5 << 24 | c7 << 28;
}

__global__ __launch_bounds__(256) void k_pack_int4(const uint32_t* __restrict__ codes,
                                                   uint32_t* __restrict__ packed,
                                                   int64_t nwords, int layout) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nwords) return;
  uint32_t lo = codes[2 * i], hi = codes[2 * i + 1];
  packed[i] = pack_word(lo, hi, layout);
}

// One team of TEAM lanes per (row, group).  Pass 1: absmax over the group.
// Pass 2: scale, then codes, eight per word.
template <int TEAM>
__global__ __launch_bounds__(256) void k_quantize_pack(const uint16_t* __restrict__ w,
                                                       uint32_t* __restrict__ packed,
                                                       void* __restrict__ scales,
                                                       int64_t n, int64_t k, int64_t group,
                                                       int layout, int scale_bf16) {
  const int lane = threadIdx.x % TEAM;
  const int64_t ngroups = k / group;
  const int64_t unit = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TEAM;
  const bool active = unit < n * ngroups;
  const int64_t u = active ? unit : 0;
  const int64_t row = u / ngroups, g = u % ngroups;
  const uint16_t* src = w + row * k + g * group;
  const int64_t gw = group / 8;  // packed words per group

  float amax = 0.f;
  for (int64_t j = lane; j < gw; j += TEAM) {
    uint4 v = *reinterpret_cast<const uint4*>(src + 8 * j);
    uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(f16_to_f32(h[e] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(f16_to_f32(h[e] >> 16)));
    }
  }
#pragma unroll
  for (int off = TEAM / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, TEAM));

  const float s32 = amax / 7.0f;  // IEEE divide
  float s;
  uint32_t sbits = 0;
  if (scale_bf16) {
    sbits = f32_to_bf16_rne(s32);
    s = bf16_to_f32(sbits);
  } else {
    s = s32;
  }
  if (!active) return;
  if (lane == 0) {
    if (scale_bf16)
      reinterpret_cast<uint16_t*>(scales)[u] = (uint16_t)sbits;
    else
      reinterpret_cast<float*>(scales)[u] = s;
  }
  uint32_t* dst = packed + (row * k + g * group) / 8;
  for (int64_t j = lane; j < gw; j += TEAM) {
    uint4 v = *reinterpret_cast<const uint4*>(src + 8 * j);
    uint32_t h[4] = {v.x, v.y, v.z, v.w};
    uint32_t q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = f16_to_f32(e & 1 ? h[e >> 1] >> 16 : h[e >> 1] & 0xFFFFu);
      int qi = 8;
      if (s != 0.f) {
        float r = rintf(x / s);  // IEEE divide by the stored scale, ties to even
        r = fminf(fmaxf(r, -8.f), 7.f);
        qi = (int)r + 8;
      }
      q[e] = (uint32_t)qi;
    }
    uint32_t lo = q[0] | q[1] << 8 | q[2] << 16 | q[3] << 24;
    uint32_t hi = q[4] | q[5] << 8 | q[6] << 16 | q[7] << 24;
    dst[j] = pack_word(lo, hi, layout);
  }
}

}  // namespace

hipError_t launch_pack_int4(const uint8_t* codes, int64_t n, int64_t k, int layout,
                            uint8_t* packed, hipStream_t s) {
  int64_t nwords = n * k / 8;
  int64_t blocks = (nwords + 255) / 256;
  hipLaunchKernelGGL(k_pack_int4, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(codes), reinterpret_cast<uint32_t*>(packed),
                     nwords, layout);
  return hipGetLastError();
}

hipError_t launch_quantize_pack_int4(const uint16_t* w, int64_t n, int64_t k, int64_t group,
                                     int layout, uint8_t* packed, void* scales, bool scale_bf16,
                                     hipStream_t s) {
  int64_t gw = group / 8;
  int64_t units = n * (k / group);
  uint32_t* out = reinterpret_cast<uint32_t*>(packed);
  int sb = scale_bf16 ? 1 : 0;
#define WQ_QP(T)                                                                         \
  do {                                                                                   \
    int64_t blocks = (units * T + 255) / 256;                                            \
    hipLaunchKernelGGL(k_quantize_pack<T>, dim3((unsigned)blocks), dim3(256), 0, s, w,   \
                       out, scales, n, k, group, layout, sb);                            \
  } while (0)
  if (gw >= 64) WQ_QP(64);
  else if (gw >= 32) WQ_QP(32);
  else if (gw >= 16) WQ_QP(16);
  else if (gw >= 8) WQ_QP(8);
  else WQ_QP(4);
#undef WQ_QP
  return hipGetLastError();
}

}  // namespace wq
