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

// Single-pass quantiser: one team of TEAM lanes per (row, group), each lane
// holding WPL 16-byte words (8 fp16 weights each) of the group in registers.
//
// code = clamp(rint(RN(w / s)), -8, 7) + 8 needs the correctly rounded
// float32 quotient only where rounding to an integer can tell it apart from
// a nearby value.  With r = RN(1 / s), one FMA (the fp16 weight converted
// inside it) gives t = RN(w r + 8.5 + 2^-18).  |w / s| <= 7.02 (s is the
// group's absmax / 7, rounded to bf16 or float32), so w r lies within 2^-21
// of w / s, RN(w / s) within 2^-22 of it, and the rounding of t (t < 16)
// adds at most 2^-21: t = RN(w / s) + 8.5 + 2^-18 + e with |e| < 2^-19.
// floor(t) is therefore rint(RN(w / s)) + 8 unless RN(w / s) is a
// half-integer (a tie, which rounds to even) or t crossed an integer, and in
// both cases fract(t) < 2^-17; a lane where fract(t) <= 2^-17 recomputes
// that code with the IEEE divide (one uniform branch per code: ties of an
// fp16 weight and a bf16 scale land in a sizeable share of the waves, but
// rarely on the same code).  The clamp to [-8, 7] cannot
// bind here: s is at least (absmax / 7)(1 - 2^-9) after rounding, so
// |w / s| < 7.014, t lies in [1.48, 15.52] and floor(t) in [1, 15] (the
// exact path keeps the clamp).  s is a normal number, so nothing over- or
// underflows.  The group's absmax is taken on the fp16 bit
// patterns: for finite values, magnitude order is the unsigned order of the
// bits without the sign.
template <int LAYOUT>
__device__ __forceinline__ uint32_t pack8(const int (&c)[8]) {
  if (LAYOUT == 0)
    return c[0] | c[1] << 4 | c[2] << 8 | c[3] << 12 | c[4] << 16 | c[5] << 20 | c[6] << 24 | c[7] << 28;
  return c[0] | c[2] << 4 | c[4] << 8 | c[6] << 12 | c[1] << 16 | c[3] << 20 | c[5] << 24 | c[7] << 28;
}

template <int TEAM, int WPL, int LAYOUT>
__global__ __launch_bounds__(256) void k_quantize_pack_r(const uint16_t* __restrict__ w,
                                                         uint32_t* __restrict__ packed,
                                                         void* __restrict__ scales, int n,
                                                         int ngroups, int64_t k, int group,
                                                         int scale_bf16) {
  constexpr int TPW = 256 / TEAM;  // teams per workgroup
  const int tid = threadIdx.x, lane = tid % TEAM;
  const int unit = (int)blockIdx.x * TPW + tid / TEAM;  // (row, group); n * ngroups < 2^31
  const bool active = unit < n * ngroups;
  const int u = active ? unit : 0;
  const int row = u / ngroups, g = u - row * ngroups;
  const int gw = group / 8;  // words per group
  const uint16_t* src = w + (int64_t)row * k + (int64_t)g * group;

  uint4 v[WPL];
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mx = {0, 0};  // largest |w| bits, two halves
#pragma unroll
  for (int i = 0; i < WPL; ++i) {
    const int j = lane + TEAM * i;
    v[i] = j < gw ? *reinterpret_cast<const uint4*>(src + 8 * j) : make_uint4(0, 0, 0, 0);
    const uint32_t h[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, h[e] & 0x7FFF7FFFu));
  }
  float amax = fmaxf(f16_to_f32(mx.x), f16_to_f32(mx.y));
#pragma unroll
  for (int off = TEAM / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, TEAM));

  const float s32 = amax / 7.0f;  // IEEE divide
  uint32_t sbits = 0;
  float s = s32;
  if (scale_bf16) {
    sbits = f32_to_bf16_rne(s32);
    s = bf16_to_f32(sbits);
  }
  if (active && lane == 0) {
    if (scale_bf16)
      reinterpret_cast<uint16_t*>(scales)[u] = (uint16_t)sbits;
    else
      reinterpret_cast<float*>(scales)[u] = s;
  }
  const float r = 1.0f / s;  // IEEE; +inf when s == 0 (codes are then 8)
  uint32_t word[WPL];
#pragma unroll
  for (int i = 0; i < WPL; ++i) {
    const uint32_t h[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    int c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = f16_to_f32(e & 1 ? h[e >> 1] >> 16 : h[e >> 1] & 0xFFFFu);
      const float t = fmaf(x, r, 8.5f + 0x1p-18f);
      const bool near = __builtin_amdgcn_fractf(t) <= 0x1p-17f;
      c[e] = (int)(uint32_t)t;  // floor: t > 0 (the clamp cannot bind, see above)
      // exact quotient for this code where any lane of the wave needs it:
      // exact ties of an fp16 weight and a bf16 scale are common enough
      // that most waves have one somewhere, but rarely at the same code
      if (__builtin_amdgcn_ballot_w64(near) != 0) {  // uniform
        const int ce = (int)fminf(fmaxf(rintf(x / s), -8.f), 7.f) + 8;
        if (near) c[e] = ce;
      }
    }
    word[i] = pack8<LAYOUT>(c);
  }
  if (!active) return;
  uint32_t* dst = packed + ((int64_t)row * k + (int64_t)g * group) / 8;
#pragma unroll
  for (int i = 0; i < WPL; ++i) {
    const int j = lane + TEAM * i;
    if (j < gw) dst[j] = s == 0.f ? 0x88888888u : word[i];
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
  // single pass with the group in registers: 8 lanes per group of up to 64
  // words (4 lanes for 4 words), 64 lanes per group of up to 512 words;
  // larger groups take the two-pass kernel below
  if (units < (int64_t(1) << 30) && group < (int64_t(1) << 30) && gw <= 8 * 64) {
    const int team = gw <= 4 ? 4 : gw <= 64 ? 8 : 64;
    const int64_t wpl = (gw + team - 1) / team;  // 1..8
    const int wsel = wpl <= 1 ? 1 : wpl <= 2 ? 2 : wpl <= 4 ? 4 : 8;
    const unsigned blocks = (unsigned)((units * team + 255) / 256);
#define WQ_QR(T, W)                                                                           \
  do {                                                                                        \
    if (layout == 0)                                                                          \
      hipLaunchKernelGGL((k_quantize_pack_r<T, W, 0>), dim3(blocks), dim3(256), 0, s, w, out,   \
                         scales, (int)n, (int)(k / group), k, (int)group, sb);                \
    else                                                                                      \
      hipLaunchKernelGGL((k_quantize_pack_r<T, W, 1>), dim3(blocks), dim3(256), 0, s, w, out,   \
                         scales, (int)n, (int)(k / group), k, (int)group, sb);                \
  } while (0)
    bool launched = true;
    if (team == 4) WQ_QR(4, 1);
    else if (team == 8 && wsel == 1) WQ_QR(8, 1);
    else if (team == 8 && wsel == 2) WQ_QR(8, 2);
    else if (team == 8 && wsel == 4) WQ_QR(8, 4);
    else if (team == 8 && wsel == 8) WQ_QR(8, 8);
    else if (team == 64 && wsel == 2) WQ_QR(64, 2);
    else if (team == 64 && wsel == 4) WQ_QR(64, 4);
    else if (team == 64 && wsel == 8) WQ_QR(64, 8);
    else launched = false;
#undef WQ_QR
    if (launched) return hipGetLastError();
  }
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
