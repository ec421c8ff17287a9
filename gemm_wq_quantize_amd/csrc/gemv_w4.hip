// W4 GEMV with fused dequantisation (gfx950).
//
//   out[j][r] = sum_k (q[r][k] - z[r][g]) * s[r][g] * x[j][k],  g = k / group
//
// (Ternary post, section 3 MMVQ: the batched GEMV with x indexed [c][k],
// split over k with a final sum and over rows with none; dequantisation as in
// the Vulkan post, section 2 GLSL shader.)
//
// Work split.  A workgroup of 256 lanes is eight half-waves; each half-wave
// owns R consecutive rows and walks K in tiles of 1024 (32 chunks of 32 k):
// lane i of the half-wave takes chunk i of the tile, one 16-byte load per row
// (32 codes).  x for the tile is staged once in LDS and read by all 8R rows of
// the workgroup; every x value read from LDS is reused for R rows from
// registers.  After the last tile the 32 lanes of a half-wave sum their
// partials with a butterfly, so the result never depends on timing.
//
// bf16 activations: a gfx950-layout word w gives the codes (2j, 2j+1) as
// (w >> 4j) & 0x000F000F; OR 0x43004300 turns them into the bf16 pair
// (128 + q) exactly, which v_dot2_f32_bf16 multiplies with the matching x
// pair (products exact in fp32).  The offset folds out per 32-k chunk:
//   sum (q - z) x = sum (128 + q) x - (128 + z) sum x,
// with sum x precomputed per chunk while staging.  fp32 activations use
// v_cvt_f32_ubyte on the masked nibbles and fp32 FMAs.
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int TILE_CHUNKS = 32;  // chunks of 32 k per tile (one per half-wave lane)
constexpr int TILE_K = TILE_CHUNKS * 32;

struct KArgs {
  const uint8_t* packed;
  const void* scales;
  const void* zeros;
  const void* x;
  void* out;
  int64_t n, k, c;
  int gshift;  // log2(group / 32); -1 = one group per row
  float zero_const;
  int scale_bf16, out_bf16;
};

__device__ __forceinline__ float load_param(const void* p, int64_t i, int bf16) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i])
              : reinterpret_cast<const float*>(p)[i];
}

// bf16 pair (128 + q_{2j}, 128 + q_{2j+1}) of word w.
template <int LAYOUT>
__device__ __forceinline__ uint32_t pair_bf16(uint32_t w, int j) {
  if (LAYOUT == 1) return ((w >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
  // plain: codes 2j, 2j+1 are the two nibbles of byte j
  uint32_t b = (w >> (8 * j)) & 0xFFu;
  return (b & 0xFu) | ((b >> 4) << 16) | 0x43004300u;
}

// Code of element e (0..7, k order) of word w.
template <int LAYOUT>
__device__ __forceinline__ float code_f32(uint32_t w, int e) {
  int pos = LAYOUT == 1 ? (e >> 1) + 4 * (e & 1) : e;
  return (float)((w >> (4 * pos)) & 0xFu);
}

template <int R, int C, bool XBF16, int LAYOUT>
__global__ __launch_bounds__(256) void k_gemv_w4(KArgs p) {
  // x tile in LDS, 16-byte units arranged so lane i of a half-wave reads
  // unit i of each piece with no bank conflict: [col][piece][chunk].
  constexpr int UPC = XBF16 ? 4 : 8;  // 16-byte units per chunk (32 k)
  __shared__ uint4 xs[C * UPC * TILE_CHUNKS];
  __shared__ float sxs[C * TILE_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 31;
  const int hw = tid >> 5;
  const int64_t row0 = ((int64_t)blockIdx.x * 8 + hw) * R;
  const int64_t nchunks = p.k / 32;
  const int64_t rowbytes = p.k / 2;
  const int ntiles = (int)((nchunks + TILE_CHUNKS - 1) / TILE_CHUNKS);
  const int64_t ngroups = p.gshift < 0 ? 1 : (nchunks >> p.gshift);

  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = min(row0 + r, p.n - 1);

  float acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < C; ++j) acc[r][j] = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int64_t chunk = (int64_t)t * TILE_CHUNKS + lane;
    const bool valid = chunk < nchunks;
    // weights + scales of this tile: issued before staging so their latency
    // overlaps the x copy
    uint4 wv[R];
    float sc[R], zb[R];
    const int64_t g = p.gshift < 0 ? 0 : (chunk >> p.gshift);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (valid) {
        wv[r] = *reinterpret_cast<const uint4*>(p.packed + rows[r] * rowbytes + chunk * 16);
        sc[r] = load_param(p.scales, rows[r] * ngroups + g, p.scale_bf16);
        float z = p.zeros ? load_param(p.zeros, rows[r] * ngroups + g, p.scale_bf16) : p.zero_const;
        zb[r] = XBF16 ? 128.f + z : z;
      } else {
        wv[r] = make_uint4(0, 0, 0, 0);
        sc[r] = 0.f;
        zb[r] = 0.f;
      }
    }

    __syncthreads();  // previous tile's readers are done with xs
    // stage x[:, tile] (zero beyond k or beyond c) and the per-chunk sums
    for (int idx = tid; idx < C * UPC * TILE_CHUNKS; idx += 256) {
      const int col = idx / (UPC * TILE_CHUNKS);
      const int u = idx % (UPC * TILE_CHUNKS);  // unit within the column's tile
      const int ch = u / UPC, piece = u % UPC;
      const int64_t kk = (int64_t)t * TILE_K + (int64_t)u * (XBF16 ? 8 : 4);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < p.c && kk < p.k) {
        if (XBF16)
          v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.x) + col * p.k + kk);
        else
          v = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.x) + col * p.k + kk);
      }
      xs[(col * UPC + piece) * TILE_CHUNKS + ch] = v;
      float ps;
      if (XBF16) {
        ps = ((bf16_to_f32(v.x & 0xFFFFu) + bf16_to_f32(v.x >> 16)) +
              (bf16_to_f32(v.y & 0xFFFFu) + bf16_to_f32(v.y >> 16))) +
             ((bf16_to_f32(v.z & 0xFFFFu) + bf16_to_f32(v.z >> 16)) +
              (bf16_to_f32(v.w & 0xFFFFu) + bf16_to_f32(v.w >> 16)));
      } else {
        ps = (__uint_as_float(v.x) + __uint_as_float(v.y)) +
             (__uint_as_float(v.z) + __uint_as_float(v.w));
      }
      // units of one chunk are UPC consecutive lanes
#pragma unroll
      for (int off = 1; off < UPC; off <<= 1) ps += __shfl_xor(ps, off);
      if (piece == 0) sxs[col * TILE_CHUNKS + ch] = ps;
    }
    __syncthreads();

    if (valid) {
      if (XBF16) {
        uint32_t wp[R][16];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t w4[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) wp[r][4 * q + j] = pair_bf16<LAYOUT>(w4[q], j);
        }
#pragma unroll
        for (int col = 0; col < C; ++col) {
          uint32_t xv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint4 v = xs[(col * 4 + q) * TILE_CHUNKS + lane];
            xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
          }
          const float sx = sxs[col * TILE_CHUNKS + lane];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float d = -zb[r] * sx;
#pragma unroll
            for (int e = 0; e < 16; ++e)
              d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[r][e]),
                                                  __builtin_bit_cast(bf16x2, xv[e]), d, false);
            acc[r][col] = fmaf(sc[r], d, acc[r][col]);
          }
        }
      } else {
        float wf[R][32];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t w4[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) wf[r][8 * q + e] = code_f32<LAYOUT>(w4[q], e);
        }
#pragma unroll
        for (int col = 0; col < C; ++col) {
          float xv[32];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            uint4 v = xs[(col * 8 + q) * TILE_CHUNKS + lane];
            xv[4 * q + 0] = __uint_as_float(v.x); xv[4 * q + 1] = __uint_as_float(v.y);
            xv[4 * q + 2] = __uint_as_float(v.z); xv[4 * q + 3] = __uint_as_float(v.w);
          }
          const float sx = sxs[col * TILE_CHUNKS + lane];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float d = -zb[r] * sx;
#pragma unroll
            for (int e = 0; e < 32; ++e) d = fmaf(wf[r][e], xv[e], d);
            acc[r][col] = fmaf(sc[r], d, acc[r][col]);
          }
        }
      }
    }
  }

  // sum the 32 lanes of the half-wave (fixed butterfly order)
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v = acc[r][j];
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) v += __shfl_xor(v, off);
      acc[r][j] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if (j >= p.c) break;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        if (row < p.n) {
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[j * p.n + row] = (uint16_t)f32_to_bf16_rne(acc[r][j]);
          else
            reinterpret_cast<float*>(p.out)[j * p.n + row] = acc[r][j];
        }
      }
    }
  }
}

template <int R, int C, bool XBF16>
hipError_t launch_rc(const KArgs& ka, int layout, hipStream_t s) {
  const int64_t rows_per_wg = 8 * R;
  const unsigned blocks = (unsigned)((ka.n + rows_per_wg - 1) / rows_per_wg);
  if (layout == 1)
    hipLaunchKernelGGL((k_gemv_w4<R, C, XBF16, 1>), dim3(blocks), dim3(256), 0, s, ka);
  else
    hipLaunchKernelGGL((k_gemv_w4<R, C, XBF16, 0>), dim3(blocks), dim3(256), 0, s, ka);
  return hipGetLastError();
}

template <int C, bool XBF16>
hipError_t launch_c(const KArgs& ka, int layout, hipStream_t s) {
  // rows per half-wave: keep enough workgroups to spread over 256 CUs and
  // keep registers in bounds for wide batches and fp32 activations
  const int64_t target_wgs = 1024;
  if (XBF16 && C <= 4 && ka.n >= 32 * target_wgs) return launch_rc<4, C, XBF16>(ka, layout, s);
  if (C <= 8 && ka.n >= 16 * target_wgs) return launch_rc<2, C, XBF16>(ka, layout, s);
  return launch_rc<1, C, XBF16>(ka, layout, s);
}

template <bool XBF16>
hipError_t launch_x(const KArgs& ka, int layout, hipStream_t s) {
  switch (ka.c) {
    case 1: return launch_c<1, XBF16>(ka, layout, s);
    case 2: return launch_c<2, XBF16>(ka, layout, s);
    case 3: return launch_c<3, XBF16>(ka, layout, s);
    case 4: return launch_c<4, XBF16>(ka, layout, s);
    default: break;
  }
  if (ka.c <= 8) return launch_c<8, XBF16>(ka, layout, s);
  if (ka.c <= 16) return launch_c<16, XBF16>(ka, layout, s);
  return launch_c<32, XBF16>(ka, layout, s);
}

}  // namespace

hipError_t launch_gemv_w4(const GemvArgs& a, hipStream_t s) {
  KArgs ka;
  ka.packed = a.packed;
  ka.scales = a.scales;
  ka.zeros = a.zeros;
  ka.x = a.x;
  ka.out = a.out;
  ka.n = a.n;
  ka.k = a.k;
  ka.c = a.c;
  ka.zero_const = a.zero_const;
  ka.scale_bf16 = a.scale_bf16 ? 1 : 0;
  ka.out_bf16 = a.out_bf16 ? 1 : 0;
  if (a.group == a.k) {
    ka.gshift = -1;
  } else {
    int sh = 0;
    while ((int64_t(32) << sh) < a.group) ++sh;
    ka.gshift = sh;
  }
  return a.x_bf16 ? launch_x<true>(ka, a.layout, s) : launch_x<false>(ka, a.layout, s);
}

}  // namespace wq
