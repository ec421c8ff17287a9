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

#include <algorithm>
#include <type_traits>

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

// (x & mask) | bits in one v_and_or_b32: gfx9 VOP3 encodings take no
// literal, so the mask comes from an SGPR and the OR-ed bits from a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask_s, uint32_t bits_v) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask_s), "v"(bits_v));
  return r;
}

// A VGPR holding constant c (for and_or's third operand).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// bf16 pair (128 + q_{2j}, 128 + q_{2j+1}) of gfx950-layout word w, given
// the magic 0x43004300 in a VGPR.
__device__ __forceinline__ uint32_t pair_bf16_fast(uint32_t w, int j, uint32_t magic_v) {
  return and_or(j == 0 ? w : w >> (4 * j), 0x000F000Fu, magic_v);
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
__global__ __launch_bounds__(256) void k_gemv_w4_tiled(KArgs p) {
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


// Streaming variant for bf16 activations (the decode path).  Same lane
// layout as k_gemv_w4_tiled, but:
//  * x is staged once per stage of sc_tiles tiles (the whole K when it fits
//    the LDS budget), so a workgroup passes at most a few barriers;
//  * weight and scale loads run D tiles ahead in a register ring, so every
//    lane keeps D x R 16-byte loads in flight;
//  * loads are raw buffer loads relative to the workgroup's first row (32-bit
//    offsets, one scalar descriptor), and rows past the end read as zero.
template <int R, int C, int LAYOUT, int D>
__global__ __launch_bounds__(256) void k_gemv_w4_stream(KArgs p, int sc_tiles) {
  extern __shared__ uint4 smem[];
  const int sch = TILE_CHUNKS * sc_tiles;                       // chunks per stage
  uint4* xs = smem;                                             // [C][4][sch]
  float* sxs = reinterpret_cast<float*>(smem + C * 4 * sch);    // [C][sch]

  const int tid = threadIdx.x;
  const int lane = tid & 31;
  const int hw = tid >> 5;
  const int64_t wg_row0 = (int64_t)blockIdx.x * 8 * R;
  const int64_t nchunks = p.k / 32;
  const int64_t rowbytes = p.k / 2;
  const int nit = (int)((nchunks + TILE_CHUNKS - 1) / TILE_CHUNKS);
  const int64_t ngroups = p.gshift < 0 ? 1 : (nchunks >> p.gshift);
  const int esz = p.scale_bf16 ? 2 : 4;
  const bool has_zeros = p.zeros != nullptr;

  // scalar descriptors over this workgroup's rows only
  const int64_t wg_rows = min((int64_t)8 * R, p.n - wg_row0);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + wg_row0 * rowbytes), 0, (int)(wg_rows * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)p.scales + wg_row0 * ngroups * esz), 0, (int)(wg_rows * ngroups * esz),
      0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(has_zeros ? (const char*)p.zeros + wg_row0 * ngroups * esz : (const char*)p.scales), 0,
      (int)(wg_rows * ngroups * esz), 0x00020000);

  uint4 wv[D][R];
  float sc[D][R], zb[D][R];
  float acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < C; ++j) acc[r][j] = 0.f;

  // local row of (half-wave, r) is hw * R + r
#define WQ_ISSUE(SLOT, IT)                                                                   \
  do {                                                                                       \
    const int ch_ = (IT) * TILE_CHUNKS + lane;                                               \
    const bool ok_ = ch_ < nchunks;                                                          \
    const int g_ = p.gshift < 0 ? 0 : (ch_ >> p.gshift);                                     \
    _Pragma("unroll") for (int r = 0; r < R; ++r) {                                          \
      const int lr_ = hw * R + r;                                                            \
      if (ok_) {                                                                             \
        wv[SLOT][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(        \
                          wrs, (int)(lr_ * rowbytes) + ch_ * 16, 0, 0));                      \
        const int so_ = (int)((lr_ * ngroups + g_) * esz);                                   \
        float s_, z_ = p.zero_const;                                                         \
        if (p.scale_bf16) {                                                                  \
          s_ = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(srs, so_, 0, 0));            \
          if (has_zeros) z_ = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(zrs, so_, 0, 0)); \
        } else {                                                                             \
          s_ = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, so_, 0, 0));        \
          if (has_zeros) z_ = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zrs, so_, 0, 0)); \
        }                                                                                    \
        sc[SLOT][r] = s_;                                                                    \
        zb[SLOT][r] = 128.f + z_;                                                            \
      } else {                                                                               \
        wv[SLOT][r] = make_uint4(0, 0, 0, 0);                                                \
        sc[SLOT][r] = 0.f;                                                                   \
        zb[SLOT][r] = 0.f;                                                                   \
      }                                                                                      \
    }                                                                                        \
  } while (0)

#pragma unroll
  for (int d = 0; d < D; ++d) WQ_ISSUE(d, d);

  for (int base = 0; base < nit; base += D) {
    if (base % sc_tiles == 0) {
      // stage x for tiles [base, base + sc_tiles) and the per-chunk sums of x
      __syncthreads();
      const int64_t k0 = (int64_t)base * TILE_K;
      const int units = C * 128 * sc_tiles;
      for (int idx = tid; idx < units; idx += 256) {
        const int col = idx / (128 * sc_tiles);
        const int u = idx % (128 * sc_tiles);
        const int t2 = u >> 7, v = u & 127;
        const int ch = v >> 2, piece = v & 3;
        const int64_t kk = k0 + (int64_t)u * 8;
        uint4 xv = make_uint4(0, 0, 0, 0);
        if (col < p.c && kk < p.k)
          xv = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.x) + col * p.k + kk);
        xs[(col * 4 + piece) * sch + t2 * TILE_CHUNKS + ch] = xv;
        float ps = ((bf16_to_f32(xv.x & 0xFFFFu) + bf16_to_f32(xv.x >> 16)) +
                    (bf16_to_f32(xv.y & 0xFFFFu) + bf16_to_f32(xv.y >> 16))) +
                   ((bf16_to_f32(xv.z & 0xFFFFu) + bf16_to_f32(xv.z >> 16)) +
                    (bf16_to_f32(xv.w & 0xFFFFu) + bf16_to_f32(xv.w >> 16)));
        ps += __shfl_xor(ps, 1);
        ps += __shfl_xor(ps, 2);
        if (piece == 0) sxs[col * sch + t2 * TILE_CHUNKS + ch] = ps;
      }
      __syncthreads();
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int it = base + d;
      if (it * TILE_CHUNKS + lane < nchunks) {
        uint32_t wp[R][16];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t w4[4] = {wv[d][r].x, wv[d][r].y, wv[d][r].z, wv[d][r].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) wp[r][4 * q + j] = pair_bf16<LAYOUT>(w4[q], j);
        }
        const int xo = (it % sc_tiles) * TILE_CHUNKS + lane;
#pragma unroll
        for (int col = 0; col < C; ++col) {
          uint32_t xv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = xs[(col * 4 + q) * sch + xo];
            xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
          }
          const float sx = sxs[col * sch + xo];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float dd = -zb[d][r] * sx;
#pragma unroll
            for (int e = 0; e < 16; ++e)
              dd = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[r][e]),
                                                   __builtin_bit_cast(bf16x2, xv[e]), dd, false);
            acc[r][col] = fmaf(sc[d][r], dd, acc[r][col]);
          }
        }
      }
      WQ_ISSUE(d, it + D);
    }
  }
#undef WQ_ISSUE

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
        const int64_t row = wg_row0 + hw * R + r;
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

// Sum over the 32 lanes of each half-wave with DPP (no LDS, no branch): the
// total lands in lanes 16..31 of each half-wave.
__device__ __forceinline__ float halfwave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad xor 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad xor 2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror 4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror 8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast 15
  return v;
}

// Persistent variant for one column of bf16 activations whose whole x fits
// in LDS (single-token decode).  One workgroup of NT lanes per CU; workgroup w owns a
// contiguous, balanced block of rows (+-1 row).  Its work is a list of items
// (row-group of R rows, tile of 1024 k) in row-group-major order, cut into
// NT/32 equal contiguous ranges, one per half-wave, so every half-wave
// streams the same number of 16-byte loads and keeps D items in flight from
// start to finish.  x and its per-chunk sums are staged in LDS once; the
// scales (and zeros) travel with the weights in the load ring, so the
// prologue waits only for x, which sits in cache after the first workgroup
// asks for it.  A half-wave reduces its partial for a
// row-group when it leaves it and parks it in an LDS slot; the slots of each
// row-group are summed in half-wave order at the end (fixed order: bitwise
// repeatable).
//
// The ring of loads stays in flight only if no load sits under a branch (the
// compiler's wait counting merges conservatively at joins), so the item loop
// issues every load unconditionally: an item that must not load (past the
// half-wave's range, or a chunk past K) gets an offset beyond the buffer,
// which the buffer unit answers with zeros, and past-the-range items get a
// zero scale -- they contribute exactly nothing.  Offsets are 32-bit,
// relative to the workgroup's rows, and advance by additions only.
constexpr uint32_t OOB = 0x80000000u;
constexpr int PERSIST_XCHUNKS = 3;  // x chunks a lane stages (C * K / 32 <= 3 * lanes)

template <int NT, int R, int C, int LAYOUT, int D, bool HZ, bool SBF>
__global__ __launch_bounds__(NT) void k_gemv_w4_persist(KArgs p, int sph) {
  constexpr int NHW = NT / 32;
  extern __shared__ uint4 smem[];
  const int nchunks = (int)(p.k / 32);
  const int nit = (nchunks + TILE_CHUNKS - 1) / TILE_CHUNKS;
  const int nch = nit * TILE_CHUNKS;                              // chunks in LDS
  const int ngroups = p.gshift < 0 ? 1 : (nchunks >> p.gshift);
  uint4* xs = smem;                                               // [C][4][nch]
  float* sxs = reinterpret_cast<float*>(smem + C * 4 * nch);      // [C][nch]
  float* slots = sxs + C * nch;                                   // [NHW][sph][R][C]
  int* hwtab = reinterpret_cast<int*>(slots + NHW * sph * R * C); // [NHW][3]: i0, i1, rg_first

  const int tid = threadIdx.x;
  const int lane = tid & 31;
  const int hw = tid >> 5;
  // this workgroup's rows (n < 2^31 is checked by the launcher)
  const int n32 = (int)p.n;
  const int q = n32 / (int)gridDim.x, rem = n32 % (int)gridDim.x;
  const int r0 = (int)blockIdx.x * q + min((int)blockIdx.x, rem);
  const int count = q + ((int)blockIdx.x < rem ? 1 : 0);
  const int nrg = (count + R - 1) / R;
  const int items = nrg * nit;
  const int i0 = (hw * items) / NHW, i1 = ((hw + 1) * items) / NHW;
  const int rg_first = i0 / nit;
  if (lane == 0) {
    hwtab[hw * 3 + 0] = i0;
    hwtab[hw * 3 + 1] = i1;
    hwtab[hw * 3 + 2] = rg_first;
  }

  const int rowbytes = (int)(p.k / 2);
  const int rgbytes = R * rowbytes;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + (int64_t)r0 * rowbytes), 0, count * rowbytes, 0x00020000);
  // scales (and zeros) of this workgroup's rows: loaded with the weights in
  // the ring (one per row and item), so the prologue waits for x only
  constexpr int ESZ = SBF ? 2 : 4;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)p.scales + (int64_t)r0 * ngroups * ESZ), 0, count * ngroups * ESZ, 0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)(HZ ? p.zeros : p.scales) + (int64_t)r0 * ngroups * ESZ), 0,
      HZ ? count * ngroups * ESZ : 0, 0x00020000);

  // issue position: byte offset of (row-group, tile) for this lane, its
  // row-group and tile, items left to issue
  int itile = i0 - rg_first * nit, left = i1 - i0, irg = rg_first;
  int ioff = rg_first * rgbytes + itile * (TILE_CHUNKS * 16) + lane * 16;
  uint4 wv[D][R];
  uint32_t sv[D][R], zv[D][R];  // raw scale / zero bits (converted when consumed)
  auto issue = [&](const int slot) {
    const int ch = itile * TILE_CHUNKS + lane;
    const bool ok = left > 0 && ch < nchunks;
    const uint32_t wo = ok ? (uint32_t)ioff : OOB;
    const int g = p.gshift < 0 ? 0 : (ch >> p.gshift);
    const uint32_t so = ok ? (uint32_t)((irg * R * ngroups + g) * ESZ) : OOB;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wv[slot][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                        wrs, wo + (uint32_t)(r * rowbytes), 0, 0));
      const uint32_t sro = so + (uint32_t)(r * ngroups * ESZ);
      if (SBF) {
        sv[slot][r] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)sro, 0, 0);
        if (HZ) zv[slot][r] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)sro, 0, 0);
      } else {
        sv[slot][r] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)sro, 0, 0);
        if (HZ) zv[slot][r] = __builtin_amdgcn_raw_buffer_load_b32(zrs, (int)sro, 0, 0);
      }
    }
    --left;
    ioff += TILE_CHUNKS * 16;
    if (++itile == nit) {
      itile = 0;
      ++irg;
      ioff += rgbytes - nit * (TILE_CHUNKS * 16);
    }
  };

  // Staging loads are issued before the weight prologue: loads complete in
  // issue order, so waiting for them must not also wait for the weights.
  // A lane stages whole 32-k chunks (all four 16-byte pieces), so the
  // lanes of one LDS write cover consecutive chunks of one piece plane:
  // no bank conflicts (lanes writing the four pieces of one chunk would hit
  // the same banks, the planes being a multiple of 256 bytes apart).
  // Unit u = tid + i * NT is chunk u / C of column u % C: a division by the
  // constant C (a division by a runtime count put some 140 more instructions
  // per wave ahead of the first weight load).  The loads stay conditional:
  // most units are past x (3 per lane cover the widest x), and the waves
  // with none skip their loads.
  constexpr int XCU = PERSIST_XCHUNKS;  // chunks per lane (the launcher bounds x)
  const int cunits = C * nch;
  uint4 xr[XCU][4];
#pragma unroll
  for (int i = 0; i < XCU; ++i) {
    const int cidx = tid + i * NT;
    const int ch = cidx / C, col = cidx - ch * C;
    const bool ok = cidx < cunits && col < p.c && ch < nchunks;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xr[i][q] = ok ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.x) + col * p.k + ch * 32 + 8 * q)
                    : make_uint4(0, 0, 0, 0);
  }
  // weight prologue: D items in flight per half-wave
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);

  // x (zero beyond k and beyond c) and the per-chunk sums of x into LDS
#pragma unroll
  for (int i = 0; i < XCU; ++i) {
    const int cidx = tid + i * NT;
    if (i * NT >= cunits) break;  // uniform over the workgroup
    if (cidx < cunits) {
      const int ch = cidx / C, col = cidx - ch * C;
      float pq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 xv = xr[i][q];
        pq[q] = ((bf16_to_f32(xv.x & 0xFFFFu) + bf16_to_f32(xv.x >> 16)) +
                 (bf16_to_f32(xv.y & 0xFFFFu) + bf16_to_f32(xv.y >> 16))) +
                ((bf16_to_f32(xv.z & 0xFFFFu) + bf16_to_f32(xv.z >> 16)) +
                 (bf16_to_f32(xv.w & 0xFFFFu) + bf16_to_f32(xv.w >> 16)));
        xs[(col * 4 + q) * nch + ch] = xv;
      }
      sxs[col * nch + ch] = (pq[0] + pq[1]) + (pq[2] + pq[3]);
    }
  }
  __syncthreads();

  const float zconst = 128.f + p.zero_const;
  const uint32_t magic_v = vconst(0x43004300u);
  float acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < C; ++j) acc[r][j] = 0.f;

  // consume position: row-group cg, tile ct
  int cg = rg_first, ct = i0 - rg_first * nit;
  const int nsteps = i1 - i0;
  for (int base = 0; base < nsteps; base += D) {
    {
      // issue priority from the share of items still to do: waves that
      // are behind (the youngest, which oldest-first arbitration serves last)
      // win the SIMD's issue slots
      const int left4 = __builtin_amdgcn_readfirstlane(4 * (nsteps - base));
      const int tot = __builtin_amdgcn_readfirstlane(nsteps);
      if (left4 > 3 * tot) __builtin_amdgcn_s_setprio(3);
      else if (left4 > 2 * tot) __builtin_amdgcn_s_setprio(2);
      else if (left4 > tot) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const bool valid = base + d < nsteps;
      const int xo = ct * TILE_CHUNKS + lane;
      uint32_t wp[R][16];
      float sc[R], zb[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w4[4] = {wv[d][r].x, wv[d][r].y, wv[d][r].z, wv[d][r].w};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            wp[r][4 * qq + j] = LAYOUT == 1 ? pair_bf16_fast(w4[qq], j, magic_v)
                                            : pair_bf16<LAYOUT>(w4[qq], j);
        // items past the half-wave's range (or chunks past k) loaded a zero
        // scale, so they contribute nothing
        if constexpr (SBF) {
          sc[r] = bf16_to_f32(sv[d][r]);
          zb[r] = HZ ? 128.f + bf16_to_f32(zv[d][r]) : zconst;
        } else {
          sc[r] = __uint_as_float(sv[d][r]);
          zb[r] = HZ ? 128.f + __uint_as_float(zv[d][r]) : zconst;
        }
      }
      issue(d);  // the ring slot is free once unpacked
#pragma unroll
      for (int col = 0; col < C; ++col) {
        uint32_t xv[16];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const uint4 v = xs[(col * 4 + qq) * nch + xo];
          xv[4 * qq + 0] = v.x; xv[4 * qq + 1] = v.y; xv[4 * qq + 2] = v.z; xv[4 * qq + 3] = v.w;
        }
        const float sx = sxs[col * nch + xo];
        float d0[R], d1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          d0[r] = -zb[r] * sx;
          d1[r] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 16; e += 2)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            d0[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[r][e]),
                                                    __builtin_bit_cast(bf16x2, xv[e]), d0[r], false);
            d1[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[r][e + 1]),
                                                    __builtin_bit_cast(bf16x2, xv[e + 1]), d1[r], false);
          }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][col] = fmaf(sc[r], d0[r] + d1[r], acc[r][col]);
      }
      if (valid && ++ct == nit) {
        // leaving row-group cg: park its partials (lane 31 of the half-wave
        // holds the sum after halfwave_sum), then start the next one
        float* dst = slots + ((hw * sph + (cg - rg_first)) * R) * C;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < C; ++j) {
            const float v = halfwave_sum(acc[r][j]);
            if (lane == 31) dst[r * C + j] = v;
            acc[r][j] = 0.f;
          }
        ct = 0;
        ++cg;
      }
    }
  }
  if (nsteps > 0 && ct != 0) {
    float* dst = slots + ((hw * sph + (cg - rg_first)) * R) * C;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float v = halfwave_sum(acc[r][j]);
        if (lane == 31) dst[r * C + j] = v;
      }
  }
  __syncthreads();

  // sum the parked partials of each (row-group, r, column) in half-wave order
  for (int idx = tid; idx < nrg * R * C; idx += NT) {
    const int rg = idx / (R * C);
    const int rc = idx - rg * R * C;
    const int r = rc / C, col = rc - r * C;
    if (col >= p.c || rg * R + r >= count) continue;
    const int ilo = rg * nit, ihi = ilo + nit;
    // half-wave h owns items [floor(h*items/NHW), floor((h+1)*items/NHW)); the
    // one owning item i is floor(((i + 1) * NHW - 1) / items)
    const int hlo = ((ilo + 1) * NHW - 1) / items, hhi = (ihi * NHW - 1) / items;
    float v = 0.f;
    for (int h = hlo; h <= hhi; ++h) {
      const int a = hwtab[h * 3 + 0], b = hwtab[h * 3 + 1];
      if (b > a && a < ihi && b > ilo) v += slots[((h * sph + (rg - hwtab[h * 3 + 2])) * R + r) * C + col];
    }
    const int64_t row = (int64_t)r0 + rg * R + r;
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.out)[col * p.n + row] = (uint16_t)f32_to_bf16_rne(v);
    else
      reinterpret_cast<float*>(p.out)[col * p.n + row] = v;
  }
}

// Decode kernel on lane quads (bf16 x, c <= 4, all of x in LDS), the
// products on the matrix cores.
//
// Lane l of a wave is (q, r) = (l / 4, l % 4): it owns output row r of the
// wave's current row-quad and chunk q (32 k) of the current item of 16
// chunks (512 k), one 16-byte load of its row per item, so each load
// instruction reads 256 contiguous bytes of each of four rows.  Quad q is
// block q of v_mfma_f32_4x4x4_16b_bf16 (16 independent 4 x 4 x 4 products
// per instruction): the B operand of lane (q, r) is four consecutive k of
// its row (bf16 128 + code, unpacked as in the other kernels), the A
// operand is the same four k of activation column r (columns past c repeat
// the last one; their results are never stored), and element i of the
// result is column i of row r.  Eight instructions cover the chunk,
// accumulating onto its zero-point fold term -(128 + z) * sum x; the VALU
// is left with the unpacking and one scale FMA per column.
//
// One workgroup of 1024 lanes per CU owns a balanced contiguous block of
// rows (+-1); its items (row-quad, 512-k slice) in row-quad-major order are
// cut into 16 equal contiguous ranges, one per wave.  x, and per chunk the
// offset term -(128 + z) * sum x of the zero-point fold, are staged in LDS
// once.  A wave sums its partial for a row-quad over the 16 quads (fixed
// DPP/swizzle order) when it leaves it and parks it in an LDS slot; each
// output is the sum of its parked partials in wave order (deterministic).
// Weight loads run D items ahead, issued without branches (past-the-end
// items read zeros with a zero scale and contribute nothing).
constexpr int QK_CH = 16;             // chunks per item: one per quad
constexpr int QK_NT = 1024;           // lanes per workgroup (one per CU)
constexpr int QK_NW = QK_NT / 64;     // waves per workgroup
constexpr int QK_XP = 9;              // 16-byte x pieces a lane stages (C * nchp * 4 <= QK_XP * QK_NT)

// Sum over the 16 quads of a wave (lanes with the same l % 4), fixed order:
// the four quads of each DPP row by rotation, then the four rows.
__device__ __forceinline__ float quadset_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror 4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror 8
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <int C, int LAYOUT, int D, bool HZ, bool SBF>
__global__ __launch_bounds__(QK_NT) void k_gemv_w4_quad(KArgs p, int spw) {
  extern __shared__ uint4 smem[];
  const int nchunks = (int)(p.k / 32);
  const int nkit = (nchunks + QK_CH - 1) / QK_CH;                  // items per row-quad
  const int nchp = nkit * QK_CH;                                     // chunks per column in LDS
  const int ngroups = p.gshift < 0 ? 1 : (nchunks >> p.gshift);
  // x pieces [nchp][C][4] with one spare piece per chunk (bank spread),
  // chunk terms [nchp][4]
  constexpr int XPC = 4 * C + 1;                                     // pieces per chunk
  uint4* xs = smem;
  float* zs = reinterpret_cast<float*>(xs + nchp * XPC);
  float* slots = zs + 4 * nchp;                                      // [NW][spw][4][C]
  int* wtab = reinterpret_cast<int*>(slots + QK_NW * spw * 4 * C);  // [NW][3]: i0, i1, rq_first

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 2, r = lane & 3;
  // this workgroup's rows (n < 2^31 is checked by the launcher)
  const int n32 = (int)p.n, nwg = (int)gridDim.x, b = (int)blockIdx.x;
  const int r0 = b * (n32 / nwg) + min(b, n32 % nwg);
  const int count = n32 / nwg + (b < n32 % nwg ? 1 : 0);
  const int nrq = (count + 3) / 4;
  const int items = nrq * nkit;
  const int i0 = wave * items / QK_NW, i1 = (wave + 1) * items / QK_NW;
  const int rq_first = i0 / nkit;
  if (lane == 0) {
    wtab[wave * 3 + 0] = i0;
    wtab[wave * 3 + 1] = i1;
    wtab[wave * 3 + 2] = rq_first;
  }

  const int rowbytes = (int)(p.k / 2);
  constexpr int ESZ = SBF ? 2 : 4;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + (int64_t)r0 * rowbytes), 0, count * rowbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)p.scales + (int64_t)r0 * ngroups * ESZ), 0, count * ngroups * ESZ, 0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)(HZ ? p.zeros : p.scales) + (int64_t)r0 * ngroups * ESZ), 0,
      HZ ? count * ngroups * ESZ : 0, 0x00020000);

  // issue position: item (row-quad, slice), this lane's chunk, byte offset of
  // its 16 bytes and its row's first scale; items left to issue
  int ikit = i0 - rq_first * nkit, left = i1 - i0;
  int ich = ikit * QK_CH + q;
  int ioff = (rq_first * 4 + r) * rowbytes + ich * 16;
  int isrow = (rq_first * 4 + r) * ngroups;
  uint4 wv[D];
  uint32_t sv[D], zv[D];
  auto issue = [&](const int slot) {
    const bool ok = left > 0 && ich < nchunks;  // rows past the block read zeros (descriptor)
    const int g = p.gshift < 0 ? 0 : (ich >> p.gshift);
    const uint32_t wo = ok ? (uint32_t)ioff : OOB;
    const uint32_t so = ok ? (uint32_t)((isrow + g) * ESZ) : OOB;
    wv[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wo, 0, 0));
    if (SBF) {
      sv[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)so, 0, 0);
      if (HZ) zv[slot] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)so, 0, 0);
    } else {
      sv[slot] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)so, 0, 0);
      if (HZ) zv[slot] = __builtin_amdgcn_raw_buffer_load_b32(zrs, (int)so, 0, 0);
    }
    --left;
    ich += QK_CH;
    ioff += QK_CH * 16;
    if (++ikit == nkit) {
      ikit = 0;
      ich = q;
      ioff += 4 * rowbytes - nkit * QK_CH * 16;
      isrow += 4 * ngroups;
    }
  };

  // x staging loads go out before the weight prologue (loads complete in
  // issue order, so waiting for x does not wait for the weights).  A lane
  // stages 16-byte pieces u = (chunk, column, piece) in [nchp][C][4] order,
  // u = tid + i * NT rotated by a per-workgroup offset: every CU reads the
  // same x, and in the same order they would all ask the same L2 channel at
  // once.  The four pieces of a chunk stay on four consecutive lanes (the
  // offset is a multiple of 4).  Chunk and column come from a division by
  // the constant C, and the loads are buffer loads without a branch (an
  // invalid piece reads zeros): with a division by a runtime count and a
  // branch per load, the address arithmetic of the staging was about 700
  // instructions per wave ahead of the first weight load.
  const int npieces = C * nchp * 4;
  const int xrot = (int)(((uint32_t)b * 2654435761u) % (uint32_t)(npieces >> 2)) * 4;
  auto piece = [&](int i) {
    const int v = tid + i * QK_NT + xrot;
    return v >= npieces ? v - npieces : v;
  };
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.x, 0, (int)(p.c * p.k * 2), 0x00020000);
  const uint32_t xcols = (uint32_t)p.c, xrow = (uint32_t)p.k * 2u;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  const float zfold = HZ ? 1.f : -(128.f + p.zero_const);
  // R rounds of x loads (R * NT >= npieces), the weight prologue, then x
  // into LDS with per chunk the offset term of the zero-point fold
  // -(128 + z) * sum x (with stored zeros: sum x, scaled per row later).
  // R is a compile-time count chosen from the x size below: rounds past x
  // would still take address-unit time ahead of the weight loads (an
  // out-of-range buffer load is not free), and with a runtime count the
  // compiler waits for every x load before the first LDS write.
  auto stage = [&](auto rounds) {
    constexpr int R = decltype(rounds)::value;
    uint4 xr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int u = piece(i);
      const uint32_t cc = (uint32_t)u >> 2, ch = cc / C, col = cc - ch * C;
      // (& rather than &&: no branch around the load)
      const bool ok = (tid + i * QK_NT < npieces) & (col < xcols) & (ch < (uint32_t)nchunks);
      const uint32_t xo = ok ? col * xrow + ch * 64u + (uint32_t)(u & 3) * 16u : OOB;
      xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)xo, 0, 0));
    }
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (i * QK_NT >= npieces) break;  // uniform
      const int u = piece(i);
      const uint4 v = xr[i];
      float sx = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), ones, 0.f, false);
      sx = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), ones, sx, false);
      sx = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), ones, sx, false);
      sx = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), ones, sx, false);
      sx += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sx), 0xB1, 0xF, 0xF, false));  // quad xor 1
      sx += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sx), 0x4E, 0xF, 0xF, false));  // quad xor 2
      if (tid + i * QK_NT < npieces) {
        const uint32_t cc = (uint32_t)u >> 2, ch = cc / C, col = cc - ch * C;
        xs[ch * XPC + col * 4 + (u & 3)] = v;
        if ((u & 3) == 0) zs[ch * 4 + col] = sx * zfold;
      }
    }
  };
  static_assert(QK_XP >= 5, "round counts");
  if (npieces <= 2 * QK_NT) stage(std::integral_constant<int, 2>{});
  else if (npieces <= 5 * QK_NT) stage(std::integral_constant<int, 5>{});
  else stage(std::integral_constant<int, QK_XP>{});
  __syncthreads();

  const float zconst = 128.f + p.zero_const;
  const uint32_t magic_v = vconst(0x43004300u);
  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;

  // park the partials of row-quad rq (this wave's slot rq - rq_first)
  auto park = [&](int rq) {
    float* dst = slots + ((wave * spw + (rq - rq_first)) * 4 + r) * C;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float v = quadset_sum(acc[j]);
      if (q == 0) dst[j] = v;
      acc[j] = 0.f;
    }
  };

  int crq = rq_first, ckit = i0 - rq_first * nkit;  // consume position
  const int nsteps = i1 - i0;
  for (int base = 0; base < nsteps; base += D) {
    {
      // issue priority from the share of items still to do: waves that are
      // behind (the youngest, which oldest-first arbitration serves last)
      // win the SIMD's issue slots
      const int left4 = 4 * (nsteps - base);
      if (left4 > 3 * nsteps) __builtin_amdgcn_s_setprio(3);
      else if (left4 > 2 * nsteps) __builtin_amdgcn_s_setprio(2);
      else if (left4 > nsteps) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const bool valid = base + d < nsteps;
      uint32_t wp[16];
      {
        const uint32_t w4[4] = {wv[d].x, wv[d].y, wv[d].z, wv[d].w};
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            wp[4 * m + j] = LAYOUT == 1 ? pair_bf16_fast(w4[m], j, magic_v) : pair_bf16<LAYOUT>(w4[m], j);
      }
      // past-the-range items and chunks past k loaded a zero scale
      float sc, zb = zconst;
      if constexpr (SBF) {
        sc = bf16_to_f32(sv[d]);
        if (HZ) zb = 128.f + bf16_to_f32(zv[d]);
      } else {
        sc = __uint_as_float(sv[d]);
        if (HZ) zb = 128.f + __uint_as_float(zv[d]);
      }
      issue(d);  // the ring slot is free once unpacked
      // A operand: column min(r, C - 1) of this lane's chunk (rows of the
      // block past c are never stored); C operand: the chunk's fold terms
      const int xo = ckit * QK_CH + q;  // chunk of this lane, < nchp
      const uint4* xp = xs + xo * XPC + min(r, C - 1) * 4;
      const uint4 xq[4] = {xp[0], xp[1], xp[2], xp[3]};
      floatx4 ch = *reinterpret_cast<const floatx4*>(zs + xo * 4);
      if (HZ) ch = -zb * ch;
#pragma unroll
      for (int st = 0; st < 8; ++st) {  // k 4 st .. 4 st + 3 of the chunk
        const uint4 xw = xq[st >> 1];
        const uint2 xa = (st & 1) ? make_uint2(xw.z, xw.w) : make_uint2(xw.x, xw.y);
        const uint2 wb = make_uint2(wp[2 * st], wp[2 * st + 1]);
        ch = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4, xa), __builtin_bit_cast(bf16x4, wb),
                                                  ch, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < C; ++j) acc[j] = fmaf(sc, ch[j], acc[j]);
      if (valid && ++ckit == nkit) {
        park(crq);
        ckit = 0;
        ++crq;
      }
    }
  }
  if (nsteps > 0 && ckit != 0) park(crq);
  __syncthreads();

  // sum the parked partials of each (row, column) in wave order
  for (int idx = tid; idx < nrq * 4 * C; idx += QK_NT) {
    const int rq = idx / (4 * C);
    const int rc = idx - rq * 4 * C;
    const int rr = rc / C, col = rc - rr * C;
    if (col >= p.c || rq * 4 + rr >= count) continue;
    const int ilo = rq * nkit, ihi = ilo + nkit;
    // wave h owns items [floor(h items / NW), floor((h + 1) items / NW)); the
    // one owning item i is floor(((i + 1) NW - 1) / items)
    const int hlo = ((ilo + 1) * QK_NW - 1) / items, hhi = (ihi * QK_NW - 1) / items;
    float v = 0.f;
    for (int h = hlo; h <= hhi; ++h) {
      const int a = wtab[h * 3 + 0], e = wtab[h * 3 + 1];
      if (e > a && a < ihi && e > ilo) v += slots[((h * spw + (rq - wtab[h * 3 + 2])) * 4 + rr) * C + col];
    }
    const int64_t row = (int64_t)r0 + rq * 4 + rr;
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.out)[col * p.n + row] = (uint16_t)f32_to_bf16_rne(v);
    else
      reinterpret_cast<float*>(p.out)[col * p.n + row] = v;
  }
}

// ---------------------------------------------------------------- MFMA GEMV
// bf16 activations, 2..32 columns: the products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16) instead of v_dot2, which leaves the VALU only
// the unpacking and the scaling.  x is the 16 x 32 A operand (one operand
// row per activation column; columns at or past c are zero), the weights of
// 16 output rows, unpacked to bf16 (128 + q) as in the other kernels, the
// 32 x 16 B operand.
//
// An item is one tile of 16 rows x 128 k (inside one scale group: groups of
// 128 k or more, or one per row).  Lane l (row n = l % 16, part g = l / 16)
// loads the 16 bytes of row n at k0 + 32 g .. k0 + 32 g + 31 and the same
// 32 k of x for column l % 16; MFMA m (m = 0..3) takes word m of each, so
// the k slots lane l brings to MFMA m are k0 + 32 g + 8 m + 0..7 on both
// operands and the instruction pairs equal k whatever its slot order.
// Result element i of lane l is column 4 g + i of row n (CB blocks of 16
// columns), so the row's scale is one value per lane.  The zero-point fold
// -(128 + z) sum x of a k group comes from a second chain with B = 1.
//
// One workgroup (1024 lanes; 512 with two column blocks, whose x operands
// take twice the registers) covers up to NRT row tiles for all of k, items
// in (k group, row tile) order split evenly over its waves: a wave walks a
// contiguous run of k groups and, for each, all the tiles, so the x operand
// (loaded from L2 one k group ahead, no staging in LDS) serves every tile.
// Each wave keeps one accumulator per tile; the partials are parked in LDS
// and added in wave order.
template <int CB, int NRT, int NT, int LAYOUT, int D, bool HZ, bool SBF>
__global__ __launch_bounds__(NT) void k_gemv_w4_mfma(KArgs p, int rows_per_wg) {
  constexpr int NW = NT / 64;
  extern __shared__ uint4 smem[];
  float* slots = reinterpret_cast<float*>(smem);  // [NW][NRT][16 CB columns][16 rows]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int k32 = (int)p.k, c = (int)p.c;
  const int nkg = (k32 + 127) / 128;
  const int ngroups = p.gshift < 0 ? 1 : ((k32 / 32) >> p.gshift);
  // this workgroup's rows: rows_per_wg each, the last ones fewer (n < 2^31
  // and rows_per_wg <= 16 NRT are checked by the launcher)
  const int r0 = (int)blockIdx.x * rows_per_wg;
  const int count = min(rows_per_wg, (int)p.n - r0);
  const int nrt = (count + 15) / 16;
  const int items = nrt * nkg;
  const int i0 = wave * items / NW, i1 = (wave + 1) * items / NW;
  const int kg_last = (i1 - 1) / max(nrt, 1);  // last k group of this wave

  const int rowbytes = k32 / 2;
  constexpr int ESZ = SBF ? 2 : 4;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + (int64_t)r0 * rowbytes), 0, count * rowbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)p.scales + (int64_t)r0 * ngroups * ESZ), 0, count * ngroups * ESZ, 0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)(HZ ? p.zeros : p.scales) + (int64_t)r0 * ngroups * ESZ), 0,
      HZ ? count * ngroups * ESZ : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, c * k32 * 2, 0x00020000);

  // x operand of k group kg for this lane (columns cb 16 + nl); only the
  // lanes of real columns load, the others hold zeros
  auto load_x = [&](uint4 (&xv)[CB][4], int kg) {
    const int kk = kg * 128 + 32 * g;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int m = 0; m < 4; ++m) xv[cb][m] = make_uint4(0, 0, 0, 0);
      const int col = cb * 16 + nl;
      if (col < c && kk < k32) {
        const int xo = (col * k32 + kk) * 2;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          xv[cb][m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * m, 0, 0));
      }
    }
  };

  // weight ring: issue position (k group, row tile), items left to issue
  int ikg = i0 / max(nrt, 1), irt = i0 - ikg * nrt, left = i1 - i0;
  uint4 wv[D];
  uint32_t sv[D], zv[D];
  auto issue = [&](const int slot) {
    // rows past the workgroup's read zeros (descriptor); k past the end is
    // masked per lane, but the scale is the row's for every lane of a live
    // item (each result element sums all 128 k of its row)
    const int kk = ikg * 128 + 32 * g, row = irt * 16 + nl;
    const bool live = left > 0, ok = live && kk < k32;
    const int gi = p.gshift < 0 ? 0 : ((ikg * 4) >> p.gshift);
    const uint32_t wo = ok ? (uint32_t)(row * rowbytes + kk / 2) : OOB;
    const uint32_t so = live ? (uint32_t)((row * ngroups + gi) * ESZ) : OOB;
    wv[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wo, 0, 0));
    if (SBF) {
      sv[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)so, 0, 0);
      if (HZ) zv[slot] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)so, 0, 0);
    } else {
      sv[slot] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)so, 0, 0);
      if (HZ) zv[slot] = __builtin_amdgcn_raw_buffer_load_b32(zrs, (int)so, 0, 0);
    }
    --left;
    if (++irt == nrt) {
      irt = 0;
      ++ikg;
    }
  };

  int ckg = i0 / max(nrt, 1), crt = i0 - ckg * nrt;  // consume position
  uint4 xc[CB][4], xn[CB][4];
  load_x(xc, ckg);
  if (ckg + 1 <= kg_last) load_x(xn, ckg + 1);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);

  const uint32_t magic_v = vconst(0x43004300u);
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const float zconst = 128.f + p.zero_const;
  floatx4 acc[NRT][CB], sx[CB];
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[t][cb] = zero4;
  // sum of x over the k group, per column, in the result layout
  auto xsum = [&]() {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      floatx4 v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xc[cb][0]), ones, zero4, 0, 0, 0);
#pragma unroll
      for (int m = 1; m < 4; ++m)
        v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xc[cb][m]), ones, v, 0, 0, 0);
      sx[cb] = v;
    }
  };
  xsum();

  const int nsteps = i1 - i0;
  for (int base = 0; base < nsteps; base += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const bool valid = base + d < nsteps;
      bf16x8 wb[4];
      {
        const uint32_t w4[4] = {wv[d].x, wv[d].y, wv[d].z, wv[d].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint4 u;
          if (LAYOUT == 1) {
            u.x = pair_bf16_fast(w4[m], 0, magic_v);
            u.y = pair_bf16_fast(w4[m], 1, magic_v);
            u.z = pair_bf16_fast(w4[m], 2, magic_v);
            u.w = pair_bf16_fast(w4[m], 3, magic_v);
          } else {
            u.x = pair_bf16<LAYOUT>(w4[m], 0);
            u.y = pair_bf16<LAYOUT>(w4[m], 1);
            u.z = pair_bf16<LAYOUT>(w4[m], 2);
            u.w = pair_bf16<LAYOUT>(w4[m], 3);
          }
          wb[m] = __builtin_bit_cast(bf16x8, u);
        }
      }
      float sc, zb = zconst;
      if constexpr (SBF) {
        sc = bf16_to_f32(sv[d]);
        if (HZ) zb = 128.f + bf16_to_f32(zv[d]);
      } else {
        sc = __uint_as_float(sv[d]);
        if (HZ) zb = 128.f + __uint_as_float(zv[d]);
      }
      issue(d);  // the ring slot is free once copied out
      if (valid) {  // uniform
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          floatx4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xc[cb][0]), wb[0], zero4, 0, 0, 0);
#pragma unroll
          for (int m = 1; m < 4; ++m)
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xc[cb][m]), wb[m], t, 0, 0, 0);
          floatx4 u;
#pragma unroll
          for (int i = 0; i < 4; ++i) u[i] = fmaf(-zb, sx[cb][i], t[i]);
          // acc += s * u on the one tile's accumulator, behind a uniform
          // branch (the empty asm keeps the compiler from updating every
          // tile's accumulator and selecting, about 60 VALU instructions per
          // item at six tiles)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            if (rt == crt) {
              asm volatile("");
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[rt][cb][i] = fmaf(sc, u[i], acc[rt][cb][i]);
            }
        }
        if (++crt == nrt) {  // next k group: its x was loaded one group ahead
          crt = 0;
          ++ckg;
          if (ckg <= kg_last) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
              for (int m = 0; m < 4; ++m) xc[cb][m] = xn[cb][m];
            if (ckg + 1 <= kg_last) load_x(xn, ckg + 1);
            xsum();
          }
        }
      }
    }
  }

  // park this wave's partial of every tile, then add them in wave order
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    if (rt >= nrt) break;  // uniform
    float* dst = slots + (wave * NRT + rt) * 256 * CB;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(cb * 16 + 4 * g + i) * 16 + nl] = acc[rt][cb][i];
  }
  __syncthreads();
  for (int idx = tid; idx < nrt * 16 * c; idx += NT) {
    const int rt = idx / (16 * c);
    const int rc = idx - rt * 16 * c;
    const int col = rc >> 4, rr = rc & 15;
    if (rt * 16 + rr >= count) continue;
    float v = 0.f;
    for (int h = 0; h < NW; ++h) v += slots[((h * NRT + rt) * 16 * CB + col) * 16 + rr];
    const int64_t row = (int64_t)r0 + rt * 16 + rr;
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.out)[col * p.n + row] = (uint16_t)f32_to_bf16_rne(v);
    else
      reinterpret_cast<float*>(p.out)[col * p.n + row] = v;
  }
}

// Wide-batch variant for bf16 activations (c = 5..32, in passes of at most
// 16 columns).  The work per weight byte grows with c, so this path is bound
// by the VALU (two MACs per v_dot2) rather than by HBM, and the kernel is laid
// out to keep the dot2 issue rate up:
//  * a wave owns 4 consecutive rows and a lane one chunk of 32 k of a 2048-k
//    tile, so each x fragment a lane reads from LDS feeds 4 rows (1 byte of
//    LDS per dot2) and 4 x 16 accumulators give plenty of independent work;
//  * a workgroup (4 waves) covers 16 rows, which leaves >= 256 workgroups
//    at the small-batch shapes;
//  * x is double-buffered in LDS per tile and filled by buffer loads that
//    write LDS directly; each lane then sums the chunks it loaded itself
//    (the per-chunk sums of x), so one barrier per tile suffices; when all
//    of x fits the two buffers (K <= 4096) it is staged once instead and the
//    loop has no barrier at all;
//  * 16-column passes run 512-lane workgroups of two column sets; 8-column
//    passes run two 256-lane workgroups per CU, or one of two column sets
//    when there are fewer than two row-groups per CU;
//  * weights and scales run two tiles ahead in a register ring, issued
//    without branches (past-the-end offsets read zero);
//  * after the last tile each wave sums its 64 lanes with DPP in a fixed
//    order.
// Load order per tile t: consume weights of t, x of t + 1 (to LDS), weights
// of t + 2.  The compiler's own wait before consuming the weights of t + 1
// then covers only the weights of t + 2 -- it cannot see the x loads, which
// are explicit asm -- and the explicit wait for x of t + 1 leaves exactly the
// weights of t + 2 in flight.
constexpr int BT_CH = 64;   // chunks per batch tile
constexpr int BT_RW = 4;    // rows per wave

__device__ __forceinline__ float wave_sum(float v) {
  v = halfwave_sum(v);  // half totals in lanes 16..31 and 48..63
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast 31
  return v;  // total in lanes 48..63
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor in SGPRs (offsets at or past num_records read 0).
__device__ __forceinline__ i32x4 sgpr_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc + voff into LDS at lds_base + 16 * lane
// (lds_base wave-uniform).  Explicit asm, so the compiler neither counts nor
// waits for it; callers wait with wait_vmcnt.  One wait state separates the
// M0 write from the load that reads M0 (the compiler's hazard checks do not
// see inside asm); no other code in this file uses M0.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// CS (1 or 2): column sets per workgroup.  With CS = 2 the workgroup has 8
// waves; waves w and w + 4 take the same 4 rows and the two halves of the
// columns, so each SIMD runs two waves on one x tile (the two load the same
// weights, which the CU's cache serves once).
// XS: all of x fits the two buffers (at most two tiles, K <= 4096): both
// tiles are staged once, buffer t holding tile t, and the item loop has no x
// loads and no barriers.
template <int C, int CS, bool XS, int LAYOUT, bool HZ, bool SBF>
__global__ __launch_bounds__(256 * CS, (C <= 8 && CS == 1) ? 2 : 1) void k_gemv_w4_batch(KArgs p) {
  static_assert(C % (4 * CS) == 0 && C <= 16, "columns per pass");
  constexpr int XC = C / (4 * CS);                       // x columns per wave and tile (loads)
  constexpr int CW = C / CS;                             // columns per wave (products)
  constexpr int WLOADS = BT_RW * (HZ ? 3 : 2);           // loads per lane per weight tile
  constexpr int RG = 4 * BT_RW;                          // rows per row-group (workgroup item)
  __shared__ __attribute__((aligned(16))) uint4 xs[2][C * 4 * BT_CH];  // [buf][col][piece][chunk]
  __shared__ float sxs[2][C * BT_CH];                    // [buf][col][chunk]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 3, wc = wave >> 2;  // row slot, column set
  const int nchunks = (int)(p.k / 32);
  const int nt = (nchunks + BT_CH - 1) / BT_CH;
  const int rowbytes = (int)(p.k / 2);
  const int ngroups = p.gshift < 0 ? 1 : (nchunks >> p.gshift);
  constexpr int ESZ = SBF ? 2 : 4;
  // persistent: workgroup w takes row-groups w, w + G, w + 2G, ...; its items
  // are (row-group, tile) in that order
  const int G = gridDim.x, w = blockIdx.x;
  const int nrg = (int)((p.n + RG - 1) / RG);
  const int nitems = (nrg > w ? (nrg - w + G - 1) / G : 0) * nt;

  const i32x4 xrs = sgpr_rsrc(p.x, (uint32_t)(p.c * p.k * 2));
  const uint32_t lds_x = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)&xs[0][0];

  // ---- weight ring: item i in slot i % 2.  Descriptors cover the wave's 4
  // rows of the item's row-group (none for items past the end).
  uint4 wv[2][BT_RW];
  float sc[2][BT_RW], zb[2][BT_RW];
  auto issue_w = [&](int slot, int i) {
    const int t = i % nt, rg = w + (i / nt) * G;
    const int64_t r0 = (int64_t)rg * RG + wr * BT_RW;
    const int wrows = i < nitems ? (int)max<int64_t>(0, min<int64_t>(BT_RW, p.n - r0)) : 0;
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.packed + r0 * rowbytes), 0, wrows * rowbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)p.scales + r0 * ngroups * ESZ), 0, wrows * ngroups * ESZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)(HZ ? p.zeros : p.scales) + r0 * ngroups * ESZ), 0,
        HZ ? wrows * ngroups * ESZ : 0, 0x00020000);
    const int ch = t * BT_CH + lane;
    const bool ok = ch < nchunks;
    const int g = p.gshift < 0 ? 0 : (ch >> p.gshift);
#pragma unroll
    for (int r = 0; r < BT_RW; ++r) {
      const uint32_t wo = ok ? (uint32_t)(r * rowbytes + ch * 16) : OOB;
      const uint32_t so = ok ? (uint32_t)((r * ngroups + g) * ESZ) : OOB;
      wv[slot][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wo, 0, 0));
      float sv, zv = p.zero_const;
      if (SBF) {
        sv = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(srs, (int)so, 0, 0));
        if (HZ) zv = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(zrs, (int)so, 0, 0));
      } else {
        sv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, (int)so, 0, 0));
        if (HZ) zv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zrs, (int)so, 0, 0));
      }
      sc[slot][r] = sv;  // 0 past the end: the item contributes nothing
      zb[slot][r] = 128.f + zv;
    }
  };

  // ---- x of item i's tile into buffer b: this wave fills chunk `lane` of
  // columns wave + 4 CS j, all four 16-byte pieces (a wave instruction
  // writes 64 consecutive 16-byte slots: one [col][piece] row of the buffer)
  auto dma_x = [&](int i, int b) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4");  // VALU-written SGPRs (descriptor, LDS bases) read by the loads
    const int ch = (i % nt) * BT_CH + lane;
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int col = wave + 4 * CS * j;
      const bool ok = i < nitems && ch < nchunks && col < p.c;
      // (OOB + 48 is still past num_records, which is below 2^31)
      const uint32_t base = ok ? (uint32_t)(((int64_t)col * p.k + (int64_t)ch * 32) * 2) : OOB;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dma16(xrs, base + q * 16,
              __builtin_amdgcn_readfirstlane(lds_x + (uint32_t)(((b * C + col) * 4 + q) * BT_CH * 16)));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // per-chunk sums of the x this lane loaded (its own loads have landed).
  // Without per-group zeros the stored value is already the offset term
  // -(128 + z) * sum x that starts every dot2 chain of the chunk.
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  const float xz = HZ ? 1.f : -(128.f + p.zero_const);
  auto sum_x = [&](int b) {
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int col = wave + 4 * CS * j;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = xs[b][(col * 4 + q) * BT_CH + lane];
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), ones, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), ones, s1, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), ones, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), ones, s1, false);
      }
      sxs[b][col * BT_CH + lane] = (s0 + s1) * xz;
    }
  };

  float acc[BT_RW][CW];
#pragma unroll
  for (int r = 0; r < BT_RW; ++r)
#pragma unroll
    for (int j = 0; j < CW; ++j) acc[r][j] = 0.f;
  const uint32_t magic_v = vconst(0x43004300u);

  // sum each accumulator over the wave's 64 chunks (fixed DPP order); lane
  // r * CW + cc stores row r, column wc * CW + cc of the row-group
  auto finish_rowgroup = [&](int i) {
    const int64_t r0 = (int64_t)(w + (i / nt) * G) * RG + wr * BT_RW;
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < BT_RW; ++r)
#pragma unroll
      for (int jj = 0; jj < CW; ++jj) {
        const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                            __builtin_bit_cast(int, wave_sum(acc[r][jj])), 63));
        if (lane == r * CW + jj) mine = v;
        acc[r][jj] = 0.f;
      }
    const int r = lane / CW, j = wc * CW + lane % CW;
    const int64_t row = r0 + r;
    if (lane < BT_RW * CW && j < p.c && row < p.n) {
      if (p.out_bf16)
        reinterpret_cast<uint16_t*>(p.out)[j * p.n + row] = (uint16_t)f32_to_bf16_rne(mine);
      else
        reinterpret_cast<float*>(p.out)[j * p.n + row] = mine;
    }
  };

  issue_w(0, 0);
  issue_w(1, 1);
  if constexpr (XS) {
    for (int t = 0; t < nt; ++t) dma_x(t, t);  // nt <= 2
    wait_vmcnt<0>();
    for (int t = 0; t < nt; ++t) sum_x(t);
  } else {
    dma_x(0, 0);
    wait_vmcnt<0>();
    sum_x(0);
  }
  __syncthreads();

  // item i uses ring slot and x buffer i % 2; the loop runs in pairs so that
  // both are compile-time constants (register arrays cannot be indexed at run
  // time)
  auto item = [&](const int i, const int slot) {
    const int b = XS ? i % nt : slot;  // x buffer
    // unpack this item's weights: 16 bf16 pairs (128 + q) per row
    uint32_t wp[BT_RW][16];
    float scr[BT_RW], zbr[BT_RW];
#pragma unroll
    for (int r = 0; r < BT_RW; ++r) {
      const uint32_t w4[4] = {wv[slot][r].x, wv[slot][r].y, wv[slot][r].z, wv[slot][r].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wp[r][4 * q + j] = LAYOUT == 1 ? pair_bf16_fast(w4[q], j, magic_v) : pair_bf16<0>(w4[q], j);
      scr[r] = sc[slot][r];
      zbr[r] = zb[slot][r];
    }
    if constexpr (!XS) dma_x(i + 1, b ^ 1);  // buffer b ^ 1 was last read in item i - 1
    issue_w(slot, i + 2);  // reuses the slot just unpacked

    // x fragments of two columns live at a time
    uint32_t xa[16], xb[16];
    float sa, sb;
    auto read_x = [&](int col, uint32_t (&xv)[16], float& sx) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = xs[b][(col * 4 + q) * BT_CH + lane];
        xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
      }
      sx = sxs[b][col * BT_CH + lane];
    };
    auto mac = [&](int cc, const uint32_t (&xv)[16], float sx) {  // cc: column within the set
      // four chains (one per row) interleaved in issue order, so
      // consecutive dot2 never depend on each other
      float d[BT_RW];
#pragma unroll
      for (int r = 0; r < BT_RW; ++r) d[r] = HZ ? -zbr[r] * sx : sx;
#pragma unroll
      for (int e = 0; e < 16; ++e)
#pragma unroll
        for (int r = 0; r < BT_RW; ++r)
          d[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[r][e]),
                                                 __builtin_bit_cast(bf16x2, xv[e]), d[r], false);
#pragma unroll
      for (int r = 0; r < BT_RW; ++r) acc[r][cc] = fmaf(scr[r], d[r], acc[r][cc]);
    };
    const int c0 = wc * CW;
    read_x(c0, xa, sa);
#pragma unroll
    for (int cc = 0; cc < CW; cc += 2) {
      read_x(c0 + cc + 1, xb, sb);
      mac(cc, xa, sa);
      __builtin_amdgcn_sched_barrier(0);
      if (cc + 2 < CW) read_x(c0 + cc + 2, xa, sa);
      mac(cc + 1, xb, sb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!XS) {
      // x of item i + 1 landed once only the weights of i + 2 are in flight
      wait_vmcnt<WLOADS>();
      sum_x(b ^ 1);
      __syncthreads();
    }
    if (i % nt == nt - 1) finish_rowgroup(i);  // uniform
  };
  for (int i = 0; i < nitems; i += 2) {
    item(i, 0);
    if (i + 1 < nitems) item(i + 1, 1);
  }
  wait_vmcnt<0>();  // nothing may still be writing LDS when the wave ends
}

constexpr int STREAM_LDS_BUDGET = 48 * 1024;  // bytes of LDS per workgroup

// D: weight tiles in flight per lane (4 for the decode batches; fewer for
// wide batches, whose LDS stage must then be shorter).
template <int R, int C, int D>
hipError_t launch_stream(const KArgs& ka, int layout, hipStream_t s) {
  const int nit = (int)((ka.k / 32 + TILE_CHUNKS - 1) / TILE_CHUNKS);
  const int per_tile = C * TILE_CHUNKS * (64 + 4);  // x units + chunk sums, bytes
  int sc_tiles = STREAM_LDS_BUDGET / per_tile;
  if (sc_tiles >= nit) {
    sc_tiles = nit;  // one stage holds all of x
  } else {
    sc_tiles = (sc_tiles / D) * D;  // stages start at ring boundaries
    if (sc_tiles < D) sc_tiles = D;
  }
  const size_t lds = (size_t)per_tile * sc_tiles;
  const unsigned blocks = (unsigned)((ka.n + 8 * R - 1) / (8 * R));
  if (layout == 1)
    hipLaunchKernelGGL((k_gemv_w4_stream<R, C, 1, D>), dim3(blocks), dim3(256), lds, s, ka, sc_tiles);
  else
    hipLaunchKernelGGL((k_gemv_w4_stream<R, C, 0, D>), dim3(blocks), dim3(256), lds, s, ka, sc_tiles);
  return hipGetLastError();
}


// ---- persistent launcher
constexpr int PERSIST_LDS_MAX = 160 * 1024;  // all of a gfx950 CU's LDS


int cu_count() { return device_cu_count(); }

// Largest number of row-groups one half-wave touches, over the two row
// counts (q and q + 1) the workgroups get.
int persist_slots(int64_t n, int grid, int R, int nit, int nhw) {
  const int64_t q = n / grid;
  int best = 1;
  for (int64_t cnt = q; cnt <= q + 1; ++cnt) {
    const int64_t items = ((cnt + R - 1) / R) * nit;
    for (int h = 0; h < nhw; ++h) {
      const int64_t a = h * items / nhw, b = (h + 1) * items / nhw;
      if (b > a) best = std::max(best, (int)((b - 1) / nit - a / nit + 1));
    }
  }
  return best;
}

// Returns hipErrorInvalidValue (without launching) when x does not fit in LDS.
template <int C>
hipError_t launch_persist(const KArgs& ka, int layout, hipStream_t s) {
  // 1024 lanes, two rows per half-wave item, one item in flight per
  // half-wave (two ran 4-6% slower at one column: with 16 waves per CU the
  // loads of the other waves keep HBM busy, and the shorter ring frees
  // registers and issue slots)
  constexpr int NT = 1024, R = 2, D = 1, NHW = NT / 32;
  if (ka.n >= (int64_t(1) << 31) || ka.k >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int64_t nchunks = ka.k / 32;
  const int nit = (int)((nchunks + TILE_CHUNKS - 1) / TILE_CHUNKS);
  const int64_t nch = (int64_t)nit * TILE_CHUNKS;
  const int64_t ngroups = ka.gshift < 0 ? 1 : (nchunks >> ka.gshift);
  int grid = cu_count();
  if ((int64_t)grid * R > ka.n) grid = (int)std::max<int64_t>(1, ka.n / R);
  const int64_t maxrows = (ka.n + grid - 1) / grid;
  // 32-bit offsets within a workgroup's rows: weights and scales
  if (maxrows * (ka.k / 2) >= (int64_t(1) << 31) || maxrows * ngroups * 4 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  const int sph = persist_slots(ka.n, grid, R, nit, NHW);
  const bool hz = ka.zeros != nullptr;
  const int64_t lds = C * nch * (64 + 4) + (int64_t)NHW * sph * R * C * 4 + NHW * 3 * 4;
  if (lds > PERSIST_LDS_MAX) return hipErrorInvalidValue;
  // per-lane staging registers of the kernel (x: PERSIST_XCHUNKS chunks)
  if (C * nch > PERSIST_XCHUNKS * NT) return hipErrorInvalidValue;
  const int sb = ka.scale_bf16 ? 1 : 0;
#define WQ_PFN(L, Z, S) reinterpret_cast<const void*>(&k_gemv_w4_persist<NT, R, C, L, D, Z, S>)
  const void* fns[2][2][2] = {{{WQ_PFN(0, false, false), WQ_PFN(0, false, true)},
                               {WQ_PFN(0, true, false), WQ_PFN(0, true, true)}},
                              {{WQ_PFN(1, false, false), WQ_PFN(1, false, true)},
                               {WQ_PFN(1, true, false), WQ_PFN(1, true, true)}}};
#undef WQ_PFN
  const void* fn = fns[layout][hz][sb];
  static std::atomic<uint64_t> lds_ok[2][2][2];  // devices where fn may use all of the LDS
  const hipError_t le = allow_dynamic_lds(fn, lds_ok[layout][hz][sb], PERSIST_LDS_MAX);
  if (le != hipSuccess) return le;
  int sph_arg = sph;
  void* args[] = {const_cast<KArgs*>(&ka), &sph_arg};
  return hipLaunchKernel(fn, dim3(grid), dim3(NT), args, (size_t)lds, s);
}

// Largest number of row-quads one wave of the quad kernel touches, over the
// two row counts (q and q + 1) the workgroups get.
int quad_slots(int64_t n, int grid, int nkit) {
  const int64_t q = n / grid;
  int best = 1;
  for (int64_t cnt = q; cnt <= q + 1; ++cnt) {
    const int64_t items = ((cnt + 3) / 4) * nkit;
    for (int h = 0; h < QK_NW; ++h) {
      const int64_t a = h * items / QK_NW, b = (h + 1) * items / QK_NW;
      if (b > a) best = std::max(best, (int)((b - 1) / nkit - a / nkit + 1));
    }
  }
  return best;
}

// Returns hipErrorInvalidValue (without launching) when x does not fit in LDS.
template <int C>
hipError_t launch_quad(const KArgs& ka, int layout, hipStream_t s) {
  constexpr int D = 2;  // items in flight per lane (one was 3-6% slower)
  if (ka.n >= (int64_t(1) << 31) || ka.k >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int64_t nchunks = ka.k / 32;
  const int nkit = (int)((nchunks + QK_CH - 1) / QK_CH);
  const int64_t nchp = (int64_t)nkit * QK_CH;
  const int64_t ngroups = ka.gshift < 0 ? 1 : (nchunks >> ka.gshift);
  int grid = cu_count();
  if ((int64_t)grid * 4 > ka.n) grid = (int)std::max<int64_t>(1, ka.n / 4);
  const int64_t maxrows = (ka.n + grid - 1) / grid + 4;
  // 32-bit offsets within a workgroup's rows (weights and scales)
  if (maxrows * (ka.k / 2) >= (int64_t(1) << 31) || maxrows * ngroups * 4 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  if (C * nchp * 4 > (int64_t)QK_XP * QK_NT) return hipErrorInvalidValue;  // staging registers
  const int spw = quad_slots(ka.n, grid, nkit);
  // x pieces (4 C + 1 per chunk), fold terms (4 per chunk), parked partials
  const int64_t lds = nchp * (4 * C + 1) * 16 + nchp * 16 + (int64_t)QK_NW * spw * 4 * C * 4 + QK_NW * 3 * 4;
  if (lds > PERSIST_LDS_MAX) return hipErrorInvalidValue;
  const bool hz = ka.zeros != nullptr;
  const int sb = ka.scale_bf16 ? 1 : 0;
#define WQ_QFN(L, Z, S) reinterpret_cast<const void*>(&k_gemv_w4_quad<C, L, D, Z, S>)
  const void* fns[2][2][2] = {{{WQ_QFN(0, false, false), WQ_QFN(0, false, true)},
                               {WQ_QFN(0, true, false), WQ_QFN(0, true, true)}},
                              {{WQ_QFN(1, false, false), WQ_QFN(1, false, true)},
                               {WQ_QFN(1, true, false), WQ_QFN(1, true, true)}}};
#undef WQ_QFN
  const void* fn = fns[layout][hz][sb];
  static std::atomic<uint64_t> lds_ok[2][2][2];  // devices where fn may use all of the LDS
  const hipError_t e = allow_dynamic_lds(fn, lds_ok[layout][hz][sb], PERSIST_LDS_MAX);
  if (e != hipSuccess) return e;
  int spw_arg = spw;
  void* args[] = {const_cast<KArgs*>(&ka), &spw_arg};
  return hipLaunchKernel(fn, dim3(grid), dim3(QK_NT), args, (size_t)lds, s);
}

// bf16 x, c <= 16 CB.  Returns hipErrorInvalidValue (without launching) for
// groups of 32 or 64 k (an item would span several) and for shapes past the
// kernel's 32-bit offsets.
template <int CB>
hipError_t launch_mfma(const KArgs& ka, int layout, hipStream_t s) {
  constexpr int NRT = CB == 1 ? 6 : 3;  // row tiles per workgroup (accumulators per lane)
  constexpr int NT = CB == 1 ? 1024 : 512;
  constexpr int D = 2;                  // items in flight per lane
  if (ka.gshift == 0 || ka.gshift == 1) return hipErrorInvalidValue;
  if (ka.n >= (int64_t(1) << 31) || ka.k >= (int64_t(1) << 24)) return hipErrorInvalidValue;
  const int64_t ngroups = ka.gshift < 0 ? 1 : ((ka.k / 32) >> ka.gshift);
  // an even share of the rows per CU, at most NRT tiles of 16 per workgroup
  const int cus = cu_count();
  int64_t rows = std::max<int64_t>(1, (ka.n + cus - 1) / cus);
  rows = std::min<int64_t>(rows, 16 * NRT);
  const int64_t grid = (ka.n + rows - 1) / rows;
  // 32-bit offsets within a workgroup's rows (weights and scales; x offsets
  // stay below 64 k < 2^31)
  if ((rows + 16) * (ka.k / 2) >= (int64_t(1) << 31) || (rows + 16) * ngroups * 4 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  const int64_t lds = (int64_t)(NT / 64) * NRT * 256 * CB * 4;
  const bool hz = ka.zeros != nullptr;
  const int sb = ka.scale_bf16 ? 1 : 0;
#define WQ_MFN(L, Z, S) reinterpret_cast<const void*>(&k_gemv_w4_mfma<CB, NRT, NT, L, D, Z, S>)
  const void* fns[2][2][2] = {{{WQ_MFN(0, false, false), WQ_MFN(0, false, true)},
                               {WQ_MFN(0, true, false), WQ_MFN(0, true, true)}},
                              {{WQ_MFN(1, false, false), WQ_MFN(1, false, true)},
                               {WQ_MFN(1, true, false), WQ_MFN(1, true, true)}}};
#undef WQ_MFN
  const void* fn = fns[layout][hz][sb];
  if (lds > 64 * 1024) {
    static std::atomic<uint64_t> lds_ok[2][2][2];  // devices where fn may use all of the LDS
    const hipError_t e = allow_dynamic_lds(fn, lds_ok[layout][hz][sb], PERSIST_LDS_MAX);
    if (e != hipSuccess) return e == hipErrorInvalidValue ? hipErrorNotSupported : e;
  }
  int rows_arg = (int)rows;
  void* args[] = {const_cast<KArgs*>(&ka), &rows_arg};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(NT), args, (size_t)lds, s);
}

// bf16 x, c <= 4: the persistent kernels when all of x fits in LDS (one
// column: two rows per lane, x from LDS per lane; two to four columns: x
// shared by lane quads), else for two to four columns the matrix-core
// kernel, else (groups of 32 or 64 k) the streaming kernel.
template <int C>
hipError_t launch_stream_c(const KArgs& ka, int layout, hipStream_t s) {
  static_assert(C <= 4, "decode batches");
  hipError_t e;
  if constexpr (C == 1) {
    e = launch_persist<C>(ka, layout, s);
  } else {
    // the quad kernel streams the decode shapes faster than the matrix-core
    // kernel (x staged once per CU, 256 contiguous bytes per row per load);
    // past its LDS the matrix-core kernel takes over
    e = launch_quad<C>(ka, layout, s);
    if (e != hipErrorInvalidValue) return e;
    e = launch_mfma<1>(ka, layout, s);
  }
  if (e != hipErrorInvalidValue) return e;
  // rows per half-wave: 2 when that still leaves >= 4 workgroups per CU
  if (ka.n >= 16 * 1024) return launch_stream<2, C, 4>(ka, layout, s);
  return launch_stream<1, C, 4>(ka, layout, s);
}

template <int R, int C, bool XBF16>
hipError_t launch_rc(const KArgs& ka, int layout, hipStream_t s) {
  const int64_t rows_per_wg = 8 * R;
  const unsigned blocks = (unsigned)((ka.n + rows_per_wg - 1) / rows_per_wg);
  if (layout == 1)
    hipLaunchKernelGGL((k_gemv_w4_tiled<R, C, XBF16, 1>), dim3(blocks), dim3(256), 0, s, ka);
  else
    hipLaunchKernelGGL((k_gemv_w4_tiled<R, C, XBF16, 0>), dim3(blocks), dim3(256), 0, s, ka);
  return hipGetLastError();
}

template <int C, bool XBF16>
hipError_t launch_c(const KArgs& ka, int layout, hipStream_t s) {
  // fp32 activations and the widest batches: rows per half-wave chosen to
  // keep enough workgroups and registers in bounds
  if (C <= 8 && ka.n >= 16 * 1024) return launch_rc<2, C, XBF16>(ka, layout, s);
  return launch_rc<1, C, XBF16>(ka, layout, s);
}


template <int C, int CS>
hipError_t launch_batch_cs(const KArgs& ka, int layout, hipStream_t s, int64_t nrg) {
  // persistent grid: as many workgroups as fit at once (two per CU for 8
  // columns in 256 lanes, else one), or one per row-group if there are fewer
  const unsigned blocks =
      (unsigned)std::min<int64_t>(nrg, (int64_t)cu_count() * (C <= 8 && CS == 1 ? 2 : 1));
  const bool hz = ka.zeros != nullptr, sb = ka.scale_bf16 != 0;
  const bool xs = (ka.k / 32 + BT_CH - 1) / BT_CH <= 2;  // x fits both buffers
#define WQ_BL(L, Z, S)                                                                           \
  do {                                                                                           \
    if (xs)                                                                                      \
      hipLaunchKernelGGL((k_gemv_w4_batch<C, CS, true, L, Z, S>), dim3(blocks), dim3(256 * CS), 0, s, ka); \
    else                                                                                         \
      hipLaunchKernelGGL((k_gemv_w4_batch<C, CS, false, L, Z, S>), dim3(blocks), dim3(256 * CS), 0, s, ka); \
  } while (0)
  if (layout == 1) {
    if (hz) { if (sb) WQ_BL(1, true, true); else WQ_BL(1, true, false); }
    else    { if (sb) WQ_BL(1, false, true); else WQ_BL(1, false, false); }
  } else {
    if (hz) { if (sb) WQ_BL(0, true, true); else WQ_BL(0, true, false); }
    else    { if (sb) WQ_BL(0, false, true); else WQ_BL(0, false, false); }
  }
#undef WQ_BL
  return hipGetLastError();
}

template <int C>
hipError_t launch_batch(const KArgs& ka, int layout, hipStream_t s) {
  const int64_t nrg = (ka.n + 4 * BT_RW - 1) / (4 * BT_RW);
  if constexpr (C > 8) {
    return launch_batch_cs<C, 2>(ka, layout, s, nrg);  // two column sets per workgroup
  } else {
    // 8 columns: two 256-lane workgroups per CU when there are row-groups
    // for them, else one 512-lane workgroup whose two column sets give each
    // SIMD a second wave
    if (nrg < 2 * (int64_t)cu_count()) return launch_batch_cs<C, 2>(ka, layout, s, nrg);
    return launch_batch_cs<C, 1>(ka, layout, s, nrg);
  }
}

hipError_t launch_bf16(const KArgs& ka, int layout, hipStream_t s) {
  switch (ka.c) {
    case 1: return launch_stream_c<1>(ka, layout, s);
    case 2: return launch_stream_c<2>(ka, layout, s);
    case 3: return launch_stream_c<3>(ka, layout, s);
    case 4: return launch_stream_c<4>(ka, layout, s);
    default: break;
  }
  // wider batches on the matrix cores: one or two blocks of 16 columns
  const hipError_t em = ka.c <= 16 ? launch_mfma<1>(ka, layout, s) : launch_mfma<2>(ka, layout, s);
  if (em != hipErrorInvalidValue) return em;
  // else (groups of 32 or 64 k) passes of at most 16 columns over
  // x[c0:c0+16] -> out[c0:c0+16]
  for (int64_t c0 = 0; c0 < ka.c; c0 += 16) {
    KArgs kp = ka;
    kp.c = std::min<int64_t>(16, ka.c - c0);
    kp.x = reinterpret_cast<const uint16_t*>(ka.x) + c0 * ka.k;
    kp.out = reinterpret_cast<char*>(ka.out) + c0 * ka.n * (ka.out_bf16 ? 2 : 4);
    const hipError_t e = kp.c <= 8 ? launch_batch<8>(kp, layout, s) : launch_batch<16>(kp, layout, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_f32(const KArgs& ka, int layout, hipStream_t s) {
  switch (ka.c) {
    case 1: return launch_c<1, false>(ka, layout, s);
    case 2: return launch_c<2, false>(ka, layout, s);
    case 3: return launch_c<3, false>(ka, layout, s);
    case 4: return launch_c<4, false>(ka, layout, s);
    default: break;
  }
  if (ka.c <= 8) return launch_c<8, false>(ka, layout, s);
  // wider batches: passes of at most 16 columns over x[c0:c0+16] -> out[c0:c0+16]
  for (int64_t c0 = 0; c0 < ka.c; c0 += 16) {
    KArgs kp = ka;
    kp.c = std::min<int64_t>(16, ka.c - c0);
    kp.x = reinterpret_cast<const float*>(ka.x) + c0 * ka.k;
    kp.out = reinterpret_cast<char*>(ka.out) + c0 * ka.n * (ka.out_bf16 ? 2 : 4);
    const hipError_t e = kp.c <= 8 ? launch_c<8, false>(kp, layout, s) : launch_c<16, false>(kp, layout, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  return a.x_bf16 ? launch_bf16(ka, a.layout, s) : launch_f32(ka, a.layout, s);
}

}  // namespace wq
