// W4A16 GEMM on the bf16 matrix cores (gfx950).
//
//   C[i][j] = s[j] * sum_k A[i][k] * (q[j][k] - z)
//
// (Helion issue "int4 gemm kernel": C = A x unpack(B) with two codes per
// byte along K; here B is stored output-major [N][K/2] in the gfx950 nibble
// order, with a per-column bf16 scale applied in the epilogue and a float32
// accumulator.)
//
// Tiling.  A 256-lane workgroup computes a 256 x 256 tile of C with four
// waves in a 2 x 2 grid; each wave owns 128 x 128 = 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16.  K advances 64 per step through a two-stage LDS
// ring: the next step's A (256 x 64 bf16) and packed B (256 x 32 bytes) are
// fetched with buffer loads into registers while the current step's MFMAs
// run, then written to the other LDS stage.  B stays packed in LDS (4x less
// LDS traffic than a bf16 tile).
//
// Dequantisation.  One 32-bit B word is exactly the 8 consecutive k one lane
// feeds to the MFMA.  Each bf16 pair (128 + q_{2j}, 128 + q_{2j+1}) comes out
// of the word with one v_and_or_b32 (plus a shift) and is exact in bf16; the
// MFMA accumulates sum_k A (128 + q), and the offset folds out in the
// epilogue with A's row sums, which every wave accumulates from the A
// fragments it already holds (v_dot2 against ones):
//   sum_k A (q - z) = sum_k A (128 + q) - (128 + z) sum_k A.
// Workgroups are renumbered so that each XCD (8 on MI355X, dispatched
// round-robin) walks a compact band of output tiles, sharing A and B rows in
// its own L2.
#include "wq_internal.h"

namespace wq {
namespace {

#ifndef WQ_G_UNROLL
#define WQ_G_UNROLL 2  // unroll of the 16-k steps inside one LDS stage
#endif
#define WQ_PRAGMA(x) _Pragma(#x)
#define WQ_UNROLL(n) WQ_PRAGMA(unroll n)

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_LD = BK + 8;   // bf16 elements per LDS row of A (16-byte pad)
constexpr int B_LDW = BK / 8;  // 32-bit words per LDS row of packed B

struct GArgs {
  const uint16_t* a;
  const uint8_t* b;
  const uint16_t* scales;
  uint16_t* c;
  int64_t m, n, k;
  float zero_const;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask_s, uint32_t bits_v) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask_s), "v"(bits_v));
  return r;
}

__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// eight codes of one gfx950-layout word -> bf16x8 of (128 + q), k order
__device__ __forceinline__ bf16x8 unpack8(uint32_t w, uint32_t magic_v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
  r[0] = and_or(w, 0x000F000Fu, magic_v);
  r[1] = and_or(w >> 4, 0x000F000Fu, magic_v);
  r[2] = and_or(w >> 8, 0x000F000Fu, magic_v);
  r[3] = and_or(w >> 12, 0x000F000Fu, magic_v);
  return __builtin_bit_cast(bf16x8, r);
}

// LDS word position of packed-B word `wd` of tile row `n` (XOR swizzle so
// the 32 rows one MFMA operand read touches fall in distinct banks).
__device__ __forceinline__ int b_slot(int n, int wd) { return n * B_LDW + (wd ^ ((n >> 2) & 7)); }

__global__ __launch_bounds__(256, 1) void k_gemm_w4a16(GArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * A_LD];
  __shared__ __attribute__((aligned(16))) uint32_t sb[2][BN * B_LDW];

  // ---- tile order: XCD-aware renumbering, then bands of 8 tile-rows
  const int nwg = p.tiles_m * p.tiles_n;
  int id = blockIdx.x;
  if (nwg % 8 == 0) id = (id % 8) * (nwg / 8) + id / 8;
  const int band = 8;
  const int per_band = band * p.tiles_n;
  const int first_m = (id / per_band) * band;
  const int band_rows = min(band, p.tiles_m - first_m);
  const int tm = first_m + (id % per_band) % band_rows;
  const int tn = (id % per_band) / band_rows;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int rows_a = (int)min((int64_t)BM, p.m - m0);
  const int rows_b = (int)min((int64_t)BN, p.n - n0);
  const int kbytes_a = (int)(p.k * 2);   // bytes per A row
  const int kbytes_b = (int)(p.k / 2);   // bytes per packed B row

  // buffer descriptors over this tile's rows; rows past M / N read as zero
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + m0 * p.k), 0, rows_a * kbytes_a, 0x00020000);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b + n0 * (p.k / 2)), 0, rows_b * kbytes_b, 0x00020000);

  // global -> register staging: A unit u = tid + 256 i (row u/8, 16 B chunk
  // u%8); B unit u = tid + 256 i (row u/2, half u%2)
  const int a_off0 = (tid >> 3) * kbytes_a + (tid & 7) * 16;  // + i * 32 rows
  const int b_off0 = (tid >> 1) * kbytes_b + (tid & 1) * 16;  // + i * 128 rows

  uint4 ra[8], rb[2];
  auto gload = [&](int kt) {
    const int ka = kt * BK * 2, kb = kt * BK / 2;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                  ars, a_off0 + i * 32 * kbytes_a + ka, 0, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                  brs, b_off0 + i * 128 * kbytes_b + kb, 0, 0));
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i, cu = tid & 7;
      *reinterpret_cast<uint4*>(&sa[st][row * A_LD + cu * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 1) + 128 * i, half = tid & 1;
      const uint32_t v4[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) sb[st][b_slot(row, half * 4 + q)] = v4[q];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  float rs[4] = {0.f, 0.f, 0.f, 0.f};  // partial row sums of A (row lane%32, k half lane/32)

  const int nk = (int)(p.k / BK);
  const int lr = lane & 31;   // operand row (A) / column (B) within a 32-block
  const int lh = lane >> 5;   // which 8-k half of the 16-k step
  const uint32_t magic_v = vconst(0x43004300u);
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    WQ_UNROLL(WQ_G_UNROLL)
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + lr;
        af[i] = *reinterpret_cast<const bf16x8*>(&sa[st][row * A_LD + ks * 16 + lh * 8]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + lr;
        bfr[j] = unpack8(sb[st][b_slot(row, ks * 2 + lh)], magic_v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (pairs taken with shufflevector: extracting lanes of a bit-cast
        // u32x4 was folded onto the first dword by this compiler)
        float t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(af[i], af[i], 0, 1), ones, rs[i], false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(af[i], af[i], 2, 3), ones, t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(af[i], af[i], 4, 5), ones, t, false);
        rs[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(af[i], af[i], 6, 7), ones, t, false);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: fold out the offset, scale per column, bf16 RNE, store.
  // Accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32.
  // Row sums: lane l holds row l%32's partial over its k half; add the other half.
  const float zb = 128.f + p.zero_const;
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] += __shfl_xor(rs[i], 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float rsum[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) rsum[e] = __shfl(rs[i], 8 * (e / 4) + 4 * lh + (e % 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + lr;
      const bool cok = col < p.n;
      const float s = cok ? bf16_to_f32(p.scales[col]) : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (e / 4) + 4 * lh + (e % 4);
        const float v = (acc[i][j][e] - zb * rsum[e]) * s;
        if (cok && row < p.m) p.c[row * p.n + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_w4a16(const uint16_t* a, const uint8_t* b, const uint16_t* scales,
                             float zero_const, int64_t m, int64_t n, int64_t k, uint16_t* c,
                             hipStream_t s) {
  GArgs p;
  p.a = a;
  p.b = b;
  p.scales = scales;
  p.c = c;
  p.m = m;
  p.n = n;
  p.k = k;
  p.zero_const = zero_const;
  p.tiles_m = (int)((m + BM - 1) / BM);
  p.tiles_n = (int)((n + BN - 1) / BN);
  const unsigned nwg = (unsigned)(p.tiles_m * p.tiles_n);
  hipLaunchKernelGGL(k_gemm_w4a16, dim3(nwg), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace wq
