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
// fetched into registers while the current step's MFMAs run, then written to
// the other LDS stage.  B stays packed in LDS (4x less LDS traffic than a
// bf16 tile); each wave unpacks its B operands in registers: one 32-bit word
// is exactly the 8 consecutive k one lane feeds to the MFMA, and the codes
// become bf16 (q - z) exactly (|q - z| <= 15 fits bf16 for integer z).
// Workgroups are renumbered so that each XCD (8 on MI355X, dispatched
// round-robin) walks a compact band of output tiles, sharing A and B rows in
// its own L2.
#include "wq_internal.h"

namespace wq {
namespace {

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

// eight codes of one gfx950-layout word -> bf16x8 of (q - z), k order
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float z) {
  uint32_t t = w & 0x0F0F0F0Fu;         // bytes: e0 e4 e1 e5
  uint32_t u = (w >> 4) & 0x0F0F0F0Fu;  // bytes: e2 e6 e3 e7
  float e0 = (float)(t & 0xFFu) - z, e4 = (float)((t >> 8) & 0xFFu) - z;
  float e1 = (float)((t >> 16) & 0xFFu) - z, e5 = (float)(t >> 24) - z;
  float e2 = (float)(u & 0xFFu) - z, e6 = (float)((u >> 8) & 0xFFu) - z;
  float e3 = (float)((u >> 16) & 0xFFu) - z, e7 = (float)(u >> 24) - z;
  bf16x8 r;
  r[0] = (__bf16)e0; r[1] = (__bf16)e1; r[2] = (__bf16)e2; r[3] = (__bf16)e3;
  r[4] = (__bf16)e4; r[5] = (__bf16)e5; r[6] = (__bf16)e6; r[7] = (__bf16)e7;
  return r;
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
  const int64_t kwords = p.k / 8;  // packed words per B row

  // ---- global -> register staging assignment
  // A: 256 rows x 8 units of 16 B; thread handles units tid + 256 i (i < 8)
  // B: 256 rows x 2 units of 16 B; thread handles units tid + 256 i (i < 2)
  const uint16_t* ga[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int u = tid + 256 * i;
    int row = u >> 3, cu = u & 7;
    int64_t gr = min(m0 + row, p.m - 1);
    ga[i] = p.a + gr * p.k + cu * 8;
  }
  const uint32_t* gb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int u = tid + 256 * i;
    int row = u >> 1, half = u & 1;
    int64_t gr = min(n0 + row, p.n - 1);
    gb[i] = reinterpret_cast<const uint32_t*>(p.b) + gr * kwords + half * 4;
  }

  uint4 ra[8], rb[2];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const uint4*>(ga[i] + k0);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = *reinterpret_cast<const uint4*>(gb[i] + k0 / 8);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int u = tid + 256 * i;
      int row = u >> 3, cu = u & 7;
      *reinterpret_cast<uint4*>(&sa[st][row * A_LD + cu * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int u = tid + 256 * i;
      int row = u >> 1, half = u & 1;
      uint32_t v4[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
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

  const int nk = (int)(p.k / BK);
  const float z = p.zero_const;
  const int lr = lane & 31;   // operand row (A) / column (B) within a 32-block
  const int lh = lane >> 5;   // which 8-k half of the 16-k step

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
#pragma unroll
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
        bfr[j] = dequant8(sb[st][b_slot(row, ks * 2 + lh)], z);
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

  // ---- epilogue: per-column scale, bf16 RNE, masked store
  // accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t col = n0 + wn * 128 + j * 32 + lr;
    const bool cok = col < p.n;
    const float s = cok ? bf16_to_f32(p.scales[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (e / 4) + 4 * lh + (e % 4);
        if (cok && row < p.m) p.c[row * p.n + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e] * s);
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
