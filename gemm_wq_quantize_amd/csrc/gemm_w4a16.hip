// W4A16 GEMM on the bf16 matrix cores (gfx950).
//
//   C[i][j] = sum_k A[i][k] * (q[j][k] - z) * s[j][k / group]
//
// (Helion issue "int4 gemm kernel": C = A x unpack(B) with two codes per
// byte along K; here B is stored output-major [N][K/2] in the gfx950 nibble
// order with bf16 scales and a float32 accumulator.  One scale per column
// (group == K) is applied in the epilogue; scales per group of K (the
// weight-only quantiser's group-128 output) are applied to B as it is
// unpacked, see "Group scales" below.)
//
// Tiling.  A 256-lane workgroup computes a 256 x 256 tile of C with four
// waves in a 2 x 2 grid; each wave owns 128 x 128 = 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (with group scales a 1 x 4 grid, 256 x 64 =
// 8 x 2 blocks each, so that every B word is dequantised by one wave).  K advances 64 per step through a three-stage LDS
// ring filled by buffer loads that write LDS directly (no register staging):
// while step t is multiplied, steps t+1 and t+2 are in flight, so one step of
// MFMA work (about 0.85 us) never has to cover a whole memory latency.  B
// stays packed in LDS (4x less LDS traffic than a bf16 tile).
//
// K order inside a 64-k step.  The MFMA sums over its 16 k slots in any
// order, so A and B only have to agree on which k each slot holds.  Lane
// half h of 16-k step s takes the 8 k of chunk 4h + s (chunk = 8 consecutive
// k = one packed B word = 16 bytes of A).  A lane then needs the four packed
// B words 4h .. 4h+3 of a row over the whole step: one ds_read_b128.
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
//
// Group scales (group a multiple of 64, so a 64-k step lies in one group).
// Each step's stage also holds, for every column of the tile, the aligned
// 4-byte word of the scale array that contains s[j][group of the step]
// (one 4-byte buffer-to-LDS load per lane; which half holds the scale
// follows from the parity of j * groups + group).  A lane converts each code
// straight to float32 (a byte convert after one mask), forms
// q * s - z * s = (q - z) * s with one FMA -- exact, the product needs at
// most 17 significant bits -- and rounds the pair to bf16 (RNE) for the
// MFMA.  No row sums are needed; the only rounding beyond the float32
// accumulation is that of (q - z) * s to bf16.  When the constant zero is a
// multiple of 2^-5 below 1024 in magnitude (8 in the quantiser's format) the
// codes come out as fp16 magic numbers instead and v_fma_mix_f32 applies the
// scale, with the same exact results (unpack8_scaled_mix).  This
// dequantisation is about 17 VALU instructions per B word (23 with the byte
// converts), so the waves split the tile by columns:
// each B word is then converted once per workgroup (with 2 x 2 waves, twice)
// at the cost of twice the A fragment reads from LDS.
#include <cmath>

#include "wq_internal.h"

namespace wq {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NSTAGE = 3;
constexpr int A_STAGE = BM * BK * 2;          // bytes: 256 rows x 128 B
constexpr int B_STAGE = BN * BK / 2;          // bytes: 256 rows x 32 B
constexpr int S_STAGE = BN * 4;               // bytes: one scale word per column
// stage size and loads per lane per stage: 40 KiB and 10 (8 A + 2 B) with
// one scale per column; 41 KiB and 11 (+1 scale word) with group scales
// (stored zeros with group scales, GZ: one more word per column and load)
template <bool GS, bool GZ> constexpr int stage_bytes() {
  return A_STAGE + B_STAGE + (GS ? S_STAGE : 0) + (GZ ? S_STAGE : 0);
}
template <bool GS, bool GZ> constexpr int loads_per_stage() { return 10 + (GS ? 1 : 0) + (GZ ? 1 : 0); }


struct GArgs {
  const uint16_t* a;
  const uint8_t* b;
  const uint16_t* scales;
  const uint16_t* zeros;  // nullable: [n] or [n][k/group] bf16 zero points
  uint16_t* c;
  int64_t m, n, k;
  float zero_const;
  int tiles_m, tiles_n;
  int ngroups;   // k / group
  int gshift;    // log2(group / 64): step t lies in group t >> gshift
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

// byte b of v as float32: v_cvt_f32_ubyte{0..3} (written out: the compiler
// otherwise extracts the byte with a separate v_bfe_u32)
__device__ __forceinline__ float cvt_ubyte(uint32_t v, int b) {
  float r;
  if (b == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
  else if (b == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
  else if (b == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// eight codes of one gfx950-layout word -> bf16x8 of (q - z) * s, k order,
// with c = -z * s.  Nibble p holds element {0,2,4,6,1,3,5,7}[p]; the even
// nibbles masked in place are the bytes of elements 0, 4, 1, 5, the odd ones
// shifted down those of 2, 6, 3, 7, and each byte converts to float with one
// v_cvt_f32_ubyteN.  q * s + c is exact in float32 (bf16 s, and z an integer
// or bf16, so z * s and the sum need at most 17 significant bits), so the
// only rounding is the one to bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 unpack8_scaled(uint32_t w, float s, float c) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t ev = w & 0x0F0F0F0Fu;         // bytes: elements 0, 4, 1, 5
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;  // bytes: elements 2, 6, 3, 7
  auto ub = [](uint32_t v, int b) { return cvt_ubyte(v, b); };
  const float e[8] = {ub(ev, 0), ub(ev, 2), ub(od, 0), ub(od, 2), ub(ev, 1), ub(ev, 3), ub(od, 1), ub(od, 3)};
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f2 v = {fmaf(e[2 * j], s, c), fmaf(e[2 * j + 1], s, c)};
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
  }
  return __builtin_bit_cast(bf16x8, r);
}

// The same eight weights with the codes taken as fp16 magic numbers: a nibble
// masked into the low mantissa bits under 0x6400 (1024) reads 1024 + q, one
// masked into bits 4..7 reads 1024 + 16 q, so four v_and_or_b32 and one
// shift give all eight codes as fp16 halves, and v_fma_mix_f32 (fp16 source,
// fp32 scale and addend) forms (1024 + q) * s + c0 and (1024 + 16 q) * s/16 +
// c1 with c0 = -(1024 + z) * s and c1 = -(64 + z) * s.  Both equal (q - z) * s
// exactly when z is a multiple of 2^-5 below 1024 in magnitude (the products
// need at most 19 significant bits and the addends at most 24), so the
// results are those of unpack8_scaled: 17 VALU instructions per word instead
// of 23.
__device__ __forceinline__ bf16x8 unpack8_scaled_mix(uint32_t w, float s, float s16, float c0, float c1,
                                                     uint32_t magic_v) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t t = w >> 8;
  const h2 p[4] = {__builtin_bit_cast(h2, and_or(w, 0x000F000Fu, magic_v)),   // elements 0, 1
                   __builtin_bit_cast(h2, and_or(w, 0x00F000F0u, magic_v)),   // 2, 3 (x 16)
                   __builtin_bit_cast(h2, and_or(t, 0x000F000Fu, magic_v)),   // 4, 5
                   __builtin_bit_cast(h2, and_or(t, 0x00F000F0u, magic_v))};  // 6, 7 (x 16)
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sj = (j & 1) ? s16 : s, cj = (j & 1) ? c1 : c0;
    const f2 v = {fmaf((float)p[j].x, sj, cj), fmaf((float)p[j].y, sj, cj)};
    r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
  }
  return __builtin_bit_cast(bf16x8, r);
}

// A-tile swizzle: physical 16-byte column of k-chunk c in row r is c ^ swz(r)
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// VALU instructions placed after each MFMA by the scheduling groups with
// group scales: three with the byte converts (5% faster than four or two,
// 8192^3 group 128), two with the fp16-magic dequantisation (0.5% faster
// than three, 2% faster than four)
template <bool MX> constexpr int g_vpm() { return MX ? 2 : 3; }

// Epilogue staging: half the tile (128 rows x 256 bf16) at a time, rows
// padded by 16 bytes so that the two rows one 2-byte LDS write touches (4
// apart) fall in different banks.
constexpr int C_PITCH = BN * 2 + 16;
static_assert(128 * C_PITCH <= NSTAGE * stage_bytes<false, false>(), "epilogue staging fits the ring");

// One workgroup tile.  WN (the wave's column half) is a template argument so
// that the row-sum split below indexes fragments at compile time; GS selects
// group scales (applied while unpacking B) over one scale per column
// (applied in the epilogue).
template <int WN, bool GS, bool GZ, bool MX>
__device__ __forceinline__ void gemm_tile(const GArgs& p, uint8_t* smem, float (*rsx)[4][32]) {
  static_assert(GS || !GZ, "stored zeros of groups come with group scales");
  static_assert(!MX || (GS && !GZ), "the fp16-magic dequantisation serves group scales with a constant zero");
  constexpr int STAGE = stage_bytes<GS, GZ>();
  constexpr int LOADS_PER_STAGE = loads_per_stage<GS, GZ>();
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave grid: 2 x 2 (128 x 128 each) with one scale per column; 1 x 4 (256
  // rows x 64 columns each) with group scales, so that each B word is
  // dequantised by one wave only
  constexpr int MI = GS ? 8 : 4;  // 32-row blocks per wave
  constexpr int NJ = GS ? 2 : 4;  // 32-column blocks per wave
  const int wm = GS ? 0 : wave >> 1;
  const int col0 = GS ? wave * 64 : WN * 128;  // the wave's first column in the tile
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int rows_a = (int)min((int64_t)BM, p.m - m0);
  const int rows_b = (int)min((int64_t)BN, p.n - n0);
  const uint32_t kbytes_a = (uint32_t)(p.k * 2);   // bytes per A row
  const uint32_t kbytes_b = (uint32_t)(p.k / 2);   // bytes per packed B row

  // descriptors over this tile's rows; rows past M / N read as zero
  const intx4 ars = make_rsrc(p.a + m0 * p.k, (uint32_t)rows_a * kbytes_a);
  const intx4 brs = make_rsrc(p.b + n0 * (p.k / 2), (uint32_t)rows_b * kbytes_b);
  // group scales of this tile's columns, [rows_b][ngroups] bf16.  The range
  // is rounded up to whole 4-byte words: the base is 4-byte aligned, so the
  // word holding the last scale is one the caller's array already touches
  // (and cannot cross a page); the half past the array is never used.
  const intx4 srs = make_rsrc(GS ? (const void*)(p.scales + n0 * p.ngroups) : (const void*)p.scales,
                              GS ? (((uint32_t)rows_b * (uint32_t)p.ngroups * 2u + 3u) & ~3u) : 0u);
  // stored zeros of the groups: the same layout, read the same way
  const intx4 zrs = make_rsrc(GZ ? (const void*)(p.zeros + n0 * p.ngroups) : (const void*)p.scales,
                              GZ ? (((uint32_t)rows_b * (uint32_t)p.ngroups * 2u + 3u) & ~3u) : 0u);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  // ---- global -> LDS assignment.  Load i (0..7) of wave w fills A slots
  // (16 B each) s = 64 (4 i + w) + lane: row s / 8, slot column s % 8
  // holding k-chunk (s % 8) ^ swz(row).  The LDS serves 16 lanes of a
  // ds_read_b128 per cycle from 64 banks; the 16 rows those lanes read
  // (same chunk) then fall on 16 distinct 16-byte bank groups.  Loads 8, 9
  // fill B slots laid out [half][row]: half h = load - 8, row 64 w + lane.
  uint32_t a_voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int row = s >> 3, chunk = (s & 7) ^ swz(row);
    a_voff[i] = (uint32_t)row * kbytes_a + (uint32_t)chunk * 16;
  }
  // B load h of wave w fills slots 64 (4 h + w) + lane of the B stage laid
  // out [row][half ^ ((row / 8) % 2)] (16 B each): row s / 2, stored half
  // s % 2.  The half swap keeps the 16 rows one B read touches in distinct
  // bank groups.
  uint32_t b_voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int s = (h * 4 + wave) * 64 + lane;
    const int row = s >> 1, half = (s & 1) ^ ((row >> 3) & 1);
    b_voff[h] = (uint32_t)row * kbytes_b + (uint32_t)half * 16;
  }
  // scale word of wave w, lane l: column 64 w + l
  const uint32_t s_voff = (uint32_t)((wave * 64 + lane) * p.ngroups) * 2u;
  const int nk = (int)(p.k / BK);

  // Step kt's loads into stage kt % 3.  Steps past the end are issued too
  // (the loop then has no branch) but at offset 2^31 or more, which is past
  // num_records: they read nothing from memory and fill an unused stage with
  // zeros.
  // loads [first, last) of step kt: 0..7 are A, 8 and 9 are B, 10 the
  // group scales, 11 the group zeros
  auto issue_part = [&](int kt, int first, int last) {
    const uint32_t st = lds0 + (uint32_t)(kt % NSTAGE) * STAGE;
    const bool live = kt < nk;
    const uint32_t ka = live ? (uint32_t)kt * (BK * 2) : 0x80000000u;
    const uint32_t kb = live ? (uint32_t)kt * (BK / 2) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i >= first && i < last)
        dma16(ars, a_voff[i] + ka,
              __builtin_amdgcn_readfirstlane(st + (uint32_t)(i * 4 + wave) * 1024));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (8 + h >= first && 8 + h < last)
        dma16(brs, b_voff[h] + kb,
              __builtin_amdgcn_readfirstlane(st + A_STAGE + (uint32_t)(h * 4 + wave) * 1024));
    if (GS && 10 >= first && 10 < last) {
      const uint32_t so = live ? ((s_voff + (uint32_t)(kt >> p.gshift) * 2u) & ~3u) : 0x80000000u;
      dma4(srs, so, __builtin_amdgcn_readfirstlane(st + A_STAGE + B_STAGE + (uint32_t)wave * 256));
    }
    if (GZ && 11 >= first && 11 < last) {
      const uint32_t so = live ? ((s_voff + (uint32_t)(kt >> p.gshift) * 2u) & ~3u) : 0x80000000u;
      dma4(zrs, so, __builtin_amdgcn_readfirstlane(st + A_STAGE + B_STAGE + S_STAGE + (uint32_t)wave * 256));
    }
  };
  auto issue = [&](int kt) { issue_part(kt, 0, LOADS_PER_STAGE); };
  // Every group of loads inside the loop sits between full scheduling
  // barriers.  Without them, the scheduling-group ordering in compute()
  // (sched_group_barrier) let this compiler move code across the asm loads
  // such that some tiles came out wrong; with them the loads keep their
  // place in program order.
  auto issue_fenced = [&](int kt, int first, int last) {
    __builtin_amdgcn_sched_barrier(0);
    issue_part(kt, first, last);
    __builtin_amdgcn_sched_barrier(0);
  };

  floatx16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // Row sums of A: this wave sums row blocks 2 WN and 2 WN + 1 only (the
  // wave of the other column half sums the other two); lane l holds row
  // l%32's partial over k half l/32.
  // Four independent accumulators per block: a chain of dependent v_dot2
  // would stall this wave's in-order issue, MFMAs included.
  float rsq[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  const int lr = lane & 31;   // operand row (A) / column (B) within a 32-block
  const int lh = lane >> 5;   // k half: chunks 4 lh .. 4 lh + 3 of every step
  const uint32_t magic_v = vconst(MX ? 0x64006400u : 0x43004300u);
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);

  // LDS byte offsets (within a stage) of this lane's operands
  int a_rd[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) a_rd[i] = (wm * 128 + i * 32 + lr) * 128;
  const int a_sw = swz(lr);  // == swz(row) for all four rows
  int b_rd[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = col0 + j * 32 + lr;
    b_rd[j] = A_STAGE + (n * 2 + (lh ^ ((lr >> 3) & 1))) * 16;
  }

  auto read_b = [&](int kt, uint4 (&bw)[NJ]) {
    const uint8_t* st = smem + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int j = 0; j < NJ; ++j) bw[j] = *reinterpret_cast<const uint4*>(st + b_rd[j]);
  };
  // group scales (and zeros) of this lane's four columns for step kt (raw words)
  auto read_s = [&](int kt, uint32_t (&sw)[NJ], uint32_t (&zw)[NJ]) {
    const uint8_t* st = smem + (kt % NSTAGE) * STAGE + A_STAGE + B_STAGE;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sw[j] = *reinterpret_cast<const uint32_t*>(st + (col0 + j * 32 + lr) * 4);
      zw[j] = GZ ? *reinterpret_cast<const uint32_t*>(st + S_STAGE + (col0 + j * 32 + lr) * 4) : 0u;
    }
  };
  // word -> float scale and offset term: the scale of column n for group g
  // is the high half when n * groups + g is odd (n and lr share parity)
  const float zb = 128.f + p.zero_const;
  const float zm0 = -(1024.f + p.zero_const), zm1 = -(64.f + p.zero_const);  // exact when MX
  float gsc[NJ], gof[NJ], gsc16[NJ], gof16[NJ];
  auto set_s = [&](int kt, const uint32_t (&sw)[NJ], const uint32_t (&zw)[NJ]) {
    const bool hi = (((lr & p.ngroups) ^ (kt >> p.gshift)) & 1) != 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      gsc[j] = __uint_as_float(hi ? (sw[j] & 0xFFFF0000u) : (sw[j] << 16));
      if constexpr (MX) {
        gsc16[j] = gsc[j] * 0.0625f;
        gof[j] = zm0 * gsc[j];
        gof16[j] = zm1 * gsc[j];
      } else {
        const float z = GZ ? __uint_as_float(hi ? (zw[j] & 0xFFFF0000u) : (zw[j] << 16)) : p.zero_const;
        gof[j] = -z * gsc[j];
      }
    }
  };
  auto read_a = [&](int kt, int ks, bf16x8 (&af)[MI]) {
    const uint8_t* st = smem + (kt % NSTAGE) * STAGE;
    const int chunk = lh * 4 + ks;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(st + a_rd[i] + ((chunk ^ a_sw) << 4));
  };
  auto compute = [&](const bf16x8 (&af)[MI], const uint4 (&bw)[NJ], int ks) {
    bf16x8 bfr[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t w = ks == 0 ? bw[j].x : ks == 1 ? bw[j].y : ks == 2 ? bw[j].z : bw[j].w;
      bfr[j] = unpack8(w, magic_v);
    }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const bf16x8 x = af[2 * WN + ii];
      // (pairs taken with shufflevector: extracting lanes of a bit-cast
      // u32x4 was folded onto the first dword by this compiler)
      rsq[ii][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), ones, rsq[ii][0], false);
      rsq[ii][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), ones, rsq[ii][1], false);
      rsq[ii][2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), ones, rsq[ii][2], false);
      rsq[ii][3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), ones, rsq[ii][3], false);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      if (t < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  };
  // Group scales: slice ks of the step's B words dequantised ahead of use
  // (dq), so the 16 MFMAs of one slice (mm) overlap the VALU work of the next.
  auto dq = [&](const uint4 (&bw)[NJ], int ks, bf16x8 (&bfr)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t w = ks == 0 ? bw[j].x : ks == 1 ? bw[j].y : ks == 2 ? bw[j].z : bw[j].w;
      bfr[j] = MX ? unpack8_scaled_mix(w, gsc[j], gsc16[j], gof[j], gof16[j], magic_v)
                  : unpack8_scaled(w, gsc[j], gof[j]);
    }
  };
  auto mm = [&](const bf16x8 (&af)[MI], const bf16x8 (&bfr)[NJ]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < MI * NJ; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, g_vpm<MX>(), 0);  // VALU
      if (t < MI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  };

  // ---- main loop.  Barrier b(t) publishes stage t (its loads landed) and
  // frees stage t - 1 (every wave has read it), after which step t + 2 is
  // issued into it.  b(t + 1) sits before the last 16-k group of step t, so
  // that step t + 1's first operands are read while that group multiplies.
  // Step t's loads go out in three groups: 0-3 right after b(t - 2), 4-6
  // and 7-9 (and the scale word) between the 16-k groups of step t - 2 (a
  // burst of ten would stall this wave's MFMA issue).  All loads of step
  // t + 2 precede the wait before b(t + 1), so that wait (at most one step
  // of loads in flight) covers step t + 1.
  asm volatile("s_nop 4");  // VALU-written SGPRs (descriptors) read by the first loads
  issue(0);
  issue(1);
  wait_vmcnt<LOADS_PER_STAGE>();
  __syncthreads();
  issue_fenced(2, 0, 4);
  uint4 bw[NJ];
  bf16x8 a0[MI], a1[MI];
  read_b(0, bw);
  if constexpr (GS) {
    uint32_t sw[NJ], zw[NJ];
    bf16x8 b0[NJ], b1[NJ];
    read_s(0, sw, zw);
    set_s(0, sw, zw);
    read_a(0, 0, a0);
    dq(bw, 0, b0);
    for (int kt = 0; kt < nk; ++kt) {
      read_a(kt, 1, a1);
      dq(bw, 1, b1);
      mm(a0, b0);
      issue_fenced(kt + 2, 4, 7);
      read_a(kt, 2, a0);
      dq(bw, 2, b0);
      mm(a1, b1);
      issue_fenced(kt + 2, 7, LOADS_PER_STAGE);
      read_a(kt, 3, a1);
      dq(bw, 3, b1);
      mm(a0, b0);
      wait_vmcnt<LOADS_PER_STAGE>();
      __syncthreads();
      issue_fenced(kt + 3, 0, 4);
      read_b(kt + 1, bw);  // bw's slices are all dequantised by now
      read_s(kt + 1, sw, zw);
      read_a(kt + 1, 0, a0);
      set_s(kt + 1, sw, zw);
      dq(bw, 0, b0);
      mm(a1, b1);
    }
  } else {
    read_a(0, 0, a0);
    for (int kt = 0; kt < nk; ++kt) {
      read_a(kt, 1, a1);
      compute(a0, bw, 0);
      issue_fenced(kt + 2, 4, 7);
      read_a(kt, 2, a0);
      compute(a1, bw, 1);
      issue_fenced(kt + 2, 7, LOADS_PER_STAGE);
      read_a(kt, 3, a1);
      compute(a0, bw, 2);
      // a1 holds the last operands read from stage kt (the barrier's release
      // waits for them); stage kt + 1 landed once only step kt + 2 is in flight
      wait_vmcnt<LOADS_PER_STAGE>();
      __syncthreads();
      issue_fenced(kt + 3, 0, 4);
      uint4 bn[NJ];
      read_b(kt + 1, bn);
      read_a(kt + 1, 0, a0);
      compute(a1, bw, 3);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bw[j] = bn[j];
    }
  }
  wait_vmcnt<0>();  // no load may still be writing LDS below

  // ---- row sums: complete the k halves, swap halves of the row blocks
  // with the other column half's wave through LDS.
#pragma unroll
  for (int ii = 0; ii < 2 && !GS; ++ii) {
    float r = (rsq[ii][0] + rsq[ii][1]) + (rsq[ii][2] + rsq[ii][3]);
    r += __shfl_xor(r, 32);
    if (lh == 0) rsx[wm][2 * WN + ii][lr] = r;
  }
  __syncthreads();  // also: every wave is done with the ring

  // ---- epilogue: fold out the offset, scale per column (both already in
  // the accumulator with group scales), bf16 RNE; stage half the tile in
  // LDS, then write it with coalesced 16-byte stores.
  // Accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32.
  float sc[NJ], zc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t col = n0 + col0 + j * 32 + lr;
    sc[j] = GS ? 1.f : (col < p.n ? bf16_to_f32(p.scales[col]) : 0.f);
    zc[j] = (!GS && p.zeros && col < p.n) ? 128.f + bf16_to_f32(p.zeros[col]) : zb;
  }
  const bool vec_ok = (p.n & 7) == 0;  // rows 16-byte aligned
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < MI / 2; ++ii) {
      const int i = MI / 2 * half + ii;
      float rsum[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 v = GS ? floatx4{0.f, 0.f, 0.f, 0.f}
                             : *reinterpret_cast<const floatx4*>(&rsx[wm][i & 3][8 * g + 4 * lh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) rsum[4 * g + e] = v[e];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = col0 + j * 32 + lr;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          // staged row: 64 wm + 32 ii + local row (wm = 0 with group scales)
          const int srow = wm * 64 + ii * 32 + 8 * (e / 4) + 4 * lh + (e % 4);
          const float v = GS ? acc[i][j][e] : (acc[i][j][e] - zc[j] * rsum[e]) * sc[j];
          *reinterpret_cast<uint16_t*>(smem + srow * C_PITCH + col * 2) =
              (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
    __syncthreads();
    // 128 staged rows x 32 chunks of 16 B; thread t takes chunks t + 256 u
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int q = tid + 256 * u;
      const int srow = q >> 5, cch = q & 31;
      const int64_t row = GS ? m0 + half * 128 + srow : m0 + (srow >> 6) * 128 + half * 64 + (srow & 63);
      const int64_t col = n0 + cch * 8;
      if (row >= p.m || col >= p.n) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(smem + srow * C_PITCH + cch * 16);
      uint16_t* dst = p.c + row * p.n + col;
      if (vec_ok && col + 8 <= p.n) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int t = 0; t < 8 && col + t < p.n; ++t) dst[t] = (uint16_t)(w[t / 2] >> (16 * (t % 2)));
      }
    }
    if (half == 0) __syncthreads();  // staging is rewritten by the second half
  }
}

template <bool GS, bool GZ, bool MX>
__global__ __launch_bounds__(256, 1) void k_gemm_w4a16(GArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * stage_bytes<GS, GZ>()];
  __shared__ __attribute__((aligned(16))) float rsx[2][4][32];  // row sums [wm][row block][row]
  // wave-uniform branch (the wave index is moved to a scalar register)
  if constexpr (GS) gemm_tile<0, GS, GZ, MX>(p, smem, rsx);
  else if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) gemm_tile<1, GS, GZ, MX>(p, smem, rsx);
  else gemm_tile<0, GS, GZ, MX>(p, smem, rsx);
}

}  // namespace

hipError_t launch_gemm_w4a16(const uint16_t* a, const uint8_t* b, const uint16_t* scales,
                             const uint16_t* zeros, int64_t group, float zero_const, int64_t m,
                             int64_t n, int64_t k, uint16_t* c, hipStream_t s) {
  GArgs p;
  p.a = a;
  p.b = b;
  p.scales = scales;
  p.zeros = zeros;
  p.c = c;
  p.m = m;
  p.n = n;
  p.k = k;
  p.zero_const = zero_const;
  p.tiles_m = (int)((m + BM - 1) / BM);
  p.tiles_n = (int)((n + BN - 1) / BN);
  p.ngroups = (int)(k / group);
  p.gshift = 0;
  while ((int64_t(BK) << p.gshift) < group) ++p.gshift;
  const unsigned nwg = (unsigned)(p.tiles_m * p.tiles_n);
  // the fp16-magic dequantisation needs z a multiple of 2^-5 with |z| < 1024
  const float zs = zero_const * 32.f;
  const bool mix = std::fabs(zero_const) < 1024.f && zs == std::nearbyint(zs);
  if (group == k)
    hipLaunchKernelGGL((k_gemm_w4a16<false, false, false>), dim3(nwg), dim3(256), 0, s, p);
  else if (zeros)
    hipLaunchKernelGGL((k_gemm_w4a16<true, true, false>), dim3(nwg), dim3(256), 0, s, p);
  else if (mix)
    hipLaunchKernelGGL((k_gemm_w4a16<true, false, true>), dim3(nwg), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm_w4a16<true, false, false>), dim3(nwg), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace wq
