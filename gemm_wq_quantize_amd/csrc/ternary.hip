// Ternary path (gfx950): PTQ1_0 block packing, the q8_1 activation
// quantiser and the ternary x int8 GEMV.
//
// Formats: Ternary post, section 2 (struct ptq1_0: qs[24] with 120 trits,
// qh[2] with 8 trits, fp16 d), section 3.1 (block_q8_1: fp16 d, fp16 s,
// int8 qs[32]) and section 3.2 (trit placement: element e < 80 is digit
// e >> 4 of byte e & 15; element 80 + e is digit e >> 3 of byte 16 + (e & 7);
// the last 8 are 2-bit fields of qh).  A trit t is stored as the digit
// u = t + 1, a qs byte is sum_j u_j 3^j (digit 0 least significant), and
// tail element 120 + e sits in qh[e & 1] at bits 2 * (e >> 1).
//
// GEMV: y[j][r] = sum_b d_w[r][b/4] * d_x[j][b] * S[r][j][b] with exact int32
// sub-block sums S = sum_{i<32} t * q = sum u * q - sum q (v_dot4 on digits),
// the per-block sums of q taken from the int8 data, never from the fp16 s.
#include "wq_internal.h"

#include <mutex>

#include <algorithm>

namespace wq {
namespace {

constexpr int PT_BYTES = 28;
constexpr int Q8_BYTES = 36;

// Activations come in one of two layouts, chosen at compile time (PT) so
// that each kernel's record-order build is unchanged by the other.  A column
// of x is nsb = k / 32 block_q8_1 records (36 bytes each) in record order.
// In the PT layout (Ternary post, section 3.1) the same bytes are regrouped:
// block sb is sub-block j = sb & 3 of 128-element block i = sb >> 2, its q
// fill slot i of planes 2 j and 2 j + 1 (k / 128 slots of 16 bytes per
// plane) and its (d, s) word is word j of slot i of plane 8.  Both layouts
// take 36 bytes per block, so columns start at the same offsets.
//
// Byte offsets of block sb from its column's start in the PT layout: its
// (d, s) word, q[0..15] and q[16..31].
struct XBlk {
  uint32_t ds, q0, q1;
};
__device__ __forceinline__ XBlk pt_block(int nsb, int sb) {
  const int nb = nsb >> 2, i = sb >> 2, j = sb & 3;
  return {(uint32_t)(16 * (8 * nb + i) + 4 * j), (uint32_t)(16 * (2 * j * nb + i)),
          (uint32_t)(16 * ((2 * j + 1) * nb + i))};
}

// The nine words of block sb of column col, (d, s) first.
template <bool PT>
__device__ __forceinline__ void xq_load(const uint8_t* __restrict__ xq, int64_t col, int nsb, int64_t sb,
                                        uint32_t& hd, uint32_t (&q)[8]) {
  if constexpr (PT) {
    const uint8_t* cb = xq + col * nsb * Q8_BYTES;
    const XBlk xb = pt_block(nsb, (int)sb);
    hd = *reinterpret_cast<const uint32_t*>(cb + xb.ds);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = *reinterpret_cast<const uint32_t*>(cb + xb.q0 + 4 * i);
      q[4 + i] = *reinterpret_cast<const uint32_t*>(cb + xb.q1 + 4 * i);
    }
  } else {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(xq + (col * nsb + sb) * Q8_BYTES);
    hd = src[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = src[1 + i];
  }
}

// ---------------------------------------------------------------- packing
__global__ __launch_bounds__(256) void k_pack_ptq1_0(const int8_t* __restrict__ trits,
                                                     const uint16_t* __restrict__ d,
                                                     uint32_t* __restrict__ blocks,
                                                     int64_t nblocks) {
  int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(trits + b * 128);
  uint32_t u[128];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 v = src[i];
    uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) u[16 * i + 4 * q + e] = (uint32_t)((int)(int8_t)(w4[q] >> (8 * e)) + 1);
  }
  uint32_t bytes[26];
#pragma unroll
  for (int i = 0; i < 16; ++i)  // byte i: elements i + 16 j
    bytes[i] = u[i] + 3 * u[i + 16] + 9 * u[i + 32] + 27 * u[i + 48] + 81 * u[i + 64];
#pragma unroll
  for (int i = 0; i < 8; ++i)  // byte 16 + i: elements 80 + i + 8 j
    bytes[16 + i] = u[80 + i] + 3 * u[88 + i] + 9 * u[96 + i] + 27 * u[104 + i] + 81 * u[112 + i];
  bytes[24] = u[120] | u[122] << 2 | u[124] << 4 | u[126] << 6;
  bytes[25] = u[121] | u[123] << 2 | u[125] << 4 | u[127] << 6;
  uint32_t* dst = blocks + b * 7;
#pragma unroll
  for (int i = 0; i < 6; ++i)
    dst[i] = bytes[4 * i] | bytes[4 * i + 1] << 8 | bytes[4 * i + 2] << 16 | bytes[4 * i + 3] << 24;
  dst[6] = bytes[24] | bytes[25] << 8 | (uint32_t)d[b] << 16;
}

// ---------------------------------------------------------------- q8_1
// One 32-lane team per block of 32 activations.
template <bool PT>
__global__ __launch_bounds__(256) void k_quantize_q8_1(const float* __restrict__ x,
                                                       uint8_t* __restrict__ out,
                                                       int64_t nblocks, int nsb) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = gid >> 5;
  const int lane = threadIdx.x & 31;
  const bool active = b < nblocks;
  const float v = active ? x[gid] : 0.f;
  float amax = fabsf(v);
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const uint32_t dbits = f32_to_f16_rne(amax / 127.0f);  // IEEE divide, RNE to fp16
  const float dv = f16_to_f32(dbits);
  int q = 0;
  if (dv != 0.f) {
    float r = rintf(v / dv);
    r = fminf(fmaxf(r, -127.f), 127.f);
    q = (int)r;
  }
  int qs = q;
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) qs += __shfl_xor(qs, off);
  if (!active) return;
  uint8_t* blk = out + b * Q8_BYTES;  // the record (record order)
  uint32_t* dsw = reinterpret_cast<uint32_t*>(blk);
  if constexpr (PT) {                 // the column's planes
    const int64_t col = b / nsb;
    uint8_t* cb = out + col * nsb * Q8_BYTES;
    const XBlk xb = pt_block(nsb, (int)(b - col * nsb));
    cb[(lane < 16 ? xb.q0 : xb.q1) + (lane & 15)] = (uint8_t)(int8_t)q;
    dsw = reinterpret_cast<uint32_t*>(cb + xb.ds);
  } else {
    blk[4 + lane] = (uint8_t)(int8_t)q;
  }
  if (lane == 0) {
    const uint32_t sbits = f32_to_f16_rne(dv * (float)qs);
    *dsw = dbits | sbits << 16;
  }
}

// ---------------------------------------------------------------- GEMV
// Lane layout: a wave covers 8 rows x 8 consecutive blocks (1024 k) per
// tile; a 256-lane workgroup covers 32 rows.  The activation tile (int8 q in
// k order, plus per-32 d and sum q) is staged in LDS once per workgroup.
//
// Digit decode: a 243-entry LDS table maps a qs byte to its digits u0..u3 in
// bytes 0..3 and u4 in bits 4-5 of byte 0.  Four table words (four
// consecutive qs bytes b..b+3, one digit position j each = elements
// 16j + b .. 16j + b + 3) are transposed with v_perm so each dword holds one
// digit position of four neighbouring bytes -- exactly four consecutive
// elements, which v_dot4 multiplies with four consecutive int8 activations.
constexpr int T_BLOCKS = 8;              // blocks per lane-row per tile
constexpr int T_K = T_BLOCKS * 128;      // 1024 k per tile
constexpr int T_SUB = T_K / 32;          // 32 activation blocks per tile

__device__ __forceinline__ void transpose4(uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3,
                                           uint32_t& d0, uint32_t& d1, uint32_t& d2,
                                           uint32_t& d3, uint32_t& d4) {
  // perm(hi, lo, sel): selector bytes 0-3 pick lo's bytes, 4-7 pick hi's
  const uint32_t a = __builtin_amdgcn_perm(l1, l0, 0x05010400u);  // l0b0 l1b0 l0b1 l1b1
  const uint32_t b = __builtin_amdgcn_perm(l3, l2, 0x05010400u);  // l2b0 l3b0 l2b1 l3b1
  const uint32_t c = __builtin_amdgcn_perm(l1, l0, 0x07030602u);  // l0b2 l1b2 l0b3 l1b3
  const uint32_t e = __builtin_amdgcn_perm(l3, l2, 0x07030602u);  // l2b2 l3b2 l2b3 l3b3
  const uint32_t r0 = __builtin_amdgcn_perm(b, a, 0x05040100u);   // byte0 of l0..l3
  d0 = r0 & 0x03030303u;
  d4 = (r0 >> 4) & 0x03030303u;
  d1 = __builtin_amdgcn_perm(b, a, 0x07060302u);
  d2 = __builtin_amdgcn_perm(e, c, 0x05040100u);
  d3 = __builtin_amdgcn_perm(e, c, 0x07060302u);
}

template <int C, bool PT>
__global__ __launch_bounds__(256) void k_gemv_ternary(const uint32_t* __restrict__ w,
                                                      const uint8_t* __restrict__ xq,
                                                      float* __restrict__ out, int64_t n,
                                                      int64_t k, int c) {
  __shared__ uint32_t lut[256];
  __shared__ uint4 xs[C * T_K / 16];      // int8 q, k order, per column
  __shared__ int xsum[C * T_SUB];         // sum of q per activation block
  __shared__ float xd[C * T_SUB];         // d per activation block

  const int tid = threadIdx.x;
  {
    uint32_t v = tid, ent = 0;
    uint32_t u0 = v % 3, u1 = (v / 3) % 3, u2 = (v / 9) % 3, u3 = (v / 27) % 3, u4 = (v / 81) % 3;
    ent = u0 | u1 << 8 | u2 << 16 | u3 << 24 | u4 << 4;
    lut[tid] = ent;  // entries >= 243 are never indexed by valid data
  }

  const int lane = tid & 63;
  const int sub = lane & 7;                 // block within the tile
  const int64_t row0 = (int64_t)blockIdx.x * 32 + (tid >> 6) * 8 + (lane >> 3);
  const int64_t row = min(row0, n - 1);
  const int64_t bpr = k / 128;              // blocks per row
  const int ntiles = (int)((bpr + T_BLOCKS - 1) / T_BLOCKS);

  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int64_t blk = (int64_t)t * T_BLOCKS + sub;
    const bool valid = blk < bpr;
    uint32_t wd[7];
    const uint32_t* src = w + (row * bpr + (valid ? blk : 0)) * 7;
#pragma unroll
    for (int i = 0; i < 7; ++i) wd[i] = src[i];

    __syncthreads();
    // stage: C columns x 32 activation blocks; one lane per (column, block)
    for (int idx = tid; idx < C * T_SUB; idx += 256) {
      const int col = idx / T_SUB, sb = idx % T_SUB;
      const int64_t gsb = (int64_t)t * T_SUB + sb;  // activation block index in the row
      uint32_t q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      uint32_t hd = 0;
      if (col < c && gsb < k / 32) {
        if constexpr (PT) {
          xq_load<true>(xq, col, (int)(k / 32), gsb, hd, q);
        } else {
          const uint32_t* s = reinterpret_cast<const uint32_t*>(xq + ((int64_t)col * (k / 32) + gsb) * Q8_BYTES);
          hd = s[0];
#pragma unroll
          for (int i = 0; i < 8; ++i) q[i] = s[1 + i];
        }
      }
      uint4* dst = &xs[(col * T_K + sb * 32) / 16];
      dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
      dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum = __builtin_amdgcn_sdot4((int)q[i], 0x01010101, sum, false);
      xsum[col * T_SUB + sb] = sum;
      xd[col * T_SUB + sb] = f16_to_f32(hd & 0xFFFFu);
    }
    __syncthreads();

    if (valid) {
      // decode the 128 digits into 32 dwords in k order (dw[i] = elements 4i..4i+3)
      uint32_t dg[32];
      // section 1: qs bytes 0..15, element 16 j + b
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t v = wd[g];
        const uint32_t l0 = lut[v & 0xFF], l1 = lut[(v >> 8) & 0xFF];
        const uint32_t l2 = lut[(v >> 16) & 0xFF], l3 = lut[v >> 24];
        uint32_t d0, d1, d2, d3, d4;
        transpose4(l0, l1, l2, l3, d0, d1, d2, d3, d4);
        dg[g] = d0; dg[4 + g] = d1; dg[8 + g] = d2; dg[12 + g] = d3; dg[16 + g] = d4;
      }
      // section 2: qs bytes 16..23, element 80 + 8 j + b
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t v = wd[4 + g];
        const uint32_t l0 = lut[v & 0xFF], l1 = lut[(v >> 8) & 0xFF];
        const uint32_t l2 = lut[(v >> 16) & 0xFF], l3 = lut[v >> 24];
        uint32_t d0, d1, d2, d3, d4;
        transpose4(l0, l1, l2, l3, d0, d1, d2, d3, d4);
        dg[20 + g] = d0; dg[22 + g] = d1; dg[24 + g] = d2; dg[26 + g] = d3; dg[28 + g] = d4;
      }
      // qh: elements 120..127; h bits 2e' of byte (e' & 1) -> digit of 120 + e'
      {
        const uint32_t h = wd[6] & 0xFFFFu;
        dg[30] = (h | (h << 14)) & 0x03030303u;
        dg[31] = ((h >> 4) | (h << 10)) & 0x03030303u;
      }
      const float dw = f16_to_f32(wd[6] >> 16);
#pragma unroll
      for (int col = 0; col < C; ++col) {
        const uint4* xv = &xs[(col * T_K + sub * 128) / 16];
        float part = 0.f;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {  // activation block within the 128
          const uint4 x0 = xv[2 * s4], x1 = xv[2 * s4 + 1];
          int sacc = -xsum[col * T_SUB + sub * 4 + s4];
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 0], (int)x0.x, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 1], (int)x0.y, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 2], (int)x0.z, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 3], (int)x0.w, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 4], (int)x1.x, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 5], (int)x1.y, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 6], (int)x1.z, sacc, false);
          sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 7], (int)x1.w, sacc, false);
          part = fmaf(xd[col * T_SUB + sub * 4 + s4], (float)sacc, part);
        }
        acc[col] = fmaf(dw, part, acc[col]);
      }
    }
  }
  // sum the 8 lanes of each row (fixed order)
#pragma unroll
  for (int j = 0; j < C; ++j) {
    float v = acc[j];
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    acc[j] = v;
  }
  if (sub == 0 && row0 < n) {
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (j < c) out[j * n + row0] = acc[j];
  }
}

// Persistent variant: x (int8 q, per-32 d and sum q) is staged in LDS once
// per workgroup, and every wave walks its own list of 8-row groups with the
// weight loads D items (one item = 8 blocks of each of the wave's 8 rows)
// ahead in a register ring -- no barrier inside the main loop.  Loads carry
// no branch: items past the end read at an offset beyond the buffer, which
// returns zeros (an all-zero block decodes to digits 0 and scale 0).
constexpr uint32_t T_OOB = 0x80000000u;

// LDS bank plan (64 banks, 4 bytes): the digit table is stored in 16 copies
// interleaved by entry (word 16 e + l % 16 holds entry e for lane l), so the
// four lanes that share a copy are the only ones that can collide; x blocks
// of 128 int8 are padded to 144 bytes so that the 8 blocks a wave reads at
// once start in 8 different bank quads.
constexpr int TP_LPR = 8;     // lanes per row in the persistent ternary GEMV
constexpr int TP_WAVES = 5;   // waves per SIMD the register budget is sized for
constexpr int TP_WAVES_SB = 4;  // the same with PTQ1_1 superblocks (12 words per item)
constexpr int LUT_COPIES = 16;
constexpr int XB_WORDS = 36;  // words per padded 128-element x block

// The digit table in LUT_COPIES interleaved copies (256 threads).
__device__ __forceinline__ void tern_lut_init(uint32_t* lut) {
  const int tid = threadIdx.x;
  {
    // Thread t owns entry t (words 16 t .. 16 t + 15) and writes its copies
    // as four 16-byte quads in the order (m + t / 4) % 4: the 16 lanes one
    // ds_write_b128 cycle serves then cover all 64 banks (writing the copies
    // in order would put every lane of a cycle in 4 banks).
    static_assert(LUT_COPIES == 16, "copy quads");
    const uint32_t v = tid;
    const uint32_t ent = (v % 3) | ((v / 3) % 3) << 8 | ((v / 9) % 3) << 16 | ((v / 27) % 3) << 24 |
                         ((v / 81) % 3) << 4;  // entries >= 243 are never indexed by valid data
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<uint4*>(lut + tid * LUT_COPIES + 4 * ((m + (tid >> 2)) & 3)) =
          make_uint4(ent, ent, ent, ent);
  }
}

// One-time staging of a workgroup's LDS: the digit table in LUT_COPIES
// interleaved copies and the activations (x blocks padded to XB_WORDS words,
// per-32 sum of q and d).  Columns c..C-1 stage zeros.
template <int C, bool PT>
__device__ __forceinline__ void tern_stage(uint32_t* lut, uint32_t* xs, int* xsum, float* xd,
                                           const uint8_t* __restrict__ xq, int bpr, int nsb, int c) {
  tern_lut_init(lut);
  const int tid = threadIdx.x;
  for (int idx = tid; idx < C * nsb; idx += 256) {
    const int col = idx / nsb, sb = idx - col * nsb;
    uint32_t q[8] = {0, 0, 0, 0, 0, 0, 0, 0}, hd = 0;
    if (col < c) {
      xq_load<PT>(xq, col, nsb, sb, hd, q);
    }
    uint32_t* dst = xs + (col * bpr + (sb >> 2)) * XB_WORDS + (sb & 3) * 8;
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dst[i] = q[i];
      sum = __builtin_amdgcn_sdot4((int)q[i], 0x01010101, sum, false);
    }
    xsum[col * nsb + sb] = sum;
    xd[col * nsb + sb] = f16_to_f32(hd & 0xFFFFu);
  }
}

// One PTQ1_0 block (its 7 words in v) against the staged activations of
// block bx of the row: acc[col] += d_w * sum_s4 d_x * (sum u q - sum q).
// lt is this lane's copy of the digit table.
// The 128 digits u = t + 1 of one block (its 7 words in v) in k order:
// dg[i] holds elements 4i..4i+3, one per byte.  lt is this lane's copy of
// the digit table.
template <int COPIES = LUT_COPIES>
__device__ __forceinline__ void tern_decode(const uint32_t (&v)[7], const uint32_t* lt,
                                            uint32_t (&dg)[32]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {  // qs bytes 0..15: element 16 j + b
    const uint32_t l0 = lt[(v[g] & 0xFF) * COPIES], l1 = lt[((v[g] >> 8) & 0xFF) * COPIES];
    const uint32_t l2 = lt[((v[g] >> 16) & 0xFF) * COPIES], l3 = lt[(v[g] >> 24) * COPIES];
    uint32_t d0, d1, d2, d3, d4;
    transpose4(l0, l1, l2, l3, d0, d1, d2, d3, d4);
    dg[g] = d0; dg[4 + g] = d1; dg[8 + g] = d2; dg[12 + g] = d3; dg[16 + g] = d4;
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {  // qs bytes 16..23: element 80 + 8 j + b
    const uint32_t x = v[4 + g];
    const uint32_t l0 = lt[(x & 0xFF) * COPIES], l1 = lt[((x >> 8) & 0xFF) * COPIES];
    const uint32_t l2 = lt[((x >> 16) & 0xFF) * COPIES], l3 = lt[(x >> 24) * COPIES];
    uint32_t d0, d1, d2, d3, d4;
    transpose4(l0, l1, l2, l3, d0, d1, d2, d3, d4);
    dg[20 + g] = d0; dg[22 + g] = d1; dg[24 + g] = d2; dg[26 + g] = d3; dg[28 + g] = d4;
  }
  {
    const uint32_t h = v[6] & 0xFFFFu;  // qh: elements 120..127
    dg[30] = (h | (h << 14)) & 0x03030303u;
    dg[31] = ((h >> 4) | (h << 10)) & 0x03030303u;
  }
}

// acc[col] += d_w * sum_s4 d_x * (sum u q - sum q) for one block's 128
// digits dg against the staged activations of block bx of the row.
template <int C>
__device__ __forceinline__ void tern_products(const uint32_t (&dg)[32], float dw, const uint32_t* xs,
                                              const int* xsum, const float* xd, int bx, int bpr,
                                              int nsb, float (&acc)[C]) {
#pragma unroll
  for (int col = 0; col < C; ++col) {
    const uint4* xv = reinterpret_cast<const uint4*>(xs + (col * bpr + bx) * XB_WORDS);
    float part = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {  // activation block within the 128
      const uint4 x0 = xv[2 * s4], x1 = xv[2 * s4 + 1];
      int sacc = -xsum[col * nsb + bx * 4 + s4];
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 0], (int)x0.x, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 1], (int)x0.y, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 2], (int)x0.z, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 3], (int)x0.w, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 4], (int)x1.x, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 5], (int)x1.y, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 6], (int)x1.z, sacc, false);
      sacc = __builtin_amdgcn_sdot4((int)dg[8 * s4 + 7], (int)x1.w, sacc, false);
      part = fmaf(xd[col * nsb + bx * 4 + s4], (float)sacc, part);
    }
    acc[col] = fmaf(dw, part, acc[col]);
  }
}

// One PTQ1_0 block (its 7 words in v) against the staged activations.
template <int C>
__device__ __forceinline__ void tern_block(const uint32_t (&v)[7], const uint32_t* lt,
                                           const uint32_t* xs, const int* xsum, const float* xd,
                                           int bx, int bpr, int nsb, float (&acc)[C]) {
  uint32_t dg[32];
  tern_decode(v, lt, dg);
  tern_products<C>(dg, f16_to_f32(v[6] >> 16), xs, xsum, xd, bx, bpr, nsb, acc);  // d = 0 past the end
}

// ---- PTQ1_1 superblocks (Ternary post, section 2 struct ptq1_1; section
// 3.1: sub-block sub = kbx & 7 of superblock kbx >> 3).  216 bytes: qs[192]
// (the qs[24] of sub-blocks 0..7), qh[13] (the 64 tail trits, five per byte
// in sub-block order, tail trit 8 sub + e at digit (8 sub + e) % 5 of byte
// (8 sub + e) / 5; digit 4 of qh[12] is the free trit), an 80-bit
// little-endian field of eight 10-bit mantissas (mantissa sub at bit 10 sub),
// and the exponent byte.  Pattern index P = exponent byte + 256 * free digit:
// P < 767 is a row of the 767 x 8 exponent codebook, P = 767 sends the
// superblock to the escape table (ascending superblock indices row * K/1024 +
// sb, eight exponents each).  d = (exponent << 10) | mantissa (sign +).
constexpr int SB_BYTES = 216;
constexpr int SB_CODEBOOK_ROWS = 767;
constexpr int SB_ESC_MAX = 2048;  // escaped superblocks staged in LDS per call

struct SbTables {
  const uint8_t* codebook;  // [767][8] exponent fields
  const int32_t* esc_idx;   // [n_esc] ascending superblock indices
  const uint8_t* esc_patt;  // [n_esc][8] their exponent fields
  int n_esc;
};

// LDS words the superblock tables take: codebook (767 x 8 bytes) + escape
// indices + escape patterns
__host__ __device__ constexpr int sb_lds_words(int n_esc) { return 1534 + n_esc + 2 * n_esc; }

// Codebook and escape table into LDS (256 threads; one-time per workgroup).
template <int NTH = 256>
__device__ __forceinline__ void tern_stage_sb(uint32_t* dst, const SbTables& t) {
  const int tid = threadIdx.x;
  const uint32_t* cb = reinterpret_cast<const uint32_t*>(t.codebook);
  for (int i = tid; i < 1534; i += NTH) dst[i] = cb[i];
  const int ne = t.n_esc;
  for (int i = tid; i < ne; i += NTH) dst[1534 + i] = (uint32_t)t.esc_idx[i];
  const uint32_t* ep = reinterpret_cast<const uint32_t*>(t.esc_patt);
  for (int i = tid; i < 2 * ne; i += NTH) dst[1534 + ne + i] = ep[i];
}

// The 128 digits and the scale of sub-block sub (= this lane's block within
// the superblock) from its 12 words: v[0..5] its qs bytes 24 sub .. 24 sub +
// 23, v[6..11] the superblock's bytes 192..215.  gidx: the superblock's
// index (the escape key); tbl: the staged tables (codebook bytes, then the
// escape indices and patterns).
template <int COPIES = LUT_COPIES>
__device__ __forceinline__ void tern_decode_sb(const uint32_t (&v)[12], const uint32_t* lt,
                                               const uint32_t* tbl, int n_esc, int gidx, int sub,
                                               uint32_t (&dg)[32], float& dw) {
  // qs: exactly the PTQ1_0 sections
  uint32_t v7[7] = {v[0], v[1], v[2], v[3], v[4], v[5], 0u};
  tern_decode<COPIES>(v7, lt, dg);
  // tail: the 8 digits from digit d0 of qh byte b0 on (b0 = 8 sub / 5,
  // d0 = 8 sub % 5), out of the three bytes b0 .. b0 + 2
  // (word selection by lane masks: a select chain on the array makes the
  // compiler index a private copy of it in scratch memory)
  const int b0 = (8 * sub) / 5, d0 = (8 * sub) % 5, w = b0 >> 2;
  const uint32_t w0 = 0u - (uint32_t)(w == 0), w1 = 0u - (uint32_t)(w == 1), w2 = 0u - (uint32_t)(w == 2);
  const uint32_t lo = (v[6] & w0) | (v[7] & w1) | (v[8] & w2);
  const uint32_t hi = (v[7] & w0) | (v[8] & w1) | (v[9] & w2);
  const uint32_t three = __builtin_amdgcn_alignbit(hi, lo, 8 * (b0 & 3));
  const uint32_t l0 = lt[(three & 0xFF) * COPIES];
  const uint32_t l1 = lt[((three >> 8) & 0xFF) * COPIES];
  const uint32_t l2 = lt[((three >> 16) & 0xFF) * COPIES];
  // the digit sequence of the three bytes, one digit per byte: table entry =
  // digits 0..3 in bytes 0..3 (two bits each) and digit 4 in bits 4..5
  const uint32_t s0 = l0 & 0x03030303u;
  const uint32_t s1 = ((l0 >> 4) & 3u) | ((l1 & 0x00030303u) << 8);
  const uint32_t s2 = ((l1 >> 24) & 3u) | (((l1 >> 4) & 3u) << 8) | ((l2 & 0x0303u) << 16);
  // digits d0 .. d0 + 7 of the sequence s0 s1 s2 (v_alignbyte shifts by 0..3
  // bytes, so d0 = 4 starts one word later)
  const bool d4 = d0 == 4;
  dg[30] = __builtin_amdgcn_alignbyte(d4 ? s2 : s1, d4 ? s1 : s0, d0 & 3);  // elements 120..123
  dg[31] = d4 ? s2 : __builtin_amdgcn_alignbyte(s2, s1, d0 & 3);            // elements 124..127
  // scale: pattern index from the exponent byte and the free trit
  const uint32_t free = (lt[(v[9] & 0xFF) * COPIES] >> 4) & 3u;
  const int pat = (int)((v[11] >> 24) | (free << 8));
  uint32_t e;
  if (pat < SB_CODEBOOK_ROWS) {
    e = (tbl[pat * 2 + (sub >> 2)] >> (8 * (sub & 3))) & 0xFFu;
  } else {  // escape: binary search of the superblock index (LDS only)
    const uint32_t* idx = tbl + 1534;
    int a = 0, z = n_esc;
    while (a < z) {
      const int m = (a + z) >> 1;
      if ((int)idx[m] < gidx) a = m + 1;
      else z = m;
    }
    a = min(a, max(n_esc - 1, 0));
    e = n_esc > 0 ? (tbl[1534 + n_esc + 2 * a + (sub >> 2)] >> (8 * (sub & 3))) & 0xFFu : 0u;
  }
  // mantissa sub: bits 10 sub .. + 9 of the field at bytes 205..214
  const uint32_t f0 = __builtin_amdgcn_alignbit(v[10], v[9], 8);   // field bits 0..31
  const uint32_t f1 = __builtin_amdgcn_alignbit(v[11], v[10], 8);  // bits 32..63
  const uint32_t f2 = v[11] >> 8;                                  // bits 64..87
  const int mb = 10 * sub, mw = mb >> 5;
  const uint32_t m0 = 0u - (uint32_t)(mw == 0), m1 = 0u - (uint32_t)(mw == 1), m2 = 0u - (uint32_t)(mw == 2);
  const uint32_t mlo = (f0 & m0) | (f1 & m1) | (f2 & m2);
  const uint32_t mhi = (f1 & m0) | (f2 & (m1 | m2));
  const uint32_t m = __builtin_amdgcn_alignbit(mhi, mlo, mb & 31) & 0x3FFu;
  dw = f16_to_f32((e << 10) | m);
}

// dynamic LDS: table [256][16], x [C][bpr][36 words], sum q [C][k/32], d [C][k/32]
// ---- Persistent GEMV on the int8 matrix cores (c <= 8, x and the digit
// table in LDS once per CU).
//
// One 1024-lane workgroup per CU owns a balanced block of rows.  Lane l is
// (q, r) = (l / 4, l % 4); quad q is block q of v_mfma_i32_4x4x4_16b_i8 (16
// independent 4 x 4 x 4 int8 products per instruction) and covers rows
// 4 (q / 8) .. 4 (q / 8) + 3 of the current 8-row group at PTQ1_0 block
// 8 t + q % 8 of the current item t (8 rows x 1024 k).  Lane (q, r) decodes
// its row's block as in the other kernels (table reads, byte transposes) to
// 32 dwords of digits u = t + 1; MFMA s of a sub-block takes digit dword s
// as its B operand and, as the A operand, the same four k of activation
// column 4 cs + r (columns past c repeat the last; their results are never
// stored).  The accumulator starts at -sum q of the sub-block, so after the
// eight instructions of a 32-k sub-block element i holds the exact int32
// sum over t q of column 4 cs + i, which the VALU scales by d_x and, per
// block, by d_w.
//
// LDS: the digit table with one copy per lane (word 64 e + l: its reads
// never meet in a bank, and the address e * 256 + 4 l is one v_perm of the
// weight word and 4 l), then one record per 128-k block: each column's 128
// int8 q (144 bytes apart), and per 32-k sub-block -sum q and d_x of each
// column.  The record length is padded so that the sixteen lanes of four
// quads (four blocks x four columns) start in sixteen different bank
// groups.  Items (8-row group, 1024-k slice) in row-group-major order are
// cut into 16 equal ranges, one per wave; a wave parks a row group's
// partials in LDS when it leaves it and the outputs add the parks in wave
// order (deterministic).
constexpr int TM_NT = 1024;
constexpr int TM_NW = TM_NT / 64;
constexpr int TM_LUT_BYTES = 243 * 64 * 4;
constexpr int TM_XCOL = 144;  // bytes between the columns of a block record
constexpr int TM_XPRE = 2;    // x blocks per lane loaded ahead of the weights

// Sums per sub-block in a record (-sum q and d_x for this many columns).
__host__ __device__ constexpr int tm_sumw(int C) { return C; }
// Record bytes per 128-k block for C columns: the smallest length >= the
// data whose 16-byte units put lanes (block b, column r), b, r < 4, in
// sixteen different groups of four banks.
__host__ __device__ constexpr int tm_record(int C) {
  const int base = C * TM_XCOL + 4 * tm_sumw(C) * 8;
  for (int pad = 0; pad < 256; pad += 16) {
    const int u = (base + pad) / 16;
    bool seen[16] = {};
    bool ok = true;
    for (int b = 0; b < 4 && ok; ++b)
      for (int r = 0; r < 4 && ok; ++r) {
        if (r >= C) continue;  // lanes past c read column c - 1 (the same address)
        const int g = (b * u + r * (TM_XCOL / 16)) & 15;
        if (seen[g]) ok = false;
        seen[g] = true;
      }
    if (ok) return base + pad;
  }
  return base;
}

// SB: the weights are PTQ1_1 superblocks (an item's eight blocks are one
// superblock; lane q % 8 decodes sub-block q % 8 from its 24 qs bytes and the
// superblock's last 24 bytes), with the codebook and escape tables staged in
// LDS after the x records.
template <int C, int D, bool SB, bool PT>
__global__ __launch_bounds__(TM_NT) void k_gemv_ternary_mq(const uint32_t* __restrict__ w,
                                                           const uint8_t* __restrict__ xq,
                                                           float* __restrict__ out, int n, int k,
                                                           int c, int spw, SbTables sbt) {
  constexpr int CS = (C + 3) / 4;        // MFMA column sets
  constexpr int RB = tm_record(C);       // record bytes per block
  constexpr int SW = tm_sumw(C);
  constexpr int XSUM = C * TM_XCOL;      // offset of the sums in a record
  constexpr int W = SB ? 12 : 7;         // words a lane loads per item
  extern __shared__ uint4 tm_smem[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(tm_smem);
  const int bpr = k / 128, nsb = k / 32;
  uint8_t* rec = lds + TM_LUT_BYTES;                                     // [bpr][RB]
  uint32_t* tbl = reinterpret_cast<uint32_t*>(rec + bpr * RB);          // superblock tables
  float* slots = reinterpret_cast<float*>(tbl + (SB ? sb_lds_words(sbt.n_esc) : 0));  // [NW][spw][8][C]
  int* wtab = reinterpret_cast<int*>(slots + TM_NW * spw * 8 * C);      // [NW][3]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 2, r = lane & 3;
  const int kb = q & 7, rin = (q >> 3) * 4 + r;  // block in the item, row in the 8-row group
  const int nwg = (int)gridDim.x, b = (int)blockIdx.x;
  const int r0 = b * (n / nwg) + min(b, n % nwg);
  const int count = n / nwg + (b < n % nwg ? 1 : 0);
  const int nro = (count + 7) / 8;
  const int nit = (bpr + 7) / 8;  // items per row group
  const int items = nro * nit;
  const int i0 = wave * items / TM_NW, i1 = (wave + 1) * items / TM_NW;
  const int ro_first = i0 / nit;
  if (lane == 0) {
    wtab[wave * 3 + 0] = i0;
    wtab[wave * 3 + 1] = i1;
    wtab[wave * 3 + 2] = ro_first;
  }
  constexpr int BB = SB ? SB_BYTES / 8 : PT_BYTES;  // weight bytes per 128-k block
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)w + (int64_t)r0 * bpr * BB), 0, count * bpr * BB, 0x00020000);

  // weight ring: issue position (row, block) of this lane, items left
  int irow = ro_first * 8 + rin, iblk = (i0 - ro_first * nit) * 8 + kb, left = i1 - i0;
  uint32_t wd[D][W];
  auto issue = [&](int slot) {
    const bool ok = left > 0 && irow < count && iblk < bpr;
    if constexpr (SB) {
      // this sub-block's qs words, then the superblock's last 24 bytes
      const uint32_t o = ok ? (uint32_t)((irow * nit + (iblk >> 3)) * SB_BYTES) : T_OOB;
#pragma unroll
      for (int j = 0; j < 6; ++j) wd[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 24 * kb + 4 * j), 0, 0);
#pragma unroll
      for (int j = 0; j < 6; ++j) wd[slot][6 + j] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 192 + 4 * j), 0, 0);
    } else {
      const uint32_t o = ok ? (uint32_t)((irow * bpr + iblk) * PT_BYTES) : T_OOB;
#pragma unroll
      for (int j = 0; j < 7; ++j) wd[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 4 * j), 0, 0);
    }
    --left;
    iblk += 8;
    if (iblk - kb >= nit * 8) {
      iblk = kb;
      irow += 8;
    }
  };
  // x blocks (q8_1, 36 bytes) of the staging: the first TM_XPRE per lane
  // are loaded before the weight prologue, since a wave's loads complete in
  // issue order and the staging would otherwise wait for its weights.  The
  // order is rotated per workgroup: every CU reads the same x.  A block is
  // three loads in either layout: 16 + 16 + 4 bytes from words 0, 4 and 8 of
  // a record, or the two 16-byte plane slots of its q (words 1 and 5) and its
  // (d, s) word.
  const int nxb = c * nsb;
  const int xrot = (int)(((uint32_t)b * 2654435761u) % (uint32_t)nxb);
  auto xblock = [&](int i) {
    const int v = i + xrot;
    return v >= nxb ? v - nxb : v;
  };
  // (buffer loads, no branch: a conditional load would put the first use of
  // its value, and so the wait for it, right behind it)
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)xq, 0, nxb * Q8_BYTES, 0x00020000);
  uint32_t xpre[TM_XPRE][9];  // the three loads' words, in load order
#pragma unroll
  for (int i = 0; i < TM_XPRE; ++i) {
    const int idx = tid + i * TM_NT;
    uint32_t o1, o2, o3;
    if constexpr (PT) {
      const int xi = xblock(idx < nxb ? idx : 0), col = xi / nsb;
      const uint32_t cb = (uint32_t)(col * nsb * Q8_BYTES);
      const XBlk xb = pt_block(nsb, xi - col * nsb);
      o1 = idx < nxb ? cb + xb.q0 : T_OOB;
      o2 = idx < nxb ? cb + xb.q1 : T_OOB;
      o3 = idx < nxb ? cb + xb.ds : T_OOB;
    } else {
      o1 = idx < nxb ? (uint32_t)(xblock(idx) * Q8_BYTES) : T_OOB;
      o2 = o1 + 16;
      o3 = o1 + 32;
    }
    const uint4 lo = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)o1, 0, 0));
    const uint4 hi = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)o2, 0, 0));
    xpre[i][0] = lo.x; xpre[i][1] = lo.y; xpre[i][2] = lo.z; xpre[i][3] = lo.w;
    xpre[i][4] = hi.x; xpre[i][5] = hi.y; xpre[i][6] = hi.z; xpre[i][7] = hi.w;
    xpre[i][8] = __builtin_amdgcn_raw_buffer_load_b32(xrs, (int)o3, 0, 0);
  }
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);

  // one-time staging: the digit table (one copy per lane), then per block
  // x q, -sum q and d_x of each column
  for (int idx = tid; idx < 243 * 16; idx += TM_NT) {
    const uint32_t e = idx >> 4;
    const uint32_t ent = (e % 3) | ((e / 3) % 3) << 8 | ((e / 9) % 3) << 16 | ((e / 27) % 3) << 24 |
                         ((e / 81) % 3) << 4;
    *reinterpret_cast<uint4*>(lds + e * 256 + (idx & 15) * 16) = make_uint4(ent, ent, ent, ent);
  }
  auto put_x = [&](int xi, const uint32_t (&bk)[9]) {
    const int col = xi / nsb, sb = xi - col * nsb;
    int sum = 0;
#pragma unroll
    for (int i = 1; i < 9; ++i) sum = __builtin_amdgcn_sdot4((int)bk[i], 0x01010101, sum, false);
    uint8_t* rb = rec + (sb >> 2) * RB;
    uint4* dst = reinterpret_cast<uint4*>(rb + col * TM_XCOL + (sb & 3) * 32);
    dst[0] = make_uint4(bk[1], bk[2], bk[3], bk[4]);
    dst[1] = make_uint4(bk[5], bk[6], bk[7], bk[8]);
    int* sums = reinterpret_cast<int*>(rb + XSUM + (sb & 3) * SW * 8);
    sums[col] = -sum;
    reinterpret_cast<float*>(sums + SW)[col] = f16_to_f32(bk[0] & 0xFFFFu);
  };
#pragma unroll
  for (int i = 0; i < TM_XPRE; ++i) {
    const int idx = tid + i * TM_NT;
    if (idx >= nxb) continue;
    if constexpr (PT) {
      // words in block order: (d, s), then q (the PT loads brought (d, s) last)
      uint32_t bk[9];
      bk[0] = xpre[i][8];
#pragma unroll
      for (int j = 1; j < 9; ++j) bk[j] = xpre[i][j - 1];
      put_x(xblock(idx), bk);
    } else {
      put_x(xblock(idx), xpre[i]);
    }
  }
  for (int idx = tid + TM_XPRE * TM_NT; idx < nxb; idx += TM_NT) {  // the rest (wide x)
    const int xi = xblock(idx);
    uint32_t bk[9];
    if constexpr (PT) {
      const int col = xi / nsb;
      uint32_t q8[8];
      xq_load<true>(xq, col, nsb, xi - col * nsb, bk[0], q8);
#pragma unroll
      for (int j = 0; j < 8; ++j) bk[1 + j] = q8[j];
    } else {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(xq + (int64_t)xi * Q8_BYTES);
#pragma unroll
      for (int j = 0; j < 9; ++j) bk[j] = src[j];
    }
    put_x(xi, bk);
  }
  if constexpr (SB) tern_stage_sb<TM_NT>(tbl, sbt);
  __syncthreads();

  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;
  // sum the 8 blocks of each row (lanes of one half-wave with equal l % 4,
  // fixed order) and park them in this wave's slot ro - ro_first
  auto park = [&](int ro) {
    float* dst = slots + ((wave * spw + (ro - ro_first)) * 8 + rin) * C;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v = acc[j];
      v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror 4
      v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror 8
      v += __shfl_xor(v, 16);
      if (kb == 0) dst[j] = v;
      acc[j] = 0.f;
    }
  };

  const uint32_t lane4 = (uint32_t)lane * 4;
  const uint32_t* lut_lane = reinterpret_cast<const uint32_t*>(lds) + lane;  // this lane's table copy
  int cro = ro_first, cit = i0 - ro_first * nit;  // consume position
  const int nsteps = i1 - i0;
  for (int base = 0; base < nsteps; base += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const bool valid = base + d < nsteps;
      uint32_t v[W];
#pragma unroll
      for (int j = 0; j < W; ++j) v[j] = wd[d][j];
      issue(d);  // the ring slot is free once copied out
      if (!valid) continue;  // uniform; no load below
      uint32_t dg[32];
      float dw;
      if constexpr (SB) {
        // (rows past the workgroup's decode garbage that is never stored)
        tern_decode_sb<64>(v, lut_lane, tbl, sbt.n_esc, (r0 + cro * 8 + rin) * nit + cit, kb, dg, dw);
      } else {
        // digits: table word of byte i of a weight word at byte offset
        // (byte << 8) | 4 lane, one v_perm
        auto look = [&](uint32_t word, int i) {
          const uint32_t a = __builtin_amdgcn_perm(word, lane4, 0x0C0C0000u | ((4u + i) << 8));
          return *reinterpret_cast<const uint32_t*>(lds + a);
        };
#pragma unroll
        for (int g = 0; g < 4; ++g) {  // qs bytes 0..15: element 16 j + byte
          uint32_t d0, d1, d2, d3, d4;
          transpose4(look(v[g], 0), look(v[g], 1), look(v[g], 2), look(v[g], 3), d0, d1, d2, d3, d4);
          dg[g] = d0; dg[4 + g] = d1; dg[8 + g] = d2; dg[12 + g] = d3; dg[16 + g] = d4;
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {  // qs bytes 16..23: element 80 + 8 j + byte
          uint32_t d0, d1, d2, d3, d4;
          transpose4(look(v[4 + g], 0), look(v[4 + g], 1), look(v[4 + g], 2), look(v[4 + g], 3), d0, d1, d2, d3, d4);
          dg[20 + g] = d0; dg[22 + g] = d1; dg[24 + g] = d2; dg[26 + g] = d3; dg[28 + g] = d4;
        }
        const uint32_t h = v[6] & 0xFFFFu;  // qh: elements 120..127
        dg[30] = (h | (h << 14)) & 0x03030303u;
        dg[31] = ((h >> 4) | (h << 10)) & 0x03030303u;
        dw = f16_to_f32(v[6] >> 16);  // 0 past the end of the row or past its rows
      }
      const int blk = min(cit * 8 + kb, bpr - 1);  // reads stay in the staged range
      const uint8_t* rb = rec + blk * RB;
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        constexpr int NJ = C < 4 ? C : 4;  // columns of this set
        const uint8_t* xp = rb + min(cs * 4 + r, c - 1) * TM_XCOL;
        float part[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) part[j] = 0.f;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int* sums = reinterpret_cast<const int*>(rb + XSUM + s4 * SW * 8) + cs * 4;
          const float* dx = reinterpret_cast<const float*>(sums + SW);
          intx4 acc_i;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc_i[j] = sums[j < NJ ? j : 0];
          const uint4 xa = *reinterpret_cast<const uint4*>(xp + s4 * 32);
          const uint4 xb = *reinterpret_cast<const uint4*>(xp + s4 * 32 + 16);
          const int xw[8] = {(int)xa.x, (int)xa.y, (int)xa.z, (int)xa.w, (int)xb.x, (int)xb.y, (int)xb.z, (int)xb.w};
#pragma unroll
          for (int s = 0; s < 8; ++s)
            acc_i = __builtin_amdgcn_mfma_i32_4x4x4i8(xw[s], (int)dg[8 * s4 + s], acc_i, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < NJ; ++j) part[j] = fmaf(dx[j], (float)acc_i[j], part[j]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[cs * 4 + j] = fmaf(dw, part[j], acc[cs * 4 + j]);
      }
      if (++cit == nit) {  // uniform: the wave leaves its row group
        park(cro);
        cit = 0;
        ++cro;
      }
    }
  }
  if (nsteps > 0 && cit != 0) park(cro);
  __syncthreads();

  // outputs: the parks of each row in wave order
  for (int idx = tid; idx < nro * 8 * c; idx += TM_NT) {
    const int ro = idx / (8 * c);
    const int rc = idx - ro * 8 * c;
    const int rr = rc / c, col = rc - rr * c;
    if (ro * 8 + rr >= count) continue;
    const int ilo = ro * nit, ihi = ilo + nit;
    // wave h owns items [floor(h items / NW), floor((h + 1) items / NW)); the
    // one owning item i is floor(((i + 1) NW - 1) / items)
    const int hlo = ((ilo + 1) * TM_NW - 1) / items, hhi = (ihi * TM_NW - 1) / items;
    float v = 0.f;
    for (int h = hlo; h <= hhi; ++h) {
      const int a = wtab[h * 3 + 0], e = wtab[h * 3 + 1];
      if (e > a && a < ihi && e > ilo) v += slots[((h * spw + (ro - wtab[h * 3 + 2])) * 8 + rr) * C + col];
    }
    out[(int64_t)col * n + r0 + ro * 8 + rr] = v;
  }
}

// LPR lanes per row (8 or 16): a wave holds 64 / LPR rows, a lane one block
// of its row per item (an item = LPR consecutive blocks of each row).
// SB: the weights are PTQ1_1 superblocks (LPR = 8: an item is one superblock
// of each row, lane sub its sub-block), with the codebook and the escape
// table staged in LDS after the activations.
template <int C, int D, int LPR, bool SB, bool PT>
__global__ __launch_bounds__(256, SB ? TP_WAVES_SB : TP_WAVES) void k_gemv_ternary_persist(const uint32_t* __restrict__ w,
                                                              const uint8_t* __restrict__ xq,
                                                              float* __restrict__ out, int n, int k,
                                                              int c, SbTables sbt) {
  static_assert(!SB || LPR == 8, "a superblock is 8 blocks");
  constexpr int W = SB ? 12 : 7;                          // words a lane loads per item
  extern __shared__ uint32_t tsm[];
  const int nsb = k / 32;
  const int bpr = k / 128;                                // blocks per row
  uint32_t* lut = tsm;                                    // [256][LUT_COPIES]
  uint32_t* xs = tsm + 256 * LUT_COPIES;                  // [C][bpr][XB_WORDS]
  int* xsum = reinterpret_cast<int*>(xs + C * bpr * XB_WORDS);  // [C][nsb]
  float* xd = reinterpret_cast<float*>(xsum + C * nsb);   // [C][nsb]
  uint32_t* tbl = reinterpret_cast<uint32_t*>(xd + C * nsb);  // superblock tables

  constexpr int RPW = 64 / LPR;  // rows per wave (one row group)
  const int tid = threadIdx.x, lane = tid & 63, sub = lane & (LPR - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntiles = (bpr + LPR - 1) / LPR;
  const int nw = gridDim.x * 4, gw = blockIdx.x * 4 + wave;
  const int nrg = (n + RPW - 1) / RPW;
  const int nitems = (nrg > gw ? (nrg - gw + nw - 1) / nw : 0) * ntiles;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)w, 0, (int)((int64_t)n * bpr * (SB ? SB_BYTES / 8 : PT_BYTES)), 0x00020000);

  // ---- weight ring: item i = (row group gw + (i / ntiles) nw, tile i % ntiles)
  uint32_t wd[D][W];
  auto issue = [&](int slot, int i) {
    const int t = i % ntiles, rg = gw + (i / ntiles) * nw;
    const int row = rg * RPW + lane / LPR, blk = t * LPR + sub;
    const bool ok = i < nitems && row < n && blk < bpr;
    if constexpr (SB) {
      // this sub-block's qs words, then the superblock's last 24 bytes
      const uint32_t o = ok ? (uint32_t)((row * ntiles + t) * SB_BYTES) : T_OOB;
#pragma unroll
      for (int q = 0; q < 6; ++q)
        wd[slot][q] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 24 * sub + 4 * q), 0, 0);
#pragma unroll
      for (int q = 0; q < 6; ++q)
        wd[slot][6 + q] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 192 + 4 * q), 0, 0);
    } else {
      const uint32_t o = ok ? (uint32_t)((row * bpr + blk) * PT_BYTES) : T_OOB;
#pragma unroll
      for (int q = 0; q < 7; ++q)
        wd[slot][q] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 4 * q), 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);

  // ---- one-time staging: digit table and the activations (and the
  // superblock tables)
  tern_stage<C, PT>(lut, xs, xsum, xd, xq, bpr, nsb, c);
  if constexpr (SB) tern_stage_sb(tbl, sbt);
  __syncthreads();

  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;

  // Items past nitems (the last group of D) copy out and refill their slot
  // like any other -- the loads stay out of branches -- but skip the math.
  auto item = [&](const int i, const int slot) {
    const int t = i % ntiles;
    const int blk = t * LPR + sub;
    uint32_t v[W];
#pragma unroll
    for (int q = 0; q < W; ++q) v[q] = wd[slot][q];
    issue(slot, i + D);  // the slot is free once copied out
    if (i >= nitems) return;  // uniform; no load below
    if constexpr (SB) {
      // (rows past n decode garbage that is never stored)
      const int row = (gw + (i / ntiles) * nw) * RPW + lane / LPR;
      uint32_t dg[32];
      float dw;
      tern_decode_sb(v, lut + (lane & (LUT_COPIES - 1)), tbl, sbt.n_esc, row * ntiles + t, sub, dg, dw);
      tern_products<C>(dg, dw, xs, xsum, xd, blk, bpr, nsb, acc);
    } else {
      // blocks past the end loaded zeros (scale 0); x reads stay in the staged range
      tern_block<C>(v, lut + (lane & (LUT_COPIES - 1)), xs, xsum, xd, blk < bpr ? blk : 0, bpr, nsb, acc);
    }
    if (t == ntiles - 1) {  // uniform: the wave leaves its 8-row group
      const int row = (gw + (i / ntiles) * nw) * RPW + lane / LPR;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        float s = acc[j];
        if (LPR == 16) s += __shfl_xor(s, 8);  // the lanes of a row, fixed order
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 1);
        if (sub == 0 && j < c && row < n) out[(int64_t)j * n + row] = s;
        acc[j] = 0.f;
      }
    }
  };
  // groups of D items keep the ring slot a compile-time constant
  for (int i = 0; i < nitems; i += D) {
    if constexpr (C <= 4) {
      // issue priority from the share of items still to do (waves that fall
      // behind are served first; 4-5% at 2 and 4 columns, a loss at 8)
      if (4 * (nitems - i) > 3 * nitems) __builtin_amdgcn_s_setprio(3);
      else if (4 * (nitems - i) > 2 * nitems) __builtin_amdgcn_s_setprio(2);
      else if (4 * (nitems - i) > nitems) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) item(i + d, d);
  }
}

// K-split variant for the narrowest batches.  With one 8-row group per wave,
// a single column leaves about two waves per SIMD (N = 17280 gives 2160
// groups), too few to hide the latencies of the digit-table reads and the
// permutes.  Here the tiles of each row group are split between S waves of
// one workgroup (4 / S row groups per 256-lane workgroup, not persistent), so
// S times more waves run, and the S partial sums of a row are added in LDS in
// part order.
template <int C, int D, int S, bool SB, bool PT>
__global__ __launch_bounds__(256, SB ? TP_WAVES_SB : TP_WAVES) void k_gemv_ternary_ksplit(const uint32_t* __restrict__ w,
                                                             const uint8_t* __restrict__ xq,
                                                             float* __restrict__ out, int n, int k,
                                                             int c, SbTables sbt) {
  constexpr int LPR = 8, RPW = 64 / LPR;
  constexpr int W = SB ? 12 : 7;                          // words a lane loads per item
  extern __shared__ uint32_t tsm[];
  const int nsb = k / 32;
  const int bpr = k / 128;
  uint32_t* lut = tsm;                                    // [256][LUT_COPIES]
  uint32_t* xs = tsm + 256 * LUT_COPIES;                  // [C][bpr][XB_WORDS]
  int* xsum = reinterpret_cast<int*>(xs + C * bpr * XB_WORDS);  // [C][nsb]
  float* xd = reinterpret_cast<float*>(xsum + C * nsb);   // [C][nsb]
  float* psum = xd + C * nsb;                             // [4 waves][RPW rows][C]
  uint32_t* tbl = reinterpret_cast<uint32_t*>(psum + 4 * RPW * C);  // superblock tables

  const int tid = threadIdx.x, lane = tid & 63, sub = lane & (LPR - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = wave % S;
  const int rg = (int)blockIdx.x * (4 / S) + wave / S;
  const int row = rg * RPW + lane / LPR;
  const int ntiles = (bpr + LPR - 1) / LPR;
  const int tps = (ntiles + S - 1) / S;                   // tiles per part
  const int t0 = part * tps;
  const int nitems = max(0, min(ntiles, t0 + tps) - t0);  // this wave's tiles
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)w, 0, (int)((int64_t)n * bpr * (SB ? SB_BYTES / 8 : PT_BYTES)), 0x00020000);

  // weight ring: item i = tile t0 + i of the row group (with superblocks: its
  // superblock t0 + i, this lane's sub-block sub)
  uint32_t wd[D][W];
  auto issue = [&](int slot, int i) {
    const int blk = (t0 + i) * LPR + sub;
    const bool ok = i < nitems && row < n && blk < bpr;
    if constexpr (SB) {
      const uint32_t o = ok ? (uint32_t)((row * ntiles + t0 + i) * SB_BYTES) : T_OOB;
#pragma unroll
      for (int q = 0; q < 6; ++q)
        wd[slot][q] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 24 * sub + 4 * q), 0, 0);
#pragma unroll
      for (int q = 0; q < 6; ++q)
        wd[slot][6 + q] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 192 + 4 * q), 0, 0);
    } else {
      const uint32_t o = ok ? (uint32_t)((row * bpr + blk) * PT_BYTES) : T_OOB;
#pragma unroll
      for (int q = 0; q < 7; ++q)
        wd[slot][q] = __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)(o + 4 * q), 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);

  tern_stage<C, PT>(lut, xs, xsum, xd, xq, bpr, nsb, c);
  if constexpr (SB) tern_stage_sb(tbl, sbt);
  __syncthreads();

  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;
  auto item = [&](const int i, const int slot) {
    uint32_t v[W];
#pragma unroll
    for (int q = 0; q < W; ++q) v[q] = wd[slot][q];
    issue(slot, i + D);       // the slot is free once copied out
    if (i >= nitems) return;  // uniform; no load below
    const int blk = (t0 + i) * LPR + sub;
    if constexpr (SB) {
      uint32_t dg[32];
      float dw;
      tern_decode_sb(v, lut + (lane & (LUT_COPIES - 1)), tbl, sbt.n_esc, row * ntiles + t0 + i, sub, dg, dw);
      tern_products<C>(dg, dw, xs, xsum, xd, blk, bpr, nsb, acc);
    } else {
      tern_block<C>(v, lut + (lane & (LUT_COPIES - 1)), xs, xsum, xd, blk < bpr ? blk : 0, bpr, nsb, acc);
    }
  };
  for (int i = 0; i < nitems; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) item(i + d, d);
  }

  // this part's row sums (the lanes of a row, fixed order) -> LDS; part 0
  // adds the parts in order
#pragma unroll
  for (int j = 0; j < C; ++j) {
    float v = acc[j];
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    if (sub == 0) psum[(wave * RPW + lane / LPR) * C + j] = v;
  }
  __syncthreads();
  if (part == 0 && sub == 0 && row < n) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if (j >= c) break;
      float v = psum[(wave * RPW + lane / LPR) * C + j];
#pragma unroll
      for (int p2 = 1; p2 < S; ++p2) v += psum[((wave + p2) * RPW + lane / LPR) * C + j];
      out[(int64_t)j * n + row] = v;
    }
  }
}

// ---- ternary x q8_1 GEMM on the fp4 x fp8 matrix cores (64 or more columns)
//
// y[c][r] = sum_b d_w[r][b] sum_j d_x[c][4b + j] S[c][r][b][j] with the
// exact sub-block sums S = sum_i t q over 32 k.  The products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales: a trit is exact in
// fp4 (e2m1: +-1 and 0) and an activation q = 16 qh + ql (qh = q >> 4 in
// -8..7, ql = q & 15) is the exact fp8 (e4m3) pair (ql, 16 qh), so one
// product over 64 k slots -- each k twice, once against ql and once against
// 16 qh -- sums one 32-k sub-block: S comes out of the float32 accumulator
// exactly (integers below 2^13), as float, so the VALU only multiplies by
// d_x (one FMA per result and sub-block; int8 products need a convert as
// well) and by d_w once per 128-k block.
//
// Two kernels first unpack the operands into a workspace: the PTQ1_0 blocks
// into one byte per k (the fp4 pair (t, t)) and a float d_w per block, x
// into two bytes per k and a float d_x per block.  The GEMM kernel then
// streams both with buffer loads that write LDS directly (no registers,
// no decode in the product loop): a 512-lane workgroup computes a 256 (r) x
// 128 (c) tile, a wave 64 x 64 (2 x 2 products per sub-block, two waves per
// SIMD), K advancing 128 per step through a two-stage LDS ring (68 KiB per
// stage) with one barrier per step; each step's ten loads per lane are
// spread over the first five of its eight product groups.  Per group the
// products of the next one are issued before the current sums are scaled
// (software pipeline), their operand reads first and part of the VALU work
// in between, so the matrix cores run while the VALU scales.
//
// Operand layout of the product (checked on the device against a host
// reference): lane l holds row / column l % 32; A's 32 fp4 k slots of lane
// half h are slots 32 h + i, B's 32 fp8 bytes of half h pair with A's slots
// 16 h + i (i < 16) and 32 + 16 h + (i - 16).  So a lane half takes 16
// consecutive weight bytes (k 16 h .. 16 h + 15 of the sub-block) and the x
// bytes of k 8 h .. 8 h + 7 and 16 + 8 h .. 16 + 8 h + 7 (16-byte chunks h and
// 2 + h of the sub-block's 64 x bytes).

// PTQ1_0 blocks -> fp4 trit pairs [n][k] (one byte per k) and float block
// scales [n][k/128]: one lane per block
__global__ __launch_bounds__(256) void k_unpack_ptq1_0_fp4(const uint32_t* __restrict__ w, int64_t nb,
                                                           uint4* __restrict__ t4, float* __restrict__ dw) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * LUT_COPIES];
  tern_lut_init(lut);
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  uint32_t v[7];
#pragma unroll
  for (int q = 0; q < 7; ++q) v[q] = w[b * 7 + q];
  uint32_t dg[32];
  tern_decode(v, lut + (threadIdx.x & (LUT_COPIES - 1)), dg);
  // digit u -> the fp4 (e2m1) pair (t, t) of t = u - 1: 0xAA, 0x00, 0x22
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_perm(0u, 0x002200AAu, dg[4 * i + e]);
    t4[b * 8 + i] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  dw[b] = f16_to_f32(v[6] >> 16);
}

// PTQ1_1 superblocks -> the same fp4 trit pairs and float block scales as
// k_unpack_ptq1_0_fp4 (sub-block sub of superblock sb is block 8 sb + sub):
// one lane per sub-block, decoded with the codebook and escape tables staged
// in LDS as in the GEMV kernels
__global__ __launch_bounds__(256) void k_unpack_ptq1_1_fp4(const uint32_t* __restrict__ w, int64_t nb,
                                                           int bpr, SbTables sbt, uint4* __restrict__ t4,
                                                           float* __restrict__ dw) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * LUT_COPIES];
  __shared__ __attribute__((aligned(16))) uint32_t tbl[sb_lds_words(SB_ESC_MAX)];
  tern_lut_init(lut);
  tern_stage_sb(tbl, sbt);
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  const int64_t row = b / bpr;
  const int blk = (int)(b - row * bpr), sub = blk & 7, nit = bpr >> 3;
  const int64_t gidx = row * nit + (blk >> 3);  // the superblock (escape key)
  const uint32_t* sw = w + gidx * (SB_BYTES / 4);
  uint32_t v[12];
#pragma unroll
  for (int j = 0; j < 6; ++j) v[j] = sw[6 * sub + j];  // this sub-block's qs
#pragma unroll
  for (int j = 0; j < 6; ++j) v[6 + j] = sw[48 + j];   // the superblock's bytes 192..215
  uint32_t dg[32];
  float d;
  tern_decode_sb(v, lut + (threadIdx.x & (LUT_COPIES - 1)), tbl, sbt.n_esc, (int)gidx, sub, dg, d);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_perm(0u, 0x002200AAu, dg[4 * i + e]);
    t4[b * 8 + i] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  dw[b] = d;
}

// block_q8_1 -> fp8 pairs [c][2k] and float d_x [c][k/32]: one lane per block
template <bool PT>
__global__ __launch_bounds__(256) void k_unpack_q8_1_fp8(const uint8_t* __restrict__ xq, int64_t nb,
                                                         uint4* __restrict__ q8, float* __restrict__ dx,
                                                         int nsb) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  uint32_t v[9];
  if constexpr (PT) {
    const int col = (int)b / nsb;  // nb * 36 < 2^31
    uint32_t xw[8];
    xq_load<true>(xq, col, nsb, (int)b - col * nsb, v[0], xw);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[1 + q] = xw[q];
  } else {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(xq) + b * 9;  // the block's record
#pragma unroll
    for (int q = 0; q < 9; ++q) v[q] = src[q];
  }
  // k takes the fp8 (e4m3) pair (ql, 16 qh), both exact (the hardware's own
  // conversion, so the encoding is the one the products read)
  uint32_t o[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q0 = (int)(int8_t)(v[1 + i] >> (16 * h)), q1 = (int)(int8_t)(v[1 + i] >> (16 * h + 8));
      int w2 = __builtin_amdgcn_cvt_pk_fp8_f32((float)(q0 & 15), (float)((q0 >> 4) * 16), 0, false);
      w2 = __builtin_amdgcn_cvt_pk_fp8_f32((float)(q1 & 15), (float)((q1 >> 4) * 16), w2, true);
      o[2 * i + h] = (uint32_t)w2;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) q8[b * 4 + i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  dx[b] = f16_to_f32(v[0] & 0xFFFFu);
}

constexpr int TG_BN = 256, TG_BM = 128;  // weight rows, x rows per tile; 128 k per step
constexpr int TG_A = TG_BN * 128;        // 32 KiB of fp4 trit pairs
constexpr int TG_B = TG_BM * 128 * 2;    // 32 KiB of fp8 (ql, 16 qh) pairs
constexpr int TG_DX = TG_BM * 16;        // 4 d_x per x row
constexpr int TG_DW = 512 * 4;           // 256 d_w (and 256 unused words)
constexpr int TG_STAGE = TG_A + TG_B + TG_DX + TG_DW;
constexpr int TG_NST = 2;
// VALU instructions of a group's scaling placed before its first and second
// product (the rest after; 8 and 24 were best of 0-32)
constexpr int TG_V1 = 8, TG_V2 = 24;
// 16-byte chunk c of weight row r sits at chunk c ^ tg_swz(r) (and of x row r
// at c ^ (r % 16)): the 16 rows one ds_read_b128 cycle serves fall in 16
// distinct bank groups
__device__ __forceinline__ int tg_swz(int r) { return (r >> 1) & 7; }

// Workspace layout (byte offsets, 256-aligned) for the unpacked operands.
struct TernWs {
  size_t dw, x, dx, bytes;
};
inline TernWs tern_ws(int64_t n, int64_t k, int64_t c) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  TernWs w;
  w.dw = al((size_t)(n * k));
  w.x = w.dw + al((size_t)(n * (k / 128) * 4));
  w.dx = w.x + al((size_t)(c * k * 2));
  w.bytes = w.dx + al((size_t)(c * (k / 32) * 4));
  return w;
}

__global__ __launch_bounds__(512, 1) void k_gemm_ternary(const uint8_t* __restrict__ wt,
                                                         const float* __restrict__ dwf,
                                                         const uint8_t* __restrict__ xt,
                                                         const float* __restrict__ dxf,
                                                         float* __restrict__ out, int n, int k,
                                                         int m, int tiles_m) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[TG_NST * TG_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;  // the wave's 64 weight rows, 64 x rows
  const int bpr = k / 128, nsb = k / 32;
  const int tm = (int)blockIdx.x % tiles_m, tn = (int)blockIdx.x / tiles_m;
  const int n0 = tn * TG_BN, m0 = tm * TG_BM;
  const int rows_a = min(TG_BN, n - n0), rows_b = min(TG_BM, m - m0);
  // descriptors over this tile's rows; rows past n / m read as zero
  const intx4 ars = make_rsrc(wt + (int64_t)n0 * k, (uint32_t)rows_a * (uint32_t)k);
  const intx4 brs = make_rsrc(xt + (int64_t)m0 * 2 * k, (uint32_t)rows_b * (uint32_t)k * 2u);
  const intx4 xds = make_rsrc(dxf + (int64_t)m0 * nsb, (uint32_t)rows_b * (uint32_t)nsb * 4u);
  const intx4 wds = make_rsrc(dwf + (int64_t)n0 * bpr, (uint32_t)rows_a * (uint32_t)bpr * 4u);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // Loads of a step: 0..3 weights (16-byte slot s = 64 (8 i + wave) + lane:
  // row s / 8, stored chunk s % 8), 4..7 x (row s / 16, stored chunk s % 16),
  // 8 the d_x (word t: row t / 4, sub-block t % 4), 9 the d_w (row t < 256)
  uint32_t a_voff[4], b_voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = (i * 8 + wave) * 64 + lane, r = s >> 3;
    a_voff[i] = (uint32_t)r * (uint32_t)k + 16u * (uint32_t)((s & 7) ^ tg_swz(r));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = (i * 8 + wave) * 64 + lane, r = s >> 4;
    b_voff[i] = (uint32_t)r * (uint32_t)k * 2u + 16u * (uint32_t)((s & 15) ^ (r & 15));
  }
  const uint32_t dx_voff = (uint32_t)((tid >> 2) * nsb + (tid & 3)) * 4u;
  const uint32_t dw_voff = tid < TG_BN ? (uint32_t)(tid * bpr) * 4u : T_OOB;
  // Loads [first, last) of step kt into stage kt % 2.  Steps past the end
  // load at T_OOB (zeros into a stage no one reads), so every lane issues
  // ten loads per step and the vmcnt waits below hold.
  auto issue_part = [&](int kt, int first, int last) {
    const uint32_t st = lds0 + (uint32_t)(kt % TG_NST) * TG_STAGE;
    const bool live = kt < bpr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i >= first && i < last)
        dma16(ars, live ? a_voff[i] + (uint32_t)kt * 128u : T_OOB,
              __builtin_amdgcn_readfirstlane(st + (uint32_t)(i * 8 + wave) * 1024u));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 + i >= first && 4 + i < last)
        dma16(brs, live ? b_voff[i] + (uint32_t)kt * 256u : T_OOB,
              __builtin_amdgcn_readfirstlane(st + TG_A + (uint32_t)(i * 8 + wave) * 1024u));
    if (8 >= first && 8 < last)
      dma4(xds, live ? dx_voff + (uint32_t)kt * 16u : T_OOB,
           __builtin_amdgcn_readfirstlane(st + TG_A + TG_B + (uint32_t)wave * 256u));
    if (9 >= first && 9 < last)
      dma4(wds, live && dw_voff != T_OOB ? dw_voff + (uint32_t)kt * 4u : T_OOB,
           __builtin_amdgcn_readfirstlane(st + TG_A + TG_B + TG_DX + (uint32_t)wave * 256u));
  };

  typedef int i32x8 __attribute__((ext_vector_type(8)));
  floatx16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  const int l32 = lane & 31, lh = lane >> 5;

  // Step kt from stage kt % 2, while step kn's loads go out.  Product group
  // nn = 4 bi + j: row block bi, sub-block j, both column blocks.
  auto compute = [&](int kt, int kn) {
    const uint8_t* st = smem + (kt % TG_NST) * TG_STAGE;
    const int ra = wn * 64 + l32, rb = wm * 64 + l32;  // + 32 bi / + 32 bj (same swizzles)
    const int sa = tg_swz(ra), sbx = rb & 15;
    const float4 dxa = *reinterpret_cast<const float4*>(st + TG_A + TG_B + rb * 16);
    const float4 dxb = *reinterpret_cast<const float4*>(st + TG_A + TG_B + (rb + 32) * 16);
    const float dx[2][4] = {{dxa.x, dxa.y, dxa.z, dxa.w}, {dxb.x, dxb.y, dxb.z, dxb.w}};
    floatx16 sp[2][2];  // sums of group nn (slot nn % 2), column blocks 0 and 1
    floatx16 t[2];      // the row block's d_x-scaled sums over its sub-blocks so far
    intx4 opa;
    i32x8 opb[2];
    auto load = [&](int nn) {
      const int bi = nn >> 2, j = nn & 3, c = 2 * j + lh;
      opa = *reinterpret_cast<const intx4*>(st + (ra + 32 * bi) * 128 + ((c ^ sa) << 4));
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const uint8_t* row = st + TG_A + (rb + 32 * bj) * 256;
        const intx4 lo = *reinterpret_cast<const intx4*>(row + (((4 * j + lh) ^ sbx) << 4));
        const intx4 hi = *reinterpret_cast<const intx4*>(row + (((4 * j + 2 + lh) ^ sbx) << 4));
        opb[bj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    auto prod = [&](int nn) {
      const floatx16 z = {};
      const i32x8 a8 = __builtin_shufflevector(opa, opa, 0, 1, 2, 3, 0, 1, 2, 3);  // fp4: 4 words read
      // A fp4 (e2m1, cbsz 4), B fp8 (e4m3, blgp 0), block scales 2^0 (E8M0 127)
      sp[nn & 1][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, opb[0], z, 4, 0, 0, 0x7f, 0, 0x7f);
      sp[nn & 1][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, opb[1], z, 4, 0, 0, 0x7f, 0, 0x7f);
    };
    auto scale = [&](int nn) {
      const int j = nn & 3;
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          t[bj][e] = j == 0 ? dx[bj][j] * sp[nn & 1][bj][e] : fmaf(dx[bj][j], sp[nn & 1][bj][e], t[bj][e]);
    };
    auto finish = [&](int bi) {  // weight scales of this lane's 16 result rows (8 (e / 4) + 4 lh + e % 4)
      float dw[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(st + TG_A + TG_B + TG_DX + (wn * 64 + bi * 32 + 8 * g + 4 * lh) * 4);
        dw[4 * g] = v.x; dw[4 * g + 1] = v.y; dw[4 * g + 2] = v.z; dw[4 * g + 3] = v.w;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[bi][0][e] = fmaf(dw[e], t[0][e], acc[bi][0][e]);
        acc[bi][1][e] = fmaf(dw[e], t[1][e], acc[bi][1][e]);
      }
    };
    load(0);
    prod(0);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      // The memory clobber keeps group nn + 1's operand reads (and so its
      // products) in this region; the asm that takes t keeps the scaling of
      // nn here too (the compiler otherwise sank it below every product).
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (nn < 7) { load(nn + 1); prod(nn + 1); }
      scale(nn);
      asm volatile("" ::"v"(t[0]), "v"(t[1]));
      if ((nn & 3) == 3) finish(nn >> 2);
      if (nn < 7) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);      // the operand reads
        __builtin_amdgcn_sched_group_barrier(0x002, TG_V1, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one product
        __builtin_amdgcn_sched_group_barrier(0x002, TG_V2, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // the other
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 100, 0);
      if (nn < 5) {  // two of the next step's ten loads per group
        __builtin_amdgcn_sched_barrier(0);
        issue_part(kn, 2 * nn, 2 * nn + 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  asm volatile("s_nop 4");  // VALU-written SGPRs (descriptors) read by the first loads
  issue_part(0, 0, 10);
  wait_vmcnt<0>();
  __syncthreads();
  for (int kt = 0; kt < bpr; ++kt) {
    compute(kt, kt + 1);  // step kt + 1 into the other stage: every wave finished step kt - 1
    wait_vmcnt<0>();      // this lane's loads of step kt + 1 landed
    __syncthreads();      // all lanes': publishes stage kt + 1, frees stage kt
  }

  // y[c][r]: lane column c, rows r = 8 (e / 4) + 4 lh + e % 4 (four consecutive)
  const bool vec_ok = (n & 3) == 0;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int col = m0 + wm * 64 + bj * 32 + l32;
      if (col >= m) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = n0 + wn * 64 + bi * 32 + 8 * g + 4 * lh;
        float* dst = out + (int64_t)col * n + r;
        const floatx16& a = acc[bi][bj];
        if (vec_ok && r + 3 < n) {
          *reinterpret_cast<float4*>(dst) = make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r + e < n) dst[e] = a[4 * g + e];
        }
      }
    }
}

}  // namespace

hipError_t launch_pack_ptq1_0(const int8_t* trits, const uint16_t* d, int64_t n, int64_t k,
                              uint8_t* blocks, hipStream_t s) {
  const int64_t nb = n * (k / 128);
  hipLaunchKernelGGL(k_pack_ptq1_0, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, trits, d,
                     reinterpret_cast<uint32_t*>(blocks), nb);
  return hipGetLastError();
}

hipError_t launch_quantize_q8_1(const float* x, int64_t c, int64_t k, uint8_t* xq, bool pt,
                                hipStream_t s) {
  const int64_t nb = c * (k / 32);
  const dim3 grid((unsigned)((nb * 32 + 255) / 256));
  if (pt)
    hipLaunchKernelGGL(k_quantize_q8_1<true>, grid, dim3(256), 0, s, x, xq, nb, (int)(k / 32));
  else
    hipLaunchKernelGGL(k_quantize_q8_1<false>, grid, dim3(256), 0, s, x, xq, nb, (int)(k / 32));
  return hipGetLastError();
}

// Items in flight per lane.  Two (with registers for five waves per SIMD)
// ran c = 2 and 4 14-15% faster than four with four waves (K=5120,
// N=17280: 14.0 -> 11.9 and 18.4 -> 15.8 us), c = 1 and 8 the same: the
// shorter ring leaves the registers for a fifth wave, and more waves hide
// the table-read and permute latencies better than deeper prefetch.
constexpr int TP_D = 2;

// K-split launch (S = 2) when x fits in LDS; returns hipErrorInvalidValue (no
// launch) otherwise.  SB: PTQ1_1 superblocks with their tables.
template <int C, bool SB>
hipError_t launch_ternary_ksplit(const uint32_t* wp, const uint8_t* xq, int64_t n, int64_t k,
                                 int64_t c, float* out, const SbTables& sbt, bool pt, hipStream_t s) {
  constexpr int S = 2;
  const int64_t lds = 256 * LUT_COPIES * 4 + C * (k / 128) * XB_WORDS * 4 + C * (k / 32) * 8 +
                      4 * 8 * C * 4 + (SB ? sb_lds_words(sbt.n_esc) * 4 : 0);
  if (lds > 160 * 1024 || n * (k / 128) * PT_BYTES >= (int64_t(1) << 31) || n >= (int64_t(1) << 30))
    return hipErrorInvalidValue;
  const void* fn = pt ? reinterpret_cast<const void*>(&k_gemv_ternary_ksplit<C, TP_D, S, SB, true>)
                      : reinterpret_cast<const void*>(&k_gemv_ternary_ksplit<C, TP_D, S, SB, false>);
  static std::atomic<uint64_t> lds_ok[2];  // devices where the kernel may use all of the LDS
  const hipError_t e = allow_dynamic_lds(fn, lds_ok[pt], 160 * 1024);
  if (e != hipSuccess) return e;
  const int64_t nrg = (n + 7) / 8;
  const int64_t grid = (nrg + (4 / S) - 1) / (4 / S);
  int n_arg = (int)n, k_arg = (int)k, c_arg = (int)c;
  SbTables t = sbt;
  void* args[] = {const_cast<uint32_t**>(&wp), const_cast<uint8_t**>(&xq), &out, &n_arg, &k_arg, &c_arg, &t};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, (size_t)lds, s);
}

// Persistent launch when x fits in LDS; returns hipErrorInvalidValue (no
// launch) otherwise.
template <int C, bool SB>
hipError_t launch_ternary_persist(const uint32_t* wp, const uint8_t* xq, int64_t n, int64_t k,
                                  int64_t c, float* out, const SbTables& sbt, bool pt, hipStream_t s) {
  const int64_t lds = 256 * LUT_COPIES * 4 + C * (k / 128) * XB_WORDS * 4 + C * (k / 32) * 8 +
                      (SB ? sb_lds_words(sbt.n_esc) * 4 : 0);
  if (lds > 160 * 1024 || n * (k / 128) * PT_BYTES >= (int64_t(1) << 31) || n >= (int64_t(1) << 30))
    return hipErrorInvalidValue;
  const void* fn = pt ? reinterpret_cast<const void*>(&k_gemv_ternary_persist<C, TP_D, TP_LPR, SB, true>)
                      : reinterpret_cast<const void*>(&k_gemv_ternary_persist<C, TP_D, TP_LPR, SB, false>);
  static std::atomic<uint64_t> lds_ok[2];  // devices where the kernel may use all of the LDS
  const hipError_t e = allow_dynamic_lds(fn, lds_ok[pt], 160 * 1024);
  if (e != hipSuccess) return e;
  const int64_t nrg = (n + 64 / TP_LPR - 1) / (64 / TP_LPR);
  // workgroups resident at once: LDS and the waves per SIMD the register
  // budget allows
  const int per_cu = (int)std::max<int64_t>(1, std::min<int64_t>(SB ? TP_WAVES_SB : TP_WAVES, (160 * 1024) / lds));
  const int64_t grid = std::min<int64_t>((nrg + 3) / 4, (int64_t)device_cu_count() * per_cu);
  int n_arg = (int)n, k_arg = (int)k, c_arg = (int)c;
  SbTables t = sbt;
  void* args[] = {const_cast<uint32_t**>(&wp), const_cast<uint8_t**>(&xq), &out, &n_arg, &k_arg, &c_arg, &t};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, (size_t)lds, s);
}

// Largest number of 8-row groups one wave of k_gemv_ternary_mq touches, over
// the two row counts (q and q + 1) the workgroups get.
int tm_slots(int64_t n, int grid, int nit) {
  const int64_t qn = n / grid;
  int best = 1;
  for (int64_t cnt = qn; cnt <= qn + 1; ++cnt) {
    const int64_t items = ((cnt + 7) / 8) * nit;
    for (int h = 0; h < TM_NW; ++h) {
      const int64_t a = h * items / TM_NW, b = (h + 1) * items / TM_NW;
      if (b > a) best = std::max(best, (int)((b - 1) / nit - a / nit + 1));
    }
  }
  return best;
}

// The matrix-core GEMV for c <= C when x and the table fit in LDS; returns
// hipErrorInvalidValue (no launch) otherwise.
template <int C, bool SB>
hipError_t launch_ternary_mq(const uint32_t* wp, const uint8_t* xq, int64_t n, int64_t k, int64_t c,
                             float* out, const SbTables& sbt, bool pt, hipStream_t s) {
  constexpr int D = 2;
  if (n >= (int64_t(1) << 30) || k >= (int64_t(1) << 24)) return hipErrorInvalidValue;
  const int64_t bpr = k / 128;
  int grid = device_cu_count();
  if ((int64_t)grid * 8 > n) grid = (int)std::max<int64_t>(1, n / 8);
  const int64_t maxrows = (n + grid - 1) / grid + 8;
  if (maxrows * bpr * PT_BYTES >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (SB && bpr % 8 != 0) return hipErrorInvalidValue;  // whole superblocks
  const int nit = (int)((bpr + 7) / 8);
  const int spw = tm_slots(n, grid, nit);
  // (at least 64 KiB: a table address of any byte value, 243..255 included,
  // stays inside the allocation)
  const int64_t lds = std::max<int64_t>(
      65536, TM_LUT_BYTES + bpr * tm_record(C) + (SB ? sb_lds_words(sbt.n_esc) * 4 : 0) +
                 (int64_t)TM_NW * spw * 8 * C * 4 + TM_NW * 3 * 4);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const void* fn = pt ? reinterpret_cast<const void*>(&k_gemv_ternary_mq<C, D, SB, true>)
                      : reinterpret_cast<const void*>(&k_gemv_ternary_mq<C, D, SB, false>);
  static std::atomic<uint64_t> lds_ok[2];  // devices where the kernel may use all of the LDS
  const hipError_t e = allow_dynamic_lds(fn, lds_ok[pt], 160 * 1024);
  if (e != hipSuccess) return e == hipErrorInvalidValue ? hipErrorNotSupported : e;
  int n_arg = (int)n, k_arg = (int)k, c_arg = (int)c, spw_arg = spw;
  SbTables t = sbt;
  void* args[] = {const_cast<uint32_t**>(&wp), const_cast<uint8_t**>(&xq), &out, &n_arg, &k_arg, &c_arg, &spw_arg, &t};
  return hipLaunchKernel(fn, dim3(grid), dim3(TM_NT), args, (size_t)lds, s);
}

// Up to 16 columns on the vector units.
hipError_t launch_ternary_narrow(const uint8_t* w, const uint8_t* xq, int64_t n, int64_t k,
                                 int64_t c, float* out, bool pt, hipStream_t s) {
  const uint32_t* wp0 = reinterpret_cast<const uint32_t*>(w);
  {
    // one column: the K-split kernel (wider splits spilled registers; the
    // matrix-core kernel was 3-6% slower at one column, and needs more LDS);
    // 2-8 columns: the matrix-core kernel
    const SbTables none{};
    hipError_t e = hipErrorInvalidValue;
    if (c == 1) {
      e = launch_ternary_ksplit<1, false>(wp0, xq, n, k, c, out, none, pt, s);
      if (e != hipErrorInvalidValue) return e;
    }
    switch (c) {
      case 1: break;
      case 2: e = launch_ternary_mq<2, false>(wp0, xq, n, k, c, out, none, pt, s); break;
      case 3: case 4: e = launch_ternary_mq<4, false>(wp0, xq, n, k, c, out, none, pt, s); break;
      default: if (c <= 8) e = launch_ternary_mq<8, false>(wp0, xq, n, k, c, out, none, pt, s); break;
    }
    if (e != hipErrorInvalidValue) return e;
    switch (c) {
      case 1: break;
      case 2: e = launch_ternary_persist<2, false>(wp0, xq, n, k, c, out, none, pt, s); break;
      case 3: case 4: e = launch_ternary_persist<4, false>(wp0, xq, n, k, c, out, none, pt, s); break;
      default: if (c <= 8) e = launch_ternary_persist<8, false>(wp0, xq, n, k, c, out, none, pt, s); break;
    }
    if (e != hipErrorInvalidValue) return e;
  }
  const unsigned blocks = (unsigned)((n + 31) / 32);
  const uint32_t* wp = reinterpret_cast<const uint32_t*>(w);
#define WQ_TG(C)                                                                                    \
  do {                                                                                              \
    if (pt)                                                                                         \
      hipLaunchKernelGGL((k_gemv_ternary<C, true>), dim3(blocks), dim3(256), 0, s, wp, xq, out, n, k, (int)c); \
    else                                                                                            \
      hipLaunchKernelGGL((k_gemv_ternary<C, false>), dim3(blocks), dim3(256), 0, s, wp, xq, out, n, k, (int)c); \
  } while (0)
  switch (c) {
    case 1: WQ_TG(1); break;
    case 2: WQ_TG(2); break;
    case 3: WQ_TG(3); break;
    case 4: WQ_TG(4); break;
    default:
      if (c <= 8) { WQ_TG(8); } else { WQ_TG(16); }
      break;
  }
#undef WQ_TG
  return hipGetLastError();
}


size_t gemm_ternary_workspace(int64_t n, int64_t k, int64_t c) { return tern_ws(n, k, c).bytes; }

// x unpacked and the product, once the weights are in the workspace
static hipError_t gemm_ternary_unpacked(const uint8_t* xq, bool pt, int64_t n, int64_t k, int64_t c,
                                        float* out, uint8_t* base, hipStream_t s) {
  const TernWs L = tern_ws(n, k, c);
  const int64_t nbx = c * (k / 32);
  const dim3 ugrid((unsigned)((nbx + 255) / 256));
  if (pt)
    hipLaunchKernelGGL(k_unpack_q8_1_fp8<true>, ugrid, dim3(256), 0, s, xq, nbx,
                       reinterpret_cast<uint4*>(base + L.x), reinterpret_cast<float*>(base + L.dx), (int)(k / 32));
  else
    hipLaunchKernelGGL(k_unpack_q8_1_fp8<false>, ugrid, dim3(256), 0, s, xq, nbx,
                       reinterpret_cast<uint4*>(base + L.x), reinterpret_cast<float*>(base + L.dx), (int)(k / 32));
  const int tiles_m = (int)((c + TG_BM - 1) / TG_BM), tiles_n = (int)((n + TG_BN - 1) / TG_BN);
  hipLaunchKernelGGL(k_gemm_ternary, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, s, base,
                     reinterpret_cast<const float*>(base + L.dw), base + L.x,
                     reinterpret_cast<const float*>(base + L.dx), out, (int)n, (int)k, (int)c, tiles_m);
  return hipGetLastError();
}

hipError_t launch_gemm_ternary(const uint8_t* w, const uint8_t* xq, bool pt, int64_t n, int64_t k,
                               int64_t c, float* out, void* ws, hipStream_t s) {
  const TernWs L = tern_ws(n, k, c);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const int64_t nbw = n * (k / 128);
  hipLaunchKernelGGL(k_unpack_ptq1_0_fp4, dim3((unsigned)((nbw + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(w), nbw, reinterpret_cast<uint4*>(base),
                     reinterpret_cast<float*>(base + L.dw));
  return gemm_ternary_unpacked(xq, pt, n, k, c, out, base, s);
}

// The GEMM's workspace comes from a memory pool of this library's own, one
// per device, allocated and freed in stream order around each call; its
// release threshold is at the maximum, so what a call frees stays in the
// pool for the next one.
static hipError_t tern_pool(hipMemPool_t* pool) {
  static std::mutex mu;
  static hipMemPool_t pools[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!pools[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    e = hipMemPoolCreate(&p, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(p);
      return e;
    }
    pools[dev] = p;
  }
  *pool = pools[dev];
  return hipSuccess;
}

// Scratch of the entry point that allocates nothing: the GEMM's unpacked
// operands, at most kTernScratchBytes.  Every device holds its own copy for
// the life of the process.  In host code `scratch` names a host-side stand-in;
// its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kTernScratchBytes];

static hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with this device current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_gemv_ternary_noalloc(const uint8_t* w, const uint8_t* xq, int64_t n, int64_t k,
                                       int64_t c, float* out, hipStream_t s) {
  if (c < 64) return launch_gemv_ternary(w, xq, false, n, k, c, out, s);  // no workspace below 64 columns
  if (gemm_ternary_workspace(n, k, c) > kTernScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_gemm_ternary(w, xq, false, n, k, c, out, ws, s);
}

// run(ws) with a workspace of `bytes` from the pool, freed in stream order
template <class F>
static hipError_t with_pool_workspace(size_t bytes, hipStream_t s, F run) {
  hipMemPool_t pool = nullptr;
  hipError_t e = tern_pool(&pool);
  if (e != hipSuccess) return e;
  void* ws = nullptr;
  e = hipMallocFromPoolAsync(&ws, bytes, pool, s);
  if (e != hipSuccess) return e;
  e = run(ws);
  const hipError_t f = hipFreeAsync(ws, s);
  return e != hipSuccess ? e : f;
}

hipError_t launch_gemv_ternary(const uint8_t* w, const uint8_t* xq, bool pt, int64_t n, int64_t k,
                               int64_t c, float* out, hipStream_t s) {
  if (c >= 64)  // a batch wide enough for the matrix cores
    return with_pool_workspace(gemm_ternary_workspace(n, k, c), s,
                               [&](void* ws) { return launch_gemm_ternary(w, xq, pt, n, k, c, out, ws, s); });
  // 17..63 columns: passes of at most 16 over x[c0:c0+16] -> out[c0:c0+16]
  for (int64_t c0 = 0; c0 < c; c0 += 16) {
    const hipError_t e = launch_ternary_narrow(w, xq + c0 * (k / 32) * Q8_BYTES, n, k,
                                               std::min<int64_t>(16, c - c0), out + c0 * n, pt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// PTQ1_1 superblocks: passes of at most 8 columns on the kernels that keep
// x in LDS (the widest pass that fits; the matrix-core kernel first, then
// the vector kernels); hipErrorInvalidValue when even one column does not
// fit (the entry point bounds k so that it does).
hipError_t launch_gemv_ternary_sb(const uint8_t* w, const uint8_t* codebook, const int32_t* esc_idx,
                                  const uint8_t* esc_patt, int64_t n_esc, const uint8_t* xq, bool pt,
                                  int64_t n, int64_t k, int64_t c, float* out, hipStream_t s) {
  const uint32_t* wp = reinterpret_cast<const uint32_t*>(w);
  const SbTables t{codebook, esc_idx, esc_patt, (int)n_esc};
  if (c >= 64) {  // a prefill batch: the superblocks unpacked, then the matrix-core product
    return with_pool_workspace(gemm_ternary_workspace(n, k, c), s, [&](void* ws) {
      const TernWs L = tern_ws(n, k, c);
      uint8_t* base = static_cast<uint8_t*>(ws);
      const int64_t nbw = n * (k / 128);
      hipLaunchKernelGGL(k_unpack_ptq1_1_fp4, dim3((unsigned)((nbw + 255) / 256)), dim3(256), 0, s, wp,
                         nbw, (int)(k / 128), t, reinterpret_cast<uint4*>(base),
                         reinterpret_cast<float*>(base + L.dw));
      return gemm_ternary_unpacked(xq, pt, n, k, c, out, base, s);
    });
  }
  for (int64_t c0 = 0; c0 < c; ) {
    const int64_t left = c - c0;
    const uint8_t* xp = xq + c0 * (k / 32) * Q8_BYTES;
    float* op = out + c0 * n;
    hipError_t e = hipErrorInvalidValue;
    int64_t done = 0;
    if (left == 1) {
      // the matrix-core kernel (its two-column form, column 0 repeated: 7%
      // faster than the K-split kernel here), else the K-split kernel
      e = launch_ternary_mq<2, true>(wp, xp, n, k, 1, op, t, pt, s);
      if (e == hipErrorInvalidValue) e = launch_ternary_ksplit<1, true>(wp, xp, n, k, 1, op, t, pt, s);
      done = 1;
    } else {
      // widest pass first, the matrix-core kernel before the vector one; a
      // pass that does not fit its x in LDS launches nothing
      const int64_t w8 = std::min<int64_t>(8, left), w4 = std::min<int64_t>(4, left);
      if (left >= 5) { e = launch_ternary_mq<8, true>(wp, xp, n, k, w8, op, t, pt, s); done = w8; }
      if (e == hipErrorInvalidValue && left >= 5) { e = launch_ternary_persist<8, true>(wp, xp, n, k, w8, op, t, pt, s); done = w8; }
      if (e == hipErrorInvalidValue && left >= 3) { e = launch_ternary_mq<4, true>(wp, xp, n, k, w4, op, t, pt, s); done = w4; }
      if (e == hipErrorInvalidValue && left >= 3) { e = launch_ternary_persist<4, true>(wp, xp, n, k, w4, op, t, pt, s); done = w4; }
      if (e == hipErrorInvalidValue) { e = launch_ternary_mq<2, true>(wp, xp, n, k, 2, op, t, pt, s); done = 2; }
      if (e == hipErrorInvalidValue) { e = launch_ternary_persist<2, true>(wp, xp, n, k, 2, op, t, pt, s); done = 2; }
      if (e == hipErrorInvalidValue) { e = launch_ternary_ksplit<1, true>(wp, xp, n, k, 1, op, t, pt, s); done = 1; }
    }
    if (e != hipSuccess) return e;
    c0 += done;
  }
  return hipSuccess;
}

}  // namespace wq
