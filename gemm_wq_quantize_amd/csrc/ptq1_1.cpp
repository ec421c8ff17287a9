// PTQ1_1 superblock encoder (host): groups the PTQ1_0 blocks of each row in
// eights, per the Ternary post, section 2 (struct ptq1_1: qs[192], qh[13],
// eight 10-bit mantissas, one exponent byte; the exponent byte and the free
// trit of qh index 768 exponent patterns, 767 meaning "look the superblock up
// in an external table").  Compression is an offline step of weight
// preparation, done once on the host; the GEMV decodes on the device.
//
// Bit positions (the post gives sizes, not positions):
//   bytes   0..191  the qs[24] of sub-blocks 0..7 in order
//   bytes 192..204  qh[13]: tail trit t = 8 sub + e (element 120 + e of
//                   sub-block sub, digit u = trit + 1) is base-3 digit t % 5
//                   of byte t / 5, digit 0 least significant; digit 4 of
//                   qh[12] is the free trit
//   bytes 205..214  80-bit little-endian field, mantissa sub at bit 10 sub
//   byte  215       exponent byte
//   pattern index P = exponent byte + 256 * free digit; P < 767 is a row of
//   the codebook, P = 767 an escape (escape table: ascending superblock
//   indices row * k/1024 + sb and their 8 exponents).
// The codebook holds the tensor's most frequent exponent patterns, ties by
// increasing pattern (exponents compared in sub-block order), at most 767.
#include "../../include/wq.h"

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <utility>
#include <vector>

namespace {

constexpr int kBlockBytes = 28;
constexpr int kSbBytes = 216;
constexpr int kCodebookRows = 767;

// The 8 exponent fields of one superblock as a 40-bit key whose numeric
// order is the lexicographic order of (e0, ..., e7).
uint64_t pattern_key(const uint16_t (&d)[8]) {
  uint64_t key = 0;
  for (int sub = 0; sub < 8; ++sub) key = (key << 5) | ((d[sub] >> 10) & 0x1Fu);
  return key;
}

void key_exponents(uint64_t key, uint8_t* out) {
  for (int sub = 7; sub >= 0; --sub) {
    out[sub] = (uint8_t)(key & 0x1Fu);
    key >>= 5;
  }
}

}  // namespace

extern "C" int wq_ptq1_1_encode(const uint8_t* blocks, int64_t n, int64_t k, uint8_t* superblocks,
                                uint8_t* codebook, int32_t* esc_idx, uint8_t* esc_patt,
                                int64_t esc_cap, int64_t* n_esc) {
  if (n < 0 || k < 0 || esc_cap < 0 || !n_esc) return WQ_EINVAL;
  *n_esc = 0;
  if (!codebook) return WQ_EINVAL;
  std::memset(codebook, 0, (size_t)kCodebookRows * 8);
  if (n == 0 || k == 0) return WQ_OK;
  if (!blocks || !superblocks || (esc_cap > 0 && (!esc_idx || !esc_patt))) return WQ_EINVAL;
  if (k % 1024 != 0) return WQ_ESHAPE;
  const int64_t nsb = k / 1024, total = n * nsb;
  if (n > (int64_t(1) << 31) / nsb) return WQ_ESHAPE;  // 32-bit superblock indices

  // scales of every superblock; d must be >= +0 (the format stores no sign)
  auto scale_bits = [&](int64_t g, int sub) -> uint16_t {
    const uint8_t* b = blocks + (g * 8 + sub) * kBlockBytes;
    return (uint16_t)(b[26] | (b[27] << 8));
  };
  std::unordered_map<uint64_t, int64_t> counts;
  std::vector<uint64_t> keys((size_t)total);
  for (int64_t g = 0; g < total; ++g) {
    uint16_t d[8];
    for (int sub = 0; sub < 8; ++sub) {
      d[sub] = scale_bits(g, sub);
      if (d[sub] & 0x8000u) return WQ_EINVAL;
    }
    keys[(size_t)g] = pattern_key(d);
    ++counts[keys[(size_t)g]];
  }
  // the codebook: by decreasing count, ties by increasing pattern
  std::vector<std::pair<uint64_t, int64_t>> ranked(counts.begin(), counts.end());
  std::sort(ranked.begin(), ranked.end(), [](const auto& a, const auto& b) {
    return a.second != b.second ? a.second > b.second : a.first < b.first;
  });
  std::unordered_map<uint64_t, int> row_of;
  const int rows = (int)std::min<size_t>(ranked.size(), kCodebookRows);
  for (int r = 0; r < rows; ++r) {
    row_of[ranked[(size_t)r].first] = r;
    key_exponents(ranked[(size_t)r].first, codebook + 8 * r);
  }
  int64_t escapes = 0;
  for (int64_t g = 0; g < total; ++g)
    if (!row_of.count(keys[(size_t)g])) ++escapes;
  *n_esc = escapes;
  if (escapes > esc_cap) return WQ_ESHAPE;

  int64_t e_out = 0;
  for (int64_t g = 0; g < total; ++g) {
    const uint8_t* src = blocks + g * 8 * kBlockBytes;
    uint8_t* dst = superblocks + g * kSbBytes;
    std::memset(dst, 0, kSbBytes);
    // qs of the eight sub-blocks, unchanged
    for (int sub = 0; sub < 8; ++sub) std::memcpy(dst + 24 * sub, src + sub * kBlockBytes, 24);
    // tail trits: element 120 + e of a block is the 2-bit digit at bits
    // 2 (e >> 1) of its qh[e & 1]; superblock tail trit 8 sub + e
    static const int pow3[5] = {1, 3, 9, 27, 81};
    int qh[13] = {0};
    for (int sub = 0; sub < 8; ++sub)
      for (int e = 0; e < 8; ++e) {
        const int u = (src[sub * kBlockBytes + 24 + (e & 1)] >> (2 * (e >> 1))) & 3;
        const int t = 8 * sub + e;
        qh[t / 5] += u * pow3[t % 5];
      }
    auto it = row_of.find(keys[(size_t)g]);
    const int p = it != row_of.end() ? it->second : kCodebookRows;
    qh[12] += (p >> 8) * pow3[4];  // the free trit
    for (int j = 0; j < 13; ++j) dst[192 + j] = (uint8_t)qh[j];
    // mantissas: 80-bit little-endian field
    uint64_t lo = 0, hi = 0;
    for (int sub = 0; sub < 8; ++sub) {
      const uint64_t m = scale_bits(g, sub) & 0x3FFu;
      const int bit = 10 * sub;
      if (bit < 64) {
        lo |= m << bit;
        if (bit + 10 > 64) hi |= m >> (64 - bit);
      } else {
        hi |= m << (bit - 64);
      }
    }
    for (int j = 0; j < 8; ++j) dst[205 + j] = (uint8_t)(lo >> (8 * j));
    dst[213] = (uint8_t)hi;
    dst[214] = (uint8_t)(hi >> 8);
    dst[215] = (uint8_t)(p & 0xFF);
    if (p == kCodebookRows) {
      esc_idx[e_out] = (int32_t)g;
      key_exponents(keys[(size_t)g], esc_patt + 8 * e_out);
      ++e_out;
    }
  }
  return WQ_OK;
}
