// C ABI of libwq: argument validation, then one launch on the caller's
// stream.  Every check happens before any HIP call, so a rejected call
// enqueues nothing and touches no output.
#include "../../include/wq.h"
#include "wq_internal.h"

#include <cstdint>

namespace {

constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// a * b for non-negative sizes, saturated at INT64_MAX (so that size checks
// on absurd arguments cannot wrap round and pass)
int64_t mul_sat(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// group is k itself, or a power of two >= 32 dividing k
bool valid_group(int64_t group, int64_t k) {
  if (group == k) return true;
  return is_pow2(group) && group >= 32 && group <= k && k % group == 0;
}

int dtype_size(int dt) { return dt == WQ_F32 ? 4 : 2; }

int hip_status(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_EHIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }


// shared validation and launch of the two GEMM entry points (zeros nullable)
int gemm_w4a16(const uint16_t* a, const uint8_t* b, int layout, const uint16_t* scales,
               const uint16_t* zeros, int64_t group, float zero_const, int64_t m, int64_t n,
               int64_t k, uint16_t* c_out, void* stream) {
  if (m < 0 || n < 0 || k < 0 || group < 0) return WQ_EINVAL;
  if (layout != WQ_LAYOUT_PLAIN && layout != WQ_LAYOUT_GFX950) return WQ_EINVAL;
  if (m == 0 || n == 0) return WQ_OK;
  if (!a || !b || !scales || !c_out) return WQ_EINVAL;
  if (k == 0 || k % 64 != 0 || k > (int64_t(1) << 22)) return WQ_ESHAPE;  // 32-bit tile offsets
  // one scale per column, or per group of a power-of-two multiple of 64 k
  if (!valid_group(group, k)) return WQ_ESHAPE;
  const bool grouped = group != k;
  if (grouped && group < 64) return WQ_EUNSUPPORTED;  // a 64-k step must lie in one group
  if (layout != WQ_LAYOUT_GFX950) return WQ_EUNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c_out, 16) ||
      !aligned(scales, grouped ? 4 : 2) || (zeros && !aligned(zeros, grouped ? 4 : 2)))
    return WQ_EALIGN;
  if (mul_sat(m / 256 + 1, n / 256 + 1) > kMaxGrid) return WQ_ESHAPE;
  return hip_status(wq::launch_gemm_w4a16(a, b, scales, zeros, group, zero_const, m, n, k, c_out,
                                          as_stream(stream)));
}
// shared validation of the two ternary GEMV entry points; *launch is false
// for an empty problem (WQ_OK, nothing to enqueue)
int check_gemv_ternary(const uint8_t* w_blocks, const uint8_t* x_q8, int64_t n, int64_t k, int64_t c,
                       const float* out, bool* launch) {
  *launch = false;
  if (n < 0 || k < 0 || c < 0) return WQ_EINVAL;
  if (n == 0 || c == 0) return WQ_OK;
  if (!w_blocks || !x_q8 || !out) return WQ_EINVAL;
  // up to 16 columns per pass on the vector units; 64 or more on the fp4 x fp8 matrix cores
  if (k == 0 || k % 128 != 0) return WQ_ESHAPE;
  if (!aligned(w_blocks, 4) || !aligned(x_q8, 4) || !aligned(out, c >= 64 ? 16 : 4)) return WQ_EALIGN;
  if (n / 32 + 1 > kMaxGrid) return WQ_ESHAPE;
  if (c >= 64) {  // 32-bit buffer offsets and the tile grid
    if (mul_sat(mul_sat(n, k / 128), 28) >= (int64_t(1) << 31) ||
        mul_sat(mul_sat(c, k / 32), 36) >= (int64_t(1) << 31))
      return WQ_ESHAPE;
    if (mul_sat(c / 128 + 1, n / 128 + 1) > kMaxGrid) return WQ_ESHAPE;
  }
  *launch = true;
  return WQ_OK;
}
int quantize_q8_1(const float* x, int64_t c, int64_t k, uint8_t* x_q8, bool pt, void* stream) {
  if (c < 0 || k < 0) return WQ_EINVAL;
  if (c == 0 || k == 0) return WQ_OK;
  if (!x || !x_q8) return WQ_EINVAL;
  if (k % (pt ? 128 : 32) != 0) return WQ_ESHAPE;
  if (pt && k > (int64_t(1) << 30)) return WQ_ESHAPE;  // a column's plane offsets in 32 bits
  if (!aligned(x, 16) || !aligned(x_q8, 4)) return WQ_EALIGN;
  if (mul_sat(c, k) / 256 + 1 > kMaxGrid) return WQ_ESHAPE;
  return hip_status(wq::launch_quantize_q8_1(x, c, k, x_q8, pt, as_stream(stream)));
}

int gemv_ternary_ptq1_1(const uint8_t* superblocks, const uint8_t* codebook, const int32_t* esc_idx,
                        const uint8_t* esc_patt, int64_t n_esc, const uint8_t* x_q8, bool pt, int64_t n,
                        int64_t k, int64_t c, float* out, void* stream) {
  if (n < 0 || k < 0 || c < 0 || n_esc < 0) return WQ_EINVAL;
  if (n == 0 || c == 0) return WQ_OK;
  if (!superblocks || !codebook || !x_q8 || !out || (n_esc > 0 && (!esc_idx || !esc_patt)))
    return WQ_EINVAL;
  // superblocks of 8 blocks; x of one column must fit in LDS beside the tables
  if (k == 0 || k % 1024 != 0 || k > 65536) return WQ_ESHAPE;
  if (n_esc > 2048) return WQ_EUNSUPPORTED;  // escape table staged in LDS
  if (n >= (int64_t(1) << 30) || mul_sat(mul_sat(n, k / 128), 28) >= (int64_t(1) << 31))
    return WQ_ESHAPE;
  if (c >= 64) {  // the matrix-core product: activations' 32-bit offsets and the tile grid
    if (mul_sat(mul_sat(c, k / 32), 36) >= (int64_t(1) << 31)) return WQ_ESHAPE;
    if (mul_sat(c / 128 + 1, n / 128 + 1) > kMaxGrid) return WQ_ESHAPE;
  }
  if (!aligned(superblocks, 4) || !aligned(codebook, 4) || !aligned(x_q8, 4) ||
      !aligned(out, c >= 64 ? 16 : 4) || (n_esc > 0 && (!aligned(esc_idx, 4) || !aligned(esc_patt, 4))))
    return WQ_EALIGN;
  return hip_status(wq::launch_gemv_ternary_sb(superblocks, codebook, esc_idx, esc_patt, n_esc, x_q8, pt,
                                               n, k, c, out, as_stream(stream)));
}
}  // namespace

extern "C" {

int wq_abi_version(void) { return 1; }

const char* wq_status_string(int status) {
  switch (status) {
    case WQ_OK: return "WQ_OK";
    case WQ_EINVAL: return "WQ_EINVAL: null pointer, bad enum or negative size";
    case WQ_EALIGN: return "WQ_EALIGN: pointer misaligned for this call";
    case WQ_ESHAPE: return "WQ_ESHAPE: sizes violate this call's divisibility or limits";
    case WQ_EUNSUPPORTED: return "WQ_EUNSUPPORTED: valid request the library does not implement";
    case WQ_EHIP: return "WQ_EHIP: HIP runtime error at launch";
    default: return "unknown wq_status";
  }
}

int wq_pack_int4(const uint8_t* codes, int64_t n, int64_t k, int layout, uint8_t* packed,
                 void* stream) {
  if (n < 0 || k < 0 || (layout != WQ_LAYOUT_PLAIN && layout != WQ_LAYOUT_GFX950)) return WQ_EINVAL;
  if (n == 0 || k == 0) return WQ_OK;
  if (!codes || !packed) return WQ_EINVAL;
  if (k % 8 != 0) return WQ_ESHAPE;
  if (!aligned(codes, 4) || !aligned(packed, 4)) return WQ_EALIGN;
  if (mul_sat(n, k) / 8 / 256 + 1 > kMaxGrid) return WQ_ESHAPE;
  return hip_status(wq::launch_pack_int4(codes, n, k, layout, packed, as_stream(stream)));
}

int wq_quantize_pack_int4(const uint16_t* w, int64_t n, int64_t k, int64_t group, int layout,
                          uint8_t* packed, void* scales, int scale_dtype, void* stream) {
  if (n < 0 || k < 0 || group < 0) return WQ_EINVAL;
  if (layout != WQ_LAYOUT_PLAIN && layout != WQ_LAYOUT_GFX950) return WQ_EINVAL;
  if (scale_dtype != WQ_F32 && scale_dtype != WQ_BF16) return WQ_EINVAL;
  if (n == 0 || k == 0) return WQ_OK;
  if (!w || !packed || !scales) return WQ_EINVAL;
  if (k % 32 != 0 || !valid_group(group, k)) return WQ_ESHAPE;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, dtype_size(scale_dtype)))
    return WQ_EALIGN;
  if (mul_sat(mul_sat(n, k / group), 64) / 256 + 1 > kMaxGrid) return WQ_ESHAPE;
  return hip_status(wq::launch_quantize_pack_int4(w, n, k, group, layout, packed, scales,
                                                  scale_dtype == WQ_BF16, as_stream(stream)));
}

int wq_gemv_w4(const uint8_t* packed, int layout, const void* scales, int scale_dtype,
               const void* zeros, float zero_const, int64_t n, int64_t k, int64_t group,
               const void* x, int x_dtype, int64_t c, void* out, int out_dtype, void* stream) {
  if (n < 0 || k < 0 || c < 0 || group < 0) return WQ_EINVAL;
  if (layout != WQ_LAYOUT_PLAIN && layout != WQ_LAYOUT_GFX950) return WQ_EINVAL;
  if (scale_dtype != WQ_F32 && scale_dtype != WQ_BF16) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EINVAL;
  if (out_dtype != WQ_F32 && out_dtype != WQ_BF16) return WQ_EINVAL;
  if (n == 0 || c == 0) return WQ_OK;
  if (!packed || !scales || !x || !out) return WQ_EINVAL;
  if (k == 0 || k % 32 != 0 || k > (int64_t(1) << 24) || !valid_group(group, k) || c > 32)
    return WQ_ESHAPE;  // k bound: 32-bit buffer offsets in every kernel
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(scales, dtype_size(scale_dtype)) ||
      (zeros && !aligned(zeros, dtype_size(scale_dtype))) || !aligned(out, dtype_size(out_dtype)))
    return WQ_EALIGN;
  if (n / 8 + 1 > kMaxGrid) return WQ_ESHAPE;
  wq::GemvArgs a;
  a.packed = packed;
  a.scales = scales;
  a.zeros = zeros;
  a.x = x;
  a.out = out;
  a.n = n;
  a.k = k;
  a.group = group;
  a.c = c;
  a.zero_const = zero_const;
  a.layout = layout;
  a.scale_bf16 = scale_dtype == WQ_BF16;
  a.x_bf16 = x_dtype == WQ_BF16;
  a.out_bf16 = out_dtype == WQ_BF16;
  return hip_status(wq::launch_gemv_w4(a, as_stream(stream)));
}


int wq_gemm_w4a16(const uint16_t* a, const uint8_t* b, int layout, const uint16_t* scales,
                  int64_t group, float zero_const, int64_t m, int64_t n, int64_t k,
                  uint16_t* c_out, void* stream) {
  return gemm_w4a16(a, b, layout, scales, nullptr, group, zero_const, m, n, k, c_out, stream);
}

int wq_gemm_w4a16_zp(const uint16_t* a, const uint8_t* b, int layout, const uint16_t* scales,
                     const uint16_t* zeros, int64_t group, int64_t m, int64_t n, int64_t k,
                     uint16_t* c_out, void* stream) {
  if (!zeros && m > 0 && n > 0) return WQ_EINVAL;
  return gemm_w4a16(a, b, layout, scales, zeros, group, 0.f, m, n, k, c_out, stream);
}

int wq_pack_ptq1_0(const int8_t* trits, const uint16_t* d, int64_t n, int64_t k, uint8_t* blocks,
                   void* stream) {
  if (n < 0 || k < 0) return WQ_EINVAL;
  if (n == 0 || k == 0) return WQ_OK;
  if (!trits || !d || !blocks) return WQ_EINVAL;
  if (k % 128 != 0) return WQ_ESHAPE;
  if (!aligned(trits, 16) || !aligned(d, 2) || !aligned(blocks, 4)) return WQ_EALIGN;
  if (mul_sat(n, k / 128) / 256 + 1 > kMaxGrid) return WQ_ESHAPE;
  return hip_status(wq::launch_pack_ptq1_0(trits, d, n, k, blocks, as_stream(stream)));
}


int wq_quantize_q8_1(const float* x, int64_t c, int64_t k, uint8_t* x_q8, void* stream) {
  return quantize_q8_1(x, c, k, x_q8, false, stream);
}

int wq_quantize_q8_1_pt(const float* x, int64_t c, int64_t k, uint8_t* x_pt, void* stream) {
  return quantize_q8_1(x, c, k, x_pt, true, stream);
}


int wq_gemv_ternary(const uint8_t* w_blocks, const uint8_t* x_q8, int64_t n, int64_t k, int64_t c,
                    float* out, void* stream) {
  bool launch = false;
  const int v = check_gemv_ternary(w_blocks, x_q8, n, k, c, out, &launch);
  if (v != WQ_OK || !launch) return v;
  return hip_status(wq::launch_gemv_ternary(w_blocks, x_q8, false, n, k, c, out, as_stream(stream)));
}

int wq_gemv_ternary_pt(const uint8_t* w_blocks, const uint8_t* x_pt, int64_t n, int64_t k, int64_t c,
                       float* out, void* stream) {
  bool launch = false;
  const int v = check_gemv_ternary(w_blocks, x_pt, n, k, c, out, &launch);
  if (v != WQ_OK || !launch) return v;
  if (k > (int64_t(1) << 30)) return WQ_ESHAPE;  // a column's plane offsets in 32 bits
  return hip_status(wq::launch_gemv_ternary(w_blocks, x_pt, true, n, k, c, out, as_stream(stream)));
}

int wq_gemv_ternary_noalloc(const uint8_t* w_blocks, const uint8_t* x_q8, int64_t n, int64_t k,
                            int64_t c, float* out, void* stream) {
  bool launch = false;
  const int v = check_gemv_ternary(w_blocks, x_q8, n, k, c, out, &launch);
  if (v != WQ_OK || !launch) return v;
  if (c >= 64 && wq::gemm_ternary_workspace(n, k, c) > wq::kTernScratchBytes) return WQ_ESHAPE;
  return hip_status(wq::launch_gemv_ternary_noalloc(w_blocks, x_q8, n, k, c, out, as_stream(stream)));
}


int wq_gemv_ternary_ptq1_1(const uint8_t* superblocks, const uint8_t* codebook,
                           const int32_t* esc_idx, const uint8_t* esc_patt, int64_t n_esc,
                           const uint8_t* x_q8, int64_t n, int64_t k, int64_t c, float* out,
                           void* stream) {
  return gemv_ternary_ptq1_1(superblocks, codebook, esc_idx, esc_patt, n_esc, x_q8, false, n, k, c, out,
                             stream);
}

int wq_gemv_ternary_ptq1_1_pt(const uint8_t* superblocks, const uint8_t* codebook,
                              const int32_t* esc_idx, const uint8_t* esc_patt, int64_t n_esc,
                              const uint8_t* x_pt, int64_t n, int64_t k, int64_t c, float* out,
                              void* stream) {
  return gemv_ternary_ptq1_1(superblocks, codebook, esc_idx, esc_patt, n_esc, x_pt, true, n, k, c, out,
                             stream);
}

}  // extern "C"
