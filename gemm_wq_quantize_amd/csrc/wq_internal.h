// Internal helpers and launcher declarations of libwq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace wq {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));

// float32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// float32 -> fp16 bit pattern, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---- Global -> LDS loads that bypass registers (buffer_load ... lds).

// Buffer descriptor in SGPRs: raw (stride 0), num_records bytes; offsets at
// or past num_records read as zero.
__device__ __forceinline__ intx4 make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  intx4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc + voff into LDS at lds_base + 16 * lane
// (lds_base wave-uniform).  Issued from asm so that the compiler does not
// wait for these loads before every LDS read; completion is awaited with
// explicit vmcnt waits (wait_vmcnt).  The compiler's hazard checks do not look
// inside asm, so the asm keeps its own: one wait state between the M0 write
// and the LDS-DMA load that reads M0.  (No other code in the kernels that use
// these loads uses M0, so clobbering it is safe.)
__device__ __forceinline__ void dma16(intx4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// 4 bytes per lane from rsrc + voff into LDS at lds_base + 4 * lane
__device__ __forceinline__ void dma4(intx4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Host-side per-device caches.  Each entry is an atomic, so concurrent first
// calls from several host threads are well defined (at worst both query the
// runtime and store the same value).
constexpr int kMaxDevices = 64;

// Compute-unit count of the current device (256 if the runtime cannot say).
inline int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];  // static storage: zero-initialised
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Lets kernel `fn` use up to `bytes` of dynamic LDS on the current device,
// once per device: `done` is the caller's per-kernel bit set of devices.
inline hipError_t allow_dynamic_lds(const void* fn, std::atomic<uint64_t>& done, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  const uint64_t bit = uint64_t(1) << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Launchers: validated arguments only.  Each returns hipSuccess or the
// launch error.
hipError_t launch_pack_int4(const uint8_t* codes, int64_t n, int64_t k, int layout,
                            uint8_t* packed, hipStream_t s);
hipError_t launch_quantize_pack_int4(const uint16_t* w, int64_t n, int64_t k, int64_t group,
                                     int layout, uint8_t* packed, void* scales, bool scale_bf16,
                                     hipStream_t s);

struct GemvArgs {
  const uint8_t* packed;
  const void* scales;
  const void* zeros;
  const void* x;
  void* out;
  int64_t n, k, group, c;
  float zero_const;
  int layout;
  bool scale_bf16, x_bf16, out_bf16;
};
hipError_t launch_gemv_w4(const GemvArgs& a, hipStream_t s);

hipError_t launch_gemm_w4a16(const uint16_t* a, const uint8_t* b, const uint16_t* scales,
                             const uint16_t* zeros, int64_t group, float zero_const, int64_t m,
                             int64_t n, int64_t k, uint16_t* c, hipStream_t s);

hipError_t launch_pack_ptq1_0(const int8_t* trits, const uint16_t* d, int64_t n, int64_t k,
                              uint8_t* blocks, hipStream_t s);
// pt: activations in the PT plane layout instead of block_q8_1 records
hipError_t launch_quantize_q8_1(const float* x, int64_t c, int64_t k, uint8_t* xq, bool pt,
                                hipStream_t s);
hipError_t launch_gemv_ternary(const uint8_t* w, const uint8_t* xq, bool pt, int64_t n, int64_t k,
                               int64_t c, float* out, hipStream_t s);
// The c >= 64 product with a caller-provided workspace of
// gemm_ternary_workspace(n, k, c) bytes (256-byte aligned).
size_t gemm_ternary_workspace(int64_t n, int64_t k, int64_t c);
hipError_t launch_gemm_ternary(const uint8_t* w, const uint8_t* xq, bool pt, int64_t n, int64_t k,
                               int64_t c, float* out, void* ws, hipStream_t s);
// launch_gemv_ternary with the c >= 64 workspace in the library's static
// scratch (nothing allocated); hipErrorInvalidValue when the workspace
// exceeds it.
constexpr size_t kTernScratchBytes = size_t(64) << 20;
hipError_t launch_gemv_ternary_noalloc(const uint8_t* w, const uint8_t* xq, int64_t n, int64_t k,
                                       int64_t c, float* out, hipStream_t s);
hipError_t launch_gemv_ternary_sb(const uint8_t* w, const uint8_t* codebook, const int32_t* esc_idx,
                                  const uint8_t* esc_patt, int64_t n_esc, const uint8_t* xq, bool pt,
                                  int64_t n, int64_t k, int64_t c, float* out, hipStream_t s);

}  // namespace wq
