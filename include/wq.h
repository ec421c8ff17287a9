/*
 * wq.h -- C ABI of libwq: weight-quantised GEMV / GEMM for AMD Instinct
 * MI355X (gfx950).
 *
 * Pages cited (titles; section names in brackets):
 *   Paddle PR    "[PHI] add int4 weight only quant kernel, add int4 weight
 *                only permute kernel" (PaddlePaddle/Paddle #64091)
 *   Vulkan post  "怎样在安卓端利用 Vulkan 编写 4-bit 专用算子：直接在 GPU 上
 *                进行解量化与计算融合"
 *   Helion issue "int4 gemm kernel" (pytorch/helion #508)
 *   Ternary post "三值量化模型的无损压缩"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a caller-owned DEVICE pointer (HIP global
 *    memory) unless stated otherwise.  The library keeps no pointer after
 *    the call returns and never frees or allocates caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    All work is enqueued asynchronously on it; no call synchronises.
 *  - Return value: WQ_OK (0) or a negative wq_status.  Argument errors are
 *    detected BEFORE anything is enqueued; then nothing runs and the output
 *    buffers are untouched.  A launch failure returns WQ_EHIP.  Faults
 *    during execution surface at the caller's next synchronisation.
 *  - Empty problems (a zero n, c or m) return WQ_OK and enqueue nothing.
 *  - Matrices are row-major and densely packed (no strides).
 *  - Calls that write the same output concurrently on different streams
 *    race; calls on one stream are ordered.
 *
 * int4 formats (Vulkan post [1 packing strategy]; Paddle PR ["int4量化
 * kernel", "int4 permute kernel"]; Helion issue [matmul_bf16_int4])
 * ----------------------------------------------------------------------
 *  A weight matrix W has N output rows and K inputs; code q[n][k] in 0..15
 *  stands for (q - zero) * scale.  Packed storage is [N][K/2] bytes, row n
 *  contiguous along K.  Within row n, the little-endian 32-bit word m holds
 *  the eight codes k = 8m .. 8m+7:
 *    WQ_LAYOUT_PLAIN   nibble p (bits 4p..4p+3) holds k = 8m + p, i.e. byte
 *                      i = q[2i] | q[2i+1] << 4 (low nibble = even k).
 *    WQ_LAYOUT_GFX950  nibble p holds k = 8m + {0,2,4,6,1,3,5,7}[p], so that
 *                      (word >> 4j) & 0x000F000F yields codes (2j, 2j+1) in
 *                      the two 16-bit halves -- one OR makes two bf16.
 *  Scales (and optional zeros) are [N][K/group] in the scale dtype; group is
 *  a power of two >= 32 that divides K, or K itself (one scale per row).
 *
 * Ternary formats (Ternary post [2 weight compression], [3.1 data format],
 * [3.2 dequantisation])
 * ------------------------------------------------------------------------
 *  PTQ1_0 block, 28 bytes per 128 trits: qs[24] (120 trits, five per byte),
 *  qh[2] (8 trits, two bits each), fp16 d.  A trit t is stored as the digit
 *  u = t + 1; a qs byte is sum_j u_j 3^j (digit 0 least significant).
 *  Element e < 80: byte e & 15, digit e >> 4.  Element 80 + e (e < 40):
 *  byte 16 + (e & 7), digit e >> 3.  Element 120 + e (e < 8): qh[e & 1],
 *  bits 2*(e >> 1) .. +1.  Weights are [N][K/128] blocks, row-major.
 *  block_q8_1, 36 bytes per 32 activations: fp16 d, fp16 s = d * sum(q),
 *  int8 q[32].  Activations are [c][K/32] blocks.
 *  PT layout of the activations ([3.1 data format]; the *_pt entry points):
 *  the same bytes per column (9K/8), regrouped by 128-element block i
 *  (K/128 of them) into nine planes of K/128 slots of 16 bytes.  Element e
 *  (0..127) of block i is byte 16 * ((e / 16) * K/128 + i) + e % 16 (plane
 *  e / 16); slot i of plane 8 holds the (d, s) words of the block's four
 *  q8_1 sub-blocks in order (the post draws plane 8 only as "all (d, s)").
 *  A batch is c consecutive PT arrays.  Requires K % 128 == 0.
 */
#ifndef WQ_H
#define WQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_EINVAL = -1,       /* null pointer, bad enum, negative size            */
  WQ_EALIGN = -2,       /* a pointer is not aligned as the call requires    */
  WQ_ESHAPE = -3,       /* sizes violate the call's divisibility/limits     */
  WQ_EUNSUPPORTED = -4, /* valid request the library does not implement     */
  WQ_EHIP = -5          /* the HIP runtime reported an error at launch      */
} wq_status;

typedef enum { WQ_F32 = 0, WQ_F16 = 1, WQ_BF16 = 2 } wq_dtype;
typedef enum { WQ_LAYOUT_PLAIN = 0, WQ_LAYOUT_GFX950 = 1 } wq_layout;

/* Version of this ABI (bumped on any incompatible change). */
int wq_abi_version(void);

/* Human-readable name of a wq_status value (static storage, never NULL). */
const char* wq_status_string(int status);

/*
 * wq_pack_int4 -- pack unsigned 4-bit codes into a packed layout.
 *   codes  [n][k] uint8, one code (0..15) per byte; values >= 16 are
 *          truncated to their low nibble.
 *   packed [n][k/2] uint8 out, in `layout`.
 * Requires k % 8 == 0, both pointers 4-byte aligned.
 * Defines: Vulkan post [1 packing strategy]; Paddle PR ["int4 permute
 * kernel"] for the gfx950 within-word order.
 */
int wq_pack_int4(const uint8_t* codes, int64_t n, int64_t k, int layout,
                 uint8_t* packed, void* stream);

/*
 * wq_quantize_pack_int4 -- fp16 weights to int4 codes + scales, packed.
 *   w      [n][k] fp16 (IEEE binary16 bit patterns).
 *   group  128-style power of two >= 32 dividing k, or k (per row).
 *   packed [n][k/2] uint8 out in `layout`.
 *   scales [n][k/group] out, scale_dtype WQ_F32 or WQ_BF16.
 * The zero point is 8.  Per row and group: scale = absmax / 7 (float32
 * IEEE divide) rounded to the scale dtype (RNE); code = clamp(rint(w /
 * scale), -8, 7) + 8 with a float32 IEEE divide by the STORED scale; an
 * all-zero group stores scale 0 and codes 8.  (The pages give only the
 * packing -- Paddle PR ["int4量化kernel"]; the formula is this library's
 * reading.)  NaN/Inf weights are outside the contract.
 * Requires k % 32 == 0; w and packed 16-byte aligned, scales 4-byte aligned.
 */
int wq_quantize_pack_int4(const uint16_t* w, int64_t n, int64_t k, int64_t group,
                          int layout, uint8_t* packed, void* scales, int scale_dtype,
                          void* stream);

/*
 * wq_gemv_w4 -- out[j][r] = sum_k (q[r][k] - z[r][g]) * s[r][g] * x[j][k],
 * g = k / group, for j < c (Ternary post [3 MMVQ], the batched form with x
 * indexed [c][k]; dequantisation as in the Vulkan post [2 GLSL shader]).
 *   packed  [n][k/2] uint8 in `layout`.
 *   scales  [n][k/group], scale_dtype WQ_F32 or WQ_BF16.
 *   zeros   NULL (then every zero point is zero_const) or [n][k/group] in
 *           the scale dtype.
 *   x       [c][k], x_dtype WQ_F32 or WQ_BF16.
 *   out     [c][n], out_dtype WQ_F32 or WQ_BF16 (RNE).
 * Accumulates in float32; the result does not depend on the stream or on
 * timing (bitwise repeatable).  Requires 1 <= c <= 32 (0 is a no-op),
 * k % 32 == 0, k <= 2^24 (32-bit buffer offsets), packed and x 16-byte
 * aligned, scales/zeros/out 4-byte aligned (out 2-byte for bf16);
 * otherwise WQ_ESHAPE / WQ_EALIGN before anything is launched.
 */
int wq_gemv_w4(const uint8_t* packed, int layout, const void* scales, int scale_dtype,
               const void* zeros, float zero_const, int64_t n, int64_t k, int64_t group,
               const void* x, int x_dtype, int64_t c, void* out, int out_dtype,
               void* stream);

/*
 * wq_gemm_w4a16 -- C[i][j] = sum_k A[i][k] * (q[j][k] - zero_const) * s[j][k / group]
 * (Helion issue [matmul_bf16_int4]; B is stored output-major [n][k/2], the
 * transpose of the issue's (K/2, N) int8 view; the group scales are the
 * weight-only quantiser's output, as in the Vulkan shader's per-group
 * scale).
 *   a       [m][k] bf16.
 *   b       [n][k/2] uint8 in `layout` (WQ_LAYOUT_GFX950 only).
 *   scales  bf16: [n] when group == k (one scale per column, applied to the
 *           float32 sum), else [n][k/group] with group a power of two,
 *           64 <= group < k (each weight becomes bf16((q - z) * s), RNE,
 *           before the bf16 multiply; group 32 is WQ_EUNSUPPORTED).
 *   c_out   [m][n] bf16 (RNE of the float32 accumulator).
 * Requires k % 64 == 0 and k <= 2^22; a, b and c_out 16-byte aligned, scales
 * 2-byte aligned (4-byte with group scales; the kernel reads whole aligned
 * 4-byte words of the scale array, so the 2 bytes after its last element
 * may be read and are ignored).  Any m and n (ragged tiles are masked).
 * With one scale per column the zero point folds out exactly through the
 * row sums of A.  With group scales each weight is bf16_rne of the exact
 * (q - z) * s whenever z * s is exact in float32 (z an integer, or any value
 * with at most 16 significant bits, e.g. a bf16 value); for other zero_const
 * values (7.3f, 0.1f) the weight is bf16_rne(q * s - fl32(z * s)), whose one
 * extra float32 rounding can move a weight by one bf16 ulp.
 */
int wq_gemm_w4a16(const uint16_t* a, const uint8_t* b, int layout, const uint16_t* scales,
                  int64_t group, float zero_const, int64_t m, int64_t n, int64_t k,
                  uint16_t* c_out, void* stream);

/*
 * wq_gemm_w4a16_zp -- C[i][j] = sum_k A[i][k] * (q[j][k] - z[j][k / group]) * s[j][k / group]:
 * wq_gemm_w4a16 with stored zero points instead of zero_const (the Vulkan
 * post's dequantisation (q - zero) * scale with a zero per group; the same
 * weights wq_gemv_w4 accepts with its zeros argument, for the prefill
 * product).
 *   zeros   bf16, the shape of scales ([n] when group == k, else
 *           [n][k/group]); required (null is WQ_EINVAL), same alignment as
 *           scales (4-byte with group scales, whose last word may be read
 *           past the array as for scales).
 * Everything else as wq_gemm_w4a16.  With one scale per column the zero
 * folds out through A's row sums; with group scales each weight is rounded
 * once, bf16_rne((q - z) * s), exact in float32 before the rounding for bf16 s
 * and z.
 */
int wq_gemm_w4a16_zp(const uint16_t* a, const uint8_t* b, int layout, const uint16_t* scales,
                     const uint16_t* zeros, int64_t group, int64_t m, int64_t n, int64_t k,
                     uint16_t* c_out, void* stream);

/*
 * wq_pack_ptq1_0 -- trits and block scales to PTQ1_0 blocks.
 *   trits   [n][k] int8 in {-1, 0, 1} (other values: outside the contract).
 *   d       [n][k/128] fp16 bit patterns.
 *   blocks  [n][k/128][28] uint8 out.
 * Requires k % 128 == 0, trits 16-byte aligned, blocks 4-byte aligned.
 */
int wq_pack_ptq1_0(const int8_t* trits, const uint16_t* d, int64_t n, int64_t k,
                   uint8_t* blocks, void* stream);

/*
 * wq_quantize_q8_1 -- float32 activations to block_q8_1 (Ternary post [3.1]).
 *   x      [c][k] float32.
 *   x_q8   [c][k/32][36] uint8 out.
 * Per 32 values: d = fp16(amax / 127) (float32 divide, RNE);
 * q = clamp(rint(x / float(d)), -127, 127) (float32 divide); s =
 * fp16(float(d) * sum(q)); amax == 0 gives d = s = 0, q = 0.
 * Requires k % 32 == 0, x 16-byte aligned, x_q8 4-byte aligned.
 */
int wq_quantize_q8_1(const float* x, int64_t c, int64_t k, uint8_t* x_q8, void* stream);

/*
 * wq_quantize_q8_1_pt -- wq_quantize_q8_1 writing the PT plane layout
 * (Ternary post [3.1]): the same blocks, bytes moved as the format section
 * above states.  x_pt [c][9k/8] uint8 out.  Requires k % 128 == 0,
 * k <= 2^30, x 16-byte aligned, x_pt 4-byte aligned.
 */
int wq_quantize_q8_1_pt(const float* x, int64_t c, int64_t k, uint8_t* x_pt, void* stream);

/*
 * wq_gemv_ternary -- out[j][r] = sum_b d_w[r][b/4] * d_x[j][b] * S[r][j][b]
 * with the exact integer sums S = sum_{i<32} t * q over each activation
 * block b (Ternary post [3 MMVQ], [3.1], [3.2]).  The stored s of the
 * activation blocks is not used: the integer sum of q replaces it.
 *   w_blocks  [n][k/128] PTQ1_0 blocks.
 *   x_q8      [c][k/32] block_q8_1.
 *   out       [c][n] float32.
 * Requires c >= 0 (0 is a no-op), k % 128 == 0, w_blocks and x_q8 4-byte
 * aligned, out 4-byte aligned (16-byte for c >= 64).  Up to 16 columns run
 * on the vector units; 17 <= c <= 63 runs as passes of at most 16 columns.
 * c >= 64 (a prefill batch) runs on the fp4 x fp8 matrix cores: trits are
 * exact in fp4 and each q is the exact fp8 pair (q & 15, 16 (q >> 4)), so one
 * v_mfma_scale_f32_32x32x64_f8f6f4 product per 32-k activation block gives S
 * exactly.  That path first unpacks both operands into a workspace of about
 * n k + 2 c k bytes, allocated and freed in stream order from a memory pool
 * the library keeps per device (what a call frees stays in the pool); an
 * allocation failure is WQ_EHIP.  It also requires n * k / 128 * 28 and
 * c * k / 32 * 36 below 2^31.
 */
int wq_gemv_ternary(const uint8_t* w_blocks, const uint8_t* x_q8, int64_t n, int64_t k,
                    int64_t c, float* out, void* stream);

/*
 * wq_gemv_ternary_pt -- wq_gemv_ternary with the activations in the PT
 * plane layout (Ternary post [3.1]: the layout the post's mmvq operator
 * reads x in).  x_pt [c][9k/8] uint8, as wq_quantize_q8_1_pt writes it; the
 * kernels, limits and errors are wq_gemv_ternary's (k <= 2^30 in addition),
 * and the results are bit-identical to wq_gemv_ternary on the same blocks in
 * record order.
 */
int wq_gemv_ternary_pt(const uint8_t* w_blocks, const uint8_t* x_pt, int64_t n, int64_t k,
                       int64_t c, float* out, void* stream);

/*
 * wq_gemv_ternary_noalloc -- wq_gemv_ternary for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results
 * bit-identical to wq_gemv_ternary's.  It calls no allocator: the c >= 64
 * product's workspace (the unpacked operands, about n k + 2 c k bytes)
 * lives in a static device array of the library, WQ_TERNARY_SCRATCH_BYTES
 * (64 MiB) on every device the library runs on, held until the process
 * ends; a larger workspace is WQ_ESHAPE, before anything is launched.  Below
 * 64 columns no workspace is used.  Every call on a device shares that
 * device's array (it keeps the last call's contents, all of which the next
 * call rewrites before reading), so calls that overlap on one device --
 * on different streams, or from several host threads -- race.
 */
#define WQ_TERNARY_SCRATCH_BYTES (64ll << 20)
int wq_gemv_ternary_noalloc(const uint8_t* w_blocks, const uint8_t* x_q8, int64_t n, int64_t k,
                            int64_t c, float* out, void* stream);

/*
 * PTQ1_1 superblocks (Ternary post [2 weight compression], struct ptq1_1;
 * [3.1 data format], sb = kbx >> 3, sub = kbx & 7): eight consecutive
 * PTQ1_0 blocks of a row in 216 bytes, 1/28 fewer than 8 x 28.  The post
 * fixes the sizes and the scheme, not the bit positions; this library's
 * layout:
 *   bytes   0..191  the qs[24] of sub-blocks 0..7, unchanged
 *   bytes 192..204  qh[13]: tail trit t = 8 sub + e (element 120 + e of
 *                   sub-block sub, stored as u = trit + 1) is base-3 digit
 *                   t % 5 of qh[t / 5] (digit 0 least significant); digit 4
 *                   of qh[12] is the free trit
 *   bytes 205..214  eight 10-bit mantissas of d, an 80-bit little-endian
 *                   field, mantissa sub at bit 10 sub
 *   byte  215       exponent byte
 *  Pattern index P = exponent byte + 256 * free digit (768 values).  P < 767
 *  selects row P of a 767 x 8 codebook of fp16 exponent fields; P = 767
 *  means the superblock's exponents are in the escape table (its index
 *  row * k/1024 + sb, in ascending order, and 8 exponent fields).  The sign
 *  of d is not stored (always +): d = (exponent << 10) | mantissa.
 */

/*
 * wq_ptq1_1_encode -- PTQ1_0 blocks to PTQ1_1 superblocks (HOST pointers;
 * compression is an offline weight-preparation step and runs on the CPU).
 *   blocks       host [n][k/128][28] PTQ1_0 blocks; every d must be >= +0.
 *   superblocks  host [n][k/1024][216] out.
 *   codebook     host [767][8] out: the tensor's most frequent exponent
 *                patterns by decreasing count (ties by increasing pattern,
 *                exponents compared in sub-block order); unused rows zero.
 *   esc_idx      host int32 [esc_cap] out, ascending superblock indices.
 *   esc_patt     host [esc_cap][8] out, their exponent fields.
 *   n_esc        out: the number of escaped superblocks (also when it
 *                exceeds esc_cap, which returns WQ_ESHAPE).
 * Requires k % 1024 == 0 and n * k / 1024 < 2^31; a negative d is
 * WQ_EINVAL.
 */
int wq_ptq1_1_encode(const uint8_t* blocks, int64_t n, int64_t k, uint8_t* superblocks,
                     uint8_t* codebook, int32_t* esc_idx, uint8_t* esc_patt, int64_t esc_cap,
                     int64_t* n_esc);

/*
 * wq_gemv_ternary_ptq1_1 -- wq_gemv_ternary on PTQ1_1 superblocks: each
 * sub-block decodes to the PTQ1_0 block it was made from (qs, its 8 tail
 * trits, d from the codebook or escape exponent and its mantissa) inside
 * the kernel, then the same exact integer sub-block sums and scaling
 * (Ternary post [3.1]: "the same as the PTQ1_0 format").
 *   superblocks  [n][k/1024][216] (device).
 *   codebook     [767][8] (device), esc_idx int32 [n_esc], esc_patt
 *                [n_esc][8] (device), as wq_ptq1_1_encode writes them.
 *   x_q8         [c][k/32] block_q8_1; out [c][n] float32.
 * Requires k % 1024 == 0 and k <= 65536 (x of a column and the tables are
 * staged in LDS), n_esc <= 2048 (else WQ_EUNSUPPORTED), all pointers 4-byte
 * aligned (out 16-byte for c >= 64).  Up to 63 columns run as passes of at
 * most 8; c >= 64 unpacks the superblocks into the fp4 trit pairs of the
 * PTQ1_0 path and runs its matrix-core product (same workspace, pool and
 * limits as wq_gemv_ternary with c >= 64).
 */
int wq_gemv_ternary_ptq1_1(const uint8_t* superblocks, const uint8_t* codebook,
                           const int32_t* esc_idx, const uint8_t* esc_patt, int64_t n_esc,
                           const uint8_t* x_q8, int64_t n, int64_t k, int64_t c, float* out,
                           void* stream);

/*
 * wq_gemv_ternary_ptq1_1_pt -- wq_gemv_ternary_ptq1_1 with the activations
 * in the PT plane layout (Ternary post [3.1]); x_pt [c][9k/8] uint8.  Same
 * kernels, limits and errors; results bit-identical to
 * wq_gemv_ternary_ptq1_1 on the same blocks in record order.
 */
int wq_gemv_ternary_ptq1_1_pt(const uint8_t* superblocks, const uint8_t* codebook,
                              const int32_t* esc_idx, const uint8_t* esc_patt, int64_t n_esc,
                              const uint8_t* x_pt, int64_t n, int64_t k, int64_t c, float* out,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
