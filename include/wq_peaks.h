/*
 * wq_peaks.h -- calibration kernels of libwq: what this device actually
 * sustains for a plain streaming read, a bf16 matrix-core loop and an fp32
 * FMA loop, so that each kernel's time can be set against the practical
 * ceiling of its bound as well as against the published peak.
 *
 * They compute nothing of the method; each writes one word per lane into
 * `sink` only so that the compiler keeps the work.  The conventions of wq.h
 * hold: device pointers, `stream` as void*, WQ_OK or a negative wq_status,
 * arguments checked before anything is enqueued, nothing synchronised.
 */
#ifndef WQ_PEAKS_H
#define WQ_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of nbytes at buf (16-byte aligned, nbytes a positive
 * multiple of 16, below 2^40): one 1024-lane workgroup per compute unit
 * reads its own contiguous share, 16 bytes per lane and load, four loads in
 * flight per lane -- the access shape of the decode GEMV without its
 * arithmetic.  sink: sink_words >= wq_peak_read_sink_words() uint32 words,
 * 4-byte aligned; each wave stores the XOR of the words its lanes read into
 * its own word (16 per workgroup, workgroups = min(CUs, 4096, nbytes / 16)),
 * the rest of sink is left as it was.  Bytes moved per call: nbytes read,
 * 64 per workgroup written.
 */
int64_t wq_peak_read_sink_words(void);
int wq_peak_read(const void* buf, int64_t nbytes, uint32_t* sink, int64_t sink_words,
                 void* stream);

/*
 * bf16 matrix-core loop: `workgroups` 256-lane workgroups (1 .. 2^20), each
 * wave issuing iters (1 .. 2^20) rounds of 8 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (seeded, fixed bf16 bits in
 * [0, 2)).  Flops per call: workgroups * 4 * iters * 8 * 2 * 32 * 32 * 16.
 * sink: workgroups * 256 floats (sink_words at least that), 4-byte aligned.
 */
int wq_peak_mfma_bf16(int workgroups, int iters, float* sink, int64_t sink_words, void* stream);

/*
 * fp32 FMA loop: `workgroups` 256-lane workgroups (1 .. 2^20), each lane
 * running 8 independent chains of iters (1 .. 2^20) v_fma_f32.  Flops per
 * call: workgroups * 256 * iters * 8 * 2.  sink as for wq_peak_mfma_bf16.
 */
int wq_peak_valu_fma(int workgroups, int iters, float* sink, int64_t sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_PEAKS_H */
