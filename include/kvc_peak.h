/*
 * kvc_peak.h -- C ABI of libkvc_peak.so: on-chip peak probes that the
 * benchmark times to report measured peaks beside the published ones.
 * Measurement support only; the compression path (kvc.h) does not use it.
 *
 * Every probe is one kernel launch enqueued on `stream` (a hipStream_t passed
 * as void*, NULL = null stream) on the current device; it returns without
 * synchronising.  The caller times the launch with events on the same stream
 * and divides the work the matching helper reports by the duration.  Return
 * value: 0 on success, 1 for a bad argument (nothing launched), 4 if the
 * launch failed.  `sink` receives one word per thread (sized by the matching
 * *_sink_words helper) so that no work is optimised away; its contents carry
 * no meaning.
 */
#ifndef KVC_PEAK_H
#define KVC_PEAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compute units of the current device (0 if the query fails). */
int kvc_peak_cus(void);

/* Read stream: every byte of buf (device, 16-byte aligned, bytes % 16 == 0)
 * is read once with 16-byte loads, consecutive lanes on consecutive chunks.
 * Work = bytes read. */
size_t kvc_peak_read_sink_words(void);
int kvc_peak_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Dense bf16 MFMA: v_mfma_f32_32x32x16_bf16 back to back, four independent
 * accumulators per wave, two 8-wave workgroups per compute unit.
 * Work = kvc_peak_mfma_flops(iters) flops. */
size_t kvc_peak_mfma_sink_words(void);
double kvc_peak_mfma_flops(int iters);
int kvc_peak_mfma(float* sink, int iters, void* stream);

/* Vector ALU issue rate of one instruction class: 16 independent chains per
 * lane, two 16-wave workgroups per compute unit (8 waves per SIMD).
 * Work = kvc_peak_valu_wave_instructions(iters) wave64 instructions. */
enum {
  KVC_PEAK_FMA = 0,      /* v_fma_f32                      */
  KVC_PEAK_ADD = 1,      /* v_add_f32                      */
  KVC_PEAK_EXP2 = 2,     /* v_exp_f32 (transcendental)     */
  KVC_PEAK_LOG2 = 3,     /* v_log_f32 (transcendental)     */
  KVC_PEAK_MAD_U64 = 4,  /* v_mad_u64_u32 + v_bitop3_b32  */
  KVC_PEAK_BITOP3 = 5    /* v_bitop3_b32 (three-input xor) */
};
size_t kvc_peak_valu_sink_words(void);
double kvc_peak_valu_wave_instructions(int iters);
int kvc_peak_valu(int op, float* sink, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PEAK_H */
