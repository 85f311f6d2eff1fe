/*
 * wts_roofline.h -- measured roofline denominators of the walk (gfx950).
 *
 * The walk's per-step cost is set by on-chip operand rates (W resident in
 * registers and LDS), by the stream rate for tiles that are not resident, and
 * by the cross-workgroup selection (Weights That Stay, Fig. 4: entry cost
 * against per-step fetches; Fig. 8: selection; Fig. 11: per-step slopes).
 * wts_roofline() measures those rates on the device the walk runs on, with
 * small kernels of the same library, so that roofline fractions are taken
 * against measured rather than published figures.
 *
 * Host-synchronous; allocates and frees about 2.2 GB of device memory; takes
 * well under a second.  Returns WTS_OK, WTS_ERR_INVALID_ARG (NULL out or a
 * bad device), WTS_ERR_NO_MEMORY or WTS_ERR_DEVICE.  A figure that could not
 * be measured on this device (e.g. the XCD-local exchange when the dispatch
 * check fails) is reported as a negative number.
 */
#ifndef WTS_ROOFLINE_H_
#define WTS_ROOFLINE_H_

#include <stdint.h>

#include "wts.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct wts_roofline_result {
  int32_t grid;               /* workgroups used (one per compute unit, <= 256)  */
  int32_t pad;
  double lds_read_GBps;       /* aggregate ds_read_b128 rate, every CU, 8 waves  */
  double mfma_i8_TOPs;        /* v_mfma_i32_16x16x64_i8, register operands, 8
                                 independent chains per wave, 8 waves per CU     */
  double mfma_bf16_TFLOPs;    /* v_mfma_f32_16x16x32_bf16, likewise               */
  double clock_MHz;           /* shader clock during the int8 MFMA run
                                 (s_memtime against the 100 MHz wall clock)    */
  double hbm_read_GBps;       /* streaming read of 2 GiB (8x the memory-side
                                 cache)                                          */
  double mall_read_GBps;      /* streaming read of 128 MiB already in the
                                 256 MB memory-side cache (above the L2s)        */
  double exchange_us[6];      /* one cross-workgroup selection round, one
                                 workgroup per CU, nothing else in the loop:
                                 [0] the two-level all-gather with the first
                                 level inside an XCD, one line per key,
                                 [1] the same at device scope, [2] a flat
                                 all-gather (8 copies, every key polled),
                                 [3] Fig. 8 as drawn: a device-scope atomic
                                 maximum and an arrival counter, [4] and [5]:
                                 [0] and [1] with the keys of one poll packed
                                 into one 128-byte line                          */
  int64_t exchange_bad[6];    /* workgroup-rounds that saw a wrong winner or
                                 whose wait expired (0 expected)                 */
  double hop_xcd_us;          /* one-way signal latency between two workgroups
                                 of one XCD through its L2                       */
  double hop_device_us;       /* the same between two XCDs, device scope         */
  double valu_dep_cycles;     /* shader cycles per dependent v_add_f32 (wave64)  */
  double valu_indep_cycles;   /* the same over four independent chains           */
  double valu_indep_2w_cycles;/* the same per wave, two waves on each SIMD       */
  double valu_indep_4w_cycles;/* the same per wave, four waves on each SIMD      */
  double dot4_2w_cycles;      /* shader cycles per v_dot4_i32_i8 (wave64) per
                                 wave, four independent chains, two waves on
                                 each SIMD (the int8 dot product a VALU
                                 projection would use instead of the MFMA)      */
} wts_roofline_result;

wts_status wts_roofline(int32_t device, wts_roofline_result* out);

#ifdef __cplusplus
}
#endif

#endif /* WTS_ROOFLINE_H_ */
