/* Per-workgroup dispatch timeline of the instrumented build.
 *
 * Only libmoe_timeline.so (the same sources compiled with MOE_TIMELINE
 * defined) exports these functions; libmoe.so carries no instrumentation.
 * Apart from the stamps, the instrumented library computes what libmoe.so
 * computes, with the same entry points (include/moe.h). It is for measuring
 * where a kernel's time goes: start-up chains, waits, tails and the spread of
 * workgroups over XCDs and compute units.
 *
 * A stamped kernel keeps, for each workgroup of its most recent dispatch (the
 * first MOE_TL_MAX_BLOCKS workgroups), one row of MOE_TL_WORDS 64-bit words:
 *   [0]  XCD id << 32 | the HW_ID register of wave 0 (bits 8-11 compute unit,
 *        bit 12 shader array, bits 13-15 shader engine, bits 4-5 SIMD)
 *   [1]  the constant 100 MHz clock (s_memrealtime) when wave 0 began
 *   [2 .. 2 + MOE_TL_MARKS)  the clock when wave 0 passed the kernel's named
 *        points, 0 when it did not (the names are listed per kernel below)
 *   [MOE_TL_WORDS - 1]  the clock when the workgroup's last wave finished
 * A row whose word [1] is 0 belongs to no workgroup of the last dispatch since
 * the last moe_timeline_clear. The clock is the same on every XCD, so rows of
 * different kernels and dispatches compare directly (10 ns per tick).
 */
#ifndef MOE_TIMELINE_H
#define MOE_TIMELINE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_TL_MAX_BLOCKS 8192
#define MOE_TL_MARKS 5
#define MOE_TL_WORDS 8

/* Stamped kernels and their marks. */
enum {
  MOE_TL_ROUTER_GEMV = 0,       /* router_gemv1_kernel: (no marks) */
  MOE_TL_ROUTE_SELECT = 1,      /* route_select_kernel: (no marks) */
  MOE_TL_DEC_ROUTE_GATEUP = 2,  /* dec_route_gateup_kernel: router rows: 0 logit published;
                                   workgroup E-1: 1 all logits seen, 2 slots published;
                                   gate/up items: 3 slot known, 4 weight loads issued */
  MOE_TL_DEC_GATEUP = 3,        /* dec_gateup_kernel: 3 slot known, 4 weight loads issued */
  MOE_TL_DEC_DOWN = 4,          /* dec_down_kernel: 0 weight loads issued, 1 h staged, 2 sums done */
  MOE_TL_BAT_PLAN = 5,          /* bat_plan_kernel: (no marks) */
  MOE_TL_BMX_GATEUP = 6,        /* bmx_gateup_kernel: 0 unit record loaded (not reached: no unit),
                                   1 A rows in LDS, 2 MFMAs done */
  MOE_TL_BMX_DOWN = 7,          /* bmx_down_kernel: as bmx_gateup_kernel */
  MOE_TL_BAT_COMBINE = 8,       /* bat_combine_kernel: (no marks) */
  MOE_TL_KERNELS = 9
};

/* moe_timeline_read: copy kernel's rows (stream-ordered after all work
 * submitted before the call; the call synchronises the device).
 *   kernel      MOE_TL_*
 *   host        host memory of max_blocks * MOE_TL_WORDS uint64_t, caller-owned
 *   max_blocks  rows to copy, 1 .. MOE_TL_MAX_BLOCKS
 * Returns MOE_OK, MOE_EINVAL (kernel or max_blocks out of range, host NULL) or
 * MOE_EHIP. */
int moe_timeline_read(int kernel, uint64_t* host, int max_blocks);

/* moe_timeline_clear: zero every kernel's rows (synchronises the device).
 * Returns MOE_OK or MOE_EHIP. */
int moe_timeline_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TIMELINE_H */
