/*
 * mla_timeline.h -- the phase timeline of libmla_nvfp4_timeline.so: the decode library built again with the
 * decode kernel's phase timestamps compiled in (MLA_TIMELINE).  It exports every function of mla_nvfp4.h,
 * with the same behaviour, plus the one below.  The product library (libmla_nvfp4.so) contains none of it.
 *
 * In the instrumented build, wave 0 of every decode workgroup keeps s_memrealtime stamps (a 100 MHz device
 * clock, 10 ns ticks) in scalar registers and writes them once, at its end, to a device array of 4,096
 * workgroups x 16 slots, indexed by the hardware workgroup index.  Slots: 0 start, 1 prologue loads issued,
 * 2 page table staged, 3 row list complete, 4 step 0 visible, 5 last step done, 6 split result tile
 * complete, 7 arrival counter taken, 8 end (0 where the workgroup's path has no such phase); 11 the
 * launch's workgroup count, 12 the XCC the workgroup ran on, 13 1 if it merged the splits or was unsplit,
 * 14 its logical index, 15 its steps.
 * Each launch overwrites the slots of its workgroups; workgroups past the first 4,096 are not recorded.
 */
#ifndef MLA_TIMELINE_H
#define MLA_TIMELINE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copies the slots of workgroups [0, n) (1 <= n <= 4096) of the last decode launch to host[n * 16]
 * (synchronous: waits for the device).  Returns 0, or 1 for a bad argument or a failed copy. */
int mla_debug_timeline(uint64_t* host, int64_t n);

#ifdef __cplusplus
}
#endif

#endif
