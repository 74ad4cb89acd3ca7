/*
 * dash_profile.h -- extra entry point of the profiling build of the library
 * (libdash_mi355x_prof.so, compiled with -DDASH_PROFILE). The release library does
 * not export it.
 *
 * It supports measuring the pipeline bubbles of the schedules (DASH paper, arXiv
 * 2601.21824, sections 3.1 and 4.2: the reduction edges and the inter-SM
 * synchronisation latency): the main kernel records, per wave, the cycles (s_memtime)
 * spent in each phase of its steps.
 */
#ifndef DASH_PROFILE_H
#define DASH_PROFILE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Later dash_attn_bwd calls write the main kernel's per-wave phase counters into
 * `buf`: a device buffer owned by the caller of at least CUs * 4 * 20 uint64
 * ([CU slot][wave][20]; unused waves are not written). Per wave, in this order:
 *   0 dV/dK of the second block                 1 step barrier
 *   2 dQ turn bookkeeping (task record, addresses)   3 waiting for the dQ turn
 *   4 waiting for the step's copies              5 (unused)
 *   6 number of steps                            7 whole kernel
 *   8 S/dP of the first block (with dQ MFMAs)    9 stores of the first dQ blocks
 *  10 S/dP of the second block + first softmax  11 other dQ stores, acknowledgement, turn
 *                                                  passed on, next step's copies issued
 *  12 dV/dK of the first block + second softmax 13 accumulator loads issued late
 *  14 number of steps whose dQ turn had not come at the poll
 *  15 reading the polled turn word (within 0)  16 item prologue
 *  17 the item's last reduction                 18 item epilogue (dK, dV stores)
 * `buf` = null detaches. The buffer must stay allocated while attached. Returns 0. */
int dash_profile_attach(void* buf);

#ifdef __cplusplus
}
#endif

#endif /* DASH_PROFILE_H */
