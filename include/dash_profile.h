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
 * `buf`: a device buffer owned by the caller of at least CUs * 8 * 20 uint64
 * ([CU slot][wave][20] with 4 waves per slot for the one-wave-per-SIMD kernel and 8
 * for the two-waves-per-SIMD kernel; unused waves are not written). Per wave of the
 * one-wave-per-SIMD kernel, in this order:
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
 * The two-waves-per-SIMD kernel uses the same slots for its roles' phases (A: S, P,
 * dV; B: dP, dS, dK): 8 S (A) or dP + dQ MFMAs + copies (B); 9 softmax and P stores (A)
 * or dQ stores (B); 5 the mid-step handoff of P (A: flag set, B: flag awaited); 3 a late turn wait; 2 turn bookkeeping (A);
 * 10 P read and dS (B); 12 dV + dQ MFMAs (A) or the first dK MFMAs (B); 13 dQ stores
 * (A) or the running sums landing (B); 4 acknowledgement and turn passed on; 0 the
 * rest of the step; 1 the step-end barrier; 6, 7, 14, 16-18 as above.
 * `buf` = null detaches. The buffer must stay allocated while attached. Returns 0. */
int dash_profile_attach(void* buf);

#ifdef __cplusplus
}
#endif

#endif /* DASH_PROFILE_H */
