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
 * `buf`: a device buffer owned by the caller of at least CUs * 4 * 8 uint64
 * ([CU slot][wave][8]; unused waves are not written). Per wave, in this order:
 *   0 body (copies issued, S/dP, softmax, dV/dK, dS^T store)   1 step barrier
 *   2 dQ MFMAs and accumulator read-add-write                    3 waiting for the dQ turn
 *   4 passing the turn on                                        5 item prologue/epilogue
 *   6 number of steps                                            7 whole kernel
 * `buf` = null detaches. The buffer must stay allocated while attached. Returns 0. */
int dash_profile_attach(void* buf);

#ifdef __cplusplus
}
#endif

#endif /* DASH_PROFILE_H */
