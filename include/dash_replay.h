/*
 * dash_replay.h -- extra entry point of the replay build of the library
 * (libdash_mi355x_replay.so, compiled with -DDASH_REPLAY). The release library does
 * not export it.
 *
 * It supports checking the ordered dQ reduction exactly (DASH paper, arXiv 2601.21824,
 * section 1 and Table 1: a deterministic backward adds the dQ partials of a tile in one
 * fixed order). In this build the dQ contraction of every contribution starts from
 * zero, the running sum is added to the partial with one fp32 addition per element,
 * and every partial is written to a caller-owned dump, so that adding the dumped
 * partials in rank order in fp32 from +0 reproduces the accumulator bit for bit.
 * Arithmetic is otherwise that of the release build.
 */
#ifndef DASH_REPLAY_H
#define DASH_REPLAY_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Later deterministic dash_attn_bwd calls write every fp32 dQ partial into `buf`: a
 * device buffer of `bytes` bytes owned by the caller, which must stay allocated while
 * attached and should start zeroed. Layout (fp32):
 *   [B*H][R/64 steps of 64 rows][2*d/32 dQ blocks of 32x32][n_kv rank slots][1024]
 * with R = N rounded up to the tile (dash_tile_size) and n_kv = R / tile; a block's 1024
 * floats are in the accumulator order of the workspace (element 4i+e of lane l at
 * 256 i + 4 l + e; row 16(i/2) + 2(i%2) + l/32 + 4e, column l%32 of the block). Rank
 * slots past a tile's contributor count stay untouched. The final fp32 sums stay in the
 * workspace accumulator (offset 0 of the workspace, B*H*R*d floats in the same block
 * order), from which the dQ cast writes bf16 dQ. A deterministic call whose dump would not
 * fit in `bytes` returns DASH_ERR_WORKSPACE before launching. `buf` = null detaches.
 * Returns 0. */
int dash_replay_attach(void* buf, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* DASH_REPLAY_H */
