/*
 * kda_probe.h -- bandwidth reference for the fused KDA decode step.
 *
 * The page "PR #50654 完整报告 -- [ROCm][Perf] Kimi-K3 Fused kernel for KDA
 * decode" (section "Implementation breakdown", item 1) names the per-token
 * read and write of each head's [128, 128] fp32 recurrent state (128 KiB of
 * HBM traffic) as the bottleneck of the decode step and the goal as
 * saturating HBM.  This entry point measures what that access pattern alone
 * achieves on the device: every 64 KiB tile is read once and written back
 * in place, with the same workgroup shape and the same 16-byte nontemporal
 * loads and stores as the decode kernel, and no arithmetic besides one
 * multiply per element.  Its time is the ceiling the decode kernel is
 * compared against.
 */
#ifndef KDA_PROBE_H
#define KDA_PROBE_H

#include <stdint.h>

#include "kda_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * tiles: device pointer, 16-byte aligned, n_tiles * 128 * 128 fp32 values.
 * mode 0: each tile is read and written back in place as value * scale
 *         (scale = 1 keeps the values): the decode kernel's traffic;
 * mode 1: read only (values are left as they are): the read ceiling;
 * mode 2: write only, every value set to scale: the write ceiling.
 * waves: workgroup size in waves, one of 4, 8, 16.  Queued on hip_stream;
 * no allocation, no synchronisation.  Returns KDA_ERR_INVALID_ARG for a
 * null pointer, n_tiles < 0 or > INT32_MAX, another wave count or mode, a
 * non-finite scale; KDA_ERR_MISALIGNED, KDA_ERR_DEVICE and KDA_ERR_LAUNCH
 * as kda_decode.  n_tiles = 0 queues nothing.
 */
kda_status kda_state_stream_probe(float* tiles, int64_t n_tiles, int32_t waves,
                                  int32_t mode, float scale, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H */
