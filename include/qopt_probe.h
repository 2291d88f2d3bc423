/*
 * libqopt measurement aid: bytes-only access patterns for the 8-bit Adam step's
 * traffic.  Not part of the method.
 *
 * Each pattern moves, for every 2048-element block of one flat parameter set, the
 * bytes a step with fp32 parameters and bf16 gradients moves: it reads 8 KB of
 * parameters, 4 KB of gradients and 2 KB of each code stream, and writes the
 * parameters and both code streams back (the block maxima are left out: 16 bytes per
 * block).  What it writes is what it read, so every buffer keeps its contents.  The
 * patterns differ only in how waves walk the blocks and order their accesses, and in
 * when they issue them: the paced patterns issue every wave's reads and writes at the
 * start of each period of the chip's real-time counter.  Timed against the step on
 * the same buffers they map the ceiling of this 57 % read / 43 % write mix on the
 * device (see the ceiling study of bench.py).
 */
#ifndef QOPT_PROBE_H
#define QOPT_PROBE_H

#include <stdint.h>

#include "qopt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of patterns; patterns are numbered 0 .. count - 1. */
int qopt_pattern_probe_count(void);

/*
 * A static description of pattern `pattern` (NULL outside the range): its lookahead
 * (blocks whose loads are in flight per wave), blocks walked consecutively per wave,
 * waves per SIMD, access width of the code streams, order of a block's accesses and,
 * for a paced pattern, the rate its period is sized for.
 */
const char* qopt_pattern_probe_name(int pattern);

/*
 * Moves the bytes described above once over `nblocks` blocks of the flat buffers
 * (device memory, each 16-byte aligned): params 2048 * nblocks fp32, grads 2048 *
 * nblocks bf16, m_codes and v_codes 2048 * nblocks bytes.  Enqueued on `stream`, in
 * launches of equal block counts holding at most 2^18 blocks each (as the step's).
 * Errors: QOPT_EINVAL (pattern out of range, NULL pointer with nblocks > 0, nblocks
 * < 0), QOPT_EALIGN, QOPT_ELAUNCH.  nblocks == 0 is a no-op.
 */
int qopt_pattern_probe(int pattern, void* params, void* grads, uint8_t* m_codes,
                       uint8_t* v_codes, int64_t nblocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QOPT_PROBE_H */
