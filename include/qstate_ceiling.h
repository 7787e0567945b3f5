/*
 * qstate_ceiling.h — bandwidth-ceiling kernels of the qstate library
 * (gfx950), the reference points a decode step's HBM throughput is read
 * against.  Measurement support: no part of the decode method.
 *
 * A decode step streams every byte of the stored state from HBM once and
 * writes it back in place once; the plainest kernels with that access
 * pattern are a streaming copy (read one buffer, write another) and an
 * in-place read-modify-write (read a buffer, write it back changed).  Both
 * move 16-byte vectors per lane, consecutive lanes on consecutive vectors,
 * with the same non-temporal hint the step kernels put on the state, or
 * with ordinary cached accesses.
 *
 * Arguments:
 *   src, dst, buf  device pointers, 16-byte aligned; for the copy, src and
 *                  dst must not overlap.  Caller-owned; nothing is
 *                  allocated or freed.
 *   bytes          a multiple of 16 (0 is a no-op).
 *   nontemporal    1: loads and stores carry the non-temporal hint;
 *                  0: ordinary accesses.
 *   pattern        rmw: every 32-bit word w becomes w ^ pattern.
 *   stream         hipStream_t (NULL: the default stream); asynchronous.
 * Returns QSTATE_OK, QSTATE_E_INVALID (null or misaligned pointer, size not
 * a multiple of 16, nontemporal not 0 or 1) or QSTATE_E_LAUNCH.
 */
#ifndef QSTATE_CEILING_H
#define QSTATE_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qstate_ceiling_copy(const void* src, void* dst, size_t bytes, int nontemporal, void* stream);
int qstate_ceiling_rmw(void* buf, size_t bytes, uint32_t pattern, int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif
