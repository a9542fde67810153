/*
 * ditnorm_measure -- a measurement utility exported by libditnorm.so beside
 * the entry points of ditnorm.h.  It is not part of the method: the
 * benchmark times it as the practical HBM ceiling of a launch (a plain copy
 * of the same bytes) and uses it to calibrate the FETCH_SIZE / WRITE_SIZE
 * counters.  Conventions (device pointers, streams, status codes) are those
 * of ditnorm.h.
 */
#ifndef DITNORM_MEASURE_H
#define DITNORM_MEASURE_H

#include "ditnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ditnorm_copy -- a plain 16-byte-vector device-to-device copy of `bytes`
 * bytes, one vector per work-item, streaming loads and stores written
 * through the L2 (the fastest copy form measured on MI355X).  `bytes` is a
 * multiple of 16 and at most (DITNORM_MAX_VECTORS - 255) * 16; both pointers
 * are 16-byte aligned and the ranges do not overlap.  Returns DITNORM_OK,
 * DITNORM_INVALID_ARGUMENT (a NULL pointer, a negative size),
 * DITNORM_UNSUPPORTED (a size or alignment outside the above, overlapping
 * ranges) or DITNORM_DEVICE_ERROR (the launch failed).
 */
int ditnorm_copy(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DITNORM_MEASURE_H */
