/*
 * xattn_debug.h — extra entry point of the debug build of the library
 * (libxattn_debug.so, compiled with -DXATTN_DEBUG=1; libxattn.so does not
 * export it). In that build the kernels check their indexing (score partial
 * stores, selection state, K/V sub-tile rows, LDS ring slots and list entries,
 * decoded work items, DuSA1 indices) and count every failed check per
 * category in device memory instead of trapping; the results are those of the
 * release build.
 */
#ifndef XATTN_DEBUG_H
#define XATTN_DEBUG_H

#include <stdint.h>

#include "xattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copies the failed-check counters of the current device (categories:
 * 0 score partial store, 1 selection state, 2 K/V rows, 3 LDS slot or list
 * entry, 4 work item, 5 DuSA1 index, 6-7 unused) into out[0..7] (host memory,
 * n >= 8) and clears them when reset != 0. Synchronises with the device.
 * Returns XATTN_ERR_ARG for n < 8, XATTN_ERR_HIP if the copy fails. */
xattn_status xattn_debug_violations(uint32_t* out, int32_t n, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_DEBUG_H */
