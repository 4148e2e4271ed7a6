/*
 * gdn_calib.h -- streaming reference kernels of libgdn_hip.so, for measurement.
 *
 * The fused decode step moves each state row once from HBM and once back
 * ("Module gdn" page, "The fusion": one read and one write of the memory per
 * token), so its speed is bounded by how fast this GPU streams an in-place
 * read-modify-write.  These calls measure that bound on the machine at hand
 * with the same access pattern and no arithmetic beyond one multiply-add per
 * element, so a benchmark can report the decode's rate against it beside the
 * published HBM peak.  They are not part of the recurrence.
 *
 *   op GDN_CALIB_RMW:  buf[i] = buf[i] * 1.0000001f + 1e-7f   (in place, src == dst)
 *   op GDN_CALIB_COPY: dst[i] = src[i]
 *
 * `variant` picks the access shape (GDN_CALIB_VARIANTS of them): a workgroup
 * of 256, 512 or 1024 threads owns a contiguous chunk of 16-byte vectors,
 * each lane issues all of its 4, 8 or 16 loads before any store, with
 * nontemporal or ordinary loads and stores, or (the last three) buffer loads
 * and stores with the decode's cache policies: nontemporal loads, stores
 * nontemporal and written through to device scope; gdn_calib_variant_name()
 * names it.  bytes must be a multiple of 16 and below 2^37 (one launch of at
 * most 2^31 threads), and src/dst 16-byte aligned device
 * pointers owned by the caller; for GDN_CALIB_COPY they must not overlap.
 * Asynchronous on `stream`; allocates nothing; returns a gdn_status
 * (include/gdn.h) with the reason in gdn_last_error().
 */
#ifndef GDN_CALIB_H
#define GDN_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_CALIB_RMW 0
#define GDN_CALIB_COPY 1
#define GDN_CALIB_VARIANTS 15

int gdn_calib_stream(int32_t op, int32_t variant, const void* src, void* dst, uint64_t bytes,
                     void* stream);

/* Static description of a variant ("" when out of range). */
const char* gdn_calib_variant_name(int32_t variant);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CALIB_H */
