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

/* The shader clock under a vector-ALU load, to set the FP32 peak (quoted at
 * 2.4 GHz) beside the clock the chip sustains.  `waves` waves of 64 lanes
 * (workgroups of four; a multiple of 4 from 4 to 8192, i.e. up to 8 per SIMD
 * over 256 CUs) each run `iters` (1 to 2^24) rounds of eight independent
 * chains of dependent FMAs, reading the shader-cycle counter and the constant
 * 100 MHz real-time counter before and after.  out: caller-owned device
 * buffer of 4 * waves uint64, 8-byte aligned; wave i writes out[4i] = shader
 * cycles, out[4i+1] = real-time ticks, out[4i+2] = the bits of the chains'
 * float sum, out[4i+3] = 0.  The clock is sum(cycles) / sum(ticks) * 100 MHz.
 * Asynchronous on `stream`; allocates nothing; returns a gdn_status with the
 * reason in gdn_last_error(). */
int gdn_calib_clock(int32_t waves, int32_t iters, uint64_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CALIB_H */
