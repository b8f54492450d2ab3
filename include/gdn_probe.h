/*
 * gdn_probe.h -- measurement helper of libgdn (not a step of the layer).
 *
 * gdn_hbm_probe streams a device buffer in place: every 16-byte vector is loaded with the
 * nontemporal hint and stored back, bit for bit (XORed with `salt`, which the caller
 * passes as 0; the kernel cannot tell, so it really stores). It is the decode kernel's
 * state pass -- each wave reading and rewriting 4 KiB contiguous, four waves to a
 * workgroup -- without the arithmetic, so its rate over a buffer much larger than the
 * GPU's caches is the practical HBM ceiling that the decode kernel's rate is stated
 * against. Conventions as include/gdn.h: device pointer, asynchronous on `stream`.
 *
 *  buf    device buffer, 16-byte aligned; bytes a multiple of 16 KiB (one workgroup's
 *         share). Its contents are unchanged when salt is 0.
 *  Errors: GDN_ERR_NULL (buf), GDN_ERR_ALIGN (buf or bytes), GDN_ERR_HIP.
 */
#ifndef GDN_PROBE_H_
#define GDN_PROBE_H_

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

gdn_status gdn_hbm_probe(void* buf, size_t bytes, uint32_t salt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PROBE_H_ */
