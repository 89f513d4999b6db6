/*
 * magicpig_testing.h -- a test aid of libmagicpig: forced launch failures,
 * so that a test can see the MP_E_HIP path of every entry point without a
 * real fault.  No part of the decode path; an application needs only
 * magicpig.h.
 */
#ifndef MAGICPIG_TESTING_H
#define MAGICPIG_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* After the next `skip` kernel launches of the library (on any thread), the
 * following `count` launches fail with hipErrorLaunchFailure without
 * launching anything, so the entry point that makes one returns MP_E_HIP with
 * the error's name in mp_last_error().  `skip` picks which launch of a
 * multi-launch call fails (0: its first).  Launches already enqueued are not
 * affected; count <= 0 clears a pending request.  Launches that run before
 * the failing one within the same entry point stay enqueued (MP_E_HIP means
 * "a launch failed", not "nothing ran"). */
void mp_debug_fail_launches(int32_t skip, int32_t count);

#ifdef __cplusplus
}
#endif

#endif /* MAGICPIG_TESTING_H */
