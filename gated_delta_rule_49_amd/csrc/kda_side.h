// kda_side.h -- a second stream per device, for work that shares the chip with a launch on the
// caller's stream and does not depend on it (nor it on that work).
//
//   kda_side_fork(s)   records an event on the caller's stream s, makes the side stream wait for
//                      it and returns the side stream with the side lock held; or returns null
//                      (lock not held) when there is no side stream, and the caller then launches
//                      on s itself.
//   kda_side_forked()  after the caller's launches on the side stream: records the join event
//                      and releases the lock (also when a launch failed).
//   kda_side_join(s)   makes s wait for the join event (only after a fork that returned a stream).
//
// The side stream (default priority) and its two events are created on first use per device and
// kept until the process ends.  The lock orders the record / wait pairs of concurrent callers: a
// join event recorded again by a later caller was recorded after this caller's launches on the
// side stream, so waiting for it also covers them.  Under stream capture the fork and the join
// become edges of the captured graph.
#pragma once
#include <hip/hip_runtime.h>

extern "C" __attribute__((visibility("hidden"))) hipStream_t kda_side_fork(hipStream_t s);
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_side_forked(void);
extern "C" __attribute__((visibility("hidden"))) hipError_t kda_side_join(hipStream_t s);
