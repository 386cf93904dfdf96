// Timing events for the benchmark's per-launch measurements.  They are recorded between the
// kernels of a timed ring on its compute stream, so they must cost the stream as little as
// possible: created without the system-scope memory fence that an ordinary event performs
// when it completes (a cache write-back and invalidation on the path between two kernels).
// They are read only after a device-wide synchronisation, which is all the timing needs.
// Not part of the ring-attention C ABI (libringattn); built into libringattn_tools.
#include <hip/hip_runtime.h>

// Creates one timing event in *ev.  Returns 0, -1 for a null pointer, else a hipError_t.
extern "C" int ra_tool_event_create(void** ev) {
  if (!ev) return -1;
  return (int)hipEventCreateWithFlags((hipEvent_t*)ev, hipEventDisableSystemFence);
}

// Milliseconds from event a to event b (both recorded and complete).  Returns 0, -1 for a
// null argument, else a hipError_t.
extern "C" int ra_tool_event_elapsed_ms(void* a, void* b, float* ms) {
  if (!a || !b || !ms) return -1;
  return (int)hipEventElapsedTime(ms, (hipEvent_t)a, (hipEvent_t)b);
}

extern "C" int ra_tool_event_destroy(void* ev) {
  if (!ev) return -1;
  return (int)hipEventDestroy((hipEvent_t)ev);
}
