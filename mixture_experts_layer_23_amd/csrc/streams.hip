// streams.hip -- side streams and fork / join events for launch sequences
// whose independent parts may overlap on the GPU (host code only).
//
// Each device gets two non-blocking side streams at the default priority and
// a ring of timing-free events, created on first use and kept until the
// process ends.  fork(from, to) makes `to` wait for everything issued to
// `from` so far; join is the same call in the other direction.  A caller's
// stream therefore sees the side work as part of its own order, also under
// stream capture (the events become graph edges).
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kMaxDevices = 64;
constexpr int kEvents = 64;
struct DeviceStreams {
  std::once_flag once;
  hipError_t status = hipSuccess;
  hipStream_t side[2] = {nullptr, nullptr};
  hipEvent_t ev[kEvents] = {};
  std::mutex mu;
  int next = 0;
};
DeviceStreams g_dev[kMaxDevices];

DeviceStreams* device_streams() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceStreams* d = &g_dev[dev];
  std::call_once(d->once, [d] {
    for (auto& s : d->side)
      if (d->status == hipSuccess) d->status = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    for (auto& e : d->ev)
      if (d->status == hipSuccess) d->status = hipEventCreateWithFlags(&e, hipEventDisableTiming);
  });
  return d->status == hipSuccess ? d : nullptr;
}
}  // namespace

hipStream_t side_stream(int i) {
  DeviceStreams* d = device_streams();
  return d ? d->side[i & 1] : nullptr;
}

int fork_stream(hipStream_t from, hipStream_t to) {
  DeviceStreams* d = device_streams();
  if (!d) {
    set_error("side streams", hipErrorInvalidDevice);
    return MOE_ELAUNCH;
  }
  hipEvent_t e;
  {
    std::lock_guard<std::mutex> g(d->mu);
    e = d->ev[d->next];
    d->next = (d->next + 1) % kEvents;
  }
  hipError_t r = hipEventRecord(e, from);
  if (r == hipSuccess) r = hipStreamWaitEvent(to, e, 0);
  if (r != hipSuccess) {
    set_error("fork / join", r);
    return MOE_ELAUNCH;
  }
  return MOE_OK;
}

}  // namespace moe
