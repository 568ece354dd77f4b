// Run-time hand-out of the last items of a launch (host side).  Blocks are
// bound to the eight XCDs round-robin by index, and the XCDs run the same
// work at speeds that differ by several percent, so a launch can leave the
// last part of each XCD's slots unbound: its last blocks claim those items in
// order from a counter, and the XCDs that run faster take more of them.
//
// The forward kernels use it.  The counters are library state, one 4-byte
// device counter per (device, stream), zero when the code object loads, never
// reset: every launch that uses one claims exactly its n_claim tickets,
// launches on one stream run one after the other, and the host keeps each
// counter's running value, passing a launch its base.  A lease holds the lock
// that keeps several host threads on one stream in order from reading the base
// to the enqueue.  The runtime gives a destroyed stream's handle to the next
// stream it creates, which then continues that counter; that is sound because
// hipStreamDestroy returns only once the stream's pending work has run
// (measured on this runtime: 25-28 ms for ~25 ms of queued forwards), so no
// launch of the old stream is still claiming.  (The stream id, which is never
// reused, is not exported by the runtime PyTorch ships.)
#pragma once
#include <hip/hip_runtime.h>

#include <mutex>

namespace vlgqa {

struct TicketLease {
  std::unique_lock<std::mutex> lock;
  unsigned* counter = nullptr;  // device address of the stream's counter, or null: static order
  unsigned* next = nullptr;     // host copy of the counter's value after the launches enqueued
  unsigned base() const { return *next; }
  // after each enqueued launch that claims: its n_claim tickets are taken
  void advance(unsigned n_claim) { *next += n_claim; }
};

// The lease of stream's counter, with no counter (static order) for a stream
// being captured into a graph (which may be replayed on another stream), the
// per-thread default stream (one handle, many streams), or more than 64
// streams on a device.
TicketLease ticket_lease(hipStream_t stream);

// Per-XCD slots that a launch of `slots` per XCD leaves to run-time claims
// (0: none), and its number of claiming blocks (the claims plus ~10% spares).
constexpr int kTailDivisor = 5;  // a fifth of every XCD's slots
inline long long tail_slots(long long slots) {
  const long long tail = slots / kTailDivisor;
  return tail >= 2 && slots * 8 < 0x3FFFFFFF ? tail : 0;
}
inline long long claim_blocks(long long tail) { return 8 * (tail + tail / 10 + 1); }

}  // namespace vlgqa
