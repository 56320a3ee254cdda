// workspace.h -- per-(device, stream) scratch buffers, kept between calls.
//
// The large-head-dim path stages its exponentials and statistics in device
// memory, and the few-heads key split stages partial outputs; the pages' host
// code allocates such a workspace per call (FastVideo wan22_vae_decode attn.cu,
// attn_forward).  Here each (device, stream) pair keeps one buffer that later
// calls on that stream reuse, grown when a larger problem arrives.
//
// Invariants:
//   * A call leases its stream's buffer from acquire() until release(), and
//     holds that entry's lock for the whole lease.  So the kernels of two calls
//     on one stream are queued one call after the other (never interleaved over
//     the same buffer), and no call can free or replace a buffer another call
//     has leased but not yet queued its work on.  Calls on different streams
//     use different entries and never wait for each other's locks.
//   * Growth is stream-ordered: the old buffer is freed with a free queued on
//     the stream (after every kernel already queued there that reads it) and the
//     new one allocated on the stream; nothing synchronises the device.
//   * release() records an event on the stream.  The next lease makes its
//     stream wait for that event first: a no-op on the same stream, and the
//     ordering edge that keeps a buffer safe if a destroyed stream's handle is
//     reused by a new stream.
//
// The bookkeeping is written against a small backend (events, stream waits,
// stream-ordered allocation) so that it can be exercised on the host with a
// simulated stream; the library instantiates it with HIP.
#pragma once

#include <cstddef>
#include <map>
#include <mutex>
#include <utility>

namespace attn {

// Backend requirements (all return 0 on success, nonzero on failure):
//   using Stream; using Event;
//   int create_event(Event*);
//   int record(Event, Stream);
//   int stream_wait(Stream, Event);
//   int malloc_async(void**, size_t, Stream);
//   int free_async(void*, Stream);
template <class Backend>
class WorkspaceCache {
 public:
  using Stream = typename Backend::Stream;
  using Event = typename Backend::Event;

  struct Entry {
    std::mutex mu;  // held from acquire() to release()
    void* ptr = nullptr;
    size_t bytes = 0;
    Event done{};
    bool has_event = false;
    bool recorded = false;
  };

  // A leased buffer: `ptr` holds at least the bytes asked for.
  struct Lease {
    Entry* entry = nullptr;
    void* ptr = nullptr;
  };

  explicit WorkspaceCache(Backend& b) : be_(b) {}

  // Lease the buffer of (dev, stream), at least `bytes` long.  On success the
  // caller queues its kernels on `stream` and then calls release(); on failure
  // nothing is held.
  int acquire(int dev, Stream stream, size_t bytes, Lease* out) {
    Entry* e = nullptr;
    {
      std::lock_guard<std::mutex> lk(map_mu_);
      e = &map_[{dev, stream}];  // map nodes never move
    }
    e->mu.lock();
    int err = 0;
    if (!e->has_event) {
      if ((err = be_.create_event(&e->done)) != 0) {
        e->mu.unlock();
        return err;
      }
      e->has_event = true;
    }
    // Order this call after the previous lease of the buffer.
    if (e->recorded && (err = be_.stream_wait(stream, e->done)) != 0) {
      e->mu.unlock();
      return err;
    }
    if (e->bytes < bytes) {
      if (e->ptr) {
        if ((err = be_.free_async(e->ptr, stream)) != 0) {
          e->mu.unlock();
          return err;
        }
        e->ptr = nullptr;
        e->bytes = 0;
      }
      void* p = nullptr;
      if ((err = be_.malloc_async(&p, bytes, stream)) != 0) {
        e->mu.unlock();
        return err;
      }
      e->ptr = p;
      e->bytes = bytes;
    }
    out->entry = e;
    out->ptr = e->ptr;
    return 0;
  }

  // End a lease: record its completion on the stream and unlock the entry.
  int release(Stream stream, Lease* l) {
    Entry* e = l->entry;
    if (!e) return 0;
    const int err = be_.record(e->done, stream);
    e->recorded = err == 0;
    l->entry = nullptr;
    l->ptr = nullptr;
    e->mu.unlock();
    return err;
  }

 private:
  Backend& be_;
  std::mutex map_mu_;
  std::map<std::pair<int, Stream>, Entry> map_;
};

}  // namespace attn
