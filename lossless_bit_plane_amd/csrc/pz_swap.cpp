// Swap engine: the copy path of the PlaneZip paper (§III, Fig. 2; the pinned
// pool of §III-A "Stream format"). A swapped-out tensor is compressed on the
// GPU into a device staging slot, and its stream's exact bytes go to host
// memory by DMA, into equal-sized pieces of a pinned pool, so that streams of
// any size never fragment the host allocator. Swapping in copies the pieces
// back into a staging slot and decompresses them into the caller's tensor.
//
// The stream's length is known only once the compression has run, so a
// worker thread waits for each compression, takes pool chunks for its length
// and issues the D2H copies on the engine's own copy stream; swap-out returns
// as soon as the compression is enqueued. Staging slots are recycled once the
// DMA (or the decompression) that read them has finished. Host code only.
#include "../../include/planezip.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <thread>
#include <unordered_map>
#include <vector>

namespace {

enum class SlotState { kFree, kCompressing, kBusy };
enum class TicketState { kQueued, kCopying, kFailed };

struct Slot {
  uint8_t *buf = nullptr;      // device: the stream, then 8 bytes of its length
  uint64_t *host_len = nullptr;  // pinned mirror of the length
  hipEvent_t ready = nullptr;  // compression and length copy done (swap-out)
  hipEvent_t done = nullptr;   // last reader of the slot done (DMA or decompression)
  SlotState state = SlotState::kFree;
};

struct Ticket {
  size_t raw_bytes = 0;
  int dtype = 0, elem_bits = 0;
  int slot = -1;  // staging slot while queued
  uint64_t comp_bytes = 0;
  std::vector<uint32_t> chunks;  // pool chunks, in stream order
  hipEvent_t on_host = nullptr;  // the D2H copies done
  hipEvent_t read_back = nullptr;  // the last H2D copy of the chunks done
  bool read_pending = false;
  TicketState state = TicketState::kQueued;
  pz_status_t status = PZ_SUCCESS;
};

struct ScopedDevice {
  int prev = -1;
  explicit ScopedDevice(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~ScopedDevice() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct pz_swapper {
  int device = 0;
  size_t chunk_bytes = 0, nchunks = 0, staging_bytes = 0;
  uint8_t *pool = nullptr;         // pinned host pool
  uint64_t *host_lens = nullptr;   // pinned, one per slot
  std::vector<Slot> slots;
  std::vector<uint32_t> free_chunks;
  hipStream_t d2h = nullptr, h2d = nullptr;

  std::mutex mu;
  std::condition_variable cv;  // slot or ticket state changes
  std::unordered_map<uint64_t, Ticket> tickets;
  std::deque<uint64_t> queue;  // tickets waiting for the worker
  uint64_t next_ticket = 1;
  bool stop = false;
  std::thread worker;

  // A free staging slot (lock held); waits for one if needed.
  int acquire_slot(std::unique_lock<std::mutex> &lock) {
    for (;;) {
      for (size_t i = 0; i < slots.size(); ++i) {
        Slot &s = slots[i];
        if (s.state == SlotState::kFree) return (int)i;
        if (s.state == SlotState::kBusy && hipEventQuery(s.done) == hipSuccess) {
          s.state = SlotState::kFree;
          return (int)i;
        }
      }
      // Every slot is compressing (the worker will move one on) or busy with
      // a copy: wait for the oldest busy one, else for the worker.
      int busy = -1;
      for (size_t i = 0; i < slots.size() && busy < 0; ++i)
        if (slots[i].state == SlotState::kBusy) busy = (int)i;
      if (busy >= 0) {
        hipEvent_t ev = slots[busy].done;
        lock.unlock();
        (void)hipEventSynchronize(ev);
        lock.lock();
      } else {
        cv.wait(lock);
      }
    }
  }

  // Runs of consecutive pool chunks, as (first chunk index in the list,
  // count), so that each run is one DMA.
  static std::vector<std::pair<size_t, size_t>> runs(const std::vector<uint32_t> &c) {
    std::vector<std::pair<size_t, size_t>> r;
    for (size_t i = 0; i < c.size();) {
      size_t j = i + 1;
      while (j < c.size() && c[j] == c[j - 1] + 1) ++j;
      r.emplace_back(i, j - i);
      i = j;
    }
    return r;
  }

  void work() {
    (void)hipSetDevice(device);
    std::unique_lock<std::mutex> lock(mu);
    for (;;) {
      cv.wait(lock, [&] { return stop || !queue.empty(); });
      if (queue.empty()) return;  // stop requested and nothing left
      const uint64_t id = queue.front();
      queue.pop_front();
      Ticket &t = tickets[id];
      Slot &s = slots[t.slot];
      hipEvent_t ready = s.ready;
      lock.unlock();
      hipError_t e = hipEventSynchronize(ready);
      lock.lock();
      const uint64_t len = *s.host_len;
      pz_status_t st = e == hipSuccess ? PZ_SUCCESS : PZ_ERROR_HIP;
      const size_t need = (size_t)((len + chunk_bytes - 1) / chunk_bytes);
      if (st == PZ_SUCCESS && need > free_chunks.size()) st = PZ_ERROR_INSUFFICIENT_BUFFER;
      if (st == PZ_SUCCESS) {
        t.comp_bytes = len;
        // In ascending order, so that adjacent chunks form one DMA.
        t.chunks.assign(free_chunks.end() - need, free_chunks.end());
        free_chunks.resize(free_chunks.size() - need);
        std::sort(t.chunks.begin(), t.chunks.end());
        for (const auto &r : runs(t.chunks)) {
          const size_t off = r.first * chunk_bytes;
          const size_t n = std::min<size_t>(r.second * chunk_bytes, len - off);
          if (hipMemcpyAsync(pool + (size_t)t.chunks[r.first] * chunk_bytes, s.buf + off, n,
                             hipMemcpyDeviceToHost, d2h) != hipSuccess)
            st = PZ_ERROR_HIP;
        }
        if (st == PZ_SUCCESS && (hipEventRecord(t.on_host, d2h) != hipSuccess ||
                                 hipEventRecord(s.done, d2h) != hipSuccess))
          st = PZ_ERROR_HIP;
      }
      if (st == PZ_SUCCESS) {
        t.state = TicketState::kCopying;
        s.state = SlotState::kBusy;
      } else {
        // Nothing of this ticket is in flight after a failed copy is
        // drained; its chunks go back.
        if (!t.chunks.empty()) {
          (void)hipStreamSynchronize(d2h);
          free_chunks.insert(free_chunks.end(), t.chunks.begin(), t.chunks.end());
          t.chunks.clear();
        }
        t.state = TicketState::kFailed;
        t.status = st;
        s.state = SlotState::kFree;
      }
      t.slot = -1;
      cv.notify_all();
    }
  }

  // The ticket, once the worker has handled it (lock held); nullptr if unknown.
  Ticket *settled(std::unique_lock<std::mutex> &lock, uint64_t id) {
    auto it = tickets.find(id);
    if (it == tickets.end()) return nullptr;
    Ticket *t = &it->second;  // (element pointers survive rehashing; iterators do not)
    cv.wait(lock, [&] { return t->state != TicketState::kQueued; });
    return t;
  }

  void teardown() {
    {
      std::lock_guard<std::mutex> lock(mu);
      stop = true;
    }
    cv.notify_all();
    if (worker.joinable()) worker.join();
    ScopedDevice dev(device);
    if (d2h) (void)hipStreamSynchronize(d2h);
    if (h2d) (void)hipStreamSynchronize(h2d);
    for (Slot &s : slots) {
      if (s.done) (void)hipEventSynchronize(s.done);
      if (s.buf) (void)hipFree(s.buf);
      if (s.ready) (void)hipEventDestroy(s.ready);
      if (s.done) (void)hipEventDestroy(s.done);
    }
    for (auto &kv : tickets) {
      if (kv.second.on_host) (void)hipEventDestroy(kv.second.on_host);
      if (kv.second.read_back) (void)hipEventDestroy(kv.second.read_back);
    }
    if (d2h) (void)hipStreamDestroy(d2h);
    if (h2d) (void)hipStreamDestroy(h2d);
    if (pool) (void)hipHostFree(pool);
    if (host_lens) (void)hipHostFree(host_lens);
  }
};

extern "C" {

pz_swapper_t *pz_swapper_create(size_t pool_chunk_bytes, size_t pool_chunks, size_t staging_bytes,
                                int staging_slots) {
  if (pool_chunk_bytes == 0 || (pool_chunk_bytes & 15u) || pool_chunks == 0 || pool_chunks > 0xFFFFFFFFull ||
      pool_chunk_bytes > ((size_t)1 << 40) / pool_chunks || staging_bytes == 0 || staging_slots < 1 ||
      staging_slots > 64)
    return nullptr;
  pz_swapper *p = new (std::nothrow) pz_swapper;
  if (!p) return nullptr;
  bool ok = hipGetDevice(&p->device) == hipSuccess;
  p->chunk_bytes = pool_chunk_bytes;
  p->nchunks = pool_chunks;
  p->staging_bytes = (staging_bytes + 15) & ~(size_t)15;
  ok = ok && hipHostMalloc(reinterpret_cast<void **>(&p->pool), pool_chunk_bytes * pool_chunks,
                           hipHostMallocDefault) == hipSuccess;
  ok = ok && hipHostMalloc(reinterpret_cast<void **>(&p->host_lens), sizeof(uint64_t) * staging_slots,
                           hipHostMallocDefault) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&p->d2h, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&p->h2d, hipStreamNonBlocking) == hipSuccess;
  if (ok) {
    try {
      p->slots.resize(staging_slots);
      p->free_chunks.reserve(pool_chunks);
    } catch (...) {
      ok = false;
    }
  }
  for (int i = 0; ok && i < staging_slots; ++i) {
    Slot &s = p->slots[i];
    s.host_len = p->host_lens + i;
    ok = hipMalloc(reinterpret_cast<void **>(&s.buf), p->staging_bytes + 16) == hipSuccess &&
         hipEventCreateWithFlags(&s.ready, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&s.done, hipEventDisableTiming) == hipSuccess;
  }
  if (ok) {
    for (size_t i = 0; i < pool_chunks; ++i) p->free_chunks.push_back((uint32_t)i);
    try {
      p->worker = std::thread([p] { p->work(); });
    } catch (...) {
      ok = false;
    }
  }
  if (!ok) {
    p->teardown();
    delete p;
    return nullptr;
  }
  return p;
}

void pz_swapper_destroy(pz_swapper_t *p) {
  if (!p) return;
  p->teardown();
  delete p;
}

size_t pz_swapper_free_chunks(pz_swapper_t *p) {
  if (!p) return 0;
  std::lock_guard<std::mutex> lock(p->mu);
  return p->free_chunks.size();
}

pz_status_t pz_swap_out(pz_swapper_t *p, const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                        void *stream, uint64_t *ticket) {
  if (!p || !ticket || raw_bytes == 0 || !d_src) return PZ_ERROR_INVALID_VALUE;
  if (PZ_MAX_COMPRESSED_BYTES(raw_bytes) > p->staging_bytes) return PZ_ERROR_INSUFFICIENT_BUFFER;
  ScopedDevice dev(p->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::unique_lock<std::mutex> lock(p->mu);
  hipEvent_t on_host = nullptr;
  if (hipEventCreateWithFlags(&on_host, hipEventDisableTiming) != hipSuccess) return PZ_ERROR_HIP;
  const int k = p->acquire_slot(lock);
  Slot &slot = p->slots[k];
  uint64_t *d_len = reinterpret_cast<uint64_t *>(slot.buf + p->staging_bytes);
  pz_status_t st = pz_compress(d_src, raw_bytes, dtype, elem_bits, slot.buf, p->staging_bytes, d_len, stream);
  if (st == PZ_SUCCESS &&
      (hipMemcpyAsync(slot.host_len, d_len, sizeof(uint64_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
       hipEventRecord(slot.ready, s) != hipSuccess))
    st = PZ_ERROR_HIP;
  if (st != PZ_SUCCESS) {
    (void)hipEventDestroy(on_host);
    return st;  // the slot stays free: nothing was enqueued, or nothing reads it
  }
  slot.state = SlotState::kCompressing;
  const uint64_t id = p->next_ticket++;
  Ticket &t = p->tickets[id];
  t.raw_bytes = raw_bytes;
  t.dtype = dtype;
  t.elem_bits = elem_bits;
  t.slot = k;
  t.on_host = on_host;
  p->queue.push_back(id);
  *ticket = id;
  p->cv.notify_all();
  return PZ_SUCCESS;
}

pz_status_t pz_swap_wait(pz_swapper_t *p, uint64_t ticket, uint64_t *comp_bytes) {
  if (!p) return PZ_ERROR_INVALID_VALUE;
  std::unique_lock<std::mutex> lock(p->mu);
  Ticket *t = p->settled(lock, ticket);
  if (!t) return PZ_ERROR_INVALID_VALUE;
  if (t->state == TicketState::kFailed) return t->status;
  hipEvent_t ev = t->on_host;
  const uint64_t n = t->comp_bytes;
  lock.unlock();
  ScopedDevice dev(p->device);
  if (hipEventSynchronize(ev) != hipSuccess) return PZ_ERROR_HIP;
  if (comp_bytes) *comp_bytes = n;
  return PZ_SUCCESS;
}

pz_status_t pz_swap_in(pz_swapper_t *p, uint64_t ticket, void *d_dst, int32_t *d_status, void *stream) {
  if (!p) return PZ_ERROR_INVALID_VALUE;
  ScopedDevice dev(p->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::unique_lock<std::mutex> lock(p->mu);
  Ticket *t = p->settled(lock, ticket);
  if (!t) return PZ_ERROR_INVALID_VALUE;
  if (t->state == TicketState::kFailed) return t->status;
  if (!d_dst) return PZ_ERROR_INVALID_VALUE;
  if (!t->read_back && hipEventCreateWithFlags(&t->read_back, hipEventDisableTiming) != hipSuccess)
    return PZ_ERROR_HIP;
  const int k = p->acquire_slot(lock);  // (t stays valid: only a release erases it)
  Slot &slot = p->slots[k];
  // The H2D copies wait for the D2H copies of the same chunks.
  pz_status_t st = hipStreamWaitEvent(p->h2d, t->on_host, 0) == hipSuccess ? PZ_SUCCESS : PZ_ERROR_HIP;
  for (const auto &r : pz_swapper::runs(t->chunks)) {
    if (st != PZ_SUCCESS) break;
    const size_t off = r.first * p->chunk_bytes;
    const size_t n = std::min<size_t>(r.second * p->chunk_bytes, t->comp_bytes - off);
    if (hipMemcpyAsync(slot.buf + off, p->pool + (size_t)t->chunks[r.first] * p->chunk_bytes, n,
                       hipMemcpyHostToDevice, p->h2d) != hipSuccess)
      st = PZ_ERROR_HIP;
  }
  if (st == PZ_SUCCESS && (hipEventRecord(t->read_back, p->h2d) != hipSuccess ||
                           hipStreamWaitEvent(s, t->read_back, 0) != hipSuccess))
    st = PZ_ERROR_HIP;
  if (st == PZ_SUCCESS)
    st = pz_decompress(slot.buf, t->comp_bytes, t->dtype, t->elem_bits, d_dst, t->raw_bytes, d_status, stream);
  // Whatever was enqueued reads the slot until this point of `stream`.
  if (hipEventRecord(slot.done, s) != hipSuccess) {
    (void)hipStreamSynchronize(s);
    (void)hipStreamSynchronize(p->h2d);
    slot.state = SlotState::kFree;
    return PZ_ERROR_HIP;
  }
  slot.state = SlotState::kBusy;
  t->read_pending = true;
  return st;
}

pz_status_t pz_swap_release(pz_swapper_t *p, uint64_t ticket) {
  if (!p) return PZ_ERROR_INVALID_VALUE;
  std::unique_lock<std::mutex> lock(p->mu);
  Ticket *t = p->settled(lock, ticket);
  if (!t) return PZ_ERROR_INVALID_VALUE;
  // No copy may still be reading or writing the chunks.
  hipEvent_t on_host = t->state == TicketState::kCopying ? t->on_host : nullptr;
  hipEvent_t read_back = t->read_pending ? t->read_back : nullptr;
  lock.unlock();
  ScopedDevice dev(p->device);
  if (on_host) (void)hipEventSynchronize(on_host);
  if (read_back) (void)hipEventSynchronize(read_back);
  lock.lock();
  auto it = p->tickets.find(ticket);
  if (it == p->tickets.end()) return PZ_ERROR_INVALID_VALUE;  // released meanwhile by another call
  t = &it->second;
  p->free_chunks.insert(p->free_chunks.end(), t->chunks.begin(), t->chunks.end());
  if (t->on_host) (void)hipEventDestroy(t->on_host);
  if (t->read_back) (void)hipEventDestroy(t->read_back);
  p->tickets.erase(ticket);
  return PZ_SUCCESS;
}

pz_status_t pz_swap_read(pz_swapper_t *p, uint64_t ticket, void *h_dst, size_t capacity, uint64_t *comp_bytes) {
  uint64_t n = 0;
  const pz_status_t st = pz_swap_wait(p, ticket, &n);
  if (st != PZ_SUCCESS) return st;
  if (comp_bytes) *comp_bytes = n;
  if (!h_dst || capacity < n) return PZ_ERROR_INSUFFICIENT_BUFFER;
  std::lock_guard<std::mutex> lock(p->mu);
  auto it = p->tickets.find(ticket);
  if (it == p->tickets.end()) return PZ_ERROR_INVALID_VALUE;
  const Ticket &t = it->second;
  for (size_t i = 0; i < t.chunks.size(); ++i) {
    const size_t off = i * p->chunk_bytes;
    const size_t len = std::min<size_t>(p->chunk_bytes, n - off);
    std::copy(p->pool + (size_t)t.chunks[i] * p->chunk_bytes,
              p->pool + (size_t)t.chunks[i] * p->chunk_bytes + len, static_cast<uint8_t *>(h_dst) + off);
  }
  return PZ_SUCCESS;
}

}  // extern "C"
