// Layer stream: page-locked host shards -> a ring of 2..8 preallocated device layer
// buffers, copied on a side stream while the current layer computes (the Soup deep
// dive, "Core feature: how layer streaming works"; the 4 GB-laptop Soup article,
// "Layer streaming: technical implementation and memory efficiency").
//
// Synchronisation uses HIP events only, never host waits:
//   copy_done[b]  recorded on the copy stream after the copy into buffer b
//   release[b]    recorded on the compute stream once every kernel of the call that
//                 used buffer b has been enqueued (at the next call)
// Call k: record release of call k-1; issue every copy j <= k + nbuf - 1 not yet issued
// (copy j waits for release[j mod nbuf] of call j - nbuf); compute waits copy_done[k mod
// nbuf].  Copies are hipMemcpyAsync from pinned memory, carried by the SDMA engines, so
// they take no compute units.
//
// Reuse mode keeps the ring's prefetch depth but plans buffers per pass from what they
// hold: a call whose shard already sits intact in a buffer (the last forward layers at
// the forward/backward turn, the first layers at the start of the next step) uses it
// with no copy; otherwise its shard is copied into the least recently used buffer, after
// that buffer's last user is released.
//
// Disk tier (the Soup deep dive, "how layer streaming works" and its table of streaming
// settings: frozen shards read from NVMe when host RAM is short, with a read-ahead depth
// of 1..8 layers, each step of depth costing one layer of pinned RAM): a reader thread
// walks the schedule, position g = pass * sched_len + j on across passes, and reads shard
// sched[j] from the file into pinned staging buffer g mod n_stage once the copy out of
// that buffer for position g - n_stage has completed (its event, recorded when that copy
// was issued).  The ring's copy of position g is issued once that read is done.  The only
// waits are host waits on the reader and the reader's waits on copy events; no GPU work
// waits on the host.
//
// Handles.  The library keeps the set of live contexts; every entry point looks its handle
// up there before touching it, so a NULL or destroyed handle gets ESTATE and is never
// dereferenced, and stream_destroy of a handle that is not live does nothing.  A destroyed
// context gives back its events, its reader thread and its tables, but its small struct is
// kept (a tombstone of a few hundred bytes), so a later context never reuses its address
// and a stale handle can never name another context.
#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <unordered_set>
#include <vector>

#include "abi_internal.hpp"
#include "lnf4.h"

using namespace lnf4;

struct DiskTier {
  int fd = -1;
  bool drop_cache = false;          // drop each shard's pages from the page cache after its read
  std::vector<int64_t> off;         // file offset of each shard
  std::vector<void*> stage;         // n_stage pinned staging buffers (caller-owned)
  size_t stage_bytes = 0;
  std::vector<hipEvent_t> stage_ev; // recorded after the copy out of each staging buffer
  std::thread reader;
  std::mutex mu;
  std::condition_variable cv;
  long base = 0;                    // first position of the reader's current run
  long read_done = 0;               // positions whose read has finished (or failed)
  long issued = 0;                  // positions whose copy has been enqueued
  bool stop = false;
  int err = 0;                      // first error: errno of a failed read, -1 a HIP wait
  long err_pos = -1;
  double read_seconds = 0.0;        // time spent in pread
  int64_t bytes_read = 0;
};

struct lnf4_stream {
  std::vector<const void*> host;
  std::vector<size_t> bytes;
  std::vector<void*> bufs;
  size_t buf_bytes = 0;
  int nbuf = 0;
  std::vector<int32_t> sched;
  bool resident = false;
  hipStream_t copy = nullptr;
  void* slot = nullptr;
  size_t slot_bytes = 0;
  std::vector<hipEvent_t> copy_done, release;
  std::vector<char> release_recorded;
  hipEvent_t slot_release = nullptr, slot_done = nullptr;
  bool slot_loaded = false;
  int slot_part_next = 0;    // next part of a load issued in parts (0: none under way)
  int slot_part_n = 0;
  int slot_part_shard = -1;
  int next_call = 0;
  int issued = 0;
  int pass = 0;
  bool resident_copied = false;
  std::vector<char> resident_ready;  // resident mode: buffer b's one copy was seen complete
  int slot_loads = 0;
  int64_t bytes_copied = 0;
  std::vector<lnf4_stream_event> log;
  // reuse mode: the plan of the current pass, what the buffers hold and when each was
  // last used (a call counter that runs on across passes; -1: never)
  bool reuse = false;
  std::vector<int> plan_buf, plan_src, plan_wait, plan_issue;  // per schedule position
  std::vector<int> holder;
  std::vector<long> last_tick;
  long tick = 0;
  DiskTier* disk = nullptr;  // ring mode only: layer shards come from a file
};

// The set of live contexts (never destroyed itself, so it outlives every caller).
static std::mutex& live_mu() {
  static std::mutex* m = new std::mutex();
  return *m;
}
static std::unordered_set<const lnf4_stream*>& live_set() {
  static auto* s = new std::unordered_set<const lnf4_stream*>();
  return *s;
}
static bool is_live(const lnf4_stream* st) {
  if (!st) return false;
  std::lock_guard<std::mutex> lk(live_mu());
  return live_set().count(st) != 0;
}

// Plan one pass in reuse mode from what the buffers hold now.  Position j: if a buffer
// holds shard sched[j], use it (plan_src[j] = the position of this pass whose copy
// filled it, -1 if an earlier pass did).  Otherwise copy into the least recently used
// buffer (lowest index on ties), after the release of its last user (plan_wait[j]: that
// position of this pass, -1 if the user was in an earlier pass), issued at call
// plan_issue[j] = max(j - nbuf + 1, plan_wait[j] + 1, 0); plan_issue is -1 where there is
// no copy.
static void plan_pass(lnf4_stream* st) {
  const int n = (int)st->sched.size(), nb = st->nbuf;
  st->plan_buf.assign(n, 0);
  st->plan_src.assign(n, -1);
  st->plan_wait.assign(n, -1);
  st->plan_issue.assign(n, -1);
  std::vector<int> holder = st->holder, filled(nb, -1), last(nb, -1);
  std::vector<long> age = st->last_tick;
  for (int j = 0; j < n; ++j) {
    const int s = st->sched[j];
    int b = -1;
    for (int q = 0; q < nb; ++q)
      if (holder[q] == s) b = q;
    if (b < 0) {
      b = 0;
      for (int q = 1; q < nb; ++q)
        if (age[q] < age[b]) b = q;
      int issue = j - nb + 1;
      if (last[b] + 1 > issue) issue = last[b] + 1;
      st->plan_wait[j] = last[b];
      st->plan_issue[j] = issue < 0 ? 0 : issue;
      holder[b] = s;
      filled[b] = j;
    }
    st->plan_src[j] = filled[b];
    st->plan_buf[j] = b;
    last[b] = j;
    age[b] = st->tick + j;
  }
}

static void log_ev(lnf4_stream* st, int kind, int call, int j, int layer, int buffer, int wait) {
  lnf4_stream_event e;
  e.kind = kind;
  e.call = call;
  e.j = j;
  e.layer = layer;
  e.buffer = buffer;
  e.wait = wait;
  st->log.push_back(e);
}

static void destroy_events(lnf4_stream* st) {
  for (hipEvent_t e : st->copy_done)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : st->release)
    if (e) (void)hipEventDestroy(e);
  if (st->slot_release) (void)hipEventDestroy(st->slot_release);
  if (st->slot_done) (void)hipEventDestroy(st->slot_done);
  st->copy_done.clear();
  st->release.clear();
  st->slot_release = st->slot_done = nullptr;
}

// Reader thread of the disk tier (see the header comment).
static void disk_reader(lnf4_stream* st) {
  DiskTier* d = st->disk;
  const long n = (long)st->sched.size();
  const long ns = (long)d->stage.size();
  long g0;
  {
    std::lock_guard<std::mutex> lk(d->mu);
    g0 = d->base;
  }
  for (long g = g0;; ++g) {
    const int s = (int)(g % ns);
    {
      std::unique_lock<std::mutex> lk(d->mu);
      d->cv.wait(lk, [&] { return d->stop || d->issued > g - ns; });
      if (d->stop) return;
    }
    int err = 0;
    // the copy out of this staging buffer for position g - ns was issued (above); wait
    // until it has read the buffer (a run starts with every staging copy complete)
    if (g - g0 >= ns && hipEventSynchronize(d->stage_ev[s]) != hipSuccess) err = -1;
    const int shard = st->sched[g % n];
    const size_t want = st->bytes[shard];
    size_t got = 0;
    const auto t0 = std::chrono::steady_clock::now();
    while (!err && got < want) {
      const ssize_t r = pread(d->fd, (char*)d->stage[s] + got, want - got, (off_t)(d->off[shard] + (int64_t)got));
      if (r < 0) {
        if (errno == EINTR) continue;
        err = errno ? errno : EIO;
      } else if (r == 0) {
        err = EIO;  // the file ends inside the shard
      } else {
        got += (size_t)r;
      }
    }
    // (the pages of a file that is being read are clean, so they can be dropped at once)
    if (d->drop_cache) (void)posix_fadvise(d->fd, (off_t)d->off[shard], (off_t)want, POSIX_FADV_DONTNEED);
    const double secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    {
      std::lock_guard<std::mutex> lk(d->mu);
      if (err && !d->err) {
        d->err = err;
        d->err_pos = g;
      }
      d->read_done = g + 1;
      d->read_seconds += secs;
      d->bytes_read += (int64_t)(got < want ? got : want);
    }
    d->cv.notify_all();
  }
}

static void disk_stop_reader(DiskTier* d) {
  if (!d->reader.joinable()) return;
  {
    std::lock_guard<std::mutex> lk(d->mu);
    d->stop = true;
  }
  d->cv.notify_all();
  d->reader.join();
}

// Wait until every copy out of the staging buffers has completed (an event never
// recorded counts as complete).
static hipError_t disk_wait_stage_copies(DiskTier* d) {
  hipError_t first = hipSuccess;
  for (hipEvent_t e : d->stage_ev) {
    if (!e) continue;
    const hipError_t r = hipEventSynchronize(e);
    if (r != hipSuccess && first == hipSuccess) first = r;
  }
  return first;
}

// Stop the reader, wait for the copies out of the staging buffers and release the tier.
static hipError_t disk_close(lnf4_stream* st) {
  DiskTier* d = st->disk;
  if (!d) return hipSuccess;
  disk_stop_reader(d);
  const hipError_t e = disk_wait_stage_copies(d);
  for (hipEvent_t ev : d->stage_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (d->fd >= 0) close(d->fd);
  delete d;
  st->disk = nullptr;
  return e;
}

// A pass reset before every copy of the pass was issued: the reader has read (or is
// reading) positions whose copies will never be issued, so it would wait for them for
// ever.  Stop it, wait for the copies already issued out of the staging buffers, and start
// a new run at the first position of the next pass, with any earlier read error cleared
// (a read that fails again is reported again).
static int disk_restart(lnf4_stream* st, long g0) {
  DiskTier* d = st->disk;
  disk_stop_reader(d);
  const hipError_t e = disk_wait_stage_copies(d);
  if (e != hipSuccess) return hip_fail(e, "stream_reset (disk tier): waiting for the staging copies");
  {
    std::lock_guard<std::mutex> lk(d->mu);
    d->stop = false;
    d->base = g0;
    d->read_done = g0;
    d->issued = g0;
    d->err = 0;
    d->err_pos = -1;
  }
  try {
    d->reader = std::thread(disk_reader, st);
  } catch (...) {
    return fail(LNF4_EINVAL, "stream_reset (disk tier): cannot restart the reader thread");
  }
  return LNF4_OK;
}

// Disk tier: copy schedule position g (whose shard is `shard`) into layer buffer `buf`
// from its staging buffer, once the reader has filled it.
static int disk_copy_into(lnf4_stream* st, int buf, int shard, long g) {
  DiskTier* d = st->disk;
  const int s = (int)(g % (long)d->stage.size());
  {
    std::unique_lock<std::mutex> lk(d->mu);
    // a failed read (at this position or an earlier one) ends the wait: the reader may
    // never reach g after an error
    d->cv.wait(lk, [&] { return d->read_done > g || (d->err != 0 && d->err_pos <= g) || d->stop; });
    if (d->err && d->err_pos <= g) {
      if (d->err < 0) return fail(LNF4_EHIP, "stream (disk tier): the reader's wait for a staging copy failed");
      return fail(LNF4_EINVAL, "stream (disk tier): reading schedule position %ld (shard %d) failed: %s", d->err_pos,
                  (int)st->sched[d->err_pos % (long)st->sched.size()], std::strerror(d->err));
    }
    if (d->read_done <= g) return fail(LNF4_ESTATE, "stream (disk tier): the reader has stopped");
  }
  hipError_t e = hipMemcpyAsync(st->bufs[buf], d->stage[s], st->bytes[shard], hipMemcpyHostToDevice, st->copy);
  if (e != hipSuccess) return hip_fail(e, "stream: hipMemcpyAsync (staging buffer -> layer buffer)");
  if ((e = hipEventRecord(d->stage_ev[s], st->copy)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(stage)");
  if ((e = hipEventRecord(st->copy_done[buf], st->copy)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(copy_done)");
  st->bytes_copied += (int64_t)st->bytes[shard];
  {
    std::lock_guard<std::mutex> lk(d->mu);
    d->issued = g + 1;
  }
  d->cv.notify_all();
  return LNF4_OK;
}

static int copy_into(lnf4_stream* st, int buf, int shard) {
  hipError_t e = hipMemcpyAsync(st->bufs[buf], st->host[shard], st->bytes[shard], hipMemcpyHostToDevice, st->copy);
  if (e != hipSuccess) return hip_fail(e, "stream: hipMemcpyAsync (host shard -> layer buffer)");
  e = hipEventRecord(st->copy_done[buf], st->copy);
  if (e != hipSuccess) return hip_fail(e, "stream: hipEventRecord(copy_done)");
  st->bytes_copied += (int64_t)st->bytes[shard];
  return LNF4_OK;
}

// host_optional (disk tier): host_shards may be NULL or hold NULL entries (shards with no
// host copy); the entries given must still be page-locked.
static int create_impl(const char* who, const void* const* host_shards, bool host_optional, const size_t* shard_bytes,
                       int32_t n_shards, void* const* dev_bufs, size_t buf_bytes, int32_t n_bufs,
                       const int32_t* schedule, int32_t sched_len, int32_t mode, hipStream_t copy_stream,
                       void* slot_buf, size_t slot_bytes, lnf4_stream** out) {
  if (!out) return fail(LNF4_EINVAL, "%s: out is NULL", who);
  *out = nullptr;
  if (mode < 0 || mode > 2) return fail(LNF4_EINVAL, "%s: mode=%d (0 ring, 1 resident, 2 ring with reuse)", who, (int)mode);
  const int32_t resident = mode == 1;
  if ((!host_shards && !host_optional) || !shard_bytes || !dev_bufs || !schedule) return fail(LNF4_EINVAL, "%s: NULL array", who);
  if (n_shards < 1 || n_shards > (1 << 20)) return fail(LNF4_EINVAL, "%s: n_shards=%d out of range", who, (int)n_shards);
  if (resident) {
    if (n_bufs != n_shards) return fail(LNF4_EINVAL, "%s: resident mode needs n_bufs == n_shards (%d != %d)", who, (int)n_bufs, (int)n_shards);
  } else if (n_bufs < 2 || n_bufs > 8) {
    return fail(LNF4_EINVAL, "%s: n_bufs=%d outside 2..8", who, (int)n_bufs);
  }
  if (sched_len < 1 || sched_len > (1 << 24)) return fail(LNF4_EINVAL, "%s: sched_len=%d out of range", who, (int)sched_len);
  if (buf_bytes == 0) return fail(LNF4_ESHAPE, "%s: buf_bytes is 0", who);
  for (int s = 0; s < n_shards; ++s) {
    if (!host_optional && !host_shards[s]) return fail(LNF4_EINVAL, "%s: host shard %d is NULL", who, s);
    if (shard_bytes[s] == 0) return fail(LNF4_ESHAPE, "%s: shard %d is empty", who, s);
  }
  for (int b = 0; b < n_bufs; ++b) {
    if (!dev_bufs[b]) return fail(LNF4_EINVAL, "%s: device buffer %d is NULL", who, b);
    if ((uintptr_t)dev_bufs[b] & 255) return fail(LNF4_EALIGN, "%s: device buffer %d not 256-byte aligned", who, b);
  }
  for (int k = 0; k < sched_len; ++k) {
    if (schedule[k] < 0 || schedule[k] >= n_shards)
      return fail(LNF4_EINVAL, "%s: schedule[%d]=%d outside 0..%d", who, k, (int)schedule[k], (int)n_shards - 1);
    // a shard that goes through the layer buffers must fit one (slot-only shards are
    // checked against the slot when they are loaded)
    if (shard_bytes[schedule[k]] > buf_bytes)
      return fail(LNF4_ESHAPE, "%s: shard %d (%zu bytes) exceeds buf_bytes %zu", who, (int)schedule[k],
                  shard_bytes[schedule[k]], buf_bytes);
  }
  if (resident)
    for (int s = 0; s < n_shards; ++s)
      if (shard_bytes[s] > buf_bytes)
        return fail(LNF4_ESHAPE, "%s: shard %d (%zu bytes) exceeds buf_bytes %zu", who, s, shard_bytes[s], buf_bytes);
  if (slot_buf) {
    if (slot_bytes == 0) return fail(LNF4_ESHAPE, "%s: slot_bytes is 0", who);
    if ((uintptr_t)slot_buf & 255) return fail(LNF4_EALIGN, "%s: slot buffer not 256-byte aligned", who);
  }
  // host memory must be page-locked, so that copies are true asynchronous DMA
  for (int s = 0; s < n_shards; ++s) {
    if (!host_shards || !host_shards[s]) continue;  // (host_optional only, checked above)
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t e = hipPointerGetAttributes(&attr, host_shards[s]);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(LNF4_EINVAL, "%s: host shard %d is not page-locked host memory", who, s);
    }
  }
  lnf4_stream* st = new (std::nothrow) lnf4_stream();
  if (!st) return fail(LNF4_EINVAL, "%s: out of host memory", who);
  if (host_shards)
    st->host.assign(host_shards, host_shards + n_shards);
  else
    st->host.assign(n_shards, nullptr);
  st->bytes.assign(shard_bytes, shard_bytes + n_shards);
  st->bufs.assign(dev_bufs, dev_bufs + n_bufs);
  st->buf_bytes = buf_bytes;
  st->nbuf = n_bufs;
  st->sched.assign(schedule, schedule + sched_len);
  st->resident = resident != 0;
  st->copy = copy_stream;
  st->slot = slot_buf;
  st->slot_bytes = slot_bytes;
  st->copy_done.assign(n_bufs, nullptr);
  st->release.assign(n_bufs, nullptr);
  st->release_recorded.assign(n_bufs, 0);
  st->reuse = mode == 2;
  st->holder.assign(n_bufs, -1);
  st->last_tick.assign(n_bufs, -1);
  if (st->reuse) plan_pass(st);
  for (int b = 0; b < n_bufs; ++b) {
    hipError_t e = hipEventCreateWithFlags(&st->copy_done[b], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->release[b], hipEventDisableTiming);
    if (e != hipSuccess) {
      destroy_events(st);
      delete st;
      return hip_fail(e, "stream_create: hipEventCreate");
    }
  }
  if (slot_buf) {
    hipError_t e = hipEventCreateWithFlags(&st->slot_release, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->slot_done, hipEventDisableTiming);
    if (e != hipSuccess) {
      destroy_events(st);
      delete st;
      return hip_fail(e, "stream_create: hipEventCreate(slot)");
    }
  }
  {
    std::lock_guard<std::mutex> lk(live_mu());
    live_set().insert(st);
  }
  *out = st;
  return LNF4_OK;
}

// The compute stream of each device: created on first use with a compute-unit mask of every
// CU, which gives it a hardware queue of its own (ordinary streams share a few queues in
// turn, and a copy stream on the compute stream's queue would serialise with it).  Never
// destroyed, so a handle once given out stays valid for the process.
static std::mutex g_compute_mu;
static std::vector<hipStream_t> g_compute, g_copy;

extern "C" {

// A stream with a compute-unit mask of every CU of `device`: the runtime gives such a
// stream a hardware queue of its own.  Created once per device and slot, kept for good.
static int dedicated_stream(std::vector<hipStream_t>& tab, int32_t device, hipStream_t* out, const char* who) {
  if (!out) return fail(LNF4_EINVAL, "%s: out is NULL", who);
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_fail(e, "dedicated stream: hipGetDeviceCount");
  if (device < 0 || device >= n) return fail(LNF4_EINVAL, "%s: device %d outside 0..%d", who, (int)device, n - 1);
  std::lock_guard<std::mutex> lk(g_compute_mu);
  if ((int)tab.size() < n) tab.resize(n, nullptr);
  if (!tab[device]) {
    int cus = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device)) != hipSuccess)
      return hip_fail(e, "dedicated stream: hipDeviceGetAttribute(multiprocessor count)");
    if (cus <= 0) return fail(LNF4_EHIP, "%s: device %d reports %d compute units", who, (int)device, cus);
    std::vector<uint32_t> mask((cus + 31) / 32, 0xffffffffu);
    if (cus % 32) mask.back() = (1u << (cus % 32)) - 1u;
    int prev = 0;
    if ((e = hipGetDevice(&prev)) != hipSuccess) return hip_fail(e, "dedicated stream: hipGetDevice");
    if ((e = hipSetDevice(device)) != hipSuccess) return hip_fail(e, "dedicated stream: hipSetDevice");
    hipStream_t st = nullptr;
    e = hipExtStreamCreateWithCUMask(&st, (uint32_t)mask.size(), mask.data());
    const hipError_t e_restore = hipSetDevice(prev);
    if (e != hipSuccess) return hip_fail(e, "dedicated stream: hipExtStreamCreateWithCUMask");
    if (e_restore != hipSuccess) {
      (void)hipStreamDestroy(st);
      return hip_fail(e_restore, "dedicated stream: hipSetDevice(restore)");
    }
    tab[device] = st;
  }
  *out = tab[device];
  return LNF4_OK;
}

int stream_compute_stream(int32_t device, hipStream_t* out) {
  return dedicated_stream(g_compute, device, out, "stream_compute_stream");
}

int stream_copy_stream(int32_t device, hipStream_t* out) {
  return dedicated_stream(g_copy, device, out, "stream_copy_stream");
}

int stream_create(const void* const* host_shards, const size_t* shard_bytes, int32_t n_shards, void* const* dev_bufs,
                  size_t buf_bytes, int32_t n_bufs, const int32_t* schedule, int32_t sched_len, int32_t mode,
                  hipStream_t copy_stream, void* slot_buf, size_t slot_bytes, lnf4_stream** out) {
  return create_impl("stream_create", host_shards, false, shard_bytes, n_shards, dev_bufs, buf_bytes, n_bufs,
                     schedule, sched_len, mode, copy_stream, slot_buf, slot_bytes, out);
}

int stream_create_disk(const char* path, const int64_t* file_offsets, int32_t drop_cache, void* const* stage_bufs,
                       size_t stage_bytes, int32_t n_stage, const void* const* host_shards, const size_t* shard_bytes,
                       int32_t n_shards, void* const* dev_bufs, size_t buf_bytes, int32_t n_bufs,
                       const int32_t* schedule, int32_t sched_len, hipStream_t copy_stream, void* slot_buf,
                       size_t slot_bytes, lnf4_stream** out) {
  const char* who = "stream_create_disk";
  if (!out) return fail(LNF4_EINVAL, "%s: out is NULL", who);
  *out = nullptr;
  if (!path || !file_offsets || !stage_bufs || !shard_bytes || !schedule) return fail(LNF4_EINVAL, "%s: NULL argument", who);
  if (n_stage < 1 || n_stage > 8) return fail(LNF4_EINVAL, "%s: n_stage=%d outside 1..8", who, (int)n_stage);
  if (n_shards < 1 || n_shards > (1 << 20)) return fail(LNF4_EINVAL, "%s: n_shards=%d out of range", who, (int)n_shards);
  if (sched_len < 1 || sched_len > (1 << 24)) return fail(LNF4_EINVAL, "%s: sched_len=%d out of range", who, (int)sched_len);
  for (int i = 0; i < n_stage; ++i)
    if (!stage_bufs[i]) return fail(LNF4_EINVAL, "%s: staging buffer %d is NULL", who, i);
  for (int k = 0; k < sched_len; ++k) {
    const int s = schedule[k];
    if (s < 0 || s >= n_shards) return fail(LNF4_EINVAL, "%s: schedule[%d]=%d outside 0..%d", who, k, s, (int)n_shards - 1);
    if (file_offsets[s] < 0) return fail(LNF4_EINVAL, "%s: file offset of shard %d is negative", who, s);
    if (shard_bytes[s] > stage_bytes) return fail(LNF4_ESHAPE, "%s: shard %d (%zu bytes) exceeds stage_bytes %zu", who, s, shard_bytes[s], stage_bytes);
  }
  const int fd = open(path, O_RDONLY | O_CLOEXEC);
  if (fd < 0) return fail(LNF4_EINVAL, "%s: cannot open %s: %s", who, path, std::strerror(errno));
  struct stat sb;
  if (fstat(fd, &sb) != 0) {
    close(fd);
    return fail(LNF4_EINVAL, "%s: cannot stat %s", who, path);
  }
  for (int k = 0; k < sched_len; ++k) {
    const int s = schedule[k];
    if (file_offsets[s] + (int64_t)shard_bytes[s] > (int64_t)sb.st_size) {
      close(fd);
      return fail(LNF4_ESHAPE, "%s: shard %d ends past the end of %s", who, s, path);
    }
  }
  lnf4_stream* st = nullptr;
  int rc = create_impl(who, host_shards, true, shard_bytes, n_shards, dev_bufs, buf_bytes, n_bufs, schedule, sched_len,
                       LNF4_STREAM_RING, copy_stream, slot_buf, slot_bytes, &st);
  if (rc) {
    close(fd);
    return rc;
  }
  for (int i = 0; i < n_stage; ++i) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t e = hipPointerGetAttributes(&attr, stage_bufs[i]);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      close(fd);
      stream_destroy(st);
      return fail(LNF4_EINVAL, "%s: staging buffer %d is not page-locked host memory", who, i);
    }
  }
  DiskTier* d = new (std::nothrow) DiskTier();
  if (!d) {
    close(fd);
    stream_destroy(st);
    return fail(LNF4_EINVAL, "%s: out of host memory", who);
  }
  d->fd = fd;
  d->drop_cache = drop_cache != 0;
  d->off.assign(file_offsets, file_offsets + n_shards);
  d->stage.assign(stage_bufs, stage_bufs + n_stage);
  d->stage_bytes = stage_bytes;
  d->stage_ev.assign(n_stage, nullptr);
  st->disk = d;
  for (int i = 0; i < n_stage; ++i) {
    hipError_t e = hipEventCreateWithFlags(&d->stage_ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      stream_destroy(st);
      return hip_fail(e, "stream_create_disk: hipEventCreate");
    }
  }
  try {
    d->reader = std::thread(disk_reader, st);
  } catch (...) {
    stream_destroy(st);
    return fail(LNF4_EINVAL, "%s: cannot start the reader thread", who);
  }
  *out = st;
  return LNF4_OK;
}

int stream_disk_stats(const lnf4_stream* st, int64_t* bytes_read, double* read_seconds) {
  if (!is_live(st)) return fail(LNF4_ESTATE, "stream_disk_stats: stream context is NULL or destroyed");
  if (!st->disk) return fail(LNF4_EINVAL, "stream_disk_stats: the context has no disk tier");
  if (!bytes_read || !read_seconds) return fail(LNF4_EINVAL, "stream_disk_stats: NULL output");
  std::lock_guard<std::mutex> lk(st->disk->mu);
  *bytes_read = st->disk->bytes_read;
  *read_seconds = st->disk->read_seconds;
  return LNF4_OK;
}

int stream_layer_step(lnf4_stream* st, int32_t k, hipStream_t compute, void** dev_ptr_out) {
  const char* who = "stream_layer_step";
  if (!is_live(st)) return fail(LNF4_ESTATE, "%s: stream context is NULL or destroyed", who);
  if (!dev_ptr_out) return fail(LNF4_EINVAL, "%s: dev_ptr_out is NULL", who);
  const int n = (int)st->sched.size();
  if (k != st->next_call) return fail(LNF4_ESTATE, "%s: call %d out of order (expected %d)", who, (int)k, st->next_call);
  if (k >= n) return fail(LNF4_ESTATE, "%s: pass finished (%d calls); call stream_reset", who, n);
  hipError_t e;
  int rc;
  if (st->resident) {
    if (!st->resident_copied) {
      for (int s = 0; s < (int)st->host.size(); ++s) {
        if ((rc = copy_into(st, s, s))) return rc;
        log_ev(st, LNF4_EV_COPY, k, s, s, s, -1);
      }
      st->resident_copied = true;
    }
    const int s = st->sched[k];
    // each buffer is written once: after its copy has been seen complete no wait is
    // enqueued (the call then issues no stream work at all, so a caller may capture the
    // resident step's launches in a graph)
    if ((int)st->resident_ready.size() != (int)st->host.size()) st->resident_ready.assign(st->host.size(), 0);
    if (!st->resident_ready[s]) {
      e = hipEventQuery(st->copy_done[s]);
      if (e == hipSuccess) {
        st->resident_ready[s] = 1;
      } else if (e == hipErrorNotReady) {
        (void)hipGetLastError();  // a pending copy is not an error
        if ((e = hipStreamWaitEvent(compute, st->copy_done[s], 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(copy_done)");
      } else {
        return hip_fail(e, "stream: hipEventQuery(copy_done)");
      }
    }
    log_ev(st, LNF4_EV_STEP, k, s, s, s, s);
    st->next_call = k + 1;
    *dev_ptr_out = st->bufs[s];
    return LNF4_OK;
  }
  const int nb = st->nbuf;
  if (st->reuse) {
    if (k > 0) {
      const int b = st->plan_buf[k - 1];
      if ((e = hipEventRecord(st->release[b], compute)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(release)");
      st->release_recorded[b] = 1;
    }
    // copies in schedule order, each once its call has come (positions with no copy pass)
    while (st->issued < n && st->plan_issue[st->issued] <= k) {
      const int j = st->issued;
      if (st->plan_issue[j] >= 0) {
        const int b = st->plan_buf[j], layer = st->sched[j];
        if (st->release_recorded[b])
          if ((e = hipStreamWaitEvent(st->copy, st->release[b], 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(release)");
        if ((rc = copy_into(st, b, layer))) return rc;
        st->holder[b] = layer;
        log_ev(st, LNF4_EV_COPY, k, j, layer, b, st->plan_wait[j]);
      }
      st->issued = j + 1;
    }
    const int b = st->plan_buf[k];
    // the last copy into b is the one that filled it with this shard (none was issued since)
    if ((e = hipStreamWaitEvent(compute, st->copy_done[b], 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(copy_done)");
    log_ev(st, LNF4_EV_STEP, k, st->plan_src[k], st->sched[k], b, st->plan_src[k]);
    st->last_tick[b] = st->tick + k;
    st->next_call = k + 1;
    *dev_ptr_out = st->bufs[b];
    return LNF4_OK;
  }
  if (k > 0) {
    const int b = (k - 1) % nb;
    if ((e = hipEventRecord(st->release[b], compute)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(release)");
    st->release_recorded[b] = 1;
  }
  while (st->issued < n && st->issued <= k + nb - 1) {
    const int j = st->issued, b = j % nb, layer = st->sched[j];
    // copy j reuses buffer b after its previous user: call j - nb of this pass, or the
    // last user of b in the previous pass
    if (st->release_recorded[b])
      if ((e = hipStreamWaitEvent(st->copy, st->release[b], 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(release)");
    if ((rc = st->disk ? disk_copy_into(st, b, layer, (long)st->pass * n + j) : copy_into(st, b, layer))) return rc;
    log_ev(st, LNF4_EV_COPY, k, j, layer, b, j >= nb ? j - nb : -1);
    st->issued = j + 1;
  }
  const int b = k % nb;
  if ((e = hipStreamWaitEvent(compute, st->copy_done[b], 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(copy_done)");
  log_ev(st, LNF4_EV_STEP, k, k, st->sched[k], b, k);
  st->next_call = k + 1;
  *dev_ptr_out = st->bufs[b];
  return LNF4_OK;
}

int stream_slot_load(lnf4_stream* st, int32_t shard, hipStream_t compute) {
  const char* who = "stream_slot_load";
  if (!is_live(st)) return fail(LNF4_ESTATE, "%s: stream context is NULL or destroyed", who);
  if (!st->slot) return fail(LNF4_EINVAL, "%s: the context has no slot buffer", who);
  if (shard < 0 || shard >= (int)st->host.size()) return fail(LNF4_EINVAL, "%s: shard %d out of range", who, (int)shard);
  if (!st->host[shard]) return fail(LNF4_EINVAL, "%s: shard %d has no host copy (the disk tier streams the layer schedule only)", who, (int)shard);
  if (st->bytes[shard] > st->slot_bytes) return fail(LNF4_ESHAPE, "%s: shard %d (%zu bytes) exceeds the slot (%zu)", who, (int)shard, st->bytes[shard], st->slot_bytes);
  if (st->slot_part_next != 0) return fail(LNF4_ESTATE, "%s: a part-wise slot load is under way", who);
  hipError_t e;
  if ((e = hipEventRecord(st->slot_release, compute)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(slot_release)");
  if ((e = hipStreamWaitEvent(st->copy, st->slot_release, 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(slot_release)");
  if ((e = hipMemcpyAsync(st->slot, st->host[shard], st->bytes[shard], hipMemcpyHostToDevice, st->copy)) != hipSuccess)
    return hip_fail(e, "stream: hipMemcpyAsync (slot)");
  if ((e = hipEventRecord(st->slot_done, st->copy)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(slot_done)");
  st->bytes_copied += (int64_t)st->bytes[shard];
  log_ev(st, LNF4_EV_SLOT_COPY, st->next_call, st->slot_loads, shard, -1, st->slot_loads - 1);
  st->slot_loads += 1;
  st->slot_loaded = true;
  return LNF4_OK;
}

int stream_slot_load_part(lnf4_stream* st, int32_t shard, int32_t part, int32_t n_parts, hipStream_t compute) {
  const char* who = "stream_slot_load_part";
  if (!is_live(st)) return fail(LNF4_ESTATE, "%s: stream context is NULL or destroyed", who);
  if (!st->slot) return fail(LNF4_EINVAL, "%s: the context has no slot buffer", who);
  if (shard < 0 || shard >= (int)st->host.size()) return fail(LNF4_EINVAL, "%s: shard %d out of range", who, (int)shard);
  if (!st->host[shard]) return fail(LNF4_EINVAL, "%s: shard %d has no host copy (the disk tier streams the layer schedule only)", who, (int)shard);
  if (n_parts < 1 || n_parts > 1024 || part < 0 || part >= n_parts)
    return fail(LNF4_EINVAL, "%s: part %d of %d out of range (1 <= n_parts <= 1024)", who, (int)part, (int)n_parts);
  if (st->bytes[shard] > st->slot_bytes) return fail(LNF4_ESHAPE, "%s: shard %d (%zu bytes) exceeds the slot (%zu)", who, (int)shard, st->bytes[shard], st->slot_bytes);
  if (part != st->slot_part_next || (part > 0 && (shard != st->slot_part_shard || n_parts != st->slot_part_n)))
    return fail(LNF4_ESTATE, "%s: expected part %d of the load under way, got part %d of %d (shard %d)", who,
                st->slot_part_next, (int)part, (int)n_parts, (int)shard);
  // part p covers bytes [p*chunk, min((p+1)*chunk, size)), chunk rounded up to 4 KiB
  const size_t size = st->bytes[shard];
  const size_t chunk = ((size + (size_t)n_parts - 1) / (size_t)n_parts + 4095) & ~(size_t)4095;
  const size_t b0 = (size_t)part * chunk < size ? (size_t)part * chunk : size;
  const size_t b1 = b0 + chunk < size ? b0 + chunk : size;
  hipError_t e;
  if (part == 0) {
    // the slot's previous user is the compute work enqueued so far
    if ((e = hipEventRecord(st->slot_release, compute)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(slot_release)");
    if ((e = hipStreamWaitEvent(st->copy, st->slot_release, 0)) != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(slot_release)");
    st->slot_loaded = false;  // a wait now would see a half-written slot
  }
  if (b1 > b0) {
    if ((e = hipMemcpyAsync((uint8_t*)st->slot + b0, (const uint8_t*)st->host[shard] + b0, b1 - b0,
                            hipMemcpyHostToDevice, st->copy)) != hipSuccess)
      return hip_fail(e, "stream: hipMemcpyAsync (slot part)");
  }
  st->bytes_copied += (int64_t)(b1 - b0);
  log_ev(st, LNF4_EV_SLOT_COPY, st->next_call, st->slot_loads, shard, -1 - part, part == 0 ? st->slot_loads - 1 : -1);
  if (part + 1 < n_parts) {
    st->slot_part_next = part + 1;
    st->slot_part_n = n_parts;
    st->slot_part_shard = shard;
    return LNF4_OK;
  }
  if ((e = hipEventRecord(st->slot_done, st->copy)) != hipSuccess) return hip_fail(e, "stream: hipEventRecord(slot_done)");
  st->slot_part_next = 0;
  st->slot_part_n = 0;
  st->slot_part_shard = -1;
  st->slot_loads += 1;
  st->slot_loaded = true;
  return LNF4_OK;
}

int stream_slot_wait(lnf4_stream* st, hipStream_t compute, void** slot_ptr_out) {
  const char* who = "stream_slot_wait";
  if (!is_live(st)) return fail(LNF4_ESTATE, "%s: stream context is NULL or destroyed", who);
  if (!st->slot) return fail(LNF4_EINVAL, "%s: the context has no slot buffer", who);
  if (!st->slot_loaded) return fail(LNF4_ESTATE, "%s: no complete slot load issued", who);
  hipError_t e = hipStreamWaitEvent(compute, st->slot_done, 0);
  if (e != hipSuccess) return hip_fail(e, "stream: hipStreamWaitEvent(slot_done)");
  log_ev(st, LNF4_EV_SLOT_WAIT, st->next_call, st->slot_loads - 1, -1, -1, st->slot_loads - 1);
  if (slot_ptr_out) *slot_ptr_out = st->slot;
  return LNF4_OK;
}

int stream_reset(lnf4_stream* st, hipStream_t compute) {
  const char* who = "stream_reset";
  if (!is_live(st)) return fail(LNF4_ESTATE, "%s: stream context is NULL or destroyed", who);
  if (!st->resident && st->next_call > 0) {
    // release the last call's buffer; earlier buffers were released by later calls
    const int b = st->reuse ? st->plan_buf[st->next_call - 1] : (st->next_call - 1) % st->nbuf;
    hipError_t e = hipEventRecord(st->release[b], compute);
    if (e != hipSuccess) return hip_fail(e, "stream: hipEventRecord(release at reset)");
    st->release_recorded[b] = 1;
  }
  if (st->disk && st->issued < (int)st->sched.size()) {
    const int rc = disk_restart(st, (long)(st->pass + 1) * (long)st->sched.size());
    if (rc) return rc;
  }
  if (st->reuse) st->tick += (long)st->sched.size();
  st->next_call = 0;
  st->issued = 0;
  st->pass += 1;
  st->log.clear();
  if (st->reuse) plan_pass(st);  // from what the buffers hold now (copies of an unfinished pass included)
  return LNF4_OK;
}

int stream_log(const lnf4_stream* st, lnf4_stream_event* ev, int32_t cap, int32_t* n) {
  if (!is_live(st)) return fail(LNF4_ESTATE, "stream_log: stream context is NULL or destroyed");
  if (!n) return fail(LNF4_EINVAL, "stream_log: n is NULL");
  if (cap < 0 || (cap > 0 && !ev)) return fail(LNF4_EINVAL, "stream_log: bad buffer");
  const int m = (int)st->log.size() < cap ? (int)st->log.size() : cap;
  for (int i = 0; i < m; ++i) ev[i] = st->log[i];
  *n = m;
  return LNF4_OK;
}

int stream_bytes_copied(const lnf4_stream* st, int64_t* bytes) {
  if (!is_live(st)) return fail(LNF4_ESTATE, "stream_bytes_copied: stream context is NULL or destroyed");
  if (!bytes) return fail(LNF4_EINVAL, "stream_bytes_copied: bytes is NULL");
  *bytes = st->bytes_copied;
  return LNF4_OK;
}

int stream_destroy(lnf4_stream* st) {
  if (!st) return LNF4_OK;
  {
    std::lock_guard<std::mutex> lk(live_mu());
    if (live_set().erase(st) == 0) return LNF4_OK;  // destroyed before (or never a context)
  }
  // every copy this context issued has completed before its buffers go back to the caller
  hipError_t first = disk_close(st);
  for (hipEvent_t e : st->copy_done) {
    const hipError_t r = e ? hipEventSynchronize(e) : hipSuccess;
    if (r != hipSuccess && first == hipSuccess) first = r;
  }
  if (st->slot_done) {
    const hipError_t r = hipEventSynchronize(st->slot_done);
    if (r != hipSuccess && first == hipSuccess) first = r;
  }
  destroy_events(st);
  // the tombstone keeps only the struct itself
  std::vector<const void*>().swap(st->host);
  std::vector<size_t>().swap(st->bytes);
  std::vector<void*>().swap(st->bufs);
  std::vector<int32_t>().swap(st->sched);
  std::vector<char>().swap(st->release_recorded);
  std::vector<lnf4_stream_event>().swap(st->log);
  std::vector<int>().swap(st->plan_buf);
  std::vector<int>().swap(st->plan_src);
  std::vector<int>().swap(st->plan_wait);
  std::vector<int>().swap(st->plan_issue);
  std::vector<int>().swap(st->holder);
  std::vector<long>().swap(st->last_tick);
  if (first != hipSuccess) return hip_fail(first, "stream_destroy: waiting for the copies in flight (the context is released)");
  return LNF4_OK;
}

}  // extern "C"
