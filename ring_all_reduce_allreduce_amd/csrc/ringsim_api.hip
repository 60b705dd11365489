// ringsim_api.hip -- host side of libringsim: communicator, validation,
// protocol choice, plan parameters and kernel launch. Exports the C ABI of
// include/ringsim.h.
//
// Call path ("NCCL" book, enqueue chapter: ncclEnqueueCheck -> taskAppend ->
// plan -> launch, collapsed): check the handle and its magic words, check the
// arguments, return early for count == 0, copy locally for one rank, choose
// the algorithm, protocol and workgroups per channel with the cost model
// (ring_model.h), fill one kernel-argument block and enqueue one kernel on
// the caller's stream. Nothing waits for the device.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "ring_model.h"
#include "tree_plan.h"
#include "ring_plan.h"
#include "ringsim_internal.h"

using namespace ringsim;

namespace {

// Sentinels at both ends of the communicator ("NCCL" book, s. 2.1: first and
// last field of ncclComm, checked to catch use after destroy).
constexpr uint64_t kLiveMagic = 0x52494e4753494d31ull;  // "RINGSIM1"
constexpr uint64_t kDeadMagic = 0xdeaddeaddeaddeadull;

enum LogLevel { kLogNone = 0, kLogWarn = 1, kLogInfo = 2 };

int log_level() {
  static const int level = [] {
    const char* e = std::getenv("RINGSIM_DEBUG");
    if (!e) return (int)kLogNone;
    if (!std::strcmp(e, "INFO")) return (int)kLogInfo;
    if (!std::strcmp(e, "WARN")) return (int)kLogWarn;
    return (int)kLogNone;
  }();
  return level;
}

#define RS_LOG(lvl, ...)                                   \
  do {                                                     \
    if (log_level() >= (lvl)) {                            \
      std::fprintf(stderr, "ringsim %s: ", (lvl) == kLogWarn ? "WARN" : "INFO"); \
      std::fprintf(stderr, __VA_ARGS__);                   \
      std::fprintf(stderr, "\n");                          \
    }                                                      \
  } while (0)

// roctx ranges around the API calls ("NCCL" book, ch. 3, s. 3.1 and the
// enqueue chapter: an NVTX mark at every API entry). With RINGSIM_ROCTX=1
// the library loads a roctx library at its first call and pushes a range
// named after the call for its duration; rocprofv3 --marker-trace shows them
// next to the kernels. Off by default, at the cost of one predictable branch
// per call; nothing is linked in.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx x;
    const char* e = std::getenv("RINGSIM_ROCTX");
    if (!e || !*e || !std::strcmp(e, "0")) return x;
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"}) {
      void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (!h) continue;
      x.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
      x.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
      if (x.push && x.pop) {
        RS_LOG(kLogInfo, "roctx ranges on (%s)", lib);
        return x;
      }
      x = Roctx{};
    }
    RS_LOG(kLogWarn, "RINGSIM_ROCTX is set but no roctx library could be loaded");
    return x;
  }();
  return r;
}

// A range for the lifetime of the object (one API call).
class RoctxRange {
 public:
  explicit RoctxRange(const char* name) : on_(roctx().push != nullptr) {
    if (on_) roctx().push(name);
  }
  ~RoctxRange() {
    if (on_) roctx().pop();
  }
  RoctxRange(const RoctxRange&) = delete;
  RoctxRange& operator=(const RoctxRange&) = delete;

 private:
  const bool on_;
};

long env_long(const char* name, long dflt) {
  const char* e = std::getenv(name);
  if (!e || !*e) return dflt;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  return (end && *end == 0) ? v : dflt;
}

// RINGSIM_ALGO: "ring", "tree", "auto" or the enum value.
int env_algo(int dflt) {
  const char* e = std::getenv("RINGSIM_ALGO");
  if (!e || !*e) return dflt;
  if (!std::strcmp(e, "ring")) return RINGSIM_ALGO_RING;
  if (!std::strcmp(e, "tree")) return RINGSIM_ALGO_TREE;
  if (!std::strcmp(e, "auto")) return RINGSIM_ALGO_AUTO;
  return (int)env_long("RINGSIM_ALGO", dflt);
}

}  // namespace

struct ringsim_comm {
  uint64_t start_magic;
  int nranks;
  int nchannels;
  int proto;
  int wpc;
  int pipe_mul;     // counter pipelines per channel: max(wpc, line_wpc_max)
  int line_wpc_max; // most workgroups per channel a line launch may take (power of two)
  int line_wpc_cfg; // configured line workgroups per channel, 0 = per call
  int wpc_cfg;      // bulk workgroups per channel were configured: no per-call choice
  int line_per_cu[3];  // resident line workgroups per CU: multi, one, half kernels
  int nslots;
  int nslots_cfg;   // configured bulk FIFO depth (nslots may be deeper for long stages)
  int device;
  size_t chunk_bytes;
  size_t slot_bytes;
  size_t flag_threshold;
  int timeout_ms;
  int skip_rank;  // testing knob (RINGSIM_DEBUG_SKIP_RANK), -1 = off
  int lds_stage;  // bulk kernel stages each step's own operand in LDS
  uint64_t timeout_ticks;
  int compute_units;
  int blocks_per_cu;
  char* fifo;
  size_t fifo_bytes;
  char* flag_fifo;
  size_t flag_fifo_bytes;
  FifoCtr* ctr;       // line protocols: [rank][channel * pipe_mul + part]
  size_t ctr_bytes;
  FifoCtr* bulk_ctr;  // bulk protocol: [rank][channel * wpc + part]
  size_t bulk_ctr_bytes;
  // Flag span (kFlagSpanGuard): upper bounds of the steps any line or tree
  // FIFO has moved since its FIFOs and counters were last zeroed, the bound
  // that triggers the next zeroing, and how often it happened.
  uint64_t line_span;
  uint64_t tree_span;
  uint64_t span_limit;
  uint64_t line_resets;
  uint64_t tree_resets;
  FifoEcho* echo;     // bulk debug FIFO records (RINGSIM_DEBUG_FIFO), null = off
  size_t echo_bytes;
  uint32_t* dev_abort;
  uint32_t* host_words;      // [0] abort request, [1] kernel error (host view)
  uint32_t* host_words_dev;  // the same words as the device sees them
  uint64_t calls;
  int last_proto;
  int last_wpc;
  int last_group;          // bulk all-reduce: slot steps per stage group of the latest ring call, 0 = whole stages
  int last_tree_channels;  // channels per tree of the latest all-reduce, 0 = ring
  int algo;                // configured all-reduce algorithm
  int last_algo;
  int tree_channels;       // channels per tree in the tree FIFO arrays
  int tree_depth;          // deeper of the two trees (edges from root to leaf)
  int8_t tree_link[2][RINGSIM_MAX_RANKS][3];
  char* tree_fifo;
  size_t tree_fifo_bytes;
  FifoCtr* tree_ctr;
  size_t tree_ctr_bytes;
  ringsim_result_t sticky;
  uint64_t end_magic;
};

namespace {

std::mutex g_live_mu;
std::unordered_set<const ringsim_comm*> g_live;

bool is_live(const ringsim_comm* c) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return g_live.count(c) != 0;
}

ringsim_result_t check_comm(const ringsim_comm* c) {
  if (!c || !is_live(c)) return RINGSIM_INVALID_USAGE;
  if (c->start_magic != kLiveMagic || c->end_magic != kLiveMagic) return RINGSIM_INVALID_USAGE;
  return RINGSIM_SUCCESS;
}

// Folds the device-visible error words into the sticky result.
ringsim_result_t poll_async(ringsim_comm* c) {
  if (c->sticky != RINGSIM_SUCCESS) return c->sticky;
  const uint32_t abort_req = __atomic_load_n(&c->host_words[0], __ATOMIC_ACQUIRE);
  const uint32_t kerr = __atomic_load_n(&c->host_words[1], __ATOMIC_ACQUIRE);
  if (abort_req || kerr == kErrAborted) {
    c->sticky = RINGSIM_ABORTED;
  } else if (kerr == kErrTimeout) {
    c->sticky = RINGSIM_INTERNAL_ERROR;
    RS_LOG(kLogWarn, "a ring kernel gave up waiting for a peer (timeout %d ms)", c->timeout_ms);
  } else if (kerr == kErrFifoEcho) {
    c->sticky = RINGSIM_INTERNAL_ERROR;
    RS_LOG(kLogWarn, "a bulk FIFO slot held another step or size than its consumer expected");
  } else if (kerr == kErrFlagSpan) {
    c->sticky = RINGSIM_INTERNAL_ERROR;
    RS_LOG(kLogWarn, "a line or tree kernel left a counter past the flag span (calls replayed from graphs)");
  }
  return c->sticky;
}

bool valid_dtype(int dtype) { return dtype >= RINGSIM_INT32 && dtype <= RINGSIM_BFLOAT16; }
bool valid_op(int op) { return op >= RINGSIM_SUM && op <= RINGSIM_MIN; }

// Device buffers: non-null, element aligned; `vec` reports 16-byte alignment.
ringsim_result_t check_bufs(const ringsim_comm* c, const void* const* sb, void* const* rb, int esize,
                            bool* vec) {
  if (!sb || !rb) return RINGSIM_INVALID_ARGUMENT;
  bool v = true;
  for (int r = 0; r < c->nranks; ++r) {
    const uintptr_t s = (uintptr_t)sb[r];
    const uintptr_t d = (uintptr_t)rb[r];
    if (!s || !d) return RINGSIM_INVALID_ARGUMENT;
    if ((s % esize) || (d % esize)) return RINGSIM_INVALID_ARGUMENT;
    if ((s & 15u) || (d & 15u)) v = false;
  }
  *vec = v;
  return RINGSIM_SUCCESS;
}

ringsim_result_t check_device(const ringsim_comm* c) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  return dev == c->device ? RINGSIM_SUCCESS : RINGSIM_INVALID_USAGE;
}

void fill_common(const ringsim_comm* c, RingArgs* a, const void* const* sb, void* const* rb) {
  std::memset(a, 0, sizeof(*a));
  for (int r = 0; r < c->nranks; ++r) {
    a->send[r] = static_cast<const char*>(sb[r]);
    a->recv[r] = static_cast<char*>(rb[r]);
  }
  a->nranks = c->nranks;
  a->nchannels = c->nchannels;
  a->ctr = c->ctr;
  a->pipe_stride = c->nchannels * c->pipe_mul;
  a->pipe_mul = c->pipe_mul;
  a->dev_abort = c->dev_abort;
  a->host_abort = c->host_words_dev;
  a->host_err = c->host_words_dev + 1;
  a->timeout_ticks = c->timeout_ticks;
  a->skip_rank = c->skip_rank;
}

int model_proto(int proto) {
  return proto == RINGSIM_PROTO_FLAG ? kModelFlag : proto == RINGSIM_PROTO_WIDE ? kModelWide : kModelBulk;
}

// Fills the protocol-dependent launch geometry; wpc is the workgroup count
// of the launch: for a line launch 1, 2, 4 or 8 (the flag FIFO holds one
// array per count, in increasing order, each [rank][channel][part][slot] with
// kFlagSlots slots of kFlagSlotBytes per part); for a bulk launch at most the
// communicator's count, whose pipelines (counters and FIFOs) keep their
// places: a launch with fewer leaves the others' counters as they are.
void fill_proto(const ringsim_comm* c, RingArgs* a, int proto, int esize, int wpc) {
  a->chunk = (int64_t)c->chunk_bytes / esize;
  if (proto == RINGSIM_PROTO_FLAG || proto == RINGSIM_PROTO_WIDE) {
    const size_t nc = (size_t)c->nranks * c->nchannels;
    size_t off = 0;
    for (int w = 1; w < wpc; w *= 2) off += nc * (size_t)line_level_bytes(w);
    a->wpc = wpc;
    a->fifo = c->flag_fifo + off;
    a->fifo_stride = c->nchannels * wpc;
    a->fifo_mul = wpc;
    a->nslots = kFlagSlots;
    a->slot_bytes = kFlagSlotBytes;
    a->group = kLineGroupSteps;
  } else {
    a->wpc = wpc;
    a->ctr = c->bulk_ctr;
    a->pipe_stride = c->nchannels * c->wpc;
    a->pipe_mul = c->wpc;
    a->fifo = c->fifo;
    a->fifo_stride = c->nchannels * c->wpc;
    a->fifo_mul = c->wpc;
    a->nslots = c->nslots;
    a->slot_bytes = (int)c->slot_bytes;
    a->lds_stage = c->lds_stage;
    a->group = 0;
    a->echo = c->echo;
  }
}

// Longest unit (bytes) any workgroup of a ring launch moves in one stage
// (ring_model.h).
int64_t max_unit_bytes(const RingArgs& a, int mode, int esize) {
  return ring_max_unit_bytes(a.count, a.nranks, a.nchannels, a.chunk, mode == kAllReduce, esize, a.wpc);
}

// Line kernels by lines per step (host mirror of the device LineMode).
enum HostLineMode : int { kHostLinesMulti = 0, kHostLinesOne = 1, kHostLinesHalf = 2 };

struct LinePlan {
  int wpc;
  int mode;  // HostLineMode
};

// The line kernel a launch with `wpc` workgroups per channel needs: the
// longest step is the longest unit part or a whole slot, whichever is
// shorter.
LinePlan line_plan(const RingArgs& a, int mode, int esize, int line_proto, int dtype, int wpc) {
  const int64_t payload = line_proto == kLineWide && dtype != RINGSIM_INT64 ? 12 : 8;
  RingArgs t = a;
  t.wpc = wpc;
  const int64_t unit_lines = div_up(max_unit_bytes(t, mode, esize), payload);
  const int64_t slot_lines = kFlagSlotBytes / 16;
  const int64_t lines = std::min(unit_lines, slot_lines);
  const int m = lines <= kThreads / 2 ? kHostLinesHalf : lines <= kThreads ? kHostLinesOne : kHostLinesMulti;
  return LinePlan{wpc, m};
}

bool line_plan_resident(const ringsim_comm* c, const LinePlan& lp) {
  return (int64_t)c->nranks * c->nchannels * lp.wpc <= (int64_t)c->line_per_cu[lp.mode] * c->compute_units;
}

// Shape of a call of `count` elements, as the planners see it.
RingArgs call_shape(const ringsim_comm* c, size_t count, int esize) {
  RingArgs a;
  std::memset(&a, 0, sizeof(a));
  a.count = (int64_t)count;
  a.nranks = c->nranks;
  a.nchannels = c->nchannels;
  a.chunk = (int64_t)c->chunk_bytes / esize;
  a.wpc = 1;
  return a;
}

// Calls up to this many bytes per rank load the own operand of a bulk step
// beside the FIFO operand instead of staging it in LDS one step ahead: the
// staging's wait costs every hop more than the own operand's load latency
// does while the memory is lightly loaded (0.5-3 us per call faster at 4,
// 8 and 16 ranks from 4 KiB to 512 KiB per rank; from 1-2 MiB up staging
// wins, by 6-22 us at 4-8 MiB).
constexpr int64_t kBulkStageMinBytes = 512 * 1024;

// FIFO depth and step groups of one bulk call. A stage longer than half the
// configured depth (in one workgroup's slot steps) made the communicator
// deepen its FIFOs at init, so that a whole stage fits half of them ("NCCL"
// book, enqueue chapter: ALLREDUCE_CHUNKSTEPS = NCCL_STEPS / 2). A call
// keeps its FIFO footprint at the configured depth wherever it can: one
// whose stages fit half the configured depth uses only that many slots of
// each FIFO, and an all-reduce with longer stages walks each loop in groups
// of half the configured depth (every stage moves one group before the next
// stage runs, as the line protocols do) over those slots. At 16 ranks x 16
// channels with 512 KiB chunks the deepened FIFOs take 256 MiB, more than
// the Infinity Cache holds beside the streaming buffers; in groups of 4
// steps over 8 slots 128 MiB (16 ranks x 128 and 256 MiB per rank: 1807 ->
// 1726 us and 3607 -> 3417 us). Only reduce-scatter and all-gather calls
// with long stages use the deepened FIFOs (the grouped kernel is built for
// the all-reduce), and the debug FIFO records keep the full depth. Groups
// change the order of steps, not the fold order of any element. Returns the
// group length (0 = whole stages) and sets a->nslots.
int bulk_call_depth(const ringsim_comm* c, RingArgs* a, int mode, int esize) {
  const int cfg = std::max(2, std::min(c->nslots_cfg, c->nslots));
  if (a->echo || a->nslots <= cfg) return 0;
  const int64_t steps = div_up(max_unit_bytes(*a, mode, esize), (int64_t)a->slot_bytes);
  if (2 * steps <= cfg) {
    a->nslots = cfg;
    return 0;
  }
  if (mode != kAllReduce) return 0;
  a->nslots = 2 * (cfg / 2);
  return cfg / 2;
}

// Bulk workgroups per channel of one call: a configured count as it is, else
// fewer than the communicator holds when the stages are short
// (bulk_call_wpc, ring_model.h).
int comm_bulk_wpc(const ringsim_comm* c, const RingArgs& shape, int mode, int esize) {
  if (c->wpc_cfg) return c->wpc;
  return bulk_call_wpc(shape.count, shape.nranks, shape.nchannels, shape.chunk, mode == kAllReduce, esize, c->wpc,
                       (int64_t)c->slot_bytes, c->nslots);
}

struct ProtoChoice {
  int proto;
  LinePlan plan;  // line protocols: workgroups per channel and kernel
  double us;      // predicted time
};

// A line protocol's launch: the configured workgroup count (the most that
// the device can hold at once, if fewer), else among 1, 2, 4, 8 (up to the
// comm's maximum) whose kernel can be resident at once, with at most two
// workgroups per compute unit, the count the cost model predicts fastest.
// One workgroup per channel is always resident (comm init checks it).
ProtoChoice pick_line(const ringsim_comm* c, const RingArgs& a, int mode, int dtype, int proto, double bytes) {
  const int esize = dtype_size(dtype);
  const int lp = proto == RINGSIM_PROTO_WIDE ? kLineWide : kLineFlag;
  const RingModel m;
  const int64_t nc = (int64_t)c->nranks * c->nchannels;
  const int top = c->line_wpc_cfg ? std::min(c->line_wpc_cfg, c->line_wpc_max) : c->line_wpc_max;
  ProtoChoice best;
  best.proto = proto;
  best.us = -1.0;
  for (int w = 1; w <= top; w *= 2) {
    const LinePlan plan = line_plan(a, mode, esize, lp, dtype, w);
    if (w > 1 && (!line_plan_resident(c, plan) || (!c->line_wpc_cfg && nc * w > 2 * (int64_t)c->compute_units)))
      continue;
    const LineShape sh{w, lp == kLineWide && dtype != RINGSIM_INT64 ? 12.0 : 8.0,
                       (double)(kFlagSlotBytes / 16), (double)c->chunk_bytes, c->compute_units};
    const double us = line_model_us(m, mode, c->nranks, c->nchannels, bytes, model_proto(proto), sh);
    // A configured count is taken as the most that may run, not a hint.
    if (best.us < 0.0 || (c->line_wpc_cfg ? w > best.plan.wpc : us < best.us)) {
      best.plan = plan;
      best.us = us;
    }
  }
  return best;
}

// The protocol of one call. A fixed protocol is taken as configured; AUTO
// takes the flag protocol below a configured threshold and bulk above it,
// else the protocol the cost model predicts fastest, each line protocol with
// the workgroups its launch would take. Every protocol walks the same
// partition (the line protocols walk each loop in groups of kLineGroupSteps
// slots), so the choice never changes a result bit.
ProtoChoice pick_proto(const ringsim_comm* c, int mode, size_t count, int dtype) {
  const int esize = dtype_size(dtype);
  const RingArgs a = call_shape(c, count, esize);
  const double bytes = (double)((mode == kAllReduce ? count : count * c->nranks) * esize);
  auto bulk = [&]() {
    ProtoChoice pc;
    pc.proto = RINGSIM_PROTO_BULK;
    pc.plan = LinePlan{comm_bulk_wpc(c, a, mode, esize), kHostLinesMulti};
    pc.us = bulk_model_us(RingModel(), mode, c->nranks, bytes);
    return pc;
  };
  if (c->proto == RINGSIM_PROTO_FLAG || c->proto == RINGSIM_PROTO_WIDE) return pick_line(c, a, mode, dtype, c->proto, bytes);
  if (c->proto == RINGSIM_PROTO_BULK) return bulk();
  if (c->flag_threshold)
    return bytes < (double)c->flag_threshold ? pick_line(c, a, mode, dtype, RINGSIM_PROTO_FLAG, bytes) : bulk();
  ProtoChoice best = bulk();
  for (const int p : {RINGSIM_PROTO_FLAG, RINGSIM_PROTO_WIDE}) {
    const ProtoChoice pc = pick_line(c, a, mode, dtype, p, bytes);
    if (pc.us < best.us) best = pc;
  }
  return best;
}

ringsim_result_t launch_local_copy(ringsim_comm* c, const void* const* sb, void* const* rb, size_t bytes,
                                   hipStream_t s) {
  if (sb[0] == rb[0] || bytes == 0) return RINGSIM_SUCCESS;
  CopyArgs ca;
  std::memset(&ca, 0, sizeof(ca));
  ca.src[0] = static_cast<const char*>(sb[0]);
  ca.dst[0] = static_cast<char*>(rb[0]);
  ca.block_bytes = (int64_t)bytes;
  ca.nranks = 1;
  ca.transpose = 0;
  if (launch_copy(ca, s) != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  return RINGSIM_SUCCESS;
}

// Payload bytes of one tree step (one WIDE line per thread: 12 bytes, 8 for
// int64).
int64_t tree_slice_bytes(int esize) { return (int64_t)kThreads * (esize == 8 ? 8 : 12); }

// Tree channels of one all-reduce and the predicted time: one step of the
// half buffer its tree owns per channel, with at most one or two tree
// workgroups per compute unit, whichever the cost model predicts faster
// (two pay off once every channel pipelines several steps).
struct TreePlan {
  int channels;
  double us;
};

TreePlan tree_plan(const ringsim_comm* c, size_t bytes_per_rank, int esize) {
  const RingModel m;
  const int64_t slice = tree_slice_bytes(esize);
  const int64_t want = div_up((int64_t)(bytes_per_rank / 2), slice);
  TreePlan best{0, 0.0};
  for (int per_cu = 1; per_cu <= 2; ++per_cu) {
    const int64_t cap = std::max<int64_t>(1, per_cu * (int64_t)c->compute_units / (4 * (int64_t)c->nranks));
    const int ch = (int)std::max<int64_t>(1, std::min<int64_t>({want, cap, (int64_t)c->tree_channels}));
    if (ch == best.channels) continue;
    const double us = tree_model_us(m, c->nranks, c->tree_depth, ch, (double)slice, (double)(slice / kThreads),
                                    (double)bytes_per_rank, c->compute_units);
    if (best.channels == 0 || us < best.us) best = TreePlan{ch, us};
  }
  return best;
}

// AUTO's algorithm: the tree only where the fold order cannot show in the
// result (integers wrap associatively; max/min pick one input), only when
// the flag-packed lines it moves are allowed (any protocol but BULK), and
// only when it is predicted to be faster than the ring.
bool auto_picks_tree(const ringsim_comm* c, int dtype, int op, size_t count) {
  const bool order_free = dtype == RINGSIM_INT32 || dtype == RINGSIM_INT64 || op == RINGSIM_MAX || op == RINGSIM_MIN;
  const bool lines_ok = c->proto != RINGSIM_PROTO_BULK;
  if (!order_free || !lines_ok || c->tree_channels < 1) return false;
  return tree_plan(c, count * (size_t)dtype_size(dtype), dtype_size(dtype)).us < pick_proto(c, kAllReduce, count, dtype).us;
}

// Is `s` being captured into a graph? (A stream the runtime cannot tell
// about is taken as not captured.)
bool is_capturing(hipStream_t s) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cap != hipStreamCaptureStatusNone;
}

// Flag span bookkeeping. An upper bound on the steps any one FIFO of a ring
// line launch moves ("NCCL" book, s. 2.3: a loop of N chunks, 2(N-1) sending
// stages for the all-reduce, N-1 for reduce-scatter and all-gather): loop l
// hands each stage a unit of at most cur_l elements (the loop's chunk; its
// workgroup parts are smaller still), moved in ceil(unit / slice) steps, and
// the chunks of all loops of the longest channel L0 add up to at most
// L0 / N + A (all-reduce) or L0.
uint64_t line_steps_bound(int mode, int64_t count, int nranks, int nchannels, int64_t chunk, int esize,
                          int64_t payload_bytes) {
  const int64_t A = 16 / esize;
  const int64_t slice = (int64_t)(kFlagSlotBytes / 16) * payload_bytes / esize;
  const int64_t L0 = std::min<int64_t>(count, channel_span(count, nchannels, A));
  if (L0 <= 0) return 0;
  const bool ar = mode == kAllReduce;
  const int64_t loops = div_up(L0, ar ? (int64_t)nranks * chunk : chunk);
  const int64_t units = ar ? L0 / nranks + A : L0;
  const int64_t sends = ar ? 2 * (int64_t)(nranks - 1) : (int64_t)(nranks - 1);
  return (uint64_t)(sends * (div_up(units, slice) + loops));
}

// The same for the double tree: a FIFO carries one tree channel, at most the
// tree's half of the buffer, one WIDE line per thread and step.
uint64_t tree_steps_bound(int64_t count, int esize) {
  const int64_t A = 16 / esize;
  const int64_t half = align_up(div_up(count, 2), A);
  return (uint64_t)(div_up(half * esize, (int64_t)kThreads * (esize == 8 ? 8 : 12)) + 1);
}

// Before a line or tree launch of `bound` steps per FIFO: zero that family's
// FIFOs and counters first if the steps since the last zeroing could take a
// counter past the span (then flags restart at 1 over all-zero lines). Not
// while the stream is captured (a zeroing kernel in a graph would run at
// every replay): the zeroing then waits for the next call made outside
// capture. A captured call counts once, its replays not at all; a kernel
// that leaves a counter past kFlagSpanGuard reports it.
ringsim_result_t guard_span(ringsim_comm* c, bool tree, uint64_t bound, hipStream_t s) {
  if (bound > kFlagSpanGuard) {
    RS_LOG(kLogWarn, "a line or tree call of %llu steps per FIFO exceeds the flag span", (unsigned long long)bound);
    return RINGSIM_INVALID_USAGE;
  }
  uint64_t& span = tree ? c->tree_span : c->line_span;
  if (span + bound > c->span_limit && !is_capturing(s)) {
    hipError_t e = tree ? launch_zero(c->tree_fifo, c->tree_fifo_bytes, s) : launch_zero(c->flag_fifo, c->flag_fifo_bytes, s);
    if (e == hipSuccess) e = tree ? launch_zero(c->tree_ctr, c->tree_ctr_bytes, s) : launch_zero(c->ctr, c->ctr_bytes, s);
    if (e != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
    span = 0;
    ++(tree ? c->tree_resets : c->line_resets);
    RS_LOG(kLogInfo, "comm %p: %s FIFOs zeroed (flag span)", (void*)c, tree ? "tree" : "line");
  }
  span += bound;
  return RINGSIM_SUCCESS;
}

ringsim_result_t launch_tree(ringsim_comm* c, const void* const* sb, void* const* rb, size_t count, int dtype,
                             int op, bool vec, hipStream_t s) {
  TreeArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < c->nranks; ++r) {
    a.send[r] = static_cast<const char*>(sb[r]);
    a.recv[r] = static_cast<char*>(rb[r]);
  }
  a.count = (int64_t)count;
  a.nranks = c->nranks;
  a.nchannels = tree_plan(c, count * (size_t)dtype_size(dtype), dtype_size(dtype)).channels;
  c->last_tree_channels = a.nchannels;
  a.ch_stride = c->tree_channels;
  a.nslots = kTreeSlots;
  a.slot_bytes = kTreeSlotBytes;
  a.head_every = kTreeSlots / 2;
  a.vec_ok = vec;
  a.skip_rank = c->skip_rank;
  std::memcpy(a.link, c->tree_link, sizeof(a.link));
  a.fifo = c->tree_fifo;
  a.ctr = c->tree_ctr;
  a.dev_abort = c->dev_abort;
  a.host_abort = c->host_words_dev;
  a.host_err = c->host_words_dev + 1;
  a.timeout_ticks = c->timeout_ticks;
  const hipError_t e = launch_tree_kernel(a, dtype, op, s);
  if (e != hipSuccess) {
    RS_LOG(kLogWarn, "tree kernel launch failed: %s", hipGetErrorString(e));
    return RINGSIM_UNHANDLED_DEVICE_ERROR;
  }
  return RINGSIM_SUCCESS;
}


ringsim_result_t run_ring(ringsim_comm* c, int mode, const void* const* sb, void* const* rb, size_t count,
                          int dtype, int op, ringsim_stream_t stream) {
  ringsim_result_t res = check_comm(c);
  if (res != RINGSIM_SUCCESS) return res;
  if ((res = poll_async(c)) != RINGSIM_SUCCESS) return res;
  if (!valid_dtype(dtype) || !valid_op(op)) return RINGSIM_INVALID_ARGUMENT;
  const int esize = dtype_size(dtype);
  const int64_t n = c->nranks;
  if (count > (size_t)(INT64_MAX / 16) / (size_t)n / (size_t)esize) return RINGSIM_INVALID_ARGUMENT;
  if (count == 0) return RINGSIM_SUCCESS;
  bool vec = false;
  if ((res = check_bufs(c, sb, rb, esize, &vec)) != RINGSIM_SUCCESS) return res;
  if ((res = check_device(c)) != RINGSIM_SUCCESS) return res;
  hipStream_t s = static_cast<hipStream_t>(stream);
  c->calls++;
  c->last_group = 0;
  if (n == 1) {
    // A single rank is a local copy ("NCCL" book, enqueue chapter, taskAppend).
    return launch_local_copy(c, sb, rb, count * esize, s);
  }
  if (mode == kAllReduce) {
    const bool tree = c->algo == RINGSIM_ALGO_TREE ||
                      (c->algo == RINGSIM_ALGO_AUTO && auto_picks_tree(c, dtype, op, count));
    c->last_algo = tree ? RINGSIM_ALGO_TREE : RINGSIM_ALGO_RING;
    c->last_tree_channels = 0;
    if (tree) {
      const ringsim_result_t g = guard_span(c, true, tree_steps_bound((int64_t)count, esize), s);
      return g != RINGSIM_SUCCESS ? g : launch_tree(c, sb, rb, count, dtype, op, vec, s);
    }
  }
  RingArgs a;
  fill_common(c, &a, sb, rb);
  a.count = (int64_t)count;
  const ProtoChoice pc = pick_proto(c, mode, count, dtype);
  const int proto = pc.proto;
  fill_proto(c, &a, proto, esize, pc.plan.wpc);
  // Vector moves need every unit to start on a 16-byte boundary; for the
  // block-strided collectives that requires whole 16-byte blocks.
  a.vec_ok = vec && (mode == kAllReduce || (count * esize) % 16 == 0);
  c->last_proto = proto;
  hipError_t e;
  if (proto == RINGSIM_PROTO_BULK) {
    const int64_t rank_bytes = (int64_t)(mode == kAllReduce ? count : count * (size_t)n) * esize;
    if (rank_bytes <= kBulkStageMinBytes) a.lds_stage = 0;
    a.group = bulk_call_depth(c, &a, mode, esize);
    c->last_group = a.group;
    c->last_wpc = a.wpc;
    e = launch_ring_bulk(a, mode, dtype, op, s);
  } else {
    const int lp = proto == RINGSIM_PROTO_WIDE ? kLineWide : kLineFlag;
    const int64_t payload = lp == kLineWide && dtype != RINGSIM_INT64 ? 12 : 8;
    const ringsim_result_t g = guard_span(
        c, false, line_steps_bound(mode, a.count, a.nranks, a.nchannels, a.chunk, esize, payload), s);
    if (g != RINGSIM_SUCCESS) return g;
    c->last_wpc = a.wpc;
    e = pc.plan.mode == kHostLinesHalf  ? launch_ring_lines_half(a, lp, mode, dtype, op, s)
        : pc.plan.mode == kHostLinesOne ? launch_ring_lines_one(a, lp, mode, dtype, op, s)
                                        : launch_ring_lines_multi(a, lp, mode, dtype, op, s);
  }
  if (e != hipSuccess) {
    RS_LOG(kLogWarn, "kernel launch failed: %s", hipGetErrorString(e));
    return RINGSIM_UNHANDLED_DEVICE_ERROR;
  }
  return RINGSIM_SUCCESS;
}

void free_comm_memory(ringsim_comm* c) {
  if (c->fifo) (void)hipFree(c->fifo);
  if (c->flag_fifo) (void)hipFree(c->flag_fifo);
  if (c->ctr) (void)hipFree(c->ctr);
  if (c->bulk_ctr) (void)hipFree(c->bulk_ctr);
  c->bulk_ctr = nullptr;
  if (c->echo) (void)hipFree(c->echo);
  c->echo = nullptr;
  if (c->tree_fifo) (void)hipFree(c->tree_fifo);
  if (c->tree_ctr) (void)hipFree(c->tree_ctr);
  c->tree_fifo = nullptr;
  c->tree_ctr = nullptr;
  if (c->dev_abort) (void)hipFree(c->dev_abort);
  if (c->host_words) (void)hipHostFree(c->host_words);
  c->fifo = c->flag_fifo = nullptr;
  c->ctr = nullptr;
  c->dev_abort = nullptr;
  c->host_words = c->host_words_dev = nullptr;
}

}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free all-reduce: the bulk ring kernel on a file-scope scratch
// ---------------------------------------------------------------------------

namespace {

// Geometry of the allocation-free call: at most kNaMaxPipes ring pipelines
// (ranks x channels x workgroups per channel), 8 FIFO slots of 32 KiB each,
// and a stage that moves at most 4 slot steps before the next stage runs
// (step groups), so one stage never fills more than half of a FIFO whatever
// the chunk size. The partition (channels, loops, chunks) is the
// communicator's, so results equal ringsim_allreduce's bit for bit.
constexpr int kNaMaxPipes = 128;
constexpr int kNaSlots = 8;
constexpr int kNaSlotBytes = kDefaultSlotBytes;
constexpr int kNaGroupSteps = kNaSlots / 2;
constexpr size_t kNaCtrBytes = (size_t)kNaMaxPipes * sizeof(FifoCtr);  // 32 KiB
constexpr size_t kNaWordBytes = 256;  // device abort word, error word, a never-set abort word
constexpr size_t kNaFifoBytes = (size_t)kNaMaxPipes * kNaSlots * kNaSlotBytes;  // 32 MiB
constexpr size_t kNaScratchBytes = kNaCtrBytes + kNaWordBytes + kNaFifoBytes;
constexpr int kNaMaxDevices = 64;

}  // namespace

// One copy per GPU, held until the process ends: counters, then the error
// words, then the FIFO slots. Host code never passes this name to a kernel
// (on the host it is only a stand-in for the symbol); it uses the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kNaScratchBytes];

namespace {

// Zeroes the counters and error words of the scratch before every call: a
// call that gave up leaves them behind, and every call starts its counters
// at zero. A kernel rather than a memset, so that calls can be captured.
__global__ void __launch_bounds__(kThreads) noalloc_clear(uint4* p, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct NaDevice {
  char* base;  // device address of `scratch` on this GPU
  int cus;
  int per_cu;  // resident bulk workgroups per compute unit
  int clock_khz;
};

std::mutex g_na_mu;
NaDevice g_na[kNaMaxDevices];
bool g_na_ready[kNaMaxDevices];

// Set-up on a device's first call, with that device current: the device
// address of its copy of the scratch array, and what the launch needs of it.
const NaDevice* na_device(int dev) {
  if (dev < 0 || dev >= kNaMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_na_mu);
  if (g_na_ready[dev]) return &g_na[dev];
  NaDevice d{};
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  d.base = static_cast<char*>(ptr);
  if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&d.clock_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || d.cus <= 0 ||
      d.clock_khz <= 0)
    return nullptr;
  d.per_cu = bulk_blocks_per_cu(2 * (size_t)kNaSlotBytes);
  if (d.per_cu <= 0) return nullptr;
  g_na[dev] = d;
  g_na_ready[dev] = true;
  return &g_na[dev];
}

}  // namespace

extern "C" {

ringsim_result_t ringsim_config_default(ringsim_config_t* cfg) {
  if (!cfg) return RINGSIM_INVALID_ARGUMENT;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->chunk_bytes = (size_t)env_long("RINGSIM_CHUNK_BYTES", 524288);
  cfg->workgroups_per_channel = (int)env_long("RINGSIM_WPC", 0);
  cfg->slot_bytes = (size_t)env_long("RINGSIM_SLOT_BYTES", kDefaultSlotBytes);
  cfg->nslots = (int)env_long("RINGSIM_NSLOTS", kDefaultSlots);
  cfg->timeout_ms = (int)env_long("RINGSIM_TIMEOUT_MS", 10000);
  cfg->flag_threshold_bytes = (size_t)env_long("RINGSIM_FLAG_THRESHOLD", 0);
  cfg->algo = env_algo(RINGSIM_ALGO_AUTO);
  cfg->line_workgroups_per_channel = (int)env_long("RINGSIM_LINE_WPC", 0);
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_comm_init(ringsim_comm_t* comm, int nranks, int nchannels, int proto) {
  return ringsim_comm_init_config(comm, nranks, nchannels, proto, nullptr);
}

ringsim_result_t ringsim_comm_init_config(ringsim_comm_t* comm, int nranks, int nchannels, int proto,
                                          const ringsim_config_t* user_cfg) {
  const RoctxRange range("ringsim_comm_init");
  if (!comm) return RINGSIM_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS) return RINGSIM_INVALID_ARGUMENT;
  if (nchannels < 1 || nchannels > RINGSIM_MAX_CHANNELS) return RINGSIM_INVALID_ARGUMENT;
  if (proto < RINGSIM_PROTO_AUTO || proto > RINGSIM_PROTO_WIDE) return RINGSIM_INVALID_ARGUMENT;
  ringsim_config_t cfg;
  ringsim_config_default(&cfg);
  if (user_cfg) {
    if (user_cfg->chunk_bytes) cfg.chunk_bytes = user_cfg->chunk_bytes;
    if (user_cfg->workgroups_per_channel) cfg.workgroups_per_channel = user_cfg->workgroups_per_channel;
    if (user_cfg->slot_bytes) cfg.slot_bytes = user_cfg->slot_bytes;
    if (user_cfg->nslots) cfg.nslots = user_cfg->nslots;
    if (user_cfg->timeout_ms) cfg.timeout_ms = user_cfg->timeout_ms;
    if (user_cfg->flag_threshold_bytes) cfg.flag_threshold_bytes = user_cfg->flag_threshold_bytes;
    if (user_cfg->algo) cfg.algo = user_cfg->algo;
    if (user_cfg->line_workgroups_per_channel) cfg.line_workgroups_per_channel = user_cfg->line_workgroups_per_channel;
  }
  if (cfg.algo < RINGSIM_ALGO_AUTO || cfg.algo > RINGSIM_ALGO_TREE) return RINGSIM_INVALID_ARGUMENT;
  if (cfg.chunk_bytes == 0 || cfg.chunk_bytes % 16 || cfg.chunk_bytes > ((size_t)1 << 30))
    return RINGSIM_INVALID_ARGUMENT;
  if (cfg.slot_bytes < 4096 || cfg.slot_bytes % 4096 || cfg.slot_bytes > ((size_t)1 << 22))
    return RINGSIM_INVALID_ARGUMENT;
  if (cfg.nslots < 2 || cfg.nslots > 4096) return RINGSIM_INVALID_ARGUMENT;
  if (cfg.workgroups_per_channel < 0 || cfg.workgroups_per_channel > RINGSIM_MAX_WORKGROUPS_PER_CHANNEL)
    return RINGSIM_INVALID_ARGUMENT;
  if (cfg.timeout_ms <= 0) return RINGSIM_INVALID_ARGUMENT;
  {
    const int lw = cfg.line_workgroups_per_channel;
    if (lw < 0 || lw > kMaxLineWpc || (lw & (lw - 1))) return RINGSIM_INVALID_ARGUMENT;
  }

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  int cus = 0, clock_khz = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || cus <= 0 ||
      clock_khz <= 0)
    return RINGSIM_UNHANDLED_DEVICE_ERROR;
  // Bulk steps stage their own operand in LDS (double-buffered) unless the
  // slot is too large or RINGSIM_LDS_STAGE=0.
  const int lds_stage = cfg.slot_bytes <= (size_t)kMaxStagedSlotBytes && env_long("RINGSIM_LDS_STAGE", 1) != 0;
  const int line_per_cu[3] = {line_multi_blocks_per_cu(), line_one_blocks_per_cu(), line_half_blocks_per_cu()};
  const int per_cu = std::min({bulk_blocks_per_cu(lds_stage ? 2 * cfg.slot_bytes : 0), line_per_cu[0],
                               line_per_cu[1], line_per_cu[2]});
  if (per_cu <= 0) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  const int64_t max_resident = (int64_t)per_cu * cus;

  // Workgroups per channel: enough ring pipelines to give every CU two
  // workgroups, but never more workgroups than can be resident at once (every
  // workgroup of a launch spins on its neighbours).
  const int64_t nc = (int64_t)nranks * nchannels;
  if (nc > max_resident) return RINGSIM_INVALID_USAGE;
  int wpc = cfg.workgroups_per_channel;
  if (wpc == 0) wpc = (int)std::max<int64_t>(1, std::min<int64_t>(RINGSIM_MAX_WORKGROUPS_PER_CHANNEL,
                                                                    (2 * (int64_t)cus) / nc));
  while (wpc > 1 && nc * wpc > max_resident) --wpc;
  if (nc * wpc > max_resident) return RINGSIM_INVALID_USAGE;

  // Line launches: up to kMaxLineWpc workgroups per channel, as many as the
  // device can hold with the line kernel that holds the most (the kernel a
  // launch needs is checked per call).
  const int line_best_cu = std::max({line_per_cu[0], line_per_cu[1], line_per_cu[2]});
  int line_wpc_max = 1;
  while (line_wpc_max < kMaxLineWpc && nc * line_wpc_max * 2 <= (int64_t)line_best_cu * cus) line_wpc_max *= 2;
  size_t line_fifo_per_nc = 0;
  for (int w = 1; w <= line_wpc_max; w *= 2) line_fifo_per_nc += (size_t)line_level_bytes(w);

  // FIFO depth: one stage of one workgroup may fill at most half of its FIFO,
  // as NCCL's chunkSteps = NCCL_STEPS/2 ("NCCL" book, enqueue chapter,
  // ALLREDUCE_CHUNKSTEPS). With every rank in stage 0 (sending only), a deeper
  // stage could fill every FIFO of the ring at once and stall it.
  const size_t stage_bytes = (size_t)align_up(div_up((int64_t)cfg.chunk_bytes, wpc), 16);
  const int slices = (int)div_up((int64_t)stage_bytes, (int64_t)cfg.slot_bytes);
  const int nslots = std::max(cfg.nslots, 2 * slices);

  // Tree channels: up to two per ring channel (a channel only splits a
  // tree's range further and never changes a value), and every workgroup of
  // a tree launch (4 per rank and channel) must be resident at once, like
  // the ring's.
  const int tree_per_cu = tree_blocks_per_cu();
  const int64_t tree_resident = (int64_t)tree_per_cu * cus;
  const int tree_channels =
      nranks < 2 ? 0 : (int)std::min<int64_t>(2 * (int64_t)nchannels, tree_resident / (4 * (int64_t)nranks));
  if (cfg.algo == RINGSIM_ALGO_TREE && nranks > 1 && tree_channels < 1) return RINGSIM_INVALID_USAGE;

  ringsim_comm* c = new (std::nothrow) ringsim_comm();
  if (!c) return RINGSIM_SYSTEM_ERROR;
  std::memset(c, 0, sizeof(*c));
  c->nranks = nranks;
  c->nchannels = nchannels;
  c->proto = proto;
  c->wpc = wpc;
  c->line_wpc_max = line_wpc_max;
  c->line_wpc_cfg = cfg.line_workgroups_per_channel;
  c->wpc_cfg = cfg.workgroups_per_channel != 0;
  c->pipe_mul = std::max(wpc, line_wpc_max);
  for (int k = 0; k < 3; ++k) c->line_per_cu[k] = line_per_cu[k];
  c->nslots = nslots;
  c->nslots_cfg = cfg.nslots;
  c->device = dev;
  c->chunk_bytes = cfg.chunk_bytes;
  c->slot_bytes = cfg.slot_bytes;
  c->flag_threshold = cfg.flag_threshold_bytes;
  c->timeout_ms = cfg.timeout_ms;
  // Testing knob: the workgroups of this rank return without doing anything,
  // so that its neighbours' bounded waits expire (failure-path tests).
  c->skip_rank = (int)env_long("RINGSIM_DEBUG_SKIP_RANK", -1);
  c->lds_stage = lds_stage;
  // Testing knob: a small flag span makes the host zero the line and tree
  // FIFOs every few calls, so that the reset path runs in tests.
  c->span_limit = (uint64_t)std::max<long>(1, env_long("RINGSIM_DEBUG_FLAG_SPAN", (long)kFlagSpanGuard));
  if (c->span_limit > kFlagSpanGuard) c->span_limit = kFlagSpanGuard;
  c->timeout_ticks = (uint64_t)cfg.timeout_ms * (uint64_t)clock_khz;
  c->compute_units = cus;
  c->blocks_per_cu = per_cu;
  c->sticky = RINGSIM_SUCCESS;
  c->algo = cfg.algo;
  c->tree_channels = tree_channels;
  c->tree_depth = double_tree_depth(nranks);
  for (int t = 0; t < 2; ++t) {
    for (int r = 0; r < nranks; ++r) {
      const TreeLinks l = double_tree(nranks, r, t);
      c->tree_link[t][r][0] = (int8_t)l.parent;
      c->tree_link[t][r][1] = (int8_t)l.kid[0];
      c->tree_link[t][r][2] = (int8_t)l.kid[1];
    }
  }

  c->fifo_bytes = (size_t)(nc * wpc) * nslots * cfg.slot_bytes;
  c->flag_fifo_bytes = (size_t)nc * line_fifo_per_nc;
  c->ctr_bytes = (size_t)(nc * c->pipe_mul) * sizeof(FifoCtr);
  c->bulk_ctr_bytes = (size_t)(nc * wpc) * sizeof(FifoCtr);
  // Debug: a (step, bytes) record beside every bulk slot, checked by its
  // consumer ("NCCL" book, s. 2.4: ncclConnFifo's size and offset per step).
  c->echo_bytes = env_long("RINGSIM_DEBUG_FIFO", 0) != 0 ? (size_t)(nc * wpc) * nslots * sizeof(FifoEcho) : 0;
  const size_t tree_fifos = (size_t)2 * tree_channels * nranks * 2;
  c->tree_fifo_bytes = tree_fifos * kTreeSlots * kTreeSlotBytes;
  c->tree_ctr_bytes = tree_fifos * sizeof(FifoCtr);
  bool ok = hipMalloc((void**)&c->fifo, c->fifo_bytes) == hipSuccess &&
            hipMalloc((void**)&c->flag_fifo, c->flag_fifo_bytes) == hipSuccess &&
            hipMalloc((void**)&c->ctr, c->ctr_bytes) == hipSuccess &&
            hipMalloc((void**)&c->bulk_ctr, c->bulk_ctr_bytes) == hipSuccess &&
            hipMalloc((void**)&c->dev_abort, 256) == hipSuccess &&
            hipHostMalloc((void**)&c->host_words, 256, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess;
  if (ok) ok = hipHostGetDevicePointer((void**)&c->host_words_dev, c->host_words, 0) == hipSuccess;
  if (ok && c->echo_bytes) ok = hipMalloc((void**)&c->echo, c->echo_bytes) == hipSuccess;
  if (ok && tree_fifos) {
    ok = hipMalloc((void**)&c->tree_fifo, c->tree_fifo_bytes) == hipSuccess &&
         hipMalloc((void**)&c->tree_ctr, c->tree_ctr_bytes) == hipSuccess &&
         hipMemset(c->tree_fifo, 0, c->tree_fifo_bytes) == hipSuccess &&
         hipMemset(c->tree_ctr, 0, c->tree_ctr_bytes) == hipSuccess;
  }
  // Flags of the flag-packed FIFO start at zero, a value no step ever uses.
  if (ok) ok = hipMemset(c->flag_fifo, 0, c->flag_fifo_bytes) == hipSuccess &&
               hipMemset(c->ctr, 0, c->ctr_bytes) == hipSuccess &&
               hipMemset(c->bulk_ctr, 0, c->bulk_ctr_bytes) == hipSuccess &&
               hipMemset(c->dev_abort, 0, 256) == hipSuccess &&
               hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    free_comm_memory(c);
    delete c;
    (void)hipGetLastError();
    return RINGSIM_UNHANDLED_DEVICE_ERROR;
  }
  std::memset(c->host_words, 0, 256);
  c->start_magic = kLiveMagic;
  c->end_magic = kLiveMagic;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(c);
  }
  RS_LOG(kLogInfo,
         "comm %p: nranks %d nchannels %d proto %d wpc %d nslots %d slot %zu chunk %zu fifo %zu B flag fifo %zu B "
         "lds stage %d resident %d/CU x %d CUs",
         (void*)c, nranks, nchannels, proto, wpc, nslots, cfg.slot_bytes, cfg.chunk_bytes, c->fifo_bytes,
         c->flag_fifo_bytes, lds_stage, per_cu, cus);
  *comm = c;
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_comm_destroy(ringsim_comm_t comm) {
  const RoctxRange range("ringsim_comm_destroy");
  ringsim_result_t res = check_comm(comm);
  if (res != RINGSIM_SUCCESS) return res;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.erase(comm);
  }
  // Every kernel bounds its waits, so this returns even after an abort. The
  // whole device is synchronized rather than the last stream the
  // communicator saw: that stream may have been destroyed since (freeing
  // device memory waits for the device anyway).
  const hipError_t e = hipDeviceSynchronize();
  free_comm_memory(comm);
  comm->start_magic = kDeadMagic;
  comm->end_magic = kDeadMagic;
  delete comm;
  return e == hipSuccess ? RINGSIM_SUCCESS : RINGSIM_UNHANDLED_DEVICE_ERROR;
}

ringsim_result_t ringsim_comm_query(ringsim_comm_t comm, ringsim_comm_info_t* info) {
  ringsim_result_t res = check_comm(comm);
  if (res != RINGSIM_SUCCESS) return res;
  if (!info) return RINGSIM_INVALID_ARGUMENT;
  std::memset(info, 0, sizeof(*info));
  info->nranks = comm->nranks;
  info->nchannels = comm->nchannels;
  info->proto = comm->proto;
  info->workgroups_per_channel = comm->wpc;
  info->nslots = comm->nslots;
  info->device = comm->device;
  info->chunk_bytes = comm->chunk_bytes;
  info->slot_bytes = comm->slot_bytes;
  info->flag_threshold_bytes = comm->flag_threshold;
  info->fifo_bytes = comm->fifo_bytes;
  info->flag_fifo_bytes = comm->flag_fifo_bytes;
  info->max_resident_workgroups = comm->blocks_per_cu * comm->compute_units;
  info->compute_units = comm->compute_units;
  info->calls = comm->calls;
  info->last_proto = comm->last_proto;
  info->algo = comm->algo;
  info->tree_channels = comm->tree_channels;
  info->tree_fifo_bytes = comm->tree_fifo_bytes;
  info->last_algo = comm->last_algo;
  info->line_max_workgroups_per_channel = comm->line_wpc_max;
  info->last_workgroups_per_channel = comm->last_wpc;
  info->last_group_steps = comm->last_group;
  info->last_tree_channels = comm->last_tree_channels;
  info->line_fifo_resets = comm->line_resets;
  info->tree_fifo_resets = comm->tree_resets;
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_allreduce(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                   size_t count, int dtype, int op, ringsim_stream_t stream) {
  const RoctxRange range("ringsim_allreduce");
  return run_ring(comm, kAllReduce, sendbufs, recvbufs, count, dtype, op, stream);
}

ringsim_result_t ringsim_reduce_scatter(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                        size_t recvcount, int dtype, int op, ringsim_stream_t stream) {
  const RoctxRange range("ringsim_reduce_scatter");
  return run_ring(comm, kReduceScatter, sendbufs, recvbufs, recvcount, dtype, op, stream);
}

ringsim_result_t ringsim_all_gather(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                    size_t sendcount, int dtype, ringsim_stream_t stream) {
  const RoctxRange range("ringsim_all_gather");
  return run_ring(comm, kAllGather, sendbufs, recvbufs, sendcount, dtype, RINGSIM_SUM, stream);
}

ringsim_result_t ringsim_alltoall(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                  size_t count, int dtype, ringsim_stream_t stream) {
  const RoctxRange range("ringsim_alltoall");
  ringsim_result_t res = check_comm(comm);
  if (res != RINGSIM_SUCCESS) return res;
  if ((res = poll_async(comm)) != RINGSIM_SUCCESS) return res;
  if (!valid_dtype(dtype)) return RINGSIM_INVALID_ARGUMENT;
  const int esize = dtype_size(dtype);
  const int64_t n = comm->nranks;
  if (count > (size_t)(INT64_MAX / 16) / (size_t)n / (size_t)esize) return RINGSIM_INVALID_ARGUMENT;
  if (count == 0) return RINGSIM_SUCCESS;
  bool vec = false;
  if ((res = check_bufs(comm, sendbufs, recvbufs, esize, &vec)) != RINGSIM_SUCCESS) return res;
  for (int r = 0; r < n; ++r)
    if (sendbufs[r] == recvbufs[r]) return RINGSIM_INVALID_ARGUMENT;  // no in-place transpose
  if ((res = check_device(comm)) != RINGSIM_SUCCESS) return res;
  hipStream_t s = static_cast<hipStream_t>(stream);
  comm->calls++;
  CopyArgs ca;
  std::memset(&ca, 0, sizeof(ca));
  for (int r = 0; r < n; ++r) {
    ca.src[r] = static_cast<const char*>(sendbufs[r]);
    ca.dst[r] = static_cast<char*>(recvbufs[r]);
  }
  ca.block_bytes = (int64_t)count * esize;
  ca.nranks = (int)n;
  ca.transpose = 1;
  return launch_copy(ca, s) == hipSuccess ? RINGSIM_SUCCESS : RINGSIM_UNHANDLED_DEVICE_ERROR;
}

ringsim_result_t ringsim_get_async_error(ringsim_comm_t comm, ringsim_result_t* async_error) {
  ringsim_result_t res = check_comm(comm);
  if (res != RINGSIM_SUCCESS) return res;
  if (!async_error) return RINGSIM_INVALID_ARGUMENT;
  // Errors only, as ncclCommGetAsyncError reports the communicator's
  // asyncResult: whether enqueued work has finished is for the caller's
  // streams and events to tell (a per-call event would cost every call
  // 2.6-4.3 us of device time on MI355X).
  *async_error = poll_async(comm);
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_abort(ringsim_comm_t comm) {
  const RoctxRange range("ringsim_abort");
  ringsim_result_t res = check_comm(comm);
  if (res != RINGSIM_SUCCESS) return res;
  __atomic_store_n(&comm->host_words[0], 1u, __ATOMIC_RELEASE);
  comm->sticky = RINGSIM_ABORTED;
  return RINGSIM_SUCCESS;
}

const char* ringsim_get_error_string(ringsim_result_t result) {
  switch (result) {
    case RINGSIM_SUCCESS: return "no error";
    case RINGSIM_UNHANDLED_DEVICE_ERROR: return "unhandled device (HIP) error";
    case RINGSIM_SYSTEM_ERROR: return "system error";
    case RINGSIM_INTERNAL_ERROR: return "internal error: a ring kernel timed out waiting for a peer";
    case RINGSIM_INVALID_ARGUMENT: return "invalid argument";
    case RINGSIM_INVALID_USAGE: return "invalid usage";
    case RINGSIM_IN_PROGRESS: return "operation in progress";
    case RINGSIM_ABORTED: return "communicator aborted";
    default: return "unknown result code";
  }
}

ringsim_result_t ringsim_debug_model(int coll, int nranks, int nchannels, size_t bytes_per_rank, double* us_bulk,
                                     double* us_flag, double* us_wide) {
  if (!us_bulk || !us_flag || !us_wide) return RINGSIM_INVALID_ARGUMENT;
  if (coll < RINGSIM_COLL_ALLREDUCE || coll > RINGSIM_COLL_ALL_GATHER) return RINGSIM_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS || nchannels < 1 || nchannels > RINGSIM_MAX_CHANNELS)
    return RINGSIM_INVALID_ARGUMENT;
  const RingModel m;
  const double b = (double)bytes_per_rank;
  *us_bulk = bulk_model_us(m, coll, nranks, b);
  // Line protocols: the fastest of 1, 2, 4, 8 workgroups per channel on a
  // 256-CU device, at most two workgroups per CU beyond one per channel.
  for (int k = 0; k < 2; ++k) {
    const int proto = k ? kModelWide : kModelFlag;
    double best = -1.0;
    for (int w = 1; w <= kMaxLineWpc; w *= 2) {
      if (w > 1 && (int64_t)nranks * nchannels * w > 2 * 256) break;
      const LineShape sh{w, k ? 12.0 : 8.0, (double)(kFlagSlotBytes / 16), 524288.0, 256};
      const double us = line_model_us(m, coll, nranks, nchannels, b, proto, sh);
      if (best < 0.0 || us < best) best = us;
    }
    *(k ? us_wide : us_flag) = best;
  }
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_debug_tree(int nranks, int rank, int* links) {
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS || rank < 0 || rank >= nranks || !links)
    return RINGSIM_INVALID_ARGUMENT;
  for (int t = 0; t < 2; ++t) {
    const TreeLinks l = double_tree(nranks, rank, t);
    links[3 * t] = l.parent;
    links[3 * t + 1] = l.kid[0];
    links[3 * t + 2] = l.kid[1];
  }
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_debug_tree_model(int nranks, int tree_channels, size_t bytes_per_rank, double* us) {
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS || tree_channels < 1 || tree_channels > RINGSIM_MAX_CHANNELS || !us)
    return RINGSIM_INVALID_ARGUMENT;
  const RingModel m;
  // A 256-CU device, as the ring model above; 4-byte elements.
  const int64_t slice = tree_slice_bytes(4);
  *us = tree_model_us(m, nranks, double_tree_depth(nranks), tree_channels, (double)slice, (double)(slice / kThreads),
                      (double)bytes_per_rank, 256);
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_debug_flag_steps(int coll, int algo, int nranks, int nchannels, size_t chunk_bytes,
                                         size_t count, int dtype, int proto, uint64_t* steps) {
  if (!steps || !valid_dtype(dtype)) return RINGSIM_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS || nchannels < 1 || nchannels > RINGSIM_MAX_CHANNELS)
    return RINGSIM_INVALID_ARGUMENT;
  if (chunk_bytes == 0 || chunk_bytes % 16 || count > ((size_t)1 << 40)) return RINGSIM_INVALID_ARGUMENT;
  if (coll < RINGSIM_COLL_ALLREDUCE || coll > RINGSIM_COLL_ALL_GATHER) return RINGSIM_INVALID_ARGUMENT;
  const int esize = dtype_size(dtype);
  if (algo == RINGSIM_ALGO_TREE) {
    if (coll != RINGSIM_COLL_ALLREDUCE) return RINGSIM_INVALID_ARGUMENT;
    *steps = tree_steps_bound((int64_t)count, esize);
    return RINGSIM_SUCCESS;
  }
  if (algo != RINGSIM_ALGO_RING || (proto != RINGSIM_PROTO_FLAG && proto != RINGSIM_PROTO_WIDE))
    return RINGSIM_INVALID_ARGUMENT;
  const int64_t payload = proto == RINGSIM_PROTO_WIDE && dtype != RINGSIM_INT64 ? 12 : 8;
  *steps = line_steps_bound(coll, (int64_t)count, nranks, nchannels, (int64_t)chunk_bytes / esize, esize, payload);
  return RINGSIM_SUCCESS;
}

ringsim_result_t ringsim_debug_plan(int coll, size_t count, int nranks, int nchannels, size_t chunk_bytes,
                                    int dtype, int64_t* rows, size_t max_rows, size_t* nrows) {
  if (!nrows || !valid_dtype(dtype)) return RINGSIM_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS || nchannels < 1 || nchannels > RINGSIM_MAX_CHANNELS)
    return RINGSIM_INVALID_ARGUMENT;
  if (chunk_bytes == 0 || chunk_bytes % 16) return RINGSIM_INVALID_ARGUMENT;
  if (coll < RINGSIM_COLL_ALLREDUCE || coll > RINGSIM_COLL_ALL_GATHER) return RINGSIM_INVALID_ARGUMENT;
  if (count > ((size_t)1 << 40)) return RINGSIM_INVALID_ARGUMENT;
  const int64_t esize = dtype_size(dtype);
  const int64_t A = 16 / esize;
  const int64_t chunk = (int64_t)chunk_bytes / esize;
  size_t k = 0;
  auto emit = [&](int64_t c, int64_t l, int64_t ch, int64_t lo, int64_t hi) {
    if (rows && k < max_rows) {
      int64_t* row = rows + 5 * k;
      row[0] = c;
      row[1] = l;
      row[2] = ch;
      row[3] = lo;
      row[4] = hi;
    }
    ++k;
  };
  for (int c = 0; c < nchannels; ++c) {
    const Range chr = channel_range((int64_t)count, nchannels, c, A);
    const int64_t L = chr.hi - chr.lo;
    if (coll == RINGSIM_COLL_ALLREDUCE) {
      const int64_t loop = (int64_t)nranks * chunk;
      int64_t l = 0;
      for (int64_t off = 0; off < L; off += loop, ++l) {
        const int64_t rem = L - off;
        const int64_t cur = ar_loop_chunk(rem, nranks, chunk, A);
        for (int kk = 0; kk < nranks; ++kk) {
          const Range r = ar_chunk(off, rem, cur, kk);
          emit(c, l, kk, chr.lo + r.lo, chr.lo + r.hi);
        }
      }
    } else {
      int64_t l = 0;
      for (int64_t off = 0; off < L; off += chunk, ++l) emit(c, l, -1, chr.lo + off, chr.lo + min64(off + chunk, L));
    }
  }
  *nrows = k;
  return RINGSIM_SUCCESS;
}


ringsim_result_t ringsim_allreduce_noalloc(int nranks, int nchannels, const void* const* sendbufs,
                                           void* const* recvbufs, size_t count, int dtype, int op,
                                           ringsim_stream_t stream) {
  if (nranks < 1 || nranks > RINGSIM_MAX_RANKS || nchannels < 1 || nchannels > RINGSIM_MAX_CHANNELS)
    return RINGSIM_INVALID_ARGUMENT;
  if ((int64_t)nranks * nchannels > kNaMaxPipes) {
    RS_LOG(kLogWarn, "allreduce_noalloc: %d ranks x %d channels exceeds the scratch limit of %d ring pipelines",
           nranks, nchannels, kNaMaxPipes);
    return RINGSIM_INVALID_ARGUMENT;
  }
  if (!valid_dtype(dtype) || !valid_op(op)) return RINGSIM_INVALID_ARGUMENT;
  const int esize = dtype_size(dtype);
  if (count > (size_t)(INT64_MAX / 16) / (size_t)nranks / (size_t)esize) return RINGSIM_INVALID_ARGUMENT;
  ringsim_config_t cfg;
  ringsim_config_default(&cfg);
  if (cfg.chunk_bytes == 0 || cfg.chunk_bytes % 16 || cfg.chunk_bytes > ((size_t)1 << 30) || cfg.timeout_ms <= 0)
    return RINGSIM_INVALID_ARGUMENT;
  if (count == 0) return RINGSIM_SUCCESS;
  if (!sendbufs || !recvbufs) return RINGSIM_INVALID_ARGUMENT;
  bool vec = true;
  for (int r = 0; r < nranks; ++r) {
    const uintptr_t s = (uintptr_t)sendbufs[r], d = (uintptr_t)recvbufs[r];
    if (!s || !d || (s % esize) || (d % esize)) return RINGSIM_INVALID_ARGUMENT;
    if ((s | d) & 15u) vec = false;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  const NaDevice* d = na_device(dev);
  if (!d) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nranks == 1) {
    if (sendbufs[0] == recvbufs[0]) return RINGSIM_SUCCESS;
    CopyArgs ca;
    std::memset(&ca, 0, sizeof(ca));
    ca.src[0] = static_cast<const char*>(sendbufs[0]);
    ca.dst[0] = static_cast<char*>(recvbufs[0]);
    ca.block_bytes = (int64_t)count * esize;
    ca.nranks = 1;
    return launch_copy(ca, s) == hipSuccess ? RINGSIM_SUCCESS : RINGSIM_UNHANDLED_DEVICE_ERROR;
  }
  // Workgroups per channel: two per compute unit, within the scratch's
  // pipelines and what the device holds at once (every workgroup spins on
  // its neighbours).
  const int64_t nc = (int64_t)nranks * nchannels;
  const int64_t resident = (int64_t)d->per_cu * d->cus;
  int wpc = (int)std::max<int64_t>(
      1, std::min<int64_t>({(int64_t)RINGSIM_MAX_WORKGROUPS_PER_CHANNEL, 2 * (int64_t)d->cus / nc, kNaMaxPipes / nc}));
  while (wpc > 1 && nc * wpc > resident) --wpc;
  if (nc * wpc > resident) return RINGSIM_INVALID_USAGE;

  RingArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < nranks; ++r) {
    a.send[r] = static_cast<const char*>(sendbufs[r]);
    a.recv[r] = static_cast<char*>(recvbufs[r]);
  }
  a.count = (int64_t)count;
  a.chunk = (int64_t)cfg.chunk_bytes / esize;
  a.nranks = nranks;
  a.nchannels = nchannels;
  a.wpc = wpc;
  a.pipe_stride = nchannels * wpc;
  a.pipe_mul = wpc;
  a.fifo_stride = nchannels * wpc;
  a.fifo_mul = wpc;
  a.nslots = kNaSlots;
  a.slot_bytes = kNaSlotBytes;
  a.vec_ok = vec;
  a.ctr = reinterpret_cast<FifoCtr*>(d->base);
  uint32_t* words = reinterpret_cast<uint32_t*>(d->base + kNaCtrBytes);
  a.dev_abort = words;
  a.host_err = words + 1;
  a.host_abort = words + 2;  // nothing sets it: this call has no abort
  a.fifo = d->base + kNaCtrBytes + kNaWordBytes;
  a.timeout_ticks = (uint64_t)cfg.timeout_ms * (uint64_t)d->clock_khz;
  a.skip_rank = -1;
  a.lds_stage = (int64_t)count * esize > kBulkStageMinBytes;  // as ringsim_allreduce's bulk calls
  a.group = kNaGroupSteps;
  const int nclear = (int)((kNaCtrBytes + kNaWordBytes) / 16);
  hipLaunchKernelGGL(noalloc_clear, dim3((nclear + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     reinterpret_cast<uint4*>(d->base), nclear);
  if (hipGetLastError() != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  if (launch_ring_bulk(a, kAllReduce, dtype, op, s) != hipSuccess) return RINGSIM_UNHANDLED_DEVICE_ERROR;
  return RINGSIM_SUCCESS;
}

}  // extern "C"
