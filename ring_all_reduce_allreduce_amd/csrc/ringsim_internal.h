// ringsim_internal.h -- structures shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ringsim.h"

namespace ringsim {

constexpr int kThreads = 256;         // threads per workgroup (4 wave64)
constexpr int kUnroll = 8;            // 16-byte vectors in flight per thread
constexpr int kDefaultSlotBytes = kThreads * 16 * kUnroll;  // 32 KiB: one pass per slot
constexpr int kDefaultSlots = 8;      // FIFO depth (NCCL_STEPS)
constexpr int kFlagLinesPerThread = 4;  // flag-packed: 16-byte lines per thread per slot
constexpr int kFlagSlotBytes = kThreads * kFlagLinesPerThread * 16;  // 16 KiB (8 KiB payload)
constexpr int kFlagSlots = 16;
constexpr int kFlagHeadEvery = kFlagSlots / 2;  // line protocols publish head every this many steps
// Slots one stage of a line-protocol workgroup moves before the next stage
// runs: it must fit in the FIFO part that is always free while both
// neighbours sit in stage 0 (the rest may hold drained but unpublished steps).
constexpr int kLineGroupSteps = kFlagSlots - kFlagHeadEvery;
// Line launches split each (rank, channel) over 1, 2, 4 or 8 workgroups;
// each count has a FIFO array of its own, kFlagSlots slots of kFlagSlotBytes
// per workgroup.
constexpr int kLineWpcLevels = 4;
constexpr int kMaxLineWpc = 1 << (kLineWpcLevels - 1);
// Bytes of the FIFO array of one workgroup count, per (rank, channel).
__host__ __device__ constexpr int64_t line_level_bytes(int wpc) { return (int64_t)wpc * kFlagSlots * kFlagSlotBytes; }

// Line formats of the flag-packed protocols (16 bytes per line).
enum LineProto : int { kLineFlag = 0, kLineWide = 1 };

// Step counters of one FIFO (sender -> receiver, pipeline). The producer owns
// `tail` (slots filled), the consumer owns `head` (slots drained). Each sits
// in its own 128-byte line so that the two sides never share a cache line
// ("NCCL" book, s. 2.1 cache-line padding; s. 2.4 ncclSendMem/ncclRecvMem).
struct alignas(256) FifoCtr {
  uint64_t tail;
  char pad0[120];
  uint64_t head;
  char pad1[120];
};
static_assert(sizeof(FifoCtr) == 256, "FifoCtr layout");

enum Mode : int { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2 };

// Compile-time variants of the bulk kernel: the plain one; one that walks
// each loop in step groups of RingArgs::group slots (all-reduce only, for the
// allocation-free entry point's small FIFO); one that writes and checks the
// debug FIFO records. Kept apart because even a never-taken runtime branch for
// either feature cost the plain kernel 0.1-0.45 us per hop on MI355X.
enum BulkVariant : int { kBulkPlain = 0, kBulkGrouped = 1, kBulkEcho = 2 };

// Error codes a kernel leaves in the host-visible error word.
enum KernelError : uint32_t { kErrNone = 0, kErrTimeout = 1, kErrAborted = 2, kErrFlagSpan = 3, kErrFifoEcho = 4 };

// Debug FIFO integrity record of one bulk slot ("NCCL" book, s. 2.4: each
// FIFO step carries its size and offset beside the data): the producer writes
// the absolute step and the payload bytes of the step it put in the slot; the
// consumer, once the tail says the step is there, checks both.
struct alignas(16) FifoEcho {
  uint64_t step;
  uint32_t bytes;
  uint32_t pad;
};

// Flag span of the line and tree FIFOs. Their flags are the low 32 bits of
// (step + 1), so a line left from step s would match step s + 2^32, and a
// zeroed line matches step 2^32 - 1. The host zeroes a communicator's line
// (or tree) FIFOs and counters before any of its calls could take a counter
// past kFlagSpanGuard; a kernel that leaves a counter above it (only
// launches the host does not see, graph replays, can get there) records
// kErrFlagSpan, its own results still exact (a call moves fewer than 2^31
// steps, so its counters stay below 2^32 - 1).
constexpr uint64_t kFlagSpanGuard = 1ull << 31;

struct RingArgs {
  const char* send[RINGSIM_MAX_RANKS];
  char* recv[RINGSIM_MAX_RANKS];
  int64_t count;        // all-reduce: per rank; reduce-scatter: recvcount; all-gather: sendcount
  int64_t chunk;        // chunk elements (multiple of 16 bytes)
  int nranks;
  int nchannels;
  int wpc;              // workgroups (pipelines) per channel in this launch
  int pipe_stride;      // pipelines per rank in the counter array
  int pipe_mul;         // counter pipeline of (channel c, part w) = c * pipe_mul + w
  int fifo_stride;      // pipelines per rank in the FIFO array of this protocol
  int fifo_mul;         // FIFO pipeline of (channel c, part w) = c * fifo_mul + w
  int nslots;
  int slot_bytes;
  int vec_ok;           // every user buffer is 16-byte aligned
  char* fifo;           // FIFO slots: [rank][pipeline][slot][slot_bytes]
  FifoCtr* ctr;         // counters: [rank][pipeline]
  uint32_t* dev_abort;  // device word: set when any workgroup gives up
  const uint32_t* host_abort;  // host-mapped word set by ringsim_abort
  uint32_t* host_err;   // host-mapped error word
  uint64_t timeout_ticks;  // bound on one wait, in wall-clock ticks
  int skip_rank;        // testing knob: workgroups of this rank return at once (-1 = none)
  int lds_stage;        // bulk: stage each step's own operand in LDS (2 x slot_bytes dynamic LDS)
  int group;            // slot steps a stage moves before the next stage runs (0 = the whole stage)
  FifoEcho* echo;       // bulk debug: [rank][pipeline][slot] beside the FIFO, null = off
};

// Double-binary-tree all-reduce (flag-packed lines). Workgroup b of the grid
// is (rank, tree, channel, role) with b = ((rank * 2 + tree) * nchannels +
// channel) * 2 + role; role 0 reduces up the tree, role 1 broadcasts down.
// FIFO f = ((tree * ch_stride + channel) * nranks + node) * 2 + dir carries
// node -> parent (dir 0, "up") or parent -> node (dir 1, "down").
struct TreeArgs {
  const char* send[RINGSIM_MAX_RANKS];
  char* recv[RINGSIM_MAX_RANKS];
  int64_t count;        // elements per rank
  int nranks;
  int nchannels;        // tree channels of this launch (<= ch_stride)
  int ch_stride;        // tree channels in the FIFO and counter arrays
  int nslots;
  int slot_bytes;       // kTreeSlotBytes: one WIDE line per thread
  int head_every;       // consumers publish `head` every this many steps
  int vec_ok;
  int skip_rank;
  int8_t link[2][RINGSIM_MAX_RANKS][3];  // per tree and rank: parent, first child, second child
  char* fifo;           // [tree][channel][node][dir][slot][slot_bytes]
  FifoCtr* ctr;         // [tree][channel][node][dir]
  uint32_t* dev_abort;
  const uint32_t* host_abort;
  uint32_t* host_err;
  uint64_t timeout_ticks;
};

constexpr int kTreeSlots = 16;
// One 16-byte WIDE line per thread: every step of a tree workgroup is a
// single load, fold and store per thread, the shortest path from a child's
// flag to the parent's store.
constexpr int kTreeSlotBytes = kThreads * 16;

struct CopyArgs {
  const char* src[RINGSIM_MAX_RANKS];
  char* dst[RINGSIM_MAX_RANKS];
  int64_t block_bytes;  // bytes of one (source rank, destination rank) block
  int nranks;
  int transpose;        // 1: all-to-all; 0: rank r copies src[r] -> dst[r]
};

// Zeroes `bytes` (a multiple of 16) at 16-byte aligned device memory p with a
// kernel (no memset node, so that it can be captured) (copy.hip).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Kernel launchers (ring_bulk.hip; ring_lines_inst.hip, built once per line
// mode as _half, _one and _multi; tree.hip; copy.hip).
hipError_t launch_ring_bulk(const RingArgs& a, int mode, int dtype, int op, hipStream_t s);
// Line protocols: the _half variant when no step of the launch holds more
// than 128 lines, _one when none holds more than 256, else _multi.
hipError_t launch_ring_lines_half(const RingArgs& a, int line_proto, int mode, int dtype, int op, hipStream_t s);
hipError_t launch_ring_lines_one(const RingArgs& a, int line_proto, int mode, int dtype, int op, hipStream_t s);
hipError_t launch_ring_lines_multi(const RingArgs& a, int line_proto, int mode, int dtype, int op, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, hipStream_t s);
// Double-binary tree: one slot (one WIDE line per thread) per step.
hipError_t launch_tree_kernel(const TreeArgs& a, int dtype, int op, hipStream_t s);
// Max co-resident workgroups per CU over every instantiation of a kernel
// family (the bulk kernels launched with `lds_bytes` of dynamic LDS).
int tree_blocks_per_cu();
int bulk_blocks_per_cu(size_t lds_bytes);
int line_half_blocks_per_cu();
int line_one_blocks_per_cu();
int line_multi_blocks_per_cu();
// Largest bulk slot that is staged in LDS (two buffers must fit beside a
// second workgroup's on the 160 KiB of a CU).
constexpr int kMaxStagedSlotBytes = 64 * 1024;

inline int dtype_size(int dtype) {
  switch (dtype) {
    case RINGSIM_INT32: return 4;
    case RINGSIM_INT64: return 8;
    case RINGSIM_FLOAT32: return 4;
    case RINGSIM_BFLOAT16: return 2;
    default: return 0;
  }
}

}  // namespace ringsim
