/*
 * ringsim.h -- C ABI of libringsim: ring collectives over N simulated ranks
 * that live in the HBM of one MI355X (gfx950).
 *
 * Every simulated rank r owns a send buffer and a receive buffer in device
 * memory. Ranks exchange data only through FIFO staging slots that the
 * library keeps in HBM, one FIFO per (sender -> receiver, channel, workgroup
 * lane), guarded by step counters. The collectives follow the ring schedule
 * of NCCL as described in the "NCCL" book (aireadcode.com), ch. 2: s. 2.2
 * (channels split the data), s. 2.3 (RingARAlgorithm: loops, chunks and the
 * chunk visited at every stage), s. 2.4 (Simple and LL protocols, FIFO
 * head/tail counters). Semantics of the collectives follow the collectives
 * table of "AI Systems Performance Engineering (3)".
 *
 * Conventions shared by every call:
 *   - Pointers named *bufs are HOST arrays of length nranks holding DEVICE
 *     pointers (one per simulated rank). The caller owns all of them; the
 *     library never frees or retains them beyond the enqueued work.
 *   - Buffers of one call must not overlap across ranks, except that a rank's
 *     send and receive buffers may alias exactly as described per call.
 *   - Device buffers should be 16-byte aligned; buffers aligned only to their
 *     element size take a slower element-wise path. Misaligned elements are
 *     rejected with RINGSIM_INVALID_ARGUMENT.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream): they return once the work is enqueued, like ncclAllReduce as
 *     called from PyTorch's ProcessGroupNCCL ("NCCL 专家课程 29:
 *     ProcessGroupNCCL、Stream、Event 与 Work"). Calls on one communicator must
 *     be issued from one host thread and must be ordered on the device (one
 *     stream, or streams ordered by events): the FIFOs are shared state.
 *   - Calls may be captured into a HIP graph (stream capture): a call
 *     enqueues kernel launches only (no memset, copy, event or
 *     synchronization), and every kernel reads where its FIFOs stand from
 *     the communicator's persistent step counters when it starts, so graph
 *     launches and direct calls may follow one another in any order as long
 *     as they are ordered on the device. What ringsim_comm_query reports
 *     about the latest call describes the capture, not the launches. A graph
 *     holding a communicator's calls must not be launched after
 *     ringsim_comm_destroy.
 *   - count == 0 is a successful no-op; nranks == 1 is a local copy
 *     ("NCCL" book, enqueue chapter, taskAppend).
 *   - Every kernel polls an abort word and bounds each wait by a timeout; a
 *     call whose kernel gave up leaves the communicator in error state, which
 *     ringsim_get_async_error reports and every later call returns.
 */
#ifndef RINGSIM_H
#define RINGSIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RINGSIM_VERSION_MAJOR 0
#define RINGSIM_VERSION_MINOR 1
#define RINGSIM_MAX_RANKS 64
#define RINGSIM_MAX_CHANNELS 64
#define RINGSIM_MAX_WORKGROUPS_PER_CHANNEL 16

/* Opaque communicator. Allocated by ringsim_comm_init*, released by
 * ringsim_comm_destroy. Guarded by magic words at both ends ("NCCL" book,
 * s. 2.1, startMagic/endMagic) and a registry of live handles: a destroyed or
 * foreign handle yields RINGSIM_INVALID_USAGE. */
typedef struct ringsim_comm* ringsim_comm_t;

/* A hipStream_t passed as an untyped pointer so that this header needs no
 * HIP headers. */
typedef void* ringsim_stream_t;

/* Result codes. The numbering follows NCCL's public result names; "invalid
 * usage = 5" is the one value the pages print ("NCCL 专家课程 17", failure
 * experiments), the others are this library's reading. */
typedef enum {
  RINGSIM_SUCCESS = 0,
  RINGSIM_UNHANDLED_DEVICE_ERROR = 1, /* a HIP call failed */
  RINGSIM_SYSTEM_ERROR = 2,           /* host allocation failed */
  RINGSIM_INTERNAL_ERROR = 3,         /* a kernel timed out waiting on a peer */
  RINGSIM_INVALID_ARGUMENT = 4,       /* bad pointer, size, dtype, op, rank count */
  RINGSIM_INVALID_USAGE = 5,          /* bad / destroyed handle, impossible config */
  RINGSIM_IN_PROGRESS = 7,            /* reserved (NCCL's nonblocking state); no call returns it */
  RINGSIM_ABORTED = 8                 /* ringsim_abort was called */
} ringsim_result_t;

typedef enum {
  RINGSIM_INT32 = 0,
  RINGSIM_INT64 = 1,
  RINGSIM_FLOAT32 = 2,
  RINGSIM_BFLOAT16 = 3
} ringsim_datatype_t;

/* Reduction operators. Floating-point hops are rounded to the buffer type
 * (round-to-nearest-even, subnormals kept); bf16 hops compute in fp32 and
 * round once to bf16. max/min order -0 below +0. Integers wrap. */
typedef enum {
  RINGSIM_SUM = 0,
  RINGSIM_PROD = 1,
  RINGSIM_MAX = 2,
  RINGSIM_MIN = 3
} ringsim_redop_t;

/* Protocols ("NCCL" book, s. 2.4; ch. 5 for their costs): BULK keeps
 * readiness in separate step counters (Simple). FLAG packs a 4-byte flag with
 * every 4 bytes of payload, so the receiver polls the data itself (LL: half
 * of every line is payload). WIDE packs one 4-byte flag with 12 bytes of
 * payload in each 16-byte line (8 bytes for int64), written and read as one
 * 128-bit access: the MI355X counterpart of LL128, for medium messages.
 * WIDE (and the tree, which moves WIDE lines) rely on one lane's naturally
 * aligned 16-byte store and load being delivered whole, which the GPU does
 * but AMD does not document as a guarantee; FLAG relies only on aligned
 * 8-byte accesses being single-copy atomic. A soak test checks WIDE lines on
 * every run; proto = FLAG with algo = RING avoids them altogether.
 * FLAG and WIDE launches split every (rank, channel) over 1, 2, 4 or 8
 * workgroups, chosen per call (line_workgroups_per_channel caps it).
 * AUTO picks the protocol with the lowest predicted time
 * (ringsim_debug_model), or FLAG below flag_threshold_bytes per rank and
 * BULK above it when a threshold is configured. Every protocol walks the
 * same chunks (FLAG and WIDE walk each loop in groups of 8 slot steps so that
 * their FIFO never limits the chunk size), so results never depend on the
 * protocol. */
typedef enum {
  RINGSIM_PROTO_AUTO = 0,
  RINGSIM_PROTO_BULK = 1,
  RINGSIM_PROTO_FLAG = 2,
  RINGSIM_PROTO_WIDE = 3
} ringsim_proto_t;

/* All-reduce algorithms. RING is the ring schedule above. TREE is the double
 * binary tree ("NCCL" book, ch. 4, ncclGetBtree / ncclGetDtree; ch. 5,
 * tree.cc: all-reduce only): two binary trees over the ranks, the second the
 * mirror (even N) or the shift by one rank (odd N) of the first, each
 * reducing one half of the buffer up to its root and broadcasting the result
 * back down. Tree 1 takes elements [h, count) with
 * h = min(count, alignUp(ceil(count/2), 16/elemsize)); a rank folds its own
 * data, then its first child's partial, then its second child's. The tree
 * moves WIDE lines (12 payload bytes and the flag in one 16-byte line, 8
 * payload bytes for int64), one line per thread and FIFO step, so a step
 * carries 3 KiB (2 KiB for int64). Each half is split over channels of one
 * step each, as many as allow one, or two, tree workgroups per compute unit
 * (4 x N x channels <= CUs, or 2 x CUs), whichever the cost model predicts
 * faster; longer channels pipeline step by step. The tree
 * needs 2*log2(N) dependent hops instead of the ring's 2(N-1). AUTO takes
 * the tree only where the fold order cannot change a result bit (integer
 * types, and max/min of any type) and the cost model predicts it faster;
 * with proto = BULK it always takes the ring. The algorithm applies to
 * ringsim_allreduce only. */
typedef enum {
  RINGSIM_ALGO_AUTO = 0,
  RINGSIM_ALGO_RING = 1,
  RINGSIM_ALGO_TREE = 2
} ringsim_algo_t;

typedef enum {
  RINGSIM_COLL_ALLREDUCE = 0,
  RINGSIM_COLL_REDUCE_SCATTER = 1,
  RINGSIM_COLL_ALL_GATHER = 2,
  RINGSIM_COLL_ALLTOALL = 3
} ringsim_coll_t;

/* Tunables; zero fields take the default. */
typedef struct {
  size_t chunk_bytes;          /* ring chunk per channel; default 524288; multiple of 16 */
  int workgroups_per_channel;  /* BULK: workgroups per (rank, channel); default 0 = the most the CU count
                                  suggests (two per CU), of which a call with short stages takes fewer
                                  (about one per 4 KiB of a channel's stage, at least two, channels x
                                  workgroups a multiple of 8); a configured count is used by every
                                  call; env RINGSIM_WPC */
  size_t slot_bytes;           /* bulk FIFO slot; default 32768; multiple of 4096 */
  int nslots;                  /* bulk FIFO depth; default 8 (NCCL_STEPS) */
  int timeout_ms;              /* bound on any single wait; default 10000, env RINGSIM_TIMEOUT_MS */
  size_t flag_threshold_bytes; /* AUTO: FLAG below this many bytes per rank; default 0 = cost model */
  int algo;                    /* ringsim_algo_t for all-reduces; default AUTO, env RINGSIM_ALGO=ring|tree|auto */
  int line_workgroups_per_channel; /* FLAG/WIDE: most workgroups per (rank, channel) of a launch: 1, 2, 4
                                      or 8 (fewer where the device cannot hold them all); default 0 = per
                                      call, the count the cost model predicts fastest with at most two
                                      workgroups per compute unit; env RINGSIM_LINE_WPC */
} ringsim_config_t;

/* Read-only description of a communicator. */
typedef struct {
  int nranks;
  int nchannels;
  int proto;
  int workgroups_per_channel;  /* BULK: the most a call takes */
  int nslots;
  int device;
  size_t chunk_bytes;
  size_t slot_bytes;
  size_t flag_threshold_bytes;
  size_t fifo_bytes;           /* bulk FIFO bytes in HBM */
  size_t flag_fifo_bytes;      /* flag-packed FIFO bytes in HBM (FLAG and WIDE share it; one array per
                                  line workgroup count 1, 2, 4, 8 up to the largest this device takes) */
  int max_resident_workgroups; /* co-resident workgroups the device can hold */
  int compute_units;
  uint64_t calls;              /* collective calls enqueued so far */
  int last_proto;              /* protocol of the latest ring call: RINGSIM_PROTO_BULK/FLAG/WIDE, 0 if none */
  int algo;                    /* configured all-reduce algorithm (ringsim_algo_t) */
  int tree_channels;           /* channels per tree in the tree FIFOs (up to 2 x nchannels); a call takes at most 2 CUs / (4N) */
  size_t tree_fifo_bytes;      /* double-tree FIFO bytes in HBM */
  int last_algo;               /* algorithm of the latest all-reduce: RINGSIM_ALGO_RING/TREE, 0 if none */
  int line_max_workgroups_per_channel; /* most workgroups per channel a FLAG/WIDE launch may take */
  int last_workgroups_per_channel;     /* workgroups per channel of the latest ring call, 0 if none */
  int last_tree_channels;              /* channels per tree of the latest all-reduce, 0 if it ran the ring */
  uint64_t line_fifo_resets;           /* times the FLAG/WIDE FIFOs and counters were zeroed (flag span) */
  uint64_t tree_fifo_resets;           /* the same for the tree FIFOs */
  int last_group_steps;                /* BULK all-reduce: slot steps a stage of the latest ring call moved
                                          before the next stage ran (0 = whole stages) */
} ringsim_comm_info_t;

/* Fills *cfg with the defaults ("NCCL" book, ch. 3, s. 3.5: every tunable is
 * a named parameter with a default that an environment variable overrides,
 * read once). Environment overrides, read by this call:
 * RINGSIM_CHUNK_BYTES, RINGSIM_WPC, RINGSIM_SLOT_BYTES, RINGSIM_NSLOTS,
 * RINGSIM_TIMEOUT_MS, RINGSIM_FLAG_THRESHOLD, RINGSIM_ALGO, RINGSIM_LINE_WPC;
 * RINGSIM_DEBUG=WARN|INFO logs to stderr. RINGSIM_DEBUG_FIFO=1 (read at comm
 * init) keeps a (step, bytes) record beside every bulk FIFO slot, written by
 * its producer and checked by its consumer ("NCCL" book, s. 2.4: the size and
 * offset each FIFO step carries); a mismatch leaves RINGSIM_INTERNAL_ERROR.
 * RINGSIM_ROCTX=1 (read at the first call) puts a roctx range named after
 * the call around every communicator and collective call (not the
 * allocation-free one), loading the roctx library at run time ("NCCL" book,
 * ch. 3, s. 3.1: an NVTX mark at every API entry); rocprofv3 --marker-trace
 * shows them beside the kernels. RINGSIM_LDS_STAGE=0 (read at comm init)
 * makes bulk steps load the rank's own operand beside the FIFO operand in
 * every call; by default calls above 512 KiB per rank stage it in LDS one
 * step ahead.
 * Testing only: RINGSIM_DEBUG_SKIP_RANK=r (read at comm init) makes
 * the workgroups of simulated rank r return at once, so that the bounded
 * waits of its neighbours expire and the failure path can be exercised. */
ringsim_result_t ringsim_config_default(ringsim_config_t* cfg);

/* Creates a communicator of `nranks` (1..RINGSIM_MAX_RANKS) simulated ranks
 * on the current HIP device, with `nchannels` (1..RINGSIM_MAX_CHANNELS) ring
 * channels and protocol `proto` (ringsim_proto_t). Follows "NCCL" book,
 * ch. 3, s. 3.1 (ncclCommInitRank: validate the rank count and arguments,
 * then allocate the communicator and its abort flag with a device-visible
 * copy) and s. 3.3 (commAlloc: the communicator's memory is allocated once,
 * at init). Ring order is r -> (r + 1) mod nranks. Allocates the FIFOs,
 * counters and the host-mapped abort and error words once; synchronous. On error *comm is left untouched: bad arguments give
 * RINGSIM_INVALID_ARGUMENT, a configuration whose workgroups cannot all be
 * resident at once gives RINGSIM_INVALID_USAGE, a failed HIP allocation
 * RINGSIM_UNHANDLED_DEVICE_ERROR. */
ringsim_result_t ringsim_comm_init(ringsim_comm_t* comm, int nranks, int nchannels, int proto);

/* As ringsim_comm_init with explicit tunables (cfg may be NULL), as
 * ncclCommInitRankConfig takes a config next to the plain call ("NCCL" book,
 * ch. 3, s. 3.1). Zero fields of *cfg take ringsim_config_default's value;
 * *cfg is read during the call only and stays the caller's. */
ringsim_result_t ringsim_comm_init_config(ringsim_comm_t* comm, int nranks, int nchannels, int proto,
                                          const ringsim_config_t* cfg);

/* Waits for all work on the device (hipDeviceSynchronize: the streams the
 * communicator was used on may no longer exist), frees its device memory
 * and invalidates the handle: its magic words are overwritten and it leaves
 * the registry of live handles, so a later call with it returns
 * RINGSIM_INVALID_USAGE instead of reading freed memory ("NCCL" book, ch. 2,
 * s. 2.1: the use-after-destroy pitfall that startMagic/endMagic catch).
 * Not to be called while a stream that holds its calls is being captured. */
ringsim_result_t ringsim_comm_destroy(ringsim_comm_t comm);

/* Copies the communicator's shape and the choices of its latest call into
 * *info (caller-owned host memory). The fields mirror what ncclComm records
 * per communicator ("NCCL" book, ch. 2, s. 2.1: rank count, channels, buffer
 * sizes; s. 2.2: channel count). Host only; RINGSIM_INVALID_ARGUMENT for a
 * NULL info, RINGSIM_INVALID_USAGE for a bad handle. */
ringsim_result_t ringsim_comm_query(ringsim_comm_t comm, ringsim_comm_info_t* info);

/* Ring all-reduce ("AI Systems Performance Engineering (3)", collectives
 * table: every rank receives the reduction; equal to reduce-scatter followed
 * by all-gather). count elements per rank; recvbufs[r] may equal
 * sendbufs[r] (in place). Chunk k of every loop is folded in rank order
 * k+1, k+2, ..., k ("NCCL" book, s. 2.3, chunk id per stage). */
ringsim_result_t ringsim_allreduce(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                   size_t count, int dtype, int op, ringsim_stream_t stream);

/* Ring reduce-scatter ("AI Systems Performance Engineering (3)", collectives
 * table: each rank keeps one block of the reduction; "In-Network SHARP
 * Aggregation": a rank receives (n-1)/n of the buffer). sendbufs[r] holds
 * nranks * recvcount elements; recvbufs[r] receives the reduced block r,
 * folded in rank order r+1, ..., r. recvbufs[r] may equal
 * sendbufs[r] + r * recvcount elements (in place). */
ringsim_result_t ringsim_reduce_scatter(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                        size_t recvcount, int dtype, int op, ringsim_stream_t stream);

/* Ring all-gather ("AI Systems Performance Engineering (3)", collectives
 * table; slice order of "NCCL 专家课程 17", section
 * "Bootstrap Ring 与 AllGather"). sendbufs[r] holds sendcount elements;
 * block b of recvbufs[r] (nranks * sendcount elements) receives sendbufs[b].
 * sendbufs[r] may equal recvbufs[r] + r * sendcount elements (in place). */
ringsim_result_t ringsim_all_gather(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                    size_t sendcount, int dtype, ringsim_stream_t stream);

/* All-to-all ("AI Systems Performance Engineering (3)", collectives table:
 * chunk j of rank i goes to rank j). Both buffers of
 * a rank hold nranks * count elements; block i of recvbufs[j] receives block
 * j of sendbufs[i]. Send and receive buffers must not overlap. */
ringsim_result_t ringsim_alltoall(ringsim_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                                  size_t count, int dtype, ringsim_stream_t stream);

/* Reports the communicator's asynchronous error state ("NCCL" book, ch. 2,
 * s. 2.1: the asyncResult field of ncclComm; s. 2.6: asyncResult turns to
 * success when every channel is done, and ncclCommGetAsyncError reads it):
 * RINGSIM_SUCCESS while no error is known, else the error a kernel (a wait
 * that expired: RINGSIM_INTERNAL_ERROR) or ringsim_abort (RINGSIM_ABORTED)
 * left behind. It says nothing about whether enqueued work has finished:
 * that is for the caller's stream or events to tell, as PyTorch's
 * ProcessGroupNCCL records an event after each collective on its stream
 * ("NCCL 专家课程 29: ProcessGroupNCCL、Stream、Event 与 Work"). The library
 * keeps no stream handle. Host only, never blocks. */
ringsim_result_t ringsim_get_async_error(ringsim_comm_t comm, ringsim_result_t* async_error);

/* Raises the abort word that every spinning kernel polls ("NCCL" book, ch. 3,
 * s. 3.1: the host abort flag and its device-visible copy; s. 3.2: every
 * blocking loop checks the abort flag every so many spins); running kernels
 * stop waiting and finish, and every later call returns RINGSIM_ABORTED.
 * Host only, never blocks. */
ringsim_result_t ringsim_abort(ringsim_comm_t comm);

/* Static text for a result code (the result names of "NCCL 专家课程 17:
 * Bootstrap 与 Communicator 初始化状态机", failure experiments). The string is
 * owned by the library and never freed. */
const char* ringsim_get_error_string(ringsim_result_t result);

/* Host-only cost model behind AUTO ("NCCL" book, ch. 5, ring.cc: latency =
 * hops x per-hop latency, bandwidth term = bytes moved / achievable bandwidth,
 * the FIFO bytes scaled by each line format: x2 for FLAG, x4/3 for WIDE),
 * with constants measured on MI355X. BULK: hops and bytes; FLAG and WIDE:
 * the slot steps of one workgroup (each costing more the more lines it
 * holds) and the line bytes, at the workgroup count per channel (1, 2, 4 or
 * 8, at most two workgroups per compute unit of a 256-CU device) that the
 * model finds fastest. Writes the predicted microseconds of one call of
 * `coll` (RINGSIM_COLL_ALLREDUCE, _REDUCE_SCATTER or _ALL_GATHER) with
 * `bytes_per_rank` bytes per rank (all-reduce buffer, reduce-scatter input,
 * all-gather output) on each protocol. Touches no device. */
ringsim_result_t ringsim_debug_model(int coll, int nranks, int nchannels, size_t bytes_per_rank, double* us_bulk,
                                     double* us_flag, double* us_wide);

/* Host-only tree shape. Writes links[6] = (parent, first child, second
 * child) of `rank` in tree 0, then the same in tree 1 (-1 = none), for a
 * double binary tree over `nranks` ranks ("NCCL" book, ch. 4, ncclGetBtree
 * and ncclGetDtree). links is caller-owned host memory of 6 ints. */
ringsim_result_t ringsim_debug_tree(int nranks, int rank, int* links);

/* Host-only cost model ("NCCL" book, ch. 5, the tree latency and bandwidth
 * terms) of the tree all-reduce with `tree_channels` channels
 * per tree and `bytes_per_rank` bytes per rank of a 4-byte type on a 256-CU
 * device: base + 2 x tree depth x the per-hop latency of one step (one WIDE
 * line per thread) + one further step per further 3 KiB of a channel, hops
 * and steps growing with the tree's workgroups per compute unit beyond one.
 * Writes the predicted microseconds. */
ringsim_result_t ringsim_debug_tree_model(int nranks, int tree_channels, size_t bytes_per_rank, double* us);

/* Host-only bound behind the flag span of the line protocols and the tree.
 * FLAG and WIDE lines, and the tree's lines, carry the low 32 bits of
 * (step + 1) as their flag ("NCCL" book, s. 2.4: LL and LL128 put a flag
 * equal to the step into every line, so the receiver polls the data
 * itself); a line left from step s would match step s + 2^32, and a zeroed
 * line step 2^32 - 1. Each communicator therefore counts, per family (ring
 * lines, tree), an upper bound of the steps any FIFO has moved since its
 * FIFOs and counters were last zeroed, and zeroes them (a kernel on the
 * call's stream) before a call that could take a counter past 2^31; a call
 * whose own bound exceeds 2^31 returns RINGSIM_INVALID_USAGE. Calls captured
 * into a graph are not counted, and a kernel that leaves a counter past 2^31
 * (only graph replays can take it there) leaves RINGSIM_INTERNAL_ERROR
 * (RINGSIM_DEBUG_FLAG_SPAN=n lowers the bound that triggers the zeroing to n
 * steps, for tests). Writes to *steps the bound for one call: `algo`
 * RINGSIM_ALGO_RING with `proto` RINGSIM_PROTO_FLAG or _WIDE and `coll`
 * RINGSIM_COLL_ALLREDUCE, _REDUCE_SCATTER or _ALL_GATHER (count as
 * ringsim_debug_plan), or RINGSIM_ALGO_TREE for an all-reduce of `count`
 * elements per rank. Touches no device. */
ringsim_result_t ringsim_debug_flag_steps(int coll, int algo, int nranks, int nchannels, size_t chunk_bytes,
                                         size_t count, int dtype, int proto, uint64_t* steps);

/* Host-only view of the partition used by the kernels ("NCCL" book, ch. 2,
 * s. 2.2: a channel owns count / nChannels of the data; s. 2.3: a loop of
 * nranks chunks, the ragged last loop's chunk size and the chunk visited at
 * every stage). For `coll`
 * (ringsim_coll_t), writes rows of 5 int64 values
 *   (channel, loop, chunk, begin, end)
 * with [begin, end) absolute element indices: for the all-reduce, chunk k of
 * every loop of every channel of a count-element buffer; for reduce-scatter
 * and all-gather (chunk = -1), the element range of every loop of every
 * channel inside one rank block of `count` elements. Writes at most max_rows
 * rows to `rows` (host memory, may be NULL to query) and the total number to
 * *nrows. Touches no device. */
ringsim_result_t ringsim_debug_plan(int coll, size_t count, int nranks, int nchannels, size_t chunk_bytes,
                                    int dtype, int64_t* rows, size_t max_rows, size_t* nrows);

/* Allocation-free ring all-reduce, for callers that cannot allocate device
 * memory at call time (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Computes exactly what ringsim_allreduce
 * computes on a communicator of `nranks` ranks and `nchannels` channels with
 * the ring algorithm (the same chunks and fold order, so equal results bit
 * for bit), with the bulk protocol, but needs no communicator: its FIFO
 * slots, step counters and error words live in a library-owned scratch
 * array in device memory, one copy per GPU (32 MiB plus 32 KiB, held until
 * the process ends), set up on the first call on each device. Arguments as
 * ringsim_allreduce; the caller passes the input and output buffers.
 * Limits: nranks * nchannels <= 128 (larger shapes return
 * RINGSIM_INVALID_ARGUMENT and log a warning with RINGSIM_DEBUG=WARN);
 * chunk size from RINGSIM_CHUNK_BYTES as ringsim_config_default. Every call
 * on one GPU shares that GPU's scratch and starts by clearing its counters
 * with a small kernel: calls that may overlap on one GPU (unordered streams,
 * other threads) race and give undefined results; order them on the device.
 * No abort and no asynchronous error report: a wait that exceeds the
 * RINGSIM_TIMEOUT_MS bound gives up, leaves the output undefined and is not
 * reported (ringsim_allreduce on a communicator reports it). Calls no
 * hipMalloc, hipFree or other allocating routine. */
ringsim_result_t ringsim_allreduce_noalloc(int nranks, int nchannels, const void* const* sendbufs,
                                           void* const* recvbufs, size_t count, int dtype, int op,
                                           ringsim_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RINGSIM_H */
