/*
 * ccl_sim.h — ReduceScatter, AllGather and AllReduce over N virtual ranks
 * whose buffers all live in one AMD MI355X (gfx950) GPU's HBM.
 *
 * One call covers all N ranks, the way a single host process drives every
 * rank with grouped calls in the native probe of "NCCL 专家课程 07：AllReduce
 * 等价分解、显存生命周期与 Kernel 证据" (blog.cptz.space), §Nsight 实验如何避免
 * 框架噪声.  The
 * "links" between ranks are HBM reads and writes; there is no second GPU.
 *
 * Pages cited below:
 *   [DECOMP]  "NCCL 专家课程 07：AllReduce 等价分解、显存生命周期与 Kernel 证据"
 *             (blog.cptz.space/posts/nccl-collective-decomposition/)
 *   [WHY-EQ]  "为什么说 AllReduce = ReduceScatter + AllGather？——结合 NCCL
 *             Ring AllReduce" (loosp.cn)
 *   [RING]    "Ring AllReduce 核心流程：梯度是怎么聚合的" (llmnex.top)
 *   [RS-PAGE] "ReduceScatter" (tier6-model.pages.dev, 集合通信)
 *   [PRIMS]   "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring
 *             all-reduce" (arganzheng.life)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Buffers.   `sendbufs` and `recvbufs` are HOST arrays of `nranks` DEVICE
 *            pointers; element r belongs to virtual rank r.  The caller
 *            allocates and owns every device buffer, including `workspace`.
 *            The library keeps no pointer after a call returns and allocates
 *            no device memory.  The kernels run on the calling thread's
 *            current HIP device, so every rank buffer and the workspace must
 *            be memory of that device (the library cannot check this: it
 *            sees plain addresses).
 * Layout.    Every rank buffer is a contiguous 1-D array of `dtype`
 *            elements.  Element i of a full buffer belongs to shard i / q
 *            (rank-major sharding, [DECOMP] §数学证明).
 * Alignment. Pointers must be aligned to the element size.  16-byte aligned
 *            pointers and shard sizes with q·sizeof(dtype) a multiple of 16
 *            take the fastest path; any other layout is handled, slower.
 * Streams.   Work is enqueued on `stream` (a hipStream_t; NULL is the null
 *            stream) and the call returns without waiting.  Buffers must stay
 *            alive until that stream work completes ([DECOMP] §显存实验必须区分
 *            steady 与 peak: freeing a buffer before the collective has read
 *            it is unsafe).
 * Workspace. Device scratch of at least ccl_sim_workspace_size(...) bytes,
 *            256-byte aligned, owned by the caller.  It carries the device
 *            copy of the pointer tables when nranks > 64, the partial sums
 *            the ring schedules pass between ranks, the per-rank halves of
 *            the recursive halving schedule, and the control block (arrival
 *            counters, step flags and an abort word) of the persistent
 *            ring.  Calls
 *            that share a workspace must be ordered on one stream.  NULL is
 *            allowed when the required size is 0.
 * Errors.    Every argument is validated before any HIP call; on any error
 *            nothing is enqueued and the output buffers are untouched (as the
 *            capacity check of [DECOMP] §Contract 实验四 rejects a
 *            non-divisible ReduceScatter on every rank before any kernel).
 *            ccl_sim_last_error() returns a message naming the failed check.
 *            A HIP failure while enqueueing returns CCL_SIM_HIP_ERROR.
 *            Count 0 is a successful no-op.
 * Overlap.   Output buffers must not overlap each other.  An output may
 *            overlap an input only in the in-place forms:
 *              AllReduce      recvbufs[r] == sendbufs[r]            ([DECOMP]
 *                             §源码五: the AllReduce tensor is both input and
 *                             output);
 *              AllGather      sendbufs[r] == recvbufs[r] + r·sendcount
 *                             ([DECOMP] §源码四, the in-place AllGather test);
 *              ReduceScatter  recvbufs[r] == sendbufs[r] + r·recvcount (the
 *                             dual of the AllGather form).
 *            Inputs may alias each other (they are only read).
 * Order.     Integer SUM / PROD wrap modulo 2^32 or 2^64; float32 SUM / PROD
 *            results depend on the combining order ([DECOMP] §等价成立的条件,
 *            condition five).  CCL_SIM_DIRECT folds ranks in ascending order
 *            0, 1, ..., N-1.  The ring schedules fold chunk c in the ring's
 *            order x^(c), x^(c+1), ..., x^(c-1).  Within one call all N
 *            outputs are bit-identical.  bf16 is accumulated in float32 and
 *            rounded to nearest even once, when a result is stored.
 *            MAX / MIN keep the running partial on ties.
 *            CCL_SIM_RECURSIVE reduces each block as the butterfly tree of
 *            its halving steps.
 * Threads.   The library holds no mutable global state except a cached
 *            per-device compute-unit count, a thread-local error message
 *            and the per-device scratch of ccl_sim_allreduce_noalloc; calls
 *            with distinct workspaces may run concurrently.
 * Debug.     With the environment variable CCL_SIM_DEBUG=1 (read on every
 *            call) each call logs its launch plan to stderr, and before a
 *            ring or recursive call that keeps partials in the workspace
 *            the library fills their part of it with all-ones bits (a NaN
 *            as float32, -1 as an integer) on the call's stream, so that a
 *            partial read before it is written shows in the result.
 */
#ifndef CCL_SIM_H
#define CCL_SIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CCL_SIM_VERSION 100      /* 1.0.0 */
#define CCL_SIM_MAX_RANKS 1024
#define CCL_SIM_INLINE_RANKS 64  /* up to this many ranks need no pointer table in the workspace */
/* Size of the library's own device scratch used by ccl_sim_allreduce_noalloc
 * (64 MiB per GPU the library runs on). */
#define CCL_SIM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum {
  CCL_SIM_SUCCESS = 0,
  CCL_SIM_INVALID_ARGUMENT = 1,      /* a check on counts, pointers, enums or overlap failed */
  CCL_SIM_UNSUPPORTED = 2,           /* valid request this device cannot run (e.g. no co-resident grid) */
  CCL_SIM_INSUFFICIENT_WORKSPACE = 3,/* workspace NULL or smaller than ccl_sim_workspace_size() */
  CCL_SIM_HIP_ERROR = 4,             /* a HIP runtime call failed while enqueueing */
  CCL_SIM_CAPACITY_MISMATCH = 5      /* ReduceScatter sendcount != nranks * recvcount */
} ccl_sim_result_t;

typedef enum {
  CCL_SIM_INT32 = 0,
  CCL_SIM_INT64 = 1,
  CCL_SIM_FLOAT32 = 2,
  CCL_SIM_BFLOAT16 = 3
} ccl_sim_dtype_t;

/* The reduction operators of [PRIMS] §二.1.  AVG combines as SUM and divides
 * the completed result by nranks once, when it is stored (the postOp of
 * [DECOMP] §源码三): one correctly rounded float32 division for float32 and
 * bf16, integer division truncating toward zero for int32 / int64.  Its
 * padding identity is 0. */
typedef enum {
  CCL_SIM_SUM = 0,
  CCL_SIM_PROD = 1,
  CCL_SIM_MAX = 2,
  CCL_SIM_MIN = 3,
  CCL_SIM_AVG = 4
} ccl_sim_op_t;

typedef enum {
  /* Read every input once: one fused kernel per collective. */
  CCL_SIM_DIRECT = 0,
  /* The ring of [RING] §1 / [PRIMS] §五: one kernel launch per ring step. */
  CCL_SIM_RING_STEPWISE = 1,
  /* The same ring steps inside one cooperative kernel.  Steps are ordered
   * in one of two ways, with the same transfers, combining order and
   * results:
   *   - a grid-wide barrier between steps;
   *   - per-workgroup step flags: before a step, each workgroup waits only
   *     for the workgroups that hold the upstream tiles of its own (the
   *     chunk it receives from rank r-1), and its partials are keyed by
   *     chunk as in CCL_SIM_RING_CHAINED.
   * By default steps of up to 2^26 elements (N·q) take the flags and larger
   * ones the barrier; the environment variable CCL_SIM_PERSISTENT_SYNC
   * (grid, flags or auto) overrides this, and any other value makes the
   * call return CCL_SIM_INVALID_ARGUMENT before anything is enqueued.
   * CCL_SIM_UNSUPPORTED when the device cannot keep the grid resident, or
   * when the runtime refuses the cooperative launch (ROCm does, for
   * instance, while another process on the same GPU holds its cooperative
   * launch resources); the other schedules are unaffected.  The grid is
   * one workgroup per CU unless the environment variable
   * CCL_SIM_PERSISTENT_BLOCKS_PER_CU asks for 1 to 4; any other value
   * (negative, or above 4, where co-residency is not established) makes
   * the call return CCL_SIM_UNSUPPORTED before anything is enqueued. */
  CCL_SIM_RING_PERSISTENT = 2,
  /* Recursive-halving ReduceScatter and recursive-doubling AllGather
   * ([RS-PAGE] §Recursive Halving ReduceScatter): log2 N steps per phase, one
   * launch per step; nranks must be a power of two (else
   * CCL_SIM_UNSUPPORTED).  Block b is reduced as a butterfly: at halving
   * step j ranks i and i XOR N/2^j combine (lower rank's partial) ⊕ (upper
   * rank's partial). */
  CCL_SIM_RECURSIVE = 3,
  /* The ring of CCL_SIM_RING_STEPWISE, each chunk's 2(N-1) steps chained in
   * one launch: a step of chunk c depends only on the step before it of the
   * same chunk (the recv-reduce-send hand-off between neighbouring ranks of
   * [RING] §1), so one workgroup follows a slice of chunk c through every
   * step, with no grid barrier and no relaunch between steps.  Same
   * routing, same combining order and same algorithmic bytes as the other
   * ring schedules, bit-identical results.  The partials live in a buffer
   * keyed by chunk (N·q accumulators), since chunks no longer move in step
   * lockstep. */
  CCL_SIM_RING_CHAINED = 4,
  /* The recursive halving / doubling of CCL_SIM_RECURSIVE in one launch.
   * Each position is reduced by its own butterfly over the ranks and
   * gathered by its own doubling tree, so one workgroup carries a slice of
   * block b through every halving and doubling step (all the ranks of a
   * step in turn), with no barrier and no relaunch.  Same pairs, combining
   * order and algorithmic bytes as CCL_SIM_RECURSIVE, bit-identical
   * results; nranks must be a power of two (else CCL_SIM_UNSUPPORTED). */
  CCL_SIM_RECURSIVE_CHAINED = 5
} ccl_sim_schedule_t;

typedef enum {
  CCL_SIM_COLL_REDUCE_SCATTER = 0,
  CCL_SIM_COLL_ALL_GATHER = 1,
  CCL_SIM_COLL_ALLREDUCE = 2
} ccl_sim_coll_t;

/* Same layout as hipStream_t; declared here so C callers need no HIP header. */
typedef struct ihipStream_t* ccl_sim_stream_t;

/*
 * ReduceScatter, rank-major ([DECOMP] §数学证明 ReduceScatter; [RS-PAGE]
 * §语义定义, equation rs-semantic-output):
 *     recvbufs[r][j] = ⊕_{s=0}^{N-1} sendbufs[s][r·recvcount + j],
 *     0 <= j < recvcount.
 * sendbufs[s] holds sendcount elements, recvbufs[r] receives recvcount.
 * The count rule is NCCL's ([DECOMP] §源码一): sendcount must equal
 * nranks·recvcount, else CCL_SIM_CAPACITY_MISMATCH and nothing is enqueued
 * ([DECOMP] §Contract 实验四).  A length that does not divide is padded first
 * with ccl_sim_pad_identity.
 * Ring schedules: N-1 steps; ring rank n ends holding chunk (n+1) mod N
 * ([PRIMS] §五.2), which is stored as recvbufs[(n+1) mod N], so the result
 * is rank-major for every schedule.
 */
ccl_sim_result_t ccl_sim_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                        size_t sendcount, size_t recvcount, ccl_sim_dtype_t dtype,
                                        ccl_sim_op_t op, ccl_sim_schedule_t schedule, void* workspace,
                                        size_t workspace_bytes, ccl_sim_stream_t stream);

/*
 * AllGather in source-rank order ([DECOMP] §数学证明 AllGather):
 *     recvbufs[r][s·sendcount + j] = sendbufs[s][j]   for every r,
 * keeping only the first recvcount elements of each output, so
 * recvcount < nranks·sendcount trims a padded result back to its logical
 * length ([DECOMP] §Contract 实验四).  recvcount > nranks·sendcount is
 * CCL_SIM_CAPACITY_MISMATCH.  Bit-exact copy for every dtype.
 * Ring schedules: rank r starts with shard r and N-1 recv-copy-send steps
 * follow ([PRIMS] §五.3, [WHY-EQ] §6).
 */
ccl_sim_result_t ccl_sim_all_gather(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                    size_t sendcount, size_t recvcount, ccl_sim_dtype_t dtype,
                                    ccl_sim_schedule_t schedule, void* workspace, size_t workspace_bytes,
                                    ccl_sim_stream_t stream);

/*
 * AllReduce ([DECOMP] §数学证明 Direct AllReduce):
 *     recvbufs[r][i] = ⊕_{s=0}^{N-1} sendbufs[s][i],  0 <= i < count,
 * identical for every r.  Any count is accepted: positions past count in
 * the last shard behave as the op's identity and are never stored (the
 * pad-and-trim of [DECOMP] condition three, done without materialising it).
 * CCL_SIM_DIRECT runs one fused kernel.  The ring schedules run the
 * 2(N-1) steps of [RING] §1, the ReduceScatter phase's last step writing
 * the completed chunk straight into the rank's output, which the AllGather
 * phase then forwards ([DECOMP] §源码三, the phase boundary fused in one
 * state machine).
 */
ccl_sim_result_t ccl_sim_allreduce(const void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                                   ccl_sim_dtype_t dtype, ccl_sim_op_t op, ccl_sim_schedule_t schedule,
                                   void* workspace, size_t workspace_bytes, ccl_sim_stream_t stream);

/*
 * ccl_sim_allreduce without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, semantics, kernels and results as ccl_sim_allreduce with the
 * same schedule; the workspace that call would need comes from a device
 * array owned by the library, CCL_SIM_NOALLOC_SCRATCH_BYTES on each GPU,
 * held from the first call on that GPU until the process ends.  The call
 * itself allocates nothing, on the device or the host.
 *
 * Limits and errors, all checked before anything is enqueued:
 *   - a call whose ccl_sim_workspace_size(CCL_SIM_COLL_ALLREDUCE, ...)
 *     exceeds CCL_SIM_NOALLOC_SCRATCH_BYTES returns
 *     CCL_SIM_INSUFFICIENT_WORKSPACE (for float32 ring AllReduce that is
 *     M of about 2^23 elements per rank; the direct schedule with at most
 *     64 ranks needs no scratch at any size);
 *   - CCL_SIM_RING_PERSISTENT returns CCL_SIM_UNSUPPORTED, since its abort
 *     word would live where the caller cannot query it;
 *   - everything else as for ccl_sim_allreduce.
 * The first call on each device reads the scratch's device address (one
 * hipGetSymbolAddress, which may load the library's code object): make it
 * outside graph capture.  Every call on one GPU uses that GPU's one
 * scratch, so calls that overlap in time on one GPU (on different streams,
 * or from different threads) race on it and give undefined results; calls
 * in stream order are safe.  Nothing in the scratch has to start at zero:
 * every partial and pointer table is written before it is read, within
 * the same call.
 */
ccl_sim_result_t ccl_sim_allreduce_noalloc(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                           size_t count, ccl_sim_dtype_t dtype, ccl_sim_op_t op,
                                           ccl_sim_schedule_t schedule, ccl_sim_stream_t stream);

/*
 * Identity padding ([DECOMP] §等价成立的条件, condition three):
 *     dsts[r][i] = srcs[r][i]     for i < count,
 *     dsts[r][i] = identity(op)   for count <= i < padded_count,
 * with identity 0 (SUM, AVG), 1 (PROD), -inf / INT_MIN (MAX), +inf /
 * INT_MAX (MIN) — never a mechanical zero.  srcs[r] == dsts[r] only fills the tail.
 * padded_count < count is CCL_SIM_INVALID_ARGUMENT.  No workspace needed.
 */
ccl_sim_result_t ccl_sim_pad_identity(const void* const* srcs, void* const* dsts, int nranks, size_t count,
                                      size_t padded_count, ccl_sim_dtype_t dtype, ccl_sim_op_t op,
                                      ccl_sim_stream_t stream);

/*
 * In the two queries below `count` is M, the logical per-rank length of the
 * full (unsharded) buffer: sendcount for ReduceScatter, recvcount for
 * AllGather, count for AllReduce.  q = ceil(M / N) is the shard length.
 *
 * Workspace bytes one call needs (0 when none, SIZE_MAX for invalid
 * arguments), each part rounded up to 256 bytes:
 *   - a control block of 17,024 bytes for the persistent ring (barrier
 *     counters, abort word, one step flag per workgroup);
 *   - two pointer tables of 8·N bytes each when nranks > 64;
 *   - the ring's double-buffered partials 2·N·q·a (a = accumulator size: 4
 *     for bf16, else the element size) for ring ReduceScatter and ring
 *     AllReduce with N >= 3; N·q·a, one partial per chunk, for the chained
 *     ring;
 *   - the recursive schedules' per-rank halves N·(N/2)·q·a for their
 *     ReduceScatter and AllReduce with N >= 4.
 * AllGather needs no partials under any schedule.
 */
size_t ccl_sim_workspace_size(ccl_sim_coll_t coll, int nranks, size_t count, ccl_sim_dtype_t dtype,
                              ccl_sim_schedule_t schedule);

/*
 * Algorithmic HBM bytes of one call: every element the schedule's data
 * movement must read or write, counted once per access (the numerator of
 * the effective bandwidth).  s = element size, a = accumulator size:
 *   DIRECT  ReduceScatter (N+1)·M·s    AllGather (N+1)·M·s    AllReduce 2N·M·s
 *   RECURSIVE (either driver)  halving step j: each position is reduced
 *           by N/2^j ranks, each reading two partials (the inputs at step
 *           1) and writing one (the output at the last step): 3(N-1)·M·s
 *           for 4- and 8-byte types; AllGather and the AllReduce's gather
 *           phase as the ring.
 *   ring    ReduceScatter: per step, each of the M positions reads the
 *           incoming partial and the rank's own element and writes the new
 *           partial; the first step's incoming partial and the last step's
 *           output are stored-type, the rest accumulator-type.  For 4- and
 *           8-byte types this is 3(N-1)·M·s.
 *           AllGather 2N·M·s (own shard placed, then N-1 copy steps).
 *           AllReduce the ReduceScatter phase plus 2(N-1)·M·s.
 * N = 1 runs the direct copy for every schedule.  Returns 0 for invalid
 * arguments.
 */
uint64_t ccl_sim_algorithmic_bytes(ccl_sim_coll_t coll, int nranks, size_t count, ccl_sim_dtype_t dtype,
                                   ccl_sim_schedule_t schedule);

/* Compute-kernel launches one call enqueues for count > 0: DIRECT 1;
 * stepwise ring N-1 (ReduceScatter), N-1 plus 1 own-shard placement
 * (out-of-place AllGather), 2(N-1) (AllReduce) — the nsteps of [DECOMP]
 * §源码二; RECURSIVE log2 N per phase (plus the placement of an
 * out-of-place AllGather); persistent ring, chained ring and chained
 * recursive 1.  Not counted: the pointer-table uploads when
 * nranks > 64 and the persistent ring's control-block reset.  N = 1: 1.
 * Returns -1 for invalid arguments. */
int ccl_sim_launch_count(ccl_sim_coll_t coll, int nranks, size_t count, ccl_sim_schedule_t schedule,
                         int in_place);

/* Chunk ring rank `rank` holds complete after the ReduceScatter phase:
 * (rank+1) mod nranks ([PRIMS] §五.2; [RING] §1).  -1 if out of range. */
int ccl_sim_ring_owner(int nranks, int rank);

/*
 * Ring routing ([RING] §2 N=4 table and pseudocode; [PRIMS] §五.2-五.3):
 * phase 0 = ReduceScatter, step t in [0, N-2]: send chunk (rank - t),
 *           receive chunk (rank - 1 - t);
 * phase 1 = AllGather after the ReduceScatter phase: send (rank + 1 - t),
 *           receive (rank - t);
 * phase 2 = stand-alone AllGather (rank r starts with shard r): send
 *           (rank - t), receive (rank - 1 - t).
 * All indices mod nranks.  Returns CCL_SIM_INVALID_ARGUMENT if out of range.
 */
ccl_sim_result_t ccl_sim_ring_route(int nranks, int phase, int step, int rank, int* send_chunk,
                                    int* recv_chunk);

/*
 * α-β (Hockney) cost model of a collective between N real ranks joined by
 * links of per-step latency α and bandwidth β ([PRIMS] §四 and §五; the ring
 * terms of [RING] §5 and [RS-PAGE] §Ring ReduceScatter).  A model, not a
 * measurement: it prices the pages' algorithms on a network so that a bench
 * row can carry modeled context.  T = steps·α + bytes_per_rank / β:
 *   ring        AllReduce 2(N-1) steps, 2(N-1)/N·S bytes; AllGather,
 *               ReduceScatter, all_to_all N-1 steps, (N-1)/N·S bytes;
 *               broadcast, reduce N-1 steps, S bytes (pipelined chain)
 *               ([PRIMS] §五.4);
 *   double tree AllReduce only: 2·ceil(log2 N) steps, 2S bytes ([PRIMS] §六);
 *   two-level   AllReduce only: intra-node ReduceScatter over ppn ranks,
 *               inter-node ring AllReduce of S/ppn over N/ppn nodes,
 *               intra-node AllGather ([PRIMS] §八).
 * algbw = S / T and busbw = algbw · factor, factor 2(N-1)/N for AllReduce,
 * (N-1)/N for AllGather, ReduceScatter and all_to_all, 1 for broadcast and
 * reduce ([PRIMS] §七, in 10^9 bytes per second).  S is in bytes as the
 * pages define it per primitive ([PRIMS] §二.1).
 */
typedef enum {
  CCL_SIM_MODEL_ALLREDUCE = 0,
  CCL_SIM_MODEL_ALL_GATHER = 1,
  CCL_SIM_MODEL_REDUCE_SCATTER = 2,
  CCL_SIM_MODEL_ALL_TO_ALL = 3,
  CCL_SIM_MODEL_BROADCAST = 4,
  CCL_SIM_MODEL_REDUCE = 5
} ccl_sim_model_coll_t;

typedef enum {
  CCL_SIM_ALGO_RING = 0,
  CCL_SIM_ALGO_DOUBLE_TREE = 1,
  CCL_SIM_ALGO_TWO_LEVEL = 2
} ccl_sim_model_algo_t;

typedef struct {
  double alpha_s;                 /* per-step latency, seconds (inter-node for two-level) */
  double beta_bytes_per_s;        /* link bandwidth, bytes per second (inter-node for two-level) */
  int ranks_per_node;             /* two-level only: ppn, must divide nranks */
  double alpha_intra_s;           /* two-level only */
  double beta_intra_bytes_per_s;  /* two-level only */
} ccl_sim_link_params_t;

typedef struct {
  double time_s;            /* latency_s + bandwidth_s */
  double latency_s;         /* steps · alpha */
  double bandwidth_s;       /* bytes_per_rank / beta (summed over phases for two-level) */
  double latency_fraction;  /* latency_s / time_s (0 when time_s is 0) */
  double algbw_gbps;        /* S / time_s in 10^9 B/s (0 when time_s is 0) */
  double busbw_gbps;        /* algbw · ccl_sim_busbw_factor */
  double steps;             /* communication steps on the critical path */
} ccl_sim_model_estimate_t;

/* Fills *out.  CCL_SIM_INVALID_ARGUMENT for nranks < 1, negative sizes or
 * latencies, non-positive bandwidths, NULL pointers or ppn not dividing
 * nranks; CCL_SIM_UNSUPPORTED for a tree or two-level model of anything but
 * AllReduce. */
ccl_sim_result_t ccl_sim_model_estimate(ccl_sim_model_coll_t coll, ccl_sim_model_algo_t algo, int nranks,
                                        double size_bytes, const ccl_sim_link_params_t* link,
                                        ccl_sim_model_estimate_t* out);

/* busbw / algbw for the collective at nranks ([PRIMS] §七); -1 if invalid. */
double ccl_sim_busbw_factor(ccl_sim_model_coll_t coll, int nranks);

/*
 * Recursive halving / doubling routing ([RS-PAGE] §Recursive Halving
 * ReduceScatter; N a power of two).  phase 0 = halving step `step` in
 * [1, log2 N]: *partner = rank XOR N/2^step, and [*first_block,
 * *first_block + *nblocks) are the blocks of q elements rank keeps and
 * reduces at that step.  phase 1 = doubling step `step` in [0, log2 N):
 * *partner = rank XOR 2^step, and the block range is what rank receives
 * from it.  CCL_SIM_INVALID_ARGUMENT when out of range.
 */
ccl_sim_result_t ccl_sim_recursive_route(int nranks, int phase, int step, int rank, int* partner,
                                         size_t* first_block, size_t* nblocks);

const char* ccl_sim_result_string(ccl_sim_result_t result);

/*
 * The persistent ring's watchdog (a diagnostic, not an operation of the
 * pages).  Its grid barrier and its flag waits poll a bounded number of
 * times.  A wait can run into that bound only if the device does not keep
 * the whole
 * cooperative grid resident (for instance while other work holds its
 * compute units); every workgroup then stops, the call's outputs are
 * incomplete, and the kernel raises an abort word in the workspace's
 * control block.  The call itself returns before the kernel runs, so it
 * cannot report this.  After the stream work of a CCL_SIM_RING_PERSISTENT
 * call with nranks >= 2 has completed, ccl_sim_persistent_aborted(workspace,
 * &aborted) reads that word (one synchronous device-to-host copy of 4 bytes
 * on the null stream; the control block opens the workspace): *aborted = 1
 * if the last persistent call that used this workspace stopped early, 0 if
 * it ran to the end.  Query before another call reuses the workspace: the
 * other schedules keep their partials where the control block was.
 * CCL_SIM_INVALID_ARGUMENT for NULL pointers, CCL_SIM_HIP_ERROR if the copy
 * fails.  Setting the environment variable CCL_SIM_DEBUG=1 makes every
 * persistent call wait for its kernel and return CCL_SIM_HIP_ERROR itself
 * when it aborted.
 * CCL_SIM_SPIN_LIMIT=n sets the poll limit (default 2^22); a tiny value
 * forces the abort from the host, for tests of this path.  Both are read
 * on every call.
 */
ccl_sim_result_t ccl_sim_persistent_aborted(const void* workspace, int* aborted);

/*
 * How a CCL_SIM_RING_PERSISTENT call orders its steps (a diagnostic, not an
 * operation of the pages): CCL_SIM_ORDER_GRID, a grid barrier between
 * steps, or CCL_SIM_ORDER_FLAGS, per-workgroup step flags.  `count` is M,
 * the logical per-rank length, as for ccl_sim_workspace_size; the answer
 * depends on N·ceil(M/N) and on CCL_SIM_PERSISTENT_SYNC, read now.  0 when
 * the call would run no ring (nranks 1, count 0); -1 for invalid arguments
 * or an unknown CCL_SIM_PERSISTENT_SYNC value.  No HIP call is made.
 */
#define CCL_SIM_ORDER_GRID 1
#define CCL_SIM_ORDER_FLAGS 2
int ccl_sim_persistent_ordering(ccl_sim_coll_t coll, int nranks, size_t count);

/* Message describing the last failed call on this thread ("" if none). */
const char* ccl_sim_last_error(void);

int ccl_sim_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CCL_SIM_H */
