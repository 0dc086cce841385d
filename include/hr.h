/*
 * hr.h -- C ABI of libhr, the MI355X (gfx950) FP16 all-reduce combine.
 *
 * The operation.  An all-reduce over a tensor-parallel group leaves on every
 * rank the elementwise sum of the ranks' FP16 contributions.  libhr computes
 * that sum as a left fold in rank order with one binary16 rounding (to
 * nearest, ties to even) after every add:
 *
 *     R[i] = fl16( ... fl16( fl16(x0[i] + x1[i]) + x2[i] ) ... + x_{G-1}[i] )
 *
 * For two ranks this is the single-rounding, commutative FP16 sum that the
 * 1Cat-vLLM pull request "[Kernel] Two-rank FP16 all-reduce through pinned
 * host memory for GPUs without P2P" describes (section "Purpose"); both ranks
 * obtain identical bits.  For more ranks the pages fix no order; the SGLang
 * pull request "[SM120] Add optional FlashInfer PCIe-IPC all-reduce for
 * switch-free hosts" (section "Accuracy") shows that the order changes bits,
 * so libhr fixes the left fold in increasing rank index.  NaN payloads are
 * whatever the hardware add produces; every other result is exact to the
 * definition above.
 *
 * Two entry points compute it:
 *
 *  - hr_reduce_f16: G contributions already resident in device memory (HBM)
 *    are folded into one output buffer by one kernel launch.
 *
 *  - hr_allreduce_f16: an exchange through a channel of W ranks (W = 2 is
 *    the two-rank method; up to HR_MAX_WORLD).  Each rank's kernel writes
 *    its contribution into pinned, device-mapped host memory, raises a
 *    per-workgroup ready flag, waits for the peers' flags and adds the
 *    peers' values, as the 1Cat-vLLM page's "Purpose" section lays out: one
 *    kernel per call, no CPU work, no stream synchronisation, so the call can
 *    be captured into a hipGraph; host slots are double buffered by call
 *    parity.  The channel is a handle so that one process can own several
 *    groups (same section).  All ranks of a channel may live in one process
 *    on one GPU ("loopback": concurrently running launches on W streams).
 *
 * Conventions for every function:
 *  - Every function returns an hr_status; nothing throws across the ABI.
 *  - Device pointers are plain HIP device addresses (hipMalloc memory or any
 *    allocator built on it); buffers hold IEEE binary16 values, contiguous,
 *    element i at byte offset 2*i.  The caller owns them and keeps them alive
 *    until the work queued on the stream has finished.
 *  - A stream argument is a hipStream_t; NULL selects the null stream of the
 *    current device.  Calls only enqueue work on that stream: they never
 *    synchronise, allocate or copy, so they may be captured into a graph.
 *  - Argument errors are reported synchronously, before anything is
 *    enqueued, and leave all state unchanged.
 */
#ifndef HR_H
#define HR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(HR_BUILDING_LIBRARY)
#define HR_API __attribute__((visibility("default")))
#else
#define HR_API
#endif

/* Same tag as hipStream_t, so a hipStream_t converts without a cast. */
typedef struct ihipStream_t *hr_stream_t;

/* Opaque channel handle; the library owns everything behind it. */
typedef struct hr_channel_s *hr_channel;

typedef enum {
    HR_OK = 0,
    HR_ERR_INVALID_ARG = 1,  /* null pointer, bad rank/G, partial overlap  */
    HR_ERR_ALIGNMENT = 2,    /* a binary16 pointer that is not 2-byte aligned */
    HR_ERR_TOO_LARGE = 3,    /* numel above the channel's max_numel          */
    HR_ERR_UNSUPPORTED = 4,  /* world_size outside 2..HR_MAX_WORLD, device unusable */
    HR_ERR_HIP = 5,          /* a HIP runtime call failed                    */
    HR_ERR_TIMEOUT = 6,      /* a wait for the peer exceeded timeout_us      */
    HR_ERR_ABORTED = 7       /* hr_channel_abort cancelled waiting kernels   */
} hr_status;

/* Largest number of contributions hr_reduce_f16 folds in one call. */
#define HR_MAX_G 16

/* Largest group a channel serves. */
#define HR_MAX_WORLD 8

/* Default cap of one exchange: 131072 binary16 values = 256 KiB per rank,
 * the payload limit the 1Cat-vLLM page admits to the host path ("Purpose"). */
#define HR_DEFAULT_MAX_NUMEL 131072u

/* Largest max_numel a channel accepts: 2^29 values = 1 GiB per slot. */
#define HR_MAX_NUMEL_LIMIT (1ull << 29)

/* Default watchdog for one wait on the peer, in microseconds. */
#define HR_DEFAULT_TIMEOUT_US 1000000u

/* Host-link rate the one-shot and the two-shot pace their workgroups by
   (MB/s; see hr_channel_config.link_mbps): the rate taken when the library's
   measurement fails (a PCIe 5.0 x16 link as measured on MI355X hosts, whose
   one-way copies reach 55 GB/s), the values that turn pacing off and that
   measure the link anew, and the smallest rate accepted. */
#define HR_DEFAULT_LINK_MBPS 50000u
#define HR_LINK_UNPACED 0xFFFFFFFFu
#define HR_LINK_CALIBRATE 0xFFFFFFFEu /* measure the link at channel creation */
#define HR_MIN_LINK_MBPS 100u      /* smaller nonzero rates are refused */

/* Exchange algorithm of a channel (all produce the same bits). */
#define HR_ALGO_AUTO 0      /* low-latency up to a size that falls with
                               the group (20480 values at 2 ranks, 8192
                               at 3, 4096 at 4 and 5, 2560 at 6, 2048 at
                               7, 1536 at 8); above it the one-shot, and
                               for 3+ ranks the two-shot from a size that
                               also falls with the group (98304 values at
                               3 ranks, 16384 at 4, 10240 at 5, 6144 at
                               6, 5120 at 7, 3072 at 8)                   */
#define HR_ALGO_ONE_SHOT 1  /* every rank reads every peer's contribution */
#define HR_ALGO_TWO_SHOT 2  /* shard owners fold, then everyone gathers;
                               needs num_blocks >= world_size             */
#define HR_ALGO_LL 3        /* low-latency one-shot: every 8-byte word in
                               host memory carries 6 bytes of values and a
                               16-bit call field, so readers poll the data
                               itself (no flags); 3/2 of the link bytes; up
                               to 32768 values (larger calls: one-shot)   */

typedef struct {
    int device;           /* HIP device ordinal the channel's kernels run on  */
    int world_size;       /* ranks W in the group, 2..HR_MAX_WORLD; 2 is the
                             source's two-rank method, larger W folds all
                             ranks left in rank order                         */
    size_t max_numel;     /* largest numel of one call; 0 = HR_DEFAULT_MAX_NUMEL;
                             at most HR_MAX_NUMEL_LIMIT                        */
    int num_blocks;       /* workgroups per rank launch; 0 = automatic.  All
                             ranks of a loopback channel run at once on one
                             GPU, so the value is clamped to the device's
                             compute units / world_size.                       */
    uint32_t timeout_us;  /* watchdog per wait; 0 = HR_DEFAULT_TIMEOUT_US      */
    int algorithm;        /* HR_ALGO_*; 0 = automatic                         */
    uint32_t link_mbps;   /* rate (MB/s) at which the host link that the
                             channel's ranks share carries writes while
                             reads run the other way.  0 = measured: the
                             first channel created with 0 on a device runs
                             the HR_LINK_CALIBRATE measurement below and the
                             library keeps the rate for every later such
                             channel on that device, for the life of the
                             process (HR_DEFAULT_LINK_MBPS if the
                             measurement fails).  The one-shot and the
                             two-shot start workgroup b's publish b - k
                             slices later than workgroups 0..k's (k = 4 for
                             one-shot calls that give every lane at most one
                             16-byte unit, 2 otherwise), a slice taking
                             world_size x slice bytes / link_mbps, so that
                             each workgroup's flag and reads are not queued
                             behind every other workgroup's writes (the link
                             carries requests in order) and the reads of
                             early slices overlap the writes of later ones.
                             A rate above the real one only lets the writes
                             queue again; one well below it delays the call.
                             HR_LINK_UNPACED: no pacing.  HR_LINK_CALIBRATE:
                             hr_create_channel times a kernel that writes
                             16 MiB to pinned host memory while it reads
                             16 MiB from it (best of 3, after a warm-up) and
                             paces 1/32 above that rate (measured best on
                             MI355X hosts: slices start just before the
                             link would run dry); this takes a few
                             milliseconds and should run while the link is
                             otherwise idle (so should the first channel
                             created with 0 on a device).                     */
} hr_channel_config;

/* Read-only description of a channel, for diagnostics and tests. */
typedef struct {
    int device;
    int world_size;
    size_t max_numel;
    int num_blocks;
    int block_threads;            /* threads per workgroup of one launch      */
    uint32_t timeout_us;
    void *host_slots;             /* host address of the slot region:
                                     [2 parity][world][slot_stride] binary16  */
    size_t slot_stride;           /* elements per slot (>= max_numel)         */
    volatile uint64_t *host_flags; /* host address of the ready flags (64-bit
                                     call numbers): flag of (rank r, block b)
                                     at index (r * num_blocks + b) * flag_stride */
    size_t flag_stride;           /* uint64 words between consecutive flags   */
    volatile uint32_t *host_error; /* sticky asynchronous status word         */
    volatile uint32_t *host_abort; /* nonzero = cancel waits                  */
    int algorithm;                /* HR_ALGO_* the channel was created with  */
    void *host_reduced;           /* two-shot reduced-shard slots
                                     [2 parity][slot_stride] binary16         */
    volatile uint64_t *host_flags2; /* two-shot reduced-shard flags, laid out
                                     like host_flags                          */
    void *host_ll;                /* low-latency slots [2 parity][world]
                                     [ll_stride] 64-bit words, each slot three
                                     planes of ll_stride / 3 words; unit u of
                                     a call (values v0..v7) is word u of each
                                     plane: v0 v1 v2, v3 v4 v5 and v6 v7 0 in
                                     bits 0..47, the call field in bits 48..63
                                     (the call number's low 15 bits | 0x8000) */
    size_t ll_stride;             /* 64-bit words per low-latency slot        */
    uint32_t link_mbps;           /* the pacing rate in effect (MB/s), or
                                     HR_LINK_UNPACED                          */
    uint64_t *dev_epochs;         /* device address of the call counters
                                     [world][num_blocks]: the last call number
                                     each rank's workgroup took.  Call numbers
                                     run 1, 2, 3, ... skipping every value
                                     whose low 32 bits are zero; a flag holds
                                     the full number, a low-latency word the
                                     call field above.                        */
} hr_channel_info;

/*
 * hr_create_channel -- set up one exchange group of world_size ranks.
 *
 * Allocates the channel's pinned, device-mapped, fine-grained host memory
 * (slots [2 parity][world][max_numel] binary16, per-workgroup ready flags,
 * the error and abort words) and its device-resident per-workgroup call
 * counters, and zeroes them.  The slot region has the 2 x world_size x
 * max_numel shape of the double-buffered workspace that the SGLang page's
 * "Modifications" section sizes.  Not capturable (it allocates); call it
 * before any capture.
 *
 * cfg:  see hr_channel_config.  *out receives the handle on success and is
 *       left untouched on failure.
 * Errors: HR_ERR_INVALID_ARG (null cfg/out, negative or out-of-range
 *       fields, link_mbps below HR_MIN_LINK_MBPS), HR_ERR_UNSUPPORTED
 *       (world_size outside 2..HR_MAX_WORLD), HR_ERR_HIP (including a failed
 *       link measurement under HR_LINK_CALIBRATE).
 */
HR_API hr_status hr_create_channel(const hr_channel_config *cfg, hr_channel *out);

/*
 * hr_allreduce_f16 -- one all-reduce call of rank `rank` (0..world_size-1).
 *
 * One-shot algorithm (below); the two-shot (HR_ALGO_TWO_SHOT, or automatic
 * for larger groups and payloads) instead has each shard's owner fold that
 * shard in rank order and publish it, and every rank gather the others'
 * folded shards: less host-link traffic for W > 2, the same bits.  The
 * low-latency one-shot (HR_ALGO_LL, or automatic for small calls: up to
 * 20480 values for two ranks, fewer for larger groups) puts a call field
 * into every 8-byte word it writes to host memory, so a peer polls the
 * values themselves: no flag, no wait for acknowledgements, one host-link
 * round trip less; the same bits again.
 *
 * Enqueues exactly one kernel on `stream`.  Its workgroups each own one
 * contiguous slice of the numel values: they copy the slice of `in` into this
 * rank's host slot of the current parity (paced at the channel's link rate),
 * make the stores visible at system scope, raise their ready flag, wait
 * (watchdog-bounded) for every peer's flag of the same call, read the peers'
 * slices from their host slots and
 * write the left fold x0 + x1 + ... in rank order, one binary16 rounding per
 * add, to `out` (for two ranks fl16(x0 + x1), the 1Cat-vLLM page's
 * "Purpose").  Parity comes from a device-resident per-workgroup call
 * counter, so a replayed graph alternates slots without host involvement.
 *
 * in, out: device binary16 buffers of numel values; out == in is allowed,
 *          any other overlap is an error.
 * numel:   0 enqueues nothing; must not exceed the channel's max_numel.
 * All ranks must issue the same sequence of numel values.  The ranks must be
 * driven from streams that can run concurrently (separate processes, or, in
 * one process, streams from hr_loopback_stream_create), each endpoint by one
 * stream at a time; all launches of a call must be in flight together or the
 * waits time out.
 * Null-stream hazard in loopback: the Algorithmiq page "fix(group): run each
 * rank on a non-blocking stream" ("What") runs every rank on a non-blocking
 * stream.  The streams of hr_loopback_stream_create are not non-blocking
 * (HIP gives a compute-unit-mask stream no flags): they wait for earlier
 * null-stream work, and later null-stream work waits for them.  Work put on
 * the null stream between the ranks' launches of one call therefore holds
 * back the ranks launched after it while the ones launched before it spin:
 * the call ends at the watchdog with the sticky HR_ERR_TIMEOUT.  Enqueue no
 * null-stream work (including a library's default-stream work) between the
 * launches of one call, or use hr_allreduce_group_f16, whose one launch has
 * no such window.
 *
 * Errors: HR_ERR_INVALID_ARG, HR_ERR_ALIGNMENT, HR_ERR_TOO_LARGE (the caller
 * keeps its own collective for larger payloads), HR_ERR_HIP; and the
 * channel's sticky HR_ERR_TIMEOUT / HR_ERR_ABORTED, in which case nothing is
 * launched.  A timed-out or aborted kernel leaves `out` unwritten.
 */
HR_API hr_status hr_allreduce_f16(hr_channel ch, int rank, const void *in, void *out,
                                  size_t numel, hr_stream_t stream);

/*
 * hr_exchange_algorithm -- which algorithm a call of numel values on this
 * channel takes: HR_ALGO_ONE_SHOT, HR_ALGO_TWO_SHOT or HR_ALGO_LL in
 * *algorithm.  A function of the channel and numel only (not of a rank's
 * buffers), which is why every rank of a call takes the same algorithm.
 * Host-only; enqueues nothing.
 * Errors: HR_ERR_INVALID_ARG (null ch or algorithm), HR_ERR_TOO_LARGE
 * (numel above the channel's max_numel).
 */
HR_API hr_status hr_exchange_algorithm(hr_channel ch, size_t numel, int *algorithm);

/*
 * hr_reduce_f16 -- fold G contributions resident in device memory.
 *
 * out[i] = left fold of inputs[0][i] .. inputs[G-1][i] with one binary16
 * rounding per add (the combine defined at the top of this header).  One
 * kernel launch on `stream`; the G pointers are copied into the launch, so
 * the `inputs` array may be freed on return.
 *
 * inputs: G device pointers, each to numel binary16 values.
 * G:      1 .. HR_MAX_G (G = 1 copies inputs[0]).
 * out:    device buffer of numel values; it may equal any input exactly, any
 *         partial overlap with an input is an error.
 * numel:  0 enqueues nothing.
 * Errors: HR_ERR_INVALID_ARG, HR_ERR_ALIGNMENT, HR_ERR_HIP.
 */
HR_API hr_status hr_reduce_f16(const void *const *inputs, int G, void *out, size_t numel,
                               hr_stream_t stream);

/*
 * hr_workspace_stride -- where to place G contributions of numel values in
 * one device buffer for hr_reduce_f16 / _bf16: contribution g at
 * base + g * stride values (stride = numel rounded up to 2 MiB, plus 4 KiB).
 * Contributions a multiple of 2 MiB apart hit the same HBM banks at equal
 * offsets; the 4 KiB shift spreads them, and the fold recognises the layout.
 * The result does not depend on the layout; only the speed does.
 * Pure host arithmetic.
 */
HR_API size_t hr_workspace_stride(size_t numel);

/*
 * hr_reduce_bf16 / hr_allreduce_bf16 -- the same two operations on bfloat16
 * values (sign, 8-bit exponent, 7-bit fraction): left fold in rank order,
 * one bfloat16 rounding to nearest even per add, subnormals kept.  The SGLang
 * page's reductions are bfloat16 ("Accuracy").  Arguments, layout, ownership
 * and errors are those of the binary16 functions; a channel carries either
 * type, but all ranks of one call must use the same one.
 */
HR_API hr_status hr_reduce_bf16(const void *const *inputs, int G, void *out, size_t numel,
                                hr_stream_t stream);
HR_API hr_status hr_allreduce_bf16(hr_channel ch, int rank, const void *in, void *out,
                                   size_t numel, hr_stream_t stream);

/*
 * hr_allreduce_group_f16 / hr_allreduce_group_bf16 -- one all-reduce call of
 * every rank of a loopback channel, in a single kernel launch on `stream`.
 *
 * Rank r's workgroups are workgroups r * num_blocks .. (r + 1) * num_blocks - 1
 * of the launch; each runs exactly what hr_allreduce_f16 (_bf16) runs for rank
 * r -- the same algorithm, host slots, flags and call counters -- so the
 * result in outs[r] is the left fold of ins[0..W-1] in rank order, bit for bit
 * what W separate calls give, and group calls and per-rank calls may follow
 * one another on the same channel.  This is the loopback's driver for groups
 * that have more ranks than the GPU schedules hardware queues at once: W
 * separate launches on W loopback streams need all W queues resident
 * together, and with eight the GPU takes turns over them; one launch of
 * W * num_blocks <= compute-unit workgroups is resident at once.  It stands in
 * for W GPUs each running its rank's kernel; it is not a multi-GPU call.
 *
 * ins, outs: world_size device buffers of numel values each (binary16, or
 *          bfloat16 for _bf16); the arrays are copied into the launch and may
 *          be freed on return.  outs[r] == ins[r] is allowed; any other
 *          overlap between rank r's output and any rank's input or output is
 *          an error.
 * numel, errors, sticky status, capture: as hr_allreduce_f16.  The launch
 *          needs every compute unit able to take one of its workgroups; work
 *          that fills the device meanwhile delays it (the watchdog bounds the
 *          wait).
 */
HR_API hr_status hr_allreduce_group_f16(hr_channel ch, const void *const *ins, void *const *outs, size_t numel,
                                        hr_stream_t stream);
HR_API hr_status hr_allreduce_group_bf16(hr_channel ch, const void *const *ins, void *const *outs, size_t numel,
                                         hr_stream_t stream);

/*
 * hr_allreduce_group_noalloc_f16 -- hr_allreduce_group_f16 for callers that
 * cannot allocate: code under hipGraph capture before any channel exists,
 * tight serving loops, harnesses that forbid hipMalloc.  It needs no channel
 * and allocates nothing: the state a channel would allocate (slots, flags,
 * call counters, error words) lives in a fixed device array inside the
 * library, HR_NOALLOC_SCRATCH_BYTES per device, which each device that the
 * library runs on holds until the process ends.  Its slots are in device
 * memory (HBM), not pinned host memory: the exchange protocol, the kernels
 * and the result bits are those of hr_allreduce_group_f16 under
 * HR_ALGO_AUTO, the left fold of ins[0..W-1] in rank order into every
 * outs[r].
 *
 * Enqueues two kernels on `stream`: a small fill that clears the array's
 * flags, counters and error words (and, for a low-latency call, the words
 * that call reads), then the group exchange.  So every call starts from a
 * cleared state and leaves the array holding its own contents; nothing
 * carries from one call to the next.  Calls that overlap on one device --
 * on different streams, or in different threads at once -- share the array
 * and race; calls on one stream do not.  The first call on a device looks up
 * the array's device address (once, under a lock); make that first call
 * outside any capture.
 *
 * ins, outs:  world_size device binary16 buffers of numel values each, as
 *             for hr_allreduce_group_f16 (outs[r] == ins[r] allowed, any
 *             other overlap with a rank's buffers an error); the arrays are
 *             copied into the launch.
 * world_size: 2..HR_MAX_WORLD.
 * numel:      at most HR_NOALLOC_MAX_NUMEL; 0 enqueues nothing.
 * status:     NULL, or a 4-byte aligned device word that the fill sets to
 *             HR_OK and the exchange to HR_ERR_TIMEOUT if a wait exceeds the
 *             default watchdog (a launch that cannot be resident at once,
 *             because other work fills the device); `outs` is then unwritten.
 * Errors (synchronous, nothing enqueued): HR_ERR_UNSUPPORTED (world_size out
 * of range, or a device whose compute-unit count needs more than the
 * array), HR_ERR_TOO_LARGE (numel above HR_NOALLOC_MAX_NUMEL),
 * HR_ERR_INVALID_ARG, HR_ERR_ALIGNMENT, HR_ERR_HIP.
 */
#define HR_NOALLOC_MAX_NUMEL 131072u
#define HR_NOALLOC_SCRATCH_BYTES (8u << 20)
HR_API hr_status hr_allreduce_group_noalloc_f16(const void *const *ins, void *const *outs, int world_size,
                                                size_t numel, uint32_t *status, hr_stream_t stream);

/*
 * hr_channel_status -- the channel's sticky asynchronous status: HR_OK, or
 * HR_ERR_TIMEOUT / HR_ERR_ABORTED once a kernel has recorded one.
 *
 * A collective that spins on its peer has no timeout of its own; the
 * openinfer pull request "fix(qwen3): re-enable CUDA Graph under TP via
 * startup decode-graph pre-capture" ("Description") turns such a wedge into a
 * loud failure with a watchdog and reports which peers never arrived.  Here
 * every device-side wait is bounded by the channel's timeout_us watchdog; a
 * kernel that hits it, or sees the abort word, records the status in a
 * host-mapped word and leaves `out` unwritten, and every later call on the
 * channel returns that status without launching, so the failure cannot be
 * missed or cascade through a replayed graph.
 *
 * ch: a channel from hr_create_channel.  Reads the host-mapped word; it does
 * not synchronise, so synchronise the rank streams first to see the outcome
 * of work already enqueued.  Recovery from an error is hr_destroy followed
 * by hr_create_channel.
 * Errors: HR_ERR_INVALID_ARG for a null channel.
 */
HR_API hr_status hr_channel_status(hr_channel ch);

/*
 * hr_channel_abort -- ask every kernel of this channel that is waiting, or
 * will wait, for its peer to stop: waits end with HR_ERR_ABORTED recorded in
 * the channel and `out` unwritten.
 *
 * The openinfer page ("Description") aborts loudly rather than letting a
 * rank that spins on a peer hang the process; this is the host's handle on
 * the same decision, for a caller that knows a peer will never arrive (a
 * rank that failed, a shutdown) and does not want to wait for the watchdog.
 * A wait reads the abort word once it has lasted 20 us (polling it sooner
 * slows every call), so a kernel stops within microseconds of that.  The
 * abort is sticky: the channel then refuses every call (hr_channel_status).
 *
 * ch: a channel from hr_create_channel.  Host-side store only; returns at
 * once.  Errors: HR_ERR_INVALID_ARG for a null channel.
 */
HR_API hr_status hr_channel_abort(hr_channel ch);

/*
 * hr_channel_timeout_info -- after HR_ERR_TIMEOUT: which peers a rank's wait
 * never heard from.
 *
 * The openinfer page ("Description") makes a wedged collective fail loudly
 * and name the peers that never arrived.  When a wait for the peers'
 * publishes (their ready flags, or their low-latency words) reaches the
 * watchdog, the kernel records three things in one 64-bit word of the
 * channel's host memory: the rank whose wait expired, the set of peers
 * whose publish it had not seen, and the call number.  When several waits
 * expire, the last record stays.  A two-shot rank waiting for a shard
 * owner's folded shard records nothing: that wait expires only because some
 * publish never arrived, and the owner's own wait records that.
 *
 * rank:      the rank whose wait expired, or -1 when nothing is recorded.
 * peer_mask: bit q is set when rank q's publish never arrived; 0 when
 *            nothing is recorded.
 * call:      the call number's low 48 bits (a channel's first call on each
 *            rank is number 1); 0 when nothing is recorded.
 * Read it once the rank streams have finished (hr_channel_status then
 * reports HR_ERR_TIMEOUT).  The allocation-free group call records nothing
 * here; its status word is its whole report.  Host-only; never blocks.
 * Errors: HR_ERR_INVALID_ARG for a null argument.
 */
HR_API hr_status hr_channel_timeout_info(hr_channel ch, int *rank, uint32_t *peer_mask, uint64_t *call);

/* hr_channel_get_info -- fill *info with the channel's layout (read-only). */
HR_API hr_status hr_channel_get_info(hr_channel ch, hr_channel_info *info);

/*
 * hr_destroy -- release the channel: its pinned host slots, flags, error and
 * abort words, and its device call counters.
 *
 * Order of teardown.  The openinfer page ("Description") destroys captured
 * graphs before the communicator they reference, and the SGLang pull request
 * "[SM120] Add optional FlashInfer PCIe-IPC all-reduce for switch-free hosts"
 * (review thread on its destroy() method) releases the all-reduce workspace
 * before the process groups it uses.  Here: destroy every graph that
 * captured calls on the channel, then synchronise the rank streams, then
 * call this.  It synchronises the channel's whole device before freeing the
 * host memory the kernels use, so it also waits for other work there
 * (another channel's waits end at the latest at that channel's watchdog).
 *
 * ch: the channel, or NULL (a no-op returning HR_OK).  The handle is invalid
 * afterwards, even when an error is returned.
 * Errors: HR_ERR_HIP when the device synchronisation fails (the memory is
 * released all the same).
 */
HR_API hr_status hr_destroy(hr_channel ch);

/*
 * hr_loopback_stream_create -- a stream for one rank of a loopback channel.
 *
 * The launches of one exchange call (one per rank) must run at the same
 * time.  The HIP runtime spreads ordinary streams over a small pool of
 * hardware queues (GPU_MAX_HW_QUEUES), and two streams that share a queue run
 * their kernels one after the other, so ordinary streams give no such
 * guarantee.  A stream
 * created here owns its hardware queue: it is created with an explicit
 * compute-unit mask (the runtime never pools such queues) that enables every
 * compute unit of `device`.  It is ordered with the null stream like any
 * stream created without hipStreamNonBlocking, so do not enqueue work on the
 * null stream between the ranks' launches of one call.
 *
 * device: HIP device ordinal.  *out receives a hipStream_t owned by the
 * caller, released with hr_loopback_stream_destroy.
 * Errors: HR_ERR_INVALID_ARG, HR_ERR_HIP.
 */
HR_API hr_status hr_loopback_stream_create(int device, hr_stream_t *out);

/* hr_loopback_stream_destroy -- release a stream from
 * hr_loopback_stream_create (after its work has finished).  NULL is a no-op. */
HR_API hr_status hr_loopback_stream_destroy(hr_stream_t stream);

/*
 * Admission: which reductions take the host-slot all-reduce.
 *
 * The 1Cat-vLLM page admits FP16 payloads of two-rank groups without peer
 * access up to 256 KiB, behind an on/off switch, and leaves everything else
 * on the caller's existing collective ("Purpose", "Path coverage").  The
 * SGLang page sizes its bound for decode: rows = max batch x tokens per
 * request per step, times hidden ("Modifications").  hr_admit applies that
 * policy (widened to bfloat16 and larger groups only when asked) and names
 * the first reason it declines, so a decline is never silent.  Pure host
 * logic: no device is touched.
 */
typedef enum {
    HR_ROUTE_HOST = 0,           /* take hr_allreduce_f16 / _bf16 */
    HR_DECLINE_DISABLED = 1,     /* policy switched off */
    HR_DECLINE_DTYPE = 2,        /* not binary16 (or bfloat16 when allowed) */
    HR_DECLINE_WORLD_SIZE = 3,   /* group size outside 2..max_world */
    HR_DECLINE_PEER_ACCESS = 4,  /* the GPUs reach each other directly */
    HR_DECLINE_TOO_LARGE = 5     /* payload above the cap */
} hr_route;

typedef enum { HR_DTYPE_F16 = 0, HR_DTYPE_BF16 = 1, HR_DTYPE_OTHER = 2 } hr_dtype;

typedef struct {
    int enabled;       /* 0 declines everything (HR_DECLINE_DISABLED)          */
    size_t max_bytes;  /* payload cap per rank; 0 = 256 KiB                    */
    int allow_bf16;    /* nonzero admits bfloat16 as well as binary16          */
    int max_world;     /* largest group admitted; 0 = 2 (the two-rank method)  */
} hr_admit_policy;

/* Route for one reduction of `numel` values of `dtype` in a group of
 * `world_size` ranks; `peer_access` nonzero when the GPUs can reach each
 * other directly.  A NULL policy is the page's default: enabled, FP16 only,
 * two ranks, 256 KiB. */
HR_API hr_route hr_admit(const hr_admit_policy *policy, hr_dtype dtype, int world_size,
                         int peer_access, size_t numel);

/* Static name of a route. */
HR_API const char *hr_route_str(hr_route r);

/* Decode-sized bound in values: max_batch x tokens_per_request (0 counts as
 * 1) x hidden -- e.g. 64 x 1 x 6144 = 393216, the SGLang page's default. */
HR_API size_t hr_decode_numel(size_t max_batch, size_t tokens_per_request, size_t hidden);

/* Static, human-readable name of a status code. */
HR_API const char *hr_status_str(hr_status s);

#ifdef __cplusplus
}
#endif

#endif /* HR_H */
