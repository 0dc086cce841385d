// exchange.hip -- the FP16 (and bfloat16) all-reduce of a W-rank group
// through pinned host slots (W = 2 is the method of the source; 3..8 extend
// it).  The slots only carry 16-bit patterns, so one channel serves both
// element types; the ranks of one call must use the same type.
//
// The method is the one the 1Cat-vLLM pull request "[Kernel] Two-rank FP16
// all-reduce through pinned host memory for GPUs without P2P" lays out in
// its "Purpose" section: one kernel per call; each workgroup writes its chunk
// of the rank's contribution into host memory that the ranks map, fences,
// raises a per-workgroup ready flag, waits for the peers' flags and adds the
// peers' chunks, one FP16 rounding per add, so every rank obtains the same
// bits; there is no CPU work and no stream synchronisation, so the call can
// be captured into a graph, and the host slots are double buffered by call
// parity.  Channels are handles so one process can own several groups (same
// section).  For W > 2 the values are folded left in rank order 0..W-1 (the
// SGLang pull request "[SM120] Add optional FlashInfer PCIe-IPC all-reduce
// for switch-free hosts", section "Accuracy", shows that order changes bits).
//
// Three algorithms, one channel, the same bits (a call takes one of them as
// a function of the channel and numel, so every rank agrees): the one-shot
// below (the source's method), the two-shot (exchange2_k) and the
// low-latency one-shot for small calls (exchange_ll_k).  Each is a device
// body of the workgroup index, launched either once per rank (the rank's
// own kernel, as on its own GPU) or once for every rank of a loopback group
// (the *_group_k kernels: rank r's workgroups are blocks r * nblocks ..).
// The per-rank kernels take the arguments of their first loads as leading
// scalars, which the build has preloaded into SGPRs.
//
// Channel memory
//   host (pinned, device-mapped, fine-grained/coherent):
//     slots  [2 parity][W rank][stride] binary16 -- the 2 x world x numel
//            workspace of the SGLang page's "Modifications" section
//     reduced-shard slots [2 parity][stride] (two-shot)
//     flags, reduced-shard flags  [W rank][nblocks], one 128-byte line each:
//            the 64-bit call number of the last slice that workgroup
//            published
//     low-latency slots [2 parity][W rank][3 planes][units] 64-bit words,
//            each three values and a 16-bit call field
//     error word, abort word, timeout record (one line each; the record
//            names the peers a timed-out wait never heard from)
//   device (HBM): epoch[W rank][nblocks] -- per-workgroup 64-bit call
//     counter (see next_call_number), device error word.
//
// Every launch has the channel's fixed workgroup count; each workgroup
// advances its call counter, so parity is uniform across a call.  Only the
// first `nactive` workgroups (a function of numel and W, so equal on every
// rank) carry values and take part in the flag handshake: fewer pollers
// means less non-posted traffic on the host link, which is what bounds
// small calls.
//
// One-shot protocol of active workgroup b of rank r at call e:
//   0. load the first batch of its slice of `in` (before the call counter,
//      so the two latencies overlap), then wait b - 2 slices (pace): the
//      link carries requests in order, and without pacing every flag and
//      read would queue behind all writes
//   1. store its slice to slot[e & 1][r] with system-coherent
//      (write-through) stores                                        (D2H)
//   2. every lane waits for its stores to be acknowledged; barrier; lane 0
//      stores flag[r][b] = e at system scope -- the "fence, then flag" of
//      the method, without a whole-cache write-back
//   3. lanes q != r of the first wave poll flag[q][b] with system-scope
//      loads until each reaches e (signed 64-bit compare, so a peer already
//      at e + 1 also releases the wait), sleeping between polls; a wait
//      that lasts over 20 us also reads the abort word, and a watchdog on
//      the constant-rate wall clock bounds the wait
//   4. barrier, then system-coherent loads of slot[e & 1][q] for every
//      peer q (H2D) and its own values (still in registers when the slice
//      gave each lane one unit, else loaded from `in` again); store the left
//      fold x0 + x1 + ... + x_{W-1}, in rank order, to `out`.
// Why one parity cannot be overwritten while a peer still reads it: a rank
// starts call e + 2 (same parity as e) only after its call e + 1 has
// finished, and in call e + 1 its workgroup 0 (always active) waited for
// every peer's flag of call e + 1, which a peer raises only after its whole
// call-e kernel has finished (stream order).
//
// Errors (timeout, abort) are written to the device error word and the
// host-mapped error word; a kernel that finds the device word set returns at
// once without touching `out`, so a failed call cannot cascade into a long
// chain of timeouts inside a replayed graph.
#include "hr_internal.h"

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

namespace hr {

constexpr int kExchThreads = 256;
constexpr int kExchUnroll = 4;                    // units per lane per publish batch
constexpr int kMaxWorld = 8;
constexpr int kMinActivePolls = 16;                // W * minimum active workgroups
constexpr uint32_t kAbortAfterUs = 20;             // waits read the abort word only after this long
constexpr uint32_t kLLLeadNs = 400;                // an LL poll's lead over the words it should find
constexpr uint32_t kLLFloorNs = 450;               // least hold of an LL poll in a per-rank launch
constexpr size_t kLine = 128;                     // bytes per flag / word line
constexpr size_t kFlagStride = kLine / sizeof(uint64_t);  // flags are 64-bit call numbers

struct ExchArgs {
    const void *in;
    void *out;
    size_t numel;
    uint16_t *slots;          // device view of the host slot region
    size_t stride;            // values per slot
    uint64_t *flags;          // device view of the host flags (publish)
    uint64_t *flags2;         // device view of the host flags (reduced shard, two-shot)
    uint16_t *reduced;        // device view of the reduced-shard slots [2][stride] (two-shot)
    uint64_t *ll;             // device view of the low-latency slots [2][W][ll_stride] (LL)
    size_t ll_stride;         // 8-byte words per low-latency slot: three planes of ll_stride / 3
    uint64_t *epochs;         // this rank's call counters (HBM)
    uint32_t *dev_error;      // HBM
    uint32_t *host_error;     // device view of the host error word
    const uint32_t *abort_w;  // device view of the host abort word
    uint64_t *diag;           // device view of the host timeout record, or null
    uint64_t timeout_ticks;
    uint64_t abort_after_ticks;  // waits shorter than this do not read the abort word
    uint16_t ll_lead_ticks;   // LL: a read's lead over the last word it should find
    uint16_t ll_floor_ticks;  // LL: the least hold before the first poll (per-rank launches)
    uint32_t pace_q16;        // wall-clock ticks per byte of a paced publish, x 2^16 (0: unpaced)
    int rank;
    int world;
    int nblocks;   // launched workgroups (the channel's fixed count)
    int nactive;   // workgroups that carry values in this call
};

template <class E>
__device__ __forceinline__ u32x4 combine(u32x4 x0, u32x4 x1) { return E::add8(x0, x1); }
template <class E>
__device__ __forceinline__ uint16_t combine(uint16_t x0, uint16_t x1) { return E::add1(x0, x1); }

// Timeline instrumentation, compiled only into the diagnostic library that
// message_fp16_all_amd/timeline.py builds with -DHR_TIMELINE: lane 0 of
// every workgroup keeps wall-clock stamps of its protocol phases and writes
// them, with its poll count, to record ((e - 1) mod calls, rank, workgroup)
// of a device buffer the tool attaches.  In the library itself HR_NOW() is a
// constant and tl_record is empty, so none of it is compiled in.
#ifdef HR_TIMELINE
constexpr int kTimelineWords = 8;  // stamps t0..t5, count, call number
__device__ uint64_t *hr_tl_buf;
__device__ uint64_t hr_tl_calls;
#define HR_NOW() static_cast<uint64_t>(wall_clock64())
#define HR_COUNT(x) (++(x))
#else
#define HR_NOW() uint64_t(0)
#define HR_COUNT(x) ((void)0)
#endif

__device__ __forceinline__ void tl_record(const ExchArgs &a, int b, uint64_t e, uint64_t t0, uint64_t t1,
                                          uint64_t t2, uint64_t t3, uint64_t t4, uint64_t t5, uint64_t count) {
#ifdef HR_TIMELINE
    if (threadIdx.x != 0 || hr_tl_buf == nullptr || hr_tl_calls == 0) return;
    const size_t rec = static_cast<size_t>((e - 1) % hr_tl_calls) * a.world * a.nblocks +
                       static_cast<size_t>(a.rank) * a.nblocks + static_cast<size_t>(b);
    uint64_t *p = hr_tl_buf + rec * kTimelineWords;
    p[0] = t0; p[1] = t1; p[2] = t2; p[3] = t3; p[4] = t4; p[5] = t5; p[6] = count; p[7] = e;
#else
    (void)a; (void)b; (void)e; (void)t0; (void)t1; (void)t2; (void)t3; (void)t4; (void)t5; (void)count;
#endif
}

// The combine takes one 16-byte unit per lane per step (W loads in flight
// per lane).  Reads of host memory lose rate when too many are in flight at
// once: measured on MI355X with two ranks, 16 MiB per rank, four units per
// lane per step took 805 us per call and one unit 781 us; 256 KiB calls (one
// unit per lane in all) are unchanged.

// Host-slot accesses are buffer loads/stores with the system-coherence bits
// (sc0 sc1): stores write through every GPU cache level to host memory and
// loads fetch from it, so the exchange needs no cache write-back or
// invalidate (which a system-scope fence would do for the whole L2).  The
// descriptor's third dword selects 32-bit data format for raw (untyped)
// access; num_records bounds every access to the slot.
constexpr int kSysCoherent = 1 | 16;                  // sc0 | sc1
constexpr int kRawBufferDword3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const uint16_t *base, size_t values) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0,
                                             static_cast<int>(values * sizeof(uint16_t)), kRawBufferDword3);
}

template <typename T>
struct HostIO;

template <>
struct HostIO<u32x4> {
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, size_t unit, u32x4 v) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(unit * 16), 0, kSysCoherent);
    }
    static __device__ __forceinline__ u32x4 load(__amdgpu_buffer_rsrc_t r, size_t unit) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(unit * 16), 0, kSysCoherent);
    }
};

template <>
struct HostIO<uint16_t> {
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, size_t unit, uint16_t v) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, static_cast<int>(unit * 2), 0, kSysCoherent);
    }
    static __device__ __forceinline__ uint16_t load(__amdgpu_buffer_rsrc_t r, size_t unit) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(unit * 2), 0, kSysCoherent);
    }
};

// True when a wait that has lasted `waited` ticks should end because the
// host raised the abort word.  Waits shorter than abort_after_ticks do not
// look: every waiting wave reading the same host line on every poll slows
// the flags themselves (measured: 17.9 -> 22.7 us per 256 KiB call), and
// flags normally arrive within microseconds.  Called by the whole wave; the
// result is the same in every lane.
__device__ __forceinline__ bool aborted(const ExchArgs &a, uint64_t waited) {
    if (waited <= a.abort_after_ticks) return false;
    uint32_t ab = 0;
    if ((threadIdx.x % 64) == 0) ab = __hip_atomic_load(a.abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return __shfl(ab, 0) != 0;
}

// After a wait timed out: the channel's timeout record takes the peers whose
// signal the wait was still missing (bit q = rank q), this rank and the call
// number's low 48 bits, packed into one 64-bit word written by one
// system-scope store, so the host never reads a mix of two records.  Several
// workgroups may time out on one call; the last record stays.
__device__ __forceinline__ void record_missing(const ExchArgs &a, uint64_t e, unsigned missing) {
    if (a.diag == nullptr) return;
    const uint64_t w = (e << 16) | (static_cast<uint64_t>(a.rank & 0xFF) << 8) | (missing & 0xFFu);
    __hip_atomic_store(a.diag, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Wait, in the first wave, until flag[q][b] >= e for every rank q whose bit
// is set in `mask` (one lane per rank, wrap-safe compare), or the abort word
// is set, or the watchdog expires.  Returns 0, HR_ERR_ABORTED or
// HR_ERR_TIMEOUT, the same in every lane of the wave; lane 0 records an
// error in both error words and, when `record` is set (the waits for peers'
// publishes, not the two-shot's wait for a shard owner, which only follows
// from a missing publish), which peers' flags never arrived.
__device__ __forceinline__ uint32_t wait_flags(const ExchArgs &a, const uint64_t *flag_base, int b, uint64_t e,
                                               unsigned mask, bool record = true) {
    const int lane = threadIdx.x;
    const bool polls = lane < kMaxWorld && ((mask >> lane) & 1u);
    const uint64_t *pf = flag_base + (static_cast<size_t>(polls ? lane : 0) * a.nblocks + b) * kFlagStride;
    bool done = !polls;
    uint32_t status = 0;
    const long long t0 = wall_clock64();
    for (;;) {
        if (!done) {
            const uint64_t f = __hip_atomic_load(pf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            done = static_cast<int64_t>(f - e) >= 0;
        }
        if (__all(done)) break;
        const uint64_t waited = static_cast<uint64_t>(wall_clock64() - t0);
        if (waited > a.timeout_ticks) {
            status = HR_ERR_TIMEOUT;
            break;
        }
        if (aborted(a, waited)) {
            status = HR_ERR_ABORTED;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (status == HR_ERR_TIMEOUT && record) {
        const unsigned missing = static_cast<unsigned>(__ballot(polls && !done));  // lane q polls rank q
        if (lane == 0) record_missing(a, e, missing);
    }
    if (lane == 0 && status != 0) {
        __hip_atomic_store(a.dev_error, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.host_error, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return status;
}

// Call numbers run 1, 2, 3, ... and skip every value whose low 32 bits are
// zero (two values at a time, so the parity keeps alternating).  They are
// 64-bit, so a flag that a workgroup has not raised for any number of calls
// still compares below the current call; and the low 32 bits, which the
// low-latency words carry, are never zero, so a word never written (zero)
// is never taken for a current one.
__device__ __forceinline__ uint64_t next_call_number(uint64_t prev) {
    const uint64_t e = prev + 1u;
    return static_cast<uint32_t>(e) == 0u ? e + 2u : e;
}

// Pacing of the publish: workgroup b > kPaceBurst starts b - kPaceBurst
// slices after the first ones (the ranks' workgroups b start together), a
// slice taking `slice_bytes` (one workgroup's publish summed over the ranks
// that share the host link) at the channel's link rate.  The link carries
// requests in order, so without pacing every flag and every read request
// queues behind all of the call's slot writes; paced, the queue stays
// short, each workgroup's handshake completes early and the reads of early
// slices overlap the writes of later ones.  The first burst + 1 workgroups
// start together: the link is idle when a call starts, and writes reach its
// rate only with a few slices in flight.  A one-shot call whose workgroups
// each carry at most one unit per lane starts five together (kPaceBurstSmall),
// others three (kPaceBurst).  Measured on MI355X, two ranks on loopback,
// graph-captured, on two boxes, burst 2 / 4: 256 KiB 16.59-16.66 /
// 16.49-16.50 us, 64 KiB 8.44-8.53 / 8.20-8.28 us; but 16 MiB per rank
// 723 / 781-841 us, and the group two-shot at W = 4 and 8 ranks 1-1.5 us
// slower with 4: their slices are larger, and a wider burst fills the
// link's request queue.
constexpr int kPaceBurst = 2;
constexpr int kPaceBurstSmall = 4;

__device__ __forceinline__ void pace(const ExchArgs &a, int b, uint64_t slice_bytes, int burst = kPaceBurst) {
    if (a.pace_q16 == 0 || b <= burst) return;
    const uint64_t wait = (static_cast<uint64_t>(b - burst) * slice_bytes * a.pace_q16) >> 16;
    const long long t0 = wall_clock64();
    while (static_cast<uint64_t>(wall_clock64() - t0) < wait) __builtin_amdgcn_s_sleep(1);
}

// Advance this workgroup's call counter (every launched workgroup does, so a
// rank's workgroups agree on the slot parity); returns the call number e, or
// 0 when the channel already holds an error.
// With commit false the caller stores the new number itself, later, with
// commit_call: only workgroup b of this rank touches epochs[b], and the next
// call on the rank starts after this kernel has ended, so the store may come
// anywhere before the workgroup ends.
__device__ __forceinline__ uint64_t next_call(const ExchArgs &a, int b, bool commit = true) {
    __shared__ uint64_t s_epoch;
    if (threadIdx.x == 0) {
        const uint32_t err = __hip_atomic_load(a.dev_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t e =
            next_call_number(__hip_atomic_load(&a.epochs[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (err == 0 && commit) __hip_atomic_store(&a.epochs[b], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_epoch = err == 0 ? e : 0u;
    }
    __syncthreads();
    return s_epoch;
}

__device__ __forceinline__ void commit_call(const ExchArgs &a, int b, uint64_t e) {
    if (threadIdx.x == 0) __hip_atomic_store(&a.epochs[b], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Low-latency words carry a 16-bit call field: the call number's low 15
// bits with the top bit set, so it is never zero.  A word left in a slot
// 2^15 call numbers earlier would look current, so each parity of a rank's
// own LL slot is cleared once every 2^14 call numbers: at calls whose low 14
// bits are 2 (even parity) or 3 (odd parity) -- the second and third calls
// of a channel, and then every 2^14 -- every launched workgroup of the rank
// zeroes its share of slot[e & 1][rank], except the first `keep` units,
// which an LL call e writes itself.  A reader at LL call e then finds in a
// peer's slot only zeros (no call field is zero) or words of calls in [c, e],
// c the peer's last clearing of that parity before e, which finished before
// e started (as in the parity argument above) and is less than 2^15 call
// numbers earlier, so no word of a call other than e carries e's call field.
// Nobody reads the slot meanwhile: peers at call c read only units below
// keep, and every peer finished its call c - 2 before this rank started call
// c.  A clearing call stores at most the slot (3 x 8 bytes per unit) once
// more; at one call in 2^14 that costs nothing measurable.
__device__ __forceinline__ bool ll_clear_due(uint64_t e) {
    const uint32_t l = static_cast<uint32_t>(e) & 0x3FFFu;
    return l == 2u || l == 3u;
}

__device__ __forceinline__ void ll_clear(const ExchArgs &a, int b, uint64_t e, size_t keep) {
    const size_t plane = a.ll_stride / 3;  // units per slot
    if (keep >= plane) return;
    const size_t n = plane - keep;
    const size_t lo = keep + n * static_cast<size_t>(b) / static_cast<size_t>(a.nblocks);
    const size_t hi = keep + n * static_cast<size_t>(b + 1) / static_cast<size_t>(a.nblocks);
    const int parity = static_cast<int>(e & 1u);
    uint64_t *mine = a.ll + static_cast<size_t>(a.world * parity + a.rank) * a.ll_stride;
    for (size_t u = lo + threadIdx.x; u < hi; u += kExchThreads) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            __hip_atomic_store(mine + k * plane + u, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // settle the zeros on this rare path, so that the common path does not
    // inherit a wait for them (see the low-latency kernel's publish)
    __builtin_amdgcn_s_waitcnt(0);
}

// Loads and stores share one counter on this GPU (vmcnt), and the compiler
// cannot wait for a load with a partial count once a store is outstanding
// too, so in these bounds-checked batch loops each host store waits for the
// one before it: a lane has one publish store in flight at a time.  Letting
// a batch's stores go out together (one explicit wait after its loads) was
// measured slower on MI355X for calls of several batches per lane (4 MiB
// per rank, two ranks: 183.6 -> 186.2 us; four ranks, 2 MiB: 313 -> 321
// us): with pacing in place, the extra writes in flight only queue on the
// link.

// Publish batches: lane units v0, v0 + kExchThreads, ... (kExchUnroll of
// them, those below `end`) loaded from `in`, then stored to a host slot.
template <typename T>
__device__ __forceinline__ void load_batch(const T *in, size_t v0, size_t end, bool active, T (&x)[kExchUnroll]) {
#pragma unroll
    for (int u = 0; u < kExchUnroll; ++u) {
        const size_t v = v0 + static_cast<size_t>(u) * kExchThreads;
        if (active && v < end) x[u] = in[v];
    }
}

template <typename T>
__device__ __forceinline__ void store_batch(__amdgpu_buffer_rsrc_t slot, size_t v0, size_t end,
                                            const T (&x)[kExchUnroll]) {
#pragma unroll
    for (int u = 0; u < kExchUnroll; ++u) {
        const size_t v = v0 + static_cast<size_t>(u) * kExchThreads;
        if (v < end) HostIO<T>::store(slot, v, x[u]);
    }
}

// Workgroup b of an active set of `nact` owns the 8-value units
// [nvec*b/nact, nvec*(b+1)/nact) of the call, nvec = numel / 8, and the last
// active workgroup also owns the numel % 8 trailing values.  The split
// depends on numel alone, so workgroup b covers the same values on every
// rank whichever access path (16-byte or 2-byte) each rank takes.
//
// W is the group size; VEC selects the lane access unit: one 16-byte unit
// (all buffers 16-byte aligned) or one value (2-byte aligned buffers); E is
// the element type (binary16 or bfloat16).
template <int W, bool VEC, class E>
__device__ __forceinline__ void exchange_body(const ExchArgs &a, const int b) {
    __shared__ uint32_t s_status;
    const int tid = threadIdx.x;
    const bool active = b < a.nactive;

    const size_t nvec = a.numel / kVecElems;
    const size_t lo = nvec * static_cast<size_t>(b) / static_cast<size_t>(a.nactive);
    const size_t hi = nvec * static_cast<size_t>(b + 1) / static_cast<size_t>(a.nactive);
    const bool last = (b == a.nactive - 1);
    const size_t tail0 = nvec * kVecElems;  // first value not covered by whole units

    typedef typename std::conditional<VEC, u32x4, uint16_t>::type T;
    constexpr size_t per = VEC ? kVecElems : 1;  // values per lane access
    const size_t ulo = lo * (kVecElems / per), uhi = hi * (kVecElems / per);
    const T *in = static_cast<const T *>(a.in);
    T *out = static_cast<T *>(a.out);

    // the first batch of this lane's values is loaded before the call
    // counter and the pacing wait, so its HBM latency overlaps them
    constexpr size_t kBatch = static_cast<size_t>(kExchThreads) * kExchUnroll;
    const uint64_t tl0 = HR_NOW();
    T x[kExchUnroll];
    load_batch<T>(in, ulo + tid, uhi, active, x);

    const uint64_t e = next_call(a, b);
    if (e == 0) return;
    if (ll_clear_due(e)) ll_clear(a, b, e, 0);
    if (!active) return;
    const uint64_t tl1 = HR_NOW();
    const int parity = static_cast<int>(e & 1u);
    const int rank = a.rank;
    __amdgpu_buffer_rsrc_t slot[W];
#pragma unroll
    for (int q = 0; q < W; ++q)
        slot[q] = slot_rsrc(a.slots + static_cast<size_t>(W * parity + q) * a.stride, a.stride);

    // 1. publish this rank's slice into its host slot (write-through),
    //    paced so that each workgroup's handshake and reads start early
    // one unit per lane in every workgroup: the decode sizes (the split
    // depends on numel alone, so every rank paces alike)
    const bool small_slices = nvec <= static_cast<size_t>(a.nactive) * kExchThreads;
    pace(a, b, (hi - lo) * 16u * W, small_slices ? kPaceBurstSmall : kPaceBurst);
    const uint64_t tl2 = HR_NOW();
    for (size_t v0 = ulo + tid;;) {
        store_batch<T>(slot[rank], v0, uhi, x);
        v0 += kBatch;
        if (v0 >= uhi) break;
        load_batch<T>(in, v0, uhi, true, x);
    }
    if (last && tail0 + tid < a.numel)
        HostIO<uint16_t>::store(slot[rank], tail0 + tid, static_cast<const uint16_t *>(a.in)[tail0 + tid]);

    // 2. every lane waits until its slot stores are acknowledged, so they
    //    are in host memory before lane 0 raises the flag
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        __hip_atomic_store(a.flags + (static_cast<size_t>(rank) * a.nblocks + b) * kFlagStride, e,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t tl3 = HR_NOW();

    // 3. the first wave waits for every peer's flag, one lane per peer
    if (tid < 64) {
        const uint32_t st = wait_flags(a, a.flags, b, e, ((1u << W) - 1u) & ~(1u << rank));
        if (tid == 0) s_status = st;
    }
    // the barrier orders every lane's slot loads after the flags the first
    // wave saw; the loads themselves read host memory, not a cached copy
    __syncthreads();
    if (s_status != 0) return;
    const uint64_t tl4 = HR_NOW();

    // 4. combine: left fold in rank order x0 + x1 + ... + x_{W-1}; when the
    //    slice gave every lane at most one unit, the lane's own unit is
    //    still in x[0] from the publish and is not read from `in` again
    const bool one_unit = uhi - ulo <= static_cast<size_t>(kExchThreads);
    for (size_t v = ulo + tid; v < uhi; v += kExchThreads) {
        T xs[W];
#pragma unroll
        for (int q = 0; q < W; ++q)  // every peer's load issued before any is used
            if (q != rank) xs[q] = HostIO<T>::load(slot[q], v);
        const T own = one_unit ? x[0] : in[v];
        T acc = rank == 0 ? own : xs[0];
#pragma unroll
        for (int q = 1; q < W; ++q) acc = combine<E>(acc, q == rank ? own : xs[q]);
        out[v] = acc;
    }
    if (last && tail0 + tid < a.numel) {
        const size_t i = tail0 + tid;
        uint16_t acc = 0;
#pragma unroll
        for (int q = 0; q < W; ++q) {
            const uint16_t xq = (q == rank) ? static_cast<const uint16_t *>(a.in)[i] : HostIO<uint16_t>::load(slot[q], i);
            acc = (q == 0) ? xq : E::add1(acc, xq);
        }
        static_cast<uint16_t *>(a.out)[i] = acc;
    }
    // timeline: entry, counter, pace done, flag raised, peers seen, combined
    tl_record(a, b, e, tl0, tl1, tl2, tl3, tl4, HR_NOW(), 0);
}

// Two-shot variant for larger payloads and groups: the active workgroups
// form W groups of m; group s covers shard s (the 8-value units
// [nvec*s/W, nvec*(s+1)/W), split into m contiguous sub-slices), so
// workgroup b covers the same values on every rank.
//   A. every workgroup publishes its own values of its sub-slice to
//      slot[e & 1][rank] and raises flag[rank][b] = e;
//   B. the workgroups of group `rank` wait for flag[q][b] of every peer q,
//      fold the sub-slice left in rank order (own values from `in`), store
//      the result to `out` and to the reduced slot red[e & 1], and raise
//      flag2[rank][b] = e;
//   C. the workgroups of every other group s wait for flag2[s][b] (rank
//      s's fold of the same sub-slice) and copy it from red[e & 1] to `out`.
// Every value is folded once, by its shard's owner, in the same order as the
// one-shot fold, so both algorithms produce the same bits.  Host-link
// traffic per rank: (1 + 1/W) N values written, 2 (W-1)/W N read, against N
// and (W-1) N for the one-shot.  Parity safety: in call e + 1 the owner
// workgroups of a rank waited for every peer's publish flag of call e + 1,
// so every peer had finished call e, including its reads of slot and
// reduced-slot parity e & 1, before the rank starts call e + 2.
template <int W, bool VEC, class E>
__device__ __forceinline__ void exchange2_body(const ExchArgs &a, const int b) {
    __shared__ uint32_t s_status;
    const int tid = threadIdx.x;
    const bool active = b < a.nactive;
    const int m = a.nactive / W;               // workgroups per shard
    const int shard = b / m, j = b % m;

    const size_t nvec = a.numel / kVecElems;
    const size_t sh_lo = nvec * static_cast<size_t>(shard) / W;
    const size_t sh_hi = nvec * static_cast<size_t>(shard + 1) / W;
    const size_t lo = sh_lo + (sh_hi - sh_lo) * static_cast<size_t>(j) / static_cast<size_t>(m);
    const size_t hi = sh_lo + (sh_hi - sh_lo) * static_cast<size_t>(j + 1) / static_cast<size_t>(m);
    const bool last = (b == a.nactive - 1);    // shard W-1, last sub-slice: owns the tail
    const size_t tail0 = nvec * kVecElems;

    typedef typename std::conditional<VEC, u32x4, uint16_t>::type T;
    constexpr size_t per = VEC ? kVecElems : 1;
    const size_t ulo = lo * (kVecElems / per), uhi = hi * (kVecElems / per);
    const T *in = static_cast<const T *>(a.in);
    T *out = static_cast<T *>(a.out);

    // first publish batch loaded ahead, as in the one-shot
    constexpr size_t kBatch = static_cast<size_t>(kExchThreads) * kExchUnroll;
    const uint64_t tl0 = HR_NOW();
    T x[kExchUnroll];
    load_batch<T>(in, ulo + tid, uhi, active, x);

    const uint64_t e = next_call(a, b);
    if (e == 0) return;
    if (ll_clear_due(e)) ll_clear(a, b, e, 0);
    if (!active) return;
    const uint64_t tl1 = HR_NOW();
    const int parity = static_cast<int>(e & 1u);
    const int rank = a.rank;
    __amdgpu_buffer_rsrc_t slot[W];
#pragma unroll
    for (int q = 0; q < W; ++q)
        slot[q] = slot_rsrc(a.slots + static_cast<size_t>(W * parity + q) * a.stride, a.stride);
    const __amdgpu_buffer_rsrc_t red = slot_rsrc(a.reduced + static_cast<size_t>(parity) * a.stride, a.stride);

    // A. publish (paced as the one-shot's)
    pace(a, b, (hi - lo) * 16u * W);
    const uint64_t tl2 = HR_NOW();
    for (size_t v0 = ulo + tid;;) {
        store_batch<T>(slot[rank], v0, uhi, x);
        v0 += kBatch;
        if (v0 >= uhi) break;
        load_batch<T>(in, v0, uhi, true, x);
    }
    if (last && tail0 + tid < a.numel)
        HostIO<uint16_t>::store(slot[rank], tail0 + tid, static_cast<const uint16_t *>(a.in)[tail0 + tid]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        __hip_atomic_store(a.flags + (static_cast<size_t>(rank) * a.nblocks + b) * kFlagStride, e,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t tl3 = HR_NOW();

    if (shard == rank) {
        // B. fold this rank's shard
        if (tid < 64) {
            const uint32_t st = wait_flags(a, a.flags, b, e, ((1u << W) - 1u) & ~(1u << rank));
            if (tid == 0) s_status = st;
        }
        __syncthreads();
        if (s_status != 0) return;
        const uint64_t tl4 = HR_NOW();
        const bool one_unit = uhi - ulo <= static_cast<size_t>(kExchThreads);  // own unit still in x[0]
        for (size_t v = ulo + tid; v < uhi; v += kExchThreads) {
            T xs[W];
#pragma unroll
            for (int q = 0; q < W; ++q)
                if (q != rank) xs[q] = HostIO<T>::load(slot[q], v);
            const T own = one_unit ? x[0] : in[v];
            T acc = rank == 0 ? own : xs[0];
#pragma unroll
            for (int q = 1; q < W; ++q) acc = combine<E>(acc, q == rank ? own : xs[q]);
            out[v] = acc;
            HostIO<T>::store(red, v, acc);
        }
        if (last && tail0 + tid < a.numel) {
            const size_t i = tail0 + tid;
            uint16_t acc = 0;
#pragma unroll
            for (int q = 0; q < W; ++q) {
                const uint16_t xq =
                    (q == rank) ? static_cast<const uint16_t *>(a.in)[i] : HostIO<uint16_t>::load(slot[q], i);
                acc = (q == 0) ? xq : E::add1(acc, xq);
            }
            static_cast<uint16_t *>(a.out)[i] = acc;
            HostIO<uint16_t>::store(red, i, acc);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(a.flags2 + (static_cast<size_t>(rank) * a.nblocks + b) * kFlagStride, e,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        // timeline: entry, counter, pace done, flag raised, peers seen, shard
        // published with flag 2; role 1 (the shard's owner)
        tl_record(a, b, e, tl0, tl1, tl2, tl3, tl4, HR_NOW(), 1);
    } else {
        // C. gather shard `shard` from its owner
        if (tid < 64) {
            const uint32_t st = wait_flags(a, a.flags2, b, e, 1u << shard, false);
            if (tid == 0) s_status = st;
        }
        __syncthreads();
        if (s_status != 0) return;
        const uint64_t tl4 = HR_NOW();
        for (size_t v0 = ulo + tid; v0 < uhi; v0 += static_cast<size_t>(kExchThreads) * kExchUnroll) {
            T x[kExchUnroll];
#pragma unroll
            for (int u = 0; u < kExchUnroll; ++u) {
                const size_t v = v0 + static_cast<size_t>(u) * kExchThreads;
                if (v < uhi) x[u] = HostIO<T>::load(red, v);
            }
#pragma unroll
            for (int u = 0; u < kExchUnroll; ++u) {
                const size_t v = v0 + static_cast<size_t>(u) * kExchThreads;
                if (v < uhi) out[v] = x[u];
            }
        }
        if (last && tail0 + tid < a.numel)
            static_cast<uint16_t *>(a.out)[tail0 + tid] = HostIO<uint16_t>::load(red, tail0 + tid);
        // timeline: entry, counter, pace done, flag raised, owner's flag 2
        // seen, shard copied; role 2 (a gathering rank)
        tl_record(a, b, e, tl0, tl1, tl2, tl3, tl4, HR_NOW(), 2);
    }
}

// Low-latency variant for small calls.  The one-shot's handshake costs two
// host-link round trips beyond the data itself: a workgroup must see its
// slot stores acknowledged before it raises its flag, and a peer must see
// the flag before it may read the slot.  Here the data carries its own
// readiness, in the manner of the low-latency protocol of NCCL and RCCL:
// every 8-byte word written to host memory holds 6 bytes of values and a
// 16-bit call field, so a reader that finds the call's field in a word also
// holds that word's values.  Every word is written and read as one naturally
// aligned 64-bit relaxed system-scope atomic, whose single-copy atomicity is
// what makes a word never seen half written.  There is no flag, no
// acknowledgement wait and no separate read; the price is 3/2 of the bytes
// on the link (three words for a unit of 8 values, the last word holding
// two), which is why only small calls take this path.
//
// Layout: LL slot [e & 1][q] holds three planes of ll_stride / 3 words; for
// each 8-value unit u of the call (x = {v0v1, v2v3, v4v5, v6v7}), word u of
// plane 0 is v0 v1 v2, of plane 1 v3 v4 v5, of plane 2 v6 v7 and a zero
// value, each with the call field in its top 16 bits; the last unit's
// missing values are zero.  Each store and load instruction covers 64
// consecutive words of one plane (whole lines; an interleaved layout makes
// partial-line writes to host memory, which the link carries at a small
// fraction of its rate).  One unit per lane: active workgroup b owns the
// units [nunits*b/nact, nunits*(b+1)/nact).  Each lane publishes its unit,
// then polls the three words of that unit in every peer's slot (all peers at
// once) until every word carries the call's field; after a barrier the
// workgroup folds left in rank order and stores, or, if any lane of it timed
// out or saw an abort, stores nothing.  No word of an earlier call carries
// the call's field (see ll_clear); parity safety is the one-shot's argument,
// with "flag" read as "word".
__device__ __forceinline__ uint64_t ll_field(uint64_t e) {
    return static_cast<uint64_t>((static_cast<uint32_t>(e) & 0x7FFFu) | 0x8000u) << 48;
}
__device__ __forceinline__ uint64_t ll_word0(u32x4 x) { return x.x | (static_cast<uint64_t>(x.y & 0xFFFFu) << 32); }
__device__ __forceinline__ uint64_t ll_word1(u32x4 x) { return (x.y >> 16) | (static_cast<uint64_t>(x.z) << 16); }
__device__ __forceinline__ uint64_t ll_word2(u32x4 x) { return x.w; }
__device__ __forceinline__ u32x4 ll_unpack(uint64_t w0, uint64_t w1, uint64_t w2) {
    u32x4 x;
    x.x = static_cast<uint32_t>(w0);
    x.y = (static_cast<uint32_t>(w0 >> 32) & 0xFFFFu) | (static_cast<uint32_t>(w1) << 16);
    x.z = static_cast<uint32_t>(w1 >> 16);
    x.w = static_cast<uint32_t>(w2);
    return x;
}
constexpr size_t kLLMaxNumel = 32768;      // values per call the LL slots hold

// 8-byte words per LL slot of a channel of max_numel values: three planes
// of one word per 8-value unit, each plane a whole number of 128-byte lines.
inline size_t ll_stride_for(size_t max_numel) {
    const size_t ll_max = max_numel < kLLMaxNumel ? max_numel : kLLMaxNumel;
    const size_t units = (ll_max + kVecElems - 1) / kVecElems;
    const size_t per_line = kLine / sizeof(uint64_t);
    return 3 * ((units + per_line - 1) / per_line * per_line);
}
// Largest call the automatic choice gives LL: its extra bytes (3/2) and its
// readers polling every peer's data cost more as the group grows.  Measured
// on MI355X, graph-captured (two ranks on two loopback streams, larger groups
// in one group launch), as the largest size at which LL beat the one-shot on
// two boxes: W = 2 20480, W = 3 8192, W = 4 4096, W = 5 4096, W = 6 2560,
// W = 7 2048, W = 8 1536 (e.g. W = 2 at 20480 values 7.1-7.3 against
// 7.4-7.5 us and at 24576 8.1-8.2 against 7.6-7.7; W = 3 at 8192 7.6 against
// 8.2 and at 10240 8.5 against 8.3; W = 5 at 4096 9.5 against 9.6; W = 6 at
// 2560 8.9 against 8.9-9.0 and at 3072 9.8 against 9.4-9.5; W = 8 at 1536
// 9.3 against 9.6-9.8 and at 2048 11.1-11.2 against 10.6-10.7).
inline size_t ll_auto_max_numel(int world) {
    switch (world) {
        case 2: return 20480;
        case 3: return 8192;
        case 4: return 4096;
        case 5: return 4096;
        case 6: return 2560;
        case 7: return 2048;
        default: return 1536;
    }
}
// A lane does not wait for its own words' acknowledgement before polling,
// and it sleeps only briefly between polls.  Measured on MI355X, two ranks
// in loopback, graph-captured, against waiting for the acknowledgement and
// sleeping 8 x 64 clocks: 4096 values 4.98-5.41 -> 4.86-4.91 us, 12288
// values 6.59-7.02 -> 6.20-6.27 us.  The polls read host memory, so a lane
// has at most one in flight and the round trip, not the sleep, sets the
// polling rate.
constexpr int kLLSleep = 1;                // s_sleep after a failed poll (x 64 clocks)

template <int W, bool VEC, class E>
__device__ __forceinline__ void exchange_ll_body(const ExchArgs &a, const int b) {
    __shared__ uint32_t s_status;
    const int tid = static_cast<int>(threadIdx.x);
    if (tid == 0) s_status = 0;
    const bool active = b < a.nactive;
    const size_t nunits = (a.numel + kVecElems - 1) / kVecElems;
    const size_t nvec = a.numel / kVecElems;
    const size_t lo = nunits * static_cast<size_t>(b) / static_cast<size_t>(a.nactive);
    const size_t hi = nunits * static_cast<size_t>(b + 1) / static_cast<size_t>(a.nactive);
    const size_t u = lo + static_cast<size_t>(tid);
    const bool has = active && u < hi;
    const uint16_t *in16 = static_cast<const uint16_t *>(a.in);
    const uint64_t tl0 = HR_NOW();

    // this lane's unit of `in` (zero past numel), loaded before the call
    // counter so that its HBM latency overlaps the counter's
    u32x4 x = {0u, 0u, 0u, 0u};
    if (has) {
        if (VEC && u < nvec) {
            x = static_cast<const u32x4 *>(a.in)[u];
        } else {
#pragma unroll
            for (int k = 0; k < kVecElems; ++k) {
                const size_t i = u * kVecElems + static_cast<size_t>(k);
                const uint32_t v = i < a.numel ? in16[i] : 0u;
                x[k / 2] |= v << (16 * (k % 2));
            }
        }
    }

    // the counter's store is deferred to after the polling (see the publish)
    const uint64_t e64 = next_call(a, b, false);  // its barrier also orders s_status's reset
    if (e64 == 0) return;
    if (ll_clear_due(e64)) ll_clear(a, b, e64, nunits);
    if (!active) {
        commit_call(a, b, e64);
        return;
    }
    const uint64_t tl1 = HR_NOW();
    const uint64_t field = ll_field(e64);
    const int parity = static_cast<int>(e64 & 1u);
    const int rank = a.rank;
    const size_t plane = a.ll_stride / 3;
    const uint64_t *slot0 = a.ll + static_cast<size_t>(W * parity) * a.ll_stride + u;  // rank 0's word 0 of unit u

    // publish: the unit's three words, relaxed 64-bit system-scope stores, no
    // wait.  On this GPU vmcnt counts stores as well as loads, and the
    // compiler waits for every outstanding access before it reuses a
    // register that an outstanding store reads; a reuse between here and the
    // first poll would make every lane wait for its words' acknowledgement
    // (a host-link round trip) before polling.  So the store operands stay
    // live until after the polling (the empty asm below), and the call
    // counter's own store comes after it too.
    uint64_t *const m0 = a.ll + static_cast<size_t>(W * parity + rank) * a.ll_stride + u;
    uint64_t *const m1 = m0 + plane, *const m2 = m0 + 2 * plane;
    const uint64_t s0 = ll_word0(x) | field, s1 = ll_word1(x) | field, s2 = ll_word2(x) | field;
    if (has) {
        __hip_atomic_store(m0, s0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(m1, s1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(m2, s2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    const uint64_t tl2 = HR_NOW();

    // hold the first poll until the call's words have nearly drained from
    // the host link: a read does not pass the writes issued before it, and
    // one that reaches host memory before the peer's words costs a second
    // round trip.  The link carries all W ranks' words (24 bytes per unit)
    // at the channel's pacing rate; the poll leaves ll_lead_ticks early, the
    // time its request takes to reach host memory.
    // Ranks launched separately start their calls up to about a microsecond
    // apart, and a short hold lets them fall into a cycle: the rank that
    // starts first polls too early, pays a second round trip, ends last and
    // so starts the next call last, when its peer repeats the mistake.  The
    // floor on the hold (ll_floor_ticks, zero for a group launch, whose ranks
    // start together) gives the first poll room for that skew.  Measured on
    // MI355X, two ranks at 4096 values, graph-captured: 4.48-4.55 us per
    // call without the floor (5.97 once), 4.25-4.36 us with 450 ns, and
    // 4.38-4.45 us with 300 or 600 ns.  Without the floor the skews of
    // consecutive calls correlated at -0.55 to -0.85 and the last lane to
    // finish polled twice in 76-97 % of the calls; with 450 ns its poll
    // phase fell from 3.0 to 2.2 us (median).
    if (has && a.pace_q16 != 0) {
        const uint64_t drain = (static_cast<uint64_t>(W) * nunits * 24u * a.pace_q16) >> 16;
        uint64_t hold = drain > a.ll_lead_ticks ? drain - a.ll_lead_ticks : 0u;
        if (hold < a.ll_floor_ticks) hold = a.ll_floor_ticks;
        if (hold != 0u) {
            const long long tw = wall_clock64();
            while (static_cast<uint64_t>(wall_clock64() - tw) < hold) __builtin_amdgcn_s_sleep(1);
        }
    }

    // gather: poll every pending peer's three words until all carry the field
    u32x4 got[W];
    unsigned pending = has ? (((1u << W) - 1u) & ~(1u << rank)) : 0u;
    uint32_t status = 0;
    uint32_t polls = 0;
    const long long t0 = wall_clock64();
    for (;;) {
        HR_COUNT(polls);
        // all pending peers' loads in flight at once
        uint64_t w0[W], w1[W], w2[W];
#pragma unroll
        for (int q = 0; q < W; ++q) {
            if ((pending >> q) & 1u) {
                const uint64_t *p = slot0 + static_cast<size_t>(q) * a.ll_stride;
                w0[q] = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                w1[q] = __hip_atomic_load(p + plane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                w2[q] = __hip_atomic_load(p + 2 * plane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
#pragma unroll
        for (int q = 0; q < W; ++q) {
            if (((pending >> q) & 1u) && ((w0[q] ^ field) >> 48) == 0 && ((w1[q] ^ field) >> 48) == 0 &&
                ((w2[q] ^ field) >> 48) == 0) {
                got[q] = ll_unpack(w0[q], w1[q], w2[q]);
                pending &= ~(1u << q);
            }
        }
        if (!__any(pending != 0u)) break;
        const uint64_t waited = static_cast<uint64_t>(wall_clock64() - t0);
        if (waited > a.timeout_ticks) {
            status = HR_ERR_TIMEOUT;
            break;
        }
        if (aborted(a, waited)) {
            status = HR_ERR_ABORTED;
            break;
        }
        __builtin_amdgcn_s_sleep(kLLSleep);
    }
    if (__any(status == HR_ERR_TIMEOUT)) {
        // the peers whose words some lane of this wave never saw
        unsigned missing = 0;
#pragma unroll
        for (int q = 0; q < W; ++q)
            if (__any((pending >> q) & 1u)) missing |= 1u << q;
        if (tid % 64 == 0) record_missing(a, e64, missing);
    }
    if (status != 0 && tid % 64 == 0) {
        __hip_atomic_store(&s_status, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_store(a.dev_error, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.host_error, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    asm volatile("" ::"v"(s0), "v"(s1), "v"(s2), "v"(m0), "v"(m1), "v"(m2));
    const uint64_t tl3 = HR_NOW();
    __syncthreads();
    commit_call(a, b, e64);
    if (s_status != 0 || !has) return;
    const uint64_t tl4 = HR_NOW();

    // left fold in rank order, own values from registers
    u32x4 acc = (rank == 0) ? x : got[0];
#pragma unroll
    for (int q = 1; q < W; ++q) acc = E::add8(acc, q == rank ? x : got[q]);
    if (VEC && u < nvec) {
        static_cast<u32x4 *>(a.out)[u] = acc;
    } else {
        uint16_t *out16 = static_cast<uint16_t *>(a.out);
#pragma unroll
        for (int k = 0; k < kVecElems; ++k) {
            const size_t i = u * kVecElems + static_cast<size_t>(k);
            if (i < a.numel) out16[i] = static_cast<uint16_t>(acc[k / 2] >> (16 * (k % 2)));
        }
    }
    // timeline: entry, counter, words issued, lane 0's words seen, workgroup's
    // words seen, stored; lane 0's polls
    tl_record(a, b, e64, tl0, tl1, tl2, tl3, tl4, HR_NOW(), polls);
}

// One launch per rank: workgroup b of the rank named in the arguments.  The
// arguments the kernel's first loads need (the input, the call counters and
// the error word, numel and the active workgroup count) come first, as five
// scalars, ahead of ExchArgs: the library is built to preload the first five
// kernel arguments, so those arrive in SGPRs when a wave starts and the
// input and call-counter loads issue without first waiting for a
// kernel-argument load.  (Measured on MI355X, two ranks on loopback,
// graph-captured, against the same kernels taking ExchArgs alone: the
// 1000-call decode graph at 10240 values 5.45-5.55 -> 5.24-5.43 us per call,
// 256 KiB 16.78-16.90 -> 16.73-16.75 us.)
__device__ __forceinline__ ExchArgs with_lead(ExchArgs a, const void *in, uint64_t *epochs, uint32_t *dev_error,
                                              size_t numel, int nactive) {
    a.in = in;
    a.epochs = epochs;
    a.dev_error = dev_error;
    a.numel = numel;
    a.nactive = nactive;
    return a;
}

template <int W, bool VEC, class E>
__global__ __launch_bounds__(kExchThreads) void exchange_k(const void *in, uint64_t *epochs, uint32_t *dev_error,
                                                           size_t numel, int nactive, ExchArgs a) {
    exchange_body<W, VEC, E>(with_lead(a, in, epochs, dev_error, numel, nactive), static_cast<int>(blockIdx.x));
}
template <int W, bool VEC, class E>
__global__ __launch_bounds__(kExchThreads) void exchange2_k(const void *in, uint64_t *epochs, uint32_t *dev_error,
                                                            size_t numel, int nactive, ExchArgs a) {
    exchange2_body<W, VEC, E>(with_lead(a, in, epochs, dev_error, numel, nactive), static_cast<int>(blockIdx.x));
}
template <int W, bool VEC, class E>
__global__ __launch_bounds__(kExchThreads) void exchange_ll_k(const void *in, uint64_t *epochs, uint32_t *dev_error,
                                                              size_t numel, int nactive, ExchArgs a) {
    exchange_ll_body<W, VEC, E>(with_lead(a, in, epochs, dev_error, numel, nactive), static_cast<int>(blockIdx.x));
}

// One launch for every rank of a loopback group: workgroups
// [r * nblocks, (r + 1) * nblocks) are rank r's workgroups 0 .. nblocks - 1,
// with rank r's buffers and call counters.  They run the same protocol
// through the same host slots and flags as W separate launches would; the
// grid (W * nblocks <= compute units) is resident at once, so no rank waits
// for a hardware queue to be scheduled.
struct GroupArgs {
    ExchArgs a;  // rank and buffers are per workgroup below
    const void *in[kMaxWorld];
    void *out[kMaxWorld];
};

__device__ __forceinline__ ExchArgs group_rank_args(const GroupArgs &g, int rank) {
    ExchArgs a = g.a;
    a.rank = rank;
    a.in = g.in[rank];
    a.out = g.out[rank];
    a.epochs = g.a.epochs + static_cast<size_t>(rank) * static_cast<size_t>(g.a.nblocks);
    return a;
}

template <int W, bool VEC, class E>
__global__ __launch_bounds__(kExchThreads) void exchange_group_k(GroupArgs g) {
    const int rank = static_cast<int>(blockIdx.x) / g.a.nblocks;
    exchange_body<W, VEC, E>(group_rank_args(g, rank), static_cast<int>(blockIdx.x) - rank * g.a.nblocks);
}
template <int W, bool VEC, class E>
__global__ __launch_bounds__(kExchThreads) void exchange2_group_k(GroupArgs g) {
    const int rank = static_cast<int>(blockIdx.x) / g.a.nblocks;
    exchange2_body<W, VEC, E>(group_rank_args(g, rank), static_cast<int>(blockIdx.x) - rank * g.a.nblocks);
}
template <int W, bool VEC, class E>
__global__ __launch_bounds__(kExchThreads) void exchange_ll_group_k(GroupArgs g) {
    const int rank = static_cast<int>(blockIdx.x) / g.a.nblocks;
    exchange_ll_body<W, VEC, E>(group_rank_args(g, rank), static_cast<int>(blockIdx.x) - rank * g.a.nblocks);
}

// Link calibration: workgroups [0, nw) store `units` 16-byte units of `src`
// to the host buffer `hw` while workgroups [nw, nw + nr) load `units` units
// of the host buffer `hrd` (four loads per lane in flight), which is how an
// exchange's publish and combine share the link; `sink` keeps the loads.
constexpr int kCalibReadUnroll = 4;

__global__ __launch_bounds__(kExchThreads) void link_probe_k(const u32x4 *src, u32x4 *hw, const u32x4 *hrd,
                                                             u32x4 *sink, int units, int nw, int nr) {
    const int b = blockIdx.x;
    const int tid = static_cast<int>(threadIdx.x);
    if (b < nw) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(hw, 0, units * 16, kRawBufferDword3);
        for (int u = b * kExchThreads + tid; u < units; u += nw * kExchThreads)
            __builtin_amdgcn_raw_buffer_store_b128(src[u], r, u * 16, 0, kSysCoherent);
        return;
    }
    const int rb = b - nw;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(hrd), 0, units * 16, kRawBufferDword3);
    const int step = nr * kExchThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int u0 = rb * kExchThreads + tid; u0 < units; u0 += step * kCalibReadUnroll) {
        u32x4 x[kCalibReadUnroll];
#pragma unroll
        for (int l = 0; l < kCalibReadUnroll; ++l) {
            const int u = u0 + l * step;
            x[l] = u < units ? __builtin_amdgcn_raw_buffer_load_b128(r, u * 16, 0, kSysCoherent) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int l = 0; l < kCalibReadUnroll; ++l) acc ^= x[l];
    }
    sink[rb * kExchThreads + tid] = acc;
}

// Active workgroups of an LL call: one unit per lane.
inline int active_blocks_ll(size_t numel) {
    const size_t nunits = (numel + kVecElems - 1) / kVecElems;
    const size_t want = (nunits + kExchThreads - 1) / kExchThreads;
    return static_cast<int>(want < 1 ? 1 : want);
}

// Active workgroups of a two-shot call: W groups of m, m about one 16-byte
// unit per lane of the shard, at least 1, at most nblocks / W.
inline int active_blocks2(size_t numel, int nblocks, int world) {
    const size_t nvec = numel / kVecElems;
    const size_t per_shard = (nvec + world - 1) / world;
    size_t m = (per_shard + kExchThreads - 1) / kExchThreads;
    if (m < 1) m = 1;
    const size_t mmax = static_cast<size_t>(nblocks / world);
    if (m > mmax) m = mmax;
    return static_cast<int>(m) * world;
}

// Active workgroups for a call of numel values: about one 16-byte unit per
// lane, at least 16 / W (so small calls still spread their flag traffic over
// a few workgroups, while large groups, whose every workgroup polls W - 1
// flags, keep the pollers few), at most the channel's workgroup count.  A
// function of numel and W alone, so every rank agrees.
inline int active_blocks(size_t numel, int nblocks, int world) {
    const size_t nvec = numel / kVecElems;
    size_t want = (nvec + kExchThreads - 1) / kExchThreads;
    const size_t floor_ = static_cast<size_t>(kMinActivePolls / world > 0 ? kMinActivePolls / world : 1);
    if (want < floor_) want = floor_;
    if (want > static_cast<size_t>(nblocks)) want = static_cast<size_t>(nblocks);
    return static_cast<int>(want);
}

// Groups of three or more take the two-shot from this many values under the
// automatic choice: the one-shot reads W - 1 peers' whole contributions, the
// two-shot 2 (W - 1) / W of one, but its second handshake adds latency, so
// the crossover falls as the group grows.  Measured on MI355X with every rank
// in one group launch (graph-captured), as the first size at which the
// two-shot was faster in two rounds: W = 3 98304, W = 4 16384, W = 5 10240,
// W = 6 6144, W = 7 5120, W = 8 3072 (e.g. W = 5 at 10240 values 13.6-13.8
// against 14.2 us, W = 7 at 4096 12.8-13.0 against 12.7 and at 5120 13.2-13.4
// against 16.2-16.4, W = 8 at 3072 12.4-12.6 against 12.8 us).
inline size_t two_shot_min_numel(int world) {
    switch (world) {
        case 3: return 98304;
        case 4: return 16384;
        case 5: return 10240;
        case 6: return 6144;
        case 7: return 5120;
        default: return 3072;
    }
}

enum class Algo { one_shot, two_shot, ll };

// The algorithm a call takes: a function of the channel and numel only (not
// of a rank's buffers), so every rank of a call takes the same one.  LL needs
// a call of at most kLLMaxNumel values (and one lane per unit); a call that
// asks for an algorithm it cannot take gets the one-shot (same bits).
// Automatic choice: LL up to ll_auto_max_numel(W) values; above that, for
// two ranks the one-shot, for three or more the one-shot and, from
// two_shot_min_numel(W), the two-shot.
inline Algo choose_algo(int algorithm, size_t numel, int world, int nblocks) {
    const bool ll_ok = numel <= kLLMaxNumel && active_blocks_ll(numel) <= nblocks;
    const bool two_ok = nblocks >= world;
    switch (algorithm) {
        case HR_ALGO_ONE_SHOT: return Algo::one_shot;
        case HR_ALGO_TWO_SHOT: return two_ok ? Algo::two_shot : Algo::one_shot;
        case HR_ALGO_LL: return ll_ok ? Algo::ll : Algo::one_shot;
        default: break;
    }
    if (ll_ok && numel <= ll_auto_max_numel(world)) return Algo::ll;
    return (two_ok && world >= 3 && numel >= two_shot_min_numel(world)) ? Algo::two_shot : Algo::one_shot;
}

template <int W, class E>
void launch_exchange(const ExchArgs &a, bool vec, Algo algo, hipStream_t s) {
    if (algo == Algo::ll) {
        if (vec)
            hipLaunchKernelGGL((exchange_ll_k<W, true, E>), dim3(a.nblocks), dim3(kExchThreads), 0, s, a.in, a.epochs, a.dev_error, a.numel, a.nactive, a);
        else
            hipLaunchKernelGGL((exchange_ll_k<W, false, E>), dim3(a.nblocks), dim3(kExchThreads), 0, s, a.in, a.epochs, a.dev_error, a.numel, a.nactive, a);
        return;
    }
    if (algo == Algo::two_shot) {
        if (vec)
            hipLaunchKernelGGL((exchange2_k<W, true, E>), dim3(a.nblocks), dim3(kExchThreads), 0, s, a.in, a.epochs, a.dev_error, a.numel, a.nactive, a);
        else
            hipLaunchKernelGGL((exchange2_k<W, false, E>), dim3(a.nblocks), dim3(kExchThreads), 0, s, a.in, a.epochs, a.dev_error, a.numel, a.nactive, a);
        return;
    }
    if (vec)
        hipLaunchKernelGGL((exchange_k<W, true, E>), dim3(a.nblocks), dim3(kExchThreads), 0, s, a.in, a.epochs, a.dev_error, a.numel, a.nactive, a);
    else
        hipLaunchKernelGGL((exchange_k<W, false, E>), dim3(a.nblocks), dim3(kExchThreads), 0, s, a.in, a.epochs, a.dev_error, a.numel, a.nactive, a);
}

template <int W, class E>
void launch_group(const GroupArgs &g, bool vec, Algo algo, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(W * g.a.nblocks));
    if (algo == Algo::ll) {
        if (vec)
            hipLaunchKernelGGL((exchange_ll_group_k<W, true, E>), grid, dim3(kExchThreads), 0, s, g);
        else
            hipLaunchKernelGGL((exchange_ll_group_k<W, false, E>), grid, dim3(kExchThreads), 0, s, g);
        return;
    }
    if (algo == Algo::two_shot) {
        if (vec)
            hipLaunchKernelGGL((exchange2_group_k<W, true, E>), grid, dim3(kExchThreads), 0, s, g);
        else
            hipLaunchKernelGGL((exchange2_group_k<W, false, E>), grid, dim3(kExchThreads), 0, s, g);
        return;
    }
    if (vec)
        hipLaunchKernelGGL((exchange_group_k<W, true, E>), grid, dim3(kExchThreads), 0, s, g);
    else
        hipLaunchKernelGGL((exchange_group_k<W, false, E>), grid, dim3(kExchThreads), 0, s, g);
}

template <class E>
void launch_group_w(const GroupArgs &g, bool vec, Algo algo, hipStream_t s) {
    switch (g.a.world) {
        case 2: launch_group<2, E>(g, vec, algo, s); break;
        case 3: launch_group<3, E>(g, vec, algo, s); break;
        case 4: launch_group<4, E>(g, vec, algo, s); break;
        case 5: launch_group<5, E>(g, vec, algo, s); break;
        case 6: launch_group<6, E>(g, vec, algo, s); break;
        case 7: launch_group<7, E>(g, vec, algo, s); break;
        case 8: launch_group<8, E>(g, vec, algo, s); break;
        default: break;
    }
}

template <class E>
void launch_exchange_w(const ExchArgs &a, bool vec, Algo algo, hipStream_t s) {
    switch (a.world) {
        case 2: launch_exchange<2, E>(a, vec, algo, s); break;
        case 3: launch_exchange<3, E>(a, vec, algo, s); break;
        case 4: launch_exchange<4, E>(a, vec, algo, s); break;
        case 5: launch_exchange<5, E>(a, vec, algo, s); break;
        case 6: launch_exchange<6, E>(a, vec, algo, s); break;
        case 7: launch_exchange<7, E>(a, vec, algo, s); break;
        case 8: launch_exchange<8, E>(a, vec, algo, s); break;
        default: break;
    }
}

}  // namespace hr

using namespace hr;

struct hr_channel_s {
    int device;
    int world_size;
    size_t max_numel;
    size_t stride;
    int nblocks;
    uint32_t timeout_us;
    uint64_t timeout_ticks;
    uint64_t abort_after_ticks;
    uint16_t ll_lead_ticks;
    uint16_t ll_floor_ticks;
    uint32_t link_mbps;        // pacing rate, or HR_LINK_UNPACED
    uint32_t pace_q16;         // wall-clock ticks per byte x 2^16, 0 when unpaced
    void *host_base;           // hipHostMalloc'ed region (host address)
    unsigned char *host_dev;   // the same region as seen by the device
    int algorithm;             // HR_ALGO_*
    size_t flags_off, flags2_off, reduced_off, ll_off, ll_stride, error_off, abort_off, diag_off, host_bytes;
    void *dev_base;            // hipMalloc: epochs[world][nblocks] (uint64), then the error word
    uint64_t *dev_epochs;
    uint32_t *dev_error;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) return;
        ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
    }
    ~DeviceGuard() {
        if (ok && prev >= 0) (void)hipSetDevice(prev);
    }
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ns nanoseconds in ticks of a clock of clock_khz, at most 65535.
uint16_t ticks16(uint32_t ns, int clock_khz) {
    const uint64_t t = static_cast<uint64_t>(ns) * static_cast<uint64_t>(clock_khz) / 1000000u;
    return static_cast<uint16_t>(t < 65535u ? t : 65535u);
}

// The pacing rate (MB/s) for the host link: the rate at which it carries
// writes while reads run the other way, which is what a paced exchange's
// publish meets, plus 1/32.  link_probe_k moves kCalibBytes each way at once
// on stream `s` (best of kCalibReps after one warm-up), with writers and
// readers in the proportion that moved the most in a sweep on MI355X (128
// and 64 workgroups).  At least HR_MIN_LINK_MBPS; 0 when a HIP call fails.
uint32_t calibrate_link(hipStream_t s, int cus) {
    constexpr size_t kCalibBytes = size_t(16) << 20;
    constexpr int kCalibReps = 3;
    const int units = static_cast<int>(kCalibBytes / sizeof(u32x4));
    int nw = cus / 2 < 128 ? cus / 2 : 128, nr = cus / 4 < 64 ? cus / 4 : 64;
    if (nw < 1) nw = 1;
    if (nr < 1) nr = 1;
    void *hw = nullptr, *hrd = nullptr, *dhw = nullptr, *dhr = nullptr, *src = nullptr, *sink = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    float best = 0.f;
    bool ok = hipHostMalloc(&hw, kCalibBytes, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
              hipHostMalloc(&hrd, kCalibBytes, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
              hipHostGetDevicePointer(&dhw, hw, 0) == hipSuccess &&
              hipHostGetDevicePointer(&dhr, hrd, 0) == hipSuccess && hipMalloc(&src, kCalibBytes) == hipSuccess &&
              hipMalloc(&sink, static_cast<size_t>(nr) * kExchThreads * sizeof(u32x4)) == hipSuccess &&
              hipMemsetAsync(src, 0, kCalibBytes, s) == hipSuccess && hipEventCreate(&ev[0]) == hipSuccess &&
              hipEventCreate(&ev[1]) == hipSuccess;
    for (int rep = -1; ok && rep < kCalibReps; ++rep) {
        ok = hipEventRecord(ev[0], s) == hipSuccess;
        if (ok) {
            hipLaunchKernelGGL(link_probe_k, dim3(nw + nr), dim3(kExchThreads), 0, s, static_cast<const u32x4 *>(src),
                               static_cast<u32x4 *>(dhw), static_cast<const u32x4 *>(dhr), static_cast<u32x4 *>(sink),
                               units, nw, nr);
            ok = hipGetLastError() == hipSuccess && hipEventRecord(ev[1], s) == hipSuccess &&
                 hipEventSynchronize(ev[1]) == hipSuccess;
        }
        float ms = 0.f;
        ok = ok && hipEventElapsedTime(&ms, ev[0], ev[1]) == hipSuccess;
        if (ok && rep >= 0 && ms > 0.f && (best == 0.f || ms < best)) best = ms;
    }
    for (hipEvent_t e : ev)
        if (e != nullptr) (void)hipEventDestroy(e);
    if (sink != nullptr) (void)hipFree(sink);
    if (src != nullptr) (void)hipFree(src);
    if (hrd != nullptr) (void)hipHostFree(hrd);
    if (hw != nullptr) (void)hipHostFree(hw);
    if (!ok || best <= 0.f) return 0;
    // pace 1/32 above the measured rate: slices then start just before the
    // link would run dry.  Measured on MI355X hosts (probe 48.4 GB/s), two
    // ranks, graph-captured, by pacing rate 45 / 48 / 50 / 52 / 55 GB/s:
    // 256 KiB 17.99 / 17.24 / 17.15 / 17.06 / 17.07 us, 1 MiB 53.5 / 51.1 /
    // 50.3 / 51.8 / 53.4 us, 16 MiB 792 / 737 / 719 / 751 / 789 us; and the
    // probe's own rate against 50 GB/s on one box: 17.05-17.46 against
    // 16.93-17.32 us at 256 KiB, 734-739 against 725-734 us at 16 MiB.
    const double mbps = static_cast<double>(kCalibBytes) / (static_cast<double>(best) * 1e-3) / 1e6 * 33.0 / 32.0;
    return mbps < HR_MIN_LINK_MBPS ? HR_MIN_LINK_MBPS : static_cast<uint32_t>(mbps);
}

// The rate a channel created with link_mbps = 0 paces by: measured once per
// device (calibrate_link, on the first such channel) and kept for the
// process; HR_DEFAULT_LINK_MBPS when the measurement fails.
std::mutex g_link_mu;
uint32_t g_link_mbps[64];

uint32_t device_link_mbps(int dev, hipStream_t s, int cus) {
    if (dev < 0 || dev >= 64) return HR_DEFAULT_LINK_MBPS;
    std::lock_guard<std::mutex> lock(g_link_mu);
    if (g_link_mbps[dev] == 0) {
        const uint32_t m = calibrate_link(s, cus);
        g_link_mbps[dev] = m != 0 ? m : HR_DEFAULT_LINK_MBPS;
    }
    return g_link_mbps[dev];
}

void release(hr_channel ch) {
    if (ch->host_base) (void)hipHostFree(ch->host_base);
    if (ch->dev_base) (void)hipFree(ch->dev_base);
    delete ch;
}

}  // namespace

extern "C" HR_API hr_status hr_create_channel(const hr_channel_config *cfg, hr_channel *out) {
    if (cfg == nullptr || out == nullptr) return HR_ERR_INVALID_ARG;
    if (cfg->world_size < 2 || cfg->world_size > kMaxWorld) return HR_ERR_UNSUPPORTED;
    if (cfg->device < 0 || cfg->num_blocks < 0) return HR_ERR_INVALID_ARG;
    if (cfg->algorithm < HR_ALGO_AUTO || cfg->algorithm > HR_ALGO_LL) return HR_ERR_INVALID_ARG;
    if (cfg->link_mbps != 0 && cfg->link_mbps < HR_MIN_LINK_MBPS) return HR_ERR_INVALID_ARG;
    const size_t max_numel = cfg->max_numel ? cfg->max_numel : HR_DEFAULT_MAX_NUMEL;
    // A slot is addressed by a buffer descriptor whose byte count and
    // offsets are 32-bit: keep one slot at or below 1 GiB.
    if (max_numel > HR_MAX_NUMEL_LIMIT) return HR_ERR_INVALID_ARG;
    const uint32_t timeout_us = cfg->timeout_us ? cfg->timeout_us : HR_DEFAULT_TIMEOUT_US;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) return HR_ERR_HIP;
    if (cfg->device >= ndev) return HR_ERR_INVALID_ARG;
    DeviceGuard guard(cfg->device);
    if (!guard.ok) return HR_ERR_HIP;

    int cus = 0, clock_khz = 0;
    if (device_cu_count(cfg->device, &cus) != hipSuccess) return HR_ERR_HIP;
    if (hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, cfg->device) != hipSuccess ||
        clock_khz <= 0)
        return HR_ERR_UNSUPPORTED;

    hr_channel ch = new (std::nothrow) hr_channel_s{};
    if (ch == nullptr) return HR_ERR_HIP;
    ch->device = cfg->device;
    const int world = cfg->world_size;
    ch->world_size = world;
    ch->max_numel = max_numel;
    ch->stride = round_up(max_numel, kLine / sizeof(uint16_t));
    // Default and ceiling: CUs / world per rank, so that all ranks of a
    // loopback channel are resident at once.
    int nb = cfg->num_blocks ? cfg->num_blocks : cus / world;
    if (nb > cus / world) nb = cus / world;
    if (nb < 1) nb = 1;
    if (cfg->algorithm == HR_ALGO_TWO_SHOT && nb < world) {
        delete ch;
        return HR_ERR_INVALID_ARG;  // the two-shot needs a workgroup per shard
    }
    ch->nblocks = nb;
    ch->algorithm = cfg->algorithm;
    ch->timeout_us = timeout_us;
    ch->timeout_ticks = static_cast<uint64_t>(timeout_us) * static_cast<uint64_t>(clock_khz) / 1000u;
    ch->abort_after_ticks = static_cast<uint64_t>(kAbortAfterUs) * static_cast<uint64_t>(clock_khz) / 1000u;
    ch->ll_lead_ticks = ticks16(kLLLeadNs, clock_khz);
    ch->ll_floor_ticks = ticks16(kLLFloorNs, clock_khz);
    ch->link_mbps = cfg->link_mbps;  // 0: the device's measured rate, below

    const size_t slot_bytes = 2 * static_cast<size_t>(world) * ch->stride * sizeof(uint16_t);
    const size_t flag_bytes = static_cast<size_t>(world) * static_cast<size_t>(nb) * kLine;
    ch->reduced_off = round_up(slot_bytes, kLine);
    ch->flags_off = ch->reduced_off + 2 * ch->stride * sizeof(uint16_t);
    ch->flags2_off = ch->flags_off + flag_bytes;
    ch->ll_off = ch->flags2_off + flag_bytes;
    // three 8-byte words per 8-value unit of the largest LL call
    ch->ll_stride = ll_stride_for(max_numel);
    ch->error_off = ch->ll_off + round_up(2 * static_cast<size_t>(world) * ch->ll_stride * sizeof(uint64_t), kLine);
    ch->abort_off = ch->error_off + kLine;
    ch->diag_off = ch->abort_off + kLine;  // the timeout record (record_missing)
    ch->host_bytes = ch->diag_off + kLine;

    // The call counters are zeroed on a private stream, so creating a channel
    // never waits for other work on the device (such as another channel's
    // kernels waiting for their peers).
    void *dev_view = nullptr;
    const size_t word_bytes = static_cast<size_t>(world) * nb * sizeof(uint64_t) + sizeof(uint64_t);
    hipStream_t init = nullptr;
    bool ok = hipHostMalloc(&ch->host_base, ch->host_bytes, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
              hipHostGetDevicePointer(&dev_view, ch->host_base, 0) == hipSuccess &&
              hipMalloc(&ch->dev_base, word_bytes) == hipSuccess &&
              hipStreamCreateWithFlags(&init, hipStreamNonBlocking) == hipSuccess &&
              hipMemsetAsync(ch->dev_base, 0, word_bytes, init) == hipSuccess &&
              hipStreamSynchronize(init) == hipSuccess;
    if (ok && ch->link_mbps == HR_LINK_CALIBRATE) {
        ch->link_mbps = calibrate_link(init, cus);
        ok = ch->link_mbps != 0;
    } else if (ok && ch->link_mbps == 0) {
        ch->link_mbps = device_link_mbps(cfg->device, init, cus);
    }
    if (init != nullptr) (void)hipStreamDestroy(init);
    if (!ok) {
        release(ch);
        return HR_ERR_HIP;
    }
    // ticks per byte = clock_khz * 1e3 / (link_mbps * 1e6)
    ch->pace_q16 = ch->link_mbps == HR_LINK_UNPACED
                       ? 0u
                       : static_cast<uint32_t>((static_cast<uint64_t>(clock_khz) << 16) /
                                               (static_cast<uint64_t>(ch->link_mbps) * 1000u));
    ch->host_dev = static_cast<unsigned char *>(dev_view);
    ch->dev_epochs = static_cast<uint64_t *>(ch->dev_base);
    ch->dev_error = reinterpret_cast<uint32_t *>(ch->dev_epochs + static_cast<size_t>(world) * nb);
    std::memset(ch->host_base, 0, ch->host_bytes);
    __atomic_thread_fence(__ATOMIC_SEQ_CST);
    *out = ch;
    return HR_OK;
}

namespace {

// The launch arguments of a call of numel values by `rank` (buffers left
// unset), and the algorithm the call takes.
ExchArgs call_args(hr_channel ch, int rank, size_t numel, Algo *algo_out) {
    ExchArgs a{};
    a.numel = numel;
    a.slots = reinterpret_cast<uint16_t *>(ch->host_dev);
    a.stride = ch->stride;
    a.flags = reinterpret_cast<uint64_t *>(ch->host_dev + ch->flags_off);
    a.flags2 = reinterpret_cast<uint64_t *>(ch->host_dev + ch->flags2_off);
    a.reduced = reinterpret_cast<uint16_t *>(ch->host_dev + ch->reduced_off);
    a.ll = reinterpret_cast<uint64_t *>(ch->host_dev + ch->ll_off);
    a.ll_stride = ch->ll_stride;
    a.epochs = ch->dev_epochs + static_cast<size_t>(rank) * ch->nblocks;
    a.dev_error = ch->dev_error;
    a.host_error = reinterpret_cast<uint32_t *>(ch->host_dev + ch->error_off);
    a.abort_w = reinterpret_cast<const uint32_t *>(ch->host_dev + ch->abort_off);
    a.diag = reinterpret_cast<uint64_t *>(ch->host_dev + ch->diag_off);
    a.timeout_ticks = ch->timeout_ticks;
    a.abort_after_ticks = ch->abort_after_ticks;
    a.ll_lead_ticks = ch->ll_lead_ticks;  // the floor is set by per-rank calls only
    a.pace_q16 = ch->pace_q16;
    a.rank = rank;
    a.world = ch->world_size;
    a.nblocks = ch->nblocks;
    const Algo algo = choose_algo(ch->algorithm, numel, ch->world_size, ch->nblocks);
    a.nactive = algo == Algo::two_shot ? active_blocks2(numel, ch->nblocks, ch->world_size)
                : algo == Algo::ll     ? active_blocks_ll(numel)
                                       : active_blocks(numel, ch->nblocks, ch->world_size);

    *algo_out = algo;
    return a;
}

template <class E>
hr_status allreduce_impl(hr_channel ch, int rank, const void *in, void *out, size_t numel, hr_stream_t stream) {
    if (ch == nullptr || rank < 0 || rank >= ch->world_size) return HR_ERR_INVALID_ARG;
    const uint32_t sticky = __atomic_load_n(
        reinterpret_cast<uint32_t *>(static_cast<unsigned char *>(ch->host_base) + ch->error_off), __ATOMIC_ACQUIRE);
    if (sticky != 0) return static_cast<hr_status>(sticky);
    if (numel == 0) return HR_OK;
    if (in == nullptr || out == nullptr) return HR_ERR_INVALID_ARG;
    if (numel > ch->max_numel) return HR_ERR_TOO_LARGE;
    if (!aligned(in, 2) || !aligned(out, 2)) return HR_ERR_ALIGNMENT;
    if (partial_overlap(in, out, numel * 2)) return HR_ERR_INVALID_ARG;

    int dev = -1;
    if (stream_device(stream, &dev) != hipSuccess) return HR_ERR_HIP;
    if (dev != ch->device) return HR_ERR_INVALID_ARG;

    Algo algo;
    ExchArgs a = call_args(ch, rank, numel, &algo);
    a.in = in;
    a.out = out;
    a.ll_floor_ticks = ch->ll_floor_ticks;
    launch_exchange_w<E>(a, aligned(in, 16) && aligned(out, 16), algo, reinterpret_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? HR_OK : HR_ERR_HIP;
}

// True when [a, a+bytes) and [b, b+bytes) share a byte (equal pointers too).
inline bool ranges_overlap(const void *a, const void *b, size_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
}

// Every rank of the channel in one launch (the loopback group).
template <class E>
hr_status group_impl(hr_channel ch, const void *const *ins, void *const *outs, size_t numel, hr_stream_t stream) {
    if (ch == nullptr) return HR_ERR_INVALID_ARG;
    const uint32_t sticky = __atomic_load_n(
        reinterpret_cast<uint32_t *>(static_cast<unsigned char *>(ch->host_base) + ch->error_off), __ATOMIC_ACQUIRE);
    if (sticky != 0) return static_cast<hr_status>(sticky);
    if (numel == 0) return HR_OK;
    if (ins == nullptr || outs == nullptr) return HR_ERR_INVALID_ARG;
    if (numel > ch->max_numel) return HR_ERR_TOO_LARGE;
    const int W = ch->world_size;
    const size_t bytes = numel * 2;
    bool vec = true;
    for (int r = 0; r < W; ++r) {
        if (ins[r] == nullptr || outs[r] == nullptr) return HR_ERR_INVALID_ARG;
        if (!aligned(ins[r], 2) || !aligned(outs[r], 2)) return HR_ERR_ALIGNMENT;
        vec = vec && aligned(ins[r], 16) && aligned(outs[r], 16);
    }
    // A rank may fold in place (out == in); any other overlap would let one
    // rank's output change what another rank publishes or re-reads.
    for (int r = 0; r < W; ++r) {
        if (partial_overlap(ins[r], outs[r], bytes)) return HR_ERR_INVALID_ARG;
        for (int q = 0; q < W; ++q) {
            if (q == r) continue;
            if (ranges_overlap(outs[r], outs[q], bytes) || ranges_overlap(outs[r], ins[q], bytes))
                return HR_ERR_INVALID_ARG;
        }
    }

    int dev = -1;
    if (stream_device(stream, &dev) != hipSuccess) return HR_ERR_HIP;
    if (dev != ch->device) return HR_ERR_INVALID_ARG;

    Algo algo;
    GroupArgs g{};
    g.a = call_args(ch, 0, numel, &algo);
    g.a.epochs = ch->dev_epochs;  // rank r's counters follow at r * nblocks
    for (int r = 0; r < W; ++r) {
        g.in[r] = ins[r];
        g.out[r] = outs[r];
    }
    launch_group_w<E>(g, vec, algo, reinterpret_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? HR_OK : HR_ERR_HIP;
}

}  // namespace

extern "C" HR_API hr_status hr_allreduce_f16(hr_channel ch, int rank, const void *in, void *out, size_t numel,
                                             hr_stream_t stream) {
    return allreduce_impl<F16>(ch, rank, in, out, numel, stream);
}

extern "C" HR_API hr_status hr_allreduce_bf16(hr_channel ch, int rank, const void *in, void *out, size_t numel,
                                              hr_stream_t stream) {
    return allreduce_impl<BF16>(ch, rank, in, out, numel, stream);
}

extern "C" HR_API hr_status hr_allreduce_group_f16(hr_channel ch, const void *const *ins, void *const *outs,
                                                   size_t numel, hr_stream_t stream) {
    return group_impl<F16>(ch, ins, outs, numel, stream);
}

extern "C" HR_API hr_status hr_allreduce_group_bf16(hr_channel ch, const void *const *ins, void *const *outs,
                                                    size_t numel, hr_stream_t stream) {
    return group_impl<BF16>(ch, ins, outs, numel, stream);
}

extern "C" HR_API hr_status hr_exchange_algorithm(hr_channel ch, size_t numel, int *algorithm) {
    if (ch == nullptr || algorithm == nullptr) return HR_ERR_INVALID_ARG;
    if (numel > ch->max_numel) return HR_ERR_TOO_LARGE;
    switch (choose_algo(ch->algorithm, numel, ch->world_size, ch->nblocks)) {
        case Algo::two_shot: *algorithm = HR_ALGO_TWO_SHOT; break;
        case Algo::ll: *algorithm = HR_ALGO_LL; break;
        default: *algorithm = HR_ALGO_ONE_SHOT; break;
    }
    return HR_OK;
}

extern "C" HR_API hr_status hr_channel_status(hr_channel ch) {
    if (ch == nullptr) return HR_ERR_INVALID_ARG;
    return static_cast<hr_status>(__atomic_load_n(
        reinterpret_cast<uint32_t *>(static_cast<unsigned char *>(ch->host_base) + ch->error_off), __ATOMIC_ACQUIRE));
}

extern "C" HR_API hr_status hr_channel_abort(hr_channel ch) {
    if (ch == nullptr) return HR_ERR_INVALID_ARG;
    __atomic_store_n(reinterpret_cast<uint32_t *>(static_cast<unsigned char *>(ch->host_base) + ch->abort_off), 1u,
                     __ATOMIC_RELEASE);
    __atomic_thread_fence(__ATOMIC_SEQ_CST);
    return HR_OK;
}

extern "C" HR_API hr_status hr_channel_timeout_info(hr_channel ch, int *rank, uint32_t *peer_mask,
                                                    uint64_t *call) {
    if (ch == nullptr || rank == nullptr || peer_mask == nullptr || call == nullptr) return HR_ERR_INVALID_ARG;
    const uint64_t w = __atomic_load_n(
        reinterpret_cast<uint64_t *>(static_cast<unsigned char *>(ch->host_base) + ch->diag_off), __ATOMIC_ACQUIRE);
    if (w == 0) {
        *rank = -1;
        *peer_mask = 0;
        *call = 0;
    } else {
        *rank = static_cast<int>((w >> 8) & 0xFFu);
        *peer_mask = static_cast<uint32_t>(w & 0xFFu);
        *call = w >> 16;
    }
    return HR_OK;
}

extern "C" HR_API hr_status hr_channel_get_info(hr_channel ch, hr_channel_info *info) {
    if (ch == nullptr || info == nullptr) return HR_ERR_INVALID_ARG;
    unsigned char *base = static_cast<unsigned char *>(ch->host_base);
    info->device = ch->device;
    info->world_size = ch->world_size;
    info->max_numel = ch->max_numel;
    info->num_blocks = ch->nblocks;
    info->block_threads = kExchThreads;
    info->timeout_us = ch->timeout_us;
    info->host_slots = base;
    info->slot_stride = ch->stride;
    info->host_flags = reinterpret_cast<volatile uint64_t *>(base + ch->flags_off);
    info->flag_stride = kFlagStride;
    info->host_error = reinterpret_cast<volatile uint32_t *>(base + ch->error_off);
    info->host_abort = reinterpret_cast<volatile uint32_t *>(base + ch->abort_off);
    info->algorithm = ch->algorithm;
    info->host_reduced = base + ch->reduced_off;
    info->host_flags2 = reinterpret_cast<volatile uint64_t *>(base + ch->flags2_off);
    info->host_ll = base + ch->ll_off;
    info->dev_epochs = ch->dev_epochs;
    info->link_mbps = ch->link_mbps;
    info->ll_stride = ch->ll_stride;
    return HR_OK;
}

extern "C" HR_API hr_status hr_destroy(hr_channel ch) {
    if (ch == nullptr) return HR_OK;
    hr_status st = HR_OK;
    {
        DeviceGuard guard(ch->device);
        if (!guard.ok || hipDeviceSynchronize() != hipSuccess) st = HR_ERR_HIP;
    }
    release(ch);
    return st;
}

extern "C" HR_API hr_status hr_loopback_stream_create(int device, hr_stream_t *out) {
    if (out == nullptr || device < 0) return HR_ERR_INVALID_ARG;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) return HR_ERR_HIP;
    if (device >= ndev) return HR_ERR_INVALID_ARG;
    DeviceGuard guard(device);
    if (!guard.ok) return HR_ERR_HIP;
    int cus = 0;
    if (device_cu_count(device, &cus) != hipSuccess) return HR_ERR_HIP;
    // every compute unit enabled: the mask only buys a dedicated queue
    std::vector<uint32_t> mask((static_cast<size_t>(cus) + 31) / 32, 0u);
    for (int i = 0; i < cus; ++i) mask[static_cast<size_t>(i) / 32] |= 1u << (i % 32);
    hipStream_t s = nullptr;
    if (hipExtStreamCreateWithCUMask(&s, static_cast<uint32_t>(mask.size()), mask.data()) != hipSuccess)
        return HR_ERR_HIP;
    *out = reinterpret_cast<hr_stream_t>(s);
    return HR_OK;
}

extern "C" HR_API hr_status hr_loopback_stream_destroy(hr_stream_t stream) {
    if (stream == nullptr) return HR_OK;
    return hipStreamDestroy(reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? HR_OK : HR_ERR_HIP;
}

// ------------------------------------------------- allocation-free group call
//
// hr_allreduce_group_noalloc_f16 runs the loopback group call without a
// channel: the state a channel allocates at creation (slots, reduced-shard
// slots, flags, low-latency words, call counters, error and abort words) sits
// in `scratch`, one array per device that lives as long as the process.  The
// array is device memory, so the slots are in HBM rather than in pinned host
// memory; the kernels are the group kernels above, unchanged (their
// system-coherent accesses are coherent on device memory too), and the fold
// and its bits are the same.  The layout is that of a channel of
// kNoAllocMaxNumel values, computed per call from the group size and the
// device's workgroup count.
//
// Every call starts from a zeroed state: a fill kernel on the call's stream
// clears the flags, the call counters, the error words and (for a
// low-latency call) the low-latency words the call reads, so the call's
// number is 1 and no value of an earlier call can release a wait.  The fill
// uses system-coherent stores, like every other access to this state, so the
// exchange kernel's system-coherent loads see the zeros.  Calls that overlap
// on one device share the array and race; calls on one stream do not.

constexpr size_t kNoAllocMaxNumel = HR_NOALLOC_MAX_NUMEL;
constexpr size_t kNoAllocBytes = HR_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

struct NoAllocLayout {
    size_t stride, ll_stride;
    size_t slots, reduced, flags, flags2, ll, epochs, dev_error, host_error, abort_w, total;
};

inline NoAllocLayout noalloc_layout(int world, int nb) {
    NoAllocLayout L{};
    L.stride = round_up(kNoAllocMaxNumel, kLine / sizeof(uint16_t));
    L.ll_stride = ll_stride_for(kNoAllocMaxNumel);
    const size_t flag_bytes = static_cast<size_t>(world) * static_cast<size_t>(nb) * kLine;
    L.slots = 0;
    L.reduced = round_up(2 * static_cast<size_t>(world) * L.stride * sizeof(uint16_t), kLine);
    L.flags = L.reduced + round_up(2 * L.stride * sizeof(uint16_t), kLine);
    L.flags2 = L.flags + flag_bytes;
    L.ll = L.flags2 + flag_bytes;
    L.epochs = L.ll + round_up(2 * static_cast<size_t>(world) * L.ll_stride * sizeof(uint64_t), kLine);
    L.dev_error = L.epochs + round_up(static_cast<size_t>(world) * nb * sizeof(uint64_t), kLine);
    L.host_error = L.dev_error + kLine;
    L.abort_w = L.host_error + kLine;
    L.total = L.abort_w + kLine;
    return L;
}

// Up to three ranges of 16-byte units and one 32-bit word, zeroed with
// system-coherent stores; workgroups stride over the units of each range.
struct NoAllocClear {
    u32x4 *base[3];
    uint32_t units[3];
    uint32_t *word;
};

__global__ __launch_bounds__(kExchThreads) void noalloc_clear_k(NoAllocClear c) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const uint32_t step = gridDim.x * kExchThreads;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        if (c.units[k] == 0) continue;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(c.base[k], 0, static_cast<int>(c.units[k] * 16), kRawBufferDword3);
        for (uint32_t u = blockIdx.x * kExchThreads + threadIdx.x; u < c.units[k]; u += step)
            __builtin_amdgcn_raw_buffer_store_b128(zero, r, static_cast<int>(u * 16), 0, kSysCoherent);
    }
    if (c.word != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(c.word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

namespace {

// The device address of `scratch` on each device (host code never uses the
// array's own name: on the host it only stands for the symbol), with the
// device's wall-clock rate; looked up once per device, on its first call.
struct NoAllocDevice {
    unsigned char *ptr = nullptr;
    int clock_khz = 0;
};
NoAllocDevice g_noalloc[64];
std::mutex g_noalloc_mu;

hipError_t noalloc_device(int dev, NoAllocDevice *out) {
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoAllocDevice &d = g_noalloc[dev];
    if (d.ptr == nullptr) {
        DeviceGuard guard(dev);
        if (!guard.ok) return hipErrorInvalidDevice;
        int clock_khz = 0;
        hipError_t e = hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess) return e;
        if (clock_khz <= 0) return hipErrorInvalidValue;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        d.clock_khz = clock_khz;
        d.ptr = static_cast<unsigned char *>(p);
    }
    *out = d;
    return hipSuccess;
}

}  // namespace

extern "C" HR_API hr_status hr_allreduce_group_noalloc_f16(const void *const *ins, void *const *outs, int world_size,
                                                           size_t numel, uint32_t *status, hr_stream_t stream) {
    if (world_size < 2 || world_size > kMaxWorld) return HR_ERR_UNSUPPORTED;
    if (numel == 0) return HR_OK;
    if (ins == nullptr || outs == nullptr) return HR_ERR_INVALID_ARG;
    if (numel > kNoAllocMaxNumel) return HR_ERR_TOO_LARGE;
    if (status != nullptr && !aligned(status, 4)) return HR_ERR_ALIGNMENT;
    const int W = world_size;
    const size_t bytes = numel * 2;
    bool vec = true;
    for (int r = 0; r < W; ++r) {
        if (ins[r] == nullptr || outs[r] == nullptr) return HR_ERR_INVALID_ARG;
        if (!aligned(ins[r], 2) || !aligned(outs[r], 2)) return HR_ERR_ALIGNMENT;
        vec = vec && aligned(ins[r], 16) && aligned(outs[r], 16);
    }
    for (int r = 0; r < W; ++r) {
        if (partial_overlap(ins[r], outs[r], bytes)) return HR_ERR_INVALID_ARG;
        for (int q = 0; q < W; ++q) {
            if (q == r) continue;
            if (ranges_overlap(outs[r], outs[q], bytes) || ranges_overlap(outs[r], ins[q], bytes))
                return HR_ERR_INVALID_ARG;
        }
    }

    int dev = -1, cus = 0;
    if (stream_device(stream, &dev) != hipSuccess) return HR_ERR_HIP;
    if (device_cu_count(dev, &cus) != hipSuccess) return HR_ERR_HIP;
    int nb = cus / W;
    if (nb < 1) nb = 1;
    const NoAllocLayout L = noalloc_layout(W, nb);
    if (L.total > kNoAllocBytes) return HR_ERR_UNSUPPORTED;  // a device with more compute units than planned for
    NoAllocDevice d;
    if (noalloc_device(dev, &d) != hipSuccess) return HR_ERR_HIP;
    unsigned char *base = d.ptr;

    const Algo algo = choose_algo(HR_ALGO_AUTO, numel, W, nb);
    GroupArgs g{};
    ExchArgs &a = g.a;
    a.numel = numel;
    a.slots = reinterpret_cast<uint16_t *>(base + L.slots);
    a.stride = L.stride;
    a.flags = reinterpret_cast<uint64_t *>(base + L.flags);
    a.flags2 = reinterpret_cast<uint64_t *>(base + L.flags2);
    a.reduced = reinterpret_cast<uint16_t *>(base + L.reduced);
    a.ll = reinterpret_cast<uint64_t *>(base + L.ll);
    a.ll_stride = L.ll_stride;
    a.epochs = reinterpret_cast<uint64_t *>(base + L.epochs);
    a.dev_error = reinterpret_cast<uint32_t *>(base + L.dev_error);
    a.host_error = status != nullptr ? status : reinterpret_cast<uint32_t *>(base + L.host_error);
    a.abort_w = reinterpret_cast<const uint32_t *>(base + L.abort_w);
    a.timeout_ticks = static_cast<uint64_t>(HR_DEFAULT_TIMEOUT_US) * static_cast<uint64_t>(d.clock_khz) / 1000u;
    a.abort_after_ticks = static_cast<uint64_t>(kAbortAfterUs) * static_cast<uint64_t>(d.clock_khz) / 1000u;
    a.pace_q16 = 0;  // the slots are in HBM: no host link to pace for
    a.rank = 0;
    a.world = W;
    a.nblocks = nb;
    a.nactive = algo == Algo::two_shot ? active_blocks2(numel, nb, W)
                : algo == Algo::ll     ? active_blocks_ll(numel)
                                       : active_blocks(numel, nb, W);
    for (int r = 0; r < W; ++r) {
        g.in[r] = ins[r];
        g.out[r] = outs[r];
    }

    // zero what the call's waits compare against: both flag arrays, the call
    // counters through the abort word, and (LL) the parity-1 low-latency
    // words of every rank -- the call number is 1
    NoAllocClear c{};
    c.base[0] = reinterpret_cast<u32x4 *>(base + L.flags);
    c.units[0] = static_cast<uint32_t>((L.ll - L.flags) / sizeof(u32x4));
    c.base[1] = reinterpret_cast<u32x4 *>(base + L.epochs);
    c.units[1] = static_cast<uint32_t>((L.total - L.epochs) / sizeof(u32x4));
    if (algo == Algo::ll) {
        // parity 1's slots: W x ll_stride 8-byte words, a whole number of 16-byte units
        c.base[2] = reinterpret_cast<u32x4 *>(base + L.ll + static_cast<size_t>(W) * L.ll_stride * sizeof(uint64_t));
        c.units[2] = static_cast<uint32_t>(static_cast<size_t>(W) * L.ll_stride * sizeof(uint64_t) / sizeof(u32x4));
    }
    c.word = status;
    const uint32_t units = c.units[0] > c.units[2] ? c.units[0] : c.units[2];
    uint32_t grid = (units + kExchThreads - 1) / kExchThreads;
    if (grid > static_cast<uint32_t>(cus)) grid = static_cast<uint32_t>(cus);
    if (grid < 1) grid = 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(noalloc_clear_k, dim3(grid), dim3(kExchThreads), 0, s, c);
    if (hipGetLastError() != hipSuccess) return HR_ERR_HIP;
    launch_group_w<F16>(g, vec, algo, s);
    return hipGetLastError() == hipSuccess ? HR_OK : HR_ERR_HIP;
}

#ifdef HR_TIMELINE
// Diagnostic library only: attach the timeline buffer (records of
// kTimelineWords 64-bit words, `calls` x world x num_blocks of them) on the
// current device; NULL detaches.
extern "C" HR_API hr_status hr_timeline_attach(void *buf, uint64_t calls) {
    if (hipMemcpyToSymbol(HIP_SYMBOL(hr_tl_buf), &buf, sizeof(buf)) != hipSuccess) return HR_ERR_HIP;
    if (hipMemcpyToSymbol(HIP_SYMBOL(hr_tl_calls), &calls, sizeof(calls)) != hipSuccess) return HR_ERR_HIP;
    return hipDeviceSynchronize() == hipSuccess ? HR_OK : HR_ERR_HIP;
}
#endif
