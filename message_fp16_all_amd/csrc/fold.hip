// fold.hip -- hr_reduce_f16 / hr_reduce_bf16: left fold of G binary16 (or
// bfloat16) contributions in HBM.
//
// R[i] = fl16(...fl16(fl16(x0[i] + x1[i]) + x2[i])... + x_{G-1}[i]), one
// rounding per add, rank order fixed (the all-reduce's local combine; the
// two-rank case is the single-rounding commutative sum of the 1Cat-vLLM pull
// request "[Kernel] Two-rank FP16 all-reduce through pinned host memory for
// GPUs without P2P", section "Purpose"; the SGLang pull request "[SM120] Add
// optional FlashInfer PCIe-IPC all-reduce for switch-free hosts", section
// "Accuracy", is why the order is fixed).
//
// Roofline: (G + 1) * N * 2 bytes of HBM traffic against (G - 1) * N adds,
// at most 7/18 add per byte -- bound by HBM bandwidth, not by VALU; there is
// no contraction, so no MFMA.
//
// Kernel shape.  Workgroups of 128 lanes; each lane owns U 16-byte units (8
// values each) per tile and issues all G*U dwordx4 loads before the first
// add, so every lane keeps G*U*16 bytes in flight; the adds run in rank
// order as packed v_pk_add_f16; U dwordx4 stores follow.  Loads are
// non-temporal and stores device-scope write-through: every byte is touched
// once, so caching it would only evict useful lines.
// A grid-stride loop over tiles covers any N; the N % 8 tail is folded one
// value at a time by the first workgroup.  Pointers that are not all 16-byte
// aligned take a one-value-per-lane kernel instead.
#include "hr_internal.h"

#include <atomic>

namespace hr {

constexpr int kFoldThreads = 128;

// Output stores: device-scope write-through (sc1).  Measured on MI355X
// against non-temporal and default stores, for G = 8 and 32 MiB
// contributions: 3-4 % less time; every output byte is written once and
// never read back by the kernel, so nothing is gained by keeping it in L2.
constexpr int kStoreDeviceScope = 16;                 // sc1
constexpr int kRawBufferDword3 = 0x00020000;          // raw (untyped) 32-bit data format

struct FoldArgs {
    const void *in[HR_MAX_G];
    void *out;
    size_t nvec;   // whole 16-byte units
    size_t numel;  // values
};

template <int G>
struct FoldShape {
    // units per lane per tile: G * U loads of 16 B in flight, <= 64 VGPRs
    static constexpr int U = (16 / G) > 0 ? (16 / G) : 1;
};

// Contributions laid out by hr_workspace_stride: one buffer, equal spacing
// of k * 2 MiB + 4 KiB.  Equal offsets of contributions that sit a multiple
// of 2 MiB apart collide in the same HBM banks; the 4 KiB shift spreads
// them (measured on MI355X at 32 MiB per contribution: G = 8 from 76 % to
// 78 % of 8 TB/s, G = 16 from 66 % to 78 %).
constexpr size_t kWorkspaceAlign = size_t(2) << 20;
constexpr size_t kWorkspaceShift = 4096;

inline bool workspace_layout(const FoldArgs &a, int G) {
    if (G < 2) return false;
    const intptr_t d = reinterpret_cast<intptr_t>(a.in[1]) - reinterpret_cast<intptr_t>(a.in[0]);
    if (d <= 0 || static_cast<size_t>(d) % kWorkspaceAlign != kWorkspaceShift) return false;
    for (int g = 2; g < G; ++g)
        if (reinterpret_cast<intptr_t>(a.in[g]) - reinterpret_cast<intptr_t>(a.in[g - 1]) != d) return false;
    return true;
}

template <int G, int U, class E>
__global__ __launch_bounds__(kFoldThreads) void fold_vec(FoldArgs a) {
    const size_t nvec = a.nvec;
    const size_t tile = static_cast<size_t>(kFoldThreads) * U;
    const size_t step = static_cast<size_t>(gridDim.x) * tile;
    u32x4 *out = static_cast<u32x4 *>(a.out);

    for (size_t base = blockIdx.x * tile + threadIdx.x; base < nvec; base += step) {
        // the output tile as a buffer resource, so its stores can carry the
        // device-scope (sc1) write-through policy; offsets stay below 4 KiB
        const size_t t0 = base - threadIdx.x;
        const size_t tn = (nvec - t0 < tile) ? nvec - t0 : tile;
        const __amdgpu_buffer_rsrc_t orsrc =
            __builtin_amdgcn_make_buffer_rsrc(out + t0, 0, static_cast<int>(tn * sizeof(u32x4)), kRawBufferDword3);
        u32x4 x[G][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t v = base + static_cast<size_t>(u) * kFoldThreads;
            if (v < nvec) {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    x[g][u] = __builtin_nontemporal_load(static_cast<const u32x4 *>(a.in[g]) + v);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t v = base + static_cast<size_t>(u) * kFoldThreads;
            if (v < nvec) {
                u32x4 acc = x[0][u];
#pragma unroll
                for (int g = 1; g < G; ++g) acc = E::add8(acc, x[g][u]);
                __builtin_amdgcn_raw_buffer_store_b128(acc, orsrc, static_cast<int>((v - t0) * sizeof(u32x4)), 0,
                                                       kStoreDeviceScope);
            }
        }
    }

    // N % 8 trailing values
    if (blockIdx.x == 0) {
        const size_t i = nvec * kVecElems + threadIdx.x;
        if (i < a.numel) {
            uint16_t acc = static_cast<const uint16_t *>(a.in[0])[i];
#pragma unroll
            for (int g = 1; g < G; ++g) acc = E::add1(acc, static_cast<const uint16_t *>(a.in[g])[i]);
            static_cast<uint16_t *>(a.out)[i] = acc;
        }
    }
}

// One value per lane, for pointers that are only 2-byte aligned.
template <class E>
__global__ __launch_bounds__(kFoldThreads) void fold_scalar(FoldArgs a, int G) {
    const size_t step = static_cast<size_t>(gridDim.x) * kFoldThreads;
    uint16_t *out = static_cast<uint16_t *>(a.out);
    for (size_t i = blockIdx.x * static_cast<size_t>(kFoldThreads) + threadIdx.x; i < a.numel; i += step) {
        uint16_t acc = static_cast<const uint16_t *>(a.in[0])[i];
        for (int g = 1; g < G; ++g) acc = E::add1(acc, static_cast<const uint16_t *>(a.in[g])[i]);
        out[i] = acc;
    }
}

namespace {

std::atomic<int> g_cus[64];

template <int G, int U, class E>
hipError_t launch_shape(const FoldArgs &a, int cus, hipStream_t s) {
    const size_t tiles = (a.nvec + static_cast<size_t>(kFoldThreads) * U - 1) / (static_cast<size_t>(kFoldThreads) * U);
    // Enough workgroups to fill every CU many times over; beyond that the
    // grid-stride loop takes over so huge N does not mean huge grids.
    const size_t cap = static_cast<size_t>(cus) * 32;
    size_t grid = tiles < cap ? tiles : cap;
    if (grid == 0) grid = 1;  // the tail alone
    hipLaunchKernelGGL((fold_vec<G, U, E>), dim3(static_cast<unsigned>(grid)), dim3(kFoldThreads), 0, s, a);
    return hipGetLastError();
}

template <int G, class E>
hipError_t launch_vec(const FoldArgs &a, int cus, hipStream_t s) {
    // Eight contributions in the workspace layout stream best with twice the
    // units per lane (measured: 46.5 against 48.3 us at 32 MiB each); with
    // other layouts that shape loses (51.6 against 49.5 us at 32 MiB
    // spacing), so it is kept to this one case.  Both shapes fold in the
    // same order and give the same bits.
    if (G == 8 && workspace_layout(a, G)) return launch_shape<G, 2 * FoldShape<G>::U, E>(a, cus, s);
    // A call too small to give every compute unit two workgroups at U units
    // per lane spreads over twice as many with one unit per lane (measured at
    // 393216 values x 8: 1.87-1.90 -> 1.78-1.81 us per call in a graph).
    constexpr int U = FoldShape<G>::U;
    if (U > 1 && a.nvec < static_cast<size_t>(2) * cus * kFoldThreads * U) return launch_shape<G, 1, E>(a, cus, s);
    return launch_shape<G, U, E>(a, cus, s);
}

template <class E>
hipError_t launch_vec_g(int G, const FoldArgs &a, int cus, hipStream_t s) {
    switch (G) {
        case 1: return launch_vec<1, E>(a, cus, s);
        case 2: return launch_vec<2, E>(a, cus, s);
        case 3: return launch_vec<3, E>(a, cus, s);
        case 4: return launch_vec<4, E>(a, cus, s);
        case 5: return launch_vec<5, E>(a, cus, s);
        case 6: return launch_vec<6, E>(a, cus, s);
        case 7: return launch_vec<7, E>(a, cus, s);
        case 8: return launch_vec<8, E>(a, cus, s);
        case 9: return launch_vec<9, E>(a, cus, s);
        case 10: return launch_vec<10, E>(a, cus, s);
        case 11: return launch_vec<11, E>(a, cus, s);
        case 12: return launch_vec<12, E>(a, cus, s);
        case 13: return launch_vec<13, E>(a, cus, s);
        case 14: return launch_vec<14, E>(a, cus, s);
        case 15: return launch_vec<15, E>(a, cus, s);
        case 16: return launch_vec<16, E>(a, cus, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t device_cu_count(int device, int *cus) {
    if (device < 0 || device >= 64) return hipErrorInvalidDevice;
    int c = g_cus[device].load(std::memory_order_relaxed);
    if (c <= 0) {
        hipError_t e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, device);
        if (e != hipSuccess) return e;
        if (c <= 0) return hipErrorInvalidDevice;
        g_cus[device].store(c, std::memory_order_relaxed);
    }
    *cus = c;
    return hipSuccess;
}

hipError_t stream_device(hr_stream_t stream, int *device) {
    if (stream == nullptr) return hipGetDevice(device);
    hipDevice_t d = 0;
    hipError_t e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &d);
    *device = static_cast<int>(d);
    return e;
}

}  // namespace hr

using namespace hr;

namespace {

template <class E>
hr_status reduce_impl(const void *const *inputs, int G, void *out, size_t numel, hr_stream_t stream) {
    if (G < 1 || G > HR_MAX_G) return HR_ERR_INVALID_ARG;
    if (numel == 0) return HR_OK;
    if (inputs == nullptr || out == nullptr) return HR_ERR_INVALID_ARG;
    if (numel > (SIZE_MAX / 2)) return HR_ERR_INVALID_ARG;
    const size_t bytes = numel * 2;
    FoldArgs a{};
    bool vec = aligned(out, 16);
    if (!aligned(out, 2)) return HR_ERR_ALIGNMENT;
    for (int g = 0; g < G; ++g) {
        if (inputs[g] == nullptr) return HR_ERR_INVALID_ARG;
        if (!aligned(inputs[g], 2)) return HR_ERR_ALIGNMENT;
        if (partial_overlap(inputs[g], out, bytes)) return HR_ERR_INVALID_ARG;
        vec = vec && aligned(inputs[g], 16);
        a.in[g] = inputs[g];
    }
    a.out = out;
    a.numel = numel;
    a.nvec = vec ? numel / kVecElems : 0;

    int dev = 0, cus = 0;
    if (stream_device(stream, &dev) != hipSuccess) return HR_ERR_HIP;
    if (device_cu_count(dev, &cus) != hipSuccess) return HR_ERR_HIP;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    hipError_t e;
    if (vec) {
        e = launch_vec_g<E>(G, a, cus, s);
    } else {
        const size_t blocks = (numel + kFoldThreads - 1) / kFoldThreads;
        const size_t cap = static_cast<size_t>(cus) * 32;
        hipLaunchKernelGGL(fold_scalar<E>, dim3(static_cast<unsigned>(blocks < cap ? blocks : cap)),
                           dim3(kFoldThreads), 0, s, a, G);
        e = hipGetLastError();
    }
    return e == hipSuccess ? HR_OK : HR_ERR_HIP;
}

}  // namespace

extern "C" HR_API hr_status hr_reduce_f16(const void *const *inputs, int G, void *out, size_t numel,
                                          hr_stream_t stream) {
    return reduce_impl<F16>(inputs, G, out, numel, stream);
}

extern "C" HR_API hr_status hr_reduce_bf16(const void *const *inputs, int G, void *out, size_t numel,
                                           hr_stream_t stream) {
    return reduce_impl<BF16>(inputs, G, out, numel, stream);
}

extern "C" HR_API const char *hr_status_str(hr_status s) {
    switch (s) {
        case HR_OK: return "HR_OK";
        case HR_ERR_INVALID_ARG: return "HR_ERR_INVALID_ARG";
        case HR_ERR_ALIGNMENT: return "HR_ERR_ALIGNMENT";
        case HR_ERR_TOO_LARGE: return "HR_ERR_TOO_LARGE";
        case HR_ERR_UNSUPPORTED: return "HR_ERR_UNSUPPORTED";
        case HR_ERR_HIP: return "HR_ERR_HIP";
        case HR_ERR_TIMEOUT: return "HR_ERR_TIMEOUT";
        case HR_ERR_ABORTED: return "HR_ERR_ABORTED";
    }
    return "HR_ERR_UNKNOWN";
}

extern "C" HR_API size_t hr_workspace_stride(size_t numel) {
    const size_t align = kWorkspaceAlign / sizeof(uint16_t);     // values
    return (numel + align - 1) / align * align + kWorkspaceShift / sizeof(uint16_t);
}
