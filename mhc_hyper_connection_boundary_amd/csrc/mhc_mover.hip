// Movers: kernels that move exactly the boundary's activation bytes (read the
// residual X [T][4][d] and the block output x [T][d]; write X' [T][4][d] and a
// [T][d] buffer in place of the layer input) and compute nothing.  Their rate
// is the ceiling an HBM-bound boundary kernel with the same access pattern can
// reach on this device; bench.py reports it beside the boundary's own rate.
// This library (libmhc_mover.so) is a measurement tool: mhc_boundary never
// calls it.
//
//   mode 0  tile-major items of 32 tokens x 256 elements, one workgroup each;
//           each load / store instruction covers 2 rows x 512 contiguous bytes;
//           nontemporal loads and stores (the fastest pattern measured)
//   mode 1  as mode 0 with plain loads and stores
//   mode 2  the streaming schedule's pattern: one persistent workgroup per
//           compute unit over tile-major items of 64 tokens x 256 elements in
//           steps of 64 elements; lane (n, g) of wave w covers token 16w + n,
//           both 64-byte halves of a 128-byte line per row; the next step is
//           requested before the current one is stored; a workgroup barrier
//           per step
//   mode 3  as mode 0 with items of 32 tokens x 512 elements: each load /
//           store instruction covers 1 row x 1024 contiguous bytes;
//           nontemporal (measured faster than mode 0)
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// A cheap change of the bits so that nothing is a plain copy the compiler could elide.
__device__ __forceinline__ u32x4_t touch(u32x4_t v) {
    v.x ^= 0x10001u;
    v.y += 1u;
    return v;
}

struct MoverArgs {
    int T, hidden;
    const char* X;
    const char* x;
    char* Xo;
    char* lo;
    unsigned xbytes, sbytes;  // bytes of X (and X'), of x (and lo)
};

// Modes 0, 1 and 3: item blockIdx.x = (tile of 32 tokens, slice of 256 or,
// for one row per instruction, 512 elements).
template <int AUX, int RPI>  // RPI: rows per load / store instruction (2 or 1)
__global__ __launch_bounds__(256) void k_mover_rows(MoverArgs a) {
    constexpr int kRunBytes = 1024 / RPI;  // contiguous bytes of a row per instruction
    constexpr int kInst = 40 / RPI;        // instructions per wave
    const int slices = a.hidden * 2 / kRunBytes;
    const int tile = blockIdx.x / slices, slice = blockIdx.x - tile * slices;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const unsigned row_bytes = (unsigned)a.hidden * 2;
    const auto rX = rsrc(a.X, a.xbytes), rx = rsrc(a.x, a.sbytes);
    const auto rXo = rsrc(a.Xo, a.xbytes), rlo = rsrc(a.lo, a.sbytes);
    // 160 rows per item: 128 of X (32 tokens x 4 streams), 32 of x; wave w
    // takes rows 40w .. 40w + 39, instruction k rows 40w + RPI*k .. + RPI - 1.
    u32x4_t v[kInst];
    unsigned off[kInst];
#pragma unroll
    for (int k = 0; k < kInst; ++k) {
        const int row = 40 * w + RPI * k + l / (64 / RPI);
        const unsigned col = (unsigned)slice * kRunBytes + (l % (64 / RPI)) * 16;
        off[k] = row < 128 ? ((unsigned)tile * 128 + row) * row_bytes + col
                           : ((unsigned)tile * 32 + row - 128) * row_bytes + col;
        v[k] = row < 128 ? __builtin_amdgcn_raw_buffer_load_b128(rX, off[k], 0, AUX)
                         : __builtin_amdgcn_raw_buffer_load_b128(rx, off[k], 0, AUX);
    }
#pragma unroll
    for (int k = 0; k < kInst; ++k) {
        const int row = 40 * w + RPI * k + l / (64 / RPI);
        if (row < 128)
            __builtin_amdgcn_raw_buffer_store_b128(touch(v[k]), rXo, off[k], 0, AUX);
        else
            __builtin_amdgcn_raw_buffer_store_b128(touch(v[k]), rlo, off[k], 0, AUX);
    }
}

// Mode 2: workgroup g takes items g, g + G, ... (tile-major; G = gridDim.x).
struct Step {
    u32x4_t X[2][4];
    u32x4_t x[2];
};

__global__ __launch_bounds__(256) void k_mover_stream(MoverArgs a) {
    const int slices = a.hidden / 256, items = (a.T / 64) * slices;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;
    const unsigned row_bytes = (unsigned)a.hidden * 2, row = 16 * w + n;
    const auto rX = rsrc(a.X, a.xbytes), rx = rsrc(a.x, a.sbytes);
    const auto rXo = rsrc(a.Xo, a.xbytes), rlo = rsrc(a.lo, a.sbytes);
    const int G = gridDim.x;
    if ((int)blockIdx.x >= items) return;
    const int positions = ((items - 1 - (int)blockIdx.x) / G + 1) * 4;  // (item, step) pairs
    auto offsets = [&](int p, unsigned& oX, unsigned& ox) {
        const int item = (int)blockIdx.x + (p >> 2) * G;
        const int tile = item / slices, slice = item - tile * slices;
        const unsigned t = (unsigned)tile * 64 + row;
        const unsigned col = ((unsigned)slice * 256 + (p & 3) * 64 + g * 8) * 2;
        oX = t * 4 * row_bytes + col;
        ox = t * row_bytes + col;
    };
    auto load = [&](Step& s, int p) {
        unsigned oX, ox;
        offsets(p, oX, ox);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                s.X[h][j] = __builtin_amdgcn_raw_buffer_load_b128(rX, oX + h * 64, j * row_bytes, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) s.x[h] = __builtin_amdgcn_raw_buffer_load_b128(rx, ox + h * 64, 0, 0);
    };
    Step cur;
    load(cur, 0);
    for (int p = 0; p < positions; ++p) {
        Step nxt;
        const bool more = p + 1 < positions;
        if (more) load(nxt, p + 1);
        unsigned oX, ox;
        offsets(p, oX, ox);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(touch(cur.X[h][j]), rXo, oX + h * 64, j * row_bytes, 0);
            __builtin_amdgcn_raw_buffer_store_b128(touch(cur.x[h]), rlo, ox + h * 64, 0, 0);
        }
        __syncthreads();
        if (more) cur = nxt;
    }
}

}  // namespace

extern "C" {

// Moves the activation bytes of a boundary call of `tokens` tokens and width
// `hidden` in mode 0, 1 or 2 (above).  X, Xo: tokens*4*hidden bf16 values;
// x, lo: tokens*hidden; all device pointers, 16-byte aligned, caller-owned.
// Returns 0 on success, 1 for arguments outside the movers' shapes (tokens a
// positive multiple of 64, hidden a multiple of 256 in [256, 16384] (of 512
// for mode 3), X under 4 GiB, non-null pointers, mode in 0..3), 2 if the
// launch failed.
int mhc_mover_run(int tokens, int hidden, const void* X, const void* x, void* Xo, void* lo, int mode,
                  void* stream) {
    if (tokens <= 0 || tokens % 64 != 0 || hidden < 256 || hidden > 16384 || hidden % 256 != 0)
        return 1;
    if (!X || !x || !Xo || !lo || mode < 0 || mode > 3) return 1;
    if (mode == 3 && hidden % 512 != 0) return 1;
    const uint64_t xbytes = (uint64_t)tokens * 4 * hidden * 2;
    if (xbytes >= ((uint64_t)1 << 32)) return 1;
    MoverArgs a;
    a.T = tokens;
    a.hidden = hidden;
    a.X = static_cast<const char*>(X);
    a.x = static_cast<const char*>(x);
    a.Xo = static_cast<char*>(Xo);
    a.lo = static_cast<char*>(lo);
    a.xbytes = (unsigned)xbytes;
    a.sbytes = (unsigned)(xbytes / 4);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int items32 = (tokens / 32) * (hidden / 256);
    if (mode == 0) {
        hipLaunchKernelGGL((k_mover_rows<2, 2>), dim3(items32), dim3(256), 0, s, a);
    } else if (mode == 1) {
        hipLaunchKernelGGL((k_mover_rows<0, 2>), dim3(items32), dim3(256), 0, s, a);
    } else if (mode == 3) {
        hipLaunchKernelGGL((k_mover_rows<2, 1>), dim3((tokens / 32) * (hidden / 512)), dim3(256), 0, s, a);
    } else {
        int dev = 0, units = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&units, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            units <= 0)
            return 2;
        hipLaunchKernelGGL(k_mover_stream, dim3(units), dim3(256), 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
