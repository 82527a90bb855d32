// CSR run by column slices: y = alpha * A x + beta * y for matrices whose x
// reads are scattered over an x too large for one L2.
//
// The columns are cut into kXbBlocks slices and the rows into ranges of at
// most kXbCap rows with about equal entry counts.  Workgroup g (dispatched to
// XCD g mod 8) owns ranges g, g + grid, ...: it sums a range's rows in LDS
// over all slices, starting with slice g mod 8 and going round, so that at any
// time the 32 workgroups of one XCD read one slice of x, which stays in that
// XCD's L2 ("Sparse matrix-vector multiplication on GPGPU clusters", Sect.
// 2.3: the reuse of the right-hand side decides the traffic; random columns
// lose it, and a slice that fits a cache restores it).  The range's rows are
// then written once, y = alpha * s + beta * y: no atomics in global memory,
// no pass over y before, and no buffer of the apply's own, so applies of one
// handle may run at once on different streams.
//
// Inside a tile the entries are ordered by row and carry their row's offset
// in the range.  A wave reads packets of 64 consecutive entries (one per
// lane), sums each packet's products per row with a segmented scan over the
// lanes, and the last lane of each row's run adds the sum into the row's LDS
// slot.  Measured on the power-law matrix (4 M rows, 42 M entries): against
// 0.42 ms when every slice added its row sums into y with device atomics
// after a pass that wrote beta * y.
#include "common.h"
#include "internal.h"

namespace spmv {
namespace {

constexpr int kNoRow = 0x7fffffff;  // lanes past the tile's end
constexpr int kXbUnroll = 4;        // packets a wave has in flight

template <typename T, int U>
struct XbPackets {
    int lr[U];  // row offset in the range
    int c[U];
    T v[U];
};

// Load packets p, p + 64, ... of a tile ending at e1 (streamed, read once).
// Every lane loads: lanes past the end read the tile's last entry (a valid
// column for the gather; they add nothing).  Loads under a lane condition
// would make the compiler wait for each earlier load before the next gather,
// and so would a select on a loaded value here: the row offsets are masked
// when they are used.
template <typename T, int U>
__device__ __forceinline__ void xb_load(const XblkView& a, int p, int e1, int lane,
                                        XbPackets<T, U>& q) {
    const T* __restrict__ val = static_cast<const T*>(a.val);
    int es[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = p + u * 64 + lane;
        es[u] = e < e1 ? e : e1 - 1;
    }
    // the columns first: the gathers wait only for them
#pragma unroll
    for (int u = 0; u < U; ++u) q.c[u] = ld_nt(a.col + es[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) q.v[u] = ld_nt(val + es[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) q.lr[u] = ld_nt(a.lrow + es[u]);
}

// One round: gather x for the packets in q (at p), load the packets one
// stride on into nq (past the tile's end they read its last entry again),
// then add q's products into the rows' LDS slots: each packet's products are
// summed per row by a segmented scan over the lanes and the last lane of
// each row's run adds the sum.
template <typename T, int U>
__device__ __forceinline__ void xb_round(const XblkView& a, const T* __restrict__ x, T* part,
                                         int p, int e1, int lane, const XbPackets<T, U>& q,
                                         XbPackets<T, U>& nq) {
    constexpr int kStride = kXbThreads * U;
    T xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) xv[u] = x[q.c[u]];
    xb_load(a, p + kStride, e1, lane, nq);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int key = p + u * 64 + lane < e1 ? q.lr[u] : kNoRow;
        const T sum = segmented_scan(key, q.v[u] * xv[u]);
        const int next = dpp_or<0x130, 0xF>(-1, key);  // lane + 1 (none for 63)
        if (key != kNoRow && next != key)
            __hip_atomic_fetch_add(part + key, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

template <typename T, int U>
__global__ __launch_bounds__(kXbThreads) void k_xblk(XblkView a, const T* __restrict__ x,
                                                     T* __restrict__ y, T alpha, T beta) {
    __shared__ T part[kXbCap<T>];
    constexpr int kStride = kXbThreads * U;  // the workgroup's packets of one round
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int first = (int)(blockIdx.x & 7) * (kXbBlocks / 8);  // this XCD's first slice
    for (int64_t r = blockIdx.x; r < a.ranges; r += gridDim.x) {
        const int rb = a.row_begin[r], nr = a.row_begin[r + 1] - rb;
        for (int i = threadIdx.x; i < nr; i += kXbThreads) part[i] = T(0);
        __syncthreads();
        for (int s = 0; s < kXbBlocks; ++s) {
            const int b = (first + s) % kXbBlocks;
            const int e1 = a.tile_ptr[r * kXbBlocks + b + 1];
            int p = a.tile_ptr[r * kXbBlocks + b] + wv * 64 * U;
            if (p < e1) {  // wave-uniform, as is the loop below
                // two sets of packets in turn (no register copies between
                // rounds, which would wait for every load in flight): a
                // round gathers x for one set, loads the other, then sums
                // the first
                XbPackets<T, U> qa, qb;
                xb_load(a, p, e1, lane, qa);
                for (;;) {
                    xb_round(a, x, part, p, e1, lane, qa, qb);
                    p += kStride;
                    if (p >= e1) break;
                    xb_round(a, x, part, p, e1, lane, qb, qa);
                    p += kStride;
                    if (p >= e1) break;
                }
            }
            // the waves move to the next slice together, so that the x
            // reads of the workgroup stay within one slice
            __syncthreads();
        }
        // alpha * 0 is NaN for a non-finite alpha, as the definition gives;
        // beta == 0 never reads y.  With beta, a thread's y loads all go out
        // before its stores (indices past the range read its last row).
        if (beta == T(0)) {
            for (int i = threadIdx.x; i < nr; i += kXbThreads)
                y[(int64_t)rb + i] = alpha * part[i];
        } else {
            constexpr int kPer = kXbCap<T> / kXbThreads;
            T yv[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = (int)threadIdx.x + k * kXbThreads;
                yv[k] = y[(int64_t)rb + (i < nr ? i : nr - 1)];
            }
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = (int)threadIdx.x + k * kXbThreads;
                if (i < nr) y[(int64_t)rb + i] = alpha * part[i] + beta * yv[k];
            }
        }
        __syncthreads();
    }
}

// setup: the candidate range starts (one thread per candidate)
__global__ __launch_bounds__(256) void k_xblk_bounds(int64_t n, int64_t nnz,
                                                     const int* __restrict__ rowptr, int64_t R0,
                                                     int* __restrict__ cand) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r <= R0) cand[r] = xblk_bound(rowptr, (int)n, nnz, r, R0);
}

// setup, one wave per row (rows of any length): lane b counts row i's entries
// in slice b and stores the count at its xblk_slot position
__global__ __launch_bounds__(256) void k_xblk_count(XblkView a, const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    int* __restrict__ cnt) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); i < a.n;
         i += waves) {
        const int e1 = rowptr[i + 1];
        int c = 0;  // lane b: entries in slice b
        for (int e = rowptr[i] + lane; e - lane < e1; e += 64) {
            const int b = e < e1 ? (int)(col[e] / a.width) : -1;
#pragma unroll
            for (int bb = 0; bb < kXbBlocks; ++bb) {
                const int k = __popcll(__ballot(b == bb));
                c += lane == bb ? k : 0;
            }
        }
        if (lane < kXbBlocks) {
            const int r = row_of(a.row_begin, 0, (int)a.ranges - 1, i);
            const int rb = a.row_begin[r];
            cnt[xblk_slot(rb, a.row_begin[r + 1] - rb, lane, i, kXbBlocks)] = c;
        }
    }
}

// setup: tile (r, b) starts at the scanned count of its first position
__global__ __launch_bounds__(256) void k_xblk_tiles(XblkView a, const int* __restrict__ pos,
                                                    int* __restrict__ tile_ptr) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.ranges * kXbBlocks) return;
    const int64_t r = t / kXbBlocks;
    const int b = (int)(t % kXbBlocks);
    const int rb = a.row_begin[r];
    tile_ptr[t] = pos[xblk_slot(rb, a.row_begin[r + 1] - rb, b, rb, kXbBlocks)];
}

// setup, one wave per row: copy row i's entries into its tiles in their
// original order (each pass of 64 entries places the lanes of every slice
// by their rank among that slice's lanes) with the row's offset in its range
template <typename T>
__global__ __launch_bounds__(256) void k_xblk_fill(XblkView a, const int* __restrict__ rowptr,
                                                   const int* __restrict__ col,
                                                   const T* __restrict__ val,
                                                   const int* __restrict__ pos,
                                                   int* __restrict__ ocol, T* __restrict__ oval,
                                                   uint16_t* __restrict__ olrow) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = __lanemask_lt();
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); i < a.n;
         i += waves) {
        const int e1 = rowptr[i + 1];
        const int r = row_of(a.row_begin, 0, (int)a.ranges - 1, i);
        const int rb = a.row_begin[r];
        const uint16_t lr = (uint16_t)(i - rb);
        // lane b holds the next position of slice b
        int at = lane < kXbBlocks
                     ? pos[xblk_slot(rb, a.row_begin[r + 1] - rb, lane, i, kXbBlocks)]
                     : 0;
        for (int e = rowptr[i] + lane; e - lane < e1; e += 64) {
            const bool in = e < e1;
            const int cv = in ? col[e] : 0;
            const int b = in ? (int)(cv / a.width) : -1;
            int o = 0;
#pragma unroll
            for (int bb = 0; bb < kXbBlocks; ++bb) {
                const uint64_t mk = __ballot(b == bb);
                const int p = __shfl(at, bb);
                if (b == bb) o = p + __popcll(mk & below);
                at += lane == bb ? __popcll(mk) : 0;
            }
            if (in) {
                ocol[o] = cv;
                oval[o] = val[e];
                olrow[o] = lr;
            }
        }
    }
}

template <typename T>
hipError_t run(const XblkView& a, void* y, const void* x, double alpha, double beta,
               hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>(a.ranges, kXbGroups);
    hipLaunchKernelGGL((k_xblk<T, kXbUnroll>), dim3(grid), dim3(kXbThreads), 0, s, a,
                       static_cast<const T*>(x), static_cast<T*>(y), (T)alpha, (T)beta);
    return hipGetLastError();
}

// one wave per row, four rows per workgroup
unsigned row_wave_grid(int64_t n) { return (unsigned)std::min<int64_t>((n + 3) / 4, 65536); }

}  // namespace

hipError_t launch_xblk(const XblkView& a, bool f64, void* y, const void* x, double alpha,
                       double beta, hipStream_t s) {
    return f64 ? run<double>(a, y, x, alpha, beta, s) : run<float>(a, y, x, alpha, beta, s);
}

hipError_t launch_xblk_bounds(int64_t n, int64_t nnz, const int* rowptr, int64_t R0, int* cand,
                              hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_xblk_bounds, dim3((unsigned)((R0 + 256) / 256)), dim3(256), 0, s, n, nnz,
                       rowptr, R0, cand);
    return hipGetLastError();
}

hipError_t launch_xblk_count(const XblkView& a, const int* rowptr, const int* col, int* cnt,
                             hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_xblk_count, dim3(row_wave_grid(a.n)), dim3(256), 0, s, a, rowptr, col,
                       cnt);
    return hipGetLastError();
}

hipError_t launch_xblk_tiles(const XblkView& a, const int* pos, int* tile_ptr, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const int64_t t = a.ranges * kXbBlocks;
    hipLaunchKernelGGL(k_xblk_tiles, dim3((unsigned)((t + 255) / 256)), dim3(256), 0, s, a, pos,
                       tile_ptr);
    return hipGetLastError();
}

hipError_t launch_xblk_fill(const XblkView& a, bool f64, const int* rowptr, const int* col,
                            const void* val, const int* pos, int* ocol, void* oval,
                            uint16_t* olrow, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    if (f64)
        hipLaunchKernelGGL(k_xblk_fill<double>, dim3(row_wave_grid(a.n)), dim3(256), 0, s, a,
                           rowptr, col, static_cast<const double*>(val), pos, ocol,
                           static_cast<double*>(oval), olrow);
    else
        hipLaunchKernelGGL(k_xblk_fill<float>, dim3(row_wave_grid(a.n)), dim3(256), 0, s, a,
                           rowptr, col, static_cast<const float*>(val), pos, ocol,
                           static_cast<float*>(oval), olrow);
    return hipGetLastError();
}

}  // namespace spmv
