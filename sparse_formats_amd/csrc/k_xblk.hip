// CSR run by column slices: y = alpha * A x + beta * y for matrices whose x
// is too large for one L2.
//
// The columns are cut into kXbBlocks slices and the rows into ranges of at
// most kXbCap rows with about equal entry counts.  Workgroup g (dispatched to
// XCD g mod 8) owns ranges g, g + grid, ...: it sums a range's rows in LDS
// over all slices, starting with slice g mod 8 and going round, so that the
// 32 workgroups of one XCD read one slice of x at about the same time, which
// stays in that XCD's L2 ("Sparse matrix-vector multiplication on GPGPU clusters", Sect.
// 2.3: the reuse of the right-hand side decides the traffic; random columns
// lose it, and a slice that fits a cache restores it).  The range's rows are
// then written once, y = alpha * s + beta * y: no atomics in global memory,
// no pass over y before, and no buffer of the apply's own, so applies of one
// handle may run at once on different streams.
//
// Inside a tile the entries are ordered by column and carry their row's
// offset in the range.  A wave reads packets of 64 consecutive entries (one
// per lane) and adds each product into its row's LDS slot.  The column order
// makes the workgroup sweep its slice of x from one end to the other: the
// lanes of a packet read neighbouring columns (one or two lines for a
// diagonal band, where several entries share a column), and the workgroups
// of an XCD, with equal shares of every slice, read each x line within a
// short time of each other.  When most entries lie near the diagonal, those
// within `band` columns of their range's rows form a ninth tile, summed
// after the slices, whose entries pack column and row offset into one 4-byte
// word (12 bytes per fp64 entry instead of 14).
//
// Measured per apply (fp64): power-law matrix (4 M rows, 42 M entries) 0.30
// ms against 0.40 ms with the entries of a tile in row order (products summed
// per row by a segmented scan over the lanes); FEM block (8 M rows, 398 M
// entries, 95 % of columns within +-10,000 of the diagonal) 1.03 ms with the
// packed band tile, 1.16 without it, 3.02 in row order.
#include "common.h"
#include "internal.h"

namespace spmv {
namespace {

constexpr int kXbUnroll = 8;        // packets a wave has in flight

template <typename T, int U>
struct XbPackets {
    int lr[U];  // row offset in the range
    int c[U];
    T v[U];
};

// Element at byte offset `off` of a wave-uniform base: the address is one
// scalar base plus a 32-bit offset per lane, which needs no 64-bit address
// arithmetic per lane.
template <typename T>
__device__ __forceinline__ T ld_at(const T* base, uint32_t off) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ T ld_nt_at(const T* base, uint32_t off) {
    return ld_nt(reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off));
}

// Load packets p, p + 64, ... of a tile ending at e1 (streamed, read once).
// Every lane loads: lanes past the end read the tile's last entry (a valid
// column for the gather; they add nothing).  Loads under a lane condition
// would make the compiler wait for each earlier load before the next gather,
// and so would a select on a loaded value here: the row offsets are masked
// when they are used.  The wave's entries are addressed from pb = min(p, e1
// - 1), so every offset is below 64 U.  A packed (band) tile has no row
// offset array: c holds column and row offset.
template <typename T, int U, bool kPk>
__device__ __forceinline__ void xb_load(const XblkView& a, int p, int e1, int lane,
                                        XbPackets<T, U>& q) {
    const int pb = min(p, e1 - 1);  // wave-uniform
    const int* __restrict__ col = a.col + pb;
    const T* __restrict__ val = static_cast<const T*>(a.val) + pb;
    const uint16_t* __restrict__ lrow = a.lrow + pb;
    uint32_t o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) o[u] = (uint32_t)(min(p + u * 64 + lane, e1 - 1) - pb);
    // the columns first: the gathers wait only for them
#pragma unroll
    for (int u = 0; u < U; ++u) q.c[u] = ld_nt_at(col, o[u] * 4);
#pragma unroll
    for (int u = 0; u < U; ++u) q.v[u] = ld_nt_at(val, o[u] * (uint32_t)sizeof(T));
    if constexpr (!kPk) {
#pragma unroll
        for (int u = 0; u < U; ++u) q.lr[u] = ld_nt_at(lrow, o[u] * 2);
    }
}

// One round: gather x for the packets in q (at p), load the packets one
// stride on into nq (past the tile's end they read its last entry again),
// then add each of q's products into its row's LDS slot.  Columns are below
// n < 2^28, so their byte offsets in x fit 32 bits.  cb: the first column of
// a packed tile's band.
template <typename T, int U, bool kPk>
__device__ __forceinline__ void xb_round(const XblkView& a, const T* __restrict__ x, T* part,
                                         int p, int e1, int lane, int cb,
                                         const XbPackets<T, U>& q, XbPackets<T, U>& nq) {
    constexpr int kStride = kXbThreads * U;
    constexpr int LB = kXbRowBits<T>;
    T xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t c = kPk ? (uint32_t)(cb + (int)((uint32_t)q.c[u] >> LB)) : (uint32_t)q.c[u];
        xv[u] = ld_at(x, c * (uint32_t)sizeof(T));
    }
    xb_load<T, U, kPk>(a, p + kStride, e1, lane, nq);
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (p + u * 64 + lane < e1) {
            const int lr = kPk ? (int)((uint32_t)q.c[u] & ((1u << LB) - 1)) : q.lr[u];
            __hip_atomic_fetch_add(part + lr, q.v[u] * xv[u], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
}

// The sets of packets of one tile: two sets in turn (no register copies
// between rounds, which would wait for every load in flight): a round
// gathers x for one set, loads the other, then sums the first.
template <typename T, int U, bool kPk>
__device__ __forceinline__ void xb_tile(const XblkView& a, const T* __restrict__ x, T* part,
                                        int p, int e1, int lane, int cb) {
    constexpr int kStride = kXbThreads * U;
    XbPackets<T, U> qa, qb;
    xb_load<T, U, kPk>(a, p, e1, lane, qa);
    for (;;) {
        xb_round<T, U, kPk>(a, x, part, p, e1, lane, cb, qa, qb);
        p += kStride;
        if (p >= e1) break;
        xb_round<T, U, kPk>(a, x, part, p, e1, lane, cb, qb, qa);
        p += kStride;
        if (p >= e1) break;
    }
}

template <typename T, int U>
__global__ __launch_bounds__(kXbThreads) void k_xblk(XblkView a, const T* __restrict__ x,
                                                     T* __restrict__ y, T alpha, T beta) {
    __shared__ T part[kXbCap<T>];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int first = (int)(blockIdx.x & 7) * (kXbBlocks / 8);  // this XCD's first slice
    for (int64_t r = blockIdx.x; r < a.ranges; r += gridDim.x) {
        const int rb = a.row_begin[r], nr = a.row_begin[r + 1] - rb;
        for (int i = threadIdx.x; i < nr; i += kXbThreads) part[i] = T(0);
        __syncthreads();
        // the slices from this XCD's own on (the workgroups of an XCD, with
        // equal shares of each slice, read the same slice of x at about the
        // same time), as two runs of consecutive tiles, then the range's
        // band.  The waves do not wait for each other between tiles: the LDS
        // adds commute, and the packets of a run are dealt to the waves in
        // turn, so they stay within about a round of each other (a barrier
        // after every tile was 1 % slower on the FEM block and 3.5 % on the
        // power-law matrix, whose slice tiles take one or two rounds each).
        {
            const int t0 = (int)r * kXbTiles;
            for (int h = 0; h < 2; ++h) {
                const int e0 = a.tile_ptr[t0 + (h ? 0 : first)];
                const int e1 = a.tile_ptr[t0 + (h ? first : kXbBlocks)];
                const int p = e0 + wv * 64 * U;
                if (p < e1) xb_tile<T, U, false>(a, x, part, p, e1, lane, 0);  // wave-uniform
            }
            const int e0 = a.tile_ptr[t0 + kXbBlocks], e1 = a.tile_ptr[t0 + kXbTiles];
            const int p = e0 + wv * 64 * U;
            if (p < e1) xb_tile<T, U, true>(a, x, part, p, e1, lane, rb - (int)a.band);
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
        const int r = row_of(a.row_begin, 0, (int)a.ranges - 1, i);
        const int rb = a.row_begin[r], nr = a.row_begin[r + 1] - rb;
        int c = 0;  // lane b: entries in tile b
        for (int e = rowptr[i] + lane; e - lane < e1; e += 64) {
            const int b = e < e1 ? xblk_tile(col[e], rb, nr, a.band, a.width, kXbBlocks) : -1;
#pragma unroll
            for (int bb = 0; bb < kXbTiles; ++bb) {
                const int k = __popcll(__ballot(b == bb));
                c += lane == bb ? k : 0;
            }
        }
        if (lane < kXbTiles) cnt[xblk_slot(rb, nr, lane, i, kXbTiles)] = c;
    }
}

// setup: tile (r, b) starts at the scanned count of its first position
__global__ __launch_bounds__(256) void k_xblk_tiles(XblkView a, const int* __restrict__ pos,
                                                    int* __restrict__ tile_ptr) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.ranges * kXbTiles) return;
    const int64_t r = t / kXbTiles;
    const int b = (int)(t % kXbTiles);
    const int rb = a.row_begin[r];
    tile_ptr[t] = pos[xblk_slot(rb, a.row_begin[r + 1] - rb, b, rb, kXbTiles)];
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
        const int rb = a.row_begin[r], nr = a.row_begin[r + 1] - rb;
        const uint16_t lr = (uint16_t)(i - rb);
        // lane b holds the next position of tile b
        int at = lane < kXbTiles ? pos[xblk_slot(rb, nr, lane, i, kXbTiles)] : 0;
        for (int e = rowptr[i] + lane; e - lane < e1; e += 64) {
            const bool in = e < e1;
            const int cv = in ? col[e] : 0;
            const int b = in ? xblk_tile(cv, rb, nr, a.band, a.width, kXbBlocks) : -1;
            int o = 0;
#pragma unroll
            for (int bb = 0; bb < kXbTiles; ++bb) {
                const uint64_t mk = __ballot(b == bb);
                const int p = __shfl(at, bb);
                if (b == bb) o = p + __popcll(mk & below);
                at += lane == bb ? __popcll(mk) : 0;
            }
            if (in) {
                // a band entry: column less the band's first, and row offset
                ocol[o] = b == kXbBlocks ? (int)xblk_pack(cv, rb, a.band, lr, a.lbits) : cv;
                oval[o] = val[e];
                olrow[o] = lr;
            }
        }
    }
}

// setup: val and row offsets in the order of the column sort (src[k] is the
// old place of entry k)
template <typename T>
__global__ __launch_bounds__(256) void k_xblk_gather(int64_t nnz, const int* __restrict__ src,
                                                     const T* __restrict__ val,
                                                     const uint16_t* __restrict__ lrow,
                                                     T* __restrict__ oval,
                                                     uint16_t* __restrict__ olrow) {
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int j = src[k];
        oval[k] = val[j];
        olrow[k] = lrow[j];
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
    const int64_t t = a.ranges * kXbTiles;
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

hipError_t launch_xblk_gather(int64_t nnz, bool f64, const int* src, const void* val,
                              const uint16_t* lrow, void* oval, uint16_t* olrow, hipStream_t s) {
    if (nnz == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((nnz + 255) / 256, 65536);
    if (f64)
        hipLaunchKernelGGL(k_xblk_gather<double>, dim3(grid), dim3(256), 0, s, nnz, src,
                           static_cast<const double*>(val), lrow, static_cast<double*>(oval),
                           olrow);
    else
        hipLaunchKernelGGL(k_xblk_gather<float>, dim3(grid), dim3(256), 0, s, nnz, src,
                           static_cast<const float*>(val), lrow, static_cast<float*>(oval), olrow);
    return hipGetLastError();
}

}  // namespace spmv
