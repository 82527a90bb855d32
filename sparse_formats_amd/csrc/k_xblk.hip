// CSR run by column blocks, one block per XCD: y = alpha * A x + beta * y
// for matrices whose x reads are scattered over an x too large for one L2.
//
// The columns are cut into kXbBlocks slices of `width` columns; the entries
// of slice b form a "tall" CSR matrix of n rows (tall row b * n + i holds
// row i's entries with columns in slice b, in their original order).  The
// waves of slice b all run on XCD b, so slice b's x reads hit that XCD's
// L2 ("Sparse matrix-vector multiplication on GPGPU clusters", Sect. 2.3:
// the reuse of the right-hand side decides the traffic; random columns lose
// it, and a slice that fits a cache restores it).  A first pass writes
// beta * y; every slice then adds alpha times its row sums into y with
// return-less atomics, so an apply keeps no buffer of its own and applies of
// one handle may run at once on different streams.
//
// Work is split by merged items, as in the load-balanced CSR kernels of
// "Load-balancing Sparse Matrix Vector Product Kernels on GPUs" (abstract):
// the items of a slice are its entries and one end marker per row, in row
// order (row t covers positions t + ptr[t] .. t + ptr[t + 1], the last one
// its end marker).  A wave takes kXbChunk consecutive items of one slice, a
// lane kXbItems of them.  A wave sums its rows in LDS (one slot per row
// ending in the wave, plus one for the row still open at its end) and adds
// each slot into y; a row that spans several waves gets one addition from
// each.
#include "common.h"
#include "internal.h"

namespace spmv {
namespace {

// one wave's chunk: every entry is added into its row's LDS slot, then the
// slots are added into y.  A lane finds its entries' rows from the row ends
// it reads: with four-bit counters of the rows ending at each of its entry
// offsets, one multiply gives every entry's row offset (a prefix sum in the
// counters).  Measured on the power-law matrix (4 M rows): 0.42 ms per apply
// against 0.48 ms when the slices wrote 8 dense partial products per row
// that a last kernel summed (about 24 M atomics replace 0.5 GB of partial
// products written and read back).
template <typename T>
__global__ __launch_bounds__(256) void k_xblk(XblkView a, const T* __restrict__ x,
                                              T* __restrict__ y, T alpha) {
    constexpr int I = kXbItems, SL = kXbChunk + 1;
    static_assert(I <= 8, "four-bit counters of at most 8 rows, 8 offsets");
    __shared__ T stage[4 * SL];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // the grid is kXbBlocks * tiles workgroups (< 2^26): 32-bit division
    const uint32_t g = (uint32_t)xcd_tile(blockIdx.x, gridDim.x), tiles = (uint32_t)a.tiles;
    const int b = (int)(g / tiles);  // slice b on XCD b
    const int64_t k = (int64_t)(g - (uint32_t)b * tiles) * 4 + wv;
    if (b >= kXbBlocks || a.wave_base[b] + k >= a.wave_base[b + 1]) return;
    const int64_t w = a.wave_base[b] + k;
    const int64_t wbeg = a.item0[b] + k * kXbChunk;
    const int64_t wend = min(wbeg + kXbChunk, a.item0[b + 1]);
    const int64_t d0 = wbeg + (int64_t)lane * I;
    const int items = d0 < wend ? (int)min<int64_t>(I, wend - d0) : 0;
    const int r0 = a.lane_row[w * 64 + lane];  // a valid row for every lane
    const int e0 = items > 0 ? (int)(d0 - r0) : 0;  // first entry (<= nnz)
    T* st = stage + wv * SL;
    for (int i = lane; i < SL; i += 64) st[i] = T(0);
    // ends of rows r0 .. r0 + I - 1 (the pointer holds I copies of nnz past
    // its end); a row ending at entry offset re < I of the lane is counted
    // in four-bit field re; rows r0 .. r0 + c - 1 end inside the lane's items
    int c;
    const uint32_t pre = xblk_row_offsets<I>(a.ptr + r0 + 1, e0, items, &c);
    const int m = items - c;  // entries e0 .. e0 + m - 1
    // the entry arrays hold I - 1 padding entries past nnz
    const T* __restrict__ val = static_cast<const T*>(a.val) + e0;
    const int* __restrict__ col = a.col + e0;
    T pr[I];
    int cc[I];
#pragma unroll
    for (int kk = 0; kk < I; ++kk) cc[kk] = col[kk], pr[kk] = val[kk];
#pragma unroll
    for (int kk = 0; kk < I; ++kk)
        if (kk < m) pr[kk] *= x[cc[kk]];
    const int rs = __builtin_amdgcn_readfirstlane(r0);  // lane 0 always holds items
    const int base = r0 - rs;
    wave_lds_sync();
#pragma unroll
    for (int kk = 0; kk < I; ++kk)
        if (kk < m)
            __hip_atomic_fetch_add(st + base + ((pre >> (4 * kk)) & 15), pr[kk], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t act = __ballot(items > 0);
    const int last = 63 - __clzll((long long)act);
    const int endrow = __shfl(r0 + c, last);  // first row not closed in this wave
    const int nclosed = endrow - rs;
    wave_lds_sync();
    // the rows closed in this wave and the one still open at its end (none
    // past the slice's last row) go into y; a zero sum is left out unless
    // alpha is not finite (alpha * 0 is then NaN, as the definition gives)
    const bool open_row = (int64_t)endrow < (int64_t)(b + 1) * a.n;
    const int64_t off = (int64_t)b * a.n;
    const bool fin = alpha - alpha == T(0);
    for (int i = lane; i < nclosed + (open_row ? 1 : 0); i += 64) {
        const T v = st[i];
        if (v != T(0) || !fin) atomic_add(y + (rs + i - off), alpha * v);
    }
}

// setup, one wave per row (rows of any length): entries of row i in each
// slice (lane b writes slice b's count)
__global__ __launch_bounds__(256) void k_xblk_count(int64_t n, int64_t width,
                                                    const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    int* __restrict__ cnt) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); i < n;
         i += waves) {
        const int e1 = rowptr[i + 1];
        int c = 0;  // lane b: entries in slice b
        for (int e = rowptr[i] + lane; e - lane < e1; e += 64) {
            const int b = e < e1 ? (int)(col[e] / width) : -1;
#pragma unroll
            for (int bb = 0; bb < kXbBlocks; ++bb) {
                const int k = __popcll(__ballot(b == bb));
                c += lane == bb ? k : 0;
            }
        }
        if (lane < kXbBlocks) cnt[lane * n + i] = c;
    }
}

// setup, one wave per row: copy row i's entries to its tall rows in their
// original order (each pass of 64 entries places the lanes of every slice
// by their rank among that slice's lanes)
template <typename T>
__global__ __launch_bounds__(256) void k_xblk_fill(int64_t n, int64_t width,
                                                   const int* __restrict__ rowptr,
                                                   const int* __restrict__ col,
                                                   const T* __restrict__ val,
                                                   const int* __restrict__ ptr,
                                                   int* __restrict__ ocol, T* __restrict__ oval) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = __lanemask_lt();
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); i < n;
         i += waves) {
        const int e1 = rowptr[i + 1];
        // lane b holds the next position of slice b
        int pos = lane < kXbBlocks ? ptr[lane * n + i] : 0;
        for (int e = rowptr[i] + lane; e - lane < e1; e += 64) {
            const bool in = e < e1;
            const int cv = in ? col[e] : 0;
            const int b = in ? (int)(cv / width) : -1;
            int o = 0;
#pragma unroll
            for (int bb = 0; bb < kXbBlocks; ++bb) {
                const uint64_t mk = __ballot(b == bb);
                const int p = __shfl(pos, bb);
                if (b == bb) o = p + __popcll(mk & below);
                pos += lane == bb ? __popcll(mk) : 0;
            }
            if (in) {
                ocol[o] = cv;
                oval[o] = val[e];
            }
        }
    }
}

// setup: the tall row holding the first item of every lane (lane j of a
// slice starts at item kXbItems * j of the slice)
__global__ __launch_bounds__(256) void k_xblk_lane_rows(XblkView a, int* __restrict__ lane_row) {
    const int64_t R = (int64_t)kXbBlocks * a.n;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < R; t += stride) {
        const int b = (int)(t / a.n);
        const int64_t rel0 = t + a.ptr[t] - a.item0[b], rel1 = t + a.ptr[t + 1] - a.item0[b];
        const int64_t base = a.wave_base[b] * 64;
        for (int64_t j = (rel0 + kXbItems - 1) / kXbItems; j * kXbItems <= rel1; ++j)
            lane_row[base + j] = (int)t;
    }
}

template <typename T>
hipError_t run(const XblkView& a, void* y, const void* x, double alpha, double beta,
               hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const hipError_t e = launch_scale(a.n, sizeof(T) == 8, y, beta, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_xblk<T>, dim3((unsigned)(kXbBlocks * a.tiles)), dim3(256), 0, s, a,
                       static_cast<const T*>(x), static_cast<T*>(y), (T)alpha);
    return hipGetLastError();
}

unsigned setup_grid(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); }
// one wave per row, four rows per workgroup
unsigned row_wave_grid(int64_t n) { return (unsigned)std::min<int64_t>((n + 3) / 4, 65536); }

}  // namespace

hipError_t launch_xblk(const XblkView& a, bool f64, void* y, const void* x, double alpha,
                       double beta, hipStream_t s) {
    return f64 ? run<double>(a, y, x, alpha, beta, s) : run<float>(a, y, x, alpha, beta, s);
}

hipError_t launch_xblk_count(int64_t n, int64_t width, const int* rowptr, const int* col,
                             int* cnt, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_xblk_count, dim3(row_wave_grid(n)), dim3(256), 0, s, n, width, rowptr,
                       col, cnt);
    return hipGetLastError();
}

hipError_t launch_xblk_fill(int64_t n, int64_t width, bool f64, const int* rowptr, const int* col,
                            const void* val, const int* ptr, int* ocol, void* oval,
                            hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (f64)
        hipLaunchKernelGGL(k_xblk_fill<double>, dim3(row_wave_grid(n)), dim3(256), 0, s, n, width,
                           rowptr, col, static_cast<const double*>(val), ptr, ocol,
                           static_cast<double*>(oval));
    else
        hipLaunchKernelGGL(k_xblk_fill<float>, dim3(row_wave_grid(n)), dim3(256), 0, s, n, width,
                           rowptr, col, static_cast<const float*>(val), ptr, ocol,
                           static_cast<float*>(oval));
    return hipGetLastError();
}

hipError_t launch_xblk_lane_rows(const XblkView& a, int* lane_row, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_xblk_lane_rows, dim3(setup_grid((int64_t)kXbBlocks * a.n)), dim3(256), 0,
                       s, a, lane_row);
    return hipGetLastError();
}

}  // namespace spmv
