// Irregular part of HYB (COO) and HEC (CSR), and CSR run by entries:
// y += alpha * A_tail * x with the work split by entries, not by rows.
//
// "Load-balancing Sparse Matrix Vector Product Kernels on GPUs" (abstract)
// balances COO/CSR work independently of the row lengths; the Trilinos
// "unpackAndCombine" discussion (few long rows) puts the long rows in a
// separate launch and combines partial results with atomic +=.  Here the
// tail entries, ordered by row, are cut into chunks of 512 consecutive
// entries, one chunk per wave, each run in passes of 64 * E consecutive
// entries with E per lane (HYB: E = 2 for fp64, 4 for fp32, so a pass is one
// 16-byte load per lane; CSR tails: one pass of E = 8).  In every pass the
// lanes add the row segments inside their runs, a segmented scan over the
// lanes sums the segments that cross lanes, and every addition into y is a
// device-scope atomic without return value (no lane ever waits for y, and
// rows shared by passes or waves need no special case).  HYB reads the row
// of every entry; the CSR forms search the row pointer.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace spmv {

// A wave's chunk of 64 * kTailPerLane consecutive entries is processed in
// P passes of 64 * E consecutive entries, E = 16 / sizeof(T) per lane: one
// 16-byte load per lane brings the values of a pass, so a load instruction
// covers 1 KiB of contiguous values (whole cache lines) and the lanes of a
// pass read the entries of neighbouring rows side by side (for banded
// matrices their x reads share lines too).  All loads of a chunk are issued
// before the first use.
typedef double d2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i2_t __attribute__((ext_vector_type(2)));
typedef int i4_t __attribute__((ext_vector_type(4)));

// COO tails (rows stored) run in passes of one 16-byte value load per lane;
// CSR tails keep one pass of kTailPerLane entries per lane, which needs a
// single row search per lane (the cross-lane work of a pass -- the scan and
// the search -- would otherwise be paid P times).
template <typename T, bool kCoo>
struct TailShape {
    static constexpr int E = kCoo ? 16 / (int)sizeof(T) : kTailPerLane;  // per lane and pass
    static constexpr int P = kTailPerLane / E;                           // passes per chunk
};

// E consecutive elements with 16-byte loads (E * sizeof a multiple of 16
// bytes, p 16-byte aligned).  kNT streams them past the caches: right for
// the COO passes, whose load instructions read whole lines once; the CSR
// tails' runs read a line in several instructions, which must find it cached.
template <bool kNT, typename V>
__device__ __forceinline__ V load16(const V* p) {
    if constexpr (kNT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
template <int E, bool kNT>
__device__ __forceinline__ void load_vec(const double* p, double (&v)[E]) {
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
        const d2_t t = load16<kNT>(reinterpret_cast<const d2_t*>(p) + k);
        v[2 * k] = t.x, v[2 * k + 1] = t.y;
    }
}
template <int E, bool kNT>
__device__ __forceinline__ void load_vec(const float* p, float (&v)[E]) {
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
        const f4_t t = load16<kNT>(reinterpret_cast<const f4_t*>(p) + k);
        v[4 * k] = t.x, v[4 * k + 1] = t.y, v[4 * k + 2] = t.z, v[4 * k + 3] = t.w;
    }
}
template <int E, bool kNT>
__device__ __forceinline__ void load_vec(const int* p, int (&v)[E]) {
    if constexpr (E == 2) {
        const i2_t t = load16<kNT>(reinterpret_cast<const i2_t*>(p));
        v[0] = t.x, v[1] = t.y;
    } else {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            const i4_t t = load16<kNT>(reinterpret_cast<const i4_t*>(p) + k);
            v[4 * k] = t.x, v[4 * k + 1] = t.y, v[4 * k + 2] = t.z, v[4 * k + 3] = t.w;
        }
    }
}

// Registers of one lane's share of a chunk: values, columns and rows of its
// E entries in each of the P passes.
template <typename T, bool kCoo>
struct TailRun {
    static constexpr int E = TailShape<T, kCoo>::E, P = TailShape<T, kCoo>::P;
    T v[P][E];
    int c[P][E];
    int r[P][E];
    int cnt[P];  // entries of this lane in each pass (0 past the end)
};

__device__ __forceinline__ int64_t pass_entry(int64_t w, int p, int lane, int E) {
    return w * kTailChunk + (int64_t)p * 64 * E + (int64_t)lane * E;
}

// Issue the loads of chunk w (values, columns and, for HYB, rows).
template <typename T, bool kCoo>
__device__ __forceinline__ void tail_fetch(int64_t w, int lane, int64_t nnz,
                                           const int* __restrict__ trow,
                                           const int* __restrict__ col,
                                           const T* __restrict__ val, TailRun<T, kCoo>& R) {
    constexpr int E = TailShape<T, kCoo>::E, P = TailShape<T, kCoo>::P;
    constexpr int kNone = 0x7fffffff;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int64_t e0 = pass_entry(w, p, lane, E);
        R.cnt[p] = e0 < nnz ? (int)min<int64_t>(E, nnz - e0) : 0;
        if (R.cnt[p] == E) {
            load_vec<E, kCoo>(val + e0, R.v[p]);
            load_vec<E, kCoo>(col + e0, R.c[p]);
            if constexpr (kCoo) load_vec<E, true>(trow + e0, R.r[p]);
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                R.v[p][k] = k < R.cnt[p] ? val[e0 + k] : T(0);
                R.c[p][k] = k < R.cnt[p] ? col[e0 + k] : 0;
                if constexpr (kCoo) R.r[p][k] = k < R.cnt[p] ? trow[e0 + k] : kNone;
            }
        }
    }
}

// Rows of chunk w's entries from the CSR tail pointer (HEC, and CSR run by
// entries; one pass of E entries per lane).  The row of every lane's first
// entry is stored when the format is built (run_row, 4 bytes per 8
// entries); the lane reads the next E row starts at once and places its
// entries among them, searching (up to the next lane's row) only if its run
// crosses more rows (rows without entries in between).
template <typename T>
__device__ __forceinline__ void tail_rows(int64_t w, int lane, const int* __restrict__ tptr,
                                          const int* __restrict__ run_row,
                                          const int* __restrict__ row_map,
                                          TailRun<T, false>& R) {
    constexpr int E = TailShape<T, false>::E;
    constexpr int kNone = 0x7fffffff;
    const int cnt = R.cnt[0];
    int* r = R.r[0];
    const int64_t q = w * 64 + lane;  // lane run index
    const int64_t e0 = q * E;
    const int64_t qs = cnt > 0 ? q : 0;  // past the last run: any valid index
    const int cur = run_row[qs], hi = run_row[qs + 1];
    int nxt[E];  // starts of the next E rows (clamped to the next run's row;
                 // cur + 1 + j itself may pass 2^31 near the last rows)
#pragma unroll
    for (int j = 0; j < E; ++j) nxt[j] = tptr[run_next_start(cur, hi, j)];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        int adv = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) adv += nxt[j] <= e0 + k;
        r[k] = k < cnt ? cur + adv : kNone;
    }
    if (cnt > 0 && nxt[E - 1] <= e0 + cnt - 1) {
        int c2 = cur + E;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (k < cnt && e0 + k >= nxt[E - 1]) {
                if (e0 + k >= tptr[c2 + 1]) c2 = row_of(tptr, c2 + 1, hi, e0 + k);
                r[k] = c2;
            }
        }
    }
    if (row_map) {  // HEC: tail rows -> matrix rows
#pragma unroll
        for (int k = 0; k < E; ++k) r[k] = k < cnt ? row_map[r[k]] : kNone;
    }
}

// Add the products p of one pass into y.  The lane's E entries are
// consecutive and ordered by row; the wave's 64 * E entries too.
//   1. each lane walks its entries and adds the rows that start and end
//      inside its run;
//   2. the lane's last segment may continue in the next lanes: a segmented
//      inclusive scan over the lanes (keyed by row) sums it, and the lane
//      where the row ends (or the last lane) adds it; a lane's first
//      segment that began in an earlier lane is added with the earlier
//      lanes' scan value;
//   3. every addition into y is a device-scope atomic without return value,
//      so no lane waits for y and rows shared with other passes or waves
//      need no special case.
template <typename T, int E>
__device__ __forceinline__ void pass_sum(int lane, int cnt, const int (&r)[E], const T (&p)[E],
                                         T* __restrict__ y, T alpha) {
    constexpr int kNone = 0x7fffffff;
    const int head_row = r[0];
    T head_sum = 0;
    bool split = false;
    int cur = r[0];
    T acc = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (k < cnt) {
            if (r[k] != cur) {
                if (!split) {
                    head_sum = acc;
                    split = true;
                } else {
                    atomic_add(y + cur, alpha * acc);
                }
                cur = r[k];
                acc = 0;
            }
            acc += p[k];
        }
    }
    const int key = cnt > 0 ? cur : kNone;  // row of the lane's last segment
    const T sum = segmented_scan(key, acc);
    const int prev_key = dpp_or<0x138, 0xF>(-1, key);    // lane - 1 (none for lane 0)
    const T prev_sum = dpp_or<0x138, 0xF>(T(0), sum);
    const int next_first = dpp_or<0x130, 0xF>(-1, head_row);  // lane + 1 (none for 63)
    if (split) {
        const T tot = head_sum + (prev_key == head_row ? prev_sum : T(0));
        atomic_add(y + head_row, alpha * tot);
    }
    if (cnt > 0 && (lane == 63 || next_first != key)) atomic_add(y + key, alpha * sum);
}

// Window path: issue the global loads of the x entries outside the window
// (xg, flagged in far).  They must go out before the next chunk's loads:
// loads complete in order, so waiting on them would drain that prefetch.
template <typename T, bool kCoo>
__device__ __forceinline__ void tail_far_gather(const T* __restrict__ x, int64_t wlo,
                                                const TailRun<T, kCoo>& R,
                                                bool (&far)[TailShape<T, kCoo>::P][TailShape<T, kCoo>::E],
                                                T (&xg)[TailShape<T, kCoo>::P][TailShape<T, kCoo>::E]) {
    constexpr int E = TailShape<T, kCoo>::E, P = TailShape<T, kCoo>::P;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int k = 0; k < E; ++k) {
            far[p][k] = k < R.cnt[p] &&
                        (uint32_t)(R.c[p][k] - (int)wlo) >= (uint32_t)WinLen<T>::value;
            xg[p][k] = far[p][k] ? x[R.c[p][k]] : T(0);
        }
}

// Finish chunk w: rows (CSR tail), products, sums into y.  With kWin, x
// entries inside the window come from LDS (element q at slot q mod
// WinLen), the others were gathered into xg.
template <typename T, bool kCoo, bool kWin>
__device__ __forceinline__ void tail_finish(int64_t w, int lane, int64_t nnz,
                                            const int* __restrict__ tptr,
                                            const int* __restrict__ run_row,
                                            const int* __restrict__ row_map,
                                            const T* __restrict__ x, T* __restrict__ y, T alpha,
                                            const T* win,
                                            const bool (&far)[TailShape<T, kCoo>::P][TailShape<T, kCoo>::E],
                                            const T (&xg)[TailShape<T, kCoo>::P][TailShape<T, kCoo>::E],
                                            TailRun<T, kCoo>& R) {
    constexpr int E = TailShape<T, kCoo>::E, P = TailShape<T, kCoo>::P;
    if (w * kTailChunk >= nnz) return;  // the whole wave leaves together
    if constexpr (!kCoo) tail_rows<T>(w, lane, tptr, run_row, row_map, R);
    // every x read is issued before the first product (entries past the
    // end read nothing and hold value 0)
    T pr[P][E];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int k = 0; k < E; ++k) {
            T xv = T(0);
            if (k < R.cnt[p]) {
                if constexpr (kWin) {
                    const T xw = win[R.c[p][k] % WinLen<T>::value];  // slot always in range
                    xv = far[p][k] ? xg[p][k] : xw;
                } else {
                    xv = x[R.c[p][k]];
                }
            }
            pr[p][k] = R.v[p][k] * xv;
        }
#pragma unroll
    for (int p = 0; p < P; ++p) pass_sum<T, E>(lane, R.cnt[p], R.r[p], pr[p], y, alpha);
}

template <typename T, bool kCoo>
__global__ __launch_bounds__(256) void k_tail(int n, int64_t nnz, const int* __restrict__ trow,
                                              const int* __restrict__ tptr,
                                              const int* __restrict__ run_row,
                                              const int* __restrict__ row_map,
                                              const int* __restrict__ col,
                                              const T* __restrict__ val,
                                              const T* __restrict__ x, T* __restrict__ y,
                                              T alpha) {
    constexpr int E = TailShape<T, kCoo>::E, P = TailShape<T, kCoo>::P;
    const int64_t w = xcd_tile(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    if (w * kTailChunk >= nnz) return;
    TailRun<T, kCoo> R;
    tail_fetch<T, kCoo>(w, threadIdx.x & 63, nnz, trow, col, val, R);
    bool far[P][E] = {};
    T xg[P][E] = {};
    tail_finish<T, kCoo, false>(w, threadIdx.x & 63, nnz, tptr, run_row, row_map, x, y, alpha, nullptr,
                                far, xg, R);
}

// Tail with x staged in LDS.  Workgroup g (16 waves) runs a contiguous
// share of the steps; a step is kTailStepChunks consecutive wave
// chunks (kTailChunksPerWave per wave) and its window starts WinLead rows
// before the step's first row.  Only the x elements entering the window are
// loaded (rows only move forward, so each element is loaded about once per
// workgroup).  Inside a step each wave runs its chunks back to back with the
// next chunk's loads in flight while the current one is summed, so the
// barriers that move the window are paid once per kTailChunksPerWave chunks.
template <typename T, bool kCoo>
__global__ __launch_bounds__(1024) void k_tail_win(int n, int64_t nnz,
                                                   const int* __restrict__ trow,
                                                   const int* __restrict__ tptr,
                                                   const int* __restrict__ run_row,
                                                   const int* __restrict__ row_map,
                                                   const int* __restrict__ col,
                                                   const T* __restrict__ val,
                                                   const T* __restrict__ x, T* __restrict__ y,
                                                   T alpha, int64_t nsteps) {
    constexpr int WL = WinLen<T>::value;
    constexpr int LEAD = WinLead<T>::value;
    constexpr int CPW = kTailChunksPerWave;
    __shared__ T win[WL];
    const int64_t g = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t s0 = g * nsteps / gridDim.x, s1 = (g + 1) * nsteps / gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t prev_whi = -1;
    for (int64_t s = s0; s < s1; ++s) {
        int64_t r_first;
        if constexpr (kCoo) {
            r_first = trow[s * (int64_t)kTailStepChunks * kTailChunk];
        } else {
            const int tr = run_row[s * (int64_t)kTailStepChunks * 64];
            r_first = row_map ? row_map[tr] : tr;
        }
        const int64_t wlo = r_first - LEAD, whi = wlo + WL;
        lds_barrier();  // the previous step is done with the slots reused now
        const int64_t from = max<int64_t>(max<int64_t>(prev_whi, wlo), 0);
        const int64_t to = min<int64_t>(whi, n);
        if (to - from > 2048) {
            window_fill<T, WL>(win, x, from, to);
        } else {
            for (int64_t q = from + threadIdx.x; q < to; q += 1024) win[q % WL] = x[q];
        }
        lds_barrier();
        prev_whi = whi;
        const int64_t w0 = s * kTailStepChunks + (int64_t)wave * CPW;
        TailRun<T, kCoo> run[2];
        tail_fetch<T, kCoo>(w0, lane, nnz, trow, col, val, run[0]);
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            bool far[TailShape<T, kCoo>::P][TailShape<T, kCoo>::E];
            T xg[TailShape<T, kCoo>::P][TailShape<T, kCoo>::E];
            tail_far_gather<T, kCoo>(x, wlo, run[k & 1], far, xg);
            if (k + 1 < CPW)
                tail_fetch<T, kCoo>(w0 + k + 1, lane, nnz, trow, col, val, run[(k + 1) & 1]);
            tail_finish<T, kCoo, true>(w0 + k, lane, nnz, tptr, run_row, row_map, x, y, alpha, win, far,
                                       xg, run[k & 1]);
        }
    }
}

template <typename T>
static hipError_t run(const TailView& t, void* y, const void* x, double alpha,
                      hipStream_t stream) {
    if (t.nnz == 0) return hipSuccess;
    const int64_t waves = (t.nnz + kTailChunk - 1) / kTailChunk;
    if (t.window) {
        const int64_t nsteps = (waves + kTailStepChunks - 1) / kTailStepChunks;
        const int64_t g = std::min<int64_t>(nsteps, kWinGroups);
        if (t.row)
            hipLaunchKernelGGL((k_tail_win<T, true>), dim3((unsigned)g), dim3(1024), 0, stream, t.n,
                               t.nnz, t.row, t.ptr, t.run_row, t.row_map, t.col, (const T*)t.val,
                               (const T*)x, (T*)y, (T)alpha, nsteps);
        else
            hipLaunchKernelGGL((k_tail_win<T, false>), dim3((unsigned)g), dim3(1024), 0, stream,
                               t.n, t.nnz, t.row, t.ptr, t.run_row, t.row_map, t.col, (const T*)t.val,
                               (const T*)x, (T*)y, (T)alpha, nsteps);
        return hipGetLastError();
    }
    const int64_t blocks = (waves + 3) / 4;
    if (t.row)
        hipLaunchKernelGGL((k_tail<T, true>), dim3((unsigned)blocks), dim3(256), 0, stream, t.n,
                           t.nnz, t.row, t.ptr, t.run_row, t.row_map, t.col, (const T*)t.val,
                           (const T*)x, (T*)y, (T)alpha);
    else
        hipLaunchKernelGGL((k_tail<T, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           t.n, t.nnz, t.row, t.ptr, t.run_row, t.row_map, t.col, (const T*)t.val,
                           (const T*)x, (T*)y, (T)alpha);
    return hipGetLastError();
}

// y = beta * y before an entry-balanced pass over the whole matrix adds its
// products with atomics (beta == 0 never reads y, so NaNs in y vanish).
template <typename T>
__global__ __launch_bounds__(256) void k_scale(int64_t n, T* __restrict__ y, T beta) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        y[i] = beta == T(0) ? T(0) : beta * y[i];
}

hipError_t launch_scale(int64_t n, bool f64, void* y, double beta, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
    if (f64)
        hipLaunchKernelGGL(k_scale<double>, dim3((unsigned)blocks), dim3(256), 0, stream, n,
                           (double*)y, beta);
    else
        hipLaunchKernelGGL(k_scale<float>, dim3((unsigned)blocks), dim3(256), 0, stream, n,
                           (float*)y, (float)beta);
    return hipGetLastError();
}

hipError_t launch_tail(const TailView& t, bool f64, void* y, const void* x, double alpha,
                       hipStream_t stream) {
    return f64 ? run<double>(t, y, x, alpha, stream) : run<float>(t, y, x, alpha, stream);
}

}  // namespace spmv
