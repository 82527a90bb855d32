// Irregular part of HYB (COO) and HEC (CSR): y += alpha * A_tail * x with the
// work split by entries, not by rows.
//
// "Load-balancing Sparse Matrix Vector Product Kernels on GPUs" (abstract)
// balances COO/CSR work independently of the row lengths; the Trilinos
// "unpackAndCombine" discussion (few long rows) puts the long rows in a
// separate launch and combines partial results with atomic +=.  Here the
// tail entries, ordered by row, are cut into chunks of 64 * E consecutive
// entries, one chunk per wave and E consecutive entries per lane:
//   1. each lane walks its E entries in order, finishing every row segment
//      that starts and ends inside its run with a plain y += alpha * sum
//      (no other lane or wave touches that row's tail);
//   2. the lane's first and last segments may continue in neighbouring
//      lanes: a segmented inclusive scan over the lanes (keyed by row, which
//      is non-decreasing along the chunk) sums them, and the lane that
//      closes a row inside the wave writes it;
//   3. only the chunk's first and last rows can be shared with other waves;
//      they are added with device-scope atomics, every other row with a
//      plain read-modify-write.
// HYB reads the row of every entry; HEC finds rows by binary search in its
// row pointer, starting from the row of each chunk's first entry (computed
// once when the format is built).
#include "common.h"
#include "internal.h"

namespace spmv {

typedef double d2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));

template <int E>
__device__ __forceinline__ void load_run(const double* p, double (&v)[E]) {
    const d2_t* q = reinterpret_cast<const d2_t*>(p);
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
        const d2_t t = ld_nt(q + k);
        v[2 * k] = t.x;
        v[2 * k + 1] = t.y;
    }
}

template <int E>
__device__ __forceinline__ void load_run(const float* p, float (&v)[E]) {
    const f4_t* q = reinterpret_cast<const f4_t*>(p);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
        const f4_t t = ld_nt(q + k);
        v[4 * k] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
    }
}

template <int E>
__device__ __forceinline__ void load_run(const int* p, int (&v)[E]) {
    const i4_t* q = reinterpret_cast<const i4_t*>(p);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
        const i4_t t = ld_nt(q + k);
        v[4 * k] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
    }
}

// largest r in [lo, hi] with ptr[r] <= e (the row holding entry e, given
// ptr[lo] <= e < ptr[hi + 1])
__device__ __forceinline__ int row_of(const int* __restrict__ ptr, int lo, int hi, int64_t e) {
    while (lo < hi) {
        const int m = (lo + hi + 1) >> 1;
        if (ptr[m] <= e)
            lo = m;
        else
            hi = m - 1;
    }
    return lo;
}

template <typename T>
__device__ __forceinline__ void add_row(T* y, int row, T v, bool shared) {
    if (shared)
        atomic_add(y + row, v);
    else
        y[row] += v;
}

template <typename T, bool kCoo>
__global__ __launch_bounds__(256) void k_tail(int n, int64_t nnz, const int* __restrict__ trow,
                                              const int* __restrict__ tptr,
                                              const int* __restrict__ chunk_row,
                                              const int* __restrict__ col,
                                              const T* __restrict__ val,
                                              const T* __restrict__ x, T* __restrict__ y,
                                              T alpha) {
    constexpr int E = kTailPerLane;
    constexpr int kNone = 0x7fffffff;
    const int64_t w = xcd_tile(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    const int64_t c0 = w * kTailChunk;
    if (c0 >= nnz) return;  // the whole wave leaves together
    const int lane = threadIdx.x & 63;
    const int64_t e0 = c0 + (int64_t)lane * E;
    const int cnt = e0 < nnz ? (int)min<int64_t>(E, nnz - e0) : 0;

    T v[E];
    int c[E];
    int r[E];
    if (cnt == E) {
        load_run<E>(val + e0, v);
        load_run<E>(col + e0, c);
        if constexpr (kCoo) load_run<E>(trow + e0, r);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            v[k] = k < cnt ? val[e0 + k] : T(0);
            c[k] = k < cnt ? col[e0 + k] : 0;
            if constexpr (kCoo) r[k] = k < cnt ? trow[e0 + k] : kNone;
        }
    }
    if constexpr (!kCoo) {
        const int lo = chunk_row[w], hi = chunk_row[w + 1];
        int cur = cnt > 0 ? row_of(tptr, lo, hi, e0) : kNone;
        int next_start = cnt > 0 ? tptr[cur + 1] : 0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (k < cnt && e0 + k >= next_start) {
                cur = row_of(tptr, cur + 1, hi, e0 + k);
                next_start = tptr[cur + 1];
            }
            r[k] = k < cnt ? cur : kNone;
        }
    }
    T p[E];
#pragma unroll
    for (int k = 0; k < E; ++k) p[k] = k < cnt ? v[k] * x[c[k]] : T(0);

    // 1. walk the run; rows that start and end inside it are exclusive
    int head_row = r[0];
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
                    y[cur] += alpha * acc;
                }
                cur = r[k];
                acc = 0;
            }
            acc += p[k];
        }
    }
    const int key = cnt > 0 ? cur : kNone;  // row of the lane's last segment
    T sum = acc;

    // 2. segmented inclusive scan of the last segments across the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int k2 = __shfl_up(key, d);
        const T s2 = __shfl_up(sum, d);
        if (lane >= d && k2 == key) sum += s2;
    }
    const int first_row = __shfl(head_row, 0);
    const int last_lane = (int)min<int64_t>(63, (nnz - c0 - 1) / E);
    const int last_row = __shfl(key, last_lane);
    const int prev_key = __shfl_up(key, 1);
    const T prev_sum = __shfl_up(sum, 1);
    const int next_first = __shfl_down(head_row, 1);

    // 3. write what closes here
    if (split) {
        const T tot = head_sum + ((lane > 0 && prev_key == head_row) ? prev_sum : T(0));
        add_row(y, head_row, alpha * tot, head_row == first_row);
    }
    if (cnt > 0 && (lane == 63 || next_first != key))
        add_row(y, key, alpha * sum, key == first_row || key == last_row);
}

template <typename T>
static hipError_t run(const TailView& t, void* y, const void* x, double alpha,
                      hipStream_t stream) {
    if (t.nnz == 0) return hipSuccess;
    const int64_t waves = (t.nnz + kTailChunk - 1) / kTailChunk;
    const int64_t blocks = (waves + 3) / 4;
    if (t.row)
        hipLaunchKernelGGL((k_tail<T, true>), dim3((unsigned)blocks), dim3(256), 0, stream, t.n,
                           t.nnz, t.row, t.ptr, t.chunk_row, t.col, (const T*)t.val,
                           (const T*)x, (T*)y, (T)alpha);
    else
        hipLaunchKernelGGL((k_tail<T, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           t.n, t.nnz, t.row, t.ptr, t.chunk_row, t.col, (const T*)t.val,
                           (const T*)x, (T*)y, (T)alpha);
    return hipGetLastError();
}

hipError_t launch_tail(const TailView& t, bool f64, void* y, const void* x, double alpha,
                       hipStream_t stream) {
    return f64 ? run<double>(t, y, x, alpha, stream) : run<float>(t, y, x, alpha, stream);
}

}  // namespace spmv
