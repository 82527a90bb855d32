// CSR apply with a sub-wave of S lanes per row.
//
// "Sparse Linear Algebra on AMD and NVIDIA GPUs -- The Race Is On" assigns a
// group of threads to each row and reduces their partial sums across the
// group, with the group size following the longest row.  On gfx950 a wave
// has 64 lanes, so S ranges over the powers of two 1..64; the S lanes of a
// group stride through the row (consecutive lanes read consecutive entries,
// so a wave's loads of val/col are contiguous) and the partial sums are
// combined with DPP / ds_swizzle moves inside the wave (no LDS traffic).
// The loads allocate in the caches: with short rows a cache line is shared
// by neighbouring groups, which would otherwise fetch it again.
#include "common.h"
#include "internal.h"

namespace spmv {

// Each group of S lanes handles R consecutive rows.  A lone row costs three
// dependent memory round trips (row pointer, then val/col, then x), so the
// group first issues the row pointers, values and columns of all R rows
// (two entries per lane and row) and only then the x reads and sums; longer
// rows finish in a plain loop.  The first pass reads with clamped indices
// and masks the products, so it has no per-entry branches.
template <typename T, int S, int R>
__global__ __launch_bounds__(256) void k_csr_vector(int n, const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    const T* __restrict__ val,
                                                    const T* __restrict__ x, T* __restrict__ y,
                                                    T alpha, T beta) {
    constexpr int kGroups = 256 / S;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t row0 = (tile * kGroups + threadIdx.x / S) * R;
    const int sub = threadIdx.x & (S - 1);
    if (row0 >= n) return;  // whole groups leave together
    int kb[R + 1];
#pragma unroll
    for (int r = 0; r <= R; ++r) kb[r] = rowptr[row0 + r < n ? row0 + r : (int64_t)n];
    T v[R][2];
    int c[R][2];
    bool ok[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int k = kb[r] + sub + u * S;
            ok[r][u] = k < kb[r + 1];
            const int kc = max(min(k, kb[r + 1] - 1), 0);  // in bounds even when masked
            v[r][u] = val[kc];
            c[r][u] = col[kc];
        }
    T sum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const T p0 = ok[r][0] ? v[r][0] * x[c[r][0]] : T(0);
        const T p1 = ok[r][1] ? v[r][1] * x[c[r][1]] : T(0);
        sum[r] = p0 + p1;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        for (int k = kb[r] + sub + 2 * S; k < kb[r + 1]; k += S) sum[r] = fma(val[k], x[col[k]], sum[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const T s_r = group_sum<S>(sum[r]);
        if (sub == 0 && row0 + r < n) y[row0 + r] = axpby(s_r, alpha, beta, y + row0 + r);
    }
}

template <typename T, int S, int R>
static hipError_t run(const CsrView& a, void* y, const void* x, double alpha, double beta,
                      hipStream_t stream) {
    constexpr int kRowsPerBlock = 256 / S * R;
    const int64_t blocks = ((int64_t)a.n + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_csr_vector<T, S, R>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       a.n, a.rowptr, a.col, (const T*)a.val, (const T*)x, (T*)y, (T)alpha,
                       (T)beta);
    return hipGetLastError();
}

template <typename T, int R>
static hipError_t dispatch_s(const CsrView& a, int subwave, void* y, const void* x, double alpha,
                             double beta, hipStream_t stream) {
    switch (subwave) {
        case 1: return run<T, 1, R>(a, y, x, alpha, beta, stream);
        case 2: return run<T, 2, R>(a, y, x, alpha, beta, stream);
        case 4: return run<T, 4, R>(a, y, x, alpha, beta, stream);
        case 8: return run<T, 8, R>(a, y, x, alpha, beta, stream);
        case 16: return run<T, 16, R>(a, y, x, alpha, beta, stream);
        case 32: return run<T, 32, R>(a, y, x, alpha, beta, stream);
        case 64: return run<T, 64, R>(a, y, x, alpha, beta, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t dispatch(const CsrView& a, int subwave, int rows, void* y, const void* x,
                           double alpha, double beta, hipStream_t stream) {
    switch (rows) {
        case 1: return dispatch_s<T, 1>(a, subwave, y, x, alpha, beta, stream);
        case 4: return dispatch_s<T, 4>(a, subwave, y, x, alpha, beta, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_csr(const CsrView& a, int subwave, int rows, bool f64, void* y,
                      const void* x, double alpha, double beta, hipStream_t stream) {
    return f64 ? dispatch<double>(a, subwave, rows, y, x, alpha, beta, stream)
               : dispatch<float>(a, subwave, rows, y, x, alpha, beta, stream);
}

}  // namespace spmv
