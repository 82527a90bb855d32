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

// Each group of S lanes handles R rows.  A lone row costs three dependent
// memory round trips (row pointer, then val/col, then x), so the group first
// issues the row pointers, values and columns of all R rows (U entries per
// lane and row, U = 16 / S for small groups so that the first pass covers 16
// entries of every row) and only then the x reads and sums; longer rows
// finish in a plain loop.  The R rows of a group are interleaved with those
// of the other groups of its wave (row = wave base + r * groups + group), so
// every load instruction covers consecutive rows: neighbouring rows share
// cache lines of val/col and, for banded matrices, entry u of neighbouring
// rows usually lies on the same diagonal, so their x reads share lines too.
// The first pass reads with clamped indices and masks the products, so it
// has no per-entry branches.
template <int S, int R>
struct CsrFirstPass {
    static constexpr int a = 16 / S, b = 16 / R;
    static constexpr int value = (a < b ? a : b) > 2 ? (a < b ? a : b) : 2;
};

template <typename T, int S, int R>
__global__ __launch_bounds__(256) void k_csr_vector(int n, const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    const T* __restrict__ val,
                                                    const T* __restrict__ x, T* __restrict__ y,
                                                    T alpha, T beta) {
    constexpr int kGroups = kWave / S;  // groups per wave
    constexpr int U = CsrFirstPass<S, R>::value;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t wave = tile * 4 + threadIdx.x / kWave;
    const int64_t base = wave * (kGroups * R) + (threadIdx.x % kWave) / S;
    const int sub = threadIdx.x & (S - 1);
    if (base >= n) return;  // whole groups leave together
    int kb[R], ke[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = base + r * kGroups;
        kb[r] = row < n ? rowptr[row] : 0;
        ke[r] = row < n ? rowptr[row + 1] : 0;
    }
    T v[R][U];
    int c[R][U];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kc = max(min(kb[r] + sub + u * S, ke[r] - 1), 0);  // in bounds even when masked
            v[r][u] = val[kc];
            c[r][u] = col[kc];
        }
    T sum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        T acc = T(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const T p = v[r][u] * x[c[r][u]];
            acc += kb[r] + sub + u * S < ke[r] ? p : T(0);
        }
        sum[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        for (int k = kb[r] + sub + U * S; k < ke[r]; k += S) sum[r] = fma(val[k], x[col[k]], sum[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const T s_r = group_sum<S>(sum[r]);
        const int64_t row = base + r * kGroups;
        if (sub == 0 && row < n) y[row] = axpby(s_r, alpha, beta, y + row);
    }
}

template <typename T, int S, int R>
static hipError_t run(const CsrView& a, void* y, const void* x, double alpha, double beta,
                      hipStream_t stream) {
    constexpr int kRowsPerBlock = 256 / S * R;  // 4 waves of 64 / S groups of R rows
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
        case 2: return dispatch_s<T, 2>(a, subwave, y, x, alpha, beta, stream);
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
