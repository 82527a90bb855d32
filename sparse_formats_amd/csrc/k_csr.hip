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

template <typename T, int S>
__global__ __launch_bounds__(256) void k_csr_vector(int n, const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    const T* __restrict__ val,
                                                    const T* __restrict__ x, T* __restrict__ y,
                                                    T alpha, T beta) {
    constexpr int kRowsPerBlock = 256 / S;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t row = tile * kRowsPerBlock + threadIdx.x / S;
    const int sub = threadIdx.x & (S - 1);
    if (row >= n) return;  // whole groups leave together
    const int k0 = rowptr[row], k1 = rowptr[row + 1];
    T s0 = 0, s1 = 0;
    int k = k0 + sub;
    // two independent chains keep two loads of val/col in flight per lane
    for (; k + S < k1; k += 2 * S) {
        const T v0 = val[k], v1 = val[k + S];
        const int c0 = col[k], c1 = col[k + S];
        s0 = fma(v0, x[c0], s0);
        s1 = fma(v1, x[c1], s1);
    }
    if (k < k1) s0 = fma(val[k], x[col[k]], s0);
    T s = group_sum<S>(s0 + s1);
    if (sub == 0) y[row] = axpby(s, alpha, beta, y + row);
}

template <typename T, int S>
static hipError_t run(const CsrView& a, void* y, const void* x, double alpha, double beta,
                      hipStream_t stream) {
    constexpr int kRowsPerBlock = 256 / S;
    const int64_t blocks = ((int64_t)a.n + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_csr_vector<T, S>), dim3((unsigned)blocks), dim3(256), 0, stream, a.n,
                       a.rowptr, a.col, (const T*)a.val, (const T*)x, (T*)y, (T)alpha, (T)beta);
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch(const CsrView& a, int subwave, void* y, const void* x, double alpha,
                           double beta, hipStream_t stream) {
    switch (subwave) {
        case 1: return run<T, 1>(a, y, x, alpha, beta, stream);
        case 2: return run<T, 2>(a, y, x, alpha, beta, stream);
        case 4: return run<T, 4>(a, y, x, alpha, beta, stream);
        case 8: return run<T, 8>(a, y, x, alpha, beta, stream);
        case 16: return run<T, 16>(a, y, x, alpha, beta, stream);
        case 32: return run<T, 32>(a, y, x, alpha, beta, stream);
        case 64: return run<T, 64>(a, y, x, alpha, beta, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_csr(const CsrView& a, int subwave, bool f64, void* y, const void* x,
                      double alpha, double beta, hipStream_t stream) {
    return f64 ? dispatch<double>(a, subwave, y, x, alpha, beta, stream)
               : dispatch<float>(a, subwave, y, x, alpha, beta, stream);
}

}  // namespace spmv
