// Vector kernels of the Krylov solvers over the sparse product (conjugate
// gradients, BiCGSTAB): the inner products and the fused vector updates of
// one iteration.  Inner products accumulate in fp64 for both value types and
// reduce in two passes over a fixed grid (partial sums per workgroup, then
// one workgroup in a fixed order), so a product of the same vectors gives the
// same bits every time.  Updates that are followed by an inner product of
// their result compute its partial sums in the same pass.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace spmv {

constexpr int kDotBlocks = kSolveBlocks;  // partial sums per inner product

__device__ __forceinline__ double block_sum(double v, double* sh) {
    // wave sums, then the 4 wave sums of the 256-thread block
    v += __shfl_xor(v, 32);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0;
    if (threadIdx.x == 0) s = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    return s;
}

// partial[2 * b + k] = block b's share of a_k . b_k (k = 0, 1; the second
// product only when a1 != nullptr)
template <typename T>
__global__ __launch_bounds__(256) void k_dot2(int64_t n, const T* __restrict__ a0,
                                              const T* __restrict__ b0, const T* __restrict__ a1,
                                              const T* __restrict__ b1,
                                              double* __restrict__ partial) {
    __shared__ double sh[4];
    double s0 = 0, s1 = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        s0 += (double)a0[i] * (double)b0[i];
        if (a1) s1 += (double)a1[i] * (double)b1[i];
    }
    const double t0 = block_sum(s0, sh);
    __syncthreads();
    const double t1 = block_sum(s1, sh);
    if (threadIdx.x == 0) {
        partial[2 * blockIdx.x] = t0;
        partial[2 * blockIdx.x + 1] = t1;
    }
}

// out[k] = sum over the blocks of partial[2 * b + k], in block order
__global__ __launch_bounds__(256) void k_dot_finish(const double* __restrict__ partial, int blocks,
                                                    double* __restrict__ out) {
    __shared__ double sh[4];
    for (int k = 0; k < 2; ++k) {
        double s = 0;
        for (int b = threadIdx.x; b < blocks; b += 256) s += partial[2 * b + k];
        const double t = block_sum(s, sh);
        __syncthreads();
        if (threadIdx.x == 0) out[k] = t;
    }
}

// x += alpha p; r -= alpha q; partial sums of r . r
template <typename T>
__global__ __launch_bounds__(256) void k_cg_xr(int64_t n, T* __restrict__ x, T* __restrict__ r,
                                               const T* __restrict__ p, const T* __restrict__ q,
                                               T alpha, double* __restrict__ partial) {
    __shared__ double sh[4];
    double s = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        x[i] += alpha * p[i];
        const T ri = r[i] - alpha * q[i];
        r[i] = ri;
        s += (double)ri * (double)ri;
    }
    const double t = block_sum(s, sh);
    if (threadIdx.x == 0) partial[2 * blockIdx.x] = t, partial[2 * blockIdx.x + 1] = 0;
}

// p = r + beta (p - omega v)   (conjugate gradients: omega = 0, v unused)
template <typename T>
__global__ __launch_bounds__(256) void k_update_p(int64_t n, T* __restrict__ p,
                                                  const T* __restrict__ r, const T* __restrict__ v,
                                                  T beta, T omega) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = r[i] + beta * (v ? p[i] - omega * v[i] : p[i]);
}

// s = r - alpha v
template <typename T>
__global__ __launch_bounds__(256) void k_axmy(int64_t n, T* __restrict__ s,
                                              const T* __restrict__ r, const T* __restrict__ v,
                                              T alpha) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        s[i] = r[i] - alpha * v[i];
}

// x += alpha p + omega s; r = s - omega t; partial sums of r . r
template <typename T>
__global__ __launch_bounds__(256) void k_bicg_xr(int64_t n, T* __restrict__ x, T* __restrict__ r,
                                                 const T* __restrict__ p, const T* __restrict__ s,
                                                 const T* __restrict__ t, T alpha, T omega,
                                                 double* __restrict__ partial) {
    __shared__ double sh[4];
    double acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        x[i] += alpha * p[i] + omega * s[i];
        const T ri = s[i] - omega * t[i];
        r[i] = ri;
        acc += (double)ri * (double)ri;
    }
    const double tt = block_sum(acc, sh);
    if (threadIdx.x == 0) partial[2 * blockIdx.x] = tt, partial[2 * blockIdx.x + 1] = 0;
}

static unsigned grid_of(int64_t n) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, kDotBlocks));
}

hipError_t launch_dot2(int64_t n, bool f64, const void* a0, const void* b0, const void* a1,
                       const void* b1, double* partial, double* out, hipStream_t s) {
    const unsigned g = kDotBlocks;  // fixed grid: the same reduction order every time
    if (f64)
        hipLaunchKernelGGL(k_dot2<double>, dim3(g), dim3(256), 0, s, n, (const double*)a0,
                           (const double*)b0, (const double*)a1, (const double*)b1, partial);
    else
        hipLaunchKernelGGL(k_dot2<float>, dim3(g), dim3(256), 0, s, n, (const float*)a0,
                           (const float*)b0, (const float*)a1, (const float*)b1, partial);
    hipLaunchKernelGGL(k_dot_finish, dim3(1), dim3(256), 0, s, partial, (int)g, out);
    return hipGetLastError();
}

hipError_t launch_cg_xr(int64_t n, bool f64, void* x, void* r, const void* p, const void* q,
                        double alpha, double* partial, double* out, hipStream_t s) {
    const unsigned g = kDotBlocks;
    if (f64)
        hipLaunchKernelGGL(k_cg_xr<double>, dim3(g), dim3(256), 0, s, n, (double*)x, (double*)r,
                           (const double*)p, (const double*)q, alpha, partial);
    else
        hipLaunchKernelGGL(k_cg_xr<float>, dim3(g), dim3(256), 0, s, n, (float*)x, (float*)r,
                           (const float*)p, (const float*)q, (float)alpha, partial);
    hipLaunchKernelGGL(k_dot_finish, dim3(1), dim3(256), 0, s, partial, (int)g, out);
    return hipGetLastError();
}

hipError_t launch_update_p(int64_t n, bool f64, void* p, const void* r, const void* v,
                           double beta, double omega, hipStream_t s) {
    if (f64)
        hipLaunchKernelGGL(k_update_p<double>, dim3(grid_of(n)), dim3(256), 0, s, n, (double*)p,
                           (const double*)r, (const double*)v, beta, omega);
    else
        hipLaunchKernelGGL(k_update_p<float>, dim3(grid_of(n)), dim3(256), 0, s, n, (float*)p,
                           (const float*)r, (const float*)v, (float)beta, (float)omega);
    return hipGetLastError();
}

hipError_t launch_axmy(int64_t n, bool f64, void* s_out, const void* r, const void* v,
                       double alpha, hipStream_t s) {
    if (f64)
        hipLaunchKernelGGL(k_axmy<double>, dim3(grid_of(n)), dim3(256), 0, s, n, (double*)s_out,
                           (const double*)r, (const double*)v, alpha);
    else
        hipLaunchKernelGGL(k_axmy<float>, dim3(grid_of(n)), dim3(256), 0, s, n, (float*)s_out,
                           (const float*)r, (const float*)v, (float)alpha);
    return hipGetLastError();
}

hipError_t launch_bicg_xr(int64_t n, bool f64, void* x, void* r, const void* p, const void* s_in,
                          const void* t, double alpha, double omega, double* partial,
                          double* out, hipStream_t s) {
    const unsigned g = kDotBlocks;
    if (f64)
        hipLaunchKernelGGL(k_bicg_xr<double>, dim3(g), dim3(256), 0, s, n, (double*)x,
                           (double*)r, (const double*)p, (const double*)s_in, (const double*)t,
                           alpha, omega, partial);
    else
        hipLaunchKernelGGL(k_bicg_xr<float>, dim3(g), dim3(256), 0, s, n, (float*)x, (float*)r,
                           (const float*)p, (const float*)s_in, (const float*)t, (float)alpha,
                           (float)omega, partial);
    hipLaunchKernelGGL(k_dot_finish, dim3(1), dim3(256), 0, s, partial, (int)g, out);
    return hipGetLastError();
}

}  // namespace spmv
