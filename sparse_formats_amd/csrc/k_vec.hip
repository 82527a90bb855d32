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

// The scalars of an iteration live in device memory (st, indexed by
// SolveState): a one-workgroup step kernel computes them from the inner
// products and the vector kernels read them, so an iteration needs no host
// round trip and can be replayed from a HIP graph.  Once st[kStDone] is set every kernel below
// leaves without writing, so iterations enqueued past convergence change
// nothing.
__device__ __forceinline__ bool solve_done(const double* st) { return st[kStDone] != 0.0; }

// Sum the partial products in block order (as k_dot_finish), then one
// thread advances the iteration's scalars:
//   kStepCgPQ     p.q
//   kStepCgRR     r.r of the new residual: beta = rr_new / rr, rr = rr_new,
//                 k += 1, done when ||r|| <= goal or k == max_iter
//   kStepBiRV     alpha = rho_new / rhat.v
//   kStepBiOmega  omega = t.s / t.t (0 when t = 0)
//   kStepBiRR     rr = r.r, rho = rho_new, k += 1, done as for CG or when
//                 omega == 0 (s was already the residual of x + alpha p);
//                 then for the next iteration rho_new = rhat.r (done on
//                 breakdown rho_new == 0) and beta = (rho_new / rho)
//                 (alpha / omega)
__device__ void solve_step(const double* __restrict__ partial, int blocks,
                           double* __restrict__ st, int step) {
    __shared__ double sh[4];
    double t[2];
    for (int k = 0; k < 2; ++k) {
        double s = 0;
        for (int b = threadIdx.x; b < blocks; b += 256) s += partial[2 * b + k];
        t[k] = block_sum(s, sh);
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    auto advance = [&](double rr) {
        st[kStRR] = rr;
        const double k = st[kStK] + 1.0;
        st[kStK] = k;
        if (!(sqrt(rr) > st[kStGoal]) || k >= st[kStMaxIt]) st[kStDone] = 1.0;
    };
    switch (step) {
        case kStepCgPQ:
            st[kStPQ] = t[0];
            break;
        case kStepCgRR:
            st[kStBeta] = st[kStRR] != 0.0 ? t[0] / st[kStRR] : 0.0;
            advance(t[0]);
            break;
        case kStepBiRV:
            st[kStAlpha] = st[kStRhoNew] / t[0];
            break;
        case kStepBiOmega:
            st[kStOmega] = t[1] > 0 ? t[0] / t[1] : 0.0;
            break;
        case kStepBiRR:
            st[kStRho] = st[kStRhoNew];
            advance(t[0]);
            if (st[kStOmega] == 0.0) st[kStDone] = 1.0;
            if (st[kStDone] != 0.0) break;
            if (t[1] == 0.0) {
                st[kStDone] = 1.0;
                break;
            }
            st[kStBeta] = (t[1] / st[kStRho]) * (st[kStAlpha] / st[kStOmega]);
            st[kStRhoNew] = t[1];
            break;
    }
}

// one workgroup: the step on the partial sums of the reduction kernel before
__global__ __launch_bounds__(256) void k_solve_step(const double* __restrict__ partial, int blocks,
                                                    double* __restrict__ st, int step) {
    if (solve_done(st)) return;
    solve_step(partial, blocks, st, step);
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

// x += alpha p; r -= alpha q; partial sums of r . r   (alpha = rr / p.q)
template <typename T>
__global__ __launch_bounds__(256) void k_cg_xr(int64_t n, T* __restrict__ x, T* __restrict__ r,
                                               const T* __restrict__ p, const T* __restrict__ q,
                                               const double* __restrict__ st,
                                               double* __restrict__ partial) {
    __shared__ double sh[4];
    if (solve_done(st)) return;
    const T alpha = (T)(st[kStPQ] != 0.0 ? st[kStRR] / st[kStPQ] : 0.0);
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

// p = r + beta (p - omega v)   (conjugate gradients: v == nullptr, p = r + beta p)
template <typename T>
__global__ __launch_bounds__(256) void k_update_p(int64_t n, T* __restrict__ p,
                                                  const T* __restrict__ r, const T* __restrict__ v,
                                                  const double* __restrict__ st) {
    if (solve_done(st)) return;
    const T beta = (T)st[kStBeta], omega = (T)(v ? st[kStOmega] : 0.0);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = r[i] + beta * (v ? p[i] - omega * v[i] : p[i]);
}

// s = r - alpha v
template <typename T>
__global__ __launch_bounds__(256) void k_axmy(int64_t n, T* __restrict__ s,
                                              const T* __restrict__ r, const T* __restrict__ v,
                                              const double* __restrict__ st) {
    if (solve_done(st)) return;
    const T alpha = (T)st[kStAlpha];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        s[i] = r[i] - alpha * v[i];
}

// x += alpha p + omega s; r = s - omega t; partial sums of r . r and of
// rhat . r (the next iteration's rho)
template <typename T>
__global__ __launch_bounds__(256) void k_bicg_xr(int64_t n, T* __restrict__ x, T* __restrict__ r,
                                                 const T* __restrict__ p, const T* __restrict__ s,
                                                 const T* __restrict__ t, const T* __restrict__ rh,
                                                 const double* __restrict__ st,
                                                 double* __restrict__ partial) {
    __shared__ double sh[4];
    if (solve_done(st)) return;
    const T alpha = (T)st[kStAlpha], omega = (T)st[kStOmega];
    double acc = 0, acc_h = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        x[i] += alpha * p[i] + omega * s[i];
        const T ri = s[i] - omega * t[i];
        r[i] = ri;
        acc += (double)ri * (double)ri;
        acc_h += (double)rh[i] * (double)ri;
    }
    const double tt = block_sum(acc, sh);
    __syncthreads();
    const double th = block_sum(acc_h, sh);
    if (threadIdx.x == 0) partial[2 * blockIdx.x] = tt, partial[2 * blockIdx.x + 1] = th;
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
    if (out) hipLaunchKernelGGL(k_dot_finish, dim3(1), dim3(256), 0, s, partial, (int)g, out);
    return hipGetLastError();
}

hipError_t launch_solve_step(const double* partial, double* st, int step, hipStream_t s) {
    hipLaunchKernelGGL(k_solve_step, dim3(1), dim3(256), 0, s, partial, (int)kDotBlocks, st, step);
    return hipGetLastError();
}

hipError_t launch_cg_xr(int64_t n, bool f64, void* x, void* r, const void* p, const void* q,
                        const double* st, double* partial, hipStream_t s) {
    const unsigned g = kDotBlocks;
    if (f64)
        hipLaunchKernelGGL(k_cg_xr<double>, dim3(g), dim3(256), 0, s, n, (double*)x, (double*)r,
                           (const double*)p, (const double*)q, st, partial);
    else
        hipLaunchKernelGGL(k_cg_xr<float>, dim3(g), dim3(256), 0, s, n, (float*)x, (float*)r,
                           (const float*)p, (const float*)q, st, partial);
    return hipGetLastError();
}

hipError_t launch_update_p(int64_t n, bool f64, void* p, const void* r, const void* v,
                           const double* st, hipStream_t s) {
    if (f64)
        hipLaunchKernelGGL(k_update_p<double>, dim3(grid_of(n)), dim3(256), 0, s, n, (double*)p,
                           (const double*)r, (const double*)v, st);
    else
        hipLaunchKernelGGL(k_update_p<float>, dim3(grid_of(n)), dim3(256), 0, s, n, (float*)p,
                           (const float*)r, (const float*)v, st);
    return hipGetLastError();
}

hipError_t launch_axmy(int64_t n, bool f64, void* s_out, const void* r, const void* v,
                       const double* st, hipStream_t s) {
    if (f64)
        hipLaunchKernelGGL(k_axmy<double>, dim3(grid_of(n)), dim3(256), 0, s, n, (double*)s_out,
                           (const double*)r, (const double*)v, st);
    else
        hipLaunchKernelGGL(k_axmy<float>, dim3(grid_of(n)), dim3(256), 0, s, n, (float*)s_out,
                           (const float*)r, (const float*)v, st);
    return hipGetLastError();
}

hipError_t launch_bicg_xr(int64_t n, bool f64, void* x, void* r, const void* p, const void* s_in,
                          const void* t, const void* rh, const double* st, double* partial,
                          hipStream_t s) {
    const unsigned g = kDotBlocks;
    if (f64)
        hipLaunchKernelGGL(k_bicg_xr<double>, dim3(g), dim3(256), 0, s, n, (double*)x,
                           (double*)r, (const double*)p, (const double*)s_in, (const double*)t,
                           (const double*)rh, st, partial);
    else
        hipLaunchKernelGGL(k_bicg_xr<float>, dim3(g), dim3(256), 0, s, n, (float*)x, (float*)r,
                           (const float*)p, (const float*)s_in, (const float*)t, (const float*)rh,
                           st, partial);
    return hipGetLastError();
}

}  // namespace spmv
