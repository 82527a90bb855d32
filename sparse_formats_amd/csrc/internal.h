// Host-side declarations shared by the library's translation units: the
// device views of each format and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spmv {

// Widths above which a SELL slice is not run by one wave but split into
// column chunks of kSellChunk columns handled by separate waves (added into
// y with atomics).  A sorted slice is as long as its longest row, so a few
// very long rows would otherwise keep one wave busy for the whole apply.
constexpr int kSellSplitWidth = 256;
constexpr int kSellChunk = 128;

// Tail entries per lane of the load-balanced tail kernel (one wave takes
// 64 * kTailPerLane consecutive entries).
constexpr int kTailPerLane = 8;
constexpr int kTailChunk = 64 * kTailPerLane;

struct CsrView {
    int n;
    const int* rowptr;
    const int* col;
    const void* val;
};

struct EllView {
    int n;
    int64_t stride;   // rows padded to a multiple of 64
    const int* len;   // [stride]
    const int* col;   // [width * stride], slot (i, j) at j * stride + i
    const void* val;
};

struct SellView {
    int n;
    int nslices;
    const int64_t* slice_ptr;  // [nslices + 1]
    const int* len;            // [64 * nslices], sorted order
    const int* perm;           // [n]
    const int* col;
    const void* val;
    int nchunks;               // column chunks of split slices
    const int4* chunks;        // (slice, j0, j1, 0)
};

struct TailView {
    int n;
    int64_t nnz;
    const int* row;        // COO row ids (HYB) or nullptr
    const int* ptr;        // CSR tail pointer [n+1] (HEC) or nullptr
    const int* chunk_row;  // HEC: row of the first entry of each wave chunk
    const int* col;
    const void* val;
};

// kernel launchers (asynchronous on `stream`); fp64 when f64, else fp32
hipError_t launch_csr(const CsrView& a, int subwave, bool f64, void* y, const void* x,
                      double alpha, double beta, hipStream_t stream);
hipError_t launch_ell(const EllView& a, bool f64, void* y, const void* x, double alpha,
                      double beta, hipStream_t stream);
hipError_t launch_sell(const SellView& a, bool f64, void* y, const void* x, double alpha,
                       double beta, hipStream_t stream);
hipError_t launch_tail(const TailView& t, bool f64, void* y, const void* x, double alpha,
                       hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

}  // namespace spmv
