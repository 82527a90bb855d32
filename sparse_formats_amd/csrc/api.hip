// Handle management, validation, COO/CSR ingest and the device-side format
// converters behind the C ABI declared in include/spmv_amd.h.
//
// Conversions run on the device from the handle's CSR copy.  Only a few
// scalars (and, for HYB/HEC, the row-length histogram; for SELL-64, the slice
// widths) come back to the host to size allocations and pick the split.
#include <cstring>
#include <hip/hip_runtime.h>
#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>
#include <rocprim/device/device_segmented_radix_sort.hpp>
#include <rocprim/device/device_select.hpp>
#include <rocprim/iterator/counting_iterator.hpp>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <functional>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "spmv_amd.h"
#include "common.h"
#include "index_math.h"
#include "internal.h"

using namespace spmv;

namespace {

thread_local std::string g_err;

struct Error {
    int code;
    std::string msg;
};

[[noreturn]] void fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    throw Error{code, buf};
}

void hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return;
    (void)hipGetLastError();
    fail(e == hipErrorOutOfMemory ? SPMV_ERR_NO_MEMORY : SPMV_ERR_HIP, "%s: %s", what,
         hipGetErrorString(e));
}

// owning device buffer
struct DevBuf {
    void* p = nullptr;
    size_t bytes = 0;
    DevBuf() = default;
    explicit DevBuf(size_t n) { alloc(n); }
    DevBuf(const DevBuf&) = delete;
    DevBuf& operator=(const DevBuf&) = delete;
    DevBuf(DevBuf&& o) noexcept : p(o.p), bytes(o.bytes) { o.p = nullptr, o.bytes = 0; }
    DevBuf& operator=(DevBuf&& o) noexcept {
        if (this != &o) {
            release();
            p = o.p, bytes = o.bytes;
            o.p = nullptr, o.bytes = 0;
        }
        return *this;
    }
    ~DevBuf() { release(); }
    void alloc(size_t n) {
        release();
        void* q = nullptr;
        hipError_t e = hipMalloc(&q, std::max<size_t>(n, 256));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            fail(SPMV_ERR_NO_MEMORY, "device allocation of %zu bytes failed: %s", n,
                 hipGetErrorString(e));
        }
        p = q;
        bytes = n;
    }
    void release() {
        if (p) (void)hipFree(p);
        p = nullptr;
        bytes = 0;
    }
    template <typename T>
    T* as() const {
        return static_cast<T*>(p);
    }
};

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

// a shape of the vector CSR kernel: lanes per row, rows per lane group,
// LDS slots per wave when staged (0: direct), col read without caching
struct VecShape {
    int subwave = 1, rows = 1, slots = 0;
    bool col_nt = false;
};

// the arrays of one converted (non-CSR) format
struct Built {
    int format = SPMV_CSR;
    // ELL-R, or the ELL part of HYB / HEC
    int64_t ell_width = 0, ell_bh = 0, ell_rows = 0;  // width, rows per block, padded rows
    DevBuf ell_col, ell_val, ell_len;
    bool ell_records = false;  // ELLPACK-R: ell_col holds (value, column) slot records
    // ELLPACK-R with the x window and a few long rows: the window kernel takes
    // each row's first ell_head slots, a wave per row of ell_long the rest
    int ell_head = 0x7fffffff;
    DevBuf ell_long;
    int64_t ell_nlong = 0;
    DevBuf ell_perm;      // sorted ELL part: row at each position (else empty)
    int ell_groups = 1;   // wave groups per 64-row tile
    int sort_window = 0;  // rows per sort window in effect (0: none)
    // SELL-64
    int64_t nslices = 0, sell_slots = 0;
    DevBuf slice_ptr, sell_len, perm, sell_col, sell_val;
    int64_t nchunks = 0;
    DevBuf chunks, chunk_off;  // column chunks of long slices, first chunk per slice
    // tail of HYB / HEC
    int64_t tail_nnz = 0, tail_runs = 0;
    DevBuf tail_row, tail_ptr, tail_col, tail_val, run_row;
    // HEC: the tail pointer over the rows that have tail entries only
    // (tail_rows: those rows; tail_cptr: their starts + the end)
    int64_t tail_nrows = 0;
    DevBuf tail_rows, tail_cptr;
    // HEC: the tail runs as the vector CSR kernel over the compressed rows
    // (added onto the ELL part, no atomics) instead of the balanced kernel
    bool tail_vector = false;
    bool tail_xblock = false;  // HEC: the tail by column slices (b.xb)
    VecShape tail_vec;
    // CSR: entry-balanced kernel (run rows over the whole matrix)
    bool csr_balanced = false;
    // CSR by column slices (the view holds the pointers below)
    bool csr_xblock = false;
    DevBuf xb_rows, xb_tiles, xb_col, xb_val, xb_lrow;
    XblkView xb{};
    void release_xblock() {
        xb = XblkView{};
        xb_rows.release(), xb_tiles.release(), xb_col.release();
        xb_val.release(), xb_lrow.release();
    }
    // SELL-64 in the permuted basis (x and y in sorted row order)
    bool permuted = false;
    // x staged in LDS by the ELL / tail kernels
    bool window = false;
    // ELL-R / SELL-64 / ELL part: col read without caching (else cached)
    bool col_nt = true;
    double band_fraction = 0;

    size_t bytes() const {
        return ell_col.bytes + ell_val.bytes + ell_len.bytes + ell_perm.bytes + slice_ptr.bytes +
               sell_len.bytes +
               perm.bytes + sell_col.bytes + sell_val.bytes + chunks.bytes + chunk_off.bytes +
               tail_row.bytes +
               tail_ptr.bytes + tail_col.bytes + tail_val.bytes + run_row.bytes + tail_rows.bytes +
               tail_cptr.bytes + ell_long.bytes + xb_rows.bytes + xb_tiles.bytes + xb_col.bytes + xb_val.bytes +
               xb_lrow.bytes;
    }
};

}  // namespace

struct spmv_handle {
    int64_t n = 0, nnz = 0;
    int dtype = SPMV_F64;
    size_t vsize = 8;
    int max_len = 0;
    int subwave = 1;
    int csr_rows = 1;     // rows per lane group of the CSR kernel
    int csr_stage_slots = 0;  // CSR: LDS slots per wave of the staged kernel (0: direct)
    bool csr_stage_col_nt = false;  // staged CSR: col read without caching
    int device = 0;           // device current at spmv_create (holds every buffer)
    DevBuf rowptr, col, val;  // canonical CSR (int32 row pointer); col and val
                              // end with 16 zero bytes (whole 16-byte loads)
    Built fmt;                // active non-CSR format (format == CSR: none)
    int format = SPMV_CSR;
};

namespace {

// ---------------------------------------------------------------------------
// setup kernels
// ---------------------------------------------------------------------------
enum : int { F_FIRST = 1, F_LAST = 2, F_MONO = 4, F_COL = 8, F_ROW = 16 };

__global__ void k_validate_csr(int64_t n, int64_t nnz, const int64_t* __restrict__ rp,
                               const int32_t* __restrict__ col, int* flags,
                               int* __restrict__ rp32) {
    const int64_t m = std::max(n + 1, nnz);
    int f = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i <= n) {
            const int64_t v = rp[i];
            rp32[i] = (int)v;
            if (i == 0 && v != 0) f |= F_FIRST;
            if (i == n && v != nnz) f |= F_LAST;
            if (i < n && rp[i + 1] < v) f |= F_MONO;
        }
        if (i < nnz) {
            const int c = col[i];
            if (c < 0 || c >= n) f |= F_COL;
        }
    }
    if (f) atomicOr(flags, f);
}

__global__ void k_validate_coo(int64_t n, int64_t nnz, const int64_t* __restrict__ row,
                               const int32_t* __restrict__ col, int* flags,
                               unsigned* __restrict__ row32) {
    int f = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nnz;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = row[i];
        const int c = col[i];
        if (r < 0 || r >= n) f |= F_ROW;
        if (c < 0 || c >= n) f |= F_COL;
        row32[i] = (unsigned)r;
    }
    if (f) atomicOr(flags, f);
}

// gather the CSR entries of COO input in sorted order
__global__ void k_gather(int64_t nnz, const int* __restrict__ order,
                         const int32_t* __restrict__ col_in, const char* __restrict__ val_in,
                         int vsize, int* __restrict__ col, char* __restrict__ val) {
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = order[k];
        col[k] = col_in[s];
        if (vsize == 8)
            reinterpret_cast<double*>(val)[k] = reinterpret_cast<const double*>(val_in)[s];
        else
            reinterpret_cast<float*>(val)[k] = reinterpret_cast<const float*>(val_in)[s];
    }
}

// rowptr[r] = first sorted entry with row >= r
__global__ void k_rowptr_from_sorted(int64_t n, int64_t nnz, const unsigned* __restrict__ rows,
                                     int* __restrict__ rowptr) {
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r <= n;
         r += (int64_t)gridDim.x * blockDim.x) {
        int64_t lo = 0, hi = nnz;
        while (lo < hi) {
            const int64_t m = (lo + hi) >> 1;
            if ((int64_t)rows[m] < r)
                lo = m + 1;
            else
                hi = m;
        }
        rowptr[r] = (int)lo;
    }
}

__global__ __launch_bounds__(256) void k_max_len(int64_t n, const int* __restrict__ rowptr,
                                                 int* out) {
    __shared__ int wmax[4];
    int m = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        m = max(m, rowptr[i + 1] - rowptr[i]);
    for (int d = 32; d > 0; d >>= 1) m = max(m, __shfl_xor(m, d));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {  // one atomic per block
        m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
        if (m) atomicMax(out, m);
    }
}

// row-length histogram; short lengths are counted in LDS first because a
// handful of bins would otherwise take an atomic from every row
constexpr int kHistLds = 2048;
__global__ __launch_bounds__(256) void k_len_hist(int64_t n, int W, const int* __restrict__ rowptr,
                                                  int* __restrict__ hist) {
    __shared__ int lh[kHistLds];
    for (int b = threadIdx.x; b < kHistLds; b += blockDim.x) lh[b] = 0;
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int L = rowptr[i + 1] - rowptr[i];
        if (L < kHistLds)
            atomicAdd(lh + L, 1);
        else
            atomicAdd(hist + L, 1);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kHistLds && b <= W; b += blockDim.x)
        if (lh[b]) atomicAdd(hist + b, lh[b]);
}

// ELL slots in blocks of bh rows, each block column by column: storage
// position t holds entry j of row i (j < min(len_i, W)), otherwise column 0 /
// value +0; len[i] = min(len_i, W), 0 for padded rows.
template <typename V>
__global__ void k_ell_fill(int64_t n, int64_t rows, int64_t bh, int64_t W,
                           const int* __restrict__ rowptr, const int* __restrict__ col,
                           const V* __restrict__ val, const int* __restrict__ perm,
                           int* __restrict__ ecol, V* __restrict__ eval, int* __restrict__ elen) {
    const int64_t total = rows * W;
    const int64_t bstride = bh * W;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t blk = t / bstride, rem = t - blk * bstride;
        const int64_t j = rem / bh, p = blk * bh + (rem - j * bh);
        const int64_t i = perm && p < n ? perm[p] : p;  // row at position p
        int c = 0;
        V v = V(0);
        if (i < n) {
            const int k0 = rowptr[i];
            const int64_t L = std::min<int64_t>(rowptr[i + 1] - k0, W);
            if (j < L) {
                c = col[k0 + j];
                v = val[k0 + j];
            }
        }
        if (eval) {
            ecol[t] = c;
            eval[t] = v;
        } else {
            st_rec(ecol, t, v, c);  // records in ecol
        }
    }
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < rows;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = perm && p < n ? perm[p] : p;
        elen[p] = i < n ? (int)std::min<int64_t>(rowptr[i + 1] - rowptr[i], W) : 0;
    }
}

// out[k * w .. k * w + w) = rec[k * r + o .. k * r + o + w): one field (w ints
// at int offset o) of each of k records of r ints
__global__ void k_ell_split(int64_t k, int r, int o, int w, const int* __restrict__ rec,
                            int* __restrict__ out) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < k;
         t += (int64_t)gridDim.x * blockDim.x)
        for (int q = 0; q < w; ++q) out[t * w + q] = rec[t * r + o + q];
}

// Windowed sort of one kEllBlock-row block of the ELL part (one workgroup
// per block): positions ordered by (position / sigma, stored length
// descending, row ascending).  The keys are unique, so a bitonic sort of
// the block's keys in LDS gives the one ordering; padding rows (>= n) have
// length 0 and the largest rows of their window, so they stay in place.
__global__ __launch_bounds__(kEllBlock) void k_ell_block_sort(int64_t n, int64_t W, int sigma,
                                                              const int* __restrict__ rowptr,
                                                              int* __restrict__ perm) {
    __shared__ unsigned long long key[kEllBlock];
    const int p = threadIdx.x;
    const int64_t pos = (int64_t)blockIdx.x * kEllBlock + p;  // also the row before sorting
    int64_t len = 0;
    if (pos < n) len = std::min<int64_t>(rowptr[pos + 1] - rowptr[pos], W);
    // window (4 bits) | 2^32 - 1 - length (32 bits) | position in block (10 bits)
    key[p] = ((unsigned long long)(p / sigma) << 42) |
             ((unsigned long long)(0xFFFFFFFFu - (unsigned)len) << 10) | (unsigned)p;
    __syncthreads();
    for (int k = 2; k <= kEllBlock; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int q = p ^ j;
            if (q > p) {
                const unsigned long long a = key[p], b = key[q];
                if ((a > b) == ((p & k) == 0)) key[p] = b, key[q] = a;
            }
            __syncthreads();
        }
    perm[pos] = (int)((int64_t)blockIdx.x * kEllBlock + (int)(key[p] & (kEllBlock - 1)));
}

// padding read by waves of 64 unsorted rows: out[0] += sum of stored
// lengths, out[1] += 64 * longest stored length (one wave per 64 rows)
__global__ __launch_bounds__(256) void k_ell_pad_count(int64_t n, int64_t W,
                                                       const int* __restrict__ rowptr,
                                                       unsigned long long* __restrict__ out) {
    const int64_t waves = (n + 63) / 64;
    const int lane = threadIdx.x & 63;
    for (int64_t w = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64; w < waves;
         w += (int64_t)gridDim.x * blockDim.x / 64) {
        const int64_t i = w * 64 + lane;
        int mx = i < n ? (int)std::min<int64_t>(rowptr[i + 1] - rowptr[i], W) : 0;
        long long sum = mx;
        for (int o = 32; o > 0; o >>= 1) {
            mx = max(mx, __shfl_xor(mx, o));
            sum += __shfl_xor(sum, o);
        }
        if (lane == 0) {
            atomicAdd(out, (unsigned long long)sum);
            atomicAdd(out + 1, 64ull * (unsigned long long)mx);
        }
    }
}

// entries within `lead` positions of their row (reach of the LDS window)
__global__ void k_band_count(int64_t n, int64_t lead, const int* __restrict__ rowptr,
                             const int* __restrict__ col, unsigned long long* out) {
    unsigned long long cnt = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        for (int k = rowptr[i]; k < rowptr[i + 1]; ++k) {
            const int64_t d = (int64_t)col[k] - i;
            cnt += (d >= -lead && d <= lead) ? 1u : 0u;
        }
    for (int d = 32; d > 0; d >>= 1) cnt += __shfl_xor(cnt, d);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(out, cnt);
}

// sort key for SELL: rows by length descending; the radix sort is stable,
// so equal lengths keep ascending row order
__global__ void k_sell_keys(int64_t n, int W, const int* __restrict__ rowptr,
                            unsigned* __restrict__ key) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        key[i] = (unsigned)(W - (rowptr[i + 1] - rowptr[i]));
}

// windowed sort key: window << 32 | (W - length)
__global__ void k_sell_keys_win(int64_t n, int64_t sigma, int W, const int* __restrict__ rowptr,
                                unsigned long long* __restrict__ key) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        key[i] = ((unsigned long long)(i / sigma) << 32) |
                 (unsigned)(W - (rowptr[i + 1] - rowptr[i]));
}

__global__ void k_iota(int64_t n, int* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = (int)i;
}

// inv[perm[r]] = r
__global__ void k_invert_perm(int64_t n, const int* __restrict__ perm, int* __restrict__ inv) {
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n;
         r += (int64_t)gridDim.x * blockDim.x)
        inv[perm[r]] = (int)r;
}

// lengths in sorted order (0 for the padding rows)
__global__ void k_sell_len(int64_t n, int64_t S, const int* __restrict__ rowptr,
                           const int* __restrict__ perm, int* __restrict__ slen) {
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < S;
         r += (int64_t)gridDim.x * blockDim.x)
        slen[r] = r < n ? rowptr[perm[r] + 1] - rowptr[perm[r]] : 0;
}

// slots of each slice: 64 * its longest row (the first one unless a sort
// window boundary or unsorted rows fall inside the slice)
__global__ void k_sell_width(int64_t ns, const int* __restrict__ slen,
                             int64_t* __restrict__ slots) {
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < ns;
         q += (int64_t)gridDim.x * blockDim.x) {
        int w = 0;
        for (int l = 0; l < 64; ++l) w = max(w, slen[q * 64 + l]);
        slots[q] = 64 * (int64_t)w;
    }
}

// one wave per slice
template <typename V>
__global__ void k_sell_fill(int64_t n, int64_t nslices, const int* __restrict__ rowptr,
                            const int* __restrict__ col, const V* __restrict__ val,
                            const int* __restrict__ perm, const int* __restrict__ inv,
                            const int64_t* __restrict__ sp, const int* __restrict__ slen,
                            int* __restrict__ scol, V* __restrict__ sval) {
    const int64_t s = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (s >= nslices) return;
    const int lane = threadIdx.x & 63;
    const int64_t r = s * 64 + lane;
    const int64_t base = sp[s];
    const int64_t w = (sp[s + 1] - base) >> 6;
    const int L = slen[r];
    const int k0 = r < n ? rowptr[perm[r]] : 0;
    for (int64_t j = 0; j < w; ++j) {
        const int64_t slot = base + 64 * j + lane;
        if (j < L) {
            // permuted basis: column c becomes the sorted position of row c
            scol[slot] = inv ? inv[col[k0 + j]] : col[k0 + j];
            sval[slot] = val[k0 + j];
        } else {
            scol[slot] = 0;
            sval[slot] = V(0);
        }
    }
}

// tail lengths max(len - K, 0)
__global__ void k_tail_len(int64_t n, int K, const int* __restrict__ rowptr,
                           int* __restrict__ tlen) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        tlen[i] = max(rowptr[i + 1] - rowptr[i] - K, 0);
}

__global__ void k_tail_flags(int64_t n, const int* __restrict__ tptr, int* __restrict__ flag) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        flag[i] = tptr[i + 1] > tptr[i] ? 1 : 0;
}

// rows with tail entries: rows[pos[i]] = i and cptr[pos[i]] = tptr[i] for
// every row i with tptr[i + 1] > tptr[i] (pos = exclusive count of such rows)
__global__ void k_compact_rows(int64_t n, const int* __restrict__ tptr,
                               const int* __restrict__ pos, int* __restrict__ rows,
                               int* __restrict__ cptr) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        if (tptr[i + 1] > tptr[i]) {
            rows[pos[i]] = (int)i;
            cptr[pos[i]] = tptr[i];
        }
}

// one wave per row: entries K.. of row i go to tail slots tptr[i]..
template <typename V>
__global__ void k_tail_fill(int64_t n, int K, const int* __restrict__ rowptr,
                            const int* __restrict__ col, const V* __restrict__ val,
                            const int* __restrict__ tptr, int* __restrict__ trow,
                            int* __restrict__ tcol, V* __restrict__ tval) {
    const int lane = threadIdx.x & 63;
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); i < n;
         i += (int64_t)gridDim.x * (blockDim.x >> 6)) {  // one wave per row
        const int t0 = tptr[i], t1 = tptr[i + 1];
        const int k0 = rowptr[i] + K;
        for (int t = t0 + lane; t < t1; t += 64) {
            tcol[t] = col[k0 + (t - t0)];
            tval[t] = val[k0 + (t - t0)];
            if (trow) trow[t] = (int)i;
        }
    }
}

// run_row[k] = row holding entry k * kTailPerLane (the first entry of lane
// run k) for k < nruns, and run_row[nruns] = n - 1; one thread per row
// writes the runs that start inside the row
__global__ void k_run_rows(int64_t n, int64_t nruns, const int* __restrict__ ptr,
                           int* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k0 = ((int64_t)ptr[i] + kTailPerLane - 1) / kTailPerLane;
        const int64_t k1 = ((int64_t)ptr[i + 1] + kTailPerLane - 1) / kTailPerLane;
        for (int64_t k = k0; k < k1; ++k) out[k] = (int)i;
        if (i == 0) out[nruns] = (int)(n - 1);
    }
}

// Histogram of the LDS slots the staged CSR kernel needs per wave (entries
// of its rw rows from the 16-byte aligned start), in buckets of 64; the last
// bucket collects everything above.
__global__ void k_stage_hist(int64_t n, int rw, const int* __restrict__ ptr, int nb,
                             unsigned* __restrict__ hist) {
    const int64_t waves = (n + rw - 1) / rw;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < waves;
         w += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r0 = w * rw, r1 = std::min<int64_t>(r0 + rw, n);
        const int need = ptr[r1] - (ptr[r0] & -4);
        atomicAdd(&hist[std::min(need / 64, nb - 1)], 1u);
    }
}

unsigned grid_for(int64_t work, int64_t per_block = 256) {
    int64_t b = (work + per_block - 1) / per_block;
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 65536));
}

unsigned bits_for(uint64_t v) {
    unsigned b = 1;
    while (b < 32 && (v >> b)) ++b;
    return b;
}

void sync(hipStream_t s) { hip_check(hipStreamSynchronize(s), "hipStreamSynchronize"); }

template <typename T>
T read_scalar(const void* dev, hipStream_t s) {
    T v{};
    hip_check(hipMemcpyAsync(&v, dev, sizeof(T), hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
    sync(s);
    return v;
}

// ---------------------------------------------------------------------------
// converters
// ---------------------------------------------------------------------------
uint64_t budget_bytes(const spmv_convert_opts& o) {
    if (o.footprint_budget_bytes) return o.footprint_budget_bytes;
    size_t fr = 0, tot = 0;
    hip_check(hipMemGetInfo(&fr, &tot), "hipMemGetInfo");
    return (uint64_t)(0.75 * (double)tot);
}

// ELL arrays of width W: one column-major block of all rows (block = 0,
// ELLPACK-R, whose slots are (value, column) records) or column-major blocks
// of `block` rows (ELL part of HYB/HEC, separate value and column arrays)
template <typename V>
void build_ell_part(const spmv_handle* h, int64_t W, int64_t block, int sigma, Built& b,
                    hipStream_t s) {
    const int64_t bh = block > 0 ? block : pad64(h->n);
    const int64_t rows = block > 0 ? (h->n + block - 1) / block * block : bh;
    b.ell_width = W;
    b.ell_bh = bh;
    b.ell_rows = rows;
    b.ell_records = block == 0;
    if (b.ell_records) {
        b.ell_col.alloc((size_t)(W * rows) * (sizeof(V) + 4));
        b.ell_val.release();
    } else {
        b.ell_col.alloc((size_t)(W * rows) * 4);
        b.ell_val.alloc((size_t)(W * rows) * sizeof(V));
    }
    b.ell_len.alloc((size_t)rows * 4);
    b.sort_window = 0;
    if (sigma > 0 && rows > 0) {  // block == kEllBlock, sigma divides it
        b.ell_perm.alloc((size_t)rows * 4);
        hipLaunchKernelGGL(k_ell_block_sort, dim3((unsigned)(rows / kEllBlock)), dim3(kEllBlock), 0,
                           s, h->n, W, sigma, h->rowptr.as<int>(), b.ell_perm.as<int>());
        hip_check(hipGetLastError(), "ell block sort");
        b.sort_window = sigma;
    }
    hipLaunchKernelGGL(k_ell_fill<V>, dim3(grid_for(std::max<int64_t>(W * rows, rows))), dim3(256),
                       0, s, h->n, rows, std::max<int64_t>(bh, 1), W, h->rowptr.as<int>(),
                       h->col.as<int>(), h->val.as<V>(), b.ell_perm.as<int>(), b.ell_col.as<int>(),
                       b.ell_records ? nullptr : b.ell_val.as<V>(), b.ell_len.as<int>());
    hip_check(hipGetLastError(), "ell fill");
}

// a timed alternative to the simpler kernel (no LDS window, no atomics) is
// kept only when it is at least this much faster
constexpr float kPreferMargin = 0.95f;
// the second HYB/HEC width candidate must be this much faster to be kept
// (the two are timed again when within 3 % of each other)
constexpr float kWidthMargin = 0.99f;
// the column-slice CSR kernel is a candidate only for x above one XCD's L2
constexpr int64_t kXbMinX = 4 << 20;
// entry indices are 32-bit in the kernels, which step past a row's end by up
// to a few hundred entries before masking: keep that headroom below 2^31
constexpr int64_t kMaxNnz = INT32_MAX - 65536;

// automatic format choice: ELL-R is a candidate only while its padded slots
// are at most this many times the stored entries
constexpr double kAutoEllPadding = 1.5;

// the ELL part of HYB/HEC is sorted inside its blocks (by default) when
// waves of 64 unsorted rows would read more than this share of padding
constexpr double kSortPadShare = 0.10;

// share of padding slots that waves of 64 unsorted rows would read in an
// ELL part of width W
double ell_pad_fraction(const spmv_handle* h, int64_t W, hipStream_t s) {
    if (h->n == 0 || W == 0) return 0.0;
    DevBuf cnt(16);
    hip_check(hipMemsetAsync(cnt.p, 0, 16, s), "hipMemsetAsync");
    hipLaunchKernelGGL(k_ell_pad_count, dim3(std::min<unsigned>(grid_for(h->n), 4096)), dim3(256), 0,
                       s, h->n, W, h->rowptr.as<int>(), cnt.as<unsigned long long>());
    hip_check(hipGetLastError(), "padding count");
    unsigned long long c[2];
    hip_check(hipMemcpyAsync(c, cnt.p, 16, hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
    sync(s);
    return c[1] ? 1.0 - (double)c[0] / (double)c[1] : 0.0;
}

// sort_window: -1 sorts inside windows of kSellSortWindow rows, 0 keeps
// the row order, k >= 1 sorts inside aligned windows of k rows (k >= n: all
// rows at once, the pJDS order).  permuted: store P A P^T (columns renumbered
// to sorted positions; apply works in the sorted basis).
// Column chunks of the long slices of a built SELL layout, on the device:
// without the LDS window the slices wider than kSellSplitWidth go to
// k_sell_chunks whole, in chunks of kSellChunk columns; with it the columns
// of the slices wider than kSellWinWide past kSellWinHead, in chunks of
// kSellWinChunk columns per group of 16 rows, up to each group's longest row
// (k_sell_win).  chunk_off[q] is the first chunk of slice q.
void build_sell_chunks(Built& b, bool window, hipStream_t s) {
    const int64_t ns = b.nslices;
    const int split = window ? kSellWinWide : kSellSplitWidth;
    const int head = window ? kSellWinHead : 0;
    const int chunk = window ? kSellWinChunk : kSellChunk;
    b.window = window;
    b.chunk_off.alloc((size_t)(ns + 1) * 4);
    hip_check(hipMemsetAsync(b.chunk_off.p, 0, 4, s), "hipMemsetAsync");
    if (ns > 0) {
        DevBuf cnt((size_t)ns * 4);
        hip_check(launch_sell_chunk_count(ns, b.slice_ptr.as<int64_t>(), b.sell_len.as<int>(),
                                          split, head, chunk, window, cnt.as<int>(), s),
                  "sell chunk counts");
        size_t tmp = 0;
        hip_check(rocprim::inclusive_scan(nullptr, tmp, cnt.as<int>(), b.chunk_off.as<int>() + 1,
                                          (size_t)ns, rocprim::plus<int>(), s),
                  "inclusive_scan");
        DevBuf work(tmp);
        hip_check(rocprim::inclusive_scan(work.p, tmp, cnt.as<int>(), b.chunk_off.as<int>() + 1,
                                          (size_t)ns, rocprim::plus<int>(), s),
                  "inclusive_scan");
        sync(s);  // before the temporaries are freed
    }
    b.nchunks = read_scalar<int>(b.chunk_off.as<int>() + ns, s);
    b.chunks.alloc((size_t)std::max<int64_t>(b.nchunks, 1) * sizeof(int4));
    hip_check(launch_sell_chunk_fill(ns, b.slice_ptr.as<int64_t>(), b.sell_len.as<int>(),
                                     b.chunk_off.as<int>(), split, head, chunk, window,
                                     b.chunks.as<int4>(), s),
              "sell chunks");
    sync(s);
}

template <typename V>
void build_sell(const spmv_handle* h, int sort_window, bool permuted, bool window, Built& b,
                hipStream_t s) {
    const int64_t n = h->n, S = pad64(n), ns = S / 64;
    b.nslices = ns;
    b.permuted = permuted;
    b.perm.alloc((size_t)std::max<int64_t>(n, 1) * 4);
    b.sell_len.alloc((size_t)S * 4);
    b.slice_ptr.alloc((size_t)(ns + 1) * 8);
    if (sort_window < 0) sort_window = window ? kSellWinSortWindow : kSellSortWindow;
    int64_t sigma = sort_window >= n ? n : sort_window;
    if (sort_window == 0) sigma = 1;  // every row its own window: row order kept
    b.sort_window = sigma <= 1 ? 0 : (int)sigma;
    if (n > 0 && sigma <= 1) {
        hipLaunchKernelGGL(k_iota, dim3(grid_for(n)), dim3(256), 0, s, n, b.perm.as<int>());
        hip_check(hipGetLastError(), "identity permutation");
    } else if (n > 0 && sigma < n) {
        // key = window << 32 | (W - length): 64-bit stable radix sort
        DevBuf keys((size_t)n * 8), keys_out((size_t)n * 8);
        hipLaunchKernelGGL(k_sell_keys_win, dim3(grid_for(n)), dim3(256), 0, s, n, sigma,
                           h->max_len, h->rowptr.as<int>(), keys.as<unsigned long long>());
        hip_check(hipGetLastError(), "sell keys");
        size_t tmp = 0;
        rocprim::counting_iterator<int> iota(0);
        const unsigned nb = 32 + bits_for((uint64_t)((n - 1) / sigma));
        hip_check(rocprim::radix_sort_pairs(nullptr, tmp, keys.as<unsigned long long>(),
                                            keys_out.as<unsigned long long>(), iota,
                                            b.perm.as<int>(), (size_t)n, 0, nb, s),
                  "radix_sort_pairs");
        DevBuf work(tmp);
        hip_check(rocprim::radix_sort_pairs(work.p, tmp, keys.as<unsigned long long>(),
                                            keys_out.as<unsigned long long>(), iota,
                                            b.perm.as<int>(), (size_t)n, 0, nb, s),
                  "radix_sort_pairs");
        sync(s);  // before the temporaries are freed
    } else if (n > 0) {
        DevBuf keys((size_t)n * 4), keys_out((size_t)n * 4);
        hipLaunchKernelGGL(k_sell_keys, dim3(grid_for(n)), dim3(256), 0, s, n, h->max_len,
                           h->rowptr.as<int>(), keys.as<unsigned>());
        hip_check(hipGetLastError(), "sell keys");
        size_t tmp = 0;
        rocprim::counting_iterator<int> iota(0);
        const unsigned nb = bits_for((uint64_t)h->max_len);
        hip_check(rocprim::radix_sort_pairs(nullptr, tmp, keys.as<unsigned>(),
                                            keys_out.as<unsigned>(), iota, b.perm.as<int>(),
                                            (size_t)n, 0, nb, s),
                  "radix_sort_pairs");
        DevBuf work(tmp);
        hip_check(rocprim::radix_sort_pairs(work.p, tmp, keys.as<unsigned>(),
                                            keys_out.as<unsigned>(), iota, b.perm.as<int>(),
                                            (size_t)n, 0, nb, s),
                  "radix_sort_pairs");
        sync(s);  // before the temporaries are freed
    }
    DevBuf slots((size_t)std::max<int64_t>(ns, 1) * 8);
    if (ns > 0) {
        hipLaunchKernelGGL(k_sell_len, dim3(grid_for(S)), dim3(256), 0, s, n, S,
                           h->rowptr.as<int>(), b.perm.as<int>(), b.sell_len.as<int>());
        hip_check(hipGetLastError(), "sell lengths");
        hipLaunchKernelGGL(k_sell_width, dim3(grid_for(ns)), dim3(256), 0, s, ns,
                           b.sell_len.as<int>(), slots.as<int64_t>());
        hip_check(hipGetLastError(), "sell widths");
        hip_check(hipMemsetAsync(b.slice_ptr.p, 0, 8, s), "hipMemsetAsync");
        size_t tmp = 0;
        hip_check(rocprim::inclusive_scan(nullptr, tmp, slots.as<int64_t>(),
                                          b.slice_ptr.as<int64_t>() + 1, (size_t)ns,
                                          rocprim::plus<int64_t>(), s),
                  "inclusive_scan");
        DevBuf work(tmp);
        hip_check(rocprim::inclusive_scan(work.p, tmp, slots.as<int64_t>(),
                                          b.slice_ptr.as<int64_t>() + 1, (size_t)ns,
                                          rocprim::plus<int64_t>(), s),
                  "inclusive_scan");
        sync(s);
    } else {
        hip_check(hipMemsetAsync(b.slice_ptr.p, 0, 8, s), "hipMemsetAsync");
    }
    b.sell_slots = read_scalar<int64_t>(b.slice_ptr.as<int64_t>() + ns, s);
    build_sell_chunks(b, window, s);
    b.sell_col.alloc((size_t)b.sell_slots * 4);
    b.sell_val.alloc((size_t)b.sell_slots * sizeof(V));
    if (ns > 0) {
        DevBuf inv;
        if (permuted) {
            inv.alloc((size_t)std::max<int64_t>(n, 1) * 4);
            hipLaunchKernelGGL(k_invert_perm, dim3(grid_for(n)), dim3(256), 0, s, n,
                               b.perm.as<int>(), inv.as<int>());
            hip_check(hipGetLastError(), "invert permutation");
        }
        hipLaunchKernelGGL(k_sell_fill<V>, dim3((unsigned)((ns + 3) / 4)), dim3(256), 0, s, n,
                           ns, h->rowptr.as<int>(), h->col.as<int>(), h->val.as<V>(),
                           b.perm.as<int>(), permuted ? inv.as<int>() : nullptr,
                           b.slice_ptr.as<int64_t>(),
                           b.sell_len.as<int>(), b.sell_col.as<int>(), b.sell_val.as<V>());
        hip_check(hipGetLastError(), "sell fill");
        sync(s);  // before the temporaries are freed
    }
    sync(s);
}

// row-length histogram -> HYB/HEC width K (ceil(n/3) rule unless requested)
// requested >= 0: that width (clamped to the longest row); -1: the
// ceil(n/3) rule; kRegularWidth: the width that holds 99 % of the rows whole
constexpr int kRegularWidth = -2;

int64_t choose_width(const spmv_handle* h, int requested, std::vector<int>& hist, hipStream_t s) {
    const int W = h->max_len;
    hist.assign((size_t)W + 1, 0);
    DevBuf dh((size_t)(W + 1) * 4);
    hip_check(hipMemsetAsync(dh.p, 0, (size_t)(W + 1) * 4, s), "hipMemsetAsync");
    if (h->n > 0) {
        hipLaunchKernelGGL(k_len_hist, dim3(std::min<unsigned>(grid_for(h->n), 2048)), dim3(256), 0,
                           s, h->n, W, h->rowptr.as<int>(), dh.as<int>());
        hip_check(hipGetLastError(), "histogram");
    }
    hip_check(hipMemcpyAsync(hist.data(), dh.p, (size_t)(W + 1) * 4, hipMemcpyDeviceToHost, s),
              "hipMemcpyAsync");
    sync(s);
    if (requested >= 0) return std::min<int64_t>(requested, W);
    if (requested == kRegularWidth) {
        // the smallest k with at most 1 % of the rows longer than k
        int64_t longer = h->n;  // rows longer than k, starting at k = -1
        for (int64_t k = 0; k <= W; ++k) {
            longer -= hist[(size_t)k];
            if (100 * longer <= h->n) return k;
        }
        return W;
    }
    const int64_t need = (h->n + 2) / 3;
    int64_t at_least = h->n;  // rows with length >= k, starting at k = 0
    int64_t K = 0;
    for (int64_t k = 1; k <= W; ++k) {
        at_least -= hist[(size_t)k - 1];
        if (at_least >= need)
            K = k;
        else
            break;
    }
    return K;
}

template <typename V>
void build_split(const spmv_handle* h, int format, int requested, int sort_window, Built& b,
                 hipStream_t s) {
    std::vector<int> hist;
    const int64_t K = choose_width(h, requested, hist, s);
    int64_t tail = 0;
    for (size_t l = (size_t)K + 1; l < hist.size(); ++l) tail += (int64_t)hist[l] * ((int64_t)l - K);
    int sigma = sort_window;
    if (sigma < 0) sigma = ell_pad_fraction(h, K, s) > kSortPadShare ? kEllBlock : 0;
    build_ell_part<V>(h, K, kEllBlock, sigma, b, s);
    b.tail_nnz = tail;
    const int64_t n = h->n;
    b.tail_ptr.alloc((size_t)(n + 1) * 4);
    {
        DevBuf tlen((size_t)std::max<int64_t>(n, 1) * 4);
        hip_check(hipMemsetAsync(b.tail_ptr.p, 0, 4, s), "hipMemsetAsync");
        if (n > 0) {
            hipLaunchKernelGGL(k_tail_len, dim3(grid_for(n)), dim3(256), 0, s, n, (int)K,
                               h->rowptr.as<int>(), tlen.as<int>());
            hip_check(hipGetLastError(), "tail lengths");
            size_t tmp = 0;
            hip_check(rocprim::inclusive_scan(nullptr, tmp, tlen.as<int>(), b.tail_ptr.as<int>() + 1,
                                              (size_t)n, rocprim::plus<int>(), s),
                      "inclusive_scan");
            DevBuf work(tmp);
            hip_check(rocprim::inclusive_scan(work.p, tmp, tlen.as<int>(), b.tail_ptr.as<int>() + 1,
                                              (size_t)n, rocprim::plus<int>(), s),
                      "inclusive_scan");
            sync(s);
        }
        sync(s);
    }
    if (format == SPMV_HYB) b.tail_row.alloc((size_t)std::max<int64_t>(tail, 1) * 4);
    // 16 zero bytes past the end: the vector kernel's whole 16-byte loads
    b.tail_col.alloc((size_t)tail * 4 + 16);
    b.tail_val.alloc((size_t)tail * sizeof(V) + 16);
    hip_check(hipMemsetAsync((char*)b.tail_col.p + (size_t)tail * 4, 0, 16, s), "hipMemsetAsync");
    hip_check(hipMemsetAsync((char*)b.tail_val.p + (size_t)tail * sizeof(V), 0, 16, s),
              "hipMemsetAsync");
    if (tail > 0) {
        hipLaunchKernelGGL(k_tail_fill<V>, dim3(grid_for(n, 4)), dim3(256), 0, s, n,
                           (int)K, h->rowptr.as<int>(), h->col.as<int>(), h->val.as<V>(),
                           b.tail_ptr.as<int>(), format == SPMV_HYB ? b.tail_row.as<int>() : nullptr,
                           b.tail_col.as<int>(), b.tail_val.as<V>());
        hip_check(hipGetLastError(), "tail fill");
    }
    b.tail_runs = (tail + kTailPerLane - 1) / kTailPerLane;
    if (format == SPMV_HEC) {
        // compress the tail pointer to the rows that have tail entries, so a
        // lane run of 8 entries crosses at most 8 (compressed) rows
        b.tail_nrows = 0;
        if (tail > 0) {
            DevBuf flag((size_t)n * 4), pos((size_t)n * 4);
            hipLaunchKernelGGL(k_tail_flags, dim3(grid_for(n)), dim3(256), 0, s, n,
                               b.tail_ptr.as<int>(), flag.as<int>());
            hip_check(hipGetLastError(), "tail flags");
            size_t tmp = 0;
            hip_check(rocprim::exclusive_scan(nullptr, tmp, flag.as<int>(), pos.as<int>(), 0,
                                              (size_t)n, rocprim::plus<int>(), s),
                      "exclusive_scan");
            DevBuf work(tmp);
            hip_check(rocprim::exclusive_scan(work.p, tmp, flag.as<int>(), pos.as<int>(), 0,
                                              (size_t)n, rocprim::plus<int>(), s),
                      "exclusive_scan");
            const int last_pos = read_scalar<int>(pos.as<int>() + (n - 1), s);
            const int last_flag = read_scalar<int>(flag.as<int>() + (n - 1), s);
            b.tail_nrows = (int64_t)last_pos + last_flag;
            b.tail_rows.alloc((size_t)b.tail_nrows * 4);
            b.tail_cptr.alloc((size_t)(b.tail_nrows + 1) * 4);
            hipLaunchKernelGGL(k_compact_rows, dim3(grid_for(n)), dim3(256), 0, s, n,
                               b.tail_ptr.as<int>(), pos.as<int>(), b.tail_rows.as<int>(),
                               b.tail_cptr.as<int>());
            hip_check(hipGetLastError(), "compact rows");
            const int tail_end = (int)tail;
            hip_check(hipMemcpyAsync(b.tail_cptr.as<int>() + b.tail_nrows, &tail_end, 4,
                                     hipMemcpyHostToDevice, s),
                      "hipMemcpyAsync");
            b.run_row.alloc((size_t)(b.tail_runs + 1) * 4);
            hipLaunchKernelGGL(k_run_rows, dim3(grid_for(b.tail_nrows)), dim3(256), 0, s,
                               b.tail_nrows, b.tail_runs, b.tail_cptr.as<int>(),
                               b.run_row.as<int>());
            hip_check(hipGetLastError(), "run rows");
            sync(s);  // before the temporaries are freed
        }
    }
    // (HYB keeps tail_ptr until its tail kernel is chosen: the column-slice
    // copy is built from the tail's CSR)
    sync(s);
}

void decide_window(const spmv_handle* h, int format, int opt, Built& b, hipStream_t s);

// wave groups per 64-row tile of the ELL kernel (without the LDS window):
// several groups only when the matrix has too few tiles to fill the GPU and
// rows long enough to share
void choose_groups(const spmv_handle* h, int opt, Built& b) {
    if (b.window) {
        b.ell_groups = 1;
        return;
    }
    if (opt > 0) {
        b.ell_groups = opt;
        return;
    }
    const int64_t tiles = (h->n + 63) / 64;  // one wave of 64 rows each
    const int64_t W = b.ell_width;
    b.ell_groups = tiles >= kEllGroupTiles               ? 1
                   : tiles < kEllGroupTiles / 4 && W >= 256 ? 16
                   : W >= 16                                ? 4
                                                            : 1;
}

// launch the kernels of one apply of `format` built in `b`
hipError_t launch_built(const spmv_handle* h, const Built& b, int format, void* y, const void* x,
                        double alpha, double beta, hipStream_t s) {
    const bool f64 = h->dtype == SPMV_F64;
    hipError_t e = hipSuccess;
    switch (format) {
        case SPMV_CSR: {
            if (b.csr_xblock) {
                e = launch_xblk(b.xb, f64, y, x, alpha, beta, s);
                break;
            }
            if (b.csr_balanced) {
                TailView t{(int)h->n, h->nnz, nullptr, h->rowptr.as<int>(), b.run_row.as<int>(),
                           nullptr, h->col.as<int>(), h->val.p, b.window};
                e = launch_scale(h->n, f64, y, beta, s);
                if (e == hipSuccess) e = launch_tail(t, f64, y, x, alpha, s);
                break;
            }
            CsrView a{(int)h->n, (int)h->nnz, h->rowptr.as<int>(), h->col.as<int>(), h->val.p};
            e = launch_csr(a, h->subwave, h->csr_rows, h->csr_stage_slots, h->csr_stage_col_nt,
                           f64, y, x, alpha, beta, s);
            break;
        }
        case SPMV_ELLR:
        case SPMV_HYB:
        case SPMV_HEC: {
            EllView a{(int)h->n, std::max<int64_t>(b.ell_bh, 1), b.ell_width * b.ell_bh,
                      (int)b.ell_width, b.ell_len.as<int>(), b.ell_perm.as<int>(),
                      b.ell_col.as<int>(), b.ell_records ? nullptr : b.ell_val.p, b.ell_records,
                      b.window, b.ell_groups, b.col_nt};
            if (b.window) a.head = b.ell_head;
            e = launch_ell(a, f64, y, x, alpha, beta, s);
            if (e == hipSuccess && b.window && b.ell_nlong > 0)
                e = launch_ell_long(a, b.ell_long.as<int>(), b.ell_nlong, f64, y, x, alpha, s);
            if (e == hipSuccess && format != SPMV_ELLR && b.tail_nnz > 0 && b.tail_xblock) {
                e = launch_xblk(b.xb, f64, y, x, alpha, 1.0, s);  // adds alpha A_tail x
            } else if (e == hipSuccess && format == SPMV_HEC && b.tail_nnz > 0 && b.tail_vector) {
                const CsrView t{(int)b.tail_nrows, (int)b.tail_nnz, b.tail_cptr.as<int>(),
                                b.tail_col.as<int>(), b.tail_val.p, b.tail_rows.as<int>()};
                const VecShape& v = b.tail_vec;
                e = launch_csr(t, v.subwave, v.rows, v.slots, v.col_nt, f64, y, x, alpha, 1.0, s);
            } else if (e == hipSuccess && format != SPMV_ELLR && b.tail_nnz > 0) {
                const bool hec = format == SPMV_HEC;
                TailView t{(int)h->n, b.tail_nnz, hec ? nullptr : b.tail_row.as<int>(),
                           hec ? b.tail_cptr.as<int>() : nullptr, b.run_row.as<int>(),
                           hec ? b.tail_rows.as<int>() : nullptr, b.tail_col.as<int>(),
                           b.tail_val.p, b.window};
                e = launch_tail(t, f64, y, x, alpha, s);
            }
            break;
        }
        case SPMV_SELL64: {
            SellView a{(int)h->n, (int)b.nslices, b.slice_ptr.as<int64_t>(), b.sell_len.as<int>(),
                       b.perm.as<int>(), b.sell_col.as<int>(), b.sell_val.p, (int)b.nchunks,
                       b.chunks.as<int4>(), b.chunk_off.as<int>(), b.permuted, b.col_nt,
                       b.window};
            e = launch_sell(a, f64, y, x, alpha, beta, s);
            break;
        }
    }
    return e;
}

// Timings at conversion read a buffer twice the size of the Infinity Cache
// (256 MB) through the caches before each timed launch, so that the launch
// meets the caches as an apply does when other work runs between applies (a
// solver's vector updates, other matrices): matrix and x not left there.
// Timed back to back instead, a matrix whose index array fits the cache
// beside x looks faster than it is in use.  The buffer is held for one
// spmv_convert call (FlushScope); without room for it the launches are timed
// back to back.
constexpr size_t kFlushBytes = size_t(512) << 20;

struct FlushScope;
thread_local FlushScope* t_flush = nullptr;

// allocated at the first timed launch of the convert call (conversions with
// every choice given time nothing and allocate nothing)
struct FlushScope {
    DevBuf buf;
    bool tried = false;
    FlushScope* prev;
    FlushScope() : prev(t_flush) { t_flush = this; }
    ~FlushScope() { t_flush = prev; }
    FlushScope(const FlushScope&) = delete;
    FlushScope& operator=(const FlushScope&) = delete;
    const DevBuf* get() {
        if (!tried) {
            tried = true;
            void* q = nullptr;
            if (hipMalloc(&q, kFlushBytes) == hipSuccess)
                buf.p = q, buf.bytes = kFlushBytes;
            else
                (void)hipGetLastError();
        }
        return buf.p ? &buf : nullptr;
    }
};

__device__ int g_flush_sink;

// read p[0, n16) through the caches (plain loads); the data only feeds a
// value stored when it equals a constant, so the loads stay
__global__ __launch_bounds__(256) void k_flush(const int4* __restrict__ p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const int4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x5a5a5a5a) g_flush_sink = acc;
}

hipError_t flush_caches(hipStream_t s) {
    const DevBuf* f = t_flush ? t_flush->get() : nullptr;
    if (!f) return hipSuccess;
    hipLaunchKernelGGL(k_flush, dim3(8192), dim3(256), 0, s, f->as<int4>(), (int64_t)(f->bytes / 16));
    return hipGetLastError();
}

// device time of `launch` (ms): one warm-up call, then the fastest of three
// timed calls, each after a cache flush (only the launch itself is timed)
template <typename F>
float time_launches(F&& launch, hipStream_t s) {
    constexpr int kReps = 3;
    hipEvent_t ev[2 * kReps];
    for (auto& e : ev) hip_check(hipEventCreate(&e), "hipEventCreate");
    hipError_t err = launch();
    for (int r = 0; r < kReps && err == hipSuccess; ++r) {
        err = flush_caches(s);
        if (err == hipSuccess) err = hipEventRecord(ev[2 * r], s);
        if (err == hipSuccess) err = launch();
        if (err == hipSuccess) err = hipEventRecord(ev[2 * r + 1], s);
    }
    if (err == hipSuccess) err = hipEventSynchronize(ev[2 * kReps - 1]);
    float ms = 1e30f;
    for (int r = 0; r < kReps && err == hipSuccess; ++r) {
        float t = 0;
        err = hipEventElapsedTime(&t, ev[2 * r], ev[2 * r + 1]);
        ms = std::min(ms, t);
    }
    for (auto& e : ev) (void)hipEventDestroy(e);
    hip_check(err, "kernel timing");
    return ms;
}



// LDS slots per wave of the staged CSR kernel with `sw` lanes per row: the
// fewest multiples of 64 that hold the entries of 99.5 % of the waves (one
// outlier wave would otherwise set the LDS of all and lower the occupancy;
// waves that do not fit read directly), at least 256, at most what four
// slices per workgroup allow.
int stage_slots_for(const CsrView& v, bool f64, int sw, hipStream_t s) {
    const int max_slots = csr_stage_max_slots(f64);
    const int rw = 64 / sw, nb = max_slots / 64 + 1;
    const int64_t waves = ((int64_t)v.n + rw - 1) / rw;
    if (waves == 0) return 256;
    DevBuf hist((size_t)nb * 4);
    hip_check(hipMemsetAsync(hist.p, 0, hist.bytes, s), "hipMemsetAsync");
    hipLaunchKernelGGL(k_stage_hist, dim3(grid_for(waves)), dim3(256), 0, s, (int64_t)v.n, rw,
                       v.rowptr, nb, hist.as<unsigned>());
    hip_check(hipGetLastError(), "stage histogram");
    std::vector<unsigned> c(nb);
    hip_check(hipMemcpyAsync(c.data(), hist.p, hist.bytes, hipMemcpyDeviceToHost, s),
              "hipMemcpyAsync");
    sync(s);
    int64_t cum = 0;
    int slots = max_slots;
    for (int b = 0; b < nb - 1; ++b) {
        cum += c[b];
        if ((double)cum >= 0.995 * (double)waves) {
            slots = (b + 1) * 64;
            break;
        }
    }
    return std::min(std::max(slots, 256), max_slots);
}

// Time the shapes of the vector CSR kernel on `v` (lanes per row from sw_lo
// to sw_hi, rows per lane group, direct or staged through LDS; a value >= 0
// or > 0 in rows / stage fixes that choice) with x = 0 and the result added
// to ys with `beta`, and return the fastest and its time.  The staged copy
// streams val past the caches; col too only when that is faster (a col array
// that fits the last-level cache beside x stays there over repeated applies).
float tune_vector(const CsrView& v, bool f64, int64_t max_len, int sw_lo, int sw_hi, int fix_rows,
                  int fix_stage, int col_cache, void* ys, const void* xs, double beta,
                  VecShape& best, hipStream_t s) {
    float best_ms = 1e30f;
    const bool col_nt = col_cache != 1;  // the staged copy streams col unless asked
    // a group that would loop more than kVecMaxPasses times over the longest
    // row serialises the launch on it: such shapes are not timed (the widest
    // one in range always is)
    const int cap = fix_stage == 1 ? std::min(sw_hi, kCsrStageMax) : sw_hi;
    while (sw_lo < cap && (max_len + sw_lo - 1) / sw_lo > kVecMaxPasses) sw_lo <<= 1;
    for (int sw = sw_lo; sw <= sw_hi; sw <<= 1)
        for (int rows = 1; rows <= kCsrRowsMax; rows <<= 1)
            for (int st = 0; st <= 1; ++st) {
                if (fix_rows && rows != fix_rows) continue;
                if (fix_stage >= 0 && st != fix_stage) continue;
                if (st && (rows != 1 || sw < kCsrStageMin || sw > kCsrStageMax)) continue;
                const int slots = st ? stage_slots_for(v, f64, sw, s) : 0;
                const float ms = time_launches([&] {
                    return launch_csr(v, sw, rows, slots, col_nt, f64, ys, xs, 1.0, beta, s);
                }, s);
                if (ms < best_ms) best_ms = ms, best = VecShape{sw, rows, slots, col_nt};
            }
    return best_ms;
}

// CSR kernel: time every shape of the vector kernel and the entry-balanced
// kernel on the device and keep the fastest (the apply does not depend on
// the values of x, so zeros are used).  Fixed values are not tuned.
// CSR by column slices (SPMV_CSR_XBLOCK): row ranges of about equal entry
// counts (at most kXbCap rows, one pass of kXbGroups workgroups when the
// rows allow), the entry counts of every row in every slice at their
// xblk_slot positions, their scan (every entry's place), the tile starts and
// the entries in tile order with their row offsets.
// a CSR matrix on the device: the handle's, or the tail of a HEC handle
struct CsrSrc {
    int64_t n, nnz;
    const int* rowptr;
    const int* col;
    const void* val;
};
CsrSrc csr_src(const spmv_handle* h) {
    return CsrSrc{h->n, h->nnz, h->rowptr.as<int>(), h->col.as<int>(), h->val.p};
}
double entries_within(const CsrSrc& a, int64_t lead, hipStream_t s);

// The column-slice copy of a CSR matrix `a` (the handle's own, or a HEC
// tail) in b.xb and its buffers; the values have the handle's dtype.
void build_xblock(const spmv_handle* h, const CsrSrc& a, Built& b, hipStream_t s) {
    const int64_t n = a.n, nnz = a.nnz;
    if ((int64_t)kXbTiles * n > (int64_t)INT32_MAX - 16)
        fail(SPMV_ERR_INVALID_ARG, "csr_kernel 3 (column slices) takes n <= %lld rows (got %lld)",
             (long long)(((int64_t)INT32_MAX - 16) / kXbTiles), (long long)n);
    XblkView& v = b.xb;
    v = XblkView{};
    v.n = n;
    v.width = std::max<int64_t>((n + kXbBlocks - 1) / kXbBlocks, 1);
    if (n == 0) return;
    const int cap = h->dtype == SPMV_F64 ? kXbCap<double> : kXbCap<float>;
    // a range's band tile: columns within `band` of its rows, packed with
    // the row offsets (band + cap + band columns fit the column bits); none
    // (band -1) unless most entries lie that close to their row
    v.lbits = h->dtype == SPMV_F64 ? kXbRowBits<double> : kXbRowBits<float>;
    v.band = xblk_band(v.lbits, cap);
    if (entries_within(a, v.band, s) < 0.5) v.band = -1;
    const int64_t passes = std::max<int64_t>(1, (n + (int64_t)kXbGroups * cap - 1) /
                                                    ((int64_t)kXbGroups * cap));
    const int64_t R0 = passes * kXbGroups;
    std::vector<int> cand((size_t)R0 + 1);
    {
        DevBuf dc(cand.size() * 4);
        hip_check(launch_xblk_bounds(n, nnz, a.rowptr, R0, dc.as<int>(), s),
                  "column-slice range bounds");
        hip_check(hipMemcpyAsync(cand.data(), dc.p, dc.bytes, hipMemcpyDeviceToHost, s),
                  "hipMemcpyAsync");
        sync(s);
    }
    v.ranges = xblk_split_ranges(cand.data(), R0, cap, nullptr);
    std::vector<int> rows((size_t)v.ranges + 1);
    xblk_split_ranges(cand.data(), R0, cap, rows.data());
    b.xb_rows.alloc(rows.size() * 4);
    hip_check(hipMemcpyAsync(b.xb_rows.p, rows.data(), rows.size() * 4, hipMemcpyHostToDevice, s),
              "hipMemcpyAsync");
    v.row_begin = b.xb_rows.as<int>();
    const int64_t slots = (int64_t)kXbTiles * n;
    DevBuf pos((size_t)(slots + 1) * 4);
    {
        DevBuf cnt((size_t)slots * 4);
        hip_check(launch_xblk_count(v, a.rowptr, a.col, cnt.as<int>(), s),
                  "column-slice counts");
        hip_check(hipMemsetAsync(pos.p, 0, 4, s), "hipMemsetAsync");
        size_t tmp = 0;
        hip_check(rocprim::inclusive_scan(nullptr, tmp, cnt.as<int>(), pos.as<int>() + 1,
                                          (size_t)slots, rocprim::plus<int>(), s),
                  "inclusive_scan");
        DevBuf work(tmp);
        hip_check(rocprim::inclusive_scan(work.p, tmp, cnt.as<int>(), pos.as<int>() + 1,
                                          (size_t)slots, rocprim::plus<int>(), s),
                  "inclusive_scan");
        sync(s);
    }
    const int64_t ntiles = v.ranges * kXbTiles;
    b.xb_tiles.alloc((size_t)(ntiles + 1) * 4);
    hip_check(launch_xblk_tiles(v, pos.as<int>(), b.xb_tiles.as<int>(), s), "column-slice tiles");
    hip_check(hipMemcpyAsync(b.xb_tiles.as<int>() + ntiles, pos.as<int>() + slots, 4,
                             hipMemcpyDeviceToDevice, s),
              "hipMemcpyAsync");
    v.tile_ptr = b.xb_tiles.as<int>();
    b.xb_col.alloc((size_t)std::max<int64_t>(nnz, 1) * 4);
    b.xb_val.alloc((size_t)std::max<int64_t>(nnz, 1) * h->vsize);
    b.xb_lrow.alloc((size_t)std::max<int64_t>(nnz, 1) * 2);
    hip_check(launch_xblk_fill(v, h->dtype == SPMV_F64, a.rowptr, a.col, a.val, pos.as<int>(),
                               b.xb_col.as<int>(), b.xb_val.p,
                               b.xb_lrow.as<uint16_t>(), s),
              "column-slice fill");
    if (nnz > 0) {
        // every tile's entries in column order (a stable sort keeps a row's
        // equal columns in their order): the workgroups of an XCD then sweep
        // their slice of x together, so each x line is read from that XCD's
        // L2 by all of them within a short time
        DevBuf kcol((size_t)nnz * 4), idx((size_t)nnz * 4), src((size_t)nnz * 4);
        hipLaunchKernelGGL(k_iota, dim3(grid_for(nnz)), dim3(256), 0, s, nnz, idx.as<int>());
        hip_check(hipGetLastError(), "column-slice sort");
        const unsigned bits = 32;  // band tiles hold packed words
        size_t tmp = 0;
        hip_check(rocprim::segmented_radix_sort_pairs(
                      nullptr, tmp, b.xb_col.as<unsigned>(), kcol.as<unsigned>(), idx.as<int>(),
                      src.as<int>(), (unsigned)nnz, (unsigned)ntiles, b.xb_tiles.as<int>(),
                      b.xb_tiles.as<int>() + 1, 0, bits, s),
                  "segmented_radix_sort_pairs");
        {
            DevBuf work(tmp);
            hip_check(rocprim::segmented_radix_sort_pairs(
                          work.p, tmp, b.xb_col.as<unsigned>(), kcol.as<unsigned>(),
                          idx.as<int>(), src.as<int>(), (unsigned)nnz, (unsigned)ntiles,
                          b.xb_tiles.as<int>(), b.xb_tiles.as<int>() + 1, 0, bits, s),
                      "segmented_radix_sort_pairs");
            sync(s);
        }
        idx.release();
        DevBuf oval((size_t)nnz * h->vsize), olrow((size_t)nnz * 2);
        hip_check(launch_xblk_gather(nnz, h->dtype == SPMV_F64, src.as<int>(), b.xb_val.p,
                                     b.xb_lrow.as<uint16_t>(), oval.p, olrow.as<uint16_t>(), s),
                  "column-slice sort");
        sync(s);
        b.xb_col = std::move(kcol);
        b.xb_val = std::move(oval);
        b.xb_lrow = std::move(olrow);
    }
    v.col = b.xb_col.as<int>();
    v.val = b.xb_val.p;
    v.lrow = b.xb_lrow.as<uint16_t>();
    sync(s);
}

void tune_csr(spmv_handle* h, const spmv_convert_opts& o, Built& b, hipStream_t s) {
    if (o.csr_kernel == SPMV_CSR_XBLOCK) {
        h->subwave = 1, h->csr_rows = 1, h->csr_stage_slots = 0, h->csr_stage_col_nt = false;
        build_xblock(h, csr_src(h), b, s);
        b.csr_xblock = true;
        return;
    }
    int rule = 1;  // smallest power of two >= the longest row, at most 64
    while (rule < 64 && rule < h->max_len) rule <<= 1;
    if (o.csr_stage == 1) rule = std::min(std::max(rule, kCsrStageMin), kCsrStageMax);
    h->subwave = o.subwave ? o.subwave : rule;
    h->csr_rows = o.csr_rows ? o.csr_rows : 1;
    h->csr_stage_slots = 0;
    h->csr_stage_col_nt = o.col_cache != 1;
    const bool f64 = h->dtype == SPMV_F64;
    const CsrView v{(int)h->n, (int)h->nnz, h->rowptr.as<int>(), h->col.as<int>(), h->val.p};
    const bool want_vec = o.csr_kernel != SPMV_CSR_BALANCED;
    const bool want_bal = o.csr_kernel != SPMV_CSR_VECTOR && h->nnz > 0;
    b.csr_balanced = !want_vec;
    if (want_bal) {
        // row of the first entry of every lane run, over the whole matrix
        b.tail_runs = (h->nnz + kTailPerLane - 1) / kTailPerLane;
        b.run_row.alloc((size_t)(b.tail_runs + 1) * 4);
        hipLaunchKernelGGL(k_run_rows, dim3(grid_for(h->n)), dim3(256), 0, s, h->n, b.tail_runs,
                           h->rowptr.as<int>(), b.run_row.as<int>());
        hip_check(hipGetLastError(), "run rows");
        const bool bal = b.csr_balanced;
        b.csr_balanced = true;  // the window is timed on the balanced kernel
        decide_window(h, SPMV_CSR, o.x_window, b, s);
        b.csr_balanced = bal;
    }
    const bool tune_vec = want_vec && !(o.subwave && o.csr_rows && o.csr_stage >= 0);
    if (o.csr_stage == 1) h->csr_stage_slots = stage_slots_for(v, f64, h->subwave, s);
    if (h->n == 0 || h->nnz == 0 || (!tune_vec && !(want_vec && want_bal))) {
        sync(s);
        return;
    }
    DevBuf xs((size_t)h->n * h->vsize), ys((size_t)h->n * h->vsize);
    hip_check(hipMemsetAsync(xs.p, 0, xs.bytes, s), "hipMemsetAsync");
    float best_ms = 1e30f;
    if (want_vec) {
        VecShape best;
        best_ms = tune_vector(v, f64, h->max_len, o.subwave ? o.subwave : (h->max_len <= 2 ? 1 : 2),
                              o.subwave ? o.subwave : 64, o.csr_rows, o.csr_stage, o.col_cache, ys.p,
                              xs.p, 0.0, best, s);
        h->subwave = best.subwave, h->csr_rows = best.rows;
        h->csr_stage_slots = best.slots, h->csr_stage_col_nt = best.col_nt;
    }
    if (want_vec && want_bal) {
        b.csr_balanced = true;
        const float ms = time_launches(
            [&] { return launch_built(h, b, SPMV_CSR, ys.p, xs.p, 1.0, 0.0, s); }, s);
        // the vector kernel adds no atomics (bit-reproducible results): the
        // balanced one must be clearly faster to be kept
        b.csr_balanced = ms < kPreferMargin * best_ms;
        if (b.csr_balanced) best_ms = ms;
    }
    if (!b.csr_balanced) b.run_row.release(), b.window = false, b.tail_runs = 0;
    // third candidate: column slices, for an x larger than one XCD's L2,
    // when its copy of the entries fits the budget
    const double xb_bytes = (double)h->nnz * (6.0 + (double)h->vsize) +  // entries, row offsets
                            (double)kXbTiles * (double)h->n * 8.0;          // counts and their scan
    if (o.csr_kernel == SPMV_CSR_AUTO && want_bal &&
        (double)h->n * (double)h->vsize > (double)kXbMinX &&
        (int64_t)kXbTiles * h->n <= (int64_t)INT32_MAX - 16 &&
        xb_bytes <= (double)budget_bytes(o)) {
        Built xb;
        bool built = true;
        try {
            build_xblock(h, csr_src(h), xb, s);
            xb.csr_xblock = true;
        } catch (const Error& e) {
            if (e.code != SPMV_ERR_NO_MEMORY) throw;
            built = false;  // no room for the optional copy: not a candidate
        }
        if (built) {
            const float ms = time_launches(
                [&] { return launch_built(h, xb, SPMV_CSR, ys.p, xs.p, 1.0, 0.0, s); }, s);
            if (ms < kPreferMargin * best_ms) {
                xb.band_fraction = b.band_fraction;
                b = std::move(xb);
            }
        }
    }
    sync(s);
}

// Tail kernel of HYB / HEC: the balanced kernel (atomics; COO for HYB, CSR
// for HEC), for HEC the vector CSR kernel over the rows that hold tail
// entries (each row added once onto the ELL part's result: no atomics,
// bit-reproducible), or for both the column-slice kernel over the tail's
// rows (a copy of the tail by column slices).  `kernel` (a spmv_csr_kernel)
// fixes the choice; SPMV_CSR_AUTO keeps the faster on the device, the
// balanced one only when clearly faster, keeps the balanced one with the LDS
// window (the vector kernel has no window), and then times the column slices
// like the CSR format.
void tune_tail(const spmv_handle* h, int format, int kernel, int col_cache, uint64_t budget,
               Built& b, hipStream_t s) {
    b.tail_vector = false;
    b.tail_xblock = false;
    const bool hyb = format == SPMV_HYB;
    if (b.tail_nnz == 0) {
        if (hyb) b.tail_ptr.release();
        return;
    }
    const CsrSrc tail{h->n, b.tail_nnz, b.tail_ptr.as<int>(), b.tail_col.as<int>(), b.tail_val.p};
    if (kernel == SPMV_CSR_XBLOCK) {
        build_xblock(h, tail, b, s);
        b.tail_xblock = true;
        b.run_row.release();
        if (hyb) b.tail_ptr.release();
        return;
    }
    const bool f64 = h->dtype == SPMV_F64;
    DevBuf xs((size_t)h->n * h->vsize), ys((size_t)h->n * h->vsize);
    hip_check(hipMemsetAsync(xs.p, 0, xs.bytes, s), "hipMemsetAsync");
    hip_check(hipMemsetAsync(ys.p, 0, ys.bytes, s), "hipMemsetAsync");
    if (!hyb && kernel != SPMV_CSR_BALANCED && !(kernel == SPMV_CSR_AUTO && b.window)) {
        const TailView t{(int)h->n, b.tail_nnz, nullptr, b.tail_cptr.as<int>(),
                         b.run_row.as<int>(), b.tail_rows.as<int>(), b.tail_col.as<int>(),
                         b.tail_val.p, false};
        const float bal_ms =
            kernel == SPMV_CSR_VECTOR
                ? 1e30f
                : time_launches([&] { return launch_tail(t, f64, ys.p, xs.p, 1.0, s); }, s);
        const CsrView v{(int)b.tail_nrows, (int)b.tail_nnz, b.tail_cptr.as<int>(),
                        b.tail_col.as<int>(), b.tail_val.p, b.tail_rows.as<int>()};
        VecShape best;
        const float vec_ms = tune_vector(v, f64, h->max_len - b.ell_width, 1, 64, 0, -1, col_cache,
                                         ys.p, xs.p, 1.0, best, s);
        sync(s);
        if (!(bal_ms < kPreferMargin * vec_ms)) {
            b.tail_vector = true;
            b.tail_vec = best;
        }
    }
    // third candidate: the tail by column slices, for an x larger than one
    // XCD's L2 when its copy fits the budget; kept only when the whole apply
    // is clearly faster with it
    const double xb_bytes = (double)b.tail_nnz * (6.0 + (double)h->vsize) +
                            (double)kXbTiles * (double)h->n * 8.0;
    if (kernel == SPMV_CSR_AUTO && (double)h->n * (double)h->vsize > (double)kXbMinX &&
        (int64_t)kXbTiles * h->n <= (int64_t)INT32_MAX - 16 && xb_bytes <= (double)budget) {
        auto run = [&] { return launch_built(h, b, format, ys.p, xs.p, 1.0, 0.0, s); };
        const float cur_ms = time_launches(run, s);
        bool built = true;
        try {
            build_xblock(h, tail, b, s);
        } catch (const Error& e) {
            if (e.code != SPMV_ERR_NO_MEMORY) throw;
            built = false;  // no room for the optional copy: not a candidate
            b.release_xblock();  // nor for what was built of it
        }
        if (built) {
            b.tail_xblock = true;
            const float xb_ms = time_launches(run, s);
            if (!(xb_ms < kPreferMargin * cur_ms)) {
                b.tail_xblock = false;
                b.release_xblock();
            }
        }
    }
    if (b.tail_xblock) b.tail_vector = false;
    if (b.tail_vector || b.tail_xblock) b.run_row.release();
    if (hyb) b.tail_ptr.release();  // HYB keeps the COO rows (and the copy)
}

// Share of the entries the LDS window reaches, and whether to use it.  On
// its own the window is only a candidate when at least half of the entries
// lie within its reach (and, for ELL-R, rows are at most 128 long); the
// apply is then timed with and without it and the faster kept (stencils
// whose x reads already coalesce gain nothing from it).  `b` must hold the
// built format.
// share of the entries of a CSR matrix whose column lies within `lead` of
// their row
double entries_within(const CsrSrc& a, int64_t lead, hipStream_t s) {
    DevBuf cnt(8);
    hip_check(hipMemsetAsync(cnt.p, 0, 8, s), "hipMemsetAsync");
    if (a.n > 0) {
        hipLaunchKernelGGL(k_band_count, dim3(grid_for(a.n)), dim3(256), 0, s, a.n, lead, a.rowptr,
                           a.col, cnt.as<unsigned long long>());
        hip_check(hipGetLastError(), "band count");
    }
    const unsigned long long c = read_scalar<unsigned long long>(cnt.p, s);
    return a.nnz ? (double)c / (double)a.nnz : 0.0;
}

// share of the entries whose column lies within the window's reach of their row
double band_fraction(const spmv_handle* h, hipStream_t s) {
    return entries_within(csr_src(h), h->dtype == SPMV_F64 ? EllWinLead<double>::value
                                                           : EllWinLead<float>::value, s);
}

// window offsets are computed in 32 bits: rows and columns plus the window
// length must stay below 2^31
bool window_fits(const spmv_handle* h) {
    return h->n < INT32_MAX - 2 * (int64_t)WinLen<float>::value;
}

// ELLPACK-R rows longer than kEllWinHeadMax are not run whole by the window
// kernel (one lane per row): it takes every row's first `head` slots -- the
// width that holds 99 % of the rows whole, a multiple of 8 up to
// kEllWinHeadMax -- and a wave per longer row takes the rest
constexpr int kEllWinHeadMax = 128;

__global__ void k_long_flags(int64_t n, const int* __restrict__ len, int head,
                             unsigned char* __restrict__ flag) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        flag[i] = len[i] > head ? 1 : 0;
}

void ell_window_split(const spmv_handle* h, Built& b, hipStream_t s) {
    b.ell_long.release();
    b.ell_nlong = 0;
    b.ell_head = 0x7fffffff;
    if (h->max_len <= kEllWinHeadMax || h->n == 0) return;
    std::vector<int> hist;
    const int64_t k = choose_width(h, kRegularWidth, hist, s);
    b.ell_head = (int)std::min<int64_t>(std::max<int64_t>((k + 7) / 8 * 8, 8), kEllWinHeadMax);
    DevBuf flag((size_t)h->n), cnt(8), rows((size_t)h->n * 4);
    hipLaunchKernelGGL(k_long_flags, dim3(grid_for(h->n)), dim3(256), 0, s, h->n,
                       b.ell_len.as<int>(), b.ell_head, flag.as<unsigned char>());
    hip_check(hipGetLastError(), "long rows");
    rocprim::counting_iterator<int> iota(0);
    size_t tmp = 0;
    hip_check(rocprim::select(nullptr, tmp, iota, flag.as<unsigned char>(), rows.as<int>(),
                              cnt.as<int64_t>(), (size_t)h->n, s),
              "select");
    DevBuf work(tmp);
    hip_check(rocprim::select(work.p, tmp, iota, flag.as<unsigned char>(), rows.as<int>(),
                              cnt.as<int64_t>(), (size_t)h->n, s),
              "select");
    b.ell_nlong = read_scalar<int64_t>(cnt.as<int64_t>(), s);
    b.ell_long.alloc((size_t)std::max<int64_t>(b.ell_nlong, 1) * 4);
    hip_check(hipMemcpyAsync(b.ell_long.p, rows.p, (size_t)b.ell_nlong * 4,
                             hipMemcpyDeviceToDevice, s),
              "hipMemcpyAsync");
    sync(s);
}

void decide_window(const spmv_handle* h, int format, int opt, Built& b, hipStream_t s) {
    b.band_fraction = band_fraction(h, s);
    const bool fits = window_fits(h);
    const bool split = format == SPMV_ELLR;  // ELLPACK-R: long rows past a head
    if (opt >= 0) {
        b.window = opt == 1 && fits;
        if (b.window && split) ell_window_split(h, b, s);
        return;
    }
    b.window = fits && h->nnz > 0 && b.band_fraction >= 0.5;
    if (!b.window) return;
    if (split) ell_window_split(h, b, s);
    DevBuf xs((size_t)h->n * h->vsize), ys((size_t)h->n * h->vsize);
    hip_check(hipMemsetAsync(xs.p, 0, xs.bytes, s), "hipMemsetAsync");
    auto run = [&] { return launch_built(h, b, format, ys.p, xs.p, 1.0, 0.0, s); };
    const float with = time_launches(run, s);
    b.window = false;
    const float without = time_launches(run, s);
    b.window = with < kPreferMargin * without;
    if (!b.window) b.ell_long.release(), b.ell_nlong = 0, b.ell_head = 0x7fffffff;
}

int run_guarded(const std::function<void()>& body) {
    try {
        body();
        return SPMV_OK;
    } catch (const Error& e) {
        g_err = e.msg;
        return e.code;
    } catch (const std::bad_alloc&) {
        g_err = "host allocation failed";
        return SPMV_ERR_NO_MEMORY;
    } catch (...) {
        g_err = "unexpected internal error";
        return SPMV_ERR_HIP;
    }
}

bool valid_format(int f) { return f >= SPMV_CSR && f <= SPMV_HEC; }

// Column-index cache policy of the ELL-family kernels: streamed past the
// caches (the default) or cached, whichever applies faster.  Cached indices
// pay when they fit the last-level cache beside x over repeated applies.
void choose_col_policy(int opt, Built& b) { b.col_nt = opt != 1; }

// HYB/HEC at ELL width `width` (as choose_width takes it): the split, the
// window and group choices, and the tail kernel
void build_split_tuned(spmv_handle* h, int format, const spmv_convert_opts& o, int width,
                       Built& b, hipStream_t s) {
    b.format = format;
    if (h->dtype == SPMV_F64)
        build_split<double>(h, format, width, o.sort_window, b, s);
    else
        build_split<float>(h, format, width, o.sort_window, b, s);
    decide_window(h, format, o.x_window, b, s);
    choose_groups(h, o.ell_groups, b);
    if (format == SPMV_HYB || format == SPMV_HEC)
        tune_tail(h, format, o.csr_kernel, o.col_cache, budget_bytes(o), b, s);
    choose_col_policy(o.col_cache, b);
}

// SELL-64 with or without the LDS window.  The window needs the rows
// sorted inside windows that divide the tile (default kSellWinSortWindow
// rows); without it the default sort window is kSellSortWindow.  x_window
// -1: when at least half of the entries lie within the window's reach, both
// layouts are built and one apply of each timed; the window is kept when
// faster by kPreferMargin.  No room for the second layout: the first one.
template <typename V>
void convert_sell(spmv_handle* h, const spmv_convert_opts& o, Built& b, hipStream_t s) {
    const bool permuted = o.permuted_basis != 0;
    auto build = [&](Built& c, bool win) {
        build_sell<V>(h, o.sort_window, permuted, win, c, s);
        choose_col_policy(o.col_cache, c);
    };
    const bool fits = window_fits(h) && h->n > 0;
    const double band = o.x_window == 0 ? 0.0 : band_fraction(h, s);
    if (o.x_window == 1 || (o.x_window == -1 && fits && h->nnz > 0 && band >= 0.5)) {
        build(b, fits);
        b.band_fraction = band;
        if (o.x_window == 1 || !fits) return;
        Built plain;
        try {
            build(plain, false);
        } catch (const Error& e) {
            if (e.code != SPMV_ERR_NO_MEMORY) throw;
            return;
        }
        plain.band_fraction = band;
        DevBuf xs((size_t)h->n * h->vsize), ys((size_t)h->n * h->vsize);
        hip_check(hipMemsetAsync(xs.p, 0, xs.bytes, s), "hipMemsetAsync");
        auto t_of = [&](const Built& c) {
            return time_launches(
                [&] { return launch_built(h, c, SPMV_SELL64, ys.p, xs.p, 1.0, 0.0, s); }, s);
        };
        const float tw = t_of(b), tp = t_of(plain);
        sync(s);
        if (!(tw < kPreferMargin * tp)) b = std::move(plain);
        return;
    }
    build(b, false);
    b.band_fraction = band;
}

// Build `format` (options already validated) and make it the active format.
void convert_into(spmv_handle* h, int format, const spmv_convert_opts& o) {
    if (format == SPMV_CSR) {
        Built b;
        tune_csr(h, o, b, nullptr);
        h->fmt = std::move(b);
        h->format = SPMV_CSR;
        return;
    }
    hipStream_t s = nullptr;
    const bool f64 = h->dtype == SPMV_F64;
    Built b;
    b.format = format;
    if (format == SPMV_ELLR) {
        const int64_t S = pad64(h->n), W = h->max_len;
        const double need = (double)W * (double)S * (4.0 + (double)h->vsize) + 4.0 * (double)S;
        const uint64_t budget = budget_bytes(o);
        if (need > (double)budget)
            fail(SPMV_ERR_FOOTPRINT,
                 "ELL-R needs %.3g bytes (%lld rows padded to %lld x width %lld) over the "
                 "budget of %.3g bytes",
                 need, (long long)h->n, (long long)S, (long long)W, (double)budget);
        if (f64)
            build_ell_part<double>(h, W, 0, 0, b, s);
        else
            build_ell_part<float>(h, W, 0, 0, b, s);
        decide_window(h, format, o.x_window, b, s);
        choose_groups(h, o.ell_groups, b);
        choose_col_policy(o.col_cache, b);
        sync(s);
    } else if (format == SPMV_SELL64) {
        if (f64)
            convert_sell<double>(h, o, b, s);
        else
            convert_sell<float>(h, o, b, s);
    } else {
        build_split_tuned(h, format, o, o.ell_width, b, s);
        if (o.ell_width < 0 && h->n > 0) {
            // second width candidate: the rows of regular length whole in the
            // ELL part (with a sorted ELL part its padding costs storage more
            // than reads), if it differs, fits the budget and applies faster
            std::vector<int> hist;
            const int64_t K2 = choose_width(h, kRegularWidth, hist, s);
            const double need = (double)K2 * (double)((h->n + kEllBlock - 1) / kEllBlock) *
                                (double)kEllBlock * (4.0 + (double)h->vsize);
            if (K2 > b.ell_width && need <= (double)budget_bytes(o)) {
                Built b2;
                build_split_tuned(h, format, o, (int)K2, b2, s);
                DevBuf xs((size_t)h->n * h->vsize), ys((size_t)h->n * h->vsize);
                hip_check(hipMemsetAsync(xs.p, 0, xs.bytes, s), "hipMemsetAsync");
                auto t_of = [&](const Built& c) {
                    return time_launches(
                        [&] { return launch_built(h, c, format, ys.p, xs.p, 1.0, 0.0, s); }, s);
                };
                float t1 = t_of(b), t2 = t_of(b2);
                if (std::fabs(t2 - t1) < 0.03f * t1)  // close: time both again
                    t1 = std::min(t1, t_of(b)), t2 = std::min(t2, t_of(b2));
                sync(s);
                // kept when faster by a clear margin: equal candidates (a
                // small, launch-bound matrix) must not flip on timing noise
                if (t2 < kWidthMargin * t1) b = std::move(b2);
            }
        }
    }
    h->fmt = std::move(b);
    h->format = format;
}

// Automatic format: build every eligible format in turn with the same
// options, time one apply of each on the device (x = 0: the apply does not
// depend on the values) and keep the fastest.  ELL-R is eligible only while
// its padded slots stay within kAutoEllPadding times the stored entries
// (its cost follows the slots, not the entries, once rows differ in length).
void convert_auto(spmv_handle* h, const spmv_convert_opts& o) {
    h->fmt = Built{};  // the previous format is released first
    h->format = SPMV_CSR;
    const double ell_slots = (double)pad64(h->n) * (double)h->max_len;
    std::vector<int> cand = {SPMV_CSR, SPMV_SELL64, SPMV_HYB, SPMV_HEC};
    if (ell_slots <= kAutoEllPadding * (double)std::max<int64_t>(h->nnz, 1))
        cand.insert(cand.begin() + 1, SPMV_ELLR);
    hipStream_t s = nullptr;
    DevBuf xs((size_t)std::max<int64_t>(h->n, 1) * h->vsize);
    DevBuf ys((size_t)std::max<int64_t>(h->n, 1) * h->vsize);
    hip_check(hipMemsetAsync(xs.p, 0, xs.bytes, s), "hipMemsetAsync");
    Built best;
    int best_fmt = -1;
    float best_ms = 0;
    for (int f : cand) {
        spmv_convert_opts of = o;
        if (f == SPMV_CSR || f == SPMV_ELLR) of.sort_window = -1;
        try {
            convert_into(h, f, of);
        } catch (const Error& e) {
            if (e.code != SPMV_ERR_FOOTPRINT) throw;
            continue;  // too large for the budget: not a candidate
        }
        const float ms = h->n == 0 ? 0.0f : time_launches([&] {
            return launch_built(h, h->fmt, f, ys.p, xs.p, 1.0, 0.0, s);
        }, s);
        if (best_fmt < 0 || ms < best_ms) {
            best = std::move(h->fmt);
            best_fmt = f;
            best_ms = ms;
        }
        h->fmt = Built{};
        h->format = SPMV_CSR;
    }
    h->fmt = std::move(best);
    h->format = best_fmt;
}


// Krylov solvers driven from the host: every product is the active format's
// apply; the scalars of an iteration are two fp64 inner products read back
// (the textbook forms of conjugate gradients and BiCGSTAB, stopping on the
// recurred residual).
// Iterations enqueued per graph replay: the host reads the state back once
// per replay, so a solve ends at most kSolveGraphIters - 1 idle iterations
// (whose kernels leave at once, applies aside) after convergence.
constexpr int kSolveGraphIters = 8;

// RAII holders for the solve's private stream and graph
struct StreamHolder {
    hipStream_t s = nullptr;
    ~StreamHolder() {
        if (s) (void)hipStreamDestroy(s);
    }
};
struct GraphHolder {
    hipGraph_t g = nullptr;
    hipGraphExec_t e = nullptr;
    ~GraphHolder() {
        if (e) (void)hipGraphExecDestroy(e);
        if (g) (void)hipGraphDestroy(g);
    }
};

// Device memory of one solve: the work vectors (each `vstride` bytes apart),
// the inner products' partial sums and the iteration's scalars.
struct SolveSpace {
    char* work = nullptr;
    size_t vstride = 0;
    double* partial = nullptr;  // [2 * kSolveBlocks]
    double* state = nullptr;    // [kStCount]
};

int solve_vectors(int method) { return method == SPMV_SOLVE_CG ? 3 : 6; }

// Krylov solve driven from the device: the iteration's scalars stay in
// device memory (st).  With `fixed` == nullptr the work vectors are
// allocated for the call and kSolveGraphIters iterations are captured once
// in a HIP graph on a private stream and replayed; with a fixed workspace
// (the no-allocation entry point) nothing is allocated or created: batches
// of kSolveGraphIters iterations are enqueued on the caller's stream.  Either
// way the host only reads the done flag after each batch, and the same
// kernels run in the same order, so both give the same iterates.  The
// recurrences are the textbook ones (see the kernels in k_vec.hip); the setup
// (b.b, r = b - A x, r.r) runs first.  Every vector, partial sum and scalar
// an iteration reads is written by the setup or earlier in the iteration.
spmv_solve_info solve(spmv_handle* h, void* x, const void* b, const spmv_solve_opts& o,
                      hipStream_t caller, const SolveSpace* fixed) {
    const int64_t n = h->n;
    const bool f64 = h->dtype == SPMV_F64;
    const size_t vb = (size_t)n * h->vsize;
    const int nvec = solve_vectors(o.method);
    auto chk = [](hipError_t e, const char* what) { hip_check(e, what); };
    StreamHolder sh;
    DevBuf work, partial, state;
    SolveSpace sp;
    hipStream_t s = caller;
    if (fixed) {
        sp = *fixed;
    } else {
        // the caller's stream may be the null stream, which cannot be
        // captured: work on a private stream ordered after the caller's work
        sync(caller);
        chk(hipStreamCreateWithFlags(&sh.s, hipStreamNonBlocking), "hipStreamCreateWithFlags");
        s = sh.s;
        work.alloc(vb * nvec);
        partial.alloc((size_t)2 * kSolveBlocks * 8);
        state.alloc(kStCount * 8);
        sp.work = work.as<char>();
        sp.vstride = vb;
        sp.partial = partial.as<double>();
        sp.state = state.as<double>();
    }
    char* w = sp.work;
    const size_t vs = sp.vstride;
    void *r = w, *p = w + vs, *q = w + 2 * vs;           // CG: r, p, q = A p
    void *rh = w + 2 * vs, *v = w + 3 * vs, *sv = w + 4 * vs, *t = w + 5 * vs;  // BiCGSTAB
    double* pd = sp.partial;
    double* st = sp.state;
    auto apply = [&](void* yy, const void* xx, double alpha, double beta) {
        chk(launch_built(h, h->fmt, h->format, yy, xx, alpha, beta, s), "apply");
    };
    double d2[2];
    auto dot = [&](const void* a0, const void* b0) {
        chk(launch_dot2(n, f64, a0, b0, nullptr, nullptr, pd, st + kStPQ, s), "dot");
        chk(hipMemcpyAsync(d2, st + kStPQ, 8, hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
        sync(s);
        return d2[0];
    };
    // setup: ||b||, r = b - A x, r.r, the state
    const double bnorm = std::sqrt(dot(b, b));
    chk(hipMemcpyAsync(r, b, vb, hipMemcpyDeviceToDevice, s), "hipMemcpyAsync");
    apply(r, x, -1.0, 1.0);
    const double rr0 = dot(r, r);
    const double goal = o.rtol * bnorm;
    double st0[kStCount] = {};
    st0[kStRR] = rr0;
    st0[kStGoal] = goal;
    st0[kStMaxIt] = (double)o.max_iter;
    st0[kStDone] = std::sqrt(rr0) > goal ? 0.0 : 1.0;
    st0[kStRho] = st0[kStAlpha] = st0[kStOmega] = 1.0;
    // BiCGSTAB's first rho = rhat . r with rhat = r, and the first beta from
    // rho = alpha = omega = 1 (p = v = 0 makes the first direction r)
    st0[kStRhoNew] = st0[kStBeta] = rr0;
    chk(hipMemcpyAsync(st, st0, sizeof st0, hipMemcpyHostToDevice, s), "hipMemcpyAsync");
    if (o.method == SPMV_SOLVE_CG) {
        chk(hipMemcpyAsync(p, r, vb, hipMemcpyDeviceToDevice, s), "hipMemcpyAsync");
    } else {
        chk(hipMemcpyAsync(rh, r, vb, hipMemcpyDeviceToDevice, s), "hipMemcpyAsync");
        chk(hipMemsetAsync(p, 0, vb, s), "hipMemsetAsync");
        chk(hipMemsetAsync(v, 0, vb, s), "hipMemsetAsync");
    }
    sync(s);
    // one iteration, enqueued on s (captured below, or run in batches on the
    // caller's stream with a fixed workspace)
    auto iteration = [&] {
        if (o.method == SPMV_SOLVE_CG) {
            apply(q, p, 1.0, 0.0);
            chk(launch_dot2(n, f64, p, q, nullptr, nullptr, pd, nullptr, s), "dot");
            chk(launch_solve_step(pd, st, kStepCgPQ, s), "step");
            chk(launch_cg_xr(n, f64, x, r, p, q, st, pd, s), "cg update");
            chk(launch_solve_step(pd, st, kStepCgRR, s), "step");
            chk(launch_update_p(n, f64, p, r, nullptr, st, s), "cg direction");
        } else {
            chk(launch_update_p(n, f64, p, r, v, st, s), "bicgstab direction");
            apply(v, p, 1.0, 0.0);
            chk(launch_dot2(n, f64, rh, v, nullptr, nullptr, pd, nullptr, s), "dot");
            chk(launch_solve_step(pd, st, kStepBiRV, s), "step");
            chk(launch_axmy(n, f64, sv, r, v, st, s), "bicgstab s");
            apply(t, sv, 1.0, 0.0);
            chk(launch_dot2(n, f64, t, sv, t, t, pd, nullptr, s), "dot");
            chk(launch_solve_step(pd, st, kStepBiOmega, s), "step");
            chk(launch_bicg_xr(n, f64, x, r, p, sv, t, rh, st, pd, s), "bicgstab update");
            chk(launch_solve_step(pd, st, kStepBiRR, s), "step");
        }
    };
    const int64_t batches = ((int64_t)o.max_iter + kSolveGraphIters - 1) / kSolveGraphIters;
    if (st0[kStDone] == 0.0 && fixed) {
        double flag = 0.0;
        for (int64_t k = 0; k < batches && flag == 0.0; ++k) {
            for (int i = 0; i < kSolveGraphIters; ++i) iteration();
            chk(hipMemcpyAsync(&flag, st + kStDone, 8, hipMemcpyDeviceToHost, s),
                "hipMemcpyAsync");
            sync(s);
        }
    } else if (st0[kStDone] == 0.0) {
        GraphHolder gh;
        chk(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
        try {
            for (int i = 0; i < kSolveGraphIters; ++i) iteration();
        } catch (...) {
            hipGraph_t g = nullptr;
            (void)hipStreamEndCapture(s, &g);
            if (g) (void)hipGraphDestroy(g);
            throw;
        }
        chk(hipStreamEndCapture(s, &gh.g), "hipStreamEndCapture");
        chk(hipGraphInstantiate(&gh.e, gh.g, nullptr, nullptr, 0), "hipGraphInstantiate");
        double flag = 0.0;
        for (int64_t k = 0; k < batches && flag == 0.0; ++k) {
            chk(hipGraphLaunch(gh.e, s), "hipGraphLaunch");
            chk(hipMemcpyAsync(&flag, st + kStDone, 8, hipMemcpyDeviceToHost, s),
                "hipMemcpyAsync");
            sync(s);
        }
    }
    chk(hipMemcpyAsync(st0, st, sizeof st0, hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
    sync(s);  // before the work vectors are freed
    const double rr = st0[kStRR];
    spmv_solve_info res;
    res.iterations = (int)st0[kStK];
    res.rel_residual = bnorm > 0 ? std::sqrt(rr) / bnorm : std::sqrt(rr);
    res.converged = std::sqrt(rr) <= goal ? 1 : 0;
    return res;
}

// arguments of spmv_solve / spmv_solve_noalloc
spmv_solve_opts check_solve_args(const spmv_handle* h, const void* x, const void* b,
                                 const spmv_solve_opts* opts) {
    if (!h) fail(SPMV_ERR_STATE, "null handle");
    if (!opts) fail(SPMV_ERR_INVALID_ARG, "opts is NULL");
    const spmv_solve_opts o = *opts;
    if (o.method != SPMV_SOLVE_CG && o.method != SPMV_SOLVE_BICGSTAB)
        fail(SPMV_ERR_INVALID_ARG, "unknown method %d", o.method);
    if (o.max_iter <= 0) fail(SPMV_ERR_INVALID_ARG, "max_iter must be positive");
    if (!(o.rtol >= 0)) fail(SPMV_ERR_INVALID_ARG, "rtol must be >= 0");
    if (h->n > 0) {
        if (!x || !b) fail(SPMV_ERR_INVALID_ARG, "x or b is NULL");
        const uintptr_t xb = (uintptr_t)x, bb = (uintptr_t)b, len = (uintptr_t)(h->n * h->vsize);
        if (xb < bb + len && bb < xb + len) fail(SPMV_ERR_INVALID_ARG, "x and b overlap");
    }
    return o;
}

// ---------------------------------------------------------------------------
// Workspace of the no-allocation solve: one array per GPU in the library's
// code object, held until the process ends.  Its head holds the iteration's
// scalars (offset 0) and the inner products' partial sums (offset 256); the
// work vectors follow from kScratchHead, each starting on a 256-byte
// boundary.  Host code never names the array itself (its host-side symbol
// is no device address): the device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr size_t kScratchHead = size_t(64) << 10;
static_assert(256 + 2 * kSolveBlocks * 8 <= kScratchHead, "scratch head too small");
static_assert(kStCount * 8 <= 256, "solver state too large");
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of this device's scratch array
char* scratch_base(int dev) {
    if (dev < 0 || dev >= kMaxDevices) fail(SPMV_ERR_STATE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress");
        if (!p) fail(SPMV_ERR_HIP, "hipGetSymbolAddress returned no address");
        g_scratch_ptr[dev] = p;
    }
    return static_cast<char*>(g_scratch_ptr[dev]);
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// the solve's layout inside this device's scratch array (the handle's device
// must be current); INVALID_ARG when the vectors do not fit
SolveSpace solve_scratch(const spmv_handle* h, int method) {
    int dev = 0;
    hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (dev != h->device)
        fail(SPMV_ERR_STATE, "the handle lives on device %d, device %d is current", h->device, dev);
    const size_t vstride = round256((size_t)h->n * h->vsize);
    const int nvec = solve_vectors(method);
    const size_t room = kScratchBytes - kScratchHead;
    if (vstride > room / nvec)
        fail(SPMV_ERR_INVALID_ARG,
             "n = %lld needs %zu bytes of work vectors; the no-allocation solve holds %zu "
             "(at most %lld rows for this method and dtype)",
             (long long)h->n, vstride * nvec, room, (long long)((room / nvec) / 256 * 256 / h->vsize));
    char* base = scratch_base(dev);
    SolveSpace sp;
    sp.state = reinterpret_cast<double*>(base);
    sp.partial = reinterpret_cast<double*>(base + 256);
    sp.work = base + kScratchHead;
    sp.vstride = vstride;
    return sp;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* spmv_last_error(void) { return g_err.c_str(); }

const char* spmv_version(void) { return "sparse_formats_amd 0.1 (gfx950)"; }

int spmv_create(spmv_t* out, int kind, int64_t n, int64_t nnz, const int64_t* rowidx,
                const int32_t* col, const void* val, int dtype, void* stream) {
    g_err.clear();
    return run_guarded([&] {
        if (!out) fail(SPMV_ERR_INVALID_ARG, "out is NULL");
        if (kind != SPMV_IN_CSR && kind != SPMV_IN_COO)
            fail(SPMV_ERR_INVALID_ARG, "unknown input kind %d", kind);
        if (dtype != SPMV_F32 && dtype != SPMV_F64)
            fail(SPMV_ERR_INVALID_ARG, "unknown dtype %d", dtype);
        if (n < 0 || nnz < 0) fail(SPMV_ERR_INVALID_ARG, "negative size (n=%lld nnz=%lld)",
                                   (long long)n, (long long)nnz);
        if (n >= INT32_MAX || nnz > kMaxNnz)
            fail(SPMV_ERR_INVALID_ARG, "n must be below 2^31-1 and nnz at most 2^31-65537");
        if (kind == SPMV_IN_CSR && !rowidx) fail(SPMV_ERR_INVALID_ARG, "rowptr is NULL");
        if (nnz > 0 && (!rowidx || !col || !val))
            fail(SPMV_ERR_INVALID_ARG, "row/col/val pointer is NULL");
        hipStream_t s = (hipStream_t)stream;
        int dev = 0;
        hip_check(hipGetDevice(&dev), "hipGetDevice");
        auto* h = new spmv_handle;
        try {
            h->device = dev;
            h->n = n;
            h->nnz = nnz;
            h->dtype = dtype;
            h->vsize = dtype == SPMV_F64 ? 8 : 4;
            h->rowptr.alloc((size_t)(n + 1) * 4);
            h->col.alloc((size_t)nnz * 4 + 16);
            h->val.alloc((size_t)nnz * h->vsize + 16);
            hip_check(hipMemsetAsync((char*)h->col.p + (size_t)nnz * 4, 0, 16, s),
                      "hipMemsetAsync");
            hip_check(hipMemsetAsync((char*)h->val.p + (size_t)nnz * h->vsize, 0, 16, s),
                      "hipMemsetAsync");
            DevBuf flags(8);
            hip_check(hipMemsetAsync(flags.p, 0, 8, s), "hipMemsetAsync");
            if (kind == SPMV_IN_CSR) {
                hipLaunchKernelGGL(k_validate_csr, dim3(grid_for(std::max(n + 1, nnz))), dim3(256),
                                   0, s, n, nnz, rowidx, col, flags.as<int>(), h->rowptr.as<int>());
                hip_check(hipGetLastError(), "validate");
                const int f = read_scalar<int>(flags.p, s);
                if (f)
                    fail(SPMV_ERR_INVALID_MATRIX, "invalid CSR:%s%s%s%s",
                         f & F_FIRST ? " rowptr[0] != 0;" : "",
                         f & F_LAST ? " rowptr[n] != nnz;" : "",
                         f & F_MONO ? " rowptr decreases;" : "",
                         f & F_COL ? " column outside [0, n);" : "");
                if (nnz > 0) {
                    hip_check(hipMemcpyAsync(h->col.p, col, (size_t)nnz * 4,
                                             hipMemcpyDeviceToDevice, s), "hipMemcpyAsync");
                    hip_check(hipMemcpyAsync(h->val.p, val, (size_t)nnz * h->vsize,
                                             hipMemcpyDeviceToDevice, s), "hipMemcpyAsync");
                }
            } else {
                DevBuf rows32((size_t)nnz * 4), rows_sorted((size_t)nnz * 4), order((size_t)nnz * 4);
                if (nnz > 0) {
                    hipLaunchKernelGGL(k_validate_coo, dim3(grid_for(nnz)), dim3(256), 0, s, n, nnz,
                                       rowidx, col, flags.as<int>(), rows32.as<unsigned>());
                    hip_check(hipGetLastError(), "validate");
                }
                const int f = read_scalar<int>(flags.p, s);
                if (f)
                    fail(SPMV_ERR_INVALID_MATRIX, "invalid COO:%s%s",
                         f & F_ROW ? " row outside [0, n);" : "",
                         f & F_COL ? " column outside [0, n);" : "");
                if (nnz > 0) {
                    size_t tmp = 0;
                    rocprim::counting_iterator<int> iota(0);
                    const unsigned nb = bits_for((uint64_t)n);
                    hip_check(rocprim::radix_sort_pairs(nullptr, tmp, rows32.as<unsigned>(),
                                                        rows_sorted.as<unsigned>(), iota,
                                                        order.as<int>(), (size_t)nnz, 0, nb, s),
                              "radix_sort_pairs");
                    DevBuf work(tmp);
                    hip_check(rocprim::radix_sort_pairs(work.p, tmp, rows32.as<unsigned>(),
                                                        rows_sorted.as<unsigned>(), iota,
                                                        order.as<int>(), (size_t)nnz, 0, nb, s),
                              "radix_sort_pairs");
                    hipLaunchKernelGGL(k_gather, dim3(grid_for(nnz)), dim3(256), 0, s, nnz,
                                       order.as<int>(), col, (const char*)val, (int)h->vsize,
                                       h->col.as<int>(), h->val.as<char>());
                    hip_check(hipGetLastError(), "gather");
                    sync(s);
                }
                hipLaunchKernelGGL(k_rowptr_from_sorted, dim3(grid_for(n + 1)), dim3(256), 0, s, n,
                                   nnz, rows_sorted.as<unsigned>(), h->rowptr.as<int>());
                hip_check(hipGetLastError(), "rowptr");
                sync(s);
            }
            hip_check(hipMemsetAsync(flags.p, 0, 4, s), "hipMemsetAsync");
            if (n > 0) {
                hipLaunchKernelGGL(k_max_len, dim3(std::min<unsigned>(grid_for(n), 1024)), dim3(256),
                                   0, s, n, h->rowptr.as<int>(), flags.as<int>());
                hip_check(hipGetLastError(), "max length");
            }
            h->max_len = read_scalar<int>(flags.p, s);
            int sw = 1;
            while (sw < 64 && sw < h->max_len) sw <<= 1;
            h->subwave = sw;
        } catch (...) {
            delete h;
            throw;
        }
        *out = h;
    });
}

int spmv_convert(spmv_t h, int format, const spmv_convert_opts* opts) {
    g_err.clear();
    return run_guarded([&] {
        if (!h) fail(SPMV_ERR_STATE, "null handle");
        FlushScope flush;  // cache flushes between the conversion's timed launches
        if (!valid_format(format) && format != SPMV_AUTO)
            fail(SPMV_ERR_INVALID_ARG, "unknown format %d", format);
        spmv_convert_opts o{-1, 0, -1, 0, SPMV_CSR_AUTO, -1, 0, 0, 0, -1, -1};
        if (opts) o = *opts;
        if (o.ell_groups != 0 && o.ell_groups != 1 && o.ell_groups != 4 && o.ell_groups != 16)
            fail(SPMV_ERR_INVALID_ARG, "ell_groups must be 0, 1, 4 or 16 (got %d)", o.ell_groups);
        if (o.permuted_basis != 0 && o.permuted_basis != 1)
            fail(SPMV_ERR_INVALID_ARG, "permuted_basis must be 0 or 1");
        if (o.permuted_basis && format != SPMV_SELL64)
            fail(SPMV_ERR_INVALID_ARG, "permuted_basis applies to SELL-64 only");
        if (o.sort_window < -1)
            fail(SPMV_ERR_INVALID_ARG, "sort_window must be -1, 0 or positive (got %d)",
                 o.sort_window);
        if ((format == SPMV_CSR || format == SPMV_ELLR) && o.sort_window > 0)
            fail(SPMV_ERR_INVALID_ARG, "sort_window applies to SELL-64, HYB and HEC only");
        if ((format == SPMV_HYB || format == SPMV_HEC || format == SPMV_AUTO) &&
            o.sort_window > 0 &&
            (o.sort_window < 64 || o.sort_window > kEllBlock || kEllBlock % o.sort_window))
            fail(SPMV_ERR_INVALID_ARG,
                 "sort_window for HYB/HEC must be -1, 0 or a power of two in 64..%d (got %d)",
                 kEllBlock, o.sort_window);
        if (o.x_window < -1 || o.x_window > 1)
            fail(SPMV_ERR_INVALID_ARG, "x_window must be -1, 0 or 1");
        if (o.csr_rows < 0 || o.csr_rows > kCsrRowsMax || (o.csr_rows & (o.csr_rows - 1)))
            fail(SPMV_ERR_INVALID_ARG, "csr_rows must be 0 or a power of two up to %d",
                 kCsrRowsMax);
        if (o.subwave < 0 || o.subwave > 64 || (o.subwave & (o.subwave - 1)))
            fail(SPMV_ERR_INVALID_ARG, "subwave must be 0 or a power of two in 1..64 (got %d)",
                 o.subwave);
        if (o.csr_kernel < SPMV_CSR_AUTO || o.csr_kernel > SPMV_CSR_XBLOCK)
            fail(SPMV_ERR_INVALID_ARG, "csr_kernel must be 0, 1, 2 or 3 (got %d)", o.csr_kernel);
        if (o.csr_kernel == SPMV_CSR_XBLOCK && format != SPMV_CSR && format != SPMV_HYB &&
            format != SPMV_HEC)
            fail(SPMV_ERR_INVALID_ARG,
                 "csr_kernel 3 (column slices) applies to the CSR format and the HYB and HEC "
                 "tails only");
        if (o.csr_kernel == SPMV_CSR_XBLOCK &&
            (o.subwave || o.csr_rows > 1 || o.csr_stage == 1 ||
             (o.x_window == 1 && format == SPMV_CSR)))
            fail(SPMV_ERR_INVALID_ARG,
                 "csr_kernel 3 (column slices) takes no subwave, csr_rows, csr_stage or (CSR) "
                 "x_window");
        if (o.col_cache < -1 || o.col_cache > 1)
            fail(SPMV_ERR_INVALID_ARG, "col_cache must be -1, 0 or 1 (got %d)", o.col_cache);
        if (o.csr_stage < -1 || o.csr_stage > 1)
            fail(SPMV_ERR_INVALID_ARG, "csr_stage must be -1, 0 or 1 (got %d)", o.csr_stage);
        if (o.csr_stage == 1 &&
            ((o.subwave && (o.subwave < kCsrStageMin || o.subwave > kCsrStageMax)) ||
             o.csr_rows > 1 || o.csr_kernel == SPMV_CSR_BALANCED))
            fail(SPMV_ERR_INVALID_ARG,
                 "csr_stage = 1 needs the vector kernel with subwave 0 or %d..%d and csr_rows 0 "
                 "or 1", kCsrStageMin, kCsrStageMax);
        if (format == SPMV_AUTO)
            convert_auto(h, o);
        else
            convert_into(h, format, o);
    });
}

int spmv_apply(spmv_t h, void* y, const void* x, double alpha, double beta, void* stream) {
    g_err.clear();
    if (!h) {
        g_err = "null handle";
        return SPMV_ERR_STATE;
    }
    if (h->n > 0 && (!y || !x)) {
        g_err = "x or y is NULL";
        return SPMV_ERR_INVALID_ARG;
    }
    const uintptr_t yb = (uintptr_t)y, xb = (uintptr_t)x, len = (uintptr_t)(h->n * h->vsize);
    if (h->n > 0 && yb < xb + len && xb < yb + len) {
        g_err = "x and y overlap";
        return SPMV_ERR_INVALID_ARG;
    }
    if (h->n == 0) return SPMV_OK;
    const hipError_t e = launch_built(h, h->fmt, h->format, y, x, alpha, beta, (hipStream_t)stream);
    if (e != hipSuccess) {
        g_err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return SPMV_ERR_HIP;
    }
    return SPMV_OK;
}

int spmv_permute(spmv_t h, void* dst, const void* src, int direction, void* stream) {
    g_err.clear();
    if (!h) {
        g_err = "null handle";
        return SPMV_ERR_STATE;
    }
    if (h->format != SPMV_SELL64) {
        g_err = "spmv_permute needs SELL-64 as the active format";
        return SPMV_ERR_STATE;
    }
    if (direction != 0 && direction != 1) {
        g_err = "direction must be 0 (to the sorted basis) or 1 (back)";
        return SPMV_ERR_INVALID_ARG;
    }
    if (h->n == 0) return SPMV_OK;
    if (!dst || !src) {
        g_err = "dst or src is NULL";
        return SPMV_ERR_INVALID_ARG;
    }
    const uintptr_t d = (uintptr_t)dst, q = (uintptr_t)src, len = (uintptr_t)(h->n * h->vsize);
    if (d < q + len && q < d + len) {
        g_err = "dst and src overlap";
        return SPMV_ERR_INVALID_ARG;
    }
    const hipError_t e = launch_permute(h->n, h->dtype == SPMV_F64, dst, src,
                                        h->fmt.perm.as<int>(), direction == 1,
                                        (hipStream_t)stream);
    if (e != hipSuccess) {
        g_err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return SPMV_ERR_HIP;
    }
    return SPMV_OK;
}

int spmv_solve(spmv_t h, void* x, const void* b, const spmv_solve_opts* opts,
               spmv_solve_info* info, void* stream) {
    g_err.clear();
    return run_guarded([&] {
        const spmv_solve_opts o = check_solve_args(h, x, b, opts);
        spmv_solve_info res{0, 1, 0.0};
        if (h->n > 0) res = solve(h, x, b, o, (hipStream_t)stream, nullptr);
        if (info) *info = res;
    });
}

int spmv_solve_noalloc(spmv_t h, void* x, const void* b, const spmv_solve_opts* opts,
                       spmv_solve_info* info, void* stream) {
    g_err.clear();
    return run_guarded([&] {
        const spmv_solve_opts o = check_solve_args(h, x, b, opts);
        spmv_solve_info res{0, 1, 0.0};
        if (h->n > 0) {
            const SolveSpace sp = solve_scratch(h, o.method);
            res = solve(h, x, b, o, (hipStream_t)stream, &sp);
        }
        if (info) *info = res;
    });
}

int spmv_destroy(spmv_t h) {
    g_err.clear();
    if (!h) return SPMV_OK;
    return run_guarded([&] {
        hipError_t e = hipDeviceSynchronize();
        delete h;
        hip_check(e, "hipDeviceSynchronize");
    });
}

int spmv_info(spmv_t h, spmv_info_t* out) {
    g_err.clear();
    if (!h) {
        g_err = "null handle";
        return SPMV_ERR_STATE;
    }
    if (!out) {
        g_err = "out is NULL";
        return SPMV_ERR_INVALID_ARG;
    }
    spmv_info_t i{};
    i.n = h->n;
    i.nnz = h->nnz;
    i.dtype = h->dtype;
    i.format = h->format;
    i.max_len = h->max_len;
    i.subwave = h->subwave;
    const Built& b = h->fmt;
    switch (h->format) {
        case SPMV_CSR: i.slots = h->nnz; break;
        case SPMV_ELLR:
            i.ell_width = (int32_t)b.ell_width;
            i.ell_stride = b.ell_bh;
            i.ell_rows = b.ell_rows;
            i.slots = b.ell_width * b.ell_rows;
            break;
        case SPMV_SELL64:
            i.nslices = (int32_t)b.nslices;
            i.slots = b.sell_slots;
            break;
        default:
            i.ell_width = (int32_t)b.ell_width;
            i.ell_stride = b.ell_bh;
            i.ell_rows = b.ell_rows;
            i.tail_nnz = b.tail_nnz;
            i.slots = b.ell_width * b.ell_rows + b.tail_nnz;
    }
    i.footprint_bytes = h->rowptr.bytes + h->col.bytes + h->val.bytes + b.bytes();
    i.x_window = b.window ? 1 : 0;
    i.csr_rows = h->csr_rows;
    i.csr_stage_slots =
        h->format == SPMV_CSR && !b.csr_balanced && !b.csr_xblock ? h->csr_stage_slots : 0;
    i.tail_kernel = (h->format == SPMV_HYB || h->format == SPMV_HEC) && b.tail_nnz > 0
                        ? (b.tail_xblock   ? SPMV_CSR_XBLOCK
                           : b.tail_vector ? SPMV_CSR_VECTOR
                                           : SPMV_CSR_BALANCED)
                        : SPMV_CSR_AUTO;
    const bool tv = h->format == SPMV_HEC && b.tail_nnz > 0 && b.tail_vector;
    i.tail_subwave = tv ? b.tail_vec.subwave : 0;
    i.tail_rows = tv ? b.tail_vec.rows : 0;
    i.tail_stage_slots = tv ? b.tail_vec.slots : 0;
    if (h->format == SPMV_CSR)
        i.col_cached =
            !b.csr_balanced && !b.csr_xblock && h->csr_stage_slots > 0 && !h->csr_stage_col_nt;
    else
        i.col_cached = !b.col_nt;
    i.csr_kernel = h->format == SPMV_CSR && b.csr_xblock     ? SPMV_CSR_XBLOCK
                   : h->format == SPMV_CSR && b.csr_balanced ? SPMV_CSR_BALANCED
                                                             : SPMV_CSR_VECTOR;
    i.sort_window = b.sort_window;
    i.ell_groups = (h->format == SPMV_ELLR || h->format == SPMV_HYB || h->format == SPMV_HEC)
                       ? b.ell_groups
                       : 0;
    i.permuted_basis = h->format == SPMV_SELL64 && b.permuted ? 1 : 0;
    i.ell_head = h->format == SPMV_ELLR && b.window && b.ell_nlong > 0 ? b.ell_head : 0;
    i.ell_long_rows = i.ell_head ? b.ell_nlong : 0;
    i.band_fraction = b.band_fraction;
    *out = i;
    return SPMV_OK;
}

int spmv_export(spmv_t h, int array, void* host_dst, int64_t capacity_bytes, int64_t* bytes) {
    g_err.clear();
    return run_guarded([&] {
        if (!h) fail(SPMV_ERR_STATE, "null handle");
        const Built& b = h->fmt;
        const int f = h->format;
        const bool ell = f == SPMV_ELLR || f == SPMV_HYB || f == SPMV_HEC;
        const void* src = nullptr;
        int64_t sz = -1;
        const int64_t vs = (int64_t)h->vsize;
        switch (array) {
            case SPMV_A_ROWPTR: src = h->rowptr.p, sz = (h->n + 1) * 4; break;
            case SPMV_A_COL: src = h->col.p, sz = h->nnz * 4; break;
            case SPMV_A_VAL: src = h->val.p, sz = h->nnz * vs; break;
            case SPMV_A_ELL_COL: if (ell) src = b.ell_col.p, sz = b.ell_width * b.ell_rows * 4; break;
            case SPMV_A_ELL_VAL: if (ell) src = b.ell_val.p, sz = b.ell_width * b.ell_rows * vs; break;
            case SPMV_A_ELL_LEN: if (ell) src = b.ell_len.p, sz = b.ell_rows * 4; break;
            case SPMV_A_SELL_PERM: if (f == SPMV_SELL64) src = b.perm.p, sz = h->n * 4; break;
            case SPMV_A_SELL_SLICE_PTR: if (f == SPMV_SELL64) src = b.slice_ptr.p, sz = (b.nslices + 1) * 8; break;
            case SPMV_A_SELL_LEN: if (f == SPMV_SELL64) src = b.sell_len.p, sz = b.nslices * 64 * 4; break;
            case SPMV_A_SELL_COL: if (f == SPMV_SELL64) src = b.sell_col.p, sz = b.sell_slots * 4; break;
            case SPMV_A_SELL_VAL: if (f == SPMV_SELL64) src = b.sell_val.p, sz = b.sell_slots * vs; break;
            case SPMV_A_TAIL_ROW: if (f == SPMV_HYB) src = b.tail_row.p, sz = b.tail_nnz * 4; break;
            case SPMV_A_TAIL_PTR: if (f == SPMV_HEC) src = b.tail_ptr.p, sz = (h->n + 1) * 4; break;
            case SPMV_A_TAIL_COL: if (f == SPMV_HYB || f == SPMV_HEC) src = b.tail_col.p, sz = b.tail_nnz * 4; break;
            case SPMV_A_TAIL_VAL: if (f == SPMV_HYB || f == SPMV_HEC) src = b.tail_val.p, sz = b.tail_nnz * vs; break;
            case SPMV_A_ELL_PERM: if (ell && b.ell_perm.p) src = b.ell_perm.p, sz = b.ell_rows * 4; break;
            default: fail(SPMV_ERR_INVALID_ARG, "unknown array id %d", array);
        }
        if (sz < 0) fail(SPMV_ERR_STATE, "array %d does not belong to the active format", array);
        if (bytes) *bytes = sz;
        if (!host_dst) return;
        if (capacity_bytes < sz)
            fail(SPMV_ERR_INVALID_ARG, "destination holds %lld bytes, array needs %lld",
                 (long long)capacity_bytes, (long long)sz);
        if (sz > 0 && b.ell_records && (array == SPMV_A_ELL_COL || array == SPMV_A_ELL_VAL)) {
            // the slots' columns or values out of the records, in pieces
            const int64_t slots = b.ell_width * b.ell_rows, piece = (int64_t)1 << 25;
            const int64_t es = array == SPMV_A_ELL_COL ? 4 : vs;
            DevBuf tmp((size_t)(std::min(slots, piece) * es));
            for (int64_t s0 = 0; s0 < slots; s0 += piece) {
                const int64_t k = std::min(slots - s0, piece);
                hipLaunchKernelGGL(k_ell_split, dim3(grid_for(k)), dim3(256), 0, nullptr, k,
                                   (int)(vs / 4 + 1), (int)(array == SPMV_A_ELL_COL ? vs / 4 : 0),
                                   (int)(es / 4), b.ell_col.as<int>() + s0 * (vs / 4 + 1),
                                   tmp.as<int>());
                hip_check(hipGetLastError(), "ell split");
                hip_check(hipMemcpy((char*)host_dst + s0 * es, tmp.p, (size_t)(k * es),
                                    hipMemcpyDeviceToHost),
                          "hipMemcpy");
            }
        } else if (sz > 0) {
            hip_check(hipMemcpy(host_dst, src, (size_t)sz, hipMemcpyDeviceToHost), "hipMemcpy");
        }
    });
}

int spmv_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    g_err.clear();
    // dst == NULL: read src only
    if (bytes < 0 || (bytes > 0 && !src) || ((uintptr_t)dst | (uintptr_t)src) % 16) {
        g_err = "bad copy arguments (null src, negative or not 16-byte aligned)";
        return SPMV_ERR_INVALID_ARG;
    }
    const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
    if (dst && bytes > 0 && d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes) {
        g_err = "copy buffers overlap";
        return SPMV_ERR_INVALID_ARG;
    }
    hipError_t e = launch_stream_copy(dst, src, bytes, (hipStream_t)stream);
    if (e != hipSuccess) {
        g_err = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return SPMV_ERR_HIP;
    }
    return SPMV_OK;
}

}  // extern "C"
