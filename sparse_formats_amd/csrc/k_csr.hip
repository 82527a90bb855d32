// CSR apply with a sub-wave of S lanes per row.  Row r's result goes to
// y[row_map[r]] when a row map is given (the HEC tail: rows that hold tail
// entries, added onto the ELL part's result with beta = 1), else to y[r].
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
// continue in further passes of U entries.  The R rows of a group are
// interleaved with those of the other groups of its wave (row = wave base +
// r * groups + group), so every load instruction covers consecutive rows:
// neighbouring rows share
// cache lines of val/col and, for banded matrices, entry u of neighbouring
// rows usually lies on the same diagonal, so their x reads share lines too.
// The first pass reads with clamped indices and masks the products, so it
// has no per-entry branches.  Pairs of lanes take 12 entries each per pass
// (24 per row: the rows of about 15-22 entries that make such a shape the
// fastest then finish in one pass); other groups cover 16 entries per pass.
template <int S, int R>
struct CsrFirstPass {
    static constexpr int a = (S == 2 ? 24 : 16) / S, b = 16 / R;
    static constexpr int value = (a < b ? a : b) > 2 ? (a < b ? a : b) : 2;
};

template <typename T, int S, int R>
__global__ __launch_bounds__(256) void k_csr_vector(int n, const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    const T* __restrict__ val,
                                                    const T* __restrict__ x, T* __restrict__ y,
                                                    const int* __restrict__ row_map, T alpha,
                                                    T beta, int64_t tile0) {
    constexpr int kGroups = kWave / S;  // groups per wave
    constexpr int U = CsrFirstPass<S, R>::value;
    const int64_t tile = tile0 + xcd_tile(blockIdx.x, gridDim.x);
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
    // longer rows: further passes of U entries per lane, each with all of its
    // loads issued before the first product (one round trip per pass)
#pragma unroll
    for (int r = 0; r < R; ++r)
        for (int k0 = kb[r] + sub + U * S; k0 < ke[r]; k0 += U * S) {
            T vv[U];
            int cc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kc = min(k0 + u * S, ke[r] - 1);
                vv[u] = val[kc];
                cc[u] = col[kc];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const T p = vv[u] * x[cc[u]];
                sum[r] += k0 + u * S < ke[r] ? p : T(0);
            }
        }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const T s_r = group_sum<S>(sum[r]);
        const int64_t row = base + r * kGroups;
        if (sub == 0 && row < n) {
            const int64_t out = row_map ? row_map[row] : row;
            y[out] = axpby(s_r, alpha, beta, y + out);
        }
    }
}

// Staged variant (one row per group, rows base .. base + 64/S - 1 per wave).
// The wave's rows hold the contiguous entries [k0, k1) of val/col; when they
// fit its LDS slice, the wave first copies them there with direct
// global-to-LDS loads of 16 bytes per lane on consecutive addresses (every
// instruction reads whole cache lines, once), then runs the group sums on
// the copy.  Without the copy each load instruction of a group touches the
// lines of 64/S separate row segments and a line is requested again by the
// next instruction, which raises the L1 to L2 request count, the limiter of
// short-row matrices.  The x reads keep the group layout (entry u of
// neighbouring rows on neighbouring lanes).  A wave whose rows do not fit
// reads val/col directly; both give the same sums.
// LDS per wave: `slots` entries of val (rounded up to whole passes of
// 64 * 16 / sizeof(T) values) and of col (whole passes of 256 columns).
template <typename T>
struct CsrStage {
    static constexpr int V = 16 / sizeof(T);  // values per 16-byte load
    static __host__ __device__ int val_slots(int slots) {
        return (slots + kWave * V - 1) / (kWave * V) * (kWave * V);
    }
    static __host__ __device__ int col_slots(int slots) { return (slots + 255) / 256 * 256; }
    static __host__ __device__ int wave_bytes(int slots) {
        return val_slots(slots) * (int)sizeof(T) + col_slots(slots) * 4;
    }
};

// Sum of the entries kb + sub, kb + sub + S, ... below ke in passes of U per
// lane (every load of a pass issued before its first product); ld(k, v, c)
// reads entry k, which is clamped to ke - 1 for the masked loads past the
// row.  The additions happen in the order of k_csr_vector<T, S, 1>, so both
// kernels give the same sums.
template <typename T, int S, int U, typename Load>
__device__ __forceinline__ T group_row_sum(int kb, int ke, int sub, const T* __restrict__ x,
                                           Load ld) {
    T acc = T(0);
    for (int k0 = kb + sub; k0 < ke; k0 += U * S) {
        T v[U];
        int c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ld(min(k0 + u * S, ke - 1), v[u], c[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const T p = v[u] * x[c[u]];
            acc += k0 + u * S < ke ? p : T(0);
        }
    }
    return acc;
}

template <typename T, int S>
__global__ __launch_bounds__(256) void k_csr_staged(int n, const int* __restrict__ rowptr,
                                                    const int* __restrict__ col,
                                                    const T* __restrict__ val,
                                                    const T* __restrict__ x, T* __restrict__ y,
                                                    const int* __restrict__ row_map, T alpha,
                                                    T beta, int slots, int col_nt, int64_t tile0) {
    using St = CsrStage<T>;
    constexpr int V = St::V;
    constexpr int U = CsrFirstPass<S, 1>::value;
    extern __shared__ __align__(16) char s_stage[];
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t base = ((tile0 + xcd_tile(blockIdx.x, gridDim.x)) * 4 + w) * (kWave / S);
    if (base >= n) return;  // whole waves leave together
    const int sub = lane & (S - 1);
    const int64_t row = base + lane / S;
    const int kb = rowptr[row < n ? row : n];
    const int ke = rowptr[row < n ? row + 1 : n];
    const int k0 = __builtin_amdgcn_readfirstlane(kb);       // lane 0: row base < n
    const int k1 = __builtin_amdgcn_readlane(ke, kWave - 1);  // end of the last row
    const int kA = k0 & -4;                                  // 16-byte aligned for both
    T sum;
    if (k1 > kA && k1 - kA <= St::val_slots(slots)) {
        // slots [0, k1 - kA) are all written below, and every read stays
        // there; a lane's last 16 bytes may pass k1 (col/val are padded by 16
        // bytes) and the last pass stays inside the rounded-up slices
        T* sv = reinterpret_cast<T*>(s_stage + w * St::wave_bytes(slots));
        int* sc = reinterpret_cast<int*>(sv + St::val_slots(slots));
        const int npv = (k1 - kA + kWave * V - 1) / (kWave * V);
        const int npc = (k1 - kA + kWave * 4 - 1) / (kWave * 4);
        for (int p = 0; p < npv; ++p) {
            const int k = kA + (p * kWave + lane) * V;
            if (k < k1) load_lds16_nt(val + k, sv + p * kWave * V);
        }
        if (col_nt) {
            for (int p = 0; p < npc; ++p) {
                const int k = kA + (p * kWave + lane) * 4;
                if (k < k1) load_lds16_nt(col + k, sc + p * kWave * 4);
            }
        } else {
            for (int p = 0; p < npc; ++p) {
                const int k = kA + (p * kWave + lane) * 4;
                if (k < k1) load_lds16(col + k, sc + p * kWave * 4);
            }
        }
        wait_vm();
        wave_lds_sync();
        sum = group_row_sum<T, S, U>(kb, ke, sub, x, [&](int k, T& v, int& c) {
            const int i = max(k - kA, 0);
            v = sv[i];
            c = sc[i];
        });
    } else {
        sum = group_row_sum<T, S, U>(kb, ke, sub, x, [&](int k, T& v, int& c) {
            const int i = max(k, 0);  // entry 0 exists: col/val are padded
            v = val[i];
            c = col[i];
        });
    }
    sum = group_sum<S>(sum);
    if (sub == 0 && row < n) {
        const int64_t out = row_map ? row_map[row] : row;
        y[out] = axpby(sum, alpha, beta, y + out);
    }
}

template <typename T, int S>
static hipError_t run_staged(const CsrView& a, int slots, bool col_nt, void* y, const void* x,
                             double alpha, double beta, hipStream_t stream) {
    constexpr int kRowsPerBlock = 256 / S;
    const int64_t blocks = ((int64_t)a.n + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks == 0) return hipSuccess;
    const size_t lds = 4 * (size_t)CsrStage<T>::wave_bytes(slots);
    if (slots < 1 || lds > kCsrStageLds) return hipErrorInvalidValue;
    const int64_t per = blocks_per_piece(kMaxLaunchItems, 256);
    for (int64_t b0 = 0; b0 < blocks; b0 += per) {
        const int64_t nb = std::min<int64_t>(blocks - b0, per);
        hipLaunchKernelGGL((k_csr_staged<T, S>), dim3((unsigned)nb), dim3(256), lds, stream, a.n,
                           a.rowptr, a.col, (const T*)a.val, (const T*)x, (T*)y, a.row_map,
                           (T)alpha, (T)beta, slots, col_nt ? 1 : 0, b0);
    }
    return hipGetLastError();
}

template <typename T, int S, int R>
static hipError_t run(const CsrView& a, void* y, const void* x, double alpha, double beta,
                      hipStream_t stream) {
    constexpr int kRowsPerBlock = 256 / S * R;  // 4 waves of 64 / S groups of R rows
    const int64_t blocks = ((int64_t)a.n + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks == 0) return hipSuccess;
    const int64_t per = blocks_per_piece(kMaxLaunchItems, 256);
    for (int64_t b0 = 0; b0 < blocks; b0 += per) {
        const int64_t nb = std::min<int64_t>(blocks - b0, per);
        hipLaunchKernelGGL((k_csr_vector<T, S, R>), dim3((unsigned)nb), dim3(256), 0, stream,
                           a.n, a.rowptr, a.col, (const T*)a.val, (const T*)x, (T*)y, a.row_map,
                           (T)alpha, (T)beta, b0);
    }
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
static hipError_t dispatch(const CsrView& a, int subwave, int rows, int slots, bool col_nt,
                           void* y, const void* x, double alpha, double beta,
                           hipStream_t stream) {
    if (slots > 0) {
        if (rows != 1) return hipErrorInvalidValue;
        switch (subwave) {
            case 2: return run_staged<T, 2>(a, slots, col_nt, y, x, alpha, beta, stream);
            case 4: return run_staged<T, 4>(a, slots, col_nt, y, x, alpha, beta, stream);
            case 8: return run_staged<T, 8>(a, slots, col_nt, y, x, alpha, beta, stream);
            case 16: return run_staged<T, 16>(a, slots, col_nt, y, x, alpha, beta, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (rows) {
        case 1: return dispatch_s<T, 1>(a, subwave, y, x, alpha, beta, stream);
        case 2: return dispatch_s<T, 2>(a, subwave, y, x, alpha, beta, stream);
        case 4: return dispatch_s<T, 4>(a, subwave, y, x, alpha, beta, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_csr(const CsrView& a, int subwave, int rows, int stage_slots, bool stage_col_nt,
                      bool f64, void* y, const void* x, double alpha, double beta,
                      hipStream_t stream) {
    return f64 ? dispatch<double>(a, subwave, rows, stage_slots, stage_col_nt, y, x, alpha, beta,
                                  stream)
               : dispatch<float>(a, subwave, rows, stage_slots, stage_col_nt, y, x, alpha, beta,
                                 stream);
}

int csr_stage_max_slots(bool f64) {
    int s = 256;  // largest multiple of 256 whose four wave slices fit
    while (4 * (size_t)(f64 ? CsrStage<double>::wave_bytes(s + 256)
                            : CsrStage<float>::wave_bytes(s + 256)) <= kCsrStageLds)
        s += 256;
    return s;
}

}  // namespace spmv
