// ELLPACK-R and SELL-64 apply: one lane per row.
//
// "Sparse matrix-vector multiplication on GPGPU clusters" (Sect. 2.1-2.2)
// maps consecutive rows to consecutive threads and stores the padded
// rectangle column by column, so that for a fixed entry index the lanes of a
// wave read consecutive slots; ELLPACK-R stops each row at its stored length
// (Fig. 2b).  The sorted variant (pJDS, here SELL-64 with one wave per slice
// of 64 sorted rows) pads each slice only to its own longest row.
// "Sparse Linear Algebra on AMD and NVIDIA GPUs -- The Race Is On" notes that
// on AMD GPUs the column-major layout must be read with one lane per row (a
// group of lanes on one row reads slots a whole stride apart); that is the
// mapping kept here.  ELLPACK-R is one column-major block of all rows; the
// ELL part of HYB/HEC is stored in column-major blocks of kEllBlock rows
// (see internal.h).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace spmv {

// ---------------------------------------------------------------------------
// ELLPACK-R (also the ELL part of HYB / HEC)
// ---------------------------------------------------------------------------
// A wave whose longest row is much longer than the others (a few long rows
// among short ones, the case the pages give against ELLPACK) would leave one
// lane reading that row's slots one by one, each slot in its own cache line
// of the column-major layout.  Once at most kEllCoopLanes lanes of a wave
// still have entries and the longest has at least kEllCoopMin left, the
// whole wave takes the remaining rows one after the other: lane k reads
// slots j0 + k, j0 + k + 64, ... of the row (kEllCoopUnroll in flight, or two
// sets of kEllRecUnroll for ELLPACK-R's records), and
// a wave sum adds the result to the row's lane.  Waves whose rows all stay
// within kEllCoopMin entries run the plain lane-per-row loop.
constexpr int kEllCoopLanes = 16;
constexpr int kEllCoopMin = 64;
constexpr int kEllCoopUnroll = 8;
// ELLPACK-R records in the window kernel: entries per round
constexpr int kEllWinRecB = 16;
// ELLPACK-R records: two sets of 4 in turn (the next set loads while the
// current one's x reads are in flight); measured on the FEM block's long rows
// against 8 at a time without the second set: 4.81 against 5.01 ms per apply
constexpr int kEllRecUnroll = 4;

// A row's slots in an ELL layout: records (kRec: value and column side by
// side, c points at the row's first record) or separate value and column
// arrays (c, v point at the row's first column and value; the value is
// streamed, the column by kColNT).  o is the slot offset from the row's first
// (j times the stride between a row's slots).
template <typename T, bool kColNT, bool kRec>
__device__ __forceinline__ void ld_slot(const int* __restrict__ c, const T* __restrict__ v,
                                        int64_t o, T& vo, int& co) {
    if constexpr (kRec) {
        ld_rec<T, kColNT>(c, o, vo, co);
    } else {
        vo = ld_nt(v + o);
        co = ld_col<kColNT>(c + o);
    }
}

// The row pointers of ld_slot for the row whose first slot is `base`.
template <typename T, bool kRec>
__device__ __forceinline__ void row_ptrs(const int* col, const T* val, int64_t base,
                                         const int*& c, const T*& v) {
    c = col + (kRec ? kRecInts<T> : 1) * base;
    v = kRec ? nullptr : val + base;
}

// Four slots o, o + d, o + 2 d, o + 3 d of a row (a lane's round of four
// entries): in the split layout the four values first, then the columns.
template <typename T, bool kColNT, bool kRec>
__device__ __forceinline__ void ld4(const int* __restrict__ c, const T* __restrict__ v,
                                    int64_t o, int64_t d, T& v0, T& v1, T& v2, T& v3, int& c0,
                                    int& c1, int& c2, int& c3) {
    if constexpr (kRec) {
        ld_rec<T, kColNT>(c, o, v0, c0);
        ld_rec<T, kColNT>(c, o + d, v1, c1);
        ld_rec<T, kColNT>(c, o + 2 * d, v2, c2);
        ld_rec<T, kColNT>(c, o + 3 * d, v3, c3);
    } else {
        v0 = ld_nt(v + o), v1 = ld_nt(v + o + d);
        v2 = ld_nt(v + o + 2 * d), v3 = ld_nt(v + o + 3 * d);
        c0 = ld_col<kColNT>(c + o), c1 = ld_col<kColNT>(c + o + d);
        c2 = ld_col<kColNT>(c + o + 2 * d), c3 = ld_col<kColNT>(c + o + 3 * d);
    }
}

// The long-row loop of ELLPACK-R records: U slots q0, q0 + 64, ... of the
// row whose first slot is bl (q clamped to its last slot, Ll - 1).
template <typename T, bool kColNT, int U>
__device__ __forceinline__ void ell_coop_load(const int* __restrict__ rec, int64_t bl, int64_t bh,
                                              int q0, int Ll, T* v, int* c) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        ld_rec<T, kColNT>(rec, bl + (int64_t)min(q0 + 64 * u, Ll - 1) * bh, v[u], c[u]);
}
// One round: gather x for the set (v, c) at q0, load the set at q0 + 64 U
// into (nv, nc), then add the first set's products of slots below Ll.
template <typename T, bool kColNT, int U>
__device__ __forceinline__ void ell_coop_round(const int* __restrict__ rec,
                                               const T* __restrict__ x, int64_t bl, int64_t bh,
                                               int q0, int Ll, const T* v, const int* c, T* nv,
                                               int* nc, T& p0, T& p1) {
    T xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) xv[u] = x[c[u]];
    ell_coop_load<T, kColNT, U>(rec, bl, bh, q0 + 64 * U, Ll, nv, nc);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool in = q0 + 64 * u < Ll;
        const T pr = fma(in ? v[u] : T(0), in ? xv[u] : T(0), T(0));
        if (u & 1)
            p1 += pr;
        else
            p0 += pr;
    }
}

template <typename T>
__device__ __forceinline__ T wave_max_len(T v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v = max(v, __shfl_xor(v, d));
    return __builtin_amdgcn_readfirstlane(v);
}

template <typename T, bool kColNT, bool kRec>
__global__ __launch_bounds__(256) void k_ell(int n, int64_t bh, int64_t bstride,
                                             const int* __restrict__ len,
                                             const int* __restrict__ perm,
                                             const int* __restrict__ col,
                                             const T* __restrict__ val, const T* __restrict__ x,
                                             T* __restrict__ y, T alpha, T beta) {
    const int64_t i = xcd_tile(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
    const bool valid = i < n;
    const int L = valid ? len[i] : 0;
    const int64_t base = ell_row_base(i, bh, bstride);
    const int* c;
    const T* v;
    row_ptrs<T, kRec>(col, val, base, c, v);
    T s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    const int M = wave_max_len(L);  // wave-uniform
    int j = 0;
    if (M <= kEllCoopMin) {
        for (; j + 4 <= L; j += 4) {
            const int64_t o = (int64_t)j * bh;
            T v0, v1, v2, v3;
            int c0, c1, c2, c3;
            ld4<T, kColNT, kRec>(c, v, o, bh, v0, v1, v2, v3, c0, c1, c2, c3);
            s0 = fma(v0, x[c0], s0);
            s1 = fma(v1, x[c1], s1);
            s2 = fma(v2, x[c2], s2);
            s3 = fma(v3, x[c3], s3);
        }
        for (; j < L; ++j) {
            T v0;
            int c0;
            ld_slot<T, kColNT, kRec>(c, v, (int64_t)j * bh, v0, c0);
            s0 = fma(v0, x[c0], s0);
        }
    } else {
        // lane per row in rounds of 4 while many lanes are busy (j is the
        // same in every lane)
        for (;;) {
            const uint64_t act = __ballot(j < L);
            if (act == 0 || (__popcll(act) <= kEllCoopLanes && M - j >= kEllCoopMin)) break;
            if (j + 4 <= L) {
                const int64_t o = (int64_t)j * bh;
                T v0, v1, v2, v3;
                int c0, c1, c2, c3;
                ld4<T, kColNT, kRec>(c, v, o, bh, v0, v1, v2, v3, c0, c1, c2, c3);
                s0 = fma(v0, x[c0], s0);
                s1 = fma(v1, x[c1], s1);
                s2 = fma(v2, x[c2], s2);
                s3 = fma(v3, x[c3], s3);
            } else {
                for (int u = j; u < L; ++u) {
                    T v0;
                    int c0;
                    ld_slot<T, kColNT, kRec>(c, v, (int64_t)u * bh, v0, c0);
                    s0 = fma(v0, x[c0], s0);
                }
            }
            j += 4;
        }
        // the rows still open, one at a time across the whole wave
        const int lane = threadIdx.x & 63;
        uint64_t open = __ballot(j < L);
        while (open) {
            const int l = __builtin_ctzll(open);
            open &= open - 1;
            const int Ll = __builtin_amdgcn_readlane(L, l);
            const int64_t il = i - lane + l;  // the wave's rows are consecutive
            const int64_t bl = ell_row_base(il, bh, bstride);
            T p0 = 0, p1 = 0;
            if constexpr (kRec) {
                // two sets of records in turn: a round gathers x for one set,
                // loads the next into the other, then adds the first.  Every
                // lane loads (lanes past the row's end read its last slot
                // again and add nothing), so no load waits on a lane test.
                constexpr int U = kEllRecUnroll;
                T va[U], vb[U];
                int ca[U], cb[U];
                int q0 = j + lane;
                ell_coop_load<T, kColNT, U>(col, bl, bh, q0, Ll, va, ca);
                for (;;) {
                    ell_coop_round<T, kColNT, U>(col, x, bl, bh, q0, Ll, va, ca, vb, cb, p0, p1);
                    q0 += 64 * U;
                    if (q0 - lane >= Ll) break;
                    ell_coop_round<T, kColNT, U>(col, x, bl, bh, q0, Ll, vb, cb, va, ca, p0, p1);
                    q0 += 64 * U;
                    if (q0 - lane >= Ll) break;
                }
            } else {
                for (int q0 = j + lane; q0 - lane < Ll; q0 += 64 * kEllCoopUnroll) {
                    T vv[kEllCoopUnroll];
                    int cc[kEllCoopUnroll];
#pragma unroll
                    for (int u = 0; u < kEllCoopUnroll; ++u) {
                        const int q = q0 + 64 * u;
                        vv[u] = q < Ll ? ld_nt(val + bl + (int64_t)q * bh) : T(0);
                        cc[u] = q < Ll ? ld_col<kColNT>(col + bl + (int64_t)q * bh) : 0;
                    }
#pragma unroll
                    for (int u = 0; u < kEllCoopUnroll; ++u) {
                        const T xv = q0 + 64 * u < Ll ? x[cc[u]] : T(0);
                        if (u & 1)
                            p1 = fma(vv[u], xv, p1);
                        else
                            p0 = fma(vv[u], xv, p0);
                    }
                }
            }
            const T tot = lane_read(group_sum<64>(p0 + p1), 0);
            if (lane == l) s0 += tot;
        }
    }
    if (!valid) return;
    const int64_t row = perm ? perm[i] : i;  // positions < n hold rows < n
    y[row] = axpby((s0 + s1) + (s2 + s3), alpha, beta, y + row);
}

// ELLPACK-R with x staged in LDS (banded matrices).  Workgroup g (1024
// threads) runs a contiguous range of row tiles of kEllWinTile rows, each
// thread taking positions r0 + tid + 1024 * h for h < kEllWinTile / 1024.
// Tile t sees the window [r0 - lead, r0 - lead + WL), so a row reads its x
// entries within about +-lead of itself from LDS and any others from global
// memory (a sorted ELL part only permutes rows inside a tile, which the
// window covers).  The window takes the whole LDS, so only 16 waves share a
// CU: each thread keeps 16 entries of each of its rows in flight per round
// (values, columns, then the x reads), and the elements entering the window
// for the next tile are loaded while the current tile computes.
template <typename T, bool kColNT, bool kRec>
__global__ __launch_bounds__(1024) void k_ell_win(int n, int64_t bh, int64_t bstride,
                                                  const int* __restrict__ len,
                                                  const int* __restrict__ perm,
                                                  const int* __restrict__ col,
                                                  const T* __restrict__ val,
                                                  const T* __restrict__ x, T* __restrict__ y,
                                                  T alpha, T beta, int64_t ntiles, int head) {
    constexpr int WL = WinLen<T>::value;
    constexpr int TILE = kEllWinTile;
    constexpr int H = TILE / 1024;  // rows per thread per tile
    constexpr int LEAD = (WL - TILE) / 2;
    // entries per round (records: addressed from a uniform base, so 16 fit
    // the registers as well)
    constexpr int B = kRec ? kEllWinRecB : 16;
    __shared__ T win[WL];
    const int64_t g = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t t0 = g * ntiles / gridDim.x, t1 = (g + 1) * ntiles / gridDim.x;
    const int tid = threadIdx.x;
    int64_t wlo = t0 * TILE - LEAD;
    window_fill<T, WL>(win, x, max<int64_t>(wlo, 0), min<int64_t>(wlo + WL, n));
    __syncthreads();
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t whi = wlo + WL;
        // the next tile's window gains [whi, whi + TILE): H elements per thread
        T pre[H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int64_t q = whi + tid + 1024 * h;
            pre[h] = (t + 1 < t1 && q < n) ? x[q] : T(0);
        }
        const int wl = (int)wlo;
        int L[H];
        int64_t row[H];
        int Lmax = 0;
#pragma unroll
        for (int h = 0; h < H; ++h) {
            row[h] = t * TILE + tid + 1024 * h;
            L[h] = row[h] < n ? min(len[row[h]], head) : 0;
            Lmax = max(Lmax, L[h]);
        }
        T sum[H][2] = {};
        for (int j = 0; j < Lmax; j += B) {
            // a round of B entries: every load of the round is issued before
            // the first use; lanes past their row's end issue none (so a
            // wave never touches lines holding only padding) and add zero
            T vv[H][B];
            int cc[H][B];
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const int64_t i = row[h] < n ? row[h] : 0;
                const int64_t base = ell_row_base(i, bh, bstride);
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int64_t jj = j + u;
                    if (j + u < L[h]) {
                        if constexpr (kRec) {
                            // ELLPACK-R is one block: slot j of row r is j bh + r,
                            // a uniform part plus the thread's place in the tile
                            const int* rb = col + kRecInts<T> * (t * TILE + jj * bh);
                            ld_rec_at<T, kColNT>(rb, (uint32_t)(tid + 1024 * h) *
                                                         (uint32_t)(4 * kRecInts<T>),
                                                 vv[h][u], cc[h][u]);
                        } else {
                            vv[h][u] = ld_nt(val + base + jj * bh);
                            cc[h][u] = ld_col<kColNT>(col + base + jj * bh);
                        }
                    } else {
                        vv[h][u] = T(0);
                        cc[h][u] = 0;
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < H; ++h) {
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const bool in = j + u < L[h];
                    // the slot read is always in range; global memory only
                    // for entries outside the window
                    T xv = win[cc[h][u] % WL];
                    if (in && (uint32_t)(cc[h][u] - wl) >= (uint32_t)WL) xv = x[cc[h][u]];
                    sum[h][u & 1] += in ? vv[h][u] * xv : T(0);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < H; ++h)
            if (row[h] < n) {
                const int64_t r = perm ? perm[row[h]] : row[h];
                y[r] = axpby(sum[h][0] + sum[h][1], alpha, beta, y + r);
            }
        if (t + 1 >= t1) break;
        lds_barrier();  // tile t is done with the slots reused now
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int64_t q = whi + tid + 1024 * h;
            if (q < n) win[q % WL] = pre[h];
        }
        lds_barrier();
        wlo += TILE;
    }
}

// ELLPACK with G wave groups per tile of 64 rows.  "Sparse Linear Algebra on
// AMD and NVIDIA GPUs -- The Race Is On" keeps the lanes of a group on one
// column of consecutive rows (coalesced, as in the one-lane-per-row kernel)
// and gives a row several groups to raise the parallelism of matrices with
// few, long rows.  Wave g takes the columns g, g + G, g + 2G, ... of its
// lanes' rows (four in flight); the G partial sums of a row meet in LDS.
template <typename T, int G, bool kColNT, bool kRec>
__global__ __launch_bounds__(64 * G) void k_ell_mg(int n, int64_t bh, int64_t bstride,
                                                   const int* __restrict__ len,
                                                   const int* __restrict__ perm,
                                                   const int* __restrict__ col,
                                                   const T* __restrict__ val,
                                                   const T* __restrict__ x, T* __restrict__ y,
                                                   T alpha, T beta, int64_t tile0) {
    __shared__ T part[G][kWave];
    const int lane = threadIdx.x & (kWave - 1), g = threadIdx.x / kWave;
    const int64_t i = (tile0 + xcd_tile(blockIdx.x, gridDim.x)) * kWave + lane;
    T s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    if (i < n) {
        const int L = len[i];
        const int64_t base = ell_row_base(i, bh, bstride);
        const int* c;
        const T* v;
        row_ptrs<T, kRec>(col, val, base, c, v);
        int j = g;
        for (; j + 3 * G < L; j += 4 * G) {
            const int64_t o = (int64_t)j * bh, d = (int64_t)G * bh;
            T v0, v1, v2, v3;
            int c0, c1, c2, c3;
            ld4<T, kColNT, kRec>(c, v, o, d, v0, v1, v2, v3, c0, c1, c2, c3);
            s0 = fma(v0, x[c0], s0);
            s1 = fma(v1, x[c1], s1);
            s2 = fma(v2, x[c2], s2);
            s3 = fma(v3, x[c3], s3);
        }
        for (; j < L; j += G) {
            T v0;
            int c0;
            ld_slot<T, kColNT, kRec>(c, v, (int64_t)j * bh, v0, c0);
            s0 = fma(v0, x[c0], s0);
        }
    }
    part[g][lane] = (s0 + s1) + (s2 + s3);
    __syncthreads();
    if (g == 0 && i < n) {
        T s = part[0][lane];
#pragma unroll
        for (int q = 1; q < G; ++q) s += part[q][lane];
        const int64_t row = perm ? perm[i] : i;
        y[row] = axpby(s, alpha, beta, y + row);
    }
}

template <typename T, bool kColNT, bool kRec>
static hipError_t run_ell_mg(const EllView& a, void* y, const void* x, double alpha,
                             double beta, hipStream_t stream) {
    const int64_t blocks = ((int64_t)a.n + kWave - 1) / kWave;
    if (a.groups != 16 && a.groups != 4) return hipErrorInvalidValue;
    const int64_t per = blocks_per_piece(kMaxLaunchItems, 64 * a.groups);
    for (int64_t b0 = 0; b0 < blocks; b0 += per) {
        const int64_t nb = std::min<int64_t>(blocks - b0, per);
        if (a.groups == 16)
            hipLaunchKernelGGL((k_ell_mg<T, 16, kColNT, kRec>), dim3((unsigned)nb), dim3(64 * 16),
                               0, stream, a.n, a.bh, a.bstride, a.len, a.perm, a.col,
                               (const T*)a.val, (const T*)x, (T*)y, (T)alpha, (T)beta, b0);
        else
            hipLaunchKernelGGL((k_ell_mg<T, 4, kColNT, kRec>), dim3((unsigned)nb), dim3(64 * 4), 0,
                               stream, a.n, a.bh, a.bstride, a.len, a.perm, a.col,
                               (const T*)a.val, (const T*)x, (T*)y, (T)alpha, (T)beta, b0);
    }
    return hipGetLastError();
}

template <typename T, bool kColNT, bool kRec>
static hipError_t run_ell(const EllView& a, void* y, const void* x, double alpha, double beta,
                          hipStream_t stream) {
    if (a.window) {
        const int64_t ntiles = ((int64_t)a.n + kEllWinTile - 1) / kEllWinTile;
        const int64_t g = std::min<int64_t>(ntiles, kWinGroups);
        hipLaunchKernelGGL((k_ell_win<T, kColNT, kRec>), dim3((unsigned)g), dim3(1024), 0, stream,
                           a.n, a.bh, a.bstride, a.len, a.perm, a.col, (const T*)a.val,
                           (const T*)x, (T*)y, (T)alpha, (T)beta, ntiles, a.head);
        return hipGetLastError();
    }
    if (a.groups > 1) return run_ell_mg<T, kColNT, kRec>(a, y, x, alpha, beta, stream);
    const int64_t blocks = ((int64_t)a.n + 255) / 256;
    hipLaunchKernelGGL((k_ell<T, kColNT, kRec>), dim3((unsigned)blocks), dim3(256), 0, stream, a.n,
                       a.bh, a.bstride, a.len, a.perm, a.col, (const T*)a.val, (const T*)x, (T*)y,
                       (T)alpha, (T)beta);
    return hipGetLastError();
}

hipError_t launch_ell(const EllView& a, bool f64, void* y, const void* x, double alpha,
                      double beta, hipStream_t stream) {
    if (a.n <= 0) return hipSuccess;
    if (a.rec) {
        if (f64)
            return a.col_nt ? run_ell<double, true, true>(a, y, x, alpha, beta, stream)
                            : run_ell<double, false, true>(a, y, x, alpha, beta, stream);
        return a.col_nt ? run_ell<float, true, true>(a, y, x, alpha, beta, stream)
                        : run_ell<float, false, true>(a, y, x, alpha, beta, stream);
    }
    if (f64)
        return a.col_nt ? run_ell<double, true, false>(a, y, x, alpha, beta, stream)
                        : run_ell<double, false, false>(a, y, x, alpha, beta, stream);
    return a.col_nt ? run_ell<float, true, false>(a, y, x, alpha, beta, stream)
                    : run_ell<float, false, false>(a, y, x, alpha, beta, stream);
}

// ELLPACK-R with the x window for a matrix with a few long rows: the window
// kernel takes every row's first `head` slots, then one wave per long row
// (the list holds the rows longer than head) takes the rest, with the long-row
// loop of the plain kernel, and adds alpha times its sum onto y (the row's
// only writer after the window kernel).  Up to kEllLongWaves waves, each
// taking rows w, w + waves, ...
constexpr int kEllLongWaves = 16384;
template <typename T, bool kColNT>
__global__ __launch_bounds__(256) void k_ell_long(int64_t bh, const int* __restrict__ len,
                                                  const int* __restrict__ rows, int64_t nlong,
                                                  int head, const int* __restrict__ rec,
                                                  const T* __restrict__ x, T* __restrict__ y,
                                                  T alpha) {
    constexpr int U = kEllRecUnroll;
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * 4;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < nlong; w += waves) {
        const int i = rows[w];
        const int Ll = len[i];  // > head
        T p0 = 0, p1 = 0;
        T va[U], vb[U];
        int ca[U], cb[U];
        int q0 = head + lane;
        ell_coop_load<T, kColNT, U>(rec, i, bh, q0, Ll, va, ca);
        for (;;) {
            ell_coop_round<T, kColNT, U>(rec, x, i, bh, q0, Ll, va, ca, vb, cb, p0, p1);
            q0 += 64 * U;
            if (q0 - lane >= Ll) break;
            ell_coop_round<T, kColNT, U>(rec, x, i, bh, q0, Ll, vb, cb, va, ca, p0, p1);
            q0 += 64 * U;
            if (q0 - lane >= Ll) break;
        }
        const T tot = group_sum<64>(p0 + p1);
        if (lane == 0) y[i] += alpha * tot;
    }
}

template <typename T, bool kColNT>
static hipError_t run_ell_long(const EllView& a, const int* rows, int64_t nlong, void* y,
                               const void* x, double alpha, hipStream_t stream) {
    const int64_t g = std::min<int64_t>((nlong + 3) / 4, kEllLongWaves / 4);
    hipLaunchKernelGGL((k_ell_long<T, kColNT>), dim3((unsigned)g), dim3(256), 0, stream, a.bh,
                       a.len, rows, nlong, a.head, a.col, (const T*)x, (T*)y, (T)alpha);
    return hipGetLastError();
}

hipError_t launch_ell_long(const EllView& a, const int* rows, int64_t nlong, bool f64, void* y,
                           const void* x, double alpha, hipStream_t stream) {
    if (nlong <= 0) return hipSuccess;
    if (!a.rec || a.perm) return hipErrorInvalidValue;  // ELLPACK-R records, rows in place
    if (f64)
        return a.col_nt ? run_ell_long<double, true>(a, rows, nlong, y, x, alpha, stream)
                        : run_ell_long<double, false>(a, rows, nlong, y, x, alpha, stream);
    return a.col_nt ? run_ell_long<float, true>(a, rows, nlong, y, x, alpha, stream)
                    : run_ell_long<float, false>(a, rows, nlong, y, x, alpha, stream);
}

// ---------------------------------------------------------------------------
// SELL-64: wave s runs slice s; lane l runs sorted row 64 s + l and writes
// y[perm[row]] (in the permuted basis y[row]).  Slices wider than
// kSellSplitWidth only get beta * y here; their columns are added by
// k_sell_chunks.
// ---------------------------------------------------------------------------
template <typename T, bool kColNT>
__global__ __launch_bounds__(256) void k_sell(int n, int nslices,
                                              const int64_t* __restrict__ slice_ptr,
                                              const int* __restrict__ len,
                                              const int* __restrict__ perm,
                                              const int* __restrict__ col,
                                              const T* __restrict__ val, const T* __restrict__ x,
                                              T* __restrict__ y, T alpha, T beta, bool permuted) {
    const int64_t s = xcd_tile(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    if (s >= nslices) return;
    const int lane = threadIdx.x & 63;
    const int64_t r = s * 64 + lane;
    const int64_t base = slice_ptr[s];
    const int64_t width = (slice_ptr[s + 1] - base) >> 6;
    int L = len[r];
    if (width > kSellSplitWidth) L = 0;
    const int* c = col + base + lane;
    const T* v = val + base + lane;
    T s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    int j = 0;
    for (; j + 4 <= L; j += 4) {
        const int64_t o = (int64_t)j * 64;
        const T v0 = ld_nt(v + o), v1 = ld_nt(v + o + 64);
        const T v2 = ld_nt(v + o + 128), v3 = ld_nt(v + o + 192);
        const int c0 = ld_col<kColNT>(c + o), c1 = ld_col<kColNT>(c + o + 64);
        const int c2 = ld_col<kColNT>(c + o + 128), c3 = ld_col<kColNT>(c + o + 192);
        s0 = fma(v0, x[c0], s0);
        s1 = fma(v1, x[c1], s1);
        s2 = fma(v2, x[c2], s2);
        s3 = fma(v3, x[c3], s3);
    }
    for (; j < L; ++j) {
        const int64_t o = (int64_t)j * 64;
        s0 = fma(ld_nt(v + o), x[ld_col<kColNT>(c + o)], s0);
    }
    if (r < n) {
        const int64_t row = permuted ? r : perm[r];
        y[row] = axpby((s0 + s1) + (s2 + s3), alpha, beta, y + row);
    }
}

// one wave per column chunk (slice, j0, j1) of a split slice
template <typename T, bool kColNT>
__global__ __launch_bounds__(256) void k_sell_chunks(int n, int nchunks,
                                                     const int4* __restrict__ chunks,
                                                     const int64_t* __restrict__ slice_ptr,
                                                     const int* __restrict__ len,
                                                     const int* __restrict__ perm,
                                                     const int* __restrict__ col,
                                                     const T* __restrict__ val,
                                                     const T* __restrict__ x, T* __restrict__ y,
                                                     T alpha, bool permuted) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nchunks) return;
    const int4 ch = chunks[w];
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)ch.x * 64 + lane;
    const int L = min(len[r], ch.z);
    const int* c = col + slice_ptr[ch.x] + lane;
    const T* v = val + slice_ptr[ch.x] + lane;
    T s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    int j = ch.y;
    for (; j + 4 <= L; j += 4) {
        const int64_t o = (int64_t)j * 64;
        const T v0 = ld_nt(v + o), v1 = ld_nt(v + o + 64);
        const T v2 = ld_nt(v + o + 128), v3 = ld_nt(v + o + 192);
        const int c0 = ld_col<kColNT>(c + o), c1 = ld_col<kColNT>(c + o + 64);
        const int c2 = ld_col<kColNT>(c + o + 128), c3 = ld_col<kColNT>(c + o + 192);
        s0 = fma(v0, x[c0], s0);
        s1 = fma(v1, x[c1], s1);
        s2 = fma(v2, x[c2], s2);
        s3 = fma(v3, x[c3], s3);
    }
    for (; j < L; ++j) {
        const int64_t o = (int64_t)j * 64;
        s0 = fma(ld_nt(v + o), x[ld_col<kColNT>(c + o)], s0);
    }
    if (r < n && ch.y < L) atomic_add(y + (permuted ? r : perm[r]), alpha * ((s0 + s1) + (s2 + s3)));
}

// One row's entries [j0, j1) of a SELL-64 slice (slots base + 64 j) with x
// from the LDS window where the column lies in it (window [wl, wl + WL),
// element q at slot q mod WL) and from global memory otherwise: rounds of
// B entries, every load of a round issued before the first use.
template <typename T, bool kColNT, int WL>
__device__ __forceinline__ T sell_row_win(int64_t base, int j0, int j1, const int* __restrict__ col,
                                          const T* __restrict__ val, const T* __restrict__ x,
                                          const T* win, int wl) {
    constexpr int B = 16;
    T s0 = 0, s1 = 0;
    for (int j = j0; j < j1; j += B) {
        T vv[B];
        int cc[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int64_t o = base + (int64_t)(j + u) * 64;
            if (j + u < j1) {
                vv[u] = ld_nt(val + o);
                cc[u] = ld_col<kColNT>(col + o);
            } else {
                vv[u] = T(0);
                cc[u] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const bool in = j + u < j1;
            T xv = win[cc[u] % WL];  // the slot read is always in range
            if (in && (uint32_t)(cc[u] - wl) >= (uint32_t)WL) xv = x[cc[u]];
            if (u & 1)
                s1 += in ? vv[u] * xv : T(0);
            else
                s0 += in ? vv[u] * xv : T(0);
        }
    }
    return s0 + s1;
}

// The same over every fourth column: entries j0, j0 + 4, ... below j1.
template <typename T, bool kColNT, int WL>
__device__ __forceinline__ T sell_row4_win(int64_t base, int j0, int j1,
                                           const int* __restrict__ col, const T* __restrict__ val,
                                           const T* __restrict__ x, const T* win, int wl) {
    constexpr int B = 16;
    T s0 = 0, s1 = 0;
    for (int j = j0; j < j1; j += 4 * B) {
        T vv[B];
        int cc[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int64_t o = base + (int64_t)(j + 4 * u) * 64;
            if (j + 4 * u < j1) {
                vv[u] = ld_nt(val + o);
                cc[u] = ld_col<kColNT>(col + o);
            } else {
                vv[u] = T(0);
                cc[u] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const bool in = j + 4 * u < j1;
            T xv = win[cc[u] % WL];
            if (in && (uint32_t)(cc[u] - wl) >= (uint32_t)WL) xv = x[cc[u]];
            if (u & 1)
                s1 += in ? vv[u] * xv : T(0);
            else
                s0 += in ? vv[u] * xv : T(0);
        }
    }
    return s0 + s1;
}

// SELL-64 with x staged in LDS.  Workgroup g (1024 threads) runs a
// contiguous range of tiles of kEllWinTile sorted positions; the window of
// tile t is placed as the ELL window of rows [t kEllWinTile, (t + 1)
// kEllWinTile) (with the rows sorted inside windows that divide the tile,
// those are exactly the tile's rows).  Wave w takes slice (tile slices) t +
// w, one lane per sorted row: the whole row in a narrow slice, written as
// alpha s + beta y; the first kSellWinHead columns in a wide slice, added
// into y.  Then the waves take the chunks of the tile's wide slices in turn
// (chunk c by wave c mod 16): a chunk is 16 rows of a slice over
// kSellWinChunk columns, lane 16 g + i on row i and the columns g, g + 4, ...
// (each 16 lanes read one line of a column), the four partial sums of a row
// joined across the lanes, and the row sums added into y.  The rows of wide
// slices were scaled by beta before the launch (k_sell_wide_beta), so no
// ordering between the waves is needed.  A zero sum of a wide slice's row is
// left out unless alpha is not finite (alpha * 0 is then NaN).
template <typename T, bool kColNT>
__global__ __launch_bounds__(1024) void k_sell_win(int n, int nslices,
                                                   const int64_t* __restrict__ slice_ptr,
                                                   const int* __restrict__ len,
                                                   const int* __restrict__ perm,
                                                   const int* __restrict__ col,
                                                   const T* __restrict__ val,
                                                   const int* __restrict__ chunk_off,
                                                   const int4* __restrict__ chunks,
                                                   const T* __restrict__ x, T* __restrict__ y,
                                                   T alpha, T beta, bool permuted,
                                                   int64_t ntiles) {
    constexpr int WL = WinLen<T>::value;
    constexpr int TILE = kEllWinTile;
    constexpr int SPT = TILE / 64;  // slices per tile (one per wave)
    constexpr int LEAD = (WL - TILE) / 2;
    static_assert(SPT == 16, "one slice per wave of a 1024-thread workgroup");
    __shared__ T win[WL];
    const int64_t g = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t t0 = g * ntiles / gridDim.x, t1 = (g + 1) * ntiles / gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool fin = alpha - alpha == T(0);
    int64_t wlo = t0 * TILE - LEAD;
    window_fill<T, WL>(win, x, max<int64_t>(wlo, 0), min<int64_t>(wlo + WL, n));
    __syncthreads();
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t whi = wlo + WL;
        // the next tile's window gains [whi, whi + TILE): one element per thread
        const int64_t q = whi + tid;
        const T pre = (t + 1 < t1 && q < n) ? x[q] : T(0);
        const int wl = (int)wlo;
        const int64_t sl = t * SPT + wave;
        if (sl < nslices) {
            const int64_t base = slice_ptr[sl];
            const bool wide = ((slice_ptr[sl + 1] - base) >> 6) > kSellWinWide;
            const int64_t p = sl * 64 + lane;
            const int L = len[p];
            const int La = wide ? min(L, kSellWinHead) : L;
            const T sum = sell_row_win<T, kColNT, WL>(base + lane, 0, La, col, val, x, win, wl);
            if (p < n) {
                const int64_t r = permuted ? p : perm[p];
                if (!wide)
                    y[r] = axpby(sum, alpha, beta, y + r);
                else if (sum != T(0) || !fin)
                    atomic_add(y + r, alpha * sum);
            }
        }
        // the chunks of the tile's wide slices: lane = 16 g + i reads row
        // 16 (group) + i at the columns j0 + g, j0 + g + 4, ...
        const int64_t sl0 = t * SPT < nslices ? t * SPT : nslices;
        const int64_t sl1 = (t + 1) * SPT < nslices ? (t + 1) * SPT : nslices;
        const int c0 = chunk_off[sl0], c1 = chunk_off[sl1];
        for (int c = c0 + wave; c < c1; c += SPT) {
            const int4 ch = chunks[c];
            const int rr = ch.w * 16 + (lane & 15), cg = lane >> 4;
            const int64_t p = (int64_t)ch.x * 64 + rr;
            const int Lb = min(len[p], ch.z);
            T sum = sell_row4_win<T, kColNT, WL>(slice_ptr[ch.x] + rr, ch.y + cg, Lb, col, val, x,
                                                 win, wl);
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            if (cg == 0 && ch.y < Lb) {  // rows of the group that reach the chunk (p < n)
                const int64_t r = permuted ? p : perm[p];
                if (sum != T(0) || !fin) atomic_add(y + r, alpha * sum);
            }
        }
        if (t + 1 >= t1) break;
        lds_barrier();  // tile t is done with the slots reused now
        if (q < n) win[q % WL] = pre;
        lds_barrier();
        wlo += TILE;
    }
}

// y = beta y at the rows of the slices wider than kSellWinWide (one wave per
// slice), before k_sell_win adds their sums with atomics
template <typename T>
__global__ __launch_bounds__(256) void k_sell_wide_beta(int n, int nslices,
                                                        const int64_t* __restrict__ slice_ptr,
                                                        const int* __restrict__ perm,
                                                        T* __restrict__ y, T beta,
                                                        bool permuted) {
    const int64_t sl = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (sl >= nslices || ((slice_ptr[sl + 1] - slice_ptr[sl]) >> 6) <= kSellWinWide) return;
    const int64_t p = sl * 64 + (threadIdx.x & 63);
    if (p >= n) return;
    const int64_t r = permuted ? p : perm[p];
    y[r] = beta == T(0) ? T(0) : beta * y[r];
}

// setup: chunks of each slice (sell_slice_chunks)
__global__ void k_sell_chunk_count(int64_t nslices, const int64_t* __restrict__ slice_ptr,
                                   const int* __restrict__ len, int split, int head, int chunk,
                                   bool groups, int* __restrict__ cnt) {
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nslices;
         q += (int64_t)gridDim.x * blockDim.x)
        cnt[q] = sell_slice_chunks(q, slice_ptr, len, split, head, chunk, groups, nullptr);
}

__global__ void k_sell_chunk_fill(int64_t nslices, const int64_t* __restrict__ slice_ptr,
                                  const int* __restrict__ len, const int* __restrict__ chunk_off,
                                  int split, int head, int chunk, bool groups,
                                  int4* __restrict__ chunks) {
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nslices;
         q += (int64_t)gridDim.x * blockDim.x)
        sell_slice_chunks(q, slice_ptr, len, split, head, chunk, groups, chunks + chunk_off[q]);
}

hipError_t launch_sell_chunk_count(int64_t nslices, const int64_t* slice_ptr, const int* len,
                                   int split, int head, int chunk, bool groups, int* cnt,
                                   hipStream_t stream) {
    if (nslices <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((nslices + 255) / 256, 65536);
    hipLaunchKernelGGL(k_sell_chunk_count, dim3((unsigned)blocks), dim3(256), 0, stream, nslices,
                       slice_ptr, len, split, head, chunk, groups, cnt);
    return hipGetLastError();
}

hipError_t launch_sell_chunk_fill(int64_t nslices, const int64_t* slice_ptr, const int* len,
                                  const int* chunk_off, int split, int head, int chunk,
                                  bool groups, int4* chunks, hipStream_t stream) {
    if (nslices <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((nslices + 255) / 256, 65536);
    hipLaunchKernelGGL(k_sell_chunk_fill, dim3((unsigned)blocks), dim3(256), 0, stream, nslices,
                       slice_ptr, len, chunk_off, split, head, chunk, groups, chunks);
    return hipGetLastError();
}

template <typename T, bool kColNT>
static hipError_t run_sell(const SellView& a, void* y, const void* x, double alpha, double beta,
                           hipStream_t stream) {
    const int64_t blocks = ((int64_t)a.nslices + 3) / 4;
    if (blocks == 0) return hipSuccess;
    if (a.window) {
        if (a.nchunks > 0) {
            hipLaunchKernelGGL(k_sell_wide_beta<T>, dim3((unsigned)blocks), dim3(256), 0, stream,
                               a.n, a.nslices, a.slice_ptr, a.perm, (T*)y, (T)beta, a.permuted);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int64_t ntiles = ((int64_t)a.nslices * 64 + kEllWinTile - 1) / kEllWinTile;
        const int64_t g = std::min<int64_t>(ntiles, kWinGroups);
        hipLaunchKernelGGL((k_sell_win<T, kColNT>), dim3((unsigned)g), dim3(1024), 0, stream, a.n,
                           a.nslices, a.slice_ptr, a.len, a.perm, a.col, (const T*)a.val,
                           a.chunk_off, a.chunks, (const T*)x, (T*)y, (T)alpha, (T)beta,
                           a.permuted, ntiles);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_sell<T, kColNT>), dim3((unsigned)blocks), dim3(256), 0, stream, a.n,
                       a.nslices, a.slice_ptr, a.len, a.perm, a.col, (const T*)a.val,
                       (const T*)x, (T*)y, (T)alpha, (T)beta, a.permuted);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nchunks == 0) return e;
    hipLaunchKernelGGL((k_sell_chunks<T, kColNT>), dim3((unsigned)((a.nchunks + 3) / 4)),
                       dim3(256), 0, stream, a.n, a.nchunks, a.chunks, a.slice_ptr, a.len, a.perm,
                       a.col, (const T*)a.val, (const T*)x, (T*)y, (T)alpha, a.permuted);
    return hipGetLastError();
}

hipError_t launch_sell(const SellView& a, bool f64, void* y, const void* x, double alpha,
                       double beta, hipStream_t stream) {
    if (f64)
        return a.col_nt ? run_sell<double, true>(a, y, x, alpha, beta, stream)
                        : run_sell<double, false>(a, y, x, alpha, beta, stream);
    return a.col_nt ? run_sell<float, true>(a, y, x, alpha, beta, stream)
                    : run_sell<float, false>(a, y, x, alpha, beta, stream);
}

// dst[r] = src[perm[r]] or dst[perm[r]] = src[r] (vectors between the
// caller's basis and the sorted one)
template <typename T>
__global__ __launch_bounds__(256) void k_permute(int64_t n, T* __restrict__ dst,
                                                 const T* __restrict__ src,
                                                 const int* __restrict__ perm, bool inverse) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n; r += stride) {
        if (inverse)
            dst[perm[r]] = src[r];
        else
            dst[r] = src[perm[r]];
    }
}

hipError_t launch_permute(int64_t n, bool f64, void* dst, const void* src, const int* perm,
                          bool inverse, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
    if (f64)
        hipLaunchKernelGGL(k_permute<double>, dim3((unsigned)blocks), dim3(256), 0, stream, n,
                           (double*)dst, (const double*)src, perm, inverse);
    else
        hipLaunchKernelGGL(k_permute<float>, dim3((unsigned)blocks), dim3(256), 0, stream, n,
                           (float*)dst, (const float*)src, perm, inverse);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// reference copy (the bandwidth the apply kernels are measured against):
// 16-byte nontemporal loads and stores
// ---------------------------------------------------------------------------
typedef int copy_vec_t __attribute__((ext_vector_type(4)));

// one 16-byte element per thread over a grid covering the whole buffer, no
// loop: measured the fastest copy shape (1-4 GiB: 6.4-6.5 TB/s, against
// 5.9 TB/s for four elements per lane in a grid-stride loop)
__global__ __launch_bounds__(256) void k_copy(copy_vec_t* __restrict__ dst,
                                              const copy_vec_t* __restrict__ src, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// read-only stream (the bandwidth of the loads alone): four 16-byte
// nontemporal loads per lane in flight over a grid of 16,384 workgroups (the
// fastest read shape measured: 7.0-7.1 TB/s); the data only feeds a value
// that is stored when it equals a constant, so the loads stay
__device__ int g_read_sink;
constexpr int kReadUnroll = 4;
constexpr int64_t kReadGroups = 16384;
__global__ __launch_bounds__(256) void k_read(const copy_vec_t* __restrict__ src, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256 * kReadUnroll;
    int acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; i < n16;
         i += stride) {
        copy_vec_t t[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            t[u] = i + u * 256 < n16 ? __builtin_nontemporal_load(src + i + u * 256)
                                     : copy_vec_t{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= t[u].x ^ t[u].y ^ t[u].z ^ t[u].w;
    }
    if (acc == 0x5a5a5a5a) g_read_sink = acc;
}

__global__ void k_copy_tail(char* dst, const char* src, int64_t from, int64_t bytes) {
    const int64_t i = from + threadIdx.x;
    if (i < bytes) dst[i] = src[i];
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    if (!dst) {  // read only (whole 16-byte words)
        if (n16 > 0) {
            const int64_t g = std::min<int64_t>((n16 + 256 * kReadUnroll - 1) / (256 * kReadUnroll),
                                                kReadGroups);
            hipLaunchKernelGGL(k_read, dim3((unsigned)g), dim3(256), 0, stream,
                               (const copy_vec_t*)src, n16);
        }
        return hipGetLastError();
    }
    // pieces of at most kMaxLaunchItems threads (the dispatch limit)
    for (int64_t off = 0; off < n16; off += kMaxLaunchItems) {
        const int64_t cnt = std::min<int64_t>(n16 - off, kMaxLaunchItems);
        hipLaunchKernelGGL(k_copy, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                           (copy_vec_t*)dst + off, (const copy_vec_t*)src + off, cnt);
    }
    if (bytes % 16)
        hipLaunchKernelGGL(k_copy_tail, dim3(1), dim3(16), 0, stream, (char*)dst,
                           (const char*)src, n16 * 16, bytes);
    return hipGetLastError();
}

}  // namespace spmv
