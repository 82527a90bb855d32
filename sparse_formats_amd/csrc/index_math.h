// Index arithmetic of the SpMV kernels, written as host-and-device functions:
// the kernels call these, and the host tests run the same code at the
// boundaries of the 32-bit and 64-bit ranges (rows and entries near 2^31,
// slot offsets past 2^32, grids at the dispatch limit).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spmv {

// MI355X dispatches workgroup b of a grid to XCD (b mod 8).  Each XCD has its
// own L2, so neighbouring tiles (which share x entries of a banded matrix)
// should run on the same XCD.  This maps dispatch order to a logical tile
// index such that XCD k works on the k-th contiguous eighth of the tiles (a
// bijection of [0, grid)).
__host__ __device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t grid) {
    const int64_t xcd = b & 7, idx = b >> 3;
    const int64_t per = grid >> 3, rem = grid & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// First slot of the row at position i of an ELL array stored in column-major
// blocks of bh rows (bstride = width * bh slots per block); entry j of the
// row is at that slot + j * bh.
__host__ __device__ __forceinline__ int64_t ell_row_base(int64_t i, int64_t bh, int64_t bstride) {
    return (i / bh) * bstride + i % bh;
}

// Largest r in [lo, hi] with ptr[r] <= e, given ptr[lo] <= e < ptr[hi + 1]
// (the row holding entry e).  The midpoint is taken without lo + hi, which
// passes 2^31 for the last rows of the largest matrices.  `ptr` is a pointer
// or anything indexable.
template <typename Ptr>
__host__ __device__ __forceinline__ int row_of(const Ptr& ptr, int lo, int hi, int64_t e) {
    while (lo < hi) {
        const int m = lo + ((hi - lo + 1) >> 1);
        if ((int64_t)ptr[m] <= e)
            lo = m;
        else
            hi = m - 1;
    }
    return lo;
}

// A lane run of entries starts in row `cur`; the next run starts in row
// `hi`.  The index of the start of row cur + 1 + j, clamped to row hi + 1
// (cur + 1 + j itself may pass 2^31 near the last rows).
__host__ __device__ __forceinline__ int run_next_start(int cur, int hi, int j) {
    return cur + 1 + (j < hi - cur ? j : hi - cur);
}

// Column-slice CSR.  Rows are cut into ranges, each summed by one workgroup
// in LDS; the entries of range r with columns in slice b form tile (r, b).
// Candidate range start for target r of R0: the row holding entry
// r * nnz / R0 (ranges of about equal entry counts); 0 for r = 0, n for r >=
// R0.  Needs n >= 1 and nnz < 2^31; r * nnz stays below 2^63 for r < 2^32.
template <typename Ptr>
__host__ __device__ __forceinline__ int xblk_bound(const Ptr& ptr, int n, int64_t nnz, int64_t r,
                                                   int64_t R0) {
    if (r >= R0) return n;
    if (r == 0) return 0;
    return row_of(ptr, 0, n - 1, r * nnz / R0);
}

// The ranges from the candidate starts cand[0..m] (non-decreasing, cand[0] =
// 0, cand[m] = n): every stretch between distinct candidates is cut into
// equal pieces of at most `cap` rows.  Writes the range starts and n to
// out[0..R] when out is given; returns R.
__host__ __device__ __forceinline__ int64_t xblk_split_ranges(const int* cand, int64_t m, int cap,
                                                              int* out) {
    int64_t R = 0;
    for (int64_t k = 0; k < m; ++k) {
        const int lo = cand[k], hi = cand[k + 1];
        if (hi <= lo) continue;
        const int64_t rows = (int64_t)hi - lo, pieces = (rows + cap - 1) / cap;
        for (int64_t p = 0; p < pieces; ++p, ++R)
            if (out) out[R] = lo + (int)(rows * p / pieces);
    }
    if (out) out[R] = m > 0 ? cand[m] : 0;
    return R;
}

// Tile of an entry of column c in the range of rows [rb, rb + nr): the
// range's band tile kS when c lies within `band` columns of those rows (none
// when band < 0), else its column slice c / width (< kS).
__host__ __device__ __forceinline__ int xblk_tile(int64_t c, int64_t rb, int64_t nr, int64_t band,
                                                  int64_t width, int kS) {
    return band >= 0 && c >= rb - band && c < rb + nr + band ? kS : (int)(c / width);
}

// Half-width of a band tile whose entries pack their column, less the
// band's first column rb - band, above a row offset of lbits bits into one
// 32-bit word: rb - band .. rb + nr + band spans at most 2^(32 - lbits)
// columns for ranges of nr <= cap rows.
__host__ __device__ constexpr int64_t xblk_band(int lbits, int64_t cap) {
    return (((int64_t)1 << (32 - lbits)) - cap) / 2;
}
// The packed word of a band entry (column c, row offset lr) of the range
// starting at row rb, and its column back.
__host__ __device__ __forceinline__ uint32_t xblk_pack(int64_t c, int64_t rb, int64_t band, int lr,
                                                       int lbits) {
    return ((uint32_t)(c - (rb - band)) << lbits) | (uint32_t)lr;
}
__host__ __device__ __forceinline__ int64_t xblk_unpack_col(uint32_t w, int64_t rb, int64_t band,
                                                            int lbits) {
    return rb - band + (int64_t)(w >> lbits);
}

// Position of the count of row i in slice b (kS slices) inside the count
// array, whose scan gives every entry's place: range r of rows [rb, rb + nr)
// owns kS * nr consecutive counts, slice-major (slice b's counts of the
// range's rows in row order).  The tile (r, b) therefore starts at position
// xblk_slot(rb, nr, b, rb, kS).
__host__ __device__ __forceinline__ int64_t xblk_slot(int64_t rb, int64_t nr, int b, int64_t i,
                                                      int kS) {
    return (int64_t)kS * rb + (int64_t)b * nr + (i - rb);
}

// LDS window of x: element q at slot q mod WL; q lies in the window
// [wl, wl + WL).  Both need wl > -WL and q < 2^31 - WL (the window
// conversions take only n < 2^31 - 1 - 2 WL), so q - wl cannot overflow.
// The window kernels write this test out in place, as (uint32_t)(q - wl) >=
// WL for a load from global memory: called through a function the compiler
// waited for each of a round's far loads in turn instead of for all of them
// together (measured: HYB apply on the FEM block 1.25 -> 1.43 ms).
__host__ __device__ __forceinline__ bool in_window(int q, int wl, int WL) {
    return (uint32_t)(q - wl) < (uint32_t)WL;
}

// Column chunks of SELL-64 slice q: a slice wider than `split` columns is
// cut into chunks of `chunk` columns from column `head` on -- with `groups`,
// for each group of 16 rows up to the group's longest row; otherwise for all
// rows up to the slice's width.  With `out` the chunks are written from
// out[0] on as (q, j0, j1, group); the count is returned.
__host__ __device__ __forceinline__ int sell_slice_chunks(int64_t q, const int64_t* slice_ptr,
                                                 const int* len, int split, int head, int chunk,
                                                 bool groups, int4* out) {
    const int w = (int)((slice_ptr[q + 1] - slice_ptr[q]) >> 6);
    if (w <= split) return 0;
    int c = 0;
    for (int g = 0; g < (groups ? 4 : 1); ++g) {
        int reach = w;  // columns this group of rows needs
        if (groups) {
            reach = 0;
            for (int i = 0; i < 16; ++i) {
                const int l = len[q * 64 + g * 16 + i];
                reach = l > reach ? l : reach;
            }
        }
        for (int j0 = head; j0 < reach; j0 += chunk, ++c)
            if (out) out[c] = make_int4((int)q, j0, j0 + chunk < reach ? j0 + chunk : reach, g);
    }
    return c;
}

// Launches whose grid grows with the rows are split into pieces of at most
// max_items work-items: the blocks per piece, for blocks of `threads`.
__host__ __device__ __forceinline__ int64_t blocks_per_piece(int64_t max_items, int threads) {
    return max_items / threads;
}

}  // namespace spmv
