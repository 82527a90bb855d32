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
// default SELL-64 sort window (rows): the sort moves rows less than this
constexpr int kSellSortWindow = 8192;

// Tail entries per lane of the load-balanced tail kernel (one wave takes
// 64 * kTailPerLane consecutive entries).
constexpr int kTailPerLane = 8;
constexpr int kTailChunk = 64 * kTailPerLane;

// LDS window of x: one workgroup of 1024 threads per CU stages the x
// entries near its rows in the whole 160 KiB of LDS, as a circular buffer
// (element q at slot q mod WinLen) that slides forward with the rows.
constexpr int kWinBytes = 160 * 1024;
template <typename T>
struct WinLen {
    static constexpr int value = kWinBytes / (int)sizeof(T);
};
// ELL: row tiles of kEllWinTile rows (one per thread), the window centred
// on the tile
constexpr int kEllWinTile = 1024;
template <typename T>
struct EllWinLead {
    static constexpr int value = (WinLen<T>::value - kEllWinTile) / 2;
};
// tail: a step's rows follow its first row, so the window leads by less
template <typename T>
struct WinLead {
    static constexpr int value = WinLen<T>::value / 2 - 1024;
};
// tail window kernel: chunks per wave and per workgroup step (16 waves)
constexpr int kTailChunksPerWave = 4;
constexpr int kTailStepChunks = 16 * kTailChunksPerWave;
// persistent workgroups launched for a window kernel: one per CU (the
// window takes a CU's whole LDS), work spread evenly over them
constexpr int kWinGroups = 256;

struct CsrView {
    int n;
    int nnz;               // col and val hold 16 bytes past entry nnz - 1
    const int* rowptr;
    const int* col;
    const void* val;
    const int* row_map = nullptr;  // output row of each row (nullptr: itself)
};

// ELL arrays are stored in blocks of `bh` rows, each block column by column:
// slot (i, j) at (i / bh) * bstride + j * bh + i % bh with bstride = width *
// bh.  ELLPACK-R uses one block of all (padded) rows, i.e. the global
// column-major layout; the ELL part of HYB/HEC uses blocks of kEllBlock rows
// so that a tile of rows reads one contiguous slab (a few pages) instead of
// `width` places a whole matrix height apart.
constexpr int kEllBlock = 1024;
// ELL with several wave groups per row tile is used (by default) when the
// matrix has too few 64-row tiles to fill the GPU: 4 groups below
// kEllGroupTiles tiles, 16 below kEllGroupTiles / 4 (measured on rows of
// hundreds of entries: 64 tiles 4.3x faster with 16 groups, 313 tiles 1.7x
// with 4, 1024 tiles best with one)
constexpr int64_t kEllGroupTiles = 512;

struct EllView {
    int n;
    int64_t bh;       // rows per block = distance between a row's slots
    int64_t bstride;  // slots per block (width * bh)
    int width;        // slots per row (every row's slots j < width exist)
    const int* len;   // [padded rows], by position
    const int* perm;  // row at each position, or nullptr (position = row)
    const int* col;   // columns, or the slot records (value, column) when rec
    const void* val;  // values (nullptr when rec)
    bool rec;         // records: kRecInts<T> ints per slot in col (ELLPACK-R)
    bool window;      // stage x in LDS (banded matrices)
    int groups;       // wave groups per 64-row tile (1, 4 or 16; without the window)
    bool col_nt = true;  // col (or the records) read without caching (else kept in the caches)
    int head = 0x7fffffff;  // the window kernel takes each row's first head slots
};
// ELLPACK-R records past the window kernel's head: one wave per row of
// `rows` (nlong rows longer than a.head) adds alpha times the sum of its
// slots a.head .. len - 1 onto y
hipError_t launch_ell_long(const EllView& a, const int* rows, int64_t nlong, bool f64, void* y,
                           const void* x, double alpha, hipStream_t stream);

// SELL-64 with x staged in LDS: rows sorted inside windows that divide
// kEllWinTile, so a tile of kEllWinTile sorted positions (kEllWinTile / 64
// slices) holds the rows of one row range and the ELL window applies.  A
// slice wider than kSellWinWide columns ("wide") is read by its wave only up
// to kSellWinHead; its further columns are cut into chunks of kSellWinChunk
// columns for each group of 16 rows that reaches past kSellWinHead.  The
// tile's waves take the chunks in turn: 16 lanes per row group and four
// columns at a time (each 16 lanes read one whole line of a column), then
// each row's sum is added into y with an atomic (the wide slices' rows are
// scaled by beta first).
constexpr int kSellWinWide = 128;
constexpr int kSellWinHead = 64;
constexpr int kSellWinChunk = 128;
// default sort window of SELL-64 with the LDS window (one tile)
constexpr int kSellWinSortWindow = kEllWinTile;

struct SellView {
    int n;
    int nslices;
    const int64_t* slice_ptr;  // [nslices + 1]
    const int* len;            // [64 * nslices], sorted order
    const int* perm;           // [n]
    const int* col;
    const void* val;
    int nchunks;               // column chunks of split slices
    const int4* chunks;        // (slice, j0, j1, row group), ordered by slice
                               // (row group: rows 16 g .. 16 g + 15 with the
                               // window; 0 without)
    const int* chunk_off;      // [nslices + 1]: first chunk of each slice
    bool permuted;             // y in sorted order (permuted basis)
    bool col_nt = true;        // col read without caching (else kept in the caches)
    bool window = false;       // x staged in LDS (chunks are then the wide
                               // slices' columns past kSellWinHead)
};
// column chunks of the slices of a SELL layout, built on the device: a slice
// wider than `split` columns gets chunks of `chunk` columns from column
// `head` on.  Without the window (groups false: split kSellSplitWidth, head
// 0, chunk kSellChunk) every row of the slice is in each chunk; with it
// (kSellWinWide, kSellWinHead, kSellWinChunk, groups true) each group of 16
// rows gets the chunks up to its own longest row.  len: [64 nslices] row
// lengths in sorted order.  cnt: [nslices] chunks of each slice.
hipError_t launch_sell_chunk_count(int64_t nslices, const int64_t* slice_ptr, const int* len,
                                   int split, int head, int chunk, bool groups, int* cnt,
                                   hipStream_t stream);
hipError_t launch_sell_chunk_fill(int64_t nslices, const int64_t* slice_ptr, const int* len,
                                  const int* chunk_off, int split, int head, int chunk,
                                  bool groups, int4* chunks, hipStream_t stream);

struct TailView {
    int n;
    int64_t nnz;
    const int* row;        // COO row ids (HYB) or nullptr
    const int* ptr;        // CSR tail pointer over the tail's rows or nullptr
                           // (HEC: only the rows with tail entries)
    const int* run_row;    // CSR tail: row (index into ptr) of the first entry of
                           // each lane run of kTailPerLane entries, plus the
                           // last row at the end
    const int* row_map;    // HEC: matrix row of each tail row; nullptr: identity
    const int* col;
    const void* val;
    bool window;           // stage x in LDS (banded matrices)
};

// CSR by column slices: the columns cut into kXbBlocks slices of `width`
// columns, the rows into ranges of at most kXbCap<T> rows (about equal
// entry counts).  One workgroup of kXbThreads sums a range in LDS, tile by
// tile: tile (r, b) holds the entries of range r with columns in slice b,
// except those within `band` columns of the range's rows, which form its
// last tile (r, kXbBlocks); each tile is stored together, by column, with
// each entry's row offset inside its range (a band tile packs both into its
// column word: band + nr + band < 2^(32 - kXbRowBits) columns).
constexpr int kXbBlocks = 8;
constexpr int kXbTiles = kXbBlocks + 1;  // the slices, then the range's band
constexpr int kXbThreads = 1024;
constexpr int kXbGroups = 256;            // persistent workgroups, one per CU
constexpr int kXbLdsBytes = 160 * 1024;   // the range's partial sums
template <typename T>
constexpr int kXbCap = kXbLdsBytes / (int)sizeof(T);
// a band tile stores each entry's column (less the band's first column) and
// row offset in one 32-bit word, the row offset in the low kXbRowBits bits
template <typename T>
constexpr int kXbRowBits = sizeof(T) == 8 ? 15 : 16;
static_assert(kXbCap<double> <= (1 << kXbRowBits<double>), "row offsets fit");
static_assert(kXbCap<float> <= (1 << kXbRowBits<float>), "row offsets fit");
struct XblkView {
    int64_t n;             // matrix rows
    int64_t width;         // columns per slice
    int64_t ranges;        // row ranges
    const int* row_begin;  // [ranges + 1] first row of each range, then n
    int64_t band;          // entries within band columns of their range form its tile kXbBlocks
    int lbits;             // kXbRowBits of the dtype
    const int* tile_ptr;   // [ranges * kXbTiles + 1] first entry of tile (r, b), then nnz
    const int* col;        // [nnz] tile order, by column inside a tile (band tiles packed)
    const uint16_t* lrow;  // [nnz] row - row_begin[r]
    const void* val;       // [nnz]
};
hipError_t launch_xblk(const XblkView& a, bool f64, void* y, const void* x, double alpha,
                       double beta, hipStream_t stream);
// setup: cand[r] = start of range r of R0 by entry count (xblk_bound), r in [0, R0]
hipError_t launch_xblk_bounds(int64_t n, int64_t nnz, const int* rowptr, int64_t R0, int* cand,
                              hipStream_t stream);
// setup: the entry counts of every row in every slice at xblk_slot positions
hipError_t launch_xblk_count(const XblkView& a, const int* rowptr, const int* col, int* cnt,
                             hipStream_t stream);
// setup: tile_ptr from the scanned counts (pos[k] = counts before position k)
hipError_t launch_xblk_tiles(const XblkView& a, const int* pos, int* tile_ptr, hipStream_t stream);
// setup: col / val / lrow in tile order from the CSR arrays and pos
hipError_t launch_xblk_fill(const XblkView& a, bool f64, const int* rowptr, const int* col,
                            const void* val, const int* pos, int* ocol, void* oval,
                            uint16_t* olrow, hipStream_t stream);
// setup: oval[k] = val[src[k]], olrow[k] = lrow[src[k]]
hipError_t launch_xblk_gather(int64_t nnz, bool f64, const int* src, const void* val,
                              const uint16_t* lrow, void* oval, uint16_t* olrow, hipStream_t stream);

// kernel launchers (asynchronous on `stream`); fp64 when f64, else fp32
// rows: rows per lane group, a power of two up to kCsrRowsMax; stage_slots >
// 0: copy each wave's entries into LDS first when they fit in that many slots
// (subwave 2..16 with one row per group; four slices per workgroup within
// kCsrStageLds bytes, the default dynamic LDS limit).  The staged copy reads
// val without keeping it in the caches, and col too when stage_col_nt.
constexpr int kCsrRowsMax = 4;
constexpr int kCsrStageMin = 2, kCsrStageMax = 16;
// vector shapes whose groups would loop more often over the longest row are
// not tried when a kernel is chosen by timing
constexpr int kVecMaxPasses = 4096;
constexpr size_t kCsrStageLds = 64 * 1024;
hipError_t launch_csr(const CsrView& a, int subwave, int rows, int stage_slots, bool stage_col_nt,
                      bool f64, void* y, const void* x, double alpha, double beta,
                      hipStream_t stream);
int csr_stage_max_slots(bool f64);
hipError_t launch_ell(const EllView& a, bool f64, void* y, const void* x, double alpha,
                      double beta, hipStream_t stream);
hipError_t launch_sell(const SellView& a, bool f64, void* y, const void* x, double alpha,
                       double beta, hipStream_t stream);
hipError_t launch_tail(const TailView& t, bool f64, void* y, const void* x, double alpha,
                       hipStream_t stream);
// dst[r] = src[perm[r]] (inverse == false) or dst[perm[r]] = src[r]
hipError_t launch_permute(int64_t n, bool f64, void* dst, const void* src, const int* perm,
                          bool inverse, hipStream_t stream);
// Krylov solver vector kernels (k_vec.hip).  partial: device double[2 *
// kSolveBlocks]; out: device double[2].  Inner products in fp64.
constexpr int kSolveBlocks = 1024;
// out[0] = a0 . b0, out[1] = a1 . b1 (0 when a1 is nullptr); out == nullptr
// leaves the sums in partial only (for launch_solve_step)
hipError_t launch_dot2(int64_t n, bool f64, const void* a0, const void* b0, const void* a1,
                       const void* b1, double* partial, double* out, hipStream_t s);
// Device-resident scalars of a solve (double st[kStCount]); the kernels below
// read them and do nothing once st[kStDone] is set.
enum SolveState : int {
    kStRR, kStGoal, kStK, kStMaxIt, kStDone, kStPQ, kStAlpha, kStBeta, kStOmega, kStRho,
    kStRhoNew, kStCount
};
enum SolveStep : int { kStepCgPQ, kStepCgRR, kStepBiRV, kStepBiOmega, kStepBiRR };
// reduce partial (as launch_dot2 leaves it) and advance st by `step`
hipError_t launch_solve_step(const double* partial, double* st, int step, hipStream_t s);
// x += alpha p, r -= alpha q (alpha = rr / p.q), partial sums of r . r
hipError_t launch_cg_xr(int64_t n, bool f64, void* x, void* r, const void* p, const void* q,
                        const double* st, double* partial, hipStream_t s);
// p = r + beta (p - omega v)  (v == nullptr: p = r + beta p)
hipError_t launch_update_p(int64_t n, bool f64, void* p, const void* r, const void* v,
                           const double* st, hipStream_t s);
// s = r - alpha v
hipError_t launch_axmy(int64_t n, bool f64, void* s_out, const void* r, const void* v,
                       const double* st, hipStream_t s);
// x += alpha p + omega s, r = s - omega t, partial sums of r . r and of
// rhat . r (for kStepBiRR)
hipError_t launch_bicg_xr(int64_t n, bool f64, void* x, void* r, const void* p, const void* s_in,
                          const void* t, const void* rh, const double* st, double* partial,
                          hipStream_t s);
// y = beta * y for n entries (beta == 0 writes zeros and never reads y)
hipError_t launch_scale(int64_t n, bool f64, void* y, double beta, hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

}  // namespace spmv
